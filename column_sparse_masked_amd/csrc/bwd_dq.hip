// dQ of column-sparse masked attention, query-stationary (bf16 MFMA, fp32
// accumulate).  FlashMask-3 paper summary, abstract: the mask-aware kernel
// visits only the tiles the column-wise sparse mask does not fully hide.
//
// The backward splits the gradient between two kernels so that neither needs
// atomic adds: the key-stationary kernel accumulates dK and dV in registers,
// and this one accumulates dQ.  Each workgroup (8 waves, two per SIMD) takes a
// query block of 128 rows from the same cost-sorted queue as the forward and
// walks the block's list of non-skipped key blocks.  Wave w holds query rows
// 32 (w % 4) .. +32 of the block (Q and dO as MFMA B operands, LSE and Delta
// of its row in each lane) and works on keys 64 (w / 4) .. +64 of every key
// block:
//     S^T = K Q^T,  dP^T = V dO^T           (A operands: K, V rows from LDS)
//     P = exp(S - LSE) (interval mask on partial tiles),
//     dS'^T = P (dP - Delta)                 (dS / scale),
//     dQ^T += K^T dS'^T                      (A operand: K^T rows from LDS,
//                                             B operand: the dS'^T accumulator)
// and dQ = scale dQ' when it is written.
// S^T and dP^T are recomputed here rather than shared with the key-stationary
// kernel: exchanging dS between the two would cost more memory traffic than
// the two extra products.  At the end the two key halves' dQ^T are summed in
// LDS and dQ is written once in bf16: deterministic, with no fp32 workspace.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {

namespace {

constexpr int kDqThreads = 512;   // 8 waves

template <int D>
struct DqSmem {
  static constexpr int KST = D + 8;    // K, V row stride (elements): conflict-free row reads
  static constexpr int KTS = BK + 8;   // K^T row stride; keys in perm16 order
  static_assert(stage_strides_ok(2 * KST, 2 * KTS), "strides the staging map needs");
  static constexpr int RED = 4 * (D / 32) * 16 * 64;   // fp32 dQ^T of 4 waves (final sum)
  union {
    struct {
      bf16 k[BK * KST];
      bf16 v[BK * KST];
    } kv;
    float red[RED];
  } u;
  bf16 kt[D * KTS];
  // partial tiles: bit i of hid[g][j] says whether key j of the tile hides
  // row 32 g + i of the query block
  uint32_t hid[BQ / 32][BK];
  uint32_t hdr[2][4];   // headers of this and the next work item
};

// Place of key x inside a K^T row: bits 2 and 3 of the offset within each
// group of 16 swapped, so that the 8 keys a lane holds in a dS^T accumulator
// (the B operand of the dQ^T product) are 8 neighbouring elements.
__device__ __forceinline__ int kt_pos(int x) { return (x & ~15) | perm16(x & 15); }

// Global -> register staging of a key block's K and V (512 threads).  A unit
// is 4 consecutive keys (4 m .. 4 m + 3) x 8 head-dim columns (chunk c) of one
// tensor; the units of a wave are 16 row-units by 4 chunks of the staging map
// (stage_row_unit, stage_chunk), which keeps the row-major stores and the
// transposed stores of K free of bank conflicts.
template <int D>
struct DqStage {
  static constexpr int CPR = D / 8;
  static constexpr int NPT = (BK / 4) * CPR;              // units per tensor
  static constexpr int NU = 2 * NPT / kDqThreads;          // units per thread
  static_assert(NPT % 64 == 0 && (2 * NPT) % kDqThreads == 0, "unit tensor is wave-uniform");
  static_assert(CPR % 4 == 0 && (BK / 4) % 16 == 0, "a wave's units are 16 row-units x 4 chunks");
  bf16x8 v[NU][4];

  static __device__ __forceinline__ unsigned unit(unsigned t, int j) { return t + kDqThreads * j; }
  static __device__ __forceinline__ int tensor(unsigned t, int j) {   // 0 = K, 1 = V
    return __builtin_amdgcn_readfirstlane((int)(unit(t, j) / NPT));
  }
  // unit p of the tensor: wave p / 64 takes row-units 16 (p / 64 / (CPR/4)) ..
  // + 16 and chunk quad (p / 64) % (CPR/4)
  static __device__ __forceinline__ int key(unsigned t, int j) {
    const int p = (int)(unit(t, j) % NPT);
    return 4 * (16 * ((p >> 6) / (CPR / 4)) + stage_row_unit(p & 63));
  }
  static __device__ __forceinline__ int col(unsigned t, int j) {
    const int p = (int)(unit(t, j) % NPT);
    return stage_chunk(p & 63, (p >> 6) % (CPR / 4));
  }
};

template <int D>
__device__ __forceinline__ void dq_load(DqStage<D>& r, BufRsrc kb, BufRsrc vb, int k0, unsigned t) {
  using S = DqStage<D>;
#pragma unroll
  for (int j = 0; j < S::NU; ++j) {
    const BufRsrc src = S::tensor(t, j) == 0 ? kb : vb;
    const uint32_t base =
        opaque(((uint32_t)S::key(t, j) * S::CPR + S::col(t, j)) * 16u) + (uint32_t)k0 * (D * 2);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r.v[j][rr] = buf_load16(src, base + (uint32_t)rr * (D * 2));
  }
}

// K and V row-major (A operands of S^T and dP^T)
template <int D>
__device__ __forceinline__ void dq_store_rows(const DqStage<D>& r, DqSmem<D>& sm, unsigned t) {
  using S = DqStage<D>;
  constexpr int KST = DqSmem<D>::KST;
#pragma unroll
  for (int j = 0; j < S::NU; ++j) {
    bf16* rm = (S::tensor(t, j) == 0 ? sm.u.kv.k : sm.u.kv.v) + opaque(S::key(t, j) * KST + 8 * S::col(t, j));
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) *reinterpret_cast<bf16x8*>(rm + rr * KST) = r.v[j][rr];
  }
}

// K transposed (A operand of dQ^T)
template <int D>
__device__ __forceinline__ void dq_store_kt(const DqStage<D>& r, DqSmem<D>& sm, unsigned t) {
  using S = DqStage<D>;
  constexpr int KTS = DqSmem<D>::KTS;
#pragma unroll
  for (int j = 0; j < S::NU; ++j) {
    if (S::tensor(t, j) != 0) continue;
    bf16* tp = sm.kt + opaque((8 * S::col(t, j)) * KTS + kt_pos(S::key(t, j)));
    const bf16x16 p01 = __builtin_shufflevector(r.v[j][0], r.v[j][1], 0, 8, 1, 9, 2, 10, 3, 11,
                                                4, 12, 5, 13, 6, 14, 7, 15);
    const bf16x16 p23 = __builtin_shufflevector(r.v[j][2], r.v[j][3], 0, 8, 1, 9, 2, 10, 3, 11,
                                                4, 12, 5, 13, 6, 14, 7, 15);
#define FM_KT_ROW(e)                                                                      \
  *reinterpret_cast<bf16x4*>(tp + (e) * KTS) =                                            \
      __builtin_shufflevector(p01, p23, 2 * (e), 2 * (e) + 1, 16 + 2 * (e), 17 + 2 * (e))
    FM_KT_ROW(0); FM_KT_ROW(1); FM_KT_ROW(2); FM_KT_ROW(3);
    FM_KT_ROW(4); FM_KT_ROW(5); FM_KT_ROW(6); FM_KT_ROW(7);
#undef FM_KT_ROW
  }
}

// 32-bit row mask of rows [lo, hi) (0 <= lo, hi <= 32; empty when hi <= lo)
__device__ __forceinline__ uint32_t row_bits(int lo, int hi) {
  return hi > lo ? (~0u >> (32 - hi)) & (~0u << lo) : 0u;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_kernel(const BwdArgs a) {
  constexpr int NS = D / 16, ND = D / 32;
  constexpr int KST = DqSmem<D>::KST, KTS = DqSmem<D>::KTS;
  __shared__ DqSmem<D> sm;
  // with the tile cache on, the cached kernel computes dQ from the stored
  // dS' instead (the queue counters are left untouched)
  if (tile_cache_on(a.counters, a.ds_cap)) return;

  const unsigned t = threadIdx.x;
  const int lane = (int)(t & 63), w = (int)(t >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const int qw = w & 3, kh = w >> 2;   // query rows 32 qw.., keys 64 kh.. of each block
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nQ);
  // in pair mode the queue holds pairs of query blocks, two tickets each
  const bool pairs = a.counters[kCtrFwdPairs] == 1u;
  const int nP = pairs ? (a.nQ + 1) >> 1 : 0;
  const uint32_t max_entries = (uint32_t)((long)a.B * a.H * (pairs ? nP : a.nQ));
  const uint32_t n_entries = min(a.counters[kCtrFwdItems], max_entries);
  const uint32_t n_items = pairs ? 2u * n_entries : n_entries;
  const int Sq = a.Sq, Sk = a.Sk;

  const ItemQueue iq{&a.counters[kCtrDqNext], a.queue_q, a.cnt_q, n_items, max_items, a.nQ, a.H, a.Hm, a.nK,
                     0u, nP, max_entries};
  if (t == 0) iq.first(sm.hdr[0]);
  __syncthreads();
  for (int n = 0;; ++n) {
    const uint32_t idx = __builtin_amdgcn_readfirstlane(sm.hdr[n & 1][0]);
    if (idx >= n_items) break;
    const uint32_t it = __builtin_amdgcn_readfirstlane(sm.hdr[n & 1][1]);
    const int cnt = __builtin_amdgcn_readfirstlane((int)sm.hdr[n & 1][2]);
    ItemPrefetch pf;
    pf.take(iq, t);
    const long bh = it / a.nQ;
    // (a ticket without an item, count -1, takes block nQ: every row past
    // the end, so that nothing is written)
    const int qb = cnt < 0 ? a.nQ : (int)(it % a.nQ);
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const long bhm = (long)b * a.Hm + (a.Hm == 1 ? 0 : h);
    const uint16_t* lst = a.list_q + (bhm * a.nQ + qb) * (long)a.nK;
    const BufRsrc qbase = make_rsrc(a.q + bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
    const BufRsrc obase = make_rsrc(a.dout + bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
    const BufRsrc kbase = make_rsrc(a.k + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
    const BufRsrc vbase = make_rsrc(a.v + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
    const BufRsrc bbase = make_rsrc(a.bounds + bhm * Sk, (uint32_t)Sk * 16u);
    auto block_start = [&](int e) { return min(e & kListIndex, a.nK - 1) * BK; };
    auto block_masked = [&](int e, int k0) { return (e & kListPartial) || (k0 + BK > Sk); };
    const int q0 = qb * BQ;
    const int qrow = q0 + 32 * qw + li;

    f32x16 acc[ND];   // dQ^T: lane holds query li, head-dim rows 32 d + 8 r + 4 hh + q
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[d][v] = 0.f;

    if (cnt > 0) {

      // hidden-row words of a partial key block (threads < BK, one key each)
      auto key_bounds = [&](int k0) __attribute__((always_inline)) {
        return __builtin_amdgcn_raw_buffer_load_b128(bbase, (k0 + (int)t) * 16, 0, 0);
      };
      auto words_of = [&](const i32x4 x, int k0, uint32_t (&wd)[BQ / 32]) __attribute__((always_inline)) {
        const bool in = k0 + (int)t < Sk;   // keys past the end hide every row
        const int lts = in ? x[0] : INT_MIN, lte = in ? x[1] : INT_MAX;
        const int uts = in ? x[2] : 0, ute = in ? x[3] : 0;
#pragma unroll
        for (int g = 0; g < BQ / 32; ++g) {
          const int base = q0 + 32 * g;
          auto clip = [&](int y) { return min(max(y, base), base + 32) - base; };
          wd[g] = row_bits(clip(lts), clip(lte)) | row_bits(clip(uts), clip(ute));
        }
      };
      auto hidden_words = [&](int k0, uint32_t (&wd)[BQ / 32]) __attribute__((always_inline)) {
        words_of(key_bounds(k0), k0, wd);
      };

      DqStage<D> st;
      int e_cur = list_entry(lst, 0);
      // The first key block's loads go first: its LDS staging then waits for
      // them only, with the Q and dO rows (needed after the barrier) in flight.
      const int k00 = block_start(e_cur);
      const bool m00 = block_masked(e_cur, k00) && t < BK;
      i32x4 bd00 = {0, 0, 0, 0};
      if (m00) bd00 = key_bounds(k00);
      dq_load<D>(st, kbase, vbase, k00, t);
      // Q and dO rows of this lane's query (B operands), LSE and Delta.  The
      // lane's offsets are rebuilt per item from its lane index rather than
      // kept, spilled, through the kernel: reloading a spill waits for every
      // load issued before it.  LSE and Delta are used only after the
      // barrier below.
      const int ln = lane_in(n);
      const int qrow0 = q0 + 32 * __builtin_amdgcn_readfirstlane(qw);
      bf16x8 qf[NS], of[NS];
      {
        const uint32_t off = (uint32_t)((ln & 31) * D + 8 * (ln >> 5)) * 2u + (uint32_t)qrow0 * (D * 2);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          qf[s] = buf_load16(qbase, off + 32u * s);
          of[s] = buf_load16(obase, off + 32u * s);
        }
      }
      const uint32_t roff = (uint32_t)(ln & 31) * 4u + (uint32_t)qrow0 * 4u;
      const float lse_raw = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.lse + bh * Sq, (uint32_t)Sq * 4u), (int)roff, 0, 0));
      const float dl_raw = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.delta + bh * Sq, (uint32_t)Sq * 4u), (int)roff, 0, 0));
      {
        if (m00) {
          uint32_t wd[BQ / 32];
          words_of(bd00, k00, wd);
#pragma unroll
          for (int g = 0; g < BQ / 32; ++g) sm.hid[g][t] = wd[g];
        }
        dq_store_rows<D>(st, sm, t);
        dq_store_kt<D>(st, sm, t);
      }
      pf.stash(sm.hdr[(n + 1) & 1], t);   // the stores above waited for loads issued after the ticket
      // Unconditional (a one-block item loads its block again, unused), so
      // that the waits for LSE and Delta count these loads as issued after
      // them on every path instead of waiting for them too.
      dq_load<D>(st, kbase, vbase, block_start(list_entry(lst, cnt > 1 ? 1 : 0)), t);
      __syncthreads();
      const bool live = qrow < Sq;
      const float lse2 = live ? lse_raw * kLog2e : INFINITY;
      const float dl = live ? dl_raw : 0.f;

      // Per key block t (K, V, hid of t and K^T of t in LDS; t+1 in registers):
      //   S^T, dP^T, dS^T of both 32-key sub-blocks | barrier | K, V, hid of
      //   t+1 -> LDS; dQ^T += K^T dS^T | barrier | K^T of t+1 -> LDS, t+2 ->
      //   registers.  K, V of t+1 are read after the second barrier, K^T of
      //   t+1 after the next first barrier.
      for (int tt = 0; tt < cnt; ++tt) {
        const int k0 = block_start(e_cur);
        const bool need_mask = block_masked(e_cur, k0);
        const bool has_next = tt + 1 < cnt;
        const int e_next = has_next ? list_entry(lst, tt + 1) : e_cur;
        const int k0n = block_start(e_next);
        const bool m_next = has_next && block_masked(e_next, k0n) && t < BK;

        bf16x8 dsb[2][2];   // dS^T of sub-blocks jj, k-halves t2 (B operands of dQ^T)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int jb = 2 * kh + jj;   // 32-key sub-block of the tile
          // ---- S^T, dP^T: lane holds query li, keys 32 jb + 8 r + 4 hh + q ----
          f32x16 s, dp;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            s[v] = 0.f;
            dp[v] = 0.f;
          }
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int kk = 0; kk < NS; ++kk) {
            const int off = (32 * jb + li) * KST + 16 * kk + 8 * hh;
            s = mfma32(as_bf16x8(&sm.u.kv.k[off]), qf[kk], s);
            dp = mfma32(as_bf16x8(&sm.u.kv.v[off]), of[kk], dp);
          }
          __builtin_amdgcn_s_setprio(0);
          // ---- dS'^T = P (dP - Delta), P = exp2(S scale log2 e - LSE log2 e) ----
          if (need_mask) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint4 h4 = *reinterpret_cast<const uint4*>(&sm.hid[qw][32 * jb + 8 * r + 4 * hh]);
              const uint32_t hq[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
              for (int q = 0; q < 4; ++q)
                s[4 * r + q] = (hq[q] >> li) & 1u ? -INFINITY : s[4 * r + q];
            }
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float p = fast_exp2(fmaf(s[v], a.scale_log2, -lse2));
            dsb[jj][v >> 3][v & 7] = (bf16)(p * (dp[v] - dl));
          }
        }
        __syncthreads();   // every wave is done with this block's K, V and hid
        if (has_next) {
          uint32_t wd[BQ / 32];
          if (m_next) hidden_words(k0n, wd);
          dq_store_rows<D>(st, sm, t);
          if (m_next)
#pragma unroll
            for (int g = 0; g < BQ / 32; ++g) sm.hid[g][t] = wd[g];
        }
        // ---- dQ^T += K^T dS^T ----
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int jb = 2 * kh + jj;
#pragma unroll
          for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
              acc[d] = mfma32(as_bf16x8(&sm.kt[(32 * d + li) * KTS + 32 * jb + 16 * t2 + 8 * hh]),
                              dsb[jj][t2], acc[d]);
        }
        // the next item's header, one scalar load in each of the first two blocks
        if (tt == 0) pf.fetch_entry(iq, sm.hdr[(n + 1) & 1]);
        if (tt == 1) pf.fetch_count(iq);
        __syncthreads();   // every wave is done with this block's K^T
        if (has_next) {
          dq_store_kt<D>(st, sm, t);
          if (tt + 2 < cnt) dq_load<D>(st, kbase, vbase, block_start(list_entry(lst, tt + 2)), t);
        }
        e_cur = e_next;
      }
      if (cnt == 1) pf.fetch_count(iq);
      pf.publish(iq, sm.hdr[(n + 1) & 1], t);
    } else {
      pf.finish_now(iq, sm.hdr[(n + 1) & 1], t);
    }

    // ---- dQ = sum of the two key halves' dQ^T, written once in bf16 ----
    // red[((qw * ND + d) * 4 + r) * 64 + lane] holds elements 4r..4r+3 of acc[d]
    float4* red = reinterpret_cast<float4*>(sm.u.red);
    if (kh == 1) {
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[((qw * ND + d) * 4 + r) * 64 + lane] =
              make_float4(acc[d][4 * r], acc[d][4 * r + 1], acc[d][4 * r + 2], acc[d][4 * r + 3]);
    }
    __syncthreads();
    if (kh == 0 && qrow < Sq) {
      bf16* drow = a.dq + (bh * Sq + qrow) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 o = red[((qw * ND + d) * 4 + r) * 64 + lane];
          bf16x4 x;
          x[0] = (bf16)((acc[d][4 * r] + o.x) * a.scale);
          x[1] = (bf16)((acc[d][4 * r + 1] + o.y) * a.scale);
          x[2] = (bf16)((acc[d][4 * r + 2] + o.z) * a.scale);
          x[3] = (bf16)((acc[d][4 * r + 3] + o.w) * a.scale);
          *reinterpret_cast<bf16x4*>(&drow[32 * d + 8 * r + 4 * hh]) = x;
        }
    }
    __syncthreads();   // every thread has read red; the next header is in LDS
  }
  // The last workgroup to leave resets the queue counters for the next call.
  if (t == 0) {
    __threadfence();
    const uint32_t done = atomicAdd(&a.counters[kCtrDqExit], 1u);
    if (done == gridDim.x - 1) {
      atomicExch(&a.counters[kCtrDqNext], 0u);
      atomicExch(&a.counters[kCtrDqExit], 0u);
    }
  }
}

hipError_t launch_attn_bwd_dq(const BwdArgs& a, int head_dim, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128)
    attn_bwd_dq_kernel<128><<<grid, kDqThreads, 0, stream>>>(a);
  else
    attn_bwd_dq_kernel<64><<<grid, kDqThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace fm
