// Forward of column-sparse masked attention on the matrix cores (bf16 in,
// fp32 accumulate).  FlashMask-3 paper summary, abstract: a mask-aware kernel
// that works only on tiles the column-wise sparse mask does not fully mask.
//
// Persistent grid: each workgroup (4 waves) repeatedly takes the next item
// (batch*head, query block) from the cost-sorted queue built by the tile pass,
// holds that block's 128 query rows in registers (32 rows per wave) and walks
// the block's list of non-skipped key blocks.  Per key block, K is staged
// row-major and V transposed in LDS, so that every MFMA operand read is one
// 16-byte LDS load.  Each wave computes S^T = K Q^T (32 keys x 32 rows per
// MFMA), applies the elementwise interval test only on partial (or ragged)
// tiles, updates an online softmax in the log2 domain and accumulates
// O^T += V^T P^T.  Keeping S^T (not S) lets the accumulator of one MFMA be the
// B operand of the next with no data movement between lanes.
//
// The next key block is fetched into registers while the current one
// computes: K during S, V during the softmax and the PV product, each written
// to LDS as soon as every wave is done with the previous contents.  Global
// loads go through buffer resources whose range check zero-fills the rows
// past the end of a ragged key (or query) range.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {

template <int D, int NQB = 1, int NBUF = 1>
struct alignas(16) FwdSmem {
  static constexpr int KST = D + 8;    // K row stride (elements): conflict-free 16-byte row reads
  static constexpr int VTS = BK + 8;   // V^T row stride (elements)
  bf16 k[NBUF][BK * KST];              // K tiles, one key per row
  bf16 vt[NBUF][D * VTS];              // V^T tiles, one head-dim column per row, keys in vt_pos order
  // partial tiles (key blocks t even / odd): bit i of hid[.][g][j] says
  // whether key j hides row 32 g + i of the item's NQB query blocks
  uint32_t hid[2][NQB * BQ / 32][BK];
  uint32_t hdr[2][4];   // headers of this and the next work item
};

// Place of key x (0 <= x < BK) inside a V^T row: bits 2 and 3 of the offset
// within each group of 16 keys are swapped, so that the 8 keys one lane holds
// in the P operand of the PV product are 8 neighbouring elements.
__device__ __forceinline__ int vt_pos(int x) { return (x & ~15) | perm16(x & 15); }

// Global -> register staging of one key block (NT threads: 256, or 512 for
// a pair of query blocks).
//   K: thread t holds column chunk t % CPR (8 head-dim values) of the NK
//      consecutive rows NK*(t / CPR) ...  (loads and LDS stores then differ
//      only by constant offsets);
//   V: units of 4 consecutive keys x 8 head-dim columns, unit p = t + NT j
//      (j < NV) at key-unit 16 ((p / 64) / (CPR / 4)) + p % 16 and chunk
//      stage_chunk(p % 64, (p / 64) % (CPR / 4)): the staging map that keeps
//      the transposed 8-byte LDS stores free of bank conflicts (the 16 lanes
//      served together write 16 distinct 8-byte places of rows that start on
//      the same bank).
template <int D, int NT = 256>
struct Stage {
  static constexpr int CPR = D / 8;               // 16-byte chunks per row
  static constexpr int NK = BK * CPR / NT;        // K rows per thread
  static constexpr int NV = (BK / 4) * CPR / NT;  // V units per thread
  static_assert(CPR % 4 == 0 && ((BK / 4) * CPR) % NT == 0, "whole V units per thread");
  static_assert(NK == 4 * NV, "a K block and a V block take the same registers");
  // One set of registers holds K of the next block until it is stored, then
  // V of that block: the two are never held at the same time in the loop.
  bf16x8 x[NK];

  static __device__ __forceinline__ int k_row(unsigned t) { return NK * (int)(t / CPR); }
  static __device__ __forceinline__ int k_col(unsigned t) { return (int)(t % CPR); }
  // first key and column chunk of V unit j of thread t
  static __device__ __forceinline__ int v_key(unsigned t, int j) {
    const int p = (int)t + NT * j;
    return 4 * (16 * ((p >> 6) / (CPR / 4)) + stage_row_unit(p & 63));
  }
  static __device__ __forceinline__ int v_col(unsigned t, int j) {
    const int p = (int)t + NT * j;
    return stage_chunk(p & 63, (p >> 6) % (CPR / 4));
  }
};

template <int D, int NT>
__device__ __forceinline__ void load_k(Stage<D, NT>& r, BufRsrc kb, int k0, unsigned t) {
  using S = Stage<D, NT>;
  const uint32_t base = opaque(((uint32_t)S::k_row(t) * S::CPR + S::k_col(t)) * 16u) + (uint32_t)k0 * (D * 2);
#pragma unroll
  for (int i = 0; i < S::NK; ++i) r.x[i] = buf_load16(kb, base + (uint32_t)i * (D * 2));
}

template <int D, int NT>
__device__ __forceinline__ void store_k(const Stage<D, NT>& r, bf16* sk, unsigned t) {
  using S = Stage<D, NT>;
  constexpr int KST = FwdSmem<D>::KST;
  bf16* dst = sk + opaque(S::k_row(t) * KST + S::k_col(t) * 8);
#pragma unroll
  for (int i = 0; i < S::NK; ++i) *reinterpret_cast<bf16x8*>(dst + i * KST) = r.x[i];
}

template <int D, int NT>
__device__ __forceinline__ void load_v(Stage<D, NT>& r, BufRsrc vb, int k0, unsigned t) {
  using S = Stage<D, NT>;
#pragma unroll
  for (int j = 0; j < S::NV; ++j) {
    const uint32_t base =
        opaque(((uint32_t)S::v_key(t, j) * S::CPR + S::v_col(t, j)) * 16u) + (uint32_t)k0 * (D * 2);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r.x[4 * j + rr] = buf_load16(vb, base + (uint32_t)rr * (D * 2));
  }
}

template <int D, int NT>
__device__ __forceinline__ void store_vt(const Stage<D, NT>& r, bf16* vt, unsigned t) {
  using S = Stage<D, NT>;
  constexpr int VTS = FwdSmem<D>::VTS;
  static_assert((8 * VTS * 2) % 128 == 0, "8 transposed rows start on the same bank");
#pragma unroll
  for (int i = 0; i < S::NV; ++i) {
    bf16* dst = vt + opaque((8 * S::v_col(t, i)) * VTS + vt_pos(S::v_key(t, i)));
    // 4 keys x 8 columns -> 8 rows of 4 keys (constant shuffles only, so the
    // compiler keeps everything in registers)
    const bf16x16 p01 = __builtin_shufflevector(r.x[4 * i], r.x[4 * i + 1], 0, 8, 1, 9, 2, 10, 3,
                                                11, 4, 12, 5, 13, 6, 14, 7, 15);
    const bf16x16 p23 = __builtin_shufflevector(r.x[4 * i + 2], r.x[4 * i + 3], 0, 8, 1, 9, 2, 10,
                                                3, 11, 4, 12, 5, 13, 6, 14, 7, 15);
#define FM_VT_ROW(e)                                                                      \
  *reinterpret_cast<bf16x4*>(dst + (e) * VTS) =                                           \
      __builtin_shufflevector(p01, p23, 2 * (e), 2 * (e) + 1, 16 + 2 * (e), 17 + 2 * (e))
    FM_VT_ROW(0); FM_VT_ROW(1); FM_VT_ROW(2); FM_VT_ROW(3);
    FM_VT_ROW(4); FM_VT_ROW(5); FM_VT_ROW(6); FM_VT_ROW(7);
#undef FM_VT_ROW
  }
}

// SPLIT: whether items may be split in two (the instance without is used
// when the problem has enough items per workgroup for the longest-first
// order to balance the grid; its code has none of the split handling).
// LDS operands of the S and PV products are read this many products ahead.
constexpr int kRASingle = 3, kRAPair = 4;

//
// PAIR: an item is a pair of neighbouring query blocks (2qp, 2qp+1) of one
// head, taken by 8 waves (waves 4 hq .. 4 hq + 3 hold the rows of block
// 2qp + hq), which walk the pair's union list of key blocks: each key block
// is loaded and staged in LDS once for both query blocks, and a wave works on
// it only when its own query block sees it.
template <int D, bool SPLIT, bool PAIR>
__global__ __launch_bounds__(PAIR ? 512 : 256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const FwdArgs a) {
  static_assert(!(SPLIT && PAIR), "pair items are not split");
  constexpr int NT = PAIR ? 512 : 256;   // threads
  constexpr int NQB = PAIR ? 2 : 1;      // query blocks per item
  constexpr int NS = D / 16;   // k-steps over the head dimension
  constexpr int ND = D / 32;   // 32-wide blocks of the head dimension
  constexpr int kRA = PAIR ? kRAPair : kRASingle;
  constexpr int NBUF = PAIR ? 2 : 1;     // K and V^T tiles in LDS (pairs: double-buffered)
  constexpr int KST = FwdSmem<D, NQB, NBUF>::KST, VTS = FwdSmem<D, NQB, NBUF>::VTS;
  __shared__ FwdSmem<D, NQB, NBUF> sm;

  const unsigned t = threadIdx.x;
  const int lane = (int)(t & 63), w = (int)(t >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const int hq = PAIR ? (w >> 2) : 0;   // which query block of the item holds this wave's rows
  const int wr = PAIR ? (w & 3) : w;    // this wave's 32-row group within that block
  // items per head: query blocks, or pairs of them
  const int nF = PAIR ? (a.nQ + 1) >> 1 : a.nQ;
  // item count and queue entries are range-checked so that a stale or foreign
  // tileinfo cannot make the kernel read outside its tensors
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * nF);
  const uint32_t n_real = min(a.counters[kCtrFwdItems], max_items);
  // the first nsplit items of the queue are taken as two halves each
  const uint32_t nsplit =
      SPLIT ? min(min(a.counters[kCtrFwdSplit], (uint32_t)max(a.split_cap, 0)), n_real) : 0u;
  const uint32_t n_items = n_real + nsplit;
  const int Sq = a.Sq, Sk = a.Sk;

  const ItemQueue iq{&a.counters[kCtrFwdNext], a.queue, PAIR ? a.cnt_p : a.cnt_q, n_items, max_items, nF, a.H,
                     a.Hm, a.nK, nsplit};
  if (t == 0) iq.first(sm.hdr[0]);
  __syncthreads();
  for (int n = 0;; ++n) {
    // the item is the same for the whole workgroup: keep it (and everything
    // derived from it) in scalar registers
    const uint32_t idx = __builtin_amdgcn_readfirstlane(sm.hdr[n & 1][0]);
    if (idx >= n_items) break;
    const uint32_t it = __builtin_amdgcn_readfirstlane(sm.hdr[n & 1][1]);
    const int cnt_all = __builtin_amdgcn_readfirstlane((int)sm.hdr[n & 1][2]);
    // a split item's ticket 2 j + p takes half p of its list of key blocks
    const bool split = SPLIT && idx < 2 * nsplit;
    const int half = (cnt_all + 1) >> 1;
    const int first = split && (idx & 1u) ? half : 0;
    const int cnt = split ? ((idx & 1u) ? cnt_all - half : half) : cnt_all;
    ItemPrefetch pf;
    pf.take(iq, t);
    const long bh = it / nF;
    const int ib = (int)(it % nF);            // the item's query block, or pair
    const int qb0 = PAIR ? 2 * ib : ib;       // its first query block
    const int qb = qb0 + hq;                  // this wave's query block
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const long bhm = (long)b * a.Hm + (a.Hm == 1 ? 0 : h);
    // the key block list: of the query block (16-bit entries, bit 15 partial),
    // or of the pair (32-bit entries with the kPair* flags)
    const uint16_t* lst = a.list_q + (bhm * a.nQ + qb) * (long)a.nK + first;
    const uint32_t* lstp = a.list_p + (bhm * nF + ib) * (long)a.nK;
    // buffer resources over this head's Q, K, V and bounds: loads past the
    // end of the rows return zeros
    const BufRsrc qbase = make_rsrc(a.q + bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
    const BufRsrc kbase = make_rsrc(a.k + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
    const BufRsrc vbase = make_rsrc(a.v + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
    const BufRsrc bbase = make_rsrc(a.bounds + bhm * Sk, (uint32_t)Sk * 16u);
    // key block list entry -> first key, whether the item needs the bounds
    // of the block (a tile partial, or ragged at the end of the keys), and
    // whether this wave's block sees it and needs the elementwise interval test
    auto block_start = [&](int e) { return min(e & (int)(PAIR ? kPairBlock : kListIndex), a.nK - 1) * BK; };
    auto block_masked = [&](int e, int k0) {
      return (e & (int)(PAIR ? (kPairPart0 | kPairPart1) : kListPartial)) || (k0 + BK > Sk);
    };
    auto wave_sees = [&](int e) { return !PAIR || (e & (int)(hq ? kPairSee1 : kPairSee0)) != 0; };
    auto wave_masked = [&](int e, int k0) {
      return PAIR ? ((e & (int)(hq ? kPairPart1 : kPairPart0)) != 0 || (k0 + BK > Sk)) : block_masked(e, k0);
    };
    // the hidden-row words of the item's query blocks for a block's bounds
    // (threads < BK, key t of the block)
    auto stage_hidden = [&](const int4 breg, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int qq = 0; qq < NQB; ++qq) {
        uint32_t wd[BQ / 32];
        hidden_rows(breg, (qb0 + qq) * BQ, wd);
#pragma unroll
        for (int g = 0; g < BQ / 32; ++g) sm.hid[buf][qq * (BQ / 32) + g][t] = wd[g];
      }
    };

    const int qrow = qb * BQ + 32 * wr + li;
    f32x16 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[d][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    if (cnt > 0) {
      // ---- first key block: global -> registers -> LDS; second K block in flight ----
      // In the loop, list entries are read one block ahead through a buffer
      // resource (a vector load whose value is the same in every lane).  The
      // first two are scalar loads: waiting for a vector load would also wait
      // for every vector load issued before it.
      const BufRsrc lbase = PAIR ? make_rsrc(lstp, (uint32_t)cnt * 4u) : make_rsrc(lst, (uint32_t)cnt * 2u);
      auto list_at = [&](int i) -> uint32_t {
        if constexpr (PAIR) return __builtin_amdgcn_raw_buffer_load_b32(lbase, i * 4, 0, 0);
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(lbase, i * 2, 0, 0);
      };
      auto list_first = [&](int i) -> int {
        if constexpr (PAIR) return (int)*(const_u32*)(lstp + i);
        return list_entry(lst, i);
      };
      Stage<D, NT> st, st_v;   // (st_v: V of the first block only)
      int e_cur = list_first(0);
      int e_next = cnt > 1 ? list_first(1) : 0;
      bf16x8 qf[NS];   // Q rows of this wave (B operand of S^T = K Q^T)
      {
        const int k0 = block_start(e_cur);
        load_k<D>(st, kbase, k0, t);
        load_v<D>(st_v, vbase, k0, t);
        int4 breg = make_int4(0, 0, 0, 0);
        if (block_masked(e_cur, k0) && t < BK) breg = load_bnd(bbase, k0, Sk, t);
        // issued after the block's loads: the staging below waits for those only
        const uint32_t qoff = ((uint32_t)qrow * D + 8u * hh) * 2u;
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = buf_load16(qbase, qoff + 32u * s);
        store_k<D>(st, sm.k[0], t);
        store_vt<D>(st_v, sm.vt[0], t);
        if (block_masked(e_cur, k0) && t < BK) stage_hidden(breg, 0);
      }
      pf.stash(sm.hdr[(n + 1) & 1], t);   // the stores above waited for loads issued after the ticket
      // The Q rows are in registers by now (loaded right after the block's K
      // and V, which the stores waited for).  Saying so with an explicit wait
      // keeps the compiler from waiting for the loads of later key blocks,
      // issued after Q, before the S products of every block.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      int4 bnext = make_int4(0, 0, 0, 0);   // (pairs) bounds of the next block, loaded a block ahead
      if (cnt > 1) {
        load_k<D>(st, kbase, block_start(e_next), t);
        if (PAIR && block_masked(e_next, block_start(e_next)) && t < BK)
          bnext = load_bnd(bbase, block_start(e_next), Sk, t);
      }
      __syncthreads();

      // Per key block t (K_t, bounds_t in LDS; V^T_t being stored, K_{t+1}
      // in registers), keys in halves h0, h1:
      //   S_t(h0) | barrier | softmax, PV_t(h0); S_t(h1) | barrier | K_{t+1}
      //   -> LDS; bounds_{t+1}, V_{t+1} -> registers; softmax, PV_t(h1);
      //   bounds_{t+1} -> LDS | barrier | V_{t+1} -> LDS, K_{t+2} -> registers.
      for (int tt = 0;; ++tt) {
        const int k0 = block_start(e_cur);
        const bool need_mask = wave_masked(e_cur, k0);
        const bool sees = wave_sees(e_cur);   // (the same in every lane of the wave)
        const bool has_next = tt + 1 < cnt;
        const int k0n = block_start(e_next);
        const bool nm_next = has_next && block_masked(e_next, k0n);
        // list entry of block t+2, consumed after the last barrier (past the
        // end of the list the range check reads 0; the load is unconditional
        // so that no path leaves it in flight into the next block)
        const uint32_t e2_pending = list_at(tt + 2);

        // The block is taken as two halves of 64 keys: S of a half, then its
        // softmax and PV, so that S needs 32 accumulator registers rather
        // than 64 (which leaves room to read the S operands ahead) and the
        // exponentials of the first half run beside the products of the
        // second.  Three barriers per block: V^T of the block, stored by
        // every thread after the previous block's last barrier, is complete
        // before the first half's PV (barrier 0); K is free once the second
        // half's S is done (barrier 1); V^T once its PV is done (barrier 2).
        float rs = 0.f;   // row sum of this block's P
        const int buf = PAIR ? (tt & 1) : 0;   // the block's K and V^T tiles
        const bf16* kcur = sm.k[buf];
        const bf16* vcur = sm.vt[buf];
        auto half_s = [&](int hk, f32x16 (&s)[2]) __attribute__((always_inline)) {
          // ---- S^T = K Q^T : lane holds query column li, keys 32*jb + 8r + 4hh + q ----
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[j][v] = 0.f;
          // k-step major: the two accumulators advance together.  Product i
          // is (k-step i / 2, key group i % 2); its K operand is read from LDS
          // kRA products ahead, and the scheduling fences keep that order
          // (left to itself the compiler reads each operand just before its
          // product, which then waits for the whole LDS round trip).
          constexpr int NP = 2 * NS;
          bf16x8 ka[NP];
          auto read_k = [&](int i) __attribute__((always_inline)) {
            ka[i] = as_bf16x8(&kcur[(32 * (2 * hk + (i & 1)) + li) * KST + 16 * (i >> 1) + 8 * hh]);
          };
#pragma unroll
          for (int i = 0; i < kRA; ++i) read_k(i);
          __builtin_amdgcn_s_setprio(1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            s[i & 1] = mfma32(ka[i], qf[i >> 1], s[i & 1]);
            if (i + kRA < NP) read_k(i + kRA);
            __builtin_amdgcn_sched_barrier(0);
          }
          __builtin_amdgcn_s_setprio(0);
          if (need_mask) {
            // words of 4 consecutive keys for this wave's 32 rows; bit li is
            // this lane's row
            const uint32_t* hw = &sm.hid[tt & 1][w][4 * hh];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const uint4 h4 = *reinterpret_cast<const uint4*>(&hw[32 * (2 * hk + j) + 8 * r]);
                const uint32_t hq[4] = {h4.x, h4.y, h4.z, h4.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const int v = 4 * r + q;
                  s[j][v] = hide_if(hq[q], li, s[j][v]);
                }
              }
          }
        };
        auto half_pv = [&](int hk, f32x16 (&s)[2]) __attribute__((always_inline)) {
          // ---- online softmax in the log2 domain ----
          // P is taken against the running reference m_run as it stands; only
          // when some row has no reference yet or a lane's P sum leaves
          // [0, 2^20] is the half's row maximum formed, the accumulators
          // rescaled and P recomputed.  O and l are sums against the same
          // reference, so their ratio does not depend on it.
          bf16x8 pb[2][2];
          float hs = 0.f;
          auto make_p = [&](float base) __attribute__((always_inline)) {
            hs = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                for (int e8 = 0; e8 < 8; ++e8) {
                  const float pv = fast_exp2(fmaf(s[j][8 * t2 + e8], a.scale_log2, -base));
                  hs += pv;
                  pb[j][t2][e8] = (bf16)pv;
                }
          };
          // the first V^T operands of the PV products are read before the
          // exponentials, whose time covers their LDS round trip
          constexpr int NP = 4 * ND;   // product i: (j, t2) = (i / (2 ND), i / ND % 2), d = i % ND
          bf16x8 va[NP];
          auto read_v = [&](int i) __attribute__((always_inline)) {
            const int j = i / (2 * ND), t2 = (i / ND) & 1, d = i % ND;
            va[i] = as_bf16x8(&vcur[(32 * d + li) * VTS + 32 * (2 * hk + j) + 16 * t2 + 8 * hh]);
          };
#pragma unroll
          for (int i = 0; i < kRA; ++i) read_v(i);
          bool ok = __all(m_run > -INFINITY);
          if (ok) {
            make_p(m_run);
            ok = __all(hs <= 0x1p20f);
          }
          if (!ok) {
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[j][v]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx * a.scale_log2);
            const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[d][v] *= alpha;
            l_run *= alpha;
            rs *= alpha;
            m_run = m_new;
            make_p((m_run == -INFINITY) ? 0.f : m_run);
          }
          rs += hs;
          // ---- O^T += V^T P^T ----
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            acc[i % ND] = mfma32(va[i], pb[i / (2 * ND)][(i / ND) & 1], acc[i % ND]);
            if (i + kRA < NP) read_v(i + kRA);
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        if constexpr (PAIR) {
          // Double-buffered: block t+1 goes into the other buffers while
          // block t computes, one barrier per block.  The buffers of block
          // t+1 held block t-1, which every wave finished before the last
          // barrier.  One set of registers carries K_{t+1} (loaded in the
          // middle of block t-1), then V_{t+1}, then K_{t+2}.
          if (has_next) {
            store_k<D>(st, sm.k[buf ^ 1], t);
            load_v<D>(st, vbase, k0n, t);
          }
          // (a wave whose query block does not see the block only stages
          // and meets the barrier)
          {
            f32x16 s0[2];
            if (sees) half_s(0, s0);
            if (sees) half_pv(0, s0);
          }
          f32x16 s1[2];
          if (sees) half_s(1, s1);
          if (has_next) {
            store_vt<D>(st, sm.vt[buf ^ 1], t);
            if (nm_next && t < BK) stage_hidden(bnext, buf ^ 1);
          }
          // read on every path (see below); block t+2's K and bounds
          const int e2 = __builtin_amdgcn_readfirstlane(e2_pending);
          if (tt + 2 < cnt) {
            const int k02 = block_start(e2);
            load_k<D>(st, kbase, k02, t);
            if (block_masked(e2, k02) && t < BK) bnext = load_bnd(bbase, k02, Sk, t);
          }
          if (sees) half_pv(1, s1);
          asm volatile("" : "+v"(rs));
          l_run += rs;
          // the next item's header, one scalar load in each of the first two blocks
          if (tt == 0) pf.fetch_entry(iq, sm.hdr[(n + 1) & 1]);
          if (tt == 1) pf.fetch_count(iq);
          __syncthreads();   // block t+1 is staged; every wave is done with block t's buffers
          if (!has_next) break;
          e_cur = e_next;
          e_next = e2;
        } else {
        // (a wave whose query block does not see the block only stages and
        // meets the barriers)
        {
          f32x16 s0[2];
          if (sees) half_s(0, s0);
          __syncthreads();   // V^T of this block is in LDS
          if (sees) half_pv(0, s0);
        }
        f32x16 s1[2];
        if (sees) half_s(1, s1);
        __syncthreads();   // every wave is done with this block's K
        int4 breg = make_int4(0, 0, 0, 0);
        if (has_next) {
          store_k<D>(st, sm.k[0], t);
          if (nm_next && t < BK) breg = load_bnd(bbase, k0n, Sk, t);
          load_v<D>(st, vbase, k0n, t);
        }
        if (sees) half_pv(1, s1);
        // keep the row sum here: left to itself the compiler sinks it past
        // the barrier and keeps the P values alive into the next loads
        asm volatile("" : "+v"(rs));
        l_run += rs;
        // the other mask buffer was last read before the first barrier of block t-1
        if (nm_next && t < BK) stage_hidden(breg, (tt + 1) & 1);

        // the next item's header, one scalar load in each of the first two blocks
        if (tt == 0) pf.fetch_entry(iq, sm.hdr[(n + 1) & 1]);
        if (tt == 1) pf.fetch_count(iq);
        __syncthreads();   // every wave is done with this block's V^T; K_{t+1} is in LDS
        // read on every path, so that no trip back to the top of the loop
        // leaves the list load in flight (the compiler would then wait for
        // every load, the next K block's included, at the top)
        const int e2 = __builtin_amdgcn_readfirstlane(e2_pending);
        if (!has_next) break;
        store_vt<D>(st, sm.vt[0], t);
        if (tt + 2 < cnt) load_k<D>(st, kbase, block_start(e2), t);
        e_cur = e_next;
        e_next = e2;
        }
      }
      if (cnt == 1) pf.fetch_count(iq);
      pf.publish(iq, sm.hdr[(n + 1) & 1], t);
    } else {
      pf.finish_now(iq, sm.hdr[(n + 1) & 1], t);
    }

    // ---- finalise: O = acc / l, LSE = (m + log2 l) ln 2.  A split item's
    // half writes the same, its own O and LSE, into its slot for the merge ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (split) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const int r = qrow - qb * BQ;   // row within the block
      bf16* orow = reinterpret_cast<bf16*>(a.partials) + ((size_t)idx * BQ + r) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 ov;
#pragma unroll
          for (int q = 0; q < 4; ++q) ov[q] = (bf16)(acc[d][4 * rr + q] * inv);
          *reinterpret_cast<bf16x4*>(&orow[32 * d + 8 * rr + 4 * hh]) = ov;
        }
      if (hh == 0) {
        float* plse = reinterpret_cast<float*>(reinterpret_cast<bf16*>(a.partials) + (size_t)2 * a.split_cap * (BQ * D));
        plse[(size_t)idx * BQ + r] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : INFINITY;
      }
    } else if (qrow < Sq) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      bf16* orow = a.o + (bh * Sq + qrow) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bf16x4 ov;
#pragma unroll
          for (int q = 0; q < 4; ++q) ov[q] = (bf16)(acc[d][4 * r + q] * inv);
          *reinterpret_cast<bf16x4*>(&orow[32 * d + 8 * r + 4 * hh]) = ov;
        }
      if (hh == 0) a.lse[bh * Sq + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : INFINITY;
    }
    __syncthreads();   // every thread has finished with LDS; the next header is in LDS
  }
  // The last workgroup to leave resets the queue counters for the next call.
  if (t == 0) {
    __threadfence();
    const uint32_t done = atomicAdd(&a.counters[kCtrFwdExit], 1u);
    if (done == gridDim.x - 1) {
      atomicExch(&a.counters[kCtrFwdNext], 0u);
      atomicExch(&a.counters[kCtrFwdExit], 0u);
    }
  }
}

int fwd_blocks_per_cu(int) { return 2; }

// Merge of the two halves of each split item (FlashMask-3 paper summary,
// abstract: softmax results over disjoint key ranges combine exactly through
// their log-sum-exps).  Each half left its own O_p (bf16) and LSE_p (+inf
// when the row sees no key of the half).  With M the larger finite LSE_p and
// w_p = exp(LSE_p - M) (0 for an empty half):
//   O = (w_0 O_0 + w_1 O_1) / (w_0 + w_1),  LSE = M + log(w_0 + w_1),
// and O = 0, LSE = +inf when both halves are empty.  Workgroup j merges
// split item j; thread t takes row t / 2 and half t % 2 of its columns.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const FwdArgs a) {
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nQ);
  const uint32_t n_real = min(a.counters[kCtrFwdItems], max_items);
  const uint32_t nsplit = min(min(a.counters[kCtrFwdSplit], (uint32_t)max(a.split_cap, 0)), n_real);
  const bf16* po = reinterpret_cast<const bf16*>(a.partials);
  const float* pl = reinterpret_cast<const float*>(po + (size_t)2 * a.split_cap * (BQ * D));
  const int t = threadIdx.x, r = t >> 1, c0 = (t & 1) * (D / 2);
  for (uint32_t j = blockIdx.x; j < nsplit; j += gridDim.x) {
    const uint32_t it = min(a.queue[j], max_items - 1);
    const long bh = it / a.nQ;
    const int row = (int)(it % a.nQ) * BQ + r;
    if (row >= a.Sq) continue;
    const float L0 = pl[(size_t)(2 * j) * BQ + r], L1 = pl[(size_t)(2 * j + 1) * BQ + r];
    const bool e0 = !(L0 < INFINITY), e1 = !(L1 < INFINITY);
    const float M = e0 ? L1 : e1 ? L0 : fmaxf(L0, L1);
    const float w0 = e0 ? 0.f : __expf(L0 - M), w1 = e1 ? 0.f : __expf(L1 - M);
    const float wsum = w0 + w1;
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const bf16* o0 = po + ((size_t)(2 * j) * BQ + r) * D;
    const bf16* o1 = po + ((size_t)(2 * j + 1) * BQ + r) * D;
    bf16* orow = a.o + (bh * a.Sq + row) * D;
#pragma unroll
    for (int c = c0; c < c0 + D / 2; c += 8) {
      const bf16x8 x = as_bf16x8(o0 + c), y = as_bf16x8(o1 + c);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)(((float)x[e] * w0 + (float)y[e] * w1) * inv);
      *reinterpret_cast<bf16x8*>(&orow[c]) = o;
    }
    if ((t & 1) == 0) a.lse[bh * a.Sq + row] = wsum > 0.f ? M + __logf(wsum) : INFINITY;
  }
}

hipError_t launch_attn_fwd(const FwdArgs& a, int head_dim, int grid, hipStream_t stream,
                           const KernelEvents& ev) {
  hipError_t err;
  if (ev.begin && (err = hipEventRecord(ev.begin, stream)) != hipSuccess) return err;
  const bool split = a.split_cap > 0;
  if (head_dim == 128) {
    if (split)
      attn_fwd_kernel<128, true, false><<<grid, 256, 0, stream>>>(a);
    else
      attn_fwd_kernel<128, false, false><<<grid, 256, 0, stream>>>(a);
  } else {
    if (split)
      attn_fwd_kernel<64, true, false><<<grid, 256, 0, stream>>>(a);
    else
      attn_fwd_kernel<64, false, false><<<grid, 256, 0, stream>>>(a);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.split_cap > 0 && grid > 0) {
    // the number of split items is on the device: one workgroup per
    // possible split item, up to the grid size, each looping
    const int mgrid = a.split_cap < grid ? a.split_cap : grid;
    if (head_dim == 128)
      fwd_merge_kernel<128><<<mgrid, 256, 0, stream>>>(a);
    else
      fwd_merge_kernel<64><<<mgrid, 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // the end event covers the merge of split items too: it is part of the forward
  if (ev.end && (err = hipEventRecord(ev.end, stream)) != hipSuccess) return err;
  return hipSuccess;
}

int fwd_pair_blocks_per_cu() { return 1; }

hipError_t launch_attn_fwd_pair(const FwdArgs& a, int grid, hipStream_t stream, const KernelEvents& ev) {
  hipError_t err;
  if (ev.begin && (err = hipEventRecord(ev.begin, stream)) != hipSuccess) return err;
  if (grid > 0) attn_fwd_kernel<128, false, true><<<grid, 512, 0, stream>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev.end && (err = hipEventRecord(ev.end, stream)) != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace fm
