// Forward of column-sparse masked attention with E4M3 (OCP fp8) inputs on
// gfx950's fp8 matrix cores.  The pages name FP8 mixed precision as part of
// FlashMask V3 (PaddlePaddle 3.2.0 release note, FlashMask V3 highlights);
// the mask handling is the one of the bf16 forward (FlashMask-3 paper
// summary, abstract: only tiles the column-wise sparse mask does not fully
// mask are computed).
//
// Values are decode(code) * descale with one fp32 descale per tensor.  Both
// products run as v_mfma_scale_f32_32x32x64_f8f6f4 (64-deep, E4M3 x E4M3,
// unit block scales), twice the bf16 rate:
//   S^T = K Q^T        the Q and K descales and the softmax scale are folded
//                      into the exponent's multiplier;
//   O^T += V^T P^T     P (in (0, 2^8], the online softmax moves its reference
//                      only when a row's maximum grows by more than 8 in the
//                      log2 domain) is rounded to E4M3; the row sum l is taken
//                      from the unrounded fp32 P, so LSE is as exact as the
//                      bf16 forward's; O = acc * descale_v / l.
//
// Operand layout.  An fp8 MFMA operand is 32 bytes per lane: lane (i, g),
// i = lane % 32, g = lane / 32, holds 32 k-values of row (or column) i, and
// A and B take the same k-values from the same (g, byte) places, so any
// assignment of the k index to (g, byte) works as long as both sides use it.
//   S: byte b of group g is head-dim 64 kk + 32 g + b (both from memory rows).
//   PV: the S accumulator of a 32-key block leaves lane (i, g) the keys
//       8 r + 4 g + q (r, q < 4) of query i; P of the two 32-key blocks j of a
//       64-key half packs as byte 16 j + 4 r + q, and V^T rows in LDS hold
//       the keys in that order (key x of half hk at 64 hk + 32 g + 16 j +
//       4 r + q), so the A operand is again 32 contiguous bytes.
// V is transposed while it is staged: each thread loads 4 keys x 16 columns
// and turns the 4 x 4 byte blocks around with byte permutes.
//
// The pipeline is the bf16 forward's (K of block t+1 loaded during S of t, V
// during its softmax and PV; three barriers per block); only head_dim 128.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int D8 = 128;          // head dimension (bytes per row)
constexpr int KST8 = D8 + 16;    // K row stride in LDS (bytes): conflict-free 16-byte reads
constexpr int VTS8 = BK + 16;    // V^T row stride in LDS (bytes)

struct alignas(16) Fp8Smem {
  uint8_t k[BK * KST8];          // K tile, one key per row
  uint8_t vt[D8 * VTS8];         // V^T tile, one head-dim column per row, keys in PV order
  uint32_t hid[2][BQ / 32][BK];  // hidden-row words of partial tiles (blocks t even / odd)
  uint32_t hdr[2][4];            // headers of this and the next work item
};

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 (E4M3) for both operands, block scales 2^0 (E8M0 code 127)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x4 load16(BufRsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// 32 bytes at a 16-byte aligned LDS address as one fp8 operand
__device__ __forceinline__ i32x8 lds32(const uint8_t* p) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Place of a group of 4 keys 4u..4u+3 (u < 32) inside a V^T row (see the
// operand layout above).
__device__ __forceinline__ int vt8_pos(int u) {
  return 64 * (u >> 4) + 32 * (u & 1) + 16 * ((u >> 3) & 1) + 4 * ((u >> 1) & 3);
}

// Global -> register staging of one key block (256 threads).
//   K: thread t holds 16-byte chunk t % 8 of rows t / 8 + 32 i (i < 4);
//   V: thread t holds columns 16 (t / 32) .. +15 of keys 4 (t % 32) .. +3.
struct Stage8 {
  i32x4 k[4];
  i32x4 v[4];
};

__device__ __forceinline__ void load_k8(Stage8& r, BufRsrc kb, int k0, unsigned t) {
  const uint32_t base = opaque((t >> 3) * D8 + (t & 7) * 16u) + (uint32_t)k0 * D8;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.k[i] = load16(kb, base + (uint32_t)i * 32 * D8);
}

__device__ __forceinline__ void store_k8(const Stage8& r, uint8_t* sk, unsigned t) {
  uint8_t* dst = sk + opaque((t >> 3) * KST8 + (t & 7) * 16u);
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<i32x4*>(dst + i * 32 * KST8) = r.k[i];
}

__device__ __forceinline__ void load_v8(Stage8& r, BufRsrc vb, int k0, unsigned t) {
  const uint32_t base = opaque(4u * (t & 31) * D8 + 16u * (t >> 5)) + (uint32_t)k0 * D8;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = load16(vb, base + (uint32_t)i * D8);
}

// Transposed store: dword m of key row i holds columns 4m..4m+3; the 4 x 4
// byte block of dword m of the four keys becomes one dword per column, whose
// bytes are the four keys in order.  Lanes 0..31 of a wave write 32 distinct
// dwords of one row.
__device__ __forceinline__ void store_vt8(const Stage8& r, uint8_t* vt, unsigned t) {
  uint8_t* dst = vt + opaque(16u * (t >> 5) * VTS8 + (uint32_t)vt8_pos((int)(t & 31)));
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t w0 = (uint32_t)r.v[0][m], w1 = (uint32_t)r.v[1][m];
    const uint32_t w2 = (uint32_t)r.v[2][m], w3 = (uint32_t)r.v[3][m];
    // interleave bytes of key pairs, then half-words of the pairs
    const uint32_t a_lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);   // w0.0 w1.0 w0.1 w1.1
    const uint32_t a_hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);   // w0.2 w1.2 w0.3 w1.3
    const uint32_t b_lo = __builtin_amdgcn_perm(w3, w2, 0x05010400u);
    const uint32_t b_hi = __builtin_amdgcn_perm(w3, w2, 0x07030602u);
    uint32_t* col = reinterpret_cast<uint32_t*>(dst + 4 * m * VTS8);
    col[0 * VTS8 / 4] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);   // column 4m
    col[1 * VTS8 / 4] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);   // column 4m + 1
    col[2 * VTS8 / 4] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);   // column 4m + 2
    col[3 * VTS8 / 4] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);   // column 4m + 3
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8_kernel(const Fp8FwdArgs a) {
  constexpr int ND = D8 / 32;   // 32-wide blocks of the head dimension
  __shared__ Fp8Smem sm;

  const unsigned t = threadIdx.x;
  const int lane = (int)(t & 63), w = (int)(t >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nQ);
  // in pair mode the queue holds pairs of query blocks, two tickets each
  const bool pairs = a.counters[kCtrFwdPairs] == 1u;
  const int nP = pairs ? (a.nQ + 1) >> 1 : 0;
  const uint32_t max_entries = (uint32_t)((long)a.B * a.H * (pairs ? nP : a.nQ));
  const uint32_t n_entries = min(a.counters[kCtrFwdItems], max_entries);
  const uint32_t n_items = pairs ? 2u * n_entries : n_entries;
  const int Sq = a.Sq, Sk = a.Sk;

  const ItemQueue iq{&a.counters[kCtrFwdNext], a.queue, a.cnt_q, n_items, max_items, a.nQ, a.H, a.Hm, a.nK,
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
    const BufRsrc qbase = make_rsrc(a.q + bh * Sq * (long)D8, (uint32_t)Sq * D8);
    const BufRsrc kbase = make_rsrc(a.k + bh * Sk * (long)D8, (uint32_t)Sk * D8);
    const BufRsrc vbase = make_rsrc(a.v + bh * Sk * (long)D8, (uint32_t)Sk * D8);
    const BufRsrc bbase = make_rsrc(a.bounds + bhm * Sk, (uint32_t)Sk * 16u);
    auto block_start = [&](int e) { return min(e & kListIndex, a.nK - 1) * BK; };
    auto block_masked = [&](int e, int k0) { return (e & kListPartial) || (k0 + BK > Sk); };

    const int qrow = qb * BQ + 32 * w + li;
    f32x16 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[d][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    if (cnt > 0) {
      const BufRsrc lbase = make_rsrc(lst, (uint32_t)cnt * 2u);
      auto list_at = [&](int i) -> uint32_t {
        return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(lbase, i * 2, 0, 0);
      };
      Stage8 st;
      // the first two list entries by scalar loads (waiting for a vector load
      // would also wait for every vector load issued before it)
      int e_cur = list_entry(lst, 0);
      int e_next = cnt > 1 ? list_entry(lst, 1) : 0;
      i32x8 qf[2];   // Q row of this lane (B operand of S^T = K Q^T): head-dims 64 kk + 32 hh ..
      {
        const int k0 = block_start(e_cur);
        load_k8(st, kbase, k0, t);
        load_v8(st, vbase, k0, t);
        int4 breg = make_int4(0, 0, 0, 0);
        if (block_masked(e_cur, k0) && t < BK) breg = load_bnd(bbase, k0, Sk, t);
        // issued after the block's loads: the staging below waits for those only
        const uint32_t qoff = (uint32_t)qrow * D8 + 32u * hh;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const i32x4 lo = load16(qbase, qoff + 64u * kk);
          const i32x4 hi = load16(qbase, qoff + 64u * kk + 16u);
          qf[kk] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        store_k8(st, sm.k, t);
        store_vt8(st, sm.vt, t);
        if (block_masked(e_cur, k0) && t < BK) {
          uint32_t wd[BQ / 32];
          hidden_rows(breg, qb * BQ, wd);
#pragma unroll
          for (int g = 0; g < BQ / 32; ++g) sm.hid[0][g][t] = wd[g];
        }
      }
      pf.stash(sm.hdr[(n + 1) & 1], t);
      if (cnt > 1) load_k8(st, kbase, block_start(e_next), t);
      __syncthreads();

      for (int tt = 0; tt < cnt; ++tt) {
        const int k0 = block_start(e_cur);
        const bool need_mask = block_masked(e_cur, k0);
        const bool has_next = tt + 1 < cnt;
        const int k0n = block_start(e_next);
        const bool nm_next = has_next && block_masked(e_next, k0n);
        const uint32_t e2_pending = (tt + 2 < cnt) ? list_at(tt + 2) : 0u;

        float rs = 0.f;
        // S^T of a 64-key half: lane holds query li, keys 32 (2 hk + j) + 8 r + 4 hh + q
        auto half_s = [&](int hk, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) s[j][v] = 0.f;
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              s[j] = mfma_fp8(lds32(&sm.k[(32 * (2 * hk + j) + li) * KST8 + 64 * kk + 32 * hh]), qf[kk], s[j]);
          __builtin_amdgcn_s_setprio(0);
          if (need_mask) {
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
                  s[j][v] = (hq[q] >> li) & 1u ? -INFINITY : s[j][v];
                }
              }
          }
        };
        auto half_pv = [&](int hk, f32x16 (&s)[2]) __attribute__((always_inline)) {
          float mx = -INFINITY;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[j][v]);
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float m_tile = mx * a.scale_log2;
          if (__any(m_tile > m_run + 8.f)) {
            const float m_new = fmaxf(m_run, m_tile);
            const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc[d][v] *= alpha;
            l_run *= alpha;
            rs *= alpha;
            m_run = m_new;
          }
          const float base = (m_run == -INFINITY) ? 0.f : m_run;
          // P of both 32-key blocks, rounded to E4M3: byte 16 j + v of the
          // operand is key 32 j + 8 (v / 4) + 4 hh + v % 4
          i32x8 pb;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              float p[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                p[q] = fast_exp2(fmaf(s[j][4 * c + q], a.scale_log2, -base));
                rs += p[q];
              }
              int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
              wd = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], wd, true);
              pb[4 * j + c] = wd;
            }
          // O^T += V^T P^T
#pragma unroll
          for (int d = 0; d < ND; ++d)
            acc[d] = mfma_fp8(lds32(&sm.vt[(32 * d + li) * VTS8 + 64 * hk + 32 * hh]), pb, acc[d]);
        };
        {
          f32x16 s0[2];
          half_s(0, s0);
          __syncthreads();   // V^T of this block is in LDS
          half_pv(0, s0);
        }
        f32x16 s1[2];
        half_s(1, s1);
        __syncthreads();   // every wave is done with this block's K
        int4 breg = make_int4(0, 0, 0, 0);
        if (has_next) {
          store_k8(st, sm.k, t);
          if (nm_next && t < BK) breg = load_bnd(bbase, k0n, Sk, t);
          load_v8(st, vbase, k0n, t);
        }
        half_pv(1, s1);
        asm volatile("" : "+v"(rs));
        l_run += rs;
        if (nm_next && t < BK) {
          uint32_t wd[BQ / 32];
          hidden_rows(breg, qb * BQ, wd);
#pragma unroll
          for (int g = 0; g < BQ / 32; ++g) sm.hid[(tt + 1) & 1][g][t] = wd[g];
        }
        if (tt == 0) pf.fetch_entry(iq, sm.hdr[(n + 1) & 1]);
        if (tt == 1) pf.fetch_count(iq);
        __syncthreads();   // every wave is done with this block's V^T; K_{t+1} is in LDS
        if (has_next) {
          store_vt8(st, sm.vt, t);
          int e2 = 0;
          if (tt + 2 < cnt) {
            e2 = __builtin_amdgcn_readfirstlane(e2_pending);
            load_k8(st, kbase, block_start(e2), t);
          }
          e_cur = e_next;
          e_next = e2;
        }
      }
      if (cnt == 1) pf.fetch_count(iq);
      pf.publish(iq, sm.hdr[(n + 1) & 1], t);
    } else {
      pf.finish_now(iq, sm.hdr[(n + 1) & 1], t);
    }

    // ---- finalise: O = acc descale_v / l, LSE = (m + log2 l) ln 2 ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qrow < Sq) {
      const float inv = l_tot > 0.f ? a.o_scale / l_tot : 0.f;
      bf16* orow = a.o + (bh * Sq + qrow) * D8;
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
    __syncthreads();
  }
  if (t == 0) {
    __threadfence();
    const uint32_t done = atomicAdd(&a.counters[kCtrFwdExit], 1u);
    if (done == gridDim.x - 1) {
      atomicExch(&a.counters[kCtrFwdNext], 0u);
      atomicExch(&a.counters[kCtrFwdExit], 0u);
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const Fp8FwdArgs& a, int grid, hipStream_t stream, const KernelEvents& ev) {
  hipError_t err;
  if (ev.begin && (err = hipEventRecord(ev.begin, stream)) != hipSuccess) return err;
  attn_fwd_fp8_kernel<<<grid, 256, 0, stream>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev.end && (err = hipEventRecord(ev.end, stream)) != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace fm
