// Backward of column-sparse masked attention (bf16 MFMA, fp32 accumulate):
// the key-stationary half.
//
//   bwd_pre_kernel   Delta_i = sum_d dO_id O_id (fp32);
//   attn_bwd_kernel  persistent, key-block stationary: each workgroup takes an
//                    item (batch*head, key block), keeps that block's K and V
//                    in registers (32 keys per wave) and its dK, dV
//                    accumulators in registers, and walks the list of query
//                    blocks that see the key block (the tiles the mask does not
//                    skip), 64 query rows at a time:
//                        S = Q K^T, P = exp(S - LSE) (interval mask on partial
//                        tiles only), dP = dO V^T, dS = P (dP - Delta) scale,
//                        dV += P^T dO, dK += dS^T Q;
//   attn_bwd_dq_kernel (its own file) then computes dQ query-stationary.
// dQ is not accumulated here: fp32 atomic adds into a shared accumulator run
// at a fraction of the rate of plain stores on this GPU, and at this kernel's
// speed they, not the matrix cores, would set its pace.
// With S = Q K^T computed as C[i][j] a lane holds one key and several query
// rows, which is exactly the A-operand shape of P^T dO and dS^T Q.  Each chunk
// of Q and dO is therefore staged twice, row-major (A operands of S and dP)
// and transposed (B operands of dV and dK), so that every MFMA operand read
// from LDS is one 16-byte load.  The next chunk is fetched into registers
// while the current one computes.
#include <climits>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace fm {

constexpr int QC = 64;   // query rows per backward chunk
constexpr int CPB = BQ / QC;   // chunks per query block

// ---------------------------------------------------------------- prologue
// Delta of every row; thread groups of D/8 threads per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o,
                                                      const bf16* __restrict__ dout,
                                                      float* __restrict__ delta, long rows) {
  constexpr int TPR = D / 8;   // threads per row, 8 elements each
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / TPR;
  const int c = (int)(gid % TPR);
  float sum = 0.f;
  if (row < rows) {
    const bf16x8 ov = reinterpret_cast<const bf16x8*>(o)[row * TPR + c];
    const bf16x8 dv = reinterpret_cast<const bf16x8*>(dout)[row * TPR + c];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += (float)ov[e] * (float)dv[e];
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (row < rows && c == 0) delta[row] = sum;
}

// ---------------------------------------------------------------- main
// Row terms ride in the matrix products.  Each staged Q row carries, in the
// 16 columns after its D values, the pair (hi, lo) of bf16 numbers whose sum
// is -LSE / scale to about 16 bits (zeros elsewhere), and each dO row the pair
// for -Delta.  With a constant B operand of ones in those two columns, one
// more k-step of S = Q K^T and dP = dO V^T yields S - LSE / scale and
// dP - Delta, so P = exp2(scale log2(e) S') and dS = scale P dP' need no
// per-row value in the lanes, whose rows differ from lane to lane.
template <int D>
struct alignas(16) BwdSmem {
  static constexpr int QST = D + 24;   // Q / dO row stride: D values, 16 row-term columns, pad
  static constexpr int QTS = QC + 8;   // Q^T / dO^T row stride; rows in vt_pos order
  bf16 q[QC * QST];
  bf16 dout[QC * QST];
  bf16 qt[D * QTS];
  bf16 dot[D * QTS];
  uint32_t item;
};

// Place of row x (0 <= x < QC) inside a Q^T / dO^T row: bits 2 and 3 of the
// offset within each group of 16 swapped, so that the 8 query rows one lane
// holds in the P^T (dS^T) operand are 8 neighbouring elements.
__device__ __forceinline__ int qt_pos(int x) { return (x & ~15) | perm16(x & 15); }

// Global -> register staging of one chunk of QC query rows of Q and dO
// (256 threads).  A unit is 4 consecutive rows (4m .. 4m+3) x 8 head-dim
// columns (chunk c) of one of the two tensors.  Each group of 16 lanes takes 4
// consecutive m by 4 consecutive c: with the row stride of 16 bytes past a
// multiple of 256, the 16 row-major 16-byte stores of a group then cover all
// LDS banks once, and the transposed 8-byte stores of a group fall on 8
// distinct bank pairs.  A wave's 4 groups cover 16 chunks of 4 rows (whole
// 256-byte rows for D = 128) so that the global loads stay row-contiguous.
// Threads < 2*QC also carry the LSE (first QC) or Delta (next QC) of one row.
template <int D>
struct ChunkStage {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int NPAIR = (QC / 4) * CPR;   // units per tensor (a multiple of 64)
  static constexpr int NU = (2 * NPAIR + 255) / 256;   // units per thread (some idle if < 256)
  static_assert(NPAIR % 64 == 0, "a unit's tensor must be uniform across a wave");
  static_assert(CPR % 4 == 0 && QC % 16 == 0, "groups are 4 row-units x 4 chunks");
  bf16x8 v[NU][4];
  float row_term;

  // 0 = Q, 1 = dO; the same in every lane of a wave (NPAIR is a multiple of 64)
  static __device__ __forceinline__ int tensor(unsigned t, int j) {
    return __builtin_amdgcn_readfirstlane((int)((t + 256u * j) / NPAIR));
  }
  static __device__ __forceinline__ bool active(unsigned t, int j) { return t + 256u * j < 2u * NPAIR; }
  // unit p = (group G, lane-in-group l): chunk c = 4 (G % (CPR/4)) + l / 4,
  // row-unit m = 4 (G / (CPR/4)) + l % 4
  static __device__ __forceinline__ int row(unsigned t, int j) {
    const unsigned p = (t + 256u * j) % NPAIR;
    return 4 * (int)(4u * ((p >> 4) / (CPR / 4)) + (p & 3u));
  }
  static __device__ __forceinline__ int col(unsigned t) {
    const unsigned p = t % NPAIR;   // 256 % NPAIR == 0, so the same for every j
    return (int)(4u * ((p >> 4) % (CPR / 4)) + ((p >> 2) & 3u));
  }
};

template <int D>
__device__ __forceinline__ void load_chunk(ChunkStage<D>& r, BufRsrc qb, BufRsrc ob, BufRsrc lb,
                                           BufRsrc db, int q0, unsigned t) {
  using C = ChunkStage<D>;
  // The row term first: the oldest load of the chunk, so that waiting for it
  // never waits for memory operations issued after the chunk's loads (the
  // dQ atomics).  Wave 0 carries LSE, wave 1 Delta (QC is the wave size);
  // rows past the end read 0 (buffer range check) and are fixed on store.
  static_assert(QC == 64, "one wave per row term");
  if (t < 2 * QC) {
    const BufRsrc src = __builtin_amdgcn_readfirstlane((int)(t < QC)) ? lb : db;   // per wave
    r.row_term = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(src, (q0 + (int)(t % QC)) * 4, 0, 0));
  }
#pragma unroll
  for (int j = 0; j < C::NU; ++j) {
    if (!C::active(t, j)) continue;
    const BufRsrc src = C::tensor(t, j) == 0 ? qb : ob;
    const uint32_t base =
        opaque(((uint32_t)C::row(t, j) * C::CPR + C::col(t)) * 16u) + (uint32_t)q0 * (D * 2);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r.v[j][rr] = buf_load16(src, base + (uint32_t)rr * (D * 2));
  }
}

template <int D, typename Smem>
__device__ __forceinline__ void store_chunk(const ChunkStage<D>& r, Smem& sm, int q0, int Sq,
                                            float scale, unsigned t) {
  using C = ChunkStage<D>;
  constexpr int QST = Smem::QST, QTS = Smem::QTS;
#pragma unroll
  for (int j = 0; j < C::NU; ++j) {
    if (!C::active(t, j)) continue;
    const bool is_q = C::tensor(t, j) == 0;
    bf16* rm = (is_q ? sm.q : sm.dout) + opaque(C::row(t, j) * QST + 8 * C::col(t));
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) *reinterpret_cast<bf16x8*>(rm + rr * QST) = r.v[j][rr];
    bf16* tp = (is_q ? sm.qt : sm.dot) + opaque((8 * C::col(t)) * QTS + qt_pos(C::row(t, j)));
    const bf16x16 p01 = __builtin_shufflevector(r.v[j][0], r.v[j][1], 0, 8, 1, 9, 2, 10, 3, 11, 4,
                                                12, 5, 13, 6, 14, 7, 15);
    const bf16x16 p23 = __builtin_shufflevector(r.v[j][2], r.v[j][3], 0, 8, 1, 9, 2, 10, 3, 11, 4,
                                                12, 5, 13, 6, 14, 7, 15);
#define FM_T_ROW(e)                                                                       \
  *reinterpret_cast<bf16x4*>(tp + (e) * QTS) =                                            \
      __builtin_shufflevector(p01, p23, 2 * (e), 2 * (e) + 1, 16 + 2 * (e), 17 + 2 * (e))
    FM_T_ROW(0); FM_T_ROW(1); FM_T_ROW(2); FM_T_ROW(3);
    FM_T_ROW(4); FM_T_ROW(5); FM_T_ROW(6); FM_T_ROW(7);
#undef FM_T_ROW
  }
  // row terms: -LSE / scale into the Q row (-inf for rows past the end and
  // rows no key sees, so P = 0 there), -Delta into the dO row, each as a
  // (hi, lo) pair of bf16
  if (t < 2 * QC) {
    const bool is_q = t < QC;
    const int row = (int)t % QC;
    float x;
    if (is_q) {
      const bool live = q0 + row < Sq && r.row_term < INFINITY;
      x = live ? -r.row_term / scale : -INFINITY;
    } else {
      x = -r.row_term;
    }
    const bf16 hi = (bf16)x;
    const bf16 lo = (bf16)(x == -INFINITY ? 0.f : x - (float)hi);
    bf16* dst = (is_q ? sm.q : sm.dout) + row * QST + D;
    dst[0] = hi;
    dst[1] = lo;
  }
}

// Columns D .. D+15 of every staged Q and dO row start as zero (the row-term
// pair is written into the first two for each chunk).
template <int D, typename Smem>
__device__ __forceinline__ void zero_row_terms(Smem& sm, unsigned t) {
  constexpr int QST = Smem::QST;
  if (t < 2 * QC) {
    bf16* dst = (t < QC ? sm.q : sm.dout) + (int)(t % QC) * QST + D;
    *reinterpret_cast<bf16x8*>(dst) = zero_bf16x8();
    *reinterpret_cast<bf16x8*>(dst + 8) = zero_bf16x8();
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_kernel(const BwdArgs a) {
  constexpr int NS = D / 16, ND = D / 32;
  using Smem = BwdSmem<D>;
  constexpr int QST = Smem::QST, QTS = Smem::QTS;
  __shared__ Smem sm;

  const unsigned t = threadIdx.x;
  const int lane = (int)(t & 63), w = (int)(t >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nK);
  const uint32_t n_items = min(a.counters[kCtrBwdItems], max_items);
  const int Sq = a.Sq, Sk = a.Sk;

  zero_row_terms<D>(sm, t);   // made visible by the first barrier below
  for (;;) {
    if (t == 0) sm.item = atomicAdd(&a.counters[kCtrBwdNext], 1u);
    __syncthreads();
    const uint32_t idx = __builtin_amdgcn_readfirstlane(sm.item);
    if (idx >= n_items) break;
    // values loaded from memory are not known to be uniform: broadcast them,
    // so that the buffer resources built from them stay in scalar registers
    const uint32_t it = __builtin_amdgcn_readfirstlane(min(a.queue[idx], max_items - 1));
    const long bh = it / a.nK;
    const int kb = (int)(it % a.nK);
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const long bhm = (long)b * a.Hm + (a.Hm == 1 ? 0 : h);
    const int cnt = __builtin_amdgcn_readfirstlane(min(a.cnt_k[bhm * a.nK + kb], a.nQ));
    const uint16_t* lst = a.list_k + (bhm * a.nK + kb) * (long)a.nQ;
    const int k0 = kb * BK;
    const bool ragged_k = k0 + BK > Sk;
    const BufRsrc qbase = make_rsrc(a.q + bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
    const BufRsrc obase = make_rsrc(a.dout + bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
    const BufRsrc kbase = make_rsrc(a.k + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
    const BufRsrc vbase = make_rsrc(a.v + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
    const BufRsrc lbase = make_rsrc(a.lse + bh * Sq, (uint32_t)Sq * 4u);
    const BufRsrc dbase = make_rsrc(a.delta + bh * Sq, (uint32_t)Sq * 4u);
    // Each item starts its walk at block kb % cnt (and wraps): neighbouring
    // key blocks, which run at the same time, then add into different dQ rows.
    const int rot = cnt > 0 ? kb % cnt : 0;
    auto list_at = [&](int i) {
      const int j = i + rot;
      return list_entry(lst, j < cnt ? j : j - cnt);
    };

    // this lane's key: bounds (keys past the end are masked for every row),
    // K and V rows as MFMA B operands
    const int jrow = k0 + 32 * w + li;
    int4 bd = make_int4(INT_MIN, INT_MAX, 0, 0);
    if (jrow < Sk) bd = a.bounds[bhm * Sk + jrow];
    bf16x8 kf[NS], vf[NS];
    {
      const uint32_t off = ((uint32_t)jrow * D + 8u * hh) * 2u;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kf[s] = buf_load16(kbase, off + 32u * s);
        vf[s] = buf_load16(vbase, off + 32u * s);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        pin_agpr(kf[s]);
        pin_agpr(vf[s]);
      }
    }
    f32x16 dk[ND], dv[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        dk[d][v] = 0.f;
        dv[d][v] = 0.f;
      }

    const int nchunks = CPB * cnt;   // each query block is CPB chunks of QC rows
    if (nchunks > 0) {
      // chunk c starts at row block_row(c) * BQ + (c % CPB) * QC
      auto chunk_q0 = [&](int c) __attribute__((always_inline)) {
        const int e = list_at(c / CPB);
        return min(e & kListIndex, a.nQ - 1) * BQ + (c % CPB) * QC;
      };
      ChunkStage<D> cs;
      int e_cur = list_at(0);
      load_chunk<D>(cs, qbase, obase, lbase, dbase, chunk_q0(0), t);
      store_chunk<D>(cs, sm, chunk_q0(0), Sq, a.scale, t);
      __syncthreads();
      // Per chunk c (its Q, dO, Q^T, dO^T and row terms in LDS):
      //   chunk c+1 -> registers; S, dP, P, dS, dV, dK | barrier |
      //   chunk c+1 -> LDS | barrier
      for (int c = 0; c < nchunks; ++c) {
        const int q0 = min(e_cur & kListIndex, a.nQ - 1) * BQ + (c % CPB) * QC;
        const bool need_mask = (e_cur & kListPartial) || ragged_k;
        const bool has_next = c + 1 < nchunks;
        int e_next = e_cur;
        if (has_next && (c + 1) % CPB == 0)
          e_next = list_at((c + 1) / CPB);
        if (has_next) load_chunk<D>(cs, qbase, obase, lbase, dbase, chunk_q0(c + 1), t);

        // S, dP, P, dS, dV and dK of the chunk's two halves (32 rows each),
        // software-pipelined so that the vector work of one half runs while
        // the matrix cores work on the other:
        //   (a)  S, dP of half 0
        //   (b1) S of half 1          |  P of half 0
        //   (b2) dP of half 1         |  dS of half 0
        //   (c1) dV from half 0       |  P of half 1
        //   (c2) dK from half 0       |  dS of half 1
        //   (d)  dV, dK from half 1
        // On partial tiles P is masked between the P and dS steps (a separate,
        // uniform branch that only rewrites P in place).
        // S, dP: lane holds key li, rows 32 ib + 8 r + 4 hh + q in element 4r+q.
        {
          f32x16 s0, dp0, s1, dp1;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            s0[v] = 0.f; dp0[v] = 0.f; s1[v] = 0.f; dp1[v] = 0.f;
          }
          bf16x8 pb[2][2], dsb[2][2];
          float pf[2][16];                 // P in fp32 between its step and dS's
          // B operand of the row-term k-step: ones in columns D, D+1
          bf16x8 ones = zero_bf16x8();
          if (hh == 0) {
            ones[0] = (bf16)1.0f;
            ones[1] = (bf16)1.0f;
          }
          auto q_op = [&](int ib, int kk) __attribute__((always_inline)) {
            return as_bf16x8(&sm.q[(32 * ib + li) * QST + 16 * kk + 8 * hh]);
          };
          auto o_op = [&](int ib, int kk) __attribute__((always_inline)) {
            return as_bf16x8(&sm.dout[(32 * ib + li) * QST + 16 * kk + 8 * hh]);
          };
          auto ot_op = [&](int ib, int d, int t2) __attribute__((always_inline)) {
            return as_bf16x8(&sm.dot[(32 * d + li) * QTS + 32 * ib + 16 * t2 + 8 * hh]);
          };
          auto qt_op = [&](int ib, int d, int t2) __attribute__((always_inline)) {
            return as_bf16x8(&sm.qt[(32 * d + li) * QTS + 32 * ib + 16 * t2 + 8 * hh]);
          };
          // P = exp2(S' scale log2(e)), S' = S - LSE / scale
          auto p_of = [&](const f32x16& sv, int v) __attribute__((always_inline)) {
            return fast_exp2(sv[v] * a.scale_log2);
          };
          // partial tile: P = 0 where the lane's key hides the row.  Bit
          // 8r + q of `hidden` covers row 32 ib + 8 r + 4 hh + q: the union of
          // the key's two intervals clipped to the half's 32 rows.
          auto mask_p = [&](int ib) __attribute__((always_inline)) {
            const int base = q0 + 32 * ib;
            auto clip = [&](int x) { return min(max(x, base), base + 32) - base; };
            auto rows = [](int lo, int hi) {
              return hi > lo ? (~0u >> (32 - hi)) & (~0u << lo) : 0u;
            };
            const uint32_t hidden =
                (rows(clip(bd.x), clip(bd.y)) | rows(clip(bd.z), clip(bd.w))) >> (4 * hh);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int keep = (int)(~hidden << (31 - (8 * (v >> 2) + (v & 3)))) >> 31;
              pf[ib][v] = __builtin_bit_cast(float, __builtin_bit_cast(int, pf[ib][v]) & keep);
            }
          };
          // scale * dS = scale P (dP - Delta) into the MFMA operand (dK then
          // needs no scaling); P packed
          auto ds_of = [&](const f32x16& dpv, int ib, int v) __attribute__((always_inline)) {
            const float p = pf[ib][v];
            const float dsv = (p * a.scale) * dpv[v];   // dP' = dP - Delta
            pb[ib][v >> 3][v & 7] = (bf16)p;
            dsb[ib][v >> 3][v & 7] = (bf16)dsv;
          };
          constexpr int EPK = 16 / NS;   // elements per MFMA in (b1), (b2)
          constexpr int EPC = 16 / ND;   // elements per MFMA in (c1), (c2)

          // (a): operand reads run 6 ahead of the MFMAs
          s0 = mfma32(q_op(0, NS), ones, s0);
          dp0 = mfma32(o_op(0, NS), ones, dp0);
#pragma unroll
          for (int kk = 0; kk < NS; ++kk) {
            s0 = mfma32(q_op(0, kk), kf[kk], s0);
            dp0 = mfma32(o_op(0, kk), vf[kk], dp0);
          }
          interleave_mfma<2 * NS + 2, 2 * NS + 2, 6, 0, 0>();
          __builtin_amdgcn_sched_barrier(0);
          // (b1)
          s1 = mfma32(q_op(1, NS), ones, s1);
#pragma unroll
          for (int kk = 0; kk < NS; ++kk) {
            s1 = mfma32(q_op(1, kk), kf[kk], s1);
#pragma unroll
            for (int e = 0; e < EPK; ++e) pf[0][EPK * kk + e] = p_of(s0, EPK * kk + e);
          }
          interleave_mfma<NS + 1, NS + 1, 3, 3 * EPK, 0>();
          __builtin_amdgcn_sched_barrier(0);
          if (need_mask) mask_p(0);
          __builtin_amdgcn_sched_barrier(0);
          // (b2)
          dp1 = mfma32(o_op(1, NS), ones, dp1);
#pragma unroll
          for (int kk = 0; kk < NS; ++kk) {
            dp1 = mfma32(o_op(1, kk), vf[kk], dp1);
#pragma unroll
            for (int e = 0; e < EPK; ++e) ds_of(dp0, 0, EPK * kk + e);
          }
          interleave_mfma<NS + 1, NS + 1, 3, 4 * EPK, 0>();
          __builtin_amdgcn_sched_barrier(0);
          // (c1)
#pragma unroll
          for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              dv[d] = mfma32(pb[0][t2], ot_op(0, d, t2), dv[d]);
#pragma unroll
              for (int e = 0; e < EPC / 2; ++e) {
                const int v = (EPC / 2) * (2 * d + t2) + e;
                pf[1][v] = p_of(s1, v);
              }
            }
          interleave_mfma<2 * ND, 2 * ND, 4, 3 * EPC / 2, 0>();
          __builtin_amdgcn_sched_barrier(0);
          if (need_mask) mask_p(1);
          __builtin_amdgcn_sched_barrier(0);
          // (c2)
#pragma unroll
          for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              dk[d] = mfma32(dsb[0][t2], qt_op(0, d, t2), dk[d]);
#pragma unroll
              for (int e = 0; e < EPC / 2; ++e) ds_of(dp1, 1, (EPC / 2) * (2 * d + t2) + e);
            }
          interleave_mfma<2 * ND, 2 * ND, 3, 4 * EPC / 2, 0>();
          __builtin_amdgcn_sched_barrier(0);
          // (d)
#pragma unroll
          for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              dv[d] = mfma32(pb[1][t2], ot_op(1, d, t2), dv[d]);
              dk[d] = mfma32(dsb[1][t2], qt_op(1, d, t2), dk[d]);
            }
          interleave_mfma<4 * ND, 4 * ND, 4, 0, 0>();
        }
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          pin_agpr(dv[d]);
          pin_agpr(dk[d]);
        }
        __syncthreads();   // every wave is done with this chunk's Q and dO
        if (has_next) store_chunk<D>(cs, sm, chunk_q0(c + 1), Sq, a.scale, t);

        __syncthreads();   // the next chunk is in LDS
        e_cur = e_next;
      }
    }

    // ---- write dK and dV: lane holds column 32d + li, keys 8r + 4hh + q ----
    {
      // uniform base + opaque 32-bit lane offset + constant: no per-element
      // 64-bit address is computed ahead and kept live through the loops
      const long base = (bh * Sk + k0) * D;
      const uint32_t lane_off = opaque((uint32_t)((32 * w + 4 * hh) * D + li));
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int jl = 32 * w + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (k0 + jl < Sk) {
            const uint32_t off = lane_off + (uint32_t)((8 * (v >> 2) + (v & 3)) * D + 32 * d);
            a.dk[base + off] = (bf16)dk[d][v];
            a.dv[base + off] = (bf16)dv[d][v];
          }
        }
    }
    __syncthreads();   // every thread has read sm.item and finished with LDS
  }
  if (t == 0) {
    __threadfence();
    const uint32_t done = atomicAdd(&a.counters[kCtrBwdExit], 1u);
    if (done == gridDim.x - 1) {
      atomicExch(&a.counters[kCtrBwdNext], 0u);
      atomicExch(&a.counters[kCtrBwdExit], 0u);
    }
  }
}

int bwd_blocks_per_cu(int) { return 1; }

hipError_t launch_attn_bwd(const BwdArgs& a, int head_dim, int grid, int dq_grid,
                           hipStream_t stream, const KernelEvents& ev) {
  const long rows = (long)a.B * a.H * a.Sq;
  hipError_t err;
  if (rows > 0) {
    const unsigned pre_grid = (unsigned)((rows * head_dim / 8 + 255) / 256);
    if (head_dim == 128)
      bwd_pre_kernel<128><<<pre_grid, 256, 0, stream>>>(a.o, a.dout, a.delta, rows);
    else
      bwd_pre_kernel<64><<<pre_grid, 256, 0, stream>>>(a.o, a.dout, a.delta, rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (ev.begin && (err = hipEventRecord(ev.begin, stream)) != hipSuccess) return err;
  if (grid > 0) {
    if (head_dim == 128)
      attn_bwd_kernel<128><<<grid, 256, 0, stream>>>(a);
    else
      attn_bwd_kernel<64><<<grid, 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (ev.end && (err = hipEventRecord(ev.end, stream)) != hipSuccess) return err;
  if (ev.begin2 && (err = hipEventRecord(ev.begin2, stream)) != hipSuccess) return err;
  if ((err = launch_attn_bwd_dq(a, head_dim, dq_grid, stream)) != hipSuccess) return err;
  if (ev.end2 && (err = hipEventRecord(ev.end2, stream)) != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace fm
