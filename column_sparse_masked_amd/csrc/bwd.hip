// Backward of column-sparse masked attention (bf16 MFMA, fp32 accumulate).
//
//   bwd_pre_kernel   Delta_i = sum_d dO_id O_id (fp32) and a zeroed fp32 dQ
//                    accumulator;
//   attn_bwd_kernel  persistent, key-block stationary: each workgroup takes an
//                    item (batch*head, key block), keeps that block's K and V
//                    in registers (32 keys per wave) and its dK, dV
//                    accumulators in registers, and walks the list of query
//                    blocks that see the key block (the tiles the mask does not
//                    skip), 64 query rows at a time:
//                        S = Q K^T, P = exp(S - LSE) (interval mask on partial
//                        tiles only), dP = dO V^T, dS = P (dP - Delta),
//                        dV += P^T dO, dK += dS^T Q,
//                        dQ += dS K   (fp32 atomics into the accumulator);
//   dq_convert_kernel  dQ = bf16(accumulator), round to nearest even.
// With S = Q K^T computed as C[i][j] a lane holds one key and several query
// rows, which is exactly the A-operand shape of P^T dO and dS^T Q.  Each chunk
// of Q and dO is therefore staged twice, row-major (A operands of S and dP)
// and transposed (B operands of dV and dK), and K is staged transposed once
// per item (B operand of dQ), so that every MFMA operand read from LDS is one
// 16-byte load.  The next chunk is fetched into registers while the current
// one computes, and the dQ atomics of a chunk are issued after those loads.
#include <climits>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace fm {

constexpr int QC = 64;   // query rows per backward chunk
constexpr int CPB = BQ / QC;   // chunks per query block

// ---------------------------------------------------------------- prologue
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o,
                                                      const bf16* __restrict__ dout,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_acc, long rows) {
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
    float4* z = reinterpret_cast<float4*>(dq_acc + row * D + 8 * c);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (row < rows && c == 0) delta[row] = sum;
}

// ---------------------------------------------------------------- main
template <int D>
struct alignas(16) BwdSmem {
  static constexpr int QST = D + 8;    // Q / dO row stride (elements)
  static constexpr int QTS = QC + 8;   // Q^T / dO^T row stride; rows in vt_pos order
  static constexpr int KTS = BK + 8;   // K^T row stride; keys in natural order
  static constexpr int DSS = BK + 8;   // dS row stride
  bf16 q[QC * QST];
  bf16 dout[QC * QST];
  bf16 qt[D * QTS];
  bf16 dot[D * QTS];
  bf16 kt[D * KTS];
  bf16 ds[QC * DSS];
  float lse2[QC];   // LSE * log2(e); +inf for rows past the end
  float delta[QC];
  uint32_t item;
};

// Place of row x (0 <= x < QC) inside a Q^T / dO^T row: bits 2 and 3 of the
// offset within each group of 16 swapped, so that the 8 query rows one lane
// holds in the P^T (dS^T) operand are 8 neighbouring elements.
__device__ __forceinline__ int qt_pos(int x) { return (x & ~15) | perm16(x & 15); }

// Global -> register staging of one chunk of QC query rows of Q and dO
// (256 threads).  A unit is 4 consecutive rows x 8 head-dim columns of one of
// the two tensors; the rows of the 16 lanes of a group are chosen so that the
// transposed 8-byte LDS stores fall on distinct banks.  Threads < 2*QC also
// carry the LSE (first QC) or Delta (next QC) of one row.
template <int D>
struct ChunkStage {
  static constexpr int CPR = D / 8;
  static constexpr int NPAIR = (QC / 4) * CPR;   // units per tensor (a multiple of 64)
  static constexpr int NU = (2 * NPAIR + 255) / 256;   // units per thread (some idle if < 256)
  static_assert(NPAIR % 64 == 0, "a unit's tensor must be uniform across a wave");
  bf16x8 v[NU][4];
  float row_term;

  // 0 = Q, 1 = dO; the same in every lane of a wave (NPAIR is a multiple of 64)
  static __device__ __forceinline__ int tensor(unsigned t, int j) {
    return __builtin_amdgcn_readfirstlane((int)((t + 256u * j) / NPAIR));
  }
  static __device__ __forceinline__ bool active(unsigned t, int j) { return t + 256u * j < 2u * NPAIR; }
  static __device__ __forceinline__ int row(unsigned t, int j) {
    const unsigned p = (t + 256u * j) % NPAIR;
    return 4 * (int)((p & 7u) + 8u * (p / (8u * CPR)));
  }
  static __device__ __forceinline__ int col(unsigned t) { return (int)((t >> 3) % CPR); }
};

template <int D>
__device__ __forceinline__ void load_chunk(ChunkStage<D>& r, BufRsrc qb, BufRsrc ob, BufRsrc lb,
                                           BufRsrc db, int q0, int Sq, unsigned t) {
  using C = ChunkStage<D>;
#pragma unroll
  for (int j = 0; j < C::NU; ++j) {
    if (!C::active(t, j)) continue;
    const BufRsrc src = C::tensor(t, j) == 0 ? qb : ob;
    const uint32_t base =
        opaque(((uint32_t)C::row(t, j) * C::CPR + C::col(t)) * 16u) + (uint32_t)q0 * (D * 2);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r.v[j][rr] = buf_load16(src, base + (uint32_t)rr * (D * 2));
  }
  r.row_term = 0.f;
  const int i = q0 + (int)(t % QC);
  if (t < QC) {
    const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lb, i * 4, 0, 0));
    r.row_term = (i < Sq) ? x * kLog2e : INFINITY;
  } else if (t < 2 * QC) {
    r.row_term = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(db, i * 4, 0, 0));
  }
}

template <int D, typename Smem>
__device__ __forceinline__ void store_chunk(const ChunkStage<D>& r, Smem& sm, unsigned t) {
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
  if (t < QC)
    sm.lse2[t] = r.row_term;
  else if (t < 2 * QC)
    sm.delta[t - QC] = r.row_term;
}

// K^T of a key block into LDS (once per item): thread t transposes 4*NV
// consecutive keys x 8 head-dim columns, as the forward does for V.
template <int D, typename Smem>
__device__ __forceinline__ void stage_kt(BufRsrc kb, int k0, Smem& sm, unsigned t) {
  constexpr int CPR = D / 8, NV = (BK / 4) * CPR / 256, KTS = Smem::KTS;
  const int key = 4 * NV * (int)((t & 7u) + 8u * (t / (8u * CPR)));
  const int c = (int)((t >> 3) % CPR);
  bf16x8 v[4 * NV];
  const uint32_t base = ((uint32_t)(k0 + key) * CPR + c) * 16u;
#pragma unroll
  for (int q = 0; q < 4 * NV; ++q) v[q] = buf_load16(kb, base + (uint32_t)q * (D * 2));
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    bf16* dst = sm.kt + (8 * c) * KTS + key + 4 * i;
    const bf16x16 p01 = __builtin_shufflevector(v[4 * i], v[4 * i + 1], 0, 8, 1, 9, 2, 10, 3, 11, 4,
                                                12, 5, 13, 6, 14, 7, 15);
    const bf16x16 p23 = __builtin_shufflevector(v[4 * i + 2], v[4 * i + 3], 0, 8, 1, 9, 2, 10, 3, 11,
                                                4, 12, 5, 13, 6, 14, 7, 15);
#define FM_T_ROW(e)                                                                       \
  *reinterpret_cast<bf16x4*>(dst + (e) * KTS) =                                           \
      __builtin_shufflevector(p01, p23, 2 * (e), 2 * (e) + 1, 16 + 2 * (e), 17 + 2 * (e))
    FM_T_ROW(0); FM_T_ROW(1); FM_T_ROW(2); FM_T_ROW(3);
    FM_T_ROW(4); FM_T_ROW(5); FM_T_ROW(6); FM_T_ROW(7);
#undef FM_T_ROW
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_kernel(const BwdArgs a) {
  constexpr int NS = D / 16, ND = D / 32;
  using Smem = BwdSmem<D>;
  constexpr int QST = Smem::QST, QTS = Smem::QTS, KTS = Smem::KTS, DSS = Smem::DSS;
  __shared__ Smem sm;

  const unsigned t = threadIdx.x;
  const int lane = (int)(t & 63), w = (int)(t >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nK);
  const uint32_t n_items = min(a.counters[kCtrBwdItems], max_items);
  const int Sq = a.Sq, Sk = a.Sk;

  for (;;) {
    if (t == 0) sm.item = atomicAdd(&a.counters[kCtrBwdNext], 1u);
    __syncthreads();
    const uint32_t idx = __builtin_amdgcn_readfirstlane(sm.item);
    if (idx >= n_items) break;
    const uint32_t it = min(a.queue[idx], max_items - 1);
    const long bh = it / a.nK;
    const int kb = (int)(it % a.nK);
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const long bhm = (long)b * a.Hm + (a.Hm == 1 ? 0 : h);
    const int cnt = min(a.cnt_k[bhm * a.nK + kb], a.nQ);
    const uint16_t* lst = a.list_k + (bhm * a.nK + kb) * (long)a.nQ;
    const int k0 = kb * BK;
    const bool ragged_k = k0 + BK > Sk;
    const BufRsrc qbase = make_rsrc(a.q + bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
    const BufRsrc obase = make_rsrc(a.dout + bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
    const BufRsrc kbase = make_rsrc(a.k + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
    const BufRsrc vbase = make_rsrc(a.v + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
    const BufRsrc lbase = make_rsrc(a.lse + bh * Sq, (uint32_t)Sq * 4u);
    const BufRsrc dbase = make_rsrc(a.delta + bh * Sq, (uint32_t)Sq * 4u);
    const BufRsrc listb = make_rsrc(lst, (uint32_t)cnt * 2u);
    auto list_at = [&](int i) -> uint32_t {
      return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(listb, i * 2, 0, 0);
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
      stage_kt<D>(kbase, k0, sm, t);
      ChunkStage<D> cs;
      int e_cur = __builtin_amdgcn_readfirstlane(list_at(0));
      load_chunk<D>(cs, qbase, obase, lbase, dbase, min(e_cur & kListIndex, a.nQ - 1) * BQ, Sq, t);
      store_chunk<D>(cs, sm, t);
      __syncthreads();

      // Per chunk c (its Q, dO, Q^T, dO^T and row terms in LDS):
      //   chunk c+1 -> registers; S, dP; P, dS (dS -> LDS); dV, dK |
      //   barrier | chunk c+1 -> LDS; dQ = dS K -> atomics | barrier
      for (int c = 0; c < nchunks; ++c) {
        const int q0 = min(e_cur & kListIndex, a.nQ - 1) * BQ + (c % CPB) * QC;
        const bool need_mask = (e_cur & kListPartial) || ragged_k;
        const bool has_next = c + 1 < nchunks;
        int e_next = e_cur;
        if (has_next) {
          if ((c + 1) % CPB == 0) e_next = __builtin_amdgcn_readfirstlane(list_at((c + 1) / CPB));
          const int q0n = min(e_next & kListIndex, a.nQ - 1) * BQ + ((c + 1) % CPB) * QC;
          load_chunk<D>(cs, qbase, obase, lbase, dbase, q0n, Sq, t);
        }

        // The chunk's two halves of 32 rows go through S, dP, P, dS and the dV,
        // dK products one after the other, which halves the live tile state.
#pragma unroll 1
        for (int ib = 0; ib < QC / 32; ++ib) {
          // ---- S = Q K^T and dP = dO V^T: lane holds key li, rows 32ib + 8r + 4hh + q ----
          f32x16 s, dp;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            s[v] = 0.f;
            dp[v] = 0.f;
          }
          // operands of the whole phase are read first: many LDS reads in
          // flight instead of one read ahead of each MFMA
          {
            bf16x8 qa[NS], oa[NS];
#pragma unroll
            for (int kk = 0; kk < NS; ++kk) {
              const int off = (32 * ib + li) * QST + 16 * kk + 8 * hh;
              qa[kk] = as_bf16x8(&sm.q[off]);
              oa[kk] = as_bf16x8(&sm.dout[off]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk = 0; kk < NS; ++kk) {
              s = mfma32(qa[kk], kf[kk], s);
              dp = mfma32(oa[kk], vf[kk], dp);
            }
          }
          // ---- P = exp(S - LSE) (interval mask on partial tiles), dS = P (dP - Delta) ----
          bf16x8 pb[2], dsb[2];
          auto p_and_ds = [&](auto masked_tile) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int il = 32 * ib + 8 * r + 4 * hh;
              const float4 l4 = *reinterpret_cast<const float4*>(&sm.lse2[il]);
              const float4 d4 = *reinterpret_cast<const float4*>(&sm.delta[il]);
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
              const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int v = 4 * r + q;
                float p = fast_exp2(fmaf(s[v], a.scale_log2, -lv[q]));
                if constexpr (decltype(masked_tile)::value) {
                  const int gi = q0 + il + q;
                  const bool masked = ((bd.x <= gi) & (gi < bd.y)) | ((bd.z <= gi) & (gi < bd.w));
                  p = masked ? 0.f : p;
                }
                const float dsv = p * (dp[v] - dl[q]);
                pb[v >> 3][v & 7] = (bf16)p;
                dsb[v >> 3][v & 7] = (bf16)dsv;
                sm.ds[(il + q) * DSS + 32 * w + li] = (bf16)dsv;
              }
            }
          };
          if (need_mask)
            p_and_ds(std::true_type{});
          else
            p_and_ds(std::false_type{});
          // ---- dV += P^T dO, dK += dS^T Q (B operands: rows of dO^T, Q^T) ----
          {
            bf16x8 ob[ND][2], qtb[ND][2];
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
              for (int t2 = 0; t2 < 2; ++t2) {
                const int off = (32 * d + li) * QTS + 32 * ib + 16 * t2 + 8 * hh;
                ob[d][t2] = as_bf16x8(&sm.dot[off]);
                qtb[d][t2] = as_bf16x8(&sm.qt[off]);
              }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = 0; d < ND; ++d)
#pragma unroll
              for (int t2 = 0; t2 < 2; ++t2) {
                dv[d] = mfma32(pb[t2], ob[d][t2], dv[d]);
                dk[d] = mfma32(dsb[t2], qtb[d][t2], dk[d]);
              }
          }
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            pin_agpr(dv[d]);
            pin_agpr(dk[d]);
          }
        }
        __syncthreads();   // dS is in LDS; every wave is done with this chunk's Q and dO
        if (has_next) store_chunk<D>(cs, sm, t);

        // ---- dQ[q0.., :] += scale dS K : wave w takes (ib, d) blocks w, w+4, ... ----
        for (int blk = w; blk < (QC / 32) * ND; blk += 4) {
          const int ib = blk / ND, d = blk % ND;
          f32x16 acc;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] = 0.f;
          {
            bf16x8 da[BK / 16], kb2[BK / 16];
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
              da[ks] = as_bf16x8(&sm.ds[(32 * ib + li) * DSS + 16 * ks + 8 * hh]);
              kb2[ks] = as_bf16x8(&sm.kt[(32 * d + li) * KTS + 16 * ks + 8 * hh]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) acc = mfma32(da[ks], kb2[ks], acc);
          }
          float* dqp = a.dq_acc + (bh * Sq + q0) * D + 32 * d + li;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int il = 32 * ib + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (q0 + il < Sq) unsafeAtomicAdd(dqp + (long)il * D, acc[v] * a.scale);
          }
        }
        __syncthreads();   // every wave is done with dS; the next chunk is in LDS
        e_cur = e_next;
      }
    }

    // ---- write dK (scaled) and dV: lane holds column 32d + li, keys 8r + 4hh + q ----
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int jl = 32 * w + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (k0 + jl < Sk) {
          const long off = (bh * Sk + k0 + jl) * D + 32 * d + li;
          a.dk[off] = (bf16)(dk[d][v] * a.scale);
          a.dv[off] = (bf16)dv[d][v];
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

// ---------------------------------------------------------------- epilogue
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         bf16* __restrict__ dq, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 x = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 y = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  bf16x8 r;
  r[0] = (bf16)x.x; r[1] = (bf16)x.y; r[2] = (bf16)x.z; r[3] = (bf16)x.w;
  r[4] = (bf16)y.x; r[5] = (bf16)y.y; r[6] = (bf16)y.z; r[7] = (bf16)y.w;
  reinterpret_cast<bf16x8*>(dq)[i] = r;
}

int bwd_blocks_per_cu(int) { return 1; }

hipError_t launch_attn_bwd(const BwdArgs& a, int head_dim, int grid, hipStream_t stream,
                           const KernelEvents& ev) {
  const long rows = (long)a.B * a.H * a.Sq;
  const long n8 = rows * head_dim / 8;
  const unsigned pre_grid = (unsigned)((n8 + 255) / 256);
  hipError_t err;
  if (head_dim == 128)
    bwd_pre_kernel<128><<<pre_grid, 256, 0, stream>>>(a.o, a.dout, a.delta, a.dq_acc, rows);
  else
    bwd_pre_kernel<64><<<pre_grid, 256, 0, stream>>>(a.o, a.dout, a.delta, a.dq_acc, rows);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev.begin && (err = hipEventRecord(ev.begin, stream)) != hipSuccess) return err;
  if (grid > 0) {
    if (head_dim == 128)
      attn_bwd_kernel<128><<<grid, 256, 0, stream>>>(a);
    else
      attn_bwd_kernel<64><<<grid, 256, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (ev.end && (err = hipEventRecord(ev.end, stream)) != hipSuccess) return err;
  dq_convert_kernel<<<pre_grid, 256, 0, stream>>>(a.dq_acc, a.dq, n8);
  return hipGetLastError();
}

}  // namespace fm
