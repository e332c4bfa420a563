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
// rows, which is exactly the A-operand shape of P^T dO and dS^T Q; Q and dO
// are therefore staged once, row-major, and read either by rows (16-byte
// loads) or by columns (transposed LDS loads).
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {

constexpr int QC = 64;   // query rows per backward chunk

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
  static constexpr int RST = D + 8;    // Q / dO row stride (elements)
  static constexpr int KST = D + 16;   // K row stride (transposed reads only)
  static constexpr int SST = BK + 8;   // dS row stride
  bf16 k[BK * KST];
  bf16 q[QC * RST];
  bf16 dout[QC * RST];
  bf16 ds[QC * SST];
  float lse2[QC];   // LSE * log2(e); +inf for rows past the end
  float delta[QC];
  uint32_t item;
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_kernel(const BwdArgs a) {
  constexpr int NS = D / 16, ND = D / 32;
  constexpr int RST = BwdSmem<D>::RST, KST = BwdSmem<D>::KST, SST = BwdSmem<D>::SST;
  __shared__ BwdSmem<D> sm;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int li = lane & 31, hh = lane >> 5;
  const int gc = (lane >> 4) & 1, m16 = lane & 15;
  // transposed-read lane offsets: P-ordered rows (8u + 4hh + e) and natural rows (8hh + 4u + e)
  const int tr_p = (4 * hh + (m16 >> 2)) * RST + 16 * gc + 4 * (m16 & 3);
  const int tr_k = (8 * hh + (m16 >> 2)) * KST + 16 * gc + 4 * (m16 & 3);
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nK);
  const uint32_t n_items = min(a.counters[kCtrBwdItems], max_items);
  const int Sq = a.Sq, Sk = a.Sk;

  for (;;) {
    if (t == 0) sm.item = atomicAdd(&a.counters[kCtrBwdNext], 1u);
    __syncthreads();
    const uint32_t idx = sm.item;
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

    // this lane's key and its bounds; K and V rows as MFMA B operands
    const int jrow = k0 + 32 * w + li;
    const bool jvalid = jrow < Sk;
    // a key past the end gets an interval covering every row
    const int4 bd = jvalid ? a.bounds[bhm * Sk + jrow] : make_int4(INT_MIN, INT_MAX, 0, 0);
    bf16x8 kf[NS], vf[NS];
    {
      const bf16x8* kp = reinterpret_cast<const bf16x8*>(a.k + (bh * Sk + jrow) * D);
      const bf16x8* vp = reinterpret_cast<const bf16x8*>(a.v + (bh * Sk + jrow) * D);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kf[s] = jvalid ? kp[2 * s + hh] : zero_bf16x8();
        vf[s] = jvalid ? vp[2 * s + hh] : zero_bf16x8();
      }
    }
    // whole K block in LDS (read by columns for dQ)
    {
      const bf16x8* kg = reinterpret_cast<const bf16x8*>(a.k + (bh * Sk + k0) * D);
      for (int c = t; c < BK * D / 8; c += 256) {
        const int j = c / (D / 8), dc = c % (D / 8);
        *reinterpret_cast<bf16x8*>(&sm.k[j * KST + dc * 8]) =
            (k0 + j < Sk) ? kg[c] : zero_bf16x8();
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

    for (int tt = 0; tt < cnt; ++tt) {
      const int e = lst[tt];
      const int qb = min(e & kListIndex, a.nQ - 1);
      const bool need_mask = (e & kListPartial) || ragged_k;
      for (int ch = 0; ch < BQ / QC; ++ch) {
        const int q0 = qb * BQ + ch * QC;
        if (q0 >= Sq) break;
        __syncthreads();
        // ---- stage Q, dO rows [q0, q0+QC), LSE and Delta ----
        {
          const bf16x8* qg = reinterpret_cast<const bf16x8*>(a.q + (bh * Sq + q0) * D);
          const bf16x8* og = reinterpret_cast<const bf16x8*>(a.dout + (bh * Sq + q0) * D);
          for (int c = t; c < QC * D / 8; c += 256) {
            const int i = c / (D / 8), dc = c % (D / 8);
            const bool ok = q0 + i < Sq;
            *reinterpret_cast<bf16x8*>(&sm.q[i * RST + dc * 8]) = ok ? qg[c] : zero_bf16x8();
            *reinterpret_cast<bf16x8*>(&sm.dout[i * RST + dc * 8]) = ok ? og[c] : zero_bf16x8();
          }
          if (t < QC) {
            const bool ok = q0 + t < Sq;
            sm.lse2[t] = ok ? a.lse[bh * Sq + q0 + t] * kLog2e : INFINITY;
            sm.delta[t] = ok ? a.delta[bh * Sq + q0 + t] : 0.f;
          }
        }
        __syncthreads();

        // ---- S = Q K^T and dP = dO V^T: lane holds key li, rows 32ib + 8r + 4hh + q ----
        f32x16 s[QC / 32], dp[QC / 32];
#pragma unroll
        for (int ib = 0; ib < QC / 32; ++ib) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            s[ib][v] = 0.f;
            dp[ib][v] = 0.f;
          }
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const int off = (32 * ib + li) * RST + 16 * st + 8 * hh;
            s[ib] = mfma32(as_bf16x8(&sm.q[off]), kf[st], s[ib]);
            dp[ib] = mfma32(as_bf16x8(&sm.dout[off]), vf[st], dp[ib]);
          }
        }
        // ---- P and dS ----
        bf16x8 pb[QC / 32][2], dsb[QC / 32][2];
#pragma unroll
        for (int ib = 0; ib < QC / 32; ++ib)
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
              float p = fast_exp2(fmaf(s[ib][v], a.scale_log2, -lv[q]));
              if (need_mask) {
                const int gi = q0 + il + q;
                const bool masked = ((bd.x <= gi) & (gi < bd.y)) | ((bd.z <= gi) & (gi < bd.w));
                p = masked ? 0.f : p;
              }
              const float dsv = p * (dp[ib][v] - dl[q]);
              pb[ib][v >> 3][v & 7] = (bf16)p;
              dsb[ib][v >> 3][v & 7] = (bf16)dsv;
              sm.ds[(il + q) * SST + 32 * w + li] = (bf16)dsv;
            }
          }
        // ---- dV += P^T dO,  dK += dS^T Q  (B operands by transposed reads) ----
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int ib = 0; ib < QC / 32; ++ib)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const int off = (32 * ib + 16 * t2) * RST + 32 * d + tr_p;
              const bf16x8 ob = cat_bf16(lds_read_tr(&sm.dout[off]), lds_read_tr(&sm.dout[off + 8 * RST]));
              const bf16x8 qbv = cat_bf16(lds_read_tr(&sm.q[off]), lds_read_tr(&sm.q[off + 8 * RST]));
              dv[d] = mfma32(pb[ib][t2], ob, dv[d]);
              dk[d] = mfma32(dsb[ib][t2], qbv, dk[d]);
            }
        __syncthreads();
        // ---- dQ[q0.., :] += scale dS K : wave w takes (ib, d) blocks w, w+4, ... ----
        for (int blk = w; blk < (QC / 32) * ND; blk += 4) {
          const int ib = blk / ND, d = blk % ND;
          f32x16 acc;
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
          for (int ks = 0; ks < BK / 16; ++ks) {
            const bf16x8 av = as_bf16x8(&sm.ds[(32 * ib + li) * SST + 16 * ks + 8 * hh]);
            const int off = (16 * ks) * KST + 32 * d + tr_k;
            const bf16x8 bv = cat_bf16(lds_read_tr(&sm.k[off]), lds_read_tr(&sm.k[off + 4 * KST]));
            acc = mfma32(av, bv, acc);
          }
          float* dqp = a.dq_acc + (bh * Sq + q0) * D + 32 * d + li;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int il = 32 * ib + 8 * (v >> 2) + 4 * hh + (v & 3);
            if (q0 + il < Sq) unsafeAtomicAdd(dqp + (long)il * D, acc[v] * a.scale);
          }
        }
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
    __syncthreads();
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
