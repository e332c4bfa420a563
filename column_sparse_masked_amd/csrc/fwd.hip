// Forward of column-sparse masked attention on the matrix cores (bf16 in,
// fp32 accumulate).  FlashMask-3 paper summary, abstract: a mask-aware kernel
// that works only on tiles the column-wise sparse mask does not fully mask.
//
// Persistent grid: each workgroup (4 waves) repeatedly takes the next item
// (batch*head, query block) from the cost-sorted queue built by the tile pass,
// holds that block's 128 query rows in registers (32 rows per wave) and walks
// the block's list of non-skipped key blocks.  Per key block, K and V are
// staged row-major in LDS; each wave computes S^T = K Q^T (32 keys x 32 rows
// per MFMA), applies the elementwise interval test only on partial (or
// ragged) tiles, updates an online softmax in the log2 domain and accumulates
// O^T += V^T P^T, reading V^T with transposed LDS loads.  Keeping S^T (not S)
// lets the accumulator of one MFMA be the B operand of the next with no data
// movement between lanes.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {

template <int D>
struct alignas(16) FwdSmem {
  static constexpr int KST = D + 8;    // K row stride (elements): 16-byte row reads
  static constexpr int VST = D + 16;   // V row stride: 8-byte transposed reads
  bf16 k[BK * KST];
  bf16 v[BK * VST];
  int4 bnd[BK];
  uint32_t item;
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(const FwdArgs a) {
  constexpr int NS = D / 16;   // k-steps over the head dimension
  constexpr int ND = D / 32;   // 32-wide blocks of the head dimension
  constexpr int KST = FwdSmem<D>::KST, VST = FwdSmem<D>::VST;
  __shared__ FwdSmem<D> sm;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int li = lane & 31, hh = lane >> 5;
  const int gc = (lane >> 4) & 1, m16 = lane & 15;
  // lane offset of the transposed V read: row 4*hh + m16/4, column 16*gc + 4*(m16%4)
  const int v_lane = (4 * hh + (m16 >> 2)) * VST + 16 * gc + 4 * (m16 & 3);
  // item count and queue entries are range-checked so that a stale or foreign
  // tileinfo cannot make the kernel read outside its tensors
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nQ);
  const uint32_t n_items = min(a.counters[kCtrFwdItems], max_items);
  const int Sq = a.Sq, Sk = a.Sk;

  for (;;) {
    if (t == 0) sm.item = atomicAdd(&a.counters[kCtrFwdNext], 1u);
    __syncthreads();
    const uint32_t idx = sm.item;
    if (idx >= n_items) break;
    const uint32_t it = min(a.queue[idx], max_items - 1);
    const long bh = it / a.nQ;
    const int qb = (int)(it % a.nQ);
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);
    const long bhm = (long)b * a.Hm + (a.Hm == 1 ? 0 : h);
    const int cnt = min(a.cnt_q[bhm * a.nQ + qb], a.nK);
    const uint16_t* lst = a.list_q + (bhm * a.nQ + qb) * (long)a.nK;

    const int qrow = qb * BQ + 32 * w + li;
    bf16x8 qf[NS];
    if (qrow < Sq) {
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(a.q + (bh * Sq + qrow) * D);
#pragma unroll
      for (int s = 0; s < NS; ++s) qf[s] = qp[2 * s + hh];
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) qf[s] = zero_bf16x8();
    }
    f32x16 acc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[d][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const bf16x8* kbase = reinterpret_cast<const bf16x8*>(a.k + bh * Sk * (long)D);
    const bf16x8* vbase = reinterpret_cast<const bf16x8*>(a.v + bh * Sk * (long)D);

    for (int tt = 0; tt < cnt; ++tt) {
      const int e = lst[tt];
      const int kb = min(e & kListIndex, a.nK - 1);
      const int k0 = kb * BK;
      const bool need_mask = (e & kListPartial) || (k0 + BK > Sk);
      __syncthreads();
      // ---- stage K and V rows [k0, k0+BK) row-major ----
#pragma unroll 2
      for (int c = t; c < BK * D / 8; c += 256) {
        const int j = c / (D / 8), dc = c % (D / 8);
        const bool ok = k0 + j < Sk;
        const long g = (long)k0 * (D / 8) + c;
        bf16x8 kv = ok ? kbase[g] : zero_bf16x8();
        bf16x8 vv = ok ? vbase[g] : zero_bf16x8();
        *reinterpret_cast<bf16x8*>(&sm.k[j * KST + dc * 8]) = kv;
        *reinterpret_cast<bf16x8*>(&sm.v[j * VST + dc * 8]) = vv;
      }
      if (need_mask) {
        // keys past the end get an interval covering every row
        for (int c = t; c < BK; c += 256)
          sm.bnd[c] = (k0 + c < Sk) ? a.bounds[bhm * Sk + k0 + c] : make_int4(INT_MIN, INT_MAX, 0, 0);
      }
      __syncthreads();

      // ---- S^T = K Q^T : lane holds query column li, keys 32*jb + 8r + 4hh + q ----
      f32x16 s[4];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[jb][v] = 0.f;
#pragma unroll
        for (int st = 0; st < NS; ++st)
          s[jb] = mfma32(as_bf16x8(&sm.k[(32 * jb + li) * KST + 16 * st + 8 * hh]), qf[st], s[jb]);
      }
      if (need_mask) {
        const int4* bl = &sm.bnd[4 * hh];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int4 bd = bl[32 * jb + 8 * (v >> 2) + (v & 3)];
            const bool masked = ((bd.x <= qrow) & (qrow < bd.y)) | ((bd.z <= qrow) & (qrow < bd.w));
            s[jb][v] = masked ? -INFINITY : s[jb][v];
          }
      }
      // ---- online softmax (log2 domain) ----
      float mx = -INFINITY;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[jb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float base = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - base);
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[d][v] *= alpha;
      // ---- P (8 keys at a time) and O^T += V^T P^T ----
      float rs = 0.f;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          bf16x8 pb;
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) {
            const float pv = fast_exp2(fmaf(s[jb][8 * t2 + e8], a.scale_log2, -base));
            rs += pv;
            pb[e8] = (bf16)pv;
          }
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const bf16* vp = &sm.v[(32 * jb + 16 * t2) * VST + 32 * d + v_lane];
            const bf16x8 vo = cat_bf16(lds_read_tr(vp), lds_read_tr(vp + 8 * VST));
            acc[d] = mfma32(vo, pb, acc[d]);
          }
        }
      l_run = l_run * alpha + rs;
    }

    // ---- finalise: O = acc / l, LSE = (m + log2 l) ln 2 ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qrow < Sq) {
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
    __syncthreads();   // every thread has read sm.item and finished with LDS
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

hipError_t launch_attn_fwd(const FwdArgs& a, int head_dim, int grid, hipStream_t stream,
                           const KernelEvents& ev) {
  hipError_t err;
  if (ev.begin && (err = hipEventRecord(ev.begin, stream)) != hipSuccess) return err;
  if (head_dim == 128)
    attn_fwd_kernel<128><<<grid, 256, 0, stream>>>(a);
  else
    attn_fwd_kernel<64><<<grid, 256, 0, stream>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev.end && (err = hipEventRecord(ev.end, stream)) != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace fm
