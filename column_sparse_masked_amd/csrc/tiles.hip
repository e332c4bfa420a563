// Tile classification for the column-sparse mask (FlashMask-3 paper summary,
// abstract: per key column, the mask keeps the bounds of the query-row ranges
// it hides).  Three kernels:
//   kbsum_kernel     per key block, min and max of each clamped bound;
//   classify_kernel  class of every (query block, key block) tile plus, per
//                    query block and per key block, the list of tiles that are
//                    not skipped (the loops of the forward and backward);
//   queue_kernel     forward and backward work items sorted by tile count,
//                    heaviest first, for the persistent kernels.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {

// One workgroup of BK threads per (key block, batch*mask head); thread t owns
// column kb*BK + t.  Output: 8 int32 per block (min/max of LTS, LTE, UTS, UTE
// after clamping to [0, Sq]); columns >= Sk do not take part.
__global__ __launch_bounds__(BK) void kbsum_kernel(const int4* __restrict__ bounds,
                                                   int* __restrict__ kbsum, int Sq, int Sk,
                                                   int nK) {
  const int kb = blockIdx.x;
  const long bhm = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int col = kb * BK + t;
  int mn[4], mx[4];
  if (col < Sk) {
    int4 b = bounds[bhm * Sk + col];
    int v[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int x = min(max(v[c], 0), Sq);
      mn[c] = x;
      mx[c] = x;
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mn[c] = INT_MAX;
      mx[c] = INT_MIN;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mn[c] = min(mn[c], __shfl_xor(mn[c], off));
      mx[c] = max(mx[c], __shfl_xor(mx[c], off));
    }
  }
  __shared__ int red[BK / 64][8];
  if (lane == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      red[wave][2 * c] = mn[c];
      red[wave][2 * c + 1] = mx[c];
    }
  }
  __syncthreads();
  if (t < 8) {
    int r = red[0][t];
#pragma unroll
    for (int w = 1; w < BK / 64; ++w) r = (t & 1) ? max(r, red[w][t]) : min(r, red[w][t]);
    kbsum[(bhm * nK + kb) * 8 + t] = r;
  }
}

// Class of query rows [q0, q1) against a key-block summary.
//   skip:    one interval covers the whole tile in every column
//            (its largest start <= q0 and its smallest end >= q1);
//   full:    each interval lies entirely before or after the tile in every
//            column (smallest start >= q1, or largest end <= q0);
//   partial: anything else.
__device__ __forceinline__ int tile_class(const int* ks, int q0, int q1) {
  const bool skip = (ks[1] <= q0 && ks[2] >= q1) || (ks[5] <= q0 && ks[6] >= q1);
  if (skip) return 0;
  const bool lower_clear = ks[0] >= q1 || ks[3] <= q0;
  const bool upper_clear = ks[4] >= q1 || ks[7] <= q0;
  return (lower_clear && upper_clear) ? 1 : 2;
}

__device__ __forceinline__ void load_ks(const int* kbsum, long idx, int* ks) {
  const int4* p = reinterpret_cast<const int4*>(kbsum + idx * 8);
  int4 a = p[0], b = p[1];
  ks[0] = a.x; ks[1] = a.y; ks[2] = a.z; ks[3] = a.w;
  ks[4] = b.x; ks[5] = b.y; ks[6] = b.z; ks[7] = b.w;
}

// grid (nQ + nK, B*Hm), 256 threads.  Blocks x < nQ classify one query block's
// row of tiles (writing cls, list_q, cnt_q); blocks x >= nQ one key block's
// column (writing list_k, cnt_k).  Lists keep increasing block order; the
// compaction uses a wave ballot and a 4-wave prefix.
__global__ __launch_bounds__(256) void classify_kernel(const int* __restrict__ kbsum,
                                                       uint8_t* __restrict__ cls,
                                                       int* __restrict__ cnt_q,
                                                       int* __restrict__ cnt_k,
                                                       uint16_t* __restrict__ list_q,
                                                       uint16_t* __restrict__ list_k, int Sq,
                                                       int nQ, int nK) {
  const long bhm = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ int wsum[4];
  const bool row_mode = (int)blockIdx.x < nQ;
  const int blk = row_mode ? (int)blockIdx.x : (int)blockIdx.x - nQ;
  const int n_other = row_mode ? nK : nQ;
  uint16_t* list = row_mode ? list_q + (bhm * nQ + blk) * (long)nK
                            : list_k + (bhm * nK + blk) * (long)nQ;
  int ks_col[8];
  if (!row_mode) load_ks(kbsum, bhm * nK + blk, ks_col);
  int base = 0;
  for (int o0 = 0; o0 < n_other; o0 += 256) {
    const int o = o0 + t;
    int c = 0;
    if (o < n_other) {
      if (row_mode) {
        int ks[8];
        load_ks(kbsum, bhm * nK + o, ks);
        const int q0 = blk * BQ;
        c = tile_class(ks, q0, min(Sq, q0 + BQ));
        cls[(bhm * nQ + blk) * (long)nK + o] = (uint8_t)c;
      } else {
        const int q0 = o * BQ;
        c = tile_class(ks_col, q0, min(Sq, q0 + BQ));
      }
    }
    const bool keep = (o < n_other) && c != 0;
    const unsigned long long m = __ballot(keep);
    const int pos = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (keep) list[off + pos] = (uint16_t)(o | (c == 2 ? kListPartial : 0));
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (t == 0) {
    if (row_mode)
      cnt_q[bhm * nQ + blk] = base;
    else
      cnt_k[bhm * nK + blk] = base;
  }
}

constexpr int kQueueThreads = 1024;
constexpr int kBuckets = 4096;   // tile counts above 4095 share the top bucket

// Exclusive prefix sum over the block (1024 threads); returns this thread's
// offset and leaves the grand total in *total.
__device__ int block_exclusive_scan(int x, int* scratch, int* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int w = 0; w < kQueueThreads / 64; ++w) {
      int s = scratch[w];
      scratch[w] = run;
      run += s;
    }
    scratch[kQueueThreads / 64] = run;
  }
  __syncthreads();
  const int res = scratch[wave] + incl - x;
  *total = scratch[kQueueThreads / 64];
  __syncthreads();
  return res;
}

// Counting sort of n items by tile count, descending.  Item it = bh*nBlk+blk
// has count cnt[(b*Hm + hm)*nBlk + blk].  Order inside a count is arbitrary.
// Sum over the workgroup of one 64-bit value per thread (every thread gets it).
__device__ long block_sum(long x, long* scratch) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if (lane == 0) scratch[wave] = x;
  __syncthreads();
  long total = 0;
  for (int w = 0; w < kQueueThreads / 64; ++w) total += scratch[w];
  __syncthreads();
  return total;
}

// Which forward items to split (split != nullptr: the forward queue).  The
// forward is a persistent grid of fwd_slots workgroups taking items longest
// first; when few items share a workgroup, the longest ones set the end of
// the kernel.  Items with more than max(16, ceil(total / (2 fwd_slots)))
// tiles (half the mean load of a workgroup) are split in two halves of their
// key blocks, at most split_cap of them; they are the first entries of the
// sorted queue.  Counted from the histogram of tile counts, which is exact
// below the top bucket; with any item in the top bucket nothing is split.
struct SplitRule {
  int fwd_slots, split_cap;
  uint32_t* out;
  long* scratch;   // kQueueThreads / 64 longs
};

__device__ void sort_items(const int* __restrict__ cnt, uint32_t* __restrict__ queue, int B,
                           int H, int Hm, int nBlk, int* hist, int* scratch, const SplitRule* split) {
  const int t = threadIdx.x;
  const long n = (long)B * H * nBlk;
  for (int i = t; i < kBuckets; i += kQueueThreads) hist[i] = 0;
  __syncthreads();
  for (long it = t; it < n; it += kQueueThreads) {
    const long bh = it / nBlk;
    const int blk = (int)(it % nBlk);
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int c = cnt[((long)b * Hm + (Hm == 1 ? 0 : h)) * nBlk + blk];
    atomicAdd(&hist[min(c, kBuckets - 1)], 1);
  }
  __syncthreads();
  if (split) {
    long tiles = 0;
    for (int i = t; i < kBuckets - 1; i += kQueueThreads) tiles += (long)i * hist[i];
    const long total = block_sum(tiles, split->scratch);
    const long slots = max(split->fwd_slots, 1);
    const long thr = max(16L, (total + 2 * slots - 1) / (2 * slots));
    long above = 0;
    for (int i = t; i < kBuckets - 1; i += kQueueThreads) above += i > thr ? hist[i] : 0;
    above = block_sum(above, split->scratch);
    if (t == 0)
      *split->out = (hist[kBuckets - 1] > 0 || thr >= kBuckets - 1)
                        ? 0u
                        : (uint32_t)min(above, (long)max(split->split_cap, 0));
  }
  // thread t owns buckets kBuckets-1-4t ... kBuckets-4-4t (descending order)
  constexpr int per = kBuckets / kQueueThreads;
  int local[per];
  int sum = 0;
#pragma unroll
  for (int u = 0; u < per; ++u) {
    local[u] = hist[kBuckets - 1 - (per * t + u)];
    sum += local[u];
  }
  int total;
  int run = block_exclusive_scan(sum, scratch, &total);
#pragma unroll
  for (int u = 0; u < per; ++u) {
    hist[kBuckets - 1 - (per * t + u)] = run;
    run += local[u];
  }
  __syncthreads();
  for (long it = t; it < n; it += kQueueThreads) {
    const long bh = it / nBlk;
    const int blk = (int)(it % nBlk);
    const int b = (int)(bh / H), h = (int)(bh % H);
    const int c = cnt[((long)b * Hm + (Hm == 1 ? 0 : h)) * nBlk + blk];
    const int pos = atomicAdd(&hist[min(c, kBuckets - 1)], 1);
    queue[pos] = (uint32_t)it;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kQueueThreads) void queue_kernel(
    const int* __restrict__ cnt_q, const int* __restrict__ cnt_k, uint32_t* __restrict__ fwd_q,
    uint32_t* __restrict__ bwd_q, uint32_t* __restrict__ counters, int B, int H, int Hm, int nQ,
    int nK, int fwd_slots, int split_cap) {
  // workgroup 0 sorts the forward (and dQ) queue, workgroup 1 the backward one
  __shared__ int hist[kBuckets];
  __shared__ int scratch[kQueueThreads / 64 + 1];
  __shared__ long lscratch[kQueueThreads / 64];
  if (blockIdx.x == 0) {
    __shared__ uint32_t nsplit;
    if (threadIdx.x == 0) nsplit = 0;
    const SplitRule rule{fwd_slots, split_cap, &nsplit, lscratch};
    if (nQ > 0) sort_items(cnt_q, fwd_q, B, H, Hm, nQ, hist, scratch, split_cap > 0 ? &rule : nullptr);
    __syncthreads();
    if (threadIdx.x == 0) {
      counters[kCtrFwdItems] = (uint32_t)((long)B * H * nQ);
      counters[kCtrFwdSplit] = nsplit;
      counters[kCtrFwdNext] = 0;
      counters[kCtrFwdExit] = 0;
      counters[kCtrDqNext] = 0;
      counters[kCtrDqExit] = 0;
    }
  } else {
    if (nK > 0) sort_items(cnt_k, bwd_q, B, H, Hm, nK, hist, scratch, nullptr);
    if (threadIdx.x == 0) {
      counters[kCtrBwdItems] = (uint32_t)((long)B * H * nK);
      counters[kCtrBwdNext] = 0;
      counters[kCtrBwdExit] = 0;
    }
  }
}

// Zero-fill of n16 16-byte words (a kernel rather than a memset, which stays
// correct when a caller captures the call into a graph).  Used by the
// backward when there are no query rows.
__global__ __launch_bounds__(256) void zero16_kernel(uint4* __restrict__ p, long n16) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero16(void* p, size_t bytes, hipStream_t stream) {
  const long n16 = (long)(bytes / 16);
  if (n16 <= 0) return hipSuccess;
  const long blocks = (n16 + 255) / 256;
  zero16_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_tile_bounds(const TileArgs& a, hipStream_t stream) {
  const unsigned bhm = (unsigned)((long)a.B * a.Hm);
  if (bhm > 0 && a.nK > 0) {
    kbsum_kernel<<<dim3(a.nK, bhm), BK, 0, stream>>>(a.bounds, a.kbsum, a.Sq, a.Sk, a.nK);
  }
  if (bhm > 0 && a.nQ + a.nK > 0) {
    classify_kernel<<<dim3(a.nQ + a.nK, bhm), 256, 0, stream>>>(a.kbsum, a.cls, a.cnt_q, a.cnt_k,
                                                                a.list_q, a.list_k, a.Sq, a.nQ, a.nK);
  }
  // always, also for empty problems: it leaves (empty) queues and zeroed
  // counters behind, with a kernel rather than a memset, which stays correct
  // when a caller replays the calls as a captured graph
  queue_kernel<<<2, kQueueThreads, 0, stream>>>(a.cnt_q, a.cnt_k, a.fwd_queue, a.bwd_queue,
                                                a.counters, a.B, a.H, a.Hm, a.nQ, a.nK, a.fwd_slots,
                                                a.split_cap);
  return hipGetLastError();
}

}  // namespace fm
