// Tile classification for the column-sparse mask (FlashMask-3 paper summary,
// abstract: per key column, the mask keeps the bounds of the query-row ranges
// it hides).  Two kernels:
//   column_kernel  per key block, the min and max of each clamped bound, then
//                  the block's column of tiles: which query blocks see it
//                  (list_k, cnt_k) and each listed tile's place in that list;
//   row_kernel     per query block, the class of every tile of its row (cls)
//                  and its non-skipped key blocks (list_q, cnt_q); the last
//                  workgroup to finish then sorts the forward and backward
//                  work items by tile count, heaviest first, for the
//                  persistent kernels, and lays out the backward's tile slots.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {

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

// Which forward items to split (on: the forward queue, splitting allowed).
// The forward is a persistent grid of fwd_slots workgroups taking items
// longest first; when few items share a workgroup, the longest ones set the
// end of the kernel.  Items with more than max(16, ceil(total / (2 fwd_slots)))
// tiles (half the mean load of a workgroup) are split in two halves of their
// key blocks, at most split_cap of them; they are the first entries of the
// sorted queue.  Counted from the histogram of tile counts, which is exact
// below the top bucket; with any item in the top bucket nothing is split.
struct SplitRule {
  bool on;    // this part sorts the forward queue and splitting is allowed
  bool any;   // splitting is allowed at all (the same in both parts)
  int fwd_slots, split_cap;
};


// atomicAdd(&hist[bucket], 1) for every active lane; returns the old value.
// When every active lane of the wave has the same bucket (common: many
// items share a tile count) that is one LDS atomic for the wave instead of
// up to 64 on one address.
__device__ __forceinline__ int wave_bucket_add(int* hist, int bucket, bool active) {
  const int lane = threadIdx.x & 63;
  const unsigned long long act = __ballot(active);
  if (act == 0) return 0;
  const int leader = __ffsll((long long)act) - 1;
  const int b0 = __shfl(bucket, leader);
  if (__ballot(active && bucket == b0) == act) {
    int base = 0;
    if (lane == leader) base = atomicAdd(&hist[b0], __popcll(act));
    return __shfl(base, leader) + __popcll(act & ((1ull << lane) - 1ull));
  }
  return active ? atomicAdd(&hist[bucket], 1) : 0;
}

// Reductions over one part of the workgroup: NT threads (whole waves), tp
// the thread's index within its part, scratch NT / 64 values of the part.
// Their barriers are workgroup-wide, so every part calls them together.
template <int NT>
__device__ int part_exclusive_scan(int x, int tp, int* scratch, int* total) {
  const int lane = tp & 63, wave = tp >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int v = scratch[w];
    base += w < wave ? v : 0;
    tot += v;
  }
  *total = tot;
  __syncthreads();
  return base + incl - x;
}

template <int NT>
__device__ long part_sum(long x, int tp, long* scratch) {
  const int lane = tp & 63, wave = tp >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if (lane == 0) scratch[wave] = x;
  __syncthreads();
  long total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) total += scratch[w];
  __syncthreads();
  return total;
}

// The queues and tile slots are built over entries rather than items: entry
// e = (b*Hm + hm)*nBlk + blk is one block of one mask head, with count
// cnt[e], and stands for the reps = H / Hm items (b*H + h)*nBlk + blk of the
// heads h that share that mask head (all H heads when Hm == 1, else h = hm),
// which all have its count.  Its item r (0 <= r < reps):
__device__ __forceinline__ uint32_t entry_item(uint32_t e, uint32_t r, uint32_t H, uint32_t Hm, uint32_t nBlk) {
  const uint32_t bhm = e / nBlk, blk = e - bhm * nBlk;
  const uint32_t b = bhm / Hm, hm = bhm - b * Hm;
  return (b * H + (Hm == 1 ? r : hm)) * nBlk + blk;
}

// x / d for x, d < 2^31, d > 0, given inv = 1.0 / d: the double product is
// within one of the quotient (its error is below 2^-20), and one step
// corrects it (q d <= x + d cannot wrap).
__device__ __forceinline__ uint32_t udiv(uint32_t x, uint32_t d, double inv) {
  uint32_t q = (uint32_t)((double)x * inv);
  const uint32_t qd = q * d;
  if (qd > x) --q;
  else if (x - qd >= d) ++q;
  return q;
}

// Entries per thread and pass whose counts are loaded together: the loads of
// one pass are then in flight at once instead of one after the other.
constexpr int kUnroll = 8;

// Where the sort and the slot scan read the entries' tile counts: global
// memory, or a copy in LDS.  Every global access of the last workgroup is a
// round trip to memory shared by all dies (the counts were written by other
// workgroups' atomics), so when both count arrays fit, the workgroup loads
// them into LDS in one sweep and reads them there.
struct GlobalCounts {
  const int* __restrict__ p;
  __device__ __forceinline__ int operator()(uint32_t e) const { return p[e]; }
};
struct LdsCounts {
  const uint16_t* p;
  __device__ __forceinline__ int operator()(uint32_t e) const { return (int)p[e]; }
};
constexpr int kCountCache = 4096;   // entries per count array held in LDS
// (sorted entries are held as 16-bit numbers, the running sums of the slot
// scan in one histogram, and the scan takes all entries in one sweep)
static_assert(kCountCache <= 65536 && kCountCache <= kBuckets && kCountCache <= kQueueThreads * kUnroll,
              "count cache size");

// Counting sort of the B*H*nBlk items by tile count, descending, by one part
// of the workgroup (NT threads; tp the index within the part).  The m =
// B*Hm*nBlk entries are sorted, and the reps items of each are written next
// to each other.  Counts are at most max_cnt (the number of blocks of the
// other axis); only min(kBuckets, max_cnt + 1) buckets are used, and larger
// counts share the top one.  Every entry lands in a bucket that was cleared,
// so the positions written are a permutation of 0 .. B*H*nBlk - 1 whatever
// the counts hold.  Order inside a count is arbitrary.  The control flow,
// and so the sequence of barriers, is the same for every part whatever its
// data, so two parts can sort two queues side by side.
template <int NT, class Counts>
__device__ void sort_items(int tp, Counts cnt, uint32_t* __restrict__ queue, int B, int H,
                           int Hm, int nBlk, int max_cnt, int* hist, int* scratch, long* lscratch,
                           SplitRule split, uint32_t* split_out, uint16_t* sorted) {
  const uint32_t m = nBlk > 0 ? (uint32_t)B * (uint32_t)Hm * (uint32_t)nBlk : 0u;
  const uint32_t reps = Hm == 1 ? (uint32_t)H : 1u;
  const int nb = min(kBuckets, max(max_cnt, 0) + 1);
  for (int i = tp; i < nb; i += NT) hist[i] = 0;
  __syncthreads();
  // the counts of kUnroll entries per thread (m > 0), clamped to a bucket.
  // Every lane loads (from a valid entry) and the result is dropped past
  // the end: no branch around a load, so the loads are in flight together.
  auto load_counts = [&](uint32_t e0, int (&c)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) c[u] = cnt(min(e0 + (uint32_t)(u * NT + tp), m - 1));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      c[u] = e0 + (uint32_t)(u * NT + tp) < m ? min(max(c[u], 0), nb - 1) : 0;
  };
  for (uint32_t e0 = 0; e0 < m; e0 += NT * kUnroll) {
    int c[kUnroll];
    load_counts(e0, c);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) wave_bucket_add(hist, c[u], e0 + (uint32_t)(u * NT + tp) < m);
  }
  __syncthreads();
  if (split.any) {
    // Which forward items to split, counted in items (the barriers run in
    // every part; when no item may be split, in none).
    long tiles = 0;
    for (int i = tp; i < min(nb, kBuckets - 1); i += NT) tiles += (long)i * hist[i];
    const long total = part_sum<NT>(tiles, tp, lscratch) * (long)reps;
    const long slots = split.on ? max(split.fwd_slots, 1) : 1;
    const long thr = max(16L, (total + 2 * slots - 1) / (2 * slots));
    long above = 0;
    for (int i = tp; i < min(nb, kBuckets - 1); i += NT) above += i > thr ? hist[i] : 0;
    above = part_sum<NT>(above, tp, lscratch) * (long)reps;
    const bool top_used = nb == kBuckets && hist[kBuckets - 1] > 0;
    if (split.on && tp == 0)
      *split_out = (top_used || thr >= kBuckets - 1) ? 0u : (uint32_t)min(above, (long)max(split.split_cap, 0));
  }
  // thread tp owns buckets nb-1-per*tp ... nb-per*(tp+1) (descending order)
  const int per = (nb + NT - 1) / NT;
  int sum = 0;
  for (int u = 0; u < per; ++u) {
    const int bk = nb - 1 - (per * tp + u);
    sum += bk >= 0 ? hist[bk] : 0;
  }
  int total;
  int run = part_exclusive_scan<NT>(sum, tp, scratch, &total);
  for (int u = 0; u < per; ++u) {
    const int bk = nb - 1 - (per * tp + u);
    if (bk >= 0) {
      const int c = hist[bk];
      hist[bk] = run;
      run += c;
    }
  }
  __syncthreads();
  for (uint32_t e0 = 0; e0 < m; e0 += NT * kUnroll) {
    int c[kUnroll];
    load_counts(e0, c);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t e = e0 + (uint32_t)(u * NT + tp);
      const int pos = wave_bucket_add(hist, c[u], e < m);
      if (e < m) {
        if (sorted) {
          sorted[pos] = (uint16_t)e;
        } else {
          for (uint32_t r = 0; r < reps; ++r)
            queue[(uint32_t)pos * reps + r] = entry_item(e, r, (uint32_t)H, (uint32_t)Hm, (uint32_t)nBlk);
        }
      }
    }
  }
  __syncthreads();
  if (sorted) {
    // the queue in order, position p holding item p % reps of the entry
    // sorted to p / reps: consecutive threads store consecutive words
    const double inv_reps = 1.0 / (double)reps, inv_blk = 1.0 / (double)nBlk;
    const uint32_t n = m * reps;
    for (uint32_t p = (uint32_t)tp; p < n; p += NT) {
      const uint32_t k = udiv(p, reps, inv_reps), r = p - k * reps;
      const uint32_t e = sorted[k];
      // item r of entry e: (b*H + h)*nBlk + blk with e = (b*Hm + hm)*nBlk + blk
      const uint32_t it = Hm == 1 ? e + udiv(e, (uint32_t)nBlk, inv_blk) * (uint32_t)(H - 1) * (uint32_t)nBlk + r * (uint32_t)nBlk
                                  : e;
      queue[p] = it;
    }
  }
}

// First tile slot of every backward item.  The slots go to the entries in
// increasing order, and within an entry to its reps items one after the
// other: with E(e) the sum of the counts of the entries before e, item r of
// entry e starts at reps * E(e) + r * cnt[e].  The tiles of one item (its
// list of query blocks, in list order) are then consecutive slots.  The
// total goes to counters[kCtrTiles]; values beyond 2^32 - 1 saturate (no
// cache is that large).  Thread t takes kUnroll consecutive entries of each
// chunk of kQueueThreads * kUnroll.
template <class Counts>
__device__ void tile_slots(Counts cnt, uint32_t* __restrict__ base, int B, int H,
                           int Hm, int nBlk, uint32_t* total_out, int* scratch) {
  const int t = threadIdx.x;
  const uint32_t m = nBlk > 0 ? (uint32_t)B * (uint32_t)Hm * (uint32_t)nBlk : 0u;
  const unsigned long long reps = Hm == 1 ? (unsigned long long)H : 1ull;
  unsigned long long run = 0;   // the same in every thread
  for (uint32_t e0 = 0; e0 < m; e0 += kQueueThreads * kUnroll) {
    const uint32_t first = e0 + (uint32_t)(t * kUnroll);
    int c[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) c[u] = cnt(min(first + u, m - 1));   // no branch around the loads
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) c[u] = first + u < m ? max(c[u], 0) : 0;
    int mine = 0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mine += c[u];
    int chunk_total;
    int excl = block_exclusive_scan(mine, scratch, &chunk_total);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t e = first + u;
      if (e < m) {
        const unsigned long long s0 = reps * (run + (unsigned long long)excl);
        for (uint32_t r = 0; r < (uint32_t)reps; ++r)
          base[entry_item(e, r, (uint32_t)H, (uint32_t)Hm, (uint32_t)nBlk)] =
              (uint32_t)min(s0 + (unsigned long long)r * (unsigned long long)c[u], 0xFFFFFFFFull);
      }
      excl += c[u];
    }
    run += (unsigned long long)chunk_total;
  }
  if (t == 0) *total_out = (uint32_t)min(reps * run, 0xFFFFFFFFull);
}

// tile_slots for counts in LDS (m <= kQueueThreads * kUnroll entries): the
// entries' running sums E(e) go to LDS (ebase), and the slots are then
// written in item order, consecutive threads storing consecutive words.
__device__ void tile_slots_lds(const uint16_t* cnt, uint32_t* __restrict__ base, int B, int H, int Hm,
                               int nBlk, uint32_t* total_out, int* scratch, int* ebase) {
  const int t = threadIdx.x;
  const uint32_t m = nBlk > 0 ? (uint32_t)B * (uint32_t)Hm * (uint32_t)nBlk : 0u;
  const uint32_t first = (uint32_t)(t * kUnroll);
  int c[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) c[u] = first + u < m ? (int)cnt[first + u] : 0;
  int mine = 0;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) mine += c[u];
  int total;
  int excl = block_exclusive_scan(mine, scratch, &total);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (first + u < m) ebase[first + u] = excl;
    excl += c[u];
  }
  __syncthreads();
  const unsigned long long reps = Hm == 1 ? (unsigned long long)H : 1ull;
  const uint32_t n = m * (uint32_t)reps;
  const double inv_blk = 1.0 / (double)nBlk, inv_h = 1.0 / (double)H;
  for (uint32_t i = (uint32_t)t; i < n; i += kQueueThreads) {
    // item i = (b*H + h)*nBlk + kb: entry (b*Hm + hm)*nBlk + kb, head r = h when Hm == 1
    const uint32_t bh = udiv(i, (uint32_t)nBlk, inv_blk), kb = i - bh * (uint32_t)nBlk;
    const uint32_t b = udiv(bh, (uint32_t)H, inv_h), h = bh - b * (uint32_t)H;
    const uint32_t e = Hm == 1 ? b * (uint32_t)nBlk + kb : i;
    const unsigned long long r = Hm == 1 ? h : 0u;
    base[i] = (uint32_t)min(reps * (unsigned long long)ebase[e] + r * (unsigned long long)cnt[e], 0xFFFFFFFFull);
  }
  if (t == 0) *total_out = (uint32_t)min(reps * (unsigned long long)total, 0xFFFFFFFFull);
}

// Compaction of one list: NT threads each hold one candidate entry (keep);
// the kept ones are written in thread order from list[base].  Returns the
// number kept (the same in every thread).  wsum: NT / 64 ints of LDS.
template <int NT>
__device__ __forceinline__ int compact(bool keep, int* wsum, int base, int* pos_out) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const unsigned long long m = __ballot(keep);
  const int pos = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int off = base, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int x = wsum[w];
    off += w < wave ? x : 0;
    total += x;
  }
  *pos_out = off + pos;
  __syncthreads();
  return total;
}

// grid (max(nK, 1), max(B*Hm, 1)), 256 threads.  Workgroup (kb, bhm): the
// summary of key block kb (threads < BK own one column each; columns >= Sk
// do not take part) into kbsum, then the block's column of tiles: for every
// query block that is not skipped, its entry in list_k (increasing order,
// bit 15 if partial) and, in cpos, that entry's position; cnt_k.  Workgroup
// (0, 0) also zeroes the counter the row kernel's workgroups count off on.
__global__ __launch_bounds__(256) void column_kernel(const int4* __restrict__ bounds, int* __restrict__ kbsum,
                                                     int* __restrict__ cnt_k, uint16_t* __restrict__ list_k,
                                                     uint16_t* __restrict__ cpos, uint32_t* __restrict__ counters,
                                                     int Sq, int Sk, int nQ, int nK, long bhm_total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (blockIdx.x == 0 && blockIdx.y == 0 && t == 0) counters[kCtrRowDone] = 0;
  const int kb = blockIdx.x;
  const long bhm = blockIdx.y;
  if (kb >= nK || bhm >= bhm_total) return;
  // ---- key-block summary ----
  const int col = kb * BK + t;
  int mn[4], mx[4];
  if (t < BK && col < Sk) {
    const int4 b = bounds[bhm * Sk + col];
    const int v[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) mn[c] = mx[c] = min(max(v[c], 0), Sq);
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
  __shared__ int red[4][8];
  __shared__ int ks[8];
  __shared__ int wsum[4];
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
    for (int w = 1; w < 4; ++w) r = (t & 1) ? max(r, red[w][t]) : min(r, red[w][t]);
    ks[t] = r;
    kbsum[(bhm * nK + kb) * 8 + t] = r;
  }
  __syncthreads();
  int ksc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) ksc[c] = ks[c];
  // ---- the block's column of tiles ----
  uint16_t* list = list_k + (bhm * nK + kb) * (long)nQ;
  uint16_t* cp = cpos + (bhm * nK + kb) * (long)nQ;
  int base = 0;
  for (int o0 = 0; o0 < nQ; o0 += 256) {
    const int o = o0 + t;
    int c = 0;
    if (o < nQ) c = tile_class(ksc, o * BQ, min(Sq, o * BQ + BQ));
    const bool keep = o < nQ && c != 0;
    int at;
    const int n = compact<256>(keep, wsum, base, &at);
    if (keep) {
      list[at] = (uint16_t)(o | (c == 2 ? kListPartial : 0));
      cp[o] = (uint16_t)at;
    }
    base += n;
  }
  if (t == 0) cnt_k[bhm * nK + kb] = base;
}

// grid (max(nQ, 1), max(B*Hm, 1)), kQueueThreads threads.  Workgroup
// (qb, bhm): the class of every tile of query block qb (cls) from the key
// block summaries, and its list of non-skipped key blocks (list_q, cnt_q).
// In pair mode the workgroup of the second block of a pair (2qp, 2qp+1), or
// of a last block without a partner, also lists the key blocks that either
// block of the pair sees (list_p, cnt_p), classing the first block's tiles
// again for it.  The last workgroup to finish (counted on
// counters[kCtrRowDone], zeroed by the column kernel) then builds, with
// every count in place, the forward queue (of blocks, and how many of them to
// split; or of pairs), the backward queue, the backward items' first tile
// slots, and the counters the attention kernels start from.
__global__ __launch_bounds__(kQueueThreads) void row_kernel(
    const int* __restrict__ kbsum, uint8_t* __restrict__ cls, int* __restrict__ cnt_q,
    const int* __restrict__ cnt_k, uint16_t* __restrict__ list_q, uint32_t* __restrict__ fwd_q,
    uint32_t* __restrict__ bwd_q, uint32_t* __restrict__ colbase, uint32_t* __restrict__ counters,
    int* __restrict__ cnt_p, uint32_t* __restrict__ list_p, int B, int H, int Hm, int Sq, int nQ, int nK,
    int fwd_slots, int split_cap, int pairs) {
  __shared__ int hist[2][kBuckets];
  __shared__ uint16_t ccache[2][kCountCache];
  __shared__ uint16_t sorted[2][kCountCache];
  __shared__ int scratch[kQueueThreads / 64 + 1];
  __shared__ long lscratch[kQueueThreads / 64];
  __shared__ uint32_t last, nsplit, ntiles;
  const int t = threadIdx.x;
  const int qb = blockIdx.x;
  const long bhm = blockIdx.y;
  const int nP = (nQ + 1) >> 1;
  if (qb < nQ && bhm < (long)B * Hm) {
    uint16_t* list = list_q + (bhm * nQ + qb) * (long)nK;
    const int q0 = qb * BQ, q1 = min(Sq, q0 + BQ);
    // (the same in every thread)
    const bool unite = pairs && ((qb & 1) || qb == nQ - 1);
    const bool second = (qb & 1) != 0;
    const int f0 = (qb - 1) * BQ, f1 = min(Sq, f0 + BQ);   // rows of the pair's first block, when second
    uint32_t* plist = list_p + (bhm * nP + (qb >> 1)) * (long)nK;
    int base = 0, ubase = 0;
    for (int o0 = 0; o0 < nK; o0 += kQueueThreads) {
      const int o = o0 + t;
      int c = 0, cf = 0;   // classes of this block's and (second) the first block's tile
      if (o < nK) {
        int ks[8];
        load_ks(kbsum, bhm * nK + o, ks);
        c = tile_class(ks, q0, q1);
        cls[(bhm * nQ + qb) * (long)nK + o] = (uint8_t)c;
        if (unite && second) cf = tile_class(ks, f0, f1);
      }
      const bool keep = o < nK && c != 0;
      int at;
      const int n = compact<kQueueThreads>(keep, scratch, base, &at);
      if (keep) list[at] = (uint16_t)(o | (c == 2 ? kListPartial : 0));
      base += n;
      if (unite) {
        const int c0 = second ? cf : c, c1 = second ? c : 0;   // blocks 2qp and 2qp+1
        const bool ukeep = o < nK && (c0 != 0 || c1 != 0);
        int uat;
        const int un = compact<kQueueThreads>(ukeep, scratch, ubase, &uat);
        if (ukeep)
          plist[uat] = (uint32_t)o | (c0 != 0 ? kPairSee0 : 0u) | (c0 == 2 ? kPairPart0 : 0u) |
                       (c1 != 0 ? kPairSee1 : 0u) | (c1 == 2 ? kPairPart1 : 0u);
        ubase += un;
      }
    }
    // the row's (and pair's) count as an atomic, performed (the value
    // returned) before this workgroup is counted as finished
    if (t == 0) {
      const int old = atomicExch(&cnt_q[bhm * nQ + qb], base);
      const int oldp = unite ? atomicExch(&cnt_p[bhm * nP + (qb >> 1)], ubase) : 0;
      asm volatile("s_waitcnt vmcnt(0)" ::"v"(old), "v"(oldp) : "memory");
    }
  }
  // ---- the last workgroup to finish builds the queues ----
  // Only the counts cross between workgroups here (the lists and classes
  // are read by later kernels).  They are written by atomics, which take
  // effect where every workgroup's atomics do, so no cache write-back is
  // needed for them; the last workgroup drops its own cached copies (an
  // acquire fence) before it reads them.
  if (t == 0) last = atomicAdd(&counters[kCtrRowDone], 1u) == gridDim.x * gridDim.y - 1 ? 1u : 0u;
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (t == 0) nsplit = 0;
  __syncthreads();
  {
    // the two halves of the workgroup sort the two queues side by side
    constexpr int kHalf = kQueueThreads / 2;
    const int part = t / kHalf, tp = t % kHalf;
    const SplitRule sr{part == 0 && split_cap > 0, split_cap > 0, fwd_slots, split_cap};
    int* sc = scratch + part * (kHalf / 64);
    long* lsc = lscratch + part * (kHalf / 64);
    // (a forward item's count is at most nK, a backward item's at most nQ;
    // forward items are query blocks, or in pair mode pairs of them)
    const int nF = pairs ? nP : nQ;
    const int* fcnt = pairs ? cnt_p : cnt_q;
    const int nBlk = part == 0 ? nF : nK, max_cnt = part == 0 ? nK : nQ;
    uint32_t* queue = part == 0 ? fwd_q : bwd_q;
    const long mq = (long)B * Hm * nF, mk = (long)B * Hm * nK;
    if (mq <= kCountCache && mk <= kCountCache) {   // the same in every thread
      int cq[kCountCache / kQueueThreads], ck[kCountCache / kQueueThreads];
      // range-checked buffer loads (zero past the end): no branch around
      // the loads, which are then in flight together
      const BufRsrc rq = make_rsrc(fcnt, (uint32_t)mq * 4u), rk = make_rsrc(cnt_k, (uint32_t)mk * 4u);
#pragma unroll
      for (int u = 0; u < kCountCache / kQueueThreads; ++u) {
        const uint32_t off = (uint32_t)(u * kQueueThreads + t) * 4u;
        cq[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(rq, off, 0, 0);
        ck[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(rk, off, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kCountCache / kQueueThreads; ++u) {
        ccache[0][u * kQueueThreads + t] = (uint16_t)min(max(cq[u], 0), 65535);
        ccache[1][u * kQueueThreads + t] = (uint16_t)min(max(ck[u], 0), 65535);
      }
      __syncthreads();
      sort_items<kHalf>(tp, LdsCounts{ccache[part]}, queue, B, H, Hm, nBlk, max_cnt, hist[part], sc, lsc, sr,
                        &nsplit, sorted[part]);
      // (the histograms are free again: they hold the running sums)
      tile_slots_lds(ccache[1], colbase, B, H, Hm, nK, &ntiles, scratch, hist[0]);
    } else {
      sort_items<kHalf>(tp, GlobalCounts{part == 0 ? fcnt : cnt_k}, queue, B, H, Hm, nBlk, max_cnt, hist[part],
                        sc, lsc, sr, &nsplit, nullptr);
      tile_slots(GlobalCounts{cnt_k}, colbase, B, H, Hm, nK, &ntiles, scratch);
    }
  }
  __syncthreads();
  if (t == 0) {
    counters[kCtrFwdItems] = (uint32_t)((long)B * H * (pairs ? nP : nQ));
    counters[kCtrFwdPairs] = pairs ? 1u : 0u;
    counters[kCtrFwdSplit] = nsplit;
    counters[kCtrFwdNext] = 0;
    counters[kCtrFwdExit] = 0;
    counters[kCtrDqNext] = 0;
    counters[kCtrDqExit] = 0;
    counters[kCtrBwdItems] = (uint32_t)((long)B * H * nK);
    counters[kCtrBwdNext] = 0;
    counters[kCtrBwdExit] = 0;
    counters[kCtrTiles] = ntiles;
    counters[kCtrRowDone] = 0;
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
  // both kernels always run, with at least one workgroup, also for empty
  // problems: they leave (empty) queues and zeroed counters behind, with
  // kernels rather than a memset, which stays correct when a caller replays
  // the calls as a captured graph
  const long bhm = (long)a.B * a.Hm;
  const unsigned gy = (unsigned)(bhm > 0 ? bhm : 1);
  column_kernel<<<dim3((unsigned)(a.nK > 0 ? a.nK : 1), gy), 256, 0, stream>>>(
      a.bounds, a.kbsum, a.cnt_k, a.list_k, a.cpos, a.counters, a.Sq, a.Sk, a.nQ, a.nK, bhm);
  row_kernel<<<dim3((unsigned)(a.nQ > 0 ? a.nQ : 1), gy), kQueueThreads, 0, stream>>>(
      a.kbsum, a.cls, a.cnt_q, a.cnt_k, a.list_q, a.fwd_queue, a.bwd_queue, a.colbase, a.counters, a.cnt_p,
      a.list_p, a.B, a.H, a.Hm, a.Sq, a.nQ, a.nK, a.fwd_slots, a.split_cap, a.pairs);
  return hipGetLastError();
}

}  // namespace fm
