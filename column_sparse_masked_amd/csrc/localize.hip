// Per-rank localisation of the column-sparse mask for context parallelism.
// FlashMask-3 paper summary, abstract: under a multi-chunk context-parallel
// assignment, each rank obtains its mask from the global boundary vectors by
// a clip-shift-max that needs no communication, and the result feeds the
// single-GPU kernel unchanged.
//
// A rank holds query chunks [start_c, start_c + len_c) of the global rows,
// listed in increasing global order and stacked as its local rows (chunk c
// starts at local row off_c = len_0 + ... + len_{c-1}).  Local row order then
// follows global row order, so an interval [g0, g1) of global rows hides
// exactly the local rows [loc(g0), loc(g1)), where loc(g) is the number of
// local rows whose global index is below g:
//     loc(g) = max over chunks with start_c <= g of
//              off_c + clip(g - start_c, 0, len_c)        (0 if there is none)
// i.e. clip into the chunk, shift by its local offset, keep the maximum.
// Each key column's four bounds are mapped independently; the key axis is
// untouched (every rank sees every key).
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {

namespace {

__device__ __forceinline__ int localize_one(int g, const LocalizeArgs& a) {
  long best = 0;
  for (int c = 0; c < a.n_chunks; ++c) {
    const long s = a.start[c];
    if ((long)g >= s) {
      const long in = min(max((long)g - s, 0L), (long)a.len[c]);
      best = max(best, (long)a.off[c] + in);
    }
  }
  return (int)best;
}

}  // namespace

__global__ __launch_bounds__(256) void localize_kernel(const int4* __restrict__ gb, int4* __restrict__ lb,
                                                       long n, const LocalizeArgs a) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const int4 x = gb[i];
    lb[i] = make_int4(localize_one(x.x, a), localize_one(x.y, a), localize_one(x.z, a), localize_one(x.w, a));
  }
}

hipError_t launch_localize(const int4* gb, int4* lb, long n, const LocalizeArgs& a, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  localize_kernel<<<(unsigned)(blocks < 8192 ? blocks : 8192), 256, 0, stream>>>(gb, lb, n, a);
  return hipGetLastError();
}

}  // namespace fm
