// C ABI of libfm: argument checks, tileinfo layout and kernel launches.
// Declared and documented in include/fm.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/fm.h"
#include "common.h"
#include "kernels.h"

namespace {

constexpr long kMaxSeq = 32768L * fm::BQ;   // list entries hold block indices < 32768
static_assert(fm::BQ == fm::BK, "tile shape is square");

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

fm_status check_problem(const fm_problem* p) {
  if (!p) return FM_ERR_NULL;
  if (p->batch < 0 || p->heads < 1 || p->mask_heads < 1 || p->seqlen_q < 0 || p->seqlen_k < 0)
    return FM_ERR_SHAPE;
  if (p->seqlen_q > kMaxSeq || p->seqlen_k > kMaxSeq) return FM_ERR_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return FM_ERR_UNSUPPORTED;
  if (p->mask_heads != 1 && p->mask_heads != p->heads) return FM_ERR_UNSUPPORTED;
  if (!(p->softmax_scale > 0.f) || !std::isfinite(p->softmax_scale)) return FM_ERR_UNSUPPORTED;
  if (p->fwd_rows != 0 && p->fwd_rows != fm::BQ && p->fwd_rows != 2 * fm::BQ) return FM_ERR_UNSUPPORTED;
  if (p->fwd_rows == 2 * fm::BQ && p->head_dim != 128) return FM_ERR_UNSUPPORTED;
  const long nQ = (p->seqlen_q + fm::BQ - 1) / fm::BQ, nK = (p->seqlen_k + fm::BK - 1) / fm::BK;
  const long items = (long)p->batch * p->heads * (nQ > nK ? nQ : nK);
  if (items >= (1L << 31)) return FM_ERR_SHAPE;
  return FM_OK;
}

struct Layout {
  int nQ, nK;
  int split_cap;   // forward items that may be split in two
  size_t counters, kbsum, cls, cnt_q, cnt_k, list_q, list_k, fwd_queue, bwd_queue, fwd_partials, cpos, colbase,
      cnt_p, list_p, total;
};

// Pair mode (forward items of two neighbouring query blocks, head_dim 128):
// asked for with fwd_rows = 256, or chosen when there are at least four
// pairs per workgroup of the pair kernel's grid (one per compute unit), so
// that the longest-first order balances the grid without splitting items.
// fm_tile_bounds and the attention calls take the same decision.
bool pairs_for(const fm_problem* p, int nQ, int cus) {
  if (p->head_dim != 128 || p->fwd_rows == fm::BQ) return false;
  if (p->fwd_rows == 2 * fm::BQ) return true;
  const long pairs = (long)p->batch * p->heads * ((nQ + 1) / 2);
  return pairs >= 2L * cus * fm::fwd_pair_blocks_per_cu();
}

// At most this many forward items are split (two partial-result slots each).
constexpr long kMaxSplitItems = 512;

// Forward items may be split only when there are fewer than four per
// workgroup of the forward's persistent grid: with more, the longest-first
// order already balances the grid, and the kernel without split handling
// runs.  fm_tile_bounds and fm_attn_fwd take the same decision.
int split_cap_for(const fm_problem* p, const Layout& L, int cus) {
  if (pairs_for(p, L.nQ, cus)) return 0;
  const long items = (long)p->batch * p->heads * L.nQ;
  const long slots = (long)cus * fm::fwd_blocks_per_cu(p->head_dim);
  return items < 4 * slots ? L.split_cap : 0;
}

Layout make_layout(const fm_problem* p) {
  Layout L;
  L.nQ = (p->seqlen_q + fm::BQ - 1) / fm::BQ;
  L.nK = (p->seqlen_k + fm::BK - 1) / fm::BK;
  const size_t bhm = (size_t)p->batch * p->mask_heads, bh = (size_t)p->batch * p->heads;
  size_t off = 0;
  L.counters = off;  off = align256(off + 16 * sizeof(uint32_t));
  L.kbsum = off;     off = align256(off + bhm * L.nK * 8 * sizeof(int32_t));
  L.cls = off;       off = align256(off + bhm * L.nQ * L.nK);
  L.cnt_q = off;     off = align256(off + bhm * L.nQ * sizeof(int32_t));
  L.cnt_k = off;     off = align256(off + bhm * L.nK * sizeof(int32_t));
  L.list_q = off;    off = align256(off + bhm * L.nQ * L.nK * sizeof(uint16_t));
  L.list_k = off;    off = align256(off + bhm * L.nK * L.nQ * sizeof(uint16_t));
  L.fwd_queue = off; off = align256(off + bh * L.nQ * sizeof(uint32_t));
  L.bwd_queue = off; off = align256(off + bh * L.nK * sizeof(uint32_t));
  const long items_q = (long)bh * L.nQ;
  L.split_cap = (int)(items_q < kMaxSplitItems ? items_q : kMaxSplitItems);
  L.fwd_partials = off;
  off = align256(off + (size_t)2 * L.split_cap * fm::BQ * ((size_t)p->head_dim * 2 + sizeof(float)));
  L.cpos = off;      off = align256(off + bhm * L.nK * L.nQ * sizeof(uint16_t));
  L.colbase = off;   off = align256(off + bh * L.nK * sizeof(uint32_t));
  // the pair lists only where pair mode can be chosen
  const size_t nP = (p->head_dim == 128 && p->fwd_rows != fm::BQ) ? (size_t)(L.nQ + 1) / 2 : 0;
  L.cnt_p = off;     off = align256(off + bhm * nP * sizeof(int32_t));
  L.list_p = off;    off = align256(off + bhm * nP * L.nK * sizeof(uint32_t));
  L.total = off;
  return L;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

std::mutex g_cu_mutex;
int g_cu_count[64] = {0};

fm_status cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FM_ERR_HIP;
  if (dev < 0 || dev >= 64) return FM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return FM_ERR_HIP;
    g_cu_count[dev] = n;
  }
  *out = g_cu_count[dev];
  return FM_OK;
}

bool tensor_ok(const void* p) { return p != nullptr; }

// Device memory of fm_attn_bwd_noalloc, for callers that cannot allocate:
// Delta of up to kScratchRows query rows (16 MiB), one copy per GPU, held
// until the process ends.  Host code never uses the array's name as an
// address: each device's copy is found with hipGetSymbolAddress once, with
// that device current, and that address is what the kernels are given.
constexpr long kScratchRows = 4L << 20;
static __device__ __align__(256) float scratch[kScratchRows];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[64] = {nullptr};

fm_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FM_ERR_HIP;
  if (dev < 0 || dev >= 64) return FM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FM_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FM_OK;
}

thread_local fm::KernelEvents g_events;

}  // namespace

extern "C" {

const char* fm_status_str(fm_status s) {
  // A C caller may pass any int; reading such a value as the C++ enum would
  // be undefined, so the argument's bits are taken as an integer.
  int code;
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case FM_OK: return "FM_OK";
    case FM_ERR_NULL: return "FM_ERR_NULL: a required pointer is NULL";
    case FM_ERR_SHAPE: return "FM_ERR_SHAPE: a size is negative or beyond the supported range";
    case FM_ERR_UNSUPPORTED:
      return "FM_ERR_UNSUPPORTED: head_dim must be 64 or 128, mask_heads 1 or heads, scale > 0";
    case FM_ERR_ALIGN: return "FM_ERR_ALIGN: a tensor pointer is not suitably aligned";
    case FM_ERR_HIP: return "FM_ERR_HIP: the HIP runtime rejected a call or launch";
    case FM_ERR_SCRATCH:
      return "FM_ERR_SCRATCH: batch * heads * seqlen_q exceeds the 4194304 rows of the static scratch array";
  }
  return "unknown fm_status";
}

fm_status fm_tile_shape(const fm_problem* p, int32_t* block_q, int32_t* block_k) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (!block_q || !block_k) return FM_ERR_NULL;
  *block_q = fm::BQ;
  *block_k = fm::BK;
  return FM_OK;
}

fm_status fm_tileinfo_layout_query(const fm_problem* p, fm_tileinfo_layout* out) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (!out) return FM_ERR_NULL;
  Layout L = make_layout(p);
  out->block_q = fm::BQ;
  out->block_k = fm::BK;
  out->n_qblocks = L.nQ;
  out->n_kblocks = L.nK;
  out->counters = L.counters;
  out->kbsum = L.kbsum;
  out->cls = L.cls;
  out->cnt_q = L.cnt_q;
  out->cnt_k = L.cnt_k;
  out->list_q = L.list_q;
  out->list_k = L.list_k;
  out->fwd_queue = L.fwd_queue;
  out->bwd_queue = L.bwd_queue;
  out->fwd_partials = L.fwd_partials;
  out->cpos = L.cpos;
  out->colbase = L.colbase;
  out->cnt_p = L.cnt_p;
  out->list_p = L.list_p;
  out->total = L.total;
  return FM_OK;
}

fm_status fm_bwd_workspace_bytes(const fm_problem* p, size_t* bytes) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (!bytes) return FM_ERR_NULL;
  const size_t rows = (size_t)p->batch * p->heads * p->seqlen_q;
  *bytes = align256(rows * sizeof(float));
  return FM_OK;
}

fm_status fm_bwd_cache_bytes(const fm_problem* p, uint64_t n_tiles, size_t* bytes) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (!bytes) return FM_ERR_NULL;
  if (n_tiles > 0xFFFFFFFEull) return FM_ERR_SHAPE;
  const size_t rows = (size_t)p->batch * p->heads * p->seqlen_q;
  *bytes = align256(rows * sizeof(float)) + (size_t)n_tiles * fm::kTileBytes;
  return FM_OK;
}

fm_status fm_localize_bounds(int32_t batch, int32_t mask_heads, int32_t seqlen_k, const int32_t* global_bounds,
                             int32_t n_chunks, const int32_t* chunk_start, const int32_t* chunk_len,
                             int32_t* local_bounds, void* stream) {
  if (batch < 0 || mask_heads < 1 || seqlen_k < 0) return FM_ERR_SHAPE;
  if (n_chunks < 1 || n_chunks > fm::kMaxLocalChunks) return FM_ERR_SHAPE;
  if (!chunk_start || !chunk_len) return FM_ERR_NULL;
  fm::LocalizeArgs a;
  a.n_chunks = n_chunks;
  long off = 0, prev_end = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const long s = chunk_start[c], l = chunk_len[c];
    if (s < 0 || l < 0 || s < prev_end) return FM_ERR_SHAPE;   // increasing, disjoint
    prev_end = s + l;
    if (prev_end > INT32_MAX) return FM_ERR_SHAPE;
    a.start[c] = (int)s;
    a.len[c] = (int)l;
    a.off[c] = (int)off;
    off += l;
  }
  if (off > kMaxSeq) return FM_ERR_SHAPE;                         // local rows must fit one problem
  const long n = (long)batch * mask_heads * seqlen_k;
  if (n > 0 && (!global_bounds || !local_bounds)) return FM_ERR_NULL;
  if (!aligned(global_bounds, 16) || !aligned(local_bounds, 16)) return FM_ERR_ALIGN;
  return fm::launch_localize(reinterpret_cast<const int4*>(global_bounds), reinterpret_cast<int4*>(local_bounds),
                             n, a, (hipStream_t)stream) == hipSuccess
             ? FM_OK
             : FM_ERR_HIP;
}

fm_status fm_device_cu_count(int32_t* cus) {
  if (!cus) return FM_ERR_NULL;
  int n = 0;
  fm_status st = cu_count(&n);
  if (st == FM_OK) *cus = n;
  return st;
}

fm_status fm_set_kernel_events(void* begin, void* end, void* begin2, void* end2) {
  if ((begin == nullptr) != (end == nullptr) || (begin2 == nullptr) != (end2 == nullptr))
    return FM_ERR_NULL;
  g_events.begin = static_cast<hipEvent_t>(begin);
  g_events.end = static_cast<hipEvent_t>(end);
  g_events.begin2 = static_cast<hipEvent_t>(begin2);
  g_events.end2 = static_cast<hipEvent_t>(end2);
  return FM_OK;
}

fm_status fm_tile_bounds(const fm_problem* p, const int32_t* bounds, void* tileinfo, void* stream) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (!tileinfo) return FM_ERR_NULL;
  if (!aligned(tileinfo, 256)) return FM_ERR_ALIGN;
  const bool has_cols = p->batch > 0 && p->seqlen_k > 0;
  if (has_cols && !bounds) return FM_ERR_NULL;
  if (bounds && !aligned(bounds, 16)) return FM_ERR_ALIGN;
  Layout L = make_layout(p);
  fm::TileArgs a;
  a.bounds = reinterpret_cast<const int4*>(bounds);
  a.kbsum = at<int>(tileinfo, L.kbsum);
  a.cls = at<uint8_t>(tileinfo, L.cls);
  a.cnt_q = at<int>(tileinfo, L.cnt_q);
  a.cnt_k = at<int>(tileinfo, L.cnt_k);
  a.list_q = at<uint16_t>(tileinfo, L.list_q);
  a.list_k = at<uint16_t>(tileinfo, L.list_k);
  a.cpos = at<uint16_t>(tileinfo, L.cpos);
  a.fwd_queue = at<uint32_t>(tileinfo, L.fwd_queue);
  a.bwd_queue = at<uint32_t>(tileinfo, L.bwd_queue);
  a.colbase = at<uint32_t>(tileinfo, L.colbase);
  a.counters = at<uint32_t>(tileinfo, L.counters);
  a.cnt_p = at<int>(tileinfo, L.cnt_p);
  a.list_p = at<uint32_t>(tileinfo, L.list_p);
  a.B = p->batch; a.H = p->heads; a.Hm = p->mask_heads;
  a.Sq = p->seqlen_q; a.Sk = p->seqlen_k; a.nQ = L.nQ; a.nK = L.nK;
  int cus = 0;
  if ((st = cu_count(&cus)) != FM_OK) return st;
  a.fwd_slots = cus * fm::fwd_blocks_per_cu(p->head_dim);
  a.split_cap = split_cap_for(p, L, cus);
  a.pairs = pairs_for(p, L.nQ, cus) ? 1 : 0;
  return fm::launch_tile_bounds(a, (hipStream_t)stream) == hipSuccess ? FM_OK : FM_ERR_HIP;
}

fm_status fm_attn_fwd(const fm_problem* p, const void* q, const void* k, const void* v,
                      const int32_t* bounds, void* tileinfo, void* o, float* lse, void* stream) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  const bool has_rows = p->batch > 0 && p->seqlen_q > 0;
  const bool has_cols = p->batch > 0 && p->seqlen_k > 0;
  if (!tileinfo) return FM_ERR_NULL;
  if (has_rows && (!tensor_ok(q) || !tensor_ok(o) || !lse)) return FM_ERR_NULL;
  if (has_cols && (!tensor_ok(k) || !tensor_ok(v) || !bounds)) return FM_ERR_NULL;
  if (!aligned(tileinfo, 256) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(bounds, 16) || !aligned(lse, 4))
    return FM_ERR_ALIGN;
  if (!has_rows) return FM_OK;
  Layout L = make_layout(p);
  int cus = 0;
  if ((st = cu_count(&cus)) != FM_OK) return st;
  fm::FwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.bounds = reinterpret_cast<const int4*>(bounds);
  a.list_q = at<uint16_t>(tileinfo, L.list_q);
  a.cnt_q = at<int>(tileinfo, L.cnt_q);
  a.queue = at<uint32_t>(tileinfo, L.fwd_queue);
  a.counters = at<uint32_t>(tileinfo, L.counters);
  a.partials = at<float>(tileinfo, L.fwd_partials);
  a.list_p = at<uint32_t>(tileinfo, L.list_p);
  a.cnt_p = at<int>(tileinfo, L.cnt_p);
  a.split_cap = split_cap_for(p, L, cus);
  a.B = p->batch; a.H = p->heads; a.Hm = p->mask_heads;
  a.Sq = p->seqlen_q; a.Sk = p->seqlen_k; a.nQ = L.nQ; a.nK = L.nK;
  a.scale_log2 = p->softmax_scale * fm::kLog2e;
  if (pairs_for(p, L.nQ, cus)) {
    const long pairs = (long)p->batch * p->heads * ((L.nQ + 1) / 2);
    const long slots = (long)cus * fm::fwd_pair_blocks_per_cu();
    const int grid = (int)(pairs < slots ? pairs : slots);
    return fm::launch_attn_fwd_pair(a, grid, (hipStream_t)stream, g_events) == hipSuccess ? FM_OK : FM_ERR_HIP;
  }
  // tickets: every item, plus a second one for each item that may be split
  const long items = (long)p->batch * p->heads * L.nQ;
  const long tickets = items + (items < a.split_cap ? items : a.split_cap);
  const long slots = (long)cus * fm::fwd_blocks_per_cu(p->head_dim);
  const int grid = (int)(tickets < slots ? tickets : slots);
  return fm::launch_attn_fwd(a, p->head_dim, grid, (hipStream_t)stream, g_events) == hipSuccess
             ? FM_OK
             : FM_ERR_HIP;
}

fm_status fm_attn_fwd_fp8(const fm_problem* p, const void* q, const void* k, const void* v,
                          const float* descale, const int32_t* bounds, void* tileinfo, void* o, float* lse,
                          void* stream) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (p->head_dim != 128) return FM_ERR_UNSUPPORTED;
  if (!descale) return FM_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (!(descale[i] > 0.f) || !std::isfinite(descale[i])) return FM_ERR_UNSUPPORTED;
  const float qk = p->softmax_scale * descale[0] * descale[1];
  if (!(qk > 0.f) || !std::isfinite(qk)) return FM_ERR_UNSUPPORTED;
  const bool has_rows = p->batch > 0 && p->seqlen_q > 0;
  const bool has_cols = p->batch > 0 && p->seqlen_k > 0;
  if (!tileinfo) return FM_ERR_NULL;
  if (has_rows && (!tensor_ok(q) || !tensor_ok(o) || !lse)) return FM_ERR_NULL;
  if (has_cols && (!tensor_ok(k) || !tensor_ok(v) || !bounds)) return FM_ERR_NULL;
  if (!aligned(tileinfo, 256) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(bounds, 16) || !aligned(lse, 4))
    return FM_ERR_ALIGN;
  if (!has_rows) return FM_OK;
  Layout L = make_layout(p);
  int cus = 0;
  if ((st = cu_count(&cus)) != FM_OK) return st;
  fm::Fp8FwdArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.o = static_cast<__bf16*>(o);
  a.lse = lse;
  a.bounds = reinterpret_cast<const int4*>(bounds);
  a.list_q = at<uint16_t>(tileinfo, L.list_q);
  a.cnt_q = at<int>(tileinfo, L.cnt_q);
  a.queue = at<uint32_t>(tileinfo, L.fwd_queue);
  a.counters = at<uint32_t>(tileinfo, L.counters);
  a.B = p->batch; a.H = p->heads; a.Hm = p->mask_heads;
  a.Sq = p->seqlen_q; a.Sk = p->seqlen_k; a.nQ = L.nQ; a.nK = L.nK;
  a.scale_log2 = qk * fm::kLog2e;
  a.o_scale = descale[2];
  const long items = (long)p->batch * p->heads * L.nQ;
  const long slots = (long)cus * fm::fwd_blocks_per_cu(p->head_dim);
  const int grid = (int)(items < slots ? items : slots);
  return fm::launch_attn_fwd_fp8(a, grid, (hipStream_t)stream, g_events) == hipSuccess ? FM_OK : FM_ERR_HIP;
}

// The backward of fm_attn_bwd and fm_attn_bwd_noalloc.  Delta (fp32, one
// value per query row) goes to the caller's `workspace`, or with
// use_scratch to the library's static scratch array (looked up after every
// argument check has passed).
static fm_status attn_bwd(const fm_problem* p, const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse,
                          const int32_t* bounds, void* tileinfo,
                          void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                          bool use_scratch, void* stream) {
  fm_status st = check_problem(p);
  if (st != FM_OK) return st;
  if (use_scratch && (long)p->batch * p->heads * p->seqlen_q > kScratchRows) return FM_ERR_SCRATCH;
  const bool has_rows = p->batch > 0 && p->seqlen_q > 0;
  const bool has_cols = p->batch > 0 && p->seqlen_k > 0;
  if (!tileinfo) return FM_ERR_NULL;
  if (has_rows && (!tensor_ok(q) || !tensor_ok(o) || !tensor_ok(dout) || !lse || !tensor_ok(dq) ||
                   (!use_scratch && !workspace)))
    return FM_ERR_NULL;
  if (has_cols && (!tensor_ok(k) || !tensor_ok(v) || !bounds || !tensor_ok(dk) || !tensor_ok(dv)))
    return FM_ERR_NULL;
  if (!aligned(tileinfo, 256) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
      !aligned(dv, 16) || !aligned(bounds, 16) || !aligned(lse, 4) || !aligned(workspace, 16))
    return FM_ERR_ALIGN;
  // the workspace must hold Delta (fm_bwd_workspace_bytes), else the first
  // kernel would write past it
  if (!use_scratch && has_rows && workspace_bytes < (size_t)p->batch * p->heads * p->seqlen_q * sizeof(float))
    return FM_ERR_SHAPE;
  if (!has_rows && !has_cols) return FM_OK;
  Layout L = make_layout(p);
  const hipStream_t s = (hipStream_t)stream;
  if (!has_rows) {
    // no query rows: every key gets zero gradient
    const size_t bytes = (size_t)p->batch * p->heads * p->seqlen_k * p->head_dim * 2;
    if (fm::launch_zero16(dk, bytes, s) != hipSuccess || fm::launch_zero16(dv, bytes, s) != hipSuccess)
      return FM_ERR_HIP;
    return FM_OK;
  }
  int cus = 0;
  if ((st = cu_count(&cus)) != FM_OK) return st;
  if (use_scratch && (st = scratch_address(&workspace)) != FM_OK) return st;
  fm::BwdArgs a;
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.o = static_cast<const __bf16*>(o);
  a.dout = static_cast<const __bf16*>(dout);
  a.lse = lse;
  a.bounds = reinterpret_cast<const int4*>(bounds);
  a.list_k = at<uint16_t>(tileinfo, L.list_k);
  a.cnt_k = at<int>(tileinfo, L.cnt_k);
  a.queue = at<uint32_t>(tileinfo, L.bwd_queue);
  a.list_q = at<uint16_t>(tileinfo, L.list_q);
  a.cnt_q = at<int>(tileinfo, L.cnt_q);
  a.queue_q = at<uint32_t>(tileinfo, L.fwd_queue);
  a.counters = at<uint32_t>(tileinfo, L.counters);
  a.dq = static_cast<__bf16*>(dq);
  a.dk = static_cast<__bf16*>(dk);
  a.dv = static_cast<__bf16*>(dv);
  a.delta = static_cast<float*>(workspace);
  // the tile cache: whatever the workspace holds beyond Delta, in whole tiles
  const size_t delta_bytes = align256((size_t)p->batch * p->heads * p->seqlen_q * sizeof(float));
  const size_t cache_tiles = !use_scratch && workspace_bytes > delta_bytes
                                 ? (workspace_bytes - delta_bytes) / fm::kTileBytes
                                 : 0;
  a.ds_cap = (uint32_t)(cache_tiles < 0xFFFFFFFEu ? cache_tiles : 0xFFFFFFFEu);
  a.ds = a.ds_cap > 0 ? reinterpret_cast<__bf16*>(static_cast<char*>(workspace) + delta_bytes) : nullptr;
  a.colbase = at<uint32_t>(tileinfo, L.colbase);
  a.cpos = at<uint16_t>(tileinfo, L.cpos);
  a.B = p->batch; a.H = p->heads; a.Hm = p->mask_heads;
  a.Sq = p->seqlen_q; a.Sk = p->seqlen_k; a.nQ = L.nQ; a.nK = L.nK;
  a.scale = p->softmax_scale;
  a.scale_log2 = p->softmax_scale * fm::kLog2e;
  a.pairs = pairs_for(p, L.nQ, cus) ? 1 : 0;
  const long items = (long)p->batch * p->heads * L.nK;
  const long slots = (long)cus * fm::bwd_blocks_per_cu(p->head_dim);
  const int grid = (int)(items < slots ? items : slots);
  const long dq_items = (long)p->batch * p->heads * L.nQ;
  const int dq_grid = (int)(dq_items < cus ? dq_items : cus);
  return fm::launch_attn_bwd(a, p->head_dim, grid, dq_grid, s, g_events) == hipSuccess ? FM_OK
                                                                                        : FM_ERR_HIP;
}

fm_status fm_attn_bwd(const fm_problem* p, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse,
                      const int32_t* bounds, void* tileinfo,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return attn_bwd(p, q, k, v, o, dout, lse, bounds, tileinfo, dq, dk, dv, workspace, workspace_bytes, false,
                  stream);
}

fm_status fm_attn_bwd_noalloc(const fm_problem* p, const void* q, const void* k, const void* v,
                              const void* o, const void* dout, const float* lse,
                              const int32_t* bounds, void* tileinfo,
                              void* dq, void* dk, void* dv, void* stream) {
  return attn_bwd(p, q, k, v, o, dout, lse, bounds, tileinfo, dq, dk, dv, nullptr, 0, true, stream);
}

}  // extern "C"
