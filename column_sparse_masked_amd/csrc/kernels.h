// Launch interfaces between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

struct TileArgs {
  const int4* bounds;
  int* kbsum;
  uint8_t* cls;
  int* cnt_q;
  int* cnt_k;
  uint16_t* list_q;
  uint16_t* list_k;
  uint16_t* cpos;       // [B*Hm][nK][nQ]: position of a listed tile in its key block's list
  uint32_t* fwd_queue;
  uint32_t* bwd_queue;
  uint32_t* colbase;    // [B*H*nK]: first tile slot of each backward item
  uint32_t* counters;
  int* cnt_p;           // pair mode: [B*Hm][nP] key blocks either block of pair qp does not skip
  uint32_t* list_p;     // pair mode: [B*Hm][nP][nK] those blocks with per-block flags
  int B, H, Hm, Sq, Sk, nQ, nK;
  int fwd_slots;   // workgroups of the forward's persistent grid
  int split_cap;   // forward items that may be split (partial-result slots / 2)
  int pairs;       // forward items are pairs of neighbouring query blocks
};

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  const int4* bounds;
  const uint16_t* list_q;
  const int* cnt_q;
  const uint32_t* queue;
  uint32_t* counters;
  float* partials;    // bf16 O [2 split_cap][BQ][D], then fp32 LSE [2 split_cap][BQ]: halves of split items
  const uint32_t* list_p;   // pair mode: union lists of query-block pairs
  const int* cnt_p;
  int split_cap;
  int B, H, Hm, Sq, Sk, nQ, nK;
  float scale_log2;   // softmax_scale * log2(e)
};

// The fp8 forward (head_dim 128): E4M3 q, k, v with per-tensor descales.
struct Fp8FwdArgs {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  __bf16* o;
  float* lse;
  const int4* bounds;
  const uint16_t* list_q;
  const int* cnt_q;
  const uint32_t* queue;
  uint32_t* counters;
  int B, H, Hm, Sq, Sk, nQ, nK;
  float scale_log2;   // softmax_scale * descale_q * descale_k * log2(e)
  float o_scale;      // descale_v
};

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  const int4* bounds;
  const uint16_t* list_k;    // key-stationary walk (dK, dV)
  const int* cnt_k;
  const uint32_t* queue;
  const uint16_t* list_q;    // query-stationary walk (dQ)
  const int* cnt_q;
  const uint32_t* queue_q;
  uint32_t* counters;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* delta;       // fp32 [B][H][Sq]
  // Tile cache: dS' = dS / scale of every non-skipped tile, bf16 [slot][BQ rows][BK keys],
  // written by the key-stationary kernel and read by the dQ kernel.  Used
  // when ds_cap > 0 and the tile pass counted at most ds_cap tiles.
  __bf16* ds;
  uint32_t ds_cap;
  const uint32_t* colbase;   // first slot of each backward item
  const uint16_t* cpos;      // [B*Hm][nK][nQ]: position of a tile in its key block's list
  int B, H, Hm, Sq, Sk, nQ, nK;
  int pairs;          // the forward queue holds pairs of query blocks
  float scale;        // softmax_scale
  float scale_log2;   // softmax_scale * log2(e)
};

hipError_t launch_tile_bounds(const TileArgs& a, hipStream_t stream);

// Context-parallel localisation of the bounds (kernel in localize.hip): a
// rank's query chunks, in increasing global order, and each chunk's first
// local row.
constexpr int kMaxLocalChunks = 64;
struct LocalizeArgs {
  int n_chunks;
  int start[kMaxLocalChunks];
  int len[kMaxLocalChunks];
  int off[kMaxLocalChunks];
};
hipError_t launch_localize(const int4* gb, int4* lb, long n, const LocalizeArgs& a, hipStream_t stream);
// Optional events recorded right before / after the main attention kernel
// (the forward kernel, the backward's dK/dV kernel) and around the backward's
// dQ kernel (null: not recorded).
struct KernelEvents {
  hipEvent_t begin = nullptr, end = nullptr;
  hipEvent_t begin2 = nullptr, end2 = nullptr;
};

hipError_t launch_attn_fwd(const FwdArgs& a, int head_dim, int grid, hipStream_t stream,
                           const KernelEvents& ev);
// Pair mode (head_dim 128): one workgroup of 8 waves per pair of query blocks.
hipError_t launch_attn_fwd_pair(const FwdArgs& a, int grid, hipStream_t stream, const KernelEvents& ev);
hipError_t launch_attn_fwd_fp8(const Fp8FwdArgs& a, int grid, hipStream_t stream, const KernelEvents& ev);
hipError_t launch_attn_bwd(const BwdArgs& a, int head_dim, int grid, int dq_grid,
                           hipStream_t stream, const KernelEvents& ev);
hipError_t launch_attn_bwd_dq(const BwdArgs& a, int head_dim, int grid, hipStream_t stream);
hipError_t launch_attn_bwd_dq_cached(const BwdArgs& a, int head_dim, hipStream_t stream);
// Zero-fills `bytes` (a multiple of 16) at the 16-byte aligned `p`.
hipError_t launch_zero16(void* p, size_t bytes, hipStream_t stream);

// Workgroups per compute unit the persistent kernels are sized for.
int fwd_blocks_per_cu(int head_dim);
int fwd_pair_blocks_per_cu();
int bwd_blocks_per_cu(int head_dim);   // the dQ kernel: one workgroup per CU

}  // namespace fm
