/*
 * fm.h - C ABI of libfm, mask-aware (column-sparse masked) attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The mask is the column-wise sparse form described in the FlashMask-3 paper
 * summary (abstract): for every key column j four int32 values give query-row
 * interval boundaries, and element (i, j) is masked iff
 *
 *        LTS[j] <= i < LTE[j]   or   UTS[j] <= i < UTE[j]
 *
 * (half-open intervals; start >= end means empty).  Masked scores are -inf.
 * A query row with no visible key outputs O = 0, LSE = +inf and gets no
 * gradient.  The softmax scale is passed in (normally 1/sqrt(head_dim)).
 *
 * Layouts (all contiguous, row-major, every tensor pointer 16-byte aligned):
 *   q, o, dout, dq     bf16  [batch][heads][seqlen_q][head_dim]
 *   k, v, dk, dv       bf16  [batch][heads][seqlen_k][head_dim]
 *   lse                fp32  [batch][heads][seqlen_q]   natural-log units
 *   bounds             int32 [batch][mask_heads][seqlen_k][4] = LTS,LTE,UTS,UTE
 * mask_heads is 1 (one mask for every head) or heads (one mask per head).
 * Bound values may be any int32; they are compared as given (clamping them to
 * [0, seqlen_q] changes nothing).
 *
 * Memory: every pointer is a device pointer owned by the caller.  The library
 * allocates nothing and keeps no per-call state; it caches only the device's
 * compute-unit count.  `tileinfo` (size from fm_tileinfo_layout_query) is written by
 * fm_tile_bounds and then read by fm_attn_fwd / fm_attn_bwd, which also use
 * work counters and scratch slots inside it; the counters are left at zero
 * when a call's kernels finish.  Calls that share a tileinfo must therefore be
 * ordered (one stream): no two of them may be in flight at once.
 *
 * Streams: `stream` is a hipStream_t (NULL = default stream).  Every entry
 * point validates its arguments on the host, enqueues its kernels on `stream`
 * and returns without synchronising.
 *
 * Errors: validation happens before anything is enqueued; a failed check
 * returns its code and enqueues nothing.  FM_ERR_HIP means a launch was
 * rejected by the runtime (hipGetLastError); faults inside kernels surface at
 * the caller's next synchronisation.  Nothing is printed.
 */
#ifndef FM_H
#define FM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FM_OK = 0,
  FM_ERR_NULL = 1,        /* a required pointer is NULL                         */
  FM_ERR_SHAPE = 2,       /* a size is negative or beyond the supported range   */
  FM_ERR_UNSUPPORTED = 3, /* head_dim not 64/128, or mask_heads not 1 or heads  */
  FM_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned            */
  FM_ERR_HIP = 5,         /* the HIP runtime rejected a call or launch          */
  FM_ERR_SCRATCH = 6      /* the problem exceeds the library's static scratch   */
} fm_status;

typedef struct {
  int32_t batch;          /* B  >= 0                                            */
  int32_t heads;          /* H  >= 1                                            */
  int32_t mask_heads;     /* Hm, 1 or H                                         */
  int32_t seqlen_q;       /* Sq >= 0                                            */
  int32_t seqlen_k;       /* Sk >= 0                                            */
  int32_t head_dim;       /* D, 64 or 128                                       */
  float softmax_scale;    /* multiplies q.k before the softmax                  */
  int32_t fwd_rows;       /* query rows per forward work item: 0 lets the
                           * library choose; 128 (one query block); 256 (two
                           * neighbouring query blocks of one head, whose
                           * workgroup stages each key block once for both;
                           * head_dim 128 only).  fm_tile_bounds and the
                           * attention calls on one tileinfo must agree on it. */
} fm_problem;

/* Byte offsets of the parts of a tileinfo buffer (each 256-byte aligned), as
 * written by fm_tile_bounds.  nQ = ceil(Sq/block_q), nK = ceil(Sk/block_k).
 *   counters  uint32[16]: [0] forward items (query-block pairs in pair mode),
 *             [1] backward items,
 *             [2],[3] forward / backward next-item counters, [4],[5] exit counters,
 *             [6],[7] the dQ kernel's next-item and exit counters,
 *             [8] forward items split in two (the first entries of fwd_queue),
 *             [9] non-skipped tiles over every (batch, head) pair (saturating),
 *             [10] the tile pass's own count of finished workgroups (left at 0),
 *             [11] 1 in pair mode (forward items of two query blocks), else 0
 *   kbsum     int32 [B][Hm][nK][8]  per key block, over its columns j < Sk, the
 *             min and max of each bound clamped to [0, Sq]:
 *             LTS min, LTS max, LTE min, LTE max, UTS min, UTS max, UTE min, UTE max
 *   cls       uint8 [B][Hm][nQ][nK] tile class: 0 skip, 1 full, 2 partial
 *   cnt_q     int32 [B][Hm][nQ]     non-skipped tiles per query block
 *   cnt_k     int32 [B][Hm][nK]     non-skipped tiles per key block
 *   list_q    uint16[B][Hm][nQ][nK] per query block, its non-skipped key blocks in
 *             increasing order (first cnt_q entries), bit 15 set if partial
 *   list_k    uint16[B][Hm][nK][nQ] per key block, its non-skipped query blocks
 *   fwd_queue uint32[B*H*nQ]         forward items (b*H+h)*nQ+qb, most tiles first;
 *             in pair mode the first B*H*nP entries, nP = ceil(nQ/2), are
 *             pair items (b*H+h)*nP+qp (query blocks 2qp and 2qp+1 < nQ),
 *             most union tiles (cnt_p) first
 *   bwd_queue uint32[B*H*nK]         backward items (b*H+h)*nK+kb, most tiles first
 *   fwd_partials bf16[2*C][block_q][D] then float[2*C][block_q], C = min(B*H*nQ, 512):
 *             for each split forward item, the output and LSE of each half of
 *             its key blocks (scratch of fm_attn_fwd; no meaning between calls)
 *   cpos      uint16[B][Hm][nK][nQ] for each non-skipped tile (qb, kb), the
 *             position of qb in list_k of kb (other entries are not written)
 *   colbase   uint32[B*H*nK]       first tile slot of each backward item
 *             (b*H+h)*nK+kb.  Slots go to the entries e = (b*Hm+hm)*nK+kb in
 *             increasing order and, within an entry, to the R = H/Hm heads
 *             that share it one after the other: head r of entry e (r = h
 *             when Hm == 1, else 0) starts at R*E(e) + r*cnt_k[e], E(e) the
 *             sum of cnt_k over the entries before e.  The tiles of item i,
 *             in its list order, take slots colbase[i] .. colbase[i] + cnt - 1
 *             of the backward's tile cache; counters[9] holds the total
 *             (values saturate at 2^32 - 1)
 *   cnt_p     int32 [B][Hm][nP]     pair mode: key blocks that either query
 *             block of pair qp does not skip (other modes: not written)
 *   list_p    uint32[B][Hm][nP][nK] pair mode: those key blocks in increasing
 *             order (first cnt_p entries): bits 0-15 the block, bit 16 set if
 *             block 2qp sees it, bit 17 if that tile is partial, bits 18 and
 *             19 the same for block 2qp+1 */
typedef struct {
  int32_t block_q, block_k, n_qblocks, n_kblocks;
  size_t counters, kbsum, cls, cnt_q, cnt_k, list_q, list_k, fwd_queue, bwd_queue, fwd_partials;
  size_t cpos, colbase, cnt_p, list_p;
  size_t total;           /* bytes the caller must allocate                     */
} fm_tileinfo_layout;

/* Human-readable name of a status code (static string). */
const char* fm_status_str(fm_status status);

/* Tile shape used by the kernels (block_q query rows x block_k key columns). */
fm_status fm_tile_shape(const fm_problem* p, int32_t* block_q, int32_t* block_k);

/* Size and layout of the tileinfo buffer for problem p (host only). */
fm_status fm_tileinfo_layout_query(const fm_problem* p, fm_tileinfo_layout* out);

/* Bytes of device workspace fm_attn_bwd needs: the fp32 [B][H][Sq] row terms
 * Delta (host only). */
fm_status fm_bwd_workspace_bytes(const fm_problem* p, size_t* bytes);

/* Bytes of a fm_attn_bwd workspace that also holds the tile cache for
 * n_tiles non-skipped tiles (32 KiB each: dS / scale in bf16), after the Delta
 * row terms: the size at which the backward computes dQ from the cache.  The
 * tile count of a problem is counter 9 of its tileinfo after fm_tile_bounds
 * (host only; FM_ERR_SHAPE for n_tiles >= 2^32 - 1). */
fm_status fm_bwd_cache_bytes(const fm_problem* p, uint64_t n_tiles, size_t* bytes);

/* Number of compute units of the current device (queried once, then cached). */
fm_status fm_device_cu_count(int32_t* cus);

/* Benchmark hook.  While set, every fm_attn_fwd / fm_attn_bwd call made from
 * this host thread records the caller's hipEvent_t `begin` on its stream right
 * before launching its main attention kernel (the forward kernel; the
 * backward's dK/dV kernel) and `end` right after it (for the forward, after
 * the merge of split items), and `begin2` / `end2` around the backward's dQ
 * kernels, so that hipEventElapsedTime(begin, end) spans the main kernel (the
 * backward's Delta prologue falls outside).
 * Events must have been created with timing enabled.  All null turns the hook
 * off; either pair may be null; giving only one event of a pair is
 * FM_ERR_NULL.  Nothing else about the calls changes; a failed record makes
 * the call return FM_ERR_HIP. */
fm_status fm_set_kernel_events(void* begin, void* end, void* begin2, void* end2);

/*
 * fm_tile_bounds - classify every (query block, key block) tile.
 * Paper summary, abstract: the mask keeps, per key column, the bounds of the
 * query-row ranges it hides, which lets whole tiles be
 * recognised as fully masked (skipped), unmasked (full) or mixed (partial).
 * Reads `bounds`; writes every part of `tileinfo` and zeroes its counters.
 * Two kernels: per key block, its min/max summary and its column of tiles
 * (list_k, cpos); per query block, its row of tiles (cls, list_q), after
 * which the last workgroup to finish sorts the work queues (heaviest items
 * first) and lays out the backward's tile slots (colbase).
 */
fm_status fm_tile_bounds(const fm_problem* p, const int32_t* bounds, void* tileinfo, void* stream);

/*
 * fm_attn_fwd - masked scaled-dot-product attention forward.
 * "FlashMask-3 targets masked distributed attention on Hopper GPUs",
 * In-depth insight (the abstract): the method is attention under a structured
 * mask held as four query-axis boundary vectors per key position, computed by
 * a mask-aware kernel that works only where the mask leaves keys visible.
 * This is that forward:
 * for every query row i: O_i = sum_j softmax_j(scale * q_i.k_j, masked -> -inf) v_j,
 * LSE_i = log sum_j exp(scale * q_i.k_j) over visible j (+inf if none).
 * Arguments: q bf16 [B][H][Sq][D], k and v bf16 [B][H][Sk][D], bounds int32
 * [B][Hm][Sk][4] (device, read only); tileinfo from fm_tile_bounds for the
 * same problem and bounds (device, read, and its forward counters and
 * partial-result slots written); o bf16 [B][H][Sq][D] and lse fp32 [B][H][Sq]
 * (device, written).  All are caller-owned.
 * Skipped tiles are never touched; the elementwise mask is evaluated only on
 * partial tiles.  bf16 MFMA with fp32 accumulation; O rounded to nearest even.
 * The query blocks that fm_tile_bounds marked for splitting are computed as
 * two halves of their key blocks, whose partial results (in tileinfo) a
 * second kernel merges; the call writes O and LSE of every row either way.
 * Errors: FM_ERR_NULL for a missing tensor that the problem needs (q, o, lse
 * when there are query rows; k, v, bounds when there are keys; tileinfo
 * always), FM_ERR_ALIGN for a tensor not 16-byte aligned (lse: 4 bytes,
 * tileinfo: 256 bytes), the problem's own checks, FM_ERR_HIP for a launch
 * the runtime rejects.  Sq = 0 or B = 0 enqueues nothing.
 */
fm_status fm_attn_fwd(const fm_problem* p, const void* q, const void* k, const void* v,
                      const int32_t* bounds, void* tileinfo, void* o, float* lse, void* stream);

/*
 * fm_attn_fwd_fp8 - the same forward with E4M3 inputs (head_dim 128 only).
 * PaddlePaddle 3.2.0 release note, FlashMask V3 highlights: FlashMask V3
 * comes with FP8 mixed precision; nothing more is specified there.
 * q, k, v are OCP E4M3 codes (1 byte per value, same [B][H][S][128] layouts
 * as the bf16 tensors, 16-byte aligned); `descale` is a HOST array of three
 * fp32 factors (q, k, v), finite and > 0: the value of a code c of tensor x
 * is decode(c) * descale[x].  O (bf16) and LSE (fp32) are those of the exact
 * attention of these values, up to rounding: both products run on the fp8
 * matrix cores with fp32 accumulation, and the softmax probabilities are
 * rounded to E4M3 (error at most 2^-4 relative, or 2^-10 absolute below
 * 2^-6) before the P.V product; the row sums, and so LSE, use the unrounded
 * fp32 probabilities.  NaN codes (0x7F, 0xFF) are not checked: they make the
 * rows that see them NaN.  Needs a tileinfo from fm_tile_bounds for the same
 * problem and bounds; no item is split.
 * Shares the forward's queue counters in tileinfo: calls on one tileinfo,
 * fp8 or not, must be ordered.  Errors: FM_ERR_UNSUPPORTED for head_dim 64
 * or a bad descale; otherwise as fm_attn_fwd.
 */
fm_status fm_attn_fwd_fp8(const fm_problem* p, const void* q, const void* k, const void* v,
                          const float* descale, const int32_t* bounds, void* tileinfo,
                          void* o, float* lse, void* stream);

/*
 * fm_attn_bwd - gradients of fm_attn_fwd given dL/dO.
 * "FlashMask-3 targets masked distributed attention on Hopper GPUs",
 * In-depth insight (the abstract): the mask-aware kernel serves long-context
 * training, so it provides the backward of the masked attention as well,
 * again visiting only the tiles the boundary vectors leave visible.  The
 * gradients are the exact ones of the forward above:
 * with P = exp(scale * q.k - LSE) (0 where masked), dP = dO v^T,
 * Delta_i = sum_d dO_id O_id, dS = P (dP - Delta):
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
 * Arguments: q, o, dout bf16 [B][H][Sq][D], k, v bf16 [B][H][Sk][D], lse
 * fp32 [B][H][Sq] (`o` and `lse` the forward's outputs), bounds int32
 * [B][Hm][Sk][4], tileinfo from fm_tile_bounds (all device, read; the
 * tileinfo's backward counters are written); dq bf16 [B][H][Sq][D], dk, dv
 * bf16 [B][H][Sk][D] (device, written).  `workspace` (device, 16-byte
 * aligned, caller-owned, contents on entry irrelevant) holds
 * `workspace_bytes` bytes, at least fm_bwd_workspace_bytes: the Delta row
 * terms, then optionally the tile cache.  Kernels: Delta; dK and dV
 * key-stationary over the tiles of each key block, which forms dS / scale
 * of every tile (the scale is applied to dK and dQ as they are written); dQ
 * query-stationary over the tiles of each query block.
 * When the workspace holds the tile cache for every non-skipped tile
 * (fm_bwd_cache_bytes of the tile count the tile pass leaves in tileinfo
 * counter 9), the dK/dV kernel also stores dS / scale there (bf16) and dQ is
 * its product with K, read back from the cache; otherwise dQ recomputes S
 * and dP.  The choice is made on the device from the tile count, so a cache
 * sized for other bounds is never overrun: the call falls back to the
 * recompute.  No atomics; the results are deterministic (the two dQ paths
 * both round dS / scale to bf16, but may differ in its last bits).
 * Errors: FM_ERR_NULL for a missing tensor that the problem needs,
 * FM_ERR_ALIGN as fm_attn_fwd (workspace: 16 bytes), FM_ERR_SHAPE when
 * workspace_bytes is below the B*H*Sq*4 bytes of Delta, the problem's own
 * checks, FM_ERR_HIP for a launch the runtime rejects.  With Sq = 0, dK and
 * dV are zero-filled; with Sk = 0, dQ is written as zero.
 */
fm_status fm_attn_bwd(const fm_problem* p, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse,
                      const int32_t* bounds, void* tileinfo,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * fm_localize_bounds - one context-parallel rank's bounds from the global ones.
 * "FlashMask-3 targets masked distributed attention on Hopper GPUs",
 * In-depth insight (the abstract): under any multi-chunk context-parallel
 * assignment, per-rank mask localisation is a clip-shift-max on the boundary
 * vectors that needs no communication, and its result feeds the single-GPU
 * kernel unchanged.
 * The rank holds n_chunks query chunks [chunk_start[c], chunk_start[c] +
 * chunk_len[c]) of the global rows (HOST arrays, 1 <= n_chunks <= 64, starts
 * and lengths >= 0, in increasing global order and disjoint), stacked in
 * that order as its local rows 0 .. Sq_local - 1 (Sq_local = sum of the
 * lengths).  Every bound g of global_bounds (device, int32
 * [batch][mask_heads][seqlen_k][4], any int32 values) becomes, in
 * local_bounds (device, same shape; may not alias), the number of local rows
 * whose global index is below g: the maximum over chunks starting at or
 * before g of the chunk's first local row plus g clipped into the chunk
 * (0 if no chunk starts at or before g).  A local row is then masked for a
 * key exactly when its global row is.  The key axis is unchanged.  Both
 * pointers 16-byte aligned.  Errors: FM_ERR_SHAPE for bad sizes or chunks
 * (overlapping, decreasing, more than 64, Sq_local beyond the library's
 * limit), FM_ERR_NULL, FM_ERR_ALIGN, FM_ERR_HIP.  One kernel on `stream`.
 */
fm_status fm_localize_bounds(int32_t batch, int32_t mask_heads, int32_t seqlen_k, const int32_t* global_bounds,
                             int32_t n_chunks, const int32_t* chunk_start, const int32_t* chunk_len,
                             int32_t* local_bounds, void* stream);

/*
 * fm_attn_bwd_noalloc - fm_attn_bwd without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The Delta row terms that
 * fm_attn_bwd keeps in `workspace` live instead in a static device array of
 * the library, 16 MiB on each GPU the library runs on (held until the process
 * ends), which limits the problem to batch * heads * seqlen_q <= 4194304 rows:
 * larger problems return FM_ERR_SCRATCH and enqueue nothing.  The call
 * allocates nothing; the array's address is looked up once per device, on the
 * first call made with that device current.  Arguments, results (the same
 * kernels run: bit-identical to fm_attn_bwd) and other errors are those of
 * fm_attn_bwd.  Every call on one GPU uses that GPU's array: calls that
 * overlap on one GPU (different streams, different host threads) race and
 * give wrong gradients, so such calls must be ordered.  The array's contents
 * between calls have no meaning (each call writes every value it reads).
 */
fm_status fm_attn_bwd_noalloc(const fm_problem* p, const void* q, const void* k, const void* v,
                              const void* o, const void* dout, const float* lse,
                              const int32_t* bounds, void* tileinfo,
                              void* dq, void* dk, void* dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FM_H */
