// dQ of column-sparse masked attention from the tile cache (bf16 MFMA, fp32
// accumulate).  FlashMask-3 paper summary, abstract: the mask-aware kernel
// visits only the tiles the column-wise sparse mask does not fully hide.
//
// The key-stationary backward kernel already forms dS' = dS / scale of every
// non-skipped tile; with the tile cache on it also stores it, one tile per
// slot (bf16, 128 rows x 128 keys, in the blocks of 4 rows x 1 key per 8
// bytes in which its waves hold it), and this kernel only has to contract it
// with K:
//     dQ_i = scale * sum over the query block's listed key blocks kb of
//            sum_j dS'_ij K_j,
// with no exponentials, no interval tests and no recomputed S or dP.  The
// work is then bound by reading the cached tiles from memory (32 KiB per
// tile against 4 MFLOP of products), not by the matrix cores.
//
// One workgroup (4 waves) per query block, taken in the forward queue's
// order (most tiles first).  Wave w accumulates dQ^T of rows 32 w .. +32:
//     dQ^T += K^T dS^T     A operand: K^T rows (8 keys of one head-dim column)
//                          B operand: dS rows (8 keys of one query row)
// Both operands need 8 consecutive keys per lane, while K holds keys as rows
// and the cache holds 4 rows per key: each tile's K (units of 4 keys x 8
// columns) and dS (units of 4 keys x 4 rows) are loaded into registers and
// stored transposed into LDS by maps free of bank conflicts, so every
// operand is one 16-byte LDS read.  Every K load instruction of a wave
// covers whole cache lines (8 lanes per 128 bytes): 16-byte loads that each
// touch half a line keep the address unit busy longer.  The loads run two
// tiles ahead of the products.
// The cache is addressed by slot: the tiles of a key block's backward item
// take consecutive slots from colbase[item] in its list order, so the slot
// of tile (qb, kb) is colbase[(b H + h) nK + kb] + cpos[kb][qb]; a table of
// up to 256 of them is resolved into LDS at the start of a query block.
#include "common.h"
#include "kernels.h"

namespace fm {

namespace {

constexpr int kCqThreads = 256;   // 4 waves
constexpr int kTab = 256;         // tiles resolved per table fill

template <int D>
struct CqSmem {
  static constexpr int ST = BK + 8;    // row stride (elements) of both transposed tiles
  static_assert((8 * ST * 2) % 128 == 0, "8 transposed rows start on the same bank");
  static_assert(ST * 2 % 128 == 16, "neighbouring transposed rows 16 bytes apart in the bank period");
  bf16 kt[D * ST];     // K^T: one head-dim column per row, keys in groups of 8 swizzled (kt_key)
  bf16 ds[BQ * ST];    // dS: one query row per row, keys in natural order
  uint32_t slot[kTab];   // cache slot of table entry i
  uint32_t key0[kTab];   // first key of its key block
};

// Place of key x of head-dim column c in the K^T tile: groups of 8 keys are
// swizzled by the column's 16-byte chunk (c / 8), so that the 8 chunks one
// load instruction brings for a key land in 8 different bank slots.
__device__ __forceinline__ int kt_key(int c, int x) { return x ^ (8 * ((c >> 3) & 7)); }

// Global -> register staging of a tile of BK keys x COLS head-dim columns of
// K, 256 threads, in units of 4 keys x 8 columns (one 16-byte chunk of 4
// neighbouring keys).  Unit p = t + 256 j of the tile: within its group of
// 64, lane bits 0-2 pick the chunk and bits 3-5 the key unit, so the 4 load
// instructions (one per key of the unit) each cover 8 whole 128-byte lines.
template <int COLS>
struct TileStage {
  static constexpr int CPR = COLS / 8;                       // 16-byte chunks per key
  static constexpr int NU = (BK / 4) * CPR / kCqThreads;     // units per thread
  static_assert(NU >= 1 && ((BK / 4) * CPR) % kCqThreads == 0 && CPR % 8 == 0, "whole units per thread");
  bf16x8 v[NU][4];
  static __device__ __forceinline__ int key(unsigned t, int j) {
    const int p = (int)t + kCqThreads * j;
    return 4 * (8 * ((p >> 6) / (CPR / 8)) + ((p >> 3) & 7));
  }
  static __device__ __forceinline__ int col(unsigned t, int j) {
    const int p = (int)t + kCqThreads * j;
    return 8 * ((p >> 6) % (CPR / 8)) + (p & 7);
  }
};

// keys k0 .. k0 + BK of a source whose keys are runs of COLS bf16 values
template <int COLS>
__device__ __forceinline__ void tile_load(TileStage<COLS>& r, BufRsrc src, int k0, unsigned t, int salt) {
  using S = TileStage<COLS>;
#pragma unroll
  for (int j = 0; j < S::NU; ++j) {
    const uint32_t base = opaque(((uint32_t)S::key(t, j) * S::CPR + S::col(t, j)) * 16u, salt) +
                          (uint32_t)k0 * (COLS * 2);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r.v[j][rr] = buf_load16(src, base + (uint32_t)rr * (COLS * 2));
  }
}

// transposed into LDS: column c of key k goes to dst[c * ST + kt_key(c, k)]
// (the 8 columns of a chunk share the swizzle; 16 lanes served together hit
// 8 chunks x 2 key units, 16 different 8-byte slots of a 128-byte period)
template <int COLS, int ST>
__device__ __forceinline__ void tile_store_t(const TileStage<COLS>& r, bf16* dst, unsigned t, int salt) {
  using S = TileStage<COLS>;
#pragma unroll
  for (int j = 0; j < S::NU; ++j) {
    const int c0 = 8 * S::col(t, j);
    bf16* tp = dst + opaque(c0 * ST + kt_key(c0, S::key(t, j)), salt);
    const bf16x16 p01 = __builtin_shufflevector(r.v[j][0], r.v[j][1], 0, 8, 1, 9, 2, 10, 3, 11,
                                                4, 12, 5, 13, 6, 14, 7, 15);
    const bf16x16 p23 = __builtin_shufflevector(r.v[j][2], r.v[j][3], 0, 8, 1, 9, 2, 10, 3, 11,
                                                4, 12, 5, 13, 6, 14, 7, 15);
#define FM_CQ_ROW(e)                                                                      \
  *reinterpret_cast<bf16x4*>(tp + (e) * ST) =                                             \
      __builtin_shufflevector(p01, p23, 2 * (e), 2 * (e) + 1, 16 + 2 * (e), 17 + 2 * (e))
    FM_CQ_ROW(0); FM_CQ_ROW(1); FM_CQ_ROW(2); FM_CQ_ROW(3);
    FM_CQ_ROW(4); FM_CQ_ROW(5); FM_CQ_ROW(6); FM_CQ_ROW(7);
#undef FM_CQ_ROW
  }
}

constexpr int kKSteps = BK / 16;   // 16-key steps per tile
constexpr int kCqRA = 3;           // products whose LDS operands are read ahead

// A cached dS tile in registers (256 threads): unit u of thread t is
// u = t + 256 i (i < 4), i.e. (c2, m, g, rr) = u / 64 and, within it, hh =
// (u / 8) % 2 and key group j = u % 8: keys 32 g + 4 j .. +4, rows
// 64 c2 + 32 m + 8 rr + 4 hh + q (q = 0..3), 32 contiguous bytes of the
// cache (the 8-byte runs of 4 neighbouring lanes of one block).  (These
// loads touch half lines: the runs of a 4-key unit are contiguous in the
// order the dK/dV kernel stores them, and a lane loads at most 16 bytes.)
struct DsStage {
  static constexpr int NU = BQ * BK / 16 / kCqThreads;   // 4-row x 4-key units per thread
  bf16x8 v[NU][2];   // keys 4 j, 4 j + 1 | keys 4 j + 2, 4 j + 3 (4 rows each)
  static __device__ __forceinline__ int unit(unsigned t, int i) { return (int)t + kCqThreads * i; }
  // byte offset of the unit in the tile
  static __device__ __forceinline__ int offset(unsigned t, int i) {
    const int u = unit(t, i);
    return (u >> 4) * 512 + ((u >> 3) & 1) * 256 + (u & 7) * 32;
  }
  // first row and first key of the unit
  static __device__ __forceinline__ int row(unsigned t, int i) {
    const int u = unit(t, i), blk = u >> 4;
    return 64 * (blk >> 5) + 32 * ((blk >> 4) & 1) + 8 * (blk & 3) + 4 * ((u >> 3) & 1);
  }
  static __device__ __forceinline__ int key(unsigned t, int i) {
    const int u = unit(t, i), blk = u >> 4;
    return 32 * ((blk >> 2) & 3) + 4 * (u & 7);
  }
};

__device__ __forceinline__ void ds_load(DsStage& r, BufRsrc src, unsigned t, int salt) {
#pragma unroll
  for (int i = 0; i < DsStage::NU; ++i) {
    const uint32_t off = opaque((uint32_t)DsStage::offset(t, i), salt);
    r.v[i][0] = buf_load16(src, off);
    r.v[i][1] = buf_load16(src, off + 16u);
  }
}

// 4 keys x 4 rows -> 4 rows x 4 keys: row q of the unit gets element q of
// each key's 4-row run (8-byte LDS stores; the 16 lanes served together
// differ in key group and row half only, i.e. in 8-byte slots of a 128-byte
// bank period)
template <int ST>
__device__ __forceinline__ void ds_store_t(const DsStage& r, bf16* dst, unsigned t, int salt) {
#pragma unroll
  for (int i = 0; i < DsStage::NU; ++i) {
    bf16* tp = dst + opaque(DsStage::row(t, i) * ST + DsStage::key(t, i), salt);
    const bf16x8 a = r.v[i][0], b = r.v[i][1];   // a: key 0 rows 0-3, key 1 rows 0-3; b: keys 2, 3
#define FM_CQ_DS_ROW(q)                                                                   \
  *reinterpret_cast<bf16x4*>(tp + (q) * ST) = __builtin_shufflevector(a, b, (q), 4 + (q), 8 + (q), 12 + (q))
    FM_CQ_DS_ROW(0); FM_CQ_DS_ROW(1); FM_CQ_DS_ROW(2); FM_CQ_DS_ROW(3);
#undef FM_CQ_DS_ROW
  }
}

// one tile's K and dS in registers
template <int D>
struct TilePair {
  TileStage<D> k;
  DsStage ds;
};

}  // namespace

template <int D>
__global__ __launch_bounds__(kCqThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dq_cached_kernel(const BwdArgs a) {
  constexpr int ND = D / 32, ST = CqSmem<D>::ST;
  __shared__ CqSmem<D> sm;
  if (!tile_cache_on(a.counters, a.ds_cap)) return;

  const unsigned t = threadIdx.x;
  const int lane = (int)(t & 63), w = (int)(t >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nQ);
  // one workgroup per queue entry, or in pair mode two per entry (a pair of
  // query blocks; the second of a last block without a partner has nothing
  // to do).  With a shared mask the queue holds the H heads of a pair next
  // to each other; workgroups x .. x + 2H - 1 take their second blocks, then
  // their first blocks, so that workgroup x + H (and x) works on head x % H
  // as in the order of single query blocks: neighbouring workgroups go to
  // different dies, and each die then sees the blocks of a few heads in turn.
  uint32_t it;
  if (a.pairs) {
    const uint32_t nP = (uint32_t)(a.nQ + 1) >> 1;
    const uint32_t G = a.Hm == 1 ? (uint32_t)a.H : 1u;
    const uint32_t grp = blockIdx.x / (2 * G), r = blockIdx.x - grp * 2 * G;
    const uint32_t entry = grp * G + (r % G), second = r < G ? 1u : 0u;
    const uint32_t raw = min(*(const_u32*)(a.queue_q + entry), (uint32_t)((long)a.B * a.H * nP) - 1u);
    const uint32_t pbh = raw / nP, blk = 2 * (raw - pbh * nP) + second;
    if (blk >= (uint32_t)a.nQ) return;
    it = pbh * (uint32_t)a.nQ + blk;
  } else {
    it = min(*(const_u32*)(a.queue_q + blockIdx.x), max_items - 1);
  }
  const long bh = it / a.nQ;
  const int qb = (int)(it % a.nQ);
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const long bhm = (long)b * a.Hm + (a.Hm == 1 ? 0 : h);
  const int cnt = min(*(const_i32*)(a.cnt_q + bhm * a.nQ + qb), a.nK);
  const uint16_t* lst = a.list_q + (bhm * a.nQ + qb) * (long)a.nK;
  const int Sq = a.Sq, Sk = a.Sk;
  const BufRsrc kbase = make_rsrc(a.k + bh * Sk * (long)D, (uint32_t)Sk * D * 2u);

  f32x16 acc[ND];   // dQ^T: lane holds row li, head-dim 32 d + 8 r + 4 hh + q
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[d][v] = 0.f;

  for (int base = 0; base < cnt; base += kTab) {
    const int n = min(kTab, cnt - base);
    if (base > 0) __syncthreads();   // every wave is done with the previous table and tiles
    if ((int)t < n) {
      const int kb = min(lst[base + (int)t] & kListIndex, a.nK - 1);
      sm.slot[t] = a.colbase[bh * a.nK + kb] + a.cpos[(bhm * a.nK + kb) * (long)a.nQ + qb];
      sm.key0[t] = (uint32_t)(kb * BK);
    }
    __syncthreads();
    // tile i's K and dS (i >= n: empty ranges, so the loads return zeros
    // without a memory access and the wait counts stay the same on every path)
    auto ds_rsrc = [&](int i) __attribute__((always_inline)) {
      // (clamped into the cache, so that no slot can address memory outside it)
      const uint32_t s = min((uint32_t)__builtin_amdgcn_readfirstlane(sm.slot[min(i, n - 1)]), a.ds_cap - 1u);
      return make_rsrc(a.ds + (size_t)s * (BQ * BK), i < n ? (uint32_t)kTileBytes : 0u);
    };
    auto k_rsrc = [&](int i) __attribute__((always_inline)) { return i < n ? kbase : make_rsrc(nullptr, 0u); };
    auto k_first = [&](int i) __attribute__((always_inline)) {
      return (int)__builtin_amdgcn_readfirstlane(sm.key0[min(i, n - 1)]);
    };

    TilePair<D> pa, pb;
    auto load_tile = [&](TilePair<D>& x, int i) __attribute__((always_inline)) {
      tile_load<D>(x.k, k_rsrc(i), k_first(i), t, i);
      ds_load(x.ds, ds_rsrc(i), t, i);
    };
    load_tile(pa, 0);
    load_tile(pb, 1);

    // Tile i (its K and dS^T in x, loaded two tiles earlier): barrier | x ->
    // LDS, transposed | barrier | tile i + 2 -> x; dQ^T += K^T_i dS_i^T.
    auto step = [&](int i, TilePair<D>& x) __attribute__((always_inline)) {
      __syncthreads();   // every wave is done with tile i - 1 in LDS
      tile_store_t<D, ST>(x.k, sm.kt, t, i);
      ds_store_t<ST>(x.ds, sm.ds, t, i);
      __syncthreads();
      load_tile(x, i + 2);
      // product j is (k-step j / ND, head-dim block j % ND); its operands are
      // read from LDS kCqRA products ahead, in the order the fences keep
      const bf16* drow = sm.ds + (32 * w + li) * ST + 8 * hh;
      constexpr int NP = kKSteps * ND;
      bf16x8 av[NP], bv[kKSteps];
      // K^T operand of (kk, d): keys (16 kk + 8 hh) ^ 8 s = 16 kk ^ y[d] of
      // column 32 d + li, s its chunk's swizzle (kt_key); y[d] is rebuilt per
      // tile so that the 32 addresses are not all kept across the loop
      uint32_t y[ND];
#pragma unroll
      for (int d = 0; d < ND; ++d) y[d] = opaque((uint32_t)(8 * hh) ^ (uint32_t)(8 * ((4 * d + (li >> 3)) & 7)), i);
      const bf16* ktl = sm.kt + li * ST;
      auto read_ops = [&](int j) __attribute__((always_inline)) {
        const int kk = j / ND, d = j % ND;
        if (d == 0) bv[kk] = as_bf16x8(drow + 16 * kk);
        av[j] = as_bf16x8(ktl + 32 * d * ST + ((uint32_t)(16 * kk) ^ y[d]));
      };
#pragma unroll
      for (int j = 0; j < kCqRA; ++j) read_ops(j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        acc[j % ND] = mfma32(av[j], bv[j / ND], acc[j % ND]);
        if (j + kCqRA < NP) read_ops(j + kCqRA);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // (exits by break, so that every trip back to the top has issued the
    // same loads in the same order: the compiler then waits for each tile's
    // own loads only, not for the next tile's as well)
    for (int i = 0;; i += 2) {
      step(i, pa);
      if (i + 1 >= n) break;
      step(i + 1, pb);
      if (i + 2 >= n) break;
    }
    // the loads past the last tile were empty; wait for them before the
    // table is refilled
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }

  // ---- dQ, written once in bf16 ----
  const int qrow = qb * BQ + 32 * w + li;
  if (qrow < Sq) {
    bf16* drow = a.dq + (bh * Sq + qrow) * D;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 x;
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = (bf16)(acc[d][4 * r + q] * a.scale);
        *reinterpret_cast<bf16x4*>(&drow[32 * d + 8 * r + 4 * hh]) = x;
      }
  }
}

hipError_t launch_attn_bwd_dq_cached(const BwdArgs& a, int head_dim, hipStream_t stream) {
  const long items = (long)a.B * a.H * (a.pairs ? 2 * ((a.nQ + 1) / 2) : a.nQ);
  if (items <= 0 || a.ds_cap == 0) return hipSuccess;
  if (head_dim == 128)
    attn_bwd_dq_cached_kernel<128><<<(unsigned)items, kCqThreads, 0, stream>>>(a);
  else
    attn_bwd_dq_cached_kernel<64><<<(unsigned)items, kCqThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace fm
