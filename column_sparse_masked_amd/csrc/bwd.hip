// Backward of column-sparse masked attention (bf16 MFMA, fp32 accumulate):
// the key-stationary half.
//
//   bwd_pre_kernel   Delta_i = sum_d dO_id O_id (fp32);
//   attn_bwd_kernel  persistent, key-block stationary: each workgroup (8 waves)
//                    takes an item (batch*head, key block), keeps that block's
//                    K and V rows and its dK, dV accumulators in registers, and
//                    walks the list of query blocks that see the key block
//                    (the tiles the mask does not skip), 64 query rows at a
//                    time:
//                        S = Q K^T, P = exp(S - LSE) (interval mask on partial
//                        tiles only), dP = dO V^T, dS' = P (dP - Delta),
//                        dV += P^T dO, dK += dS'^T Q, and dK = scale dK at
//                        the end (dS = scale dS': the scale is applied once
//                        per output instead of once per score);
//   attn_bwd_dq_kernel (its own file) then computes dQ query-stationary.
// dQ is not accumulated here: fp32 atomic adds into a shared accumulator run
// at a fraction of the rate of plain stores on this GPU, and at this kernel's
// speed they, not the matrix cores, would set its pace.
// With S = Q K^T computed as C[i][j] a lane holds one key and several query
// rows, which is exactly the A-operand shape of P^T dO and dS^T Q.  Each chunk
// of Q and dO is therefore staged twice, row-major (A operands of S and dP)
// and transposed (B operands of dV and dK), so that every MFMA operand read
// from LDS is one 16-byte load.  The next chunk is fetched into registers
// while the current one computes.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace fm {

constexpr int QC = 64;   // query rows per backward chunk
constexpr int CPB = BQ / QC;   // chunks per query block

// ---------------------------------------------------------------- prologue
// Delta of every row; thread groups of D/8 threads per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o,
                                                      const bf16* __restrict__ dout,
                                                      float* __restrict__ delta, long rows) {
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
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (row < rows && c == 0) delta[row] = sum;
}

// ---------------------------------------------------------------- main
// Workgroup of 8 waves, two per SIMD.  Waves g and g+4 share key group g
// (32 keys of the block): for each 64-row chunk, wave (g, m) computes S and dP
// of the chunk's half m (rows 32 m .. +32) for its keys, then dV and dK of its
// keys for head-dim half m (columns D/2 m .. +D/2) over the whole chunk,
// taking the other half's P and dS from its partner through LDS.  Per wave
// that is 64 accumulator registers for dK/dV (instead of 128), which leaves
// room for two waves per SIMD.
// Step c has two phases split by barriers:
//   1. S, dP of chunk c; P, dS (to LDS for the partner); dV, dK over this
//      wave's own half of the chunk's rows (P, dS still in registers);
//   2. dV, dK over the partner's half (P, dS from LDS); the transposed and
//      row-major copies of chunk c+1 stored from registers; chunk c+3 loaded.
// The transposed copy is double-buffered so that phase 1 can read chunk c's
// while phase 2 writes chunk c+1's.  Of the two waves on a SIMD the older
// one reaches its exponentials first; the other's products then keep the
// matrix cores busy, and in turn the older wave's own-half products run
// while the other computes its exponentials.
constexpr int kBwdThreads = 512;

// Row terms start the accumulators.  With each chunk, -LSE / scale and
// -Delta of its rows are staged in LDS as fp32 (rterm); the S and dP
// accumulators of a wave start from them instead of from zero (a lane's 16
// rows are 4 runs of 4 consecutive rows: four 16-byte reads, the same for
// every lane of a row half), so the products yield S - LSE / scale and
// dP - Delta, and P = exp2(scale log2(e) S') and dS' = P dP' need no
// per-row value in the lanes, whose rows differ from lane to lane.
// The LDS of a workgroup is three separate arrays (row-major staging,
// transposed staging, P / dS exchange) rather than one structure, so that the
// compiler can tell apart accesses to different arrays and move the stores
// of one past the reads of another.  BwdSmem points into them.
template <int D>
struct BwdSmem {
  static constexpr int QST = D + 24;   // Q / dO row stride (elements): D values, then padding
  static constexpr int QTS = QC + 8;   // Q^T / dO^T row stride; rows in qt_pos order
  static constexpr int RM = QC * QST;  // elements of one row-major tile
  static constexpr int TR = D * QTS;   // elements of one transposed tile
  static_assert(stage_strides_ok(2 * QST, 2 * QTS), "strides the staging map needs");
  bf16* q;      // [QC * QST]
  bf16* dout;   // [QC * QST]
  bf16* tr;     // [2 buffers][Q^T, dO^T][D * QTS], one row per head-dim column
  // P and dS' of (key group g, half m) in the A-operand layout of the
  // dV / dK products: pds[g][m][0 = P, 1 = dS][t2][lane]
  bf16x8 (*pds)[2][2][2][64];
  float (*rterm)[QC];   // [0]: -LSE / scale (-inf: no P), [1]: -Delta of the chunk's rows
  __device__ __forceinline__ bf16* qt(int buf) const { return tr + (2 * buf) * TR; }
  __device__ __forceinline__ bf16* dot(int buf) const { return tr + (2 * buf + 1) * TR; }
};

// Place of row x (0 <= x < QC) inside a Q^T / dO^T row: bits 2 and 3 of the
// offset within each group of 16 swapped, so that the 8 query rows one lane
// holds in the P^T (dS^T) operand are 8 neighbouring elements.
__device__ __forceinline__ int qt_pos(int x) { return (x & ~15) | perm16(x & 15); }

// Global -> register staging of one chunk of QC query rows of Q and dO
// (512 threads).  A unit is 4 consecutive rows (4m .. 4m+3) x 8 head-dim
// columns (chunk c) of one of the two tensors, assigned by the staging map
// (stage_row_unit, stage_chunk) that keeps both the row-major and the
// transposed LDS stores free of bank conflicts.  Threads < 2*QC also carry
// the LSE (first QC) or Delta (next QC) of one row.
template <int D>
struct ChunkStage {
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int NPAIR = (QC / 4) * CPR;   // units per tensor (a multiple of 64)
  static_assert(NPAIR % 64 == 0 && 2 * NPAIR <= kBwdThreads, "one unit per thread");
  static_assert(CPR % 4 == 0 && QC == 64, "a wave's units are the 16 row-units x 4 chunks");
  bf16x8 v[4];
  float row_term;

  // (constant true when every thread has a unit, so that no branch surrounds
  // the loads and stores)
  static __device__ __forceinline__ bool active(unsigned t) {
    return 2 * NPAIR == kBwdThreads || t < 2u * NPAIR;
  }
  // 0 = Q, 1 = dO; the same in every lane of a wave (NPAIR is a multiple of 64)
  static __device__ __forceinline__ int tensor(unsigned t) {
    return __builtin_amdgcn_readfirstlane((int)(t / NPAIR));
  }
  // unit p of the tensor: lane p % 64 of chunk quad p / 64
  static __device__ __forceinline__ int row(unsigned t) {
    return 4 * stage_row_unit((int)(t % NPAIR) & 63);
  }
  static __device__ __forceinline__ int col(unsigned t) {
    const int p = (int)(t % NPAIR);
    return stage_chunk(p & 63, p >> 6);
  }
};

template <int D>
__device__ __forceinline__ void load_chunk(ChunkStage<D>& r, BufRsrc qb, BufRsrc ob, BufRsrc lb,
                                           BufRsrc db, int q0, unsigned t) {
  using C = ChunkStage<D>;
  // The row term first (the oldest load of the chunk).  Wave 0 carries LSE,
  // wave 1 Delta (QC is the wave size); rows past the end read 0 (buffer
  // range check) and are fixed on store.  The other waves issue the load too,
  // through an empty range (zeros, no memory access): with the same loads in
  // every wave and no branch around them, the compiler counts the loads in
  // flight exactly and waits for a chunk without waiting for the next one.
  static_assert(QC == 64, "one wave per row term");
  {
    const int wv = __builtin_amdgcn_readfirstlane((int)(t / QC));
    const BufRsrc src = wv == 0 ? lb : wv == 1 ? db : make_rsrc(nullptr, 0u);
    r.row_term = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(src, (q0 + (int)(t % QC)) * 4, 0, 0));
  }
  if (C::active(t)) {
    const BufRsrc src = C::tensor(t) == 0 ? qb : ob;
    const uint32_t base =
        opaque(((uint32_t)C::row(t) * C::CPR + C::col(t)) * 16u, q0) + (uint32_t)q0 * (D * 2);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) r.v[rr] = buf_load16(src, base + (uint32_t)rr * (D * 2));
  }
}

// Row-major Q and dO (A operands of S and dP) and the row terms.
template <int D, typename Smem>
__device__ __forceinline__ void store_rowmajor(const ChunkStage<D>& r, const Smem& sm, int q0, int Sq,
                                               float inv_scale, unsigned t) {
  using C = ChunkStage<D>;
  constexpr int QST = Smem::QST;
  if (C::active(t)) {
    bf16* rm = (C::tensor(t) == 0 ? sm.q : sm.dout) + opaque(C::row(t) * QST + 8 * C::col(t), q0);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) *reinterpret_cast<bf16x8*>(rm + rr * QST) = r.v[rr];
  }
  // row terms: -LSE / scale (-inf for rows past the end and rows no key
  // sees, so P = 0 there) and -Delta
  if (t < 2 * QC) {
    const bool is_q = t < QC;
    const int row = (int)t % QC;
    float x;
    if (is_q) {
      const bool live = q0 + row < Sq && r.row_term < INFINITY;
      x = live ? -r.row_term * inv_scale : -INFINITY;
    } else {
      x = -r.row_term;
    }
    sm.rterm[is_q ? 0 : 1][row] = x;
  }
}

// Transposed Q and dO (B operands of dK and dV) into buffer `buf`, one row of
// 4 elements at a time so that the stores can be spread between other work.
// The thread's unit covers rows 8 c + e (e = 0..7) of the transposed tile, c
// its column chunk.  salt: a scalar that changes from chunk to chunk (keeps
// the lane addresses inside the loop).
template <int D, typename Smem>
struct TransposedStore {
  using C = ChunkStage<D>;
  bf16* tp;
  bf16x16 p01, p23;   // rows 0,1 and 2,3 of the unit, interleaved element by element

  __device__ __forceinline__ TransposedStore(const ChunkStage<D>& r, const Smem& sm, int buf, int salt,
                                             unsigned t) {
    const int c = C::col(t);
    tp = (C::tensor(t) == 0 ? sm.qt(buf) : sm.dot(buf)) + opaque((8 * c) * Smem::QTS + qt_pos(C::row(t)), salt);
    p01 = __builtin_shufflevector(r.v[0], r.v[1], 0, 8, 1, 9, 2, 10, 3, 11, 4, 12, 5, 13, 6, 14, 7, 15);
    p23 = __builtin_shufflevector(r.v[2], r.v[3], 0, 8, 1, 9, 2, 10, 3, 11, 4, 12, 5, 13, 6, 14, 7, 15);
  }
  // transposed row 8 c + e (e a constant after unrolling)
  __device__ __forceinline__ void row(int e) const {
    bf16x4 x;
    x[0] = p01[2 * e];
    x[1] = p01[2 * e + 1];
    x[2] = p23[2 * e];
    x[3] = p23[2 * e + 1];
    *reinterpret_cast<bf16x4*>(tp + e * Smem::QTS) = x;
  }
};

template <int D, typename Smem>
__device__ __forceinline__ void store_transposed(const ChunkStage<D>& r, const Smem& sm, int buf, int salt,
                                                 unsigned t) {
  if (!ChunkStage<D>::active(t)) return;
  const TransposedStore<D, Smem> ts(r, sm, buf, salt, t);
#pragma unroll
  for (int e = 0; e < 8; ++e) ts.row(e);
}

// One key-stationary work item (batch*head, key block): what the kernel needs
// of it in scalar registers.
struct BwdItem {
  uint32_t idx;           // queue position (>= the item count: no item)
  int kb, k0, cnt, rot, nchunks;
  long bh, bhm;
  const uint16_t* lst;    // the key block's list of non-skipped query blocks
  BufRsrc qbase, obase, kbase, vbase, lbase, dbase;
  BufRsrc dsrc;           // the item's tiles in the tile cache (empty when it is off)

  // List word of chunk c (clamped to the last chunk: entries past the end
  // are loaded but not used).  Each item starts its walk at block kb % cnt
  // (and wraps): neighbouring key blocks, which run at the same time, then
  // read different query blocks.
  __device__ __forceinline__ ListWord lword(int c) const {
    const int j = min(c, nchunks - 1) / CPB + rot;
    return list_word(lst, j < cnt ? j : j - cnt);
  }
};

template <int D>
__device__ __forceinline__ BwdItem bwd_item(const BwdArgs& a, const uint32_t (&hdr)[4], bool cache) {
  // values read from LDS are not known to be uniform: broadcast them, so that
  // the buffer resources built from them stay in scalar registers
  BwdItem x;
  x.idx = __builtin_amdgcn_readfirstlane(hdr[0]);
  const uint32_t it = __builtin_amdgcn_readfirstlane(hdr[1]);
  x.cnt = __builtin_amdgcn_readfirstlane((int)hdr[2]);
  x.nchunks = CPB * x.cnt;   // each query block is CPB chunks of QC rows
  x.bh = it / a.nK;
  x.kb = (int)(it % a.nK);
  x.k0 = x.kb * BK;
  x.rot = x.cnt > 0 ? x.kb % x.cnt : 0;
  const int b = (int)(x.bh / a.H), h = (int)(x.bh % a.H);
  x.bhm = (long)b * a.Hm + (a.Hm == 1 ? 0 : h);
  x.lst = a.list_k + (x.bhm * a.nK + x.kb) * (long)a.nQ;
  const int Sq = a.Sq, Sk = a.Sk;
  x.qbase = make_rsrc(a.q + x.bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
  x.obase = make_rsrc(a.dout + x.bh * Sq * (long)D, (uint32_t)Sq * D * 2u);
  x.kbase = make_rsrc(a.k + x.bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
  x.vbase = make_rsrc(a.v + x.bh * Sk * (long)D, (uint32_t)Sk * D * 2u);
  x.lbase = make_rsrc(a.lse + x.bh * Sq, (uint32_t)Sq * 4u);
  x.dbase = make_rsrc(a.delta + x.bh * Sq, (uint32_t)Sq * 4u);
  // the item's tiles take consecutive slots from colbase[it], in list order;
  // with the cache off the range is empty and the stores are dropped
  // (`it` is already clamped to a valid item; an item whose slots would run
  // past the cache gets an empty range, so no store can leave the cache)
  const uint32_t cb = cache ? *(const_u32*)(a.colbase + it) : 0u;
  const bool fits = cache && (uint64_t)cb + (uint32_t)x.cnt <= a.ds_cap;
  x.dsrc = make_rsrc(a.ds + (fits ? (size_t)cb * (BQ * BK) : 0), fits ? (uint32_t)x.cnt * kTileBytes : 0u);
  return x;
}

// Cache policy of the tile-cache stores: non-temporal (the tiles are read
// back only by the next kernel, so they should not displace the Q and dO
// rows this kernel reuses from the caches; measured 1.5% faster on the
// kernel at the 128K workload, where the cache is 21 GiB).
constexpr int kStoreNonTemporal = 2;

// This wave's dS' = dS / scale of one chunk into the item's tile of the cache.  A
// tile is stored as the waves hold it: for chunk c2 (two per tile), wave
// (g, m) and register pair rr, a block of 512 bytes in which lane l (key
// 32 g + l % 32) has 8 bytes, rows 32 m + 8 rr + 4 (l / 32) + q (q = 0..3)
// of the chunk.  Block (c2, m, g, rr) is at ((c2 * 2 + m) * 4 + g) * 4 + rr
// times 512 bytes, so every store instruction writes 512 contiguous bytes
// (whole cache lines) straight from the packed registers.  `soff` is the byte
// offset of the chunk's blocks in the item's tiles.
__device__ __forceinline__ void store_ds_tile(BufRsrc r, const bf16x8 (&dsb)[2], int g, int m, int soff,
                                              int salt) {
  const int ln = lane_in(salt);
  const uint32_t lane_off = (uint32_t)(((m * 4 + g) * 4) * 512 + 8 * ln);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const i32x4 wv = __builtin_bit_cast(i32x4, dsb[rr >> 1]);
    u32x2 x;
    x[0] = (unsigned)((rr & 1) ? wv[2] : wv[0]);
    x[1] = (unsigned)((rr & 1) ? wv[3] : wv[1]);
    __builtin_amdgcn_raw_buffer_store_b64(x, r, (int)(lane_off + 512 * rr), soff, kStoreNonTemporal);
  }
}

template <int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_bwd_kernel(const BwdArgs a) {
  constexpr int NS = D / 16;        // k-steps over the head dimension
  constexpr int NDH = D / 64;       // 32-wide head-dim blocks per half of D
  using Smem = BwdSmem<D>;
  constexpr int QST = Smem::QST, QTS = Smem::QTS;
  __shared__ __attribute__((aligned(16))) bf16 lds_rm[2 * Smem::RM];
  __shared__ __attribute__((aligned(16))) bf16 lds_t[4 * Smem::TR];
  __shared__ bf16x8 lds_pds[4][2][2][2][64];
  __shared__ __attribute__((aligned(16))) float lds_rterm[2][QC];
  __shared__ uint32_t lds_hdr[2][4];   // headers of this and the next item
  Smem sm;
  sm.q = lds_rm;
  sm.dout = lds_rm + Smem::RM;
  sm.tr = lds_t;
  sm.pds = lds_pds;
  sm.rterm = lds_rterm;

  const unsigned t = threadIdx.x;
  const int lane = (int)(t & 63), w = (int)(t >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const int g = w & 3, m = w >> 2;   // key group; chunk half (S, dP) and head-dim half (dK, dV)
  const uint32_t max_items = (uint32_t)((long)a.B * a.H * a.nK);
  const uint32_t n_items = min(a.counters[kCtrBwdItems], max_items);
  // row stride (elements) of the dK / dV tile staged in LDS for the stores
  constexpr int EST = D + 8;
  static_assert(2 * BK * EST <= 4 * Smem::TR, "the dK / dV tile fits the transposed staging buffers");
  const int Sq = a.Sq, Sk = a.Sk;
  const float inv_scale = 1.0f / a.scale;

  const ItemQueue iq{&a.counters[kCtrBwdNext], a.queue, a.cnt_k, n_items, max_items, a.nK, a.H, a.Hm, a.nQ};
  const bool cache = tile_cache_on(a.counters, a.ds_cap);
  if (t == 0) iq.first(lds_hdr[0]);
  __syncthreads();
  // first row of chunk c of a query block with list entry e
  auto row0 = [&](int e, int c) __attribute__((always_inline)) {
    return min(e & kListIndex, a.nQ - 1) * BQ + (c % CPB) * QC;
  };

  // An item's loads that do not wait for its LDS (the lane's key bounds, K
  // and V rows as MFMA B operands, the first list words and the first chunk
  // of Q and dO) are issued before the previous item's dK and dV are written,
  // so that they are in flight during those stores.
  ItemPrefetch pf;
  i32x4 bd;        // the lane's key bounds (LTS, LTE, UTS, UTE)
  bool key_live;   // the lane's key is < Sk
  bf16x8 kf[NS], vf[NS];
  ListWord lw0, lw1, lw2, lw3;
  ChunkStage<D> r0, r1;
  auto preload = [&](const BwdItem& x) __attribute__((always_inline)) {
    // (a branch-free load: keys past the end read zeros here and are masked
    // for every row where the bounds are used)
    const int jrow = x.k0 + 32 * g + li;
    bd = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(a.bounds + x.bhm * Sk, (uint32_t)Sk * 16u),
                                               jrow * 16, 0, 0);
    key_live = jrow < Sk;
    const uint32_t off = ((uint32_t)jrow * D + 8u * hh) * 2u;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = buf_load16(x.kbase, off + 32u * s);
      vf[s] = buf_load16(x.vbase, off + 32u * s);
    }
    int bq0 = Sq;   // no chunk: rows at Sq read as zeros without memory accesses
    if (x.nchunks > 0) {
      lw0 = x.lword(0);
      lw1 = x.lword(1);
      lw2 = x.lword(2);
      lw3 = x.lword(3);
      bq0 = row0(list_value(lw0), 0);
    }
    load_chunk<D>(r0, x.qbase, x.obase, x.lbase, x.dbase, bq0, t);
  };
  BwdItem cur = bwd_item<D>(a, lds_hdr[0], cache);
  if (cur.idx < n_items) {
    pf.take(iq, t);   // the ticket of the next item, before the item's loads
    preload(cur);
  }

  for (int n = 0;; ++n) {
    if (cur.idx >= n_items) break;
    // the step code below reads the item through these names
    const int cnt = cur.cnt, nchunks = cur.nchunks, kb = cur.kb, k0 = cur.k0;
    const bool ragged_k = k0 + BK > Sk;
    const BufRsrc qbase = cur.qbase, obase = cur.obase, lbase = cur.lbase, dbase = cur.dbase;
    (void)kb;
    auto lword = [&](int c) __attribute__((always_inline)) { return cur.lword(c); };

    // dK^T, dV^T: lane holds key 32 g + li, columns D/2 m + 32 dd + 8 r + 4 hh + q
    f32x16 dk[NDH], dv[NDH];
#pragma unroll
    for (int dd = 0; dd < NDH; ++dd)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        dk[dd][v] = 0.f;
        dv[dd][v] = 0.f;
      }

    if (nchunks > 0) {
      // B operand of the dV (tensor 0) / dK (tensor 1) product of rows of
      // half hf, head-dim block dd, k-half t2, from transposed buffer buf
      auto boff = [&](int hf, int dd, int t2) __attribute__((always_inline)) {
        return (D / 2 * m + 32 * dd + li) * QTS + 32 * hf + 16 * t2 + 8 * hh;
      };
      const int mo = 1 - m;   // the partner's half

      // X: registers holding chunk c+1 (loaded two steps earlier)
      auto step = [&](int c, ChunkStage<D>& X) __attribute__((always_inline)) {
        asm volatile("" ::"s"(lw0.word), "s"(lw1.word), "s"(lw2.word), "s"(lw3.word));
        const int e0 = list_value(lw0);
        const int q0 = row0(e0, c);
        const bool need_mask = (e0 & kListPartial) || ragged_k;
        const int q0n = row0(list_value(lw1), c + 1);
        // past the last chunk: rows at Sq, which the loads' range check
        // turns into zeros without memory accesses
        const int q0l = c + 3 < nchunks ? row0(list_value(lw3), c + 3) : Sq;
        lw0 = lw1;
        lw1 = lw2;
        lw2 = lw3;
        const int bc = c & 1, bn = bc ^ 1;   // transposed buffers of chunks c and c+1
        const bf16* qtc = sm.qt(bc);
        const bf16* dotc = sm.dot(bc);

        // ---- phase 1: S, dP of rows 32 m + 8 r + 4 hh + q (element 4r+q),
        // key li, starting from the rows' terms ----
        f32x16 s, dp;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 ls = *reinterpret_cast<const float4*>(&sm.rterm[0][32 * m + 8 * r4 + 4 * hh]);
          const float4 ld = *reinterpret_cast<const float4*>(&sm.rterm[1][32 * m + 8 * r4 + 4 * hh]);
          s[4 * r4] = ls.x;
          s[4 * r4 + 1] = ls.y;
          s[4 * r4 + 2] = ls.z;
          s[4 * r4 + 3] = ls.w;
          dp[4 * r4] = ld.x;
          dp[4 * r4 + 1] = ld.y;
          dp[4 * r4 + 2] = ld.z;
          dp[4 * r4 + 3] = ld.w;
        }
        const bf16* qrow = sm.q + (32 * m + li) * QST + 8 * hh;
        const bf16* drow = sm.dout + (32 * m + li) * QST + 8 * hh;
        if constexpr (D == 128) {
          // operands read two k-steps ahead; the fences keep that order
          bf16x8 qa[NS], da[NS];
          auto read_ops = [&](int i) __attribute__((always_inline)) {
            qa[i] = as_bf16x8(qrow + 16 * i);
            da[i] = as_bf16x8(drow + 16 * i);
          };
          read_ops(0);
          read_ops(1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            s = mfma32(qa[i], kf[i], s);
            dp = mfma32(da[i], vf[i], dp);
            if (i + 2 < NS) read_ops(i + 2);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < NS; ++kk) {
            s = mfma32(as_bf16x8(qrow + 16 * kk), kf[kk], s);
            dp = mfma32(as_bf16x8(drow + 16 * kk), vf[kk], dp);
          }
        }
        if (need_mask) {
          // bit 8r + q: the lane's key hides row 32 m + 8 r + 4 hh + q
          const int base = q0 + 32 * m;
          auto clip = [&](int x) { return min(max(x, base), base + 32) - base; };
          auto rows = [](int lo, int hi) {
            return hi > lo ? (~0u >> (32 - hi)) & (~0u << lo) : 0u;
          };
          const uint32_t hidden =
              key_live ? (rows(clip(bd[0]), clip(bd[1])) | rows(clip(bd[2]), clip(bd[3]))) >> (4 * hh)
                       : ~0u;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s[v] = (hidden >> (8 * (v >> 2) + (v & 3))) & 1u ? -INFINITY : s[v];
        }
        // P = exp2(S' scale log2(e)); dS' = P dP' (dS / scale), 8 values (one
        // k-step of the dV / dK products) at a time
        bf16x8 pb[2], dsb[2];
        auto make_half = [&](int t2) __attribute__((always_inline)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = fast_exp2(s[8 * t2 + e] * a.scale_log2);
            pb[t2][e] = (bf16)p;
            dsb[t2][e] = (bf16)(p * dp[8 * t2 + e]);
          }
        };
        auto cache_and_exchange = [&]() __attribute__((always_inline)) {
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            sm.pds[g][m][0][t2][lane] = pb[t2];
            sm.pds[g][m][1][t2][lane] = dsb[t2];
          }
          // the chunk's dS' into the tile cache: tile j of the item is
          // its j-th list entry (the walk starts at entry rot)
          int j = c / CPB + cur.rot;
          j = j < cnt ? j : j - cnt;
          store_ds_tile(cur.dsrc, dsb, g, m, j * kTileBytes + (c % CPB) * (kTileBytes / CPB), c);
        };
        // ---- dV += P^T dO, dK += dS^T Q, head-dim half m, own rows ----
        constexpr int NP = NDH * 2;   // product pairs per half: (dd, t2)
        if constexpr (D == 128) {
          // the first k-step's products run beside the second k-step's
          // exponentials: pair i is (dd, t2) = (i % 2, i / 2)
          make_half(0);
          bf16x8 bo[NP][2];
          auto read_b = [&](int i) __attribute__((always_inline)) {
            const int off = boff(m, i & 1, i >> 1);
            bo[i][0] = as_bf16x8(dotc + off);
            bo[i][1] = as_bf16x8(qtc + off);
          };
          read_b(0);
          read_b(1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            dv[i & 1] = mfma32(bo[i][0], pb[0], dv[i & 1]);
            dk[i & 1] = mfma32(bo[i][1], dsb[0], dk[i & 1]);
            read_b(i + 2);
          }
          make_half(1);
          __builtin_amdgcn_sched_barrier(0);
          cache_and_exchange();
#pragma unroll
          for (int i = 2; i < NP; ++i) {
            dv[i & 1] = mfma32(bo[i][0], pb[1], dv[i & 1]);
            dk[i & 1] = mfma32(bo[i][1], dsb[1], dk[i & 1]);
          }
        } else {
          make_half(0);
          make_half(1);
          cache_and_exchange();
#pragma unroll
          for (int dd = 0; dd < NDH; ++dd)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const int off = boff(m, dd, t2);
              dv[dd] = mfma32(as_bf16x8(dotc + off), pb[t2], dv[dd]);
              dk[dd] = mfma32(as_bf16x8(qtc + off), dsb[t2], dk[dd]);
            }
        }
        __syncthreads();   // P, dS in LDS; row-major c read

        // ---- phase 2: dV, dK over the partner's rows; chunk c+1 staged
        // (past the last chunk the stores write unused rows: harmless);
        // chunk c+3 loaded into the registers the stores have read ----
        bf16x8 ph[2], dh[2];
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          ph[t2] = sm.pds[g][mo][0][t2][lane];
          dh[t2] = sm.pds[g][mo][1][t2][lane];
        }
        if constexpr (D == 128) {
          const TransposedStore<D, Smem> ts(X, sm, bn, q0n, t);
          bf16x8 bo[NP][2];
          auto read_b = [&](int i) __attribute__((always_inline)) {
            const int off = boff(mo, i >> 1, i & 1);
            bo[i][0] = as_bf16x8(dotc + off);
            bo[i][1] = as_bf16x8(qtc + off);
          };
          read_b(0);
          read_b(1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            dv[i >> 1] = mfma32(bo[i][0], ph[i & 1], dv[i >> 1]);
            dk[i >> 1] = mfma32(bo[i][1], dh[i & 1], dk[i >> 1]);
            if (i + 2 < NP) read_b(i + 2);
            ts.row(2 * i);
            ts.row(2 * i + 1);
            if (i == 1) store_rowmajor<D>(X, sm, q0n, Sq, inv_scale, t);
            if (i == NP - 1) {
              load_chunk<D>(X, qbase, obase, lbase, dbase, q0l, t);
              lw3 = lword(c + 4);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int dd = 0; dd < NDH; ++dd)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
              const int off = boff(mo, dd, t2);
              dv[dd] = mfma32(as_bf16x8(dotc + off), ph[t2], dv[dd]);
              dk[dd] = mfma32(as_bf16x8(qtc + off), dh[t2], dk[dd]);
            }
          store_transposed<D>(X, sm, bn, q0n, t);
          store_rowmajor<D>(X, sm, q0n, Sq, inv_scale, t);
          load_chunk<D>(X, qbase, obase, lbase, dbase, q0l, t);
          lw3 = lword(c + 4);
        }
        // the next item's header, one scalar load in each of the first two steps
        if (c == 0) pf.fetch_entry(iq, lds_hdr[(n + 1) & 1]);
        if (c == 1) pf.fetch_count(iq);
        __syncthreads();   // chunk c+1 in LDS; transposed c and P, dS read
      };

      // chunk 0 (in r0) staged; chunk 1 -> r1, chunk 2 -> r0
      const int bq0 = row0(list_value(lw0), 0);
      store_transposed<D>(r0, sm, 0, bq0, t);
      store_rowmajor<D>(r0, sm, bq0, Sq, inv_scale, t);
      // K, V are in registers by now (loaded before chunk 0, which the stores
      // waited for); an explicit wait says so to the compiler, which would
      // otherwise wait for them, and with them for the loads of later chunks,
      // inside every step
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      pf.stash(lds_hdr[(n + 1) & 1], t);
      load_chunk<D>(r1, qbase, obase, lbase, dbase, nchunks > 1 ? row0(list_value(lw1), 1) : Sq, t);
      load_chunk<D>(r0, qbase, obase, lbase, dbase, nchunks > 2 ? row0(list_value(lw2), 2) : Sq, t);
      __syncthreads();
      // two chunks per trip (nchunks is even), so that the register sets stay
      // statically named
      static_assert(CPB % 2 == 0, "an even number of chunks per item");
      for (int c = 0; c < nchunks; c += 2) {
        step(c, r1);
        step(c + 1, r0);
      }
      pf.publish(iq, lds_hdr[(n + 1) & 1], t);
    } else {
      pf.finish_now(iq, lds_hdr[(n + 1) & 1], t);
    }
    // ---- dK and dV of this item, then the next item's first loads ----
    // The accumulators go to LDS as bf16 rows of dK and dV (one 8-byte store
    // per 4 columns), so that the global stores are 16 bytes of a row per
    // lane; the transposed staging buffers are free once the last step has
    // passed its barrier.
    {
      bf16* const tile = lds_t;   // [2 tensors][BK keys][EST]
      const int krow = 32 * g + li;
#pragma unroll
      for (int dd = 0; dd < NDH; ++dd)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int col = D / 2 * m + 32 * dd + 8 * r + 4 * hh;
          bf16x4 xk, xv;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            xk[q] = (bf16)(dk[dd][4 * r + q] * a.scale);
            xv[q] = (bf16)dv[dd][4 * r + q];
          }
          *reinterpret_cast<bf16x4*>(&tile[krow * EST + col]) = xk;
          *reinterpret_cast<bf16x4*>(&tile[(BK + krow) * EST + col]) = xv;
        }
    }
    __syncthreads();   // the tile and the next item's header are in LDS
    const BwdItem nxt = bwd_item<D>(a, lds_hdr[(n + 1) & 1], cache);
    {
      // rows past the end of the keys fall outside the buffer range: the
      // stores are dropped
      const uint32_t bytes = (uint32_t)Sk * D * 2u;
      const BufRsrc kout = make_rsrc(a.dk + cur.bh * Sk * (long)D, bytes);
      const BufRsrc vout = make_rsrc(a.dv + cur.bh * Sk * (long)D, bytes);
      constexpr int CPR = D / 8;                  // 16-byte chunks per row
      constexpr int PER = BK * CPR / kBwdThreads; // chunks per thread and tensor
      static_assert(BK * CPR % kBwdThreads == 0, "whole chunks per thread");
#pragma unroll
      for (int tensor = 0; tensor < 2; ++tensor)
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int i = (int)t + kBwdThreads * j;
          const int row = i / CPR, ch = i % CPR;
          const bf16x8 x = as_bf16x8(&lds_t[(tensor * BK + row) * EST + 8 * ch]);
          const uint32_t off = ((uint32_t)(k0 + row) * D + 8u * ch) * 2u;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), tensor == 0 ? kout : vout,
                                                 (int)off, 0, 0);
        }
    }
    if (nxt.idx < n_items) {
      pf.take(iq, t);
      preload(nxt);
    }
    __syncthreads();   // every wave has read the tile: the staging buffers are free
    cur = nxt;
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

int bwd_blocks_per_cu(int) { return 1; }

hipError_t launch_attn_bwd(const BwdArgs& a, int head_dim, int grid, int dq_grid,
                           hipStream_t stream, const KernelEvents& ev) {
  const long rows = (long)a.B * a.H * a.Sq;
  hipError_t err;
  if (rows > 0) {
    const unsigned pre_grid = (unsigned)((rows * head_dim / 8 + 255) / 256);
    if (head_dim == 128)
      bwd_pre_kernel<128><<<pre_grid, 256, 0, stream>>>(a.o, a.dout, a.delta, rows);
    else
      bwd_pre_kernel<64><<<pre_grid, 256, 0, stream>>>(a.o, a.dout, a.delta, rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (ev.begin && (err = hipEventRecord(ev.begin, stream)) != hipSuccess) return err;
  if (grid > 0) {
    if (head_dim == 128)
      attn_bwd_kernel<128><<<grid, kBwdThreads, 0, stream>>>(a);
    else
      attn_bwd_kernel<64><<<grid, kBwdThreads, 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (ev.end && (err = hipEventRecord(ev.end, stream)) != hipSuccess) return err;
  if (ev.begin2 && (err = hipEventRecord(ev.begin2, stream)) != hipSuccess) return err;
  // dQ: from the tile cache when it is on, else recomputed; each of the two
  // kernels reads the tile count and leaves at once when it is not the one
  // (the cached kernel is launched only when the workspace holds a cache)
  if ((err = launch_attn_bwd_dq_cached(a, head_dim, stream)) != hipSuccess) return err;
  if ((err = launch_attn_bwd_dq(a, head_dim, dq_grid, stream)) != hipSuccess) return err;
  if (ev.end2 && (err = hipEventRecord(ev.end2, stream)) != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace fm
