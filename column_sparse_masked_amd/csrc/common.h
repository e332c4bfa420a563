// Device-side definitions shared by the libfm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <climits>
#include <stdint.h>

namespace fm {

// Tile shape: BQ query rows x BK key columns.  The forward gives each of the 4
// waves of a workgroup 32 query rows; the backward gives each wave 32 keys.
constexpr int BQ = 128;
constexpr int BK = 128;
constexpr int kListPartial = 0x8000;   // bit 15 of a list entry: tile is partial
constexpr int kListIndex = 0x7fff;

// counters[] slots inside the tileinfo buffer
constexpr int kCtrFwdItems = 0, kCtrBwdItems = 1, kCtrFwdNext = 2, kCtrBwdNext = 3,
              kCtrFwdExit = 4, kCtrBwdExit = 5, kCtrDqNext = 6, kCtrDqExit = 7,
              kCtrFwdSplit = 8,   // forward items split in two (the first of the queue)
              kCtrTiles = 9,      // non-skipped tiles over all (batch, head) pairs (saturating)
              kCtrRowDone = 10,   // tile pass: row-kernel workgroups finished
              kCtrFwdPairs = 11;  // 1 when forward items are pairs of query blocks

// Union-list entries of a query-block pair (pair mode): the key block, and
// for each of the two query blocks whether it sees the block and whether
// that tile is partial.
constexpr uint32_t kPairBlock = 0xFFFFu, kPairSee0 = 1u << 16, kPairPart0 = 1u << 17,
                   kPairSee1 = 1u << 18, kPairPart1 = 1u << 19;

// Bytes of one cached tile of dS / scale (bf16, BQ rows of BK keys).
constexpr int kTileBytes = BQ * BK * 2;

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// s_waitcnt operand that waits for every vector memory load of the wave and
// for nothing else (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15)
constexpr int kWaitVmcnt0 = 0x0F70;

// D = A(32x16) * B(16x32) + C on the matrix cores.  Lane l supplies
//   A[l%32][8*(l/32) .. +8]   and   B[8*(l/32) .. +8][l%32],
// and holds C[8*(v/4) + 4*(l/32) + v%4][l%32] in element v of the result.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of key (or query) offset x inside a 16-wide group when a transposed
// operand is staged in LDS: swap bits 2 and 3.  A 32x32 accumulator lane holds
// offsets {8a + 4h + q}; after the swap those 8 offsets are contiguous, so the
// accumulator can be fed back as an MFMA operand without moving data between
// lanes, and the matching operand is one 16-byte LDS read.
__device__ __forceinline__ int perm16(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Staging map of a tile of rows x 16-byte column chunks that is stored in LDS
// both row-major (one 16-byte store per row of a unit) and transposed (one
// 8-byte store of a unit's 4 rows per column).  A unit is 4 rows x 1 chunk;
// the 64 lanes of a wave take 16 row-units by the 4 chunks of chunk quad q:
//     row-unit  l % 16,     chunk  4 q + ((l % 16) / 2 + l / 16) % 4.
// This GPU's LDS serves 8-byte accesses 16 lanes at a time and 16-byte stores
// 8 lanes at a time; two of those lanes conflict when they touch the same
// bank at different addresses, banks repeating every 128 bytes.
//   transposed stores: the 16 lanes have 16 distinct row-units, i.e. 16
//     distinct 8-byte places within a transposed row; with 8 transposed rows
//     a multiple of 128 bytes long, the lanes' rows (8 apart) start on the
//     same bank, so the places do not collide;
//   row-major stores: the 8 lanes have row-units of both parities and all 4
//     chunks, one lane per (parity, chunk); with 4 rows = 64 (mod 128) bytes
//     that is 8 distinct 16-byte places.
// (A permutation of rows instead of this map would also spread the
// transposed stores, but 16-byte reads are served 16 lanes at a time at full
// rate only when address bits 4-5 follow lane bits 0-1, which permuted rows
// break for the operand reads of the transposed tile.)
__device__ __forceinline__ int stage_row_unit(int lane) { return lane & 15; }
__device__ __forceinline__ int stage_chunk(int lane, int quad) {
  return 4 * quad + ((((lane & 15) >> 1) + (lane >> 4)) & 3);
}
// Byte strides that the map needs: 4 row-major rows = 64 (mod 128), 8
// transposed rows = 0 (mod 128).
constexpr bool stage_strides_ok(int row_bytes, int trow_bytes) {
  return (4 * row_bytes) % 128 == 64 && (8 * trow_bytes) % 128 == 0;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
  return z;
}

}  // namespace fm

namespace fm {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t BufRsrc;

// Buffer resource over [base, base + bytes): raw 16-byte loads through it
// return zeros at offsets at or past `bytes` (the hardware range check), which
// zero-fills ragged tiles without branches.  bytes < 2^31.
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// -inf where bit `bit` of `word` is set, else x: the bit, sign-extended to a
// whole word, selects between the two bit patterns (two instructions, no
// condition register).
__device__ __forceinline__ float hide_if(uint32_t word, int bit, float x) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)word, bit, 1);
  float r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "s"(0xff800000u), "v"(x));
  return r;
}

// Bounds of key k0 + t (forward kernels) for an elementwise-masked tile;
// keys past the end get an interval that covers every row.
__device__ __forceinline__ int4 load_bnd(BufRsrc bb, int k0, int Sk, int t) {
  const i32x4 x = __builtin_amdgcn_raw_buffer_load_b128(bb, (k0 + t) * 16, 0, 0);
  return (k0 + t < Sk) ? make_int4(x[0], x[1], x[2], x[3]) : make_int4(INT_MIN, INT_MAX, 0, 0);
}

// Hidden-row words of one key: word g has bit i set when the key's bounds
// hide row q0 + 32 g + i (the union of its two intervals, clipped).
__device__ __forceinline__ void hidden_rows(const int4 bd, int q0, uint32_t (&wd)[BQ / 32]) {
#pragma unroll
  for (int g = 0; g < BQ / 32; ++g) {
    const int base = q0 + 32 * g;
    auto clip = [&](int y) { return min(max(y, base), base + 32) - base; };
    auto rows = [](int lo, int hi) { return hi > lo ? (~0u >> (32 - hi)) & (~0u << lo) : 0u; };
    wd[g] = rows(clip(bd.x), clip(bd.y)) | rows(clip(bd.z), clip(bd.w));
  }
}

__device__ __forceinline__ bf16x8 buf_load16(BufRsrc r, uint32_t byte_offset) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_offset, 0, 0));
}

// Returns x unchanged, but opaque to the optimiser: a per-lane base offset
// passed through this inside a loop is not hoisted out of it, so the constant
// parts of the addresses built on it fold into the instructions' immediate
// offset fields instead of occupying one register each for the whole kernel.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// The same inside a loop, tied to `salt`, a scalar that changes from one trip
// to the next (which is what keeps the value from being hoisted).  This asm
// has no side effects, so unlike the one above it does not stop the
// scheduler from moving memory accesses past it.
__device__ __forceinline__ uint32_t opaque(uint32_t x, int salt) {
  asm("" : "+v"(x) : "s"(salt));
  return x;
}

// This lane's index in its wave (0..63), computed afresh where it is called
// inside a loop (tied to `salt`, as above): a value rebuilt from it in two
// instructions then takes no register, nor a spill slot, across the loop.
__device__ __forceinline__ int lane_in(int salt) {
  int r;
  asm("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r) : "s"(salt));
  return r;
}

// Entry i of a uint16 tile list, read through the scalar cache: the list of
// a work item is the same for the whole workgroup, so the aligned 32-bit word
// holding the entry is fetched with a scalar load (constant address space).
// Such loads are tracked by lgkmcnt, not vmcnt, so waiting for one does not
// drain the vector memory queue.  The word may reach two bytes past the last
// entry; the tile-info buffer always continues past a list (the work queues
// follow it).
typedef __attribute__((address_space(4))) const uint32_t const_u32;
__device__ __forceinline__ int list_entry(const uint16_t* lst, int i) {
  const uintptr_t addr = reinterpret_cast<uintptr_t>(lst + i);
  const uint32_t word = *(const_u32*)(addr & ~(uintptr_t)3);
  return (int)((addr & 2) ? (word >> 16) : (word & 0xffffu));
}

// The same in two parts: the scalar load of the word holding entry i, and the
// shift that extracts the entry, so that the wait for the load can be placed
// where the entry is used rather than where it is loaded.
struct ListWord {
  uint32_t word, shift;
};
__device__ __forceinline__ ListWord list_word(const uint16_t* lst, int i) {
  const uintptr_t addr = reinterpret_cast<uintptr_t>(lst + i);
  return {*(const_u32*)(addr & ~(uintptr_t)3), (uint32_t)(addr & 2) * 8u};
}
__device__ __forceinline__ int list_value(ListWord x) { return (int)((x.word >> x.shift) & 0xffffu); }

// ---- work items, taken one ahead ----
// The persistent kernels take items from a cost-sorted queue with an atomic
// ticket.  Reading an item's header only when the item starts costs three
// dependent memory round trips (ticket, queue entry, tile count) before the
// item's first load can be issued.  Instead, wave 0 fetches the header of the
// next item while the current one computes, one dependent step at a time at
// points a block of work apart, and publishes it in LDS before the barrier
// that ends the current item.
typedef __attribute__((address_space(4))) const int const_i32;

struct ItemQueue {
  uint32_t* ticket;       // next queue position to hand out
  const uint32_t* queue;  // item ids, heaviest first
  const int* cnt;         // non-skipped tiles per (b * Hm + hm, block)
  uint32_t n_items, max_items;
  int nBlk, H, Hm, cap;   // blocks per head; heads; mask heads; tile count cap
  // The first nsplit queue entries are taken twice (two halves of their key
  // blocks): ticket v < 2 nsplit is entry v / 2, ticket v >= 2 nsplit entry
  // v - nsplit; n_items counts tickets.
  uint32_t nsplit = 0;
  // nP > 0: the queue holds pairs (b*H + h)*nP + qp of blocks 2qp, 2qp+1 (pair
  // mode), at most max_entries of them, and ticket v is block 2qp + v % 2 of
  // entry v / 2; a second block past the last one (nBlk odd) is no item.
  int nP = 0;
  uint32_t max_entries = 0;

  __device__ __forceinline__ uint32_t position(uint32_t v) const {
    if (nP > 0) return v >> 1;
    return v < 2 * nsplit ? v >> 1 : v - nsplit;
  }
  __device__ __forceinline__ uint32_t entries() const { return nP > 0 ? max_entries : max_items; }
  // The item of ticket v with queue entry raw (clamped to the queue's range);
  // none: the ticket has no item (its block would be nBlk).
  __device__ __forceinline__ uint32_t item_of(uint32_t v, uint32_t raw, bool& none) const {
    raw = min(raw, entries() - 1);
    none = false;
    if (nP <= 0) return raw;
    const uint32_t bh = raw / (uint32_t)nP, qp = raw - bh * (uint32_t)nP;
    const uint32_t blk = 2 * qp + (v & 1u);
    none = blk >= (uint32_t)nBlk;
    return min(bh * (uint32_t)nBlk + min(blk, (uint32_t)nBlk - 1), max_items - 1);
  }

  // index of item `it` (= (b * H + h) * nBlk + blk) in `cnt`
  __device__ __forceinline__ long cnt_index(uint32_t it) const {
    const uint32_t bh = it / (uint32_t)nBlk, blk = it % (uint32_t)nBlk;
    const uint32_t b = bh / (uint32_t)H, h = bh % (uint32_t)H;
    return ((long)b * Hm + (Hm == 1 ? 0 : (long)h)) * nBlk + blk;
  }
  // The first item's header, read directly (thread 0, before the first item).
  // A ticket without an item has count -1.
  __device__ __forceinline__ void first(uint32_t (&hdr)[4]) const {
    const uint32_t idx = atomicAdd(ticket, 1u);
    uint32_t it = 0;
    int c = 0;
    if (idx < n_items) {
      bool none;
      it = item_of(idx, queue[position(idx)], none);
      c = none ? -1 : min(cnt[cnt_index(it)], cap);
    }
    hdr[0] = idx;
    hdr[1] = it;
    hdr[2] = (uint32_t)c;
  }
};

// Fetch of the next item's header, in steps placed far apart in the current
// item:
//   take()         top of the item, before its first load: thread 0 takes
//                  the ticket (a vector atomic, so it returns before any of
//                  the item's loads and waiting for it costs nothing extra);
//   stash()        after the item's first wait for its own loads: thread 0
//                  puts the ticket into the next header slot in LDS;
//   fetch_entry()  after a barrier, right before another: every wave reads
//                  the ticket and issues the scalar load of the queue entry;
//   fetch_count()  right before a later barrier: the scalar load of the
//                  item's tile count;
//   publish()      thread 0 writes the header; the barrier that ends the
//                  current item makes it visible.
// A scalar load is waited for together with every LDS access in flight, so
// each one is issued right before a barrier and its value used only after
// it.  Every wave runs the scalar steps itself (the values are the same), so
// no branch on the wave index is needed.
struct ItemPrefetch {
  uint32_t ticket_v = 0;   // thread 0: the ticket
  uint32_t idx = 0, item = 0;
  int cnt = 0;

  __device__ __forceinline__ void take(const ItemQueue& q, unsigned t) {
    if (t == 0) ticket_v = atomicAdd(q.ticket, 1u);
  }
  __device__ __forceinline__ void stash(uint32_t (&hdr)[4], unsigned t) const {
    if (t == 0) hdr[3] = ticket_v;
  }
  __device__ __forceinline__ void fetch_entry(const ItemQueue& q, const uint32_t (&hdr)[4]) {
    idx = __builtin_amdgcn_readfirstlane(hdr[3]);
    item = *(const_u32*)(q.queue + min(q.position(idx), q.entries() - 1));   // raw until fetch_count
  }
  __device__ __forceinline__ void fetch_count(const ItemQueue& q) {
    bool none;
    item = q.item_of(idx, item, none);
    cnt = none ? -1 : *(const_i32*)(q.cnt + q.cnt_index(item));   // raw until publish
  }
  __device__ __forceinline__ void publish(const ItemQueue& q, uint32_t (&hdr)[4], unsigned t) const {
    if (t == 0) {
      hdr[0] = idx;
      hdr[1] = item;
      hdr[2] = (uint32_t)min(cnt, q.cap);
    }
  }
  // all steps after take() at once, for an item without blocks of work
  __device__ __forceinline__ void finish_now(const ItemQueue& q, uint32_t (&hdr)[4], unsigned t) {
    stash(hdr, t);
    __syncthreads();
    fetch_entry(q, hdr);
    fetch_count(q);
    publish(q, hdr, t);
  }
};

// Whether the backward runs with the tile cache: the caller gave room for
// it and the tile pass counted no more tiles than that (same in every
// thread: both values are uniform).
__device__ __forceinline__ bool tile_cache_on(const uint32_t* counters, uint32_t cap) {
  return cap > 0 && *(const_u32*)(counters + kCtrTiles) <= cap;
}

__device__ __forceinline__ const bf16x8& as_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

}  // namespace fm
