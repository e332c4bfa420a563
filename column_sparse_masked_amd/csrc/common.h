// Device-side definitions shared by the libfm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
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
              kCtrFwdExit = 4, kCtrBwdExit = 5, kCtrDqNext = 6, kCtrDqExit = 7;

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

// Physical row of row d of a transposed LDS tile (rows indexed by the head
// dimension).  Staging lanes store rows 8 apart at the same column; rotating
// the rows of every group of 8 by 2 (d/8 + d/32) spreads those stores over
// distinct banks, while 16 consecutive rows (one MFMA operand read) still map
// to 16 distinct rows of the same group of 16.
__device__ __forceinline__ int trow(int d) {
  return (d & ~7) | (((d & 7) + 2 * (d >> 3) + 2 * (d >> 5)) & 7);
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

__device__ __forceinline__ const bf16x8& as_bf16x8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

}  // namespace fm
