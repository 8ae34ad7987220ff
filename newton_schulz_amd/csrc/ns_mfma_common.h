// Device helpers shared by the bf16 MFMA Newton-Schulz kernels (gfx950):
// vector types, buffer descriptors, the global -> LDS DMA load, the LDS tile
// layouts with their XOR swizzles, and compile-time loops.
#pragma once

#include "muon_device.h"
#include "muon_internal.h"

#include <utility>

using muon::bf16_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_ptr_t;

namespace {

constexpr uint32_t kOOB = 0x80000000u; // buffer offset past any matrix: loads return 0
constexpr int kRsrcWord3 = 0x00020000; // raw buffer, 32-bit data format (gfx9 family)

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; a field at its maximum does not wait.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// A pointer every lane holds the same value of, moved to scalar registers
// (buffer descriptors need it; a value read from a device table is not known
// to be uniform otherwise).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

__device__ __forceinline__ void dma16(const __amdgpu_buffer_rsrc_t& r, char* lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// The same 16-byte global -> LDS load for the operand stages, written as
// inline asm on a descriptor held as four words.  The compiler then does not
// track these LDS writes: the k-loop orders them itself (s_waitcnt vmcnt
// before each barrier), and no conservative wait for the most recent load is
// inserted ahead of LDS reads of other stage buffers.  M0 holds the LDS
// destination of the wave's 1 KiB block.
//
// The compiler does not look inside inline asm for hazards, so the asm keeps
// its own: a vector-ALU write of an SGPR (v_readlane reloading a spilled
// scalar, v_readfirstlane) needs 5 wait states before a vector-memory
// instruction reads that SGPR (descriptor, offset), and an M0 write needs 1
// before an LDS-DMA load.  Without them the load may take a stale offset and
// fill the stage with the wrong data, depending on where register pressure
// places the reloads.
__device__ __forceinline__ u32x4_t rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  return u32x4_t{static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32) & 0xffffu, bytes,
                 static_cast<uint32_t>(kRsrcWord3)};
}
__device__ __forceinline__ void dma16_asm(const u32x4_t& r, char* lds, uint32_t voff,
                                          uint32_t soff) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)lds));
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff),
      "s"(r), "s"(soff), "s"(m0)
      : "memory", "m0");
}
// Four such loads from one descriptor and offset in one asm block, so the
// five wait states are paid once for the four.
__device__ __forceinline__ void dma16x4_asm(const u32x4_t& r, char* const (&lds)[4],
                                            const uint32_t (&voff)[4], uint32_t soff) {
  const uint32_t m0[4] = {static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)lds[0])),
                          static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)lds[1])),
                          static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)lds[2])),
                          static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)lds[3]))};
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %4, %5 offen lds\n\t"
      "s_mov_b32 m0, %7\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %4, %5 offen lds\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %4, %5 offen lds\n\t"
      "s_mov_b32 m0, %9\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %3, %4, %5 offen lds" ::"v"(voff[0]),
      "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(r), "s"(soff), "s"(m0[0]), "s"(m0[1]),
      "s"(m0[2]), "s"(m0[3])
      : "memory", "m0");
}
// NG loads of one operand stage: groups of four, then singles.
template <int NG, typename FL, typename FV>
__device__ __forceinline__ void dma16_group(const u32x4_t& r, uint32_t soff, FL&& lds_of, FV&& voff_of) {
  static_assert(NG >= 1, "no loads");
  constexpr int G4 = NG / 4;
#pragma unroll
  for (int g = 0; g < G4; ++g) {
    char* const l[4] = {lds_of(4 * g), lds_of(4 * g + 1), lds_of(4 * g + 2), lds_of(4 * g + 3)};
    const uint32_t v[4] = {voff_of(4 * g), voff_of(4 * g + 1), voff_of(4 * g + 2), voff_of(4 * g + 3)};
    dma16x4_asm(r, l, v, soff);
  }
#pragma unroll
  for (int q = 4 * G4; q < NG; ++q) dma16_asm(r, lds_of(q), voff_of(q), soff);
}

// Four consecutive k of one column of a row-major [k][col] LDS tile per lane
// (ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte words addressed by lanes i / 4 + 4 r, r = 0..3).
__device__ __forceinline__ i16x4_t ld_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(p));
}

// ---- K-contiguous operand tile: R rows x BK (= 64), 128-byte rows of
// 16-byte chunks.  The chunk swizzle chunk ^ (row ^ row >> 3) & 7 puts the
// 16 rows one LDS cycle of a fragment read serves (same logical chunk,
// consecutive rows) on distinct banks.
template <int BK>
__device__ __forceinline__ int rt_swz(int row) {
  static_assert(BK == 64, "swizzle laid out for 64-element rows");
  return (row ^ (row >> 3)) & 7;
}
template <int BK>
__device__ __forceinline__ int rt_off(int row, int chunk) {
  return row * (2 * BK) + ((chunk ^ rt_swz<BK>(row)) << 4);
}

// ---- K-major operand tile: BK rows (k) x R columns, 2R-byte rows, chunk
// swizzle 4 (k & 3): the four k rows a transposed read touches land on
// distinct banks.  col is a multiple of 4.
template <int R>
__device__ __forceinline__ int kt_off(int k, int col) {
  return k * (2 * R) + (((col >> 3) ^ ((k & 3) << 2)) << 4) + ((col & 7) << 1);
}

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): indices
// stay compile-time constants, so register arrays are never indexed at run time.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <int V>
using ic = std::integral_constant<int, V>;

}  // namespace
