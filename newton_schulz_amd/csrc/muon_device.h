// Device-side helpers shared by the libmuon kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef uint16_t bf16_t;  // bfloat16 bit pattern

// bf16 -> fp32 is exact: the pattern is the high half of the fp32 pattern.
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN;
// overflow rounds to infinity.  On the bit pattern u: a NaN gives
// (u >> 16) | 0x40, anything else the high half of u + 0x7fff + ((u >> 16) & 1).
// gfx950 does this in one instruction, v_cvt_pk_bf16_f32 (two values at a
// time): on an MI355X its result equals that rule for every one of the 2^32
// inputs, NaN payloads included, so the kernels use it.
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed pair of bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.0f));
}

template <typename T> struct Elem;

// fp32 -> the nearest bf16 value, as fp32.
__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// The bf16 iteration with the iterate carried past bf16.  The iterate is
// X = hi + lo: hi the stored bf16 matrix the products read, lo its rounding
// residual (kept in a plane of its own).  The MFMA applies B' with its
// diagonal d rounded to bf16, so it sums (B'_bf16 hi)_ij; the diagonal's
// contribution d X_ij = bf16(d) hi + (d - bf16(d)) hi + d lo is completed:
// r hi (r = ns_diag_residual(d), rounded to bf16) as one more MFMA against a
// diagonal operand in the k-step that contracts over row i (wide; column j
// when tall), d lo after the last MFMA (ns_lo_term).  Without this, the
// small singular values that the iteration lifts by up to a^steps are lost in
// the bf16 storage of X.  Every kernel computing it keeps this order (no
// contraction), so they give the same bits.
__device__ __forceinline__ float ns_diag_residual(float d) { return d - bf16_round(d); }
__device__ __forceinline__ float ns_lo_term(float acc, float d, float lo) { return acc + d * lo; }

template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
  // the value a store keeps
  static __device__ __forceinline__ float round(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
  static __device__ __forceinline__ float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

}  // namespace muon

// A batch of same-shape matrices on the device: either base + i * stride
// (bytes) or an explicit device table of pointers.
struct MatRef {
  const char* base;
  int64_t stride;
  const uint64_t* table;
};

__host__ __device__ __forceinline__ char* mat_at(const MatRef& r, int64_t i) {
  return r.table ? reinterpret_cast<char*>(r.table[i]) : const_cast<char*>(r.base) + i * r.stride;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Map the hardware id to a logical id so that each XCD receives one
// contiguous run of logical tiles: neighbours in logical order share L2.
__device__ __forceinline__ int64_t xcd_logical_id(int64_t hw, int64_t grid) {
  const int64_t per = grid / 8, rem = grid % 8;
  const int64_t x = hw % 8, k = hw / 8;
  return x * per + (x < rem ? x : rem) + k;
}
