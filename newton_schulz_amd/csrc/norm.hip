// Frobenius norm of every Newton-Schulz unit, reduced deterministically.
//
// X_0 = Y / (||Y||_F + eps) starts the iteration; the blog "Muon Optimizer +
// FSDP" (section "Memory control", item 4) advises keeping the normalisation
// scalars in FP32 even when the buffers are BF16.  The squares are exact
// (bf16^2 fits fp32; fp32^2 fits fp64) and summed in fp64 in a fixed order,
// with no atomics, so the scale is bit-reproducible.  Two sources:
//   - the momentum pass's per-4096-element partials (norm_from_blocks_kernel
//     adds a unit's blocks), when the caller hands them over: no second read;
//   - otherwise a pass over the units: per thread over its interleaved
//     pieces, a fixed shared-memory tree, then the parts of a unit in index
//     order (norm_partial_kernel + norm_finalize_kernel).
// The scale 1/(||Y|| + eps) is folded into the first iteration's epilogues
// instead of rewriting Y.
#include "muon_device.h"
#include "muon_internal.h"

using muon::bf16_t;

namespace {

// The elements of a unit are cut into pieces of 256 groups of 8 (one group
// per thread); workgroup p of a unit's P takes pieces p, p + P, p + 2 P, ...
// At any moment the workgroups of a unit read neighbouring pieces, so the
// grid streams through each unit as a few moving windows (much friendlier to
// HBM pages than P separate contiguous runs).  The order of every sum depends
// on the unit size and P only.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void norm_partial_kernel(NsNormArgs a) {
  const int64_t u = blockIdx.y;
  const int64_t p = blockIdx.x, P = a.parts;
  const T* base = reinterpret_cast<const T*>(mat_at(a.in, u));
  const int64_t ue = a.unit_elems;
  double acc = 0.0;
  if (VEC) {
    const int64_t ng = ue / 8;  // full 8-element groups
    // U pieces per trip, all loaded before the first use (a part of ~32K
    // elements is one trip in bf16, two in fp32); a group past the unit
    // contributes zeros.  Within a group the eight squares are added as a
    // fixed pairwise tree.
    constexpr int U = sizeof(T) == 2 ? 16 : 8;
    for (int64_t q0 = p; q0 * 256 < ng; q0 += U * P) {
      if (sizeof(T) == 2) {
        uint4 v[U];
#pragma unroll
        for (int r = 0; r < U; ++r) {
          const int64_t g = (q0 + r * P) * 256 + threadIdx.x;
          v[r] = g < ng ? *reinterpret_cast<const uint4*>(base + 8 * g) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < U; ++r) {
          const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
          double q[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
            q[2 * i] = static_cast<double>(lo * lo);
            q[2 * i + 1] = static_cast<double>(hi * hi);
          }
          acc += ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
        }
      } else {
        float4 x[U], y[U];
#pragma unroll
        for (int r = 0; r < U; ++r) {
          const int64_t g = (q0 + r * P) * 256 + threadIdx.x;
          const float4* f = reinterpret_cast<const float4*>(base + 8 * g);
          x[r] = g < ng ? f[0] : make_float4(0.f, 0.f, 0.f, 0.f);
          y[r] = g < ng ? f[1] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int r = 0; r < U; ++r) {
          const float v[8] = {x[r].x, x[r].y, x[r].z, x[r].w, y[r].x, y[r].y, y[r].z, y[r].w};
          double q[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) q[i] = static_cast<double>(v[i]) * static_cast<double>(v[i]);
          acc += ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
        }
      }
    }
    if (p == 0) {  // the last ue % 8 elements
      for (int64_t e = 8 * ng + threadIdx.x; e < ue; e += 256) {
        const double v = static_cast<double>(muon::Elem<T>::load(base + e));
        acc += v * v;
      }
    }
  } else {
    for (int64_t e = p * 256 + threadIdx.x; e < ue; e += P * 256) {
      const double v = static_cast<double>(muon::Elem<T>::load(base + e));
      acc += v * v;
    }
  }
  __shared__ double red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.partial[u * a.parts + p] = red[0];
}

// Unit u's scale, zero flag and non-finite report from its sum of squares.
__device__ __forceinline__ void finish_unit(const NsNormArgs& a, int64_t u, double s) {
  const double nrm = sqrt(s);
  a.scale[u] = static_cast<float>(1.0 / (nrm + static_cast<double>(a.eps)));
  a.zflag[u] = (s == 0.0) ? 1 : 0;
  if (a.nonfinite && !isfinite(s)) atomicOr(a.nonfinite, 1);
}

// One wave per unit: lane l adds parts l, l + 64, l + 128, ... in order, then
// an xor butterfly adds the 64 lane sums (both partners of a step form the
// same sum, so every lane ends with the same, fixed-order total).
__global__ __launch_bounds__(256) void norm_finalize_kernel(NsNormArgs a) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (u >= a.units) return;
  double s = 0.0;
  for (int p = lane; p < a.parts; p += 64) s += a.partial[u * a.parts + p];
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) s += __shfl_xor(s, k, 64);
  if (lane == 0) finish_unit(a, u, s);
}

// The same from the momentum pass's per-block partials, one workgroup per
// unit: unit u owns blocks b0 .. b0 + blocks_per_unit - 1, b0 = (address of
// u - sq_base) / block_bytes (the host has checked that every unit starts on
// a block boundary inside the partials).  Thread t adds blocks t, t + 256,
// ... in order, eight loads in flight ahead of the adds; then a butterfly per
// wave and the four wave sums pairwise.
__global__ __launch_bounds__(256) void norm_from_blocks_kernel(NsNormArgs a) {
  const int64_t u = blockIdx.x;
  const int64_t b0 = (reinterpret_cast<const char*>(mat_at(a.in, u)) - a.sq_base) / a.block_bytes;
  const double* q = a.sq + b0;
  const int64_t nb = a.blocks_per_unit;
  constexpr int R = 8;
  double s = 0.0;
  for (int64_t p0 = threadIdx.x; p0 < nb; p0 += R * 256) {
    double v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t p = p0 + r * 256;
      v[r] = p < nb ? q[p] : 0.0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) s += v[r];
  }
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) s += __shfl_xor(s, k, 64);
  __shared__ double ws[4];
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) finish_unit(a, u, (ws[0] + ws[1]) + (ws[2] + ws[3]));
}

// The units whose norm is not zero, in ascending order, and their number:
// one workgroup walks the flags 256 at a time; a wave's lanes count the
// nonzero units before them with a ballot, the four wave counts give each
// wave its offset, so every unit lands at its rank.
__global__ __launch_bounds__(256) void compact_units_kernel(const int* __restrict__ zflag, int64_t units,
                                                            int* __restrict__ list, int* __restrict__ count) {
  __shared__ int wcnt[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t base = 0;  // nonzero units before this chunk
  for (int64_t u0 = 0; u0 < units; u0 += 256) {
    const int64_t u = u0 + threadIdx.x;
    const bool keep = u < units && zflag[u] == 0;
    const uint64_t mask = __ballot(keep);
    const int before = __popcll(mask & ((uint64_t{1} << lane) - 1));
    if (lane == 0) wcnt[wave] = __popcll(mask);
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wave; ++w) off += wcnt[w];
    if (keep) list[base + off + before] = static_cast<int>(u);
    base += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();  // wcnt is rewritten by the next chunk
  }
  if (threadIdx.x == 0) *count = static_cast<int>(base);
}

// out[u] = s[u] * in[u] element by element (s = 1 without scale), read as Ti
// and stored as To (bf16: rounded to nearest even)
template <typename Ti, typename To>
__global__ __launch_bounds__(256) void scale_copy_kernel(MatRef in, MatRef out, int64_t n,
                                                         const float* scale) {
  const int64_t u = blockIdx.y;
  const Ti* src = reinterpret_cast<const Ti*>(mat_at(in, u));
  To* dst = reinterpret_cast<To*>(mat_at(out, u));
  const float s = scale ? scale[u] : 1.0f;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    muon::Elem<To>::store(dst + e, s * muon::Elem<Ti>::load(src + e));
  }
}

}  // namespace

// MatRef of units [u0, ...) of r.
static MatRef shifted(MatRef r, int64_t u0) {
  if (r.table) r.table += u0;
  else r.base += u0 * r.stride;
  return r;
}

hipError_t launch_norm(hipStream_t s, const NsNormArgs& a, int io_bf16, bool vec) {
  if (a.units == 0) return hipSuccess;
  if (a.sq != nullptr) {
    if (a.units > 0x7fffffff) return hipErrorInvalidValue;
    norm_from_blocks_kernel<<<static_cast<unsigned>(a.units), 256, 0, s>>>(a);
    return hipGetLastError();
  }
  constexpr int64_t kMaxY = 65535;
  for (int64_t u0 = 0; u0 < a.units; u0 += kMaxY) {
    NsNormArgs c = a;
    c.units = (a.units - u0 < kMaxY) ? a.units - u0 : kMaxY;
    c.in = shifted(a.in, u0);
    c.partial = a.partial + u0 * a.parts;
    c.scale = a.scale + u0;
    c.zflag = a.zflag + u0;
    dim3 grid(static_cast<unsigned>(c.parts), static_cast<unsigned>(c.units));
    if (io_bf16) {
      if (vec) norm_partial_kernel<bf16_t, true><<<grid, 256, 0, s>>>(c);
      else norm_partial_kernel<bf16_t, false><<<grid, 256, 0, s>>>(c);
    } else {
      if (vec) norm_partial_kernel<float, true><<<grid, 256, 0, s>>>(c);
      else norm_partial_kernel<float, false><<<grid, 256, 0, s>>>(c);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    norm_finalize_kernel<<<static_cast<unsigned>((c.units + 3) / 4), 256, 0, s>>>(c);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_compact_units(hipStream_t s, const int* zflag, int64_t units, int* list, int* count) {
  if (units <= 0 || units > 0x7fffffff) return hipErrorInvalidValue;
  compact_units_kernel<<<1, 256, 0, s>>>(zflag, units, list, count);
  return hipGetLastError();
}

hipError_t launch_scale_copy(hipStream_t s, MatRef in, MatRef out, int64_t unit_elems,
                             int64_t units, const float* scale, int io_bf16) {
  return launch_convert(s, in, io_bf16, out, io_bf16, unit_elems, units, scale);
}

hipError_t launch_convert(hipStream_t s, MatRef in, int in_bf16, MatRef out, int out_bf16,
                          int64_t unit_elems, int64_t units, const float* scale) {
  if (units == 0 || unit_elems == 0) return hipSuccess;
  int64_t bx = (unit_elems + 255) / 256;
  if (bx > 1024) bx = 1024;
  constexpr int64_t kMaxY = 65535;
  for (int64_t u0 = 0; u0 < units; u0 += kMaxY) {
    const int64_t n = (units - u0 < kMaxY) ? units - u0 : kMaxY;
    dim3 grid(static_cast<unsigned>(bx), static_cast<unsigned>(n));
    const MatRef i0 = shifted(in, u0), o0 = shifted(out, u0);
    const float* s0 = scale ? scale + u0 : nullptr;
    if (in_bf16 && out_bf16) scale_copy_kernel<bf16_t, bf16_t><<<grid, 256, 0, s>>>(i0, o0, unit_elems, s0);
    else if (in_bf16) scale_copy_kernel<bf16_t, float><<<grid, 256, 0, s>>>(i0, o0, unit_elems, s0);
    else if (out_bf16) scale_copy_kernel<float, bf16_t><<<grid, 256, 0, s>>>(i0, o0, unit_elems, s0);
    else scale_copy_kernel<float, float><<<grid, 256, 0, s>>>(i0, o0, unit_elems, s0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
