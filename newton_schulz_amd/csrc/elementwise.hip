// Streaming kernels of the Muon step: momentum (+ Nesterov) and weight apply.
//
// Both are HBM-bound passes.  The vector path is a one-shot launch: workgroup
// b owns the 4096 consecutive elements [4096 b, 4096 b + 4096), each thread
// two groups of 8 elements 2048 apart, all loads issued before any store, with
// 16-byte (bf16) / 32-byte (fp32) accesses.  On MI355X this streams ~10%
// faster than a persistent grid-stride loop over the same range: the
// dispatcher hands out workgroups in address order, so the HBM pages in use
// at any moment stay few.  Unaligned ranges take a grid-stride scalar loop.
// Every arithmetic operation is a separate IEEE binary32 operation rounded to
// nearest-even (contraction is disabled for this file), so the results are
// bit-identical to a binary32 evaluation of the same sequence.
//
// The momentum pass can also leave, per block of 4096 elements, the sum of
// squares of the update as stored, in binary64: the Frobenius norms that
// start the Newton-Schulz iteration then need no second read of the update.
// Each square of a bf16 or fp32 value is exact in binary64; the sums run in a
// fixed order (per thread, then a butterfly across each wave, then the four
// wave sums pairwise), so the partials are reproducible bit for bit.
#include "muon_device.h"
#include "muon_internal.h"

#pragma clang fp contract(off)

using muon::bf16_t;

namespace {

typedef float f32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));

template <typename T> struct Vec8;
template <> struct Vec8<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  template <bool NT = false>
  __device__ __forceinline__ void store(float* p) const {
    f32x4_nt* q = reinterpret_cast<f32x4_nt*>(p);
    const f32x4_nt a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    if (NT) {
      __builtin_nontemporal_store(a, q);
      __builtin_nontemporal_store(b, q + 1);
    } else {
      q[0] = a;
      q[1] = b;
    }
  }
};
template <> struct Vec8<bf16_t> {
  float v[8];
  __device__ __forceinline__ void load(const bf16_t* p) {
    uint4 a = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  template <bool NT = false>
  __device__ __forceinline__ void store(bf16_t* p) const {
    uint4 a;
    a.x = muon::pack_bf16x2(v[0], v[1]);
    a.y = muon::pack_bf16x2(v[2], v[3]);
    a.z = muon::pack_bf16x2(v[4], v[5]);
    a.w = muon::pack_bf16x2(v[6], v[7]);
    if (NT)
      __builtin_nontemporal_store(u32x4_nt{a.x, a.y, a.z, a.w}, reinterpret_cast<u32x4_nt*>(p));
    else
      *reinterpret_cast<uint4*>(p) = a;
  }
};

__device__ __forceinline__ void momentum_one(float g, float& m, float& u, float beta, float c1,
                                             bool nesterov) {
  const float t = c1 * g;
  const float bm = beta * m;
  const float mn = bm + t;
  m = mn;
  if (nesterov) {
    const float bmn = beta * mn;
    u = t + bmn;
  } else {
    u = mn;
  }
}

// one-shot vector path: EW_U groups of 8 elements per thread, EW_BS threads
constexpr int EW_BS = 256, EW_U = 2;  // 4096 elements per workgroup
static_assert(EW_BS * EW_U * 8 == MUON_SQ_BLOCK, "a workgroup's range is one partial block");

// exact square of a stored value
__device__ __forceinline__ double sq64(float v) {
  const double d = static_cast<double>(v);
  return d * d;
}

// Sum of the 256 threads' values in a fixed order; thread 0 gets the total.
__device__ __forceinline__ double block_sum(double v) {
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) v += __shfl_xor(v, k, 64);
  __shared__ double ws[EW_BS / 64];
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = v;
  __syncthreads();
  return (ws[0] + ws[1]) + (ws[2] + ws[3]);
}

template <typename G, typename U, bool SQ>
__global__ __launch_bounds__(EW_BS) void momentum_vec_kernel(const G* __restrict__ grad,
                                                             float* __restrict__ mom,
                                                             U* __restrict__ upd, int64_t numel,
                                                             float beta, float c1, int nesterov,
                                                             double* __restrict__ sq) {
  const bool nes = nesterov != 0;
  const int64_t nvec = numel / 8;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (EW_U * EW_BS) + threadIdx.x;
  double acc = 0.0;
  Vec8<G> g[EW_U];
  Vec8<float> m[EW_U];
#pragma unroll
  for (int k = 0; k < EW_U; ++k) {
    const int64_t i = base + k * EW_BS;
    if (i < nvec) {
      g[k].load(grad + 8 * i);
      m[k].load(mom + 8 * i);
    }
  }
#pragma unroll
  for (int k = 0; k < EW_U; ++k) {
    const int64_t i = base + k * EW_BS;
    if (i < nvec) {
      Vec8<U> u;
#pragma unroll
      for (int e = 0; e < 8; ++e) momentum_one(g[k].v[e], m[k].v[e], u.v[e], beta, c1, nes);
      // the momentum is next read a whole step later: do not keep it cached;
      // U is read next by a launch that streams far more than the caches
      // hold (non-temporal stores measured 1% faster here, and no slower for
      // the Newton-Schulz launch that reads U)
      m[k].template store<true>(mom + 8 * i);
      u.template store<true>(upd + 8 * i);
      if (SQ) {
        double q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = sq64(muon::Elem<U>::round(u.v[e]));
        acc += ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
      }
    }
  }
  // The last numel % 8 elements; they lie in the last workgroup's range (the
  // grid has one workgroup per started 4096 elements).
  if (blockIdx.x == gridDim.x - 1) {
    for (int64_t i = nvec * 8 + threadIdx.x; i < numel; i += EW_BS) {
      float mm = mom[i], u;
      momentum_one(muon::Elem<G>::load(grad + i), mm, u, beta, c1, nes);
      mom[i] = mm;
      muon::Elem<U>::store(upd + i, u);
      if (SQ) acc += sq64(muon::Elem<U>::round(u));
    }
  }
  if (SQ) {
    const double t = block_sum(acc);
    if (threadIdx.x == 0) sq[blockIdx.x] = t;
  }
}

// Partials of an update written by the scalar path: workgroup b sums the
// squares of elements [4096 b, 4096 b + 4096), thread t elements t + 256 j
// in j order.
template <typename U>
__global__ __launch_bounds__(EW_BS) void sq_blocks_kernel(const U* __restrict__ upd, int64_t numel,
                                                          double* __restrict__ sq) {
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * MUON_SQ_BLOCK;
  double acc = 0.0;
  for (int j = 0; j < MUON_SQ_BLOCK / EW_BS; ++j) {
    const int64_t i = b0 + j * EW_BS + threadIdx.x;
    if (i < numel) acc += sq64(muon::Elem<U>::load(upd + i));
  }
  const double t = block_sum(acc);
  if (threadIdx.x == 0) sq[blockIdx.x] = t;
}

template <typename G, typename U>
__global__ __launch_bounds__(256) void momentum_scalar_kernel(const G* __restrict__ grad,
                                                              float* __restrict__ mom,
                                                              U* __restrict__ upd, int64_t numel,
                                                              float beta, float c1, int nesterov) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nth = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const bool nes = nesterov != 0;
  for (int64_t i = tid; i < numel; i += nth) {
    float m = mom[i], u;
    momentum_one(muon::Elem<G>::load(grad + i), m, u, beta, c1, nes);
    mom[i] = m;
    muon::Elem<U>::store(upd + i, u);
  }
}

__device__ __forceinline__ float apply_one(float w, float u, float eta, float decay, bool wd) {
  const float w1 = wd ? w * decay : w;
  const float step = eta * u;
  return w1 - step;
}

template <typename U, bool WANT_BF16>
__global__ __launch_bounds__(EW_BS) void apply_vec_kernel(float* __restrict__ master,
                                                          const U* __restrict__ upd,
                                                          bf16_t* __restrict__ wbf, int64_t numel,
                                                          float eta, float decay, int has_wd) {
  const bool wd = has_wd != 0;
  const int64_t nvec = numel / 8;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (EW_U * EW_BS) + threadIdx.x;
  Vec8<float> w[EW_U];
  Vec8<U> u[EW_U];
#pragma unroll
  for (int k = 0; k < EW_U; ++k) {
    const int64_t i = base + k * EW_BS;
    if (i < nvec) {
      w[k].load(master + 8 * i);
      u[k].load(upd + 8 * i);
    }
  }
#pragma unroll
  for (int k = 0; k < EW_U; ++k) {
    const int64_t i = base + k * EW_BS;
    if (i < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[k].v[e] = apply_one(w[k].v[e], u[k].v[e], eta, decay, wd);
      // neither copy of the weights is read again within the step
      w[k].template store<true>(master + 8 * i);
      if (WANT_BF16) {
        Vec8<bf16_t> b;
#pragma unroll
        for (int e = 0; e < 8; ++e) b.v[e] = w[k].v[e];
        b.template store<true>(wbf + 8 * i);
      }
    }
  }
  if (blockIdx.x == gridDim.x - 1) {  // the last numel % 8 elements
    for (int64_t i = nvec * 8 + threadIdx.x; i < numel; i += EW_BS) {
      const float x = apply_one(master[i], muon::Elem<U>::load(upd + i), eta, decay, wd);
      master[i] = x;
      if (WANT_BF16) wbf[i] = muon::f32_to_bf16(x);
    }
  }
}

template <typename U, bool WANT_BF16>
__global__ __launch_bounds__(256) void apply_scalar_kernel(float* __restrict__ master,
                                                           const U* __restrict__ upd,
                                                           bf16_t* __restrict__ wbf, int64_t numel,
                                                           float eta, float decay, int has_wd) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nth = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const bool wd = has_wd != 0;
  for (int64_t i = tid; i < numel; i += nth) {
    const float x = apply_one(master[i], muon::Elem<U>::load(upd + i), eta, decay, wd);
    master[i] = x;
    if (WANT_BF16) wbf[i] = muon::f32_to_bf16(x);
  }
}

// one workgroup per started 4096 elements; the last one also takes the
// scalar tail, which lies in its range
inline unsigned vec_grid(int64_t numel) {
  const int64_t blocks = (numel + MUON_SQ_BLOCK - 1) / MUON_SQ_BLOCK;
  return static_cast<unsigned>(blocks < 1 ? 1 : blocks);
}

inline unsigned stream_grid(int64_t work_items, int cus) {
  // grid-stride scalar path: up to 8 workgroups of 256 threads per CU
  int64_t blocks = (work_items + 255) / 256;
  const int64_t cap = static_cast<int64_t>(cus) * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return static_cast<unsigned>(blocks);
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

hipError_t launch_momentum(hipStream_t s, int cus, const void* grad, int gdt, float* mom,
                           void* upd, int udt, int64_t numel, float beta, float c1,
                           int nesterov, double* sq) {
  if (numel <= 0) return hipSuccess;
  // one workgroup per 4096 elements must fit a 1-D grid
  if ((numel + MUON_SQ_BLOCK - 1) / MUON_SQ_BLOCK > 0x7fffffff) return hipErrorInvalidValue;
  const bool vec = aligned(grad, 16) && aligned(mom, 16) && aligned(upd, 16);
#define MUON_MOM(G, U)                                                                        \
  do {                                                                                        \
    if (vec && sq)                                                                            \
      momentum_vec_kernel<G, U, true><<<vec_grid(numel), EW_BS, 0, s>>>(                      \
          static_cast<const G*>(grad), mom, static_cast<U*>(upd), numel, beta, c1, nesterov,  \
          sq);                                                                                \
    else if (vec)                                                                             \
      momentum_vec_kernel<G, U, false><<<vec_grid(numel), EW_BS, 0, s>>>(                     \
          static_cast<const G*>(grad), mom, static_cast<U*>(upd), numel, beta, c1, nesterov,  \
          nullptr);                                                                           \
    else                                                                                      \
      momentum_scalar_kernel<G, U><<<stream_grid(numel, cus), 256, 0, s>>>(                   \
          static_cast<const G*>(grad), mom, static_cast<U*>(upd), numel, beta, c1, nesterov);  \
    if (!vec && sq)                                                                           \
      sq_blocks_kernel<U><<<vec_grid(numel), EW_BS, 0, s>>>(static_cast<const U*>(upd), numel, \
                                                             sq);                             \
  } while (0)
  if (gdt == 1 && udt == 1) MUON_MOM(bf16_t, bf16_t);
  else if (gdt == 1 && udt == 0) MUON_MOM(bf16_t, float);
  else if (gdt == 0 && udt == 1) MUON_MOM(float, bf16_t);
  else MUON_MOM(float, float);
#undef MUON_MOM
  return hipGetLastError();
}

hipError_t launch_apply(hipStream_t s, int cus, float* master, const void* upd, int udt,
                        void* wbf, int64_t numel, float eta, float decay, int has_wd) {
  if (numel <= 0) return hipSuccess;
  if ((numel + MUON_SQ_BLOCK - 1) / MUON_SQ_BLOCK > 0x7fffffff) return hipErrorInvalidValue;
  const bool vec = aligned(master, 16) && aligned(upd, 16) && (wbf == nullptr || aligned(wbf, 16));
  bf16_t* wb = static_cast<bf16_t*>(wbf);
#define MUON_APPLY(U, B)                                                                         \
  do {                                                                                           \
    if (vec)                                                                                     \
      apply_vec_kernel<U, B><<<vec_grid(numel), EW_BS, 0, s>>>(                                   \
          master, static_cast<const U*>(upd), wb, numel, eta, decay, has_wd);                    \
    else                                                                                         \
      apply_scalar_kernel<U, B><<<stream_grid(numel, cus), 256, 0, s>>>(                         \
          master, static_cast<const U*>(upd), wb, numel, eta, decay, has_wd);                    \
  } while (0)
  if (udt == 1) {
    if (wb) MUON_APPLY(bf16_t, true); else MUON_APPLY(bf16_t, false);
  } else {
    if (wb) MUON_APPLY(float, true); else MUON_APPLY(float, false);
  }
#undef MUON_APPLY
  return hipGetLastError();
}
