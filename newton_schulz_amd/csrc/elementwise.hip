// Streaming kernels of the Muon step: momentum (+ Nesterov) and weight apply.
//
// Both are HBM-bound passes; each thread moves 8 elements per iteration with
// 16-byte (bf16) / 32-byte (fp32) vector accesses, grid-stride over the flat
// range.  Every arithmetic operation is a separate IEEE binary32 operation
// rounded to nearest-even (contraction is disabled for this file), so the
// results are bit-identical to a binary32 evaluation of the same sequence.
#include "muon_device.h"
#include "muon_internal.h"

#pragma clang fp contract(off)

using muon::bf16_t;

namespace {

template <typename T> struct Vec8;
template <> struct Vec8<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void store(float* p) const {
    float4* q = reinterpret_cast<float4*>(p);
    q[0] = make_float4(v[0], v[1], v[2], v[3]);
    q[1] = make_float4(v[4], v[5], v[6], v[7]);
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
  __device__ __forceinline__ void store(bf16_t* p) const {
    uint4 a;
    a.x = muon::pack_bf16x2(v[0], v[1]);
    a.y = muon::pack_bf16x2(v[2], v[3]);
    a.z = muon::pack_bf16x2(v[4], v[5]);
    a.w = muon::pack_bf16x2(v[6], v[7]);
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

template <typename G, typename U, bool VEC>
__global__ __launch_bounds__(256) void momentum_kernel(const G* __restrict__ grad,
                                                       float* __restrict__ mom,
                                                       U* __restrict__ upd, int64_t numel,
                                                       float beta, float c1, int nesterov) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nth = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const bool nes = nesterov != 0;
  if (VEC) {
    const int64_t nvec = numel / 8;
    for (int64_t i = tid; i < nvec; i += nth) {
      Vec8<G> g;
      Vec8<float> m;
      Vec8<U> u;
      g.load(grad + 8 * i);
      m.load(mom + 8 * i);
#pragma unroll
      for (int k = 0; k < 8; ++k) momentum_one(g.v[k], m.v[k], u.v[k], beta, c1, nes);
      m.store(mom + 8 * i);
      u.store(upd + 8 * i);
    }
    for (int64_t i = nvec * 8 + tid; i < numel; i += nth) {
      float m = mom[i], u;
      momentum_one(muon::Elem<G>::load(grad + i), m, u, beta, c1, nes);
      mom[i] = m;
      muon::Elem<U>::store(upd + i, u);
    }
  } else {
    for (int64_t i = tid; i < numel; i += nth) {
      float m = mom[i], u;
      momentum_one(muon::Elem<G>::load(grad + i), m, u, beta, c1, nes);
      mom[i] = m;
      muon::Elem<U>::store(upd + i, u);
    }
  }
}

__device__ __forceinline__ float apply_one(float w, float u, float eta, float decay, bool wd) {
  const float w1 = wd ? w * decay : w;
  const float step = eta * u;
  return w1 - step;
}

template <typename U, bool VEC, bool WANT_BF16>
__global__ __launch_bounds__(256) void apply_kernel(float* __restrict__ master,
                                                    const U* __restrict__ upd,
                                                    bf16_t* __restrict__ wbf, int64_t numel,
                                                    float eta, float decay, int has_wd) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nth = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const bool wd = has_wd != 0;
  int64_t start_tail = 0;
  if (VEC) {
    const int64_t nvec = numel / 8;
    for (int64_t i = tid; i < nvec; i += nth) {
      Vec8<float> w;
      Vec8<U> u;
      w.load(master + 8 * i);
      u.load(upd + 8 * i);
#pragma unroll
      for (int k = 0; k < 8; ++k) w.v[k] = apply_one(w.v[k], u.v[k], eta, decay, wd);
      w.store(master + 8 * i);
      if (WANT_BF16) {
        Vec8<bf16_t> b;
#pragma unroll
        for (int k = 0; k < 8; ++k) b.v[k] = w.v[k];
        b.store(wbf + 8 * i);
      }
    }
    start_tail = nvec * 8;
  }
  for (int64_t i = start_tail + tid; i < numel; i += nth) {
    const float w = apply_one(master[i], muon::Elem<U>::load(upd + i), eta, decay, wd);
    master[i] = w;
    if (WANT_BF16) wbf[i] = muon::f32_to_bf16(w);
  }
}

inline unsigned stream_grid(int64_t work_items, int cus) {
  // enough waves to saturate HBM: up to 8 workgroups of 256 threads per CU
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
                           int nesterov) {
  const bool vec = aligned(grad, 16) && aligned(mom, 16) && aligned(upd, 16);
  const unsigned grid = stream_grid(vec ? (numel + 7) / 8 : numel, cus);
#define MUON_MOM(G, U)                                                                      \
  do {                                                                                      \
    if (vec)                                                                                \
      momentum_kernel<G, U, true><<<grid, 256, 0, s>>>(static_cast<const G*>(grad), mom,    \
                                                       static_cast<U*>(upd), numel, beta,   \
                                                       c1, nesterov);                       \
    else                                                                                    \
      momentum_kernel<G, U, false><<<grid, 256, 0, s>>>(static_cast<const G*>(grad), mom,   \
                                                        static_cast<U*>(upd), numel, beta,  \
                                                        c1, nesterov);                      \
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
  const bool vec = aligned(master, 16) && aligned(upd, 16) && (wbf == nullptr || aligned(wbf, 16));
  const unsigned grid = stream_grid(vec ? (numel + 7) / 8 : numel, cus);
  bf16_t* wb = static_cast<bf16_t*>(wbf);
#define MUON_APPLY(U, V, B)                                                                 \
  apply_kernel<U, V, B><<<grid, 256, 0, s>>>(master, static_cast<const U*>(upd), wb, numel, \
                                             eta, decay, has_wd)
  if (udt == 1) {
    if (vec) { if (wb) MUON_APPLY(bf16_t, true, true); else MUON_APPLY(bf16_t, true, false); }
    else { if (wb) MUON_APPLY(bf16_t, false, true); else MUON_APPLY(bf16_t, false, false); }
  } else {
    if (vec) { if (wb) MUON_APPLY(float, true, true); else MUON_APPLY(float, true, false); }
    else { if (wb) MUON_APPLY(float, false, true); else MUON_APPLY(float, false, false); }
  }
#undef MUON_APPLY
  return hipGetLastError();
}
