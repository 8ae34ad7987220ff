// Generic Newton-Schulz products for any shape: the fp32 verification mode
// and bf16 shapes the MFMA path does not take (a dimension not a multiple of
// 8, or unaligned bases).  Same products, epilogues and rounding points as
// the MFMA path; 64 x 64 tiles, BK 16, fused multiply-add accumulation.
// bf16 storage accumulates in fp32 (as the matrix cores do).  The fp32 mode
// stores every matrix in fp32 but accumulates and finishes each product in
// fp64: the iteration lifts singular values near the storage precision by up
// to a^steps, and with fp32 sums over fp32 data nothing is left to resolve
// them (an exactly rank-1 fp32 input then misses 1e-4 relative error; with
// fp64 sums it stays near 4e-6).
#include <type_traits>

#include "muon_device.h"
#include "muon_internal.h"

using muon::bf16_t;

namespace {

constexpr int TS = 64;
constexpr int BKS = 16;

template <typename T, bool TRANS>
__device__ __forceinline__ void stage(float (*sh)[TS + 4], const T* __restrict__ src, int64_t ld,
                                      int row0, int rows_valid, int k0, int K, int tid) {
  // 64 rows x 16 k; K-contiguous sources are read along k, K-major along r.
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 256 * q;
    int r, kk;
    if (TRANS) { r = e % TS; kk = e / TS; }
    else { kk = e % BKS; r = e / BKS; }
    const int gr = row0 + r, gk = k0 + kk;
    float v = 0.0f;
    if (gr < rows_valid && gk < K)
      v = muon::Elem<T>::load(TRANS ? src + static_cast<int64_t>(gk) * ld + gr
                                    : src + static_cast<int64_t>(gr) * ld + gk);
    sh[kk][r] = v;
  }
}

__device__ __forceinline__ float fma_acc(float x, float y, float c) { return __builtin_fmaf(x, y, c); }
__device__ __forceinline__ double fma_acc(float x, float y, double c) {
  return __builtin_fma(static_cast<double>(x), static_cast<double>(y), c);
}

template <typename T, bool TM, bool TN, int EPI>
__global__ __launch_bounds__(256) void ns_gemm_simple_kernel(NsGemmArgs a) {
  using Acc = std::conditional_t<std::is_same<T, float>::value, double, float>;
  __shared__ float sM[BKS][TS + 4];
  __shared__ float sN[BKS][TS + 4];
  const int tid = threadIdx.x;
  const int64_t lid = blockIdx.x;
  const int64_t u = lid / a.tiles_per_unit;
  const int t = static_cast<int>(lid - u * a.tiles_per_unit);
  int ti, tj;
  if (EPI == EPI_UPDATE) {
    ti = t % a.tiles_m;
    tj = t / a.tiles_m;
  } else {
    upper_tile(t, ti, tj);
  }
  const int m0 = ti * TS, n0 = tj * TS;
  const bool zero_unit = a.zflag != nullptr && a.zflag[u] != 0;
  if (zero_unit && !(EPI == EPI_UPDATE && a.zero_write)) return;

  const int ty = tid / 16, tx = tid % 16;
  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = Acc(0);

  if (!zero_unit) {
    const T* pm = reinterpret_cast<const T*>(mat_at(a.pm, u));
    const T* pn = reinterpret_cast<const T*>(mat_at(a.pn, u));
    for (int k0 = 0; k0 < a.K; k0 += BKS) {
      stage<T, TM>(sM, pm, a.ldm, m0, a.M, k0, a.K, tid);
      stage<T, TN>(sN, pn, a.ldn, n0, a.N, k0, a.K, tid);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BKS; ++kk) {
        float x[4], y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = sM[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = sN[kk][tx * 4 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fma_acc(x[i], y[j], acc[i][j]);
      }
      __syncthreads();
    }
  }

  Acc s = Acc(1);
  if (a.scale != nullptr && a.scale_pow > 0) {
    s = a.scale[u];
    if (a.scale_pow == 2) s = s * s;
  }
  T* dst = reinterpret_cast<T*>(mat_at(a.dst, u));
  // the corrected bf16 update (ns_diag_residual, ns_lo_term) reads the source at the
  // output position through epi and keeps its residual row-major, M x N per
  // unit; never for a zero unit (its workspace was never filled)
  const bool corr = EPI == EPI_UPDATE && a.dvec != nullptr && !zero_unit;
  const T* ep = (EPI == EPI_SYMSQ || corr) ? reinterpret_cast<const T*>(mat_at(a.epi, u)) : nullptr;
  const int64_t plane = u * static_cast<int64_t>(a.M) * a.N;
  const bf16_t* lo_in = reinterpret_cast<const bf16_t*>(a.lo_in);
  bf16_t* lo_out = reinterpret_cast<bf16_t*>(a.lo_out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gi = m0 + ty * 4 + i;
    if (gi >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gj = n0 + tx * 4 + j;
      if (gj >= a.N) continue;
      Acc v = acc[i][j];
      if (EPI == EPI_GRAM) {
        v = s * v;
      } else if (EPI == EPI_SYMSQ) {
        v = Acc(a.cb) * Acc(muon::Elem<T>::load(ep + static_cast<int64_t>(gi) * a.lde + gj)) + Acc(a.cc) * v;
        if (gi == gj) {
          v += Acc(a.ca);
          if (a.dvec != nullptr) a.dvec[u * static_cast<int64_t>(a.M) + gi] = static_cast<float>(v);
        }
      } else {
        if (corr) {
          // d per row for X' = B'X (the K-major X operand), per column for Y' = YB'
          const float d = a.dvec[u * static_cast<int64_t>(a.K) + (TN ? gi : gj)];
          const float hi = muon::Elem<T>::load(ep + static_cast<int64_t>(gi) * a.lde + gj);
          const int64_t e = plane + static_cast<int64_t>(gi) * a.N + gj;
          const float lo = lo_in ? muon::bf16_to_f32(lo_in[e]) : 0.0f;
          float w = static_cast<float>(v) + muon::ns_diag_residual(d) * hi;
          if (lo_in) w = muon::ns_lo_term(w, d, lo);
          v = w;
        }
        v = zero_unit ? Acc(0) : s * v;
        if (corr && lo_out) {
          const float f = static_cast<float>(v);
          lo_out[plane + static_cast<int64_t>(gi) * a.N + gj] = muon::f32_to_bf16(f - muon::bf16_round(f));
        }
      }
      if (EPI == EPI_UPDATE) {
        muon::Elem<T>::store(dst + static_cast<int64_t>(gi) * a.ldd + gj, static_cast<float>(v));
      } else if (ti != tj || gi <= gj) {
        muon::Elem<T>::store(dst + static_cast<int64_t>(gi) * a.ldd + gj, static_cast<float>(v));
        muon::Elem<T>::store(dst + static_cast<int64_t>(gj) * a.ldd + gi, static_cast<float>(v));
      }
    }
  }
}

template <typename T, bool TM, bool TN, int EPI>
hipError_t go(hipStream_t s, const NsGemmArgs& a) {
  const int64_t grid = a.units * a.tiles_per_unit;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL / 256) return hipErrorInvalidValue;
  ns_gemm_simple_kernel<T, TM, TN, EPI><<<static_cast<unsigned>(grid), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(hipStream_t s, const NsGemmArgs& a, int epi, bool tm, bool tn) {
  if (epi == EPI_GRAM && !tm && !tn) return go<T, false, false, EPI_GRAM>(s, a);
  if (epi == EPI_GRAM && tm && tn) return go<T, true, true, EPI_GRAM>(s, a);
  if (epi == EPI_SYMSQ && !tm && !tn) return go<T, false, false, EPI_SYMSQ>(s, a);
  if (epi == EPI_UPDATE && !tm && tn) return go<T, false, true, EPI_UPDATE>(s, a);
  if (epi == EPI_UPDATE && !tm && !tn) return go<T, false, false, EPI_UPDATE>(s, a);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ns_gemm_simple(hipStream_t s, const NsGemmArgs& a, int epi, bool trans_m,
                                 bool trans_n, int io_bf16) {
  if (io_bf16) return dispatch<bf16_t>(s, a, epi, trans_m, trans_n);
  return dispatch<float>(s, a, epi, trans_m, trans_n);
}
