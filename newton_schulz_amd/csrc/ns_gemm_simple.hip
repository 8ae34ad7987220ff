// Generic Newton-Schulz products for any shape: the fp32 verification mode
// and bf16 shapes the MFMA path does not take (a dimension not a multiple of
// 8, or unaligned bases).  Same products, epilogues and rounding points as
// the MFMA path; fp32 fused multiply-add accumulation, 64 x 64 tiles, BK 16.
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

template <typename T, bool TM, bool TN, int EPI>
__global__ __launch_bounds__(256) void ns_gemm_simple_kernel(NsGemmArgs a) {
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
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

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
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(x[i], y[j], acc[i][j]);
      }
      __syncthreads();
    }
  }

  float s = 1.0f;
  if (a.scale != nullptr && a.scale_pow > 0) {
    s = a.scale[u];
    if (a.scale_pow == 2) s = s * s;
  }
  T* dst = reinterpret_cast<T*>(mat_at(a.dst, u));
  const T* ep = (EPI == EPI_SYMSQ) ? reinterpret_cast<const T*>(mat_at(a.epi, u)) : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gi = m0 + ty * 4 + i;
    if (gi >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gj = n0 + tx * 4 + j;
      if (gj >= a.N) continue;
      float v = acc[i][j];
      if (EPI == EPI_GRAM) {
        v = s * v;
      } else if (EPI == EPI_SYMSQ) {
        v = a.cb * muon::Elem<T>::load(ep + static_cast<int64_t>(gi) * a.lde + gj) + a.cc * v;
        if (gi == gj) v += a.ca;
      } else {
        v = zero_unit ? 0.0f : s * v;
      }
      if (EPI == EPI_UPDATE) {
        muon::Elem<T>::store(dst + static_cast<int64_t>(gi) * a.ldd + gj, v);
      } else if (ti != tj || gi <= gj) {
        muon::Elem<T>::store(dst + static_cast<int64_t>(gi) * a.ldd + gj, v);
        muon::Elem<T>::store(dst + static_cast<int64_t>(gj) * a.ldd + gi, v);
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
