// The three matrix products of one quintic Newton-Schulz iteration on gfx950
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Per iteration, with X the m x n iterate (m <= n; a tall matrix is kept in
// its own orientation and the products are taken on its transpose):
//   gram   A  = alpha X X^T          upper-triangle tiles only, mirrored
//   symsq  B  = b A + c A A          A is symmetric, so A A = A A^T; upper
//                                    tiles, b A added in the epilogue
//   update X' = beta (a X + B X)     a X read in the epilogue
// alpha = s^2 and beta = s fold the first iteration's normalisation
// X_0 = s Y (s = 1 / (||Y||_F + eps)) into the products, so Y itself is
// never rewritten.  Every product is C = P_M P_N^T with both operands read
// K-contiguous from LDS; an operand stored K-major in memory (the X operand
// of the wide update, both Gram operands of a tall matrix) is transposed on
// its way into LDS (8x8 register transpose), so no transpose pass exists.
//
// Tiling: BM x BN workgroup tile, BK = 64, 256 threads = 4 waves in 2 x 2,
// each wave (BM/2) x (BN/2) as 32 x 32 MFMA tiles.  Double-buffered LDS with
// an XOR swizzle on the 16-byte chunk index; global loads of stage k+1 are
// issued before the MFMAs of stage k.  Workgroup ids are remapped so that each
// XCD (own L2) receives a contiguous run of tiles.
#include "muon_device.h"
#include "muon_internal.h"

using muon::bf16_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int BK = 64;  // bf16 elements of K per stage: one 128-byte LDS row

__device__ __forceinline__ int lds_off(int row, int chunk) {
  const int sw = (row ^ (row >> 3)) & 7;
  return row * 128 + ((chunk ^ sw) << 4);
}

__device__ __forceinline__ uint32_t half_of(const uint4& v, int i) {
  const uint32_t w = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
  return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// Moves one R x BK operand tile global -> registers -> LDS (row-major, K
// contiguous, swizzled).
//   !TRANS: element (r, k) at src[r * ld + k]; thread t owns 16-byte chunk
//           t & 7 of rows (t >> 3) + 32 q.
//   TRANS : element (r, k) at src[k * ld + r]; thread t < R owns the 8 x 8
//           block (k in 8 kb .. 8 kb + 7, r in 8 rb .. 8 rb + 7), loads its 8
//           16-byte rows and writes 8 transposed 16-byte LDS rows.
template <int R, bool TRANS>
struct TileLoader {
  static constexpr int NREG = TRANS ? 8 : R / 32;
  static constexpr int RB = R / 8;
  uint4 r[NREG];

  __device__ __forceinline__ void load(const bf16_t* __restrict__ src, int64_t ld, int row0,
                                       int rows_valid, int k0, int K, int tid) {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    if (!TRANS) {
      const int c = tid & 7;
      const int k = k0 + 8 * c;
#pragma unroll
      for (int q = 0; q < NREG; ++q) {
        const int gr = row0 + (tid >> 3) + 32 * q;
        r[q] = (gr < rows_valid && k < K)
                   ? *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(gr) * ld + k)
                   : z;
      }
    } else {
      if (tid < R) {
        const int rb = tid % RB, kb = tid / RB;
        const int gr = row0 + 8 * rb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int k = k0 + 8 * kb + j;
          r[j] = (k < K && gr < rows_valid)
                     ? *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(k) * ld + gr)
                     : z;
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
    if (!TRANS) {
      const int c = tid & 7;
#pragma unroll
      for (int q = 0; q < NREG; ++q)
        *reinterpret_cast<uint4*>(lds + lds_off((tid >> 3) + 32 * q, c)) = r[q];
    } else {
      if (tid < R) {
        const int rb = tid % RB, kb = tid / RB;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint4 o;
          o.x = half_of(r[0], i) | (half_of(r[1], i) << 16);
          o.y = half_of(r[2], i) | (half_of(r[3], i) << 16);
          o.z = half_of(r[4], i) | (half_of(r[5], i) << 16);
          o.w = half_of(r[6], i) | (half_of(r[7], i) << 16);
          *reinterpret_cast<uint4*>(lds + lds_off(8 * rb + i, kb)) = o;
        }
      }
    }
  }
};

__device__ __forceinline__ void load4_bf16(const bf16_t* p, float v[4]) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(w.x << 16);
  v[1] = __uint_as_float(w.x & 0xffff0000u);
  v[2] = __uint_as_float(w.y << 16);
  v[3] = __uint_as_float(w.y & 0xffff0000u);
}

__device__ __forceinline__ void store4_bf16(bf16_t* p, const float v[4]) {
  uint2 w;
  w.x = muon::pack_bf16x2(v[0], v[1]);
  w.y = muon::pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = w;
}

template <int BM, int BN, bool TM, bool TN, int EPI>
__global__ __launch_bounds__(256, 1) void ns_gemm_mfma_kernel(NsGemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int64_t lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int64_t u = lid / a.tiles_per_unit;
  const int t = static_cast<int>(lid - u * a.tiles_per_unit);
  int ti, tj;
  if (EPI == EPI_UPDATE) {
    ti = t % a.tiles_m;
    tj = t / a.tiles_m;
  } else {
    upper_tile(t, ti, tj);
  }
  const int m0 = ti * BM, n0 = tj * BN;

  const bool zero_unit = a.zflag != nullptr && a.zflag[u] != 0;
  if (zero_unit && !(EPI == EPI_UPDATE && a.zero_write)) return;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = (f32x16_t)(0.0f);

  if (!zero_unit) {
    const bf16_t* pm = reinterpret_cast<const bf16_t*>(mat_at(a.pm, u));
    const bf16_t* pn = reinterpret_cast<const bf16_t*>(mat_at(a.pn, u));
    TileLoader<BM, TM> lm;
    TileLoader<BN, TN> ln;
    const int KT = (a.K + BK - 1) / BK;

    lm.load(pm, a.ldm, m0, a.M, 0, a.K, tid);
    ln.load(pn, a.ldn, n0, a.N, 0, a.K, tid);
    lm.store(smem, tid);
    ln.store(smem + BM * 128, tid);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      char* sm = smem + (kt & 1) * STAGE;
      char* sn = sm + BM * 128;
      const bool more = kt + 1 < KT;
      if (more) {
        lm.load(pm, a.ldm, m0, a.M, (kt + 1) * BK, a.K, tid);
        ln.load(pn, a.ldn, n0, a.N, (kt + 1) * BK, a.K, tid);
      }
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int chunk = 2 * kk + (lane >> 5);
        bf16x8_t fa[FN], fb[FM];
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
          fa[ni] = *reinterpret_cast<const bf16x8_t*>(
              sn + lds_off(wn * WN + ni * 32 + (lane & 31), chunk));
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
          fb[mi] = *reinterpret_cast<const bf16x8_t*>(
              sm + lds_off(wm * WM + mi * 32 + (lane & 31), chunk));
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
          for (int ni = 0; ni < FN; ++ni)
            acc[mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ni], fb[mi], acc[mi][ni], 0, 0, 0);
      }
      if (more) {
        char* nm = smem + ((kt + 1) & 1) * STAGE;
        lm.store(nm, tid);
        ln.store(nm + BM * 128, tid);
      }
      __syncthreads();
    }
  }

  // Epilogue.  MFMA operand A carried the N side, so lane l holds column
  // mm = l % 32 of the 32 x 32 result in MFMA terms = row i of C, and for
  // register group g the four consecutive columns j0 .. j0 + 3 of C.
  float s = 1.0f;
  if (a.scale != nullptr && a.scale_pow > 0) {
    s = a.scale[u];
    if (a.scale_pow == 2) s = s * s;
  }
  bf16_t* dst = reinterpret_cast<bf16_t*>(mat_at(a.dst, u));
  const bf16_t* ep = (EPI == EPI_GRAM) ? nullptr : reinterpret_cast<const bf16_t*>(mat_at(a.epi, u));
#pragma unroll
  for (int mi = 0; mi < FM; ++mi) {
    const int i = m0 + wm * WM + mi * 32 + (lane & 31);
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = n0 + wn * WN + ni * 32 + 8 * g + 4 * (lane >> 5);
        if (i >= a.M || j0 >= a.N) continue;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = acc[mi][ni][4 * g + q];
        if (EPI == EPI_GRAM) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = s * v[q];
        } else if (EPI == EPI_SYMSQ) {
          float e[4];
          load4_bf16(ep + static_cast<int64_t>(i) * a.lde + j0, e);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = a.cb * e[q] + a.cc * v[q];
        } else {
          if (zero_unit) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = 0.0f;
          } else {
            float e[4];
            load4_bf16(ep + static_cast<int64_t>(i) * a.lde + j0, e);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = s * (a.ca * e[q] + v[q]);
          }
        }
        if (EPI == EPI_UPDATE) {
          store4_bf16(dst + static_cast<int64_t>(i) * a.ldd + j0, v);
        } else if (ti != tj) {
          store4_bf16(dst + static_cast<int64_t>(i) * a.ldd + j0, v);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[static_cast<int64_t>(j0 + q) * a.ldd + i] = muon::f32_to_bf16(v[q]);
        } else {
          // diagonal tile: keep the i <= j half and mirror it, so the stored
          // matrix is exactly symmetric
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = j0 + q;
            if (i <= j) {
              const bf16_t h = muon::f32_to_bf16(v[q]);
              dst[static_cast<int64_t>(i) * a.ldd + j] = h;
              dst[static_cast<int64_t>(j) * a.ldd + i] = h;
            }
          }
        }
      }
    }
  }
}

template <int T, bool TM, bool TN, int EPI>
hipError_t go(hipStream_t s, const NsGemmArgs& a) {
  const int64_t grid = a.units * a.tiles_per_unit;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL / 256) return hipErrorInvalidValue;
  ns_gemm_mfma_kernel<T, T, TM, TN, EPI><<<static_cast<unsigned>(grid), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int T>
hipError_t dispatch(hipStream_t s, const NsGemmArgs& a, int epi, bool tm, bool tn) {
  if (epi == EPI_GRAM && !tm && !tn) return go<T, false, false, EPI_GRAM>(s, a);
  if (epi == EPI_GRAM && tm && tn) return go<T, true, true, EPI_GRAM>(s, a);
  if (epi == EPI_SYMSQ && !tm && !tn) return go<T, false, false, EPI_SYMSQ>(s, a);
  if (epi == EPI_UPDATE && !tm && tn) return go<T, false, true, EPI_UPDATE>(s, a);
  if (epi == EPI_UPDATE && !tm && !tn) return go<T, false, false, EPI_UPDATE>(s, a);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_ns_gemm_mfma(hipStream_t s, const NsGemmArgs& a, int epi, bool trans_m,
                               bool trans_n, int tile) {
  if (tile == 256) return dispatch<256>(s, a, epi, trans_m, trans_n);
  if (tile == 128) return dispatch<128>(s, a, epi, trans_m, trans_n);
  return hipErrorInvalidValue;
}
