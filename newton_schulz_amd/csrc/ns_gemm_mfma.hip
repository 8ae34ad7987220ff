// The three matrix products of one quintic Newton-Schulz iteration on gfx950
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// The iterate X (m x n, m <= n) is kept in two layouts: R = X row-major and
// T = X^T row-major.  With them every product reads both operands along a
// contiguous K:
//   gram   A  = alpha X X^T        P_M = P_N = R (K = n); upper tiles, mirrored
//   symsq  B  = b A + c A A        P_M = P_N = A (A symmetric, so A A = A A^T)
//   update X' = beta (a X + B X)   P_M = B (K = m), P_N = T (row j of T is
//                                  column j of X); a X read from R; X' stored
//                                  as R and/or T
// alpha = s^2 and beta = s fold the first iteration's normalisation
// X_0 = s Y (s = 1 / (||Y||_F + eps)) into the products.
//
// Tiling: BM x BN workgroup tile, BK = 64, 256 threads = 4 waves in 2 x 2,
// each wave (BM/2) x (BN/2) as 32 x 32 MFMA tiles.  Operand tiles move
// global -> LDS with buffer_load_dwordx4 ... lds (no registers): each wave
// instruction fills 8 LDS rows of 128 bytes, lane l writing 16 bytes at
// 16 l, so each lane fetches the global chunk that the XOR swizzle places
// there.  Chunks outside the matrix get an offset past the buffer's size and
// the hardware returns zeros.  Two LDS stages: the loads of stage k+1 are in
// flight while stage k feeds the MFMAs.  Workgroup ids are remapped so that
// each XCD (own L2) gets a contiguous run of tiles.
#include "muon_device.h"
#include "muon_internal.h"

#include <utility>

using muon::bf16_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

namespace {

constexpr int BK = 64;                 // bf16 elements of K per stage: one 128-byte LDS row
constexpr uint32_t kOOB = 0x80000000u; // buffer offset past any matrix: loads return 0
constexpr int kRsrcWord3 = 0x00020000; // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ swz(row)) << 4);
}

// A pointer every lane holds the same value of, moved to scalar registers
// (needed for buffer descriptors; a value read from a device table is not
// known to be uniform otherwise).
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

// Per-lane addressing of one operand tile of R rows (R/8 row groups of 8 LDS
// rows; wave w issues groups w, w + 4, ...).
template <int R>
struct OperandStream {
  static constexpr int NG = R / 32;  // row groups per wave
  uint32_t base[NG];                 // byte offset of this lane's chunk at k = 0, or kOOB
  __amdgpu_buffer_rsrc_t rsrc;

  // src: rows x ld bf16 matrix; the tile covers rows [row0, row0 + R).
  __device__ __forceinline__ void init(const bf16_t* src, int64_t ld, int rows, int row0, int wave,
                                       int lane) {
    rsrc = make_rsrc(src, static_cast<uint32_t>(static_cast<int64_t>(rows) * ld * 2));
    const int rin = lane >> 3;  // row within the group (0..7)
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int row = 8 * (wave + 4 * q) + rin;
      const int gr = row0 + row;
      const int lc = (lane & 7) ^ swz(row);  // logical chunk stored at LDS chunk lane & 7
      base[q] = (gr < rows) ? static_cast<uint32_t>((static_cast<int64_t>(gr) * ld + 8 * lc) * 2)
                            : kOOB;
    }
  }

  // Issue the loads of K slice [k0, k0 + BK) into the LDS tile at `lds`.
  __device__ __forceinline__ void issue(char* lds, int k0, int K, int wave, int lane) {
    const int rin = lane >> 3;
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int g = wave + 4 * q;
      const int row = 8 * g + rin;
      const int lc = (lane & 7) ^ swz(row);
      const bool ok = base[q] != kOOB && (k0 + 8 * lc) < K;
      const uint32_t off = ok ? base[q] + static_cast<uint32_t>(k0 * 2) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + g * 1024), 16,
                                               off, 0, 0, 0);
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

// Finish four consecutive outputs C[i][j0 .. j0 + 3] held by one lane.
template <int EPI>
__device__ __forceinline__ void epilogue_group(const NsGemmArgs& a, float v[4], int i, int j0,
                                               float s, bool zero_unit, bool diag,
                                               const bf16_t* ep, bf16_t* dst, bf16_t* dstt) {
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
    if (dst) store4_bf16(dst + static_cast<int64_t>(i) * a.ldd + j0, v);
    if (dstt) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dstt[static_cast<int64_t>(j0 + q) * a.ldt + i] = muon::f32_to_bf16(v[q]);
    }
  } else if (!diag) {
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

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256, 1) void ns_gemm_mfma_kernel(NsGemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    OperandStream<BM> sm_;
    OperandStream<BN> sn_;
    sm_.init(uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.pm, u))), a.ldm, a.M, m0, wave, lane);
    sn_.init(uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.pn, u))), a.ldn, a.N, n0, wave, lane);
    const int KT = (a.K + BK - 1) / BK;

    sm_.issue(smem, 0, a.K, wave, lane);
    sn_.issue(smem + BM * 128, 0, a.K, wave, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    auto compute = [&](const char* sm) {
      const char* sn = sm + BM * 128;
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
    };
    // steady state without branches: stage kt + 1 loads while stage kt computes
    for (int kt = 0; kt < KT - 1; ++kt) {
      char* nm = smem + ((kt + 1) & 1) * STAGE;
      sm_.issue(nm, (kt + 1) * BK, a.K, wave, lane);
      sn_.issue(nm + BM * 128, (kt + 1) * BK, a.K, wave, lane);
      compute(smem + (kt & 1) * STAGE);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    compute(smem + ((KT - 1) & 1) * STAGE);
  }

  // Epilogue.  MFMA operand A carried the N side, so lane l holds row
  // i = m0 + ... + l % 32 of C and, per register group g, the four
  // consecutive columns j0 .. j0 + 3.
  float s = 1.0f;
  if (a.scale != nullptr && a.scale_pow > 0) {
    s = a.scale[u];
    if (a.scale_pow == 2) s = s * s;
  }
  bf16_t* dst = a.dst.base || a.dst.table ? uniform_ptr(reinterpret_cast<bf16_t*>(mat_at(a.dst, u))) : nullptr;
  bf16_t* dstt = a.dst_t.base || a.dst_t.table ? uniform_ptr(reinterpret_cast<bf16_t*>(mat_at(a.dst_t, u))) : nullptr;
  const bf16_t* ep = (EPI == EPI_GRAM) ? nullptr : uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.epi, u)));
  const bool diag = (EPI != EPI_UPDATE) && ti == tj;
  static_for<FM>([&](auto MI) {
    constexpr int mi = decltype(MI)::value;
    const int i = m0 + wm * WM + mi * 32 + (lane & 31);
    static_for<FN>([&](auto NI) {
      constexpr int ni = decltype(NI)::value;
      static_for<4>([&](auto G) {
        constexpr int g = decltype(G)::value;
        const int j0 = n0 + wn * WN + ni * 32 + 8 * g + 4 * (lane >> 5);
        float v[4] = {acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2],
                      acc[mi][ni][4 * g + 3]};
        if (i < a.M && j0 < a.N)
          epilogue_group<EPI>(a, v, i, j0, s, zero_unit, diag, ep, dst, dstt);
      });
    });
  });
}

template <int T, int EPI>
hipError_t go(hipStream_t s, const NsGemmArgs& a) {
  const int64_t grid = a.units * a.tiles_per_unit;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL / 256) return hipErrorInvalidValue;
  ns_gemm_mfma_kernel<T, T, EPI><<<static_cast<unsigned>(grid), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int T>
hipError_t dispatch(hipStream_t s, const NsGemmArgs& a, int epi) {
  if (epi == EPI_GRAM) return go<T, EPI_GRAM>(s, a);
  if (epi == EPI_SYMSQ) return go<T, EPI_SYMSQ>(s, a);
  if (epi == EPI_UPDATE) return go<T, EPI_UPDATE>(s, a);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Prep: transpose Y into the missing layout and reduce its Frobenius norm.
// One 64 x 64 tile per workgroup; squares summed exactly in fp64 per tile,
// then per unit in a fixed order (deterministic).
// ---------------------------------------------------------------------------
constexpr int PT = 64;

__global__ __launch_bounds__(256) void prep_kernel(MatRef in, MatRef outT, int rows, int cols,
                                                   int tiles_r, int tiles_c, double* partial) {
  __shared__ uint16_t tile[PT][PT + 8];
  __shared__ double red[256];
  const int64_t u = blockIdx.y;
  const int t = blockIdx.x;
  const int tr = t % tiles_r, tc = t / tiles_r;
  const int r0 = tr * PT, c0 = tc * PT;
  const bf16_t* src = reinterpret_cast<const bf16_t*>(mat_at(in, u));
  bf16_t* dst = reinterpret_cast<bf16_t*>(mat_at(outT, u));
  const int tid = threadIdx.x;
  double acc = 0.0;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + 256 * q;  // 512 chunks of 8 elements: 64 rows x 8 chunks
    const int r = e >> 3, c = (e & 7) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + r < rows && c0 + c < cols)
      v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(r0 + r) * cols + c0 + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo = __uint_as_float(w[k] << 16), hi = __uint_as_float(w[k] & 0xffff0000u);
      acc += static_cast<double>(lo * lo);
      acc += static_cast<double>(hi * hi);
      tile[r][c + 2 * k] = static_cast<uint16_t>(w[k] & 0xffffu);
      tile[r][c + 2 * k + 1] = static_cast<uint16_t>(w[k] >> 16);
    }
  }
  red[tid] = acc;
  __syncthreads();
  // transposed write: out row (c0 + c) holds column c of the tile
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = tid + 256 * q;
    const int c = e >> 3, r = (e & 7) * 8;
    if (c0 + c < cols && r0 + r < rows) {
      uint4 o;
      o.x = tile[r + 0][c] | (static_cast<uint32_t>(tile[r + 1][c]) << 16);
      o.y = tile[r + 2][c] | (static_cast<uint32_t>(tile[r + 3][c]) << 16);
      o.z = tile[r + 4][c] | (static_cast<uint32_t>(tile[r + 5][c]) << 16);
      o.w = tile[r + 6][c] | (static_cast<uint32_t>(tile[r + 7][c]) << 16);
      *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(c0 + c) * rows + r0 + r) = o;
    }
  }
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) partial[u * (static_cast<int64_t>(tiles_r) * tiles_c) + t] = red[0];
}

__global__ __launch_bounds__(256) void prep_finalize_kernel(const double* partial, int parts,
                                                            float* scale, int* zflag,
                                                            int* nonfinite, float eps) {
  __shared__ double red[256];
  const int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (int p = tid; p < parts; p += 256) acc += partial[u * parts + p];
  red[tid] = acc;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    const double sq = red[0];
    scale[u] = static_cast<float>(1.0 / (sqrt(sq) + static_cast<double>(eps)));
    zflag[u] = (sq == 0.0) ? 1 : 0;
    if (nonfinite && !isfinite(sq)) atomicOr(nonfinite, 1);
  }
}

}  // namespace

hipError_t launch_ns_gemm_mfma(hipStream_t s, const NsGemmArgs& a, int epi, int tile) {
  if (tile == 256) return dispatch<256>(s, a, epi);
  if (tile == 128) return dispatch<128>(s, a, epi);
  return hipErrorInvalidValue;
}

int prep_parts(int rows, int cols) { return ((rows + PT - 1) / PT) * ((cols + PT - 1) / PT); }

hipError_t launch_prep(hipStream_t s, MatRef in, MatRef outT, int rows, int cols, int64_t units,
                       double* partial, float* scale, int* zflag, int* nonfinite, float eps) {
  const int tr = (rows + PT - 1) / PT, tc = (cols + PT - 1) / PT;
  constexpr int64_t kMaxY = 65535;
  for (int64_t u0 = 0; u0 < units; u0 += kMaxY) {
    const int64_t n = (units - u0 < kMaxY) ? units - u0 : kMaxY;
    MatRef i0 = in, o0 = outT;
    if (i0.table) i0.table += u0; else i0.base += u0 * i0.stride;
    if (o0.table) o0.table += u0; else o0.base += u0 * o0.stride;
    double* p0 = partial + u0 * static_cast<int64_t>(tr) * tc;
    prep_kernel<<<dim3(static_cast<unsigned>(tr * tc), static_cast<unsigned>(n)), 256, 0, s>>>(
        i0, o0, rows, cols, tr, tc, p0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    prep_finalize_kernel<<<static_cast<unsigned>(n), 256, 0, s>>>(p0, tr * tc, scale + u0,
                                                                   zflag + u0, nonfinite, eps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
