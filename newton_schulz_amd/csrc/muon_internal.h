// Host-side declarations of the kernel launchers inside libmuon.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon.h"
#include "muon_device.h"

// Epilogue kinds of the Newton-Schulz matrix products.
enum NsEpi : int {
  EPI_GRAM = 0,    // A = alpha * (P P^T), upper tiles, mirrored
  EPI_SYMSQ = 1,   // B = b * A + c * (A A), upper tiles, mirrored
  EPI_UPDATE = 2   // X' = beta * (a * X + acc), all tiles
};

// One batched product C = op(P_M) op(P_N)^T over `units` independent units.
// P_M supplies the rows of C (M of them), P_N its columns (N), K is the
// contraction length.  trans_m / trans_n: the operand is stored K-major
// (element (r, k) at k * ld + r) instead of K-contiguous (r * ld + k).  dst
// receives C row-major.
struct NsGemmArgs {
  MatRef pm, pn, dst;
  MatRef epi;                  // EPI_SYMSQ: the matrix A of the b A term
  int64_t ldm, ldn, ldd, lde;  // leading dimensions in elements
  int M, N, K;
  int tiles_m, tiles_n, tiles_per_unit;
  int64_t units;
  int cus;             // compute units of the device (persistent grid size)
  const float* scale;  // per-unit normalisation factor s, or nullptr
  int scale_pow;       // 0: not applied, 1: multiply by s, 2: by s*s
  const int* zflag;    // per-unit "norm is zero" flag, or nullptr
  int zero_write;      // EPI_UPDATE: write zeros for zero units (last iteration)
  float ca, cb, cc;    // quintic coefficients a, b, c
  // Iterate carried past bf16 (ns_diag_residual, ns_lo_term).  EPI_SYMSQ:
  // dvec, when set, receives B's diagonal in fp32 before rounding (K floats
  // per unit, unit u at u * K).  EPI_UPDATE: dvec set = complete the
  // diagonal (the MFMA kernel reads the iterate at the output position from
  // its own k-stages, the generic kernel through epi / lde); lo_in = the
  // input's residual plane (nullptr: the input is exact in bf16), lo_out =
  // receives the output's residual (nullptr: not kept).  The MFMA kernel
  // keeps residuals in its own tile-major order (tile lid at lid * BM * BN *
  // 2 bytes, each lane's values contiguous); the generic kernel row-major.
  float* dvec;
  const char* lo_in;
  char* lo_out;
  // Only the units listed: ulist[0 .. *ucount) are unit indices in ascending
  // order (the nonzero ones, launch_compact_units), and the tiles are those
  // of the listed units, so a zero unit takes no tile slot; nullptr: every
  // unit.  The residual plane is indexed by the listed tile number, so every
  // product that reads or writes it must see the same list.
  const int* ulist;
  const int* ucount;
};

struct NsNormArgs {
  MatRef in;
  int64_t unit_elems;
  int64_t units;
  int parts;           // partial sums per unit
  double* partial;     // [units][parts]
  float* scale;        // [units] : 1 / (||Y||_F + eps)
  int* zflag;          // [units] : ||Y||_F == 0
  int* nonfinite;      // device flag or nullptr
  float eps;
  // norms from momentum partials instead of a pass over `in`: unit u's blocks
  // start at (address of unit u - sq_base) / block_bytes
  const double* sq;    // or nullptr
  const char* sq_base;
  int64_t block_bytes;
  int64_t blocks_per_unit;
};

// The whole iteration (quintic, or its Gram form) of wide units with
// m <= 128 in one launch (ns_small.hip): src = the units Y (m x n, rows
// contiguous), dst = the result, xa / xb = two iterate regions of m x n per
// unit (quintic only).
struct NsSmallArgs {
  MatRef src, dst, xa, xb;
  int m, n, steps;
  int gram;            // 1: Gram form (m x m iteration, then X = s Q Y)
  int64_t units;
  const float* scale;  // per-unit s = 1 / (||Y||_F + eps)
  const int* zflag;    // per-unit "norm is zero" flag, or nullptr
  float* dvec;         // quintic: B's fp32 diagonal, m floats per unit
  char* lo;            // quintic: residual planes, nb 32 KiB blocks per unit
  int ncoef;           // rows of coef: iteration k uses row min(k, ncoef - 1)
  float coef[MUON_NS_FUSED_MAX_ROWS][3];  // (a, b, c) per iteration
};

hipError_t launch_ns_small(hipStream_t s, const NsSmallArgs& a);

hipError_t launch_momentum(hipStream_t s, int cus, const void* grad, int gdt, float* mom,
                           void* upd, int udt, int64_t numel, float beta, float c1,
                           int nesterov, double* sq);
hipError_t launch_apply(hipStream_t s, int cus, float* master, const void* upd, int udt,
                        void* wbf, int64_t numel, float eta, float decay, int has_wd);

hipError_t launch_norm(hipStream_t s, const NsNormArgs& a, int io_bf16, bool vec);
// list[0 .. *count) = the units u < units with zflag[u] == 0, ascending.
hipError_t launch_compact_units(hipStream_t s, const int* zflag, int64_t units, int* list, int* count);
// out[u] = s[u] * in[u], element-wise over units of unit_elems (steps == 0, copies).
hipError_t launch_scale_copy(hipStream_t s, MatRef in, MatRef out, int64_t unit_elems,
                             int64_t units, const float* scale, int io_bf16);
// The same, read as bf16 or fp32 (in_bf16) and stored as bf16 (rounded to
// nearest even) or fp32 (out_bf16); scale may be null (factor 1).
hipError_t launch_convert(hipStream_t s, MatRef in, int in_bf16, MatRef out, int out_bf16,
                          int64_t unit_elems, int64_t units, const float* scale);

// bf16 MFMA path (all of M, N, K, leading dims multiples of 8; 16-byte aligned
// bases; each operand smaller than 2 GiB).  tile: 128 or 256.
hipError_t launch_ns_gemm_mfma(hipStream_t s, const NsGemmArgs& a, int epi, bool trans_m,
                               bool trans_n, int tile);
// Generic path (any sizes; fp32 or bf16 storage, fp32 FMA accumulation).
hipError_t launch_ns_gemm_simple(hipStream_t s, const NsGemmArgs& a, int epi, bool trans_m,
                                 bool trans_n, int io_bf16);

// Tile bookkeeping shared by host and device.
__host__ __device__ __forceinline__ void upper_tile(int t, int& ti, int& tj) {
  // Column-wise enumeration of the upper triangle: t = tj*(tj+1)/2 + ti, ti <= tj.
  int j = static_cast<int>((sqrtf(8.0f * static_cast<float>(t) + 1.0f) - 1.0f) * 0.5f);
  while (j * (j + 1) / 2 > t) --j;
  while ((j + 1) * (j + 2) / 2 <= t) ++j;
  tj = j;
  ti = t - j * (j + 1) / 2;
}

// Where one batched Newton-Schulz call runs: a context's slab, or (ctx null)
// the allocation-free entry point's static scratch.  outputs_in_place (ctx
// null only): every output is its own input or all outputs are disjoint from
// every input, as that entry point checks before the call.
struct muon_ctx;
struct NsEnv {
  muon_ctx* ctx = nullptr;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  int cus = 256;
  int device = 0;
  bool outputs_in_place = false;
  const char** err = nullptr;  // receives a static error text (ctx null)
};
muon_status_t ns_batched(const NsEnv& env, void* stream, const void* const* mats, int64_t count,
                         muon_shape_t shape, int32_t io_dtype, const muon_ns_params_t* prm,
                         void* const* out, int* nonfinite_flag);

// Which updates of a `steps`-iteration call keep the iterate's residual: it
// is written by updates 0 .. steps - 3 and read by the update after each.
__host__ __device__ __forceinline__ bool ns_lo_written(int k, int steps) { return k + 3 <= steps; }
__host__ __device__ __forceinline__ bool ns_lo_read(int k, int steps) { return k >= 1 && k + 2 <= steps; }
