// The whole quintic Newton-Schulz iteration of units with m <= 128 in one
// launch (bf16 MFMA, fp32 accumulation), e.g. the per-head 128 x 2560 q/k/v
// matrices of per-head Muon.
//
// One workgroup owns one unit for all iterations: 8 waves, 2 x 4 over a
// 128 x 128 output, 64 x 32 each; every 32 x 32 accumulator takes the
// operands of the 128 x 128 tiles of the separate product launches in their
// order.  A and B' stay in LDS as bf16; the m x n
// iterate streams through LDS in 128-column blocks.  With X_0 = s Y
// (s = 1 / (||Y||_F + eps)) folded into the first products:
//   A_0 = s^2 Y Y^T                          one pass over the input
//   per iteration k:
//     B' = a I + b A_k + c A_k A_k           K = 128, from LDS
//     per column block j:  X'_j = f B' X_j   (f = s when k = 0, else 1)
//                          store X'_j;  A_{k+1} += X'_j X'_j^T
// The Gram product of the next iteration is accumulated from the bf16 block
// just stored, so each iteration reads the iterate once and writes it once
// (separate launches read it twice), and no product pays a launch and a
// tile prologue of its own.  Rounding points (A, B', every iterate in bf16),
// the MFMA shape and the order of every sum are those of the separate
// launches; A and B' take their lower triangle from the upper one as the
// mirrored tiles there do.
//
// Units are wide (m = rows <= n = cols), rows contiguous (ld = n), with
// m % 8 == n % 8 == 0; rows past m and columns past n read as zeros.
#include "ns_mfma_common.h"

namespace {

constexpr int SM = 128;            // rows and columns of A and B' (m padded)
constexpr int NWV = 8;             // waves: 2 along the rows x NWV / 2 along the columns
constexpr int WNC = SM / (NWV / 2);   // output columns per wave
constexpr int FN = WNC / 32;          // 32-column accumulator blocks per wave
constexpr int HALF = SM * 64 * 2;  // one 64-k half of a 128-row K-contiguous tile
constexpr int SLAB = SM * SM * 2;  // a 128 x 128 bf16 block
constexpr int NGR = SM / (8 * NWV);   // row-slab DMA instructions per wave (128 rows x 64 k)
constexpr int NGC = SM / (4 * NWV);   // column-block DMA instructions per wave (128 k x 128 cols)
constexpr int NST = SM * SM / 8 / (64 * NWV);  // 16-byte stores per lane per block

// Element (i, j) of a 128 x 128 bf16 matrix kept as two 64-column halves in
// the K-contiguous tile layout (columns are the contraction index).
__device__ __forceinline__ char* rt_at(char* t, int i, int j) {
  return t + (j >> 6) * HALF + rt_off<64>(i, (j & 63) >> 3) + ((j & 7) << 1);
}

// MFMA operand: rows rb .. rb + 31, k = 16 kk + 8 (lane / 32) + 0..7, kk < 8
__device__ __forceinline__ bf16x8_t rt_frag(const char* t, int rb, int kk, int lane) {
  return *reinterpret_cast<const bf16x8_t*>(t + (kk >> 2) * HALF +
                                            rt_off<64>(rb + (lane & 31), 2 * (kk & 3) + (lane >> 5)));
}

// MFMA operand from a K-major 128 x 128 block (k = memory row): columns
// rb .. rb + 31, four consecutive k per ds_read_b64_tr_b16, kk < 8
__device__ __forceinline__ bf16x8_t kt_frag(const char* t, int rb, int kk, int lane) {
  const int gq = lane >> 4, j = lane & 15;
  const int col = rb + 16 * (gq & 1) + 4 * (j & 3);
  const int k = 16 * kk + 8 * (gq >> 1) + (j >> 2);
  const u32x2_t lo = __builtin_bit_cast(u32x2_t, ld_tr16(t + kt_off<SM>(k, col)));
  const u32x2_t hi = __builtin_bit_cast(u32x2_t, ld_tr16(t + kt_off<SM>(k + 4, col)));
  const u32x4_t v = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8_t, v);
}

struct Acc {
  f32x16_t v[2][FN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) v[mi][ni] = (f32x16_t)(0.0f);
  }
  // acc += P_M P_N^T over one k16 step; fa: N side, fb: M side
  __device__ __forceinline__ void mma(const bf16x8_t (&fa)[FN], const bf16x8_t (&fb)[2]) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < FN; ++ni)
        v[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ni], fb[mi], v[mi][ni], 0, 0, 0);
  }
};

// Lane l holds row wm 64 + mi 32 + l % 32 and, per register group g, columns
// wn WNC + ni 32 + 8 g + 4 (l / 32) + 0..3 of the accumulated product.
template <typename F>
__device__ __forceinline__ void for_acc(int wm, int wn, int lane, F&& f) {
  static_for<2>([&](auto MI) {
    static_for<FN>([&](auto NI) {
      static_for<4>([&](auto G) {
        constexpr int mi = decltype(MI)::value, ni = decltype(NI)::value, g = decltype(G)::value;
        f(mi, ni, g, wm * 64 + mi * 32 + (lane & 31), wn * WNC + ni * 32 + 8 * g + 4 * (lane >> 5));
      });
    });
  });
}

__device__ __forceinline__ uint2 pack4(const float (&v)[4]) {
  uint2 w;
  w.x = muon::pack_bf16x2(v[0], v[1]);
  w.y = muon::pack_bf16x2(v[2], v[3]);
  return w;
}

// lower triangle <- upper triangle (the mirrored tiles of separate launches)
__device__ __forceinline__ void mirror_lower(char* t, int tid) {
  for (int e = tid; e < SM * SM; e += 64 * NWV) {
    const int i = e >> 7, j = e & (SM - 1);
    if (i > j) *reinterpret_cast<uint16_t*>(rt_at(t, i, j)) = *reinterpret_cast<const uint16_t*>(rt_at(t, j, i));
  }
}

__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool GRAM>
__global__ __launch_bounds__(64 * NWV, 1) void ns_small_kernel(NsSmallArgs a) {
  __shared__ __attribute__((aligned(1024))) char bp[2 * HALF];  // B'
  __shared__ __attribute__((aligned(1024))) char am[2 * HALF];  // A; the X' block staging
  __shared__ __attribute__((aligned(1024))) char s0[SLAB];      // iterate blocks / row slabs
  __shared__ __attribute__((aligned(1024))) char s1[SLAB];
  __shared__ __attribute__((aligned(1024))) char s2[SLAB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NWV / 2), wn = wave % (NWV / 2);
  const int64_t u = blockIdx.x;
  const int m = a.m, n = a.n;
  const uint32_t ubytes = static_cast<uint32_t>(static_cast<int64_t>(m) * n * 2);
  const int nb = (n + SM - 1) / SM;  // column blocks

  // 16-byte row-contiguous stores of one 128 x 128 block (zeros when src_tile
  // is null); chunks outside the unit get an offset the hardware drops
  auto store_block = [&](const bf16_t* dst, int c0, const char* src_tile) {
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(dst, ubytes);
#pragma unroll
    for (int it = 0; it < NST; ++it) {
      const int e = tid + 64 * NWV * it;
      const int row = e >> 4, ch = e & 15;
      const u32x4_t val = src_tile ? *reinterpret_cast<const u32x4_t*>(src_tile + (ch >> 3) * HALF +
                                                                        rt_off<64>(row, ch & 7))
                                   : u32x4_t{0u, 0u, 0u, 0u};
      const uint32_t off = (row < m && c0 + 8 * ch < n)
                               ? static_cast<uint32_t>((static_cast<int64_t>(row) * n + c0 + 8 * ch) * 2)
                               : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(val, dr, off, 0, 0);
    }
  };

  const bf16_t* y = uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.src, u)));
  const bf16_t* out = uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.dst, u)));
  if (a.zflag != nullptr && a.zflag[u] != 0) {  // a zero unit's result is exactly zero
    for (int c = 0; c < nb; ++c) store_block(out, c * SM, nullptr);
    return;
  }
  const float s = a.scale[u];

  // ---- A_0 = s^2 Y Y^T: 128-row x 64-k slabs of Y, two stage buffers
  {
    const u32x4_t rs = rsrc_words(y, ubytes);
    uint32_t base[NGR];
    int kc[NGR];
#pragma unroll
    for (int q = 0; q < NGR; ++q) {
      const int row = 8 * (wave + NWV * q) + (lane >> 3);
      const int lc = (lane & 7) ^ rt_swz<64>(row);
      kc[q] = 8 * lc;
      base[q] = row < m ? static_cast<uint32_t>((static_cast<int64_t>(row) * n + 8 * lc) * 2) : kOOB;
    }
    auto issue = [&](char* st, int k0) {
      dma16_group<NGR>(
          rs, static_cast<uint32_t>(k0 * 2), [&](int q) { return st + (wave + NWV * q) * 1024; },
          [&](int q) { return k0 + kc[q] < n ? base[q] : kOOB; });
    };
    Acc acc;
    acc.zero();
    const int KT = (n + 63) / 64;
    issue(s0, 0);
    issue(s1, 64);
    for (int kt = 0; kt < KT; ++kt) {
      char* st = (kt & 1) ? s1 : s0;
      // this wave's loads of stage kt have landed (stage kt + 1 may fly)
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NGR) : "memory");
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t fa[FN], fb[2];
#pragma unroll
        for (int i = 0; i < FN; ++i) fa[i] = rt_frag(st, wn * WNC + i * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) fb[i] = rt_frag(st, wm * 64 + i * 32, kk, lane);
        acc.mma(fa, fb);
      }
      barrier_lds();  // every wave is done with stage kt's buffer
      issue(st, (kt + 2) * 64);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const float s2 = s * s;
    for_acc(wm, wn, lane, [&](int mi, int ni, int g, int i, int j) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = s2 * acc.v[mi][ni][4 * g + q];
      *reinterpret_cast<uint2*>(rt_at(am, i, j)) = pack4(v);
    });
    barrier_lds();
    mirror_lower(am, tid);
    barrier_lds();
  }

  // C = X Y^T over K = 128 for two K-contiguous 128 x 128 tiles in LDS
  auto product = [&](const char* x, const char* yy, Acc& acc) {
    acc.zero();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8_t fa[FN], fb[2];
#pragma unroll
      for (int i = 0; i < FN; ++i) fa[i] = rt_frag(yy, wn * WNC + i * 32, kk, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i) fb[i] = rt_frag(x, wm * 64 + i * 32, kk, lane);
      acc.mma(fa, fb);
    }
  };
  // f acc rounded to bf16 into d, then the lower triangle from the upper one
  auto store_sym = [&](const Acc& acc, char* d, float f) {
    for_acc(wm, wn, lane, [&](int mi, int ni, int g, int i, int j) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = f * acc.v[mi][ni][4 * g + q];
      *reinterpret_cast<uint2*>(rt_at(d, i, j)) = pack4(v);
    });
    barrier_lds();
    mirror_lower(d, tid);
    barrier_lds();
  };
  // d = a I + b A + c A A (A in am) with iteration k's coefficients; with
  // dg set, the diagonal before rounding also goes to dg[0 .. m) (global: the
  // on-chip memory is taken), visible to the whole workgroup after the
  // barrier
  auto symsq = [&](char* d, int k, float* dg) {
    const int r = k < a.ncoef ? k : a.ncoef - 1;
    const float ca = a.coef[r][0], cb = a.coef[r][1], cc = a.coef[r][2];
    Acc acc;
    product(am, am, acc);
    for_acc(wm, wn, lane, [&](int mi, int ni, int g, int i, int j) {
      const uint2 w = *reinterpret_cast<const uint2*>(rt_at(am, i, j));
      const float e[4] = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                          __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = cb * e[q] + cc * acc.v[mi][ni][4 * g + q];
        if (i == j + q) {
          v[q] += ca;
          if (dg != nullptr && i < m) dg[i] = v[q];
        }
      }
      *reinterpret_cast<uint2*>(rt_at(d, i, j)) = pack4(v);
    });
    if (dg != nullptr) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    barrier_lds();
    mirror_lower(d, tid);
    barrier_lds();
  };
  // ax = B' X_c for the K-major iterate block in sl (B' in bp); with diag,
  // B's diagonal residual r (bf16) on the 16 rows each step contracts over,
  // as one more MFMA per accumulator of their 32-row block: the same operand
  // and order as the 128-tile launches
  auto block_product = [&](const char* sl, Acc& ax, bool diag, const float (&drow)[2]) {
      ax.zero();
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        bf16x8_t fa[FN], fb[2];
#pragma unroll
        for (int i = 0; i < FN; ++i) fa[i] = kt_frag(sl, wn * WNC + i * 32, kk, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i) fb[i] = rt_frag(bp, wm * 64 + i * 32, kk, lane);
        ax.mma(fa, fb);
        if (diag && (kk >> 2) == wm) {
          const int mis = (kk >> 1) & 1;
          const int idx = wm * 64 + mis * 32 + (lane & 31);
          const int e = idx - 16 * kk - 8 * (lane >> 5);
          const uint32_t rb = (e >= 0 && e < 8)
                                  ? static_cast<uint32_t>(muon::f32_to_bf16(muon::ns_diag_residual(drow[mis])))
                                  : 0u;
          const uint32_t w = (e & 1) ? (rb << 16) : rb;
          const int q = e >> 1;
          const u32x4_t v = {q == 0 ? w : 0u, q == 1 ? w : 0u, q == 2 ? w : 0u, q == 3 ? w : 0u};
          const bf16x8_t fd = __builtin_bit_cast(bf16x8_t, v);
          static_for<FN>([&](auto NI) {
            constexpr int ni = decltype(NI)::value;
            if (mis == 0)
              ax.v[0][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ni], fd, ax.v[0][ni], 0, 0, 0);
            else
              ax.v[1][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ni], fd, ax.v[1][ni], 0, 0, 0);
          });
        }
      }
  };
  // The column pass of the quintic with B's fp32 diagonal and the iterate's
  // residual (dg set): iterate blocks alternate between s0 and s1, residual
  // blocks between s2 and am, and each X' block is staged in the slab its
  // input block came in (free once its product is done), so one block of
  // each is always in flight.  Residual blocks come in by global->LDS DMA in
  // the plane's byte order, every wave fetching the 1 KiB pieces it reads
  // back itself (piece q of wave w at (w + NWV q) KiB: its chunk q), so no
  // register load queues behind the DMA in flight.  At the top of block c,
  // issued after its loads: the residual and X' stores of block c - 1 and
  // the loads of block c + 1 (both kinds of memory operation count, in issue
  // order) -- the wait counts below.
  auto column_pass_res = [&](const bf16_t* xd, float f, bool next, Acc& an, const float (&drow)[2],
                             const char* lo_in, char* lo_out, auto&& issue_x) {
    // memory operations per wave: NGC per iterate block, NLO per residual
    // block, NST X' stores and NLS residual stores per block
    constexpr int NLO = 4 * FN, NLS = 4 * FN;
    static_assert(NGC == 4 && NST == 4 && NLO == 4 && NLS == 4,
                  "wait counts below assume 4 operations per group");
    const u32x4_t lrs = rsrc_words(lo_in ? lo_in : lo_out, static_cast<uint32_t>(nb) * SLAB);
    auto issue_lo = [&](char* buf, int c) {
      if (lo_in == nullptr) return;
      dma16_group<NLO>(
          lrs, static_cast<uint32_t>(c) * SLAB, [&](int q) { return buf + (wave + NWV * q) * 1024; },
          [&](int q) { return c < nb ? static_cast<uint32_t>((wave + NWV * q) * 1024 + lane * 16) : kOOB; });
    };
    auto slab = [&](int c) { return (c & 1) ? s1 : s0; };
    auto lobuf = [&](int c) { return (c & 1) ? am : s2; };
    const int n_in = (lo_in ? NLO : 0) + NGC;
    const int n_out = (lo_out ? NLS : 0) + NST;
    issue_lo(lobuf(0), 0);
    issue_x(slab(0), 0);
    issue_lo(lobuf(1), 1);
    issue_x(slab(1), SM);
    for (int c = 0; c < nb; ++c) {
      char* sl = slab(c);
      const int nw = (c == 0 ? 0 : n_out) + n_in;  // 4 .. 16, a multiple of 4
      if (nw == 4)
        asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
      else if (nw == 8)
        asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      else if (nw == 12)
        asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
      Acc ax;
      block_product(sl, ax, true, drow);
      // this wave's residual chunks of block c, from the pieces it fetched
      u32x4_t lov[NLO];
#pragma unroll
      for (int ch = 0; ch < NLO; ++ch)
        lov[ch] = lo_in ? *reinterpret_cast<const u32x4_t*>(lobuf(c) + (ch * NWV + wave) * 1024 + lane * 16)
                        : u32x4_t{0u, 0u, 0u, 0u};
      barrier_lds();  // every wave is done reading block c: stage X' over it
      static_for<2>([&](auto MI) {
        constexpr int mi = decltype(MI)::value;
        u32x4_t lon[2 * FN];
        static_for<FN>([&](auto NI) {
          static_for<4>([&](auto G) {
            constexpr int ni = decltype(NI)::value, g = decltype(G)::value;
            const int i = wm * 64 + mi * 32 + (lane & 31);
            const int j = wn * WNC + ni * 32 + 8 * g + 4 * (lane >> 5);
            const u32x4_t lc = lov[mi * 2 * FN + 2 * ni + g / 2];
            const uint32_t l0 = (g & 1) ? lc.z : lc.x, l1 = (g & 1) ? lc.w : lc.y;
            const float lo[4] = {__uint_as_float(l0 << 16), __uint_as_float(l0 & 0xffff0000u),
                                 __uint_as_float(l1 << 16), __uint_as_float(l1 & 0xffff0000u)};
            float v[4], r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              v[q] = ax.v[mi][ni][4 * g + q];
              if (lo_in) v[q] = muon::ns_lo_term(v[q], drow[mi], lo[q]);
              v[q] = f * v[q];
              r[q] = v[q] - muon::bf16_round(v[q]);
            }
            u32x4_t& lw = lon[2 * ni + g / 2];
            if (g & 1) {
              lw.z = muon::pack_bf16x2(r[0], r[1]);
              lw.w = muon::pack_bf16x2(r[2], r[3]);
            } else {
              lw.x = muon::pack_bf16x2(r[0], r[1]);
              lw.y = muon::pack_bf16x2(r[2], r[3]);
            }
            *reinterpret_cast<uint2*>(rt_at(sl, i, j)) = pack4(v);
          });
        });
        if (lo_out) {
#pragma unroll
          for (int ch = 0; ch < 2 * FN; ++ch)
            __builtin_nontemporal_store(
                lon[ch], reinterpret_cast<u32x4_t*>(lo_out + static_cast<int64_t>(c) * SLAB +
                                                    ((mi * 2 * FN + ch) * NWV + wave) * 1024 + lane * 16));
        }
      });
      barrier_lds();
      store_block(xd, c * SM, sl);
      if (next) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          bf16x8_t fa[FN], fb[2];
#pragma unroll
          for (int i = 0; i < FN; ++i) fa[i] = rt_frag(sl, wn * WNC + i * 32, kk, lane);
#pragma unroll
          for (int i = 0; i < 2; ++i) fb[i] = rt_frag(sl, wm * 64 + i * 32, kk, lane);
          an.mma(fa, fb);
        }
      }
      barrier_lds();  // block c's slab and residual buffer are free again
      issue_lo(lobuf(c), c + 2);
      issue_x(sl, (c + 2) * SM);
    }
    // whatever reads this pass's output next sees every store, and the
    // zero-filling loads issued past the last block have landed
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // xd = f B xs (B in bp) block by block; with `next`, an accumulates
  // xd xd^T from the stored bf16 blocks.  With dg set (quintic), B's fp32
  // diagonal is completed and the iterate's residual carried
  // (ns_diag_residual, ns_lo_term) in column_pass_res: lo_in / lo_out are the
  // unit's residual planes (one 32 KiB block per column block, each lane's
  // values of a 32-row block as 2 FN contiguous 16-byte chunks; lo_in null
  // for the exact bf16 input, lo_out null when not kept).  Without dg, three
  // iterate blocks rotate through s0 .. s2 and X' is staged in am.
  auto column_pass = [&](const bf16_t* xs, const bf16_t* xd, float f, bool next, Acc& an,
                         const float* dg, const char* lo_in, char* lo_out) {
    float drow[2] = {0.0f, 0.0f};
    if (dg != nullptr) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int i = wm * 64 + mi * 32 + (lane & 31);
        if (i < m) drow[mi] = dg[i];
      }
      // use the values here, so that their wait comes before the pass's
      // loads are issued rather than behind them
      asm volatile("" : "+v"(drow[0]), "+v"(drow[1]));
    }
    const u32x4_t rs = rsrc_words(xs, ubytes);
    uint32_t base[NGC];
    int cc[NGC];
#pragma unroll
    for (int q = 0; q < NGC; ++q) {
      const int kr = 4 * (wave + NWV * q) + (lane >> 4);
      const int col = 8 * ((lane & 15) ^ ((kr & 3) << 2));
      cc[q] = col;
      base[q] = kr < m ? static_cast<uint32_t>((static_cast<int64_t>(kr) * n + col) * 2) : kOOB;
    }
    auto issue = [&](char* sl, int c0) {
      dma16_group<NGC>(
          rs, static_cast<uint32_t>(c0 * 2), [&](int q) { return sl + (wave + NWV * q) * 1024; },
          [&](int q) { return c0 + cc[q] < n ? base[q] : kOOB; });
    };
    an.zero();
    if (dg != nullptr) {
      column_pass_res(xd, f, next, an, drow, lo_in, lo_out, issue);
      return;
    }
    issue(s0, 0);
    issue(s1, SM);
    issue(s2, 2 * SM);
    for (int c = 0; c < nb; ++c) {
      char* sl = (c % 3 == 0) ? s0 : ((c % 3 == 1) ? s1 : s2);
      // wait for this wave's block-c loads; issued after them: blocks c + 1,
      // c + 2 (NGC loads each) and the stores of blocks c - 2, c - 1 (NST each)
      if (c == 0)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NGC) : "memory");
      else if (c == 1)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NGC + NST) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * NGC + 2 * NST) : "memory");
      Acc ax;
      block_product(sl, ax, false, drow);
      {
        for_acc(wm, wn, lane, [&](int mi, int ni, int g, int i, int j) {
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = f * ax.v[mi][ni][4 * g + q];
          *reinterpret_cast<uint2*>(rt_at(am, i, j)) = pack4(v);
        });
      }
      barrier_lds();
      store_block(xd, c * SM, am);
      if (next) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          bf16x8_t fa[FN], fb[2];
#pragma unroll
          for (int i = 0; i < FN; ++i) fa[i] = rt_frag(am, wn * WNC + i * 32, kk, lane);
#pragma unroll
          for (int i = 0; i < 2; ++i) fb[i] = rt_frag(am, wm * 64 + i * 32, kk, lane);
          an.mma(fa, fb);
        }
      }
      barrier_lds();  // block c's buffer and the staging are free again
      issue(sl, (c + 3) * SM);
    }
    // whatever reads this pass's output next sees every store
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  };

  if constexpr (!GRAM) {
    // B's fp32 diagonal and the residual planes of this unit
    float* dg = a.dvec ? a.dvec + u * static_cast<int64_t>(m) : nullptr;
    char* lo = a.lo ? a.lo + u * static_cast<int64_t>(nb) * SLAB : nullptr;
    for (int k = 0; k < a.steps; ++k) {
      const bool last = k + 1 == a.steps;
      symsq(bp, k, dg);  // B'
      const bf16_t* xs = k == 0 ? y : uniform_ptr(reinterpret_cast<const bf16_t*>(
                                          mat_at(((k - 1) & 1) ? a.xb : a.xa, u)));
      const bf16_t* xd = last ? out : uniform_ptr(reinterpret_cast<const bf16_t*>(
                                          mat_at((k & 1) ? a.xb : a.xa, u)));
      Acc an;  // A_{k+1}
      column_pass(xs, xd, k == 0 ? s : 1.0f, !last, an, dg,
                  (dg && ns_lo_read(k, a.steps)) ? lo : nullptr,
                  (dg && ns_lo_written(k, a.steps)) ? lo : nullptr);
      if (!last) store_sym(an, am, 1.0f);
    }
  } else {
    // Gram form: P_k = a I + b A_k + c A_k^2, Q_{k+1} = P_k Q_k (Q_1 = P_0),
    // A_{k+1} = (P_k A_k) P_k, all m x m in LDS (A in am, P in bp, Q and a
    // scratch product in the free slab buffers); then X = s Q Y.
    char* q = s1;
    char* t = s0;
    for (int k = 0; k < a.steps; ++k) {
      char* p = k == 0 ? q : bp;
      symsq(p, k, nullptr);
      if (k > 0) {
        Acc c;
        product(p, q, c);
        store_sym(c, t, 1.0f);
        char* w = q;
        q = t;
        t = w;
      }
      if (k + 1 < a.steps) {
        Acc c;
        product(p, am, c);
        store_sym(c, t, 1.0f);
        Acc c2;
        product(t, p, c2);
        store_sym(c2, am, 1.0f);
      }
    }
    // Q into bp, the slab buffers carry the input blocks
#pragma unroll
    for (int it = 0; it < 2 * HALF / 16 / (64 * NWV); ++it) {
      const int e = 16 * (tid + 64 * NWV * it);
      *reinterpret_cast<u32x4_t*>(bp + e) = *reinterpret_cast<const u32x4_t*>(q + e);
    }
    barrier_lds();
    Acc unused;
    column_pass(y, out, s, false, unused, nullptr, nullptr, nullptr);
  }
}

}  // namespace

hipError_t launch_ns_small(hipStream_t s, const NsSmallArgs& a) {
  if (a.units <= 0) return hipSuccess;
  if (a.m < 1 || a.m > SM || a.n < a.m || a.m % 8 || a.n % 8 || a.steps < 1 ||
      a.ncoef < 1 || a.ncoef > MUON_NS_FUSED_MAX_ROWS ||
      static_cast<int64_t>(a.m) * a.n * 2 >= (int64_t{1} << 31) || a.units > 0x7fffffff)
    return hipErrorInvalidValue;
  if (a.gram)
    ns_small_kernel<true><<<static_cast<unsigned>(a.units), 64 * NWV, 0, s>>>(a);
  else
    ns_small_kernel<false><<<static_cast<unsigned>(a.units), 64 * NWV, 0, s>>>(a);
  return hipGetLastError();
}
