// The three matrix products of one quintic Newton-Schulz iteration on gfx950
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Per iteration, with X the m x n iterate (m <= n; a tall matrix Y = X^T is
// kept in its own orientation):
//   gram   A  = alpha X X^T          upper-triangle tiles only, mirrored
//   symsq  B' = a I + b A + c A A    A symmetric, so A A = A A^T; upper tiles
//   update X' = beta B' X            (tall: Y' = beta Y B')
// B' X equals the iteration's a X + B X with B = b A + c A A; carrying the
// a I term inside B' means the update reads no third operand.
// alpha = s^2 and beta = s fold the first iteration's normalisation
// X_0 = s Y (s = 1 / (||Y||_F + eps)) into the products, so Y is never
// rewritten.  Every product is C = P_M P_N^T over a contraction index k.  An
// operand is "K-contiguous" when its rows run along k in memory (X rows for
// the wide Gram, A, B, Y rows for the tall update) and "K-major" when k is
// its memory row index (the X operand of the wide update, both Y operands of
// the tall Gram).  Both kinds are copied into LDS unchanged; K-major tiles
// are read by the MFMA loop with ds_read_b64_tr_b16, which hands each lane
// four consecutive k of one column, so no transposed copy of any matrix is
// ever made.
//
// Tiling: BM x BN workgroup tile, BK = 64.  256 x 256 tiles run 8 waves
// (2 along M x 4 along N, two waves per SIMD, each 128 x 64): a second wave
// on every SIMD issues its LDS reads and MFMAs while the first waits, which a
// single wave per SIMD cannot hide.  128 x 128 tiles run 4 waves of 64 x 64.
// MFMA fragments are double-buffered in registers: the LDS reads of k16 step
// kk + 1 are interleaved with the MFMAs of step kk.  Operand tiles move
// global -> LDS with buffer_load_dwordx4 ... lds: each wave instruction
// fills 1024 contiguous LDS bytes (lane l at 16 l), so every lane fetches the
// global chunk the XOR swizzle puts at its slot; chunks outside the matrix get
// an offset past the buffer's size and the hardware returns zeros.  Two LDS
// stages (the loads of stage k+1 fly while stage k feeds the MFMAs).  The
// epilogue stages the bf16 tile through LDS so global stores are 16-byte and
// row-contiguous, and writes the mirror tile of symmetric outputs from
// transposed LDS reads.  The grid is persistent (one workgroup per CU, each
// walking its tiles); the workgroups of one XCD (own L2) always work on
// neighbouring tiles.  The same kernel also serves the m x m products of the
// Gram form of the iteration (P Q for symmetric commuting P, Q through the
// Gram epilogue).
#include "ns_mfma_common.h"

#include <cstdlib>
#include <cstring>

namespace {

template <int R, bool KMAJOR, int NW, int BK>
struct Operand;

template <int R, int NW, int BK>
struct Operand<R, false, NW, BK> {
  static constexpr int CPR = BK / 8;          // 16-byte chunks per tile row
  static constexpr int RPI = 64 / CPR;        // tile rows per wave instruction
  static constexpr int NG = R / (RPI * NW);   // instructions per wave per stage
  uint32_t base[NG];
  int kc[NG];
  u32x4_t rsrc;

  // src: rows x ld matrix; tile rows [row0, row0 + R).  Lane l of an
  // instruction fills LDS bytes 16 l .. 16 l + 15 of its 1 KiB block, i.e.
  // physical chunk l % CPR of row l / CPR, which holds the logical chunk
  // that the swizzle maps there.
  __device__ __forceinline__ void init(const bf16_t* src, int64_t ld, int rows, int /*K*/,
                                       int row0, int wave, int lane) {
    rsrc = rsrc_words(src, static_cast<uint32_t>(static_cast<int64_t>(rows) * ld * 2));
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int row = RPI * (wave + NW * q) + lane / CPR;
      const int lc = (lane % CPR) ^ rt_swz<BK>(row);
      const int gr = row0 + row;
      kc[q] = 8 * lc;
      base[q] = (gr < rows) ? static_cast<uint32_t>((static_cast<int64_t>(gr) * ld + 8 * lc) * 2)
                            : kOOB;
    }
  }
  __device__ __forceinline__ void issue(char* lds, int k0, int K, int64_t /*ld*/, int wave,
                                        bool full) const {
    const uint32_t soff = static_cast<uint32_t>(k0 * 2);
    dma16_group<NG>(
        rsrc, soff, [&](int q) { return lds + (wave + NW * q) * 1024; },
        [&](int q) { return (full || k0 + kc[q] < K) ? base[q] : kOOB; });
  }
  // MFMA operand for tile rows rb .. rb + 31, k = 16 kk + 8 (lane / 32) + 0..7
  __device__ __forceinline__ bf16x8_t frag(const char* t, int rb, int kk, int lane) const {
    return *reinterpret_cast<const bf16x8_t*>(t + rt_off<BK>(rb + (lane & 31), 2 * kk + (lane >> 5)));
  }
};

template <int R, int NW, int BK>
struct Operand<R, true, NW, BK> {
  static constexpr int CPR = R / 8;         // 16-byte chunks per tile row
  static constexpr int RPI = 64 / CPR;      // tile rows per wave instruction
  static constexpr int NG = BK / RPI / NW;  // instructions per wave per stage
  uint32_t base[NG];
  int kr[NG];
  u32x4_t rsrc;

  // src: K x ld matrix (k = memory row); tile columns [col0, col0 + R).
  __device__ __forceinline__ void init(const bf16_t* src, int64_t ld, int cols, int K, int col0,
                                       int wave, int lane) {
    rsrc = rsrc_words(src, static_cast<uint32_t>(static_cast<int64_t>(K) * ld * 2));
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int k = RPI * (wave + NW * q) + lane / CPR;
      const int c = (lane % CPR) ^ ((k & 3) << 2);
      const int col = col0 + 8 * c;
      kr[q] = k;
      base[q] = (col < cols) ? static_cast<uint32_t>((static_cast<int64_t>(k) * ld + col) * 2)
                             : kOOB;
    }
  }
  __device__ __forceinline__ void issue(char* lds, int k0, int K, int64_t ld, int wave,
                                        bool full) const {
    const uint32_t soff = static_cast<uint32_t>(static_cast<int64_t>(k0) * ld * 2);
    dma16_group<NG>(
        rsrc, soff, [&](int q) { return lds + (wave + NW * q) * 1024; },
        [&](int q) { return (full || k0 + kr[q] < K) ? base[q] : kOOB; });
  }
  __device__ __forceinline__ bf16x8_t frag(const char* t, int rb, int kk, int lane) const {
    const int gq = lane >> 4, j = lane & 15;
    const int col = rb + 16 * (gq & 1) + 4 * (j & 3);
    const int k = 16 * kk + 8 * (gq >> 1) + (j >> 2);
    const u32x2_t lo = __builtin_bit_cast(u32x2_t, ld_tr16(t + kt_off<R>(k, col)));
    const u32x2_t hi = __builtin_bit_cast(u32x2_t, ld_tr16(t + kt_off<R>(k + 4, col)));
    const u32x4_t v = {lo.x, lo.y, hi.x, hi.y};
    return __builtin_bit_cast(bf16x8_t, v);
  }
};

// ---- staged output tile: BM x BN bf16 in LDS, 2 BN-byte rows; chunk swizzle
// g(row) = 4 (row & 3) | (row >> 2) & 3 keeps both the per-lane 8-byte
// writes (32 consecutive rows) and the transposed mirror reads on spread banks.
template <int BN>
__device__ __forceinline__ int ct_off(int row, int col) {
  const int g = ((row & 3) << 2) | ((row >> 2) & 3);
  return row * (2 * BN) + (((col >> 3) ^ g) << 4) + ((col & 7) << 1);
}

// The staged tile spans NP of the stage buffers, BM / NP rows in each.
template <int BM, int BN, int NP>
struct OutTile {
  char* p[4];
  __device__ __forceinline__ char* part(int q) const {
    if (NP == 1) return p[0];
    if (NP == 2) return q ? p[1] : p[0];
    return q < 2 ? (q ? p[1] : p[0]) : (q == 3 ? p[3] : p[2]);
  }
  __device__ __forceinline__ char* at(int row, int col) const {
    constexpr int RP = BM / NP;
    return part(row / RP) + ct_off<BN>(row % RP, col);
  }
};

template <int BM, int BN, int NWN, int BK, int NS, bool TM, bool TN, int EPI>
__global__ __launch_bounds__(128 * NWN, 1) void ns_gemm_mfma_kernel(NsGemmArgs a) {
  constexpr int NW = 2 * NWN, NT = 64 * NW;  // waves: 2 along M x NWN along N
  constexpr int WM = BM / 2, WN = BN / NWN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int STAGE = (BM + BN) * BK * 2;
  constexpr int NP = (BM * BN * 2 + STAGE - 1) / STAGE;  // stage buffers the output tile spans
  // NS stage buffers, NS - 1 stages in flight.  Only NS = 2 with BK = 64 is
  // instantiated: a four-buffer ring of BK = 32 stages (three in flight)
  // measured slower on gfx950, its extra barrier per 32 k costing more than
  // the deeper prefetch gains.
  static_assert(NS == 2 && BK == 64, "two stage buffers of 64 k");
  static_assert(NP <= NS && (NP & (NP - 1)) == 0 && STAGE >= (BM / NP) * BN * 2,
                "output tile must fit the stage buffers");
  // Distinct LDS objects per stage: the DMA writes into one are then provably
  // disjoint from the reads of the others, so no wait on the loads in flight
  // is inserted ahead of the MFMAs.
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[NS > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char st3[NS > 2 ? STAGE : 16];
  // corrected update: bf16(r), r = d - bf16(d), and d along the tile's
  // diagonal side
  constexpr int DS = EPI == EPI_UPDATE ? (TN ? BM : BN) : 1;
  __shared__ uint16_t corr_r[DS];
  __shared__ float corr_d[DS];
  auto buf = [&](auto I) -> char* {
    constexpr int i = decltype(I)::value % NS;
    if constexpr (i == 0) return st0;
    else if constexpr (i == 1) return st1;
    else if constexpr (i == 2) return st2;
    else return st3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;

  // Persistent tiles: workgroup hw runs on XCD hw % 8 (round-robin dispatch,
  // each XCD with its own L2), and the cnt workgroups of an XCD always work on
  // cnt neighbouring tiles, which share operand panels in L2.  Gram and
  // update hand out those chunks of cnt tiles round-robin over the XCDs, so
  // all XCDs work on the same few units at once and share their panels in
  // the MALL (1-3% faster there); the symmetric square keeps one contiguous
  // run per XCD (the round-robin order measured 2% slower for it).  A
  // workgroup moves on to its next tile without leaving the CU.
  // With a unit list, only the listed units' tiles (a zero unit takes no
  // slot, so the remaining tiles spread evenly over the workgroups); a list
  // of every unit is not consulted.  List and count are read through the
  // scalar cache (constant address space: nothing writes them during the
  // launch), so a tile's unit costs no vector-memory round trip.
  using cint_ptr = const __attribute__((address_space(4))) int*;
  const int64_t nlisted = a.ulist != nullptr ? static_cast<int64_t>(*(cint_ptr)(a.ucount)) : a.units;
  const bool use_list = nlisted != a.units;
  const int64_t total = nlisted * a.tiles_per_unit;
  const int G = static_cast<int>(gridDim.x), hw = static_cast<int>(blockIdx.x);
  const int xg = hw % 8, q8 = G / 8, r8 = G % 8;
  const int cnt = q8 + (xg < r8 ? 1 : 0);
  const bool rr = EPI != EPI_SYMSQ && r8 == 0;
  const int64_t P = static_cast<int64_t>(xg) * q8 + min(xg, r8);
  const int64_t t_first = rr ? static_cast<int64_t>(xg) * q8 + hw / 8 : total * P / G + hw / 8;
  const int64_t t_end = rr ? total : total * (P + cnt) / G;
  const int64_t t_step = rr ? G : cnt;

  // unit and tile coordinates of logical tile l
  auto coords = [&](int64_t l, int64_t& uu, int& ti, int& tj) __attribute__((always_inline)) {
    uu = l / a.tiles_per_unit;
    const int t = static_cast<int>(l - uu * a.tiles_per_unit);
    if (use_list) uu = ((cint_ptr)(a.ulist))[uu];
    if (EPI == EPI_UPDATE) {
      // grouped raster: bands of up to GN tile columns, row-major inside a
      // band, so the ~32 tiles an XCD runs at once form an 8 x 4 block that
      // shares its operand panels in L2
      constexpr int GN = 4;
      const int band = t / (a.tiles_m * GN);
      const int w = min(GN, a.tiles_n - band * GN);
      const int r = t - band * a.tiles_m * GN;
      ti = r / w;
      tj = band * GN + r % w;
    } else {
      upper_tile(t, ti, tj);
    }
  };
  // corrected update: B's fp32 diagonal along the tile's diagonal side
  // (rows for X' = B'X, columns for Y' = YB'); thread i < DS holds entry i.
  // The next tile's entry is requested during this tile, so the load's
  // latency is hidden.
  const bool upd_corr = EPI == EPI_UPDATE && a.dvec != nullptr;
  auto load_d = [&](int64_t l) __attribute__((always_inline)) {
    int64_t uu;
    int ti, tj;
    coords(l, uu, ti, tj);
    const int d0 = TN ? ti * BM : tj * BN, dlim = TN ? a.M : a.N;
    return (tid < DS && d0 + tid < dlim) ? a.dvec[uu * static_cast<int64_t>(a.K) + d0 + tid] : 0.0f;
  };
  float dpre = 0.0f;
  int64_t dpre_lid = -1;

  for (int64_t lid = t_first; lid < t_end; lid += t_step) {
  int64_t u;
  int ti, tj;
  coords(lid, u, ti, tj);
  const int m0 = ti * BM, n0 = tj * BN;

  const bool zero_unit = a.zflag != nullptr && a.zflag[u] != 0;
  if (zero_unit && !(EPI == EPI_UPDATE && a.zero_write)) continue;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) acc[mi][ni] = (f32x16_t)(0.0f);

  // update with the iterate carried past bf16 (ns_diag_residual): B's fp32
  // diagonal along the output's rows (wide, X' = B'X) or columns (tall,
  // Y' = YB').  Not for a zero unit: it writes zeros and its workspace was
  // never filled.
  const bool corr = upd_corr && !zero_unit;
  if (corr) {
    const float d = dpre_lid == lid ? dpre : load_d(lid);
    if (tid < DS) {
      corr_d[tid] = d;
      corr_r[tid] = muon::f32_to_bf16(muon::ns_diag_residual(d));
    }
    // visible to every wave at the k-loop's first barrier
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  }
  if (upd_corr && lid + t_step < t_end) {
    dpre = load_d(lid + t_step);
    dpre_lid = lid + t_step;
  }

  if (!zero_unit) {
    using OpM = Operand<BM, TM, NW, BK>;
    using OpN = Operand<BN, TN, NW, BK>;
    OpM om;
    OpN on;
    om.init(uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.pm, u))), a.ldm, a.M, a.K, m0,
            wave, lane);
    on.init(uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.pn, u))), a.ldn, a.N, a.K, n0,
            wave, lane);
    const int KT = (a.K + BK - 1) / BK;
    const int KF = a.K / BK;  // stages lying fully inside K
    auto issue = [&](char* st, int kt) {
      const bool full = kt < KF;
      om.issue(st, kt * BK, a.K, a.ldm, wave, full);
      on.issue(st + BM * BK * 2, kt * BK, a.K, a.ldn, wave, full);
    };
    constexpr int NL = OpM::NG + OpN::NG;  // load instructions per wave per stage

    // Register double buffer of MFMA fragments: the LDS reads of k16 step
    // kk + 1 are issued among the MFMAs of step kk.
    bf16x8_t fa[2][FN], fb[2][FM];
    auto frags = [&](const char* sm, int kk, auto BUF) {
      constexpr int b = decltype(BUF)::value;
      const char* sn = sm + BM * BK * 2;
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) fa[b][ni] = on.frag(sn, wn * WN + ni * 32, kk, lane);
#pragma unroll
      for (int mi = 0; mi < FM; ++mi) fb[b][mi] = om.frag(sm, wm * WM + mi * 32, kk, lane);
    };
    auto mfmas = [&](auto BUF, auto BEGIN, auto END) {
      constexpr int b = decltype(BUF)::value;
      static_for<decltype(END)::value - decltype(BEGIN)::value>([&](auto P) {
        constexpr int p = decltype(P)::value + decltype(BEGIN)::value;
        constexpr int mi = p / FN, ni = p % FN;
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b][ni], fb[b][mi], acc[mi][ni], 0, 0, 0);
      });
    };
    constexpr int KK = BK / 16;                                      // k16 steps per stage
    constexpr int NMF = FM * FN;                                     // MFMAs per k16 step
    constexpr int NRD = (TN ? 2 : 1) * FN + (TM ? 2 : 1) * FM;       // LDS reads per k16 step
    constexpr int TAIL = NMF / 2;                                    // MFMAs after the barrier
    // interleave: one MFMA, then one LDS read, while reads remain
    auto interleave = [&](auto NM) {
      static_for<decltype(NM)::value>([&](auto I) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
        if constexpr (decltype(I)::value < NRD)
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);          // DS read
      });
    };

    // Stage kt in buffer kt % NS (its first fragments already in registers).
    // Near its end: wait until this wave's loads of stage kt + 1 have landed
    // (the NS - 2 later stages may still fly) and this wave's reads of stage
    // kt are done; the barrier then makes stage kt + 1 visible and frees
    // buffer kt % NS, which receives stage kt + NS.
    // The diagonal's residual r (in bf16) as a matrix-core operand: for k16
    // step kk of stage kt, whose 16 k-indices are the output rows (wide,
    // X' = B'X) or columns (tall, Y' = YB') k16 .. k16 + 15 of this tile,
    // the 32 x 16 slice of diag(r) meets the step's X (Y) fragment in one
    // more MFMA per accumulator of that 32-block: acc += r hi, exactly, with
    // no vector-ALU write to the accumulators inside the loop.  A lane's
    // slice row holds at most one nonzero k.
    auto diag_frag = [&](int idx, int k16, uint32_t rv) __attribute__((always_inline)) {
      const int e = idx - k16 - 8 * (lane >> 5);  // which of the lane's 8 k is idx
      const uint32_t rb = (e >= 0 && e < 8) ? rv : 0u;
      const uint32_t w = (e & 1) ? (rb << 16) : rb;
      const int q = e >> 1;
      const u32x4_t v = {q == 0 ? w : 0u, q == 1 ? w : 0u, q == 2 ? w : 0u, q == 3 ? w : 0u};
      return __builtin_bit_cast(bf16x8_t, v);
    };
    auto diag_mfmas = [&](int kt, auto KI, auto BUF, const uint32_t (&rv)[2]) __attribute__((always_inline)) {
      constexpr int kk = decltype(KI)::value, b = decltype(BUF)::value;
      const int k16 = kt * BK + 16 * kk - (TN ? m0 : n0);
      if constexpr (TN) {
        // rows k16 .. k16 + 15: wave row wm = k16 / WM, block (k16 % WM) / 32
        if (corr && k16 >= 0 && k16 < BM && k16 / WM == wm) {
          const int mis = (k16 % WM) / 32;
          const bf16x8_t fd = diag_frag(wm * WM + mis * 32 + (lane & 31), k16, rv[kk / 2]);
          static_for<FM>([&](auto MI) __attribute__((always_inline)) {
            constexpr int mi = decltype(MI)::value;
            if (mi == mis) {
              static_for<FN>([&](auto NI) __attribute__((always_inline)) {
                constexpr int ni = decltype(NI)::value;
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[b][ni], fd, acc[mi][ni], 0, 0, 0);
              });
            }
          });
        }
      } else {
        // columns k16 .. k16 + 15: wave column wn = k16 / WN, block (k16 % WN) / 32
        if (corr && k16 >= 0 && k16 < BN && k16 / WN == wn) {
          const int nis = (k16 % WN) / 32;
          const bf16x8_t fd = diag_frag(wn * WN + nis * 32 + (lane & 31), k16, rv[kk / 2]);
          static_for<FN>([&](auto NI) __attribute__((always_inline)) {
            constexpr int ni = decltype(NI)::value;
            if (ni == nis) {
              static_for<FM>([&](auto MI) __attribute__((always_inline)) {
                constexpr int mi = decltype(MI)::value;
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fd, fb[b][mi], acc[mi][ni], 0, 0, 0);
              });
            }
          });
        }
      }
    };

    auto stage = [&](auto S, int kt_new) {
      char* cur = buf(S);
      const char* nxt = buf(ic<decltype(S)::value + 1>{});
      const int kt_cur = kt_new - NS;
      // the stage's diagonal residuals, read once: entries r0 + l % 32 and
      // r0 + 32 + l % 32 of this tile's diagonal side (none outside it)
      uint32_t rv[2] = {0u, 0u};
      if constexpr (EPI == EPI_UPDATE) {
        const int r0 = kt_cur * BK - (TN ? m0 : n0);
        if (corr && r0 >= 0 && r0 < (TN ? BM : BN)) {
          rv[0] = corr_r[r0 + (lane & 31)];
          rv[1] = corr_r[r0 + 32 + (lane & 31)];
        }
      }
      static_for<KK>([&](auto KI) {
        constexpr int kk = decltype(KI)::value;
        constexpr int b = kk & 1;
        if constexpr (kk + 1 < KK) {
          frags(cur, kk + 1, ic<b ^ 1>{});
          mfmas(ic<b>{}, ic<0>{}, ic<NMF>{});
          interleave(ic<NMF>{});
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (EPI == EPI_UPDATE) diag_mfmas(kt_cur, ic<kk>{}, ic<b>{}, rv);
        } else {
          mfmas(ic<b>{}, ic<0>{}, ic<NMF - TAIL>{});
          __builtin_amdgcn_sched_barrier(0);
          // a bare s_barrier: __syncthreads() adds a workgroup fence, which
          // would also wait for the loads still meant to be in flight
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"((NS - 2) * NL) : "memory");
          issue(cur, kt_new);
          __builtin_amdgcn_sched_barrier(0);
          frags(nxt, 0, ic<0>{});
          mfmas(ic<b>{}, ic<NMF - TAIL>{}, ic<NMF>{});
          interleave(ic<TAIL>{});
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (EPI == EPI_UPDATE) diag_mfmas(kt_cur, ic<kk>{}, ic<b>{}, rv);
        }
      });
    };

    // The first NS stages load up front; the loop runs whole rounds of NS
    // stages (fixed LDS objects, no branches): stages at or past K load
    // zeros (offsets fall outside the buffer) and add nothing.
    static_for<NS>([&](auto S) { issue(buf(S), decltype(S)::value); });
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"((NS - 1) * NL) : "memory");
    frags(buf(ic<0>{}), 0, ic<0>{});
    for (int kt = 0; kt < KT; kt += NS) {
      static_for<NS>([&](auto S) { stage(S, kt + decltype(S)::value + NS); });
    }
  }

  // ---- epilogue: finish values in registers, stage bf16 tile in LDS, store.
  // Its LDS and global addresses depend on the lane only; an opaque copy of
  // the lane index keeps the compiler from hoisting them out of the tile loop,
  // where they would hold registers through the k-loop.
  int elane = lane;
  asm volatile("" : "+v"(elane));
  const int etid = wave * 64 + elane;
  // MFMA operand A carried the N side, so lane l holds local row
  // wm WM + mi 32 + l % 32 of C and, per register group g, four consecutive
  // local columns wn WN + ni 32 + 8 g + 4 (l / 32) + 0..3.
  float s = 1.0f;
  if (a.scale != nullptr && a.scale_pow > 0) {
    s = a.scale[u];
    if (a.scale_pow == 2) s = s * s;
  }
  // every wave is done reading the operand stages, and the (zero-filled)
  // loads the last k-stages issued past K have landed
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
  __syncthreads();
  OutTile<BM, BN, NP> ct;
  ct.p[0] = buf(ic<0>{});
  ct.p[1] = buf(ic<1>{});
  ct.p[2] = buf(ic<2 % NS>{});
  ct.p[3] = buf(ic<3 % NS>{});
  const bool diag_tile = ti == tj;
  if (EPI == EPI_SYMSQ) {
    // symsq adds b A: fetch that tile of A into the staging area with one
    // round of global->LDS loads, laid out exactly like the output tile, and
    // finish the values in place.
    const bf16_t* ep = uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.epi, u)));
    const __amdgpu_buffer_rsrc_t er =
        make_rsrc(ep, static_cast<uint32_t>(static_cast<int64_t>(a.M) * a.lde * 2));
    constexpr int RB = 2 * BN;                   // bytes per staged row
    constexpr int RP = BM / NP;                  // rows per part
    constexpr int IPP = RP * RB / 1024;          // wave instructions per part
    static_assert(IPP * 1024 == RP * RB && (NP * IPP) % NW == 0, "staging split");
#pragma unroll
    for (int q = 0; q < NP * IPP / NW; ++q) {
      const int g = wave + NW * q;
      const int h = g / IPP;                     // which part
      const int pos = (g - h * IPP) * 1024 + elane * 16;
      const int rl = pos / RB;                   // row within the part
      const int pc = (pos % RB) >> 4;            // physical chunk
      const int gsw = ((rl & 3) << 2) | ((rl >> 2) & 3);
      const int row = rl + h * RP;
      const int col = 8 * (pc ^ gsw);
      const int gi = m0 + row, gj = n0 + col;
      const uint32_t off = (gi < a.M && gj < a.N)
                               ? static_cast<uint32_t>((static_cast<int64_t>(gi) * a.lde + gj) * 2)
                               : kOOB;
      dma16(er, ct.part(h) + (g - h * IPP) * 1024, off, 0);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    __syncthreads();
  }
  // Residual planes are tile-major: lane l of wave w keeps its values of the
  // 32-row block mi, columns ni 32 + 16 h .. (h = 0, 1: two register groups
  // g = 2 h, 2 h + 1) as 16-byte chunk (mi 2 FN + 2 ni + h) of the tile, at
  // chunk * NW KiB + w KiB + 16 l: whole-wave, contiguous 1 KiB accesses.
  constexpr int TILE_LO = BM * BN * 2;
  auto lo_chunk = [&](const char* plane, int ch) {
    return plane + lid * TILE_LO + (ch * NW + wave) * 1024 + elane * 16;
  };
  static_for<FM>([&](auto MI) {
    constexpr int mi = decltype(MI)::value;
    const int il = wm * WM + mi * 32 + (elane & 31);
    u32x4_t lov[2 * FN];   // input residuals of this 32-row block
    u32x4_t lon[2 * FN];   // output residuals
    const bool use_lo = corr && a.lo_in != nullptr;
    if (use_lo) {
#pragma unroll
      for (int ch = 0; ch < 2 * FN; ++ch)
        lov[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(lo_chunk(a.lo_in, mi * 2 * FN + ch)));
    }
    static_for<FN>([&](auto NI) {
      constexpr int ni = decltype(NI)::value;
      static_for<4>([&](auto G) {
        constexpr int g = decltype(G)::value;
        const int jl = wn * WN + ni * 32 + 8 * g + 4 * (elane >> 5);
        float v[4] = {acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2],
                      acc[mi][ni][4 * g + 3]};
        uint2* slot = reinterpret_cast<uint2*>(ct.at(il, jl));
        if (EPI != EPI_SYMSQ) {
          if (use_lo) {
            // + d lo: d per row (wide, X' = B'X) or per column (tall, Y' = YB')
            const u32x4_t lc = lov[2 * ni + g / 2];
            const uint32_t l0 = (g & 1) ? lc.z : lc.x, l1 = (g & 1) ? lc.w : lc.y;
            const float lo[4] = {__uint_as_float(l0 << 16), __uint_as_float(l0 & 0xffff0000u),
                                 __uint_as_float(l1 << 16), __uint_as_float(l1 & 0xffff0000u)};
            float d[4];
            if (TN) {
              d[0] = d[1] = d[2] = d[3] = corr_d[il];
            } else {
              const float4 dv = *reinterpret_cast<const float4*>(corr_d + jl);
              d[0] = dv.x; d[1] = dv.y; d[2] = dv.z; d[3] = dv.w;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = muon::ns_lo_term(v[q], d[q], lo[q]);
          }
          const float f = zero_unit ? 0.0f : s;  // a zero unit's update writes zeros
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = f * v[q];
          if (corr && a.lo_out) {
            float r[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) r[q] = v[q] - muon::bf16_round(v[q]);
            u32x4_t& lo_out = lon[2 * ni + g / 2];
            if (g & 1) {
              lo_out.z = muon::pack_bf16x2(r[0], r[1]);
              lo_out.w = muon::pack_bf16x2(r[2], r[3]);
            } else {
              lo_out.x = muon::pack_bf16x2(r[0], r[1]);
              lo_out.y = muon::pack_bf16x2(r[2], r[3]);
            }
          }
        } else {
          const uint2 w = *slot;
          const float e[4] = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                              __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[q] = a.cb * e[q] + a.cc * v[q];
            if (diag_tile && il == jl + q) {
              v[q] += a.ca;
              // B's diagonal before rounding, for the update's correction
              if (a.dvec != nullptr && m0 + il < a.M) a.dvec[u * static_cast<int64_t>(a.M) + m0 + il] = v[q];
            }
          }
        }
        uint2 w;
        w.x = muon::pack_bf16x2(v[0], v[1]);
        w.y = muon::pack_bf16x2(v[2], v[3]);
        *slot = w;
      });
      // one 32 x 32 block at a time: keeps accumulator reads from being
      // hoisted all together (register pressure)
      __builtin_amdgcn_sched_barrier(0);
    });
    if (corr && a.lo_out) {
#pragma unroll
      for (int ch = 0; ch < 2 * FN; ++ch)
        __builtin_nontemporal_store(lon[ch], reinterpret_cast<u32x4_t*>(
                                                 const_cast<char*>(lo_chunk(a.lo_out, mi * 2 * FN + ch))));
    }
  });
  __syncthreads();

  // Stores go through a buffer descriptor: 32-bit offsets (a unit is under
  // 2 GiB), and a chunk outside the matrix gets an offset past the buffer's
  // size, which the hardware drops.
  const bf16_t* dst = uniform_ptr(reinterpret_cast<const bf16_t*>(mat_at(a.dst, u)));
  const __amdgpu_buffer_rsrc_t dr =
      make_rsrc(dst, static_cast<uint32_t>(static_cast<int64_t>(a.M) * a.ldd * 2));
  const int ldd = static_cast<int>(a.ldd);
  const bool diag = (EPI != EPI_UPDATE) && diag_tile;
  constexpr int CH = BN / 8;  // 16-byte chunks per tile row
  // primary: C rows, 16-byte row-contiguous stores (a diagonal tile of a
  // symmetric output takes its lower half from the mirrored upper half)
#pragma unroll
  for (int it = 0; it < BM * CH / NT; ++it) {
    const int e = etid + it * NT;
    const int rl = e / CH, c = e % CH;
    const int i = m0 + rl, j = n0 + 8 * c;
    u32x4_t val;
    if (!diag || 8 * c >= rl) {
      val = *reinterpret_cast<const u32x4_t*>(ct.at(rl, 8 * c));
    } else {
      uint16_t h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int cl = 8 * c + q;
        h[q] = (cl >= rl) ? *reinterpret_cast<const uint16_t*>(ct.at(rl, cl))
                          : *reinterpret_cast<const uint16_t*>(ct.at(cl, rl));
      }
      val = __builtin_bit_cast(u32x4_t, h);
    }
    const uint32_t off = (i < a.M && j < a.N) ? static_cast<uint32_t>(i * ldd + j) * 2u : kOOB;
    // the update's output is read back only by the next launch, after far
    // more traffic than the caches hold: store it non-temporally (nt)
    __builtin_amdgcn_raw_buffer_store_b128(val, dr, off, 0, EPI == EPI_UPDATE ? 2 : 0);
  }
  if (EPI != EPI_UPDATE && !diag) {
    // mirror: row j of the output gets C[i .. i + 7][j] from two transposed
    // reads; blocks of 32 columns x 16 rows, one per wave at a time
    constexpr int BJ = BN / 32, BI = BM / 16;
    const int gq = elane >> 4, jx = elane & 15;
    for (int b = wave; b < BJ * BI; b += NW) {
      const int jb = (b % BJ) * 32, ib = (b / BJ) * 16;
      const int col = jb + 16 * (gq & 1) + 4 * (jx & 3);
      const int row = ib + 8 * (gq >> 1) + (jx >> 2);
      const i16x4_t lo = ld_tr16(ct.at(row, col));
      const i16x4_t hi = ld_tr16(ct.at(row + 4, col));
      const int jl = jb + 16 * (gq & 1) + jx;  // column of C = output row
      const int il = ib + 8 * (gq >> 1);       // first of 8 rows of C = output column
      const int orow = n0 + jl, ocol = m0 + il;
      const short v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const uint32_t off =
          (orow < a.N && ocol < a.M) ? static_cast<uint32_t>(orow * ldd + ocol) * 2u : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), dr, off, 0, 0);
    }
  }
  // the next tile's loads overwrite the staging area: every wave must have
  // read its part first (the stores themselves may still be in flight)
  __syncthreads();
  }
}

template <int T, bool TM, bool TN, int EPI>
hipError_t go(hipStream_t s, const NsGemmArgs& a) {
  // 256 x 256 tiles: 8 waves (two per SIMD) of 128 x 64; 128 x 128: 4 waves
  // of 64 x 64.  BK = 64, two stage buffers.
  constexpr int NWN = T == 256 ? 4 : 2;
  constexpr int BK = 64, NS = 2;
  const int64_t tiles = a.units * a.tiles_per_unit;
  if (tiles <= 0) return hipSuccess;
  // one workgroup per CU for 256-tiles (LDS and registers of a CU), two for
  // 128-tiles; each walks its tiles in turn
  const int64_t cap = static_cast<int64_t>(a.cus > 0 ? a.cus : 256) * (T == 256 ? 1 : 2);
  const int64_t grid = tiles < cap ? tiles : cap;
  ns_gemm_mfma_kernel<T, T, NWN, BK, NS, TM, TN, EPI><<<static_cast<unsigned>(grid), 128 * NWN, 0, s>>>(a);
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
