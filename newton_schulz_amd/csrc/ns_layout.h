// Workspace layout of one Newton-Schulz call (host only).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "muon.h"

// Per call: `units` Newton-Schulz units of ur x uc (m = min, n = max).
// Regions (byte offsets into the workspace, 256-byte aligned):
//   xa, xb   two m*n iterate buffers        (ping-pong)
//   a, b     two m*m buffers                (A = X X^T, B' = aI + bA + cA^2)
//   scale    float per unit                 1 / (||Y||_F + eps)
//   zflag    int per unit                   ||Y||_F == 0
//   partial  double per unit and part       norm partial sums
//   lo       bf16 residual plane per unit   the iterate's part below bf16
//            (BF16 compute only; padded to whole 256 x 256 tiles once
//            m >= 256, else 128 x 128, which also holds the 128-tiles that
//            ns_mfma_tile may pick for m >= 256)
//   dvec     float per unit and row of A    diagonal of B' before rounding
// BF16 units whose smaller side is under kNsTinySide run the iteration in
// fp32 instead (their bf16 A and B' alone take some Gaussian draws past the
// bf16 error bar): the slab then starts with the inputs widened to fp32
// (stage, 4 bytes per element), followed at `sub` by the fp32 layout of the
// same units; total covers both layouts.
constexpr int64_t kNsTinySide = 16;
struct NsLayout {
  int64_t units = 0, ur = 0, uc = 0, m = 0, n = 0;
  int parts = 1;  // norm partial sums per unit
  size_t lo_unit = 0;  // residual plane bytes per unit
  size_t xa = 0, xb = 0, a = 0, b = 0, scale = 0, zflag = 0, partial = 0, lo = 0, dvec = 0,
         stage = 0, sub = 0, total = 0;
};

bool ns_layout(const muon_shape_t& s, int64_t count, int32_t compute, NsLayout* L);

// Output tile side of one bf16 MFMA product launch over `units` outputs of
// rows x cols (upper-triangle tiles only when `upper`): 256 once the smaller
// side reaches 256, else 128 -- and 128 also where the launch has so few
// 256-tiles that 128-tiles, two workgroups per CU, finish sooner.  Every
// accumulator sums the same products in the same order at either size, so
// the choice changes the time, not the result.
int ns_mfma_tile(int64_t rows, int64_t cols, bool upper, int64_t units, int cus);
