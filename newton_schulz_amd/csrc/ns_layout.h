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
//            (BF16 compute only; tile-padded: the products' tiles of T x T,
//            T = 256 once m >= 256, else 128)
//   dvec     float per unit and row of A    diagonal of B' before rounding
struct NsLayout {
  int64_t units = 0, ur = 0, uc = 0, m = 0, n = 0;
  int parts = 1;  // norm partial sums per unit
  size_t lo_unit = 0;  // residual plane bytes per unit
  size_t xa = 0, xb = 0, a = 0, b = 0, scale = 0, zflag = 0, partial = 0, lo = 0, dvec = 0,
         total = 0;
};

bool ns_layout(const muon_shape_t& s, int64_t count, int32_t compute, NsLayout* L);
