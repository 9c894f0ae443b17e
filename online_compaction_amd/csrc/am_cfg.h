// Attention Matching: launch constants shared by the fit's kernels and its host entry point.
#pragma once

#include "kvc_internal.h"

namespace kvc {

// Attention Matching launch constants: H heads, R proxy rows, m_max the stride of the per-unit
// outputs; S1, S2 the split counts of the two P_C products (P_C V and P_C^T Z) and St that of
// the target's keys; mode and xsel select a product's epilogue and which of the two
// transposed-operand buffers it reads (both set per launch by the host).
struct AmCfg {
  int H, R, m_max, S1, S2, St, mode, xsel;
};
// The value fit iterates on the smaller side of P_C (R x m): with R <= m (padded to 64) the
// residual Z = P_C V - Y lives on the R proxy rows and the Gram matrix is P_C P_C^T; otherwise
// on the m kept keys with P_C^T P_C. Host and device decide it the same way.
__host__ __device__ inline bool am_rows_side(int R, int m) { return ((R + 63) & ~63) <= ((m + 63) & ~63); }

}  // namespace kvc
