// fmoe_fused_args.h -- argument block of the one-launch layer kernel, shared
// by the host dispatch and the kernel.
#pragma once

#include <stdint.h>

#include "fmoe_internal.h"

namespace fmoe {

// Counter and flag block at the start of the workspace (176 lines of 256 B).
constexpr int kFusedCtrLines = 176;
constexpr size_t kFusedCtrBytes = (size_t)kFusedCtrLines * 256;

struct FusedArgs {
  ExpertSrc src;
  const float* Wr;
  const float* wsg;
  const float* x;
  const float* resid;
  const float* gamma;
  float* h_out;
  float* y_out;
  float* moe_out;
  float* w_out;
  int32_t* idx_out;
  float eps;
  int H, I, E, k;
  double* lg64;      // [E+1]
  float* abuf;       // [(k+1) * I]
  uint8_t* aprep;    // [(k+1) * xprep_bytes(I)]
  int* ccnt;         // [(k+1) * I/32]
  float* partials;   // [nD]
  int* ctr;          // FusedCtr
  int nR, nGU, nD;   // item counts per phase
  int gu_rows;       // gate/up rows per item
  int d_rows;        // down rows per item
};

}  // namespace fmoe
