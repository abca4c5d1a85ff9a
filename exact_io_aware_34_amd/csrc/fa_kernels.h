// Internal interface between the host API (fa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
constexpr int MASK_TILE = 128;  // block-mask granularity (rows and columns)
constexpr int FWD_BR = 128;     // query rows per forward workgroup (== MASK_TILE)

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const uint8_t* mask;  // nullptr = dense
  int BH, N;
  int n_qtiles, n_ktiles, mask_tiles;
  float scale, scale_log2e;
  float rescale_thr;  // raw-score growth of the running max that forces a rescale
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // workspace: D_i = sum_c dO_ic o_ic, (B*H, N)
  const uint8_t* mask;
  int BH, N;
  int n_ktiles, n_qtiles, mask_tiles;
  float scale, scale_log2e;
};

hipError_t launch_forward(FwdParams p, int dtype, int d, bool causal, hipStream_t st);
hipError_t launch_backward(BwdParams p, int dtype, int d, bool causal, hipStream_t st);

}  // namespace fa
