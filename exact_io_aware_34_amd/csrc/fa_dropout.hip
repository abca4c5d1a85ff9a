// The dropout keep mask written out: one thread per 4 x 4 (query, key)
// block, i.e. one Philox-4x32-10 call (see philox4x32_10 in fa_device.h for
// the mapping of elements to random bytes).  The attention kernels never
// store the mask -- they regenerate it where they need it; this kernel lets
// a caller or a test see exactly the mask those kernels apply.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

__global__ __launch_bounds__(256) void dropout_mask_kernel(DropMaskParams p) {
  const long long nq = (p.N + 3) / 4;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= (long long)p.BH * nq * nq) return;
  const int bh = (int)(t / (nq * nq));
  const long long rem = t - (long long)bh * nq * nq;
  const int iq = (int)(rem / nq), jq = (int)(rem - (long long)iq * nq);
  const u32x4 r = philox4x32_10((uint32_t)jq, (uint32_t)iq, (uint32_t)bh, p.off, p.k0, p.k1);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int i = 4 * iq + w;
    if (i >= p.N) break;
    uint8_t* row = p.keep + ((size_t)bh * p.N + i) * p.N;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = 4 * jq + b;
      if (j < p.N) row[j] = ((r[w] >> (8 * b)) & 0xFFu) >= p.t8 ? 1 : 0;
    }
  }
}

}  // namespace

hipError_t launch_dropout_mask(DropMaskParams p, hipStream_t st) {
  const long long nq = (p.N + 3) / 4;
  const long long threads = (long long)p.BH * nq * nq;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     p);
  return hipGetLastError();
}

}  // namespace fa
