// One unit of a modulation GEMV (fast-stack article §2.2, the time
// modulation of AdaRMS): 16 output features `tile` of out[b] = W cond[b] +
// bias for every request b, W tiled [3072][1024] bf16.  256 threads: wave w
// takes the reduction columns 256 w .. +255 (8 MFMA steps of 32), its 32 KB
// weight slab loaded at once with streaming loads; the four wave sums meet
// in `red` (4 x 256 floats of LDS) and are added in wave order.  Shared by
// the modulation kernel and the work-groups the attention launch runs on
// its idle CUs, so both give the same bits.
#pragma once
#include "dmx_device.hpp"
#include "dmx_internal.hpp"

namespace dmx {

__device__ __forceinline__ void mod_unit(const ModJob& job, int tile, int B, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int k0 = wave * 256;
  bf16x8 wf[8];
  const uint16_t* wp = job.w + ((size_t)tile * (kH / 32) + wave * 8) * 512 + lane * 8;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)  // read once per launch: streaming loads
    wf[ks] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(wp + ks * 512));
  const uint16_t* cond = job.cond;
  for (int b0 = 0; b0 < B; b0 += 16) {
    const int rows = min(16, B - b0);
    f32x4 acc = zero_f32x4();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 av = lr < rows ? load_bf16x8(cond + (size_t)(b0 + lr) * kH + k0 + ks * 32 + lk) : zero_bf16x8();
      acc = mfma16(av, wf[ks], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave * 256 + ((lane >> 4) * 4 + r) * 16 + lr] = acc[r];
    __syncthreads();
    if (threadIdx.x < rows * 16) {
      const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
      const float v = red[r * 16 + c] + red[256 + r * 16 + c] + red[512 + r * 16 + c] + red[768 + r * 16 + c];
      const int n = tile * 16 + c;
      job.out[(size_t)(b0 + r) * 3 * kH + n] = v + bf2f(job.bias[n]);
    }
    __syncthreads();
  }
}

}  // namespace dmx
