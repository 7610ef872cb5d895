// Device-side helpers shared by the dmx kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmx {

// Suffix-layer shape constants (shape table of the OpenDM DM0.5 fast-stack
// article, §2.2).
constexpr int kH = 1024;          // hidden
constexpr int kI = 4096;          // intermediate
constexpr int kD = 256;           // head_dim
constexpr int kHQ = 8;            // query heads
constexpr int kHK = 4;            // KV heads
constexpr int kGroup = kHQ / kHK; // query heads per KV head
constexpr int kQKV = (kHQ + 2 * kHK) * kD;  // 4096 projected features
constexpr float kEps = 1e-6f;

// MFMA operand types: 8 bf16 (as raw 16-bit) per lane, fp32 accumulators.
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// float -> bf16 bits with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// v if keep, else zeros, selected per component (a select of whole vector
// structs can be lowered through private memory)
__device__ __forceinline__ uint4 keep_or_zero(bool keep, uint4 v) {
  return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = 0;
  return z;
}

__device__ __forceinline__ f32x4 zero_f32x4() {
  f32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

// D += A * B for a 16x16 output tile over 32 reduction elements.
// Lane l: A row l%16, B column l%16, both at reduction offsets 8*(l/16)..+7;
// D holds rows 4*(l/16)+0..3 of column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float group16_sum(float v);

// sum over the 64 lanes: DPP inside each 16-lane row, then across the 4 rows
__device__ __forceinline__ float wave_sum(float v) {
  v = group16_sum(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Reductions inside each aligned row of 16 lanes with DPP row rotations (no
// LDS crossbar traffic): after the four steps every lane of the row holds the
// result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

__device__ __forceinline__ float group16_sum(float v) {
  v += dpp_f<kRowRor1>(v);
  v += dpp_f<kRowRor2>(v);
  v += dpp_f<kRowRor4>(v);
  v += dpp_f<kRowRor8>(v);
  return v;
}

// GELU, tanh form: 0.5 z (1 + tanh u), u = sqrt(2/pi) (z + 0.044715 z^3),
// evaluated through the identity 0.5 (1 + tanh u) = 1 / (1 + e^(-2u)) with
// the hardware base-2 exponential and reciprocal (each ~1 ulp).  Large |u|
// saturate correctly: e^(-2u) -> inf gives -0, -> 0 gives z.
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float e = __builtin_amdgcn_exp2f(c2 * (z + 0.044715f * z * z * z));
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// one 16-byte-per-lane load from global memory straight into LDS: lane i's
// 16 bytes land at lds_dst + 16 i (lds_dst uniform across the wave)
__device__ __forceinline__ void lds_copy16(const uint16_t* src, uint16_t* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}
// work-group barrier that orders LDS traffic around it (no memory fence, so
// loads into LDS that are still in flight are not waited for)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace dmx
