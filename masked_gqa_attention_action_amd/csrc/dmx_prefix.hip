// Prefix (prefill) decoder layer pieces that are not projections or
// attention (OpenDM fast-stack article, §2.2, prefix row of the shape table
// and fusion list: image features merged into the input embeddings, a norm
// after the attention followed by the residual; the layer is the Gemma3-4B
// decoder the table names): RMS norms with the (1 + w) weight, the residual
// adds around them, and the image-feature merge.  Rows are tokens of one
// request; hidden 2560.  One work-group of 320 threads per row, each thread
// owning 8 consecutive features (16-byte loads).
#include "dmx_device.hpp"
#include "dmx_internal.hpp"
#include "dmx_tiles.hpp"

namespace dmx {

namespace {
constexpr int kPH = kPrefixHidden;
constexpr int kPThreads = kPH / 8;  // 320
static_assert(kPThreads % 64 == 0, "whole waves");

__device__ __forceinline__ void ld8(const uint16_t* p, float v[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf2f((uint16_t)(w[i] & 0xffffu));
    v[2 * i + 1] = bf2f((uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ void ld8(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ uint4 pk8(const float v[8]) {
  return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
}

// 1 / rms of a row whose 8 values per thread are v (sum over the work-group)
__device__ __forceinline__ float row_rscale(const float v[8], float* red) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  ss = wave_sum(ss);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red is free again
  if ((threadIdx.x & 63) == 0) red[wave] = ss;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kPThreads / 64; ++w) t += red[w];
  return 1.0f / sqrtf(t * (1.0f / kPH) + kEps);
}
}  // namespace

// xn = rmsnorm(x; w) of row-major bf16 rows, written tiled (a GEMM's A operand)
__global__ __launch_bounds__(kPThreads) void k_prefix_rmsnorm(const uint16_t* x, const uint16_t* w, uint16_t* out) {
  __shared__ float red[kPThreads / 64];
  const int t = blockIdx.x, c = threadIdx.x * 8;
  float v[8], wv[8];
  ld8(x + (size_t)t * kPH + c, v);
  ld8(w + c, wv);
  const float r = row_rscale(v, red);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * r * (1.f + wv[i]);
  *reinterpret_cast<uint4*>(out + tile_off(t, c, kPH)) = pk8(v);
}

// x1 = resid + rmsnorm(y; w_post) for projection rows y (fp32, row-major by
// tiled row).  resid is fp32 (x1 of the same layer) or, when resid_f32 is
// null, the bf16 row-major layer input.  Outputs (each optional): x1 in fp32,
// rmsnorm(x1; w_next) tiled bf16, bf16(x1) row-major.
__global__ __launch_bounds__(kPThreads) void k_prefix_post_norm(const float* y, const float* resid_f32,
                                                               const uint16_t* resid_bf16, const uint16_t* w_post,
                                                               const uint16_t* w_next, float* x1_out,
                                                               uint16_t* xn_tiled, uint16_t* out_bf16) {
  __shared__ float red[kPThreads / 64];
  const int t = blockIdx.x, c = threadIdx.x * 8;
  float v[8], wv[8], rs[8];
  ld8(y + (size_t)t * kPH + c, v);
  ld8(w_post + c, wv);
  if (resid_f32)
    ld8(resid_f32 + (size_t)t * kPH + c, rs);
  else
    ld8(resid_bf16 + (size_t)t * kPH + c, rs);
  const float r = row_rscale(v, red);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = rs[i] + v[i] * r * (1.f + wv[i]);
  if (x1_out) {
    *reinterpret_cast<float4*>(x1_out + (size_t)t * kPH + c) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(x1_out + (size_t)t * kPH + c + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  if (out_bf16) *reinterpret_cast<uint4*>(out_bf16 + (size_t)t * kPH + c) = pk8(v);
  if (w_next) {
    float xn[8];
    ld8(w_next + c, wv);
    const float r2 = row_rscale(v, red);
#pragma unroll
    for (int i = 0; i < 8; ++i) xn[i] = v[i] * r2 * (1.f + wv[i]);
    *reinterpret_cast<uint4*>(xn_tiled + tile_off(t, c, kPH)) = pk8(xn);
  }
}

// out[t] = img[idx[t]] when 0 <= idx[t] < n_img, tok[t] when idx[t] < 0; an
// index past the image rows gives a zero row.  One thread per 16 bytes.
__global__ __launch_bounds__(256) void k_image_merge(const uint16_t* tok, const uint16_t* img, const int32_t* idx,
                                                    int T, int n_img, int hidden, uint16_t* out) {
  const int per_row = hidden / 8;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)T * per_row) return;
  const int t = (int)(i / per_row), c = (int)(i - (long)t * per_row) * 8;
  const int s = idx[t];
  uint4 val = make_uint4(0u, 0u, 0u, 0u);
  if (s < 0)
    val = *reinterpret_cast<const uint4*>(tok + (size_t)t * hidden + c);
  else if (s < n_img)
    val = *reinterpret_cast<const uint4*>(img + (size_t)s * hidden + c);
  *reinterpret_cast<uint4*>(out + (size_t)t * hidden + c) = val;
}

hipError_t launch_prefix_rmsnorm(const uint16_t* x, const uint16_t* w, int T, uint16_t* out, hipStream_t s) {
  k_prefix_rmsnorm<<<dim3(T), dim3(kPThreads), 0, s>>>(x, w, out);
  return hipGetLastError();
}

hipError_t launch_prefix_post_norm(const float* y, const float* resid_f32, const uint16_t* resid_bf16,
                                   const uint16_t* w_post, const uint16_t* w_next, int T, float* x1_out,
                                   uint16_t* xn_tiled, uint16_t* out_bf16, hipStream_t s) {
  k_prefix_post_norm<<<dim3(T), dim3(kPThreads), 0, s>>>(y, resid_f32, resid_bf16, w_post, w_next, x1_out,
                                                        xn_tiled, out_bf16);
  return hipGetLastError();
}

hipError_t launch_image_merge(const uint16_t* tok, const uint16_t* img, const int32_t* idx, int T, int n_img,
                              int hidden, uint16_t* out, hipStream_t s) {
  const long n = (long)T * (hidden / 8);
  k_image_merge<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(tok, img, idx, T, n_img, hidden, out);
  return hipGetLastError();
}

}  // namespace dmx
