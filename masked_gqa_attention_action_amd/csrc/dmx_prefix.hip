// Prefix (prefill) decoder layer pieces that are not projections or
// attention (OpenDM fast-stack article, §2.2, prefix row of the shape table
// and fusion list: image features merged into the input embeddings, a norm
// after the attention followed by the residual; the layer is the Gemma3-4B
// decoder the table names): RMS norms with the (1 + w) weight, the residual
// adds around them, and the image-feature merge.  Rows are tokens of one
// request; hidden 2560.  The norms take 8 rows per work-group, one per wave,
// each lane owning 5 pieces of 8 consecutive features (16-byte loads): the
// 16-byte pieces they write into the tiled layout then fill whole 128-byte
// lines (8 rows of one 32-column step) inside one work-group, where one row
// per work-group left every line to be merged from 8 work-groups.
#include "dmx_device.hpp"
#include "dmx_internal.hpp"
#include "dmx_tiles.hpp"

namespace dmx {

namespace {
constexpr int kPH = kPrefixHidden;
constexpr int kNormRows = 8;           // rows (waves) per work-group
constexpr int kPieces = kPH / 8 / 64;  // 8-feature pieces per lane: 5
static_assert(kPieces * 8 * 64 == kPH, "whole pieces");

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

// 1 / rms of the wave's row, lane l holding features (64 p + l) * 8 .. + 7 in
// v[p]: each piece's squares summed in order, each piece summed over the
// wave (lane 0's sum: the rotating reduction rounds differently per lane),
// the piece sums added in piece order
__device__ __forceinline__ float row_rscale(const float v[kPieces][8]) {
  float t = 0.f;
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[p][i] * v[p][i];
    t += __shfl(wave_sum(ss), 0, 64);
  }
  return 1.0f / sqrtf(t * (1.0f / kPH) + kEps);
}
}  // namespace

// xn = rmsnorm(x; w) of row-major bf16 rows, written tiled (a GEMM's A operand)
__global__ __launch_bounds__(64 * kNormRows) void k_prefix_rmsnorm(const uint16_t* x, const uint16_t* w, int T,
                                                                   uint16_t* out) {
  const int lane = threadIdx.x & 63, t = blockIdx.x * kNormRows + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[kPieces][8];
#pragma unroll
  for (int p = 0; p < kPieces; ++p) ld8(x + (size_t)t * kPH + (p * 64 + lane) * 8, v[p]);
  const float r = row_rscale(v);
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const int c = (p * 64 + lane) * 8;
    float wv[8];
    ld8(w + c, wv);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[p][i] = v[p][i] * r * (1.f + wv[i]);
    *reinterpret_cast<uint4*>(out + tile_off(t, c, kPH)) = pk8(v[p]);
  }
}

// x1 = resid + rmsnorm(y; w_post) for projection rows y (fp32, row-major by
// tiled row).  resid is fp32 (x1 of the same layer) or, when resid_f32 is
// null, the bf16 row-major layer input.  Outputs (each optional): x1 in fp32,
// rmsnorm(x1; w_next) tiled bf16, bf16(x1) row-major.
__global__ __launch_bounds__(64 * kNormRows) void k_prefix_post_norm(const float* y, const float* resid_f32,
                                                                     const uint16_t* resid_bf16, const uint16_t* w_post,
                                                                     const uint16_t* w_next, int T, float* x1_out,
                                                                     uint16_t* xn_tiled, uint16_t* out_bf16) {
  const int lane = threadIdx.x & 63, t = blockIdx.x * kNormRows + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[kPieces][8], rs[kPieces][8];
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const size_t o = (size_t)t * kPH + (p * 64 + lane) * 8;
    ld8(y + o, v[p]);
    if (resid_f32)
      ld8(resid_f32 + o, rs[p]);
    else
      ld8(resid_bf16 + o, rs[p]);
  }
  const float r = row_rscale(v);
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const int c = (p * 64 + lane) * 8;
    float wv[8];
    ld8(w_post + c, wv);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[p][i] = rs[p][i] + v[p][i] * r * (1.f + wv[i]);
    const size_t o = (size_t)t * kPH + c;
    if (x1_out) {
      *reinterpret_cast<float4*>(x1_out + o) = make_float4(v[p][0], v[p][1], v[p][2], v[p][3]);
      *reinterpret_cast<float4*>(x1_out + o + 4) = make_float4(v[p][4], v[p][5], v[p][6], v[p][7]);
    }
    if (out_bf16) *reinterpret_cast<uint4*>(out_bf16 + o) = pk8(v[p]);
  }
  if (w_next) {
    const float r2 = row_rscale(v);
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
      const int c = (p * 64 + lane) * 8;
      float wv[8], xn[8];
      ld8(w_next + c, wv);
#pragma unroll
      for (int i = 0; i < 8; ++i) xn[i] = v[p][i] * r2 * (1.f + wv[i]);
      *reinterpret_cast<uint4*>(xn_tiled + tile_off(t, c, kPH)) = pk8(xn);
    }
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
  k_prefix_rmsnorm<<<dim3((T + kNormRows - 1) / kNormRows), dim3(64 * kNormRows), 0, s>>>(x, w, T, out);
  return hipGetLastError();
}

hipError_t launch_prefix_post_norm(const float* y, const float* resid_f32, const uint16_t* resid_bf16,
                                   const uint16_t* w_post, const uint16_t* w_next, int T, float* x1_out,
                                   uint16_t* xn_tiled, uint16_t* out_bf16, hipStream_t s) {
  k_prefix_post_norm<<<dim3((T + kNormRows - 1) / kNormRows), dim3(64 * kNormRows), 0, s>>>(
      y, resid_f32, resid_bf16, w_post, w_next, T, x1_out, xn_tiled, out_bf16);
  return hipGetLastError();
}

hipError_t launch_image_merge(const uint16_t* tok, const uint16_t* img, const int32_t* idx, int T, int n_img,
                              int hidden, uint16_t* out, hipStream_t s) {
  const long n = (long)T * (hidden / 8);
  k_image_merge<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(tok, img, idx, T, n_img, hidden, out);
  return hipGetLastError();
}

}  // namespace dmx
