// Denoise sampler kernels around the action-expert stack.  The pages describe
// the action chunk as decoded by diffusion over a fixed number of steps
// (OpenDM fast-stack article §1 and §4; DM05 inference guide §2, the
// diffusion step count) but give no formula for the sampler.  The readings
// implemented here:
//   t_k = 1 - k / n;  temb(t) = [sin(1000 t w_i) | cos(1000 t w_i)],
//   w_i = 10000^(-i / 512);  cond = swish(W_t2 swish(W_t1 temb + b_t1) + b_t2);
//   x = W_in a + b_in per chunk token;  after the layers, the final AdaRMS
//   norm with [scale | shift] = W_f cond + b_f, v = W_out xf + b_out, and the
//   Euler step a <- a - v / n.
// The schedule side (temb, time MLP, final modulation) depends on the step
// only and runs once per schedule; per step, the stack is bracketed by the
// action in-projection and the fused final norm + out-projection + Euler
// update, the latter fused with the next step's in-projection (and its input
// pack) between steps.
#include "dmx_device.hpp"
#include "dmx_internal.hpp"
#include "dmx_tiles.hpp"

namespace dmx {

// temb of every step of an n-step schedule, bf16 [n][1024].  Angles and their
// sine / cosine in double precision; one bf16 rounding at the end.
__global__ __launch_bounds__(512) void k_time_embed(int n_steps, uint16_t* temb) {
  const int s = blockIdx.x, i = threadIdx.x;
  const double t = 1.0 - (double)s / n_steps;
  const double ang = 1000.0 * t * pow(10000.0, -(double)i / (kH / 2));
  temb[(size_t)s * kH + i] = f2bf((float)sin(ang));
  temb[(size_t)s * kH + kH / 2 + i] = f2bf((float)cos(ang));
}

// Rows of a small batch through one linear layer:
//   y[r][n] = act(W[n] . x[r] + bias[n]),  W tiled [N][1024], x bf16 rows
// x_stride elements apart.  Work-group = 16 output features (N / 16 groups);
// its 32 KB weight slab sits in registers while 16-row blocks of x stream by.
// Outputs (each optional): fp32 [R][ldo]; bf16 [R * rep][N] with each row
// written rep times (row r's copies at r * rep .. r * rep + rep - 1).
template <bool SWISH>
__global__ __launch_bounds__(256) void k_gemv_rows(const uint16_t* W, const uint16_t* bias, const uint16_t* x,
                                                  int x_stride, int R, float* out_f32, int ldo, uint16_t* out_bf16,
                                                  int rep) {
  __shared__ float red[4][16 * 16];
  const int tile = blockIdx.x, N = gridDim.x * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int k0 = wave * 256;
  bf16x8 wf[8];
  const uint16_t* wp = W + ((size_t)tile * (kH / 32) + wave * 8) * 512 + lane * 8;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) wf[ks] = load_bf16x8(wp + ks * 512);
  for (int r0 = 0; r0 < R; r0 += 16) {
    const int rows = min(16, R - r0);
    f32x4 acc = zero_f32x4();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 av = lr < rows ? load_bf16x8(x + (size_t)(r0 + lr) * x_stride + k0 + ks * 32 + lk) : zero_bf16x8();
      acc = mfma16(av, wf[ks], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][((lane >> 4) * 4 + r) * 16 + lr] = acc[r];
    __syncthreads();
    if (threadIdx.x < rows * 16) {
      const int r = threadIdx.x >> 4, c = threadIdx.x & 15, n = tile * 16 + c;
      float v = red[0][r * 16 + c] + red[1][r * 16 + c] + red[2][r * 16 + c] + red[3][r * 16 + c] + bf2f(bias[n]);
      if (SWISH) v = v / (1.0f + expf(-v));
      if (out_f32) out_f32[(size_t)(r0 + r) * ldo + n] = v;
      if (out_bf16) {
        const uint16_t h = f2bf(v);
        for (int i = 0; i < rep; ++i) out_bf16[((size_t)(r0 + r) * rep + i) * N + n] = h;
      }
    }
    __syncthreads();
  }
}

// x[row] = bf16(W_in a[row] + b_in): a fp32 [rows][A], W_in bf16 [1024][A]
// row-major, x bf16 [rows][1024].  One work-group per token row, 4 features
// per thread.
__global__ __launch_bounds__(256) void k_action_in(const float* a, const uint16_t* w_in, const uint16_t* b_in, int A,
                                                  uint16_t* x) {
  __shared__ float sa[kMaxActionDim];
  const int row = blockIdx.x;
  if (threadIdx.x < A) sa[threadIdx.x] = a[(size_t)row * A + threadIdx.x];
  __syncthreads();
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = threadIdx.x * 4 + i;
    const uint16_t* wr = w_in + (size_t)n * A;
    float acc = 0.f;
    for (int j = 0; j < A; j += 8) {
      const uint4 raw = *reinterpret_cast<const uint4*>(wr + j);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += bf2f((uint16_t)(w4[e] & 0xffffu)) * sa[j + 2 * e];
        acc += bf2f((uint16_t)(w4[e] >> 16)) * sa[j + 2 * e + 1];
      }
    }
    y[i] = acc + bf2f(b_in[n]);
  }
  *reinterpret_cast<uint2*>(x + (size_t)row * kH + threadIdx.x * 4) = make_uint2(pack2(y[0], y[1]), pack2(y[2], y[3]));
}

// The step's velocity and Euler update for one token row:
//   xf = x / sqrt(mean x^2 + eps) * (1 + scale) + shift   (fmod = [scale | shift])
//   v  = W_out xf + b_out;  a += dt * v  (and traj = a when given)
// x bf16 [rows][1024] (the stack's output), W_out bf16 [A][1024] row-major,
// a / traj fp32 [rows][A].  256 threads per row: thread t normalises columns
// 4t .. 4t+3 into LDS; for the out-projection 8 threads share one output j
// (32 outputs per pass), thread p of the 8 taking the 16-byte column groups
// p, p + 8, ... (so one LDS read instruction spans 256 contiguous bytes); the
// 8 partial sums are added by a 3-step butterfly.  The W_out groups of the
// first pass are loaded before anything else.  The row's new actions end in
// sa[0 .. A).
template <int A>
struct VelPre {
  uint2 x;         // columns 4t .. 4t+3 of the row
  uint4 w[16];     // W_out groups of pass 0
};

template <int A>
__device__ __forceinline__ void velocity_prefetch(const uint16_t* x, const uint16_t* w_out, int row, VelPre<A>& p) {
  const int jo = threadIdx.x >> 3, q = threadIdx.x & 7;
  p.x = *reinterpret_cast<const uint2*>(x + (size_t)row * kH + threadIdx.x * 4);
  const uint16_t* wr = w_out + (size_t)min(jo, A - 1) * kH + q * 8;
#pragma unroll
  for (int i = 0; i < 16; ++i) p.w[i] = *reinterpret_cast<const uint4*>(wr + i * 64);
}

__device__ __forceinline__ float dot8(const uint4 w, const float* xf) {
  const float4 x0 = *reinterpret_cast<const float4*>(xf);
  const float4 x1 = *reinterpret_cast<const float4*>(xf + 4);
  float t = bf2f((uint16_t)(w.x & 0xffffu)) * x0.x;
  t += bf2f((uint16_t)(w.x >> 16)) * x0.y;
  t += bf2f((uint16_t)(w.y & 0xffffu)) * x0.z;
  t += bf2f((uint16_t)(w.y >> 16)) * x0.w;
  t += bf2f((uint16_t)(w.z & 0xffffu)) * x1.x;
  t += bf2f((uint16_t)(w.z >> 16)) * x1.y;
  t += bf2f((uint16_t)(w.w & 0xffffu)) * x1.z;
  t += bf2f((uint16_t)(w.w >> 16)) * x1.w;
  return t;
}

template <int A>
__device__ __forceinline__ void row_velocity(const VelPre<A>& p, const float* fmod, const uint16_t* w_out,
                                             const uint16_t* b_out, float dt, float* a, float* traj, int row,
                                             float* sx, float* rss, float* sa) {
  const int c = threadIdx.x * 4, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float v[4] = {bf2f((uint16_t)(p.x.x & 0xffffu)), bf2f((uint16_t)(p.x.x >> 16)), bf2f((uint16_t)(p.x.y & 0xffffu)),
                bf2f((uint16_t)(p.x.y >> 16))};
  const float ss = wave_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
  if (lane == 0) rss[wave] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf((rss[0] + rss[1] + rss[2] + rss[3]) * (1.0f / kH) + kEps);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = v[i] * r * (1.f + fmod[c + i]) + fmod[kH + c + i];
  *reinterpret_cast<float4*>(sx + c) = make_float4(v[0], v[1], v[2], v[3]);
  __syncthreads();
  const int jo = threadIdx.x >> 3, q = threadIdx.x & 7;
#pragma unroll
  for (int pass = 0; pass < (A + 31) / 32; ++pass) {
    const int j = pass * 32 + jo;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 w = pass == 0 ? p.w[i]
                                : *reinterpret_cast<const uint4*>(w_out + (size_t)min(j, A - 1) * kH + (i * 8 + q) * 8);
      acc += dot8(w, sx + (i * 8 + q) * 8);
    }
    acc += __shfl_xor(acc, 1, 64);
    acc += __shfl_xor(acc, 2, 64);
    acc += __shfl_xor(acc, 4, 64);
    if (j < A && q == 0) {
      const float an = a[(size_t)row * A + j] + dt * (acc + bf2f(b_out[j]));
      a[(size_t)row * A + j] = an;
      if (traj) traj[(size_t)row * A + j] = an;
      sa[j] = an;
    }
  }
}

template <int A>
__global__ __launch_bounds__(256) void k_final_velocity(const uint16_t* x, const float* fmod, const uint16_t* w_out,
                                                       const uint16_t* b_out, float dt, float* a, float* traj) {
  __shared__ __attribute__((aligned(16))) float sx[kH];
  __shared__ float rss[4], sa[A];
  VelPre<A> p;
  velocity_prefetch<A>(x, w_out, blockIdx.x, p);
  row_velocity<A>(p, fmod, w_out, b_out, dt, a, traj, blockIdx.x, sx, rss, sa);
}

// The end of step k and the start of step k + 1 for one token row, fused:
// the velocity and Euler update of k_final_velocity, then
// x = bf16(W_in a + b_in) for the next step (k_action_in's sums, in its
// order), and, when the next step's first modulation is known (scale1 not
// null), the packed input the first layer reads: bf16(x * (1 + scale1)) tiled
// at row prow and the 64 sums of squares of 16 columns of x, summed in column
// order as k_pack_rows does.  The in-projection's weights (4 rows of A per
// thread) are loaded at kernel start when they fit 16 registers of 16 bytes.
template <int A>
__global__ __launch_bounds__(256) void k_step_tail(const uint16_t* x, const float* fmod, const uint16_t* w_out,
                                                  const uint16_t* b_out, const uint16_t* w_in, const uint16_t* b_in,
                                                  float dt, float* a, float* traj, uint16_t* x_next, int T, int TP,
                                                  const float* scale1, int scale_stride, uint16_t* xp, float* ss) {
  constexpr bool PRE_IN = A <= 32;
  constexpr int NIN = PRE_IN ? A / 8 : 1;  // 16-byte groups of a W_in row held per output
  __shared__ __attribute__((aligned(16))) float sx[kH];
  __shared__ float rss[4], sa[A];
  const int row = blockIdx.x, c = threadIdx.x * 4;
  VelPre<A> p;
  velocity_prefetch<A>(x, w_out, row, p);
  uint4 win[4][NIN];
  if (PRE_IN) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < NIN; ++g) win[i][g] = *reinterpret_cast<const uint4*>(w_in + (size_t)(c + i) * A + g * 8);
  }
  row_velocity<A>(p, fmod, w_out, b_out, dt, a, traj, row, sx, rss, sa);
  __syncthreads();
  // step k + 1: the action in-projection (as k_action_in)
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = c + i;
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < A; j += 8) {
      const uint4 raw = PRE_IN ? win[i][j / 8] : *reinterpret_cast<const uint4*>(w_in + (size_t)n * A + j);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += bf2f((uint16_t)(w4[e] & 0xffffu)) * sa[j + 2 * e];
        acc += bf2f((uint16_t)(w4[e] >> 16)) * sa[j + 2 * e + 1];
      }
    }
    y[i] = acc + bf2f(b_in[n]);
  }
  const uint32_t p01 = pack2(y[0], y[1]), p23 = pack2(y[2], y[3]);
  *reinterpret_cast<uint2*>(x_next + (size_t)row * kH + c) = make_uint2(p01, p23);
  if (!scale1) return;
  {  // the packed input of the next step's first layer (as k_pack_rows, with
     // its rounding: no fused multiply-adds); sx is free again
#pragma clang fp contract(off)
    const int b = row / T, t = row - b * T, prow = b * TP + t;
    const float xb[4] = {bf2f((uint16_t)(p01 & 0xffffu)), bf2f((uint16_t)(p01 >> 16)),
                         bf2f((uint16_t)(p23 & 0xffffu)), bf2f((uint16_t)(p23 >> 16))};
    const float* sp = scale1 + (size_t)b * scale_stride + c;
    *reinterpret_cast<uint2*>(xp + tile_off(prow, c & ~7, kH) + (c & 7)) =
        make_uint2(pack2(xb[0] * (1.f + sp[0]), xb[1] * (1.f + sp[1])),
                   pack2(xb[2] * (1.f + sp[2]), xb[3] * (1.f + sp[3])));
#pragma unroll
    for (int i = 0; i < 4; ++i) sx[c + i] = xb[i] * xb[i];
    __syncthreads();
    if (threadIdx.x < kSsParts) {
      float acc = 0.f;
      for (int i = 0; i < 16; ++i) acc += sx[threadIdx.x * 16 + i];
      ss[(size_t)prow * kSsParts + threadIdx.x] = acc;
    }
  }
}

#define DMX_ACTION_DIMS(X) X(16) X(32) X(48) X(64) X(80) X(96) X(112) X(128)

hipError_t launch_time_embed(int n_steps, uint16_t* temb, hipStream_t s) {
  k_time_embed<<<dim3(n_steps), dim3(kH / 2), 0, s>>>(n_steps, temb);
  return hipGetLastError();
}

hipError_t launch_gemv_rows(const uint16_t* W, const uint16_t* bias, int N, bool swish, const uint16_t* x,
                            int x_stride, int R, float* out_f32, int ldo, uint16_t* out_bf16, int rep, hipStream_t s) {
  if (swish)
    k_gemv_rows<true><<<dim3(N / 16), dim3(256), 0, s>>>(W, bias, x, x_stride, R, out_f32, ldo, out_bf16, rep);
  else
    k_gemv_rows<false><<<dim3(N / 16), dim3(256), 0, s>>>(W, bias, x, x_stride, R, out_f32, ldo, out_bf16, rep);
  return hipGetLastError();
}

hipError_t launch_action_in(const float* a, const uint16_t* w_in, const uint16_t* b_in, int rows, int A, uint16_t* x,
                            hipStream_t s) {
  k_action_in<<<dim3(rows), dim3(256), 0, s>>>(a, w_in, b_in, A, x);
  return hipGetLastError();
}

hipError_t launch_final_velocity(const uint16_t* x, const float* fmod, const uint16_t* w_out, const uint16_t* b_out,
                                 int rows, int A, float dt, float* a, float* traj, hipStream_t s) {
  switch (A) {
#define DMX_CASE(N) \
  case N: k_final_velocity<N><<<dim3(rows), dim3(256), 0, s>>>(x, fmod, w_out, b_out, dt, a, traj); break;
    DMX_ACTION_DIMS(DMX_CASE)
#undef DMX_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_step_tail(const uint16_t* x, const float* fmod, const uint16_t* w_out, const uint16_t* b_out,
                            const uint16_t* w_in, const uint16_t* b_in, int rows, int A, float dt, float* a,
                            float* traj, uint16_t* x_next, int T, int TP, const float* scale1, int scale_stride,
                            uint16_t* xp, float* ss, hipStream_t s) {
  switch (A) {
#define DMX_CASE(N)                                                                                               \
  case N:                                                                                                         \
    k_step_tail<N><<<dim3(rows), dim3(256), 0, s>>>(x, fmod, w_out, b_out, w_in, b_in, dt, a, traj, x_next, T, TP, \
                                                    scale1, scale_stride, xp, ss);                                \
    break;
    DMX_ACTION_DIMS(DMX_CASE)
#undef DMX_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dmx
