// Weight-streaming skinny GEMMs for the action-expert projections on gfx950.
//
// y[m][n] = sum_k A[m][k] * W[n][k]: M = batch * chunk tokens (10..800) and the
// weight matrix W [N][K] bf16 is the big operand (4..17 MB), so the cost is
// streaming W from HBM once.  One work-group (WG) owns NT output features and
// the whole K range; its NWAVES waves split K.  Every wave issues all of its
// weight loads at kernel start, straight into registers in the MFMA B-operand
// layout (lane l: 16 contiguous bytes of feature row l%16), then runs the M
// rows of A past them in 64-row blocks on v_mfma_f32_16x16x32_bf16.  The
// waves' partial tiles are summed in LDS in a fixed order and the WG applies
// the epilogue.  No WG ever waits for another WG: every reduction stays
// inside the WG, so results are deterministic and need no device-scope
// fences.
//
// A operand sources:
//   A_GLOBAL   bf16 rows read from global memory (context, GEGLU hidden,
//              prefix-side normed inputs).
//   A_NORM_B / A_NORM_F  AdaRMS prenorm fused as a prologue (OpenDM DM0.5
//              fast-stack article, §2.2, "Adarms 调制 prenorm"): the WG reads
//              the bf16 / fp32 residual rows of its 64-row block, forms
//              xn = x / rms(x) * (1 + scale[b]) + shift[b] in fp32, rounds it
//              to bf16 into LDS, and feeds the MFMAs from LDS.
// Epilogues (the same article's chaining of time modulation with GEGLU
// gate-up and MLP down):
//   EPI_F32    raw fp32 store (QKV before QK-norm / RoPE)
//   EPI_MOD    + bias, fp32 store (AdaRMS modulation vectors)
//   EPI_RESID_* out = resid + gate[b] * y, bf16 / fp32 variants
//   EPI_GEGLU  tile = 16 gate + 16 up features; h = gelu_tanh(gate) * up
#include "dmx_device.hpp"
#include "dmx_internal.hpp"

namespace dmx {

namespace {
constexpr int XLD = kH + 8;  // LDS row stride (bf16) of the normed activation block
}

template <int EPI, int NT>
__device__ __forceinline__ int w_row(const GemmArgs& a, int tile, int r) {
  if (EPI == EPI_GEGLU) return r < 16 ? tile * 16 + r : a.wrow_up + tile * 16 + (r - 16);
  return tile * NT + r;
}

template <int EPI, int NT>
__device__ __forceinline__ void epi_store(const GemmArgs& a, int tile, int m, int c, float v) {
  const int n = tile * NT + c;
  const size_t idx = (size_t)m * a.ldo + n;
  if (EPI == EPI_F32) {
    a.out_f32[idx] = v;
  } else if (EPI == EPI_MOD) {
    a.out_f32[idx] = v + bf2f(a.bias[n]);
  } else {
    const float gv = a.gate[(size_t)(m / a.T) * a.gate_stride + n];
    if (EPI == EPI_RESID_BB) a.out_bf16[idx] = f2bf(bf2f(a.resid[idx]) + gv * v);
    if (EPI == EPI_RESID_BF) a.out_f32[idx] = bf2f(a.resid[idx]) + gv * v;
    if (EPI == EPI_RESID_FB) a.out_bf16[idx] = f2bf(a.resid_f32[idx] + gv * v);
  }
}

__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf2f((uint16_t)(w[i] & 0xffffu));
    v[2 * i + 1] = bf2f((uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// AdaRMS prologue: rows [m0, m0 + rows) of x (row length kH) -> bf16 xn in LDS.
// Each wave normalises rows wave, wave + NWAVES, ...; lane l owns the 16
// columns 8l..8l+7 and 512+8l..512+8l+7.
template <typename TX, int NWAVES>
__device__ __forceinline__ void adarms_to_lds(const TX* x, const float* mod, int T, int m0, int rows,
                                              uint16_t* sx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = wave; r < rows; r += NWAVES) {
    const int m = m0 + r, b = m / T;
    float v[16];
    load8(x + (size_t)m * kH + lane * 8, v);
    load8(x + (size_t)m * kH + 512 + lane * 8, v + 8);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += v[i] * v[i];
    ss = wave_sum(ss);
    const float rn = 1.0f / sqrtf(ss * (1.0f / kH) + kEps);
    const float* sc = mod + (size_t)b * 3 * kH;
    const float* sh = sc + kH;
    float s8[16], h8[16];
    load8(sc + lane * 8, s8);
    load8(sc + 512 + lane * 8, s8 + 8);
    load8(sh + lane * 8, h8);
    load8(sh + 512 + lane * 8, h8 + 8);
    uint4 o0, o1;
    o0.x = pack2(v[0] * rn * (1.f + s8[0]) + h8[0], v[1] * rn * (1.f + s8[1]) + h8[1]);
    o0.y = pack2(v[2] * rn * (1.f + s8[2]) + h8[2], v[3] * rn * (1.f + s8[3]) + h8[3]);
    o0.z = pack2(v[4] * rn * (1.f + s8[4]) + h8[4], v[5] * rn * (1.f + s8[5]) + h8[5]);
    o0.w = pack2(v[6] * rn * (1.f + s8[6]) + h8[6], v[7] * rn * (1.f + s8[7]) + h8[7]);
    o1.x = pack2(v[8] * rn * (1.f + s8[8]) + h8[8], v[9] * rn * (1.f + s8[9]) + h8[9]);
    o1.y = pack2(v[10] * rn * (1.f + s8[10]) + h8[10], v[11] * rn * (1.f + s8[11]) + h8[11]);
    o1.z = pack2(v[12] * rn * (1.f + s8[12]) + h8[12], v[13] * rn * (1.f + s8[13]) + h8[13]);
    o1.w = pack2(v[14] * rn * (1.f + s8[14]) + h8[14], v[15] * rn * (1.f + s8[15]) + h8[15]);
    *reinterpret_cast<uint4*>(sx + r * XLD + lane * 8) = o0;
    *reinterpret_cast<uint4*>(sx + r * XLD + 512 + lane * 8) = o1;
  }
}

template <int EPI, int NT, int NWAVES, int KSTEPS, int ASRC>
__global__ __launch_bounds__(NWAVES * 64) void k_gemm(GemmArgs a) {
  constexpr int NTT = NT / 16;
  constexpr int KW = KSTEPS * 32;  // reduction elements per wave
  constexpr bool NORM = ASRC != A_GLOBAL;
  // LDS: normed activation block (NORM only) and the cross-wave reduction
  // area, which reuses the same bytes once the MFMAs are done.
  constexpr int RED_BYTES = NWAVES * 64 * NT * 4;
  constexpr int XS_BYTES = NORM ? 64 * XLD * 2 : 0;
  constexpr int SMEM = XS_BYTES > RED_BYTES ? XS_BYTES : RED_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  float* red = reinterpret_cast<float*>(smem);
  uint16_t* sx = reinterpret_cast<uint16_t*>(smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int k0 = wave * KW;
  const int lr = lane & 15, lk = (lane >> 4) * 8;

  // weight slab of this wave: NT rows x KW columns, every load in flight now
  bf16x8 wf[KSTEPS][NTT];
#pragma unroll
  for (int nt = 0; nt < NTT; ++nt) {
    const uint16_t* wp = a.W + (size_t)w_row<EPI, NT>(a, tile, nt * 16 + lr) * a.K + k0 + lk;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) wf[ks][nt] = load_bf16x8(wp + ks * 32);
  }

  for (int m0 = 0; m0 < a.M; m0 += 64) {
    const int rows = min(64, a.M - m0);
    const int mts = (rows + 15) >> 4;
    if (NORM) {
      if (ASRC == A_NORM_B)
        adarms_to_lds<uint16_t, NWAVES>(a.xb, a.nmod, a.T, m0, rows, sx);
      else
        adarms_to_lds<float, NWAVES>(a.xf, a.nmod, a.T, m0, rows, sx);
      __syncthreads();
    }
    f32x4 acc[4][NTT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) acc[mt][nt] = zero_f32x4();
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      bf16x8 av[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r = mt * 16 + lr;
        if (NORM) {
          av[mt] = (mt < mts && r < rows) ? *reinterpret_cast<const bf16x8*>(sx + r * XLD + k0 + ks * 32 + lk)
                                          : zero_bf16x8();
        } else {
          av[mt] = (mt < mts && r < rows) ? load_bf16x8(a.A + (size_t)(m0 + r) * a.K + k0 + ks * 32 + lk)
                                          : zero_bf16x8();
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < mts) {
#pragma unroll
          for (int nt = 0; nt < NTT; ++nt) acc[mt][nt] = mfma16(av[mt], wf[ks][nt], acc[mt][nt]);
        }
      }
    }
    if (NORM) __syncthreads();  // everyone is done reading sx before it becomes `red`
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt < mts) {
#pragma unroll
        for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[(wave * 64 + mt * 16 + (lane >> 4) * 4 + r) * NT + nt * 16 + lr] = acc[mt][nt][r];
      }
    }
    __syncthreads();
    if (EPI == EPI_GEGLU) {
      for (int e = threadIdx.x; e < rows * 16; e += NWAVES * 64) {
        const int r = e >> 4, c = e & 15;
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
          g += red[(w * 64 + r) * NT + c];
          u += red[(w * 64 + r) * NT + 16 + c];
        }
        a.out_bf16[(size_t)(m0 + r) * a.ldo + tile * 16 + c] = f2bf(gelu_tanh(g) * u);
      }
    } else {
      for (int e = threadIdx.x; e < rows * NT; e += NWAVES * 64) {
        const int r = e / NT, c = e - (e / NT) * NT;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) v += red[(w * 64 + r) * NT + c];
        epi_store<EPI, NT>(a, tile, m0 + r, c, v);
      }
    }
    __syncthreads();
  }
}

#define DMX_GEMM(EPI, NT, NW, KS, SRC) \
  k_gemm<EPI, NT, NW, KS, SRC><<<dim3(a.ntiles), dim3((NW) * 64), 0, s>>>(a)

int gemm_config(GemmKind kind, GemmArgs& a) {
  switch (kind) {
    case GEMM_MOD: a.ntiles = 3 * kH / 16; a.K = kH; break;
    case GEMM_QKV1024: a.ntiles = kQKV / 16; a.K = kH; break;
    case GEMM_QKV1024_NORM: a.ntiles = kQKV / 16; a.K = kH; break;
    case GEMM_QKV2560: a.ntiles = kQKV / 16; a.K = 2560; break;
    case GEMM_OPROJ: a.ntiles = kH / 16; a.K = kHQ * kD; break;
    case GEMM_OPROJ_F32: a.ntiles = kH / 16; a.K = kHQ * kD; break;
    case GEMM_GATEUP: a.ntiles = kI / 16; a.K = kH; a.wrow_up = kI; break;
    case GEMM_GATEUP_NORM_F32: a.ntiles = kI / 16; a.K = kH; a.wrow_up = kI; break;
    case GEMM_DOWN: a.ntiles = kH / 16; a.K = kI; break;
    case GEMM_DOWN_F32RES: a.ntiles = kH / 16; a.K = kI; break;
  }
  return a.ntiles;
}

hipError_t launch_gemm(GemmKind kind, const GemmArgs& a, hipStream_t s) {
  switch (kind) {
    case GEMM_MOD: DMX_GEMM(EPI_MOD, 16, 4, 8, A_GLOBAL); break;
    case GEMM_QKV1024: DMX_GEMM(EPI_F32, 16, 4, 8, A_GLOBAL); break;
    case GEMM_QKV1024_NORM: DMX_GEMM(EPI_F32, 16, 4, 8, A_NORM_B); break;
    case GEMM_QKV2560: DMX_GEMM(EPI_F32, 16, 4, 20, A_GLOBAL); break;
    case GEMM_OPROJ: DMX_GEMM(EPI_RESID_BB, 16, 8, 8, A_GLOBAL); break;
    case GEMM_OPROJ_F32: DMX_GEMM(EPI_RESID_BF, 16, 8, 8, A_GLOBAL); break;
    case GEMM_GATEUP: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_GLOBAL); break;
    case GEMM_GATEUP_NORM_F32: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_NORM_F); break;
    case GEMM_DOWN: DMX_GEMM(EPI_RESID_BB, 16, 8, 16, A_GLOBAL); break;
    case GEMM_DOWN_F32RES: DMX_GEMM(EPI_RESID_FB, 16, 8, 16, A_GLOBAL); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Modulation vectors of several (W_mod, b_mod) pairs in one launch:
// out_j[b] = W_j * cond[b] + b_j.  Work-group (j, tile) owns 16 features of
// matrix j; all loads of its 32 KB weight slab are issued up front.
__global__ __launch_bounds__(256) void k_mod_multi(ModBatch mb) {
  const int j = blockIdx.x / (3 * kH / 16), tile = blockIdx.x - j * (3 * kH / 16);
  const ModJob& job = mb.job[j];
  __shared__ float red[4][16 * 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int k0 = wave * 256;
  bf16x8 wf[8];
  const uint16_t* wp = job.w + (size_t)(tile * 16 + lr) * kH + k0 + lk;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) wf[ks] = load_bf16x8(wp + ks * 32);
  const uint16_t* cond = job.cond;
  for (int b0 = 0; b0 < mb.B; b0 += 16) {
    const int rows = min(16, mb.B - b0);
    f32x4 acc = zero_f32x4();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 av = lr < rows ? load_bf16x8(cond + (size_t)(b0 + lr) * kH + k0 + ks * 32 + lk) : zero_bf16x8();
      acc = mfma16(av, wf[ks], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][((lane >> 4) * 4 + r) * 16 + lr] = acc[r];
    __syncthreads();
    if (threadIdx.x < rows * 16) {
      const int r = threadIdx.x >> 4, c = threadIdx.x & 15;
      const float v = red[0][r * 16 + c] + red[1][r * 16 + c] + red[2][r * 16 + c] + red[3][r * 16 + c];
      const int n = tile * 16 + c;
      job.out[(size_t)(b0 + r) * 3 * kH + n] = v + bf2f(job.bias[n]);
    }
    __syncthreads();
  }
}

hipError_t launch_mod_multi(const ModBatch& mb, hipStream_t s) {
  if (mb.n == 0) return hipSuccess;
  k_mod_multi<<<dim3(mb.n * (3 * kH / 16)), dim3(256), 0, s>>>(mb);
  return hipGetLastError();
}

}  // namespace dmx
