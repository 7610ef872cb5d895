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
//   A_MOD /    AdaRMS prenorm fused into the projection (OpenDM DM0.5
//              fast-stack article, §2.2, "Adarms 调制 prenorm"):
//                xn W^T = r * ((x * (1 + scale)) W^T) + shift W^T,
//              r = 1 / sqrt(mean x^2 + eps) per row.  The A operand is the raw
//              bf16 residual row scaled by (1 + scale) (one bf16 rounding, as
//              rounding xn would be); shift W^T is one extra MFMA tile whose
//              row 0 is the shift vector; r comes from per-tile row sums of
//              squares that the GEMM producing x wrote in its epilogue (or
//              from a row-statistics kernel), summed in a fixed order.
//   A_MODPRE   as A_MOD with the A rows already bf16(x * (1 + scale)): the
//              O-projection epilogue writes them from fp32 x1, so x1 is
//              rounded once on its way into the gate-up projection.
// Epilogues (the same article's chaining of time modulation with GEGLU
// gate-up and MLP down):
//   EPI_F32    raw fp32 store (QKV before QK-norm / RoPE)
//   EPI_MOD    + bias, fp32 store (AdaRMS modulation vectors)
//   EPI_RESID_* out = resid + gate[b] * y, bf16 / fp32 variants
//   EPI_GEGLU  tile = 16 gate + 16 up features; h = gelu_tanh(gate) * up
#include "dmx_device.hpp"
#include "dmx_internal.hpp"

#include <algorithm>

namespace dmx {

namespace {
constexpr int XLD = kH + 8;  // LDS row stride (bf16) of the normed activation block
}

template <int EPI, int NT>
__device__ __forceinline__ int w_row(const GemmArgs& a, int tile, int r) {
  if (EPI == EPI_GEGLU) return r < 16 ? tile * 16 + r : a.wrow_up + tile * 16 + (r - 16);
  return tile * NT + r;
}

// Stores one output element; returns the value the next AdaRMS normalises
// (the stored bf16 value, or the fp32 residual x1) for the row statistics.
template <int EPI, int NT>
__device__ __forceinline__ float epi_store(const GemmArgs& a, int tile, int m, int c, float v) {
  const int n = tile * NT + c;
  const size_t idx = (size_t)m * a.ldo + n;
  if (EPI == EPI_F32) {
    a.out_f32[idx] = v;
  } else if (EPI == EPI_MOD) {
    a.out_f32[idx] = v + bf2f(a.bias[n]);
  } else {
    const size_t b = (size_t)(m / a.T) * a.gate_stride;
    const float gv = a.gate[b + n];
    if (EPI == EPI_RESID_BB) a.out_bf16[idx] = f2bf(bf2f(a.resid[idx]) + gv * v);
    if (EPI == EPI_RESID_BF) {
      const float x1 = bf2f(a.resid[idx]) + gv * v;
      a.out_f32[idx] = x1;
      if (a.out_bf16) a.out_bf16[idx] = f2bf(a.xs_scale ? x1 * (1.0f + a.xs_scale[b + n]) : x1);
      return x1;
    }
    if (EPI == EPI_RESID_FB) {
      const uint16_t hb = f2bf(a.resid_f32[idx] + gv * v);
      a.out_bf16[idx] = hb;
      return bf2f(hb);
    }
  }
  return 0.f;
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

// Row sums of squares of this WG's outputs as the next AdaRMS sees them: LDS
// holds the squares of the block's outputs in `sq`; the sum runs over the
// tile's columns in order (k_row_ssq reproduces it).
template <int NT>
__device__ __forceinline__ void write_row_ssq(const GemmArgs& a, int tile, int m0, int rows, const float* sq) {
  for (int r = threadIdx.x; r < rows; r += blockDim.x) {
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < NT; ++c) t += sq[r * NT + c];
    a.ss_out[(size_t)(m0 + r) * a.ss_out_n + tile] = t;
  }
}

template <int EPI, int NT, int NWAVES, int KSTEPS, int ASRC, int MT>
__global__ __launch_bounds__(NWAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_gemm(GemmArgs a) {
  constexpr int NTT = NT / 16;
  constexpr int KW = KSTEPS * 32;  // reduction elements per wave
  constexpr bool MOD = ASRC != A_GLOBAL;   // AdaRMS fused: shift tile + row scale
  constexpr bool SCALE = ASRC == A_MOD;    // ... and the (1 + scale) product on A
  constexpr int MB = MT * 16;      // rows per block
  constexpr int RROWS = MB + (MOD ? 16 : 0);  // + the shift tile
  static_assert(!MOD || NWAVES * KW == kH, "the modulated A operand spans one hidden row");
  __shared__ float red[NWAVES * RROWS * NT];
  __shared__ float sq[MB * NT];
  __shared__ float sS[SCALE ? kH : 4], sH[MOD ? kH : 1], sR[MOD ? MB : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int k0 = wave * KW;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  constexpr bool SSQ = EPI == EPI_RESID_BF || EPI == EPI_RESID_FB;

  // weight slab of this wave: NT rows x KW columns, every load in flight now
  bf16x8 wf[KSTEPS][NTT];
#pragma unroll
  for (int nt = 0; nt < NTT; ++nt) {
    const uint16_t* wp = a.W + (size_t)w_row<EPI, NT>(a, tile, nt * 16 + lr) * a.K + k0 + lk;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) wf[ks][nt] = load_bf16x8(wp + ks * 32);
  }
  __builtin_amdgcn_sched_barrier(0);

  // row blocks: MOD kernels take one request's rows per block (T <= MB);
  // others take MB consecutive rows, blockIdx.y, blockIdx.y + gridDim.y, ...
  const int bstride = MOD ? a.T : MB;
  for (int m0 = blockIdx.y * bstride; m0 < a.M; m0 += gridDim.y * bstride) {
    const int rows = min(MOD ? a.T : MB, a.M - m0);
    const int mts = (rows + 15) >> 4;
    f32x4 acc[MT][NTT], accs[NTT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) acc[mt][nt] = zero_f32x4();
#pragma unroll
    for (int nt = 0; nt < NTT; ++nt) accs[nt] = zero_f32x4();

    // ---- all A fragments of the block (and the modulation inputs) at once
    bf16x8 av[KSTEPS][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = min(m0 + mt * 16 + lr, m0 + rows - 1);  // rows past the block feed unused outputs
      const uint16_t* ap = (MOD ? a.xb : a.A) + (size_t)r * a.K + k0 + lk;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) av[ks][mt] = load_bf16x8(ap + ks * 32);
    }
    float4 msc = make_float4(0.f, 0.f, 0.f, 0.f), msh = msc;
    float4 ssp[4];
    if (MOD) {
      const float* mb = a.nmod + (size_t)(m0 / a.T) * 3 * kH;
      if (SCALE) msc = *reinterpret_cast<const float4*>(mb + threadIdx.x * 4);  // 256 threads x 4 = 1024
      msh = *reinterpret_cast<const float4*>(mb + kH + threadIdx.x * 4);
      // row statistics: thread (row rr, quarter qq) sums a quarter of the row's partials
      const int rr = threadIdx.x >> 2, qq = threadIdx.x & 3;
      const int per = a.ss_in_n >> 2;  // ss_in_n is a multiple of 4, at most 64
#pragma unroll
      for (int i = 0; i < 4; ++i) ssp[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (rr < rows) {
        const float* sp = a.ss_in + (size_t)(m0 + rr) * a.ss_in_n + qq * per;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i * 4 < per) ssp[i] = *reinterpret_cast<const float4*>(sp + i * 4);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the whole block is in flight before any use

    if (MOD) {
      if (SCALE)
        reinterpret_cast<float4*>(sS)[threadIdx.x] =
            make_float4(1.f + msc.x, 1.f + msc.y, 1.f + msc.z, 1.f + msc.w);
      reinterpret_cast<float4*>(sH)[threadIdx.x] = msh;
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) t += ssp[i].x + ssp[i].y + ssp[i].z + ssp[i].w;
      t += __shfl_xor(t, 1, 64);
      t += __shfl_xor(t, 2, 64);
      const int rr = threadIdx.x >> 2;
      if ((threadIdx.x & 3) == 0 && rr < MB) sR[rr] = 1.0f / sqrtf(t * (1.0f / kH) + kEps);
      __syncthreads();
      // A <- bf16(x * (1 + scale)) (A_MOD); the shift tile's row 0 <- bf16(shift)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const float4 s0 = *reinterpret_cast<const float4*>(sS + (SCALE ? k0 + ks * 32 + lk : 0));
        const float4 s1 = *reinterpret_cast<const float4*>(sS + (SCALE ? k0 + ks * 32 + lk + 4 : 0));
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (!SCALE) break;
          bf16x8 t8;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const uint32_t p = pack2(bf2f((uint16_t)av[ks][mt][e]) * sv[e], bf2f((uint16_t)av[ks][mt][e + 1]) * sv[e + 1]);
            t8[e] = (short)(p & 0xffffu);
            t8[e + 1] = (short)(p >> 16);
          }
          av[ks][mt] = t8;
        }
        bf16x8 hs = zero_bf16x8();
        if (lr == 0) {
          const float4 h0 = *reinterpret_cast<const float4*>(sH + k0 + ks * 32 + lk);
          const float4 h1 = *reinterpret_cast<const float4*>(sH + k0 + ks * 32 + lk + 4);
          const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const uint32_t p = pack2(hv[e], hv[e + 1]);
            hs[e] = (short)(p & 0xffffu);
            hs[e + 1] = (short)(p >> 16);
          }
        }
#pragma unroll
        for (int nt = 0; nt < NTT; ++nt) accs[nt] = mfma16(hs, wf[ks][nt], accs[nt]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < mts) {
#pragma unroll
          for (int nt = 0; nt < NTT; ++nt) acc[mt][nt] = mfma16(av[ks][mt], wf[ks][nt], acc[mt][nt]);
        }

    // ---- cross-wave reduction (fixed order) and epilogue
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mts) {
#pragma unroll
        for (int nt = 0; nt < NTT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[(wave * RROWS + mt * 16 + (lane >> 4) * 4 + r) * NT + nt * 16 + lr] = acc[mt][nt][r];
      }
    }
    if (MOD && lane < 16) {  // row 0 of the shift tile
#pragma unroll
      for (int nt = 0; nt < NTT; ++nt) red[(wave * RROWS + MB) * NT + nt * 16 + lr] = accs[nt][0];
    }
    __syncthreads();
    if (EPI == EPI_GEGLU) {
      for (int e = threadIdx.x; e < rows * 16; e += NWAVES * 64) {
        const int r = e >> 4, c = e & 15;
        float g = 0.f, u = 0.f, gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
          g += red[(w * RROWS + r) * NT + c];
          u += red[(w * RROWS + r) * NT + 16 + c];
          if (MOD) {
            gs += red[(w * RROWS + MB) * NT + c];
            us += red[(w * RROWS + MB) * NT + 16 + c];
          }
        }
        if (MOD) {
          g = sR[r] * g + gs;
          u = sR[r] * u + us;
        }
        a.out_bf16[(size_t)(m0 + r) * a.ldo + tile * 16 + c] = f2bf(gelu_tanh(g) * u);
      }
    } else {
      for (int e = threadIdx.x; e < rows * NT; e += NWAVES * 64) {
        const int r = e / NT, c = e - (e / NT) * NT;
        float v = 0.f, vs = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
          v += red[(w * RROWS + r) * NT + c];
          if (MOD) vs += red[(w * RROWS + MB) * NT + c];
        }
        if (MOD) v = sR[r] * v + vs;
        const float seen = epi_store<EPI, NT>(a, tile, m0 + r, c, v);
        if (SSQ) sq[r * NT + c] = seen * seen;
      }
      if (SSQ && a.ss_out) {
        __syncthreads();
        write_row_ssq<NT>(a, tile, m0, rows, sq);
      }
    }
    __syncthreads();
  }
}

#define DMX_GEMM(EPI, NT, NW, KS, SRC, MT, MSPLIT) \
  k_gemm<EPI, NT, NW, KS, SRC, MT><<<dim3(a.ntiles, MSPLIT), dim3((NW) * 64), 0, s>>>(a)

int gemm_config(GemmKind kind, GemmArgs& a) {
  switch (kind) {
    case GEMM_MOD: a.ntiles = 3 * kH / 16; a.K = kH; break;
    case GEMM_QKV1024: a.ntiles = kQKV / 16; a.K = kH; break;
    case GEMM_QKV1024_MOD: a.ntiles = kQKV / 16; a.K = kH; break;
    case GEMM_QKV2560: a.ntiles = kQKV / 16; a.K = 2560; break;
    case GEMM_OPROJ: a.ntiles = kH / 16; a.K = kHQ * kD; break;
    case GEMM_OPROJ_F32: a.ntiles = kH / 16; a.K = kHQ * kD; break;
    case GEMM_GATEUP: a.ntiles = kI / 16; a.K = kH; a.wrow_up = kI; break;
    case GEMM_GATEUP_MOD: a.ntiles = kI / 16; a.K = kH; a.wrow_up = kI; break;
    case GEMM_DOWN: a.ntiles = kH / 16; a.K = kI; break;
    case GEMM_DOWN_F32RES: a.ntiles = kH / 16; a.K = kI; break;
  }
  return a.ntiles;
}

hipError_t launch_gemm(GemmKind kind, const GemmArgs& a, hipStream_t s) {
  // row blocks: one per WG up to 4 (more rows loop inside the WG)
  const int mb16 = std::min(4, (a.M + 15) / 16), mb32 = std::min(4, (a.M + 31) / 32);
  const int nreq = std::min(4, a.T > 0 ? (a.M + a.T - 1) / a.T : 1);  // MOD: one request per block
  switch (kind) {
    case GEMM_MOD: DMX_GEMM(EPI_MOD, 16, 4, 8, A_GLOBAL, 1, mb16); break;
    case GEMM_QKV1024: DMX_GEMM(EPI_F32, 16, 4, 8, A_GLOBAL, 2, mb32); break;
    case GEMM_QKV1024_MOD: DMX_GEMM(EPI_F32, 16, 4, 8, A_MOD, 4, nreq); break;
    case GEMM_QKV2560: DMX_GEMM(EPI_F32, 16, 4, 20, A_GLOBAL, 1, 4); break;
    case GEMM_OPROJ: DMX_GEMM(EPI_RESID_BB, 16, 8, 8, A_GLOBAL, 1, mb16); break;
    case GEMM_OPROJ_F32: DMX_GEMM(EPI_RESID_BF, 16, 8, 8, A_GLOBAL, 1, mb16); break;
    case GEMM_GATEUP: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_GLOBAL, 2, mb32); break;
    case GEMM_GATEUP_MOD: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_MODPRE, 4, nreq); break;
    case GEMM_DOWN: DMX_GEMM(EPI_RESID_BB, 16, 8, 16, A_GLOBAL, 1, mb16); break;
    case GEMM_DOWN_F32RES: DMX_GEMM(EPI_RESID_FB, 16, 8, 16, A_GLOBAL, 1, mb16); break;
  }
  return hipGetLastError();
}

// Row sums of squares of bf16 rows x [M][1024] -> ss[M][64]: lane p of the
// row's wave sums the squares of columns 16p .. 16p+15 in column order, with
// every square rounded before the add, exactly as write_row_ssq does.
__global__ __launch_bounds__(256) void k_row_ssq(const uint16_t* x, int M, float* ss) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const uint4 r0 = *reinterpret_cast<const uint4*>(x + (size_t)m * kH + lane * 16);
  const uint4 r1 = *reinterpret_cast<const uint4*>(x + (size_t)m * kH + lane * 16 + 8);
  const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float lo = bf2f((uint16_t)(w[i] & 0xffffu)), hi = bf2f((uint16_t)(w[i] >> 16));
    const float l2 = lo * lo, h2 = hi * hi;
    t += l2;
    t += h2;
  }
  ss[(size_t)m * kSsParts + lane] = t;
}

hipError_t launch_row_ssq(const uint16_t* x, int M, float* ss, hipStream_t s) {
  k_row_ssq<<<dim3((M + 3) / 4), dim3(256), 0, s>>>(x, M, ss);
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
