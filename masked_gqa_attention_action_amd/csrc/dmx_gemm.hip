// Weight-streaming skinny GEMMs for the action-expert projections on gfx950.
//
// y[m][n] = sum_k A[m][k] * W[n][k]: M = batch * chunk tokens (10..800) and the
// weight matrix W [N][K] bf16 is the big operand (4..17 MB), so the cost is
// streaming W from HBM once.  One work-group (WG) owns NT output features and
// the whole K range; its NWAVES waves split K.  Every wave issues all of its
// weight loads at kernel start, straight into registers in the MFMA B-operand
// layout, then runs the rows of A past them in blocks of MT 16-row tiles on
// v_mfma_f32_16x16x32_bf16.  The waves' partial tiles are summed in LDS in a
// fixed order and the WG applies the epilogue.  No WG ever waits for another
// WG: every reduction stays inside the WG, so results are deterministic and
// need no device-scope fences.
//
// Both operands are stored tiled (dmx_tiles.hpp): one 16-row x 32-column tile
// is 1 KB laid out as the 64 lanes' MFMA fragments, so every load instruction
// of a wave reads 1 KB of contiguous memory.  Weights are tiled once by the
// caller; activations are written tiled by the kernel that produces them, with
// each request's rows padded to a multiple of 16 (padding rows hold anything
// and their outputs are never stored).
//
// A operand sources:
//   A_GLOBAL   tiled bf16 rows (context, GEGLU hidden, normed inputs).
//   A_MODPRE   AdaRMS prenorm fused into the projection (OpenDM DM0.5
//              fast-stack article, §2.2, "Adarms 调制 prenorm"):
//                xn W^T = r * ((x * (1 + scale)) W^T) + shift W^T,
//              r = 1 / sqrt(mean x^2 + eps) per row.  The A rows arrive as
//              bf16(x * (1 + scale)) (one bf16 rounding, as rounding xn would
//              be), written by the kernel that produces x (the input pack, the
//              O-projection epilogue from fp32 x1, the down epilogue for the
//              next layer); shift W^T is one extra MFMA tile whose row 0 is
//              the shift vector; r comes from per-tile row sums of squares of
//              x that the same producer wrote, summed in a fixed order.
// Epilogues (the same article's chaining of time modulation with GEGLU
// gate-up and MLP down); every store moves 8 consecutive features:
//   EPI_F32    raw fp32 store (QKV before QK-norm / RoPE)
//   EPI_QKV    QK-norm weights and RoPE on rotation-pair tiles (the article's
//              "QKV projection, QK-Norm and RoPE in one go"): tile u holds the
//              16 features j .. j+15 of head u/8's first half and their
//              partners j+128 ..; the epilogue stores rope((1 + w) * x) for q
//              and k heads as tiled fp32 with the tile's row sums of squares
//              of x, and x of the v heads as tiled bf16.  RoPE is linear, so the per-row RMS factor
//              is applied by the consumer: q = rope(x * r * (1 + w)) = r * y.
//   EPI_RESID_* out = resid + gate[b] * y, bf16 / fp32 variants
//   EPI_GEGLU  tile = 16 gate + 16 up features; h = gelu_tanh(gate) * up
#include "dmx_device.hpp"
#include "dmx_internal.hpp"
#include "dmx_mod.hpp"
#include "dmx_tiles.hpp"

#include <algorithm>

namespace dmx {

// Row sums of squares of this WG's outputs as the next AdaRMS sees them: LDS
// holds the squares of the block's outputs in `sq`; the sum runs over the
// tile's columns in order (k_pack_rows reproduces it).
template <int NT>
__device__ __forceinline__ void write_row_ssq(const GemmArgs& a, int tile, int m0, int nrows, const float* sq) {
  for (int r = threadIdx.x; r < nrows; r += blockDim.x) {
    if (!row_valid(m0 + r, a.T, a.TP)) continue;
    float t = 0.f;
#pragma unroll
    for (int c = 0; c < NT; ++c) t += sq[r * NT + c];
    a.ss_out[(size_t)(m0 + r) * a.ss_out_n + tile] = t;
  }
}

__device__ __forceinline__ void st8f(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ uint4 pack8(const float v[8]) {
  return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
}

// Global operands of one epilogue task (8 features n .. n+7 of tiled row
// prow), fetched while the MFMA operands are still in flight.
struct EpiPre {
  float4 g[2], sc[2], rf[2];  // gate, scale (x1 copy), fp32 residual
  uint4 rb;                   // bf16 residual
  uint4 wl, wh;               // QKV: norm weights of the pair's two halves
};

template <int EPI>
__device__ __forceinline__ void epi_fetch(const GemmArgs& a, int prow, int n, EpiPre& p) {
  const int b = prow / a.TP, t = prow - b * a.TP;
  const size_t lrow = (size_t)b * a.T + t;  // row of a row-major [batch][tokens] tensor
  if (EPI == EPI_RESID_BB || EPI == EPI_RESID_BF || EPI == EPI_RESID_FB) {
    const float* gp = a.gate + (size_t)b * a.gate_stride + n;
    p.g[0] = *reinterpret_cast<const float4*>(gp);
    p.g[1] = *reinterpret_cast<const float4*>(gp + 4);
  }
  if (EPI == EPI_RESID_BB || EPI == EPI_RESID_BF) p.rb = *reinterpret_cast<const uint4*>(a.resid + lrow * a.ldo + n);
  if ((EPI == EPI_RESID_BF || EPI == EPI_RESID_FB) && a.xs_scale) {
    const float* sp = a.xs_scale + (size_t)b * a.gate_stride + n;
    p.sc[0] = *reinterpret_cast<const float4*>(sp);
    p.sc[1] = *reinterpret_cast<const float4*>(sp + 4);
  }
  if (EPI == EPI_RESID_FB) {
    const float* rp = a.resid_f32 + (size_t)prow * a.ldo + n;
    p.rf[0] = *reinterpret_cast<const float4*>(rp);
    p.rf[1] = *reinterpret_cast<const float4*>(rp + 4);
  }
  if (EPI == EPI_QKV) {  // n = dim of the first half within the head, head = the tile's
    const int h = n >> 8;
    if (h < kHQ + kHK) {
      const uint16_t* wn = h < kHQ ? a.qn_w : a.kn_w;
      p.wl = *reinterpret_cast<const uint4*>(wn + (n & 127));
      p.wh = *reinterpret_cast<const uint4*>(wn + 128 + (n & 127));
    }
  }
}

__device__ __forceinline__ void unpack8(uint4 r, float v[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf2f((uint16_t)(w[i] & 0xffffu));
    v[2 * i + 1] = bf2f((uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ void f4x2(const float4 q[2], float v[8]) {
  v[0] = q[0].x; v[1] = q[0].y; v[2] = q[0].z; v[3] = q[0].w;
  v[4] = q[1].x; v[5] = q[1].y; v[6] = q[1].z; v[7] = q[1].w;
}

// Epilogue of 8 consecutive output features n .. n+7 of tiled row prow.
// Returns in `seen` the values the next AdaRMS normalises (for row sums).
template <int EPI>
__device__ __forceinline__ void epi_store8(const GemmArgs& a, int prow, int n, const EpiPre& p, float v[8],
                                           float seen[8]) {
  const int b = prow / a.TP, t = prow - b * a.TP;
  const size_t lrow = (size_t)b * a.T + t;
  if (EPI == EPI_F32) {
    st8f(a.out_f32 + (size_t)prow * a.ldo + n, v);
    return;
  }
  float g[8];
  f4x2(p.g, g);
  if (EPI == EPI_RESID_BB) {
    float r[8];
    unpack8(p.rb, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = r[i] + g[i] * v[i];
    *reinterpret_cast<uint4*>(a.out_bf16 + lrow * a.ldo + n) = pack8(v);
  } else if (EPI == EPI_RESID_BF) {
    float r[8];
    unpack8(p.rb, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = r[i] + g[i] * v[i];
      seen[i] = v[i];
    }
    st8f(a.out_f32 + (size_t)prow * a.ldo + n, v);
    if (a.xs_scale) {
      float sc[8];
      f4x2(p.sc, sc);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] * (1.0f + sc[i]);
    }
    *reinterpret_cast<uint4*>(a.out_pk + tile_off(prow, n, a.ldo)) = pack8(v);
  } else if (EPI == EPI_RESID_FB) {
    float r[8];
    f4x2(p.rf, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = r[i] + g[i] * v[i];
    const uint4 hb = pack8(v);
    *reinterpret_cast<uint4*>(a.out_bf16 + lrow * a.ldo + n) = hb;
    unpack8(hb, seen);
    if (a.out_pk) {  // the next layer's A operand: bf16(x) itself or bf16(bf16(x) * (1 + scale))
      uint4 pk = hb;
      if (a.xs_scale) {
        float sc[8], xs[8];
        f4x2(p.sc, sc);
#pragma unroll
        for (int i = 0; i < 8; ++i) xs[i] = seen[i] * (1.0f + sc[i]);
        pk = pack8(xs);
      }
      *reinterpret_cast<uint4*>(a.out_pk + tile_off(prow, n, a.ldo)) = pk;
    }
  }
}

// Epilogue constants of an output tile: NOUT output features (pairs for QKV)
// per row, OUTW of them per task, TPR tasks per row.
template <int EPI, int NT>
struct EpiShape {
  static constexpr int NOUT = (EPI == EPI_GEGLU || EPI == EPI_QKV) ? 16 : NT;
  static constexpr int OUTW = EPI == EPI_GEGLU ? 4 : 8;
  static constexpr int TPR = NOUT / OUTW;
};

// First output feature of task column c0 of output tile `tile` (the
// operand fetch and the stores address it).
template <int EPI, int NT>
__device__ __forceinline__ int epi_feature(int tile, int c0) {
  return EPI == EPI_QKV ? (tile >> 3) * kD + (tile & 7) * 16 + c0 : tile * NT + c0;
}

// One epilogue task: block row r, OUTW features of output tile `tile` from
// tile column c0.  Rsum(r, c) is the projection sum of block row r and tile
// column c, Ssum(r, c) the shift tile's sum for row r's request (MOD), both
// with their partial sums added in one fixed order; sR[r] is the row's 1 /
// rms (MOD), sF the tile's 16 rotation frequencies (QKV); sq / sQ are the
// tile's LDS scratch; cur holds the task's global operands (epi_fetch).
template <int EPI, int NT, bool MOD, class RF, class SF>
__device__ __forceinline__ void epi_task(const GemmArgs& a, int tile, int m0, int r, int c0, RF Rsum, SF Ssum,
                                         const float* sR, const double* sF, float* sq, float* sQ,
                                         const EpiPre& cur) {
  constexpr bool SSQ = EPI == EPI_RESID_BF || EPI == EPI_RESID_FB;
  constexpr bool QKV = EPI == EPI_QKV;
  constexpr int NOUT = EpiShape<EPI, NT>::NOUT;
  const int n = epi_feature<EPI, NT>(tile, c0);
  float v[8], seen[8];
  if (QKV) {
    // 8 rotation pairs: first-half features f .. f+7 and partners f+128 ..
    const int h = tile >> 3;  // head
    const int f = n;
    float lo[8], hi[8], sq8 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float tl = Rsum(r, c0 + i), th = Rsum(r, 16 + c0 + i);
      if (MOD) {
        const float sl = Ssum(r, c0 + i), sh = Ssum(r, 16 + c0 + i);
        lo[i] = sR[r] * tl + sl;
        hi[i] = sR[r] * th + sh;
      } else {
        lo[i] = tl;
        hi[i] = th;
      }
      sq8 += lo[i] * lo[i] + hi[i] * hi[i];
    }
    if (h < kHQ + kHK) {
      float wl[8], wh[8];
      unpack8(cur.wl, wl);
      unpack8(cur.wh, wh);
      const int prow = m0 + r, b = prow / a.TP;
      const double pos = (double)a.pos0[b] + (double)(prow - b * a.TP);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        double rev = pos * sF[c0 + i];
        rev -= floor(rev);
        const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
        const float x0 = lo[i] * (1.f + wl[i]), x1 = hi[i] * (1.f + wh[i]);
        lo[i] = x0 * cs - x1 * sn;
        hi[i] = x1 * cs + x0 * sn;
      }
    }
    if (h >= kHQ && h < kHQ + kHK) {  // k heads: fp32, scaled by 1 / rms when staged
      float* yo = a.out_f32 + tile_off_f32(m0 + r, f, kQKV);
      float* yh = a.out_f32 + tile_off_f32(m0 + r, f + 128, kQKV);
      *reinterpret_cast<float4*>(yo) = make_float4(lo[0], lo[1], lo[2], lo[3]);
      *reinterpret_cast<float4*>(yo + 256) = make_float4(lo[4], lo[5], lo[6], lo[7]);
      *reinterpret_cast<float4*>(yh) = make_float4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<float4*>(yh + 256) = make_float4(hi[4], hi[5], hi[6], hi[7]);
    } else {  // q and v heads: bf16, as the attention's MFMA consumes them
      const int fq = h < kHQ ? f : f - kHK * kD;
      *reinterpret_cast<uint4*>(a.out_pk + tile_off(m0 + r, fq, kQVB)) = pack8(lo);
      *reinterpret_cast<uint4*>(a.out_pk + tile_off(m0 + r, fq + 128, kQVB)) = pack8(hi);
    }
    sQ[r * 2 + (c0 >> 3)] = sq8;
  } else if (EPI == EPI_GEGLU) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float g = Rsum(r, c0 + i), u = Rsum(r, 16 + c0 + i);
      if (MOD) {
        const float gs = Ssum(r, c0 + i), us = Ssum(r, 16 + c0 + i);
        g = sR[r] * g + gs;
        u = sR[r] * u + us;
      }
      v[i] = gelu_tanh(g) * u;
    }
    *reinterpret_cast<uint2*>(a.out_pk + tile_off(m0 + r, tile * 16 + (c0 & ~7), a.ldo) + (c0 & 7)) =
        make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = Rsum(r, c0 + i);
      v[i] = MOD ? sR[r] * t + Ssum(r, c0 + i) : t;
    }
    epi_store8<EPI>(a, m0 + r, n, cur, v, seen);
    if (SSQ) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sq[r * NOUT + c0 + i] = seen[i] * seen[i];
    }
  }
}

// Epilogue of one output tile (NT columns `tile`) over block rows m0 ..
// m0 + nrows - 1, run by every thread of the work-group (it synchronises).
// Rsum, Ssum, sR, sF, sq and sQ as for epi_task (sq / sQ for nrows rows).
// pre0: the global operands of the thread's first task, if fetched.
template <int EPI, int NT, bool MOD, class RF, class SF>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& a, int tile, int m0, int nrows, RF Rsum, SF Ssum,
                                              const float* sR, const double* sF, float* sq, float* sQ,
                                              const EpiPre* pre0) {
  constexpr bool SSQ = EPI == EPI_RESID_BF || EPI == EPI_RESID_FB;
  constexpr bool QKV = EPI == EPI_QKV;
  constexpr int NOUT = EpiShape<EPI, NT>::NOUT, OUTW = EpiShape<EPI, NT>::OUTW, TPR = EpiShape<EPI, NT>::TPR;
  // task e: row r = e / TPR, OUTW features from c0; the thread's first task
  // is peeled so that the prefetched operands are used without a copy
  auto task = [&](int e, const EpiPre& cur) {
    const int r = e / TPR, c0 = (e - r * TPR) * OUTW;
    epi_task<EPI, NT, MOD>(a, tile, m0, r, c0, Rsum, Ssum, sR, sF, sq, sQ, cur);
  };
  auto task_row_ok = [&](int e) { return row_valid(m0 + e / TPR, a.T, a.TP); };
  int e0 = threadIdx.x;
  if (pre0) {
    if (e0 < nrows * TPR && task_row_ok(e0)) task(e0, *pre0);
    e0 += blockDim.x;
  }
  for (int e = e0; e < nrows * TPR; e += blockDim.x) {
    if (!task_row_ok(e)) continue;
    const int r = e / TPR, c0 = (e - r * TPR) * OUTW;
    EpiPre cur;
    epi_fetch<EPI>(a, m0 + r, epi_feature<EPI, NT>(tile, c0), cur);
    task(e, cur);
  }
  if (SSQ && a.ss_out) {
    __syncthreads();
    write_row_ssq<NOUT>(a, tile, m0, nrows, sq);
  }
  if (QKV && (tile >> 3) < kHQ + kHK) {
    __syncthreads();
    for (int r = threadIdx.x; r < nrows; r += blockDim.x)
      if (row_valid(m0 + r, a.T, a.TP)) a.ss_q[(size_t)(m0 + r) * kQkvTiles + tile] = sQ[r * 2] + sQ[r * 2 + 1];
  }
}

// Epilogue of the NST output tiles tile0 .. of a large-M block (rows m0 ..
// m0 + nrows - 1, at most BM) in one pass: every task's global operands are
// fetched first (TMAX tasks per thread at most), then the tasks run, with no
// barrier between tiles; sq / sQ hold NST tiles' scratch (BM rows each).
// Rsum(r, c) and Ssum(r, c) take the block column c.  The arithmetic of each
// output is epi_task's, as in tile_epilogue.
template <int EPI, int NT, int NST, int BM, int TMAX, bool MOD, class RF, class SF>
__device__ __forceinline__ void block_epilogue(const GemmArgs& a, int tile0, int m0, int nrows, RF Rsum, SF Ssum,
                                               const float* sR, const double* sF, float* sq, float* sQ) {
  constexpr bool SSQ = EPI == EPI_RESID_BF || EPI == EPI_RESID_FB;
  constexpr bool QKV = EPI == EPI_QKV;
  constexpr int NOUT = EpiShape<EPI, NT>::NOUT, OUTW = EpiShape<EPI, NT>::OUTW, TPR = EpiShape<EPI, NT>::TPR;
  const int per_tile = nrows * TPR, ntask = NST * per_tile;
  EpiPre pre[TMAX];
  bool ok[TMAX];
#pragma unroll
  for (int k = 0; k < TMAX; ++k) {
    const int e = threadIdx.x + k * blockDim.x;
    const int st = e / per_tile, rc = e - st * per_tile, r = rc / TPR, c0 = (rc - r * TPR) * OUTW;
    ok[k] = e < ntask && row_valid(m0 + r, a.T, a.TP);
    if (ok[k]) epi_fetch<EPI>(a, m0 + r, epi_feature<EPI, NT>(tile0 + st, c0), pre[k]);
  }
#pragma unroll
  for (int k = 0; k < TMAX; ++k) {
    if (!ok[k]) continue;
    const int e = threadIdx.x + k * blockDim.x;
    const int st = e / per_tile, rc = e - st * per_tile, r = rc / TPR, c0 = (rc - r * TPR) * OUTW;
    epi_task<EPI, NT, MOD>(
        a, tile0 + st, m0, r, c0, [&](int rr, int c) { return Rsum(rr, st * NT + c); },
        [&](int rr, int c) { return Ssum(rr, st * NT + c); }, sR, sF + st * 16, sq + st * BM * NOUT,
        sQ + st * BM * 2, pre[k]);
  }
  if (SSQ && a.ss_out) {
    __syncthreads();
    for (int i = threadIdx.x; i < NST * nrows; i += blockDim.x) {
      const int st = i / nrows, r = i - st * nrows;
      if (!row_valid(m0 + r, a.T, a.TP)) continue;
      const float* q = sq + st * BM * NOUT + r * NOUT;
      float t = 0.f;
#pragma unroll
      for (int c = 0; c < NOUT; ++c) t += q[c];
      a.ss_out[(size_t)(m0 + r) * a.ss_out_n + tile0 + st] = t;
    }
  }
  if (QKV) {
    __syncthreads();
    for (int i = threadIdx.x; i < NST * nrows; i += blockDim.x) {
      const int st = i / nrows, r = i - st * nrows;
      if (((tile0 + st) >> 3) < kHQ + kHK && row_valid(m0 + r, a.T, a.TP))
        a.ss_q[(size_t)(m0 + r) * kQkvTiles + tile0 + st] = sQ[st * BM * 2 + r * 2] + sQ[st * BM * 2 + r * 2 + 1];
    }
  }
}

template <int EPI, int NT, int NWAVES, int KSTEPS, int ASRC, int MT>
__global__ __launch_bounds__(NWAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_gemm(GemmArgs a) {
  constexpr int NTT = NT / 16;
  constexpr int KW = KSTEPS * 32;  // reduction elements per wave
  constexpr bool MOD = ASRC == A_MODPRE;   // AdaRMS fused: shift tile + row scale
  constexpr int MB = MT * 16;      // rows per block
  constexpr int RROWS = MB + (MOD ? 16 : 0);  // + the shift tile
  constexpr bool SSQ = EPI == EPI_RESID_BF || EPI == EPI_RESID_FB;
  constexpr bool QKV = EPI == EPI_QKV;
  static_assert(!QKV || NT == 32, "rotation-pair tiles");
  constexpr int NOUT = (EPI == EPI_GEGLU || QKV) ? 16 : NT;  // output features (pairs for QKV) per row
  constexpr int OUTW = EPI == EPI_GEGLU ? 4 : 8;  // outputs per epilogue task
  constexpr int TPR = NOUT / OUTW;                // epilogue tasks per row
  static_assert(!MOD || NWAVES * KW == kH, "the modulated A operand spans one hidden row");
  __shared__ __attribute__((aligned(16))) float red[NWAVES * RROWS * NT];
  __shared__ float sq[SSQ ? MB * NOUT : 1];
  __shared__ __attribute__((aligned(16))) float sH[MOD ? kH : 4], sR[MOD ? MB : 1];
  __shared__ double sF[QKV ? 16 : 1];   // rotation frequencies of the tile (revolutions per position)
  __shared__ float sQ[QKV ? MB * 2 : 1];  // half-tile sums of squares

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int kst = a.K >> 5;           // 32-column steps of a row
  const int ks0 = wave * KSTEPS;      // this wave's first step
  const int k0 = wave * KW;
  const int lk = (lane >> 4) * 8;
  const int lr = lane & 15;

  // weight slab of this wave: NT rows x KW columns, every load in flight now
  bf16x8 wf[KSTEPS][NTT];
#pragma unroll
  for (int nt = 0; nt < NTT; ++nt) {
    const int wt = EPI == EPI_GEGLU ? (nt == 0 ? tile : a.wtile_up + tile)
                   : QKV ? (tile >> 3) * 16 + nt * 8 + (tile & 7)
                         : tile * NTT + nt;
    const uint16_t* wp = a.W + ((size_t)wt * kst + ks0) * 512 + lane * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)  // read once per launch: streaming loads
      wf[ks][nt] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(wp + ks * 512));
  }
  __builtin_amdgcn_sched_barrier(0);
  if (QKV && threadIdx.x < 16) {
    const int j = (tile & 7) * 16 + threadIdx.x;  // dim of the head's first half
    sF[threadIdx.x] = exp2(-(double)j / 128.0 * log2((double)a.rope_base)) * 0.15915494309189533577;
  }

  // row blocks of MB rows; MOD kernels keep every block inside one request
  // (TP / 16 tiles per request, nsub blocks per request); blocks blockIdx.y,
  // blockIdx.y + gridDim.y, ...
  const int nsub = MOD ? (a.TP + MB - 1) / MB : 1;
  const int nblk = MOD ? (a.M / a.TP) * nsub : (a.M + MB - 1) / MB;
  for (int blk = blockIdx.y; blk < nblk; blk += gridDim.y) {
    const int m0 = MOD ? (blk / nsub) * a.TP + (blk % nsub) * MB : blk * MB;
    const int mts = min(MT, (MOD ? a.TP - (blk % nsub) * MB : a.M - m0) >> 4);  // tiles in this block
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
      const int mtile = (m0 >> 4) + min(mt, mts - 1);  // tiles past the block re-read the last one
      const uint16_t* ap = a.A + ((size_t)mtile * kst + ks0) * 512 + lane * 8;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) av[ks][mt] = load_bf16x8(ap + ks * 512);
    }
    float4 msh = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 ssp[4];
    if (MOD) {
      const float* mb = a.nmod + (size_t)(m0 / a.TP) * 3 * kH;
      msh = *reinterpret_cast<const float4*>(mb + kH + threadIdx.x * 4);
      // row statistics: thread (row rr, quarter qq) sums a quarter of the row's partials
      const int rr = threadIdx.x >> 2, qq = threadIdx.x & 3;
      const int per = a.ss_in_n >> 2;  // ss_in_n is a multiple of 4, at most 64
#pragma unroll
      for (int i = 0; i < 4; ++i) ssp[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (rr < mts * 16 && row_valid(m0 + rr, a.T, a.TP)) {
        const float* sp = a.ss_in + (size_t)(m0 + rr) * a.ss_in_n + qq * per;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i * 4 < per) ssp[i] = *reinterpret_cast<const float4*>(sp + i * 4);
      }
    }
    // the epilogue's global operands of this thread's first task
    EpiPre pre;
    {
      const int r = threadIdx.x / TPR, c0 = (threadIdx.x % TPR) * OUTW;
      if (r < mts * 16 && row_valid(m0 + r, a.T, a.TP))
        epi_fetch<EPI>(a, m0 + r, QKV ? (tile >> 3) * kD + (tile & 7) * 16 + c0 : tile * NT + c0, pre);
    }
    __builtin_amdgcn_sched_barrier(0);  // the whole block is in flight before any use

    if (MOD) {
      reinterpret_cast<float4*>(sH)[threadIdx.x] = msh;
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) t += ssp[i].x + ssp[i].y + ssp[i].z + ssp[i].w;
      t += __shfl_xor(t, 1, 64);
      t += __shfl_xor(t, 2, 64);
      const int rr = threadIdx.x >> 2;
      if ((threadIdx.x & 3) == 0 && rr < MB) sR[rr] = 1.0f / sqrtf(t * (1.0f / kH) + kEps);
      __syncthreads();
      // the shift tile's row 0 <- bf16(shift)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
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
    tile_epilogue<EPI, NT, MOD>(
        a, tile, m0, mts * 16,
        [&](int r, int c) {
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < NWAVES; ++w) t += red[(w * RROWS + r) * NT + c];
          return t;
        },
        [&](int, int c) {
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < NWAVES; ++w) t += red[(w * RROWS + MB) * NT + c];
          return t;
        },
        sR, sF, sq, sQ, &pre);
    __syncthreads();
  }
}

// Row scales of a large-M block (AdaRMS: 1 / rms of each row, from the row's
// sums-of-squares partials, summed as k_gemm sums them): thread (row rr,
// quarter qq) of pass p handles row p * NTHR / 4 + rr.  fetch issues the
// loads (before the K loop, so that their latency hides behind its operand
// loads), store finishes the sums into sR.
template <int BM, int NTHR>
struct RowSS {
  static constexpr int NP = (BM * 4 + NTHR - 1) / NTHR;  // passes
  float4 v[NP][4];
  __device__ __forceinline__ void fetch(const GemmArgs& a, int m0, int nrows) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int rr = p * (NTHR / 4) + (threadIdx.x >> 2), qq = threadIdx.x & 3;
      const int per = a.ss_in_n >> 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[p][i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (rr < nrows && row_valid(m0 + rr, a.T, a.TP)) {
        const float* sp = a.ss_in + (size_t)(m0 + rr) * a.ss_in_n + qq * per;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i * 4 < per) v[p][i] = *reinterpret_cast<const float4*>(sp + i * 4);
      }
    }
  }
  __device__ __forceinline__ void store(float* sR) const {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int rr = p * (NTHR / 4) + (threadIdx.x >> 2), qq = threadIdx.x & 3;
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) t += v[p][i].x + v[p][i].y + v[p][i].z + v[p][i].w;
      t += __shfl_xor(t, 1, 64);
      t += __shfl_xor(t, 2, 64);
      if (qq == 0 && rr < BM) sR[rr] = 1.0f / sqrtf(t * (1.0f / kH) + kEps);
    }
  }
};

// Rotation frequencies of the NST output tiles from tile0 (QKV), as k_gemm
// computes them: revolutions per position of the tile's 16 first-half dims.
template <int NST>
__device__ __forceinline__ void rope_freqs(const GemmArgs& a, int tile0, double* sF) {
  if (threadIdx.x < NST * 16) {
    const int tile = tile0 + (threadIdx.x >> 4);
    const int j = (tile & 7) * 16 + (threadIdx.x & 15);
    sF[threadIdx.x] = exp2(-(double)j / 128.0 * log2((double)a.rope_base)) * 0.15915494309189533577;
  }
}

// Large-M projections (batches of requests, the prefix QKV over 2048
// tokens): the same arithmetic as k_gemm, bit for bit, on a schedule that
// keeps the MFMA units busy.  K is split into NR ranges of KSR 32-column steps
// (k_gemm's waves); each range is accumulated from zero in step order by the
// same MFMA, and the range sums are added in range order.  The shift
// tile of the fused AdaRMS holds one row per request of the block.  The
// epilogue is the same tile_epilogue, once per output tile of the block.
// A work-group of 4 waves (2 x 2) owns BM rows x BNF 16-column fragments: wave
// (wm, wn) the rows wm*WMT*16 .. and the fragments wn*WNF ..; every fragment is
// loaded straight from the tiled operands into registers (one 1 KB load per
// wave and fragment) PD steps ahead of its MFMAs.
template <int EPI, int NT, int NR, int KSR, int ASRC, int WMT, int WNF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_big(GemmArgs a) {
  constexpr bool MOD = ASRC == A_MODPRE;
  constexpr bool QKV = EPI == EPI_QKV;
  constexpr bool SSQ = EPI == EPI_RESID_BF || EPI == EPI_RESID_FB;
  constexpr int NOUT = (EPI == EPI_GEGLU || QKV) ? 16 : NT;
  constexpr int NTT = NT / 16;       // fragments per output tile
  constexpr int BM = 2 * WMT * 16;   // rows per block
  constexpr int BNF = 2 * WNF;       // fragments per block
  constexpr int BN = BNF * 16;       // columns per block
  constexpr int NST = BNF / NTT;     // output tiles per block
  constexpr int KS = NR * KSR;       // 32-column steps of K
  constexpr int MAXREQ = BM / 16 + 1;  // requests a block can touch (at least 16 rows each)
  // steps in flight per wave: 8 where the fragments are few (64 x 64 blocks,
  // 32 KB per wave), else what the registers allow
  constexpr int PD = WMT + WNF <= 4 ? 8 : 2;
  static_assert(KSR % PD == 0 && BNF % NTT == 0, "block shape");
  static_assert(!MOD || KS * 32 == kH, "the modulated A operand spans one hidden row");
  constexpr int TLD = BN + 4;  // sTot row stride (floats): rows 4 banks apart
  __shared__ __attribute__((aligned(16))) float sTot[BM * TLD];  // range sums [row][column]
  __shared__ float sShift[MOD ? MAXREQ * BN : 1];               // shift sums [request][column]
  __shared__ float sR[MOD ? BM : 1];
  __shared__ double sF[QKV ? NST * 16 : 1];
  __shared__ float sq[SSQ ? NST * BM * NOUT : 1];
  __shared__ float sQ[QKV ? NST * BM * 2 : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = blockIdx.y * BM;
  const int nrows = min(BM, a.M - m0);
  const int last_tile = a.M / 16 - 1;
  const int b0 = m0 / a.TP;
  const int nreq = MOD ? (m0 + nrows - 1) / a.TP - b0 + 1 : 0;
  const bool shift_wave = MOD && wm == 0;

  // operand base pointers (step 0) of this wave's fragments
  const uint16_t* ap[WMT];
  const uint16_t* wp[WNF];
#pragma unroll
  for (int i = 0; i < WMT; ++i) {
    const int mtile = min(m0 / 16 + wm * WMT + i, last_tile);  // rows past M re-read the last tile
    ap[i] = a.A + (size_t)mtile * KS * 512 + lane * 8;
  }
#pragma unroll
  for (int j = 0; j < WNF; ++j) {
    const int fj = wn * WNF + j, st = fj / NTT, nt = fj % NTT;
    const int tile = blockIdx.x * NST + st;
    const int wt = EPI == EPI_GEGLU ? (nt == 0 ? tile : a.wtile_up + tile)
                   : QKV ? (tile >> 3) * 16 + nt * 8 + (tile & 7)
                         : tile * NTT + nt;
    wp[j] = a.W + (size_t)wt * KS * 512 + lane * 8;
  }
  // shift vector of request b0 + lr (lanes past the block's requests read
  // request b0's and hold zeros); every wave loads it, so that all waves
  // issue the same loads and the ring's waits stay exact
  const bool h_ok = MOD && lr < nreq;
  const float* hp = MOD ? a.nmod + (size_t)(b0 + (h_ok ? lr : 0)) * 3 * kH + kH + lq * 8 : nullptr;

  // a ring of PD steps in flight per wave: step s lives in slot s % PD from
  // PD steps before its MFMAs until they have run
  bf16x8 Ab[PD][WMT], Wb[PD][WNF];
  float4 Hb[PD][2];
  auto load = [&](int ks, bf16x8* A, bf16x8* W, float4* Hs) {
#pragma unroll
    for (int i = 0; i < WMT; ++i) A[i] = load_bf16x8(ap[i] + (size_t)ks * 512);
#pragma unroll
    for (int j = 0; j < WNF; ++j) W[j] = load_bf16x8(wp[j] + (size_t)ks * 512);  // shared by the row blocks
    if (MOD) {
      Hs[0] = *reinterpret_cast<const float4*>(hp + ks * 32);
      Hs[1] = *reinterpret_cast<const float4*>(hp + ks * 32 + 4);
    }
  };
  f32x4 acc[WMT][WNF], accs[WNF], tot[WMT][WNF];  // tot: the range sums so far
  auto mma = [&](const bf16x8* A, const bf16x8* W, const float4* Hs) {
    if (shift_wave) {
      const float hv[8] = {Hs[0].x, Hs[0].y, Hs[0].z, Hs[0].w, Hs[1].x, Hs[1].y, Hs[1].z, Hs[1].w};
      bf16x8 hs;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t p = h_ok ? pack2(hv[e], hv[e + 1]) : 0u;
        hs[e] = (short)(p & 0xffffu);
        hs[e + 1] = (short)(p >> 16);
      }
#pragma unroll
      for (int j = 0; j < WNF; ++j) accs[j] = mfma16(hs, W[j], accs[j]);
    }
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNF; ++j) acc[i][j] = mfma16(A[i], W[j], acc[i][j]);
  };
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNF; ++j) acc[i][j] = zero_f32x4();
#pragma unroll
    for (int j = 0; j < WNF; ++j) accs[j] = zero_f32x4();
  };
  // range r's sum added to the total (in registers; the shift sums in LDS)
  auto flush = [&](int r) {
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNF; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tot[i][j][e] = (r == 0 ? 0.f : tot[i][j][e]) + acc[i][j][e];
        }
    if (shift_wave) {
#pragma unroll
      for (int j = 0; j < WNF; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * lq + e < nreq) {
            float* d = sShift + (4 * lq + e) * BN + (wn * WNF + j) * 16 + lr;
            *d = (r == 0 ? 0.f : *d) + accs[j][e];
          }
    }
  };

  RowSS<BM, 256> rss;
  if (MOD) rss.fetch(a, m0, nrows);
#pragma unroll
  for (int d = 0; d < PD; ++d) load(d, Ab[d], Wb[d], Hb[d]);
  if (MOD) rss.store(sR);  // read after the K loop's last barrier
  if (QKV) rope_freqs<NST>(a, blockIdx.x * NST, sF);
  zero_acc();
#pragma unroll 1
  for (int s0 = 0; s0 < KS; s0 += PD) {
#pragma unroll
    for (int d = 0; d < PD; ++d) {
      const int ks = s0 + d;
      mma(Ab[d], Wb[d], Hb[d]);
      __builtin_amdgcn_sched_barrier(0);  // keep the refill PD steps ahead of its use
      load(min(ks + PD, KS - 1), Ab[d], Wb[d], Hb[d]);  // past the end: re-read the last step, unused
      __builtin_amdgcn_sched_barrier(0);
      if ((ks + 1) % KSR == 0) {  // end of a range
        flush(ks / KSR);
        zero_acc();
      }
    }
  }

  // the total into LDS: lane (lr, lq) holds rows 4 lq .. 4 lq + 3 of each tile, column lr
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNF; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sTot[((wm * WMT + i) * 16 + 4 * lq + e) * TLD + (wn * WNF + j) * 16 + lr] = tot[i][j][e];
  __syncthreads();
  constexpr int TMAX = (NST * BM * EpiShape<EPI, NT>::TPR + 255) / 256;
  block_epilogue<EPI, NT, NST, BM, TMAX, MOD>(
      a, blockIdx.x * NST, m0, nrows, [&](int r, int c) { return sTot[r * TLD + c]; },
      [&](int r, int c) { return sShift[((m0 + r) / a.TP - b0) * BN + c]; }, sR, sF, sq, sQ);
}

// Block (column cb, row rb) of work-group blockIdx when the grid is dealt to
// XCDs in compact pieces.  The dispatcher deals work-groups round robin, so
// the work-groups of linear id = k mod 8 share XCD k's L2; they take the k-th
// eighth of the blocks in strip order (strips of W column blocks, left to
// right, each row by row), so that each XCD fetches a few row blocks of A and
// W column blocks instead of most of both.
__device__ __forceinline__ void xcd_block(int W, int& cb, int& rb) {
  const int gx = gridDim.x, gy = gridDim.y, n = gx * gy;
  const int L = blockIdx.y * gx + blockIdx.x, k = L & 7, sl = L >> 3;
  const int idx = k * (n >> 3) + min(k, n & 7) + sl;  // class k holds n / 8 (+ 1 for k < n % 8) blocks
  const int nfull = gx / W, per = gy * W;              // whole strips, blocks per whole strip
  const int st = idx / per;
  if (st < nfull) {
    const int p = idx - st * per;
    rb = p / W;
    cb = st * W + p % W;
  } else {  // the narrower last strip
    const int w2 = gx - nfull * W, p = idx - nfull * per;
    rb = p / w2;
    cb = nfull * W + p % w2;
  }
}

// Wide large-M projections, the same arithmetic as k_gemm bit for bit, with
// the operands shared through LDS.  A work-group of NWM x NWN waves owns BM =
// NWM * WMT * 16 rows x NWN * 64 columns (8 waves, two per SIMD: 2 x 4 for
// 256 columns, 4 x 2 for 128).  Each 32-column step's operand fragments
// (BM/16 A tiles, 4 NWN W fragments, 1 KB each) are copied from HBM straight
// into an LDS stage by loads that bypass registers (global_load_lds, 16 B per
// lane, so a wave's fragment lands as one contiguous 1 KB block), STAGES - 1
// steps ahead of their use; each wave reads its WMT A tiles and 4 W fragments
// of the next step from LDS while the MFMAs of the current one run.  K is
// split into the same NR ranges of KSR steps as the skinny kernel's waves;
// each range is accumulated from zero in step order and the range sums are
// added in range order in registers.
// KG > 1 (blocks too few or too small to keep 8 waves per CU busy): KG
// groups of NWM x NWN waves share the block, group g running ranges
// g NR / KG .. with a stage ring of its own, in the same barriers; every
// group keeps its range sums apart (in the accumulators if it has one), and
// after the loop group 0 adds them all in range order (the other groups'
// through LDS), EPH rows at a time.
template <int EPI, int NT, int NR, int KSR, int ASRC, int WMT, int NWN, int STG, int KG, int NWM>
__global__ __launch_bounds__(64 * NWM * NWN * KG) __attribute__((amdgpu_waves_per_eu(NWM * NWN * KG / 4, 2))) void k_gemm_lds(
    GemmArgs a) {
  constexpr bool MOD = ASRC == A_MODPRE;
  constexpr bool QKV = EPI == EPI_QKV;
  constexpr bool SSQ = EPI == EPI_RESID_BF || EPI == EPI_RESID_FB;
  constexpr int NOUT = (EPI == EPI_GEGLU || QKV) ? 16 : NT;
  constexpr int NWG = NWM * NWN;       // waves per K group (NWM along M, NWN along N)
  constexpr int NW = NWG * KG;         // waves
  constexpr int WNF = 4;               // W fragments per wave
  constexpr int BM = NWM * WMT * 16;   // rows per block
  constexpr int BNF = NWN * WNF;       // fragments per block
  constexpr int BN = BNF * 16;         // columns per block
  constexpr int NTT = NT / 16, NST = BNF / NTT;
  constexpr int KS = NR * KSR;
  constexpr int NRG = NR / KG;         // ranges per K group
  constexpr int KSG = NRG * KSR;       // steps per K group
  constexpr int AF = BM / 16;          // A tiles per step
  constexpr int SF = AF + BNF;         // fragments per step
  constexpr int DPW = SF / NWG;        // fragments each wave copies per step
  // a ring of STAGES steps, AHEAD = STAGES - 1 of them copied ahead: LDS
  // latency times bandwidth needs about 100 KB in flight per CU
  constexpr int STAGES = STG, AHEAD = STAGES - 1;
  constexpr int MAXREQ = BM / 16 + 1;
  constexpr int STAGE_EL = SF * 512;   // bf16 elements per stage
  constexpr int TLD = BN + 4;           // sTot row stride (floats): rows 4 banks apart
  // the epilogue runs in passes of EPH rows (one row half of the waves each
  // when the block has more than 128 rows), their sums staged in sTot
  constexpr int EPH = BM > 128 ? BM / 2 : BM;
  // the other groups' range sums [group - 1][range][row][column] after the
  // loop (sTot behind them)
  constexpr int XCH = (KG - 1) * NRG * EPH * TLD * 4;
  constexpr int RING = KG * STAGES * STAGE_EL * 2;
  // after the loop: the exchanged sums, sTot and (K groups) the epilogue's
  // sums of squares of every output tile of the block
  constexpr int SQB = SSQ ? (KG > 1 ? NST : 1) * BM * NOUT * 4 : 0;
  constexpr int POST = XCH + EPH * TLD * 4 + (KG > 1 ? SQB : 0);
  constexpr int RAW = RING > POST ? RING : POST;
  // NR == 1: one range, accumulated straight through K (the projections
  // that always run this schedule, so no other schedule's sum order binds)
  constexpr bool RANGES = NR > 1;
  static_assert(RANGES || !MOD, "the AdaRMS-fused projections follow the skinny kernel's ranges");
  static_assert(KG == 1 || (!MOD && !QKV && RANGES && NR % KG == 0), "K groups: plain projections");
  static_assert(SF % NWG == 0 && BNF % NTT == 0 && KSG % 2 == 0 && AHEAD <= KSG && AHEAD * DPW < 64, "block shape");
  static_assert(!MOD || KS * 32 == kH, "the modulated A operand spans one hidden row");
  // One LDS array for everything: the stages during the K loop (the range
  // sums [row][column] after it), then the bf16 shift vectors, the shift
  // sums [request][column], the row scales, the rotation frequencies and the
  // epilogue's sums of squares.  With several LDS arrays the compiler makes
  // every LDS read of the loop wait for all copies in flight; the loop's
  // explicit waits and barriers order the copies and the reads instead.
  constexpr int O_HB = RAW;
  constexpr int O_SHIFT = O_HB + (MOD ? MAXREQ * kH * 2 : 0);
  constexpr int O_R = O_SHIFT + (MOD ? MAXREQ * BN * 4 : 0);
  constexpr int O_F = (O_R + (MOD ? BM * 4 : 0) + 7) & ~7;
  constexpr int O_Q2 = KG > 1 ? XCH + EPH * TLD * 4 : O_F + (QKV ? NST * 16 * 8 : 0);
  constexpr int O_Q = KG > 1 ? O_F : O_Q2 + SQB;
  constexpr int LDS_BYTES = O_Q + (QKV ? NST * BM * 2 * 4 : 0);  // sQ: every tile's (one-pass epilogue)
  __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];
  uint16_t* stage = reinterpret_cast<uint16_t*>(smem);
  float* sTot = reinterpret_cast<float*>(smem + XCH);
  float* sX = reinterpret_cast<float*>(smem);
  uint16_t* sHb = reinterpret_cast<uint16_t*>(smem + O_HB);
  float* sShift = reinterpret_cast<float*>(smem + O_SHIFT);
  float* sR = reinterpret_cast<float*>(smem + O_R);
  double* sF = reinterpret_cast<double*>(smem + O_F);
  float* sq = reinterpret_cast<float*>(smem + O_Q2);
  float* sQ = reinterpret_cast<float*>(smem + O_Q);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = wave / NWG, wig = wave % NWG;  // K group, wave in the group
  const int wm = wig / NWN, wn = wig % NWN;
  const int lr = lane & 15, lq = lane >> 4;
  int cb = blockIdx.x, rb = blockIdx.y;
  if (a.xcd_strip > 0) xcd_block(a.xcd_strip, cb, rb);
  const int cblk = cb;  // column block (of this launch's columns)
  const int tile0 = a.tile0 + cblk * NST;  // the block's first output tile
  const int m0 = rb * BM;
  const int nrows = min(BM, a.M - m0);
  const int last_tile = a.M / 16 - 1;
  const int b0 = m0 / a.TP;
  const int nreq = MOD ? (m0 + nrows - 1) / a.TP - b0 + 1 : 0;

  // fragments this wave copies: f = wig * DPW + d (A tiles first, then W),
  // from the group's first step on
  const uint16_t* gsrc[DPW];
#pragma unroll
  for (int d = 0; d < DPW; ++d) {
    const int f = wig * DPW + d;
    if (f < AF) {
      gsrc[d] = a.A + (size_t)min(m0 / 16 + f, last_tile) * KS * 512 + lane * 8;  // rows past M: last tile
    } else {
      const int fj = f - AF, st = fj / NTT, nt = fj % NTT;
      const int tile = tile0 + st;
      const int wt = EPI == EPI_GEGLU ? (nt == 0 ? tile : a.wtile_up + tile)
                     : QKV ? (tile >> 3) * 16 + nt * 8 + (tile & 7)
                           : tile * NTT + nt;
      gsrc[d] = a.W + (size_t)wt * KS * 512 + lane * 8;
    }
    gsrc[d] += (size_t)g * KSG * 512;
  }
  uint16_t* const ring = stage + g * STAGES * STAGE_EL;  // the group's stages
  auto issue = [&](int ks) {
    uint16_t* dst = ring + (ks % STAGES) * STAGE_EL;
#pragma unroll
    for (int d = 0; d < DPW; ++d)
      lds_copy16(gsrc[d] + (size_t)ks * 512, dst + (wig * DPW + d) * 512);
  };

  // accs / stot: the shift tile's sums of this wave's W fragments (range,
  // total); every wave runs them, so that the loop has no branch (with one,
  // the compiler waits for every LDS read in flight before the MFMAs); the
  // waves of row half 0 keep theirs
  // rs (K groups): the group's range sums, range q of the group in rs[q]
  f32x4 acc[WMT][WNF], tot[WMT][WNF], accs[WNF], stot[WNF], rs[KG > 1 && NRG > 1 ? NRG : 1][WMT][WNF];
#pragma unroll
  for (int i = 0; i < WMT; ++i)
#pragma unroll
    for (int j = 0; j < WNF; ++j) acc[i][j] = zero_f32x4();
#pragma unroll
  for (int j = 0; j < WNF; ++j) accs[j] = zero_f32x4();

  // this wave's fragments of step ks from its stage (A tiles, W fragments,
  // the shift row of each request; lanes past the block's requests read
  // request 0's and zero it)
  auto read_frags = [&](int ks, bf16x8* af, bf16x8* wf, bf16x8& hs) {
    const uint16_t* st = ring + (ks % STAGES) * STAGE_EL;
#pragma unroll
    for (int i = 0; i < WMT; ++i) af[i] = *reinterpret_cast<const bf16x8*>(st + (wm * WMT + i) * 512 + lane * 8);
#pragma unroll
    for (int j = 0; j < WNF; ++j)
      wf[j] = *reinterpret_cast<const bf16x8*>(st + (AF + wn * WNF + j) * 512 + lane * 8);
    if (MOD) hs = *reinterpret_cast<const bf16x8*>(sHb + (lr < nreq ? lr : 0) * kH + ks * 32 + lq * 8);
  };
  auto step_mma = [&](int ks, const bf16x8* af, const bf16x8* wf, bf16x8 hs) {
    if (MOD) {
      const bf16x8 h = __builtin_bit_cast(bf16x8, keep_or_zero(lr < nreq, __builtin_bit_cast(uint4, hs)));
#pragma unroll
      for (int j = 0; j < WNF; ++j) accs[j] = mfma16(h, wf[j], accs[j]);
    }
#pragma unroll
    for (int i = 0; i < WMT; ++i)
#pragma unroll
      for (int j = 0; j < WNF; ++j) acc[i][j] = mfma16(af[i], wf[j], acc[i][j]);
    if (KG > 1 && NRG > 1 && (ks + 1) % KSR == 0) {  // end of a range: its sums kept apart
#pragma unroll
      for (int q = 0; q + 1 < NRG; ++q)
#pragma unroll
        for (int i = 0; i < WMT; ++i)
#pragma unroll
          for (int j = 0; j < WNF; ++j) rs[q][i][j] = rs[q + 1][i][j];
#pragma unroll
      for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int j = 0; j < WNF; ++j) {
          rs[NRG - 1][i][j] = acc[i][j];
          acc[i][j] = zero_f32x4();
        }
    } else if (KG == 1 && RANGES && (ks + 1) % KSR == 0) {  // end of a range: add its sums in range order
      const bool first = ks + 1 == KSR;
#pragma unroll
      for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int j = 0; j < WNF; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) tot[i][j][e] = (first ? 0.f : tot[i][j][e]) + acc[i][j][e];
          acc[i][j] = zero_f32x4();
        }
      if (MOD) {
#pragma unroll
        for (int j = 0; j < WNF; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) stot[j][e] = (first ? 0.f : stot[j][e]) + accs[j][e];
          accs[j] = zero_f32x4();
        }
      }
    }
  };

  // Step ks: its fragments were read from LDS during step ks - 1.  Wait for
  // step ks + 1's copies (own, then everyone's at the barrier, which also
  // means every wave has consumed step ks - 1's fragments), refill step
  // ks - 1's stage with step ks + AHEAD, read step ks + 1's fragments, then
  // run step ks's MFMAs while those reads are in flight.
  // set-up inputs first (the block's shift vectors, the rows' sums-of-squares
  // partials), then the first copies, then the set-up: its loads land while
  // the copies are in flight
  constexpr int NTHR = NW * 64;
  constexpr int SHP = (MAXREQ * (kH / 2) + NTHR - 1) / NTHR;  // shift pairs per thread
  float2 shv[MOD ? SHP : 1];
  RowSS<BM, NTHR> rss;
  if (MOD) {
#pragma unroll
    for (int k = 0; k < SHP; ++k) {
      const int i = threadIdx.x + k * NTHR, q = i / (kH / 2), k2 = (i - q * (kH / 2)) * 2;
      shv[k] = q < nreq ? *reinterpret_cast<const float2*>(a.nmod + (size_t)(b0 + q) * 3 * kH + kH + k2)
                        : make_float2(0.f, 0.f);
    }
    rss.fetch(a, m0, nrows);
  }
#pragma unroll
  for (int k = 0; k < AHEAD; ++k) issue(k);
  if (MOD) {  // the shift vectors rounded to bf16, as the shift tile holds them
#pragma unroll
    for (int k = 0; k < SHP; ++k) {
      const int i = threadIdx.x + k * NTHR, q = i / (kH / 2), k2 = (i - q * (kH / 2)) * 2;
      if (q < nreq) *reinterpret_cast<uint32_t*>(sHb + q * kH + k2) = pack2(shv[k].x, shv[k].y);
    }
    rss.store(sR);
  }
  if (QKV) rope_freqs<NST>(a, tile0, sF);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the set-up's LDS writes are done before the barrier
  wait_vmcnt<(AHEAD - 1) * DPW>();
  lds_barrier();
  bf16x8 af0[WMT], wf0[WNF], af1[WMT], wf1[WNF], hs0 = zero_bf16x8(), hs1 = zero_bf16x8();
  read_frags(0, af0, wf0, hs0);
#pragma unroll 1
  for (int ks = 0; ks < KSG; ks += 2) {
    // even step ks (fragments in set 0), then odd step ks + 1 (set 1); KSG is even
    wait_vmcnt<(AHEAD - 2) * DPW>();
    lds_barrier();
    issue(min(ks + AHEAD, KSG - 1));
    read_frags(ks + 1, af1, wf1, hs1);
    step_mma(ks, af0, wf0, hs0);
    wait_vmcnt<(AHEAD - 2) * DPW>();
    lds_barrier();
    issue(min(ks + 1 + AHEAD, KSG - 1));
    read_frags(min(ks + 2, KSG - 1), af0, wf0, hs0);  // past the end: a landed stage, unused
    step_mma(ks + 1, af1, wf1, hs1);
  }
  wait_vmcnt<0>();
  __syncthreads();  // every copy has landed and every stage read: the stages become sTot

  if (KG > 1) {
    // per epilogue pass of EPH rows: the other groups' range sums of the
    // pass's rows into LDS, then group 0 adds every range in range order
    // (0 + r0, + r1, ...) into sTot; a group with one range holds it in acc
    auto rsum = [&](int q, int i, int j) -> const f32x4& { return NRG == 1 ? acc[i][j] : rs[q][i][j]; };
#pragma unroll 1
    for (int p0 = 0; p0 < BM; p0 += EPH) {
      const bool in_pass = wm * WMT * 16 >= p0 && wm * WMT * 16 < p0 + EPH;
      auto xidx = [&](int gq, int i, int j, int e) {
        return (gq * EPH + (wm * WMT + i) * 16 - p0 + 4 * lq + e) * TLD + (wn * WNF + j) * 16 + lr;
      };
      if (g > 0 && in_pass) {
#pragma unroll
        for (int q = 0; q < NRG; ++q)
#pragma unroll
          for (int i = 0; i < WMT; ++i)
#pragma unroll
            for (int j = 0; j < WNF; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) sX[xidx((g - 1) * NRG + q, i, j, e)] = rsum(q, i, j)[e];
      }
      __syncthreads();
      if (g == 0 && in_pass) {
#pragma unroll
        for (int i = 0; i < WMT; ++i)
#pragma unroll
          for (int j = 0; j < WNF; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              tot[i][j][e] = 0.f + rsum(0, i, j)[e];
#pragma unroll
              for (int q = 1; q < NRG; ++q) tot[i][j][e] += rsum(q, i, j)[e];
            }
#pragma unroll
        for (int gq = 0; gq < (KG - 1) * NRG; ++gq)
#pragma unroll
          for (int i = 0; i < WMT; ++i)
#pragma unroll
            for (int j = 0; j < WNF; ++j)
#pragma unroll
              for (int e = 0; e < 4; ++e) tot[i][j][e] += sX[xidx(gq, i, j, e)];
#pragma unroll
        for (int i = 0; i < WMT; ++i)
#pragma unroll
          for (int j = 0; j < WNF; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sTot[((wm * WMT + i) * 16 - p0 + 4 * lq + e) * TLD + (wn * WNF + j) * 16 + lr] = tot[i][j][e];
      }
      __syncthreads();
      const int prows = min(EPH, nrows - p0);
      if (EPH == BM) {  // one pass: every output tile's operands fetched first
        constexpr int TMAX = (NST * EPH * EpiShape<EPI, NT>::TPR + NW * 64 - 1) / (NW * 64);
        block_epilogue<EPI, NT, NST, EPH, TMAX, false>(
            a, tile0, m0, nrows, [&](int r, int c) { return sTot[r * TLD + c]; },
            [&](int, int) { return 0.f; }, sR, sF, sq, sQ);
      } else {
#pragma unroll 1
        for (int st = 0; st < NST; ++st) {
          if (prows > 0)
            tile_epilogue<EPI, NT, false>(
                a, tile0 + st, m0 + p0, prows, [&](int r, int c) { return sTot[r * TLD + st * NT + c]; },
                [&](int, int) { return 0.f; }, sR, sF, sq, sQ, nullptr);
          __syncthreads();
        }
      }
    }
    return;
  }

  // the shift sums [request][column], lane (lr, lq) holding requests 4 lq .. 4 lq + 3
  if (MOD && wm == 0) {
#pragma unroll
    for (int j = 0; j < WNF; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * lq + e < nreq) sShift[(4 * lq + e) * BN + (wn * WNF + j) * 16 + lr] = stot[j][e];
  }
#pragma unroll 1
  for (int p0 = 0; p0 < BM; p0 += EPH) {
    // the pass's sums into LDS: lane (lr, lq) holds rows 4 lq .. 4 lq + 3 of each tile, column lr
    if (wm * WMT * 16 >= p0 && wm * WMT * 16 < p0 + EPH) {
#pragma unroll
      for (int i = 0; i < WMT; ++i)
#pragma unroll
        for (int j = 0; j < WNF; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sTot[((wm * WMT + i) * 16 - p0 + 4 * lq + e) * TLD + (wn * WNF + j) * 16 + lr] =
                RANGES ? tot[i][j][e] : acc[i][j][e];
    }
    __syncthreads();
    const int prows = min(EPH, nrows - p0);
    if constexpr (QKV && EPH == BM) {
      // the rotation epilogue in one pass over the block's tiles, every
      // task's operands fetched first (as k_gemm_big runs it; the fused
      // gate-up measured no faster this way, 27.9 vs 27.4 us)
      constexpr int TMAX = (NST * BM * EpiShape<EPI, NT>::TPR + NW * 64 - 1) / (NW * 64);
      block_epilogue<EPI, NT, NST, BM, TMAX, MOD>(
          a, tile0, m0, nrows, [&](int r, int c) { return sTot[r * TLD + c]; },
          [&](int r, int c) { return sShift[((m0 + r) / a.TP - b0) * BN + c]; }, sR, sF, sq, sQ);
    } else {
#pragma unroll 1
      for (int st = 0; st < NST; ++st) {  // (one pass over all tiles measured no faster for these)
        const int tile = tile0 + st;
        if (prows > 0)
          tile_epilogue<EPI, NT, MOD>(
              a, tile, m0 + p0, prows, [&](int r, int c) { return sTot[r * TLD + st * NT + c]; },
              [&](int r, int c) { return sShift[((m0 + p0 + r) / a.TP - b0) * BN + st * NT + c]; },
              sR + p0, sF + st * 16, sq, sQ, nullptr);
        __syncthreads();
      }
    }
  }
}

#define DMX_GEMM(EPI, NT, NW, KS, SRC, MT, GY) \
  k_gemm<EPI, NT, NW, KS, SRC, MT><<<dim3(a.ntiles, GY), dim3((NW) * 64), 0, s>>>(a)

int gemm_config(GemmKind kind, GemmArgs& a) {
  switch (kind) {
    case GEMM_QKV1024: a.ntiles = kQKV / 16; a.K = kH; break;
    case GEMM_QKV1024_MODPRE: a.ntiles = kQKV / 32; a.K = kH; break;
    case GEMM_QKV2560: a.ntiles = kQKV / 16; a.K = 2560; break;
    case GEMM_OPROJ: a.ntiles = kH / 16; a.K = kHQ * kD; break;
    case GEMM_OPROJ_F32: a.ntiles = kH / 16; a.K = kHQ * kD; break;
    case GEMM_GATEUP: a.ntiles = kI / 16; a.K = kH; a.wtile_up = kI / 16; break;
    case GEMM_GATEUP_MOD: a.ntiles = kI / 16; a.K = kH; a.wtile_up = kI / 16; break;
    case GEMM_DOWN: a.ntiles = kH / 16; a.K = kI; break;
    case GEMM_DOWN_F32RES: a.ntiles = kH / 16; a.K = kI; break;
    case GEMM_PRE_OPROJ: a.ntiles = kPrefixHidden / 16; a.K = kHQ * kD; break;
    case GEMM_PRE_GATEUP: a.ntiles = kPrefixInter / 16; a.K = kPrefixHidden; a.wtile_up = kPrefixInter / 16; break;
    case GEMM_PRE_DOWN: a.ntiles = kPrefixHidden / 16; a.K = kPrefixInter; break;
  }
  return a.ntiles;
}

#define DMX_GEMM_BIG(EPI, NT, NR, KSR, SRC, WMT, WNF)                                              \
  k_gemm_big<EPI, NT, NR, KSR, SRC, WMT, WNF>                                                        \
      <<<dim3(a.ntiles * (NT) / (32 * (WNF)), (a.M + 32 * (WMT) - 1) / (32 * (WMT))), dim3(256), 0, s>>>(a)

// XS: strips of XS column blocks dealt to XCDs (xcd_block), 0 for the plain grid
#define DMX_GEMM_LDS_W(XS, EPI, NT, NR, KSR, SRC, WMT, NWN, STG, KG, NWM)                          \
  do {                                                                                              \
    GemmArgs b_ = a;                                                                                \
    b_.xcd_strip = (XS);                                                                            \
    k_gemm_lds<EPI, NT, NR, KSR, SRC, WMT, NWN, STG, KG, NWM>                                       \
        <<<dim3(b_.ntiles * (NT) / (64 * (NWN)), (b_.M + 16 * (NWM) * (WMT) - 1) / (16 * (NWM) * (WMT))), \
           dim3(64 * (NWM) * (NWN) * (KG)), 0, s>>>(b_);                                            \
  } while (0)
// two waves along M
#define DMX_GEMM_LDS(XS, EPI, NT, NR, KSR, SRC, WMT, NWN, STG, KG) \
  DMX_GEMM_LDS_W(XS, EPI, NT, NR, KSR, SRC, WMT, NWN, STG, KG, 2)

// Row count from which the large-M schedules run a projection: k_gemm_lds
// for the plain wide ones (the prefix QKV), the AdaRMS-fused gate-up, the
// AdaRMS-fused QKV (128 x 128 blocks of 8 waves, 4 along M: 21.6 us at 1024
// rows against 25.6 on k_gemm_big) and the 1024-column projections (64 x 64
// blocks, 256 for 1024 rows, each shared by 4 K groups of 2 waves);
// k_gemm_big for the plain gate-up.
constexpr int kBigGemmRows = 256;

hipError_t launch_gemm(GemmKind kind, const GemmArgs& a, hipStream_t s) {
  // prefix layer: the large-M schedule at every row count; the 2560-column
  // projections on 192 x 128 blocks in 2 K groups (220 blocks for 2048 rows,
  // where 128 x 256 blocks leave 96 CUs idle)
  switch (kind) {
    case GEMM_PRE_OPROJ: DMX_GEMM_LDS(5, EPI_F32, 16, 2, 32, A_GLOBAL, 6, 2, 4, 2); return hipGetLastError();
    case GEMM_PRE_GATEUP: {
      // 256 x 256 blocks; where they would run 2.5 or 1.25 rounds over the
      // CUs (1024 or 2048 rows), the last 128 tiles run in a launch of their
      // own as 128 x 256 blocks, one round of blocks with 3/4 the bytes
      // (the prefix layer 532 -> 519 us at 2048 tokens; 524 with 256 x 128)
      const int gy = (a.M + 255) / 256, tail = (gy == 4 || gy == 8) ? 128 : 0;
      GemmArgs b = a;
      b.ntiles = a.ntiles - tail;
      {
        const GemmArgs& a = b;
        DMX_GEMM_LDS(0, EPI_GEGLU, 32, 1, 80, A_GLOBAL, 8, 4, 4, 1);
      }
      if (tail) {
        b.tile0 = b.ntiles;
        b.ntiles = tail;
        const GemmArgs& a = b;
        DMX_GEMM_LDS(4, EPI_GEGLU, 32, 1, 80, A_GLOBAL, 4, 4, 4, 1);
      }
      return hipGetLastError();
    }
    case GEMM_PRE_DOWN: DMX_GEMM_LDS(5, EPI_F32, 16, 2, 160, A_GLOBAL, 6, 2, 4, 2); return hipGetLastError();
    default: break;
  }
  if (a.M >= kBigGemmRows) {
    switch (kind) {
      case GEMM_QKV1024: DMX_GEMM_LDS(0, EPI_F32, 16, 4, 8, A_GLOBAL, 4, 4, 6, 1); break;
      case GEMM_QKV1024_MODPRE: DMX_GEMM_LDS_W(0, EPI_QKV, 32, 4, 8, A_MODPRE, 2, 2, 8, 1, 4); break;
      case GEMM_QKV2560: DMX_GEMM_LDS(4, EPI_F32, 16, 4, 20, A_GLOBAL, 4, 4, 6, 1); break;
      case GEMM_OPROJ: DMX_GEMM_LDS(8, EPI_RESID_BB, 16, 8, 8, A_GLOBAL, 2, 1, 4, 4); break;
      case GEMM_OPROJ_F32: DMX_GEMM_LDS(8, EPI_RESID_BF, 16, 8, 8, A_GLOBAL, 2, 1, 4, 4); break;
      case GEMM_GATEUP: DMX_GEMM_BIG(EPI_GEGLU, 32, 4, 8, A_GLOBAL, 4, 4); break;
      case GEMM_GATEUP_MOD: DMX_GEMM_LDS(0, EPI_GEGLU, 32, 4, 8, A_MODPRE, 4, 4, 5, 1); break;
      case GEMM_DOWN: DMX_GEMM_LDS(8, EPI_RESID_BB, 16, 8, 16, A_GLOBAL, 2, 1, 4, 4); break;
      case GEMM_DOWN_F32RES: DMX_GEMM_LDS(8, EPI_RESID_FB, 16, 8, 16, A_GLOBAL, 2, 1, 4, 4); break;
      default: break;  // the prefix kinds returned above
    }
    return hipGetLastError();
  }
  // row blocks: one per WG up to 4 (more blocks loop inside the WG)
  const int tiles = a.M / 16;
  const int mb1 = std::min(4, tiles), mb2 = std::min(4, (tiles + 1) / 2);
  // MOD kinds: blocks stay inside one request, so the row tiles per block
  // follow the request's padded rows (TP / 16 = 1 .. 4): a block tile past
  // the request would re-read the last one for nothing
  const int nreq = std::min(4, a.M / a.TP);
  const int tpr = a.TP / 16;  // row tiles per request
  const int nreq2 = std::min(8, (a.M / a.TP) * ((a.TP + 31) / 32));
  const int nreq1 = std::min(8, (a.M / a.TP) * tpr);
  switch (kind) {
    case GEMM_QKV1024: DMX_GEMM(EPI_F32, 16, 4, 8, A_GLOBAL, 2, mb2); break;
    case GEMM_QKV1024_MODPRE:
      if (tpr % 2 == 0)
        DMX_GEMM(EPI_QKV, 32, 4, 8, A_MODPRE, 2, nreq2);
      else
        DMX_GEMM(EPI_QKV, 32, 4, 8, A_MODPRE, 1, nreq1);
      break;
    case GEMM_QKV2560: DMX_GEMM(EPI_F32, 16, 4, 20, A_GLOBAL, 1, 4); break;
    case GEMM_OPROJ: DMX_GEMM(EPI_RESID_BB, 16, 8, 8, A_GLOBAL, 1, mb1); break;
    case GEMM_OPROJ_F32: DMX_GEMM(EPI_RESID_BF, 16, 8, 8, A_GLOBAL, 1, mb1); break;
    case GEMM_GATEUP: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_GLOBAL, 2, mb2); break;
    case GEMM_GATEUP_MOD:
      switch (tpr) {
        case 1: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_MODPRE, 1, nreq); break;
        case 2: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_MODPRE, 2, nreq); break;
        case 3: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_MODPRE, 3, nreq); break;
        default: DMX_GEMM(EPI_GEGLU, 32, 4, 8, A_MODPRE, 4, nreq); break;
      }
      break;
    case GEMM_DOWN: DMX_GEMM(EPI_RESID_BB, 16, 8, 16, A_GLOBAL, 1, mb1); break;
    case GEMM_DOWN_F32RES: DMX_GEMM(EPI_RESID_FB, 16, 8, 16, A_GLOBAL, 1, mb1); break;
    default: break;
  }
  return hipGetLastError();
}

// Row-major bf16 rows [B][T][K] -> tiled rows [B*TP][K] (request b's token t
// at tiled row b*TP + t).  One wave per row; lane j takes the 16-column
// groups j, j + 64, ...  With ss != null (K = 1024) it also writes the row's
// 64 sums of squares of 16 columns, summed in column order with every square
// rounded before the add, exactly as the GEMM epilogues do.  With scale !=
// null (K = 1024) the tiled copy holds bf16(x * (1 + scale[b])) instead of x
// (the A operand of an AdaRMS-fused projection), scale[b] at scale + b *
// scale_stride; the sums of squares are always those of x.
__global__ __launch_bounds__(256) void k_pack_rows(const uint16_t* x, int B, int T, int TP, int K, uint16_t* out,
                                                   float* ss, const float* scale, int scale_stride) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= B * T) return;
  const int b = m / T, t = m - b * T;
  const int prow = b * TP + t;
  const uint16_t* src = x + (size_t)m * K;
  for (int j = lane; j < K / 16; j += 64) {
    const uint4 r0 = *reinterpret_cast<const uint4*>(src + j * 16);
    const uint4 r1 = *reinterpret_cast<const uint4*>(src + j * 16 + 8);
    const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    uint32_t o[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    if (scale) {
      const float* sp = scale + (size_t)b * scale_stride + j * 16;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s0 = 1.f + sp[2 * i], s1 = 1.f + sp[2 * i + 1];
        o[i] = pack2(bf2f((uint16_t)(w[i] & 0xffffu)) * s0, bf2f((uint16_t)(w[i] >> 16)) * s1);
      }
    }
    *reinterpret_cast<uint4*>(out + tile_off(prow, j * 16, K)) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(out + tile_off(prow, j * 16 + 8, K)) = make_uint4(o[4], o[5], o[6], o[7]);
    if (ss) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float lo = bf2f((uint16_t)(w[i] & 0xffffu)), hi = bf2f((uint16_t)(w[i] >> 16));
        const float l2 = lo * lo, h2 = hi * hi;
        acc += l2;
        acc += h2;
      }
      ss[(size_t)prow * kSsParts + j] = acc;
    }
  }
}

hipError_t launch_pack_rows(const uint16_t* x, int B, int T, int TP, int K, uint16_t* out, float* ss,
                            hipStream_t s, const float* scale, int scale_stride) {
  const int rows = B * T;
  k_pack_rows<<<dim3((rows + 3) / 4), dim3(256), 0, s>>>(x, B, T, TP, K, out, ss, scale, scale_stride);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Modulation vectors of several (W_mod, b_mod) pairs in one launch:
// out_j[b] = W_j * cond[b] + b_j.  Work-group (j, tile) owns 16 features of
// matrix j (tiled weights); all loads of its 32 KB weight slab are issued up
// front.
__global__ __launch_bounds__(256) void k_mod_multi(ModBatch mb) {
  const int j = blockIdx.x / (3 * kH / 16), tile = blockIdx.x - j * (3 * kH / 16);
  __shared__ float red[4 * 256];
  mod_unit(mb.job[j], tile, mb.B, red);
}

hipError_t launch_mod_multi(const ModBatch& mb, hipStream_t s) {
  if (mb.n == 0) return hipSuccess;
  k_mod_multi<<<dim3(mb.n * (3 * kH / 16)), dim3(256), 0, s>>>(mb);
  return hipGetLastError();
}

}  // namespace dmx
