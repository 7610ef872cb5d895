// Masked GQA suffix attention on gfx950 (OpenDM DM0.5 fast-stack article,
// §2.2: logits over the prefix KV cache and the suffix KV together under the
// prefix-visibility mask, online softmax, value-weighted sum).
//
// Work decomposition (flash-decoding style, split over the prefix):
//   one work-group per (request b, KV head g, key split s).  Splits 0..S-1 own
//   kps consecutive prefix rows each; split S owns the chunk's own suffix keys.
//   The 2 query heads that share KV head g are stacked into one tile of
//   2*chunk query rows (row r: head 2g + r / chunk, token r % chunk), so every
//   K/V row is read from HBM once per request.
//   Keys stream through LDS in blocks of 32: K as [key][dim], V transposed to
//   [dim][key] so both MFMA operands read 16 contiguous bytes per lane.
//   QK^T and PV run on v_mfma_f32_16x16x32_bf16; row max / sum use cross-lane
//   shuffles inside each 16-lane row group; the softmax runs in the log2
//   domain.  A block whose 32 keys are all invisible is skipped without
//   reading its K/V; invisible keys inside a block are zero-filled in LDS and
//   their logits replaced by -inf (selection, never multiplication), so masked
//   rows may hold anything, NaN included.
// Each split writes (running max, running sum, output / sum) per row; a
// combine kernel merges the S + 1 partials per row.
#include "dmx_device.hpp"
#include "dmx_internal.hpp"

namespace dmx {

namespace {
constexpr int KB = 32;          // keys per LDS block
constexpr int KLD = kD + 8;     // K row stride in LDS (bf16 elements), padded
constexpr int VLD = KB + 8;     // V^T row stride in LDS (bf16 elements), padded
constexpr int PLD = KB + 8;     // P tile row stride (bf16 elements)
constexpr int kMaxKps = 64;     // prefix keys per split (upper bound)
constexpr float kNegBig = -1e30f;
}  // namespace

// RoPE frequency table in LDS, in revolutions per position:
// f[j] = rope_base^(-j/128) / (2 pi), j < 128 (pairs j, j + 128).
__device__ __forceinline__ void rope_table(double* f, float base) {
  if (threadIdx.x < kD / 2) {
    const double lb = log2((double)base);
    f[threadIdx.x] = exp2(-(double)threadIdx.x / (kD / 2) * lb) * 0.15915494309189533577;
  }
}

// sin / cos of pos * f (revolutions), reduced exactly in double first.
__device__ __forceinline__ void rope_sincos(double pos, double f, float& sn, float& cs) {
  double rev = pos * f;
  rev -= floor(rev);
  const float r = (float)rev;
  sn = __builtin_amdgcn_sinf(r);
  cs = __builtin_amdgcn_cosf(r);
}

// Q fragments of one stacked query row built from the raw fp32 projection:
// lane (lr, lq) holds dims lq*8 + ks*32 + e (ks < 8, e < 8) of its row, which
// includes both halves (ks and ks + 4) of every rotation pair it touches.
struct QRaw {
  float4 x[8][2];
};

__device__ __forceinline__ void q_load(const AttnArgs& a, int b, int i, int head, int lq, QRaw& q) {
  const float* src = a.raw + (size_t)(b * a.C + i) * kQKV + head * kD + lq * 8;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    q.x[ks][0] = *reinterpret_cast<const float4*>(src + ks * 32);
    q.x[ks][1] = *reinterpret_cast<const float4*>(src + ks * 32 + 4);
  }
}

__device__ __forceinline__ void q_finish(const AttnArgs& a, const double* ftab, const uint16_t* qn, const QRaw& q,
                                         int b, int i, bool ok, int lq, bf16x8 qf[8]) {
  float ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const float4 x0 = q.x[ks][0], x1 = q.x[ks][1];
    ss += x0.x * x0.x + x0.y * x0.y + x0.z * x0.z + x0.w * x0.w + x1.x * x1.x + x1.y * x1.y + x1.z * x1.z +
          x1.w * x1.w;
  }
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  const float rn = 1.0f / sqrtf(ss * (1.0f / kD) + kEps);
  const double pos = (double)a.pos0[b] + (double)i;
  // rotation pairs: dims lq*8 + ks*32 + e (ks < 4) and the same + 128 (ks + 4)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const float lo[8] = {q.x[ks][0].x, q.x[ks][0].y, q.x[ks][0].z, q.x[ks][0].w,
                         q.x[ks][1].x, q.x[ks][1].y, q.x[ks][1].z, q.x[ks][1].w};
    const float hi[8] = {q.x[ks + 4][0].x, q.x[ks + 4][0].y, q.x[ks + 4][0].z, q.x[ks + 4][0].w,
                         q.x[ks + 4][1].x, q.x[ks + 4][1].y, q.x[ks + 4][1].z, q.x[ks + 4][1].w};
    const uint4 wl4 = *reinterpret_cast<const uint4*>(qn + lq * 8 + ks * 32);
    const uint4 wh4 = *reinterpret_cast<const uint4*>(qn + 128 + lq * 8 + ks * 32);
    const uint32_t wl[4] = {wl4.x, wl4.y, wl4.z, wl4.w}, wh[4] = {wh4.x, wh4.y, wh4.z, wh4.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sn, cs;
      rope_sincos(pos, ftab[lq * 8 + ks * 32 + e], sn, cs);
      const float w0 = 1.f + bf2f((uint16_t)((e & 1) ? (wl[e >> 1] >> 16) : (wl[e >> 1] & 0xffffu)));
      const float w1 = 1.f + bf2f((uint16_t)((e & 1) ? (wh[e >> 1] >> 16) : (wh[e >> 1] & 0xffffu)));
      const float x0 = lo[e] * rn * w0, x1 = hi[e] * rn * w1;
      qf[ks][e] = ok ? (short)f2bf(x0 * cs - x1 * sn) : (short)0;
      qf[ks + 4][e] = ok ? (short)f2bf(x1 * cs + x0 * sn) : (short)0;
    }
  }
}

// Suffix keys of one 32-key block built from the raw projection into LDS:
// thread t handles key j = t / 16 and dims d0 = (t % 16) * 8 .. +7 plus their
// rotation partners d0 + 128 (K), and the 16 V dims (t % 16) * 16 .. +15.
struct SufRaw {
  float4 k[4], v[4];
};

__device__ __forceinline__ void suffix_load(const AttnArgs& a, int b, int g, int kb0, SufRaw& r) {
  const int j = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int key = min(kb0 + j, a.C - 1);  // rows past the chunk read a valid row and are zeroed later
  const float* row = a.raw + (size_t)(b * a.C + key) * kQKV;
  const float* kr = row + (kHQ + g) * kD;
  r.k[0] = *reinterpret_cast<const float4*>(kr + c * 8);
  r.k[1] = *reinterpret_cast<const float4*>(kr + c * 8 + 4);
  r.k[2] = *reinterpret_cast<const float4*>(kr + 128 + c * 8);
  r.k[3] = *reinterpret_cast<const float4*>(kr + 128 + c * 8 + 4);
  const float* vr = row + (kHQ + kHK + g) * kD + c * 16;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) r.v[q4] = *reinterpret_cast<const float4*>(vr + q4 * 4);
}

__device__ __forceinline__ void suffix_store(const AttnArgs& a, const double* ftab, const uint16_t* kn, const SufRaw& r,
                                             int b, int kb0, const int* vis, uint16_t* sK, uint16_t* sVt) {
  const int j = threadIdx.x >> 4, c = threadIdx.x & 15;
  const int key = kb0 + j;
  const bool ok = vis[j] != 0;
  const float lo[8] = {r.k[0].x, r.k[0].y, r.k[0].z, r.k[0].w, r.k[1].x, r.k[1].y, r.k[1].z, r.k[1].w};
  const float hi[8] = {r.k[2].x, r.k[2].y, r.k[2].z, r.k[2].w, r.k[3].x, r.k[3].y, r.k[3].z, r.k[3].w};
  const uint4 wlo = *reinterpret_cast<const uint4*>(kn + c * 8), whi = *reinterpret_cast<const uint4*>(kn + 128 + c * 8);
  const uint32_t wl[4] = {wlo.x, wlo.y, wlo.z, wlo.w}, wh[4] = {whi.x, whi.y, whi.z, whi.w};
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += lo[e] * lo[e] + hi[e] * hi[e];
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float rn = 1.0f / sqrtf(ss * (1.0f / kD) + kEps);
  const double pos = (double)a.pos0[b] + (double)key;
  uint32_t ko[4], kh[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    float o0[2], o1[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * e2 + h;
      float sn, cs;
      rope_sincos(pos, ftab[c * 8 + e], sn, cs);
      const float w0 = 1.f + bf2f((uint16_t)(h ? (wl[e2] >> 16) : (wl[e2] & 0xffffu)));
      const float w1 = 1.f + bf2f((uint16_t)(h ? (wh[e2] >> 16) : (wh[e2] & 0xffffu)));
      const float x0 = lo[e] * rn * w0, x1 = hi[e] * rn * w1;
      o0[h] = ok ? x0 * cs - x1 * sn : 0.f;
      o1[h] = ok ? x1 * cs + x0 * sn : 0.f;
    }
    ko[e2] = pack2(o0[0], o0[1]);
    kh[e2] = pack2(o1[0], o1[1]);
  }
  *reinterpret_cast<uint4*>(sK + j * KLD + c * 8) = make_uint4(ko[0], ko[1], ko[2], ko[3]);
  *reinterpret_cast<uint4*>(sK + j * KLD + 128 + c * 8) = make_uint4(kh[0], kh[1], kh[2], kh[3]);
  const float vv[16] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w, r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w,
                        r.v[2].x, r.v[2].y, r.v[2].z, r.v[2].w, r.v[3].x, r.v[3].y, r.v[3].z, r.v[3].w};
#pragma unroll
  for (int e = 0; e < 16; ++e) sVt[(c * 16 + e) * VLD + j] = ok ? f2bf(vv[e]) : (uint16_t)0;
}

// K / V rows (bf16, from global) of one 32-key block: thread t owns 16-byte
// chunks t and t + 512 of the 32 x 32 chunk grid.  Rows are read whether
// visible or not (rows past the split's end read its last row); invisible rows
// are replaced by zeros when staged, so their contents never reach the math.
struct KVRegs {
  uint4 k[2], v[2];
};

__device__ __forceinline__ void kv_load(const uint16_t* Kb, const uint16_t* Vb, int kb0, int key_hi, KVRegs& r) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = threadIdx.x + h * 512;
    const int j = c >> 5, ch = c & 31;
    const size_t row = (size_t)min(kb0 + j, key_hi - 1);
    r.k[h] = *reinterpret_cast<const uint4*>(Kb + row * kD + ch * 8);
    r.v[h] = *reinterpret_cast<const uint4*>(Vb + row * kD + ch * 8);
  }
}

__device__ __forceinline__ void kv_store(const KVRegs& r, const int* vis, uint16_t* sK, uint16_t* sVt) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = threadIdx.x + h * 512;
    const int j = c >> 5, ch = c & 31;
    const bool ok = vis[j] != 0;
    const uint4 kk = ok ? r.k[h] : make_uint4(0, 0, 0, 0);
    const uint4 vv = ok ? r.v[h] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(sK + j * KLD + ch * 8) = kk;
    const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sVt[(ch * 8 + 2 * e) * VLD + j] = (uint16_t)(w4[e] & 0xffffu);
      sVt[(ch * 8 + 2 * e + 1) * VLD + j] = (uint16_t)(w4[e] >> 16);
    }
  }
}

// One split of one (request, KV head): every global load of the split (mask,
// query rows, both K/V blocks or the raw suffix rows) is issued up front, then
// the blocks are staged through LDS and processed.
template <bool FUSED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_attn_partial(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[KB * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[kD * VLD];
  __shared__ __attribute__((aligned(16))) uint16_t sP[8][16 * PLD];
  __shared__ int sVis[kMaxKps];
  __shared__ double sF[kD / 2];
  __shared__ __attribute__((aligned(16))) uint16_t sNW[2][kD];  // q / k norm weights

  const int nsplit = a.S + 1;
  const int split = blockIdx.x % nsplit;
  const int bg = blockIdx.x / nsplit;
  const int g = bg % kHK, b = bg / kHK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int R = 2 * a.C, MT = (R + 15) >> 4;

  const bool suffix = (split == a.S);
  const int key_lo = suffix ? 0 : split * a.kps;
  const int key_hi = suffix ? a.C : min(a.P, key_lo + a.kps);
  const int nkeys = key_hi - key_lo;
  const int nblk = (nkeys + KB - 1) / KB;  // <= 2
  const size_t kv_rows = suffix ? (size_t)a.C : (size_t)a.P;
  const uint16_t* Kb = (suffix ? a.ks : a.kp) + (size_t)(b * kHK + g) * kv_rows * kD;
  const uint16_t* Vb = (suffix ? a.vs : a.vp) + (size_t)(b * kHK + g) * kv_rows * kD;
  const bool from_global = !(FUSED && suffix);

  // ---- load phase: everything this WG reads from global memory
  const int mt = wave;
  const bool active = mt < MT;
  const int row = mt * 16 + lr;
  const bool qok = active && (row < R);
  const int hh = qok ? row / a.C : 0;
  const int qi = qok ? row - hh * a.C : 0;
  KVRegs kv[2];
  SufRaw sr[2];
  QRaw qr;
  bf16x8 qf[8];
  int mvis = 0;
  uint4 nw = make_uint4(0, 0, 0, 0);
  if (FUSED && threadIdx.x >= 64 && threadIdx.x < 128) {
    const int t = threadIdx.x - 64;  // 64 threads x 16 B = both 512-B weight vectors
    nw = *reinterpret_cast<const uint4*>((t < 32 ? a.qn_w : a.kn_w) + (t & 31) * 8);
  }
  if (threadIdx.x < kMaxKps && threadIdx.x < nkeys)
    mvis = suffix || a.mask[(size_t)b * a.P + key_lo + threadIdx.x] != 0;
  if (from_global) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
      if (bi < nblk) kv_load(Kb, Vb, key_lo + bi * KB, key_hi, kv[bi]);
  } else {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
      if (bi < nblk) suffix_load(a, b, g, bi * KB, sr[bi]);
  }
  if (FUSED) {
    q_load(a, b, qi, kGroup * g + hh, lq, qr);
  } else {
    const uint16_t* qp = a.q + ((size_t)(b * a.C + qi) * kHQ + (kGroup * g + hh)) * kD + lq * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = load_bf16x8(qp + ks * 32);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- compute phase
  if (threadIdx.x < kMaxKps) sVis[threadIdx.x] = mvis;
  if (FUSED && threadIdx.x >= 64 && threadIdx.x < 128) {
    const int t = threadIdx.x - 64;
    *reinterpret_cast<uint4*>(&sNW[t >> 5][(t & 31) * 8]) = nw;
  }
  if (FUSED) rope_table(sF, a.rope_base);
  __syncthreads();
  if (FUSED) q_finish(a, sF, sNW[0], qr, b, qi, qok, lq, qf);
  else if (!qok) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = zero_bf16x8();
  }

  f32x4 o[16];
  float mrun[4], lrun[4];
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) o[dt] = zero_f32x4();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mrun[r] = kNegBig;
    lrun[r] = 0.f;
  }
  const float sl2 = 1.4426950408889634f / 16.0f;  // log2(e) / sqrt(head_dim)
  uint16_t* pt = &sP[wave][0];

#pragma unroll
  for (int bi = 0; bi < 2; ++bi) {
    if (bi >= nblk) break;
    const int* vis = sVis + bi * KB;
    int any = 0;
    for (int j = 0; j < KB; ++j) any |= vis[j];
    if (!any) continue;  // uniform across the WG
    if (from_global)
      kv_store(kv[bi], vis, sK, sVt);
    else
      suffix_store(a, sF, sNW[1], sr[bi], b, bi * KB, vis, sK, sVt);
    __syncthreads();
    if (active) {
      const bool vis0 = vis[lr] != 0, vis1 = vis[16 + lr] != 0;
      f32x4 s0 = zero_f32x4(), s1 = zero_f32x4();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(sK + lr * KLD + ks * 32 + lq * 8);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(sK + (16 + lr) * KLD + ks * 32 + lq * 8);
        s0 = mfma16(qf[ks], k0, s0);
        s1 = mfma16(qf[ks], k1, s1);
      }
      float alpha[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = vis0 ? s0[r] * sl2 : -INFINITY;
        const float x1 = vis1 ? s1[r] * sl2 : -INFINITY;
        const float mloc = group16_max(fmaxf(x0, x1));
        const float mnew = fmaxf(mrun[r], mloc);
        alpha[r] = exp2f(mrun[r] - mnew);
        mrun[r] = mnew;
        const float p0 = exp2f(x0 - mnew), p1 = exp2f(x1 - mnew);
        lrun[r] = lrun[r] * alpha[r] + p0 + p1;
        pt[(lq * 4 + r) * PLD + lr] = f2bf(p0);
        pt[(lq * 4 + r) * PLD + 16 + lr] = f2bf(p1);
      }
#pragma unroll
      for (int dt = 0; dt < 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[dt][r] *= alpha[r];
      __builtin_amdgcn_wave_barrier();
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(pt + lr * PLD + lq * 8);
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sVt + (dt * 16 + lr) * VLD + lq * 8);
        o[dt] = mfma16(pa, vf, o[dt]);
      }
    }
    __syncthreads();
  }

  // write this split's partial rows: running max, running sum, output / sum
  if (active) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float l = group16_sum(lrun[r]);
      const int prow_i = mt * 16 + lq * 4 + r;
      const size_t prow = ((size_t)bg * nsplit + split) * a.R16 + prow_i;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) a.part_o[prow * kD + dt * 16 + lr] = f2bf(o[dt][r] * inv);
      if (lr == 0) {
        a.part_ml[prow * 2] = mrun[r];
        a.part_ml[prow * 2 + 1] = l;
      }
    }
  }
}

// One wave per (request, KV head, stacked row): merge the split partials.
// Lane s first fetches split s's (max, sum); then every lane accumulates its
// 4 output dims over the splits with all loads of a batch in flight.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, uint16_t* ctx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = 2 * a.C;
  const int wid = blockIdx.x * 4 + wave;
  if (wid >= a.B * kHK * R) return;
  const int row = wid % R, bg = wid / R;
  const int g = bg % kHK, b = bg / kHK;
  const int nsplit = a.S + 1;  // <= 65
  const size_t base = (size_t)bg * nsplit * a.R16 + row;
  float m0 = kNegBig, l0 = 0.f, m1 = kNegBig, l1 = 0.f;
  if (lane < nsplit) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (base + (size_t)lane * a.R16) * 2);
    m0 = ml.x;
    l0 = ml.y;
  }
  if (lane + 64 < nsplit) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (base + (size_t)(lane + 64) * a.R16) * 2);
    m1 = ml.x;
    l1 = ml.y;
  }
  float M = fmaxf(l0 > 0.f ? m0 : kNegBig, l1 > 0.f ? m1 : kNegBig);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float w0 = l0 > 0.f ? l0 * exp2f(m0 - M) : 0.f;
  const float w1 = l1 > 0.f ? l1 * exp2f(m1 - M) : 0.f;
  const float L = wave_sum(w0 + w1);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    uint2 raw[8];
    float ws[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u;
      ws[u] = s < 64 ? __shfl(w0, s & 63, 64) : __shfl(w1, s & 63, 64);
      raw[u] = make_uint2(0, 0);
      if (s < nsplit && ws[u] != 0.f)
        raw[u] = *reinterpret_cast<const uint2*>(a.part_o + (base + (size_t)s * a.R16) * kD + lane * 4);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < nsplit && ws[u] != 0.f) {
        acc[0] += ws[u] * bf2f((uint16_t)(raw[u].x & 0xffffu));
        acc[1] += ws[u] * bf2f((uint16_t)(raw[u].x >> 16));
        acc[2] += ws[u] * bf2f((uint16_t)(raw[u].y & 0xffffu));
        acc[3] += ws[u] * bf2f((uint16_t)(raw[u].y >> 16));
      }
    }
  }
  const float inv = 1.0f / L;
  const int hh = row / a.C, i = row - hh * a.C;
  uint16_t* dst = ctx + ((size_t)(b * a.C + i) * kHQ + kGroup * g + hh) * kD + lane * 4;
  uint2 outv;
  outv.x = pack2(acc[0] * inv, acc[1] * inv);
  outv.y = pack2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(dst) = outv;
}

void attn_config(int B, int C, int P, AttnArgs& a) {
  a.B = B;
  a.C = C;
  a.P = P;
  a.kps = kMaxKps;
  a.S = (P + a.kps - 1) / a.kps;
  a.R16 = ((2 * C + 15) / 16) * 16;
}

hipError_t launch_attention(const AttnArgs& a, uint16_t* ctx, hipStream_t s) {
  if (a.raw)
    k_attn_partial<true><<<dim3(a.B * kHK * (a.S + 1)), dim3(512), 0, s>>>(a);
  else
    k_attn_partial<false><<<dim3(a.B * kHK * (a.S + 1)), dim3(512), 0, s>>>(a);
  const int rows = a.B * kHK * 2 * a.C;
  k_attn_combine<<<dim3((rows + 3) / 4), dim3(256), 0, s>>>(a, ctx);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// AdaRMS prenorm (fast-stack article §2.2, "Adarms 调制 prenorm"):
// xn = x / sqrt(mean x^2 + eps) * (1 + scale[b]) + shift[b], one WG per row.
// The input row is bf16 (layer input) or fp32 (the layer-internal residual).
__device__ __forceinline__ void load4(const uint16_t* p, float v[4]) {
  const uint2 raw = *reinterpret_cast<const uint2*>(p);
  v[0] = bf2f((uint16_t)(raw.x & 0xffffu));
  v[1] = bf2f((uint16_t)(raw.x >> 16));
  v[2] = bf2f((uint16_t)(raw.y & 0xffffu));
  v[3] = bf2f((uint16_t)(raw.y >> 16));
}
__device__ __forceinline__ void load4(const float* p, float v[4]) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x;
  v[1] = f.y;
  v[2] = f.z;
  v[3] = f.w;
}

template <typename TX>
__global__ __launch_bounds__(256) void k_adarms_norm(const TX* x, const float* mod, int T, uint16_t* xn) {
  __shared__ float part[4];
  const int m = blockIdx.x, b = m / T;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float v[4];
  load4(x + (size_t)m * kH + threadIdx.x * 4, v);
  float ss = wave_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  ss = part[0] + part[1] + part[2] + part[3];
  const float r = 1.0f / sqrtf(ss * (1.0f / kH) + kEps);
  const float* sc = mod + (size_t)b * 3 * kH + threadIdx.x * 4;
  const float* sh = sc + kH;
  uint2 o;
  o.x = pack2(v[0] * r * (1.f + sc[0]) + sh[0], v[1] * r * (1.f + sc[1]) + sh[1]);
  o.y = pack2(v[2] * r * (1.f + sc[2]) + sh[2], v[3] * r * (1.f + sc[3]) + sh[3]);
  *reinterpret_cast<uint2*>(xn + (size_t)m * kH + threadIdx.x * 4) = o;
}

hipError_t launch_adarms_norm(const uint16_t* x, const float* mod, int M, int T, uint16_t* xn,
                              hipStream_t s) {
  k_adarms_norm<uint16_t><<<dim3(M), dim3(256), 0, s>>>(x, mod, T, xn);
  return hipGetLastError();
}

hipError_t launch_adarms_norm_f32(const float* x, const float* mod, int M, int T, uint16_t* xn,
                                  hipStream_t s) {
  k_adarms_norm<float><<<dim3(M), dim3(256), 0, s>>>(x, mod, T, xn);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// QK-RMSNorm ((1 + w) weights) + RoPE (pairs j, j + 128) on the raw fp32 QKV
// projection, written out as bf16 q / k / v (fast-stack article §2.2, "QKV 投影
// QK-Norm RoPE 一次完成").  One wave per token; lane l owns elements
// 2l, 2l+1, 128+2l, 129+2l of every head.  Angles are formed and reduced
// modulo 2*pi in double precision before the fp32 sine / cosine.
__global__ __launch_bounds__(256) void k_qknorm_rope(const float* raw, const uint16_t* qn_w,
                                                     const uint16_t* kn_w, const int32_t* pos0,
                                                     float base, int M, int T, uint16_t* q,
                                                     uint16_t* k, uint16_t* v, int kv_rows,
                                                     int kv_row0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = blockIdx.x * 4 + wave;
  if (m >= M) return;
  const int b = m / T, t = m - (m / T) * T;
  const double pos = (double)pos0[b] + (double)t;
  const double lb = log2((double)base);
  const double two_pi = 6.283185307179586476925;
  float cs[2], sn[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int j = 2 * lane + e;
    double th = pos * exp2(-(double)j / 128.0 * lb);
    th -= floor(th / two_pi) * two_pi;
    sincosf((float)th, &sn[e], &cs[e]);
  }
  const float* src = raw + (size_t)m * kQKV;
  for (int h = 0; h < kHQ + kHK; ++h) {
    const bool isq = h < kHQ;
    const uint16_t* wn = isq ? qn_w : kn_w;
    const float2 lo = *reinterpret_cast<const float2*>(src + h * kD + 2 * lane);
    const float2 hi = *reinterpret_cast<const float2*>(src + h * kD + 128 + 2 * lane);
    const float ss = wave_sum(lo.x * lo.x + lo.y * lo.y + hi.x * hi.x + hi.y * hi.y);
    const float r = 1.0f / sqrtf(ss * (1.0f / kD) + kEps);
    const float a0 = lo.x * r * (1.f + bf2f(wn[2 * lane])), a1 = lo.y * r * (1.f + bf2f(wn[2 * lane + 1]));
    const float c0 = hi.x * r * (1.f + bf2f(wn[128 + 2 * lane])), c1 = hi.y * r * (1.f + bf2f(wn[129 + 2 * lane]));
    const uint32_t outlo = pack2(a0 * cs[0] - c0 * sn[0], a1 * cs[1] - c1 * sn[1]);
    const uint32_t outhi = pack2(c0 * cs[0] + a0 * sn[0], c1 * cs[1] + a1 * sn[1]);
    uint16_t* dst = isq ? q + ((size_t)m * kHQ + h) * kD
                        : k + (((size_t)b * kHK + (h - kHQ)) * kv_rows + kv_row0 + t) * kD;
    *reinterpret_cast<uint32_t*>(dst + 2 * lane) = outlo;
    *reinterpret_cast<uint32_t*>(dst + 128 + 2 * lane) = outhi;
  }
  for (int hv = 0; hv < kHK; ++hv) {
    const float4 x4 = *reinterpret_cast<const float4*>(src + (kHQ + kHK + hv) * kD + 4 * lane);
    uint2 o;
    o.x = pack2(x4.x, x4.y);
    o.y = pack2(x4.z, x4.w);
    *reinterpret_cast<uint2*>(v + (((size_t)b * kHK + hv) * kv_rows + kv_row0 + t) * kD + 4 * lane) = o;
  }
}

hipError_t launch_qknorm_rope(const float* raw, const uint16_t* qn_w, const uint16_t* kn_w,
                              const int32_t* pos0, float base, int M, int T, uint16_t* q,
                              uint16_t* k, uint16_t* v, int kv_rows, int kv_row0, hipStream_t s) {
  k_qknorm_rope<<<dim3((M + 3) / 4), dim3(256), 0, s>>>(raw, qn_w, kn_w, pos0, base, M, T, q, k, v,
                                                        kv_rows, kv_row0);
  return hipGetLastError();
}

__global__ void k_fill_zero(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = (n16 + 255) / 256;
  k_fill_zero<<<dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s>>>((uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace dmx
