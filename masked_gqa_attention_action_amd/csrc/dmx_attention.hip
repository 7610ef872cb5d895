// Masked GQA suffix attention on gfx950 (OpenDM DM0.5 fast-stack article,
// §2.2: logits over the prefix KV cache and the suffix KV together under the
// prefix-visibility mask, online softmax, value-weighted sum).
//
// Work decomposition (flash-decoding style, split over the prefix):
//   one work-group per (request b, KV head g, key split s).  Splits 0..S-1 own
//   kps consecutive prefix rows each; splits S..S+NS-1 own the chunk's own
//   suffix keys, 32 each.
//   The 2 query heads that share KV head g are stacked into 2*TP query rows
//   (TP = chunk padded to 16; row r: head 2g + r / TP, token r % TP), so every
//   K/V row is read from HBM once per request; wave w owns stacked rows
//   16w .. 16w+15 (one token tile of one head).
//   In the fused layer the queries and suffix keys arrive from the QKV
//   epilogue already rotated: q = r * y with y = rope((1 + w) * x) and
//   r = 1 / sqrt(mean x^2 + eps) from the epilogue's sums of squares, so this
//   kernel only scales and rounds them.
//   All K/V blocks (32 keys) of the split are staged row-major in LDS at once.
//   The products run transposed on v_mfma_f32_16x16x32_bf16:
//     S^T = K Q^T   (A = K rows from LDS, B = the wave's query fragments),
//     O^T = V^T P^T (A = V^T through the gfx950 LDS transpose read, B = P^T
//                    straight from the S^T accumulators: each lane holds keys
//                    4q..4q+3 and 16+4q..16+4q+3 of its row, and V^T is read
//                    with the same key order, so P never leaves registers).
//   Each lane therefore owns one query row: the online-softmax rescale is one
//   scalar per lane, and the output dims 16t + 4q .. +3 go out as 8-byte
//   stores.  The softmax runs in the log2 domain.  A block whose 32 keys are
//   all invisible is skipped; invisible keys inside a block are zero-filled
//   in LDS and their logits replaced by -inf (selection, never
//   multiplication), so masked rows may hold anything, NaN included.
// Each split writes (running max, running sum, output / sum) per row, the
// outputs as 16 x 256 row tiles, each row's 16 dims of a dim tile contiguous
// (a store instruction of a wave covers 512 contiguous bytes; padded query
// rows write nothing, so a tile's few valid rows touch few cache lines); a
// combine kernel merges the S + NS partials of each row in split order.
#include "dmx_device.hpp"
#include "dmx_internal.hpp"
#include "dmx_mod.hpp"
#include "dmx_tiles.hpp"

namespace dmx {

namespace {
constexpr int KB = 32;          // keys per block
constexpr int KLD = kD + 8;     // K row stride in LDS (bf16): 528 B, 16 B past a bank period
constexpr int VLD = kD + 16;    // V row stride in LDS (bf16): 544 B, 32 B past a bank period
constexpr int kMaxNB = 4;       // blocks per split (upper bound)
// splits per batch of the combine's loads (upper bound: from 22 on the
// compiler runs out of scalar registers for the load addresses)
constexpr int kCombineMaxBatch = 21;
#define DMX_COMBINE_BATCHES(X)                                                                      \
  X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16) X(17) X(18) \
  X(19) X(20) X(21)
// Query heads of a KV group per attention work-group: one (4 waves) while the
// grid is small, both (8 waves, each K/V block read once for the pair) once
// one-head work-groups would exceed two per CU (batches).  Each wave's rows
// see the same blocks in the same order either way, so the outputs match.
constexpr int kAttnPairFromWgs = 512;
constexpr float kNegBig = -1e30f;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
}  // namespace

// Q fragments of one stacked query row from the tiled bf16 epilogue output
// (rope((1 + w) * x), not yet divided by the row's rms): lane (lr, lq) holds
// dims ks*32 + lq*8 + e (ks < 8, e < 8) of its row, which is the MFMA B
// fragment as loaded; each load instruction of the wave reads 1 KB of
// contiguous memory.  The head's 8 sums of squares come along: the query's
// 1 / rms scales its logits instead of the operand.
__device__ __forceinline__ void q_load(const AttnArgs& a, int prow, int head, int lq, bf16x8 qf[8], float4 ss[2]) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = load_bf16x8(a.qvb + tile_off(prow, head * kD + ks * 32 + lq * 8, kQVB));
  const float* sp = a.ss_q + (size_t)prow * kQkvTiles + head * 8;
  ss[0] = *reinterpret_cast<const float4*>(sp);
  ss[1] = *reinterpret_cast<const float4*>(sp + 4);
}

__device__ __forceinline__ float q_rnorm(const float4 ss[2]) {
  const float t = ((ss[0].x + ss[0].y) + (ss[0].z + ss[0].w)) + ((ss[1].x + ss[1].y) + (ss[1].z + ss[1].w));
  return 1.0f / sqrtf(t * (1.0f / kD) + kEps);
}

// Suffix keys of one 32-key block from the epilogue output into LDS: thread
// t handles key j = t / 16 (+ 16 i for the i-th of its keys when the
// work-group has 256 threads) and the 16 dims (t % 16) * 16 .. +15 of K
// (fp32, scaled by the key row's 1 / rms) and V (bf16 already).
struct SufRaw {
  float4 k[4];
  uint4 v[2];
  float ss;
};

__device__ __forceinline__ void suffix_load(const AttnArgs& a, int b, int g, int kb0, int j, SufRaw& r) {
  const int c = threadIdx.x & 15;
  const int key = min(kb0 + j, a.C - 1);  // rows past the chunk read a valid row and are zeroed later
  const int prow = b * a.TP + key;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float* kr = a.y + tile_off_f32(prow, (kHQ + g) * kD + c * 16 + h * 8, kQKV);
    r.k[2 * h] = *reinterpret_cast<const float4*>(kr);
    r.k[2 * h + 1] = *reinterpret_cast<const float4*>(kr + 256);
    r.v[h] = *reinterpret_cast<const uint4*>(a.qvb + tile_off(prow, (kHQ + g) * kD + c * 16 + h * 8, kQVB));
  }
  r.ss = c < 8 ? a.ss_q[(size_t)prow * kQkvTiles + (kHQ + g) * 8 + c] : 0.f;
}

__device__ __forceinline__ void suffix_store(const SufRaw& r, uint32_t vis, int j, uint16_t* sK, uint16_t* sV) {
  const int c = threadIdx.x & 15;
  const bool ok = (vis >> j) & 1u;
  const float t = group16_sum(r.ss);  // the 16 threads of key j form one DPP row
  const float rn = 1.0f / sqrtf(t * (1.0f / kD) + kEps);
  const float kv[16] = {r.k[0].x, r.k[0].y, r.k[0].z, r.k[0].w, r.k[1].x, r.k[1].y, r.k[1].z, r.k[1].w,
                        r.k[2].x, r.k[2].y, r.k[2].z, r.k[2].w, r.k[3].x, r.k[3].y, r.k[3].z, r.k[3].w};
  uint32_t kp[8];
#pragma unroll
  for (int e2 = 0; e2 < 8; ++e2) kp[e2] = ok ? pack2(kv[2 * e2] * rn, kv[2 * e2 + 1] * rn) : 0u;
  *reinterpret_cast<uint4*>(sK + j * KLD + c * 16) = make_uint4(kp[0], kp[1], kp[2], kp[3]);
  *reinterpret_cast<uint4*>(sK + j * KLD + c * 16 + 8) = make_uint4(kp[4], kp[5], kp[6], kp[7]);
  *reinterpret_cast<uint4*>(sV + j * VLD + c * 16) = keep_or_zero(ok, r.v[0]);
  *reinterpret_cast<uint4*>(sV + j * VLD + c * 16 + 8) = keep_or_zero(ok, r.v[1]);
}

// K / V rows (bf16, from global) of one 32-key block: thread t of NTHR owns
// 16-byte chunks t, t + NTHR, ... of the 32 x 32 chunk grid.  Rows are read
// whether visible or not (rows past the split's end read its last row);
// invisible rows are replaced by zeros when staged, so their contents never
// reach the math.
template <int NTHR>
struct KVRegs {
  uint4 k[1024 / NTHR], v[1024 / NTHR];
};

template <int NTHR>
__device__ __forceinline__ void kv_load(const uint16_t* Kb, const uint16_t* Vb, int kb0, int key_hi,
                                        KVRegs<NTHR>& r) {
#pragma unroll
  for (int h = 0; h < 1024 / NTHR; ++h) {
    const int c = threadIdx.x + h * NTHR;
    const int j = c >> 5, ch = c & 31;
    const size_t row = (size_t)min(kb0 + j, key_hi - 1);
    r.k[h] = *reinterpret_cast<const uint4*>(Kb + row * kD + ch * 8);
    r.v[h] = *reinterpret_cast<const uint4*>(Vb + row * kD + ch * 8);
  }
}

template <int NTHR>
__device__ __forceinline__ void kv_store(const KVRegs<NTHR>& r, uint32_t vis, uint16_t* sK, uint16_t* sV) {
#pragma unroll
  for (int h = 0; h < 1024 / NTHR; ++h) {
    const int c = threadIdx.x + h * NTHR;
    const int j = c >> 5, ch = c & 31;
    const bool ok = (vis >> j) & 1u;
    *reinterpret_cast<uint4*>(sK + j * KLD + ch * 8) = keep_or_zero(ok, r.k[h]);
    *reinterpret_cast<uint4*>(sV + j * VLD + ch * 8) = keep_or_zero(ok, r.v[h]);
  }
}

// V^T operand of O^T = V^T P^T for dims 16t .. 16t+15 of a block staged
// row-major: lane (i, q) gets V[key][16t + i] for keys 4q .. 4q+3 (elements
// 0..3) and 16+4q .. 16+4q+3 (elements 4..7), the key order of the P^T
// fragment.  In the transpose read, lane k of each 16-lane group names the
// 4-element chunk V[key0 + k/4][16t + 4(k%4) ..], and lane i receives
// element i%4 of the chunks named by lanes i/4 + 4e, e = 0..3.
__device__ __forceinline__ bf16x8 v_frag(const uint16_t* sV, int t, int lane) {
  const int k = lane & 15, q = lane >> 4;
  const uint16_t* p0 = sV + (4 * q + (k >> 2)) * VLD + t * 16 + 4 * (k & 3);
  const uint16_t* p1 = p0 + 16 * VLD;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(p0));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(p1));
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = lo[e];
    r[4 + e] = hi[e];
  }
  return r;
}

// Work-groups are dealt to the 8 XCDs of the chip in turn (work-group w to
// XCD (w + r) mod 8, with an offset r that the dispatches before set), and
// each XCD has its own L2.  Work item lists ordered by (request, KV head) are
// therefore split into 8 contiguous chunks, chunk x served by the
// work-groups w = x (mod 8), which share an XCD, so the splits (and merge units) of one request / KV
// head share one or two L2s: its queries are fetched into few L2s and its
// partials merged where they were written.  Placement changes only where data
// is cached, never the results.  Returns the work item of this work-group, or
// -1 for a spare one (grid = 8 * ceil(items / 8)).
__device__ __forceinline__ int xcd_chunked(int wg, int grid, int items) {
  const int per = grid >> 3;
  const int item = (wg & 7) * per + (wg >> 3);
  return item < items ? item : -1;
}

// Merge of the split partials of one unit: 16 stacked rows (row tile mt) x
// 16 dims (dim tile t) of request / KV head bg.  One wave: lane (lr, lq) owns
// row lr and dims 16t + 4lq .. +3.  All loads of a batch of splits are in
// flight together (each instruction reads 512 contiguous bytes); inside a
// batch the row maximum is taken first, so every split costs one exp2 and one
// multiply-add per output, in split order.  Batches after the first (prefixes
// longer than CB splits) rescale what came before.
template <int CB>  // splits per batch of loads
__device__ __forceinline__ void combine_unit(const AttnArgs& a, uint16_t* ctx, int bg, int mt, int t, int lane) {
  const int lr = lane & 15, lq = lane >> 4;
  const int TT = a.TP >> 4, MT = 2 * TT;
  const int g = bg % kHK, b = bg / kHK;
  const int nsplit = a.S + a.NS;
  const int row = mt * 16 + lr;
  const int hh = mt / TT, i = (mt - hh * TT) * 16 + lr;
  const size_t ml0 = (size_t)bg * nsplit * a.R16 + row;
  const size_t o0 = ((size_t)bg * nsplit * MT + mt) * (16 * kD) + t * 256 + (lr * 4 + lq) * 4;
  if (i >= a.C) return;  // padded row: nothing was written for it
  float M = kNegBig, L = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nsplit; s0 += CB) {
    float2 ml[CB];
    uint2 ov[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int s = min(s0 + u, nsplit - 1);  // past the end: re-read the last split, skipped below
      ml[u] = *reinterpret_cast<const float2*>(a.part_ml + (ml0 + (size_t)s * a.R16) * 2);
      ov[u] = *reinterpret_cast<const uint2*>(a.part_o + o0 + (size_t)s * MT * (16 * kD));
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < CB; ++u)
      if (s0 + u < nsplit && ml[u].y > 0.f) Mb = fmaxf(Mb, ml[u].x);
    const float so = exp2f(M - Mb);  // 0 before the first visible split, 1 if the max held
    L *= so;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= so;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float w = (s0 + u < nsplit && ml[u].y > 0.f) ? ml[u].y * exp2f(ml[u].x - Mb) : 0.f;
      L += w;
      acc[0] += w * bf2f((uint16_t)(ov[u].x & 0xffffu));
      acc[1] += w * bf2f((uint16_t)(ov[u].x >> 16));
      acc[2] += w * bf2f((uint16_t)(ov[u].y & 0xffffu));
      acc[3] += w * bf2f((uint16_t)(ov[u].y >> 16));
    }
    M = Mb;
  }
  const float inv = 1.0f / L;
  const int col = (kGroup * g + hh) * kD + t * 16 + 4 * lq;
  uint16_t* dst = a.ctx_tiled ? ctx + tile_off(b * a.TP + i, col & ~7, kHQ * kD) + (col & 7)
                              : ctx + (size_t)(b * a.C + i) * kHQ * kD + col;
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(acc[0] * inv, acc[1] * inv), pack2(acc[2] * inv, acc[3] * inv));
}

// The same merge with 8 dims per lane (two 4-dim chunks of the partial
// layout: one 16-byte load per split): lanes 0-31 take dim tile 2 tp, lanes
// 32-63 dim tile 2 tp + 1; lane (lr, hq) owns row lr and dims 16 t + 8 hq ..
// +7.  Every output goes through exactly combine_unit's operations, so the
// two forms give the same bits; this one runs for batches (half the waves,
// twice the bytes per load).
template <int CB>
__device__ __forceinline__ void combine_unit8(const AttnArgs& a, uint16_t* ctx, int bg, int mt, int tp, int lane) {
  const int lr = lane & 15, hq = (lane >> 4) & 1, t = 2 * tp + (lane >> 5);
  const int TT = a.TP >> 4, MT = 2 * TT;
  const int g = bg % kHK, b = bg / kHK;
  const int nsplit = a.S + a.NS;
  const int row = mt * 16 + lr;
  const int hh = mt / TT, i = (mt - hh * TT) * 16 + lr;
  const size_t ml0 = (size_t)bg * nsplit * a.R16 + row;
  const size_t o0 = ((size_t)bg * nsplit * MT + mt) * (16 * kD) + t * 256 + (lr * 4 + 2 * hq) * 4;
  if (i >= a.C) return;  // padded row: nothing was written for it
  float M = kNegBig, L = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += CB) {
    float2 ml[CB];
    uint4 ov[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const int s = min(s0 + u, nsplit - 1);  // past the end: re-read the last split, skipped below
      ml[u] = *reinterpret_cast<const float2*>(a.part_ml + (ml0 + (size_t)s * a.R16) * 2);
      ov[u] = *reinterpret_cast<const uint4*>(a.part_o + o0 + (size_t)s * MT * (16 * kD));
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < CB; ++u)
      if (s0 + u < nsplit && ml[u].y > 0.f) Mb = fmaxf(Mb, ml[u].x);
    const float so = exp2f(M - Mb);  // 0 before the first visible split, 1 if the max held
    L *= so;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= so;
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const float w = (s0 + u < nsplit && ml[u].y > 0.f) ? ml[u].y * exp2f(ml[u].x - Mb) : 0.f;
      L += w;
      const uint32_t wd[4] = {ov[u].x, ov[u].y, ov[u].z, ov[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += w * bf2f((uint16_t)(wd[q] & 0xffffu));
        acc[2 * q + 1] += w * bf2f((uint16_t)(wd[q] >> 16));
      }
    }
    M = Mb;
  }
  const float inv = 1.0f / L;
  const int col = (kGroup * g + hh) * kD + t * 16 + 8 * hq;
  uint16_t* dst = a.ctx_tiled ? ctx + tile_off(b * a.TP + i, col, kHQ * kD)
                              : ctx + (size_t)(b * a.C + i) * kHQ * kD + col;
  *reinterpret_cast<uint4*>(dst) = make_uint4(pack2(acc[0] * inv, acc[1] * inv), pack2(acc[2] * inv, acc[3] * inv),
                                              pack2(acc[4] * inv, acc[5] * inv), pack2(acc[6] * inv, acc[7] * inv));
}

// One split of one (request, KV head), for HPW of its query heads (HPW = 1:
// one work-group per query head, 4 waves; 2: both heads, 8 waves): every
// global load of the split (mask, query rows, all K/V blocks or the raw
// suffix rows) is issued up front; the blocks are then staged into LDS
// together and processed without further work-group barriers.  Work items
// run (request, KV head, split, head), so the work-groups that share a
// split's K/V rows sit on one XCD.
template <bool FUSED, int NB, int HPW>
__global__ __launch_bounds__(256 * HPW) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_attn_partial(AttnArgs a) {
  constexpr int NTHR = 256 * HPW;
  constexpr int KPT = 512 / NTHR;  // suffix keys staged per thread
  static_assert(HPW == 1 || HPW == kGroup, "one query head or the whole group per work-group");
  __shared__ __attribute__((aligned(16))) uint16_t sK[NB][KB * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NB][KB * VLD];
  __shared__ uint32_t sMask[NB];

  if constexpr (HPW == 1) {
    if ((int)blockIdx.x >= a.attn_grid) {  // modulation units on the CUs the splits leave idle
      const int nside = gridDim.x - a.attn_grid;
      for (int u = blockIdx.x - a.attn_grid; u < a.side_n * (3 * kH / 16); u += nside) {
        const int j = u / (3 * kH / 16);
        mod_unit(a.side[j], u - j * (3 * kH / 16), a.side_B, reinterpret_cast<float*>(&sK[0][0]));
      }
      return;
    }
  }
  const int nsplit = a.S + a.NS;
  const int per_split = kGroup / HPW;  // work-groups per split
  const int item = xcd_chunked(blockIdx.x, a.attn_grid, a.B * kHK * nsplit * per_split);
  if (item < 0) return;
  const int hsel = item % per_split;  // first query head of this work-group within the group
  const int split = (item / per_split) % nsplit;
  const int bg = item / per_split / nsplit;
  const int g = bg % kHK, b = bg / kHK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int TT = a.TP >> 4, MT = 2 * TT;  // token tiles per head, stacked row tiles

  const bool suffix = split >= a.S;
  const int key_lo = suffix ? (split - a.S) * KB : split * a.kps;
  const int key_hi = suffix ? min(a.C, key_lo + KB) : min(a.P, key_lo + a.kps);
  const int nkeys = key_hi - key_lo;
  const int nblk = (nkeys + KB - 1) / KB;  // <= NB
  const size_t kv_rows = suffix ? (size_t)a.C : (size_t)a.P;
  const uint16_t* Kb = (suffix ? a.ks : a.kp) + (size_t)(b * kHK + g) * kv_rows * kD;
  const uint16_t* Vb = (suffix ? a.vs : a.vp) + (size_t)(b * kHK + g) * kv_rows * kD;
  const bool from_global = !(FUSED && suffix);

  // ---- load phase: everything this WG reads from global memory
  const int mt = hsel * TT + wave;  // stacked row tile of this wave
  const bool active = wave < HPW * TT;
  const int row = mt * 16 + lr;            // stacked row
  const int hh = active ? mt / TT : 0;     // head within the group
  const int qi = (mt - hh * TT) * 16 + lr; // token
  const bool qok = active && qi < a.C;
  KVRegs<NTHR> kv[NB];
  SufRaw sr[KPT];
  float4 qss[2];
  bf16x8 qf[8];
  // the key's mask byte: loaded first, tested only once every load is in
  // flight (testing it at once would hold the K/V loads behind its latency).
  // The load is unconditional (threads without a prefix key read a byte of
  // the queries and ignore it): a conditional one leaves a copy of its
  // result at the branch's end that waits for it just the same.
  const bool mkey = threadIdx.x < NB * KB && threadIdx.x < nkeys;
  const uint8_t* mp = (mkey && !suffix) ? a.mask + (size_t)b * a.P + key_lo + threadIdx.x
                                        : reinterpret_cast<const uint8_t*>(FUSED ? a.qvb : a.q);
  const int mraw = *mp;
  if (from_global) {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
      if (bi < nblk) kv_load(Kb, Vb, key_lo + bi * KB, key_hi, kv[bi]);
  } else {
#pragma unroll
    for (int i = 0; i < KPT; ++i) suffix_load(a, b, g, key_lo, (threadIdx.x >> 4) + i * (NTHR / 16), sr[i]);
  }
  if (FUSED) {
    q_load(a, b * a.TP + min(qi, a.C - 1), kGroup * g + hh, lq, qf, qss);
  } else {
    const uint16_t* qp = a.q + ((size_t)(b * a.C + min(qi, a.C - 1)) * kHQ + (kGroup * g + hh)) * kD + lq * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = load_bf16x8(qp + ks * 32);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- compute phase
  int mr = mraw;
  asm volatile("" : "+v"(mr));  // the byte stays live on both split kinds (its register is not reused early)
  const int mvis = mkey && (suffix || mr != 0);
  if (wave < (NB * KB) / 64) {  // visibility words: bit j of word bi = key bi * 32 + j
    const uint64_t bal = __ballot(mvis);
    if (lane == 0) sMask[2 * wave] = (uint32_t)bal;
    if (lane == 0 && 2 * wave + 1 < NB) sMask[2 * wave + 1] = (uint32_t)(bal >> 32);
  }
  __syncthreads();
  // stage every block (zero rows for invisible keys)
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) {
    if (bi >= nblk) break;
    const uint32_t vis = sMask[bi];
    if (vis == 0u) continue;
    if (from_global)
      kv_store(kv[bi], vis, sK[bi], sV[bi]);
    else if (bi == 0) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) suffix_store(sr[i], vis, (threadIdx.x >> 4) + i * (NTHR / 16), sK[0], sV[0]);
    }
  }
  if (!qok) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = zero_bf16x8();
  }
  __syncthreads();
  if (active) {

  // lane (lr, lq) owns stacked row mt*16 + lr; o[t][e] = O[row][16t + 4lq + e]
  f32x4 o[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) o[t] = zero_f32x4();
  float mrun = kNegBig, lrun = 0.f;
  // log2(e) / sqrt(head_dim), times the query row's 1 / rms in the fused path
  const float sl2 = (1.4426950408889634f / 16.0f) * (FUSED ? q_rnorm(qss) : 1.0f);

#pragma unroll
  for (int bi = 0; bi < NB; ++bi) {
    if (bi >= nblk) break;
    const uint32_t vis = sMask[bi];
    if (vis == 0u) continue;  // uniform across the WG
    const uint16_t* bK = sK[bi];
    // S^T tiles: s0 keys 0..15, s1 keys 16..31; s?[r] = S[row][key 4lq + r (+16)]
    f32x4 s0 = zero_f32x4(), s1 = zero_f32x4();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(bK + lr * KLD + ks * 32 + lq * 8);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(bK + (16 + lr) * KLD + ks * 32 + lq * 8);
      s0 = mfma16(k0, qf[ks], s0);
      s1 = mfma16(k1, qf[ks], s1);
    }
    float x[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = ((vis >> (4 * lq + r)) & 1u) ? s0[r] * sl2 : -INFINITY;
      x[4 + r] = ((vis >> (16 + 4 * lq + r)) & 1u) ? s1[r] * sl2 : -INFINITY;
      mloc = fmaxf(mloc, fmaxf(x[r], x[4 + r]));
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mnew = fmaxf(mrun, mloc);
    const float alpha = exp2f(mrun - mnew);
    mrun = mnew;
    float psum = 0.f;
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = exp2f(x[e] - mnew), p1 = exp2f(x[e + 1] - mnew);
      psum += p0 + p1;
      const uint32_t pk = pack2(p0, p1);
      pf[e] = (short)(pk & 0xffffu);
      pf[e + 1] = (short)(pk >> 16);
    }
    lrun = lrun * alpha + psum;
    const uint16_t* bV = sV[bi];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      o[t] *= alpha;
      o[t] = mfma16(v_frag(bV, t, lane), pf, o[t]);
    }
  }

  // this split's partial row: running max, running sum, output / sum; the
  // outputs of row tile mt as [t][lr][lq][4] (dims 16t + 4lq .. of row lr)
  float l = lrun + __shfl_xor(lrun, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const size_t pidx = (size_t)bg * nsplit + split;
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint16_t* dst = a.part_o + (pidx * MT + mt) * (16 * kD) + (lr * 4 + lq) * 4;
  if (qok) {  // padded query rows write nothing
#pragma unroll
  for (int t = 0; t < 16; ++t)
    *reinterpret_cast<uint2*>(dst + t * 256) = make_uint2(pack2(o[t][0] * inv, o[t][1] * inv),
                                                          pack2(o[t][2] * inv, o[t][3] * inv));
  if (lq == 0) *reinterpret_cast<float2*>(a.part_ml + (pidx * a.R16 + row) * 2) = make_float2(mrun, l);
  }
  }  // active
}

// Separate merge kernel: one wave per (request, KV head, row tile, dim
// tile), placed like the splits (xcd_chunked) so the partials are read from
// the L2 that received them.
template <int CB, bool WIDE>
__global__ __launch_bounds__(64) void k_attn_combine(AttnArgs a, uint16_t* ctx) {
  const int MT = 2 * (a.TP >> 4);
  constexpr int UPM = WIDE ? 8 : 16;  // waves per (request, KV head, row tile)
  const int item = xcd_chunked(blockIdx.x, gridDim.x, a.B * kHK * MT * UPM);
  if (item < 0) return;
  const int t = item % UPM, rest = item / UPM;
  if (WIDE)
    combine_unit8<CB>(a, ctx, rest / MT, rest % MT, t, threadIdx.x);
  else
    combine_unit<CB>(a, ctx, rest / MT, rest % MT, t, threadIdx.x);
}

void attn_config(int B, int C, int P, AttnArgs& a) {
  a.B = B;
  a.C = C;
  a.P = P;
  a.kps = kAttnKps;
  a.S = (P + a.kps - 1) / a.kps;
  a.NS = (C + KB - 1) / KB;
  a.TP = padded_tokens(C);
  a.R16 = 2 * a.TP;
}

template <int HPW>
static void launch_partial_hpw(AttnArgs a, int side_wgs, hipStream_t s) {
  constexpr int NB = kAttnKps / KB;
  static_assert(NB <= kMaxNB && NB * KB == kAttnKps && NB >= 2, "keys per split");
  const int items = a.B * kHK * (a.S + a.NS) * (kGroup / HPW);
  a.attn_grid = 8 * ((items + 7) / 8);
  const dim3 grid(a.attn_grid + side_wgs);
  if (a.y)
    k_attn_partial<true, NB, HPW><<<grid, dim3(256 * HPW), 0, s>>>(a);
  else
    k_attn_partial<false, NB, HPW><<<grid, dim3(256 * HPW), 0, s>>>(a);
}

bool attn_has_idle_cus(const AttnArgs& a) { return a.B * kHK * (a.S + a.NS) * kGroup <= kAttnPairFromWgs; }

hipError_t launch_attn_partial(const AttnArgs& a, hipStream_t s) {
  if (!attn_has_idle_cus(a)) {
    if (a.side_n > 0) {  // no idle CUs to fill: the modulation units in a launch of their own
      ModBatch mb{};
      mb.B = a.side_B;
      mb.n = a.side_n;
      for (int j = 0; j < a.side_n; ++j) mb.job[j] = a.side[j];
      const hipError_t e = launch_mod_multi(mb, s);
      if (e != hipSuccess) return e;
    }
    launch_partial_hpw<kGroup>(a, 0, s);
  } else {
    // two modulation units per extra work-group (one each, or three, measured slower)
    launch_partial_hpw<1>(a, (a.side_n * (3 * kH / 16) + 1) / 2, s);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, uint16_t* ctx, hipStream_t s) {
  // load batches of equal size, at most kCombineMaxBatch splits each: loads
  // past the last split re-read it and are discarded, and each such wasted
  // load measured ~2.5 us per 18-layer step, so the batch fits the count
  const int nsplit = a.S + a.NS;
  const int nbatch = (nsplit + kCombineMaxBatch - 1) / kCombineMaxBatch;
  const int cb = (nsplit + nbatch - 1) / nbatch;
  // batches: 8 dims per lane (16-byte loads, half the waves); one request:
  // 4 dims per lane (more waves in flight for its few rows)
  const bool wide = a.B > 1;
  const dim3 grid(a.B * kHK * (a.R16 / 16) * (wide ? 8 : 16));  // a multiple of 8
  switch (cb) {
#define DMX_CASE(N)                                                  \
  case N:                                                            \
    if (wide)                                                        \
      k_attn_combine<N, true><<<grid, dim3(64), 0, s>>>(a, ctx);     \
    else                                                             \
      k_attn_combine<N, false><<<grid, dim3(64), 0, s>>>(a, ctx);    \
    break;
    DMX_COMBINE_BATCHES(DMX_CASE)
#undef DMX_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, uint16_t* ctx, hipStream_t s) {
  const hipError_t e = launch_attn_partial(a, s);
  return e != hipSuccess ? e : launch_attn_combine(a, ctx, s);
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


// ---------------------------------------------------------------------------
// QK-RMSNorm ((1 + w) weights) + RoPE (pairs j, j + 128) on the raw fp32 QKV
// projection, written out as bf16 q / k / v (fast-stack article §2.2, "QKV 投影
// QK-Norm RoPE 一次完成").  One wave per token; lane l owns elements
// 2l, 2l+1, 128+2l, 129+2l of every head.  Angles are formed and reduced
// modulo 2*pi in double precision before the fp32 sine / cosine.
__global__ __launch_bounds__(256) void k_qknorm_rope(const float* raw, const uint16_t* qn_w,
                                                     const uint16_t* kn_w, const int32_t* pos0,
                                                     float base, int M, int T, int TP, uint16_t* q,
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
  const float* src = raw + (size_t)(b * TP + t) * kQKV;
  // every load of the token first (its 12 q / k heads, 4 v heads, the norm weights)
  float2 los[kHQ + kHK], his[kHQ + kHK];
  float4 xv[kHK];
#pragma unroll
  for (int h = 0; h < kHQ + kHK; ++h) {
    los[h] = *reinterpret_cast<const float2*>(src + h * kD + 2 * lane);
    his[h] = *reinterpret_cast<const float2*>(src + h * kD + 128 + 2 * lane);
  }
#pragma unroll
  for (int hv = 0; hv < kHK; ++hv) xv[hv] = *reinterpret_cast<const float4*>(src + (kHQ + kHK + hv) * kD + 4 * lane);
  float wq[4], wk[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = (e >> 1) * 128 + 2 * lane + (e & 1);
    wq[e] = 1.f + bf2f(qn_w[j]);
    wk[e] = 1.f + bf2f(kn_w[j]);
  }
#pragma unroll
  for (int h = 0; h < kHQ + kHK; ++h) {
    const bool isq = h < kHQ;
    const float* wn = isq ? wq : wk;
    const float2 lo = los[h], hi = his[h];
    const float ss = wave_sum(lo.x * lo.x + lo.y * lo.y + hi.x * hi.x + hi.y * hi.y);
    const float r = 1.0f / sqrtf(ss * (1.0f / kD) + kEps);
    const float a0 = lo.x * r * wn[0], a1 = lo.y * r * wn[1];
    const float c0 = hi.x * r * wn[2], c1 = hi.y * r * wn[3];
    const uint32_t outlo = pack2(a0 * cs[0] - c0 * sn[0], a1 * cs[1] - c1 * sn[1]);
    const uint32_t outhi = pack2(c0 * cs[0] + a0 * sn[0], c1 * cs[1] + a1 * sn[1]);
    uint16_t* dst = isq ? q + ((size_t)m * kHQ + h) * kD
                        : k + (((size_t)b * kHK + (h - kHQ)) * kv_rows + kv_row0 + t) * kD;
    *reinterpret_cast<uint32_t*>(dst + 2 * lane) = outlo;
    *reinterpret_cast<uint32_t*>(dst + 128 + 2 * lane) = outhi;
  }
#pragma unroll
  for (int hv = 0; hv < kHK; ++hv) {
    const float4 x4 = xv[hv];
    uint2 o;
    o.x = pack2(x4.x, x4.y);
    o.y = pack2(x4.z, x4.w);
    *reinterpret_cast<uint2*>(v + (((size_t)b * kHK + hv) * kv_rows + kv_row0 + t) * kD + 4 * lane) = o;
  }
}

hipError_t launch_qknorm_rope(const float* raw, const uint16_t* qn_w, const uint16_t* kn_w,
                              const int32_t* pos0, float base, int B, int T, int TP, uint16_t* q,
                              uint16_t* k, uint16_t* v, int kv_rows, int kv_row0, hipStream_t s) {
  const int M = B * T;
  k_qknorm_rope<<<dim3((M + 3) / 4), dim3(256), 0, s>>>(raw, qn_w, kn_w, pos0, base, M, T, TP, q, k, v,
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
