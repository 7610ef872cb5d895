// Prefix (prefill) attention on 32x32x16 MFMA.  Built with the compiler
// option that keeps MFMA accumulators in VGPRs: the online softmax rescales
// the 128 fp32 accumulators of every lane once per key block, which in AGPRs
// costs a read and a write around every multiply.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <type_traits>
#include <vector>

#include "dmx_device.hpp"
#include "dmx_internal.hpp"
#include "dmx_tiles.hpp"

namespace dmx {

// ---------------------------------------------------------------------------
// Prefix attention of the prefill (OpenDM fast-stack article, §2.3: the LLM
// attention with the prefix-causal mask mapping): query token i of head h
// reads key tokens j <= i that are valid prefix tokens, from KV head h / 2 of
// the layer's cache.
//
// Work item = (KV head g, block of 64 query tokens, split of at most `sb`
// key blocks of 32).  Its work-group of 4 waves holds both query heads of the
// group: wave w takes head 2g + w/2 and query rows 32 (w % 2) .. +31 of the
// block, so the four waves share one K/V stream.  Products run transposed on
// 32x32x16 MFMA: S^T = K Q^T (Q^T in registers), O^T += V^T P^T (P^T never
// leaves registers).  Lane l owns query row l % 32; its 16 logits per block
// are keys 8 (r / 4) + 4 (l / 32) + r % 4.  The online softmax takes two
// blocks (64 keys) per round.
//
// V^T comes from a transposed copy, [4][Tp / 32][256][32] (Tp = tokens
// rounded up to 32: each key block's V^T one contiguous 16 KB run), that
// k_prefix_vt writes with zeros for invisible keys: an MFMA operand needs its
// 8 keys of one dimension contiguous.  K rows and V^T rows
// are copied from HBM straight into a ring of LDS stages (global_load_lds,
// 16 B per lane, one pair of blocks ahead); every read of a stage is then a
// plain LDS load that the compiler can tell apart from the stages being
// filled.  Rows are stored unpadded with their 16-byte chunks XOR-swizzled
// (K by key, V^T by dimension), so the fragment reads hit distinct banks.
// Invisible keys' logits are masked by selection and their values are exact
// zeros, so whatever the cache holds there cannot reach an output.
//
// Items are ordered by query block, longest key ranges first.  A query
// block whose keys span several splits gets normalised partial outputs and
// (max, sum) per split, merged by k_prefix_attn_merge; a single split writes
// the context directly.
namespace {
constexpr float kNegBig = -1e30f;
constexpr int kPaKB = 32;        // keys per block
constexpr int kPaMaxSplit = 64;  // key blocks per split (upper bound)
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// K: 16-byte chunk c (of 32) of key row j sits at chunk c ^ swz_k(j);
// V^T: chunk c (of 4, 8 keys each) of dimension row d at chunk c ^ swz_v(d)
__device__ __forceinline__ int swz_k(int j) { return j & 15; }
__device__ __forceinline__ int swz_v(int d) { return (d >> 2) & 3; }

// Scheduling of a run of N LDS fragment reads each feeding one MFMA, in
// program order: kAhead reads, then MFMA / read pairs, then the last kAhead
// MFMAs, so that reads stay in flight under the MFMAs instead of each
// waiting for its own.
// With LEAD false the first kAhead reads were issued earlier, in another
// scheduling region.
constexpr int kAhead = 4;
constexpr float kLazyLog2 = 8.0f;  // how far a logit may sit above the softmax reference (log2 units)
template <int N, bool LEAD = true>
__device__ __forceinline__ void pipeline_reads() {
#pragma unroll
  for (int i = 0; i < kAhead; ++i)
    if (LEAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
#pragma unroll
  for (int i = 0; i < N - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
#pragma unroll
  for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// query block qb, split index and key-block range of work item `item`
// (items ordered by query block, longest first); false past the last item
struct PaItem {
  int qb, split, ns, first, kb_lo, kb_hi;
};
__host__ __device__ __forceinline__ bool pa_item(int item, int T, int sb, PaItem& it) {
  const int nqb = (T + 63) / 64, nkb_all = (T + kPaKB - 1) / kPaKB;
  int first = 0;
  for (int qb = nqb - 1; qb >= 0; --qb) {
    const int nkb = min(nkb_all, 2 * qb + 2);
    const int ns = (nkb + sb - 1) / sb;
    if (item < first + ns) {
      it.qb = qb;
      it.split = item - first;
      it.ns = ns;
      it.first = first;
      it.kb_lo = it.split * sb;
      it.kb_hi = min(it.kb_lo + sb, nkb);
      return true;
    }
    first += ns;
  }
  return false;
}
}  // namespace

int prefix_attn_items(int T, int sb) {
  const int nqb = (T + 63) / 64, nkb_all = (T + kPaKB - 1) / kPaKB;
  int n = 0;
  for (int qb = 0; qb < nqb; ++qb) n += (min(nkb_all, 2 * qb + 2) + sb - 1) / sb;
  return n;
}

// ctx element offset of (token, column col .. col+3) of the context
template <bool CTX_TILED>
__device__ __forceinline__ size_t ctx_off(int row, int col) {
  return CTX_TILED ? tile_off(row, col & ~7, kHQ * kD) + (col & 7) : (size_t)row * kHQ * kD + col;
}

// vt[g][kb][d][.] = v[g][32 kb + j][d] for valid keys 32 kb + j < T, else 0.
// Inside each block of 32 keys, 16-byte chunk c = 2m + h holds keys 16m + 4h
// + e and 16m + 8 + 4h + e (e < 4): the 8 keys one lane of the P^T operand
// holds, so one 16-byte read gives the matching V^T operand.  One work-group
// per (block of 32 keys, KV head), staged through LDS.
__global__ __launch_bounds__(256) void k_prefix_vt(const uint16_t* v, const uint8_t* valid, int T, int kv_rows,
                                                  int Tp, uint16_t* vt) {
  __shared__ uint16_t tile[kPaKB][kD + 2];
  const int kb = blockIdx.x, g = blockIdx.y;
  {
    const int j = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 32;  // key row, 32 dims
    const int key = kb * kPaKB + j;
    const bool ok = key < T && valid[key] != 0;
    const uint16_t* src = v + ((size_t)g * kv_rows + min(key, T - 1)) * kD + c0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 raw = ok ? *reinterpret_cast<const uint4*>(src + c * 8) : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tile[j][c0 + c * 8 + 2 * e] = (uint16_t)(w4[e] & 0xffffu);
        tile[j][c0 + c * 8 + 2 * e + 1] = (uint16_t)(w4[e] >> 16);
      }
    }
  }
  __syncthreads();
  const int d = threadIdx.x;  // one dimension row: the block's 32 keys, 64 bytes
  uint16_t* dst = vt + (((size_t)g * (Tp / kPaKB) + kb) * kD + d) * kPaKB;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int k0 = 16 * (c >> 1) + 4 * (c & 1);  // keys k0 .. k0+3, then k0+8 .. k0+11
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ka = k0 + (e >> 1) * 8 + 2 * (e & 1);
      w4[e] = (uint32_t)tile[ka][d] | ((uint32_t)tile[ka + 1][d] << 16);
    }
    *reinterpret_cast<uint4*>(dst + c * 8) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

template <bool CTX_TILED>
__global__ __launch_bounds__(256) void k_prefix_attn(const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                                                    const uint8_t* valid, int T, int kv_rows, int Tp, int sb,
                                                    int items, uint16_t* ctx, uint16_t* part_o, float* part_ml) {
  constexpr int STAGES = 4;  // two pairs of blocks: one being read, one loading
  constexpr int PIECES = 4;  // 1 KB pieces of K (and of V^T) each wave copies per block
  // One array per stage, each holding a block's K rows and V^T rows, and
  // the stage of every copy and read known at compile time: the compiler
  // then sees that the stage being read is not one being filled (it tracks
  // copies into LDS per array) and waits only where the code says so.
  __shared__ __attribute__((aligned(16))) uint16_t sKV0[2][kPaKB * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sKV1[2][kPaKB * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sKV2[2][kPaKB * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sKV3[2][kPaKB * kD];
  __shared__ uint32_t sVis[kPaMaxSplit + STAGES];
  auto stage = [&](auto ST) -> uint16_t(*)[kPaKB * kD] {
    constexpr int S = decltype(ST)::value;
    if constexpr (S == 0) return sKV0;
    else if constexpr (S == 1) return sKV1;
    else if constexpr (S == 2) return sKV2;
    else return sKV3;
  };
  // the wave index is uniform: kept in a scalar register, so that the copies'
  // LDS destinations and sources need no per-lane arithmetic
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x % kHK, item = blockIdx.x / kHK;
  PaItem it;
  if (!pa_item(item, T, sb, it)) return;  // uniform per work-group
  const int nblk = it.kb_hi - it.kb_lo;
  // blocks run in groups of STAGES with no branch between them (a branch in
  // the loop makes the compiler wait for every copy in flight); the padding
  // blocks at the end have no visible key and add exactly nothing
  const int npad = (nblk + STAGES - 1) / STAGES * STAGES;
  const int hq = g * kGroup + (wave >> 1);
  const int h = lane >> 5;
  const int row = it.qb * 64 + (wave & 1) * 32 + (lane & 31);  // this lane's query token

  // Q^T operand: lane l holds dims 16 s + 8 h .. +7 of its row, s < 16
  bf16x8 qf[16];
  const uint16_t* qp = q + ((size_t)min(row, T - 1) * kHQ + hq) * kD + 8 * h;
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) qf[s2] = load_bf16x8(qp + 16 * s2);
  // visibility of the 32 keys of every block of the split (none in the
  // padding blocks)
  for (int i = wave; i < npad; i += 4) {
    const int j = (it.kb_lo + i) * kPaKB + lane;
    const bool ok = i < nblk && lane < kPaKB && j < T && valid[j] != 0;
    const uint64_t b = __ballot(ok);
    if (lane == 0) sVis[i] = (uint32_t)b;
  }
  // this wave's copy sources: the split's K rows and V^T rows from uniform
  // bases, plus per-lane 32-bit element offsets (a key past the tokens reads
  // the last token's row; its logit is masked)
  const uint16_t* kbase = k + ((size_t)g * kv_rows + (size_t)it.kb_lo * kPaKB) * kD;
  const uint16_t* vbase = vt + ((size_t)g * (Tp / kPaKB) + it.kb_lo) * kD * kPaKB;
  int krow[PIECES];
  uint32_t kcol[PIECES], vofs[PIECES];
#pragma unroll
  for (int d = 0; d < PIECES; ++d) {
    const int piece = wave * PIECES + d;
    const int j = piece * 2 + (lane >> 5);  // K: key row of the block
    krow[d] = j;
    kcol[d] = ((lane & 31) ^ swz_k(j)) * 8;
    const int dv = piece * 16 + (lane >> 2);  // V^T: dimension row
    vofs[d] = dv * kPaKB + ((lane & 3) ^ swz_v(dv)) * 8;
  }
  const int last_key_row = T - 1 - it.kb_lo * kPaKB;  // rows past it are clamped
  wait_vmcnt<0>();
  // consume the Q registers here: otherwise their loads may be scheduled past
  // the wait above and the first MFMA of every block would wait for all the
  // copies in flight
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) __asm__ volatile("" ::"v"(qf[s2]));
  __syncthreads();

  // block i of the split into stage ST (past the end: the last block again,
  // into a stage that is never read, so every wave issues PIECES * 2 copies
  // per call and the counter arithmetic stays uniform)
  auto issue = [&](auto ST, int i) {
    uint16_t(*b)[kPaKB * kD] = stage(ST);
    const int ib = min(i, nblk - 1);
    const uint16_t* vblk = vbase + (size_t)ib * kD * kPaKB;
#pragma unroll
    for (int d = 0; d < PIECES; ++d) {
      const int piece = wave * PIECES + d;
      const uint32_t r = min(ib * kPaKB + krow[d], last_key_row);  // rows past the tokens: the last one
      lds_copy16(kbase + (r * kD + kcol[d]), &b[0][piece * 512]);
      lds_copy16(vblk + vofs[d], &b[1][piece * 512]);
    }
  };
  issue(std::integral_constant<int, 0>{}, 0);
  issue(std::integral_constant<int, 1>{}, 1);

  f32x16 o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float mrun = kNegBig, lrun = 0.f;
  const float sl2 = 1.4426950408889634f / 16.0f;  // log2(e) / sqrt(head_dim)

  // LDS element offsets of this lane's fragment reads inside a stage.  K:
  // chunk 2 s2 + h of key row j sits at chunk 16 (s2 / 8) + ((2 (s2 % 8) + h)
  // ^ swz_k(j)) (the swizzle is below 16), so eight offsets serve all 16
  // steps.  V^T: dimension row 32 t + l % 32 has swz_v = (l % 32 / 4) % 4 for
  // every t, so two offsets (m = 0, 1) serve all 8 dimension tiles.
  // Byte offsets; each round re-reads them through an empty asm statement,
  // so the compiler forms every address as offset + immediate at its read
  // instead of keeping one hoisted address per read live across the loop.
  int koff[8], voff[2];
  {
    const int j = lane & 31;
#pragma unroll
    for (int lo = 0; lo < 8; ++lo) koff[lo] = 2 * (j * kD + ((2 * lo + h) ^ swz_k(j)) * 8);
#pragma unroll
    for (int m = 0; m < 2; ++m) voff[m] = 2 * (j * kPaKB + ((2 * m + h) ^ swz_v(j)) * 8);
  }

  // Blocks ib and ib + 1, held in stages SA = ib % STAGES and SB = SA + 1,
  // in one softmax round of 64 keys: one maximum, one rescale of the
  // accumulators and one barrier per pair.  The pair's copies are the only
  // ones in flight when the round starts; the next pair goes into the
  // stages the previous round read (free once every wave is past the
  // barrier), so one pair is always loading under the current one.
  auto pair = [&](auto SA, auto SB, int ib) {
    constexpr int A = decltype(SA)::value, B = decltype(SB)::value;
    wait_vmcnt<0>();  // this wave's copies of blocks ib, ib + 1 landed
    lds_barrier();    // everyone's have; the previous pair's stages are free
    issue(std::integral_constant<int, (A + 2) % STAGES>{}, ib + 2);
    issue(std::integral_constant<int, (B + 2) % STAGES>{}, ib + 3);
    __builtin_amdgcn_sched_barrier(0);  // the copies go out before the round's reads
    const char* bK[2] = {reinterpret_cast<const char*>(stage(SA)[0]), reinterpret_cast<const char*>(stage(SB)[0])};
    const char* bV[2] = {reinterpret_cast<const char*>(stage(SA)[1]), reinterpret_cast<const char*>(stage(SB)[1])};
    __asm__ volatile("" : "+v"(koff[0]), "+v"(koff[1]), "+v"(koff[2]), "+v"(koff[3]), "+v"(koff[4]), "+v"(koff[5]),
                     "+v"(koff[6]), "+v"(koff[7]), "+v"(voff[0]), "+v"(voff[1]));

    f32x16 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[u][r] = 0.f;
    {
      // K fragment (s2, u) at byte koff[s2 % 8] + 256 (s2 / 8); the two blocks'
      // chains alternate, and each read is issued kAhead MFMAs early
      bf16x8 kf[32];
#pragma unroll
      for (int i = 0; i < 32; ++i)
        kf[i] = *reinterpret_cast<const bf16x8*>(bK[i & 1] + koff[(i >> 1) & 7] + 256 * (i >> 4));
#pragma unroll
      for (int i = 0; i < 32; ++i) sacc[i & 1] = mfma32(kf[i], qf[i >> 1], sacc[i & 1]);
      pipeline_reads<32>();
    }
    // key `key` of block u is read when its bit is set in the block's
    // visibility and key <= row - kb0 (causal); the logit of any other key is
    // replaced, bit for bit, by -inf (a select by bit mask: whatever the
    // cache holds there, NaN included, cannot pass)
    float x[2][16];
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int lim = row - (it.kb_lo + ib + u) * kPaKB;
      const uint32_t causal = lim >= kPaKB - 1 ? 0xffffffffu : lim < 0 ? 0u : (2u << lim) - 1u;
      const uint32_t keep = sVis[ib + u] & causal;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * h + (r & 3);
        const uint32_t sel = (uint32_t)((int32_t)(keep << (31 - key)) >> 31);  // all ones when kept
        x[u][r] = __uint_as_float((__float_as_uint(sacc[u][r]) & sel) | (__float_as_uint(-INFINITY) & ~sel));
        mloc = fmaxf(mloc, x[u][r]);
      }
    }
    // Maxima in raw logit units; the scale log2(e) / 16 enters each exponent
    // through one fused multiply-add.  mrun is the reference the exponents
    // are taken against, not always the running maximum: it moves (and the
    // accumulators are rescaled) only in rounds where some row of the wave
    // saw a logit more than kLazyLog2 above it (in log2 units), so every
    // exponent stays below 2^kLazyLog2 and most rounds skip the 128
    // multiplies.  Sums and outputs share the reference, so o / l and the
    // merge's weights are unchanged by where it sits.
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    // the round's first V fragments go out before the branch
    bf16x8 vf[32];
#pragma unroll
    for (int i = 0; i < kAhead; ++i)
      vf[i] = *reinterpret_cast<const bf16x8*>(bV[i >> 4] + voff[(i >> 3) & 1] + 2048 * (i & 7));
    if (__builtin_amdgcn_ballot_w64((mloc - mrun) * sl2 > kLazyLog2) != 0) {
      const float mnew = fmaxf(mrun, mloc);
      const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * sl2);  // exp2(-inf) = 0 in hardware
      mrun = mnew;
      lrun *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
    }
    const float nm = -mrun * sl2;
    bf16x8 pf[2][2];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(x[u][r], sl2, nm));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(x[u][r + 1], sl2, nm));
        psum += p0 + p1;
        const uint32_t pk = pack2(p0, p1);
        pf[u][r >> 3][r & 7] = (short)(pk & 0xffffu);
        pf[u][r >> 3][(r & 7) + 1] = (short)(pk >> 16);
      }
    lrun += psum;
    // V^T operand of dims 32 t + (l % 32): chunk 2m + h of the dimension's
    // row holds keys 16 m + 4 h + e and 16 m + 8 + 4 h + e (e < 4), the key
    // order of P^T's elements above
    // (dimension row 32 t + l % 32 sits at byte voff[m] + 2048 t); fragment i is
    // (u, m) = (i / 16, i / 8 % 2) of dims tile t = i % 8, so consecutive
    // MFMAs update different accumulators
    {
#pragma unroll
      for (int i = kAhead; i < 32; ++i)
        vf[i] = *reinterpret_cast<const bf16x8*>(bV[i >> 4] + voff[(i >> 3) & 1] + 2048 * (i & 7));
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i & 7] = mfma32(vf[i], pf[i >> 4][(i >> 3) & 1], o[i & 7]);
      pipeline_reads<32, false>();
    }
  };
#pragma unroll 1
  for (int ib = 0; ib < npad; ib += STAGES) {
    pair(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, ib);
    pair(std::integral_constant<int, 2>{}, std::integral_constant<int, 3>{}, ib + 2);
  }
  wait_vmcnt<0>();  // the trailing copies (never read) are done before the work-group ends

  const float l = lrun + __shfl_xor(lrun, 32, 64);
  const float inv = l > 0.f ? 1.0f / l : 0.f;  // no visible key: zero output
  if (it.ns == 1) {
    if (row >= T) return;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int col = hq * kD + 32 * t + 8 * q4 + 4 * h;
        *reinterpret_cast<uint2*>(ctx + ctx_off<CTX_TILED>(row, col)) =
            make_uint2(pack2(o[t][4 * q4] * inv, o[t][4 * q4 + 1] * inv),
                       pack2(o[t][4 * q4 + 2] * inv, o[t][4 * q4 + 3] * inv));
      }
    return;
  }
  // partial of this split: [g][item][wave][32 rows][256] bf16 normalised, and (max, sum), the max scaled to log2 units as the merge expects
  const size_t pidx = ((size_t)g * items + item) * 4 + wave;
  uint16_t* po = part_o + (pidx * 32 + (lane & 31)) * kD;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * t + 8 * q4 + 4 * h;
      *reinterpret_cast<uint2*>(po + d) = make_uint2(pack2(o[t][4 * q4] * inv, o[t][4 * q4 + 1] * inv),
                                                     pack2(o[t][4 * q4 + 2] * inv, o[t][4 * q4 + 3] * inv));
    }
  if (lane < 32) *reinterpret_cast<float2*>(part_ml + (pidx * 32 + lane) * 2) = make_float2(mrun * sl2, l);
}

// Merge of the splits of one (KV head, query block, wave tile): for each of
// the tile's 32 rows, M = max m_s, w_s = l_s 2^(m_s - M), out = sum_s w_s o_s /
// sum_s w_s (zero when no split saw a visible key), in split order.  One
// work-group of 256 threads per (g, query block, tile); 8 threads per row,
// 32 dims each.  Query blocks with a single split return at once.
constexpr int kMergeBatch = 4;
// splits of one query block at most: 4096 tokens, 12-block splits
constexpr int kMergeMaxSplits = 12;
static_assert(kMergeMaxSplits * kPrefixAttnSplits[3] * kPaKB >= 4096, "merge bound below the longest query block's splits");
template <bool CTX_TILED>
__global__ __launch_bounds__(256) void k_prefix_attn_merge(int T, int sb, int items, const uint16_t* part_o,
                                                          const float* part_ml, uint16_t* ctx) {
  const int nqb = (T + 63) / 64;
  const int tile = blockIdx.x & 3, g = (blockIdx.x >> 2) % kHK, qb = (blockIdx.x >> 2) / kHK;
  if (qb >= nqb) return;
  // the first item of query block qb
  const int nkb_all = (T + kPaKB - 1) / kPaKB;
  int first = 0;
  for (int b = nqb - 1; b > qb; --b) first += (min(nkb_all, 2 * b + 2) + sb - 1) / sb;
  const int ns = (min(nkb_all, 2 * qb + 2) + sb - 1) / sb;
  if (ns == 1) return;
  const int rr = threadIdx.x >> 3, d0 = (threadIdx.x & 7) * 32;
  const int row = qb * 64 + (tile & 1) * 32 + rr;
  if (row >= T) return;
  const int hq = g * kGroup + (tile >> 1);
  // Every split's (max, sum) and the first batch's outputs are requested
  // before any arithmetic, later batches as a whole: a few dependent loads
  // per thread instead of two passes of one load per split.  The sums run in
  // split order, as before.
  float2 ml[kMergeMaxSplits];
#pragma unroll
  for (int s2 = 0; s2 < kMergeMaxSplits; ++s2)
    if (s2 < ns) {
      const size_t pidx = ((size_t)g * items + first + s2) * 4 + tile;
      ml[s2] = *reinterpret_cast<const float2*>(part_ml + (pidx * 32 + rr) * 2);
    }
  uint4 raw[kMergeBatch][4];
  auto fetch = [&](int s0) {
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b)
      if (s0 + b < ns) {
        const size_t pidx = ((size_t)g * items + first + s0 + b) * 4 + tile;
        const uint16_t* po = part_o + (pidx * 32 + rr) * kD + d0;
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[b][c] = *reinterpret_cast<const uint4*>(po + c * 8);
      }
  };
  fetch(0);
  float M = kNegBig;
#pragma unroll
  for (int s2 = 0; s2 < kMergeMaxSplits; ++s2)
    if (s2 < ns) M = fmaxf(M, ml[s2].x);
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  float L = 0.f;
#pragma unroll
  for (int s0 = 0; s0 < kMergeMaxSplits; s0 += kMergeBatch) {
    if (s0 >= ns) break;
    if (s0 > 0) fetch(s0);
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      if (s0 + b >= ns) break;
      const float w = ml[s0 + b].y * exp2f(ml[s0 + b].x - M);
      L += w;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t wv[4] = {raw[b][c].x, raw[b][c].y, raw[b][c].z, raw[b][c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[c * 8 + 2 * e] += w * bf2f((uint16_t)(wv[e] & 0xffffu));
          acc[c * 8 + 2 * e + 1] += w * bf2f((uint16_t)(wv[e] >> 16));
        }
      }
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int col = hq * kD + d0 + 4 * c;
    *reinterpret_cast<uint2*>(ctx + ctx_off<CTX_TILED>(row, col)) =
        make_uint2(pack2(acc[4 * c] * inv, acc[4 * c + 1] * inv), pack2(acc[4 * c + 2] * inv, acc[4 * c + 3] * inv));
  }
}

// workspace: V^T [4][256][Tp], then the split partials ([4][items][4][32][256]
// bf16 and [4][items][4][32][2] fp32)
static size_t vt_bytes(int T) { return (size_t)kHK * kD * ((T + kPaKB - 1) / kPaKB * kPaKB) * 2; }

size_t prefix_attention_ws_bytes(int T) {
  const int items = prefix_attn_items(T, kPrefixAttnSplits[3]);  // the smallest split: the most items
  return vt_bytes(T) + (size_t)kHK * items * 4 * 32 * (kD * 2 + 2 * sizeof(float));
}

// Compute units of the current device (cached per device id).
static int device_cus() {
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// Split size for T tokens: the candidate whose work items finish first when
// dealt in launch order to whichever CU frees up first (one work-group per
// CU: the LDS ring fills it), an item costing its padded block count plus two
// blocks of fixed work (queries in, outputs out); ties go to the larger split
// (fewer partials to merge).  Host arithmetic only.
static int prefix_attn_split(int T, int cus) {
  int best = kPrefixAttnSplits[0];
  long best_t = -1;
  for (int sb : kPrefixAttnSplits) {
    std::priority_queue<long, std::vector<long>, std::greater<long>> free_at;
    for (int c = 0; c < cus; ++c) free_at.push(0);
    long end = 0;
    const int items = prefix_attn_items(T, sb);
    for (int item = 0; item < items; ++item) {
      PaItem it;
      pa_item(item, T, sb, it);
      const long cost = (it.kb_hi - it.kb_lo + 3) / 4 * 4 + 2;
      for (int g = 0; g < kHK; ++g) {
        const long t = free_at.top() + cost;
        free_at.pop();
        free_at.push(t);
        end = std::max(end, t);
      }
    }
    if (best_t < 0 || end < best_t) {
      best_t = end;
      best = sb;
    }
  }
  return best;
}

// prefix_attn_split, remembered per token count (the entry holds the CU
// count it was computed for; concurrent callers can only store equal values)
static int prefix_attn_split_cached(int T, int cus) {
  static int cache[4097];
  if (T < 1 || T > 4096 || cus >= (1 << 22)) return prefix_attn_split(T, cus);
  const int e = cache[T];
  if (e != 0 && (e >> 8) == cus) return e & 255;
  const int sb = prefix_attn_split(T, cus);
  cache[T] = (cus << 8) | sb;
  return sb;
}

hipError_t launch_prefix_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint8_t* valid,
                                   int T, int kv_rows, uint16_t* ctx, bool ctx_tiled, void* ws, hipStream_t s) {
  const int sb = prefix_attn_split_cached(T, device_cus());
  const int items = prefix_attn_items(T, sb);
  if (((T + kPaKB - 1) / kPaKB + sb - 1) / sb > kMergeMaxSplits) return hipErrorInvalidValue;  // beyond the merge
  const int Tp = (T + kPaKB - 1) / kPaKB * kPaKB;
  unsigned char* w = static_cast<unsigned char*>(ws);
  uint16_t* vt = reinterpret_cast<uint16_t*>(w);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(w + vt_bytes(T));
  float* part_ml = reinterpret_cast<float*>(w + vt_bytes(T) + (size_t)kHK * items * 4 * 32 * kD * 2);
  k_prefix_vt<<<dim3(Tp / kPaKB, kHK), dim3(256), 0, s>>>(v, valid, T, kv_rows, Tp, vt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(kHK * items);
  if (ctx_tiled)
    k_prefix_attn<true><<<grid, dim3(256), 0, s>>>(q, k, vt, valid, T, kv_rows, Tp, sb, items, ctx, part_o,
                                                           part_ml);
  else
    k_prefix_attn<false><<<grid, dim3(256), 0, s>>>(q, k, vt, valid, T, kv_rows, Tp, sb, items, ctx, part_o,
                                                            part_ml);
  e = hipGetLastError();
  if (e != hipSuccess || (T + kPaKB - 1) / kPaKB <= sb) return e;  // every query block in one split
  const dim3 mgrid(4 * kHK * ((T + 63) / 64));
  if (ctx_tiled)
    k_prefix_attn_merge<true><<<mgrid, dim3(256), 0, s>>>(T, sb, items, part_o, part_ml, ctx);
  else
    k_prefix_attn_merge<false><<<mgrid, dim3(256), 0, s>>>(T, sb, items, part_o, part_ml, ctx);
  return hipGetLastError();
}

}  // namespace dmx
