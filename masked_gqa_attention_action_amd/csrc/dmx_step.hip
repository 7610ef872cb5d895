// Persistent denoise-step kernel: the whole action-expert stack of one
// request (batch 1) for one or more denoising steps in a single launch
// (OpenDM DM0.5 fast-stack article, §2.2: one large fused kernel instead of
// many small ops; §3: replayed from a graph per prefix bucket).
//
// Why one kernel.  A layer is a chain of dependent stages (QKV -> attention
// -> O-projection -> GEGLU -> down), and each of its projections streams
// megabytes of weights that depend on nothing.  Separate kernels load each
// stage's weights only after the stage before has finished.  Here every
// work-group keeps its weight slices for the next stage in flight while it
// waits for that stage's inputs, so weight streaming overlaps the chain.
//
// Placement.  256 work-groups, one per CU.  The dispatcher deals work-groups
// to the 8 XCCs in turn: work-group w runs on XCC (w + r) mod 8, with an
// offset r that the dispatches before set, so the 32 work-groups w = x
// (mod 8) always share an XCC, and a hand-off among them (~1 us) is cheaper
// than one that crosses XCCs (2.5 - 3 us).  Below, "XCC x" is that group of
// work-groups.  XCC x owns query head x: it projects q head x and the
// K/V head x / 2 of its group (the two XCCs of a group both compute it), runs
// head x's attention over the prefix and chunk keys, merges the splits and
// multiplies the context by head x's 256 columns of W_o.  The eight heads'
// O-projection partials meet in one cross-XCC reduction; the MLP is split
// the same way (XCC x owns intermediate features 512x .. 512x + 511, whose
// down-projection partial is its share of the second reduction).  Each
// reduction is done redundantly by every XCC for all columns (work-group j
// of an XCC reduces columns 32j .. 32j + 31), so it only waits for the 8
// work-groups that wrote those columns.
//
// Stages of layer l (every work-group passes every stage in order):
//   QKV  j < 24: rotation-pair tile j of [q head x | k head g | v head g],
//        AdaRMS #1 fused (shift tile, row rms), QK-norm weights and RoPE in
//        the epilogue (the attention applies the rows' 1 / rms)
//   ATT  j < nsplit: split j of head x's keys (prefix blocks of 32 keys,
//        then the chunk's own keys), partial output + (max, sum) per row
//   MRG  4 waves per work-group, one (row tile, 16 dims) unit each: merge
//        of the splits into head x's context
//   OP   y_x = ctx_x W_o[:, 256x ..]^T for output columns 32j .. 32j + 31
//   RS1  x1 = x + gate1 (y_0 + ... + y_7) for columns 32j ..; tiled
//        bf16(x1 (1 + scale2)) and row sums of squares for the gate-up
//   GU   gate-up tile (16 gate + 16 up features of XCC x's slice), AdaRMS #2
//        fused, GEGLU
//   DP   y2_x = h_x W_down[:, 512x ..]^T for output columns 32j ..
//   RS2  out = x1 + gate2 (y2_0 + ... + y2_7); the next layer's tiled
//        bf16(out (1 + scale1)) and row sums of squares
// The modulation vectors of layer l + 2 (or of the next step's layers 0
// and 1) are computed by single waves between the OP and RS1 stages of layer
// l: they depend only on the conditioning.
//
// Hand-offs.  Work-group w publishes a monotonic counter prog[w] after each
// stage, once its stores are complete (write-through stores with the sc1
// cache bit, then a full wait).  A fifth wave per work-group does nothing
// but poll the counters of the stage's producers (sc1 loads) and then meets
// the compute waves at a barrier, so their prefetch loads stay in flight
// during the wait.  Every wait is bounded: past the time limit the
// work-group records the stage in an error word and the whole grid exits.
// Data that crosses work-groups is written with sc1 stores and read with
// sc1 loads; counters are relative to the value a work-group reads for
// itself at kernel start (all equal after a completed launch or a reset).
#include "dmx_device.hpp"
#include "dmx_internal.hpp"
#include "dmx_tiles.hpp"

namespace dmx {

namespace {

typedef uint32_t u32;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4s;
typedef __attribute__((address_space(3))) bf16x4s lds_bf16x4s;

constexpr int kThreads = 320;   // 4 compute waves + 1 sync wave
constexpr int kCompute = 256;
constexpr int kAux = 16;        // sc1: coherent at device scope
constexpr int kFlagStride = 32; // counters 128 bytes apart
constexpr int KB = 32;          // keys per attention block
constexpr int KLD = kD + 8;     // K row stride in LDS (bf16)
constexpr int VLD = kD + 16;    // V row stride in LDS (bf16)
constexpr float kNegBig = -1e30f;

// stage indices within a layer
enum { S_QKV = 0, S_ATT, S_MRG, S_OP, S_RS1, S_GU, S_DP, S_RS2, S_NUM };

// A buffer read and written coherently by all CUs of the device.
struct Coh {
  __amdgpu_buffer_rsrc_t r;
  __device__ explicit Coh(const void* p)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000)) {}
  __device__ uint4 ld16(u32 off) const {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  __device__ bf16x8 ldf(u32 off) const {  // an MFMA fragment
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
    return __builtin_bit_cast(bf16x8, v);
  }
  __device__ float4 ld16f(u32 off) const {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
  }
  __device__ uint2 ld8(u32 off) const {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAux);
    return make_uint2(v[0], v[1]);
  }
  __device__ u32 ld4(u32 off) const { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kAux); }
  __device__ float ld4f(u32 off) const { return __uint_as_float(ld4(off)); }
  __device__ void st16(u32 off, uint4 v) const {
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(t, r, off, 0, kAux);
  }
  __device__ void st16f(u32 off, float4 v) const {
    st16(off, make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)));
  }
  __device__ void st8(u32 off, uint2 v) const {
    const u32x2 t = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(t, r, off, 0, kAux);
  }
  __device__ void st4(u32 off, u32 v) const { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kAux); }
  __device__ void st4f(u32 off, float v) const { st4(off, __float_as_uint(v)); }
};

__device__ __forceinline__ void lgkm_wait() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// LDS hand-off between the waves of the work-group that leaves vector memory
// loads in flight (prefetches): LDS writes complete, then the barrier
__device__ __forceinline__ void lds_sync() {
  lgkm_wait();
  lds_barrier();
}

__device__ __forceinline__ uint4 pack8f(const float v[8]) {
  return make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
}
__device__ __forceinline__ void unpack8f(uint4 r, float v[8]) {
  const u32 w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf2f((uint16_t)(w[i] & 0xffffu));
    v[2 * i + 1] = bf2f((uint16_t)(w[i] >> 16));
  }
}
__device__ __forceinline__ float f4c(float4 v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }
__device__ __forceinline__ bf16x8 ldw(const uint16_t* p) {  // weights: read once per launch
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}

// byte offset of the 8-column chunk (row, col) of a tiled bf16 matrix [*][K]
__device__ __forceinline__ u32 tb(int row, int col, int K) { return (u32)tile_off(row, col, K) * 2u; }
// byte offset of the first half of the 8-column chunk of a tiled fp32 matrix
__device__ __forceinline__ u32 tf(int row, int col, int K) { return (u32)tile_off_f32(row, col, K) * 4u; }

}  // namespace

// ---------------------------------------------------------------------------
struct StepSmem {
  union {
    struct {  // attention: K / V blocks of the split
      uint16_t K[kStepMaxNB][KB * KLD];
      uint16_t V[kStepMaxNB][KB * VLD];
    } kv;
    struct {
      uint16_t slab[64 * 512];  // a projection's weight fragments, [fragment][lane][8], 64 KB
      float red[4][80 * 32];    // [wave][row (64 rows + the shift row at 64)][32 columns]
      float tmp[64 * 33];       // transposes of the reductions
    } g;
  } u;
  float xres[64 * 32];   // this work-group's 32 columns of the layer input x (bf16 values)
  float x1k[64 * 32];    // ... of x1 (fp32)
  uint16_t cond[4][kH];  // per wave: the conditioning of its modulation unit (bf16)
  uint16_t shift[kH];    // the AdaRMS shift of the current projection (bf16)
  float rms[64];         // 1 / rms of the rows (AdaRMS)
  double freq[16];       // RoPE frequencies of the tile (revolutions per position)
  float sq[128];         // QKV: half-tile sums of squares
  u32 mask[kStepMaxNB];
  u32 ok;
};

namespace {

// ---- synchronisation --------------------------------------------------------
// hand-off counters and the error word sit at fixed offsets of the workspace
constexpr u32 kProg = StepLayout::prog, kErr = StepLayout::err;
constexpr long long kTimeout = 100000000LL;  // a wait gives up after 1 s (100 MHz wall clock)

struct Sync {
  Coh R;     // the workspace
  u32 base;  // this launch's counter origin
};

// Work-group-wide end of a stage: every compute wave's stores are complete,
// then the sync wave publishes `code`.
__device__ __forceinline__ void stage_end(const Sync& s, u32 code) {
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  if (threadIdx.x == kCompute) s.R.st4(kProg + (u32)blockIdx.x * kFlagStride * 4u, s.base + code);
}

// Wait until the counters of the producers reach `code`: n work-groups,
// producer i = first + i * stride.  Polled by the sync wave; the compute
// waves wait at the barrier with their loads in flight.  Returns false when
// this or another work-group gave up (the caller then exits); ws is the
// workspace base, for the error word's atomic.
__device__ __forceinline__ bool stage_wait(const Sync& s, StepSmem& sm, char* ws, u32 code, int first, int stride,
                                           int n) {
  if (threadIdx.x >= kCompute) {
    const int lane = threadIdx.x - kCompute;
    const u32 target = s.base + code;
    const long long t0 = wall_clock64();
    u32 ok = 1;
    while (true) {
      bool good = true;
      for (int i = lane; i < n; i += 64) {
        const u32 v = s.R.ld4(kProg + (u32)(first + i * stride) * kFlagStride * 4u);
        good = good && (int)(v - target) >= 0;
      }
      const u32 e = s.R.ld4(kErr);
      if (__all(good)) break;
      if (e != 0) {
        ok = 0;
        break;
      }
      if (wall_clock64() - t0 > kTimeout) {  // the first to give up names itself and the stage
        if (lane == 0)
          atomicCAS(reinterpret_cast<u32*>(ws + kErr), 0u, 0x80000000u | ((u32)blockIdx.x << 20) | (code & 0xfffffu));
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) sm.ok = ok;
    __builtin_amdgcn_s_waitcnt(0);
  }
  __builtin_amdgcn_s_barrier();
  return sm.ok != 0;
}

// ---- modulation (one wave, 16 features of one W_mod) ------------------------------
struct ModUnit {
  bf16x8 w[32];
  uint4 c[2];  // this lane's 16 elements of the conditioning
};
__device__ __forceinline__ void mod_zero(ModUnit& u) {
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) u.w[ks] = zero_bf16x8();
  u.c[0] = u.c[1] = make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void mod_fetch(const uint16_t* W, const uint16_t* cond, int tile, int lane, ModUnit& u) {
  const uint16_t* p = W + (size_t)tile * 32 * 512 + lane * 8;
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) u.w[ks] = ldw(p + ks * 512);
  u.c[0] = *reinterpret_cast<const uint4*>(cond + lane * 16);
  u.c[1] = *reinterpret_cast<const uint4*>(cond + lane * 16 + 8);
}
// out[tile * 16 + c] = W[tile * 16 + c] . cond + bias, written at byte offset
// o_out of the workspace: row 0 of the MFMA A operand holds cond (staged in
// this wave's own LDS row), the other 15 rows are zero.  No work-group
// barrier: only this wave touches its LDS row.
__device__ __forceinline__ void mod_finish(const ModUnit& u, StepSmem& sm, const uint16_t* bias, int tile,
                                           const Coh& R, u32 o_out, int wave, int lane) {
  const int lr = lane & 15, lq = lane >> 4;
  uint16_t* cw = sm.cond[wave];
  *reinterpret_cast<uint4*>(cw + lane * 16) = u.c[0];
  *reinterpret_cast<uint4*>(cw + lane * 16 + 8) = u.c[1];
  lgkm_wait();
  f32x4 acc = zero_f32x4();
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) {
    const bf16x8 a = lr == 0 ? *reinterpret_cast<const bf16x8*>(cw + ks * 32 + lq * 8) : zero_bf16x8();
    acc = mfma16(a, u.w[ks], acc);
  }
  if (lq == 0) R.st4f(o_out + (u32)(tile * 16 + lr) * 4u, acc[0] + bf2f(bias[tile * 16 + lr]));
}

// the modulation unit of one wave: 384 per linear layer n (2 norms x 192
// tiles of 16 features), unit u on work-group u % 256, wave u / 256
struct MJob {
  int n, nm, tile;  // n < 0: none
};
__device__ __forceinline__ MJob mod_job(int n, int u) {
  MJob m;
  m.n = u < 384 ? n : -1;
  m.nm = u / 192;
  m.tile = u % 192;
  return m;
}

// ---- projections: weights copied into the LDS slab ahead of use ------------
// A projection of this kernel owns two 16-row weight tiles (n-tiles) of a
// tiled matrix with `kt` 32-column steps per row, over the steps [k0, k0 +
// 4 KSW): wave w copies steps k0 + KSW w .. +KSW of both n-tiles into the
// slab (fragment nt * 4 KSW + (step - k0)) with loads that write LDS
// directly, and later reads exactly those fragments, so only its own
// copies have to have landed (vmcnt), no barrier.
template <int KSW>
__device__ __forceinline__ void slab_fetch(const uint16_t* W, int rt0, int rt1, int kt, int k0, StepSmem& sm,
                                           int wave, int lane) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint16_t* p = W + ((size_t)(nt ? rt1 : rt0) * kt + k0 + wave * KSW) * 512 + lane * 8;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) lds_copy16(p + ks * 512, sm.u.g.slab + (nt * 4 * KSW + wave * KSW + ks) * 512);
  }
}
template <int KSW>
__device__ __forceinline__ bf16x8 slab_frag(const StepSmem& sm, int nt, int ks, int wave, int lane) {
  return *reinterpret_cast<const bf16x8*>(sm.u.g.slab + (nt * 4 * KSW + wave * KSW + ks) * 512 + lane * 8);
}

// AdaRMS-fused projection with K = 1024 (QKV, gate-up): red[wave][r][c] <-
// this wave's partial sums over its 8 steps for the block rows (0 .. 16 MT)
// and for the shift row (row 64).  A (offset oA) is tiled bf16 [TP][1024]
// holding bf16(x (1 + scale)); the shift vector is fp32 [1024] at offset oSh
// of M; sm.rms <- the rows' 1 / rms from the 32 partial sums of squares per
// row at offset oSs (fp32 [TP][32]).
template <int MT>
__device__ __forceinline__ void gemm1024_mod(const Coh& R, u32 oA, const Coh& M, u32 oSh, u32 oSs, int C,
                                             StepSmem& sm, int tid) {
  const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lq = lane >> 4;
  bf16x8 av[8][MT];
  if (tid < kCompute) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) av[ks][mt] = R.ldf(oA + (u32)((mt * 32 + wave * 8 + ks) * 512 + lane * 8) * 2u);
    const float4 hv = M.ld16f(oSh + (u32)tid * 16u);  // shift[4 tid .. 4 tid + 3]
    // row statistics: thread (row r, quarter q) sums 8 of the row's 32 partials
    float4 sp0 = make_float4(0.f, 0.f, 0.f, 0.f), sp1 = sp0;
    const int rr = tid >> 2, qq = tid & 3;
    if (rr < MT * 16 && rr < C) {
      sp0 = R.ld16f(oSs + (u32)(rr * 32 + qq * 8) * 4u);
      sp1 = R.ld16f(oSs + (u32)(rr * 32 + qq * 8 + 4) * 4u);
    }
    wait_vmcnt<0>();  // this wave's weight copies (issued earlier), A and the vectors
    *reinterpret_cast<uint2*>(sm.shift + tid * 4) = make_uint2(pack2(hv.x, hv.y), pack2(hv.z, hv.w));
    float t = ((sp0.x + sp0.y) + (sp0.z + sp0.w)) + ((sp1.x + sp1.y) + (sp1.z + sp1.w));
    t += __shfl_xor(t, 1, 64);
    t += __shfl_xor(t, 2, 64);
    if (qq == 0) sm.rms[rr] = 1.0f / sqrtf(t * (1.0f / kH) + kEps);
  }
  lds_sync();
  if (tid < kCompute) {
    f32x4 acc[MT][2], accs[2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = zero_f32x4();
    accs[0] = accs[1] = zero_f32x4();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 hs = lr == 0 ? *reinterpret_cast<const bf16x8*>(sm.shift + wave * 256 + ks * 32 + lq * 8) : zero_bf16x8();
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const bf16x8 wf = slab_frag<8>(sm, nt, ks, wave, lane);
        accs[nt] = mfma16(hs, wf, accs[nt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = mfma16(av[ks][mt], wf, acc[mt][nt]);
      }
    }
    float* red = sm.u.g.red[wave];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(mt * 16 + lq * 4 + r) * 32 + nt * 16 + lr] = acc[mt][nt][r];
    if (lq == 0) {
      red[64 * 32 + lr] = accs[0][0];
      red[64 * 32 + 16 + lr] = accs[1][0];
    }
  }
  lds_sync();
}

__device__ __forceinline__ float red_sum(const StepSmem& sm, int r, int c) {
  return ((sm.u.g.red[0][r * 32 + c] + sm.u.g.red[1][r * 32 + c]) + sm.u.g.red[2][r * 32 + c]) +
         sm.u.g.red[3][r * 32 + c];
}

// Projection without AdaRMS (O-projection, down partial): K = 4 KSW steps
// of A (offset oA, tiled bf16 [TP][4 KSW * 32]), wave w takes steps KSW w ..
template <int MT, int KSW>
__device__ __forceinline__ void gemm_ksplit(const Coh& R, u32 oA, StepSmem& sm, int tid) {
  if (tid < kCompute) {
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lq = lane >> 4;
    constexpr int kt = 4 * KSW;  // 32-column steps of a row of A
    bf16x8 av[KSW][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < KSW; ++ks) av[ks][mt] = R.ldf(oA + (u32)((mt * kt + wave * KSW + ks) * 512 + lane * 8) * 2u);
    wait_vmcnt<0>();
    f32x4 acc[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = zero_f32x4();
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const bf16x8 wf = slab_frag<KSW>(sm, nt, ks, wave, lane);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = mfma16(av[ks][mt], wf, acc[mt][nt]);
      }
    float* red = sm.u.g.red[wave];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(mt * 16 + lq * 4 + r) * 32 + nt * 16 + lr] = acc[mt][nt][r];
  }
  lds_sync();
}

// the reduced output fragment (rows 16 mt + 4 lq + e, column 16 nt + lr) of
// thread (wave mt, lane) as a float4 over e
__device__ __forceinline__ float4 red_frag(const StepSmem& sm, int mt, int nt, int lane) {
  const int lr = lane & 15, lq = lane >> 4;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = red_sum(sm, mt * 16 + lq * 4 + e, nt * 16 + lr);
  return make_float4(v[0], v[1], v[2], v[3]);
}

// byte offset of the partial-output fragment (row tile mt, column tile nt of
// 64) of lane `lane` from XCC h in a [8][4][64][64][4] fp32 partial buffer
__device__ __forceinline__ u32 part_frag(int h, int mt, int nt, int lane) {
  return (u32)((((h * 4 + mt) * 64 + nt) * 64 + lane) * 4) * 4u;
}

// ---- attention -------------------------------------------------------------------
struct KVPre {  // one split's prefix K / V rows (256 threads, 4 chunks each per block)
  uint4 k[kStepMaxNB][4], v[kStepMaxNB][4];
  int vis;      // visibility of key tid of the split (tid < 32 NB)
};

__device__ __forceinline__ void kv_zero(KVPre& p) {
#pragma unroll
  for (int bi = 0; bi < kStepMaxNB; ++bi)
#pragma unroll
    for (int h = 0; h < 4; ++h) p.k[bi][h] = p.v[bi][h] = make_uint4(0, 0, 0, 0);
  p.vis = 0;
}

__device__ __forceinline__ void kv_fetch(const uint16_t* Kb, const uint16_t* Vb, const uint8_t* mask, int key_lo,
                                         int key_hi, int nblk, KVPre& p, int tid) {
#pragma unroll
  for (int bi = 0; bi < kStepMaxNB; ++bi)
    if (bi < nblk) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int c = tid + h * 256, jj = c >> 5, ch = c & 31;
        const size_t row = (size_t)min(key_lo + bi * KB + jj, key_hi - 1);
        p.k[bi][h] = *reinterpret_cast<const uint4*>(Kb + row * kD + ch * 8);
        p.v[bi][h] = *reinterpret_cast<const uint4*>(Vb + row * kD + ch * 8);
      }
    }
  if (tid < nblk * KB && key_lo + tid < key_hi) p.vis = mask[key_lo + tid] != 0;
}

__device__ __forceinline__ bf16x8 v_frag_s(const uint16_t* sV, int t, int lane) {
  const int k = lane & 15, q = lane >> 4;
  const uint16_t* p0 = sV + (4 * q + (k >> 2)) * VLD + t * 16 + 4 * (k & 3);
  const uint16_t* p1 = p0 + 16 * VLD;
  const bf16x4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4s*)(p0));
  const bf16x4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4s*)(p1));
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = lo[e];
    r[4 + e] = hi[e];
  }
  return r;
}

}  // namespace

// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(kThreads) void k_step(const StepArgs a) {
  __shared__ StepSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool cw = tid < kCompute;
  const int w = blockIdx.x, x = w & 7, j = w >> 3, g = x >> 1;
  const int C = a.C, L = a.n_layers;
  const int TP = MT * 16;
  const int NL = L * a.n_steps;  // linear layers of the run

  typedef StepLayout SL;
  const Coh R(a.ws);                                                        // the workspace
  const Coh M(a.mod_table ? (const void*)a.mod_table : (const void*)a.ws);  // modulation vectors
  Sync sy{R, 0u};
  if (tid == 0) sm.ok = R.ld4(kProg + (u32)w * kFlagStride * 4u);
  __syncthreads();
  sy.base = sm.ok;
  __syncthreads();

  // this XCC's buffers (byte offsets into the workspace)
  const u32 oXS = SL::xcc + (u32)x * SL::xcc_stride(TP) + SL::xs(TP);
  const u32 oSSX = SL::xcc + (u32)x * SL::xcc_stride(TP) + SL::ssx(TP);
  const int nmrg = MT * 16;            // merge units (row tile, 16 dims)
  const int mrg_wgs = (nmrg + 3) / 4;  // work-groups holding merge units
  const int qkv_wgs = 24;

  // modulation vectors (scale | shift | gate) of linear layer n, norm nm: byte
  // offset in M (the table, or the ring slot the run computes them into)
  auto modo = [&](int n, int nm) -> u32 {
    if (a.mod_table) return (u32)((n * 2 + nm) * 3 * kH) * 4u;
    return SL::mods + (u32)(((n % kStepModSlots) * 2 + nm) * 3 * kH) * 4u;
  };
  auto mod_w = [&](const MJob& m) { return m.nm ? a.L[m.n % L].w_mod2 : a.L[m.n % L].w_mod1; };
  auto mod_b = [&](const MJob& m) { return m.nm ? a.L[m.n % L].b_mod2 : a.L[m.n % L].b_mod1; };
  auto mod_cond = [&](const MJob& m) { return a.cond + (size_t)(m.n / L) * kH; };
  int ci = 0;  // stages published by this launch

  // ---- prologue: modulation of linear layers 0 and 1, the input pack
  if (!a.mod_table) {
    const int u = w + 256 * wave;  // 768 units: layer u / 384
    MJob m = mod_job(u / 384, u % 384);
    if (u >= 768 || m.n >= NL) m.n = -1;
    if (cw && m.n >= 0) {
      ModUnit mu;
      mod_fetch(mod_w(m), mod_cond(m), m.tile, lane, mu);
      mod_finish(mu, sm, mod_b(m), m.tile, R, modo(m.n, m.nm), wave, lane);
    }
    stage_end(sy, ++ci);
    if (!stage_wait(sy, sm, a.ws, ci, 0, 1, 256)) return;
  } else {
    ++ci;
  }
  // pack: this work-group's 32 columns of x, scaled by 1 + scale1 of layer 0
  {
    const u32 m1 = modo(0, 0);
    const int r = tid >> 2, q = tid & 3;  // row, 8-column group
    if (cw && r < C) {
      float v[8];
      unpack8f(*reinterpret_cast<const uint4*>(a.x + (size_t)r * kH + 32 * j + 8 * q), v);
      const float4 s0 = M.ld16f(m1 + (u32)(32 * j + 8 * q) * 4u), s1 = M.ld16f(m1 + (u32)(32 * j + 8 * q + 4) * 4u);
      const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      float o[8], s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sm.xres[r * 32 + 8 * q + i] = v[i];
        o[i] = v[i] * (1.f + sc[i]);
        s += v[i] * v[i];
      }
      R.st16(oXS + tb(r, 32 * j + 8 * q, kH), pack8f(o));
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (q == 0) R.st4f(oSSX + (u32)(r * 32 + j) * 4u, s);
    }
    stage_end(sy, ++ci);
  }

  // QKV weights of layer 0: rotation tile j of [q head x | k head g | v head g]
  const int hsel = j >> 3, t8 = j & 7;
  const int hq = hsel == 0 ? x : hsel == 1 ? kHQ + g : kHQ + kHK + g;  // head of W_qkv's rows
  if (cw && j < qkv_wgs) slab_fetch<8>(a.L[0].w_qkv, hq * 16 + t8, hq * 16 + 8 + t8, 32, 0, sm, wave, lane);
  if (!stage_wait(sy, sm, a.ws, ci, x, 8, 32)) return;

  for (int n = 0; n < NL; ++n) {
    // the thread's indices from an opaque copy of the thread index, so the
    // compiler does not hoist every per-lane address of the stages out of
    // the loop (where they would all stay live at once)
    int tid = threadIdx.x;
    __asm__ volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lq = lane >> 4;
    const bool cw = tid < kCompute;
    // the same for the scalars the stages branch on or add to addresses
    int w = blockIdx.x, C = a.C, Sp = a.S, nsplit = a.S + a.NS, kps = a.kps, P = a.P;
    __asm__ volatile("" : "+s"(w), "+s"(C), "+s"(Sp), "+s"(nsplit), "+s"(kps), "+s"(P));
    uint16_t* trace = a.trace;
    const float* mod_table = a.mod_table;
    __asm__ volatile("" : "+s"(trace), "+s"(mod_table));
    const int x = w & 7, j = w >> 3, g = x >> 1;
    const int hsel = j >> 3, t8 = j & 7;
    const int hq = hsel == 0 ? x : hsel == 1 ? kHQ + g : kHQ + kHK + g;
    const u32 X0 = SL::xcc + (u32)x * SL::xcc_stride(TP);
    const u32 oXS = X0 + SL::xs(TP), oSSX = X0 + SL::ssx(TP), oQB = X0 + SL::qb(TP), oVB = X0 + SL::vb(TP);
    const u32 oKF = X0 + SL::kf(TP), oSSQ = X0 + SL::ssq(TP), oPO = X0 + SL::po(TP), oPML = X0 + SL::pml(TP);
    const u32 oCTX = X0 + SL::ctx(TP), oX1S = X0 + SL::x1s(TP), oSS1 = X0 + SL::ss1(TP), oH = X0 + SL::h(TP);
    auto modo = [&](int nn, int nm) -> u32 {
      if (mod_table) return (u32)((nn * 2 + nm) * 3 * kH) * 4u;
      return SL::mods + (u32)(((nn % kStepModSlots) * 2 + nm) * 3 * kH) * 4u;
    };
    const int l = n % L;
    const StepLayer& Ly = a.L[l];
    const u32 mod1 = modo(n, 0), mod2 = modo(n, 1);
    const bool last = n + 1 == NL;
    // ================= QKV
    if (j < qkv_wgs) {
      gemm1024_mod<MT>(R, oXS, M, mod1 + kH * 4u, oSSX, C, sm, tid);
      if (tid < 16) {
        const int jj = t8 * 16 + tid;  // dim of the head's first half
        sm.freq[tid] = exp2(-(double)jj / 128.0 * a.rope_lb) * 0.15915494309189533577;
      }
      lds_sync();
      const uint16_t* nw = hsel == 0 ? Ly.q_norm : Ly.k_norm;
      if (cw && tid < TP * 2) {
        const int r = tid >> 1, c0 = (tid & 1) * 8;  // row, 8 rotation pairs from c0
        float lo[8], hi[8], sqv = 0.f;
        const float rs = sm.rms[r];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lo[i] = rs * red_sum(sm, r, c0 + i) + red_sum(sm, 64, c0 + i);
          hi[i] = rs * red_sum(sm, r, 16 + c0 + i) + red_sum(sm, 64, 16 + c0 + i);
          sqv += lo[i] * lo[i] + hi[i] * hi[i];
        }
        const int f = t8 * 16 + c0;
        if (hsel < 2) {  // q and k heads: (1 + w) and RoPE
          float wl[8], wh[8];
          unpack8f(*reinterpret_cast<const uint4*>(nw + f), wl);
          unpack8f(*reinterpret_cast<const uint4*>(nw + 128 + f), wh);
          const double pos = (double)a.pos0[0] + (double)r;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            double rev = pos * sm.freq[c0 + i];
            rev -= floor(rev);
            const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
            const float x0 = lo[i] * (1.f + wl[i]), x1 = hi[i] * (1.f + wh[i]);
            lo[i] = x0 * cs - x1 * sn;
            hi[i] = x1 * cs + x0 * sn;
          }
        }
        sm.sq[r * 2 + (c0 >> 3)] = sqv;
        if (r < C) {
          if (hsel == 1) {  // k head: fp32, divided by the row rms when staged
            R.st16f(oKF + tf(r, f, kD), make_float4(lo[0], lo[1], lo[2], lo[3]));
            R.st16f(oKF + tf(r, f, kD) + 1024u, make_float4(lo[4], lo[5], lo[6], lo[7]));
            R.st16f(oKF + tf(r, f + 128, kD), make_float4(hi[0], hi[1], hi[2], hi[3]));
            R.st16f(oKF + tf(r, f + 128, kD) + 1024u, make_float4(hi[4], hi[5], hi[6], hi[7]));
          } else {
            const u32 ob = hsel == 0 ? oQB : oVB;
            R.st16(ob + tb(r, f, kD), pack8f(lo));
            R.st16(ob + tb(r, f + 128, kD), pack8f(hi));
          }
        }
      }
      lds_sync();
      if (cw && hsel < 2 && tid < C) R.st4f(oSSQ + (u32)(tid * 16 + hsel * 8 + t8) * 4u, sm.sq[tid * 2] + sm.sq[tid * 2 + 1]);
    }
    stage_end(sy, ++ci);
    // prefetch: this split's prefix K / V rows and their visibility
    const bool att = j < nsplit;
    const bool suffix = j >= Sp;
    const int key_lo = suffix ? (j - Sp) * KB : j * kps;
    const int key_hi = suffix ? min(C, key_lo + KB) : min(P, key_lo + kps);
    const int nblk = att ? (key_hi - key_lo + KB - 1) / KB : 0;
    KVPre kvp;
    kv_zero(kvp);
    if (cw && att && !suffix)
      kv_fetch(Ly.k_pre + (size_t)g * P * kD, Ly.v_pre + (size_t)g * P * kD, a.mask, key_lo, key_hi, nblk, kvp, tid);
    if (!stage_wait(sy, sm, a.ws, ci, x, 8, qkv_wgs)) return;

    // ================= ATT
    if (att) {
      int vis_t = 0;
      if (cw) vis_t = suffix ? (tid < KB && key_lo + tid < key_hi) : kvp.vis;
      if (cw && wave < 2) {
        const uint64_t bal = __ballot(vis_t);
        if (lane == 0 && 2 * wave < kStepMaxNB) sm.mask[2 * wave] = (u32)bal;
        if (lane == 0 && 2 * wave + 1 < kStepMaxNB) sm.mask[2 * wave + 1] = (u32)(bal >> 32);
      }
      lds_sync();
      // stage the blocks (zero rows for invisible keys)
      if (cw) {
        if (!suffix) {
#pragma unroll
          for (int bi = 0; bi < kStepMaxNB; ++bi) {
            if (bi < nblk) {
              const u32 vis = sm.mask[bi];
#pragma unroll
              for (int h = 0; h < 4; ++h) {
                const int c = tid + h * 256, jj = c >> 5, ch = c & 31;
                const bool ok = (vis >> jj) & 1u;
                *reinterpret_cast<uint4*>(sm.u.kv.K[bi] + jj * KLD + ch * 8) = keep_or_zero(ok, kvp.k[bi][h]);
                *reinterpret_cast<uint4*>(sm.u.kv.V[bi] + jj * VLD + ch * 8) = keep_or_zero(ok, kvp.v[bi][h]);
              }
            }
          }
        } else {
          // the chunk's own keys: thread t -> key t / 8, dims (t % 8) * 32 ..;
          // K divided by the key row's rms
          const int jj = tid >> 3, c = tid & 7;
          const int key = min(key_lo + jj, C - 1);
          const bool ok = (sm.mask[0] >> jj) & 1u;
          float4 kq[8];
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            kq[2 * h] = R.ld16f(oKF + tf(key, c * 32 + h * 8, kD));
            kq[2 * h + 1] = R.ld16f(oKF + tf(key, c * 32 + h * 8, kD) + 1024u);
          }
          uint4 vq[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) vq[h] = R.ld16(oVB + tb(key, c * 32 + h * 8, kD));
          const float4 s0 = R.ld16f(oSSQ + (u32)(key * 16 + 8) * 4u), s1 = R.ld16f(oSSQ + (u32)(key * 16 + 12) * 4u);
          const float tsum = ((s0.x + s0.y) + (s0.z + s0.w)) + ((s1.x + s1.y) + (s1.z + s1.w));
          const float rn = 1.0f / sqrtf(tsum * (1.0f / kD) + kEps);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float kv8[8] = {kq[2 * h].x,     kq[2 * h].y,     kq[2 * h].z,     kq[2 * h].w,
                                  kq[2 * h + 1].x, kq[2 * h + 1].y, kq[2 * h + 1].z, kq[2 * h + 1].w};
            u32 kp[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) kp[e] = ok ? pack2(kv8[2 * e] * rn, kv8[2 * e + 1] * rn) : 0u;
            *reinterpret_cast<uint4*>(sm.u.kv.K[0] + jj * KLD + c * 32 + h * 8) = make_uint4(kp[0], kp[1], kp[2], kp[3]);
            *reinterpret_cast<uint4*>(sm.u.kv.V[0] + jj * VLD + c * 32 + h * 8) = keep_or_zero(ok, vq[h]);
          }
        }
      }
      // queries of row tile `wave` (rope((1 + w) x)) and their rows' 1 / rms
      bf16x8 qf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[ks] = zero_bf16x8();
      float sl2 = 0.f;
      const int qi = wave * 16 + lr;
      if (cw && wave < MT) {
        const int qr = min(qi, C - 1);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = R.ldf(oQB + tb(qr, ks * 32 + lq * 8, kD));
        const float4 s0 = R.ld16f(oSSQ + (u32)(qr * 16) * 4u), s1 = R.ld16f(oSSQ + (u32)(qr * 16 + 4) * 4u);
        const float tsum = ((s0.x + s0.y) + (s0.z + s0.w)) + ((s1.x + s1.y) + (s1.z + s1.w));
        sl2 = (1.4426950408889634f / 16.0f) * (1.0f / sqrtf(tsum * (1.0f / kD) + kEps));
        if (qi >= C) {
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) qf[ks] = zero_bf16x8();
        }
      }
      lds_sync();
      if (cw && wave < MT) {
        f32x4 o[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) o[t] = zero_f32x4();
        float mrun = kNegBig, lrun = 0.f;
#pragma unroll
        for (int bi = 0; bi < kStepMaxNB; ++bi) {
          if (bi >= nblk) break;
          const u32 vis = sm.mask[bi];
          if (vis == 0u) continue;
          const uint16_t* bK = sm.u.kv.K[bi];
          f32x4 s0 = zero_f32x4(), s1 = zero_f32x4();
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(bK + lr * KLD + ks * 32 + lq * 8);
            const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(bK + (16 + lr) * KLD + ks * 32 + lq * 8);
            s0 = mfma16(k0, qf[ks], s0);
            s1 = mfma16(k1, qf[ks], s1);
          }
          float xv[8];
          float mloc = -INFINITY;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            xv[r] = ((vis >> (4 * lq + r)) & 1u) ? s0[r] * sl2 : -INFINITY;
            xv[4 + r] = ((vis >> (16 + 4 * lq + r)) & 1u) ? s1[r] * sl2 : -INFINITY;
            mloc = fmaxf(mloc, fmaxf(xv[r], xv[4 + r]));
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
            const float p0 = exp2f(xv[e] - mnew), p1 = exp2f(xv[e + 1] - mnew);
            psum += p0 + p1;
            const u32 pk = pack2(p0, p1);
            pf[e] = (short)(pk & 0xffffu);
            pf[e + 1] = (short)(pk >> 16);
          }
          lrun = lrun * alpha + psum;
          const uint16_t* bV = sm.u.kv.V[bi];
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            o[t] *= alpha;
            o[t] = mfma16(v_frag_s(bV, t, lane), pf, o[t]);
          }
        }
        float lsum = lrun + __shfl_xor(lrun, 16, 64);
        lsum += __shfl_xor(lsum, 32, 64);
        const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
        if (qi < C) {
          // partial of split j, row tile `wave`: [dim tile t][lr][lq][4]
          const u32 ob = oPO + (u32)(((j * 4 + wave) * 16) * 256 + (lr * 4 + lq) * 4) * 2u;
#pragma unroll
          for (int t = 0; t < 16; ++t)
            R.st8(ob + (u32)t * 512u,
                  make_uint2(pack2(o[t][0] * inv, o[t][1] * inv), pack2(o[t][2] * inv, o[t][3] * inv)));
          if (lq == 0) R.st8(oPML + (u32)((j * 64 + qi) * 2) * 4u, make_uint2(__float_as_uint(mrun), __float_as_uint(lsum)));
        }
      }
    }
    stage_end(sy, ++ci);
    if (!stage_wait(sy, sm, a.ws, ci, x, 8, nsplit)) return;

    // ================= MRG: unit (row tile mt, dims 16 t ..) per wave
    {
      const int u = j * 4 + wave;
      if (cw && u < nmrg) {
        const int mt = u >> 4, t = u & 15;
        const int i = mt * 16 + lr;
        if (i < C) {
          float2 ml[kStepMaxSplits];
          uint2 ov[kStepMaxSplits];
#pragma unroll
          for (int s = 0; s < kStepMaxSplits; ++s) {
            ml[s] = make_float2(kNegBig, 0.f);
            ov[s] = make_uint2(0, 0);
            if (s < nsplit) {
              const uint2 m = R.ld8(oPML + (u32)((s * 64 + i) * 2) * 4u);
              ml[s] = make_float2(__uint_as_float(m.x), __uint_as_float(m.y));
              ov[s] = R.ld8(oPO + (u32)((((s * 4 + mt) * 16 + t) * 256) + (lr * 4 + lq) * 4) * 2u);
            }
          }
          float Mx = kNegBig;
#pragma unroll
          for (int s = 0; s < kStepMaxSplits; ++s)
            if (ml[s].y > 0.f) Mx = fmaxf(Mx, ml[s].x);
          float Ls = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < kStepMaxSplits; ++s) {
            const float wgt = ml[s].y > 0.f ? ml[s].y * exp2f(ml[s].x - Mx) : 0.f;
            Ls += wgt;
            acc[0] += wgt * bf2f((uint16_t)(ov[s].x & 0xffffu));
            acc[1] += wgt * bf2f((uint16_t)(ov[s].x >> 16));
            acc[2] += wgt * bf2f((uint16_t)(ov[s].y & 0xffffu));
            acc[3] += wgt * bf2f((uint16_t)(ov[s].y >> 16));
          }
          const float inv = 1.0f / Ls;
          const int col = t * 16 + 4 * lq;
          R.st8(oCTX + tb(i, col & ~7, kD) + (u32)(col & 7) * 2u,
                make_uint2(pack2(acc[0] * inv, acc[1] * inv), pack2(acc[2] * inv, acc[3] * inv)));
        }
      }
    }
    stage_end(sy, ++ci);
    // prefetch: O-projection weights (W_o rows 32 j .., head x's columns) and
    // this wave's modulation unit (linear layer n + 2)
    if (cw) slab_fetch<2>(Ly.w_o, 2 * j, 2 * j + 1, 64, 8 * x, sm, wave, lane);
    MJob mj = mod_job(n + 2, w + 256 * wave);
    if (mod_table || mj.n >= NL) mj.n = -1;
    ModUnit mu;
    mod_zero(mu);
    if (cw && mj.n >= 0) mod_fetch(mod_w(mj), mod_cond(mj), mj.tile, lane, mu);
    if (!stage_wait(sy, sm, a.ws, ci, x, 8, mrg_wgs)) return;

    // ================= OP: y_x for columns 32 j .. (K = head x's 256 dims)
    gemm_ksplit<MT, 2>(R, oCTX, sm, tid);
    if (cw && wave < MT) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) R.st16f(SL::ypart + part_frag(x, wave, 2 * j + nt, lane), red_frag(sm, wave, nt, lane));
    }
    stage_end(sy, ++ci);
    if (cw && mj.n >= 0) mod_finish(mu, sm, mod_b(mj), mj.tile, R, modo(mj.n, mj.nm), wave, lane);
    // prefetch: gate-up weights (gate tile 32 x + j, up tile 256 + 32 x + j)
    if (cw) slab_fetch<8>(Ly.w_gu, 32 * x + j, kI / 16 + 32 * x + j, 32, 0, sm, wave, lane);
    if (!stage_wait(sy, sm, a.ws, ci, 8 * j, 1, 8)) return;

    // ================= RS1: x1 = x + gate1 (y_0 + .. + y_7), columns 32 j ..
    {
      if (cw && wave < MT) {
        float4 ys[2][8];
#pragma unroll
        for (int h = 0; h < 8; ++h)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) ys[nt][h] = R.ld16f(SL::ypart + part_frag(h, wave, 2 * j + nt, lane));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int c = 32 * j + 16 * nt + lr;
          const float g1 = M.ld4f(mod1 + (u32)(2 * kH + c) * 4u), s2 = M.ld4f(mod2 + (u32)c * 4u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y = f4c(ys[nt][0], e);
#pragma unroll
            for (int h = 1; h < 8; ++h) y += f4c(ys[nt][h], e);
            const int r = wave * 16 + lq * 4 + e;
            const float x1 = sm.xres[r * 32 + 16 * nt + lr] + g1 * y;
            sm.x1k[r * 32 + 16 * nt + lr] = x1;
            sm.u.g.tmp[r * 33 + 16 * nt + lr] = x1 * (1.f + s2);
          }
        }
      }
      lds_sync();
      const int r = tid >> 2, q = tid & 3;
      if (cw && r < C) {
        float o[8], s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          o[i] = sm.u.g.tmp[r * 33 + 8 * q + i];
          const float v = sm.x1k[r * 32 + 8 * q + i];
          s += v * v;
        }
        R.st16(oX1S + tb(r, 32 * j + 8 * q, kH), pack8f(o));
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q == 0) R.st4f(oSS1 + (u32)(r * 32 + j) * 4u, s);
      }
    }
    stage_end(sy, ++ci);
    if (!stage_wait(sy, sm, a.ws, ci, x, 8, 32)) return;

    // ================= GU: 16 gate + 16 up features of XCC x's slice
    gemm1024_mod<MT>(R, oX1S, M, mod2 + kH * 4u, oSS1, C, sm, tid);
    if (cw) {
      const int r = tid >> 2, c0 = (tid & 3) * 4;  // row, 4 outputs
      if (r < C) {
        const float rs = sm.rms[r];
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gt = rs * red_sum(sm, r, c0 + i) + red_sum(sm, 64, c0 + i);
          const float up = rs * red_sum(sm, r, 16 + c0 + i) + red_sum(sm, 64, 16 + c0 + i);
          hv[i] = gelu_tanh(gt) * up;
        }
        const int col = 16 * j + c0;
        R.st8(oH + tb(r, col & ~7, 512) + (u32)(col & 7) * 2u, make_uint2(pack2(hv[0], hv[1]), pack2(hv[2], hv[3])));
      }
    }
    stage_end(sy, ++ci);
    // prefetch: down weights (rows 32 j .., XCC x's 512 columns)
    if (cw) slab_fetch<4>(Ly.w_down, 2 * j, 2 * j + 1, 128, 16 * x, sm, wave, lane);
    if (!stage_wait(sy, sm, a.ws, ci, x, 8, 32)) return;

    // ================= DP: y2_x for columns 32 j .. (K = XCC x's 512 features)
    gemm_ksplit<MT, 4>(R, oH, sm, tid);
    if (cw && wave < MT) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) R.st16f(SL::y2part + part_frag(x, wave, 2 * j + nt, lane), red_frag(sm, wave, nt, lane));
    }
    stage_end(sy, ++ci);
    // prefetch: the next layer's QKV weights
    if (cw && j < qkv_wgs && !last)
      slab_fetch<8>(a.L[(n + 1) % L].w_qkv, hq * 16 + t8, hq * 16 + 8 + t8, 32, 0, sm, wave, lane);
    if (!stage_wait(sy, sm, a.ws, ci, 8 * j, 1, 8)) return;

    // ================= RS2: out = x1 + gate2 (y2_0 + .. + y2_7), columns 32 j ..
    {
      const u32 m1n = last ? 0u : modo(n + 1, 0);  // the next layer's scale1
      if (cw && wave < MT) {
        float4 ys[2][8];
#pragma unroll
        for (int h = 0; h < 8; ++h)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) ys[nt][h] = R.ld16f(SL::y2part + part_frag(h, wave, 2 * j + nt, lane));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int c = 32 * j + 16 * nt + lr;
          const float g2 = M.ld4f(mod2 + (u32)(2 * kH + c) * 4u);
          const float s1n = last ? 0.f : M.ld4f(m1n + (u32)c * 4u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float y = f4c(ys[nt][0], e);
#pragma unroll
            for (int h = 1; h < 8; ++h) y += f4c(ys[nt][h], e);
            const int r = wave * 16 + lq * 4 + e;
            const float ob = bf2f(f2bf(sm.x1k[r * 32 + 16 * nt + lr] + g2 * y));  // the layer output, bf16
            sm.xres[r * 32 + 16 * nt + lr] = ob;
            sm.u.g.tmp[r * 33 + 16 * nt + lr] = ob * (1.f + s1n);
          }
        }
      }
      lds_sync();
      const int r = tid >> 2, q = tid & 3;
      if (cw && r < C) {
        float o[8], v[8], s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          o[i] = sm.u.g.tmp[r * 33 + 8 * q + i];
          v[i] = sm.xres[r * 32 + 8 * q + i];
          s += v[i] * v[i];
        }
        if (!last) R.st16(oXS + tb(r, 32 * j + 8 * q, kH), pack8f(o));
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (q == 0 && !last) R.st4f(oSSX + (u32)(r * 32 + j) * 4u, s);
        if (x == 0) {
          const uint4 ov = pack8f(v);
          if (trace) *reinterpret_cast<uint4*>(trace + ((size_t)n * C + r) * kH + 32 * j + 8 * q) = ov;
          if (last) *reinterpret_cast<uint4*>(a.x + (size_t)r * kH + 32 * j + 8 * q) = ov;
        }
      }
    }
    stage_end(sy, ++ci);
    if (!last && !stage_wait(sy, sm, a.ws, ci, x, 8, 32)) return;
  }
}

// ---------------------------------------------------------------------------
void step_config(int C, int P, int& S, int& NS, int& kps) {
  NS = (C + KB - 1) / KB;
  int nb = 2;
  while (nb < kStepMaxNB && (P + KB * nb - 1) / (KB * nb) + NS > kStepMaxSplits) ++nb;
  kps = KB * nb;
  S = (P + kps - 1) / kps;
}

bool step_supported(int B, int C, int P, int n_layers) {
  if (B != 1 || C < 1 || C > 64 || P < 0 || P > 2048 || n_layers < 1 || n_layers > kStepMaxLayers) return false;
  int S, NS, kps;
  step_config(C, P, S, NS, kps);
  return S + NS <= kStepMaxSplits;
}

hipError_t launch_step(const StepArgs& a, hipStream_t s) {
  switch (a.TP) {
    case 16: k_step<1><<<dim3(256), dim3(kThreads), 0, s>>>(a); break;
    case 32: k_step<2><<<dim3(256), dim3(kThreads), 0, s>>>(a); break;
    case 48: k_step<3><<<dim3(256), dim3(kThreads), 0, s>>>(a); break;
    case 64: k_step<4><<<dim3(256), dim3(kThreads), 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t step_occupancy_ok(int TP, bool* ok) {
  int per_cu = 0, dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  switch (TP) {
    case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step<1>, kThreads, 0); break;
    case 32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step<2>, kThreads, 0); break;
    case 48: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step<3>, kThreads, 0); break;
    default: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_step<4>, kThreads, 0); break;
  }
  if (e != hipSuccess) return e;
  *ok = per_cu >= 1 && cus * per_cu >= 256;
  return hipSuccess;
}

}  // namespace dmx
