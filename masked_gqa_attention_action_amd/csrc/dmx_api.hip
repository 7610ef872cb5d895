// C ABI of libdmx: argument validation, workspace layout and the order in
// which the stage kernels run.  Citations of the pages are in include/dmx.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/dmx.h"
#include "dmx_device.hpp"
#include "dmx_internal.hpp"
#include "dmx_tiles.hpp"

using namespace dmx;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DMX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DMX_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define DMX_REQUIRE_PTR(p)                                                             \
  do {                                                                                 \
    if ((p) == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: %s is null", fn, #p);    \
    if (!aligned16(p)) return fail(DMX_ERR_MISALIGNED, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

#define DMX_TRY(expr)             \
  do {                            \
    const int st_ = (expr);       \
    if (st_ != DMX_OK) return st_; \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

// Workspace carve-up.  Everything a layer needs between its stages, plus
// (for a stack) the modulation vectors of every layer of one step.  Rows of
// the tiled / fp32 intermediates are tiled rows (each request padded to TP).
struct WsLayout {
  size_t mod1, mod2, apk, xp, raw, ss_q, qvb, ctx, x1, x1s, h, part_o, part_ml, ss_a, ss_b, stack_mod, step, total;
  bool has_step;  // the persistent step kernel's region (batch 1 stacks)
  int TP;
  AttnArgs attn;
};

bool ws_layout(int B, int T, int P, int n_layers, WsLayout& L) {
  if (B < 1 || T < 1 || P < 0 || B > DMX_MAX_BATCH || T > 4096 || P > DMX_MAX_PREFIX || n_layers < 0 ||
      n_layers > DMX_MAX_LAYERS)
    return false;
  L.TP = padded_tokens(T);
  const size_t M = (size_t)B * L.TP;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.mod1 = take((size_t)B * 3 * kH * 4);
  L.mod2 = take((size_t)B * 3 * kH * 4);
  L.apk = take(M * DMX_PREFIX_HIDDEN * 2);  // tiled copy of a row-major A operand
  L.xp = take(M * kH * 2);                  // tiled layer input
  L.raw = take(M * kQKV * 4);               // fp32 QKV projection (tiled in the fused layer)
  L.ss_q = take(M * kQkvTiles * 4);         // its q / k head sums of squares
  L.qvb = take(M * kQVB * 2);               // tiled bf16 q and v heads of the chunk
  L.ctx = take(M * kHQ * kD * 2);           // tiled attention output
  L.x1 = take(M * kH * 4);   // fp32 residual between the two halves of a layer
  L.x1s = take(M * kH * 2);  // tiled bf16(x1 * (1 + scale2)), the gate-up A operand
  L.h = take(M * kI * 2);    // tiled GEGLU output
  attn_config(B, T, P, L.attn);
  const size_t prow = (size_t)B * kHK * (L.attn.S + L.attn.NS) * L.attn.R16;
  L.part_o = take(prow * kD * 2);
  L.part_ml = take(prow * 2 * 4);
  L.ss_a = take(M * kSsParts * 4);  // row sums of squares of x1, one per O-projection tile
  L.ss_b = take(M * kSsParts * 4);  // ... of a layer input (pack pass or the down tiles)
  L.stack_mod = take((size_t)n_layers * 2 * B * 3 * kH * 4);
  L.has_step = n_layers > 0 && step_supported(B, T, P, n_layers);
  L.step = L.has_step ? take(StepLayout::bytes(L.TP)) : 0;
  L.total = off;
  return true;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_ws(const char* fn, void* ws, size_t ws_bytes, int B, int T, int P, WsLayout& L, int n_layers = 0) {
  if (!ws_layout(B, T, P, n_layers, L)) return fail(DMX_ERR_UNSUPPORTED, "%s: unsupported sizes", fn);
  if (ws == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: ws is null", fn);
  if (!aligned16(ws)) return fail(DMX_ERR_MISALIGNED, "%s: ws is not 16-byte aligned", fn);
  if (ws_bytes < L.total)
    return fail(DMX_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, L.total);
  return DMX_OK;
}

int check_bt(const char* fn, int B, int T, int max_t) {
  if (B < 1 || B > DMX_MAX_BATCH) return fail(DMX_ERR_UNSUPPORTED, "%s: batch %d not in [1, %d]", fn, B, DMX_MAX_BATCH);
  if (T < 1 || T > max_t) return fail(DMX_ERR_UNSUPPORTED, "%s: tokens %d not in [1, %d]", fn, T, max_t);
  return DMX_OK;
}

GemmArgs gemm_args() {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  return a;
}

// ---- stage enqueuers (arguments already validated) -------------------------
int enq_mods(const ModJob* jobs, int n, int B, hipStream_t s) {
  for (int j0 = 0; j0 < n; j0 += kMaxModJobs) {
    ModBatch mb;
    memset(&mb, 0, sizeof mb);
    mb.B = B;
    mb.n = n - j0 < kMaxModJobs ? n - j0 : kMaxModJobs;
    for (int j = 0; j < mb.n; ++j) mb.job[j] = jobs[j0 + j];
    DMX_TRY(hip_check(launch_mod_multi(mb, s), "modulation launch"));
  }
  return DMX_OK;
}

int enq_adarms(const dmx_bf16* x, const dmx_bf16* cond, const dmx_bf16* w_mod, const dmx_bf16* b_mod,
               int B, int T, dmx_bf16* xn, float* mod, hipStream_t s) {
  const ModJob job{w_mod, b_mod, cond, mod};
  DMX_TRY(enq_mods(&job, 1, B, s));
  return hip_check(launch_adarms_norm(x, mod, B * T, T, xn, s), "AdaRMS norm launch");
}

int enq_qkv(const dmx_bf16* xn, const dmx_bf16* w_qkv, const dmx_bf16* qn, const dmx_bf16* kn, int B, int T,
            int hidden, const int32_t* pos0, float base, dmx_bf16* q, dmx_bf16* k, dmx_bf16* v,
            int kv_rows, int kv_row0, void* ws, const WsLayout& L, hipStream_t s) {
  const GemmKind kind = hidden == kH ? GEMM_QKV1024 : GEMM_QKV2560;
  uint16_t* apk = at<uint16_t>(ws, L.apk);
  float* raw = at<float>(ws, L.raw);
  DMX_TRY(hip_check(launch_pack_rows(xn, B, T, L.TP, hidden, apk, nullptr, s), "pack launch"));
  GemmArgs a = gemm_args();
  gemm_config(kind, a);
  a.A = apk;
  a.W = w_qkv;
  a.M = B * L.TP;
  a.T = T;
  a.TP = L.TP;
  a.out_f32 = raw;
  a.ldo = kQKV;
  DMX_TRY(hip_check(launch_gemm(kind, a, s), "QKV GEMM launch"));
  return hip_check(launch_qknorm_rope(raw, qn, kn, pos0, base, B, T, L.TP, q, k, v, kv_rows, kv_row0, s),
                   "QK-norm/RoPE launch");
}

AttnArgs attn_args(const WsLayout& L, void* ws) {
  AttnArgs a = L.attn;
  a.q = a.ks = a.vs = a.kp = a.vp = nullptr;
  a.y = nullptr;
  a.ss_q = nullptr;
  a.qvb = nullptr;
  a.mask = nullptr;
  a.part_o = at<uint16_t>(ws, L.part_o);
  a.part_ml = at<float>(ws, L.part_ml);
  a.ctx_tiled = 0;
  a.side_n = a.side_B = a.attn_grid = 0;
  return a;
}

int enq_attention(const dmx_bf16* q, const dmx_bf16* ks, const dmx_bf16* vs, const dmx_bf16* kp,
                  const dmx_bf16* vp, const uint8_t* mask, dmx_bf16* ctx, void* ws, const WsLayout& L,
                  hipStream_t s) {
  AttnArgs a = attn_args(L, ws);
  a.q = q;
  a.ks = ks;
  a.vs = vs;
  a.kp = kp;
  a.vp = vp;
  a.mask = mask;
  return hip_check(launch_attention(a, ctx, s), "attention launch");
}

// Gated-residual projection of a row-major A operand (tiled into the
// workspace first): out = resid + gate[b] * (A * W^T), all bf16 row-major.
int enq_resid_gemm(GemmKind kind, const dmx_bf16* A, int K, const dmx_bf16* W, const float* mod,
                   const dmx_bf16* resid, int B, int T, dmx_bf16* out, void* ws, const WsLayout& L, hipStream_t s) {
  uint16_t* apk = at<uint16_t>(ws, L.apk);
  DMX_TRY(hip_check(launch_pack_rows(A, B, T, L.TP, K, apk, nullptr, s), "pack launch"));
  GemmArgs a = gemm_args();
  gemm_config(kind, a);
  a.A = apk;
  a.W = W;
  a.M = B * L.TP;
  a.T = T;
  a.TP = L.TP;
  a.out_bf16 = out;
  a.ldo = kH;
  a.gate = mod + 2 * kH;
  a.gate_stride = 3 * kH;
  a.resid = resid;
  return hip_check(launch_gemm(kind, a, s), "projection GEMM launch");
}

int enq_geglu(const dmx_bf16* xn2, const dmx_bf16* w_gu, const dmx_bf16* w_down, const float* mod2,
              const dmx_bf16* resid, int B, int T, dmx_bf16* out, void* ws, const WsLayout& L,
              hipStream_t s) {
  uint16_t* apk = at<uint16_t>(ws, L.apk);
  uint16_t* h = at<uint16_t>(ws, L.h);
  DMX_TRY(hip_check(launch_pack_rows(xn2, B, T, L.TP, kH, apk, nullptr, s), "pack launch"));
  GemmArgs a = gemm_args();
  gemm_config(GEMM_GATEUP, a);
  a.A = apk;
  a.W = w_gu;
  a.M = B * L.TP;
  a.T = T;
  a.TP = L.TP;
  a.out_pk = h;
  a.ldo = kI;
  DMX_TRY(hip_check(launch_gemm(GEMM_GATEUP, a, s), "gate-up GEMM launch"));
  a = gemm_args();
  gemm_config(GEMM_DOWN, a);
  a.A = h;
  a.W = w_down;
  a.M = B * L.TP;
  a.T = T;
  a.TP = L.TP;
  a.out_bf16 = out;
  a.ldo = kH;
  a.gate = mod2 + 2 * kH;
  a.gate_stride = 3 * kH;
  a.resid = resid;
  return hip_check(launch_gemm(GEMM_DOWN, a, s), "down projection launch");
}

// One stage of the fused layer chain (modulation vectors mod1 / mod2 already
// computed, the workspace holding x_in tiled in xp and its row sums of squares
// in ss_b, 64 per row).  In order:
//   DMX_STAGE_QKV      QKV GEMM with AdaRMS #1, QK-norm weights and RoPE fused
//   DMX_STAGE_ATTN     attention splits (1 / rms of q, k applied on load)
//   DMX_STAGE_COMBINE  merge of the splits into the tiled context
//   DMX_STAGE_OPROJ    O-projection + gated residual: fp32 x1, tiled
//                      bf16(x1 * (1 + scale2)) and row sums of squares of x1
//   DMX_STAGE_GATEUP   gate-up GEMM with AdaRMS #2 fused + GEGLU
//   DMX_STAGE_DOWN     down projection + gated residual: row-major x_out, its
//                      tiled copy (scaled by the next layer's 1 + scale1 when
//                      that is known) and row sums of squares, for the next layer
struct LayerCtx {
  const dmx_layer_weights* w;
  const dmx_prefix_kv* kv;
  const dmx_bf16* x_in;
  const int32_t* pos0;
  int B, C;
  dmx_bf16* x_out;
  const float *mod1, *mod2;
  void* ws;
  const WsLayout* L;
  const float* next_scale1;  // the next layer's modulation (its scale first), or null
  ModJob side[2] = {};       // modulation GEMVs the attention launch runs on idle CUs
  int side_n = 0;
};

int enq_layer_stage(const LayerCtx& c, int stage, hipStream_t s) {
  const WsLayout& L = *c.L;
  void* ws = c.ws;
  const int M = c.B * L.TP;
  GemmArgs g = gemm_args();
  g.M = M;
  g.T = c.C;
  g.TP = L.TP;
  switch (stage) {
    case DMX_STAGE_QKV: {
      const GemmKind kind = GEMM_QKV1024_MODPRE;  // the tiled x holds bf16(x * (1 + scale1))
      gemm_config(kind, g);
      g.A = at<uint16_t>(ws, L.xp);
      g.nmod = c.mod1;
      g.ss_in = at<float>(ws, L.ss_b);
      g.ss_in_n = kSsParts;
      g.W = c.w->w_qkv;
      g.out_f32 = at<float>(ws, L.raw);
      g.ldo = kQKV;
      g.qn_w = c.w->q_norm;
      g.kn_w = c.w->k_norm;
      g.pos0 = c.pos0;
      g.rope_base = 10000.0f;
      g.ss_q = at<float>(ws, L.ss_q);
      g.out_pk = at<uint16_t>(ws, L.qvb);
      return hip_check(launch_gemm(kind, g, s), "QKV GEMM launch");
    }
    case DMX_STAGE_ATTN:
    case DMX_STAGE_COMBINE: {
      AttnArgs a = attn_args(L, ws);
      a.y = at<float>(ws, L.raw);
      a.ss_q = at<float>(ws, L.ss_q);
      a.qvb = at<uint16_t>(ws, L.qvb);
      a.kp = c.kv->k;
      a.vp = c.kv->v;
      a.mask = c.kv->mask;
      a.ctx_tiled = 1;
      if (stage == DMX_STAGE_ATTN) {
        a.side_n = c.side_n;
        a.side_B = c.B;
        for (int j = 0; j < c.side_n; ++j) a.side[j] = c.side[j];
        return hip_check(launch_attn_partial(a, s), "attention launch");
      }
      return hip_check(launch_attn_combine(a, at<uint16_t>(ws, L.ctx), s), "attention combine launch");
    }
    case DMX_STAGE_OPROJ:  // x1 = x + gate1 * (ctx W_o^T)
      gemm_config(GEMM_OPROJ_F32, g);
      g.A = at<uint16_t>(ws, L.ctx);
      g.W = c.w->w_o;
      g.out_f32 = at<float>(ws, L.x1);
      g.out_pk = at<uint16_t>(ws, L.x1s);
      g.xs_scale = c.mod2;
      g.ldo = kH;
      g.gate = c.mod1 + 2 * kH;
      g.gate_stride = 3 * kH;
      g.resid = c.x_in;
      g.ss_out = at<float>(ws, L.ss_a);
      g.ss_out_n = kSsParts;
      return hip_check(launch_gemm(GEMM_OPROJ_F32, g, s), "O-projection launch");
    case DMX_STAGE_GATEUP:
      gemm_config(GEMM_GATEUP_MOD, g);
      g.A = at<uint16_t>(ws, L.x1s);
      g.nmod = c.mod2;
      g.ss_in = at<float>(ws, L.ss_a);
      g.ss_in_n = kSsParts;
      g.W = c.w->w_gu;
      g.out_pk = at<uint16_t>(ws, L.h);
      g.ldo = kI;
      return hip_check(launch_gemm(GEMM_GATEUP_MOD, g, s), "gate-up GEMM launch");
    case DMX_STAGE_DOWN:  // out = x1 + gate2 * (GEGLU(xn2) W_down^T)
      gemm_config(GEMM_DOWN_F32RES, g);
      g.A = at<uint16_t>(ws, L.h);
      g.W = c.w->w_down;
      g.out_bf16 = c.x_out;
      g.out_pk = at<uint16_t>(ws, L.xp);
      g.ldo = kH;
      g.gate = c.mod2 + 2 * kH;
      g.gate_stride = 3 * kH;
      g.resid_f32 = at<float>(ws, L.x1);
      g.ss_out = at<float>(ws, L.ss_b);
      g.ss_out_n = kSsParts;
      g.xs_scale = c.next_scale1;
      return hip_check(launch_gemm(GEMM_DOWN_F32RES, g, s), "down projection launch");
  }
  return fail(DMX_ERR_INVALID_ARG, "unknown layer stage %d", stage);
}

int enq_layer_chain(const LayerCtx& c, hipStream_t s) {
  for (int stage = DMX_STAGE_QKV; stage <= DMX_STAGE_DOWN; ++stage) DMX_TRY(enq_layer_stage(c, stage, s));
  return DMX_OK;
}

// tiled copy of a row-major layer input, scaled by the layer's 1 + scale1
// (mod1: the layer's modulation, scale first), and its row statistics
int enq_pack_input(const dmx_bf16* x, int B, int C, const float* mod1, void* ws, const WsLayout& L,
                   hipStream_t s) {
  return hip_check(launch_pack_rows(x, B, C, L.TP, kH, at<uint16_t>(ws, L.xp), at<float>(ws, L.ss_b), s, mod1,
                                    3 * kH),
                   "input pack launch");
}

int enq_layer(const dmx_layer_weights* w, const dmx_prefix_kv* kv, const dmx_bf16* x_in,
              const dmx_bf16* cond, const int32_t* pos0, int B, int C, dmx_bf16* x_out, void* ws,
              const WsLayout& L, hipStream_t s) {
  float* mod1 = at<float>(ws, L.mod1);
  float* mod2 = at<float>(ws, L.mod2);
  const ModJob jobs[2] = {{w->w_mod1, w->b_mod1, cond, mod1}, {w->w_mod2, w->b_mod2, cond, mod2}};
  DMX_TRY(enq_mods(jobs, 2, B, s));
  DMX_TRY(enq_pack_input(x_in, B, C, mod1, ws, L, s));
  const LayerCtx c{w, kv, x_in, pos0, B, C, x_out, mod1, mod2, ws, &L, nullptr};
  return enq_layer_chain(c, s);
}

int check_layer_weights(const char* fn, const dmx_layer_weights* w) {
  if (w == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: weights struct is null", fn);
  DMX_REQUIRE_PTR(w->w_mod1);
  DMX_REQUIRE_PTR(w->b_mod1);
  DMX_REQUIRE_PTR(w->w_qkv);
  DMX_REQUIRE_PTR(w->q_norm);
  DMX_REQUIRE_PTR(w->k_norm);
  DMX_REQUIRE_PTR(w->w_o);
  DMX_REQUIRE_PTR(w->w_mod2);
  DMX_REQUIRE_PTR(w->b_mod2);
  DMX_REQUIRE_PTR(w->w_gu);
  DMX_REQUIRE_PTR(w->w_down);
  return DMX_OK;
}

int check_kv(const char* fn, const dmx_bf16* k, const dmx_bf16* v, const uint8_t* mask, int P) {
  if (P < 0 || P > DMX_MAX_PREFIX)
    return fail(DMX_ERR_UNSUPPORTED, "%s: p_bucket %d not in [0, %d]", fn, P, DMX_MAX_PREFIX);
  if (P > 0) {
    DMX_REQUIRE_PTR(k);
    DMX_REQUIRE_PTR(v);
    if (mask == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: mask is null", fn);
  }
  return DMX_OK;
}

}  // namespace

// ============================================================================
extern "C" {

int dmx_select_bucket(int32_t prefix_len, const int32_t* buckets, int32_t n, int32_t fast_prefix_len,
                      int32_t min_tokens, int32_t* idx_out) {
  if (idx_out) *idx_out = -1;
  if (buckets == nullptr || idx_out == nullptr || prefix_len <= 0 || fast_prefix_len <= 0 ||
      min_tokens < 0 || n < 0)
    return fail(DMX_ERR_INVALID_ARG, "dmx_select_bucket: invalid argument");
  if (n == 0) return fail(DMX_ERR_BAD_BUCKETS, "dmx_select_bucket: empty bucket list");
  int32_t prev = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t bk = buckets[i];
    if (bk <= 0 || bk > fast_prefix_len)
      return fail(DMX_ERR_BAD_BUCKETS, "dmx_select_bucket: bucket %d outside (0, %d]", bk, fast_prefix_len);
    if (i > 0 && bk <= prev)
      return fail(DMX_ERR_BAD_BUCKETS, "dmx_select_bucket: buckets not strictly increasing");
    prev = bk;
  }
  if (prefix_len > fast_prefix_len)
    return fail(DMX_ERR_PREFIX_TOO_LONG, "dmx_select_bucket: prefix %d above cap %d", prefix_len,
                fast_prefix_len);
  // buckets are strictly increasing: the first eligible one that holds the prefix is the smallest
  for (int32_t i = 0; i < n; ++i) {
    if (buckets[i] >= min_tokens && buckets[i] >= prefix_len) {
      *idx_out = i;
      return DMX_OK;
    }
  }
  return DMX_FALLBACK_EAGER;
}

size_t dmx_workspace_bytes(int32_t batch, int32_t tokens, int32_t p_bucket) {
  WsLayout L;
  if (!ws_layout(batch, tokens, p_bucket, 0, L)) return 0;
  return L.total;
}

size_t dmx_stack_workspace_bytes(int32_t n_layers, int32_t batch, int32_t chunk, int32_t p_bucket) {
  WsLayout L;
  if (n_layers < 1 || !ws_layout(batch, chunk, p_bucket, n_layers, L)) return 0;
  return L.total;
}

int dmx_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dmx_workspace_init";
  DMX_REQUIRE_PTR(ws);
  return hip_check(launch_fill_zero(ws, ws_bytes & ~(size_t)15, (hipStream_t)stream), "workspace fill");
}

int dmx_pack_weight(const dmx_bf16* w, int32_t rows, int32_t cols, dmx_bf16* out, void* stream) {
  const char* fn = "dmx_pack_weight";
  DMX_REQUIRE_PTR(w);
  DMX_REQUIRE_PTR(out);
  if (rows < 16 || cols < 32 || rows % 16 != 0 || cols % 32 != 0 || cols > 16384 || rows > (1 << 20))
    return fail(DMX_ERR_UNSUPPORTED, "%s: %d x %d (rows a multiple of 16, cols of 32 up to 16384)", fn, rows, cols);
  const uintptr_t wa = reinterpret_cast<uintptr_t>(w), oa = reinterpret_cast<uintptr_t>(out);
  const uintptr_t bytes = (uintptr_t)rows * cols * 2;
  if (wa < oa + bytes && oa < wa + bytes) return fail(DMX_ERR_INVALID_ARG, "%s: out overlaps w", fn);
  return hip_check(launch_pack_rows(w, 1, rows, rows, cols, out, nullptr, (hipStream_t)stream), "pack launch");
}

int dmx_adarms_prenorm(const dmx_bf16* x, const dmx_bf16* cond, const dmx_bf16* w_mod, const dmx_bf16* b_mod,
                       int32_t batch, int32_t tokens, dmx_bf16* x_norm, float* mod, void* stream) {
  const char* fn = "dmx_adarms_prenorm";
  DMX_REQUIRE_PTR(x);
  DMX_REQUIRE_PTR(cond);
  DMX_REQUIRE_PTR(w_mod);
  DMX_REQUIRE_PTR(b_mod);
  DMX_REQUIRE_PTR(x_norm);
  DMX_REQUIRE_PTR(mod);
  DMX_TRY(check_bt(fn, batch, tokens, 4096));
  return enq_adarms(x, cond, w_mod, b_mod, batch, tokens, x_norm, mod, (hipStream_t)stream);
}

int dmx_qkv_qknorm_rope(const dmx_bf16* x_norm, const dmx_bf16* w_qkv, const dmx_bf16* q_norm_w,
                        const dmx_bf16* k_norm_w, int32_t batch, int32_t tokens, int32_t hidden,
                        const int32_t* pos0, float rope_base, dmx_bf16* q, dmx_bf16* k, dmx_bf16* v,
                        int32_t kv_rows, int32_t kv_row0, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dmx_qkv_qknorm_rope";
  DMX_REQUIRE_PTR(x_norm);
  DMX_REQUIRE_PTR(w_qkv);
  DMX_REQUIRE_PTR(q_norm_w);
  DMX_REQUIRE_PTR(k_norm_w);
  DMX_REQUIRE_PTR(pos0);
  DMX_REQUIRE_PTR(q);
  DMX_REQUIRE_PTR(k);
  DMX_REQUIRE_PTR(v);
  DMX_TRY(check_bt(fn, batch, tokens, 4096));
  if (hidden != kH && hidden != DMX_PREFIX_HIDDEN)
    return fail(DMX_ERR_UNSUPPORTED, "%s: hidden %d (1024 or 2560 supported)", fn, hidden);
  if (!(rope_base > 1.0f)) return fail(DMX_ERR_INVALID_ARG, "%s: rope_base must be > 1", fn);
  if (kv_row0 < 0 || kv_rows < 1 || (int64_t)kv_row0 + tokens > kv_rows)
    return fail(DMX_ERR_INVALID_ARG, "%s: rows [%d, %d) do not fit kv_rows %d", fn, kv_row0, kv_row0 + tokens,
                kv_rows);
  WsLayout L;
  DMX_TRY(check_ws(fn, ws, ws_bytes, batch, tokens, 0, L));
  return enq_qkv(x_norm, w_qkv, q_norm_w, k_norm_w, batch, tokens, hidden, pos0, rope_base, q, k, v, kv_rows,
                 kv_row0, ws, L, (hipStream_t)stream);
}

int dmx_suffix_attention(const dmx_bf16* q, const dmx_bf16* k_suf, const dmx_bf16* v_suf, const dmx_bf16* k_pre,
                         const dmx_bf16* v_pre, const uint8_t* mask, int32_t batch, int32_t chunk,
                         int32_t p_bucket, dmx_bf16* ctx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dmx_suffix_attention";
  DMX_REQUIRE_PTR(q);
  DMX_REQUIRE_PTR(k_suf);
  DMX_REQUIRE_PTR(v_suf);
  DMX_REQUIRE_PTR(ctx);
  DMX_TRY(check_bt(fn, batch, chunk, DMX_MAX_CHUNK));
  DMX_TRY(check_kv(fn, k_pre, v_pre, mask, p_bucket));
  WsLayout L;
  DMX_TRY(check_ws(fn, ws, ws_bytes, batch, chunk, p_bucket, L));
  return enq_attention(q, k_suf, v_suf, k_pre, v_pre, mask, ctx, ws, L, (hipStream_t)stream);
}

int dmx_oproj_gated_residual(const dmx_bf16* ctx, const dmx_bf16* w_o, const float* mod, const dmx_bf16* residual,
                             int32_t batch, int32_t tokens, dmx_bf16* out, void* ws, size_t ws_bytes,
                             void* stream) {
  const char* fn = "dmx_oproj_gated_residual";
  DMX_REQUIRE_PTR(ctx);
  DMX_REQUIRE_PTR(w_o);
  DMX_REQUIRE_PTR(mod);
  DMX_REQUIRE_PTR(residual);
  DMX_REQUIRE_PTR(out);
  DMX_TRY(check_bt(fn, batch, tokens, 4096));
  WsLayout L;
  DMX_TRY(check_ws(fn, ws, ws_bytes, batch, tokens, 0, L));
  return enq_resid_gemm(GEMM_OPROJ, ctx, kHQ * kD, w_o, mod, residual, batch, tokens, out, ws, L,
                        (hipStream_t)stream);
}

int dmx_geglu_mlp(const dmx_bf16* x_norm2, const dmx_bf16* w_gu, const dmx_bf16* w_down, const float* mod2,
                  const dmx_bf16* residual, int32_t batch, int32_t tokens, dmx_bf16* out, void* ws,
                  size_t ws_bytes, void* stream) {
  const char* fn = "dmx_geglu_mlp";
  DMX_REQUIRE_PTR(x_norm2);
  DMX_REQUIRE_PTR(w_gu);
  DMX_REQUIRE_PTR(w_down);
  DMX_REQUIRE_PTR(mod2);
  DMX_REQUIRE_PTR(residual);
  DMX_REQUIRE_PTR(out);
  DMX_TRY(check_bt(fn, batch, tokens, 4096));
  WsLayout L;
  DMX_TRY(check_ws(fn, ws, ws_bytes, batch, tokens, 0, L));
  return enq_geglu(x_norm2, w_gu, w_down, mod2, residual, batch, tokens, out, ws, L, (hipStream_t)stream);
}

int dmx_suffix_layer_forward(const dmx_layer_weights* w, const dmx_prefix_kv* kv, const dmx_bf16* x_in,
                             const dmx_bf16* cond, const int32_t* pos0, int32_t batch, int32_t chunk,
                             dmx_bf16* x_out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dmx_suffix_layer_forward";
  DMX_TRY(check_layer_weights(fn, w));
  if (kv == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: kv struct is null", fn);
  DMX_TRY(check_kv(fn, kv->k, kv->v, kv->mask, kv->p_bucket));
  DMX_REQUIRE_PTR(x_in);
  DMX_REQUIRE_PTR(cond);
  DMX_REQUIRE_PTR(pos0);
  DMX_REQUIRE_PTR(x_out);
  DMX_TRY(check_bt(fn, batch, chunk, DMX_MAX_CHUNK));
  WsLayout L;
  DMX_TRY(check_ws(fn, ws, ws_bytes, batch, chunk, kv->p_bucket, L));
  return enq_layer(w, kv, x_in, cond, pos0, batch, chunk, x_out, ws, L, (hipStream_t)stream);
}

// ---- allocation-free layer call ---------------------------------------------
}  // extern "C"

// Scratch of dmx_suffix_layer_forward_noalloc: a file-scope device array, one
// copy on every GPU the library runs on, held until the process ends.  Its
// name is a host-side stand-in in host code, never a device address: each
// device's address is looked up once with hipGetSymbolAddress (with that
// device current) and only that address reaches kernels.
static __device__ __align__(256) unsigned char scratch[DMX_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// the device `stream` launches on (the current device for the null stream)
int stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) return hip_check(hipGetDevice(dev), "hipGetDevice");
  return hip_check(hipStreamGetDevice(s, dev), "hipStreamGetDevice");
}

// The scratch address on `dev`, looked up on the device's first call.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(DMX_ERR_UNSUPPORTED, "scratch: device %d beyond the %d supported", dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    DMX_TRY(hip_check(hipGetDevice(&cur), "hipGetDevice"));
    if (cur != dev) DMX_TRY(hip_check(hipSetDevice(dev), "hipSetDevice"));
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    DMX_TRY(hip_check(e, "hipGetSymbolAddress(scratch)"));
    if (p == nullptr) return fail(DMX_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DMX_OK;
}
}  // namespace

extern "C" {

int dmx_suffix_layer_forward_noalloc(const dmx_layer_weights* w, const dmx_prefix_kv* kv, const dmx_bf16* x_in,
                                     const dmx_bf16* cond, const int32_t* pos0, int32_t batch, int32_t chunk,
                                     dmx_bf16* x_out, void* stream) {
  const char* fn = "dmx_suffix_layer_forward_noalloc";
  DMX_TRY(check_layer_weights(fn, w));
  if (kv == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: kv struct is null", fn);
  DMX_TRY(check_kv(fn, kv->k, kv->v, kv->mask, kv->p_bucket));
  DMX_REQUIRE_PTR(x_in);
  DMX_REQUIRE_PTR(cond);
  DMX_REQUIRE_PTR(pos0);
  DMX_REQUIRE_PTR(x_out);
  DMX_TRY(check_bt(fn, batch, chunk, DMX_MAX_CHUNK));
  WsLayout L;
  if (!ws_layout(batch, chunk, kv->p_bucket, 0, L)) return fail(DMX_ERR_UNSUPPORTED, "%s: unsupported sizes", fn);
  if (L.total > (size_t)DMX_NOALLOC_SCRATCH_BYTES)
    return fail(DMX_ERR_WORKSPACE,
                "%s: batch %d, chunk %d, p_bucket %d need %zu bytes of scratch, above the fixed %d "
                "(use dmx_suffix_layer_forward with a workspace)",
                fn, batch, chunk, kv->p_bucket, L.total, DMX_NOALLOC_SCRATCH_BYTES);
  hipStream_t s = (hipStream_t)stream;
  int dev = -1;
  DMX_TRY(stream_device(s, &dev));
  void* ws = nullptr;
  DMX_TRY(scratch_on(dev, &ws));
  return enq_layer(w, kv, x_in, cond, pos0, batch, chunk, x_out, ws, L, s);
}

// ---- stack and graphs -------------------------------------------------------
struct dmx_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

static int check_stack(const char* fn, const dmx_stack_desc* d, WsLayout& L) {
  if (d == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: desc is null", fn);
  if (d->n_layers < 1 || d->n_layers > DMX_MAX_LAYERS || d->n_steps < 1 || d->layers == nullptr ||
      d->k_pre == nullptr || d->v_pre == nullptr)
    return fail(DMX_ERR_INVALID_ARG, "%s: bad layer / step description", fn);
  DMX_TRY(check_bt(fn, d->batch, d->chunk, DMX_MAX_CHUNK));
  for (int l = 0; l < d->n_layers; ++l) {
    DMX_TRY(check_layer_weights(fn, &d->layers[l]));
    DMX_TRY(check_kv(fn, d->k_pre[l], d->v_pre[l], d->mask, d->p_bucket));
  }
  DMX_REQUIRE_PTR(d->cond);
  DMX_REQUIRE_PTR(d->pos0);
  DMX_REQUIRE_PTR(d->x);
  if (d->mod_table && !aligned16(d->mod_table))
    return fail(DMX_ERR_MISALIGNED, "%s: mod_table is not 16-byte aligned", fn);
  if (d->persistent != 0 && d->persistent != 1)
    return fail(DMX_ERR_INVALID_ARG, "%s: persistent must be 0 or 1", fn);
  if (d->layer_trace && !d->persistent)
    return fail(DMX_ERR_UNSUPPORTED, "%s: layer_trace needs the persistent step kernel", fn);
  if (d->layer_trace && !aligned16(d->layer_trace))
    return fail(DMX_ERR_MISALIGNED, "%s: layer_trace is not 16-byte aligned", fn);
  if (d->persistent) {
    if (!step_supported(d->batch, d->chunk, d->p_bucket, d->n_layers))
      return fail(DMX_ERR_UNSUPPORTED,
                  "%s: the persistent step kernel runs batch 1, chunk <= 64, p_bucket <= 2048, <= %d layers", fn,
                  kStepMaxLayers);
    bool ok = false;
    DMX_TRY(hip_check(step_occupancy_ok(padded_tokens(d->chunk), &ok), "occupancy query"));
    if (!ok) return fail(DMX_ERR_UNSUPPORTED, "%s: 256 work-groups of the step kernel cannot be resident at once", fn);
  }
  return check_ws(fn, d->ws, d->ws_bytes, d->batch, d->chunk, d->p_bucket, L, d->n_layers);
}

// The persistent step kernel: the whole run of a batch-1 stack in one launch.
static int enq_stack_step(const dmx_stack_desc* d, const WsLayout& L, hipStream_t s) {
  StepArgs a;
  memset(&a, 0, sizeof a);
  for (int l = 0; l < d->n_layers; ++l) {
    const dmx_layer_weights& w = d->layers[l];
    a.L[l] = StepLayer{w.w_mod1, w.b_mod1, w.w_qkv, w.q_norm, w.k_norm, w.w_o,
                       w.w_mod2, w.b_mod2, w.w_gu,  w.w_down, d->k_pre[l], d->v_pre[l]};
  }
  a.cond = d->cond;
  a.mask = d->mask;
  a.pos0 = d->pos0;
  a.x = d->x;
  a.trace = d->layer_trace;
  a.mod_table = d->mod_table;
  a.ws = at<char>(d->ws, L.step);
  a.n_layers = d->n_layers;
  a.n_steps = d->n_steps;
  a.C = d->chunk;
  a.TP = L.TP;
  a.P = d->p_bucket;
  step_config(d->chunk, d->p_bucket, a.S, a.NS, a.kps);
  a.rope_lb = log2(10000.0);
  return hip_check(launch_step(a, s), "step kernel launch");
}

// zero the step kernel's hand-off counters and error word
static int step_sync_reset(const dmx_stack_desc* d, const WsLayout& L, hipStream_t s) {
  return hip_check(launch_fill_zero(at<char>(d->ws, L.step), StepLayout::mods, s), "step counter reset");
}

// One pass of the stack.  Per step, one launch computes the modulation
// vectors of every layer (they depend only on the step's conditioning), then
// the layers run their fused chains.
// modulation vectors of (step, layer, norm): the cached table, or the
// workspace slot the current step's vectors are computed into
static float* stack_mod(const dmx_stack_desc* d, const WsLayout& L, int st, int l, int which) {
  const size_t vec = (size_t)d->batch * 3 * kH;
  if (d->mod_table) return const_cast<float*>(d->mod_table) + (((size_t)st * d->n_layers + l) * 2 + which) * vec;
  return at<float>(d->ws, L.stack_mod) + ((size_t)l * 2 + which) * vec;
}

// the modulation vectors of every layer for step st, in one launch, into `out`
// ([n_layers][2][batch][3072])
static int enq_step_mods(const dmx_stack_desc* d, int st, float* out, hipStream_t s) {
  ModJob jobs[2 * DMX_MAX_LAYERS];
  const dmx_bf16* cond = d->cond + (size_t)st * d->batch * kH;
  const size_t vec = (size_t)d->batch * 3 * kH;
  for (int l = 0; l < d->n_layers; ++l) {
    jobs[2 * l] = ModJob{d->layers[l].w_mod1, d->layers[l].b_mod1, cond, out + (size_t)(2 * l) * vec};
    jobs[2 * l + 1] = ModJob{d->layers[l].w_mod2, d->layers[l].b_mod2, cond, out + (size_t)(2 * l + 1) * vec};
  }
  return enq_mods(jobs, 2 * d->n_layers, d->batch, s);
}

// the two modulation GEMVs of layer l at step st, into the workspace slots
static void layer_mod_jobs(const dmx_stack_desc* d, const WsLayout& L, int st, int l, ModJob jobs[2]) {
  const dmx_bf16* cond = d->cond + (size_t)st * d->batch * kH;
  jobs[0] = ModJob{d->layers[l].w_mod1, d->layers[l].b_mod1, cond, stack_mod(d, L, st, l, 0)};
  jobs[1] = ModJob{d->layers[l].w_mod2, d->layers[l].b_mod2, cond, stack_mod(d, L, st, l, 1)};
}

// Layer l of step st as the stack runs it.  Each down projection hands the
// next layer its input already scaled by that layer's 1 + scale1 when the
// next layer's modulation is known by then: inside a step always, across
// steps with a cached table.
// chained: the next step's input is this step's output (a plain stack run);
// otherwise each step's input is written anew (the sampler's in-projection).
static LayerCtx stack_layer(const dmx_stack_desc* d, const WsLayout& L, const dmx_prefix_kv* kv, int st, int l,
                            bool chained = true) {
  const float* next = nullptr;
  if (l + 1 < d->n_layers)
    next = stack_mod(d, L, st, l + 1, 0);
  else if (chained && d->mod_table && st + 1 < d->n_steps)
    next = stack_mod(d, L, st + 1, 0, 0);
  LayerCtx c{&d->layers[l], kv, d->x, d->pos0, d->batch, d->chunk, d->x, stack_mod(d, L, st, l, 0),
             stack_mod(d, L, st, l, 1), d->ws, &L, next};
  // without a table and with CUs the attention leaves idle, the next layer's
  // modulation vectors are computed by the attention launch of this one (its
  // down projection reads the next scale)
  if (!d->mod_table && attn_has_idle_cus(L.attn) && l + 1 < d->n_layers) {
    layer_mod_jobs(d, L, st, l + 1, c.side);
    c.side_n = 2;
  }
  return c;
}

// The sampler's per-step work around the stack (null: a plain stack run).
struct SamplerRun {
  const dmx_sampler_weights* w;
  const float* fmod;  // [n_steps][2048] final-norm modulation
  float* actions;     // [batch * chunk][A]
  float* traj;        // optional [n_steps][batch * chunk][A]
};

static int enq_stack(const dmx_stack_desc* d, const WsLayout& L, hipStream_t s, const SamplerRun* smp = nullptr) {
  if (d->persistent) {
    if (smp) return fail(DMX_ERR_UNSUPPORTED, "the sampler runs the stack in stage mode (persistent = 0)");
    return enq_stack_step(d, L, s);
  }
  const int rows = d->batch * d->chunk;
  for (int st = 0; st < d->n_steps; ++st) {
    // the sampler's first in-projection; later ones come with the step tail
    if (smp && st == 0)
      DMX_TRY(hip_check(launch_action_in(smp->actions, smp->w->w_in, smp->w->b_in, rows, smp->w->action_dim, d->x, s),
                        "action in-projection launch"));
    if (!d->mod_table) {
      if (attn_has_idle_cus(L.attn)) {  // layer 0's; every later layer's comes with the attention before it
        ModJob jobs[2];
        layer_mod_jobs(d, L, st, 0, jobs);
        DMX_TRY(enq_mods(jobs, 2, d->batch, s));
      } else {  // no idle CUs (batches): every layer's in one launch
        DMX_TRY(enq_step_mods(d, st, at<float>(d->ws, L.stack_mod), s));
      }
    }
    // the first layer's scaled tiled input and its row statistics: a pack
    // pass at the start of the run, and of every step whose modulation was
    // not known before it (no table); otherwise the last down projection
    // (plain stack) or the step tail (sampler) wrote them
    if (st == 0 || !d->mod_table)
      DMX_TRY(enq_pack_input(d->x, d->batch, d->chunk, stack_mod(d, L, st, 0, 0), d->ws, L, s));
    for (int l = 0; l < d->n_layers; ++l) {
      const dmx_prefix_kv kv{d->k_pre[l], d->v_pre[l], d->mask, d->p_bucket};
      DMX_TRY(enq_layer_chain(stack_layer(d, L, &kv, st, l, smp == nullptr), s));
    }
    if (smp) {
      const int A = smp->w->action_dim;
      const float dt = -1.0f / (float)d->n_steps;
      const float* fmod = smp->fmod + (size_t)st * 2 * kH;
      float* traj = smp->traj ? smp->traj + (size_t)st * rows * A : nullptr;
      if (st + 1 < d->n_steps) {
        const float* scale1 = d->mod_table ? stack_mod(d, L, st + 1, 0, 0) : nullptr;
        DMX_TRY(hip_check(launch_step_tail(d->x, fmod, smp->w->w_out, smp->w->b_out, smp->w->w_in, smp->w->b_in, rows,
                                           A, dt, smp->actions, traj, d->x, d->chunk, L.TP, scale1, 3 * kH,
                                           at<uint16_t>(d->ws, L.xp), at<float>(d->ws, L.ss_b), s),
                          "step tail launch"));
      } else {
        DMX_TRY(hip_check(launch_final_velocity(d->x, fmod, smp->w->w_out, smp->w->b_out, rows, A, dt, smp->actions,
                                                traj, s),
                          "final velocity launch"));
      }
    }
  }
  return DMX_OK;
}

// Capture what `enq` enqueues on `s` into an instantiated graph.
}  // extern "C"
template <typename F>
static int capture_graph(hipStream_t s, dmx_graph** out, F&& enq) {
  hipGraph_t g = nullptr;
  int st = hip_check(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "hipStreamBeginCapture");
  if (st == DMX_OK) {
    st = enq();
    const hipError_t ce = hipStreamEndCapture(s, &g);
    if (st == DMX_OK) st = hip_check(ce, "hipStreamEndCapture");
  }
  hipGraphExec_t e = nullptr;
  if (st == DMX_OK) st = hip_check(hipGraphInstantiate(&e, g, nullptr, nullptr, 0), "hipGraphInstantiate");
  if (st != DMX_OK) {
    if (g) (void)hipGraphDestroy(g);
    return st;
  }
  *out = new dmx_graph{g, e};
  return DMX_OK;
}
extern "C" {

int dmx_stack_forward(const dmx_stack_desc* d, void* stream) {
  WsLayout L;
  DMX_TRY(check_stack("dmx_stack_forward", d, L));
  if (d->persistent) DMX_TRY(step_sync_reset(d, L, (hipStream_t)stream));
  return enq_stack(d, L, (hipStream_t)stream);
}

int dmx_stack_sync_check(const dmx_stack_desc* d, void* stream) {
  const char* fn = "dmx_stack_sync_check";
  WsLayout L;
  DMX_TRY(check_stack(fn, d, L));
  if (!d->persistent) return DMX_OK;
  hipStream_t s = (hipStream_t)stream;
  uint32_t err = 0;
  DMX_TRY(hip_check(hipStreamSynchronize(s), "hipStreamSynchronize"));
  DMX_TRY(hip_check(hipMemcpy(&err, at<char>(d->ws, L.step) + StepLayout::err, 4, hipMemcpyDeviceToHost),
                    "error word read"));
  if (err == 0) return DMX_OK;
  DMX_TRY(step_sync_reset(d, L, s));
  DMX_TRY(hip_check(hipStreamSynchronize(s), "hipStreamSynchronize"));
  return fail(DMX_ERR_SYNC, "%s: work-group %u gave up waiting at stage %u of the run (error word 0x%08x)", fn,
              (err >> 20) & 0x7ffu, err & 0xfffffu, err);
}

int dmx_stack_stage_launch(const dmx_stack_desc* d, int32_t layer, int32_t stage, int32_t reps, void* stream) {
  const char* fn = "dmx_stack_stage_launch";
  WsLayout L;
  DMX_TRY(check_stack(fn, d, L));
  if (layer < 0 || layer >= d->n_layers) return fail(DMX_ERR_INVALID_ARG, "%s: layer %d out of range", fn, layer);
  if (stage < DMX_STAGE_MODS || stage > DMX_STAGE_DOWN)
    return fail(DMX_ERR_INVALID_ARG, "%s: unknown stage %d", fn, stage);
  if (reps < 1 || reps > 100000) return fail(DMX_ERR_INVALID_ARG, "%s: reps %d not in [1, 100000]", fn, reps);
  if (d->persistent) return fail(DMX_ERR_UNSUPPORTED, "%s: the stage kernels belong to stage mode", fn);
  hipStream_t s = (hipStream_t)stream;
  const dmx_prefix_kv kv{d->k_pre[layer], d->v_pre[layer], d->mask, d->p_bucket};
  const LayerCtx c = stack_layer(d, L, &kv, 0, layer);
  for (int r = 0; r < reps; ++r) {
    if (stage == DMX_STAGE_MODS) {  // what a step launches
      if (attn_has_idle_cus(L.attn)) {  // one layer's two (a step: layer 0's; later ones ride on the attention)
        ModJob jobs[2];
        layer_mod_jobs(d, L, 0, layer, jobs);
        DMX_TRY(enq_mods(jobs, 2, d->batch, s));
      } else {
        DMX_TRY(enq_step_mods(d, 0, at<float>(d->ws, L.stack_mod), s));
      }
    }
    else if (stage == DMX_STAGE_PACK)
      DMX_TRY(enq_pack_input(d->x, d->batch, d->chunk, stack_mod(d, L, 0, 0, 0), d->ws, L, s));
    else
      DMX_TRY(enq_layer_stage(c, stage, s));
  }
  return DMX_OK;
}

size_t dmx_stack_mod_table_bytes(int32_t n_layers, int32_t n_steps, int32_t batch) {
  if (n_layers < 1 || n_layers > DMX_MAX_LAYERS || n_steps < 1 || n_steps > 1000 || batch < 1 ||
      batch > DMX_MAX_BATCH)
    return 0;
  return (size_t)n_steps * n_layers * 2 * batch * 3 * kH * sizeof(float);
}

int dmx_stack_mod_table_fill(const dmx_stack_desc* d, float* table, void* stream) {
  const char* fn = "dmx_stack_mod_table_fill";
  WsLayout L;
  DMX_TRY(check_stack(fn, d, L));
  DMX_REQUIRE_PTR(table);
  if (d->n_steps > 1000) return fail(DMX_ERR_UNSUPPORTED, "%s: more than 1000 steps", fn);
  const size_t step = (size_t)d->n_layers * 2 * d->batch * 3 * kH;
  for (int st = 0; st < d->n_steps; ++st) DMX_TRY(enq_step_mods(d, st, table + (size_t)st * step, (hipStream_t)stream));
  return DMX_OK;
}

int dmx_stack_graph_create(const dmx_stack_desc* d, void* stream, dmx_graph** out) {
  const char* fn = "dmx_stack_graph_create";
  if (out == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: out is null", fn);
  *out = nullptr;
  if (stream == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: capture needs a non-null stream", fn);
  WsLayout L;
  DMX_TRY(check_stack(fn, d, L));
  hipStream_t s = (hipStream_t)stream;
  if (d->persistent) DMX_TRY(step_sync_reset(d, L, s));
  return capture_graph(s, out, [&] { return enq_stack(d, L, s); });
}

int dmx_graph_launch(dmx_graph* g, void* stream) {
  if (g == nullptr) return fail(DMX_ERR_INVALID_ARG, "dmx_graph_launch: graph is null");
  return hip_check(hipGraphLaunch(g->exec, (hipStream_t)stream), "hipGraphLaunch");
}

void dmx_graph_destroy(dmx_graph* g) {
  if (g == nullptr) return;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}

// ---------------------------------------------------------------------------
// Prefix (prefill) layer.  Workspace: the pieces of one layer at TP = tokens
// padded to 16 rows (tiled activations, fp32 projection outputs).
namespace {
struct PrefixLayout {
  size_t xn, raw, q, ctx, y, x1, xn2, h, pos, attn, total;
  int TP;
};

bool prefix_layout(int T, PrefixLayout& L) {
  if (T < 1 || T > DMX_MAX_PREFIX) return false;
  const size_t TP = padded_tokens(T);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return at;
  };
  L.TP = (int)TP;
  L.xn = take(TP * kPrefixHidden * 2);        // tiled rmsnorm(x; w_in)
  L.raw = take(TP * kQKV * 4);                // fp32 QKV projection
  L.q = take((size_t)T * kHQ * kD * 2);        // row-major q
  L.ctx = take(TP * kHQ * kD * 2);            // tiled attention output
  L.y = take(TP * kPrefixHidden * 4);         // fp32 O-projection / down output
  L.x1 = take(TP * kPrefixHidden * 4);        // fp32 x1
  L.xn2 = take(TP * kPrefixHidden * 2);       // tiled rmsnorm(x1; w_pre_ffn)
  L.h = take(TP * kPrefixInter * 2);          // tiled GEGLU output
  L.pos = take(16);                           // position of token 0 (zero)
  L.attn = take(prefix_attention_ws_bytes(T));  // attention split partials
  L.total = off;
  return true;
}

int check_prefix_weights(const char* fn, const dmx_prefix_layer_weights* w) {
  if (w == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: weights struct is null", fn);
  DMX_REQUIRE_PTR(w->w_in);
  DMX_REQUIRE_PTR(w->w_qkv);
  DMX_REQUIRE_PTR(w->q_norm);
  DMX_REQUIRE_PTR(w->k_norm);
  DMX_REQUIRE_PTR(w->w_o);
  DMX_REQUIRE_PTR(w->w_post_attn);
  DMX_REQUIRE_PTR(w->w_pre_ffn);
  DMX_REQUIRE_PTR(w->w_gu);
  DMX_REQUIRE_PTR(w->w_down);
  DMX_REQUIRE_PTR(w->w_post_ffn);
  return DMX_OK;
}

int enq_prefix_layer(const dmx_prefix_layer_weights* w, const dmx_bf16* x_in, const uint8_t* valid, int T,
                     dmx_bf16* kc, dmx_bf16* vc, int kv_rows, dmx_bf16* x_out, void* ws, const PrefixLayout& L,
                     hipStream_t s) {
  uint16_t* xn = at<uint16_t>(ws, L.xn);
  float* raw = at<float>(ws, L.raw);
  uint16_t* q = at<uint16_t>(ws, L.q);
  uint16_t* ctx = at<uint16_t>(ws, L.ctx);
  float* y = at<float>(ws, L.y);
  float* x1 = at<float>(ws, L.x1);
  uint16_t* xn2 = at<uint16_t>(ws, L.xn2);
  uint16_t* h = at<uint16_t>(ws, L.h);
  int32_t* pos = at<int32_t>(ws, L.pos);
  GemmArgs g = gemm_args();
  g.M = L.TP;
  g.T = T;
  g.TP = L.TP;
  // xn -> QKV (fp32) -> QK-norm + RoPE: q, and k / v into the cache
  DMX_TRY(hip_check(launch_prefix_rmsnorm(x_in, w->w_in, T, xn, s), "prefix norm launch"));
  DMX_TRY(hip_check(launch_fill_zero(pos, 16, s), "position fill"));
  GemmArgs a = g;
  gemm_config(GEMM_QKV2560, a);
  a.A = xn;
  a.W = w->w_qkv;
  a.out_f32 = raw;
  a.ldo = kQKV;
  DMX_TRY(hip_check(launch_gemm(GEMM_QKV2560, a, s), "prefix QKV launch"));
  DMX_TRY(hip_check(launch_qknorm_rope(raw, w->q_norm, w->k_norm, pos, 10000.0f, 1, T, L.TP, q, kc, vc, kv_rows, 0, s),
                    "prefix QK-norm/RoPE launch"));
  DMX_TRY(hip_check(launch_prefix_attention(q, kc, vc, valid, T, kv_rows, ctx, true, at<void>(ws, L.attn), s), "prefix attention launch"));
  // x1 = x + rmsnorm(ctx W_o^T); xn2 = rmsnorm(x1)
  a = g;
  gemm_config(GEMM_PRE_OPROJ, a);
  a.A = ctx;
  a.W = w->w_o;
  a.out_f32 = y;
  a.ldo = kPrefixHidden;
  DMX_TRY(hip_check(launch_gemm(GEMM_PRE_OPROJ, a, s), "prefix O-projection launch"));
  DMX_TRY(hip_check(launch_prefix_post_norm(y, nullptr, x_in, w->w_post_attn, w->w_pre_ffn, T, x1, xn2, nullptr, s),
                    "prefix post-attention norm launch"));
  // x_out = x1 + rmsnorm(GEGLU(xn2) W_down^T)
  a = g;
  gemm_config(GEMM_PRE_GATEUP, a);
  a.A = xn2;
  a.W = w->w_gu;
  a.out_pk = h;
  a.ldo = kPrefixInter;
  DMX_TRY(hip_check(launch_gemm(GEMM_PRE_GATEUP, a, s), "prefix gate-up launch"));
  a = g;
  gemm_config(GEMM_PRE_DOWN, a);
  a.A = h;
  a.W = w->w_down;
  a.out_f32 = y;
  a.ldo = kPrefixHidden;
  DMX_TRY(hip_check(launch_gemm(GEMM_PRE_DOWN, a, s), "prefix down launch"));
  return hip_check(launch_prefix_post_norm(y, x1, nullptr, w->w_post_ffn, nullptr, T, nullptr, nullptr, x_out, s),
                   "prefix post-MLP norm launch");
}
}  // namespace

int dmx_image_merge(const dmx_bf16* tok, const dmx_bf16* img, const int32_t* idx, int32_t tokens, int32_t n_img,
                    int32_t hidden, dmx_bf16* out, void* stream) {
  const char* fn = "dmx_image_merge";
  DMX_REQUIRE_PTR(tok);
  DMX_REQUIRE_PTR(out);
  if (idx == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: idx is null", fn);
  if (tokens < 1 || hidden < 8 || hidden % 8 != 0 || n_img < 0 || (long)tokens * hidden > (1L << 31))
    return fail(DMX_ERR_UNSUPPORTED, "%s: tokens %d / hidden %d / n_img %d unsupported", fn, tokens, hidden, n_img);
  if (n_img > 0) DMX_REQUIRE_PTR(img);
  return hip_check(launch_image_merge(tok, img, idx, tokens, n_img, hidden, out, (hipStream_t)stream),
                   "image merge launch");
}

size_t dmx_prefix_attention_workspace_bytes(int32_t tokens) {
  if (tokens < 1 || tokens > DMX_MAX_PREFIX) return 0;
  return prefix_attention_ws_bytes(tokens) + 256;
}

int dmx_prefix_attention(const dmx_bf16* q, const dmx_bf16* k, const dmx_bf16* v, const uint8_t* valid,
                         int32_t tokens, int32_t kv_rows, dmx_bf16* ctx, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dmx_prefix_attention";
  DMX_REQUIRE_PTR(q);
  DMX_REQUIRE_PTR(k);
  DMX_REQUIRE_PTR(v);
  DMX_REQUIRE_PTR(ctx);
  DMX_REQUIRE_PTR(ws);
  if (valid == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: valid is null", fn);
  if (tokens < 1 || tokens > DMX_MAX_PREFIX || kv_rows < tokens || kv_rows > DMX_MAX_PREFIX)
    return fail(DMX_ERR_UNSUPPORTED, "%s: tokens %d / kv_rows %d unsupported", fn, tokens, kv_rows);
  if (ws_bytes < prefix_attention_ws_bytes(tokens))
    return fail(DMX_ERR_WORKSPACE, "%s: workspace %zu bytes, needs %zu", fn, ws_bytes,
                prefix_attention_ws_bytes(tokens));
  return hip_check(launch_prefix_attention(q, k, v, valid, tokens, kv_rows, ctx, false, ws, (hipStream_t)stream),
                   "prefix attention launch");
}

size_t dmx_prefix_workspace_bytes(int32_t tokens) {
  PrefixLayout L;
  return prefix_layout(tokens, L) ? L.total : 0;
}

int dmx_prefix_layer_forward(const dmx_prefix_layer_weights* w, const dmx_bf16* x_in, const uint8_t* valid,
                             int32_t tokens, dmx_bf16* k_cache, dmx_bf16* v_cache, int32_t kv_rows, dmx_bf16* x_out,
                             void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dmx_prefix_layer_forward";
  DMX_TRY(check_prefix_weights(fn, w));
  DMX_REQUIRE_PTR(x_in);
  DMX_REQUIRE_PTR(k_cache);
  DMX_REQUIRE_PTR(v_cache);
  DMX_REQUIRE_PTR(x_out);
  if (valid == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: valid is null", fn);
  PrefixLayout L;
  if (!prefix_layout(tokens, L) || kv_rows < tokens || kv_rows > DMX_MAX_PREFIX)
    return fail(DMX_ERR_UNSUPPORTED, "%s: tokens %d / kv_rows %d unsupported", fn, tokens, kv_rows);
  if (x_in == x_out) return fail(DMX_ERR_INVALID_ARG, "%s: x_in and x_out overlap", fn);
  if (ws == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: ws is null", fn);
  if (!aligned16(ws)) return fail(DMX_ERR_MISALIGNED, "%s: ws is not 16-byte aligned", fn);
  if (ws_bytes < L.total)
    return fail(DMX_ERR_WORKSPACE, "%s: workspace %zu bytes, needs %zu", fn, ws_bytes, L.total);
  return enq_prefix_layer(w, x_in, valid, tokens, k_cache, v_cache, kv_rows, x_out, ws, L, (hipStream_t)stream);
}

// ---- denoise sampler ---------------------------------------------------------
// schedule buffer: final-norm modulation fp32 [n][2048], then bf16 scratch:
// temb [n][1024] and the time MLP's hidden rows [n][1024]
struct SchedLayout {
  size_t fmod, temb, h1, total;
};
static SchedLayout sched_layout(int n) {
  SchedLayout S;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  S.fmod = take((size_t)n * 2 * kH * sizeof(float));
  S.temb = take((size_t)n * kH * 2);
  S.h1 = take((size_t)n * kH * 2);
  S.total = off;
  return S;
}

size_t dmx_sampler_schedule_bytes(int32_t n_steps) {
  if (n_steps < 1 || n_steps > DMX_MAX_STEPS) return 0;
  return sched_layout(n_steps).total;
}

static int check_sampler_weights(const char* fn, const dmx_sampler_weights* w) {
  if (w == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: sampler weights struct is null", fn);
  if (w->action_dim < 16 || w->action_dim > DMX_MAX_ACTION || w->action_dim % 16 != 0)
    return fail(DMX_ERR_UNSUPPORTED, "%s: action_dim %d is not a multiple of 16 in [16, %d]", fn, w->action_dim,
                DMX_MAX_ACTION);
  DMX_REQUIRE_PTR(w->w_in);
  DMX_REQUIRE_PTR(w->b_in);
  DMX_REQUIRE_PTR(w->w_t1);
  DMX_REQUIRE_PTR(w->b_t1);
  DMX_REQUIRE_PTR(w->w_t2);
  DMX_REQUIRE_PTR(w->b_t2);
  DMX_REQUIRE_PTR(w->w_fmod);
  DMX_REQUIRE_PTR(w->b_fmod);
  DMX_REQUIRE_PTR(w->w_out);
  DMX_REQUIRE_PTR(w->b_out);
  return DMX_OK;
}

int dmx_sampler_schedule_fill(const dmx_sampler_weights* w, int32_t n_steps, int32_t batch, dmx_bf16* cond,
                              void* sched, size_t sched_bytes, void* stream) {
  const char* fn = "dmx_sampler_schedule_fill";
  DMX_TRY(check_sampler_weights(fn, w));
  if (n_steps < 1 || n_steps > DMX_MAX_STEPS)
    return fail(DMX_ERR_INVALID_ARG, "%s: n_steps %d not in [1, %d]", fn, n_steps, DMX_MAX_STEPS);
  if (batch < 1 || batch > DMX_MAX_BATCH)
    return fail(DMX_ERR_INVALID_ARG, "%s: batch %d not in [1, %d]", fn, batch, DMX_MAX_BATCH);
  DMX_REQUIRE_PTR(cond);
  DMX_REQUIRE_PTR(sched);
  const SchedLayout S = sched_layout(n_steps);
  if (sched_bytes < S.total)
    return fail(DMX_ERR_WORKSPACE, "%s: schedule buffer of %zu bytes, %zu needed", fn, sched_bytes, S.total);
  hipStream_t s = (hipStream_t)stream;
  uint16_t* temb = at<uint16_t>(sched, S.temb);
  uint16_t* h1 = at<uint16_t>(sched, S.h1);
  DMX_TRY(hip_check(launch_time_embed(n_steps, temb, s), "time embedding launch"));
  DMX_TRY(hip_check(launch_gemv_rows(w->w_t1, w->b_t1, kH, true, temb, kH, n_steps, nullptr, 0, h1, 1, s),
                    "time MLP launch"));
  DMX_TRY(hip_check(launch_gemv_rows(w->w_t2, w->b_t2, kH, true, h1, kH, n_steps, nullptr, 0, cond, batch, s),
                    "time MLP launch"));
  return hip_check(launch_gemv_rows(w->w_fmod, w->b_fmod, 2 * kH, false, cond, batch * kH, n_steps,
                                    at<float>(sched, S.fmod), 2 * kH, nullptr, 0, s),
                   "final modulation launch");
}

static int check_sampler(const char* fn, const dmx_sampler_desc* d, WsLayout& L, SamplerRun& run) {
  if (d == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: desc is null", fn);
  DMX_TRY(check_stack(fn, d->stack, L));
  DMX_TRY(check_sampler_weights(fn, d->w));
  DMX_REQUIRE_PTR(d->sched);
  DMX_REQUIRE_PTR(d->actions);
  if (d->trajectory && !aligned16(d->trajectory))
    return fail(DMX_ERR_MISALIGNED, "%s: trajectory is not 16-byte aligned", fn);
  const SchedLayout S = sched_layout(d->stack->n_steps);
  if (d->stack->n_steps > DMX_MAX_STEPS || d->sched_bytes < S.total)
    return fail(DMX_ERR_WORKSPACE, "%s: schedule buffer of %zu bytes, %zu needed for %d steps", fn, d->sched_bytes,
                S.total, d->stack->n_steps);
  run = SamplerRun{d->w, at<float>(const_cast<void*>(d->sched), S.fmod), d->actions, d->trajectory};
  return DMX_OK;
}

int dmx_sampler_forward(const dmx_sampler_desc* d, void* stream) {
  const char* fn = "dmx_sampler_forward";
  WsLayout L;
  SamplerRun run;
  DMX_TRY(check_sampler(fn, d, L, run));
  return enq_stack(d->stack, L, (hipStream_t)stream, &run);
}

int dmx_sampler_graph_create(const dmx_sampler_desc* d, void* stream, dmx_graph** out) {
  const char* fn = "dmx_sampler_graph_create";
  if (out == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: out is null", fn);
  *out = nullptr;
  if (stream == nullptr) return fail(DMX_ERR_INVALID_ARG, "%s: capture needs a non-null stream", fn);
  WsLayout L;
  SamplerRun run;
  DMX_TRY(check_sampler(fn, d, L, run));
  hipStream_t s = (hipStream_t)stream;
  return capture_graph(s, out, [&] { return enq_stack(d->stack, L, s, &run); });
}

const char* dmx_status_string(int status) {
  switch (status) {
    case DMX_OK: return "ok";
    case DMX_FALLBACK_EAGER: return "fallback: run eagerly, unbucketed";
    case DMX_ERR_INVALID_ARG: return "invalid argument";
    case DMX_ERR_BAD_BUCKETS: return "bad bucket list";
    case DMX_ERR_PREFIX_TOO_LONG: return "prefix too long";
    case DMX_ERR_UNSUPPORTED: return "unsupported size";
    case DMX_ERR_MISALIGNED: return "misaligned pointer";
    case DMX_ERR_WORKSPACE: return "workspace too small";
    case DMX_ERR_HIP: return "HIP runtime error";
    case DMX_ERR_SYNC: return "persistent kernel gave up waiting";
    default: return "unknown status";
  }
}

const char* dmx_last_error_string(void) { return g_last_error.c_str(); }

}  // extern "C"

// the error text of this thread, set by code outside this file
namespace dmx {
int set_last_error(int status, const char* msg) {
  g_last_error = msg;
  return status;
}
}  // namespace dmx
