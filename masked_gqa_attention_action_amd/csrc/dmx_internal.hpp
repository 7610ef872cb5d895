// Internal launch interface between the C ABI layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace dmx {

// Epilogues.  RESID variants: out = resid + gate[b] * y with the residual and
// output stored as bf16 (B) or fp32 (F): RESID_BB, RESID_BF (bf16 in, fp32
// out), RESID_FB (fp32 in, bf16 out).
// EPI_QKV: tile = 16 features j.. of a head's first half + their rotation
// partners j+128..; stores rope((1 + w) * x) (q, k heads) or x (v heads) as
// tiled fp32 plus per-(row, tile) sums of squares of x.
enum Epi { EPI_F32 = 0, EPI_RESID_BB = 2, EPI_GEGLU = 3, EPI_RESID_BF = 4, EPI_RESID_FB = 5, EPI_QKV = 6 };

// A-operand sources of the GEMM (see dmx_gemm.hip).
enum ASrc { A_GLOBAL = 0, A_MODPRE = 2 };

// Skinny GEMM y[m][n] = sum_k A[m][k] * W[n][k] with a fused epilogue.  A and W
// are tiled (dmx_tiles.hpp); rows are tiled rows (request b, token t at
// b * TP + t).  Row-major [batch][tokens] tensors (resid / out_bf16 of the
// bf16-residual epilogues) are indexed by b * T + t; fp32 intermediates and
// out_f32 by the tiled row.
struct GemmArgs {
  const uint16_t* A;  // tiled bf16 [M][K]; A_MODPRE: bf16(x * (1 + scale))
  const float* nmod;  // A_MODPRE: modulation [B][3][1024] (scale | shift | gate)
  const float* ss_in; // A_MODPRE: row sums of squares of x, [M][ss_in_n] partials
  int ss_in_n;        //   a multiple of 4 up to 64
  float* ss_out;      // EPI_RESID_BF / _FB: optional [M][ss_out_n] partials, one
  int ss_out_n;       //   per N-tile of 16 features (ntiles == ss_out_n)
  const float* xs_scale;  // EPI_RESID_BF: out_pk = bf16(out * (1 + xs_scale[b][n]));
                          // EPI_RESID_FB: out_pk = bf16(bf16(out) * (1 + xs_scale[b][n]));
                          //   row b at xs_scale + b * gate_stride (null: no scaling)
  const uint16_t* W;  // tiled weights [N][K]
  int M, K;           // M = B * TP tiled rows
  int T, TP;          // tokens per request and their padded count
  int ntiles;         // grid.x = ntiles work-groups
  int tile0;          // k_gemm_lds: the launch's first output tile (its grid covers tiles tile0 ..)
  int xcd_strip;      // k_gemm_lds: blocks dealt to XCDs in strips of this many column blocks (0: plain grid)
  int wtile_up;       // GEGLU: weight tile of the first "up" feature
  float* out_f32;     // EPI_F32 / EPI_RESID_BF output [M][ldo]
  uint16_t* out_bf16; // EPI_RESID_BB / EPI_RESID_FB row-major output
  uint16_t* out_pk;   // tiled bf16 output (GEGLU h, RESID_BF x1s, RESID_FB copy)
  int ldo;            // features per output row
  const float* gate;       // EPI_RESID_*: gate of request b at gate + b * gate_stride
  int gate_stride;
  const uint16_t* resid;   // EPI_RESID_B*: bf16 residual, row-major
  const float* resid_f32;  // EPI_RESID_FB: fp32 residual [M][ldo]
  // EPI_QKV: the k heads go to out_f32, tiled fp32 [M][4096] (only the k
  // heads' columns written); the q and v heads to out_pk, tiled bf16
  // [M][kQVB] (q heads at columns 0 .. 2047, v heads after them);
  // ss_q [M][kQkvTiles] sums of squares
  const uint16_t *qn_w, *kn_w;  // (1 + w) weights of the q / k heads, [256]
  const int32_t* pos0;          // token t of request b at position pos0[b] + t
  float rope_base;
  float* ss_q;
};
constexpr int kQkvTiles = 96;  // 32-feature tiles of the 12 q / k heads (8 per head)
constexpr int kQVB = (kHQ + kHK) * kD;  // columns of the tiled bf16 q + v heads

// Gemm shape presets (host picks one per projection).
enum GemmKind {
  GEMM_QKV1024 = 1,         // N = 4096, K = 1024, fp32 out, A given
  GEMM_QKV1024_MODPRE = 10, // rotation-pair tiles, AdaRMS fused (A = bf16(x * (1 + scale))), EPI_QKV
  GEMM_QKV2560 = 3,         // N = 4096, K = 2560, fp32 out
  GEMM_OPROJ = 4,           // N = 1024, K = 2048, gated residual (bf16 -> bf16)
  GEMM_OPROJ_F32 = 5,       // as GEMM_OPROJ, fp32 output (layer-internal residual)
  GEMM_GATEUP = 6,          // N = 2 x 4096, K = 1024, GEGLU, A given
  GEMM_GATEUP_MOD = 7,      // as above with the AdaRMS prenorm of x1 fused (A = bf16(x1 * (1 + scale)))
  GEMM_DOWN = 8,            // N = 1024, K = 4096, gated residual (bf16 -> bf16)
  GEMM_DOWN_F32RES = 9,     // as GEMM_DOWN, fp32 residual input
  // prefix (prefill) layer, hidden 2560, intermediate 10240; any row count
  // runs on the large-M schedule
  GEMM_PRE_OPROJ = 20,      // N = 2560, K = 2048, fp32 out
  GEMM_PRE_GATEUP = 21,     // N = 2 x 10240, K = 2560, GEGLU (h tiled bf16)
  GEMM_PRE_DOWN = 22,       // N = 2560, K = 10240, fp32 out
};
int gemm_config(GemmKind kind, GemmArgs& a);
hipError_t launch_gemm(GemmKind kind, const GemmArgs& a, hipStream_t s);

// Row-major bf16 [B][T][K] -> tiled [B*TP][K]; with ss (K = 1024) also the 64
// row sums of squares of 16 columns per row, the values and summation order
// of the GEMM epilogues.
constexpr int kSsParts = 1024 / 16;
hipError_t launch_pack_rows(const uint16_t* x, int B, int T, int TP, int K, uint16_t* out, float* ss,
                            hipStream_t s, const float* scale = nullptr, int scale_stride = 0);

// Several modulation GEMVs in one launch: out_j[b] = W_j cond_j[b] + bias_j.
struct ModJob {
  const uint16_t* w;     // [3072][1024]
  const uint16_t* bias;  // [3072]
  const uint16_t* cond;  // [B][1024]
  float* out;            // [B][3072]
};
constexpr int kMaxModJobs = 40;
struct ModBatch {
  ModJob job[kMaxModJobs];
  int n, B;
};
hipError_t launch_mod_multi(const ModBatch& mb, hipStream_t s);

hipError_t launch_adarms_norm(const uint16_t* x, const float* mod, int M, int T, uint16_t* xn,
                              hipStream_t s);

// raw: fp32 QKV projection [B*TP][4096] (tiled rows); q / k / v row-major
hipError_t launch_qknorm_rope(const float* raw, const uint16_t* qn_w, const uint16_t* kn_w,
                              const int32_t* pos0, float base, int B, int T, int TP, uint16_t* q,
                              uint16_t* k, uint16_t* v, int kv_rows, int kv_row0, hipStream_t s);

struct AttnArgs {
  const uint16_t *q, *ks, *vs, *kp, *vp;
  // fused path: when y != nullptr, q / ks / vs are ignored and built from the
  // QKV epilogue's output: y tiled fp32 [B*TP][4096] (rope((1 + w) * x) for
  // the k heads), qvb tiled bf16 [B*TP][kQVB] (the same for the q heads, x for
  // the v heads) and ss_q [B*TP][96] (8 sums of squares of x per q / k head):
  // k = y / sqrt(mean x^2 + eps), and the q heads' 1 / sqrt(mean x^2 + eps)
  // scales the logits.
  const float* y;
  const float* ss_q;
  const uint16_t* qvb;
  const uint8_t* mask;
  int B, C, P;
  int TP;       // padded chunk (tiled rows per request)
  int ctx_tiled;  // 1: ctx is written tiled [B*TP][2048]; 0: row-major [B][C][2048]
  int S;        // prefix splits; splits S .. S+NS-1 hold the suffix keys
  int NS;       // suffix splits (32 keys each)
  int kps;      // prefix keys per split (multiple of 32)
  int R16;      // stacked query rows (2 * C) rounded up to 16
  // optional work for the CUs the splits leave idle: the modulation GEMVs
  // side[0 .. side_n) for side_B requests, in 16-feature units spread over
  // the extra work-groups (blocks attn_grid .. of the partial launch)
  ModJob side[2];
  int side_n, side_B;
  int attn_grid;  // work-groups of the splits (set by the launch)
  uint16_t* part_o;  // [B][HK][S + NS][R16 / 16][16 dim tiles][16 rows][4][4] bf16, normalised partial
                     // outputs (dims 16t + 4q .. +3 of row r at [t][r][q]); padded rows never written
  float* part_ml;    // [B][HK][S + NS][R16][2] running max (log2 domain) and sum
};
constexpr int kAttnKps = 64;  // prefix keys per attention split (32 .. 128, multiple of 32)
void attn_config(int B, int C, int P, AttnArgs& a);
hipError_t launch_attention(const AttnArgs& a, uint16_t* ctx, hipStream_t s);  // partial + combine
hipError_t launch_attn_partial(const AttnArgs& a, hipStream_t s);
// true when the split launch leaves CUs idle (one query head per work-group)
bool attn_has_idle_cus(const AttnArgs& a);
hipError_t launch_attn_combine(const AttnArgs& a, uint16_t* ctx, hipStream_t s);
// prefix (prefill) layer pieces, hidden kPrefixHidden, one request
constexpr int kPrefixHidden = 2560, kPrefixInter = 10240;
hipError_t launch_prefix_rmsnorm(const uint16_t* x, const uint16_t* w, int T, uint16_t* out, hipStream_t s);
hipError_t launch_prefix_post_norm(const float* y, const float* resid_f32, const uint16_t* resid_bf16,
                                   const uint16_t* w_post, const uint16_t* w_next, int T, float* x1_out,
                                   uint16_t* xn_tiled, uint16_t* out_bf16, hipStream_t s);
hipError_t launch_image_merge(const uint16_t* tok, const uint16_t* img, const int32_t* idx, int T, int n_img,
                              int hidden, uint16_t* out, hipStream_t s);
// prefix attention of the prefill: q row-major [T][8][256]; k, v [4][kv_rows][256];
// valid [T]; ctx tiled [TP][2048] (ctx_tiled) or row-major [T][8][256]; ws of
// prefix_attention_ws_bytes(T) bytes for the split partials
// split sizes (key blocks of 32 per work item) the launch chooses among; the
// workspace is sized for the smallest
constexpr int kPrefixAttnSplits[4] = {24, 20, 16, 12};
int prefix_attn_items(int T, int sb);
size_t prefix_attention_ws_bytes(int T);
hipError_t launch_prefix_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint8_t* valid,
                                   int T, int kv_rows, uint16_t* ctx, bool ctx_tiled, void* ws, hipStream_t s);

// denoise sampler pieces
constexpr int kMaxActionDim = 128;
hipError_t launch_time_embed(int n_steps, uint16_t* temb, hipStream_t s);
// y[r] = act(W x[r] + bias), W tiled [N][1024]; outputs as k_gemv_rows documents
hipError_t launch_gemv_rows(const uint16_t* W, const uint16_t* bias, int N, bool swish, const uint16_t* x,
                            int x_stride, int R, float* out_f32, int ldo, uint16_t* out_bf16, int rep, hipStream_t s);
hipError_t launch_action_in(const float* a, const uint16_t* w_in, const uint16_t* b_in, int rows, int A, uint16_t* x,
                            hipStream_t s);
hipError_t launch_final_velocity(const uint16_t* x, const float* fmod, const uint16_t* w_out, const uint16_t* b_out,
                                 int rows, int A, float dt, float* a, float* traj, hipStream_t s);
// final_velocity of one step + action_in of the next (+ its input pack when
// scale1 is given): rows = B * T, the packed input at tiled rows b * TP + t
hipError_t launch_step_tail(const uint16_t* x, const float* fmod, const uint16_t* w_out, const uint16_t* b_out,
                            const uint16_t* w_in, const uint16_t* b_in, int rows, int A, float dt, float* a,
                            float* traj, uint16_t* x_next, int T, int TP, const float* scale1, int scale_stride,
                            uint16_t* xp, float* ss, hipStream_t s);

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// ---- persistent denoise-step kernel (batch 1; dmx_step.hip) ----------------
constexpr int kStepMaxLayers = 32;
constexpr int kStepMaxNB = 3;       // 32-key blocks per attention split
constexpr int kStepMaxSplits = 32;  // attention splits per head (one per work-group of an XCC)
constexpr int kStepModSlots = 4;    // ring of modulation vectors (linear layer index % 4)
struct StepLayer {
  const uint16_t *w_mod1, *b_mod1, *w_qkv, *q_norm, *k_norm, *w_o, *w_mod2, *b_mod2, *w_gu, *w_down, *k_pre, *v_pre;
};
// Byte layout of the step kernel's workspace for TP padded chunk rows (a
// multiple of 16 up to 64), 256-byte aligned pieces.
constexpr uint32_t step_align(uint32_t v) { return (v + 255u) & ~255u; }
struct StepLayout {
  static constexpr uint32_t al(uint32_t v) { return step_align(v); }
  static constexpr uint32_t prog = 0;                                  // [256] counters, 128 B apart
  static constexpr uint32_t err = prog + 256u * 128u;                  // error word
  static constexpr uint32_t mods = err + 256u;                         // [kStepModSlots][2][3072] fp32
  static constexpr uint32_t ypart = step_align(mods + kStepModSlots * 2u * 3072u * 4u);  // [8][4][64][64][4] fp32
  static constexpr uint32_t y2part = ypart + 8u * 4u * 64u * 256u * 4u;
  static constexpr uint32_t xcc = y2part + 8u * 4u * 64u * 256u * 4u;  // per-XCC buffers from here
  // per-XCC buffers (offsets within an XCC's region)
  static constexpr uint32_t xs(int) { return 0; }                               // tiled bf16 [TP][1024]
  static constexpr uint32_t ssx(int TP) { return al(xs(TP) + TP * 1024u * 2u); }  // fp32 [TP][32]
  static constexpr uint32_t qb(int TP) { return al(ssx(TP) + TP * 32u * 4u); }    // tiled bf16 [TP][256]
  static constexpr uint32_t vb(int TP) { return al(qb(TP) + TP * 256u * 2u); }    // tiled bf16 [TP][256]
  static constexpr uint32_t kf(int TP) { return al(vb(TP) + TP * 256u * 2u); }    // tiled fp32 [TP][256]
  static constexpr uint32_t ssq(int TP) { return al(kf(TP) + TP * 256u * 4u); }   // fp32 [TP][16]
  static constexpr uint32_t po(int TP) { return al(ssq(TP) + TP * 16u * 4u); }    // bf16 [32][4][16][256]
  static constexpr uint32_t pml(int TP) { return al(po(TP) + kStepMaxSplits * 4u * 16u * 256u * 2u); }  // fp32 [32][64][2]
  static constexpr uint32_t ctx(int TP) { return al(pml(TP) + kStepMaxSplits * 64u * 2u * 4u); }  // tiled bf16 [TP][256]
  static constexpr uint32_t x1s(int TP) { return al(ctx(TP) + TP * 256u * 2u); }  // tiled bf16 [TP][1024]
  static constexpr uint32_t ss1(int TP) { return al(x1s(TP) + TP * 1024u * 2u); } // fp32 [TP][32]
  static constexpr uint32_t h(int TP) { return al(ss1(TP) + TP * 32u * 4u); }     // tiled bf16 [TP][512]
  static constexpr uint32_t xcc_stride(int TP) { return al(h(TP) + TP * 512u * 2u); }
  static constexpr size_t bytes(int TP) { return (size_t)xcc + 8u * (size_t)xcc_stride(TP); }
};
struct StepArgs {
  StepLayer L[kStepMaxLayers];
  const uint16_t* cond;      // [n_steps][1024]
  const uint8_t* mask;       // [P]
  const int32_t* pos0;       // [1]
  uint16_t* x;               // [C][1024]: the input, replaced by the output
  uint16_t* trace;           // optional [n_steps][n_layers][C][1024]: every layer's output
  const float* mod_table;    // optional [n_steps][n_layers][2][3072]
  char* ws;                  // the workspace (StepLayout)
  int n_layers, n_steps, C, TP, P, S, NS, kps;
  double rope_lb;            // log2 of the RoPE base
};
// attention split shape of the step kernel for chunk C and prefix P
void step_config(int C, int P, int& S, int& NS, int& kps);
bool step_supported(int B, int C, int P, int n_layers);
hipError_t launch_step(const StepArgs& a, hipStream_t s);
// whether 256 work-groups of the step kernel can be resident at once
hipError_t step_occupancy_ok(int TP, bool* ok);


}  // namespace dmx
