/*
 * dmx.h -- C ABI of the MI355X (gfx950) action-expert layer library (libdmx.so).
 *
 * The library computes the forward pass of the action-expert ("suffix") layer
 * that a DM0.5-style vision-language-action model runs in every diffusion
 * denoising step, as described in:
 *   [Art]   "TensorRT+Triton+FlexAttention：OpenDM VLA快速推理加速栈深度剖析"
 *           (OpenDM DM0.5 fast-inference stack article).  §2.2 "Triton 大 Kernel"
 *           gives the shapes (suffix: hidden 1024, intermediate 4096, head_dim 256,
 *           8 query / 4 KV heads; prefix: hidden 2560) and the fused steps; §3
 *           "CUDA Graph" gives the prefix-length buckets, graph capture per bucket
 *           and the address-stable prefix KV cache.
 *   [Guide] "DM05 推理指南" (OpenDM docs/zh/dm05_inference.md), §4 "Fast Backend
 *           约束" (bucket-list rules, 1024-token cap, eager fallback), §6 (10
 *           diffusion steps by default).
 *
 * Conventions (all entry points)
 *   - dmx_bf16 is a bfloat16 bit pattern.  Tensors are contiguous, row-major, in
 *     the layouts stated per call; there are no strides.
 *   - Pointers are DEVICE pointers unless marked "host".  Every device pointer
 *     must be 16-byte aligned (DMX_ERR_MISALIGNED otherwise).
 *   - The caller owns all device memory.  Compute calls never allocate, free or
 *     synchronise; they enqueue kernels on `stream` (a hipStream_t; NULL = the
 *     null stream) and return.  The library owns only dmx_graph objects.
 *   - Every argument is validated on the host before any launch.  A failed
 *     validation launches nothing.  Status codes: 0 = OK, 1 = the explicit eager
 *     fallback of the bucket rule, negative = error.  No exception crosses the ABI.
 *     dmx_last_error_string() gives the calling thread's last error text.
 *   - There is no silent fallback to another implementation.
 *   - Weight matrices (w_mod*, w_qkv, w_o, w_gu, w_down) are passed TILED:
 *     dmx_pack_weight() converts a row-major [rows][cols] matrix once, at load
 *     time.  Shapes below are the logical row-major ones.  Bias and norm
 *     vectors stay plain.
 *   - Arithmetic: bf16 storage, fp32 accumulation.
 *   - Workspace: `ws` is caller-owned device scratch of at least
 *     dmx_workspace_bytes(batch, tokens, p_bucket) bytes (a stack:
 *     dmx_stack_workspace_bytes).  It needs no initialisation and holds nothing
 *     between calls.  Calls that share a workspace must be ordered on one stream.
 */
#ifndef DMX_H_
#define DMX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t dmx_bf16;

/* Status codes. */
#define DMX_OK 0
#define DMX_FALLBACK_EAGER 1
#define DMX_ERR_INVALID_ARG (-1)
#define DMX_ERR_BAD_BUCKETS (-2)
#define DMX_ERR_PREFIX_TOO_LONG (-3)
#define DMX_ERR_UNSUPPORTED (-4)
#define DMX_ERR_MISALIGNED (-5)
#define DMX_ERR_WORKSPACE (-6)
#define DMX_ERR_HIP (-7)
#define DMX_ERR_SYNC (-8) /* a persistent step kernel gave up waiting (see dmx_stack_sync_check) */

/* Fixed shapes of the suffix layer ([Art §2.2] shape table). */
#define DMX_HIDDEN 1024
#define DMX_INTER 4096
#define DMX_HEAD_DIM 256
#define DMX_Q_HEADS 8
#define DMX_KV_HEADS 4
#define DMX_PREFIX_HIDDEN 2560
#define DMX_MAX_CHUNK 64
#define DMX_MAX_BATCH 64
#define DMX_MAX_PREFIX 4096
#define DMX_MAX_LAYERS 64

/* ------------------------------------------------------------------------ */
/* Bucket selection ([Art §3]; [Guide §4] constraints).  Pure host code.
 *   prefix_len       current prefix length in tokens.
 *   buckets (host)   candidate bucket sizes, n entries.
 *   fast_prefix_len  the cap (1024 by default; 2048 for the single-2048-bucket
 *                    memory-demo layout).
 *   min_tokens       buckets below this (too small for the image tokens) are
 *                    skipped, i.e. never chosen.
 *   idx_out (host)   index into buckets of the chosen bucket, -1 if none.
 * Returns, checked in this order:
 *   DMX_ERR_INVALID_ARG      null pointer, prefix_len <= 0, cap <= 0,
 *                            min_tokens < 0 or n < 0;
 *   DMX_ERR_BAD_BUCKETS      list empty, not strictly increasing, or holding a
 *                            value <= 0 or above the cap;
 *   DMX_ERR_PREFIX_TOO_LONG  prefix_len > fast_prefix_len (rejected);
 *   DMX_OK                   *idx_out = smallest non-skipped bucket >= prefix_len;
 *   DMX_FALLBACK_EAGER       no such bucket: run unbucketed (P = prefix_len),
 *                            without a captured graph. */
int dmx_select_bucket(int32_t prefix_len, const int32_t* buckets, int32_t n,
                      int32_t fast_prefix_len, int32_t min_tokens, int32_t* idx_out);

/* Workspace bytes for `batch` requests of `tokens` tokens each against a prefix
 * bucket of p_bucket rows; covers every compute call below at those sizes
 * (including dmx_qkv_qknorm_rope with tokens up to 2048 at hidden 2560 when
 * asked for those sizes).  Returns 0 for unsupported sizes. */
size_t dmx_workspace_bytes(int32_t batch, int32_t tokens, int32_t p_bucket);

/* Zero-fill a workspace (enqueued on `stream`, no allocation); optional. */
int dmx_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Weight tiling.  Copies the row-major bf16 matrix w [rows][cols] into `out`
 * (rows * cols elements, not overlapping w) in the tiled layout every weight
 * argument of this library takes: 16-row x 32-column tiles of 512 elements,
 * tile (rt, ct) at element (rt * cols/32 + ct) * 512; inside a tile, the 8
 * elements w[rt*16 + l%16][ct*32 + 8*(l/16) .. +7] sit at l * 8 (l < 64): the
 * per-lane operand fragments of the gfx950 16x16x32 bf16 matrix instruction,
 * so a projection streams each weight tile as 1 KB of contiguous memory.
 * rows % 16 == 0, cols % 32 == 0, cols <= 16384.  Enqueued on `stream`. */
int dmx_pack_weight(const dmx_bf16* w, int32_t rows, int32_t cols, dmx_bf16* out, void* stream);

/* ------------------------------------------------------------------------ */
/* AdaRMS time-modulated prenorm ([Art §2.2] "Adarms 调制 prenorm").
 *   mod[b] = W_mod * cond[b] + b_mod            (fp32, [batch][3][1024]:
 *                                                 scale | shift | gate)
 *   x_norm[b][t][j] = x[b][t][j] / sqrt(mean_j x^2 + 1e-6) * (1 + scale[j]) + shift[j]
 *   x      [batch][tokens][1024] bf16     cond  [batch][1024] bf16
 *   w_mod  [3072][1024] bf16 (tiled)      b_mod [3072] bf16
 *   x_norm [batch][tokens][1024] bf16 (out)
 *   mod    [batch][3072] fp32 (out); its last third is the residual gate. */
int dmx_adarms_prenorm(const dmx_bf16* x, const dmx_bf16* cond, const dmx_bf16* w_mod,
                       const dmx_bf16* b_mod, int32_t batch, int32_t tokens,
                       dmx_bf16* x_norm, float* mod, void* stream);

/* QKV projection + per-head QK-RMSNorm + RoPE "in one go" ([Art §2.2]).
 *   qkv = x_norm * W_qkv^T, W_qkv [4096][hidden]: rows 0..2047 the 8 query
 *   heads, 2048..3071 the 4 key heads, 3072..4095 the 4 value heads (256 rows
 *   each).  q and k heads: u / sqrt(mean(u^2) + 1e-6) * (1 + w) with
 *   w = q_norm_w / k_norm_w ([256], shared by the heads), then RoPE at position
 *   pos0[b] + t: pairs (j, j + 128), angle pos * rope_base^(-j/128).
 *   x_norm [batch][tokens][hidden] bf16, hidden = 1024 (suffix) or 2560 (prefix)
 *   pos0   [batch] int32 (device)
 *   q      [batch][tokens][8][256] bf16 (out)
 *   k, v   [batch][4][kv_rows][256] bf16 (out); token t goes to row kv_row0 + t,
 *          so kv_rows = p_bucket writes straight into a prefix KV cache.
 *   Needs kv_row0 + tokens <= kv_rows. */
int dmx_qkv_qknorm_rope(const dmx_bf16* x_norm, const dmx_bf16* w_qkv,
                        const dmx_bf16* q_norm_w, const dmx_bf16* k_norm_w, int32_t batch,
                        int32_t tokens, int32_t hidden, const int32_t* pos0, float rope_base,
                        dmx_bf16* q, dmx_bf16* k, dmx_bf16* v, int32_t kv_rows,
                        int32_t kv_row0, void* ws, size_t ws_bytes, void* stream);

/* Masked GQA suffix attention ([Art §2.2]: logits read the prefix KV cache and
 * the suffix KV together under the prefix-visibility mask, online softmax,
 * value-weighted sum).  Query head h reads KV head h / 2.  Every query of a
 * request sees the prefix rows j with mask[b][j] != 0 and all `chunk` suffix
 * rows.  Masked rows are never read (their contents may be anything,
 * NaN included).  Scale 1/16.
 *   q      [batch][chunk][8][256] bf16
 *   k_suf, v_suf [batch][4][chunk][256] bf16
 *   k_pre, v_pre [batch][4][p_bucket][256] bf16 (post-norm, post-RoPE cache)
 *   mask   [batch][p_bucket] uint8, nonzero = visible (p_bucket may be 0)
 *   ctx    [batch][chunk][8][256] bf16 (out) */
int dmx_suffix_attention(const dmx_bf16* q, const dmx_bf16* k_suf, const dmx_bf16* v_suf,
                         const dmx_bf16* k_pre, const dmx_bf16* v_pre, const uint8_t* mask,
                         int32_t batch, int32_t chunk, int32_t p_bucket, dmx_bf16* ctx,
                         void* ws, size_t ws_bytes, void* stream);

/* O-projection + gated residual:
 *   out[b][t] = residual[b][t] + gate[b] * (ctx[b][t] * W_o^T),
 *   gate[b] = mod[b][2048..3071] (the third chunk of dmx_adarms_prenorm's mod).
 *   ctx [batch][tokens][2048] bf16; w_o [1024][2048] bf16 (tiled);
 *   mod [batch][3072] fp32; residual, out [batch][tokens][1024] bf16.
 *   out may alias residual. */
int dmx_oproj_gated_residual(const dmx_bf16* ctx, const dmx_bf16* w_o, const float* mod,
                             const dmx_bf16* residual, int32_t batch, int32_t tokens,
                             dmx_bf16* out, void* ws, size_t ws_bytes, void* stream);

/* GEGLU gate-up, MLP down and the second gated residual ([Art §2.2]):
 *   [a | u] = x_norm2 * W_gu^T (a: rows 0..4095, u: rows 4096..8191)
 *   h = gelu_tanh(a) * u
 *   out = residual + gate2 * (h * W_down^T),  gate2 = mod2[b][2048..3071]
 *   x_norm2 [batch][tokens][1024] bf16; w_gu [8192][1024], w_down [1024][4096] (tiled);
 *   mod2 [batch][3072] fp32; residual, out [batch][tokens][1024] bf16.
 *   out may alias residual. */
int dmx_geglu_mlp(const dmx_bf16* x_norm2, const dmx_bf16* w_gu, const dmx_bf16* w_down,
                  const float* mod2, const dmx_bf16* residual, int32_t batch, int32_t tokens,
                  dmx_bf16* out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* One whole action-expert layer ([Art §2.2], suffix path): AdaRMS -> QKV +
 * QK-norm + RoPE -> masked GQA attention over [visible prefix ; suffix] ->
 * O-projection + gated residual -> AdaRMS -> GEGLU -> down + gated residual.
 * Token t of request b sits at position pos0[b] + t. */
typedef struct dmx_layer_weights {
  const dmx_bf16* w_mod1; /* [3072][1024] */
  const dmx_bf16* b_mod1; /* [3072] */
  const dmx_bf16* w_qkv;  /* [4096][1024] */
  const dmx_bf16* q_norm; /* [256] */
  const dmx_bf16* k_norm; /* [256] */
  const dmx_bf16* w_o;    /* [1024][2048] */
  const dmx_bf16* w_mod2; /* [3072][1024] */
  const dmx_bf16* b_mod2; /* [3072] */
  const dmx_bf16* w_gu;   /* [8192][1024] */
  const dmx_bf16* w_down; /* [1024][4096] */
} dmx_layer_weights;

typedef struct dmx_prefix_kv {
  const dmx_bf16* k;    /* [batch][4][p_bucket][256] */
  const dmx_bf16* v;    /* [batch][4][p_bucket][256] */
  const uint8_t* mask;  /* [batch][p_bucket] */
  int32_t p_bucket;
} dmx_prefix_kv;

/*   w, kv (host structs holding device pointers).
 *   x_in, x_out [batch][chunk][1024] bf16 (x_out may alias x_in);
 *   cond [batch][1024] bf16; pos0 [batch] int32. */
int dmx_suffix_layer_forward(const dmx_layer_weights* w, const dmx_prefix_kv* kv,
                             const dmx_bf16* x_in, const dmx_bf16* cond,
                             const int32_t* pos0, int32_t batch, int32_t chunk,
                             dmx_bf16* x_out, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free variant of dmx_suffix_layer_forward, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments and results as
 * dmx_suffix_layer_forward (the same kernels, bit for bit), without `ws`: the
 * layer's intermediates live in a fixed scratch array of
 * DMX_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; nothing is allocated or freed by any call.
 *   Limit: the sizes must fit the scratch, i.e. dmx_workspace_bytes(batch,
 *   chunk, kv->p_bucket) <= DMX_NOALLOC_SCRATCH_BYTES (batch 1 with chunk <= 64
 *   and p_bucket <= 2048 always does); larger sizes return DMX_ERR_WORKSPACE
 *   and launch nothing.
 *   All calls on one GPU share its scratch, which keeps the last call's
 *   contents (nothing in it needs to start at zero): calls that overlap on one
 *   GPU (other streams, other threads) race and give undefined results;
 *   order them on one stream. */
#define DMX_NOALLOC_SCRATCH_BYTES (12 * 1024 * 1024)
int dmx_suffix_layer_forward_noalloc(const dmx_layer_weights* w, const dmx_prefix_kv* kv,
                                     const dmx_bf16* x_in, const dmx_bf16* cond,
                                     const int32_t* pos0, int32_t batch, int32_t chunk,
                                     dmx_bf16* x_out, void* stream);

/* ------------------------------------------------------------------------ */
/* The action-expert stack of one denoising run, replayed from a per-bucket
 * hipGraph ([Art §3]: graphs captured once per prefix bucket, replayed per
 * request, KV addresses fixed).  For step s in 0..n_steps-1 and layer l in
 * 0..n_layers-1:  x <- layer_l(x, cond[s], k_pre[l], v_pre[l], mask).
 * Everything that varies per request (x, cond, mask, pos0, KV contents) lives
 * in the fixed buffers named here: write new values into them and replay. */
typedef struct dmx_stack_desc {
  int32_t n_layers, n_steps, batch, chunk, p_bucket;
  const dmx_layer_weights* layers; /* host array [n_layers] */
  const dmx_bf16* const* k_pre;    /* host array [n_layers] of device [batch][4][p_bucket][256] */
  const dmx_bf16* const* v_pre;    /* host array [n_layers] of the same */
  const uint8_t* mask;             /* device [batch][p_bucket] */
  const dmx_bf16* cond;            /* device [n_steps][batch][1024] */
  const int32_t* pos0;             /* device [batch] */
  dmx_bf16* x;                     /* device [batch][chunk][1024], updated in place */
  void* ws;                         /* >= dmx_stack_workspace_bytes(...) */
  size_t ws_bytes;
  /* Optional device [n_steps][n_layers][2][batch][3072] fp32: the AdaRMS
   * modulation vectors W_mod * cond[s][b] + b_mod of every step, layer and
   * norm (index 0: the attention's, 1: the MLP's), as filled by
   * dmx_stack_mod_table_fill.  The conditioning of a step depends on the
   * timestep only, and the steps are fixed once a profile is captured ([Art]
   * §4), so the table is computed once per schedule and reused by every
   * request.  NULL: the vectors are computed from cond inside every step. */
  const float* mod_table;
  /* 0: every layer as its chain of stage kernels (any batch).
   * 1: the persistent step kernel (batch 1, chunk <= 64, p_bucket <= 2048,
   *    n_layers <= 32): the whole run in one launch of 256 co-resident
   *    work-groups, one per CU, each XCC of the chip owning one query head
   *    and 1/8 of the MLP, with every stage's weight slices prefetched while
   *    the stage before finishes ([Art] §2.2: one large fused kernel instead
   *    of many small ops).  Its summation order differs from the stage
   *    kernels', so the two agree to the floating-point tolerance, not bit for
   *    bit; each is deterministic.  Stages hand off through counters in the
   *    workspace with bounded waits: a run that waits past its limit (work-
   *    groups not all resident) stops early with an error word set, which
   *    dmx_stack_sync_check reports. */
  int32_t persistent;
  /* Optional device [n_steps][n_layers][batch][chunk][1024] bf16: every
   * layer's output (persistent mode only; NULL: none). */
  dmx_bf16* layer_trace;
} dmx_stack_desc;

typedef struct dmx_graph dmx_graph;

/* Workspace bytes of a stack run: dmx_workspace_bytes(batch, chunk, p_bucket)
 * plus the modulation vectors of every layer of one step.  0 if unsupported
 * (n_layers above DMX_MAX_LAYERS included). */
size_t dmx_stack_workspace_bytes(int32_t n_layers, int32_t batch, int32_t chunk, int32_t p_bucket);

/* Bytes of the modulation table of a stack (0 if unsupported). */
size_t dmx_stack_mod_table_bytes(int32_t n_layers, int32_t n_steps, int32_t batch);
/* Fill `table` (>= dmx_stack_mod_table_bytes) with the modulation vectors of
 * every step and layer of `d` from its cond buffer (d->mod_table is ignored).
 * Enqueued on `stream`. */
int dmx_stack_mod_table_fill(const dmx_stack_desc* d, float* table, void* stream);

/* Eager run of the stack (same kernels as the graph). */
int dmx_stack_forward(const dmx_stack_desc* d, void* stream);
/* Persistent mode: waits for `stream` and reads the run's error word.
 * DMX_OK, or DMX_ERR_SYNC (the work-group and stage that gave up are in
 * dmx_last_error_string) after which the hand-off counters are reset so the
 * next run starts clean.  DMX_OK without doing anything in stage mode. */
int dmx_stack_sync_check(const dmx_stack_desc* d, void* stream);
/* Capture the stack on `stream` into a graph.  *out (host).  Nothing of the
 * stack runs; in persistent mode the hand-off counters in the workspace are
 * reset on `stream` before the capture. */
int dmx_stack_graph_create(const dmx_stack_desc* d, void* stream, dmx_graph** out);
/* Replay a captured graph on `stream`. */
int dmx_graph_launch(dmx_graph* g, void* stream);
void dmx_graph_destroy(dmx_graph* g);

/* Per-kernel timing (no citation: a measurement entry point).  Enqueues
 * `reps` back-to-back launches of ONE kernel of the stack, with the arguments
 * the stack passes it for layer `layer` at step 0, so that the kernel's
 * average launch duration can be timed with events (e.g. inside a graph).
 * Run the stack once first: the kernel then reads the intermediates a real
 * pass leaves in the workspace.  A stage that writes x (DMX_STAGE_DOWN)
 * changes the stack's state; others only rewrite workspace intermediates.
 * stage: one of DMX_STAGE_*; reps in [1, 100000]. */
#define DMX_STAGE_MODS 0     /* modulation vectors of a step (one launch per step): one layer's when the
                                attention leaves CUs idle (a step launches layer 0's, each later layer's
                                come with the attention launch of the layer before it; here: layer
                                `layer`'s), else every layer's */
#define DMX_STAGE_PACK 1     /* tiled copy (scaled by 1 + scale1) + row statistics of the stack input */
#define DMX_STAGE_QKV 2      /* QKV + AdaRMS + QK-norm weights + RoPE */
#define DMX_STAGE_ATTN 3     /* masked GQA attention splits (+ the next layer's modulation vectors, on the
                                CUs the splits leave idle, when there are such and the stack has no table) */
#define DMX_STAGE_COMBINE 4  /* merge of the splits */
#define DMX_STAGE_OPROJ 5    /* O-projection + gated residual */
#define DMX_STAGE_GATEUP 6   /* AdaRMS + GEGLU gate-up */
#define DMX_STAGE_DOWN 7     /* MLP down + gated residual */
int dmx_stack_stage_launch(const dmx_stack_desc* d, int32_t layer, int32_t stage, int32_t reps, void* stream);

/* ------------------------------------------------------------------------ */
/* Prefix (prefill) side: the Gemma3-4B decoder layer of the prefix path
 * ([Art §2.2] shape table: hidden 2560, intermediate 10240, head_dim 256,
 * 8 Q / 4 KV heads; its fusion list: image features merged into the input
 * embeddings, QKV + QK-Norm + RoPE in one pass, a norm after the attention and
 * the residual), with the prefix-causal mask of [Art §2.3].  One request. */
#define DMX_PREFIX_INTER 10240

/* Image features merged into the input embeddings ([Art §2.2], prefix path):
 *   out[t] = img[idx[t]] if 0 <= idx[t] < n_img, tok[t] if idx[t] < 0, and a
 *   zero row for an index past the image rows.
 *   tok, out [tokens][hidden] bf16; img [n_img][hidden] bf16; idx [tokens]
 *   int32 (device).  hidden % 8 == 0.  Enqueued on `stream`. */
int dmx_image_merge(const dmx_bf16* tok, const dmx_bf16* img, const int32_t* idx, int32_t tokens,
                    int32_t n_img, int32_t hidden, dmx_bf16* out, void* stream);

/* Workspace bytes of dmx_prefix_attention for `tokens` tokens (0 if
 * unsupported): the partial outputs of query blocks whose keys are split. */
size_t dmx_prefix_attention_workspace_bytes(int32_t tokens);

/* Prefix attention ([Art §2.3]: the LLM attention under the prefix-causal
 * mask mapping).  Query token i of head h reads key token j of KV head h / 2
 * exactly when j <= i and valid[j] != 0 (bucket padding is not valid);
 * softmax of q.k / 16 over that set; a query with no such key gets zeros.
 *   q   [tokens][8][256] bf16 (normed and rotated, as dmx_qkv_qknorm_rope
 *       writes it)
 *   k, v [4][kv_rows][256] bf16: the layer's cache, tokens at rows 0 ..
 *       tokens - 1 (kv_rows >= tokens); invalid rows are never read
 *   valid [tokens] uint8 (device)
 *   ctx [tokens][8][256] bf16 (out).  tokens <= DMX_MAX_PREFIX.
 *   ws: >= dmx_prefix_attention_workspace_bytes(tokens) bytes (caller-owned,
 *   no initialisation). */
int dmx_prefix_attention(const dmx_bf16* q, const dmx_bf16* k, const dmx_bf16* v, const uint8_t* valid,
                         int32_t tokens, int32_t kv_rows, dmx_bf16* ctx, void* ws, size_t ws_bytes, void* stream);

/* Weights of one prefix layer (device pointers; matrices tiled by
 * dmx_pack_weight; norm weights use the (1 + w) convention). */
typedef struct {
  const dmx_bf16* w_in;         /* [2560] pre-attention norm */
  const dmx_bf16* w_qkv;        /* [4096][2560] */
  const dmx_bf16* q_norm;       /* [256] */
  const dmx_bf16* k_norm;       /* [256] */
  const dmx_bf16* w_o;          /* [2560][2048] */
  const dmx_bf16* w_post_attn;  /* [2560] norm after the attention */
  const dmx_bf16* w_pre_ffn;    /* [2560] norm before the MLP */
  const dmx_bf16* w_gu;         /* [20480][2560]: gate rows, then up rows */
  const dmx_bf16* w_down;       /* [2560][10240] */
  const dmx_bf16* w_post_ffn;   /* [2560] norm after the MLP */
} dmx_prefix_layer_weights;

/* Workspace bytes of dmx_prefix_layer_forward for `tokens` tokens (0 if
 * unsupported). */
size_t dmx_prefix_workspace_bytes(int32_t tokens);

/* One prefix decoder layer (reading of the pages' pieces in Gemma3 order):
 *   xn  = rmsnorm(x_in; w_in)
 *   q, k, v = QKV(xn) + QK-norm + RoPE at positions 0 .. tokens - 1; k and v
 *             go to rows 0 .. tokens - 1 of k_cache / v_cache [4][kv_rows][256]
 *   ctx = prefix attention (above) with `valid`
 *   x1  = x_in + rmsnorm(ctx W_o^T; w_post_attn)
 *   x_out = x1 + rmsnorm(GEGLU(rmsnorm(x1; w_pre_ffn)) W_down^T; w_post_ffn),
 *           GEGLU(u) = gelu_tanh(u W_g^T) * (u W_up^T)
 *   x_in, x_out [tokens][2560] bf16 (may not overlap); valid [tokens] uint8.
 *   rmsnorm(u; w) = u / sqrt(mean u^2 + 1e-6) * (1 + w).
 *   1 <= tokens <= kv_rows <= DMX_MAX_PREFIX.  All launches on `stream`. */
int dmx_prefix_layer_forward(const dmx_prefix_layer_weights* w, const dmx_bf16* x_in, const uint8_t* valid,
                             int32_t tokens, dmx_bf16* k_cache, dmx_bf16* v_cache, int32_t kv_rows,
                             dmx_bf16* x_out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Denoise sampler around the action-expert stack.  The pages decode the
 * action chunk by diffusion over a fixed number of steps ([Art §1], [Art §4];
 * [Guide §2]: the diffusion step count, fixed once graphs are captured) and
 * give no formula for the sampler; the readings implemented:
 *   t_k   = 1 - k / n_steps, k = 0 .. n_steps - 1 (noise at t = 1)
 *   temb  = [sin(1000 t w_i) | cos(1000 t w_i)], w_i = 10000^(-i / 512)
 *   cond  = swish(W_t2 swish(W_t1 temb + b_t1) + b_t2), swish(z) = z / (1 + e^-z)
 *   x     = W_in a + b_in for each chunk token (the stack's input)
 *   x    <- the stack's layers with cond(t_k)
 *   xf    = x / sqrt(mean x^2 + 1e-6) * (1 + scale) + shift,
 *           [scale | shift] = W_fmod cond + b_fmod
 *   v     = W_out xf + b_out;   a <- a - v / n_steps   (Euler step)
 * Action dimension A: a multiple of 16 in [16, DMX_MAX_ACTION]. */
#define DMX_MAX_ACTION 128
#define DMX_MAX_STEPS 1000

typedef struct dmx_sampler_weights {
  int32_t action_dim;      /* A */
  const dmx_bf16* w_in;    /* [1024][A] row-major */
  const dmx_bf16* b_in;    /* [1024] */
  const dmx_bf16* w_t1;    /* [1024][1024], tiled (dmx_pack_weight) */
  const dmx_bf16* b_t1;    /* [1024] */
  const dmx_bf16* w_t2;    /* [1024][1024], tiled */
  const dmx_bf16* b_t2;    /* [1024] */
  const dmx_bf16* w_fmod;  /* [2048][1024], tiled: scale rows, then shift rows */
  const dmx_bf16* b_fmod;  /* [2048] */
  const dmx_bf16* w_out;   /* [A][1024] row-major */
  const dmx_bf16* b_out;   /* [A] */
} dmx_sampler_weights;

/* Bytes of a schedule buffer for n_steps steps (0 if unsupported). */
size_t dmx_sampler_schedule_bytes(int32_t n_steps);

/* The step-only part of a schedule, computed once per (weights, n_steps):
 * cond[k][b] = cond(t_k) for every request b (bf16 [n_steps][batch][1024],
 * the stack's conditioning buffer), and in `sched` the final norm's
 * modulation of every step plus scratch.  Enqueued on `stream`. */
int dmx_sampler_schedule_fill(const dmx_sampler_weights* w, int32_t n_steps, int32_t batch, dmx_bf16* cond,
                              void* sched, size_t sched_bytes, void* stream);

/* A denoising run: the stack (its cond holding the schedule's conditioning,
 * n_steps equal to the schedule's; its x buffer receives each step's expert
 * input and output) bracketed per step by the action in-projection and the
 * final norm + out-projection + Euler update. */
typedef struct dmx_sampler_desc {
  const dmx_stack_desc* stack;
  const dmx_sampler_weights* w;
  const void* sched;      /* filled by dmx_sampler_schedule_fill for stack->n_steps */
  size_t sched_bytes;
  float* actions;         /* device [batch][chunk][A] fp32: the noise on entry, the denoised chunk after */
  float* trajectory;      /* optional device [n_steps][batch][chunk][A]: actions after each step */
} dmx_sampler_desc;

/* Eager run (every kernel enqueued on `stream`). */
int dmx_sampler_forward(const dmx_sampler_desc* d, void* stream);
/* Capture the run on `stream` into a graph (nothing runs); replay with
 * dmx_graph_launch after writing new noise / KV / mask into the buffers. */
int dmx_sampler_graph_create(const dmx_sampler_desc* d, void* stream, dmx_graph** out);

/* ------------------------------------------------------------------------ */
/* Lazily captured graph profiles ([Art §5] table, default backend): a
 * request's prefix length is rounded up to a multiple of 16 tokens, and each
 * such bucket (with the run's batch, chunk, steps and layers) is a profile.
 * A profile's first call runs eager, its second call is captured into a graph
 * (and runs), later calls replay that graph.  At most `capacity` (1 ..
 * DMX_LAZY_MAX_PROFILES) profiles hold graphs.  A new profile beyond that
 * either replaces the least recently used one (evict = 1) or runs eager
 * without becoming a profile (evict = 0).  A profile whose buffers changed
 * (another address in its descriptor) starts again from its first call. */
#define DMX_LAZY_GRANULE 16
#define DMX_LAZY_MAX_PROFILES 8
#define DMX_ACTION_EAGER 0
#define DMX_ACTION_CAPTURE 1
#define DMX_ACTION_REPLAY 2

/* Bucket of a prefix length: 16 * ceil(prefix_len / 16).  Negative status for
 * prefix_len < 1 (DMX_ERR_INVALID_ARG) or above max_len
 * (DMX_ERR_PREFIX_TOO_LONG). */
int32_t dmx_lazy_bucket(int32_t prefix_len, int32_t max_len);

typedef struct dmx_profile_cache dmx_profile_cache;
int dmx_profile_cache_create(int32_t capacity, int32_t evict, dmx_profile_cache** out);
void dmx_profile_cache_destroy(dmx_profile_cache* c);

/* The policy alone (host only, enqueues nothing): the action for a call of
 * profile `key` whose buffers hash to `fingerprint`, and the key of the
 * profile it displaces (-1 if none; that profile's graph is destroyed).
 * Updates the cache's bookkeeping exactly as a run would. */
int dmx_profile_cache_plan(dmx_profile_cache* c, int64_t key, uint64_t fingerprint, int32_t* action,
                           int64_t* evicted);
/* Number of profiles held, and their keys from least to most recently used
 * (keys: host array of at least DMX_LAZY_MAX_PROFILES, may be NULL). */
int dmx_profile_cache_keys(const dmx_profile_cache* c, int64_t* keys);

/* One denoising run of `d` through the cache: its profile key is (p_bucket,
 * batch, chunk, n_steps, n_layers), its fingerprint the descriptor's buffer
 * addresses.  *action (host, optional) receives what was done.  Capture and
 * replay use `stream`, which must not be the null stream. */
int dmx_profile_cache_run_sampler(dmx_profile_cache* c, const dmx_sampler_desc* d, void* stream, int32_t* action);

/* ------------------------------------------------------------------------ */
const char* dmx_status_string(int status);
const char* dmx_last_error_string(void);

#ifdef __cplusplus
}
#endif
#endif /* DMX_H_ */
