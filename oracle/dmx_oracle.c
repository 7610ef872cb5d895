/*
 * dmx oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation (float64, nested loops)
 * of the action-expert ("suffix") layer forward that the HIP library computes,
 * of the prefix (prefill) decoder layer that writes the KV cache it reads, and
 * of the denoise sampler around the layer stack (time conditioning, action
 * projections, Euler steps; readings throughout, as the pages give no formula:
 * parity of those readings is unpinned against the pages and pinned by
 * closed forms and library routines only).
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library.  It shares no code, header, table or constant with
 * the HIP path, and never calls into it.
 *
 * Sources (cited by title and section; the reader has the pages):
 *   [Art]   "TensorRT+Triton+FlexAttention：OpenDM VLA快速推理加速栈深度剖析"
 *           (OpenDM DM0.5 fast-inference stack article).
 *           §2.2 "Triton 大 Kernel" holds the shape table (suffix: hidden 1024,
 *           intermediate 4096, head_dim 256, 8 Q / 4 KV heads) and the list of
 *           fused steps; §3 "CUDA Graph" holds the prefix-length buckets.
 *   [Guide] "DM05 推理指南" (OpenDM docs/zh/dm05_inference.md),
 *           §4 "Fast Backend 约束" (bucket-list rules, 1024-token cap, eager
 *           fallback).
 *
 * Where the pages only name a step, the reading taken is stated at the
 * function.  Every reading is listed in the repository's design notes.
 *
 * Layouts: row-major, contiguous.  Weights are [out][in].
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Status codes of the bucket rule (same meaning as the library's, written
 * independently here). */
#define ORC_OK 0
#define ORC_FALLBACK_EAGER 1
#define ORC_ERR_INVALID_ARG (-1)
#define ORC_ERR_BAD_BUCKETS (-2)
#define ORC_ERR_PREFIX_TOO_LONG (-3)

int orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/*
 * Prefix-length bucket rule.  [Art §3]: buckets 576/704/768/896/1024 by
 * default (a single 2048 bucket with fast-prefix-len 2048 for the memory
 * demo); the bucket is chosen by the current prefix length; a prefix longer
 * than the largest bucket but within fast_prefix_len takes the slower eager
 * path.  [Guide §4 constraints]: the list must be non-empty, strictly
 * increasing and not above the cap; buckets too small for the image tokens
 * are skipped; a prefix above the cap is rejected.
 *
 * Reading: the chosen bucket is the smallest non-skipped bucket >= len
 * ("skipped" = below min_tokens).  Checks run in the order
 * arguments -> list -> cap -> choice.
 */
int orc_select_bucket(int32_t prefix_len, const int32_t* buckets, int32_t n,
                      int32_t cap, int32_t min_tokens, int32_t* idx_out) {
  int32_t i;
  if (idx_out) *idx_out = -1;
  if (buckets == NULL || idx_out == NULL || prefix_len <= 0 || cap <= 0 ||
      min_tokens < 0 || n < 0)
    return ORC_ERR_INVALID_ARG;
  if (n == 0) return ORC_ERR_BAD_BUCKETS;
  for (i = 0; i < n; ++i) {
    if (buckets[i] <= 0 || buckets[i] > cap) return ORC_ERR_BAD_BUCKETS;
    if (i > 0 && buckets[i] <= buckets[i - 1]) return ORC_ERR_BAD_BUCKETS;
  }
  if (prefix_len > cap) return ORC_ERR_PREFIX_TOO_LONG;
  for (i = 0; i < n; ++i) {
    if (buckets[i] < min_tokens) continue; /* skipped: too small for the images */
    if (buckets[i] >= prefix_len) {
      *idx_out = i;
      return ORC_OK;
    }
  }
  return ORC_FALLBACK_EAGER;
}

/* y[t][o] = sum_k a[t][k] * w[o][k], k ascending.  A plain matrix product. */
void orc_linear(const double* a, const double* w, int T, int K, int N, double* y) {
  long tn;
#pragma omp parallel for schedule(static)
  for (tn = 0; tn < (long)T * N; ++tn) {
    long t = tn / N, o = tn % N;
    const double* ar = a + t * (long)K;
    const double* wr = w + o * (long)K;
    double s = 0.0;
    int k;
    for (k = 0; k < K; ++k) s += ar[k] * wr[k];
    y[tn] = s;
  }
}

/*
 * AdaRMS time-modulated prenorm ([Art §2.2] "Adarms 调制 prenorm").
 * Reading: one affine modulation of the conditioning vector,
 *   m = W_mod * cond + b_mod,  m = [scale | shift | gate]  (each H long),
 * then an RMS norm of each token row with no separate learned weight,
 *   xn[t][j] = x[t][j] / sqrt(mean_j x[t][j]^2 + eps) * (1 + scale[j]) + shift[j].
 * mod_out receives m (3H values); gate is its last third.
 */
void orc_adarms(const double* x, const double* cond, const double* w_mod,
                const double* b_mod, int T, int H, double eps, double* xn_out,
                double* mod_out) {
  int t, j;
  orc_linear(cond, w_mod, 1, H, 3 * H, mod_out);
  for (j = 0; j < 3 * H; ++j) mod_out[j] += b_mod[j];
  for (t = 0; t < T; ++t) {
    const double* xr = x + (long)t * H;
    double ss = 0.0, r;
    for (j = 0; j < H; ++j) ss += xr[j] * xr[j];
    r = 1.0 / sqrt(ss / H + eps);
    for (j = 0; j < H; ++j)
      xn_out[(long)t * H + j] = xr[j] * r * (1.0 + mod_out[j]) + mod_out[H + j];
  }
}

/* Per-vector RMS norm with the (1 + w) weight convention of the Gemma family
 * named in [Art §2.2]'s shape table. */
static void rms_norm_1pw(double* u, const double* w, int D, double eps) {
  double ss = 0.0, r;
  int d;
  for (d = 0; d < D; ++d) ss += u[d] * u[d];
  r = 1.0 / sqrt(ss / D + eps);
  for (d = 0; d < D; ++d) u[d] = u[d] * r * (1.0 + w[d]);
}

/* Rotary embedding of one head vector at integer position pos.
 * Reading: pairs (j, j + D/2); angle = pos * base^(-2j/D). */
static void rope_rotate(double* u, int D, double pos, double base) {
  int j, half = D / 2;
  for (j = 0; j < half; ++j) {
    double theta = pos * pow(base, -2.0 * (double)j / (double)D);
    double c = cos(theta), s = sin(theta);
    double a = u[j], b = u[j + half];
    u[j] = a * c - b * s;
    u[j + half] = b * c + a * s;
  }
}

/*
 * QKV projection, QK-RMSNorm and RoPE "in one go" ([Art §2.2]).
 *   qkv = xn * W_qkv^T; rows of W_qkv: HQ query heads, then HK key heads, then
 *   HK value heads, each D rows.  q and k get the per-head RMS norm (weights
 *   qn_w / kn_w of length D shared by all heads, (1 + w) convention), then
 *   RoPE at position pos[t].  v is left as projected.
 * Outputs: q [T][HQ][D], k and v [HK][T][D].
 */
void orc_qkv_qknorm_rope(const double* xn, const double* w_qkv, const double* qn_w,
                         const double* kn_w, int T, int H, int HQ, int HK, int D,
                         const int32_t* pos, double base, double eps, double* q,
                         double* k, double* v) {
  int NQKV = (HQ + 2 * HK) * D;
  double* qkv = (double*)malloc(sizeof(double) * (size_t)T * NQKV);
  int t, h, d;
  orc_linear(xn, w_qkv, T, H, NQKV, qkv);
  for (t = 0; t < T; ++t) {
    const double* row = qkv + (long)t * NQKV;
    for (h = 0; h < HQ; ++h) {
      double* dst = q + ((long)t * HQ + h) * D;
      for (d = 0; d < D; ++d) dst[d] = row[h * D + d];
      rms_norm_1pw(dst, qn_w, D, eps);
      rope_rotate(dst, D, (double)pos[t], base);
    }
    for (h = 0; h < HK; ++h) {
      double* kd = k + ((long)h * T + t) * D;
      double* vd = v + ((long)h * T + t) * D;
      for (d = 0; d < D; ++d) {
        kd[d] = row[(HQ + h) * D + d];
        vd[d] = row[(HQ + HK + h) * D + d];
      }
      rms_norm_1pw(kd, kn_w, D, eps);
      rope_rotate(kd, D, (double)pos[t], base);
    }
  }
  free(qkv);
}

/*
 * Masked GQA attention of the action chunk ([Art §2.2]: qk logits read the
 * prefix KV cache and the suffix KV together under the prefix-visibility mask,
 * then softmax, then the value-weighted sum).
 *   Query head h reads KV head h / (HQ/HK).
 *   Key set of every query: the prefix rows j with mask[j] != 0, plus all C
 *   suffix rows (readings: the chunk attends to itself bidirectionally; the
 *   mask is shared by all heads and queries; masked rows are never read).
 *   p = exp(s - max s) / sum exp(s - max s), s = scale * q.k (two-pass
 *   softmax over the explicit key set -- the plain definition).
 * Layouts: q, ctx [C][HQ][D]; ks, vs [HK][C][D]; kp, vp [HK][P][D]; mask [P].
 * prob_sums (optional, [C][HQ]) receives sum p for each row.
 */
void orc_attention(const double* q, const double* ks, const double* vs,
                   const double* kp, const double* vp, const uint8_t* mask, int C,
                   int P, int HQ, int HK, int D, double scale, double* ctx,
                   double* prob_sums) {
  int group = HQ / HK;
  long ih;
#pragma omp parallel for schedule(dynamic)
  for (ih = 0; ih < (long)C * HQ; ++ih) {
    int i = (int)(ih / HQ), h = (int)(ih % HQ), g = h / group;
    const double* qi = q + ((long)i * HQ + h) * D;
    /* gather the key set: visible prefix rows then suffix rows */
    int nkeys = 0, j, d, n;
    const double** krow = (const double**)malloc(sizeof(double*) * (size_t)(P + C));
    const double** vrow = (const double**)malloc(sizeof(double*) * (size_t)(P + C));
    double* s = (double*)malloc(sizeof(double) * (size_t)(P + C + 1));
    double mx, sum, psum;
    double* out = ctx + ((long)i * HQ + h) * D;
    for (j = 0; j < P; ++j) {
      if (mask[j] == 0) continue;
      krow[nkeys] = kp + ((long)g * P + j) * D;
      vrow[nkeys] = vp + ((long)g * P + j) * D;
      ++nkeys;
    }
    for (j = 0; j < C; ++j) {
      krow[nkeys] = ks + ((long)g * C + j) * D;
      vrow[nkeys] = vs + ((long)g * C + j) * D;
      ++nkeys;
    }
    /* logits */
    for (n = 0; n < nkeys; ++n) {
      double dot = 0.0;
      for (d = 0; d < D; ++d) dot += qi[d] * krow[n][d];
      s[n] = dot * scale;
    }
    /* pass 1: max; pass 2: exponentials and their sum */
    mx = s[0];
    for (n = 1; n < nkeys; ++n)
      if (s[n] > mx) mx = s[n];
    sum = 0.0;
    for (n = 0; n < nkeys; ++n) {
      s[n] = exp(s[n] - mx);
      sum += s[n];
    }
    psum = 0.0;
    for (n = 0; n < nkeys; ++n) {
      s[n] /= sum;
      psum += s[n];
    }
    if (prob_sums) prob_sums[ih] = psum;
    for (d = 0; d < D; ++d) out[d] = 0.0;
    for (n = 0; n < nkeys; ++n)
      for (d = 0; d < D; ++d) out[d] += s[n] * vrow[n][d];
    free(krow);
    free(vrow);
    free(s);
  }
}

/*
 * O-projection and the gated residual ([Art §2.2] time-modulation chaining):
 *   out[t][j] = resid[t][j] + gate[j] * sum_k ctx[t][k] * W_o[j][k].
 * Reading: the gate is the raw modulation chunk (no sigmoid / tanh).
 */
void orc_oproj_gated_residual(const double* ctx, const double* w_o, const double* gate,
                              const double* resid, int T, int K, int H, double* out) {
  int t, j;
  orc_linear(ctx, w_o, T, K, H, out);
  for (t = 0; t < T; ++t)
    for (j = 0; j < H; ++j)
      out[(long)t * H + j] = resid[(long)t * H + j] + gate[j] * out[(long)t * H + j];
}

/* GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). */
double orc_gelu_tanh(double z) {
  const double c = sqrt(2.0 / 3.14159265358979323846);
  return 0.5 * z * (1.0 + tanh(c * (z + 0.044715 * z * z * z)));
}

/*
 * GEGLU gate-up, MLP down and the second gated residual ([Art §2.2]
 * "GEGLU gate-up" and "MLP down", chained with the time modulation):
 *   [a | u] = xn2 * W_gu^T  (a: rows 0..I-1 of W_gu, u: rows I..2I-1)
 *   hdn = gelu_tanh(a) * u
 *   out = resid + gate2 * (hdn * W_d^T)
 * h_out (optional, [T][I]) receives hdn.
 */
void orc_geglu_mlp(const double* xn2, const double* w_gu, const double* w_d,
                   const double* gate2, const double* resid, int T, int H, int I,
                   double* out, double* h_out) {
  double* gu = (double*)malloc(sizeof(double) * (size_t)T * 2 * I);
  double* hdn = (double*)malloc(sizeof(double) * (size_t)T * I);
  int t, n, j;
  orc_linear(xn2, w_gu, T, H, 2 * I, gu);
  for (t = 0; t < T; ++t)
    for (n = 0; n < I; ++n)
      hdn[(long)t * I + n] =
          orc_gelu_tanh(gu[(long)t * 2 * I + n]) * gu[(long)t * 2 * I + I + n];
  if (h_out)
    for (t = 0; t < T * I; ++t) h_out[t] = hdn[t];
  orc_linear(hdn, w_d, T, I, H, out);
  for (t = 0; t < T; ++t)
    for (j = 0; j < H; ++j)
      out[(long)t * H + j] = resid[(long)t * H + j] + gate2[j] * out[(long)t * H + j];
  free(gu);
  free(hdn);
}

/*
 * One action-expert layer for one request ([Art §2.2], suffix path):
 *   AdaRMS #1 -> QKV + QK-norm + RoPE -> masked GQA attention over
 *   [visible prefix KV ; suffix KV] -> O-projection + gated residual ->
 *   AdaRMS #2 -> GEGLU gate-up -> MLP down + gated residual.
 * x, out [C][H]; cond [H]; kp, vp [HK][P][D]; mask [P]; token t sits at
 * position pos0 + t.  Attention scale 1/sqrt(D).
 * Optional probes (may be NULL): xn1 [C][H], mod1/mod2 [3H], q [C][HQ][D],
 * ks/vs [HK][C][D], ctx [C][HQ][D], x1 [C][H], xn2 [C][H].
 */
void orc_layer(const double* x, const double* cond, const double* w_mod1,
               const double* b_mod1, const double* w_qkv, const double* qn_w,
               const double* kn_w, const double* w_o, const double* w_mod2,
               const double* b_mod2, const double* w_gu, const double* w_d,
               const double* kp, const double* vp, const uint8_t* mask, int C, int P,
               int H, int I, int HQ, int HK, int D, int32_t pos0, double base,
               double eps, double* out, double* p_xn1, double* p_mod1, double* p_q,
               double* p_ks, double* p_vs, double* p_ctx, double* p_x1,
               double* p_xn2, double* p_mod2) {
  size_t sH = (size_t)C * H, sQ = (size_t)C * HQ * D, sKV = (size_t)HK * C * D;
  double* xn1 = (double*)malloc(sizeof(double) * sH);
  double* mod1 = (double*)malloc(sizeof(double) * 3 * (size_t)H);
  double* q = (double*)malloc(sizeof(double) * sQ);
  double* ks = (double*)malloc(sizeof(double) * sKV);
  double* vs = (double*)malloc(sizeof(double) * sKV);
  double* ctx = (double*)malloc(sizeof(double) * sQ);
  double* x1 = (double*)malloc(sizeof(double) * sH);
  double* xn2 = (double*)malloc(sizeof(double) * sH);
  double* mod2 = (double*)malloc(sizeof(double) * 3 * (size_t)H);
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
  int t;
  size_t z;
  for (t = 0; t < C; ++t) pos[t] = pos0 + t;
  orc_adarms(x, cond, w_mod1, b_mod1, C, H, eps, xn1, mod1);
  orc_qkv_qknorm_rope(xn1, w_qkv, qn_w, kn_w, C, H, HQ, HK, D, pos, base, eps, q, ks, vs);
  orc_attention(q, ks, vs, kp, vp, mask, C, P, HQ, HK, D, 1.0 / sqrt((double)D), ctx, NULL);
  orc_oproj_gated_residual(ctx, w_o, mod1 + 2 * H, x, C, HQ * D, H, x1);
  orc_adarms(x1, cond, w_mod2, b_mod2, C, H, eps, xn2, mod2);
  orc_geglu_mlp(xn2, w_gu, w_d, mod2 + 2 * H, x1, C, H, I, out, NULL);
#define ORC_COPY(dst, src, n) \
  if (dst)                    \
    for (z = 0; z < (n); ++z) (dst)[z] = (src)[z];
  ORC_COPY(p_xn1, xn1, sH)
  ORC_COPY(p_mod1, mod1, 3 * (size_t)H)
  ORC_COPY(p_q, q, sQ)
  ORC_COPY(p_ks, ks, sKV)
  ORC_COPY(p_vs, vs, sKV)
  ORC_COPY(p_ctx, ctx, sQ)
  ORC_COPY(p_x1, x1, sH)
  ORC_COPY(p_xn2, xn2, sH)
  ORC_COPY(p_mod2, mod2, 3 * (size_t)H)
#undef ORC_COPY
  free(xn1);
  free(mod1);
  free(q);
  free(ks);
  free(vs);
  free(ctx);
  free(x1);
  free(xn2);
  free(mod2);
  free(pos);
}

/* ---------------------------------------------------------------------------
 * Prefix (prefill) side -- the Gemma3-4B decoder layer of the prefix path
 * named in [Art §2.2]'s shape table (hidden 2560, intermediate 10240,
 * head_dim 256, 8 Q / 4 KV heads) and its fusion list (image features merged
 * into the input embeddings; QKV + QK-Norm + RoPE in one pass; norm after the
 * attention, then the residual), with the prefix mask of [Art §2.3] (the
 * prefix-causal mask mapping handed to FlexAttention).
 * ------------------------------------------------------------------------- */

/* RMS norm of each row with the (1 + w) weight convention:
 *   y[t] = x[t] / sqrt(mean_j x[t][j]^2 + eps) * (1 + w). */
void orc_rmsnorm(const double* x, const double* w, int T, int H, double eps, double* y) {
  int t, j;
  for (t = 0; t < T; ++t) {
    double ss = 0.0, r;
    for (j = 0; j < H; ++j) ss += x[(long)t * H + j] * x[(long)t * H + j];
    r = 1.0 / sqrt(ss / H + eps);
    for (j = 0; j < H; ++j) y[(long)t * H + j] = x[(long)t * H + j] * r * (1.0 + w[j]);
  }
}

/* Image features merged into the input embeddings ([Art §2.2], prefix path):
 * token t takes image-feature row idx[t] when idx[t] >= 0, else its own text
 * embedding.  tok [T][H], img [NI][H], out [T][H]. */
void orc_image_merge(const double* tok, const double* img, const int32_t* idx, int T, int H,
                     double* out) {
  int t, j;
  for (t = 0; t < T; ++t) {
    const double* src = idx[t] >= 0 ? img + (long)idx[t] * H : tok + (long)t * H;
    for (j = 0; j < H; ++j) out[(long)t * H + j] = src[j];
  }
}

/*
 * Prefix attention ([Art §2.3]: FlexAttention with the prefix-causal mask
 * mapping).  Reading: query token i sees key token j exactly when j <= i and
 * token j is a valid prefix token (valid[j] != 0; the padding of a bucket is
 * not).  GQA: query head h reads KV head h / (HQ/HK).  Two-pass softmax over
 * that key set; a query with no visible key gets a zero output.
 * q, ctx [T][HQ][D]; k, v [HK][T][D]; valid [T].
 */
void orc_prefix_attention(const double* q, const double* k, const double* v, const uint8_t* valid,
                          int T, int HQ, int HK, int D, double scale, double* ctx) {
  int group = HQ / HK;
  long ih;
#pragma omp parallel for schedule(dynamic)
  for (ih = 0; ih < (long)T * HQ; ++ih) {
    int i = (int)(ih / HQ), h = (int)(ih % HQ), g = h / group;
    const double* qi = q + ((long)i * HQ + h) * D;
    double* out = ctx + ((long)i * HQ + h) * D;
    double* s = (double*)malloc(sizeof(double) * (size_t)(i + 1));
    double mx = 0.0, sum = 0.0;
    int j, d, any = 0;
    for (d = 0; d < D; ++d) out[d] = 0.0;
    for (j = 0; j <= i; ++j) {
      double dot = 0.0;
      if (!valid[j]) continue;
      for (d = 0; d < D; ++d) dot += qi[d] * k[((long)g * T + j) * D + d];
      s[j] = dot * scale;
      if (!any || s[j] > mx) mx = s[j];
      any = 1;
    }
    if (any) {
      for (j = 0; j <= i; ++j) {
        if (!valid[j]) continue;
        s[j] = exp(s[j] - mx);
        sum += s[j];
      }
      for (j = 0; j <= i; ++j) {
        if (!valid[j]) continue;
        for (d = 0; d < D; ++d) out[d] += s[j] / sum * v[((long)g * T + j) * D + d];
      }
    }
    free(s);
  }
}

/*
 * One prefix decoder layer for one request ([Art §2.2] prefix row of the shape
 * table and fusion list; Gemma3-4B).  Reading (the pages name the pieces, the
 * order follows the Gemma3 decoder they name):
 *   xn  = rmsnorm(x; w_in)
 *   q, k, v = QKV(xn) with QK-RMSNorm and RoPE at positions 0 .. T-1
 *   ctx = prefix attention(q, k, v; valid), scale 1/sqrt(D)
 *   x1  = x + rmsnorm(ctx W_o^T; w_post_attn)            (norm after attention, residual)
 *   xn2 = rmsnorm(x1; w_pre_ffn)
 *   hdn = gelu_tanh(xn2 W_g^T) * (xn2 W_u^T)             (W_gu rows: gate, then up)
 *   out = x1 + rmsnorm(hdn W_d^T; w_post_ffn)
 * k, v [HK][T][D] are the layer's KV cache (what the suffix reads).
 * x, out [T][H]; valid [T].
 */
void orc_prefix_layer(const double* x, const double* w_in, const double* w_qkv, const double* qn_w,
                      const double* kn_w, const double* w_o, const double* w_post_attn,
                      const double* w_pre_ffn, const double* w_gu, const double* w_d,
                      const double* w_post_ffn, const uint8_t* valid, int T, int H, int I, int HQ,
                      int HK, int D, double base, double eps, double* out, double* k, double* v) {
  size_t sH = (size_t)T * H, sQ = (size_t)T * HQ * D;
  double* xn = (double*)malloc(sizeof(double) * sH);
  double* q = (double*)malloc(sizeof(double) * sQ);
  double* ctx = (double*)malloc(sizeof(double) * sQ);
  double* a = (double*)malloc(sizeof(double) * sH);
  double* x1 = (double*)malloc(sizeof(double) * sH);
  double* gu = (double*)malloc(sizeof(double) * (size_t)T * 2 * I);
  double* hdn = (double*)malloc(sizeof(double) * (size_t)T * I);
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
  int t, n;
  size_t z;
  for (t = 0; t < T; ++t) pos[t] = t;
  orc_rmsnorm(x, w_in, T, H, eps, xn);
  orc_qkv_qknorm_rope(xn, w_qkv, qn_w, kn_w, T, H, HQ, HK, D, pos, base, eps, q, k, v);
  orc_prefix_attention(q, k, v, valid, T, HQ, HK, D, 1.0 / sqrt((double)D), ctx);
  orc_linear(ctx, w_o, T, HQ * D, H, a);
  orc_rmsnorm(a, w_post_attn, T, H, eps, xn);
  for (z = 0; z < sH; ++z) x1[z] = x[z] + xn[z];
  orc_rmsnorm(x1, w_pre_ffn, T, H, eps, xn);
  orc_linear(xn, w_gu, T, H, 2 * I, gu);
  for (t = 0; t < T; ++t)
    for (n = 0; n < I; ++n)
      hdn[(long)t * I + n] = orc_gelu_tanh(gu[(long)t * 2 * I + n]) * gu[(long)t * 2 * I + I + n];
  orc_linear(hdn, w_d, T, I, H, a);
  orc_rmsnorm(a, w_post_ffn, T, H, eps, xn);
  for (z = 0; z < sH; ++z) out[z] = x1[z] + xn[z];
  free(xn);
  free(q);
  free(ctx);
  free(a);
  free(x1);
  free(gu);
  free(hdn);
  free(pos);
}

/* ---------------------------------------------------------------------------
 * Denoise sampler around the action-expert stack.  The pages describe the
 * action chunk as decoded by diffusion in a fixed number of steps ([Art §1],
 * [Art §4]; [Guide §2], the diffusion step count) and give none of the
 * sampler's formulas.  Every step below is therefore a reading, the plainest
 * one for a flow-matching action expert with AdaRMS time conditioning:
 *   t_k = 1 - k / n, k = 0 .. n-1, from noise (t = 1) to data (t = 0);
 *   temb(t)[i] = sin(1000 t w_i), temb(t)[H/2 + i] = cos(1000 t w_i),
 *       w_i = 10000^(-i / (H/2));
 *   cond(t) = swish(W_t2 swish(W_t1 temb(t) + b_t1) + b_t2),
 *       swish(z) = z / (1 + exp(-z));
 *   x = a W_in^T + b_in for each chunk token (action in-projection);
 *   x <- the action-expert layers run with cond(t_k);
 *   [scale | shift] = W_f cond + b_f, xf = x / sqrt(mean x^2 + eps) (1 + scale) + shift;
 *   v = xf W_out^T + b_out (the velocity);
 *   a <- a + dt v, dt = -1 / n (one Euler step of the flow ODE).
 */

/* temb(t), H values (sin half, then cos half). */
void orc_time_embedding(double t, int H, double* out) {
  int half = H / 2, i;
  for (i = 0; i < half; ++i) {
    double w = pow(10000.0, -(double)i / half);
    out[i] = sin(1000.0 * t * w);
    out[half + i] = cos(1000.0 * t * w);
  }
}

double orc_swish(double z) { return z / (1.0 + exp(-z)); }

/* cond = swish(W_t2 swish(W_t1 temb + b_t1) + b_t2); W_t1, W_t2 [H][H]. */
void orc_time_mlp(const double* temb, const double* w1, const double* b1, const double* w2,
                  const double* b2, int H, double* cond) {
  double* h1 = (double*)malloc(sizeof(double) * (size_t)H);
  int j;
  orc_linear(temb, w1, 1, H, H, h1);
  for (j = 0; j < H; ++j) h1[j] = orc_swish(h1[j] + b1[j]);
  orc_linear(h1, w2, 1, H, H, cond);
  for (j = 0; j < H; ++j) cond[j] = orc_swish(cond[j] + b2[j]);
  free(h1);
}

/* x[c] = W_in a[c] + b_in; a [C][A], W_in [H][A] -> x [C][H]. */
void orc_action_in(const double* a, const double* w_in, const double* b_in, int C, int A, int H,
                   double* x) {
  int c, j;
  orc_linear(a, w_in, C, A, H, x);
  for (c = 0; c < C; ++c)
    for (j = 0; j < H; ++j) x[(long)c * H + j] += b_in[j];
}

/* Velocity of the chunk: the final AdaRMS norm (modulation [scale | shift] =
 * W_f cond + b_f, W_f [2H][H]) of the expert's output x [C][H], then
 * v = xf W_out^T + b_out, W_out [A][H] -> v [C][A]. */
void orc_final_velocity(const double* x, const double* cond, const double* w_f, const double* b_f,
                        const double* w_out, const double* b_out, int C, int H, int A, double eps,
                        double* v) {
  double* m = (double*)malloc(sizeof(double) * 2 * (size_t)H);
  double* xf = (double*)malloc(sizeof(double) * (size_t)C * H);
  int c, j;
  orc_linear(cond, w_f, 1, H, 2 * H, m);
  for (j = 0; j < 2 * H; ++j) m[j] += b_f[j];
  for (c = 0; c < C; ++c) {
    const double* xr = x + (long)c * H;
    double ss = 0.0, r;
    for (j = 0; j < H; ++j) ss += xr[j] * xr[j];
    r = 1.0 / sqrt(ss / H + eps);
    for (j = 0; j < H; ++j) xf[(long)c * H + j] = xr[j] * r * (1.0 + m[j]) + m[H + j];
  }
  orc_linear(xf, w_out, C, H, A, v);
  for (c = 0; c < C; ++c)
    for (j = 0; j < A; ++j) v[(long)c * A + j] += b_out[j];
  free(m);
  free(xf);
}

/* a <- a + dt v over n values (one Euler step). */
void orc_euler(double* a, const double* v, long n, double dt) {
  long i;
  for (i = 0; i < n; ++i) a[i] += dt * v[i];
}
