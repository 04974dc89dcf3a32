/*
 * Decode-step oracle -- TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Parity status: every building block is pinned by the not-gpu tests
 * (closed forms, invariants, special cases, brute-force full-sequence
 * recomputation).  The model conventions themselves (norm form, rotate-half
 * RoPE, 1/sqrt(d) scale, delta-rule front end) are readings of pages that
 * print no model equations; they are pinned only by agreement between this
 * file and the independent brute-force recomputation, which follows the
 * same readings ("parity unpinned by the pages" for the conventions).
 *
 * Method being checked: the ForgeMegakernel abstract (arxivdaily /
 * arxiv.science, abstract) -- a decode step is bandwidth bound because every
 * weight and KV-cache byte crosses HBM once per token; its megakernel must
 * reach exactly the result of the plain step below.  The delta-rule layer
 * follows the MK-KDA pull request (github choiceoh/stkernel #230, phase
 * chain in_proj -> gates -> conv -> delta -> o_proj) and the update rule
 * S <- g S + beta k (v^T - k^T S) of the hybrid workload.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

float orc_bf16_to_f32(uint16_t h) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)h << 16;
  return v.f;
}

uint16_t orc_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v = {f};
  if ((v.u & 0x7F800000u) == 0x7F800000u && (v.u & 0x007FFFFFu)) return (uint16_t)((v.u >> 16) | 0x40u);
  uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }
double orc_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

void orc_rmsnorm(const float* x, const uint16_t* gain, int n, double eps, float* y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int i = 0; i < n; ++i) {
    double g = gain ? (double)orc_bf16_to_f32(gain[i]) : 1.0;
    y[i] = (float)((double)x[i] * inv * g);
  }
}

void orc_matvec(const uint16_t* W, const float* x, int rows, int cols, float* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const uint16_t* wr = W + (size_t)r * (size_t)cols;
    double acc = 0.0;
    for (int k = 0; k < cols; ++k) acc += (double)orc_bf16_to_f32(wr[k]) * (double)x[k];
    y[r] = (float)acc;
  }
}

/* Rotate-half: pairs (i, i + d/2), angle pos * base^(-2i/d). */
/* OCP 8-bit floating point specification, E4M3 encoding: the low-bit weight format of the MK-KDA
 * pull request's weight stream (github choiceoh/stkernel #230, PR summary) taken at 8 bits, in the
 * variant gfx950 reads natively. */
double orc_e4m3(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

void orc_matvec_fp8(const uint8_t* W, const float* scale, const float* x, int rows, int cols, float* y) {
  double lut[256];
  for (int c = 0; c < 256; ++c) lut[c] = orc_e4m3((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const uint8_t* wr = W + (size_t)r * (size_t)cols;
    double acc = 0.0;
    for (int k = 0; k < cols; ++k) acc += lut[wr[k]] * (double)x[k];
    y[r] = (float)((double)scale[r] * acc);
  }
}

/* OCP Microscaling (MX) formats specification: MXFP4 elements are E2M1, scaled per block of 32 by
 * an E8M0 power of two -- the 4-bit weight stream with block scales of the MK-KDA pull request
 * (github choiceoh/stkernel #230, PR summary), in the MX encoding gfx950 reads natively. */
double orc_e2m1(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

double orc_e8m0(uint8_t e) { return e == 0xFF ? NAN : ldexp(1.0, (int)e - 127); }

void orc_matvec_fp4(const uint8_t* W, const uint8_t* S, const float* x, int rows, int cols, float* y) {
  double lut[16];
  for (int c = 0; c < 16; ++c) lut[c] = orc_e2m1((uint8_t)c);
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const uint8_t* wr = W + (size_t)r * (size_t)(cols / 2);
    const uint8_t* sr = S + (size_t)r * (size_t)(cols / 32);
    double acc = 0.0;
    for (int k = 0; k < cols; ++k) {
      const uint8_t byte = wr[k / 2];
      const double w = orc_e8m0(sr[k / 32]) * lut[(k & 1) ? byte >> 4 : byte & 15];
      acc += w * (double)x[k];
    }
    y[r] = (float)acc;
  }
}

/* one projection of the model, in its weight format */
static void proj(const orc_model* m, const void* W, const void* scale, const float* x, int rows, int cols, float* y) {
  if (m->weight_format == ORC_W_FP8) orc_matvec_fp8((const uint8_t*)W, (const float*)scale, x, rows, cols, y);
  else if (m->weight_format == ORC_W_FP4) orc_matvec_fp4((const uint8_t*)W, (const uint8_t*)scale, x, rows, cols, y);
  else orc_matvec((const uint16_t*)W, x, rows, cols, y);
}

void orc_rope(float* u, int d, int pos, double base) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double theta = (double)pos * pow(base, -2.0 * (double)i / (double)d);
    double c = cos(theta), s = sin(theta);
    double a = u[i], b = u[i + half];
    u[i] = (float)(a * c - b * s);
    u[i + half] = (float)(b * c + a * s);
  }
}

void orc_attend(const float* q, const uint16_t* const* krows, const uint16_t* const* vrows, int n, int d,
                float* o, double* probs) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double scale = 1.0 / sqrt((double)d);
  double mx = -INFINITY;
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += (double)q[i] * (double)orc_bf16_to_f32(krows[j][i]);
    s[j] = acc * scale;
    if (s[j] > mx) mx = s[j];
  }
  double den = 0.0;
  for (int j = 0; j < n; ++j) {
    s[j] = exp(s[j] - mx);
    den += s[j];
  }
  for (int j = 0; j < n; ++j) s[j] /= den;
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int j = 0; j < n; ++j) acc += s[j] * (double)orc_bf16_to_f32(vrows[j][i]);
    o[i] = (float)acc;
  }
  if (probs)
    for (int j = 0; j < n; ++j) probs[j] = s[j];
  free(s);
}

void orc_conv_step(const float* u, const uint16_t* conv_w, float* state, int C, int W, float* y) {
  for (int c = 0; c < C; ++c) {
    float* st = state + (size_t)c * (size_t)(W - 1);
    const uint16_t* wc = conv_w + (size_t)c * (size_t)W;
    double acc = 0.0;
    for (int j = 0; j < W - 1; ++j) acc += (double)orc_bf16_to_f32(wc[j]) * (double)st[j];
    acc += (double)orc_bf16_to_f32(wc[W - 1]) * (double)u[c];
    y[c] = (float)orc_silu(acc);
    for (int j = 0; j + 1 < W - 1; ++j) st[j] = st[j + 1];
    st[W - 2] = u[c];
  }
}

/* S is dk x dv; st holds it transposed, st[j*dk + i] = S[i][j]. */
void orc_delta_step(float* st, const float* q, const float* k, const float* v, double g, double beta,
                    int dk, int dv, int decay_first, float* o) {
  for (int j = 0; j < dv; ++j) {
    float* col = st + (size_t)j * (size_t)dk; /* S[:, j] */
    double kS = 0.0;                          /* (k^T S)_j with the old S */
    for (int i = 0; i < dk; ++i) kS += (double)k[i] * (double)col[i];
    if (decay_first) kS *= g;                 /* k^T (g S) */
    double err = (double)v[j] - kS;
    for (int i = 0; i < dk; ++i) col[i] = (float)(g * (double)col[i] + beta * (double)k[i] * err);
    double acc = 0.0;                         /* o_j = (S^T q)_j with the new S */
    for (int i = 0; i < dk; ++i) acc += (double)col[i] * (double)q[i];
    o[j] = (float)acc;
  }
}

int orc_argmax(const float* v, int n) {
  int best = 0;
  for (int i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  return best;
}

/* ------------------------------------------------------------------------ */

static void add_into(float* x, const float* d, int n) {
  for (int i = 0; i < n; ++i) x[i] = (float)((double)x[i] + (double)d[i]);
}

static size_t kv_index(const orc_model* m, const orc_cache* c, int attn_layer, int page, int kvh, int slot) {
  size_t per_page = (size_t)m->n_kv_heads * (size_t)m->page_size * (size_t)m->head_dim;
  return ((size_t)attn_layer * (size_t)c->num_pages + (size_t)page) * per_page +
         ((size_t)kvh * (size_t)m->page_size + (size_t)slot) * (size_t)m->head_dim;
}

static int check_inputs(const orc_model* m, const orc_cache* c, const int32_t* tokens, const int32_t* positions,
                        const int32_t* ctx_lens, int batch) {
  if (batch < 1 || batch > c->max_batch) return -1;
  for (int b = 0; b < batch; ++b) {
    if (tokens[b] < 0 || tokens[b] >= m->vocab) return -2;
    if (ctx_lens[b] < 1 || positions[b] != ctx_lens[b] - 1) return -3;
    int need = (ctx_lens[b] + m->page_size - 1) / m->page_size;
    if (need > c->max_pages_per_seq) return -4;
    for (int p = 0; p < need; ++p) {
      int id = c->page_table[(size_t)b * (size_t)c->max_pages_per_seq + (size_t)p];
      if (id < 0 || id >= c->num_pages) return -4;
    }
  }
  return 0;
}

static void attention_layer(const orc_model* m, const orc_layer* L, orc_cache* c, int attn_layer, int b, int pos,
                            int ctx, const float* r, float* o) {
  int d = m->head_dim, Hq = m->n_q_heads, Hkv = m->n_kv_heads;
  float* q = (float*)malloc(sizeof(float) * (size_t)Hq * d);
  float* k = (float*)malloc(sizeof(float) * (size_t)Hkv * d);
  float* v = (float*)malloc(sizeof(float) * (size_t)Hkv * d);
  proj(m, L->wq, L->s_wq, r, Hq * d, m->hidden, q);
  proj(m, L->wk, L->s_wk, r, Hkv * d, m->hidden, k);
  proj(m, L->wv, L->s_wv, r, Hkv * d, m->hidden, v);
  if (m->qk_norm) {
    for (int h = 0; h < Hq; ++h) orc_rmsnorm(q + (size_t)h * d, L->q_norm, d, m->rms_eps, q + (size_t)h * d);
    for (int h = 0; h < Hkv; ++h) orc_rmsnorm(k + (size_t)h * d, L->k_norm, d, m->rms_eps, k + (size_t)h * d);
  }
  for (int h = 0; h < Hq; ++h) orc_rope(q + (size_t)h * d, d, pos, m->rope_base);
  for (int h = 0; h < Hkv; ++h) orc_rope(k + (size_t)h * d, d, pos, m->rope_base);
  /* append the new K/V (rounded to bf16) at pos */
  const int32_t* table = c->page_table + (size_t)b * (size_t)c->max_pages_per_seq;
  for (int h = 0; h < Hkv; ++h) {
    size_t at = kv_index(m, c, attn_layer, table[pos / m->page_size], h, pos % m->page_size);
    for (int i = 0; i < d; ++i) {
      c->k_pages[at + i] = orc_f32_to_bf16(k[(size_t)h * d + i]);
      c->v_pages[at + i] = orc_f32_to_bf16(v[(size_t)h * d + i]);
    }
  }
  const uint16_t** kr = (const uint16_t**)malloc(sizeof(void*) * (size_t)ctx);
  const uint16_t** vr = (const uint16_t**)malloc(sizeof(void*) * (size_t)ctx);
  for (int h = 0; h < Hq; ++h) {
    int g = h * Hkv / Hq; /* contiguous query-head groups share one KV head */
    for (int j = 0; j < ctx; ++j) {
      size_t at = kv_index(m, c, attn_layer, table[j / m->page_size], g, j % m->page_size);
      kr[j] = c->k_pages + at;
      vr[j] = c->v_pages + at;
    }
    orc_attend(q + (size_t)h * d, kr, vr, ctx, d, o + (size_t)h * d, NULL);
  }
  free(kr); free(vr); free(q); free(k); free(v);
}

/* The delta-rule mixer of one sequence after its projections: conv step on u (rolling state cs),
 * per-head L2 norm of q and k with q scaled by dk^-1/2, gates g = sigmoid(a_h), beta =
 * sigmoid(a_{nh+h}), then the state update and readout of every head (st: S^T, [nh][dv][dk]). */
void orc_delta_mixer(const orc_model* m, const uint16_t* conv_w, const float* u, const float* a, float* cs,
                     float* st, float* o) {
  int nh = m->n_delta_heads, dk = m->delta_dk, dv = m->delta_dv, W = m->conv_width;
  int C = nh * (2 * dk + dv);
  float* y = (float*)malloc(sizeof(float) * (size_t)C);
  orc_conv_step(u, conv_w, cs, C, W, y);
  float* qh = (float*)malloc(sizeof(float) * (size_t)dk);
  float* kh = (float*)malloc(sizeof(float) * (size_t)dk);
  for (int h = 0; h < nh; ++h) {
    const float* yq = y + (size_t)h * dk;
    const float* yk = y + (size_t)nh * dk + (size_t)h * dk;
    const float* yv = y + (size_t)2 * nh * dk + (size_t)h * dv;
    double nq = 0.0, nk = 0.0;
    for (int i = 0; i < dk; ++i) { nq += (double)yq[i] * yq[i]; nk += (double)yk[i] * yk[i]; }
    double sq = 1.0 / sqrt(nq + 1e-6) / sqrt((double)dk), sk = 1.0 / sqrt(nk + 1e-6);
    for (int i = 0; i < dk; ++i) { qh[i] = (float)(yq[i] * sq); kh[i] = (float)(yk[i] * sk); }
    double g = orc_sigmoid(a[h]), beta = orc_sigmoid(a[nh + h]);
    orc_delta_step(st + (size_t)h * (size_t)dv * (size_t)dk, qh, kh, yv, g, beta, dk, dv, m->delta_decay_first,
                   o + (size_t)h * dv);
  }
  free(qh); free(kh); free(y);
}

static void delta_layer(const orc_model* m, const orc_layer* L, orc_cache* c, int delta_layer_idx, int b,
                        const float* r, float* o) {
  int nh = m->n_delta_heads, dk = m->delta_dk, dv = m->delta_dv, W = m->conv_width;
  int C = nh * (2 * dk + dv);
  float* u = (float*)malloc(sizeof(float) * (size_t)C);
  float* a = (float*)malloc(sizeof(float) * (size_t)(2 * nh));
  proj(m, L->w_qkv_delta, L->s_w_qkv_delta, r, C, m->hidden, u);
  proj(m, L->w_gates, L->s_w_gates, r, 2 * nh, m->hidden, a);
  float* cs = c->conv_state + ((size_t)delta_layer_idx * (size_t)c->max_batch + (size_t)b) * (size_t)C * (size_t)(W - 1);
  float* st = c->delta_state + ((size_t)delta_layer_idx * (size_t)c->max_batch + (size_t)b) * (size_t)nh *
                                   (size_t)dv * (size_t)dk;
  orc_delta_mixer(m, L->conv_w, u, a, cs, st, o);
  free(u); free(a);
}

/* Router of a mixture-of-experts MLP: the top-k experts by logit (Mixtral / OLMoE style top-k gating),
 * repeated selection of the largest remaining logit, ties to the lower index. */
void orc_moe_select(const float* logits, int n, int k, int32_t* sel) {
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < n; ++e) {
      int taken = 0;
      for (int i = 0; i < j; ++i) taken |= sel[i] == e;
      if (!taken && (best < 0 || logits[e] > logits[best])) best = e;
    }
    sel[j] = best;
  }
}

/* gate probabilities p = softmax(logits) over every expert, then the chosen k renormalised */
void orc_moe_weights(const float* logits, int n, int k, const int32_t* sel, double* w) {
  double mx = logits[0];
  for (int e = 1; e < n; ++e) mx = logits[e] > mx ? logits[e] : mx;
  double z = 0.0;
  for (int e = 0; e < n; ++e) z += exp((double)logits[e] - mx);
  double s = 0.0;
  for (int j = 0; j < k; ++j) {
    w[j] = exp((double)logits[sel[j]] - mx) / z;
    s += w[j];
  }
  for (int j = 0; j < k; ++j) w[j] /= s;
}

/* The MoE MLP of one sequence (layer l, sequence b of `batch`): r = RMSNorm(x) * gain, router
 * logits, top-k experts (or the forced ones), x += sum_j w_j down_e(silu(gate_e r) * up_e r). */
static void moe_mlp(const orc_model* m, const orc_layer* L, int l, int b, int batch, float* x, orc_dump* dump) {
  int H = m->hidden, F = m->ffn, E = m->n_experts, k = m->top_k;
  float* r = (float*)malloc(sizeof(float) * (size_t)H);
  float* rl = (float*)malloc(sizeof(float) * (size_t)E);
  float* gt = (float*)malloc(sizeof(float) * (size_t)F);
  float* up = (float*)malloc(sizeof(float) * (size_t)F);
  float* y = (float*)malloc(sizeof(float) * (size_t)H);
  double* acc = (double*)calloc((size_t)H, sizeof(double));
  int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  double* wt = (double*)malloc(sizeof(double) * (size_t)k);
  orc_rmsnorm(x, L->mlp_norm, H, m->rms_eps, r);
  orc_matvec(L->w_router, r, E, H, rl);
  orc_moe_select(rl, E, k, sel);
  size_t at = ((size_t)l * batch + b);
  if (dump && dump->router) memcpy(dump->router + at * (size_t)E, rl, sizeof(float) * (size_t)E);
  if (dump && dump->sel) memcpy(dump->sel + at * (size_t)k, sel, sizeof(int32_t) * (size_t)k);
  if (dump && dump->force) memcpy(sel, dump->force + at * (size_t)k, sizeof(int32_t) * (size_t)k);
  orc_moe_weights(rl, E, k, sel, wt);
  const uint16_t *wg = (const uint16_t*)L->w_gate, *wu = (const uint16_t*)L->w_up, *wd = (const uint16_t*)L->w_down;
  for (int j = 0; j < k; ++j) {
    size_t e = (size_t)sel[j];
    orc_matvec(wg + e * (size_t)F * H, r, F, H, gt);
    orc_matvec(wu + e * (size_t)F * H, r, F, H, up);
    for (int i = 0; i < F; ++i) gt[i] = (float)(orc_silu(gt[i]) * (double)up[i]);
    orc_matvec(wd + e * (size_t)H * F, gt, H, F, y);
    for (int i = 0; i < H; ++i) acc[i] += wt[j] * (double)y[i];
  }
  for (int i = 0; i < H; ++i) x[i] = (float)((double)x[i] + acc[i]);
  free(r); free(rl); free(gt); free(up); free(y); free(acc); free(sel); free(wt);
}

int orc_decode_step(const orc_model* m, const orc_weights* w, orc_cache* c, const int32_t* tokens,
                    const int32_t* positions, const int32_t* ctx_lens, int batch, float* logits, orc_dump* dump) {
  int rc = check_inputs(m, c, tokens, positions, ctx_lens, batch);
  if (rc) return rc;
  int H = m->hidden, F = m->ffn;
  int mix = m->n_q_heads * m->head_dim;
  if (m->n_delta_heads * m->delta_dv > mix) mix = m->n_delta_heads * m->delta_dv;
  float* x = (float*)malloc(sizeof(float) * (size_t)H);
  float* r = (float*)malloc(sizeof(float) * (size_t)H);
  float* t = (float*)malloc(sizeof(float) * (size_t)H);
  float* o = (float*)malloc(sizeof(float) * (size_t)mix);
  float* gt = (float*)malloc(sizeof(float) * (size_t)F);
  float* up = (float*)malloc(sizeof(float) * (size_t)F);
  for (int b = 0; b < batch; ++b) {
    int pos = positions[b], ctx = ctx_lens[b];
    for (int i = 0; i < H; ++i) x[i] = orc_bf16_to_f32(w->embed[(size_t)tokens[b] * (size_t)H + i]);
    int ia = 0, id = 0;
    for (int l = 0; l < m->n_layers; ++l) {
      const orc_layer* L = &w->layers[l];
      memset(o, 0, sizeof(float) * (size_t)mix);
      orc_rmsnorm(x, L->attn_norm, H, m->rms_eps, r);
      if (m->layer_kind[l] == ORC_ATTN) {
        attention_layer(m, L, c, ia++, b, pos, ctx, r, o);
        proj(m, L->wo, L->s_wo, o, H, m->n_q_heads * m->head_dim, t);
      } else {
        delta_layer(m, L, c, id++, b, r, o);
        proj(m, L->wo_delta, L->s_wo_delta, o, H, m->n_delta_heads * m->delta_dv, t);
      }
      add_into(x, t, H);
      if (dump && dump->mixer_o) memcpy(dump->mixer_o + ((size_t)l * batch + b) * (size_t)mix, o, sizeof(float) * (size_t)mix);
      if (dump && dump->x_mixer) memcpy(dump->x_mixer + ((size_t)l * batch + b) * (size_t)H, x, sizeof(float) * (size_t)H);
      if (m->n_experts > 0) {
        moe_mlp(m, L, l, b, batch, x, dump);
        if (dump && dump->x_mlp) memcpy(dump->x_mlp + ((size_t)l * batch + b) * (size_t)H, x, sizeof(float) * (size_t)H);
        continue;
      }
      /* SwiGLU MLP */
      orc_rmsnorm(x, L->mlp_norm, H, m->rms_eps, r);
      proj(m, L->w_gate, L->s_w_gate, r, F, H, gt);
      proj(m, L->w_up, L->s_w_up, r, F, H, up);
      for (int i = 0; i < F; ++i) gt[i] = (float)(orc_silu(gt[i]) * (double)up[i]);
      proj(m, L->w_down, L->s_w_down, gt, H, F, t);
      add_into(x, t, H);
      if (dump && dump->mlp_m) memcpy(dump->mlp_m + ((size_t)l * batch + b) * (size_t)F, gt, sizeof(float) * (size_t)F);
      if (dump && dump->x_mlp) memcpy(dump->x_mlp + ((size_t)l * batch + b) * (size_t)H, x, sizeof(float) * (size_t)H);
    }
    orc_rmsnorm(x, w->final_norm, H, m->rms_eps, r);
    if (dump && dump->final_r) memcpy(dump->final_r + (size_t)b * H, r, sizeof(float) * (size_t)H);
    const uint16_t* lm = m->tied_embeddings ? w->embed : w->lm_head;
    orc_matvec(lm, r, m->vocab, H, logits + (size_t)b * (size_t)m->vocab);
  }
  free(x); free(r); free(t); free(o); free(gt); free(up);
  return 0;
}
