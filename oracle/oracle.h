/*
 * Decode-step oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU implementation of one transformer decode step (and the
 * gated delta-rule layer of the hybrid model), written from the definition
 * and never from the GPU path.  Only the test-suite, the smoke check and the
 * bench's CPU-baseline leg load it; the product path never does.
 *
 * The "independent mid-state test oracle" is the ForgeMegakernel abstract's
 * (arxivdaily / arxiv.science, abstract): it derives the intermediate states
 * of the decode step so that each can be checked separately, as the MK-KDA
 * pull request (github choiceoh/stkernel #230, PR summary) gates output,
 * conv state and recurrent state separately.
 *
 * Precision: inputs and stored values are fp32 (weights bf16); every dot
 * product, norm and softmax accumulates in double.
 */
#ifndef MK_ORACLE_H
#define MK_ORACLE_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_ATTN = 0, ORC_DELTA = 1 };

typedef struct {
  int n_layers, hidden, vocab, ffn;
  int n_q_heads, n_kv_heads, head_dim, qk_norm, tied_embeddings;
  double rms_eps, rope_base;
  int n_delta_heads, delta_dk, delta_dv, conv_width;
  const int32_t* layer_kind; /* [n_layers]: ORC_ATTN or ORC_DELTA */
  int page_size;
  int delta_decay_first;     /* 0: S <- gS + b k(v^T - k^T S) with the old S throughout; 1: decay first */
} orc_model;

typedef struct { /* bf16 bit patterns, [out][in] row-major */
  const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *q_norm, *k_norm;
  const uint16_t *w_qkv_delta, *w_gates, *conv_w, *wo_delta;
  const uint16_t *mlp_norm, *w_gate, *w_up, *w_down;
} orc_layer;

typedef struct {
  const uint16_t *embed, *final_norm, *lm_head;
  const orc_layer* layers;
} orc_weights;

typedef struct {
  uint16_t *k_pages, *v_pages;  /* [n_attn_layers][num_pages][n_kv_heads][page_size][head_dim] */
  int num_pages, max_pages_per_seq;
  const int32_t* page_table;    /* [batch][max_pages_per_seq] */
  float* delta_state;           /* [n_delta_layers][batch][heads][dv][dk]  (S transposed) */
  float* conv_state;            /* [n_delta_layers][batch][channels][conv_width-1], oldest first */
  int max_batch;
} orc_cache;

/* Optional mid-state dump (any pointer may be NULL).  Per layer l, sequence b:
 *   x_mixer [L][B][hidden]   residual after the attention / delta sub-layer
 *   x_mlp   [L][B][hidden]   residual after the MLP
 *   mixer_o [L][B][mix_dim]  attention output o (Hq*d) or delta readout (heads*dv), before o_proj
 *   mlp_m   [L][B][ffn]      silu(gate) * up
 *   final_r [B][hidden]      normalised input of the LM head
 * mix_dim = max(n_q_heads*head_dim, n_delta_heads*delta_dv). */
typedef struct {
  float *x_mixer, *x_mlp, *mixer_o, *mlp_m, *final_r;
} orc_dump;

/* ---- building blocks (exported so the tests can pin each one) ---- */
float orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);
/* y = x * (mean(x^2) + eps)^-1/2 * gain (gain may be NULL = 1) */
void orc_rmsnorm(const float* x, const uint16_t* gain, int n, double eps, float* y);
/* y[r] = sum_k W[r][k] x[k], W bf16 [rows][cols] */
void orc_matvec(const uint16_t* W, const float* x, int rows, int cols, float* y);
/* rotate-half rotary embedding of one head vector u[d] at position pos */
void orc_rope(float* u, int d, int pos, double base);
/* single-head attention over n keys: o = softmax(q.K^T / sqrt(d)) V; K, V bf16 rows [n][d]
 * given as row pointers.  probs (may be NULL) receives the n softmax weights. */
void orc_attend(const float* q, const uint16_t* const* krows, const uint16_t* const* vrows, int n, int d,
                float* o, double* probs);
double orc_silu(double z);
double orc_sigmoid(double z);
/* one causal depthwise conv step for C channels: window = (state[c][0..W-2], u[c]);
 * y[c] = silu(sum_j w[c][j] window[j]); state <- last W-1 inputs.  conv_w bf16 [C][W]. */
void orc_conv_step(const float* u, const uint16_t* conv_w, float* state, int C, int W, float* y);
/* one gated delta-rule step for one head: st = S^T [dv][dk] updated in place; o[dv] = S^T q. */
void orc_delta_step(float* st, const float* q, const float* k, const float* v, double g, double beta,
                    int dk, int dv, int decay_first, float* o);

/* ---- the decode step ----
 * For every b < batch: consume tokens[b] at position positions[b] (== ctx_lens[b]-1), append K/V
 * (or update the conv / delta states), write logits[b][vocab].  Returns 0 or a negative code for
 * inputs outside the contract (nothing is written then). */
int orc_decode_step(const orc_model* m, const orc_weights* w, orc_cache* c, const int32_t* tokens,
                    const int32_t* positions, const int32_t* ctx_lens, int batch, float* logits,
                    orc_dump* dump);

/* greedy choice: argmax, ties to the lowest index */
int orc_argmax(const float* v, int n);

#ifdef __cplusplus
}
#endif
#endif
