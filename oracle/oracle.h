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
  int weight_format;         /* ORC_W_BF16, ORC_W_FP8 or ORC_W_FP4: the projection matrices' format */
  /* Mixture of experts (0 = dense MLPs): with n_experts > 0 every layer's MLP is top_k of n_experts
   * SwiGLU experts of width ffn, chosen per sequence by a router (bf16 weights only). */
  int n_experts, top_k;
} orc_model;

/* Projection weights (wq wk wv wo w_qkv_delta w_gates wo_delta w_gate w_up w_down): bf16 bit
 * patterns; or with ORC_W_FP8 one OCP E4M3 byte per weight and one fp32 scale per output row,
 * W[r][k] = scale[r] * e4m3(code[r][k]); or with ORC_W_FP4 OCP MX FP4: E2M1 codes two per byte
 * (weight 2i in the low nibble of byte i of the row, 2i + 1 in the high nibble) and one E8M0 scale
 * byte per block of 32 consecutive weights of a row, W[r][k] = e8m0(S[r][k / 32]) * e2m1(code).
 * Norm gains, conv_w, embedding and LM head stay bf16. */
enum { ORC_W_BF16 = 0, ORC_W_FP8 = 1, ORC_W_FP4 = 2 };

typedef struct { /* [out][in] row-major; projections bf16 or fp8 (weight_format), the rest bf16 */
  const uint16_t *attn_norm;
  const void *wq, *wk, *wv, *wo;
  const uint16_t *q_norm, *k_norm;
  const void *w_qkv_delta, *w_gates;
  const uint16_t *conv_w;
  const void *wo_delta;
  const uint16_t *mlp_norm;
  const void *w_gate, *w_up, *w_down;
  /* the projection of the same name's scales: ORC_W_FP8 fp32 [out] row scales, ORC_W_FP4 E8M0
   * bytes [out][in / 32]; unused for bf16 */
  const void *s_wq, *s_wk, *s_wv, *s_wo, *s_w_qkv_delta, *s_w_gates, *s_wo_delta, *s_w_gate, *s_w_up, *s_w_down;
  /* n_experts > 0: router bf16 [n_experts][hidden]; w_gate / w_up are then [n_experts][ffn][hidden]
   * and w_down [n_experts][hidden][ffn], expert-major */
  const uint16_t* w_router;
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
 * mix_dim = max(n_q_heads*head_dim, n_delta_heads*delta_dv).  mlp_m is left untouched for MoE layers.
 * Mixture of experts (n_experts > 0):
 *   router  [L][B][n_experts] router logits
 *   sel     [L][B][top_k]     the experts this oracle's own routing chooses (descending logit,
 *                             ties to the lower index)
 *   force   [L][B][top_k]     input: when set, these experts are used instead of its own choice
 *                             (their weights still come from its own logits) */
typedef struct {
  float *x_mixer, *x_mlp, *mixer_o, *mlp_m, *final_r;
  float* router;
  int32_t* sel;
  const int32_t* force;
} orc_dump;

/* ---- building blocks (exported so the tests can pin each one) ---- */
float orc_bf16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float f);
/* y = x * (mean(x^2) + eps)^-1/2 * gain (gain may be NULL = 1) */
void orc_rmsnorm(const float* x, const uint16_t* gain, int n, double eps, float* y);
/* y[r] = sum_k W[r][k] x[k], W bf16 [rows][cols] */
void orc_matvec(const uint16_t* W, const float* x, int rows, int cols, float* y);
/* value of an OCP 8-bit floating-point E4M3 code (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent 0 is subnormal; 0x7F and 0xFF are NaN; no infinities; largest finite 448) */
double orc_e4m3(uint8_t code);
/* y[r] = scale[r] * sum_k e4m3(W[r][k]) x[k], W fp8 codes [rows][cols] */
void orc_matvec_fp8(const uint8_t* W, const float* scale, const float* x, int rows, int cols, float* y);
/* value of an OCP MX E2M1 code (low 4 bits: sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * exponent 0 is subnormal; no infinities or NaN; largest 6) */
double orc_e2m1(uint8_t code);
/* value of an OCP MX E8M0 scale byte: 2^(e - 127); 0xFF is NaN */
double orc_e8m0(uint8_t e);
/* y[r] = sum_k e8m0(S[r][k / 32]) e2m1(W[r][k]) x[k]; W packed E2M1 [rows][cols / 2], S E8M0
 * [rows][cols / 32]; cols a multiple of 32 */
void orc_matvec_fp4(const uint8_t* W, const uint8_t* S, const float* x, int rows, int cols, float* y);
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

/* the delta-rule mixer of one sequence from its projections u[C] (q | k | v) and gate logits a[2*heads]:
 * conv step (cs = that sequence's conv state [C][W-1], updated), per-head L2 norm of q and k (q also
 * scaled by dk^-1/2), g = sigmoid(a[h]), beta = sigmoid(a[heads+h]), state update and readout of every
 * head (st = that sequence's S^T [heads][dv][dk], updated); o[heads*dv]. */
void orc_delta_mixer(const orc_model* m, const uint16_t* conv_w, const float* u, const float* a, float* cs,
                     float* st, float* o);

/* ---- the decode step ----
 * For every b < batch: consume tokens[b] at position positions[b] (== ctx_lens[b]-1), append K/V
 * (or update the conv / delta states), write logits[b][vocab].  Returns 0 or a negative code for
 * inputs outside the contract (nothing is written then). */
int orc_decode_step(const orc_model* m, const orc_weights* w, orc_cache* c, const int32_t* tokens,
                    const int32_t* positions, const int32_t* ctx_lens, int batch, float* logits,
                    orc_dump* dump);

/* Mixture-of-experts routing of one sequence: the k largest of n router logits (ties to the lower
 * index), in descending order, into sel[k]. */
void orc_moe_select(const float* logits, int n, int k, int32_t* sel);
/* the weights of the k chosen experts: softmax over all n logits, renormalised over the chosen k
 * (so they sum to 1) */
void orc_moe_weights(const float* logits, int n, int k, const int32_t* sel, double* w);

/* greedy choice: argmax, ties to the lowest index */
int orc_argmax(const float* v, int n);

#ifdef __cplusplus
}
#endif
#endif
