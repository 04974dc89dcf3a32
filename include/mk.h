/*
 * mk.h -- C ABI of the persistent decode megakernel for AMD MI355X (gfx950).
 *
 * One call, mk_decode_step, runs a whole transformer decode step -- RMSNorm,
 * QKV projection, RoPE, paged KV-cache attention, o_proj, SwiGLU MLP and the
 * LM head, plus the gated delta-rule layers of hybrid models -- as ONE
 * persistent kernel launch.  This is the decode megakernel of the
 * ForgeMegakernel abstract (arxivdaily / arxiv.science, abstract): decode is
 * bandwidth bound because every weight and KV-cache byte crosses HBM once per
 * token, and the megakernel is built from a fine-grained per-compute-unit
 * instruction stream, dependency counters instead of grid-wide
 * synchronisation, and an on-chip buffer pool that stages weight and KV tiles.
 * The delta-rule layer follows the MK-KDA pull request (github
 * choiceoh/stkernel #230, phase chain in_proj -> gates -> conv -> delta ->
 * o_proj), whose host also refuses inputs outside the kernel's contract.
 *
 * Conventions
 *   - Every function returns mk_status; none throws, aborts or prints.  The
 *     text of the last failure on the calling thread is in mk_last_error().
 *   - "device pointer" = memory on the GPU the context was created on; the
 *     caller allocates all of it (PyTorch in the Python binding) and keeps it
 *     alive for the lifetime of the context.  The library BORROWS it.
 *   - Every device pointer must be 16-byte aligned (MK_ERR_INVALID_ARG).
 *   - bf16 tensors are raw bf16 bit patterns (uint16), row-major, weights in
 *     [out_features][in_features] order.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 1u

typedef enum {
  MK_OK = 0,
  MK_ERR_INVALID_ARG = -1,  /* null / misaligned pointer, out-of-range size, bad batch */
  MK_ERR_UNSUPPORTED = -2,  /* a model shape the kernel was not built for */
  MK_ERR_HIP = -3,          /* a HIP runtime call failed (message in mk_last_error) */
  MK_ERR_DEVICE_INPUT = -4, /* the device found an out-of-contract token/position/page (sticky) */
  MK_ERR_TIMEOUT = -5,      /* a dependency wait exceeded its spin limit (sticky) */
  MK_ERR_STATE = -6         /* the context is in an error state; call mk_reset */
} mk_status;

typedef enum { MK_LAYER_ATTN = 0, MK_LAYER_DELTA = 1 } mk_layer_kind;

/* Model description (host memory; copied by mk_create).
 *   hidden % 8 == 0, head_dim in {64, 128}, n_q_heads % n_kv_heads == 0,
 *   page_size == 16, delta_dk == 128 or 64, delta_dv % 32 == 0, conv_width == 4.
 * RMSNorm: y = x * (mean(x^2) + rms_eps)^-1/2 * gain.  RoPE: rotate-half pairs
 * (i, i + d/2) at angle pos * rope_base^(-2i/d).  Query head h reads KV head
 * floor(h * n_kv_heads / n_q_heads).  Delta layers (hybrid): in_proj to
 * [q | k | v] (heads * (2*dk + dv) channels), gates projection to
 * [g-logits | beta-logits] (2 * heads), causal depthwise conv of width
 * conv_width with a rolling state, SiLU, per-head L2 norm of q and k, q
 * scaled by dk^-1/2, g = sigmoid, beta = sigmoid, S <- g S + beta k (v^T - k^T S),
 * o = S^T q.  The mixer norm of a delta layer uses attn_norm. */
typedef struct {
  uint32_t abi_version;     /* MK_ABI_VERSION */
  uint32_t struct_size;     /* sizeof(mk_model_desc) */
  int32_t n_layers, hidden, vocab, ffn;
  int32_t n_q_heads, n_kv_heads, head_dim, qk_norm, tied_embeddings;
  float rms_eps, rope_base;
  int32_t n_delta_heads, delta_dk, delta_dv, conv_width; /* 0 when there are no delta layers */
  const int32_t* layer_kind; /* host array [n_layers] of mk_layer_kind */
  int32_t max_batch, max_ctx, page_size;
} mk_model_desc;

/* Per-layer weights: device pointers to bf16.  Attention layers set attn_norm,
 * wq [Hq*d][H], wk [Hkv*d][H], wv [Hkv*d][H], wo [H][Hq*d] and, with qk_norm,
 * q_norm [d], k_norm [d].  Delta layers set attn_norm, w_qkv_delta [C][H],
 * w_gates [2*heads][H], conv_w [C][conv_width], wo_delta [H][heads*dv].
 * Every layer sets mlp_norm [H], w_gate [F][H], w_up [F][H], w_down [H][F].
 * Unused fields may be NULL. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *q_norm, *k_norm;
  const void *w_qkv_delta, *w_gates, *conv_w, *wo_delta;
  const void *mlp_norm, *w_gate, *w_up, *w_down;
} mk_layer_weights;

typedef struct {
  const void* embed;       /* bf16 [vocab][hidden] */
  const void* final_norm;  /* bf16 [hidden] */
  const void* lm_head;     /* bf16 [vocab][hidden]; ignored (== embed) when tied_embeddings */
  const mk_layer_weights* layers; /* HOST array [n_layers] */
} mk_weights;

/* Caller-owned decode state (device pointers).  Paged KV cache: page_size
 * positions per page, logical page p of sequence b is physical page
 * page_table[b][p].  Delta layers keep S transposed (S^T[dv][dk], fp32) and the
 * last conv_width-1 pre-conv inputs per channel, oldest first. */
typedef struct {
  void* k_pages;  /* bf16 [n_attn_layers][num_pages][n_kv_heads][page_size][head_dim] */
  void* v_pages;  /* same layout */
  int32_t num_pages, max_pages_per_seq;
  const int32_t* page_table; /* int32 [max_batch][max_pages_per_seq] */
  float* delta_state;        /* fp32 [n_delta_layers][max_batch][heads][dv][dk] or NULL */
  float* conv_state;         /* fp32 [n_delta_layers][max_batch][C][conv_width-1] or NULL */
} mk_kv_cache;

typedef struct mk_ctx mk_ctx; /* opaque, library-owned host object */

/* Bytes of device workspace mk_create needs for this model (queues, dependency
 * counters, RoPE table, inter-op activations, attention partials). */
mk_status mk_workspace_size(const mk_model_desc* desc, size_t* bytes);

/* Compile the model into per-compute-unit instruction queues and upload them
 * into `workspace` (device memory of at least mk_workspace_size bytes, caller
 * owned, 256-byte aligned).  Synchronous.  On success *out owns host state only. */
mk_status mk_create(const mk_model_desc* desc, const mk_weights* weights, const mk_kv_cache* cache,
                    void* workspace, size_t workspace_bytes, mk_ctx** out);

/* One decode step for sequences b < batch: consume tokens[b] at position
 * positions[b] (== ctx_lens[b] - 1, ctx_lens counts cached tokens including
 * the new one), append its K/V (or update its conv / delta state) and write
 * fp32 logits_out[b][vocab].  tokens, positions, ctx_lens are device int32
 * arrays; pages for positions[b] must already be mapped in page_table.
 * Asynchronous on hip_stream (a hipStream_t; NULL = default stream).
 * Host-detected errors return at once with nothing enqueued.  Device-detected
 * input errors are sticky: the offending row gets NaN logits and no cache or
 * state write, and mk_sync_status reports MK_ERR_DEVICE_INPUT. */
mk_status mk_decode_step(mk_ctx* ctx, const int32_t* tokens, const int32_t* positions, const int32_t* ctx_lens,
                         int32_t batch, float* logits_out, void* hip_stream);

/* Wait for the last step and return the sticky device status. */
mk_status mk_sync_status(mk_ctx* ctx);

/* Clear the sticky error and all dependency counters (synchronous). */
mk_status mk_reset(mk_ctx* ctx);

/* Thread-local text for the last failing call on this thread ("" if none). */
const char* mk_last_error(void);

void mk_destroy(mk_ctx* ctx);

/* ---- introspection (host-only; no GPU needed) ---- */
typedef struct {
  int32_t n_cus;            /* compute units the plan was made for */
  int32_t n_ops, n_stages;  /* queue entries over all units, dependency stages */
  int32_t max_ops_per_cu;
  double weight_bytes;      /* weight bytes streamed per step */
  double max_cu_bytes, mean_cu_bytes; /* per-unit streamed weight bytes (balance) */
  int32_t errors;           /* violations found by the plan checker (0 = valid) */
} mk_plan_info;

/* Run the scheduler and its checker on the host for n_cus compute units. */
mk_status mk_plan(const mk_model_desc* desc, int32_t n_cus, mk_plan_info* info);

/* ---- mid-state access for checking against the oracle ---- */
typedef enum {
  MK_MID_X_MIXER = 0, /* fp32 [batch][hidden] residual after layer l's attention / delta sub-layer */
  MK_MID_X_MLP = 1,   /* fp32 [batch][hidden] residual after layer l's MLP */
  MK_MID_MIXER_O = 2, /* fp32 [batch][Hq*d or heads*dv] attention / delta output before o_proj */
  MK_MID_MLP_M = 3,   /* fp32 [batch][ffn] silu(gate) * up */
  MK_MID_PROJ = 4,    /* fp32 [batch][(Hq+2Hkv)*d] raw q|k|v of an attention layer (before norm / RoPE),
                         or [batch][C + 2*heads] in_proj|gates of a delta layer (before the conv) */
  MK_MID_EMBED = 5    /* fp32 [batch][hidden] embedding rows (layer ignored) */
} mk_midstate;

/* Copy mid-state `kind` of `layer` from the last step into dst (device memory,
 * fp32, `count` floats = batch * width), ordered on hip_stream. */
mk_status mk_copy_midstate(mk_ctx* ctx, int32_t kind, int32_t layer, float* dst, size_t count, void* hip_stream);

/* ---- per-op timing trace (diagnostic) ----
 * With MK_TRACE=1 in the environment at mk_create, the kernel records for every queue entry the
 * low 32 bits of the GPU's 100 MHz real-time clock when the op starts, when its inputs are in
 * hand (projections and attention: after the input poll; other ops: = start) and when it ends
 * (after the closing barrier of its workgroup), plus its opcode and stage.  The library owns the
 * trace buffer (allocated at mk_create only in this mode).
 * mk_copy_trace waits for the last step and copies into host memory `dst` (`count` uint32):
 *   [0] n_ops, [1] n_cus, [2 .. 2+n_cus] queue offsets (op range of CU c: [off[c], off[c+1])),
 *   then per op 4 words {opcode << 16 | stage, t_start, t_ready, t_end}.
 * Returns MK_ERR_STATE when tracing is off and MK_ERR_INVALID_ARG when count is too small
 * (mk_trace_words gives the size). */
mk_status mk_trace_words(mk_ctx* ctx, size_t* count);
mk_status mk_copy_trace(mk_ctx* ctx, uint32_t* dst, size_t count);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
