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

#define MK_ABI_VERSION 3u

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

/* Projection weight formats.  Low-bit weight streaming is how the MK-KDA pull request (github
 * choiceoh/stkernel #230, PR summary: its W4 weight stream; fp8 o_proj operands) cuts the bytes a
 * decode step moves; at 8 bits it halves them against bf16.
 *   MK_WEIGHTS_BF16     every projection bf16.
 *   MK_WEIGHTS_FP8_E4M3 every projection matrix (wq wk wv wo w_qkv_delta w_gates wo_delta w_gate
 *                       w_up w_down) is one OCP 8-bit floating-point E4M3 code per weight (sign,
 *                       4 exponent bits with bias 7, 3 mantissa bits, exponent 0 subnormal, 0x7F /
 *                       0xFF NaN, no infinities), [out][in] row-major, with one fp32 scale per
 *                       output row: W[r][k] = scale[r] * e4m3(code[r][k]).  Embedding, LM head,
 *                       norm gains, conv taps and the KV cache stay bf16.  Codes must not be
 *                       NaN.  Every projection input length (hidden, ffn, n_q_heads * head_dim,
 *                       n_delta_heads * delta_dv) must be a multiple of 16, of 512 when max_batch
 *                       is 5 to 8; otherwise mk_create / mk_plan return MK_ERR_UNSUPPORTED.
 *   MK_WEIGHTS_FP4_MX   every projection matrix is OCP MX fp4: E2M1 codes (sign, 2 exponent bits
 *                       with bias 1, 1 mantissa bit, exponent 0 subnormal; values 0 .. 6, no
 *                       infinities or NaN) packed two per byte, weight 2i of a row in the low
 *                       nibble of byte i and 2i + 1 in the high nibble, uint8 [out][in / 2]; with
 *                       one E8M0 scale byte (2^(e - 127), 0xFF NaN: not allowed) per block of 32
 *                       consecutive weights of a row, uint8 [out][in / 32]:
 *                       W[r][k] = 2^(S[r][k / 32] - 127) * e2m1(code(r, k)).  The same tensors
 *                       stay bf16 as for fp8.  One sequence per step: max_batch must be 1, and
 *                       every projection input length a multiple of 32 (at most 16384);
 *                       otherwise MK_ERR_UNSUPPORTED. */
typedef enum { MK_WEIGHTS_BF16 = 0, MK_WEIGHTS_FP8_E4M3 = 1, MK_WEIGHTS_FP4_MX = 2 } mk_weight_format;

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
  int32_t weight_format;     /* mk_weight_format of the projection matrices */
  /* Mixture of experts (0 = dense MLPs).  With n_experts > 0 every layer's MLP is top_k of
   * n_experts SwiGLU experts of width ffn: router logits z = w_router RMSNorm(x), the top_k experts
   * of each sequence by logit (ties to the lower index), weights softmax(z) renormalised over the
   * chosen, and x += sum of the chosen experts' outputs times their weights (the "full layer (MoE +
   * Attention) megakernel" of the Muse Spark post, LMSYS, as summarised on the khabar-ai page).
   * n_experts <= 64, 1 <= top_k <= min(8, n_experts), bf16 weights, max_batch <= 4, no verify
   * windows; otherwise MK_ERR_UNSUPPORTED. */
  int32_t n_experts, top_k;
} mk_model_desc;

/* Per-layer weights: device pointers to bf16 (projections in the model's weight_format).
 * Attention layers set attn_norm, wq [Hq*d][H], wk [Hkv*d][H], wv [Hkv*d][H], wo [H][Hq*d] and,
 * with qk_norm, q_norm [d], k_norm [d].  Delta layers set attn_norm, w_qkv_delta [C][H],
 * w_gates [2*heads][H], conv_w [C][conv_width], wo_delta [H][heads*dv].
 * Every layer sets mlp_norm [H], w_gate [F][H], w_up [F][H], w_down [H][F].
 * With MK_WEIGHTS_FP8_E4M3 each projection the layer sets also sets its <name>_scale: fp32 [out]
 * row scales (device, 16-byte aligned); with MK_WEIGHTS_FP4_MX its E8M0 block scales, uint8
 * [out][in / 32] (device, 16-byte aligned).  Unused fields may be NULL. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *q_norm, *k_norm;
  const void *w_qkv_delta, *w_gates, *conv_w, *wo_delta;
  const void *mlp_norm, *w_gate, *w_up, *w_down;
  const void *wq_scale, *wk_scale, *wv_scale, *wo_scale, *w_qkv_delta_scale, *w_gates_scale, *wo_delta_scale;
  const void *w_gate_scale, *w_up_scale, *w_down_scale;
  /* n_experts > 0: router bf16 [n_experts][H]; w_gate and w_up are then [n_experts][F][H] and
   * w_down [n_experts][H][F], expert-major, each one allocation */
  const void* w_router;
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
 * counters, RoPE table, inter-op activations, attention partials, the per-op trace
 * section and the multi-step words): the instruction streams, dependency state and
 * staging a decode megakernel keeps (ForgeMegakernel abstract). */
mk_status mk_workspace_size(const mk_model_desc* desc, size_t* bytes);

/* Compile the model into per-compute-unit instruction queues (the fine-grained
 * instruction stream per compute unit of the ForgeMegakernel abstract) and upload
 * them into `workspace` (device memory of at least mk_workspace_size bytes, caller
 * owned, 256-byte aligned).  Synchronous.  On success *out owns host state only. */
mk_status mk_create(const mk_model_desc* desc, const mk_weights* weights, const mk_kv_cache* cache,
                    void* workspace, size_t workspace_bytes, mk_ctx** out);

/* One decode step -- the whole step in one persistent launch (the decode
 * megakernel of the ForgeMegakernel abstract) -- for sequences b < batch: consume tokens[b] at position
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

/* n_steps greedy decode steps in ONE launch, the token fed back on the GPU.  The launch count
 * per decoded token is what the Muse Spark megakernel posts (khabar-ai page, the post on SGLang
 * megakernels: launches per decode step) cut; the greedy choice is the argmax the ForgeMegakernel
 * abstract's decode produces token by token.  Step s (0 <= s < n_steps) of sequence b consumes
 * tokens[b] (s = 0) or tokens_out[s-1][b] at position positions[b] + s with ctx_lens[b] + s cached
 * tokens, exactly as n_steps calls of mk_decode_step would, and writes
 *   logits_out[s][b][vocab]  fp32, device, 16-byte aligned, n_steps * batch * vocab floats;
 *   tokens_out[s][b]         int32, device, 16-byte aligned: argmax of that step's logits (ties
 *                            to the lowest index; -1 where the row was out of contract).
 * Pages for positions[b] .. positions[b] + n_steps - 1 must be mapped.  1 <= n_steps <=
 * MK_MAX_STEPS.  Asynchronous on hip_stream; errors as for mk_decode_step (a row that leaves the
 * contract at some step -- its position past max_ctx, an unmapped page -- raises the sticky
 * MK_ERR_DEVICE_INPUT and gets NaN logits from that step on). */
#define MK_MAX_STEPS 4096
mk_status mk_decode_steps(mk_ctx* ctx, const int32_t* tokens, const int32_t* positions, const int32_t* ctx_lens,
                          int32_t batch, int32_t n_steps, float* logits_out, int32_t* tokens_out, void* hip_stream);

/* A speculative-decoding verify window: `window` consecutive tokens of each sequence in ONE step,
 * as the MK-KDA pull request's multi-token window runs (github choiceoh/stkernel #230, commit
 * message: a spec window of at most 8 query tokens, the host refusing wider ones).  Token t
 * (0 <= t < window) of sequence b is tokens[b * window + t] at position positions[b] + t and sees
 * ctx_lens[b] + t cached tokens (positions[b] == ctx_lens[b] - 1): the cache up to positions[b]
 * and the window's earlier tokens, exactly as `window` calls of mk_decode_step fed these tokens
 * would.  Every window token's K/V is appended.  logits_out[b][t][vocab] fp32 (device, 16-byte
 * aligned).  1 <= window <= MK_MAX_WINDOW, batch * window <= max_batch (the window's tokens run
 * as rows of the batched projections).  Pages for positions[b] .. positions[b] + window - 1 must
 * be mapped.  Delta-rule layers run their recurrence over the window's tokens in order (the conv
 * window rolling through them, the state written back after the last); a sequence with any window
 * token out of contract gets zero outputs and no state write.  Asynchronous on hip_stream; errors
 * as for mk_decode_step. */
#define MK_MAX_WINDOW 8
mk_status mk_decode_window(mk_ctx* ctx, const int32_t* tokens, const int32_t* positions, const int32_t* ctx_lens,
                           int32_t batch, int32_t window, float* logits_out, void* hip_stream);

/* mk_create for callers that cannot allocate device memory (code under HIP graph capture,
 * allocation-free serving loops, harnesses that forbid hipMalloc): the same context, with the
 * library's static device scratch of MK_STATIC_SCRATCH_BYTES as its workspace instead of a
 * caller-provided one.  Allocates no device memory (no hipMalloc / hipFree); it clears the scratch
 * with a fill kernel and uploads the plan, synchronously.  Each GPU holds one such scratch for
 * the life of the process, shared by every call on that GPU: a later mk_create_static on the same
 * GPU takes it over, after which the earlier context's calls return MK_ERR_STATE (destroy it).
 * Contexts on one GPU's scratch must not be stepped concurrently (they would race).
 * MK_ERR_INVALID_ARG when the model's workspace (mk_workspace_size) exceeds the scratch. */
#define MK_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
mk_status mk_create_static(const mk_model_desc* desc, const mk_weights* weights, const mk_kv_cache* cache,
                           mk_ctx** out);

/* Wait for the last step and return the sticky device status: input-contract violations the
 * kernel found (the contract the MK-KDA pull request's host check enforces, github
 * choiceoh/stkernel #230) or a dependency wait that hit the watchdog. */
mk_status mk_sync_status(mk_ctx* ctx);

/* Clear the sticky error, the dependency counters and the tagged activations, and restart the
 * step tags (synchronous): the recovery path after MK_ERR_DEVICE_INPUT or MK_ERR_TIMEOUT. */
mk_status mk_reset(mk_ctx* ctx);

/* Thread-local text for the last failing call on this thread ("" if none).  (Library
 * housekeeping; no passage of the pages defines it.) */
const char* mk_last_error(void);

/* Free the host state of a context (the caller's device buffers are untouched). */
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

/* Run the scheduler -- the host side that compiles a model into per-unit instruction streams
 * and dependency stages (ForgeMegakernel abstract) -- and its checker on the host for n_cus
 * compute units. */
mk_status mk_plan(const mk_model_desc* desc, int32_t n_cus, mk_plan_info* info);

/* ---- dependency-protocol emulator (host-only; no GPU needed) ----
 * The abstract's megakernel replaces grid-wide synchronisation with dependencies between the
 * compute units' instruction streams (ForgeMegakernel abstract, arxivdaily / arxiv.science); here
 * a consumer polls its inputs for the launch's parity, which is sound only if every value it may
 * poll is written exactly once per launch.  mk_emulate replays the queues mk_create would upload
 * (the same scheduler, and the kernel's own attention planner) for n_cus compute units over
 * n_launches launches, in a random interleaving drawn from `seed`, and reports what it found:
 * polls satisfied by an earlier launch's value, reads after a counter wait that found unwritten
 * data, values written twice or not at all in a launch, and launches in which every remaining
 * unit waits (where the kernel's watchdog would end the step).  Positions are ctx_lens - 1.
 * Returns MK_OK when the run completed (findings are in *rep; their text in mk_last_error()),
 * MK_ERR_INVALID_ARG / MK_ERR_UNSUPPORTED for bad arguments or descriptions. */
#define MK_EMU_COUNTERS 1u          /* every dependency through stage counters (the diagnostic plan) */
#define MK_EMU_IDLE_ITEMS_SILENT 2u /* model a kernel whose attention items without a chunk write nothing */
#define MK_EMU_DEAD_ROWS_SILENT 4u  /* model a kernel that writes no mixer rows for sequences outside the
                                       step and polls only the rows of live sequences */
#define MK_EMU_STALL_ONE_OP 8u      /* one op of the first launch never writes (a stuck producer) */
typedef struct {
  int32_t n_cus;            /* compute units to emulate (>= 1) */
  int32_t n_launches;       /* launches in the sequence */
  const int32_t* batch;     /* host [n_launches]: batch of each launch, in [1, max_batch] */
  const int32_t* ctx_lens;  /* host [n_launches][max_batch]: context lengths; entries past batch ignored */
  uint64_t seed;            /* interleaving seed */
  uint32_t flags;           /* MK_EMU_* */
} mk_emu_config;
typedef struct {
  int64_t ops_run, polls;   /* ops completed, polls satisfied */
  int64_t stale_accepts;    /* polls that accepted a value written by an earlier launch */
  int64_t unsynced_reads;   /* reads after a counter wait that found a value not written this launch */
  int64_t double_writes;    /* tagged values written twice in one launch */
  int64_t unwritten_cells;  /* pollable values not written in a launch */
  int32_t deadlocks;        /* launches that stopped with every remaining unit waiting */
  int32_t first_bad_launch; /* first launch with a finding, -1 if none */
} mk_emu_report;
mk_status mk_emulate(const mk_model_desc* desc, const mk_emu_config* cfg, mk_emu_report* rep);

/* ---- mid-state access for checking against the oracle ---- */
typedef enum {
  MK_MID_X_MIXER = 0, /* fp32 [batch][hidden] residual after layer l's attention / delta sub-layer */
  MK_MID_X_MLP = 1,   /* fp32 [batch][hidden] residual after layer l's MLP */
  MK_MID_MIXER_O = 2, /* fp32 [batch][Hq*d or heads*dv] attention / delta output before o_proj */
  MK_MID_MLP_M = 3,   /* fp32 [batch][ffn] silu(gate) * up */
  MK_MID_PROJ = 4,    /* fp32 [batch][(Hq+2Hkv)*d] raw q|k|v of an attention layer (before norm / RoPE),
                         or [batch][C + 2*heads] in_proj|gates of a delta layer (before the conv) */
  MK_MID_EMBED = 5,   /* fp32 [batch][hidden] embedding rows (layer ignored) */
  MK_MID_ROUTER = 6   /* fp32 [batch][n_experts] router logits of a mixture-of-experts layer */
} mk_midstate;

/* Copy mid-state `kind` of `layer` from the last step into dst (device memory,
 * fp32, `count` floats = batch * width), ordered on hip_stream: the intermediate states an
 * independent mid-state oracle checks (ForgeMegakernel abstract). */
mk_status mk_copy_midstate(mk_ctx* ctx, int32_t kind, int32_t layer, float* dst, size_t count, void* hip_stream);

/* ---- per-op timing trace (diagnostic) ----
 * With MK_TRACE=1 in the environment at mk_create, the kernel records for every queue entry the
 * low 32 bits of the GPU's 100 MHz real-time clock when the op starts, when its inputs are in
 * hand (projections and attention: after the input poll; other ops: = start) and when it ends
 * (after the closing barrier of its workgroup), plus its opcode and stage, in a section of the
 * caller's workspace (the multi-step kernels record none).
 * mk_copy_trace waits for the last step and copies into host memory `dst` (`count` uint32):
 *   [0] n_ops, [1] n_cus, [2 .. 2+n_cus] queue offsets (op range of CU c: [off[c], off[c+1])),
 *   then per op 8 words {opcode << 16 | stage, t_start, t_ready, t_end, loader first issue, loader
 *   last issue, loader ticks blocked on a full ring, 0} (the loader wave streams the op's bytes).
 * Returns MK_ERR_STATE when tracing is off and MK_ERR_INVALID_ARG when count is too small
 * (mk_trace_words gives the size). */
mk_status mk_trace_words(mk_ctx* ctx, size_t* count);
mk_status mk_copy_trace(mk_ctx* ctx, uint32_t* dst, size_t count);

/* Measurement aid: a plain streaming read of `bytes` (a multiple of 16) of device memory at `buf`
 * (16-byte aligned), every byte once, by `blocks` workgroups of 256 threads (1..65536) in a
 * grid-stride loop of non-temporal 16-byte loads, eight in flight per thread; `out` (device,
 * `blocks` uint32) receives one XOR fold per workgroup so the loads cannot be dropped.  It is the achievable-read ceiling the decode kernel's
 * HBM rate is set against (the roofline of a weight-streaming decode step, ForgeMegakernel
 * abstract: decode is bound by the bytes it reads).  Asynchronous on hip_stream. */
mk_status mk_stream_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
