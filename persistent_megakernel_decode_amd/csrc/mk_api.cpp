// mk_api.cpp -- the C ABI declared in include/mk.h.
//
// Host side of the persistent decode megakernel: input contracts (the MK-KDA
// pull request, github choiceoh/stkernel #230, host check hunk: the host
// refuses inputs outside the kernel's contract before launching), workspace
// layout, plan upload and the single cooperative launch per decode step.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/mk.h"
#include "mk_internal.h"
#include "mk_sched.h"

extern "C" __global__ void mk_megakernel_b1(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b2(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b4(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b1_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b2_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b4_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b8_trace(mk::KArgs A);

namespace {

thread_local std::string g_last_error;

mk_status fail(mk_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

mk_status hip_fail(hipError_t e, const char* what) {
  return fail(MK_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define MK_HIP(call)                                \
  do {                                              \
    hipError_t e_ = (call);                         \
    if (e_ != hipSuccess) return hip_fail(e_, #call); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

const void* kernel_for(int B, bool traced) {
  switch (B) {
    case 1: return traced ? (const void*)mk_megakernel_b1_trace : (const void*)mk_megakernel_b1;
    case 2: return traced ? (const void*)mk_megakernel_b2_trace : (const void*)mk_megakernel_b2;
    case 4: return traced ? (const void*)mk_megakernel_b4_trace : (const void*)mk_megakernel_b4;
    default: return traced ? (const void*)mk_megakernel_b8_trace : (const void*)mk_megakernel_b8;
  }
}

__global__ void fill_u32(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

}  // namespace

struct mk_ctx {
  mk::ModelShape shape;
  mk::Plan plan;
  int device = 0;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  mk::KArgs args{};
  uint32_t epoch = 0;
  uint32_t tag = 0;  // launch tag of the last launch (activation parity = bit 0)
  uint32_t max_stage_ops = 1;
  hipStream_t last_stream = nullptr;
  mk_status sticky = MK_OK;
  const void* kernel = nullptr;
  bool plain_launch = false;
  uint32_t* trace = nullptr;  // MK_TRACE=1: device buffer, 4 words per op (library-owned)
  std::mutex busy;
  ~mk_ctx() {
    if (trace) (void)hipFree(trace);
  }
};

extern "C" {

const char* mk_last_error(void) { return g_last_error.c_str(); }

static int device_cus(int* n) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return dev;
}

mk_status mk_workspace_size(const mk_model_desc* desc, size_t* bytes) {
  if (!bytes) return fail(MK_ERR_INVALID_ARG, "bytes is null");
  mk::ModelShape m;
  mk_status st;
  std::string e = mk::validate_desc(desc, &m, &st);
  if (!e.empty()) return fail(st, e);
  int ncu = 0;
  if (device_cus(&ncu) < 0) return fail(MK_ERR_HIP, "cannot query the current HIP device");
  mk::Plan p;
  e = mk::build_plan(m, ncu, nullptr, nullptr, &p);
  if (!e.empty()) return fail(MK_ERR_UNSUPPORTED, e);
  *bytes = p.lay.total;
  return MK_OK;
}

mk_status mk_plan(const mk_model_desc* desc, int32_t n_cus, mk_plan_info* info) {
  if (!info) return fail(MK_ERR_INVALID_ARG, "info is null");
  mk::ModelShape m;
  mk_status st;
  std::string e = mk::validate_desc(desc, &m, &st);
  if (!e.empty()) return fail(st, e);
  mk::Plan p;
  e = mk::build_plan(m, n_cus, nullptr, nullptr, &p);
  if (!e.empty()) return fail(MK_ERR_UNSUPPORTED, e);
  std::string why;
  info->errors = mk::check_plan(m, p, &why);
  info->n_cus = n_cus;
  info->n_ops = (int32_t)p.ops.size();
  info->n_stages = (int32_t)p.stages.size();
  info->max_ops_per_cu = 0;
  for (int c = 0; c < n_cus; ++c)
    info->max_ops_per_cu = std::max<int32_t>(info->max_ops_per_cu, (int32_t)(p.queue_off[c + 1] - p.queue_off[c]));
  info->weight_bytes = p.weight_bytes;
  double mx = 0, sum = 0;
  for (double b : p.cu_bytes) { mx = std::max(mx, b); sum += b; }
  info->max_cu_bytes = mx;
  info->mean_cu_bytes = sum / n_cus;
  if (info->errors) g_last_error = why;
  return MK_OK;
}

mk_status mk_create(const mk_model_desc* desc, const mk_weights* w, const mk_kv_cache* c, void* workspace,
                    size_t workspace_bytes, mk_ctx** out) {
  if (!out) return fail(MK_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  mk::ModelShape m;
  mk_status st;
  std::string e = mk::validate_desc(desc, &m, &st);
  if (!e.empty()) return fail(st, e);
  if (!w || !c || !workspace) return fail(MK_ERR_INVALID_ARG, "weights, cache and workspace must be non-null");
  if (((uintptr_t)workspace & 255u) != 0) return fail(MK_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const mk_model_desc& d = m.d;
  // pointer contract: every tensor the model uses is present and 16-byte aligned
  auto need = [&](const void* p, const char* name) -> std::string {
    if (!p) return std::string(name) + " is null";
    if (!aligned16(p)) return std::string(name) + " is not 16-byte aligned";
    return "";
  };
  std::string pe;
  if (pe.empty()) pe = need(w->embed, "embed");
  if (pe.empty()) pe = need(w->final_norm, "final_norm");
  if (pe.empty() && !d.tied_embeddings) pe = need(w->lm_head, "lm_head");
  if (pe.empty() && !w->layers) pe = "layers is null";
  for (int l = 0; pe.empty() && l < d.n_layers; ++l) {
    const mk_layer_weights& L = w->layers[l];
    pe = need(L.attn_norm, "attn_norm");
    if (pe.empty()) pe = need(L.mlp_norm, "mlp_norm");
    if (pe.empty()) pe = need(L.w_gate, "w_gate");
    if (pe.empty()) pe = need(L.w_up, "w_up");
    if (pe.empty()) pe = need(L.w_down, "w_down");
    if (m.kinds[l] == MK_LAYER_ATTN) {
      if (pe.empty()) pe = need(L.wq, "wq");
      if (pe.empty()) pe = need(L.wk, "wk");
      if (pe.empty()) pe = need(L.wv, "wv");
      if (pe.empty()) pe = need(L.wo, "wo");
      if (pe.empty() && d.qk_norm) pe = need(L.q_norm, "q_norm");
      if (pe.empty() && d.qk_norm) pe = need(L.k_norm, "k_norm");
    } else {
      if (pe.empty()) pe = need(L.w_qkv_delta, "w_qkv_delta");
      if (pe.empty()) pe = need(L.w_gates, "w_gates");
      if (pe.empty()) pe = need(L.conv_w, "conv_w");
      if (pe.empty()) pe = need(L.wo_delta, "wo_delta");
    }
    if (!pe.empty()) pe = "layer " + std::to_string(l) + ": " + pe;
  }
  if (pe.empty() && m.n_attn) {
    pe = need(c->k_pages, "k_pages");
    if (pe.empty()) pe = need(c->v_pages, "v_pages");
    if (pe.empty()) pe = need(c->page_table, "page_table");
    if (pe.empty() && (c->num_pages < 1 || c->max_pages_per_seq < 1)) pe = "num_pages and max_pages_per_seq must be positive";
    if (pe.empty() && (int64_t)c->max_pages_per_seq * d.page_size < d.max_ctx)
      pe = "max_pages_per_seq * page_size must cover max_ctx";
  }
  if (pe.empty() && m.n_delta) {
    pe = need(c->delta_state, "delta_state");
    if (pe.empty()) pe = need(c->conv_state, "conv_state");
  }
  if (!pe.empty()) return fail(MK_ERR_INVALID_ARG, pe);

  int ncu = 0;
  const int dev = device_cus(&ncu);
  if (dev < 0) return fail(MK_ERR_HIP, "cannot query the current HIP device");
  mk_ctx* ctx = new mk_ctx();
  ctx->shape = m;
  ctx->device = dev;
  e = mk::build_plan(m, ncu, w, c, &ctx->plan);
  if (!e.empty()) { delete ctx; return fail(MK_ERR_UNSUPPORTED, e); }
  std::string why;
  if (mk::check_plan(m, ctx->plan, &why)) { delete ctx; return fail(MK_ERR_UNSUPPORTED, "plan check failed: " + why); }
  mk::Plan& P = ctx->plan;
  if (workspace_bytes < P.lay.total) {
    delete ctx;
    return fail(MK_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(P.lay.total) + " bytes");
  }
  ctx->ws = (char*)workspace;
  ctx->ws_bytes = workspace_bytes;
  // MK_TRACE=1: the traced kernels (per-op timing stamps; diagnostic)
  const char* trace_env = getenv("MK_TRACE");
  const bool traced = trace_env && atoi(trace_env) != 0;
  ctx->kernel = kernel_for(P.kernel_batch, traced);

  // one resident workgroup per compute unit is required by the persistent design
  int per_cu = 0;
  hipError_t he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ctx->kernel, mk::NTHREADS, 0);
  if (he != hipSuccess || per_cu < 1) {
    delete ctx;
    return fail(MK_ERR_UNSUPPORTED, "the megakernel cannot be resident on a compute unit");
  }

  mk::relocate(&P, (uint64_t)(uintptr_t)workspace);
  const mk::Layout& Y = P.lay;
  // zero everything (activations, counters, tickets, status), then upload the plan
  he = hipMemset(workspace, 0, Y.total);
  if (he == hipSuccess) he = hipMemcpy(ctx->ws + Y.ops, P.ops.data(), P.ops.size() * sizeof(mk::Op), hipMemcpyHostToDevice);
  if (he == hipSuccess)
    he = hipMemcpy(ctx->ws + Y.queue_off, P.queue_off.data(), P.queue_off.size() * 4, hipMemcpyHostToDevice);
  if (he == hipSuccess)
    he = hipMemcpy(ctx->ws + Y.stages, P.stages.data(), P.stages.size() * sizeof(mk::Stage), hipMemcpyHostToDevice);
  if (he == hipSuccess)
    he = hipMemcpy(ctx->ws + Y.layers, P.layers.data(), P.layers.size() * sizeof(mk::LayerDesc), hipMemcpyHostToDevice);
  if (he == hipSuccess && m.n_attn) {  // RoPE table: angle pos * base^(-2i/d), computed in double
    const int hd = d.head_dim;
    std::vector<float> rope((size_t)d.max_ctx * hd);
    for (int p = 0; p < d.max_ctx; ++p)
      for (int i = 0; i < hd / 2; ++i) {
        const double th = (double)p * std::pow((double)d.rope_base, -2.0 * i / hd);
        rope[((size_t)p * (hd / 2) + i) * 2] = (float)std::cos(th);
        rope[((size_t)p * (hd / 2) + i) * 2 + 1] = (float)std::sin(th);
      }
    he = hipMemcpy(ctx->ws + Y.rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice);
  }
  if (he != hipSuccess) {
    delete ctx;
    return hip_fail(he, "uploading the plan");
  }
  uint32_t mx = 1;
  for (const auto& s : P.stages) mx = std::max(mx, s.nops);
  ctx->max_stage_ops = mx;

  mk::KArgs& A = ctx->args;
  A.ops = (const mk::Op*)(ctx->ws + Y.ops);
  A.queue_off = (const uint32_t*)(ctx->ws + Y.queue_off);
  A.stages = (const mk::Stage*)(ctx->ws + Y.stages);
  A.counters = (uint32_t*)(ctx->ws + Y.counters);
  A.layers = (const mk::LayerDesc*)(ctx->ws + Y.layers);
  A.rope = (const float*)(ctx->ws + Y.rope);
  A.status = (uint32_t*)(ctx->ws + Y.status);
  A.row_ok = (int32_t*)(ctx->ws + Y.row_ok);
  A.x0 = (float*)(ctx->ws + Y.x0);
  A.embed = (const uint16_t*)w->embed;
  A.page_table = m.n_attn ? c->page_table : nullptr;
  A.H = d.hidden; A.V = d.vocab; A.Hq = d.n_q_heads; A.Hkv = d.n_kv_heads; A.d = d.head_dim; A.G = m.G;
  A.qk_norm = d.qk_norm; A.max_batch = d.max_batch; A.max_ctx = d.max_ctx; A.page_size = d.page_size;
  A.num_pages = m.n_attn ? c->num_pages : 0;
  A.max_pages_per_seq = m.n_attn ? c->max_pages_per_seq : 1;
  A.nh = d.n_delta_heads; A.dk = d.delta_dk; A.dv = d.delta_dv; A.C = m.C; A.convw = d.conv_width;
  A.n_cus = ncu; A.n_items = P.n_items; A.mix = P.mix_dim;
  A.rms_eps = d.rms_eps;
  double ms = 2000.0;
  if (const char* s = getenv("MK_WATCHDOG_MS")) ms = std::max(1.0, atof(s));  // diagnostic only
  A.spin_limit = (uint64_t)(ms * 1e5);  // s_memrealtime runs at 100 MHz
  // Diagnostic: MK_PLAIN_LAUNCH=1 launches with hipLaunchKernel instead of the cooperative launch
  // (for tools that cannot follow cooperative dispatches).  mk_create has already checked that one
  // workgroup per CU is resident; should some workgroup still not be scheduled, the spin-wait
  // watchdog ends every wait and the step reports MK_ERR_TIMEOUT.
  if (const char* s = getenv("MK_PLAIN_LAUNCH")) ctx->plain_launch = atoi(s) != 0;
  A.trace = nullptr;
  if (traced) {
    const size_t bytes = P.ops.size() * 4 * sizeof(uint32_t);
    he = hipMalloc((void**)&ctx->trace, bytes);
    if (he == hipSuccess) he = hipMemset(ctx->trace, 0, bytes);
    if (he != hipSuccess) {
      delete ctx;
      return hip_fail(he, "allocating the trace buffer");
    }
    A.trace = ctx->trace;
  }
  *out = ctx;
  return MK_OK;
}

static mk_status zero_counters(mk_ctx* ctx, hipStream_t s) {
  const mk::Layout& Y = ctx->plan.lay;
  hipLaunchKernelGGL(fill_u32, dim3(64), dim3(256), 0, s, (uint32_t*)(ctx->ws + Y.counters), Y.counters_bytes / 4, 0u);
  MK_HIP(hipGetLastError());
  return MK_OK;
}

mk_status mk_decode_step(mk_ctx* ctx, const int32_t* tokens, const int32_t* positions, const int32_t* ctx_lens,
                         int32_t batch, float* logits_out, void* hip_stream) {
  if (!ctx) return fail(MK_ERR_INVALID_ARG, "ctx is null");
  if (ctx->sticky != MK_OK) return fail(MK_ERR_STATE, "context holds a device error; call mk_reset");
  if (!tokens || !positions || !ctx_lens || !logits_out) return fail(MK_ERR_INVALID_ARG, "null input or output pointer");
  if (!aligned16(tokens) || !aligned16(positions) || !aligned16(ctx_lens) || !aligned16(logits_out))
    return fail(MK_ERR_INVALID_ARG, "inputs and logits must be 16-byte aligned");
  if (batch < 1 || batch > ctx->shape.d.max_batch)
    return fail(MK_ERR_INVALID_ARG, "batch " + std::to_string(batch) + " outside [1, max_batch]");
  std::unique_lock<std::mutex> lk(ctx->busy, std::try_to_lock);
  if (!lk.owns_lock()) return fail(MK_ERR_STATE, "another thread is stepping this context");
  hipStream_t s = (hipStream_t)hip_stream;
  // counters count cumulatively (epoch * ops); restart the epochs long before 32-bit overflow
  if ((uint64_t)(ctx->epoch + 1) * ctx->max_stage_ops >= (1ull << 31)) {
    mk_status r = zero_counters(ctx, s);
    if (r != MK_OK) return r;
    ctx->epoch = 0;
  }
  mk::KArgs A = ctx->args;
  A.tokens = tokens;
  A.positions = positions;
  A.ctx_lens = ctx_lens;
  A.logits = logits_out;
  A.batch = batch;
  A.epoch = ctx->epoch + 1;
  // consecutive launches alternate the parity; the 31-bit tag restarts at 1 or 2 to keep it so
  A.tag = ctx->tag + 1 <= 0x7FFFFFFFu ? ctx->tag + 1 : (ctx->tag & 1u) ? 2u : 1u;
  void* kargs[] = {&A};
  hipError_t e = ctx->plain_launch
                     ? hipLaunchKernel(ctx->kernel, dim3(ctx->plan.n_cus), dim3(mk::NTHREADS), kargs, 0, s)
                     : hipLaunchCooperativeKernel(ctx->kernel, dim3(ctx->plan.n_cus), dim3(mk::NTHREADS), kargs, 0, s);
  if (e != hipSuccess) return hip_fail(e, ctx->plain_launch ? "hipLaunchKernel" : "hipLaunchCooperativeKernel");
  ctx->epoch += 1;
  ctx->tag = A.tag;
  ctx->last_stream = s;
  return MK_OK;
}

mk_status mk_sync_status(mk_ctx* ctx) {
  if (!ctx) return fail(MK_ERR_INVALID_ARG, "ctx is null");
  MK_HIP(hipStreamSynchronize(ctx->last_stream));
  uint32_t st[2] = {0, 0};
  MK_HIP(hipMemcpy(st, ctx->ws + ctx->plan.lay.status, sizeof st, hipMemcpyDeviceToHost));
  if (st[0] & mk::ST_TIMEOUT) ctx->sticky = MK_ERR_TIMEOUT;
  else if (st[0] & mk::ST_BAD_INPUT) ctx->sticky = MK_ERR_DEVICE_INPUT;
  if (ctx->sticky == MK_ERR_TIMEOUT) return fail(MK_ERR_TIMEOUT, "a dependency wait exceeded its spin limit");
  if (ctx->sticky == MK_ERR_DEVICE_INPUT) return fail(MK_ERR_DEVICE_INPUT, "out-of-contract token, position or page");
  return MK_OK;
}

mk_status mk_reset(mk_ctx* ctx) {
  if (!ctx) return fail(MK_ERR_INVALID_ARG, "ctx is null");
  MK_HIP(hipDeviceSynchronize());
  const mk::Layout& Y = ctx->plan.lay;
  mk_status r = zero_counters(ctx, nullptr);
  if (r != MK_OK) return r;
  hipLaunchKernelGGL(fill_u32, dim3(1), dim3(64), 0, nullptr, (uint32_t*)(ctx->ws + Y.status), (size_t)64, 0u);
  for (const auto& Q : Y.layer)
    hipLaunchKernelGGL(fill_u32, dim3(1), dim3(256), 0, nullptr, (uint32_t*)(ctx->ws + Q.tickets),
                       Y.tickets_bytes_per_layer / 4, 0u);
  // a stopped launch can leave activations of either parity: clear them (parity 0, row_ok tag 0)
  // and restart the tags at 1
  hipLaunchKernelGGL(fill_u32, dim3(256), dim3(256), 0, nullptr, (uint32_t*)(ctx->ws + Y.act_begin),
                     (Y.act_end - Y.act_begin) / 4, 0u);
  MK_HIP(hipGetLastError());
  MK_HIP(hipDeviceSynchronize());
  ctx->epoch = 0;
  ctx->tag = 0;
  ctx->sticky = MK_OK;
  return MK_OK;
}

void mk_destroy(mk_ctx* ctx) { delete ctx; }

mk_status mk_trace_words(mk_ctx* ctx, size_t* count) {
  if (!ctx || !count) return fail(MK_ERR_INVALID_ARG, "null argument");
  *count = 2 + (size_t)ctx->plan.n_cus + 1 + ctx->plan.ops.size() * 4;
  return MK_OK;
}

mk_status mk_copy_trace(mk_ctx* ctx, uint32_t* dst, size_t count) {
  if (!ctx || !dst) return fail(MK_ERR_INVALID_ARG, "null argument");
  if (!ctx->trace) return fail(MK_ERR_STATE, "tracing is off (set MK_TRACE=1 before mk_create)");
  size_t need = 0;
  mk_trace_words(ctx, &need);
  if (count < need) return fail(MK_ERR_INVALID_ARG, "trace buffer too small: need " + std::to_string(need) + " words");
  MK_HIP(hipStreamSynchronize(ctx->last_stream));
  const mk::Plan& P = ctx->plan;
  dst[0] = (uint32_t)P.ops.size();
  dst[1] = (uint32_t)P.n_cus;
  for (int c = 0; c <= P.n_cus; ++c) dst[2 + c] = P.queue_off[c];
  MK_HIP(hipMemcpy(dst + 3 + P.n_cus, ctx->trace, P.ops.size() * 4 * sizeof(uint32_t), hipMemcpyDeviceToHost));
  return MK_OK;
}

mk_status mk_copy_midstate(mk_ctx* ctx, int32_t kind, int32_t layer, float* dst, size_t count, void* hip_stream) {
  if (!ctx || !dst) return fail(MK_ERR_INVALID_ARG, "null argument");
  const mk_model_desc& d = ctx->shape.d;
  if (layer < 0 || layer >= d.n_layers) return fail(MK_ERR_INVALID_ARG, "layer out of range");
  const auto& Q = ctx->plan.lay.layer[layer];
  size_t off, width;
  switch (kind) {
    case MK_MID_X_MIXER: off = Q.x_mix; width = d.hidden; break;
    case MK_MID_X_MLP: off = Q.x_out; width = d.hidden; break;
    case MK_MID_MIXER_O: off = Q.mix_o; width = ctx->plan.mix_dim; break;
    case MK_MID_MLP_M: off = Q.m; width = d.ffn; break;
    case MK_MID_PROJ:
      off = Q.qkv;
      width = ctx->shape.kinds[layer] == MK_LAYER_ATTN ? (size_t)(d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim
                                                       : (size_t)ctx->shape.C + 2 * d.n_delta_heads;
      break;
    case MK_MID_EMBED: off = ctx->plan.lay.x0; width = d.hidden; break;
    default: return fail(MK_ERR_INVALID_ARG, "unknown mid-state kind");
  }
  if (count > (size_t)d.max_batch * width) return fail(MK_ERR_INVALID_ARG, "count exceeds max_batch * width");
  MK_HIP(hipMemcpyAsync(dst, ctx->ws + off, count * sizeof(float), hipMemcpyDeviceToDevice, (hipStream_t)hip_stream));
  return MK_OK;
}

}  // extern "C"
