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
extern "C" __global__ void mk_megakernel_steps_b1(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b2(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b4(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b1_f8(mk::KArgs A);  // fp8 projections
extern "C" __global__ void mk_megakernel_b2_f8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b4_f8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b8_f8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b1_f8_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b2_f8_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b4_f8_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b8_f8_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b1_f8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b2_f8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b4_f8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b8_f8(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b1_f4(mk::KArgs A);  // MX fp4 projections (one sequence)
extern "C" __global__ void mk_megakernel_b1_f4_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b1_f4(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b1_moe(mk::KArgs A);  // mixture-of-experts MLPs (bf16)
extern "C" __global__ void mk_megakernel_b2_moe(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b4_moe(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b1_moe_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b2_moe_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_b4_moe_trace(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b1_moe(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b2_moe(mk::KArgs A);
extern "C" __global__ void mk_megakernel_steps_b4_moe(mk::KArgs A);

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

const void* kernel_for(int B, bool traced, int32_t wf, bool moe) {
  if (moe) {  // (at most 4 sequences)
    switch (B) {
      case 1: return traced ? (const void*)mk_megakernel_b1_moe_trace : (const void*)mk_megakernel_b1_moe;
      case 2: return traced ? (const void*)mk_megakernel_b2_moe_trace : (const void*)mk_megakernel_b2_moe;
      default: return traced ? (const void*)mk_megakernel_b4_moe_trace : (const void*)mk_megakernel_b4_moe;
    }
  }
  if (wf == MK_WEIGHTS_FP4_MX) return traced ? (const void*)mk_megakernel_b1_f4_trace : (const void*)mk_megakernel_b1_f4;
  if (wf == MK_WEIGHTS_FP8_E4M3) {
    switch (B) {
      case 1: return traced ? (const void*)mk_megakernel_b1_f8_trace : (const void*)mk_megakernel_b1_f8;
      case 2: return traced ? (const void*)mk_megakernel_b2_f8_trace : (const void*)mk_megakernel_b2_f8;
      case 4: return traced ? (const void*)mk_megakernel_b4_f8_trace : (const void*)mk_megakernel_b4_f8;
      default: return traced ? (const void*)mk_megakernel_b8_f8_trace : (const void*)mk_megakernel_b8_f8;
    }
  }
  switch (B) {
    case 1: return traced ? (const void*)mk_megakernel_b1_trace : (const void*)mk_megakernel_b1;
    case 2: return traced ? (const void*)mk_megakernel_b2_trace : (const void*)mk_megakernel_b2;
    case 4: return traced ? (const void*)mk_megakernel_b4_trace : (const void*)mk_megakernel_b4;
    default: return traced ? (const void*)mk_megakernel_b8_trace : (const void*)mk_megakernel_b8;
  }
}

const void* steps_kernel_for(int B, int32_t wf, bool moe) {
  if (moe) {
    switch (B) {
      case 1: return (const void*)mk_megakernel_steps_b1_moe;
      case 2: return (const void*)mk_megakernel_steps_b2_moe;
      default: return (const void*)mk_megakernel_steps_b4_moe;
    }
  }
  if (wf == MK_WEIGHTS_FP4_MX) return (const void*)mk_megakernel_steps_b1_f4;
  if (wf == MK_WEIGHTS_FP8_E4M3) {
    switch (B) {
      case 1: return (const void*)mk_megakernel_steps_b1_f8;
      case 2: return (const void*)mk_megakernel_steps_b2_f8;
      case 4: return (const void*)mk_megakernel_steps_b4_f8;
      default: return (const void*)mk_megakernel_steps_b8_f8;
    }
  }
  switch (B) {
    case 1: return (const void*)mk_megakernel_steps_b1;
    case 2: return (const void*)mk_megakernel_steps_b2;
    case 4: return (const void*)mk_megakernel_steps_b4;
    default: return (const void*)mk_megakernel_steps_b8;
  }
}

// Streaming read: every 16-byte word of [p, p + n) once, grid-stride, eight non-temporal 16-byte
// loads in flight per thread (the cache policy the megakernel's weight stream uses).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4_t* __restrict__ p, size_t n, uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4_t a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Verify windows: row r = b * win + t gets position positions[b] + t, context ctx_lens[b] + t (a
// value out of range at t = 0 stays out of range) and sequence b's page-table row.
__global__ void expand_window(const int32_t* pos, const int32_t* ctx, const int32_t* pt, int mpps_src, int batch,
                              int win, int32_t* rpos, int32_t* rctx, int32_t* rpt, int mpps_dst) {
  const int rows = batch * win, per = 2 + (pt ? mpps_dst : 0);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < rows * per; i += gridDim.x * blockDim.x) {
    const int r = i / per, k = i % per, b = r / win, t = r % win;
    if (k == 0) {
      const int p = pos[b];
      const int64_t q = (int64_t)p + t;
      rpos[r] = p < 0 ? p : (int)(q < 0x7FFFFFFF ? q : 0x7FFFFFFF);
    } else if (k == 1) {
      const int c = ctx[b];
      const int64_t q = (int64_t)c + t;
      rctx[r] = c < 1 ? c : (int)(q < 0x7FFFFFFF ? q : 0x7FFFFFFF);
    } else {
      const int p = k - 2;
      rpt[(size_t)r * mpps_dst + p] = p < mpps_src ? pt[(size_t)b * mpps_src + p] : -1;
    }
  }
}

__global__ void fill_u32(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---- the static scratch of mk_create_static ----
// Callers that cannot allocate device memory (code under graph capture, allocation-free serving
// loops) get a workspace from this file-scope array instead of bringing one.  Each GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch` is only a stand-in:
// its device address on the current GPU comes from hipGetSymbolAddress, taken once per device.
constexpr size_t STATIC_SCRATCH_BYTES = MK_STATIC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
uint64_t g_scratch_gen[MAX_DEVICES] = {};  // bumped by every mk_create_static on that device

}  // namespace

struct mk_ctx {
  mk::ModelShape shape;
  mk::Plan plan;
  int device = 0;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  mk::KArgs args{};
  uint32_t epoch = 0;
  uint32_t tag = 0;  // tag of the last step run (activation parity = bit 0)
  uint32_t max_stage_ops = 1;
  hipStream_t last_stream = nullptr;
  mk_status sticky = MK_OK;
  const void* kernel = nullptr;        // one decode step per launch
  const void* kernel_steps = nullptr;  // several steps per launch, tokens chosen on the device
  bool plain_launch = false;
  uint32_t* trace = nullptr;  // MK_TRACE=1: the workspace's trace section, TRACE_WORDS per op
  uint64_t static_gen = 0;    // mk_create_static: the device scratch generation this context owns (0 = own workspace)
  std::mutex busy;
};

// A context made by mk_create_static owns the device's static scratch until the next
// mk_create_static on that device; after that every call that touches its workspace is refused.
static bool scratch_taken_over(const mk_ctx* ctx) {
  if (!ctx->static_gen) return false;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  return g_scratch_gen[ctx->device] != ctx->static_gen;
}
#define MK_CHECK_SCRATCH(ctx)                                                                           \
  do {                                                                                                  \
    if (scratch_taken_over(ctx))                                                                        \
      return fail(MK_ERR_STATE, "a later mk_create_static on this device took over the static scratch"); \
  } while (0)

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
  {  // every workspace reference becomes a device address at mk_create
    mk::Plan r = p;
    mk::relocate(&r, 1ull << 40);
    const std::string u = mk::unrelocated(r);
    if (!u.empty()) {
      why += u + "\n";
      ++info->errors;
    }
  }
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

mk_status mk_emulate(const mk_model_desc* desc, const mk_emu_config* cfg, mk_emu_report* rep) {
  if (!cfg || !rep) return fail(MK_ERR_INVALID_ARG, "cfg and rep must be non-null");
  mk::ModelShape m;
  mk_status st;
  std::string e = mk::validate_desc(desc, &m, &st);
  if (!e.empty()) return fail(st, e);
  if (cfg->n_cus < 1 || cfg->n_launches < 0) return fail(MK_ERR_INVALID_ARG, "n_cus must be positive, n_launches >= 0");
  if (cfg->n_launches > 0 && (!cfg->batch || !cfg->ctx_lens)) return fail(MK_ERR_INVALID_ARG, "batch and ctx_lens must be non-null");
  for (int i = 0; i < cfg->n_launches; ++i)
    if (cfg->batch[i] < 1 || cfg->batch[i] > m.d.max_batch)
      return fail(MK_ERR_INVALID_ARG, "launch " + std::to_string(i) + ": batch outside [1, max_batch]");
  std::string found = mk::emulate(m, *cfg, rep);
  g_last_error = found;
  return MK_OK;
}

static mk_status create_impl(const mk_model_desc* desc, const mk_weights* w, const mk_kv_cache* c, void* workspace,
                             size_t workspace_bytes, mk_ctx** out, uint64_t static_gen) {
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
  const bool scaled = d.weight_format == MK_WEIGHTS_FP8_E4M3 || d.weight_format == MK_WEIGHTS_FP4_MX;
  for (int l = 0; pe.empty() && l < d.n_layers; ++l) {
    const mk_layer_weights& L = w->layers[l];
    // a projection and, for fp8 / fp4 weights, its scales
    auto proj = [&](const void* p, const void* sc, const char* name, const char* sname) {
      if (pe.empty()) pe = need(p, name);
      if (pe.empty() && scaled) pe = need(sc, sname);
    };
    pe = need(L.attn_norm, "attn_norm");
    if (pe.empty()) pe = need(L.mlp_norm, "mlp_norm");
    if (pe.empty() && d.n_experts > 0) pe = need(L.w_router, "w_router");
    proj(L.w_gate, L.w_gate_scale, "w_gate", "w_gate_scale");
    proj(L.w_up, L.w_up_scale, "w_up", "w_up_scale");
    proj(L.w_down, L.w_down_scale, "w_down", "w_down_scale");
    if (m.kinds[l] == MK_LAYER_ATTN) {
      proj(L.wq, L.wq_scale, "wq", "wq_scale");
      proj(L.wk, L.wk_scale, "wk", "wk_scale");
      proj(L.wv, L.wv_scale, "wv", "wv_scale");
      proj(L.wo, L.wo_scale, "wo", "wo_scale");
      if (pe.empty() && d.qk_norm) pe = need(L.q_norm, "q_norm");
      if (pe.empty() && d.qk_norm) pe = need(L.k_norm, "k_norm");
    } else {
      proj(L.w_qkv_delta, L.w_qkv_delta_scale, "w_qkv_delta", "w_qkv_delta_scale");
      proj(L.w_gates, L.w_gates_scale, "w_gates", "w_gates_scale");
      if (pe.empty()) pe = need(L.conv_w, "conv_w");
      proj(L.wo_delta, L.wo_delta_scale, "wo_delta", "wo_delta_scale");
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
  ctx->kernel = kernel_for(P.kernel_batch, traced, d.weight_format, d.n_experts > 0);
  ctx->kernel_steps = steps_kernel_for(P.kernel_batch, d.weight_format, d.n_experts > 0);

  // one resident workgroup per compute unit is required by the persistent design
  int per_cu = 0, per_cu_steps = 0;
  hipError_t he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ctx->kernel, mk::NTHREADS, 0);
  if (he == hipSuccess) he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_steps, ctx->kernel_steps, mk::NTHREADS, 0);
  if (he != hipSuccess || per_cu < 1 || per_cu_steps < 1) {
    delete ctx;
    return fail(MK_ERR_UNSUPPORTED, "the megakernel cannot be resident on a compute unit");
  }

  mk::relocate(&P, (uint64_t)(uintptr_t)workspace);
  {
    const std::string u = mk::unrelocated(P);
    if (!u.empty()) {
      delete ctx;
      return fail(MK_ERR_STATE, "plan: " + u);
    }
  }
  const mk::Layout& Y = P.lay;
  // zero everything (activations, counters, tickets, status), then upload the plan
  // (a fill kernel rather than a memset, so the same code serves the static scratch)
  hipLaunchKernelGGL(fill_u32, dim3(256), dim3(256), 0, nullptr, (uint32_t*)workspace, Y.total / 4, 0u);
  he = hipGetLastError();
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
  A.n_layers = d.n_layers; A.H = d.hidden; A.V = d.vocab; A.Hq = d.n_q_heads; A.Hkv = d.n_kv_heads; A.d = d.head_dim; A.G = m.G;
  A.qk_norm = d.qk_norm; A.max_batch = d.max_batch; A.max_ctx = d.max_ctx; A.page_size = d.page_size;
  A.num_pages = m.n_attn ? c->num_pages : 0;
  A.max_pages_per_seq = m.n_attn ? c->max_pages_per_seq : 1;
  A.nh = d.n_delta_heads; A.dk = d.delta_dk; A.dv = d.delta_dv; A.C = m.C; A.convw = d.conv_width;
  A.n_cus = ncu; A.n_items = P.n_items; A.mix = P.mix_dim;
  A.n_experts = d.n_experts; A.top_k = d.top_k;
  A.rms_eps = d.rms_eps;
  A.win = 1;      // mk_decode_window overrides it
  A.n_steps = 1;  // mk_decode_steps overrides these four
  A.n_lm = P.n_lm;
  A.tokens_out = nullptr;
  A.step_done = (uint32_t*)(ctx->ws + Y.step_done);
  A.amax = nullptr;
  double ms = 2000.0;
  // diagnostic only; the tests set a tiny limit to force the timeout path from the host
  if (const char* s = getenv("MK_WATCHDOG_MS")) ms = std::max(0.001, atof(s));
  A.spin_limit = (uint64_t)(ms * 1e5);  // s_memrealtime runs at 100 MHz
  A.spin_check_mask = ms < 0.01 ? 0u : 63u;
  // Diagnostic: MK_PLAIN_LAUNCH=1 launches with hipLaunchKernel instead of the cooperative launch
  // (for tools that cannot follow cooperative dispatches).  mk_create has already checked that one
  // workgroup per CU is resident; should some workgroup still not be scheduled, the spin-wait
  // watchdog ends every wait and the step reports MK_ERR_TIMEOUT.
  if (const char* s = getenv("MK_PLAIN_LAUNCH")) ctx->plain_launch = atoi(s) != 0;
  ctx->trace = traced ? (uint32_t*)(ctx->ws + Y.trace) : nullptr;  // zeroed with the workspace
  A.trace = ctx->trace;
  ctx->static_gen = static_gen;
  *out = ctx;
  return MK_OK;
}

mk_status mk_create(const mk_model_desc* desc, const mk_weights* w, const mk_kv_cache* c, void* workspace,
                    size_t workspace_bytes, mk_ctx** out) {
  return create_impl(desc, w, c, workspace, workspace_bytes, out, 0);
}

mk_status mk_create_static(const mk_model_desc* desc, const mk_weights* w, const mk_kv_cache* c, mk_ctx** out) {
  if (!out) return fail(MK_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  mk::ModelShape m;
  mk_status st;
  std::string e = mk::validate_desc(desc, &m, &st);
  if (!e.empty()) return fail(st, e);
  int ncu = 0;
  const int dev = device_cus(&ncu);
  if (dev < 0) return fail(MK_ERR_HIP, "cannot query the current HIP device");
  if (dev >= MAX_DEVICES) return fail(MK_ERR_UNSUPPORTED, "device index above the static scratch table");
  mk::Plan p;
  e = mk::build_plan(m, ncu, nullptr, nullptr, &p);
  if (!e.empty()) return fail(MK_ERR_UNSUPPORTED, e);
  if (p.lay.total > STATIC_SCRATCH_BYTES)
    return fail(MK_ERR_INVALID_ARG, "the model needs " + std::to_string(p.lay.total) +
                                        " bytes of workspace; the static scratch holds " +
                                        std::to_string(STATIC_SCRATCH_BYTES) + " (use mk_create with a workspace)");
  void* ptr = nullptr;
  uint64_t gen = 0;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {  // this device's copy of the array, with this device current
      hipError_t he = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (he != hipSuccess) {
        g_scratch_ptr[dev] = nullptr;
        return hip_fail(he, "hipGetSymbolAddress(scratch)");
      }
    }
    ptr = g_scratch_ptr[dev];
    gen = ++g_scratch_gen[dev];
  }
  return create_impl(desc, w, c, ptr, STATIC_SCRATCH_BYTES, out, gen);
}

static mk_status zero_counters(mk_ctx* ctx, hipStream_t s) {
  const mk::Layout& Y = ctx->plan.lay;
  hipLaunchKernelGGL(fill_u32, dim3(64), dim3(256), 0, s, (uint32_t*)(ctx->ws + Y.counters), Y.counters_bytes / 4, 0u);
  MK_HIP(hipGetLastError());
  return MK_OK;
}

// Checks shared by both decode entry points.  Returns MK_OK or the failure (with its message set).
static mk_status check_step_args(mk_ctx* ctx, const int32_t* tokens, const int32_t* positions, const int32_t* ctx_lens,
                                 int32_t batch, const float* logits_out) {
  if (!ctx) return fail(MK_ERR_INVALID_ARG, "ctx is null");
  if (ctx->sticky != MK_OK) return fail(MK_ERR_STATE, "context holds a device error; call mk_reset");
  if (!tokens || !positions || !ctx_lens || !logits_out) return fail(MK_ERR_INVALID_ARG, "null input or output pointer");
  if (!aligned16(tokens) || !aligned16(positions) || !aligned16(ctx_lens) || !aligned16(logits_out))
    return fail(MK_ERR_INVALID_ARG, "inputs and logits must be 16-byte aligned");
  if (batch < 1 || batch > ctx->shape.d.max_batch)
    return fail(MK_ERR_INVALID_ARG, "batch " + std::to_string(batch) + " outside [1, max_batch]");
  return MK_OK;
}

// One launch of `n_steps` decode steps (the caller holds ctx->busy).  Step s of the launch uses tag
// A.tag + s and counter epoch A.epoch + s.
static mk_status launch_steps(mk_ctx* ctx, mk::KArgs& A, uint32_t n_steps, const void* kernel, hipStream_t s) {
  // counters count cumulatively (epoch * ops); restart the epochs long before 32-bit overflow
  if ((uint64_t)(ctx->epoch + n_steps) * ctx->max_stage_ops >= (1ull << 31)) {
    mk_status r = zero_counters(ctx, s);
    if (r != MK_OK) return r;
    ctx->epoch = 0;
  }
  A.epoch = ctx->epoch + 1;
  // consecutive steps alternate the parity; the 31-bit tag restarts at 1 or 2 to keep it so
  A.tag = (uint64_t)ctx->tag + n_steps <= 0x7FFFFFFFu ? ctx->tag + 1 : (ctx->tag & 1u) ? 2u : 1u;
  void* kargs[] = {&A};
  hipError_t e = ctx->plain_launch
                     ? hipLaunchKernel(kernel, dim3(ctx->plan.n_cus), dim3(mk::NTHREADS), kargs, 0, s)
                     : hipLaunchCooperativeKernel(kernel, dim3(ctx->plan.n_cus), dim3(mk::NTHREADS), kargs, 0, s);
  if (e != hipSuccess) return hip_fail(e, ctx->plain_launch ? "hipLaunchKernel" : "hipLaunchCooperativeKernel");
  ctx->epoch += n_steps;
  ctx->tag = A.tag + n_steps - 1;
  ctx->last_stream = s;
  return MK_OK;
}

mk_status mk_decode_step(mk_ctx* ctx, const int32_t* tokens, const int32_t* positions, const int32_t* ctx_lens,
                         int32_t batch, float* logits_out, void* hip_stream) {
  mk_status r = check_step_args(ctx, tokens, positions, ctx_lens, batch, logits_out);
  if (r != MK_OK) return r;
  std::unique_lock<std::mutex> lk(ctx->busy, std::try_to_lock);
  if (!lk.owns_lock()) return fail(MK_ERR_STATE, "another thread is stepping this context");
  MK_CHECK_SCRATCH(ctx);
  mk::KArgs A = ctx->args;
  A.tokens = tokens;
  A.positions = positions;
  A.ctx_lens = ctx_lens;
  A.logits = logits_out;
  A.batch = batch;
  return launch_steps(ctx, A, 1, ctx->kernel, (hipStream_t)hip_stream);
}

mk_status mk_decode_window(mk_ctx* ctx, const int32_t* tokens, const int32_t* positions, const int32_t* ctx_lens,
                           int32_t batch, int32_t window, float* logits_out, void* hip_stream) {
  if (!ctx) return fail(MK_ERR_INVALID_ARG, "ctx is null");
  if (window < 1 || window > MK_MAX_WINDOW)
    return fail(MK_ERR_INVALID_ARG, "window " + std::to_string(window) + " outside [1, MK_MAX_WINDOW]");
  if (ctx->shape.d.n_experts > 0 && window > 1)
    return fail(MK_ERR_UNSUPPORTED, "verify windows are not supported for mixture-of-experts models");
  if (batch < 1 || (int64_t)batch * window > ctx->shape.d.max_batch)
    return fail(MK_ERR_INVALID_ARG, "batch * window = " + std::to_string((int64_t)batch * window) +
                                        " outside [1, max_batch]");
  mk_status r = check_step_args(ctx, tokens, positions, ctx_lens, batch * window, logits_out);
  if (r != MK_OK) return r;
  std::unique_lock<std::mutex> lk(ctx->busy, std::try_to_lock);
  if (!lk.owns_lock()) return fail(MK_ERR_STATE, "another thread is stepping this context");
  MK_CHECK_SCRATCH(ctx);
  const mk::Layout& Y = ctx->plan.lay;
  mk::KArgs A = ctx->args;
  A.tokens = tokens;
  A.positions = (const int32_t*)(ctx->ws + Y.win_pos);
  A.ctx_lens = (const int32_t*)(ctx->ws + Y.win_ctx);
  if (A.page_table) {
    A.page_table = (const int32_t*)(ctx->ws + Y.win_pages);
    A.max_pages_per_seq = Y.win_pages_per_row;
  }
  A.logits = logits_out;
  A.batch = batch * window;  // rows
  A.win = window;
  hipStream_t s = (hipStream_t)hip_stream;
  hipLaunchKernelGGL(expand_window, dim3(4), dim3(256), 0, s, positions, ctx_lens, ctx->args.page_table,
                     ctx->args.max_pages_per_seq, batch, window, (int32_t*)(ctx->ws + Y.win_pos),
                     (int32_t*)(ctx->ws + Y.win_ctx), (int32_t*)(ctx->ws + Y.win_pages), Y.win_pages_per_row);
  MK_HIP(hipGetLastError());
  return launch_steps(ctx, A, 1, ctx->kernel, s);
}

mk_status mk_decode_steps(mk_ctx* ctx, const int32_t* tokens, const int32_t* positions, const int32_t* ctx_lens,
                          int32_t batch, int32_t n_steps, float* logits_out, int32_t* tokens_out, void* hip_stream) {
  mk_status r = check_step_args(ctx, tokens, positions, ctx_lens, batch, logits_out);
  if (r != MK_OK) return r;
  if (!tokens_out || !aligned16(tokens_out)) return fail(MK_ERR_INVALID_ARG, "tokens_out must be a 16-byte aligned device pointer");
  if (n_steps < 1 || n_steps > MK_MAX_STEPS)
    return fail(MK_ERR_INVALID_ARG, "n_steps " + std::to_string(n_steps) + " outside [1, MK_MAX_STEPS]");
  std::unique_lock<std::mutex> lk(ctx->busy, std::try_to_lock);
  if (!lk.owns_lock()) return fail(MK_ERR_STATE, "another thread is stepping this context");
  MK_CHECK_SCRATCH(ctx);
  mk::KArgs A = ctx->args;
  A.tokens = tokens;
  A.positions = positions;
  A.ctx_lens = ctx_lens;
  A.logits = logits_out;
  A.batch = batch;
  A.n_steps = n_steps;
  A.tokens_out = tokens_out;
  A.amax = (uint32_t*)(ctx->ws + ctx->plan.lay.amax);
  return launch_steps(ctx, A, (uint32_t)n_steps, ctx->kernel_steps, (hipStream_t)hip_stream);
}

mk_status mk_sync_status(mk_ctx* ctx) {
  if (!ctx) return fail(MK_ERR_INVALID_ARG, "ctx is null");
  MK_CHECK_SCRATCH(ctx);
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
  MK_CHECK_SCRATCH(ctx);
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

mk_status mk_stream_read(const void* buf, size_t bytes, uint32_t* out, int32_t blocks, void* hip_stream) {
  if (!buf || !out || !aligned16(buf) || bytes % 16 || bytes == 0)
    return fail(MK_ERR_INVALID_ARG, "buf must be non-null and 16-byte aligned, bytes a positive multiple of 16");
  if (blocks < 1 || blocks > 65536) return fail(MK_ERR_INVALID_ARG, "blocks outside [1, 65536]");
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)hip_stream, (const u32x4_t*)buf,
                     bytes / 16, out);
  MK_HIP(hipGetLastError());
  return MK_OK;
}

mk_status mk_trace_words(mk_ctx* ctx, size_t* count) {
  if (!ctx || !count) return fail(MK_ERR_INVALID_ARG, "null argument");
  *count = 2 + (size_t)ctx->plan.n_cus + 1 + ctx->plan.ops.size() * mk::TRACE_WORDS;
  return MK_OK;
}

mk_status mk_copy_trace(mk_ctx* ctx, uint32_t* dst, size_t count) {
  if (!ctx || !dst) return fail(MK_ERR_INVALID_ARG, "null argument");
  MK_CHECK_SCRATCH(ctx);
  if (!ctx->trace) return fail(MK_ERR_STATE, "tracing is off (set MK_TRACE=1 before mk_create)");
  size_t need = 0;
  mk_trace_words(ctx, &need);
  if (count < need) return fail(MK_ERR_INVALID_ARG, "trace buffer too small: need " + std::to_string(need) + " words");
  MK_HIP(hipStreamSynchronize(ctx->last_stream));
  const mk::Plan& P = ctx->plan;
  dst[0] = (uint32_t)P.ops.size();
  dst[1] = (uint32_t)P.n_cus;
  for (int c = 0; c <= P.n_cus; ++c) dst[2 + c] = P.queue_off[c];
  MK_HIP(hipMemcpy(dst + 3 + P.n_cus, ctx->trace, P.ops.size() * mk::TRACE_WORDS * sizeof(uint32_t),
                   hipMemcpyDeviceToHost));
  return MK_OK;
}

mk_status mk_copy_midstate(mk_ctx* ctx, int32_t kind, int32_t layer, float* dst, size_t count, void* hip_stream) {
  if (!ctx || !dst) return fail(MK_ERR_INVALID_ARG, "null argument");
  MK_CHECK_SCRATCH(ctx);
  const mk_model_desc& d = ctx->shape.d;
  if (layer < 0 || layer >= d.n_layers) return fail(MK_ERR_INVALID_ARG, "layer out of range");
  const auto& Q = ctx->plan.lay.layer[layer];
  size_t off, width;
  switch (kind) {
    case MK_MID_X_MIXER: off = Q.x_mix; width = d.hidden; break;
    case MK_MID_X_MLP: off = Q.x_out; width = d.hidden; break;
    case MK_MID_MIXER_O: off = Q.mix_o; width = ctx->plan.mix_dim; break;
    case MK_MID_MLP_M:
      if (d.n_experts > 0) return fail(MK_ERR_UNSUPPORTED, "mixture-of-experts layers keep one MLP state per expert");
      off = Q.m;
      width = d.ffn;
      break;
    case MK_MID_ROUTER:
      if (d.n_experts < 1) return fail(MK_ERR_INVALID_ARG, "the model has no router");
      off = Q.router;
      width = d.n_experts;
      break;
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
