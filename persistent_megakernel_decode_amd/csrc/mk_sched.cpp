// mk_sched.cpp -- compiles a model into per-compute-unit instruction queues.
//
// The ForgeMegakernel abstract (arxivdaily / arxiv.science, abstract) gives
// each SM a fine-grained instruction stream and replaces global
// synchronisation with dependency counters.  This scheduler produces exactly
// that for gfx950: every projection is cut into row tiles (one or more per
// compute unit, balanced to within one row), attention into (sequence, KV
// head, position chunk) items, and the delta rule into (sequence, head,
// 32-column block) items.  Ops are grouped into dependency stages; every
// queue lists its ops in one global stage order, so the lowest unfinished
// stage is always runnable and the persistent grid cannot deadlock.
//
// Split-K is never used: the MK-KDA pull request (github choiceoh/stkernel
// #230, commit message) measured split-K slowing an o_proj down once slices
// got short, and at these shapes every projection has at least as many rows
// as there are compute units (tiny test shapes aside).
#include "mk_sched.h"

#include <algorithm>
#include <cstdlib>
#include <cmath>
#include <cstdio>
#include <cstring>

namespace mk {

static constexpr uint64_t WS_TAG = 1ull << 62;  // marks a workspace-relative address
static inline uint64_t ws(size_t off) { return WS_TAG | (uint64_t)off; }
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename... Args>
static std::string fmt(const char* f, Args... a) {
  char buf[512];
  snprintf(buf, sizeof buf, f, a...);
  return buf;
}

std::string validate_desc(const mk_model_desc* desc, ModelShape* out, mk_status* st) {
  *st = MK_ERR_INVALID_ARG;
  if (!desc) return "null model description";
  if (desc->abi_version != MK_ABI_VERSION) return fmt("abi_version %u, library speaks %u", desc->abi_version, MK_ABI_VERSION);
  if (desc->struct_size != sizeof(mk_model_desc)) return fmt("struct_size %u != %zu", desc->struct_size, sizeof(mk_model_desc));
  const mk_model_desc& d = *desc;
  if (d.n_layers < 1 || d.hidden < 8 || d.vocab < 1 || d.ffn < 8) return "n_layers, hidden, vocab and ffn must be positive";
  if (!d.layer_kind) return "layer_kind is null";
  if (d.max_batch < 1 || d.max_ctx < 1) return "max_batch and max_ctx must be positive";
  if (d.weight_format != MK_WEIGHTS_BF16 && d.weight_format != MK_WEIGHTS_FP8_E4M3 && d.weight_format != MK_WEIGHTS_FP4_MX)
    return fmt("weight_format %d is not a mk_weight_format", d.weight_format);
  *st = MK_ERR_UNSUPPORTED;
  if (d.max_batch > 8) return "max_batch above 8 is not supported";
  if (d.hidden % 8 || d.ffn % 8) return "hidden and ffn must be multiples of 8";
  if (d.page_size != 16) return "page_size must be 16";
  if (!(d.rms_eps > 0.0f) || !(d.rope_base > 1.0f)) return "rms_eps must be > 0 and rope_base > 1";
  if (d.weight_format == MK_WEIGHTS_FP8_E4M3) {
    if (d.hidden % 16 || d.ffn % 16) return "fp8 weights need hidden and ffn to be multiples of 16";
  }
  if (d.n_experts < 0 || d.n_experts > 64) return "n_experts must be 0 to 64";
  if (d.n_experts > 0) {
    if (d.top_k < 1 || d.top_k > 8 || d.top_k > d.n_experts) return "top_k must be 1 to min(8, n_experts)";
    if (d.n_experts % 4) return "n_experts must be a multiple of 4";
    if (d.weight_format != MK_WEIGHTS_BF16) return "mixture-of-experts models take bf16 weights";
    if (d.max_batch > 4) return "mixture-of-experts models run at most 4 sequences per step";
  }
  if (d.weight_format == MK_WEIGHTS_FP4_MX) {
    if (d.max_batch != 1) return "fp4 weights run one sequence per step (max_batch 1)";
    if (d.hidden % 32 || d.ffn % 32) return "fp4 weights need hidden and ffn to be multiples of 32";
  }
  out->d = d;
  out->kinds.assign(d.layer_kind, d.layer_kind + d.n_layers);
  out->n_attn = out->n_delta = 0;
  for (int32_t k : out->kinds) {
    if (k == MK_LAYER_ATTN) ++out->n_attn;
    else if (k == MK_LAYER_DELTA) ++out->n_delta;
    else return fmt("layer kind %d is not ATTN or DELTA", k);
  }
  if (out->n_attn) {
    if (d.head_dim != 64 && d.head_dim != 128) return "head_dim must be 64 or 128";
    if (d.n_kv_heads < 1 || d.n_q_heads < 1 || d.n_q_heads % d.n_kv_heads) return "n_q_heads must be a multiple of n_kv_heads";
    out->G = d.n_q_heads / d.n_kv_heads;
    if (out->G * d.head_dim > 512) return "query heads per KV head times head_dim must not exceed 512";
  }
  if (out->n_delta) {
    if (d.delta_dk != 64 && d.delta_dk != 128) return "delta_dk must be 64 or 128";
    if (d.delta_dv < 32 || d.delta_dv % 32) return "delta_dv must be a positive multiple of 32";
    if (d.conv_width != 4) return "conv_width must be 4";
    if (d.n_delta_heads < 1) return "n_delta_heads must be positive";
    out->C = d.n_delta_heads * (2 * d.delta_dk + d.delta_dv);
  }
  *st = MK_OK;
  return "";
}

// GEMV ops (batch <= 4) run on the matrix cores in row groups of R = 16 / P rows, each row cut into
// pieces of 32 P inputs.  P = 8 for one or two sequences, 4 for up to four (P x batch <= 16).
static int gemv_part(int B) { return B <= 2 ? 8 : 4; }
// Pieces per row group: ceil(K / (32 P)) rounded up to 1, 2, 4, or a multiple of 8 (8 pieces fill a
// ring slot, one per compute wave).
static int gemv_pg(int K, int P) {
  const int real = (K + 32 * P - 1) / (32 * P);
  if (real <= 8) {
    int p = 1;
    while (p < real) p *= 2;
    return p;
  }
  return (real + 7) / 8 * 8;
}
static bool gemv_pg_ok(uint32_t pg) { return pg == 1 || pg == 2 || pg == 4 || (pg % 8 == 0 && pg <= (uint32_t)GEMV_MAX_PG); }
static uint32_t gemv_slots(uint32_t nrg, uint32_t pg) { return pg >= 8 ? nrg * (pg / 8) : (nrg * pg + 7) / 8; }

namespace {
// scales of a projection's (up to three) weight runs: fp32 row scales for fp8 weights, E8M0 block
// scale rows (K / 32 bytes per row) for fp4 weights
struct RowScales {
  bool f8 = false, f4 = false;
  uint64_t s[3] = {0, 0, 0};
};

// A mixture-of-experts stage: each op is one row tile of every expert (W / W2 expert 0's rows, the
// others moe_wstride bytes apart); the kernel runs it for the experts the router chose.
struct MoeOp {
  uint8_t opcode = 0;  // OP_MOE_GU or OP_MOE_DOWN (0: an ordinary GEMV stage)
  uint64_t router = 0, wstride = 0;
  uint32_t xstride = 0;
};

struct Builder {
  const ModelShape& m;
  Plan& P;
  int n_cus;
  std::vector<std::vector<Op>> stage_ops;  // per stage
  std::string err;

  int new_stage() {
    stage_ops.emplace_back();
    return (int)stage_ops.size() - 1;
  }

  // Row-tiled GEMV stage over N output rows of length K.  With sc.f8 the weight runs W / W2 / W3
  // are fp8 codes and sc.s the fp32 row scales of each run.
  void gemv(int stage, int wait, int layer, uint32_t N, uint32_t K, uint8_t epi, bool norm, uint64_t W, uint64_t W2,
            uint64_t W3, uint32_t b1, uint32_t b2, uint64_t in, uint32_t ld_in, uint64_t gamma, uint64_t out,
            uint32_t ld_out, uint64_t res, const RowScales& sc = RowScales{}, const MoeOp& moe = MoeOp{}) {
    if (!err.empty()) return;
    const int B = P.kernel_batch;
    if (sc.f8 && K % 16) {
      err = fmt("fp8 projection with %u inputs (needs a multiple of 16)", K);
      return;
    }
    if (sc.f4 && (K % 32 || B != 1)) {
      err = fmt("fp4 projection with %u inputs at batch width %d (needs a multiple of 32, one sequence)", K, B);
      return;
    }
    if (B >= 8) {
      mmv(stage, wait, layer, N, K, epi, norm, W, W2, W3, b1, b2, in, ld_in, gamma, out, ld_out, res, sc);
      return;
    }
    const int Pp = gemv_part(B), R = 16 / Pp;
    const uint32_t flags = sc.f8 ? OPF_FP8 : (sc.f4 ? OPF_FP4 : 0u);
    const uint32_t kv = gemv_kv(K, flags);  // stream elements per row
    const int pg = gemv_pg((int)kv, Pp);
    // (fp8: at most 4 input fragments of 16 per wave; fp4: 2 of 32)
    if (pg > GEMV_MAX_PG || (sc.f8 && pg > 32) || (sc.f4 && pg > 16)) {
      err = fmt("projection with %u inputs is too long for batch width %d", K, B);
      return;
    }
    if (K % 8) {
      err = fmt("projection input length %u is not a multiple of 8", K);
      return;
    }
    if (N % R || (b1 < N && b1 % R) || (b2 < N && b2 % R)) {
      err = fmt("projection rows (%u, split at %u / %u) must come in groups of %d", N, b1, b2, R);
      return;
    }
    const int RW = std::min(pg, 8);
    const int mult = epi == EPI_SWIGLU ? 2 : 1;
    uint32_t maxrows = (uint32_t)(RED_FLOATS / (RW * B * mult));
    if (moe.opcode) maxrows = std::min<uint32_t>(maxrows, 64 * NC);  // (one accumulator row per compute thread)
    maxrows -= maxrows % R;
    // tiles of whole row groups, as even as the groups allow
    const uint32_t NG = N / R;
    uint32_t T = std::min<uint32_t>((uint32_t)n_cus, NG);
    if ((NG + T - 1) / T * R > maxrows) {
      T = (N + maxrows - 1) / maxrows;
      T = (T + n_cus - 1) / n_cus * n_cus;
    }
    const uint32_t bnd[3] = {b1, b2, 0xFFFFFFFFu};
    for (uint32_t t = 0; t < T; ++t) {
      const uint32_t t0 = R * (uint32_t)((uint64_t)NG * t / T), t1 = R * (uint32_t)((uint64_t)NG * (t + 1) / T);
      for (uint32_t r0 = t0, r1; r0 < t1; r0 = r1) {
      // an op streams at most two weight runs: cut a tile that would touch three tensors
      r1 = t1;
      if (epi != EPI_SWIGLU) {
        const int sa = r0 < b1 ? 0 : (r0 < b2 ? 1 : 2);
        if (sa < 2) r1 = std::min<uint32_t>(t1, bnd[sa + 1]);
      }
      Op o{};
      o.opcode = OP_GEMV;
      o.epi = epi;
      o.norm = norm ? 1 : 0;
      o.wait_stage = (int16_t)wait;
      o.sig_stage = (int16_t)stage;
      o.layer = (uint32_t)layer;
      o.row0 = r0;
      o.nrows = r1 - r0;
      o.K = K;
      o.flags = flags;
      o.part = (uint8_t)Pp;
      o.ppr = (uint32_t)pg;
      o.nslots = gemv_slots(o.nrows * mult / R, (uint32_t)pg) + (norm ? gain_slots(K) : 0u);
      o.ld_in = ld_in;
      o.ld_out = ld_out;
      // weight runs: at most two contiguous row runs per op (scales: the same runs, srb bytes a row)
      const uint64_t rb = (uint64_t)kv * 2, srb = sc.f4 ? K / 32 : 4;
      if (epi == EPI_SWIGLU) {
        o.W = W ? W + r0 * rb : 0;
        o.W2 = W2 ? W2 + r0 * rb : 0;
        o.Ws = sc.s[0] ? sc.s[0] + r0 * srb : 0;
        o.Ws2 = sc.s[1] ? sc.s[1] + r0 * srb : 0;
        o.b1 = o.nrows;
      } else {
        const uint64_t segs[3] = {W, W2, W3};
        const uint32_t start[3] = {0u, b1, b2}, end[3] = {b1, b2, 0xFFFFFFFFu};
        int sa = r0 < b1 ? 0 : (r0 < b2 ? 1 : 2);
        o.W = segs[sa] ? segs[sa] + (uint64_t)(r0 - start[sa]) * rb : 0;
        o.Ws = sc.s[sa] ? sc.s[sa] + (uint64_t)(r0 - start[sa]) * srb : 0;
        const uint32_t na = std::min<uint32_t>(o.nrows, end[sa] - r0);
        o.b1 = na;
        o.W2 = 0;
        if (na < o.nrows) {
          if (sa == 2 || o.nrows - na > end[sa + 1] - start[sa + 1]) {
            err = "a projection tile spans more than two weight tensors";
            return;
          }
          o.W2 = segs[sa + 1];
          o.Ws2 = sc.s[sa + 1];
        }
      }
      o.in = in; o.gamma = gamma; o.out = out; o.res = res;
      if (moe.opcode) {
        o.opcode = moe.opcode;
        o.Ws = moe.router;
        o.moe_wstride = moe.wstride;
        o.moe_xstride = moe.xstride;
      }
      stage_ops[stage].push_back(o);
      }
    }
  }

  // Matrix-core GEMV stage (batch 8): row tiles of 16, k-outer streaming.  Same row-space and
  // weight-run conventions as gemv().
  void mmv(int stage, int wait, int layer, uint32_t N, uint32_t K, uint8_t epi, bool norm, uint64_t W, uint64_t W2,
           uint64_t W3, uint32_t b1, uint32_t b2, uint64_t in, uint32_t ld_in, uint64_t gamma, uint64_t out,
           uint32_t ld_out, uint64_t res, const RowScales& sc) {
    if (sc.f4) {
      err = "fp4 weights on the batch-8 path";
      return;
    }
    const uint32_t flags = sc.f8 ? OPF_FP8 : 0u;
    const uint32_t kv = gemv_kv(K, flags);  // stream elements per row (fp8: a segment is 512 codes)
    if (K % 16 || kv % MMV_KSEG) {
      err = fmt("projection input length %u is not a multiple of %d (batch-8 matrix-core path)", K,
                sc.f8 ? 2 * MMV_KSEG : MMV_KSEG);
      return;
    }
    const bool swiglu = epi == EPI_SWIGLU;
    const uint32_t maxrows = swiglu ? 16 * MMV_TILES / 2 : 16 * MMV_TILES;
    uint32_t T = std::min<uint32_t>((uint32_t)n_cus, N);
    if ((N + T - 1) / T > maxrows) {
      T = (N + maxrows - 1) / maxrows;
      T = (T + n_cus - 1) / n_cus * n_cus;
    }
    const uint32_t bnd[3] = {b1, b2, 0xFFFFFFFFu};
    for (uint32_t t = 0; t < T; ++t) {
      const uint32_t t0 = (uint32_t)((uint64_t)N * t / T), t1 = (uint32_t)((uint64_t)N * (t + 1) / T);
      for (uint32_t r0 = t0, r1; r0 < t1; r0 = r1) {
        r1 = t1;
        if (!swiglu) {
          const int sa = r0 < b1 ? 0 : (r0 < b2 ? 1 : 2);
          if (sa < 2) r1 = std::min<uint32_t>(t1, bnd[sa + 1]);
        }
        Op o{};
        o.opcode = OP_MMV;
        o.epi = epi;
        o.norm = norm ? 1 : 0;
        o.wait_stage = (int16_t)wait;
        o.sig_stage = (int16_t)stage;
        o.layer = (uint32_t)layer;
        o.row0 = r0;
        o.nrows = r1 - r0;
        o.K = K;
        o.flags = flags;
        o.ppr = kv / MMV_KSEG;
        const uint32_t ntiles = (swiglu ? 2 : 1) * ((o.nrows + 15) / 16);
        o.nslots = ntiles * o.ppr;
        o.ld_in = ld_in;
        o.ld_out = ld_out;
        const uint64_t rb = (uint64_t)kv * 2;
        if (swiglu) {
          o.W = W ? W + r0 * rb : 0;
          o.W2 = W2 ? W2 + r0 * rb : 0;
          o.Ws = sc.s[0] ? sc.s[0] + r0 * 4ull : 0;
          o.Ws2 = sc.s[1] ? sc.s[1] + r0 * 4ull : 0;
          o.b1 = o.nrows;
        } else {
          const uint64_t segs[3] = {W, W2, W3};
          const uint32_t start[3] = {0u, b1, b2}, end[3] = {b1, b2, 0xFFFFFFFFu};
          const int sa = r0 < b1 ? 0 : (r0 < b2 ? 1 : 2);
          o.W = segs[sa] ? segs[sa] + (uint64_t)(r0 - start[sa]) * rb : 0;
          o.Ws = sc.s[sa] ? sc.s[sa] + (uint64_t)(r0 - start[sa]) * 4 : 0;
          const uint32_t na = std::min<uint32_t>(o.nrows, end[sa] - r0);
          o.b1 = na;
          o.W2 = 0;
          if (na < o.nrows) {
            if (sa == 2 || o.nrows - na > end[sa + 1] - start[sa + 1]) {
              err = "a projection tile spans more than two weight tensors";
              return;
            }
            o.W2 = segs[sa + 1];
            o.Ws2 = sc.s[sa + 1];
          }
        }
        o.in = in; o.gamma = gamma; o.out = out; o.res = res;
        stage_ops[stage].push_back(o);
      }
    }
  }

  void items(int stage, int wait, int layer, uint8_t opcode, int n, uint32_t nslots) {
    for (int i = 0; i < n; ++i) {
      Op o{};
      o.opcode = opcode;
      o.wait_stage = (int16_t)wait;
      o.sig_stage = (int16_t)stage;
      o.layer = (uint32_t)layer;
      o.row0 = (uint32_t)i;
      o.nslots = nslots;
      stage_ops[stage].push_back(o);
    }
  }
};
}  // namespace

std::string build_plan(const ModelShape& m, int n_cus, const mk_weights* w, const mk_kv_cache* c, Plan* plan,
                       int dep_mode) {
  const mk_model_desc& d = m.d;
  Plan& P = *plan;
  P = Plan{};
  P.n_cus = n_cus;
  if (n_cus < 1) return "n_cus must be positive";
  P.kernel_batch = d.max_batch <= 1 ? 1 : d.max_batch <= 2 ? 2 : d.max_batch <= 4 ? 4 : 8;
  const int B = P.kernel_batch;  // activation buffers are B rows wide
  const int H = d.hidden, F = d.ffn, L = d.n_layers;
  const int hd = m.n_attn ? d.head_dim : 0;
  const int Hq = d.n_q_heads, Hkv = d.n_kv_heads;
  const int qkv_w = m.n_attn ? (Hq + 2 * Hkv) * hd : 0;
  const int nh = d.n_delta_heads, dk = d.delta_dk, dv = d.delta_dv;
  const int u_w = m.n_delta ? m.C + 2 * nh : 0;
  P.mix_dim = std::max(m.n_attn ? Hq * hd : 0, m.n_delta ? nh * dv : 0);
  // attention items per layer: a whole number of items per CU, at least one per (sequence, KV head)
  {
    // at least two chunks per (sequence, KV head) on average, so that chunks of one length
    // balance across CUs for ragged contexts
    int per_cu = (2 * Hkv * d.max_batch + n_cus - 1) / n_cus;
    if (const char* e = getenv("MK_ATTN_ITEMS_PER_CU"))  // diagnostic: down to one chunk per (sequence, KV head)
      per_cu = std::max((Hkv * d.max_batch + n_cus - 1) / n_cus, atoi(e));
    P.n_items = m.n_attn ? n_cus * per_cu : 0;
  }
  const int gmax = m.n_attn ? 512 / hd : 0;

  // ---------------- workspace layout (offsets; sizes of the queue sections are known after planning)
  Layout& Y = P.lay;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  // activation sections first (their offsets are needed while building ops)
  Y.rope = take(m.n_attn ? (size_t)d.max_ctx * (hd / 2) * 2 * sizeof(float) : 16);
  Y.status = take(256);
  Y.row_ok = take((size_t)B * 4);
  Y.x0 = take((size_t)B * H * 4);
  Y.layer.resize(L);
  Y.tickets_bytes_per_layer = (size_t)B * std::max(Hkv, nh) * 4;
  for (int l = 0; l < L; ++l) {
    auto& Q = Y.layer[l];
    if (m.kinds[l] == MK_LAYER_ATTN) {
      Q.qkv = take((size_t)B * qkv_w * 4);
      Q.part = take((size_t)P.n_items * gmax * (hd + 4) * 4);
    } else {
      Q.qkv = take((size_t)B * u_w * 4);
    }
    Q.tickets = take(Y.tickets_bytes_per_layer);
    Q.mix_o = take((size_t)B * P.mix_dim * 4);
    Q.x_mix = take((size_t)B * H * 4);
    Q.m = take((size_t)std::max(1, d.n_experts) * B * F * 4);  // (one row block per expert)
    Q.router = take((size_t)B * std::max(1, d.n_experts) * 4);
    Q.x_out = take((size_t)B * H * 4);
  }
  // multi-step launches: the tag of the last step each CU has finished (cleared with the
  // activations: a reset restarts the tags)
  Y.step_done = take((size_t)n_cus * 4);
  Y.act_begin = Y.row_ok;
  Y.act_end = off;

  // ---------------- stages and ops
  Builder bd{m, P, n_cus, {}, ""};
  auto wptr = [&](const void* p) -> uint64_t { return (uint64_t)(uintptr_t)p; };
  const bool f8 = d.weight_format == MK_WEIGHTS_FP8_E4M3, f4 = d.weight_format == MK_WEIGHTS_FP4_MX;
  auto scales = [&](const void* a, const void* b = nullptr, const void* c3 = nullptr) {
    RowScales r;
    r.f8 = f8;
    r.f4 = f4;
    if (f8 || f4) {
      r.s[0] = wptr(a);
      r.s[1] = wptr(b);
      r.s[2] = wptr(c3);
    }
    return r;
  };
  const mk_layer_weights* LW = w ? w->layers : nullptr;
  const uint64_t NONE = ~0u;
  const int s_embed = bd.new_stage();
  bd.items(s_embed, NO_STAGE, 0, OP_EMBED, n_cus, 0);
  int prev = s_embed;
  uint64_t x_in = ws(Y.x0);
  int ia = 0, id = 0;
  P.layers.resize(L);
  for (int l = 0; l < L; ++l) {
    const auto& Q = Y.layer[l];
    const mk_layer_weights* lw = LW ? &LW[l] : nullptr;
    LayerDesc& D = P.layers[l];
    D.qkv = ws(Q.qkv);
    D.tickets = ws(Q.tickets);
    D.mix_o = ws(Q.mix_o);
    int s_mix;
    if (m.kinds[l] == MK_LAYER_ATTN) {
      D.part = ws(Q.part);
      if (lw) { D.q_norm = wptr(lw->q_norm); D.k_norm = wptr(lw->k_norm); }
      if (c) {
        const size_t per_layer = (size_t)c->num_pages * Hkv * d.page_size * hd * 2;
        D.k_pages = wptr(c->k_pages) + per_layer * ia;
        D.v_pages = wptr(c->v_pages) + per_layer * ia;
      }
      D.kind = LAYER_ATTN;
      D.mix_width = (uint32_t)(Hq * hd);
      const int s_qkv = bd.new_stage();
      bd.gemv(s_qkv, prev, l, (uint32_t)qkv_w, (uint32_t)H, EPI_STORE, true, lw ? wptr(lw->wq) : 0,
              lw ? wptr(lw->wk) : 0, lw ? wptr(lw->wv) : 0, (uint32_t)(Hq * hd), (uint32_t)((Hq + Hkv) * hd), x_in,
              (uint32_t)H, lw ? wptr(lw->attn_norm) : 0, ws(Q.qkv), (uint32_t)qkv_w, 0,
              scales(lw ? lw->wq_scale : nullptr, lw ? lw->wk_scale : nullptr, lw ? lw->wv_scale : nullptr));
      const int s_attn = bd.new_stage();
      bd.items(s_attn, s_qkv, l, OP_ATTN, P.n_items, 0);
      s_mix = bd.new_stage();
      bd.gemv(s_mix, s_attn, l, (uint32_t)H, (uint32_t)(Hq * hd), EPI_RESID, false, lw ? wptr(lw->wo) : 0, 0, 0,
              (uint32_t)NONE, (uint32_t)NONE, ws(Q.mix_o), (uint32_t)P.mix_dim, 0, ws(Q.x_mix), (uint32_t)H, x_in,
              scales(lw ? lw->wo_scale : nullptr));
      ++ia;
    } else {
      D.kind = LAYER_DELTA;
      D.mix_width = (uint32_t)(nh * dv);
      D.gates = ws(Q.qkv) + (uint64_t)m.C * 4;
      if (lw) D.conv_w = wptr(lw->conv_w);
      if (c) {
        D.conv_state = wptr(c->conv_state) + (uint64_t)id * d.max_batch * m.C * (d.conv_width - 1) * 4;
        D.delta_state = wptr(c->delta_state) + (uint64_t)id * d.max_batch * nh * dv * dk * 4;
      }
      const int s_in = bd.new_stage();
      bd.gemv(s_in, prev, l, (uint32_t)u_w, (uint32_t)H, EPI_STORE, true, lw ? wptr(lw->w_qkv_delta) : 0,
              lw ? wptr(lw->w_gates) : 0, 0, (uint32_t)m.C, (uint32_t)NONE, x_in, (uint32_t)H,
              lw ? wptr(lw->attn_norm) : 0, ws(Q.qkv), (uint32_t)u_w, 0,
              scales(lw ? lw->w_qkv_delta_scale : nullptr, lw ? lw->w_gates_scale : nullptr));
      const int s_delta = bd.new_stage();
      const int n_items = d.max_batch * nh * (dv / 32);
      bd.items(s_delta, s_in, l, OP_DELTA, n_items, (uint32_t)(32 * dk * 4 / SLOT));
      s_mix = bd.new_stage();
      bd.gemv(s_mix, s_delta, l, (uint32_t)H, (uint32_t)(nh * dv), EPI_RESID, false, lw ? wptr(lw->wo_delta) : 0, 0,
              0, (uint32_t)NONE, (uint32_t)NONE, ws(Q.mix_o), (uint32_t)P.mix_dim, 0, ws(Q.x_mix), (uint32_t)H, x_in,
              scales(lw ? lw->wo_delta_scale : nullptr));
      ++id;
    }
    if (d.n_experts > 0) {
      // mixture of experts: router logits, then every chosen expert's gate / up and down rows
      const uint32_t E = (uint32_t)d.n_experts;
      const int s_rt = bd.new_stage();
      bd.gemv(s_rt, s_mix, l, E, (uint32_t)H, EPI_STORE, true, lw ? wptr(lw->w_router) : 0, 0, 0, (uint32_t)NONE,
              (uint32_t)NONE, ws(Q.x_mix), (uint32_t)H, lw ? wptr(lw->mlp_norm) : 0, ws(Q.router), E, 0);
      MoeOp mo;
      mo.router = ws(Q.router);
      mo.wstride = (uint64_t)F * H * 2;
      mo.xstride = (uint32_t)((size_t)B * F * 4);
      mo.opcode = OP_MOE_GU;
      const int s_gu = bd.new_stage();
      bd.gemv(s_gu, s_rt, l, (uint32_t)F, (uint32_t)H, EPI_SWIGLU, true, lw ? wptr(lw->w_gate) : 0,
              lw ? wptr(lw->w_up) : 0, 0, (uint32_t)NONE, (uint32_t)NONE, ws(Q.x_mix), (uint32_t)H,
              lw ? wptr(lw->mlp_norm) : 0, ws(Q.m), (uint32_t)F, 0, RowScales{}, mo);
      mo.opcode = OP_MOE_DOWN;
      const int s_down = bd.new_stage();
      bd.gemv(s_down, s_gu, l, (uint32_t)H, (uint32_t)F, EPI_RESID, false, lw ? wptr(lw->w_down) : 0, 0, 0,
              (uint32_t)NONE, (uint32_t)NONE, ws(Q.m), (uint32_t)F, 0, ws(Q.x_out), (uint32_t)H, ws(Q.x_mix),
              RowScales{}, mo);
      prev = s_down;
      x_in = ws(Q.x_out);
      continue;
    }
    const int s_gu = bd.new_stage();
    bd.gemv(s_gu, s_mix, l, (uint32_t)F, (uint32_t)H, EPI_SWIGLU, true, lw ? wptr(lw->w_gate) : 0,
            lw ? wptr(lw->w_up) : 0, 0, (uint32_t)NONE, (uint32_t)NONE, ws(Q.x_mix), (uint32_t)H,
            lw ? wptr(lw->mlp_norm) : 0, ws(Q.m), (uint32_t)F, 0,
            scales(lw ? lw->w_gate_scale : nullptr, lw ? lw->w_up_scale : nullptr));
    const int s_down = bd.new_stage();
    bd.gemv(s_down, s_gu, l, (uint32_t)H, (uint32_t)F, EPI_RESID, false, lw ? wptr(lw->w_down) : 0, 0, 0,
            (uint32_t)NONE, (uint32_t)NONE, ws(Q.m), (uint32_t)F, 0, ws(Q.x_out), (uint32_t)H, ws(Q.x_mix),
            scales(lw ? lw->w_down_scale : nullptr));
    prev = s_down;
    x_in = ws(Q.x_out);
  }
  const int s_lm = bd.new_stage();
  const void* lm = w ? (d.tied_embeddings ? w->embed : w->lm_head) : nullptr;
  bd.gemv(s_lm, prev, L, (uint32_t)d.vocab, (uint32_t)H, EPI_LOGITS, true, wptr(lm), 0, 0, (uint32_t)NONE,
          (uint32_t)NONE, x_in, (uint32_t)H, w ? wptr(w->final_norm) : 0, 0, (uint32_t)d.vocab, 0);
  if (!bd.err.empty()) return bd.err;
  P.n_lm = (int)bd.stage_ops[s_lm].size();

  // ---------------- distribute ops to queues (op j of a stage -> CU j mod n_cus), in stage order
  const int S = (int)bd.stage_ops.size();
  P.stages.resize(S);
  std::vector<std::vector<Op>> q(n_cus);
  P.cu_bytes.assign(n_cus, 0.0);
  for (int s = 0; s < S; ++s) {
    auto& ops = bd.stage_ops[s];
    P.stages[s].nops = (uint32_t)ops.size();
    for (size_t j = 0; j < ops.size(); ++j) {
      Op o = ops[j];
      o.sig_index = (uint32_t)j;
      const int cu = (int)(j % (size_t)n_cus);
      if (o.opcode == OP_GEMV || o.opcode == OP_MMV || o.opcode == OP_MOE_GU || o.opcode == OP_MOE_DOWN) {
        // streamed weight bytes: 2 per bf16 weight; 1 per fp8 code plus 4 per fp32 row scale; half
        // a byte per fp4 code plus one scale byte per 32 codes
        const double rows = (double)o.nrows * (o.epi == EPI_SWIGLU ? 2 : 1);
        const double bytes = (o.flags & OPF_FP8) ? rows * (o.K + 4.0)
                           : (o.flags & OPF_FP4) ? rows * (o.K / 2.0 + o.K / 32.0) : rows * o.K * 2;
        const bool moe = o.opcode == OP_MOE_GU || o.opcode == OP_MOE_DOWN;  // (every expert's rows)
        P.cu_bytes[cu] += moe ? bytes * m.d.n_experts : bytes;
        P.weight_bytes += moe ? bytes * m.d.n_experts : bytes;
      }
      q[cu].push_back(o);
    }
  }
  // Dependencies: an op whose wait stage was written by EMBED, a projection, attention or the
  // delta rule (tagged activations) polls its inputs; a stage is signalled only if some op waits
  // on its counter (MK_STAGE_COUNTERS=1 keeps the counters everywhere: diagnostic).
  {
    bool tags = dep_mode != 1;
    if (dep_mode < 0)
      if (const char* e = getenv("MK_STAGE_COUNTERS")) tags = atoi(e) == 0;
    std::vector<uint8_t> counted(S, 0);
    for (auto& qc : q)
      for (Op& o : qc) {
        if (o.wait_stage == NO_STAGE) continue;
        const uint8_t pop = bd.stage_ops[o.wait_stage][0].opcode;
        const bool tagged_src = pop == OP_EMBED || pop == OP_GEMV || pop == OP_MMV || pop == OP_ATTN || pop == OP_DELTA ||
                                pop == OP_MOE_GU || pop == OP_MOE_DOWN;
        const bool tagged_dst = o.opcode == OP_GEMV || o.opcode == OP_MMV || o.opcode == OP_ATTN || o.opcode == OP_DELTA ||
                                o.opcode == OP_MOE_GU || o.opcode == OP_MOE_DOWN;
        if (tags && tagged_src && tagged_dst) o.flags |= OPF_TAGGED_IN;
        else counted[o.wait_stage] = 1;
      }
    for (auto& qc : q)
      for (Op& o : qc)
        if (o.sig_stage != NO_STAGE && !counted[o.sig_stage]) o.flags |= OPF_NO_SIGNAL;
  }
  P.queue_off.assign(n_cus + 1, 0);
  for (int c2 = 0; c2 < n_cus; ++c2) {
    P.queue_off[c2 + 1] = P.queue_off[c2] + (uint32_t)q[c2].size();
    P.ops.insert(P.ops.end(), q[c2].begin(), q[c2].end());
  }
  Y.ops = take(P.ops.size() * sizeof(Op));
  Y.queue_off = take(P.queue_off.size() * 4);
  Y.stages = take(P.stages.size() * sizeof(Stage));
  Y.counters_bytes = (size_t)S * NSUB * CTR_STRIDE * 4;
  Y.counters = take(Y.counters_bytes);
  Y.layers = take((size_t)L * sizeof(LayerDesc));
  // per-op timing stamps of the traced kernels (MK_TRACE=1), 4 words per op; kept in every
  // workspace so that tracing never needs memory of its own
  Y.trace = take(P.ops.size() * TRACE_WORDS * sizeof(uint32_t));
  // verify windows: the launch's per-row positions, context lengths and page-table rows (pages
  // covering max_ctx), expanded from the per-sequence inputs before the launch
  Y.win_pages_per_row = (d.max_ctx + d.page_size - 1) / d.page_size;
  Y.win_pos = take((size_t)B * 4);
  Y.win_ctx = take((size_t)B * 4);
  Y.win_pages = take((size_t)B * Y.win_pages_per_row * 4);
  // multi-step launches: per LM-head op and sequence, the (value, index) of its largest logit, one
  // half per step parity (written every step before it is read: never cleared)
  Y.amax = take((size_t)2 * P.n_lm * 8 * 2 * 4);
  Y.total = off;
  return "";
}

static uint64_t reloc(uint64_t v, uint64_t base) { return (v & WS_TAG) ? base + (v & ~WS_TAG) : v; }

void relocate(Plan* plan, uint64_t base) {
  for (Op& o : plan->ops) {
    o.in = reloc(o.in, base);
    o.out = reloc(o.out, base);
    o.res = reloc(o.res, base);
    if (o.opcode == OP_MOE_GU || o.opcode == OP_MOE_DOWN) o.Ws = reloc(o.Ws, base);  // the router logits
  }
  for (LayerDesc& D : plan->layers) {
    D.qkv = reloc(D.qkv, base);
    D.gates = reloc(D.gates, base);
    D.part = reloc(D.part, base);
    D.tickets = reloc(D.tickets, base);
    D.mix_o = reloc(D.mix_o, base);
  }
}

std::string unrelocated(const Plan& P) {
  for (size_t i = 0; i < P.ops.size(); ++i) {
    const Op& o = P.ops[i];
    for (uint64_t v : {o.W, o.W2, o.Ws, o.Ws2, o.in, o.gamma, o.out, o.res})
      if (v & WS_TAG) return fmt("op %zu (opcode %u) keeps a workspace-relative address", i, (unsigned)o.opcode);
  }
  for (size_t l = 0; l < P.layers.size(); ++l) {
    const LayerDesc& D = P.layers[l];
    for (uint64_t v : {D.qkv, D.gates, D.q_norm, D.k_norm, D.k_pages, D.v_pages, D.part, D.tickets, D.mix_o, D.conv_w,
                       D.conv_state, D.delta_state})
      if (v & WS_TAG) return fmt("layer %zu keeps a workspace-relative address", l);
  }
  return "";
}

int check_plan(const ModelShape& m, const Plan& P, std::string* why) {
  int errors = 0;
  auto bad = [&](const std::string& s) {
    if (errors < 20) *why += s + "\n";
    ++errors;
  };
  const int S = (int)P.stages.size();
  std::vector<uint32_t> seen(S, 0);
  std::vector<std::vector<uint32_t>> idx(S);
  for (int c = 0; c < P.n_cus; ++c) {
    int last = -1;
    for (uint32_t i = P.queue_off[c]; i < P.queue_off[c + 1]; ++i) {
      const Op& o = P.ops[i];
      if (o.sig_stage < 0 || o.sig_stage >= S) { bad(fmt("cu %d op %u: bad signal stage", c, i)); continue; }
      if (o.sig_stage < last) bad(fmt("cu %d op %u: queue not in stage order", c, i));
      last = o.sig_stage;
      if (o.wait_stage != NO_STAGE && o.wait_stage >= o.sig_stage)
        bad(fmt("cu %d op %u: waits on stage %d, not earlier than its own %d", c, i, o.wait_stage, o.sig_stage));
      if ((o.flags & OPF_TAGGED_IN) && (o.opcode == OP_EMBED || o.wait_stage == NO_STAGE))
        bad(fmt("cu %d op %u: polls tagged inputs it cannot check", c, i));
      seen[o.sig_stage]++;
      idx[o.sig_stage].push_back(o.sig_index);
      if (o.opcode == OP_MOE_GU || o.opcode == OP_MOE_DOWN) {
        const bool gu = o.opcode == OP_MOE_GU;
        if (m.d.n_experts < 1 || !o.Ws || (gu ? o.epi != EPI_SWIGLU : o.epi != EPI_RESID) || o.nrows > 64u * NC ||
            (o.flags & (OPF_FP8 | OPF_FP4)) || o.moe_xstride < (uint64_t)P.kernel_batch * m.d.ffn * 4)
          bad(fmt("cu %d op %u: mixture-of-experts op", c, i));
      }
      if (o.opcode == OP_GEMV || o.opcode == OP_MOE_GU || o.opcode == OP_MOE_DOWN) {
        const uint32_t mult = o.epi == EPI_SWIGLU ? 2 : 1;
        const uint32_t Pp = o.part, R = Pp ? 16 / Pp : 1, pg = o.ppr;
        const uint32_t RW = std::min<uint32_t>(pg, 8);
        if (P.kernel_batch > 4) bad(fmt("cu %d op %u: matrix-core GEMV takes at most 4 sequences", c, i));
        if (Pp != (uint32_t)gemv_part(P.kernel_batch)) bad(fmt("cu %d op %u: %u input parts for batch %d", c, i, Pp, P.kernel_batch));
        if (!gemv_pg_ok(pg)) bad(fmt("cu %d op %u: %u pieces per row group", c, i, pg));
        if ((uint64_t)pg * 32 * Pp < gemv_kv(o.K, o.flags)) bad(fmt("cu %d op %u: pieces do not cover a row", c, i));
        if ((o.flags & OPF_FP8) && (o.K % 16 || o.epi == EPI_LOGITS || pg > 32))
          bad(fmt("cu %d op %u: fp8 weights off the batch-1 projection path", c, i));
        if ((o.flags & OPF_FP4) && (o.K % 32 || o.epi == EPI_LOGITS || pg > 16 || P.kernel_batch != 1 || (o.flags & OPF_FP8)))
          bad(fmt("cu %d op %u: fp4 weights off the batch-1 projection path", c, i));
        if (o.nrows == 0 || o.nrows % R) bad(fmt("cu %d op %u: %u rows, not whole groups of %u", c, i, o.nrows, R));
        if (o.epi != EPI_SWIGLU && o.b1 < o.nrows && o.b1 % R) bad(fmt("cu %d op %u: weight runs split a row group", c, i));
        if (o.epi == EPI_SWIGLU && o.b1 != o.nrows) bad(fmt("cu %d op %u: gate / up runs", c, i));
        if ((uint64_t)o.nrows * mult * RW * P.kernel_batch > (uint64_t)RED_FLOATS)
          bad(fmt("cu %d op %u: tile exceeds the partial-sum area", c, i));
        if (o.nslots != gemv_slots(o.nrows * mult / R, pg) + (o.norm ? gain_slots(o.K) : 0u))
          bad(fmt("cu %d op %u: slot count", c, i));
      }
      if (o.opcode == OP_MMV) {
        const uint32_t ntiles = (o.epi == EPI_SWIGLU ? 2 : 1) * ((o.nrows + 15) / 16);
        if (ntiles > (uint32_t)MMV_TILES) bad(fmt("cu %d op %u: %u row tiles, at most %d", c, i, ntiles, MMV_TILES));
        const uint32_t kv = gemv_kv(o.K, o.flags);
        if (kv % MMV_KSEG || o.ppr * MMV_KSEG != kv) bad(fmt("cu %d op %u: K segments do not cover a row", c, i));
        if ((o.flags & OPF_FP8) && (o.K % 16 || o.epi == EPI_LOGITS)) bad(fmt("cu %d op %u: fp8 operands", c, i));
        if (o.flags & OPF_FP4) bad(fmt("cu %d op %u: fp4 weights on the batch-8 path", c, i));
        if (o.nslots != ntiles * o.ppr) bad(fmt("cu %d op %u: slot count", c, i));
        if (P.kernel_batch > 16) bad(fmt("cu %d op %u: batch wider than a matrix tile", c, i));
      }
    }
  }
  for (int s = 0; s < S; ++s) {
    if (seen[s] != P.stages[s].nops) bad(fmt("stage %d: %u ops signal it, table says %u", s, seen[s], P.stages[s].nops));
    std::vector<uint32_t> v = idx[s];
    std::sort(v.begin(), v.end());
    for (size_t j = 0; j < v.size(); ++j)
      if (v[j] != j) { bad(fmt("stage %d: signal indices are not 0..n-1", s)); break; }
  }
  // every GEMV stage covers its rows exactly once
  std::vector<std::vector<std::pair<uint32_t, uint32_t>>> rows(S);
  for (const Op& o : P.ops)
    if (o.opcode == OP_GEMV || o.opcode == OP_MMV) rows[o.sig_stage].push_back({o.row0, o.row0 + o.nrows});
  for (int s = 0; s < S; ++s) {
    auto& r = rows[s];
    if (r.empty()) continue;
    std::sort(r.begin(), r.end());
    if (r[0].first != 0) bad(fmt("stage %d: rows do not start at 0", s));
    for (size_t j = 1; j < r.size(); ++j)
      if (r[j].first != r[j - 1].second) bad(fmt("stage %d: row gap or overlap at %u", s, r[j].first));
  }
  // streamed weight bytes == the model's projection bytes
  const mk_model_desc& d = m.d;
  // (a projection of rows x cols: 2 bytes per bf16 weight, or 1 per fp8 code and 4 per row scale, or
  // half a byte per fp4 code and one per 32-code block scale)
  const bool f8 = d.weight_format == MK_WEIGHTS_FP8_E4M3, f4 = d.weight_format == MK_WEIGHTS_FP4_MX;
  auto pbytes = [&](double rows, double cols) {
    return f8 ? rows * (cols + 4.0) : (f4 ? rows * (cols / 2 + cols / 32) : rows * cols * 2);
  };
  double want = (double)d.vocab * d.hidden * 2;  // the LM head stays bf16
  for (int l = 0; l < d.n_layers; ++l) {
    if (d.n_experts > 0)  // router plus every expert
      want += pbytes(d.n_experts, d.hidden) + d.n_experts * (2 * pbytes(d.ffn, d.hidden) + pbytes(d.hidden, d.ffn));
    else
      want += 2 * pbytes(d.ffn, d.hidden) + pbytes(d.hidden, d.ffn);
    if (m.kinds[l] == MK_LAYER_ATTN)
      want += pbytes((double)(d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim, d.hidden) +
              pbytes(d.hidden, (double)d.n_q_heads * d.head_dim);
    else
      want += pbytes((double)m.C + 2.0 * d.n_delta_heads, d.hidden) + pbytes(d.hidden, (double)d.n_delta_heads * d.delta_dv);
  }
  if (std::fabs(want - P.weight_bytes) > 0.5) bad(fmt("streamed %.0f weight bytes, model has %.0f", P.weight_bytes, want));
  return errors;
}

}  // namespace mk
