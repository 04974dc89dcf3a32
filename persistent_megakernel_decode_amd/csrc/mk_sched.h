// mk_sched.h -- host-side scheduler: compiles a model description into
// per-compute-unit Op queues, dependency stages and a workspace layout.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_internal.h"

namespace mk {

// Byte offsets of every workspace section (all 256-byte aligned).
struct Layout {
  size_t ops = 0, queue_off = 0, stages = 0, counters = 0, layers = 0, rope = 0, status = 0, row_ok = 0, x0 = 0;
  size_t trace = 0;  // per-op timing stamps (traced kernels only)
  size_t step_done = 0, amax = 0;  // multi-step launches: per-CU step tags, LM-head greedy partials
  size_t win_pos = 0, win_ctx = 0, win_pages = 0;  // verify windows: per-row positions, contexts, page rows
  int win_pages_per_row = 0;
  struct PerLayer {
    size_t qkv = 0, part = 0, tickets = 0, mix_o = 0, x_mix = 0, m = 0, x_out = 0;
    size_t router = 0;  // mixture of experts: router logits fp32 [B][n_experts]
  };
  std::vector<PerLayer> layer;
  size_t counters_bytes = 0, tickets_bytes_per_layer = 0;
  size_t act_begin = 0, act_end = 0;  // tagged activations (row_ok .. the last layer's sections)
  size_t total = 0;
};

struct Plan {
  int n_cus = 0;
  int kernel_batch = 1;          // compiled batch width of the kernel variant
  int n_items = 0;               // attention items per attention layer
  int mix_dim = 0;
  int n_lm = 0;                  // LM-head ops (one greedy partial per op and sequence)
  std::vector<Op> ops;           // all queues concatenated (device pointers are offsets until relocated)
  std::vector<uint32_t> queue_off;
  std::vector<Stage> stages;
  std::vector<LayerDesc> layers;
  Layout lay;
  double weight_bytes = 0;
  std::vector<double> cu_bytes;  // streamed weight bytes per CU
};

// Validated copy of the caller's description.
struct ModelShape {
  mk_model_desc d{};
  std::vector<int32_t> kinds;
  int n_attn = 0, n_delta = 0, G = 1, C = 0;
};

// Returns "" on success, else a message.  `status` receives the mk_status code.
std::string validate_desc(const mk_model_desc* desc, ModelShape* out, mk_status* status);

// Builds the plan with device pointers expressed relative to:
//   workspace base (bit 62 tag) -- relocated by relocate(); weights / cache pointers are taken
//   verbatim from `w` / `c` when given (NULL = leave zero, for host-only planning).
// dep_mode: 0 = tagged activations wherever possible (the default plan), 1 = every dependency
// through the stage counters (diagnostic), -1 = from the MK_STAGE_COUNTERS environment variable.
std::string build_plan(const ModelShape& m, int n_cus, const mk_weights* w, const mk_kv_cache* c, Plan* plan,
                       int dep_mode = -1);

// Rewrites workspace-relative addresses in the plan into absolute device addresses.
void relocate(Plan* plan, uint64_t workspace_base);

// Structural checks (stage order, coverage, capacities).  Returns the number of violations and
// appends their descriptions to `why`.
int check_plan(const ModelShape& m, const Plan& plan, std::string* why);
// After relocate(): the first op or layer field still holding a workspace-relative address, or "".
std::string unrelocated(const Plan& plan);

// Replays the compiled queues over a launch sequence on the CPU (mk_emu.cpp).  Fills *rep and
// returns a description of the first problems found ("" when none).
std::string emulate(const ModelShape& m, const mk_emu_config& cfg, mk_emu_report* rep);

}  // namespace mk
