// mk_internal.h -- the compiled plan shared by the host scheduler (mk_sched.cpp)
// and the gfx950 megakernel (mk_kernel.hip).
//
// The ForgeMegakernel abstract (arxivdaily / arxiv.science, abstract) builds a
// decode megakernel from three structures: a fine-grained instruction stream
// per compute unit, dependency counters in place of grid-wide
// synchronisation, and an on-chip buffer pool that stages data for the
// compute.  Here they are:
//   * Op          -- one queue entry; each workgroup (one per CU) runs its own
//                    queue of Ops in order.
//   * Stage       -- a set of Ops whose completion others wait on; each Stage
//                    owns NSUB split counters in global memory that count
//                    finished Ops, cumulatively over steps (epoch * count).
//   * LDS ring    -- NSLOT slots of SLOT bytes, filled by a loader wave with
//                    LDS-DMA loads of the weight / KV / state bytes every Op
//                    streams, consumed by the compute waves.
#pragma once
#include <stdint.h>

namespace mk {

// ---- workgroup shape ----
constexpr int NC = 8;                  // compute waves per workgroup (wave 0 is the loader)
constexpr int NTHREADS = 64 * (NC + 1);
constexpr int PIECE = 1024;            // bytes moved by one LDS-DMA instruction (64 lanes x 16 B)
constexpr int SLOT_PIECES = 8;         // pieces per ring slot (== NC: one piece per compute wave)
constexpr int SLOT = PIECE * SLOT_PIECES;
constexpr int NSLOT = 16;              // 128 KB ring
#ifndef MK_LOAD_DEPTH
#define MK_LOAD_DEPTH 4
#endif
constexpr int LOAD_DEPTH = MK_LOAD_DEPTH;          // slots in flight per loader wave before it marks the oldest
constexpr int RED_FLOATS = 4096;       // 16 KB partial-sum / merge area
constexpr int SCRATCH_FLOATS = 512;    // 2 KB small cross-wave scratch

// ---- dependency counters ----
constexpr int NSUB = 16;               // split sub-counters per stage
constexpr int CTR_STRIDE = 32;         // u32 between sub-counters (128 B, one cache line each)

// ---- GEMV geometry ----
constexpr int PIECE_ELEMS = PIECE / 2; // bf16 weights per piece
constexpr int GEMV_MAX_PG = 64;        // pieces per row group: a wave keeps at most 8 input fragments

enum Opcode : uint8_t { OP_NOP = 0, OP_EMBED = 1, OP_GEMV = 2, OP_ATTN = 3, OP_DELTA = 4, OP_MMV = 5, OP_MOE_GU = 6,
                       OP_MOE_DOWN = 7 };
enum Epi : uint8_t { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3, EPI_MOE_ACC = 4 };

constexpr int16_t NO_STAGE = -1;
constexpr uint32_t LAYER_ATTN = 0, LAYER_DELTA = 1;  // the values of mk_layer_kind

// Op flags.  Every activation that crosses compute units carries its decode step's parity in the
// lowest mantissa bit of each fp32 value (row_ok carries the step's tag itself), and every such
// value is written exactly once per step, so an op can poll its inputs themselves instead of a
// stage counter (OPF_TAGGED_IN).  Step s of a launch has tag `tag + s`; launches are serialized and
// the next one starts at the following tag, so consecutive steps always alternate the parity.  A stage that no op waits on by counter skips its signal and the
// store-completion wait before it (OPF_NO_SIGNAL).
constexpr uint32_t OPF_TAGGED_IN = 1u;
constexpr uint32_t OPF_NO_SIGNAL = 2u;
// A GEMV op whose weights are fp8 (E4M3 codes, one byte each, with fp32 row scales Ws / Ws2): the
// loader streams a row of K codes exactly as a bf16 row of K / 2 weights (gemv_kv), so slots,
// pieces and row groups are counted in those 16-bit units; the compute waves read 16 codes per
// 16-byte chunk against 16 inputs.
constexpr uint32_t OPF_FP8 = 4u;
// A GEMV op whose weights are MX fp4 (E2M1 codes packed two per byte, low nibble first, with one
// E8M0 scale byte per 32 weights: Ws / Ws2 point at the runs' scale rows of K / 32 bytes): the
// loader streams a row of K codes as a bf16 row of K / 4 weights, and every 16-byte chunk the
// compute waves read is one 32-weight block.
constexpr uint32_t OPF_FP4 = 8u;
// The projection weight format a kernel is compiled for (OPF_FP8 / OPF_FP4 ops need it); WF_MOE:
// bf16 weights with mixture-of-experts ops (OP_MOE_GU / OP_MOE_DOWN)
constexpr int WF_BF16 = 0, WF_FP8 = 1, WF_FP4 = 2, WF_MOE = 3;

// One queue entry (128 bytes).  Pointers are device addresses.
//
// A GEMV op computes output rows [row0, row0 + nrows) of a row space that may
// be the concatenation of several weight tensors (q | k | v, or in_proj |
// gates).  Its weight stream is at most two contiguous row runs: stream rows
// [0, b1) start at W (already offset to the op's first row) and stream rows
// [b1, ...) start at W2.  EPI_SWIGLU streams the op's gate rows (W) then the
// same rows of the up projection (W2, b1 = nrows) and writes silu(gate) * up.
//
// GEMV ops (batch <= 4) run on the matrix cores: the stream is cut into row
// groups of R = 16 / part rows, each row split into pieces of 32 * part inputs
// (a piece of one group is 16 x 32 bf16, one 16x16x32 operand).  `ppr` holds
// the pieces per row group PG (1, 2, 4, or a multiple of 8 up to 64, padded
// up from ceil(K / (32 part))); a ring slot holds 8 consecutive pieces, so a
// group spans PG / 8 slots, or a slot holds 8 / PG groups.
//
// An MMV op (batch 8: the projection is a skinny GEMM on the matrix cores) covers the same row
// space in tiles of 16 rows (SWIGLU: gate and up tiles interleaved, gate tile i = 2i, up tile
// i = 2i + 1), at most MMV_TILES tiles, and streams K in segments of MMV_KSEG inputs: ring slot
// s holds tile s % ntiles of segment s / ntiles (16 rows x 256 inputs, 8 KB); `ppr` holds the
// number of segments K / MMV_KSEG.
// A GEMV op (batch <= 4) with norm == 1 streams its RMSNorm gain first: gain_slots(K) ring slots
// holding the K bf16 gains in order, then its weights (`nslots` counts both).
constexpr uint32_t gain_slots(uint32_t K) { return (K * 2 + SLOT - 1) / SLOT; }
constexpr int MMV_KSEG = 256;
constexpr int MMV_TILES = 8;
struct alignas(16) Op {
  uint8_t opcode;
  uint8_t epi;
  uint8_t norm;        // GEMV: 1 = RMSNorm the input with `gamma`
  uint8_t part;        // GEMV: input parts per matrix-core tile (4 or 8)
  int16_t wait_stage;  // stage this op waits for (NO_STAGE = none)
  int16_t sig_stage;   // stage this op counts towards (NO_STAGE = none)
  uint32_t sig_index;  // index of this op within sig_stage (selects the sub-counter)
  uint32_t layer;      // model layer
  uint32_t row0;       // GEMV: first output row;  ATTN / DELTA: item index
  uint32_t nrows;      // GEMV: output rows
  uint32_t K;          // GEMV: input length
  uint32_t ppr;        // GEMV: pieces per row group;  MMV: K segments
  uint32_t nslots;     // GEMV / DELTA: ring slots the op consumes (ATTN: computed at run time)
  uint32_t ld_in;      // floats between batch rows of `in`
  uint32_t ld_out;     // floats between batch rows of `out` / `res`
  uint32_t b1;         // GEMV: stream rows taken from W before switching to W2
  uint32_t flags;      // OPF_* bits
  uint32_t moe_xstride;  // OP_MOE_*: bytes between experts' SwiGLU outputs (m [n_experts][B][F])
  uint64_t W, W2;      // GEMV weight runs, bf16 rows of K (OPF_FP8: fp8 rows of K)
  uint64_t Ws;         // OPF_FP8: fp32 row scales of the W run (at the op's first row); OPF_FP4: E8M0 scale rows
  uint64_t in;         // fp32 [batch][ld_in]
  uint64_t gamma;      // bf16 [K] norm gain (norm == 1)
  uint64_t out;        // fp32 [batch][ld_out] (EPI_LOGITS writes the launch's logits instead)
  uint64_t res;        // fp32 [batch][ld_out] residual (EPI_RESID)
  uint64_t Ws2;        // OPF_FP8: fp32 row scales of the W2 run; OPF_FP4: its E8M0 scale rows
  uint64_t moe_wstride;  // OP_MOE_*: bytes between experts' weight matrices (W / W2 are expert 0's)
};
static_assert(sizeof(Op) == 128, "Op must stay 128 bytes");
// stream elements per row of a GEMV op: 16-bit weights, pairs of fp8 codes, or quads of fp4 codes
constexpr uint32_t gemv_kv(uint32_t K, uint32_t flags) {
  return (flags & OPF_FP4) ? K / 4 : ((flags & OPF_FP8) ? K / 2 : K);
}

// Per-layer device pointers used by ATTN / DELTA ops.
struct alignas(16) LayerDesc {
  uint64_t qkv;          // attn: fp32 [B][(Hq + 2 Hkv) d] raw projections;  delta: u fp32 [B][C]
  uint64_t gates;        // delta: fp32 [B][2 heads]
  uint64_t q_norm, k_norm;
  uint64_t k_pages, v_pages;   // this attention layer's pages
  uint64_t part;         // attn: fp32 partials [n_items][G][d + 2]
  uint64_t tickets;      // attn: u32 [B][Hkv] merge tickets
  uint64_t mix_o;        // fp32 [B][mix] attention / delta output before o_proj
  uint64_t conv_w;       // delta: bf16 [C][W]
  uint64_t conv_state;   // delta: fp32 [B][C][W-1]
  uint64_t delta_state;  // delta: fp32 [B][heads][dv][dk]
  uint32_t kind;         // LAYER_ATTN or LAYER_DELTA
  uint32_t mix_width;    // floats of mix_o one row holds for this layer (Hq d, or heads dv)
};

struct Stage {
  uint32_t nops;         // ops that signal this stage per step
  uint32_t pad;
};

// Everything the kernel needs, passed by value.
struct KArgs {
  // plan
  const Op* ops;              // all queues, concatenated
  const uint32_t* queue_off;  // [n_cus + 1] start of each CU's queue in ops
  const Stage* stages;
  uint32_t* counters;         // [n_stages][NSUB * CTR_STRIDE]
  const LayerDesc* layers;
  const float* rope;          // [max_ctx][d/2][2] (cos, sin)
  uint32_t* status;           // [0] sticky error bits, [1] tag of the first launch that raised any
  int32_t* row_ok;            // [max_batch]
  float* x0;                  // embedding output fp32 [max_batch][H]
  const uint16_t* embed;
  const int32_t* page_table;
  // model
  int32_t n_layers, H, V, Hq, Hkv, d, G, qk_norm, max_batch, max_ctx, page_size, num_pages, max_pages_per_seq;
  int32_t nh, dk, dv, C, convw;
  int32_t n_cus, n_items;     // attention work items per attention layer
  int32_t mix;                // floats between batch rows of the attention / delta output
  int32_t n_experts, top_k;   // mixture-of-experts MLPs (0: dense)
  float rms_eps;
  // per launch
  const int32_t* tokens;
  const int32_t* positions;
  const int32_t* ctx_lens;
  float* logits;
  int32_t batch;
  uint32_t epoch;             // stage counters reach (epoch + s) * count at the end of step s
  uint32_t tag;               // tag of step 0: bit 0 is the activation parity, row_ok holds tag << 1 | ok
  uint64_t spin_limit;        // watchdog, in s_memrealtime ticks (100 MHz)
  uint32_t spin_check_mask;   // the watchdog reads the clock once every (mask + 1) polls
  uint32_t* trace;            // MK_TRACE=1: TRACE_WORDS per op (see below); else null
  // multi-step launches (the token fed back on the device): step s consumes the argmax of step
  // s - 1 at positions + s, writes logits + s * batch * V; tag + s is step s's activation tag
  int32_t n_steps;            // steps in this launch (>= 1)
  int32_t n_lm;               // LM-head ops (argmax partials per sequence)
  int32_t* tokens_out;        // [n_steps][batch] greedy token of each step, or null
  // verify windows: rows b*win .. b*win + win - 1 are tokens 0 .. win - 1 of sequence b; the host
  // expands positions, context lengths and page-table rows per row (positions / ctx_lens /
  // page_table then point at that copy), and the delta-rule items run sequence b's window with
  // state row b.  win = 1 is one token per sequence.  `batch` counts rows.
  int32_t win;
  uint32_t* step_done;        // [n_cus] tag of the last step whose stores this CU has completed
  uint32_t* amax;             // [2][n_lm][max batch width][2] per-op (value bits, index) of the LM head,
                              // double-buffered by step parity
};

// Per-op trace record of the traced kernels: {opcode << 16 | stage, start, inputs ready, end,
// loader first issue, loader last issue, loader ticks blocked on a full ring, 0} (100 MHz clock).
constexpr int TRACE_WORDS = 8;

// status bits
constexpr uint32_t ST_BAD_INPUT = 1u;
constexpr uint32_t ST_TIMEOUT = 2u;

}  // namespace mk
