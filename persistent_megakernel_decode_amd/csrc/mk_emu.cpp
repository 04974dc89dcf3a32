// mk_emu.cpp -- a CPU model of the megakernel's dependency protocol (host only, no GPU).
//
// The ForgeMegakernel abstract (arxivdaily / arxiv.science, abstract) replaces grid-wide
// synchronisation with fine-grained dependencies between the compute units' instruction streams,
// and asks that the generated kernel be correct.  On gfx950 the dependencies are the data itself:
// every activation that crosses compute units carries the launch's parity in its lowest mantissa
// bit, and a consumer polls its inputs until they show the current parity (the LMSYS megakernel
// post summarised on the khabar-ai page uses data as its own readiness signal in the same way).
// That is sound only if every value a consumer may poll is written exactly once in every launch.
//
// This emulator replays the queues the scheduler compiles (build_plan, the same code the GPU
// path uploads) with the attention split of mk_attn_plan.h (the kernel's own planner) over a
// sequence of launches with varying batches and contexts.  Compute units run in a random
// interleaving; every tagged value is a cell remembering the launch that last wrote it.  A poll
// accepts a cell that shows the current parity, as the kernel does, and the emulator counts the
// accepts whose cell was written by an earlier launch (stale accepts).  After each launch it checks
// that every pollable cell was written exactly once.  A launch in which every remaining unit
// waits is reported as a deadlock (where the kernel's watchdog would raise MK_ERR_TIMEOUT).
//
// The per-op read and write sets below restate what each kernel op touches (mk_kernel.hip); the
// emulator does no arithmetic.
#include <algorithm>
#include <cstdint>
#include <random>
#include <string>
#include <vector>

#include "../../include/mk.h"
#include "mk_attn_plan.h"
#include "mk_internal.h"
#include "mk_sched.h"

namespace mk {
namespace {

constexpr uint64_t WS_BIT = 1ull << 62;

struct Buf {
  size_t off = 0, floats = 0;          // workspace section: byte offset, size in floats
  bool full_tag = false;               // row_ok: compared with the whole launch tag
  std::vector<uint32_t> lastw;         // launch tag of the last write (0 = cleared)
  std::vector<uint8_t> nw;             // writes in the current launch
  std::vector<uint8_t> pollable;       // cells some consumer may poll in some launch
};

struct Range {
  int buf;
  uint32_t lo, hi;  // cells [lo, hi)
};

enum PhaseKind { PH_POLL, PH_WRITE, PH_COUNTER, PH_READ };

struct Phase {
  PhaseKind kind;
  std::vector<Range> r;
  int stage = -1;
};

struct CuState {
  uint32_t oi = 0, oend = 0;       // queue range
  std::vector<Phase> ph;
  size_t pi = 0;                   // phase index
  size_t chunk = 0;                // write chunk within a PH_WRITE
  std::vector<std::pair<int, uint32_t>> pending;  // PH_POLL cells still to see the current parity
  bool started = false;            // the current phase has been entered
  bool blocked = false, done = false, stalled = false;
  int wbuf = -1;                   // blocked on (wbuf, wcell), or on a counter (wbuf = -2)
  uint32_t wcell = 0;
};

struct Emu {
  const ModelShape& m;
  const Plan& P;
  const mk_emu_config& cfg;
  mk_emu_report& rep;
  std::string msg;
  std::vector<Buf> bufs;
  int b_x0 = -1, b_rowok = -1;
  struct LayerBufs { int qkv = -1, part = -1, mix_o = -1, x_mix = -1, m = -1, x_out = -1; };
  std::vector<LayerBufs> lb;
  std::vector<uint32_t> stage_done;
  int B = 1, D = 0, G = 1, GMAX = 1, Hq = 0, Hkv = 0;
  uint32_t tag = 0;
  int batch = 0;
  int ctx[APLAN_MAXB] = {0};
  int plan[APLAN_WORDS] = {0};
  std::mt19937_64 rng;

  Emu(const ModelShape& m_, const Plan& P_, const mk_emu_config& c, mk_emu_report& r)
      : m(m_), P(P_), cfg(c), rep(r), rng(c.seed) {}

  void note(const std::string& s) {
    if (msg.size() < 2000) msg += s + "\n";
  }

  int add_buf(size_t off, size_t floats) {
    Buf b;
    b.off = off;
    b.floats = floats;
    b.lastw.assign(floats, 0);
    b.nw.assign(floats, 0);
    b.pollable.assign(floats, 1);
    bufs.push_back(std::move(b));
    return (int)bufs.size() - 1;
  }

  void setup() {
    const mk_model_desc& d = m.d;
    B = P.kernel_batch;
    Hq = d.n_q_heads;
    Hkv = d.n_kv_heads;
    D = m.n_attn ? d.head_dim : 0;
    G = m.G;
    GMAX = m.n_attn ? 512 / D : 1;
    const Layout& Y = P.lay;
    b_x0 = add_buf(Y.x0, (size_t)B * d.hidden);
    b_rowok = add_buf(Y.row_ok, (size_t)B);
    bufs[b_rowok].full_tag = true;
    for (int b = d.max_batch; b < B; ++b) bufs[b_rowok].pollable[b] = 0;
    const int qkv_w = m.n_attn ? (Hq + 2 * Hkv) * D : 0;
    const int u_w = m.n_delta ? m.C + 2 * d.n_delta_heads : 0;
    lb.resize(d.n_layers);
    for (int l = 0; l < d.n_layers; ++l) {
      const auto& Q = Y.layer[l];
      const bool attn = m.kinds[l] == MK_LAYER_ATTN;
      LayerBufs& L = lb[l];
      L.qkv = add_buf(Q.qkv, (size_t)B * (attn ? qkv_w : u_w));
      if (attn) {
        L.part = add_buf(Q.part, (size_t)P.n_items * GMAX * (D + 4));
        Buf& pb = bufs[L.part];
        for (size_t i = 0; i < pb.floats; ++i) {  // polled: (m, l) and o[D] of heads below G
          const size_t g = (i / (D + 4)) % GMAX, w = i % (D + 4);
          pb.pollable[i] = g < (size_t)G && (w < 2 || w >= 4);
        }
      }
      L.mix_o = add_buf(Q.mix_o, (size_t)B * P.mix_dim);
      const size_t width = P.layers[l].mix_width;
      for (size_t i = 0; i < bufs[L.mix_o].floats; ++i) bufs[L.mix_o].pollable[i] = (i % P.mix_dim) < width;
      L.x_mix = add_buf(Q.x_mix, (size_t)B * d.hidden);
      L.m = add_buf(Q.m, (size_t)std::max(1, d.n_experts) * B * d.ffn);  // (one row block per expert)
      if (d.n_experts > 0) add_buf(Q.router, (size_t)B * d.n_experts);
      L.x_out = add_buf(Q.x_out, (size_t)B * d.hidden);
    }
  }

  // workspace-relative address -> (buffer, first cell)
  bool resolve(uint64_t addr, int* buf, uint32_t* cell) const {
    if (!(addr & WS_BIT)) return false;
    const size_t off = (size_t)(addr & ~WS_BIT);
    for (size_t i = 0; i < bufs.size(); ++i) {
      const Buf& b = bufs[i];
      if (off >= b.off && off < b.off + b.floats * 4) {
        *buf = (int)i;
        *cell = (uint32_t)((off - b.off) / 4);
        return true;
      }
    }
    return false;
  }
  Range at(uint64_t addr, uint32_t lo, uint32_t n) {
    int bi = -1;
    uint32_t c = 0;
    if (!resolve(addr, &bi, &c)) {
      note("emulator: an op address lies outside every tagged section");
      ++rep.unsynced_reads;
      return Range{b_x0, 0, 0};
    }
    return Range{bi, c + lo, c + lo + n};
  }

  bool live(int b) const { return b < batch && ctx[b] > 0; }

  // ------------------------------------------------------------------ per-op read / write sets
  void phases_of(const Op& o, std::vector<Phase>& ph) {
    ph.clear();
    const mk_model_desc& d = m.d;
    const bool tagged = (o.flags & OPF_TAGGED_IN) != 0;
    if (o.wait_stage != NO_STAGE && !tagged) {
      Phase w{PH_COUNTER, {}, o.wait_stage};
      ph.push_back(w);
    }
    const PhaseKind in_kind = tagged ? PH_POLL : PH_READ;
    switch (o.opcode) {
      case OP_EMBED: {
        Phase w{PH_WRITE, {}, -1};
        const int c = cur_cu;
        const uint32_t h0 = (uint32_t)((int64_t)d.hidden * c / P.n_cus), h1 = (uint32_t)((int64_t)d.hidden * (c + 1) / P.n_cus);
        for (int b = 0; b < B; ++b) w.r.push_back(Range{b_x0, b * (uint32_t)d.hidden + h0, b * (uint32_t)d.hidden + h1});
        if (!(cfg.flags & MK_EMU_DEAD_ROWS_SILENT)) {
          for (int l = 0; l < d.n_layers; ++l) {
            const uint32_t wd = P.layers[l].mix_width;
            const uint32_t c0 = (uint32_t)((int64_t)wd * c / P.n_cus), c1 = (uint32_t)((int64_t)wd * (c + 1) / P.n_cus);
            for (int b = 0; b < B; ++b) {
              const bool written = m.kinds[l] == MK_LAYER_ATTN ? live(b) : b < d.max_batch;
              if (!written) w.r.push_back(Range{lb[l].mix_o, b * (uint32_t)P.mix_dim + c0, b * (uint32_t)P.mix_dim + c1});
            }
          }
        }
        if (c == 0) w.r.push_back(Range{b_rowok, 0, (uint32_t)d.max_batch});
        ph.push_back(w);
        break;
      }
      case OP_GEMV:
      case OP_MMV: {
        Phase in{in_kind, {}, -1};
        for (int b = 0; b < B; ++b) {
          if ((cfg.flags & MK_EMU_DEAD_ROWS_SILENT) && is_mixer_out(o.in) && !mixer_row_written(o.layer, b)) continue;
          in.r.push_back(at(o.in, b * o.ld_in, o.K));
        }
        if (o.epi == EPI_RESID)
          for (int b = 0; b < B; ++b) in.r.push_back(at(o.res, b * o.ld_out + o.row0, o.nrows));
        ph.push_back(in);
        if (o.epi == EPI_LOGITS) {
          Phase rk{PH_POLL, {}, -1};
          for (int b = 0; b < batch; ++b) rk.r.push_back(Range{b_rowok, (uint32_t)b, (uint32_t)b + 1});
          ph.push_back(rk);
        } else {
          Phase w{PH_WRITE, {}, -1};
          for (int b = 0; b < B; ++b) w.r.push_back(at(o.out, b * o.ld_out + o.row0, o.nrows));
          ph.push_back(w);
        }
        break;
      }
      case OP_MOE_GU:
      case OP_MOE_DOWN: {
        // a row tile of every expert: the router logits, then (gate / up) the normalised input and a
        // write of every expert's rows (the chosen ones computed, the others zero), or (down) every
        // expert's SwiGLU rows, whichever the router chose, and the residual
        const bool gu = o.opcode == OP_MOE_GU;
        const uint32_t E = (uint32_t)d.n_experts, xs = o.moe_xstride / 4;
        Phase in{in_kind, {}, -1};
        for (int b = 0; b < B; ++b) in.r.push_back(at(o.Ws, b * E, E));
        for (uint32_t e = 0; e < (gu ? 1u : E); ++e)
          for (int b = 0; b < B; ++b) in.r.push_back(at(o.in, e * xs + b * o.ld_in, o.K));
        if (!gu)
          for (int b = 0; b < B; ++b) in.r.push_back(at(o.res, b * o.ld_out + o.row0, o.nrows));
        ph.push_back(in);
        Phase w{PH_WRITE, {}, -1};
        for (uint32_t e = 0; e < (gu ? E : 1u); ++e)
          for (int b = 0; b < B; ++b) w.r.push_back(at(o.out, e * xs + b * o.ld_out + o.row0, o.nrows));
        ph.push_back(w);
        break;
      }
      case OP_ATTN: {
        const AttnItem it = attn_item_from([&](int i) { return plan[i]; }, batch, Hkv, o.row0);
        const uint32_t pslot = o.row0 * GMAX * (D + 4);
        const LayerBufs& L = lb[o.layer];
        if (!it.valid) {
          if (!(cfg.flags & MK_EMU_IDLE_ITEMS_SILENT)) {
            Phase w{PH_WRITE, {Range{L.part, pslot, pslot + (uint32_t)(G * (D + 4))}}, -1};
            ph.push_back(w);
          }
          break;
        }
        const uint32_t row = it.b * (uint32_t)((Hq + 2 * Hkv) * D);
        const int pos = ctx[it.b] - 1;
        const bool has_new = pos >= it.p0 && pos < it.p1;
        Phase in{in_kind, {Range{L.qkv, row + it.kvh * G * D, row + (it.kvh + 1) * G * D}}, -1};
        if (has_new) {
          in.r.push_back(Range{L.qkv, row + (Hq + it.kvh) * D, row + (Hq + it.kvh + 1) * D});
          in.r.push_back(Range{L.qkv, row + (Hq + Hkv + it.kvh) * D, row + (Hq + Hkv + it.kvh + 1) * D});
        }
        ph.push_back(in);
        if (has_new) {
          Phase rk{PH_POLL, {Range{b_rowok, (uint32_t)it.b, (uint32_t)it.b + 1}}, -1};
          ph.push_back(rk);
        }
        Phase w{PH_WRITE, {}, -1};
        for (int g = 0; g < G; ++g) {
          const uint32_t h = pslot + g * (D + 4);
          w.r.push_back(Range{L.part, h, h + 2});
          w.r.push_back(Range{L.part, h + 4, h + 4 + D});
        }
        ph.push_back(w);
        if (attn_is_merger(it, Hkv, o.row0)) {
          Phase mp{PH_POLL, {}, -1};  // the merger polls every chunk's partial, tags always
          for (int c = 0; c < it.n_b; ++c) {
            const uint32_t s = (uint32_t)(it.first_item + c * Hkv) * GMAX * (D + 4);
            for (int g = 0; g < G; ++g) {
              const uint32_t h = s + g * (D + 4);
              mp.r.push_back(Range{L.part, h, h + 2});
              mp.r.push_back(Range{L.part, h + 4, h + 4 + D});
            }
          }
          ph.push_back(mp);
          const uint32_t orow = it.b * (uint32_t)P.mix_dim + it.kvh * G * D;
          Phase mw{PH_WRITE, {Range{L.mix_o, orow, orow + (uint32_t)(G * D)}}, -1};
          ph.push_back(mw);
        }
        break;
      }
      case OP_DELTA: {
        const LayerBufs& L = lb[o.layer];
        const int nh = d.n_delta_heads, dk = d.delta_dk, dv = d.delta_dv, ncb = dv / 32;
        const int cb = (int)(o.row0 % (uint32_t)ncb), bh = (int)(o.row0 / (uint32_t)ncb);
        const int b = bh / nh, h = bh % nh;
        const uint32_t row = b * (uint32_t)(m.C + 2 * nh);
        Phase in{in_kind, {}, -1};
        in.r.push_back(Range{L.qkv, row + h * dk, row + (h + 1) * dk});
        in.r.push_back(Range{L.qkv, row + nh * dk + h * dk, row + nh * dk + (h + 1) * dk});
        const uint32_t vc = row + 2 * nh * dk + h * dv + cb * 32;
        in.r.push_back(Range{L.qkv, vc, vc + 32});
        in.r.push_back(Range{L.qkv, row + m.C + h, row + m.C + h + 1});
        in.r.push_back(Range{L.qkv, row + m.C + nh + h, row + m.C + nh + h + 1});
        ph.push_back(in);
        const uint32_t orow = b * (uint32_t)P.mix_dim + h * dv + cb * 32;
        Phase w{PH_WRITE, {Range{L.mix_o, orow, orow + 32}}, -1};
        ph.push_back(w);
        break;
      }
      default:
        break;
    }
  }
  int cur_cu = 0;

  bool is_mixer_out(uint64_t addr) const {
    int bi = -1;
    uint32_t c = 0;
    if (!resolve(addr, &bi, &c)) return false;
    for (const auto& L : lb)
      if (L.mix_o == bi) return true;
    return false;
  }
  bool mixer_row_written(uint32_t layer, int b) const {
    return m.kinds[layer] == MK_LAYER_ATTN ? live(b) : b < m.d.max_batch;
  }

  // ------------------------------------------------------------------ one launch
  bool cell_ok(const Buf& bf, uint32_t i) const {
    return bf.full_tag ? bf.lastw[i] == tag : (bf.lastw[i] & 1u) == (tag & 1u);
  }

  // Returns false when the launch ended in a deadlock.
  bool run_launch(int li, std::vector<CuState>& cu) {
    const mk_model_desc& d = m.d;
    std::fill(stage_done.begin(), stage_done.end(), 0u);
    for (int c = 0; c < P.n_cus; ++c) {
      CuState& s = cu[c];
      s = CuState{};
      s.oi = P.queue_off[c];
      s.oend = P.queue_off[c + 1];
      s.done = s.oi >= s.oend;
    }
    const bool stall = (cfg.flags & MK_EMU_STALL_ONE_OP) && li == 0;
    // the stalled op: the first attention or delta op of the middle compute unit, else its first op
    int stall_cu = P.n_cus / 2;
    uint32_t stall_op = P.queue_off[stall_cu];
    for (uint32_t i = P.queue_off[stall_cu]; i < P.queue_off[stall_cu + 1]; ++i)
      if (P.ops[i].opcode == OP_ATTN || P.ops[i].opcode == OP_DELTA) { stall_op = i; break; }

    std::vector<int> runnable;
    for (int c = 0; c < P.n_cus; ++c)
      if (!cu[c].done) runnable.push_back(c);
    int remaining = (int)runnable.size();
    std::vector<int> blocked;

    auto wake_range = [&](int bi, uint32_t lo, uint32_t hi) {
      for (size_t k = 0; k < blocked.size();) {
        CuState& s = cu[blocked[k]];
        if (s.wbuf == bi && s.wcell >= lo && s.wcell < hi) {
          s.blocked = false;
          runnable.push_back(blocked[k]);
          blocked[k] = blocked.back();
          blocked.pop_back();
        } else {
          ++k;
        }
      }
    };
    auto wake_counters = [&]() {
      for (size_t k = 0; k < blocked.size();) {
        CuState& s = cu[blocked[k]];
        if (s.wbuf == -2) {
          s.blocked = false;
          runnable.push_back(blocked[k]);
          blocked[k] = blocked.back();
          blocked.pop_back();
        } else {
          ++k;
        }
      }
    };

    while (remaining > 0) {
      if (runnable.empty()) {
        ++rep.deadlocks;
        note("launch " + std::to_string(li) + ": every remaining compute unit waits (the watchdog would end it)");
        return false;
      }
      const size_t pick = (size_t)(rng() % runnable.size());
      const int c = runnable[pick];
      CuState& s = cu[c];
      cur_cu = c;
      // load the next op's phases
      if (s.ph.empty() || s.pi >= s.ph.size()) {
        if (!s.ph.empty()) {  // the op has finished: signal its stage
          const Op& o = P.ops[s.oi];
          if (o.sig_stage != NO_STAGE && !(o.flags & OPF_NO_SIGNAL)) {
            if (++stage_done[o.sig_stage] == P.stages[o.sig_stage].nops) wake_counters();
          }
          ++rep.ops_run;
          ++s.oi;
          s.ph.clear();
          s.pi = 0;
          if (s.oi >= s.oend) {
            s.done = true;
            runnable[pick] = runnable.back();
            runnable.pop_back();
            --remaining;
            continue;
          }
        }
        phases_of(P.ops[s.oi], s.ph);
        s.pi = 0;
        s.chunk = 0;
        s.started = false;
        if (s.ph.empty()) {  // an op with nothing to do: finishes at once
          s.ph.push_back(Phase{PH_WRITE, {}, -1});
        }
      }
      Phase& ph = s.ph[s.pi];
      auto block_on = [&](int bi, uint32_t cell) {
        s.blocked = true;
        s.wbuf = bi;
        s.wcell = cell;
        blocked.push_back(c);
        runnable[pick] = runnable.back();
        runnable.pop_back();
      };
      if (ph.kind == PH_COUNTER) {
        if (stage_done[ph.stage] >= P.stages[ph.stage].nops) {
          ++s.pi;
        } else {
          block_on(-2, 0);
        }
        continue;
      }
      if (ph.kind == PH_POLL || ph.kind == PH_READ) {
        if (!s.started) {  // first look: every cell read once; those not yet current are pending
          s.started = true;
          s.pending.clear();
          for (const Range& r : ph.r) {
            const Buf& bf = bufs[r.buf];
            for (uint32_t i = r.lo; i < r.hi; ++i) {
              if (ph.kind == PH_READ) {  // after a counter wait: the value must be this launch's
                if (bf.lastw[i] != tag) {
                  ++rep.unsynced_reads;
                  if (rep.unsynced_reads <= 3) note("launch " + std::to_string(li) + ": a read after its counter wait found an unwritten value");
                }
                continue;
              }
              if (!cell_ok(bf, i)) s.pending.push_back({r.buf, i});
              else if (bf.lastw[i] != tag) {
                ++rep.stale_accepts;
                if (rep.stale_accepts <= 3)
                  note("launch " + std::to_string(li) + ": op " + std::to_string(s.oi) + " accepted a value of launch " +
                       std::to_string(bf.lastw[i]));
              }
            }
          }
        } else {  // re-read the pending cells, as the kernel re-reads stale fragments
          size_t k = 0;
          for (size_t j = 0; j < s.pending.size(); ++j) {
            const Buf& bf = bufs[s.pending[j].first];
            const uint32_t i = s.pending[j].second;
            if (!cell_ok(bf, i)) s.pending[k++] = s.pending[j];
            else if (bf.lastw[i] != tag) {
              ++rep.stale_accepts;
              if (rep.stale_accepts <= 3) note("launch " + std::to_string(li) + ": stale value accepted on re-read");
            }
          }
          s.pending.resize(k);
        }
        if (!s.pending.empty()) {
          block_on(s.pending[0].first, s.pending[0].second);
        } else {
          ++rep.polls;
          ++s.pi;
          s.started = false;
        }
        continue;
      }
      // PH_WRITE: the ranges in two halves, so that consumers can see a partly written op
      if (stall && s.oi == stall_op) {
        s.stalled = true;
        block_on(-3, 0);  // never woken
        continue;
      }
      const size_t n = ph.r.size(), half = (n + 1) / 2;
      const size_t lo = s.chunk == 0 ? 0 : half, hi = s.chunk == 0 ? half : n;
      for (size_t k = lo; k < hi; ++k) {
        const Range& r = ph.r[k];
        Buf& bf = bufs[r.buf];
        for (uint32_t i = r.lo; i < r.hi; ++i) {
          bf.lastw[i] = tag;
          if (++bf.nw[i] == 2) {
            ++rep.double_writes;
            if (rep.double_writes <= 3) note("launch " + std::to_string(li) + ": a tagged value written twice");
          }
        }
        wake_range(r.buf, r.lo, r.hi);
      }
      if (s.chunk == 0 && half < n) {
        s.chunk = 1;
      } else {
        s.chunk = 0;
        ++s.pi;
      }
    }
    // every pollable cell written exactly once in this launch
    for (Buf& bf : bufs) {
      for (size_t i = 0; i < bf.floats; ++i) {
        if (bf.pollable[i] && bf.nw[i] == 0) {
          ++rep.unwritten_cells;
          if (rep.unwritten_cells <= 3) note("launch " + std::to_string(li) + ": a pollable value was not written");
        }
        bf.nw[i] = 0;
      }
    }
    (void)d;
    return true;
  }

  void run() {
    setup();
    stage_done.assign(P.stages.size(), 0u);
    std::vector<CuState> cu(P.n_cus);
    const mk_model_desc& d = m.d;
    const int K = Hkv > 0 ? P.n_items / Hkv : 0;
    for (int li = 0; li < cfg.n_launches; ++li) {
      tag = (uint32_t)li + 1;
      batch = cfg.batch[li];
      int cv[APLAN_MAXB] = {0};
      for (int b = 0; b < APLAN_MAXB; ++b) {
        ctx[b] = 0;
        if (b < batch && b < d.max_batch) ctx[b] = attn_clamp_ctx(cfg.ctx_lens[(size_t)li * d.max_batch + b], d.max_ctx);
        cv[b] = ctx[b];
      }
      if (m.n_attn) attn_plan_make(cv, K, attn_pps(D), NC, plan);
      const int64_t bad0 = rep.stale_accepts + rep.unsynced_reads + rep.double_writes + rep.unwritten_cells;
      const bool ok = run_launch(li, cu);
      const int64_t bad1 = rep.stale_accepts + rep.unsynced_reads + rep.double_writes + rep.unwritten_cells;
      if ((bad1 != bad0 || !ok) && rep.first_bad_launch < 0) rep.first_bad_launch = li;
      if (!ok) break;  // the kernel would have stopped with a timeout; mk_reset starts afresh
    }
  }
};

}  // namespace

std::string emulate(const ModelShape& m, const mk_emu_config& cfg, mk_emu_report* rep) {
  *rep = mk_emu_report{};
  rep->first_bad_launch = -1;
  Plan P;
  const int dep = (cfg.flags & MK_EMU_COUNTERS) ? 1 : 0;
  std::string e = build_plan(m, cfg.n_cus, nullptr, nullptr, &P, dep);
  if (!e.empty()) return e;
  Emu emu(m, P, cfg, *rep);
  emu.run();
  return emu.msg;
}

}  // namespace mk
