// mk_attn_plan.h -- the decode step's split of every sequence's cached context into attention
// chunks, shared by the gfx950 megakernel (which builds it once per step in LDS) and the host
// (the protocol emulator replays the kernel's own plan over launch sequences).
//
// Split-KV decode attention (paged GQA decode, the ForgeKernel blog post on ai6s.net, results
// section) cuts each (sequence, KV head) context into chunks that run on different compute units
// and are merged with the log-sum-exp rule.  Here every KV head gets at most K = n_items / Hkv
// chunks per step.  Each step picks one chunk length cs_all (a multiple of the positions one ring
// slot holds, at least `min_slots` slots, the smallest such length that needs at most K chunks per
// KV head); each sequence then keeps its chunk count at cs_all but evens its chunks out (lengths a
// multiple of pps, at most cs_all), so a ragged batch leaves no short last chunk per sequence.
//
// Items: item i of a layer is chunk i / Hkv (counted over the sequences in order) of KV head
// i % Hkv.  Chunks past the step's total are items with no work.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define MK_HD __host__ __device__ __forceinline__
#else
#define MK_HD inline
#endif

namespace mk {

constexpr int APLAN_MAXB = 8;
// Flat plan words: [0, 8) clamped context per sequence (0 = not live), [8, 16) chunk length per
// sequence, [16, 25) chunks of the sequences before b (entry 8 = all chunks).
constexpr int APLAN_CTX = 0, APLAN_CS = 8, APLAN_FIRST = 16, APLAN_WORDS = 25;

// A sequence takes part in attention this step when it is in the batch and its context length
// lies in [1, max_ctx].
MK_HD int attn_clamp_ctx(int c, int max_ctx) { return (c >= 1 && c <= max_ctx) ? c : 0; }

// cv[b]: clamped context of sequence b (0 for b >= batch).  K: chunks per KV head.  pps: positions
// per ring slot.  min_slots: the least slots per chunk (shorter chunks leave compute waves idle and
// only add partials for the merger to fold).  Writes the APLAN_WORDS plan words.
MK_HD void attn_plan_make(const int* cv, int K, int pps, int min_slots, int* plan) {
  int total = 0, nz = 0, maxc = 0;
  for (int b = 0; b < APLAN_MAXB; ++b) {
    total += cv[b];
    nz += cv[b] > 0 ? 1 : 0;
    maxc = cv[b] > maxc ? cv[b] : maxc;
  }
  int cs_all = 0;
  if (total > 0 && K >= nz) {
    int lo = ((total + K - 1) / K + pps - 1) / pps;
    if (lo < min_slots) lo = min_slots;
    int hi = (maxc + pps - 1) / pps;
    if (lo > hi) lo = hi;
    while (lo < hi) {  // smallest slot count whose chunks fit K per KV head
      const int mid = (lo + hi) / 2, c = mid * pps;
      int n = 0;
      for (int b = 0; b < APLAN_MAXB; ++b) n += (cv[b] + c - 1) / c;
      if (n <= K) hi = mid;
      else lo = mid + 1;
    }
    cs_all = lo * pps;
  }
  int acc = 0;
  for (int b = 0; b < APLAN_MAXB; ++b) {
    const int nb = cv[b] > 0 && cs_all > 0 ? (cv[b] + cs_all - 1) / cs_all : 0;
    const int cs = nb > 0 ? ((cv[b] + nb - 1) / nb + pps - 1) / pps * pps : 0;
    plan[APLAN_CTX + b] = cv[b];
    plan[APLAN_CS + b] = cs;
    plan[APLAN_FIRST + b] = acc;
    acc += nb;
  }
  plan[APLAN_FIRST + APLAN_MAXB] = acc;
}

struct AttnItem {
  int b, kvh, p0, p1, n_b, first_item;  // first_item: item index of chunk 0 of (b, kvh)
  bool valid;
};

// Item i -> (sequence, KV head, position range [p0, p1)).  `word(i)` returns plan word i, so the
// kernel can read the plan from LDS and the host from an array.
template <typename Word>
MK_HD AttnItem attn_item_from(Word word, int batch, int Hkv, uint32_t item) {
  AttnItem it{0, 0, 0, 0, 0, 0, false};
  const int bc = (int)(item / (uint32_t)Hkv), kvh = (int)(item % (uint32_t)Hkv);
  for (int b = 0; b < batch && b < APLAN_MAXB; ++b) {
    const int c0 = word(APLAN_FIRST + b), c1 = word(APLAN_FIRST + b + 1);
    if (bc < c1) {
      const int k = bc - c0, c = word(APLAN_CTX + b), cs = word(APLAN_CS + b);
      it.b = b;
      it.kvh = kvh;
      it.p0 = k * cs;
      it.p1 = c < (k + 1) * cs ? c : (k + 1) * cs;
      it.n_b = c1 - c0;
      it.first_item = c0 * Hkv + kvh;
      it.valid = true;
      return it;
    }
  }
  return it;
}

// The chunk of (b, kvh) that merges all of that pair's partials: the last one in item order.
MK_HD bool attn_is_merger(const AttnItem& it, int Hkv, uint32_t item) {
  return it.valid && item == (uint32_t)(it.first_item + (it.n_b - 1) * Hkv);
}

// Positions per ring slot for head_dim d (a slot holds K and V of pps positions, 8 KB).
MK_HD int attn_pps(int d) { return 4096 / (2 * d); }

}  // namespace mk
