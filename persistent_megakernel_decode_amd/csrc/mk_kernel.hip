// mk_kernel.hip -- the persistent decode megakernel for gfx950 (MI355X).
//
// One workgroup per compute unit runs the whole decode step.  Structure after
// the ForgeMegakernel abstract (arxivdaily / arxiv.science, abstract): a
// fine-grained instruction stream per compute unit (each workgroup walks its
// own queue of Ops), dependency counters instead of grid-wide
// synchronisation, and an on-chip buffer pool (a 128 KB LDS ring) that stages
// the weight, KV and recurrent-state bytes each Op streams.
//
// Per workgroup: wave 0 is the LOADER.  It walks the queue ahead of the
// compute waves and issues global_load_lds_dwordx4 (1 KB per instruction,
// non-temporal) into free ring slots.  Weights never depend on activations,
// so the loader never waits on a dependency counter: it keeps HBM busy while
// the compute waves wait for the previous stage (the prefetch-ahead of the
// per-layer megakernel described in the LMSYS Muse Spark post quoted on the
// khabar-ai page).  Waves 1..NC COMPUTE: per Op they wait on the producer
// stage's counters, read their small fp32 inputs, consume the ring slots,
// write outputs and signal.
//
// Cross-CU coherence without cache flushes: MI355X has one L2 per XCD and the
// L2s are not coherent with each other.  Every activation that crosses
// compute units is written and read with sc1 (agent-scope) buffer accesses,
// which bypass the non-coherent L2 state; a producer waits vmcnt(0) for its
// stores, then increments a split counter with a relaxed agent-scope atomic.
// No buffer_wbl2 / buffer_inv is issued anywhere on the path.
#include <hip/hip_runtime.h>

#include "mk_internal.h"

namespace mk {

typedef uint32_t u32;
typedef uint64_t u64;
typedef __attribute__((ext_vector_type(4))) u32 u32x4;
typedef __attribute__((ext_vector_type(2))) u32 u32x2;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14])
#define MK_VMCNT(n) ((((n) & 0xF) | (((n) >> 4) << 14)) | 0x70 | 0xF00)
#define MK_LGKMCNT0 (0xF | 0x70 | (0x3 << 14))

constexpr int AUX_NT = 2;    // cache policy: non-temporal (streamed once)
constexpr int AUX_SC1 = 16;  // cache policy: agent-scope coherent

// ------------------------------------------------------------------ LDS
// The ring is its own object so the compiler's LDS-DMA tracking never makes
// ordinary LDS accesses of the loader wait for outstanding DMA.
__shared__ __attribute__((aligned(16))) u32x4 g_ring[NSLOT * SLOT / 16];
__shared__ __attribute__((aligned(16))) float g_red[RED_FLOATS];
__shared__ __attribute__((aligned(16))) float g_scr[SCRATCH_FLOATS];
__shared__ u32 g_full[NSLOT];   // slot seq / NSLOT + 1 once the slot's bytes landed
__shared__ u32 g_done[NSLOT];   // cumulative consumption count (NC per slot use)
__shared__ u32 g_bar;           // compute-wave barrier counter
__shared__ u32 g_abort;         // set on watchdog expiry: every wave leaves
__shared__ u32 g_bcast[4];

// ------------------------------------------------------------------ helpers
// Uniform, kernel-invariant data (queues, plan tables, inputs) read through the constant
// address space, which the compiler turns into scalar loads.
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "scalar loads move whole dwords");
  constexpr int N = sizeof(T) / 4;
  const __attribute__((address_space(4))) u32* q = (const __attribute__((address_space(4))) u32*)p;
  u32 tmp[N];
#pragma unroll
  for (int i = 0; i < N; ++i) tmp[i] = q[i];
  T out;
  __builtin_memcpy(&out, tmp, sizeof(T));
  return out;
}

// Agent-coherent accesses for data that crosses compute units: relaxed agent-scope atomics,
// i.e. global loads / stores with the sc1 cache-policy bit, with per-lane addresses.
__device__ __forceinline__ float ld_sc1(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load((const u32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_sc1(float* p, float v) {
  __hip_atomic_store((u32*)p, __builtin_bit_cast(u32, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ld8_sc1(const float* p, float* out) {  // 8 consecutive floats, 8-B aligned
  const uint64_t* q = (const uint64_t*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t v = __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    out[2 * i] = __builtin_bit_cast(float, (u32)v);
    out[2 * i + 1] = __builtin_bit_cast(float, (u32)(v >> 32));
  }
}
__device__ __forceinline__ u32 ld_u32_sc1(const u32* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_i32_sc1(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __builtin_bit_cast(float, (u32)h << 16); }
__device__ __forceinline__ float bflo(u32 w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bfhi(u32 w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even (finite inputs)
  u32 u = __builtin_bit_cast(u32, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ u32 lane_id() { return threadIdx.x & 63u; }

__device__ __forceinline__ float wave_sum(float v) {  // full-wave sum, result in every lane
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ u32 lds_ld(const u32* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ bool aborted() { return lds_ld(&g_abort) != 0; }

// LDS read for the loader wave.  The compiler cannot tell that the ring (the only LDS the
// DMA writes) and the control words are distinct, and would drain every outstanding DMA
// (vmcnt(0)) before each ordinary LDS read, serialising the stream.  This read is opaque to
// that tracking; it waits for its own result inside the same asm block.
__device__ __forceinline__ u32 lds_ld_loader(const u32* p) {
  const u32 addr = (u32)(uintptr_t)(const __attribute__((address_space(3))) u32*)p;
  u32 v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ bool aborted_loader() { return lds_ld_loader(&g_abort) != 0; }


__device__ void raise_status(const KArgs& A, u32 bits) {
  __hip_atomic_fetch_or(A.status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every spin in the kernel is bounded: past the watchdog limit the waiting wave raises
// ST_TIMEOUT and sets the workgroup abort flag, and every wave of the workgroup leaves.
struct Watchdog {
  uint64_t t0, limit;
  u32* status;
  __device__ explicit Watchdog(const KArgs& A) : t0(__builtin_amdgcn_s_memrealtime()), limit(A.spin_limit), status(A.status) {}
  __device__ bool expired() {
    if (__builtin_amdgcn_s_memrealtime() - t0 <= limit) return false;
    if (lane_id() == 0) {
      __hip_atomic_fetch_or(status, ST_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&g_abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    return true;
  }
};

// Barrier among the NC compute waves (the loader never joins).  Returns false on abort.
__device__ bool cbar(const KArgs& A, u32& gen) {
  __builtin_amdgcn_s_waitcnt(MK_LGKMCNT0);
  gen += NC;
  if (lane_id() == 0) __hip_atomic_fetch_add(&g_bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  Watchdog wd(A);
  while (__hip_atomic_load(&g_bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < gen) {
    if (aborted() || wd.expired()) return false;
    __builtin_amdgcn_s_sleep(0);
  }
  return true;
}

// Wait until ring slot `seq` holds its bytes.  Returns false on abort.
__device__ bool wait_full(const KArgs& A, u32 seq) {
  const u32 pos = seq % NSLOT, want = seq / NSLOT + 1;
  Watchdog wd(A);
  while (lds_ld(&g_full[pos]) != want) {
    if (aborted() || wd.expired()) return false;
    __builtin_amdgcn_s_sleep(0);
  }
  return true;
}
__device__ __forceinline__ void release_slot(u32 seq, u32 n) {
  __builtin_amdgcn_s_waitcnt(MK_LGKMCNT0);  // this wave's reads of the slot are complete
  if (lane_id() == 0) __hip_atomic_fetch_add(&g_done[seq % NSLOT], n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ------------------------------------------------------------------ per-row validity
// A row is served only when its token, context length, position and current page are in range.
__device__ bool row_ok_local(const KArgs& A, int b) {
  if (b >= A.batch) return false;
  int tok = A.tokens[b], ctx = A.ctx_lens[b], pos = A.positions[b];
  if (tok < 0 || tok >= A.V) return false;
  if (ctx < 1 || ctx > A.max_ctx || pos != ctx - 1) return false;
  if (!A.page_table) return true;  // no attention layers: no pages to check
  int pi = pos / A.page_size;
  if (pi >= A.max_pages_per_seq) return false;
  int pg = A.page_table[(size_t)b * A.max_pages_per_seq + pi];
  return pg >= 0 && pg < A.num_pages;
}

// ------------------------------------------------------------------ attention work split
struct AttnItem {
  int b, kvh, p0, p1, n_b, first_item;  // first_item: item index of chunk 0 of (b, kvh)
  bool valid;
};

__device__ __forceinline__ int clamp_ctx(const KArgs& A, int c) { return (c >= 1 && c <= A.max_ctx) ? c : 0; }

// Item i -> (sequence, KV head, position range).  Uniform; reads ctx_lens with scalar loads.
__device__ AttnItem attn_item(const KArgs& A, u32 item, int pps) {
  AttnItem it{0, 0, 0, 0, 0, 0, false};
  int64_t total = 0;
  for (int b = 0; b < A.batch; ++b) total += clamp_ctx(A, sload(A.ctx_lens + b));
  if (total == 0) return it;
  const int cs = attn_chunk_size(total, A.Hkv, A.n_cus, pps);
  const int bc = (int)(item / (u32)A.Hkv), kvh = (int)(item % (u32)A.Hkv);
  int acc = 0;
  for (int b = 0; b < A.batch; ++b) {
    const int ctx = clamp_ctx(A, sload(A.ctx_lens + b));
    const int nb = (ctx + cs - 1) / cs;
    if (bc < acc + nb) {
      const int c = bc - acc;
      it.b = b; it.kvh = kvh; it.p0 = c * cs; it.p1 = min(ctx, (c + 1) * cs);
      it.n_b = nb; it.first_item = acc * A.Hkv + kvh; it.valid = true;
      return it;
    }
    acc += nb;
  }
  return it;
}

__device__ __forceinline__ int attn_pps(int d) { return 4096 / (2 * d); }  // positions per ring slot

// ------------------------------------------------------------------ loader
__device__ __forceinline__ void dma16(const void* g, u32x4* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, AUX_NT);
}

// Publish "slot `seq` holds its bytes" (after the matching s_waitcnt vmcnt).  Written as an opaque
// LDS store for the same reason as lds_ld_loader: the compiler would otherwise drain every DMA first.
__device__ __forceinline__ void mark_full(u32 seq) {
  const u32 addr = (u32)(uintptr_t)(__attribute__((address_space(3))) u32*)&g_full[seq % NSLOT];
  const u32 v = seq / NSLOT + 1;
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(addr), "v"(v) : "memory");
}

// Wait until the oldest of n in-flight slots has landed (8 DMA instructions per slot).
__device__ __forceinline__ void wait_oldest(u32 n) {
  switch (n) {
    case 1: __builtin_amdgcn_s_waitcnt(MK_VMCNT(0)); break;
    case 2: __builtin_amdgcn_s_waitcnt(MK_VMCNT(8)); break;
    case 3: __builtin_amdgcn_s_waitcnt(MK_VMCNT(16)); break;
    case 4: __builtin_amdgcn_s_waitcnt(MK_VMCNT(24)); break;
    default: __builtin_amdgcn_s_waitcnt(MK_VMCNT(32)); break;
  }
}
static_assert(LOAD_DEPTH == 4, "wait_oldest covers LOAD_DEPTH + 1 in-flight slots");

// GEMV stream: piece p of the op = (stream row p / ppr, row piece p % ppr).
__device__ void issue_gemv(const Op& o, u32 s, u32x4* dst) {
  const u32 lane = lane_id();
  const u32 nrt = o.epi == EPI_SWIGLU ? 2 * o.nrows : o.nrows;
  const u32 K = o.K;
  const uint16_t* W0 = (const uint16_t*)o.W;
#pragma unroll
  for (int i = 0; i < SLOT_PIECES; ++i) {
    const u32 p = s * SLOT_PIECES + i;
    const u32 rl = p / o.ppr, kp = p - rl * o.ppr;
    const uint16_t* rowp = W0;  // dummy piece (past the op's rows): row 0 of W, always mapped
    u32 e = (lane * 8) % K;
    if (rl < nrt && kp * PIECE_ELEMS < K) {
      const uint16_t* Wt;
      u32 r;
      if (o.epi == EPI_SWIGLU) {
        const bool up = rl >= o.nrows;
        Wt = up ? (const uint16_t*)o.W2 : W0;
        r = o.row0 + (up ? rl - o.nrows : rl);
      } else {
        const u32 g = o.row0 + rl;
        if (g < o.b1) { Wt = W0; r = g; }
        else if (g < o.b2) { Wt = (const uint16_t*)o.W2; r = g - o.b1; }
        else { Wt = (const uint16_t*)o.W3; r = g - o.b2; }
      }
      rowp = Wt + (size_t)r * K;
      const u32 ee = kp * PIECE_ELEMS + lane * 8;
      e = ee < K ? ee : e;
    }
    dma16(rowp + e, dst + i * 64);
  }
}

// Attention stream: slot s = PPS positions of K (pieces 0-3) then the same positions of V (4-7).
__device__ void issue_attn(const KArgs& A, const LayerDesc& Ld, const AttnItem& it, u32 s, u32x4* dst) {
  const u32 lane = lane_id();
  const int d = A.d, pps = attn_pps(d), ppp = pps / 4;  // positions per piece
  const size_t page_elems = (size_t)A.Hkv * A.page_size * d;
#pragma unroll
  for (int i = 0; i < SLOT_PIECES; ++i) {
    const uint16_t* base = (const uint16_t*)(i < 4 ? Ld.k_pages : Ld.v_pages);
    const int pp = it.p0 + (int)s * pps + (i & 3) * ppp;
    const uint16_t* src = base + lane * 8;  // dummy: page 0
    if (pp < it.p1) {
      int pi = pp / A.page_size;
      pi = pi < A.max_pages_per_seq ? pi : 0;
      int pg = sload(A.page_table + (size_t)it.b * A.max_pages_per_seq + pi);
      pg = (pg >= 0 && pg < A.num_pages) ? pg : 0;
      src = base + (size_t)pg * page_elems + ((size_t)it.kvh * A.page_size + (pp % A.page_size)) * d + lane * 8;
    }
    dma16(src, dst + i * 64);
  }
}

// Delta stream: rows of S^T (fp32) of one column block, contiguous.
__device__ void issue_delta(const KArgs& A, const LayerDesc& Ld, u32 item, u32 s, u32x4* dst) {
  const u32 lane = lane_id();
  const u32 ncb = (u32)A.dv / 32, cb = item % ncb, bh = item / ncb;  // bh = b * nh + h
  const u32 rps = SLOT / (A.dk * 4);
  const char* src = (const char*)Ld.delta_state +
                    (((size_t)bh * A.dv + cb * 32 + s * rps) * A.dk) * 4;
#pragma unroll
  for (int i = 0; i < SLOT_PIECES; ++i) dma16(src + i * PIECE + lane * 16, dst + i * 64);
}

__device__ u32 op_slots(const KArgs& A, const Op& o) {
  if (o.opcode == OP_ATTN) {
    const int pps = attn_pps(A.d);
    AttnItem it = attn_item(A, o.row0, pps);
    return it.valid ? (u32)((it.p1 - it.p0 + pps - 1) / pps) : 0u;
  }
  return o.nslots;
}

__device__ void loader(const KArgs& A, u32 q0, u32 q1) {
  u32 seq = 0, marked = 0;
  for (u32 oi = q0; oi < q1; ++oi) {
    const Op o = sload(A.ops + oi);
    const u32 ns = op_slots(A, o);
    if (ns == 0) continue;
    LayerDesc Ld{};
    AttnItem it{};
    if (o.opcode == OP_ATTN || o.opcode == OP_DELTA) Ld = sload(A.layers + o.layer);
    if (o.opcode == OP_ATTN) it = attn_item(A, o.row0, attn_pps(A.d));
    for (u32 s = 0; s < ns; ++s) {
      const u32 pos = seq % NSLOT, round = seq / NSLOT;
      Watchdog wd(A);
      while (lds_ld_loader(&g_done[pos]) < round * NC) {  // slot still holds unconsumed bytes
        if (marked < seq) {
          wait_oldest(seq - marked);
          mark_full(marked++);
        } else {
          if (aborted_loader() || wd.expired()) {
            __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));
            return;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      u32x4* dst = g_ring + pos * (SLOT / 16);
      if (o.opcode == OP_GEMV) issue_gemv(o, s, dst);
      else if (o.opcode == OP_ATTN) issue_attn(A, Ld, it, s, dst);
      else issue_delta(A, Ld, o.row0, s, dst);
      ++seq;
      if (seq - marked > LOAD_DEPTH) {
        __builtin_amdgcn_s_waitcnt(MK_VMCNT(8 * LOAD_DEPTH));
        mark_full(marked++);
      }
    }
  }
  while (marked < seq) {
    wait_oldest(seq - marked);
    mark_full(marked++);
  }
}

// ------------------------------------------------------------------ dependency wait / signal
__device__ bool wait_stage(const KArgs& A, int stage) {
  const u32 lane = lane_id();
  const Stage st = sload(A.stages + stage);
  const u32 per = st.nops / NSUB, rem = st.nops % NSUB;
  const u32 tgt = A.epoch * (per + (lane < rem ? 1u : 0u));
  const u32* c = A.counters + (size_t)stage * NSUB * CTR_STRIDE + (size_t)(lane % NSUB) * CTR_STRIDE;
  Watchdog wd(A);
  while (true) {
    const u32 v = lane < (u32)NSUB ? ld_u32_sc1(c) : 0xFFFFFFFFu;
    if (__builtin_amdgcn_ballot_w64(v < tgt) == 0) return true;
    if (aborted() || wd.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ void signal_stage(const KArgs& A, int stage, u32 index) {
  u32* c = A.counters + (size_t)stage * NSUB * CTR_STRIDE + (size_t)(index % NSUB) * CTR_STRIDE;
  __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ EMBED
// x0[b][h] = E[token_b][h] for this CU's slice of h (rows with b >= batch or a bad token are zero).
__device__ void op_embed(const KArgs& A, u32 w) {
  const u32 t = w * 64 + lane_id();
  const int cu = (int)blockIdx.x;
  const int h0 = (int)((int64_t)A.H * cu / A.n_cus), h1 = (int)((int64_t)A.H * (cu + 1) / A.n_cus);
  for (int b = 0; b < A.max_batch; ++b) {
    const int tok = b < A.batch ? A.tokens[b] : -1;
    const bool ok = tok >= 0 && tok < A.V;
    for (int h = h0 + (int)t; h < h1; h += NC * 64)
      st_sc1(A.x0 + (size_t)b * A.H + h, ok ? bf2f(A.embed[(size_t)tok * A.H + h]) : 0.0f);
  }
}

// Second phase of EMBED, CU 0 only: validate every row (token, context, position, every page of
// [0, ctx) mapped), publish row_ok and raise ST_BAD_INPUT for out-of-contract rows.
__device__ void op_embed_finish(const KArgs& A, u32 w, u32& gen) {
  if (blockIdx.x != 0) return;
  for (int b = 0; b < A.max_batch; ++b) {
    bool ok = row_ok_local(A, b);
    float bad = 0.0f;
    if (ok && A.page_table) {
      const int npg = (A.ctx_lens[b] + A.page_size - 1) / A.page_size;
      if (npg > A.max_pages_per_seq) bad = 1.0f;
      for (int p = (int)(w * 64 + lane_id()); p < npg && bad == 0.0f; p += NC * 64) {
        const int pg = A.page_table[(size_t)b * A.max_pages_per_seq + p];
        if (pg < 0 || pg >= A.num_pages) bad = 1.0f;
      }
    }
    bad = wave_max(bad);
    if (lane_id() == 0) g_scr[w] = bad;
    if (!cbar(A, gen)) return;
    if (w == 0 && lane_id() == 0) {
      float any = 0.0f;
      for (int j = 0; j < NC; ++j) any = fmaxf(any, g_scr[j]);
      const bool final_ok = ok && any == 0.0f;
      __hip_atomic_store(A.row_ok + b, final_ok ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (b < A.batch && !final_ok) raise_status(A, ST_BAD_INPUT);
    }
    if (!cbar(A, gen)) return;
  }
}

// ------------------------------------------------------------------ GEMV (VALU, batch B)
template <int B>
struct MMax { static constexpr int v = B <= 2 ? 4 : (B <= 4 ? 2 : 1); };

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <int B>
__device__ bool op_gemv(const KArgs& A, const Op& o, u32 w, u32& seq, u32& gen) {
  constexpr int MM = MMax<B>::v;
  const u32 lane = lane_id();
  const u32 ppr = o.ppr, K = o.K;
  const bool swiglu = o.epi == EPI_SWIGLU;
  const u32 nrt = swiglu ? 2 * o.nrows : o.nrows;
  const u32 M = ppr >= 8 ? ppr / 8 : 1;
  const u32 RW = ppr >= 8 ? 8 : ppr;

  // this wave's input fragments: piece kp covers elements [kp*512, kp*512+512), lane owns 8 of them
  float xf[MM][B][8];
#pragma unroll
  for (int t = 0; t < MM; ++t) {
    const u32 kp = ppr >= 8 ? w + 8 * t : w % ppr;
    const u32 k0 = kp * PIECE_ELEMS + lane * 8;
    const bool valid = (u32)t < M && kp < ppr && k0 < K;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (valid) ld8_sc1((const float*)o.in + (size_t)b * o.ld_in + k0, xf[t][b]);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xf[t][b][e] = 0.0f;
      }
    }
  }
  if (o.norm) {
    const bool distinct = ppr >= 8 || w < ppr;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float ss = 0.0f;
      if (distinct) {
#pragma unroll
        for (int t = 0; t < MM; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += xf[t][b][e] * xf[t][b][e];
      }
      ss = wave_sum(ss);
      if (lane == 0) g_scr[w * B + b] = ss;
    }
    if (!cbar(A, gen)) return false;
    float rstd[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float tot = 0.0f;
      for (int j = 0; j < NC; ++j) tot += g_scr[j * B + b];
      rstd[b] = 1.0f / sqrtf(tot / (float)K + A.rms_eps);
    }
    const uint16_t* gm = (const uint16_t*)o.gamma;
#pragma unroll
    for (int t = 0; t < MM; ++t) {
      const u32 kp = ppr >= 8 ? w + 8 * t : w % ppr;
      const u32 k0 = kp * PIECE_ELEMS + lane * 8;
      if ((u32)t < M && kp < ppr && k0 < K) {
        const u32x4 gv = *(const u32x4*)(gm + k0);
        const float g[8] = {bflo(gv.x), bfhi(gv.x), bflo(gv.y), bfhi(gv.y),
                            bflo(gv.z), bfhi(gv.z), bflo(gv.w), bfhi(gv.w)};
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
          for (int e = 0; e < 8; ++e) xf[t][b][e] *= rstd[b] * g[e];
      }
    }
  }

  // stream the tile: wave w takes piece w of every slot
  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;
  for (u32 s = 0; s < o.nslots; ++s, ++seq) {
    if (!wait_full(A, seq)) return false;
    const u32 p = s * SLOT_PIECES + w;
    const u32 rl = p / ppr, kp = p - rl * ppr;
    const u32 t = ppr >= 8 ? kp / 8 : 0;
    if (rl < nrt && kp * PIECE_ELEMS < K && kp * PIECE_ELEMS + lane * 8 < K) {
      const u32x4 wv = g_ring[(seq % NSLOT) * (SLOT / 16) + w * 64 + lane];
      const float wf[8] = {bflo(wv.x), bfhi(wv.x), bflo(wv.y), bfhi(wv.y),
                           bflo(wv.z), bfhi(wv.z), bflo(wv.w), bfhi(wv.w)};
#pragma unroll
      for (int tt = 0; tt < MM; ++tt) {
        if ((u32)tt == t) {
#pragma unroll
          for (int b = 0; b < B; ++b)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[b] += wf[e] * xf[tt][b][e];
        }
      }
    }
    release_slot(seq, 1);
    const bool row_end = ppr >= 8 ? (s % M == M - 1) : true;
    if (row_end) {
      const u32 j = ppr >= 8 ? w : kp;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float r = wave_sum(acc[b]);
        if (lane == 0 && rl < nrt) g_red[(rl * RW + j) * B + b] = r;
        acc[b] = 0.0f;
      }
    }
  }
  if (!cbar(A, gen)) return false;

  // epilogue: one output row per compute thread
  for (u32 r = w * 64 + lane; r < o.nrows; r += NC * 64) {
    const u32 row = o.row0 + r;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = 0.0f;
      for (u32 j = 0; j < RW; ++j) v += g_red[(r * RW + j) * B + b];
      if (o.epi == EPI_SWIGLU) {
        float u = 0.0f;
        for (u32 j = 0; j < RW; ++j) u += g_red[((r + o.nrows) * RW + j) * B + b];
        st_sc1((float*)o.out + (size_t)b * o.ld_out + row, silu(v) * u);
      } else if (o.epi == EPI_RESID) {
        const float x = ld_sc1((const float*)o.res + (size_t)b * o.ld_out + row);
        st_sc1((float*)o.out + (size_t)b * o.ld_out + row, x + v);
      } else if (o.epi == EPI_STORE) {
        st_sc1((float*)o.out + (size_t)b * o.ld_out + row, v);
      } else if (b < A.batch) {  // EPI_LOGITS
        const bool ok = ld_i32_sc1(A.row_ok + b) != 0;
        A.logits[(size_t)b * A.V + row] = ok ? v : __builtin_nanf("");
      }
    }
  }
  return true;
}

// ------------------------------------------------------------------ ATTENTION (split-KV + merge)
// One item = (sequence b, KV head, position chunk).  The G query heads sharing the KV head are
// processed together; each compute wave runs an online softmax over its ring slots, the waves are
// merged in LDS, the chunk's (m, l, o) partial goes to global memory, and the last chunk of (b, kvh)
// to finish (a ticket) merges all chunks with the log-sum-exp rule.
template <int D>
__device__ bool op_attn(const KArgs& A, const Op& o, u32 w, u32& seq, u32& gen) {
  constexpr int DPL = D / 64;        // dims per lane
  constexpr int PPS = 4096 / (2 * D);
  constexpr int GMAX = 512 / D;
  const u32 lane = lane_id();
  const AttnItem it = attn_item(A, o.row0, PPS);
  if (!it.valid) return true;
  const u32 ns = (u32)((it.p1 - it.p0 + PPS - 1) / PPS);
  const LayerDesc Ld = sload(A.layers + o.layer);
  const int G = A.G, b = it.b, kvh = it.kvh;
  const int pos = A.positions[b];
  const bool ok = row_ok_local(A, b);
  const int qkv_ld = (A.Hq + 2 * A.Hkv) * D;
  const float* qkv = (const float*)Ld.qkv + (size_t)b * qkv_ld;
  const float scale = 1.0f / sqrtf((float)D);
  const int posc = (pos >= 0 && pos < A.max_ctx) ? pos : 0;
  const float* rope = A.rope + (size_t)posc * (D / 2) * 2;

  // rotary embedding of a head held as dims [lane*DPL, lane*DPL + DPL): partner lane ^ 32
  auto rotate = [&](float* v) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const int i = (int)lane * DPL + e, j = i % (D / 2);
      const float c = rope[2 * j], s = rope[2 * j + 1];
      const float other = __shfl_xor(v[e], 32, 64);
      v[e] = i < D / 2 ? v[e] * c - other * s : v[e] * c + other * s;
    }
  };
  auto headnorm = [&](float* v, const uint16_t* gain) {
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) ss += v[e] * v[e];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + A.rms_eps);
#pragma unroll
    for (int e = 0; e < DPL; ++e) v[e] *= r * bf2f(gain[lane * DPL + e]);
  };

  float qv[GMAX][DPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
      const int h = kvh * G + g;
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[g][e] = ld_sc1(qkv + h * D + lane * DPL + e);
      if (A.qk_norm) headnorm(qv[g], (const uint16_t*)Ld.q_norm);
      rotate(qv[g]);
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[g][e] *= scale;
    }
  }
  const bool has_new = pos >= it.p0 && pos < it.p1;
  float kn[DPL], vn[DPL];
  if (has_new) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      kn[e] = ld_sc1(qkv + (A.Hq + kvh) * D + lane * DPL + e);
      vn[e] = ld_sc1(qkv + (A.Hq + A.Hkv + kvh) * D + lane * DPL + e);
    }
    if (A.qk_norm) headnorm(kn, (const uint16_t*)Ld.k_norm);
    rotate(kn);
    uint16_t kb[DPL], vb[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {  // the cache holds bf16: attend to the rounded values
      kb[e] = f2bf(kn[e]); vb[e] = f2bf(vn[e]);
      kn[e] = bf2f(kb[e]); vn[e] = bf2f(vb[e]);
    }
    if (ok && w == 0) {
      const int pg = A.page_table[(size_t)b * A.max_pages_per_seq + pos / A.page_size];
      const size_t off = (((size_t)pg * A.Hkv + kvh) * A.page_size + pos % A.page_size) * D + lane * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        ((uint16_t*)Ld.k_pages)[off + e] = kb[e];
        ((uint16_t*)Ld.v_pages)[off + e] = vb[e];
      }
    }
  }

  float m[GMAX], l[GMAX], ov[GMAX][DPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY; l[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) ov[g][e] = 0.0f;
  }
  for (u32 s = 0; s < ns; ++s, ++seq) {
    if (s % NC != w) continue;
    if (!wait_full(A, seq)) return false;
    const uint16_t* kr = (const uint16_t*)(g_ring + (seq % NSLOT) * (SLOT / 16));
    const uint16_t* vr = kr + 2048;  // V half of the slot (4 KB)
    const int pbase = it.p0 + (int)s * PPS;
    const int np = min(PPS, it.p1 - pbase);
    for (int pp = 0; pp < np; ++pp) {
      float k[DPL], v[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        k[e] = bf2f(kr[pp * D + lane * DPL + e]);
        v[e] = bf2f(vr[pp * D + lane * DPL + e]);
      }
      if (pbase + pp == pos) {  // the new token: its K/V are not in the cache the loader read
#pragma unroll
        for (int e = 0; e < DPL; ++e) { k[e] = kn[e]; v[e] = vn[e]; }
      }
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g < G) {
          float part = 0.0f;
#pragma unroll
          for (int e = 0; e < DPL; ++e) part += qv[g][e] * k[e];
          const float sc = wave_sum(part);
          const float mn = fmaxf(m[g], sc);
          const float corr = __expf(m[g] - mn), pr = __expf(sc - mn);
          l[g] = l[g] * corr + pr;
#pragma unroll
          for (int e = 0; e < DPL; ++e) ov[g][e] = ov[g][e] * corr + pr * v[e];
          m[g] = mn;
        }
      }
    }
    release_slot(seq, NC);
  }
  // merge the waves of this workgroup
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
      if (lane == 0) { g_scr[(w * GMAX + g) * 2] = m[g]; g_scr[(w * GMAX + g) * 2 + 1] = l[g]; }
#pragma unroll
      for (int e = 0; e < DPL; ++e) g_red[(w * GMAX + g) * D + lane * DPL + e] = ov[g][e];
    }
  }
  if (!cbar(A, gen)) return false;
  float* part = (float*)Ld.part + (size_t)o.row0 * GMAX * (D + 2);
  for (int t = (int)(w * 64 + lane); t < G * D; t += NC * 64) {
    const int g = t / D, dim = t % D;
    float M = -INFINITY;
    for (int j = 0; j < NC; ++j) M = fmaxf(M, g_scr[(j * GMAX + g) * 2]);
    float Ls = 0.0f, Os = 0.0f;
    for (int j = 0; j < NC; ++j) {
      const float mj = g_scr[(j * GMAX + g) * 2];
      const float f = mj == -INFINITY ? 0.0f : __expf(mj - M);
      Ls += f * g_scr[(j * GMAX + g) * 2 + 1];
      Os += f * g_red[(j * GMAX + g) * D + dim];
    }
    st_sc1(part + g * (D + 2) + 2 + dim, Os);
    if (dim == 0) { st_sc1(part + g * (D + 2), M); st_sc1(part + g * (D + 2) + 1, Ls); }
  }
  __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));
  if (!cbar(A, gen)) return false;
  u32* ticket = (u32*)Ld.tickets + (size_t)b * A.Hkv + kvh;
  if (w == 0 && lane == 0) {
    const u32 prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g_bcast[0] = (prev == (u32)it.n_b - 1) ? 1u : 0u;
  }
  if (!cbar(A, gen)) return false;
  if (g_bcast[0]) {  // last chunk of (b, kvh): log-sum-exp merge of all its chunks
    for (int t = (int)(w * 64 + lane); t < G * D; t += NC * 64) {
      const int g = t / D, dim = t % D;
      float M = -INFINITY;
      for (int c = 0; c < it.n_b; ++c) {
        const float* pc = (const float*)Ld.part + (size_t)(it.first_item + c * A.Hkv) * GMAX * (D + 2) + g * (D + 2);
        M = fmaxf(M, ld_sc1(pc));
      }
      float den = 0.0f, num = 0.0f;
      for (int c = 0; c < it.n_b; ++c) {
        const float* pc = (const float*)Ld.part + (size_t)(it.first_item + c * A.Hkv) * GMAX * (D + 2) + g * (D + 2);
        const float f = __expf(ld_sc1(pc) - M);
        den += f * ld_sc1(pc + 1);
        num += f * ld_sc1(pc + 2 + dim);
      }
      st_sc1((float*)Ld.mix_o + (size_t)b * A.mix + (kvh * G + g) * D + dim, num / den);
    }
    if (w == 0 && lane == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

// ------------------------------------------------------------------ GATED DELTA RULE
// One item = (sequence b, head h, block of 32 value columns).  S^T rows of the block stream through
// the ring; q and k go through the causal conv (rolling state), SiLU and L2 norm; then per value
// column j: kS_j = S[:, j] . k, S'[:, j] = g S[:, j] + beta k (v_j - kS_j), o_j = S'[:, j] . q.
// The q / k conv state is shared by the blocks of (b, h): the last block to finish writes it.
template <int DK>
__device__ bool op_delta(const KArgs& A, const Op& o, u32 w, u32& seq, u32& gen) {
  constexpr int DPL = DK / 64;
  constexpr int RPS = SLOT / (DK * 4);  // S^T rows per slot
  constexpr int NSL = 32 / RPS;
  const u32 lane = lane_id();
  const u32 ncb = (u32)A.dv / 32, cb = o.row0 % ncb, bh = o.row0 / ncb;
  const int b = (int)(bh / (u32)A.nh), h = (int)(bh % (u32)A.nh);
  const LayerDesc Ld = sload(A.layers + o.layer);
  const bool ok = row_ok_local(A, b);
  const int C = A.C, W = A.convw;
  const int ldu = C + 2 * A.nh;
  const float* u = (const float*)Ld.qkv + (size_t)b * ldu;
  const float* gts = (const float*)Ld.gates + (size_t)b * ldu;
  float* cst = (float*)Ld.conv_state + (size_t)b * C * (W - 1);
  const uint16_t* cw = (const uint16_t*)Ld.conv_w;

  auto conv = [&](int c, float* newstate_last) -> float {  // causal conv of channel c with its window
    float acc = 0.0f;
    for (int j = 0; j < W - 1; ++j) acc += bf2f(cw[(size_t)c * W + j]) * cst[(size_t)c * (W - 1) + j];
    const float x = ld_sc1(u + c);
    acc += bf2f(cw[(size_t)c * W + W - 1]) * x;
    *newstate_last = x;
    return silu(acc);
  };

  for (u32 s = 0; s < (u32)NSL; ++s, ++seq) {
    if (s % NC != w) continue;
    if (!wait_full(A, seq)) return false;
    float q[DPL], k[DPL], xq[DPL], xk[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const int i = (int)lane * DPL + e;
      q[e] = conv(h * DK + i, &xq[e]);
      k[e] = conv(A.nh * DK + h * DK + i, &xk[e]);
    }
    float nq = 0.0f, nk = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) { nq += q[e] * q[e]; nk += k[e] * k[e]; }
    nq = wave_sum(nq); nk = wave_sum(nk);
    const float sq = 1.0f / sqrtf(nq + 1e-6f) / sqrtf((float)DK), sk = 1.0f / sqrtf(nk + 1e-6f);
#pragma unroll
    for (int e = 0; e < DPL; ++e) { q[e] *= sq; k[e] *= sk; }
    const float gate = 1.0f / (1.0f + __expf(-ld_sc1(gts + h)));
    const float beta = 1.0f / (1.0f + __expf(-ld_sc1(gts + A.nh + h)));
    // value channels of this slot's rows: lane r < RPS computes row r's conv
    const int j0 = (int)cb * 32 + (int)s * RPS;
    const int vch = 2 * A.nh * DK + h * A.dv + j0 + (int)lane;
    float vx = 0.0f, vval = 0.0f;
    if ((int)lane < RPS) vval = conv(vch, &vx);
    const float* srows = (const float*)(g_ring + (seq % NSLOT) * (SLOT / 16));
    float* sdst = (float*)Ld.delta_state + (((size_t)bh * A.dv + j0) * DK);
    for (int r = 0; r < RPS; ++r) {
      float sv[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) sv[e] = srows[r * DK + lane * DPL + e];
      float kS = 0.0f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) kS += sv[e] * k[e];
      kS = wave_sum(kS);
      const float vj = __shfl(vval, r, 64);
      const float err = vj - kS;
      float oj = 0.0f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        sv[e] = gate * sv[e] + beta * k[e] * err;
        oj += sv[e] * q[e];
      }
      oj = wave_sum(oj);
      if (ok) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) sdst[(size_t)r * DK + lane * DPL + e] = sv[e];
        if (lane == 0) st_sc1((float*)Ld.mix_o + (size_t)b * A.mix + h * A.dv + j0 + r, oj);
      }
    }
    // rolling conv state of this slot's value channels
    if (ok && (int)lane < RPS) {
      float* st = cst + (size_t)vch * (W - 1);
      for (int j = 0; j + 1 < W - 1; ++j) st[j] = st[j + 1];
      st[W - 2] = vx;
    }
    (void)xq; (void)xk;
    release_slot(seq, NC);
  }
  // q / k conv states: written once all blocks of (b, h) have read them (ticket)
  __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));
  if (!cbar(A, gen)) return false;
  u32* ticket = (u32*)Ld.tickets + bh;
  if (w == 0 && lane == 0) {
    const u32 prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g_bcast[0] = (prev == ncb - 1) ? 1u : 0u;
  }
  if (!cbar(A, gen)) return false;
  if (g_bcast[0]) {
    if (ok) {
      for (int t = (int)(w * 64 + lane); t < 2 * DK; t += NC * 64) {
        const int c = t < DK ? h * DK + t : A.nh * DK + h * DK + (t - DK);
        const float x = ld_sc1(u + c);
        float* st = cst + (size_t)c * (W - 1);
        for (int j = 0; j + 1 < W - 1; ++j) st[j] = st[j + 1];
        st[W - 2] = x;
      }
    }
    if (w == 0 && lane == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return true;
}

// ------------------------------------------------------------------ compute waves
template <int B>
__device__ void compute(const KArgs& A, u32 q0, u32 q1, u32 w) {
  u32 seq = 0, gen = 0;
  for (u32 oi = q0; oi < q1; ++oi) {
    const Op o = sload(A.ops + oi);
    if (w == 0 && o.wait_stage != NO_STAGE) wait_stage(A, o.wait_stage);
    if (!cbar(A, gen)) return;
    bool alive = true;
    switch (o.opcode) {
      case OP_EMBED:
        op_embed(A, w);
        if (!cbar(A, gen)) return;
        op_embed_finish(A, w, gen);
        break;
      case OP_GEMV: alive = op_gemv<B>(A, o, w, seq, gen); break;
      case OP_ATTN: alive = A.d == 128 ? op_attn<128>(A, o, w, seq, gen) : op_attn<64>(A, o, w, seq, gen); break;
      case OP_DELTA: alive = A.dk == 128 ? op_delta<128>(A, o, w, seq, gen) : op_delta<64>(A, o, w, seq, gen); break;
      default: break;
    }
    if (!alive || aborted()) return;
    __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));  // this wave's outputs are complete
    if (!cbar(A, gen)) return;
    if (w == 0 && lane_id() == 0 && o.sig_stage != NO_STAGE) signal_stage(A, o.sig_stage, o.sig_index);
  }
}

template <int B>
__device__ void megakernel_body(const KArgs& A) {
  const u32 wv = threadIdx.x >> 6;
  if (threadIdx.x < NSLOT) { g_full[threadIdx.x] = 0; g_done[threadIdx.x] = 0; }
  if (threadIdx.x == 0) { g_bar = 0; g_abort = 0; }
  __syncthreads();
  const u32 q0 = A.queue_off[blockIdx.x], q1 = A.queue_off[blockIdx.x + 1];
  if (wv == 0) loader(A, q0, q1);
  else compute<B>(A, q0, q1, wv - 1);
}

}  // namespace mk

extern "C" __global__ void __launch_bounds__(mk::NTHREADS, 1) mk_megakernel_b1(mk::KArgs A) { mk::megakernel_body<1>(A); }
extern "C" __global__ void __launch_bounds__(mk::NTHREADS, 1) mk_megakernel_b2(mk::KArgs A) { mk::megakernel_body<2>(A); }
extern "C" __global__ void __launch_bounds__(mk::NTHREADS, 1) mk_megakernel_b4(mk::KArgs A) { mk::megakernel_body<4>(A); }
extern "C" __global__ void __launch_bounds__(mk::NTHREADS, 1) mk_megakernel_b8(mk::KArgs A) { mk::megakernel_body<8>(A); }
