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
typedef uint16_t __attribute__((may_alias)) u16_alias;  // partial writes into float / vector LDS areas
typedef u32 __attribute__((may_alias)) u32_alias;
typedef u32x4 __attribute__((may_alias)) u32x4_alias;
typedef __attribute__((ext_vector_type(2))) u32 u32x2;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14])
#define MK_VMCNT(n) ((((n) & 0xF) | (((n) >> 4) << 14)) | 0x70 | 0xF00)
#define MK_LGKMCNT0 (0xF | 0x70 | (0x3 << 14))

// Per-op timing stamps are compiled into a second set of kernels only (built from a translation
// unit that defines MK_TRACE_STAMPS=1), so the untraced kernels carry no trace code at all.
#ifndef MK_TRACE_STAMPS
#define MK_TRACE_STAMPS 0
#endif

constexpr int AUX_NT = 2;    // cache policy: non-temporal (streamed once)
constexpr int AUX_SC1 = 16;  // cache policy: agent-scope coherent

// ------------------------------------------------------------------ LDS
// The ring is its own object so the compiler's LDS-DMA tracking never makes
// ordinary LDS accesses of the loader wait for outstanding DMA.
__shared__ __attribute__((aligned(16))) u32x4 g_ring[NSLOT * SLOT / 16];
__shared__ __attribute__((aligned(16))) float g_red[RED_FLOATS];
__shared__ __attribute__((aligned(16))) float g_scr[SCRATCH_FLOATS];
// Ring protocol: slots are numbered by a per-launch sequence number (slot seq lives in ring
// position seq % NSLOT).  The loader publishes g_filled = the number of slots whose bytes have
// landed; compute wave w publishes g_consumed[w] = the sequence number below which it will read
// no slot again.  The loader may fill slot seq once seq < min_w g_consumed[w] + NSLOT.
__shared__ u32 g_filled;
__shared__ __attribute__((aligned(16))) u32 g_consumed[NC];
__shared__ u32 g_bar;           // compute-wave barrier counter
__shared__ u32 g_abort;         // set on watchdog expiry: every wave leaves
__shared__ u32 g_bcast[4];
#if MK_TRACE_STAMPS
__shared__ u32 g_trace_oi;  // queue index of the running op (written and read by compute wave 0 only)
#endif

// ------------------------------------------------------------------ helpers
// An opaque copy of a uniform value in its own scalar register(s).
template <typename T>
__device__ __forceinline__ T opq(T v) {
  asm volatile("" : "+s"(v));
  return v;
}

// The launch arguments, read through an opaque pointer to the kernel-argument segment: loads
// through it cannot be hoisted past the point where it is taken, so a value is re-read (a cached
// scalar load) in each op that needs it instead of being held -- and spilled -- for the whole
// launch.  The arguments are the kernel's only parameter, at offset 0.
__device__ __forceinline__ const KArgs& kargs() {
  const __attribute__((address_space(4))) KArgs* p =
      (const __attribute__((address_space(4))) KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const KArgs*)p;
}

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
// i.e. global loads / stores with the sc1 cache-policy bit, with per-lane addresses.  The pointers
// are cast to the global address space first: through a generic pointer they become FLAT
// accesses, which also count against the LDS counter (every LDS wait then waits for them too).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gptr(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}
__device__ __forceinline__ float ld_sc1(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load(gptr((const u32*)p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_sc1(float* p, float v) {
  __hip_atomic_store(gptr((u32*)p), __builtin_bit_cast(u32, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <int N>  // N consecutive floats (N even), 8-B aligned
__device__ __forceinline__ void ldn_sc1(const float* p, float* out) {
  const auto q = gptr((const uint64_t*)p);
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const uint64_t v = __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    out[2 * i] = __builtin_bit_cast(float, (u32)v);
    out[2 * i + 1] = __builtin_bit_cast(float, (u32)(v >> 32));
  }
}
__device__ __forceinline__ void ld8_sc1(const float* p, float* out) { ldn_sc1<8>(p, out); }
__device__ __forceinline__ void ld4_sc1(const float* p, float* out) { ldn_sc1<4>(p, out); }
__device__ __forceinline__ void ld2_sc1(const float* p, float* out) { ldn_sc1<2>(p, out); }
__device__ __forceinline__ u32 ld_u32_sc1(const u32* p) {
  return __hip_atomic_load(gptr(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_i32_sc1(const int32_t* p) {
  return __hip_atomic_load(gptr(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged activations: bit 0 of every fp32 value that EMBED or a projection writes holds the
// launch parity (a relative change of at most 2^-23).  Each value is written once per launch and
// consecutive launches differ in parity, so a value that shows the current parity is this
// launch's: a reader can poll the data itself instead of a completion counter, and the writer
// needs neither a store-completion wait nor a signal.
__device__ __forceinline__ float tagv(float v, u32 par) {
  return __builtin_bit_cast(float, (__builtin_bit_cast(u32, v) & ~1u) | par);
}
__device__ __forceinline__ bool tag_ok(float v, u32 par) { return (__builtin_bit_cast(u32, v) & 1u) == par; }
__device__ __forceinline__ void st_tag(float* p, float v, u32 par) { st_sc1(p, tagv(v, par)); }
template <int N>
__device__ __forceinline__ bool tags_ok(const float* x, u32 par) {
  u32 a = ~0u, o = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    a &= __builtin_bit_cast(u32, x[i]);
    o |= __builtin_bit_cast(u32, x[i]);
  }
  return ((par ? a : o) & 1u) == par;
}

__device__ __forceinline__ float bf2f(uint16_t h) { return __builtin_bit_cast(float, (u32)h << 16); }
__device__ __forceinline__ float bflo(u32 w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bfhi(u32 w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even (finite inputs)
  u32 u = __builtin_bit_cast(u32, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// x = hi + lo with both halves bf16 (hi rounded to nearest even by the hardware conversion, lo the
// rounded remainder: hi + lo carries about 16 significant bits of x)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_bf16x8(const float* x, u32x4& hi, u32x4& lo) {
  u32 h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x2 v = {x[2 * e], x[2 * e + 1]};
    const bf16x2 vh = __builtin_convertvector(v, bf16x2);
    const bf16x2 vl = __builtin_convertvector(v - __builtin_convertvector(vh, f32x2), bf16x2);
    h[e] = __builtin_bit_cast(u32, vh);
    l[e] = __builtin_bit_cast(u32, vl);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Lane index, recomputed at every use: an opaque instruction pair the compiler cannot hoist, so
// lane-derived addresses are not kept alive across the whole persistent loop (which would crowd
// out the registers the ops need).
__device__ __forceinline__ u32 lane_id() {
  u32 r;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
  return r;
}

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Full-wave sum, returned in every lane: four DPP steps give every lane its 16-lane row sum
// (quad xor 1, quad xor 2, half-row mirror, row mirror), then the four row sums are read out.
__device__ __forceinline__ float wave_sum(float v) {
  v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dppf<0x141>(v);  // row_half_mirror
  v += dppf<0x140>(v);  // row_mirror
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}
// Sums of four values over the whole wave at once: after the call, lane q (q < 4) holds the
// 64-lane sum of v[q].  Butterfly over the quad (xor 1, xor 2) so each lane keeps one value
// index (lane & 3), rotate-add within each 16-lane row, then pair rows with the lane-32 and
// lane-16 swaps.  Fixed order, so bitwise reproducible.
// c + (c of the lane 32 away), and c + (c of the row 16 lanes away), written as the swap
// instruction itself.  The s_nop covers the wait states the swap needs after a VALU write of its
// operands.
__device__ __forceinline__ float add_swap32(float c) {
  float x = c, y = c;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
  return x + y;
}
__device__ __forceinline__ float add_swap16(float c) {
  float x = c, y = c;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
  return x + y;
}
__device__ __forceinline__ float reduce4(float v0, float v1, float v2, float v3) {
  const bool b0 = (threadIdx.x & 1u) != 0, b1 = (threadIdx.x & 2u) != 0;
  const float a = (b0 ? v1 : v0) + dppf<0xB1>(b0 ? v0 : v1);   // pair sums of v[lane & 1]
  const float b = (b0 ? v3 : v2) + dppf<0xB1>(b0 ? v2 : v3);   // pair sums of v[2 + (lane & 1)]
  float c = (b1 ? b : a) + dppf<0x4E>(b1 ? a : b);             // quad sums of v[lane & 3]
  c += dppf<0x124>(c);                                          // row_ror:4
  c += dppf<0x128>(c);                                          // row_ror:8
  return add_swap16(add_swap32(c));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// LDS flags are read by whole waves and every lane sees the same word; readfirstlane tells the
// compiler so, which keeps every spin loop (and everything carried around it) in scalar registers.
__device__ __forceinline__ u32 lds_ld(const u32* p) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
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
// The clock is read only once a wait has actually spun, and then every 64 polls: the fast path
// (condition already true) costs nothing.
struct Watchdog {
  uint64_t t0, limit;
  u32* status;
  u32 polls;
  __device__ explicit Watchdog(const KArgs& A) : t0(0), limit(A.spin_limit), status(A.status), polls(0) {}
  __device__ bool expired() {
    if ((polls++ & 63u) != 0) return false;
    const uint64_t now = __builtin_amdgcn_s_memrealtime();
    if (t0 == 0) { t0 = now; return false; }
    if (now - t0 <= limit) return false;
    // every lane raises the (idempotent) flags: a lane-0 branch here gets merged into the
    // caller's loop exit by the compiler, which turns every spin loop divergent
    __hip_atomic_fetch_or(status, ST_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&g_abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return true;
  }
};

// Barrier among the NC compute waves (the loader never joins).  Returns false on abort.
__device__ __forceinline__ bool cbar(const KArgs& A, u32& gen) {
  __builtin_amdgcn_s_waitcnt(MK_LGKMCNT0);
  gen += NC;
  if (lane_id() == 0) __hip_atomic_fetch_add(&g_bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  Watchdog wd(A);
  while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&g_bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) < gen) {
    if (aborted() || wd.expired()) return false;
    __builtin_amdgcn_s_sleep(0);
  }
  return true;
}

// Wait until ring slot `seq` holds its bytes.  Returns false on abort.
__device__ __forceinline__ bool wait_full(const KArgs& A, u32 seq) {
  Watchdog wd(A);
  while (lds_ld(&g_filled) <= seq) {
    if (aborted() || wd.expired()) return false;
    __builtin_amdgcn_s_sleep(0);
  }
  return true;
}
// Bounded wait for a tagged value: returns `v` once it (or a re-read of `p`) shows this launch's
// parity; past the watchdog limit the timeout is raised and the last value returned.
__device__ __forceinline__ float tagged_fix(const KArgs& A, const float* p, float v) {
  const u32 par = A.tag & 1u;
  if (tag_ok(v, par)) return v;
  Watchdog wd(A);
  do {
    if (aborted() || wd.expired()) break;
    __builtin_amdgcn_s_sleep(1);
    v = ld_sc1(p);
  } while (!tag_ok(v, par));
  return v;
}
__device__ __forceinline__ float ld_tagged(const KArgs& A, const float* p) { return tagged_fix(A, p, ld_sc1(p)); }
// row_ok[b] holds tag << 1 | ok, written once per launch by EMBED: wait for this launch's entry.
__device__ __forceinline__ bool row_ok_wait(const KArgs& A, int b) {
  const u32 want = A.tag & 0x7FFFFFFFu;
  u32 v = (u32)ld_i32_sc1(A.row_ok + b);
  Watchdog wd(A);
  while ((v >> 1) != want) {
    if (aborted() || wd.expired()) return false;
    __builtin_amdgcn_s_sleep(1);
    v = (u32)ld_i32_sc1(A.row_ok + b);
  }
  return (v & 1u) != 0;
}
// The same for an entry loaded earlier (`v`), so that the load overlaps other work.
__device__ __forceinline__ bool row_ok_fix(const KArgs& A, int b, int32_t v) {
  return ((u32)v >> 1) == (A.tag & 0x7FFFFFFFu) ? (v & 1) != 0 : row_ok_wait(A, b);
}

// Traced kernels: stamp "inputs in hand" for the running op (compute wave 0, lane 0 only).
__device__ __forceinline__ void trace_ready(const KArgs& A, u32 w) {
#if MK_TRACE_STAMPS
  if (w == 0 && lane_id() == 0) A.trace[(size_t)g_trace_oi * 4 + 2] = (u32)__builtin_amdgcn_s_memrealtime();
#endif
}

// Compute wave w will read no ring slot below `upto` again.  Monotonic per wave.
__device__ __forceinline__ void release_upto(u32 w, u32 upto) {
  __builtin_amdgcn_s_waitcnt(MK_LGKMCNT0);  // this wave's reads of those slots are complete
  if (lane_id() == 0) __hip_atomic_store(&g_consumed[w], upto, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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

// The launch's attention split, built once per launch by the loader wave before it streams
// anything and read from LDS by every wave.  Each KV head gets at most n_items / Hkv chunks, all
// of one length (a multiple of the positions one ring slot holds; a sequence's last chunk may be
// shorter).  Layout: [0] ready flag, [1 + b] context length of sequence b,
// [9 + b] its chunk length, [17 + b] chunks of the sequences before b (b = 8: all chunks).
constexpr int APLAN_MAXB = 8;
__shared__ int g_aplan[1 + 3 * APLAN_MAXB + 1];

__device__ __forceinline__ void attn_plan_build(const KArgs& A, int pps) {
  int cv[APLAN_MAXB];
  int total = 0, nz = 0;
#pragma unroll
  for (int b = 0; b < APLAN_MAXB; ++b) {
    cv[b] = b < A.batch ? clamp_ctx(A, sload(A.ctx_lens + b)) : 0;
    total += cv[b];
    nz += cv[b] > 0 ? 1 : 0;
  }
  const int K = A.Hkv > 0 ? A.n_items / A.Hkv : 0;  // chunks per KV head; >= batch by construction
  // one chunk length for the launch: the smallest multiple of pps that needs at most K chunks
  // per KV head (binary search; one chunk per sequence always fits since K >= batch)
  int cs_all = 0;
  if (total > 0 && K >= nz) {
    int maxc = 0;
#pragma unroll
    for (int b = 0; b < APLAN_MAXB; ++b) maxc = max(maxc, cv[b]);
    // and at least one ring slot per compute wave: shorter chunks leave waves idle and only add
    // partials for the merger to fold
    int lo = max(((total + K - 1) / K + pps - 1) / pps, (int)NC), hi = (maxc + pps - 1) / pps;
    if (lo > hi) lo = hi;
    while (lo < hi) {
      const int mid = (lo + hi) / 2, c = mid * pps;
      int n = 0;
#pragma unroll
      for (int b = 0; b < APLAN_MAXB; ++b) n += (cv[b] + c - 1) / c;
      if (n <= K) hi = mid;
      else lo = mid + 1;
    }
    cs_all = lo * pps;
  }
  if (lane_id() == 0) {
    int acc = 0;
#pragma unroll
    for (int b = 0; b < APLAN_MAXB; ++b) {
      // the sequence's chunk count at length cs_all, then its chunks evened out at that count
      // (lengths a multiple of pps, at most cs_all; ceil(cv / cs) stays nb), so a ragged batch
      // leaves no short last chunk per sequence
      const int nb = cv[b] > 0 && cs_all > 0 ? (cv[b] + cs_all - 1) / cs_all : 0;
      const int cs = nb > 0 ? ((cv[b] + nb - 1) / nb + pps - 1) / pps * pps : 0;
      g_aplan[1 + b] = cv[b];
      g_aplan[9 + b] = cs;
      g_aplan[17 + b] = acc;
      acc += nb;
    }
    g_aplan[17 + APLAN_MAXB] = acc;
    __hip_atomic_store(&g_aplan[0], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// Item i -> (sequence, KV head, position range), from the launch plan in LDS.  Uniform.
__device__ AttnItem attn_item(const KArgs& A, u32 item, int pps) {
  AttnItem it{0, 0, 0, 0, 0, 0, false};
  (void)pps;
  Watchdog wd(A);
  while (lds_ld((const u32*)&g_aplan[0]) == 0) {
    if (aborted() || wd.expired()) return it;
    __builtin_amdgcn_s_sleep(1);
  }
  const int bc = (int)(item / (u32)A.Hkv), kvh = (int)(item % (u32)A.Hkv);
  for (int b = 0; b < A.batch && b < APLAN_MAXB; ++b) {
    const int c0 = (int)lds_ld((const u32*)&g_aplan[17 + b]), c1 = (int)lds_ld((const u32*)&g_aplan[18 + b]);
    if (bc < c1) {
      const int k = bc - c0, c = (int)lds_ld((const u32*)&g_aplan[1 + b]), cs = (int)lds_ld((const u32*)&g_aplan[9 + b]);
      it.b = b; it.kvh = kvh; it.p0 = k * cs; it.p1 = min(c, (k + 1) * cs);
      it.n_b = c1 - c0; it.first_item = c0 * A.Hkv + kvh; it.valid = true;
      return it;
    }
  }
  return it;
}
// attn_item with a one-entry cache keyed by the item index
struct ItemCache {
  u32 item = 0xFFFFFFFFu;
  AttnItem it{};
  __device__ const AttnItem& get(const KArgs& A, u32 i, int pps) {
    if (i != item) { it = attn_item(A, i, pps); item = i; }
    return it;
  }
  __device__ void restate() {  // see compute(): the fields are uniform
    item = __builtin_amdgcn_readfirstlane(item);
    it.b = __builtin_amdgcn_readfirstlane(it.b);
    it.kvh = __builtin_amdgcn_readfirstlane(it.kvh);
    it.p0 = __builtin_amdgcn_readfirstlane(it.p0);
    it.p1 = __builtin_amdgcn_readfirstlane(it.p1);
    it.n_b = __builtin_amdgcn_readfirstlane(it.n_b);
    it.first_item = __builtin_amdgcn_readfirstlane(it.first_item);
    it.valid = __builtin_amdgcn_readfirstlane((int)it.valid) != 0;
  }
};

__device__ __forceinline__ int attn_pps(int d) { return 4096 / (2 * d); }  // positions per ring slot

// ------------------------------------------------------------------ loader

// Publish "slots below n hold their bytes" (after the matching s_waitcnt vmcnt).  Written as an
// opaque LDS store for the same reason as lds_ld_loader: the compiler would otherwise drain every
// DMA first.  No wait: LDS operations of a wave complete in order.
__device__ __forceinline__ void publish_filled(u32 n) {
  const u32 addr = (u32)(uintptr_t)(__attribute__((address_space(3))) u32*)&g_filled;
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(n) : "memory");
}
// Smallest g_consumed over the compute waves: ring slots below it are free.
__device__ __forceinline__ u32 min_consumed() {
  const u32 addr = (u32)(uintptr_t)(__attribute__((address_space(3))) u32*)&g_consumed[0];
  u32x4 a, b;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(a), "=v"(b) : "v"(addr) : "memory");
  const u32 m = min(min(min(a.x, a.y), min(a.z, a.w)), min(min(b.x, b.y), min(b.z, b.w)));
  return __builtin_amdgcn_readfirstlane(m);
}
static_assert(NC == 8, "min_consumed reads eight counters");

// Wait until the oldest of n in-flight slots has landed (8 DMA instructions per slot).
// n slots in flight (8 DMA instructions each, issued in order): wait until the oldest is complete
__device__ __forceinline__ void wait_oldest(u32 n) {
  switch (n) {
    case 1: __builtin_amdgcn_s_waitcnt(MK_VMCNT(0)); break;
    case 2: __builtin_amdgcn_s_waitcnt(MK_VMCNT(8)); break;
    case 3: __builtin_amdgcn_s_waitcnt(MK_VMCNT(16)); break;
    case 4: __builtin_amdgcn_s_waitcnt(MK_VMCNT(24)); break;
    case 5: __builtin_amdgcn_s_waitcnt(MK_VMCNT(32)); break;
    case 6: __builtin_amdgcn_s_waitcnt(MK_VMCNT(40)); break;
    case 7: __builtin_amdgcn_s_waitcnt(MK_VMCNT(48)); break;
    default: __builtin_amdgcn_s_waitcnt(MK_VMCNT(56)); break;
  }
}
static_assert(LOAD_DEPTH >= 1 && LOAD_DEPTH <= 7, "wait_oldest covers LOAD_DEPTH + 1 in-flight slots (vmcnt <= 63)");

// Every loader address is a uniform (scalar) base plus the lane's fixed 16-byte offset, so a
// DMA costs only scalar work: no per-lane address arithmetic on the issue path.
__device__ __forceinline__ void dma_at(const char* base, u32 lane_off, u32x4* lds) {
  __builtin_amdgcn_global_load_lds(base + lane_off, (__attribute__((address_space(3))) void*)lds, 16, 0, AUX_NT);
}

// GEMV stream: the op's rows in order, each row as ppr (a power of two) pieces of 1 KB.  Slot s
// holds pieces 8s .. 8s+7.  A piece past the row's end or a row past the op is a dummy that
// re-reads the first 1 KB of W (an L2 hit) and is never used; a piece that straddles the row's
// end reads, in its lanes past the end, the row's first bytes instead.
__device__ __forceinline__ uint64_t uni64(uint64_t v) {  // value held in scalar registers
  const u32 lo = __builtin_amdgcn_readfirstlane((u32)v), hi = __builtin_amdgcn_readfirstlane((u32)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// The GEMV stream's two row runs, as scalar values.
struct GemvSeg {
  uint64_t wa, wb;
  u32 na, rowbytes;
};
__device__ __forceinline__ GemvSeg gemv_seg(const Op& o) {
  GemvSeg g;
  g.wa = uni64(o.W);
  g.wb = uni64(o.W2);
  g.na = __builtin_amdgcn_readfirstlane(o.b1);
  g.rowbytes = __builtin_amdgcn_readfirstlane(o.K * 2);
  return g;
}
__device__ __forceinline__ const char* gemv_row(const GemvSeg& g, u32 rl) {
  const bool a = rl < g.na;
  const uint64_t base = a ? g.wa : g.wb;
  const u32 r = a ? rl : rl - g.na;
  return (const char*)(base + (uint64_t)r * g.rowbytes);
}

// Loader-side walk over a GEMV op's slots (layout in the GEMV section below): the current row group
// and the slot within it, advanced once per slot, so the issue path needs no divisions.
// GEMV slot layout (batch <= 4; the compute side is described in the GEMV section).  A slot holds Rs
// row segments of SB = 8 KB / Rs bytes in LDS order: segment j is stream row rho0 + j, inputs
// [kappa0, kappa0 + SB / 2).  With PG >= 8 pieces per row group a slot is one group's R = 16 / P
// rows (Rs = R) at kappa0 = t SB / 2 for its t-th slot; with PG < 8 it holds 8 / PG whole groups
// (Rs = 8 R / PG, kappa0 = 0).  So the loader streams Rs contiguous runs per slot, one M0 value
// each.  Within each 1 KB block of the slot, 16-byte chunk c sits at position gemv_pos(c): the
// compute lanes' operand reads (which stride 64 bytes through a row, and with P = 4 cover two row
// segments per eight lanes) then fall in eight distinct bank groups per eight lanes, while eight
// consecutive DMA lanes still fetch one whole 128-byte line.
__device__ __forceinline__ u32 gemv_lg_rs(u32 P, u32 pg) {  // log2 of the row segments per slot
  const u32 lgR = P == 8 ? 1u : 2u;
  return pg >= 8 ? lgR : lgR + 3 - (u32)__builtin_ctz(pg);
}
__device__ __forceinline__ u32 gemv_pos(u32 c, u32 blk, u32 lgrs) {  // an involution on c
  const u32 par = lgrs <= 3 ? (blk >> (3 - lgrs)) & 1 : 0u;  // parity of the segment holding the block
  return c ^ ((c >> 3) & 3) ^ (par << 1);
}

// Loader-side walk over a GEMV op's slots, advanced once per slot (no divisions on the issue path).
struct GemvWalk {
  u32 s, g, t;          // slot; PG >= 8: row group and its slot
  u32 pg, nf, R, lgrs, nrt, K;
  u32 voff0, voff1;     // this DMA lane's byte offset in a block of an even / odd segment
  bool plain;           // every slot is R whole row segments (PG >= 8, no padding)
  uint64_t grow;        // PG >= 8: address of the current group's first row
};
__device__ __forceinline__ GemvWalk gemv_walk(const Op& o, const GemvSeg& gsg, u32 lane) {
  GemvWalk gw;
  gw.s = gw.g = gw.t = 0;
  gw.pg = o.ppr;
  gw.nf = gw.pg >= 8 ? gw.pg / 8 : 1u;
  gw.R = 16u / o.part;
  gw.lgrs = gemv_lg_rs(o.part, gw.pg);
  gw.nrt = o.epi == EPI_SWIGLU ? 2 * o.nrows : o.nrows;
  gw.K = o.K;
  // DMA lane d fills LDS chunk d of a block with the block's chunk gemv_pos(d)
  gw.voff0 = 16 * (lane ^ ((lane >> 3) & 3));
  gw.voff1 = 16 * (lane ^ ((lane >> 3) & 3) ^ 2u);
  gw.plain = gw.pg >= 8 && gw.lgrs <= 3 && gw.nf * (4096u >> gw.lgrs) == gw.K;
  gw.grow = uni64((uint64_t)gemv_row(gsg, 0));
  return gw;
}
// Rs contiguous segments of BPS KB each: one scalar base per segment, the instruction offset
// stepping both addresses through the segment's blocks.
template <u32 BPS>
__device__ __forceinline__ void dma_segments(const char* base, u32 rowbytes, u32 voff0, u32 voff1, u32x4* dst) {
  constexpr u32 RS = 8 / BPS;
#pragma unroll
  for (u32 j = 0; j < RS; ++j) {
    const char* p = base + (size_t)j * rowbytes + ((j & 1) ? voff1 : voff0);
    auto* l = (__attribute__((address_space(3))) void*)((char*)dst + j * 1024 * BPS);
    __builtin_amdgcn_global_load_lds(p, l, 16, 0, AUX_NT);
    if constexpr (BPS >= 2) __builtin_amdgcn_global_load_lds(p, l, 16, 1024, AUX_NT);
    if constexpr (BPS >= 4) {
      __builtin_amdgcn_global_load_lds(p, l, 16, 2048, AUX_NT);
      __builtin_amdgcn_global_load_lds(p, l, 16, 3072, AUX_NT);
    }
  }
}
// One ring slot of a GEMV op.  Rows past the op and inputs past K (padding of the last group or
// piece) re-read bytes of the op's rows: their products meet zero inputs, and nothing is stored for
// rows past the op.
__device__ __forceinline__ void issue_gemv(const GemvSeg& gsg, GemvWalk& gw, u32 lane, u32x4* dst) {
  if (gw.plain) {  // the common case: R row segments of one group, base advanced per slot
    const char* base = (const char*)gw.grow + gw.t * (8192u >> gw.lgrs);
    if (gw.lgrs == 1) dma_segments<4>(base, gsg.rowbytes, gw.voff0, gw.voff1, dst);
    else dma_segments<2>(base, gsg.rowbytes, gw.voff0, gw.voff1, dst);
    if (++gw.t == gw.nf) {
      gw.t = 0;
      ++gw.g;
      gw.grow = uni64((uint64_t)gemv_row(gsg, gw.g * gw.R));
    }
    ++gw.s;
    return;
  }
  const u32 rho0 = gw.pg >= 8 ? gw.g * gw.R : gw.s << gw.lgrs;
  const u32 rs = 1u << gw.lgrs, half = 4096u >> gw.lgrs;  // segments; inputs per segment
  const u32 kappa0 = gw.pg >= 8 ? gw.t * half : 0u;
  const bool one_run = rho0 + rs <= gsg.na || rho0 >= gsg.na;
  if (gw.lgrs <= 3 && rho0 + rs <= gw.nrt && one_run && kappa0 + half <= gw.K) {  // the common case
    const char* base = gemv_row(gsg, rho0) + 2 * kappa0;
    if (gw.lgrs == 1) dma_segments<4>(base, gsg.rowbytes, gw.voff0, gw.voff1, dst);
    else if (gw.lgrs == 2) dma_segments<2>(base, gsg.rowbytes, gw.voff0, gw.voff1, dst);
    else dma_segments<1>(base, gsg.rowbytes, gw.voff0, gw.voff1, dst);
  } else {
    // per lane: each block's chunk gemv_pos(lane) -> segment, input; clamp rows and inputs
    const u32 sb = 8192u >> gw.lgrs;
#pragma unroll
    for (int blk = 0; blk < SLOT_PIECES; ++blk) {
      const u32 byte = (u32)blk * 1024 + 16 * gemv_pos(lane, blk, gw.lgrs);
      u32 row = rho0 + byte / sb, k = kappa0 + (byte % sb) / 2;
      if (row >= gw.nrt) row = gw.nrt - 1;
      if (k >= gw.K) k = 0;
      __builtin_amdgcn_global_load_lds(gemv_row(gsg, row) + 2 * k, (__attribute__((address_space(3))) void*)(dst + blk * 64), 16, 0, AUX_NT);
    }
  }
  ++gw.s;
  if (gw.pg >= 8 && ++gw.t == gw.nf) {
    gw.t = 0;
    ++gw.g;
  }
}

// Attention stream: slot s = PPS positions of K (pieces 0-3) then the same positions of V (4-7).
// Chunks start on page boundaries and a slot holds one page (d = 128) or two (d = 64), so a slot
// needs at most two page-table entries.  The loader keeps 64 consecutive entries of one sequence
// in a VGPR (one per lane) and refills the window only when a page falls outside it.
//
// K rows are stored swizzled: 16-byte chunk c of row r sits at chunk position c ^ (r mod CPR)
// (CPR = chunks per row), so the 16 rows one matrix-core operand read touches fall in distinct
// LDS banks.  A DMA lane chooses its source address, so the swizzle costs nothing: lane i of
// piece j fills row r = j*RPP + i/CPR, chunk position i mod CPR.
struct PageWindow {
  int b = -1;
  u32 base = 0;
  int v = 0;  // lane i: physical page of logical page base + i
};
__device__ __forceinline__ int page_lookup(const KArgs& A, PageWindow& pw, int b, u32 pi) {
  if (b != pw.b || pi < pw.base || pi >= pw.base + 64) {
    pw.b = b;
    pw.base = pi;
    const u32 lp = pi + lane_id();
    int v = lp < (u32)A.max_pages_per_seq ? A.page_table[(size_t)b * A.max_pages_per_seq + lp] : 0;
    pw.v = (v >= 0 && v < A.num_pages) ? v : 0;  // out-of-range entries stream page 0 (rows get masked)
  }
  return __builtin_amdgcn_readlane(pw.v, (int)(pi - pw.base));
}
struct AttnLanes {  // per-lane byte offsets of each piece within its page's (kv head) block
  u32 koff[4], voff[4];
  u32 kpage[4];     // page of the slot (0 or 1) each piece reads
};
__device__ AttnLanes attn_lanes(u32 d) {
  AttnLanes L;
  const u32 lane = lane_id(), cpr = d / 8, rpp = 64 / cpr, rb = 2 * d;
#pragma unroll
  for (u32 j = 0; j < 4; ++j) {
    const u32 r = j * rpp + lane / cpr, q = lane % cpr;
    L.koff[j] = (r % 16) * rb + ((q ^ (r % cpr)) * 16);
    L.voff[j] = (r % 16) * rb + q * 16;
    L.kpage[j] = r / 16;
  }
  return L;
}
__device__ void issue_attn(const KArgs& A, const LayerDesc& Ld, const AttnItem& it, u32 s, const AttnLanes& L,
                           PageWindow& pw, u32 lane16, u32x4* dst) {
  const u32 d = (u32)A.d, pps = 4096u / (2u * d);
  const size_t page_bytes = (size_t)A.Hkv * 16 * d * 2, head_off = (size_t)it.kvh * 16 * d * 2;
  const u32 pbase = (u32)it.p0 + s * pps, pi0 = pbase / 16;
  const char* kb = (const char*)Ld.k_pages;
  const char* vb = (const char*)Ld.v_pages;
  size_t off[2];
#pragma unroll
  for (u32 k = 0; k < 2; ++k) {
    const bool used = (pi0 + k) * 16 < (u32)it.p1 && (k == 0 || pps > 16);
    off[k] = used ? (size_t)page_lookup(A, pw, it.b, pi0 + k) * page_bytes + head_off : 0;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t o = L.kpage[j] ? off[1] : off[0];
    dma_at(kb + o, L.koff[j], dst + j * 64);
    dma_at(vb + o, L.voff[j], dst + (4 + j) * 64);
  }
  (void)lane16;
}

// Matrix-core GEMV stream: slot s = 16 rows (tile s % nt) x 256 inputs (segment s / nt).  DMA j
// carries input block j (32 inputs) of the 16 rows: lane i fills row i / 4, 16-byte chunk
// position i % 4, which holds chunk (i % 4) ^ ((row / 4) % 4) of the block -- so the 16 rows a
// matrix-core operand read touches fall in distinct LDS banks.  The immediate offset of DMA j
// moves the global address by 64 j; M0 is set 64 j lower so the LDS side lands at 1024 j.
// Rows past the op stream the tile's first row again (bytes that are never stored).
__device__ __forceinline__ void issue_mmv(const GemvSeg& gsg, u32 s, u32 nt, u32 nrows, bool swiglu, u32 lane,
                                          u32x4* dst) {
  const u32 kseg = s / nt, t = s - kseg * nt;
  const u32 lrow = lane >> 2;
  const u32 chunk = (lane & 3) ^ ((lrow >> 2) & 3);
  const u32 half0 = swiglu ? (t & 1) * nrows : 0u;     // stream row of the tile's half
  const u32 trow = swiglu ? 16 * (t >> 1) : 16 * t;    // first row of the tile within its half
  const u32 r = trow + lrow < nrows ? trow + lrow : trow;
  const char* vaddr = gemv_row(gsg, half0 + r) + (size_t)kseg * (MMV_KSEG * 2) + chunk * 16;
  char* lds = (char*)dst;
#define MK_MMV_DMA(j) __builtin_amdgcn_global_load_lds(vaddr, (__attribute__((address_space(3))) void*)(lds + (j) * 960), 16, (j) * 64, AUX_NT)
  MK_MMV_DMA(0); MK_MMV_DMA(1); MK_MMV_DMA(2); MK_MMV_DMA(3);
  MK_MMV_DMA(4); MK_MMV_DMA(5); MK_MMV_DMA(6); MK_MMV_DMA(7);
#undef MK_MMV_DMA
}
static_assert(MMV_KSEG == 256 && SLOT == 16 * MMV_KSEG * 2, "an MMV slot is 16 rows x 256 bf16");

// Delta stream: rows of S^T (fp32) of one column block, contiguous.
__device__ void issue_delta(const KArgs& A, const LayerDesc& Ld, u32 item, u32 s, u32 lane16, u32x4* dst) {
  const u32 ncb = (u32)A.dv / 32, cb = item % ncb, bh = item / ncb;  // bh = b * nh + h
  const u32 rps = SLOT / (A.dk * 4);
  const char* src = (const char*)Ld.delta_state + (((size_t)bh * A.dv + cb * 32 + s * rps) * A.dk) * 4;
#pragma unroll
  for (int i = 0; i < SLOT_PIECES; ++i) dma_at(src + i * PIECE, lane16, dst + i * 64);
}

__device__ u32 op_slots(const KArgs& A, const Op& o, ItemCache& ic) {
  if (o.opcode == OP_ATTN) {
    const int pps = attn_pps(A.d);
    const AttnItem& it = ic.get(A, o.row0, pps);
    return it.valid ? (u32)((it.p1 - it.p0 + pps - 1) / pps) : 0u;
  }
  return o.nslots;
}

__device__ __forceinline__ void loader(const KArgs& A0, u32 q0, u32 q1) {
  const KArgs& A = A0;
  u32 seq = 0, marked = 0, limit = NSLOT;  // slots below `limit` may be filled
  const u32 lane16 = lane_id() * 16;
  attn_plan_build(A, A.d == 64 ? 32 : 16);
  ItemCache ic;
  PageWindow pw;
  const AttnLanes al = attn_lanes(A.d == 64 ? 64u : 128u);
  for (u32 oi = q0; oi < q1; ++oi) {
    const KArgs& A = kargs();
    const Op o = sload(A.ops + oi);
    const u32 ns = op_slots(A, o, ic);
    if (ns == 0) continue;
    LayerDesc Ld{};
    AttnItem it{};
    const GemvSeg gsg = gemv_seg(o);
    GemvWalk gw{};
    if (o.opcode == OP_GEMV) gw = gemv_walk(o, gsg, lane16 >> 4);
    const u32 mmv_nt = (o.epi == EPI_SWIGLU ? 2u : 1u) * ((o.nrows + 15) / 16);
    if (o.opcode == OP_ATTN || o.opcode == OP_DELTA) Ld = sload(A.layers + o.layer);
    if (o.opcode == OP_ATTN) it = ic.get(A, o.row0, attn_pps(A.d));
    for (u32 s = 0; s < ns; ++s) {
      if (seq >= limit) {  // the ring looks full: publish what has landed, then re-read the consumers
        Watchdog wd(A);
        while (true) {
          if (marked < seq) {
            wait_oldest(seq - marked);
            publish_filled(++marked);
          }
          limit = min_consumed() + NSLOT;
          if (seq < limit) break;
          if (marked == seq) {
            if (aborted_loader() || wd.expired()) {
              __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));
              return;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
      }
      u32x4* dst = g_ring + (seq % NSLOT) * (SLOT / 16);
      if (o.opcode == OP_GEMV) issue_gemv(gsg, gw, lane16 >> 4, dst);
      else if (o.opcode == OP_MMV) issue_mmv(gsg, s, mmv_nt, o.nrows, o.epi == EPI_SWIGLU, lane16 >> 4, dst);
      else if (o.opcode == OP_ATTN) issue_attn(A, Ld, it, s, al, pw, lane16, dst);
      else issue_delta(A, Ld, o.row0, s, lane16, dst);
      ++seq;
      if (seq - marked > LOAD_DEPTH) {
        __builtin_amdgcn_s_waitcnt(MK_VMCNT(8 * LOAD_DEPTH));
        publish_filled(++marked);
      }
    }
  }
  while (marked < seq) {
    wait_oldest(seq - marked);
    publish_filled(++marked);
  }
}

// ------------------------------------------------------------------ dependency wait / signal
__device__ __forceinline__ bool wait_stage(const KArgs& A, int stage) {
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

__device__ __forceinline__ void signal_stage(const KArgs& A, int stage, u32 index) {
  u32* c = A.counters + (size_t)stage * NSUB * CTR_STRIDE + (size_t)(index % NSUB) * CTR_STRIDE;
  __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ EMBED
// x0[b][h] = E[token_b][h] for this CU's slice of h, for all B activation rows (rows with
// b >= batch or a bad token are zero), tagged.
template <int B>
__device__ __forceinline__ void op_embed(const KArgs& A, u32 w) {
  const u32 t = w * 64 + lane_id(), par = A.tag & 1u;
  const int cu = (int)blockIdx.x;
  const int h0 = (int)((int64_t)A.H * cu / A.n_cus), h1 = (int)((int64_t)A.H * (cu + 1) / A.n_cus);
  for (int b = 0; b < B; ++b) {
    const int tok = b < A.batch ? A.tokens[b] : -1;
    const bool ok = tok >= 0 && tok < A.V;
    for (int h = h0 + (int)t; h < h1; h += NC * 64)
      st_tag(A.x0 + (size_t)b * A.H + h, ok ? bf2f(A.embed[(size_t)tok * A.H + h]) : 0.0f, par);
  }
}

// Second phase of EMBED, CU 0 only: validate every row (token, context, position, every page of
// [0, ctx) mapped), publish row_ok and raise ST_BAD_INPUT for out-of-contract rows.
__device__ __forceinline__ void op_embed_finish(const KArgs& A, u32 w, u32& gen) {
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
      __hip_atomic_store(A.row_ok + b, (int32_t)((A.tag << 1) | (final_ok ? 1u : 0u)), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (b < A.batch && !final_ok) raise_status(A, ST_BAD_INPUT);
    }
    if (!cbar(A, gen)) return;
  }
}

// ------------------------------------------------------------------ matrix-core and lane helpers
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Lane `l` of a float.  Takes the value by copy: clang's __builtin_bit_cast applied directly to an
// element of an ext_vector (v[i]) reads element 0, so vector elements must never be its operand.
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ float row_max16(float v) {  // max over the 16 lanes of a DPP row
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  return fmaxf(v, dppf<0x140>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  return v + dppf<0x140>(v);
}

// ------------------------------------------------------------------ GEMV (matrix cores, batch <= 4)
// y_b = W x_b for B <= 4 sequences, on the matrix cores although the op is bound by the weight
// stream: the 16x16x32 bf16 tiles take the multiply-adds off the vector ALUs (which are left with
// the ring protocol) and cost the same for every B up to 4.  A tile's A operand is a row group of
// R = 16 / P weight rows, each cut into P parts of 32 inputs (tile row m = r P + p); the B operand
// holds the inputs cut the same way (column n = b P + p, x as bf16 hi + lo halves so that the
// products keep fp32 accuracy).  Only the entries whose parts match belong to W x; each wave sums
// them over p once per row group, after all of the group's pieces are accumulated.
//
// A lane's A and B elements sit at the same inputs: tile row / column block (lane & 15) / P (a
// weight row of the group, or a sequence), inputs q 32 P + 32 ((lane & 15) % P) + 8 (lane >> 4)
// + 0..7 of piece q.  The loader writes each piece in exactly that lane order.
template <int B>
struct GemvWidth { static constexpr int P = B <= 2 ? 8 : 4; };

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ u32 gemv_koff(u32 lane, u32 P) { return 32 * ((lane & 15) & (P - 1)) + 8 * (lane >> 4); }

// Wait until the ring holds slots below `need`; `avail` remembers how far g_filled had got, so a
// batch already covered skips the LDS read.  Returns false on abort.
__device__ __forceinline__ bool wait_avail(const KArgs& A, u32 need, u32& avail) {
  Watchdog wd(A);
  u32 f;
  while ((f = lds_ld(&g_filled)) < need) {
    if (aborted() || wd.expired()) return false;
    __builtin_amdgcn_s_sleep(0);
  }
  avail = f;
  return true;
}

// d[i] for i = lane & 3: the entry of this lane whose tile row and column share their part (P = 4),
// or may share it (P = 8).
__device__ __forceinline__ float gemv_pick(const f32x4 d, u32 lane) {
  const u32 j = lane & 3;
  const float lo = (j & 1) ? d[1] : d[0], hi = (j & 1) ? d[3] : d[2];
  return (j & 2) ? hi : lo;
}

// Sum one row group's matched entries over the parts and store this wave's partials: g_red[(row *
// RW + j) * B + b] for the group's R rows and B sequences.
template <int B, int P>
__device__ __forceinline__ void gemv_extract(const f32x4 d, u32 lane, u32 g, u32 j, u32 RW, u32 nrt) {
  constexpr u32 R = 16 / P;
  float v = gemv_pick(d, lane);
  if constexpr (P == 8) {
    // tile row 4 (lane >> 4) + (lane & 3) is part 4 ((lane >> 4) & 1) + (lane & 3); the column is
    // part lane & 7: they match in the low quad of each 8 lanes in even 16-lane rows and in the
    // high quad in odd rows.  Mirror the odd rows' 8-lane halves so that both sit in the low quad.
    if (((lane >> 2) ^ (lane >> 4)) & 1) v = 0.0f;
    v = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                                              0x141, 0xA, 0xF, false));  // row_half_mirror, odd rows
  }
  v += dppf<0xB1>(v);  // quad sums
  v += dppf<0x4E>(v);
  if constexpr (P == 8) v = add_swap16(v);  // rows 2r and 2r + 1
  // P = 4: lane 16 r + 4 b + q holds (row r, sequence b);  P = 8: lane 32 r + 8 b + q (q < 4)
  const u32 r = P == 4 ? lane >> 4 : lane >> 5, b = P == 4 ? (lane >> 2) & 3 : (lane >> 3) & 1;
  const bool mine = P == 4 ? (lane & 3) == 0 : (lane & 23) == 0;
  const u32 row = g * R + r;
  if (mine && b < (u32)B && row < nrt) g_red[(row * RW + j) * B + b] = v;
}

// Per-row-group accumulation.  Two or more sequences make the projection a (skinny) matrix
// product: each piece is two 16x16x32 tiles on the matrix cores (inputs hi and lo) and the group
// is extracted with gemv_extract.  One sequence makes it a matrix-vector product: each lane takes
// the dot product of its 8 weights with its 8 inputs on the vector ALUs (v_dot2c_f32_bf16 against
// the hi and lo halves), accumulates the group's pieces, and the group's two rows are reduced
// across the wave once (wavefront shuffles).
__device__ __forceinline__ float dot2(u32 wp, u32 xp, float acc) {  // acc + two bf16 products (exact in fp32)
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp), __builtin_bit_cast(bf16x2, xp), acc, false);
}
template <int B, int P>
struct GemvAcc {
  f32x4 h, l;
  __device__ __forceinline__ void init() {
    h = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    l = h;
  }
  __device__ __forceinline__ void add(const u32x4 wv, const bf16x8 xh, const bf16x8 xl) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, wv);
    h = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xh, h, 0, 0, 0);
    l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xl, l, 0, 0, 0);
  }
  __device__ __forceinline__ void merge(const GemvAcc& o) {
    h += o.h;
    l += o.l;
  }
  __device__ __forceinline__ void finish(u32 lane, u32 g, u32 j, u32 RW, u32 nrt) {
    gemv_extract<B, P>(h + l, lane, g, j, RW, nrt);
  }
};
template <>
struct GemvAcc<1, 8> {
  float h, l;
  __device__ __forceinline__ void init() { h = l = 0.0f; }
  __device__ __forceinline__ void add(const u32x4 wv, const bf16x8 xh8, const bf16x8 xl8) {
    const u32x4 xh = __builtin_bit_cast(u32x4, xh8), xl = __builtin_bit_cast(u32x4, xl8);
    h = dot2(wv.x, xh.x, h);
    l = dot2(wv.x, xl.x, l);
    h = dot2(wv.y, xh.y, h);
    l = dot2(wv.y, xl.y, l);
    h = dot2(wv.z, xh.z, h);
    l = dot2(wv.z, xl.z, l);
    h = dot2(wv.w, xh.w, h);
    l = dot2(wv.w, xl.w, l);
  }
  __device__ __forceinline__ void merge(const GemvAcc& o) {
    h += o.h;
    l += o.l;
  }
  // Lane l holds row (l >> 3) & 1 of the group: fold lane bits 0-2 (quad steps and the half-row
  // mirror), 4 and 5 (lane-16 and lane-32 swaps), keeping bit 3 apart; lanes 0 and 8 store.
  __device__ __forceinline__ void finish(u32 lane, u32 g, u32 j, u32 RW, u32 nrt) {
    float v = h + l;
    v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dppf<0x141>(v);  // row_half_mirror: the other quad of the 8 lanes
    v = add_swap32(add_swap16(v));
    const u32 row = 2 * g + ((lane >> 3) & 1);
    if ((lane & ~8u) == 0 && row < nrt) g_red[row * RW + j] = v;
  }
};

// One GEMV op with NF input fragments per wave (1, 2, or up to 8).  Row groups are taken GB at a
// time (GB NF = 4 slots per wait for NF <= 2).  With PG < 8 pieces per group (NF = 1) a slot holds
// 8 / PG groups and wave w works on group (slot 8 / PG + w / PG), piece w % PG.
template <int B, int P, int NF>
__device__ __forceinline__ bool op_gemv_nf(const KArgs& A, const Op& o, u32 w, u32& seq, u32& gen) {
  constexpr u32 R = 16 / P, KP = 32 * P;
  constexpr u32 GB = NF == 1 ? 4 : (NF == 2 ? 2 : 1);
  const u32 lane = lane_id();
  // the Op's fields as independent scalars (see op_mmv)
  const u32 epi = opq((u32)o.epi), norm = opq((u32)o.norm), flags = opq(o.flags), nrows = opq(o.nrows);
  const u32 pg = opq(o.ppr), K = opq(o.K), nslots = opq(o.nslots), row0 = opq(o.row0);
  const u32 ld_in = opq(o.ld_in), ld_out = opq(o.ld_out);
  const uint64_t in = opq(o.in), gamma = opq(o.gamma), outp = opq(o.out), resp = opq(o.res);
  const bool swiglu = epi == EPI_SWIGLU;
  const u32 nrt = swiglu ? 2 * nrows : nrows;  // stream rows
  const u32 nrg = nrt / R;                      // row groups
  const u32 nf = pg >= 8 ? pg / 8 : 1;
  const u32 RW = pg >= 8 ? 8 : pg;
  const u32 bl = (lane & 15) / P;  // this lane's sequence in the B operand
  const u32 koff = gemv_koff(lane, P);
  // this lane's A operand in a slot: row segment seg, inputs piece * KP + koff of it, at the chunk's
  // swizzled position in its 1 KB block
  const u32 lgrs = gemv_lg_rs(P, pg), sb = 8192u >> lgrs;
  const u32 seg = (pg >= 8 ? 0u : (w / pg) * R) + (lane & 15) / P;
  const u32 abyte = seg * sb + 2 * ((pg >= 8 ? w : w % pg) * KP + koff);
  const u32 achunk = (abyte >> 10) * 64 + gemv_pos((abyte & 1023) >> 4, abyte >> 10, lgrs);

  // this wave's input fragments: fragment f is piece 8 f + w of every row group (w % PG if PG < 8).
  // RMSNorm factors out of the sum: the tiles multiply x * gain (input and gain loads share one
  // round trip) and the epilogue scales each output by (mean x^2 + eps)^-1/2, so no barrier stands
  // between the loads and the stream.
  float xf[NF][8];
  u32x4 gv[NF];
  const uint16_t* gm = (const uint16_t*)gamma;
  const float* xin = (const float*)in + (size_t)(B == 1 ? 0u : bl) * ld_in;
  u32 fv = 0;  // fragments this lane loads
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const u32 q = pg >= 8 ? 8 * f + w : w % pg;
    const u32 k0 = q * KP + koff;
    const bool v = (u32)f < nf && (B == 1 || bl < (u32)B) && k0 < K;
    fv |= v ? 1u << f : 0u;
    if (v) ld8_sc1(xin + k0, xf[f]);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[f][e] = 0.0f;
    }
    gv[f] = v && norm ? *(const __attribute__((address_space(1))) u32x4*)(gm + k0) : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  }
  // residual rows of this thread (epilogue row r = thread index), fetched now, off the critical path
  const u32 tid = w * 64 + lane, par = A.tag & 1u;
  float rv[B];
#pragma unroll
  for (int b = 0; b < B; ++b)
    rv[b] = epi == EPI_RESID && tid < nrows ? ld_sc1((const float*)resp + (size_t)b * ld_out + row0 + tid)
          : epi == EPI_LOGITS ? __builtin_bit_cast(float, ld_i32_sc1(A.row_ok + b)) : 0.0f;  // row_ok for logits
  if (flags & OPF_TAGGED_IN) {
    // poll the inputs themselves: re-read every fragment that does not yet show this launch's parity
    if (flags & OPF_LIVE_ROWS) {  // rows of sequences not live this launch may be unwritten: skip them
      const int bb = B == 1 ? 0 : (int)min(bl, (u32)B - 1);
      if (!(bb < A.batch && clamp_ctx(A, A.ctx_lens[bb]) > 0)) fv = 0;
    }
    u32 todo = 0;
#pragma unroll
    for (int f = 0; f < NF; ++f) todo |= ((fv >> f) & 1u) && !tags_ok<8>(xf[f], par) ? 1u << f : 0u;
    Watchdog wd(A);
    while (__builtin_amdgcn_ballot_w64(todo != 0) != 0) {
      if (aborted() || wd.expired()) return false;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const u32 q = pg >= 8 ? 8 * f + w : w % pg;
        if ((todo >> f) & 1u) ld8_sc1(xin + q * KP + koff, xf[f]);
      }
      todo = 0;
#pragma unroll
      for (int f = 0; f < NF; ++f) todo |= ((fv >> f) & 1u) && !tags_ok<8>(xf[f], par) ? 1u << f : 0u;
    }
  }
  trace_ready(A, w);
  if (norm) {
    // sum of squares per sequence (each input appears once among the waves with distinct pieces),
    // read back in the epilogue
    float ss = 0.0f;
    if ((pg >= 8 || w < pg) && (B > 1 || bl == 0)) {  // (at B = 1 the row-1 lanes repeat the row-0 inputs)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += xf[f][e] * xf[f][e];
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float t = wave_sum(bl == (u32)b ? ss : 0.0f);
      if (lane == 0) g_scr[w * B + b] = t;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const u32x4 g4 = gv[f];
      const float g[8] = {bflo(g4.x), bfhi(g4.x), bflo(g4.y), bfhi(g4.y), bflo(g4.z), bfhi(g4.z), bflo(g4.w), bfhi(g4.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) xf[f][e] *= g[e];
    }
  }
  bf16x8 xh[NF], xl[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    u32x4 h, l;
    split_bf16x8(xf[f], h, l);
    xh[f] = __builtin_bit_cast(bf16x8, h);
    xl[f] = __builtin_bit_cast(bf16x8, l);
  }

  u32 avail = seq;
  if (NF > 1 || pg >= 8) {
    // groups in order; a group's nf slots are consecutive and wave w takes piece w of each
    u32 g0 = 0;
    if constexpr (NF <= 2) {
      // whole batches of GB groups (NF = nf here): straight-line code, so the groups' matrix-core
      // chains and extractions interleave
      constexpr u32 NS = GB * NF;
      for (; g0 + GB <= nrg; g0 += GB) {
        if (seq + NS > avail && !wait_avail(A, seq + NS, avail)) return false;
        u32x4 wv[NS];
#pragma unroll
        for (u32 i = 0; i < NS; ++i) wv[i] = g_ring[((seq + i) % NSLOT) * (SLOT / 16) + achunk];
        release_upto(w, seq + NS);
        GemvAcc<B, P> acc[GB];
#pragma unroll
        for (u32 gb = 0; gb < GB; ++gb) acc[gb].init();
#pragma unroll
        for (u32 f = 0; f < NF; ++f)
#pragma unroll
          for (u32 gb = 0; gb < GB; ++gb) acc[gb].add(wv[gb * NF + f], xh[f], xl[f]);
#pragma unroll
        for (u32 gb = 0; gb < GB; ++gb) acc[gb].finish(lane, g0 + gb, w, RW, nrt);
        seq += NS;
      }
    }
    // remaining groups one at a time (every group when NF = 8, with nf <= 8 slots each)
    for (; g0 < nrg; ++g0) {
      if (seq + nf > avail && !wait_avail(A, seq + nf, avail)) return false;
      u32x4 wv[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f)
        if ((u32)f < nf) wv[f] = g_ring[((seq + f) % NSLOT) * (SLOT / 16) + achunk];
      release_upto(w, seq + nf);
      // two accumulators (even / odd fragments) keep four chains in flight
      GemvAcc<B, P> a0, a1;
      a0.init();
      a1.init();
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if ((u32)f < nf) {
          if (f & 1) a1.add(wv[f], xh[f], xl[f]);
          else a0.add(wv[f], xh[f], xl[f]);
        }
      }
      a0.merge(a1);
      a0.finish(lane, g0, w, RW, nrt);
      seq += nf;
    }
  } else {
    // PG < 8: each slot holds 8 / PG groups, one piece of a group per wave
    const u32 lgpg = (u32)__builtin_ctz(pg);
    const u32 gsub = w >> lgpg;          // this wave's group within a slot
    const u32 full = nrg >> (3 - lgpg);  // slots whose groups all exist
    u32 s0 = 0;
    for (; s0 + 4 <= full; s0 += 4) {
      if (seq + 4 > avail && !wait_avail(A, seq + 4, avail)) return false;
      u32x4 wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = g_ring[((seq + i) % NSLOT) * (SLOT / 16) + achunk];
      release_upto(w, seq + 4);
      GemvAcc<B, P> acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i].init();
        acc[i].add(wv[i], xh[0], xl[0]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i].finish(lane, (((s0 + i) * 8) >> lgpg) + gsub, w & (pg - 1), RW, nrt);
      seq += 4;
    }
    for (; s0 < nslots; ++s0) {
      if (seq + 1 > avail && !wait_avail(A, seq + 1, avail)) return false;
      const u32x4 wv = g_ring[(seq % NSLOT) * (SLOT / 16) + achunk];
      release_upto(w, seq + 1);
      const u32 g = ((s0 * 8) >> lgpg) + gsub;
      if (g < nrg) {
        GemvAcc<B, P> acc;
        acc.init();
        acc.add(wv, xh[0], xl[0]);
        acc.finish(lane, g, w & (pg - 1), RW, nrt);
      }
      seq += 1;
    }
  }
  if (!cbar(A, gen)) return false;

  // epilogue: one output row per compute thread
  float rstd[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    rstd[b] = 1.0f;
    if (norm) {
      float tot = 0.0f;
      for (int j = 0; j < NC; ++j) tot += g_scr[j * B + b];
      rstd[b] = 1.0f / sqrtf(tot / (float)K + A.rms_eps);
    }
  }
  bool okb[B];
#pragma unroll
  for (int b = 0; b < B; ++b) okb[b] = epi == EPI_LOGITS && b < A.batch && row_ok_fix(A, b, __builtin_bit_cast(int32_t, rv[b]));
  for (u32 r = tid; r < nrows; r += NC * 64) {
    const u32 row = row0 + r;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = 0.0f;
      for (u32 j = 0; j < RW; ++j) v += g_red[(r * RW + j) * B + b];
      v *= rstd[b];
      if (epi == EPI_SWIGLU) {
        float u = 0.0f;
        for (u32 j = 0; j < RW; ++j) u += g_red[((r + nrows) * RW + j) * B + b];
        st_tag((float*)outp + (size_t)b * ld_out + row, silu(v) * (u * rstd[b]), par);
      } else if (epi == EPI_RESID) {
        const float* rp = (const float*)resp + (size_t)b * ld_out + row;
        const float x = tagged_fix(A, rp, r == tid ? rv[b] : ld_sc1(rp));
        st_tag((float*)outp + (size_t)b * ld_out + row, x + v, par);
      } else if (epi == EPI_STORE) {
        st_tag((float*)outp + (size_t)b * ld_out + row, v, par);
      } else if (b < A.batch) {  // EPI_LOGITS
        A.logits[(size_t)b * A.V + row] = okb[b] ? v : __builtin_nanf("");
      }
    }
  }
  return true;
}

template <int B>
__device__ __forceinline__ bool op_gemv(const KArgs& A, const Op& o, u32 w, u32& seq, u32& gen) {
  constexpr int P = GemvWidth<B>::P;
  const u32 pg = o.ppr;
  if (pg <= 8) return op_gemv_nf<B, P, 1>(A, o, w, seq, gen);
  if (pg == 16) return op_gemv_nf<B, P, 2>(A, o, w, seq, gen);
  return op_gemv_nf<B, P, 8>(A, o, w, seq, gen);
}

// ------------------------------------------------------------------ MATRIX-CORE GEMV (batch 8)
// With eight sequences a projection is a skinny GEMM: each 16-row tile is multiplied on the matrix
// cores (16x16x32 bf16) by the 8 input columns (split into bf16 hi + lo, so the products keep fp32
// accuracy).  Wave w takes input block w of every ring slot (k-outer: all tiles of one 256-input
// segment, then the next segment) and keeps one 16x16 accumulator per tile; the eight waves'
// partial sums are added in LDS, four tiles per pass.  RMSNorm factors out of the sum: the tiles
// multiply x * gain, each lane accumulates x^2 on the side, and the epilogue scales by
// (mean x^2 + eps)^-1/2.
template <int B>
__device__ __forceinline__ bool op_mmv(const KArgs& A, const Op& o, u32 w, u32& seq, u32& gen) {
  static_assert(B <= 8 && NC == 8, "one pass holds 8 waves x 4 tiles x 16 rows x 8 columns");
  static_assert(NC * 4 * 16 * 8 <= RED_FLOATS, "MMV partial-sum area");
  const u32 lane = lane_id();
  // the Op's fields as independent scalars: kept whole, its 8-dword load groups are what the
  // compiler spills and reloads inside the stream loop
  const u32 epi = opq((u32)o.epi), norm = opq((u32)o.norm), nrows = opq(o.nrows), nks = opq(o.ppr), K = opq(o.K);
  const u32 flags = opq(o.flags);
  const u32 row0 = opq(o.row0), ld_in = opq(o.ld_in), ld_out = opq(o.ld_out);
  const uint64_t in = opq(o.in), gamma = opq(o.gamma), outp = opq(o.out), resp = opq(o.res);
  const bool swiglu = epi == EPI_SWIGLU;
  const u32 ntg = (nrows + 15) / 16, nt = swiglu ? 2 * ntg : ntg;
  const u32 col = lane & 15, kq = lane >> 4;  // operand row / output column, and k-chunk of the lane
  const bool cval = col < (u32)B;
  const u32 aoff = w * 1024 + col * 64 + ((kq ^ ((col >> 2) & 3)) * 16);  // this lane's A bytes in a slot
  const float* xin = (const float*)in + (size_t)(cval ? col : 0) * ld_in;
  const uint16_t* gm = (const uint16_t*)gamma;
  const int32_t rok = epi == EPI_LOGITS && lane < (u32)B ? ld_i32_sc1(A.row_ok + lane) : 0;  // lane b: row_ok[b]

  f32x4 acc[MMV_TILES];
#pragma unroll
  for (int t = 0; t < MMV_TILES; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float ssq = 0.0f;

  // this lane's inputs of segment ks: x[col][ks*256 + 32 w + 8 kq .. + 8] and their gains
  auto fetch = [&](u32 ks, float* xv, u32x4& gv) {
    const u32 k0 = ks * MMV_KSEG + w * 32 + kq * 8;
    if (cval && ks < nks) ld8_sc1(xin + k0, xv);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = 0.0f;
    }
    gv = (norm && ks < nks) ? *(const u32x4*)(gm + k0) : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  };
  // tagged inputs: wait until this lane's block of segment ks shows this launch's parity (lanes of
  // sequences that are not live are not checked with OPF_LIVE_ROWS)
  const u32 par = A.tag & 1u;
  const bool tcheck = (flags & OPF_TAGGED_IN) && cval &&
                      (!(flags & OPF_LIVE_ROWS) || ((int)col < A.batch && clamp_ctx(A, A.ctx_lens[col]) > 0));
  auto ready = [&](u32 ks, float* xv) -> bool {
    const bool need = tcheck && ks < nks;
    Watchdog wd(A);
    while (__builtin_amdgcn_ballot_w64(need && !tags_ok<8>(xv, par)) != 0) {
      if (aborted() || wd.expired()) return false;
      __builtin_amdgcn_s_sleep(1);
      if (need && !tags_ok<8>(xv, par)) ld8_sc1(xin + ks * MMV_KSEG + w * 32 + kq * 8, xv);
    }
    return true;
  };
  // one segment: this wave's input block times every tile of the segment (the slots must be full)
  auto consume = [&](const float* xv, const u32x4& gv) {
    const float g[8] = {bflo(gv.x), bfhi(gv.x), bflo(gv.y), bfhi(gv.y), bflo(gv.z), bfhi(gv.z), bflo(gv.w), bfhi(gv.w)};
    float xg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ssq += xv[e] * xv[e];
      xg[e] = xv[e] * g[e];
    }
    u32x4 hi, lo;
    split_bf16x8(xg, hi, lo);
    const bf16x8 bh = __builtin_bit_cast(bf16x8, hi), bl = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
    for (int t = 0; t < MMV_TILES; ++t) {
      if ((u32)t < nt) {
        const char* slot = (const char*)(g_ring + ((seq + t) % NSLOT) * (SLOT / 16));
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(slot + aoff));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[t], 0, 0, 0);
      }
    }
    seq += nt;
  };

  // Segments four at a time, the inputs of each fetched four segments ahead (a segment of a
  // 2-tile op streams in about half a microsecond; an input fetch takes longer).  Thin ops wait
  // for and release several segments at once (gs segments, at most 8 slots), so the ring protocol
  // is paid per 8 slots rather than per segment.
  const u32 gs = nt <= 2 ? 4u : (nt <= 4 ? 2u : 1u);
  float xr[4][8];
  u32x4 gr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) fetch(i, xr[i], gr[i]);
  for (u32 ks = 0; ks < nks; ks += 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ks + i < nks) {
        if ((u32)i % gs == 0 && !wait_full(A, seq + min(gs, nks - (ks + i)) * nt - 1)) return false;
        if ((flags & OPF_TAGGED_IN) && !ready(ks + i, xr[i])) return false;
        consume(xr[i], gr[i]);
        if (((u32)i + 1) % gs == 0 || ks + i + 1 == nks) release_upto(w, seq);
        fetch(ks + i + 4, xr[i], gr[i]);
      }
    }
  }

  // per-column sum of squares: lanes col, col + 16, col + 32, col + 48 of every wave
  const float ss = add_swap32(add_swap16(ssq));
  if (lane < 16) g_scr[w * 16 + lane] = ss;
  const u32 tid = w * 64 + lane;
#pragma unroll
  for (int pp = 0; pp < MMV_TILES / 4; ++pp) {
    if ((u32)(pp * 4) >= nt) break;
    if (!cbar(A, gen)) return false;  // the previous pass's partials are read; g_scr is written
    if (cval) {
#pragma unroll
      for (int tp = 0; tp < 4; ++tp)
#pragma unroll
        for (int i = 0; i < 4; ++i) g_red[((w * 4 + tp) * 16 + kq * 4 + i) * B + col] = acc[pp * 4 + tp][i];
    }
    if (!cbar(A, gen)) return false;
    auto colsum = [&](u32 tp, u32 row, u32 b) {
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < NC; ++ww) v += g_red[((ww * 4 + tp) * 16 + row) * B + b];
      if (norm) {
        float tot = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NC; ++ww) tot += g_scr[ww * 16 + b];
        v *= 1.0f / sqrtf(tot / (float)K + A.rms_eps);
      }
      return v;
    };
    const u32 row = (tid / B) % 16, b = tid % B;
    const int32_t rokb = __shfl(rok, (int)b, 64);  // row_ok[b] (all lanes active here)
    if (swiglu) {
      const u32 pr = tid / (16 * B);  // gate / up tile pair within the pass
      if (pr < 2 && (u32)(pp * 4) + 2 * pr + 1 < nt) {
        const float gv = colsum(2 * pr, row, b), uv = colsum(2 * pr + 1, row, b);
        const u32 orow = 16 * ((u32)(pp * 2) + pr) + row;
        if (orow < nrows) st_tag((float*)outp + (size_t)b * ld_out + row0 + orow, silu(gv) * uv, A.tag & 1u);
      }
    } else {
      const u32 tp = tid / (16 * B);
      if (tp < 4 && (u32)(pp * 4) + tp < nt) {
        const float v = colsum(tp, row, b);
        const u32 orow = 16 * ((u32)(pp * 4) + tp) + row, grow = row0 + orow;
        if (orow < nrows) {
          if (epi == EPI_RESID) {
            const float x = ld_tagged(A, (const float*)resp + (size_t)b * ld_out + grow);
            st_tag((float*)outp + (size_t)b * ld_out + grow, x + v, A.tag & 1u);
          } else if (epi == EPI_STORE) {
            st_tag((float*)outp + (size_t)b * ld_out + grow, v, A.tag & 1u);
          } else if ((int)b < A.batch) {  // EPI_LOGITS
            const bool ok = row_ok_fix(A, (int)b, rokb);
            A.logits[(size_t)b * A.V + grow] = ok ? v : __builtin_nanf("");
          }
        }
      }
    }
  }
  return true;
}

// ------------------------------------------------------------------ ATTENTION (split-KV + merge)
// One item = (sequence b, KV head, position chunk).  The G query heads sharing the KV head are
// processed together.  Scores come from the matrix cores: Q (G heads, split into bf16 hi + lo so
// the product keeps fp32 accuracy) times K^T, 16 positions per 16x16x32 tile.  Each compute wave
// runs an online softmax over its ring slots and accumulates P V on the vector ALUs; the waves are
// merged in LDS, the chunk's (m, l, o) partial goes to global memory (tagged), and the last chunk
// of (b, kvh) in item order merges all chunks with the log-sum-exp rule.
template <int D>
__device__ __forceinline__ bool op_attn(const KArgs& A, const Op& o, u32 w, u32& seq, u32& gen, ItemCache& ic) {
  constexpr int DPL = D / 64;          // dims per lane in the vector layout
  constexpr int PPS = 4096 / (2 * D);  // positions per ring slot
  constexpr int NB = PPS / 16;         // 16-position score tiles per slot
  constexpr int KB = D / 32;           // k-blocks of one score tile
  constexpr int GMAX = 512 / D;
  constexpr int CPR = D / 8;           // 16-byte chunks per K row
  constexpr int RB = 2 * D;            // bytes per K or V row
  constexpr int QF = 768;              // query fragments: [KB][hi, lo][64 lanes] x 16 bytes
  constexpr int PA = QF + KB * 2 * 64 * 4;  // per-wave probabilities: [NC][PPS][GMAX]
  static_assert(PA + NC * PPS * GMAX <= RED_FLOATS, "attention LDS areas");
  const u32 lane = lane_id();
  const AttnItem it = ic.get(A, o.row0, PPS);
  if (!it.valid) return true;
  const u32 ns = (u32)((it.p1 - it.p0 + PPS - 1) / PPS);
  const u32 seq0 = seq;
  seq += ns;
  const LayerDesc Ld = sload(A.layers + o.layer);
  const int G = A.G, b = it.b, kvh = it.kvh;
  const int pos = A.positions[b];
  const int32_t rok = ld_i32_sc1(A.row_ok + b);  // checked where it is used
  const bool tagged = (o.flags & OPF_TAGGED_IN) != 0;
  const int qkv_ld = (A.Hq + 2 * A.Hkv) * D;
  const float* qkv = (const float*)Ld.qkv + (size_t)b * qkv_ld;
  const float scale = 1.0f / sqrtf((float)D);
  const int posc = (pos >= 0 && pos < A.max_ctx) ? pos : 0;
  const float* rope = A.rope + (size_t)posc * (D / 2) * 2;
  float* kvn = g_red + 512;            // [2][D] the new token's rotated K and its V, bf16-rounded

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

  // 1. one task per wave: query heads 0..G-1, then (chunk holding the new token) its K and V.
  //    A query head goes straight into the matrix-core A operand in LDS (row = head, split into
  //    bf16 hi + lo): 16-byte chunk (kb, hi/lo, kc, row) holds dims 32 kb + 8 kc .. + 7.  Rows past
  //    G are zeroed by every wave in the same pass.
  u16_alias* qfh = (u16_alias*)(g_red + QF);
  const bool has_new = pos >= it.p0 && pos < it.p1;
  for (int c = (int)(w * 64 + lane); c < KB * 2 * 4 * 16; c += NC * 64)
    if ((c & 15) >= G) ((u32x4*)(g_red + QF))[c] = u32x4{0u, 0u, 0u, 0u};
  const int ntask = G + (has_new ? 2 : 0);
  for (int t = (int)w; t < ntask; t += NC) {
    const int row = t < G ? kvh * G + t : (t == G ? A.Hq + kvh : A.Hq + A.Hkv + kvh);
    float v[DPL];
    const float* src = qkv + row * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) v[e] = ld_sc1(src + e);
    if (tagged) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[e] = tagged_fix(A, src + e, v[e]);
    }
    if (t <= G) {
      if (A.qk_norm) headnorm(v, (const uint16_t*)(t < G ? Ld.q_norm : Ld.k_norm));
      rotate(v);
    }
    if (t < G) {
      const int i0 = (int)lane * DPL;  // this lane's first dim (DPL consecutive dims, one chunk)
      const int chunk = ((i0 >> 5) * 2) * 64 + ((i0 >> 3) & 3) * 16 + t, j = i0 & 7;
      if constexpr (DPL == 2) {
        const f32x2 x = {v[0] * scale, v[1] * scale};
        const bf16x2 xh = __builtin_convertvector(x, bf16x2);
        const bf16x2 xl = __builtin_convertvector(x - __builtin_convertvector(xh, f32x2), bf16x2);
        *(u32_alias*)(qfh + chunk * 8 + j) = __builtin_bit_cast(u32, xh);
        *(u32_alias*)(qfh + (chunk + 64) * 8 + j) = __builtin_bit_cast(u32, xl);
      } else {
        const f32x2 x = {v[0] * scale, 0.0f};
        const bf16x2 xh = __builtin_convertvector(x, bf16x2);
        const bf16x2 xl = __builtin_convertvector(x - __builtin_convertvector(xh, f32x2), bf16x2);
        qfh[chunk * 8 + j] = (uint16_t)__builtin_bit_cast(u32, xh);
        qfh[(chunk + 64) * 8 + j] = (uint16_t)__builtin_bit_cast(u32, xl);
      }
    } else {
      uint16_t hb[DPL];  // the cache holds bf16: attend to the rounded values
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        hb[e] = f2bf(v[e]);
        kvn[(t - G) * D + lane * DPL + e] = bf2f(hb[e]);
      }
      if (row_ok_fix(A, b, rok)) {
        const int pg = A.page_table[(size_t)b * A.max_pages_per_seq + pos / 16];
        const size_t off = (((size_t)pg * A.Hkv + kvh) * 16 + pos % 16) * D + lane * DPL;
        uint16_t* dp = (uint16_t*)(t == G ? Ld.k_pages : Ld.v_pages) + off;
#pragma unroll
        for (int e = 0; e < DPL; ++e) dp[e] = hb[e];
      }
    }
  }
  if (!cbar(A, gen)) return false;
  trace_ready(A, w);
  const u32x4* qf = (const u32x4*)(g_red + QF);

  // 3. this wave's slots: w, w + NC, ...  Score tile lanes: position p = 16*blk + lane % 16,
  //    heads hr .. hr + 3 with hr = 4 * (lane / 16).
  const int hr = (int)(lane >> 4) * 4;
  float m[4], l[4], ov[GMAX][DPL];
#pragma unroll
  for (int i = 0; i < 4; ++i) { m[i] = -INFINITY; l[i] = 0.0f; }
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int e = 0; e < DPL; ++e) ov[g][e] = 0.0f;
  release_upto(w, seq0 + min(w, ns));  // slots before this wave's first belong to other waves
  for (u32 s = w; s < ns; s += NC) {
    const u32 sq = seq0 + s;
    if (!wait_full(A, sq)) return false;
    char* kslot = (char*)(g_ring + (sq % NSLOT) * (SLOT / 16));
    char* vslot = kslot + 4096;
    const int pbase = it.p0 + (int)s * PPS;
    const int np = min(PPS, it.p1 - pbase);
    if (has_new && pos >= pbase && pos < pbase + PPS) {
      // the new token's K/V are not in the cache the loader read: put them into the slot
      const int r = pos - pbase, d0 = (int)lane * DPL, c = d0 / 8;
      u16_alias* kd = (u16_alias*)(kslot + r * RB + ((c ^ (r % CPR)) * 16)) + (d0 % 8);
      u16_alias* vd = (u16_alias*)(vslot + r * RB) + d0;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        kd[e] = f2bf(kvn[d0 + e]);
        vd[e] = f2bf(kvn[D + d0 + e]);
      }
    }
    f32x4 sc[NB];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      const int p = blk * 16 + (int)(lane & 15);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int c = kb * 4 + (int)(lane >> 4);
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4_alias*)(kslot + p * RB + ((c ^ (p % CPR)) * 16)));
        const bf16x8 qh = __builtin_bit_cast(bf16x8, qf[(kb * 2) * 64 + lane]);
        const bf16x8 ql = __builtin_bit_cast(bf16x8, qf[(kb * 2 + 1) * 64 + lane]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, kf, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, kf, acc, 0, 0, 0);
      }
      sc[blk] = acc;
    }
    float mx[4], corr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const bool live = blk * 16 + (int)(lane & 15) < np;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!live) sc[blk][i] = -INFINITY;
        mx[i] = fmaxf(mx[i], sc[blk][i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mn = fmaxf(m[i], row_max16(mx[i]));
      corr[i] = __expf(m[i] - mn);  // 0 on the first slot (m = -inf)
      float ps = 0.0f;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        sc[blk][i] = __expf(sc[blk][i] - mn);
        ps += sc[blk][i];
      }
      l[i] = l[i] * corr[i] + row_sum16(ps);
      m[i] = mn;
    }
    // P V on the vector ALUs.  Lane owns DPL dims of every head.  The probabilities go through
    // this wave's LDS area as P[p][head] and come back as broadcast reads (every lane reads the
    // same address); the rescale factors are broadcast with readlane.  Heads past G carry finite
    // junk (zero queries) and are never stored.  Rows past the chunk are zeroed so that stale
    // ring bytes cannot reach the sums.
    float* pw = g_red + PA + w * (PPS * GMAX);
    if (hr < GMAX) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) *(f32x4*)(pw + (blk * 16 + (int)(lane & 15)) * GMAX + hr) = sc[blk];
    }
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const float cr = readlane_f(corr[g & 3], (g >> 2) * 16);
#pragma unroll
      for (int e = 0; e < DPL; ++e) ov[g][e] *= cr;
    }
    // four positions at a time: their V words and probabilities in flight together, then the
    // products (a rolled loop: fully unrolled, every load would be hoisted and spilled)
#pragma unroll 1
    for (int p0 = 0; p0 < PPS; p0 += 4) {
      u32 vw[4];
      f32x4 pv[4][GMAX / 4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = p0 + j;
        u32 u;
        if constexpr (DPL == 2) u = *(const u32_alias*)(vslot + p * RB + lane * 4);
        else u = *(const u16_alias*)(vslot + p * RB + lane * 2);
        vw[j] = p < np ? u : 0u;
#pragma unroll
        for (int g4 = 0; g4 < GMAX / 4; ++g4) pv[j][g4] = *(const f32x4*)(pw + p * GMAX + 4 * g4);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float vv[DPL];
        if constexpr (DPL == 2) { vv[0] = bflo(vw[j]); vv[1] = bfhi(vw[j]); }
        else vv[0] = bflo(vw[j]);
#pragma unroll
        for (int g4 = 0; g4 < GMAX / 4; ++g4)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < DPL; ++e) ov[4 * g4 + i][e] += pv[j][g4][i] * vv[e];
      }
    }
    release_upto(w, seq0 + min(s + NC, ns));
  }
  release_upto(w, seq0 + ns);
  if (!cbar(A, gen)) return false;  // every wave is done with the query / new-token areas

  // merge the waves of this workgroup
  if ((lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (hr + i < G) {
        g_scr[(w * GMAX + hr + i) * 2] = m[i];
        g_scr[(w * GMAX + hr + i) * 2 + 1] = l[i];
      }
    }
  }
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) g_red[(w * GMAX + g) * D + lane * DPL + e] = ov[g][e];
    }
  }
  if (!cbar(A, gen)) return false;
  // partial of item i, head g: part[(i * GMAX + g) * (D + 4)] = m, l, -, -, o[0..D) (o 16-B aligned)
  float* part = (float*)Ld.part + (size_t)o.row0 * GMAX * (D + 4);
  const u32 par = A.tag & 1u;
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
    // tagged (M is finite: a chunk holds at least one position, so some wave saw a score)
    st_tag(part + g * (D + 4) + 4 + dim, Os, par);
    if (dim == 0) { st_tag(part + g * (D + 4), M, par); st_tag(part + g * (D + 4) + 1, Ls, par); }
  }
  // The last chunk of (b, kvh) in item order merges all of its chunks with the log-sum-exp rule,
  // polling their tagged partials.  Items go to CUs round-robin in item order, so every chunk it
  // waits for sits at the same or an earlier position in its CU's queue: by induction on the item
  // index every item completes, and no two mergers can wait on each other.
  if (o.row0 != (u32)(it.first_item + (it.n_b - 1) * A.Hkv)) return true;
  if (!cbar(A, gen)) return false;  // every thread is done with the wave partials in LDS
  {
    // Thread t owns output quad t % NQ (head g, 4 dims) of chunks t / NQ, t / NQ + NG, ...: it
    // reads each chunk's (m, l) pair and its quad (MQ chunks per round trip, re-reading together
    // whichever still show the previous launch's parity) and folds them into a running
    // (max, denominator, numerator); the NG chunk groups are then combined in LDS with the same
    // log-sum-exp rule.
    const int tid = (int)(w * 64 + lane), nb = it.n_b;
    const float* part0 = (const float*)Ld.part + (size_t)it.first_item * GMAX * (D + 4);
    const size_t cstride = (size_t)A.Hkv * GMAX * (D + 4);  // floats between chunks of (b, kvh)
    const int NQ = G * D / 4, NG = NC * 64 / NQ;  // output quads; chunk groups
    const int q = tid % NQ, cg = tid / NQ, g = q / (D / 4), d0 = 4 * (q % (D / 4));
    const float* ph = part0 + g * (D + 4);  // this head's row in chunk 0
    float Mt = -INFINITY, den = 0.0f, num[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int MQ = 8;
    for (int c0 = cg; cg < NG && c0 < nb; c0 += MQ * NG) {  // (threads past NG x NQ idle)
      float v[MQ][6];  // m, l, o[4]
#pragma unroll
      for (int k = 0; k < MQ; ++k) {
        const int c = c0 + k * NG;
        if (c < nb) {
          ld4_sc1(ph + (size_t)c * cstride + 4 + d0, v[k] + 2);
          ld2_sc1(ph + (size_t)c * cstride, v[k]);
        } else {
#pragma unroll
          for (int e = 0; e < 6; ++e) v[k][e] = tagv(e == 0 ? -1.0e30f : 0.0f, par);
        }
      }
      Watchdog wd(A);
      while (true) {
        u32 stale = 0;
#pragma unroll
        for (int k = 0; k < MQ; ++k) stale |= tags_ok<6>(v[k], par) ? 0u : 1u << k;
        if (stale == 0 || aborted() || wd.expired()) break;
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int k = 0; k < MQ; ++k)
          if ((stale >> k) & 1u) {
            ld4_sc1(ph + (size_t)(c0 + k * NG) * cstride + 4 + d0, v[k] + 2);
            ld2_sc1(ph + (size_t)(c0 + k * NG) * cstride, v[k]);
          }
      }
      float mr = Mt;
#pragma unroll
      for (int k = 0; k < MQ; ++k) mr = fmaxf(mr, v[k][0]);
      const float sc = Mt == -INFINITY ? 0.0f : __expf(Mt - mr);
      den *= sc;
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] *= sc;
#pragma unroll
      for (int k = 0; k < MQ; ++k) {
        if (c0 + k * NG < nb) {
          const float f = __expf(v[k][0] - mr);
          den += f * v[k][1];
#pragma unroll
          for (int e = 0; e < 4; ++e) num[e] += f * v[k][2 + e];
        }
      }
      Mt = mr;
    }
    // combine the chunk groups: acc[cg][q] = (max, den, num[4]) (a group with no chunk has max -inf)
    float* acc = g_red;
    if (cg < NG) {
      float* a6 = acc + (cg * NQ + q) * 6;
      a6[0] = Mt; a6[1] = den;
#pragma unroll
      for (int e = 0; e < 4; ++e) a6[2 + e] = num[e];
    }
    if (!cbar(A, gen)) return false;
    if (tid < NQ) {
      float M = -INFINITY;
      for (int j = 0; j < NG; ++j) M = fmaxf(M, acc[(j * NQ + q) * 6]);
      float dn = 0.0f, nm[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int j = 0; j < NG; ++j) {
        const float* a6 = acc + (j * NQ + q) * 6;
        const float f = a6[0] == -INFINITY ? 0.0f : __expf(a6[0] - M);
        dn += f * a6[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) nm[e] += f * a6[2 + e];
      }
      float* dst = (float*)Ld.mix_o + (size_t)b * A.mix + (kvh * G + g) * D + d0;
#pragma unroll
      for (int e = 0; e < 4; ++e) st_tag(dst + e, nm[e] / dn, par);
    }
  }
  return true;
}

// ------------------------------------------------------------------ GATED DELTA RULE
// One item = (sequence b, head h, block of 32 value columns).  S^T rows of the block stream through
// the ring; q and k go through the causal conv (rolling state), SiLU and L2 norm; then per value
// column j: kS_j = S[:, j] . k, S'[:, j] = g S[:, j] + beta k (v_j - kS_j), o_j = S'[:, j] . q.
// The q / k conv state is shared by the blocks of (b, h): the last block to finish writes it.
template <int DK>
__device__ __forceinline__ bool op_delta(const KArgs& A, const Op& o, u32 w, u32& seq, u32& gen) {
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
  const bool tagged = (o.flags & OPF_TAGGED_IN) != 0;
  auto rd = [&](const float* p) { return tagged ? ld_tagged(A, p) : ld_sc1(p); };
  float* cst = (float*)Ld.conv_state + (size_t)b * C * (W - 1);
  const uint16_t* cw = (const uint16_t*)Ld.conv_w;

  auto conv = [&](int c, float* newstate_last) -> float {  // causal conv of channel c with its window
    float acc = 0.0f;
    for (int j = 0; j < W - 1; ++j) acc += bf2f(cw[(size_t)c * W + j]) * cst[(size_t)c * (W - 1) + j];
    const float x = rd(u + c);
    acc += bf2f(cw[(size_t)c * W + W - 1]) * x;
    *newstate_last = x;
    return silu(acc);
  };

  const u32 seq0 = seq;
  seq += NSL;
  release_upto(w, seq0 + min(w, (u32)NSL));
  for (u32 s = w; s < (u32)NSL; s += NC) {
    const u32 sq = seq0 + s;
    if (!wait_full(A, sq)) return false;
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
    const float rq = 1.0f / sqrtf(nq + 1e-6f) / sqrtf((float)DK), rk = 1.0f / sqrtf(nk + 1e-6f);
#pragma unroll
    for (int e = 0; e < DPL; ++e) { q[e] *= rq; k[e] *= rk; }
    const float gate = 1.0f / (1.0f + __expf(-rd(gts + h)));
    const float beta = 1.0f / (1.0f + __expf(-rd(gts + A.nh + h)));
    // value channels of this slot's rows: lane r < RPS computes row r's conv
    const int j0 = (int)cb * 32 + (int)s * RPS;
    const int vch = 2 * A.nh * DK + h * A.dv + j0 + (int)lane;
    float vx = 0.0f, vval = 0.0f;
    if ((int)lane < RPS) vval = conv(vch, &vx);
    const float* srows = (const float*)(g_ring + (sq % NSLOT) * (SLOT / 16));
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
      }
      // every item writes its outputs (zero for a row out of contract), tagged
      if (lane == 0) st_tag((float*)Ld.mix_o + (size_t)b * A.mix + h * A.dv + j0 + r, ok ? oj : 0.0f, A.tag & 1u);
    }
    // rolling conv state of this slot's value channels
    if (ok && (int)lane < RPS) {
      float* st = cst + (size_t)vch * (W - 1);
      for (int j = 0; j + 1 < W - 1; ++j) st[j] = st[j + 1];
      st[W - 2] = vx;
    }
    (void)xq; (void)xk;
    release_upto(w, seq0 + min(s + NC, (u32)NSL));
  }
  release_upto(w, seq0 + NSL);
  // q / k conv states: written once all blocks of (b, h) have read them (ticket)
  __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));
  if (!cbar(A, gen)) return false;
  u32* ticket = (u32*)Ld.tickets + bh;
  if (w == 0 && lane == 0) {
    const u32 prev = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    g_bcast[0] = (prev == ncb - 1) ? 1u : 0u;
  }
  if (!cbar(A, gen)) return false;
  if (lds_ld(&g_bcast[0])) {
    if (ok) {
      for (int t = (int)(w * 64 + lane); t < 2 * DK; t += NC * 64) {
        const int c = t < DK ? h * DK + t : A.nh * DK + h * DK + (t - DK);
        const float x = rd(u + c);
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
__device__ __forceinline__ void compute(u32 q0, u32 q1, u32 w) {
  u32 seq = 0, gen = 0;
  ItemCache ic;
  for (u32 oi = q0; oi < q1; ++oi) {
    const KArgs& A = kargs();
    const Op o = sload(A.ops + oi);
#if MK_TRACE_STAMPS
    if (w == 0 && lane_id() == 0) {
      const u32 t = (u32)__builtin_amdgcn_s_memrealtime();
      u32* tr = A.trace + (size_t)oi * 4;
      tr[0] = ((u32)o.opcode << 16) | (u32)(uint16_t)o.sig_stage;
      tr[1] = t;
      tr[2] = t;
      g_trace_oi = oi;
    }
#endif
    if (o.wait_stage != NO_STAGE && !(o.flags & OPF_TAGGED_IN)) {  // inputs finished by counter
      if (w == 0) wait_stage(A, o.wait_stage);
      if (!cbar(A, gen)) return;
    }
    bool alive = true;
    switch (o.opcode) {
      case OP_EMBED:
        op_embed<B>(A, w);
        if (!cbar(A, gen)) return;
        op_embed_finish(A, w, gen);
        break;
      case OP_GEMV:
        if constexpr (B < 8) alive = op_gemv<B>(A, o, w, seq, gen);
        break;
      case OP_MMV:
        if constexpr (B == 8) alive = op_mmv<B>(A, o, w, seq, gen);
        break;
      case OP_ATTN: alive = A.d == 128 ? op_attn<128>(A, o, w, seq, gen, ic) : op_attn<64>(A, o, w, seq, gen, ic); break;
      case OP_DELTA: alive = A.dk == 128 ? op_delta<128>(A, o, w, seq, gen) : op_delta<64>(A, o, w, seq, gen); break;
      default: break;
    }
    // Every value carried from op to op is wave-uniform.  The ops' lane-0 branches and early
    // exits make the compiler's divergence analysis lose track of that, which would demote the
    // carried state (and every loop around it) to vector registers; restate it.
    alive = __builtin_amdgcn_readfirstlane((int)alive) != 0;
    seq = __builtin_amdgcn_readfirstlane(seq);
    gen = __builtin_amdgcn_readfirstlane(gen);
    ic.restate();
    if (!alive || aborted()) return;
    const bool sig = o.sig_stage != NO_STAGE && !(o.flags & OPF_NO_SIGNAL);
    if (sig) __builtin_amdgcn_s_waitcnt(MK_VMCNT(0));  // this wave's outputs are complete
    if (!cbar(A, gen)) return;  // (also: the next op may overwrite this op's LDS areas)
    if (sig && w == 0 && lane_id() == 0) signal_stage(A, o.sig_stage, o.sig_index);
#if MK_TRACE_STAMPS
    if (w == 0 && lane_id() == 0) A.trace[(size_t)oi * 4 + 3] = (u32)__builtin_amdgcn_s_memrealtime();
#endif
  }
}

template <int B>
__device__ __forceinline__ void megakernel_body(const KArgs& A) {
  const u32 wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index: uniform per wave
  if (threadIdx.x < NC) g_consumed[threadIdx.x] = 0;
  if (threadIdx.x == 0) { g_filled = 0; g_aplan[0] = 0; }
  if (threadIdx.x == 0) { g_bar = 0; g_abort = 0; }
  __syncthreads();
  const u32 q0 = A.queue_off[blockIdx.x], q1 = A.queue_off[blockIdx.x + 1];
  if (wv == 0) loader(A, q0, q1);
  else compute<B>(q0, q1, wv - 1);
}

}  // namespace mk

#if MK_TRACE_STAMPS
#define MK_KNAME(b) mk_megakernel_##b##_trace
#else
#define MK_KNAME(b) mk_megakernel_##b
#endif
extern "C" __global__ void __launch_bounds__(mk::NTHREADS, 1) MK_KNAME(b1)(mk::KArgs A) { mk::megakernel_body<1>(A); }
extern "C" __global__ void __launch_bounds__(mk::NTHREADS, 1) MK_KNAME(b2)(mk::KArgs A) { mk::megakernel_body<2>(A); }
extern "C" __global__ void __launch_bounds__(mk::NTHREADS, 1) MK_KNAME(b4)(mk::KArgs A) { mk::megakernel_body<4>(A); }
extern "C" __global__ void __launch_bounds__(mk::NTHREADS, 1) MK_KNAME(b8)(mk::KArgs A) { mk::megakernel_body<8>(A); }
