// gfx950 kernels of the FIFO send/recv data plane.
//
// One launch holds both endpoints of every channel: each channel is served
// by `lanes` workgroup pairs; in a pair one workgroup is the producer and
// the other the consumer (zero-copy: the receiver), and each pair has its
// own head/tail/ptrExchange words.  Hand-off sequences follow
// "【NCCL】transport数据传输（二）" (p2pTransport: zero-copy with ptrExchange,
// copy through the peer's buffer; shmTransport: the same through host
// memory) and the POST / POLL outline of "Intra-Node Transport (P2P)",
// section 4.  The LL line format carries the flag inside the data ("RDMA and
// GPUDirect", section 四.1, option 2).
//
// Memory ordering on gfx950.  The eight XCDs each have their own L2, not
// kept coherent with each other for device memory by plain accesses.  Two
// orderings are built; a connection picks one:
//  * coherent (default): every access to shared protocol data -- FIFO
//    payload, zero-copy destination, counters, ptrExchange -- carries the
//    cache policy of the connection's scope (device: sc1; system: sc0 sc1),
//    the policy the compiler itself uses for relaxed atomics at that scope,
//    so each access is performed at the coherence point instead of in a
//    private L2 line.  A wave's s_waitcnt on all its outstanding accesses
//    completes them at that scope before the workgroup barrier that precedes
//    the counter store (release side); the peer issues its data accesses
//    only after its counter load has returned (acquire side).  No L2-wide
//    writeback or invalidate is needed, which is what makes this path fast.
//  * fenced: plain data accesses and the compiler's scoped release/acquire
//    fences, per wave (an L2 writeback before the counter store, an L2
//    invalidate after the counter load).  A workgroup barrier does not wait
//    for the other waves' stores, so every wave fences itself.
// Source payload and destination buffers that no peer reads during the
// launch are streamed with non-temporal accesses.  Every wait is bounded by
// the connection's timeout and also watches the host abort word, so every
// wave reaches the end of the kernel.

#include "xfer_internal.h"
#include "xfer.h"

namespace xfer {
namespace {

constexpr int kUnroll = 16;    // 16-byte vectors in flight per thread in the copy loop
constexpr int kLLUnroll = 8;   // LL lines polled together per thread

template <int SC>
__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) {
  if constexpr (SC == kScopeSystem)
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int SC>
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  if constexpr (SC == kScopeSystem)
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int SC>
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) {
  if constexpr (SC == kScopeSystem)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int SC>
__device__ __forceinline__ void fence_release() {
  if constexpr (SC == kScopeSystem)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "");
  else
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

template <int SC>
__device__ __forceinline__ void fence_acquire() {
  if constexpr (SC == kScopeSystem)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  else
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

enum : int { kOrdCoherent = 0, kOrdFenced = 1 };

// Cache-policy immediates of gfx950 buffer instructions.
constexpr int kPolSC0 = 1, kPolNT = 2, kPolSC1 = 16;

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Ordering of one connection: the cache policy of shared protocol data and
// the two halves of a hand-off.
template <int SC, int ORD>
struct Order {
  static constexpr int kShared =
      ORD == kOrdFenced ? 0 : (SC == kScopeSystem ? (kPolSC0 | kPolSC1) : kPolSC1);
  // This wave's earlier accesses are complete at the connection's scope.
  static __device__ __forceinline__ void release() {
    if constexpr (ORD == kOrdFenced) {
      fence_release<SC>();
    } else {
      compiler_fence();
      __builtin_amdgcn_s_waitcnt(0);
      compiler_fence();
    }
  }
  // Accesses after this point are issued after the counter load returned.
  static __device__ __forceinline__ void acquire() {
    if constexpr (ORD == kOrdFenced)
      fence_acquire<SC>();
    else
      compiler_fence();
  }
};

// Lane 0's v for the whole wave.  readfirstlane works on (signed) 32-bit
// ints, so each half is held as uint32_t and widening zero-extends it.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Every lane loads the same word (one request per wave); the value is made
// wave-uniform explicitly.
template <int SC>
__device__ __forceinline__ uint64_t wave_load(const uint64_t* p) {
  return uniform_u64(ld_u64<SC>(p));
}

// A failure of the connection: the host's status word (pinned host memory)
// and its mirror beside the counters, which every later launch on the
// connection reads on entry.
__device__ __forceinline__ void raise_err(const ConnArgs& A, uint32_t code) {
  __hip_atomic_store(&A.status->err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(A.err_dev, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Bound of one wait: wall-clock ticks (s_memrealtime) plus the host abort
// word.  Reading the clock is a scalar-memory round trip that would sit
// between two polls, so it is read only every 64th poll (the first read
// starts the clock) and the abort word every 1024th: a wait ends at most
// about 64 polls after its bound.
struct Deadline {
  uint64_t start, ticks;
  Status* st;
  uint32_t n;
  __device__ Deadline(uint64_t t, Status* s) : start(0), ticks(t), st(s), n(0) {}
  __device__ __forceinline__ uint32_t expired() {
    if (((++n) & 63u) != 0u) return 0;
    if ((n & 1023u) == 0u &&
        __hip_atomic_load(&st->abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
      return XFER_ERR_ABORTED;
    const uint64_t now = wall_clock64();
    if (start == 0) {
      start = now;
      return 0;
    }
    return now - start > ticks ? XFER_ERR_TIMEOUT : 0;
  }
};

// Channel range: ceil(n / nch) rounded up to 16 bytes per channel, in order.
struct Range {
  uint64_t beg, len, k;
};

__device__ __forceinline__ Range chan_range(uint64_t n, uint32_t nch, uint32_t c, uint64_t S) {
  uint64_t per = (n + nch - 1) / nch;
  per = (per + 15) & ~uint64_t(15);
  const uint64_t b = min(n, static_cast<uint64_t>(c) * per);
  const uint64_t e = min(n, b + per);
  Range r;
  r.beg = b;
  r.len = e - b;
  r.k = (r.len + S - 1) / S;
  return r;
}

// ------------------------------------------------------------ lane blocks
// A slot is cut into blocks of blockDim.x 16-byte vectors (one per thread);
// lane w of P owns blocks w, w + P, w + 2P, ...  Ownership depends only on
// the position in the slot, never on the chunk length, so a slot byte is
// always written and drained by the same lane pair and that lane's head
// covers every byte its producer will overwrite.  A short chunk still
// spreads over as many lanes as it has blocks.  LL uses the same map over
// lines (a block is blockDim.x lines), except on connections whose whole
// step fits the lanes at one line per thread: their lanes own stripes of
// lines (ll_striped).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over n bytes: the buffer unit checks every access
// against n (an access past it reads 0 and writes nothing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, static_cast<int>(n),
                                           0x00020000);
}

// Two fixed lane layouts (CYC template argument); both give every slot byte
// one owning lane whatever the chunk length:
//  * contiguous (SIMPLE): lane w owns the slice [w * sub, (w + 1) * sub) of
//    the slot, sub = S / P rounded up to 16 bytes -- measured faster for the
//    FIFO round trip;
//  * block-cyclic (zero-copy): blocks of blockDim.x vectors dealt round-robin
//    to the lanes -- measured faster for writes straight into B, and short
//    chunks spread over more lanes.
// A LaneSpan is the lane's addressable part of a chunk of L16 vector bytes:
// base = first byte, lim = bytes addressable from base.
struct LaneSpan {
  uint32_t base, lim;
};

__device__ __forceinline__ uint32_t contiguous_slice(uint64_t S, uint32_t P) {
  return static_cast<uint32_t>((((S + P - 1) / P) + 15) & ~uint64_t(15));
}

template <bool CYC>
__device__ __forceinline__ LaneSpan lane_span(uint32_t L16, uint64_t S, uint32_t P, uint32_t w) {
  if constexpr (CYC) {
    return LaneSpan{0, L16};
  } else {
    const uint32_t sub = contiguous_slice(S, P);
    const uint32_t lo = min(L16, w * sub), hi = min(L16, (w + 1) * sub);
    return LaneSpan{lo, hi - lo};
  }
}

// Byte offset (from the lane's base) of this thread's u-th vector.
template <bool CYC>
__device__ __forceinline__ uint32_t lane_vec(uint32_t w, uint32_t P, uint32_t u) {
  if constexpr (CYC)
    return ((w + u * P) * blockDim.x + threadIdx.x) << 4;
  else
    return (u * blockDim.x + threadIdx.x) << 4;
}

// Vector groups (of blockDim.x vectors) a lane covers in a full step of S bytes.
template <bool CYC>
__device__ __forceinline__ uint32_t lane_blocks(uint64_t S, uint32_t P) {
  const uint32_t B = blockDim.x * 16u;
  if constexpr (CYC) {
    const uint64_t nb = (S + B - 1) / B;
    return static_cast<uint32_t>((nb + P - 1) / P);
  } else {
    return (contiguous_slice(S, P) + B - 1) / B;
  }
}

// Bytes of a chunk past its last whole vector (only the final chunk of a
// transfer has them) are copied bytewise by the lane that owns offset L16.
template <int LP, int SP, bool CYC>
__device__ __forceinline__ void lane_tail(const uint8_t* s, uint8_t* d, uint32_t L, uint64_t S,
                                          uint32_t P, uint32_t w) {
  const uint32_t L16 = L & ~15u;
  if (L == L16 || threadIdx.x >= L - L16) return;
  uint32_t owner;
  if constexpr (CYC)
    owner = (L16 / (blockDim.x * 16u)) % P;
  else
    owner = min(P - 1, L16 / contiguous_slice(S, P));
  if (owner != w) return;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, L), rd = make_rsrc(d, L);
  __builtin_amdgcn_raw_buffer_store_b8(
      __builtin_amdgcn_raw_buffer_load_b8(rs, L16 + threadIdx.x, 0, LP), rd, L16 + threadIdx.x, 0,
      SP);
}

// Lane w's share of a chunk of L (< 2^31) bytes, from s to d (both chunk
// bases), with load policy LP and store policy SP: kUnroll vectors in
// flight per thread before their stores.  Either end may sit at any byte
// address: compute queues run in unaligned-access mode (the FIFO side is
// always 16-byte aligned).  The descriptors are opaque to alias analysis,
// so a batch of loads stays ahead of its stores.
template <int LP, int SP, bool CYC>
__device__ __forceinline__ void lane_copy(const uint8_t* s, uint8_t* d, uint64_t L64, uint64_t S,
                                          uint32_t P, uint32_t w) {
  const uint32_t L = static_cast<uint32_t>(L64);
  const LaneSpan sp = lane_span<CYC>(L & ~15u, S, P, w);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s + sp.base, sp.lim),
                               rd = make_rsrc(d + sp.base, sp.lim);
  const uint32_t B = blockDim.x * 16u;
  const uint32_t groups = (sp.lim + B - 1) / B;  // vector groups spanned from base
  for (uint32_t u0 = 0; (CYC ? w + u0 * P : u0) < groups; u0 += kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      r[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_vec<CYC>(w, P, u0 + u), 0, LP);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(r[u], rd, lane_vec<CYC>(w, P, u0 + u), 0, SP);
  }
  lane_tail<LP, SP, CYC>(s, d, L, S, P, w);
}

// A lane's share of one step held in registers (software-pipelined
// producers): kUnroll vectors per thread.  Every thread always issues
// exactly kUnroll loads or stores; the buffer unit drops the ones past the
// chunk (loads read 0), so the count of accesses in flight is a constant.
struct Batch {
  u32x4 r[kUnroll];
};

template <int LP, bool CYC>
__device__ __forceinline__ void batch_load(Batch& b, const uint8_t* s, uint32_t L, uint64_t S,
                                           uint32_t P, uint32_t w) {
  const LaneSpan sp = lane_span<CYC>(L & ~15u, S, P, w);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(s + sp.base, sp.lim);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    b.r[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane_vec<CYC>(w, P, u), 0, LP);
}

template <int SP, bool CYC>
__device__ __forceinline__ void batch_store(const Batch& b, uint8_t* d, uint32_t L, uint64_t S,
                                            uint32_t P, uint32_t w) {
  const LaneSpan sp = lane_span<CYC>(L & ~15u, S, P, w);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(d + sp.base, sp.lim);
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    __builtin_amdgcn_raw_buffer_store_b128(b.r[u], rd, lane_vec<CYC>(w, P, u), 0, SP);
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14]).  Vector memory operations complete in issue order, so
// after "stores, then N loads" vmcnt(N) means the stores are complete.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  compiler_fence();
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  compiler_fence();
}

// Per-workgroup state of one side of a lane across the messages of a launch.
struct Side {
  LaneCtrl* tx;     // the send side's block of this lane: head, ptrExchange
  LaneCtrl* rx;     // the receive side's block: tail (and a relay's proxy tails)
  TraceRec* tr;     // this (channel, lane, side)'s step-trace ring, or nullptr
  uint32_t jit;     // jitter seed of this (channel, lane, side), 0 = none
  uint64_t base;    // step counter at launch start (own counter: tail or head)
  uint64_t seen;    // last observed peer counter (wave-uniform)
  bool dead;        // the connection carries a failure from an earlier launch
  Range r;          // the channel's range and steps in the current message
};

// DBG: the debug kernel variant, which writes the step trace and applies
// the jitter.  Without it the trace ring and the jitter seed are constants
// (null, 0), so every debug branch folds away.  UNIFORM: the side is a
// whole workgroup (its values are made wave-uniform); otherwise one thread
// (a zero-copy receiver lane).
template <bool DBG, bool UNIFORM = true>
__device__ __forceinline__ Side make_side(const ConnArgs& A, uint32_t c, uint32_t w, bool producer,
                                          int sc) {
  Side s;
  const uint64_t lane = static_cast<uint64_t>(c) * A.lanes + w;
  s.tx = A.ctrl_tx + lane;
  s.rx = A.ctrl_rx + lane;
  s.tr = DBG && A.trace ? A.trace + (lane * 2 + (producer ? 0u : 1u)) * A.trace_per : nullptr;
  s.jit = DBG && A.jitter ? (A.jitter ^ static_cast<uint32_t>(lane * 2 + (producer ? 0u : 1u)) *
                                            0x9E3779B9u) | 1u
                          : 0u;
  s.r = Range{0, 0, 0};  // set per message
  // A side is the only writer of its own counter, and the previous launch
  // that wrote it has completed, so a plain coherent load reads it.
  // The connection's failure mirror is read in the same round trip: a
  // launch queued behind a failed one starts on whatever that one left (a
  // half-advanced counter, an address still in ptrExchange), so it does
  // nothing at all.
  const uint64_t* own = producer ? &s.rx->tail : &s.tx->head;
  uint64_t v;
  uint32_t e;
  if (sc == kScopeSystem) {
    v = ld_u64<kScopeSystem>(own);
    e = ld_u32<kScopeSystem>(A.err_dev);
  } else {
    v = ld_u64<kScopeAgent>(own);
    e = ld_u32<kScopeAgent>(A.err_dev);
  }
  if constexpr (UNIFORM) {
    s.base = uniform_u64(v);
    s.dead = __builtin_amdgcn_readfirstlane(e) != 0;
  } else {
    s.base = v;
    s.dead = e != 0;
  }
  s.seen = 0;
  return s;
}

// Step trace, written by thread 0 of a side when the connection has a trace
// buffer: event 0 when the step is acquired (credit, a destination, or the
// data ready), event 1 just before the step is published (tail or head),
// at slots 2g and 2g+1 of the side's ring (modulo its size).  The ring's
// index in the buffer names the channel, lane and side.
__device__ __forceinline__ void trace_write(TraceRec* base, uint32_t per, uint32_t lanes,
                                            TraceRec* ring, uint64_t g, uint32_t ev,
                                            uint64_t value) {
  const uint64_t region = static_cast<uint64_t>(ring - base) / per;
  const uint64_t lane = region >> 1;
  TraceRec r;
  r.time = wall_clock64();
  r.step = g;
  r.value = value;
  r.channel = static_cast<uint32_t>(lane / lanes);
  r.lane = static_cast<uint16_t>(lane % lanes);
  r.side = static_cast<uint8_t>(region & 1u);
  r.event = static_cast<uint8_t>(ev);
  ring[(2 * g + ev) % per] = r;
}

__device__ __forceinline__ void trace_step(const ConnArgs& A, const Side& sd, uint64_t g,
                                           uint32_t ev, uint64_t value) {
  if (sd.tr != nullptr) trace_write(A.trace, A.trace_per, A.lanes, sd.tr, g, ev, value);
}

// Jitter (debug variant): each wave sleeps a pseudo-random 0..15 x 512
// cycles at point p of step g, a function of the side's seed, g, p and the
// wave, so producer and consumer, and the waves of one side, reach their
// accesses in orders that undisturbed runs rarely take.  Wave-uniform;
// every wait stays bounded, it only starts later.
__device__ __forceinline__ void jitter(const Side& sd, uint64_t g, uint32_t p) {
  if (sd.jit == 0) return;
  uint32_t h = sd.jit ^ static_cast<uint32_t>(g) * 0x85EBCA6Bu ^ (p + 1u) * 0xC2B2AE35u ^
               (threadIdx.x >> 6) * 0x27D4EB2Fu;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  for (uint32_t i = h & 15u; i > 0; --i) __builtin_amdgcn_s_sleep(8);
}

// Shared by the waves of a workgroup: the first failure seen by any wave.
struct Shared {
  uint32_t err;
  uint32_t werr;    // outcome of a wait polled by one wave (wait_count)
  uint64_t wval;    // the counter value that ended it
  uint64_t ptr[2];  // zero-copy destinations, indexed by step parity
};

__device__ __forceinline__ bool wg_failed(Shared& sh, uint32_t local_err, const ConnArgs& A) {
  if (local_err) sh.err = local_err;
  __syncthreads();
  const uint32_t e = sh.err;
  if (e && threadIdx.x == 0) raise_err(A, e);
  return e != 0;
}

// Slot of step g: g mod nslots.  A 64-bit remainder is a long chain of
// scalar instructions that sits on the latency path of every small message,
// so a power-of-two slot count takes a mask instead.
__device__ __forceinline__ uint8_t* slot_of(const ConnArgs& A, uint32_t c, uint64_t g) {
  const uint32_t ns = A.nslots;
  const uint64_t s = (ns & (ns - 1u)) == 0u ? (g & (ns - 1u)) : g % ns;
  return A.fifo + (static_cast<uint64_t>(c) * ns + s) * A.slot_bytes;
}

// The same slot in the FIFO the consumer drains.
__device__ __forceinline__ uint8_t* slot_rx(const ConnArgs& A, uint32_t c, uint64_t g) {
  return A.fifo_rx + (slot_of(A, c, g) - A.fifo);
}

__device__ __forceinline__ uint32_t chunk_len(const Side& sd, uint64_t S, uint64_t j) {
  return static_cast<uint32_t>(min(S, sd.r.len - j * S));
}

// ------------------------------------------------------------------ SIMPLE
// Waits until *p + add > g (add = nslots for a producer's credit, 0 for a
// consumer's ready count) and returns in v the value that ended the wait.
// Written without a subtraction because the counter may run ahead of g.
//
// With WG, a counter in host memory (system scope) is polled by wave 0 alone,
// which hands the outcome to the other waves through LDS: each poll is a
// read across PCIe, and every wave of every waiting workgroup polling at
// once crowds out the DMA copies that share the link (they ran a third
// slower under such polling).  Every wave of the workgroup must then reach
// the call, and a workgroup barrier must separate two such calls (each step
// ends with one).  Counters in HBM are polled by every wave, which is
// cheaper than a barrier per step.
template <int SC, bool WG>
__device__ __forceinline__ uint32_t wait_count(const uint64_t* p, uint64_t add, uint64_t g,
                                               uint64_t ticks, Status* st, Shared& sh,
                                               uint64_t& v) {
  uint32_t err = 0;
  if constexpr (WG && SC == kScopeSystem) {
    if (threadIdx.x < static_cast<uint32_t>(warpSize)) {
      Deadline dl(ticks, st);
      uint64_t x;
      while (g >= (x = wave_load<SC>(p)) + add) {
        if ((err = dl.expired())) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (threadIdx.x == 0) {
        sh.werr = err;
        sh.wval = x;
      }
    }
    __syncthreads();
    err = sh.werr;
    v = sh.wval;
  } else {
    Deadline dl(ticks, st);
    while (g >= (v = wave_load<SC>(p)) + add) {
      if ((err = dl.expired())) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return err;
}

// Waits until step g has credit: g < head + nslots.  head may run ahead of
// g: an LL consumer whose lane owns no lines of a step has nothing to wait
// for and frees that step at once.
template <int SC, int ORD, bool WG>
__device__ __forceinline__ uint32_t wait_credit(const ConnArgs& A, Side& sd, uint64_t g,
                                                uint64_t ticks, Shared& sh) {
  if (g < sd.seen + A.nslots) return 0;
  uint64_t h = 0;
  const uint32_t err = wait_count<SC, WG>(&sd.tx->head, A.nslots, g, ticks, A.status, sh, h);
  if (err) return err;
  Order<SC, ORD>::acquire();  // the consumer's reads of the slot precede our writes
  sd.seen = h;
  return 0;
}

// Coherent producer whose share of a step fits one register batch, software
// pipelined: the source of step j+1 is loaded while the FIFO stores of
// step j drain, and vmcnt(kUnroll) then covers exactly those stores.
template <int SC, int ORD>
__device__ bool simple_send_piped(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t g0,
                                  const uint8_t* src, uint64_t ticks, Shared& sh) {
  using O = Order<SC, ORD>;
  const uint64_t S = A.step_bytes;
  const uint32_t P = A.lanes;
  Batch b;
  batch_load<kPolNT, false>(b, src + sd.r.beg, chunk_len(sd, S, 0), S, P, w);
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = g0 + j;
    const uint32_t err = wait_credit<SC, ORD, true>(A, sd, g, ticks, sh);
    if (!err && threadIdx.x == 0) trace_step(A, sd, g, 0, sd.seen);
    if (!err) {
      jitter(sd, g, 0);
      const uint32_t L = chunk_len(sd, S, j);
      uint8_t* slot = slot_of(A, c, g);
      batch_store<O::kShared, false>(b, slot, L, S, P, w);
      lane_tail<kPolNT, O::kShared, false>(src + sd.r.beg + j * S, slot, L, S, P, w);
      compiler_fence();  // the next loads issue after these stores: vmcnt counts on that
      if (j + 1 < sd.r.k) {
        batch_load<kPolNT, false>(b, src + sd.r.beg + (j + 1) * S, chunk_len(sd, S, j + 1), S, P, w);
        wait_vmcnt<kUnroll>();
      } else {
        wait_vmcnt<0>();
      }
    }
    jitter(sd, g, 1);
    if (wg_failed(sh, err, A)) return false;
    if (threadIdx.x == 0) {
      trace_step(A, sd, g, 1, g + 1);
      st_u64<SC>(&sd.rx->tail, g + 1);
    }
  }
  return true;
}

// Producer of message m: for each step g, wait for credit g - head < nslots,
// write the chunk into slot g mod nslots, release, tail = g+1.
template <int SC, int ORD, bool AL>
__device__ bool simple_send(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t g0,
                            const uint8_t* src, uint64_t ticks, Shared& sh) {
  using O = Order<SC, ORD>;
  const uint64_t S = A.step_bytes;
  if constexpr (ORD == kOrdCoherent) {
    if (lane_blocks<false>(S, A.lanes) <= kUnroll)
      return simple_send_piped<SC, ORD>(A, c, w, sd, g0, src, ticks, sh);
  }
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = g0 + j;
    const uint32_t err = wait_credit<SC, ORD, true>(A, sd, g, ticks, sh);
    if (!err && threadIdx.x == 0) trace_step(A, sd, g, 0, sd.seen);
    if (!err) {
      jitter(sd, g, 0);
      lane_copy<kPolNT, O::kShared, false>(src + sd.r.beg + j * S, slot_of(A, c, g), chunk_len(sd, S, j),
                                    S, A.lanes, w);
      O::release();
    }
    jitter(sd, g, 1);
    if (wg_failed(sh, err, A)) return false;
    if (threadIdx.x == 0) {
      trace_step(A, sd, g, 1, g + 1);
      st_u64<SC>(&sd.rx->tail, g + 1);
    }
  }
  return true;
}

// Consumer of message m: wait for tail > g, acquire, copy the slot out,
// head = g+1.
//
// On a relay connection the step reaches the consumer through the host
// proxies: it waits on the receive proxy's tail (gtail) and drains the
// receive FIFO; head still goes back to the producer.
template <int SC, int ORD, bool AL>
__device__ bool simple_recv(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t g0,
                            uint8_t* dst, uint64_t ticks, Shared& sh) {
  using O = Order<SC, ORD>;
  const uint64_t S = A.step_bytes;
  // (the proxy tails are per channel, in lane 0's control block)
  const uint64_t* ready = A.relay ? &A.ctrl_rx[static_cast<uint64_t>(c) * A.lanes].gtail : &sd.rx->tail;
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = g0 + j;
    uint32_t err = 0;
    if (sd.seen <= g) {
      uint64_t t = 0;
      err = wait_count<SC, true>(ready, 0, g, ticks, A.status, sh, t);
      if (!err) {
        O::acquire();
        sd.seen = t;
      }
    }
    if (!err && threadIdx.x == 0) trace_step(A, sd, g, 0, sd.seen);
    if (!err) {
      jitter(sd, g, 0);
      lane_copy<O::kShared, kPolNT, false>(slot_rx(A, c, g), dst + sd.r.beg + j * S,
                                           chunk_len(sd, S, j), S, A.lanes, w);
      // Our slot reads are complete before the slot is handed back: each
      // loaded value has already fed its store.  Coherent ordering needs no
      // wait for the destination stores; fenced ordering keeps its fence.
      if constexpr (ORD == kOrdFenced) O::release();
    }
    jitter(sd, g, 1);
    if (wg_failed(sh, err, A)) return false;
    if (threadIdx.x == 0) {
      trace_step(A, sd, g, 1, g + 1);
      st_u64<SC>(&sd.tx->head, g + 1);
    }
  }
  return true;
}

// ---------------------------------------------------------------------- LL
// Line = {4 payload bytes, flag = g+1}, stored and loaded as one 64-bit
// access at the connection's scope; the last word of a chunk is zero-padded.
// Chunks are under 2^31 bytes (half a slot of at most 1 GiB), so line
// indices and byte offsets within a chunk fit 32 bits.
template <bool AL>
__device__ __forceinline__ uint32_t ll_src_word(const uint8_t* p, uint32_t L, uint32_t line) {
  const uint32_t off = line * 4u;
  if (AL && off + 4u <= L) return *reinterpret_cast<const uint32_t*>(p + off);
  uint32_t v = 0;
  for (uint32_t b = 0; b < 4u && off + b < L; ++b) v |= static_cast<uint32_t>(p[off + b]) << (8u * b);
  return v;
}

template <bool AL>
__device__ __forceinline__ void ll_dst_word(uint8_t* p, uint32_t L, uint32_t line, uint32_t v) {
  const uint32_t off = line * 4u;
  if (AL && off + 4u <= L) {
    *reinterpret_cast<uint32_t*>(p + off) = v;
    return;
  }
  for (uint32_t b = 0; b < 4u && off + b < L; ++b) p[off + b] = static_cast<uint8_t>(v >> (8u * b));
}

// The striped LL layout (ll_layout, on the host): lane w owns lines
// [w q, (w + 1) q) of every slot, and its threads cover `group` consecutive
// steps at once, thread t taking line w q + t mod q of step t / q of the
// group.  Vector memory operations complete in issue order, so one thread
// looping over the steps of a message would hold each step's source load
// behind the previous step's line store and each flag poll behind the
// previous step's destination and head stores: a round trip per step.
// Here the steps of a group go to different waves and overlap.  The
// consumer frees a group with one head store, for its last step (its steps'
// slots are distinct, and the producer has credit for all of them once head
// reaches the group's first step).  Striped connections run kernels of
// their own (kProtoLLStriped), so each kernel holds one layout only.

// A source word of a striped send loaded ahead of it: the word of this
// thread's line in the first group of the send (`ok` false: none).  The
// ping-pong's endpoint X sends the same buffer a every round and never
// writes it (its receive writes c, which may not overlap a), so it loads
// the next round's word before it polls for the reply: the load then does
// not wait, in issue order, behind the reply's destination and head stores.
struct NextWord {
  bool ok;
  uint32_t word;
};

template <bool AL>
__device__ __forceinline__ NextWord ll_striped_first_word(const ConnArgs& A, uint32_t w,
                                                          const Side& sd, const uint8_t* src) {
  const uint32_t u = threadIdx.x >> A.ll_stripe_log2;
  const uint32_t i = (w << A.ll_stripe_log2) + (threadIdx.x & ((1u << A.ll_stripe_log2) - 1u));
  NextWord nw{false, 0u};
  if (u < A.ll_group && u < sd.r.k) {
    const uint32_t L = chunk_len(sd, A.step_bytes, u);
    if (i < (L + 3u) / 4u) {
      nw.word = ll_src_word<AL>(src + sd.r.beg + u * A.step_bytes, L, i);
      nw.ok = true;
    }
  }
  return nw;
}

template <int SC, int ORD, bool AL>
__device__ __forceinline__ bool ll_send_striped(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd,
                                                uint64_t g0, const uint8_t* src, uint64_t ticks,
                                                Shared& sh, const NextWord* pre = nullptr) {
  const uint64_t S = A.step_bytes;
  const uint32_t m = A.ll_group;
  const uint32_t u = threadIdx.x >> A.ll_stripe_log2;  // (wave-uniform)
  const uint32_t li = threadIdx.x & ((1u << A.ll_stripe_log2) - 1u);
  const uint32_t i = (w << A.ll_stripe_log2) + li;     // this thread's line of a step
  uint32_t err = 0;
  for (uint64_t j0 = 0; j0 < sd.r.k && !err; j0 += m) {
    const uint64_t j = j0 + u;
    if (u >= m || j >= sd.r.k) continue;
    const uint64_t g = g0 + j;
    if ((err = wait_credit<SC, ORD, false>(A, sd, g, ticks, sh))) break;
    const uint32_t L = chunk_len(sd, S, j);
    if (li == 0) {  // the lines are the publication: stamp before this thread's
      trace_step(A, sd, g, 0, sd.seen);
      trace_step(A, sd, g, 1, g + 1);
    }
    jitter(sd, g, 0);
    if (i < (L + 3u) / 4u) {
      uint64_t* lines = reinterpret_cast<uint64_t*>(slot_of(A, c, g));
      const uint64_t flag = static_cast<uint64_t>(static_cast<uint32_t>(g + 1)) << 32;
      const uint32_t v = pre != nullptr && j0 == 0 && pre->ok
                             ? pre->word
                             : ll_src_word<AL>(src + sd.r.beg + j * S, L, i);
      st_u64<SC>(&lines[i], flag | v);
    }
  }
  return !wg_failed(sh, err, A);
}

// What a striped receive does before its first poll: nothing, or (the
// ping-pong's endpoint X) load its next send's source word.
struct NoAhead {
  static constexpr bool kActive = false;
  __device__ void operator()() const {}
};

template <int SC, int ORD, bool AL, typename Ahead = NoAhead>
__device__ __forceinline__ bool ll_recv_striped(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd,
                                                uint64_t g0, uint8_t* dst, uint64_t ticks,
                                                Shared& sh, Ahead ahead = Ahead()) {
  using O = Order<SC, ORD>;
  if constexpr (Ahead::kActive) {
    ahead();
    compiler_fence();  // issued before the polls below
  }
  const uint64_t S = A.step_bytes;
  const uint32_t m = A.ll_group;
  const uint32_t u = threadIdx.x >> A.ll_stripe_log2;
  const uint32_t li = threadIdx.x & ((1u << A.ll_stripe_log2) - 1u);
  const uint32_t i = (w << A.ll_stripe_log2) + li;
  for (uint64_t j0 = 0; j0 < sd.r.k; j0 += m) {
    const uint32_t nb = static_cast<uint32_t>(min(static_cast<uint64_t>(m), sd.r.k - j0));
    const uint64_t j = j0 + u, g = g0 + j;
    uint32_t err = 0;
    if (u < nb) {
      jitter(sd, g, 0);
      const uint32_t L = chunk_len(sd, S, j);
      if (i < (L + 3u) / 4u) {
        const uint32_t want = static_cast<uint32_t>(g + 1);
        const uint64_t* line = reinterpret_cast<const uint64_t*>(slot_of(A, c, g)) + i;
        uint64_t v = ld_u64<SC>(line);
        if (static_cast<uint32_t>(v >> 32) != want) {
          Deadline dl(ticks, A.status);
          do {
            v = ld_u64<SC>(line);
          } while (static_cast<uint32_t>(v >> 32) != want && !(err = dl.expired()));
        }
        if (!err) ll_dst_word<AL>(dst + sd.r.beg + j * S, L, i, static_cast<uint32_t>(v));
      }
    }
    // Our line reads are complete before the slots go back: every value has
    // fed its flag test.  Fenced ordering keeps its release fence.
    if constexpr (ORD == kOrdFenced) O::release();
    if (u < nb) jitter(sd, g, 1);
    if (wg_failed(sh, err, A)) return false;
    if (threadIdx.x == 0) {
      const uint64_t gb = g0 + j0;
      for (uint32_t x = 0; sd.tr != nullptr && x < nb; ++x) {
        trace_step(A, sd, gb + x, 0, gb + x + 1);  // every line of the step seen
        trace_step(A, sd, gb + x, 1, gb + nb);     // the head that hands it back
      }
      st_u64<SC>(&sd.tx->head, gb + nb);
    }
  }
  return true;
}

template <int SC, int ORD, bool AL, bool STRIPED>
__device__ __forceinline__ bool ll_send(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t g0,
                        const uint8_t* src, uint64_t ticks, Shared& sh) {
  if constexpr (STRIPED) return ll_send_striped<SC, ORD, AL>(A, c, w, sd, g0, src, ticks, sh);
  const uint64_t S = A.step_bytes;
  const uint32_t P = A.lanes, nthr = blockDim.x;
  uint32_t err = 0;
  for (uint64_t j = 0; j < sd.r.k && !err; ++j) {
    const uint64_t g = g0 + j;
    if ((err = wait_credit<SC, ORD, false>(A, sd, g, ticks, sh))) break;
    const uint32_t L = chunk_len(sd, S, j);
    const uint32_t nl = (L + 3u) / 4u;
    uint64_t* lines = reinterpret_cast<uint64_t*>(slot_of(A, c, g));
    const uint8_t* s = src + sd.r.beg + j * S;
    const uint64_t flag = static_cast<uint64_t>(static_cast<uint32_t>(g + 1)) << 32;
    if (threadIdx.x == 0) {  // the lines are the publication: stamp before thread 0's
      trace_step(A, sd, g, 0, sd.seen);
      trace_step(A, sd, g, 1, g + 1);
    }
    jitter(sd, g, 0);  // each wave's lines go out at its own moment
    if (nl <= nthr * P) {  // one pass: at most one line per thread
      const uint32_t i = w * nthr + threadIdx.x;
      if (i < nl) st_u64<SC>(&lines[i], flag | ll_src_word<AL>(s, L, i));
      continue;
    }
    for (uint32_t blk = w; blk * nthr < nl; blk += P) {
      const uint32_t i = blk * nthr + threadIdx.x;
      if (i < nl) st_u64<SC>(&lines[i], flag | ll_src_word<AL>(s, L, i));
    }
  }
  return !wg_failed(sh, err, A);
}

template <int SC, int ORD, bool AL, bool STRIPED>
__device__ __forceinline__ bool ll_recv(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t g0,
                        uint8_t* dst, uint64_t ticks, Shared& sh) {
  if constexpr (STRIPED) return ll_recv_striped<SC, ORD, AL>(A, c, w, sd, g0, dst, ticks, sh);
  using O = Order<SC, ORD>;
  const uint64_t S = A.step_bytes;
  const uint32_t P = A.lanes, nthr = blockDim.x;
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = g0 + j;
    const uint32_t want = static_cast<uint32_t>(g + 1);
    const uint32_t L = chunk_len(sd, S, j);
    const uint32_t nl = (L + 3u) / 4u;
    const uint64_t* lines = reinterpret_cast<const uint64_t*>(slot_of(A, c, g));
    uint8_t* d = dst + sd.r.beg + j * S;
    uint32_t err = 0;
    jitter(sd, g, 0);
    if (nl <= nthr * P) {  // one pass: at most one line per thread
      const uint32_t i = w * nthr + threadIdx.x;
      if (i < nl) {
        uint64_t v = ld_u64<SC>(&lines[i]);
        if (static_cast<uint32_t>(v >> 32) != want) {
          Deadline dl(ticks, A.status);
          do {
            v = ld_u64<SC>(&lines[i]);
          } while (static_cast<uint32_t>(v >> 32) != want && !(err = dl.expired()));
        }
        if (!err) ll_dst_word<AL>(d, L, i, static_cast<uint32_t>(v));
      }
    } else {
      for (uint32_t b0 = w; b0 * nthr < nl && !err; b0 += static_cast<uint32_t>(kLLUnroll) * P) {
        uint64_t v[kLLUnroll];
        bool pend = false;
#pragma unroll
        for (int u = 0; u < kLLUnroll; ++u) {
          const uint32_t i = (b0 + static_cast<uint32_t>(u) * P) * nthr + threadIdx.x;
          v[u] = i < nl ? ld_u64<SC>(&lines[i]) : (static_cast<uint64_t>(want) << 32);
          pend |= static_cast<uint32_t>(v[u] >> 32) != want;
        }
        if (pend) {
          Deadline dl(ticks, A.status);
          while (pend) {
            pend = false;
#pragma unroll
            for (int u = 0; u < kLLUnroll; ++u) {
              if (static_cast<uint32_t>(v[u] >> 32) != want) {
                v[u] = ld_u64<SC>(&lines[(b0 + static_cast<uint32_t>(u) * P) * nthr + threadIdx.x]);
                pend |= static_cast<uint32_t>(v[u] >> 32) != want;
              }
            }
            if (pend && (err = dl.expired())) break;
          }
        }
        if (!err) {
#pragma unroll
          for (int u = 0; u < kLLUnroll; ++u) {
            const uint32_t i = (b0 + static_cast<uint32_t>(u) * P) * nthr + threadIdx.x;
            if (i < nl) ll_dst_word<AL>(d, L, i, static_cast<uint32_t>(v[u]));
          }
        }
      }
    }
    // Our line reads are complete before the slot is handed back: every
    // value has been consumed by its flag test.  Coherent ordering needs
    // nothing more (the destination stores may still be in flight); fenced
    // ordering keeps its release fence.
    if constexpr (ORD == kOrdFenced) O::release();
    jitter(sd, g, 1);
    if (wg_failed(sh, err, A)) return false;
    if (threadIdx.x == 0) {
      trace_step(A, sd, g, 0, static_cast<uint64_t>(want));  // every line of the step seen
      trace_step(A, sd, g, 1, g + 1);
      st_u64<SC>(&sd.tx->head, g + 1);
    }
  }
  return true;
}

// LL has no polled tail: the producer records its final step count once.
template <int SC>
__device__ __forceinline__ void ll_close(Side& sd, uint64_t end_step) {
  if (threadIdx.x == 0) st_u64<SC>(&sd.rx->tail, end_step);
}

// --------------------------------------------------------------- zero-copy
// Wave 0 waits for a published destination (the base of the step's chunk in
// B), takes it and clears the word; the address reaches the other waves
// through LDS (`out`) after the caller's barrier.  `first` is the value of
// a poll of the word that wave 0 issued earlier (0: none, or nothing was
// published yet), so that accesses issued after that poll do not delay it.
template <int SC, int ORD>
__device__ __forceinline__ uint32_t take_address(const ConnArgs& A, Side& sd, uint64_t ticks,
                                                 uint64_t& out, uint64_t first = 0) {
  uint32_t err = 0;
  if (threadIdx.x < 64) {
    uint64_t p = uniform_u64(first);
    if (p == 0) {
      Deadline dl(ticks, A.status);
      while ((p = wave_load<SC>(&sd.tx->ptrx)) == 0) {
        if ((err = dl.expired())) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (threadIdx.x == 0) {
      if (!err) {
        Order<SC, ORD>::acquire();
        st_u64<SC>(&sd.tx->ptrx, 0);
      }
      out = p;
    }
  }
  return err;
}

// Coherent zero-copy producer whose share fits one register batch,
// pipelined like simple_send_piped (the source does not depend on the
// address).  The receiver publishes step j+1's destination as soon as it
// sees step j's taken, so wave 0 takes it while step j's stores drain
// instead of after step j's tail: two LDS words, by step parity, keep the
// other waves' read of step j's address clear of that write (the barrier
// of step j separates the read of a word from its next write).  Wave 0's
// first poll of the word goes out before step j+1's source loads: vector
// memory completes in issue order, so a poll issued after them would wait
// for all of them.
template <int SC, int ORD>
__device__ bool zc_send_piped(const ConnArgs& A, uint32_t w, Side& sd, uint64_t g0,
                              const uint8_t* src, uint64_t ticks, Shared& sh) {
  using O = Order<SC, ORD>;
  const uint64_t S = A.step_bytes;
  const uint32_t P = A.lanes;
  Batch b;
  batch_load<kPolNT, true>(b, src + sd.r.beg, chunk_len(sd, S, 0), S, P, w);
  if (wg_failed(sh, take_address<SC, ORD>(A, sd, ticks, sh.ptr[0]), A)) return false;
  if (threadIdx.x == 0) trace_step(A, sd, g0, 0, sh.ptr[0]);
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = g0 + j;
    uint8_t* p = reinterpret_cast<uint8_t*>(sh.ptr[j & 1]);
    const uint32_t L = chunk_len(sd, S, j);
    jitter(sd, g, 0);
    batch_store<O::kShared, true>(b, p, L, S, P, w);
    lane_tail<kPolNT, O::kShared, true>(src + sd.r.beg + j * S, p, L, S, P, w);
    compiler_fence();  // the next loads issue after these stores: vmcnt counts on that
    uint32_t err = 0;
    if (j + 1 < sd.r.k) {
      uint64_t first = 0;
      if (threadIdx.x < 64) first = ld_u64<SC>(&sd.tx->ptrx);
      batch_load<kPolNT, true>(b, src + sd.r.beg + (j + 1) * S, chunk_len(sd, S, j + 1), S, P, w);
      err = take_address<SC, ORD>(A, sd, ticks, sh.ptr[(j + 1) & 1], first);
      if (!err && threadIdx.x == 0) trace_step(A, sd, g + 1, 0, sh.ptr[(j + 1) & 1]);
      wait_vmcnt<kUnroll>();
    } else {
      wait_vmcnt<0>();
    }
    jitter(sd, g, 1);
    if (wg_failed(sh, err, A)) return false;
    if (threadIdx.x == 0) {
      trace_step(A, sd, g, 1, g + 1);
      st_u64<SC>(&sd.rx->tail, g + 1);
    }
  }
  return true;
}

// Producer: take the published destination, clear the word, write the chunk
// straight there, release, tail = g+1.
template <int SC, int ORD, bool AL>
__device__ bool zc_send(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t g0,
                        const uint8_t* src, uint64_t ticks, Shared& sh) {
  using O = Order<SC, ORD>;
  const uint64_t S = A.step_bytes;
  if constexpr (ORD == kOrdCoherent) {
    if (lane_blocks<true>(S, A.lanes) <= kUnroll)
      return zc_send_piped<SC, ORD>(A, w, sd, g0, src, ticks, sh);
  }
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = g0 + j;
    if (wg_failed(sh, take_address<SC, ORD>(A, sd, ticks, sh.ptr[0]), A)) return false;
    if (threadIdx.x == 0) trace_step(A, sd, g, 0, sh.ptr[0]);
    jitter(sd, g, 0);
    lane_copy<kPolNT, O::kShared, true>(src + sd.r.beg + j * S, reinterpret_cast<uint8_t*>(sh.ptr[0]),
                                  chunk_len(sd, S, j), S, A.lanes, w);
    O::release();
    jitter(sd, g, 1);
    if (wg_failed(sh, 0, A)) return false;
    if (threadIdx.x == 0) {
      trace_step(A, sd, g, 1, g + 1);
      st_u64<SC>(&sd.rx->tail, g + 1);
    }
  }
  return true;
}

// ------------------------------------------------------- zero-copy direct
// The destination is known before the launch ("zero copy" second kind on the
// transfer page): no ptrExchange.  The producer writes step j's chunk at its
// own offset of B, releases and publishes tail = g+1; pipelined like the
// other producers when its share of a step fits one register batch.
template <int SC, int ORD, bool AL>
__device__ bool zcd_send(const ConnArgs& A, uint32_t w, Side& sd, uint64_t g0,
                         const uint8_t* src, uint8_t* dst, uint64_t ticks, Shared& sh) {
  using O = Order<SC, ORD>;
  const uint64_t S = A.step_bytes;
  const uint32_t P = A.lanes;
  if (ORD == kOrdCoherent && lane_blocks<true>(S, P) <= kUnroll) {
    Batch b;
    batch_load<kPolNT, true>(b, src + sd.r.beg, chunk_len(sd, S, 0), S, P, w);
    for (uint64_t j = 0; j < sd.r.k; ++j) {
      const uint64_t g = g0 + j;
      uint8_t* p = dst + sd.r.beg + j * S;
      const uint32_t L = chunk_len(sd, S, j);
      if (threadIdx.x == 0) trace_step(A, sd, g, 0, reinterpret_cast<uint64_t>(p));
      jitter(sd, g, 0);
      batch_store<O::kShared, true>(b, p, L, S, P, w);
      lane_tail<kPolNT, O::kShared, true>(src + sd.r.beg + j * S, p, L, S, P, w);
      compiler_fence();  // the next loads issue after these stores: vmcnt counts on that
      if (j + 1 < sd.r.k) {
        batch_load<kPolNT, true>(b, src + sd.r.beg + (j + 1) * S, chunk_len(sd, S, j + 1), S, P, w);
        wait_vmcnt<kUnroll>();
      } else {
        wait_vmcnt<0>();
      }
      jitter(sd, g, 1);
      if (wg_failed(sh, 0, A)) return false;
      if (threadIdx.x == 0) {
        trace_step(A, sd, g, 1, g + 1);
        st_u64<SC>(&sd.rx->tail, g + 1);
      }
    }
    return true;
  }
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = g0 + j;
    if (threadIdx.x == 0) trace_step(A, sd, g, 0, reinterpret_cast<uint64_t>(dst + sd.r.beg + j * S));
    jitter(sd, g, 0);
    lane_copy<kPolNT, O::kShared, true>(src + sd.r.beg + j * S, dst + sd.r.beg + j * S,
                                        chunk_len(sd, S, j), S, P, w);
    O::release();
    jitter(sd, g, 1);
    if (wg_failed(sh, 0, A)) return false;
    if (threadIdx.x == 0) {
      trace_step(A, sd, g, 1, g + 1);
      st_u64<SC>(&sd.rx->tail, g + 1);
    }
  }
  return true;
}

// The launch's messages of one connection, repeated `iters` times.
template <int MAXB>
struct MsgList {
  const MsgDesc* msgs;
  uint32_t n;
  uint64_t nbytes;
  __device__ uint32_t count() const { return n ? n : 1u; }
  __device__ MsgDesc at(uint32_t i) const { return n ? msgs[i] : MsgDesc{0, nbytes}; }
};

// Walks the steps of a channel over every message of the launch, in order.
template <int MAXB>
struct StepCursor {
  uint32_t rep, mi;
  uint64_t j, off;
  Range r;
  bool done;
  __device__ void load(const MsgList<MAXB>& L, const ConnArgs& A, uint32_t c) {
    const MsgDesc md = L.at(mi);
    off = md.off;
    r = chan_range(md.len, A.nch, c, A.step_bytes);
  }
  // Positions on the first step at or after (rep, mi, j).
  __device__ void settle(const MsgList<MAXB>& L, const ConnArgs& A, uint32_t c, uint32_t iters) {
    while (!done && j >= r.k) {
      j = 0;
      if (++mi == L.count()) {
        mi = 0;
        if (++rep == iters) {
          done = true;
          return;
        }
      }
      load(L, A, c);
    }
  }
};

// Steps of channel c over every message of the launch.
template <int MAXB, int NMSG>
__device__ uint64_t launch_steps(const ConnArgs& A, uint32_t c, const RunArgs<MAXB, NMSG>& args) {
  const MsgList<MAXB> L{args.msgs, args.nmsgs, A.nbytes};
  uint64_t per_rep = 0;
  for (uint32_t i = 0; i < L.count(); ++i) per_rep += chan_range(L.at(i).len, A.nch, c, A.step_bytes).k;
  return per_rep * args.iters;
}

// Receiver of one lane, run by one thread: publish the destination of the
// next step (the base of its chunk in B) whenever the word is clear;
// complete steps once tail passes them by publishing head.
template <int SC, int ORD, int MAXB, int NMSG>
__device__ void zc_recv(const ConnArgs& A, uint32_t c, Side& sd, const RunArgs<MAXB, NMSG>& args,
                        uint64_t ticks) {
  using O = Order<SC, ORD>;
  const MsgList<MAXB> L{args.msgs, args.nmsgs, A.nbytes};
  const uint64_t S = A.step_bytes;
  const uint64_t total = launch_steps(A, c, args);
  StepCursor<MAXB> cur{0, 0, 0, 0, Range{0, 0, 0}, total == 0};
  if (!cur.done) {
    cur.load(L, A, c);
    cur.settle(L, A, c, args.iters);
  }
  uint64_t ndone = 0, npub = 0;
  Deadline dl(ticks, A.status);
  // The word is clear when a launch starts: each earlier launch on the
  // connection ended with every published address taken, and after a failed
  // one every later launch returns on entry (its failure mirror is set) and
  // the host refuses new runs.  So the first address goes out without a
  // poll, one round trip earlier.
  bool clear = true;
  while (ndone < total) {
    bool moved = false;
    if (!cur.done && (clear || ld_u64<SC>(&sd.tx->ptrx) == 0)) {
      clear = false;
      const uint64_t addr = reinterpret_cast<uint64_t>(A.dst + cur.off + cur.r.beg + cur.j * S);
      jitter(sd, sd.base + npub, 0);
      trace_step(A, sd, sd.base + npub++, 0, addr);
      O::release();
      st_u64<SC>(&sd.tx->ptrx, addr);
      ++cur.j;
      cur.settle(L, A, c, args.iters);
      moved = true;
    }
    const uint64_t t = ld_u64<SC>(&sd.rx->tail);
    if (t > sd.base + ndone) {
      O::acquire();
      for (uint64_t q = sd.base + ndone; sd.tr != nullptr && q < t; ++q) trace_step(A, sd, q, 1, t);
      st_u64<SC>(&sd.tx->head, t);
      ndone = t - sd.base;
      moved = true;
    }
    if (moved) {
      dl = Deadline(ticks, A.status);
    } else {
      const uint32_t e = dl.expired();
      if (e) {
        raise_err(A, e);
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

// Receiver of one lane of zero-copy direct, run by one thread: answer tail
// with head until the launch's last step on the channel has landed.
template <int SC, int ORD, int MAXB, int NMSG>
__device__ void zcd_recv(const ConnArgs& A, uint32_t c, Side& sd, const RunArgs<MAXB, NMSG>& args,
                         uint64_t ticks) {
  const uint64_t end = sd.base + launch_steps(A, c, args);
  uint64_t done = sd.base;
  Deadline dl(ticks, A.status);
  while (done < end) {
    const uint64_t t = ld_u64<SC>(&sd.rx->tail);
    if (t > done) {
      Order<SC, ORD>::acquire();
      for (uint64_t q = done; sd.tr != nullptr && q < t; ++q) {
        trace_step(A, sd, q, 0, t);
        trace_step(A, sd, q, 1, t);
      }
      jitter(sd, t, 1);
      done = t;
      st_u64<SC>(&sd.tx->head, t);
      dl = Deadline(ticks, A.status);
      continue;
    }
    const uint32_t e = dl.expired();
    if (e) {
      raise_err(A, e);
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// ------------------------------------------------------------------ kernels
// XCD this wave runs on (hardware register XCC_ID; a read, no memory access).
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 7u;
}

// Logical workgroup of this block.  A dispatch's blocks are dealt
// round-robin to the 8 XCDs, but each hardware queue starts the deal at an
// XCD of its own: block b runs on XCD (b + r) % 8, with r fixed per queue
// (measured 0, 5, 6 and 7 on different streams of one process).  Remap 1
// takes p = b; remap 2, which the host enables only once it has seen that
// deal on this device (xcc_rotation_ok), takes p = (b + r) mod total with r
// read back from the block's own XCD id, so that p % 8 is its XCD
// whichever stream launched it.  Both are permutations of the grid, the
// second because r is the same for every block of the dispatch.  Then (the
// host pads the grid to a multiple of 16; logical ids past the real
// workgroups exit at once) position p % 8 serves the total/16 consecutive
// pairs starting at (p % 8) * total/16: its first total/16 blocks are their
// producers, the rest their consumers.  A pair then shares one XCD,
// producers spread evenly over the XCDs and over each XCD's dispatch order,
// and with remap 2 a channel's XCD, on which the latency of its polled
// lines depends, does not change with the stream.
__device__ __forceinline__ uint32_t logical_wg(uint32_t remap, uint32_t total) {
  const uint32_t b0 = blockIdx.x;
  if (!remap) return b0;
  uint32_t b = b0;
  if (remap == 2) {
    b += (xcc_id() - b0) & 7u;
    if (b >= total) b -= total;
  }
  const uint32_t half = total / 16u, s = b / 8u;
  return 2u * ((b % 8u) * half + s % half) + s / half;
}

// Debug variant: the block takes logical workgroup `local` of connection A
// for this launch.  Were the remap ever to hand one logical workgroup to two
// blocks, another would go unserved and the pair's slot hand-backs would no
// longer cover each other's bytes; the second claimer raises
// XFER_ERR_INTERNAL and leaves.  Returns whether the block may go on.  Every
// thread of the block must call it.
template <bool DBG>
__device__ __forceinline__ bool claim_wg(const ConnArgs& A, uint32_t local, Shared& sh) {
  if constexpr (!DBG) {
    return true;
  } else {
    if (A.claims == nullptr) return true;
    if (threadIdx.x == 0) {
      const uint64_t prev = __hip_atomic_exchange(&A.claims[local], A.launch_seq, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      if (prev == A.launch_seq) {
        sh.err = XFER_ERR_INTERNAL;
        raise_err(A, XFER_ERR_INTERNAL);
      }
    }
    __syncthreads();
    return sh.err == 0;
  }
}

// Records the XCD id of each block (the host's check of the deal).
__global__ void xcc_probe_kernel(uint32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

// Zero-copy launches (through ptrExchange, or with the destination known):
// blocks [0, rx_wgs) are receiver workgroups, in which the first
// kRxLanesPerWave threads of each wave are the receivers of one lane each
// (a connection's lanes in channel-major order); they are dispatched first,
// since every producer waits for its first address.  The blocks after them
// are the producers, one workgroup per lane, in the connections' order.  A
// receiver moves a few words per step and no payload, so it takes a thread
// rather than a workgroup: every CU the launch occupies beyond the
// receivers' few copies payload.
// With grouping (xcd_remap != 0) the host pads both regions to multiples
// of 8 blocks; blocks dealt to one XCD then share their index mod 8, and
// XCD-slot x takes the x-th eighth of the producers in order, so the lanes
// of a channel (and of a connection, as far as they fill an eighth) run on
// one XCD, as the paired layout of the other protocols keeps a pair.
template <int PROTO, int SC, int ORD, bool AL, int MAXB, int NMSG, bool DBG>
__device__ void zero_copy_wg(const RunArgs<MAXB, NMSG>& args, Shared& sh) {
  const uint32_t b = blockIdx.x;
  const uint64_t ticks = args.timeout_ticks;
  uint32_t ci = 0;
  if (b < args.rx_wgs) {
    if constexpr (MAXB > 1) {
      while (ci + 1 < args.nconn && b >= args.conn[ci + 1].rx_begin) ++ci;
    }
    const ConnArgs& A = args.conn[ci];
    const uint32_t r = b - A.rx_begin, nl = A.nch * A.lanes;
    if (r >= zc_receiver_wgs(A.nch, A.lanes, blockDim.x)) return;  // padding of the region
    if (!claim_wg<DBG>(A, nl + r, sh)) return;  // (receiver ids follow the producers')
    const uint32_t li = threadIdx.x % 64u;
    const uint32_t t = (r * (blockDim.x / 64u) + threadIdx.x / 64u) * kRxLanesPerWave + li;
    if (li >= kRxLanesPerWave || t >= nl || !((A.roles >> 1) & 1u))
      return;  // no lane, or receivers switched off
    const uint32_t c = t / A.lanes, w = t % A.lanes;
    Side sd = make_side<DBG, false>(A, c, w, false, SC);
    if (sd.dead) return;
    if constexpr (PROTO == kProtoZC)
      zc_recv<SC, ORD, MAXB, NMSG>(A, c, sd, args, ticks);
    else
      zcd_recv<SC, ORD, MAXB, NMSG>(A, c, sd, args, ticks);
    return;
  }
  uint32_t pw = b - args.rx_wgs;
  if (args.xcd_remap) {
    const uint32_t eighth = (args.total_wgs - args.rx_wgs) / 8u;
    pw = (pw % 8u) * eighth + pw / 8u;
  }
  if constexpr (MAXB > 1) {
    while (ci + 1 < args.nconn && pw >= args.conn[ci + 1].wg_begin) ++ci;
  }
  const ConnArgs& A = args.conn[ci];
  const uint32_t local = pw - A.wg_begin;
  const uint32_t c = local / A.lanes, w = local % A.lanes;
  if (c >= A.nch) return;
  if (!claim_wg<DBG>(A, local, sh)) return;
  if (!(A.roles & 1u)) return;  // producers switched off for fault injection
  Side sd = make_side<DBG>(A, c, w, true, SC);
  if (sd.dead) return;
  const MsgList<MAXB> L{args.msgs, args.nmsgs, A.nbytes};
  uint64_t g0 = sd.base;
  for (uint32_t rep = 0; rep < args.iters; ++rep) {
    for (uint32_t mi = 0; mi < L.count(); ++mi) {
      const MsgDesc md = L.at(mi);
      sd.r = chan_range(md.len, A.nch, c, A.step_bytes);
      if (sd.r.k == 0) continue;
      bool ok;
      if constexpr (PROTO == kProtoZC)
        ok = zc_send<SC, ORD, AL>(A, c, w, sd, g0, A.src + md.off, ticks, sh);
      else
        ok = zcd_send<SC, ORD, AL>(A, w, sd, g0, A.src + md.off, A.dst + md.off, ticks, sh);
      if (!ok) return;
      g0 += sd.r.k;
    }
  }
}

template <int PROTO, int SC, int ORD, bool AL, int MAXB, int NMSG, bool DBG>
__global__ void __launch_bounds__(1024) run_kernel(RunArgs<MAXB, NMSG> args) {
  constexpr bool kStriped = PROTO == kProtoLLStriped;
  __shared__ Shared sh;
  if (threadIdx.x == 0) sh.err = 0;
  __syncthreads();
  if constexpr (PROTO == kProtoZC || PROTO == kProtoZCD) {
    zero_copy_wg<PROTO, SC, ORD, AL, MAXB, NMSG, DBG>(args, sh);
  } else {
    const uint32_t lw = logical_wg(args.xcd_remap, args.total_wgs);
    uint32_t ci = 0;
    if constexpr (MAXB > 1) {
      while (ci + 1 < args.nconn && lw >= args.conn[ci + 1].wg_begin) ++ci;
    }
    const ConnArgs& A = args.conn[ci];
    const uint32_t local = lw - A.wg_begin;
    const uint32_t pair = local >> 1, role = local & 1u;
    const uint32_t c = pair / A.lanes, w = pair % A.lanes;
    if (c >= A.nch) return;  // padding of a paired launch (its grid is a multiple of 16)
    if (!claim_wg<DBG>(A, local, sh)) return;
    if (!((A.roles >> role) & 1u)) return;  // side switched off for fault injection
    Side sd = make_side<DBG>(A, c, w, role == 0, SC);
    if (sd.dead) return;
    const uint64_t ticks = args.timeout_ticks;
    const MsgList<MAXB> L{args.msgs, args.nmsgs, A.nbytes};
    uint64_t g0 = sd.base;
    for (uint32_t rep = 0; rep < args.iters; ++rep) {
      for (uint32_t mi = 0; mi < L.count(); ++mi) {
        const MsgDesc md = L.at(mi);
        sd.r = chan_range(md.len, A.nch, c, A.step_bytes);
        if (sd.r.k == 0) continue;
        bool ok;
        if constexpr (PROTO == kProtoSimple)
          ok = role == 0 ? simple_send<SC, ORD, AL>(A, c, w, sd, g0, A.src + md.off, ticks, sh)
                         : simple_recv<SC, ORD, AL>(A, c, w, sd, g0, A.dst + md.off, ticks, sh);
        else
          ok = role == 0 ? ll_send<SC, ORD, AL, kStriped>(A, c, w, sd, g0, A.src + md.off, ticks, sh)
                         : ll_recv<SC, ORD, AL, kStriped>(A, c, w, sd, g0, A.dst + md.off, ticks, sh);
        if (!ok) return;
        g0 += sd.r.k;
      }
    }
    if constexpr (PROTO != kProtoSimple) {
      if (role == 0 && g0 != sd.base) ll_close<SC>(sd, g0);
    }
  }
}

// Endpoint X's action before it polls for a reply: load the source word of
// its next send (when there is one).
template <bool AL>
struct LoadNext {
  static constexpr bool kActive = true;
  const ConnArgs* F;
  const Side* fs;
  uint32_t w;
  bool more;
  NextWord* out;
  __device__ void operator()() const {
    *out = more ? ll_striped_first_word<AL>(*F, w, *fs, F->src) : NextWord{false, 0u};
  }
};

// Ping-pong: pair side 0 is endpoint X (send on fwd, then receive on rev),
// side 1 is endpoint Y (receive on fwd into b, then send b on rev).
template <int PROTO, int SC, int ORD, bool AL, bool DBG>
__global__ void __launch_bounds__(1024) ping_kernel(PingArgs args) {
  constexpr bool kStriped = PROTO == kProtoLLStriped;
  __shared__ Shared sh;
  if (threadIdx.x == 0) sh.err = 0;
  __syncthreads();
  const uint32_t lw = logical_wg(args.xcd_remap, args.total_wgs);
  const uint32_t pair = lw >> 1, side = lw & 1u;
  const ConnArgs& F = args.fwd;
  const ConnArgs& R = args.rev;
  const uint32_t c = pair / F.lanes, w = pair % F.lanes;
  if (c >= F.nch) return;
  if (!claim_wg<DBG>(F, lw, sh)) return;
  Side fs = make_side<DBG>(F, c, w, side == 0, SC);
  Side rs = make_side<DBG>(R, c, w, side == 1, SC);
  if (fs.dead || rs.dead) return;
  fs.r = chan_range(F.nbytes, F.nch, c, F.step_bytes);
  rs.r = chan_range(R.nbytes, R.nch, c, R.step_bytes);
  const uint64_t k = fs.r.k;
  if (k == 0) return;
  const uint64_t ticks = args.timeout_ticks;
  NextWord next{false, 0u};  // endpoint X's source word of its next send, loaded ahead
  for (uint32_t it = 0; it < args.iters; ++it) {
    const uint64_t gf = fs.base + it * k, gr = rs.base + it * k;
    bool ok;
    if (side == 0) {
      if constexpr (kStriped) {
        // the next round's source word is loaded before the reply's polls
        ok = ll_send_striped<SC, ORD, AL>(F, c, w, fs, gf, F.src, ticks, sh, &next);
        if (ok)
          ok = ll_recv_striped<SC, ORD, AL>(R, c, w, rs, gr, R.dst, ticks, sh,
                                            LoadNext<AL>{&F, &fs, w, it + 1 < args.iters, &next});
      } else if constexpr (PROTO != kProtoSimple) {
        ok = ll_send<SC, ORD, AL, kStriped>(F, c, w, fs, gf, F.src, ticks, sh) &&
             ll_recv<SC, ORD, AL, kStriped>(R, c, w, rs, gr, R.dst, ticks, sh);
      } else {
        ok = simple_send<SC, ORD, AL>(F, c, w, fs, gf, F.src, ticks, sh) &&
             simple_recv<SC, ORD, AL>(R, c, w, rs, gr, R.dst, ticks, sh);
      }
    } else {
      if constexpr (PROTO != kProtoSimple)
        ok = ll_recv<SC, ORD, AL, kStriped>(F, c, w, fs, gf, F.dst, ticks, sh) &&
             ll_send<SC, ORD, AL, kStriped>(R, c, w, rs, gr, R.src, ticks, sh);
      else
        ok = simple_recv<SC, ORD, AL>(F, c, w, fs, gf, F.dst, ticks, sh) &&
             simple_send<SC, ORD, AL>(R, c, w, rs, gr, R.src, ticks, sh);
    }
    if (!ok) return;
  }
  if constexpr (PROTO != kProtoSimple) {
    if (side == 0)
      ll_close<SC>(fs, fs.base + args.iters * k);
    else
      ll_close<SC>(rs, rs.base + args.iters * k);
  }
}

// --------------------------------------------------------- dispatch tables
template <int MAXB, int NMSG>
using RunFn = void (*)(RunArgs<MAXB, NMSG>);
using PingFn = void (*)(PingArgs);

template <int MAXB, int NMSG, int P, int SC, int ORD, bool DBG>
RunFn<MAXB, NMSG> pick_run_al(bool al) {
  return al ? run_kernel<P, SC, ORD, true, MAXB, NMSG, DBG>
            : run_kernel<P, SC, ORD, false, MAXB, NMSG, DBG>;
}

template <int MAXB, int NMSG, int P, int SC, bool DBG>
RunFn<MAXB, NMSG> pick_run_ord(int ord, bool al) {
  return ord == kOrdFenced ? pick_run_al<MAXB, NMSG, P, SC, kOrdFenced, DBG>(al)
                           : pick_run_al<MAXB, NMSG, P, SC, kOrdCoherent, DBG>(al);
}

template <int MAXB, int NMSG, int P, bool DBG>
RunFn<MAXB, NMSG> pick_run_dbg(const Variant& v) {
  return v.scope == kScopeSystem
             ? pick_run_ord<MAXB, NMSG, P, kScopeSystem, DBG>(v.ordering, v.aligned)
             : pick_run_ord<MAXB, NMSG, P, kScopeAgent, DBG>(v.ordering, v.aligned);
}

template <int MAXB, int NMSG, int P>
RunFn<MAXB, NMSG> pick_run_sc(const Variant& v) {
  return v.debug ? pick_run_dbg<MAXB, NMSG, P, true>(v) : pick_run_dbg<MAXB, NMSG, P, false>(v);
}

template <int MAXB, int NMSG>
RunFn<MAXB, NMSG> pick_run(const Variant& v) {
  switch (v.proto) {
    case kProtoSimple: return pick_run_sc<MAXB, NMSG, kProtoSimple>(v);
    case kProtoLL: return pick_run_sc<MAXB, NMSG, kProtoLL>(v);
    case kProtoLLStriped: return pick_run_sc<MAXB, NMSG, kProtoLLStriped>(v);
    case kProtoZCD: return pick_run_sc<MAXB, NMSG, kProtoZCD>(v);
    default: return pick_run_sc<MAXB, NMSG, kProtoZC>(v);
  }
}

template <int P, int SC, int ORD, bool DBG>
PingFn pick_ping_al(bool al) {
  return al ? ping_kernel<P, SC, ORD, true, DBG> : ping_kernel<P, SC, ORD, false, DBG>;
}

template <int P, int SC, bool DBG>
PingFn pick_ping_ord(int ord, bool al) {
  return ord == kOrdFenced ? pick_ping_al<P, SC, kOrdFenced, DBG>(al)
                           : pick_ping_al<P, SC, kOrdCoherent, DBG>(al);
}

template <int P, bool DBG>
PingFn pick_ping_dbg(const Variant& v) {
  return v.scope == kScopeSystem ? pick_ping_ord<P, kScopeSystem, DBG>(v.ordering, v.aligned)
                                 : pick_ping_ord<P, kScopeAgent, DBG>(v.ordering, v.aligned);
}

template <int P>
PingFn pick_ping_sc(const Variant& v) {
  return v.debug ? pick_ping_dbg<P, true>(v) : pick_ping_dbg<P, false>(v);
}

PingFn pick_ping(const Variant& v) {
  return v.proto == kProtoLL          ? pick_ping_sc<kProtoLL>(v)
         : v.proto == kProtoLLStriped ? pick_ping_sc<kProtoLLStriped>(v)
                                      : pick_ping_sc<kProtoSimple>(v);
}

}  // namespace

// hipLaunchKernel and hipLaunchCooperativeKernel report this launch's own
// status (no sticky error state).
template <typename Fn, typename Args>
static hipError_t launch(Fn fn, const Args& a, uint32_t grid, int block, hipStream_t s,
                         bool coop = false) {
  void* kargs[] = {const_cast<Args*>(&a)};
  const void* f = reinterpret_cast<const void*>(fn);
  return coop ? hipLaunchCooperativeKernel(f, dim3(grid), dim3(block), kargs, 0, s)
              : hipLaunchKernel(f, dim3(grid), dim3(block), kargs, 0, s);
}

hipError_t launch_run1(const Variant& v, const RunOne& a, int block, hipStream_t s, bool coop) {
  return launch(pick_run<1, 1>(v), a, a.total_wgs, block, s, coop);
}

hipError_t launch_runL(const Variant& v, const RunList& a, int block, hipStream_t s, bool coop) {
  return launch(pick_run<1, kMaxMsgs>(v), a, a.total_wgs, block, s, coop);
}

hipError_t launch_runB(const Variant& v, const RunBatch& a, int block, hipStream_t s, bool coop) {
  return launch(pick_run<16, 1>(v), a, a.total_wgs, block, s, coop);
}

hipError_t launch_ping(const Variant& v, const PingArgs& a, int block, hipStream_t s, bool coop) {
  return launch(pick_ping(v), a, a.total_wgs, block, s, coop);
}

// Whether the current device deals blocks to 8 XCDs in strict rotation on
// every stream: a probe grid on each of several streams (more than the
// hardware queues a process gets) must see XCD (x0 + b) % 8 at block b,
// with x0 in 0..7.  A device partitioned into fewer XCDs, or any other
// deal, fails the check.
hipError_t xcc_rotation_ok(bool* ok) {
  constexpr int kStreams = 8, kBlocks = 64;
  *ok = false;
  uint32_t* d = nullptr;
  hipError_t e = hipMalloc(&d, sizeof(uint32_t) * kStreams * kBlocks);
  if (e != hipSuccess) return e;
  hipStream_t st[kStreams] = {};
  int made = 0;
  for (; made < kStreams && e == hipSuccess; ++made) e = hipStreamCreate(&st[made]);
  if (e != hipSuccess) --made;
  for (int i = 0; i < made && e == hipSuccess; ++i)
    e = launch(xcc_probe_kernel, d + i * kBlocks, kBlocks, 64, st[i]);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  uint32_t h[kStreams * kBlocks];
  if (e == hipSuccess) e = hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost);
  bool good = e == hipSuccess && made == kStreams;
  for (int i = 0; good && i < kStreams; ++i) {
    const uint32_t x0 = h[i * kBlocks];
    for (int b = 0; good && b < kBlocks; ++b) good = x0 < 8u && h[i * kBlocks + b] == (x0 + b) % 8u;
  }
  for (int i = 0; i < made; ++i) (void)hipStreamDestroy(st[i]);
  (void)hipFree(d);
  *ok = good;
  return e;
}

hipError_t max_resident(const Variant& v, int kind, int block, int* wgs) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // kind: 0 one transfer, 1 a batch, 2 the ping-pong, 3 a message list
  const void* fn = kind == 0   ? reinterpret_cast<const void*>(pick_run<1, 1>(v))
                   : kind == 1 ? reinterpret_cast<const void*>(pick_run<16, 1>(v))
                   : kind == 3 ? reinterpret_cast<const void*>(pick_run<1, kMaxMsgs>(v))
                               : reinterpret_cast<const void*>(pick_ping(v));
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0);
  if (e != hipSuccess) return e;
  *wgs = per_cu * cus;
  return hipSuccess;
}

}  // namespace xfer
