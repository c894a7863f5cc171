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
// Memory ordering on gfx950.  The eight XCDs each have their own L2; for
// device memory an agent-scope release writes back dirty L2 lines and an
// agent-scope acquire invalidates them.  A workgroup barrier does not wait
// for the other waves' stores to reach L2, so a release by one thread after
// the barrier would not cover them: every wave issues its own release fence
// before the barrier that precedes the counter store, and every wave polls
// the counter itself and issues its own acquire fence before it reads the
// data.  Host FIFOs (or host control words) use system scope throughout.
// Every wait is bounded by the connection's timeout and also watches the
// host abort word, so every wave reaches the end of the kernel.

#include "xfer_internal.h"
#include "xfer.h"

namespace xfer {
namespace {

constexpr int kUnroll = 8;     // 16-byte vectors in flight per thread in the copy loop
constexpr int kLLUnroll = 4;   // LL lines polled together per thread

template <int SC>
__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) {
  if constexpr (SC == kScopeSystem)
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Every lane loads the same word (one request per wave); the value is made
// wave-uniform explicitly.
template <int SC>
__device__ __forceinline__ uint64_t wave_load(const uint64_t* p) {
  const uint64_t v = ld_u64<SC>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ void raise_err(Status* st, uint32_t code) {
  __hip_atomic_store(&st->err, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Bound of one wait: wall-clock ticks (s_memrealtime) plus the host abort word.
struct Deadline {
  uint64_t start, ticks;
  Status* st;
  uint32_t n;
  __device__ Deadline(uint64_t t, Status* s) : start(wall_clock64()), ticks(t), st(s), n(0) {}
  __device__ __forceinline__ uint32_t expired() {
    if (((++n) & 255u) == 0u &&
        __hip_atomic_load(&st->abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM))
      return XFER_ERR_ABORTED;
    if (wall_clock64() - start > ticks) return XFER_ERR_TIMEOUT;
    return 0;
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

// Lane w's part of a chunk of L <= S bytes.  Each lane owns a fixed slice of
// the slot, cut from the full step size S (16-byte granular), so a slot byte
// is always written and drained by the same lane pair and one lane's head
// covers every byte its producer will overwrite; a short chunk just leaves
// the upper slices empty.
__device__ __forceinline__ void lane_share16(uint64_t L, uint64_t S, uint32_t P, uint32_t w,
                                             uint64_t& lo, uint64_t& hi) {
  const uint64_t sub = (((S + P - 1) / P) + 15) & ~uint64_t(15);
  lo = min(L, static_cast<uint64_t>(w) * sub);
  hi = min(L, static_cast<uint64_t>(w + 1) * sub);
}

// Lane w's lines of an LL chunk of L <= S payload bytes (one line per 4
// bytes), again a fixed slice of the slot's S / 4 lines.
__device__ __forceinline__ void lane_share_lines(uint64_t L, uint64_t S, uint32_t P, uint32_t w,
                                                 uint64_t& lo, uint64_t& hi) {
  const uint64_t nl = (L + 3) / 4;
  const uint64_t sub = (S / 4 + P - 1) / P;
  lo = min(nl, static_cast<uint64_t>(w) * sub);
  hi = min(nl, static_cast<uint64_t>(w + 1) * sub);
}

// Workgroup copy of n bytes, both ends 16-byte aligned: 16-byte vector
// loads, kUnroll in flight per thread, then the stores; ragged tail bytewise.
// The pointers are deliberately not __restrict__: with it the compiler sinks
// each load next to its store and only one vector is in flight per thread.
__device__ __forceinline__ void copy_aligned(const uint8_t* s, uint8_t* d, uint64_t n, uint32_t tid,
                                             uint32_t nthr) {
  const uint4* s4 = reinterpret_cast<const uint4*>(s);
  uint4* d4 = reinterpret_cast<uint4*>(d);
  const uint64_t nv = n >> 4;
  const uint64_t stride = static_cast<uint64_t>(nthr) * kUnroll;
  uint64_t i = tid;
  for (; i + static_cast<uint64_t>(kUnroll - 1) * nthr < nv; i += stride) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = s4[i + static_cast<uint64_t>(u) * nthr];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) d4[i + static_cast<uint64_t>(u) * nthr] = r[u];
  }
  for (; i < nv; i += nthr) d4[i] = s4[i];
  const uint64_t done = nv << 4;
  if (tid < n - done) d[done + tid] = s[done + tid];
}

__device__ __forceinline__ void copy_bytes(const uint8_t* __restrict__ s, uint8_t* __restrict__ d,
                                           uint64_t n, uint32_t tid, uint32_t nthr) {
  for (uint64_t i = tid; i < n; i += nthr) d[i] = s[i];
}

template <bool AL>
__device__ __forceinline__ void wg_copy(const uint8_t* s, uint8_t* d, uint64_t n) {
  if constexpr (AL)
    copy_aligned(s, d, n, threadIdx.x, blockDim.x);
  else
    copy_bytes(s, d, n, threadIdx.x, blockDim.x);
}

// Per-workgroup state of one side of a lane across the messages of a launch.
struct Side {
  LaneCtrl* lc;
  uint64_t base;    // step counter at launch start (own counter: tail or head)
  uint64_t seen;    // last observed peer counter (wave-uniform)
  Range r;
};

__device__ __forceinline__ Side make_side(const ConnArgs& A, uint32_t c, uint32_t w, bool producer,
                                          int sc) {
  Side s;
  s.lc = A.ctrl + static_cast<uint64_t>(c) * A.lanes + w;
  s.r = chan_range(A.nbytes, A.nch, c, A.step_bytes);
  // A side is the only writer of its own counter, and the previous launch
  // that wrote it has completed, so a plain coherent load reads it.
  const uint64_t* own = producer ? &s.lc->tail : &s.lc->head;
  s.base = sc == kScopeSystem ? wave_load<kScopeSystem>(own) : wave_load<kScopeAgent>(own);
  s.seen = 0;
  return s;
}

// Shared by the waves of a workgroup: the first failure seen by any wave.
struct Shared {
  uint32_t err;
  uint32_t pad;
  uint64_t ptr;
};

__device__ __forceinline__ bool wg_failed(Shared& sh, uint32_t local_err, Status* st) {
  if (local_err) sh.err = local_err;
  __syncthreads();
  const uint32_t e = sh.err;
  if (e && threadIdx.x == 0) raise_err(st, e);
  return e != 0;
}

// ------------------------------------------------------------------ SIMPLE
// Producer of message m: for each step g, wait for credit g - head < nslots,
// write the chunk into slot g mod nslots, release, tail = g+1.
template <int SC, bool AL>
__device__ bool simple_send(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t m,
                            const uint8_t* src, uint64_t ticks, Shared& sh) {
  const uint64_t S = A.step_bytes;
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = sd.base + m * sd.r.k + j;
    uint32_t err = 0;
    if (g - sd.seen >= A.nslots) {
      Deadline dl(ticks, A.status);
      uint64_t h;
      while (g - (h = wave_load<SC>(&sd.lc->head)) >= A.nslots) {
        if ((err = dl.expired())) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (!err) {
        fence_acquire<SC>();  // the consumer's reads of the slot precede our writes
        sd.seen = h;
      }
    }
    if (!err) {
      const uint64_t L = min(S, sd.r.len - j * S);
      uint64_t lo, hi;
      lane_share16(L, S, A.lanes, w, lo, hi);
      uint8_t* slot = A.fifo + (static_cast<uint64_t>(c) * A.nslots + g % A.nslots) * A.slot_bytes;
      wg_copy<AL>(src + sd.r.beg + j * S + lo, slot + lo, hi - lo);
      fence_release<SC>();
    }
    if (wg_failed(sh, err, A.status)) return false;
    if (threadIdx.x == 0) st_u64<SC>(&sd.lc->tail, g + 1);
  }
  return true;
}

// Consumer of message m: wait for tail > g, acquire, copy the slot out,
// release, head = g+1.
template <int SC, bool AL>
__device__ bool simple_recv(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t m,
                            uint8_t* dst, uint64_t ticks, Shared& sh) {
  const uint64_t S = A.step_bytes;
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = sd.base + m * sd.r.k + j;
    uint32_t err = 0;
    if (sd.seen <= g) {
      Deadline dl(ticks, A.status);
      uint64_t t;
      while ((t = wave_load<SC>(&sd.lc->tail)) <= g) {
        if ((err = dl.expired())) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (!err) {
        fence_acquire<SC>();
        sd.seen = t;
      }
    }
    if (!err) {
      const uint64_t L = min(S, sd.r.len - j * S);
      uint64_t lo, hi;
      lane_share16(L, S, A.lanes, w, lo, hi);
      const uint8_t* slot =
          A.fifo + (static_cast<uint64_t>(c) * A.nslots + g % A.nslots) * A.slot_bytes;
      wg_copy<AL>(slot + lo, dst + sd.r.beg + j * S + lo, hi - lo);
      fence_release<SC>();  // our slot reads complete before the slot is handed back
    }
    if (wg_failed(sh, err, A.status)) return false;
    if (threadIdx.x == 0) st_u64<SC>(&sd.lc->head, g + 1);
  }
  return true;
}

// ---------------------------------------------------------------------- LL
// Line = {4 payload bytes, flag = g+1}, stored and loaded as one 64-bit
// access; the last word of a chunk is zero-padded.
template <bool AL>
__device__ __forceinline__ uint32_t ll_src_word(const uint8_t* p, uint64_t L, uint64_t line) {
  const uint64_t off = line * 4;
  if (AL && off + 4 <= L) return *reinterpret_cast<const uint32_t*>(p + off);
  uint32_t v = 0;
  for (uint64_t b = 0; b < 4 && off + b < L; ++b) v |= static_cast<uint32_t>(p[off + b]) << (8 * b);
  return v;
}

template <bool AL>
__device__ __forceinline__ void ll_dst_word(uint8_t* p, uint64_t L, uint64_t line, uint32_t v) {
  const uint64_t off = line * 4;
  if (AL && off + 4 <= L) {
    *reinterpret_cast<uint32_t*>(p + off) = v;
    return;
  }
  for (uint64_t b = 0; b < 4 && off + b < L; ++b) p[off + b] = static_cast<uint8_t>(v >> (8 * b));
}

template <int SC, bool AL>
__device__ bool ll_send(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t m,
                        const uint8_t* src, uint64_t ticks, Shared& sh) {
  const uint64_t S = A.step_bytes;
  uint32_t err = 0;
  for (uint64_t j = 0; j < sd.r.k && !err; ++j) {
    const uint64_t g = sd.base + m * sd.r.k + j;
    if (g - sd.seen >= A.nslots) {
      Deadline dl(ticks, A.status);
      uint64_t h;
      while (g - (h = wave_load<SC>(&sd.lc->head)) >= A.nslots) {
        if ((err = dl.expired())) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (err) break;
      fence_acquire<SC>();
      sd.seen = h;
    }
    const uint64_t L = min(S, sd.r.len - j * S);
    uint64_t lo, hi;
    lane_share_lines(L, S, A.lanes, w, lo, hi);
    uint64_t* lines = reinterpret_cast<uint64_t*>(
        A.fifo + (static_cast<uint64_t>(c) * A.nslots + g % A.nslots) * A.slot_bytes);
    const uint8_t* s = src + sd.r.beg + j * S;
    const uint64_t flag = static_cast<uint64_t>(static_cast<uint32_t>(g + 1)) << 32;
    for (uint64_t i = lo + threadIdx.x; i < hi; i += blockDim.x)
      st_u64<SC>(&lines[i], flag | ll_src_word<AL>(s, L, i));
  }
  return !wg_failed(sh, err, A.status);
}

template <int SC, bool AL>
__device__ bool ll_recv(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t m,
                        uint8_t* dst, uint64_t ticks, Shared& sh) {
  const uint64_t S = A.step_bytes;
  const uint32_t nthr = blockDim.x;
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = sd.base + m * sd.r.k + j;
    const uint32_t want = static_cast<uint32_t>(g + 1);
    const uint64_t L = min(S, sd.r.len - j * S);
    uint64_t lo, hi;
    lane_share_lines(L, S, A.lanes, w, lo, hi);
    const uint64_t* lines = reinterpret_cast<const uint64_t*>(
        A.fifo + (static_cast<uint64_t>(c) * A.nslots + g % A.nslots) * A.slot_bytes);
    uint8_t* d = dst + sd.r.beg + j * S;
    uint32_t err = 0;
    for (uint64_t i0 = lo + threadIdx.x; i0 < hi && !err; i0 += static_cast<uint64_t>(kLLUnroll) * nthr) {
      uint64_t v[kLLUnroll];
      bool pend = false;
#pragma unroll
      for (int u = 0; u < kLLUnroll; ++u) {
        const uint64_t i = i0 + static_cast<uint64_t>(u) * nthr;
        v[u] = i < hi ? ld_u64<SC>(&lines[i]) : (static_cast<uint64_t>(want) << 32);
        pend |= static_cast<uint32_t>(v[u] >> 32) != want;
      }
      if (pend) {
        Deadline dl(ticks, A.status);
        while (pend) {
          pend = false;
#pragma unroll
          for (int u = 0; u < kLLUnroll; ++u) {
            if (static_cast<uint32_t>(v[u] >> 32) != want) {
              v[u] = ld_u64<SC>(&lines[i0 + static_cast<uint64_t>(u) * nthr]);
              pend |= static_cast<uint32_t>(v[u] >> 32) != want;
            }
          }
          if (pend && (err = dl.expired())) break;
        }
      }
      if (!err) {
#pragma unroll
        for (int u = 0; u < kLLUnroll; ++u) {
          const uint64_t i = i0 + static_cast<uint64_t>(u) * nthr;
          if (i < hi) ll_dst_word<AL>(d, L, i, static_cast<uint32_t>(v[u]));
        }
      }
    }
    fence_release<SC>();  // our line reads complete before the slot is handed back
    if (wg_failed(sh, err, A.status)) return false;
    if (threadIdx.x == 0) st_u64<SC>(&sd.lc->head, g + 1);
  }
  return true;
}

// LL has no polled tail: the producer records its final step count once.
template <int SC>
__device__ __forceinline__ void ll_close(Side& sd, uint64_t iters) {
  if (threadIdx.x == 0) st_u64<SC>(&sd.lc->tail, sd.base + iters * sd.r.k);
}

// --------------------------------------------------------------- zero-copy
// Producer: take the published destination, clear the word, write the chunk
// straight there, release, tail = g+1.
template <int SC, bool AL>
__device__ bool zc_send(const ConnArgs& A, uint32_t c, uint32_t w, Side& sd, uint64_t m,
                        const uint8_t* src, uint64_t ticks, Shared& sh) {
  const uint64_t S = A.step_bytes;
  for (uint64_t j = 0; j < sd.r.k; ++j) {
    const uint64_t g = sd.base + m * sd.r.k + j;
    uint32_t err = 0;
    if (threadIdx.x < 64) {  // wave 0 takes the address
      Deadline dl(ticks, A.status);
      uint64_t p;
      while ((p = wave_load<SC>(&sd.lc->ptrx)) == 0) {
        if ((err = dl.expired())) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (threadIdx.x == 0) {
        if (!err) {
          fence_acquire<SC>();
          st_u64<SC>(&sd.lc->ptrx, 0);
        }
        sh.ptr = p;
      }
    }
    if (wg_failed(sh, err, A.status)) return false;
    uint8_t* p = reinterpret_cast<uint8_t*>(sh.ptr);
    const uint64_t L = min(S, sd.r.len - j * S);
    uint64_t lo, hi;
    lane_share16(L, S, A.lanes, w, lo, hi);
    wg_copy<AL>(src + sd.r.beg + j * S + lo, p, hi - lo);
    fence_release<SC>();
    if (wg_failed(sh, 0, A.status)) return false;
    if (threadIdx.x == 0) st_u64<SC>(&sd.lc->tail, g + 1);
  }
  return true;
}

// Receiver (one thread): publish the destination of the next step whenever
// the word is clear; complete step g once tail > g by publishing head.
template <int SC>
__device__ void zc_recv(const ConnArgs& A, uint32_t w, Side& sd, uint64_t iters, uint8_t* dst,
                        uint64_t ticks) {
  if (threadIdx.x != 0) return;
  const uint64_t total = iters * sd.r.k, S = A.step_bytes;
  uint64_t npub = 0, ndone = 0;
  Deadline dl(ticks, A.status);
  while (ndone < total) {
    bool moved = false;
    if (npub < total && ld_u64<SC>(&sd.lc->ptrx) == 0) {
      const uint64_t j = npub % sd.r.k;
      const uint64_t L = min(S, sd.r.len - j * S);
      uint64_t lo, hi;
      lane_share16(L, S, A.lanes, w, lo, hi);
      const uint64_t addr = reinterpret_cast<uint64_t>(dst + sd.r.beg + j * S + lo);
      fence_release<SC>();
      st_u64<SC>(&sd.lc->ptrx, addr);
      ++npub;
      moved = true;
    }
    const uint64_t t = ld_u64<SC>(&sd.lc->tail);
    if (t > sd.base + ndone) {
      fence_acquire<SC>();
      st_u64<SC>(&sd.lc->head, t);
      ndone = t - sd.base;
      moved = true;
    }
    if (moved) {
      dl = Deadline(ticks, A.status);
    } else {
      const uint32_t e = dl.expired();
      if (e) {
        raise_err(A.status, e);
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
}

// ------------------------------------------------------------------ kernels
__device__ __forceinline__ uint32_t logical_wg(uint32_t remap, uint32_t total) {
  const uint32_t b = blockIdx.x;
  return remap ? (b % 8u) * (total / 8u) + b / 8u : b;
}

template <int PROTO, int SC, bool AL, int MAXB>
__global__ void __launch_bounds__(1024) run_kernel(RunArgs<MAXB> args) {
  __shared__ Shared sh;
  if (threadIdx.x == 0) sh.err = 0;
  __syncthreads();
  const uint32_t lw = logical_wg(args.xcd_remap, args.total_wgs);
  uint32_t ci = 0;
  if constexpr (MAXB > 1) {
    while (ci + 1 < args.nconn && lw >= args.conn[ci + 1].wg_begin) ++ci;
  }
  const ConnArgs& A = args.conn[ci];
  const uint32_t local = lw - A.wg_begin;
  const uint32_t pair = local >> 1, role = local & 1u;
  const uint32_t c = pair / A.lanes, w = pair % A.lanes;
  if (c >= A.nch) return;  // never taken: the host sizes the grid exactly
  if (!((A.roles >> role) & 1u)) return;  // side switched off for fault injection
  Side sd = make_side(A, c, w, role == 0, SC);
  if (sd.r.k == 0) return;
  const uint64_t ticks = args.timeout_ticks;
  if constexpr (PROTO == kProtoZC) {
    if (role == 1) {
      zc_recv<SC>(A, w, sd, args.iters, A.dst, ticks);
      return;
    }
  }
  for (uint32_t m = 0; m < args.iters; ++m) {
    bool ok;
    if constexpr (PROTO == kProtoSimple)
      ok = role == 0 ? simple_send<SC, AL>(A, c, w, sd, m, A.src, ticks, sh)
                     : simple_recv<SC, AL>(A, c, w, sd, m, A.dst, ticks, sh);
    else if constexpr (PROTO == kProtoLL)
      ok = role == 0 ? ll_send<SC, AL>(A, c, w, sd, m, A.src, ticks, sh)
                     : ll_recv<SC, AL>(A, c, w, sd, m, A.dst, ticks, sh);
    else
      ok = zc_send<SC, AL>(A, c, w, sd, m, A.src, ticks, sh);
    if (!ok) return;
  }
  if constexpr (PROTO == kProtoLL) {
    if (role == 0) ll_close<SC>(sd, args.iters);
  }
}

// Ping-pong: pair side 0 is endpoint X (send on fwd, then receive on rev),
// side 1 is endpoint Y (receive on fwd into b, then send b on rev).
template <int PROTO, int SC, bool AL>
__global__ void __launch_bounds__(1024) ping_kernel(PingArgs args) {
  __shared__ Shared sh;
  if (threadIdx.x == 0) sh.err = 0;
  __syncthreads();
  const uint32_t lw = logical_wg(args.xcd_remap, args.total_wgs);
  const uint32_t pair = lw >> 1, side = lw & 1u;
  const ConnArgs& F = args.fwd;
  const ConnArgs& R = args.rev;
  const uint32_t c = pair / F.lanes, w = pair % F.lanes;
  if (c >= F.nch) return;
  Side fs = make_side(F, c, w, side == 0, SC);
  Side rs = make_side(R, c, w, side == 1, SC);
  if (fs.r.k == 0) return;
  const uint64_t ticks = args.timeout_ticks;
  for (uint32_t it = 0; it < args.iters; ++it) {
    bool ok;
    if (side == 0) {
      if constexpr (PROTO == kProtoLL)
        ok = ll_send<SC, AL>(F, c, w, fs, it, F.src, ticks, sh) &&
             ll_recv<SC, AL>(R, c, w, rs, it, R.dst, ticks, sh);
      else
        ok = simple_send<SC, AL>(F, c, w, fs, it, F.src, ticks, sh) &&
             simple_recv<SC, AL>(R, c, w, rs, it, R.dst, ticks, sh);
    } else {
      if constexpr (PROTO == kProtoLL)
        ok = ll_recv<SC, AL>(F, c, w, fs, it, F.dst, ticks, sh) &&
             ll_send<SC, AL>(R, c, w, rs, it, R.src, ticks, sh);
      else
        ok = simple_recv<SC, AL>(F, c, w, fs, it, F.dst, ticks, sh) &&
             simple_send<SC, AL>(R, c, w, rs, it, R.src, ticks, sh);
    }
    if (!ok) return;
  }
  if constexpr (PROTO == kProtoLL) {
    if (side == 0)
      ll_close<SC>(fs, args.iters);
    else
      ll_close<SC>(rs, args.iters);
  }
}

// --------------------------------------------------------- dispatch tables
template <int MAXB>
using RunFn = void (*)(RunArgs<MAXB>);
using PingFn = void (*)(PingArgs);

template <int MAXB, int P, int SC>
RunFn<MAXB> pick_run_al(bool al) {
  return al ? run_kernel<P, SC, true, MAXB> : run_kernel<P, SC, false, MAXB>;
}

template <int MAXB, int P>
RunFn<MAXB> pick_run_sc(int sc, bool al) {
  return sc == kScopeSystem ? pick_run_al<MAXB, P, kScopeSystem>(al)
                            : pick_run_al<MAXB, P, kScopeAgent>(al);
}

template <int MAXB>
RunFn<MAXB> pick_run(const Variant& v) {
  switch (v.proto) {
    case kProtoSimple: return pick_run_sc<MAXB, kProtoSimple>(v.scope, v.aligned);
    case kProtoLL: return pick_run_sc<MAXB, kProtoLL>(v.scope, v.aligned);
    default: return pick_run_sc<MAXB, kProtoZC>(v.scope, v.aligned);
  }
}

template <int P, int SC>
PingFn pick_ping_al(bool al) {
  return al ? ping_kernel<P, SC, true> : ping_kernel<P, SC, false>;
}

template <int P>
PingFn pick_ping_sc(int sc, bool al) {
  return sc == kScopeSystem ? pick_ping_al<P, kScopeSystem>(al) : pick_ping_al<P, kScopeAgent>(al);
}

PingFn pick_ping(const Variant& v) {
  return v.proto == kProtoLL ? pick_ping_sc<kProtoLL>(v.scope, v.aligned)
                             : pick_ping_sc<kProtoSimple>(v.scope, v.aligned);
}

}  // namespace

hipError_t launch_run1(const Variant& v, const RunArgs<1>& a, int block, hipStream_t s) {
  hipLaunchKernelGGL(pick_run<1>(v), dim3(a.total_wgs), dim3(block), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_runB(const Variant& v, const RunArgs<16>& a, int block, hipStream_t s) {
  hipLaunchKernelGGL(pick_run<16>(v), dim3(a.total_wgs), dim3(block), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ping(const Variant& v, const PingArgs& a, int block, hipStream_t s) {
  hipLaunchKernelGGL(pick_ping(v), dim3(a.total_wgs), dim3(block), 0, s, a);
  return hipGetLastError();
}

hipError_t max_resident(const Variant& v, int kind, int block, int* wgs) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const void* fn = kind == 0   ? reinterpret_cast<const void*>(pick_run<1>(v))
                   : kind == 1 ? reinterpret_cast<const void*>(pick_run<16>(v))
                               : reinterpret_cast<const void*>(pick_ping(v));
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0);
  if (e != hipSuccess) return e;
  *wgs = per_cu * cus;
  return hipSuccess;
}

}  // namespace xfer
