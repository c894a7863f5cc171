// Layouts shared by the host runtime (conn.cpp) and the gfx950 kernels
// (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace xfer {

// One lane = one producer/consumer workgroup pair of a channel.  Each lane
// has its own counters; every word sits on its own 128-byte line so the
// producer's tail and the consumer's head never share a cache line.  The
// receive side owns tail, the send side owns head and ptrExchange ("transport
// 建立", p2pRecvConnect listing).  A connection addresses them through two
// arrays of blocks, the send side's (head, ptrExchange) and the receive
// side's (tail, proxy tails): one array serving both in write mode, two
// separate allocations under P2P read, where the SIMPLE FIFO follows the send
// side's blocks in the same allocation.
//
// A relay connection (the shm transport's memcpy mode) adds the two host
// proxies' tails: ytail (send proxy: step copied from the send FIFO into the
// staging FIFO) and gtail (receive proxy: step copied on into the receive
// FIFO, polled by the consumer instead of tail).  They are per channel: only
// lane 0's are used.
struct alignas(128) LaneCtrl {
  uint64_t tail;
  uint64_t pad0[15];
  uint64_t head;
  uint64_t pad1[15];
  uint64_t ptrx;
  uint64_t pad2[15];
  uint64_t ytail;
  uint64_t pad3[15];
  uint64_t gtail;
  uint64_t pad4[15];
};
static_assert(sizeof(LaneCtrl) == 640, "control block layout");

// Per-connection status words in pinned host memory: the code of an
// in-kernel failure (0 = none; a later failure may overwrite an earlier
// code, never with 0) and the host's abort request.
struct alignas(128) Status {
  uint32_t err;
  uint32_t pad0[31];
  uint32_t abort_flag;
  uint32_t pad1[31];
};

// One step-trace record (the public xfer_trace_rec, same layout).
struct TraceRec {
  uint64_t time;     // s_memrealtime ticks
  uint64_t step;     // global step g
  uint64_t value;    // event-specific
  uint32_t channel;
  uint16_t lane;
  uint8_t side;      // 0 producer, 1 consumer / receiver
  uint8_t event;     // 0 acquire, 1 publish
};
static_assert(sizeof(TraceRec) == 32, "trace record layout");

// Kernel protocols: the public ones, and LL in the striped line layout
// (ll_layout), which gets kernels of its own.
enum : uint32_t { kProtoSimple = 0, kProtoLL = 1, kProtoZC = 2, kProtoZCD = 3, kProtoLLStriped = 4 };
enum : int { kScopeAgent = 0, kScopeSystem = 1 };

// Device view of one connection for one run.
struct ConnArgs {
  uint8_t* fifo;    // channel c, slot s: fifo + (c * nslots + s) * slot_bytes (producer's)
  uint8_t* fifo_rx; // the FIFO the consumer drains: fifo, or a relay's receive FIFO
  LaneCtrl* ctrl_tx; // send side's blocks [nch * lanes], lane (c, w) at c * lanes + w
  LaneCtrl* ctrl_rx; // receive side's blocks, same indexing (may equal ctrl_tx)
  Status* status; // device view of the pinned status block
  const uint8_t* src;
  uint8_t* dst;
  uint64_t nbytes;
  uint64_t slot_bytes;
  uint64_t step_bytes;
  uint32_t nch, nslots, lanes;
  uint32_t wg_begin;   // first logical workgroup of this connection (zero-copy: of its
                       // producers, counted from the first producer of the launch)
  uint32_t rx_begin;   // zero-copy: first receiver workgroup of this connection
  uint32_t roles;  // bit 0: producer side runs, bit 1: consumer side runs
  uint32_t relay;  // 1: the consumer waits on gtail and drains fifo_rx
  TraceRec* trace;     // step trace, or nullptr: [nch * lanes * 2] rings of trace_per records
  uint32_t trace_per;  // records per (channel, lane, side) ring
  uint32_t jitter;     // debug variant: seed of random delays in the step loops, 0 = none
  uint32_t* err_dev;   // mirror of status->err beside the counters (same memory and scope),
                       // read by every workgroup on entry
  uint64_t* claims;    // debug variant: per logical workgroup, the last launch that claimed it
  uint64_t launch_seq; // debug variant: this launch's number on the connection (from 1)
  uint32_t ll_stripe_log2;  // LL striped layout (ll_layout): log2 of a lane's lines per slot,
                            // 0 when the connection does not use it
  uint32_t ll_group;        // LL striped layout: steps a lane's threads cover at once
};

// One message of a launch: bytes [off, off + len) of the connection's src
// move to the same range of its dst.
struct MsgDesc {
  uint64_t off, len;
};
constexpr int kMaxMsgs = 128;  // messages carried by one launch's arguments

// A launch runs, for each connection, its message list `iters` times in
// order (nmsgs == 0: the single message {0, conn.nbytes}).  Every message is
// partitioned and numbered exactly as a separate run would be; the FIFO
// pipeline just flows from one message into the next.
// NMSG: capacity of the message list.  Only message-list launches carry
// one (kMaxMsgs); the others carry a single unused entry, since the size of
// the argument block is paid on every launch (about 1.2 us more per launch
// with 2 KiB more, measured on an empty kernel).
template <int MAXB, int NMSG>
struct RunArgs {
  ConnArgs conn[MAXB];
  uint32_t nconn;
  uint32_t iters;
  uint32_t total_wgs;
  uint32_t xcd_remap;    // 0: dispatch order; 1: pairs on one XCD; 2: the same by XCD id
  uint64_t timeout_ticks;
  uint32_t nmsgs;        // single-connection launches only
  uint32_t rx_wgs;       // zero-copy: receiver workgroups, blocks [0, rx_wgs) of the grid
  MsgDesc msgs[NMSG];
};
using RunOne = RunArgs<1, 1>;           // one transfer (xfer_run, xfer_run_loop)
using RunList = RunArgs<1, kMaxMsgs>;   // a message list (xfer_run_messages)
using RunBatch = RunArgs<16, 1>;        // several connections (xfer_run_batch)
static_assert(sizeof(RunList) <= 4096 && sizeof(RunBatch) <= 4096,
              "kernel arguments are limited to 4 KiB");

struct PingArgs {
  ConnArgs fwd, rev;     // fwd: a -> b (X sends), rev: b -> c (Y sends)
  uint64_t timeout_ticks;
  uint32_t iters;
  uint32_t total_wgs;
  uint32_t xcd_remap;
  uint32_t pad;
};

// Workgroups of one connection's launch.  SIMPLE and LL: a producer and a
// consumer workgroup per lane.  Both zero-copy protocols: a producer
// workgroup per lane, and receiver workgroups in which the first
// kRxLanesPerWave threads of each wave serve one lane each (a receiver has
// a few words to move per step, no payload).
constexpr uint32_t kRxLanesPerWave = 16;
__host__ __device__ inline uint32_t zc_receiver_wgs(uint32_t nch, uint32_t lanes, uint32_t block) {
  const uint32_t per_wg = kRxLanesPerWave * (block / 64u);
  return (nch * lanes + per_wg - 1) / per_wg;
}
__host__ __device__ inline bool zero_copy_proto(int proto) { return proto == kProtoZC || proto == kProtoZCD; }
__host__ __device__ inline uint32_t conn_wgs(int proto, uint32_t nch, uint32_t lanes, uint32_t block) {
  return zero_copy_proto(proto) ? nch * lanes + zc_receiver_wgs(nch, lanes, block)
                                : nch * lanes * 2u;
}

// LL line layout of a connection.  When a whole step fits the lanes at one
// line per thread, lane w owns the stripe [w q, (w + 1) q) of every slot's
// lines, q = the step's lines over the lanes rounded up to a power of two of
// at least a wave, and its threads cover group = min(block / q, nslots)
// consecutive steps at once (thread t: step t / q of the group, line
// w q + t mod q).  Otherwise (*log2q = 0) lanes own blocks of `block` lines
// dealt round-robin.  Fixed per connection: it depends on the step size,
// lanes, block size and slot count only.
__host__ __device__ inline void ll_layout(uint64_t step_bytes, uint32_t lanes, uint32_t block,
                                          uint32_t nslots, uint32_t* log2q, uint32_t* group) {
  *log2q = 0;
  *group = 1;
  const uint64_t lines = step_bytes / 4u;
  if (lines > uint64_t(block) * lanes) return;
  const uint64_t per = (lines + lanes - 1u) / lanes;
  uint32_t l2 = 6;  // a wave
  while ((uint64_t(1) << l2) < per) ++l2;
  if ((1u << l2) > block) return;
  *log2q = l2;
  *group = block >> l2;
  if (*group > nslots) *group = nslots;
}

// Kernel-variant selector and launchers (kernels.hip).
struct Variant {
  int proto;     // kProto* (LL connections in the striped layout: kProtoLLStriped)
  int scope;     // kScope*
  int ordering;  // 0: coherent accesses, 1: scoped fences
  int aligned;   // all of src/dst 16-byte aligned
  int debug;     // 1: the debug variant (step trace, jitter)
};

// coop: a cooperative grid (every workgroup resident at once, or refused).
hipError_t launch_run1(const Variant& v, const RunOne& a, int block, hipStream_t s,
                       bool coop = false);
hipError_t launch_runL(const Variant& v, const RunList& a, int block, hipStream_t s,
                       bool coop = false);
hipError_t launch_runB(const Variant& v, const RunBatch& a, int block, hipStream_t s,
                       bool coop = false);
hipError_t launch_ping(const Variant& v, const PingArgs& a, int block, hipStream_t s,
                       bool coop = false);
// Workgroups of `block` threads the device can hold resident at once for
// the variant's kernel of launch kind 0 (one transfer), 1 (a batch of
// connections), 2 (the ping-pong) or 3 (a message list).
hipError_t max_resident(const Variant& v, int kind, int block, int* wgs);
// Whether the current device deals a launch's blocks to 8 XCDs in strict
// rotation on every stream (the kernels may then place blocks by XCD id).
hipError_t xcc_rotation_ok(bool* ok);

}  // namespace xfer
