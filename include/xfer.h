/*
 * xfer.h -- C ABI of the MI355X (gfx950) FIFO send/recv data plane.
 *
 * A connection moves a source buffer A into a destination buffer B through
 * a ring of fixed-size FIFO slots per channel; the producer and consumer
 * synchronise through head and tail step counters.  Both endpoints run as
 * concurrent workgroup sets inside one kernel launch on one GPU.  Sources:
 *   - "【NCCL】transport数据传输（二）" (NCCL v2.25.1-1), p2pTransport:
 *     "zero copy方式传递数据" (ptrExchange hand-off) and "copy方式传递数据"
 *     (LL and SIMPLE copy through the peer's buffer); shmTransport
 *     "正常方式" (the same hand-off through a host-memory FIFO);
 *   - "transport建立" (NCCL v2.25.1-1): setup driver peer loop and channel
 *     masks (section 具体说明), where head/tail/ptrExchange live
 *     (p2pRecvConnect listing; shmRecvConnect listing);
 *   - "RDMA and GPUDirect" series article, section 四.1: LL carries its
 *     completion flag inside the data;
 *   - "Intra-Node Transport (P2P)", section 4 "POST / POLL": the steady state
 *     is host-silent; the connector must be mirrored into device memory.
 *
 * Conventions (shared by every entry point):
 *   - Every function returns an xfer_status; XFER_OK is 0.  On failure a
 *     thread-local message is available from xfer_last_error().
 *   - Buffers named src/dst/a/b/c are DEVICE pointers owned by the caller
 *     (for instance torch tensors' data_ptr()).  They must stay valid until
 *     the work queued on `stream` has completed.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *   - Runs are stream-ordered and asynchronous: a run returns after the
 *     launch; in-kernel failures (a wait that exceeded the connection's
 *     timeout, a host abort) are reported by xfer_conn_query() once the
 *     stream has been synchronised, and make every later run on that
 *     connection fail with XFER_ERR_STATE.  A run already queued behind the
 *     failed one when it failed does nothing: its workgroups read the
 *     failure beside the counters on entry and leave every word as it is.
 *   - Launch order: the library's launches on one device run one at a time,
 *     in the order they are made, whatever their streams.  Every launch
 *     needs all its workgroups resident at once, and two launches sharing
 *     the GPU could each hold part of it and wait on the rest.  Launches on
 *     one stream are ordered by the stream; a launch on another stream than
 *     the device's previous launch first waits on the host until the device
 *     has finished its work (hipDeviceSynchronize), so switching streams
 *     costs a host-side wait and is not allowed under stream capture (keep
 *     captured runs on one stream, or use xfer_run_noalloc).  Kernels of
 *     other code running beside a launch only delay the dispatch of its
 *     workgroups; a kernel that waits on one of this library's launches must
 *     not hold the GPU's resources meanwhile.  Connections created with
 *     xfer_attr.cooperative launch cooperative grids, which the runtime
 *     starts only with every workgroup resident.  xfer_run_noalloc does not
 *     take part in this order (see there).
 *   - Step counters are 64-bit, start at 0 when the connection is created,
 *     and persist across runs; step g (0-based) publishes tail = g+1.
 *   - Runs on one connection must be serialised (same stream, or synchronised
 *     streams).  Two launches that overlap on one connection race.
 *   - Pinned host memory (host FIFOs, staging FIFOs, host counters) is
 *     allocated on the NUMA node closest to the GPU where the runtime names
 *     one; environment XFER_HOST_NUMA=0 turns that off.
 *   - Host threads: calls on one connection must not overlap in time (the
 *     connection keeps host-side step bookkeeping); calls on different
 *     connections may come from different threads at once.  The library's
 *     shared state (per-device checks, occupancy caches) is locked.
 */
#ifndef XFER_H
#define XFER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  XFER_OK = 0,
  XFER_ERR_INVALID_ARG = 1, /* argument outside the documented domain */
  XFER_ERR_NO_MEMORY = 2,   /* device or pinned host allocation failed */
  XFER_ERR_HIP = 3,         /* a HIP runtime call failed (message names it) */
  XFER_ERR_INTERNAL = 4,
  XFER_ERR_TIMEOUT = 5,     /* an in-kernel wait passed the connection's timeout */
  XFER_ERR_ABORTED = 6,     /* xfer_conn_abort() stopped the kernel */
  XFER_ERR_RANGE = 7,       /* an LL connection would pass 2^32-1 steps (32-bit flags) */
  XFER_ERR_STATE = 8        /* the connection carries an earlier in-kernel failure */
} xfer_status;

typedef enum {
  XFER_PROTO_SIMPLE = 0,   /* copy through FIFO slots, tail/head per step */
  XFER_PROTO_LL = 1,       /* 8-byte lines {4 data bytes, 4-byte flag = step+1}, no polled tail */
  XFER_PROTO_ZEROCOPY = 2, /* receiver publishes the destination per step in ptrExchange */
  XFER_PROTO_ZEROCOPY_DIRECT = 3 /* destination known before the launch: the producer writes
                                    each step at its own offset of dst and publishes tail, the
                                    receiver answers with head; ptrExchange unused
                                    ("【NCCL】transport数据传输（二）", p2pTransport, zero copy,
                                    second kind) */
} xfer_proto;

typedef enum {
  XFER_FIFO_DEVICE = 0, /* FIFO in HBM (the P2P transport's placement) */
  XFER_FIFO_HOST = 1,   /* FIFO in pinned host memory (the shm transport's placement) */
  XFER_FIFO_RELAY = 2   /* copy-engine relay, SIMPLE only ("【NCCL】transport数据传输（二）",
                           shmTransport, useMemcpy): the producer fills a send FIFO in HBM
                           and publishes tail; a host send proxy copies each step into a
                           staging FIFO in pinned host memory (device-to-host DMA) and
                           publishes its own tail; a host receive proxy copies it on into a
                           receive FIFO in HBM (host-to-device DMA) and publishes a third
                           tail, which the consumer polls; head stays the producer's credit.
                           The control words live in host memory. */
} xfer_fifo_loc;

typedef enum {
  XFER_CTRL_DEFAULT = 0, /* device memory for HBM FIFOs, host memory for host FIFOs */
  XFER_CTRL_DEVICE = 1,  /* head/tail/ptrExchange words in HBM */
  XFER_CTRL_HOST = 2     /* head/tail/ptrExchange words in pinned host memory */
} xfer_ctrl_loc;

/* How a hand-off orders the payload before the counter that publishes it.
 * COHERENT: payload and control words are accessed with the cache policy of
 * the connection's scope (performed at the coherence point, not in an XCD's
 * private L2); each wave waits for its accesses to complete before the
 * counter store, and the peer reads the payload only after its counter load
 * returned.  FENCED: plain payload accesses with the scoped release/acquire
 * fences of the compiler's memory model (an L2 writeback before the counter
 * store, an L2 invalidate after the counter load), several times slower. */
typedef enum {
  XFER_ORDER_COHERENT = 0,
  XFER_ORDER_FENCED = 1
} xfer_ordering;

/* Optional creation attributes; zero-filled fields take the defaults. */
typedef struct {
  int wgs_per_channel;  /* workgroups per channel on each side (lanes), 1..16; default 1 */
  int block_threads;    /* threads per workgroup, a multiple of 64 in 64..1024; default 256 */
  int ctrl_loc;         /* xfer_ctrl_loc */
  uint32_t timeout_ms;  /* bound on every in-kernel wait; default 10000 */
  int xcd_pairing;      /* 0 (default) or 1: place each producer/consumer pair on one XCD,
                           an XCD's producers dispatched before its consumers (the grid is
                           padded to a multiple of 16 workgroups; padding exits at once).
                           Zero-copy launches have no pairs and ignore this: each thread
                           of a few receiver workgroups, dispatched first, is the
                           receiver of one lane, and one producer workgroup per lane
                           follows.
                           Each hardware queue starts dealing blocks to the XCDs at an XCD
                           of its own; where a one-time check at the first creation on a
                           device sees a strict rotation over 8 XCDs on every stream,
                           blocks take their place from the XCD id they read, so a pair's
                           XCD does not depend on the stream (environment
                           XFER_XCD_BY_ID=0 turns this off);
                           -1: dispatch order (producers on even block ids, which the
                           hardware deals to XCDs 0, 2, 4 and 6 only) */
  int roles;            /* fault injection: 0 = both sides (default), 1 = producer only,
                           2 = consumer/receiver only; a lone side ends its waits with
                           XFER_ERR_TIMEOUT (or XFER_ERR_ABORTED after xfer_conn_abort) */
  int ordering;         /* xfer_ordering */
  int p2p_read;         /* 0 (default): write mode, the SIMPLE FIFO belongs to the receive side,
                           which the producer writes into.  1: P2P read, the FIFO is appended
                           to the send side's memory (after its head/ptrExchange blocks) and
                           the consumer reads it from there; tail stays in the receive side's
                           own blocks ("transport建立", p2pSendSetup and p2pRecvConnect
                           listings; "【NCCL】transport数据传输（二）", SIMPLE copy mode).
                           The protocol steps are unchanged.  SIMPLE with the FIFO and
                           control words in HBM only; otherwise INVALID_ARG. */
  int place_trials;     /* 0 or 1 (default): no placement.  K in 2..8: placement by measured
                           latency.  A device-scope poll is served beyond the XCD's L2, and
                           the time of one hand-off depends on the physical 2-4 KiB granule
                           of the polled line (two classes, about 0.14 us apart one-way,
                           repeating every 16 KiB).  The FIFO, then the counter blocks, are
                           tried at K offsets 2 KiB apart inside allocations that much
                           larger; each offset is timed by a short ping-pong (16 bytes per
                           channel) against a reference connection in the launch shape the
                           connection uses, and the fastest is kept.  The FIFO, counters and
                           status are zeroed again afterwards, so the connection starts like
                           a new one.  Creation takes a few milliseconds longer.  SIMPLE or
                           LL in write mode with the FIFO and control words in HBM;
                           otherwise INVALID_ARG. */
  int cooperative;      /* 0 (default) or 1: launch this connection's transfers as cooperative
                           grids (hipLaunchCooperativeKernel), which the runtime starts only
                           with every workgroup resident at once and otherwise refuses with
                           XFER_ERR_HIP, whatever else holds the GPU.  Without it, the library
                           checks the grid against the GPU's capacity and orders its own
                           launches (see "Launch order"), but kernels of other code can still
                           delay part of a grid.  Costs about 15-18 us per launch on MI355X.
                           A batch or ping-pong needs the same setting on all its
                           connections.  Not with xfer_run_noalloc.  Otherwise INVALID_ARG. */
} xfer_attr;

/* State of one channel, read back after the stream has been synchronised. */
typedef struct {
  uint64_t head;         /* consumer's counter (steps drained) */
  uint64_t tail;         /* producer's counter (steps published; LL: written once per run) */
  uint64_t ptr_exchange; /* zero-copy address word; 0 when idle */
  uint64_t steps;        /* steps this channel has completed over all runs (host bookkeeping) */
  int lanes;             /* workgroup pairs serving the channel, each with its own counters */
  int lanes_agree;       /* 1 when every lane's head, tail and ptrExchange equal lane 0's */
  int error;             /* xfer_status of the connection's in-kernel failures (sticky) */
  int reserved;
} xfer_chan_state;

typedef struct xfer_conn xfer_conn;

/* ---------------------------------------------------------------- setup
 * xfer_conn_create / _ex: allocate and wire one connection: per channel a
 * FIFO of nslots x slot_bytes (none for zero-copy), zeroed, and a control
 * block holding head, tail and ptrExchange, zeroed (the receive side's
 * connect wires tail to its own block and head/ptrExchange to the send
 * side's, "transport建立", p2pRecvConnect listing; the shm transport keeps
 * the FIFO and tail in host memory, shmRecvConnect listing).  With
 * attr->p2p_read the send side's blocks and the SIMPLE FIFO after them form
 * one allocation and the receive side's blocks (tail) another
 * (p2pSendSetup listing).  The connection's device descriptor is uploaded to
 * HBM ("Intra-Node Transport (P2P)" section 3, connector mirror).
 *   proto       xfer_proto.
 *   nchannels   1..64 (64-bit channel masks).
 *   nslots      >= 1 FIFO slots per channel (ignored by zero-copy).
 *   slot_bytes  bytes per slot, at most 1 GiB: SIMPLE and zero-copy a
 *               multiple of 16 (a zero-copy step moves slot_bytes); LL a
 *               multiple of 8, of which half is payload.
 *   fifo_loc    xfer_fifo_loc.
 *   attr        NULL for defaults.
 *   out         receives the connection; owned by the caller until
 *               xfer_conn_destroy().
 * Errors: INVALID_ARG for any value outside these domains (no allocation is
 * made), NO_MEMORY / HIP when an allocation fails (nothing leaks). */
int xfer_conn_create(int proto, int nchannels, int nslots, size_t slot_bytes, int fifo_loc,
                     xfer_conn** out);
int xfer_conn_create_ex(int proto, int nchannels, int nslots, size_t slot_bytes, int fifo_loc,
                        const xfer_attr* attr, xfer_conn** out);

/* Frees the FIFO, control blocks and descriptor.  The caller must have
 * synchronised every stream that ran on the connection.  NULL is a no-op. */
int xfer_conn_destroy(xfer_conn* c);

/* ------------------------------------------------------------------ runs
 * xfer_run: queue one transfer of nbytes from src to dst on stream.  The
 * bytes are split over the channels (each channel takes a contiguous range;
 * the range size is ceil(nbytes / nchannels) rounded up to 16 bytes, so
 * trailing channels may be empty) and each channel's range into steps of
 * the step size.  One launch holds every channel's producer and consumer
 * workgroups.  Producer step g: wait until g - head < nslots, write the
 * chunk into slot g mod nslots, release, tail = g+1.  Consumer: wait until
 * tail > g, acquire, copy the slot into dst, release, head = g+1
 * ("【NCCL】transport数据传输（二）", copy mode; "Intra-Node Transport
 * (P2P)" section 4, POST / POLL).  LL replaces tail polling by the per-line
 * flags; zero-copy replaces the slot by the published destination.
 *   src, dst  device buffers of nbytes; any alignment (16-byte-aligned
 *             buffers take the fast path); they must not overlap.
 *   nbytes    0 queues nothing and returns XFER_OK.
 * Errors: INVALID_ARG (NULL buffer with nbytes > 0, overlap, grid larger
 * than the GPU can hold resident at once), RANGE, STATE, HIP. */
int xfer_run(xfer_conn* c, const void* src, void* dst, size_t nbytes, void* stream);

/* xfer_run_batch: the transfers of n connections (n <= XFER_MAX_BATCH) in
 * ONE launch, e.g. the edges of a ring of logical endpoints.  All
 * connections must share protocol, memory scope, ordering, block size and
 * timeout.  No transfer's destination may overlap another transfer's source
 * or destination (the connections run in no fixed order against each
 * other); INVALID_ARG otherwise.
 * Arrays are host arrays of length n. */
#define XFER_MAX_BATCH 16
int xfer_run_batch(xfer_conn* const* conns, const void* const* src, void* const* dst,
                   const size_t* nbytes, int n, void* stream);

/* xfer_run_messages: n messages on one connection, in as few launches as
 * possible (up to 128 messages per launch).  Message i moves sizes[i] bytes
 * from src + offsets[i] to dst + offsets[i]; offsets and sizes are host
 * arrays of n entries.  The result, the counters and the FIFO bytes are
 * those of n xfer_run calls in order (each message is partitioned and
 * numbered as its own transfer); the FIFO pipeline simply flows from one
 * message into the next instead of draining at each launch boundary.
 * Zero-size messages are skipped; n == 0 queues nothing.
 * Messages must not overlap one another: channels reach different messages
 * at different times, so overlapping writes would race.
 * Errors: INVALID_ARG (NULL arrays, NULL buffers with bytes to move, two
 * non-empty messages overlapping, the span of the messages overlapping
 * between src and dst), RANGE, STATE, HIP. */
int xfer_run_messages(xfer_conn* c, const void* src, void* dst, const size_t* offsets,
                      const size_t* sizes, int n, void* stream);

/* xfer_run_loop: iters messages of nbytes from src to dst back to back on
 * one connection in one launch (each message is a full transfer; dst holds
 * the last).  Measures per-message cost without launch overhead. */
int xfer_run_loop(xfer_conn* c, const void* src, void* dst, size_t nbytes, int iters,
                  void* stream);

/* xfer_run_pingpong: iters round trips in one launch.  Endpoint X sends a
 * to b over fwd, endpoint Y receives it into b and sends b to cbuf over
 * rev, X receives it into cbuf, then the next round starts.  fwd and rev
 * must have the same protocol (SIMPLE or LL), channel count, slot size and
 * lanes.  One-way latency = elapsed / (2 * iters), the method of a
 * ping-pong latency test ("RDMA and GPUDirect", section 十.3). */
int xfer_run_pingpong(xfer_conn* fwd, xfer_conn* rev, const void* a, void* b, void* cbuf,
                      size_t nbytes, int iters, void* stream);

/* xfer_run_noalloc: for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  One transfer of nbytes from src to dst, like xfer_run on a
 * new connection created with (proto, nchannels, nslots, slot_bytes, attr,
 * FIFO in HBM): the same kernels, the same destination bytes.  Its FIFO,
 * control blocks and status words live in a fixed array of
 * XFER_NOALLOC_SCRATCH_BYTES in each GPU's memory, owned by the library and
 * held until the process ends; no connection is made and nothing is
 * allocated (the first call on a device takes the array's address there and
 * queries the device's clock rate and, per kernel variant, its resident
 * capacity).
 *   The array's FIFO room is XFER_NOALLOC_SCRATCH_BYTES less 1 MiB:
 *   nchannels x nslots x slot_bytes beyond it is INVALID_ARG (zero-copy uses
 *   no FIFO).  attr: NULL or wgs_per_channel, block_threads, timeout_ms,
 *   xcd_pairing (-1: dispatch order; 0 or 1: pairs on one XCD by block id)
 *   and ordering; ctrl_loc must be DEFAULT or DEVICE, roles and p2p_read 0,
 *   place_trials 0 or 1, cooperative 0 (otherwise INVALID_ARG).
 *   src, dst, nbytes as for xfer_run.  stream as everywhere.
 *   status: NULL, or a word the device can write (device memory, or mapped
 *   pinned host memory); when a transfer is queued, the in-kernel failure
 *   code (0 = none, else XFER_ERR_TIMEOUT or XFER_ERR_ABORTED ...) is
 *   written there after it, in stream order.
 * Every call queues a small clearing kernel, the transfer, and (with
 * status) a one-thread report kernel on `stream`.  Every call on a GPU uses
 * that GPU's one array, which keeps the last call's contents until the next
 * call clears it: calls that overlap in time on one GPU race and must be
 * ordered by the caller (one stream, or events).  These calls do not take
 * part in the ordering of the library's other launches (below, "Launch
 * order"): the caller must not run them alongside another launch of this
 * library whose grid together with this one exceeds what the GPU holds
 * resident.  Errors: INVALID_ARG, RANGE, HIP; nothing is queued then. */
#define XFER_NOALLOC_SCRATCH_BYTES (16u << 20)
int xfer_run_noalloc(int proto, int nchannels, int nslots, size_t slot_bytes,
                     const xfer_attr* attr, const void* src, void* dst, size_t nbytes,
                     uint32_t* status, void* stream);

/* --------------------------------------------------------------- inspect */
/* Synchronous read of one channel's control words (lane 0 reported; the
 * lanes_agree field compares the others) and of the sticky error.  The
 * caller synchronises the stream first. */
int xfer_conn_query(const xfer_conn* c, int channel, xfer_chan_state* out);

/* Address and size of one channel's FIFO (device pointer, or the device view
 * of the pinned host block).  Zero-copy connections have none (NULL, 0). */
int xfer_conn_fifo(const xfer_conn* c, int channel, void** fifo, size_t* bytes);

/* Synchronous copy of one channel's FIFO into host memory host_dst of
 * `bytes` (must equal the FIFO size).  For a relay this is the send FIFO. */
int xfer_conn_read_fifo(const xfer_conn* c, int channel, void* host_dst, size_t bytes);

/* The same for FIFO `which` of a relay connection: 0 send (HBM), 1 staging
 * (pinned host), 2 receive (HBM); other connections take which = 0 only.
 * Errors: INVALID_ARG (which out of range, wrong size, NULL), HIP. */
int xfer_conn_read_fifo_ex(const xfer_conn* c, int which, int channel, void* host_dst,
                           size_t bytes);

/* A relay connection's proxy tails for one channel (they are per channel,
 * kept in lane 0's control block): the send proxy's (steps copied into the
 * staging FIFO) and the receive proxy's (steps copied into the receive FIFO).
 * The caller synchronises the stream first.  Errors: INVALID_ARG (not a
 * relay, bad channel, NULL output). */
int xfer_conn_query_relay(const xfer_conn* c, int channel, uint64_t* send_proxy_tail,
                          uint64_t* recv_proxy_tail);

/* ------------------------------------------------------------ step trace
 * Debug aid, off by default (the tracing that the pages' INFO/TRACE logs
 * give the host side, here for the device side).  xfer_conn_set_trace
 * gives the connection a caller-owned DEVICE buffer of nrecords records;
 * runs queued afterwards (until it is set to NULL) stamp two events per step
 * and side, written by the side's first thread:
 *   producer  ACQUIRE  credit obtained (value: head seen), or for zero-copy
 *                      the destination taken from ptrExchange (value: its
 *                      address) and for zero-copy direct the step's own
 *                      destination;
 *             PUBLISH  just before tail = g+1 is stored (value: g+1); for LL,
 *                      just before the step's lines are stored;
 *   consumer  ACQUIRE  the step is ready (value: tail seen; LL: the flag;
 *                      zero-copy receiver: the address it publishes, stamped
 *                      before it is published);
 *             PUBLISH  just before head is stored (value: the head stored).
 * The buffer is split into nchannels x lanes x 2 rings of
 * nrecords / (nchannels x lanes x 2) records: ring (c, w, side) starts at
 * record ((c * lanes + w) * 2 + side) * per, and event e of global step g
 * goes to its slot (2g + e) mod per, so each ring keeps the latest per / 2
 * steps.  Slots never written keep the caller's contents.  Times are
 * s_memrealtime ticks (the device's constant wall clock, 100 MHz on MI355X),
 * comparable across workgroups: a PUBLISH precedes every ACQUIRE that
 * depends on it.  The buffer must stay valid until the traced runs complete.
 * Errors: INVALID_ARG (NULL connection, misaligned buffer, fewer than 2
 * records per ring). */
typedef struct {
  uint64_t time;    /* s_memrealtime ticks */
  uint64_t step;    /* global step g */
  uint64_t value;   /* see above */
  uint32_t channel;
  uint16_t lane;
  uint8_t side;     /* 0 producer, 1 consumer or receiver */
  uint8_t event;    /* xfer_trace_event */
} xfer_trace_rec;

typedef enum { XFER_TRACE_ACQUIRE = 0, XFER_TRACE_PUBLISH = 1 } xfer_trace_event;

int xfer_conn_set_trace(xfer_conn* c, void* records, size_t nrecords);

/* Debug aid for race hunting, off by default: with a non-zero seed, runs
 * queued afterwards sleep every wave a pseudo-random 0..15 x 512 cycles
 * (a function of the seed, the channel, lane and side, the step and the
 * wave) where a step is acquired and where it is published, in every
 * protocol.  Producer and consumer, and the waves of one side, then reach
 * the shared words in orders that undisturbed runs rarely take; results must
 * not change.  0 turns it off.  Traced or jittered connections run the
 * debug kernel variant; the others run kernels without any of this code.
 * Errors: INVALID_ARG (NULL connection). */
int xfer_conn_set_jitter(xfer_conn* c, uint32_t seed);

/* Sets the connection's host-side abort word; every in-kernel wait of a
 * running or later launch on it ends with XFER_ERR_ABORTED. */
int xfer_conn_abort(xfer_conn* c);

/* Grid (workgroups, padding included) and block size one run of this
 * connection launches. */
int xfer_conn_launch_shape(const xfer_conn* c, int* workgroups, int* block_threads);

/* Thread-local message of the last failure in this thread ("" if none). */
const char* xfer_last_error(void);
const char* xfer_status_string(int status);

/* --------------------------------------------------------------- schedule
 * Host-side peer/channel schedule of the setup driver ("transport建立",
 * section 具体说明 and the two setup listings after it). */

/* Loop i: recv_peer = (rank - i) mod nranks, send_peer = (rank + i) mod nranks. */
int xfer_sched_peers(int rank, int nranks, int i, int* recv_peer, int* send_peer);

/* Ring masks: only the first loop's peers carry channels 0..nchannels-1;
 * recv_mask and send_mask are caller arrays of nranks entries, indexed by
 * peer.  A single rank has no ring edge (all zero). */
int xfer_sched_ring_masks(int rank, int nranks, int nchannels, uint64_t* recv_mask,
                          uint64_t* send_mask);

typedef enum {
  XFER_OP_RECV_SETUP = 0,   /* receive-side setup of (peer, channel) */
  XFER_OP_SEND_SETUP = 1,   /* send-side setup of (peer, channel) */
  XFER_OP_CONNECT_BATCH = 2 /* connect everything set up since the last batch */
} xfer_op_kind;

typedef struct {
  int kind;
  int peer;    /* -1 for XFER_OP_CONNECT_BATCH */
  int channel; /* -1 for XFER_OP_CONNECT_BATCH */
} xfer_setup_op;

/* Ordered setup plan of one rank: per loop i = 1..nranks-1, receive setups
 * for the set bits of recv_mask[recv_peer] (ascending), then send setups for
 * send_mask[send_peer]; a CONNECT_BATCH after every max_peers loops (the
 * pages' default is 128) and after the last loop.  *nops receives the full
 * count even when it exceeds cap (then XFER_ERR_INVALID_ARG is returned and
 * only cap ops are written); ops may be NULL when cap is 0. */
int xfer_sched_plan(int rank, int nranks, const uint64_t* recv_mask, const uint64_t* send_mask,
                    int max_peers, xfer_setup_op* ops, int cap, int* nops);

/* Connects nranks logical endpoints on this GPU by running every rank's
 * plan: each SEND_SETUP(peer d, channel ch) of rank s must be matched by a
 * RECV_SETUP(peer s, channel ch) in rank d's plan; at rank s's CONNECT_BATCH
 * the edges it set up since its last batch are created, one connection per
 * directed edge with as many channels as the edge has mask bits.
 * recv_masks/send_masks are nranks x nranks row-major (row = rank).
 * edges is an nranks x nranks array filled with the connection of edge
 * s -> d at [s * nranks + d] (NULL where there is none); *nedges receives
 * their number.  The caller destroys them.  On error nothing is left
 * allocated. */
int xfer_endpoints_connect(int nranks, const uint64_t* recv_masks, const uint64_t* send_masks,
                           int max_peers, int proto, int nslots, size_t slot_bytes, int fifo_loc,
                           const xfer_attr* attr, xfer_conn** edges, int* nedges);

#ifdef __cplusplus
}
#endif
#endif /* XFER_H */
