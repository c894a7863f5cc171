// Host runtime of the FIFO send/recv data plane: connection setup and
// teardown, argument checks, and the launch of the one kernel that holds
// both endpoints.  Setup = allocate + zero + wire (the transport's
// Setup/ProxySetup/Connect sequence, "transport建立" section 具体说明);
// teardown = free.  After setup the host is silent: a run only launches.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <sys/syscall.h>
#include <unistd.h>

#include <algorithm>
#include <array>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "relay.h"
#include "xfer.h"
#include "xfer_internal.h"

struct xfer_conn {
  int proto = 0, nch = 0, nslots = 0, fifo_loc = 0, ctrl_loc = 0;
  int lanes = 1, block = 256, xcd_pairing = 0, roles = 3, ordering = 0, p2p_read = 0;
  bool coop = false;  // cooperative launches (xfer_attr.cooperative)
  uint32_t xcd_remap = 0;  // the kernels' remap: 0 dispatch order, 1 paired, 2 paired by XCD id
  size_t slot_bytes = 0, step_bytes = 0;
  uint32_t timeout_ms = 0;
  uint64_t timeout_ticks = 0;
  int device = 0;
  int scope = xfer::kScopeAgent;
  uint8_t* fifo = nullptr;       // device view of the FIFO (a relay's send FIFO)
  void* fifo_mem = nullptr;      // allocation (device pointer or pinned host pointer)
  uint8_t* fifo_rx = nullptr;    // relay: receive FIFO in HBM
  uint8_t* stage = nullptr;      // relay: staging FIFO in pinned host memory
  xfer::Relay* relay = nullptr;  // relay: the host proxies
  xfer::LaneCtrl* ctrl = nullptr;  // device view of the send side's control blocks
  void* ctrl_mem = nullptr;        // their allocation (P2P read: followed by the FIFO)
  xfer::LaneCtrl* ctrl_rx = nullptr;  // the receive side's blocks (== ctrl in write mode)
  void* ctrl_rx_mem = nullptr;        // P2P read: the receive side's own allocation
  size_t fifo_alloc = 0, ctrl_alloc = 0, ctrl_rx_alloc = 0;  // HBM bytes of the allocations
  xfer::Status* status_host = nullptr;
  xfer::Status* status_dev = nullptr;
  uint32_t* err_dev = nullptr;     // device view of the failure mirror beside the counters
  uint64_t* claims = nullptr;      // debug launches: per logical workgroup, last launch claiming it
  uint64_t launch_seq = 0;         // launches made on the connection
  xfer::TraceRec* trace = nullptr;  // caller's step-trace buffer (device), or nullptr
  uint32_t trace_per = 0;           // records per (channel, lane, side) ring
  uint32_t jitter = 0;              // seed of the debug jitter, 0 = none
  std::vector<uint64_t> steps;   // per channel, host bookkeeping of completed steps
  std::vector<uint64_t> add;     // per channel, steps a run adds (scratch of the run calls)
  int cap_one[2][2] = {{-1, -1}, {-1, -1}};  // resident capacity of a single-transfer
                                              // launch, by [aligned][debug]; -1 unknown
};

static_assert(sizeof(xfer_trace_rec) == sizeof(xfer::TraceRec) &&
                  offsetof(xfer_trace_rec, value) == offsetof(xfer::TraceRec, value) &&
                  offsetof(xfer_trace_rec, event) == offsetof(xfer::TraceRec, event),
              "the public trace record and the kernels' must share one layout");

namespace xfer {

static thread_local std::string g_last_error;

void set_error(int code, const std::string& msg) {
  (void)code;
  g_last_error = msg;
}

namespace {

constexpr uint32_t kDefaultTimeoutMs = 10000;
constexpr int kDefaultBlock = 256;
// An HBM FIFO starts this far into its allocation (write mode), or this far
// past the send side's control blocks (P2P read).
constexpr size_t kFifoAlign = size_t(64) << 10;
// The failure mirror: one 128-byte line after the control blocks (after the
// receive side's blocks under P2P read), in the same memory as the counters.
constexpr size_t kErrLine = 128;

int fail(int code, const std::string& msg) {
  set_error(code, msg);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  set_error(XFER_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return XFER_ERR_HIP;
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) changed = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (changed && prev >= 0) (void)hipSetDevice(prev);
  }
};

// Host allocations made while this is alive prefer the NUMA node closest to
// the device, so host-FIFO traffic does not cross the socket interconnect; the
// thread's previous memory policy is restored afterwards.  Disabled by
// XFER_HOST_NUMA=0, and a no-op where the node is unknown.
class NearNuma {
 public:
  explicit NearNuma(int device) {
    const char* env = getenv("XFER_HOST_NUMA");
    if (env && env[0] == '0') return;
    int node = -1;
    if (hipDeviceGetAttribute(&node, hipDeviceAttributeHostNumaId, device) != hipSuccess) {
      (void)hipGetLastError();  // an unsupported query must not linger as the last error
      return;
    }
    if (node < 0 || node >= kBits) return;
    if (syscall(SYS_get_mempolicy, &old_mode_, old_mask_, kBits, nullptr, 0) != 0) return;
    unsigned long mask[kWords] = {0};
    mask[node / 64] = 1ul << (node % 64);
    if (syscall(SYS_set_mempolicy, kPreferred, mask, kBits) != 0) return;
    active_ = true;
  }
  ~NearNuma() {
    if (active_) syscall(SYS_set_mempolicy, old_mode_, old_mask_, kBits);
  }
  unsigned flag() const { return active_ ? hipHostMallocNumaUser : 0u; }

 private:
  static constexpr int kBits = 4096, kWords = kBits / 64, kPreferred = 1;
  bool active_ = false;
  int old_mode_ = 0;
  unsigned long old_mask_[kWords] = {0};
};

void release(xfer_conn* c) {
  if (!c) return;
  DeviceGuard g(c->device);
  relay_stop(c->relay);  // joins the proxies before their buffers go
  if (c->fifo_rx) (void)hipFree(c->fifo_rx);
  if (c->stage) (void)hipHostFree(c->stage);
  if (c->fifo_mem) {
    if (c->fifo_loc == XFER_FIFO_HOST)
      (void)hipHostFree(c->fifo_mem);
    else
      (void)hipFree(c->fifo_mem);
  }
  if (c->ctrl_mem) {
    if (c->ctrl_loc == XFER_CTRL_HOST)
      (void)hipHostFree(c->ctrl_mem);
    else
      (void)hipFree(c->ctrl_mem);
  }
  if (c->ctrl_rx_mem) (void)hipFree(c->ctrl_rx_mem);
  if (c->claims) (void)hipFree(c->claims);
  if (c->status_host) (void)hipHostFree(c->status_host);
  delete c;
}

struct Partition {
  uint64_t per;
  uint64_t beg(uint64_t n, int c) const { return std::min<uint64_t>(n, per * uint64_t(c)); }
  uint64_t len(uint64_t n, int c) const {
    const uint64_t b = beg(n, c);
    return std::min<uint64_t>(n, b + per) - b;
  }
};

// Channel ranges of ceil(n / nch) rounded up to 16 bytes, in channel order
// (any split moves the same bytes; this one fixes head/tail and FIFO state).
Partition partition(uint64_t n, int nch) {
  uint64_t per = (n + uint64_t(nch) - 1) / uint64_t(nch);
  per = (per + 15) & ~uint64_t(15);
  return Partition{per};
}

uint64_t steps_of(uint64_t len, uint64_t S) { return (len + S - 1) / S; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_runnable(const xfer_conn* c, const char* who) {
  if (!c) return fail(XFER_ERR_INVALID_ARG, std::string(who) + ": NULL connection");
  const uint32_t err = __atomic_load_n(&c->status_host->err, __ATOMIC_ACQUIRE);
  if (err) {
    const std::string proxy = relay_error(c->relay);
    return fail(XFER_ERR_STATE, std::string(who) + ": connection failed earlier in a kernel (" +
                                    xfer_status_string(int(err)) +
                                    (proxy.empty() ? "" : ", " + proxy) + ")");
  }
  return XFER_OK;
}

// Hands a run to a relay connection's proxies: its messages, numbered from
// each channel's step count before the run.
void relay_job(const xfer_conn* c, std::vector<uint64_t> lens, uint64_t iters) {
  if (!c->relay) return;
  RelayJob job;
  job.lens = std::move(lens);
  job.iters = iters;
  job.base = c->steps;
  relay_submit(c->relay, job);
}

// Bookkeeping of the steps a run adds, and the LL 32-bit flag bound.
int plan_steps(const xfer_conn* c, uint64_t nbytes, uint64_t iters, std::vector<uint64_t>& add,
               const char* who) {
  const Partition P = partition(nbytes, c->nch);
  add.assign(size_t(c->nch), 0);
  for (int ch = 0; ch < c->nch; ++ch) {
    add[size_t(ch)] = steps_of(P.len(nbytes, ch), c->step_bytes) * iters;
    if (c->proto == XFER_PROTO_LL && c->steps[size_t(ch)] + add[size_t(ch)] > 0xFFFFFFFFull)
      return fail(XFER_ERR_RANGE, std::string(who) +
                                      ": LL connection would pass 2^32-1 steps (32-bit flags)");
  }
  return XFER_OK;
}

void commit_steps(xfer_conn* c, const std::vector<uint64_t>& add) {
  for (int ch = 0; ch < c->nch; ++ch) c->steps[size_t(ch)] += add[size_t(ch)];
}

// Device view of one launch of c; numbers the launch (debug launches check
// with it that no two blocks take one logical workgroup).
ConnArgs conn_args(xfer_conn* c, const void* src, void* dst, uint64_t nbytes, uint32_t wg_begin,
                   uint32_t rx_begin = 0) {
  ConnArgs a;
  memset(&a, 0, sizeof(a));
  a.rx_begin = rx_begin;
  a.err_dev = c->err_dev;
  a.claims = c->claims;
  a.launch_seq = ++c->launch_seq;
  if (c->proto == XFER_PROTO_LL)
    ll_layout(c->step_bytes, uint32_t(c->lanes), uint32_t(c->block), uint32_t(c->nslots),
              &a.ll_stripe_log2, &a.ll_group);
  a.fifo = c->fifo;
  a.fifo_rx = c->fifo_rx ? c->fifo_rx : c->fifo;
  a.relay = c->fifo_rx ? 1u : 0u;
  a.trace = c->trace;
  a.trace_per = c->trace_per;
  a.jitter = c->jitter;
  a.ctrl_tx = c->ctrl;
  a.ctrl_rx = c->ctrl_rx;
  a.status = c->status_dev;
  a.src = static_cast<const uint8_t*>(src);
  a.dst = static_cast<uint8_t*>(dst);
  a.nbytes = nbytes;
  a.slot_bytes = c->slot_bytes;
  a.step_bytes = c->step_bytes;
  a.nch = uint32_t(c->nch);
  a.nslots = uint32_t(c->nslots);
  a.lanes = uint32_t(c->lanes);
  a.wg_begin = wg_begin;
  a.roles = uint32_t(c->roles);
  return a;
}

// Both zero-copy modes write straight into the destination: no FIFO.
bool zero_copy(int proto) {
  return proto == XFER_PROTO_ZEROCOPY || proto == XFER_PROTO_ZEROCOPY_DIRECT;
}

uint32_t wgs_of(const xfer_conn* c) {
  return conn_wgs(c->proto, uint32_t(c->nch), uint32_t(c->lanes), uint32_t(c->block));
}

// Zero-copy: the connection's receiver workgroups (each thread one lane).
uint32_t rx_wgs_of(const xfer_conn* c) {
  return zero_copy(c->proto) ? zc_receiver_wgs(uint32_t(c->nch), uint32_t(c->lanes),
                                               uint32_t(c->block))
                             : 0u;
}

uint32_t round8(uint32_t x) { return (x + 7u) & ~7u; }

// Zero-copy grid of rx receiver and p producer workgroups: with grouping
// by XCD each region is padded to a multiple of 8 blocks (the padding exits
// at once); *rx_region receives the receiver region's size.
uint32_t zc_grid(const xfer_conn* c, uint32_t rx, uint32_t p, uint32_t* rx_region) {
  *rx_region = c->xcd_pairing ? round8(rx) : rx;
  return *rx_region + (c->xcd_pairing ? round8(p) : p);
}

// Launched grid.  Pairing keeps a pair (producer 2q, consumer 2q+1) on one
// XCD, producers first in each XCD's dispatch order (the kernel's
// logical_wg); its remap needs a grid of a multiple of 16, so the grid is
// padded with workgroups that exit at once.  Zero-copy launches have no
// pairs: their receiver workgroups come first, then the producers (zc_grid).
uint32_t grid_of(const xfer_conn* c, uint32_t total) {
  if (zero_copy(c->proto)) {
    uint32_t rx = 0;
    return zc_grid(c, rx_wgs_of(c), total - rx_wgs_of(c), &rx);
  }
  return c->xcd_pairing ? (total + 15u) & ~15u : total;
}

// The receiver region of a single connection's zero-copy launch (0 otherwise).
uint32_t rx_region_of(const xfer_conn* c) {
  if (!zero_copy(c->proto)) return 0;
  uint32_t rx = 0;
  (void)zc_grid(c, rx_wgs_of(c), wgs_of(c) - rx_wgs_of(c), &rx);
  return rx;
}

// Whether blocks may take their place from their XCD id on this device
// (xcc_rotation_ok), checked once per device.
int xcc_remap_ok(int dev, bool* ok) {
  static std::mutex mu;
  static std::map<int, bool> known;
  std::lock_guard<std::mutex> lk(mu);
  auto it = known.find(dev);
  if (it != known.end()) {
    *ok = it->second;
    return XFER_OK;
  }
  const char* env = getenv("XFER_XCD_BY_ID");
  if (env && env[0] == '0') {
    known[dev] = *ok = false;
    return XFER_OK;
  }
  const hipError_t e = xcc_rotation_ok(ok);
  if (e != hipSuccess) return hip_fail(e, "xfer_conn_create: XCD deal check");
  known[dev] = *ok;
  return XFER_OK;
}

// Resident-workgroup capacity per (device, kernel variant, block size),
// queried once: the runtime query costs far more than a launch.
int resident_capacity(int dev, const Variant& v, int kind, int block, int* cap) {
  static std::mutex mu;
  static std::map<std::array<int, 8>, int> cache;
  hipError_t e = hipSuccess;
  const std::array<int, 8> key{dev, v.proto, v.scope, v.ordering, v.aligned, v.debug, kind, block};
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      *cap = it->second;
      return XFER_OK;
    }
  }
  e = max_resident(v, kind, block, cap);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = *cap;
  return XFER_OK;
}

// The caller has made `dev` current (DeviceGuard).  `memo`, when given, is
// the connection's own record of this capacity.
int check_resident(int dev, const Variant& v, int kind, int block, uint32_t total,
                   const char* who, int* memo = nullptr) {
  int cap = memo ? *memo : -1;
  if (cap < 0) {
    const int rc = resident_capacity(dev, v, kind, block, &cap);
    if (rc) return rc;
    if (memo) *memo = cap;
  }
  if (int64_t(total) > int64_t(cap))
    return fail(XFER_ERR_INVALID_ARG,
                std::string(who) + ": " + std::to_string(total) +
                    " workgroups exceed the " + std::to_string(cap) +
                    " the GPU holds resident at once; both endpoints must run concurrently");
  return XFER_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The library's launches on one device run one at a time, in the order they
// were made, whatever their streams.  Each launch needs all its workgroups
// resident at once (producers and consumers wait on each other), and the
// resident check above compares one grid with the whole GPU: two launches
// that each fit but together do not could both start partly resident and
// wait on their undispatched halves until the timeout.  On one stream,
// stream order already serialises them, so nothing is added there (an event
// recorded after every launch measured 3-5 us per launch).  A launch on
// another stream than the previous launch first waits, on the host, for the
// device to finish what it holds, and goes ahead once no other launch of
// the library came in meanwhile.  The device is synchronised without the
// lock held, so a thread that still has to hand a relay its job after its
// launch is never kept from doing so.  No stream handle is kept for later
// use: the caller may destroy a stream at any time (destroying one waits
// for its work, so a new stream that gets the old handle carries none of
// it).  Kernels of other code do not wait on these, so they only delay a
// dispatch, never block it.
class LaunchGate {
 public:
  template <typename Launch>
  hipError_t run(int dev, hipStream_t s, Launch&& launch) {
    std::unique_lock<std::mutex> lk(mu_);
    Dev& d = devs_[dev];
    while (d.busy && d.last != s) {
      const uint64_t seen = d.launches;
      lk.unlock();
      const hipError_t e = hipDeviceSynchronize();
      lk.lock();
      if (e != hipSuccess) return e;
      if (d.launches == seen) d.busy = false;  // every launch so far has completed
    }
    const hipError_t e = launch();
    if (e != hipSuccess) return e;
    d.busy = true;
    d.last = s;
    ++d.launches;
    return hipSuccess;
  }

 private:
  struct Dev {
    bool busy = false;           // a launch may still be on the device
    hipStream_t last = nullptr;  // the stream of the last launch (compared, never used)
    uint64_t launches = 0;
  };
  std::mutex mu_;
  std::map<int, Dev> devs_;
};

LaunchGate& gate() {
  static LaunchGate* g = new LaunchGate();  // never destroyed: launches may come during exit
  return *g;
}

}  // namespace
}  // namespace xfer

using namespace xfer;

extern "C" const char* xfer_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* xfer_status_string(int s) {
  switch (s) {
    case XFER_OK: return "XFER_OK";
    case XFER_ERR_INVALID_ARG: return "XFER_ERR_INVALID_ARG";
    case XFER_ERR_NO_MEMORY: return "XFER_ERR_NO_MEMORY";
    case XFER_ERR_HIP: return "XFER_ERR_HIP";
    case XFER_ERR_INTERNAL: return "XFER_ERR_INTERNAL";
    case XFER_ERR_TIMEOUT: return "XFER_ERR_TIMEOUT";
    case XFER_ERR_ABORTED: return "XFER_ERR_ABORTED";
    case XFER_ERR_RANGE: return "XFER_ERR_RANGE";
    case XFER_ERR_STATE: return "XFER_ERR_STATE";
    default: return "XFER_ERR_UNKNOWN";
  }
}

// Back to the state of a new connection: FIFO, control blocks and status
// zeroed, no steps counted.
static int zero_state(xfer_conn* c) {
  DeviceGuard g(c->device);
  hipError_t e = hipSuccess;
  if (c->fifo_mem && c->fifo_alloc) e = hipMemset(c->fifo_mem, 0, c->fifo_alloc);
  if (e == hipSuccess && c->ctrl_mem) e = hipMemset(c->ctrl_mem, 0, c->ctrl_alloc);
  if (e == hipSuccess && c->ctrl_rx_mem) e = hipMemset(c->ctrl_rx_mem, 0, c->ctrl_rx_alloc);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipMemset(connection state)");
  memset(c->status_host, 0, sizeof(Status));
  c->steps.assign(size_t(c->nch), 0);
  return XFER_OK;
}

// Placement by measured latency (xfer_attr.place_trials).  A device-scope
// poll is served beyond the XCD's L2, and the one-way time of a flag handed
// between two workgroups of one XCD depends on the physical address of the
// line: about 0.44 us on some 2-4 KiB granules and 0.58 us on others, in a
// pattern that repeats every 16 KiB.  Slots a multiple of 16 KiB long share
// their first line's class, and the counter block has one of its own; a
// small message pays the difference at every hand-off.  The FIFO and then
// the counters are moved through `trials` offsets kPlaceStep apart inside
// allocations made that much larger, and each offset is timed by a short
// ping-pong against a reference connection (whose share of the time is the
// same for every trial, in the launch shape the connection itself uses).
constexpr size_t kPlaceStep = size_t(2) << 10;

static int time_trial(xfer_conn* c, xfer_conn* ref, uint8_t* p, size_t msg, hipEvent_t* ev,
                      float* ms) {
  constexpr int kIters = 256;  // round trips timed per trial
  int rc = zero_state(c);
  // a short untimed round first: the timed one starts from a warm state
  if (!rc) rc = xfer_run_pingpong(c, ref, p, p + msg, p + 2 * msg, msg, 16, nullptr);
  hipError_t e = hipSuccess;
  if (!rc) e = hipEventRecord(ev[0], nullptr);
  if (!rc && e == hipSuccess)
    rc = xfer_run_pingpong(c, ref, p, p + msg, p + 2 * msg, msg, kIters, nullptr);
  if (!rc && e == hipSuccess) e = hipEventRecord(ev[1], nullptr);
  if (!rc && e == hipSuccess) e = hipEventSynchronize(ev[1]);
  if (!rc && e == hipSuccess) e = hipEventElapsedTime(ms, ev[0], ev[1]);
  if (!rc && e != hipSuccess) rc = hip_fail(e, "xfer_conn_create: placement trial");
  if (!rc) {
    const uint32_t err = __atomic_load_n(&c->status_host->err, __ATOMIC_ACQUIRE) |
                         __atomic_load_n(&ref->status_host->err, __ATOMIC_ACQUIRE);
    if (err)
      rc = fail(XFER_ERR_INTERNAL, std::string("xfer_conn_create: placement trial failed (") +
                                       xfer_status_string(int(err)) + ")");
  }
  return rc;
}

static int place_by_latency(xfer_conn* c, int proto, int fifo_loc, const xfer_attr& attr,
                            int trials) {
  xfer_attr one = attr;
  one.place_trials = 0;
  xfer_conn* ref = nullptr;
  void* buf = nullptr;
  hipEvent_t ev[2] = {nullptr, nullptr};
  auto finish = [&](int rc) {
    std::string msg = rc ? g_last_error : std::string();
    (void)hipDeviceSynchronize();  // no trial kernel may still use what is freed
    for (hipEvent_t x : ev)
      if (x) (void)hipEventDestroy(x);
    if (buf) (void)hipFree(buf);
    release(ref);
    if (!rc) {
      rc = zero_state(c);
      if (rc) msg = g_last_error;
    }
    return rc ? fail(rc, msg) : XFER_OK;
  };
  int rc = xfer_conn_create_ex(proto, c->nch, c->nslots, c->slot_bytes, fifo_loc, &one, &ref);
  if (rc) return finish(rc);
  DeviceGuard g(c->device);
  const size_t msg = 16 * size_t(c->nch);  // one 16-byte word per channel: every channel is timed
  hipError_t e = hipMalloc(&buf, 3 * msg);
  if (e == hipSuccess) e = hipMemset(buf, 0, 3 * msg);
  if (e == hipSuccess) e = hipEventCreate(&ev[0]);
  if (e == hipSuccess) e = hipEventCreate(&ev[1]);
  if (e != hipSuccess) return finish(hip_fail(e, "xfer_conn_create: placement trial set-up"));
  uint8_t* p = static_cast<uint8_t*>(buf);
  uint8_t* const fifo0 = c->fifo;
  LaneCtrl* const ctrl0 = c->ctrl;
  // the FIFO first (counters at their first offset), then the counters
  for (int what = 0; what < 2; ++what) {
    float best_ms = 0.f;
    int best = 0;
    for (int k = 0; k < trials; ++k) {
      const size_t off = size_t(k) * kPlaceStep;
      if (what == 0) {
        c->fifo = fifo0 + off;
      } else {
        c->ctrl = reinterpret_cast<LaneCtrl*>(reinterpret_cast<uint8_t*>(ctrl0) + off);
        c->ctrl_rx = c->ctrl;
      }
      float ms = 0.f;
      rc = time_trial(c, ref, p, msg, ev, &ms);
      if (rc) return finish(rc);
      if (k == 0 || ms < best_ms) {
        best = k;
        best_ms = ms;
      }
    }
    const size_t off = size_t(best) * kPlaceStep;
    if (what == 0) {
      c->fifo = fifo0 + off;
    } else {
      c->ctrl = reinterpret_cast<LaneCtrl*>(reinterpret_cast<uint8_t*>(ctrl0) + off);
      c->ctrl_rx = c->ctrl;
    }
  }
  return finish(XFER_OK);
}

extern "C" int xfer_conn_create_ex(int proto, int nchannels, int nslots, size_t slot_bytes,
                                   int fifo_loc, const xfer_attr* attr, xfer_conn** out) {
  if (!out) return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: out is NULL");
  *out = nullptr;
  if (proto < XFER_PROTO_SIMPLE || proto > XFER_PROTO_ZEROCOPY_DIRECT)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: unknown protocol " + std::to_string(proto));
  if (nchannels < 1 || nchannels > 64)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: nchannels must be in 1..64");
  if (nslots < 1) return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: nslots must be >= 1");
  const size_t gran = proto == XFER_PROTO_LL ? 8 : 16;
  if (slot_bytes < gran || slot_bytes % gran || slot_bytes > (size_t(1) << 30))
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: slot_bytes must be a positive multiple of " +
                                          std::to_string(gran) + " up to 1 GiB");
  if (fifo_loc != XFER_FIFO_DEVICE && fifo_loc != XFER_FIFO_HOST && fifo_loc != XFER_FIFO_RELAY)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: fifo_loc must be DEVICE, HOST or RELAY");
  if (fifo_loc == XFER_FIFO_RELAY && proto != XFER_PROTO_SIMPLE)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: the relay carries SIMPLE only");
  xfer_attr a;
  memset(&a, 0, sizeof(a));
  if (attr) a = *attr;
  const int lanes = a.wgs_per_channel ? a.wgs_per_channel : 1;
  const int block = a.block_threads ? a.block_threads : kDefaultBlock;
  if (lanes < 1 || lanes > 16)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: wgs_per_channel must be in 1..16");
  if (block < 64 || block > 1024 || block % 64)
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_conn_create: block_threads must be a multiple of 64 in 64..1024");
  if (a.ctrl_loc < XFER_CTRL_DEFAULT || a.ctrl_loc > XFER_CTRL_HOST)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: bad ctrl_loc");
  if (a.xcd_pairing < -1 || a.xcd_pairing > 1)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: xcd_pairing must be -1, 0 or 1");
  if (a.roles < 0 || a.roles > 2)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: roles must be 0, 1 or 2");
  if (a.ordering != XFER_ORDER_COHERENT && a.ordering != XFER_ORDER_FENCED)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: ordering must be COHERENT or FENCED");
  if (fifo_loc == XFER_FIFO_RELAY && a.ctrl_loc == XFER_CTRL_DEVICE)
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_conn_create: a relay's control words live in host memory (its proxies poll "
                "them)");
  if (a.p2p_read != 0 && a.p2p_read != 1)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: p2p_read must be 0 or 1");
  if (a.p2p_read &&
      (proto != XFER_PROTO_SIMPLE || fifo_loc != XFER_FIFO_DEVICE || a.ctrl_loc == XFER_CTRL_HOST))
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_conn_create: P2P read moves the SIMPLE FIFO of a device connection to the "
                "send side (SIMPLE, FIFO and control words in HBM)");
  if (a.place_trials < 0 || a.place_trials > 8)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: place_trials must be in 0..8");
  if (a.cooperative != 0 && a.cooperative != 1)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: cooperative must be 0 or 1");
  if (a.place_trials > 1 && (zero_copy(proto) || fifo_loc != XFER_FIFO_DEVICE ||
                             a.ctrl_loc == XFER_CTRL_HOST || a.p2p_read))
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_conn_create: place_trials needs SIMPLE or LL in write mode with the FIFO "
                "and control words in HBM");
  // Room to move the FIFO and the counter blocks by up to trials-1 steps.
  const size_t place_slack = a.place_trials > 1 ? size_t(a.place_trials - 1) * kPlaceStep : 0;
  const size_t fifo_bytes =
      zero_copy(proto) ? 0 : size_t(nchannels) * size_t(nslots) * slot_bytes;
  if (!zero_copy(proto) && fifo_bytes / size_t(nchannels) / size_t(nslots) != slot_bytes)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_create: FIFO size overflows");

  xfer_conn* c = new (std::nothrow) xfer_conn();
  if (!c) return fail(XFER_ERR_NO_MEMORY, "xfer_conn_create: out of host memory");
  c->proto = proto;
  c->nch = nchannels;
  c->nslots = nslots;
  c->fifo_loc = fifo_loc;
  c->ctrl_loc = a.ctrl_loc == XFER_CTRL_DEFAULT
                    ? (fifo_loc == XFER_FIFO_DEVICE ? XFER_CTRL_DEVICE : XFER_CTRL_HOST)
                    : a.ctrl_loc;
  c->lanes = lanes;
  c->block = block;
  // Pairing by default: in dispatch order producers sit at even block ids,
  // which the hardware deals to XCDs 0, 2, 4 and 6 only; for zero-copy,
  // whose receivers are nearly idle, half the XCDs would do all the copying.
  c->xcd_pairing = a.xcd_pairing == -1 ? 0 : 1;
  c->roles = a.roles == 0 ? 3 : a.roles;
  c->ordering = a.ordering;
  c->p2p_read = a.p2p_read;
  c->coop = a.cooperative == 1;
  c->slot_bytes = slot_bytes;
  c->step_bytes = proto == XFER_PROTO_LL ? slot_bytes / 2 : slot_bytes;
  c->timeout_ms = a.timeout_ms ? a.timeout_ms : kDefaultTimeoutMs;
  c->scope = (fifo_loc == XFER_FIFO_HOST || c->ctrl_loc == XFER_CTRL_HOST) ? kScopeSystem
                                                                            : kScopeAgent;
  c->steps.assign(size_t(nchannels), 0);

  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "hipGetDevice");
  }
  int khz = 0;
  e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, c->device);
  if (e != hipSuccess || khz <= 0) {
    delete c;
    return e != hipSuccess ? hip_fail(e, "hipDeviceGetAttribute(WallClockRate)")
                           : fail(XFER_ERR_HIP, "device reports no wall-clock rate");
  }
  c->timeout_ticks = uint64_t(c->timeout_ms) * uint64_t(khz);
  if (c->xcd_pairing) {
    bool by_id = false;
    const int rc = xcc_remap_ok(c->device, &by_id);
    if (rc) {
      delete c;
      return rc;
    }
    c->xcd_remap = by_id ? 2u : 1u;
  }

  // FIFO: HBM, or pinned host memory mapped into the device (fine-grained,
  // so device accesses reach host memory rather than a non-coherent cache).
  NearNuma near(c->device);  // pinned host blocks below land next to the device
  if (fifo_bytes && !c->p2p_read) {
    if (fifo_loc == XFER_FIFO_HOST) {
      e = hipHostMalloc(&c->fifo_mem, fifo_bytes,
                        hipHostMallocMapped | hipHostMallocCoherent | near.flag());
      if (e != hipSuccess) {
        c->fifo_mem = nullptr;
        release(c);
        return fail(XFER_ERR_NO_MEMORY, std::string("hipHostMalloc(FIFO): ") + hipGetErrorString(e));
      }
      memset(c->fifo_mem, 0, fifo_bytes);
      void* dptr = nullptr;
      e = hipHostGetDevicePointer(&dptr, c->fifo_mem, 0);
      if (e != hipSuccess) {
        release(c);
        return hip_fail(e, "hipHostGetDevicePointer(FIFO)");
      }
      c->fifo = static_cast<uint8_t*>(dptr);
    } else {
      // Large allocations start on large power-of-two boundaries, so every
      // channel's source, slot and destination addresses would share their
      // low bits and meet on the same HBM channels in lock step; the FIFO
      // starts kFifoAlign into its allocation instead (measured 0.2-1 %
      // faster on the 32-channel workload).
      e = hipMalloc(&c->fifo_mem, fifo_bytes + kFifoAlign + place_slack);
      if (e != hipSuccess) {
        c->fifo_mem = nullptr;
        release(c);
        return fail(XFER_ERR_NO_MEMORY, std::string("hipMalloc(FIFO): ") + hipGetErrorString(e));
      }
      c->fifo_alloc = fifo_bytes + kFifoAlign + place_slack;
      e = hipMemset(c->fifo_mem, 0, c->fifo_alloc);
      if (e != hipSuccess) {
        release(c);
        return hip_fail(e, "hipMemset(FIFO)");
      }
      c->fifo = static_cast<uint8_t*>(c->fifo_mem) + kFifoAlign;
    }
  }
  // Control blocks: one per lane, head = tail = ptrExchange = 0.
  const size_t ctrl_bytes = sizeof(LaneCtrl) * size_t(nchannels) * size_t(lanes);
  if (c->p2p_read) {
    // P2P read ("transport建立", p2pSendSetup / p2pRecvConnect listings):
    // the SIMPLE buffer is appended to the send side's memory (its control
    // blocks), which the receive side reads; tail sits in the receive
    // side's own blocks.  Both allocations live in HBM.
    const size_t fifo_off = (ctrl_bytes + kFifoAlign - 1) / kFifoAlign * kFifoAlign;
    const size_t rx_bytes = ctrl_bytes + kErrLine;
    e = hipMalloc(&c->ctrl_mem, fifo_off + fifo_bytes);
    if (e != hipSuccess) {
      c->ctrl_mem = nullptr;
      release(c);
      return fail(XFER_ERR_NO_MEMORY, std::string("hipMalloc(send side): ") + hipGetErrorString(e));
    }
    e = hipMalloc(&c->ctrl_rx_mem, rx_bytes);
    if (e != hipSuccess) {
      c->ctrl_rx_mem = nullptr;
      release(c);
      return fail(XFER_ERR_NO_MEMORY,
                  std::string("hipMalloc(receive side): ") + hipGetErrorString(e));
    }
    c->ctrl_alloc = fifo_off + fifo_bytes;
    c->ctrl_rx_alloc = rx_bytes;
    e = hipMemset(c->ctrl_mem, 0, c->ctrl_alloc);
    if (e == hipSuccess) e = hipMemset(c->ctrl_rx_mem, 0, c->ctrl_rx_alloc);
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipMemset(control blocks)");
    }
    c->ctrl = static_cast<LaneCtrl*>(c->ctrl_mem);
    c->ctrl_rx = static_cast<LaneCtrl*>(c->ctrl_rx_mem);
    c->fifo = static_cast<uint8_t*>(c->ctrl_mem) + fifo_off;
    c->err_dev = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(c->ctrl_rx_mem) + ctrl_bytes);
  } else if (c->ctrl_loc == XFER_CTRL_HOST) {
    e = hipHostMalloc(&c->ctrl_mem, ctrl_bytes + kErrLine,
                      hipHostMallocMapped | hipHostMallocCoherent | near.flag());
    if (e != hipSuccess) {
      c->ctrl_mem = nullptr;
      release(c);
      return fail(XFER_ERR_NO_MEMORY, std::string("hipHostMalloc(ctrl): ") + hipGetErrorString(e));
    }
    memset(c->ctrl_mem, 0, ctrl_bytes + kErrLine);
    void* dptr = nullptr;
    e = hipHostGetDevicePointer(&dptr, c->ctrl_mem, 0);
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipHostGetDevicePointer(ctrl)");
    }
    c->ctrl = static_cast<LaneCtrl*>(dptr);
    c->err_dev = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(dptr) + ctrl_bytes);
  } else {
    e = hipMalloc(&c->ctrl_mem, ctrl_bytes + place_slack + kErrLine);
    if (e != hipSuccess) {
      c->ctrl_mem = nullptr;
      release(c);
      return fail(XFER_ERR_NO_MEMORY, std::string("hipMalloc(ctrl): ") + hipGetErrorString(e));
    }
    c->ctrl_alloc = ctrl_bytes + place_slack + kErrLine;
    e = hipMemset(c->ctrl_mem, 0, c->ctrl_alloc);
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipMemset(ctrl)");
    }
    c->ctrl = static_cast<LaneCtrl*>(c->ctrl_mem);
    c->err_dev = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(c->ctrl_mem) + ctrl_bytes +
                                             place_slack);
  }
  if (!c->p2p_read) c->ctrl_rx = c->ctrl;
  // Claims of the debug launches' logical workgroups, all clear.
  e = hipMalloc(reinterpret_cast<void**>(&c->claims), sizeof(uint64_t) * wgs_of(c));
  if (e != hipSuccess) {
    c->claims = nullptr;
    release(c);
    return fail(XFER_ERR_NO_MEMORY, std::string("hipMalloc(claims): ") + hipGetErrorString(e));
  }
  e = hipMemset(c->claims, 0, sizeof(uint64_t) * wgs_of(c));
  if (e != hipSuccess) {
    release(c);
    return hip_fail(e, "hipMemset(claims)");
  }
  // Status words (error, abort) in pinned host memory.
  void* st = nullptr;
  e = hipHostMalloc(&st, sizeof(Status), hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) {
    release(c);
    return fail(XFER_ERR_NO_MEMORY, std::string("hipHostMalloc(status): ") + hipGetErrorString(e));
  }
  c->status_host = static_cast<Status*>(st);
  memset(c->status_host, 0, sizeof(Status));
  void* sdev = nullptr;
  e = hipHostGetDevicePointer(&sdev, st, 0);
  if (e != hipSuccess) {
    release(c);
    return hip_fail(e, "hipHostGetDevicePointer(status)");
  }
  c->status_dev = static_cast<Status*>(sdev);
  if (fifo_loc == XFER_FIFO_RELAY) {
    // The staging FIFO (pinned host) and the receive FIFO (HBM), both zeroed,
    // then the two proxies.
    e = hipHostMalloc(reinterpret_cast<void**>(&c->stage), fifo_bytes,
                      hipHostMallocDefault | near.flag());
    if (e != hipSuccess) {
      c->stage = nullptr;
      release(c);
      return fail(XFER_ERR_NO_MEMORY, std::string("hipHostMalloc(staging FIFO): ") +
                                          hipGetErrorString(e));
    }
    memset(c->stage, 0, fifo_bytes);
    e = hipMalloc(reinterpret_cast<void**>(&c->fifo_rx), fifo_bytes);
    if (e != hipSuccess) {
      c->fifo_rx = nullptr;
      release(c);
      return fail(XFER_ERR_NO_MEMORY, std::string("hipMalloc(receive FIFO): ") +
                                          hipGetErrorString(e));
    }
    e = hipMemset(c->fifo_rx, 0, fifo_bytes);
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipMemset(receive FIFO)");
    }
    e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      release(c);
      return hip_fail(e, "hipDeviceSynchronize");
    }
    RelayConfig rc;
    rc.device = c->device;
    rc.nch = nchannels;
    rc.lanes = lanes;
    rc.nslots = nslots;
    rc.slot_bytes = slot_bytes;
    rc.step_bytes = c->step_bytes;
    rc.send_fifo = c->fifo;
    rc.stage = c->stage;
    rc.recv_fifo = c->fifo_rx;
    rc.ctrl = static_cast<LaneCtrl*>(c->ctrl_mem);
    rc.status = c->status_host;
    rc.err_mirror = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(c->ctrl_mem) + ctrl_bytes);
    std::string why;
    const int r = relay_start(rc, &c->relay, &why);
    if (r) {
      c->relay = nullptr;
      release(c);
      return fail(r, "xfer_conn_create: " + why);
    }
  }
  e = hipDeviceSynchronize();  // the zeroing above is complete before any run
  if (e != hipSuccess) {
    release(c);
    return hip_fail(e, "hipDeviceSynchronize");
  }
  if (a.place_trials > 1) {
    const int rc = place_by_latency(c, proto, fifo_loc, a, a.place_trials);
    if (rc) {
      const std::string msg = g_last_error;
      release(c);
      return fail(rc, msg);
    }
  }
  *out = c;
  return XFER_OK;
}

extern "C" int xfer_conn_create(int proto, int nchannels, int nslots, size_t slot_bytes,
                                int fifo_loc, xfer_conn** out) {
  return xfer_conn_create_ex(proto, nchannels, nslots, slot_bytes, fifo_loc, nullptr, out);
}

extern "C" int xfer_conn_destroy(xfer_conn* c) {
  release(c);
  return XFER_OK;
}

// Runs of a traced or jittered connection take the debug kernel variant.
static bool debug_of(const xfer_conn* c) { return c->trace != nullptr || c->jitter != 0; }

// The kernel protocol of c: LL connections in the striped line layout run
// kernels of their own.
static int kernel_proto(const xfer_conn* c) {
  if (c->proto != XFER_PROTO_LL) return c->proto;
  uint32_t l2 = 0, group = 0;
  ll_layout(c->step_bytes, uint32_t(c->lanes), uint32_t(c->block), uint32_t(c->nslots), &l2,
            &group);
  return l2 ? int(kProtoLLStriped) : int(kProtoLL);
}

Variant variant_of(const xfer_conn* c, bool aligned) {
  return Variant{kernel_proto(c), c->scope, c->ordering, aligned ? 1 : 0, debug_of(c) ? 1 : 0};
}

extern "C" int xfer_run_loop(xfer_conn* c, const void* src, void* dst, size_t nbytes, int iters,
                             void* stream) {
  int rc = check_runnable(c, "xfer_run");
  if (rc) return rc;
  if (iters < 1) return fail(XFER_ERR_INVALID_ARG, "xfer_run_loop: iters must be >= 1");
  if (nbytes == 0) return XFER_OK;
  if (!src || !dst) return fail(XFER_ERR_INVALID_ARG, "xfer_run: NULL src or dst with nbytes > 0");
  if (overlap(src, nbytes, dst, nbytes))
    return fail(XFER_ERR_INVALID_ARG, "xfer_run: src and dst overlap");
  std::vector<uint64_t>& add = c->add;  // reused: no allocation per run
  rc = plan_steps(c, nbytes, uint64_t(iters), add, "xfer_run");
  if (rc) return rc;
  DeviceGuard g(c->device);
  const uint32_t total = grid_of(c, wgs_of(c));
  const Variant v = variant_of(c, aligned16(src) && aligned16(dst));
  rc = check_resident(c->device, v, 0, c->block, total, "xfer_run",
                      &c->cap_one[v.aligned][v.debug]);
  if (rc) return rc;
  RunOne args;
  memset(&args, 0, sizeof(args));
  args.conn[0] = conn_args(c, src, dst, nbytes, 0);
  args.nconn = 1;
  args.iters = uint32_t(iters);
  args.total_wgs = total;
  args.xcd_remap = c->xcd_remap;
  args.timeout_ticks = c->timeout_ticks;
  args.rx_wgs = rx_region_of(c);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e =
      gate().run(c->device, s, [&] { return launch_run1(v, args, c->block, s, c->coop); });
  if (e != hipSuccess) return hip_fail(e, "xfer_run launch");
  relay_job(c, {uint64_t(nbytes)}, uint64_t(iters));
  commit_steps(c, add);
  return XFER_OK;
}

extern "C" int xfer_run(xfer_conn* c, const void* src, void* dst, size_t nbytes, void* stream) {
  return xfer_run_loop(c, src, dst, nbytes, 1, stream);
}

extern "C" int xfer_run_messages(xfer_conn* c, const void* src, void* dst, const size_t* offsets,
                                 const size_t* sizes, int n, void* stream) {
  int rc = check_runnable(c, "xfer_run_messages");
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!offsets || !sizes)))
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_messages: need n >= 0 and offset/size arrays");
  // The span every message lies in, for the NULL and overlap checks.
  size_t lo = SIZE_MAX, hi = 0;
  std::vector<MsgDesc> msgs;
  msgs.reserve(size_t(n));
  for (int i = 0; i < n; ++i) {
    if (sizes[i] == 0) continue;
    if (offsets[i] > SIZE_MAX - sizes[i])
      return fail(XFER_ERR_INVALID_ARG, "xfer_run_messages: offset + size overflows");
    lo = std::min(lo, offsets[i]);
    hi = std::max(hi, offsets[i] + sizes[i]);
    msgs.push_back(MsgDesc{uint64_t(offsets[i]), uint64_t(sizes[i])});
  }
  if (msgs.empty()) return XFER_OK;
  if (!src || !dst)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_messages: NULL src or dst with bytes to move");
  {
    // Channels reach different messages at different times, so two messages
    // that write the same bytes would race; sequential runs would not.
    std::vector<MsgDesc> by_off(msgs);
    std::sort(by_off.begin(), by_off.end(),
              [](const MsgDesc& a, const MsgDesc& b) { return a.off < b.off; });
    for (size_t i = 1; i < by_off.size(); ++i)
      if (by_off[i - 1].off + by_off[i - 1].len > by_off[i].off)
        return fail(XFER_ERR_INVALID_ARG, "xfer_run_messages: two messages overlap");
  }
  if (overlap(static_cast<const uint8_t*>(src) + lo, hi - lo, static_cast<uint8_t*>(dst) + lo,
              hi - lo))
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_messages: src and dst ranges overlap");
  std::vector<uint64_t> add(size_t(c->nch), 0), one;
  bool aligned = aligned16(src) && aligned16(dst);
  for (const MsgDesc& m : msgs) {
    rc = plan_steps(c, m.len, 1, one, "xfer_run_messages");
    if (rc) return rc;
    for (int ch = 0; ch < c->nch; ++ch) {
      add[size_t(ch)] += one[size_t(ch)];
      if (c->proto == XFER_PROTO_LL && c->steps[size_t(ch)] + add[size_t(ch)] > 0xFFFFFFFFull)
        return fail(XFER_ERR_RANGE, "xfer_run_messages: LL connection would pass 2^32-1 steps");
    }
    aligned = aligned && (m.off & 15u) == 0;
  }
  DeviceGuard g(c->device);
  const uint32_t total = grid_of(c, wgs_of(c));
  const Variant v = variant_of(c, aligned);
  rc = check_resident(c->device, v, 3, c->block, total, "xfer_run_messages");
  if (rc) return rc;
  RunList args;
  for (size_t first = 0; first < msgs.size(); first += kMaxMsgs) {
    const size_t cnt = std::min<size_t>(kMaxMsgs, msgs.size() - first);
    memset(&args, 0, sizeof(args));
    args.conn[0] = conn_args(c, src, dst, 0, 0);
    args.nconn = 1;
    args.iters = 1;
    args.total_wgs = total;
    args.xcd_remap = c->xcd_remap;
    args.timeout_ticks = c->timeout_ticks;
    args.nmsgs = uint32_t(cnt);
    args.rx_wgs = rx_region_of(c);
    for (size_t i = 0; i < cnt; ++i) args.msgs[i] = msgs[first + i];
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e =
        gate().run(c->device, s, [&] { return launch_runL(v, args, c->block, s, c->coop); });
    if (e != hipSuccess) return hip_fail(e, "xfer_run_messages launch");
  }
  if (c->relay) {
    std::vector<uint64_t> lens;
    lens.reserve(msgs.size());
    for (const MsgDesc& m : msgs) lens.push_back(m.len);
    relay_job(c, std::move(lens), 1);
  }
  commit_steps(c, add);
  return XFER_OK;
}

extern "C" int xfer_run_batch(xfer_conn* const* conns, const void* const* src, void* const* dst,
                              const size_t* nbytes, int n, void* stream) {
  if (n < 1 || n > XFER_MAX_BATCH || !conns || !src || !dst || !nbytes)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_batch: need 1 <= n <= XFER_MAX_BATCH and arrays");
  std::vector<std::vector<uint64_t>> adds(static_cast<size_t>(n));
  RunBatch args;
  memset(&args, 0, sizeof(args));
  uint32_t total = 0;  // workgroups (zero-copy: producer workgroups)
  uint32_t rx_total = 0;  // zero-copy: receiver workgroups, dispatched before every producer
  bool aligned = true;
  int live = 0;
  const xfer_conn* first = nullptr;
  for (int i = 0; i < n; ++i) {
    xfer_conn* c = conns[i];
    int rc = check_runnable(c, "xfer_run_batch");
    if (rc) return rc;
    for (int j = 0; j < i; ++j)
      if (conns[j] == c) return fail(XFER_ERR_INVALID_ARG, "xfer_run_batch: a connection appears twice");
    if (!first) first = c;
    if (kernel_proto(c) != kernel_proto(first) || c->scope != first->scope ||
        c->ordering != first->ordering || c->block != first->block || c->coop != first->coop ||
        c->timeout_ticks != first->timeout_ticks || c->device != first->device)
      return fail(XFER_ERR_INVALID_ARG,
                  "xfer_run_batch: connections must share protocol (for LL, its line layout), "
                  "memory scope, ordering, block size, timeout and device");
    if (nbytes[i] == 0) continue;
    if (!src[i] || !dst[i])
      return fail(XFER_ERR_INVALID_ARG, "xfer_run_batch: NULL src or dst with nbytes > 0");
    if (overlap(src[i], nbytes[i], dst[i], nbytes[i]))
      return fail(XFER_ERR_INVALID_ARG, "xfer_run_batch: src and dst overlap");
    rc = plan_steps(c, nbytes[i], 1, adds[size_t(i)], "xfer_run_batch");
    if (rc) return rc;
    aligned = aligned && aligned16(src[i]) && aligned16(dst[i]);
    args.conn[live] = conn_args(c, src[i], dst[i], nbytes[i], total, rx_total);
    rx_total += rx_wgs_of(c);
    total += wgs_of(c) - rx_wgs_of(c);
    ++live;
  }
  if (!live) return XFER_OK;
  // The connections' channels run in no fixed order against each other, so
  // a destination that another transfer also writes or reads would race.
  for (int i = 0; i < n; ++i) {
    if (!nbytes[i]) continue;
    for (int j = 0; j < n; ++j) {
      if (j == i || !nbytes[j]) continue;
      if ((j > i && overlap(dst[i], nbytes[i], dst[j], nbytes[j])) ||
          overlap(dst[i], nbytes[i], src[j], nbytes[j]))
        return fail(XFER_ERR_INVALID_ARG,
                    "xfer_run_batch: transfer " + std::to_string(i) +
                        "'s destination overlaps transfer " + std::to_string(j) +
                        (overlap(dst[i], nbytes[i], dst[j], nbytes[j]) ? "'s destination"
                                                                       : "'s source"));
    }
  }
  DeviceGuard g(first->device);
  Variant v = variant_of(first, aligned);
  for (int i = 0; i < n; ++i)
    if (debug_of(conns[i])) v.debug = 1;  // the others pass no buffer and no seed
  uint32_t rx_region = 0;
  const uint32_t grid = zero_copy(first->proto) ? zc_grid(first, rx_total, total, &rx_region)
                                                : grid_of(first, total);
  int rc = check_resident(first->device, v, 1, first->block, grid, "xfer_run_batch");
  if (rc) return rc;
  args.nconn = uint32_t(live);
  args.iters = 1;
  args.total_wgs = grid;
  args.xcd_remap = first->xcd_remap;
  args.timeout_ticks = first->timeout_ticks;
  args.rx_wgs = rx_region;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e =
      gate().run(first->device, s,
                 [&] { return launch_runB(v, args, first->block, s, first->coop); });
  if (e != hipSuccess) return hip_fail(e, "xfer_run_batch launch");
  for (int i = 0; i < n; ++i) {
    if (!nbytes[i]) continue;
    relay_job(conns[i], {uint64_t(nbytes[i])}, 1);
    commit_steps(conns[i], adds[size_t(i)]);
  }
  return XFER_OK;
}

extern "C" int xfer_run_pingpong(xfer_conn* fwd, xfer_conn* rev, const void* a, void* b, void* cbuf,
                                 size_t nbytes, int iters, void* stream) {
  int rc = check_runnable(fwd, "xfer_run_pingpong");
  if (rc) return rc;
  rc = check_runnable(rev, "xfer_run_pingpong");
  if (rc) return rc;
  if (fwd == rev) return fail(XFER_ERR_INVALID_ARG, "xfer_run_pingpong: fwd and rev must differ");
  if (zero_copy(fwd->proto) || fwd->proto != rev->proto || fwd->nch != rev->nch ||
      fwd->slot_bytes != rev->slot_bytes || fwd->lanes != rev->lanes || fwd->block != rev->block ||
      fwd->ordering != rev->ordering || fwd->device != rev->device || fwd->relay || rev->relay ||
      fwd->coop != rev->coop)
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_run_pingpong: fwd and rev must be SIMPLE or LL with equal channels, slot "
                "size, lanes, block size, ordering and device, and no relay");
  if (iters < 1) return fail(XFER_ERR_INVALID_ARG, "xfer_run_pingpong: iters must be >= 1");
  if (nbytes == 0) return XFER_OK;
  if (!a || !b || !cbuf)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_pingpong: NULL buffer with nbytes > 0");
  if (overlap(a, nbytes, b, nbytes) || overlap(b, nbytes, cbuf, nbytes) ||
      overlap(a, nbytes, cbuf, nbytes))
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_pingpong: buffers overlap");
  std::vector<uint64_t> addf, addr;
  rc = plan_steps(fwd, nbytes, uint64_t(iters), addf, "xfer_run_pingpong");
  if (rc) return rc;
  rc = plan_steps(rev, nbytes, uint64_t(iters), addr, "xfer_run_pingpong");
  if (rc) return rc;
  DeviceGuard g(fwd->device);
  const uint32_t total = grid_of(fwd, wgs_of(fwd));
  const int scope = (fwd->scope == kScopeSystem || rev->scope == kScopeSystem) ? kScopeSystem
                                                                               : kScopeAgent;
  const Variant v{kernel_proto(fwd), scope, fwd->ordering,
                  (aligned16(a) && aligned16(b) && aligned16(cbuf)) ? 1 : 0,
                  (debug_of(fwd) || debug_of(rev)) ? 1 : 0};
  rc = check_resident(fwd->device, v, 2, fwd->block, total, "xfer_run_pingpong");
  if (rc) return rc;
  PingArgs args;
  memset(&args, 0, sizeof(args));
  args.fwd = conn_args(fwd, a, b, nbytes, 0);
  args.rev = conn_args(rev, b, cbuf, nbytes, 0);
  args.iters = uint32_t(iters);
  args.total_wgs = total;
  args.xcd_remap = fwd->xcd_remap;
  args.timeout_ticks = std::max(fwd->timeout_ticks, rev->timeout_ticks);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e =
      gate().run(fwd->device, s, [&] { return launch_ping(v, args, fwd->block, s, fwd->coop); });
  if (e != hipSuccess) return hip_fail(e, "xfer_run_pingpong launch");
  commit_steps(fwd, addf);
  commit_steps(rev, addr);
  return XFER_OK;
}

extern "C" int xfer_conn_query(const xfer_conn* c, int channel, xfer_chan_state* out) {
  if (!c || !out || channel < 0 || channel >= c->nch)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_query: bad connection, channel or out");
  // head and ptrExchange from the send side's blocks, tail from the receive
  // side's (one and the same array unless the connection reads P2P)
  std::vector<LaneCtrl> tx(static_cast<size_t>(c->lanes)), rx(static_cast<size_t>(c->lanes));
  const size_t first = size_t(channel) * size_t(c->lanes);
  const size_t bytes = sizeof(LaneCtrl) * size_t(c->lanes);
  if (c->ctrl_loc == XFER_CTRL_HOST) {
    memcpy(tx.data(), static_cast<const LaneCtrl*>(c->ctrl_mem) + first, bytes);
    rx = tx;
  } else {
    DeviceGuard g(c->device);
    hipError_t e = hipMemcpy(tx.data(), c->ctrl + first, bytes, hipMemcpyDeviceToHost);
    if (e == hipSuccess)
      e = hipMemcpy(rx.data(), c->ctrl_rx + first, bytes, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "xfer_conn_query: hipMemcpy");
  }
  memset(out, 0, sizeof(*out));
  out->head = tx[0].head;
  out->tail = rx[0].tail;
  out->ptr_exchange = tx[0].ptrx;
  out->steps = c->steps[size_t(channel)];
  out->lanes = c->lanes;
  out->lanes_agree = 1;
  for (size_t w = 0; w < tx.size(); ++w)
    if (tx[w].head != tx[0].head || rx[w].tail != rx[0].tail || tx[w].ptrx != tx[0].ptrx)
      out->lanes_agree = 0;
  out->error = int(__atomic_load_n(&c->status_host->err, __ATOMIC_ACQUIRE));
  return XFER_OK;
}

extern "C" int xfer_conn_fifo(const xfer_conn* c, int channel, void** fifo, size_t* bytes) {
  if (!c || !fifo || !bytes || channel < 0 || channel >= c->nch)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_fifo: bad connection, channel or outputs");
  if (!c->fifo) {
    *fifo = nullptr;
    *bytes = 0;
    return XFER_OK;
  }
  *bytes = size_t(c->nslots) * c->slot_bytes;
  *fifo = c->fifo + size_t(channel) * (*bytes);
  return XFER_OK;
}

extern "C" int xfer_conn_read_fifo(const xfer_conn* c, int channel, void* host_dst, size_t bytes) {
  void* f = nullptr;
  size_t n = 0;
  int rc = xfer_conn_fifo(c, channel, &f, &n);
  if (rc) return rc;
  if (bytes != n || (n && !host_dst))
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_read_fifo: bytes must equal the FIFO size");
  if (!n) return XFER_OK;
  if (c->fifo_loc == XFER_FIFO_HOST) {
    memcpy(host_dst, static_cast<const uint8_t*>(c->fifo_mem) + size_t(channel) * n, n);
    return XFER_OK;
  }
  DeviceGuard g(c->device);
  hipError_t e = hipMemcpy(host_dst, f, n, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "xfer_conn_read_fifo: hipMemcpy");
  return XFER_OK;
}

extern "C" int xfer_conn_read_fifo_ex(const xfer_conn* c, int which, int channel, void* host_dst,
                                      size_t bytes) {
  if (!c || channel < 0 || channel >= c->nch || which < 0 || which > 2 ||
      (which > 0 && !c->relay))
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_conn_read_fifo_ex: bad connection or channel, or which not in 0..2 (1 and "
                "2 need a relay)");
  if (which == 0) return xfer_conn_read_fifo(c, channel, host_dst, bytes);
  const size_t n = size_t(c->nslots) * c->slot_bytes;
  if (bytes != n || !host_dst)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_read_fifo_ex: bytes must equal the FIFO size");
  if (which == 1) {
    memcpy(host_dst, c->stage + size_t(channel) * n, n);
    return XFER_OK;
  }
  DeviceGuard g(c->device);
  hipError_t e = hipMemcpy(host_dst, c->fifo_rx + size_t(channel) * n, n, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "xfer_conn_read_fifo_ex: hipMemcpy");
  return XFER_OK;
}

extern "C" int xfer_conn_query_relay(const xfer_conn* c, int channel, uint64_t* send_proxy_tail,
                                     uint64_t* recv_proxy_tail) {
  if (!c || !c->relay || channel < 0 || channel >= c->nch || !send_proxy_tail || !recv_proxy_tail)
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_conn_query_relay: needs a relay connection, a channel and two outputs");
  const LaneCtrl* l = static_cast<const LaneCtrl*>(c->ctrl_mem) + size_t(channel) * size_t(c->lanes);
  *send_proxy_tail = __atomic_load_n(&l[0].ytail, __ATOMIC_ACQUIRE);
  *recv_proxy_tail = __atomic_load_n(&l[0].gtail, __ATOMIC_ACQUIRE);
  return XFER_OK;
}

extern "C" int xfer_conn_set_trace(xfer_conn* c, void* records, size_t nrecords) {
  if (!c) return fail(XFER_ERR_INVALID_ARG, "xfer_conn_set_trace: NULL connection");
  if (!records) {
    c->trace = nullptr;
    c->trace_per = 0;
    return XFER_OK;
  }
  if (reinterpret_cast<uintptr_t>(records) % alignof(TraceRec))
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_set_trace: records must be 8-byte aligned");
  const size_t rings = size_t(c->nch) * size_t(c->lanes) * 2;
  const size_t per = nrecords / rings;
  if (per < 2 || per > 0xFFFFFFFFu)
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_conn_set_trace: need at least 2 records per channel, lane and side (" +
                    std::to_string(2 * rings) + " in all)");
  c->trace = static_cast<TraceRec*>(records);
  c->trace_per = uint32_t(per);
  return XFER_OK;
}

extern "C" int xfer_conn_set_jitter(xfer_conn* c, uint32_t seed) {
  if (!c) return fail(XFER_ERR_INVALID_ARG, "xfer_conn_set_jitter: NULL connection");
  c->jitter = seed;
  return XFER_OK;
}

extern "C" int xfer_conn_abort(xfer_conn* c) {
  if (!c) return fail(XFER_ERR_INVALID_ARG, "xfer_conn_abort: NULL connection");
  __atomic_store_n(&c->status_host->abort_flag, 1u, __ATOMIC_RELEASE);
  return XFER_OK;
}

extern "C" int xfer_conn_launch_shape(const xfer_conn* c, int* workgroups, int* block_threads) {
  if (!c || !workgroups || !block_threads)
    return fail(XFER_ERR_INVALID_ARG, "xfer_conn_launch_shape: NULL argument");
  *workgroups = int(grid_of(c, wgs_of(c)));
  *block_threads = c->block;
  return XFER_OK;
}

extern "C" int xfer_endpoints_connect(int nranks, const uint64_t* recv_masks,
                                      const uint64_t* send_masks, int max_peers, int proto,
                                      int nslots, size_t slot_bytes, int fifo_loc,
                                      const xfer_attr* attr, xfer_conn** edges, int* nedges) {
  if (nranks < 1 || nranks > 4096 || !recv_masks || !send_masks || !edges || !nedges ||
      max_peers < 1)
    return fail(XFER_ERR_INVALID_ARG, "xfer_endpoints_connect: bad arguments");
  const size_t nn = size_t(nranks) * size_t(nranks);
  for (size_t i = 0; i < nn; ++i) edges[i] = nullptr;
  *nedges = 0;
  // Every rank's plan.
  std::vector<std::vector<xfer_setup_op>> plans(static_cast<size_t>(nranks));
  for (int r = 0; r < nranks; ++r) {
    int nops = 0;
    const uint64_t* rm = recv_masks + size_t(r) * size_t(nranks);
    const uint64_t* sm = send_masks + size_t(r) * size_t(nranks);
    xfer_sched_plan(r, nranks, rm, sm, max_peers, nullptr, 0, &nops);
    plans[size_t(r)].resize(size_t(nops));
    int rc = xfer_sched_plan(r, nranks, rm, sm, max_peers, plans[size_t(r)].data(), nops, &nops);
    if (rc) return rc;
  }
  // Receive-side setups, as (receiver, sender) -> channel mask.
  std::vector<uint64_t> recv_set(nn, uint64_t(0)), send_set(nn, uint64_t(0));
  for (int d = 0; d < nranks; ++d)
    for (const xfer_setup_op& op : plans[size_t(d)])
      if (op.kind == XFER_OP_RECV_SETUP)
        recv_set[size_t(d) * size_t(nranks) + size_t(op.peer)] |= uint64_t(1) << op.channel;
  auto undo = [&]() {
    for (size_t i = 0; i < nn; ++i) {
      xfer_conn_destroy(edges[i]);
      edges[i] = nullptr;
    }
    *nedges = 0;
  };
  for (int s = 0; s < nranks; ++s) {
    std::vector<int> pending;  // send peers set up since the last connect batch
    for (const xfer_setup_op& op : plans[size_t(s)]) {
      if (op.kind == XFER_OP_SEND_SETUP) {
        const size_t e = size_t(s) * size_t(nranks) + size_t(op.peer);
        if (!(recv_set[size_t(op.peer) * size_t(nranks) + size_t(s)] & (uint64_t(1) << op.channel))) {
          undo();
          return fail(XFER_ERR_INVALID_ARG,
                      "xfer_endpoints_connect: rank " + std::to_string(s) + " sends to rank " +
                          std::to_string(op.peer) + " on channel " + std::to_string(op.channel) +
                          " but that rank sets up no matching receive");
        }
        if (!send_set[e]) pending.push_back(op.peer);
        send_set[e] |= uint64_t(1) << op.channel;
      } else if (op.kind == XFER_OP_CONNECT_BATCH) {
        for (int d : pending) {
          const size_t e = size_t(s) * size_t(nranks) + size_t(d);
          const int nch = __builtin_popcountll(send_set[e]);
          int rc = xfer_conn_create_ex(proto, nch, nslots, slot_bytes, fifo_loc, attr, &edges[e]);
          if (rc) {
            const std::string msg = g_last_error;
            undo();
            return fail(rc, "xfer_endpoints_connect: " + msg);
          }
          ++*nedges;
        }
        pending.clear();
      }
    }
  }
  for (size_t i = 0; i < nn; ++i) {
    const size_t s = i % size_t(nranks), d = i / size_t(nranks);  // recv_set is [d][s]
    if (recv_set[i] != send_set[s * size_t(nranks) + d]) {
      undo();
      return fail(XFER_ERR_INVALID_ARG, "xfer_endpoints_connect: rank " + std::to_string(d) +
                                            " receives from rank " + std::to_string(s) +
                                            " on channels the sender does not set up");
    }
  }
  return XFER_OK;
}
