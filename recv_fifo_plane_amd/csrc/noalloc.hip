// xfer_run_noalloc: one transfer whose FIFO, control blocks and status words
// live in a fixed device array of this library instead of a connection's
// own allocations, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).  The
// transfer runs the same kernels as xfer_run on a new connection of the
// same shape, so its destination bytes are those of xfer_run.
//
// The array is per GPU (each device holds its own copy of a __device__
// variable) and is reached through the address hipGetSymbolAddress returns
// on that device, taken once per device at the first call.  Every call on a
// GPU uses the whole of that GPU's array: calls that overlap in time on one
// GPU race, and each call first clears what a new connection starts with at
// zero (counters, status words, and for LL the FIFO lines, whose flags
// would otherwise match the restarted step numbers).
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "xfer.h"
#include "xfer_internal.h"

namespace xfer {

void set_error(int code, const std::string& msg);  // conn.cpp

namespace {

constexpr size_t kScratchBytes = size_t(XFER_NOALLOC_SCRATCH_BYTES);
// Layout of the array: the status block, the failure mirror on its own
// line, the control blocks, and the FIFO from 1 MiB on.
constexpr size_t kStatusOff = 0, kErrOff = 256, kCtrlOff = 1024;
constexpr size_t kFifoOff = size_t(1) << 20;
constexpr size_t kMaxCtrl = size_t(64) * 16 * sizeof(LaneCtrl);  // 64 channels x 16 lanes
static_assert(sizeof(Status) <= kErrOff - kStatusOff, "status block layout");
static_assert(kCtrlOff + kMaxCtrl <= kFifoOff, "control blocks fit below the FIFO");
static_assert(kFifoOff < kScratchBytes, "room for a FIFO");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Zeroes na words from a, then nb words from b (plain vector stores; the
// transfer kernel that follows on the stream sees them at its start).
__global__ void clear_kernel(uint64_t* a, uint64_t na, uint64_t* b, uint64_t nb) {
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  for (uint64_t i = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < na + nb; i += stride) {
    if (i < na)
      a[i] = 0;
    else
      b[i - na] = 0;
  }
}

// Copies the transfer's failure code (0 = none) to the caller's word.
__global__ void report_kernel(const Status* st, uint32_t* out) {
  if (threadIdx.x == 0) {
    const uint32_t e = __hip_atomic_load(const_cast<uint32_t*>(&st->err), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(out, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

constexpr int kMaxDevices = 64;
constexpr int kBlocks = 16;  // block sizes 64, 128, ..., 1024

// Per device: the array's device address and the wall-clock rate (taken at
// the first call), and the resident capacity of each kernel variant and
// block size (queried on its first use).  Fixed tables: nothing here
// allocates.
struct DevState {
  bool ready;
  uint8_t* base;
  uint64_t khz;
  int cap[5][2][2][kBlocks];  // [kernel proto][ordering][aligned][block / 64 - 1]; 0 = not queried
};
DevState g_dev[kMaxDevices];
std::mutex g_mu;

int fail(int code, const char* msg) {
  set_error(code, msg);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  set_error(XFER_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return XFER_ERR_HIP;
}

// Set-up of the current device `dev`, once.
int setup(int dev, DevState** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  DevState& d = g_dev[dev];
  if (!d.ready) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "xfer_run_noalloc: hipGetSymbolAddress(scratch)");
    int khz = 0;
    e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return hip_fail(e, "xfer_run_noalloc: wall-clock rate");
    if (khz <= 0) return fail(XFER_ERR_HIP, "xfer_run_noalloc: device reports no wall-clock rate");
    d.base = static_cast<uint8_t*>(p);
    d.khz = uint64_t(khz);
    d.ready = true;
  }
  *out = &d;
  return XFER_OK;
}

int capacity(DevState* d, const Variant& v, int block, int* cap) {
  std::lock_guard<std::mutex> lk(g_mu);
  int& c = d->cap[v.proto][v.ordering][v.aligned][block / 64 - 1];
  if (c == 0) {
    int n = 0;
    const hipError_t e = max_resident(v, 0, block, &n);
    if (e != hipSuccess) return hip_fail(e, "xfer_run_noalloc: hipOccupancyMaxActiveBlocksPerMultiprocessor");
    c = n > 0 ? n : -1;
  }
  *cap = c;
  return XFER_OK;
}

// hipLaunchKernel reports this launch's own status (no sticky error state).
template <typename... Args>
hipError_t launch(void (*fn)(Args...), uint32_t grid, uint32_t block, hipStream_t s,
                  Args... args) {
  void* kargs[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(block), kargs, 0, s);
}

bool overlap(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

}  // namespace
}  // namespace xfer

using namespace xfer;

extern "C" int xfer_run_noalloc(int proto, int nchannels, int nslots, size_t slot_bytes,
                                const xfer_attr* attr, const void* src, void* dst, size_t nbytes,
                                uint32_t* status, void* stream) {
  // The domain of xfer_conn_create_ex, restricted to what the array holds:
  // FIFO and control words in HBM, write mode, no placement trials.
  if (proto < XFER_PROTO_SIMPLE || proto > XFER_PROTO_ZEROCOPY_DIRECT)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: unknown protocol");
  if (nchannels < 1 || nchannels > 64)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: nchannels must be in 1..64");
  if (nslots < 1) return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: nslots must be >= 1");
  const size_t gran = proto == XFER_PROTO_LL ? 8 : 16;
  if (slot_bytes < gran || slot_bytes % gran || slot_bytes > (size_t(1) << 30))
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_run_noalloc: slot_bytes must be a positive multiple of 16 (LL: 8) up to "
                "1 GiB");
  xfer_attr a;
  memset(&a, 0, sizeof(a));
  if (attr) a = *attr;
  const int lanes = a.wgs_per_channel ? a.wgs_per_channel : 1;
  const int block = a.block_threads ? a.block_threads : 256;
  if (lanes < 1 || lanes > 16)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: wgs_per_channel must be in 1..16");
  if (block < 64 || block > 1024 || block % 64)
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_run_noalloc: block_threads must be a multiple of 64 in 64..1024");
  if (a.xcd_pairing < -1 || a.xcd_pairing > 1)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: xcd_pairing must be -1, 0 or 1");
  if (a.ordering != XFER_ORDER_COHERENT && a.ordering != XFER_ORDER_FENCED)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: ordering must be COHERENT or FENCED");
  if ((a.ctrl_loc != XFER_CTRL_DEFAULT && a.ctrl_loc != XFER_CTRL_DEVICE) || a.roles != 0 ||
      a.p2p_read != 0 || a.place_trials < 0 || a.place_trials > 1 || a.cooperative != 0)
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_run_noalloc: control words stay in HBM, both roles run, no P2P read, no "
                "placement trials and no cooperative launch");
  const bool zc = proto == XFER_PROTO_ZEROCOPY || proto == XFER_PROTO_ZEROCOPY_DIRECT;
  const uint64_t room = kScratchBytes - kFifoOff;
  const uint64_t per_ch = zc ? 0 : uint64_t(nslots) * slot_bytes;
  if (!zc && (per_ch / uint64_t(nslots) != slot_bytes || per_ch > room ||
              per_ch * uint64_t(nchannels) > room))
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_run_noalloc: nchannels x nslots x slot_bytes exceeds the FIFO room of the "
                "fixed array (XFER_NOALLOC_SCRATCH_BYTES less 1 MiB)");
  const uint64_t fifo_bytes = per_ch * uint64_t(nchannels);
  if (nbytes == 0) return XFER_OK;
  if (!src || !dst) return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: NULL src or dst");
  if (overlap(src, dst, nbytes))
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: src and dst overlap");
  const uint64_t step = proto == XFER_PROTO_LL ? slot_bytes / 2 : slot_bytes;
  if (proto == XFER_PROTO_LL) {
    // the largest channel range: ceil(n / nch) rounded up to 16 bytes
    uint64_t per = (uint64_t(nbytes) + uint64_t(nchannels) - 1) / uint64_t(nchannels);
    per = (per + 15) & ~uint64_t(15);
    if ((per + step - 1) / step > 0xFFFFFFFFull)
      return fail(XFER_ERR_RANGE, "xfer_run_noalloc: LL transfer would pass 2^32-1 steps");
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "xfer_run_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(XFER_ERR_INVALID_ARG, "xfer_run_noalloc: device index beyond 63");
  DevState* d = nullptr;
  int rc = setup(dev, &d);
  if (rc) return rc;
  const bool aligned = (reinterpret_cast<uintptr_t>(src) & 15u) == 0 &&
                       (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
  // (the public protocol numbers are the kernels' own; striped LL has its own)
  uint32_t ll_l2 = 0, ll_group = 0;
  if (proto == XFER_PROTO_LL)
    ll_layout(step, uint32_t(lanes), uint32_t(block), uint32_t(nslots), &ll_l2, &ll_group);
  const Variant v{ll_l2 ? int(kProtoLLStriped) : proto, kScopeAgent, a.ordering, aligned ? 1 : 0,
                  0};
  // Pairs placed on one XCD by block id (the XCD-id placement needs a
  // device probe that allocates, so it is not used here); zero-copy
  // launches have no pairs.
  const bool pairing = a.xcd_pairing != -1;
  const uint32_t wgs = conn_wgs(proto, uint32_t(nchannels), uint32_t(lanes), uint32_t(block));
  const uint32_t rx = zc ? zc_receiver_wgs(uint32_t(nchannels), uint32_t(lanes), uint32_t(block))
                         : 0u;
  // zero-copy grouping pads the receiver and producer regions to 8 blocks each
  const uint32_t rx_region = pairing ? (rx + 7u) & ~7u : rx;
  const uint32_t grid = !pairing ? wgs
                        : zc     ? rx_region + ((wgs - rx + 7u) & ~7u)
                                 : (wgs + 15u) & ~15u;
  int cap = 0;
  rc = capacity(d, v, block, &cap);
  if (rc) return rc;
  if (int64_t(grid) > int64_t(cap))
    return fail(XFER_ERR_INVALID_ARG,
                "xfer_run_noalloc: more workgroups than the GPU holds resident at once");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* base = d->base;
  const uint64_t ctrl_bytes = uint64_t(nchannels) * uint64_t(lanes) * sizeof(LaneCtrl);
  const uint64_t na = (kCtrlOff + ctrl_bytes) / 8;
  const uint64_t nb = proto == XFER_PROTO_LL ? fifo_bytes / 8 : 0;
  const uint64_t cblocks = std::min<uint64_t>(1024, (na + nb + 255) / 256);
  e = launch(clear_kernel, uint32_t(cblocks), 256, s, reinterpret_cast<uint64_t*>(base), na,
             reinterpret_cast<uint64_t*>(base + kFifoOff), nb);
  if (e != hipSuccess) return hip_fail(e, "xfer_run_noalloc: clear launch");
  RunOne args;
  memset(&args, 0, sizeof(args));
  ConnArgs& c = args.conn[0];
  c.fifo = zc ? nullptr : base + kFifoOff;
  c.fifo_rx = c.fifo;
  c.ctrl_tx = reinterpret_cast<LaneCtrl*>(base + kCtrlOff);
  c.ctrl_rx = c.ctrl_tx;
  c.status = reinterpret_cast<Status*>(base + kStatusOff);
  c.err_dev = reinterpret_cast<uint32_t*>(base + kErrOff);
  c.src = static_cast<const uint8_t*>(src);
  c.dst = static_cast<uint8_t*>(dst);
  c.nbytes = nbytes;
  c.slot_bytes = slot_bytes;
  c.step_bytes = step;
  c.nch = uint32_t(nchannels);
  c.nslots = uint32_t(nslots);
  c.lanes = uint32_t(lanes);
  c.roles = 3;
  if (proto == XFER_PROTO_LL)
    ll_layout(step, uint32_t(lanes), uint32_t(block), uint32_t(nslots), &c.ll_stripe_log2,
              &c.ll_group);
  args.nconn = 1;
  args.iters = 1;
  args.total_wgs = grid;
  args.xcd_remap = pairing ? 1u : 0u;
  args.rx_wgs = rx_region;
  args.timeout_ticks = uint64_t(a.timeout_ms ? a.timeout_ms : 10000u) * d->khz;
  e = launch_run1(v, args, block, s);
  if (e != hipSuccess) return hip_fail(e, "xfer_run_noalloc: transfer launch");
  if (status) {
    e = launch(report_kernel, 1, 64, s, const_cast<const Status*>(
                   reinterpret_cast<Status*>(base + kStatusOff)), status);
    if (e != hipSuccess) return hip_fail(e, "xfer_run_noalloc: status launch");
  }
  return XFER_OK;
}
