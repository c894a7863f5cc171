// Host proxies of a relay connection: the copy-engine relay of the shm
// transport's memcpy mode ("【NCCL】transport数据传输（二）", shmTransport,
// useMemcpy).  A send proxy copies each step the producer has published
// (tail) from the send FIFO in HBM into a staging FIFO in pinned host memory
// and publishes ytail; a receive proxy copies it on into the receive FIFO in
// HBM and publishes gtail, which the consumer polls.  Both copies run on the
// GPU's DMA engines through the HSA runtime (device-to-host,
// host-to-device).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "xfer_internal.h"

namespace xfer {

struct RelayConfig {
  int device = 0;
  int nch = 0, lanes = 0, nslots = 0;
  uint64_t slot_bytes = 0, step_bytes = 0;
  uint8_t* send_fifo = nullptr;  // HBM: the producer's FIFO
  uint8_t* stage = nullptr;      // pinned host staging FIFO
  uint8_t* recv_fifo = nullptr;  // HBM: the consumer's FIFO
  LaneCtrl* ctrl = nullptr;      // host view of the control blocks, [nch * lanes]
  Status* status = nullptr;      // host view of the connection's status words
  uint32_t* err_mirror = nullptr;  // host view of the failure mirror the kernels read on entry
};

// The work one run hands the proxies: its messages (byte counts, in launch
// order, partitioned exactly as the kernels partition them) repeated iters
// times, numbered from each channel's step count before the run.
struct RelayJob {
  std::vector<uint64_t> lens;
  uint64_t iters = 1;
  std::vector<uint64_t> base;  // per channel
};

class Relay;

// Starts both proxy threads; on failure returns an xfer status and *err.
int relay_start(const RelayConfig& cfg, Relay** out, std::string* err);
// Stops and joins the proxies and frees their streams and events; jobs not
// yet relayed are dropped.  Only call once no launch on the connection is
// still running.
void relay_stop(Relay* r);
// Queues a run's job for both proxies (runs are relayed in order).
void relay_submit(Relay* r, const RelayJob& job);
// The first proxy failure, empty if none.
std::string relay_error(Relay* r);

}  // namespace xfer
