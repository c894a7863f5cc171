// Host-side peer/channel schedule of the setup driver ("transport建立",
// NCCL v2.25.1-1, section 具体说明 and the receive/send setup listings after
// it): loop i pairs a rank with recv peer (rank - i) mod n and send peer
// (rank + i) mod n; per set channel bit, receive-side setup comes before
// send-side setup; ring connections carry channels only in the first loop;
// connects run in batches of max_peers loops (default 128) and after the last.
#include <stdint.h>

#include <string>

#include "xfer.h"

namespace xfer {
void set_error(int code, const std::string& msg);  // conn.cpp
}

extern "C" int xfer_sched_peers(int rank, int nranks, int i, int* recv_peer, int* send_peer) {
  if (nranks < 1 || rank < 0 || rank >= nranks || i < 0 || !recv_peer || !send_peer) {
    xfer::set_error(XFER_ERR_INVALID_ARG, "xfer_sched_peers: need 0 <= rank < nranks, i >= 0");
    return XFER_ERR_INVALID_ARG;
  }
  const int r = (rank - i % nranks + nranks) % nranks;
  *recv_peer = r;
  *send_peer = (rank + i) % nranks;
  return XFER_OK;
}

extern "C" int xfer_sched_ring_masks(int rank, int nranks, int nchannels, uint64_t* recv_mask,
                                     uint64_t* send_mask) {
  if (nranks < 1 || rank < 0 || rank >= nranks || nchannels < 1 || nchannels > 64 || !recv_mask ||
      !send_mask) {
    xfer::set_error(XFER_ERR_INVALID_ARG,
                    "xfer_sched_ring_masks: need 0 <= rank < nranks and 1 <= nchannels <= 64");
    return XFER_ERR_INVALID_ARG;
  }
  for (int p = 0; p < nranks; ++p) recv_mask[p] = send_mask[p] = 0;
  if (nranks < 2) return XFER_OK;  // a lone rank has no ring neighbour
  const uint64_t all = nchannels == 64 ? ~uint64_t(0) : (uint64_t(1) << nchannels) - 1;
  int rp = 0, sp = 0;
  xfer_sched_peers(rank, nranks, 1, &rp, &sp);
  recv_mask[rp] = all;
  send_mask[sp] = all;
  return XFER_OK;
}

extern "C" int xfer_sched_plan(int rank, int nranks, const uint64_t* recv_mask,
                               const uint64_t* send_mask, int max_peers, xfer_setup_op* ops,
                               int cap, int* nops) {
  if (nranks < 1 || rank < 0 || rank >= nranks || max_peers < 1 || !recv_mask || !send_mask ||
      !nops || cap < 0 || (cap > 0 && !ops)) {
    xfer::set_error(XFER_ERR_INVALID_ARG,
                    "xfer_sched_plan: bad rank/nranks/max_peers or NULL arrays");
    return XFER_ERR_INVALID_ARG;
  }
  int count = 0;
  auto push = [&](int kind, int peer, int ch) {
    if (count < cap) ops[count] = xfer_setup_op{kind, peer, ch};
    ++count;
  };
  int in_batch = 0;
  for (int i = 1; i < nranks; ++i) {
    int rp = 0, sp = 0;
    xfer_sched_peers(rank, nranks, i, &rp, &sp);
    for (int ch = 0; ch < 64; ++ch)
      if (recv_mask[rp] & (uint64_t(1) << ch)) push(XFER_OP_RECV_SETUP, rp, ch);
    for (int ch = 0; ch < 64; ++ch)
      if (send_mask[sp] & (uint64_t(1) << ch)) push(XFER_OP_SEND_SETUP, sp, ch);
    // every loop counts toward the batch, whether or not it set anything up
    if (++in_batch == max_peers || i + 1 == nranks) {
      push(XFER_OP_CONNECT_BATCH, -1, -1);
      in_batch = 0;
    }
  }
  *nops = count;
  if (count > cap) {
    xfer::set_error(XFER_ERR_INVALID_ARG, "xfer_sched_plan: ops array too small (nops = " +
                                              std::to_string(count) + ")");
    return XFER_ERR_INVALID_ARG;
  }
  return XFER_OK;
}
