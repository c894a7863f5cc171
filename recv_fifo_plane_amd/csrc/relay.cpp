// Host proxies of a relay connection (see relay.h).
//
// The copies run on the GPU's DMA engines through the HSA runtime's
// asynchronous copy (device-to-host for the send proxy, host-to-device for
// the receive proxy); each signals its completion through an HSA signal that
// the proxy polls without a lock.  No HIP stream is involved, so a relay's
// copies never wait behind the connection's own kernel in a shared hardware
// queue, and they take no compute unit.
//
// For every channel a proxy walks the job's steps in order, with a ring of
// nslots signals:
//  - issue: once the step's input tail has passed g (send proxy: every
//    lane's tail, written by the producer; receive proxy: the send proxy's
//    tail), queue the copy of its chunk from slot g mod nslots of the source
//    FIFO into the same slot of the destination FIFO.  Consecutive ready
//    steps whose chunks are full and whose slots do not wrap go out as one
//    copy (and one signal);
//  - retire: once the oldest queued copy has completed, store the proxy's
//    output tail (its last step + 1) into host memory.
// Channels are swept round-robin, so a slow channel never holds the others
// back.  No slot of the three FIFOs is reused early: the producer's credit is
// the consumer's head, and the consumer drains step g only after the receive
// proxy's copy of it completed, which in turn followed the send proxy's.  The
// producer's stores were released at system scope before its tail, and the
// consumer's loads are system-coherent, as these copies require.  The proxy
// tails are per channel and sit in lane 0's control block.
#include "relay.h"

#include <hip/hip_runtime.h>
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <new>
#include <thread>

#include "xfer.h"

namespace xfer {

namespace {

// Chunk lengths of one channel's steps in a job, in step order: channel
// ranges of ceil(n / nch) rounded up to 16 bytes, steps of step_bytes.
void channel_steps(const RelayConfig& cfg, const RelayJob& job, int ch,
                   std::vector<uint64_t>& lens) {
  lens.clear();
  const uint64_t S = cfg.step_bytes;
  for (uint64_t it = 0; it < job.iters; ++it) {
    for (uint64_t n : job.lens) {
      uint64_t per = (n + uint64_t(cfg.nch) - 1) / uint64_t(cfg.nch);
      per = (per + 15) & ~uint64_t(15);
      const uint64_t b = std::min<uint64_t>(n, per * uint64_t(ch));
      const uint64_t len = std::min<uint64_t>(n, b + per) - b;
      for (uint64_t off = 0; off < len; off += S) lens.push_back(std::min<uint64_t>(S, len - off));
    }
  }
}

// The HSA agents of the copies: the connection's GPU and a CPU.
struct Agents {
  hsa_agent_t gpu{0}, cpu{0};
  uint32_t bdf = 0, domain = 0;
  bool have_gpu = false, have_cpu = false;
};

hsa_status_t find_agents(hsa_agent_t a, void* p) {
  Agents* ag = static_cast<Agents*>(p);
  hsa_device_type_t type;
  if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &type) != HSA_STATUS_SUCCESS)
    return HSA_STATUS_SUCCESS;
  if (type == HSA_DEVICE_TYPE_CPU && !ag->have_cpu) {
    ag->cpu = a;
    ag->have_cpu = true;
  } else if (type == HSA_DEVICE_TYPE_GPU && !ag->have_gpu) {
    uint32_t bdf = 0, domain = 0;
    if (hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf) ==
            HSA_STATUS_SUCCESS &&
        hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_DOMAIN),
                           &domain) == HSA_STATUS_SUCCESS &&
        bdf == ag->bdf && domain == ag->domain) {
      ag->gpu = a;
      ag->have_gpu = true;
    }
  }
  return HSA_STATUS_SUCCESS;
}

class Proxy {
 public:
  Proxy(const RelayConfig& cfg, bool send) : cfg_(cfg), send_(send) {}

  int init(const Agents& ag, std::string* err) {
    ag_ = ag;
    signals_.assign(size_t(cfg_.nch) * size_t(cfg_.nslots), hsa_signal_t{0});
    for (hsa_signal_t& sg : signals_) {
      if (hsa_signal_create(0, 0, nullptr, &sg) != HSA_STATUS_SUCCESS) {
        sg.handle = 0;
        *err = "relay proxy: hsa_signal_create failed";
        return XFER_ERR_NO_MEMORY;
      }
    }
    thread_ = std::thread(&Proxy::loop, this);
    return XFER_OK;
  }

  void stop() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stopping_.store(true, std::memory_order_release);
    }
    cv_.notify_all();
    if (thread_.joinable()) thread_.join();
    // A copy the proxy abandoned may still be in flight: let it land before
    // its signal and buffers go (bounded: a copy that never completes has
    // failed, and its buffers are freed regardless).
    for (hsa_signal_t sg : signals_) {
      if (!sg.handle) continue;
      (void)hsa_signal_wait_scacquire(sg, HSA_SIGNAL_CONDITION_LT, 1, 2000000000ull,
                                      HSA_WAIT_STATE_BLOCKED);
      (void)hsa_signal_destroy(sg);
    }
    signals_.clear();
  }

  void submit(const RelayJob& job) {
    {
      std::lock_guard<std::mutex> lk(mu_);
      queue_.push_back(job);
    }
    cv_.notify_one();
  }

  std::string error() {
    std::lock_guard<std::mutex> lk(mu_);
    return error_;
  }

 private:
  LaneCtrl& lane(int ch, int w) const {
    return cfg_.ctrl[size_t(ch) * size_t(cfg_.lanes) + size_t(w)];
  }

  // Whether step g of a channel has reached this proxy.
  bool ready(int ch, uint64_t g) const {
    if (!send_) return __atomic_load_n(&lane(ch, 0).ytail, __ATOMIC_ACQUIRE) > g;
    for (int w = 0; w < cfg_.lanes; ++w)
      if (__atomic_load_n(&lane(ch, w).tail, __ATOMIC_ACQUIRE) <= g) return false;
    return true;
  }

  // The kernels failed, the host asked for an abort, or the connection is
  // being destroyed: stop relaying.
  bool abandoned() const {
    return stopping_.load(std::memory_order_acquire) ||
           __atomic_load_n(&cfg_.status->err, __ATOMIC_ACQUIRE) != 0 ||
           __atomic_load_n(&cfg_.status->abort_flag, __ATOMIC_ACQUIRE) != 0;
  }

  // A proxy failure ends the connection like an in-kernel one: the sticky
  // error word is set and the abort word ends every kernel wait.
  void raise(const std::string& what) {
    {
      std::lock_guard<std::mutex> lk(mu_);
      if (error_.empty()) error_ = std::string(send_ ? "send" : "receive") + " proxy: " + what;
    }
    uint32_t zero = 0;
    __atomic_compare_exchange_n(&cfg_.status->err, &zero, uint32_t(XFER_ERR_HIP), false,
                                __ATOMIC_ACQ_REL, __ATOMIC_ACQUIRE);
    zero = 0;
    __atomic_compare_exchange_n(cfg_.err_mirror, &zero, uint32_t(XFER_ERR_HIP), false,
                                __ATOMIC_ACQ_REL, __ATOMIC_ACQUIRE);
    __atomic_store_n(&cfg_.status->abort_flag, 1u, __ATOMIC_RELEASE);
  }

  // Relays one job; false if it was abandoned or failed.
  bool run(const RelayJob& job) {
    struct Copy {
      uint64_t end;  // the proxy's tail once this copy has landed
      size_t sig;    // its signal
    };
    struct Chan {
      std::vector<uint64_t> lens;
      size_t issued = 0;
      std::deque<Copy> inflight;
    };
    std::vector<Chan> ch(size_t(cfg_.nch));
    size_t pending = 0;  // channels with steps left to issue or retire
    for (int c = 0; c < cfg_.nch; ++c) {
      channel_steps(cfg_, job, c, ch[size_t(c)].lens);
      if (!ch[size_t(c)].lens.empty()) ++pending;
    }
    uint8_t* from = send_ ? cfg_.send_fifo : cfg_.stage;
    uint8_t* to = send_ ? cfg_.stage : cfg_.recv_fifo;
    const hsa_agent_t from_agent = send_ ? ag_.gpu : ag_.cpu;
    const hsa_agent_t to_agent = send_ ? ag_.cpu : ag_.gpu;
    const uint64_t ns = uint64_t(cfg_.nslots), S = cfg_.slot_bytes;
    uint32_t idle = 0;
    while (pending) {
      bool moved = false;
      for (int c = 0; c < cfg_.nch; ++c) {
        Chan& s = ch[size_t(c)];
        const uint64_t base = job.base[size_t(c)];
        // retire, in order
        while (!s.inflight.empty()) {
          const Copy& cp = s.inflight.front();
          const hsa_signal_value_t v =
              hsa_signal_load_scacquire(signals_[size_t(c) * ns + cp.sig]);
          if (v > 0) break;
          if (v < 0) {
            raise("an asynchronous copy failed");
            return false;
          }
          __atomic_store_n(send_ ? &lane(c, 0).ytail : &lane(c, 0).gtail, cp.end, __ATOMIC_RELEASE);
          s.inflight.pop_front();
          moved = true;
          if (s.issued == s.lens.size() && s.inflight.empty()) --pending;
        }
        // issue: a slot's signal is free once the copy that used it retired,
        // which the end-to-end credit guarantees before its step is ready
        if (s.issued == s.lens.size() || s.inflight.size() == size_t(ns) ||
            !ready(c, base + s.issued))
          continue;
        const size_t first = s.issued;
        const uint64_t g0 = base + first;
        size_t last = first + 1;
        uint64_t bytes = s.lens[first];
        while (last < s.lens.size() && s.lens[last - 1] == S && (g0 + (last - first)) % ns != 0 &&
               ready(c, base + last)) {
          bytes += s.lens[last];
          ++last;
        }
        const size_t slot = size_t(g0 % ns);
        const hsa_signal_t sg = signals_[size_t(c) * ns + slot];
        if (hsa_signal_load_scacquire(sg) != 0) {
          raise("a copy signal was still busy");
          return false;
        }
        hsa_signal_store_relaxed(sg, 1);
        const size_t off = size_t((uint64_t(c) * ns + slot) * S);
        if (hsa_amd_memory_async_copy(to + off, to_agent, from + off, from_agent, size_t(bytes), 0,
                                      nullptr, sg) != HSA_STATUS_SUCCESS) {
          hsa_signal_store_relaxed(sg, 0);
          raise("hsa_amd_memory_async_copy refused a copy");
          return false;
        }
        s.inflight.push_back(Copy{base + last, slot});
        s.issued = last;
        moved = true;
      }
      if (moved) {
        idle = 0;
        continue;
      }
      if (abandoned()) return false;
      if (++idle > 64) std::this_thread::yield();
    }
    return true;
  }

  void loop() {
    for (;;) {
      RelayJob job;
      {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return stopping_.load(std::memory_order_acquire) || !queue_.empty(); });
        if (stopping_.load(std::memory_order_acquire)) return;
        job = std::move(queue_.front());
        queue_.pop_front();
      }
      if (!run(job)) {
        // The connection has failed (or is going away): later runs on it
        // are refused, so the queued jobs will never be relayed.
        std::lock_guard<std::mutex> lk(mu_);
        queue_.clear();
      }
    }
  }

  RelayConfig cfg_;
  bool send_;
  Agents ag_;
  std::vector<hsa_signal_t> signals_;  // [nch * nslots], one per slot
  std::thread thread_;
  std::mutex mu_;
  std::condition_variable cv_;
  std::deque<RelayJob> queue_;
  std::atomic<bool> stopping_{false};
  std::string error_;
};

}  // namespace

class Relay {
 public:
  explicit Relay(const RelayConfig& cfg) : send(cfg, true), recv(cfg, false) {}
  Proxy send, recv;
  bool hsa_up = false;
};

int relay_start(const RelayConfig& cfg, Relay** out, std::string* err) {
  *out = nullptr;
  // The GPU's HSA agent is the one at the device's PCI domain and
  // bus/device (function 0).
  int bus = 0, dev = 0, domain = 0;
  if (hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, cfg.device) != hipSuccess ||
      hipDeviceGetAttribute(&dev, hipDeviceAttributePciDeviceId, cfg.device) != hipSuccess ||
      hipDeviceGetAttribute(&domain, hipDeviceAttributePciDomainId, cfg.device) != hipSuccess) {
    *err = "relay: cannot read the device's PCI location";
    return XFER_ERR_HIP;
  }
  Relay* r = new (std::nothrow) Relay(cfg);
  if (!r) {
    *err = "relay: out of host memory";
    return XFER_ERR_NO_MEMORY;
  }
  if (hsa_init() != HSA_STATUS_SUCCESS) {  // reference-counted; the HIP runtime holds one too
    delete r;
    *err = "relay: hsa_init failed";
    return XFER_ERR_HIP;
  }
  r->hsa_up = true;
  Agents ag;
  ag.bdf = (uint32_t(bus) << 8) | (uint32_t(dev) << 3);
  ag.domain = uint32_t(domain);
  int rc = XFER_OK;
  if (hsa_iterate_agents(find_agents, &ag) != HSA_STATUS_SUCCESS || !ag.have_gpu || !ag.have_cpu) {
    *err = "relay: no HSA agent for the device and the host";
    rc = XFER_ERR_HIP;
  }
  if (!rc) rc = r->send.init(ag, err);
  if (!rc) rc = r->recv.init(ag, err);
  if (rc) {
    relay_stop(r);
    return rc;
  }
  *out = r;
  return XFER_OK;
}

void relay_stop(Relay* r) {
  if (!r) return;
  r->send.stop();
  r->recv.stop();
  if (r->hsa_up) (void)hsa_shut_down();
  delete r;
}

void relay_submit(Relay* r, const RelayJob& job) {
  r->send.submit(job);
  r->recv.submit(job);
}

std::string relay_error(Relay* r) {
  if (!r) return std::string();
  std::string e = r->send.error();
  return e.empty() ? r->recv.error() : e;
}

}  // namespace xfer
