/*
 * oracle.h -- plain, slow CPU oracle of the FIFO send/recv data plane.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source
 * with the GPU library and includes none of its headers.
 *
 * What it models (sources: the pages on the NCCL transport layer):
 *  - the peer loop and channel masks of the transport setup driver
 *    ("transport建立", section 具体说明);
 *  - the producer/consumer data transfer through a ring of FIFO slots with
 *    head/tail step counters: the copy mode and the zero-copy mode with the
 *    ptrExchange word ("【NCCL】transport数据传输（二）", p2pTransport:
 *    "zero copy方式传递数据" (both kinds: the destination exchanged through
 *    ptrExchange during the kernel, or known before it) and "copy方式传递数据";
 *    the same hand-off over
 *    host memory in its shmTransport "正常方式" section);
 *  - the LL idea of a completion flag carried inside the data
 *    ("RDMA and GPUDirect" series article, section 四.1, signalling option 2);
 *  - the host-silent post/poll steady state ("Intra-Node Transport (P2P)",
 *    section 4, "POST / POLL");
 *  - the copy-engine relay of the shm transport's "useMemcpy" mode on the
 *    transfer page: host proxy threads move each step from the send FIFO to a
 *    host staging FIFO and on to the receive FIFO with memory copies.
 *
 * Readings of what the pages leave open are listed in the implementation
 * file next to the code that takes them.
 */
#ifndef RFP_ORACLE_H
#define RFP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* protocols */
#define ORC_SIMPLE 0
#define ORC_LL 1
#define ORC_ZC 2
#define ORC_ZCD 3 /* zero-copy with the destination known before the launch (no ptrExchange) */
#define ORC_RELAY 4 /* SIMPLE relayed by host proxies: send FIFO -> staging FIFO -> receive FIFO */

/* error returns (negative) */
#define ORC_E_ARG (-1)
#define ORC_E_RANGE (-2) /* an LL flag would pass 2^32-1 */
#define ORC_E_NOMEM (-3)
#define ORC_E_CAP (-4)   /* output array too small */

/* protocol violations (positive), found by the simulator or the enumerator */
#define ORC_V_OVERWRITE 1     /* producer wrote a slot whose previous step was not drained */
#define ORC_V_READ_UNFILLED 2 /* consumer read a slot/line that does not hold its step's payload,
                                 or a zero-copy receiver completed a step whose bytes had not
                                 landed in the destination */
#define ORC_V_READ_EARLY 3    /* consumer read a slot before observing tail > step */
#define ORC_V_WINDOW 4        /* more than nslots steps in flight */
#define ORC_V_WRONG_PTR 5     /* zero-copy producer took an address not published for its step */
#define ORC_V_DEADLOCK 6      /* no actor can move and the run is not finished */
#define ORC_V_RESULT 7        /* final destination differs from the source, or a guard byte changed */
#define ORC_V_COUNTERS 8      /* final head/tail/ptrExchange differ from the closed form */
#define ORC_V_CONFLUENCE 9    /* two interleavings ended in different final states */
#define ORC_V_STATE_LIMIT 10  /* the enumerator hit its state budget */

/* deliberate protocol mistakes, for the tests that prove the enumerator catches them */
#define ORC_MUT_NONE 0
#define ORC_MUT_WEAK_CREDIT 1 /* credit test admits nslots+1 steps in flight */
#define ORC_MUT_EARLY_TAIL 2  /* SIMPLE, ZCD: tail published before the chunk is written */
#define ORC_MUT_NO_ACQUIRE 3  /* SIMPLE: consumer loads the slot before it checks tail */
#define ORC_MUT_TORN_LINE 4   /* LL: flag and data halves of a line stored separately, flag first */
#define ORC_MUT_ZC_NO_WAIT 5  /* ZC: receiver publishes without waiting for ptrExchange == 0 */
#define ORC_MUT_ZC_NO_RESET 6 /* ZC: producer does not clear ptrExchange after reading it */
#define ORC_MUT_EARLY_HEAD 7  /* SIMPLE/LL: consumer frees the slot (head) before reading it */
#define ORC_MUT_ZC_AHEAD_PAST_END 8 /* ZC take-ahead order: also waits for an address after the
                                       transfer's last step */
#define ORC_MUT_RELAY_EARLY 9 /* RELAY: the send proxy copies a slot without waiting for tail */
#define ORC_MUT_GROUP_NO_BARRIER 10 /* LL group order: head for a group is published once the
                                       group's first step is read, not all of its steps */

/* producer program orders: the pages' order, and the orders the GPU kernels
 * use where they differ from it (each must stay safe and confluent) */
#define ORC_ORDER_PAGES 0
#define ORC_ORDER_ZC_TAKE_AHEAD 1 /* ZC: the producer takes step g+1's address, when g+1 is a step
                                     of the same transfer, after writing step g and before it
                                     publishes tail = g+1 */
/* LL, the striped kernels' order with groups of m steps (1 <= m <= ORC_GROUP_MAX):
 * steps are taken in aligned groups of m; on the producer side, step j is
 * written by sub-producer j mod m, which takes its steps in order and each
 * only on credit, independently of the other sub-producers; on the consumer
 * side, sub-consumer j mod m reads step j's lines, the sub-consumers of a
 * group meet at a barrier once all of the group's steps are read, and then
 * one head store, head = the group's last step + 1, frees the whole group
 * (issued by sub-consumer 0 before it reads its next step; the others go on
 * to the next group's steps at once).  m may exceed nslots in the model (the
 * kernels never build that): the enumerator then finds the deadlock that
 * rules it out. */
#define ORC_GROUP_MAX 4
#define ORC_ORDER_LL_GROUP(m) (0x100 + (m))

/* setup-plan op kinds */
#define ORC_OP_RECV_SETUP 0
#define ORC_OP_SEND_SETUP 1
#define ORC_OP_CONNECT_BATCH 2

/* ---- host schedule ---- */
int orc_peers(int rank, int nranks, int i, int* recv_peer, int* send_peer);
int orc_ring_masks(int rank, int nranks, int nchannels, uint64_t* recv_mask, uint64_t* send_mask);
/* ops: 3 ints per op (kind, peer, channel); channel and peer are -1 for CONNECT_BATCH */
int orc_plan(int rank, int nranks, const uint64_t* recv_mask, const uint64_t* send_mask,
             int max_peers, int* ops, int cap, int* nops);

/* ---- partition ---- */
uint64_t orc_step_bytes(int proto, uint64_t slot_bytes);
int orc_partition(uint64_t nbytes, int nchannels, uint64_t* beg, uint64_t* len);

/* ---- protocol simulation ---- */
typedef struct orc_conn orc_conn;
orc_conn* orc_conn_new(int proto, int nchannels, int nslots, uint64_t slot_bytes);
void orc_conn_free(orc_conn* c);
void orc_conn_set_mutation(orc_conn* c, int mutation);
void orc_conn_set_order(orc_conn* c, int order);
/* one transfer A[0:n] -> B[0:n] through the FIFO; 0, a violation code, or an error */
int orc_run(orc_conn* c, const uint8_t* A, uint8_t* B, uint64_t n);
/* iters round trips: a -> b on fwd, then b -> c on rev, each as one transfer */
int orc_run_pingpong(orc_conn* fwd, orc_conn* rev, const uint8_t* a, uint8_t* b, uint8_t* c,
                     uint64_t n, int iters);
/* Threaded mode: the same transfer with the producer and consumer of every
 * channel (and, for RELAY, its two proxies) as actors on nthreads real
 * threads (1 .. the number of actors; more are clamped), handing off through
 * C11 atomics.  Its end state must equal orc_run's. */
int orc_run_threaded(orc_conn* c, const uint8_t* A, uint8_t* B, uint64_t n, int nthreads);
/* Threaded ping-pong (SIMPLE or LL): endpoint X and endpoint Y on two
 * threads, pinned to two distinct cores when the process may use two;
 * *seconds = wall time of the iters round trips. */
int orc_pingpong_threaded(orc_conn* fwd, orc_conn* rev, const uint8_t* a, uint8_t* b,
                          uint8_t* c, uint64_t n, int iters, double* seconds);
/* out = {head, tail, ptrExchange, steps (the persistent step base)} */
int orc_conn_state(const orc_conn* c, int channel, uint64_t* out4);
const uint8_t* orc_conn_fifo(const orc_conn* c, int channel, uint64_t* bytes);
/* RELAY: FIFO `which` of a channel (0 send, 1 staging, 2 receive); for other
 * modes which = 0 is the one FIFO */
const uint8_t* orc_conn_fifo_ex(const orc_conn* c, int which, int channel, uint64_t* bytes);
/* RELAY: out = {send proxy's tail, receive proxy's tail} of a channel */
int orc_conn_relay_state(const orc_conn* c, int channel, uint64_t* out2);

/* ---- exhaustive interleaving check ---- */
typedef struct {
  uint64_t states;      /* distinct states reached */
  uint64_t terminals;   /* distinct final states (1 when confluent) */
  uint64_t transitions; /* actions fired */
  int violation;        /* first violation found, 0 if none */
  int channel;          /* channel of that violation, -1 if global */
  char msg[256];
} orc_enum_result;

/* Enumerates every interleaving of the producer and consumer actions of one
 * transfer of A[0:n] on a fresh connection, after prior_runs deterministic
 * transfers of the same bytes (so a nonzero step base is covered), with the
 * producer in program order `order`. */
int orc_enumerate(int proto, int nchannels, int nslots, uint64_t slot_bytes, const uint8_t* A,
                  uint64_t n, int mutation, int order, int prior_runs, uint64_t max_states,
                  orc_enum_result* out);

#ifdef __cplusplus
}
#endif
#endif
