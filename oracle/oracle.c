/*
 * oracle.c -- plain, slow CPU oracle of the FIFO send/recv data plane.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg are its only users.  It shares no code with the GPU
 * library.  Everything here is sequential C; a "transfer" is simulated as a
 * sequence of atomic actions by a producer and a consumer per channel, the
 * same actions the exhaustive enumerator at the bottom of this file
 * interleaves in every possible order.
 *
 * Readings taken where the pages are silent or disagree (each is marked
 * "Reading" at the code that takes it):
 *  R1  Step g of a connection is 0-based; finishing it publishes tail = g+1.
 *      head and tail start at 0 when the connection is created (the net
 *      transport's proxy-connect code on "transport建立" clears head to 0,
 *      and the credit index the receiver writes first is 1 while head is 0,
 *      "【NCCL】transport数据传输（二）", netTransport, phase 2).
 *  R2  A producer may fill step g iff g - head < nslots; step g uses slot
 *      g mod nslots.  The pages reuse the slots circularly ("RDMA and
 *      GPUDirect" series article, section 四.3) and bump head when a buffer is
 *      free again (transfer page, netTransport phase 4); the test itself is
 *      not printed.
 *  R3  A consumer may drain step g iff tail > g.
 *  R4  LL: each 8-byte line holds 4 payload bytes (bytes 0..3) and a 4-byte
 *      flag (bytes 4..7), little-endian; the flag of step g is g+1, so the
 *      zero-filled FIFO of a new connection never looks valid.  The last
 *      word of a chunk is zero-padded.  The consumer polls the flags; no tail
 *      is polled.  The transfer page says LL bumps tail, the RDMA article
 *      says LL carries its flag in the data: the flag reading wins, and the
 *      producer writes its final step count to tail once, as bookkeeping, so
 *      head == tail holds at the end.  Flags are 32-bit: a connection may not
 *      pass 2^32-1 LL steps.
 *  R5  An LL slot of slot_bytes carries slot_bytes/2 payload bytes; SIMPLE
 *      and zero-copy steps carry slot_bytes.
 *  R6  Partition: per = ceil(n / C) rounded up to a multiple of 16; channel
 *      c moves [c*per, min(n, (c+1)*per)), possibly empty.  Chunk j of a
 *      channel holds min(S, len - j*S) bytes; both sides derive chunk sizes
 *      from n, so no size FIFO is modelled.  Slot bytes past a short chunk
 *      keep what they held.
 *  R7  Zero-copy: per step, the receiver publishes the destination of step g
 *      into ptrExchange only when the word is 0; the producer reads it,
 *      clears it, writes the chunk there, then publishes tail = g+1; the
 *      receiver, seeing tail > g, publishes head = g+1.  No slots are reused,
 *      so the producer never waits on head.  (Order of the five actions:
 *      transfer page, p2pTransport, "zero copy方式传递数据", first kind.)
 *      The oracle's address token is (offset of the chunk in B) + 1.
 *      Zero-copy direct (ORC_ZCD, the page's second kind): the destination is
 *      known before the launch, so ptrExchange is not used; per step the
 *      producer writes the chunk into B and publishes tail = g+1, and the
 *      receiver, seeing tail > g, publishes head = g+1.
 *  R8  The step base persists across transfers on one connection; a step
 *      never spans two transfers.
 *  R9  Copy-engine relay (ORC_RELAY; the shm transport's "useMemcpy" mode on
 *      the transfer page): the producer fills the send FIFO and publishes
 *      tail; a send proxy, seeing tail > g, copies slot g into a host staging
 *      FIFO and publishes its own tail; a receive proxy, seeing that, copies
 *      the staging slot into the receive FIFO and publishes a third tail; the
 *      consumer drains the receive FIFO once that tail passes g and publishes
 *      head, which is the producer's credit end to end.  All three FIFOs
 *      have nslots slots of slot_bytes; a proxy copies exactly the chunk.
 */
#include "oracle.h"
#include "oracle_internal.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define GUARD 64 /* guard bytes on each side of the enumerator's destination */

/* ------------------------------------------------------------------ schedule
 * The setup driver's peer loop ("transport建立", 具体说明): in loop i a rank
 * receives from (rank - i) mod n and sends to (rank + i) mod n; the page's
 * example has rank 0 of 8 receive from 7 and send to 1 in the first loop. */
int orc_peers(int rank, int nranks, int i, int* recv_peer, int* send_peer) {
  if (nranks < 1 || rank < 0 || rank >= nranks || i < 0 || !recv_peer || !send_peer)
    return ORC_E_ARG;
  *recv_peer = ((rank - i) % nranks + nranks) % nranks;
  *send_peer = (rank + i) % nranks;
  return 0;
}

static uint64_t full_mask(int nch) { return nch >= 64 ? ~0ull : ((1ull << nch) - 1ull); }

/* Ring connections: only the first loop's peers carry channels (same
 * section).  Reading: the ring uses channels 0..C-1 on both its edges; a
 * single rank has no ring edge. */
int orc_ring_masks(int rank, int nranks, int nchannels, uint64_t* recv_mask, uint64_t* send_mask) {
  if (nranks < 1 || rank < 0 || rank >= nranks || nchannels < 1 || nchannels > 64 || !recv_mask ||
      !send_mask)
    return ORC_E_ARG;
  for (int p = 0; p < nranks; ++p) recv_mask[p] = send_mask[p] = 0;
  if (nranks == 1) return 0;
  int rp, sp;
  orc_peers(rank, nranks, 1, &rp, &sp);
  recv_mask[rp] = full_mask(nchannels);
  send_mask[sp] = full_mask(nchannels);
  return 0;
}

/* Setup plan: per loop, receive-side setups for each set channel bit of the
 * receive peer's mask (ascending), then send-side setups for the send peer's
 * mask; a connect phase runs once max_peers loops have gathered, and after
 * the last loop (same page, 具体说明 and the two setup listings after it).
 * Reading: every loop counts toward max_peers, even one with empty masks. */
int orc_plan(int rank, int nranks, const uint64_t* recv_mask, const uint64_t* send_mask,
             int max_peers, int* ops, int cap, int* nops) {
  if (nranks < 1 || rank < 0 || rank >= nranks || max_peers < 1 || !recv_mask || !send_mask ||
      !nops || cap < 0 || (cap > 0 && !ops))
    return ORC_E_ARG;
  int k = 0, gathered = 0;
#define EMIT(kind_, peer_, ch_)        \
  do {                                 \
    if (k < cap) {                     \
      ops[3 * k + 0] = (kind_);        \
      ops[3 * k + 1] = (peer_);        \
      ops[3 * k + 2] = (ch_);          \
    }                                  \
    ++k;                               \
  } while (0)
  for (int i = 1; i < nranks; ++i) {
    int rp, sp;
    orc_peers(rank, nranks, i, &rp, &sp);
    for (int c = 0; c < 64; ++c)
      if ((recv_mask[rp] >> c) & 1ull) EMIT(ORC_OP_RECV_SETUP, rp, c);
    for (int c = 0; c < 64; ++c)
      if ((send_mask[sp] >> c) & 1ull) EMIT(ORC_OP_SEND_SETUP, sp, c);
    ++gathered;
    if (gathered == max_peers || i == nranks - 1) {
      EMIT(ORC_OP_CONNECT_BATCH, -1, -1);
      gathered = 0;
    }
  }
#undef EMIT
  *nops = k;
  return k > cap ? ORC_E_CAP : 0;
}

/* ----------------------------------------------------------------- partition */
uint64_t orc_step_bytes(int proto, uint64_t slot_bytes) {
  return proto == ORC_LL ? slot_bytes / 2 : slot_bytes; /* Reading R5 */
}

int orc_partition(uint64_t n, int nch, uint64_t* beg, uint64_t* len) {
  if (nch < 1 || !beg || !len) return ORC_E_ARG;
  uint64_t per = (n + (uint64_t)nch - 1) / (uint64_t)nch; /* Reading R6 */
  per = (per + 15) / 16 * 16;
  for (int c = 0; c < nch; ++c) {
    uint64_t b = (uint64_t)c * per, e = (uint64_t)(c + 1) * per;
    if (b > n) b = n;
    if (e > n) e = n;
    beg[c] = b;
    len[c] = e - b;
  }
  return 0;
}

/* ------------------------------------------------------------ connection */

/* FIFOs per channel: none for the zero-copy modes, three for the relay. */
static int nfifos(int proto) {
  return proto == ORC_RELAY ? 3 : (proto == ORC_SIMPLE || proto == ORC_LL) ? 1 : 0;
}
static int has_fifo(int proto) { return nfifos(proto) > 0; }

orc_conn* orc_conn_new(int proto, int nch, int nslots, uint64_t slot_bytes) {
  if (proto < ORC_SIMPLE || proto > ORC_RELAY || nch < 1 || nch > 64 || nslots < 1) return NULL;
  if (proto == ORC_LL ? (slot_bytes < 8 || slot_bytes % 8) : (slot_bytes < 16 || slot_bytes % 16))
    return NULL;
  orc_conn* c = (orc_conn*)calloc(1, sizeof(*c));
  if (!c) return NULL;
  c->proto = proto;
  c->nch = nch;
  c->nslots = nslots;
  c->slot_bytes = slot_bytes;
  c->step_bytes = orc_step_bytes(proto, slot_bytes);
  c->ctrl = (orc_ctrl*)calloc((size_t)nch, sizeof(orc_ctrl)); /* Reading R1: all zero */
  if (has_fifo(proto))
    c->fifo = (uint8_t*)calloc((size_t)nfifos(proto) * nch * nslots, slot_bytes);
  if (!c->ctrl || (has_fifo(proto) && !c->fifo)) {
    orc_conn_free(c);
    return NULL;
  }
  return c;
}

void orc_conn_free(orc_conn* c) {
  if (!c) return;
  free(c->fifo);
  free(c->ctrl);
  free(c);
}

void orc_conn_set_order(orc_conn* c, int order) {
  if (c) c->order = order;
}

void orc_conn_set_mutation(orc_conn* c, int mutation) {
  if (c) c->mutation = mutation;
}

int orc_conn_state(const orc_conn* c, int ch, uint64_t* out4) {
  if (!c || ch < 0 || ch >= c->nch || !out4) return ORC_E_ARG;
  out4[0] = c->ctrl[ch].head;
  out4[1] = c->ctrl[ch].tail;
  out4[2] = c->ctrl[ch].ptrx;
  out4[3] = c->ctrl[ch].base;
  return 0;
}

const uint8_t* orc_conn_fifo_ex(const orc_conn* c, int which, int ch, uint64_t* bytes) {
  if (!c || ch < 0 || ch >= c->nch || !c->fifo || which < 0 || which >= nfifos(c->proto)) {
    if (bytes) *bytes = 0;
    return NULL;
  }
  const uint64_t per = (uint64_t)c->nslots * c->slot_bytes;
  if (bytes) *bytes = per;
  return c->fifo + ((uint64_t)which * c->nch + (uint64_t)ch) * per;
}

const uint8_t* orc_conn_fifo(const orc_conn* c, int ch, uint64_t* bytes) {
  return orc_conn_fifo_ex(c, 0, ch, bytes);
}

int orc_conn_relay_state(const orc_conn* c, int ch, uint64_t* out2) {
  if (!c || ch < 0 || ch >= c->nch || !out2 || c->proto != ORC_RELAY) return ORC_E_ARG;
  out2[0] = c->ctrl[ch].ytail;
  out2[1] = c->ctrl[ch].gtail;
  return 0;
}

/* ----------------------------------------------------------------- world
 * The mutable state of one transfer in progress: control words, per-channel
 * cursors of both sides, per-slot bookkeeping for the invariants, the FIFO
 * bytes and the destination.  The enumerator clones and fingerprints it. */
typedef struct {
  uint64_t beg, len, k; /* channel range and its number of steps */
  uint64_t pj, pline, pptr;
  uint64_t pnext; /* ZC take-ahead: address taken for step pj+1, 0 if none */
  uint32_t pphase, pfinal;
  uint64_t cj, cline, cnpub;
  uint32_t cphase, pad;
  uint64_t sj, rj; /* RELAY: next step of the send proxy and of the receive proxy */
  /* LL group order: for sub-producer and sub-consumer x < m, the next step
   * (x, x + m, ...) and the line within it; cbar is the first step of the
   * group the sub-consumers read (the one past their last barrier), and cj
   * the first step of the group whose head is still to be published */
  uint64_t gpj[ORC_GROUP_MAX], gpl[ORC_GROUP_MAX], gcj[ORC_GROUP_MAX], gcl[ORC_GROUP_MAX];
  uint64_t cbar;
} orc_cur;

typedef struct {
  const orc_conn* cfg;
  const uint8_t* A;
  uint64_t n;
  uint8_t* meta; /* orc_ctrl[nch] | orc_cur[nch] | fill[F][nch*nslots] | drain[F][nch*nslots] |
                    regs, F = max(1, FIFOs) */
  uint64_t meta_bytes;
  uint8_t* fifo;
  uint8_t* B;
} world;

static orc_ctrl* W_ctrl(const world* w) { return (orc_ctrl*)w->meta; }
static orc_cur* W_cur(const world* w) {
  return (orc_cur*)(w->meta + sizeof(orc_ctrl) * (size_t)w->cfg->nch);
}
static int ntrack(const orc_conn* c) { return nfifos(c->proto) > 1 ? nfifos(c->proto) : 1; }
/* step that last started filling each slot of FIFO f, -1 if none in this transfer */
static int64_t* W_fill_in(const world* w, int f) {
  return (int64_t*)(w->meta + (sizeof(orc_ctrl) + sizeof(orc_cur)) * (size_t)w->cfg->nch) +
         (size_t)f * w->cfg->nch * w->cfg->nslots;
}
/* step whose payload was last drained from each slot of FIFO f, -1 if none */
static int64_t* W_drain_in(const world* w, int f) {
  return W_fill_in(w, ntrack(w->cfg) + f);
}
static int64_t* W_fill(const world* w) { return W_fill_in(w, 0); }
/* consumer registers of the NO_ACQUIRE mutation (one slot per channel) */
static uint8_t* W_regs(const world* w) { return (uint8_t*)W_fill_in(w, 2 * ntrack(w->cfg)); }

static uint64_t meta_size(const orc_conn* c) {
  return (sizeof(orc_ctrl) + sizeof(orc_cur)) * (uint64_t)c->nch +
         2ull * (uint64_t)ntrack(c) * sizeof(int64_t) * (uint64_t)c->nch * c->nslots +
         (uint64_t)c->nch * c->slot_bytes;
}

static uint64_t fifo_size(const orc_conn* c) {
  return (uint64_t)nfifos(c->proto) * c->nch * c->nslots * c->slot_bytes;
}

/* Fills meta for a new transfer of n bytes; FIFO and B are set by the caller. */
static int world_begin(world* w, const orc_conn* c, const uint8_t* A, uint64_t n) {
  w->cfg = c;
  w->A = A;
  w->n = n;
  memset(w->meta, 0, (size_t)w->meta_bytes);
  orc_ctrl* q = W_ctrl(w);
  orc_cur* u = W_cur(w);
  uint64_t beg[64], len[64];
  orc_partition(n, c->nch, beg, len);
  for (int ch = 0; ch < c->nch; ++ch) {
    q[ch] = c->ctrl[ch];
    u[ch].beg = beg[ch];
    u[ch].len = len[ch];
    u[ch].k = (len[ch] + c->step_bytes - 1) / c->step_bytes;
    if (c->proto == ORC_LL && q[ch].base + u[ch].k > 0xFFFFFFFFull) return ORC_E_RANGE;
    for (int x = 0; x < ORC_GROUP_MAX; ++x) u[ch].gpj[x] = u[ch].gcj[x] = (uint64_t)x;
  }
  int64_t* fill = W_fill(w); /* every FIFO's fill and drain marks, contiguous */
  for (int i = 0; i < 2 * ntrack(c) * c->nch * c->nslots; ++i) fill[i] = -1;
  return 0;
}

static uint64_t chunk_len(const world* w, const orc_cur* u, uint64_t j) {
  uint64_t S = w->cfg->step_bytes, rest = u->len - j * S;
  return rest < S ? rest : S;
}

static uint8_t* slot_ptr_in(const world* w, int f, int ch, uint64_t g) {
  const orc_conn* c = w->cfg;
  return w->fifo + (((uint64_t)f * c->nch + (uint64_t)ch) * c->nslots + g % (uint64_t)c->nslots) *
                       c->slot_bytes;
}
static uint8_t* slot_ptr(const world* w, int ch, uint64_t g) { return slot_ptr_in(w, 0, ch, g); }

/* Reading R2: the credit test, g - head < nslots over the integers (a head
 * already past g, which only a broken consumer publishes, is credit too). */
static int credit_ok(const world* w, const orc_ctrl* q, uint64_t g) {
  uint64_t ns = (uint64_t)w->cfg->nslots;
  return w->cfg->mutation == ORC_MUT_WEAK_CREDIT ? g <= q->head + ns : g < q->head + ns;
}

static size_t slot_index(const world* w, int ch, uint64_t g) {
  return (size_t)ch * w->cfg->nslots + (size_t)(g % (uint64_t)w->cfg->nslots);
}
static int slot_free_in(const world* w, int f, int ch, uint64_t g) {
  int64_t fl = W_fill_in(w, f)[slot_index(w, ch, g)];
  return fl < 0 || W_drain_in(w, f)[slot_index(w, ch, g)] == fl;
}
static void mark_fill_in(const world* w, int f, int ch, uint64_t g) {
  W_fill_in(w, f)[slot_index(w, ch, g)] = (int64_t)g;
}
static void mark_drain_in(const world* w, int f, int ch, uint64_t g) {
  W_drain_in(w, f)[slot_index(w, ch, g)] = (int64_t)g;
}
static int64_t fill_of_in(const world* w, int f, int ch, uint64_t g) {
  return W_fill_in(w, f)[slot_index(w, ch, g)];
}
static int slot_free(const world* w, int ch, uint64_t g) { return slot_free_in(w, 0, ch, g); }
static void mark_fill(const world* w, int ch, uint64_t g) { mark_fill_in(w, 0, ch, g); }
static void mark_drain(const world* w, int ch, uint64_t g) { mark_drain_in(w, 0, ch, g); }
static int64_t fill_of(const world* w, int ch, uint64_t g) { return fill_of_in(w, 0, ch, g); }

/* LL line helpers, Reading R4. */
static uint64_t ll_lines(uint64_t L) { return (L + 3) / 4; }

static uint32_t ll_word(const uint8_t* src, uint64_t L, uint64_t line) {
  uint32_t wv = 0;
  for (uint64_t b = 0; b < 4 && 4 * line + b < L; ++b) wv |= (uint32_t)src[4 * line + b] << (8 * b);
  return wv;
}

static void put32(uint8_t* p, uint32_t v) {
  for (int b = 0; b < 4; ++b) p[b] = (uint8_t)(v >> (8 * b));
}
static uint32_t get32(const uint8_t* p) {
  return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
}

/* ------------------------------------------------------------------ actors */
enum { ACT_PROD = 0, ACT_CONS = 1, ACT_PUB = 2, ACT_SPROXY = 3, ACT_RPROXY = 4, N_ACT = 5 };
/* LL group order: sub-producers and sub-consumers x < m are actors of their
 * own; ACT_PROD then only writes the bookkeeping tail and ACT_PUB is the
 * group's head store. */
enum { ACT_GPROD = N_ACT, ACT_GCONS = N_ACT + ORC_GROUP_MAX, N_ACT_ALL = N_ACT + 2 * ORC_GROUP_MAX };

/* Group size m of the LL group order, 0 in every other order. */
static int ll_group(const orc_conn* c) {
  if (c->proto != ORC_LL || c->order <= ORC_ORDER_LL_GROUP(0) ||
      c->order > ORC_ORDER_LL_GROUP(ORC_GROUP_MAX))
    return 0;
  return c->order - ORC_ORDER_LL_GROUP(0);
}

/* One past the last step of the aligned group that starts at step s. */
static uint64_t group_end(const orc_cur* u, int m, uint64_t s) {
  return s + (uint64_t)m < u->k ? s + (uint64_t)m : u->k;
}

/* Whether the ZC producer, having written step pj, takes step pj+1's
 * address before it publishes tail (the kernels' pipelined order). */
static int zc_takes_ahead(const orc_conn* c, const orc_cur* u) {
  if (c->order != ORC_ORDER_ZC_TAKE_AHEAD) return 0;
  return u->pj + 1 < u->k || c->mutation == ORC_MUT_ZC_AHEAD_PAST_END;
}

static int prod_enabled(const world* w, int ch) {
  const orc_conn* c = w->cfg;
  const orc_ctrl* q = &W_ctrl(w)[ch];
  const orc_cur* u = &W_cur(w)[ch];
  uint64_t g = q->base + u->pj;
  switch (c->proto) {
    case ORC_SIMPLE:
    case ORC_RELAY:
      return u->pj < u->k && (u->pphase != 0 || credit_ok(w, q, g));
    case ORC_LL:
      if (ll_group(c)) { /* the bookkeeping tail, once every sub-producer is done */
        for (int x = 0; x < ll_group(c); ++x)
          if (u->gpj[x] < u->k) return 0;
        return !u->pfinal;
      }
      if (u->pj == u->k) return !u->pfinal;
      return u->pline > 0 || u->pphase != 0 || credit_ok(w, q, g);
    case ORC_ZCD: /* the destination is known: nothing to wait for */
      return u->pj < u->k;
    default: /* ORC_ZC: taking an address needs a published one */
      if (u->pj >= u->k) return 0;
      if (u->pphase == 0) return u->pnext != 0 || q->ptrx != 0;
      if (u->pphase == 2 && zc_takes_ahead(c, u)) return q->ptrx != 0;
      return 1;
  }
}

static int cons_enabled(const world* w, int ch) {
  const orc_conn* c = w->cfg;
  const orc_ctrl* q = &W_ctrl(w)[ch];
  const orc_cur* u = &W_cur(w)[ch];
  if (u->cj >= u->k) return 0;
  uint64_t g = q->base + u->cj;
  switch (c->proto) {
    case ORC_SIMPLE:
      if (c->mutation == ORC_MUT_NO_ACQUIRE) return u->cphase == 1 ? q->tail > g : 1;
      if (c->mutation == ORC_MUT_EARLY_HEAD) return u->cphase == 0 ? q->tail > g : 1;
      return u->cphase == 0 ? q->tail > g : 1;
    case ORC_LL: {
      if (ll_group(c)) return 0; /* the sub-consumers read instead */
      if (u->cphase == 1) return 1;
      const uint8_t* line = slot_ptr(w, ch, g) + 8 * u->cline;
      return get32(line + 4) == (uint32_t)(g + 1);
    }
    case ORC_RELAY: /* the receive proxy's tail */
      return u->cphase == 0 ? q->gtail > g : 1;
    default: /* ORC_ZC and ORC_ZCD receiver, completion cursor */
      return q->tail > g;
  }
}

static int pub_enabled(const world* w, int ch) {
  const orc_conn* c = w->cfg;
  const orc_ctrl* q = &W_ctrl(w)[ch];
  const orc_cur* u = &W_cur(w)[ch];
  if (ll_group(c)) { /* the group's head store: after the barrier, or (mutation) after step cj */
    if (u->cj >= u->k) return 0;
    return c->mutation == ORC_MUT_GROUP_NO_BARRIER ? u->gcj[0] > u->cj : u->cj < u->cbar;
  }
  if (c->proto != ORC_ZC) return 0;
  return u->cnpub < u->k && (c->mutation == ORC_MUT_ZC_NO_WAIT || q->ptrx == 0);
}

/* RELAY proxies: the send proxy moves step g once tail > g, the receive
 * proxy once the send proxy's tail > g. */
static int proxy_enabled(const world* w, int ch, int act) {
  const orc_conn* c = w->cfg;
  if (c->proto != ORC_RELAY) return 0;
  const orc_ctrl* q = &W_ctrl(w)[ch];
  const orc_cur* u = &W_cur(w)[ch];
  if (act == ACT_SPROXY)
    return u->sj < u->k && (c->mutation == ORC_MUT_RELAY_EARLY || q->tail > q->base + u->sj);
  return u->rj < u->k && q->ytail > q->base + u->rj;
}

static int gprod_enabled(const world* w, int ch, int x);
static int gcons_enabled(const world* w, int ch, int x);

static int enabled(const world* w, int ch, int act) {
  if (act >= ACT_GCONS) return gcons_enabled(w, ch, act - ACT_GCONS);
  if (act >= ACT_GPROD) return gprod_enabled(w, ch, act - ACT_GPROD);
  switch (act) {
    case ACT_PROD: return prod_enabled(w, ch);
    case ACT_CONS: return cons_enabled(w, ch);
    case ACT_PUB: return pub_enabled(w, ch);
    default: return proxy_enabled(w, ch, act);
  }
}

/* SIMPLE producer of step g: copy the chunk into slot g mod nslots, then
 * publish tail = g+1 (transfer page, copy mode; "Intra-Node Transport (P2P)"
 * section 4, POST / POLL: write the buffer, advance tail). */
static int simple_prod(world* w, int ch) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t g = q->base + u->pj, L = chunk_len(w, u, u->pj);
  int early = c->mutation == ORC_MUT_EARLY_TAIL;
  int do_copy = early ? (u->pphase == 1) : (u->pphase == 0);
  if (do_copy) {
    if (!slot_free(w, ch, g)) return ORC_V_OVERWRITE;
    memcpy(slot_ptr(w, ch, g), w->A + u->beg + u->pj * c->step_bytes, (size_t)L);
    mark_fill(w, ch, g);
  } else {
    q->tail = g + 1;
  }
  if (u->pphase == 0) {
    u->pphase = 1;
  } else {
    u->pphase = 0;
    u->pj++;
  }
  return 0;
}

/* SIMPLE consumer of step g: once tail > g, copy the slot into B, then free
 * the slot by publishing head = g+1 (same passages, consumer side). */
static int simple_cons(world* w, int ch) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t g = q->base + u->cj, L = chunk_len(w, u, u->cj);
  uint8_t* dst = w->B + u->beg + u->cj * c->step_bytes;
  const uint8_t* slot = slot_ptr(w, ch, g);
  if (c->mutation == ORC_MUT_NO_ACQUIRE) {
    uint8_t* reg = W_regs(w) + (size_t)ch * c->slot_bytes;
    if (u->cphase == 0) { /* load issued before the tail check */
      if (fill_of(w, ch, g) != (int64_t)g) return ORC_V_READ_UNFILLED;
      if (q->tail <= g) return ORC_V_READ_EARLY;
      memcpy(reg, slot, (size_t)L);
      u->cphase = 1;
    } else if (u->cphase == 1) {
      memcpy(dst, reg, (size_t)L);
      mark_drain(w, ch, g);
      u->cphase = 2;
    } else {
      q->head = g + 1;
      u->cphase = 0;
      u->cj++;
    }
    return 0;
  }
  int early = c->mutation == ORC_MUT_EARLY_HEAD;
  int do_copy = early ? (u->cphase == 1) : (u->cphase == 0);
  if (do_copy) {
    if (fill_of(w, ch, g) != (int64_t)g) return ORC_V_READ_UNFILLED;
    memcpy(dst, slot, (size_t)L);
    mark_drain(w, ch, g);
  } else {
    q->head = g + 1;
  }
  if (u->cphase == 0) {
    u->cphase = 1;
  } else {
    u->cphase = 0;
    u->cj++;
  }
  return 0;
}

/* LL producer: each 4 payload bytes go out as one 8-byte line {data, g+1}
 * stored at once; up to `budget` lines per action. */
static int ll_prod(world* w, int ch, uint64_t budget) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  if (u->pj == u->k) { /* Reading R4: bookkeeping tail, written once */
    q->tail = q->base + u->k;
    u->pfinal = 1;
    return 0;
  }
  uint64_t g = q->base + u->pj, L = chunk_len(w, u, u->pj), nl = ll_lines(L);
  const uint8_t* src = w->A + u->beg + u->pj * c->step_bytes;
  uint8_t* slot = slot_ptr(w, ch, g);
  if (u->pline == 0 && u->pphase == 0) {
    if (!slot_free(w, ch, g)) return ORC_V_OVERWRITE;
    mark_fill(w, ch, g);
  }
  uint32_t flag = (uint32_t)(g + 1);
  while (budget--) {
    uint8_t* line = slot + 8 * u->pline;
    if (c->mutation == ORC_MUT_TORN_LINE && u->pphase == 0) {
      put32(line + 4, flag); /* flag half first, data half in a later action */
      u->pphase = 1;
      continue;
    }
    if (c->mutation == ORC_MUT_TORN_LINE) {
      put32(line, ll_word(src, L, u->pline));
      u->pphase = 0;
    } else {
      put32(line, ll_word(src, L, u->pline));
      put32(line + 4, flag);
    }
    if (++u->pline == nl) {
      u->pline = 0;
      u->pj++;
      break;
    }
  }
  return 0;
}

/* LL consumer: poll each line until its flag equals g+1, keep its data
 * bytes, and after the last line free the slot with head = g+1. */
static int ll_cons(world* w, int ch, uint64_t budget) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t g = q->base + u->cj, L = chunk_len(w, u, u->cj), nl = ll_lines(L);
  int early = c->mutation == ORC_MUT_EARLY_HEAD;
  if (u->cphase == 1) {
    if (!early) mark_drain(w, ch, g);
    q->head = g + 1;
    u->cphase = 0;
    u->cline = 0;
    u->cj++;
    return 0;
  }
  if (early && u->cline == 0 && q->head != g + 1) { /* frees the slot at its first line */
    q->head = g + 1;
    return 0;
  }
  const uint8_t* slot = slot_ptr(w, ch, g);
  const uint8_t* src = w->A + u->beg + u->cj * c->step_bytes;
  uint8_t* dst = w->B + u->beg + u->cj * c->step_bytes;
  uint32_t flag = (uint32_t)(g + 1);
  while (budget--) {
    const uint8_t* line = slot + 8 * u->cline;
    if (get32(line + 4) != flag) break;
    uint32_t wv = get32(line);
    if (wv != ll_word(src, L, u->cline)) return ORC_V_READ_UNFILLED;
    for (uint64_t b = 0; b < 4 && 4 * u->cline + b < L; ++b) dst[4 * u->cline + b] = (uint8_t)(wv >> (8 * b));
    if (++u->cline == nl) {
      if (early) { /* head already published; the step is done */
        mark_drain(w, ch, g);
        u->cline = 0;
        u->cj++;
      } else {
        u->cphase = 1;
      }
      break;
    }
  }
  return 0;
}

/* LL in groups of m steps (the striped kernels' order, ORC_ORDER_LL_GROUP):
 * the lines and flags are those of Reading R4; what changes is who writes
 * and reads which step, and when a slot is handed back.  Sub-producer x
 * writes steps x, x+m, ... in order, each only on credit (Reading R2), so
 * different sub-producers may be in different groups at once.  Sub-consumer
 * x reads step (group start) + x of the group its barrier released it into;
 * the group's last reader completes the barrier, and one head store, head =
 * (group end), then frees every slot of the group. */
static int gprod_enabled(const world* w, int ch, int x) {
  const orc_conn* c = w->cfg;
  if (x >= ll_group(c)) return 0;
  const orc_ctrl* q = &W_ctrl(w)[ch];
  const orc_cur* u = &W_cur(w)[ch];
  if (u->gpj[x] >= u->k) return 0;
  return u->gpl[x] > 0 || credit_ok(w, q, q->base + u->gpj[x]);
}

static int gprod(world* w, int ch, int x, uint64_t budget) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t j = u->gpj[x], g = q->base + j, L = chunk_len(w, u, j), nl = ll_lines(L);
  const uint8_t* src = w->A + u->beg + j * c->step_bytes;
  uint8_t* slot = slot_ptr(w, ch, g);
  if (u->gpl[x] == 0) {
    if (!slot_free(w, ch, g)) return ORC_V_OVERWRITE;
    mark_fill(w, ch, g);
  }
  while (budget--) {
    uint8_t* line = slot + 8 * u->gpl[x];
    put32(line, ll_word(src, L, u->gpl[x]));
    put32(line + 4, (uint32_t)(g + 1));
    if (++u->gpl[x] == nl) {
      u->gpl[x] = 0;
      u->gpj[x] += (uint64_t)ll_group(c);
      break;
    }
  }
  return 0;
}

static int gcons_enabled(const world* w, int ch, int x) {
  const orc_conn* c = w->cfg;
  if (x >= ll_group(c)) return 0;
  const orc_ctrl* q = &W_ctrl(w)[ch];
  const orc_cur* u = &W_cur(w)[ch];
  uint64_t j = u->gcj[x];
  if (j >= group_end(u, ll_group(c), u->cbar)) return 0; /* done, or waiting at the barrier */
  if (x == 0 && u->cj < u->cbar) return 0; /* sub-consumer 0 stores the last group's head first */
  const uint8_t* line = slot_ptr(w, ch, q->base + j) + 8 * u->gcl[x];
  return get32(line + 4) == (uint32_t)(q->base + j + 1);
}

static int gcons(world* w, int ch, int x, uint64_t budget) {
  const orc_conn* c = w->cfg;
  const int m = ll_group(c);
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t j = u->gcj[x], g = q->base + j, L = chunk_len(w, u, j), nl = ll_lines(L);
  const uint8_t* slot = slot_ptr(w, ch, g);
  const uint8_t* src = w->A + u->beg + j * c->step_bytes;
  uint8_t* dst = w->B + u->beg + j * c->step_bytes;
  while (budget--) {
    const uint8_t* line = slot + 8 * u->gcl[x];
    if (get32(line + 4) != (uint32_t)(g + 1)) break;
    uint32_t wv = get32(line);
    if (wv != ll_word(src, L, u->gcl[x])) return ORC_V_READ_UNFILLED;
    for (uint64_t b = 0; b < 4 && 4 * u->gcl[x] + b < L; ++b)
      dst[4 * u->gcl[x] + b] = (uint8_t)(wv >> (8 * b));
    if (++u->gcl[x] == nl) {
      mark_drain(w, ch, g);
      u->gcl[x] = 0;
      u->gcj[x] += (uint64_t)m;
      uint64_t s = u->cbar, e = group_end(u, m, s);
      int all = 1; /* the barrier: every step of the group read */
      for (int y = 0; y < m && s + (uint64_t)y < e; ++y)
        if (u->gcj[y] < s + (uint64_t)m) all = 0;
      if (all) u->cbar = e;
      break;
    }
  }
  return 0;
}

/* The group's head store frees every slot of the group at once. */
static int ghead(world* w, int ch) {
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t e = group_end(u, ll_group(w->cfg), u->cj);
  q->head = q->base + e;
  u->cj = e;
  return 0;
}

/* Reading R4's bookkeeping tail, once every sub-producer is done. */
static int gfinal(world* w, int ch) {
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  q->tail = q->base + u->k;
  u->pj = u->k;
  u->pfinal = 1;
  return 0;
}

/* Zero-copy producer (Reading R7): take the published address, clear the
 * word, write the chunk straight into B there, publish tail = g+1.  In the
 * take-ahead order the producer takes step g+1's address between writing
 * step g and publishing its tail (phase 2), and step g+1 then starts from
 * that address instead of the word. */
static uint64_t zc_take(const orc_conn* c, orc_ctrl* q) {
  uint64_t p = q->ptrx;
  if (c->mutation != ORC_MUT_ZC_NO_RESET) q->ptrx = 0;
  return p;
}

static int zc_prod(world* w, int ch) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t g = q->base + u->pj, off = u->beg + u->pj * c->step_bytes;
  if (u->pphase == 0) {
    uint64_t p = u->pnext ? u->pnext : zc_take(c, q);
    u->pnext = 0;
    if (p != off + 1) return ORC_V_WRONG_PTR;
    u->pptr = p;
    u->pphase = 1;
  } else if (u->pphase == 1) {
    memcpy(w->B + (u->pptr - 1), w->A + off, (size_t)chunk_len(w, u, u->pj));
    u->pphase = 2;
  } else if (u->pphase == 2 && zc_takes_ahead(c, u)) {
    uint64_t p = zc_take(c, q);
    if (p != off + c->step_bytes + 1) return ORC_V_WRONG_PTR;
    u->pnext = p;
    u->pphase = 3;
  } else {
    q->tail = g + 1;
    u->pphase = 0;
    u->pj++;
  }
  return 0;
}

/* Zero-copy receiver, publishing cursor: offer the next step's destination
 * once the word is clear. */
static int zc_pub(world* w, int ch) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  q->ptrx = u->beg + u->cnpub * c->step_bytes + 1;
  u->cnpub++;
  return 0;
}

/* Zero-copy receiver, completion cursor: tail > g means step g landed, so
 * its bytes must be in B when the receiver takes it. */
static int zc_done(world* w, int ch) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t off = u->beg + u->cj * c->step_bytes;
  if (memcmp(w->B + off, w->A + off, (size_t)chunk_len(w, u, u->cj)) != 0)
    return ORC_V_READ_UNFILLED;
  q->head = q->base + u->cj + 1;
  u->cj++;
  return 0;
}

/* Zero-copy direct producer (the page's second kind): write the chunk into
 * B at its own offset, then publish tail = g+1. */
static int zcd_prod(world* w, int ch) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t g = q->base + u->pj, off = u->beg + u->pj * c->step_bytes;
  int early = c->mutation == ORC_MUT_EARLY_TAIL;
  if ((u->pphase == 0) != early) {
    memcpy(w->B + off, w->A + off, (size_t)chunk_len(w, u, u->pj));
  } else {
    q->tail = g + 1;
  }
  if (u->pphase == 0) {
    u->pphase = 1;
  } else {
    u->pphase = 0;
    u->pj++;
  }
  return 0;
}

/* RELAY proxy step: copy the chunk of step g from FIFO `from` to FIFO `to`
 * (the slot there must be free: its previous step drained), then publish
 * the proxy's tail = g+1. */
static int relay_move(world* w, int ch, int from, int to, uint64_t* cursor, uint64_t* tail_out) {
  const orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t g = q->base + *cursor;
  if (fill_of_in(w, from, ch, g) != (int64_t)g) return ORC_V_READ_UNFILLED;
  if (!slot_free_in(w, to, ch, g)) return ORC_V_OVERWRITE;
  memcpy(slot_ptr_in(w, to, ch, g), slot_ptr_in(w, from, ch, g), (size_t)chunk_len(w, u, *cursor));
  mark_drain_in(w, from, ch, g);
  mark_fill_in(w, to, ch, g);
  *tail_out = g + 1;
  (*cursor)++;
  return 0;
}

/* RELAY consumer: once the receive proxy's tail passes g, copy receive slot
 * g into B, then publish head = g+1 (the producer's credit). */
static int relay_cons(world* w, int ch) {
  const orc_conn* c = w->cfg;
  orc_ctrl* q = &W_ctrl(w)[ch];
  orc_cur* u = &W_cur(w)[ch];
  uint64_t g = q->base + u->cj;
  if (u->cphase == 0) {
    if (fill_of_in(w, 2, ch, g) != (int64_t)g) return ORC_V_READ_UNFILLED;
    memcpy(w->B + u->beg + u->cj * c->step_bytes, slot_ptr_in(w, 2, ch, g),
           (size_t)chunk_len(w, u, u->cj));
    mark_drain_in(w, 2, ch, g);
    u->cphase = 1;
  } else {
    q->head = g + 1;
    u->cphase = 0;
    u->cj++;
  }
  return 0;
}

static int fire(world* w, int ch, int act, uint64_t budget) {
  orc_ctrl* rq = &W_ctrl(w)[ch];
  orc_cur* ru = &W_cur(w)[ch];
  switch (w->cfg->proto) {
    case ORC_SIMPLE:
      return act == ACT_PROD ? simple_prod(w, ch) : simple_cons(w, ch);
    case ORC_LL:
      if (ll_group(w->cfg)) {
        if (act >= ACT_GCONS) return gcons(w, ch, act - ACT_GCONS, budget);
        if (act >= ACT_GPROD) return gprod(w, ch, act - ACT_GPROD, budget);
        return act == ACT_PROD ? gfinal(w, ch) : ghead(w, ch);
      }
      return act == ACT_PROD ? ll_prod(w, ch, budget) : ll_cons(w, ch, budget);
    case ORC_ZCD:
      return act == ACT_PROD ? zcd_prod(w, ch) : zc_done(w, ch);
    case ORC_RELAY:
      switch (act) {
        case ACT_PROD: return simple_prod(w, ch);
        case ACT_CONS: return relay_cons(w, ch);
        case ACT_SPROXY: return relay_move(w, ch, 0, 1, &ru->sj, &rq->ytail);
        default: return relay_move(w, ch, 1, 2, &ru->rj, &rq->gtail);
      }
    default:
      return act == ACT_PROD ? zc_prod(w, ch) : act == ACT_PUB ? zc_pub(w, ch) : zc_done(w, ch);
  }
}

/* Steps the producer of a channel has begun, for the in-flight bound. */
static int window_ok(const world* w, int ch) {
  const orc_conn* c = w->cfg;
  if (!has_fifo(c->proto)) return 1;
  const orc_ctrl* q = &W_ctrl(w)[ch];
  const orc_cur* u = &W_cur(w)[ch];
  const int m = ll_group(c);
  if (m) { /* one past the highest step any sub-producer has begun */
    uint64_t top = 0;
    for (int x = 0; x < m; ++x) {
      uint64_t j = u->gpj[x];
      uint64_t t = u->gpl[x] > 0 ? j + 1 : (j >= (uint64_t)m ? j - (uint64_t)m + 1 : 0);
      if (t > top) top = t;
    }
    return q->base + top <= q->head + (uint64_t)c->nslots;
  }
  uint64_t begun = u->pj;
  if (u->pj < u->k && (u->pphase != 0 || (c->proto == ORC_LL && u->pline > 0))) ++begun;
  return q->base + begun <= q->head + (uint64_t)c->nslots;
}

static int world_done(const world* w) {
  const orc_conn* c = w->cfg;
  const orc_cur* u = W_cur(w);
  for (int ch = 0; ch < c->nch; ++ch) {
    if (u[ch].pj != u[ch].k || u[ch].cj != u[ch].k) return 0;
    if (c->proto == ORC_LL && !u[ch].pfinal) return 0;
    for (int x = 0; x < ll_group(c); ++x) /* no sub-consumer still reading */
      if (u[ch].gcj[x] < u[ch].k) return 0;
    if (c->proto == ORC_RELAY && (u[ch].sj != u[ch].k || u[ch].rj != u[ch].k)) return 0;
  }
  return 1;
}

/* Closed-form end state: head == tail == base + k, ptrExchange == 0. */
static int final_counters_ok(const world* w, int* bad_ch) {
  const orc_ctrl* q = W_ctrl(w);
  const orc_cur* u = W_cur(w);
  for (int ch = 0; ch < w->cfg->nch; ++ch) {
    uint64_t want = q[ch].base + u[ch].k;
    if (q[ch].head != want || q[ch].tail != want || q[ch].ptrx != 0 ||
        (w->cfg->proto == ORC_RELAY && (q[ch].ytail != want || q[ch].gtail != want))) {
      *bad_ch = ch;
      return 0;
    }
  }
  return 1;
}

/* Commits a finished transfer back into the connection. */
static void world_commit(const world* w, orc_conn* c) {
  const orc_ctrl* q = W_ctrl(w);
  const orc_cur* u = W_cur(w);
  for (int ch = 0; ch < c->nch; ++ch) {
    c->ctrl[ch] = q[ch];
    c->ctrl[ch].base = q[ch].base + u[ch].k; /* Reading R8 */
  }
}

/* ----------------------------------------------------------- deterministic run
 * Round-robin over channels; each actor that can move takes one action (an
 * LL action covers every line it can write or read within the current step). */
int orc_run(orc_conn* c, const uint8_t* A, uint8_t* B, uint64_t n) {
  if (!c || (n && (!A || !B))) return ORC_E_ARG;
  world w;
  memset(&w, 0, sizeof(w));
  w.meta_bytes = meta_size(c);
  w.meta = (uint8_t*)malloc((size_t)w.meta_bytes);
  if (!w.meta) return ORC_E_NOMEM;
  int rc = world_begin(&w, c, A, n);
  if (rc) {
    free(w.meta);
    return rc;
  }
  w.fifo = c->fifo;
  w.B = B;
  while (!world_done(&w)) {
    int moved = 0;
    for (int ch = 0; ch < c->nch && !rc; ++ch) {
      static const int order[N_ACT_ALL] = {
          ACT_GPROD, ACT_GPROD + 1, ACT_GPROD + 2, ACT_GPROD + 3, ACT_PROD, ACT_PUB, ACT_SPROXY,
          ACT_RPROXY, ACT_GCONS, ACT_GCONS + 1, ACT_GCONS + 2, ACT_GCONS + 3, ACT_CONS};
      for (int a = 0; a < N_ACT_ALL && !rc; ++a) {
        if (!enabled(&w, ch, order[a])) continue;
        rc = fire(&w, ch, order[a], ~0ull);
        if (!rc && !window_ok(&w, ch)) rc = ORC_V_WINDOW;
        moved = 1;
      }
    }
    if (rc) break;
    if (!moved) {
      rc = ORC_V_DEADLOCK;
      break;
    }
  }
  int bad = -1;
  if (!rc && !final_counters_ok(&w, &bad)) rc = ORC_V_COUNTERS;
  if (!rc && n && memcmp(A, B, (size_t)n) != 0) rc = ORC_V_RESULT;
  if (!rc) world_commit(&w, c);
  free(w.meta);
  return rc;
}

int orc_run_pingpong(orc_conn* fwd, orc_conn* rev, const uint8_t* a, uint8_t* b, uint8_t* cbuf,
                     uint64_t n, int iters) {
  if (!fwd || !rev || iters < 0) return ORC_E_ARG;
  for (int it = 0; it < iters; ++it) {
    int rc = orc_run(fwd, a, b, n);
    if (rc) return rc;
    rc = orc_run(rev, b, cbuf, n);
    if (rc) return rc;
  }
  return 0;
}

/* ------------------------------------------------------------- enumerator
 * Depth-first search over every interleaving of single actions (one line
 * for LL).  States are deduplicated by a 128-bit fingerprint of the whole
 * state (meta, FIFO bytes, destination with its guard zones). */
typedef struct {
  uint64_t a, b;
} fp128;

static fp128 fingerprint(const uint8_t* p, uint64_t n) {
  uint64_t h1 = 0x9E3779B97F4A7C15ull ^ n, h2 = 0xC2B2AE3D27D4EB4Full + n;
  for (uint64_t i = 0; i < n; ++i) {
    h1 = (h1 ^ p[i]) * 0x100000001B3ull;
    h2 = (h2 + p[i] + 1) * 0xFF51AFD7ED558CCDull;
    h2 ^= h2 >> 29;
  }
  h1 ^= h1 >> 31;
  h1 *= 0x94D049BB133111EBull;
  h1 ^= h1 >> 32;
  fp128 r = {h1, h2};
  return r;
}

typedef struct {
  fp128* slots;
  uint8_t* used;
  uint64_t cap, count;
} fpset;

static int fpset_grow(fpset* s);

static int fpset_insert(fpset* s, fp128 f) { /* 1 = new, 0 = seen, <0 = no memory */
  if ((s->count + 1) * 2 > s->cap && fpset_grow(s)) return ORC_E_NOMEM;
  uint64_t i = f.a & (s->cap - 1);
  while (s->used[i]) {
    if (s->slots[i].a == f.a && s->slots[i].b == f.b) return 0;
    i = (i + 1) & (s->cap - 1);
  }
  s->used[i] = 1;
  s->slots[i] = f;
  s->count++;
  return 1;
}

static int fpset_grow(fpset* s) {
  uint64_t ncap = s->cap ? s->cap * 2 : 1024;
  fp128* ns = (fp128*)calloc((size_t)ncap, sizeof(fp128));
  uint8_t* nu = (uint8_t*)calloc((size_t)ncap, 1);
  if (!ns || !nu) {
    free(ns);
    free(nu);
    return ORC_E_NOMEM;
  }
  fpset old = *s;
  s->slots = ns;
  s->used = nu;
  s->cap = ncap;
  s->count = 0;
  for (uint64_t i = 0; i < old.cap; ++i)
    if (old.used[i]) fpset_insert(s, old.slots[i]);
  free(old.slots);
  free(old.used);
  return 0;
}

static const char* vname(int v) {
  switch (v) {
    case ORC_V_OVERWRITE: return "producer overwrote a slot that was not drained";
    case ORC_V_READ_UNFILLED: return "consumer read a slot or line that did not hold its step";
    case ORC_V_READ_EARLY: return "consumer read a slot before observing its tail";
    case ORC_V_WINDOW: return "more than nslots steps in flight";
    case ORC_V_WRONG_PTR: return "producer took an address not published for its step";
    case ORC_V_DEADLOCK: return "no actor can move before the transfer ends";
    case ORC_V_RESULT: return "destination differs from source or a guard byte changed";
    case ORC_V_COUNTERS: return "final head/tail/ptrExchange not at their closed form";
    case ORC_V_CONFLUENCE: return "two interleavings ended in different states";
    case ORC_V_STATE_LIMIT: return "state budget exhausted";
    default: return "error";
  }
}

static const char* aname(int act) {
  static const char* names[N_ACT_ALL] = {
      "producer",       "consumer",       "publisher",      "send proxy",     "receive proxy",
      "sub-producer 0", "sub-producer 1", "sub-producer 2", "sub-producer 3", "sub-consumer 0",
      "sub-consumer 1", "sub-consumer 2", "sub-consumer 3"};
  return act >= 0 && act < N_ACT_ALL ? names[act] : "?";
}

typedef struct {
  uint8_t** items;
  uint64_t n, cap;
} blobstack;

static int bs_push(blobstack* s, uint8_t* b) {
  if (s->n == s->cap) {
    uint64_t nc = s->cap ? s->cap * 2 : 256;
    uint8_t** ni = (uint8_t**)realloc(s->items, (size_t)nc * sizeof(uint8_t*));
    if (!ni) return ORC_E_NOMEM;
    s->items = ni;
    s->cap = nc;
  }
  s->items[s->n++] = b;
  return 0;
}

static uint8_t guard_byte(uint64_t i) { return (uint8_t)(i * 151u + 89u); }

int orc_enumerate(int proto, int nch, int nslots, uint64_t slot_bytes, const uint8_t* A, uint64_t n,
                  int mutation, int order, int prior_runs, uint64_t max_states,
                  orc_enum_result* out) {
  if (!out || (n && !A) || prior_runs < 0) return ORC_E_ARG;
  int group_order = order > ORC_ORDER_LL_GROUP(0) && order <= ORC_ORDER_LL_GROUP(ORC_GROUP_MAX);
  if (order != ORC_ORDER_PAGES && order != ORC_ORDER_ZC_TAKE_AHEAD && !group_order)
    return ORC_E_ARG;
  if (group_order && proto != ORC_LL) return ORC_E_ARG;
  memset(out, 0, sizeof(*out));
  out->channel = -1;
  orc_conn* c = orc_conn_new(proto, nch, nslots, slot_bytes);
  if (!c) return ORC_E_ARG;
  int rc = 0;
  if (prior_runs) {
    uint8_t* tmp = (uint8_t*)malloc((size_t)(n ? n : 1));
    if (!tmp) {
      orc_conn_free(c);
      return ORC_E_NOMEM;
    }
    for (int r = 0; r < prior_runs && !rc; ++r) rc = orc_run(c, A, tmp, n);
    free(tmp);
    if (rc) {
      orc_conn_free(c);
      return rc;
    }
  }
  c->mutation = mutation;
  c->order = order;

  uint64_t mb = meta_size(c), fb = fifo_size(c), bb = n + 2 * GUARD, blob = mb + fb + bb;
  world w;
  memset(&w, 0, sizeof(w));
  w.meta_bytes = mb;
  uint8_t* root = (uint8_t*)malloc((size_t)blob);
  uint8_t* first_terminal = (uint8_t*)malloc((size_t)blob);
  if (!root || !first_terminal) {
    free(root);
    free(first_terminal);
    orc_conn_free(c);
    return ORC_E_NOMEM;
  }
#define BIND(wp, base)                    \
  do {                                    \
    (wp)->meta = (base);                  \
    (wp)->fifo = (base) + mb;             \
    (wp)->B = (base) + mb + fb + GUARD;   \
  } while (0)
  BIND(&w, root);
  rc = world_begin(&w, c, A, n);
  if (c->fifo) memcpy(w.fifo, c->fifo, (size_t)fb);
  for (uint64_t i = 0; i < bb; ++i) root[mb + fb + i] = guard_byte(i);

  fpset seen = {0};
  blobstack st = {0};
  int have_terminal = 0;
  if (!rc) {
    fpset_insert(&seen, fingerprint(root, blob));
    rc = bs_push(&st, root);
    root = NULL;
  }
  while (!rc && st.n) {
    uint8_t* cur = st.items[--st.n];
    world v = w;
    BIND(&v, cur);
    if (world_done(&v)) {
      int bad = -1;
      out->terminals++;
      if (!final_counters_ok(&v, &bad)) {
        rc = ORC_V_COUNTERS;
        out->channel = bad;
      } else if (n && memcmp(v.B, A, (size_t)n) != 0) {
        rc = ORC_V_RESULT;
      } else {
        for (uint64_t i = 0; i < GUARD && !rc; ++i)
          if (v.B[-(int64_t)GUARD + (int64_t)i] != guard_byte(i) ||
              v.B[n + i] != guard_byte(GUARD + n + i))
            rc = ORC_V_RESULT;
      }
      if (!rc) {
        if (!have_terminal) {
          memcpy(first_terminal, cur, (size_t)blob);
          have_terminal = 1;
        } else if (memcmp(first_terminal, cur, (size_t)blob) != 0) {
          rc = ORC_V_CONFLUENCE;
        }
      }
      free(cur);
      continue;
    }
    int any = 0;
    for (int ch = 0; ch < nch && !rc; ++ch) {
      for (int act = 0; act < N_ACT_ALL && !rc; ++act) {
        if (!enabled(&v, ch, act)) continue;
        any = 1;
        uint8_t* nxt = (uint8_t*)malloc((size_t)blob);
        if (!nxt) {
          rc = ORC_E_NOMEM;
          break;
        }
        memcpy(nxt, cur, (size_t)blob);
        world x = w;
        BIND(&x, nxt);
        int vr = fire(&x, ch, act, 1);
        if (!vr && !window_ok(&x, ch)) vr = ORC_V_WINDOW;
        out->transitions++;
        if (vr) {
          rc = vr;
          out->channel = ch;
          snprintf(out->msg, sizeof(out->msg), "channel %d %s: %s", ch, aname(act), vname(vr));
          free(nxt);
          break;
        }
        int ins = fpset_insert(&seen, fingerprint(nxt, blob));
        if (ins < 0) {
          rc = ins;
          free(nxt);
        } else if (ins == 0) {
          free(nxt);
        } else if (seen.count > max_states) {
          rc = ORC_V_STATE_LIMIT;
          free(nxt);
        } else {
          rc = bs_push(&st, nxt);
          if (rc) free(nxt);
        }
      }
    }
    if (!rc && !any) rc = ORC_V_DEADLOCK;
    free(cur);
  }
#undef BIND
  out->states = seen.count;
  out->violation = rc > 0 ? rc : 0;
  if (rc > 0 && !out->msg[0]) snprintf(out->msg, sizeof(out->msg), "%s", vname(rc));
  for (uint64_t i = 0; i < st.n; ++i) free(st.items[i]);
  free(st.items);
  free(seen.slots);
  free(seen.used);
  free(root);
  free(first_terminal);
  orc_conn_free(c);
  return rc < 0 ? rc : 0;
}
