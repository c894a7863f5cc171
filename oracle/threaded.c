/*
 * threaded.c -- the oracle's threaded mode: the same producer and consumer
 * actions as the sequential simulator in oracle.c (Readings R1-R8 there),
 * run by real threads that hand off through C11 atomics.
 *
 * TEST INFRASTRUCTURE ONLY: a second opinion for the tests (its end state
 * must equal the sequential one) and the benchmark's multi-core CPU
 * baseline.  It shares no code with the GPU library.
 *
 * Hand-offs, in the pages' terms ("【NCCL】transport数据传输（二）", copy mode
 * and zero-copy first kind; "Intra-Node Transport (P2P)" section 4, POST /
 * POLL):
 *  - SIMPLE producer of step g: wait until g - head < nslots (acquire), copy
 *    the chunk into slot g mod nslots, publish tail = g+1 (release).
 *    Consumer: wait until tail > g (acquire), copy the slot out, publish
 *    head = g+1 (release).
 *  - LL: the producer waits for the same credit, then stores each line
 *    {4 data bytes, flag g+1} as one 64-bit atomic store; the consumer loads
 *    each line until its flag is g+1 ("RDMA and GPUDirect" section 四.1,
 *    option 2) and then publishes head; the producer writes its final step
 *    count to tail once at the end (Reading R4).
 *  - Copy-engine relay (the shm transport's useMemcpy mode): a send proxy,
 *    seeing tail > g, copies send slot g into the staging FIFO and publishes
 *    its tail; a receive proxy copies staging slot g into the receive FIFO
 *    once that tail passes g and publishes its own tail, which the consumer
 *    polls; head stays the producer's credit end to end.
 *  - Zero-copy: the receiver publishes the next destination whenever the
 *    word is 0 and publishes head once tail passes a step; the producer
 *    takes the address, clears the word, writes the chunk into B there and
 *    publishes tail.  Zero-copy direct: the destination is known, so the
 *    producer writes the chunk at its own offset of B and publishes tail,
 *    and the receiver only answers tail with head.
 *
 * Each channel has two actors (producer; consumer or receiver), four for the
 * relay (plus the two proxies).  Actors are dealt round-robin to the
 * threads; a thread sweeps its actors, each taking whatever action is ready
 * without blocking, so any thread count from 1 to the number of actors makes
 * progress.
 */
#define _GNU_SOURCE
#include <pthread.h>
#include <sched.h>
#include <stdatomic.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "oracle.h"
#include "oracle_internal.h"

#define IDLE_LIMIT_S 20.0 /* no action anywhere for this long: report a deadlock */

/* Shared, atomic copy of a connection's control words during a job. */
typedef struct {
  const orc_conn* c;
  _Atomic uint64_t* head;
  _Atomic uint64_t* tail;
  _Atomic uint64_t* ptrx;
  _Atomic uint64_t* ytail; /* relay: send proxy's tail */
  _Atomic uint64_t* gtail; /* relay: receive proxy's tail */
} tconn;

/* One side's cursor over one channel of one transfer. */
typedef struct {
  uint64_t base, beg, len, k; /* step base, channel range, steps */
  uint64_t j;                 /* producer: next step; consumer/receiver: next step to complete */
  uint64_t line;              /* LL consumer: next line of step j */
  uint64_t npub;              /* zero-copy receiver: steps published */
  int done;
} tside;

static double now_s(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

static int tconn_init(tconn* t, const orc_conn* c) {
  t->c = c;
  t->head = calloc((size_t)c->nch, sizeof(*t->head));
  t->tail = calloc((size_t)c->nch, sizeof(*t->tail));
  t->ptrx = calloc((size_t)c->nch, sizeof(*t->ptrx));
  t->ytail = calloc((size_t)c->nch, sizeof(*t->ytail));
  t->gtail = calloc((size_t)c->nch, sizeof(*t->gtail));
  if (!t->head || !t->tail || !t->ptrx || !t->ytail || !t->gtail) return ORC_E_NOMEM;
  for (int ch = 0; ch < c->nch; ++ch) {
    atomic_init(&t->head[ch], c->ctrl[ch].head);
    atomic_init(&t->tail[ch], c->ctrl[ch].tail);
    atomic_init(&t->ptrx[ch], c->ctrl[ch].ptrx);
    atomic_init(&t->ytail[ch], c->ctrl[ch].ytail);
    atomic_init(&t->gtail[ch], c->ctrl[ch].gtail);
  }
  return 0;
}

static void tconn_free(tconn* t) {
  free(t->head);
  free(t->tail);
  free(t->ptrx);
  free(t->ytail);
  free(t->gtail);
}

/* Cursors of every channel for a transfer of n bytes (Reading R6). */
static void sides_begin(tside* s, const orc_conn* c, const uint64_t* base, uint64_t n) {
  uint64_t beg[64], len[64];
  orc_partition(n, c->nch, beg, len);
  for (int ch = 0; ch < c->nch; ++ch) {
    memset(&s[ch], 0, sizeof(s[ch]));
    s[ch].base = base[ch];
    s[ch].beg = beg[ch];
    s[ch].len = len[ch];
    s[ch].k = (len[ch] + c->step_bytes - 1) / c->step_bytes;
  }
}

static uint64_t chunk(const orc_conn* c, const tside* s, uint64_t j) {
  uint64_t rest = s->len - j * c->step_bytes;
  return rest < c->step_bytes ? rest : c->step_bytes;
}

/* Slot g of a channel in FIFO f (relay: 0 send, 1 staging, 2 receive). */
static uint8_t* slot_in(const orc_conn* c, int f, int ch, uint64_t g) {
  return c->fifo + (((uint64_t)f * c->nch + (uint64_t)ch) * c->nslots + g % (uint64_t)c->nslots) *
                       c->slot_bytes;
}
static uint8_t* slot(const orc_conn* c, int ch, uint64_t g) { return slot_in(c, 0, ch, g); }

/* Line value of `line` in a chunk of L bytes: data word in bytes 0..3 and the
 * flag in bytes 4..7, little-endian (Reading R4), as one 64-bit integer. */
static uint64_t ll_line_value(const uint8_t* src, uint64_t L, uint64_t line, uint32_t flag) {
  uint32_t w = 0;
  for (uint64_t b = 0; b < 4 && 4 * line + b < L; ++b) w |= (uint32_t)src[4 * line + b] << (8 * b);
  uint8_t bytes[8];
  for (int b = 0; b < 4; ++b) {
    bytes[b] = (uint8_t)(w >> (8 * b));
    bytes[4 + b] = (uint8_t)(flag >> (8 * b));
  }
  uint64_t v;
  memcpy(&v, bytes, 8);
  return v;
}

/* ---------------------------------------------------------------- actions
 * Each returns 1 if it took an action, 0 if it had to wait, or a negative
 * value (minus a violation code) on a protocol violation. */
static int credit(const tconn* t, int ch, uint64_t g) {
  uint64_t h = atomic_load_explicit(&t->head[ch], memory_order_acquire);
  return g - h < (uint64_t)t->c->nslots;
}

static int try_prod(const tconn* t, int ch, tside* s, const uint8_t* A) {
  const orc_conn* c = t->c;
  if (s->j == s->k) {
    if (c->proto == ORC_LL) atomic_store_explicit(&t->tail[ch], s->base + s->k, memory_order_release);
    s->done = 1;
    return 1;
  }
  const uint64_t g = s->base + s->j, L = chunk(c, s, s->j);
  const uint8_t* src = A + s->beg + s->j * c->step_bytes;
  if (!credit(t, ch, g)) return 0;
  uint8_t* d = slot(c, ch, g);
  if (c->proto == ORC_SIMPLE || c->proto == ORC_RELAY) {
    memcpy(d, src, (size_t)L);
    atomic_store_explicit(&t->tail[ch], g + 1, memory_order_release);
  } else {
    const uint32_t flag = (uint32_t)(g + 1);
    for (uint64_t line = 0; line < (L + 3) / 4; ++line)
      atomic_store_explicit((_Atomic uint64_t*)(void*)(d + 8 * line),
                            ll_line_value(src, L, line, flag), memory_order_relaxed);
  }
  s->j++;
  return 1;
}

/* Zero-copy producer: the address token is (offset of the chunk in B) + 1. */
static int try_zc_prod(const tconn* t, int ch, tside* s, const uint8_t* A, uint8_t* B) {
  const orc_conn* c = t->c;
  if (s->j == s->k) {
    s->done = 1;
    return 1;
  }
  uint64_t p = atomic_load_explicit(&t->ptrx[ch], memory_order_acquire);
  if (p == 0) return 0;
  atomic_store_explicit(&t->ptrx[ch], 0, memory_order_release);
  const uint64_t off = s->beg + s->j * c->step_bytes;
  if (p != off + 1) return -ORC_V_WRONG_PTR;
  memcpy(B + (p - 1), A + off, (size_t)chunk(c, s, s->j));
  atomic_store_explicit(&t->tail[ch], s->base + s->j + 1, memory_order_release);
  s->j++;
  return 1;
}

/* Zero-copy direct producer: the destination is known, so it writes the
 * chunk at its own offset of B and publishes tail. */
static int try_zcd_prod(const tconn* t, int ch, tside* s, const uint8_t* A, uint8_t* B) {
  const orc_conn* c = t->c;
  if (s->j == s->k) {
    s->done = 1;
    return 1;
  }
  const uint64_t off = s->beg + s->j * c->step_bytes;
  memcpy(B + off, A + off, (size_t)chunk(c, s, s->j));
  atomic_store_explicit(&t->tail[ch], s->base + s->j + 1, memory_order_release);
  s->j++;
  return 1;
}

static int prod_action(const tconn* t, int ch, tside* s, const uint8_t* A, uint8_t* B) {
  switch (t->c->proto) {
    case ORC_ZC:
      return try_zc_prod(t, ch, s, A, B);
    case ORC_ZCD:
      return try_zcd_prod(t, ch, s, A, B);
    default:
      return try_prod(t, ch, s, A);
  }
}

static int cons_action(const tconn* t, int ch, tside* s, uint8_t* B) {
  const orc_conn* c = t->c;
  if (c->proto == ORC_ZC || c->proto == ORC_ZCD) {
    int moved = 0;
    if (c->proto == ORC_ZCD) s->npub = s->k; /* nothing to publish */
    if (s->npub < s->k && atomic_load_explicit(&t->ptrx[ch], memory_order_acquire) == 0) {
      atomic_store_explicit(&t->ptrx[ch], s->beg + s->npub * c->step_bytes + 1,
                            memory_order_release);
      s->npub++;
      moved = 1;
    }
    while (s->j < s->k &&
           atomic_load_explicit(&t->tail[ch], memory_order_acquire) > s->base + s->j) {
      atomic_store_explicit(&t->head[ch], s->base + s->j + 1, memory_order_release);
      s->j++;
      moved = 1;
    }
    if (s->npub == s->k && s->j == s->k) s->done = 1;
    return moved;
  }
  if (s->j == s->k) {
    s->done = 1;
    return 1;
  }
  const uint64_t g = s->base + s->j, L = chunk(c, s, s->j);
  uint8_t* dst = B + s->beg + s->j * c->step_bytes;
  const uint8_t* sl = slot(c, ch, g);
  if (c->proto == ORC_SIMPLE) {
    if (atomic_load_explicit(&t->tail[ch], memory_order_acquire) <= g) return 0;
    memcpy(dst, sl, (size_t)L);
  } else if (c->proto == ORC_RELAY) {
    if (atomic_load_explicit(&t->gtail[ch], memory_order_acquire) <= g) return 0;
    memcpy(dst, slot_in(c, 2, ch, g), (size_t)L);
  } else {
    const uint32_t flag = (uint32_t)(g + 1);
    const uint64_t nl = (L + 3) / 4;
    int moved = 0;
    while (s->line < nl) {
      uint64_t v = atomic_load_explicit((_Atomic uint64_t*)(void*)(sl + 8 * s->line),
                                        memory_order_relaxed);
      uint8_t bytes[8];
      memcpy(bytes, &v, 8);
      uint32_t f = (uint32_t)bytes[4] | (uint32_t)bytes[5] << 8 | (uint32_t)bytes[6] << 16 |
                   (uint32_t)bytes[7] << 24;
      if (f != flag) return moved;
      for (uint64_t b = 0; b < 4 && 4 * s->line + b < L; ++b) dst[4 * s->line + b] = bytes[b];
      s->line++;
      moved = 1;
    }
    s->line = 0;
  }
  atomic_store_explicit(&t->head[ch], g + 1, memory_order_release);
  s->j++;
  return 1;
}

/* Relay proxy: once `in` passes step g, copy slot g of FIFO `from` into
 * FIFO `to` and publish `out` = g+1. */
static int proxy_action(const tconn* t, int ch, tside* s, int from, int to, _Atomic uint64_t* in,
                        _Atomic uint64_t* out) {
  const orc_conn* c = t->c;
  if (s->j == s->k) {
    s->done = 1;
    return 1;
  }
  const uint64_t g = s->base + s->j;
  if (atomic_load_explicit(in, memory_order_acquire) <= g) return 0;
  memcpy(slot_in(c, to, ch, g), slot_in(c, from, ch, g), (size_t)chunk(c, s, s->j));
  atomic_store_explicit(out, g + 1, memory_order_release);
  s->j++;
  return 1;
}

/* ------------------------------------------------------------------ jobs */
typedef struct {
  const tconn* t;
  int ch, role; /* 0: producer, 1: consumer / receiver, 2: send proxy, 3: receive proxy */
  tside* s;
  const uint8_t* A;
  uint8_t* B;
} actor;

typedef struct {
  actor* actors;
  int nactors, nthreads;
  atomic_int err;
  atomic_ullong actions;
} job;

typedef struct {
  job* jb;
  int id;
} worker_arg;

static void* worker(void* p) {
  worker_arg* wa = (worker_arg*)p;
  job* jb = wa->jb;
  double idle_since = 0.0;
  unsigned long long seen = 0;
  for (;;) {
    if (atomic_load_explicit(&jb->err, memory_order_relaxed)) return NULL;
    int live = 0, moved = 0;
    for (int i = wa->id; i < jb->nactors; i += jb->nthreads) {
      actor* a = &jb->actors[i];
      if (a->s->done) continue;
      int r;
      switch (a->role) {
        case 0: r = prod_action(a->t, a->ch, a->s, a->A, a->B); break;
        case 1: r = cons_action(a->t, a->ch, a->s, a->B); break;
        case 2:
          r = proxy_action(a->t, a->ch, a->s, 0, 1, &a->t->tail[a->ch], &a->t->ytail[a->ch]);
          break;
        default:
          r = proxy_action(a->t, a->ch, a->s, 1, 2, &a->t->ytail[a->ch], &a->t->gtail[a->ch]);
          break;
      }
      if (r < 0) {
        int zero = 0;
        atomic_compare_exchange_strong(&jb->err, &zero, -r);
        return NULL;
      }
      if (r > 0) moved = 1;
      if (!a->s->done) live = 1;
    }
    if (!live) return NULL;
    if (moved) {
      atomic_fetch_add_explicit(&jb->actions, 1, memory_order_relaxed);
      idle_since = 0.0;
      continue;
    }
    unsigned long long now_actions = atomic_load_explicit(&jb->actions, memory_order_relaxed);
    if (idle_since == 0.0 || now_actions != seen) {
      idle_since = now_s();
      seen = now_actions;
    } else if (now_s() - idle_since > IDLE_LIMIT_S) {
      int zero = 0;
      atomic_compare_exchange_strong(&jb->err, &zero, ORC_V_DEADLOCK);
      return NULL;
    }
    sched_yield();
  }
}

static int run_job(job* jb) {
  pthread_t th[256];
  worker_arg wa[256];
  int started = 0;
  for (int i = 0; i < jb->nthreads; ++i) {
    wa[i].jb = jb;
    wa[i].id = i;
    if (pthread_create(&th[i], NULL, worker, &wa[i]) != 0) {
      int zero = 0;
      atomic_compare_exchange_strong(&jb->err, &zero, ORC_E_NOMEM);
      break;
    }
    ++started;
  }
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  return atomic_load(&jb->err);
}

static int end_state_ok(const tconn* t, const tside* prod, const tside* cons) {
  for (int ch = 0; ch < t->c->nch; ++ch) {
    uint64_t want = prod[ch].base + prod[ch].k;
    if (atomic_load(&t->head[ch]) != want || atomic_load(&t->tail[ch]) != want ||
        atomic_load(&t->ptrx[ch]) != 0 || cons[ch].j != cons[ch].k)
      return 0;
    if (t->c->proto == ORC_RELAY &&
        (atomic_load(&t->ytail[ch]) != want || atomic_load(&t->gtail[ch]) != want))
      return 0;
  }
  return 1;
}

static void commit(orc_conn* c, const tconn* t, const tside* prod) {
  for (int ch = 0; ch < c->nch; ++ch) {
    c->ctrl[ch].head = atomic_load(&t->head[ch]);
    c->ctrl[ch].tail = atomic_load(&t->tail[ch]);
    c->ctrl[ch].ptrx = atomic_load(&t->ptrx[ch]);
    c->ctrl[ch].ytail = atomic_load(&t->ytail[ch]);
    c->ctrl[ch].gtail = atomic_load(&t->gtail[ch]);
    c->ctrl[ch].base = prod[ch].base + prod[ch].k; /* Reading R8 */
  }
}

int orc_run_threaded(orc_conn* c, const uint8_t* A, uint8_t* B, uint64_t n, int nthreads) {
  if (!c || (n && (!A || !B)) || nthreads < 1) return ORC_E_ARG;
  /* the threads run the pages' program order; the LL group order is the enumerator's */
  if (c->proto == ORC_LL && c->order != ORC_ORDER_PAGES) return ORC_E_ARG;
  const int per_ch = c->proto == ORC_RELAY ? 4 : 2; /* actors per channel */
  if (nthreads > per_ch * c->nch) nthreads = per_ch * c->nch;
  uint64_t base[64];
  for (int ch = 0; ch < c->nch; ++ch) base[ch] = c->ctrl[ch].base;
  tside prod[64], cons[64], sprx[64], rprx[64];
  sides_begin(prod, c, base, n);
  sides_begin(cons, c, base, n);
  sides_begin(sprx, c, base, n);
  sides_begin(rprx, c, base, n);
  if (c->proto == ORC_LL)
    for (int ch = 0; ch < c->nch; ++ch)
      if (base[ch] + prod[ch].k > 0xFFFFFFFFull) return ORC_E_RANGE;
  tconn t;
  int rc = tconn_init(&t, c);
  actor actors[256];
  job jb;
  memset(&jb, 0, sizeof(jb));
  if (!rc) {
    for (int ch = 0; ch < c->nch; ++ch) {
      actors[per_ch * ch] = (actor){&t, ch, 0, &prod[ch], A, B};
      actors[per_ch * ch + 1] = (actor){&t, ch, 1, &cons[ch], A, B};
      if (per_ch == 4) {
        actors[per_ch * ch + 2] = (actor){&t, ch, 2, &sprx[ch], A, B};
        actors[per_ch * ch + 3] = (actor){&t, ch, 3, &rprx[ch], A, B};
      }
    }
    jb.actors = actors;
    jb.nactors = per_ch * c->nch;
    jb.nthreads = nthreads;
    atomic_init(&jb.err, 0);
    atomic_init(&jb.actions, 0);
    rc = run_job(&jb);
  }
  if (!rc && !end_state_ok(&t, prod, cons)) rc = ORC_V_COUNTERS;
  if (!rc && n && memcmp(A, B, (size_t)n) != 0) rc = ORC_V_RESULT;
  if (!rc) commit(c, &t, prod);
  tconn_free(&t);
  return rc;
}

/* ------------------------------------------------------------- ping-pong
 * Two endpoints on two threads (each pinned to its own core when the
 * process may use two): X sends a on fwd then receives c on rev; Y receives
 * b on fwd then sends b back on rev; iters round trips.  Each endpoint runs
 * its actors for one transfer until they finish before it starts the next. */
typedef struct {
  const tconn *fwd, *rev;
  const uint8_t* a;
  uint8_t *b, *cbuf;
  uint64_t n;
  int iters, x, cpu;
  atomic_int* err;
  uint64_t fwd_base[64], rev_base[64];
} pp_arg;

static void pin(int cpu) {
  if (cpu < 0) return;
  cpu_set_t set;
  CPU_ZERO(&set);
  CPU_SET(cpu, &set);
  pthread_setaffinity_np(pthread_self(), sizeof(set), &set);
}

/* Runs one side's actors of a transfer to completion; 0 or a violation. */
static int run_side(const tconn* t, int role, uint64_t* base, const uint8_t* A, uint8_t* B,
                    uint64_t n, atomic_int* err, int pinned) {
  const orc_conn* c = t->c;
  tside s[64];
  sides_begin(s, c, base, n);
  double idle_since = 0.0;
  for (;;) {
    int live = 0, moved = 0;
    for (int ch = 0; ch < c->nch; ++ch) {
      if (s[ch].done) continue;
      int r = role == 0 ? prod_action(t, ch, &s[ch], A, B) : cons_action(t, ch, &s[ch], B);
      if (r < 0) return -r;
      if (r > 0) moved = 1;
      if (!s[ch].done) live = 1;
    }
    if (!live) break;
    if (atomic_load_explicit(err, memory_order_relaxed)) return ORC_V_DEADLOCK;
    if (moved) {
      idle_since = 0.0;
      continue;
    }
    if (idle_since == 0.0) {
      idle_since = now_s();
    } else if (now_s() - idle_since > IDLE_LIMIT_S) {
      return ORC_V_DEADLOCK;
    }
    if (!pinned) sched_yield(); /* sharing a core with the other endpoint */
  }
  for (int ch = 0; ch < c->nch; ++ch) base[ch] += s[ch].k;
  return 0;
}

static void* pp_worker(void* p) {
  pp_arg* a = (pp_arg*)p;
  pin(a->cpu);
  for (int it = 0; it < a->iters; ++it) {
    int rc;
    if (a->x) {
      rc = run_side(a->fwd, 0, a->fwd_base, a->a, NULL, a->n, a->err, a->cpu >= 0);
      if (!rc) rc = run_side(a->rev, 1, a->rev_base, NULL, a->cbuf, a->n, a->err, a->cpu >= 0);
    } else {
      rc = run_side(a->fwd, 1, a->fwd_base, NULL, a->b, a->n, a->err, a->cpu >= 0);
      if (!rc) rc = run_side(a->rev, 0, a->rev_base, a->b, NULL, a->n, a->err, a->cpu >= 0);
    }
    if (rc) {
      int zero = 0;
      atomic_compare_exchange_strong(a->err, &zero, rc);
      return NULL;
    }
  }
  return NULL;
}

int orc_pingpong_threaded(orc_conn* fwd, orc_conn* rev, const uint8_t* a, uint8_t* b,
                          uint8_t* cbuf, uint64_t n, int iters, double* seconds) {
  if (!fwd || !rev || iters < 0 || fwd->nch != rev->nch || (n && (!a || !b || !cbuf)))
    return ORC_E_ARG;
  if (fwd->proto >= ORC_ZC || rev->proto >= ORC_ZC) return ORC_E_ARG; /* SIMPLE and LL only */
  tconn tf, tr;
  int rc = tconn_init(&tf, fwd);
  if (!rc) rc = tconn_init(&tr, rev);
  /* the first two CPUs this process may run on */
  int cpus[2] = {-1, -1}, found = 0;
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof(set), &set) == 0)
    for (int i = 0; i < CPU_SETSIZE && found < 2; ++i)
      if (CPU_ISSET(i, &set)) cpus[found++] = i;
  if (found < 2) cpus[0] = cpus[1] = -1;
  atomic_int err;
  atomic_init(&err, 0);
  pp_arg ax, ay;
  memset(&ax, 0, sizeof(ax));
  ax.fwd = &tf;
  ax.rev = &tr;
  ax.a = a;
  ax.b = b;
  ax.cbuf = cbuf;
  ax.n = n;
  ax.iters = iters;
  ax.err = &err;
  for (int ch = 0; ch < fwd->nch; ++ch) {
    ax.fwd_base[ch] = fwd->ctrl[ch].base;
    ax.rev_base[ch] = rev->ctrl[ch].base;
  }
  ay = ax;
  ax.x = 1;
  ax.cpu = cpus[0];
  ay.x = 0;
  ay.cpu = cpus[1];
  double t0 = now_s();
  if (!rc) {
    pthread_t tx, ty;
    if (pthread_create(&ty, NULL, pp_worker, &ay) != 0) {
      rc = ORC_E_NOMEM;
    } else {
      if (pthread_create(&tx, NULL, pp_worker, &ax) != 0) {
        atomic_store(&err, ORC_E_NOMEM);
      } else {
        pthread_join(tx, NULL);
      }
      pthread_join(ty, NULL);
      rc = atomic_load(&err);
    }
  }
  double t1 = now_s();
  if (seconds) *seconds = t1 - t0;
  if (!rc) {
    for (int ch = 0; ch < fwd->nch; ++ch) {
      /* Every side advanced its bases identically; X's view is the record. */
      fwd->ctrl[ch].head = atomic_load(&tf.head[ch]);
      fwd->ctrl[ch].tail = atomic_load(&tf.tail[ch]);
      fwd->ctrl[ch].ptrx = atomic_load(&tf.ptrx[ch]);
      fwd->ctrl[ch].base = ax.fwd_base[ch];
      rev->ctrl[ch].head = atomic_load(&tr.head[ch]);
      rev->ctrl[ch].tail = atomic_load(&tr.tail[ch]);
      rev->ctrl[ch].ptrx = atomic_load(&tr.ptrx[ch]);
      rev->ctrl[ch].base = ax.rev_base[ch];
      if (fwd->ctrl[ch].head != fwd->ctrl[ch].base || fwd->ctrl[ch].tail != fwd->ctrl[ch].base ||
          rev->ctrl[ch].head != rev->ctrl[ch].base || rev->ctrl[ch].tail != rev->ctrl[ch].base)
        rc = ORC_V_COUNTERS;
    }
  }
  tconn_free(&tf);
  tconn_free(&tr);
  return rc;
}
