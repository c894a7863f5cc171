/*
 * oracle_internal.h -- connection state shared by the oracle's sequential
 * simulator (oracle.c) and its threaded mode (threaded.c).
 *
 * TEST INFRASTRUCTURE ONLY, like the rest of oracle/.
 */
#ifndef RFP_ORACLE_INTERNAL_H
#define RFP_ORACLE_INTERNAL_H

#include <stdint.h>

/* Per-channel control words and the persistent step base (Readings R1, R8);
 * ytail and gtail are the RELAY proxies' tails (send proxy, receive proxy). */
typedef struct {
  uint64_t head, tail, ptrx, base;
  uint64_t ytail, gtail;
} orc_ctrl;

struct orc_conn {
  int proto, nch, nslots, mutation, order;
  uint64_t slot_bytes, step_bytes;
  uint8_t* fifo; /* nch * nslots * slot_bytes per FIFO, zero at creation; none for zero-copy,
                    three (send | staging | receive) for RELAY */
  orc_ctrl* ctrl;
};

#endif
