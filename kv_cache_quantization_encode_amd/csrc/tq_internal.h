// Internal declarations shared by the host code and the launchers of libtq.
#ifndef TQ_INTERNAL_H_
#define TQ_INTERNAL_H_

#include <stddef.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

// Channel parts of a key configuration (see tq_tables.h).
struct Parts {
  int d;
  int mode;
  int m;                // rows of S (PROD)
  int n_parts;          // 1, or 2 for GROUPED
  int part_d[2];
  int part_bits[2];     // index bits
  int part_width[2];    // storage width of one index (1, 2, 4 or 8 bits)
  int part_row_off[2];  // byte offset of the part inside an index row
  int idx_row_bytes;
};

int index_width(int bits);
tq_status describe(const tq_key_config* cfg, Parts* p);

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Compute units of the current device (cached per device); -1 on error.
int cu_count();

}  // namespace tq

#endif  // TQ_INTERNAL_H_
