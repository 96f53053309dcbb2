// Layout of the seed-derived table blob that tq_build_codebook writes and the
// kernels read.  Internal to libtq (shared by the host builder and the HIP
// kernels); callers treat the blob as opaque bytes.
#ifndef TQ_TABLES_H_
#define TQ_TABLES_H_

#include <stdint.h>

#define TQ_BLOB_MAGIC 0x31425154u /* "TQB1" little-endian */
#define TQ_BLOB_VERSION 1u
#define TQ_BLOB_ALIGN 256u
#define TQ_MAX_PARTS 2
#define TQ_MAX_HINT 512 /* bins of a bucketize hint grid (the 8-bit codebook needs 512, the others 16-256) */

// One "part" is a group of channels quantised with its own norm, rotation and
// codebook: the whole key for MSE/PROD, each half for GROUPED.
typedef struct {
  uint32_t magic;
  uint32_t version;
  uint32_t total_bytes;
  uint32_t header_bytes;
  int32_t d;           // full head dimension
  int32_t mode;        // tq_mode
  int32_t m;           // rows of S (PROD), else 0
  int32_t n_parts;     // 1 or 2
  int32_t part_d[TQ_MAX_PARTS];       // channels per part (power of two)
  int32_t part_bits[TQ_MAX_PARTS];    // index bits per part
  int32_t part_levels[TQ_MAX_PARTS];  // 2^bits
  // byte offsets from the start of the blob, each TQ_BLOB_ALIGN-aligned
  uint32_t off_centroids[TQ_MAX_PARTS];  // float[levels]
  uint32_t off_bounds[TQ_MAX_PARTS];     // float[levels + 1]: levels-1 boundaries, then +inf, +inf
  uint32_t off_sigma[TQ_MAX_PARTS];      // float[part_d], each +1 or -1
  uint32_t off_hint[TQ_MAX_PARTS];       // tq_hint[hint_n]
  int32_t hint_n[TQ_MAX_PARTS];          // bins of the bucketize hint grid
  float hint_lo[TQ_MAX_PARTS];           // grid origin
  float hint_scale[TQ_MAX_PARTS];        // bins per unit
  uint32_t off_S;                        // uint16 (fp16 bits) [m][d] row-major, PROD only
  uint32_t pad0;
  double mse[TQ_MAX_PARTS];              // Lloyd-Max distortion of N(0,1) per part
} tq_blob_header;

// Bucketize hint: for y falling in bin g = clamp(floor((y - lo) * scale)),
// idx = h + [y >= t_h] + [y >= t_h1], where h counts the boundaries that lie
// below the bin (minus a margin) and t_h, t_h1 are the next two boundaries.
// The builder checks that no third boundary can be passed within a bin.
typedef struct {
  float t_h;
  float t_h1;
  int32_t h;
  int32_t pad;
} tq_hint;

#endif  // TQ_TABLES_H_
