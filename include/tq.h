/*
 * tq.h -- C ABI of libtq, the MI355X (gfx950) TurboQuant KV-cache library.
 *
 * The method (as described on the "tqlite" README, the difai.kr tutorial
 * "实现 TurboQuant (第5部分)", the m.lqnn.cn bit-packing article and the
 * electron-rare/turboquant validation script):
 *   keys   -> L2 norm, random rotation Pi = Hadamard x random signs, snap each
 *             rotated coordinate to a Lloyd-Max Gaussian codebook, optionally a
 *             1-bit QJL sign sketch of the residual, bit-pack;
 *   values -> per-token group quantisation at 2 or 4 bits (fp16 scale, zero);
 *   decode -> estimate q.k straight from the packed bytes, softmax, weighted
 *             sum of the dequantised values.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE memory unless the argument is marked (host).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work on it; none synchronises or allocates device
 *     memory, and the library keeps no mutable global state apart from
 *     tq_decode_attention_noalloc's device array and its cached address
 *     (calls from several host threads are safe; calls that write the same
 *     buffers race exactly as the kernels they enqueue would).
 *   - The caller owns every buffer.
 *   - Arguments are validated on the host before anything is launched; a bad
 *     argument returns TQ_ERR_ARG / TQ_ERR_UNSUPPORTED and enqueues nothing.
 *     A failed launch returns TQ_ERR_HIP.  Faults inside kernels surface at
 *     the caller's next synchronisation, as for any HIP kernel.
 *   - No call aborts or throws.
 *
 * Packed layouts (the bit-packing article, sections 二, 三, "3 比特怎么办", 四):
 *   w-bit index / value fields: element j of a row goes to byte j*w/8 at bit
 *   (j mod 8/w)*w, first element in the lowest bits.  Index widths: 1-bit ->
 *   1, 2-bit -> 2, 3- and 4-bit -> 4 (3-bit stored as 4-bit), 5..8-bit -> 8.
 *   QJL sign i of a key goes to byte i/8 with weight 2^(i mod 8) (bit = 1 iff
 *   the projection is >= 0).  Norms, scales and zeros are IEEE fp16 (RNE).
 *   Records are structure-of-arrays planes, one row per record:
 *     idx   [n_records][tq_idx_row_bytes(cfg)]     uint8
 *     signs [n_records][d/8]                        uint8   (PROD, GROUPED_PROD)
 *     norm  [n_records]  fp16  (grouped modes: [n_records][2], outlier half first)
 *     rnorm [n_records]  fp16  residual norm ||k - k_mse_hat||   (PROD, GROUPED_PROD)
 *     codes [n_records][d*bits/8] uint8, scale/zero [n_records][d/group] fp16
 *   A 128-d prod key with 3 bits is 32 + 16 + 2 + 2 = 52 bytes, the record the
 *   bit-packing article (sec 四) counts.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_ARG = -1,          /* NULL / misaligned pointer, bad size or shape        */
  TQ_ERR_UNSUPPORTED = -2,  /* valid in principle, not implemented by this library */
  TQ_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required          */
  TQ_ERR_HIP = -4           /* a HIP runtime call failed (no device, launch error) */
} tq_status;

/* Quantisation modes: the "tqlite" README's mode table (三种量化模式). */
typedef enum {
  TQ_MODE_MSE = 0,      /* rotation + Lloyd-Max codebook, d*bits bits per key      */
  TQ_MODE_PROD = 1,     /* MSE at (bits-1) index bits + 1-bit QJL residual signs   */
  TQ_MODE_GROUPED = 2,  /* two halves, each its own norm, rotation and codebook    */
  TQ_MODE_GROUPED_PROD = 3  /* GROUPED, then 1-bit QJL signs of the whole key's
                               residual (m = d rows) and its fp16 norm           */
} tq_mode;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

typedef struct {
  int32_t d;            /* head dimension: power of two, 16 <= d <= 256; the
                           decode kernels support d = 128                          */
  int32_t mode;         /* tq_mode                                                  */
  int32_t bits;         /* MSE: index bits 1..8.  PROD: total bits 2..9, the index
                           takes bits-1 and the QJL sign 1 (the pages disagree on
                           this split; (b-1)+1 is the reading taken).  Ignored for
                           GROUPED and GROUPED_PROD (whose QJL sign comes on top
                           of the halves' index bits: the "tqlite" README's mode
                           table charges the QJL stage d + 32 bits on top of the
                           MSE stage's).                                           */
  int32_t bits_outlier; /* GROUPED(_PROD): index bits 1..8 of channels [0, d_outlier) */
  int32_t bits_normal;  /* GROUPED(_PROD): index bits 1..8 of the other channels      */
  int32_t d_outlier;    /* GROUPED(_PROD): channels in the outlier half; 0 or d/2,
                           both meaning d/2 (each half needs its own power-of-two
                           Walsh-Hadamard transform, and d/2 is the only split of
                           d into two powers of two).  The outlier channels are
                           moved to the front of keys and queries first
                           (tq_select_outlier_channels).  MSE / PROD: must be 0.   */
  uint64_t seed;        /* derives sigma and S; use one seed per layer ("tqlite"
                           README, 设计要点: independent seed per layer)            */
} tq_key_config;

/* Bytes of one index row (the idx plane's row pitch) for `cfg`; 0 if invalid. */
size_t tq_idx_row_bytes(const tq_key_config* cfg);

/*
 * tq_build_codebook -- (host) build every seed-derived constant of `cfg` into
 * one self-describing little-endian blob ("tables"):
 *   - the Lloyd-Max quantiser of N(0,1) with 2^b levels (one per half in
 *     GROUPED), centroids and boundaries rounded from float64 to float32; the
 *     "tqlite" README (Lloyd-Max 高斯码本) and the validation script's
 *     get_codebook(d, bits) / "mse_total" (test_mse_codebook_table1);
 *   - the random signs sigma of Pi = H diag(sigma) / sqrt(d) ("tqlite" README:
 *     rotation = Hadamard x random signs);
 *   - PROD, GROUPED_PROD: the QJL matrix S, d x d i.i.d. N(0,1) stored as
 *     fp16 (difai.kr tutorial, 算法概述: sign(S @ residual)).
 * sigma and S come from SplitMix64 (Steele, Lea & Flood 2014) seeded with
 * seed XOR tag*0x9E3779B97F4A7C15 (tags 1 sigma, 2 S, 3 outlier sigma,
 * 4 normal sigma), S through Box-Muller on 53-bit uniforms.
 *   blob_host       (host) output buffer, 256-byte aligned size *bytes; NULL to
 *                   query the size.
 *   bytes           (host) in: capacity of blob_host; out: bytes required.
 *   mse_total_host  (host, nullable) out: float64 expected total squared error
 *                   of a unit vector (Table 1's "mse_total"); two values for
 *                   GROUPED (outlier half, normal half), else one.
 * The blob is position independent: upload it to device memory unchanged and
 * pass the device copy as `tables` below.  Returns TQ_ERR_ARG if *bytes is too
 * small (and sets *bytes).  Takes well under a second on the host.
 */
tq_status tq_build_codebook(const tq_key_config* cfg, void* blob_host, size_t* bytes,
                            double* mse_total_host);

/*
 * tq_encode_keys -- quantise and pack n_vec keys.
 * Per key: n = ||k||; y = H (sigma * k / n) (the 128-point fast Walsh-Hadamard
 * transform, the "tqlite" README's 已知限制 asking for O(d log d)); each y_j
 * goes to the Lloyd-Max cell #{t : y_j >= t}; PROD also forms the residual
 * r = y - c[idx], the signs [S r >= 0] and rho = n ||r|| / sqrt(d).
 * GROUPED does the same per half (d/2-point transform, own norm n_j, sigma and
 * codebook); GROUPED_PROD then sketches the whole key's residual in the frame
 * of the two rotations, w = concat_j (n_j / sqrt(d/2)) r_j: signs [S w >= 0],
 * rho = ||w|| = ||k - k_grouped_hat||.
 * Norm range: the norm is formed with a power-of-two prescale where the plain
 * fp32 sum of squares would under- or overflow, so index and sign bytes are
 * exact for keys with 2^-126 <= ||k|| <= 2^120.  A stored fp16 norm (or rho)
 * saturates: above 65504 it is +inf, below 2^-25 it is 0 (the bytes are still
 * those of the unit vector k / ||k||); scale such keys before encoding when
 * they are to be decoded.
 *   tables     device copy of the tq_build_codebook blob for `cfg`.
 *   keys       [n_vec rows] x d elements of `dtype`, row i at keys + i*row_stride
 *              elements; 16-byte aligned, row_stride*elemsize a multiple of 16.
 *   slots      (nullable) int64 [n_vec]: record index that row i is written to;
 *              a slot outside [0, n_records) skips the row.  NULL: slot = i.
 *   n_records  rows of every output plane.
 *   idx, norm  always; signs, rnorm for PROD and GROUPED_PROD (NULL otherwise).
 * The kernel compares the tables' header (mode, d, index bits, rows of S) with
 * cfg and writes nothing for tables built for another configuration.
 * Output planes must be 16-byte aligned.  n_vec == 0 is a no-op.
 */
tq_status tq_encode_keys(const tq_key_config* cfg, const void* tables,
                         const void* keys, int32_t dtype, int64_t n_vec, int64_t row_stride,
                         const int64_t* slots, int64_t n_records,
                         uint8_t* idx, uint8_t* signs, uint16_t* norm, uint16_t* rnorm,
                         void* stream);

/*
 * tq_encode_keys_batched -- tq_encode_keys for up to 32 independent key sets
 * in one launch, e.g. the layers of a prefill, each quantised with its own
 * tables (the "tqlite" README: every layer draws its rotation from its own
 * seed).  All sets share cfg's mode and widths, dtype, n_vec, row_stride and
 * n_records; entry i names the tables, key rows, slots and output planes of
 * set i, with the meaning, layout and alignment rules of tq_encode_keys.  The
 * outputs equal n_batch calls of tq_encode_keys, bit for bit; a launch of
 * many small sets avoids paying a launch and a table staging per set.
 *   batch    (host) array of n_batch entries, 0 <= n_batch <= 32.
 * Errors: those of tq_encode_keys for any entry (nothing is launched then),
 * TQ_ERR_ARG for n_batch outside [0, 32] or a NULL batch.
 */
typedef struct {
  const void* tables;    /* device tables blob of this set (same mode and widths as cfg) */
  const void* keys;      /* [n_vec rows] of dtype, row_stride elements apart            */
  const int64_t* slots;  /* nullable, as in tq_encode_keys                              */
  uint8_t* idx;
  uint8_t* signs;        /* PROD / GROUPED_PROD, else NULL                              */
  uint16_t* norm;
  uint16_t* rnorm;       /* PROD / GROUPED_PROD, else NULL                              */
} tq_key_batch;

tq_status tq_encode_keys_batched(const tq_key_config* cfg, const tq_key_batch* batch, int32_t n_batch,
                                 int32_t dtype, int64_t n_vec, int64_t row_stride, int64_t n_records,
                                 void* stream);

/*
 * tq_encode_values -- per-token group quantisation of n_vec value rows
 * (bit-packing article sec 二: 2-bit values four per byte; sec 三: 4-bit two per
 * byte).  For each group of `group` consecutive channels: s = fp16((max-min) /
 * (2^bits - 1)), z = fp16(min), code = clamp(rint((v - z) / s), 0, 2^bits - 1)
 * computed in float32 with the fp16-rounded s and z (ties to even); s == 0
 * gives code 0.
 *   bits 2 or 4; group 32; d = 128.  Layout and slot rules as tq_encode_keys.
 */
tq_status tq_encode_values(int32_t bits, int32_t group, int32_t d,
                           const void* values, int32_t dtype, int64_t n_vec, int64_t row_stride,
                           const int64_t* slots, int64_t n_records,
                           uint8_t* codes, uint16_t* scale, uint16_t* zero, void* stream);

/*
 * tq_append_kv -- tq_encode_keys and tq_encode_values of the same n_vec tokens
 * in one launch (the append step of the compressed store: bit-packing article
 * sec 五, new tokens are encoded straight into the packed planes).  Key and
 * value blocks run side by side, so a short append costs one encoder's latency
 * instead of two.  The outputs equal those of the two calls, bit for bit.
 *   keys, values  [n_vec rows] x d elements of the same `dtype`, rows at
 *                 key_stride / value_stride elements (as in the two calls).
 *   slots         (nullable) shared by keys and values; n_records rows in
 *                 every plane.
 * Every other argument, the layouts and the errors are those of
 * tq_encode_keys (cfg, tables, idx, signs, norm, rnorm) and tq_encode_values
 * (v_bits, v_group, codes, scale, zero).  n_vec == 0 is a no-op.
 */
tq_status tq_append_kv(const tq_key_config* cfg, const void* tables, const void* keys,
                       const void* values, int32_t dtype, int64_t n_vec, int64_t key_stride,
                       int64_t value_stride, const int64_t* slots, int64_t n_records,
                       uint8_t* idx, uint8_t* signs, uint16_t* norm, uint16_t* rnorm,
                       int32_t v_bits, int32_t v_group, uint8_t* codes, uint16_t* scale,
                       uint16_t* zero, void* stream);

/*
 * tq_decode_attention -- one decode step of attention over the packed cache.
 * For query head h of sequence b (KV head h / (Hq/Hkv)), over tokens
 * t < ctx_len[b]:
 *   s_t = q . k_hat_t, estimated from the packed bytes as
 *         (n_t/d) <q', c[idx_t]> + rho_t sqrt(pi/2)/(d sqrt(d)) <S q', 2 bit_t - 1>
 *         with q' = H (sigma * q)  (difai.kr tutorial, 算法概述: <q,k_hat> +
 *         sqrt(pi/2) (S@q)^T sign_bits, with the ||r|| and 1/m that make it
 *         unbiased); MSE/GROUPED keep the first term (per half); GROUPED_PROD
 *         sums the halves' first terms and rho_t sqrt(pi/2)/(d sqrt(d/2))
 *         <S q'', 2 bit_t - 1> with q'' the two halves' transforms;
 *   p = softmax(sm_scale * s), out = sum_t p_t v_hat_t, v_hat = code*s + z.
 * The split-K scheme (partial max, sum and output per token chunk, merged in
 * a second kernel) keeps every result deterministic: no atomics.
 *   q          [B][Hq][d] of q_dtype, contiguous, 16-byte aligned.
 *   ctx_len    int32 [B]; each 0 <= ctx_len[b] <= max_ctx (values outside are
 *              clamped into that range on the device).  A sequence with
 *              ctx_len 0 gets out = 0 and lse = -inf.
 *   key planes [B][Hkv][max_ctx] records, as written by tq_encode_keys with
 *              slot = (b*Hkv + h)*max_ctx + t.
 *   value planes: same record indexing; v_bits 2 or 4, v_group 32.
 *   sm_scale   softmax scale (1/sqrt(d) for standard attention).
 *   out        [B][Hq][d] float32.
 *   lse        (nullable) [B][Hq] float32 natural-log sum of exp(sm_scale*s).
 *   scores     (nullable) [B][Hq][max_ctx] float32 raw s_t (entries with
 *              t >= ctx_len[b] are not written).
 *   workspace  device scratch; with workspace == NULL the call only stores the
 *              required size in *workspace_bytes (host) and returns TQ_OK.
 * Supported: d = 128; PROD with bits 2..9 (index 1..8 bits); MSE with bits
 * 1..8 (indices of 4 to 6 bits are scored with one lookup table per
 * coordinate instead of one per byte; indices of 7 and 8 bits, whose tables
 * would exceed LDS, directly as sum_j q'_j c[idx_j] in float32);
 * GROUPED with (outlier, normal) index bits (4, 2),
 * (3, 2), (2, 2) or (4, 1); GROUPED_PROD with (3, 2) or (4, 1) (the lookup
 * tables of (4, 2) plus signs exceed a workgroup's 160 KiB of LDS);
 * Hq % Hkv == 0.  Other shapes return
 * TQ_ERR_UNSUPPORTED.  (Encode supports every mode and width above.)
 */
tq_status tq_decode_attention(const tq_key_config* cfg, const void* tables,
                              const void* q, int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                              const int32_t* ctx_len, int32_t max_ctx,
                              const uint8_t* idx, const uint8_t* signs,
                              const uint16_t* norm, const uint16_t* rnorm,
                              int32_t v_bits, int32_t v_group,
                              const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                              float sm_scale, float* out, float* lse, float* scores,
                              void* workspace, size_t* workspace_bytes, void* stream);

/*
 * tq_decode_attention_append -- one decode step that first appends the step's
 * new token: for every sequence b with ctx_len[b] > 0 and every KV head h, the
 * key k_new[b][h] and value v_new[b][h] become token t = ctx_len[b] - 1 of the
 * cache (bit-packing article sec 五: the store appends each new token's packed
 * record), and the step attends over tokens 0 .. t as tq_decode_attention
 * does.  The key is encoded as tq_encode_keys encodes it ("tqlite" README
 * 设计要点; difai.kr tutorial 算法概述: norm, random signs and Walsh-Hadamard
 * rotation, Lloyd-Max index, for PROD the QJL signs of the residual and its
 * norm), the value as tq_encode_values does (per 32-channel group, fp16 scale
 * and zero); the records are stored at slot (b*Hkv + h)*max_ctx + t of the
 * planes, which are therefore writable here.  Within this call token t is
 * attended from its encoding: its score is computed in float32 from the
 * record (not through the lookup tables) and its value is the record's
 * dequantised value.  One launch does both, so the append costs no launch of
 * its own.
 *   k_new, v_new  [B][Hkv][d] of kv_dtype (TQ_F32, TQ_BF16, TQ_F16),
 *              contiguous, aligned to their element size; both non-NULL.
 *   other arguments as tq_decode_attention (same workspace size).
 * Supported: every key format tq_decode_attention supports except indices
 * of 7 or 8 bits, which return TQ_ERR_UNSUPPORTED (the appending encoder
 * keeps a codebook's boundaries one per lane of one wave, at most 64).  The
 * grouped modes encode each half with its own norm, transform and codebook,
 * and GROUPED_PROD sketches the halves' weighted residuals together, as
 * tq_encode_keys does.  Contiguous planes here, a paged pool with
 * tq_decode_attention_paged_append.
 * Records of the appended tokens may differ from tq_encode_keys' where a
 * rotated coordinate lies within float32 rounding of a codebook boundary or
 * a projection within rounding of zero (each side's float32 arithmetic
 * decides those ties); values are bit-identical.
 */
tq_status tq_decode_attention_append(const tq_key_config* cfg, const void* tables,
                                     const void* q, int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                     const int32_t* ctx_len, int32_t max_ctx,
                                     const void* k_new, const void* v_new, int32_t kv_dtype,
                                     uint8_t* idx, uint8_t* signs, uint16_t* norm, uint16_t* rnorm,
                                     int32_t v_bits, int32_t v_group,
                                     uint8_t* v_codes, uint16_t* v_scale, uint16_t* v_zero,
                                     float sm_scale, float* out, float* lse, float* scores,
                                     void* workspace, size_t* workspace_bytes, void* stream);

/*
 * tq_decode_attention_noalloc -- tq_decode_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results (bit for bit) and
 * errors as tq_decode_attention, without the workspace: the split-K partials
 * go to an 8 MiB device array owned by the library, one per GPU, held until
 * the process ends.  Its device address is looked up on the first call on
 * each device (with that device current); no call allocates or frees memory.
 * A shape whose partials (B * Hq * n_split * 130 floats, the size
 * tq_decode_attention's workspace query reports) exceed 8 MiB returns
 * TQ_ERR_WORKSPACE and enqueues nothing.  Every call on one GPU shares its
 * array: calls that overlap on one GPU (two streams, or host threads on one
 * device) race on it and must be serialised by the caller; calls on one
 * stream are ordered and safe.  Nothing in the array needs clearing between
 * calls (every partial a call reads, that call writes first).
 */
tq_status tq_decode_attention_noalloc(const tq_key_config* cfg, const void* tables,
                                      const void* q, int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                      const int32_t* ctx_len, int32_t max_ctx,
                                      const uint8_t* idx, const uint8_t* signs,
                                      const uint16_t* norm, const uint16_t* rnorm,
                                      int32_t v_bits, int32_t v_group,
                                      const uint8_t* v_codes, const uint16_t* v_scale, const uint16_t* v_zero,
                                      float sm_scale, float* out, float* lse, float* scores, void* stream);

/*
 * tq_decode_attention_paged -- tq_decode_attention over a paged cache: the
 * compressed store appends fixed-size chunks of tokens, each chunk a page of
 * the planes (bit-packing article sec 五: the store appends packed chunks).
 * Page p holds page_size consecutive tokens of every KV head: the record of
 * token t of (sequence b, KV head h) is
 *     (block_table[b][t / page_size] * Hkv + h) * page_size + t % page_size,
 * which is also the slot tq_encode_keys / tq_encode_values write it to.
 *   block_table         int32 [B][max_blocks_per_seq] device array; entries
 *                       for pages below ctx_len[b] name pages of the pool;
 *                       entries past them are never read.  An entry outside
 *                       [0, n_pages) is clamped into it on the device, so a
 *                       stale table reads wrong tokens but never outside the
 *                       planes.
 *   page_size           tokens per page, a positive multiple of 64.
 *   n_pages             pages in the pool: the planes hold n_pages * Hkv *
 *                       page_size records.
 *   scores              (nullable) [B][Hq][max_blocks_per_seq * page_size].
 * Every other argument, the workspace query and the errors are those of
 * tq_decode_attention with max_ctx = max_blocks_per_seq * page_size; a bad
 * page_size, max_blocks_per_seq or n_pages returns TQ_ERR_ARG.  Results equal those of
 * tq_decode_attention on the same tokens laid out contiguously, bit for bit.
 */
tq_status tq_decode_attention_paged(const tq_key_config* cfg, const void* tables,
                                    const void* q, int32_t q_dtype, int32_t B, int32_t Hq,
                                    int32_t Hkv, const int32_t* ctx_len,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    int32_t page_size, int32_t n_pages,
                                    const uint8_t* idx, const uint8_t* signs,
                                    const uint16_t* norm, const uint16_t* rnorm,
                                    int32_t v_bits, int32_t v_group,
                                    const uint8_t* v_codes, const uint16_t* v_scale,
                                    const uint16_t* v_zero,
                                    float sm_scale, float* out, float* lse, float* scores,
                                    void* workspace, size_t* workspace_bytes, void* stream);

/*
 * tq_decode_attention_paged_append -- tq_decode_attention_append over a paged
 * pool (bit-packing article sec 五: each new token's packed record goes into
 * the store's current chunk, and the kernels read the chunks in place): the
 * new token t = ctx_len[b] - 1 of (b, h) is encoded into record
 *     (block_table[b][t / page_size] * Hkv + h) * page_size + t % page_size
 * (the entry clamped into [0, n_pages) as every entry is) and attended in the
 * same launch.  The block table must already name the page of t (a new
 * page, when t opens one).  Arguments as tq_decode_attention_paged, plus
 * k_new, v_new and kv_dtype as tq_decode_attention_append; same support and
 * errors as those two.
 */
tq_status tq_decode_attention_paged_append(const tq_key_config* cfg, const void* tables, const void* q,
                                           int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                           const int32_t* ctx_len, const int32_t* block_table,
                                           int32_t max_blocks_per_seq, int32_t page_size, int32_t n_pages,
                                           const void* k_new, const void* v_new, int32_t kv_dtype,
                                           uint8_t* idx, uint8_t* signs, uint16_t* norm, uint16_t* rnorm,
                                           int32_t v_bits, int32_t v_group,
                                           uint8_t* v_codes, uint16_t* v_scale, uint16_t* v_zero,
                                           float sm_scale, float* out, float* lse, float* scores,
                                           void* workspace, size_t* workspace_bytes, void* stream);

/*
 * tq_dequantize_keys -- dense k_hat rows from packed key records: the
 * dequantise path of the "tqlite" README (fake quantisation, prefill) and of
 * validate_paper.py's prod quantiser:
 *   k_hat = (n / sqrt(d)) Pi^T c[idx]  (+ rho sqrt(pi/2) / m  Pi^T S^T (2 bit - 1), PROD)
 * (GROUPED: each half with its own norm, rotation and codebook, no QJL term;
 * GROUPED_PROD: those halves plus rho sqrt(pi/2) / m blockdiag(Pi_o, Pi_n)^T
 * S^T (2 bit - 1)).
 *   n_vec       output rows.
 *   slots       (nullable) int64 [n_vec]: record read for output row i (NULL:
 *               record i); a slot outside [0, n_records) gives a zero row.
 *   idx ..      the key planes of tq_encode_keys, n_records rows each.
 *   out         [n_vec] rows of d elements of out_dtype (TQ_F32 / TQ_BF16 /
 *               TQ_F16, rounded to nearest even), row i at out + i*out_stride
 *               elements; 16-byte aligned, out_stride*elemsize a multiple of 16.
 * Computed in float32.  n_vec == 0 is a no-op; d must be 128.
 */
tq_status tq_dequantize_keys(const tq_key_config* cfg, const void* tables, int64_t n_vec,
                             const int64_t* slots, int64_t n_records,
                             const uint8_t* idx, const uint8_t* signs, const uint16_t* norm,
                             const uint16_t* rnorm, void* out, int32_t out_dtype, int64_t out_stride,
                             void* stream);

/*
 * tq_dequantize_values -- v_hat = code * s + z (one float32 fma per element)
 * for n_vec rows of the value planes of tq_encode_values (bit-packing article
 * sec 二/三 for the code layout).  Slots, output layout and errors as
 * tq_dequantize_keys; bits 2 or 4, group 32, d 128.
 */
tq_status tq_dequantize_values(int32_t bits, int32_t group, int32_t d, int64_t n_vec,
                               const int64_t* slots, int64_t n_records,
                               const uint8_t* codes, const uint16_t* scale, const uint16_t* zero,
                               void* out, int32_t out_dtype, int64_t out_stride, void* stream);

/*
 * tq_channel_moments -- per-channel sums over n_vec rows of d = 128 channels:
 * out[0][c] = sum_r x[r][c], out[1][c] = sum_r x[r][c]^2 (float64), from which
 * the caller takes per-channel variances to pick GROUPED mode's outlier
 * channels (the "tqlite" README's mode table: higher-variance channels get the
 * higher bit width).  The channels chosen are then moved to the front of the
 * keys and of the queries alike, which leaves every q.k unchanged.
 *   x            n_vec rows of dtype, row r at x + r*row_stride elements.
 *   out          device float64 [2][128], 8-byte aligned.
 *   workspace    device scratch (8-byte aligned); NULL: *workspace_bytes
 *                receives the size and nothing runs.
 * Deterministic: partial sums over fixed row ranges, added in a fixed order.
 */
tq_status tq_channel_moments(const void* x, int32_t dtype, int64_t n_vec, int64_t row_stride, int32_t d,
                             double* out, void* workspace, size_t* workspace_bytes, void* stream);

/*
 * tq_select_outlier_channels -- the channel order of GROUPED(_PROD) mode from
 * n_vec key rows (the "tqlite" README's mode table: the high-variance channels
 * get the higher bit width).  Each channel's population variance
 * Q/n - (S/n)^2 is formed in float64 from the sums of tq_channel_moments; the
 * n_outlier largest are chosen (equal variances: the lower channel first).
 * perm[0 .. n_outlier) lists the chosen channels in increasing order, then
 * perm[n_outlier .. d) the others in increasing order.  Apply it to keys and
 * queries alike (k[:, perm], q[..., perm]); q.k is unchanged.  n_vec == 0
 * gives the identity.  The one-pass variance loses accuracy only for a
 * channel whose mean exceeds its spread by about 10^6.
 *   x, dtype, n_vec, row_stride, d   as tq_channel_moments (d = 128).
 *   n_outlier  0 <= n_outlier <= d (d/2 for GROUPED mode).
 *   perm       device int32 [d].
 *   workspace  device scratch (8-byte aligned); NULL: *workspace_bytes
 *              receives the size and nothing runs.
 * Deterministic (fixed reduction order).
 */
tq_status tq_select_outlier_channels(const void* x, int32_t dtype, int64_t n_vec, int64_t row_stride,
                                     int32_t d, int32_t n_outlier, int32_t* perm, void* workspace,
                                     size_t* workspace_bytes, void* stream);

/*
 * tq_stream_read -- the measurement reference for the decode's roofline (not
 * part of the method): one pass over `bytes` of device memory with 16-byte
 * nontemporal loads, the way the decode streams the packed cache.  Timing it
 * gives the read bandwidth the GPU actually sustains, next to the
 * specification's peak.
 *   src     device buffer, 16-byte aligned; bytes > 0, a multiple of 16.
 *   sink    device uint32 [TQ_STREAM_READ_SINK]: one xor of the words each
 *           thread read (keeps the loads; no other meaning), overwritten.
 * Errors: TQ_ERR_ARG for a null or misaligned pointer or a bad size; launch
 * failures as TQ_ERR_HIP.
 */
#define TQ_STREAM_READ_SINK 65536
tq_status tq_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Static description of a status code (never NULL). */
const char* tq_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
