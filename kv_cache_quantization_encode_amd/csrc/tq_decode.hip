// Split-K decode attention over the packed TurboQuant cache, for gfx950.
//
// What is computed (difai.kr tutorial, 算法概述, with the ||r|| and 1/m that
// make the QJL term unbiased; "tqlite" README mode table; bit-packing article
// sec 五: the fused kernels read the packed bytes directly and unpack with
// shifts and masks):
//   s_t = (n_t / d) <q', c[idx_t]> + rho_t sqrt(pi/2) / (m sqrt(d)) <S q', 2 bit_t - 1>
//   (GROUPED: (n0/64) <q'_0, c0[idx]> + (n1/64) <q'_1, c1[idx]> over the halves)
//   p = softmax(sm_scale s), out = sum_t p_t (code_t * scale_t + zero_t).
//
// One workgroup (16 waves) takes one (sequence, KV head, quad of query heads,
// token chunk).  Its prologue rotates the four queries (q' = H sigma q by
// shuffle butterflies in registers), projects them (S q', on MFMA: the QJL
// matrix product is the one dense contraction of the method) and turns them
// into lookup tables: for every byte position p of a packed key and every byte
// value v, the four heads' partial inner products over the coordinates that
// byte holds.  An entry is an integer in [0, 16383] in units of a per-head
// step, offset by the smallest value of its position (both derived from |q'|
// and the codebook's end points), four heads packed in 64 bits.  A key's
// score is then one table read per packed byte (48 for a 3-bit prod key):
// four reads are added with one 64-bit add each (the 16-bit fields cannot
// carry into each other) and then folded into 32-bit sums per head with
// v_dot2_u32_u16, so the sums are exact integers.
// Half of the waves score 64-token tiles (lane = token) and run the online
// softmax; the other half accumulate p.V for those tiles one round later on
// MFMA (v_mfma_f32_16x16x32_f16: A = the weights, rows value group x head;
// B = the codes, one column per channel), with the 2- or 4-bit code fields
// left in place as fp16 subnormal bit patterns (a byte's fields up to field
// f, masked: prefix value * 2^-24), so no conversion is spent per code and
// per-channel sums are differences of consecutive prefix sums at the end.
// The value scale is folded into the weight (p * scale, as fp16) and the
// zero point is summed separately (sum_t p_t zero_t, fp32).  Softmax weights are carried as p * 2^14 and the
// scales of each tile are renormalised by a power of two, so weights keep the
// fp16 normal range whatever the values' magnitude.  The chunk's (max, sum,
// unnormalised output) goes to the workspace; a second kernel merges chunks
// in a fixed order.
// Appending (tq_decode_attention_append): the workgroup whose chunk ends with
// the step's new token encodes that token's key and value in its prologue,
// stores the record, and adds the token to its combine with a float32 score
// computed from the record; the loop covers the chunk without it.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <atomic>
#include <type_traits>

#include "tq.h"
#include "tq_internal.h"
#include "tq_tables.h"

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int KD = 128;
#ifndef TQ_DEC_WAVES
#define TQ_DEC_WAVES 16
#endif
constexpr int NW = TQ_DEC_WAVES;  // waves per workgroup
constexpr int NT = NW * 64;       // threads per workgroup
constexpr int NS = NW / 2;        // score waves (and p.V waves)
constexpr int PAGE_CACHE = 512;   // block-table entries a workgroup keeps in LDS
constexpr int TILE = 64;          // tokens per wave tile
// Record of an appended token in LDS (dwords): index row, QJL sign row, fp16
// norm, fp16 residual norm, four fp16 zeros, four fp16 scales, value codes.
constexpr int NR_IDX = 0, NR_SIGN = 32, NR_NORM = 36, NR_RNORM = 37, NR_Z = 38, NR_S = 40, NR_CODE = 48;
constexpr int NREC = 64;
constexpr int KENC_WAVE = 8, VENC_WAVE = 9;  // waves that encode an appended key / value (idle then)
constexpr int QH = 4;             // query heads per workgroup
static_assert(KENC_WAVE >= 8 && VENC_WAVE >= 8 && KENC_WAVE + QH <= NW && VENC_WAVE < NW,
              "the encoding waves are neither the S q' MFMA waves nor past the workgroup");
// A wave's weight slot holds the MFMA A operand of its tile's p.V: rows
// m = 4 group + head, 64 tokens, fp16, as [chunk][token group kq][m][j] with
// token 32 chunk + 4 j + kq; each (chunk, kq) block is padded by 16 halves so
// that the score lanes' 2-byte stores spread over the LDS banks.
constexpr int ABLK = 16 * 8 + 16;   // halves per (chunk, kq) block
constexpr int WSLOT = 8 * ABLK / 2; // dwords of a wave's weight slot
constexpr int PART = KD + 2;      // floats per partial: max, sum, out[128]
constexpr float LOG2E = 1.4426950408889634f;
// Table reads are summed in 16-bit fields, CHAIN at a time, before a flush
// into 32-bit sums: entries round into [0, EMAX + 1] so that CHAIN of them
// fit.  Formats with per-coordinate tables (128 reads per key, each rounded)
// take chains of two and twice the resolution.
template <bool COORD> constexpr int chain_len() { return COORD ? 2 : 4; }
template <bool COORD> constexpr float entry_max() { return COORD ? 32766.0f : 16382.0f; }
constexpr float PSCALE = 14.0f;   // softmax weights are carried as p * 2^14
constexpr float SQRT_HALF_PI = 1.2533141373155003f;

constexpr int width_of(int b) { return b == 1 ? 1 : b == 2 ? 2 : b <= 4 ? 4 : 8; }
constexpr int stride_of(int b) { return b == 3 ? 128 : 256; }  // 3-bit in nibbles: bytes <= 0x77
constexpr int CEN = 64;  // centroids staged per part (index widths up to 6 bits)

// Table classes of a key format, in key-byte order: the index bytes of part 0,
// (GROUPED, GROUPED_PROD) the index bytes of part 1, (PROD, GROUPED_PROD) the
// QJL sign bytes.  Indices of 4 to 6 bits (one part) use one table per
// coordinate instead of one per byte (kind 3): a byte table of 4-bit fields
// would have 256 entries for each of 64 bytes (128 KiB), and a 5- or 6-bit
// index fills a byte alone, so its table has 2^b entries.  Indices of 7 and 8
// bits (kind 4) would need 128 such tables of 128 or 256 entries, more than
// LDS holds: they are scored directly, sum_j q'_j c[idx_j] in float32 with the
// codebook in LDS, and have no table positions.
template <int MODE, int B0, int B1>
struct Fmt {
  static constexpr bool GROUPED = MODE == TQ_MODE_GROUPED || MODE == TQ_MODE_GROUPED_PROD;
  static constexpr bool QJL = MODE == TQ_MODE_PROD || MODE == TQ_MODE_GROUPED_PROD;
  static constexpr bool DIRECT = !GROUPED && B0 >= 7;  // index scored directly (no tables)
  static constexpr bool COORD = !GROUPED && B0 >= 4 && !DIRECT;  // per-coordinate tables for the index
  static constexpr int NPART = GROUPED ? 2 : 1;
  static constexpr int PD = KD / NPART;  // coordinates per part
  static constexpr int W0 = width_of(B0);
  static constexpr int W1 = GROUPED ? width_of(B1) : 1;
  static constexpr int IP0 = PD * W0 / 8;
  static constexpr int IP1 = GROUPED ? PD * W1 / 8 : 0;
  static constexpr int SP = QJL ? KD / 8 : 0;
  static constexpr int IDXB = IP0 + IP1;                 // idx row bytes
  static constexpr int KWORDS = (IDXB + SP) / 4;         // idx + sign words per key
  static constexpr int NC = NPART + (QJL ? 1 : 0);       // table classes
  // kind of class c: 0 / 1 index bytes of part 0 / 1, 2 sign bytes, 3 index
  // coordinates of part 0 (one table per coordinate), 4 index coordinates of
  // part 0 scored directly (no table)
  static constexpr int kind(int c) {
    return c == 0 ? (DIRECT ? 4 : COORD ? 3 : 0) : c == 2 ? 2 : (GROUPED ? 1 : 2);
  }
  // positions (tables) of class c and the key bytes it spans
  static constexpr int npos(int c) {
    return kind(c) == 4 ? 0 : kind(c) == 3 ? PD : kind(c) == 0 ? IP0 : kind(c) == 1 ? IP1 : SP;
  }
  static constexpr int nbytes(int c) { return kind(c) >= 3 ? IP0 : npos(c); }
  static constexpr int stride(int c) {
    return kind(c) == 4 ? 1 : kind(c) == 3 ? (1 << B0) : kind(c) == 0 ? stride_of(B0) : kind(c) == 1 ? stride_of(B1) : 256;
  }
  static constexpr int kbyte(int c) { return c == 0 ? 0 : kbyte(c - 1) + nbytes(c - 1); }  // first key byte
  static constexpr int pos0(int c) { return c == 0 ? 0 : pos0(c - 1) + npos(c - 1); }     // first position
  static constexpr int ent(int c) { return c == 0 ? 0 : ent(c - 1) + npos(c - 1) * stride(c - 1); }  // first entry
  static constexpr int cls(int pos) { return pos < pos0(1) || NC == 1 ? 0 : (NC == 2 || pos < pos0(2)) ? 1 : 2; }
  // table-read chains (CHAIN positions each), class by class
  static constexpr int CHAIN = chain_len<COORD>();
  static constexpr float EMAX = entry_max<COORD>();
  static constexpr int chain0(int c) { return pos0(c) / CHAIN; }
  static constexpr int chain_cls(int g) { return cls(g * CHAIN); }
  // coordinates one position of the index class of part p covers (table range)
  static constexpr int cpb(int p) { return COORD ? 1 : 8 / (p ? W1 : W0); }
  static constexpr int ENTRIES = ent(NC - 1) + npos(NC - 1) * stride(NC - 1);
  // the table region also holds the workgroup's end sums (NS x QH x (6 + KD) floats)
  static constexpr int LUT_ENTRIES = ENTRIES > 2176 ? ENTRIES : 2176;
  static constexpr int POSITIONS = pos0(NC - 1) + npos(NC - 1);
  static constexpr int HPOS0 = COORD ? PD : 0;  // first position built from nibble halves
  static_assert(IP0 % CHAIN == 0 && IP1 % CHAIN == 0 && SP % CHAIN == 0, "whole chains per class");
  // the weight ring also holds the half tables while the lookup tables are built
  static constexpr int RING_BYTES_W = NW * WSLOT * 4;
  static constexpr int HALF_BYTES = (POSITIONS - HPOS0) * 32 * 16;
  static constexpr int RING_BYTES = RING_BYTES_W > HALF_BYTES ? RING_BYTES_W : HALF_BYTES;
};

// 16-byte aligned, so that the compiler can read and write the float4 /
// 16-byte fields below (the MFMA operands in the ring, per-head factors,
// staged queries) with single ds_read_b128 / ds_write_b128 instructions; at
// the 8-byte alignment of its uint64 tables it splits them into pairs.
template <int MODE, int B0, int B1, int VB>
struct alignas(16) Lds {
  using F = Fmt<MODE, B0, B1>;
  uint64_t lut[F::LUT_ENTRIES];
  float qp[(QH + 1) * KD];  // rotated queries, then (appending) the new key's residual
  float qs[QH * KD];
  uint32_t nrec[NREC];     // appending: the new token's record (see NR_*)
  unsigned char nb8[2 * KD];  // appending: its index and value-code fields, one per byte
  float vhat[KD];          // appending: its dequantised value
  float xnew[QH];          // appending: its score per head (log2 softmax units)
  uint32_t ring[F::RING_BYTES / 4];
  float cen[2 * CEN];
  float rng[3][QH];    // largest byte range of each class and head (float bits, atomicMax)
  float offi[2][QH];   // index classes: sum over coordinates of the smallest term
  float sgp[8][QH];    // sign class: sum of |S q'| over each 16-row tile
  float uu[3][QH];     // per class and head: score step and offset, in log2 softmax units
  float oo[3][QH];
  float abuf[2 * (NW / 2) * QH];
  int ksf[NW / 2];     // final value-scale exponent of each score wave
  int prod[NW / 2];    // rounds the score wave of each pair has published
  int cons[NW / 2];    // rounds the p.V wave of each pair has finished
  int pages[PAGE_CACHE];  // block-table entries of this workgroup's token range (paged cache)
  // last, so that the fields above keep their offsets in every format
  alignas(16) float qT[F::DIRECT ? KD * QH : 4];  // DIRECT: rotated queries as [coordinate][head]
  float c8[F::DIRECT ? 1 << B0 : 4];              // DIRECT: the codebook
};

struct DecArgs {
  const unsigned char* tables;
  const void* q;
  int q_dtype;
  int B, Hq, Hkv, G, n_quads;
  const int* ctx_len;
  int max_ctx;
  const uint8_t* idx;
  const uint8_t* signs;
  const uint16_t* norm;
  const uint16_t* rnorm;
  const uint8_t* vcodes;
  const uint16_t* vscale;
  const uint16_t* vzero;
  float sm_scale;
  float* scores;
  float* part;
  int n_split;
  int chunk;  // tokens per split (multiple of TILE)
  // paged cache (NULL block_table: records of (b, h) are contiguous)
  const int* block_table;  // [B][max_blocks] physical page of each logical page
  int max_blocks;
  int page_size;  // tokens per page, a multiple of TILE
  int n_pages;    // pages in the pool (block-table entries are clamped below it)
  // appending (knew != NULL): token ctx_len[b] - 1 of every (b, KV head) is
  // encoded from knew / vnew ([B][Hkv][KD], kv_dtype) inside this launch,
  // attended from the encoding and stored into the planes below
  const void* knew;
  const void* vnew;
  int kv_dtype;
  uint8_t* w_idx;
  uint8_t* w_signs;
  uint16_t* w_norm;
  uint16_t* w_rnorm;
  uint8_t* w_vcodes;
  uint16_t* w_vscale;
  uint16_t* w_vzero;
};

// a query element as loaded: f32 bits, or bf16 / fp16 bits in the low half
__device__ inline float q_word_to_float(uint32_t w, int dt) {
  if (dt == TQ_F32) return __uint_as_float(w);
  if (dt == TQ_BF16) return __uint_as_float(w << 16);
  return __half2float(__ushort_as_half((unsigned short)w));
}

__device__ inline float h2f(uint32_t bits16) { return __half2float(__ushort_as_half((unsigned short)bits16)); }

// Entry of the table at byte offset BASE indexed by byte k of w.  Under
// 64 KiB the index times 8 is a single SDWA shift and BASE folds into the
// ds_read immediate; past it, a field extract and a shift-add.
// (BASE and k are constants once the caller's loop is unrolled.)
__device__ __forceinline__ uint64_t lut_read(const unsigned char* smem, uint32_t BASE, uint32_t w, int k) {
  uint32_t off;
  if (BASE + 2048u <= 65536u) {
    switch (k) {
      case 0: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(off) : "v"(w)); break;
      case 1: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(off) : "v"(w)); break;
      case 2: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(off) : "v"(w)); break;
      default: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(off) : "v"(w)); break;
    }
    return *(const uint64_t*)(smem + off + BASE);
  } else {
    // (the empty asm keeps the byte extract whole, so that shift and add
    // become one v_lshl_or / v_lshl_add)
    uint32_t b = __builtin_amdgcn_ubfe(w, 8 * k, 8);
    asm("" : "+v"(b));
    off = (b << 3) + BASE;
    return *(const uint64_t*)(smem + off);
  }
}

// Entry of the table at byte offset BASE indexed by nibble k of w (a field
// extract and a shift-add).
__device__ __forceinline__ uint64_t lut_read_nib(const unsigned char* smem, uint32_t BASE, uint32_t w, int k) {
  uint32_t b = __builtin_amdgcn_ubfe(w, 4 * k, 4);
  asm("" : "+v"(b));
  return *(const uint64_t*)(smem + (b << 3) + BASE);
}

template <int I, int N, typename Fn>
__device__ inline void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<I + 1, N>(fn);
  }
}

// DPP lane moves (gfx9 encodings): quad permutations, half-row and row mirrors.
template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;

// Sum over each aligned group of N (1, 2, 4 or 8) lanes, in all N.
template <int N>
__device__ inline float group_sum(float v) {
  if constexpr (N >= 2) v += dpp<DPP_XOR1>(v);
  if constexpr (N >= 4) v += dpp<DPP_XOR2>(v);
  if constexpr (N >= 8) v += dpp<DPP_HALF_MIRROR>(v);
  return v;
}

// The value of lane l ^ ST, without LDS traffic: quad permutes (1, 2), row
// rotations by 4 and 12 written into alternate banks of four lanes (4), a
// row rotation by 8 (8), permlane swaps (16, 32; the swap's two outputs hold
// the upper and the lower lane of each pair).
template <int ST>
__device__ inline float lane_xor(float v, int lane) {
  if constexpr (ST == 1) return dpp<DPP_XOR1>(v);
  if constexpr (ST == 2) return dpp<DPP_XOR2>(v);
  if constexpr (ST == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x12C, 0xF, 0x5, false);  // banks 0, 2: lane + 4
    return __int_as_float(__builtin_amdgcn_update_dpp(up, __float_as_int(v), 0x124, 0xF, 0xA, false));  // 1, 3: lane - 4
  }
  if constexpr (ST == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  if constexpr (ST == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? p[0] : p[1]);
  }
  if constexpr (ST == 32) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? p[0] : p[1]);
  }
  return v;
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS accesses
// only, so global loads already in flight (the next tile) stay in flight.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Pairwise hand-over through LDS counters: a release publishes this wave's
// LDS writes (LDS only, so global loads in flight stay in flight); a wait
// spins until the partner's counter reaches v.  Every wait of the protocol
// ends (the partner only ever waits on rounds already finished); the spin is
// also capped, so that a wait can never outlive the kernel.
__device__ inline void pair_publish(int* c, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ inline void pair_wait(int* c, int v) {
  for (int spin = 0; spin < (1 << 22); ++spin) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= v) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A value every lane holds alike, moved to a scalar register.
__device__ inline float uniform(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }

// x[l] + x[l ^ 16] and x[l] + x[l ^ 32] in every lane: a permlane swap of a
// value with itself hands each lane pair both values, one in each output.
__device__ inline float sum_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ inline float sum_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ inline float max_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Over the whole wave, in every lane: within rows of 16 by DPP, across rows
// by permlane swaps (no LDS traffic).
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  return max_xor32(max_xor16(v));
}

__device__ inline float wave_sum(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  v += dpp<DPP_ROW_MIRROR>(v);
  return sum_xor32(sum_xor16(v));
}

// Largest of a non-negative integer over the wave (row reductions by DPP,
// then the four rows through readlane).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_XOR1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_XOR2, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_HALF_MIRROR, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, DPP_ROW_MIRROR, 0xF, 0xF, true));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

template <int MODE, int B0, int B1, int VB>
__global__ __launch_bounds__(NT) void decode_kernel(DecArgs a) {
  using F = Fmt<MODE, B0, B1>;
  // Static LDS (its offsets are known to the compiler, so table offsets fold
  // into the ds_read immediates).
  __shared__ Lds<MODE, B0, B1, VB> L;
  unsigned char* smem = (unsigned char*)&L;
  uint64_t* lut = L.lut;    // tables: per class [position][value], four 16-bit heads
  float* qp = L.qp;         // [QH][KD] rotated queries
  float* qs = L.qs;         // [QH][KD] S q' (PROD)
  uint32_t* wbuf = L.ring;  // [2][NW/2][4 groups][32 pairs][QH] half2 weights (groups padded)
  float* cen = L.cen;       // [2][CEN] centroids of each part
  float* abuf = L.abuf;     // [2][NW/2][QH] p.V rescale factors

  const tq_blob_header* H = (const tq_blob_header*)a.tables;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it are scalar
  const int split = blockIdx.x, quad = blockIdx.y, bh = blockIdx.z;
  const int b = bh / a.Hkv, hkv = bh % a.Hkv;

  // Tables built for another format than this kernel's: nothing is read past
  // the header; the workgroup's partials become NaN (and so the outputs).
  const bool tables_ok = H->magic == TQ_BLOB_MAGIC && H->d == KD && H->mode == MODE && H->part_bits[0] == B0 &&
                         (!F::GROUPED || H->part_bits[1] == B1) && (!F::QJL || H->m == KD);
  if (!tables_ok) {
    for (int i = tid; i < QH * PART; i += NT) {
      const int gq = QH * quad + i / PART;
      if (gq < a.G)
        a.part[(((long long)b * a.Hq + hkv * a.G + gq) * a.n_split + split) * PART + i % PART] = __builtin_nanf("");
    }
    return;
  }
  // lengths outside [0, max_ctx] are clamped into it: no read leaves the sequence's records
  const int ctx = min(max(a.ctx_len[b], 0), a.max_ctx);
  const int t_begin = split * a.chunk;
  // Appending (knew set): token tn = ctx - 1, the last of its split's range,
  // is encoded in this launch.  The loop covers the range without it; it
  // enters the workgroup's final combine as one more softmax term.
  const int tn = a.knew && ctx > 0 ? ctx - 1 : -1;
  const bool has_new = tn >= t_begin && tn < min(ctx, t_begin + a.chunk);
  const int t_end = has_new ? tn : min(ctx, t_begin + a.chunk);

  const long long rec0 = ((long long)b * a.Hkv + hkv) * a.max_ctx;
  // ---- main loop, split between two kinds of waves.  Score waves (the first
  // half) read key bytes, look up the tables, run the online softmax and
  // publish fp16 weights p*scale; p.V waves (second half) accumulate those
  // weights against the value codes one round later.  Wave pw of each half
  // owns tiles pw, pw + NS, pw + 2 NS, ...; a two-slot LDS ring carries the
  // weights and the rescale factor from score wave pw to p.V wave pw, and a
  // pair of LDS counters orders producer and consumer.  No barrier holds the
  // pairs in step, so the score waves' table-lookup phases drift apart and
  // share the LDS instead of all contending for it at once.  Each wave loads
  // its next tile's data one round ahead.
  constexpr int VROW = KD * VB / 8;  // bytes of a value-code row
  const bool scorer = wave < NS;
  const int pw = scorer ? wave : wave - NS;
  // p.V lanes: lane = (column n = lane & 15, token group kq = lane >> 4) of
  // the MFMA B operand.  Column n of block beta (0..7) is channel 8 n + beta,
  // so a lane needs the same 8 channels (two bytes of 2-bit codes, four of
  // 4-bit ones) of each of its 16 tokens 32 chunk + 4 j + kq (j = 0..7).  It
  // loads the aligned dword holding them (2-bit: lanes 2i and 2i + 1 load the
  // same one, each picks its half): one load instruction of the wave covers
  // four consecutive rows.
  constexpr int NCODE = 16;  // code dwords of a lane per tile: [chunk][j]
  const int pn = lane & 15, kq = lane >> 4;
  const int cbyte = VB == 2 ? 4 * (pn >> 1) : 4 * pn;  // dword of the lane's channels in a row
  const uint32_t cb0 = VB == 2 ? 2 * (pn & 1) : 0;     // their first byte in that dword
  const int n_tiles = t_end > t_begin ? (t_end - t_begin + TILE - 1) / TILE : 0;
  const int rounds = (n_tiles + NS - 1) / NS;
  auto tile_tb = [&](int r) { return t_begin + (r * NS + pw) * TILE; };

  struct KeyData {
    uint32_t kw[F::KWORDS];
    uint32_t nrm, rn;  // fp16 norm(s), fp16 residual norm
    uint2 zv, sv;      // fp16 zero / scale of the four value groups
  };
  // Token indices are clamped into [t_begin, max(t_end - 1, t_begin)], a
  // range inside this (sequence, head)'s rows, so loads need no branches;
  // lanes past t_end get score -inf and weight 0.
  const int t_last = t_end - 1 > t_begin ? t_end - 1 : t_begin;
  // Record of token t of the tile starting at tb is tile_base(tb) + t: rec0
  // for a contiguous cache; for a paged one, through the block table entry of
  // the tile's page (a tile never straddles pages; tiles past the end use the
  // page of t_last, where their clamped tokens are).  Entries are clamped
  // into the pool, so a stale block table cannot send a read outside it.
  // The workgroup's block-table entries are staged in LDS by the prologue (a
  // global read here would wait behind the tile loads already in flight);
  // the host sizes the splits so that they fit in PAGE_CACHE entries.
  // (an appended token tn, outside the loop's range, may open a page of its own: staged too)
  const int t_stage = has_new ? tn : t_last;
  const int lp0 = a.block_table ? t_begin / a.page_size : 0;
  const int n_pages_wg = a.block_table && (t_end > t_begin || has_new)
                             ? min(t_stage / a.page_size - lp0 + 1, PAGE_CACHE) : 0;
  auto tile_base = [&](int tb) -> long long {
    if (!a.block_table) return rec0;
    const int tc = min(tb, t_last);
    const int lp = tc / a.page_size;
    return ((long long)L.pages[lp - lp0] * a.Hkv + hkv) * a.page_size - (long long)lp * a.page_size;
  };
  auto load_keys = [&](int tb, KeyData& d) {
    const int t = tb + TILE <= t_end ? tb + lane : min(tb + lane, t_last);
    const long long rec = tile_base(tb) + t;
    const uint32_t* ip = (const uint32_t*)(a.idx + rec * F::IDXB);
#pragma unroll
    for (int k = 0; k < F::IDXB / 4; ++k) d.kw[k] = ip[k];
    if constexpr (F::QJL) {
      const uint4 sv = *(const uint4*)(a.signs + rec * (KD / 8));
      d.kw[F::IDXB / 4 + 0] = sv.x; d.kw[F::IDXB / 4 + 1] = sv.y;
      d.kw[F::IDXB / 4 + 2] = sv.z; d.kw[F::IDXB / 4 + 3] = sv.w;
      d.rn = a.rnorm[rec];
    } else {
      d.rn = 0;
    }
    d.nrm = F::GROUPED ? *(const uint32_t*)(a.norm + 2 * rec) : (uint32_t)a.norm[rec];
    d.zv = *(const uint2*)(a.vzero + rec * 4);
    d.sv = *(const uint2*)(a.vscale + rec * 4);
  };
  // value codes of this lane's tokens: c[8 chunk + j] for token 32 chunk + 4 j + kq.
  // Buffer loads against a range of the tile's rows below t_end: a load past
  // it returns 0 without touching memory (its token's weight is 0), so the
  // addresses are one offset per lane plus immediates, with no clamping.
  // They are nontemporal (nt: streamed past the caches; the codes are read
  // once, and each load of the wave covers whole lines).
  const int voff = kq * VROW + cbyte;
  auto load_codes = [&](int tb, uint32_t* c) {
    // (the tile's base and row count are wave-uniform: moved to scalar
    // registers, the descriptor needs no per-lane loop)
    const unsigned long long p = (unsigned long long)(a.vcodes + (tile_base(tb) + tb) * VROW);
    const unsigned long long pu = (unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p) |
                                  ((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) << 32);
    const int rows = __builtin_amdgcn_readfirstlane(min(max(t_end - tb, 0), TILE));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)pu, 0, rows * VROW, 0x00020000);
#pragma unroll
    for (int k = 0; k < NCODE; ++k)
      c[k] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff + (32 * (k >> 3) + 4 * (k & 7)) * VROW, 0, 2);
  };

  // ---- prologue: rotate the queries, project them, build the tables.
  // Global reads go out first, in the order they are needed: the queries and
  // sigma, the rows of S, then (after the first barrier) each wave's first
  // tile, whose latency the projection and table building cover.
  const int n_parts = H->n_parts;
  const float* cent0 = (const float*)(a.tables + H->off_centroids[0]);
  const float* cent1 = (const float*)(a.tables + H->off_centroids[n_parts > 1 ? 1 : 0]);
  const int lev0 = H->part_levels[0], lev1 = H->part_levels[n_parts > 1 ? 1 : 0];
  // waves 0..QH-1: head `wave` of the quad; lane holds coordinates lane, lane + 64
  float x0 = 0.0f, x1 = 0.0f, sg0 = 0.0f, sg1 = 0.0f;
  const int gq_w = QH * quad + wave;  // query head within the GQA group
  // raw query words first (both halves in flight together), converted below
  uint32_t qw0 = 0, qw1 = 0;
  if (wave < QH && gq_w < a.G) {
    const long long qrow = ((long long)b * a.Hq + hkv * a.G + gq_w) * KD;
    if (a.q_dtype == TQ_F32) {
      qw0 = ((const uint32_t*)a.q)[qrow + lane];
      qw1 = ((const uint32_t*)a.q)[qrow + lane + 64];
    } else {
      qw0 = ((const uint16_t*)a.q)[qrow + lane];
      qw1 = ((const uint16_t*)a.q)[qrow + lane + 64];
    }
  }
  float cmin0 = 0.0f, cmax0 = 0.0f, cmin1 = 0.0f, cmax1 = 0.0f;
  if (wave < QH) {
    const float* sig0 = (const float*)(a.tables + H->off_sigma[0]);
    const float* sig1 = (const float*)(a.tables + H->off_sigma[n_parts > 1 ? 1 : 0]);
    sg0 = sig0[lane];
    sg1 = F::GROUPED ? sig1[lane] : sig0[lane + 64];
    cmin0 = cent0[0];
    cmax0 = cent0[lev0 - 1];
    cmin1 = cent1[0];
    cmax1 = cent1[lev1 - 1];
  }
  // S q' on MFMA: wave w < 8 takes rows 16w .. 16w + 15 of S (operand A: row
  // 16w + (lane & 15), coordinates 32 ks + 8 (lane >> 4) .. + 7 of step ks).
  uint4 sfrag[4] = {};
  if constexpr (F::QJL) {
    if (wave < 8) {
      const uint4* sp = (const uint4*)((const uint16_t*)(a.tables + H->off_S) +
                                       (size_t)(16 * wave + (lane & 15)) * KD + 8 * (lane >> 4));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sfrag[ks] = sp[4 * ks];
    }
  }
  if (tid < 2 * CEN) {
    const int part = tid / CEN, k = tid % CEN;
    cen[tid] = part < n_parts && k < (part ? lev1 : lev0) ? (part ? cent1 : cent0)[k] : 0.0f;
  }
  if constexpr (F::DIRECT) {
    if (tid < (1 << B0)) L.c8[tid] = tid < lev0 ? cent0[tid] : 0.0f;
  }
  if (F::QJL && tid < QH) L.rng[F::NC - 1][tid] = 0.0f;
  if (tid < NW / 2) {
    L.prod[tid] = 0;
    L.cons[tid] = 0;
  }
  for (int i = tid; i < n_pages_wg; i += NT) {
    const int pg = a.block_table[(long long)b * a.max_blocks + lp0 + i];
    L.pages[i] = min(max(pg, 0), a.n_pages - 1);
  }

  // ---- appending: the workgroup whose range holds token tn encodes that
  // token's key and value from knew / vnew (the key in wave KENC_WAVE, the
  // value in VENC_WAVE, both idle until the first barrier).  The record goes
  // to LDS; quad 0's workgroup stores it into the planes for later calls.
  // Nothing in this launch reads it back from global memory: its score and
  // value are taken from the encoding itself.
  // Key ("tqlite" README 设计要点 and mode table; difai.kr tutorial 算法概述):
  // n = ||k||, y = H (sigma * k) / n, idx_j = number of boundaries <= y_j
  // (GROUPED: per half); PROD: r = y - c[idx], signs [S r >= 0] (S r on the
  // MFMA below, as a fifth column next to the queries), rho = n ||r|| /
  // sqrt(d); GROUPED_PROD: the signs of S w, w = concat_j (n_j / 8) r_j, and
  // rho = ||w||.  Value
  // (bit-packing article, sections 二/三): per 32-channel group
  // s = fp16((max - min) / (2^VB - 1)), z = fp16(min),
  // code = clamp(rint((v - z) / s), 0, 2^VB - 1) in float32, 0 when s = 0.
  {
    if (has_new && wave == KENC_WAVE) {
      // lane holds coordinates lane and lane + 64: one 128-point transform,
      // or (GROUPED) the two halves' 64-point ones, each half with its own
      // norm, sigma and codebook
      const long long kr = ((long long)b * a.Hkv + hkv) * KD;
      uint32_t w0, w1;
      if (a.kv_dtype == TQ_F32) {
        w0 = ((const uint32_t*)a.knew)[kr + lane];
        w1 = ((const uint32_t*)a.knew)[kr + lane + 64];
      } else {
        w0 = ((const uint16_t*)a.knew)[kr + lane];
        w1 = ((const uint16_t*)a.knew)[kr + lane + 64];
      }
      const float* sig0 = (const float*)(a.tables + H->off_sigma[0]);
      const float* sig1 = (const float*)(a.tables + H->off_sigma[F::GROUPED ? 1 : 0]);
      const float* bnd0 = (const float*)(a.tables + H->off_bounds[0]);
      const float* bnd1 = (const float*)(a.tables + H->off_bounds[F::GROUPED ? 1 : 0]);
      const float sgk0 = sig0[lane], sgk1 = F::GROUPED ? sig1[lane] : sig0[lane + 64];
      const int nl1 = F::GROUPED ? lev1 : lev0;  // levels of the codebook of coordinate lane + 64
      // boundary / centroid `lane` of each part (gathered by readlane / shuffle below)
      const float bl0 = lane < lev0 - 1 ? bnd0[lane] : INFINITY;
      const float bl1 = lane < nl1 - 1 ? bnd1[lane] : INFINITY;
      const float cl0 = lane < lev0 ? cent0[lane] : 0.0f;
      const float cl1 = lane < nl1 ? (F::GROUPED ? cent1 : cent0)[lane] : 0.0f;
      float k0 = q_word_to_float(w0, a.kv_dtype), k1 = q_word_to_float(w1, a.kv_dtype);
      // sums of squares on the coordinates scaled by the power of two that
      // brings the largest (of the key, or of each half) into [1, 2): no
      // fp32 under- or overflow for finite keys; the norms are scaled back
      float kmax0 = wave_max(fabsf(k0)), kmax1 = wave_max(fabsf(k1));
      if (!F::GROUPED) kmax0 = kmax1 = fmaxf(kmax0, kmax1);
      const int ke0 = kmax0 > 0.0f ? min(max(ilogbf(kmax0), -126), 127) : 0;
      const int ke1 = kmax1 > 0.0f ? min(max(ilogbf(kmax1), -126), 127) : 0;
      k0 = ldexpf(k0, -ke0);
      k1 = ldexpf(k1, -ke1);
      float ss0 = wave_sum(k0 * k0), ss1 = wave_sum(k1 * k1);
      if (!F::GROUPED) ss0 = ss1 = ss0 + ss1;
      const float inv0 = ss0 > 0.0f ? 1.0f / sqrtf(ss0) : 0.0f;  // a zero key (half) has y = 0
      const float inv1 = ss1 > 0.0f ? 1.0f / sqrtf(ss1) : 0.0f;
      float y0 = k0 * sgk0, y1 = k1 * sgk1;
      if constexpr (!F::GROUPED) {
        const float t = y0;
        y0 = t + y1;
        y1 = t - y1;
      }
      static_for<0, 6>([&](auto ii) {
        constexpr int st = 32 >> decltype(ii)::value;
        const float z0 = lane_xor<st>(y0, lane), z1 = lane_xor<st>(y1, lane);
        const bool up = lane & st;
        y0 = up ? z0 - y0 : y0 + z0;
        y1 = up ? z1 - y1 : y1 + z1;
      });
      y0 *= inv0;
      y1 *= inv1;
      int i0 = 0, i1 = 0;
      for (int t = 0; t < lev0 - 1; ++t)
        i0 += y0 >= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bl0), t)) ? 1 : 0;
      for (int t = 0; t < nl1 - 1; ++t)
        i1 += y1 >= __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bl1), t)) ? 1 : 0;
      L.nb8[lane] = (unsigned char)i0;
      L.nb8[lane + 64] = (unsigned char)i1;
      const float n0 = ldexpf(sqrtf(ss0), ke0), n1 = ldexpf(sqrtf(ss1), ke1);
      float rho = 0.0f;
      if constexpr (F::QJL) {
        float r0 = y0 - __shfl(cl0, i0), r1 = y1 - __shfl(cl1, i1);
        if constexpr (F::GROUPED) {
          // the sketch takes w = concat_j (n_j / 8) r_j, here divided by
          // max(n_0, n_1) / 8 (the signs do not change), rho = ||w||
          const float nmax = fmaxf(n0, n1);
          r0 *= nmax > 0.0f ? n0 / nmax : 0.0f;
          r1 *= nmax > 0.0f ? n1 / nmax : 0.0f;
          rho = nmax * sqrtf(wave_sum(fmaf(r0, r0, r1 * r1))) * 0.125f;
        } else {
          rho = ldexpf(sqrtf(ss0) * sqrtf(wave_sum(fmaf(r0, r0, r1 * r1))) * 0.088388347648318441f,
                       ke0);  // n ||r|| / sqrt(128)
        }
        qp[QH * KD + lane] = r0;
        qp[QH * KD + lane + 64] = r1;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      // index row: part 0's fields (W0 bits, coordinates 0 ..), then part 1's
      // (W1 bits, coordinates 64 ..) for GROUPED
      if (lane < F::IP0 / 4) {
        constexpr int W = F::W0, PER = 32 / W;
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) v |= (uint32_t)L.nb8[lane * PER + i] << (W * i);
        L.nrec[NR_IDX + lane] = v;
      } else if (F::GROUPED && lane < F::IDXB / 4) {
        constexpr int W = F::W1, PER = 32 / W;
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) v |= (uint32_t)L.nb8[64 + (lane - F::IP0 / 4) * PER + i] << (W * i);
        L.nrec[NR_IDX + lane] = v;
      }
      if (lane == 0) {
        const uint32_t h0 = __half_as_ushort(__float2half_rn(n0)), h1 = __half_as_ushort(__float2half_rn(n1));
        L.nrec[NR_NORM] = F::GROUPED ? h0 | (h1 << 16) : h0;
        L.nrec[NR_RNORM] = __half_as_ushort(__float2half_rn(rho));
      }
    }
    if (has_new && wave == VENC_WAVE) {
      const long long vr = ((long long)b * a.Hkv + hkv) * KD;
      uint32_t w0, w1;
      if (a.kv_dtype == TQ_F32) {
        w0 = ((const uint32_t*)a.vnew)[vr + lane];
        w1 = ((const uint32_t*)a.vnew)[vr + lane + 64];
      } else {
        w0 = ((const uint16_t*)a.vnew)[vr + lane];
        w1 = ((const uint16_t*)a.vnew)[vr + lane + 64];
      }
      // channel lane is in group lane / 32, channel lane + 64 in 2 + lane / 32
      const float v0 = q_word_to_float(w0, a.kv_dtype), v1 = q_word_to_float(w1, a.kv_dtype);
      float mn0 = v0, mx0 = v0, mn1 = v1, mx1 = v1;
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) {
        mn0 = fminf(mn0, __shfl_xor(mn0, m));
        mx0 = fmaxf(mx0, __shfl_xor(mx0, m));
        mn1 = fminf(mn1, __shfl_xor(mn1, m));
        mx1 = fmaxf(mx1, __shfl_xor(mx1, m));
      }
      constexpr float LV = (float)((1 << VB) - 1);
      const __half s0h = __float2half_rn(__fdiv_rn(mx0 - mn0, LV)), s1h = __float2half_rn(__fdiv_rn(mx1 - mn1, LV));
      const __half z0h = __float2half_rn(mn0), z1h = __float2half_rn(mn1);
      const float s0 = __half2float(s0h), s1 = __half2float(s1h);
      const float z0 = __half2float(z0h), z1 = __half2float(z1h);
      const int c0 = s0 == 0.0f ? 0 : (int)fminf(fmaxf(rintf(__fdiv_rn(v0 - z0, s0)), 0.0f), LV);
      const int c1 = s1 == 0.0f ? 0 : (int)fminf(fmaxf(rintf(__fdiv_rn(v1 - z1, s1)), 0.0f), LV);
      L.nb8[KD + lane] = (unsigned char)c0;
      L.nb8[KD + lane + 64] = (unsigned char)c1;
      L.vhat[lane] = fmaf((float)c0, s0, z0);  // the value as the cache holds it
      L.vhat[lane + 64] = fmaf((float)c1, s1, z1);
      if ((lane & 31) == 0) {
        const int g = lane >> 5;
        uint16_t* zz = (uint16_t*)&L.nrec[NR_Z];
        uint16_t* sz = (uint16_t*)&L.nrec[NR_S];
        zz[g] = __half_as_ushort(z0h);
        zz[2 + g] = __half_as_ushort(z1h);
        sz[g] = __half_as_ushort(s0h);
        sz[2 + g] = __half_as_ushort(s1h);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      if (lane < VROW / 4) {
        constexpr int PER = 32 / VB;
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) v |= (uint32_t)L.nb8[KD + lane * PER + i] << (VB * i);
        L.nrec[NR_CODE + lane] = v;
      }
    }
  }

  // Walsh-Hadamard transform of sigma * q in registers (one 128-point
  // transform, or two 64-point ones for GROUPED): butterflies on lane bits
  // through shuffles, the top stage inside the lane.  Then, per index class,
  // the table step and offset: a byte holding coordinates J takes values
  // sum_{j in J} q'_j c[f_j]; its range is (c_max - c_min) sum_J |q'_j| and
  // its smallest value sum_J min(q'_j c_min, q'_j c_max).
  if (wave < QH) {
    x0 = q_word_to_float(qw0, a.q_dtype) * sg0;
    x1 = q_word_to_float(qw1, a.q_dtype) * sg1;
    if constexpr (!F::GROUPED) {
      const float t = x0;
      x0 = t + x1;
      x1 = t - x1;
    }
    static_for<0, 6>([&](auto ii) {
      constexpr int st = 32 >> decltype(ii)::value;
      const float y0 = lane_xor<st>(x0, lane), y1 = lane_xor<st>(x1, lane);
      const bool up = lane & st;
      x0 = up ? y0 - x0 : x0 + y0;
      x1 = up ? y1 - x1 : x1 + y1;
    });
    qp[wave * KD + lane] = x0;
    qp[wave * KD + lane + 64] = x1;
    if constexpr (F::DIRECT) {
      L.qT[lane * QH + wave] = x0;
      L.qT[(lane + 64) * QH + wave] = x1;
    }
    constexpr int CPB0 = F::cpb(0), CPB1 = F::cpb(1);
    const float g0 = group_sum<CPB0>(fabsf(x0));
    const float lo0 = fminf(x0 * cmin0, x0 * cmax0);
    if constexpr (F::GROUPED) {
      const float g1 = group_sum<CPB1>(fabsf(x1));
      const float r0 = wave_max(g0) * (cmax0 - cmin0), r1 = wave_max(g1) * (cmax1 - cmin1);
      const float o0 = wave_sum(lo0), o1 = wave_sum(fminf(x1 * cmin1, x1 * cmax1));
      if (lane == 0) {
        L.rng[0][wave] = r0;
        L.rng[1][wave] = r1;
        L.offi[0][wave] = o0;
        L.offi[1][wave] = o1;
      }
    } else {
      const float g1 = group_sum<CPB0>(fabsf(x1));
      const float r0 = wave_max(fmaxf(g0, g1)) * (cmax0 - cmin0);
      const float o0 = wave_sum(lo0 + fminf(x1 * cmin0, x1 * cmax0));
      if (lane == 0) {
        L.rng[0][wave] = r0;
        L.offi[0][wave] = o0;
      }
    }
  }
  // Only LDS data is shared here, so the barrier need not wait for global
  // loads.  Each wave's first tile goes out now (a split past the sequence's
  // end loads nothing: its block-table entries need not name a page); the
  // projection and table building below cover its latency.  The prologue's
  // own loads (the rows of S) are waited for first: score and p.V waves
  // issue different numbers of tile loads, and a count-based wait for S
  // after them would also wait for part of the tile.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  lds_barrier();
  KeyData kd;
  uint32_t codes[NCODE];
  if (n_tiles > 0) {
    if (scorer) load_keys(tile_tb(0), kd);
    else load_codes(tile_tb(0), codes);
  }
  if constexpr (F::QJL) {
    if (wave < 8) {
      // operand B: query head n = lane & 15 (heads past QH are zero), the
      // same coordinates as A's; q' split into fp16 hi + lo (S is fp16, so
      // each product is exact and the sum is fp32)
      const int n = lane & 15;
      floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half8_t bh = {}, bl = {};
        if (n < QH || (n == QH && has_new)) {
          const float4* src = (const float4*)(qp + n * KD + 32 * ks + 8 * (lane >> 4));
          const float4 v0 = src[0], v1 = src[1];
          const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            bh[i] = (_Float16)v[i];
            bl[i] = (_Float16)(v[i] - (float)bh[i]);
          }
        }
        const half8_t af = __builtin_bit_cast(half8_t, sfrag[ks]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bl, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bh, acc, 0, 0, 0);
      }
      // lane holds S q' of head n for rows 16 wave + 4 (lane >> 4) + i
      if (n < QH) {
#pragma unroll
        for (int i = 0; i < 4; ++i) qs[n * KD + 16 * wave + 4 * (lane >> 4) + i] = acc[i];
      }
      if (has_new) {
        // the appended key's sign bits: column QH, rows 16 wave + 4 g + i in
        // lane 16 g + QH; bit 4 g + i of the wave's two sign bytes
        uint32_t bits16 = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t bm = __builtin_amdgcn_ballot_w64(acc[i] >= 0.0f);
#pragma unroll
          for (int g = 0; g < 4; ++g) bits16 |= (uint32_t)((bm >> (16 * g + QH)) & 1u) << (4 * g + i);
        }
        if (lane == 0) ((uint16_t*)&L.nrec[NR_SIGN])[wave] = (uint16_t)bits16;
      }
      // sign bytes 2 wave (lanes 0..31) and 2 wave + 1 (lanes 32..63): a
      // byte's values are sum_i +-(S q')_i over its 8 rows, range 2 sum |.|
      float v = fabsf(acc[0]) + fabsf(acc[1]) + fabsf(acc[2]) + fabsf(acc[3]);
      v = sum_xor16(v);
      const float rmax = 2.0f * max_xor32(v);
      const float tot = sum_xor32(v);
      if (lane < QH) {
        atomicMax((int*)&L.rng[F::NC - 1][lane], __float_as_int(rmax));
        L.sgp[wave][lane] = tot;
      }
    }
    lds_barrier();
  }
  // the appended record (complete in LDS now) into the planes, by quad 0
  if (has_new && quad == 0 && wave == KENC_WAVE) {
    // its record: rec0 + tn, or through the staged entry of tn's page
    const long long rec = a.block_table ? ((long long)L.pages[tn / a.page_size - lp0] * a.Hkv + hkv) * a.page_size +
                                              tn % a.page_size
                                        : rec0 + tn;
    if (lane < F::IDXB / 4) ((uint32_t*)(a.w_idx + rec * F::IDXB))[lane] = L.nrec[NR_IDX + lane];
    if (F::QJL && lane >= NR_SIGN && lane < NR_SIGN + 4)
      ((uint32_t*)(a.w_signs + rec * (KD / 8)))[lane - NR_SIGN] = L.nrec[lane];
    if (lane == NR_NORM) {
      if (F::GROUPED) *(uint32_t*)(a.w_norm + 2 * rec) = L.nrec[NR_NORM];  // the two halves' norms
      else a.w_norm[rec] = (uint16_t)L.nrec[NR_NORM];
    }
    if (F::QJL && lane == NR_RNORM) a.w_rnorm[rec] = (uint16_t)L.nrec[NR_RNORM];
    if (lane == NR_Z || lane == NR_Z + 1) ((uint32_t*)(a.w_vzero + rec * 4))[lane - NR_Z] = L.nrec[lane];
    if (lane == NR_S || lane == NR_S + 1) ((uint32_t*)(a.w_vscale + rec * 4))[lane - NR_S] = L.nrec[lane];
    if (lane >= NR_CODE && lane < NR_CODE + VROW / 4) ((uint32_t*)(a.w_vcodes + rec * VROW))[lane - NR_CODE] = L.nrec[lane];
  }
  {
    if (has_new && wave >= KENC_WAVE && wave < KENC_WAVE + QH) {
      // the appended token's score for head hh = wave - KENC_WAVE, from its
      // record, in float32:
      // <q, k_hat> = (n / PD) sum_j q'_j c[idx_j]   (GROUPED: per half, with
      //              the half's norm, transform and codebook)
      //            + rho sqrt(pi/2) / (m sqrt(PD)) sum_i (S q')_i (2 bit_i - 1)
      // with the stored fp16 norms (what a later call reads back)
      const int hh = wave - KENC_WAVE;
      const float r16 = h2f(L.nrec[NR_RNORM]);
      const float c0 = cen[L.nb8[lane]], c1 = cen[(F::GROUPED ? CEN : 0) + L.nb8[lane + 64]];
      float dot;
      if constexpr (F::GROUPED) {  // (n_j / PD) <q'_j, c_j[idx_j]> per half
        const float d0 = wave_sum(qp[hh * KD + lane] * c0), d1 = wave_sum(qp[hh * KD + lane + 64] * c1);
        dot = fmaf(h2f(L.nrec[NR_NORM] & 0xFFFFu) / (float)F::PD, d0, h2f(L.nrec[NR_NORM] >> 16) / (float)F::PD * d1);
      } else {
        const float di = wave_sum(fmaf(qp[hh * KD + lane], c0, qp[hh * KD + lane + 64] * c1));
        dot = h2f(L.nrec[NR_NORM]) / (float)F::PD * di;
      }
      if constexpr (F::QJL) {
        const float sg0 = (L.nrec[NR_SIGN + (lane >> 5)] >> (lane & 31)) & 1u ? 1.0f : -1.0f;
        const float sg1 = (L.nrec[NR_SIGN + 2 + (lane >> 5)] >> (lane & 31)) & 1u ? 1.0f : -1.0f;
        const float ds = wave_sum(fmaf(qs[hh * KD + lane], sg0, qs[hh * KD + lane + 64] * sg1));
        dot = fmaf(r16 * (SQRT_HALF_PI / ((float)KD * sqrtf((float)F::PD))), ds, dot);
      }
      if (lane == 0) {
        L.xnew[hh] = dot * (a.sm_scale * LOG2E);
        const int gq = QH * quad + hh;
        if (a.scores && gq < a.G) a.scores[((long long)b * a.Hq + hkv * a.G + gq) * a.max_ctx + tn] = dot;
      }
    }
  }
  // Half tables: for each byte position, nibble half and nibble value, the
  // four heads' partial sums over the coordinates (or sign rows) that nibble
  // holds, less the smallest such sum, in table steps (the low half carries
  // the +1/2 of the rounding).  A byte's entry is then lo[v & 15] + hi[v >> 4]
  // rounded down.  They live in the weight ring, unused until the main loop.
  float4* halves = (float4*)wbuf;  // [POSITIONS - HPOS0][2][16]
  for (int i = tid; i < (F::POSITIONS - F::HPOS0) * 32; i += NT) {
    const int pos = F::HPOS0 + (i >> 5), half = (i >> 4) & 1, n = i & 15;
    const int c = F::cls(pos);
    const int p = pos - F::pos0(c);
    const int kind = F::kind(c);
    float sv[QH] = {0.0f, 0.0f, 0.0f, 0.0f}, mn[QH] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (kind == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool one = (n >> k) & 1;
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) {
          const float z = qs[hh * KD + 8 * p + 4 * half + k];
          sv[hh] += one ? z : -z;
          mn[hh] -= fabsf(z);
        }
      }
    } else {
      const int W = kind ? F::W1 : F::W0;
      const int per = 4 / W;  // coordinates per nibble
      const int fmask = (1 << (kind ? B1 : B0)) - 1;
      const float* cn = cen + (kind ? CEN : 0);
      const float c_lo = cn[0], c_hi = cn[(kind ? lev1 : lev0) - 1];
      const int j0 = (kind ? F::PD : 0) + p * (8 / W) + half * per;
      for (int k = 0; k < per; ++k) {
        const float cv = cn[(n >> (W * k)) & fmask];
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) {
          const float z = qp[hh * KD + j0 + k];
          sv[hh] = fmaf(cv, z, sv[hh]);
          mn[hh] += fminf(z * c_lo, z * c_hi);
        }
      }
    }
    const float4 rg = *(const float4*)L.rng[c];
    const float rgv[QH] = {rg.x, rg.y, rg.z, rg.w};
    float o[QH];
#pragma unroll
    for (int hh = 0; hh < QH; ++hh) {
      const float inv = rgv[hh] > 0.0f ? F::EMAX / rgv[hh] : 0.0f;
      o[hh] = fmaf(sv[hh] - mn[hh], inv, half ? 0.0f : 0.5f);
    }
    halves[i] = make_float4(o[0], o[1], o[2], o[3]);
  }
  if constexpr (F::COORD) {
    // per-coordinate tables of the index class: entry (j, v) =
    // q'_j c[v] - min(q'_j c_lo, q'_j c_hi) in table steps, rounded
    const float4 rg = *(const float4*)L.rng[0];
    const float rgv[QH] = {rg.x, rg.y, rg.z, rg.w};
    const float c_lo = cen[0], c_hi = cen[lev0 - 1];
    for (int i = tid; i < F::PD << B0; i += NT) {
      const int j = i >> B0, v = i & ((1 << B0) - 1);
      const float cv = cen[v];
      uint32_t e[QH];
#pragma unroll
      for (int hh = 0; hh < QH; ++hh) {
        const float z = qp[hh * KD + j];
        const float inv = rgv[hh] > 0.0f ? F::EMAX / rgv[hh] : 0.0f;
        e[hh] = (uint32_t)fmaf(fmaf(cv, z, -fminf(z * c_lo, z * c_hi)), inv, 0.5f);
      }
      lut[F::ent(0) + i] = (uint64_t)(e[0] | (e[1] << 16)) | ((uint64_t)(e[2] | (e[3] << 16)) << 32);
    }
  }
  lds_barrier();
  // One thread per (position, low nibble) walks the high nibbles: its low
  // half stays in registers, the high halves are read by sixteen lanes at once.
  for (int t = tid; t < (F::POSITIONS - F::HPOS0) * 16; t += NT) {
    const int hp = t >> 4, lo = t & 15;  // half-table position
    const int pos = F::HPOS0 + hp;
    const int c = F::cls(pos);
    const int S = F::stride(c);
    uint64_t* dst = lut + F::ent(c) + (pos - F::pos0(c)) * S;
    const float4 lo4 = halves[hp * 32 + lo];
#pragma unroll 4
    for (int hi = 0; hi < 16; ++hi) {
      const int v = hi * 16 + lo;
      if (v < S) {
        const float4 hi4 = halves[hp * 32 + 16 + hi];
        const uint32_t e0 = (uint32_t)(lo4.x + hi4.x), e1 = (uint32_t)(lo4.y + hi4.y);
        const uint32_t e2 = (uint32_t)(lo4.z + hi4.z), e3 = (uint32_t)(lo4.w + hi4.w);
        dst[v] = (uint64_t)(e0 | (e1 << 16)) | ((uint64_t)(e2 | (e3 << 16)) << 32);
      }
    }
  }
  // per class and head: the table step (range / EMAX) and the summed
  // offsets, with the score multiplier of the class and the softmax scale
  // (log2 units) folded in
  const float xscale = a.sm_scale * LOG2E;
  if (tid < F::NC * QH) {
    const int c = tid >> 2, hh = tid & 3;
    const int kind = F::kind(c);
    float off;
    if (kind == 4) {
      off = 0.0f;  // (the direct class sums q'_j c[idx_j] as they are)
    } else if (kind == 2) {
      off = 0.0f;
      for (int w = 0; w < 8; ++w) off -= L.sgp[w][hh];
    } else {
      off = L.offi[kind == 3 ? 0 : kind][hh];
    }
    // q' holds sqrt(PD) Pi q (per half when GROUPED): the sign class's
    // rho sqrt(pi/2) / m <S Pi q, .> is rho sqrt(pi/2) / (m sqrt(PD)) <S q', .>
    const float mul = kind == 2 ? SQRT_HALF_PI / ((float)KD * sqrtf((float)F::PD)) : 1.0f / (float)F::PD;
    const float unit = kind == 4 ? 1.0f : L.rng[c][hh] / F::EMAX;
    L.uu[c][hh] = mul * unit * xscale;
    L.oo[c][hh] = mul * off * xscale;
  }
  lds_barrier();

  const half2_t e10 = {(_Float16)1.0f, (_Float16)0.0f}, e01 = {(_Float16)0.0f, (_Float16)1.0f};
  float* red = (float*)smem;  // [NS][QH][2 + 4 + KD], over the tables once every wave is done
  constexpr int RS = 2 + 4 + KD;
  static_assert(sizeof(L.lut) >= NS * QH * RS * sizeof(float), "the end sums fit over the tables");
  float* mine = red + pw * QH * RS;
  // The two kinds of waves run separate loops (one barrier after each), so
  // neither keeps the other's registers live.
  if (scorer) {
    float UU[F::NC][QH], OO[F::NC][QH];
#pragma unroll
    for (int c = 0; c < F::NC; ++c) {
      const float4 uv = *(const float4*)L.uu[c], ov = *(const float4*)L.oo[c];
      UU[c][0] = uniform(uv.x); UU[c][1] = uniform(uv.y); UU[c][2] = uniform(uv.z); UU[c][3] = uniform(uv.w);
      OO[c][0] = uniform(ov.x); OO[c][1] = uniform(ov.y); OO[c][2] = uniform(ov.z); OO[c][3] = uniform(ov.w);
    }
    float m_run[QH], l_run[QH], zacc[QH][4];
#pragma unroll
    for (int hh = 0; hh < QH; ++hh) {
      m_run[hh] = -INFINITY;
      l_run[hh] = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) zacc[hh][k] = 0.0f;
    }
    // value scales are multiplied by 2^ks (ks in [-15, 15], one per tile,
    // kept while the tile's largest scale times 2^ks stays in [2^-8, 2))
    int ks = 0;
    float ksc = 1.0f;
    auto s_round = [&](int r, KeyData& kd) {
      const int tb = tile_tb(r);
      if (r < rounds && tb < t_end) {
        // ---------------- scores: lane = token
        const int t = tb + lane;
        const bool valid = t < t_end;
        float x[QH];
        {
          // per-token multipliers of the classes: norm (part 0), then the
          // second half's norm (GROUPED) and the residual norm (QJL)
          const float m0 = F::GROUPED ? h2f(kd.nrm & 0xFFFFu) : h2f(kd.nrm);
          const float m1 = F::GROUPED ? h2f(kd.nrm >> 16) : h2f(kd.rn);
          const float m2 = h2f(kd.rn);
          // The table reads run in batches of two chains (eight reads),
          // software-pipelined: batch i + 1 is issued before batch i is
          // summed, so one batch's latency hides behind the other's.
          constexpr int CHAIN = F::CHAIN;
          constexpr int NCH = F::POSITIONS / CHAIN;
          // chains per batch: two, or one for 5- and 6-bit indices (a whole
          // 128-byte index row in registers leaves no room for eight reads)
          constexpr int BCH = F::COORD && F::W0 == 8 ? 1 : 2;
          constexpr int NB = NCH / BCH;
          static_assert(NCH % BCH == 0, "whole batches of chains");
          uint32_t acc[F::NC][QH];
          uint64_t E[BCH * CHAIN];
          auto issue = [&](auto bb, uint64_t* dst) {
            constexpr int bt = decltype(bb)::value;
#pragma unroll
            for (int j = 0; j < BCH * CHAIN; ++j) {
              const int g = BCH * bt + j / CHAIN;
              const int c = F::chain_cls(g);
              const int pos = (g - F::chain0(c)) * CHAIN + j % CHAIN;
              const uint32_t base = (uint32_t)(F::ent(c) + pos * F::stride(c)) * 8u;
              if (F::kind(c) == 3 && F::W0 == 4) {
                dst[j] = lut_read_nib(smem, base, kd.kw[pos >> 3], pos & 7);  // coordinate = nibble
              } else {
                const int byte = F::kbyte(c) + pos;  // (kind 3 with 8-bit fields: coordinate = byte)
                dst[j] = lut_read(smem, base, kd.kw[byte >> 2], byte & 3);
              }
            }
          };
          auto reduce = [&](auto bb, const uint64_t* src) {
            constexpr int bt = decltype(bb)::value;
#pragma unroll
            for (int i = 0; i < BCH; ++i) {
              const int g = BCH * bt + i;
              const int c = F::chain_cls(g);
              const int q = g - F::chain0(c);
              uint64_t sum = src[CHAIN * i];
#pragma unroll
              for (int k = 1; k < CHAIN; ++k) sum += src[CHAIN * i + k];
              const uint32_t lo = (uint32_t)sum, hi = (uint32_t)(sum >> 32);
              if (q == 0) {
                acc[c][0] = lo & 0xFFFFu;
                acc[c][1] = lo >> 16;
                acc[c][2] = hi & 0xFFFFu;
                acc[c][3] = hi >> 16;
              } else {
                const ushort2_t l2 = __builtin_bit_cast(ushort2_t, lo), h2 = __builtin_bit_cast(ushort2_t, hi);
                const ushort2_t u10 = {1, 0}, u01 = {0, 1};
                acc[c][0] = __builtin_amdgcn_udot2(l2, u10, acc[c][0], false);
                acc[c][1] = __builtin_amdgcn_udot2(l2, u01, acc[c][1], false);
                acc[c][2] = __builtin_amdgcn_udot2(h2, u10, acc[c][2], false);
                acc[c][3] = __builtin_amdgcn_udot2(h2, u01, acc[c][3], false);
              }
            }
          };
          static_for<0, NB>([&](auto bb) {
            issue(bb, E);
            __builtin_amdgcn_sched_barrier(0);
            reduce(bb, E);
            __builtin_amdgcn_sched_barrier(0);
          });
          // DIRECT: the index class as sum_j q'_j c[idx_j] in float32, the
          // centroid gathered from LDS by the index byte, the four heads' q'_j
          // one broadcast read
          float accf[QH] = {0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (F::DIRECT) {
            const float4* qT4 = (const float4*)L.qT;
            const unsigned char* c8b = (const unsigned char*)L.c8;
#pragma unroll
            for (int j = 0; j < KD; ++j) {
              const uint32_t off = ((kd.kw[j >> 2] >> (8 * (j & 3))) & 0xFFu) * 4u;
              const float c = *(const float*)(c8b + off);
              const float4 qv = qT4[j];
              accf[0] = fmaf(qv.x, c, accf[0]);
              accf[1] = fmaf(qv.y, c, accf[1]);
              accf[2] = fmaf(qv.z, c, accf[2]);
              accf[3] = fmaf(qv.w, c, accf[3]);
            }
          }
#pragma unroll
          for (int hh = 0; hh < QH; ++hh) {
            float v = F::DIRECT ? m0 * (accf[hh] * UU[0][hh]) : m0 * fmaf((float)acc[0][hh], UU[0][hh], OO[0][hh]);
            if constexpr (F::NC > 1) v = fmaf(m1, fmaf((float)acc[1][hh], UU[1][hh], OO[1][hh]), v);
            if constexpr (F::NC > 2) v = fmaf(m2, fmaf((float)acc[2][hh], UU[2][hh], OO[2][hh]), v);
            x[hh] = valid ? v : -INFINITY;  // log2 softmax units
          }
          if (a.scores && valid) {
            const float inv_x = 1.0f / xscale;
#pragma unroll
            for (int hh = 0; hh < QH; ++hh) {
              const int gq = QH * quad + hh;
              if (gq < a.G) a.scores[((long long)b * a.Hq + hkv * a.G + gq) * a.max_ctx + t] = x[hh] * inv_x;
            }
          }
        }
        // ---------------- online softmax (base 2).  The wave-wide max is
        // only recomputed when some lane exceeds the running max; otherwise
        // every p = 2^(x - m) <= 1 already and nothing needs rescaling.
        float alpha[QH] = {1.0f, 1.0f, 1.0f, 1.0f};
        bool exceed = false;
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) exceed |= x[hh] > m_run[hh];
        if (__builtin_amdgcn_ballot_w64(exceed) != 0) {
#pragma unroll
          for (int hh = 0; hh < QH; ++hh) {
            const float mn = uniform(fmaxf(m_run[hh], wave_max(x[hh])));
            alpha[hh] = m_run[hh] == -INFINITY ? 0.0f : exp2f(m_run[hh] - mn);
            m_run[hh] = mn;
            l_run[hh] *= alpha[hh];
#pragma unroll
            for (int k = 0; k < 4; ++k) zacc[hh][k] *= alpha[hh];
          }
        }
        // the tile's largest value scale (fp16 >= 0: compared as integers);
        // a new power of two when it leaves [2^-8, 2) times the current one
        const uint32_t smx2 = max(kd.sv.x & 0x7FFF7FFFu, kd.sv.y & 0x7FFF7FFFu);
        const uint32_t smx = wave_max_u32(max(smx2 & 0xFFFFu, smx2 >> 16));
        float fac = 1.0f;
        {
          const float smax = h2f(smx);
          const float rel = smax * ksc;
          if (smax > 0.0f && (rel >= 2.0f || rel < 0.00390625f)) {
            int e;
            (void)frexpf(smax, &e);        // smax = m 2^e, m in [0.5, 1)
            const int knew = min(max(1 - e, -15), 15);
            fac = ldexpf(1.0f, knew - ks);
            ks = knew;
            ksc = ldexpf(1.0f, ks);
          }
        }
        const uint2 zv = kd.zv, sv = kd.sv;
        // the next tile's key bytes go out now, into the buffer this tile's
        // lookups are done with
        load_keys(tile_tb(r + 1), kd);
        float zz[4];
        zz[0] = h2f(zv.x & 0xFFFFu); zz[1] = h2f(zv.x >> 16);
        zz[2] = h2f(zv.y & 0xFFFFu); zz[3] = h2f(zv.y >> 16);
        float p[QH];
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) {
          // p * 2^14 (m_run is finite: lane 0 holds a valid token)
          p[hh] = __builtin_amdgcn_exp2f(x[hh] - (m_run[hh] - PSCALE));
          l_run[hh] += p[hh];
#pragma unroll
          for (int k = 0; k < 4; ++k) zacc[hh][k] = fmaf(p[hh], zz[k], zacc[hh][k]);
        }
        // weights (p 2^14) * (scale 2^ks) as fp16 (both factors rounded to
        // fp16, then two heads per packed multiply) into the A operand of the
        // p.V wave: row 4 group + head, this token's place (chunk, kq, j)
        uint16_t* wb16 = (uint16_t*)(wbuf + ((r & 1) * NS + pw) * WSLOT) +
                         ((lane >> 5) * 4 + (lane & 3)) * ABLK + ((lane >> 2) & 7);
        const half2_t p01 = __builtin_convertvector((float2_t){p[0], p[1]}, half2_t);
        const half2_t p23 = __builtin_convertvector((float2_t){p[2], p[3]}, half2_t);
        const half2_t kk2 = {(_Float16)ksc, (_Float16)ksc};
        const half2_t s01 = __builtin_bit_cast(half2_t, sv.x) * kk2, s23 = __builtin_bit_cast(half2_t, sv.y) * kk2;
        const _Float16 sk[4] = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const half2_t s2 = {sk[k], sk[k]};
          const half2_t w01 = p01 * s2, w23 = p23 * s2;
          wb16[(4 * k + 0) * 8] = __builtin_bit_cast(uint32_t, w01) & 0xFFFFu;
          wb16[(4 * k + 1) * 8] = __builtin_bit_cast(uint32_t, w01) >> 16;
          wb16[(4 * k + 2) * 8] = __builtin_bit_cast(uint32_t, w23) & 0xFFFFu;
          wb16[(4 * k + 3) * 8] = __builtin_bit_cast(uint32_t, w23) >> 16;
        }
        if (lane == 0) {
#pragma unroll
          for (int hh = 0; hh < QH; ++hh) abuf[((r & 1) * NS + pw) * QH + hh] = alpha[hh] * fac;
        }
      }
    };
    for (int r = 0; r <= rounds; ++r) {
      if (r >= 2) pair_wait(&L.cons[pw], r - 1);  // slot r & 1 read by the p.V wave
      s_round(r, kd);
      pair_publish(&L.prod[pw], r + 1);
    }
    lds_barrier();  // every wave is done with the tables before the sums go over them
#pragma unroll
    for (int hh = 0; hh < QH; ++hh) {
      const float ls = wave_sum(l_run[hh]);
      float zs[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) zs[k] = wave_sum(zacc[hh][k]);
      if (lane == 0) {
        mine[hh * RS + 0] = m_run[hh];
        mine[hh * RS + 1] = ls;
#pragma unroll
        for (int k = 0; k < 4; ++k) mine[hh * RS + 2 + k] = zs[k];
      }
    }
    if (lane == 0) L.ksf[pw] = ks;
  } else {
    // acc[beta]: the MFMA accumulator of column block beta; lane holds rows
    // 4 kq + i (value group kq, head i) of column pn (channel 8 pn + beta)
    floatx4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = (floatx4){0.0f, 0.0f, 0.0f, 0.0f};
    // two code buffers in turn: round r consumes tile r - 1 while the codes
    // of tile r arrive in the other
    uint32_t codes2[NCODE];
    auto pv_round = [&](int r, const uint32_t* cur, uint32_t* nxt) {
      const int tb = r >= 1 ? tile_tb(r - 1) : t_end;
      if (tb < t_end) {
        load_codes(tile_tb(r), nxt);  // next round's tile
        const uint32_t* wsrc = wbuf + (((r - 1) & 1) * NS + pw) * WSLOT;
        const float4 al = *(const float4*)(abuf + (((r - 1) & 1) * NS + pw) * QH);
        const float alv[QH] = {uniform(al.x), uniform(al.y), uniform(al.z), uniform(al.w)};
        if (alv[0] != 1.0f || alv[1] != 1.0f || alv[2] != 1.0f || alv[3] != 1.0f) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int i = 0; i < QH; ++i) acc[k][i] *= alv[i];
        }
        // ---------------- p.V on MFMA: per 32-token chunk, A = the weights
        // (rows group x head), B = the codes (column n of block beta: channel
        // 8 n + beta).  B elements are the code fields left in place as fp16
        // subnormal bit patterns: a byte's fields up to field f, masked, so
        // one byte permute serves a whole byte and the byte's last field
        // needs no mask; block beta then sums prefixes, told apart at the end.
        // byte bb of the lane's channels in tokens A, B -> bytes 0 and 2
        uint32_t psel[VB];
#pragma unroll
        for (int bb = 0; bb < VB; ++bb) psel[bb] = 0x0c000c00u | ((4u + cb0 + bb) << 16) | (cb0 + bb);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const half8_t A = *(const half8_t*)(wsrc + ((cc * 4 + kq) * ABLK + pn * 8) / 2);
          // per code byte bb: Y[i] = byte bb of tokens 2i and 2i + 1 in bytes
          // 0 and 2, then the blocks of the byte's fields
#pragma unroll
          for (int bb = 0; bb < VB; ++bb) {
            uint32_t Y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t cA = cur[8 * cc + 2 * i], cB = cur[8 * cc + 2 * i + 1];
              Y[i] = __builtin_amdgcn_perm(cB, cA, psel[bb]);
            }
            constexpr int PER = 8 / VB;  // fields per byte
#pragma unroll
            for (int f = 0; f < PER; ++f) {
              // prefix of fields 0..f of the byte (the last one unmasked)
              const uint32_t mask = (VB == 2 ? (f == 0 ? 0x00030003u : f == 1 ? 0x000F000Fu : f == 2 ? 0x003F003Fu : 0x00FF00FFu)
                                             : (f == 0 ? 0x000F000Fu : 0x00FF00FFu));
              const bool bare = f == PER - 1;
              u32x4_t bv;
#pragma unroll
              for (int i = 0; i < 4; ++i) bv[i] = bare ? Y[i] : Y[i] & mask;
              acc[PER * bb + f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(half8_t, bv), acc[PER * bb + f], 0, 0, 0);
            }
          }
        }
      }
    };
    for (int r = 0; r <= rounds; r += 2) {
      pair_wait(&L.prod[pw], r);
      pv_round(r, codes2, codes);
      pair_publish(&L.cons[pw], r);
      if (r + 1 <= rounds) {
        pair_wait(&L.prod[pw], r + 1);
        pv_round(r + 1, codes, codes2);
        pair_publish(&L.cons[pw], r + 1);
      }
    }
    lds_barrier();
    // Undo the placement: block beta holds, in units of 2^-24, the prefix
    // sum over the fields of its byte up to beta's, field f weighted by its
    // place value 2^(VB f); a channel's sum is the difference of consecutive
    // prefixes over its place value.  Channel 8 pn + beta is in value group
    // pn / 4, so the lanes whose rows are that group hold it.
    if (kq == (pn >> 2)) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        constexpr int PER = 8 / VB;  // fields per byte
        const int f = k % PER;
        const float unit = 16777216.0f / (float)(1 << (VB * f));
#pragma unroll
        for (int i = 0; i < QH; ++i) {
          const float v = f == 0 ? acc[k][i] : acc[k][i] - acc[k - 1][i];
          mine[i * RS + 6 + 8 * pn + k] = v * unit;
        }
      }
    }
  }
  __syncthreads();
  // Combine the NS streams (score wave pw + p.V wave pw) of this workgroup:
  // p.V sums are in units of 2^ks of their stream's final value scale.
  for (int i = tid; i < QH * KD; i += NT) {
    const int hh = i / KD, j = i % KD;
    const int gq = QH * quad + hh;
    float M = -INFINITY;
    for (int w = 0; w < NS; ++w) M = fmaxf(M, red[(w * QH + hh) * RS]);
    const float xn = has_new ? L.xnew[hh] : -INFINITY;  // the appended token (weight 2^PSCALE at its own max)
    M = fmaxf(M, xn);
    float Ls = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
      for (int w = 0; w < NS; ++w) {
        const float* rr = red + (w * QH + hh) * RS;
        const float f = rr[0] == -INFINITY ? 0.0f : exp2f(rr[0] - M);
        Ls = fmaf(rr[1], f, Ls);
        O = fmaf(fmaf(rr[6 + j], ldexpf(1.0f, -L.ksf[w]), rr[2 + j / 32]), f, O);
      }
      if (has_new) {
        const float f = exp2f(xn - (M - PSCALE));
        Ls += f;
        O = fmaf(L.vhat[j], f, O);
      }
    }
    if (gq < a.G) {
      float* dst = a.part + (((long long)b * a.Hq + hkv * a.G + gq) * a.n_split + split) * PART;
      if (j == 0) {
        dst[0] = M;
        dst[1] = Ls;
      }
      dst[2 + j] = O;
    }
  }
}

// out[b][h][:] = sum_s O_s 2^(M_s - M) / sum_s L_s 2^(M_s - M), in split order.
// A NaN sum (tables that do not match the kernel's format) makes the row NaN.
// The largest M_s is found by the block's threads together (a strided share
// each, then a reduction); the weighted sums run in split order, the first
// splits' partials already loaded with the maxima, the rest unrolled so that
// several splits' partials are in flight at once (a long context has tens of
// splits per head).
__global__ __launch_bounds__(KD) void merge_kernel(const float* part, int n_split, float* out,
                                                   float* lse) {
  static_assert(KD == 128, "two waves per block");
  const int bh = blockIdx.x, j = threadIdx.x;
  const float* p = part + (long long)bh * n_split * PART;
  // the first PRE splits' (max, sum, output element) go out with the loads
  // of the maxima, so that a short merge reads the partials in one round
  constexpr int PRE = 8;
  float pm[PRE], pl[PRE], po[PRE];
#pragma unroll
  for (int s = 0; s < PRE; ++s) {
    const bool in = s < n_split;
    pm[s] = in ? p[s * PART] : -INFINITY;
    pl[s] = in ? p[s * PART + 1] : 0.0f;
    po[s] = in ? p[s * PART + 2 + j] : 0.0f;
  }
  __shared__ float s_max[2];
  __shared__ int s_bad[2];
  float M = -INFINITY;
  bool bad = false;
  for (int s = j; s < n_split; s += KD) {
    M = fmaxf(M, p[s * PART]);
    bad |= p[s * PART + 1] != p[s * PART + 1];
  }
  M = wave_max(M);
  const bool wbad = __builtin_amdgcn_ballot_w64(bad) != 0;
  if ((j & 63) == 0) {
    s_max[j >> 6] = M;
    s_bad[j >> 6] = wbad;
  }
  __syncthreads();
  M = fmaxf(s_max[0], s_max[1]);
  bad = s_bad[0] | s_bad[1];
  float Ls = 0.0f, O = 0.0f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < PRE; ++s) {
      if (s < n_split) {
        const float f = pm[s] == -INFINITY ? 0.0f : exp2f(pm[s] - M);
        Ls = fmaf(pl[s], f, Ls);
        O = fmaf(po[s], f, O);
      }
    }
#pragma unroll 8
    for (int s = PRE; s < n_split; ++s) {
      const float* r = p + s * PART;
      const float f = r[0] == -INFINITY ? 0.0f : exp2f(r[0] - M);
      Ls = fmaf(r[1], f, Ls);
      O = fmaf(r[2 + j], f, O);
    }
  }
  const float nan = __builtin_nanf("");
  out[(long long)bh * KD + j] = bad ? nan : Ls > 0.0f ? O / Ls : 0.0f;
  if (lse && j == 0)
    lse[bh] = bad ? nan : Ls > 0.0f ? (M + log2f(Ls) - PSCALE) * 0.69314718055994531f : -INFINITY;
}

template <int MODE, int B0, int B1, int VB>
hipError_t launch(const DecArgs& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<MODE, B0, B1, VB>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int MODE, int B0, int B1>
hipError_t launch_vb(int vb, const DecArgs& a, dim3 grid, hipStream_t s) {
  return vb == 2 ? launch<MODE, B0, B1, 2>(a, grid, s) : launch<MODE, B0, B1, 4>(a, grid, s);
}

// Formats with a kernel: returns false for the rest.
bool supported(const tq::Parts& P) {
  if (P.mode == TQ_MODE_GROUPED_PROD) {
    const int b0 = P.part_bits[0], b1 = P.part_bits[1];
    return (b0 == 3 && b1 == 2) || (b0 == 4 && b1 == 1);
  }
  if (P.mode == TQ_MODE_GROUPED) {
    const int b0 = P.part_bits[0], b1 = P.part_bits[1];
    return (b0 == 4 && b1 == 2) || (b0 == 2 && b1 == 2) || (b0 == 3 && b1 == 2) || (b0 == 4 && b1 == 1);
  }
  return P.part_bits[0] >= 1 && P.part_bits[0] <= 8;
}

hipError_t dispatch(const tq::Parts& P, int vb, const DecArgs& a, dim3 grid, hipStream_t s) {
  if (P.mode == TQ_MODE_PROD) {
    switch (P.part_bits[0]) {
      case 1: return launch_vb<TQ_MODE_PROD, 1, 0>(vb, a, grid, s);
      case 2: return launch_vb<TQ_MODE_PROD, 2, 0>(vb, a, grid, s);
      case 3: return launch_vb<TQ_MODE_PROD, 3, 0>(vb, a, grid, s);
      case 4: return launch_vb<TQ_MODE_PROD, 4, 0>(vb, a, grid, s);
      case 5: return launch_vb<TQ_MODE_PROD, 5, 0>(vb, a, grid, s);
      case 6: return launch_vb<TQ_MODE_PROD, 6, 0>(vb, a, grid, s);
      case 7: return launch_vb<TQ_MODE_PROD, 7, 0>(vb, a, grid, s);
      default: return launch_vb<TQ_MODE_PROD, 8, 0>(vb, a, grid, s);
    }
  }
  if (P.mode == TQ_MODE_MSE) {
    switch (P.part_bits[0]) {
      case 1: return launch_vb<TQ_MODE_MSE, 1, 0>(vb, a, grid, s);
      case 2: return launch_vb<TQ_MODE_MSE, 2, 0>(vb, a, grid, s);
      case 3: return launch_vb<TQ_MODE_MSE, 3, 0>(vb, a, grid, s);
      case 4: return launch_vb<TQ_MODE_MSE, 4, 0>(vb, a, grid, s);
      case 5: return launch_vb<TQ_MODE_MSE, 5, 0>(vb, a, grid, s);
      case 6: return launch_vb<TQ_MODE_MSE, 6, 0>(vb, a, grid, s);
      case 7: return launch_vb<TQ_MODE_MSE, 7, 0>(vb, a, grid, s);
      default: return launch_vb<TQ_MODE_MSE, 8, 0>(vb, a, grid, s);
    }
  }
  const int b0 = P.part_bits[0], b1 = P.part_bits[1];
  if (P.mode == TQ_MODE_GROUPED_PROD) {
    if (b0 == 3 && b1 == 2) return launch_vb<TQ_MODE_GROUPED_PROD, 3, 2>(vb, a, grid, s);
    return launch_vb<TQ_MODE_GROUPED_PROD, 4, 1>(vb, a, grid, s);
  }
  if (b0 == 4 && b1 == 2) return launch_vb<TQ_MODE_GROUPED, 4, 2>(vb, a, grid, s);
  if (b0 == 2 && b1 == 2) return launch_vb<TQ_MODE_GROUPED, 2, 2>(vb, a, grid, s);
  if (b0 == 3 && b1 == 2) return launch_vb<TQ_MODE_GROUPED, 3, 2>(vb, a, grid, s);
  return launch_vb<TQ_MODE_GROUPED, 4, 1>(vb, a, grid, s);
}

}  // namespace

namespace {

tq_status decode_impl(const tq_key_config* cfg, const void* tables, const void* q, int32_t q_dtype,
                      int32_t B, int32_t Hq, int32_t Hkv, const int32_t* ctx_len, int32_t max_ctx,
                      const int32_t* block_table, int32_t max_blocks, int32_t page_size, int32_t n_pages,
                      const uint8_t* idx, const uint8_t* signs, const uint16_t* norm,
                      const uint16_t* rnorm, int32_t v_bits, int32_t v_group, const uint8_t* v_codes,
                      const uint16_t* v_scale, const uint16_t* v_zero, float sm_scale, float* out,
                      float* lse, float* scores, void* workspace, size_t* workspace_bytes,
                      void* stream, const void* k_new = nullptr, const void* v_new = nullptr,
                      int32_t kv_dtype = TQ_F32) {
  tq::Parts P;
  tq_status st = tq::describe(cfg, &P);
  if (st != TQ_OK) return st;
  if (P.d != KD || !supported(P)) return TQ_ERR_UNSUPPORTED;
  if (v_bits != 2 && v_bits != 4) return TQ_ERR_UNSUPPORTED;
  if (v_group != 32) return TQ_ERR_UNSUPPORTED;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_ERR_ARG;
  // appending (tq_decode_attention_append): both new rows; not for indices
  // of 7 or 8 bits (their codebooks exceed the one-wave encoder's lanes)
  if (k_new || v_new) {
    if (!k_new || !v_new) return TQ_ERR_ARG;
    if (P.mode != TQ_MODE_GROUPED && P.mode != TQ_MODE_GROUPED_PROD && P.part_bits[0] >= 7) return TQ_ERR_UNSUPPORTED;
    if (kv_dtype != TQ_F32 && kv_dtype != TQ_BF16 && kv_dtype != TQ_F16) return TQ_ERR_ARG;
    const uintptr_t al = kv_dtype == TQ_F32 ? 3 : 1;
    if (((uintptr_t)k_new & al) || ((uintptr_t)v_new & al)) return TQ_ERR_ARG;
  }
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_ctx <= 0) return TQ_ERR_ARG;
  if (!workspace_bytes) return TQ_ERR_ARG;
  const int cus = tq::cu_count();
  if (cus <= 0) return TQ_ERR_HIP;
  const int G = Hq / Hkv;
  const int n_quads = (G + QH - 1) / QH;
  const long long groups = (long long)B * Hkv * n_quads;
  if ((long long)B * Hkv > 65535 || n_quads > 65535) return TQ_ERR_ARG;
  // split the context so that the grid covers every CU about once
  const int max_tiles = (max_ctx + TILE - 1) / TILE;
  int n_split = (int)((cus + groups - 1) / groups);
  const int tiles_per_split_min = NW;  // at least one tile per wave
  if (n_split > (max_tiles + tiles_per_split_min - 1) / tiles_per_split_min)
    n_split = (max_tiles + tiles_per_split_min - 1) / tiles_per_split_min;
  if (n_split < 1) n_split = 1;
  // paged: a split spans at most chunk / page_size + 2 pages, all staged in LDS
  if (page_size > 0) {
    const int max_chunk_tiles = (PAGE_CACHE - 1) * (page_size / TILE);
    if (n_split < (max_tiles + max_chunk_tiles - 1) / max_chunk_tiles)
      n_split = (max_tiles + max_chunk_tiles - 1) / max_chunk_tiles;
  }
  const int chunk_tiles = (max_tiles + n_split - 1) / n_split;
  n_split = (max_tiles + chunk_tiles - 1) / chunk_tiles;
  const size_t need = (size_t)B * Hq * n_split * PART * sizeof(float);
  if (!workspace) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) return TQ_ERR_WORKSPACE;
  if (!tables || !q || !ctx_len || !idx || !norm || !v_codes || !v_scale || !v_zero || !out)
    return TQ_ERR_ARG;
  if (P.m > 0 && (!signs || !rnorm)) return TQ_ERR_ARG;
  if (!tq::aligned16(tables) || !tq::aligned16(idx) || !tq::aligned16(v_codes) ||
      !tq::aligned16(workspace) || !tq::aligned16(q))
    return TQ_ERR_ARG;
  if (P.m > 0 && !tq::aligned16(signs)) return TQ_ERR_ARG;
  if (((uintptr_t)v_scale & 7) || ((uintptr_t)v_zero & 7) || ((uintptr_t)norm & 3) ||
      ((uintptr_t)out & 3))
    return TQ_ERR_ARG;
  if (max_ctx > 0x7fffffff / 2) return TQ_ERR_ARG;

  DecArgs a;
  a.tables = (const unsigned char*)tables;
  a.q = q;
  a.q_dtype = q_dtype;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.n_quads = n_quads;
  a.ctx_len = ctx_len;
  a.max_ctx = max_ctx;
  a.idx = idx;
  a.signs = signs;
  a.norm = norm;
  a.rnorm = rnorm;
  a.vcodes = v_codes;
  a.vscale = v_scale;
  a.vzero = v_zero;
  a.sm_scale = sm_scale;
  a.scores = scores;
  a.part = (float*)workspace;
  a.n_split = n_split;
  a.chunk = chunk_tiles * TILE;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.page_size = page_size;
  a.n_pages = n_pages;
  a.knew = k_new;
  a.vnew = v_new;
  a.kv_dtype = kv_dtype;
  // appending stores the new records into the planes the decode reads
  a.w_idx = const_cast<uint8_t*>(idx);
  a.w_signs = const_cast<uint8_t*>(signs);
  a.w_norm = const_cast<uint16_t*>(norm);
  a.w_rnorm = const_cast<uint16_t*>(rnorm);
  a.w_vcodes = const_cast<uint8_t*>(v_codes);
  a.w_vscale = const_cast<uint16_t*>(v_scale);
  a.w_vzero = const_cast<uint16_t*>(v_zero);
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(n_split, n_quads, B * Hkv);
  if (dispatch(P, v_bits, a, grid, s) != hipSuccess) return TQ_ERR_HIP;
  hipLaunchKernelGGL(merge_kernel, dim3(B * Hq), dim3(KD), 0, s, (const float*)workspace, n_split,
                     out, lse);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // namespace

// ---- the allocation-free variant: the split-K partials live in a device
// array of the library's own, one copy per GPU, held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed to a kernel.
namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(8) << 20;
__device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch[MAX_DEVICES];

// Device address of this device's scratch array, or NULL (status in *st).
void* scratch_of_current_device(tq_status* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    *st = TQ_ERR_HIP;
    return nullptr;
  }
  if (dev < 0 || dev >= MAX_DEVICES) {
    *st = TQ_ERR_UNSUPPORTED;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      *st = TQ_ERR_HIP;
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *st = TQ_OK;
  return p;
}

}  // namespace

extern "C" tq_status tq_decode_attention_noalloc(const tq_key_config* cfg, const void* tables, const void* q,
                                                int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                                const int32_t* ctx_len, int32_t max_ctx, const uint8_t* idx,
                                                const uint8_t* signs, const uint16_t* norm,
                                                const uint16_t* rnorm, int32_t v_bits, int32_t v_group,
                                                const uint8_t* v_codes, const uint16_t* v_scale,
                                                const uint16_t* v_zero, float sm_scale, float* out,
                                                float* lse, float* scores, void* stream) {
  // size of the partials for this shape (a query: nothing is launched)
  size_t need = 0;
  tq_status st = decode_impl(cfg, tables, q, q_dtype, B, Hq, Hkv, ctx_len, max_ctx, nullptr, 0, 0, 0, idx,
                             signs, norm, rnorm, v_bits, v_group, v_codes, v_scale, v_zero, sm_scale, out,
                             lse, scores, nullptr, &need, stream);
  if (st != TQ_OK) return st;
  if (need > NOALLOC_SCRATCH_BYTES) return TQ_ERR_WORKSPACE;
  void* ws = scratch_of_current_device(&st);
  if (!ws) return st;
  size_t have = NOALLOC_SCRATCH_BYTES;
  return decode_impl(cfg, tables, q, q_dtype, B, Hq, Hkv, ctx_len, max_ctx, nullptr, 0, 0, 0, idx, signs, norm,
                     rnorm, v_bits, v_group, v_codes, v_scale, v_zero, sm_scale, out, lse, scores, ws, &have,
                     stream);
}

extern "C" tq_status tq_decode_attention(const tq_key_config* cfg, const void* tables, const void* q,
                                        int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                        const int32_t* ctx_len, int32_t max_ctx, const uint8_t* idx,
                                        const uint8_t* signs, const uint16_t* norm,
                                        const uint16_t* rnorm, int32_t v_bits, int32_t v_group,
                                        const uint8_t* v_codes, const uint16_t* v_scale,
                                        const uint16_t* v_zero, float sm_scale, float* out,
                                        float* lse, float* scores, void* workspace,
                                        size_t* workspace_bytes, void* stream) {
  return decode_impl(cfg, tables, q, q_dtype, B, Hq, Hkv, ctx_len, max_ctx, nullptr, 0, 0, 0, idx, signs,
                     norm, rnorm, v_bits, v_group, v_codes, v_scale, v_zero, sm_scale, out, lse, scores,
                     workspace, workspace_bytes, stream);
}

extern "C" tq_status tq_decode_attention_paged(
    const tq_key_config* cfg, const void* tables, const void* q, int32_t q_dtype, int32_t B, int32_t Hq,
    int32_t Hkv, const int32_t* ctx_len, const int32_t* block_table, int32_t max_blocks_per_seq,
    int32_t page_size, int32_t n_pages, const uint8_t* idx, const uint8_t* signs, const uint16_t* norm,
    const uint16_t* rnorm, int32_t v_bits, int32_t v_group, const uint8_t* v_codes,
    const uint16_t* v_scale, const uint16_t* v_zero, float sm_scale, float* out, float* lse,
    float* scores, void* workspace, size_t* workspace_bytes, void* stream) {
  if (page_size <= 0 || page_size % TILE != 0 || max_blocks_per_seq <= 0 || n_pages <= 0) return TQ_ERR_ARG;
  if ((long long)n_pages * Hkv * page_size > 0x7fffffffffffLL) return TQ_ERR_ARG;
  if ((long long)max_blocks_per_seq * page_size > 0x3fffffffLL) return TQ_ERR_ARG;
  if (workspace && !block_table) return TQ_ERR_ARG;
  return decode_impl(cfg, tables, q, q_dtype, B, Hq, Hkv, ctx_len, max_blocks_per_seq * page_size,
                     block_table, max_blocks_per_seq, page_size, n_pages, idx, signs, norm, rnorm, v_bits, v_group,
                     v_codes, v_scale, v_zero, sm_scale, out, lse, scores, workspace, workspace_bytes,
                     stream);
}

extern "C" tq_status tq_decode_attention_append(const tq_key_config* cfg, const void* tables, const void* q,
                                               int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                               const int32_t* ctx_len, int32_t max_ctx, const void* k_new,
                                               const void* v_new, int32_t kv_dtype, uint8_t* idx,
                                               uint8_t* signs, uint16_t* norm, uint16_t* rnorm,
                                               int32_t v_bits, int32_t v_group, uint8_t* v_codes,
                                               uint16_t* v_scale, uint16_t* v_zero, float sm_scale,
                                               float* out, float* lse, float* scores, void* workspace,
                                               size_t* workspace_bytes, void* stream) {
  if (workspace && (!k_new || !v_new)) return TQ_ERR_ARG;
  return decode_impl(cfg, tables, q, q_dtype, B, Hq, Hkv, ctx_len, max_ctx, nullptr, 0, 0, 0, idx, signs,
                     norm, rnorm, v_bits, v_group, v_codes, v_scale, v_zero, sm_scale, out, lse, scores,
                     workspace, workspace_bytes, stream, k_new, v_new, kv_dtype);
}

extern "C" tq_status tq_decode_attention_paged_append(
    const tq_key_config* cfg, const void* tables, const void* q, int32_t q_dtype, int32_t B, int32_t Hq,
    int32_t Hkv, const int32_t* ctx_len, const int32_t* block_table, int32_t max_blocks_per_seq,
    int32_t page_size, int32_t n_pages, const void* k_new, const void* v_new, int32_t kv_dtype, uint8_t* idx,
    uint8_t* signs, uint16_t* norm, uint16_t* rnorm, int32_t v_bits, int32_t v_group, uint8_t* v_codes,
    uint16_t* v_scale, uint16_t* v_zero, float sm_scale, float* out, float* lse, float* scores, void* workspace,
    size_t* workspace_bytes, void* stream) {
  if (page_size <= 0 || page_size % TILE != 0 || max_blocks_per_seq <= 0 || n_pages <= 0) return TQ_ERR_ARG;
  if ((long long)n_pages * Hkv * page_size > 0x7fffffffffffLL) return TQ_ERR_ARG;
  if ((long long)max_blocks_per_seq * page_size > 0x3fffffffLL) return TQ_ERR_ARG;
  if (workspace && (!block_table || !k_new || !v_new)) return TQ_ERR_ARG;
  return decode_impl(cfg, tables, q, q_dtype, B, Hq, Hkv, ctx_len, max_blocks_per_seq * page_size, block_table,
                     max_blocks_per_seq, page_size, n_pages, idx, signs, norm, rnorm, v_bits, v_group, v_codes,
                     v_scale, v_zero, sm_scale, out, lse, scores, workspace, workspace_bytes, stream, k_new, v_new,
                     kv_dtype);
}
