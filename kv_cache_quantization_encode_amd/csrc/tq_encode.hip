// Key and value encoders for gfx950.
//
// Keys ("tqlite" README, mode table and 设计要点; difai.kr tutorial 算法概述;
// bit-packing article sections 二-四):
//   n = ||k||, y = H (sigma * k) / n  (128-point fast Walsh-Hadamard transform,
//   O(d log d) as the "tqlite" README's 已知限制 asks), idx_j = #{t : y_j >= t},
//   PROD: r = y - c[idx], signs [S r >= 0] (the one dense contraction, on
//   MFMA), rho = n ||r|| / sqrt(d).
//   GROUPED: the same per half of 64 channels (own norm, sigma, codebook).
//   GROUPED_PROD: GROUPED, then the signs of S w for the whole key's residual
//   in the halves' rotated frame, w = concat_j (n_j / 8) r_j (difai.kr
//   tutorial 算法概述: one sketch of k - decompress(k)), rho = ||w||.
// Values (bit-packing article sections 二/三): per-token groups of 32 channels,
// asymmetric min/max with fp16 scale and zero, 2- or 4-bit codes.
//
// Thread mapping of the key encoder.  A wave encodes 16 keys per tile.  Lane l
// works on key (l & 15) and holds 32 of its 128 coordinates in registers x[r]:
// on load, x[8c + i] is coordinate 32c + 8g + i with g = l >> 4.  The
// transform runs five butterfly stages inside each lane (coordinate bits 0, 1,
// 2, 5, 6) and two across lanes (bits 3 and 4) with v_permlane16_swap /
// v_permlane32_swap: each swap hands a lane both inputs of one butterfly, and
// in doing so trades the lane bit for a register bit.  After the transform x[r]
// is coordinate 32g + r, so each lane owns a contiguous quarter of the key:
// exactly the operand layout v_mfma_f32_16x16x32_f16 wants for B = R^T
// (lane l: column l & 15, eight consecutive k per lane group), and a
// contiguous run of packed index bytes.
//
// That is the float32 path.  For bf16 and fp16 keys the loaded words are
// already MFMA operands: register group c of lane (key n, g) holds the eight
// coordinates 32c + 8g .. + 7, the B layout of v_mfma_f32_16x16x32_{bf16,f16}
// for a K step over the 32 coordinates of block c.  The transform's five
// stages on coordinate bits 0-4 then run as one such MFMA per block and
// output half, against a +-1 matrix that also holds sigma (exact products,
// fp32 sums); the stages on bits 5 and 6 stay in the lane.  Afterwards
// x[8c + j] is coordinate 32c + 8g + j: four runs of eight.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <atomic>

#include "tq.h"
#include "tq_internal.h"
#include "tq_tables.h"

namespace {

__device__ inline int index_width_dev(int bits) { return bits == 1 ? 1 : bits == 2 ? 2 : bits <= 4 ? 4 : 8; }

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int KD = 128;        // head dimension of the kernels
constexpr int TILE_KEYS = 16;  // keys per wave tile
constexpr int WAVES = 4;       // waves per block
constexpr int MAX_LEVELS = 256;

struct KeyArgs {
  const unsigned char* tables;
  const void* keys;
  long long n_vec;
  long long row_stride;  // elements
  const long long* slots;
  long long n_records;
  uint8_t* idx;
  uint8_t* signs;
  uint16_t* norm;
  uint16_t* rnorm;
  int idx_row_bytes;
  int n_tiles;
  // the configuration as the host describes it: index bits and storage
  // widths per part, rows of S.  The kernel checks the tables' header against
  // them and stores with these widths, so tables of another configuration
  // cannot make it write past a record.
  int bits0, bits1, w0, w1, m;
};

// The 32 coordinates a lane loads of one key, as loaded (16-bit types: four
// uint4; float32: eight), so that the next tile can be in flight while the
// current one is encoded.
template <int DT>
struct RawKey {
  static constexpr int N = DT == TQ_F32 ? 8 : 4;
  uint4 v[N];
};

template <int DT>
__device__ inline void load_raw(const void* base, long long row_off, int g, RawKey<DT>& r) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (DT == TQ_F32) {
      const uint4* p = (const uint4*)((const float*)base + row_off + 32 * c + 8 * g);
      r.v[2 * c] = p[0];
      r.v[2 * c + 1] = p[1];
    } else {
      r.v[c] = *(const uint4*)((const uint16_t*)base + row_off + 32 * c + 8 * g);
    }
  }
}

// x[r] = sigma_r * (coordinate loaded into register r), the sign applied to
// the bit pattern (sigmask bit r set: sigma_r = -1).  For bfloat16 the low
// element is the shifted word plus the sign bit (adding 2^31 flips bit 31, so
// shift and sign are one operation) and the high element is a mask and an
// xor (again one operation).
template <int DT>
__device__ inline void unpack_raw(const RawKey<DT>& r, uint32_t sigmask, float* x) {
  auto sbit = [&](int i) { return ((sigmask >> i) & 1u) << 31; };
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (DT == TQ_F32) {
      const uint32_t w[8] = {r.v[2 * c].x, r.v[2 * c].y, r.v[2 * c].z, r.v[2 * c].w,
                             r.v[2 * c + 1].x, r.v[2 * c + 1].y, r.v[2 * c + 1].z, r.v[2 * c + 1].w};
#pragma unroll
      for (int k = 0; k < 8; ++k) x[8 * c + k] = __uint_as_float(w[k] ^ sbit(8 * c + k));
    } else {
      const uint32_t w[4] = {r.v[c].x, r.v[c].y, r.v[c].z, r.v[c].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = 8 * c + 2 * k;
        if constexpr (DT == TQ_BF16) {
          x[i] = __uint_as_float((w[k] << 16) + sbit(i));
          x[i + 1] = __uint_as_float((w[k] & 0xFFFF0000u) ^ sbit(i + 1));
        } else {
          x[i] = __uint_as_float(__float_as_uint(__half2float(__ushort_as_half((unsigned short)(w[k] & 0xFFFFu)))) ^ sbit(i));
          x[i + 1] = __uint_as_float(__float_as_uint(__half2float(__ushort_as_half((unsigned short)(w[k] >> 16)))) ^ sbit(i + 1));
        }
      }
    }
  }
}

__device__ inline float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }

// In-lane butterflies on register bit `bit` (stride s = 1 << bit).
template <int S>
__device__ inline void stage_in_lane(float* x) {
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if ((r & S) == 0) {
      float a = x[r], b = x[r + S];
      x[r] = a + b;
      x[r + S] = a - b;
    }
  }
}

// Cross-lane butterflies on lane bit 4 (xor 16, paired with register bit 3)
// and lane bit 5 (xor 32, paired with register bit 4).
__device__ inline void stage_cross16(float* x) {
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if ((r & 8) == 0) {
      auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[r]), __float_as_uint(x[r + 8]),
                                                false, false);
      float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
      x[r] = a + b;
      x[r + 8] = a - b;
    }
  }
}

__device__ inline void stage_cross32(float* x) {
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if ((r & 16) == 0) {
      auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[r]), __float_as_uint(x[r + 16]),
                                                false, false);
      float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
      x[r] = a + b;
      x[r + 16] = a - b;
    }
  }
}

__device__ inline int bucketize(float y, const tq_hint* hint, int hn, float lo, float scale) {
  // grid bin floor((y - lo) * scale) clamped to [0, hn - 1]: clamped first,
  // the conversion's truncation is the floor (NaN -> 0: fmax returns the number)
  const float f = fminf(fmaxf((y - lo) * scale, 0.0f), (float)(hn - 1));
  const tq_hint* h = hint + (int)f;
  return h->h + (y >= h->t_h ? 1 : 0) + (y >= h->t_h1 ? 1 : 0);
}

// Pack 32 indices of width W (coordinates 32g .. 32g+31 of one part) and
// store them at dst (byte offset already applied; 4-byte aligned).
template <int W>
__device__ inline void store_fields(uint8_t* dst, const int* q) {
  constexpr int PER = 32 / W;  // fields per dword
  uint32_t* d = (uint32_t*)dst;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    uint32_t v;
    if constexpr (W <= 2) {
      // sixteen or more fields: one shift-or each (the empty asm keeps the
      // chain from being regrouped into separate shifts and three-input ors)
      v = (uint32_t)q[k * PER + PER - 1];
#pragma unroll
      for (int r = PER - 2; r >= 0; --r) {
        asm("" : "+v"(v));
        v = (v << W) | (uint32_t)q[k * PER + r];
      }
    } else {
      v = 0;
#pragma unroll
      for (int r = 0; r < PER; ++r) v |= (uint32_t)q[k * PER + r] << (W * r);
    }
    d[k] = v;
  }
}

__device__ inline void store_idx(int w, uint8_t* dst, const int* q) {
  switch (w) {
    case 1: store_fields<1>(dst, q); break;
    case 2: store_fields<2>(dst, q); break;
    case 4: store_fields<4>(dst, q); break;
    default: store_fields<8>(dst, q); break;
  }
}

// Pack 8 indices of width w (eight consecutive coordinates) and store their
// w bytes at dst (w-byte aligned).
__device__ __forceinline__ void store_run(int w, uint8_t* dst, const int* q) {
  if (w == 8) {
    uint2 v;
    v.x = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
    v.y = (uint32_t)q[4] | ((uint32_t)q[5] << 8) | ((uint32_t)q[6] << 16) | ((uint32_t)q[7] << 24);
    *(uint2*)dst = v;
    return;
  }
  uint32_t v = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) v |= (uint32_t)q[r] << (w * r);
  if (w == 4) *(uint32_t*)dst = v;
  else if (w == 2) *(uint16_t*)dst = (uint16_t)v;
  else *dst = (uint8_t)v;
}

// The MFMA transform's fixed operand for block c and output half mt (see the
// header): row m of the 16 x 32 A fragment is output coordinate
// 8 (m / 4) + 4 mt + m % 4 of the block, column k input coordinate k, entry
// (-1)^popcount(row & k) times sigma of input 32c + k, as bf16 or fp16 bits.
__device__ inline uint16_t hadamard_entry(int mt, int m, int k, float sigma, bool bf16) {
  const int row = 8 * (m >> 2) + 4 * mt + (m & 3);
  const bool neg = (__popc(row & k) & 1) != (sigma < 0.0f);
  return bf16 ? (neg ? 0xBF80u : 0x3F80u) : (neg ? 0xBC00u : 0x3C00u);
}

// ---------------------------------------------------------------- values
// A wave encodes 16 rows per tile, four at a time: lane l handles 8
// consecutive channels of row 16 tile + 4 j + l / 16; the four lanes of one
// 32-channel group agree on min and max through two xor shuffles.
struct ValArgs {
  const void* values;
  long long n_vec;
  long long row_stride;
  const long long* slots;
  long long n_records;
  uint8_t* codes;
  uint16_t* scale;
  uint16_t* zero;
  long long n_tiles;
};

// a / (2^BITS - 1) rounded to nearest even, for a >= 0, in three operations:
// the quotient by the rounded reciprocal, its remainder (exact by fma), and
// one correction.  For the divisors 3 and 15 this equals the IEEE quotient
// for every finite a >= 0 (checked exhaustively over all 2^31 such floats on
// the host with C fmaf); a = +inf keeps the IEEE result through the select.
template <int BITS>
__device__ inline float div_levels(float a) {
  static_assert(BITS == 2 || BITS == 4, "checked for the divisors 3 and 15");
  constexpr float L = (float)((1 << BITS) - 1);
  constexpr float Y = 1.0f / L;
  const float q0 = a * Y;
  const float r = __builtin_fmaf(-q0, L, a);
  const float q = __builtin_fmaf(r, Y, q0);
  return a == __builtin_huge_valf() ? a : q;
}

// Eight channels of one row as loaded (16-bit types: one uint4; float32: two),
// so that the next tile's rows can be in flight while this one is encoded.
template <int DT>
struct RawRow8 {
  uint4 v[DT == TQ_F32 ? 2 : 1];
};

template <int DT>
__device__ inline void load_row8(const void* base, long long elem_off, RawRow8<DT>& r) {
  if constexpr (DT == TQ_F32) {
    const uint4* p = (const uint4*)((const float*)base + elem_off);
    r.v[0] = p[0];
    r.v[1] = p[1];
  } else {
    r.v[0] = *(const uint4*)((const uint16_t*)base + elem_off);
  }
}

template <int DT>
__device__ inline void unpack_row8(const RawRow8<DT>& r, float* out) {
  if constexpr (DT == TQ_F32) {
    const uint32_t w[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w, r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = __uint_as_float(w[k]);
  } else {
    const uint32_t w[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (DT == TQ_BF16) {
        out[2 * k] = __uint_as_float(w[k] << 16);
        out[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      } else {
        out[2 * k] = __half2float(__ushort_as_half((unsigned short)(w[k] & 0xFFFFu)));
        out[2 * k + 1] = __half2float(__ushort_as_half((unsigned short)(w[k] >> 16)));
      }
    }
  }
}

// Block `bid` of `nb` blocks (of 256 threads) that share the value tiles.
// Each wave requests its next tile's rows before encoding the current one, so
// that two tiles per wave are in flight.
template <int BITS, int DT>
__device__ __forceinline__ void encode_values_body(const ValArgs& a, int bid, int nb) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15;          // 8-channel chunk within the row
  const long long tiles_per_grid = (long long)nb * (blockDim.x >> 6);
  RawRow8<DT> raw[4], raw_next[4];
  auto request = [&](long long tile, RawRow8<DT>* r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long long row = tile * 16 + 4 * j + (lane >> 4);
      const long long rr = row < a.n_vec ? row : a.n_vec - 1;
      load_row8<DT>(a.values, rr * a.row_stride + 8 * sub, r[j]);
    }
  };
  long long tile = (long long)bid * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (tile < a.n_tiles) request(tile, raw);
  for (; tile < a.n_tiles; tile += tiles_per_grid) {
    if (tile + tiles_per_grid < a.n_tiles) request(tile + tiles_per_grid, raw_next);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long long row = tile * 16 + 4 * j + (lane >> 4);
      const bool valid = row < a.n_vec;
      float v[8];
      unpack_row8<DT>(raw[j], v);
      float mn = v[0], mx = v[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, v[i]);
        mx = fmaxf(mx, v[i]);
      }
      // the four lanes of a group: xor-1 and xor-2 exchanges
      mn = fminf(mn, __shfl_xor(mn, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mn = fminf(mn, __shfl_xor(mn, 2));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      constexpr float LEVELS = (float)((1 << BITS) - 1);
      const float s32 = div_levels<BITS>(__fsub_rn(mx, mn));
      const __half s16 = __float2half_rn(s32);
      const __half z16 = __float2half_rn(mn);
      const float s = __half2float(s16), z = __half2float(z16);
      // code = rint((v - z) / s) with the correctly rounded quotient.  x * rcp(s)
      // lies within 2^-22 |q| of the exact quotient, and so does the rounded
      // one.  Quotients that matter lie in [-1, 2^BITS], so unless q is within
      // 1e-5 of a half-integer both round to the same code; such a code is
      // redone with a full division.
      const float rs = __builtin_amdgcn_rcpf(s);
      float c[8], x[8];
      float dev[8];  // |q - rint(q)| per channel
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = __fsub_rn(v[i], z);
        const float q = x[i] * rs;
        c[i] = rintf(q);
        dev[i] = fabsf(q - c[i]);
      }
      // Per channel, so that a wave divides only where one of its lanes has
      // that channel near a half-integer (bf16 inputs often put a quotient
      // exactly on one; divisions for all eight channels would be taken by
      // about a quarter of the row groups).
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (dev[i] > 0.5f - 1e-5f) c[i] = rintf(__fdiv_rn(x[i], s));
      uint32_t packed = 0;
      if (s != 0.0f) {
        // codes packed in float arithmetic: c 2^(BITS i) is exact below 2^24
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo = fmaf(__builtin_amdgcn_fmed3f(c[i], 0.0f, LEVELS), (float)(1u << (BITS * i)), lo);
          hi = fmaf(__builtin_amdgcn_fmed3f(c[4 + i], 0.0f, LEVELS), (float)(1u << (BITS * i)), hi);
        }
        packed = (uint32_t)lo | ((uint32_t)hi << (4 * BITS));
      }
      // destination record (the slot table is read here, where it is used)
      const long long slot = !valid ? -1 : a.slots ? a.slots[row] : row;
      if (slot >= 0 && slot < a.n_records) {
        if (BITS == 2) {
          *(uint16_t*)(a.codes + slot * (KD * BITS / 8) + 2 * sub) = (uint16_t)packed;
        } else {
          *(uint32_t*)(a.codes + slot * (KD * BITS / 8) + 4 * sub) = packed;
        }
        if ((sub & 3) == 0) {
          a.scale[slot * (KD / 32) + (sub >> 2)] = __half_as_ushort(s16);
          a.zero[slot * (KD / 32) + (sub >> 2)] = __half_as_ushort(z16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = raw_next[j];
  }
}

// Launch kinds of the key encoder: one key set; up to MAX_KEY_BATCH sets, each
// with its own tables (entries take consecutive runs of blocks_per_entry
// blocks); or one key set and the value rows of the same tokens (the first
// key_blocks blocks take the keys, the rest the values).  The encoder body is
// written once, in the kernel itself: moved into a device function it was
// compiled to 198 instead of 166 VGPRs (2 instead of 3 waves per SIMD).
enum { KEYS_ONE = 0, KEYS_BATCH = 1, KEYS_AND_VALUES = 2 };
constexpr int MAX_KEY_BATCH = 32;
template <int KIND> struct KeyLaunch { KeyArgs k; };
template <> struct KeyLaunch<KEYS_BATCH> {
  KeyArgs e[MAX_KEY_BATCH];  // read in place from the kernel arguments
  int blocks_per_entry;
};
template <> struct KeyLaunch<KEYS_AND_VALUES> {
  KeyArgs k;
  ValArgs v;
  int key_blocks;
};
static_assert(sizeof(KeyLaunch<KEYS_BATCH>) <= 4096, "kernel arguments stay within 4 KiB");

template <int KIND>
__device__ __forceinline__ const KeyArgs& key_set(const KeyLaunch<KIND>& L, int ent) {
  if constexpr (KIND == KEYS_BATCH) return L.e[ent];
  else return L.k;
}

// MODE: TQ_MODE_MSE / PROD / GROUPED / GROUPED_PROD.  DT: input dtype.  VB: value bits
// (KEYS_AND_VALUES only).
// Waves per SIMD the register allocation is held to: three (at most 168
// VGPRs) for 16-bit inputs in MSE and PROD mode; two for GROUPED and float32
// inputs, which need more registers and would spill at three.
constexpr bool grouped_mode(int mode) { return mode == TQ_MODE_GROUPED || mode == TQ_MODE_GROUPED_PROD; }
constexpr bool qjl_mode(int mode) { return mode == TQ_MODE_PROD || mode == TQ_MODE_GROUPED_PROD; }
constexpr int key_waves_per_simd(int mode, int dt) { return grouped_mode(mode) || dt == TQ_F32 ? 2 : qjl_mode(mode) ? 3 : 4; }
// Waves per key-encoder block: eight for the MSE encoder of 16-bit keys (at
// most 128 VGPRs, four waves per SIMD, two blocks per CU sharing the LDS of
// two), four otherwise (LDS holds three blocks per CU).  Launches that mix key
// and value blocks use four.
constexpr int key_block_waves(int mode, int dt, int kind) {
  return kind != KEYS_AND_VALUES && mode == TQ_MODE_MSE && dt != TQ_F32 ? 8 : 4;
}

template <int MODE, int DT, int KIND, int VB>
__global__ __launch_bounds__(key_block_waves(MODE, DT, KIND) * 64, key_waves_per_simd(MODE, DT)) void encode_keys_kernel(KeyLaunch<KIND> L) {
  constexpr int WAVES = key_block_waves(MODE, DT, KIND);
  if constexpr (KIND == KEYS_AND_VALUES) {
    if ((int)blockIdx.x >= L.key_blocks) {
      encode_values_body<VB, DT>(L.v, blockIdx.x - L.key_blocks, gridDim.x - L.key_blocks);
      return;
    }
  }
  int ent = 0, bid = blockIdx.x, nb = gridDim.x;
  if constexpr (KIND == KEYS_BATCH) {
    ent = blockIdx.x / L.blocks_per_entry;
    bid = blockIdx.x - ent * L.blocks_per_entry;
    nb = L.blocks_per_entry;
  } else if constexpr (KIND == KEYS_AND_VALUES) {
    nb = L.key_blocks;
  }
  const KeyArgs& a = key_set<KIND>(L, ent);
  const tq_blob_header* H = (const tq_blob_header*)a.tables;
  constexpr bool GRP = grouped_mode(MODE), QJL = qjl_mode(MODE);
  constexpr int NP = GRP ? 2 : 1;
  // tables of another configuration: nothing is written (uniform per block)
  if (H->magic != TQ_BLOB_MAGIC || H->d != KD || H->mode != MODE || H->n_parts != NP ||
      H->part_bits[0] != a.bits0 || (NP == 2 && H->part_bits[1] != a.bits1) || H->m != a.m ||
      H->hint_n[0] > TQ_MAX_HINT || (NP == 2 && H->hint_n[1] > TQ_MAX_HINT))
    return;
  __shared__ __align__(16) tq_hint s_hint[NP][TQ_MAX_HINT];
  __shared__ float s_cent[QJL ? NP * MAX_LEVELS : 1];
  constexpr int SPITCH = KD + 8;  // halves per padded row of S
  __shared__ __align__(16) _Float16 s_S[QJL ? KD * SPITCH : 8];
  constexpr bool MF = DT != TQ_F32;  // transform bits 0-4 on MFMA (16-bit inputs)
  // A fragments of the transform: [block c][half mt][lane][8]
  __shared__ __align__(16) uint16_t s_H[MF ? 4 * 2 * 64 * 8 : 8];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;     // lane group: quarter of the key
  const int kk = lane & 15;    // key within the tile

  // Rows past n_vec load the last row (kept in bounds) and are encoded but
  // never stored; keys do not mix in any step, the projection included.
  const int tile_step = nb * WAVES;
  auto row_of = [&](int tile) {
    const long long row = (long long)tile * TILE_KEYS + kk;
    return row < a.n_vec ? row : a.n_vec - 1;
  };
  // This wave's first tile goes out before the tables are staged.
  RawKey<DT> raw, raw_next;
  int tile = bid * WAVES + wave;
  if (tile < a.n_tiles) load_raw<DT>(a.keys, row_of(tile) * a.row_stride, g, raw);

  // Bucketize.  Formats with two or four cells and one part ("direct") take
  // the index arithmetically; all others look up a hint grid in LDS.  Those
  // small codebooks are symmetric (Gaussian Lloyd-Max), so their cells are
  // equally wide about zero: boundaries {0} (two cells) or {-t, 0, t} (four
  // cells).  The index is then [y >= 0], taken as [x >= 0] on the unscaled
  // coordinate x = n y (exact), resp. floor(y / t + 2), taken as
  // floor(clamp(fma(x, 1 / (t n), 2), 0, 3)): three operations per
  // coordinate, differing from the count of boundaries at or below y only
  // where y is within a few ulps of a boundary.  A table that is not
  // symmetric goes to the hint grid instead.
  const int lev0 = H->part_levels[0];
  const float* bnd = (const float*)(a.tables + H->off_bounds[0]);
  const float bt0 = bnd[0], bt1 = bnd[1], bt2 = bnd[2];
  const bool direct2 = NP == 1 && lev0 == 2 && bt0 == 0.0f;
  const bool direct = direct2 || (NP == 1 && lev0 == 4 && bt1 == 0.0f && bt2 > 0.0f && bt0 == -bt2);
  const float ua = 1.0f / bt2, ub = 2.0f;
  const float utop = (float)(lev0 - 1);
  // sigma of the coordinates loaded into x[r]: 32 (r >> 3) + 8 g + (r & 7)
  float4 sg[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = 32 * c + 8 * g;
    const int part = GRP ? j / (KD / 2) : 0;
    const float4* sp = (const float4*)((const float*)(a.tables + H->off_sigma[part]) + (j - part * (KD / 2)));
    sg[2 * c] = sp[0];
    sg[2 * c + 1] = sp[1];
  }
  // The other staged tables (rows of S, centroids, sigma for the transform's
  // A fragments) are read into registers here, all at once, and written to
  // LDS further down: a launch of a few tiles per block (an append) waits on
  // this staging, so it is one round of global reads rather than a chain.
  constexpr int NT = WAVES * 64;
  static_assert(MAX_LEVELS <= NT, "one centroid per thread");
  constexpr int S_PER_THREAD = KD * KD / 8 / NT;
  uint4 srow[QJL ? S_PER_THREAD : 1];
  float cv[NP];
  if constexpr (QJL) {
    const uint4* S = (const uint4*)(a.tables + H->off_S);
#pragma unroll
    for (int k = 0; k < S_PER_THREAD; ++k) srow[k] = S[threadIdx.x + k * NT];
    // at most MAX_LEVELS (<= NT) centroids per part: one per thread
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float* c = (const float*)(a.tables + H->off_centroids[p]);
      cv[p] = (int)threadIdx.x < min(H->part_levels[p], MAX_LEVELS) ? c[threadIdx.x] : 0.0f;
    }
  }
  constexpr int H_PER_THREAD = 4 * 2 * 64 * 8 / NT;
  float svh[MF ? H_PER_THREAD : 1];
  if constexpr (MF) {
#pragma unroll
    for (int m = 0; m < H_PER_THREAD; ++m) {
      const int i = threadIdx.x + m * NT;
      const int c = i >> 10, ln = (i >> 3) & 63, e = i & 7;
      const int k = 8 * (ln >> 4) + e;
      const int part = GRP ? c >> 1 : 0;
      const int j = GRP ? 32 * (c & 1) + k : 32 * c + k;  // coordinate within the part
      svh[m] = ((const float*)(a.tables + H->off_sigma[part]))[j];
    }
  }
  int hn[NP];
  float hlo[NP], hsc[NP];
  for (int p = 0; p < NP; ++p) {
    hn[p] = H->hint_n[p];
    hlo[p] = H->hint_lo[p];
    hsc[p] = H->hint_scale[p];
    if (!direct) {
      const uint4* src = (const uint4*)(a.tables + H->off_hint[p]);
      constexpr int PER_THREAD = TQ_MAX_HINT / (WAVES * 64);
      // (unconditional reads of clamped entries keep hv in registers)
      const int last = max(hn[p], 1) - 1;
      uint4 hv[PER_THREAD];
#pragma unroll
      for (int k = 0; k < PER_THREAD; ++k) hv[k] = src[min((int)threadIdx.x + k * WAVES * 64, last)];
#pragma unroll
      for (int k = 0; k < PER_THREAD; ++k) {
        const int i = threadIdx.x + k * WAVES * 64;
        if (i < hn[p]) *(uint4*)&s_hint[p][i] = hv[k];
      }
    }
  }
  if constexpr (QJL) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
      if ((int)threadIdx.x < min(H->part_levels[p], MAX_LEVELS)) s_cent[p * MAX_LEVELS + threadIdx.x] = cv[p];
    // S in LDS, rows padded to 136 halves so that the sixteen rows one MFMA
    // fragment read touches fall in distinct banks.  Fragment (nt, ks) of lane
    // (kk, g): row 16 nt + kk, coordinates 32 g + 8 ks .. + 7 (float32 path)
    // or 32 ks + 8 g .. + 7 (MFMA path), matching the B = R^T layout after
    // the transform.
#pragma unroll
    for (int k = 0; k < S_PER_THREAD; ++k) {
      const int i = threadIdx.x + k * NT;
      *(uint4*)(s_S + (i / (KD / 8)) * SPITCH + 8 * (i % (KD / 8))) = srow[k];
    }
  }
  if constexpr (MF) {
#pragma unroll
    for (int m = 0; m < H_PER_THREAD; ++m) {
      const int i = threadIdx.x + m * NT;
      const int mt = (i >> 9) & 1, ln = (i >> 3) & 63, e = i & 7;
      s_H[i] = hadamard_entry(mt, ln & 15, 8 * (ln >> 4) + e, svh[m], DT == TQ_BF16);
    }
  }
  // sign mask: bit r set when sigma of the coordinate loaded into x[r] is -1
  uint32_t sigmask = 0;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const float4 v = sg[r >> 2];
    const float sv = (r & 3) == 0 ? v.x : (r & 3) == 1 ? v.y : (r & 3) == 2 ? v.z : v.w;
    if (sv < 0) sigmask |= 1u << r;
  }
  __syncthreads();

  const float inv_sqrt_d = 1.0f / sqrtf((float)KD);
  const int w0 = a.w0;
  const int w1 = NP == 2 ? a.w1 : 0;

  for (; tile < a.n_tiles; tile += tile_step) {
    // the next tile of this wave is requested before this one is encoded
    if (tile + tile_step < a.n_tiles) load_raw<DT>(a.keys, row_of(tile + tile_step) * a.row_stride, g, raw_next);
    const long long row = (long long)tile * TILE_KEYS + kk;
    const bool valid = row < a.n_vec;
    const long long slot = a.slots ? a.slots[row_of(tile)] : row;
    float x[32];
    if constexpr (MF) {
      // coordinate bits 0-4 of each block c by MFMA (see the header): the
      // loaded words of block c are the B operand, fragment (c, mt) of the
      // +-1 matrix with sigma the A operand; output half mt of block c lands
      // in x[8c + 4mt .. + 3] as coordinates 32c + 8g + 4mt .. + 3
      const uint4* hfr = (const uint4*)s_H + lane;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint4 af = hfr[(2 * c + mt) * 64];
          floatx4 d;
          if constexpr (DT == TQ_BF16)
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                        __builtin_bit_cast(bf16x8, raw.v[c]),
                                                        floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          else
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, af), __builtin_bit_cast(half8, raw.v[c]),
                                                       floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) x[8 * c + 4 * mt + i] = d[i];
        }
      }
      raw = raw_next;
      stage_in_lane<8>(x);              // coordinate bit 5
      if (!GRP) stage_in_lane<16>(x);   // coordinate bit 6
    } else {
      unpack_raw<DT>(raw, sigmask, x);
      raw = raw_next;
    }
    // squared norm per part (part = register bit 4 in both layouts); after the
    // MFMA transform the sums are of y = H (sigma k), PD times those of k
    float ss0 = 0.0f, ss1 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ss0 = fmaf(x[r], x[r], ss0);
      ss1 = fmaf(x[r + 16], x[r + 16], ss1);
    }
    ss0 = xor_sum(xor_sum(ss0, 16), 32);
    ss1 = xor_sum(xor_sum(ss1, 16), 32);
    // A sum of squares outside [2^-100, 2^100] may have lost range (fp32
    // squares underflow for keys below about 1e-19 and overflow above about
    // 1.8e19; zero keys come here too): it is redone on the coordinates
    // scaled by the power of two that brings the largest into [1, 2), and
    // the norm scaled back.  Decided per wave, so ordinary tiles pay one test.
    float nsc0 = 1.0f, nsc1 = 1.0f;  // norm = sqrt(ss) * nsc
    {
      const float st = GRP ? fminf(ss0, ss1) : ss0 + ss1;
      const float sb = GRP ? fmaxf(ss0, ss1) : ss0 + ss1;
      const bool odd = !(st >= 0x1p-100f && sb <= 0x1p100f);
      if (__builtin_amdgcn_ballot_w64(odd) != 0) {
        float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          m0 = fmaxf(m0, fabsf(x[r]));
          m1 = fmaxf(m1, fabsf(x[r + 16]));
        }
        m0 = fmaxf(m0, __shfl_xor(m0, 16));
        m0 = fmaxf(m0, __shfl_xor(m0, 32));
        m1 = fmaxf(m1, __shfl_xor(m1, 16));
        m1 = fmaxf(m1, __shfl_xor(m1, 32));
        if (!GRP) m0 = m1 = fmaxf(m0, m1);
        const int e0 = m0 > 0.0f ? max(ilogbf(m0), -126) : 0;
        const int e1 = m1 > 0.0f ? max(ilogbf(m1), -126) : 0;
        const float s0 = ldexpf(1.0f, -e0), s1 = ldexpf(1.0f, -e1);
        ss0 = 0.0f;
        ss1 = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float u0 = x[r] * s0, u1 = x[r + 16] * s1;
          ss0 = fmaf(u0, u0, ss0);
          ss1 = fmaf(u1, u1, ss1);
        }
        ss0 = xor_sum(xor_sum(ss0, 16), 32);
        ss1 = xor_sum(xor_sum(ss1, 16), 32);
        nsc0 = ldexpf(1.0f, e0);
        nsc1 = ldexpf(1.0f, e1);
      }
    }

    if constexpr (!MF) {
      stage_in_lane<1>(x);
      stage_in_lane<2>(x);
      stage_in_lane<4>(x);
      stage_in_lane<8>(x);
      if (!GRP) stage_in_lane<16>(x);
      stage_cross16(x);
      stage_cross32(x);
      // now x[r] is coordinate 32g + r
    }
    // (1/PD is a power of two: the sums scale exactly)
    constexpr float INV_PD = MF ? (GRP ? 1.0f / 64.0f : 1.0f / 128.0f) : 1.0f;
    float n_part[2];
    if (GRP) {
      n_part[0] = sqrtf(ss0 * INV_PD) * nsc0;
      n_part[1] = sqrtf(ss1 * INV_PD) * nsc1;
    } else {
      n_part[0] = n_part[1] = sqrtf((ss0 + ss1) * INV_PD) * nsc0;
    }
    // the part of register r: lane group (float32 layout) or register bit 4
    auto part_of = [&](int r) { return GRP ? (MF ? (r >> 4) : (g >> 1)) : 0; };
    const float inv_p[2] = {n_part[0] > 0.0f ? 1.0f / n_part[0] : 0.0f, n_part[1] > 0.0f ? 1.0f / n_part[1] : 0.0f};
    const float n = n_part[0], inv = inv_p[0];  // single-part modes
    // x stays unscaled (y = x / n = x * inv where needed)
    int q[32];
    if (direct2) {
#pragma unroll
      for (int r = 0; r < 32; ++r) q[r] = x[r] >= 0.0f ? 1 : 0;
    } else if (direct) {
      // symmetric four-cell codebook (see above); clamped to [0, levels - 1]
      // first, the conversion's truncation is the floor.  A zero key (n = 0)
      // gets fma(0, 0, ub): the cell of y = 0.
      const float un = ua * inv;
#pragma unroll
      for (int r = 0; r < 32; ++r) q[r] = (int)__builtin_amdgcn_fmed3f(fmaf(x[r], un, ub), 0.0f, utop);
    } else {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        // eight hint reads in flight at a time (each holds three registers)
        if (r % 8 == 0) __builtin_amdgcn_sched_barrier(0);
        const int pr = NP == 2 ? part_of(r) : 0;
        q[r] = bucketize(x[r] * inv_p[pr], s_hint[pr], hn[pr], hlo[pr], hsc[pr]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    const bool store = valid && slot >= 0 && slot < a.n_records;

    if (store) {
      uint8_t* dst = a.idx + slot * a.idx_row_bytes;
      if constexpr (MF) {
        // four runs of eight coordinates, 32c + 8g .. + 7
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int pc = GRP ? c >> 1 : 0;
          const int w = pc ? w1 : w0;
          const int cs = GRP ? 32 * (c & 1) + 8 * g : 32 * c + 8 * g;  // first coordinate within the part
          store_run(w, dst + (pc ? (KD / 2) * w0 / 8 : 0) + cs * w / 8, q + 8 * c);
        }
      } else if (GRP) {
        const int part = g >> 1;
        const int w = part ? w1 : w0;
        const int off = part ? (KD / 2) * w0 / 8 + 32 * (g - 2) * w / 8 : 32 * g * w / 8;
        store_idx(w, dst + off, q);
      } else {
        store_idx(w0, dst + 32 * g * w0 / 8, q);
      }
      if (g == 0) {
        if (GRP) {
          const uint32_t pk = (uint32_t)__half_as_ushort(__float2half_rn(n_part[0])) |
                              ((uint32_t)__half_as_ushort(__float2half_rn(n_part[1])) << 16);
          *(uint32_t*)(a.norm + 2 * slot) = pk;
        } else {
          a.norm[slot] = __half_as_ushort(__float2half_rn(n));
        }
      }
    }

    if constexpr (QJL) {
      // GROUPED_PROD weights each half's residual by n_j / max(n_o, n_n):
      // w / (max / 8), in [0, 1] times the residual's own scale for fp16
      float wgt_p[2] = {1.0f, 1.0f}, nmax = n;
      if constexpr (GRP) {
        nmax = fmaxf(n_part[0], n_part[1]);
        wgt_p[0] = nmax > 0.0f ? n_part[0] / nmax : 0.0f;
        wgt_p[1] = nmax > 0.0f ? n_part[1] / nmax : 0.0f;
      }
      // residual split into fp16 hi + lo, two coordinates at a time: hi
      // rounded toward zero (any hi works: res - hi is then below hi's ulp and
      // of res's sign, so lo carries the next 11 bits), lo = res - hi as one
      // mixed-precision fma per coordinate
      float rr = 0.0f;
      half8 bhi[4], blo[4];
#pragma unroll
      for (int r = 0; r < 32; r += 2) {
        float res[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int pr = part_of(r + e);
          res[e] = fmaf(x[r + e], inv_p[pr], -s_cent[pr * MAX_LEVELS + q[r + e]]);
          if constexpr (GRP) res[e] *= wgt_p[pr];
          rr = fmaf(res[e], res[e], rr);
        }
        const auto h2 = __builtin_amdgcn_cvt_pkrtz(res[0], res[1]);
        const uint32_t hw = __builtin_bit_cast(uint32_t, h2);
        float l0, l1;  // res - hi, each from one half of hw (exact)
        asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l0) : "v"(hw), "v"(res[0]));
        asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(l1) : "v"(hw), "v"(res[1]));
        const auto lo2 = __builtin_amdgcn_cvt_pkrtz(l0, l1);
        bhi[r >> 3][r & 7] = (_Float16)h2[0];
        bhi[r >> 3][(r & 7) + 1] = (_Float16)h2[1];
        blo[r >> 3][r & 7] = (_Float16)lo2[0];
        blo[r >> 3][(r & 7) + 1] = (_Float16)lo2[1];
      }
      rr = xor_sum(xor_sum(rr, 16), 32);
      // The fragment offset is made opaque to the compiler each tile, so that it
      // reads S from LDS per use instead of keeping all 32 fragments live (an
      // offset, not a pointer, so the reads stay LDS reads and not flat ones).
      // K step ks covers the lane's register group ks: coordinates 32g + 8ks
      // (float32 layout) or 32ks + 8g (MFMA layout) .. + 7.
      int soff = kk * SPITCH + (MF ? 8 : 32) * g;
      asm volatile("" : "+v"(soff));
      const _Float16* sbase = s_S + soff;
      floatx4 acc[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        acc[nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const half8 sf = *(const half8*)(sbase + (16 * nt) * SPITCH + (MF ? 32 : 8) * ks);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sf, blo[ks], acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(sf, bhi[ks], acc[nt], 0, 0, 0);
        }
      }
      // Lane holds projections of key kk onto S rows 16nt + 4g + i.  Their
      // sign bits, shifted in one per funnel shift from (nt, i) = (7, 3) down
      // to (0, 0), give T with bit 4nt + i set for a negative projection
      // (bit = [z >= 0] is its complement; z = -0 reads as negative, a case
      // within the zero band).
      uint32_t T = 0;
#pragma unroll
      for (int nt = 7; nt >= 0; --nt)
#pragma unroll
        for (int i = 3; i >= 0; --i) T = __builtin_amdgcn_alignbit(T, __float_as_uint(acc[nt][i]), 31);
      T = ~T;
      // Sign dword w of the key holds rows 32w .. 32w+31: nibble 2w of T at
      // bit 4g and nibble 2w+1 at bit 16 + 4g, from each lane group g.
      uint32_t dw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t byte = (T >> (8 * w)) & 0xFFu;
        dw[w] = ((byte | (byte << 12)) & 0x000F000Fu) << (4 * g);
      }
      // OR over the four lane groups, lane group g keeping dword g: swap
      // halves with the group two away, then single dwords with the neighbour.
      const int hg = g >> 1, bg = g & 1;
      const uint32_t keep0 = hg ? dw[2] : dw[0], keep1 = hg ? dw[3] : dw[1];
      const uint32_t give0 = hg ? dw[0] : dw[2], give1 = hg ? dw[1] : dw[3];
      const uint32_t m0 = keep0 | __shfl_xor(give0, 32), m1 = keep1 | __shfl_xor(give1, 32);
      const uint32_t mine = (bg ? m1 : m0) | __shfl_xor(bg ? m0 : m1, 16);
      if (store) {
        *(uint32_t*)(a.signs + slot * (KD / 8) + 4 * g) = mine;
        if (g == 0) {
          // rho = n ||r|| / sqrt(d), or ||w|| = max ||w / (max / 8)|| / 8
          const float rho = GRP ? nmax * sqrtf(rr) * 0.125f : n * sqrtf(rr) * inv_sqrt_d;
          a.rnorm[slot] = __half_as_ushort(__float2half_rn(rho));
        }
      }
    }
  }
}

template <int BITS, int DT>
__global__ __launch_bounds__(256) void encode_values_kernel(ValArgs a) {
  encode_values_body<BITS, DT>(a, blockIdx.x, gridDim.x);
}

int grid_for(long long tiles, int per_block) {
  long long blocks = (tiles + per_block - 1) / per_block;
  const long long cap = 256LL * 8;  // enough to fill 256 CUs several times
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

#ifndef TQ_VAL_ROUNDS
#define TQ_VAL_ROUNDS 1
#endif
// Blocks of the value encoder: one per four tiles, at most as many as the
// device holds at once.  The blocks loop over the tiles, so a block that had
// to wait for a free slot would run its whole share late.
template <int BITS, int DT>
int value_blocks(long long tiles, int cus) {
  static std::atomic<int> resident{0};  // blocks per CU (occupancy of the kernel)
  int r = resident.load(std::memory_order_relaxed);
  if (r <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, encode_values_kernel<BITS, DT>, 256, 0) != hipSuccess ||
        r <= 0) {
      (void)hipGetLastError();
      r = 4;
    }
    resident.store(r, std::memory_order_relaxed);
  }
  long long blocks = (tiles + 3) / 4;
  const long long cap = (long long)cus * r * TQ_VAL_ROUNDS;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

template <int BITS, int DT>
void launch_values(const ValArgs& a, int cus, hipStream_t s) {
  hipLaunchKernelGGL((encode_values_kernel<BITS, DT>), dim3(value_blocks<BITS, DT>(a.n_tiles, cus)), dim3(256), 0,
                     s, a);
}

// Argument checks and kernel arguments of the key encoder.  Returns TQ_OK with
// *empty set when there is nothing to encode (n_vec == 0).
tq_status key_args(const tq_key_config* cfg, const void* tables, const void* keys, int32_t dtype,
                   int64_t n_vec, int64_t row_stride, const int64_t* slots, int64_t n_records,
                   uint8_t* idx, uint8_t* signs, uint16_t* norm, uint16_t* rnorm, tq::Parts& P,
                   KeyArgs& a, bool& empty) {
  tq_status st = tq::describe(cfg, &P);
  if (st != TQ_OK) return st;
  if (P.d != KD) return TQ_ERR_UNSUPPORTED;
  if (n_vec < 0 || n_records < 0) return TQ_ERR_ARG;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_ERR_ARG;
  empty = n_vec == 0;
  if (empty) return TQ_OK;
  if (!tables || !keys || !idx || !norm) return TQ_ERR_ARG;
  const int esz = dtype == TQ_F32 ? 4 : 2;
  if (row_stride < KD || ((row_stride * esz) & 15) || !tq::aligned16(keys)) return TQ_ERR_ARG;
  if (!tq::aligned16(tables) || !tq::aligned16(idx) || ((uintptr_t)norm & 3)) return TQ_ERR_ARG;
  if (P.m > 0) {
    if (!signs || !rnorm || !tq::aligned16(signs) || ((uintptr_t)rnorm & 1)) return TQ_ERR_ARG;
  } else if (signs || rnorm) {
    return TQ_ERR_ARG;
  }
  if (slots && ((uintptr_t)slots & 7)) return TQ_ERR_ARG;
  for (int p = 0; p < P.n_parts; ++p)
    if (P.part_width[p] * P.part_d[p] / 8 % 4) return TQ_ERR_UNSUPPORTED;
  const long long tiles = (n_vec + TILE_KEYS - 1) / TILE_KEYS;
  if (tiles > 0x7fffffffLL) return TQ_ERR_ARG;
  a.tables = (const unsigned char*)tables;
  a.keys = keys;
  a.n_vec = n_vec;
  a.row_stride = row_stride;
  a.slots = (const long long*)slots;
  a.n_records = n_records;
  a.idx = idx;
  a.signs = signs;
  a.norm = norm;
  a.rnorm = rnorm;
  a.idx_row_bytes = P.idx_row_bytes;
  a.n_tiles = (int)tiles;
  a.bits0 = P.part_bits[0];
  a.bits1 = P.n_parts > 1 ? P.part_bits[1] : 0;
  a.w0 = P.part_width[0];
  a.w1 = P.n_parts > 1 ? P.part_width[1] : 0;
  a.m = P.m;
  return TQ_OK;
}

// Key-encoder blocks: a few per CU, each wave looping over tiles so that a
// block's table staging is paid once for several tiles and the next tile's
// load overlaps the current one.  Measured on MI355X: two blocks per CU suit
// the MSE and grouped encoders (launches of 65536 keys are dominated by that
// staging), eight the prod encoder (long launches, where more blocks in
// flight keep the loads and the MFMA work overlapped).
int key_blocks(const tq::Parts& P, int n_tiles, int cus, int kw) {
  const long long want = ((long long)n_tiles + kw - 1) / kw;
  const long long cap = (long long)cus * (P.m > 0 ? 8 : 2);
  return (int)(want < cap ? want : cap);
}

tq_status val_args(int32_t bits, int32_t group, int32_t d, const void* values, int32_t dtype,
                   int64_t n_vec, int64_t row_stride, const int64_t* slots, int64_t n_records,
                   uint8_t* codes, uint16_t* scale, uint16_t* zero, ValArgs& a, bool& empty) {
  if (bits != 2 && bits != 4) return TQ_ERR_UNSUPPORTED;
  if (group != 32 || d != KD) return TQ_ERR_UNSUPPORTED;
  if (n_vec < 0 || n_records < 0) return TQ_ERR_ARG;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_ERR_ARG;
  empty = n_vec == 0;
  if (empty) return TQ_OK;
  if (!values || !codes || !scale || !zero) return TQ_ERR_ARG;
  const int esz = dtype == TQ_F32 ? 4 : 2;
  if (row_stride < KD || ((row_stride * esz) & 15) || !tq::aligned16(values)) return TQ_ERR_ARG;
  if (!tq::aligned16(codes) || ((uintptr_t)scale & 1) || ((uintptr_t)zero & 1)) return TQ_ERR_ARG;
  if (slots && ((uintptr_t)slots & 7)) return TQ_ERR_ARG;
  a.values = values;
  a.n_vec = n_vec;
  a.row_stride = row_stride;
  a.slots = (const long long*)slots;
  a.n_records = n_records;
  a.codes = codes;
  a.scale = scale;
  a.zero = zero;
  a.n_tiles = (n_vec + 15) / 16;
  return TQ_OK;
}

}  // namespace

extern "C" tq_status tq_encode_keys(const tq_key_config* cfg, const void* tables, const void* keys,
                                   int32_t dtype, int64_t n_vec, int64_t row_stride,
                                   const int64_t* slots, int64_t n_records, uint8_t* idx,
                                   uint8_t* signs, uint16_t* norm, uint16_t* rnorm, void* stream) {
  tq::Parts P;
  KeyArgs a;
  bool empty = false;
  tq_status st = key_args(cfg, tables, keys, dtype, n_vec, row_stride, slots, n_records, idx, signs, norm,
                          rnorm, P, a, empty);
  if (st != TQ_OK || empty) return st;
  const int cus = tq::cu_count();
  if (cus <= 0) return TQ_ERR_HIP;
  const int kw = key_block_waves(P.mode, dtype, KEYS_ONE);
  const dim3 grid((unsigned)key_blocks(P, a.n_tiles, cus, kw)), block(kw * 64);
  hipStream_t s = (hipStream_t)stream;
  const KeyLaunch<KEYS_ONE> L{a};
#define TQ_LAUNCH_KEYS(M)                                                                                  \
  do {                                                                                                     \
    if (dtype == TQ_F32) hipLaunchKernelGGL((encode_keys_kernel<M, TQ_F32, KEYS_ONE, 0>), grid, block, 0, s, L);      \
    else if (dtype == TQ_BF16) hipLaunchKernelGGL((encode_keys_kernel<M, TQ_BF16, KEYS_ONE, 0>), grid, block, 0, s, L); \
    else hipLaunchKernelGGL((encode_keys_kernel<M, TQ_F16, KEYS_ONE, 0>), grid, block, 0, s, L);            \
  } while (0)
  if (P.mode == TQ_MODE_MSE) TQ_LAUNCH_KEYS(TQ_MODE_MSE);
  else if (P.mode == TQ_MODE_PROD) TQ_LAUNCH_KEYS(TQ_MODE_PROD);
  else if (P.mode == TQ_MODE_GROUPED) TQ_LAUNCH_KEYS(TQ_MODE_GROUPED);
  else TQ_LAUNCH_KEYS(TQ_MODE_GROUPED_PROD);
#undef TQ_LAUNCH_KEYS
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

extern "C" tq_status tq_encode_values(int32_t bits, int32_t group, int32_t d, const void* values,
                                     int32_t dtype, int64_t n_vec, int64_t row_stride,
                                     const int64_t* slots, int64_t n_records, uint8_t* codes,
                                     uint16_t* scale, uint16_t* zero, void* stream) {
  ValArgs a;
  bool empty = false;
  tq_status st = val_args(bits, group, d, values, dtype, n_vec, row_stride, slots, n_records, codes, scale,
                          zero, a, empty);
  if (st != TQ_OK || empty) return st;
  const int cus = tq::cu_count();
  if (cus <= 0) return TQ_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if (bits == 2) {
    if (dtype == TQ_F32) launch_values<2, TQ_F32>(a, cus, s);
    else if (dtype == TQ_BF16) launch_values<2, TQ_BF16>(a, cus, s);
    else launch_values<2, TQ_F16>(a, cus, s);
  } else {
    if (dtype == TQ_F32) launch_values<4, TQ_F32>(a, cus, s);
    else if (dtype == TQ_BF16) launch_values<4, TQ_BF16>(a, cus, s);
    else launch_values<4, TQ_F16>(a, cus, s);
  }
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

extern "C" tq_status tq_encode_keys_batched(const tq_key_config* cfg, const tq_key_batch* batch,
                                           int32_t n_batch, int32_t dtype, int64_t n_vec,
                                           int64_t row_stride, int64_t n_records, void* stream) {
  if (n_batch < 0 || n_batch > MAX_KEY_BATCH || (n_batch > 0 && !batch)) return TQ_ERR_ARG;
  tq::Parts P;
  KeyLaunch<KEYS_BATCH> b;
  bool empty = false;
  if (n_batch == 0) {  // nothing to encode; the shared arguments are still checked
    tq_status st = tq::describe(cfg, &P);
    if (st != TQ_OK) return st;
    return n_vec < 0 || n_records < 0 ? TQ_ERR_ARG : TQ_OK;
  }
  for (int i = 0; i < n_batch; ++i) {
    KeyArgs a;
    tq_status st = key_args(cfg, batch[i].tables, batch[i].keys, dtype, n_vec, row_stride, batch[i].slots,
                            n_records, batch[i].idx, batch[i].signs, batch[i].norm, batch[i].rnorm, P, a,
                            empty);
    if (st != TQ_OK) return st;
    if (empty) return TQ_OK;
    b.e[i] = a;
  }
  const int cus = tq::cu_count();
  if (cus <= 0) return TQ_ERR_HIP;
  // A few blocks per CU shared out among the entries (at least one block
  // each).  The batch as a whole is a long launch, where four blocks per CU
  // suit the MSE and grouped encoders better than the two of a single short
  // set (measured on MI355X: 28 sets of 65536 MSE keys, 0.188 -> 0.175 ms).
  const int n_tiles = b.e[0].n_tiles;
  int per = cus * (P.m > 0 ? 8 : 4) / n_batch;
  const int kw = key_block_waves(P.mode, dtype, KEYS_BATCH);
  const int want = (n_tiles + kw - 1) / kw;
  if (per > want) per = want;
  if (per < 1) per = 1;
  b.blocks_per_entry = per;
  const dim3 grid((unsigned)(per * n_batch)), block(kw * 64);
  hipStream_t s = (hipStream_t)stream;
#define TQ_LAUNCH_KB(M)                                                                                     \
  do {                                                                                                      \
    if (dtype == TQ_F32) hipLaunchKernelGGL((encode_keys_kernel<M, TQ_F32, KEYS_BATCH, 0>), grid, block, 0, s, b);      \
    else if (dtype == TQ_BF16) hipLaunchKernelGGL((encode_keys_kernel<M, TQ_BF16, KEYS_BATCH, 0>), grid, block, 0, s, b); \
    else hipLaunchKernelGGL((encode_keys_kernel<M, TQ_F16, KEYS_BATCH, 0>), grid, block, 0, s, b);            \
  } while (0)
  if (P.mode == TQ_MODE_MSE) TQ_LAUNCH_KB(TQ_MODE_MSE);
  else if (P.mode == TQ_MODE_PROD) TQ_LAUNCH_KB(TQ_MODE_PROD);
  else if (P.mode == TQ_MODE_GROUPED) TQ_LAUNCH_KB(TQ_MODE_GROUPED);
  else TQ_LAUNCH_KB(TQ_MODE_GROUPED_PROD);
#undef TQ_LAUNCH_KB
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

extern "C" tq_status tq_append_kv(const tq_key_config* cfg, const void* tables, const void* keys,
                                 const void* values, int32_t dtype, int64_t n_vec, int64_t key_stride,
                                 int64_t value_stride, const int64_t* slots, int64_t n_records,
                                 uint8_t* idx, uint8_t* signs, uint16_t* norm, uint16_t* rnorm,
                                 int32_t v_bits, int32_t v_group, uint8_t* codes, uint16_t* scale,
                                 uint16_t* zero, void* stream) {
  tq::Parts P;
  KeyArgs ka;
  ValArgs va;
  bool empty = false;
  tq_status st = key_args(cfg, tables, keys, dtype, n_vec, key_stride, slots, n_records, idx, signs, norm,
                          rnorm, P, ka, empty);
  if (st != TQ_OK) return st;
  st = val_args(v_bits, v_group, KD, values, dtype, n_vec, value_stride, slots, n_records, codes, scale,
                zero, va, empty);
  if (st != TQ_OK || empty) return st;
  const int cus = tq::cu_count();
  if (cus <= 0) return TQ_ERR_HIP;
  const int kb = key_blocks(P, ka.n_tiles, cus, 4);
  const long long blocks = (long long)kb + grid_for(va.n_tiles, 4);
  const dim3 grid((unsigned)blocks), block(256);
  hipStream_t s = (hipStream_t)stream;
  const KeyLaunch<KEYS_AND_VALUES> L{ka, va, kb};
  static_assert(key_block_waves(TQ_MODE_MSE, TQ_BF16, KEYS_AND_VALUES) * 64 == 256,
                "key and value blocks share one block size");
#define TQ_LAUNCH_KV(M, B)                                                                                     \
  do {                                                                                                         \
    if (dtype == TQ_F32) hipLaunchKernelGGL((encode_keys_kernel<M, TQ_F32, KEYS_AND_VALUES, B>), grid, block, 0, s, L);      \
    else if (dtype == TQ_BF16) hipLaunchKernelGGL((encode_keys_kernel<M, TQ_BF16, KEYS_AND_VALUES, B>), grid, block, 0, s, L); \
    else hipLaunchKernelGGL((encode_keys_kernel<M, TQ_F16, KEYS_AND_VALUES, B>), grid, block, 0, s, L);            \
  } while (0)
#define TQ_LAUNCH_KV_M(M)               \
  do {                                  \
    if (v_bits == 2) TQ_LAUNCH_KV(M, 2); \
    else TQ_LAUNCH_KV(M, 4);             \
  } while (0)
  if (P.mode == TQ_MODE_MSE) TQ_LAUNCH_KV_M(TQ_MODE_MSE);
  else if (P.mode == TQ_MODE_PROD) TQ_LAUNCH_KV_M(TQ_MODE_PROD);
  else if (P.mode == TQ_MODE_GROUPED) TQ_LAUNCH_KV_M(TQ_MODE_GROUPED);
  else TQ_LAUNCH_KV_M(TQ_MODE_GROUPED_PROD);
#undef TQ_LAUNCH_KV_M
#undef TQ_LAUNCH_KV
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
