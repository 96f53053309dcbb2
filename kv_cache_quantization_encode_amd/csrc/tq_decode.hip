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
// shuffle butterflies in registers), projects them (S q'), and turns them into
// lookup tables: for every byte position p of a packed key and every byte
// value v, the four heads' partial inner products over the coordinates that
// byte holds, as fp16.  A key's score is then one table read per packed byte
// (48 for a 3-bit prod key) instead of 4 x 256 multiply-adds.  Half of the
// waves score 64-token tiles (lane = token) and run the online softmax; the
// other half accumulate p.V for those tiles one round later (lane = token-pair
// slot and 8-channel slice) on v_dot2_f32_f16 over token pairs, with the 2- or
// 4-bit code fields left in place as fp16 subnormal bit patterns (a byte's
// fields up to channel i, masked: prefix value * 2^-24), so no conversion is
// spent per code and per-channel sums are differences of consecutive prefix
// sums at the end.  The value scale is folded into the weight (p * scale) and
// the zero point is summed separately (sum_t p_t zero_t).  The chunk's (max,
// sum, unnormalised output) goes to the workspace; a second kernel merges
// chunks in a fixed order.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <atomic>
#include <type_traits>

#include "tq.h"
#include "tq_internal.h"
#include "tq_tables.h"

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int KD = 128;
#ifndef TQ_DEC_WAVES
#define TQ_DEC_WAVES 16
#endif
#ifndef TQ_DEC_LOOKUP_BATCH
#define TQ_DEC_LOOKUP_BATCH 8
#endif
constexpr int NW = TQ_DEC_WAVES;  // waves per workgroup
constexpr int NT = NW * 64;   // threads per workgroup
constexpr int PAGE_CACHE = 512;  // block-table entries a workgroup keeps in LDS
constexpr int TILE = 64;      // tokens per wave tile
constexpr int QH = 4;         // query heads per workgroup
constexpr int WGRP = 32 * QH + 16;  // dwords per value group of a wave's weight slot (padded)
constexpr int WSLOT = 4 * WGRP;     // dwords of a wave's weight slot
constexpr int PART = KD + 2;  // floats per partial: max, sum, out[128]
constexpr float LOG2E = 1.4426950408889634f;

constexpr int width_of(int b) { return b == 1 ? 1 : b == 2 ? 2 : 4; }
constexpr int stride_of(int b) { return b == 3 ? 128 : 256; }  // 3-bit in nibbles: bytes <= 0x77

template <int MODE, int B0, int B1>
struct Fmt {
  static constexpr bool GROUPED = MODE == TQ_MODE_GROUPED;
  static constexpr bool PROD = MODE == TQ_MODE_PROD;
  static constexpr int PD = GROUPED ? KD / 2 : KD;           // coordinates per part
  static constexpr int W0 = width_of(B0);
  static constexpr int W1 = GROUPED ? width_of(B1) : 1;
  static constexpr int CPB0 = 8 / W0, CPB1 = 8 / W1;           // coordinates per byte
  static constexpr int P0 = PD * W0 / 8;                        // class-0 byte positions
  static constexpr int P1 = PROD ? KD / 8 : GROUPED ? PD * W1 / 8 : 0;
  static constexpr int S0 = stride_of(B0);
  static constexpr int S1 = GROUPED ? stride_of(B1) : 256;
  static constexpr int E0 = P0 * S0, E1 = P1 * S1;              // table entries, [position][value]
  static constexpr int IDXB = P0 + (GROUPED ? P1 : 0);          // idx row bytes
  static constexpr int KWORDS = (IDXB + (PROD ? KD / 8 : 0)) / 4;  // idx + sign words
  // the weight ring also holds the half tables while the lookup tables are built
  static constexpr int RING_BYTES_W = NW * WSLOT * 4;
  static constexpr int HALF_BYTES = (P0 + P1) * 32 * 16;
  static constexpr int RING_BYTES = RING_BYTES_W > HALF_BYTES ? RING_BYTES_W : HALF_BYTES;
};

template <int MODE, int B0, int B1>
struct Lds {
  using F = Fmt<MODE, B0, B1>;
  uint2 lut[F::E0 + F::E1];
  float qp[QH * KD];
  float qs[QH * KD];
  uint32_t ring[F::RING_BYTES / 4];
  int amax[2 * QH];
  float cen[32];
  float abuf[2 * (NW / 2) * QH];
  float hmul[2 * QH];
  int pages[PAGE_CACHE];  // block-table entries of this workgroup's token range (paged cache)
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
__device__ __forceinline__ uint2 lut_read(const unsigned char* smem, uint32_t BASE, uint32_t w, int k) {
  uint32_t off;
  if (BASE + 2048u <= 65536u) {
    switch (k) {
      case 0: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(off) : "v"(w)); break;
      case 1: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(off) : "v"(w)); break;
      case 2: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(off) : "v"(w)); break;
      default: asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(off) : "v"(w)); break;
    }
    return *(const uint2*)(smem + off + BASE);
  } else {
    // (the empty asm keeps the byte extract whole, so that shift and add
    // become one v_lshl_or / v_lshl_add)
    uint32_t b = __builtin_amdgcn_ubfe(w, 8 * k, 8);
    asm("" : "+v"(b));
    off = (b << 3) + BASE;
    return *(const uint2*)(smem + off);
  }
}

template <int I, int N, typename Fn>
__device__ inline void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<I + 1, N>(fn);
  }
}

// Largest power of two P with P * bound <= 16384 (1 for a zero bound), from
// the exponent of bound = m 2^e, m in [0.5, 1).
__device__ inline float pow2_scale(float bound) {
  if (!(bound > 0.0f)) return 1.0f;
  int e;
  const float m = frexpf(bound, &e);
  int k = (m > 0.5f ? 14 : 15) - e;
  k = k > 126 ? 126 : k < -126 ? -126 : k;
  return ldexpf(1.0f, k);
}

// DPP lane moves (gfx9 encodings): quad permutations, half-row and row mirrors.
template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;

// Sum over each aligned group of eight lanes, in all eight.
__device__ inline float sum8(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  return v + dpp<DPP_HALF_MIRROR>(v);
}

// Maximum over the wave of a value that is already uniform in each aligned
// group of eight lanes (for any value: pass it through max8 first).
__device__ inline float wave_max_of_eights(float v) {
  v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ inline float max8(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  return fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS accesses
// only, so global loads already in flight (the next tile) stay in flight.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A value every lane holds alike, moved to a scalar register.
__device__ inline float uniform(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

template <int MODE, int B0, int B1, int VB>
__global__ __launch_bounds__(NT) void decode_kernel(DecArgs a) {
  using F = Fmt<MODE, B0, B1>;
  // Static LDS (its offsets are known to the compiler, so table offsets fold
  // into the ds_read immediates).
  __shared__ Lds<MODE, B0, B1> L;
  unsigned char* smem = (unsigned char*)&L;
  uint2* lut = L.lut;       // tables: class 0 [value][position], class 1 [position][value]
  float* qp = L.qp;         // [QH][KD] rotated queries
  float* qs = L.qs;         // [QH][KD] S q' (PROD)
  uint32_t* wbuf = L.ring;  // [2][NW/2][4 groups][32 pairs][QH] half2 weights (groups padded)
  int* amax = L.amax;       // [2][QH]
  float* cen = L.cen;       // [2][16] centroids of each part
  float* abuf = L.abuf;     // [2][NW/2][QH] softmax rescale factors
  float* hmul = L.hmul;     // [2][QH] score multipliers

  const tq_blob_header* H = (const tq_blob_header*)a.tables;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it are scalar
  const int split = blockIdx.x, quad = blockIdx.y, bh = blockIdx.z;
  const int b = bh / a.Hkv, hkv = bh % a.Hkv;
  // lengths outside [0, max_ctx] are clamped into it: no read leaves the sequence's records
  const int ctx = min(max(a.ctx_len[b], 0), a.max_ctx);
  const int t_begin = split * a.chunk;
  const int t_end = min(ctx, t_begin + a.chunk);

  const long long rec0 = ((long long)b * a.Hkv + hkv) * a.max_ctx;
  // ---- main loop, split between two kinds of waves.  Score waves (the first
  // half) read key bytes, look up the tables, run the online softmax and
  // publish fp16 weights p*scale; p.V waves (second half) accumulate those
  // weights against the value codes one round later.  Wave pw of each half
  // owns tiles pw, pw + NS, pw + 2 NS, ...; a two-slot LDS ring carries the
  // weights and the softmax rescale factor from score wave pw to p.V wave pw,
  // and one barrier per round separates producer and consumer.  Each wave
  // loads its next tile's data one round ahead.
  constexpr int NS = NW / 2;
  constexpr int VROW = KD * VB / 8;  // bytes of a value-code row
  const bool scorer = wave < NS;
  const int pw = scorer ? wave : wave - NS;
  const int slot = lane >> 4, u = lane & 15, grp = u >> 2;
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
  // page of t_last, where their clamped tokens are).
  // The workgroup's block-table entries are staged in LDS by the prologue (a
  // global read here would wait behind the tile loads already in flight);
  // the host sizes the splits so that they fit in PAGE_CACHE entries.
  const int lp0 = a.block_table ? t_begin / a.page_size : 0;
  const int n_pages_wg =
      a.block_table && t_end > t_begin ? min(t_last / a.page_size - lp0 + 1, PAGE_CACHE) : 0;
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
    if constexpr (F::PROD) {
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
  // value codes of this lane's token pairs (slot + 4k): [2k] even token, [2k+1] odd token
  auto load_codes = [&](int tb, uint32_t* c) {
    const long long tbase = tile_base(tb);
    if (tb + TILE <= t_end) {  // whole tile: one base address, immediate offsets
      const uint8_t* base = a.vcodes + (tbase + tb + 2 * slot) * VROW + VB * u;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint8_t* pa = base + ((k >> 1) * 8 + (k & 1)) * VROW;
        c[k] = VB == 2 ? (uint32_t) * (const uint16_t*)pa : *(const uint32_t*)pa;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int t = min(tb + 2 * slot + (k >> 1) * 8 + (k & 1), t_last);
        const uint8_t* pa = a.vcodes + (tbase + t) * VROW + VB * u;
        c[k] = VB == 2 ? (uint32_t) * (const uint16_t*)pa : *(const uint32_t*)pa;
      }
    }
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
  if (wave < QH) {
    const float* sig0 = (const float*)(a.tables + H->off_sigma[0]);
    const float* sig1 = (const float*)(a.tables + H->off_sigma[n_parts > 1 ? 1 : 0]);
    sg0 = sig0[lane];
    sg1 = F::GROUPED ? sig1[lane] : sig0[lane + 64];
  }
  // q_s = S q': thread -> (row tid / 8, 16-column chunk tid % 8), all 128 rows at once
  static_assert(NT == 8 * KD, "S q' takes one row per eight threads");
  const int srow = tid >> 3, sch = tid & 7;
  uint4 sA = make_uint4(0, 0, 0, 0), sB = sA;
  if constexpr (F::PROD) {
    const uint4* sp = (const uint4*)((const uint16_t*)(a.tables + H->off_S) + (size_t)srow * KD + 16 * sch);
    sA = sp[0];
    sB = sp[1];
  }
  if (tid < 32) {
    const int part = tid >> 4, k = tid & 15;
    cen[tid] = part < n_parts && k < (part ? lev1 : lev0) ? (part ? cent1 : cent0)[k] : 0.0f;
  }
  if (!F::GROUPED && tid < QH) amax[QH + tid] = 0;
  for (int i = tid; i < n_pages_wg; i += NT) L.pages[i] = a.block_table[(long long)b * a.max_blocks + lp0 + i];

  // Walsh-Hadamard transform of sigma * q in registers (one 128-point
  // transform, or two 64-point ones for GROUPED): butterflies on lane bits
  // through shuffles, the top stage inside the lane.
  if (wave < QH) {
    x0 = q_word_to_float(qw0, a.q_dtype) * sg0;
    x1 = q_word_to_float(qw1, a.q_dtype) * sg1;
    if constexpr (!F::GROUPED) {
      const float t = x0;
      x0 = t + x1;
      x1 = t - x1;
    }
#pragma unroll
    for (int st = 32; st >= 1; st >>= 1) {
      const float y0 = __shfl_xor(x0, st), y1 = __shfl_xor(x1, st);
      const bool up = lane & st;
      x0 = up ? y0 - x0 : x0 + y0;
      x1 = up ? y1 - x1 : x1 + y1;
    }
    qp[wave * KD + lane] = x0;
    qp[wave * KD + lane + 64] = x1;
    // largest |q'| per table class (GROUPED: per half)
    const float m0 = wave_max_of_eights(max8(F::GROUPED ? fabsf(x0) : fmaxf(fabsf(x0), fabsf(x1))));
    const float m1 = F::GROUPED ? wave_max_of_eights(max8(fabsf(x1))) : 0.0f;
    if (lane == 0) {
      amax[wave] = __float_as_int(m0);
      if (F::GROUPED) amax[QH + wave] = __float_as_int(m1);
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
  uint32_t codes[16];
  if (n_tiles > 0) {
    if (scorer) load_keys(tile_tb(0), kd);
    else load_codes(tile_tb(0), codes);
  }
  if constexpr (F::PROD) {
    const uint32_t sw[8] = {sA.x, sA.y, sA.z, sA.w, sB.x, sB.y, sB.z, sB.w};
    float part[QH] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int hh = 0; hh < QH; ++hh) {
      const float4* qv = (const float4*)(qp + hh * KD + 16 * sch);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 v = qv[c];
        part[hh] = fmaf(h2f(sw[2 * c] & 0xFFFFu), v.x, part[hh]);
        part[hh] = fmaf(h2f(sw[2 * c] >> 16), v.y, part[hh]);
        part[hh] = fmaf(h2f(sw[2 * c + 1] & 0xFFFFu), v.z, part[hh]);
        part[hh] = fmaf(h2f(sw[2 * c + 1] >> 16), v.w, part[hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < QH; ++hh) {
      part[hh] = sum8(part[hh]);
      if (sch == 0) qs[hh * KD + srow] = part[hh];
      const float m = wave_max_of_eights(fabsf(part[hh]));
      if (lane == 0) atomicMax(&amax[QH + hh], __float_as_int(m));
    }
  }
  if constexpr (F::PROD) lds_barrier();
  // per-head, per-class power-of-two table scale: the largest possible entry
  // (|q'| bound x largest centroid x coordinates per byte) stays <= 16384
  auto table_scale = [&](int cls, int hh) {
    float cmax = 1.0f;
    int cpb = 8;
    if (!(F::PROD && cls == 1)) {
      cmax = fabsf(cen[cls ? 16 + lev1 - 1 : lev0 - 1]);  // LDS: no wait behind the tile loads
      cpb = cls == 0 ? F::CPB0 : F::CPB1;
    }
    return pow2_scale(__int_as_float(amax[cls * QH + hh]) * cmax * cpb);
  };
  // per-token multipliers of the two table classes, with the scales undone:
  // hmul[0][h] multiplies the norm, hmul[1][h] the residual norm (PROD) or
  // the second half's norm (GROUPED).  Kept in LDS, read where used.
  if (tid < QH) {
    hmul[tid] = 1.0f / (table_scale(0, tid) * (float)F::PD);
    hmul[QH + tid] = F::PROD ? 1.2533141373155003f / ((float)KD * sqrtf((float)KD) * table_scale(1, tid))
                             : 1.0f / (table_scale(1, tid) * (float)F::PD);
  }
  // Half tables: for each byte position, class, nibble half and nibble value,
  // the four heads' partial sums over the coordinates (or sign rows) that
  // nibble holds, already scaled.  A byte's entry is then lo[v & 15] +
  // hi[v >> 4].  They live in the weight ring, unused until the main loop.
  float4* halves = (float4*)wbuf;  // [P0 + P1][2][16]
  for (int i = tid; i < (F::P0 + F::P1) * 32; i += NT) {
    const int pos = i >> 5, half = (i >> 4) & 1, n = i & 15;
    const bool c1 = pos >= F::P0;
    const int p = c1 ? pos - F::P0 : pos;
    float sv[QH] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c1 && F::PROD) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float sg = ((n >> k) & 1) ? 1.0f : -1.0f;
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) sv[hh] = fmaf(sg, qs[hh * KD + 8 * p + 4 * half + k], sv[hh]);
      }
    } else {
      const int W = c1 ? F::W1 : F::W0;
      const int per = 4 / W;  // coordinates per nibble
      const int fmask = (1 << (c1 ? B1 : B0)) - 1;
      const float* cn = cen + (c1 ? 16 : 0);
      const int j0 = (c1 ? F::PD : 0) + p * (8 / W) + half * per;
      for (int k = 0; k < per; ++k) {
        const float c = cn[(n >> (W * k)) & fmask];
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) sv[hh] = fmaf(c, qp[hh * KD + j0 + k], sv[hh]);
      }
    }
    const int cls = c1 ? 1 : 0;
    halves[i] = make_float4(sv[0] * table_scale(cls, 0), sv[1] * table_scale(cls, 1),
                            sv[2] * table_scale(cls, 2), sv[3] * table_scale(cls, 3));
  }
  lds_barrier();
  // One thread per (position, low nibble) walks the high nibbles: its low
  // half stays in registers, the high halves are read by sixteen lanes at once.
  for (int t = tid; t < (F::P0 + F::P1) * 16; t += NT) {
    const int pos = t >> 4, lo = t & 15;
    const bool c1 = pos >= F::P0;
    const int S = c1 ? F::S1 : F::S0;
    uint2* dst = lut + (c1 ? F::E0 + (pos - F::P0) * F::S1 : pos * F::S0);
    const float4 lo4 = halves[pos * 32 + lo];
#pragma unroll 4
    for (int hi = 0; hi < 16; ++hi) {
      const int v = hi * 16 + lo;
      if (v < S) {
        const float4 hi4 = halves[pos * 32 + 16 + hi];
        // round to nearest even, two heads per conversion
        const half2_t e01 = __builtin_convertvector((float2_t){lo4.x + hi4.x, lo4.y + hi4.y}, half2_t);
        const half2_t e23 = __builtin_convertvector((float2_t){lo4.z + hi4.z, lo4.w + hi4.w}, half2_t);
        dst[v] = make_uint2(__builtin_bit_cast(uint32_t, e01), __builtin_bit_cast(uint32_t, e23));
      }
    }
  }
  lds_barrier();
  const float xscale = a.sm_scale * LOG2E;

  const half2_t e10 = {(_Float16)1.0f, (_Float16)0.0f}, e01 = {(_Float16)0.0f, (_Float16)1.0f};
  float* red = (float*)smem;  // [NS][QH][2 + 4 + KD], over the tables once every wave is done
  constexpr int RS = 2 + 4 + KD;
  float* mine = red + pw * QH * RS;
  // The two kinds of waves run separate loops with the same number of
  // barriers (rounds + 1), so neither keeps the other's registers live.
  if (scorer) {
    float m_run[QH], l_run[QH], zacc[QH][4];
#pragma unroll
    for (int hh = 0; hh < QH; ++hh) {
      m_run[hh] = -INFINITY;
      l_run[hh] = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) zacc[hh][k] = 0.0f;
    }
    // two key buffers in turn: a round scores one while the next tile's
    // bytes arrive in the other
    auto s_round = [&](int r, KeyData& kd) {
      const int tb = tile_tb(r);
      if (r < rounds && tb < t_end) {
        // ---------------- scores: lane = token
        const int t = tb + lane;
        const bool valid = t < t_end;
        float sc[QH];
        {
          const float m0 = F::GROUPED ? h2f(kd.nrm & 0xFFFFu) : h2f(kd.nrm);
          const float m1 = F::GROUPED ? h2f(kd.nrm >> 16) : h2f(kd.rn);
          // table sums in fp32: fdot2(entry pair, (1,0)) adds one fp16 exactly
          float A[QH] = {0, 0, 0, 0}, Bc[QH] = {0, 0, 0, 0};
          // Index nibbles of 3-bit codes have their high bit clear (tq_encode_keys
          // writes them so), so a byte is a table index as it stands.
#pragma unroll
          for (int p = 0; p < F::P0; ++p) {
            // cap the table reads in flight (each holds two registers); the
            // empty asm keeps each batch's accumulation ahead of the next
            // batch instead of letting it sink below all the reads
            if (p % TQ_DEC_LOOKUP_BATCH == 0) {
              if (p > 0) asm volatile("" : "+v"(A[0]), "+v"(A[1]), "+v"(A[2]), "+v"(A[3]));
              __builtin_amdgcn_sched_barrier(0);
            }
            const uint2 e = lut_read(smem, (uint32_t)(p * F::S0) * 8u, kd.kw[p >> 2], p & 3);
            const half2_t x01 = __builtin_bit_cast(half2_t, e.x), x23 = __builtin_bit_cast(half2_t, e.y);
            if (p == 0) {  // the first entries start the sums (the same values fdot2 onto 0 gives)
              A[0] = (float)x01[0]; A[1] = (float)x01[1]; A[2] = (float)x23[0]; A[3] = (float)x23[1];
            } else {
              A[0] = __builtin_amdgcn_fdot2(x01, e10, A[0], false);
              A[1] = __builtin_amdgcn_fdot2(x01, e01, A[1], false);
              A[2] = __builtin_amdgcn_fdot2(x23, e10, A[2], false);
              A[3] = __builtin_amdgcn_fdot2(x23, e01, A[3], false);
            }
          }
#pragma unroll
          for (int p = 0; p < F::P1; p += (F::PROD ? 2 : 1)) {
            if (p % TQ_DEC_LOOKUP_BATCH == 0) {
              if (p > 0) asm volatile("" : "+v"(Bc[0]), "+v"(Bc[1]), "+v"(Bc[2]), "+v"(Bc[3]));
              __builtin_amdgcn_sched_barrier(0);
            }
            const int byte = F::P0 + p;
            const uint2 e = lut_read(smem, (uint32_t)(F::E0 + p * F::S1) * 8u, kd.kw[byte >> 2], byte & 3);
            half2_t x01 = __builtin_bit_cast(half2_t, e.x), x23 = __builtin_bit_cast(half2_t, e.y);
            if constexpr (F::PROD) {
              // QJL sign bytes two at a time: their fp16 entries are added in
              // fp16 first (one packed add per head pair), halving the
              // accumulate work of this smaller term of the score
              const uint2 f = lut_read(smem, (uint32_t)(F::E0 + (p + 1) * F::S1) * 8u, kd.kw[(byte + 1) >> 2], (byte + 1) & 3);
              x01 += __builtin_bit_cast(half2_t, f.x);
              x23 += __builtin_bit_cast(half2_t, f.y);
            }
            if (p == 0) {
              Bc[0] = (float)x01[0]; Bc[1] = (float)x01[1]; Bc[2] = (float)x23[0]; Bc[3] = (float)x23[1];
            } else {
              Bc[0] = __builtin_amdgcn_fdot2(x01, e10, Bc[0], false);
              Bc[1] = __builtin_amdgcn_fdot2(x01, e01, Bc[1], false);
              Bc[2] = __builtin_amdgcn_fdot2(x23, e10, Bc[2], false);
              Bc[3] = __builtin_amdgcn_fdot2(x23, e01, Bc[3], false);
            }
          }
          const float4 h0 = *(const float4*)hmul, h1 = *(const float4*)(hmul + QH);
          const float mul0[QH] = {h0.x, h0.y, h0.z, h0.w}, mul1[QH] = {h1.x, h1.y, h1.z, h1.w};
#pragma unroll
          for (int hh = 0; hh < QH; ++hh) {
            if constexpr (F::P1 > 0) sc[hh] = valid ? m0 * mul0[hh] * A[hh] + m1 * mul1[hh] * Bc[hh] : -INFINITY;
            else sc[hh] = valid ? m0 * mul0[hh] * A[hh] : -INFINITY;  // MSE: one table class
          }
          if (a.scores && valid) {
#pragma unroll
            for (int hh = 0; hh < QH; ++hh) {
              const int gq = QH * quad + hh;
              if (gq < a.G) a.scores[((long long)b * a.Hq + hkv * a.G + gq) * a.max_ctx + t] = sc[hh];
            }
          }
        }
        // ---------------- online softmax (base 2).  The wave-wide max is
        // only recomputed when some lane exceeds the running max; otherwise
        // every p = 2^(x - m) <= 1 already and nothing needs rescaling.
        float x[QH], alpha[QH] = {1.0f, 1.0f, 1.0f, 1.0f};
        bool exceed = false;
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) {
          x[hh] = sc[hh] * xscale;  // -inf for missing tokens
          exceed |= x[hh] > m_run[hh];
        }
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
        const uint2 zv = kd.zv, sv = kd.sv;
        load_keys(tile_tb(r + 1), kd);
        float zz[4], ss[4];
        zz[0] = h2f(zv.x & 0xFFFFu); zz[1] = h2f(zv.x >> 16);
        zz[2] = h2f(zv.y & 0xFFFFu); zz[3] = h2f(zv.y >> 16);
        ss[0] = h2f(sv.x & 0xFFFFu); ss[1] = h2f(sv.x >> 16);
        ss[2] = h2f(sv.y & 0xFFFFu); ss[3] = h2f(sv.y >> 16);
        float p[QH];
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) {
          // m_run is finite (lane 0 holds a valid token) and x - m_run <= 0
          p[hh] = __builtin_amdgcn_exp2f(x[hh] - m_run[hh]);
          l_run[hh] += p[hh];
#pragma unroll
          for (int k = 0; k < 4; ++k) zacc[hh][k] = fmaf(p[hh], zz[k], zacc[hh][k]);
        }
        // weights p * scale as fp16 (p rounded to fp16, then two heads per
        // packed multiply), paired by token: [group][pair][head] = (w_even, w_odd);
        // the group stride is padded so that neither these stores nor the p.V
        // waves' 16-byte reads pile onto a few LDS banks
        uint16_t* wb16 = (uint16_t*)(wbuf + ((r & 1) * NS + pw) * WSLOT);
        const int pair = lane >> 1, odd = lane & 1;
        const half2_t p01 = __builtin_convertvector((float2_t){p[0], p[1]}, half2_t);
        const half2_t p23 = __builtin_convertvector((float2_t){p[2], p[3]}, half2_t);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const half2_t s2 = {(_Float16)ss[k], (_Float16)ss[k]};
          const half2_t w01 = p01 * s2, w23 = p23 * s2;
          wb16[(k * WGRP + pair * QH + 0) * 2 + odd] = __builtin_bit_cast(uint32_t, w01) & 0xFFFFu;
          wb16[(k * WGRP + pair * QH + 1) * 2 + odd] = __builtin_bit_cast(uint32_t, w01) >> 16;
          wb16[(k * WGRP + pair * QH + 2) * 2 + odd] = __builtin_bit_cast(uint32_t, w23) & 0xFFFFu;
          wb16[(k * WGRP + pair * QH + 3) * 2 + odd] = __builtin_bit_cast(uint32_t, w23) >> 16;
        }
        if (lane == 0) {
#pragma unroll
          for (int hh = 0; hh < QH; ++hh) abuf[((r & 1) * NS + pw) * QH + hh] = alpha[hh];
        }
      }
    };
    for (int r = 0; r <= rounds; ++r) {
      s_round(r, kd);
      lds_barrier();
    }
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
  } else {
    float acc[QH][8];
#pragma unroll
    for (int hh = 0; hh < QH; ++hh)
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[hh][k] = 0.0f;
    // two code buffers in turn: a round consumes one while the next tile's
    // codes arrive in the other
    uint32_t codes2[16];
    auto pv_round = [&](int r, const uint32_t* cur, uint32_t* nxt) {
      const int tb = r >= 1 ? tile_tb(r - 1) : t_end;
      if (tb < t_end) {
        load_codes(tile_tb(r), nxt);  // next round's tile
        const uint32_t* wsrc = wbuf + (((r - 1) & 1) * NS + pw) * WSLOT;
        const float4 al = *(const float4*)(abuf + (((r - 1) & 1) * NS + pw) * QH);
        const float alv[QH] = {uniform(al.x), uniform(al.y), uniform(al.z), uniform(al.w)};
        if (alv[0] != 1.0f || alv[1] != 1.0f || alv[2] != 1.0f || alv[3] != 1.0f) {
#pragma unroll
          for (int hh = 0; hh < QH; ++hh)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[hh][k] *= alv[hh];
        }
        // ---------------- p.V: lane = (slot, 8-dim slice u); slot takes token pairs slot + 4k
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int pr = slot + 4 * k;
          const uint32_t cA = cur[2 * k], cB = cur[2 * k + 1];
          const uint4 wv = *(const uint4*)(wsrc + grp * WGRP + pr * QH);
          const uint32_t wh[QH] = {wv.x, wv.y, wv.z, wv.w};
          // pairs[i] holds, for the two tokens (low and high half), the
          // prefix of channel i: the channels of its byte up to i, so that
          // one byte permute serves a whole byte and the last prefix of each
          // byte needs no mask.  The channel sums are told apart at the end.
          uint32_t pairs[8];
          if (VB == 2) {
            const uint32_t Y1 = __builtin_amdgcn_perm(cB, cA, 0x0c040c00u);  // byte 0 of A, of B -> bytes 0, 2
            const uint32_t Y2 = __builtin_amdgcn_perm(cB, cA, 0x0c050c01u);  // byte 1 of A, of B -> bytes 0, 2
            pairs[0] = Y1 & 0x00030003u; pairs[1] = Y1 & 0x000F000Fu; pairs[2] = Y1 & 0x003F003Fu; pairs[3] = Y1;
            pairs[4] = Y2 & 0x00030003u; pairs[5] = Y2 & 0x000F000Fu; pairs[6] = Y2 & 0x003F003Fu; pairs[7] = Y2;
          } else {
#pragma unroll
            for (int b = 0; b < 4; ++b) {  // byte b of A and of B -> bytes 0, 2
              const uint32_t Yb = __builtin_amdgcn_perm(cB, cA, 0x0c000c00u | ((4u + b) << 16) | (uint32_t)b);
              pairs[2 * b] = Yb & 0x000F000Fu;
              pairs[2 * b + 1] = Yb;
            }
          }
#pragma unroll
          for (int hh = 0; hh < QH; ++hh) {
            const half2_t w2 = __builtin_bit_cast(half2_t, wh[hh]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
              acc[hh][i] = __builtin_amdgcn_fdot2(w2, __builtin_bit_cast(half2_t, pairs[i]), acc[hh][i], false);
          }
        }
      }
    };
    for (int r = 0; r <= rounds; r += 2) {
      pv_round(r, codes2, codes);
      lds_barrier();
      if (r + 1 <= rounds) {
        pv_round(r + 1, codes, codes2);
        lds_barrier();
      }
    }
    // Undo the placement: accumulator i holds, in units of 2^-24, the
    // prefix sum over the channels of its byte up to i, channel j weighted
    // by its field's place value step_j; a channel's sum is the difference
    // of consecutive prefixes over its place value.
#pragma unroll
    for (int hh = 0; hh < QH; ++hh) {
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        r[i] = acc[hh][i];
        r[i] += __shfl_xor(r[i], 16);
        r[i] += __shfl_xor(r[i], 32);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        constexpr int PER = 8 / VB;  // channels per byte
        const int f = i % PER;       // field within the byte
        const float step = (float)(1 << (VB * f));
        const float v = f == 0 ? r[i] : r[i] - r[i - 1];
        if (lane < 16) mine[hh * RS + 6 + 8 * u + i] = v * (16777216.0f / step);
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < QH * KD; i += NT) {
    const int hh = i / KD, j = i % KD;
    const int gq = QH * quad + hh;
    float M = -INFINITY;
    for (int w = 0; w < NS; ++w) M = fmaxf(M, red[(w * QH + hh) * RS]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
      for (int w = 0; w < NS; ++w) {
        const float* rr = red + (w * QH + hh) * RS;
        const float f = rr[0] == -INFINITY ? 0.0f : exp2f(rr[0] - M);
        L = fmaf(rr[1], f, L);
        O = fmaf(rr[6 + j] + rr[2 + j / 32], f, O);
      }
    }
    if (gq < a.G) {
      float* dst = a.part + (((long long)b * a.Hq + hkv * a.G + gq) * a.n_split + split) * PART;
      if (j == 0) {
        dst[0] = M;
        dst[1] = L;
      }
      dst[2 + j] = O;
    }
  }
}

// out[b][h][:] = sum_s O_s 2^(M_s - M) / sum_s L_s 2^(M_s - M), in split order.
__global__ __launch_bounds__(KD) void merge_kernel(const float* part, int n_split, float* out,
                                                   float* lse) {
  const int bh = blockIdx.x, j = threadIdx.x;
  const float* p = part + (long long)bh * n_split * PART;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, p[s * PART]);
  float L = 0.0f, O = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const float* r = p + s * PART;
      const float f = r[0] == -INFINITY ? 0.0f : exp2f(r[0] - M);
      L = fmaf(r[1], f, L);
      O = fmaf(r[2 + j], f, O);
    }
  }
  out[(long long)bh * KD + j] = L > 0.0f ? O / L : 0.0f;
  if (lse && j == 0) lse[bh] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
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
  if (P.mode == TQ_MODE_GROUPED) {
    const int b0 = P.part_bits[0], b1 = P.part_bits[1];
    return (b0 == 4 && b1 == 2) || (b0 == 2 && b1 == 2) || (b0 == 3 && b1 == 2) || (b0 == 4 && b1 == 1);
  }
  return P.part_bits[0] >= 1 && P.part_bits[0] <= 3;
}

hipError_t dispatch(const tq::Parts& P, int vb, const DecArgs& a, dim3 grid, hipStream_t s) {
  if (P.mode == TQ_MODE_PROD) {
    switch (P.part_bits[0]) {
      case 1: return launch_vb<TQ_MODE_PROD, 1, 0>(vb, a, grid, s);
      case 2: return launch_vb<TQ_MODE_PROD, 2, 0>(vb, a, grid, s);
      default: return launch_vb<TQ_MODE_PROD, 3, 0>(vb, a, grid, s);
    }
  }
  if (P.mode == TQ_MODE_MSE) {
    switch (P.part_bits[0]) {
      case 1: return launch_vb<TQ_MODE_MSE, 1, 0>(vb, a, grid, s);
      case 2: return launch_vb<TQ_MODE_MSE, 2, 0>(vb, a, grid, s);
      default: return launch_vb<TQ_MODE_MSE, 3, 0>(vb, a, grid, s);
    }
  }
  const int b0 = P.part_bits[0], b1 = P.part_bits[1];
  if (b0 == 4 && b1 == 2) return launch_vb<TQ_MODE_GROUPED, 4, 2>(vb, a, grid, s);
  if (b0 == 2 && b1 == 2) return launch_vb<TQ_MODE_GROUPED, 2, 2>(vb, a, grid, s);
  if (b0 == 3 && b1 == 2) return launch_vb<TQ_MODE_GROUPED, 3, 2>(vb, a, grid, s);
  return launch_vb<TQ_MODE_GROUPED, 4, 1>(vb, a, grid, s);
}

}  // namespace

namespace {

tq_status decode_impl(const tq_key_config* cfg, const void* tables, const void* q, int32_t q_dtype,
                      int32_t B, int32_t Hq, int32_t Hkv, const int32_t* ctx_len, int32_t max_ctx,
                      const int32_t* block_table, int32_t max_blocks, int32_t page_size,
                      const uint8_t* idx, const uint8_t* signs, const uint16_t* norm,
                      const uint16_t* rnorm, int32_t v_bits, int32_t v_group, const uint8_t* v_codes,
                      const uint16_t* v_scale, const uint16_t* v_zero, float sm_scale, float* out,
                      float* lse, float* scores, void* workspace, size_t* workspace_bytes,
                      void* stream) {
  tq::Parts P;
  tq_status st = tq::describe(cfg, &P);
  if (st != TQ_OK) return st;
  if (P.d != KD || !supported(P)) return TQ_ERR_UNSUPPORTED;
  if (v_bits != 2 && v_bits != 4) return TQ_ERR_UNSUPPORTED;
  if (v_group != 32) return TQ_ERR_UNSUPPORTED;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16 && q_dtype != TQ_F16) return TQ_ERR_ARG;
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
  if (P.mode == TQ_MODE_PROD && (!signs || !rnorm)) return TQ_ERR_ARG;
  if (!tq::aligned16(tables) || !tq::aligned16(idx) || !tq::aligned16(v_codes) ||
      !tq::aligned16(workspace) || !tq::aligned16(q))
    return TQ_ERR_ARG;
  if (P.mode == TQ_MODE_PROD && !tq::aligned16(signs)) return TQ_ERR_ARG;
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
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(n_split, n_quads, B * Hkv);
  if (dispatch(P, v_bits, a, grid, s) != hipSuccess) return TQ_ERR_HIP;
  hipLaunchKernelGGL(merge_kernel, dim3(B * Hq), dim3(KD), 0, s, (const float*)workspace, n_split,
                     out, lse);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // namespace

extern "C" tq_status tq_decode_attention(const tq_key_config* cfg, const void* tables, const void* q,
                                        int32_t q_dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                        const int32_t* ctx_len, int32_t max_ctx, const uint8_t* idx,
                                        const uint8_t* signs, const uint16_t* norm,
                                        const uint16_t* rnorm, int32_t v_bits, int32_t v_group,
                                        const uint8_t* v_codes, const uint16_t* v_scale,
                                        const uint16_t* v_zero, float sm_scale, float* out,
                                        float* lse, float* scores, void* workspace,
                                        size_t* workspace_bytes, void* stream) {
  return decode_impl(cfg, tables, q, q_dtype, B, Hq, Hkv, ctx_len, max_ctx, nullptr, 0, 0, idx, signs,
                     norm, rnorm, v_bits, v_group, v_codes, v_scale, v_zero, sm_scale, out, lse, scores,
                     workspace, workspace_bytes, stream);
}

extern "C" tq_status tq_decode_attention_paged(
    const tq_key_config* cfg, const void* tables, const void* q, int32_t q_dtype, int32_t B, int32_t Hq,
    int32_t Hkv, const int32_t* ctx_len, const int32_t* block_table, int32_t max_blocks_per_seq,
    int32_t page_size, const uint8_t* idx, const uint8_t* signs, const uint16_t* norm,
    const uint16_t* rnorm, int32_t v_bits, int32_t v_group, const uint8_t* v_codes,
    const uint16_t* v_scale, const uint16_t* v_zero, float sm_scale, float* out, float* lse,
    float* scores, void* workspace, size_t* workspace_bytes, void* stream) {
  if (page_size <= 0 || page_size % TILE != 0 || max_blocks_per_seq <= 0) return TQ_ERR_ARG;
  if ((long long)max_blocks_per_seq * page_size > 0x3fffffffLL) return TQ_ERR_ARG;
  if (workspace && !block_table) return TQ_ERR_ARG;
  return decode_impl(cfg, tables, q, q_dtype, B, Hq, Hkv, ctx_len, max_blocks_per_seq * page_size,
                     block_table, max_blocks_per_seq, page_size, idx, signs, norm, rnorm, v_bits, v_group,
                     v_codes, v_scale, v_zero, sm_scale, out, lse, scores, workspace, workspace_bytes,
                     stream);
}
