// Dequantisers for gfx950: packed records back to dense k_hat and v_hat rows
// (the "tqlite" README's dequantise path for prefill and fake quantisation;
// validate_paper.py's prod dequantize).
//
// Keys (one lane per key):
//   k_hat = Pi^T w,  w = (n / sqrt(d)) c[idx]  (+ rho sqrt(pi/2) / m S^T (2 bit - 1), PROD)
// with Pi^T = diag(sigma) H / sqrt(d), so k_hat = sigma * H(w) / sqrt(d): the
// same 128-point Walsh-Hadamard transform as the encoder, run on w in the
// lane's registers (two 64-point transforms for GROUPED, each half with its
// own norm, codebook and sigma; GROUPED_PROD adds the QJL term, built in the
// halves' rotated frame, before the two transforms).  The QJL term S^T (2 bit - 1) takes two sign
// rows per v_dot2_f32_f16 against S stored in LDS as fp16 row pairs; every lane
// reads the same pair at once (an LDS broadcast).
// Values (sixteen lanes per row, eight channels each): v_hat = code * s + z.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "tq.h"
#include "tq_internal.h"
#include "tq_tables.h"

namespace {

constexpr int KD = 128;
constexpr int DQ_THREADS = 256;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct DqKeyArgs {
  const unsigned char* tables;
  long long n_vec;
  const long long* slots;
  long long n_records;
  const uint8_t* idx;
  const uint8_t* signs;
  const uint16_t* norm;
  const uint16_t* rnorm;
  void* out;
  int out_dtype;
  long long out_stride;  // elements
  int idx_row_bytes;
};

__device__ inline float h2f(uint32_t bits16) { return __half2float(__ushort_as_half((unsigned short)bits16)); }

__device__ inline void store_row(void* out, int dt, long long off, const float* v) {
  if (dt == TQ_F32) {
    float4* p = (float4*)((float*)out + off);
#pragma unroll
    for (int k = 0; k < KD / 4; ++k) p[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  } else {
    uint4* p = (uint4*)((uint16_t*)out + off);
#pragma unroll
    for (int k = 0; k < KD / 8; ++k) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = v[8 * k + 2 * i], b = v[8 * k + 2 * i + 1];
        uint32_t lo, hi;
        if (dt == TQ_BF16) {  // round to nearest even
          const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
          lo = (ua + 0x7FFFu + ((ua >> 16) & 1u)) >> 16;
          hi = (ub + 0x7FFFu + ((ub >> 16) & 1u)) >> 16;
        } else {
          lo = __half_as_ushort(__float2half_rn(a));
          hi = __half_as_ushort(__float2half_rn(b));
        }
        w[i] = lo | (hi << 16);
      }
      p[k] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// In-register Walsh-Hadamard transform of v[0 .. N) (unnormalised).
template <int N>
__device__ inline void fwht(float* v) {
#pragma unroll
  for (int s = 1; s < N; s <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & s) == 0) {
        const float a = v[i], b = v[i + s];
        v[i] = a + b;
        v[i + s] = a - b;
      }
    }
  }
}

// MODE: tq_mode; W0/W1: storage widths (bits) of the index fields of each part.
template <int MODE, int W0, int W1>
__global__ __launch_bounds__(DQ_THREADS) void dequant_keys_kernel(DqKeyArgs a) {
  constexpr bool GROUPED = MODE == TQ_MODE_GROUPED || MODE == TQ_MODE_GROUPED_PROD;
  constexpr bool PROD = MODE == TQ_MODE_PROD || MODE == TQ_MODE_GROUPED_PROD;  // QJL term
  constexpr int NP = GROUPED ? 2 : 1;
  constexpr int PD = KD / NP;                                  // coordinates per part
  constexpr int IDXB = PD * W0 / 8 + (GROUPED ? PD * W1 / 8 : 0);
  __shared__ float s_cent[NP][256];
  __shared__ float s_sig[KD];
  __shared__ __align__(16) uint32_t s_sp[PROD ? (KD / 2) * KD : 4];  // (S[2i][j], S[2i+1][j]) fp16 pairs
  const tq_blob_header* H = (const tq_blob_header*)a.tables;
  const int tid = threadIdx.x;
  for (int p = 0; p < NP; ++p) {
    const float* c = (const float*)(a.tables + H->off_centroids[p]);
    for (int i = tid; i < H->part_levels[p]; i += DQ_THREADS) s_cent[p][i] = c[i];
    const float* sg = (const float*)(a.tables + H->off_sigma[p]);
    for (int i = tid; i < PD; i += DQ_THREADS) s_sig[p * PD + i] = sg[i];
  }
  if constexpr (PROD) {
    // item = (row pair ip, eight columns): two 16-byte reads, interleaved
    const uint16_t* S = (const uint16_t*)(a.tables + H->off_S);
    constexpr int ITEMS = (KD / 2) * (KD / 8) / DQ_THREADS;
    uint4 r0[ITEMS], r1[ITEMS];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int it = tid + k * DQ_THREADS, ip = it / (KD / 8), j = 8 * (it % (KD / 8));
      r0[k] = *(const uint4*)(S + (2 * ip) * KD + j);
      r1[k] = *(const uint4*)(S + (2 * ip + 1) * KD + j);
    }
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int it = tid + k * DQ_THREADS, ip = it / (KD / 8), j = 8 * (it % (KD / 8));
      const uint32_t a0[4] = {r0[k].x, r0[k].y, r0[k].z, r0[k].w}, a1[4] = {r1[k].x, r1[k].y, r1[k].z, r1[k].w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = __builtin_amdgcn_perm(a1[i], a0[i], 0x05040100u);      // (row 2ip, row 2ip+1) of column j+2i
        o[2 * i + 1] = __builtin_amdgcn_perm(a1[i], a0[i], 0x07060302u);  // ... of column j+2i+1
      }
      uint4* d = (uint4*)(s_sp + ip * KD + j);
      d[0] = make_uint4(o[0], o[1], o[2], o[3]);
      d[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
  __syncthreads();

  const long long row = (long long)blockIdx.x * DQ_THREADS + tid;
  if (row >= a.n_vec) return;
  const long long rec = a.slots ? a.slots[row] : row;
  float w[KD];
  const bool have = rec >= 0 && rec < a.n_records;
  if (!have) {
#pragma unroll
    for (int j = 0; j < KD; ++j) w[j] = 0.0f;
    store_row(a.out, a.out_dtype, row * a.out_stride, w);
    return;
  }
  uint32_t kw[IDXB / 4];
  const uint32_t* ip = (const uint32_t*)(a.idx + rec * a.idx_row_bytes);
#pragma unroll
  for (int k = 0; k < IDXB / 4; ++k) kw[k] = ip[k];
  float n_part[2];
  if (GROUPED) {
    const uint32_t nn = *(const uint32_t*)(a.norm + 2 * rec);
    n_part[0] = h2f(nn & 0xFFFFu);
    n_part[1] = h2f(nn >> 16);
  } else {
    n_part[0] = n_part[1] = h2f(a.norm[rec]);
  }
  // QJL term first: w_j = sum_i S_ij (2 bit_i - 1), two rows per dot2
  if constexpr (PROD) {
    const uint4 sv = *(const uint4*)(a.signs + rec * (KD / 8));
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int j = 0; j < KD; ++j) w[j] = 0.0f;
    const _Float16 one = (_Float16)1.0f, mone = (_Float16)-1.0f;
#pragma unroll 2
    for (int p = 0; p < KD / 2; ++p) {
      const uint32_t bits = (sw[p >> 4] >> (2 * (p & 15))) & 3u;
      const half2_t sgn = {(bits & 1u) ? one : mone, (bits & 2u) ? one : mone};
      const uint4* sp = (const uint4*)(s_sp + p * KD);
#pragma unroll
      for (int jc = 0; jc < KD / 4; ++jc) {
        const uint4 v = sp[jc];
        w[4 * jc + 0] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.x), sgn, w[4 * jc + 0], false);
        w[4 * jc + 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.y), sgn, w[4 * jc + 1], false);
        w[4 * jc + 2] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.z), sgn, w[4 * jc + 2], false);
        w[4 * jc + 3] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, v.w), sgn, w[4 * jc + 3], false);
      }
    }
    const float alpha = h2f(a.rnorm[rec]) * 1.2533141373155003f / (float)KD;  // rho sqrt(pi/2) / m
#pragma unroll
    for (int j = 0; j < KD; ++j) w[j] *= alpha;
  } else {
#pragma unroll
    for (int j = 0; j < KD; ++j) w[j] = 0.0f;
  }
  // codebook term: w_j += (n / sqrt(PD)) c[idx_j]
#pragma unroll
  for (int j = 0; j < KD; ++j) {
    const int part = GROUPED ? j / PD : 0;
    const int W = part ? W1 : W0;
    const int jl = j - part * PD;
    const int bit = (part ? PD * W0 : 0) + jl * W;  // bit offset inside the index row
    const uint32_t v = (kw[bit >> 5] >> (bit & 31)) & ((1u << W) - 1u);
    const float scale = n_part[part] * (part ? 0.125f : (GROUPED ? 0.125f : 0.08838834764831845f));
    w[j] = fmaf(scale, s_cent[part][v], w[j]);
  }
  fwht<PD>(w);
  if (GROUPED) fwht<PD>(w + PD);
  const float inv = GROUPED ? 0.125f : 0.08838834764831845f;  // 1 / sqrt(PD)
#pragma unroll
  for (int j = 0; j < KD; ++j) w[j] *= s_sig[j] * inv;
  store_row(a.out, a.out_dtype, row * a.out_stride, w);
}

struct DqValArgs {
  long long n_vec;
  const long long* slots;
  long long n_records;
  const uint8_t* codes;
  const uint16_t* scale;
  const uint16_t* zero;
  void* out;
  int out_dtype;
  long long out_stride;
};

template <int BITS>
__global__ __launch_bounds__(DQ_THREADS) void dequant_values_kernel(DqValArgs a) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const long long row = ((long long)blockIdx.x * DQ_THREADS + threadIdx.x) >> 4;
  if (row >= a.n_vec) return;
  const long long rec = a.slots ? a.slots[row] : row;
  float v[8];
  if (rec >= 0 && rec < a.n_records) {
    const uint32_t c = BITS == 2 ? (uint32_t) * (const uint16_t*)(a.codes + rec * (KD * BITS / 8) + 2 * sub)
                                 : *(const uint32_t*)(a.codes + rec * (KD * BITS / 8) + 4 * sub);
    const float s = h2f(a.scale[rec * (KD / 32) + (sub >> 2)]);
    const float z = h2f(a.zero[rec * (KD / 32) + (sub >> 2)]);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fmaf((float)((c >> (BITS * i)) & ((1u << BITS) - 1u)), s, z);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  const long long off = row * a.out_stride + 8 * sub;
  if (a.out_dtype == TQ_F32) {
    float4* p = (float4*)((float*)a.out + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo, hi;
      if (a.out_dtype == TQ_BF16) {
        const uint32_t ua = __float_as_uint(v[2 * i]), ub = __float_as_uint(v[2 * i + 1]);
        lo = (ua + 0x7FFFu + ((ua >> 16) & 1u)) >> 16;
        hi = (ub + 0x7FFFu + ((ub >> 16) & 1u)) >> 16;
      } else {
        lo = __half_as_ushort(__float2half_rn(v[2 * i]));
        hi = __half_as_ushort(__float2half_rn(v[2 * i + 1]));
      }
      w[i] = lo | (hi << 16);
    }
    *(uint4*)((uint16_t*)a.out + off) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int MODE, int W0>
hipError_t launch_keys_w1(int w1, const DqKeyArgs& a, dim3 g, hipStream_t s) {
  switch (w1) {
    case 1: hipLaunchKernelGGL((dequant_keys_kernel<MODE, W0, 1>), g, dim3(DQ_THREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((dequant_keys_kernel<MODE, W0, 2>), g, dim3(DQ_THREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((dequant_keys_kernel<MODE, W0, 4>), g, dim3(DQ_THREADS), 0, s, a); break;
    default: hipLaunchKernelGGL((dequant_keys_kernel<MODE, W0, 8>), g, dim3(DQ_THREADS), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_keys(int w0, int w1, const DqKeyArgs& a, dim3 g, hipStream_t s) {
  if (MODE != TQ_MODE_GROUPED && MODE != TQ_MODE_GROUPED_PROD) w1 = 1;
  switch (w0) {
    case 1: return launch_keys_w1<MODE, 1>(w1, a, g, s);
    case 2: return launch_keys_w1<MODE, 2>(w1, a, g, s);
    case 4: return launch_keys_w1<MODE, 4>(w1, a, g, s);
    default: return launch_keys_w1<MODE, 8>(w1, a, g, s);
  }
}

bool out_ok(void* out, int dt, long long stride) {
  if (!out || !tq::aligned16(out)) return false;
  if (dt != TQ_F32 && dt != TQ_BF16 && dt != TQ_F16) return false;
  const int esz = dt == TQ_F32 ? 4 : 2;
  return stride >= KD && (stride * esz) % 16 == 0;
}

}  // namespace

extern "C" tq_status tq_dequantize_keys(const tq_key_config* cfg, const void* tables, int64_t n_vec,
                                       const int64_t* slots, int64_t n_records, const uint8_t* idx,
                                       const uint8_t* signs, const uint16_t* norm, const uint16_t* rnorm,
                                       void* out, int32_t out_dtype, int64_t out_stride, void* stream) {
  tq::Parts P;
  tq_status st = tq::describe(cfg, &P);
  if (st != TQ_OK) return st;
  if (P.d != KD) return TQ_ERR_UNSUPPORTED;
  if (n_vec < 0 || n_records < 0) return TQ_ERR_ARG;
  if (!out_ok(out, out_dtype, out_stride) && n_vec > 0) return TQ_ERR_ARG;
  if (n_vec == 0) return TQ_OK;
  if (!tables || !idx || !norm || !tq::aligned16(tables) || !tq::aligned16(idx) || ((uintptr_t)norm & 3))
    return TQ_ERR_ARG;
  if (P.m > 0 && (!signs || !rnorm || !tq::aligned16(signs) || ((uintptr_t)rnorm & 1)))
    return TQ_ERR_ARG;
  if (slots && ((uintptr_t)slots & 7)) return TQ_ERR_ARG;
  DqKeyArgs a;
  a.tables = (const unsigned char*)tables;
  a.n_vec = n_vec;
  a.slots = (const long long*)slots;
  a.n_records = n_records;
  a.idx = idx;
  a.signs = signs;
  a.norm = norm;
  a.rnorm = rnorm;
  a.out = out;
  a.out_dtype = out_dtype;
  a.out_stride = out_stride;
  a.idx_row_bytes = P.idx_row_bytes;
  const long long blocks = (n_vec + DQ_THREADS - 1) / DQ_THREADS;
  if (blocks > 0x7fffffffLL) return TQ_ERR_ARG;
  const dim3 g((unsigned)blocks);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (P.mode == TQ_MODE_MSE) e = launch_keys<TQ_MODE_MSE>(P.part_width[0], 1, a, g, s);
  else if (P.mode == TQ_MODE_PROD) e = launch_keys<TQ_MODE_PROD>(P.part_width[0], 1, a, g, s);
  else if (P.mode == TQ_MODE_GROUPED) e = launch_keys<TQ_MODE_GROUPED>(P.part_width[0], P.part_width[1], a, g, s);
  else e = launch_keys<TQ_MODE_GROUPED_PROD>(P.part_width[0], P.part_width[1], a, g, s);
  return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

extern "C" tq_status tq_dequantize_values(int32_t bits, int32_t group, int32_t d, int64_t n_vec,
                                         const int64_t* slots, int64_t n_records, const uint8_t* codes,
                                         const uint16_t* scale, const uint16_t* zero, void* out,
                                         int32_t out_dtype, int64_t out_stride, void* stream) {
  if (bits != 2 && bits != 4) return TQ_ERR_UNSUPPORTED;
  if (group != 32 || d != KD) return TQ_ERR_UNSUPPORTED;
  if (n_vec < 0 || n_records < 0) return TQ_ERR_ARG;
  if (!out_ok(out, out_dtype, out_stride) && n_vec > 0) return TQ_ERR_ARG;
  if (n_vec == 0) return TQ_OK;
  if (!codes || !scale || !zero || !tq::aligned16(codes) || ((uintptr_t)scale & 1) || ((uintptr_t)zero & 1))
    return TQ_ERR_ARG;
  if (slots && ((uintptr_t)slots & 7)) return TQ_ERR_ARG;
  DqValArgs a;
  a.n_vec = n_vec;
  a.slots = (const long long*)slots;
  a.n_records = n_records;
  a.codes = codes;
  a.scale = scale;
  a.zero = zero;
  a.out = out;
  a.out_dtype = out_dtype;
  a.out_stride = out_stride;
  const long long blocks = (n_vec * 16 + DQ_THREADS - 1) / DQ_THREADS;
  if (blocks > 0x7fffffffLL) return TQ_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (bits == 2) hipLaunchKernelGGL(dequant_values_kernel<2>, dim3((unsigned)blocks), dim3(DQ_THREADS), 0, s, a);
  else hipLaunchKernelGGL(dequant_values_kernel<4>, dim3((unsigned)blocks), dim3(DQ_THREADS), 0, s, a);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
