// Per-channel moments of a set of key rows, and the outlier channels of the
// grouped modes chosen from them ("tqlite" README, mode table: the
// high-variance channels get the higher bit width).  Deterministic two-pass
// reduction in float64: each block sums a fixed range of rows per channel;
// one block then adds the partial sums in block order and, for the
// selection, ranks the channels by variance.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include "tq.h"
#include "tq_internal.h"

namespace {

constexpr int KD = 128;
constexpr int ST_THREADS = 256;          // 2 row lanes x 128 channels
constexpr int ROWS_PER_BLOCK = 1024;

__device__ inline float load1(const void* x, int dt, long long i) {
  if (dt == TQ_F32) return ((const float*)x)[i];
  const uint16_t v = ((const uint16_t*)x)[i];
  if (dt == TQ_BF16) return __uint_as_float((uint32_t)v << 16);
  return __half2float(__ushort_as_half(v));
}

__global__ __launch_bounds__(ST_THREADS) void moments_partial(const void* x, int dt, long long n,
                                                              long long stride, double* part) {
  const int c = threadIdx.x % KD, r0 = threadIdx.x / KD;
  const long long first = (long long)blockIdx.x * ROWS_PER_BLOCK;
  const long long last = first + ROWS_PER_BLOCK < n ? first + ROWS_PER_BLOCK : n;
  double s = 0.0, q = 0.0;
  for (long long r = first + r0; r < last; r += ST_THREADS / KD) {
    const double v = (double)load1(x, dt, r * stride + c);
    s += v;
    q = fma(v, v, q);
  }
  __shared__ double sh[2][ST_THREADS];
  sh[0][threadIdx.x] = s;
  sh[1][threadIdx.x] = q;
  __syncthreads();
  if (threadIdx.x < KD) {
    double S = 0.0, Q = 0.0;
    for (int k = 0; k < ST_THREADS / KD; ++k) {
      S += sh[0][k * KD + threadIdx.x];
      Q += sh[1][k * KD + threadIdx.x];
    }
    part[((long long)blockIdx.x * 2 + 0) * KD + threadIdx.x] = S;
    part[((long long)blockIdx.x * 2 + 1) * KD + threadIdx.x] = Q;
  }
}

__global__ __launch_bounds__(KD) void moments_final(const double* part, int n_blocks, double* out) {
  double S = 0.0, Q = 0.0;
  for (int b = 0; b < n_blocks; ++b) {
    S += part[((long long)b * 2 + 0) * KD + threadIdx.x];
    Q += part[((long long)b * 2 + 1) * KD + threadIdx.x];
  }
  out[threadIdx.x] = S;
  out[KD + threadIdx.x] = Q;
}

// One thread per channel: the variance from the summed moments, its rank
// among the channels (larger variance first, the lower channel first among
// equals), then the channel's place in the order: chosen channels first, each
// group in increasing channel order.
__global__ __launch_bounds__(KD) void select_final(const double* part, int n_blocks, long long n, int n_outlier,
                                                   int* perm) {
  __shared__ double var[KD];
  __shared__ int chosen[KD];
  const int c = threadIdx.x;
  double S = 0.0, Q = 0.0;
  for (int b = 0; b < n_blocks; ++b) {
    S += part[((long long)b * 2 + 0) * KD + c];
    Q += part[((long long)b * 2 + 1) * KD + c];
  }
  const double mean = n > 0 ? S / (double)n : 0.0;
  var[c] = n > 0 ? Q / (double)n - mean * mean : 0.0;
  __syncthreads();
  const double v = var[c];
  int rank = 0;
  for (int j = 0; j < KD; ++j) rank += (var[j] > v || (var[j] == v && j < c)) ? 1 : 0;
  const int mine = rank < n_outlier ? 1 : 0;
  chosen[c] = mine;
  __syncthreads();
  int before = 0;  // channels below c in the same group
  for (int j = 0; j < c; ++j) before += chosen[j] == mine ? 1 : 0;
  perm[mine ? before : n_outlier + before] = c;
}

size_t moment_workspace(long long n_vec) {
  const long long blocks = n_vec > 0 ? (n_vec + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK : 1;
  return (size_t)blocks * 2 * KD * sizeof(double);
}

}  // namespace

extern "C" tq_status tq_select_outlier_channels(const void* x, int32_t dtype, int64_t n_vec, int64_t row_stride,
                                               int32_t d, int32_t n_outlier, int32_t* perm, void* workspace,
                                               size_t* workspace_bytes, void* stream) {
  if (d != KD) return TQ_ERR_UNSUPPORTED;
  if (n_vec < 0 || !workspace_bytes || n_outlier < 0 || n_outlier > KD) return TQ_ERR_ARG;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_ERR_ARG;
  const long long blocks = n_vec > 0 ? (n_vec + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK : 1;
  if (blocks > 0x7fffffffLL) return TQ_ERR_ARG;
  const size_t need = moment_workspace(n_vec);
  if (!workspace) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) return TQ_ERR_WORKSPACE;
  if (!perm || ((uintptr_t)perm & 3) || ((uintptr_t)workspace & 7)) return TQ_ERR_ARG;
  if (n_vec > 0 && (!x || row_stride < KD)) return TQ_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (n_vec > 0)
    hipLaunchKernelGGL(moments_partial, dim3((unsigned)blocks), dim3(ST_THREADS), 0, s, x, dtype, n_vec,
                       row_stride, (double*)workspace);
  hipLaunchKernelGGL(select_final, dim3(1), dim3(KD), 0, s, (const double*)workspace, n_vec > 0 ? (int)blocks : 0,
                     (long long)n_vec, (int)n_outlier, perm);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

extern "C" tq_status tq_channel_moments(const void* x, int32_t dtype, int64_t n_vec, int64_t row_stride,
                                       int32_t d, double* out, void* workspace, size_t* workspace_bytes,
                                       void* stream) {
  if (d != KD) return TQ_ERR_UNSUPPORTED;
  if (n_vec < 0 || !workspace_bytes) return TQ_ERR_ARG;
  if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16) return TQ_ERR_ARG;
  const long long blocks = n_vec > 0 ? (n_vec + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK : 1;
  if (blocks > 0x7fffffffLL) return TQ_ERR_ARG;
  const size_t need = moment_workspace(n_vec);
  if (!workspace) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) return TQ_ERR_WORKSPACE;
  if (!out || ((uintptr_t)out & 7) || ((uintptr_t)workspace & 7)) return TQ_ERR_ARG;
  if (n_vec > 0 && (!x || row_stride < KD)) return TQ_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (n_vec > 0)
    hipLaunchKernelGGL(moments_partial, dim3((unsigned)blocks), dim3(ST_THREADS), 0, s, x, dtype, n_vec,
                       row_stride, (double*)workspace);
  hipLaunchKernelGGL(moments_final, dim3(1), dim3(KD), 0, s, (const double*)workspace,
                     n_vec > 0 ? (int)blocks : 0, out);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
