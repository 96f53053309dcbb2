// Read-bandwidth reference for the roofline: one streaming pass over a device
// buffer with 16-byte nontemporal loads, the access the decode makes of the
// packed cache (every byte read once).  What it reaches on a given GPU is the
// practical ceiling the decode's achieved bandwidth is set against, next to
// the specification's peak.
#include <hip/hip_runtime.h>

#include "tq.h"
#include "tq_internal.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int PR_THREADS = 256;
constexpr int PR_BLOCKS = TQ_STREAM_READ_SINK / PR_THREADS;  // one block per CU on a 256-CU GPU
constexpr int PR_UNROLL = 8;                                 // loads in flight per thread

// Thread i reads words i, i + T, i + 2T, ... (T threads in all), eight at a
// time, and folds them with xor into one word of the sink, so that no load
// can be dropped.
__global__ __launch_bounds__(PR_THREADS) void stream_read_kernel(const u32x4_t* __restrict__ p, long long n,
                                                                 uint32_t* sink) {
  const long long T = (long long)gridDim.x * PR_THREADS;
  long long i = (long long)blockIdx.x * PR_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (PR_UNROLL - 1) * T < n; i += PR_UNROLL * T) {
    u32x4_t v[PR_UNROLL];
#pragma unroll
    for (int u = 0; u < PR_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * T);
#pragma unroll
    for (int u = 0; u < PR_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += T) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[(long long)blockIdx.x * PR_THREADS + threadIdx.x] = acc;
}

}  // namespace

extern "C" tq_status tq_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || (bytes & 15) || !tq::aligned16(src) || ((uintptr_t)sink & 3))
    return TQ_ERR_ARG;
  hipLaunchKernelGGL(stream_read_kernel, dim3(PR_BLOCKS), dim3(PR_THREADS), 0, (hipStream_t)stream,
                     (const u32x4_t*)src, (long long)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}
