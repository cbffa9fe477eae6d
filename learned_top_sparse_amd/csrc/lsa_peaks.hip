// lsa_peaks.hip -- microbenchmarks of the ceilings the path's kernels are judged
// against on the machine itself (int8 and bf16 MFMA issue, HBM streaming read, random
// 256-byte row gathers).  Measurement only: no part of the method uses them.  The
// caller times each launch with events on the stream it passes.
#include <hip/hip_runtime.h>

#include "lsa_device.h"
#include "lsa_peaks.h"

#define LSA_API extern "C" __attribute__((visibility("default")))

namespace {

using lsa::v4f;
using lsa::v4i;
using lsa::v8bf;

constexpr int PK_NT = 256;  // threads per workgroup

// Four independent accumulator chains per wave, operands held in registers.
template <int KIND>
__global__ __launch_bounds__(PK_NT) void peak_mfma_kernel(long long iters, int32_t* __restrict__ sink) {
  const int tid = threadIdx.x;
  const int seed = (int)(blockIdx.x * PK_NT + tid);
  int out = 0;
  if constexpr (KIND == LSA_PEAK_MFMA_I8) {
    v4i a = v4i{seed, seed ^ 0x5a5a5a5a, seed * 3, seed + 7};
    v4i b = v4i{seed ^ 0x01010101, seed * 5, seed - 11, seed ^ 0x33333333};
    v4i c0 = v4i{0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    for (long long i = 0; i < iters; ++i) {
      c0 = lsa::mfma_i8(a, b, c0);
      c1 = lsa::mfma_i8(b, a, c1);
      c2 = lsa::mfma_i8(a, a, c2);
      c3 = lsa::mfma_i8(b, b, c3);
    }
    const v4i s = c0 + c1 + c2 + c3;
    out = s[0] ^ s[1] ^ s[2] ^ s[3];
  } else {
    v8bf a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(float)((seed + e) & 7);
      b[e] = (__bf16)(float)((seed ^ e) & 3);
    }
    v4f c0 = v4f{0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (long long i = 0; i < iters; ++i) {
      c0 = lsa::mfma_bf16(a, b, c0);
      c1 = lsa::mfma_bf16(b, a, c1);
      c2 = lsa::mfma_bf16(a, a, c2);
      c3 = lsa::mfma_bf16(b, b, c3);
    }
    const v4f s = c0 + c1 + c2 + c3;
    out = (int)(s[0] + s[1] + s[2] + s[3]);
  }
  sink[blockIdx.x * PK_NT + tid] = out;
}

// Streaming read: every 16-byte element once.  Workgroup x streams one contiguous span
// of the buffer (the chip's best read pattern among those measured: a grid-stride loop
// reached 6.0-6.1 TB/s, contiguous spans with plain loads 6.15, with non-temporal loads
// 6.7); every thread keeps eight 16-byte non-temporal loads in flight; the XOR of what a
// thread read goes to sink.
__global__ __launch_bounds__(PK_NT) void peak_read_kernel(const v4i* __restrict__ src, long long n16,
                                                          int32_t* __restrict__ sink) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long b0 = (long long)blockIdx.x * per;
  const long long b1 = b0 + per < n16 ? b0 + per : n16;
  v4i acc = v4i{0, 0, 0, 0};
  long long j = b0 + threadIdx.x;
  for (; j + 7 * PK_NT < b1; j += 8 * PK_NT) {
    v4i x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(src + j + u * PK_NT);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u];
  }
  for (; j < b1; j += PK_NT) acc ^= src[j];
  sink[blockIdx.x * PK_NT + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Random gather of 256-byte rows: 16 lanes read one row per load instruction (four
// rows per instruction), each wave walks its share of the index list with eight rows
// per lane group in flight.
__global__ __launch_bounds__(PK_NT) void peak_gather_kernel(const v4i* __restrict__ rows, long long n_rows,
                                                            const int32_t* __restrict__ idx, long long n_idx,
                                                            int32_t* __restrict__ sink) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63, grp = lane >> 4, c = lane & 15;
  const long long wave = ((long long)blockIdx.x * PK_NT + threadIdx.x) >> 6;
  const long long n_waves = (long long)gridDim.x * (PK_NT / 64);
  v4i acc = v4i{0, 0, 0, 0};
  // a wave's step covers 4 * U consecutive list entries
  for (long long base = wave * 4 * U; base < n_idx; base += n_waves * 4 * U) {
    int j[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long e = base + 4 * u + grp;
      const long long jj = e < n_idx ? idx[e] : 0;
      j[u] = (int)(jj < 0 ? 0 : (jj >= n_rows ? n_rows - 1 : jj));
    }
    v4i x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = rows[(long long)j[u] * 16 + c];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= x[u];
  }
  sink[blockIdx.x * PK_NT + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

LSA_API int32_t lsa_peak_sink_ints(int32_t n_blocks) { return n_blocks * PK_NT; }

LSA_API int lsa_peak_mfma(int32_t kind, int64_t iters, int32_t n_blocks, int32_t* sink, void* stream) {
  if ((kind != LSA_PEAK_MFMA_I8 && kind != LSA_PEAK_MFMA_BF16) || iters < 1 || n_blocks < 1 || !sink) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == LSA_PEAK_MFMA_I8)
    hipLaunchKernelGGL(peak_mfma_kernel<LSA_PEAK_MFMA_I8>, dim3(n_blocks), dim3(PK_NT), 0, st, (long long)iters, sink);
  else
    hipLaunchKernelGGL(peak_mfma_kernel<LSA_PEAK_MFMA_BF16>, dim3(n_blocks), dim3(PK_NT), 0, st, (long long)iters,
                       sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

LSA_API int lsa_peak_read(const void* src, int64_t bytes, int32_t n_blocks, int32_t* sink, void* stream) {
  if (!src || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)src) % 16 != 0 || n_blocks < 1 || !sink) return -1;
  hipLaunchKernelGGL(peak_read_kernel, dim3(n_blocks), dim3(PK_NT), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4i*>(src), (long long)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

LSA_API int lsa_peak_gather(const void* rows, int64_t n_rows, const int32_t* idx, int64_t n_idx, int32_t n_blocks,
                            int32_t* sink, void* stream) {
  if (!rows || n_rows < 1 || ((uintptr_t)rows) % 16 != 0 || !idx || n_idx < 1 || n_blocks < 1 || !sink) return -1;
  hipLaunchKernelGGL(peak_gather_kernel, dim3(n_blocks), dim3(PK_NT), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4i*>(rows), (long long)n_rows, idx, (long long)n_idx, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
