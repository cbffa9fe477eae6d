// lsa_device.h -- device-side helpers shared by the gfx950 kernels of the path.
//
// MFMA lane layouts used below (checked on gfx950 with an in-bounds probe):
//   v_mfma_i32_16x16x64_i8 / v_mfma_f32_16x16x32_bf16: lane l supplies row (l & 15)
//   of A and column (l & 15) of B, each with 16 bytes of the K dimension; the K
//   chunk a lane supplies is chosen by l >> 4 and is the SAME for A and B, so any
//   consistent assignment of K elements to (l >> 4, register bytes) gives the
//   full dot product.  Output register i of lane l holds C[4*(l>>4) + i][l & 15].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Exchange between the two 32-lane halves: returns, in every lane, the sum of
// "a" of the lower-half lane and "b" of the upper-half lane that pair up
// (lane l < 32 gets a[l] + a[l+32]; lane l >= 32 gets b[l-32] + b[l]).
__device__ __forceinline__ int xhalf32_sum(int a, int b) {
  auto r = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)b, false, false);
  return (int)(r[0] + r[1]);
}
// Same between 16-lane rows inside each half (rows 0<->1, 2<->3).
__device__ __forceinline__ int xrow16_sum(int a, int b) {
  auto r = __builtin_amdgcn_permlane16_swap((unsigned)a, (unsigned)b, false, false);
  return (int)(r[0] + r[1]);
}
__device__ __forceinline__ long long xhalf32_sum64(long long a, long long b) {
  auto lo = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)b, false, false);
  auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(a >> 32), (unsigned)(b >> 32), false, false);
  long long x = (long long)(((unsigned long long)hi[0] << 32) | lo[0]);
  long long y = (long long)(((unsigned long long)hi[1] << 32) | lo[1]);
  return x + y;
}
__device__ __forceinline__ long long xrow16_sum64(long long a, long long b) {
  auto lo = __builtin_amdgcn_permlane16_swap((unsigned)a, (unsigned)b, false, false);
  auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(a >> 32), (unsigned)(b >> 32), false, false);
  long long x = (long long)(((unsigned long long)hi[0] << 32) | lo[0]);
  long long y = (long long)(((unsigned long long)hi[1] << 32) | lo[1]);
  return x + y;
}

__device__ __forceinline__ int wave_max(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_maxf(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Count of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0));
}

// Block-wide exclusive prefix sum of one int per thread (NT threads, NT/64 waves).
// `tmp` needs NT/64 + 1 ints of LDS.  Returns the exclusive prefix; *total gets the sum.
// Contains two __syncthreads; every thread of the block must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / 64;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    int c = tmp[w];
    off += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

}  // namespace lsa
