// lsa_idx_tiles.h -- the int8 MFMA tile helpers of the indexer kernels: fragment layout,
// query loading, the weighted-ReLU epilogue op and the cross-lane sums.
#pragma once
#include "lsa_device.h"

namespace lsa {

// 16-byte chunk of the d_I bytes supplied by lane row g at K-step ks.  A and B
// use the same assignment, so the product is the full dot product.  At one K-step
// the four lane rows read four consecutive chunks, so every load instruction takes
// whole 64-byte pieces of its 16 key rows.
template <int D>
__device__ __forceinline__ int kchunk(int g, int ks) { return ks * 4 + g; }

// XOR swizzle of 16-byte chunk c of row r in an LDS key tile whose rows are RB
// bytes: 8 consecutive rows read at one logical chunk hit 8 distinct bank groups,
// and 8 consecutive chunks of one row (the staging writes) do too.
template <int RB>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (RB >= 128) return c ^ (r & 7);
  else return c ^ ((r >> 1) & 3);
}

// Four values: lane row g ends with the full sum of value g.
__device__ __forceinline__ int reduce_scatter4(const int (&v)[4]) {
  int r0 = xhalf32_sum(v[0], v[2]);
  int r1 = xhalf32_sum(v[1], v[3]);
  return xrow16_sum(r0, r1);
}
__device__ __forceinline__ void reduce_scatter8_64(const long long (&v)[8], long long (&out)[2]) {
  long long r1[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) r1[t] = xhalf32_sum64(v[t], v[4 + t]);
#pragma unroll
  for (int t = 0; t < 2; ++t) out[t] = xrow16_sum64(r1[t], r1[2 + t]);
}

// Requests the A fragments (index-query heads) and the raw head weights of one
// query.  Loads are unconditional (clamped to a valid head) so they are all in
// flight at once; query_weights() then gives a padding head weight 0, which
// cancels whatever its row produces.  Split in two so a caller can put more loads
// in flight before the weights are first used.
template <int D, int MT>
__device__ __forceinline__ void issue_query(const int8_t* __restrict__ q_idx, const int32_t* __restrict__ w,
                                            int w_per_query, long long row, int H_I, v4i (&A)[MT][D / 64],
                                            int (&wv)[MT][4]) {
  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
  const int32_t* wr = w + (w_per_query ? row * H_I : 0);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = min(16 * mt + r16, H_I - 1);
    const int8_t* qr = q_idx + (row * H_I + h) * D;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) A[mt][ks] = *(const v4i*)(qr + 16 * kchunk<D>(g, ks));
#pragma unroll
    for (int e = 0; e < 4; ++e) wv[mt][e] = wr[min(16 * mt + 4 * (lane >> 4) + e, H_I - 1)];
  }
}
template <int MT>
__device__ __forceinline__ void query_weights(const int (&wv)[MT][4], int H_I, bool valid, int (&wt)[MT][4]) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) wt[mt][e] = (valid && 16 * mt + 4 * g + e < H_I) ? wv[mt][e] : 0;
}
template <int D, int MT>
__device__ __forceinline__ void load_query(const int8_t* __restrict__ q_idx, const int32_t* __restrict__ w,
                                           int w_per_query, long long row, int H_I, bool valid,
                                           v4i (&A)[MT][D / 64], int (&wt)[MT][4]) {
  int wv[MT][4];
  issue_query<D, MT>(q_idx, w, w_per_query, row, H_I, A, wv);
  query_weights<MT>(wv, H_I, valid, wt);
}

constexpr int BUF_RSRC_WORD3 = 0x00020000;  // 32-bit data format, raw (untyped) access

// acc + max(x, 0) * w as one v_mad_i32_i24 (24-bit signed operands, 32-bit add).
// Written out because the compiler otherwise splits the chain into multiplies and
// three-way adds, which costs a quarter more VALU issue in the indexer epilogue --
// the part of the indexer that bounds it, since each VALU op here takes about as
// long to issue as a quarter of an int8 MFMA.
__device__ __forceinline__ int relu_mad24(int x, int w, int acc) {
  const int r = max(x, 0);
  asm("v_mad_i32_i24 %0, %1, %2, %0" : "+v"(acc) : "v"(r), "v"(w));
  return acc;
}
// max(x, 0) * w as one v_mul_i32_i24: the first term of a chain, so no register has
// to be set to zero for it.
__device__ __forceinline__ int relu_mul24(int x, int w) {
  const int r = max(x, 0);
  int p;
  asm("v_mul_i32_i24 %0, %1, %2" : "=v"(p) : "v"(r), "v"(w));
  return p;
}

// acc + max(x, 0) * w in 64 bits as one v_mad_i64_i32 (signed 32 x 32 -> 64-bit product
// plus a 64-bit add): the block scores' epilogue.  Written out because the compiler
// forms the widened product from two v_mad_u64_u32 and register moves, doubling the
// epilogue's VALU issue.  The instruction's carry-out goes to an SGPR pair nobody reads.
__device__ __forceinline__ long long relu_mad64(int x, int w, long long acc) {
  const int r = max(x, 0);
  unsigned long long carry;
  asm("v_mad_i64_i32 %0, %1, %2, %3, %0" : "+v"(acc), "=s"(carry) : "v"(w), "v"(r));
  return acc;
}
// max(x, 0) * w in 64 bits: the first term of a chain (the addend is the constant 0).
__device__ __forceinline__ long long relu_mul64(int x, int w) {
  const int r = max(x, 0);
  long long p;
  unsigned long long carry;
  asm("v_mad_i64_i32 %0, %1, %2, %3, 0" : "=v"(p), "=s"(carry) : "v"(w), "v"(r));
  return p;
}

}  // namespace lsa
