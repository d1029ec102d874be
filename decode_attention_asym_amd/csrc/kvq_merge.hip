// kvq_merge.hip -- the cross-split merge of decode attention partials.
//
// Each split of a row leaves o (unnormalized), m and l in the base-2 domain;
// the merge is the exact log-sum-exp combination of softmax pieces over
// disjoint token ranges (the split-K decode of the attention in "Asymmetric
// Key-Value Quantization: 2-Bit Values and 4-Bit Keys under Long-Context
// Drift", section 1, computed in parts).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Merge the split partials of one (batch, query head) row:
// M = max m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s (log2 domain);
// empty splits (m = -inf) contribute nothing.  One block of 256 threads per
// row, S <= 256: thread t first owns split t's weight; then it accumulates
// channels 4q..4q+3 (q = t % (D/4)) over the splits s = t / (D/4) (mod
// 256 / (D/4)), so every split record is read once, as 16-byte loads with
// several of them in flight per thread, and the split lanes are summed in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeMaxSplits = kMergeThreads;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ partial, float* __restrict__ out,
                                                              int S) {
  constexpr int Q = D / 4, NS = kMergeThreads / Q, W = D + 4, NW = kMergeThreads / kLanes;
  __shared__ float wsh[kMergeMaxSplits];
  __shared__ float red[2][NW];
  __shared__ f32x4 osh[NS][Q];
  const int t = threadIdx.x, lane = t % kLanes, wv = t / kLanes;
  const float* pr = partial + static_cast<int64_t>(blockIdx.x) * S * W;
  const int q = t % Q, sp = t / Q;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // the first four records of this thread go out with the weights' loads,
  // so the block waits for one round trip to memory instead of two
  f32x4 v0[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    v0[k] = sp + k * NS < S ? *reinterpret_cast<const f32x4*>(pr + (sp + k * NS) * W + 4 * q) : zero4;

  const float ms = t < S ? pr[t * W + D] : -INFINITY;
  const float ls = t < S ? pr[t * W + D + 1] : 0.0f;
  float x = ms;
#pragma unroll
  for (int o = kLanes / 2; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  if (lane == 0) red[0][wv] = x;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red[0][i]);
  const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
  float lw = w == 0.0f ? 0.0f : w * ls;
#pragma unroll
  for (int o = kLanes / 2; o >= 1; o >>= 1) lw += __shfl_xor(lw, o);
  if (lane == 0) red[1][wv] = lw;
  wsh[t] = w;
  __syncthreads();

  // four records in flight per thread; an empty split's record is never used
  // (its o may be anything), so it is selected away rather than scaled by 0
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float ws = sp + k * NS < S ? wsh[sp + k * NS] : 0.0f;
    acc += ws != 0.0f ? ws * v0[k] : zero4;
  }
  int s = sp + 4 * NS;
  for (; s + 3 * NS < S; s += 4 * NS) {
    f32x4 v[4];
    float ws[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = *reinterpret_cast<const f32x4*>(pr + (s + k * NS) * W + 4 * q);
#pragma unroll
    for (int k = 0; k < 4; ++k) ws[k] = wsh[s + k * NS];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += ws[k] != 0.0f ? ws[k] * v[k] : zero4;
  }
  for (; s < S; s += NS) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(pr + s * W + 4 * q);
    const float ws = wsh[s];
    acc += ws != 0.0f ? ws * v : zero4;
  }
  osh[sp][q] = acc;
  __syncthreads();
  if (sp == 0) {
    float L = red[1][0];
#pragma unroll
    for (int i = 1; i < NW; ++i) L += red[1][i];
#pragma unroll
    for (int i = 1; i < NS; ++i) acc += osh[i][q];
    *reinterpret_cast<f32x4*>(out + static_cast<int64_t>(blockIdx.x) * D + 4 * q) = acc / L;
  }
}

// The same merge with one wave per row, for S <= 64 records (the common
// case: the records of groups of four splits, or a few splits): lane t holds
// record t's m and l, the maximum and the weighted l-sum are wave
// reductions, and lane l accumulates channels 4q..4q+3 (q = l % (D/4)) over
// the records s = l / (D/4) (mod 64 / (D/4)), all of its loads in flight at
// once, eight at a time; the 64 / (D/4) lane groups are then summed with
// cross-lane moves.  No LDS and no barrier: four rows per 256-thread block.
constexpr int kMergeWaveMaxSplits = kLanes;
constexpr int kMergeWaveRows = 4;

template <int D>
__global__ __launch_bounds__(kLanes * kMergeWaveRows) void merge_wave_kernel(const float* __restrict__ partial,
                                                                              float* __restrict__ out, int rows,
                                                                              int S) {
  constexpr int Q = D / 4, NH = kLanes / Q, W = D + 4;
  const int l = threadIdx.x % kLanes;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kMergeWaveRows + threadIdx.x / kLanes;
  if (row >= rows) return;  // whole waves: the row is wave-uniform
  const float* pr = partial + row * S * W;
  const int q = l % Q, h = l / Q;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // the first eight records of this lane go out with the m / l loads
  f32x4 v0[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int sp = h + k * NH;
    v0[k] = sp < S ? *reinterpret_cast<const f32x4*>(pr + sp * W + 4 * q) : zero4;
  }
  const float ms = l < S ? pr[l * W + D] : -INFINITY;
  const float ls = l < S ? pr[l * W + D + 1] : 0.0f;
  float M = ms;
#pragma unroll
  for (int o = kLanes / 2; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  // an empty record (m = -inf) has weight 0 and its o and l are never used
  const float w = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
  float L = w == 0.0f ? 0.0f : w * ls;
#pragma unroll
  for (int o = kLanes / 2; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  f32x4 acc = zero4;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float ws = __shfl(w, (h + k * NH) % kLanes);
    acc += h + k * NH < S && ws != 0.0f ? ws * v0[k] : zero4;
  }
  // (the loop bound is wave-uniform: every lane takes part in the weight
  // shuffles, whose source lanes must be active)
  for (int base = 8 * NH; base < S; base += 8 * NH) {
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int sp = base + h + k * NH;
      v[k] = sp < S ? *reinterpret_cast<const f32x4*>(pr + sp * W + 4 * q) : zero4;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int sp = base + h + k * NH;
      const float ws = __shfl(w, sp % kLanes);
      acc += sp < S && ws != 0.0f ? ws * v[k] : zero4;
    }
  }
  // sum the lane groups (lanes q, q + Q, ...): a butterfly over the group bits
#pragma unroll
  for (int o = Q; o < kLanes; o <<= 1) {
    acc[0] += __shfl_xor(acc[0], o);
    acc[1] += __shfl_xor(acc[1], o);
    acc[2] += __shfl_xor(acc[2], o);
    acc[3] += __shfl_xor(acc[3], o);
  }
  if (h == 0) *reinterpret_cast<f32x4*>(out + row * D + 4 * q) = acc / L;
}

}  // namespace

hipError_t launch_merge(const float* partial, float* out, int rows, int splits, int D, hipStream_t s) {
  if (splits < 1 || splits > kMergeMaxSplits || (D != 64 && D != 128) || rows < 1) return hipErrorInvalidValue;
  if (splits <= kMergeWaveMaxSplits) {
    const dim3 grid(static_cast<unsigned>((rows + kMergeWaveRows - 1) / kMergeWaveRows)), block(kLanes * kMergeWaveRows);
    if (D == 64)
      hipLaunchKernelGGL(merge_wave_kernel<64>, grid, block, 0, s, partial, out, rows, splits);
    else
      hipLaunchKernelGGL(merge_wave_kernel<128>, grid, block, 0, s, partial, out, rows, splits);
  } else if (D == 64) {
    hipLaunchKernelGGL(merge_kernel<64>, dim3(static_cast<unsigned>(rows)), dim3(kMergeThreads), 0, s, partial, out, splits);
  } else {
    hipLaunchKernelGGL(merge_kernel<128>, dim3(static_cast<unsigned>(rows)), dim3(kMergeThreads), 0, s, partial, out, splits);
  }
  return hipGetLastError();
}

}  // namespace kvq
