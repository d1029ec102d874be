// kvq_drift.hip -- drift detection over quantized groups: per-group key and
// value code histograms and their KL divergence from calibration histograms.
//
// "Asymmetric Key-Value Quantization: 2-Bit Values and 4-Bit Keys under
// Long-Context Drift", section 3.3: the divergence of the current
// distribution of quantized values from the calibration distribution,
// D_KL(p_cur || p_cal) = sum_i p_cur(i) ln(p_cur(i) / p_cal(i)), a threshold
// (0.1 by default) marking the token range for requantization.  Here a
// group's distribution is the histogram of its G x D key codes (and of its
// value codes); the calibration is a histogram of code counts per kv head.
//
// One wave per (group, slice).  Codes are counted without unpacking them: b
// code words (b = bit width) are folded into b bit planes of 32 codes each
// (plane k holds bit k of every code), the count of value v is the popcount
// of the AND of the planes or their complements, and the 2^b per-lane counts
// are summed over the wave by a reduce-scatter (each exchange halves the
// counters a lane keeps), so each lane ends with the total of one bin.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int B>
constexpr uint32_t plane_mask() { return B == 4 ? 0x11111111u : 0x55555555u; }

// Adds the counts of the 32 / B codes in each of B words w[0..B) to cnt[2^B].
template <int B>
__device__ __forceinline__ void count_words(const uint32_t (&w)[B], uint32_t (&cnt)[1 << B]) {
  constexpr uint32_t M = plane_mask<B>();
  uint32_t P[B];
#pragma unroll
  for (int k = 0; k < B; ++k) {
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < B; ++j) x |= ((w[j] >> k) & M) << j;
    P[k] = x;  // bit (B * i + j) = bit k of code i of word j
  }
  if constexpr (B == 2) {
    const uint32_t n0 = ~P[0], n1 = ~P[1];
    cnt[0] += __builtin_popcount(n0 & n1);
    cnt[1] += __builtin_popcount(P[0] & n1);
    cnt[2] += __builtin_popcount(n0 & P[1]);
    cnt[3] += __builtin_popcount(P[0] & P[1]);
  } else {
    const uint32_t n0 = ~P[0], n1 = ~P[1], n2 = ~P[2], n3 = ~P[3];
    const uint32_t lo[4] = {n0 & n1, P[0] & n1, n0 & P[1], P[0] & P[1]};
    const uint32_t hi[4] = {n2 & n3, P[2] & n3, n2 & P[3], P[2] & P[3]};
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int l = 0; l < 4; ++l) cnt[4 * h + l] += __builtin_popcount(lo[l] & hi[h]);
  }
}

// Counts of the codes in BYTES contiguous bytes at p (a multiple of 1 KiB or
// 512 B), spread over the wave's lanes.
template <int B, int BYTES>
__device__ __forceinline__ void count_block(const uint8_t* p, int l, uint32_t (&cnt)[1 << B]) {
  constexpr int DW = BYTES / 4 / kLanes;  // dwords per lane
  static_assert(BYTES % (4 * kLanes) == 0 && DW % B == 0, "whole bit-plane batches per lane");
  uint32_t w[DW];
  if constexpr (DW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
      const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + i * kLanes + l);
      w[4 * i] = x[0]; w[4 * i + 1] = x[1]; w[4 * i + 2] = x[2]; w[4 * i + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < DW; ++i) w[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p) + i * kLanes + l);
  }
#pragma unroll
  for (int i = 0; i < DW / B; ++i) {
    uint32_t ww[B];
#pragma unroll
    for (int j = 0; j < B; ++j) ww[j] = w[B * i + j];
    count_words<B>(ww, cnt);
  }
}

// Reduce-scatter of NB per-lane counters over the 64 lanes: the exchange with
// the lane MASK = 64 S / NB away (S = NB/2, NB/4, .., 1) keeps the upper or
// lower S counters, so afterwards lane l holds in x[0] the sum over 2^log2(NB)
// lanes of bin ((l >> (6 - log2 NB)) & (NB - 1)) (lane bit 5 selects the
// upper half first); the remaining exchanges sum it over the other lanes.
template <int NB, int S>
__device__ __forceinline__ void reduce_scatter(uint32_t (&x)[NB], int l) {
  if constexpr (S >= 1) {
    constexpr int MASK = 64 * S / NB;
    const bool upper = (l & MASK) != 0;
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const uint32_t give = upper ? x[i] : x[i + S];
      const uint32_t keep = upper ? x[i + S] : x[i];
      x[i] = keep + static_cast<uint32_t>(__shfl_xor(static_cast<int>(give), MASK));
    }
    reduce_scatter<NB, S / 2>(x, l);
  }
}
template <int NB>
__device__ __forceinline__ uint32_t wave_bins(uint32_t (&x)[NB], int l) {
  reduce_scatter<NB, NB / 2>(x, l);
  uint32_t t = x[0];
#pragma unroll
  for (int m = 32 / NB; m >= 1; m /= 2) t += static_cast<uint32_t>(__shfl_xor(static_cast<int>(t), m));
  return t;
}
template <int NB>
__device__ __forceinline__ int bin_of_lane(int l) {
  constexpr int LOG = NB == 16 ? 4 : 2;
  return (l >> (6 - LOG)) & (NB - 1);
}

// KL term of one bin: p ln(p / q), 0 for p = 0, +inf for p > 0 = q (fp64;
// p = c / per with per = G * D a power of two, so c * (1 / per) is exact).
__device__ __forceinline__ double kl_term(uint32_t c, double inv_per, uint64_t cq, double tot) {
  if (c == 0) return 0.0;
  if (cq == 0) return __builtin_inf();
  const double p = static_cast<double>(c) * inv_per;
  const double q = static_cast<double>(cq) / tot;
  return p * log(p / q);
}

__device__ __forceinline__ double wave_sum_f64(double t) {
#pragma unroll
  for (int m = 32; m >= 1; m /= 2) t += __shfl_xor(t, m);
  return t;
}

template <int D, int KB, int VB, int G, bool HIST>
__global__ __launch_bounds__(64) void drift_kernel(DriftArgs a) {
  constexpr int NBK = 1 << KB, NBV = 1 << VB;
  constexpr int KBYTES = G * D * KB / 8, VBYTES = G * D * VB / 8;
  const Layout& L = a.L;
  const int l = threadIdx.x;
  const int64_t g = a.g0 + blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int hkv = static_cast<int>(slice % a.Hkv);
  const uint8_t* page = a.cache + page_offset(L, slice, g);
  uint32_t ck[NBK], cv[NBV];
#pragma unroll
  for (int i = 0; i < NBK; ++i) ck[i] = 0;
#pragma unroll
  for (int i = 0; i < NBV; ++i) cv[i] = 0;
  count_block<KB, KBYTES>(page + L.off_kcodes, l, ck);
  count_block<VB, VBYTES>(page + L.off_vcodes, l, cv);
  const uint32_t tk = wave_bins<NBK>(ck, l), tv = wave_bins<NBV>(cv, l);
  const int bk = bin_of_lane<NBK>(l), bv = bin_of_lane<NBV>(l);
  if constexpr (HIST) {
    if ((l & (64 / NBK - 1)) == 0) atomicAdd(reinterpret_cast<unsigned long long*>(a.hist_k) + hkv * NBK + bk, tk);
    if ((l & (64 / NBV - 1)) == 0) atomicAdd(reinterpret_cast<unsigned long long*>(a.hist_v) + hkv * NBV + bv, tv);
  } else {
    // calibration totals
    const uint64_t* qk = a.cal_k + hkv * NBK;
    const uint64_t* qv = a.cal_v + hkv * NBV;
    uint64_t sk = 0, sv = 0;
#pragma unroll
    for (int i = 0; i < NBK; ++i) sk += qk[i];
#pragma unroll
    for (int i = 0; i < NBV; ++i) sv += qv[i];
    static_assert(((G * D) & (G * D - 1)) == 0, "G * D is a power of two");
    // one term per lane: key bin bk in the first lane of each key bin's lanes,
    // value bin bv in the second lane of each value bin's lanes, so one fp64
    // logarithm serves both
    const bool kl = (l & (64 / NBK - 1)) == 0, vl = (l & (64 / NBV - 1)) == 1;
    const double term = kl_term(kl ? tk : (vl ? tv : 0u), 1.0 / static_cast<double>(G * D),
                                kl ? qk[bk] : qv[bv], static_cast<double>(kl ? sk : sv));
    const double klk = wave_sum_f64(kl ? term : 0.0);
    const double klv = wave_sum_f64(vl ? term : 0.0);
    if (l == 0) {
      const int64_t o = slice * a.ng + (g - a.g0);
      a.kl_k[o] = klk;
      a.kl_v[o] = klv;
      a.flags[o] = static_cast<uint8_t>((klk > a.threshold ? 1 : 0) | (klv > a.threshold ? 2 : 0));
    }
  }
}

__global__ void fill_u64_kernel(uint64_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int D, int KB, int VB, int G>
hipError_t drift_t(const DriftArgs& a, bool hist, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(a.ng), static_cast<unsigned>(a.L.slices));
  if (hist)
    hipLaunchKernelGGL((drift_kernel<D, KB, VB, G, true>), grid, dim3(kLanes), 0, s, a);
  else
    hipLaunchKernelGGL((drift_kernel<D, KB, VB, G, false>), grid, dim3(kLanes), 0, s, a);
  return hipGetLastError();
}
template <int D, int KB, int VB>
hipError_t drift_g(const DriftArgs& a, bool hist, hipStream_t s) {
  return a.L.G == 32 ? drift_t<D, KB, VB, 32>(a, hist, s) : drift_t<D, KB, VB, 64>(a, hist, s);
}
template <int D, int KB>
hipError_t drift_v(const DriftArgs& a, bool hist, hipStream_t s) {
  return a.L.vbits == 2 ? drift_g<D, KB, 2>(a, hist, s) : drift_g<D, KB, 4>(a, hist, s);
}
template <int D>
hipError_t drift_k(const DriftArgs& a, bool hist, hipStream_t s) {
  return a.L.kbits == 2 ? drift_v<D, 2>(a, hist, s) : drift_v<D, 4>(a, hist, s);
}

}  // namespace

hipError_t launch_code_histograms(const DriftArgs& a, hipStream_t s) {
  const int64_t nk = static_cast<int64_t>(a.Hkv) << a.L.kbits, nv = static_cast<int64_t>(a.Hkv) << a.L.vbits;
  hipLaunchKernelGGL(fill_u64_kernel, dim3(static_cast<unsigned>((nk + 255) / 256)), dim3(256), 0, s, a.hist_k, nk);
  hipLaunchKernelGGL(fill_u64_kernel, dim3(static_cast<unsigned>((nv + 255) / 256)), dim3(256), 0, s, a.hist_v, nv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ng <= 0) return e;
  return a.L.D == 64 ? drift_k<64>(a, true, s) : drift_k<128>(a, true, s);
}

hipError_t launch_drift_check(const DriftArgs& a, hipStream_t s) {
  if (a.ng <= 0) return hipSuccess;
  return a.L.D == 64 ? drift_k<64>(a, false, s) : drift_k<128>(a, false, s);
}

}  // namespace kvq
