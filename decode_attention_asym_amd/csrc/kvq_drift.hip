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
// One wave per few consecutive groups of one slice.  Codes are counted
// without unpacking them: b code words (b = bit width) are transposed into b
// bit planes of 32 codes each (plane k holds bit k of every code), the count
// of value v is the popcount of the AND of the planes or their complements,
// and the 2^b per-lane counts are summed over the wave by a reduce-scatter
// (each exchange halves the counters a lane keeps), so each lane ends with
// the total of one bin.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Groups one KL pass covers: each bin's total sits in 64 / 2^b lanes after
// the reduction, so a pass can give every group's key and value bins a lane
// of their own while the lanes still cover a logarithm each: two groups when
// a width is 4 bits (16 bins in lanes of 4), four with 2-bit keys and values.
// A wave visits four consecutive groups of one slice (two passes, or one):
// the per-wave set-up (calibration probabilities, page addressing) is paid
// once for them, and with two passes the next pass's codes load while a pass
// is reduced.  (Eight groups per wave with 2-bit codes measured slower on the
// smaller caches: fewer waves.)
template <int KB, int VB>
constexpr int groups_per_pass() { return KB == 2 && VB == 2 ? 4 : 2; }
template <int KB, int VB>
constexpr int groups_per_wave() { return 4; }

// Bits of a where m is set, bits of b elsewhere.
__device__ __forceinline__ uint32_t pick(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }
// The value x, opaque to the optimizer (no instruction): keeps the compiler
// from folding the plane transposes into the count products, which it
// otherwise expands into more instructions than it saves.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

// Counting works on bit planes: B words of B-bit codes are transposed so that
// plane k holds bit k of every one of their 32 codes (the same bit position in
// every plane belongs to the same code); the number of codes equal to v is then
// the popcount of the AND of the planes (or their complements) selected by v.
// Counts of the value whose low (and high) bits are all zero are not formed
// per batch: they follow at the end from the number of codes a lane counted.
//
// Two 2-bit words: bit 2i + j of plane k is bit k of code i of word j.
// Adds to c[1..3].
__device__ __forceinline__ void count_batch2(uint32_t w0, uint32_t w1, uint32_t (&c)[4]) {
  const uint32_t p0 = opaque(pick(0xAAAAAAAAu, w1 << 1, w0)), p1 = opaque(pick(0x55555555u, w0 >> 1, w1));
  c[1] += __builtin_popcount(p0 & ~p1);
  c[2] += __builtin_popcount(~p0 & p1);
  c[3] += __builtin_popcount(p0 & p1);
}
// c[0] from the lane's code total.
__device__ __forceinline__ void finish2(uint32_t total, uint32_t (&c)[4]) { c[0] = total - c[1] - c[2] - c[3]; }

// Four 4-bit words: a 4 x 4 bit transpose inside every nibble position in two
// stages (pairs of words swap single bits, then pairs of pairs swap bit pairs),
// so bit 4i + j of plane k is bit k of code i of word j.  Code v = 4h + l:
// low planes (p0, p1) select l, high planes (p2, p3) select h.  Adds to c[4h + l]
// for h, l >= 1, and to lc[l] / hc[h] the codes whose low / high half is l / h.
__device__ __forceinline__ void count_batch4(const uint32_t (&w)[4], uint32_t (&c)[16], uint32_t (&lc)[4],
                                             uint32_t (&hc)[4]) {
  const uint32_t a0 = opaque(pick(0xAAAAAAAAu, w[1] << 1, w[0])), a1 = opaque(pick(0x55555555u, w[0] >> 1, w[1]));
  const uint32_t a2 = opaque(pick(0xAAAAAAAAu, w[3] << 1, w[2])), a3 = opaque(pick(0x55555555u, w[2] >> 1, w[3]));
  const uint32_t p0 = opaque(pick(0xCCCCCCCCu, a2 << 2, a0)), p2 = opaque(pick(0x33333333u, a0 >> 2, a2));
  const uint32_t p1 = opaque(pick(0xCCCCCCCCu, a3 << 2, a1)), p3 = opaque(pick(0x33333333u, a1 >> 2, a3));
  const uint32_t lo[4] = {0u, p0 & ~p1, ~p0 & p1, p0 & p1};
  const uint32_t hi[4] = {0u, p2 & ~p3, ~p2 & p3, p2 & p3};
#pragma unroll
  for (int h = 1; h < 4; ++h)
#pragma unroll
    for (int l = 1; l < 4; ++l) c[4 * h + l] += __builtin_popcount(lo[l] & hi[h]);
#pragma unroll
  for (int k = 1; k < 4; ++k) {
    lc[k] += __builtin_popcount(lo[k]);
    hc[k] += __builtin_popcount(hi[k]);
  }
}
__device__ __forceinline__ void finish4(uint32_t total, const uint32_t (&lc)[4], const uint32_t (&hc)[4],
                                        uint32_t (&c)[16]) {
#pragma unroll
  for (int l = 1; l < 4; ++l) c[l] = lc[l] - c[4 + l] - c[8 + l] - c[12 + l];
#pragma unroll
  for (int h = 1; h < 4; ++h) c[4 * h] = hc[h] - c[4 * h + 1] - c[4 * h + 2] - c[4 * h + 3];
  uint32_t r = total;
#pragma unroll
  for (int v = 1; v < 16; ++v) r -= c[v];
  c[0] = r;
}

// The DW dwords of a code block that lane l holds (16-byte non-temporal loads
// when DW is a multiple of 4): dword i of lane l is dword (i / 4) * 256 + 4 l +
// i % 4 of the block (or i * 64 + l), the same assignment for every block.
template <int DW>
__device__ __forceinline__ void load_block(const uint8_t* p, int l, uint32_t (&w)[DW]) {
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
}

// Per-lane counts of the codes in DW dwords of B-bit codes.
template <int B, int DW>
__device__ __forceinline__ void count_lane(const uint32_t (&w)[DW], uint32_t (&c)[1 << B]) {
  static_assert(DW % B == 0, "whole bit-plane batches per lane");
#pragma unroll
  for (int i = 0; i < (1 << B); ++i) c[i] = 0;
  if constexpr (B == 2) {
#pragma unroll
    for (int i = 0; i < DW / 2; ++i) count_batch2(w[2 * i], w[2 * i + 1], c);
    finish2(DW * 16, c);
  } else {
    uint32_t lc[4] = {0u, 0u, 0u, 0u}, hc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
      const uint32_t ww[4] = {w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
      count_batch4(ww, c, lc, hc);
    }
    finish4(DW * 8, lc, hc, c);
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

// Sum of t over the lanes l' with l' = l (mod STRIDE), in every such lane.
template <int STRIDE>
__device__ __forceinline__ double strided_sum_f64(double t) {
#pragma unroll
  for (int m = STRIDE; m < kLanes; m *= 2) t += __shfl_xor(t, m);
  return t;
}

// One wave per groups_per_wave() consecutive groups of one slice.
template <int D, int KB, int VB, int G, bool HIST>
__global__ __launch_bounds__(64) void drift_kernel(DriftArgs a) {
  constexpr int NBK = 1 << KB, NBV = 1 << VB;
  constexpr int NG = groups_per_pass<KB, VB>(), GPW = groups_per_wave<KB, VB>();
  constexpr int KDW = G * D * KB / 8 / 4 / kLanes, VDW = G * D * VB / 8 / 4 / kLanes;  // dwords per lane
  static_assert(G * D * KB / 8 == KDW * 4 * kLanes && G * D * VB / 8 == VDW * 4 * kLanes, "whole dwords per lane");
  const Layout& L = a.L;
  const int l = threadIdx.x;
  const int64_t slice = blockIdx.y;
  const int hkv = static_cast<int>(slice % a.Hkv);
  const int64_t gb = a.g0 + static_cast<int64_t>(blockIdx.x) * GPW;
  const int64_t ge = min(gb + GPW, a.g0 + a.ng);
  const uint8_t* page = a.cache + page_offset(L, slice, gb);
  const int bk = bin_of_lane<NBK>(l), bv = bin_of_lane<NBV>(l);

  // KL terms, one fp64 logarithm per lane for the NG groups of a pass: with
  // RS = min(64 / 2^b_K, 64 / 2^b_V) lanes per bin, group i's key bins sit in
  // the lanes i mod RS and its value bins in the lanes NG + i mod RS (within
  // each bin's lanes, one lane).  A bin's term is p ln(p / q), 0 for p = 0,
  // +inf for p > 0 = q, with p = c / (G D) (exact: G D is a power of two) and
  // the calibration probability q = count / total formed once per wave.
  static_assert(((G * D) & (G * D - 1)) == 0, "G * D is a power of two");
  constexpr int RS = (64 / NBK) < (64 / NBV) ? 64 / NBK : 64 / NBV;
  static_assert(2 * NG <= RS, "a lane per group and bin");
  const int rk = l & (64 / NBK - 1), rv = l & (64 / NBV - 1);
  const int kslot = rk < NG ? rk : -1, vslot = rv >= NG && rv < 2 * NG ? rv - NG : -1;
  double q = 0.0;
  if constexpr (!HIST) {
    const uint64_t* qk = a.cal_k + hkv * NBK;
    const uint64_t* qv = a.cal_v + hkv * NBV;
    uint64_t sk = 0, sv = 0;
#pragma unroll
    for (int i = 0; i < NBK; ++i) sk += qk[i];
#pragma unroll
    for (int i = 0; i < NBV; ++i) sv += qv[i];
    const bool kk = kslot >= 0;
    const uint64_t cq = kk ? qk[bk] : qv[bv];
    // a bin without calibration counts (all of them, for an empty
    // calibration) has q = 0, so any count there makes the KL +inf
    q = cq == 0 ? 0.0 : static_cast<double>(cq) / static_cast<double>(kk ? sk : sv);
  }

  uint32_t hk[NBK], hv[NBV];  // per-lane totals over the wave's groups (histogram mode)
#pragma unroll
  for (int i = 0; i < NBK; ++i) hk[i] = 0;
#pragma unroll
  for (int i = 0; i < NBV; ++i) hv[i] = 0;
  // one register set per group of a pass; the next pass's codes load while
  // this pass's counts are reduced and turned into KL terms
  uint32_t kw[NG][KDW], vw[NG][VDW];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    if (gb + i < ge) {
      load_block<KDW>(page + i * L.page_bytes + L.off_kcodes, l, kw[i]);
      load_block<VDW>(page + i * L.page_bytes + L.off_vcodes, l, vw[i]);
    }
  }
#pragma unroll 1
  for (int64_t g = gb; g < ge; g += NG) {
    uint32_t ck[NG][NBK], cv[NG][NBV];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (g + i < ge) {
        count_lane<KB, KDW>(kw[i], ck[i]);
        count_lane<VB, VDW>(vw[i], cv[i]);
      } else {
#pragma unroll
        for (int k = 0; k < NBK; ++k) ck[i][k] = 0;
#pragma unroll
        for (int k = 0; k < NBV; ++k) cv[i][k] = 0;
      }
    }
    const uint8_t* pn = page + (g + NG - gb) * L.page_bytes;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (g + NG + i < ge) {
        load_block<KDW>(pn + i * L.page_bytes + L.off_kcodes, l, kw[i]);
        load_block<VDW>(pn + i * L.page_bytes + L.off_vcodes, l, vw[i]);
      }
    }
    if constexpr (HIST) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
#pragma unroll
        for (int k = 0; k < NBK; ++k) hk[k] += ck[i][k];
#pragma unroll
        for (int k = 0; k < NBV; ++k) hv[k] += cv[i][k];
      }
    } else {
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const uint32_t tk = wave_bins<NBK>(ck[i], l), tv = wave_bins<NBV>(cv[i], l);
        c = kslot == i ? tk : vslot == i ? tv : c;
      }
      const double p = static_cast<double>(c) * (1.0 / static_cast<double>(G * D));
      const double term = c == 0 ? 0.0 : (q == 0.0 ? __builtin_inf() : p * log(p / q));
      // lane j < 2 NG ends with the sum of the terms in lanes j mod RS: group
      // j's key KL for j < NG, group j - NG's value KL after that
      const double t = strided_sum_f64<RS>(term);
      const double tv = __shfl(t, (l + NG) & (kLanes - 1));
      if (l < NG && g + l < ge) {
        const int64_t o = slice * a.ng + (g + l - a.g0);
        a.kl_k[o] = t;
        a.kl_v[o] = tv;
        a.flags[o] = static_cast<uint8_t>((t > a.threshold ? 1 : 0) | (tv > a.threshold ? 2 : 0));
      }
    }
  }
  if constexpr (HIST) {
    const uint32_t tk = wave_bins<NBK>(hk, l), tv = wave_bins<NBV>(hv, l);
    if ((l & (64 / NBK - 1)) == 0) atomicAdd(reinterpret_cast<unsigned long long*>(a.hist_k) + hkv * NBK + bk, tk);
    if ((l & (64 / NBV - 1)) == 0) atomicAdd(reinterpret_cast<unsigned long long*>(a.hist_v) + hkv * NBV + bv, tv);
  }
}

__global__ void fill_u64_kernel(uint64_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int D, int KB, int VB, int G>
hipError_t drift_t(const DriftArgs& a, bool hist, hipStream_t s) {
  constexpr int GPW = groups_per_wave<KB, VB>();
  dim3 grid(static_cast<unsigned>((a.ng + GPW - 1) / GPW), static_cast<unsigned>(a.L.slices));
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
