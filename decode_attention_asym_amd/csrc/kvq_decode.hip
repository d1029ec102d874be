// kvq_decode.hip -- fused dequant + single-query decode attention on the
// packed cache, split over the token axis, and the cross-split merge.
//
// Computes softmax(q K^T / sqrt(d)) V ("Asymmetric Key-Value Quantization:
// 2-Bit Values and 4-Bit Keys under Long-Context Drift", section 1) over
// keys quantized per channel and values quantized per token ("[Framework] The
// Asymmetric Key-Value Cache Compression", section III), plus the fp16
// window of recent tokens.  Decode attention is bound by reading the cache
// (the "Loading ... takes longer than computing" remark of the NOVA-KV
// abstract), so the kernel is built to stream every byte once.
//
// Per wave: one (batch, kv head) slice and one contiguous range of token
// groups (a split).  The GQA query heads of the slice are the 16 columns of
// the MFMA B operand (unused columns compute on zeros).
//
// Scale folding (exact in real arithmetic):
//   keys, per channel c of group g:  q . khat_t = sum_c (q_c s_gc) code_tc + sum_c q_c z_gc
//   values, per token t, group j:    sum_t p_t vhat_tc = sum_t (p_t s_tj) code_tc + sum_t p_t z_tj
// so both products run on raw integer codes: (q_c s_gc) is the B operand of
// QK^T once per token group, (p_t s_tj) the B operand of PV once per chunk,
// and the zero-point sums are added as per-head biases.  Codes enter the MFMA
// as fp16 1024 + 2^p code (see kvq_layout.h); the 2^p are folded into the B
// operands and the 1024 offsets are subtracted using the same fp16 B values.
// Softmax runs in the log2 domain (exp2), log2(e)/sqrt(D) folded into q.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Constants kept out of the optimizer's sight so that (w & mask) | magic
// selects one v_and_or_b32 with the mask in an SGPR and the magic in a VGPR
// (gfx9 VOP3 encodings take no literal operands).
__device__ __forceinline__ uint32_t sgpr_const(uint32_t x) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(x));
  return r;
}
__device__ __forceinline__ uint32_t vgpr_const(uint32_t x) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(x));
  return r;
}

struct Unpack {
  uint32_t magic;   // 0x64006400: fp16 1024 in both halves
  uint32_t m[4];    // field masks
};

template <int BITS>
__device__ __forceinline__ Unpack make_unpack() {
  Unpack u;
  u.magic = vgpr_const(0x64006400u);
  if (BITS == 4) {
    u.m[0] = sgpr_const(0x000F000Fu);
    u.m[1] = sgpr_const(0x00F000F0u);
    u.m[2] = u.m[0];
    u.m[3] = u.m[1];
  } else {
    u.m[0] = sgpr_const(0x00030003u);
    u.m[1] = sgpr_const(0x000C000Cu);
    u.m[2] = sgpr_const(0x00300030u);
    u.m[3] = sgpr_const(0x00C000C0u);
  }
  return u;
}

// 4-bit word -> 8 fp16 values 1024 + mult(e) * code_e, mult = 1, 1, 16, 16, 1, 1, 16, 16.
__device__ __forceinline__ half8 unpack4(uint32_t w, const Unpack& u) {
  uint32_t w8 = w >> 8;
  u32x4 r = {(w & u.m[0]) | u.magic, (w & u.m[1]) | u.magic, (w8 & u.m[0]) | u.magic, (w8 & u.m[1]) | u.magic};
  return __builtin_bit_cast(half8, r);
}
// One 2-bit sub-block (the low byte of each half of w) -> 8 fp16 values
// 1024 + 4^(e>>1) * code_e.
__device__ __forceinline__ half8 unpack2(uint32_t w, const Unpack& u) {
  u32x4 r = {(w & u.m[0]) | u.magic, (w & u.m[1]) | u.magic, (w & u.m[2]) | u.magic, (w & u.m[3]) | u.magic};
  return __builtin_bit_cast(half8, r);
}

template <int BITS>
__host__ __device__ constexpr float code_mult(int e) {
  return BITS == 4 ? (((e >> 1) & 1) ? 16.0f : 1.0f) : static_cast<float>(1 << (2 * (e >> 1)));
}

template <int W>
__device__ __forceinline__ void load_lane_words(const uint8_t* base, int l, uint32_t (&w)[W]) {
  if constexpr (W >= 4) {
#pragma unroll
    for (int v = 0; v < W / 4; ++v) {
      u32x4 x = *reinterpret_cast<const u32x4*>(base + v * (kLanes * 16) + l * 16);
      w[4 * v + 0] = x[0]; w[4 * v + 1] = x[1]; w[4 * v + 2] = x[2]; w[4 * v + 3] = x[3];
    }
  } else {
    u32x2 x = *reinterpret_cast<const u32x2*>(base + l * 8);
    w[0] = x[0]; w[1] = x[1];
  }
}

template <int BITS, int NPER>
__device__ __forceinline__ half8 a_operand(const uint32_t* words, int idx, const Unpack& u) {
  // idx-th 8-element operand of a lane: 4-bit -> one word each; 2-bit -> two per word
  if constexpr (BITS == 4) {
    return unpack4(words[idx], u);
  } else {
    uint32_t w = words[idx >> 1];
    return unpack2((idx & 1) ? (w >> 8) : w, u);
  }
}

__device__ __forceinline__ float wave_sum_j(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float wave_max_j(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float load_q(const void* p, int dtype, int64_t i) {
  if (dtype == 0) return static_cast<const float*>(p)[i];
  uint16_t u = static_cast<const uint16_t*>(p)[i];
  if (dtype == 1) return __half2float(__ushort_as_half(u));
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

__device__ __forceinline__ float h2f_lo(uint32_t w) { return __half2float(__ushort_as_half(static_cast<uint16_t>(w))); }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return __half2float(__ushort_as_half(static_cast<uint16_t>(w >> 16))); }

template <int D, int KB, int VB, int G>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  constexpr int NKB = D / 32, NMT = D / 16, NCG = D / G, CPG = G / kChunk;
  constexpr int KW = 2 * NKB * KB / 4, VW = NMT * VB / 4;
  const Layout& L = a.L;
  const int l = threadIdx.x, l16 = l & 15, j = l >> 4;
  const int S = a.splits;
  const int64_t slice = blockIdx.x / S;
  const int s = static_cast<int>(blockIdx.x % S);
  const int b = static_cast<int>(slice / a.Hkv), hkv = static_cast<int>(slice % a.Hkv);
  const bool hv = l16 < a.gqa;
  const int hq = hkv * a.gqa + (hv ? l16 : 0);

  // ---- query: lane owns channels 32 kb + 8 j + e of head l16, times log2(e)/sqrt(D)
  float qv[NKB][8];
  const float qscale = kLog2e * (D == 128 ? 0.08838834764831845f : 0.125f);
  if (a.rotate) {
    extern __shared__ float qsh[];  // gqa * D floats, sized at launch
    const int64_t base = (static_cast<int64_t>(b) * a.Hq + hkv * a.gqa) * D;
    for (int idx = l; idx < a.gqa * D; idx += kLanes) qsh[idx] = load_q(a.q, a.in_dtype, base + idx);
    __syncthreads();
    for (int h = 1; h < D; h <<= 1) {
      for (int k = l; k < a.gqa * (D / 2); k += kLanes) {
        int r = k / (D / 2), p = k % (D / 2);
        int i0 = r * D + (p / h) * 2 * h + (p % h);
        float x0 = qsh[i0], x1 = qsh[i0 + h];
        qsh[i0] = x0 + x1;
        qsh[i0 + h] = x0 - x1;
      }
      __syncthreads();
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        qv[kb][e] = hv ? qsh[(hv ? l16 : 0) * D + 32 * kb + 8 * j + e] * (qscale * (D == 128 ? 0.08838834764831845f : 0.125f)) : 0.0f;
  } else {
    const int64_t base = (static_cast<int64_t>(b) * a.Hq + hq) * D;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[kb][e] = hv ? load_q(a.q, a.in_dtype, base + 32 * kb + 8 * j + e) * qscale : 0.0f;
  }
  // qm = q / mult: the B operand of QK^T is fp16(qm * key scale)
  float qm[NKB][8];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) qm[kb][e] = qv[kb][e] * (1.0f / code_mult<KB>(e));

  const Unpack uk = make_unpack<KB>();
  const Unpack uv = make_unpack<VB>();
  const half2v neg1024 = {static_cast<_Float16>(-1024.0f), static_cast<_Float16>(-1024.0f)};

  float m = -INFINITY, lsum = 0.0f;
  f32x4 acc[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zacc[NCG];
#pragma unroll
  for (int i = 0; i < NCG; ++i) zacc[i] = 0.0f;

  // online softmax over one chunk's 8 scores per lane (tokens tau(j, e))
  auto softmax_step = [&](float (&sc)[8], float (&p)[8]) {
    float cmax = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cmax = fmaxf(cmax, sc[e]);
    cmax = wave_max_j(cmax);
    if (__any(cmax > m)) {
      float mnew = fmaxf(m, cmax);
      float al = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
      for (int i = 0; i < NMT; ++i) acc[i] *= al;
#pragma unroll
      for (int i = 0; i < NCG; ++i) zacc[i] *= al;
      lsum *= al;
      m = mnew;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(sc[e] - m);
      lsum += p[e];
    }
  };

  const int64_t g0 = static_cast<int64_t>(s) * a.groups_per_split;
  const int64_t g1 = g0 + a.groups_per_split < a.ngroups ? g0 + a.groups_per_split : a.ngroups;
  for (int64_t g = g0; g < g1; ++g) {
    const uint8_t* page = a.cache + page_offset(L, slice, g);
    // B operand of QK^T for this group and the per-head bias
    half8 bq[NKB];
    float bacc[4] = {0.f, 0.f, 0.f, 0.f};
    float corr = 0.0f;
    {
      const u32x4* kps = reinterpret_cast<const u32x4*>(page + L.off_kparams) + j * NKB;
      const u32x4* kpz = reinterpret_cast<const u32x4*>(page + L.off_kparams + 2 * D) + j * NKB;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        u32x4 sw = kps[kb], zw = kpz[kb];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t sv = sw[e >> 1], zv = zw[e >> 1];
          float sf = (e & 1) ? h2f_hi(sv) : h2f_lo(sv);
          float zf = (e & 1) ? h2f_hi(zv) : h2f_lo(zv);
          bq[kb][e] = static_cast<_Float16>(qm[kb][e] * sf);
          bacc[e >> 1] += qm[kb][e] * zf;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          half2v pr = {bq[kb][2 * i], bq[kb][2 * i + 1]};
          corr = __builtin_amdgcn_fdot2(pr, neg1024, corr, false);
        }
      }
    }
    float bias = corr;
#pragma unroll
    for (int i = 0; i < 4; ++i) bias += bacc[i] * code_mult<KB>(2 * i);
    bias = wave_sum_j(bias);

#pragma unroll
    for (int ch = 0; ch < CPG; ++ch) {
      uint32_t kw[KW], vw[VW];
      load_lane_words<KW>(page + L.off_kcodes + ch * L.kc_chunk_bytes, l, kw);
      load_lane_words<VW>(page + L.off_vcodes + ch * L.vc_chunk_bytes, l, vw);
      uint32_t vp[8 * NCG];
      {
        const u32x4* vpp = reinterpret_cast<const u32x4*>(page + L.off_vparams + ch * L.vp_chunk_bytes) + j * 2 * NCG;
#pragma unroll
        for (int v = 0; v < 2 * NCG; ++v) {
          u32x4 x = vpp[v];
          vp[4 * v] = x[0]; vp[4 * v + 1] = x[1]; vp[4 * v + 2] = x[2]; vp[4 * v + 3] = x[3];
        }
      }
      // QK^T: two 16-token tiles
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_operand<KB, 8>(kw, kb, uk), bq[kb], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_operand<KB, 8>(kw, NKB + kb, uk), bq[kb], c1, 0, 0, 0);
      }
      float sc[8], p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = c0[r] + bias;
        sc[4 + r] = c1[r] + bias;
      }
      softmax_step(sc, p);
      // PV B operands, one per value group, and the zero-point / offset sums
      half8 bp[NCG];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        float zsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t w = vp[e * NCG + cg];
          bp[cg][e] = static_cast<_Float16>(p[e] * (1.0f / code_mult<VB>(e)) * h2f_lo(w));
          zsum += p[e] * h2f_hi(w);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          half2v pr = {bp[cg][2 * i], bp[cg][2 * i + 1]};
          zsum = __builtin_amdgcn_fdot2(pr, neg1024, zsum, false);
        }
        zacc[cg] += zsum;
      }
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_operand<VB, 8>(vw, mt, uv), bp[(16 * mt) / G], acc[mt], 0, 0, 0);
    }
  }

  // ---- fp16 window chunks: the last split
  if (s == S - 1 && a.rc1 > a.rc0) {
    half8 bqr[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) bqr[kb][e] = static_cast<_Float16>(qv[kb][e]);
    for (int64_t rc = a.rc0; rc < a.rc1; ++rc) {
      const uint8_t* rch = a.cache + ring_chunk_offset(L, slice, rc * kChunk);
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        half8 a0 = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(rch + ((0 * NKB + kb) * kLanes + l) * 16));
        half8 a1 = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(rch + ((1 * NKB + kb) * kLanes + l) * 16));
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bqr[kb], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bqr[kb], c1, 0, 0, 0);
      }
      const int64_t pos0 = rc * kChunk;
      const bool partial = pos0 + kChunk > a.n;
      float sc[8], p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = c0[r];
        sc[4 + r] = c1[r];
      }
      uint32_t vmask[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
      if (partial) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bool valid = pos0 + tau(j, e) < a.n;
          if (!valid) {
            sc[e] = -INFINITY;
            vmask[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
      }
      softmax_step(sc, p);
      half8 bp;
#pragma unroll
      for (int e = 0; e < 8; ++e) bp[e] = static_cast<_Float16>(p[e]);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        u32x4 vwd = *reinterpret_cast<const u32x4*>(rch + kChunk * D * 2 + (mt * kLanes + l) * 16);
        vwd[0] &= vmask[0]; vwd[1] &= vmask[1]; vwd[2] &= vmask[2]; vwd[3] &= vmask[3];
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, vwd), bp, acc[mt], 0, 0, 0);
      }
    }
  }

  // ---- finalize
  lsum = wave_sum_j(lsum);
#pragma unroll
  for (int i = 0; i < NCG; ++i) zacc[i] = wave_sum_j(zacc[i]);
  if (hv) {
    const int64_t row = static_cast<int64_t>(b) * a.Hq + hq;
    if (S == 1) {
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int c0 = 16 * mt + 4 * j;
        f32x4 o = (acc[mt] + zacc[c0 / G]) * inv;
        *reinterpret_cast<f32x4*>(a.out + row * D + c0) = o;
      }
    } else {
      float* pr = a.partial + (row * S + s) * (D + 4);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int c0 = 16 * mt + 4 * j;
        f32x4 o = acc[mt] + zacc[c0 / G];
        *reinterpret_cast<f32x4*>(pr + c0) = o;
      }
      if (j == 0) {
        pr[D] = m;
        pr[D + 1] = lsum;
      }
    }
  }
}

// Merge the split partials of one (batch, query head) row:
// M = max m_s, out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s (log2 domain);
// empty splits (m = -inf) contribute nothing.
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ partial, float* __restrict__ out,
                                                    int S, int D) {
  const int64_t row = blockIdx.x;
  const int c = threadIdx.x;
  const float* pr = partial + row * S * (D + 4);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pr[s * (D + 4) + D]);
  float Lsum = 0.0f, O = 0.0f;
  for (int s = 0; s < S; ++s) {
    float ms = pr[s * (D + 4) + D];
    if (ms == -INFINITY) continue;
    float w = __builtin_amdgcn_exp2f(ms - M);
    Lsum += w * pr[s * (D + 4) + D + 1];
    O += w * pr[s * (D + 4) + c];
  }
  out[row * D + c] = O / Lsum;
}

template <int D, int KB, int VB, int G>
hipError_t decode_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(a.L.slices * a.splits));
  const size_t lds = a.rotate ? static_cast<size_t>(a.gqa) * D * sizeof(float) : 0;
  hipLaunchKernelGGL((decode_kernel<D, KB, VB, G>), grid, dim3(kLanes), lds, s, a);
  return hipGetLastError();
}
template <int D, int KB, int VB>
hipError_t decode_g(const DecodeArgs& a, hipStream_t s) {
  return a.L.G == 32 ? decode_t<D, KB, VB, 32>(a, s) : decode_t<D, KB, VB, 64>(a, s);
}
template <int D, int KB>
hipError_t decode_v(const DecodeArgs& a, hipStream_t s) {
  return a.L.vbits == 2 ? decode_g<D, KB, 2>(a, s) : decode_g<D, KB, 4>(a, s);
}
template <int D>
hipError_t decode_k(const DecodeArgs& a, hipStream_t s) {
  return a.L.kbits == 2 ? decode_v<D, 2>(a, s) : decode_v<D, 4>(a, s);
}

}  // namespace

bool decode_supported(int D, int kbits, int vbits, int G) {
  return (D == 64 || D == 128) && (kbits == 2 || kbits == 4) && (vbits == 2 || vbits == 4) &&
         (G == 32 || G == 64) && G <= D;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  return a.L.D == 64 ? decode_k<64>(a, s) : decode_k<128>(a, s);
}

hipError_t launch_merge(const float* partial, float* out, int rows, int splits, int D, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>(rows)), dim3(D), 0, s, partial, out, splits, D);
  return hipGetLastError();
}

}  // namespace kvq
