// kvq_append.hip -- quantize-and-pack kernels of kvq_append.
//
// Entry conversion, the fp16 window and the group flush follow
// "[Framework] The Asymmetric Key-Value Cache Compression", section III (keys
// per channel, values per token, recent tokens kept in fp16) and section IV
// (Walsh-Hadamard rotation of keys, fused here into the append).  The
// quantizer is the asymmetric min/max uniform quantizer: scale =
// (max - min) / (2^b - 1) and code = round-half-even((x - min) / scale), both
// in IEEE binary32, so the codes are reproducible bit for bit on any IEEE
// machine.  This file is built with -ffp-contract=off and relies on hipcc's
// default correctly rounded binary32 division.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ float load_in(const void* p, int dtype, int64_t i) {
  if (dtype == 0) return static_cast<const float*>(p)[i];
  uint16_t u = static_cast<const uint16_t*>(p)[i];
  if (dtype == 1) return __half2float(__ushort_as_half(u));
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

__device__ __forceinline__ float round_fp16(float x) { return __half2float(__float2half_rn(x)); }

__device__ __forceinline__ uint16_t fp16_bits(float x) { return __half_as_ushort(__float2half_rn(x)); }

// code = clamp(rne((x - mn) / s), 0, levels); 0 when the group is constant.
__device__ __forceinline__ uint32_t quant_code(float x, float mn, float s, float levels) {
  if (s == 0.0f) return 0u;
  float q = rintf((x - mn) / s);
  q = fminf(fmaxf(q, 0.0f), levels);
  return static_cast<uint32_t>(q);
}

// Symmetric code: clamp(rne(x / s), -c0, c0) + c0; c0 when s == 0.
__device__ __forceinline__ uint32_t quant_code_sym(float x, float s, float c0) {
  if (s == 0.0f) return static_cast<uint32_t>(c0);
  float q = rintf(x / s);
  q = fminf(fmaxf(q, -c0), c0);
  return static_cast<uint32_t>(q + c0);
}

// Group parameters.  Asymmetric: s = (max - min) / (2^b - 1), zero = min.
// With `hybrid`, also the symmetric quantizer (s = max|x| / c0, c0 = 2^(b-1) - 1,
// zero = fp16(-c0 * fp16(s))), kept only if its largest reconstruction error
// |x - (code * scale16 + zero16)| (product exact, sum and difference rounded
// in binary32) is strictly smaller.  x(i) yields the group's i-th value.
struct GroupQ {
  float s, mn;          // binary32 scale and minimum the codes use
  uint16_t scale16, zero16;
  bool sym;
};
template <int COUNT, int BITS, typename F>
__device__ GroupQ group_params(F&& x, bool hybrid) {
  float mn = x(0), mx = mn, M = fabsf(mn);
  for (int i = 1; i < COUNT; ++i) {
    const float v = x(i);
    mn = v < mn ? v : mn;
    mx = v > mx ? v : mx;
    M = fabsf(v) > M ? fabsf(v) : M;
  }
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  M = M + 0.0f;
  constexpr float levels = static_cast<float>((1 << BITS) - 1), c0 = static_cast<float>((1 << (BITS - 1)) - 1);
  GroupQ r;
  r.s = (mx - mn) / levels;
  r.mn = mn;
  r.scale16 = fp16_bits(r.s);
  r.zero16 = fp16_bits(mn);
  r.sym = false;
  if (hybrid) {
    const float ss = M / c0;
    const uint16_t sc16 = fp16_bits(ss);
    const float s16 = __half2float(__ushort_as_half(sc16));
    const uint16_t z16 = fp16_bits(-(s16 * c0));
    const float zs = __half2float(__ushort_as_half(z16));
    const float sa = __half2float(__ushort_as_half(r.scale16)), za = __half2float(__ushort_as_half(r.zero16));
    float ea = 0.0f, es = 0.0f;
    for (int i = 0; i < COUNT; ++i) {
      const float v = x(i);
      const float xa = __fadd_rn(__fmul_rn(static_cast<float>(quant_code(v, mn, r.s, levels)), sa), za);
      const float xs = __fadd_rn(__fmul_rn(static_cast<float>(quant_code_sym(v, ss, c0)), s16), zs);
      ea = fmaxf(ea, fabsf(__fsub_rn(v, xa)));
      es = fmaxf(es, fabsf(__fsub_rn(v, xs)));
    }
    if (es < ea) {
      r.s = ss;
      r.scale16 = sc16;
      r.zero16 = z16;
      r.sym = true;
    }
  }
  return r;
}

template <int BITS>
__device__ __forceinline__ uint32_t code_of(float x, float mn, float s, bool sym) {
  constexpr float levels = static_cast<float>((1 << BITS) - 1), c0 = static_cast<float>((1 << (BITS - 1)) - 1);
  return sym ? quant_code_sym(x, s, c0) : quant_code(x, mn, s, levels);
}

constexpr float kInvSqrt128 = 0.08838834764831845f;  // nearest binary32 to 1/sqrt(128)
constexpr float kInvSqrt64 = 0.125f;

// Fast Walsh-Hadamard transform of `rows` rows of D fp32 values in LDS:
// butterflies (a + b, a - b) with span 1, 2, ..., D/2 in Sylvester order,
// then one multiply by the binary32 constant nearest 1/sqrt(D).  Every output
// depends only on the fixed butterfly sequence, so the result is independent
// of how threads share the work.
template <int D, int STRIDE = D>
__device__ void fwht_rows(float* x, int rows, int tid, int nthreads) {
  for (int h = 1; h < D; h <<= 1) {
    for (int k = tid; k < rows * (D / 2); k += nthreads) {
      int r = k / (D / 2), p = k % (D / 2);
      int i0 = (p / h) * 2 * h + (p % h);
      float a = x[r * STRIDE + i0], b = x[r * STRIDE + i0 + h];
      x[r * STRIDE + i0] = a + b;
      x[r * STRIDE + i0 + h] = a - b;
    }
    __syncthreads();
  }
  const float c = D == 128 ? kInvSqrt128 : kInvSqrt64;
  for (int k = tid; k < rows * D; k += nthreads) x[(k / D) * STRIDE + k % D] = x[(k / D) * STRIDE + k % D] * c;
  __syncthreads();
}

// One block per (flushed group, slice): gathers the group's G tokens (from
// the fp16 window ring, or from the input for tokens of this call), computes
// per-channel key and per-token value parameters, and writes the page.
template <int D, int KB, int VB, int G>
__global__ __launch_bounds__(256) void flush_kernel(AppendArgs a) {
  constexpr int NKB = D / 32, NCG = D / G;
  constexpr int CPG = G / kChunk;
  // token rows padded by one bank (4 bytes) so that the lanes reading one
  // channel of 16 or 32 consecutive tokens hit different LDS banks
  constexpr int KS = D + 1, VS = D + 2;
  __shared__ float kx[G * KS];
  __shared__ __half vx[G * VS];  // values are fp16 after entry conversion
  __shared__ float ks[D], kmn[D];
  __shared__ float vs[G * NCG], vmn[G * NCG];
  __shared__ bool ksym[D], vsym[G * NCG];
  __shared__ float knrm[G];

  const Layout& L = a.L;
  const int tid = threadIdx.x;
  const int64_t g = a.g_first + blockIdx.x;
  const int64_t pos0 = L.S0 + g * G;  // token position of the group's first token
  const int64_t slice = blockIdx.y;
  if (a.flags != nullptr && a.flags[slice * a.flag_stride + (g - a.flag_g0)] == 0) return;  // not requantized
  const int64_t in_base = slice * a.T * D;  // [B][H_kv] flattened == slice
  uint8_t* ring = a.cache;

  // 1. gather (entry conversion of new tokens; window tokens are fp16 already)
  bool any_new = false;
  if (pos0 >= a.n_old && a.in_dtype != 0) {
    // the whole group comes from this call's 2-byte input: G * D contiguous
    // elements per tensor, read as 16-byte vectors, every load of a thread
    // issued before the first is used
    constexpr int NVEC = G * D / 8, PER = NVEC / 256;
    static_assert(NVEC % 256 == 0, "whole vectors per thread");
    const uint4* kp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + in_base + (pos0 - a.n_old) * D);
    const uint4* vp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + in_base + (pos0 - a.n_old) * D);
    uint4 kv[PER], vv[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      kv[r] = kp[tid + 256 * r];
      vv[r] = vp[tid + 256 * r];
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int e0 = (tid + 256 * r) * 8, i = e0 / D, c0 = e0 % D;
      const uint32_t kw[4] = {kv[r].x, kv[r].y, kv[r].z, kv[r].w}, vw[4] = {vv[r].x, vv[r].y, vv[r].z, vv[r].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t ku = static_cast<uint16_t>(kw[e >> 1] >> (16 * (e & 1)));
        const uint16_t vu = static_cast<uint16_t>(vw[e >> 1] >> (16 * (e & 1)));
        const float kf = a.in_dtype == 1 ? __half2float(__ushort_as_half(ku)) : __uint_as_float(static_cast<uint32_t>(ku) << 16);
        const float vf = a.in_dtype == 1 ? __half2float(__ushort_as_half(vu)) : __uint_as_float(static_cast<uint32_t>(vu) << 16);
        kx[i * KS + c0 + e] = kf;
        vx[i * VS + c0 + e] = __float2half_rn(vf);
      }
    }
  } else {
  for (int idx = tid; idx < G * D; idx += blockDim.x) {
    int i = idx / D, c = idx % D;
    int64_t p = pos0 + i;
    if (p >= a.n_old) {
      int64_t src = in_base + (p - a.n_old) * D + c;
      kx[i * KS + c] = load_in(a.k, a.in_dtype, src);
      vx[i * VS + c] = __float2half_rn(load_in(a.v, a.in_dtype, src));
    } else {
      const uint8_t* rc = ring + ring_chunk_offset(L, slice, p);
      int t = static_cast<int>(p % kChunk);
      kx[i * KS + c] = __half2float(*reinterpret_cast<const __half*>(rc + ring_k_offset(L, t, c)));
      vx[i * VS + c] = *reinterpret_cast<const __half*>(rc + ring_v_offset(L, t, c));
    }
  }
  }
  any_new = (pos0 + G) > a.n_old;
  __syncthreads();
  if (any_new) {
    // rows [first_new, G) come from the input: rotate (keys) then round to fp16
    int first_new = a.n_old > pos0 ? static_cast<int>(a.n_old - pos0) : 0;
    if (a.rotate) fwht_rows<D, KS>(kx + first_new * KS, G - first_new, tid, blockDim.x);
    for (int idx = first_new * D + tid; idx < G * D; idx += blockDim.x)
      kx[(idx / D) * KS + idx % D] = round_fp16(kx[(idx / D) * KS + idx % D]);
    __syncthreads();
  }

  uint8_t* page = a.cache + page_offset(L, slice, g);

  // key token norms: each key row is divided by its norm and rounded to fp16
  // before the key quantizer; the norm is stored as fp16 (0 for a zero row,
  // whose normalized values are 0)
  if (L.token_norm) {
    // one wave per row: lane t takes the square sum of elements 2t, 2t + 1
    // (or, for D = 64, lanes 0..31), then each tree level adds pairs (2t,
    // 2t + 1) of the level below: a fixed order, so the norm does not depend
    // on how the work is shared; then a correctly rounded square root
    const int lane = tid % kLanes, wave = tid / kLanes, nwaves = blockDim.x / kLanes;
    for (int i = wave; i < G; i += nwaves) {
      const float* row = kx + i * KS;
      float t = 0.0f;
      if (lane < D / 2) t = __fadd_rn(__fmul_rn(row[2 * lane], row[2 * lane]), __fmul_rn(row[2 * lane + 1], row[2 * lane + 1]));
      for (int w = D / 2; w > 1; w /= 2) {
        const float a0 = __shfl(t, (2 * lane) % kLanes), a1 = __shfl(t, (2 * lane + 1) % kLanes);
        t = lane < w / 2 ? __fadd_rn(a0, a1) : 0.0f;
      }
      if (lane == 0) {
        const float nrm = sqrtf(t);
        knrm[i] = nrm;
        uint16_t* kn = reinterpret_cast<uint16_t*>(page + L.off_knorm + (i / kChunk) * L.kn_chunk_bytes);
        kn[knorm_elem(i % kChunk)] = fp16_bits(nrm);
      }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
      const float nrm = knrm[idx / D];
      float& xk = kx[(idx / D) * KS + idx % D];
      xk = nrm == 0.0f ? 0.0f : round_fp16(xk / nrm);
    }
    __syncthreads();
  }

  // 2. parameters: keys per channel over G tokens, values per token over G channels
  const bool hybrid = a.hybrid != 0;
  for (int c = tid; c < D; c += blockDim.x) {
    const GroupQ q = group_params<G, KB>([&](int i) { return kx[i * KS + c]; }, hybrid);
    ks[c] = q.s;
    kmn[c] = q.mn;
    ksym[c] = q.sym;
    uint16_t* kp = reinterpret_cast<uint16_t*>(page + L.off_kparams);
    int pi = kparam_index(L, c);
    kp[pi] = q.scale16;
    kp[D + pi] = q.zero16;
  }
  for (int task = tid; task < G * NCG; task += blockDim.x) {
    int i = task / NCG, cg = task % NCG;
    const __half* row = vx + i * VS + cg * G;
    const GroupQ q = group_params<G, VB>([&](int c) { return __half2float(row[c]); }, hybrid);
    vs[task] = q.s;
    vmn[task] = q.mn;
    vsym[task] = q.sym;
    uint16_t* vp = reinterpret_cast<uint16_t*>(page + L.off_vparams + (i / kChunk) * L.vp_chunk_bytes);
    vp[vparam_scale_elem(L, i % kChunk, cg)] = q.scale16;
    vp[vparam_zero_elem(L, i % kChunk, cg)] = q.zero16;
  }
  __syncthreads();

  // 3. key codes: each task assembles one dword of one lane of one chunk
  {
    constexpr int KW = 2 * NKB * KB / 4;
    for (int task = tid; task < CPG * kLanes * KW; task += blockDim.x) {
      int ch = task / (kLanes * KW);
      int l = (task / KW) % kLanes;
      int d = task % KW;
      int l16 = l & 15, j = l >> 4;
      uint32_t word = 0;
      constexpr int SUBS = KB == 4 ? 1 : 2;
      for (int sub = 0; sub < SUBS; ++sub) {
        int combo = KB == 4 ? d : 2 * d + sub;
        int mt = combo / NKB, kb = combo % NKB;
        int i = ch * kChunk + 16 * mt + l16;  // token within the group
        for (int e = 0; e < 8; ++e) {
          int c = 32 * kb + 8 * j + e;
          uint32_t code = code_of<KB>(kx[i * KS + c], kmn[c], ks[c], ksym[c]);
          int bit = KB == 4 ? 16 * (e & 1) + 4 * (e >> 1) : 16 * (e & 1) + 8 * sub + 2 * (e >> 1);
          word |= code << bit;
        }
      }
      *reinterpret_cast<uint32_t*>(page + L.off_kcodes + ch * L.kc_chunk_bytes + lane_dword_offset(KW, l, d)) = word;
    }
  }
  // 4. value codes
  {
    constexpr int NMT = D / 16;
    constexpr int VW = NMT * VB / 4;
    for (int task = tid; task < CPG * kLanes * VW; task += blockDim.x) {
      int ch = task / (kLanes * VW);
      int l = (task / VW) % kLanes;
      int d = task % VW;
      int l16 = l & 15, j = l >> 4;
      uint32_t word = 0;
      constexpr int SUBS = VB == 4 ? 1 : 2;
      for (int sub = 0; sub < SUBS; ++sub) {
        int mt = VB == 4 ? d : 2 * d + sub;
        int c = 16 * mt + l16;
        int cg = c / G;
        for (int e = 0; e < 8; ++e) {
          int i = ch * kChunk + tau(j, e);
          uint32_t code = code_of<VB>(__half2float(vx[i * VS + c]), vmn[i * NCG + cg], vs[i * NCG + cg], vsym[i * NCG + cg]);
          int bit = VB == 4 ? 16 * (e & 1) + 4 * (e >> 1) : 16 * (e & 1) + 8 * sub + 2 * (e >> 1);
          word |= code << bit;
        }
      }
      *reinterpret_cast<uint32_t*>(page + L.off_vcodes + ch * L.vc_chunk_bytes + lane_dword_offset(VW, l, d)) = word;
    }
  }
}

// One block of D threads per (fp16 position written, slice): the sink
// positions of this call first, then its window positions.
template <int D>
__global__ __launch_bounds__(128) void window_write_kernel(AppendArgs a) {
  __shared__ float kx[D];
  const Layout& L = a.L;
  const int c = threadIdx.x;
  const int64_t p = blockIdx.x < a.n_sink_write ? a.s_first + blockIdx.x : a.w_first + (blockIdx.x - a.n_sink_write);
  const int64_t slice = blockIdx.y;
  const int64_t src = (slice * a.T + (p - a.n_old)) * D + c;
  kx[c] = load_in(a.k, a.in_dtype, src);
  float v = round_fp16(load_in(a.v, a.in_dtype, src));
  __syncthreads();
  if (a.rotate) fwht_rows<D>(kx, 1, c, D);
  uint8_t* rc = a.cache + fp16_chunk_offset(L, slice, p);
  int t = static_cast<int>(p % kChunk);
  *reinterpret_cast<__half*>(rc + ring_k_offset(L, t, c)) = __float2half_rn(kx[c]);
  *reinterpret_cast<__half*>(rc + ring_v_offset(L, t, c)) = __float2half_rn(v);
}

template <int D, int KB, int VB, int G>
hipError_t flush_t(const AppendArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(a.n_flush), static_cast<unsigned>(a.L.slices));
  hipLaunchKernelGGL((flush_kernel<D, KB, VB, G>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int KB, int VB>
hipError_t flush_g(const AppendArgs& a, hipStream_t s) {
  return a.L.G == 32 ? flush_t<D, KB, VB, 32>(a, s) : flush_t<D, KB, VB, 64>(a, s);
}

template <int D, int KB>
hipError_t flush_v(const AppendArgs& a, hipStream_t s) {
  return a.L.vbits == 2 ? flush_g<D, KB, 2>(a, s) : flush_g<D, KB, 4>(a, s);
}

template <int D>
hipError_t flush_k(const AppendArgs& a, hipStream_t s) {
  return a.L.kbits == 2 ? flush_v<D, 2>(a, s) : flush_v<D, 4>(a, s);
}

}  // namespace

hipError_t launch_flush(const AppendArgs& a, hipStream_t s) {
  if (a.n_flush <= 0) return hipSuccess;
  return a.L.D == 64 ? flush_k<64>(a, s) : flush_k<128>(a, s);
}

hipError_t launch_window_write(const AppendArgs& a, hipStream_t s) {
  if (a.n_write + a.n_sink_write <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.n_sink_write + a.n_write), static_cast<unsigned>(a.L.slices));
  if (a.L.D == 64)
    hipLaunchKernelGGL((window_write_kernel<64>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((window_write_kernel<128>), grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
