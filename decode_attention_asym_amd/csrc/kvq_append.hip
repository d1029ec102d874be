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

#include <type_traits>

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

// Two bf16 values (one dword) -> two fp16 values, each rounded to nearest even
// from the exact binary32 value (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 r = {static_cast<_Float16>(__uint_as_float(w << 16)), static_cast<_Float16>(__uint_as_float(w & 0xffff0000u))};
  return __builtin_bit_cast(uint32_t, r);
}

// rne(fl(n / s)) for |n / s| <= 16, given rs = fl(1 / s) (correctly
// rounded).  fl(n * rs) is within 2^-19 of n / s (two roundings of relative
// size 2^-24 on a quotient below 16) and fl(n / s) within 2^-20 of it, so the
// two round to the same integer unless n * rs lies within 2^-18 of a
// half-integer.  The test is wider (2^-12); a wave in which some lane falls
// inside it (a few percent of waves per code) takes the correctly rounded
// division for those lanes.
constexpr float kTieGuard = 0.5f - 0x1.0p-12f;
__device__ __forceinline__ float rne_quotient(float n, float s, float rs) {
  const float f = n * rs;
  float t = rintf(f);
  const bool near = fabsf(f - t) > kTieGuard;
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    if (near) t = rintf(n / s);
  }
  return t;
}

// code = clamp(rne((x - mn) / s), 0, levels) as a float; 0 when the group is
// constant.  The clamp never acts, so it is left out: every x of the group
// lies in [mn, mx], fl is monotonic, and s = fl(fl(mx - mn) / levels), so the
// quotient is at most levels * (1 + 2^-22) and at least -0, which round to
// levels and 0 (the same holds for the reciprocal product the rounding helper
// forms first).
__device__ __forceinline__ float quant_code_f(float x, float mn, float s, float rs) {
  if (s == 0.0f) return 0.0f;
  return rne_quotient(x - mn, s, rs);
}
__device__ __forceinline__ uint32_t quant_code(float x, float mn, float s, float rs, float) {
  return static_cast<uint32_t>(quant_code_f(x, mn, s, rs));
}

// Symmetric code: clamp(rne(x / s), -c0, c0) + c0 as a float; c0 when s == 0
// (|x| <= max|x| and s = fl(max|x| / c0): the clamp never acts, as above).
__device__ __forceinline__ float quant_code_sym_f(float x, float s, float rs, float c0) {
  if (s == 0.0f) return c0;
  return rne_quotient(x, s, rs) + c0;
}
__device__ __forceinline__ uint32_t quant_code_sym(float x, float s, float rs, float c0) {
  return static_cast<uint32_t>(quant_code_sym_f(x, s, rs, c0));
}

__device__ __forceinline__ float recip(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

// Group parameters.  Asymmetric: s = (max - min) / (2^b - 1), zero = min.
// With HYB, also the symmetric quantizer (s = max|x| / c0, c0 = 2^(b-1) - 1,
// zero = fp16(-c0 * fp16(s))), kept only if its largest reconstruction error
// |x - (code * scale16 + zero16)| (product exact, sum and difference rounded
// in binary32) is strictly smaller.
//
// Two adjacent lanes share a group: x(i), i < COUNT / 2, yields this lane's
// half of it, and minima, maxima and largest errors are combined with the
// partner lane (lane ^ 1); both lanes return the same parameters.  Minimum,
// maximum and largest error do not depend on the order of their operands
// (inputs are finite; a zero's sign is normalized by the + 0).
struct GroupQ {
  float s, mn;          // binary32 scale and minimum the codes use
  float rs;             // fl(1 / s), 0 when s == 0
  uint16_t scale16, zero16;
  bool sym;
};
template <int COUNT, int BITS, bool HYB, typename F>
__device__ __forceinline__ GroupQ group_params_pair(F&& x) {
  constexpr int H = COUNT / 2;
  float mn = x(0), mx = mn, M = fabsf(mn);
  for (int i = 1; i < H; ++i) {
    const float v = x(i);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
    if constexpr (HYB) M = fmaxf(M, fabsf(v));
  }
  mn = fminf(mn, __shfl_xor(mn, 1));
  mx = fmaxf(mx, __shfl_xor(mx, 1));
  if constexpr (HYB) M = fmaxf(M, __shfl_xor(M, 1));
  mn = mn + 0.0f;
  mx = mx + 0.0f;
  constexpr float levels = static_cast<float>((1 << BITS) - 1), c0 = static_cast<float>((1 << (BITS - 1)) - 1);
  GroupQ r;
  r.s = (mx - mn) / levels;
  r.rs = recip(r.s);
  r.mn = mn;
  r.scale16 = fp16_bits(r.s);
  r.zero16 = fp16_bits(mn);
  r.sym = false;
  if constexpr (HYB) {
    M = M + 0.0f;
    const float ss = M / c0, rss = recip(ss);
    const uint16_t sc16 = fp16_bits(ss);
    const float s16 = __half2float(__ushort_as_half(sc16));
    const uint16_t z16 = fp16_bits(-(s16 * c0));
    const float zs = __half2float(__ushort_as_half(z16));
    const float sa = __half2float(__ushort_as_half(r.scale16)), za = __half2float(__ushort_as_half(r.zero16));
    float ea = 0.0f, es = 0.0f;
    for (int i = 0; i < H; ++i) {
      const float v = x(i);
      const float xa = __fadd_rn(__fmul_rn(static_cast<float>(quant_code(v, mn, r.s, r.rs, levels)), sa), za);
      const float xs = __fadd_rn(__fmul_rn(static_cast<float>(quant_code_sym(v, ss, rss, c0)), s16), zs);
      ea = fmaxf(ea, fabsf(__fsub_rn(v, xa)));
      es = fmaxf(es, fabsf(__fsub_rn(v, xs)));
    }
    ea = fmaxf(ea, __shfl_xor(ea, 1));
    es = fmaxf(es, __shfl_xor(es, 1));
    if (es < ea) {
      r.s = ss;
      r.rs = rss;
      r.scale16 = sc16;
      r.zero16 = z16;
      r.sym = true;
    }
  }
  return r;
}

// The operands of one code: the quotient's numerator n (fl(x - min) for the
// asymmetric quantizer, x for the symmetric one), its scale s, rs = fl(1/s)
// (0 when s = 0) and the offset added to the rounded quotient (0, or c0 for
// the symmetric quantizer).  fl(x - min) is formed as fma(x, 1, -min): the
// exact difference rounded once, as a binary32 subtraction rounds it, and
// with x an fp16 value the conversion folds into the fma.  The group's
// quantizer choice is folded into its stored operands: a symmetric group
// stores min = 0 (fma(x, 1, -0) is x exactly, signed zeros included) and
// offset c0, an asymmetric one its minimum and offset 0, so no code selects
// between the two.
struct QOp {
  float n, s, rs, off;
};
// `one` is 1.0f taken from an SGPR (opaque_one): with a literal 1.0 the
// compiler rewrites the fma as a subtraction and converts x from fp16 in an
// instruction of its own; with an operand it cannot see it keeps the fma and
// selects one v_fma_mix_f32 (fp16 input, exact product, one rounding).
__device__ __forceinline__ QOp quant_op(float x, float mn, float s, float rs, float off, float one) {
  return QOp{__builtin_fmaf(x, one, -mn), s, rs, off};
}
__device__ __forceinline__ float opaque_one() {
  uint32_t r;
  asm("s_mov_b32 %0, 0x3f800000" : "=s"(r));
  return __uint_as_float(r);
}

// Packs N codes into a dword: the code of field k (its operands op(k)) goes
// to bit bit_of(k); the fields of a byte are summed as floats (exact small
// integers) and each byte is inserted by one v_cvt_pk_u8_f32.  A code is
// rne(fl(n / s)) + off, formed as rint(fl(n * rs)) (rne_quotient's rule): the
// quotients of all N fields are rounded first and one ballot over them tells
// whether any lane has a field within 2^-12 of a half-integer; only then are
// the operands formed again and those fields take the correctly rounded
// division.  A group with s = 0 has n = 0 (every x equals the minimum, or is
// zero for the symmetric quantizer) and rs = 0, so its quotient is 0 without
// a test.  OFF: some operands carry an offset (the hybrid quantizer).
template <int N, bool OFF, typename BitF, typename OpF>
__device__ __forceinline__ uint32_t pack_codes(BitF&& bit_of, OpF&& op) {
  float t[N], off[N];
  uint64_t near = 0;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const QOp q = op(k);
    const float f = q.n * q.rs;
    t[k] = rintf(f);
    off[k] = q.off;
    near |= __builtin_amdgcn_ballot_w64(fabsf(f - t[k]) > kTieGuard);
  }
  if (near != 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const QOp q = op(k);
      const float f = q.n * q.rs;
      if (fabsf(f - rintf(f)) > kTieGuard) t[k] = rintf(q.n / q.s);
    }
  }
  // a byte's first field starts its sum (an fma onto +0 would cost an add)
  float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  bool started[4] = {false, false, false, false};
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int bit = bit_of(k), by = bit >> 3;
    const float code = OFF ? t[k] + off[k] : t[k];
    const float mult = static_cast<float>(1 << (bit & 7));
    b[by] = started[by] ? __builtin_fmaf(code, mult, b[by]) : code * mult;
    started[by] = true;
  }
  uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(b[0], 0, 0u);
  w = __builtin_amdgcn_cvt_pk_u8_f32(b[1], 1, w);
  w = __builtin_amdgcn_cvt_pk_u8_f32(b[2], 2, w);
  return __builtin_amdgcn_cvt_pk_u8_f32(b[3], 3, w);
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
// F32K: keys are staged in binary32 (needed by the rotation and the token
// norms, which round to fp16 only after their arithmetic); without either,
// keys are fp16 from entry conversion on and staged as fp16, which halves
// their LDS and lets four blocks share a CU at G = 64 instead of three.
// Threads of a flush block.  The loops below stride by this constant rather
// than blockDim.x, so the compiler unrolls them and folds their per-task index
// and address arithmetic (the launch always uses this many).
constexpr int kFlushThreads = 256;
template <int D, int KB, int VB, int G, bool F32K>
__global__ __launch_bounds__(kFlushThreads) void flush_kernel(AppendArgs a) {
  constexpr int NKB = D / 32, NCG = D / G;
  constexpr int CPG = G / kChunk;
  // token rows padded by one bank (4 bytes) so that the lanes reading one
  // channel of 16 or 32 consecutive tokens hit different LDS banks
  using KT = typename std::conditional<F32K, float, __half>::type;
  constexpr int KS = F32K ? D + 1 : D + 2, VS = D + 2;
  // (rows are written as dwords: 4-byte aligned rows, 16-byte aligned bases)
  __shared__ __attribute__((aligned(16))) KT kx[G * KS];
  __shared__ __attribute__((aligned(16))) __half vx[G * VS];  // values are fp16 after entry conversion
  // a staged key as binary32, and the store of an entry-converted key (fp16
  // staging rounds it to fp16 here, as the entry conversion does anyway)
  auto kget = [&](int i) __attribute__((always_inline)) -> float {
    if constexpr (F32K) return kx[i]; else return __half2float(kx[i]);
  };
  auto kput = [&](int i, float x) __attribute__((always_inline)) {
    if constexpr (F32K) kx[i] = x; else kx[i] = __float2half_rn(x);
  };
  __shared__ float ks[D], kmn[D], krs[D];
  __shared__ float vs[G * NCG], vmn[G * NCG], vrs[G * NCG];
  // hybrid quantizer: the offset added to a group's rounded quotients (c0 for
  // a symmetric group, whose stored minimum is then 0; 0 otherwise)
  __shared__ float koff[D], voff[G * NCG];
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
      for (int p = 0; p < 4; ++p) {
        // an fp16 pair as it is, a bf16 pair converted to fp16 (nearest even)
        // two at a time; stored as one dword (rows are 4-byte aligned)
        const uint32_t vh = a.in_dtype == 1 ? vw[p] : bf16x2_to_f16x2(vw[p]);
        if constexpr (F32K) {
          // binary32 keys are staged as given (rotation and norms come first,
          // the fp16 rounding after them)
          const uint32_t w = kw[p];
          kx[i * KS + c0 + 2 * p] = a.in_dtype == 1 ? __half2float(__ushort_as_half(static_cast<uint16_t>(w)))
                                                    : __uint_as_float(w << 16);
          kx[i * KS + c0 + 2 * p + 1] = a.in_dtype == 1 ? __half2float(__ushort_as_half(static_cast<uint16_t>(w >> 16)))
                                                        : __uint_as_float(w & 0xffff0000u);
        } else {
          *reinterpret_cast<uint32_t*>(&kx[i * KS + c0 + 2 * p]) = a.in_dtype == 1 ? kw[p] : bf16x2_to_f16x2(kw[p]);
        }
        *reinterpret_cast<uint32_t*>(&vx[i * VS + c0 + 2 * p]) = vh;
      }
    }
  } else {
  for (int idx = tid; idx < G * D; idx += kFlushThreads) {
    int i = idx / D, c = idx % D;
    int64_t p = pos0 + i;
    if (p >= a.n_old) {
      int64_t src = in_base + (p - a.n_old) * D + c;
      kput(i * KS + c, load_in(a.k, a.in_dtype, src));
      vx[i * VS + c] = __float2half_rn(load_in(a.v, a.in_dtype, src));
    } else {
      const uint8_t* rc = ring + ring_chunk_offset(L, slice, p);
      int t = static_cast<int>(p % kChunk);
      kput(i * KS + c, __half2float(*reinterpret_cast<const __half*>(rc + ring_k_offset(L, t, c))));
      vx[i * VS + c] = *reinterpret_cast<const __half*>(rc + ring_v_offset(L, t, c));
    }
  }
  }
  any_new = (pos0 + G) > a.n_old;
  __syncthreads();
  if (F32K && any_new) {
    // rows [first_new, G) come from the input: rotate (keys) then round to fp16
    int first_new = a.n_old > pos0 ? static_cast<int>(a.n_old - pos0) : 0;
    if constexpr (F32K) {
      if (a.rotate) fwht_rows<D, KS>(kx + first_new * KS, G - first_new, tid, kFlushThreads);
      for (int idx = first_new * D + tid; idx < G * D; idx += kFlushThreads)
        kx[(idx / D) * KS + idx % D] = round_fp16(kx[(idx / D) * KS + idx % D]);
    }
    __syncthreads();
  }

  uint8_t* page = a.cache + page_offset(L, slice, g);

  // key token norms: each key row is divided by its norm and rounded to fp16
  // before the key quantizer; the norm is stored as fp16 (0 for a zero row,
  // whose normalized values are 0)
  if constexpr (F32K) {
    if (L.token_norm) {
      // one wave per row: lane t takes the square sum of elements 2t, 2t + 1
      // (or, for D = 64, lanes 0..31), then each tree level adds pairs (2t,
      // 2t + 1) of the level below: a fixed order, so the norm does not depend
      // on how the work is shared; then a correctly rounded square root
      const int lane = tid % kLanes, wave = tid / kLanes, nwaves = kFlushThreads / kLanes;
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
      for (int idx = tid; idx < G * D; idx += kFlushThreads) {
        const float nrm = knrm[idx / D];
        const int k = (idx / D) * KS + idx % D;
        kput(k, nrm == 0.0f ? 0.0f : round_fp16(kget(k) / nrm));
      }
      __syncthreads();
    }
  }

  // 2. parameters: keys per channel over G tokens, values per token over G
  // channels; two adjacent lanes per group, each over half of it
  auto params = [&](auto hyb_c) __attribute__((always_inline)) {
    constexpr bool HYB = decltype(hyb_c)::value;
    for (int t = tid; t < 2 * D; t += kFlushThreads) {
      const int c = t >> 1, h = t & 1;
      const GroupQ q = group_params_pair<G, KB, HYB>([&](int i) { return kget((h * (G / 2) + i) * KS + c); });
      if (h == 0) {
        ks[c] = q.s;
        krs[c] = q.rs;
        kmn[c] = HYB && q.sym ? 0.0f : q.mn;
        if constexpr (HYB) koff[c] = q.sym ? static_cast<float>((1 << (KB - 1)) - 1) : 0.0f;
        uint16_t* kp = reinterpret_cast<uint16_t*>(page + L.off_kparams);
        const int pi = kparam_index(L, c);
        kp[pi] = q.scale16;
        kp[D + pi] = q.zero16;
      }
    }
    for (int t = tid; t < 2 * G * NCG; t += kFlushThreads) {
      const int task = t >> 1, h = t & 1;
      const int i = task / NCG, cg = task % NCG;
      const __half* row = vx + i * VS + cg * G + h * (G / 2);
      const GroupQ q = group_params_pair<G, VB, HYB>([&](int c) { return __half2float(row[c]); });
      if (h == 0) {
        vs[task] = q.s;
        vrs[task] = q.rs;
        vmn[task] = HYB && q.sym ? 0.0f : q.mn;
        if constexpr (HYB) voff[task] = q.sym ? static_cast<float>((1 << (VB - 1)) - 1) : 0.0f;
        uint16_t* vp = reinterpret_cast<uint16_t*>(page + L.off_vparams + (i / kChunk) * L.vp_chunk_bytes);
        vp[vparam_scale_elem(L, i % kChunk, cg)] = q.scale16;
        vp[vparam_zero_elem(L, i % kChunk, cg)] = q.zero16;
      }
    }
    __syncthreads();
  };
  // 3. key codes: each task assembles one dword of one lane of one chunk
  // 4. value codes, likewise
  auto codes = [&](auto hyb_c) __attribute__((always_inline)) {
    constexpr bool HYB = decltype(hyb_c)::value;
    const float one = opaque_one();
    // the page's code blocks: uniform bases, 32-bit offsets within the page
    uint8_t* const kcodes = page + L.off_kcodes;
    uint8_t* const vcodes = page + L.off_vcodes;
    const uint32_t kc_chunk = static_cast<uint32_t>(L.kc_chunk_bytes), vc_chunk = static_cast<uint32_t>(L.vc_chunk_bytes);
    {
      constexpr int KW = 2 * NKB * KB / 4;
      for (int task = tid; task < CPG * kLanes * KW; task += kFlushThreads) {
        int ch = task / (kLanes * KW);
        int l = (task / KW) % kLanes;
        int d = task % KW;
        int l16 = l & 15, j = l >> 4;
        // field k: element e = k % 8 of sub-block k / 8
        constexpr int SUBS = KB == 4 ? 1 : 2;
        const uint32_t word = pack_codes<8 * SUBS, HYB>(
            [&](int k) { const int e = k & 7, sub = k >> 3;
                         return KB == 4 ? 16 * (e & 1) + 4 * (e >> 1) : 16 * (e & 1) + 8 * sub + 2 * (e >> 1); },
            [&](int k) {
              const int e = k & 7, sub = k >> 3;
              const int combo = KB == 4 ? d : 2 * d + sub;
              const int mt = combo / NKB, kb = combo % NKB;
              const int i = ch * kChunk + 16 * mt + l16;  // token within the group
              const int c = 32 * kb + 8 * j + e;
              return quant_op(kget(i * KS + c), kmn[c], ks[c], krs[c], HYB ? koff[c] : 0.0f, one);
            });
        *reinterpret_cast<uint32_t*>(kcodes + (static_cast<uint32_t>(ch) * kc_chunk +
                                               static_cast<uint32_t>(lane_dword_offset(KW, l, d)))) = word;
      }
    }
    {
      constexpr int NMT = D / 16;
      constexpr int VW = NMT * VB / 4;
      for (int task = tid; task < CPG * kLanes * VW; task += kFlushThreads) {
        int ch = task / (kLanes * VW);
        int l = (task / VW) % kLanes;
        int d = task % VW;
        int l16 = l & 15, j = l >> 4;
        constexpr int SUBS = VB == 4 ? 1 : 2;
        const uint32_t word = pack_codes<8 * SUBS, HYB>(
            [&](int k) { return vcode_bit(VB, VB == 4 ? d : 2 * d + (k >> 3), k & 7); },
            [&](int k) {
              const int e = k & 7, mt = VB == 4 ? d : 2 * d + (k >> 3);
              const int c = 16 * mt + l16, cg = c / G;
              const int i = ch * kChunk + tau(j, e);
              const int pv = i * NCG + cg;
              return quant_op(__half2float(vx[i * VS + c]), vmn[pv], vs[pv], vrs[pv], HYB ? voff[pv] : 0.0f, one);
            });
        *reinterpret_cast<uint32_t*>(vcodes + (static_cast<uint32_t>(ch) * vc_chunk +
                                               static_cast<uint32_t>(lane_dword_offset(VW, l, d)))) = word;
      }
    }
  };
  if (a.hybrid != 0) {
    params(std::true_type{});
    codes(std::true_type{});
  } else {
    params(std::false_type{});
    codes(std::false_type{});
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
  if (a.rotate || a.L.token_norm)
    hipLaunchKernelGGL((flush_kernel<D, KB, VB, G, true>), grid, dim3(kFlushThreads), 0, s, a);
  else
    hipLaunchKernelGGL((flush_kernel<D, KB, VB, G, false>), grid, dim3(kFlushThreads), 0, s, a);
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
