// kvq_decode.hip -- fused dequant + single-query decode attention on the
// packed cache, split over the token axis, and the cross-split merge.
//
// Computes softmax(q K^T / sqrt(d)) V ("Asymmetric Key-Value Quantization:
// 2-Bit Values and 4-Bit Keys under Long-Context Drift", section 1) over
// keys quantized per channel and values quantized per token ("[Framework] The
// Asymmetric Key-Value Cache Compression", section III), plus the fp16
// window of recent tokens.  Decode attention is bound by reading the cache
// (the NOVA-KV abstract on the page "WUSH-KV: KV Cache Quantization with
// Data-Adaptive Transforms" makes this point), so the kernel is built to
// stream every byte once.
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
// as fp16 subnormals 2^-24 * 2^p * code (see kvq_layout.h): the 2^p factors
// are folded into the B operands and the 2^-24 into the scores and the final
// output, all exact.  Softmax runs in the log2 domain (exp2), log2(e)/sqrt(D)
// folded into q.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTwo24 = 16777216.0f;  // undoes the 2^-24 of subnormal code operands

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Field masks kept in SGPRs (v_and_b32 with an SGPR operand instead of a
// 32-bit literal per instruction).
__device__ __forceinline__ uint32_t sgpr_const(uint32_t x) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(x));
  return r;
}

template <int BITS>
struct CodeMasks {
  uint32_t m[4];
  __device__ __forceinline__ CodeMasks() {
    if (BITS == 4) {
      m[0] = sgpr_const(0x000F000Fu);
      m[1] = sgpr_const(0x00F000F0u);
      m[2] = m[0];
      m[3] = m[1];
    } else {
      m[0] = sgpr_const(0x00030003u);
      m[1] = sgpr_const(0x000C000Cu);
      m[2] = sgpr_const(0x00300030u);
      m[3] = sgpr_const(0x00C000C0u);
    }
  }
};

// A b-bit field at bit p of a 16-bit half, with every other bit of the half
// clear, is the fp16 subnormal 2^(p - 24) * code exactly.
//
// Precision note (measured on gfx950): the matrix cores' fp32 result of a
// 32-product sum is biased low by a few ulp (about -4e-6 relative) when an
// input is a small subnormal, and equally so when a large offset is added
// and cancelled (the 1024 + code encoding); only sums of normal-range inputs
// are unbiased.  The PV code sum is then amplified by its cancellation
// against the zero-point sum (|sum p s code| / |output| is 30-70 on long
// diffuse contexts), which puts the attention output's relative error at
// 1e-4 .. 1.5e-3 against exact arithmetic.  Normal-range code operands would
// cost one more VALU operation per operand dword (about a quarter more VALU
// work per chunk).
// 4-bit word -> 8 values 2^-24 * mult(e) * code_e, mult = 1, 1, 16, 16, 1, 1, 16, 16.
__device__ __forceinline__ half8 unpack4(uint32_t w, const CodeMasks<4>& u) {
  const uint32_t w8 = w >> 8;
  return __builtin_bit_cast(half8, u32x4{w & u.m[0], w & u.m[1], w8 & u.m[0], w8 & u.m[1]});
}
// One 2-bit sub-block (the low byte of each half of w) -> 8 values
// 2^-24 * 4^(e>>1) * code_e.
__device__ __forceinline__ half8 unpack2(uint32_t w, const CodeMasks<2>& u) {
  return __builtin_bit_cast(half8, u32x4{w & u.m[0], w & u.m[1], w & u.m[2], w & u.m[3]});
}

template <int BITS>
__host__ __device__ constexpr float code_mult(int e) {
  return BITS == 4 ? (((e >> 1) & 1) ? 16.0f : 1.0f) : static_cast<float>(1 << (2 * (e >> 1)));
}

template <int BITS>
__device__ __forceinline__ half8 a_operand(const uint32_t* words, int idx, const CodeMasks<BITS>& u) {
  // idx-th 8-element operand of a lane: 4-bit -> one word each; 2-bit -> two per word
  if constexpr (BITS == 4) {
    return unpack4(words[idx], u);
  } else {
    const uint32_t w = words[idx >> 1];
    return unpack2((idx & 1) ? (w >> 8) : w, u);
  }
}

// Reductions over the four lane groups j of a column (lanes l16, l16 + 16,
// l16 + 32, l16 + 48), on the VALU with gfx950's lane swaps.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_fmaxf(a, b); }
__device__ __forceinline__ float wave_max_j(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_j(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float load_q(const void* p, int dtype, int64_t i) {
  if (dtype == 0) return static_cast<const float*>(p)[i];
  uint16_t u = static_cast<const uint16_t*>(p)[i];
  if (dtype == 1) return __half2float(__ushort_as_half(u));
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

__device__ __forceinline__ float h2f_lo(uint32_t w) { return __half2float(__ushort_as_half(static_cast<uint16_t>(w))); }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return __half2float(__ushort_as_half(static_cast<uint16_t>(w >> 16))); }

// All arithmetic helpers below are plain C++ (no inline assembly), so the
// compiler sees every VGPR they write and inserts the wait states an MFMA
// needs before reading a freshly written operand.
__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ __forceinline__ uint32_t as_u32(half2v x) { return __builtin_bit_cast(uint32_t, x); }
// fp16 pair (fp16(a0 * s.lo), fp16(a1 * s.hi)) from fp32 a and an fp16 pair s,
// each rounded once (fma with +0 keeps the product and selects v_fma_mix*).
__device__ __forceinline__ uint32_t mix_mul2(float a0, float a1, uint32_t s) {
  const half2v sv = as_h2(s);
  const half2v r = {static_cast<_Float16>(__builtin_fmaf(a0, static_cast<float>(sv[0]), 0.0f)),
                    static_cast<_Float16>(__builtin_fmaf(a1, static_cast<float>(sv[1]), 0.0f))};
  return as_u32(r);
}
// fp16 pair (fp16(a0 * s.lo - c.lo), fp16(a1 * s.hi - c.hi)), one rounding each.
__device__ __forceinline__ uint32_t mix_fms2(float a0, float a1, uint32_t s, uint32_t c) {
  const half2v sv = as_h2(s), cv = as_h2(c);
  const half2v r = {static_cast<_Float16>(__builtin_fmaf(a0, static_cast<float>(sv[0]), -static_cast<float>(cv[0]))),
                    static_cast<_Float16>(__builtin_fmaf(a1, static_cast<float>(sv[1]), -static_cast<float>(cv[1])))};
  return as_u32(r);
}
// Two-part fp16 operand of x = a * s (a fp32, s an fp16 pair): part 0 =
// fp16(x), part 1 = fp16(x - part 0).  In column-split mode a lane produces
// the part its columns hold: mask 0 gives part 0, all-ones part 1.
__device__ __forceinline__ uint32_t split_part(float a0, float a1, uint32_t s, uint32_t mask) {
  return mix_fms2(a0, a1, s, mix_mul2(a0, a1, s) & mask);
}
// Exact-residual product of fp16 pairs: with x = fp16(a * s), the fp16 fma
// a * s - x is exact (the rounding error of a product of two fp16 values is
// an fp16 value), so fp16(b * s + (a * s - x)) is the second part of
// (a + b) * s for a two-part a + b.
__device__ __forceinline__ half2v pk_mul(half2v a, half2v b) { return a * b; }
__device__ __forceinline__ half2v pk_fma(half2v a, half2v b, half2v c) { return __builtin_elementwise_fma(a, b, c); }
__device__ __forceinline__ uint32_t pack_h2(float x0, float x1) {
  const half2v r = {static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
  return as_u32(r);
}
// Sum with the lane 8 places away inside each row of 16 (row_ror:8): lanes h
// and h + 8 both receive x_h + x_{h+8}.
__device__ __forceinline__ float add_ror8(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
}

// ---- LDS staging of the code stream ----------------------------------------
// Chunks are copied global -> LDS with gfx950's direct loads (no VGPRs held
// while in flight), several chunks ahead of the one being processed.  The
// copies are issued from inline assembly so the compiler neither reorders nor
// conservatively waits for them; the kernel waits with explicit vmcnt values
// (every vector-memory instruction of the main loop is one of these copies,
// issued in a fixed pattern, and vector memory returns in order).
#define KVQ_AS3 __attribute__((address_space(3)))
// M0 is named as clobbered by the copies below; the compiler reserves M0 and
// warns about it, but nothing else in these kernels uses M0.
#pragma clang diagnostic ignored "-Winline-asm"

// The destination LDS address is taken from M0; an LDS-DMA instruction that
// reads M0 right after an SALU write of it needs a wait state (s_nop).  The
// cache is streamed once per decode, so the copies are non-temporal (nt):
// measured on MI355X, the same copy pattern streams at 6.9 TB/s with nt and
// 6.1 TB/s without.
// 1 KiB: lane l copies global [base + 16 l, +16) to LDS [lds + 16 l, +16)
__device__ __forceinline__ void dma_1k(const uint8_t* gbase, uint32_t lane16, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(lane16), "s"(gbase), "s"(lds) : "memory", "m0");
}
// 256 B: lane l copies global [base + 4 l, +4) to LDS [lds + 4 l, +4)
__device__ __forceinline__ void dma_256(const uint8_t* gbase, uint32_t lane4, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 1\n\tglobal_load_lds_dword %0, %1 nt"
               :: "v"(lane4), "s"(gbase), "s"(lds) : "memory", "m0");
}
// Outstanding LDS reads are drained before a slot is overwritten.
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <int BYTES>
__device__ __forceinline__ void dma_block(const uint8_t* g, uint32_t lane16, uint32_t lane4, uint32_t lds) {
  static_assert(BYTES % 256 == 0, "DMA blocks are whole 256-byte units");
#pragma unroll
  for (int o = 0; o + 1024 <= BYTES; o += 1024) dma_1k(g + o, lane16, lds + o);
#pragma unroll
  for (int o = BYTES / 1024 * 1024; o < BYTES; o += 256) dma_256(g + o, lane4, lds + o);
}
template <int BYTES>
constexpr int dma_count() { return BYTES / 1024 + (BYTES % 1024) / 256; }
// Number of chunks among the NBUF - 1 issued after chunk position ch (mod
// CPG) that start a group, i.e. that also carry key parameters.
template <int NBUF, int CPG>
constexpr int kp_after(int ch) {
  int n = 0;
  for (int k = 1; k < NBUF; ++k) n += ((ch + k) % CPG) == 0;
  return n;
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Page geometry of one token group (the same numbers as make_layout's,
// as compile-time constants of the kernel instance).
template <int D, int KB, int VB, int G>
struct PageShape {
  static constexpr int NCG = D / G, CPG = G / kChunk;
  static constexpr int KC = kChunk * D * KB / 8, VC = kChunk * D * VB / 8;
  static constexpr int VPB = (kChunk * NCG * 4 + 255) / 256 * 256, KPB = 4 * D;
  static constexpr int OFF_KC = 0, OFF_KP = CPG * KC, OFF_VC = OFF_KP + KPB, OFF_VP = OFF_VC + CPG * VC;
  static constexpr int BYTES = OFF_VP + CPG * VPB;
};

// Running-max slack of the online softmax (base-2 units): the accumulators
// are rescaled only when a chunk's maximum exceeds the running maximum by more
// than this, so weights stay <= 2^0.5 and the fp16 PV operand p * scale stays
// below 65504 for any scale of fp16 data.
constexpr float kMaxSlack = 0.5f;

template <int D, int KB, int VB, int G, bool CS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(CS ? 3 : 2)))
void decode_kernel(DecodeArgs a) {
  using PS = PageShape<D, KB, VB, G>;
  constexpr int NKB = D / 32, NMT = D / 16, NCG = PS::NCG, CPG = PS::CPG;
  constexpr int KW = 2 * NKB * KB / 4, VW = NMT * VB / 4, VPW = 8 * NCG;
  // B operands carry each value as two fp16 parts (hi + lo) so the folded
  // products keep ~22 bits: in CS mode (at most 8 heads) hi sits in columns
  // 0-7 and lo in columns 8-15 of one MFMA; otherwise two MFMAs.
  constexpr int NP = CS ? 1 : 2;
  const Layout& L = a.L;
  const int l = threadIdx.x, l16 = l & 15, j = l >> 4;
  const int S = a.splits;
  const int64_t slice = blockIdx.x / S;
  const int s = static_cast<int>(blockIdx.x % S);
  const int b = static_cast<int>(slice / a.Hkv), hkv = static_cast<int>(slice % a.Hkv);
  const int h = CS ? (l16 & 7) : l16;
  const bool lo_lane = CS && l16 >= 8;
  const bool hv = h < a.gqa;
  const int hq = hkv * a.gqa + (hv ? h : 0);
  const uint32_t part_mask = lo_lane ? 0xFFFFFFFFu : 0u;  // this lane's part (CS mode)

  // ---- query: lane owns channels 32 kb + 8 j + e of head h, times log2(e)/sqrt(D)
  float qm[NKB][8];
  const float qscale = kLog2e * (D == 128 ? 0.08838834764831845f : 0.125f);
  if (a.rotate) {
    extern __shared__ float qsh[];  // gqa * D floats, sized at launch
    const int64_t base = (static_cast<int64_t>(b) * a.Hq + hkv * a.gqa) * D;
    for (int idx = l; idx < a.gqa * D; idx += kLanes) qsh[idx] = load_q(a.q, a.in_dtype, base + idx);
    __syncthreads();
    for (int hh = 1; hh < D; hh <<= 1) {
      for (int k = l; k < a.gqa * (D / 2); k += kLanes) {
        int r = k / (D / 2), p = k % (D / 2);
        int i0 = r * D + (p / hh) * 2 * hh + (p % hh);
        float x0 = qsh[i0], x1 = qsh[i0 + hh];
        qsh[i0] = x0 + x1;
        qsh[i0 + hh] = x0 - x1;
      }
      __syncthreads();
    }
    const float rs = qscale * (D == 128 ? 0.08838834764831845f : 0.125f);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        qm[kb][e] = hv ? qsh[(hv ? h : 0) * D + 32 * kb + 8 * j + e] * rs : 0.0f;
  } else {
    const int64_t base = (static_cast<int64_t>(b) * a.Hq + hq) * D;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) qm[kb][e] = hv ? load_q(a.q, a.in_dtype, base + 32 * kb + 8 * j + e) * qscale : 0.0f;
  }
  // Per-split fp16 parts of the query (part 1 = fp16(x - part 0)):
  //   qz: q itself, the B operand of the key zero-point bias and of the window;
  //   qh / ql: q / mult (the code multipliers of the key operand), from which
  //   the per-group B operand q * scale / mult is formed by exact-residual fp16
  //   products.  In CS mode ql holds part 0 on hi lanes (so the same
  //   instructions produce each lane's own part).
  uint32_t qz[NP][NKB][4], qh[NKB][4], ql[NKB][4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = qm[kb][2 * i], x1 = qm[kb][2 * i + 1];
      const float h0 = static_cast<float>(static_cast<_Float16>(x0)), h1 = static_cast<float>(static_cast<_Float16>(x1));
      const uint32_t z_hi = pack_h2(x0, x1), z_lo = pack_h2(x0 - h0, x1 - h1);
      const float d0 = x0 * (1.0f / code_mult<KB>(2 * i)), d1 = x1 * (1.0f / code_mult<KB>(2 * i + 1));
      const float e0 = static_cast<float>(static_cast<_Float16>(d0)), e1 = static_cast<float>(static_cast<_Float16>(d1));
      const uint32_t d_hi = pack_h2(d0, d1), d_lo = pack_h2(d0 - e0, d1 - e1);
      if (CS) {
        qz[0][kb][i] = lo_lane ? z_lo : z_hi;
        ql[kb][i] = lo_lane ? d_lo : d_hi;
      } else {
        qz[0][kb][i] = z_hi;
        qz[NP - 1][kb][i] = z_lo;
        ql[kb][i] = d_lo;
      }
      qh[kb][i] = d_hi;
    }

  const CodeMasks<KB> uk;
  const CodeMasks<VB> uv;

  // Online-softmax state (per column, uniform over j).  m is the running max
  // in log2 units; acc holds the PV sums in units of 2^-24 while quantized
  // chunks are processed (subnormal code operands), real units afterwards.
  float m = -INFINITY, mslack = -INFINITY, lsum = 0.0f;
  f32x4 acc[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // zero-point sums per value group and per code-multiplier class i = e >> 1
  // (the weights below are p / mult; the classes are rescaled at the end)
  constexpr int NI = VB == 4 ? 2 : 4;
  float zacc[NCG][NI];
#pragma unroll
  for (int i = 0; i < NCG; ++i)
#pragma unroll
    for (int c = 0; c < NI; ++c) zacc[i][c] = 0.0f;

  // (called wave-uniformly; mnew = max(m, chunk max) per column)
  auto rescale = [&](float mnew) __attribute__((always_inline)) {
    const float al = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
    for (int i = 0; i < NMT; ++i) acc[i] *= al;
#pragma unroll
    for (int i = 0; i < NCG; ++i)
#pragma unroll
      for (int c = 0; c < NI; ++c) zacc[i][c] *= al;
    lsum *= al;
    m = mnew;
    mslack = mnew + kMaxSlack;
  };

  const int g0 = s * static_cast<int>(a.groups_per_split);
  const int g1 = min(g0 + static_cast<int>(a.groups_per_split), static_cast<int>(a.ngroups));

  // ---- LDS ring of NBUF chunk slots: [key codes][value codes][value params][key params]
  constexpr int KC = PS::KC, VC = PS::VC, VPB = PS::VPB, KPB = PS::KPB;
  constexpr int SLOT = KC + VC + VPB + KPB;
  // Slots per wave: three chunks in flight when the ring stays small enough
  // for three waves per SIMD (12 per CU within 160 KiB of LDS), else two.
  constexpr int NBUF = 4 * SLOT <= 13 * 1024 ? 4 : 3;
  constexpr int NBASE = dma_count<KC>() + dma_count<VC>() + dma_count<VPB>(), NKP = dma_count<KPB>();
  __shared__ __attribute__((aligned(16))) uint8_t ring[NBUF * SLOT];
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((KVQ_AS3 uint8_t*)ring));
  const uint32_t lane16 = static_cast<uint32_t>(l) * 16, lane4 = static_cast<uint32_t>(l) * 4;

  if (g1 > g0) {
    const uint8_t* slice_pages = a.cache + page_offset(L, slice, 0);

    // copy position chi of group gi into the slot at LDS address sl; a group's
    // first chunk also carries the group's key scale/zero rows
    auto issue = [&](int gi, auto chi_c, uint32_t sl) __attribute__((always_inline)) {
      constexpr int chi = decltype(chi_c)::value;
      const uint8_t* page = slice_pages + static_cast<int64_t>(gi) * PS::BYTES;
      lds_reads_done();
      dma_block<KC>(page + PS::OFF_KC + chi * KC, lane16, lane4, sl);
      dma_block<VC>(page + PS::OFF_VC + chi * VC, lane16, lane4, sl + KC);
      dma_block<VPB>(page + PS::OFF_VP + chi * VPB, lane16, lane4, sl + KC + VC);
      if constexpr (chi == 0) dma_block<KPB>(page + PS::OFF_KP, lane16, lane4, sl + KC + VC + VPB);
    };

    uint32_t bq[NP][NKB][4];  // B operand of QK^T (fp16 pairs), per part
    float cb = 0.0f;          // this group's zero-point score bias (log2 units)
    // exponent offsets per value-code multiplier class: exp2(score - m - log2(mult))
    // is p / mult, the weight the PV operand needs
    float bmc[NI];
    auto set_bmc = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < NI; ++c) bmc[c] = (cb - m) - (VB == 4 ? 4.0f * (c & 1) : 2.0f * c);
    };

    auto process = [&](const uint8_t* sl, bool group_start, auto&& refill) __attribute__((always_inline)) {
      if (group_start) {
        // B operand from this group's key scales: q * s / mult in two parts
        // (exact-residual fp16 products), and the bias sum_c q_c z_c by MFMA
        // (every row of the bias tile is the same sum)
        const u32x4* ps = reinterpret_cast<const u32x4*>(sl + KC + VC + VPB) + j * NKB;
        const u32x4* pz = reinterpret_cast<const u32x4*>(sl + KC + VC + VPB + 2 * D) + j * NKB;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4 sw = ps[kb];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const half2v sv = as_h2(sw[i]), hh = as_h2(qh[kb][i]);
            const half2v x = pk_mul(hh, sv);
            const half2v y = pk_fma(hh, sv, -x);  // exact: hh * sv - x
            if (CS) {
              bq[0][kb][i] = as_u32(pk_fma(as_h2(ql[kb][i]), sv, as_h2(as_u32(y) & part_mask)));
            } else {
              bq[0][kb][i] = as_u32(x);
              bq[NP - 1][kb][i] = as_u32(pk_fma(as_h2(ql[kb][i]), sv, y));
            }
          }
        }
        f32x4 cbt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const half8 az = __builtin_bit_cast(half8, pz[kb]);
#pragma unroll
          for (int pp = 0; pp < NP; ++pp) {
            const half8 bz = __builtin_bit_cast(half8, u32x4{qz[pp][kb][0], qz[pp][kb][1], qz[pp][kb][2], qz[pp][kb][3]});
            cbt = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, bz, cbt, 0, 0, 0);
          }
        }
        cb = CS ? add_ror8(cbt[0]) : cbt[0];
        set_bmc();
      }
      uint32_t kw[KW], vw[VW], vp[VPW];
      if constexpr (KW >= 4) {
#pragma unroll
        for (int v = 0; v < KW / 4; ++v) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(sl + v * (kLanes * 16) + l * 16);
          kw[4 * v] = x[0]; kw[4 * v + 1] = x[1]; kw[4 * v + 2] = x[2]; kw[4 * v + 3] = x[3];
        }
      } else {
        const u32x2 x = *reinterpret_cast<const u32x2*>(sl + l * 8);
        kw[0] = x[0]; kw[1] = x[1];
      }
      if constexpr (VW >= 4) {
#pragma unroll
        for (int v = 0; v < VW / 4; ++v) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(sl + KC + v * (kLanes * 16) + l * 16);
          vw[4 * v] = x[0]; vw[4 * v + 1] = x[1]; vw[4 * v + 2] = x[2]; vw[4 * v + 3] = x[3];
        }
      } else {
        const u32x2 x = *reinterpret_cast<const u32x2*>(sl + KC + l * 8);
        vw[0] = x[0]; vw[1] = x[1];
      }
      {
        const u32x4* vpp = reinterpret_cast<const u32x4*>(sl + KC + VC) + j * (VPW / 4);
#pragma unroll
        for (int v = 0; v < VPW / 4; ++v) {
          const u32x4 x = vpp[v];
          vp[4 * v] = x[0]; vp[4 * v + 1] = x[1]; vp[4 * v + 2] = x[2]; vp[4 * v + 3] = x[3];
        }
      }
      // QK^T: two 16-token tiles; C = 2^-24 * (score - bias)
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const half8 a0 = a_operand<KB>(kw, kb, uk);
        const half8 a1 = a_operand<KB>(kw, NKB + kb, uk);
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          const half8 bb = __builtin_bit_cast(half8, u32x4{bq[pp][kb][0], bq[pp][kb][1], bq[pp][kb][2], bq[pp][kb][3]});
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bb, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bb, c1, 0, 0, 0);
        }
      }
      float t[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        t[r] = CS ? add_ror8(c0[r]) : c0[r];
        t[4 + r] = CS ? add_ror8(c1[r]) : c1[r];
      }
      // online softmax over the chunk's 8 scores per lane (tokens tau(j, e))
      const float tmax = fmax2(fmax2(fmax2(t[0], t[1]), fmax2(t[2], t[3])), fmax2(fmax2(t[4], t[5]), fmax2(t[6], t[7])));
      const float cmax = wave_max_j(__builtin_fmaf(tmax, kTwo24, cb));
      if (__builtin_amdgcn_ballot_w64(cmax > mslack)) {
        rescale(fmax2(m, cmax));
        set_bmc();
      }
      // pm = p / mult (the exponent offset per class), lsum += pm * mult
      float pm[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pm[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[e], kTwo24, bmc[VB == 4 ? ((e >> 1) & 1) : (e >> 1)]));
        lsum = __builtin_fmaf(pm[e], code_mult<VB>(e), lsum);
      }
      // PV B operand p * value scale / mult (one fp16 part: its rounding is far
      // below the matrix cores' own error on these sums) and the zero-point sums.
      // In CS mode lanes 8-15 produce duplicate columns, cleared before the window.
      uint32_t bp[NCG][4];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t sp = vp[cg * 8 + i], zp = vp[cg * 8 + 4 + i];
          bp[cg][i] = mix_mul2(pm[2 * i], pm[2 * i + 1], sp);
          float& z = zacc[cg][VB == 4 ? (i & 1) : i];
          z = __builtin_fmaf(pm[2 * i], h2f_lo(zp), z);
          z = __builtin_fmaf(pm[2 * i + 1], h2f_hi(zp), z);
        }
      }
      // the slot's data has long been read into registers: refill it with a
      // later chunk before the PV products
      refill();
      // PV on the subnormal code operands
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const half8 av = a_operand<VB>(vw, mt, uv);
        const uint32_t* bw = bp[(16 * mt) / G];
        const half8 bb = __builtin_bit_cast(half8, u32x4{bw[0], bw[1], bw[2], bw[3]});
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bb, acc[mt], 0, 0, 0);
      }
    };

    // Ring slots rotate through LDS addresses ring_lds + k * SLOT; chunk c of
    // the split sits in slot c % NBUF.  Once chunk c's data is in registers its
    // slot is refilled with chunk c + NBUF, so NBUF chunks are in flight while
    // one is being computed.
    uint32_t sl_proc = ring_lds;
    auto next_slot = [&](uint32_t x) { return x + SLOT == ring_lds + NBUF * SLOT ? ring_lds : x + SLOT; };
    // prologue: NBUF chunks in flight (split boundaries are group-aligned;
    // copies past the split's end repeat its last group, so the number of
    // copies per issue never changes)
    static_for<0, NBUF>([&](auto k) {
      constexpr int K = decltype(k)::value;
      issue(min(g0 + K / CPG, g1 - 1), std::integral_constant<int, K % CPG>{}, ring_lds + K * SLOT);
    });
    for (int g = g0; g < g1; ++g) {
      static_for<0, CPG>([&](auto chc) {
        constexpr int ch = decltype(chc)::value;
        constexpr int ahead = ch + NBUF;
        // copies issued after chunk c's: chunks c+1 .. c+NBUF-1, NBASE each,
        // plus NKP for each of them that starts a group
        wait_vmcnt<(NBUF - 1) * NBASE + kp_after<NBUF, CPG>(ch) * NKP>();
        const uint32_t sl = sl_proc;
        process(ring + (sl - ring_lds), ch == 0, [&]() __attribute__((always_inline)) {
          issue(min(g + ahead / CPG, g1 - 1), std::integral_constant<int, ahead % CPG>{}, sl);
        });
        sl_proc = next_slot(sl_proc);
      });
    }
    wait_vmcnt<0>();  // no copy into LDS outlives the loop
  }
  // quantized-chunk sums to real units; in CS mode lanes 8-15 held duplicate
  // columns and now start the window's second parts from zero
#pragma unroll
  for (int i = 0; i < NMT; ++i) acc[i] = lo_lane ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i] * kTwo24;

  // ---- fp16 window chunks: the last split
  if (s == S - 1 && a.rc1 > a.rc0) {
    for (int64_t rc = a.rc0; rc < a.rc1; ++rc) {
      const uint8_t* rch = a.cache + ring_chunk_offset(L, slice, rc * kChunk);
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const half8 a0 = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(rch + ((0 * NKB + kb) * kLanes + l) * 16));
        const half8 a1 = __builtin_bit_cast(half8, *reinterpret_cast<const u32x4*>(rch + ((1 * NKB + kb) * kLanes + l) * 16));
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          const half8 bb = __builtin_bit_cast(half8, u32x4{qz[pp][kb][0], qz[pp][kb][1], qz[pp][kb][2], qz[pp][kb][3]});
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bb, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bb, c1, 0, 0, 0);
        }
      }
      const int64_t pos0 = rc * kChunk;
      const bool partial = pos0 + kChunk > a.n;
      float sc[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = CS ? add_ror8(c0[r]) : c0[r];
        sc[4 + r] = CS ? add_ror8(c1[r]) : c1[r];
      }
      uint32_t vmask[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
      if (partial) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (pos0 + tau(j, e) >= a.n) {
            sc[e] = -INFINITY;
            vmask[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
      }
      float cmax = fmax2(fmax2(fmax2(sc[0], sc[1]), fmax2(sc[2], sc[3])), fmax2(fmax2(sc[4], sc[5]), fmax2(sc[6], sc[7])));
      cmax = wave_max_j(cmax);
      if (__builtin_amdgcn_ballot_w64(cmax > mslack)) rescale(fmax2(m, cmax));
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sc[e] - m);
        lsum += p[e];
      }
      uint32_t bpr[NP][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t one = 0x3C003C00u;  // fp16 1.0 pair
        if (CS) {
          bpr[0][i] = split_part(p[2 * i], p[2 * i + 1], one, part_mask);
        } else {
          const uint32_t hi = mix_mul2(p[2 * i], p[2 * i + 1], one);
          bpr[0][i] = hi;
          bpr[NP - 1][i] = mix_fms2(p[2 * i], p[2 * i + 1], one, hi);
        }
      }
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        u32x4 vwd = *reinterpret_cast<const u32x4*>(rch + kChunk * D * 2 + (mt * kLanes + l) * 16);
        vwd[0] &= vmask[0]; vwd[1] &= vmask[1]; vwd[2] &= vmask[2]; vwd[3] &= vmask[3];
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          const half8 bb = __builtin_bit_cast(half8, u32x4{bpr[pp][0], bpr[pp][1], bpr[pp][2], bpr[pp][3]});
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, vwd), bb, acc[mt], 0, 0, 0);
        }
      }
    }
  }

  // ---- finalize: combine the two parts (CS), reduce over lane groups, write
  if (CS) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mt][r] = add_ror8(acc[mt][r]);
  }
  lsum = wave_sum_j(lsum);
  float zsum[NCG];
#pragma unroll
  for (int i = 0; i < NCG; ++i) {
    float z = 0.0f;
#pragma unroll
    for (int c = 0; c < NI; ++c) z = __builtin_fmaf(zacc[i][c], VB == 4 ? ((c & 1) ? 16.0f : 1.0f) : static_cast<float>(1 << (2 * c)), z);
    zsum[i] = wave_sum_j(z);
  }
  if (hv && !lo_lane) {
    const int64_t row = static_cast<int64_t>(b) * a.Hq + hq;
    if (a.write_final) {
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int c0 = 16 * mt + 4 * j;
        f32x4 o = (acc[mt] + zsum[c0 / G]) * inv;
        *reinterpret_cast<f32x4*>(a.out + row * D + c0) = o;
      }
    } else {
      float* pr = a.partial + (row * S + s) * (D + 4);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int c0 = 16 * mt + 4 * j;
        f32x4 o = acc[mt] + zsum[c0 / G];
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

  const int q = t % Q, sp = t / Q;
  // four records in flight per thread; an empty split's record is never used
  // (its o may be anything), so it is selected away rather than scaled by 0
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  int s = sp;
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

template <int D, int KB, int VB, int G>
hipError_t decode_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(a.L.slices * a.splits));
  const size_t lds = a.rotate ? static_cast<size_t>(a.gqa) * D * sizeof(float) : 0;
  if (a.gqa <= 8)
    hipLaunchKernelGGL((decode_kernel<D, KB, VB, G, true>), grid, dim3(kLanes), lds, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, KB, VB, G, false>), grid, dim3(kLanes), lds, s, a);
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
  if (splits < 1 || splits > kMergeMaxSplits || (D != 64 && D != 128)) return hipErrorInvalidValue;
  if (D == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(static_cast<unsigned>(rows)), dim3(kMergeThreads), 0, s, partial, out, splits);
  else
    hipLaunchKernelGGL(merge_kernel<128>, dim3(static_cast<unsigned>(rows)), dim3(kMergeThreads), 0, s, partial, out, splits);
  return hipGetLastError();
}

}  // namespace kvq
