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
// groups (a split).  The GQA query heads of the slice are columns of the MFMA
// B operand, replicated across the 16 columns so that the per-score softmax
// work is shared out over the replicas (see decode_split).  Launches:
// decode_kernel (one wave per workgroup; the splits' partials go to memory
// for the merge kernel), decode_fused_kernel (a slice's 4 or 8 splits as the
// waves of one workgroup, merged in LDS) and decode_mixed_kernel (groups of
// several bit widths).  In a one-call decode step the wave whose window chunk
// holds the appended token also writes that token's window slots.
//
// Scale folding (exact in real arithmetic):
//   keys, per channel c of group g:  q . khat_t = sum_c (q_c s_gc) code_tc + sum_c q_c z_gc
//   values, per token t, group j:    sum_t p_t vhat_tc = sum_t (p_t s_tj) code_tc + sum_t p_t z_tj
// so both products run on raw integer codes: (q_c s_gc) is the B operand of
// QK^T once per token group, (p_t s_tj) the B operand of PV once per chunk,
// and the zero-point sums are added as per-head biases.  Key codes enter the
// MFMA as fp16 subnormals 2^-24 * 2^p * code, value codes as the normal fp16
// values 2^p * code (see kvq_layout.h and the precision note below): the 2^p
// factors are folded into the B operands and the 2^-24 into the scores, all
// exact.  Softmax runs in the log2 domain (exp2), log2(e)/sqrt(D) folded
// into q.
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
// clear, is the fp16 subnormal 2^(p - 24) * code exactly (key operands).
//
// Precision (measured on gfx950 with chains of MFMAs against exact sums): the
// matrix cores' fp32 result is biased low when an input is an fp16 subnormal
// (about -7e-6 relative over 128 MFMAs with weights spread like softmax
// weights, in either operand), and the bias scales with the size of the
// terms, not of the sum; with normal-range inputs the error has no
// measurable bias.  The value codes' product sum cancels against the
// zero-point sum (|sum p s code| / |output| is 30-70 on long diffuse
// contexts), so a bias there is amplified into the output: the value
// operands are therefore normal-range (see v_operand).  The key codes keep
// the subnormal form: their bias moves a score by ~1e-5 in log2 units, far
// below the tolerance (also with token norms multiplied into the scores:
// normal-range key operands measured no different there).
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
// Value operand of M-tile mt (16 channels x 32 tokens) from the lane's value
// code words, as normal-range fp16 values equal to the codes: the words are
// laid out (vcode_bit in kvq_layout.h) so that one mask leaves every code of
// the tile in the low bits of a nibble of its own, which the fp4 (e2m1, 2-bit
// codes: value code / 2, scaled by 2) or fp8 (e4m3, 4-bit codes: value
// code * 2^-9, scaled by 2^9) -> fp16 conversions turn into code exactly, two
// per instruction.
template <int VB>
__device__ __forceinline__ half8 v_operand(const uint32_t* words, int mt) {
  if constexpr (VB == 2) {
    const uint32_t w = words[mt >> 1];
    const uint32_t m = ((mt & 1) ? (w >> 2) : w) & 0x33333333u;
    return __builtin_bit_cast(half8, u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 0)),
                                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 1)),
                                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 2)),
                                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 3))});
  } else {
    const uint32_t w = words[mt];
    const uint32_t m0 = w & 0x0F0F0F0Fu, m1 = (w >> 4) & 0x0F0F0F0Fu;
    return __builtin_bit_cast(half8, u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m0, 512.0f, false)),
                                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m0, 512.0f, true)),
                                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m1, 512.0f, false)),
                                           __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m1, 512.0f, true))});
  }
}

// Reductions over the four lane groups j of a column (lanes l16, l16 + 16,
// l16 + 32, l16 + 48), on the VALU with gfx950's lane swaps.
// max(a, b) as the median of (a, b, +inf): one v_med3_f32, with none of the
// input canonicalization fmaxf needs (+inf comes from an SGPR so the compiler
// does not turn the median back into fmaxf)
__device__ __forceinline__ float fmax2(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, __uint_as_float(sgpr_const(0x7f800000u)));
}
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
// A block of BYTES (a multiple of 4): 1 KiB copies, 256-byte copies, and for
// a remainder one 4-byte-per-lane copy issued by only the lanes it needs.
template <int BYTES>
__device__ __forceinline__ void dma_block(const uint8_t* g, uint32_t lane16, uint32_t lane4, uint32_t lds) {
  static_assert(BYTES % 4 == 0, "DMA blocks are whole dwords");
#pragma unroll
  for (int o = 0; o + 1024 <= BYTES; o += 1024) dma_1k(g + o, lane16, lds + o);
#pragma unroll
  for (int o = BYTES / 1024 * 1024; o + 256 <= BYTES; o += 256) dma_256(g + o, lane4, lds + o);
  if constexpr (BYTES % 256 != 0) {
    constexpr int o = BYTES / 256 * 256;
    if (lane4 < static_cast<uint32_t>(BYTES % 256)) dma_256(g + o, lane4, lds + o);
  }
}
template <int BYTES>
constexpr int dma_count() { return BYTES / 1024 + (BYTES % 1024) / 256 + (BYTES % 256 != 0 ? 1 : 0); }
// N copy instructions issued by lane 0 alone, 4 bytes each (global
// [g + 256 k, +4) to LDS [lds + 256 k, +4)): they stand in for N copies whose
// data is not needed, keeping the count of copy instructions (which the
// waits count; a copy counts once whatever lanes are active) at one memory
// line each instead of 256 bytes or 1 KiB.
template <int N>
__device__ __forceinline__ void dma_filler(const uint8_t* g, uint32_t lane4, uint32_t lds) {
  if (lane4 == 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) dma_256(g + 256 * k, 0u, lds + 256 * k);
  }
}
// Number of chunks among the NBUF - 1 issued after chunk position ch (mod
// CPG) that start a group, i.e. that also carry key parameters.
template <int NBUF, int CPG>
constexpr int kp_after(int ch) {
  int n = 0;
  for (int k = 1; k < NBUF; ++k) n += ((ch + k) % CPG) == 0;
  return n;
}
// Parameter buffers for n chunks in flight: while chunk c is processed the
// refill brings chunk c + n, so the groups of chunks c .. c + n are live,
// except that a group's last chunk has read its parameters before the refill.
template <int CPG>
constexpr int param_buffers(int n) { return CPG == 1 ? n : n / CPG + 1; }
// Chunks in flight per wave: as many as fit, with their parameter buffers, in
// BUDGET bytes of LDS.  The one-wave launches take 12800 bytes, so that
// twelve waves (three per SIMD) fit in a CU's 160 KiB: measured on gfx950,
// 13312 bytes per workgroup already cost a workgroup slot per CU (allocation
// is rounded up beyond the byte count).
constexpr int kRingBudget = 12800;
// LDS ring budget per wave of the workgroup-merged launch
constexpr int kFusedRingBudget = 12800;
template <int SLOT, int PB, int CPG, int BUDGET = kRingBudget>
constexpr int ring_depth() {
  int n = 2;
  while ((n + 1) * SLOT + param_buffers<CPG>(n + 1) * PB <= BUDGET) ++n;
  return n;
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Page geometry of one token group (the same numbers as make_layout's,
// as compile-time constants of the kernel instance).
template <int D, int KB, int VB, int G, bool TN>
struct PageShape {
  static constexpr int NCG = D / G, CPG = G / kChunk;
  static constexpr int KC = kChunk * D * KB / 8, VC = kChunk * D * VB / 8;
  static constexpr int VPB = (kChunk * NCG * 4 + 255) / 256 * 256, KPB = 4 * D, KNB = TN ? kChunk * 2 : 0;
  static constexpr int OFF_KC = 0, OFF_VC = CPG * KC, OFF_KP = OFF_VC + CPG * VC, OFF_VP = OFF_KP + KPB;
  static constexpr int OFF_KN = OFF_VP + CPG * VPB;
  static constexpr int BYTES = OFF_KN + CPG * KNB;
  // the group's parameter block [KP][VP per chunk][key norms per chunk]
  static constexpr int PB = KPB + CPG * VPB + CPG * KNB;
};

// LDS bytes of the chunk ring and parameter buffers of one page shape.
template <int D, int KB, int VB, int G, bool TN, int BUDGET = kRingBudget>
constexpr int ring_bytes() {
  using PS = PageShape<D, KB, VB, G, TN>;
  constexpr int SLOT = PS::KC + PS::VC;
  constexpr int n = ring_depth<SLOT, PS::PB, PS::CPG, BUDGET>();
  return n * SLOT + param_buffers<PS::CPG>(n) * PS::PB;
}

// Running-max slack of the online softmax (base-2 units): the accumulators
// are rescaled only when a chunk's maximum exceeds the running maximum by more
// than this, so weights stay <= 2^0.5 and the fp16 PV operand p * scale stays
// below 65504 for any scale of fp16 data.
constexpr float kMaxSlack = 0.5f;

// Lane i of each row of 16 receives lane (i + N) mod 16 (DPP row_ror:16-N).
template <int N>
__device__ __forceinline__ uint32_t row_from(uint32_t x) {
  static_assert(N > 0 && N < 16, "row rotation");
  return __builtin_amdgcn_update_dpp(0u, x, 0x120 + (16 - N), 0xf, 0xf, true);
}
template <int N>
__device__ __forceinline__ float row_from(float x) {
  return __uint_as_float(row_from<N>(__float_as_uint(x)));
}
// Max / sum over the R replicas of a head slot (lanes h, h + 16/R, ... of a row).
template <int R>
__device__ __forceinline__ float replica_max(float x) {
  if constexpr (R >= 2) x = fmax2(x, row_from<8>(x));
  if constexpr (R >= 4) x = fmax2(x, row_from<4>(x));
  return x;
}
template <int R>
__device__ __forceinline__ float replica_sum(float x) {
  if constexpr (R >= 2) x += row_from<8>(x);
  if constexpr (R >= 4) x += row_from<4>(x);
  return x;
}

// The token this step appends when its fp16 window write is left to the
// decode (kvq_append_decode_attn): the wave whose window chunks include its
// position first stages its key and value rows in its LDS ring (free once the
// ring's copies are done), as fp16 rounded to nearest even from binary32 like
// the window write does: lane l converts elements 2l and 2l + 1 of each row
// (rows of new_k / new_v are [B][H_kv][1][D]).  In that chunk the lanes whose
// key or value elements belong to the token then take them from LDS instead
// of the cache (take_new_keys, take_new_value), and after the window pass
// the same lanes store them to the window (put_new_token): no store comes
// between the pass's loads, which therefore all go out at once.
template <int D>
__device__ __forceinline__ void stage_new_token(const NewToken& nt, int in_dtype, int64_t slice, uint8_t* ring) {
  const int l = threadIdx.x & (kLanes - 1);
  if (2 * l < D) {
    const int64_t i = slice * D + 2 * l;
    uint32_t kh, vh;
    if (in_dtype == 0) {
      const float* k = static_cast<const float*>(nt.k) + i;
      const float* v = static_cast<const float*>(nt.v) + i;
      kh = pack_h2(k[0], k[1]);
      vh = pack_h2(v[0], v[1]);
    } else {
      const uint32_t kw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(nt.k) + i);
      const uint32_t vw = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(nt.v) + i);
      kh = in_dtype == 1 ? kw : pack_h2(__uint_as_float(kw << 16), __uint_as_float(kw & 0xffff0000u));
      vh = in_dtype == 1 ? vw : pack_h2(__uint_as_float(vw << 16), __uint_as_float(vw & 0xffff0000u));
    }
    *reinterpret_cast<uint32_t*>(ring + 4 * l) = kh;
    *reinterpret_cast<uint32_t*>(ring + 2 * D + 4 * l) = vh;
  }
}
// Keys: the lanes of token column t % 16 hold channels 32 kb + 8 j .. + 7 of
// tile t / 16 in one 16-byte operand.
template <int D>
__device__ __forceinline__ void take_new_keys(const uint8_t* staged, int t, int l, int kb, u32x4& k0, u32x4& k1) {
  const int tile = t >> 4, j = l >> 4;
  const u32x4 w = *reinterpret_cast<const u32x4*>(staged + 2 * (32 * kb + 8 * j));
  if (tile == 0) k0 = w; else k1 = w;
}
// Values: lane group j with tau(j, e) = t holds element e of channel
// 16 mt + l % 16 in operand mt.
template <int D>
__device__ __forceinline__ void take_new_value(const uint8_t* staged, int e, int l, int mt, u32x4& vw) {
  const uint32_t h = *reinterpret_cast<const uint16_t*>(staged + 2 * D + 2 * (16 * mt + (l & 15)));
  const int hi = e & 1, dw = e >> 1;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (k == dw) vw[k] = hi ? ((vw[k] & 0xffffu) | (h << 16)) : ((vw[k] & 0xffff0000u) | h);
}
// The token's window slots from the staged rows: key token t (tile t / 16)
// by the four lanes of column t % 16 (16 bytes per kb each), value element e
// of every channel by the lanes of group jv with tau(jv, e) = t.
template <int D>
__device__ __forceinline__ void put_new_token(const uint8_t* staged, uint8_t* rch, int t, int l, int jv, int e) {
  constexpr int NKB = D / 32, NMT = D / 16;
  const int tile = t >> 4, j = l >> 4;
  if ((l & 15) == (t & 15)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      *reinterpret_cast<u32x4*>(rch + ((tile * NKB + kb) * kLanes + l) * 16) =
          *reinterpret_cast<const u32x4*>(staged + 2 * (32 * kb + 8 * j));
  }
  if (j == jv) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      *reinterpret_cast<uint16_t*>(rch + kChunk * D * 2 + (mt * kLanes + l) * 16 + 2 * e) =
          *reinterpret_cast<const uint16_t*>(staged + 2 * D + 2 * (16 * mt + (l & 15)));
  }
}

// Column layout.  Lane l holds MFMA column l16 = l % 16 and lane group
// j = l / 16.  The gqa query heads of the slice take head slots 0..GQC-1
// (GQC = 4 for gqa <= 4, 8 for gqa = 8, 16 for gqa = 16); the 16 columns hold
// R = 16 / GQC replicas of them (column l16 = head slot l16 % GQC, replica
// rp = l16 / GQC).  The query side of QK^T carries two fp16 parts: with
// GQC < 16, odd replicas hold the second part in their columns, so one MFMA
// produces both and a DPP add with the column GQC places away gives every
// lane the full score; with GQC = 16 the parts take two MFMAs.  Each replica
// then keeps only NV = 8 / R of the 8 scores a lane holds (tokens tau(j, e),
// e in [NV rp, NV rp + NV)), so the softmax, the PV weights and the
// zero-point sums cost NV values per lane instead of 8.  Replica 0 gathers
// the PV weights of the other replicas by DPP row rotation and owns the
// output; the other replicas' PV columns are never read.
//
// GQC = 1 (one query head per kv head, multi-head attention): the query head
// takes all four head slots of the GQC = 4 layout, so every column carries a
// live score, and head slot h serves value group h % NCG: its lanes form the
// PV weights and zero-point sums of that group only, the PV B operand is the
// same for every M-tile, and the output of a tile is read from the column of
// its group's slot.  Per chunk a lane then forms one group's weights instead
// of NCG (for D = 128, G = 32 a quarter of the weight, zero-sum and gather
// work), where the four-slot layout with one live slot left three quarters
// of the lanes computing a softmax nobody read.
//
// decode_split is one wave's work: split s of slice `slice`, with the LDS
// ring at `ring` (ring_bytes<...>() bytes) and, for rotated keys, gqa * D
// floats at qsh for the query's transform, shared by the workgroup's waves
// (all of them work on the same slice).  With FUSED the split's (o, m, l)
// goes to the start of its ring instead of global memory, for the
// workgroup's own merge (decode_fused_kernel).  NEWTOK: the window pass takes
// a deferred appended token from the step's input (DecodeArgs::new_pos); the
// mixed-width kernel, whose caches never defer it, is built without it.
template <int D, int KB, int VB, int G, int GQC, bool TN, bool FUSED = false, bool NEWTOK = true>
__device__ __forceinline__ void decode_split(const DecodeArgs& a, const int64_t slice, const int s, uint8_t* ring,
                                             float* qsh, const NewToken& nt) {
  using PS = PageShape<D, KB, VB, G, TN>;
  constexpr int NKB = D / 32, NMT = D / 16, NCG = PS::NCG, CPG = PS::CPG;
  constexpr int KW = 2 * NKB * KB / 4, VW = NMT * VB / 4;
  static_assert(GQC == 1 || GQC == 4 || GQC == 8 || GQC == 16, "head slots per replica");
  constexpr bool MHA = GQC == 1;                          // one query head in every slot
  constexpr int GS = MHA ? 4 : GQC;                       // head slots
  constexpr int R = 16 / GS, NV = 8 / R, NPR = NV / 2;    // replicas, values and value pairs per lane
  constexpr int NCGL = MHA ? 1 : NCG;                     // value groups a lane forms weights for
  constexpr int VPL = NV * NCGL;                          // value-parameter dwords a lane reads per chunk
  static_assert(!MHA || NCG <= GS, "a value group per head slot");
  // B operands of QK^T carry each value as two fp16 parts (hi + lo) so the
  // folded products keep ~22 bits: in the columns of odd replicas (NP = 1
  // MFMA) when GS < 16, else as two MFMAs.
  constexpr int NP = GS < 16 ? 1 : 2;
  const Layout& L = a.L;
  const int l = threadIdx.x & (kLanes - 1), l16 = l & 15, j = l >> 4;
  const int S = a.splits;
  const int b = static_cast<int>(slice / a.Hkv), hkv = static_cast<int>(slice % a.Hkv);
  const int h = l16 % GS, rp = l16 / GS;
  // hv: the slot carries a query head (all slots with MHA, whose head is 0)
  const bool hv = MHA || h < a.gqa;
  const int hh = MHA ? 0 : (hv ? h : 0);                  // the slot's query head within the slice
  const int hq = hkv * a.gqa + hh;
  // MHA: the value group of this slot, and whether it writes that group's tiles
  const int cgh = h % NCG;
  const bool owner = !MHA || h < NCG;

  const bool lo_cols = NP == 1 && (rp & 1);               // this lane's columns hold the second part
  // full QK^T sum from the two parts' columns
  auto combine = [&](float x) __attribute__((always_inline)) {
    if constexpr (NP == 1) {
      return x + row_from<GS>(x);
    } else {
      return x;
    }
  };

  // ---- query: lane owns channels 32 kb + 8 j + e of head h, times log2(e)/sqrt(D)
  float qm[NKB][8];
  const float qscale = kLog2e * (D == 128 ? 0.08838834764831845f : 0.125f);
  if (a.rotate) {
    // every element and butterfly once per workgroup, spread over its threads
    const int64_t base = (static_cast<int64_t>(b) * a.Hq + hkv * a.gqa) * D;
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int idx = tid; idx < a.gqa * D; idx += nth) qsh[idx] = load_q(a.q, a.in_dtype, base + idx);
    __syncthreads();
    for (int hh = 1; hh < D; hh <<= 1) {
      for (int k = tid; k < a.gqa * (D / 2); k += nth) {
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
        qm[kb][e] = hv ? qsh[hh * D + 32 * kb + 8 * j + e] * rs : 0.0f;
  } else {
    // the lane's 8 channels of each kb are contiguous: one 16-byte load for
    // 2-byte inputs, two for f32 (rows are 16-byte aligned: D is 64 or 128);
    // every load of the lane is issued before the first conversion, so the
    // query costs one memory latency (with the dtype tested per kb, each kb's
    // load waited for the previous one)
    const int64_t base = (static_cast<int64_t>(b) * a.Hq + hq) * D + 8 * j;
    if (a.in_dtype == 0) {
      u32x4 x[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        x[kb][0] = *reinterpret_cast<const u32x4*>(static_cast<const float*>(a.q) + base + 32 * kb);
        x[kb][1] = *reinterpret_cast<const u32x4*>(static_cast<const float*>(a.q) + base + 32 * kb + 4);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) qm[kb][e] = hv ? __uint_as_float(x[kb][e >> 2][e & 3]) * qscale : 0.0f;
    } else {
      u32x4 w[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        w[kb] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + base + 32 * kb);
      const bool f16 = a.in_dtype == 1;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t u = (w[kb][e >> 1] >> (16 * (e & 1))) & 0xffffu;
          const float x = f16 ? __half2float(__ushort_as_half(static_cast<uint16_t>(u))) : __uint_as_float(u << 16);
          qm[kb][e] = hv ? x * qscale : 0.0f;
        }
    }
  }
  // Per-split fp16 parts of the query (part 1 = fp16(x - part 0)):
  //   qz: q itself, the B operand of the key zero-point bias and of the window;
  //   qh / ql: q / mult (the code multipliers of the key operand), from which
  //   the per-group B operand q * scale / mult is formed by exact-residual fp16
  //   products.  With NP = 1, qz and ql hold this lane's own part (ql = part 0
  //   in first-part columns) and qh is zero in first-part columns, so the same
  //   three instructions produce either part: x = qh s, y = qh s - x (exact),
  //   part = fp16(ql s + y).
  //   With key token norms the keys' scales are at most 1 (normalized rows lie
  //   in [-1, 1]) and often far below it, so q * scale / mult would sit in
  //   the fp16 subnormals with few bits left; q / mult is then scaled by 2^E,
  //   E per split such that max |q| 2^E < 2^14, and the scores by 2^(24 - E)
  //   instead of 2^24 (exact powers of two).
  float qup = 1.0f, kscale = kTwo24;
  if constexpr (TN) {
    float mx = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qm[kb][e]));
    // over the wave: the 16 columns of each row, then the four rows
    mx = fmax2(mx, row_from<8>(mx));
    mx = fmax2(mx, row_from<4>(mx));
    mx = fmax2(mx, row_from<2>(mx));
    mx = fmax2(mx, row_from<1>(mx));
    mx = wave_max_j(mx);
    const int E = mx > 0.0f ? min(40, max(-24, 14 - __builtin_amdgcn_frexp_expf(mx))) : 40;
    qup = __builtin_ldexpf(1.0f, E);
    kscale = __builtin_ldexpf(kTwo24, -E);
  }
  uint32_t qz[NP][NKB][4], qh[NKB][4], ql[NKB][4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = qm[kb][2 * i], x1 = qm[kb][2 * i + 1];
      const float h0 = static_cast<float>(static_cast<_Float16>(x0)), h1 = static_cast<float>(static_cast<_Float16>(x1));
      const uint32_t z_hi = pack_h2(x0, x1), z_lo = pack_h2(x0 - h0, x1 - h1);
      const float d0 = (x0 * qup) * (1.0f / code_mult<KB>(2 * i)), d1 = (x1 * qup) * (1.0f / code_mult<KB>(2 * i + 1));
      const float e0 = static_cast<float>(static_cast<_Float16>(d0)), e1 = static_cast<float>(static_cast<_Float16>(d1));
      const uint32_t d_hi = pack_h2(d0, d1), d_lo = pack_h2(d0 - e0, d1 - e1);
      if constexpr (NP == 1) {
        qz[0][kb][i] = lo_cols ? z_lo : z_hi;
        ql[kb][i] = lo_cols ? d_lo : d_hi;
        qh[kb][i] = lo_cols ? d_hi : 0u;
      } else {
        qz[0][kb][i] = z_hi;
        qz[NP - 1][kb][i] = z_lo;
        ql[kb][i] = d_lo;
        qh[kb][i] = d_hi;
      }
    }

  const CodeMasks<KB> uk;

  // Online-softmax state (per head, uniform over replicas and j).  m is the
  // running max in log2 units; acc holds the PV sums (the value codes enter
  // as normal-range fp16 values, the weights as fp16 p * s).  lsum and zacc
  // are this lane's share (its value slots).
  float m = -INFINITY, mslack = -INFINITY, lsum = 0.0f;
  f32x4 acc[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // zero-point sums per value group, weighted by p (MHA: this slot's group)
  float zacc[NCGL];
#pragma unroll
  for (int i = 0; i < NCGL; ++i) zacc[i] = 0.0f;

  // (called wave-uniformly; mnew = max(m, chunk max) per head)
  auto rescale = [&](float mnew) __attribute__((always_inline)) {
    const float al = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
    for (int i = 0; i < NMT; ++i) acc[i] *= al;
#pragma unroll
    for (int i = 0; i < NCGL; ++i) zacc[i] *= al;
    lsum *= al;
    m = mnew;
    mslack = mnew + kMaxSlack;
  };
  // this lane's NV scores out of the 8 it holds (tokens tau(j, e), e = NV rp + k)
  auto own_values = [&](const float (&t)[8], float (&u)[NV]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < NV; ++k) u[k] = t[k];
#pragma unroll
    for (int r = 1; r < R; ++r)
#pragma unroll
      for (int k = 0; k < NV; ++k) u[k] = rp == r ? t[NV * r + k] : u[k];
  };
  // PV B operand of replica 0 from the replicas' value pairs: pair i sits in
  // replica i / NPR, slot i % NPR
  auto gather_pairs = [&](const uint32_t (&c)[NPR], uint32_t (&o)[4]) __attribute__((always_inline)) {
    static_for<0, 4>([&](auto ic) {
      constexpr int i = decltype(ic)::value, r = i / NPR;
      if constexpr (r == 0) {
        o[i] = c[i % NPR];
      } else {
        o[i] = row_from<GS * r>(c[i % NPR]);
      }
    });
  };

  const int g0 = static_cast<int>(a.g_base) + s * static_cast<int>(a.groups_per_split);
  const int g1 = min(g0 + static_cast<int>(a.groups_per_split), static_cast<int>(a.g_base + a.ngroups));

  // ---- LDS: a ring of NBUF chunk slots [key codes][value codes], and NPB
  // parameter buffers, each one group's block [key scale/zero rows][value
  // params per chunk], copied with the group's first chunk
  constexpr int KC = PS::KC, VC = PS::VC, VPB = PS::VPB, KPB = PS::KPB, PB = PS::PB;
  constexpr int SLOT = KC + VC;
  // NBUF chunks are in flight; a group's parameters stay until its last chunk
  // has read them, and the refill that reuses a buffer comes after that read.
  constexpr int BUDGET = FUSED ? kFusedRingBudget : kRingBudget;
  constexpr int NBUF = ring_depth<SLOT, PB, CPG, BUDGET>(), NPB = param_buffers<CPG>(NBUF);
  constexpr int NBASE = dma_count<KC>() + dma_count<VC>(), NKP = dma_count<PB>();
  static_assert(NBUF * SLOT + NPB * PB == ring_bytes<D, KB, VB, G, TN, BUDGET>(), "ring size");
  const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((KVQ_AS3 uint8_t*)ring));
  const uint32_t pbuf_lds = ring_lds + NBUF * SLOT;
  const uint32_t lane16 = static_cast<uint32_t>(l) * 16, lane4 = static_cast<uint32_t>(l) * 4;
  // byte offset of this lane's value parameters inside a chunk's part of the
  // parameter block (layout [j][pair][group][scale, zero] dwords, see kvq_layout.h)
  // (MHA: the NPR = 1 pair's scale and zero of group cgh only)
  const int vp_off = KPB + ((j * 4 + NPR * rp) * NCG + (MHA ? cgh : 0)) * 8;

  if (g1 > g0) {
    const uint8_t* slice_pages = a.cache + page_offset(L, slice, 0);

    // copy position chi of group gi into the slot at LDS address sl; a group's
    // first chunk also brings the group's parameter block into buffer gi % NPB
    auto pbuf_of = [&](int gi) __attribute__((always_inline)) {
      return pbuf_lds + static_cast<uint32_t>((gi - g0) % NPB) * PB;
    };
    // Copies for positions past the split's end keep the per-chunk copy count
    // fixed (the waits count copies): the same number of copy instructions,
    // each 4 bytes from one lane: their code part from the split's last page
    // into a slot nobody reads, their parameter part from the split's last
    // group's parameter block into that group's own buffer (identical bytes
    // at the same offsets).
    auto issue = [&](int gi, auto chi_c, uint32_t sl) __attribute__((always_inline)) {
      constexpr int chi = decltype(chi_c)::value;
      const bool real = gi < g1;
      const int gp = real ? gi : g1 - 1;
      const uint8_t* page = slice_pages + static_cast<int64_t>(gp) * L.page_bytes;  // page slots (>= PS::BYTES)
      lds_reads_done();
      if (real) {
        dma_block<KC>(page + PS::OFF_KC + chi * KC, lane16, lane4, sl);
        dma_block<VC>(page + PS::OFF_VC + chi * VC, lane16, lane4, sl + KC);
      } else {
        dma_filler<dma_count<KC>() + dma_count<VC>()>(page, lane4, sl);
      }
      if constexpr (chi == 0) {
        if (real) {
          dma_block<PB>(page + PS::OFF_KP, lane16, lane4, pbuf_of(gp));
        } else {
          dma_filler<dma_count<PB>()>(page + PS::OFF_KP, lane4, pbuf_of(gp));
        }
      }
    };

    uint32_t bq[NP][NKB][4];  // B operand of QK^T (fp16 pairs), per part
    float cb = 0.0f;          // this group's zero-point score bias (log2 units)
    // exponent offset: exp2(score + bias - m) is the softmax weight p
    float bmc;
    // (with key token norms the bias is inside each score, so it is left out)
    auto set_bmc = [&]() __attribute__((always_inline)) { bmc = (TN ? 0.0f : cb) - m; };

    auto process = [&](const uint8_t* sl, const uint8_t* pbk, int ch, auto&& refill) __attribute__((always_inline)) {
      if (ch == 0) {
        // B operand from this group's key scales: q * s / mult in two parts
        // (exact-residual fp16 products), and the bias sum_c q_c z_c by MFMA
        // (every row of the bias tile is the same sum)
        const u32x4* ps = reinterpret_cast<const u32x4*>(pbk) + j * NKB;
        const u32x4* pz = reinterpret_cast<const u32x4*>(pbk + 2 * D) + j * NKB;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4 sw = ps[kb];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const half2v sv = as_h2(sw[i]), hh = as_h2(qh[kb][i]);
            const half2v x = pk_mul(hh, sv);
            const half2v y = pk_fma(hh, sv, -x);  // exact: hh * sv - x
            if constexpr (NP == 1) {
              bq[0][kb][i] = as_u32(pk_fma(as_h2(ql[kb][i]), sv, y));
            } else {
              bq[0][kb][i] = as_u32(x);
              bq[1][kb][i] = as_u32(pk_fma(as_h2(ql[kb][i]), sv, y));
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
        cb = combine(cbt[0]);
        set_bmc();
      }
      uint32_t kw[KW], vw[VW], vp[VPL], kn[TN ? NPR : 1];
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
      if constexpr (VPL % 4 == 0) {
#pragma unroll
        for (int v = 0; v < VPL / 4; ++v) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(pbk + ch * VPB + vp_off + 16 * v);
          vp[4 * v] = x[0]; vp[4 * v + 1] = x[1]; vp[4 * v + 2] = x[2]; vp[4 * v + 3] = x[3];
        }
      } else {
        const u32x2 x = *reinterpret_cast<const u32x2*>(pbk + ch * VPB + vp_off);
        vp[0] = x[0]; vp[1] = x[1];
      }
      if constexpr (TN) {
        // this lane's token norms: fp16 pairs of its token pairs
        const uint8_t* knp = pbk + KPB + CPG * VPB + ch * PS::KNB + (j * 4 + NPR * rp) * 4;
        if constexpr (NPR == 4) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(knp);
          kn[0] = x[0]; kn[1] = x[1]; kn[2] = x[2]; kn[3] = x[3];
        } else if constexpr (NPR == 2) {
          const u32x2 x = *reinterpret_cast<const u32x2*>(knp);
          kn[0] = x[0]; kn[1] = x[1];
        } else {
          kn[0] = *reinterpret_cast<const uint32_t*>(knp);
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
        t[r] = combine(c0[r]);
        t[4 + r] = combine(c1[r]);
      }
      float u[NV];
      own_values(t, u);
      // online softmax over the head's 32 chunk scores (NV per lane): a lane
      // whose own maximum passes the head's slack bound calls for a rescale;
      // only then is the per-head maximum reduced over replicas and lane groups
      // with key token norms each score is norm * (q . khat_normalized)
      float sc[NV];
      if constexpr (TN) {
#pragma unroll
        for (int k = 0; k < NV; ++k)
          sc[k] = __builtin_fmaf(u[k], kscale, cb) * ((k & 1) ? h2f_hi(kn[k >> 1]) : h2f_lo(kn[k >> 1]));
      }
      float tmax = TN ? sc[0] : u[0];
#pragma unroll
      for (int k = 1; k < NV; ++k) tmax = fmax2(tmax, TN ? sc[k] : u[k]);
      const float lmax = TN ? tmax : __builtin_fmaf(tmax, kTwo24, cb);
      if (__builtin_amdgcn_ballot_w64(lmax > mslack)) {
        rescale(fmax2(m, wave_max_j(replica_max<R>(lmax))));
        set_bmc();
      }
      // softmax weights p
      float pm[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        pm[k] = __builtin_amdgcn_exp2f(TN ? sc[k] + bmc : __builtin_fmaf(u[k], kTwo24, bmc));
        lsum += pm[k];
      }
      // PV weights p * value scale (one fp16 part) and the zero-point sums
      uint32_t bpc[NCGL][NPR];
#pragma unroll
      for (int cg = 0; cg < NCGL; ++cg) {
#pragma unroll
        for (int pp = 0; pp < NPR; ++pp) {
          const uint32_t sp = vp[(pp * NCGL + cg) * 2], zp = vp[(pp * NCGL + cg) * 2 + 1];
          bpc[cg][pp] = mix_mul2(pm[2 * pp], pm[2 * pp + 1], sp);
          zacc[cg] = __builtin_fmaf(pm[2 * pp], h2f_lo(zp), zacc[cg]);
          zacc[cg] = __builtin_fmaf(pm[2 * pp + 1], h2f_hi(zp), zacc[cg]);
        }
      }
      // the slot's data has long been read into registers: refill it with a
      // later chunk before the PV products
      refill();
      uint32_t bp[NCGL][4];
#pragma unroll
      for (int cg = 0; cg < NCGL; ++cg) gather_pairs(bpc[cg], bp[cg]);
      // PV on the normal-range code operands
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const half8 av = v_operand<VB>(vw, mt);
        const uint32_t* bw = bp[MHA ? 0 : (16 * mt) / G];
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
    // prologue: NBUF chunks in flight (split boundaries are group-aligned)
    static_for<0, NBUF>([&](auto k) {
      constexpr int K = decltype(k)::value;
      issue(g0 + K / CPG, std::integral_constant<int, K % CPG>{}, ring_lds + K * SLOT);
    });
    for (int g = g0; g < g1; ++g) {
      static_for<0, CPG>([&](auto chc) {
        constexpr int ch = decltype(chc)::value;
        constexpr int ahead = ch + NBUF;
        // copies issued after chunk c's: chunks c+1 .. c+NBUF-1, NBASE each,
        // plus NKP for each of them that starts a group
        wait_vmcnt<(NBUF - 1) * NBASE + kp_after<NBUF, CPG>(ch) * NKP>();
        const uint32_t sl = sl_proc;
        process(ring + (sl - ring_lds), ring + (pbuf_of(g) - ring_lds), ch, [&]() __attribute__((always_inline)) {
          issue(g + ahead / CPG, std::integral_constant<int, ahead % CPG>{}, sl);
        });
        sl_proc = next_slot(sl_proc);
      });
    }
    wait_vmcnt<0>();  // no copy into LDS outlives the loop
  }
  // ---- fp16 chunks (the attention-sink chunks, then the recent window's),
  // spread over the splits (split s takes chunks S - 1 - s, 2S - 1 - s, ...)
  // so that no wave adds more than its share of these latency-bound reads to
  // the end of the kernel
  {
    const int64_t nfc = a.do_fp16 ? a.nsc + (a.rc1 - a.rc0) : 0;
    // the deferred appended token, when one of this split's window chunks
    // holds it: staged in the ring (its copies are done: the loop above ends
    // with none in flight)
    int64_t new_rc = -1;
    if constexpr (NEWTOK) {
      if (nt.pos >= 0) {
        const int64_t fcn = a.nsc + (nt.pos / kChunk - a.rc0), f0 = S - 1 - s;
        if (fcn >= f0 && fcn < nfc && (fcn - f0) % S == 0) {
          new_rc = nt.pos / kChunk;
          stage_new_token<D>(nt, a.in_dtype, slice, ring);
        }
      }
    }
    for (int64_t fc = S - 1 - s; fc < nfc; fc += S) {
      const int64_t rc = fc < a.nsc ? fc : a.rc0 + (fc - a.nsc);  // absolute chunk index
      uint8_t* rch = a.cache + fp16_chunk_offset(L, slice, rc * kChunk);
      const int64_t pos0 = rc * kChunk;
      // the step's appended token, when its window write was left to the
      // decode and it falls in this chunk: token tn of the chunk
      const int tn = NEWTOK && rc == new_rc ? static_cast<int>(nt.pos - pos0) : -1;
      const bool new_keys = tn >= 0 && l16 == (tn & 15);
      // every load of the chunk first (keys, then values): one memory latency
      u32x4 kq[2][NKB], vq[NMT];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        kq[0][kb] = *reinterpret_cast<const u32x4*>(rch + ((0 * NKB + kb) * kLanes + l) * 16);
        kq[1][kb] = *reinterpret_cast<const u32x4*>(rch + ((1 * NKB + kb) * kLanes + l) * 16);
      }
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
        vq[mt] = *reinterpret_cast<const u32x4*>(rch + kChunk * D * 2 + (mt * kLanes + l) * 16);
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        u32x4 k0 = kq[0][kb], k1 = kq[1][kb];
        if (new_keys) take_new_keys<D>(ring, tn, l, kb, k0, k1);
        const half8 a0 = __builtin_bit_cast(half8, k0);
        const half8 a1 = __builtin_bit_cast(half8, k1);
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          const half8 bb = __builtin_bit_cast(half8, u32x4{qz[pp][kb][0], qz[pp][kb][1], qz[pp][kb][2], qz[pp][kb][3]});
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bb, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bb, c1, 0, 0, 0);
        }
      }
      const bool partial = pos0 + kChunk > a.n;
      float sc[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[r] = combine(c0[r]);
        sc[4 + r] = combine(c1[r]);
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
      float u[NV];
      own_values(sc, u);
      float lmax = u[0];
#pragma unroll
      for (int k = 1; k < NV; ++k) lmax = fmax2(lmax, u[k]);
      if (__builtin_amdgcn_ballot_w64(lmax > mslack)) rescale(fmax2(m, wave_max_j(replica_max<R>(lmax))));
      float p[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        p[k] = __builtin_amdgcn_exp2f(u[k] - m);
        lsum += p[k];
      }
      // two-part fp16 weights (the window's values are fp16 data, no scales)
      uint32_t ph[NPR], pl[NPR];
#pragma unroll
      for (int pp = 0; pp < NPR; ++pp) {
        const uint32_t one = 0x3C003C00u;  // fp16 1.0 pair
        ph[pp] = mix_mul2(p[2 * pp], p[2 * pp + 1], one);
        pl[pp] = mix_fms2(p[2 * pp], p[2 * pp + 1], one, ph[pp]);
      }
      uint32_t bpr[2][4];
      gather_pairs(ph, bpr[0]);
      gather_pairs(pl, bpr[1]);
      int jv = -1, ev = 0;
      if (tn >= 0) tau_inv(tn, &jv, &ev);
      const bool new_values = j == jv;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        u32x4 vwd = vq[mt];
        if (new_values) take_new_value<D>(ring, ev, l, mt, vwd);
        vwd[0] &= vmask[0]; vwd[1] &= vmask[1]; vwd[2] &= vmask[2]; vwd[3] &= vmask[3];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const half8 bb = __builtin_bit_cast(half8, u32x4{bpr[pp][0], bpr[pp][1], bpr[pp][2], bpr[pp][3]});
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, vwd), bb, acc[mt], 0, 0, 0);
        }
      }
    }
    // the appended token's window slots, after every load of the pass (and
    // before a workgroup record overwrites the staged rows)
    if (NEWTOK && new_rc >= 0) {
      const int tn = static_cast<int>(nt.pos - new_rc * kChunk);
      int jv = -1, ev = 0;
      tau_inv(tn, &jv, &ev);
      put_new_token<D>(ring, a.cache + fp16_chunk_offset(L, slice, new_rc * kChunk), tn, l, jv, ev);
    }
  }

  // ---- finalize: reduce the lane shares over replicas and lane groups, write
  lsum = wave_sum_j(replica_sum<R>(lsum));
  float zsum[NCGL];
#pragma unroll
  for (int i = 0; i < NCGL; ++i) zsum[i] = wave_sum_j(replica_sum<R>(zacc[i]));
  // tile mt's output: o = acc + the zero-point sum of its value group, held by
  // this lane (MHA: only the lanes of the group's slot hold the tile's column)
  auto tile_mine = [&](int mt) __attribute__((always_inline)) { return !MHA || (16 * mt) / G == cgh; };
  auto tile_o = [&](int mt) __attribute__((always_inline)) { return acc[mt] + zsum[MHA ? 0 : (16 * mt) / G]; };
  const bool ml_writer = j == 0 && (!MHA || h == 0);  // one lane per head writes m and l
  if constexpr (FUSED) {
    // record [head slot h][D + 4] floats: o, then m and l (the ring's copies
    // have all landed: the main loop ends with no copy in flight)
    if (hv && owner && rp == 0) {
      float* pr = reinterpret_cast<float*>(ring) + hh * (D + 4);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int c0 = 16 * mt + 4 * j;
        if (tile_mine(mt)) *reinterpret_cast<f32x4*>(pr + c0) = tile_o(mt);
      }
      if (ml_writer) {
        pr[D] = m;
        pr[D + 1] = lsum;
      }
    }
    return;
  }
  if (hv && owner && rp == 0) {
    const int64_t row = static_cast<int64_t>(b) * a.Hq + hq;
    if (a.write_final) {
      const float inv = 1.0f / lsum;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int c0 = 16 * mt + 4 * j;
        if (tile_mine(mt)) *reinterpret_cast<f32x4*>(a.out + row * D + c0) = tile_o(mt) * inv;
      }
    } else {
      float* pr = a.partial + (row * a.splits_total + a.split_off + s) * (D + 4);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int c0 = 16 * mt + 4 * j;
        if (tile_mine(mt)) *reinterpret_cast<f32x4*>(pr + c0) = tile_o(mt);
      }
      if (ml_writer) {
        pr[D] = m;
        pr[D + 1] = lsum;
      }
    }
  }
}

template <int D, int KB, int VB, int G, int GQC, bool TN>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(GQC < 16 ? 3 : 2)))
void decode_kernel(DecodeArgs a, NewToken nt) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[ring_bytes<D, KB, VB, G, TN>()];
  extern __shared__ float qsh[];  // gqa * D floats for rotated keys, sized at launch
  decode_split<D, KB, VB, G, GQC, TN>(a, blockIdx.x / a.splits, static_cast<int>(blockIdx.x % a.splits), ring, qsh, nt);
}

// ---- splits merged inside the workgroup --------------------------------------
// A slice's splits run in groups of W = 4 or 8 as the waves of one workgroup
// (workgroup gi of the slice, wave w = split W gi + w), each streaming its
// range through its own LDS ring; after one barrier the workgroup merges its
// W splits' (o, m, l) records from LDS with the log-sum-exp combination of
// the merge kernel.  With one group per slice it writes the output, so the
// partials never go to memory and no merge launch follows; with NG = S / W
// groups it writes the group's merged record (o relative to the group's
// maximum, that maximum, l) to partial slot gi of NG, for the merge kernel.
// The dynamic LDS holds W regions of fused_region_bytes (ring, then the
// split's record at its start) and the rotated query's gqa * D floats after
// them.
template <int D, int KB, int VB, int G, int GQC, bool TN>
constexpr int fused_region_bytes() {
  constexpr int rb = ring_bytes<D, KB, VB, G, TN, kFusedRingBudget>(), rec = GQC * (D + 4) * 4;
  return ((rb > rec ? rb : rec) + 15) / 16 * 16;
}

template <int D, int KB, int VB, int G, int GQC, bool TN>
__global__ __launch_bounds__(kLanes * kMaxFusedSplits) __attribute__((amdgpu_waves_per_eu(GQC < 16 ? 3 : 2)))
void decode_fused_kernel(DecodeArgs a, NewToken nt) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int RW = fused_region_bytes<D, KB, VB, G, GQC, TN>(), Q = D / 4, RS = D + 4;
  const int W = static_cast<int>(blockDim.x) / kLanes, NG = a.splits / W;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kLanes);
  float* qsh = reinterpret_cast<float*>(lds + W * RW);
  const int64_t slice = blockIdx.x / NG;
  const int gi = static_cast<int>(blockIdx.x % NG);
  decode_split<D, KB, VB, G, GQC, TN, true>(a, slice, gi * W + w, lds + w * RW, qsh, nt);
  __syncthreads();
  // thread t: channels 4q .. 4q + 3 of head slot hh; M = max_s m_s,
  // out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, and a split with no
  // tokens (m = -inf) contributes nothing (its o is never read)
  const int b = static_cast<int>(slice / a.Hkv), hkv = static_cast<int>(slice % a.Hkv);
  for (int t = threadIdx.x; t < a.gqa * Q; t += blockDim.x) {
    const int hh = t / Q, q = t % Q;
    float M = -INFINITY;
    for (int sp = 0; sp < W; ++sp) M = fmaxf(M, reinterpret_cast<const float*>(lds + sp * RW)[hh * RS + D]);
    float L = 0.0f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < W; ++sp) {
      const float* pr = reinterpret_cast<const float*>(lds + sp * RW) + hh * RS;
      const float ms = pr[D];
      if (ms != -INFINITY) {
        const float ws = __builtin_amdgcn_exp2f(ms - M);
        L += ws * pr[D + 1];
        acc += ws * *reinterpret_cast<const f32x4*>(pr + 4 * q);
      }
    }
    const int64_t row = static_cast<int64_t>(b) * a.Hq + hkv * a.gqa + hh;
    if (NG == 1) {
      *reinterpret_cast<f32x4*>(a.out + row * D + 4 * q) = acc / L;
    } else {
      float* pr = a.partial + (row * NG + gi) * RS;
      *reinterpret_cast<f32x4*>(pr + 4 * q) = acc;
      if (q == 0) {
        pr[D] = M;
        pr[D + 1] = L;
      }
    }
  }
}

// Groups of several bit widths in one launch: each block looks up its piece
// (a range of groups of one width, see MixedPlan) and runs that width's body
// over it; the LDS ring is sized for the widest body.
template <int D, int G>
constexpr int mixed_ring_bytes() {
  constexpr int a = ring_bytes<D, 2, 2, G, false>(), b = ring_bytes<D, 2, 4, G, false>();
  constexpr int c = ring_bytes<D, 4, 2, G, false>(), d = ring_bytes<D, 4, 4, G, false>();
  constexpr int e = ring_bytes<D, 2, 2, G, true>(), f = ring_bytes<D, 2, 4, G, true>();
  constexpr int g = ring_bytes<D, 4, 2, G, true>(), h = ring_bytes<D, 4, 4, G, true>();
  constexpr int m1 = a > b ? a : b, m2 = c > d ? c : d, m3 = e > f ? e : f, m4 = g > h ? g : h;
  constexpr int m5 = m1 > m2 ? m1 : m2, m6 = m3 > m4 ? m3 : m4;
  return m5 > m6 ? m5 : m6;
}

template <int D, int G, int GQC, bool TN>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(GQC < 16 ? 3 : 2)))
void decode_mixed_kernel(DecodeArgs a, MixedPlan mp) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[mixed_ring_bytes<D, G>()];
  extern __shared__ float qsh[];  // gqa * D floats for rotated keys, sized at launch
  const int64_t slice = blockIdx.x % a.L.slices;
  const MixedPiece pc = mp.p[blockIdx.x / a.L.slices];
  // the piece's range and slot through the split arithmetic of decode_split:
  // split s (its fp16 index, or 0) of groups_per_split = g1 - g0 starting
  // s pieces before g0
  const int s = pc.f16 >= 0 ? pc.f16 : 0;
  const int64_t gps = pc.g1 - pc.g0;
  DecodeArgs r = a;
  r.splits = mp.nf16 > 0 ? mp.nf16 : 1;
  r.groups_per_split = gps;
  r.g_base = pc.g0 - s * gps;
  r.ngroups = pc.g1 - r.g_base;
  r.split_off = pc.slot - s;
  r.do_fp16 = pc.f16 >= 0 ? 1 : 0;
  switch (pc.bits) {
    case 0x22: decode_split<D, 2, 2, G, GQC, TN, false, false>(r, slice, s, ring, qsh, NewToken{}); break;
    case 0x24: decode_split<D, 2, 4, G, GQC, TN, false, false>(r, slice, s, ring, qsh, NewToken{}); break;
    case 0x42: decode_split<D, 4, 2, G, GQC, TN, false, false>(r, slice, s, ring, qsh, NewToken{}); break;
    default: decode_split<D, 4, 4, G, GQC, TN, false, false>(r, slice, s, ring, qsh, NewToken{}); break;
  }
}

// The one-wave launch: one workgroup of one wave per (slice, split).
template <int D, int KB, int VB, int G, int GQC, bool TN>
hipError_t one_wave_launch_i(const DecodeArgs& a, const NewToken& nt, hipStream_t s) {
  const size_t lds = a.rotate ? static_cast<size_t>(a.gqa) * D * sizeof(float) : 0;
  hipLaunchKernelGGL((decode_kernel<D, KB, VB, G, GQC, TN>), dim3(static_cast<unsigned>(a.L.slices * a.splits)),
                     dim3(kLanes), lds, s, a, nt);
  return hipGetLastError();
}

// The fused launch: one workgroup of S waves per slice.  fused_plan gives
// its dynamic LDS bytes, or 0 when it does not apply: S not a multiple of 4
// up to kMaxFusedSplits, more LDS than a workgroup may hold, or (by the
// runtime's occupancy calculator) neither one pass of the CUs for all slices
// nor as many waves per CU as the one-wave launch of the same decode, so that
// merging in the workgroup never costs the stream its waves in flight.  Measured on MI355X, workgroups of 2, 3 or 6
// waves ran 1-33% slower than the one-wave launch at the same split count
// (175B-shaped MHA layer at 2 splits 973 against 855 us; 32k K4/V2 layer at
// 6 splits 330 against 302 us): a workgroup's waves do not spread evenly over
// a CU's four SIMDs unless they come in fours; at 4 splits the 32k layer
// decodes in 301.5 us merged against 304.2 us with the merge kernel.
template <int D, int KB, int VB, int G, int GQC, bool TN>
size_t fused_plan_i(const DecodeArgs& a, int W) {
  const int S = a.splits;
  if ((W != 4 && W != 8) || W > kMaxFusedSplits || S < W || S % W != 0) return 0;
  const size_t qb = a.rotate ? static_cast<size_t>(a.gqa) * D * sizeof(float) : 0;
  const size_t lds = static_cast<size_t>(W) * fused_region_bytes<D, KB, VB, G, GQC, TN>() + qb;
  int dev = 0, max_lds = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      lds > static_cast<size_t>(max_lds))
    return 0;
  int nf = 0, n1 = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nf, decode_fused_kernel<D, KB, VB, G, GQC, TN>, kLanes * W, lds) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n1, decode_kernel<D, KB, VB, G, GQC, TN>, kLanes, qb) != hipSuccess)
    return 0;
  const bool one_pass = static_cast<int64_t>(nf) * cus >= a.L.slices * (S / W);
  return one_pass || nf * W >= n1 ? lds : 0;
}

template <int D, int KB, int VB, int G, int GQC, bool TN>
hipError_t fused_launch_i(const DecodeArgs& a, const NewToken& nt, int W, hipStream_t s) {
  const size_t lds = fused_plan_i<D, KB, VB, G, GQC, TN>(a, W);
  if (lds == 0) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_fused_kernel<D, KB, VB, G, GQC, TN>),
                     dim3(static_cast<unsigned>(a.L.slices * (a.splits / W))), dim3(kLanes * W), lds, s, a, nt);
  return hipGetLastError();
}

// Calls F<D, KB, VB, G, GQC, TN>::run(a, x...) for the instance that serves a.
template <template <int, int, int, int, int, bool> class F, typename... X>
auto instance_of(const DecodeArgs& a, X... x) {
  auto gq = [&](auto d, auto kb, auto vb, auto g, auto tn) {
    constexpr int D_ = decltype(d)::value, KB_ = decltype(kb)::value, VB_ = decltype(vb)::value;
    constexpr int G_ = decltype(g)::value;
    constexpr bool TN_ = decltype(tn)::value;
    if (a.gqa == 1) return F<D_, KB_, VB_, G_, 1, TN_>::run(a, x...);
    if (a.gqa <= 4) return F<D_, KB_, VB_, G_, 4, TN_>::run(a, x...);
    if (a.gqa <= 8) return F<D_, KB_, VB_, G_, 8, TN_>::run(a, x...);
    return F<D_, KB_, VB_, G_, 16, TN_>::run(a, x...);
  };
  using std::integral_constant;
  auto tn = [&](auto d, auto kb, auto vb, auto g) {
    return a.L.token_norm ? gq(d, kb, vb, g, integral_constant<bool, true>{})
                          : gq(d, kb, vb, g, integral_constant<bool, false>{});
  };
  auto gg = [&](auto d, auto kb, auto vb) {
    return a.L.G == 32 ? tn(d, kb, vb, integral_constant<int, 32>{}) : tn(d, kb, vb, integral_constant<int, 64>{});
  };
  auto vv = [&](auto d, auto kb) {
    return a.L.vbits == 2 ? gg(d, kb, integral_constant<int, 2>{}) : gg(d, kb, integral_constant<int, 4>{});
  };
  auto kk = [&](auto d) {
    return a.L.kbits == 2 ? vv(d, integral_constant<int, 2>{}) : vv(d, integral_constant<int, 4>{});
  };
  return a.L.D == 64 ? kk(integral_constant<int, 64>{}) : kk(integral_constant<int, 128>{});
}

template <int D, int KB, int VB, int G, int GQC, bool TN>
struct FusedPlan {
  static size_t run(const DecodeArgs& a, int W) { return fused_plan_i<D, KB, VB, G, GQC, TN>(a, W); }
};
template <int D, int KB, int VB, int G, int GQC, bool TN>
struct FusedLaunch {
  static hipError_t run(const DecodeArgs& a, const NewToken& nt, int W, hipStream_t s) {
    return fused_launch_i<D, KB, VB, G, GQC, TN>(a, nt, W, s);
  }
};
template <int D, int KB, int VB, int G, int GQC, bool TN>
struct OneWaveLaunch {
  static hipError_t run(const DecodeArgs& a, const NewToken& nt, hipStream_t s) {
    return one_wave_launch_i<D, KB, VB, G, GQC, TN>(a, nt, s);
  }
};

}  // namespace

size_t decode_fused_lds(const DecodeArgs& a, int W) { return instance_of<FusedPlan>(a, W); }

hipError_t launch_decode_fused(const DecodeArgs& a, const NewToken& nt, int W, hipStream_t s) {
  return instance_of<FusedLaunch>(a, nt, W, s);
}

bool decode_supported(int D, int kbits, int vbits, int G) {
  return (D == 64 || D == 128) && (kbits == 2 || kbits == 4) && (vbits == 2 || vbits == 4) &&
         (G == 32 || G == 64) && G <= D;
}

hipError_t launch_decode(const DecodeArgs& a, const NewToken& nt, hipStream_t s) {
  return instance_of<OneWaveLaunch>(a, nt, s);
}

namespace {
template <int D, int G, bool TN>
hipError_t mixed_t(const DecodeArgs& a, const MixedPlan& mr, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(a.L.slices * mr.npieces));
  const size_t lds = a.rotate ? static_cast<size_t>(a.gqa) * D * sizeof(float) : 0;
  if (a.gqa == 1)
    hipLaunchKernelGGL((decode_mixed_kernel<D, G, 1, TN>), grid, dim3(kLanes), lds, s, a, mr);
  else if (a.gqa <= 4)
    hipLaunchKernelGGL((decode_mixed_kernel<D, G, 4, TN>), grid, dim3(kLanes), lds, s, a, mr);
  else if (a.gqa <= 8)
    hipLaunchKernelGGL((decode_mixed_kernel<D, G, 8, TN>), grid, dim3(kLanes), lds, s, a, mr);
  else
    hipLaunchKernelGGL((decode_mixed_kernel<D, G, 16, TN>), grid, dim3(kLanes), lds, s, a, mr);
  return hipGetLastError();
}
template <int D, int G>
hipError_t mixed_g(const DecodeArgs& a, const MixedPlan& mr, hipStream_t s) {
  return a.L.token_norm ? mixed_t<D, G, true>(a, mr, s) : mixed_t<D, G, false>(a, mr, s);
}
template <int D>
hipError_t mixed_d(const DecodeArgs& a, const MixedPlan& mr, hipStream_t s) {
  return a.L.G == 32 ? mixed_g<D, 32>(a, mr, s) : mixed_g<D, 64>(a, mr, s);
}
}  // namespace

hipError_t launch_decode_mixed(const DecodeArgs& a, const MixedPlan& mr, hipStream_t s) {
  if (mr.npieces < 1 || mr.npieces > kMaxPieces) return hipErrorInvalidValue;
  return a.L.D == 64 ? mixed_d<64>(a, mr, s) : mixed_d<128>(a, mr, s);
}


}  // namespace kvq
