// kvq_layout.h -- device memory layout of the packed KV cache.
//
// The cache is laid out so that every wave of the decode kernel reads each
// 32-token chunk with one 16-byte load per lane per 1 KiB, and so that the
// dwords a lane receives are exactly its operands of the
// v_mfma_f32_16x16x32_f16 instruction after a two-operation unpack.
//
// MFMA operand convention used throughout (wave64, lane l, l16 = l % 16,
// j = l / 16, element e = 0..7 of the lane's eight fp16 operand values):
//   A (16 x 32, M x K): row l16, column 8j + e
//   B (32 x 16, K x N): row 8j + e, column l16
//   C (16 x 16):        rows 4j + r (r = 0..3), column l16
//
// Keys (QK^T): A = key codes, rows = 16 tokens of an M-tile mt (0 or 1 of a
// 32-token chunk), columns = 32 channels of k-block kb; B = scaled queries,
// columns = query heads.  C row 4j + r of tile mt is token 16 mt + 4j + r.
//
// Values (PV): A = value codes transposed, rows = 16 channels of M-tile mt,
// columns = the 32 tokens of the chunk in the order tau(j, e) below; B =
// softmax weights times value scales, columns = query heads.  tau makes lane
// (head l16, j) own exactly the tokens whose scores it holds in the C tiles
// of the QK step, so no data moves between lanes between the two products:
//   tau(j, e) = 4j + e           for e < 4
//             = 16 + 4j + e - 4  for e >= 4
//
// Key code unpack: a 32-bit word w holds fields for two fp16 lanes of a
// half8 (low half -> even e, high half -> odd e).  w & mask turns a b-bit
// field at bit position p of each half into the fp16 subnormal
// 2^(p - 24) * code exactly; a shift by 8 brings the upper byte of each half
// down.  The 2^p factors are folded into the other operand (powers of two,
// exact).  Value codes are laid out for gfx950's fp4 / fp8 -> fp16
// conversions instead (vcode_bit below), which give normal-range fp16 codes.
//
//   4-bit word, operand pair i = e >> 1: field at 4 * (i & 1) after shifting
//     by 8 * (i >> 1); multiplier 16^(i & 1).  Bit of element e:
//     16 * (e & 1) + 4 * (e >> 1).
//   2-bit word holds two sub-blocks s (low byte, high byte of each half):
//     element e of sub-block s at bit 16 * (e & 1) + 8 * s + 2 * (e >> 1);
//     multiplier 4^(e >> 1).
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define KVQ_HD __host__ __device__ __forceinline__
#else
#define KVQ_HD inline
#endif

namespace kvq {

constexpr int kChunk = 32;     // tokens per chunk (the K of the PV MFMA)
constexpr int kLanes = 64;

struct Layout {
  int D, kbits, vbits, G, R;
  int S0;                       // attention-sink tokens kept in fp16 (a multiple of G and of 32)
  int token_norm;               // 1: quantized key tokens carry an fp16 norm
  int sink_chunks;              // S0 / 32
  int nkb, nmt, ncg;            // D/32 key k-blocks, D/16 value M-tiles, D/G value groups
  int chunks_per_group;         // G / 32
  int kw, vw;                   // dwords per lane per chunk of key / value codes
  int64_t kc_chunk_bytes;       // key code bytes of one chunk
  int64_t vc_chunk_bytes;
  int64_t vp_chunk_bytes;       // value scale/zero bytes of one chunk
  int64_t kp_bytes;             // key scale + zero bytes of one group
  int64_t kn_chunk_bytes;       // key token norms of one chunk (64, or 0 without token norms)
  int64_t off_kcodes, off_kparams, off_vcodes, off_vparams, off_knorm, page_bytes;
  int64_t pages;                // pages (token groups) per slice
  int cap;                      // window ring slots per slice (R + G)
  int ring_chunks;              // cap / 32
  int64_t ring_chunk_bytes;     // K part then V part, fp16, 32 * D * 2 each
  int64_t slices;               // B * H_kv
  int64_t pages_offset, ring_offset, total_bytes;
  int64_t sink_offset;          // fp16 sink chunks, per slice, in the window ring's chunk format
};

KVQ_HD int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// page_stride > 0 spaces the group pages that far apart (>= this layout's own
// page size): caches whose groups have different bit widths give every
// group a slot of the widest page.
inline Layout make_layout(int B, int Hkv, int D, int max_tokens, int kbits, int vbits, int G, int R, int S0 = 0,
                          int token_norm = 0, int64_t page_stride = 0) {
  Layout L{};
  L.D = D; L.kbits = kbits; L.vbits = vbits; L.G = G; L.R = R;
  L.S0 = S0; L.sink_chunks = S0 / kChunk;
  L.token_norm = token_norm;
  L.nkb = D / 32; L.nmt = D / 16; L.ncg = D / G;
  L.chunks_per_group = G / kChunk;
  L.kw = 2 * L.nkb * kbits / 4;            // 4-bit: one dword per (mt, kb); 2-bit: half of that
  L.vw = L.nmt * vbits / 4;                // 4-bit: one dword per mt; 2-bit: half
  L.kc_chunk_bytes = (int64_t)kLanes * L.kw * 4;
  L.vc_chunk_bytes = (int64_t)kLanes * L.vw * 4;
  L.vp_chunk_bytes = align_up((int64_t)kChunk * L.ncg * 4, 256);  // whole 256-byte DMA blocks
  L.kp_bytes = (int64_t)D * 4;
  L.kn_chunk_bytes = token_norm ? (int64_t)kChunk * 2 : 0;
  // page: [key codes per chunk][value codes per chunk][key scale, zero rows]
  // [value params per chunk][key token norms per chunk]; the parameters are
  // one contiguous block
  L.off_kcodes = 0;
  L.off_vcodes = L.off_kcodes + L.chunks_per_group * L.kc_chunk_bytes;
  L.off_kparams = L.off_vcodes + L.chunks_per_group * L.vc_chunk_bytes;
  L.off_vparams = L.off_kparams + L.kp_bytes;
  L.off_knorm = L.off_vparams + L.chunks_per_group * L.vp_chunk_bytes;
  L.page_bytes = L.off_knorm + L.chunks_per_group * L.kn_chunk_bytes;
  if (page_stride > L.page_bytes) L.page_bytes = page_stride;
  int64_t over = (int64_t)max_tokens - S0 - R;
  L.pages = over > 0 ? over / G : 0;
  L.cap = R + G;
  L.ring_chunks = L.cap / kChunk;
  L.ring_chunk_bytes = (int64_t)kChunk * D * 2 * 2;
  L.slices = (int64_t)B * Hkv;
  L.pages_offset = 0;
  L.ring_offset = align_up(L.slices * L.pages * L.page_bytes, 256);
  L.sink_offset = align_up(L.ring_offset + L.slices * L.ring_chunks * L.ring_chunk_bytes, 256);
  L.total_bytes = align_up(L.sink_offset + L.slices * L.sink_chunks * L.ring_chunk_bytes, 256);
  return L;
}

// ---- token order of the PV step -------------------------------------------
KVQ_HD int tau(int j, int e) { return e < 4 ? 4 * j + e : 16 + 4 * j + (e - 4); }
KVQ_HD void tau_inv(int t, int* j, int* e) {
  if (t < 16) { *j = t >> 2; *e = t & 3; }
  else { *j = (t - 16) >> 2; *e = 4 + (t & 3); }
}

// Byte offset, inside a chunk's code block, of dword d of lane l when each
// lane holds w dwords stored as 16-byte vectors (w >= 4) or one w-dword vector.
KVQ_HD int64_t lane_dword_offset(int w, int l, int d) {
  int vw = w >= 4 ? 4 : w;
  return (int64_t)(d / vw) * (kLanes * vw * 4) + (int64_t)l * vw * 4 + (d % vw) * 4;
}

// Location of the key code of token t (0..31 within its chunk), channel c.
KVQ_HD void kcode_loc(const Layout& L, int t, int c, int64_t* byte, int* bit) {
  int mt = t >> 4, t16 = t & 15;
  int kb = c >> 5, j = (c >> 3) & 3, e = c & 7;
  int l = j * 16 + t16;
  int combo = mt * L.nkb + kb;
  if (L.kbits == 4) {
    *byte = lane_dword_offset(L.kw, l, combo);
    *bit = 16 * (e & 1) + 4 * (e >> 1);
  } else {
    *byte = lane_dword_offset(L.kw, l, combo >> 1);
    *bit = 16 * (e & 1) + 8 * (combo & 1) + 2 * (e >> 1);
  }
}

// Bit of element e (0..7) of value M-tile mt inside its code word (word mt
// for 4-bit codes, mt / 2 for 2-bit).  The two elements of each operand pair
// (e, e + 1 with e even) share a byte, each in the low bits of one nibble, so
// a masked word is read by the fp4 / fp8 -> fp16 conversions:
//   2-bit: byte e / 2, nibble e % 2, the nibble's low (mt even) or high
//          (mt odd) two bits; (w >> 2 (mt odd)) & 0x33333333 leaves the
//          tile's codes as fp4 e2m1 nibbles of value code / 2, byte k holding
//          pair k.
//   4-bit: elements 0..3 in the low nibbles of bytes 0..3, elements 4..7 in
//          the high nibbles; w & 0x0F0F0F0F (and (w >> 4) & 0x0F0F0F0F) are
//          four fp8 e4m3 bytes of value code * 2^-9, 16-bit half h holding
//          pair h (pairs 2 + h).
KVQ_HD int vcode_bit(int vbits, int mt, int e) {
  return vbits == 4 ? 16 * ((e >> 1) & 1) + 8 * (e & 1) + 4 * (e >> 2) : 8 * (e >> 1) + 4 * (e & 1) + 2 * (mt & 1);
}

// Location of the value code of token t (0..31 within its chunk), channel c.
KVQ_HD void vcode_loc(const Layout& L, int t, int c, int64_t* byte, int* bit) {
  int mt = c >> 4, c16 = c & 15;
  int j, e;
  tau_inv(t, &j, &e);
  int l = j * 16 + c16;
  *byte = lane_dword_offset(L.vw, l, L.vbits == 4 ? mt : mt >> 1);
  *bit = vcode_bit(L.vbits, mt, e);
}

// Index (in fp16 elements) of channel c's key scale within a group's scale
// row; the zero row follows the scale row (D elements later).  Lane group j
// reads its 8 * nkb channels {32 kb + 8 j + e} as one contiguous run.
KVQ_HD int kparam_index(const Layout& L, int c) {
  int kb = c >> 5, j = (c >> 3) & 3, e = c & 7;
  return j * (L.D / 4) + kb * 8 + e;
}

// fp16 element index, inside a chunk's value-parameter block, of the scale of
// (token t, value group cg); the zero is 2 elements (one dword) later.  The
// block is [j][pair i][group cg][scale pair, zero pair] dwords, where pair i
// holds tokens tau(j, 2i) and tau(j, 2i + 1): a lane that owns consecutive
// token pairs of lane group j reads all their scales and zeros as one run,
// and each scale dword is one fp16 pair of a PV B operand as it is.
KVQ_HD int vparam_scale_elem(const Layout& L, int t, int cg) {
  int j, e;
  tau_inv(t, &j, &e);
  return (((j * 4 + (e >> 1)) * L.ncg + cg) * 2) * 2 + (e & 1);
}
KVQ_HD int vparam_zero_elem(const Layout& L, int t, int cg) { return vparam_scale_elem(L, t, cg) + 2; }

// fp16 element index, inside a chunk's key-norm block, of token t's norm:
// [j][pair i][e & 1] (the same token pairs as the value parameters).
KVQ_HD int knorm_elem(int t) {
  int j, e;
  tau_inv(t, &j, &e);
  return (j * 4 + (e >> 1)) * 2 + (e & 1);
}

// Byte offsets inside a ring chunk of the fp16 window copy of token t, channel c.
// Keys are stored as the QK A operand, values as the PV A operand.
KVQ_HD int64_t ring_k_offset(const Layout& L, int t, int c) {
  int mt = t >> 4, t16 = t & 15;
  int kb = c >> 5, j = (c >> 3) & 3, e = c & 7;
  int l = j * 16 + t16;
  return ((int64_t)(mt * L.nkb + kb) * kLanes + l) * 16 + e * 2;
}
KVQ_HD int64_t ring_v_offset(const Layout& L, int t, int c) {
  int mt = c >> 4, c16 = c & 15;
  int j, e;
  tau_inv(t, &j, &e);
  int l = j * 16 + c16;
  return (int64_t)kChunk * L.D * 2 + ((int64_t)mt * kLanes + l) * 16 + e * 2;
}

// Address helpers (byte offsets from the cache base).
KVQ_HD int64_t page_offset(const Layout& L, int64_t slice, int64_t g) {
  return L.pages_offset + (slice * L.pages + g) * L.page_bytes;
}
KVQ_HD int64_t ring_chunk_offset(const Layout& L, int64_t slice, int64_t pos) {
  return L.ring_offset + (slice * L.ring_chunks + (pos / kChunk) % L.ring_chunks) * L.ring_chunk_bytes;
}
// The fp16 chunk holding token position pos: a sink chunk for pos < S0, else
// the window ring's.
KVQ_HD int64_t fp16_chunk_offset(const Layout& L, int64_t slice, int64_t pos) {
  return pos < L.S0 ? L.sink_offset + (slice * L.sink_chunks + pos / kChunk) * L.ring_chunk_bytes
                    : ring_chunk_offset(L, slice, pos);
}

// Quantized tokens among n: whole groups of G aligned to token S0 (after the
// fp16 sink), leaving at least R recent tokens in fp16.
KVQ_HD int64_t num_quantized(int64_t n, int G, int R, int S0 = 0) {
  int64_t over = n - S0 - R;
  return over > 0 ? over / G * G : 0;
}

}  // namespace kvq
