// kvq_internal.h -- launcher interface between the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"
#include "kvq_layout.h"

namespace kvq {

struct AppendArgs {
  uint8_t* cache;
  Layout L;
  const void* k;        // [B][H_kv][T][D] in_dtype
  const void* v;
  int in_dtype;         // 0 f32, 1 f16, 2 bf16
  int rotate;
  int hybrid;           // per-group symmetric/asymmetric choice
  int Hkv;
  int64_t T;            // tokens in this call
  int64_t n_old;        // tokens per sequence before the call
  int64_t g_first;      // first group flushed by this call
  int64_t n_flush;      // groups flushed by this call
  int64_t w_first;      // first window position written by this call
  int64_t n_write;      // window positions written by this call
  int64_t s_first;      // first sink position written by this call
  int64_t n_sink_write; // sink positions written by this call
  // requantization: only groups g with flags[slice * flag_stride + g - flag_g0]
  // != 0 are rewritten (all when flags is null)
  const uint8_t* flags;
  int64_t flag_g0;
  int64_t flag_stride;
};

// Drift detection over groups [g0, g0 + ng) of every slice.
struct DriftArgs {
  const uint8_t* cache;
  Layout L;
  int Hkv;
  int64_t g0, ng;
  const uint64_t* cal_k;  // [H_kv][2^k_bits] calibration code counts
  const uint64_t* cal_v;  // [H_kv][2^v_bits]
  double threshold;
  double* kl_k;           // [slices][ng]
  double* kl_v;
  uint8_t* flags;         // bit 0: key KL > threshold, bit 1: value KL > threshold
  uint64_t* hist_k;       // [H_kv][2^k_bits] (histogram mode)
  uint64_t* hist_v;
};

struct DecodeArgs {
  uint8_t* cache;       // the decode writes only the window slots of a NewToken
  Layout L;
  const void* q;        // [B][H_q][D] in_dtype
  int in_dtype;
  int rotate;
  int gqa;
  int Hq, Hkv;
  int64_t n;            // tokens per sequence
  int64_t ngroups;      // quantized groups of this launch
  int splits;           // splits of this launch
  int64_t groups_per_split;
  int64_t g_base;       // first group of this launch (groups [g_base, g_base + ngroups))
  int split_off;        // this launch's first split slot in the partials
  int splits_total;     // split slots per row in the partials
  int do_fp16;          // this launch also covers the sink and window chunks
  int64_t rc0, rc1;     // window chunks [rc0, rc1) (absolute 32-token chunk indices)
  int64_t nsc;          // sink chunks holding tokens (ceil(min(n, S0) / 32))
  float* partial;       // [B*H_q][splits][D + 4] when !write_final
  float* out;           // [B][H_q][D] when write_final (splits == 1)
  int write_final;
};

// Groups of several bit widths decoded by one launch, as a table of pieces
// in dispatch order: piece k of every slice covers groups [g0, g1) of one
// width (bits = 16 * key bits + value bits), writes partial slot `slot` and
// takes the fp16 chunks of index f16 among nf16 sharers (none if f16 < 0).
// Block b runs piece b / slices of slice b % slices, so all slices' piece 0
// is dispatched first, then piece 1, ...
constexpr int kMaxRuns = 8;
constexpr int kMaxPieces = 48;
struct MixedPiece {
  int bits, g0, g1, slot, f16;
};
struct MixedPlan {
  int npieces, nf16;
  MixedPiece p[kMaxPieces];
};

// Bytes of the per-device scratch array behind kvq_decode_attn_noalloc (split
// partials), and its device address on the current device (looked up once per
// device, with that device current).
constexpr size_t kNoallocScratchBytes = KVQ_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

// Both return hipSuccess or the launch error.
hipError_t launch_flush(const AppendArgs& a, hipStream_t s);
hipError_t launch_window_write(const AppendArgs& a, hipStream_t s);
// The token appended by a step whose fp16 window write is left to the decode
// (pos >= 0: its position, a window position): k and v ([B][H_kv][1][D],
// in_dtype) hold it; the wave whose window chunk holds the position takes it
// from there instead of the cache and stores it to the window.
struct NewToken {
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t pos = -1;
};
hipError_t launch_decode(const DecodeArgs& a, const NewToken& nt, hipStream_t s);
// A decode of one launch (every group of one width) whose split count S per
// slice is a multiple of W (4 or 8) can run each slice's splits in groups of
// W as the waves of one workgroup, merged in LDS: with S = W the workgroup
// writes `out` (partial unused); otherwise each writes its group's merged
// record to partial slot gi of S / W per row, for the merge kernel.
// decode_fused_lds: that launch's dynamic LDS bytes, 0 when it does not apply
// or would hold fewer waves per CU than launch_decode and not fit one pass.
constexpr int kMaxFusedSplits = 8;
size_t decode_fused_lds(const DecodeArgs& a, int W);
hipError_t launch_decode_fused(const DecodeArgs& a, const NewToken& nt, int W, hipStream_t s);
// a: splits_total (= npieces), L (any of the widths' layouts) and the common fields
hipError_t launch_decode_mixed(const DecodeArgs& a, const MixedPlan& mp, hipStream_t s);
hipError_t launch_merge(const float* partial, float* out, int rows, int splits, int D, hipStream_t s);
hipError_t launch_code_histograms(const DriftArgs& a, hipStream_t s);
hipError_t launch_drift_check(const DriftArgs& a, hipStream_t s);

bool decode_supported(int D, int kbits, int vbits, int G);

}  // namespace kvq
