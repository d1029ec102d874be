// kvq_internal.h -- launcher interface between the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  const uint8_t* cache;
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

// Runs of groups with equal bit widths decoded by one launch: run i covers
// groups [g_base[i], g_base[i] + ngroups[i]) with splits[i] splits of gps[i]
// groups, in split slots [split_off[i], split_off[i] + splits[i]); bits[i] is
// 16 * key bits + value bits; run fp16_run also covers the fp16 chunks.
constexpr int kMaxRuns = 8;
struct MixedRuns {
  int n;
  int fp16_run;
  int bits[kMaxRuns];
  int splits[kMaxRuns];
  int split_off[kMaxRuns];
  int64_t g_base[kMaxRuns];
  int64_t ngroups[kMaxRuns];
  int64_t gps[kMaxRuns];
};

// Both return hipSuccess or the launch error.
hipError_t launch_flush(const AppendArgs& a, hipStream_t s);
hipError_t launch_window_write(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// a: splits_total, L (any of the runs' layouts) and the common fields
hipError_t launch_decode_mixed(const DecodeArgs& a, const MixedRuns& mr, hipStream_t s);
hipError_t launch_merge(const float* partial, float* out, int rows, int splits, int D, hipStream_t s);
hipError_t launch_code_histograms(const DriftArgs& a, hipStream_t s);
hipError_t launch_drift_check(const DriftArgs& a, hipStream_t s);

bool decode_supported(int D, int kbits, int vbits, int G);

}  // namespace kvq
