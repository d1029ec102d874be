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
  int64_t ngroups;      // quantized groups per sequence
  int splits;
  int64_t groups_per_split;
  int64_t rc0, rc1;     // window chunks [rc0, rc1) (absolute 32-token chunk indices)
  int64_t nsc;          // sink chunks holding tokens (ceil(min(n, S0) / 32))
  float* partial;       // [B*H_q][splits][D + 4] when !write_final
  float* out;           // [B][H_q][D] when write_final (splits == 1)
  int write_final;
};

// Both return hipSuccess or the launch error.
hipError_t launch_flush(const AppendArgs& a, hipStream_t s);
hipError_t launch_window_write(const AppendArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_merge(const float* partial, float* out, int rows, int splits, int D, hipStream_t s);

bool decode_supported(int D, int kbits, int vbits, int G);

}  // namespace kvq
