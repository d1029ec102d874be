/*
 * kvq.h -- C ABI of libkvq: asymmetric low-bit KV-cache quantization fused
 * into single-query decode attention, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (pages cited by title and section):
 *   - Keys are quantized per channel, with min/max statistics over groups of
 *     G consecutive tokens; values are quantized per token, with statistics
 *     over groups of G consecutive channels; the most recent tokens stay in
 *     an fp16 window and are never quantized.  "[Framework] The Asymmetric
 *     Key-Value Cache Compression", section III (KIVI partitioning);
 *     "Asymmetric Key-Value Quantization: 2-Bit Values and 4-Bit Keys under
 *     Long-Context Drift", section 3.1 (keys per channel at 4 bits, values
 *     per token at 2 bits).
 *   - Each group stores an fp16 scale and an fp16 zero (the group minimum);
 *     codes are round-half-even((x - min) / scale) with scale =
 *     (max - min) / (2^b - 1) in IEEE binary32 (the textbook asymmetric
 *     uniform quantizer; the pages name the scheme but print no formula).
 *   - Optionally keys (at append) and queries (at decode) are rotated by the
 *     normalized Walsh-Hadamard transform, "[Framework] ...", section IV
 *     (stage 1, Y = X H, computed with the fast transform).
 *   - Decode attention is softmax(q K^T / sqrt(d)) V over every cached token,
 *     "Asymmetric Key-Value Quantization ...", section 1, computed directly
 *     on the packed cache (split over the token axis, merged with the
 *     online-softmax rule).
 *
 * Conventions for every entry point:
 *   - All device buffers are owned by the caller.  The library never
 *     allocates or frees device memory; a handle holds host metadata only.
 *   - Device pointers must be 16-byte aligned (the cache buffer 256-byte
 *     aligned) unless stated otherwise.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Device work is enqueued on it and the call returns without waiting,
 *     except kvq_export / kvq_import, which synchronize the stream.
 *   - Every call validates its arguments before enqueueing anything.  Errors
 *     are returned as kvq_status; nothing is thrown or aborted across the ABI.
 *     kvq_last_error() gives a message for the calling thread's last error.
 *   - After a device launch error (KVQ_E_DEVICE) the handle is poisoned:
 *     later calls on it return KVQ_E_STATE.  A handle is not thread-safe.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvq_cache kvq_cache; /* opaque host-side handle */

typedef enum {
  KVQ_OK = 0,
  KVQ_E_ARG = 1,         /* null / misaligned pointer, bad size, workspace too small */
  KVQ_E_UNSUPPORTED = 2, /* configuration outside what the kernels implement */
  KVQ_E_CAPACITY = 3,    /* append would exceed max_tokens; nothing was changed */
  KVQ_E_DEVICE = 4,      /* a HIP call or kernel launch failed; handle poisoned */
  KVQ_E_STATE = 5        /* handle poisoned, or an operation invalid in this state */
} kvq_status;

typedef enum { KVQ_F32 = 0, KVQ_F16 = 1, KVQ_BF16 = 2 } kvq_dtype;

typedef struct {
  uint32_t struct_size; /* must equal sizeof(kvq_config) */
  int32_t batch;        /* B >= 1 sequences, advancing in lockstep */
  int32_t num_q_heads;  /* H_q; a multiple of num_kv_heads, H_q / H_kv in {1, 2, 4, 8, 16} */
  int32_t num_kv_heads; /* H_kv >= 1; query head h uses kv head h / (H_q / H_kv) */
  int32_t head_dim;     /* D in {64, 128} */
  int32_t max_tokens;   /* capacity per sequence, >= 1 */
  int32_t k_bits;       /* key code width in {2, 4} */
  int32_t v_bits;       /* value code width in {2, 4} */
  int32_t group_size;   /* G in {32, 64}: tokens per key group, channels per value group; G <= D */
  int32_t residual;     /* R: recent tokens kept in fp16; a multiple of 32, 0 <= R <= 1024 */
  int32_t rotate;       /* 0 or 1: Walsh-Hadamard rotation of keys (append) and queries (decode) */
  int32_t in_dtype;     /* kvq_dtype of the k, v and q buffers passed in */
  int32_t sink_tokens;  /* S0: the first S0 tokens stay in fp16 (attention sinks); a multiple of G
                           in [0, 1024]; quantized groups then start at token S0 (0: no sink) */
  int32_t hybrid;       /* 0 or 1: per group, keep a symmetric quantizer (scale max|x| / c0,
                           c0 = 2^(b-1) - 1, zero = -c0 * scale) instead of the asymmetric one
                           when its largest reconstruction error on the group is smaller */
  int32_t token_norm;   /* 0 or 1: divide each quantized key token by its L2 norm (binary32,
                           pairwise summation tree, correctly rounded sqrt) before quantizing,
                           keep the norm as fp16 and multiply it back into the score; with
                           rotate = 1 this is the rotate-then-scale key pipeline */
  int32_t adapt_delta;  /* Delta >= 0, a multiple of G (0: off): position-adaptive bit widths.
                           A group's bits are fixed when it is quantized, from the length n
                           after that append: (k_bits_high, v_bits_high) if its last token is
                           among the last Delta of n, else (k_bits_low, v_bits_low) if it is
                           among the first Delta tokens, else (k_bits, v_bits).  The cache then
                           depends on how tokens were appended (a long prefill gets all three
                           regions, groups quantized while decoding are recent), and every group
                           slot is sized for the widest of the three. */
  int32_t k_bits_low, v_bits_low, k_bits_high, v_bits_high; /* in {2, 4}; used when adapt_delta > 0 */
} kvq_config;

/* Device bytes the cache buffer must hold for `cfg`, or 0 if `cfg` is
 * invalid or unsupported (kvq_last_error says why). */
size_t kvq_cache_bytes(const kvq_config* cfg);

/* Device bytes of workspace kvq_decode_attn may need for `cfg` at any split
 * count it chooses (split partials: B * H_q * S_max * (D + 4) floats).
 * 0 if `cfg` is invalid. */
size_t kvq_workspace_bytes(const kvq_config* cfg);

/* Create a handle over the caller's device buffer `cache_buf` of
 * `cache_bytes` >= kvq_cache_bytes(cfg) bytes (256-byte aligned).  The cache
 * starts empty (0 tokens per sequence).  No device work is done.  The buffer
 * contents need no initialization.  On success *out receives the handle. */
kvq_status kvq_create(const kvq_config* cfg, void* cache_buf, size_t cache_bytes, kvq_cache** out);

/* Append n_tokens tokens to every sequence.
 *   k, v: device, [B][H_kv][n_tokens][D] contiguous, elements of in_dtype.
 * Each element is widened to fp32; keys are rotated if cfg.rotate; then every
 * element is rounded to fp16 (round-to-nearest-even) and lands in the fp16
 * window.  Whenever the window holds R + G tokens the oldest G are quantized
 * (keys per channel, values per token) into packed codes with fp16
 * scale/zero, so after n tokens floor(max(0, n - R) / G) * G tokens are
 * quantized and the rest are in the window.  A prefill is one call with
 * n_tokens = N; a decode step appends 1.  Appending one token at a time gives
 * bit-identical cache contents to one call with all of them.
 * n_tokens == 0 is a no-op.  Exceeding max_tokens returns KVQ_E_CAPACITY
 * and changes nothing.  The k and v buffers may be reused once the work
 * enqueued on `stream` has completed. */
kvq_status kvq_append(kvq_cache* cache, const void* k, const void* v, int32_t n_tokens, void* stream);

/* Decode attention of one query per head over all cached tokens.
 *   q:   device, [B][H_q][D] contiguous, elements of in_dtype.
 *   out: device, [B][H_q][D] fp32, out = softmax(q K^T / sqrt(D)) V with K, V
 *        the dequantized cache (keys rotated and q rotated when cfg.rotate).
 *   workspace: device scratch of ws_bytes >= kvq_workspace_bytes(cfg); its
 *        contents on entry do not matter and are clobbered.
 * The split count over the token axis is chosen from the cache shape and the
 * number of compute units.  When every group has the same bits and a slice
 * has 4 or 8 splits, the splits of a slice run as the waves of one workgroup
 * and are merged there (the cross-split combination of kvq_merge_partials,
 * in LDS), unless that launch would hold fewer waves per compute unit; the
 * workspace is then not touched and no merge kernel follows.  With more than
 * 8 splits the count is rounded up to a multiple of 4 and each 4 consecutive
 * splits of a slice are merged in one workgroup into one partial record, the
 * merge kernel combining S/4 records per row (under the same occupancy rule,
 * and only when no workgroup is left without token groups).
 * kvq_decode_plan tells which.  Requires at least one cached token
 * (KVQ_E_STATE otherwise). */
kvq_status kvq_decode_attn(kvq_cache* cache, const void* q, float* out, void* workspace, size_t ws_bytes,
                           void* stream);

/* Bytes of the device scratch array kvq_decode_attn_noalloc keeps its split
 * partials in (one array per device, held until the process ends). */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* kvq_decode_attn for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the split partials live in a file-scope device
 * array of KVQ_NOALLOC_SCRATCH_BYTES bytes that the library holds on every
 * device it runs on, looked up once per device on the first call there.
 * Same split count, kernels and result as kvq_decode_attn.
 *   q:   device, [B][H_q][D] of in_dtype;  out: device, [B][H_q][D] float32
 *        (16-byte aligned).
 * Returns KVQ_E_ARG, enqueuing nothing, when this decode's partials
 * (B * H_q * R * (D + 4) floats, R the merge records per row that
 * kvq_decode_plan gives for the default split count) exceed
 * KVQ_NOALLOC_SCRATCH_BYTES; KVQ_E_DEVICE if the array's address cannot be
 * obtained.  No device memory is allocated or freed.  Every call on one
 * device shares that device's array, and every split record a call reads is
 * written by the same call first (nothing needs clearing), so calls that
 * overlap in time on one device -- on different streams or from different
 * threads -- race and must be serialized by the caller. */
kvq_status kvq_decode_attn_noalloc(kvq_cache* cache, const void* q, float* out, void* stream);

/* As kvq_decode_attn with an explicit split count 1 <= num_splits <= the
 * S_max sized by kvq_workspace_bytes (values above the number of token
 * groups are clamped).  Any split count gives the same result up to
 * floating-point summation order. */
kvq_status kvq_decode_attn_splits(kvq_cache* cache, const void* q, float* out, void* workspace, size_t ws_bytes,
                                  int32_t num_splits, void* stream);

/* How kvq_decode_attn_splits(num_splits) would run on the cache's current
 * tokens, without launching anything: *splits_used receives the split count
 * S per slice, *merge_records 0 when the decode writes `out` itself (one
 * split, or all splits of each slice merged inside the decode kernel), else
 * the partial records per row the merge kernel then combines (S, or S/4 when
 * groups of four splits are merged inside the decode kernel).  Either
 * pointer may be NULL.  KVQ_E_STATE on an empty cache, KVQ_E_ARG for a split
 * count outside [1, S_max]; the split count of kvq_decode_attn is
 * kvq_default_splits. */
kvq_status kvq_decode_plan(kvq_cache* cache, int32_t num_splits, int32_t* splits_used, int32_t* merge_records);

/* The two halves of kvq_decode_attn, for callers that merge partial results
 * themselves (e.g. several caches holding disjoint token ranges of the same
 * sequences, as when a long context is sharded over devices).
 *
 * kvq_decode_partials: split the cached tokens into num_splits ranges
 * (clamped as in kvq_decode_attn_splits; *splits_used receives the count S)
 * and write, for every row r = b * H_q + h and split s, at
 * partials + (r * S + s) * (D + 4) floats:
 *   [0, D)  o = sum_t 2^(x_t - m) v_t   (unnormalized)
 *   D       m, a reference point with max_t x_t - 0.5 <= m <= max_t x_t
 *           (the kernel moves it lazily; -inf for an empty split)
 *   D + 1   l = sum_t 2^(x_t - m)
 * with x_t = log2(e) * q . k_t / sqrt(D) (scores in the base-2 domain).
 * Split s covers the contiguous token groups [s * c, min(ng, (s + 1) * c))
 * with c = ceil(ng / S) (ng quantized groups), plus the fp16 window's 32-token
 * chunks w (counted from the first window token) with w mod S = S - 1 - s.
 * (A position-adaptive cache decodes pieces of one width each instead: with
 * T = the slice's page bytes / num_splits, every run smaller than T is one
 * piece, and the other runs are cut in group order into a piece of T minus
 * each small run's bytes, then pieces of T (the fp16 chunks are shared by the
 * pieces of T); slots follow that order (the big runs' pieces, then the small
 * runs), and S is the number of pieces.  When that does not apply (all runs
 * small, more than 8 runs, more pieces than fit) each run is split on its
 * own in proportion to its page bytes, at least once, the run with the most
 * splits taking the fp16 chunks, and S is at most num_splits + runs - 1;
 * KVQ_E_UNSUPPORTED when the runs outnumber the workspace maximum of splits.)
 * bytes must be >= H_q * B * S * (D + 4) * 4.  Requires a non-empty cache. */
kvq_status kvq_decode_partials(kvq_cache* cache, const void* q, float* partials, size_t bytes, int32_t num_splits,
                               int32_t* splits_used, void* stream);

/* One decode step: kvq_append of one token (k, v: [B][H_kv][1][D]) followed
 * by kvq_decode_attn (or kvq_decode_partials); results and cache contents
 * are those of the two calls.  The workspace / partials must hold
 * kvq_workspace_bytes (all splits the library may use).  Every argument is
 * checked before any work is enqueued, so on an error nothing has been
 * appended.  When the token goes to the fp16 window (not the sink, not
 * quantized by this append) of a cache without key rotation or
 * position-adaptive widths, the decode kernel writes its window slots itself
 * (one launch fewer per step); k and v are read by that kernel, so they must
 * stay unchanged until the work enqueued on `stream` has completed. */
kvq_status kvq_append_decode_attn(kvq_cache* cache, const void* k, const void* v, const void* q, float* out,
                                  void* workspace, size_t ws_bytes, void* stream);
kvq_status kvq_append_decode_partials(kvq_cache* cache, const void* k, const void* v, const void* q,
                                      float* partials, size_t bytes, int32_t num_splits, int32_t* splits_used,
                                      void* stream);

/* Merge `splits` partials per row (layout above, `rows` rows) into
 * out[rows][head_dim] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
 * M = max_s m_s; splits with m_s = -inf contribute nothing, and a row whose
 * splits are all empty yields NaN.  head_dim in {64, 128}; 1 <= splits <= 256
 * (the most kvq_workspace_bytes ever provides for), else KVQ_E_ARG. */
kvq_status kvq_merge_partials(const float* partials, float* out, int32_t rows, int32_t splits, int32_t head_dim,
                              void* stream);

/* Key token norms (cfg.token_norm = 1 only, else KVQ_E_STATE), as fp16 bit
 * patterns [bc][H_kv][n_q] for sequences [b0, b0 + bc): export copies them
 * out (synchronizes `stream`), import writes them for the n_q quantized
 * tokens of a cache filled by kvq_import (call it after kvq_import). */
kvq_status kvq_export_key_norms(kvq_cache* cache, int32_t b0, int32_t bc, void* host_k_norm, void* stream);
kvq_status kvq_import_key_norms(kvq_cache* cache, int32_t b0, int32_t bc, const void* host_k_norm, void* stream);

/* Drift detection ("Asymmetric Key-Value Quantization: 2-Bit Values and
 * 4-Bit Keys under Long-Context Drift", section 3.3: the KL divergence of the
 * current distribution of quantized values from the calibration
 * distribution, a threshold of 0.1 by default triggering requantization).
 * Quantized groups are numbered 0 .. kvq_num_quantized / G - 1 in token
 * order; a group's distribution is the histogram of its G x D key codes (of
 * its value codes).  Not for position-adaptive caches (KVQ_E_UNSUPPORTED).
 *
 * kvq_code_histograms: code counts over groups [g0, g1) of every sequence,
 *   per kv head, into device arrays k_hist [H_kv][2^k_bits] and
 *   v_hist [H_kv][2^v_bits] (uint64, 8-byte aligned, overwritten); the
 *   calibration histograms kvq_drift_check takes.
 * kvq_drift_check: for every slice s = b * H_kv + h and group g in [g0, g1),
 *   with p the group's counts / (G * D) and q the calibration counts of head h
 *   divided by their total: kl = sum_i p_i ln(p_i / q_i) (bins with p_i = 0
 *   add 0; p_i > 0 = q_i makes it +inf), fp64, for keys and values, into
 *   device arrays kl_k, kl_v [B * H_kv][g1 - g0] (double), and
 *   flags (uint8, same shape) = (kl_k > threshold) | (kl_v > threshold) << 1.
 *   A calibration histogram with no counts gives +inf.
 * kvq_requantize: quantize groups [g0, g1) again from the tokens k, v
 *   (device, [B][H_kv][(g1 - g0) * G][D], in_dtype, entry conversion and
 *   rotation as in kvq_append), for the groups whose flag is nonzero
 *   (flags: device uint8 [B * H_kv][g1 - g0] as written by kvq_drift_check,
 *   or NULL for all); each group keeps its bit widths.  The uniform quantizer
 *   recomputes its scale and zero from the given tokens (no Lloyd-Max
 *   levels).  KVQ_E_ARG for a range outside the quantized groups. */
kvq_status kvq_code_histograms(kvq_cache* cache, int64_t g0, int64_t g1, uint64_t* k_hist, uint64_t* v_hist,
                               void* stream);
kvq_status kvq_drift_check(kvq_cache* cache, int64_t g0, int64_t g1, const uint64_t* cal_k, const uint64_t* cal_v,
                           double threshold, double* kl_k, double* kl_v, uint8_t* flags, void* stream);
kvq_status kvq_requantize(kvq_cache* cache, int64_t g0, int64_t g1, const void* k, const void* v,
                          const uint8_t* flags, void* stream);

/* Split count kvq_decode_attn would use for the current token count. */
int32_t kvq_default_splits(const kvq_cache* cache);

/* Tokens per sequence currently cached, and how many of them are quantized. */
int64_t kvq_num_tokens(const kvq_cache* cache);
int64_t kvq_num_quantized(const kvq_cache* cache);

/* Forget all tokens (n = 0).  No device work. */
kvq_status kvq_reset(kvq_cache* cache);

/* Free the host handle (never the caller's device buffers).  NULL is a no-op. */
kvq_status kvq_destroy(kvq_cache* cache);

/* Message for the calling thread's most recent non-OK status ("" if none). */
const char* kvq_last_error(void);

/* Canonical (layout-independent) form of the cache for sequences
 * [batch_begin, batch_begin + batch_count), all kv heads, with
 * nq = kvq_num_quantized, nr = n - nq.  Host buffers; any may be NULL to skip:
 *   k_codes  uint8  [bc][H_kv][nq][D*k_bits/8]  codes packed along channels,
 *                   little-endian: channel c at bit k_bits*(c mod (8/k_bits))
 *                   of byte floor(k_bits*c/8)
 *   k_scale, k_zero uint16 fp16 bits [bc][H_kv][nq/G][D]   (per channel, per token group)
 *   v_codes  uint8  [bc][H_kv][nq][D*v_bits/8]
 *   v_scale, v_zero uint16 fp16 bits [bc][H_kv][nq][D/G]   (per token, per channel group)
 *   k_resid, v_resid uint16 fp16 bits [bc][H_kv][nr][D]     (the fp16 window, oldest first)
 * Synchronizes `stream`, then copies and converts.  For checkpoints and tests. */
kvq_status kvq_export(kvq_cache* cache, int32_t batch_begin, int32_t batch_count, void* k_codes, void* k_scale,
                      void* k_zero, void* v_codes, void* v_scale, void* v_zero, void* k_resid, void* v_resid,
                      void* stream);

/* Codes one per byte, uint8 [bc][H_kv][nq][D] (keys, values; either may be
 * NULL), whatever the groups' bit widths: the export for position-adaptive
 * caches, where kvq_export's packed code arrays are KVQ_E_UNSUPPORTED (its
 * parameter and fp16 arrays keep their shapes).  Synchronizes `stream`. */
kvq_status kvq_export_codes_u8(kvq_cache* cache, int32_t batch_begin, int32_t batch_count, void* k_codes,
                               void* v_codes, void* stream);

/* Key and value bit widths of the quantized groups, oldest first: writes
 * min(ng, cap) entries to each non-NULL array and returns ng (the number of
 * quantized groups per sequence), or -1 for a NULL handle.  Without
 * adapt_delta every entry is (k_bits, v_bits). */
int64_t kvq_group_bits(const kvq_cache* cache, uint8_t* k_bits, uint8_t* v_bits, int64_t cap);

/* Inverse of kvq_export: write canonical arrays (same shapes, none NULL) for
 * sequences [batch_begin, batch_begin + batch_count) holding n_tokens tokens
 * each into the device cache, and set the cache's token count to n_tokens
 * (every sequence shares one count, so import every sequence before decoding).
 * Synchronizes `stream`.  KVQ_E_CAPACITY if n_tokens > max_tokens;
 * KVQ_E_UNSUPPORTED for a position-adaptive cache (adapt_delta > 0). */
kvq_status kvq_import(kvq_cache* cache, int64_t n_tokens, int32_t batch_begin, int32_t batch_count,
                      const void* k_codes, const void* k_scale, const void* k_zero, const void* v_codes,
                      const void* v_scale, const void* v_zero, const void* k_resid, const void* v_resid,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
