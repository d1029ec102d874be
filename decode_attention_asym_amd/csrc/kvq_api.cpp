// kvq_api.cpp -- host side of libkvq: validation, layout planning, host-side
// token counters, split choice, launches, canonical export/import.
//
// The window bookkeeping follows "[Framework] The Asymmetric Key-Value Cache
// Compression", section III (a full-precision window of the most recent
// tokens): after n tokens, floor(max(0, n - R) / G) * G tokens are quantized
// in whole groups aligned to token 0 and the rest stay in fp16, so a group is
// flushed whenever the window reaches R + G tokens.  All sequences advance in
// lockstep, so the host knows every count without reading the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

using kvq::Layout;

struct kvq_cache {
  kvq_config cfg;
  Layout L;                 // middle bits; page_bytes is the group slot size
  uint8_t* buf;
  int64_t n;
  bool poisoned;
  int cu_count;
  std::vector<uint8_t> gk, gv;  // key / value bits of each quantized group
  // dynamic LDS of the workgroup-merged decode per (splits, key bits, value
  // bits, group size), 0 where it does not apply (kvq::decode_fused_lds,
  // asked once)
  std::map<int64_t, size_t> fused_lds;
};

namespace {

thread_local std::string g_err;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  g_err = msg;
  return st;
}

kvq_status ok() { return KVQ_OK; }

kvq_status validate(const kvq_config* c) {
  if (!c) return fail(KVQ_E_ARG, "config is NULL");
  if (c->struct_size != sizeof(kvq_config))
    return fail(KVQ_E_ARG, "config.struct_size %u != sizeof(kvq_config) %zu", c->struct_size, sizeof(kvq_config));
  if (c->batch < 1 || c->num_kv_heads < 1 || c->num_q_heads < 1 || c->max_tokens < 1)
    return fail(KVQ_E_ARG, "batch, heads and max_tokens must be positive");
  if (c->num_q_heads % c->num_kv_heads != 0)
    return fail(KVQ_E_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", c->num_q_heads, c->num_kv_heads);
  int gqa = c->num_q_heads / c->num_kv_heads;
  if (gqa != 1 && gqa != 2 && gqa != 4 && gqa != 8 && gqa != 16)
    return fail(KVQ_E_UNSUPPORTED, "query heads per kv head %d not in {1,2,4,8,16}", gqa);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(KVQ_E_UNSUPPORTED, "head_dim %d not in {64,128}", c->head_dim);
  if ((c->k_bits != 2 && c->k_bits != 4) || (c->v_bits != 2 && c->v_bits != 4))
    return fail(KVQ_E_UNSUPPORTED, "k_bits %d / v_bits %d not in {2,4}", c->k_bits, c->v_bits);
  if ((c->group_size != 32 && c->group_size != 64) || c->group_size > c->head_dim)
    return fail(KVQ_E_UNSUPPORTED, "group_size %d not in {32,64} or larger than head_dim", c->group_size);
  if (c->residual < 0 || c->residual > 1024 || c->residual % 32 != 0)
    return fail(KVQ_E_UNSUPPORTED, "residual %d must be a multiple of 32 in [0, 1024]", c->residual);
  if (c->rotate != 0 && c->rotate != 1) return fail(KVQ_E_ARG, "rotate must be 0 or 1");
  if (c->sink_tokens < 0 || c->sink_tokens > 1024 || c->sink_tokens % c->group_size != 0)
    return fail(KVQ_E_UNSUPPORTED, "sink_tokens %d must be a multiple of group_size in [0, 1024]", c->sink_tokens);
  if (c->hybrid != 0 && c->hybrid != 1) return fail(KVQ_E_ARG, "hybrid must be 0 or 1");
  if (c->token_norm != 0 && c->token_norm != 1) return fail(KVQ_E_ARG, "token_norm must be 0 or 1");
  if (c->adapt_delta < 0 || c->adapt_delta % c->group_size != 0)
    return fail(KVQ_E_UNSUPPORTED, "adapt_delta %d must be a non-negative multiple of group_size", c->adapt_delta);
  if (c->adapt_delta > 0) {
    for (int b : {c->k_bits_low, c->v_bits_low, c->k_bits_high, c->v_bits_high})
      if (b != 2 && b != 4) return fail(KVQ_E_UNSUPPORTED, "adaptive bit widths must be 2 or 4");
    if (!kvq::decode_supported(c->head_dim, c->k_bits_low, c->v_bits_low, c->group_size) ||
        !kvq::decode_supported(c->head_dim, c->k_bits_high, c->v_bits_high, c->group_size))
      return fail(KVQ_E_UNSUPPORTED, "no kernel for an adaptive (head_dim, bits, group) combination");
  }
  if (c->in_dtype < KVQ_F32 || c->in_dtype > KVQ_BF16) return fail(KVQ_E_ARG, "in_dtype %d unknown", c->in_dtype);
  if (!kvq::decode_supported(c->head_dim, c->k_bits, c->v_bits, c->group_size))
    return fail(KVQ_E_UNSUPPORTED, "no kernel for this (head_dim, bits, group) combination");
  return KVQ_OK;
}

Layout layout_bits(const kvq_config* c, int kb, int vb, int64_t stride) {
  return kvq::make_layout(c->batch, c->num_kv_heads, c->head_dim, c->max_tokens, kb, vb, c->group_size, c->residual,
                          c->sink_tokens, c->token_norm, stride);
}

// The cache layout: middle bits, with group slots as large as the widest page.
Layout layout_of(const kvq_config* c) {
  int64_t stride = layout_bits(c, c->k_bits, c->v_bits, 0).page_bytes;
  if (c->adapt_delta > 0) {
    stride = std::max(stride, layout_bits(c, c->k_bits_low, c->v_bits_low, 0).page_bytes);
    stride = std::max(stride, layout_bits(c, c->k_bits_high, c->v_bits_high, 0).page_bytes);
  }
  return layout_bits(c, c->k_bits, c->v_bits, stride);
}

// Layout of the pages of one bit width inside this cache's group slots.
Layout layout_for(const kvq_cache* h, int kb, int vb) { return layout_bits(&h->cfg, kb, vb, h->L.page_bytes); }

// Layout of each of the first ng groups' pages.
std::vector<Layout> group_layouts(const kvq_cache* h, int64_t ng) {
  std::vector<Layout> gl(static_cast<size_t>(ng), h->L);
  if (h->cfg.adapt_delta > 0)
    for (int64_t g = 0; g < ng; ++g) gl[g] = layout_for(h, h->gk[g], h->gv[g]);
  return gl;
}

// Runs of consecutive groups with equal bit widths among groups [g0, g1).
struct Run { int64_t g0, g1; int kb, vb; };
std::vector<Run> runs_of(const kvq_cache* h, int64_t g0, int64_t g1) {
  std::vector<Run> r;
  for (int64_t g = g0; g < g1; ++g) {
    if (r.empty() || r.back().kb != h->gk[g] || r.back().vb != h->gv[g]) r.push_back({g, g, h->gk[g], h->gv[g]});
    r.back().g1 = g + 1;
  }
  return r;
}

int max_splits(const kvq_config* c) {
  int64_t slices = static_cast<int64_t>(c->batch) * c->num_kv_heads;
  int64_t s = (16384 + slices - 1) / slices;
  return static_cast<int>(std::min<int64_t>(256, std::max<int64_t>(1, s)));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

kvq_status check_handle(const kvq_cache* h) {
  if (!h) return fail(KVQ_E_ARG, "handle is NULL");
  if (h->poisoned) return fail(KVQ_E_STATE, "handle poisoned by an earlier device error");
  return KVQ_OK;
}

kvq_status device_error(kvq_cache* h, hipError_t e, const char* what) {
  h->poisoned = true;
  return fail(KVQ_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

int64_t nquant_of(const kvq_cache* h, int64_t n) {
  return kvq::num_quantized(n, h->cfg.group_size, h->cfg.residual, h->cfg.sink_tokens);
}
int64_t ngroups_of(const kvq_cache* h) { return nquant_of(h, h->n) / h->cfg.group_size; }

// Whether a decode of one run of (kb, vb) groups at S splits per slice may
// run them in groups of W as the waves of one workgroup, merged there (asked
// of the kernels once per bit widths, split count and group size).
bool fused_allowed(kvq_cache* h, int kb, int vb, int64_t S, int W) {
  if (W < 2 || W > kvq::kMaxFusedSplits || S < W || S % W != 0 || S > INT32_MAX) return false;
  const int64_t key = (static_cast<int64_t>(S) << 24) | (kb << 16) | (vb << 8) | W;
  auto it = h->fused_lds.find(key);
  if (it == h->fused_lds.end()) {
    kvq::DecodeArgs a{};
    a.L = layout_for(h, kb, vb);
    a.rotate = h->cfg.rotate;
    a.gqa = h->cfg.num_q_heads / h->cfg.num_kv_heads;
    a.splits = static_cast<int>(S);
    it = h->fused_lds.emplace(key, kvq::decode_fused_lds(a, W)).first;
  }
  return it->second > 0;
}

// Split count for a decode over n tokens.
int choose_splits(kvq_cache* h, int64_t n) {
  if (h->cu_count <= 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      h->cu_count = cus;
    else
      h->cu_count = 256;
  }
  // One pass of the CUs: as many workgroups as fit at once (12 per CU, 8 for
  // the 16-head kernels, whose VGPRs allow two waves per SIMD), and at least
  // two splits per slice.  Measured on MI355X (step us, default splits
  // before -> after): 32k K4/V2 319 -> 313 (8 -> 6 splits), 8k K2/V2 47.5 ->
  // 45 (32 -> 24); the 175B-shaped MHA stays at 2 (1 split: 880 us, 2: 867).
  const int64_t slices = h->L.slices;
  const int64_t per_cu = h->cfg.num_q_heads / h->cfg.num_kv_heads > 8 ? 8 : 12;
  const int64_t target = static_cast<int64_t>(h->cu_count) * per_cu;
  int64_t s = std::max<int64_t>(2, (target + slices - 1) / slices);
  // where one pass takes 4 to 6 splits, 4 splits merged inside the decode
  // kernel (one workgroup of four waves per slice) save the merge launch:
  // measured on the 32k K4/V2 layer, 301.5 us against 306.2 us for 6 splits
  // and the merge kernel (4 and 6 splits stream the cache equally fast)
  if (s >= 4 && s <= 6 && h->cfg.adapt_delta == 0 && fused_allowed(h, h->cfg.k_bits, h->cfg.v_bits, 4, 4)) s = 4;
  int64_t ng = nquant_of(h, n) / h->cfg.group_size;
  s = std::min<int64_t>(s, std::max<int64_t>(1, ng / 2));
  s = std::min<int64_t>(s, max_splits(&h->cfg));
  return static_cast<int>(std::max<int64_t>(1, s));
}

// Pieces of a decode over runs of several widths, for one launch (see
// kvq::MixedPlan).  With S splits' worth of page bytes per slice, T = bytes /
// S: a run smaller than T ("short") is one piece; the long runs are cut, in
// group order, into S pieces: first one partner piece of T minus each short
// run's bytes, then pieces of T.  All long pieces come first in dispatch
// order and fill the CUs; the partners finish first and their slots take
// the short pieces, so every slot ends with about T bytes.  The fp16 chunks
// go to the pieces of T.  Returns false (use one launch per run) when the
// runs do not fit this scheme.
bool plan_pieces(const kvq_cache* h, const std::vector<Run>& runs, int64_t S, kvq::MixedPlan* mp) {
  const kvq_config& c = h->cfg;
  std::vector<int64_t> pb(runs.size()), bytes(runs.size());
  int64_t total = 0;
  for (size_t i = 0; i < runs.size(); ++i) {
    pb[i] = layout_bits(&c, runs[i].kb, runs[i].vb, 0).page_bytes;
    bytes[i] = (runs[i].g1 - runs[i].g0) * pb[i];
    total += bytes[i];
  }
  const double T = static_cast<double>(total) / static_cast<double>(S);
  std::vector<size_t> shorts, longs;
  for (size_t i = 0; i < runs.size(); ++i) (static_cast<double>(bytes[i]) < T ? shorts : longs).push_back(i);
  const int64_t nshort = static_cast<int64_t>(shorts.size());
  if (longs.empty() || nshort >= S) return false;
  // byte targets of the long pieces, in dispatch order
  std::vector<double> target;
  for (size_t i : shorts) target.push_back(T - static_cast<double>(bytes[i]));
  while (static_cast<int64_t>(target.size()) < S) target.push_back(T);
  std::vector<kvq::MixedPiece> body, tail;
  size_t ti = 0;
  int nf16 = 0;
  for (size_t li = 0; li < longs.size(); ++li) {
    const Run& r = runs[longs[li]];
    int64_t g = r.g0;
    while (g < r.g1) {
      const double want = ti < target.size() ? target[ti] : T;
      // the boundary nearest to `want` bytes, at least one group, within the run
      int64_t n = std::max<int64_t>(1, static_cast<int64_t>(want / pb[longs[li]] + 0.5));
      if (li + 1 == longs.size() && ti + 1 >= target.size()) n = r.g1 - g;  // the last piece takes the rest
      n = std::min<int64_t>(n, r.g1 - g);
      const bool partner = ti < shorts.size();
      body.push_back({16 * r.kb + r.vb, static_cast<int>(g), static_cast<int>(g + n), 0, partner ? -1 : nf16++});
      g += n;
      ++ti;
    }
  }
  for (size_t i : shorts) tail.push_back({16 * runs[i].kb + runs[i].vb, static_cast<int>(runs[i].g0),
                                          static_cast<int>(runs[i].g1), 0, -1});
  if (nf16 == 0) {  // no piece of T: the first long piece takes the fp16 chunks
    body[0].f16 = 0;
    nf16 = 1;
  }
  const size_t np = body.size() + tail.size();
  if (np > static_cast<size_t>(kvq::kMaxPieces) || static_cast<int64_t>(np) > max_splits(&c)) return false;
  mp->npieces = static_cast<int>(np);
  mp->nf16 = nf16;
  size_t k = 0;
  for (const auto& pc : body) mp->p[k++] = pc;
  for (const auto& pc : tail) mp->p[k++] = pc;
  for (size_t q = 0; q < np; ++q) mp->p[q].slot = static_cast<int>(q);
  return true;
}

// Split counts of the runs of equal-bit groups: about S times the run's share
// of the page bytes each, at least one, at most S + runs - 1 in total (short
// runs get a split of their own without shortening the long runs': on the
// 32k layer with a 16-group head and tail, 6 + 2 splits ran in 331 us where
// sharing 6 took 354 us) and never more than the workspace holds.
std::vector<int64_t> run_splits(const kvq_cache* h, const std::vector<Run>& runs, int64_t S) {
  std::vector<double> wgt(runs.size());
  double tot_w = 0;
  for (size_t i = 0; i < runs.size(); ++i) {
    wgt[i] = double(runs[i].g1 - runs[i].g0) * double(layout_bits(&h->cfg, runs[i].kb, runs[i].vb, 0).page_bytes);
    tot_w += wgt[i];
  }
  std::vector<int64_t> sp(runs.size());
  int64_t tot = 0;
  for (size_t i = 0; i < runs.size(); ++i) {
    sp[i] = std::max<int64_t>(1, static_cast<int64_t>(double(S) * wgt[i] / tot_w + 0.5));
    sp[i] = std::min<int64_t>(sp[i], runs[i].g1 - runs[i].g0);
    tot += sp[i];
  }
  const int64_t nr = static_cast<int64_t>(runs.size());
  const int64_t cap = std::max<int64_t>(nr, std::min<int64_t>(S + nr - 1, max_splits(&h->cfg)));
  while (tot > cap) {
    size_t k = static_cast<size_t>(std::max_element(sp.begin(), sp.end()) - sp.begin());
    --sp[k];
    --tot;
  }
  return sp;
}

}  // namespace

extern "C" {

const char* kvq_last_error(void) { return g_err.c_str(); }

size_t kvq_cache_bytes(const kvq_config* cfg) {
  if (validate(cfg) != KVQ_OK) return 0;
  return static_cast<size_t>(layout_of(cfg).total_bytes);
}

size_t kvq_workspace_bytes(const kvq_config* cfg) {
  if (validate(cfg) != KVQ_OK) return 0;
  return static_cast<size_t>(cfg->batch) * cfg->num_q_heads * max_splits(cfg) * (cfg->head_dim + 4) * sizeof(float);
}

kvq_status kvq_create(const kvq_config* cfg, void* cache_buf, size_t cache_bytes, kvq_cache** out) {
  kvq_status st = validate(cfg);
  if (st != KVQ_OK) return st;
  if (!out) return fail(KVQ_E_ARG, "out is NULL");
  if (!cache_buf || !aligned(cache_buf, 256)) return fail(KVQ_E_ARG, "cache buffer NULL or not 256-byte aligned");
  Layout L = layout_of(cfg);
  if (cache_bytes < static_cast<size_t>(L.total_bytes))
    return fail(KVQ_E_ARG, "cache buffer holds %zu bytes, %lld needed", cache_bytes, (long long)L.total_bytes);
  kvq_cache* h = new (std::nothrow) kvq_cache{};
  if (!h) return fail(KVQ_E_ARG, "out of host memory");
  h->cfg = *cfg;
  h->L = L;
  h->buf = static_cast<uint8_t*>(cache_buf);
  h->n = 0;
  h->poisoned = false;
  h->cu_count = 0;
  try {
    h->gk.assign(static_cast<size_t>(L.pages), static_cast<uint8_t>(cfg->k_bits));
    h->gv.assign(static_cast<size_t>(L.pages), static_cast<uint8_t>(cfg->v_bits));
  } catch (...) {
    delete h;
    return fail(KVQ_E_ARG, "out of host memory");
  }
  *out = h;
  return ok();
}

kvq_status kvq_destroy(kvq_cache* h) {
  delete h;
  return ok();
}

kvq_status kvq_reset(kvq_cache* h) {
  if (!h) return fail(KVQ_E_ARG, "handle is NULL");
  h->n = 0;
  return ok();
}

int64_t kvq_num_tokens(const kvq_cache* h) { return h ? h->n : -1; }

int64_t kvq_num_quantized(const kvq_cache* h) {
  return h ? nquant_of(h, h->n) : -1;
}

}  // extern "C"

namespace {

// deferred: when not null and the call appends one token that goes to the
// fp16 window (not the sink, not flushed) of a cache without key rotation or
// position-adaptive widths, the window write is left to the decode that
// follows (the token's position is returned; the decode must run), else -1.
kvq_status append_impl(kvq_cache* h, const void* k, const void* v, int32_t n_tokens, void* stream,
                       int64_t* deferred = nullptr) {
  if (deferred) *deferred = -1;
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  if (n_tokens < 0) return fail(KVQ_E_ARG, "n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return ok();
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16)) return fail(KVQ_E_ARG, "k/v NULL or not 16-byte aligned");
  const int64_t n_new = h->n + n_tokens;
  if (n_new > h->cfg.max_tokens)
    return fail(KVQ_E_CAPACITY, "append of %d tokens to %lld exceeds max_tokens %d", n_tokens, (long long)h->n,
                h->cfg.max_tokens);
  const int G = h->cfg.group_size, S0 = h->cfg.sink_tokens;
  const int64_t nq_old = nquant_of(h, h->n), nq_new = nquant_of(h, n_new);
  kvq::AppendArgs a{};
  a.cache = h->buf;
  a.L = h->L;
  a.k = k;
  a.v = v;
  a.in_dtype = h->cfg.in_dtype;
  a.rotate = h->cfg.rotate;
  a.hybrid = h->cfg.hybrid;
  a.Hkv = h->cfg.num_kv_heads;
  a.T = n_tokens;
  a.n_old = h->n;
  a.g_first = nq_old / G;
  a.n_flush = (nq_new - nq_old) / G;
  // new tokens that stay fp16: the part of the sink [0, S0) they reach, and
  // the window [S0 + nq_new, n_new)
  a.s_first = h->n;
  a.n_sink_write = std::max<int64_t>(0, std::min<int64_t>(n_new, S0) - h->n);
  a.w_first = std::max<int64_t>(h->n, S0 + nq_new);
  a.n_write = std::max<int64_t>(0, n_new - a.w_first);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const kvq_config& c = h->cfg;
  const int64_t gf = a.g_first, gl = a.g_first + a.n_flush;
  if (c.adapt_delta > 0) {
    // bits of the groups quantized now, from their place in the n_new tokens
    for (int64_t g = gf; g < gl; ++g) {
      const int64_t p1 = S0 + g * G + G;  // one past the group's last token
      const int region = p1 > n_new - c.adapt_delta ? 2 : (p1 <= c.adapt_delta ? 0 : 1);
      h->gk[g] = static_cast<uint8_t>(region == 2 ? c.k_bits_high : region == 0 ? c.k_bits_low : c.k_bits);
      h->gv[g] = static_cast<uint8_t>(region == 2 ? c.v_bits_high : region == 0 ? c.v_bits_low : c.v_bits);
    }
  }
  // flush before the window write: the write may reuse ring slots the flush
  // reads; one launch per run of groups with equal bits
  hipError_t e = hipSuccess;
  for (const Run& r : runs_of(h, gf, gl)) {
    kvq::AppendArgs ar = a;
    ar.L = layout_for(h, r.kb, r.vb);
    ar.g_first = r.g0;
    ar.n_flush = r.g1 - r.g0;
    e = kvq::launch_flush(ar, s);
    if (e != hipSuccess) return device_error(h, e, "flush kernel launch");
  }
  if (deferred && n_tokens == 1 && !c.rotate && c.adapt_delta == 0 && a.n_sink_write == 0 && a.n_write == 1 &&
      a.w_first == h->n) {
    *deferred = h->n;
  } else {
    e = kvq::launch_window_write(a, s);
    if (e != hipSuccess) return device_error(h, e, "window write kernel launch");
  }
  h->n = n_new;
  return ok();
}

}  // namespace

extern "C" {

kvq_status kvq_append(kvq_cache* h, const void* k, const void* v, int32_t n_tokens, void* stream) {
  return append_impl(h, k, v, n_tokens, stream);
}

int32_t kvq_default_splits(const kvq_cache* h) {
  if (!h) return 0;
  return choose_splits(const_cast<kvq_cache*>(h), h->n);
}

namespace {

// How a decode of the cache's tokens is cut: the runs of groups with equal
// bits, their splits (or the piece table of a one-launch mixed decode), and
// whether the splits are merged inside the decode kernel.
struct SplitPlan {
  std::vector<Run> runs;
  bool mixed = false;
  kvq::MixedPlan pieces{};
  std::vector<int64_t> sp, gps;  // splits and groups per split of each run
  int64_t S = 0;                 // splits per slice
  int W = 0;                     // one run whose splits are merged in workgroups of W (0: none)
  int64_t slots = 0;             // partial records per row for the merge kernel (0: none)
};

// Arguments of every decode launch over the cache's current tokens.
kvq::DecodeArgs decode_args(const kvq_cache* h, const void* q, float* out, float* partials) {
  const kvq_config& c = h->cfg;
  kvq::DecodeArgs a{};
  a.cache = h->buf;
  a.q = q;
  a.in_dtype = c.in_dtype;
  a.rotate = c.rotate;
  a.gqa = c.num_q_heads / c.num_kv_heads;
  a.Hq = c.num_q_heads;
  a.Hkv = c.num_kv_heads;
  a.n = h->n;
  a.rc0 = (c.sink_tokens + nquant_of(h, h->n)) / kvq::kChunk;
  a.rc1 = std::max(a.rc0, (h->n + kvq::kChunk - 1) / kvq::kChunk);
  a.nsc = (std::min<int64_t>(h->n, c.sink_tokens) + kvq::kChunk - 1) / kvq::kChunk;
  a.partial = partials;
  a.out = out;
  return a;
}

// Validate a split count against the cache and plan the decode; allow_fused
// lets one run merge its splits in the decode kernel's workgroups: all of a
// slice's when it has 4 or 8, in groups of four when it has more (the count
// rounded up to a multiple of four, trailing splits possibly empty but no
// workgroup without groups, and the groups' records merged by the merge
// kernel); each when that launch fits as
// many waves per CU as the one-wave launch or all its workgroups at once
// (asked of the kernels once per bit widths, split count and group size).
kvq_status plan_splits(kvq_cache* h, int32_t num_splits, bool allow_fused, SplitPlan* p) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  if (h->n <= 0) return fail(KVQ_E_STATE, "decode on an empty cache");
  if (num_splits < 1) return fail(KVQ_E_ARG, "num_splits %d < 1", num_splits);
  if (num_splits > max_splits(&h->cfg))
    return fail(KVQ_E_ARG, "num_splits %d above the workspace maximum %d", num_splits, max_splits(&h->cfg));
  const kvq_config& c = h->cfg;
  const int64_t ng = ngroups_of(h);
  p->runs = runs_of(h, 0, ng);
  if (p->runs.empty()) p->runs.push_back({0, 0, c.k_bits, c.v_bits});
  if (static_cast<int64_t>(p->runs.size()) > max_splits(&c))
    return fail(KVQ_E_UNSUPPORTED, "%zu runs of equal bit widths exceed the split maximum %d", p->runs.size(),
                max_splits(&c));
  const std::vector<Run>& runs = p->runs;
  p->mixed = runs.size() > 1 && runs.size() <= static_cast<size_t>(kvq::kMaxRuns) &&
             plan_pieces(h, runs, std::min<int64_t>(num_splits, ng), &p->pieces);
  p->sp.assign(runs.size(), 1);
  p->gps.assign(runs.size(), 0);
  p->S = 0;
  p->W = 0;
  if (p->mixed) {
    p->S = p->pieces.npieces;
    p->slots = p->S;
    return ok();
  }
  if (ng > 0) p->sp = run_splits(h, runs, std::min<int64_t>(num_splits, ng));
  for (size_t i = 0; i < runs.size(); ++i) {
    const int64_t len = runs[i].g1 - runs[i].g0;
    if (len > 0) {
      p->gps[i] = (len + p->sp[i] - 1) / p->sp[i];
      p->sp[i] = (len + p->gps[i] - 1) / p->gps[i];  // no empty split
    }
    p->S += p->sp[i];
  }
  p->slots = p->S;
  if (allow_fused && runs.size() == 1) {
    if (fused_allowed(h, runs[0].kb, runs[0].vb, p->S, static_cast<int>(p->S))) {
      p->W = static_cast<int>(p->S);
      p->slots = 0;
    } else if (p->S > kvq::kMaxFusedSplits) {
      // every workgroup keeps some groups (trailing splits may be empty)
      const int64_t len = runs[0].g1 - runs[0].g0, S4 = (p->S + 3) / 4 * 4, gps = (len + S4 - 1) / S4;
      if (len > 0 && (len + gps - 1) / gps > S4 - 4 && fused_allowed(h, runs[0].kb, runs[0].vb, S4, 4)) {
        p->S = S4;
        p->sp[0] = S4;
        p->gps[0] = gps;
        p->W = 4;
        p->slots = S4 / 4;
      }
    }
  }
  return ok();
}

// Validate and launch the split kernels (one per run of groups with equal
// bits).  allow_final selects direct output when the whole decode is one
// split, or one run whose 4 or 8 splits per slice are merged inside the
// workgroup, and the grouped in-workgroup merge of more splits; *merged tells
// the caller that `out` is written (no merge left), else *records is the
// number of partial records per row the merge kernel reads.
using kvq::NewToken;
kvq_status launch_splits(kvq_cache* h, const void* q, float* out, float* partials, size_t bytes, int32_t num_splits,
                         bool allow_final, int32_t* records, bool* merged, hipStream_t s, bool noalloc = false,
                         NewToken nt = NewToken{}) {
  if (merged) *merged = false;
  SplitPlan p;
  kvq_status st = plan_splits(h, num_splits, allow_final, &p);
  if (st != KVQ_OK) return st;
  if (!q || !aligned(q, 16)) return fail(KVQ_E_ARG, "q NULL or not 16-byte aligned");
  const kvq_config& c = h->cfg;
  const int64_t rows = static_cast<int64_t>(c.batch) * c.num_q_heads;
  const int64_t S = p.S;
  const bool final = allow_final && (S == 1 || p.W == S);
  if (final) {
    if (!out || !aligned(out, 16)) return fail(KVQ_E_ARG, "out NULL or not 16-byte aligned");
  } else {
    size_t need = static_cast<size_t>(rows * p.slots * (c.head_dim + 4) * sizeof(float));
    if (noalloc && bytes < need)
      return fail(KVQ_E_ARG,
                  "this decode needs %zu bytes of split partials (%lld rows x %lld records), above the %zu-byte "
                  "no-allocation scratch; use kvq_decode_attn with a workspace",
                  need, (long long)rows, (long long)p.slots, bytes);
    if (!partials || !aligned(partials, 16) || bytes < need)
      return fail(KVQ_E_ARG, "workspace/partials NULL, misaligned or %zu < %zu bytes", bytes, need);
  }
  kvq::DecodeArgs a = decode_args(h, q, out, partials);
  a.write_final = final && p.W == 0 ? 1 : 0;
  a.splits_total = static_cast<int>(S);
  hipError_t e = hipSuccess;
  if (p.mixed) {
    a.L = h->L;
    e = kvq::launch_decode_mixed(a, p.pieces, s);
    if (e != hipSuccess) return device_error(h, e, "decode kernel launch");
  } else {
    // the fp16 chunks go with the run that has the most splits
    const size_t fp16_run = static_cast<size_t>(std::max_element(p.sp.begin(), p.sp.end()) - p.sp.begin());
    int64_t off = 0;
    for (size_t i = 0; i < p.runs.size(); ++i) {
      a.L = layout_for(h, p.runs[i].kb, p.runs[i].vb);
      a.g_base = p.runs[i].g0;
      a.ngroups = p.runs[i].g1 - p.runs[i].g0;
      a.splits = static_cast<int>(p.sp[i]);
      a.groups_per_split = p.gps[i];
      a.split_off = static_cast<int>(off);
      a.do_fp16 = i == fp16_run ? 1 : 0;
      e = p.W > 0 ? kvq::launch_decode_fused(a, nt, p.W, s) : kvq::launch_decode(a, nt, s);
      if (e != hipSuccess) return device_error(h, e, "decode kernel launch");
      off += p.sp[i];
    }
  }
  if (records) *records = static_cast<int32_t>(final ? 0 : p.slots);
  if (merged) *merged = final;
  return ok();
}

}  // namespace

kvq_status kvq_decode_attn_splits(kvq_cache* h, const void* q, float* out, void* ws, size_t ws_bytes,
                                  int32_t num_splits, void* stream) {
  if (!out || !aligned(out, 16)) return fail(KVQ_E_ARG, "out NULL or not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t S = 0;
  bool merged = false;
  kvq_status st = launch_splits(h, q, out, static_cast<float*>(ws), ws_bytes, num_splits, true, &S, &merged, s);
  if (st != KVQ_OK || merged) return st;
  const int64_t rows = static_cast<int64_t>(h->cfg.batch) * h->cfg.num_q_heads;
  hipError_t e = kvq::launch_merge(static_cast<float*>(ws), out, static_cast<int>(rows), S, h->cfg.head_dim, s);
  if (e != hipSuccess) return device_error(h, e, "merge kernel launch");
  return ok();
}

kvq_status kvq_decode_plan(kvq_cache* h, int32_t num_splits, int32_t* splits_used, int32_t* merge_records) {
  SplitPlan p;
  kvq_status st = plan_splits(h, num_splits, true, &p);
  if (st != KVQ_OK) return st;
  if (splits_used) *splits_used = static_cast<int32_t>(p.S);
  if (merge_records) *merge_records = p.S == 1 || p.W == p.S ? 0 : static_cast<int32_t>(p.slots);
  return ok();
}

kvq_status kvq_decode_partials(kvq_cache* h, const void* q, float* partials, size_t bytes, int32_t num_splits,
                               int32_t* splits_used, void* stream) {
  return launch_splits(h, q, nullptr, partials, bytes, num_splits, false, splits_used, nullptr,
                       static_cast<hipStream_t>(stream));
}

namespace {
// Append one token and decode.  Everything a launch could reject is checked
// before the first launch.
kvq_status append_decode(kvq_cache* h, const void* k, const void* v, const void* q, float* out, float* partials,
                         size_t bytes, int32_t num_splits, bool allow_final, int32_t* splits_used, bool* merged,
                         hipStream_t s) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  const kvq_config& c = h->cfg;
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16)) return fail(KVQ_E_ARG, "k/v NULL or not 16-byte aligned");
  if (!q || !aligned(q, 16)) return fail(KVQ_E_ARG, "q NULL or not 16-byte aligned");
  if (h->n + 1 > c.max_tokens) return fail(KVQ_E_CAPACITY, "append of 1 token to %lld exceeds max_tokens %d",
                                           (long long)h->n, c.max_tokens);
  if (num_splits < 1 || num_splits > max_splits(&c))
    return fail(KVQ_E_ARG, "num_splits %d outside [1, %d]", num_splits, max_splits(&c));
  const int64_t rows = static_cast<int64_t>(c.batch) * c.num_q_heads;
  const size_t need = static_cast<size_t>(rows * max_splits(&c) * (c.head_dim + 4) * sizeof(float));
  if (!partials || !aligned(partials, 16) || bytes < need)
    return fail(KVQ_E_ARG, "workspace/partials NULL, misaligned or %zu < %zu bytes", bytes, need);
  if (allow_final && (!out || !aligned(out, 16))) return fail(KVQ_E_ARG, "out NULL or not 16-byte aligned");
  if (static_cast<int64_t>(runs_of(h, 0, ngroups_of(h)).size()) + 1 > max_splits(&c))
    return fail(KVQ_E_UNSUPPORTED, "runs of equal bit widths exceed the split maximum %d", max_splits(&c));
  // the token's window write goes with the decode when it can (one launch
  // fewer per step); the decode below then must run, and everything it could
  // reject was checked above
  int64_t deferred = -1;
  st = append_impl(h, k, v, 1, s, &deferred);
  if (st != KVQ_OK) return st;
  NewToken nt;
  if (deferred >= 0) nt = NewToken{k, v, deferred};
  return launch_splits(h, q, out, partials, bytes, num_splits, allow_final, splits_used, merged, s, false, nt);
}
}  // namespace

kvq_status kvq_append_decode_attn(kvq_cache* h, const void* k, const void* v, const void* q, float* out, void* ws,
                                  size_t ws_bytes, void* stream) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t S_req = choose_splits(h, h->n + 1);  // as kvq_decode_attn after the append
  int32_t S = 0;
  bool merged = false;
  st = append_decode(h, k, v, q, out, static_cast<float*>(ws), ws_bytes, S_req, true, &S, &merged, s);
  if (st != KVQ_OK || merged) return st;
  const int64_t rows = static_cast<int64_t>(h->cfg.batch) * h->cfg.num_q_heads;
  hipError_t e = kvq::launch_merge(static_cast<float*>(ws), out, static_cast<int>(rows), S, h->cfg.head_dim, s);
  if (e != hipSuccess) return device_error(h, e, "merge kernel launch");
  return ok();
}

kvq_status kvq_append_decode_partials(kvq_cache* h, const void* k, const void* v, const void* q, float* partials,
                                      size_t bytes, int32_t num_splits, int32_t* splits_used, void* stream) {
  return append_decode(h, k, v, q, nullptr, partials, bytes, num_splits, false, splits_used, nullptr,
                       static_cast<hipStream_t>(stream));
}

kvq_status kvq_merge_partials(const float* partials, float* out, int32_t rows, int32_t splits, int32_t head_dim,
                              void* stream) {
  if (!partials || !out || !aligned(partials, 16) || !aligned(out, 16))
    return fail(KVQ_E_ARG, "partials/out NULL or not 16-byte aligned");
  if (rows < 1 || splits < 1) return fail(KVQ_E_ARG, "rows and splits must be positive");
  if (splits > 256) return fail(KVQ_E_ARG, "splits %d above 256", splits);
  if (head_dim != 64 && head_dim != 128) return fail(KVQ_E_UNSUPPORTED, "head_dim %d not in {64,128}", head_dim);
  hipError_t e = kvq::launch_merge(partials, out, rows, splits, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVQ_E_DEVICE, "merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

kvq_status kvq_decode_attn(kvq_cache* h, const void* q, float* out, void* ws, size_t ws_bytes, void* stream) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  return kvq_decode_attn_splits(h, q, out, ws, ws_bytes, choose_splits(h, h->n), stream);
}

kvq_status kvq_decode_attn_noalloc(kvq_cache* h, const void* q, float* out, void* stream) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  if (!out || !aligned(out, 16)) return fail(KVQ_E_ARG, "out NULL or not 16-byte aligned");
  void* scratch = nullptr;
  hipError_t e = kvq::noalloc_scratch(&scratch);
  if (e != hipSuccess) return fail(KVQ_E_DEVICE, "no-allocation scratch address: %s", hipGetErrorString(e));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t S = 0;
  bool merged = false;
  st = launch_splits(h, q, out, static_cast<float*>(scratch), kvq::kNoallocScratchBytes, choose_splits(h, h->n), true,
                     &S, &merged, s, true);
  if (st != KVQ_OK || merged) return st;
  const int64_t rows = static_cast<int64_t>(h->cfg.batch) * h->cfg.num_q_heads;
  e = kvq::launch_merge(static_cast<const float*>(scratch), out, static_cast<int>(rows), S, h->cfg.head_dim, s);
  if (e != hipSuccess) return device_error(h, e, "merge kernel launch");
  return ok();
}

// ---------------------------------------------------------------- drift detection

namespace {
kvq_status drift_common(kvq_cache* h, int64_t g0, int64_t g1, kvq::DriftArgs* a) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  if (h->cfg.adapt_delta > 0) return fail(KVQ_E_UNSUPPORTED, "drift detection on a position-adaptive cache");
  const int64_t ng = ngroups_of(h);
  if (g0 < 0 || g1 < g0 || g1 > ng)
    return fail(KVQ_E_ARG, "group range [%lld, %lld) outside the %lld quantized groups", (long long)g0, (long long)g1,
                (long long)ng);
  *a = kvq::DriftArgs{};
  a->cache = h->buf;
  a->L = h->L;
  a->Hkv = h->cfg.num_kv_heads;
  a->g0 = g0;
  a->ng = g1 - g0;
  return KVQ_OK;
}
}  // namespace

kvq_status kvq_code_histograms(kvq_cache* h, int64_t g0, int64_t g1, uint64_t* k_hist, uint64_t* v_hist,
                               void* stream) {
  kvq::DriftArgs a;
  kvq_status st = drift_common(h, g0, g1, &a);
  if (st != KVQ_OK) return st;
  if (!k_hist || !v_hist || !aligned(k_hist, 8) || !aligned(v_hist, 8))
    return fail(KVQ_E_ARG, "histogram arrays NULL or not 8-byte aligned");
  a.hist_k = k_hist;
  a.hist_v = v_hist;
  hipError_t e = kvq::launch_code_histograms(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(h, e, "histogram kernel launch");
  return ok();
}

kvq_status kvq_drift_check(kvq_cache* h, int64_t g0, int64_t g1, const uint64_t* cal_k, const uint64_t* cal_v,
                           double threshold, double* kl_k, double* kl_v, uint8_t* flags, void* stream) {
  kvq::DriftArgs a;
  kvq_status st = drift_common(h, g0, g1, &a);
  if (st != KVQ_OK) return st;
  if (!cal_k || !cal_v || !kl_k || !kl_v || !flags || !aligned(cal_k, 8) || !aligned(cal_v, 8) || !aligned(kl_k, 8) ||
      !aligned(kl_v, 8))
    return fail(KVQ_E_ARG, "drift arrays NULL or not 8-byte aligned");
  if (!(threshold >= 0.0)) return fail(KVQ_E_ARG, "threshold must be >= 0");
  a.cal_k = cal_k;
  a.cal_v = cal_v;
  a.threshold = threshold;
  a.kl_k = kl_k;
  a.kl_v = kl_v;
  a.flags = flags;
  hipError_t e = kvq::launch_drift_check(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(h, e, "drift kernel launch");
  return ok();
}

kvq_status kvq_requantize(kvq_cache* h, int64_t g0, int64_t g1, const void* k, const void* v, const uint8_t* flags,
                          void* stream) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  const int64_t ng = ngroups_of(h);
  if (g0 < 0 || g1 < g0 || g1 > ng)
    return fail(KVQ_E_ARG, "group range [%lld, %lld) outside the %lld quantized groups", (long long)g0, (long long)g1,
                (long long)ng);
  if (g1 == g0) return ok();
  if (!k || !v || !aligned(k, 16) || !aligned(v, 16)) return fail(KVQ_E_ARG, "k/v NULL or not 16-byte aligned");
  const int G = h->cfg.group_size;
  kvq::AppendArgs a{};
  a.cache = h->buf;
  a.k = k;
  a.v = v;
  a.in_dtype = h->cfg.in_dtype;
  a.rotate = h->cfg.rotate;
  a.hybrid = h->cfg.hybrid;
  a.Hkv = h->cfg.num_kv_heads;
  a.T = (g1 - g0) * G;
  a.n_old = h->cfg.sink_tokens + g0 * G;  // every token of the range comes from k, v
  a.flags = flags;
  a.flag_g0 = g0;
  a.flag_stride = g1 - g0;
  for (const Run& r : runs_of(h, g0, g1)) {
    a.L = layout_for(h, r.kb, r.vb);
    a.g_first = r.g0;
    a.n_flush = r.g1 - r.g0;
    hipError_t e = kvq::launch_flush(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_error(h, e, "requantize kernel launch");
  }
  return ok();
}

// ---------------------------------------------------------------- export / import

}  // extern "C"

namespace {
// Runs fn(bi, hk, pages, ring, sink) for every (batch row bi < bc, kv head hk)
// on up to 16 host threads, each with its own staging buffers of the given
// sizes; returns the first device error any slice met (hipSuccess if none).
template <typename F>
hipError_t for_each_slice(int64_t bc, int64_t hkv, size_t page_bytes, size_t ring_bytes, size_t sink_bytes, F& fn) {
  const int64_t total = bc * hkv;
  const int64_t hw = std::max<int64_t>(1, std::thread::hardware_concurrency());
  const int64_t nt = std::max<int64_t>(1, std::min<int64_t>({16, hw, total}));
  std::atomic<int64_t> next{0};
  std::atomic<int> err{static_cast<int>(hipSuccess)};
  auto work = [&]() {
    std::vector<uint8_t> pages(page_bytes), ring(ring_bytes), sink(sink_bytes);
    for (int64_t i = next++; i < total; i = next++) {
      if (err.load() != static_cast<int>(hipSuccess)) return;
      const hipError_t e = fn(i / hkv, i % hkv, pages, ring, sink);
      if (e != hipSuccess) err.store(static_cast<int>(e));
    }
  };
  std::vector<std::thread> th;
  for (int64_t t = 1; t < nt; ++t) th.emplace_back(work);
  work();
  for (auto& t : th) t.join();
  return static_cast<hipError_t>(err.load());
}
}  // namespace

extern "C" {


kvq_status kvq_export(kvq_cache* h, int32_t b0, int32_t bc, void* k_codes, void* k_scale, void* k_zero,
                      void* v_codes, void* v_scale, void* v_zero, void* k_resid, void* v_resid, void* stream) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  const kvq_config& c = h->cfg;
  if (b0 < 0 || bc < 0 || b0 + bc > c.batch) return fail(KVQ_E_ARG, "batch range [%d, %d) out of [0, %d)", b0, b0 + bc, c.batch);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(h, e, "stream synchronize");
  if (c.adapt_delta > 0 && (k_codes || v_codes))
    return fail(KVQ_E_UNSUPPORTED, "packed code export needs one bit width; use kvq_export_codes_u8");
  const Layout& L = h->L;
  const int D = c.head_dim, G = c.group_size, kb = c.k_bits, vb = c.v_bits, ncg = D / G;
  const int64_t nq = nquant_of(h, h->n), nr = h->n - nq, ng = nq / G;
  const int64_t ns = std::min<int64_t>(h->n, c.sink_tokens);  // fp16 index r < ns: sink token r
  const int64_t krow = D * kb / 8, vrow = D * vb / 8;
  const std::vector<Layout> GL = group_layouts(h, ng);
  // one slice: copy its pages, window ring and sink to host buffers and
  // write its canonical rows (slices are independent: threads take them in turn)
  auto one = [&](int64_t bi, int64_t hk, std::vector<uint8_t>& pages, std::vector<uint8_t>& ring,
                 std::vector<uint8_t>& sink) -> hipError_t {
      hipError_t e = hipSuccess;
      const int64_t slice = (b0 + bi) * c.num_kv_heads + hk;
      const int64_t oi = bi * c.num_kv_heads + hk;  // output slice index
      if (ng > 0) {
        e = hipMemcpy(pages.data(), h->buf + kvq::page_offset(L, slice, 0), pages.size(), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return e;
      }
      e = hipMemcpy(ring.data(), h->buf + L.ring_offset + slice * L.ring_chunks * L.ring_chunk_bytes, ring.size(),
                    hipMemcpyDeviceToHost);
      if (e != hipSuccess) return e;
      if (!sink.empty()) {
        e = hipMemcpy(sink.data(), h->buf + L.sink_offset + slice * L.sink_chunks * L.ring_chunk_bytes, sink.size(),
                      hipMemcpyDeviceToHost);
        if (e != hipSuccess) return e;
      }
      for (int64_t t = 0; t < nq; ++t) {
        const uint8_t* page = pages.data() + (t / G) * L.page_bytes;
        const Layout& PL = GL[t / G];
        const int ch = static_cast<int>((t % G) / kvq::kChunk), tt = static_cast<int>(t % kvq::kChunk);
        if (k_codes) {
          uint8_t* row = static_cast<uint8_t*>(k_codes) + (oi * nq + t) * krow;
          std::memset(row, 0, static_cast<size_t>(krow));
          for (int cc = 0; cc < D; ++cc) {
            int64_t byte; int bit;
            kvq::kcode_loc(L, tt, cc, &byte, &bit);
            uint32_t w;
            std::memcpy(&w, page + L.off_kcodes + ch * L.kc_chunk_bytes + byte, 4);
            uint32_t code = (w >> bit) & ((1u << kb) - 1u);
            row[(cc * kb) / 8] |= static_cast<uint8_t>(code << ((cc * kb) % 8));
          }
        }
        if (v_codes) {
          uint8_t* row = static_cast<uint8_t*>(v_codes) + (oi * nq + t) * vrow;
          std::memset(row, 0, static_cast<size_t>(vrow));
          for (int cc = 0; cc < D; ++cc) {
            int64_t byte; int bit;
            kvq::vcode_loc(L, tt, cc, &byte, &bit);
            uint32_t w;
            std::memcpy(&w, page + L.off_vcodes + ch * L.vc_chunk_bytes + byte, 4);
            uint32_t code = (w >> bit) & ((1u << vb) - 1u);
            row[(cc * vb) / 8] |= static_cast<uint8_t>(code << ((cc * vb) % 8));
          }
        }
        for (int cg = 0; cg < ncg; ++cg) {
          const uint16_t* vpp = reinterpret_cast<const uint16_t*>(page + PL.off_vparams + ch * PL.vp_chunk_bytes);
          if (v_scale) static_cast<uint16_t*>(v_scale)[(oi * nq + t) * ncg + cg] = vpp[kvq::vparam_scale_elem(PL, tt, cg)];
          if (v_zero) static_cast<uint16_t*>(v_zero)[(oi * nq + t) * ncg + cg] = vpp[kvq::vparam_zero_elem(PL, tt, cg)];
        }
      }
      for (int64_t g = 0; g < ng; ++g) {
        const uint16_t* kp = reinterpret_cast<const uint16_t*>(pages.data() + g * L.page_bytes + GL[g].off_kparams);
        for (int cc = 0; cc < D; ++cc) {
          int pi = kvq::kparam_index(GL[g], cc);
          if (k_scale) static_cast<uint16_t*>(k_scale)[(oi * ng + g) * D + cc] = kp[pi];
          if (k_zero) static_cast<uint16_t*>(k_zero)[(oi * ng + g) * D + cc] = kp[D + pi];
        }
      }
      for (int64_t t = 0; t < nr; ++t) {
        const int64_t pos = t < ns ? t : c.sink_tokens + nq + (t - ns);
        const uint8_t* rc = pos < c.sink_tokens
                                ? sink.data() + (pos / kvq::kChunk) * L.ring_chunk_bytes
                                : ring.data() + ((pos / kvq::kChunk) % L.ring_chunks) * L.ring_chunk_bytes;
        const int tt = static_cast<int>(pos % kvq::kChunk);
        for (int cc = 0; cc < D; ++cc) {
          uint16_t kvb, vvb;
          std::memcpy(&kvb, rc + kvq::ring_k_offset(L, tt, cc), 2);
          std::memcpy(&vvb, rc + kvq::ring_v_offset(L, tt, cc), 2);
          if (k_resid) static_cast<uint16_t*>(k_resid)[(oi * nr + t) * D + cc] = kvb;
          if (v_resid) static_cast<uint16_t*>(v_resid)[(oi * nr + t) * D + cc] = vvb;
        }
      }
      return hipSuccess;
  };
  e = for_each_slice(bc, c.num_kv_heads, static_cast<size_t>(ng * L.page_bytes),
                     static_cast<size_t>(L.ring_chunks * L.ring_chunk_bytes),
                     static_cast<size_t>(L.sink_chunks * L.ring_chunk_bytes), one);
  if (e != hipSuccess) return device_error(h, e, "export copy");
  return ok();
}

kvq_status kvq_export_codes_u8(kvq_cache* h, int32_t b0, int32_t bc, void* k_codes, void* v_codes, void* stream) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  const kvq_config& c = h->cfg;
  if (b0 < 0 || bc < 0 || b0 + bc > c.batch) return fail(KVQ_E_ARG, "batch range out of bounds");
  if (!k_codes && !v_codes) return fail(KVQ_E_ARG, "code arrays are NULL");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(h, e, "stream synchronize");
  const Layout& L = h->L;
  const int D = c.head_dim, G = c.group_size;
  const int64_t nq = nquant_of(h, h->n), ng = nq / G;
  const std::vector<Layout> GL = group_layouts(h, ng);
  std::vector<uint8_t> pages(static_cast<size_t>(ng * L.page_bytes));
  for (int64_t bi = 0; bi < bc; ++bi)
    for (int64_t hk = 0; hk < c.num_kv_heads; ++hk) {
      if (ng == 0) continue;
      const int64_t slice = (b0 + bi) * c.num_kv_heads + hk;
      const int64_t oi = bi * c.num_kv_heads + hk;
      e = hipMemcpy(pages.data(), h->buf + kvq::page_offset(L, slice, 0), pages.size(), hipMemcpyDeviceToHost);
      if (e != hipSuccess) return device_error(h, e, "export copy");
      for (int64_t t = 0; t < nq; ++t) {
        const uint8_t* page = pages.data() + (t / G) * L.page_bytes;
        const Layout& PL = GL[t / G];
        const int ch = static_cast<int>((t % G) / kvq::kChunk), tt = static_cast<int>(t % kvq::kChunk);
        for (int cc = 0; cc < D; ++cc) {
          int64_t byte; int bit; uint32_t w;
          if (k_codes) {
            kvq::kcode_loc(PL, tt, cc, &byte, &bit);
            std::memcpy(&w, page + PL.off_kcodes + ch * PL.kc_chunk_bytes + byte, 4);
            static_cast<uint8_t*>(k_codes)[(oi * nq + t) * D + cc] = static_cast<uint8_t>((w >> bit) & ((1u << PL.kbits) - 1u));
          }
          if (v_codes) {
            kvq::vcode_loc(PL, tt, cc, &byte, &bit);
            std::memcpy(&w, page + PL.off_vcodes + ch * PL.vc_chunk_bytes + byte, 4);
            static_cast<uint8_t*>(v_codes)[(oi * nq + t) * D + cc] = static_cast<uint8_t>((w >> bit) & ((1u << PL.vbits) - 1u));
          }
        }
      }
    }
  return ok();
}

int64_t kvq_group_bits(const kvq_cache* h, uint8_t* k_bits, uint8_t* v_bits, int64_t cap) {
  if (!h) return -1;
  const int64_t ng = ngroups_of(h);
  for (int64_t g = 0; g < std::min(ng, cap); ++g) {
    if (k_bits) k_bits[g] = h->gk[g];
    if (v_bits) v_bits[g] = h->gv[g];
  }
  return ng;
}

// Key token norms live in each page's norm block, one 64-byte block per chunk.
static kvq_status key_norms_copy(kvq_cache* h, int32_t b0, int32_t bc, void* out, const void* in, void* stream) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  const kvq_config& c = h->cfg;
  if (!c.token_norm) return fail(KVQ_E_STATE, "the cache has no key token norms (token_norm = 0)");
  if (b0 < 0 || bc < 0 || b0 + bc > c.batch) return fail(KVQ_E_ARG, "batch range out of bounds");
  if (!out && !in) return fail(KVQ_E_ARG, "norm array is NULL");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(h, e, "stream synchronize");
  const Layout& L = h->L;
  const int G = c.group_size;
  const int64_t nq = nquant_of(h, h->n), ng = nq / G;
  const std::vector<Layout> GL = group_layouts(h, ng);
  std::vector<uint8_t> pages(static_cast<size_t>(ng * L.page_bytes));
  for (int64_t bi = 0; bi < bc; ++bi)
    for (int64_t hk = 0; hk < c.num_kv_heads; ++hk) {
      const int64_t slice = (b0 + bi) * c.num_kv_heads + hk;
      const int64_t oi = bi * c.num_kv_heads + hk;
      if (ng == 0) continue;
      e = hipMemcpy(pages.data(), h->buf + kvq::page_offset(L, slice, 0), pages.size(), hipMemcpyDeviceToHost);
      if (e != hipSuccess) return device_error(h, e, "key norm copy");
      for (int64_t t = 0; t < nq; ++t) {
        const Layout& PL = GL[t / G];
        uint16_t* kn = reinterpret_cast<uint16_t*>(pages.data() + (t / G) * L.page_bytes + PL.off_knorm +
                                                   ((t % G) / kvq::kChunk) * PL.kn_chunk_bytes);
        const int el = kvq::knorm_elem(static_cast<int>(t % kvq::kChunk));
        if (out) static_cast<uint16_t*>(out)[oi * nq + t] = kn[el];
        else kn[el] = static_cast<const uint16_t*>(in)[oi * nq + t];
      }
      if (in) {
        e = hipMemcpy(h->buf + kvq::page_offset(L, slice, 0), pages.data(), pages.size(), hipMemcpyHostToDevice);
        if (e != hipSuccess) return device_error(h, e, "key norm copy");
      }
    }
  return ok();
}

kvq_status kvq_export_key_norms(kvq_cache* h, int32_t b0, int32_t bc, void* host_k_norm, void* stream) {
  if (!host_k_norm) return fail(KVQ_E_ARG, "norm array is NULL");
  return key_norms_copy(h, b0, bc, host_k_norm, nullptr, stream);
}

kvq_status kvq_import_key_norms(kvq_cache* h, int32_t b0, int32_t bc, const void* host_k_norm, void* stream) {
  if (!host_k_norm) return fail(KVQ_E_ARG, "norm array is NULL");
  return key_norms_copy(h, b0, bc, nullptr, host_k_norm, stream);
}

kvq_status kvq_import(kvq_cache* h, int64_t n_tokens, int32_t b0, int32_t bc, const void* k_codes,
                      const void* k_scale, const void* k_zero, const void* v_codes, const void* v_scale,
                      const void* v_zero, const void* k_resid, const void* v_resid, void* stream) {
  kvq_status st = check_handle(h);
  if (st != KVQ_OK) return st;
  const kvq_config& c = h->cfg;
  if (n_tokens < 0) return fail(KVQ_E_ARG, "n_tokens < 0");
  if (n_tokens > c.max_tokens) return fail(KVQ_E_CAPACITY, "n_tokens %lld > max_tokens %d", (long long)n_tokens, c.max_tokens);
  if (b0 < 0 || bc < 0 || b0 + bc > c.batch) return fail(KVQ_E_ARG, "batch range out of bounds");
  if (!k_codes || !k_scale || !k_zero || !v_codes || !v_scale || !v_zero || !k_resid || !v_resid)
    return fail(KVQ_E_ARG, "import arrays must not be NULL");
  if (c.adapt_delta > 0) return fail(KVQ_E_UNSUPPORTED, "import into a position-adaptive cache");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(h, e, "stream synchronize");
  const Layout& L = h->L;
  const int D = c.head_dim, G = c.group_size, kb = c.k_bits, vb = c.v_bits, ncg = D / G;
  const int64_t nq = nquant_of(h, n_tokens), nr = n_tokens - nq, ng = nq / G;
  const int64_t ns = std::min<int64_t>(n_tokens, c.sink_tokens);
  const int64_t krow = D * kb / 8, vrow = D * vb / 8;
  std::vector<uint8_t> pages(static_cast<size_t>(ng * L.page_bytes));
  std::vector<uint8_t> ring(static_cast<size_t>(L.ring_chunks * L.ring_chunk_bytes));
  std::vector<uint8_t> sink(static_cast<size_t>(L.sink_chunks * L.ring_chunk_bytes));
  for (int64_t bi = 0; bi < bc; ++bi)
    for (int64_t hk = 0; hk < c.num_kv_heads; ++hk) {
      const int64_t slice = (b0 + bi) * c.num_kv_heads + hk;
      const int64_t oi = bi * c.num_kv_heads + hk;
      std::fill(pages.begin(), pages.end(), 0);
      std::fill(ring.begin(), ring.end(), 0);
      std::fill(sink.begin(), sink.end(), 0);
      for (int64_t t = 0; t < nq; ++t) {
        uint8_t* page = pages.data() + (t / G) * L.page_bytes;
        const int ch = static_cast<int>((t % G) / kvq::kChunk), tt = static_cast<int>(t % kvq::kChunk);
        const uint8_t* krw = static_cast<const uint8_t*>(k_codes) + (oi * nq + t) * krow;
        const uint8_t* vrw = static_cast<const uint8_t*>(v_codes) + (oi * nq + t) * vrow;
        for (int cc = 0; cc < D; ++cc) {
          int64_t byte; int bit; uint32_t w;
          uint32_t code = (krw[(cc * kb) / 8] >> ((cc * kb) % 8)) & ((1u << kb) - 1u);
          kvq::kcode_loc(L, tt, cc, &byte, &bit);
          uint8_t* dst = page + L.off_kcodes + ch * L.kc_chunk_bytes + byte;
          std::memcpy(&w, dst, 4); w |= code << bit; std::memcpy(dst, &w, 4);
          code = (vrw[(cc * vb) / 8] >> ((cc * vb) % 8)) & ((1u << vb) - 1u);
          kvq::vcode_loc(L, tt, cc, &byte, &bit);
          dst = page + L.off_vcodes + ch * L.vc_chunk_bytes + byte;
          std::memcpy(&w, dst, 4); w |= code << bit; std::memcpy(dst, &w, 4);
        }
        for (int cg = 0; cg < ncg; ++cg) {
          uint16_t* vpp = reinterpret_cast<uint16_t*>(page + L.off_vparams + ch * L.vp_chunk_bytes);
          vpp[kvq::vparam_scale_elem(L, tt, cg)] = static_cast<const uint16_t*>(v_scale)[(oi * nq + t) * ncg + cg];
          vpp[kvq::vparam_zero_elem(L, tt, cg)] = static_cast<const uint16_t*>(v_zero)[(oi * nq + t) * ncg + cg];
        }
      }
      for (int64_t g = 0; g < ng; ++g) {
        uint16_t* kp = reinterpret_cast<uint16_t*>(pages.data() + g * L.page_bytes + L.off_kparams);
        for (int cc = 0; cc < D; ++cc) {
          int pi = kvq::kparam_index(L, cc);
          kp[pi] = static_cast<const uint16_t*>(k_scale)[(oi * ng + g) * D + cc];
          kp[D + pi] = static_cast<const uint16_t*>(k_zero)[(oi * ng + g) * D + cc];
        }
      }
      for (int64_t t = 0; t < nr; ++t) {
        const int64_t pos = t < ns ? t : c.sink_tokens + nq + (t - ns);
        uint8_t* rc = pos < c.sink_tokens ? sink.data() + (pos / kvq::kChunk) * L.ring_chunk_bytes
                                          : ring.data() + ((pos / kvq::kChunk) % L.ring_chunks) * L.ring_chunk_bytes;
        const int tt = static_cast<int>(pos % kvq::kChunk);
        for (int cc = 0; cc < D; ++cc) {
          std::memcpy(rc + kvq::ring_k_offset(L, tt, cc), static_cast<const uint16_t*>(k_resid) + (oi * nr + t) * D + cc, 2);
          std::memcpy(rc + kvq::ring_v_offset(L, tt, cc), static_cast<const uint16_t*>(v_resid) + (oi * nr + t) * D + cc, 2);
        }
      }
      if (ng > 0) {
        e = hipMemcpy(h->buf + kvq::page_offset(L, slice, 0), pages.data(), pages.size(), hipMemcpyHostToDevice);
        if (e != hipSuccess) return device_error(h, e, "import copy");
      }
      e = hipMemcpy(h->buf + L.ring_offset + slice * L.ring_chunks * L.ring_chunk_bytes, ring.data(), ring.size(),
                    hipMemcpyHostToDevice);
      if (e != hipSuccess) return device_error(h, e, "import copy");
      if (!sink.empty()) {
        e = hipMemcpy(h->buf + L.sink_offset + slice * L.sink_chunks * L.ring_chunk_bytes, sink.data(), sink.size(),
                      hipMemcpyHostToDevice);
        if (e != hipSuccess) return device_error(h, e, "import copy");
      }
    }
  h->n = n_tokens;
  return ok();
}

}  // extern "C"
