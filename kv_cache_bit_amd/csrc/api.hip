// api.hip -- extern "C" entry points of libnsnq: host-side validation, launch
// configuration and counter bookkeeping.  Every check runs before any HIP
// call, so a rejected call touches neither the GPU nor the cache.

#include <atomic>

#include "../../include/nsnq.h"
#include "nsnq_device.hpp"
#include "nsnq_launch.hpp"

namespace nsnq {
hipError_t launch_kmeans_clear(double* acc, int n, hipStream_t stream);
}

using namespace nsnq;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

nsnq_status check_params(const nsnq_params* p) {
  if (!p) return NSNQ_EINVAL;
  if (p->bits != 1 && p->bits != 2) return NSNQ_EINVAL;
  if (p->n_codewords != 256 || p->head_dim <= 0 || p->block_tokens <= 0) return NSNQ_EINVAL;
  if (p->head_dim != 128) return NSNQ_EUNSUPPORTED;
  if (p->block_tokens != 64 && p->block_tokens != 128) return NSNQ_EUNSUPPORTED;
  if ((p->flags & ~(NSNQ_SCALE_ADJUST | NSNQ_DOUBLE_QUANT)) != 0) return NSNQ_EINVAL;
  if (p->vq_candidates == nullptr) {
    if (p->vq_span != 0) return NSNQ_EINVAL;
  } else if (p->bits != 2 || p->vq_span < 16 || p->vq_span > 128 || p->vq_span % 16 != 0 ||
             !aligned16(p->vq_candidates)) {
    return NSNQ_EINVAL;
  }
  return NSNQ_OK;
}

int sub_of(const nsnq_params* p) { return p->bits == 2 ? 4 : 8; }

nsnq_status check_kv(const nsnq_kv& kv) {
  if (!kv.codes || !kv.scales || !kv.mu || !kv.resid) return NSNQ_EINVAL;
  if (!aligned16(kv.codes) || !aligned16(kv.scales) || !aligned16(kv.mu) || !aligned16(kv.resid))
    return NSNQ_EINVAL;
  return NSNQ_OK;
}

nsnq_status check_cache(const nsnq_params* p, const nsnq_cache* c) {
  if (!c) return NSNQ_EINVAL;
  if (c->batch <= 0 || c->kv_heads <= 0 || c->cap_tokens <= 0) return NSNQ_EINVAL;
  if (c->cap_tokens % p->block_tokens != 0) return NSNQ_EINVAL;
  if (c->n_quant < 0 || c->n_quant % p->block_tokens != 0 || c->n_quant > c->cap_tokens) return NSNQ_EINVAL;
  if (c->n_resid < 0 || c->n_resid > p->block_tokens) return NSNQ_EINVAL;
  if ((int64_t)c->batch * c->kv_heads * c->cap_tokens > (int64_t)1 << 40) return NSNQ_EINVAL;
  if ((c->seq_quant == nullptr) != (c->seq_resid == nullptr)) return NSNQ_EINVAL;
  if (c->seq_quant && ((((uintptr_t)c->seq_quant) & 3u) || (((uintptr_t)c->seq_resid) & 3u))) return NSNQ_EINVAL;
  if (c->seq_quant && c->max_len < 0) return NSNQ_EINVAL;
  nsnq_status s = check_kv(c->k);
  if (s != NSNQ_OK) return s;
  return check_kv(c->v);
}

nsnq_status hip_status(hipError_t e) { return e == hipSuccess ? NSNQ_OK : NSNQ_EHIP; }

// One launch: encode `nblk` blocks per stream from src (strides given) to
// token n_quant, and copy `rc_r` tokens starting at source token `rc_t0` into
// the residual window.
nsnq_status run_encode(const nsnq_params* p, const uint16_t* cb, const uint16_t* k, const uint16_t* v,
                       int64_t sb, int64_t sh, int64_t st, int nblk, int rc_t0, int rc_r, const nsnq_cache* c,
                       hipStream_t stream) {
  if (nblk <= 0 && rc_r <= 0) return NSNQ_OK;
  EncodeArgs a{};
  a.src[0] = k;
  a.src[1] = v;
  a.sb = sb;
  a.sh = sh;
  a.st = st;
  a.codes[0] = c->k.codes;
  a.codes[1] = c->v.codes;
  a.scales[0] = c->k.scales;
  a.scales[1] = c->v.scales;
  a.mu[0] = c->k.mu;
  a.mu[1] = c->v.mu;
  a.resid[0] = c->k.resid;
  a.resid[1] = c->v.resid;
  a.codebook = cb;
  a.H = c->kv_heads;
  a.n_units = c->batch * c->kv_heads;
  a.cap = c->cap_tokens;
  a.dst_tok0 = c->n_quant;
  a.nblk = nblk > 0 ? nblk : 0;
  a.R = p->block_tokens;
  a.rc_t0 = rc_t0;
  a.rc_r = rc_r;
  a.signs = p->hadamard_signs;
  a.scale_adjust = (p->flags & NSNQ_SCALE_ADJUST) ? 1 : 0;
  a.dq = (p->flags & NSNQ_DOUBLE_QUANT) ? 1 : 0;
  a.cand = p->vq_candidates;
  a.span = p->vq_candidates ? p->vq_span : 0;
  return hip_status(launch_encode(a, sub_of(p), p->block_tokens, stream));
}

bool is_ragged(const nsnq_cache* c) { return c->seq_quant != nullptr; }

// Host bounds of a ragged cache from its length bound.
int64_t ragged_quant_bound(int64_t max_len, int R) { return max_len / R * R; }
void set_ragged_bounds(nsnq_cache* c, int max_len, int R) {
  c->max_len = max_len;
  c->n_quant = (int32_t)ragged_quant_bound(max_len, R);
  c->n_resid = max_len < R ? max_len : R;
}

// Ragged flush: one launch over every row's window; rows that are not full
// exit at once.
nsnq_status run_ragged_flush(const nsnq_params* p, const uint16_t* cb, const nsnq_cache* c, hipStream_t stream) {
  const int R = p->block_tokens;
  const int64_t st = p->head_dim, sh = (int64_t)R * p->head_dim, sb = sh * c->kv_heads;
  EncodeArgs a{};
  a.src[0] = c->k.resid;
  a.src[1] = c->v.resid;
  a.sb = sb;
  a.sh = sh;
  a.st = st;
  a.codes[0] = c->k.codes;
  a.codes[1] = c->v.codes;
  a.scales[0] = c->k.scales;
  a.scales[1] = c->v.scales;
  a.mu[0] = c->k.mu;
  a.mu[1] = c->v.mu;
  a.resid[0] = c->k.resid;
  a.resid[1] = c->v.resid;
  a.codebook = cb;
  a.H = c->kv_heads;
  a.n_units = c->batch * c->kv_heads;
  a.cap = c->cap_tokens;
  a.nblk = 1;
  a.R = R;
  a.signs = p->hadamard_signs;
  a.scale_adjust = (p->flags & NSNQ_SCALE_ADJUST) ? 1 : 0;
  a.dq = (p->flags & NSNQ_DOUBLE_QUANT) ? 1 : 0;
  a.cand = p->vq_candidates;
  a.span = p->vq_candidates ? p->vq_span : 0;
  a.fl_quant = c->seq_quant;
  a.fl_resid = c->seq_resid;
  return hip_status(launch_encode(a, sub_of(p), R, stream));
}

}  // namespace

extern "C" {

int32_t nsnq_abi_version(void) { return NSNQ_ABI_VERSION; }

const char* nsnq_status_str(nsnq_status st) {
  switch (st) {
    case NSNQ_OK: return "ok";
    case NSNQ_EINVAL: return "invalid argument";
    case NSNQ_EUNSUPPORTED: return "unsupported parameters";
    case NSNQ_EHIP: return "HIP runtime error";
    case NSNQ_EWORKSPACE: return "workspace missing or too small";
    case NSNQ_ESCRATCH: return "call needs more than the library's static scratch (NSNQ_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

nsnq_status nsnq_buffer_bytes(const nsnq_params* p, int32_t cap_tokens, size_t* codes, size_t* scales, size_t* mu,
                              size_t* resid) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  const int R = p->block_tokens;
  if (cap_tokens < 0 || cap_tokens % R != 0 || !codes || !scales || !mu || !resid) return NSNQ_EINVAL;
  const size_t nb = (size_t)(cap_tokens / R);
  *codes = (size_t)cap_tokens * (p->head_dim / sub_of(p));
  if (p->flags & NSNQ_DOUBLE_QUANT) {
    *scales = nb * (size_t)(((2 * R + R / 2 + 4) + 15) / 16 * 16);
    *mu = nb * 80;
  } else {
    *scales = (size_t)cap_tokens * 4;
    *mu = nb * (size_t)p->head_dim * 2;
  }
  *resid = (size_t)R * p->head_dim * 2;
  return NSNQ_OK;
}

size_t nsnq_build_codebook_workspace_bytes(const nsnq_params* p) {
  if (check_params(p) != NSNQ_OK) return 0;
  return sizeof(double) * ((size_t)kCodewords * sub_of(p) + kCodewords + 1);
}

nsnq_status nsnq_build_codebook(const nsnq_params* p, const float* samples, int64_t n, int32_t iters,
                                const float* init, float* centroids, uint16_t* codebook, float* distortion,
                                void* ws, size_t ws_bytes, void* stream) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  if (!samples || !centroids || !codebook || n < p->n_codewords || iters < 0) return NSNQ_EINVAL;
  if (!aligned16(samples) || !aligned16(centroids) || !aligned16(codebook)) return NSNQ_EINVAL;
  if (init && !aligned16(init)) return NSNQ_EINVAL;
  if (!ws || ws_bytes < nsnq_build_codebook_workspace_bytes(p) || !aligned16(ws)) return NSNQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int sub = sub_of(p);
  double* acc = (double*)ws;
  KmeansArgs a{};
  a.samples = samples;
  a.n = n;
  a.cent = centroids;
  a.sums = acc;
  a.counts = acc + kCodewords * sub;
  a.dsum = acc + kCodewords * sub + kCodewords;
  a.distortion = distortion;
  a.codebook = codebook;
  hipError_t e = launch_kmeans_init(init ? init : samples, centroids, sub, st);
  if (e == hipSuccess) e = launch_kmeans_clear(acc, kCodewords * sub + kCodewords + 1, st);
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    a.it = it;
    e = launch_kmeans_iter(a, sub, st);
  }
  if (e == hipSuccess) e = launch_kmeans_finish(a, sub, st);
  return hip_status(e);
}

nsnq_status nsnq_finetune_codebook(const nsnq_params* p, const float* samples, int64_t n, int32_t iters, float lr,
                                   float* centroids, uint16_t* codebook, float* loss, void* ws, size_t ws_bytes,
                                   void* stream) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  if (!samples || !centroids || !codebook || n < 1 || iters < 0 || !(lr >= 0.f) || lr > 1e30f) return NSNQ_EINVAL;
  if (!aligned16(samples) || !aligned16(centroids) || !aligned16(codebook)) return NSNQ_EINVAL;
  if (!ws || ws_bytes < nsnq_build_codebook_workspace_bytes(p) || !aligned16(ws)) return NSNQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int sub = sub_of(p);
  double* acc = (double*)ws;
  KmeansArgs a{};
  a.samples = samples;
  a.n = n;
  a.cent = centroids;
  a.sums = acc;
  a.counts = acc + kCodewords * sub;
  a.dsum = acc + kCodewords * sub + kCodewords;
  a.distortion = loss;
  a.codebook = codebook;
  a.lr = lr;
  hipError_t e = launch_kmeans_clear(acc, kCodewords * sub + kCodewords + 1, st);
  for (int it = 0; it < iters && e == hipSuccess; ++it) {
    a.it = it;
    e = launch_finetune_iter(a, sub, st);
  }
  if (e == hipSuccess) e = launch_kmeans_finish(a, sub, st);
  return hip_status(e);
}

nsnq_status nsnq_encode_kv(const nsnq_params* p, const uint16_t* codebook, const uint16_t* k, const uint16_t* v,
                           int64_t stride_b, int64_t stride_h, int64_t stride_t, int32_t L, nsnq_cache* cache,
                           void* stream) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  s = check_cache(p, cache);
  if (s != NSNQ_OK) return s;
  if (!codebook || !aligned16(codebook) || L < 0) return NSNQ_EINVAL;
  if (L == 0) return NSNQ_OK;
  if (!k || !v || !aligned16(k) || !aligned16(v)) return NSNQ_EINVAL;
  // 16-byte aligned token rows: every stride a multiple of 8 elements
  if (stride_t < p->head_dim || stride_b < 0 || stride_h < 0) return NSNQ_EINVAL;
  if ((stride_t % 8) || (stride_h % 8) || (stride_b % 8)) return NSNQ_EINVAL;
  if (cache->n_resid != 0 || is_ragged(cache)) return NSNQ_EINVAL;
  const int R = p->block_tokens;
  const int r = ((L - 1) % R) + 1;
  const int nq = L - r;
  if ((int64_t)cache->n_quant + nq > cache->cap_tokens) return NSNQ_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  s = run_encode(p, codebook, k, v, stride_b, stride_h, stride_t, nq / R, nq, r, cache, st);
  if (s != NSNQ_OK) return s;
  cache->n_quant += nq;
  cache->n_resid = r;
  return NSNQ_OK;
}

nsnq_status nsnq_encode_kv_ragged(const nsnq_params* p, const uint16_t* codebook, const uint16_t* k,
                                  const uint16_t* v, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                  const int32_t* lengths, int32_t max_len, nsnq_cache* cache, void* stream) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  s = check_cache(p, cache);
  if (s != NSNQ_OK) return s;
  if (!is_ragged(cache) || cache->n_quant != 0 || cache->n_resid != 0 || cache->max_len != 0) return NSNQ_EINVAL;
  if (!codebook || !aligned16(codebook) || !lengths || (((uintptr_t)lengths) & 3u) || max_len < 0)
    return NSNQ_EINVAL;
  if (!k || !v || !aligned16(k) || !aligned16(v)) return NSNQ_EINVAL;
  if (stride_t < p->head_dim || stride_b < 0 || stride_h < 0) return NSNQ_EINVAL;
  if ((stride_t % 8) || (stride_h % 8) || (stride_b % 8)) return NSNQ_EINVAL;
  const int R = p->block_tokens;
  const int nq_max = max_len > 0 ? max_len - (((max_len - 1) % R) + 1) : 0;  // largest row n_quant
  if (ragged_quant_bound(max_len, R) > cache->cap_tokens) return NSNQ_EINVAL;
  EncodeArgs a{};
  a.src[0] = k;
  a.src[1] = v;
  a.sb = stride_b;
  a.sh = stride_h;
  a.st = stride_t;
  a.codes[0] = cache->k.codes;
  a.codes[1] = cache->v.codes;
  a.scales[0] = cache->k.scales;
  a.scales[1] = cache->v.scales;
  a.mu[0] = cache->k.mu;
  a.mu[1] = cache->v.mu;
  a.resid[0] = cache->k.resid;
  a.resid[1] = cache->v.resid;
  a.codebook = codebook;
  a.H = cache->kv_heads;
  a.n_units = cache->batch * cache->kv_heads;
  a.cap = cache->cap_tokens;
  a.nblk = nq_max / R;
  a.R = R;
  a.signs = p->hadamard_signs;
  a.scale_adjust = (p->flags & NSNQ_SCALE_ADJUST) ? 1 : 0;
  a.dq = (p->flags & NSNQ_DOUBLE_QUANT) ? 1 : 0;
  a.cand = p->vq_candidates;
  a.span = p->vq_candidates ? p->vq_span : 0;
  a.lens = lengths;
  a.lens_max = max_len;
  a.out_quant = cache->seq_quant;
  a.out_resid = cache->seq_resid;
  s = hip_status(launch_encode(a, sub_of(p), R, (hipStream_t)stream));
  if (s != NSNQ_OK) return s;
  set_ragged_bounds(cache, max_len, R);
  return NSNQ_OK;
}

nsnq_status nsnq_flush_residual(const nsnq_params* p, const uint16_t* codebook, nsnq_cache* cache, void* stream) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  s = check_cache(p, cache);
  if (s != NSNQ_OK) return s;
  if (!codebook || !aligned16(codebook)) return NSNQ_EINVAL;
  const int R = p->block_tokens;
  if (is_ragged(cache)) {
    if (cache->n_resid < R) return NSNQ_OK;  // no row can be full
    if (ragged_quant_bound(cache->max_len, R) > cache->cap_tokens) return NSNQ_EINVAL;
    s = run_ragged_flush(p, codebook, cache, (hipStream_t)stream);
    if (s != NSNQ_OK) return s;
    AppendArgs a{};  // counters only
    a.H = cache->kv_heads;
    a.R = R;
    a.cap = cache->cap_tokens;
    a.seq_quant = cache->seq_quant;
    a.seq_resid = cache->seq_resid;
    return hip_status(launch_append(a, cache->batch, (hipStream_t)stream));  // lengths, so bounds, unchanged
  }
  if (cache->n_resid != R) return NSNQ_EINVAL;
  if ((int64_t)cache->n_quant + R > cache->cap_tokens) return NSNQ_EINVAL;
  const int64_t st = p->head_dim, sh = (int64_t)R * p->head_dim, sb = sh * cache->kv_heads;
  s = run_encode(p, codebook, cache->k.resid, cache->v.resid, sb, sh, st, 1, 0, 0, cache, (hipStream_t)stream);
  if (s != NSNQ_OK) return s;
  cache->n_quant += R;
  cache->n_resid = 0;
  return NSNQ_OK;
}

nsnq_status nsnq_append_kv(const nsnq_params* p, const uint16_t* codebook, const uint16_t* k_new,
                           const uint16_t* v_new, nsnq_cache* cache, void* stream) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  s = check_cache(p, cache);
  if (s != NSNQ_OK) return s;
  if (!codebook || !aligned16(codebook) || !k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
    return NSNQ_EINVAL;
  const int R = p->block_tokens;
  const bool may_flush = cache->n_resid == R;
  if (is_ragged(cache)) {
    if (ragged_quant_bound((int64_t)cache->max_len + 1, R) > cache->cap_tokens) return NSNQ_EINVAL;
  } else if (may_flush && (int64_t)cache->n_quant + R > cache->cap_tokens) {
    return NSNQ_EINVAL;
  }
  hipStream_t st = (hipStream_t)stream;
  AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.kresid = cache->k.resid;
  a.vresid = cache->v.resid;
  a.H = cache->kv_heads;
  a.R = R;
  a.cap = cache->cap_tokens;
  if (is_ragged(cache)) {
    if (may_flush) {
      s = run_ragged_flush(p, codebook, cache, st);
      if (s != NSNQ_OK) return s;
    }
    a.seq_quant = cache->seq_quant;
    a.seq_resid = cache->seq_resid;
    s = hip_status(launch_append(a, cache->batch, st));
    if (s != NSNQ_OK) return s;
    set_ragged_bounds(cache, cache->max_len + 1, R);
    return NSNQ_OK;
  }
  if (may_flush) {
    const int64_t tst = p->head_dim, sh = (int64_t)R * p->head_dim, sb = sh * cache->kv_heads;
    s = run_encode(p, codebook, cache->k.resid, cache->v.resid, sb, sh, tst, 1, 0, 0, cache, st);
    if (s != NSNQ_OK) return s;
    cache->n_quant += R;
    cache->n_resid = 0;
  }
  a.pos = cache->n_resid;
  s = hip_status(launch_append(a, cache->batch, st));
  if (s != NSNQ_OK) return s;
  cache->n_resid += 1;
  return NSNQ_OK;
}

nsnq_status nsnq_dequant(const nsnq_params* p, const uint16_t* codebook, const nsnq_cache* cache, int32_t which,
                         int32_t tok0, int32_t ntok, int32_t out_dtype, void* out, void* stream) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  s = check_cache(p, cache);
  if (s != NSNQ_OK) return s;
  if (!codebook || !aligned16(codebook)) return NSNQ_EINVAL;
  if (which != 0 && which != 1) return NSNQ_EINVAL;
  if (out_dtype != 0 && out_dtype != 1) return NSNQ_EINVAL;
  if (tok0 < 0 || ntok < 0 || (int64_t)tok0 + ntok > cache->n_quant) return NSNQ_EINVAL;
  if (ntok == 0) return NSNQ_OK;
  if (!out || !aligned16(out)) return NSNQ_EINVAL;
  const nsnq_kv& kv = which == 0 ? cache->k : cache->v;
  DequantArgs a{};
  a.codes = kv.codes;
  a.scales = kv.scales;
  a.mu = kv.mu;
  a.codebook = codebook;
  a.out = out;
  a.H = cache->kv_heads;
  a.cap = cache->cap_tokens;
  a.R = p->block_tokens;
  a.tok0 = tok0;
  a.ntok = ntok;
  a.out_f16 = out_dtype;
  a.signs = p->hadamard_signs;
  a.seq_quant = cache->seq_quant;
  a.dq = (p->flags & NSNQ_DOUBLE_QUANT) ? 1 : 0;
  return hip_status(launch_dequant(a, sub_of(p), cache->batch * cache->kv_heads, (hipStream_t)stream));
}

namespace {

struct DecodePlan {
  bool mfma;  // matrix-core kernel (grouped heads) instead of LUT scoring
  int gh, split_tokens, nsplit_q, nsplit;
  size_t lds;
};

// Query heads per work-group.  Matrix-core kernel: G itself for G = 2, 4, 8,
// 16, else 16 when G is a multiple of 16.  LUT kernel (G = 1 and the rest):
// the largest of 4, 2, 1 dividing G; with keys stored before RoPE at most 2:
// the four-head variant needs more than 256 registers (one wave per SIMD),
// and two-head groups at two waves per SIMD are faster even though each
// rebuilds the keys.
int mfma_heads_per_group(int G) {
  if (G == 2 || G == 4 || G == 8 || G == 16) return G;
  if (G > 16 && G % 16 == 0) return 16;
  return 0;
}
int heads_per_group(int G, bool rope) {
  if (G % 4 == 0 && !rope) return 4;
  return (G % 2 == 0) ? 2 : 1;
}

// prerope: keys stored before RoPE (LUT kernel only, at most 2 heads per group)
DecodePlan plan_decode(const nsnq_params* p, const nsnq_cache* c, int q_heads, int num_splits,
                       bool prerope = false) {
  DecodePlan pl{};
  const int G = q_heads / c->kv_heads;
  const int R = p->block_tokens;
  const int gq = prerope ? 0 : mfma_heads_per_group(G);
  pl.mfma = gq > 0;
  pl.gh = pl.mfma ? gq : heads_per_group(G, prerope);
  const int nblk = c->n_quant / R;
  const int max_ts = decode_max_split_tokens(sub_of(p), pl.gh, R);
  const int max_bps = max_ts / R;  // blocks per split
  // Split count over the compressed blocks; the splits then take nblk /
  // nsplit_q blocks each, as evenly as whole blocks allow (no short last
  // split), between 1 and max_bps blocks.
  int64_t nsq = 0;
  if (nblk > 0) {
    if (num_splits > 0) {
      nsq = num_splits;
    } else {
      // about 1024 work-groups over the grid, each with at least 512 tokens so
      // each of its 4 waves streams at least two 64-token chunks.  The
      // grouped-head kernel has long per-group set-up and only a few groups
      // fit a CU: there the grid is sized to what the device holds at once
      // (residual-window groups included), so every group starts in the first
      // round instead of a short second round trailing the first.
      const int64_t units = (int64_t)c->batch * c->kv_heads * (G / pl.gh);
      int64_t want = (1024 + units - 1) / units;
      if (pl.mfma) {
        const int64_t cap = decode_mfma_resident_groups(sub_of(p), pl.gh, (p->flags & NSNQ_DOUBLE_QUANT) != 0);
        const int64_t fit = (cap - (c->n_resid > 0 ? units : 0)) / units;
        if (cap > 0 && fit >= 4) want = fit;
      }
      const int min_bps = (512 + R - 1) / R;
      const int64_t most = nblk / min_bps > 0 ? nblk / min_bps : 1;
      nsq = want < most ? want : most;
    }
    if (nsq > nblk) nsq = nblk;
    if (nsq > kMaxSplits - 1) nsq = kMaxSplits - 1;
    const int64_t least = (nblk + max_bps - 1) / max_bps;
    if (nsq < least) nsq = least;
    if (nsq < 1) nsq = 1;
  }
  pl.nsplit_q = (int)nsq;
  pl.split_tokens = nsq > 0 ? (int)((nblk + nsq - 1) / nsq) * R : R;  // the longest split
  pl.nsplit = pl.nsplit_q + (c->n_resid > 0 ? 1 : 0);
  pl.lds = pl.mfma ? decode_mfma_lds_bytes(sub_of(p), pl.gh) : decode_lds_bytes(sub_of(p), pl.gh, pl.split_tokens, R);
  return pl;
}

}  // namespace

size_t nsnq_decode_workspace_bytes(const nsnq_params* p, const nsnq_cache* cache, int32_t q_heads,
                                   int32_t num_splits) {
  if (check_params(p) != NSNQ_OK || !cache || cache->kv_heads <= 0 || q_heads <= 0 ||
      q_heads % cache->kv_heads != 0 || cache->batch <= 0 || cache->n_quant < 0 || cache->n_resid < 0)
    return 0;
  // enough for both kernels' plans (the pre-RoPE call always uses the LUT kernel)
  const DecodePlan pl = plan_decode(p, cache, q_heads, num_splits);
  const DecodePlan pr = plan_decode(p, cache, q_heads, num_splits, true);
  const int ns = pl.nsplit > pr.nsplit ? pl.nsplit : pr.nsplit;
  return sizeof(float) * (size_t)cache->batch * q_heads * (size_t)ns * (kDim + 2);
}

namespace {
nsnq_status run_decode(const nsnq_params* p, const uint16_t* codebook, const uint16_t* q, int32_t q_heads,
                       const nsnq_cache* cache, float softmax_scale, const nsnq_rope* rope, int32_t num_splits,
                       uint16_t* out, void* ws, size_t ws_bytes, void* stream);
}

nsnq_status nsnq_decode_attention(const nsnq_params* p, const uint16_t* codebook, const uint16_t* q,
                                  int32_t q_heads, const nsnq_cache* cache, float softmax_scale,
                                  int32_t num_splits, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  return run_decode(p, codebook, q, q_heads, cache, softmax_scale, nullptr, num_splits, out, ws, ws_bytes, stream);
}

nsnq_status nsnq_decode_attention_prerope(const nsnq_params* p, const uint16_t* codebook, const uint16_t* q,
                                          int32_t q_heads, const nsnq_cache* cache, float softmax_scale,
                                          const nsnq_rope* rope, int32_t num_splits, uint16_t* out, void* ws,
                                          size_t ws_bytes, void* stream) {
  if (!rope) return NSNQ_EINVAL;
  return run_decode(p, codebook, q, q_heads, cache, softmax_scale, rope, num_splits, out, ws, ws_bytes, stream);
}

}  // extern "C"

// ---- decode attention without a caller workspace ---------------------------
// The split partials go to a static device array instead of a workspace the
// caller allocates.  Every device the library runs on holds its own copy for
// the life of the process.  In host code `scratch` names a host-side shadow,
// not device memory: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[NSNQ_SCRATCH_BYTES];

namespace {
std::atomic<void*> scratch_ptr[kMaxDevices];

// Device address of the current device's scratch, or null (status in *st).
void* device_scratch(nsnq_status* st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    *st = NSNQ_EHIP;
    return nullptr;
  }
  void* ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    // concurrent first calls on one device look up the same address
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      *st = NSNQ_EHIP;
      return nullptr;
    }
    scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  *st = NSNQ_OK;
  return ptr;
}
}  // namespace

extern "C" nsnq_status nsnq_decode_attention_noalloc(const nsnq_params* p, const uint16_t* codebook,
                                                     const uint16_t* q, int32_t q_heads, const nsnq_cache* cache,
                                                     float softmax_scale, int32_t num_splits, uint16_t* out,
                                                     void* stream) {
  // every host check first: a call that is rejected touches no device state
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  s = check_cache(p, cache);
  if (s != NSNQ_OK) return s;
  if (q_heads <= 0 || q_heads % cache->kv_heads != 0 || num_splits < 0) return NSNQ_EINVAL;
  const size_t need = nsnq_decode_workspace_bytes(p, cache, q_heads, num_splits);
  if (need > (size_t)NSNQ_SCRATCH_BYTES) return NSNQ_ESCRATCH;
  void* ws = device_scratch(&s);
  if (!ws) return s;
  // the kernels write every partial they read: nothing needs clearing
  return run_decode(p, codebook, q, q_heads, cache, softmax_scale, nullptr, num_splits, out, ws,
                    (size_t)NSNQ_SCRATCH_BYTES, stream);
}

namespace {
nsnq_status run_decode(const nsnq_params* p, const uint16_t* codebook, const uint16_t* q, int32_t q_heads,
                       const nsnq_cache* cache, float softmax_scale, const nsnq_rope* rope, int32_t num_splits,
                       uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  nsnq_status s = check_params(p);
  if (s != NSNQ_OK) return s;
  s = check_cache(p, cache);
  if (s != NSNQ_OK) return s;
  if (!codebook || !q || !out || !aligned16(codebook) || !aligned16(q) || !aligned16(out)) return NSNQ_EINVAL;
  if (q_heads <= 0 || q_heads % cache->kv_heads != 0) return NSNQ_EINVAL;
  const int G = q_heads / cache->kv_heads;
  if (G > 64 || num_splits < 0) return NSNQ_EINVAL;
  if (cache->n_quant + cache->n_resid < 1) return NSNQ_EINVAL;
  if (!(softmax_scale > 0.f) || softmax_scale > 1e30f) return NSNQ_EINVAL;
  const size_t need = nsnq_decode_workspace_bytes(p, cache, q_heads, num_splits);
  if (!ws || !aligned16(ws) || ws_bytes < need) return NSNQ_EWORKSPACE;
  if (rope) {
    if (!rope->cos || !rope->sin || !aligned16(rope->cos) || !aligned16(rope->sin)) return NSNQ_EINVAL;
    const int64_t last = (int64_t)rope->pos0 + (is_ragged(cache) ? (int64_t)cache->max_len
                                                                  : (int64_t)cache->n_quant + cache->n_resid);
    if (rope->pos0 < 0 || last > rope->max_pos) return NSNQ_EINVAL;
  }
  const DecodePlan pl = plan_decode(p, cache, q_heads, num_splits, rope != nullptr);
  if (pl.nsplit > kMaxSplits) return NSNQ_EUNSUPPORTED;  // context too long for one combine
  DecodeArgs a{};
  a.q = q;
  a.kcodes = cache->k.codes;
  a.kscales = cache->k.scales;
  a.kmu = cache->k.mu;
  a.kresid = cache->k.resid;
  a.vcodes = cache->v.codes;
  a.vscales = cache->v.scales;
  a.vmu = cache->v.mu;
  a.vresid = cache->v.resid;
  a.codebook = codebook;
  a.ws = (float*)ws;
  a.Hq = q_heads;
  a.Hkv = cache->kv_heads;
  a.G = G;
  a.cap = cache->cap_tokens;
  a.R = p->block_tokens;
  a.lgR = __builtin_ctz((unsigned)p->block_tokens);
  a.n_quant = cache->n_quant;
  a.n_resid = cache->n_resid;
  a.split_tokens = pl.split_tokens;
  a.nsplit_q = pl.nsplit_q;
  a.nsplit = pl.nsplit;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.signs = p->hadamard_signs;
  a.seq_quant = cache->seq_quant;
  a.seq_resid = cache->seq_resid;
  a.dq = (p->flags & NSNQ_DOUBLE_QUANT) ? 1 : 0;
  if (rope) {
    a.rope_cos = rope->cos;
    a.rope_sin = rope->sin;
    a.rope_pos0 = rope->pos0;
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = pl.mfma ? launch_decode_mfma(a, sub_of(p), pl.gh, cache->batch, st)
                         : launch_decode(a, sub_of(p), pl.gh, cache->batch, pl.lds, st);
  if (e != hipSuccess) return NSNQ_EHIP;
  CombineArgs cb{};
  cb.ws = (const float*)ws;
  cb.out = out;
  cb.Hq = q_heads;
  cb.nsplit = pl.nsplit;
  return hip_status(launch_combine(cb, cache->batch, st));
}
}  // namespace

extern "C" {

// --------------------------------------------------------------- fp16 ------

namespace {
int fp16_split_tokens(int G, int T, int num_splits, int units) {
  int ts;
  if (num_splits > 0) {
    ts = (T + num_splits - 1) / num_splits;
  } else {
    int64_t want = (2048 + units - 1) / units;
    if (want < 1) want = 1;
    ts = (int)((T + want - 1) / want);
  }
  ts = (ts + 63) / 64 * 64;
  if (ts < 64) ts = 64;
  while ((T + ts - 1) / ts > kMaxSplits) ts += 64;
  while (ts > 64 && fp16_decode_lds_bytes(G, ts) > 160 * 1024) ts -= 64;
  return ts;
}
}  // namespace

size_t nsnq_fp16_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t n_tokens, int32_t num_splits) {
  (void)num_splits;
  if (batch <= 0 || q_heads <= 0 || n_tokens <= 0) return 0;
  // worst case over G: one split per 64 tokens
  const size_t ns = (size_t)(n_tokens + 63) / 64;
  return sizeof(float) * (size_t)batch * q_heads * ns * (kDim + 2);
}

nsnq_status nsnq_fp16_decode_attention(const uint16_t* q, int32_t q_heads, const uint16_t* k, const uint16_t* v,
                                       int32_t batch, int32_t kv_heads, int32_t n_tokens, float softmax_scale,
                                       int32_t num_splits, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return NSNQ_EINVAL;
  if (batch <= 0 || kv_heads <= 0 || q_heads <= 0 || q_heads % kv_heads != 0 || n_tokens <= 0 || num_splits < 0)
    return NSNQ_EINVAL;
  const int G = q_heads / kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return NSNQ_EUNSUPPORTED;
  if (!(softmax_scale > 0.f)) return NSNQ_EINVAL;
  const int ts = fp16_split_tokens(G, n_tokens, num_splits, batch * kv_heads);
  const int nsplit = (n_tokens + ts - 1) / ts;
  if (nsplit > kMaxSplits || fp16_decode_lds_bytes(G, ts) > 160 * 1024) return NSNQ_EUNSUPPORTED;
  const size_t need = sizeof(float) * (size_t)batch * q_heads * nsplit * (kDim + 2);
  if (!ws || !aligned16(ws) || ws_bytes < need) return NSNQ_EWORKSPACE;
  Fp16DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.ws = (float*)ws;
  a.Hq = q_heads;
  a.Hkv = kv_heads;
  a.G = G;
  a.T = n_tokens;
  a.split_tokens = ts;
  a.nsplit = nsplit;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t st = (hipStream_t)stream;
  if (launch_fp16_decode(a, batch, st) != hipSuccess) return NSNQ_EHIP;
  CombineArgs cb{};
  cb.ws = (const float*)ws;
  cb.out = out;
  cb.Hq = q_heads;
  cb.nsplit = nsplit;
  return hip_status(launch_combine(cb, batch, st));
}

}  // extern "C"
