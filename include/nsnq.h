/*
 * nsnq.h -- C ABI of libnsnq: NSNQuant KV-cache vector quantisation and
 * decode attention over the compressed cache, for AMD MI355X (gfx950).
 *
 * The method (NSNQuant, "A Double Normalization Approach for Calibration-Free
 * Low-Bit Vector Quantization of KV Cache"; summarised on the atlas.scime.ai,
 * gist.science and pith.science pages) encodes each key/value head vector x of
 * dimension d by
 *   1. token-wise normalisation to norm sqrt(d), keeping n1 = ||x|| / sqrt(d);
 *   2. subtracting the channel-wise mean mu of the block of R tokens being
 *      quantised;
 *   3. a second token-wise normalisation, keeping n2;
 *   4. an orthonormal Hadamard rotation (Sylvester order; optionally
 *      randomised by a sign vector, see nsnq_params);
 *   5. vector quantisation of each run of s consecutive elements against one
 *      256-word codebook fit by k-means on seeded standard-normal samples;
 * while the most recent tokens stay in an fp16 residual window of R tokens.
 * Attention over the cache folds n1, n2 and mu into the scores and the value
 * sum (technical summary, sec. 4, "Attention Computation").
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE memory unless stated otherwise, owned by the
 *    caller, and must stay valid until the work queued on `stream` has run.
 *    fp16 values are IEEE binary16 bit patterns (uint16_t).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is asynchronous on it; nothing is synchronised.
 *  - Argument checks run on the host before anything is launched.  On error
 *    nothing is launched and a status other than NSNQ_OK is returned.  A
 *    launch failure returns NSNQ_EHIP.  Device faults surface at the caller's
 *    next synchronisation.  Inputs must be finite (not checked).
 *  - The library allocates no memory and prints nothing.  Its only global
 *    state is per device (up to 64 devices per process): the kernels'
 *    dynamic-LDS attribute, one occupancy query per grouped-head kernel
 *    variant and the device address of the static scratch of
 *    nsnq_decode_attention_noalloc, each set once on first use with atomic
 *    records (concurrent first calls are safe), and that static scratch
 *    itself (NSNQ_SCRATCH_BYTES of device memory per device, from the load
 *    of the library to the end of the process).  Calls on different streams
 *    are independent, except nsnq_decode_attention_noalloc calls, which
 *    share one device's scratch.
 *  - Value weights of the decode kernels that run on the matrix cores are
 *    carried in fp16 with a power-of-two factor per 64-token chunk (undone
 *    exactly in fp32), so the stored scales may take any finite fp16 value.
 *  - Layouts are dense and row-major.  For a cache of `batch` rows,
 *    `kv_heads` heads and capacity `cap_tokens` (a multiple of R), with
 *    S = d / s slots per vector (s = 4 at 2 bits, 8 at 1 bit):
 *      codes  uint8  [batch][kv_heads][cap_tokens][S]
 *      scales fp16   [batch][kv_heads][cap_tokens][2]   (n1, n2)
 *      mu     fp16   [batch][kv_heads][cap_tokens / R][d]
 *      resid  fp16   [batch][kv_heads][R][d]
 *    With NSNQ_DOUBLE_QUANT, scales and mu instead hold one byte record per
 *    block of R tokens, [batch][kv_heads][cap_tokens / R][record]:
 *      scales record, 16 * ceil((2R + R/2 + 4) / 16) bytes:
 *        [0, 2R)           N2 fp16 per token of the block
 *        [2R, 2R + R/2)    s1 4-bit codes (token t: byte t/2, low nibble
 *                          for even t)
 *        then              S1, Z1 fp16 (step and zero of the codes), zeros
 *      mu record, 80 bytes:
 *        [0, 64)           mean 4-bit codes (channel c: byte c/2, low nibble
 *                          for even c)
 *        [64, 80)          (S, Z) fp16 of the channel groups 0-31, ..., 96-127
 *    nsnq_buffer_bytes() gives every buffer's size.
 *    Every pointer must be 16-byte aligned.
 */
#ifndef NSNQ_H
#define NSNQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NSNQ_ABI_VERSION 7

typedef int32_t nsnq_status;
enum {
  NSNQ_OK = 0,
  NSNQ_EINVAL = 1,       /* bad argument, shape, counter or alignment */
  NSNQ_EUNSUPPORTED = 2, /* valid but not implemented (e.g. d != 128) */
  NSNQ_EHIP = 3,         /* a HIP launch or runtime call failed */
  NSNQ_EWORKSPACE = 4,   /* workspace missing or too small */
  NSNQ_ESCRATCH = 5      /* the call needs more than NSNQ_SCRATCH_BYTES of
                            static scratch (nsnq_decode_attention_noalloc) */
};

/* Format flags. */
enum {
  /* Scale adjustment "Strategy 3" (technical summary sec. 3, Scale
   * Adjustment): the quantised head vector c_hat is scaled by
   * alpha = |u|^2 / (u . c_hat) so that its component along the Hadamard-
   * domain vector u is preserved (the error is orthogonal to u).  alpha is
   * folded into the stored n2, so dequantisation and attention are unchanged. */
  NSNQ_SCALE_ADJUST = 1,
  /* Double quantisation (technical summary sec. 3, DQ; machine review,
   * implementation details: groups of 32 channels for the mean, of R tokens
   * for s1, 4-bit round-to-nearest).  Each group stores Z = fp16(min) and
   * S = fp16((max - min) / 15); a value v is coded q = clamp(rint((v - Z) / S),
   * 0, 15) (q = 0 when S = 0) and read back as Z + S q.  The encoder divides
   * tokens by the read-back s1 and subtracts the read-back mean, so the stored
   * values reconstruct the vector up to the VQ error.  n2 stays fp16.  Changes
   * the scales / mu layout (above). */
  NSNQ_DOUBLE_QUANT = 2
};

/* Format parameters.  head_dim must be 128, bits 1 or 2 (sub-vectors of 8 or 4
 * elements, one uint8 code each), n_codewords 256, block_tokens (R, the size of
 * both the residual window and the mean block) 64 or 128.
 *   flags           NSNQ_* flags above (0 = the plain pipeline).
 *   hadamard_signs  NULL for the plain (Sylvester) Hadamard transform, or a
 *                   device array of head_dim int8 values +1/-1: the randomised
 *                   Hadamard transform u = H diag(signs) w (technical summary
 *                   sec. 2).  Encode, dequant and attention of one cache must
 *                   use the same signs.
 *   vq_candidates   NULL (the encoder compares every codeword), or a device
 *                   copy of the table nsnq_vq_candidates() builds for the
 *                   codebook passed to the encode calls (2 bits only); the
 *                   codes are the same, the search is shorter.
 *   vq_span         0 with vq_candidates NULL, else the number of list entries
 *                   to search that nsnq_vq_candidates() returned (a multiple of
 *                   16, at most 128; spans over 96 use the exhaustive search). */
typedef struct {
  int32_t head_dim;
  int32_t bits;
  int32_t n_codewords;
  int32_t block_tokens;
  int32_t flags;
  int32_t vq_span;
  const int8_t* hadamard_signs;
  const uint8_t* vq_candidates;
} nsnq_params;

/* One of the K or V halves of a cache (layouts above). */
typedef struct {
  uint8_t* codes;
  uint16_t* scales;
  uint16_t* mu;
  uint16_t* resid;
} nsnq_kv;

/* A one-layer compressed cache.
 *
 * Uniform cache (seq_quant = seq_resid = NULL): n_quant (a multiple of R) and
 * n_resid (0..R) are HOST counters, the same for every batch row; the calls
 * below read and update them.
 *
 * Ragged cache (both non-NULL): seq_quant and seq_resid are DEVICE int32
 * arrays [batch] holding each row's own counters (same rules per row); the
 * kernels read and update them.  Rows are independent sequences of different
 * lengths (serving batches).  The host then keeps bounds, maintained by the
 * calls: max_len >= every row's n_quant + n_resid, and from it
 * n_quant = R * floor(max_len / R) and n_resid = min(R, max_len), which size
 * launches and workspaces (a loose bound costs only idle work-groups).
 * max_len is unused for uniform caches. */
typedef struct {
  nsnq_kv k, v;
  int32_t batch;
  int32_t kv_heads;
  int32_t cap_tokens;
  int32_t n_quant;
  int32_t n_resid;
  int32_t max_len;
  int32_t* seq_quant;
  int32_t* seq_resid;
} nsnq_cache;

/* ABI version (NSNQ_ABI_VERSION) and a static text for a status. */
int32_t nsnq_abi_version(void);
const char* nsnq_status_str(nsnq_status st);

/* Sizes in bytes of the four buffers of ONE (batch row, KV head) unit of a
 * cache of capacity cap_tokens (a multiple of R) in format p: codes, scales,
 * mu (K or V alike) and resid.  Multiply by batch * kv_heads.  Host only. */
nsnq_status nsnq_buffer_bytes(const nsnq_params* p, int32_t cap_tokens, size_t* codes, size_t* scales,
                              size_t* mu, size_t* resid);

/* Fit the codebook with Lloyd's k-means (technical summary sec. 3, "Codebook
 * Construction": k-means on synthetic torch.randn data, once, for any model).
 *   samples      fp32 [n][s] training vectors, s = 4 (bits 2) or 8 (bits 1);
 *                n >= n_codewords.
 *   init         fp32 [256][s] initial centroids, or NULL for the first 256
 *                samples.
 *   iters        Lloyd iterations (>= 0).  Each assigns every sample to its
 *                nearest centroid (squared Euclidean, ties to the lowest
 *                index) and moves each centroid to the mean of its members; a
 *                centroid without members stays put.
 *   centroids    fp32 [256][s] out: final centroids.
 *   codebook     fp16 [256][s] out: centroids rounded to nearest even.
 *   distortion   fp32 [iters] out (may be NULL): mean squared error per
 *                element of iteration i's assignment.
 *   ws/ws_bytes  device workspace of at least
 *                nsnq_build_codebook_workspace_bytes() bytes.
 */
size_t nsnq_build_codebook_workspace_bytes(const nsnq_params* p);
nsnq_status nsnq_build_codebook(const nsnq_params* p, const float* samples, int64_t n,
                                int32_t iters, const float* init, float* centroids,
                                uint16_t* codebook, float* distortion, void* ws,
                                size_t ws_bytes, void* stream);

/* Refine a codebook for the cosine distance (technical summary sec. 3,
 * Codebook Construction: after the k-means start, the codebook is tuned on
 * synthetic standard-normal data to minimise the cosine distance between
 * original and quantised vectors).  Reading: full-batch gradient descent with
 * a fixed step on  loss = mean over x of (1 - cos(x, x_hat)), where x runs over
 * the training head vectors and x_hat concatenates the nearest codewords
 * (squared Euclidean, ties to the lowest index) of x's sub-vectors; each step
 * assigns, then moves every codeword by -lr * d loss / d codeword with the
 * assignment held fixed.
 *   samples      fp32 [n][head_dim] training head vectors (n >= 1).
 *   centroids    fp32 [256][s] in: the start (the k-means centroids);
 *                out: the refined centroids.
 *   codebook     fp16 [256][s] out: the refined centroids rounded to nearest even.
 *   loss         fp32 [iters] out (may be NULL): step i's loss, before its move.
 *   ws/ws_bytes  as for nsnq_build_codebook (same size). */
nsnq_status nsnq_finetune_codebook(const nsnq_params* p, const float* samples, int64_t n, int32_t iters, float lr,
                                   float* centroids, uint16_t* codebook, float* loss, void* ws, size_t ws_bytes,
                                   void* stream);

/* Candidate lists for the 2-bit encoder's nearest-codeword search (technical
 * summary sec. 3, "Vector Quantization": squared Euclidean distance over
 * 4-element sub-vectors, 256 codewords; ties to the lowest index).  Each
 * sub-vector u of a Hadamard-domain vector of norm sqrt(128) lies in one of 16
 * orthant boxes (bit i of the orthant index set when u_i < 0; every |u_i| <=
 * 12).  For each box the list holds, in ascending order, every codeword whose
 * Voronoi cell meets the box, found by an exact fp64 linear programme per
 * (codeword, box); the nearest codeword of any u in the box is on its list, so
 * searching the list returns the same code as searching all 256.
 *   codebook_host  fp16 [256][4], HOST memory (the codebook of the encode calls).
 *   table_host     HOST out, NSNQ_VQ_TABLE_BYTES bytes: [16 boxes][128] codeword
 *                  indices, each list padded by repeating its last entry.
 *   span           out: the longest list rounded up to a multiple of 16, for
 *                  nsnq_params.vq_span.
 * Copy the table to device memory and set vq_candidates / vq_span in the
 * params of the encode calls.  Host only, synchronous, about 0.1 s.
 * NSNQ_EUNSUPPORTED for bits != 2 (1-bit boxes keep most codewords) or when a
 * list would exceed 128 entries. */
#define NSNQ_VQ_TABLE_BYTES 2048
nsnq_status nsnq_vq_candidates(const nsnq_params* p, const uint16_t* codebook_host, uint8_t* table_host,
                               int32_t* span);

/* 4-bit quantisation of the codebook entries (technical summary sec. 3,
 * "Double Quantization": besides the mean o and the scale s1, the codebook
 * entries themselves are stored in 4 bits).  The entries in storage order
 * ([256][s]) form groups of NSNQ_CODEBOOK_DQ_GROUP; each group keeps
 * Z = fp16(min) and S = fp16((max - min) / 15), each entry the code
 * q = clamp(rint((v - Z) / S), 0, 15) (0 when S = 0), all formed in double.
 *   codebook_host      fp16 [256][s], HOST memory (s = 4 at 2 bits, 8 at 1).
 *   record_host        HOST out, NSNQ_CODEBOOK_DQ_BYTES(bits) bytes: 128 s
 *                      bytes of codes (entry i: byte i/2, low nibble for even
 *                      i), then (S, Z) fp16 per group.
 *   codebook_hat_host  HOST out, fp16 [256][s]: the read-back codebook
 *                      fp16(Z + S q), which the encode, dequant and attention
 *                      calls then take as their codebook.
 * Host only, synchronous.  NSNQ_EINVAL for a non-finite entry. */
#define NSNQ_CODEBOOK_DQ_GROUP 32
#define NSNQ_CODEBOOK_DQ_BYTES(bits) (128 * ((bits) == 2 ? 4 : 8) + 4 * (256 * ((bits) == 2 ? 4 : 8) / 32))
nsnq_status nsnq_codebook_dq(const nsnq_params* p, const uint16_t* codebook_host, uint8_t* record_host,
                             uint16_t* codebook_hat_host);

/* Prefill encode (technical summary secs. 1-4).  k and v are fp16 streams
 * indexed [b][h][t][c] at element offsets b*stride_b + h*stride_h +
 * t*stride_t + c (c contiguous), t < L.  Of the L tokens, the first L - r are
 * encoded in blocks of R at token positions n_quant.. of the cache, where
 * r = ((L - 1) mod R) + 1 (0 when L = 0); the last r are copied verbatim into
 * resid.  Requires cache->n_resid == 0 and n_quant + L - r <= cap_tokens;
 * afterwards n_quant += L - r and n_resid = r.  codebook: fp16 [256][s]. */
nsnq_status nsnq_encode_kv(const nsnq_params* p, const uint16_t* codebook, const uint16_t* k,
                           const uint16_t* v, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                           int32_t L, nsnq_cache* cache, void* stream);

/* Ragged prefill: row b encodes the first lengths[b] tokens of its streams
 * exactly as nsnq_encode_kv does for L = lengths[b] (device int32 array
 * [batch], 0 <= lengths[b] <= max_len), writing seq_quant[b] and
 * seq_resid[b].  Requires a ragged cache with n_quant == n_resid == max_len
 * == 0 (empty; the device counters are overwritten) and
 * R * floor(max_len / R) <= cap_tokens.  Afterwards the host bounds are those
 * of max_len.  Uniform caches: EINVAL. */
nsnq_status nsnq_encode_kv_ragged(const nsnq_params* p, const uint16_t* codebook, const uint16_t* k,
                                  const uint16_t* v, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                                  const int32_t* lengths, int32_t max_len, nsnq_cache* cache, void* stream);

/* Flush a full residual window (technical summary sec. 4, "Residuals"): the R
 * residual tokens are encoded as one block at position n_quant, then
 * n_quant += R and n_resid = 0.  Uniform cache: requires n_resid == R and
 * n_quant + R <= cap_tokens; the caller then writes the new token into
 * resid[.., n_resid, :] and increments n_resid (or calls nsnq_append_kv).
 * Ragged cache: every row whose seq_resid is R is flushed, the others are
 * left alone (nothing is launched when the bound n_resid is below R); the
 * bounds do not change. */
nsnq_status nsnq_flush_residual(const nsnq_params* p, const uint16_t* codebook, nsnq_cache* cache,
                                void* stream);

/* Append one token per row (the decode step's new key and value): k_new and
 * v_new fp16 [batch][kv_heads][d].  A row whose residual window is full is
 * first flushed as by nsnq_flush_residual, then the token is written at its
 * window position and its n_resid incremented.  Works on uniform caches
 * (host counters; requires n_quant + R <= cap_tokens when n_resid == R) and
 * ragged caches (device counters, per row; max_len grows by one and requires
 * R * floor((max_len + 1) / R) <= cap_tokens). */
nsnq_status nsnq_append_kv(const nsnq_params* p, const uint16_t* codebook, const uint16_t* k_new,
                           const uint16_t* v_new, nsnq_cache* cache, void* stream);

/* Reconstruct quantised tokens [tok0, tok0 + ntok) of the K (which = 0) or V
 * (which = 1) half: x_hat = N1 * (N2 * D H c_hat + MU_block), D = diag(signs)
 * (identity without signs), the inverse of the
 * encode using only stored values (technical summary sec. 1: the byproducts
 * rebuild the tensor; sec. 4: dequantisation kernel).  Requires
 * 0 <= tok0, tok0 + ntok <= n_quant.  out: [batch][kv_heads][ntok][d] as fp32
 * (out_dtype 0) or fp16 (out_dtype 1).  Ragged cache: tokens at or past a
 * row's seq_quant are written as zeros. */
nsnq_status nsnq_dequant(const nsnq_params* p, const uint16_t* codebook, const nsnq_cache* cache,
                         int32_t which, int32_t tok0, int32_t ntok, int32_t out_dtype, void* out,
                         void* stream);

/* Decode attention for one query token per batch row over the n_quant
 * compressed and n_resid fp16 tokens of the cache (technical summary sec. 4,
 * "Attention Computation"; the figure "Overall structure of attention under
 * NSNQuant").  q: fp16 [batch][q_heads][d]; query head h reads KV head
 * h / (q_heads / kv_heads).  softmax over scale * q.k.  num_splits: number of
 * token ranges per head processed in parallel (0 = choose).  out: fp16
 * [batch][q_heads][d].  ws/ws_bytes: device workspace of at least
 * nsnq_decode_workspace_bytes(p, cache, q_heads, num_splits) bytes.
 * Requires n_quant + n_resid >= 1 (ragged cache: per row, else that row's
 * output is zero). */
size_t nsnq_decode_workspace_bytes(const nsnq_params* p, const nsnq_cache* cache, int32_t q_heads,
                                   int32_t num_splits);
nsnq_status nsnq_decode_attention(const nsnq_params* p, const uint16_t* codebook, const uint16_t* q,
                                  int32_t q_heads, const nsnq_cache* cache, float softmax_scale,
                                  int32_t num_splits, uint16_t* out, void* ws, size_t ws_bytes,
                                  void* stream);

/* Decode attention without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc).  The same computation, kernels and launch plan as
 * nsnq_decode_attention (same arguments, same results bit for bit), with the
 * split partials in a static device array of NSNQ_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends.  Calls no
 * hipMalloc / hipFree and allocates nothing.
 *   Returns NSNQ_ESCRATCH, before touching the device, when the call would
 *   need more than NSNQ_SCRATCH_BYTES (nsnq_decode_workspace_bytes() of the
 *   same arguments gives the need: 4 (d + 2) bytes per (row, query head,
 *   split); e.g. 12.8 MB for 256 rows x 32 heads x 3 splits).  Nothing in
 *   the scratch has to start at zero: every call writes all it reads.
 *   All calls on one device share that device's scratch, which keeps the last
 *   call's contents: calls that can overlap on one device (different streams
 *   or threads without ordering) race and must be serialised by the caller;
 *   calls in one stream are ordered.  The first call on a device looks up the
 *   scratch's device address (hipGetSymbolAddress) with that device current. */
#define NSNQ_SCRATCH_BYTES (16u << 20)
nsnq_status nsnq_decode_attention_noalloc(const nsnq_params* p, const uint16_t* codebook, const uint16_t* q,
                                          int32_t q_heads, const nsnq_cache* cache, float softmax_scale,
                                          int32_t num_splits, uint16_t* out, void* stream);

/* Keys quantised before RoPE (technical summary sec. 4, Attention
 * Computation: NSN is applied to keys before the rotary embedding).  Token t
 * of a row (compressed tokens first, then the residual window) sits at
 * position pos0 + t; its reconstructed key is rotated in the rotate-half
 * convention, pairs (c, c + 64) for c < 64:
 *   k'[c]      = k[c] cos[pos][c] - k[c + 64] sin[pos][c]
 *   k'[c + 64] = k[c + 64] cos[pos][c] + k[c] sin[pos][c]
 * with the caller's tables cos, sin: device fp32 [max_pos][64] (any
 * frequencies, e.g. theta_c = base^(-2c/128), or scaled ones).  q is the
 * already-rotated query.  Requires pos0 >= 0 and pos0 + (tokens of the
 * longest row, or max_len for a ragged cache) <= max_pos. */
typedef struct {
  const float* cos;
  const float* sin;
  int32_t max_pos;
  int32_t pos0;
} nsnq_rope;

/* Decode attention as nsnq_decode_attention, with the keys of the cache
 * stored before RoPE (nsnq_rope above).  Values are unchanged.  Workspace:
 * nsnq_decode_workspace_bytes (it covers both calls). */
nsnq_status nsnq_decode_attention_prerope(const nsnq_params* p, const uint16_t* codebook, const uint16_t* q,
                                          int32_t q_heads, const nsnq_cache* cache, float softmax_scale,
                                          const nsnq_rope* rope, int32_t num_splits, uint16_t* out, void* ws,
                                          size_t ws_bytes, void* stream);

/* Comparator: the same decode attention over an uncompressed fp16 cache
 * k, v [batch][kv_heads][n_tokens][d] (d = 128), used to measure the gain of
 * the compressed cache.  Workspace from nsnq_fp16_decode_workspace_bytes(). */
size_t nsnq_fp16_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t n_tokens,
                                        int32_t num_splits);
nsnq_status nsnq_fp16_decode_attention(const uint16_t* q, int32_t q_heads, const uint16_t* k,
                                       const uint16_t* v, int32_t batch, int32_t kv_heads,
                                       int32_t n_tokens, float softmax_scale, int32_t num_splits,
                                       uint16_t* out, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NSNQ_H */
