// nsnq_launch.hpp -- kernel argument blocks and launchers (host <-> device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsnq {

// Devices per process the library keeps per-device state for: the kernels'
// dynamic-LDS attribute, one occupancy query per grouped-head kernel variant
// and the address of the static decode scratch.
constexpr int kMaxDevices = 64;

struct EncodeArgs {
  const uint16_t* src[2];  // K, V fp16 streams
  int64_t sb, sh, st;      // element strides (batch, head, token)
  uint8_t* codes[2];
  uint16_t* scales[2];
  uint16_t* mu[2];
  const uint16_t* codebook;  // fp16 [256][SUB]
  uint16_t* resid[2];
  int H;                     // heads
  int n_units;               // batch * heads
  int cap;                   // cache capacity (tokens)
  int dst_tok0;              // first destination token (multiple of R)
  int nblk;                  // blocks per stream
  int R;                     // block / window size
  int rc_t0, rc_r;           // residual copy: first source token and count (0 = none)
  const int8_t* signs;       // randomised-Hadamard signs [128] or null
  int scale_adjust;          // fold alpha = |u|^2 / (u . c_hat) into n2
  int dq;                    // double-quantised scales / mean records
  // ragged prefill: per-row stream lengths (device [B]); the block / residual
  // split of each row follows its own length, and the row counters are
  // written to out_quant / out_resid.  Null for uniform launches.
  const int32_t* lens;
  int lens_max;  // lengths are clamped to [0, lens_max]
  int32_t* out_quant;
  int32_t* out_resid;
  // ragged flush: only rows with fl_resid[b] == R are encoded, at token
  // fl_quant[b].  Null otherwise.
  const int32_t* fl_quant;
  const int32_t* fl_resid;
  // 2-bit nearest-codeword search over per-orthant candidate lists
  // ([16][128] codeword indices, device), the first `span` entries of each;
  // span = 0 compares every codeword
  const uint8_t* cand;
  int span;
  int n_enc;  // candidate lists: encoding work-groups per K/V half (each loops over blocks)
};

struct AppendArgs {
  const uint16_t* k_new;  // [B][H][d]
  const uint16_t* v_new;
  uint16_t* kresid;
  uint16_t* vresid;
  int H, R, cap;
  int pos;                // uniform: window position to write
  int32_t* seq_quant;     // ragged: per-row counters (null for uniform)
  int32_t* seq_resid;
};

struct DequantArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* mu;
  const uint16_t* codebook;
  void* out;
  int H, cap, R, tok0, ntok, out_f16;
  const int8_t* signs;
  const int32_t* seq_quant;  // ragged: tokens >= seq_quant[b] come out as 0
  int dq;                    // double-quantised scales / mean records
};

// ---- double-quantised records (byte layout in nsnq.h) ----------------------
__host__ __device__ constexpr int dq_record_bytes(int R) { return ((2 * R + R / 2 + 4) + 15) / 16 * 16; }
constexpr int kDqMuRecord = 80;

// (s1 code of token tb, n2 bits) of a scales record, as q << 16 | n2.
__device__ __forceinline__ uint32_t dq_token(const uint8_t* rec, int R, int tb) {
  const uint32_t n2 = *reinterpret_cast<const uint16_t*>(rec + 2 * tb);
  const uint32_t q = (rec[2 * R + tb / 2] >> (4 * (tb & 1))) & 15u;
  return n2 | (q << 16);
}
// (S1, Z1) fp16 pair of a scales record.
__device__ __forceinline__ uint32_t dq_s1_params(const uint8_t* rec, int R) {
  return *reinterpret_cast<const uint32_t*>(rec + 2 * R + R / 2);
}
// Read-back value Z + S q of an (S, Z) fp16 pair.
__device__ __forceinline__ float dq_value(uint32_t sz, uint32_t q) {
  const float S = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz & 0xffff));
  const float Z = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz >> 16));
  return fmaf(S, (float)q, Z);
}
// Mean of channels 2j and 2j + 1 (j < 64) from a mean record.
__device__ __forceinline__ void dq_mu_pair(const uint8_t* rec, int j, float& m0, float& m1) {
  const uint32_t b = rec[j];
  const uint32_t sz = *reinterpret_cast<const uint32_t*>(rec + 64 + 4 * (j / 16));
  m0 = dq_value(sz, b & 15u);
  m1 = dq_value(sz, b >> 4);
}

struct DecodeArgs {
  const uint16_t* q;  // [B][Hq][d]
  const uint8_t* kcodes;
  const uint16_t* kscales;
  const uint16_t* kmu;
  const uint16_t* kresid;
  const uint8_t* vcodes;
  const uint16_t* vscales;
  const uint16_t* vmu;
  const uint16_t* vresid;
  const uint16_t* codebook;
  float* ws;         // partials [B][Hq][nsplit][d + 2]
  int Hq, Hkv, G;    // G = Hq / Hkv
  int cap, R;
  int lgR;           // log2 R (R is a power of two)
  int n_quant, n_resid;
  int split_tokens;  // compressed tokens of the longest split (multiple of R)
  // grid order, set by the launchers: 0 = blockIdx.x is the split (each row's
  // splits, residual group included, dispatch together), 1 = blockIdx.y is
  // the split (all compressed splits dispatch before the residual groups)
  int split_slow;
  int nsplit_q;      // splits over the compressed tokens (split_block)
  int nsplit;        // nsplit_q + (n_resid > 0)
  float scale_log2;  // softmax scale * log2(e)
  const int8_t* signs;  // randomised-Hadamard signs [128] or null
  const int32_t* seq_quant;  // ragged: per-row counters (null: n_quant / n_resid)
  const int32_t* seq_resid;
  int dq;                    // double-quantised scales / mean records
  // keys stored before RoPE: token t of a row sits at position rope_pos0 + t
  // and is rotated with the tables rope_cos / rope_sin [position][64] (null:
  // keys are used as stored)
  const float* rope_cos;
  const float* rope_sin;
  int rope_pos0;
};

// Compressed split s of a decode launch covers blocks [split_block(a, s),
// split_block(a, s + 1)) of the host bound n_quant: nsplit_q splits as even as
// whole blocks allow.
__device__ __forceinline__ int split_block(const DecodeArgs& a, int s) {
  return (int)(((int64_t)s * (a.n_quant >> a.lgR)) / a.nsplit_q);
}

// Per-row token counts of a decode launch (ragged counters are clamped to the
// host bounds the launch was sized for).
__device__ __forceinline__ int row_quant(const DecodeArgs& a, int b) {
  return a.seq_quant ? max(0, min(a.seq_quant[b], a.n_quant)) : a.n_quant;
}
__device__ __forceinline__ int row_resid(const DecodeArgs& a, int b) {
  return a.seq_resid ? max(0, min(a.seq_resid[b], a.n_resid)) : a.n_resid;
}

struct CombineArgs {
  const float* ws;
  uint16_t* out;
  int Hq, nsplit;
  int nbh;  // batch rows x query heads (set by the launcher)
};

struct KmeansArgs {
  const float* samples;  // [n][SUB]
  int64_t n;
  float* cent;           // [256][SUB] current centroids
  double* sums;          // [256][SUB]
  double* counts;        // [256]
  double* dsum;          // [1]
  float* distortion;     // [iters] or null
  uint16_t* codebook;    // [256][SUB] fp16 out
  int it;
  double lr;             // cosine refinement: gradient step
};

struct Fp16DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* ws;
  int Hq, Hkv, G, T;
  int split_tokens, nsplit;
  float scale_log2;
};

hipError_t launch_encode(const EncodeArgs& a, int sub, int R, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, int B, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs& a, int sub, int n_units, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int sub, int gh, int B, size_t lds_bytes, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs& a, int sub, int gq, int B, hipStream_t stream);
size_t decode_mfma_lds_bytes(int sub, int gq);
// work-groups of the grouped-head kernel the device holds at once (0 if unknown)
int decode_mfma_resident_groups(int sub, int gq, bool dq);
hipError_t launch_combine(const CombineArgs& a, int B, hipStream_t stream);
size_t decode_lds_bytes(int sub, int gh, int split_tokens, int R);
constexpr int kMaxSplits = 1024;  // partials one combine can merge
int decode_max_split_tokens(int sub, int gh, int R);
hipError_t launch_kmeans_init(const float* src, float* cent, int sub, hipStream_t stream);
hipError_t launch_kmeans_iter(const KmeansArgs& a, int sub, hipStream_t stream);
hipError_t launch_kmeans_finish(const KmeansArgs& a, int sub, hipStream_t stream);
hipError_t launch_finetune_iter(const KmeansArgs& a, int sub, hipStream_t stream);
hipError_t launch_fp16_decode(const Fp16DecodeArgs& a, int B, hipStream_t stream);
size_t fp16_decode_lds_bytes(int G, int split_tokens);

}  // namespace nsnq
