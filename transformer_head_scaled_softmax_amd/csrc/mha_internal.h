// mha_internal.h -- kernel parameter blocks and launchers shared by the host
// dispatch (mha_api.cpp) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

namespace mha {

enum class DType : int { F32 = 0, BF16 = 1, F16 = 2 };

// Attention over strided [B, H, N, d] views.  Element (b, h, n, c) of a tensor
// lives at base + b*s_b + h*s_h + n*s_n + c (strides in elements), so the same
// kernels read per-head tensors and the row-major projection outputs
// [B*N, H*d] (where s_h = d and s_n = H*d) without a reshuffle.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* key_lens;  // device int32[B] or nullptr
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int B, H, Nq, Nk, dk, dv;
  int causal;
  float scale;
  // Query heads per key/value head: head h reads key/value head h / kv_group
  // (0 or 1: one each).  Strides k_sh, v_sh step over key/value heads.
  int kv_group;
  // Causal mask anchored at the end of the filled keys (decoding against a
  // cache): query i sits at position L - Nq + i and sees keys j <= L - Nq + i.
  // 0: query i sees keys j <= i (self-attention, Nq == Nk).
  int causal_end;
  // Optional row statistic for training: lse[(b*H + h)*Nq + i] = natural log
  // of the softmax denominator of row i over its visible keys (-inf for a row
  // with none).  nullptr: not written.
  float* lse;
};

// Gradients of attention on dense per-head tensors [B, H, N, d] (k, v:
// [B, Hkv, N, d]): q, k, v,
// out (the forward output), dout (dLoss/dout) and lse (the forward's row
// statistic, [B, H, Nq]) in; dq, dk, dv out.  dsum is scratch [B, H, Nq] that
// the dQ kernel fills with D_i = dout_i . out_i for the dK/dV kernel.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;
  const int32_t* key_lens;  // device int32[B] or nullptr
  int B, H, Nq, Nk;
  int causal;
  float scale;
  // Key/value heads: k, v, dk, dv are [B, Hkv, Nk, d]; query head h uses
  // key/value head h / (H / Hkv) (Hkv == H: one each), and the gradients of a
  // shared key/value head sum over its query heads.
  int Hkv;
  // bf16/f16 only: the query heads of a key/value head are split into `parts`
  // equal runs (bwd_head_parts); with parts > 1 each run's dK/dV workgroups
  // leave fp32 sums in `part` ([2][parts][B*Hkv][Nk][64]: dK unscaled, then
  // dV) and a combining kernel adds the runs in order.
  int parts;
  float* part;
};

// How many runs the dK/dV pass splits each group of H / Hkv query heads into
// (bf16/f16, head size 64): the fewest (a divisor of the group size) that give
// at least kBwdMinBlocks workgroups -- one workgroup per key block of one
// key/value head alone can leave the chip with one round of workgroups whose
// lengths differ by the causal mask.  A pure function of the sizes, so the
// workspace query and the launch agree.
constexpr int kBwdMinBlocks = 2048;
// Whether the bf16/f16 backward pass runs as one launch (both parts in one
// workgroup per (b, h)): at most 64 queries and 64 keys, one key/value head
// per query head.
inline bool bwd_single_launch(int H, int Hkv, int Nq, int Nk) {
  return Hkv == H && Nq >= 1 && Nk >= 1 && Nq <= 64 && Nk <= 64;
}
inline int bwd_dkdv_keys_per_block(int Nk) { return Nk > 64 ? 128 : 64; }
inline int bwd_head_parts(int B, int H, int Hkv, int Nk) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || Nk <= 0 || H % Hkv) return 1;
  const int G = H / Hkv;
  const int kpb = bwd_dkdv_keys_per_block(Nk);
  const int64_t units = int64_t(B) * Hkv * ((Nk + kpb - 1) / kpb);
  int P = 1;
  while (P < G && units * P < kBwdMinBlocks) {
    ++P;
    while (G % P) ++P;
  }
  return P;
}

// One decoding step against a key/value cache, head size 64: q [B, H, Nq, 64]
// (the Nq newest positions), caches k, v [B, Hkv, S, 64], out [B, H, Nq, 64].
// Query head h reads cache head h / (H / Hkv); the R = (H / Hkv) * Nq query
// rows that share a cache head are consecutive in q and out.  Sequence b has
// L = clamp(cache_lens[b], 0, S) filled slots; with `causal`, query i sees
// slots j <= L - Nq + i, otherwise all L.
//
// The filled slots of all caches, laid end to end (cache (b, g) at
// Hkv * sum_{b' < b} L_b' + g * L_b), are cut into `waves` equal ranges, one
// per wave of the decoding kernel.  A wave's range falls into pieces at cache
// boundaries; a piece that is a whole cache writes its output rows, any other
// piece leaves its softmax state in record (cache + wave) of `part`, and the
// wave that starts a cache writes the first and last wave over it to `span`.
// The combining kernel then merges the records of the caches that were cut.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* cache_lens;  // device int32[B] or nullptr
  float* part;                // [B*Hkv + waves, R, kDecodePartFloats]
  int2* span;                 // [B*Hkv]
  int B, H, Hkv, Nq, S;
  int causal;
  float scale;
  int waves;
};

// One projection problem: C[m, n] = sum_k X[m, k] * W[n, k] (+ bias[n]).
// X [M, K] row-major with row stride ldx; W [N, K] row-major (stride K);
// C [M, N] row-major with row stride ldc.  For launch_gemm_ln the row is then
// z = C + residual (same layout as C) and C = LayerNorm(z) * gamma + beta.
struct GemmProblem {
  const void* x;
  const void* w;
  const void* bias;  // nullable, [N]
  void* c;
  int M, N, K;
  int64_t ldx, ldc;
  // launch_gemm_ln only:
  const void* residual;  // [M, N], row stride ldc
  const void* gamma;     // nullable (1), [N]
  const void* beta;      // nullable (0), [N]
  float eps;
  float2* stats;         // [M, ln_stats_stride(N)]: per row and column tile, (sum, centred sum of squares)
};

// Scratch of launch_gemm_ln: per-row statistics of up to one 64-column tile
// each (the narrowest tiles).
__host__ __device__ inline int ln_stats_stride(int N) { return (N + 63) / 64; }

constexpr int kMaxGemmProblems = 3;

struct GemmBatch {
  GemmProblem p[kMaxGemmProblems];
  int count;
};

// Fused Q/K/V projection and attention on short sequences: x_q [B*Nq, D] and
// x_kv [B*Nk, D] row-major (xkv == xq for self-attention), W_* [H*64, D],
// biases [H*64] (nullable), o [B*Nq, H*64] (head-major concatenation).
struct ProjAttnArgs {
  const void* xq;
  const void* xkv;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* bq;
  const void* bk;
  const void* bv;
  void* o;
  const int32_t* key_lens;  // device int32[B] or nullptr
  int B, Nq, Nk, D, H;
  int causal;
  float scale;
  // Query heads per key/value head (0 or 1: one each): W_K, W_V, b_K, b_V hold
  // H / kv_group heads and head h uses head h / kv_group of them.
  int kv_group;
};

// Launchers return hipSuccess or the launch error; they validate nothing
// beyond what their kernels assume (the public entry points validate first).
// Non-null t0/t1 receive the kernel's own start and end timestamps
// (hipExtLaunchKernel events).
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream, hipEvent_t t0 = nullptr,
                           hipEvent_t t1 = nullptr);
hipError_t launch_attn_mfma(const AttnArgs& a, DType dt, hipStream_t stream, hipEvent_t t0 = nullptr,
                            hipEvent_t t1 = nullptr);
// Queries per workgroup of the bf16/f16 attention launch: 32 (one wave per
// workgroup, reading its own key/value tiles), 256 or 512 (four or eight waves
// of 64 queries sharing each key/value tile staged in LDS).  All three give
// the same results bit for bit.  Shared tiles serve more queries per byte
// read, but a query length that is not a multiple of the workgroup's leaves
// waves idle, and few workgroups leave compute units idle: the utilisation
// u = (queries / query slots) x (workgroups / workgroup slots of the rounds
// they take) -- one 512-query or two 256-query workgroups per compute unit,
// 256 compute units -- decides, from measurements on one MI355X of the three
// kernels over 38 shapes (96-8192 queries, cross-attention up to 4096 keys):
//   * at most 64 queries: 32;
//   * from 4096 queries with u(512) >= 0.9: 512 (2-3% ahead of 256 at 8192);
//   * u(256) >= 0.7 under the causal mask, >= 0.45 without it: 256 (up to
//     1.6x ahead of the others at a few hundred queries with many heads);
//   * otherwise, up to 2048 queries: 32 (its small workgroups fill the chip
//     when there are few heads or the 256-query blocks are mostly empty);
//     beyond: 256.
// MHA_ATTENTION_BLOCK=32, 256 or 512 in the environment, read on every call,
// forces one of the kernels.
inline double attention_block_use(int64_t B, int64_t H, int64_t Nq, int64_t qb, int64_t per_round) {
  const int64_t nqb = (Nq + qb - 1) / qb, wgs = nqb * B * H;
  if (wgs <= 0) return 0.0;
  const int64_t rounds = (wgs + per_round - 1) / per_round;
  return double(Nq) / double(nqb * qb) * double(wgs) / double(rounds * per_round);
}
inline int attention_block_queries(int B, int H, int Nq, bool causal) {
  if (const char* force = getenv("MHA_ATTENTION_BLOCK"))
    for (int qb : {32, 256, 512})
      if (atoi(force) == qb) return qb;
  if (Nq <= 64) return 32;
  constexpr int64_t kComputeUnits = 256;
  if (Nq >= 4096 && attention_block_use(B, H, Nq, 512, kComputeUnits) >= 0.9) return 512;
  if (attention_block_use(B, H, Nq, 256, 2 * kComputeUnits) >= (causal ? 0.7 : 0.45)) return 256;
  return Nq <= 2048 ? 32 : 256;
}

hipError_t launch_gemm_mfma(const GemmBatch& g, DType dt, hipStream_t stream, hipEvent_t t0 = nullptr,
                            hipEvent_t t1 = nullptr);
// Output projection followed by the residual connection and layer
// normalisation: the projection's epilogue adds the bias and the residual and
// leaves per-tile row statistics in p.stats and the rows as fp16 differences
// from their tile means in p.c; a second kernel merges the statistics and
// normalises the rows in place.  t0/t1 time the projection, t2/t3 the second
// kernel.
hipError_t launch_gemm_ln(const GemmProblem& p, DType dt, hipStream_t stream, hipEvent_t t0 = nullptr,
                          hipEvent_t t1 = nullptr, hipEvent_t t2 = nullptr, hipEvent_t t3 = nullptr);
hipError_t launch_proj_attn(const ProjAttnArgs& a, DType dt, hipStream_t stream, hipEvent_t t0 = nullptr,
                            hipEvent_t t1 = nullptr);
// Backward pass (bf16/f16, head size 64): the dQ kernel (events ev[0..1]),
// then the dK/dV kernel (ev[2..3]); or, when bwd_single_launch, one kernel
// (ev[0..1]); ev may be nullptr.
hipError_t launch_bwd_mfma(const BwdArgs& a, DType dt, hipStream_t stream, hipEvent_t const* ev);
// The same for fp32 with head sizes dk, dv <= kF32MaxHeadDim (vector ALUs).
hipError_t launch_bwd_f32(const BwdArgs& a, int dk, int dv, hipStream_t stream, hipEvent_t const* ev);
hipError_t launch_decode_mfma(const DecodeArgs& a, DType dt, hipStream_t stream, hipEvent_t t0 = nullptr,
                              hipEvent_t t1 = nullptr, hipEvent_t t2 = nullptr, hipEvent_t t3 = nullptr);
// Whether launch_proj_attn handles a problem: head size 64, D a multiple of
// 64, and self-attention with Nq == Nk <= 128 or cross-attention with
// Nq <= 64, Nk <= 128.
inline bool proj_attn_supported(bool self, int Nq, int Nk, int D, int d_k, int d_v) {
  if (D < 64 || D % 64 != 0 || d_k != 64 || d_v != 64 || Nq < 1 || Nk < 1) return false;
  return self ? (Nq == Nk && Nq <= 128) : (Nq <= 64 && Nk <= 128);
}

// Limits the launchers rely on.
constexpr int kF32MaxHeadDim = 128;
constexpr int kMfmaHeadDim = 64;
// Decoding kernel: at most this many query rows per cache head (H / Hkv * Nq);
// one wave per workgroup, three per compute unit (at most one per SIMD): the
// HBM stream is as fast with three as with four, and each wave's range is
// longer, so fewer caches are cut and the start and end cost less (measured:
// 640, 768, 896 and 1024 waves over 8192-slot caches of 16 sequences, 768 the
// fastest at 16 and at 4 cache heads); a partial state is (reference maximum,
// sum, 2 pad, 64 accumulators) in fp32.
constexpr int kDecodeMaxRows = 64;

constexpr int kDecodeWaves = 256 * 3;
constexpr int kDecodePartFloats = 68;

// Built-in device memory of the decoding kernels for callers that cannot
// allocate (mha_decode_forward_noalloc): one array of this many bytes per GPU.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
// The current device's copy of that array (its address is looked up once per
// device); hipSuccess or the runtime's error.
hipError_t decode_scratch(void** ptr);

}  // namespace mha
