// mha_api.cpp -- the C ABI declared in include/mha.h: host-side argument
// validation (no HIP call before it passes), workspace layout, and dispatch to
// the kernels.  Every entry point returns a status; none aborts or throws.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <string>

#include "../../include/mha.h"
#include "mha_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t elem_size(int dtype) { return dtype == MHA_F32 ? 4 : 2; }

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// Checks common to both entry points.
int check_common(int mask_kind, int Nq, int Nk, int dtype, float scale) {
  if (mask_kind != MHA_MASK_NONE && mask_kind != MHA_MASK_CAUSAL)
    return fail(MHA_ERR_INVALID_ARG, "unknown mask_kind %d", mask_kind);
  if (mask_kind == MHA_MASK_CAUSAL && Nq != Nk)
    return fail(MHA_ERR_INVALID_ARG, "the causal mask needs Nq == Nk (got %d, %d)", Nq, Nk);
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16)
    return fail(MHA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!std::isfinite(scale)) return fail(MHA_ERR_INVALID_ARG, "scale must be finite");
  return MHA_OK;
}

constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxBufferBytes = int64_t(1) << 31;

struct ProjLayout {
  size_t q_off, k_off, v_off, o_off, total;
};

// H_kv key/value heads (H_kv == H: one per query head; 0 means H).
bool proj_layout(int B, int Nq, int Nk, int H, int d_k, int d_v, int dtype, ProjLayout* L, int H_kv = 0) {
  if (H_kv == 0) H_kv = H;
  if (B < 0 || Nq < 0 || Nk < 0 || H < 1 || d_k < 1 || d_v < 1) return false;
  if (H_kv < 1 || H_kv > H || H % H_kv) return false;
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16) return false;
  const size_t es = elem_size(dtype);
  const size_t q = round256(size_t(B) * Nq * H * d_k * es);
  const size_t k = round256(size_t(B) * Nk * H_kv * d_k * es);
  const size_t v = round256(size_t(B) * Nk * H_kv * d_v * es);
  const size_t o = round256(size_t(B) * Nq * H * d_v * es);
  L->q_off = 0;
  L->k_off = q;
  L->v_off = q + k;
  L->o_off = q + k + v;
  L->total = q + k + v + o;
  return true;
}

// mha_proj_ln_forward's workspace: the projection path's, then the
// normalisation's per-row tile statistics.
struct LnLayout {
  size_t stats_off, total;
};

LnLayout ln_layout(const ProjLayout& P, int B, int Nq, int D) {
  const int M = B * Nq;
  LnLayout L;
  L.stats_off = P.total;
  L.total = L.stats_off + round256(size_t(M) * mha::ln_stats_stride(D) * 2 * sizeof(float));
  return L;
}


// Element strides (batch, head, row) of the four tensors of a per-head call;
// the feature index is contiguous.
struct Strides4 {
  int64_t q[3], k[3], v[3], o[3];
};

Strides4 dense_strides(int H, int Nq, int Nk, int d_k, int d_v) {
  Strides4 s;
  const int64_t qs[3] = {int64_t(H) * Nq * d_k, int64_t(Nq) * d_k, d_k};
  const int64_t ks[3] = {int64_t(H) * Nk * d_k, int64_t(Nk) * d_k, d_k};
  const int64_t vs[3] = {int64_t(H) * Nk * d_v, int64_t(Nk) * d_v, d_v};
  const int64_t os[3] = {int64_t(H) * Nq * d_v, int64_t(Nq) * d_v, d_v};
  for (int i = 0; i < 3; ++i) {
    s.q[i] = qs[i];
    s.k[i] = ks[i];
    s.v[i] = vs[i];
    s.o[i] = os[i];
  }
  return s;
}

int forward_impl(const void* q, const void* k, const void* v, void* out, int B, int H, int Nq,
                 int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                 int dtype, void* stream, hipEvent_t const* ev, float* lse = nullptr, bool want_lse = false,
                 const Strides4* strides = nullptr, int kv_group = 1) {
  g_last_error.clear();
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(MHA_ERR_INVALID_ARG, "B, H, Nq, Nk must be >= 0 (got %d, %d, %d, %d)", B, H, Nq, Nk);
  if (d_k < 1 || d_v < 1) return fail(MHA_ERR_INVALID_ARG, "d_k, d_v must be >= 1 (got %d, %d)", d_k, d_v);
  int st = check_common(mask_kind, Nq, Nk, dtype, scale);
  if (st) return st;
  if (dtype == MHA_F32) {
    if (d_k > mha::kF32MaxHeadDim || d_v > mha::kF32MaxHeadDim)
      return fail(MHA_ERR_UNSUPPORTED, "fp32 supports d_k, d_v <= %d (got %d, %d)",
                  mha::kF32MaxHeadDim, d_k, d_v);
  } else if (d_k != mha::kMfmaHeadDim || d_v != mha::kMfmaHeadDim) {
    return fail(MHA_ERR_UNSUPPORTED, "bf16/f16 support d_k == d_v == %d (got %d, %d)",
                mha::kMfmaHeadDim, d_k, d_v);
  }
  const Strides4 S = strides ? *strides : dense_strides(H, Nq, Nk, d_k, d_v);
  const int64_t* all[4] = {S.q, S.k, S.v, S.o};
  for (const int64_t* t : all)
    for (int i = 0; i < 3; ++i)
      if (t[i] < 0) return fail(MHA_ERR_INVALID_ARG, "strides must be >= 0");
  if (B == 0 || H == 0 || Nq == 0) return MHA_OK;  // nothing to write
  if (!q || !out) return fail(MHA_ERR_INVALID_ARG, "q and out must be non-null");
  if (Nk > 0 && (!k || !v)) return fail(MHA_ERR_INVALID_ARG, "k and v must be non-null when Nk > 0");
  const uintptr_t align = dtype == MHA_F32 ? 4 : 16;
  if (!aligned(q, align) || !aligned(k, align) || !aligned(v, align) || !aligned(out, align))
    return fail(MHA_ERR_INVALID_ARG, "q, k, v, out must be %d-byte aligned", (int)align);
  if (dtype != MHA_F32)
    for (const int64_t* t : all)
      for (int i = 0; i < 3; ++i)
        if (t[i] % 8) return fail(MHA_ERR_INVALID_ARG, "bf16/f16 strides must be multiples of 8 elements");
  // Output rows must not overlap one another (inputs may share rows).
  if ((Nq > 1 && S.o[2] < d_v) || (H > 1 && S.o[1] < d_v) || (B > 1 && S.o[0] < d_v))
    return fail(MHA_ERR_INVALID_ARG, "output strides must separate the output rows");
  if (key_lens && !aligned(key_lens, 4)) return fail(MHA_ERR_INVALID_ARG, "key_lens must be 4-byte aligned");
  if ((want_lse && !lse) || !aligned(lse, 4))
    return fail(MHA_ERR_INVALID_ARG, "lse must be %s4-byte aligned", want_lse ? "non-null and " : "");
  const int64_t rows_per_block =
      dtype == MHA_F32 ? 4 : mha::attention_block_queries(B, H, Nq, mask_kind == MHA_MASK_CAUSAL);
  if ((Nq + rows_per_block - 1) / rows_per_block * int64_t(H) * B > kMaxBlocks)
    return fail(MHA_ERR_UNSUPPORTED, "problem too large for one launch");
  // The matrix-core kernel addresses one (b, h) slice with 32-bit byte offsets
  // (row strides included, plus the tiles read past the ends).
  if (dtype != MHA_F32 && ((int64_t(Nk) + 128) * std::max<int64_t>(std::max(S.k[2], S.v[2]), d_k) * 2 >= kMaxBufferBytes ||
                           (int64_t(Nq) + 128) * std::max<int64_t>(std::max(S.q[2], S.o[2]), d_k) * 2 >= kMaxBufferBytes))
    return fail(MHA_ERR_UNSUPPORTED, "sequences too long for 32-bit per-head offsets");

  mha::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.key_lens = key_lens;
  a.q_sb = S.q[0];
  a.q_sh = S.q[1];
  a.q_sn = S.q[2];
  a.k_sb = S.k[0];
  a.k_sh = S.k[1];
  a.k_sn = S.k[2];
  a.v_sb = S.v[0];
  a.v_sh = S.v[1];
  a.v_sn = S.v[2];
  a.o_sb = S.o[0];
  a.o_sh = S.o[1];
  a.o_sn = S.o[2];
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.dk = d_k;
  a.dv = d_v;
  a.causal = mask_kind == MHA_MASK_CAUSAL;
  a.scale = scale;
  a.lse = lse;
  a.kv_group = kv_group;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t t0 = ev ? ev[0] : nullptr, t1 = ev ? ev[1] : nullptr;
  hipError_t e = dtype == MHA_F32 ? mha::launch_attn_f32(a, s, t0, t1)
                                  : mha::launch_attn_mfma(a, static_cast<mha::DType>(dtype), s, t0, t1);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return MHA_OK;
}

}  // namespace

extern "C" {

int mha_forward(const void* q, const void* k, const void* v, void* out, int B, int H, int Nq,
                int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                int dtype, void* stream) {
  return forward_impl(q, k, v, out, B, H, Nq, Nk, d_k, d_v, mask_kind, key_lens, scale, dtype,
                      stream, nullptr);
}

int mha_forward_timed(const void* q, const void* k, const void* v, void* out, int B, int H, int Nq,
                      int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                      int dtype, void* stream, void* const* events) {
  return forward_impl(q, k, v, out, B, H, Nq, Nk, d_k, d_v, mask_kind, key_lens, scale, dtype,
                      stream, reinterpret_cast<hipEvent_t const*>(events));
}

int mha_forward_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int Nq,
                    int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                    void* stream) {
  return forward_impl(q, k, v, out, B, H, Nq, Nk, d_k, d_v, mask_kind, key_lens, scale, dtype, stream, nullptr,
                      lse, true);
}

int mha_forward_strided(const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
                        const void* v, const int64_t* v_strides, void* out, const int64_t* out_strides, float* lse,
                        int B, int H, int Nq, int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens,
                        float scale, int dtype, void* stream) {
  g_last_error.clear();
  if (!q_strides || !k_strides || !v_strides || !out_strides)
    return fail(MHA_ERR_INVALID_ARG, "the four stride arrays must be non-null");
  Strides4 S;
  for (int i = 0; i < 3; ++i) {
    S.q[i] = q_strides[i];
    S.k[i] = k_strides[i];
    S.v[i] = v_strides[i];
    S.o[i] = out_strides[i];
  }
  return forward_impl(q, k, v, out, B, H, Nq, Nk, d_k, d_v, mask_kind, key_lens, scale, dtype, stream, nullptr,
                      lse, false, &S);
}

int mha_forward_gqa(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H, int H_kv,
                    int Nq, int Nk, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                    void* stream) {
  g_last_error.clear();
  if (H > 0 && (H_kv < 1 || H_kv > H || H % H_kv))
    return fail(MHA_ERR_INVALID_ARG, "H_kv must divide H (got H = %d, H_kv = %d)", H, H_kv);
  Strides4 S = dense_strides(H, Nq, Nk, d_k, d_v);
  if (H > 0) {
    S.k[0] = int64_t(H_kv) * Nk * d_k;  // k, v: [B, H_kv, Nk, d]
    S.v[0] = int64_t(H_kv) * Nk * d_v;
  }
  return forward_impl(q, k, v, out, B, H, Nq, Nk, d_k, d_v, mask_kind, key_lens, scale, dtype, stream, nullptr,
                      lse, false, &S, H > 0 ? H / H_kv : 1);
}

size_t mha_proj_workspace_bytes(int B, int Nq, int Nk, int D, int H, int d_k, int d_v, int dtype) {
  ProjLayout L;
  if (D < 1 || !proj_layout(B, Nq, Nk, H, d_k, d_v, dtype, &L)) return 0;
  return L.total;
}

}  // extern "C"

namespace {

// Whether the fused projection+attention kernel takes these sizes.
bool fused_supported(bool self, int B, int Nq, int Nk, int D, int d_k, int d_v) {
  return mha::proj_attn_supported(self, Nq, Nk, D, d_k, d_v) && int64_t(B) * Nq * D * 2 < kMaxBufferBytes &&
         int64_t(B) * Nk * D * 2 < kMaxBufferBytes;
}

// Whether the projection path runs as the fused projection+attention kernel
// plus the output projection (short sequences): wherever the fused kernel
// applies, except cross-attention with d_model >= 768 over 65..96 keys, where
// the three-kernel plan measured 2-19% faster.  (Both plans timed on one
// MI355X over cross-attention with B 16-64, Nq 32-64, Nk 64-128, d_model
// 512-1024: the fused plan wins by 8% at d_model 512, ties at 640 and at
// 64 keys, and wins by 20% from 112 keys; self-attention fused at every
// size of that sweep.)
//
// Small batches: the fused kernel's grid is one workgroup per head and 128
// token rows (self-attention: 128 / NPQ sequences of NPQ = 32, 64 or 128
// padded rows) or two sequences (cross-attention), which leaves most compute
// units idle when there are few sequences, while the three-kernel plan spreads
// over many more workgroups.  With D / 64 heads, the fused plan is taken from
// D / 8 workgroups (self-attention) or 256 (cross-attention) on; measured on
// one MI355X, the three kernels were 4-13% faster for self-attention below
// that (B 1-8 at d_model 512, B 4-8 at 1024) and 10-34% for cross-attention
// (B 4-16), the fused kernel 5-20% faster above it.
bool use_fused(bool self, int B, int Nq, int Nk, int D, int d_k, int d_v) {
  if (!fused_supported(self, B, Nq, Nk, D, d_k, d_v) || (!self && D >= 768 && Nk > 64 && Nk <= 96)) return false;
  const int64_t heads = D / 64;
  const int64_t per_wg = self ? 128 / (Nq <= 32 ? 32 : Nq <= 64 ? 64 : 128) : 2;
  const int64_t wgs = (B + per_wg - 1) / per_wg * heads;
  return wgs >= (self ? D / 8 : 256);
}

// The residual connection and layer normalisation after the sublayer
// (mha_proj_ln_forward); nullptr in proj_forward_impl: none.
struct LnSpec {
  const void* gamma;
  const void* beta;
  float eps;
};


// out = O_cat W_O^T + b_O; with ln, out = LayerNorm(x_q + that) * gamma + beta:
// residual and statistics in the projection's epilogue (events 4..5), the
// normalisation in a second pass (events 6..7).  The statistics go to the
// workspace.
int output_projection(const void* O, const void* W_O, const void* b_O, void* out, const void* x_q, int M, int D,
                      int HV, mha::DType dt, hipStream_t s, const LnSpec* ln, char* ws, const LnLayout* lnl,
                      hipEvent_t const* ev) {
  auto evt = [&](int i) -> hipEvent_t { return ev ? ev[i] : nullptr; };
  mha::GemmProblem p{O, W_O, b_O, out, M, D, HV, HV, D};
  hipError_t e;
  if (ln) {
    p.residual = x_q;
    p.gamma = ln->gamma;
    p.beta = ln->beta;
    p.eps = ln->eps;
    p.stats = reinterpret_cast<float2*>(ws + lnl->stats_off);
    e = mha::launch_gemm_ln(p, dt, s, evt(4), evt(5), evt(6), evt(7));
    if (e != hipSuccess) return hip_fail(e, "output projection + normalisation launch");
    return MHA_OK;
  }
  mha::GemmBatch go{};
  go.p[0] = p;
  go.count = 1;
  e = mha::launch_gemm_mfma(go, dt, s, evt(4), evt(5));
  if (e != hipSuccess) return hip_fail(e, "output projection launch");
  return MHA_OK;
}

// mha_proj_forward (and, with ln, mha_proj_ln_forward) with optional profiling
// events (ev == nullptr: none).
int proj_forward_impl(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                      const void* W_V, const void* W_O, const void* b_Q, const void* b_K,
                      const void* b_V, const void* b_O, void* out, int B, int Nq, int Nk, int D,
                      int H, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                      int dtype, void* workspace, size_t workspace_bytes, void* stream,
                      hipEvent_t const* ev, int plan, const LnSpec* ln, int H_kv = 0) {
  g_last_error.clear();
  if (plan < MHA_PLAN_AUTO || plan > MHA_PLAN_FUSED) return fail(MHA_ERR_INVALID_ARG, "unknown plan %d", plan);
  if (H_kv == 0) H_kv = H;
  if (H >= 1 && (H_kv < 1 || H_kv > H || H % H_kv))
    return fail(MHA_ERR_INVALID_ARG, "H_kv must divide H (got H = %d, H_kv = %d)", H, H_kv);
  if (B < 0 || Nq < 0 || Nk < 0)
    return fail(MHA_ERR_INVALID_ARG, "B, Nq, Nk must be >= 0 (got %d, %d, %d)", B, Nq, Nk);
  if (D < 1 || H < 1 || d_k < 1 || d_v < 1)
    return fail(MHA_ERR_INVALID_ARG, "D, H, d_k, d_v must be >= 1 (got %d, %d, %d, %d)", D, H, d_k, d_v);
  if (!x_kv && Nk != Nq)
    return fail(MHA_ERR_INVALID_ARG, "self-attention (x_kv == NULL) needs Nk == Nq (got %d, %d)", Nq, Nk);
  int st = check_common(mask_kind, Nq, Nk, dtype, scale);
  if (st) return st;
  if (dtype == MHA_F32) return fail(MHA_ERR_UNSUPPORTED, "the projection path supports bf16 and f16 only");
  if (d_k != mha::kMfmaHeadDim || d_v != mha::kMfmaHeadDim)
    return fail(MHA_ERR_UNSUPPORTED, "the projection path supports d_k == d_v == %d (got %d, %d)",
                mha::kMfmaHeadDim, d_k, d_v);
  if (D % 8 != 0) return fail(MHA_ERR_UNSUPPORTED, "D must be a multiple of 8 (got %d)", D);
  if (ln && (!std::isfinite(ln->eps) || ln->eps < 0.0f))
    return fail(MHA_ERR_INVALID_ARG, "ln_eps must be finite and >= 0");
  if (B == 0 || Nq == 0) return MHA_OK;  // nothing to write
  if (!x_q || !W_Q || !W_K || !W_V || !W_O || !out)
    return fail(MHA_ERR_INVALID_ARG, "x_q, W_Q, W_K, W_V, W_O and out must be non-null");
  const void* xkv = x_kv ? x_kv : x_q;
  for (const void* p : {x_q, xkv, W_Q, W_K, W_V, W_O, (const void*)out})
    if (!aligned(p, 16)) return fail(MHA_ERR_INVALID_ARG, "x_q, x_kv, W_*, out must be 16-byte aligned");
  for (const void* p : {b_Q, b_K, b_V, b_O})
    if (p && !aligned(p, 2)) return fail(MHA_ERR_INVALID_ARG, "biases must be 2-byte aligned");
  if (ln) {
    if (!aligned(ln->gamma, 16) || !aligned(ln->beta, 16) || !aligned(b_O, 8))
      return fail(MHA_ERR_INVALID_ARG, "ln_gamma and ln_beta must be 16-byte aligned, b_O 8-byte aligned");
  }
  if (key_lens && !aligned(key_lens, 4)) return fail(MHA_ERR_INVALID_ARG, "key_lens must be 4-byte aligned");
  ProjLayout L;
  proj_layout(B, Nq, Nk, H, d_k, d_v, dtype, &L, H_kv);
  const LnLayout LN = ln_layout(L, B, Nq, D);
  const size_t need = ln ? LN.total : L.total;
  if (!workspace) return fail(MHA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(workspace, 256)) return fail(MHA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(MHA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const int64_t nqb = (Nq + 63) / 64;
  if (nqb * H * B > kMaxBlocks || int64_t(B) * std::max(Nq, Nk) > (int64_t(1) << 31) / 64)
    return fail(MHA_ERR_UNSUPPORTED, "problem too large for one launch");
  // 32-bit byte offsets: a 256-row tile of x or W, and one head's rows of the
  // projected Q, K, V (row stride H*d) must each span less than 2^31 bytes.
  const int64_t hd = int64_t(H) * std::max(d_k, d_v);
  if (256 * int64_t(std::max<int64_t>(D, hd)) * 2 >= kMaxBufferBytes ||
      (int64_t(std::max(Nq, Nk)) + 128) * hd * 2 >= kMaxBufferBytes)
    return fail(MHA_ERR_UNSUPPORTED, "dimensions too large for 32-bit tile offsets");

  char* ws = static_cast<char*>(workspace);
  void* Qw = ws + L.q_off;
  void* Kw = ws + L.k_off;
  void* Vw = ws + L.v_off;
  void* Ow = ws + L.o_off;
  const int HK = H * d_k, HV = H * d_v;
  const int HKk = H_kv * d_k, HVk = H_kv * d_v;  // widths of the projected K and V rows
  hipStream_t s = static_cast<hipStream_t>(stream);
  const mha::DType dt = static_cast<mha::DType>(dtype);

  auto evt = [&](int i) -> hipEvent_t { return ev ? ev[i] : nullptr; };

  // Short sequences: projections and attention in one fused launch that
  // writes the head-major concatenation directly, then the output projection.
  if (plan == MHA_PLAN_FUSED && !fused_supported(xkv == x_q, B, Nq, Nk, D, d_k, d_v))
    return fail(MHA_ERR_UNSUPPORTED, "these sizes have no fused projection+attention kernel");
  if (plan == MHA_PLAN_FUSED || (plan == MHA_PLAN_AUTO && use_fused(xkv == x_q, B, Nq, Nk, D, d_k, d_v))) {
    mha::ProjAttnArgs pa{};
    pa.xq = x_q;
    pa.xkv = xkv;
    pa.wq = W_Q;
    pa.wk = W_K;
    pa.wv = W_V;
    pa.bq = b_Q;
    pa.bk = b_K;
    pa.bv = b_V;
    pa.o = Ow;
    pa.key_lens = key_lens;
    pa.B = B;
    pa.Nq = Nq;
    pa.Nk = Nk;
    pa.D = D;
    pa.H = H;
    pa.causal = mask_kind == MHA_MASK_CAUSAL;
    pa.scale = scale;
    pa.kv_group = H / H_kv;
    hipError_t e = mha::launch_proj_attn(pa, dt, s, evt(0), evt(1));
    if (e != hipSuccess) return hip_fail(e, "fused projection/attention launch");
    return output_projection(Ow, W_O, b_O, out, x_q, B * Nq, D, HV, dt, s, ln, ws, &LN, ev);
  }

  // 1. Q, K, V projections in one launch; outputs row-major [B*N, H*d].
  mha::GemmBatch g{};
  g.p[0] = {x_q, W_Q, b_Q, Qw, B * Nq, HK, D, D, HK};
  g.p[1] = {xkv, W_K, b_K, Kw, B * Nk, HKk, D, D, HKk};
  g.p[2] = {xkv, W_V, b_V, Vw, B * Nk, HVk, D, D, HVk};
  g.count = 3;
  hipError_t e = mha::launch_gemm_mfma(g, dt, s, evt(0), evt(1));
  if (e != hipSuccess) return hip_fail(e, "Q/K/V projection launch");

  // 2. Attention per head, reading the projections in place (head h = columns
  //    [h*d, (h+1)*d)) and writing the head-major concatenation [B*Nq, H*d_v].
  mha::AttnArgs a{};
  a.q = Qw;
  a.k = Kw;
  a.v = Vw;
  a.out = Ow;
  a.key_lens = key_lens;
  a.q_sn = HK;
  a.q_sh = d_k;
  a.q_sb = int64_t(Nq) * HK;
  a.k_sn = HKk;
  a.k_sh = d_k;
  a.k_sb = int64_t(Nk) * HKk;
  a.v_sn = HVk;
  a.v_sh = d_v;
  a.v_sb = int64_t(Nk) * HVk;
  a.kv_group = H / H_kv;  // query head h reads key/value head h / (H / H_kv)
  a.o_sn = HV;
  a.o_sh = d_v;
  a.o_sb = int64_t(Nq) * HV;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.dk = d_k;
  a.dv = d_v;
  a.causal = mask_kind == MHA_MASK_CAUSAL;
  a.scale = scale;
  e = mha::launch_attn_mfma(a, dt, s, evt(2), evt(3));
  if (e != hipSuccess) return hip_fail(e, "attention launch");

  // 3. Output projection (and the residual connection and normalisation).
  return output_projection(Ow, W_O, b_O, out, x_q, B * Nq, D, HV, dt, s, ln, ws, &LN, ev);
}

}  // namespace

extern "C" {

int mha_proj_forward(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                     const void* W_V, const void* W_O, const void* b_Q, const void* b_K,
                     const void* b_V, const void* b_O, void* out, int B, int Nq, int Nk, int D,
                     int H, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return proj_forward_impl(x_q, x_kv, W_Q, W_K, W_V, W_O, b_Q, b_K, b_V, b_O, out, B, Nq, Nk, D, H,
                           d_k, d_v, mask_kind, key_lens, scale, dtype, workspace, workspace_bytes,
                           stream, nullptr, MHA_PLAN_AUTO, nullptr);
}

int mha_proj_forward_timed(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                           const void* W_V, const void* W_O, const void* b_Q, const void* b_K,
                           const void* b_V, const void* b_O, void* out, int B, int Nq, int Nk,
                           int D, int H, int d_k, int d_v, int mask_kind, const int32_t* key_lens,
                           float scale, int dtype, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* events, int plan) {
  return proj_forward_impl(x_q, x_kv, W_Q, W_K, W_V, W_O, b_Q, b_K, b_V, b_O, out, B, Nq, Nk, D, H,
                           d_k, d_v, mask_kind, key_lens, scale, dtype, workspace, workspace_bytes,
                           stream, reinterpret_cast<hipEvent_t const*>(events), plan, nullptr);
}

int mha_proj_ln_forward(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K, const void* W_V,
                        const void* W_O, const void* b_Q, const void* b_K, const void* b_V, const void* b_O,
                        const void* ln_gamma, const void* ln_beta, float ln_eps, void* out, int B, int Nq, int Nk,
                        int D, int H, int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const LnSpec ln{ln_gamma, ln_beta, ln_eps};
  return proj_forward_impl(x_q, x_kv, W_Q, W_K, W_V, W_O, b_Q, b_K, b_V, b_O, out, B, Nq, Nk, D, H, d_k, d_v,
                           mask_kind, key_lens, scale, dtype, workspace, workspace_bytes, stream, nullptr,
                           MHA_PLAN_AUTO, &ln);
}

int mha_proj_ln_forward_timed(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                              const void* W_V, const void* W_O, const void* b_Q, const void* b_K, const void* b_V,
                              const void* b_O, const void* ln_gamma, const void* ln_beta, float ln_eps, void* out,
                              int B, int Nq, int Nk, int D, int H, int d_k, int d_v, int mask_kind,
                              const int32_t* key_lens, float scale, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream, void* const* events, int plan) {
  const LnSpec ln{ln_gamma, ln_beta, ln_eps};
  return proj_forward_impl(x_q, x_kv, W_Q, W_K, W_V, W_O, b_Q, b_K, b_V, b_O, out, B, Nq, Nk, D, H, d_k, d_v,
                           mask_kind, key_lens, scale, dtype, workspace, workspace_bytes, stream,
                           reinterpret_cast<hipEvent_t const*>(events), plan, &ln);
}

size_t mha_proj_ln_workspace_bytes(int B, int Nq, int Nk, int D, int H, int d_k, int d_v, int dtype) {
  ProjLayout L;
  if (D < 1 || !proj_layout(B, Nq, Nk, H, d_k, d_v, dtype, &L)) return 0;
  return ln_layout(L, B, Nq, D).total;
}

int mha_proj_fused(int B, int Nq, int Nk, int D, int d_k, int d_v, int self_attention) {
  return use_fused(self_attention != 0, B, Nq, Nk, D, d_k, d_v) ? 1 : 0;
}

int mha_forward_block_queries(int B, int H, int Nq, int mask_kind, int dtype) {
  if (B < 1 || H < 1 || Nq < 1 || (mask_kind != MHA_MASK_NONE && mask_kind != MHA_MASK_CAUSAL)) return 0;
  if (dtype == MHA_F32) return 4;
  if (dtype != MHA_BF16 && dtype != MHA_F16) return 0;
  return mha::attention_block_queries(B, H, Nq, mask_kind == MHA_MASK_CAUSAL);
}

size_t mha_proj_gqa_workspace_bytes(int B, int Nq, int Nk, int D, int H, int H_kv, int d_k, int d_v, int dtype) {
  ProjLayout L;
  if (D < 1 || H_kv < 1 || !proj_layout(B, Nq, Nk, H, d_k, d_v, dtype, &L, H_kv)) return 0;
  return L.total;
}

int mha_proj_forward_gqa(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K, const void* W_V,
                         const void* W_O, const void* b_Q, const void* b_K, const void* b_V, const void* b_O,
                         void* out, int B, int Nq, int Nk, int D, int H, int H_kv, int d_k, int d_v, int mask_kind,
                         const int32_t* key_lens, float scale, int dtype, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (H_kv < 1) {
    g_last_error.clear();
    return fail(MHA_ERR_INVALID_ARG, "H_kv must divide H (got H = %d, H_kv = %d)", H, H_kv);
  }
  return proj_forward_impl(x_q, x_kv, W_Q, W_K, W_V, W_O, b_Q, b_K, b_V, b_O, out, B, Nq, Nk, D, H, d_k, d_v,
                           mask_kind, key_lens, scale, dtype, workspace, workspace_bytes, stream, nullptr,
                           MHA_PLAN_AUTO, nullptr, H_kv);
}

int mha_proj_forward_gqa_timed(const void* x_q, const void* x_kv, const void* W_Q, const void* W_K,
                               const void* W_V, const void* W_O, const void* b_Q, const void* b_K, const void* b_V,
                               const void* b_O, void* out, int B, int Nq, int Nk, int D, int H, int H_kv, int d_k,
                               int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                               void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  if (H_kv < 1) {
    g_last_error.clear();
    return fail(MHA_ERR_INVALID_ARG, "H_kv must divide H (got H = %d, H_kv = %d)", H, H_kv);
  }
  return proj_forward_impl(x_q, x_kv, W_Q, W_K, W_V, W_O, b_Q, b_K, b_V, b_O, out, B, Nq, Nk, D, H, d_k, d_v,
                           mask_kind, key_lens, scale, dtype, workspace, workspace_bytes, stream,
                           reinterpret_cast<hipEvent_t const*>(events), MHA_PLAN_AUTO, nullptr, H_kv);
}

}  // extern "C"

namespace {

// Workspace of the backward pass: D_i = dout_i . out_i per row, fp32
// [B, H, Nq]; then, when the dK/dV pass splits the query heads of each shared
// key/value head into runs (bf16/f16), the runs' fp32 sums of dK and dV,
// [2][parts][B*H_kv][Nk][64].
size_t backward_dsum_bytes(int B, int H, int Nq) { return round256(size_t(B) * H * Nq * sizeof(float)); }
int backward_parts(int B, int H, int H_kv, int Nq, int Nk, int dtype) {
  return dtype == MHA_F32 || Nq == 0 ? 1 : mha::bwd_head_parts(B, H, H_kv, Nk);
}
size_t backward_workspace(int B, int H, int H_kv, int Nq, int Nk, int dtype) {
  const int P = backward_parts(B, H, H_kv, Nq, Nk, dtype);
  const size_t part = P > 1 ? round256(size_t(2) * P * B * H_kv * Nk * mha::kMfmaHeadDim * sizeof(float)) : 0;
  return backward_dsum_bytes(B, H, Nq) + part;
}

int backward_impl(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq, int Nk, int d_k, int d_v,
                  int mask_kind, const int32_t* key_lens, float scale, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream, hipEvent_t const* ev) {
  g_last_error.clear();
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(MHA_ERR_INVALID_ARG, "B, H, Nq, Nk must be >= 0 (got %d, %d, %d, %d)", B, H, Nq, Nk);
  if (H > 0 && (H_kv < 1 || H_kv > H || H % H_kv))
    return fail(MHA_ERR_INVALID_ARG, "H_kv must divide H (got H = %d, H_kv = %d)", H, H_kv);
  if (d_k < 1 || d_v < 1) return fail(MHA_ERR_INVALID_ARG, "d_k, d_v must be >= 1 (got %d, %d)", d_k, d_v);
  int st = check_common(mask_kind, Nq, Nk, dtype, scale);
  if (st) return st;
  if (dtype == MHA_F32) {
    if (d_k > mha::kF32MaxHeadDim || d_v > mha::kF32MaxHeadDim)
      return fail(MHA_ERR_UNSUPPORTED, "fp32 supports d_k, d_v <= %d (got %d, %d)", mha::kF32MaxHeadDim, d_k, d_v);
  } else if (d_k != mha::kMfmaHeadDim || d_v != mha::kMfmaHeadDim) {
    return fail(MHA_ERR_UNSUPPORTED, "bf16/f16 support d_k == d_v == %d (got %d, %d)", mha::kMfmaHeadDim, d_k, d_v);
  }
  if (B == 0 || H == 0 || (Nq == 0 && Nk == 0)) return MHA_OK;  // nothing to write
  if (Nq > 0 && (!q || !out || !dout || !lse || !dq))
    return fail(MHA_ERR_INVALID_ARG, "q, out, dout, lse and dq must be non-null when Nq > 0");
  if (Nk > 0 && (!k || !v || !dk || !dv))
    return fail(MHA_ERR_INVALID_ARG, "k, v, dk and dv must be non-null when Nk > 0");
  const uintptr_t align = dtype == MHA_F32 ? 4 : 16;
  for (const void* p : {q, k, v, out, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned(p, align))
      return fail(MHA_ERR_INVALID_ARG, "q, k, v, out, dout, dq, dk, dv must be %d-byte aligned", (int)align);
  if (!aligned(lse, 4)) return fail(MHA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (key_lens && !aligned(key_lens, 4)) return fail(MHA_ERR_INVALID_ARG, "key_lens must be 4-byte aligned");
  // 32-bit byte offsets within one head, plus the tile read past its end.
  if (dtype != MHA_F32 && (int64_t(std::max(Nq, Nk)) + 128) * d_k * 2 >= kMaxBufferBytes)
    return fail(MHA_ERR_UNSUPPORTED, "sequences too long for 32-bit per-head offsets");
  const int64_t rows_per_block = dtype == MHA_F32 ? 4 : 64;
  if ((int64_t(std::max(Nq, Nk)) + rows_per_block - 1) / rows_per_block * int64_t(H) * B > kMaxBlocks ||
      int64_t(B) * H_kv * Nk / 16 > kMaxBlocks)
    return fail(MHA_ERR_UNSUPPORTED, "problem too large for one launch");
  const size_t need = backward_workspace(B, H, H_kv, Nq, Nk, dtype);
  if (need > 0) {
    if (!workspace) return fail(MHA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(workspace, 256)) return fail(MHA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
      return fail(MHA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  }
  mha::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsum = static_cast<float*>(workspace);
  a.parts = backward_parts(B, H, H_kv, Nq, Nk, dtype);
  a.part = a.parts > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + backward_dsum_bytes(B, H, Nq))
                       : nullptr;
  a.key_lens = key_lens;
  a.B = B;
  a.H = H;
  a.Hkv = H_kv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.causal = mask_kind == MHA_MASK_CAUSAL;
  a.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dtype == MHA_F32 ? mha::launch_bwd_f32(a, d_k, d_v, s, ev)
                                  : mha::launch_bwd_mfma(a, static_cast<mha::DType>(dtype), s, ev);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return MHA_OK;
}

}  // namespace

extern "C" {

size_t mha_backward_workspace_bytes(int B, int H, int Nq, int Nk, int d_k, int d_v, int dtype) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d_k < 1 || d_v < 1) return 0;
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16) return 0;
  return backward_workspace(B, H, H, Nq, Nk, dtype);
}

int mha_backward_single_launch(int B, int H, int H_kv, int Nq, int Nk, int d_k, int d_v, int dtype) {
  if (B < 1 || H < 1 || d_k != mha::kMfmaHeadDim || d_v != mha::kMfmaHeadDim) return 0;
  if (dtype != MHA_BF16 && dtype != MHA_F16) return 0;
  return mha::bwd_single_launch(H, H_kv, Nq, Nk) ? 1 : 0;
}

size_t mha_backward_gqa_workspace_bytes(int B, int H, int H_kv, int Nq, int Nk, int d_k, int d_v, int dtype) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d_k < 1 || d_v < 1) return 0;
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16) return 0;
  if (H > 0 && (H_kv < 1 || H_kv > H || H % H_kv)) return 0;
  return backward_workspace(B, H, H > 0 ? H_kv : 1, Nq, Nk, dtype);
}

int mha_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d_k, int d_v, int mask_kind,
                 const int32_t* key_lens, float scale, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return backward_impl(q, k, v, out, dout, lse, dq, dk, dv, B, H, H, Nq, Nk, d_k, d_v, mask_kind, key_lens, scale,
                       dtype, workspace, workspace_bytes, stream, nullptr);
}

int mha_backward_gqa(const void* q, const void* k, const void* v, const void* out, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq, int Nk,
                     int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, out, dout, lse, dq, dk, dv, B, H, H_kv, Nq, Nk, d_k, d_v, mask_kind, key_lens,
                       scale, dtype, workspace, workspace_bytes, stream, nullptr);
}

int mha_backward_gqa_timed(const void* q, const void* k, const void* v, const void* out, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int Nq, int Nk,
                           int d_k, int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  return backward_impl(q, k, v, out, dout, lse, dq, dk, dv, B, H, H_kv, Nq, Nk, d_k, d_v, mask_kind, key_lens,
                       scale, dtype, workspace, workspace_bytes, stream, reinterpret_cast<hipEvent_t const*>(events));
}

int mha_backward_timed(const void* q, const void* k, const void* v, const void* out, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d_k,
                       int d_v, int mask_kind, const int32_t* key_lens, float scale, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream, void* const* events) {
  return backward_impl(q, k, v, out, dout, lse, dq, dk, dv, B, H, H, Nq, Nk, d_k, d_v, mask_kind, key_lens, scale,
                       dtype, workspace, workspace_bytes, stream, reinterpret_cast<hipEvent_t const*>(events));
}

}  // extern "C"

namespace {

// How mha_decode_forward runs a problem: the balanced decoding kernel for
// bf16/f16 head size 64 with at most kDecodeMaxRows query rows per cache head,
// else the attention kernels (with shared key/value heads and the causal mask
// anchored at the end of the cache).  A pure function of the sizes, so the
// workspace query and the call agree.  Workspace: one partial state per
// (cache + wave) and row, then one span entry per cache.
struct DecodePlan {
  bool split_kernel;
  int waves;
  size_t span_off, workspace;
};

DecodePlan decode_plan(int B, int H, int H_kv, int Nq, int d_k, int d_v, int dtype) {
  DecodePlan p{false, 0, 0, 0};
  if (dtype == MHA_F32 || d_k != mha::kMfmaHeadDim || d_v != mha::kMfmaHeadDim) return p;
  const int64_t R = int64_t(H / H_kv) * Nq;
  if (R > mha::kDecodeMaxRows) return p;
  p.split_kernel = true;
  p.waves = mha::kDecodeWaves;
  const size_t caches = size_t(B) * H_kv;
  p.span_off = round256((caches + p.waves) * R * mha::kDecodePartFloats * sizeof(float));
  p.workspace = p.span_off + round256(caches * 2 * sizeof(int32_t));
  return p;
}

int check_decode_sizes(int B, int H, int H_kv, int Nq, int S, int d_k, int d_v) {
  if (B < 0 || Nq < 0 || S < 0)
    return fail(MHA_ERR_INVALID_ARG, "B, Nq, S must be >= 0 (got %d, %d, %d)", B, Nq, S);
  if (H < 1 || H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(MHA_ERR_INVALID_ARG, "need 1 <= H_kv <= H with H a multiple of H_kv (got H=%d, H_kv=%d)", H, H_kv);
  if (d_k < 1 || d_v < 1) return fail(MHA_ERR_INVALID_ARG, "d_k, d_v must be >= 1 (got %d, %d)", d_k, d_v);
  return MHA_OK;
}

int decode_forward_impl(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int H,
                        int H_kv, int Nq, int S, int d_k, int d_v, int mask_kind, const int32_t* cache_lens,
                        float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                        hipEvent_t const* ev, bool builtin_scratch = false) {
  g_last_error.clear();
  int st = check_decode_sizes(B, H, H_kv, Nq, S, d_k, d_v);
  if (st) return st;
  if (mask_kind != MHA_MASK_NONE && mask_kind != MHA_MASK_CAUSAL)
    return fail(MHA_ERR_INVALID_ARG, "unknown mask_kind %d", mask_kind);
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16)
    return fail(MHA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!std::isfinite(scale)) return fail(MHA_ERR_INVALID_ARG, "scale must be finite");
  if (dtype == MHA_F32) {
    if (d_k > mha::kF32MaxHeadDim || d_v > mha::kF32MaxHeadDim)
      return fail(MHA_ERR_UNSUPPORTED, "fp32 supports d_k, d_v <= %d (got %d, %d)", mha::kF32MaxHeadDim, d_k, d_v);
  } else if (d_k != mha::kMfmaHeadDim || d_v != mha::kMfmaHeadDim) {
    return fail(MHA_ERR_UNSUPPORTED, "bf16/f16 support d_k == d_v == %d (got %d, %d)", mha::kMfmaHeadDim, d_k,
                d_v);
  }
  if (B == 0 || Nq == 0) return MHA_OK;  // nothing to write
  if (!q || !out) return fail(MHA_ERR_INVALID_ARG, "q and out must be non-null");
  if (S > 0 && (!k_cache || !v_cache))
    return fail(MHA_ERR_INVALID_ARG, "k_cache and v_cache must be non-null when S > 0");
  const uintptr_t align = dtype == MHA_F32 ? 4 : 16;
  if (!aligned(q, align) || !aligned(k_cache, align) || !aligned(v_cache, align) || !aligned(out, align))
    return fail(MHA_ERR_INVALID_ARG, "q, k_cache, v_cache, out must be %d-byte aligned", (int)align);
  if (cache_lens && !aligned(cache_lens, 4)) return fail(MHA_ERR_INVALID_ARG, "cache_lens must be 4-byte aligned");
  // 32-bit byte offsets within one cache head (plus the loads past its end).
  if ((int64_t(S) + 1024) * std::max(d_k, d_v) * elem_size(dtype) >= kMaxBufferBytes)
    return fail(MHA_ERR_UNSUPPORTED, "cache too long for 32-bit per-head offsets");

  const DecodePlan plan = decode_plan(B, H, H_kv, Nq, d_k, d_v, dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto evt = [&](int i) -> hipEvent_t { return ev ? ev[i] : nullptr; };
  if (plan.split_kernel) {
    if (int64_t(B) * H * Nq / 4 > kMaxBlocks || int64_t(B) * H_kv + plan.waves > (int64_t(1) << 31) / 64)
      return fail(MHA_ERR_UNSUPPORTED, "problem too large for one launch");
    if (builtin_scratch) {
      // mha_decode_forward_noalloc: the library's own per-device array.
      if (plan.workspace > mha::kDecodeScratchBytes)
        return fail(MHA_ERR_UNSUPPORTED,
                    "this step needs %zu bytes of scratch; the built-in scratch holds %zu "
                    "(call mha_decode_forward with a workspace)",
                    plan.workspace, mha::kDecodeScratchBytes);
      hipError_t e = mha::decode_scratch(&workspace);
      if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
      workspace_bytes = mha::kDecodeScratchBytes;
    }
    if (!workspace) return fail(MHA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", plan.workspace);
    if (!aligned(workspace, 256)) return fail(MHA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < plan.workspace)
      return fail(MHA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, plan.workspace);
    mha::DecodeArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.out = out;
    a.cache_lens = cache_lens;
    a.part = static_cast<float*>(workspace);
    a.span = reinterpret_cast<int2*>(static_cast<char*>(workspace) + plan.span_off);
    a.B = B;
    a.H = H;
    a.Hkv = H_kv;
    a.Nq = Nq;
    a.S = S;
    a.causal = mask_kind == MHA_MASK_CAUSAL;
    a.scale = scale;
    a.waves = plan.waves;
    hipError_t e = mha::launch_decode_mfma(a, static_cast<mha::DType>(dtype), s, evt(0), evt(1), evt(2), evt(3));
    if (e != hipSuccess) return hip_fail(e, "decoding launch");
    return MHA_OK;
  }

  const int64_t rows_per_block =
      dtype == MHA_F32 ? 4 : mha::attention_block_queries(B, H, Nq, mask_kind == MHA_MASK_CAUSAL);
  if ((Nq + rows_per_block - 1) / rows_per_block * int64_t(H) * B > kMaxBlocks)
    return fail(MHA_ERR_UNSUPPORTED, "problem too large for one launch");
  mha::AttnArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.key_lens = cache_lens;
  a.q_sn = d_k;
  a.q_sh = int64_t(Nq) * d_k;
  a.q_sb = int64_t(H) * Nq * d_k;
  a.k_sn = d_k;
  a.k_sh = int64_t(S) * d_k;
  a.k_sb = int64_t(H_kv) * S * d_k;
  a.v_sn = d_v;
  a.v_sh = int64_t(S) * d_v;
  a.v_sb = int64_t(H_kv) * S * d_v;
  a.o_sn = d_v;
  a.o_sh = int64_t(Nq) * d_v;
  a.o_sb = int64_t(H) * Nq * d_v;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = S;
  a.dk = d_k;
  a.dv = d_v;
  a.causal = mask_kind == MHA_MASK_CAUSAL;
  a.scale = scale;
  a.kv_group = H / H_kv;
  a.causal_end = 1;
  hipError_t e = dtype == MHA_F32 ? mha::launch_attn_f32(a, s, evt(0), evt(1))
                                  : mha::launch_attn_mfma(a, static_cast<mha::DType>(dtype), s, evt(0), evt(1));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return MHA_OK;
}

}  // namespace

extern "C" {

size_t mha_decode_workspace_bytes(int B, int H, int H_kv, int Nq, int S, int d_k, int d_v, int dtype) {
  if (B < 0 || Nq < 0 || S < 0 || H < 1 || H_kv < 1 || H_kv > H || H % H_kv != 0 || d_k < 1 || d_v < 1)
    return 0;
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16) return 0;
  return decode_plan(B, H, H_kv, Nq, d_k, d_v, dtype).workspace;
}

int mha_decode_forward(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int H,
                       int H_kv, int Nq, int S, int d_k, int d_v, int mask_kind, const int32_t* cache_lens,
                       float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_forward_impl(q, k_cache, v_cache, out, B, H, H_kv, Nq, S, d_k, d_v, mask_kind, cache_lens, scale,
                             dtype, workspace, workspace_bytes, stream, nullptr);
}

int mha_decode_forward_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int H,
                               int H_kv, int Nq, int S, int d_k, int d_v, int mask_kind, const int32_t* cache_lens,
                               float scale, int dtype, void* stream) {
  return decode_forward_impl(q, k_cache, v_cache, out, B, H, H_kv, Nq, S, d_k, d_v, mask_kind, cache_lens, scale,
                             dtype, nullptr, 0, stream, nullptr, true);
}

int mha_decode_forward_timed(const void* q, const void* k_cache, const void* v_cache, void* out, int B, int H,
                             int H_kv, int Nq, int S, int d_k, int d_v, int mask_kind, const int32_t* cache_lens,
                             float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events) {
  return decode_forward_impl(q, k_cache, v_cache, out, B, H, H_kv, Nq, S, d_k, d_v, mask_kind, cache_lens, scale,
                             dtype, workspace, workspace_bytes, stream, reinterpret_cast<hipEvent_t const*>(events));
}

int mha_decode_split(int B, int H, int H_kv, int Nq, int S, int d_k, int d_v, int dtype) {
  if (B < 0 || Nq < 0 || S < 0 || H < 1 || H_kv < 1 || H_kv > H || H % H_kv != 0 || d_k < 1 || d_v < 1)
    return 0;
  if (dtype != MHA_F32 && dtype != MHA_BF16 && dtype != MHA_F16) return 0;
  const DecodePlan p = decode_plan(B, H, H_kv, Nq, d_k, d_v, dtype);
  return p.split_kernel ? p.waves : 0;
}

const char* mha_status_string(int status) {
  switch (status) {
    case MHA_OK: return "ok";
    case MHA_ERR_INVALID_ARG: return "invalid argument";
    case MHA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MHA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MHA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mha_last_error_message(void) { return g_last_error.c_str(); }

const char* mha_last_error(void) { return g_last_error.c_str(); }

int mha_version(void) { return 200; }

}  // extern "C"
