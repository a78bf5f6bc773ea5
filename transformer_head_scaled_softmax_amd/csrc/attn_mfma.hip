// attn_mfma.hip -- bf16 / fp16 scaled dot-product attention, head size 64, on
// the gfx950 matrix cores (v_mfma_f32_32x32x16_{bf16,f16}).
//
// What is computed is the pages' formula, softmax(scale * Q K^T) V per head
// ("Scaled Dot-Product Attention: Step by Step", trishampatil.com), with
// padded keys j >= L and, under the causal mask, future keys j > i given
// weight exactly 0 ("Why Masking Is Required", trishampatil.com; "Two masks,
// not one", alexdo.xyz).  The score matrix never leaves registers: keys are
// streamed through LDS in tiles of 64 and the row softmax is carried as a
// running maximum and sum (an exact rearrangement of the same result).
//
// Work split.  A workgroup owns 32*NW consecutive queries of one (b, h); each
// wave owns 32 of them.  Per key tile a wave computes the TRANSPOSED scores
// S^T (64 keys x 32 queries) = K_tile * Q^T, so that each lane ends up holding
// 32 scores of one query (lanes l and l+32 share a query and split its keys).
// That layout is exactly the B operand of the second product
// O^T (64 features x 32 queries) += V^T * P^T, so the probabilities P go from
// the score accumulators to the second MFMA without touching LDS.  V is
// stored transposed in LDS when the tile is staged so both MFMA operands read
// contiguous 8-byte or 16-byte runs.
//
// MFMA 32x32x16 lane layout (checked on the device): A[m][k] comes from lane
// m + 32*(k/8), element k%8; B[k][n] from lane n + 32*(k/8), element k%8;
// C[m][n] lands in lane n + 32*((m/4)%2), register 4*(m/8) + m%4.
//
// Softmax bookkeeping, per query: m_ref is the running reference maximum (in
// log2 units), p = exp2(s * scale * log2e - m_ref).  m_ref is raised (and the
// accumulators rescaled) only when a tile's maximum exceeds it by more than
// kLazyLog2 -- otherwise p may grow up to 2^kLazyLog2, which fp32 holds
// exactly as well; the final division by the running sum cancels m_ref.
#include "mha_internal.h"

namespace mha {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kD = kMfmaHeadDim;  // 64
constexpr int kBN = 64;           // keys per tile
constexpr int kKS = 72;           // K tile row stride (elements): 144 B -> conflict-free 16 B reads
constexpr int kVS = 68;           // V^T tile row stride (elements): 136 B -> conflict-free 8 B reads
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyLog2 = 8.0f;

struct BF16 {
  __device__ static f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float x, float y) {  // round to nearest even
    bf16x2_t r = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, r);
  }
};

struct F16 {
  __device__ static f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float x, float y) {
    f16x2_t r = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, r);
  }
};

__device__ inline float lanes_max(float x) {  // max over lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float lanes_sum(float x) {  // sum over lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <class Op, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_mfma_kernel(AttnArgs a, int nqb) {
  constexpr int NT = NW * 64;
  constexpr int QB = NW * 32;
  constexpr int KCH = (kBN * 8) / NT;       // 16-byte K chunks per thread per tile
  constexpr int VCH = (kBN / 2 * 8) / NT;   // 16-byte chunk pairs (two key rows) of V
  static_assert(KCH >= 1 && VCH >= 1, "tile too small for the workgroup");

  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kBN * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kD * kVS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;

  // Longest query blocks first: under the causal mask later blocks see more keys.
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int b = bh / a.H, h = bh % a.H;

  int L = a.Nk;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), a.Nk);
  const int q0 = qb * QB;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + col;
  const bool qvalid = qi < a.Nq;
  const int kend = a.causal ? min(L, qi + 1) : L;               // keys this query sees
  const int kend_blk = a.causal ? min(L, min(q0 + QB, a.Nq)) : L;  // keys the block needs
  const int kmin_wave = a.causal ? min(L, qw0 + 1) : L;          // tiles below: no masking
  const int ntiles = (kend_blk + kBN - 1) / kBN;

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + b * a.q_sb + h * a.q_sh;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.k_sb + h * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.v_sb + h * a.v_sh;

  // This lane's query as the B operand of S^T = K Q^T: features 16kk + 8half .. +7.
  // A negative scale is folded in by negating q (exact), so the softmax below
  // always multiplies by a non-negative c2.
  const uint32_t qsign = a.scale < 0.0f ? 0x80008000u : 0u;
  const float c2 = fabsf(a.scale) * kLog2e;
  u32x4_t qreg[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (qvalid) v = *reinterpret_cast<const u32x4_t*>(qbase + (int64_t)qi * a.q_sn + kk * 16 + half * 8);
    qreg[kk] = v ^ qsign;
  }

  u32x4_t kreg[KCH];
  u32x4_t vreg[VCH][2];
  auto load_tile = [&](int t) {
    const int j0 = t * kBN;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT, row = idx >> 3, ch = idx & 7, j = j0 + row;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j < kend_blk) v = *reinterpret_cast<const u32x4_t*>(kbase + (int64_t)j * a.k_sn + ch * 8);
      kreg[c] = v;
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = tid + c * NT, pr = idx >> 3, ch = idx & 7, j = j0 + 2 * pr;
      u32x4_t v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
      if (j < kend_blk) v0 = *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)j * a.v_sn + ch * 8);
      if (j + 1 < kend_blk) v1 = *reinterpret_cast<const u32x4_t*>(vbase + (int64_t)(j + 1) * a.v_sn + ch * 8);
      vreg[c][0] = v0;
      vreg[c][1] = v1;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + c * NT, row = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4_t*>(&ks[buf][row * kKS + ch * 8]) = kreg[c];
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = tid + c * NT, pr = idx >> 3, ch = idx & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = vreg[c][0][e >> 1], w1 = vreg[c][1][e >> 1];
        const uint32_t pair = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
        *reinterpret_cast<uint32_t*>(&vt[buf][(ch * 8 + e) * kVS + 2 * pr]) = pair;
      }
    }
  };

  f32x16_t o[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;
  float m_ref = -INFINITY, lsum = 0.0f;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * kBN;
    if (t + 1 < ntiles) load_tile(t + 1);

    // S^T = K_tile Q^T: two 32-key blocks.
    f32x16_t s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[jb][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(&ks[buf][(jb * 32 + col) * kKS + kk * 16 + half * 8]);
        s[jb] = Op::mma(av, qreg[kk], s[jb]);
      }
    }

    // Register (jb, r) of this lane holds key j0 + 32jb + 8(r/4) + 4half + r%4.
    const bool masked = j0 + kBN > kmin_wave;  // wave-uniform
    const int lim = kend - j0 - 4 * half;
    float mx = -INFINITY;
    if (masked) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = jb * 32 + (r >> 2) * 8 + (r & 3);
          if (off >= lim) s[jb][r] = -INFINITY;
          mx = fmaxf(mx, s[jb][r]);
        }
    } else {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
    }
    mx = lanes_max(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c2;

    // Each query decides for itself (never because of another row of the
    // wave), so a row's arithmetic does not depend on its neighbours' data.
    const bool need = mt > m_ref + kLazyLog2;  // implies mt is finite
    if (__any(need)) {
      const float m_new = need ? mt : m_ref;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      lsum *= alpha;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
      m_ref = m_new;
    }
    const float mu = (m_ref == -INFINITY) ? 0.0f : m_ref;

    float ls = 0.0f;
    if (masked) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = (s[jb][r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(s[jb][r], c2, -mu));
          s[jb][r] = p;
          ls += p;
        }
    } else {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[jb][r], c2, -mu));
          s[jb][r] = p;
          ls += p;
        }
    }
    lsum += ls;

    // O^T += V^T P^T over four 16-key steps.  For step t4 this lane's P values
    // are registers 8(t4%2) .. +7 of s[t4/2]: keys 16t4 + 4half + {0..3} and
    // 16t4 + 8 + 4half + {0..3}; V^T supplies the same keys for feature rows.
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int jb = t4 >> 1, base = (t4 & 1) * 8;
      u32x4_t pb;
      pb[0] = Op::pack(s[jb][base + 0], s[jb][base + 1]);
      pb[1] = Op::pack(s[jb][base + 2], s[jb][base + 3]);
      pb[2] = Op::pack(s[jb][base + 4], s[jb][base + 5]);
      pb[3] = Op::pack(s[jb][base + 6], s[jb][base + 7]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const uint16_t* vrow = &vt[buf][(cb * 32 + col) * kVS + t4 * 16 + half * 4];
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 8);
        const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
        o[cb] = Op::mma(av, pb, o[cb]);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float ltot = lanes_sum(lsum);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (qvalid) {
    uint16_t* orow = static_cast<uint16_t*>(a.out) + b * a.o_sb + h * a.o_sh + (int64_t)qi * a.o_sn;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = cb * 32 + g * 8 + half * 4;
        u32x2_t w;
        w[0] = Op::pack(o[cb][4 * g + 0] * inv, o[cb][4 * g + 1] * inv);
        w[1] = Op::pack(o[cb][4 * g + 2] * inv, o[cb][4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + c) = w;
      }
  }
}

template <class Op, int NW>
hipError_t launch(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const int nqb = (a.Nq + NW * 32 - 1) / (NW * 32);
  const int64_t blocks = (int64_t)nqb * a.H * a.B;
  if (blocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL((attn_mfma_kernel<Op, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, t0, t1,
                        0, a, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  // Short query blocks (sentence-length sequences) use 2 waves per workgroup
  // so the grid has many workgroups; long ones use 4 waves to share each
  // staged K/V tile among 128 queries.
  const bool longq = a.Nq > 64;
  if (dt == DType::BF16) return longq ? launch<BF16, 4>(a, stream, t0, t1) : launch<BF16, 2>(a, stream, t0, t1);
  return longq ? launch<F16, 4>(a, stream, t0, t1) : launch<F16, 2>(a, stream, t0, t1);
}

}  // namespace mha
