// attn_f32.hip -- fp32 scaled dot-product attention on the vector ALUs.
//
// For fp32 inputs with any head size up to 128.  One wave per query row; the
// four waves of a workgroup take four consecutive rows of one (b, h) and share
// each 64-key tile of K and V staged in LDS.  The score row of a tile is one
// key per lane; the softmax is carried across tiles as a running maximum and
// running sum (an exact rearrangement of the row softmax of "Scaled Dot-Product
// Attention: Step by Step", trishampatil.com); the weighted sum of V rows is
// one output feature per lane.  Masked keys (padding j >= L, future j > i
// under the causal mask -- "Why Masking Is Required", trishampatil.com; "Two
// masks, not one", alexdo.xyz) get weight exactly 0 and padded rows are never
// read.
#include <hip/hip_ext.h>

#include "mha_internal.h"

namespace mha {
namespace {

constexpr int kRows = 4;     // query rows per workgroup (one per wave)
constexpr int kTile = 64;    // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a, int nqb) {
  __shared__ float ks[kTile][kF32MaxHeadDim + 1];  // +1 column: lane t reads row t conflict-free
  __shared__ float vs[kTile][kF32MaxHeadDim];
  __shared__ float qs[kRows][kF32MaxHeadDim];
  __shared__ float ps[kRows][kTile];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qb = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;
  const int h = bh % a.H, b = bh / a.H;

  int L = a.Nk;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), a.Nk);
  const int i = qb * kRows + wave;
  const bool valid = i < a.Nq;
  const int coff = a.causal_end ? L - a.Nq : 0;  // causal: query i sees keys j <= i + coff
  const int kend = valid ? (a.causal ? min(L, i + 1 + coff) : L) : 0;
  const int ilast = min(qb * kRows + kRows, a.Nq) - 1;
  const int kend_blk = a.causal ? min(L, ilast + 1 + coff) : L;
  const int kvh = a.kv_group > 1 ? h / a.kv_group : h;  // key/value head read by head h

  const float* qp = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)i * a.q_sn;
  const float* kp = static_cast<const float*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const float* vp = static_cast<const float*>(a.v) + b * a.v_sb + kvh * a.v_sh;
  for (int c = lane; c < a.dk; c += 64) qs[wave][c] = valid ? qp[c] : 0.0f;

  // Scores are kept in log2 units: s * scale * log2(e), exponentiated with exp2.
  const float c2 = a.scale * kLog2e;
  float m = -INFINITY, l = 0.0f, acc0 = 0.0f, acc1 = 0.0f;

  for (int j0 = 0; j0 < kend_blk; j0 += kTile) {
    __syncthreads();  // previous tile fully consumed (and qs visible)
    // Only the tile's rows below the workgroup's key end are loaded (wave w
    // takes rows w, w + 4, ..., a lane per column): scores are formed only for
    // visible keys and the weighted sum runs over the loaded rows, so the
    // other rows are never read.
    const int nrows = min(kTile, kend_blk - j0);
    for (int r = wave; r < nrows; r += kRows)
      for (int c = lane; c < a.dk; c += 64) ks[r][c] = kp[(int64_t)(j0 + r) * a.k_sn + c];
    for (int r = wave; r < nrows; r += kRows)
      for (int c = lane; c < a.dv; c += 64) vs[r][c] = vp[(int64_t)(j0 + r) * a.v_sn + c];
    __syncthreads();

    const int j = j0 + lane;
    const bool vis = j < kend;
    float s = -INFINITY;
    if (vis) {
      // Four partial sums, so the products do not wait on one another.
      float d0 = 0.0f, d1 = 0.0f, d2 = 0.0f, d3 = 0.0f;
      int c = 0;
      for (; c + 4 <= a.dk; c += 4) {
        d0 = fmaf(qs[wave][c], ks[lane][c], d0);
        d1 = fmaf(qs[wave][c + 1], ks[lane][c + 1], d1);
        d2 = fmaf(qs[wave][c + 2], ks[lane][c + 2], d2);
        d3 = fmaf(qs[wave][c + 3], ks[lane][c + 3], d3);
      }
      for (; c < a.dk; ++c) d0 = fmaf(qs[wave][c], ks[lane][c], d0);
      s = ((d0 + d1) + (d2 + d3)) * c2;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m - m_new);
    const float p = (vis && m_new != -INFINITY) ? exp2f(s - m_new) : 0.0f;
    l = l * alpha + wave_sum(p);
    ps[wave][lane] = p;
    __syncthreads();

    float s0 = 0.0f, s1 = 0.0f;
    const int nk = min(kTile, kend_blk - j0);
    for (int u = 0; u < nk; ++u) {
      const float pu = ps[wave][u];
      if (lane < a.dv) s0 = fmaf(pu, vs[u][lane], s0);
      if (lane + 64 < a.dv) s1 = fmaf(pu, vs[u][lane + 64], s1);
    }
    acc0 = acc0 * alpha + s0;
    acc1 = acc1 * alpha + s1;
    m = m_new;
  }

  if (valid) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    // Row statistic for the backward pass: ln(sum_j exp(scale q.k_j)).
    if (a.lse && lane == 0)
      a.lse[((int64_t)b * a.H + h) * a.Nq + i] = l > 0.0f ? (m + log2f(l)) * 0.6931471805599453f : -INFINITY;
    float* op = static_cast<float*>(a.out) + b * a.o_sb + h * a.o_sh + (int64_t)i * a.o_sn;
    if (lane < a.dv) op[lane] = acc0 * inv;
    if (lane + 64 < a.dv) op[lane + 64] = acc1 * inv;
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const int nqb = (a.Nq + kRows - 1) / kRows;
  const int64_t blocks = (int64_t)nqb * a.H * a.B;
  if (blocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, t0, t1, 0, a, nqb);
  return hipGetLastError();
}

}  // namespace mha
