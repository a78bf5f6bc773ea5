// bwd_f32.hip -- gradients of fp32 scaled dot-product attention on the vector
// ALUs, any head size up to 128.
//
// The same derivatives as the matrix-core backward pass (the exact gradients
// of softmax(scale * Q K^T) V with masked keys at weight 0; the pages use the
// path for teacher-forced training: "Training (Teacher Forcing + Masking)",
// trishampatil.com): with P recomputed from the forward's row statistic lse,
//   dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dO_i . v_j - D_i),  D_i = dO_i . out_i,
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
//
// Two kernels, one wave per row.  The dQ kernel gives each wave one query
// row (four rows per workgroup share 64-key tiles of K and V in LDS): one key
// per lane for P and dS, then one output feature per lane for dQ; it also
// writes D_i.  The dK/dV kernel gives each wave one key row (four per
// workgroup share 64-query tiles of Q, dO, lse and D): one query per lane for P
// and dS, one feature per lane for dK and dV, summed over the query heads that
// share the key/value head.
#include <hip/hip_ext.h>

#include "mha_internal.h"

namespace mha {
namespace {

constexpr int kRows = 4;   // rows per workgroup (one per wave)
constexpr int kTile = 64;  // streamed rows per tile
constexpr int kDm = kF32MaxHeadDim;
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ inline float lse_offset(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(BwdArgs a, int dk, int dv, int nqb) {
  __shared__ float ks[kTile][kDm + 1];  // +1 column: lane t reads row t conflict-free
  __shared__ float vs[kTile][kDm + 1];
  __shared__ float qs[kRows][kDm];
  __shared__ float os[kRows][kDm];
  __shared__ float dss[kRows][kTile];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qb = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb;
  const int b = bh / a.H;

  int L = a.Nk;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), a.Nk);
  const int i = qb * kRows + wave;
  const bool valid = i < a.Nq;
  const int kend = valid ? (a.causal ? min(L, i + 1) : L) : 0;
  const int ilast = min(qb * kRows + kRows, a.Nq) - 1;
  const int kend_blk = a.causal ? min(L, ilast + 1) : L;

  const float* qp = static_cast<const float*>(a.q) + ((int64_t)bh * a.Nq + i) * dk;
  const float* op = static_cast<const float*>(a.out) + ((int64_t)bh * a.Nq + i) * dv;
  const float* gp = static_cast<const float*>(a.dout) + ((int64_t)bh * a.Nq + i) * dv;
  const int64_t kvhead = (int64_t)b * a.Hkv + (bh % a.H) / (a.H / a.Hkv);  // key/value head read
  const float* kp = static_cast<const float*>(a.k) + kvhead * a.Nk * dk;
  const float* vp = static_cast<const float*>(a.v) + kvhead * a.Nk * dv;
  // D_i = dO_i . out_i; the wave's query row and dO row go to LDS.
  float dpart = 0.0f;
  for (int c = lane; c < kDm; c += 64) {
    const float q = valid && c < dk ? qp[c] : 0.0f;
    const float g = valid && c < dv ? gp[c] : 0.0f;
    const float o = valid && c < dv ? op[c] : 0.0f;
    qs[wave][c] = q;
    os[wave][c] = g;
    dpart = fmaf(g, o, dpart);
  }
  const float D = wave_sum(dpart);
  const float lse2 = valid ? lse_offset(a.lse[(int64_t)bh * a.Nq + i]) : INFINITY;
  if (valid && lane == 0) a.dsum[(int64_t)bh * a.Nq + i] = D;
  const float c2 = a.scale * kLog2e;

  float acc0 = 0.0f, acc1 = 0.0f;  // dQ features lane, lane + 64
  for (int j0 = 0; j0 < kend_blk; j0 += kTile) {
    __syncthreads();  // previous tile consumed (and qs, os visible)
    for (int idx = threadIdx.x; idx < kTile * dk; idx += 256) {
      const int r = idx / dk, c = idx - r * dk, j = j0 + r;
      ks[r][c] = j < kend_blk ? kp[(int64_t)j * dk + c] : 0.0f;
    }
    for (int idx = threadIdx.x; idx < kTile * dv; idx += 256) {
      const int r = idx / dv, c = idx - r * dv, j = j0 + r;
      vs[r][c] = j < kend_blk ? vp[(int64_t)j * dv + c] : 0.0f;
    }
    __syncthreads();

    const int j = j0 + lane;
    float ds = 0.0f;
    if (j < kend) {
      float s = 0.0f, dp = 0.0f;
      for (int c = 0; c < dk; ++c) s = fmaf(qs[wave][c], ks[lane][c], s);
      for (int c = 0; c < dv; ++c) dp = fmaf(os[wave][c], vs[lane][c], dp);
      const float p = exp2f(fmaf(s, c2, -lse2));
      ds = p * (dp - D);
    }
    dss[wave][lane] = ds;
    __syncthreads();

    const int nk = min(kTile, kend_blk - j0);
    for (int u = 0; u < nk; ++u) {
      const float d = dss[wave][u];
      if (lane < dk) acc0 = fmaf(d, ks[u][lane], acc0);
      if (lane + 64 < dk) acc1 = fmaf(d, ks[u][lane + 64], acc1);
    }
  }

  if (valid) {
    float* dqp = static_cast<float*>(a.dq) + ((int64_t)bh * a.Nq + i) * dk;
    if (lane < dk) dqp[lane] = acc0 * a.scale;
    if (lane + 64 < dk) dqp[lane + 64] = acc1 * a.scale;
  }
}

__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(BwdArgs a, int dk, int dv, int nkb) {
  __shared__ float qs[kTile][kDm + 1];
  __shared__ float gs[kTile][kDm + 1];
  __shared__ float ls[kTile], ds_[kTile];  // per query of the tile: exp2 offset, D
  __shared__ float kr[kRows][kDm];
  __shared__ float vr[kRows][kDm];
  __shared__ float ps[kRows][kTile], dss[kRows][kTile];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kb = blockIdx.x % nkb;
  const int bkv = blockIdx.x / nkb;  // (b, key/value head); its G query heads are streamed in turn
  const int b = bkv / a.Hkv, G = a.H / a.Hkv;

  int L = a.Nk;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), a.Nk);
  const int j = kb * kRows + wave;
  const bool live = j < L;  // padded keys (and rows past Nk) get zero gradients
  // Queries that see a key of this workgroup: all, or under the causal mask
  // those from its first key on; none when all its keys are padding.
  const int kfirst = kb * kRows;
  const int qstart = kfirst < L ? (a.causal ? kfirst : 0) : a.Nq;

  const float* kp = static_cast<const float*>(a.k) + ((int64_t)bkv * a.Nk + j) * dk;
  const float* vp = static_cast<const float*>(a.v) + ((int64_t)bkv * a.Nk + j) * dv;
  for (int c = lane; c < kDm; c += 64) {
    kr[wave][c] = live && c < dk ? kp[c] : 0.0f;
    vr[wave][c] = live && c < dv ? vp[c] : 0.0f;
  }
  const float c2 = a.scale * kLog2e;

  float dv0 = 0.0f, dv1 = 0.0f, dk0 = 0.0f, dk1 = 0.0f;  // features lane, lane + 64
  for (int g = 0; g < G; ++g) {
    const int64_t bh = (int64_t)b * a.H + (bkv % a.Hkv) * G + g;  // query head of this pass
    const float* qp = static_cast<const float*>(a.q) + bh * a.Nq * dk;
    const float* gp = static_cast<const float*>(a.dout) + bh * a.Nq * dv;
    for (int i0 = qstart; i0 < a.Nq; i0 += kTile) {
      __syncthreads();  // previous tile consumed (and kr, vr visible)
      const int nq = min(kTile, a.Nq - i0);
      for (int idx = threadIdx.x; idx < kTile * dk; idx += 256) {
        const int r = idx / dk, c = idx - r * dk;
        qs[r][c] = r < nq ? qp[(int64_t)(i0 + r) * dk + c] : 0.0f;
      }
      for (int idx = threadIdx.x; idx < kTile * dv; idx += 256) {
        const int r = idx / dv, c = idx - r * dv;
        gs[r][c] = r < nq ? gp[(int64_t)(i0 + r) * dv + c] : 0.0f;
      }
      if (threadIdx.x < kTile) {
        const int r = threadIdx.x;
        ls[r] = r < nq ? lse_offset(a.lse[(int64_t)bh * a.Nq + i0 + r]) : INFINITY;
        ds_[r] = r < nq ? a.dsum[(int64_t)bh * a.Nq + i0 + r] : 0.0f;
      }
      __syncthreads();

      const int i = i0 + lane;
      float p = 0.0f, ds = 0.0f;
      if (live && lane < nq && (!a.causal || j <= i)) {
        float s = 0.0f, dp = 0.0f;
        for (int c = 0; c < dk; ++c) s = fmaf(qs[lane][c], kr[wave][c], s);
        for (int c = 0; c < dv; ++c) dp = fmaf(gs[lane][c], vr[wave][c], dp);
        p = exp2f(fmaf(s, c2, -ls[lane]));
        ds = p * (dp - ds_[lane]);
      }
      ps[wave][lane] = p;
      dss[wave][lane] = ds;
      __syncthreads();

      for (int u = 0; u < nq; ++u) {
        const float pu = ps[wave][u], du = dss[wave][u];
        if (lane < dv) dv0 = fmaf(pu, gs[u][lane], dv0);
        if (lane + 64 < dv) dv1 = fmaf(pu, gs[u][lane + 64], dv1);
        if (lane < dk) dk0 = fmaf(du, qs[u][lane], dk0);
        if (lane + 64 < dk) dk1 = fmaf(du, qs[u][lane + 64], dk1);
      }
    }
  }

  if (j < a.Nk) {
    float* dkp = static_cast<float*>(a.dk) + ((int64_t)bkv * a.Nk + j) * dk;
    float* dvp = static_cast<float*>(a.dv) + ((int64_t)bkv * a.Nk + j) * dv;
    if (lane < dk) dkp[lane] = dk0 * a.scale;
    if (lane + 64 < dk) dkp[lane + 64] = dk1 * a.scale;
    if (lane < dv) dvp[lane] = dv0;
    if (lane + 64 < dv) dvp[lane + 64] = dv1;
  }
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, int dk, int dv, hipStream_t stream, hipEvent_t const* ev) {
  auto evt = [&](int i) -> hipEvent_t { return ev ? ev[i] : nullptr; };
  const int nqb = (a.Nq + kRows - 1) / kRows, nkb = (a.Nk + kRows - 1) / kRows;
  const int64_t bh = (int64_t)a.B * a.H, bkv = (int64_t)a.B * a.Hkv;
  // The dQ kernel writes D, which the dK/dV kernel reads: stream order.
  if (nqb * bh > 0) {
    hipExtLaunchKernelGGL(bwd_dq_f32_kernel, dim3((unsigned)(nqb * bh)), dim3(256), 0, stream, evt(0), evt(1), 0, a,
                          dk, dv, nqb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nkb * bkv > 0) {
    hipExtLaunchKernelGGL(bwd_dkdv_f32_kernel, dim3((unsigned)(nkb * bkv)), dim3(256), 0, stream, evt(2), evt(3), 0,
                          a, dk, dv, nkb);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace mha
