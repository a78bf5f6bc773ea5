// gemm_mfma.hip -- bf16 / fp16 projection GEMMs on the gfx950 matrix cores.
//
// Computes C[m, n] = sum_k X[m, k] * W[n, k] (+ bias[n]) for the Q/K/V input
// projections and the output projection W^O ("Query / Key / Value Roles" and
// "The Output Projection W^O", trishampatil.com); W is in the
// [out_features, in_features] layout of nn.Linear ("A faithful layer in code",
// aicassindra.com), so both operands are contiguous along the contraction.
// Accumulation is fp32; C is rounded to nearest-even into the input type.
//
// Up to three independent problems (Q, K and V) share one launch: the grid is
// the concatenation of their tile grids.  A workgroup of four waves computes a
// 64 (rows of X) x 128 (rows of W) tile; each wave a 32 x 64 sub-tile as two
// 32x32 MFMA blocks of C^T = W X^T, so that a lane ends up with four
// consecutive output features of one row and stores them as one 8-byte write.
// K advances 64 at a time through double-buffered LDS tiles.
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

constexpr int kTM = 64;    // rows of X per tile
constexpr int kTN = 128;   // rows of W (output features) per tile
constexpr int kBK = 64;    // contraction step
constexpr int kLS = 72;    // LDS row stride (elements): 144 B -> conflict-free 16 B reads
constexpr int kThreads = 256;

struct BF16 {
  __device__ static f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float x, float y) {
    bf16x2_t r = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static float to_float(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
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
  __device__ static float to_float(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
};

struct TileMap {
  int start[kMaxGemmProblems + 1];  // first workgroup of each problem
  int tiles_n[kMaxGemmProblems];    // tiles along N of each problem
};

template <class Op>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmBatch g, TileMap tm) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kTM * kLS];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kTN * kLS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int bid = blockIdx.x;
  // Select this workgroup's problem with unrolled compares (a runtime index
  // into the kernel-argument array would be lowered through scratch memory).
  GemmProblem P = g.p[0];
  int start = 0, tiles_n = tm.tiles_n[0];
#pragma unroll
  for (int i = 1; i < kMaxGemmProblems; ++i)
    if (i < g.count && bid >= tm.start[i]) {
      P = g.p[i];
      start = tm.start[i];
      tiles_n = tm.tiles_n[i];
    }
  const int local = bid - start;
  const int m0 = (local / tiles_n) * kTM;
  const int n0 = (local % tiles_n) * kTN;

  const uint16_t* X = static_cast<const uint16_t*>(P.x);
  const uint16_t* W = static_cast<const uint16_t*>(P.w);
  const int M = P.M, N = P.N, K = P.K;

  // Staging: X tile 64 x 64 -> 512 chunks of 8 elements (2 per thread);
  // W tile 128 x 64 -> 1024 chunks (4 per thread).
  u32x4_t xr[2], wr[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
      const int m = m0 + row, k = k0 + ch * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (m < M && k < K) v = *reinterpret_cast<const u32x4_t*>(X + (int64_t)m * P.ldx + k);
      xr[c] = v;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
      const int n = n0 + row, k = k0 + ch * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (n < N && k < K) v = *reinterpret_cast<const u32x4_t*>(W + (int64_t)n * K + k);
      wr[c] = v;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4_t*>(&xs[buf][row * kLS + ch * 8]) = xr[c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4_t*>(&ws[buf][row * kLS + ch * 8]) = wr[c];
    }
  };

  // Wave (wm, wn): rows [32wm, 32wm+32) of the X tile, features [64wn, 64wn+64).
  const int wm = wave & 1, wn = wave >> 1;
  f32x16_t acc[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nb][r] = 0.0f;

  const int nk = (K + kBK - 1) / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const u32x4_t bx = *reinterpret_cast<const u32x4_t*>(&xs[buf][(wm * 32 + col) * kLS + kk * 16 + half * 8]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const u32x4_t aw = *reinterpret_cast<const u32x4_t*>(
            &ws[buf][(wn * 64 + nb * 32 + col) * kLS + kk * 16 + half * 8]);
        acc[nb] = Op::mma(aw, bx, acc[nb]);
      }
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // acc[nb] register r holds C[m0 + 32wm + col][n0 + 64wn + 32nb + 8(r/4) + 4half + r%4].
  const int m = m0 + wm * 32 + col;
  if (m >= M) return;
  uint16_t* C = static_cast<uint16_t*>(P.c) + (int64_t)m * P.ldc;
  const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int n = n0 + wn * 64 + nb * 32 + gq * 8 + half * 4;
      if (n >= N) continue;  // N is a multiple of 4, so the 4-run is whole
      float v0 = acc[nb][4 * gq + 0], v1 = acc[nb][4 * gq + 1];
      float v2 = acc[nb][4 * gq + 2], v3 = acc[nb][4 * gq + 3];
      if (bias) {
        v0 += Op::to_float(bias[n + 0]);
        v1 += Op::to_float(bias[n + 1]);
        v2 += Op::to_float(bias[n + 2]);
        v3 += Op::to_float(bias[n + 3]);
      }
      u32x2_t w;
      w[0] = Op::pack(v0, v1);
      w[1] = Op::pack(v2, v3);
      *reinterpret_cast<u32x2_t*>(C + n) = w;
    }
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmBatch& g, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  TileMap tm{};
  int total = 0;
  for (int i = 0; i < g.count; ++i) {
    const int tmn = (g.p[i].M + kTM - 1) / kTM;
    const int tnn = (g.p[i].N + kTN - 1) / kTN;
    tm.start[i] = total;
    tm.tiles_n[i] = tnn > 0 ? tnn : 1;
    total += tmn * tnn;
  }
  for (int i = g.count; i <= kMaxGemmProblems; ++i) tm.start[i] = total;
  if (total == 0) return hipSuccess;
  if (dt == DType::BF16)
    hipExtLaunchKernelGGL(gemm_mfma_kernel<BF16>, dim3(total), dim3(kThreads), 0, stream, t0, t1, 0, g, tm);
  else
    hipExtLaunchKernelGGL(gemm_mfma_kernel<F16>, dim3(total), dim3(kThreads), 0, stream, t0, t1, 0, g, tm);
  return hipGetLastError();
}

}  // namespace mha
