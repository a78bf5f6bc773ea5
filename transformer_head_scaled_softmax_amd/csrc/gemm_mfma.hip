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
// the concatenation of their tile grids.  A workgroup of four waves (2 x 2)
// computes a TM (rows of X) x TN (rows of W) tile, 128 x 128 when the problem
// has enough tiles to fill the chip; each wave holds a (TM/2) x (TN/2)
// sub-tile as 32x32 MFMA blocks of C^T = W X^T, so a lane ends up with four
// consecutive output features of one row (one 8-byte store), and each operand
// read from LDS feeds two MFMAs.
//
// Latency hiding: K advances 64 at a time through two LDS buffers, and global
// loads run two steps ahead in two register sets, so each load has two steps of
// MFMA work to arrive.  Loads are buffer loads whose range check returns zeros
// past the tile's last valid row, so they need no branches.  Tiles are ordered
// so that the workgroups of one XCD (block id mod 8) take consecutive tiles,
// which share rows of X in that XCD's L2.
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

constexpr int kBK = 64;    // contraction step
constexpr int kLS = 72;    // LDS row stride (elements): 144 B -> conflict-free 16 B reads
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)
constexpr int kDeadOffset = (int)0x80000000u;     // beyond any range check: loads return zeros

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
  int start[kMaxGemmProblems + 1];  // first tile of each problem
  int tiles_n[kMaxGemmProblems];    // tiles along N of each problem
  int total;
};

// Buffer resource over `bytes` bytes from `base` (clamped to the 32-bit range
// check); loads at or beyond `bytes` return zeros.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, (int)kBufferWord3);
}

template <class Op, int TM, int TN>
__global__ __launch_bounds__(kThreads, 2) void gemm_mfma_kernel(GemmBatch g, TileMap tm) {
  constexpr int WM = TM / 2, WN = TN / 2;  // wave tile: rows of X x rows of W
  constexpr int MB = WM / 32, NB = WN / 32;  // 32x32 MFMA blocks per wave
  constexpr int XC = TM * 8 / kThreads;      // 16-byte X chunks per thread per step
  constexpr int WC = TN * 8 / kThreads;      // 16-byte W chunks per thread per step
  static_assert(MB >= 1 && NB >= 1 && XC >= 1 && WC >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][TM * kLS];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][TN * kLS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;

  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a
  // contiguous range of tiles (tiles of one row band are adjacent).
  const int T = tm.total, q = T / kXcds, rem = T % kXcds;
  const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int tile = x * q + min(x, rem) + j;

  // Select this tile's problem with unrolled compares (a runtime index into the
  // kernel-argument array would be lowered through scratch memory).
  GemmProblem P = g.p[0];
  int start = 0, tiles_n = tm.tiles_n[0];
#pragma unroll
  for (int i = 1; i < kMaxGemmProblems; ++i)
    if (i < g.count && tile >= tm.start[i]) {
      P = g.p[i];
      start = tm.start[i];
      tiles_n = tm.tiles_n[i];
    }
  const int local = tile - start;
  const int m0 = (local / tiles_n) * TM;
  const int n0 = (local % tiles_n) * TN;
  const int M = P.M, N = P.N, K = P.K;

  // The tile's rows of X and W as range-checked buffers: rows past M (or N)
  // read as zeros.
  const uint16_t* X = static_cast<const uint16_t*>(P.x) + (int64_t)m0 * P.ldx;
  const uint16_t* W = static_cast<const uint16_t*>(P.w) + (int64_t)n0 * K;
  const int xrows = min(TM, M - m0), wrows = min(TN, N - n0);
  const __amdgpu_buffer_rsrc_t xr_src = make_rsrc(X, ((int64_t)(xrows - 1) * P.ldx + K) * 2);
  const __amdgpu_buffer_rsrc_t wr_src = make_rsrc(W, ((int64_t)(wrows - 1) * K + K) * 2);

  int xoff[XC], woff[WC];
#pragma unroll
  for (int c = 0; c < XC; ++c) {
    const int idx = tid + c * kThreads;
    xoff[c] = ((idx >> 3) * (int)P.ldx + (idx & 7) * 8) * 2;
  }
#pragma unroll
  for (int c = 0; c < WC; ++c) {
    const int idx = tid + c * kThreads;
    woff[c] = ((idx >> 3) * K + (idx & 7) * 8) * 2;
  }

  // Steps at or past K load from an offset that fails the range check (zeros,
  // no memory access), so the loads are unconditional and never branch.
  auto load = [&](int k0, u32x4_t (&xr)[XC], u32x4_t (&wr)[WC]) {
    const bool live = k0 < K;
#pragma unroll
    for (int c = 0; c < XC; ++c)
      xr[c] = __builtin_amdgcn_raw_buffer_load_b128(xr_src, live ? xoff[c] + k0 * 2 : kDeadOffset, 0, 0);
#pragma unroll
    for (int c = 0; c < WC; ++c)
      wr[c] = __builtin_amdgcn_raw_buffer_load_b128(wr_src, live ? woff[c] + k0 * 2 : kDeadOffset, 0, 0);
  };
  // Chunks past K (only in the last step when K is not a multiple of 64) would
  // read the next row, so they are stored as zeros.
  auto store = [&](int buf, int k0, const u32x4_t (&xr)[XC], const u32x4_t (&wr)[WC]) {
    const bool tail = k0 + kBK > K;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < XC; ++c) {
      const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
      const bool ok = !tail || k0 + ch * 8 < K;
      *reinterpret_cast<u32x4_t*>(&xs[buf][row * kLS + ch * 8]) = ok ? xr[c] : zero;
    }
#pragma unroll
    for (int c = 0; c < WC; ++c) {
      const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
      const bool ok = !tail || k0 + ch * 8 < K;
      *reinterpret_cast<u32x4_t*>(&ws[buf][row * kLS + ch * 8]) = ok ? wr[c] : zero;
    }
  };

  // Wave (wm, wn): rows [wm*WM, +WM) of the X tile, features [wn*WN, +WN).
  const int wm = wave & 1, wn = wave >> 1;
  f32x16_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  // Each k16 step reads MB X operands and NB W operands and issues MB*NB MFMAs.
  auto compute = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      u32x4_t bx[MB], aw[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        bx[mb] = *reinterpret_cast<const u32x4_t*>(&xs[buf][(wm * WM + mb * 32 + col) * kLS + kk * 16 + half * 8]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        aw[nb] = *reinterpret_cast<const u32x4_t*>(&ws[buf][(wn * WN + nb * 32 + col) * kLS + kk * 16 + half * 8]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = Op::mma(aw[nb], bx[mb], acc[mb][nb]);
    }
  };

  const int nk = (K + kBK - 1) / kBK;
  u32x4_t xa[XC], wa[WC], xb[XC], wb[WC];  // two register sets: steps of even / odd index
  load(0, xa, wa);
  load(kBK, xb, wb);
  store(0, 0, xa, wa);
  __syncthreads();
  // Step kt computes LDS buffer kt%2, refills the register set it emptied with
  // step kt+2, and stores step kt+1 (loaded one step earlier) into the other
  // buffer.  Unrolled by two so each register set keeps a fixed name.
  for (int kt = 0; kt < nk; kt += 2) {
    load((kt + 2) * kBK, xa, wa);
    compute(0);
    if (kt + 1 < nk) store(1, (kt + 1) * kBK, xb, wb);
    __syncthreads();
    if (kt + 1 >= nk) break;
    load((kt + 3) * kBK, xb, wb);
    compute(1);
    if (kt + 2 < nk) store(0, (kt + 2) * kBK, xa, wa);
    __syncthreads();
  }

  // Epilogue through LDS, so global stores are whole 128-byte row segments:
  // acc[mb][nb] register r holds C[m0 + wm*WM + 32mb + col][n0 + wn*WN + 32nb +
  // 8(r/4) + 4half + r%4]; each wave writes its WM x WN sub-tile (bias added,
  // rounded) row-major into its own slice of the X staging buffer, then copies
  // it out 16 bytes per lane.  The main loop ended with a barrier, so the
  // staging buffer is free.
  constexpr int SS = WN + 8;  // staging row stride (elements)
  static_assert(4 * WM * SS <= 2 * TM * kLS, "staging does not fit");
  uint16_t* stage = &xs[0][0] + wave * WM * SS;
  const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int cl = nb * 32 + gq * 8 + half * 4;  // column within the wave tile
      const int n = n0 + wn * WN + cl;
      float b0 = 0.0f, b1 = 0.0f, b2 = 0.0f, b3 = 0.0f;
      if (bias && n < N) {  // N is a multiple of 4, so the 4-run is whole
        b0 = Op::to_float(bias[n + 0]);
        b1 = Op::to_float(bias[n + 1]);
        b2 = Op::to_float(bias[n + 2]);
        b3 = Op::to_float(bias[n + 3]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        u32x2_t w;
        w[0] = Op::pack(acc[mb][nb][4 * gq + 0] + b0, acc[mb][nb][4 * gq + 1] + b1);
        w[1] = Op::pack(acc[mb][nb][4 * gq + 2] + b2, acc[mb][nb][4 * gq + 3] + b3);
        *reinterpret_cast<u32x2_t*>(&stage[(mb * 32 + col) * SS + cl]) = w;
      }
    }
  __syncthreads();
  constexpr int CPR = WN / 8;  // 16-byte chunks per staged row
#pragma unroll
  for (int i = 0; i < WM * CPR / 64; ++i) {
    const int id = lane + 64 * i, row = id / CPR, ch = id % CPR;
    const int m = m0 + wm * WM + row, n = n0 + wn * WN + ch * 8;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&stage[row * SS + ch * 8]);
    if (m < M && n < N)  // N is a multiple of 8, so the 8-run is whole
      *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(P.c) + (int64_t)m * P.ldc + n) = v;
  }
}

template <class Op, int TM, int TN>
hipError_t launch(const GemmBatch& g, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  TileMap tm{};
  int total = 0;
  for (int i = 0; i < g.count; ++i) {
    const int tmn = (g.p[i].M + TM - 1) / TM;
    const int tnn = (g.p[i].N + TN - 1) / TN;
    tm.start[i] = total;
    tm.tiles_n[i] = tnn > 0 ? tnn : 1;
    total += tmn * tnn;
  }
  for (int i = g.count; i <= kMaxGemmProblems; ++i) tm.start[i] = total;
  tm.total = total;
  if (total == 0) return hipSuccess;
  hipExtLaunchKernelGGL((gemm_mfma_kernel<Op, TM, TN>), dim3(total), dim3(kThreads), 0, stream, t0, t1, 0, g, tm);
  return hipGetLastError();
}

int64_t count_tiles(const GemmBatch& g, int tm, int tn) {
  int64_t n = 0;
  for (int i = 0; i < g.count; ++i) n += (int64_t)((g.p[i].M + tm - 1) / tm) * ((g.p[i].N + tn - 1) / tn);
  return n;
}

template <class Op>
hipError_t launch_sized(const GemmBatch& g, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  // The largest tile that still gives every CU a workgroup.
  if (count_tiles(g, 128, 128) >= 256) return launch<Op, 128, 128>(g, stream, t0, t1);
  if (count_tiles(g, 128, 64) >= 256) return launch<Op, 128, 64>(g, stream, t0, t1);
  return launch<Op, 64, 64>(g, stream, t0, t1);
}

}  // namespace

hipError_t launch_gemm_mfma(const GemmBatch& g, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  return dt == DType::BF16 ? launch_sized<BF16>(g, stream, t0, t1) : launch_sized<F16>(g, stream, t0, t1);
}

}  // namespace mha
