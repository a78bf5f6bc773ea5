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
// the concatenation of their tile grids.  A workgroup computes a TM (rows of X)
// x TN (rows of W) tile; its waves form a WGM x WGN grid and each holds a
// (TM/WGM) x (TN/WGN) sub-tile as 32x32 MFMA blocks of C^T = W X^T, so a lane
// ends up with four consecutive output features of one row.
//
// Operand staging: K advances 64 at a time through S stages of LDS that are
// filled by LDS-direct buffer loads (each lane's 16 bytes go straight from
// memory into LDS, with no register round trip), issued S-1 steps ahead
// (S = 2 in the configurations used: latency is hidden by a second
// workgroup or a second wave per SIMD rather than by deeper staging).  A
// step's wait is an explicit vmcnt that lets the later stages stay in flight,
// followed by one barrier.  A 64-element row of a stage is 128 bytes of eight
// 16-byte chunks; chunk c of row r sits in slot c ^ (r & 7) ^ ((r >> 3) & 1),
// which keeps the MFMA operand reads (16 bytes per lane, 32 consecutive rows)
// free of bank conflicts; the loads place chunks by choosing, for each lane's
// fixed LDS slot, the global chunk that belongs there.
//
// The buffer range check returns zeros past a tile's last valid row, so edge
// tiles need no branches (rows past M or N only feed outputs that are never
// stored).  Tiles are ordered so that the workgroups of one XCD (block id mod
// 8) take consecutive tiles, which share rows of X in that XCD's L2.  The tile
// shape is chosen per launch from the problem sizes (see launch_sized).
#include <type_traits>

#include "mfma_util.h"

namespace mha {
namespace {

constexpr int kBK = 64;  // contraction step (one 128-byte row per operand row)
constexpr int kXcds = 8;

struct TileMap {
  int start[kMaxGemmProblems + 1];  // first tile of each problem
  int tiles_n[kMaxGemmProblems];    // tiles along N of each problem
  int total;
};

// Residual connection and layer normalisation after the output projection
// ("Residual Connections and Layer Normalization", trishampatil.com:
// LayerNorm(x + Sublayer(x)), normalised across each token's features; "Add &
// Norm", alexdo.xyz): z = C + bias + residual, then (z - mean) / sqrt(var +
// eps) * gamma + beta with the biased variance.
//
// A tile holds only TN of a row's N features, so the statistics are made in
// two steps.  In the projection's epilogue each tile reduces its part of every
// row -- the sum and the sum of squares about the tile's own mean, fp32, from
// the values in registers -- and stores them, with the row values as
// differences from the tile mean in fp16, scaled by a power of two derived
// from that sum of squares (in place in the output rows: 2 bytes with 11
// significant bits, so this intermediate rounding is 2^-12 relative to the
// row's spread rather than bf16's 2^-9 of its size, and the scale keeps any
// spread inside fp16's range).  A
// second kernel then merges each row's parts (the pairwise update of Chan,
// Golub and LeVeque for means and centred sums of squares) and normalises the
// row in place.  The kernel boundary is what makes every tile's stores visible
// to the second pass: within one launch that would take an agent-scope
// release (an L2 write-back) in every workgroup and an acquire (an L2
// invalidate) in every merging one, which measured several times slower.
//
// The exponent k of the power of two a tile's stored differences are divided
// by, read from the bits of their fp32 sum of squares s2 (so the epilogue and
// the normalisation pass derive the same k from the same stored value).  With
// e = floor(log2 s2), every difference is below sqrt(s2) < 2^(k + 14), so the
// scaled values stay within +-2^14 (fp16's largest finite value is 65504),
// while a typical one, sqrt(s2 / 64), stays near 2^11 -- far above fp16's
// subnormals whatever the row's magnitude.  Clamped so that 2^k is a normal
// fp32 value; the limit left is the fp32 sum of squares itself (differences
// above ~1e18 overflow it).
__device__ inline int ln_tile_exponent(float s2) {
  const int e = (int)((__float_as_uint(s2) >> 23) & 0xffu) - 127;
  return min(100, max(-100, ((e + 1) >> 1) - 13));
}
__device__ inline float ln_pow2(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// ln_tile_stats: register 4gq + e of acc[mb][nb] holds row wm*WM + 32mb + col
// of the tile and column wn*WN + 32nb + 8gq + 4half + e; a row's partial sums
// are combined over the lane halves, then over the WGN waves sharing the row
// through `red` (2 x [WGN][TM] floats of LDS).  Columns past N are left out;
// rows past M are computed from zeros and never stored.
template <class Op, int TM, int WGN, int MB, int NB, int WM, int WN>
__device__ inline void ln_tile_stats(f32x16_t (&acc)[MB][NB], const GemmProblem& P, int m0, int n0, int tcol,
                                     int wm, int wn, int col, int half, float* red) {
  const int M = P.M, N = P.N;
  const int64_t ldc = P.ldc;
  const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
  const uint16_t* res = static_cast<const uint16_t*>(P.residual);
  auto unpack4 = [](u32x2_t v, float (&f)[4]) {
    f[0] = Op::to_float((uint16_t)(v[0] & 0xffffu));
    f[1] = Op::to_float((uint16_t)(v[0] >> 16));
    f[2] = Op::to_float((uint16_t)(v[1] & 0xffffu));
    f[3] = Op::to_float((uint16_t)(v[1] >> 16));
  };
  float s1[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + wm * WM + 32 * mb + col;
    s1[mb] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int n = n0 + wn * WN + 32 * nb + 8 * gq + 4 * half;
        if (n < N) {  // N is a multiple of 8: the 4-run is whole
          float add[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (bias) unpack4(*reinterpret_cast<const u32x2_t*>(bias + n), add);
          if (m < M) {
            float r4[4];
            unpack4(*reinterpret_cast<const u32x2_t*>(res + (int64_t)m * ldc + n), r4);
#pragma unroll
            for (int e = 0; e < 4; ++e) add[e] += r4[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[mb][nb][4 * gq + e] += add[e];
            s1[mb] += acc[mb][nb][4 * gq + e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mb][nb][4 * gq + e] = 0.0f;
        }
      }
    s1[mb] = lanes_sum(s1[mb]);
  }
  const int rbase = wm * WM + col;
  float* red1 = red;
  float* red2 = red + WGN * TM;
  if (half == 0)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red1[wn * TM + rbase + 32 * mb] = s1[mb];
  __syncthreads();
  const float inv_nt = 1.0f / (float)min(N - n0, WGN * WN);  // valid columns of this tile
  float sum[MB], s2[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < WGN; ++w) t += red1[w * TM + rbase + 32 * mb];
    sum[mb] = t;
    const float mean_t = t * inv_nt;
    s2[mb] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        if (n0 + wn * WN + 32 * nb + 8 * gq + 4 * half < N)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float dz = acc[mb][nb][4 * gq + e] - mean_t;
            acc[mb][nb][4 * gq + e] = dz;  // stored as the difference from the tile mean
            s2[mb] = fmaf(dz, dz, s2[mb]);
          }
    s2[mb] = lanes_sum(s2[mb]);
  }
  if (half == 0)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red2[wn * TM + rbase + 32 * mb] = s2[mb];
  __syncthreads();
  const int stride = ln_stats_stride(N);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + wm * WM + 32 * mb + col;
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < WGN; ++w) t += red2[w * TM + rbase + 32 * mb];
    if (wn == 0 && half == 0 && m < M) P.stats[(int64_t)m * stride + tcol] = float2{sum[mb], t};
    // The differences leave as fp16 scaled by 2^-k (ln_tile_exponent of the
    // stored sum of squares), which keeps them inside fp16's range.
    const float sc = ln_pow2(-ln_tile_exponent(t));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] *= sc;
  }
}

// The second pass: one wave per row; each lane takes 8-feature chunks lane,
// lane + 64, ... of the row.  `tn` is the projection's tile width.
template <class Op>
__global__ __launch_bounds__(256) void ln_rows_kernel(GemmProblem P, int tn) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int M = P.M, N = P.N;
  if (m >= M) return;
  const int stride = ln_stats_stride(N), tiles = (N + tn - 1) / tn;
  const float2* st = P.stats + m * stride;
  // Merge the tile statistics: lanes take tiles, then reduce over the wave.
  const float inv_n = 1.0f / (float)N;
  float sum = 0.0f;
  for (int j = lane; j < tiles; j += 64) sum += st[j].x;
  const float mean = wave_sum(sum) * inv_n;
  float m2 = 0.0f;
  for (int j = lane; j < tiles; j += 64) {
    const float nj = (float)min(tn, N - j * tn);
    const float d = st[j].x / nj - mean;
    m2 += st[j].y + nj * d * d;
  }
  const float rstd = 1.0f / sqrtf(wave_sum(m2) * inv_n + P.eps);
  const uint16_t* gam = static_cast<const uint16_t*>(P.gamma);
  const uint16_t* bet = static_cast<const uint16_t*>(P.beta);
  uint16_t* row = static_cast<uint16_t*>(P.c) + m * P.ldc;
  for (int f0 = lane * 8; f0 < N; f0 += 512) {  // N is a multiple of 8: chunks are whole
    const u32x4_t z = *reinterpret_cast<const u32x4_t*>(row + f0);  // scaled fp16 differences from the tile mean
    const int jt = f0 / tn;
    const float2 stj = st[jt];
    const float unscale = ln_pow2(ln_tile_exponent(stj.y));
    const float shift = stj.x / (float)min(tn, N - jt * tn) - mean;  // (stored + mean_t) - mean
    u32x4_t gv = {0u, 0u, 0u, 0u}, bv = {0u, 0u, 0u, 0u};
    if (gam) gv = *reinterpret_cast<const u32x4_t*>(gam + f0);
    if (bet) bv = *reinterpret_cast<const u32x4_t*>(bet + f0);
    u32x4_t y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint16_t zs = (uint16_t)(z[i] >> (16 * e)), gs = (uint16_t)(gv[i] >> (16 * e)),
                       bs = (uint16_t)(bv[i] >> (16 * e));
        const float gf = gam ? Op::to_float(gs) : 1.0f;
        const float bf = bet ? Op::to_float(bs) : 0.0f;
        v[e] = fmaf(fmaf(F16::to_float(zs), unscale, shift) * rstd, gf, bf);
      }
      y[i] = Op::pack(v[0], v[1]);
    }
    *reinterpret_cast<u32x4_t*>(row + f0) = y;
  }
}

// LN: the epilogue applies the residual connection and layer normalisation
// (launch_gemm_ln).
template <class Op, int TM, int TN, int WGM, int WGN, int S, int MINB, bool LN = false>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_mfma_kernel(GemmBatch g, TileMap tm) {
  constexpr int NW = WGM * WGN, NT = 64 * NW;
  constexpr int WM = TM / WGM, WN = TN / WGN;  // wave tile: rows of X x rows of W
  constexpr int MB = WM / 32, NB = WN / 32;    // 32x32 MFMA blocks per wave
  constexpr int ROWS = TM + TN;                // operand rows per stage (X, then W)
  constexpr int STAGE = ROWS * kBK;            // elements per stage
  constexpr int CHUNKS = ROWS / 8;             // 1 KiB loads per stage
  constexpr int LPW = (CHUNKS + NW - 1) / NW;  // per wave (the last round may be partial)
  static_assert(MB >= 1 && NB >= 1 && WM % 32 == 0 && WN % 32 == 0, "bad wave tile");
  // With a partial last round the waves issue different numbers of loads, which
  // only the two-stage schedule (it waits for all of them) tolerates.
  static_assert((CHUNKS % NW == 0 || S == 2) && NW % 2 == 0, "loads must split over an even wave count");
  static_assert(S >= 2 && (S - 1) * LPW < 64, "too many loads in flight");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[S * STAGE];

  const int tid = threadIdx.x;
  // The wave index as a scalar: it selects buffer resources and LDS addresses.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;

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
  const int ldx = (int)P.ldx;

  // The tile's rows of X and W as range-checked buffers.
  const uint16_t* X = static_cast<const uint16_t*>(P.x) + (int64_t)m0 * P.ldx;
  const uint16_t* W = static_cast<const uint16_t*>(P.w) + (int64_t)n0 * K;
  const int xrows = min(TM, M - m0), wrows = min(TN, N - n0);
  const __amdgpu_buffer_rsrc_t xr_src = make_rsrc(X, ((int64_t)(xrows - 1) * ldx + K) * 2);
  const __amdgpu_buffer_rsrc_t wr_src = make_rsrc(W, ((int64_t)(wrows - 1) * K + K) * 2);

  // Load i of this wave fills 1 KiB chunk c = wave + NW*i of a stage: rows
  // 8c .. 8c+7, lane l at row 8c + l/8, slot l%8.  The global chunk for that
  // slot is slot ^ (row & 7) ^ ((row >> 3) & 1) = (l%8) ^ (l/8) ^ (c & 1), and
  // c & 1 == wave & 1 because NW is even.
  const int gchunk = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
  const int lrow = lane >> 3;
  int goff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int row = 8 * (wave + NW * i) + lrow;
    goff[i] = row < TM ? (row * ldx + gchunk * 8) * 2 : ((row - TM) * K + gchunk * 8) * 2;
  }
  const int nk = (K + kBK - 1) / kBK;
  // Issue the loads of step kt into stage kt % S; steps at or past nk (and the
  // chunks of the last step that lie past K) read nothing, so every step
  // issues the same number of loads and the vmcnt waits stay exact.
  auto issue = [&](int kt) {
    uint16_t* dst = lds + (kt % S) * STAGE;
    const int k0 = kt * kBK;
    // Bit 31 set = past every range check.  Arithmetic rather than a select,
    // so that the compiler cannot split the load into two predicated copies
    // (which would make the number of loads per step data-dependent).
    const int dead = (int)((uint32_t)(kt >= nk || k0 + gchunk * 8 >= K) << 31);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int c = wave + NW * i;  // uniform per wave
      if (c >= CHUNKS) break;
      const int off = (goff[i] + k0 * 2) | dead;
      uint16_t* d = dst + c * 512;
      if (c < TM / 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr_src, MHA_LDS(d), 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr_src, MHA_LDS(d), 16, off, 0, 0, 0);
    }
  };

  // Wave (wm, wn): rows [wm*WM, +WM) of the X tile, features [wn*WN, +WN).
  const int wm = wave % WGM, wn = wave / WGM;
  f32x16_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  // Operand rows start at multiples of 32, so the swizzle of a lane's row
  // depends on the lane alone.
  const int swz = operand_swizzle(lane);
  auto compute = [&](int buf) {
    const uint16_t* st = lds + buf * STAGE;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int slot = (kk * 2 + half) ^ swz;
      u32x4_t bx[MB], aw[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        bx[mb] = *reinterpret_cast<const u32x4_t*>(&st[(wm * WM + mb * 32 + col) * kBK + slot * 8]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        aw[nb] = *reinterpret_cast<const u32x4_t*>(&st[(TM + wn * WN + nb * 32 + col) * kBK + slot * 8]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = Op::mma(aw[nb], bx[mb], acc[mb][nb]);
    }
  };

  // Chunks of the last step that lie past K were not loaded; zero them (only
  // when K is not a multiple of 64).
  auto zero_tail = [&](int buf) {
    uint16_t* st = lds + buf * STAGE;
    const int kvalid = K - (nk - 1) * kBK;  // 8..56, a multiple of 8
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < ROWS * 8; i += NT) {
      const int row = i >> 3, c = i & 7;
      if (c * 8 >= kvalid) {
        const int slot = c ^ operand_swizzle(row);
        *reinterpret_cast<u32x4_t*>(&st[row * kBK + slot * 8]) = zero;
      }
    }
  };

#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    // This wave's loads of step kt have landed once at most the S-2 later
    // steps are still in flight; the barrier then publishes every wave's
    // loads and retires every wave's reads of stage (kt - 1) % S, which the
    // next issue overwrites.
    wait_vmcnt<(S - 2) * LPW>();
    stage_barrier();
    issue(kt + S - 1);
    if ((K & (kBK - 1)) && kt == nk - 1) {
      zero_tail(kt % S);
      stage_barrier();
    }
    compute(kt % S);
  }

  // Epilogue through LDS, so global stores are whole row segments:
  // acc[mb][nb] register r holds C[m0 + wm*WM + 32mb + col][n0 + wn*WN + 32nb +
  // 8(r/4) + 4half + r%4]; each wave writes its WM x WN sub-tile (bias added,
  // rounded) row-major into its own slice of LDS, then copies it out 16 bytes
  // per lane.  First drain the loads of steps past the end and let every wave
  // finish its last reads.
  wait_vmcnt<0>();
  stage_barrier();
  constexpr int SS = WN + 8;  // staging row stride (elements)
  static_assert(NW * WM * SS <= S * STAGE, "staging does not fit");
  uint16_t* stage = lds + wave * WM * SS;
  const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
  float* ln_red = reinterpret_cast<float*>(lds + NW * WM * SS);  // after the staging area
  if constexpr (LN) {
    static_assert(NW * WM * SS * 2 + 2 * WGN * TM * 4 <= S * STAGE * 2, "norm scratch does not fit");
    ln_tile_stats<Op, TM, WGN, MB, NB, WM, WN>(acc, P, m0, n0, n0 / TN, wm, wn, col, half, ln_red);
    bias = nullptr;  // already added
  }
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
        using Store = typename std::conditional<LN, F16, Op>::type;  // LN: fp16 differences
        u32x2_t w;
        w[0] = Store::pack(acc[mb][nb][4 * gq + 0] + b0, acc[mb][nb][4 * gq + 1] + b1);
        w[1] = Store::pack(acc[mb][nb][4 * gq + 2] + b2, acc[mb][nb][4 * gq + 3] + b3);
        *reinterpret_cast<u32x2_t*>(&stage[(mb * 32 + col) * SS + cl]) = w;
      }
    }
  __syncthreads();
  constexpr int CPR = WN / 8;  // 16-byte chunks per staged row
  static_assert((WM * CPR) % 64 == 0, "staged tile must split over the lanes");
#pragma unroll
  for (int i = 0; i < WM * CPR / 64; ++i) {
    const int id = lane + 64 * i, row = id / CPR, ch = id % CPR;
    const int m = m0 + wm * WM + row, n = n0 + wn * WN + ch * 8;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&stage[row * SS + ch * 8]);
    if (m < M && n < N)  // N is a multiple of 8, so the 8-run is whole
      *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(P.c) + (int64_t)m * P.ldc + n) = v;
  }
}

template <class Op, int TM, int TN, int WGM, int WGN, int S, int MINB, bool LN = false>
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
  hipExtLaunchKernelGGL((gemm_mfma_kernel<Op, TM, TN, WGM, WGN, S, MINB, LN>), dim3(total), dim3(64 * WGM * WGN),
                        0, stream, t0, t1, 0, g, tm);
  return hipGetLastError();
}

// The instantiated configurations, with the rule that picks one.  LDS per
// workgroup is S * (TM + TN) * 128 bytes; a CU has 160 KiB, so each of these
// runs two workgroups per CU.  Measured on the device (projection shapes from
// 4096 x 512 x 512 up to 16384 x 6144 x 2048): two stages beat three or four
// at every tile size (the smaller footprint lets a second workgroup share the
// CU), eight waves per CU beat four, 128 x 128 tiles win once they give at
// least one and a half rounds of the chip, and below that the shape that
// still gives every CU a workgroup wins (within 5% of the best in every case
// measured).  When 128 x 64 tiles make exactly one round (the output
// projections of the sentence-length layers: 4096 x 512 and 2048 x 1024), eight
// waves per workgroup hide more latency than four with a second workgroup that
// never comes (4096 x 512 x 512: 6.3-6.5 vs 6.8-6.9 us; with the residual and
// norm statistics 8.9-9.0 vs 9.4-9.7 us; 2048 x 1024 x 1024: unchanged), and
// with no second workgroup to share the CU a third stage costs nothing and
// keeps one more step of loads in flight (2048 x 1024 x 1024: 11.5 -> 9.3 us;
// 4096 x 512 x 512 with the norm statistics: 8.8-9.2 -> 8.0-8.1 us; without
// them unchanged at 6.5-7.0 us; four stages: no better than three).
int tiles(const GemmBatch& g, int tm, int tn) {
  int n = 0;
  for (int i = 0; i < g.count; ++i) n += ((g.p[i].M + tm - 1) / tm) * ((g.p[i].N + tn - 1) / tn);
  return n;
}

template <class Op>
hipError_t launch_sized(const GemmBatch& g, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (tiles(g, 128, 128) >= 384) return launch<Op, 128, 128, 2, 4, 2, 2>(g, stream, t0, t1);  // 64 KiB, 8 waves
  const int t64 = tiles(g, 128, 64);
  if (t64 == 256) return launch<Op, 128, 64, 4, 2, 3, 1>(g, stream, t0, t1);  // one round: 8 waves, 72 KiB
  if (t64 >= 256) return launch<Op, 128, 64, 2, 2, 2, 2>(g, stream, t0, t1);                 // 48 KiB
  return launch<Op, 64, 64, 2, 2, 2, 2>(g, stream, t0, t1);                                    // 32 KiB
}

template <class Op>
hipError_t launch_ln(const GemmProblem& p, hipStream_t stream, hipEvent_t t0, hipEvent_t t1, hipEvent_t t2,
                     hipEvent_t t3) {
  GemmBatch g{};
  g.p[0] = p;
  g.count = 1;
  hipError_t e;
  int tn;
  if (tiles(g, 128, 128) >= 384) {
    e = launch<Op, 128, 128, 2, 4, 2, 2, true>(g, stream, t0, t1);
    tn = 128;
  } else if (tiles(g, 128, 64) == 256) {
    e = launch<Op, 128, 64, 4, 2, 3, 1, true>(g, stream, t0, t1);
    tn = 64;
  } else if (tiles(g, 128, 64) >= 256) {
    e = launch<Op, 128, 64, 2, 2, 2, 2, true>(g, stream, t0, t1);
    tn = 64;
  } else {
    e = launch<Op, 64, 64, 2, 2, 2, 2, true>(g, stream, t0, t1);
    tn = 64;
  }
  if (e != hipSuccess || p.M == 0) return e;
  hipExtLaunchKernelGGL((ln_rows_kernel<Op>), dim3((unsigned)((p.M + 3) / 4)), dim3(256), 0, stream, t2, t3, 0, p,
                        tn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_ln(const GemmProblem& p, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1,
                          hipEvent_t t2, hipEvent_t t3) {
  return dt == DType::BF16 ? launch_ln<BF16>(p, stream, t0, t1, t2, t3) : launch_ln<F16>(p, stream, t0, t1, t2, t3);
}

hipError_t launch_gemm_mfma(const GemmBatch& g, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  return dt == DType::BF16 ? launch_sized<BF16>(g, stream, t0, t1) : launch_sized<F16>(g, stream, t0, t1);
}

}  // namespace mha
