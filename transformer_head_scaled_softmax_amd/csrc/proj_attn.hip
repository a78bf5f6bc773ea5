// proj_attn.hip -- fused Q/K/V projection and attention for short
// self-attention (N <= 128 tokens per sequence, head size 64).
//
// Per head h this computes Q = x W_Q^T, K = x W_K^T, V = x W_V^T restricted to
// the head's 64 output features ("Query / Key / Value Roles", "Multi-Head
// Attention", trishampatil.com; weights in the [out_features, in_features]
// layout of nn.Linear, "A faithful layer in code", aicassindra.com), rounds
// them to the input type exactly as the unfused path stores them, and then
// softmax(scale * Q K^T) V with padded keys (j >= L) and, under the causal
// mask, future keys (j > i) given weight exactly 0 ("Scaled Dot-Product
// Attention: Step by Step", "Why Masking Is Required", trishampatil.com).
// The head's output goes straight into its columns of the head-major
// concatenation that the output projection reads.
//
// A workgroup owns 128 token rows -- 128/NP whole sequences padded to NP rows
// (NP = 32, 64 or 128) -- and one head, so the projections' K/V never leave
// the CU: the projection phase is a 128 x 192 GEMM tile (rows of x times the
// 192 rows W_Q[h], W_K[h], W_V[h]) with the contraction over D streamed through
// a two-stage LDS pipeline of LDS-direct loads (eight waves, two per SIMD);
// the Q, K, V tiles then sit
// in LDS for the attention phase, where each wave takes 32 query rows of one
// sequence and all of that sequence's (at most 128) keys at once, so the
// softmax is the plain one: exact row maximum, exponentials, sum.
#include "mfma_util.h"

namespace mha {
namespace {

constexpr int kD = kMfmaHeadDim;                 // 64
constexpr int kBK = 64;                          // contraction step
constexpr int kRows = 128;                       // token rows per workgroup
constexpr int kWRows = 3 * kD;                   // W_Q, W_K, W_V rows of one head
constexpr int kStageRows = kRows + kWRows;       // 320 rows of 128 bytes
constexpr int kStage = kStageRows * kBK;         // elements per stage
constexpr int kS = 2;                            // pipeline stages (80 KiB)
constexpr int kNW = 8;                           // waves (two per SIMD)
constexpr int kLPW = kStageRows / 8 / kNW;       // 1 KiB loads per wave per stage (5)
constexpr int kXLoads = kRows / 8 / kNW;         // the first 2 of them are rows of x
constexpr int kXB = 2 * 4 / kNW;                 // 32-token blocks per wave in the projection
constexpr int kXcds = 8;
constexpr uint32_t kDead = 0x80000000u;          // beyond any range check: nothing is read
static_assert(kRows % (8 * kNW) == 0 && kWRows % (8 * kNW) == 0 && kD % 8 == 0, "loads must split evenly");
static_assert(kNW == 4 || kNW == 8, "wave layouts are written for 4 or 8 waves");

template <class Op, int NP>
__global__ __launch_bounds__(kNW * 64, 1) void proj_attn_kernel(ProjAttnArgs a, int groups) {
  constexpr int IPW = kRows / NP;  // sequences per workgroup
  constexpr int KB = NP / 32;      // 32-key blocks per sequence
  static_assert(NP == 32 || NP == 64 || NP == 128, "unsupported padding");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kS * kStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: selects resources
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int swz = operand_swizzle(lane);  // = operand_swizzle(32m + col) for any m

  // XCD-aware order over (group, head) units, head fastest: the workgroups of
  // one XCD (block id mod 8) take a contiguous range, so they share the group's
  // rows of x and the heads' weights in that XCD's L2.
  const int T = groups * a.H, q = T / kXcds, rem = T % kXcds;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int unit = xcd * q + min(xcd, rem) + j;
  const int grp = unit / a.H, h = unit % a.H;
  const int b0 = grp * IPW;
  const int N = a.N, D = a.D;

  // ---- Projection phase: C^T[f][t] = sum_k W[f][k] x[t][k], f over the 192
  // rows of the head's three weight matrices, t over the 128 token rows.
  const __amdgpu_buffer_rsrc_t xsrc = make_rsrc(a.x, (int64_t)a.B * N * D * 2);
  const int64_t hoff = (int64_t)h * kD * D;
  const __amdgpu_buffer_rsrc_t wsrc0 = make_rsrc(static_cast<const uint16_t*>(a.wq) + hoff, (int64_t)kD * D * 2);
  const __amdgpu_buffer_rsrc_t wsrc1 = make_rsrc(static_cast<const uint16_t*>(a.wk) + hoff, (int64_t)kD * D * 2);
  const __amdgpu_buffer_rsrc_t wsrc2 = make_rsrc(static_cast<const uint16_t*>(a.wv) + hoff, (int64_t)kD * D * 2);

  // Load i of this wave fills 1 KiB chunk c = wave + NW*i of a stage: rows
  // 8c .. 8c+7, lane l at row 8c + l/8, slot l%8, which holds global chunk
  // slot ^ operand_swizzle(row) = (l%8) ^ (l/8) ^ (c & 1), and c & 1 = wave & 1.
  // Stage rows 0..127 are token rows (sequence r / NP, token r % NP), rows
  // 128 + 64w + r are row r of W_Q[h], W_K[h], W_V[h] for w = 0, 1, 2; the
  // loads i >= kXLoads read weight rows.
  const int gchunk = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
  uint32_t goff[kLPW];
  int wmat[kLPW];  // weight matrix of load i (uniform per wave)
#pragma unroll
  for (int i = 0; i < kLPW; ++i) {
    const int row = 8 * (wave + kNW * i) + (lane >> 3);
    wmat[i] = (8 * (wave + kNW * i) - kRows) / kD;
    if (i < kXLoads) {
      const int item = row / NP, t = row % NP;
      const bool valid = t < N && b0 + item < a.B;
      goff[i] = valid ? (uint32_t)((((b0 + item) * N + t) * D + gchunk * 8) * 2) : kDead;
    } else {
      goff[i] = (uint32_t)((((row - kRows) % kD) * D + gchunk * 8) * 2);
    }
  }
  const int nk = D / kBK;
  auto issue = [&](int kt) {
    uint16_t* dst = lds + (kt % kS) * kStage;
    const uint32_t k0 = (uint32_t)kt * kBK * 2;
    const uint32_t dead = kt < nk ? 0u : kDead;  // steps past the end read nothing
#pragma unroll
    for (int i = 0; i < kLPW; ++i) {
      const int off = (int)((goff[i] + k0) | dead);
      uint16_t* d = dst + (wave + kNW * i) * 512;
      if (i < kXLoads)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xsrc, MHA_LDS(d), 16, off, 0, 0, 0);
      else if (wmat[i] == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc0, MHA_LDS(d), 16, off, 0, 0, 0);
      else if (wmat[i] == 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc1, MHA_LDS(d), 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc2, MHA_LDS(d), 16, off, 0, 0, 0);
    }
  };

  // Wave (wx, ww) = (wave % (NW/2), wave / (NW/2)): token blocks
  // kXB*wx .. kXB*wx + kXB-1 times the 32-feature half ww of each of Q, K, V
  // -- 3*kXB blocks of 32x32, kXB + 3 operand reads per 16-wide step.
  const int wx = wave % (kNW / 2), ww = wave / (kNW / 2);
  f32x16_t acc[3][kXB];
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int xb = 0; xb < kXB; ++xb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][xb][r] = 0.0f;
  auto compute = [&](int buf) {
    const uint16_t* st = lds + buf * kStage;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int slot = (kk * 2 + half) ^ swz;
      u32x4_t bx[kXB], aw[3];
#pragma unroll
      for (int xb = 0; xb < kXB; ++xb)
        bx[xb] = *reinterpret_cast<const u32x4_t*>(&st[(32 * (kXB * wx + xb) + col) * kBK + slot * 8]);
#pragma unroll
      for (int m = 0; m < 3; ++m)
        aw[m] = *reinterpret_cast<const u32x4_t*>(&st[(kRows + 64 * m + 32 * ww + col) * kBK + slot * 8]);
#pragma unroll
      for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int xb = 0; xb < kXB; ++xb) acc[m][xb] = Op::mma(aw[m], bx[xb], acc[m][xb]);
    }
  };

#pragma unroll
  for (int s = 0; s < kS - 1; ++s) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    // This wave's loads of step kt have landed once at most the kS-2 later
    // steps are in flight; the barrier publishes every wave's loads and
    // retires every wave's reads of the stage the next issue overwrites.
    wait_vmcnt<(kS - 2) * kLPW>();
    stage_barrier();
    issue(kt + kS - 1);
    compute(kt % kS);
  }
  wait_vmcnt<0>();  // the loads of steps past the end
  stage_barrier();

  // ---- Q, K, V tiles into LDS (over the stages, now free): 128 rows of 64
  // features each, rounded to the input type with the bias added.  Q and K
  // use the operand swizzle; V uses the layout of the transposing reads
  // below.  Rows of padding tokens are zero, so masked keys multiply finite
  // values.  A negative scale is folded into Q by negating it (exact).
  uint16_t* qt = lds;
  uint16_t* kt_ = lds + kRows * kD;
  uint16_t* vt = lds + 2 * kRows * kD;
  const uint32_t qsign = a.scale < 0.0f ? 0x80008000u : 0u;
  const uint16_t* bias[3] = {static_cast<const uint16_t*>(a.bq), static_cast<const uint16_t*>(a.bk),
                             static_cast<const uint16_t*>(a.bv)};
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    uint16_t* dst = m == 0 ? qt : (m == 1 ? kt_ : vt);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      // Registers 4jj .. 4jj+3 of acc[m][xb]: features f0 .. f0+3 of token t.
      const int f0 = 32 * ww + 8 * jj + 4 * half;
      float bb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (bias[m]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bb[e] = Op::to_float(bias[m][h * kD + f0 + e]);
      }
      const int c = f0 >> 3;  // 16-byte chunk of the row
#pragma unroll
      for (int xb = 0; xb < kXB; ++xb) {
        const int t = 32 * (kXB * wx + xb) + col;
        const bool valid = t % NP < N && b0 + t / NP < a.B;
        u32x2_t v = {0u, 0u};
        if (valid) {
          v[0] = Op::pack(acc[m][xb][4 * jj + 0] + bb[0], acc[m][xb][4 * jj + 1] + bb[1]);
          v[1] = Op::pack(acc[m][xb][4 * jj + 2] + bb[2], acc[m][xb][4 * jj + 3] + bb[3]);
          if (m == 0) {
            v[0] ^= qsign;
            v[1] ^= qsign;
          }
        }
        const int slot = m == 2 ? (c ^ (((t >> 1) & 1) << 2)) : (c ^ operand_swizzle(t));
        *reinterpret_cast<u32x2_t*>(&dst[t * kD + slot * 8 + 4 * half]) = v;
      }
    }
  }
  __syncthreads();

  // ---- Attention phase: wave w < 4 takes token rows 32w .. 32w+31 of the
  // tile, i.e. queries q0 .. q0+31 of sequence `item`; the sequence's keys are
  // tile rows kb0 .. kb0+NP-1.  Further waves are done.
  if (wave >= kRows / 32) return;  // wave-uniform; no barrier follows
  const int item = (32 * wave) / NP, q0 = (32 * wave) % NP, kb0 = item * NP;
  const int b = b0 + item;
  if (b >= a.B || q0 >= N) return;
  int L = N;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), N);
  const int qi = q0 + col;
  const int kend = a.causal ? min(L, qi + 1) : L;  // keys this lane's query sees
  const float c2 = fabsf(a.scale) * kLog2e;

  u32x4_t qreg[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qreg[kk] = *reinterpret_cast<const u32x4_t*>(&qt[(32 * wave + col) * kD + ((2 * kk + half) ^ swz) * 8]);

  // S^T = K Q^T: register r of s[kb] holds key 32kb + 8(r/4) + 4half + r%4.
  f32x16_t s[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4_t av =
          *reinterpret_cast<const u32x4_t*>(&kt_[(kb0 + 32 * kb + col) * kD + ((2 * kk + half) ^ swz) * 8]);
      s[kb] = Op::mma(av, qreg[kk], s[kb]);
    }
  }
  // Row maximum over the visible keys (both halves of the query's lanes).
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * kb + 8 * (r >> 2) + 4 * half + (r & 3) < kend) mx = fmaxf(mx, s[kb][r]);
  mx = lanes_max(mx);
  const float mc = mx == -INFINITY ? 0.0f : mx * c2;

  // P = exp2(s * c2 - mc) for visible keys, 0 for the rest, packed in the
  // order of the P^T operand: 16-key step t4 takes registers 8(t4%2) .. +7 of
  // s[t4/2], i.e. keys 16t4 + 4half + {0..3} and 16t4 + 8 + 4half + {0..3}.
  u32x4_t pb[2 * KB];
  float ls = 0.0f;
#pragma unroll
  for (int t4 = 0; t4 < 2 * KB; ++t4)
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const int jb = t4 >> 1, r = (t4 & 1) * 8 + 2 * w4;
      const int key = 32 * jb + 8 * (r >> 2) + 4 * half + (r & 3);  // key of register r; r+1 is key+1
      const float p0 = key < kend ? __builtin_amdgcn_exp2f(fmaf(s[jb][r], c2, -mc)) : 0.0f;
      const float p1 = key + 1 < kend ? __builtin_amdgcn_exp2f(fmaf(s[jb][r + 1], c2, -mc)) : 0.0f;
      pb[t4][w4] = Op::pack(p0, p1);
      ls = Op::sum2(pb[t4][w4], ls);
    }
  const float ltot = lanes_sum(ls);

  // O^T += V^T P^T.  ds_read_b64_tr_b16: in each group of 16 lanes, lane
  // 4k + q points at key row (k0 + k), features c0 + 4q .. +3, and lane l'
  // then holds feature c0 + l' of keys k0 .. k0+3 (the A-operand layout).
  // V rows are 128 bytes with chunk c stored at c ^ (bit 1 of the row) << 2,
  // which keeps these reads free of bank conflicts.
  const int tr_k = (lane & 15) >> 2, tr_q = lane & 3, tr_cg = (lane >> 4) & 1;
  const int tr_row = 4 * half + tr_k;
  int tr_col[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int cidx = cb * 32 + 16 * tr_cg + 4 * tr_q;
    tr_col[cb] = ((((cidx >> 3) ^ (((tr_k >> 1) & 1) << 2))) << 3) + (cidx & 7);
  }
  auto vread = [&](int row, int cb) -> u32x2_t {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    lds_s16x4_t* p = (lds_s16x4_t*)(const __attribute__((address_space(3))) uint16_t*)&vt[row * kD + tr_col[cb]];
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
  };
  f32x16_t o[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;
#pragma unroll
  for (int t4 = 0; t4 < 2 * KB; ++t4)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const u32x2_t lo = vread(kb0 + 16 * t4 + tr_row, cb);
      const u32x2_t hi = vread(kb0 + 16 * t4 + 8 + tr_row, cb);
      const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
      o[cb] = Op::mma(av, pb[t4], o[cb]);
    }

  // Epilogue: normalise, stage the 32 x 64 output in this wave's own Q rows
  // (no other wave reads them), and store whole 128-byte rows.  Register
  // (cb, 4g + e) is feature 32cb + 8g + 4half + e of query q0 + col.
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  uint16_t* stage = qt + 32 * wave * kD;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2_t w;
      w[0] = Op::pack(o[cb][4 * g + 0] * inv, o[cb][4 * g + 1] * inv);
      w[1] = Op::pack(o[cb][4 * g + 2] * inv, o[cb][4 * g + 3] * inv);
      *reinterpret_cast<u32x2_t*>(&stage[col * kD + ((4 * cb + g) ^ swz) * 8 + 4 * half]) = w;
    }
  const int ldo = a.H * kD;
  uint16_t* obase = static_cast<uint16_t*>(a.o) + ((int64_t)b * N + q0) * ldo + h * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = lane + 64 * i, row = id >> 3, ch = id & 7;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&stage[row * kD + (ch ^ operand_swizzle(row)) * 8]);
    if (q0 + row < N) *reinterpret_cast<u32x4_t*>(obase + (int64_t)row * ldo + ch * 8) = v;
  }
}

template <class Op, int NP>
hipError_t launch(const ProjAttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  constexpr int IPW = kRows / NP;
  const int groups = (a.B + IPW - 1) / IPW;
  const int64_t blocks = (int64_t)groups * a.H;
  if (blocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL((proj_attn_kernel<Op, NP>), dim3((unsigned)blocks), dim3(kNW * 64), 0, stream, t0, t1, 0, a,
                        groups);
  return hipGetLastError();
}

template <class Op>
hipError_t launch_sized(const ProjAttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (a.N <= 32) return launch<Op, 32>(a, stream, t0, t1);
  if (a.N <= 64) return launch<Op, 64>(a, stream, t0, t1);
  return launch<Op, 128>(a, stream, t0, t1);
}

}  // namespace

bool proj_attn_supported(int N, int D, int d_k, int d_v) {
  return N >= 1 && N <= kRows && D >= kBK && D % kBK == 0 && d_k == kD && d_v == kD;
}

hipError_t launch_proj_attn(const ProjAttnArgs& a, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  return dt == DType::BF16 ? launch_sized<BF16>(a, stream, t0, t1) : launch_sized<F16>(a, stream, t0, t1);
}

}  // namespace mha
