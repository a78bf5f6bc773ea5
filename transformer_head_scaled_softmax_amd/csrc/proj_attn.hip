// proj_attn.hip -- fused Q/K/V projection and attention for short sequences
// (Nq, Nk <= 128 tokens, head size 64), self-attention and encoder-decoder
// cross-attention.
//
// Per head h this computes Q = x_q W_Q^T, K = x_kv W_K^T, V = x_kv W_V^T
// restricted to the head's 64 output features ("Query / Key / Value Roles",
// "Multi-Head Attention", "Cross-Attention", trishampatil.com; weights in the
// [out_features, in_features] layout of nn.Linear, "A faithful layer in code",
// aicassindra.com), rounds them to the input type exactly as the unfused path
// stores them, and then softmax(scale * Q K^T) V with padded keys (j >= L)
// and, under the causal mask, future keys (j > i) given weight exactly 0
// ("Scaled Dot-Product Attention: Step by Step", "Why Masking Is Required",
// trishampatil.com).  The head's output goes straight into its columns of the
// head-major concatenation that the output projection reads.
//
// A workgroup owns one head and a few whole sequences: their x_q rows, each
// sequence padded to NPQ rows, and (cross-attention) their x_kv rows padded to
// NPK rows -- for self-attention the x_q rows serve for K and V too.  The
// projection phase is one GEMM tile (those token rows times the 192 rows
// W_Q[h], W_K[h], W_V[h]) with the contraction over D streamed through a
// pipeline of LDS-direct loads (three stages for a grid of one round where
// they fit, else two); eight waves (two per SIMD) split it
// into equal tasks of 32x32 MFMA blocks.  The Q, K, V tiles then sit in LDS
// for the attention phase, where each wave takes 32 queries of one sequence
// and all of that sequence's (at most 128) keys at once, so the softmax is the
// plain one: exact row maximum, exponentials, sum.  For a sequence whose keys
// fit one 64-key tile of the streaming kernel its arithmetic is step for step
// the same, so both plans return bit-identical results there.
#include "mfma_util.h"

namespace mha {
namespace {

constexpr int kD = kMfmaHeadDim;         // 64
constexpr int kBK = 64;                  // contraction step
constexpr int kWRows = 3 * kD;           // W_Q, W_K, W_V rows of one head
constexpr int kNW = 8;                   // waves (two per SIMD)
constexpr int kCUs = 256;                // compute units: a grid of at most this many workgroups is one round
constexpr int kXcds = 8;
constexpr uint32_t kDead = 0x80000000u;  // beyond any range check: nothing is read

// The tile of one workgroup.  Stage rows: [0, XQ) x_q, [XQ, XQ + XK) x_kv
// (cross-attention only), then 64 rows each of W_Q[h], W_K[h], W_V[h].
// Projection tasks of MPT MFMA blocks per 16-wide step -- self: (token block,
// feature half) x {Q, K, V}; cross: an x_q block x {Q half 0, Q half 1}, then
// (x_kv block, feature half) x {K, V}.
template <bool SELF, int NPQ, int NPK>
struct Tile {
  static constexpr int IPW = SELF ? 128 / NPQ : 2;  // sequences per workgroup
  static constexpr int XQ = IPW * NPQ;
  static constexpr int XK = SELF ? 0 : IPW * NPK;
  static constexpr int KR = SELF ? XQ : XK;         // rows of the K and V tiles
  static constexpr int XQB = XQ / 32, KRB = KR / 32;
  static constexpr int WR0 = XQ + XK;                // first weight row
  static constexpr int ROWS = WR0 + kWRows;
  static constexpr int STAGE = ROWS * kBK;           // elements per stage
  static constexpr int LPW = ROWS / 8 / kNW;         // 1 KiB loads per wave per stage
  static constexpr int MPT = SELF ? 3 : 2;
  static constexpr int T = SELF ? 2 * XQB : XQB + 2 * KRB;
  static constexpr int TPW = (T + kNW - 1) / kNW;    // tasks of the busiest wave
  static_assert(NPQ % 32 == 0 && NPK % 32 == 0 && NPQ <= 128 && NPK <= 128, "row padding");
  static_assert(ROWS % (8 * kNW) == 0, "loads must split evenly over the waves");
  static_assert(XQ <= 32 * kNW / 2, "one wave per 32 queries in the attention phase");
  static_assert((XQ + 2 * KR) * kD <= 2 * STAGE, "Q, K, V tiles must fit in the stages");
  // Three pipeline stages fit a CU's 160 KiB of LDS for every self-attention
  // tile and for cross-attention over at most 32 keys.
  static constexpr bool kThreeStages = 3 * STAGE * 2 <= 160 * 1024;
};

template <class Op, bool SELF, int NPQ, int NPK, int kS>
__global__ __launch_bounds__(kNW * 64, 1) void proj_attn_kernel(ProjAttnArgs a, int groups) {
  using TL = Tile<SELF, NPQ, NPK>;
  static_assert(kS == 2 || (kS == 3 && TL::kThreeStages), "pipeline stages must fit in LDS");
  constexpr int KB = NPK / 32;  // 32-key blocks per sequence
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kS * TL::STAGE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: selects resources
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int swz = operand_swizzle(lane);  // = operand_swizzle(32m + col) for any m

  // XCD-aware order over (group, head) units, head fastest: the workgroups of
  // one XCD (block id mod 8) take a contiguous range, so they share the group's
  // rows of x and the heads' weights in that XCD's L2.
  const int U = groups * a.H, q = U / kXcds, rem = U % kXcds;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int unit = xcd * q + min(xcd, rem) + j;
  const int grp = unit / a.H, h = unit % a.H;
  const int b0 = grp * TL::IPW;
  const int Nq = a.Nq, Nk = a.Nk, D = a.D;

  // ---- Projection phase: C^T[f][t] = sum_k W[f][k] x[t][k].
  const __amdgpu_buffer_rsrc_t xqsrc = make_rsrc(a.xq, (int64_t)a.B * Nq * D * 2);
  const __amdgpu_buffer_rsrc_t xkvsrc = make_rsrc(a.xkv, (int64_t)a.B * Nk * D * 2);
  // Head h projects K and V with the rows of its key/value head (shared by
  // kv_group consecutive query heads; recomputed by each of them).
  const int kvh = a.kv_group > 1 ? h / a.kv_group : h;
  const int64_t hoff = (int64_t)h * kD * D, kvoff = (int64_t)kvh * kD * D;
  const __amdgpu_buffer_rsrc_t wsrc0 = make_rsrc(static_cast<const uint16_t*>(a.wq) + hoff, (int64_t)kD * D * 2);
  const __amdgpu_buffer_rsrc_t wsrc1 = make_rsrc(static_cast<const uint16_t*>(a.wk) + kvoff, (int64_t)kD * D * 2);
  const __amdgpu_buffer_rsrc_t wsrc2 = make_rsrc(static_cast<const uint16_t*>(a.wv) + kvoff, (int64_t)kD * D * 2);

  // Load i of this wave fills 1 KiB chunk c = wave + NW*i of a stage: rows
  // 8c .. 8c+7, lane l at row 8c + l/8, slot l%8, which holds global chunk
  // slot ^ operand_swizzle(row) = (l%8) ^ (l/8) ^ (c & 1), and c & 1 = wave & 1.
  // A chunk lies in one region (all region bounds are multiples of 32 rows):
  // src[i] = 0 x_q, 1 x_kv, 2..4 W_Q, W_K, W_V -- uniform per wave.
  const int gchunk = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
  uint32_t goff[TL::LPW];
  int src[TL::LPW];
#pragma unroll
  for (int i = 0; i < TL::LPW; ++i) {
    const int row0 = 8 * (wave + kNW * i), row = row0 + (lane >> 3);
    if (row0 < TL::XQ) {
      src[i] = 0;
      const int item = row / NPQ, t = row % NPQ;
      const bool valid = t < Nq && b0 + item < a.B;
      goff[i] = valid ? (uint32_t)((((b0 + item) * Nq + t) * D + gchunk * 8) * 2) : kDead;
    } else if (row0 < TL::WR0) {
      src[i] = 1;
      const int r = row - TL::XQ, item = r / NPK, t = r % NPK;
      const bool valid = t < Nk && b0 + item < a.B;
      goff[i] = valid ? (uint32_t)((((b0 + item) * Nk + t) * D + gchunk * 8) * 2) : kDead;
    } else {
      src[i] = 2 + (row0 - TL::WR0) / kD;
      goff[i] = (uint32_t)((((row - TL::WR0) % kD) * D + gchunk * 8) * 2);
    }
  }
  const int nk = D / kBK;
  // Every step issues exactly LPW loads per wave (steps past the end read
  // nothing), so the vmcnt waits below stay exact.
  auto issue = [&](int kt) {
    uint16_t* dst = lds + (kt % kS) * TL::STAGE;
    const uint32_t k0 = (uint32_t)kt * kBK * 2;
    const uint32_t dead = kt < nk ? 0u : kDead;
#pragma unroll
    for (int i = 0; i < TL::LPW; ++i) {
      const int off = (int)((goff[i] + k0) | dead);
      uint16_t* d = dst + (wave + kNW * i) * 512;
      if (src[i] == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xqsrc, MHA_LDS(d), 16, off, 0, 0, 0);
      else if (src[i] == 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xkvsrc, MHA_LDS(d), 16, off, 0, 0, 0);
      else if (src[i] == 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc0, MHA_LDS(d), 16, off, 0, 0, 0);
      else if (src[i] == 3)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc1, MHA_LDS(d), 16, off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wsrc2, MHA_LDS(d), 16, off, 0, 0, 0);
    }
  };

  // Task tau = wave + NW*jt (live if tau < T): its token block (stage row
  // 32*xrow + col) and the first stage row of each of its MPT weight blocks;
  // block m lands in tile tdst (0 Q, 1 K, 2 V) at feature half tfh and tile
  // row block tblk.
  int xrow[TL::TPW], wrow[TL::TPW][TL::MPT], tdst[TL::TPW][TL::MPT], tfh[TL::TPW][TL::MPT], tblk[TL::TPW];
  bool tlive[TL::TPW];
#pragma unroll
  for (int jt = 0; jt < TL::TPW; ++jt) {
    const int tau = wave + kNW * jt;
    tlive[jt] = tau < TL::T;
    if (SELF) {
      const int xb = tau % TL::XQB, hf = tau / TL::XQB;
      xrow[jt] = xb;
      tblk[jt] = xb;
#pragma unroll
      for (int m = 0; m < TL::MPT; ++m) {
        wrow[jt][m] = TL::WR0 + 64 * m + 32 * hf;
        tdst[jt][m] = m;
        tfh[jt][m] = hf;
      }
    } else if (tau < TL::XQB) {  // Q task: both halves of W_Q
      xrow[jt] = tau;
      tblk[jt] = tau;
#pragma unroll
      for (int m = 0; m < TL::MPT; ++m) {
        wrow[jt][m] = TL::WR0 + 32 * m;
        tdst[jt][m] = 0;
        tfh[jt][m] = m;
      }
    } else {  // K/V task: one half of W_K and of W_V
      const int t2 = tau - TL::XQB, xb = t2 % TL::KRB, hf = t2 / TL::KRB;
      xrow[jt] = TL::XQB + xb;
      tblk[jt] = xb;
#pragma unroll
      for (int m = 0; m < TL::MPT; ++m) {
        wrow[jt][m] = TL::WR0 + 64 * (m + 1) + 32 * hf;
        tdst[jt][m] = m + 1;
        tfh[jt][m] = hf;
      }
    }
  }
  f32x16_t acc[TL::TPW][TL::MPT];
#pragma unroll
  for (int jt = 0; jt < TL::TPW; ++jt)
#pragma unroll
    for (int m = 0; m < TL::MPT; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[jt][m][r] = 0.0f;
  // One 64-deep step of every live task of this wave: all operands of the
  // task's step are read from LDS first, then its products run, so the
  // products do not wait on the reads one by one.
  auto compute = [&](int buf) {
    const uint16_t* st = lds + buf * TL::STAGE;
#pragma unroll
    for (int jt = 0; jt < TL::TPW; ++jt) {
      if (!tlive[jt]) continue;  // wave-uniform
      u32x4_t bx[kBK / 16], aw[kBK / 16][TL::MPT];
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int slot = (kk * 2 + half) ^ swz;
        bx[kk] = *reinterpret_cast<const u32x4_t*>(&st[(32 * xrow[jt] + col) * kBK + slot * 8]);
#pragma unroll
        for (int m = 0; m < TL::MPT; ++m)
          aw[kk][m] = *reinterpret_cast<const u32x4_t*>(&st[(wrow[jt][m] + col) * kBK + slot * 8]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk)
#pragma unroll
        for (int m = 0; m < TL::MPT; ++m) acc[jt][m] = Op::mma(aw[kk][m], bx[kk], acc[jt][m]);
    }
  };

#pragma unroll
  for (int s = 0; s < kS - 1; ++s) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    // This wave's loads of step kt have landed once at most the kS-2 later
    // steps are in flight; the barrier publishes every wave's loads and
    // retires every wave's reads of the stage the next issue overwrites.
    wait_vmcnt<(kS - 2) * TL::LPW>();
    stage_barrier();
    issue(kt + kS - 1);
    compute(kt % kS);
  }
  wait_vmcnt<0>();  // the loads of steps past the end
  stage_barrier();

  // ---- Q, K, V tiles into LDS (over the stages, now free), 64 features per
  // row, rounded to the input type with the bias added.  Q and K use the
  // operand swizzle; V uses the layout of the transposing reads below.  Rows
  // of padding tokens are zero, so masked keys multiply finite values.  A
  // negative scale is folded into Q by negating it (exact).
  uint16_t* qt = lds;
  uint16_t* kt_ = lds + TL::XQ * kD;
  uint16_t* vt = kt_ + TL::KR * kD;
  const uint32_t qsign = a.scale < 0.0f ? 0x80008000u : 0u;
#pragma unroll
  for (int jt = 0; jt < TL::TPW; ++jt) {
    if (!tlive[jt]) continue;
#pragma unroll
    for (int m = 0; m < TL::MPT; ++m) {
      const int mat = tdst[jt][m];
      uint16_t* dst = mat == 0 ? qt : (mat == 1 ? kt_ : vt);
      const int np = mat == 0 ? NPQ : NPK, nvalid = mat == 0 ? Nq : Nk;
      const int t = 32 * tblk[jt] + col;  // tile row
      const bool valid = t % np < nvalid && b0 + t / np < a.B;
      // A select, not a table indexed by mat (which would live in scratch
      // memory when mat depends on the wave's task).
      const uint16_t* bias = static_cast<const uint16_t*>(mat == 0 ? a.bq : (mat == 1 ? a.bk : a.bv));
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        // Registers 4jj .. 4jj+3: features f0 .. f0+3 of tile row t.
        const int f0 = 32 * tfh[jt][m] + 8 * jj + 4 * half;
        float bb[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bias) {
#pragma unroll
          for (int e = 0; e < 4; ++e) bb[e] = Op::to_float(bias[(mat == 0 ? h : kvh) * kD + f0 + e]);
        }
        u32x2_t v = {0u, 0u};
        if (valid) {
          v[0] = Op::pack(acc[jt][m][4 * jj + 0] + bb[0], acc[jt][m][4 * jj + 1] + bb[1]);
          v[1] = Op::pack(acc[jt][m][4 * jj + 2] + bb[2], acc[jt][m][4 * jj + 3] + bb[3]);
          if (mat == 0) {
            v[0] ^= qsign;
            v[1] ^= qsign;
          }
        }
        const int c = f0 >> 3;  // 16-byte chunk of the row
        const int slot = mat == 2 ? (c ^ (((t >> 1) & 1) << 2)) : (c ^ operand_swizzle(t));
        *reinterpret_cast<u32x2_t*>(&dst[t * kD + slot * 8 + 4 * half]) = v;
      }
    }
  }
  __syncthreads();

  // ---- Attention phase: wave w < XQ/32 takes Q tile rows 32w .. 32w+31,
  // i.e. queries q0 .. q0+31 of sequence `item`, whose keys are K/V tile rows
  // kb0 .. kb0+NPK-1.  Further waves are done.
  if (wave >= TL::XQ / 32) return;  // wave-uniform; no barrier follows
  const int item = (32 * wave) / NPQ, q0 = (32 * wave) % NPQ, kb0 = item * NPK;
  const int b = b0 + item;
  if (b >= a.B || q0 >= Nq) return;
  int L = Nk;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), Nk);
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
  // The row sum is kept as four partial sums (one per register pair of a
  // step), combined as (0 + 1) + (2 + 3) -- the order of the per-head
  // attention kernel, so the two agree bit for bit on one 64-key tile.
  u32x4_t pb[2 * KB];
  float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int t4 = 0; t4 < 2 * KB; ++t4)
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const int jb = t4 >> 1, r = (t4 & 1) * 8 + 2 * w4;
      const int key = 32 * jb + 8 * (r >> 2) + 4 * half + (r & 3);  // key of register r; r+1 is key+1
      const float p0 = key < kend ? __builtin_amdgcn_exp2f(fmaf(s[jb][r], c2, -mc)) : 0.0f;
      const float p1 = key + 1 < kend ? __builtin_amdgcn_exp2f(fmaf(s[jb][r + 1], c2, -mc)) : 0.0f;
      pb[t4][w4] = Op::pack(p0, p1);
      lp[w4] = Op::sum2(pb[t4][w4], lp[w4]);
    }
  const float ltot = lanes_sum((lp[0] + lp[1]) + (lp[2] + lp[3]));

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
  uint16_t* obase = static_cast<uint16_t*>(a.o) + ((int64_t)b * Nq + q0) * ldo + h * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = lane + 64 * i, row = id >> 3, ch = id & 7;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&stage[row * kD + (ch ^ operand_swizzle(row)) * 8]);
    if (q0 + row < Nq) *reinterpret_cast<u32x4_t*>(obase + (int64_t)row * ldo + ch * 8) = v;
  }
}

// A grid of at most one round takes a third pipeline stage where it fits: the
// projection loop waits on operand latency there (base encoder sublayer: 14.6
// -> 14.1 us).  Larger grids keep two stages, so that two workgroups share a
// CU (B = 384: 71.3 us with two stages, 75.2 us with three).
template <class Op, bool SELF, int NPQ, int NPK>
hipError_t launch(const ProjAttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  using TL = Tile<SELF, NPQ, NPK>;
  const int groups = (a.B + TL::IPW - 1) / TL::IPW;
  const int64_t blocks = (int64_t)groups * a.H;
  if (blocks == 0) return hipSuccess;
  if constexpr (TL::kThreeStages) {
    if (blocks <= kCUs) {
      hipExtLaunchKernelGGL((proj_attn_kernel<Op, SELF, NPQ, NPK, 3>), dim3((unsigned)blocks), dim3(kNW * 64), 0,
                            stream, t0, t1, 0, a, groups);
      return hipGetLastError();
    }
  }
  hipExtLaunchKernelGGL((proj_attn_kernel<Op, SELF, NPQ, NPK, 2>), dim3((unsigned)blocks), dim3(kNW * 64), 0, stream,
                        t0, t1, 0, a, groups);
  return hipGetLastError();
}

template <class Op, int NPQ>
hipError_t launch_cross(const ProjAttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (a.Nk <= 32) return launch<Op, false, NPQ, 32>(a, stream, t0, t1);
  if (a.Nk <= 64) return launch<Op, false, NPQ, 64>(a, stream, t0, t1);
  if (a.Nk <= 96) return launch<Op, false, NPQ, 96>(a, stream, t0, t1);
  return launch<Op, false, NPQ, 128>(a, stream, t0, t1);
}

template <class Op>
hipError_t launch_sized(const ProjAttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (a.xkv == a.xq) {
    if (a.Nq <= 32) return launch<Op, true, 32, 32>(a, stream, t0, t1);
    if (a.Nq <= 64) return launch<Op, true, 64, 64>(a, stream, t0, t1);
    return launch<Op, true, 128, 128>(a, stream, t0, t1);
  }
  return a.Nq <= 32 ? launch_cross<Op, 32>(a, stream, t0, t1) : launch_cross<Op, 64>(a, stream, t0, t1);
}

}  // namespace

hipError_t launch_proj_attn(const ProjAttnArgs& a, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  return dt == DType::BF16 ? launch_sized<BF16>(a, stream, t0, t1) : launch_sized<F16>(a, stream, t0, t1);
}

}  // namespace mha
