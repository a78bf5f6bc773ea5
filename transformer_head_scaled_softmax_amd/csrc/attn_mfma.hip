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
// Work split.  A workgroup owns 32*NW*QS consecutive queries of one (b, h);
// each wave owns 32*QS of them, as QS sub-blocks of 32 that share every K
// operand read.  Per key tile a wave computes the TRANSPOSED scores
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
// Softmax bookkeeping, per query: m_ref is a reference maximum (in log2
// units) and p = exp2(s * scale * log2e - m_ref), accumulated into a running
// sum and the O^T accumulators; the final division by the sum cancels m_ref, so
// any reference gives the same result in exact arithmetic.  Each tile is first
// exponentiated against the current reference without computing its maximum;
// only if a query's partial sum is not finite or exceeds a guard (2^64 for
// bf16 P, 2^15 for f16 P) -- its first visible tile, or a new maximum far above
// the reference -- does that query take the tile's true maximum as its new
// reference, rescale its accumulators and exponentiate the tile again.  Row
// sums come from the packed P values with v_dot2, i.e. from exactly the
// rounded values the P*V product multiplies.
#include "mfma_util.h"

namespace mha {
namespace {

constexpr int kD = kMfmaHeadDim;  // 64
constexpr int kBN = 64;           // keys per tile
constexpr int kKS = 72;           // K tile row stride (elements): 144 B -> conflict-free 16 B reads
constexpr int kDeadOffset = (int)0x80000000u;  // beyond any range check: loads return zeros

template <class Op, int NW, int QS>
__global__ __launch_bounds__(NW * 64, NW >= 8 ? 1 : 2) void attn_mfma_kernel(AttnArgs a, int nqb) {
  constexpr int NT = NW * 64;
  constexpr int QW = 32 * QS;         // queries per wave: QS sub-blocks of 32
  constexpr int QB = NW * QW;         // queries per workgroup
  constexpr int CH = (kBN * 8) / NT;  // 16-byte chunks of K (and of V) per thread per tile
  static_assert(CH >= 1, "tile too small for the workgroup");

  // K and V tiles, double-buffered; after the key loop the same memory stages
  // the output rows (32 rows of kKS elements per wave).
  constexpr int kTiles = 2 * kBN * kKS + 2 * kBN * kD;
  __shared__ __attribute__((aligned(16))) uint16_t lds[kTiles > NW * 32 * kKS ? kTiles : NW * 32 * kKS];
  uint16_t (*ks)[kBN * kKS] = reinterpret_cast<uint16_t (*)[kBN * kKS]>(lds);
  uint16_t (*vs)[kBN * kD] = reinterpret_cast<uint16_t (*)[kBN * kD]>(lds + 2 * kBN * kKS);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;

  // Longest query blocks first: under the causal mask later blocks see more keys.
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int b = bh / a.H, h = bh % a.H;

  int L = a.Nk;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), a.Nk);
  const int kvh = a.kv_group > 1 ? h / a.kv_group : h;  // key/value head read by head h
  const int coff = a.causal_end ? L - a.Nq : 0;         // causal: query i sees keys j <= i + coff
  const int q0 = qb * QB;
  const int qw0 = q0 + wave * QW;
  int qi[QS], kend[QS];
  bool qvalid[QS];
#pragma unroll
  for (int u = 0; u < QS; ++u) {
    qi[u] = qw0 + 32 * u + col;
    qvalid[u] = qi[u] < a.Nq;
    kend[u] = a.causal ? min(L, qi[u] + 1 + coff) : L;  // keys this query sees (<= 0: none)
  }
  const int kend_blk = a.causal ? min(L, min(q0 + QB, a.Nq) + coff) : L;    // keys the workgroup needs
  const int kmin_wave = a.causal ? min(L, qw0 + 1 + coff) : L;              // tiles below: no masking
  const int kmax_wave = a.causal ? min(L, min(qw0 + QW, a.Nq) + coff) : L;  // tiles from here: skip
  const int ntiles = (max(kend_blk, 0) + kBN - 1) / kBN;

  // Range-checked buffers over this (b, h): query rows past Nq and key/value
  // rows at or past the workgroup's key end read as zeros, so padded rows are
  // never loaded and the loads need no branches.
  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + b * a.q_sb + h * a.q_sh;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.v_sb + kvh * a.v_sh;
  const __amdgpu_buffer_rsrc_t qsrc = make_rsrc(qbase, ((int64_t)(a.Nq - 1) * a.q_sn + kD) * 2);
  const __amdgpu_buffer_rsrc_t ksrc =
      make_rsrc(kbase, kend_blk > 0 ? ((int64_t)(kend_blk - 1) * a.k_sn + kD) * 2 : 0);
  const __amdgpu_buffer_rsrc_t vsrc =
      make_rsrc(vbase, kend_blk > 0 ? ((int64_t)(kend_blk - 1) * a.v_sn + kD) * 2 : 0);

  // This lane's queries as B operands of S^T = K Q^T: features 16kk + 8half .. +7.
  // A negative scale is folded in by negating q (exact), so the softmax below
  // always multiplies by a non-negative c2.
  const uint32_t qsign = a.scale < 0.0f ? 0x80008000u : 0u;
  const float c2 = fabsf(a.scale) * kLog2e;
  u32x4_t qreg[QS][4];
#pragma unroll
  for (int u = 0; u < QS; ++u) {
    const int qoff = qvalid[u] ? (int)(qi[u] * a.q_sn * 2) + half * 16 : kDeadOffset;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qreg[u][kk] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, qoff + kk * 32, 0, 0) ^ qsign;
  }

  // Staging: each thread moves CH 16-byte chunks of the K tile and of the V
  // tile.  K rows keep a padded stride (conflict-free 16-byte operand reads);
  // V rows are dense 128-byte rows whose chunks are XOR-swizzled by bit 1 of
  // the row, which makes the transposing operand reads below conflict-free.
  int koff[CH], voff[CH], kpos[CH], vpos[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = tid + c * NT, row = idx >> 3, ch = idx & 7;
    koff[c] = (int)((row * a.k_sn + ch * 8) * 2);
    voff[c] = (int)((row * a.v_sn + ch * 8) * 2);
    kpos[c] = row * kKS + ch * 8;
    vpos[c] = row * kD + ((ch ^ (((row >> 1) & 1) << 2)) << 3);
  }
  const int ktile = (int)(kBN * a.k_sn * 2), vtile = (int)(kBN * a.v_sn * 2);
  // Tiles at or past the workgroup's key end fall outside the range check, so
  // the prefetch issued after the last tile reads nothing.
  u32x4_t kreg[CH], vreg[CH];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      kreg[c] = __builtin_amdgcn_raw_buffer_load_b128(ksrc, koff[c] + t * ktile, 0, 0);
      vreg[c] = __builtin_amdgcn_raw_buffer_load_b128(vsrc, voff[c] + t * vtile, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      *reinterpret_cast<u32x4_t*>(&ks[buf][kpos[c]]) = kreg[c];
      *reinterpret_cast<u32x4_t*>(&vs[buf][vpos[c]]) = vreg[c];
    }
  };

  // V^T operand of O^T += V^T P^T through ds_read_b64_tr_b16.  In each group of
  // 16 lanes the instruction hands lane l element l%4 of the 4-element runs read
  // by lanes l/4 + 4k (k = 0..3); so lane 4k + q points at key row (k0 + k),
  // features (c0 + 4q .. +3), and lane l' then holds features c0 + l' of keys
  // k0 .. k0+3 -- the A-operand layout (feature row, 4 consecutive keys).
  // Group g = lane/16 covers features 16(g%2) of the block and key half g/2.
  const int tr_k = (lane & 15) >> 2, tr_q = lane & 3, tr_cg = (lane >> 4) & 1;
  const int tr_row = 4 * half + tr_k;  // + 16 t4 (+ 8 for keys 8..15 of the step)
  int tr_col[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int cidx = cb * 32 + 16 * tr_cg + 4 * tr_q;
    tr_col[cb] = ((((cidx >> 3) ^ (((tr_k >> 1) & 1) << 2))) << 3) + (cidx & 7);
  }
  auto vread = [&](int buf, int row, int cb) -> u32x2_t {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    lds_s16x4_t* p = (lds_s16x4_t*)(const __attribute__((address_space(3))) uint16_t*)&vs[buf][row * kD + tr_col[cb]];
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
  };

  f32x16_t o[QS][2];
  float m_ref[QS], lsum[QS];
#pragma unroll
  for (int u = 0; u < QS; ++u) {
    m_ref[u] = -INFINITY;
    lsum[u] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[u][cb][r] = 0.0f;
  }

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * kBN;
    load_tile(t + 1);

    if (j0 < kmax_wave) {  // wave-uniform: tiles past all of this wave's rows are skipped
      // S^T = K_tile Q^T: two 32-key blocks; each K operand read serves every
      // query sub-block of the wave.
      // All eight K operands are read before the first product, so the
      // products do not wait on LDS one pair at a time.
      u32x4_t kop[2][4];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          kop[jb][kk] = *reinterpret_cast<const u32x4_t*>(&ks[buf][(jb * 32 + col) * kKS + kk * 16 + half * 8]);
      __builtin_amdgcn_sched_barrier(0);  // keep the eight reads ahead of the products
      f32x16_t s[QS][2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int u = 0; u < QS; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[u][jb][r] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int u = 0; u < QS; ++u) s[u][jb] = Op::mma(kop[jb][kk], qreg[u][kk], s[u][jb]);
      }

      // V^T operands of O^T += V^T P^T for the whole tile, read once and used
      // by every query sub-block: step t4 supplies keys 16t4 + 4half + {0..3}
      // and 16t4 + 8 + 4half + {0..3} of this lane's feature row.
      u32x4_t vop[4][2];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const u32x2_t lo = vread(buf, 16 * t4 + tr_row, cb);
          const u32x2_t hi = vread(buf, 16 * t4 + 8 + tr_row, cb);
          vop[t4][cb] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }

      // Register (jb, r) of this lane holds key j0 + 32jb + 8(r/4) + 4half + r%4;
      // invisible keys become -inf (only diagonal and tail tiles have any).
      if (j0 + kBN > kmin_wave) {
#pragma unroll
        for (int u = 0; u < QS; ++u) {
          const int lim = kend[u] - j0 - 4 * half;
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (jb * 32 + (r >> 2) * 8 + (r & 3) >= lim) s[u][jb][r] = -INFINITY;
        }
      }

      // Sub-blocks one after the other: softmax, then P V, with no branch
      // between one sub-block's P V MFMAs and the next one's softmax
      // arithmetic, so the two can be interleaved.
#pragma unroll
      for (int u = 0; u < QS; ++u) {
        u32x4_t pb[4];

        // P = exp2(s * c2 - m_ref), packed to the MFMA input type in the order
        // the P^T operand needs (step t4 takes registers 8(t4%2) .. +7 of
        // s[t4/2]); the row sum comes from the packed values with v_dot2.
        float ls = 0.0f;
        auto exponentiate = [&](float mu, bool select_masked) {
          // Four partial sums (one per register pair of a step) keep the
          // v_dot2 accumulation chains short.
          float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const int jb = t4 >> 1, r = (t4 & 1) * 8 + 2 * w;
              float p0 = __builtin_amdgcn_exp2f(fmaf(s[u][jb][r], c2, -mu));
              float p1 = __builtin_amdgcn_exp2f(fmaf(s[u][jb][r + 1], c2, -mu));
              if (select_masked) {
                p0 = s[u][jb][r] == -INFINITY ? 0.0f : p0;
                p1 = s[u][jb][r + 1] == -INFINITY ? 0.0f : p1;
              }
              pb[t4][w] = Op::pack(p0, p1);
              lp[w] = Op::sum2(pb[t4][w], lp[w]);
            }
          ls = (lp[0] + lp[1]) + (lp[2] + lp[3]);
        };
        // Optimistic pass against the current reference.  It is kept unless
        // this query's partial sum is not finite or exceeds kGuard (a new
        // maximum far above the reference, or masked keys with no reference
        // yet).  While no query of the wave has a reference (its first tile)
        // the pass would always fail; the short-sequence configuration (QS = 1,
        // mostly a single tile) skips it then, which halves its softmax work
        // (7.95 vs 8.2 us on the base decoder workload).  Long sequences keep
        // the branch-free loop (the check cost 3% there).
        bool need = true;
        if (QS > 1 || !__all(m_ref[u] == -INFINITY)) {
          exponentiate(m_ref[u], false);
          need = lanes_max(ls <= Op::kGuard ? 0.0f : 1.0f) > 0.0f;
        }
        if (__any(need)) {
          float mx = -INFINITY;
#pragma unroll
          for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[u][jb][r]);
          mx = lanes_max(mx);
          const float mt = (mx == -INFINITY) ? -INFINITY : mx * c2;
          // Queries that passed keep their reference, so a row's arithmetic
          // never depends on other rows' data.
          const float m_new = need ? fmaxf(m_ref[u], mt) : m_ref[u];
          const float alpha = (need && m_new != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref[u] - m_new) : 1.0f;
          lsum[u] *= alpha;
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[u][cb][r] *= alpha;
          m_ref[u] = m_new;
          // Masked keys get exactly 0, also when scale is 0 or no key is visible yet.
          exponentiate(m_ref[u] == -INFINITY ? 0.0f : m_ref[u], true);
        }
        lsum[u] += ls;

#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) o[u][cb] = Op::mma(vop[t4][cb], pb[t4], o[u][cb]);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue through LDS so the output rows leave as whole 128-byte segments:
  // register (cb, 4g + e) of this lane is feature 32cb + 8g + 4half + e of query
  // 32u + col.  Each wave stages one 32-query sub-block at a time in its own
  // 32 x kKS slice of the tile memory (free after the loop's last barrier) and
  // copies it out 16 bytes per lane.
  uint16_t* stage = lds + wave * 32 * kKS;
#pragma unroll
  for (int u = 0; u < QS; ++u) {
    const float ltot = lanes_sum(lsum[u]);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    // Row statistic for the backward pass: ln(sum_j exp(scale q.k_j)) =
    // (m_ref + log2(sum)) * ln 2, whatever reference the row ended with.
    if (a.lse && half == 0 && qvalid[u])
      a.lse[((int64_t)b * a.H + h) * a.Nq + qi[u]] =
          ltot > 0.0f ? (m_ref[u] + __builtin_amdgcn_logf(ltot)) * 0.6931471805599453f : -INFINITY;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2_t w;
        w[0] = Op::pack(o[u][cb][4 * g + 0] * inv, o[u][cb][4 * g + 1] * inv);
        w[1] = Op::pack(o[u][cb][4 * g + 2] * inv, o[u][cb][4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t*>(&stage[col * kKS + cb * 32 + g * 8 + half * 4]) = w;
      }
    uint16_t* obase = static_cast<uint16_t*>(a.out) + b * a.o_sb + h * a.o_sh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = lane + 64 * i, row = id >> 3, ch = id & 7;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&stage[row * kKS + ch * 8]);
      const int q = qw0 + 32 * u + row;
      if (q < a.Nq) *reinterpret_cast<u32x4_t*>(obase + (int64_t)q * a.o_sn + ch * 8) = v;
    }
  }
}

template <class Op, int NW, int QS>
hipError_t launch(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  constexpr int QB = NW * 32 * QS;
  const int nqb = (a.Nq + QB - 1) / QB;
  const int64_t blocks = (int64_t)nqb * a.H * a.B;
  if (blocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL((attn_mfma_kernel<Op, NW, QS>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, t0,
                        t1, 0, a, nqb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  // Short query blocks (sentence-length sequences) use one wave (32 queries)
  // per workgroup so the grid has many workgroups in flight; long ones use
  // eight waves of 64 queries, so each staged K/V tile serves 512 queries and
  // the tiles are read from L2 half as often as with four waves (measured:
  // 282 vs 297 us on the long causal workload).
  const bool longq = a.Nq > 64;
  if (dt == DType::BF16)
    return longq ? launch<BF16, 8, 2>(a, stream, t0, t1) : launch<BF16, 1, 1>(a, stream, t0, t1);
  return longq ? launch<F16, 8, 2>(a, stream, t0, t1) : launch<F16, 1, 1>(a, stream, t0, t1);
}

}  // namespace mha
