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
// Two kernels, with the same arithmetic step for step (same results bit for
// bit).  attn_mfma_kernel gives a workgroup 512 (or 256) consecutive queries
// of one (b, h): eight (four) waves of 64, each as two sub-blocks of 32 that
// share every K operand read, and every wave sharing each key/value tile
// staged in LDS.  attn_short_kernel gives one wave 32 queries and arranges its
// memory traffic so that it waits for memory once per tile.  The launcher
// picks the workgroup size from how well each would fill the chip
// (attention_block_queries): one-wave workgroups for query blocks of at most
// 64 rows and where the larger ones would leave waves or compute units idle.  In both, per key tile a wave computes the
// TRANSPOSED scores S^T (64 keys x 32 queries) = K_tile * Q^T, so that each
// lane ends up holding 32 scores of one query (lanes l and l+32 share a query
// and split its keys).  That layout is exactly the B operand of the second
// product O^T (64 features x 32 queries) += V^T * P^T, so the probabilities P
// go from the score accumulators to the second MFMA without touching LDS.  V
// stays row-major in LDS and its V^T operands are read with the transposing
// ds_read_b64_tr_b16.
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
// reference, rescale its accumulators and exponentiate the tile again.  With
// bf16 P (the exponent range of fp32) the long kernel first runs the key loop
// without that guard after each query's first tile, and keeps the result when
// every row sum stays at most 2^100 and every accumulator is finite; otherwise
// the workgroup runs the guarded loop.  Row sums come from the packed P values
// with v_dot2, i.e. from exactly the rounded values the P*V product multiplies.
#include <type_traits>

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
  static_assert(NW == 4 || NW == 8, "a tile is eight 1 KiB groups of K and eight of V");
  constexpr int GPW = 8 / NW;  // 1 KiB groups of each tile that one wave moves

  // K and V tiles, double-buffered; after the key loop the same memory stages
  // the output rows (32 rows of kKS elements per wave).
  constexpr int kTiles = 4 * kBN * kD;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kTiles > NW * 32 * kKS ? kTiles : NW * 32 * kKS];
  uint16_t (*ks)[kBN * kD] = reinterpret_cast<uint16_t (*)[kBN * kD]>(lds);
  uint16_t (*vs)[kBN * kD] = reinterpret_cast<uint16_t (*)[kBN * kD]>(lds + 2 * kBN * kD);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: wave-uniform branches
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;

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

  // Tiles go straight from memory into LDS (buffer loads with an LDS
  // destination): wave w moves rows 8w .. 8w+7 of the K tile and of the V
  // tile, one 16-byte chunk per lane, lane l landing at byte 16l of the
  // wave's 1 KiB group.  Both tiles are dense 128-byte rows whose chunks are
  // XOR-swizzled, so lane l fetches the global chunk that belongs in its
  // slot: for K the operand swizzle of the row (conflict-free 16-byte
  // operand reads), for V bit 1 of the row (conflict-free transposing reads).
  // Wave w moves groups w, w + NW, ...: rows 8 NW apart.  NW is even, so the
  // swizzle of a lane's row is the same in every group it moves.
  const int grow = 8 * wave + (lane >> 3), gslot = lane & 7;
  const int koff = (int)((grow * a.k_sn + ((gslot ^ operand_swizzle(grow)) << 3)) * 2);
  const int voff = (int)((grow * a.v_sn + ((gslot ^ (((grow >> 1) & 1) << 2)) << 3)) * 2);
  const int kgrp = (int)(8 * NW * a.k_sn * 2), vgrp = (int)(8 * NW * a.v_sn * 2);
  const int ktile = (int)(kBN * a.k_sn * 2), vtile = (int)(kBN * a.v_sn * 2);
  // Tiles at or past the workgroup's key end fall outside the range check, so
  // the prefetch issued during the last tile reads nothing.
  auto issue_tile = [&](int t, int buf) {
#pragma unroll
    for (int g = 0; g < GPW; ++g) {
      const int grp = wave + NW * g;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, MHA_LDS(&ks[buf][grp * 512]), 16, koff + g * kgrp + t * ktile, 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vsrc, MHA_LDS(&vs[buf][grp * 512]), 16, voff + g * vgrp + t * vtile, 0,
                                               0, 0);
    }
  };
  const int kswz = operand_swizzle(col);  // = operand_swizzle(32jb + col)

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
  // One pass over the key tiles.  FAST (bf16 only): once every query of a
  // sub-block has a reference (its first visible tile), tiles are
  // exponentiated against it with no guard; the pass is checked at the end.
  auto key_pass = [&](auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    bool refd[QS];  // wave-uniform: every query of sub-block u has a reference
#pragma unroll
    for (int u = 0; u < QS; ++u) {
      refd[u] = false;
      m_ref[u] = -INFINITY;
      lsum[u] = 0.0f;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[u][cb][r] = 0.0f;
    }

    issue_tile(0, 0);
    wait_vmcnt<0>();
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      const int j0 = t * kBN;

      if (j0 >= kmax_wave) issue_tile(t + 1, buf ^ 1);
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
            kop[jb][kk] = *reinterpret_cast<const u32x4_t*>(&ks[buf][(jb * 32 + col) * kD + (((2 * kk + half) ^ kswz) << 3)]);
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
        // The next tile's loads go out after this tile's last LDS reads.
        issue_tile(t + 1, buf ^ 1);

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
          // (7.95 vs 8.2 us on the base decoder workload), and so do four-wave
          // workgroups, which serve sequences of a few key tiles.  Eight-wave
          // workgroups (long sequences) keep the branch-free loop (the check
          // cost 3% there).
          // The common path asks only whether any lane's partial sum failed the
          // guard (one compare and a wave vote); which queries must rescale --
          // lanes l and l + 32 hold one query and decide together -- is worked
          // out only on the rare path.  The unguarded pass takes the rare path
          // only until every query of the sub-block has a reference.
          bool ran = false, any_need = true;
          if ((QS > 1 && NW == 8) || !__all(m_ref[u] == -INFINITY)) {
            exponentiate(m_ref[u], false);
            ran = true;
            if constexpr (FAST)
              any_need = !refd[u];
            else
              any_need = __any(!(ls <= Op::kGuard));
          }
          if (any_need) {
            const bool need = ran ? lanes_max(ls <= Op::kGuard ? 0.0f : 1.0f) > 0.0f : true;
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
            if constexpr (FAST) refd[u] = __all(m_ref[u] != -INFINITY);
          }
          lsum[u] += ls;

#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) o[u][cb] = Op::mma(vop[t4][cb], pb[t4], o[u][cb]);
        }
      }

      wait_vmcnt<0>();
      stage_barrier();
    }
  };
  // P in bf16 has the exponent range of fp32, so a tile whose scores rise far
  // above the reference still gives finite weights; the unguarded pass is
  // kept if every partial row sum stays at most 2^100 and every accumulator
  // is finite (the partial sums never decrease, so no intermediate exceeded
  // them either).  Otherwise the whole workgroup redoes the pass with the
  // guard.  fp16 weights overflow at 2^16, so that type always takes the
  // guarded pass.
  constexpr bool kWideP = Op::kGuard > 1.0e6f;
  if constexpr (kWideP) {
    key_pass(std::true_type{});
    bool ok = true;
#pragma unroll
    for (int u = 0; u < QS; ++u) {
      ok = ok && lsum[u] <= 0x1p100f;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ok = ok && fabsf(o[u][cb][r]) <= 3.0e38f;
    }
    if (__syncthreads_or(!ok)) key_pass(std::false_type{});
  } else {
    key_pass(std::false_type{});
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

// One wave per workgroup: 32 queries of one (b, h), for query blocks of at
// most 64 rows (sentence-length self-attention, cross-attention from short
// query sequences) and for longer ones whose 512-query workgroups would be
// poorly used (a few hundred queries, or few heads).  The arithmetic is step for step that of attn_mfma_kernel
// with one 32-query sub-block.  What differs is the memory traffic, which is
// what bounds a wave that is alone on its SIMD for the whole of a short
// launch: it is arranged so that a wave waits for memory once.
//   * The queries and the first tile of keys and values are requested
//     together with the key length, over the keys the wave can see whatever
//     the length is (up to its last query under the causal mask, else all
//     Nk).  Key rows past the length are masked after the products; value
//     rows past the wave's last visible key are zeroed in the registers once
//     the length has arrived, so whatever those rows hold never reaches the
//     output.  Decoding against a cache is the exception: slots past the
//     filled length are never read there, so its loads wait for the length.
//   * K needs no LDS: each lane loads its operands of S^T = K Q^T straight
//     from memory in the MFMA layout (features 16kk + 8half .. +7 of key
//     32jb + col).  V goes through LDS for the transposing operand reads.
//   * Later tiles are requested one tile ahead, bounded by the length.
//   * The output is staged through LDS and leaves as whole 128-byte rows
//     (rows written in 8-byte pieces from the registers take several times
//     longer to complete).
template <class Op, bool kCacheEnd>
__global__ __launch_bounds__(64, 2) void attn_short_kernel(AttnArgs a) {
  // One value tile; after the key loop it stages the output rows.
  __shared__ __attribute__((aligned(16))) uint16_t vs[kBN * kD];
  static_assert(32 * kKS <= kBN * kD, "output staging exceeds the tile memory");
  const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;

  // Longest query blocks first: under the causal mask later blocks see more keys.
  const int nqb = (a.Nq + 31) >> 5;
  const int BH = a.B * a.H;
  const int bh = blockIdx.x % BH;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int b = bh / a.H, h = bh % a.H;
  const int kvh = a.kv_group > 1 ? h / a.kv_group : h;
  const int q0 = qb * 32;
  const int qi = q0 + col;
  const bool qvalid = qi < a.Nq;

  // The key length is requested before anything else, so that it heads the
  // memory queues, as a vector load (range 0 without lengths: no access) so
  // that it is waited for only where it is used.
  const __amdgpu_buffer_rsrc_t lsrc = make_rsrc(a.key_lens, a.key_lens ? (int64_t)a.B * 4 : 0);
  const int lraw = (int)__builtin_amdgcn_raw_buffer_load_b32(lsrc, b * 4, 0, 0);

  const uint16_t* qbase = static_cast<const uint16_t*>(a.q) + b * a.q_sb + h * a.q_sh;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.v_sb + kvh * a.v_sh;

  // This lane's query as the B operand of S^T = K Q^T; a negative scale is
  // folded in by negating q (exact).
  const float c2 = fabsf(a.scale) * kLog2e;
  const __amdgpu_buffer_rsrc_t qsrc = make_rsrc(qbase, ((int64_t)(a.Nq - 1) * a.q_sn + kD) * 2);
  u32x4_t qreg[4];
  {
    const int qoff = qvalid ? (int)(qi * a.q_sn * 2) + half * 16 : kDeadOffset;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qreg[kk] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, qoff + kk * 32, 0, 0);
  }
  // Key and value loads are range-checked: rows at or past the range read
  // as zeros and touch no memory.
  __amdgpu_buffer_rsrc_t ksrc, vsrc;
  auto set_range = [&](int rows) {
    ksrc = make_rsrc(kbase, rows > 0 ? ((int64_t)(rows - 1) * a.k_sn + kD) * 2 : 0);
    vsrc = make_rsrc(vbase, rows > 0 ? ((int64_t)(rows - 1) * a.v_sn + kD) * 2 : 0);
  };
  // Keys 32jb .. 32jb + 31 of tile t, straight into the operand registers.
  auto load_k_block = [&](int t, int jb, u32x4_t (&kb)[4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kb[kk] = __builtin_amdgcn_raw_buffer_load_b128(
          ksrc, (int)(((t * kBN + jb * 32 + col) * a.k_sn + kk * 16 + half * 8) * 2), 0, 0);
  };
  auto load_k = [&](int t, u32x4_t (&kop)[2][4]) {
    load_k_block(t, 0, kop[0]);
    load_k_block(t, 1, kop[1]);
  };
  // V through LDS: each lane moves 8 16-byte chunks of a tile (rows of 128
  // bytes whose chunks are XOR-swizzled by bit 1 of the row, the layout of
  // the transposing reads).  Chunk c of a lane is row lane/8 + 8c, chunk
  // lane%8; the swizzle bit is the same for all eight.
  const int vrow = lane >> 3, vch = lane & 7;
  const int voff = (int)((vrow * a.v_sn + vch * 8) * 2), vstep = (int)(8 * a.v_sn * 2);
  const int vpos = vrow * kD + ((vch ^ (((vrow >> 1) & 1) << 2)) << 3);
  const int vtile = (int)(kBN * a.v_sn * 2);
  u32x4_t vreg[8];
  // Rows 32i .. 32i + 31 of tile t are chunks 4i .. 4i + 3.
  auto load_v_block = [&](int t, int i) {
#pragma unroll
    for (int c = 4 * i; c < 4 * i + 4; ++c)
      vreg[c] = __builtin_amdgcn_raw_buffer_load_b128(vsrc, voff + c * vstep + t * vtile, 0, 0);
  };
  auto load_v = [&](int t) {
    load_v_block(t, 0);
    load_v_block(t, 1);
  };
  auto store_v = [&]() {
#pragma unroll
    for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4_t*>(&vs[vpos + c * 8 * kD]) = vreg[c];
  };

  // The first 32 rows of the first tile are requested before the length is
  // known, up to the last key the wave may see whatever the length is (the
  // key length decides only the rest).  A cache (mask anchored at its
  // filled end) is read only below its length: there everything waits for it.
  const int krows0 = a.causal ? min(a.Nk, min(q0 + 32, a.Nq)) : a.Nk;
  u32x4_t kop[2][4];
  if constexpr (!kCacheEnd) {
    set_range(krows0);
    load_k_block(0, 0, kop[0]);
    load_v_block(0, 0);
  }
  const int L = a.key_lens ? min(max(__builtin_amdgcn_readfirstlane(lraw), 0), a.Nk) : a.Nk;

  const int coff = kCacheEnd ? L - a.Nq : 0;  // causal: query i sees keys j <= i + coff
  const int kend = a.causal ? min(L, qi + 1 + coff) : L;                     // keys this query sees
  const int kend_blk = a.causal ? min(L, min(q0 + 32, a.Nq) + coff) : L;     // keys the wave needs
  const int kmin = a.causal ? min(L, q0 + 1 + coff) : L;                     // tiles below: no mask
  const int ntiles = (max(kend_blk, 0) + kBN - 1) / kBN;
  // From here on, loads stop at the wave's last visible key; a tile past it
  // loads nothing (its rows are all beyond the range) and returns zeros.
  set_range(kend_blk);
  if constexpr (kCacheEnd) {
    load_k_block(0, 0, kop[0]);
    load_v_block(0, 0);
  }
  load_k_block(0, 1, kop[1]);
  load_v_block(0, 1);
  // V^T operands through ds_read_b64_tr_b16 (see attn_mfma_kernel).
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
    lds_s16x4_t* p = (lds_s16x4_t*)(const __attribute__((address_space(3))) uint16_t*)&vs[row * kD + tr_col[cb]];
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
  };

  if (a.scale < 0.0f) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qreg[kk] ^= 0x80008000u;
  }
  // Masked keys give exp2(-inf) = 0 by themselves unless the scale is 0.
  const bool zero_scale = c2 == 0.0f;

  f32x16_t o[2];
  float m_ref = -INFINITY, lsum = 0.0f;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.0f;

  // Per tile: the scores and their softmax while the tile's values are still
  // in flight, then the values through LDS (one buffer: a wave's LDS accesses
  // are carried out in order, so the previous tile's reads come first) and
  // the products with P.
  auto tile = [&](int t, auto prefetch) {
    constexpr bool more = decltype(prefetch)::value;
    const int j0 = t * kBN;

    // S^T = K_tile Q^T: two 32-key blocks.
    f32x16_t s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[jb][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s[jb] = Op::mma(kop[jb][kk], qreg[kk], s[jb]);
    }
    // The next tile's keys land in the operand registers just consumed.
    if constexpr (more) load_k(t + 1, kop);
    // Register (jb, r) holds key j0 + 32jb + 8(r/4) + 4half + r%4; invisible
    // keys -- padding, the future, and whatever the rows past the length hold
    // -- become -inf.
    if (j0 + kBN > kmin) {
      const int lim = kend - j0 - 4 * half;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (jb * 32 + (r >> 2) * 8 + (r & 3) >= lim) s[jb][r] = -INFINITY;
    }

    // Softmax as in attn_mfma_kernel: P = exp2(s * c2 - m_ref) packed in the
    // P^T operand order, row sums from the packed values in four v_dot2
    // chains; the optimistic pass against the reference is skipped while no
    // query of the wave has one (its first tile).
    u32x4_t pb[4];
    float ls = 0.0f;
    auto exponentiate = [&](float mu, bool select_masked) {
      float lp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int jb = t4 >> 1, r = (t4 & 1) * 8 + 2 * w;
          float p0 = __builtin_amdgcn_exp2f(fmaf(s[jb][r], c2, -mu));
          float p1 = __builtin_amdgcn_exp2f(fmaf(s[jb][r + 1], c2, -mu));
          if (select_masked) {
            p0 = s[jb][r] == -INFINITY ? 0.0f : p0;
            p1 = s[jb][r + 1] == -INFINITY ? 0.0f : p1;
          }
          pb[t4][w] = Op::pack(p0, p1);
          lp[w] = Op::sum2(pb[t4][w], lp[w]);
        }
      ls = (lp[0] + lp[1]) + (lp[2] + lp[3]);
    };
    bool ran = false, any_need = true;  // as in attn_mfma_kernel
    if (!__all(m_ref == -INFINITY)) {
      exponentiate(m_ref, false);
      ran = true;
      any_need = __any(!(ls <= Op::kGuard));
    }
    if (any_need) {
      const bool need = ran ? lanes_max(ls <= Op::kGuard ? 0.0f : 1.0f) > 0.0f : true;
      float mx = -INFINITY;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
      mx = lanes_max(mx);
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c2;
      const float m_new = need ? fmaxf(m_ref, mt) : m_ref;
      const float alpha = (need && m_new != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.0f;
      lsum *= alpha;
      // Before the first tile the accumulators hold nothing to rescale.
      if (t > 0) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
      }
      m_ref = m_new;
      const float mu = m_ref == -INFINITY ? 0.0f : m_ref;
      if (zero_scale)
        exponentiate(mu, true);
      else
        exponentiate(mu, false);
    }
    lsum += ls;

    // Value rows of the first tile that were requested before the length was
    // known and lie past the wave's last visible key become zeros.
    if (!kCacheEnd && t == 0 && kend_blk < min(krows0, 32)) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (vrow + 8 * c >= kend_blk) vreg[c] = u32x4_t{0u, 0u, 0u, 0u};
    }
    store_v();
    if constexpr (more) load_v(t + 1);
    // V^T operands of the tile: step t4 supplies keys 16t4 + 4half + {0..3}
    // and 16t4 + 8 + 4half + {0..3} of this lane's feature row.
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      u32x4_t vop[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const u32x2_t lo = vread(16 * t4 + tr_row, cb);
        const u32x2_t hi = vread(16 * t4 + 8 + tr_row, cb);
        vop[cb] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) o[cb] = Op::mma(vop[cb], pb[t4], o[cb]);
    }
  };
  // The steady state prefetches unconditionally and the last tile not at all,
  // so that every path into a tile has the same loads in flight (the
  // compiler's memory-wait counts are taken over all paths).
  for (int t = 0; t + 1 < ntiles; ++t) tile(t, std::true_type{});
  if (ntiles > 0) tile(ntiles - 1, std::false_type{});

  // Register (cb, 4g + e) of this lane is feature 32cb + 8g + 4half + e of
  // query qi; the rows are staged in the value tile memory (its last reads
  // come first in LDS order) and copied out 16 bytes per lane.
  const float ltot = lanes_sum(lsum);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (a.lse && half == 0 && qvalid)
    a.lse[((int64_t)b * a.H + h) * a.Nq + qi] =
        ltot > 0.0f ? (m_ref + __builtin_amdgcn_logf(ltot)) * 0.6931471805599453f : -INFINITY;
  uint16_t* stage = vs;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2_t w;
      w[0] = Op::pack(o[cb][4 * g + 0] * inv, o[cb][4 * g + 1] * inv);
      w[1] = Op::pack(o[cb][4 * g + 2] * inv, o[cb][4 * g + 3] * inv);
      *reinterpret_cast<u32x2_t*>(&stage[col * kKS + cb * 32 + g * 8 + half * 4]) = w;
    }
  __builtin_amdgcn_wave_barrier();
  // Range-checked stores: rows past the last query get an offset beyond the
  // range and are dropped, with no branch around the LDS reads.
  uint16_t* obase = static_cast<uint16_t*>(a.out) + b * a.o_sb + h * a.o_sh;
  const __amdgpu_buffer_rsrc_t osrc = make_rsrc(obase, ((int64_t)(a.Nq - 1) * a.o_sn + kD) * 2);
  u32x4_t ov[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = lane + 64 * i, row = id >> 3, ch = id & 7;
    ov[i] = *reinterpret_cast<const u32x4_t*>(&stage[row * kKS + ch * 8]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = lane + 64 * i, row = id >> 3, ch = id & 7;
    const int q = q0 + row;
    const int off = q < a.Nq ? (int)(q * a.o_sn * 2) + ch * 16 : kDeadOffset;
    __builtin_amdgcn_raw_buffer_store_b128(ov[i], osrc, off, 0, 0);
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

template <class Op>
hipError_t launch_short(const AttnArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const int nqb = (a.Nq + 31) / 32;
  const int64_t blocks = (int64_t)nqb * a.H * a.B;
  if (blocks == 0) return hipSuccess;
  if (a.causal_end)
    hipExtLaunchKernelGGL((attn_short_kernel<Op, true>), dim3((unsigned)blocks), dim3(64), 0, stream, t0, t1, 0, a);
  else
    hipExtLaunchKernelGGL((attn_short_kernel<Op, false>), dim3((unsigned)blocks), dim3(64), 0, stream, t0, t1, 0, a);
  return hipGetLastError();
}

// Workgroups of qb queries: 32 (one wave), or 256 / 512 (four or eight waves
// of 64 queries sharing each staged K/V tile).
template <class Op>
hipError_t launch_sized(const AttnArgs& a, int qb, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  switch (qb) {
    case 512: return launch<Op, 8, 2>(a, stream, t0, t1);
    case 256: return launch<Op, 4, 2>(a, stream, t0, t1);
    default: return launch_short<Op>(a, stream, t0, t1);
  }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs& a, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const int qb = attention_block_queries(a.B, a.H, a.Nq, a.causal);
  if (dt == DType::BF16)
    return launch_sized<BF16>(a, qb, stream, t0, t1);
  return launch_sized<F16>(a, qb, stream, t0, t1);
}

}  // namespace mha
