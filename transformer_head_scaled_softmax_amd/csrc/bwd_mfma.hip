// bwd_mfma.hip -- gradients of bf16 / fp16 scaled dot-product attention, head
// size 64, on the gfx950 matrix cores (v_mfma_f32_32x32x16_{bf16,f16}).
//
// The pages' use of the path is teacher-forced training, where one forward
// pass covers the whole sequence and gradients flow back through it
// ("Training (Teacher Forcing + Masking)", trishampatil.com; "One forward pass
// covers the whole sequence", alexdo.xyz).  They give no gradient formulas;
// these are the exact derivatives of the forward definition
// softmax(scale * Q K^T) V with masked keys at weight 0, for output gradient
// dO:
//
//   P_ij  = exp(scale q_i.k_j - lse_i)  (visible keys; 0 otherwise)
//   dV_j  = sum_i P_ij dO_i             dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i),         D_i = dO_i . out_i
//   dQ_i  = scale sum_j dS_ij k_j       dK_j = scale sum_i dS_ij q_i
//
// lse_i is the forward pass's row statistic (natural log of the softmax
// denominator), so P is recomputed tile by tile and never stored.
//
// Two kernels, no atomics.  bwd_dq_kernel owns a block of queries and
// streams the keys (three products per tile: S^T, dP^T, dQ^T); it also forms
// D_i for its rows and leaves them in a workspace.  bwd_dkdv_kernel owns a
// block of keys and streams the queries (four products: S, dP, dV^T, dK^T).
// With key/value heads shared by G query heads ("Limitations of the Original
// Design", trishampatil.com) a dK/dV workgroup streams the queries of a run of
// G / parts query heads one head after the other, so a shared head's gradient
// sums in its accumulators; with more than one run the runs' fp32 sums go to
// the workspace and bwd_combine_kernel adds them in order.
// The products are arranged so that the score-shaped accumulators (S, dP)
// feed the next MFMA as its B operand straight from registers: a 32x32
// accumulator holds, in lane n + 32*half, rows 16t + 8(e/4) + 4half + e%4
// (t = 0, 1; e = 0..7) of column n, and those eight values are the B operand
// of one 16-deep MFMA step when the A operand is read with the same row order
// -- which the transposing LDS read ds_read_b64_tr_b16 delivers.
//
// MFMA 32x32x16 lane layout (checked on the device): A[m][k] comes from lane
// m + 32*(k/8), element k%8; B[k][n] from lane n + 32*(k/8), element k%8;
// C[m][n] lands in lane n + 32*((m/4)%2), register 4*(m/8) + m%4.
#include <type_traits>

#include "mfma_util.h"

namespace mha {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = kMfmaHeadDim;  // 64
constexpr int kBT = 64;           // rows per streamed LDS tile
constexpr int kSS = 72;           // row stride (elements) of the epilogue staging
constexpr int kDead = (int)0x80000000u;  // beyond any range check: loads return zeros

// Tiles in LDS are dense 128-byte rows whose 16-byte chunks are permuted per
// row: chunk c of row r sits in slot c ^ dual_swizzle(r).  The permutation
// keeps both access patterns conflict-free: row operands (16 bytes per lane
// from 16 consecutive rows: the slots of rows of one parity are all distinct)
// and the transposing reads (8 bytes per lane from 4 consecutive rows and 4
// adjacent chunks: rows 4a, 4a+1 and 4a+2, 4a+3 use chunk sets that differ in
// bit 2).
__device__ inline int dual_swizzle(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

__device__ inline u32x4_t row_read(const uint16_t* tile, int row, int chunk) {
  return *reinterpret_cast<const u32x4_t*>(&tile[row * kD + ((chunk ^ dual_swizzle(row)) << 3)]);
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4k + q supplies the
// address of row (r0 + k), features (c0 + 4q .. +3); lane l of the group then
// receives feature c0 + l of rows r0 .. r0+3.
__device__ inline u32x2_t tr_read(const uint16_t* p) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  lds_s16x4_t* lp = (lds_s16x4_t*)(const __attribute__((address_space(3))) uint16_t*)p;
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
}

// Per-lane offsets of the transposed A operand A[m = feature][k = tile row]
// for 16-row step t of a 32-row sub-block: rows 16t + 4half + {0..3} (first
// half of the operand) and 16t + 8 + 4half + {0..3} (second half), features
// 32cb + (lane & 31).  Offsets are relative to row 16t of the sub-block (the
// swizzle does not depend on t).
struct TrOffsets {
  int off[2][2];  // [lo/hi][cb]
  __device__ TrOffsets(int lane) {
    const int half = lane >> 5, k = (lane & 15) >> 2, q = lane & 3, cg = (lane >> 4) & 1;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 8 * hi + 4 * half + k;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int c = cb * 32 + 16 * cg + 4 * q;
        off[hi][cb] = row * kD + (((c >> 3) ^ dual_swizzle(row)) << 3) + (c & 7);
      }
    }
  }
};

__device__ inline u32x4_t tr_operand(const uint16_t* tile, const TrOffsets& o, int row16, int cb) {
  const u32x2_t lo = tr_read(tile + row16 * kD + o.off[0][cb]);
  const u32x2_t hi = tr_read(tile + row16 * kD + o.off[1][cb]);
  return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// Tile memory of a workgroup of NW waves: two 64-row tiles of each streamed
// operand, or the epilogue's staging rows if that is more.
template <int NW>
constexpr int kLdsElems = 4 * kBT * kD > NW * 32 * kSS ? 4 * kBT * kD : NW * 32 * kSS;

// lse in natural-log units -> the exp2 argument offset; a row with no
// visible key (lse = -inf) gets +inf so every weight of it is 0.
__device__ inline float lse_to_log2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// Stores a 64-feature x 32-row accumulator pair (register (cb, 4g + e) of lane
// (col, half) = feature 32cb + 8g + 4half + e of row col) times `mul` as
// 32 rows of the output, through this wave's staging area, 16 bytes per lane.
template <class Op>
__device__ inline void store_rows(const f32x16_t (&acc)[2], float mul, uint16_t* stage, uint16_t* out,
                                  int row0, int nrows, int lane) {
  const int half = lane >> 5, col = lane & 31;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2_t w;
      w[0] = Op::pack(acc[cb][4 * g + 0] * mul, acc[cb][4 * g + 1] * mul);
      w[1] = Op::pack(acc[cb][4 * g + 2] * mul, acc[cb][4 * g + 3] * mul);
      *reinterpret_cast<u32x2_t*>(&stage[col * kSS + cb * 32 + g * 8 + half * 4]) = w;
    }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = lane + 64 * i, row = id >> 3, ch = id & 7;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(&stage[row * kSS + ch * 8]);
    if (row0 + row < nrows) *reinterpret_cast<u32x4_t*>(out + (int64_t)(row0 + row) * kD + ch * 8) = v;
  }
}

// ---------------------------------------------------------------------------
// dQ: a workgroup owns 32*NW queries of one (b, h), one wave per 32 queries.
// Per 64-key tile a wave computes S^T = K Q^T and dP^T = V dO^T (keys x
// queries, so each lane holds one query's scores), P^T and dS^T, then
// dQ^T += K^T dS^T with K^T read transposed from the same LDS tile.
template <class Op, int NW, bool FUSED>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& a, int nqb, int block, float* dsh) {
  constexpr int NT = NW * 64;
  constexpr int QB = NW * 32;
  constexpr int CH = (kBT * 8) / NT;  // 16-byte chunks of K (and of V) per thread per tile
  static_assert(CH >= 1, "tile too small for the workgroup");
  // K, V double-buffered; afterwards the epilogue staging (32 x kSS per wave).
  __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems<NW>];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int BH = a.B * a.H;
  const int bh = block % BH;
  const int qb = nqb - 1 - (int)(block / BH);  // longest first under the causal mask
  const int b = bh / a.H;

  int L = a.Nk;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), a.Nk);
  const int q0 = qb * QB, qw0 = q0 + wave * 32;
  const int qi = qw0 + col;
  const bool qvalid = qi < a.Nq;
  const int kend = a.causal ? min(L, qi + 1) : L;  // keys this lane's query sees
  const int kend_blk = a.causal ? min(L, min(q0 + QB, a.Nq)) : L;
  const int kmin_wave = a.causal ? min(L, qw0 + 1) : L;               // tiles below: no masking
  const int kmax_wave = a.causal ? min(L, min(qw0 + 32, a.Nq)) : L;   // tiles from here: skip
  const int ntiles = (max(kend_blk, 0) + kBT - 1) / kBT;

  const int kvh = (bh % a.H) / (a.H / a.Hkv);  // key/value head read by this query head
  const int64_t qhead = (int64_t)bh * a.Nq * kD, khead = ((int64_t)b * a.Hkv + kvh) * a.Nk * kD;
  const __amdgpu_buffer_rsrc_t qsrc = make_rsrc(static_cast<const uint16_t*>(a.q) + qhead, (int64_t)a.Nq * kD * 2);
  const __amdgpu_buffer_rsrc_t dosrc =
      make_rsrc(static_cast<const uint16_t*>(a.dout) + qhead, (int64_t)a.Nq * kD * 2);
  const __amdgpu_buffer_rsrc_t osrc = make_rsrc(static_cast<const uint16_t*>(a.out) + qhead, (int64_t)a.Nq * kD * 2);
  const int64_t kvbytes = (int64_t)max(kend_blk, 0) * kD * 2;
  const __amdgpu_buffer_rsrc_t ksrc = make_rsrc(static_cast<const uint16_t*>(a.k) + khead, kvbytes);
  const __amdgpu_buffer_rsrc_t vsrc = make_rsrc(static_cast<const uint16_t*>(a.v) + khead, kvbytes);

  // This lane's query as B operands (features 16kk + 8half .. +7) of
  // S^T = K Q^T and dP^T = V dO^T; out only for D.
  const int qoff = qvalid ? qi * (kD * 2) + half * 16 : kDead;
  u32x4_t qreg[4], doreg[4];
  float dpart = 0.0f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qreg[kk] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, qoff + kk * 32, 0, 0);
    doreg[kk] = __builtin_amdgcn_raw_buffer_load_b128(dosrc, qoff + kk * 32, 0, 0);
    const u32x4_t ov = __builtin_amdgcn_raw_buffer_load_b128(osrc, qoff + kk * 32, 0, 0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dpart = fmaf(Op::to_float(doreg[kk][w] & 0xffff), Op::to_float(ov[w] & 0xffff), dpart);
      dpart = fmaf(Op::to_float(doreg[kk][w] >> 16), Op::to_float(ov[w] >> 16), dpart);
    }
  }
  const float Dq = lanes_sum(dpart);  // D_i = dO_i . out_i (both lane halves)
  float lse2 = INFINITY;
  if (qvalid) {
    lse2 = lse_to_log2(a.lse[(int64_t)bh * a.Nq + qi]);
    if (half == 0) {
      if (FUSED)
        dsh[qi - q0] = Dq;  // for the dK/dV part of the same workgroup
      else
        a.dsum[(int64_t)bh * a.Nq + qi] = Dq;
    }
  }
  const float c2 = a.scale * kLog2e;

  uint16_t* const kbuf0 = lds;
  uint16_t* const vbuf0 = lds + 2 * kBT * kD;
  int goff[CH], spos[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = tid + c * NT, row = idx >> 3, ch = idx & 7;
    goff[c] = (row * kD + ch * 8) * 2;
    spos[c] = row * kD + ((ch ^ dual_swizzle(row)) << 3);
  }
  u32x4_t kreg[CH], vreg[CH];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      kreg[c] = __builtin_amdgcn_raw_buffer_load_b128(ksrc, goff[c] + t * (kBT * kD * 2), 0, 0);
      vreg[c] = __builtin_amdgcn_raw_buffer_load_b128(vsrc, goff[c] + t * (kBT * kD * 2), 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      *reinterpret_cast<u32x4_t*>(&kbuf0[buf * kBT * kD + spos[c]]) = kreg[c];
      *reinterpret_cast<u32x4_t*>(&vbuf0[buf * kBT * kD + spos[c]]) = vreg[c];
    }
  };
  const TrOffsets tro(lane);

  f32x16_t dq[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[cb][r] = 0.0f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * kBT;
    const uint16_t* ks = kbuf0 + buf * kBT * kD;
    const uint16_t* vs = vbuf0 + buf * kBT * kD;
    load_tile(t + 1);

    // One tile.  MASK: some key of the tile is invisible to some query of the
    // wave (diagonal or padded tail); the other tiles take the branch without
    // the per-element selects.
    auto tile = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // S^T and dP^T - D, two 32-key blocks: register (jb, r) of this lane is
      // key j0 + 32jb + 8(r/4) + 4half + r%4 of query qi.  The dP^T
      // accumulators start at -D, so they end as dP - D.
      f32x16_t s[2], dp[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[jb][r] = 0.0f;
          dp[jb][r] = -Dq;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          s[jb] = Op::mma(row_read(ks, jb * 32 + col, 2 * kk + half), qreg[kk], s[jb]);
          dp[jb] = Op::mma(row_read(vs, jb * 32 + col, 2 * kk + half), doreg[kk], dp[jb]);
        }
      }
      const int lim = kend - j0 - 4 * half;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        u32x4_t dsb;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int jb = t4 >> 1, r = (t4 & 1) * 8 + 2 * w;
          float p0 = __builtin_amdgcn_exp2f(fmaf(s[jb][r], c2, -lse2));
          float p1 = __builtin_amdgcn_exp2f(fmaf(s[jb][r + 1], c2, -lse2));
          if (MASK) {
            const int kr = jb * 32 + (r >> 2) * 8 + (r & 3);
            p0 = kr >= lim ? 0.0f : p0;
            p1 = kr + 1 >= lim ? 0.0f : p1;
          }
          dsb[w] = Op::pack(p0 * dp[jb][r], p1 * dp[jb][r + 1]);
        }
        // dQ^T += K^T dS^T for keys 16t4 .. +15, K^T read transposed.
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) dq[cb] = Op::mma(tr_operand(ks, tro, 16 * t4, cb), dsb, dq[cb]);
      }
    };
    if (j0 < kmax_wave) {  // wave-uniform
      if (j0 + kBT > kmin_wave)
        tile(std::true_type{});
      else
        tile(std::false_type{});
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // dQ = scale * (dQ^T)^T; rows past Nq are not written.
  uint16_t* stage = lds + wave * 32 * kSS;
  store_rows<Op>(dq, a.scale, stage, static_cast<uint16_t*>(a.dq) + qhead, qw0, a.Nq, lane);
}

template <class Op, int NW>
__global__ __launch_bounds__(NW * 64, NW >= 8 ? 1 : 2) void bwd_dq_kernel(BwdArgs a, int nqb) {
  bwd_dq_body<Op, NW, false>(a, nqb, blockIdx.x, nullptr);
}

// ---------------------------------------------------------------------------
// dK, dV: a workgroup owns 32*NW keys of one (b, key/value head), one wave
// per 32 keys, for one run of query heads.
// Query tiles of 64 (Q, dO, lse, D) stream through LDS; per 32-query
// sub-block a wave computes S = Q K^T and dP = dO V^T (queries x keys, so each
// lane holds one key's column), P and dS, then dV^T += dO^T P and
// dK^T += Q^T dS with dO^T and Q^T read transposed from the same tiles.
template <class Op, int NW, bool FUSED>
__device__ __forceinline__ void bwd_dkdv_body(const BwdArgs& a, int nkb, int block, const float* dsh) {
  constexpr int NT = NW * 64;
  constexpr int KB = NW * 32;
  constexpr int CH = (kBT * 8) / NT;  // 16-byte chunks of Q (and of dO) per thread per tile
  static_assert(CH >= 1 && NT >= 2 * kBT, "tile too small for the workgroup");
  // Q, dO double-buffered; afterwards the epilogue staging (32 x kSS per wave).
  __shared__ __attribute__((aligned(16))) uint16_t lds[kLdsElems<NW>];
  __shared__ __attribute__((aligned(16))) float rowstat[2][2][kBT];   // [buf][lse2 | D][row]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  // One (b, key/value head, run of query heads, key block); the GP query heads
  // of the run, which share the key/value head, are streamed one after the
  // other.
  const int BHkv = a.B * a.Hkv, G = a.H / a.Hkv, GP = G / a.parts;
  const int unit = block % (BHkv * a.parts);
  const int kb = (int)(block / (BHkv * a.parts));  // low key blocks first: under the causal mask they see most queries
  const int bkv = unit % BHkv, run = unit / BHkv;
  const int b = bkv / a.Hkv, kvh = bkv % a.Hkv;

  int L = a.Nk;
  if (a.key_lens) L = min(max(a.key_lens[b], 0), a.Nk);
  const int k0 = kb * KB, kw0 = k0 + wave * 32;
  const int kj = kw0 + col;  // this lane's key
  // Query tiles that see a key of this workgroup: all, or under the causal
  // mask those from the tile holding query k0; none if every key is padding.
  const int tfirst = a.causal ? k0 / kBT : 0;
  const int ntiles_q = (a.Nq + kBT - 1) / kBT;
  const int nt = k0 < L ? ntiles_q - tfirst : 0;  // tiles per query head
  const int iend = nt * GP;                         // iteration it: head it / nt of the run, tile tfirst + it % nt
  const bool wave_live = kw0 < L;
  const bool pad_mask = kw0 + 32 > L;  // some key of this wave is padding

  // Per-head sources of the streamed side (query head kvh*G + run*GP + j of batch b).
  const int64_t khead = ((int64_t)b * a.Hkv + kvh) * a.Nk * kD;
  auto head_of = [&](int it) { return (int64_t)b * a.H + kvh * G + run * GP + (nt > 0 ? it / nt : 0); };
  auto qsrc_of = [&](const void* base, int64_t bhq) {
    return make_rsrc(static_cast<const uint16_t*>(base) + bhq * a.Nq * kD, (int64_t)a.Nq * kD * 2);
  };
  auto ssrc_of = [&](const float* base, int64_t bhq) { return make_rsrc(base + bhq * a.Nq, (int64_t)a.Nq * 4); };
  const int64_t kvbytes = (int64_t)L * kD * 2;
  const __amdgpu_buffer_rsrc_t ksrc = make_rsrc(static_cast<const uint16_t*>(a.k) + khead, kvbytes);
  const __amdgpu_buffer_rsrc_t vsrc = make_rsrc(static_cast<const uint16_t*>(a.v) + khead, kvbytes);

  // This lane's key as B operands (features 16kk + 8half .. +7) of S = Q K^T
  // and dP = dO V^T; keys at or past L read as zeros.
  const int koff = kj < L ? kj * (kD * 2) + half * 16 : kDead;
  u32x4_t kreg[4], vreg[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    kreg[kk] = __builtin_amdgcn_raw_buffer_load_b128(ksrc, koff + kk * 32, 0, 0);
    vreg[kk] = __builtin_amdgcn_raw_buffer_load_b128(vsrc, koff + kk * 32, 0, 0);
  }
  const float c2 = a.scale * kLog2e;

  uint16_t* const qbuf0 = lds;
  uint16_t* const obuf0 = lds + 2 * kBT * kD;
  int goff[CH], spos[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = tid + c * NT, row = idx >> 3, ch = idx & 7;
    goff[c] = (row * kD + ch * 8) * 2;
    spos[c] = row * kD + ((ch ^ dual_swizzle(row)) << 3);
  }
  // Wave 0 stages lse (as the exp2 offset), wave 1 D (wave-uniform, so the
  // buffer resource stays scalar).
  const int srow = tid & (kBT - 1), skind = __builtin_amdgcn_readfirstlane(wave);
  u32x4_t qreg[CH], oreg[CH];
  float sreg = 0.0f;
  // Iteration it: query head head_of(it), tile tfirst + it % nt; iterations
  // past the end read nothing (their head's range check ends at Nq rows).
  auto load_tile = [&](int it) {
    const int64_t bhq = head_of(it < iend ? it : iend - 1);
    const int t = it < iend ? tfirst + it % nt : ntiles_q;
    const __amdgpu_buffer_rsrc_t qsrc = qsrc_of(a.q, bhq), dosrc = qsrc_of(a.dout, bhq);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      qreg[c] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, goff[c] + t * (kBT * kD * 2), 0, 0);
      oreg[c] = __builtin_amdgcn_raw_buffer_load_b128(dosrc, goff[c] + t * (kBT * kD * 2), 0, 0);
    }
    if (FUSED && skind == 1)
      sreg = t * kBT + srow < a.Nq ? dsh[t * kBT + srow] : 0.0f;  // D from this workgroup's dQ part
    else if (skind < 2)
      sreg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           skind ? ssrc_of(a.dsum, bhq) : ssrc_of(a.lse, bhq), (t * kBT + srow) * 4, 0, 0));
  };
  auto store_tile = [&](int t, int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      *reinterpret_cast<u32x4_t*>(&qbuf0[buf * kBT * kD + spos[c]]) = qreg[c];
      *reinterpret_cast<u32x4_t*>(&obuf0[buf * kBT * kD + spos[c]]) = oreg[c];
    }
    if (skind == 0) rowstat[buf][0][srow] = t * kBT + srow < a.Nq ? lse_to_log2(sreg) : INFINITY;
    if (skind == 1) rowstat[buf][1][srow] = sreg;  // 0 past Nq
  };
  const TrOffsets tro(lane);

  f32x16_t dv[2], dk[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv[cb][r] = 0.0f;
      dk[cb][r] = 0.0f;
    }

  if (iend > 0) {
    load_tile(0);
    store_tile(tfirst, 0);
  }
  __syncthreads();

  for (int it = 0; it < iend; ++it) {
    const int t = tfirst + it % nt;
    const int buf = it & 1;
    const uint16_t* qs = qbuf0 + buf * kBT * kD;
    const uint16_t* os = obuf0 + buf * kBT * kD;
    load_tile(it + 1);

    // One tile of 64 queries as two 32-query sub-blocks.  MASK: some pair of
    // the tile is invisible (padded keys of this wave, or queries before its
    // last key under the causal mask); other tiles skip the per-element selects.
    auto tile = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int i0 = t * kBT + sb * 32, rb = sb * 32;
        // Register r of this lane is query i0 + 8(r/4) + 4half + r%4: its exp2
        // offset, and -D as the start of the dP accumulator (which then ends
        // as dP - D).
        f32x16_t s, dp;
        float lv[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 l4 = *reinterpret_cast<const float4*>(&rowstat[buf][0][rb + 8 * g + 4 * half]);
          const float4 d4 = *reinterpret_cast<const float4*>(&rowstat[buf][1][rb + 8 * g + 4 * half]);
          lv[4 * g + 0] = l4.x;
          lv[4 * g + 1] = l4.y;
          lv[4 * g + 2] = l4.z;
          lv[4 * g + 3] = l4.w;
          dp[4 * g + 0] = -d4.x;
          dp[4 * g + 1] = -d4.y;
          dp[4 * g + 2] = -d4.z;
          dp[4 * g + 3] = -d4.w;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.0f;
        // S = Q K^T and dP = dO V^T (queries x keys).
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          s = Op::mma(row_read(qs, rb + col, 2 * kk + half), kreg[kk], s);
          dp = Op::mma(row_read(os, rb + col, 2 * kk + half), vreg[kk], dp);
        }
        u32x4_t pb[2], dsb[2];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -lv[r]));
          float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], c2, -lv[r + 1]));
          if (MASK) {
            const int i = i0 + 8 * (r >> 2) + 4 * half + (r & 3);
            p0 = (kj < L && (!a.causal || kj <= i)) ? p0 : 0.0f;
            p1 = (kj < L && (!a.causal || kj <= i + 1)) ? p1 : 0.0f;
          }
          // Registers 8st .. 8st+7 form the B operand of step st.
          pb[r >> 3][(r & 7) >> 1] = Op::pack(p0, p1);
          dsb[r >> 3][(r & 7) >> 1] = Op::pack(p0 * dp[r], p1 * dp[r + 1]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS, the transposed operands read
        // from the same tiles.
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            dv[cb] = Op::mma(tr_operand(os, tro, rb + 16 * st, cb), pb[st], dv[cb]);
            dk[cb] = Op::mma(tr_operand(qs, tro, rb + 16 * st, cb), dsb[st], dk[cb]);
          }
      }
    };
    // Wave-uniform: skip tiles entirely before the wave's first key (causal).
    const int t0q = t * kBT;
    if (wave_live && (!a.causal || t0q + kBT > kw0)) {
      if (pad_mask || (a.causal && t0q < kw0 + 31))
        tile(std::true_type{});
      else
        tile(std::false_type{});
    }

    if (it + 1 < iend) store_tile(tfirst + (it + 1) % nt, buf ^ 1);
    __syncthreads();
  }

  if (a.parts > 1) {
    // This run's fp32 sums, rows [key][64] (dK unscaled); 16 bytes per lane:
    // registers 4g .. 4g+3 of block cb are features cb*32 + 8g + 4*half + 0..3.
    const int64_t per = (int64_t)BHkv * a.Nk * kD;  // elements of one run of one tensor
    float* pk = a.part + ((int64_t)run * BHkv + bkv) * a.Nk * kD + (int64_t)kj * kD + 4 * half;
    float* pv = pk + (int64_t)a.parts * per;
    if (kj < a.Nk) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t wk, wv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            wk[e] = dk[cb][4 * g + e];
            wv[e] = dv[cb][4 * g + e];
          }
          *reinterpret_cast<f32x4_t*>(pk + cb * 32 + 8 * g) = wk;
          *reinterpret_cast<f32x4_t*>(pv + cb * 32 + 8 * g) = wv;
        }
    }
    return;
  }

  // dV = (dV^T)^T, dK = scale * (dK^T)^T; padded keys get zeros, rows past Nk
  // are not written.
  uint16_t* stage = lds + wave * 32 * kSS;
  store_rows<Op>(dv, 1.0f, stage, static_cast<uint16_t*>(a.dv) + khead, kw0, a.Nk, lane);
  __builtin_amdgcn_wave_barrier();
  store_rows<Op>(dk, a.scale, stage, static_cast<uint16_t*>(a.dk) + khead, kw0, a.Nk, lane);
}

template <class Op, int NW>
__global__ __launch_bounds__(NW * 64, NW >= 8 ? 1 : 2) void bwd_dkdv_kernel(BwdArgs a, int nkb) {
  bwd_dkdv_body<Op, NW, false>(a, nkb, blockIdx.x, nullptr);
}

// Sentence-length problems (at most 64 queries and 64 keys per head, one
// key/value head per query head): both parts in one launch, one workgroup per
// (b, h) -- the dQ part, then, after a barrier, the dK/dV part, which takes D
// from LDS (written by the dQ part of the same workgroup) rather than from the
// workspace.  Same arithmetic as the two kernels, one launch fewer.
template <class Op>
__global__ __launch_bounds__(128, 2) void bwd_short_kernel(BwdArgs a) {
  __shared__ float dsh[kBT];
  bwd_dq_body<Op, 2, true>(a, 1, blockIdx.x, dsh);
  __syncthreads();
  bwd_dkdv_body<Op, 2, true>(a, 1, blockIdx.x, dsh);
}

// dK, dV of shared key/value heads from the runs' fp32 sums: element by
// element, runs added in order (deterministic), dK scaled, rounded once.  One
// thread per 8 features of a row of dK or dV.
template <class Op>
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdArgs a, int64_t chunks) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= 2 * chunks) return;
  const int t = id >= chunks;  // 0: dK, 1: dV
  const int64_t c = id - t * chunks;
  const int64_t per = chunks * 8;  // elements of one run of one tensor
  const float* src = a.part + (int64_t)t * a.parts * per + c * 8;
  f32x4_t s0 = *reinterpret_cast<const f32x4_t*>(src);
  f32x4_t s1 = *reinterpret_cast<const f32x4_t*>(src + 4);
  for (int p = 1; p < a.parts; ++p) {
    s0 += *reinterpret_cast<const f32x4_t*>(src + p * per);
    s1 += *reinterpret_cast<const f32x4_t*>(src + p * per + 4);
  }
  const float mul = t ? 1.0f : a.scale;
  u32x4_t w;
  w[0] = Op::pack(s0[0] * mul, s0[1] * mul);
  w[1] = Op::pack(s0[2] * mul, s0[3] * mul);
  w[2] = Op::pack(s1[0] * mul, s1[1] * mul);
  w[3] = Op::pack(s1[2] * mul, s1[3] * mul);
  *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(t ? a.dv : a.dk) + c * 8) = w;
}

template <class Op, int NW>
hipError_t launch_dq(const BwdArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const int nqb = (a.Nq + NW * 32 - 1) / (NW * 32);
  const int64_t blocks = (int64_t)nqb * a.B * a.H;
  if (blocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL((bwd_dq_kernel<Op, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, t0, t1, 0, a,
                        nqb);
  return hipGetLastError();
}

// The dK/dV kernel and, for split head groups, the combining kernel; t0 and t1
// span both.
template <class Op, int NW>
hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  static_assert(NW * 32 == 128 || NW * 32 == 64, "key block size");
  const int nkb = (a.Nk + NW * 32 - 1) / (NW * 32);
  const int64_t blocks = (int64_t)nkb * a.B * a.Hkv * a.parts;
  if (blocks == 0) return hipSuccess;
  const bool split = a.parts > 1;
  hipExtLaunchKernelGGL((bwd_dkdv_kernel<Op, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, t0,
                        split ? nullptr : t1, 0, a, nkb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  const int64_t chunks = (int64_t)a.B * a.Hkv * a.Nk * (kD / 8);
  hipExtLaunchKernelGGL(bwd_combine_kernel<Op>, dim3((unsigned)((2 * chunks + 255) / 256)), dim3(256), 0, stream,
                        nullptr, t1, 0, a, chunks);
  return hipGetLastError();
}

template <class Op>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream, hipEvent_t const* ev) {
  auto evt = [&](int i) -> hipEvent_t { return ev ? ev[i] : nullptr; };
  if (bwd_single_launch(a.H, a.Hkv, a.Nq, a.Nk)) {
    const int64_t blocks = (int64_t)a.B * a.H;
    if (blocks == 0) return hipSuccess;
    hipExtLaunchKernelGGL(bwd_short_kernel<Op>, dim3((unsigned)blocks), dim3(128), 0, stream, evt(0), evt(1), 0, a);
    return hipGetLastError();
  }
  // The dQ kernel writes D, which the dK/dV kernel reads: stream order.
  // dQ workgroups: two waves (64 queries) for at most 64 queries; eight (256
  // queries share each K/V tile) from 4096 queries when that still gives at
  // least 512 workgroups (two rounds of the chip); four (128) otherwise.
  // Measured on one MI355X, whole backward pass, causal, bf16 (same results bit
  // for bit), four waves against eight: 23.1 vs 28.7 us at B 64, h 8, n 100;
  // 25.4 vs 31.2 us at n 128; 91.8 vs 102.7 us at B 8, h 16, n 1024; 147.8 vs
  // 159.4 us at B 4, h 16, n 2048; 292 vs 337 us at B 1, h 4, n 8192 and 571
  // vs 658 us at B 1, h 2, n 16384 (128 eight-wave workgroups); 953 vs 944 us
  // at B 2, h 16, n 8192 (1024 of them; the dQ kernel alone 407 vs 397 us).
  // dK/dV workgroups: four waves (128 keys) beyond 64 keys (eight were 1%
  // slower at n = 8192).
  const bool wide = a.Nq >= 4096 && (int64_t)((a.Nq + 255) / 256) * a.B * a.H >= 512;
  hipError_t e = a.Nq <= 64 ? launch_dq<Op, 2>(a, stream, evt(0), evt(1))
                 : wide     ? launch_dq<Op, 8>(a, stream, evt(0), evt(1))
                            : launch_dq<Op, 4>(a, stream, evt(0), evt(1));
  if (e != hipSuccess) return e;
  return bwd_dkdv_keys_per_block(a.Nk) == 128 ? launch_dkdv<Op, 4>(a, stream, evt(2), evt(3))
                                              : launch_dkdv<Op, 2>(a, stream, evt(2), evt(3));
}

}  // namespace

hipError_t launch_bwd_mfma(const BwdArgs& a, DType dt, hipStream_t stream, hipEvent_t const* ev) {
  return dt == DType::BF16 ? launch_bwd<BF16>(a, stream, ev) : launch_bwd<F16>(a, stream, ev);
}

}  // namespace mha
