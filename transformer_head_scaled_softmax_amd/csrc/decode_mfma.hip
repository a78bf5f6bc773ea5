// decode_mfma.hip -- one decoding step against a key/value cache, head size
// 64, bf16 / fp16, on the gfx950 matrix cores.
//
// During generation the keys and values of the positions already produced are
// kept and only the newest position is computed ("Translation and
// summarization (encoder-decoder)" and "This parallelism is a training-time
// property", alexdo.xyz; "Inference (Autoregressive Loop)",
// trishampatil.com).  Each new query row still computes the pages' formula,
// softmax(scale * q K^T) V over the cache slots it may see: under the causal
// mask query i of Nq new ones sits at position L - Nq + i and sees the slots
// up to it; without the mask (cross-attention against a source's cache) it
// sees all L filled slots.  Grouped- and multi-query attention share one cache
// head among H / Hkv consecutive query heads ("Many heads, many subspaces",
// zeroshotmind.com; "Limitations of the Original Design", trishampatil.com).
//
// The step reads the whole filled cache once and does 4 * 64 flops per key and
// query row, so it is bound by HBM bandwidth.  The work is cut along the keys:
// a workgroup owns one chunk of one (sequence, cache head) and all R =
// (H / Hkv) * Nq query rows that read that cache head, so every cache byte is
// read once whatever the group size.  Each wave streams its own run of the
// chunk through a private ring of LDS stages filled by direct-to-LDS buffer
// loads; nothing is shared between waves until the end, so the key loop has
// no barriers.  Per 32-key block a wave computes the transposed scores
// S^T (32 keys x 32 rows) = K Q^T, turns them into probabilities in registers
// and adds V^T P^T into its O^T accumulators -- the same register layouts as
// the prefill attention kernel, with a 32-key block instead of a 64-key tile.
// At the end the waves merge their (reference maximum, sum, accumulators)
// states through LDS; a single-chunk launch writes the normalised rows, a
// multi-chunk launch writes the merged state of its chunk and a second kernel
// combines the chunks of each row.
//
// MFMA 32x32x16 lane layout: see mfma_util.h.
#include "mfma_util.h"

namespace mha {
namespace {

constexpr int kD = kMfmaHeadDim;           // 64
constexpr int kBlk = 32;                   // keys per block
constexpr int kHalfStage = kBlk * kD;      // elements of one K (or V) block: 4 KiB
constexpr int kStage = 2 * kHalfStage;     // K block, then V block
constexpr int kLoadsPerBlock = 8;          // 1 KiB direct-to-LDS loads per wave per block
constexpr int kDeadOffset = (int)0x80000000u;

// s_waitcnt lgkmcnt(0) with the other counters unconstrained (gfx9 encoding).
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// NW waves per workgroup, NS ring stages per wave, QB sub-blocks of 32 rows.
template <class Op, int NW, int NS, int QB>
__global__ __launch_bounds__(NW * 64, (NW * NS * kStage * 2 <= 80 * 1024) ? 2 : 1) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(NS >= 2 && (NS - 1) * kLoadsPerBlock < 64, "bad stage count");
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NW * NS * kStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;

  // Chunk-major order: the first chunks of every cache come first (all of
  // them hold keys); later chunks of short caches exit at once.
  const int BG = a.B * a.Hkv;
  const int bg = blockIdx.x % BG;
  const int split = blockIdx.x / BG;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.H / a.Hkv, R = G * a.Nq;

  int L = a.S;
  if (a.cache_lens) L = min(max(a.cache_lens[b], 0), a.S);
  const int c0 = split * a.chunk;
  if (a.nsplit > 1 && c0 >= L) return;  // nothing in this chunk; the combine skips it
  const int c1 = min(c0 + a.chunk, L);

  // Query rows r = (head within the group) * Nq + i, consecutive in q and out.
  // Row col + 32u of this lane: its key end within the chunk.
  const int64_t row0 = ((int64_t)b * a.H + (int64_t)g * G) * a.Nq;
  int kend[QB];
  bool rvalid[QB];
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    const int r = col + 32 * u;
    rvalid[u] = r < R;
    const int i = rvalid[u] ? r % a.Nq : 0;
    kend[u] = a.causal ? min(c1, L - a.Nq + i + 1) : c1;
  }
  // Blocks whose keys all lie below every row's key end need no mask.
  const int kmask = a.causal ? min(c1, L - a.Nq + 1) : c1;

  // This wave's run of the chunk: [w0, w1), a whole number of blocks.
  const int per_wave = a.chunk / NW;
  const int w0 = c0 + wave * per_wave;
  const int w1 = min(w0 + per_wave, c1);
  const int nblk = w1 > w0 ? (w1 - w0 + kBlk - 1) / kBlk : 0;

  // The filled slots of this cache head as range-checked buffers: slots at or
  // past L read as zeros and never touch memory.
  const int64_t cache_off = (int64_t)bg * a.S * kD;
  const __amdgpu_buffer_rsrc_t ksrc = make_rsrc(static_cast<const uint16_t*>(a.k) + cache_off, (int64_t)L * kD * 2);
  const __amdgpu_buffer_rsrc_t vsrc = make_rsrc(static_cast<const uint16_t*>(a.v) + cache_off, (int64_t)L * kD * 2);

  // Query rows as B operands of S^T = K Q^T (features 16kk + 8half .. +7); a
  // negative scale is folded in by negating q (exact).
  const uint32_t qsign = a.scale < 0.0f ? 0x80008000u : 0u;
  const float c2 = fabsf(a.scale) * kLog2e;
  const __amdgpu_buffer_rsrc_t qsrc =
      make_rsrc(static_cast<const uint16_t*>(a.q) + row0 * kD, (int64_t)R * kD * 2);
  u32x4_t qreg[QB][4];
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    const int qoff = rvalid[u] ? (col + 32 * u) * kD * 2 + half * 16 : kDeadOffset;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qreg[u][kk] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, qoff + kk * 32, 0, 0) ^ qsign;
  }

  // Direct-to-LDS loads: load i of a half-stage fills rows 8i .. 8i+7, lane l
  // at row 8i + l/8, slot l%8.  K rows carry global chunk
  // slot ^ operand_swizzle(row) = (l%8) ^ (l/8) ^ (i&1); V rows carry chunk
  // slot ^ (bit 1 of the row) * 4 = (l%8) ^ ((l/16)&1)*4, the layout the
  // transposing reads below expect.
  const int lrow = lane >> 3;
  const int gk0 = (lane & 7) ^ lrow, gv = (lane & 7) ^ (((lane >> 4) & 1) << 2);
  uint16_t* ring = lds + wave * NS * kStage;
  auto issue = [&](int t) {
    uint16_t* dst = ring + (t % NS) * kStage;
    const int j0 = w0 + t * kBlk;
    const int dead = (int)((uint32_t)(t >= nblk) << 31);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (j0 + 8 * i + lrow) * (kD * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrc, MHA_LDS(dst + i * 512), 16,
                                               (row + ((gk0 ^ (i & 1)) << 4)) | dead, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (j0 + 8 * i + lrow) * (kD * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vsrc, MHA_LDS(dst + kHalfStage + i * 512), 16,
                                               (row + (gv << 4)) | dead, 0, 0, 0);
    }
  };

  // V^T operands through ds_read_b64_tr_b16 (as in the prefill kernel): lane
  // 4k + q of each 16-lane group points at key row k0 + k, features
  // c0 + 4q .. +3, and receives features c0 + (lane % 16) of keys k0 .. k0+3.
  const int tr_k = (lane & 15) >> 2, tr_q = lane & 3, tr_cg = (lane >> 4) & 1;
  const int tr_row = 4 * half + tr_k;
  int tr_col[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int cidx = cb * 32 + 16 * tr_cg + 4 * tr_q;
    tr_col[cb] = (((cidx >> 3) ^ (((tr_k >> 1) & 1) << 2)) << 3) + (cidx & 7);
  }
  auto vread = [&](const uint16_t* vs, int row, int cb) -> u32x2_t {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
    lds_s16x4_t* p = (lds_s16x4_t*)(const __attribute__((address_space(3))) uint16_t*)&vs[row * kD + tr_col[cb]];
    return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(p));
  };

  f32x16_t o[QB][2];
  float m_ref[QB], lsum[QB];
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    m_ref[u] = -INFINITY;
    lsum[u] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[u][cb][r] = 0.0f;
  }

  const int swz = operand_swizzle(col);  // block rows start at multiples of 32
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);
  for (int t = 0; t < nblk; ++t) {
    // Block t has landed once at most the NS-2 later blocks are in flight.
    // Every LDS read of the stage about to be refilled was consumed by the
    // previous block's MFMAs; the lgkm wait makes that explicit.
    wait_vmcnt<(NS - 2) * kLoadsPerBlock>();
    wait_lgkm0();
    asm volatile("" ::: "memory");
    issue(t + NS - 1);

    const uint16_t* ks = ring + (t % NS) * kStage;
    const uint16_t* vs = ks + kHalfStage;
    const int j0 = w0 + t * kBlk;

    f32x16_t s[QB];
#pragma unroll
    for (int u = 0; u < QB; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[u][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4_t av = *reinterpret_cast<const u32x4_t*>(&ks[col * kD + (((kk * 2 + half) ^ swz) << 3)]);
#pragma unroll
      for (int u = 0; u < QB; ++u) s[u] = Op::mma(av, qreg[u][kk], s[u]);
    }

    // V^T operands of the block: step t4 covers keys 16t4 + 4half + {0..3}
    // and 16t4 + 8 + 4half + {0..3} of this lane's feature row.
    u32x4_t vop[2][2];
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const u32x2_t lo = vread(vs, 16 * t4 + tr_row, cb);
        const u32x2_t hi = vread(vs, 16 * t4 + 8 + tr_row, cb);
        vop[t4][cb] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }

    // Register r of this lane holds key j0 + 8(r/4) + 4half + r%4 of row
    // col + 32u; keys at or past the row's end become -inf.
    if (j0 + kBlk > kmask) {
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        const int lim = kend[u] - j0 - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((r >> 2) * 8 + (r & 3) >= lim) s[u][r] = -INFINITY;
      }
    }

#pragma unroll
    for (int u = 0; u < QB; ++u) {
      // P = exp2(s * c2 - m_ref) packed in the order of the P^T operand
      // (step t4 takes registers 8t4 .. 8t4+7); the row sum comes from the
      // packed values.  Optimistic against the current reference; redone
      // with the block's true maximum only when the partial sum is not
      // finite or exceeds kGuard (first visible block, or a much larger
      // score).
      u32x4_t pb[2];
      float ls = 0.0f;
      auto exponentiate = [&](float mu, bool select_masked) {
        ls = 0.0f;
#pragma unroll
        for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int r = 8 * t4 + 2 * w;
            float p0 = __builtin_amdgcn_exp2f(fmaf(s[u][r], c2, -mu));
            float p1 = __builtin_amdgcn_exp2f(fmaf(s[u][r + 1], c2, -mu));
            if (select_masked) {
              p0 = s[u][r] == -INFINITY ? 0.0f : p0;
              p1 = s[u][r + 1] == -INFINITY ? 0.0f : p1;
            }
            pb[t4][w] = Op::pack(p0, p1);
            ls = Op::sum2(pb[t4][w], ls);
          }
      };
      exponentiate(m_ref[u], false);
      const bool need = lanes_max(ls <= Op::kGuard ? 0.0f : 1.0f) > 0.0f;
      if (__any(need)) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[u][r]);
        mx = lanes_max(mx);
        const float mt = (mx == -INFINITY) ? -INFINITY : mx * c2;
        const float m_new = need ? fmaxf(m_ref[u], mt) : m_ref[u];
        const float alpha = (need && m_new != -INFINITY) ? __builtin_amdgcn_exp2f(m_ref[u] - m_new) : 1.0f;
        lsum[u] *= alpha;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[u][cb][r] *= alpha;
        m_ref[u] = m_new;
        exponentiate(m_ref[u] == -INFINITY ? 0.0f : m_ref[u], true);
      }
      lsum[u] += ls;
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) o[u][cb] = Op::mma(vop[t4][cb], pb[t4], o[u][cb]);
    }
  }

  // Merge the waves' states through LDS (the rings are free once every wave's
  // loads, including the dead ones past its run, have drained).  Wave w
  // leaves, per row r: its reference maximum and sum at mls[w][r], and its
  // accumulators at acc[w][r][f] (feature f).
  wait_vmcnt<0>();
  __syncthreads();
  constexpr int RM = 32 * QB;
  static_assert(NW * RM * (kD + 2) * 4 <= NW * NS * kStage * 2, "merge buffer does not fit");
  float* accs = reinterpret_cast<float*>(lds);
  float* mls = accs + NW * RM * kD;
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    const int r = col + 32 * u;
    float* dst = accs + (wave * RM + r) * kD;
    // register (cb, 4q + e) of this lane is feature 32cb + 8q + 4half + e
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(&dst[32 * cb + 8 * q + 4 * half]) =
            float4{o[u][cb][4 * q + 0], o[u][cb][4 * q + 1], o[u][cb][4 * q + 2], o[u][cb][4 * q + 3]};
    const float ltot = lanes_sum(lsum[u]);
    if (half == 0) {
      mls[(wave * RM + r) * 2 + 0] = m_ref[u];
      mls[(wave * RM + r) * 2 + 1] = ltot;
    }
  }
  __syncthreads();

  // Thread -> (row, 8 features).  Reference M = the largest of the waves'
  // references; a wave with no visible key has -inf and weight 0.
  for (int idx = tid; idx < R * 8; idx += NT) {
    const int r = idx >> 3, f0 = (idx & 7) * 8;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mls[(w * RM + r) * 2]);
    float l = 0.0f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = mls[(w * RM + r) * 2];
        const float sc = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        l = fmaf(mls[(w * RM + r) * 2 + 1], sc, l);
        const float* src = accs + (w * RM + r) * kD + f0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(src[e], sc, acc[e]);
      }
    }
    if (a.nsplit == 1) {
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      u32x4_t w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = Op::pack(acc[2 * e] * inv, acc[2 * e + 1] * inv);
      *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.out) + (row0 + r) * kD + f0) = w4;
    } else {
      float* rec = a.part + (((int64_t)bg * a.nsplit + split) * R + r) * kDecodePartFloats;
      if (f0 == 0) *reinterpret_cast<float2*>(rec) = float2{M, l};
      *reinterpret_cast<float4*>(rec + 4 + f0) = float4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<float4*>(rec + 8 + f0) = float4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

// Combines the chunk states of each row: out = sum_c acc_c 2^(M_c - M) /
// sum_c l_c 2^(M_c - M), M = max_c M_c, over the chunks that hold keys.
// Thread -> (row, 8 features); rows with no visible key anywhere give 0.
template <class Op>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const int G = a.H / a.Hkv, R = G * a.Nq;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.Hkv * R;
  if (idx >= rows * 8) return;
  const int64_t grow = idx >> 3;  // (b*Hkv + g) * R + r
  const int f0 = (int)(idx & 7) * 8;
  const int bg = (int)(grow / R), r = (int)(grow % R);
  const int b = bg / a.Hkv;
  int L = a.S;
  if (a.cache_lens) L = min(max(a.cache_lens[b], 0), a.S);
  const int live = (L + a.chunk - 1) / a.chunk;
  const float* base = a.part + ((int64_t)bg * a.nsplit * R + r) * kDecodePartFloats;
  const int64_t step = (int64_t)R * kDecodePartFloats;
  float M = -INFINITY;
  for (int c = 0; c < live; ++c) M = fmaxf(M, base[c * step]);
  float l = 0.0f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  if (M != -INFINITY) {
    for (int c = 0; c < live; ++c) {
      const float* rec = base + c * step;
      const float mc = rec[0];
      const float sc = mc == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mc - M);
      l = fmaf(rec[1], sc, l);
      const float4 x0 = *reinterpret_cast<const float4*>(rec + 4 + f0);
      const float4 x1 = *reinterpret_cast<const float4*>(rec + 8 + f0);
      acc[0] = fmaf(x0.x, sc, acc[0]);
      acc[1] = fmaf(x0.y, sc, acc[1]);
      acc[2] = fmaf(x0.z, sc, acc[2]);
      acc[3] = fmaf(x0.w, sc, acc[3]);
      acc[4] = fmaf(x1.x, sc, acc[4]);
      acc[5] = fmaf(x1.y, sc, acc[5]);
      acc[6] = fmaf(x1.z, sc, acc[6]);
      acc[7] = fmaf(x1.w, sc, acc[7]);
    }
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  u32x4_t w4;
#pragma unroll
  for (int e = 0; e < 4; ++e) w4[e] = Op::pack(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  const int64_t orow = ((int64_t)b * a.H + (int64_t)(bg % a.Hkv) * G) * a.Nq + r;
  *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(a.out) + orow * kD + f0) = w4;
}

template <class Op, int NW, int NS, int QB>
hipError_t launch(const DecodeArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1, hipEvent_t t2,
                  hipEvent_t t3) {
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.nsplit;
  if (blocks == 0) return hipSuccess;
  hipExtLaunchKernelGGL((decode_mfma_kernel<Op, NW, NS, QB>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                        t0, t1, 0, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const int64_t threads = (int64_t)a.B * a.Hkv * (a.H / a.Hkv) * a.Nq * 8;
  hipExtLaunchKernelGGL((decode_combine_kernel<Op>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                        stream, t2, t3, 0, a);
  return hipGetLastError();
}

template <class Op>
hipError_t launch_rows(const DecodeArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1, hipEvent_t t2,
                       hipEvent_t t3) {
  const int R = a.H / a.Hkv * a.Nq;
  return R <= 32 ? launch<Op, 4, 4, 1>(a, stream, t0, t1, t2, t3) : launch<Op, 4, 4, 2>(a, stream, t0, t1, t2, t3);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1,
                              hipEvent_t t2, hipEvent_t t3) {
  return dt == DType::BF16 ? launch_rows<BF16>(a, stream, t0, t1, t2, t3)
                           : launch_rows<F16>(a, stream, t0, t1, t2, t3);
}

}  // namespace mha
