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
// The step reads the whole filled cache once and does 4 * 64 flops per slot
// and query row, so it is bound by HBM bandwidth.  Caches of one batch have
// unequal fill lengths, so the work is balanced on the device: the filled
// slots of all caches, laid end to end, are cut into equal ranges, one per
// wave (each workgroup is one wave, three per compute unit, so at most one
// per SIMD).  A wave's range falls into pieces at cache boundaries.  For each
// piece the wave takes all R = (H / Hkv) * Nq query rows that read that cache
// head -- so every cache byte is read once whatever the group size -- and
// streams the piece's slots in 32-slot blocks through a ring of LDS stages
// filled by direct-to-LDS buffer loads.  Per block it computes the transposed
// scores S^T (32 slots x 32 rows) = K Q^T, turns them into probabilities in
// registers and adds V^T P^T into its O^T accumulators: the register layouts
// of the prefill attention kernel, with a 32-slot block instead of a 64-key
// tile.  A piece that is a whole cache writes its normalised rows; the other
// pieces leave their softmax state (reference maximum, sum, accumulators) for
// a second kernel that merges the pieces of each cut cache.
//
// MFMA 32x32x16 lane layout: see mfma_util.h.
#include <atomic>
#include <mutex>

#include "mfma_util.h"

// Device memory of mha_decode_forward_noalloc: the partial softmax states and
// the per-cache wave spans that the allocation-free entry point would
// otherwise take from a caller's workspace.  Every GPU the library runs on
// holds its own copy for the life of the process.  In host code the name
// stands for a host-side shadow, not a device address: the launch uses the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[mha::kDecodeScratchBytes];

namespace mha {
namespace {

constexpr int kD = kMfmaHeadDim;           // 64
constexpr int kBlk = 32;                   // slots per block
constexpr int kHalfStage = kBlk * kD;      // elements of one K (or V) block: 4 KiB
constexpr int kStage = 2 * kHalfStage;     // K block, then V block
constexpr int kLoadsPerBlock = 8;          // 1 KiB direct-to-LDS loads per block
constexpr int kDeadOffset = (int)0x80000000u;

// s_waitcnt lgkmcnt(0) with the other counters unconstrained (gfx9 encoding).
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// 64-bit wave-uniform value into scalar registers; 64-bit cross-lane moves.
__device__ inline int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ inline int64_t shfl64(int64_t x, int src) {
  const int lo = __shfl((int)(uint32_t)x, src), hi = __shfl((int)(uint32_t)((uint64_t)x >> 32), src);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ inline int64_t shfl_up64(int64_t x, int d) {
  const int lo = __shfl_up((int)(uint32_t)x, d), hi = __shfl_up((int)(uint32_t)((uint64_t)x >> 32), d);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// ds_read_b64_tr_b16 through inline assembly.  With the intrinsic the
// compiler waits for every direct-to-LDS load in flight before the read (it
// cannot tell that they fill other stages of the ring), which would drain the
// ring at every block.  The results must pass through lds_wait before use.
__device__ inline u32x2_t ds_read_tr(uint32_t lds_byte_addr) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_byte_addr) : "memory");
  return r;
}

// Waits for every LDS read in flight; the operands are tied through the wait
// so that no use of them can be scheduled before it.
__device__ inline void lds_wait(u32x2_t (&v)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}

// One wave per workgroup; NS ring stages; QB sub-blocks of 32 query rows.
template <class Op, int NS, int QB>
__global__ __launch_bounds__(64, 1) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(NS >= 2 && (NS - 1) * kLoadsPerBlock < 64, "bad stage count");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * kStage];

  const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
  const int w = blockIdx.x;
  const int Hkv = a.Hkv, G = a.H / Hkv, R = G * a.Nq;
  auto fill = [&](int b) -> int { return a.cache_lens ? min(max(a.cache_lens[b], 0), a.S) : a.S; };

  // Slots of the caches laid end to end: batch entry b holds Hkv caches of
  // L_b slots each.  Lane l sums the entries [l*c, (l+1)*c); an inclusive scan
  // over the lanes gives each lane's block of positions.
  const int c = (a.B + 63) / 64;
  int64_t mine = 0;
  for (int i = 0; i < c; ++i) {
    const int b = lane * c + i;
    if (b < a.B) mine += fill(b);
  }
  int64_t incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t y = shfl_up64(incl, d);
    if (lane >= d) incl += y;
  }
  const int64_t T = uniform64((int64_t)Hkv * shfl64(incl, 63));
  if (T == 0) return;  // every cache is empty: the combining kernel writes the zeros
  const int64_t W = min((int64_t)a.waves, T);  // every wave's range is non-empty
  if (w >= W) return;
  const int64_t lo = (int64_t)w * T / W, hi = (int64_t)(w + 1) * T / W;

  // The batch entry holding position lo: first the lane block, then a walk.
  const int64_t blk_lo = (int64_t)Hkv * (incl - mine), blk_hi = (int64_t)Hkv * incl;
  const int src = __builtin_ctzll(__ballot(blk_lo <= lo && lo < blk_hi));
  int b = src * c;
  int64_t pos_b = uniform64(shfl64(blk_lo, src));
  int Lb = fill(b);
  while (lo >= pos_b + (int64_t)Hkv * Lb) {
    pos_b += (int64_t)Hkv * Lb;
    Lb = fill(++b);
  }
  int g = (int)((lo - pos_b) / Lb);
  int x = (int)((lo - pos_b) % Lb);

  const uint32_t qsign = a.scale < 0.0f ? 0x80008000u : 0u;
  const float c2 = fabsf(a.scale) * kLog2e;
  const int swz = operand_swizzle(col);  // block rows start at multiples of 32

  // Direct-to-LDS loads: load i of a half-stage fills rows 8i .. 8i+7, lane l
  // at row 8i + l/8, slot l%8.  K rows carry global chunk
  // slot ^ operand_swizzle(row) = (l%8) ^ (l/8) ^ (i&1); V rows carry chunk
  // slot ^ (bit 1 of the row) * 4 = (l%8) ^ ((l/16)&1)*4, the layout the
  // transposing reads expect.
  const int lrow = lane >> 3;
  const int gk0 = (lane & 7) ^ lrow, gv = (lane & 7) ^ (((lane >> 4) & 1) << 2);

  // V^T operands through ds_read_b64_tr_b16 (as in the prefill kernel): lane
  // 4k + q of each 16-lane group points at slot row k0 + k, features
  // c0 + 4q .. +3, and receives features c0 + (lane % 16) of slots k0 .. k0+3.
  const int tr_k = (lane & 15) >> 2, tr_q = lane & 3, tr_cg = (lane >> 4) & 1;
  const int tr_row = 4 * half + tr_k;
  int tr_col[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int cidx = cb * 32 + 16 * tr_cg + 4 * tr_q;
    tr_col[cb] = (((cidx >> 3) ^ (((tr_k >> 1) & 1) << 2)) << 3) + (cidx & 7);
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)lds;
  uint32_t tr_addr[2][2];  // byte address within a stage's V block: [slot half 0/8][cb]
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) tr_addr[hh][cb] = lds_base + 2 * (kHalfStage + (8 * hh + tr_row) * kD + tr_col[cb]);

  // Pieces of this wave's range [lo, hi): slots [x, xe) of cache (b, g).
  int64_t pos = lo;
  for (;;) {
    const int bg = b * Hkv + g;
    const int64_t pcache = pos - x;  // position of slot 0 of this cache
    const int xe = (int)min((int64_t)Lb, (int64_t)x + (hi - pos));
    const int64_t row0 = ((int64_t)b * a.H + (int64_t)g * G) * a.Nq;

    // Query rows r = (head within the group) * Nq + i, consecutive in q and
    // out, as B operands of S^T = K Q^T (features 16kk + 8half .. +7); a
    // negative scale is folded in by negating q (exact).
    const __amdgpu_buffer_rsrc_t qsrc =
        make_rsrc(static_cast<const uint16_t*>(a.q) + row0 * kD, (int64_t)R * kD * 2);
    u32x4_t qreg[QB][4];
    int kend[QB];
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      const int r = col + 32 * u;
      const bool valid = r < R;
      const int qoff = valid ? r * kD * 2 + half * 16 : kDeadOffset;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qreg[u][kk] = __builtin_amdgcn_raw_buffer_load_b128(qsrc, qoff + kk * 32, 0, 0) ^ qsign;
      const int i = valid ? r % a.Nq : 0;
      kend[u] = a.causal ? min(xe, Lb - a.Nq + i + 1) : xe;  // this row's slot end in the piece
    }
    // Blocks whose slots all lie below every row's end need no mask.
    const int kmask = a.causal ? min(xe, Lb - a.Nq + 1) : xe;
    const int nblk = (xe - x + kBlk - 1) / kBlk;

    // The filled slots of this cache head as range-checked buffers: slots at
    // or past L read as zeros and never touch memory.
    const int64_t cache_off = (int64_t)bg * a.S * kD;
    const __amdgpu_buffer_rsrc_t ksrc =
        make_rsrc(static_cast<const uint16_t*>(a.k) + cache_off, (int64_t)Lb * kD * 2);
    const __amdgpu_buffer_rsrc_t vsrc =
        make_rsrc(static_cast<const uint16_t*>(a.v) + cache_off, (int64_t)Lb * kD * 2);
    auto issue = [&](int t) {
      uint16_t* dst = lds + (t % NS) * kStage;
      const int j0 = x + t * kBlk;
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

    // The previous piece's LDS reads have all been consumed by its MFMAs and
    // its loads drained; the ring can be refilled.
    wait_lgkm0();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st);
    for (int t = 0; t < nblk; ++t) {
      // Block t has landed once at most the NS-2 later blocks are in flight;
      // every LDS read of the stage about to be refilled was consumed by the
      // previous block's MFMAs (the lgkm wait makes that explicit).
      wait_vmcnt<(NS - 2) * kLoadsPerBlock>();
      wait_lgkm0();
      asm volatile("" ::: "memory");
      issue(t + NS - 1);

        const uint16_t* ks = lds + (t % NS) * kStage;
      const int j0 = x + t * kBlk;

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

      // V^T operands of the block, read now and waited for before the P V
      // products: step t4 covers slots 16t4 + 4half + {0..3} and
      // 16t4 + 8 + 4half + {0..3} of this lane's feature row.
      u32x2_t vtr[8];
      const uint32_t stage_bytes = (uint32_t)((t % NS) * kStage * 2);
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            vtr[4 * t4 + 2 * cb + hh] = ds_read_tr(tr_addr[hh][cb] + stage_bytes + t4 * 16 * kD * 2);

      // Register r of this lane holds slot j0 + 8(r/4) + 4half + r%4 of row
      // col + 32u; slots at or past the row's end become -inf.
      if (j0 + kBlk > kmask) {
#pragma unroll
        for (int u = 0; u < QB; ++u) {
          const int lim = kend[u] - j0 - 4 * half;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if ((r >> 2) * 8 + (r & 3) >= lim) s[u][r] = -INFINITY;
        }
      }

      bool vready = false;
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
            for (int q = 0; q < 4; ++q) {
              const int r = 8 * t4 + 2 * q;
              float p0 = __builtin_amdgcn_exp2f(fmaf(s[u][r], c2, -mu));
              float p1 = __builtin_amdgcn_exp2f(fmaf(s[u][r + 1], c2, -mu));
              if (select_masked) {
                p0 = s[u][r] == -INFINITY ? 0.0f : p0;
                p1 = s[u][r + 1] == -INFINITY ? 0.0f : p1;
              }
              pb[t4][q] = Op::pack(p0, p1);
              ls = Op::sum2(pb[t4][q], ls);
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
        if (!vready) {
          lds_wait(vtr);
          vready = true;
        }
#pragma unroll
        for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const u32x2_t lo2 = vtr[4 * t4 + 2 * cb], hi2 = vtr[4 * t4 + 2 * cb + 1];
            o[u][cb] = Op::mma(u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]}, pb[t4], o[u][cb]);
          }
      }
    }
    wait_vmcnt<0>();  // the dead loads past the piece write LDS too

    // The wave holding slot 0 of a cache records the waves over it: the owner
    // of position p is floor(((p + 1) W - 1) / T).
    if (x == 0 && lane == 0) {
      const int w1 = (int)(((pcache + Lb) * W - 1) / T);
      a.span[bg] = int2{w, w1};
    }
    // Register (cb, 4q + e) of this lane is feature 32cb + 8q + 4half + e of
    // row col + 32u.
    const bool whole = x == 0 && xe == Lb;
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      const int r = col + 32 * u;
      const float ltot = lanes_sum(lsum[u]);
      if (r < R) {
        if (whole) {
          const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
          uint16_t* orow = static_cast<uint16_t*>(a.out) + (row0 + r) * kD;
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              u32x2_t v2;
              v2[0] = Op::pack(o[u][cb][4 * q + 0] * inv, o[u][cb][4 * q + 1] * inv);
              v2[1] = Op::pack(o[u][cb][4 * q + 2] * inv, o[u][cb][4 * q + 3] * inv);
              *reinterpret_cast<u32x2_t*>(orow + 32 * cb + 8 * q + 4 * half) = v2;
            }
        } else {
          float* rec = a.part + ((int64_t)(bg + w) * R + r) * kDecodePartFloats;
          if (half == 0) *reinterpret_cast<float2*>(rec) = float2{m_ref[u], ltot};
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(rec + 4 + 32 * cb + 8 * q + 4 * half) =
                  float4{o[u][cb][4 * q + 0], o[u][cb][4 * q + 1], o[u][cb][4 * q + 2], o[u][cb][4 * q + 3]};
        }
      }
    }

    pos += xe - x;
    if (pos >= hi) break;
    // Next cache with filled slots (one exists: pos < hi <= T).
    x = 0;
    if (++g == Hkv) {
      g = 0;
      do {
        Lb = fill(++b);
      } while (Lb == 0);
    }
  }
}

// Merges the pieces of each cut cache: out = sum_p acc_p 2^(M_p - M) /
// sum_p l_p 2^(M_p - M), M = max_p M_p, over the waves p that cover the cache.
// One wave per row, lanes over the 64 features; the pieces are taken 32 at a
// time with all their loads in flight at once and merged online (reference
// raised per group).  Rows of empty caches get zeros; rows of caches that one
// wave covered whole are already written.
template <class Op>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int kGroup = 32;
  const int G = a.H / a.Hkv, R = G * a.Nq;
  const int lane = threadIdx.x & 63;
  const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b*Hkv + g) * R + r
  if (grow >= (int64_t)a.B * a.Hkv * R) return;
  const int bg = (int)(grow / R), r = (int)(grow % R);
  const int b = bg / a.Hkv;
  const int64_t orow = ((int64_t)b * a.H + (int64_t)(bg % a.Hkv) * G) * a.Nq + r;
  uint16_t* out = static_cast<uint16_t*>(a.out) + orow * kD + lane;
  const int L = a.cache_lens ? min(max(a.cache_lens[b], 0), a.S) : a.S;
  const int2 sp = a.span[bg];  // stale when L == 0, and then unused
  if (L == 0) {
    *out = 0;
    return;
  }
  if (sp.x == sp.y) return;
  const int n = sp.y - sp.x + 1;
  const float* base = a.part + ((int64_t)(bg + sp.x) * R + r) * kDecodePartFloats;
  const int64_t step = (int64_t)R * kDecodePartFloats;

  float M = -INFINITY, l = 0.0f, acc = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kGroup) {
    const int m = min(kGroup, n - c0);
    const float* grp = base + c0 * step;
    float mj = -INFINITY, lj = 0.0f;
    if (lane < m) {
      mj = grp[lane * step];
      lj = grp[lane * step + 1];
    }
    float xs[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) xs[j] = j < m ? grp[j * step + 4 + lane] : 0.0f;
    const float Mn = fmaxf(M, wave_max(mj));
    if (Mn == -INFINITY) continue;  // no visible slot in any piece so far
    const float alpha = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    const float sc = mj == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mj - Mn);
    l = fmaf(l, alpha, wave_sum(lj * sc));
    acc *= alpha;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) acc = fmaf(xs[j], __shfl(sc, j), acc);
    M = Mn;
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  *out = (uint16_t)(Op::pack(acc * inv, 0.0f) & 0xffffu);
}

template <class Op, int NS, int QB>
hipError_t launch(const DecodeArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1, hipEvent_t t2,
                  hipEvent_t t3) {
  hipExtLaunchKernelGGL((decode_mfma_kernel<Op, NS, QB>), dim3((unsigned)a.waves), dim3(64), 0, stream, t0, t1, 0,
                        a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.H * a.Nq;
  hipExtLaunchKernelGGL((decode_combine_kernel<Op>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, t2,
                        t3, 0, a);
  return hipGetLastError();
}

template <class Op>
hipError_t launch_rows(const DecodeArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1, hipEvent_t t2,
                       hipEvent_t t3) {
  const int R = a.H / a.Hkv * a.Nq;
  // Two ring stages (one block in flight while the other is computed):
  // measured 52.0 vs 53.0 (three) and 53.5 us (four) on the long decoding
  // workload, 19.5 vs 20.0 us with grouped-query heads.
  return R <= 32 ? launch<Op, 2, 1>(a, stream, t0, t1, t2, t3) : launch<Op, 2, 2>(a, stream, t0, t1, t2, t3);
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      // Once per device, with that device current: its copy's address.
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1,
                              hipEvent_t t2, hipEvent_t t3) {
  return dt == DType::BF16 ? launch_rows<BF16>(a, stream, t0, t1, t2, t3)
                           : launch_rows<F16>(a, stream, t0, t1, t2, t3);
}

}  // namespace mha
