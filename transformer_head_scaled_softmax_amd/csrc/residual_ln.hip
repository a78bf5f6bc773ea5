// residual_ln.hip -- the residual connection and layer normalisation after the
// attention sublayer, as a pass of its own: out = LayerNorm(out + residual) *
// gamma + beta per row of D features ("Residual Connections and Layer
// Normalization", trishampatil.com; "Add & Norm", alexdo.xyz), the biased
// variance, fp32 statistics in two passes over values held in registers.
// Used after the output projection when rows are too wide for the projection
// kernel to own them whole (see launch_gemm_ln).  One wave per row; each lane
// holds 8-feature chunks lane, lane + 64, ... of the row.
#include "mfma_util.h"

namespace mha {
namespace {

constexpr int kMaxChunks = 16;  // rows of up to 16 * 64 * 8 = 8192 features

template <class Op>
__global__ __launch_bounds__(256) void residual_ln_kernel(uint16_t* out, const uint16_t* residual,
                                                          const uint16_t* gamma, const uint16_t* beta, float eps,
                                                          int M, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  uint16_t* o = out + m * D;
  const uint16_t* r = residual + m * D;
  auto unpack8 = [](u32x4_t v, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = Op::to_float((uint16_t)(v[i] & 0xffffu));
      f[2 * i + 1] = Op::to_float((uint16_t)(v[i] >> 16));
    }
  };
  float z[kMaxChunks][8];
  float s1 = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int f0 = (j * 64 + lane) * 8;
    if (f0 < D) {  // D is a multiple of 8: the chunk is whole
      float a[8], b[8];
      unpack8(*reinterpret_cast<const u32x4_t*>(o + f0), a);
      unpack8(*reinterpret_cast<const u32x4_t*>(r + f0), b);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        z[j][e] = a[e] + b[e];
        s1 += z[j][e];
      }
    }
  }
  const float inv_d = 1.0f / (float)D;
  const float mean = wave_sum(s1) * inv_d;
  float s2 = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j)
    if ((j * 64 + lane) * 8 < D)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dz = z[j][e] - mean;
        s2 = fmaf(dz, dz, s2);
      }
  const float rstd = 1.0f / sqrtf(wave_sum(s2) * inv_d + eps);
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int f0 = (j * 64 + lane) * 8;
    if (f0 < D) {
      float gv[8], bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gv[e] = 1.0f;
        bv[e] = 0.0f;
      }
      if (gamma) unpack8(*reinterpret_cast<const u32x4_t*>(gamma + f0), gv);
      if (beta) unpack8(*reinterpret_cast<const u32x4_t*>(beta + f0), bv);
      u32x4_t w;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = Op::pack(fmaf((z[j][2 * i] - mean) * rstd, gv[2 * i], bv[2 * i]),
                        fmaf((z[j][2 * i + 1] - mean) * rstd, gv[2 * i + 1], bv[2 * i + 1]));
      *reinterpret_cast<u32x4_t*>(o + f0) = w;
    }
  }
}

template <class Op>
hipError_t launch(void* out, const void* residual, const void* gamma, const void* beta, float eps, int M, int D,
                  hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (M == 0) return hipSuccess;
  hipExtLaunchKernelGGL((residual_ln_kernel<Op>), dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream, t0, t1, 0,
                        static_cast<uint16_t*>(out), static_cast<const uint16_t*>(residual),
                        static_cast<const uint16_t*>(gamma), static_cast<const uint16_t*>(beta), eps, M, D);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_residual_ln(void* out, const void* residual, const void* gamma, const void* beta, float eps,
                              int M, int D, DType dt, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  return dt == DType::BF16 ? launch<BF16>(out, residual, gamma, beta, eps, M, D, stream, t0, t1)
                           : launch<F16>(out, residual, gamma, beta, eps, M, D, stream, t0, t1);
}

}  // namespace mha
