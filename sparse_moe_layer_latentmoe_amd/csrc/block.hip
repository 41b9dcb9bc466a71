// The block's pre-norm RMSNorm ahead of the layer (page "Nemotron 3 Ultra
// 架构深度拆解报告", CH9 §9.3: each block normalises its residual stream, runs
// the mixer and adds the residual back), split for the GEMMs that follow:
// per token t
//   xt[t] = bf16(gamma * h[t])          fp32 product, rounded to nearest even
//   rn[t] = 1 / sqrt(mean(h[t]^2) + eps)
// so that RMSNorm(h)[t] = rn[t] * xt[t].  The latent and shared-up
// projections read xt and multiply their fp32 sums by rn[t]; the residual add
// is the output projection's epilogue.  The sum of squares is accumulated in
// fp64 (each square of a bf16 value is exact there), so rn is the fp32
// rounding of the exact factor up to the last bits of the square root.
#include "kernels.h"
#include "lmoe_device.h"

namespace lmoe {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kPrenormThreads = 256;

// One work-group per token row; each thread handles 8 consecutive columns
// per pass (D is a multiple of 8).
__global__ __launch_bounds__(kPrenormThreads) void prenorm_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ gamma, int D, float eps,
    uint16_t* __restrict__ xt, float* __restrict__ rn) {
  __shared__ double part[kPrenormThreads / 64];
  const size_t row = (size_t)blockIdx.x * D;
  double ss = 0.0;
  for (int c = threadIdx.x * 8; c < D; c += kPrenormThreads * 8) {
    const u16x8 hv = *reinterpret_cast<const u16x8*>(h + row + c);
    const u16x8 gv = *reinterpret_cast<const u16x8*>(gamma + c);
    u16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float a = bf16_to_f32(hv[i]);
      ss = fma((double)a, (double)a, ss);
      o[i] = f32_to_bf16(a * bf16_to_f32(gv[i]));
    }
    *reinterpret_cast<u16x8*>(xt + row + c) = o;
  }
  // fixed-order reduction: butterfly within each wave, then the waves in order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kPrenormThreads / 64; ++w) tot += part[w];
    rn[blockIdx.x] = (float)(1.0 / sqrt(tot / D + (double)eps));
  }
}

hipError_t prenorm(const uint16_t* h, const uint16_t* gamma, int T, int D, float eps,
                   uint16_t* xt, float* rn, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  prenorm_kernel<<<T, kPrenormThreads, 0, s>>>(h, gamma, D, eps, xt, rn);
  return hipGetLastError();
}

}  // namespace lmoe
