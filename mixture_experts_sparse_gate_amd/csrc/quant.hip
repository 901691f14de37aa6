// Block-FP8 form of expert weights: FP8 weights shrink the model
// ("MoE架构：突破单卡算力瓶颈的密钥" §1.3) and are held with a scale per block
// ("Block FP8" serving on MI300, CUDA-to-ROCm section of "4大技术模块掌握
// Tutel MoE…"). Blocks of 128 x 128 of each [K, Ncols] matrix; scale =
// amax / 448; codes are OCP E4M3 (bias 7, 3 mantissa bits, largest finite
// 448, exponent field 0 for subnormals m * 2^-9) of w / scale, rounded to
// nearest with ties to even. Both divisions are IEEE fp32 divisions.
//
// The codes are stored in K-groups of 8: the 8 consecutive K values of one
// column are 8 contiguous bytes, which is the 8-element fragment one lane of
// the FFN kernel's 32x32x16 MFMA reads (a plain 8-byte LDS read, converted
// to bf16 exactly).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kQBlock = 128;
constexpr int kQThreads = 256;

// E4M3 code of q, saturated at 448 (|q| can exceed 448 only when the scale
// itself is an inexact fp32 subnormal; up to 464 it rounds to 448 anyway):
// below 2^-6 the
// codes are the multiples of 2^-9, so the code is q * 512 rounded to the
// nearest integer, ties to even (8 is 2^-6, the first normal code, so the
// two ranges meet); above, the fp32 mantissa is rounded to 3 bits, ties to
// even, and the exponent rebased from 127 to 7 (a carry out of the mantissa
// moves to the next exponent, as it should).
__device__ inline uint32_t e4m3_code(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fminf(fabsf(q), 448.f);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t b = __float_as_uint(a);
    mag = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  }
  return sign | mag;
}

// One 128 x 128 block per workgroup. Thread t handles column t % 128 and
// the K-groups t / 128, t / 128 + 2, ...: its reads of a row are coalesced
// across the wave, and each K-group's 8 codes leave as one 8-byte store,
// consecutive threads writing consecutive columns.
template <typename E>
__global__ __launch_bounds__(kQThreads) void quantize_fp8_kernel(const E* __restrict__ W, int K, int Ncols,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ scales) {
  __shared__ float wmax[kQThreads / kWave];
  const int nb = blockIdx.x, kb = blockIdx.y, g = blockIdx.z;
  const int KB = K / kQBlock, NB = Ncols / kQBlock;
  const int tid = threadIdx.x, col = tid % kQBlock, kg0 = tid / kQBlock;
  const int64_t n = (int64_t)nb * kQBlock + col;
  const E* src = W + ((int64_t)g * K + (int64_t)kb * kQBlock) * Ncols + n;
  float v[8][8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[j][e] = (float)src[(int64_t)((kg0 + 2 * j) * 8 + e) * Ncols];
      amax = fmaxf(amax, fabsf(v[j][e]));
    }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  if (lane_id() == 0) wmax[tid / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = amax / 448.f;
  if (tid == 0) scales[((int64_t)g * KB + kb) * NB + nb] = s;
  uint8_t* dst = codes + (((int64_t)g * (K / 8) + (int64_t)kb * (kQBlock / 8)) * Ncols + n) * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t lo = 0, hi = 0;
    if (s > 0.f) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= e4m3_code(v[j][e] / s) << (8 * e);
        hi |= e4m3_code(v[j][e + 4] / s) << (8 * e);
      }
    }
    *reinterpret_cast<u32x2*>(dst + (int64_t)(kg0 + 2 * j) * Ncols * 8) = u32x2{lo, hi};
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const void* W, bool bf16_, int groups, int K, int Ncols, uint8_t* codes,
                               float* scales, hipStream_t s) {
  const dim3 grid(Ncols / kQBlock, K / kQBlock, groups);
  if (bf16_)
    hipLaunchKernelGGL(quantize_fp8_kernel<bf16>, grid, dim3(kQThreads), 0, s, static_cast<const bf16*>(W), K,
                       Ncols, codes, scales);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<float>, grid, dim3(kQThreads), 0, s, static_cast<const float*>(W), K,
                       Ncols, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
