// Measurement aids: the chip's own ceilings, timed in the same run as the
// layer, so that the layer's kernels can be judged against measured peaks
// as well as published ones.
//   copy_kernel  a plain device copy with 16-byte loads and stores (the
//                STREAM "copy" pattern): HBM bandwidth for mixed read/write
//                traffic once the buffers exceed the 256 MB last-level cache
//   mfma_kernel  bf16 32x32x16 MFMAs on register operands only (four sets
//                of hashed values), four independent accumulators per wave:
//                the matrix cores' rate with no memory traffic at all
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyBlock) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                          int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kCopyBlock * kCopyUnroll;
  for (int64_t i0 = (int64_t)blockIdx.x * kCopyBlock * kCopyUnroll + threadIdx.x; i0 < n16; i0 += stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * kCopyBlock;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + u * kCopyBlock;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

constexpr int kMfmaWaves = 8;  // per block: two waves per SIMD

// a bf16 pair of finite values from 32 hashed bits: random signs and
// mantissas, exponents within 2^-7 .. 2^0 (so that the sums stay finite)
__device__ inline uint32_t bf16_pair(uint32_t r) {
  const uint32_t lo = (r & 0x8000u) | ((0x78u + ((r >> 8) & 7u)) << 7) | (r & 0x7Fu);
  const uint32_t hi = ((r >> 16) & 0x8000u) | ((0x78u + ((r >> 24) & 7u)) << 7) | ((r >> 16) & 0x7Fu);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(kMfmaWaves * kWave) void mfma_kernel(int iters, float* sink) {
  const int lane = lane_id();
  // four operand sets of hashed bf16 values, one per accumulator, so that
  // consecutive MFMAs see different data (as a GEMM's do: the matrix cores'
  // power, and so the clock under the board's power cap, depends on it);
  // built from the lane and wave indices, which the compiler cannot fold
  const uint32_t seed = (uint32_t)(lane + 64 * (threadIdx.x / kWave) + 512 * blockIdx.x) * 2654435761u;
  u32x4 a[4], b[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h = seed ^ (uint32_t)(0x9E3779B9u * (uint32_t)(8 * c + i + 1));
      h ^= h >> 15;
      h *= 0x2C1B3C6Du;
      h ^= h >> 12;
      a[c][i] = bf16_pair(h);
      h *= 0x297A2D39u;
      h ^= h >> 15;
      b[c][i] = bf16_pair(h);
    }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[c]),
                                                       __builtin_bit_cast(bf16x8, b[c]), acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (lane == 0) sink[blockIdx.x * kMfmaWaves + threadIdx.x / kWave] = s;
}

}  // namespace

hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  const int64_t per_block = (int64_t)kCopyBlock * kCopyUnroll;
  const int64_t want = (n16 + per_block - 1) / per_block;
  const int blocks = (int)(want < 256 * 16 ? want : 256 * 16);
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kCopyBlock), 0, s, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

int probe_mfma_blocks() { return 256; }
int64_t probe_mfma_flops_per_iter() { return (int64_t)probe_mfma_blocks() * kMfmaWaves * 4 * 2 * 32 * 32 * 16; }

hipError_t launch_probe_mfma(int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_kernel, dim3(probe_mfma_blocks()), dim3(kMfmaWaves * kWave), 0, s, iters, sink);
  return hipGetLastError();
}

}  // namespace moe
