// Gate-weighted combine: y_t = sum over the kept choices j of g_j(x_t) E_j(x_t)
// (the weighted sum of expert outputs on "MoE架构：突破单卡算力瓶颈的密钥" §1.2).
//
// One wave per token. The k rows of y_perm are read with 16-byte loads and
// accumulated in fp32 in j order, then rounded once. Dropped choices add
// nothing; a token with every choice dropped gets zeros. Row indices outside
// [0, R) are treated as dropped, so a bad row map cannot read out of bounds.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kUnroll = 8;  // 16-byte chunks per lane per pass

template <typename E>
__global__ __launch_bounds__(kBlock) void combine_kernel(CombineParams p) {
  constexpr int CE = ElemTraits<E>::kPerChunk;
  const int lane = lane_id();
  const int t = blockIdx.x * kWaves + threadIdx.x / kWave;
  if (t >= p.T) return;
  const int k = p.k, d = p.d;
  const int nchunk = d / CE;
  const E* yp = static_cast<const E*>(p.y_perm);
  E* y = static_cast<E*>(p.y) + (int64_t)t * d;
  for (int q0 = 0; q0 < nchunk; q0 += kWave * kUnroll) {
    float acc[kUnroll][CE];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int i = 0; i < CE; ++i) acc[u][i] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int row = p.row_of[t * k + j];
      if (row < 0 || row >= p.R) continue;
      const float w = p.topk_w[t * k + j];
      const E* src = yp + (int64_t)row * d;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int q = q0 + u * kWave + lane;
        if (q < nchunk) {
          const u32x4 c = load16(src + q * CE);
#pragma unroll
          for (int i = 0; i < CE; ++i) acc[u][i] += w * chunk_elem<E>(c, i);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = q0 + u * kWave + lane;
      if (q < nchunk) {
#pragma unroll
        for (int i = 0; i < CE; i += 4)
          Store<E>::four(y + q * CE + i, acc[u][i], acc[u][i + 1], acc[u][i + 2], acc[u][i + 3]);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, bool bf16_, hipStream_t s) {
  dim3 grid((p.T + kWaves - 1) / kWaves);
  if (bf16_)
    hipLaunchKernelGGL(combine_kernel<bf16>, grid, dim3(kBlock), 0, s, p);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
