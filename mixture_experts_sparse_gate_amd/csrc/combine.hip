// Gate-weighted combine: y_t = sum over the kept choices j of g_j(x_t) E_j(x_t)
// (the weighted sum of expert outputs on "MoE架构：突破单卡算力瓶颈的密钥" §1.2).
//
// One wave per token. The k rows of y_perm are read with 16-byte loads and
// accumulated in fp32 in j order (one fma per term), then rounded once. Dropped choices add
// nothing; a token with every choice dropped gets zeros. Row indices outside
// [0, R) are treated as dropped, so a bad row map cannot read out of bounds.
// For k <= 8 the wave reads its row indices and weights first and then has
// the loads of all k rows in flight at once (fewer chunks per pass as k
// grows); larger k takes one row after the other.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;

// the chunk's CE values, fp32 -> one 16-byte store
template <typename E> __device__ inline void store_chunk(E* dst, const float* v);
template <> __device__ inline void store_chunk<float>(float* dst, const float* v) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}
template <> __device__ inline void store_chunk<bf16>(bf16* dst, const float* v) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4*>(dst) = w;
}

// KB > 0: k <= KB, every row's loads of a pass in flight together; KB == 0: any k
template <typename E, int KB>
__global__ __launch_bounds__(kBlock) void combine_kernel(CombineParams p) {
  constexpr int CE = ElemTraits<E>::kPerChunk;
  constexpr int U = KB == 0 ? 8 : KB <= 2 ? 8 : KB <= 4 ? 4 : 2;  // 16-byte chunks per lane per pass
  constexpr int NB = KB == 0 ? 1 : KB;                             // rows in flight
  const int lane = lane_id();
  const int t = blockIdx.x * kWaves + threadIdx.x / kWave;
  if (t >= p.T) return;
  const int k = p.k, d = p.d;
  const int nchunk = d / CE;
  const E* yp = static_cast<const E*>(p.y_perm);
  E* y = static_cast<E*>(p.y) + (int64_t)t * d;
  int rows[NB];
  float wts[NB];
  if constexpr (KB > 0) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int r = j < k ? p.row_of[t * k + j] : -1;
      rows[j] = r >= 0 && r < p.R ? r : -1;
      wts[j] = j < k ? p.topk_w[t * k + j] : 0.f;
    }
  }
  for (int q0 = 0; q0 < nchunk; q0 += kWave * U) {
    float acc[U][CE];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < CE; ++i) acc[u][i] = 0.f;
    const int jn = KB > 0 ? 1 : k;  // rounds of NB rows
    for (int jr = 0; jr < jn; ++jr) {
      if constexpr (KB == 0) {
        const int r = p.row_of[t * k + jr];
        rows[0] = r >= 0 && r < p.R ? r : -1;
        wts[0] = p.topk_w[t * k + jr];
      }
      u32x4 c[NB][U];
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = q0 + u * kWave + lane;
          c[j][u] = rows[j] >= 0 && q < nchunk ? load16(yp + (int64_t)rows[j] * d + q * CE) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (rows[j] < 0) continue;  // wave-uniform
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int i = 0; i < CE; ++i) acc[u][i] = __builtin_fmaf(wts[j], chunk_elem<E>(c[j][u], i), acc[u][i]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u * kWave + lane;
      if (q < nchunk) store_chunk<E>(y + q * CE, acc[u]);
    }
  }
}

template <typename E>
void launch_e(const CombineParams& p, dim3 grid, hipStream_t s) {
  if (p.k <= 2) hipLaunchKernelGGL((combine_kernel<E, 2>), grid, dim3(kBlock), 0, s, p);
  else if (p.k <= 4) hipLaunchKernelGGL((combine_kernel<E, 4>), grid, dim3(kBlock), 0, s, p);
  else if (p.k <= 8) hipLaunchKernelGGL((combine_kernel<E, 8>), grid, dim3(kBlock), 0, s, p);
  else hipLaunchKernelGGL((combine_kernel<E, 0>), grid, dim3(kBlock), 0, s, p);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, bool bf16_, hipStream_t s) {
  dim3 grid((p.T + kWaves - 1) / kWaves);
  if (bf16_)
    launch_e<bf16>(p, grid, s);
  else
    launch_e<float>(p, grid, s);
  return hipGetLastError();
}

}  // namespace moe
