// Load-balance terms of a routing: the load each expert receives from the
// gate (the column sums of the sparse gate matrix, before capacity drops:
// gate_output.sum(dim=0) on "MoE架构：突破单卡算力瓶颈的密钥" §3.1 and
// gates.sum(dim=0) on "MoE稀疏计算加速技术解析与应用实践" §4.1) and the two
// losses those pages define on it.
//
// Every sum runs in a fixed order, so the results are the same bits on every
// call: a block adds its 256 tokens' choices in (token, choice) order, split
// into G consecutive ranges whose sums are then added in range order; the
// final kernel adds the blocks' sums in block order the same way.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kAuxThreads = 256;
constexpr int kAuxMaxK = 32;  // k <= 32 (checked by the C ABI)

// G ranges per expert: as many as the block's threads allow (N <= 256)
__device__ inline int aux_ranges(int N) { return max(1, kAuxThreads / N); }

__global__ __launch_bounds__(kAuxThreads) void aux_partial_kernel(AuxParams p) {
  __shared__ int si[kAuxTok * kAuxMaxK];
  __shared__ float sw[kAuxTok * kAuxMaxK];
  __shared__ float part[kAuxThreads];  // [G][N], G * N <= 256
  const int tid = threadIdx.x, N = p.N, G = aux_ranges(N);
  const int t0 = blockIdx.x * kAuxTok;
  const int n = min(kAuxTok, p.T - t0) * p.k;  // the block's choices
  const int64_t base = (int64_t)t0 * p.k;
  for (int i0 = 0; i0 < n; i0 += 4 * kAuxThreads) {  // four loads of each array in flight per thread
    int vi[4];
    float vw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kAuxThreads + tid;
      vi[u] = i < n ? p.topk_idx[base + i] : 0;
      vw[u] = i < n ? p.topk_w[base + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kAuxThreads + tid;
      if (i < n) {
        si[i] = vi[u];
        sw[i] = vw[u];
      }
    }
  }
  __syncthreads();
  // thread (expert e, range g); weights are >= 0, so adding 0 for another
  // expert's choice leaves the sum's bits unchanged
  const int e = tid % N, g = tid / N;
  if (g < G) {
    const int lo = (int)((int64_t)n * g / G), hi = (int)((int64_t)n * (g + 1) / G);
    float s = 0.f;
    int i = lo;
    for (; i + 8 <= hi; i += 8) {  // eight entries' LDS reads in flight, added in order
      int ii[8];
      float ww[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ii[u] = si[i + u];
        ww[u] = sw[i + u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) s += ii[u] == e ? ww[u] : 0.f;
    }
    for (; i < hi; ++i) s += si[i] == e ? sw[i] : 0.f;
    part[g * N + e] = s;
  }
  __syncthreads();
  if (tid < N) {
    float s = 0.f;
    for (int r = 0; r < G; ++r) s += part[r * N + tid];
    p.partial[(int64_t)blockIdx.x * N + tid] = s;
  }
}

__global__ __launch_bounds__(kAuxThreads) void aux_final_kernel(AuxParams p, int nb) {
  __shared__ float part[kAuxThreads];
  __shared__ float imp[kAuxThreads];  // N <= 256
  const int tid = threadIdx.x, N = p.N, G = aux_ranges(N);
  const int e = tid % N, g = tid / N;
  if (g < G) {
    const int lo = (int)((int64_t)nb * g / G), hi = (int)((int64_t)nb * (g + 1) / G);
    float s = 0.f;
    int b = lo;
    for (; b + 8 <= hi; b += 8) {  // eight loads in flight, added in block order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = p.partial[(int64_t)(b + u) * N + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < hi; ++b) s += p.partial[(int64_t)b * N + e];
    part[g * N + e] = s;
  }
  __syncthreads();
  if (tid < N) {
    float s = 0.f;
    for (int r = 0; r < G; ++r) s += part[r * N + tid];
    imp[tid] = s;
    if (p.importance) p.importance[tid] = s;
  }
  __syncthreads();
  if (tid == 0 && p.losses) {
    float sum = 0.f;
    for (int i = 0; i < N; ++i) sum += imp[i];
    const float mean = sum / (float)N;
    float sq = 0.f;
    for (int i = 0; i < N; ++i) {
      const float dv = mean - imp[i];
      sq = fmaf(dv, dv, sq);
    }
    p.losses[0] = sq;                                // sum of squared deviations from the mean
    p.losses[1] = 0.1f * sqrtf(sq / (float)(N - 1));  // 0.1 std, N - 1 denominator (N = 1: 0/0, NaN)
  }
}

}  // namespace

int aux_blocks(int64_t T) { return (int)((T + kAuxTok - 1) / kAuxTok); }

hipError_t launch_aux_loss(const AuxParams& p, hipStream_t s) {
  const int nb = aux_blocks(p.T);
  hipLaunchKernelGGL(aux_partial_kernel, dim3(nb), dim3(kAuxThreads), 0, s, p);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(kAuxThreads), 0, s, p, nb);
  return hipGetLastError();
}

}  // namespace moe
