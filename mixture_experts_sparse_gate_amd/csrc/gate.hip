// Gate kernels: logits, top-k selection and gate weights.
//
// Plain gate: logits = x W_g (+ bias). Noisy gate: logits = x W_g +
// eps * softplus(x W_n) (+ bias), the noisy top-k gating of
// "MoE稀疏计算加速技术解析与应用实践" §2.1 and
// "MoE架构：稀疏激活机制如何提升模型计算效率" §2.1, with eps an input.
// Cosine gate: logits_j = cos(x P, e_j) / tau (+ bias_j); the projection x P
// runs on the grouped MFMA GEMM, this file only does the cosine, the
// selection and the weights.
//
// Selection: the k largest fp32 logits, ties to the lower expert index.
// Weights: softmax over the k selected logits (renormalised) or over all N
// (full probabilities), in fp32.
//
// The plain/noisy logits are a skinny product (N or 2N columns against
// d-long rows of x): bound by reading x from HBM, so they run on the vector
// ALUs with each wave's 64 lanes splitting d and a butterfly
// reduce-scatter across lanes, not on MFMA.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxExpertsPerLane = 4;  // N <= 256

// Top-k selection and weights for one token; every lane of the wave calls
// it with the same arguments. `lg` is the token's N logits in LDS.
__device__ void select_token(const float* lg, int N, int k, int renorm, int32_t* idx_out,
                             float* w_out) {
  const int lane = lane_id();
  float v[kMaxExpertsPerLane];
  bool valid[kMaxExpertsPerLane];
#pragma unroll
  for (int i = 0; i < kMaxExpertsPerLane; ++i) {
    const int e = lane + kWave * i;
    valid[i] = e < N;
    v[i] = valid[i] ? lg[e] : 0.f;
  }
  uint32_t taken = 0;
  int my_e = 0;
  float my_l = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      if (valid[i] && !((taken >> i) & 1u)) {
        const uint32_t e = lane + kWave * i;
        const uint64_t key = ((uint64_t)float_order_key(v[i]) << 32) | (0xFFFFFFFFu - e);
        best = key > best ? key : best;
      }
    }
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    if ((e & (kWave - 1)) == lane) taken |= 1u << (e / kWave);
    if (lane == j) {
      my_e = e;
      my_l = lg[e];
    }
  }
  const float m = __shfl(my_l, 0, kWave);  // the largest logit
  float s;
  if (renorm) {
    s = wave_sum(lane < k ? expf(my_l - m) : 0.f);
  } else {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i)
      if (valid[i]) part += expf(v[i] - m);
    s = wave_sum(part);
  }
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = expf(my_l - m) / s;
  }
}

// Top-k selection and weights for TW tokens at once (same rules as
// select_token); the TW reductions are independent, so their shuffles
// interleave instead of running back to back. lg[t] holds token t's N
// logits in LDS; tokens at or past `valid` are skipped.
template <int TW>
__device__ void select_tokens(const float (*lg)[kWave * kMaxExpertsPerLane], int valid, int N, int k,
                              int renorm, int32_t* idx_out, float* w_out) {
  const int lane = lane_id();
  float v[TW][kMaxExpertsPerLane];
  uint32_t taken[TW];
  int my_e[TW];
  float my_l[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    taken[t] = 0;
    my_e[t] = 0;
    my_l[t] = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxExpertsPerLane; ++i) {
      const int e = lane + kWave * i;
      v[t][i] = e < N ? lg[t][e] : 0.f;
    }
  }
  for (int j = 0; j < k; ++j) {
    uint64_t best[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      best[t] = 0;
#pragma unroll
      for (int i = 0; i < kMaxExpertsPerLane; ++i) {
        const uint32_t e = lane + kWave * i;
        if (e < (uint32_t)N && !((taken[t] >> i) & 1u)) {
          const uint64_t key = ((uint64_t)float_order_key(v[t][i]) << 32) | (0xFFFFFFFFu - e);
          best[t] = key > best[t] ? key : best[t];
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        const uint64_t o = shfl_xor_u64(best[t], m);
        best[t] = o > best[t] ? o : best[t];
      }
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best[t]);
      if ((e & (kWave - 1)) == lane) taken[t] |= 1u << (e / kWave);
      if (lane == j) {
        my_e[t] = e;
        my_l[t] = lg[t][e];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    if (t >= valid) break;
    const float m = __shfl(my_l[t], 0, kWave);
    float s;
    if (renorm) {
      s = wave_sum(lane < k ? expf(my_l[t] - m) : 0.f);
    } else {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxExpertsPerLane; ++i)
        if (lane + kWave * i < N) part += expf(v[t][i] - m);
      s = wave_sum(part);
    }
    if (lane < k) {
      idx_out[t * k + lane] = my_e[t];
      w_out[t * k + lane] = expf(my_l[t] - m) / s;
    }
  }
}

// In-place butterfly reduce-scatter over the 64 lanes: afterwards each lane
// holds max(V/64, 1) fully reduced values. Returns the index (in 0..V) of
// v[0]; v[i] is index + i. When V < 64, 64/V lanes hold each value.
template <int V>
__device__ inline int butterfly_reduce(float (&v)[V], int lane) {
  int base = 0;
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const int m = 32 >> s;
    const int cur = (V >> s) > 0 ? (V >> s) : 1;
    const bool hi = (lane & m) != 0;
    // bitwise blend rather than a ?: on two elements, which the compiler
    // would turn into a lane-dependent array index (and spill the array)
    const uint32_t hmask = hi ? 0xFFFFFFFFu : 0u;
    if (cur > 1) {
      const int half = cur / 2;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const uint32_t lo_b = __float_as_uint(v[i]), hi_b = __float_as_uint(v[i + half]);
        const float send = __uint_as_float((lo_b & hmask) | (hi_b & ~hmask));
        const float keep = __uint_as_float((hi_b & hmask) | (lo_b & ~hmask));
        v[i] = keep + __shfl_xor(send, m, kWave);
      }
      if (hi) base += half;
    } else {
      v[0] += __shfl_xor(v[0], m, kWave);
    }
  }
  return base;
}

__device__ inline float softplusf(float z) { return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z))); }

// Loads NCB consecutive gate-matrix elements of row dd starting at column c0
// (zeros past column N), widened to fp32.
template <typename E, int NCB>
__device__ inline void load_wrow(const E* w, int N, int dd, int c0, bool vec, float (&out)[NCB]) {
  constexpr int CE = ElemTraits<E>::kPerChunk;
  const E* row = w + (int64_t)dd * N + c0;
  if (vec) {
#pragma unroll
    for (int q = 0; q < NCB / CE; ++q) {
      const u32x4 c = load16(row + q * CE);
#pragma unroll
      for (int i = 0; i < CE; ++i) out[q * CE + i] = chunk_elem<E>(c, i);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCB; ++c)
      out[c] = (c0 + c < N) ? ElemTraits<E>::to_f32(row[c]) : 0.f;
  }
}

// Plain / noisy gate logits for a column block of NCB experts. Each wave
// owns TW tokens; lane l reduces d-chunks l, l+64, ... into TW x NV
// accumulators, then the wave reduce-scatters them. With one column block
// (gridDim.y == 1) the wave goes on to select; otherwise it writes logits
// and a separate kernel selects.
template <typename E, int TW, int NCB, bool NOISY>
__global__ __launch_bounds__(kBlock) void gate_logits_kernel(GateParams p) {
  constexpr int CE = ElemTraits<E>::kPerChunk;
  constexpr int NV = NOISY ? 2 * NCB : NCB;
  constexpr int V = TW * NV;
  __shared__ float sums[kWavesPerBlock][V];
  __shared__ float lg[kWavesPerBlock][TW][NCB];

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int t0 = (blockIdx.x * kWavesPerBlock + wave) * TW;
  const int c0 = blockIdx.y * NCB;
  const int N = p.N, d = p.d, T = p.T;
  const E* x = static_cast<const E*>(p.x);
  const E* wg = static_cast<const E*>(p.w_gate);
  const E* wn = static_cast<const E*>(p.w_noise);
  const bool vec = (N % CE == 0) && (c0 + NCB <= N);

  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;

  const int nq = d / CE;
  for (int q = lane; q < nq; q += kWave) {
    u32x4 xc[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t)
      xc[t] = (t0 + t < T) ? load16(x + (int64_t)(t0 + t) * d + q * CE) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int ii = 0; ii < CE; ++ii) {
      const int dd = q * CE + ii;
      float xe[TW];
#pragma unroll
      for (int t = 0; t < TW; ++t) xe[t] = chunk_elem<E>(xc[t], ii);
      float w[NCB];
      load_wrow<E, NCB>(wg, N, dd, c0, vec, w);
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int c = 0; c < NCB; ++c) acc[t * NV + c] += xe[t] * w[c];
      if (NOISY) {
        load_wrow<E, NCB>(wn, N, dd, c0, vec, w);
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
          for (int c = 0; c < NCB; ++c) acc[t * NV + NCB + c] += xe[t] * w[c];
      }
    }
  }

  const int base = butterfly_reduce<V>(acc, lane);
  constexpr int R = V >= kWave ? V / kWave : 1;
  constexpr int DUP = V >= kWave ? 1 : kWave / V;
  if ((lane & (DUP - 1)) == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) sums[wave][base + i] = acc[i];
  }
  __syncthreads();

  const bool fused = gridDim.y == 1;
  for (int i = lane; i < TW * NCB; i += kWave) {
    const int t = i / NCB, c = i % NCB;
    const int tok = t0 + t, col = c0 + c;
    if (tok >= T || col >= N) continue;
    float l = sums[wave][t * NV + c];
    if (NOISY) l += p.noise[(int64_t)tok * N + col] * softplusf(sums[wave][t * NV + NCB + c]);
    if (p.logit_bias) l += p.logit_bias[col];
    if (p.logits) p.logits[(int64_t)tok * N + col] = l;
    if (fused) lg[wave][t][c] = l;
  }
  if (!fused) return;
  __syncthreads();
  for (int t = 0; t < TW; ++t) {
    const int tok = t0 + t;
    if (tok >= T) break;
    select_token(lg[wave][t], N, p.k, p.renorm, p.topk_idx + (int64_t)tok * p.k,
                 p.topk_w + (int64_t)tok * p.k);
  }
}

// Selection from a logits buffer, one wave per token.
__global__ __launch_bounds__(kBlock) void gate_select_kernel(const float* __restrict__ logits,
                                                             int T, int N, int k, int renorm,
                                                             int32_t* topk_idx, float* topk_w) {
  __shared__ float lg[kWavesPerBlock][kWave * kMaxExpertsPerLane];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int tok = blockIdx.x * kWavesPerBlock + wave;
  if (tok < T)
    for (int e = lane; e < N; e += kWave) lg[wave][e] = logits[(int64_t)tok * N + e];
  __syncthreads();
  if (tok < T)
    select_token(lg[wave], N, k, renorm, topk_idx + (int64_t)tok * k, topk_w + (int64_t)tok * k);
}

// Cosine gate from the projection z = x P (fp32, [T, p], p <= 256). Experts
// are staged through LDS in groups of 64 (one per lane) with a padded row
// stride so that lanes reading different rows hit different banks; with
// N <= 64 (one group) the table and its norms are staged once per block and
// each wave then walks its own token batches without block barriers.
constexpr int kCosTW = 8;                              // tokens per wave per batch
constexpr int kCosMaxP = 256;
constexpr int kCosPad = 4;

__global__ __launch_bounds__(kBlock) void cosine_select_kernel(CosineParams p) {
  __shared__ __attribute__((aligned(16))) float zs[kWavesPerBlock][kCosTW][kCosMaxP];
  __shared__ __attribute__((aligned(16))) float es[kWave][kCosMaxP + kCosPad];
  __shared__ float lg[kWavesPerBlock][kCosTW][kWave * kMaxExpertsPerLane];
  __shared__ float enorm[kWave];

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int P = p.p, N = p.N, T = p.T;
  const int groups = (N + kWave - 1) / kWave;
  const int nbatch = (T + kCosTW - 1) / kCosTW;

  auto stage_group = [&](int g) {
    // 16-byte copies of the group's rows (P is a multiple of 8)
    const int q4 = P / 4;
    for (int i = threadIdx.x; i < kWave * q4; i += kBlock) {
      const int r = i / q4, c = (i % q4) * 4, e = g * kWave + r;
      *reinterpret_cast<f32x4*>(&es[r][c]) =
          e < N ? *reinterpret_cast<const f32x4*>(p.emb + (int64_t)e * P + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // norms: each wave takes 16 rows, lanes split the row
    for (int r = wave * (kWave / kWavesPerBlock); r < (wave + 1) * (kWave / kWavesPerBlock); ++r) {
      const int e = g * kWave + r;
      float ss = 0.f;
      if (e < N)
        for (int c = lane; c < P; c += kWave) {
          const float v = p.emb[(int64_t)e * P + c];
          ss += v * v;
        }
      ss = wave_sum(ss);
      if (lane == 0) enorm[r] = fmaxf(sqrtf(ss), 1e-12f);
    }
    __syncthreads();
  };
  if (groups == 1) stage_group(0);

  // each wave takes batches wave-major over the whole grid; with several
  // expert groups the block moves in step (the table is re-staged per group)
  const int wstride = gridDim.x * kWavesPerBlock;
  const int nb_iter = groups == 1 ? nbatch : (nbatch + wstride - 1) / wstride * wstride;
  for (int b = blockIdx.x * kWavesPerBlock + wave; b < nb_iter; b += wstride) {
    const int t0 = b * kCosTW;
    const bool live = b < nbatch;
    float (*z)[kCosMaxP] = zs[wave];
    // this wave's z rows and their norms (read only by this wave): all loads
    // first, so that they are in flight together
    constexpr int ZPL = kCosMaxP / kWave;
    float zv[kCosTW][ZPL];
#pragma unroll
    for (int t = 0; t < kCosTW; ++t)
#pragma unroll
      for (int i = 0; i < ZPL; ++i) {
        const int tok = t0 + t, c = lane + kWave * i;
        zv[t][i] = (live && tok < T && c < P) ? p.z[(int64_t)tok * P + c] : 0.f;
      }
    float zn[kCosTW];
#pragma unroll
    for (int t = 0; t < kCosTW; ++t) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < ZPL; ++i) {
        z[t][lane + kWave * i] = zv[t][i];
        ss += zv[t][i] * zv[t][i];
      }
      zn[t] = ss;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
      for (int t = 0; t < kCosTW; ++t) zn[t] += __shfl_xor(zn[t], m, kWave);
#pragma unroll
    for (int t = 0; t < kCosTW; ++t) zn[t] = fmaxf(sqrtf(zn[t]), 1e-12f);
    for (int g = 0; g < groups; ++g) {
      if (groups > 1) {
        __syncthreads();  // everyone done with the previous group
        stage_group(g);
      }
      // lane = expert of the group
      float acc[kCosTW];
#pragma unroll
      for (int t = 0; t < kCosTW; ++t) acc[t] = 0.f;
      for (int c = 0; c < P; c += 4) {
        const f32x4 ev = *reinterpret_cast<const f32x4*>(&es[lane][c]);
#pragma unroll
        for (int t = 0; t < kCosTW; ++t) {
          const f32x4 zv = *reinterpret_cast<const f32x4*>(&z[t][c]);
          acc[t] += zv[0] * ev[0] + zv[1] * ev[1] + zv[2] * ev[2] + zv[3] * ev[3];
        }
      }
      const int e = g * kWave + lane;
      if (e < N) {
        const float en = enorm[lane];
        const float bias = p.logit_bias ? p.logit_bias[e] : 0.f;
#pragma unroll
        for (int t = 0; t < kCosTW; ++t) lg[wave][t][e] = acc[t] / (zn[t] * en) * p.inv_temperature + bias;
      }
    }
    if (!live) continue;
    __builtin_amdgcn_wave_barrier();
    const int valid = min(kCosTW, T - t0);
    if (p.logits)
      for (int t = 0; t < valid; ++t)
        for (int e = lane; e < N; e += kWave) p.logits[(int64_t)(t0 + t) * N + e] = lg[wave][t][e];
    select_tokens<kCosTW>(lg[wave], valid, N, p.k, p.renorm, p.topk_idx + (int64_t)t0 * p.k,
                          p.topk_w + (int64_t)t0 * p.k);
  }
}

template <typename E, int TW, bool NOISY>
hipError_t launch_tw(const GateParams& p, hipStream_t s) {
  int ncb = 8;
  const int cap = NOISY ? 16 : 32;
  while (ncb < p.N && ncb < cap) ncb *= 2;
  const int toks_per_block = kWavesPerBlock * TW;
  dim3 grid((p.T + toks_per_block - 1) / toks_per_block, (p.N + ncb - 1) / ncb);
  if (ncb == 8)
    hipLaunchKernelGGL((gate_logits_kernel<E, TW, 8, NOISY>), grid, dim3(kBlock), 0, s, p);
  else if (ncb == 16)
    hipLaunchKernelGGL((gate_logits_kernel<E, TW, 16, NOISY>), grid, dim3(kBlock), 0, s, p);
  else if constexpr (!NOISY)  // the noisy gate caps column blocks at 16 (2 x 16 accumulators)
    hipLaunchKernelGGL((gate_logits_kernel<E, TW, 32, NOISY>), grid, dim3(kBlock), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || grid.y == 1) return err;
  dim3 g2((p.T + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(gate_select_kernel, g2, dim3(kBlock), 0, s, p.logits, p.T, p.N, p.k,
                     p.renorm, p.topk_idx, p.topk_w);
  return hipGetLastError();
}

template <typename E, bool NOISY>
hipError_t launch_e(const GateParams& p, hipStream_t s) {
  // Four tokens per wave once there are enough tokens to fill the chip.
  if (p.T >= 4096) return launch_tw<E, 4, NOISY>(p, s);
  return launch_tw<E, 1, NOISY>(p, s);
}

}  // namespace

hipError_t launch_gate_plain_noisy(const GateParams& p, bool bf16_, bool noisy, hipStream_t s) {
  if (bf16_) return noisy ? launch_e<bf16, true>(p, s) : launch_e<bf16, false>(p, s);
  return noisy ? launch_e<float, true>(p, s) : launch_e<float, false>(p, s);
}

hipError_t launch_cosine_select(const CosineParams& p, hipStream_t s) {
  const int nbatch = (p.T + kCosTW - 1) / kCosTW;
  const int want = (nbatch + kWavesPerBlock - 1) / kWavesPerBlock;
  const int grid = want < 256 ? want : 256;  // persistent: one block per CU stages the table once
  hipLaunchKernelGGL(cosine_select_kernel, dim3(grid), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
