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
// The plain/noisy logits are the product x [W_g | W_n], skinny (N or 2N
// columns against d-long rows of x) and bound by reading x. In bf16 it runs
// on MFMA (32x32x16): blocks of four waves take 32 tokens and 32 columns over
// a K slice, each wave a quarter of it, with the gate matrices' slice staged
// in LDS and read back transposed (ds_read_b64_tr_b16); the waves' sums add
// up in LDS and K slices (only as many as it takes to fill the chip) add up
// in fixed order in the selection kernel, so the logits are deterministic.
// The fp32 build keeps a vector-ALU kernel: each wave's 64 lanes split d and
// a butterfly reduce-scatter across lanes sums them.
#include <algorithm>

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
    __syncthreads();
    // norms from the staged rows (zeros past N): four threads per row
    {
      const int r = threadIdx.x / 4, qd = threadIdx.x % 4;
      float ss = 0.f;
      for (int c = qd; c < P; c += 4) ss = fmaf(es[r][c], es[r][c], ss);
      ss += __shfl_xor(ss, 1, kWave);
      ss += __shfl_xor(ss, 2, kWave);
      if (qd == 0) enorm[r] = fmaxf(sqrtf(ss), 1e-12f);
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

// Cosine gate for N <= 64 experts and p <= 256, 64 tokens per block. The
// block stages its z rows and the expert table in LDS (every load in flight
// at once), takes the norms from there, computes the 64 x N dot products on
// the fp32 MFMA (one 32-token x 32-expert tile per wave, over all of p), and
// selects with four lanes per token. Logits are acc / (|z| |e|) / tau + bias
// as in the general kernel above.
constexpr int kCgTok = 64;
constexpr int kCgMaxN = 64;
constexpr int kCgMaxP = 256;
constexpr int kCgStride = kCgMaxP + 4;  // floats per staged row: 16-byte row reads spread over the banks
constexpr int kCgLg = kCgMaxN + 1;      // floats per logit row

__global__ __launch_bounds__(kBlock) void cosine_gate_kernel(CosineParams p) {
  __shared__ __attribute__((aligned(16))) float zt[kCgTok * kCgStride];
  __shared__ __attribute__((aligned(16))) float et[kCgMaxN * kCgStride];
  __shared__ float lg[kCgTok * kCgLg];
  __shared__ float zn[kCgTok], en[kCgMaxN];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int P = p.p, N = p.N, T = p.T;
  const int t0 = blockIdx.x * kCgTok;

  // ---- staging: 16-byte pieces, row r = 4 j + tid / 64, piece tid % 64
  // (pieces past p, rows past T or N are zeros)
  constexpr int J = kCgTok * (kCgMaxP / 4) / kBlock;
  static_assert(kCgTok == kCgMaxN && J * kBlock == kCgTok * (kCgMaxP / 4), "staging shape");
  const int c4 = tid % (kCgMaxP / 4);
  const bool col_ok = 4 * c4 < P;
  f32x4 zv[J], ev[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int r = j * (kBlock / (kCgMaxP / 4)) + tid / (kCgMaxP / 4);
    zv[j] = col_ok && t0 + r < T ? *reinterpret_cast<const f32x4*>(p.z + (int64_t)(t0 + r) * P + 4 * c4)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
    ev[j] = col_ok && r < N ? *reinterpret_cast<const f32x4*>(p.emb + (int64_t)r * P + 4 * c4)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int r = j * (kBlock / (kCgMaxP / 4)) + tid / (kCgMaxP / 4);
    if (col_ok) {
      *reinterpret_cast<f32x4*>(&zt[r * kCgStride + 4 * c4]) = zv[j];
      *reinterpret_cast<f32x4*>(&et[r * kCgStride + 4 * c4]) = ev[j];
    }
  }
  __syncthreads();

  // ---- norms: four threads per row, summed over the quad
  {
    const int r = tid / 4, qd = tid % 4;
    float sz = 0.f, se = 0.f;
    for (int c = qd; c < P; c += 4) {
      const float a = zt[r * kCgStride + c], b = et[r * kCgStride + c];
      sz = fmaf(a, a, sz);
      se = fmaf(b, b, se);
    }
    sz += __shfl_xor(sz, 1, kWave);
    sz += __shfl_xor(sz, 2, kWave);
    se += __shfl_xor(se, 1, kWave);
    se += __shfl_xor(se, 2, kWave);
    if (qd == 0) {
      zn[r] = fmaxf(sqrtf(sz), 1e-12f);
      en[r] = fmaxf(sqrtf(se), 1e-12f);
    }
  }
  __syncthreads();

  // ---- dots: wave w takes tokens 32 (w % 2) .. and experts 32 (w / 2) ..
  // One MFMA step multiplies k pair {c + i, c + 4 + i} (lane half h brings
  // k = c + 4h + i of its row), so each lane reads 16 bytes per 4 steps.
  // The lane ends up with token tt*32 + lane%32 and experts
  // eb + 8(r/4) + 4(lane/32) + r%4 of its 16 accumulators.
  {
    const int tt = wave & 1, eb = (wave >> 1) * 32;
    if (eb < N) {
      const int row = lane & 31, h = lane >> 5;
      const float* za = &zt[(tt * 32 + row) * kCgStride + 4 * h];
      const float* ea = &et[(eb + row) * kCgStride + 4 * h];
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      for (int c = 0; c < P; c += 8) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(ea + c);
        const f32x4 b = *reinterpret_cast<const f32x4*>(za + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], acc, 0, 0, 0);
      }
      const int t = tt * 32 + row;
      const float znt = zn[t];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = eb + 8 * (r >> 2) + 4 * h + (r & 3);
        if (e < N) {
          const float bias = p.logit_bias ? p.logit_bias[e] : 0.f;
          lg[t * kCgLg + e] = acc[r] / (znt * en[e]) * p.inv_temperature + bias;
        }
      }
    }
  }
  __syncthreads();
  if (p.logits)
    for (int i = tid; i < kCgTok * N; i += kBlock) {
      const int t = i / N, e = i % N;
      if (t0 + t < T) p.logits[(int64_t)(t0 + t) * N + e] = lg[t * kCgLg + e];
    }

  // ---- selection: four lanes per token, lane q holding experts 16q .. 16q+15.
  // Keys are (logit order, inverted index), so the largest key is the largest
  // logit with ties to the lower index; the j-th winner is the largest key
  // below the (j-1)-th.
  const int tq = tid >> 2, qd = tid & 3, tok = t0 + tq;
  const float* lrow = &lg[tq * kCgLg];
  uint64_t key[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = 16 * qd + i;
    key[i] = e < N ? ((uint64_t)float_order_key(lrow[e]) << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0ull;
  }
  auto next_below = [&](uint64_t below) {
    uint64_t b = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) b = key[i] < below && key[i] > b ? key[i] : b;
    uint64_t o = shfl_xor_u64(b, 1);
    b = o > b ? o : b;
    o = shfl_xor_u64(b, 2);
    return o > b ? o : b;
  };
  auto expert_of = [](uint64_t kk) { return (int)(0xFFFFFFFFu - (uint32_t)kk); };
  const float m = lrow[expert_of(next_below(~0ull))];  // the largest logit
  float s = 0.f;
  if (!p.renorm) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * qd + i < N) s += expf(lrow[16 * qd + i] - m);
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
  } else {
    uint64_t b = ~0ull;
    for (int j = 0; j < p.k; ++j) {
      b = next_below(b);
      s += expf(lrow[expert_of(b)] - m);
    }
  }
  uint64_t b = ~0ull;
  for (int j = 0; j < p.k; ++j) {
    b = next_below(b);
    if (tok < T && (j & 3) == qd) {
      const int e = expert_of(b);
      p.topk_idx[(int64_t)tok * p.k + j] = e;
      p.topk_w[(int64_t)tok * p.k + j] = expf(lrow[e] - m) / s;
    }
  }
}

// ---- bf16 plain / noisy gate product on MFMA
constexpr int kGtTok = 32;          // tokens per block (one MFMA tile)
constexpr int kGtCols = 32;         // columns per chunk
constexpr int kGtWaves = 4;         // waves per block, splitting the block's K slice
constexpr int kGtMaxKr = 1024;      // K per slice at most: LDS rows of 64 bytes -> 64 KiB
constexpr int kGtTargetBlocks = 256;

struct GatePartialParams {
  const bf16* x;
  const bf16* wg;
  const bf16* wn;
  float* partial;  // [ks][T][ncc * 32]
  int T, d, N, NC, ncp, kr;
  bool vec;        // N % 8 == 0: 8 consecutive columns lie in one matrix, 16-byte aligned
};

// partial[z][t][c0 + c] = sum over k in slice z of x[t][k] * Wc[k][c0 + c],
// Wc = [W_g | W_n] (columns past NC read as zeros). Grid: (token tiles,
// column chunks, K slices); wave w covers quarter w of the slice.
__global__ __launch_bounds__(kGtWaves * kWave) void gate_partial_kernel(GatePartialParams p) {
  __shared__ __attribute__((aligned(1024))) char wl[kGtMaxKr * kGtCols * 2];
  __shared__ __attribute__((aligned(16))) float red[kGtWaves][kGtTok][kGtCols];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kGtTok;
  const int c0 = blockIdx.y * kGtCols;
  const int k_lo = blockIdx.z * p.kr;
  const int nk = min(p.kr, p.d - k_lo);  // > 0: every slice starts inside d
  const int krw = p.kr / kGtWaves;       // multiple of 16

  // stage the slice's gate rows: row kk (k = k_lo + kk) as 32 bf16 columns,
  // 64 bytes, zeros past d and past NC
  for (int gi = threadIdx.x; gi < p.kr * 4; gi += kGtWaves * kWave) {
    const int kk = gi >> 2, col = c0 + 8 * (gi & 3);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (kk < nk && col < p.NC) {
      const int64_t k = k_lo + kk;
      if (p.vec) {
        v = col < p.N ? load16(p.wg + k * p.N + col) : load16(p.wn + k * p.N + (col - p.N));
      } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = col + e;
          const bf16* src = c < p.N ? p.wg + k * p.N + c : p.wn + k * p.N + (c - p.N);
          h[e] = c < p.NC ? (uint32_t)__builtin_bit_cast(uint16_t, *src) : 0u;
        }
        v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      }
    }
    store16(wl + gi * 16, v);
  }
  __syncthreads();

  // this wave: rows [wave * krw, wave * krw + krw) of the slice
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int q16 = lane >> 4, r16 = lane & 15;
  // x fragment: token t0 + lrow, 8 K values from k_lo + kk + 8 lhalf; rows past T
  // read zeros through the descriptor's range, K past d is masked below
  const int rows = min(kGtTok, p.T - t0);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x + (int64_t)t0 * p.d, (uint32_t)((int64_t)rows * p.d * 2));
  const int xoff = (lrow * p.d + k_lo + 8 * lhalf) * 2;
  // gate fragment (transposing read): 16-lane group q, lane r: rows 8(q/2) + 4j + r/4
  // of the 16-K step, columns 16(q%2) + 4(r%4) .. +3
  const int woff = (8 * (q16 >> 1) + (r16 >> 2)) * 64 + 32 * (q16 & 1) + 8 * (r16 & 3);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int kw0 = wave * krw, kw1 = min(kw0 + krw, nk);
  constexpr int U = 4;
  for (int kk = kw0; kk < kw1; kk += 16 * U) {
    u32x4 xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kk + 16 * u;
      // a 16-K step past the wave's rows, or the half of one past d, reads nothing
      xv[u] = (k + 8 * lhalf < kw1) ? __builtin_amdgcn_raw_buffer_load_b128(xr, xoff + k * 2, 0, 0)
                                     : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kk + 16 * u;
      if (k >= kw1) break;
      const char* w = wl + k * 64 + woff;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)w);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(w + 4 * 64));
      const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
      const u32x4 wf = u32x4{a[0], a[1], b[0], b[1]};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wf),
                                                    __builtin_bit_cast(bf16x8, xv[u]), acc, 0, 0, 0);
    }
  }
  // lane holds token lrow, columns 8(r/4) + 4 lhalf + r%4
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<f32x4*>(&red[wave][lrow][8 * g + 4 * lhalf]) =
        f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
  __syncthreads();
  // the four quarters, added in order; 256 threads x 4 columns
  const int tt = threadIdx.x >> 3, cc = (threadIdx.x & 7) * 4;
  if (t0 + tt < p.T) {
    f32x4 v = *reinterpret_cast<const f32x4*>(&red[0][tt][cc]);
#pragma unroll
    for (int w = 1; w < kGtWaves; ++w) v += *reinterpret_cast<const f32x4*>(&red[w][tt][cc]);
    *reinterpret_cast<f32x4*>(p.partial + ((int64_t)blockIdx.z * p.T + t0 + tt) * p.ncp + c0 + cc) = v;
  }
}

// Logits from the K slices' partial products (added in slice order), then
// selection; one wave per token, lanes over the columns.
template <bool NOISY>
__global__ __launch_bounds__(kBlock) void gate_finish_kernel(const float* __restrict__ partial, int ks,
                                                             int ncp, GateParams p) {
  __shared__ float lg[kWavesPerBlock][kWave * kMaxExpertsPerLane];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int tok = blockIdx.x * kWavesPerBlock + wave;
  if (tok >= p.T) return;  // no block barrier below
  const int N = p.N;
  const int64_t slice = (int64_t)p.T * ncp;
  const float* src = partial + (int64_t)tok * ncp;
  // slices added in order, eight loads in flight at a time
  auto sum_slices = [&](int c) {
    float l = src[c];
    int z = 1;
    for (; z + 8 <= ks; z += 8) {
      float t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = src[(z + i) * slice + c];
#pragma unroll
      for (int i = 0; i < 8; ++i) l += t[i];
    }
    for (; z < ks; ++z) l += src[z * slice + c];
    return l;
  };
  for (int c = lane; c < N; c += kWave) {
    float l = sum_slices(c);
    if (NOISY) l += p.noise[(int64_t)tok * N + c] * softplusf(sum_slices(N + c));
    if (p.logit_bias) l += p.logit_bias[c];
    if (p.logits) p.logits[(int64_t)tok * N + c] = l;
    lg[wave][c] = l;
  }
  // the wave reads back what its own lanes wrote: LDS keeps one wave's
  // operations in order, the compiler keeps their program order
  select_token(lg[wave], N, p.k, p.renorm, p.topk_idx + (int64_t)tok * p.k, p.topk_w + (int64_t)tok * p.k);
}

// One kernel for gates of at most 32 logit columns (N <= 32 plain, N <= 16
// noisy): 32 tokens per block, the 8 waves splitting d. Each wave stages its
// own gate rows (128 at a time) in its own LDS region and runs them through
// the MFMA; the waves' sums add up in LDS in wave order, then the block
// forms the logits and selects for its 32 tokens. NCG: 8-column groups of
// the logit columns that hold gate columns (the rest of each staged row is
// left as it is: it only feeds output columns that are never read).
constexpr int kGfWaves = 8;
constexpr int kGfRows = 128;
// a wave whose slice of d has at most this many 128-row chunks (NCG <= 2)
// issues all of its loads before its first MFMA
constexpr int kGfMaxChunks = 4;
static_assert(kGtTok * kGtCols % (kGfWaves * kWave) == 0, "logit entries per thread");

template <bool NOISY, int NCG>
__global__ __launch_bounds__(kGfWaves * kWave) void gate_fused_kernel(GatePartialParams q, int krw,
                                                                       GateParams p) {
  __shared__ __attribute__((aligned(1024))) char wl[kGfWaves][kGfRows * kGtCols * 2];
  __shared__ __attribute__((aligned(16))) float red[kGfWaves][kGtTok][kGtCols];
  __shared__ int hs[kGtCols];  // the block's choices per expert, for the dispatch
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kGtTok;
  if (threadIdx.x < kGtCols) hs[threadIdx.x] = 0;  // read after the barriers below
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int q16 = lane >> 4, r16 = lane & 15;
  const int rows = min(kGtTok, q.T - t0);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(q.x + (int64_t)t0 * q.d, (uint32_t)((int64_t)rows * q.d * 2));
  const int xoff = (lrow * q.d + 8 * lhalf) * 2;
  const int woff = (8 * (q16 >> 1) + (r16 >> 2)) * 64 + 32 * (q16 & 1) + 8 * (r16 & 3);
  char* const mine = wl[wave];
  const uint32_t wbytes = (uint32_t)((int64_t)q.d * q.N * 2);
  const __amdgpu_buffer_rsrc_t wgr = make_rsrc(q.wg, wbytes);
  const __amdgpu_buffer_rsrc_t wnr = make_rsrc(q.wn, wbytes);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // the noise and bias each thread adds to its logits below, loaded now so
  // that they arrive while the product runs (32 tokens x N <= 32 columns:
  // at most two entries per thread)
  constexpr int kPre = kGtTok * kGtCols / (kGfWaves * kWave);
  float pre_noise[kPre], pre_bias[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int i = threadIdx.x + j * kGfWaves * kWave;
    const int t = i / p.N, c = i % p.N;
    const bool ok = i < kGtTok * p.N && t0 + t < p.T;
    pre_noise[j] = NOISY && ok ? p.noise[(int64_t)(t0 + t) * p.N + c] : 0.f;
    pre_bias[j] = p.logit_bias && ok ? p.logit_bias[c] : 0.f;
  }
  const int kw0 = wave * krw, kw1 = min(kw0 + krw, q.d);
  constexpr int U = kGfRows / 16;           // 16-K steps per chunk
  constexpr int G = kGfRows * NCG / kWave;  // 16-byte gate granules per lane per chunk
  static_assert(NCG >= 1 && NCG <= kGtCols / 8 && G >= 1, "column groups");
  // one chunk's x fragments and gate rows; an offset past a descriptor's
  // range reads zeros (x past the wave's rows; gate granules of the other
  // matrix, past NC or past the wave's rows), so chunks past the end load
  // nothing but zeros
  auto load_chunk = [&](int kc, u32x4 (&xd)[U], u32x4 (&wd)[G]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kc + 16 * u;
      xd[u] = __builtin_amdgcn_raw_buffer_load_b128(xr, (k + 8 * lhalf < kw1) ? xoff + k * 2 : (int)kOutOfRange, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int gi = i * kWave + lane;
      const int kk = gi / NCG, col = 8 * (gi % NCG);
      const bool row_ok = kc + kk < kw1;
      const uint32_t row = (uint32_t)(kc + kk) * q.N;
      const uint32_t og = (row_ok && col < q.N) ? (row + col) * 2u : kOutOfRange;
      const uint32_t on = (row_ok && col >= q.N && col < q.NC) ? (row + col - q.N) * 2u : kOutOfRange;
      wd[i] = __builtin_amdgcn_raw_buffer_load_b128(wgr, (int)og, 0, 0);
      if (NOISY) wd[i] |= __builtin_amdgcn_raw_buffer_load_b128(wnr, (int)on, 0, 0);
    }
  };
  auto mfma_chunk = [&](const u32x4 (&xd)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const char* w = mine + 16 * u * 64 + woff;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)w);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(w + 4 * 64));
      const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
      const u32x4 wf = u32x4{a[0], a[1], b[0], b[1]};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wf),
                                                    __builtin_bit_cast(bf16x8, xd[u]), acc, 0, 0, 0);
    }
  };
  // granule i of this lane: its place in the wave's staged rows (row of
  // 64 bytes, 16-byte column group)
  auto stage_gate = [&](const u32x4 (&wd)[G]) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int gi = i * kWave + lane;
      store16(mine + ((gi / NCG) * 4 + gi % NCG) * 16, wd[i]);
    }
  };
  const int nch = (kw1 - kw0 + kGfRows - 1) / kGfRows;  // the wave's chunks (<= 0: none)
  if (NCG <= 2 && q.vec && nch <= kGfMaxChunks) {
    // every chunk's x fragments and gate rows requested at once, then
    // staged and multiplied chunk by chunk (one round trip per wave instead
    // of one per chunk)
    u32x4 xa[kGfMaxChunks][U], wa[kGfMaxChunks][G];
#pragma unroll
    for (int c = 0; c < kGfMaxChunks; ++c)
      if (c < nch) load_chunk(kw0 + c * kGfRows, xa[c], wa[c]);
#pragma unroll
    for (int c = 0; c < kGfMaxChunks; ++c)
      if (c < nch) {
        stage_gate(wa[c]);
        mfma_chunk(xa[c]);
      }
  } else if (q.vec) {
    // steps past the wave's rows meet zero rows and zero x: they add nothing
    u32x4 xv[U], wv[G];
    load_chunk(kw0, xv, wv);
    for (int kc = kw0; kc < kw1; kc += kGfRows) {
      u32x4 xn[U], wn[G];
      load_chunk(kc + kGfRows, xn, wn);  // in flight while this chunk computes
      stage_gate(wv);
      mfma_chunk(xv);
#pragma unroll
      for (int u = 0; u < U; ++u) xv[u] = xn[u];
#pragma unroll
      for (int i = 0; i < G; ++i) wv[i] = wn[i];
    }
  } else {
    for (int kc = kw0; kc < kw1; kc += kGfRows) {
      u32x4 xv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = kc + 16 * u;
        xv[u] = __builtin_amdgcn_raw_buffer_load_b128(xr, (k + 8 * lhalf < kw1) ? xoff + k * 2 : (int)kOutOfRange, 0, 0);
      }
      for (int gi = lane; gi < kGfRows * NCG; gi += kWave) {
        const int kk = gi / NCG, col = 8 * (gi % NCG);
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = col + e;
          const int64_t k = kc + kk;
          const bf16* src = c < q.N ? q.wg + k * q.N + c : q.wn + k * q.N + (c - q.N);
          h[e] = (kc + kk < kw1 && c < q.NC) ? (uint32_t)__builtin_bit_cast(uint16_t, *src) : 0u;
        }
        store16(mine + (kk * 4 + gi % NCG) * 16,
                u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
      }
      mfma_chunk(xv);
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<f32x4*>(&red[wave][lrow][8 * g + 4 * lhalf]) =
        f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
  __syncthreads();
  // logits of the block's tokens (waves' sums in wave order), into LDS rows
  // of 256 floats for the selection (the gate-row area is free now)
  constexpr int kLg = kGtCols + 1;  // floats per logit row
  float* const lg = reinterpret_cast<float*>(&wl[0][0]);
  const int N = p.N;
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int i = threadIdx.x + j * kGfWaves * kWave;
    const int t = i / N, c = i % N, tok = t0 + t;
    if (i >= kGtTok * N || tok >= p.T) continue;
    float l = red[0][t][c];
#pragma unroll
    for (int w = 1; w < kGfWaves; ++w) l += red[w][t][c];
    if (NOISY) {
      float u = red[0][t][N + c];
#pragma unroll
      for (int w = 1; w < kGfWaves; ++w) u += red[w][t][N + c];
      l += pre_noise[j] * softplusf(u);
    }
    if (p.logit_bias) l += pre_bias[j];
    if (p.logits) p.logits[(int64_t)tok * N + c] = l;
    lg[t * kLg + c] = l;
  }
  __syncthreads();
  // selection: eight lanes per token on waves 0-3, lane q of a group holding
  // experts 4q .. 4q+3. Keys are (logit order, inverted index): the largest
  // key is the largest logit with ties to the lower index, and the j-th
  // winner is the largest key below the (j-1)-th.
  const int tid = threadIdx.x;
  if (tid < kGtTok * 8) {  // wave-uniform
    const int tq = tid >> 3, q = tid & 7, tok = t0 + tq;
    const float* lrow = lg + tq * kLg;
    uint64_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * q + i;
      key[i] = e < N ? ((uint64_t)float_order_key(lrow[e]) << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0ull;
    }
    auto next_below = [&](uint64_t below) {
      uint64_t b = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) b = key[i] < below && key[i] > b ? key[i] : b;
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) {
        const uint64_t o = shfl_xor_u64(b, m);
        b = o > b ? o : b;
      }
      return b;
    };
    auto expert_of = [](uint64_t kk) { return (int)(0xFFFFFFFFu - (uint32_t)kk); };
    const float m = lrow[expert_of(next_below(~0ull))];  // the largest logit
    float s = 0.f;
    if (!p.renorm) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < N) s += expf(lrow[4 * q + i] - m);
#pragma unroll
      for (int mm = 1; mm < 8; mm <<= 1) s += __shfl_xor(s, mm, kWave);
    } else {
      uint64_t b = ~0ull;
      for (int j = 0; j < p.k; ++j) {
        b = next_below(b);
        s += expf(lrow[expert_of(b)] - m);
      }
    }
    uint64_t b = ~0ull;
    for (int j = 0; j < p.k; ++j) {
      b = next_below(b);
      if (tok < p.T && (j & 7) == q) {
        const int e = expert_of(b);
        p.topk_idx[(int64_t)tok * p.k + j] = e;
        p.topk_w[(int64_t)tok * p.k + j] = expf(lrow[e] - m) / s;
        if (p.hist) atomicAdd(&hs[e], 1);
      }
    }
  }
  if (p.hist) {
    __syncthreads();
    if (tid < N) p.hist[(int64_t)blockIdx.x * N + tid] = hs[tid];
  }
}

hipError_t launch_gate_bf16(const GateParams& p, bool noisy, hipStream_t s) {
  GatePartialParams g{};
  g.x = static_cast<const bf16*>(p.x);
  g.wg = static_cast<const bf16*>(p.w_gate);
  g.wn = static_cast<const bf16*>(noisy ? p.w_noise : p.w_gate);
  g.partial = p.partial;
  g.T = p.T;
  g.d = p.d;
  g.N = p.N;
  g.NC = noisy ? 2 * p.N : p.N;
  g.vec = p.N % 8 == 0;
  if (g.NC <= kGtCols) {
    // one kernel: each wave takes a multiple of 16 of d
    const int krw = ((p.d + kGfWaves - 1) / kGfWaves + 15) / 16 * 16;
    const dim3 grid((p.T + kGtTok - 1) / kGtTok);
    const dim3 block(kGfWaves * kWave);
    const int ncg = (g.NC + 7) / 8;
    if (noisy) {
      if (ncg <= 2)
        hipLaunchKernelGGL((gate_fused_kernel<true, 2>), grid, block, 0, s, g, krw, p);
      else
        hipLaunchKernelGGL((gate_fused_kernel<true, 4>), grid, block, 0, s, g, krw, p);
    } else {
      if (ncg <= 1)
        hipLaunchKernelGGL((gate_fused_kernel<false, 1>), grid, block, 0, s, g, krw, p);
      else if (ncg <= 2)
        hipLaunchKernelGGL((gate_fused_kernel<false, 2>), grid, block, 0, s, g, krw, p);
      else
        hipLaunchKernelGGL((gate_fused_kernel<false, 4>), grid, block, 0, s, g, krw, p);
    }
    return hipGetLastError();
  }
  const GateSplit sp = gate_split(p.T, p.d, p.N, noisy);
  g.ncp = sp.ncc * kGtCols;
  g.kr = sp.kr;
  const dim3 grid((p.T + kGtTok - 1) / kGtTok, sp.ncc, sp.ks);
  hipLaunchKernelGGL(gate_partial_kernel, grid, dim3(kGtWaves * kWave), 0, s, g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g2((p.T + kWavesPerBlock - 1) / kWavesPerBlock);
  if (noisy)
    hipLaunchKernelGGL((gate_finish_kernel<true>), g2, dim3(kBlock), 0, s, p.partial, sp.ks, g.ncp, p);
  else
    hipLaunchKernelGGL((gate_finish_kernel<false>), g2, dim3(kBlock), 0, s, p.partial, sp.ks, g.ncp, p);
  return hipGetLastError();
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

static_assert(kGtTok == kGateHistTokens, "the gate's histogram blocks");

}  // namespace

bool gate_writes_hist(bool bf16_, bool noisy, int N) { return bf16_ && (noisy ? 2 * N : N) <= kGtCols; }

GateSplit gate_split(int64_t T, int d, int N, bool noisy) {
  GateSplit sp{};
  const int NC = noisy ? 2 * N : N;
  sp.ncc = (NC + kGtCols - 1) / kGtCols;
  const int64_t tiles = (T + kGtTok - 1) / kGtTok;
  // as many K slices as it takes to reach ~kGtTargetBlocks blocks, each at
  // least 64 deep and at most kGtMaxKr
  const int64_t want = (kGtTargetBlocks + tiles * sp.ncc - 1) / (tiles * sp.ncc);
  const int lo = (d + kGtMaxKr - 1) / kGtMaxKr, hi = (d + 63) / 64;
  const int ks = (int)std::min<int64_t>(std::max<int64_t>(want, lo), hi);
  sp.kr = ((d + ks - 1) / ks + 63) / 64 * 64;
  sp.ks = (d + sp.kr - 1) / sp.kr;
  return sp;
}

size_t gate_partial_bytes(int64_t T, int d, int N, bool noisy) {
  const GateSplit sp = gate_split(T, d, N, noisy);
  return (size_t)sp.ks * (size_t)T * sp.ncc * kGtCols * sizeof(float);
}

hipError_t launch_gate_plain_noisy(const GateParams& p, bool bf16_, bool noisy, hipStream_t s) {
  if (bf16_) return launch_gate_bf16(p, noisy, s);
  return noisy ? launch_e<float, true>(p, s) : launch_e<float, false>(p, s);
}

hipError_t launch_cosine_select(const CosineParams& p, hipStream_t s) {
  if (p.N <= kCgMaxN && p.p <= kCgMaxP) {
    hipLaunchKernelGGL(cosine_gate_kernel, dim3((p.T + kCgTok - 1) / kCgTok), dim3(kBlock), 0, s, p);
    return hipGetLastError();
  }
  const int nbatch = (p.T + kCosTW - 1) / kCosTW;
  const int want = (nbatch + kWavesPerBlock - 1) / kWavesPerBlock;
  const int grid = want < 256 ? want : 256;  // persistent: one block per CU stages the table once
  hipLaunchKernelGGL(cosine_select_kernel, dim3(grid), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
