// Dispatch: capacity-limited slots in token order and the permute into
// expert-contiguous rows (grouping tokens by expert before one batched
// matmul per group, as on "MoE架构：稀疏激活机制如何提升模型计算效率" §3.1;
// capacity_factor on "MoE稀疏计算加速技术解析与应用实践" §3.2).
//
// A choice (t, j) of expert e takes slot #{t' < t : e in topk_idx[t']}; it
// is kept iff that slot is below the capacity C, and then lands in row
// off[e] + slot, off being the exclusive scan of kept = min(count, C).
//
// Small index kernels compute this deterministically without any global
// atomics, linear in T:
//   count  one block per tile of kDispatchTile tokens: per-expert histogram
//          of the tile in LDS (integer adds, so order does not matter). The
//          single-kernel gate writes the same counts per 32 tokens itself,
//          and then no count kernel runs.
//   scan   (only when the count table is large) one block per expert: the
//          exclusive prefix over tiles of that expert's counts, and its total
//   rows   one block per tile, one token per thread: per expert, the tile's
//          starting slot and the totals (from the scan's output, or, for a
//          small count table, summed by each block from the table itself),
//          kept and the offsets; then in each 64-token wave a lane's rank
//          among earlier lanes with the same expert is a popcount of an LDS
//          bitmask, and the earlier waves' masks give the wave's own
//          starting slot
// and a third kernel, permute, copies each token's row of x once into its
// kept rows with 16-byte loads and stores (one wave per token).
//
// A routing the caller supplies (moe_dispatch) may name an expert outside
// [0, N) or the same expert twice for one token: such a choice is dropped
// (row -1) and counts for no expert; the gate never produces either.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kMaxN = 256;

// Whether choice i = t*k + j (expert e) occupies a slot: e in [0, N) and,
// for a caller's routing, no earlier choice of the same token names e.
__device__ inline bool counted_choice(const DispatchParams& p, int i, int e) {
  if ((unsigned)e >= (unsigned)p.N) return false;
  if (p.caller_routing) {
    const int j = i % p.k;
    for (int jj = 1; jj <= j; ++jj)
      if (p.topk_idx[i - jj] == e) return false;
  }
  return true;
}

__global__ __launch_bounds__(kBlock) void count_kernel(DispatchParams p) {
  __shared__ int hist[kMaxN];
  const int N = p.N, k = p.k;
  for (int e = threadIdx.x; e < N; e += kBlock) hist[e] = 0;
  __syncthreads();
  const int t_lo = blockIdx.x * kDispatchTile;
  const int t_hi = min(p.T, t_lo + kDispatchTile);
  for (int i = t_lo * k + threadIdx.x; i < t_hi * k; i += kBlock) {
    const int e = p.topk_idx[i];
    if (counted_choice(p, i, e)) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += kBlock) p.tile_counts[blockIdx.x * N + e] = hist[e];
}

// Exclusive prefix over tiles of one expert's counts (block e), for count
// tables too large for every rows block to sum itself. src: [nsrc, N]
// counts of consecutive groups of tokens, rpt groups per dispatch tile.
// Writes p.tile_start[tile * N + e] (the choices of e in the tokens before
// the tile) and p.totals[e]. Each thread sums a contiguous run of groups,
// the runs' sums are scanned across the block, and each thread then walks
// its run again writing the prefix at every tile boundary.
__global__ __launch_bounds__(kBlock) void scan_kernel(DispatchParams p, const int32_t* src, int nsrc, int rpt) {
  __shared__ int wsum[kWaves];
  const int e = blockIdx.x, N = p.N, tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int S = (nsrc + kBlock - 1) / kBlock;  // groups per thread
  const int r0 = tid * S, r1 = min(nsrc, r0 + S);
  int sum = 0;
  for (int r = r0; r < r1; r += 8) {  // eight loads in flight
    int c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = r + u < r1 ? src[(int64_t)(r + u) * N + e] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += c[u];
  }
  int inc = sum;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const int o = __shfl_up(inc, m, kWave);
    if (lane >= m) inc += o;
  }
  if (lane == kWave - 1) wsum[wave] = inc;
  __syncthreads();
  int base = inc - sum;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  if (tid == kBlock - 1) p.totals[e] = base + sum;
  for (int r = r0; r < r1; ++r) {
    if (r % rpt == 0) p.tile_start[(int64_t)(r / rpt) * N + e] = base;
    base += src[(int64_t)r * N + e];
  }
}

static_assert(kDispatchTile == kBlock, "rows_kernel: one token per thread");

__global__ __launch_bounds__(kBlock) void rows_kernel(DispatchParams p, int ntiles) {
  __shared__ unsigned long long mask[kWaves][kMaxN];
  __shared__ int start_s[kMaxN];
  __shared__ int kept_s[kMaxN];
  __shared__ int off_s[kMaxN];
  const int N = p.N, k = p.k, C = p.C;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int tile = blockIdx.x;
  if (tile == 0 && p.zero)
    for (int i = threadIdx.x; i < p.zero_n; i += kBlock) p.zero[i] = 0;
  if (p.tile_start) {
    // the scan kernel's prefixes and totals
    for (int e = threadIdx.x; e < N; e += kBlock) {
      start_s[e] = p.tile_start[(int64_t)tile * N + e];
      const int total = p.totals[e];
      kept_s[e] = min(total, C);
      if (tile == 0) p.expert_count[e] = total;
    }
  } else if (p.hist32) {
    // per expert: choices of the tokens before this tile, and of all tokens,
    // from the gate's per-32-token counts (entries (b, e) of the [nb, N]
    // table, eight loads in flight per thread before any is added up)
    constexpr int kPer = kDispatchTile / kGateHistTokens;  // gate blocks per tile
    const int nb = (p.T + kGateHistTokens - 1) / kGateHistTokens, ne = nb * N;
    for (int e = threadIdx.x; e < N; e += kBlock) start_s[e] = off_s[e] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < ne; i0 += 8 * kBlock) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kBlock + threadIdx.x;
        c[u] = i < ne ? p.hist32[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kBlock + threadIdx.x;
        if (c[u]) {
          atomicAdd(&off_s[i % N], c[u]);  // totals, for now
          if (i / N < tile * kPer) atomicAdd(&start_s[i % N], c[u]);
        }
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < N; e += kBlock) {
      const int total = off_s[e];
      kept_s[e] = min(total, C);
      if (tile == 0) p.expert_count[e] = total;
    }
  }
  // per expert: slots taken by earlier tiles, total, kept
  for (int e = threadIdx.x; e < N && !p.hist32 && !p.tile_start; e += kBlock) {
    int before = 0, total = 0;
    int t = 0;
    for (; t + 8 <= ntiles; t += 8) {  // eight loads in flight
      int c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = p.tile_counts[(t + i) * N + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        before += t + i < tile ? c[i] : 0;
        total += c[i];
      }
    }
    for (; t < ntiles; ++t) {
      const int c = p.tile_counts[t * N + e];
      before += t < tile ? c : 0;
      total += c;
    }
    start_s[e] = before;
    kept_s[e] = min(total, C);
    if (tile == 0) p.expert_count[e] = total;
  }
  for (int i = threadIdx.x; i < kWaves * N; i += kBlock) mask[i / N][i % N] = 0ull;
  __syncthreads();
  // exclusive scan of kept over experts (N <= 256 values; wave 0 does it)
  if (wave == 0) {
    int v[kMaxN / kWave];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kMaxN / kWave; ++i) {
      const int ee = lane * (kMaxN / kWave) + i;
      v[i] = ee < N ? kept_s[ee] : 0;
      sum += v[i];
    }
    int inc = sum;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int o = __shfl_up(inc, m, kWave);
      if (lane >= m) inc += o;
    }
    int run = inc - sum;
#pragma unroll
    for (int i = 0; i < kMaxN / kWave; ++i) {
      const int ee = lane * (kMaxN / kWave) + i;
      if (ee < N) {
        off_s[ee] = run;
        if (tile == 0) p.expert_off[ee] = run;
      }
      run += v[i];
    }
    if (tile == 0 && lane == kWave - 1) p.expert_off[N] = inc;
  }
  // this tile's choices, as per-wave bitmasks per expert
  const int t = tile * kDispatchTile + threadIdx.x;
  const bool live = t < p.T;
  if (live && p.zero_tok)
    for (int i = 0; i < p.zero_tok_n; ++i) p.zero_tok[(int64_t)t * p.zero_tok_n + i] = 0;
  if (live) {
    for (int j = 0; j < k; ++j) {
      const int e = p.topk_idx[t * k + j];
      if (counted_choice(p, t * k + j, e)) atomicOr(&mask[wave][e], 1ull << lane);
    }
  }
  __syncthreads();
  if (live) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int j = 0; j < k; ++j) {
      const int e = p.topk_idx[t * k + j];
      int row = -1;
      if (counted_choice(p, t * k + j, e)) {
        int slot = start_s[e] + __popcll(mask[wave][e] & below);
        for (int w = 0; w < wave; ++w) slot += __popcll(mask[w][e]);
        if (slot < C) {
          row = off_s[e] + slot;
          p.token_of_row[row] = t * k + j;
        }
      }
      p.row_of[t * k + j] = row;
    }
  }
}

// One wave per token: the row of x is read once into registers (kUnroll
// 16-byte chunks per lane at a time) and written to each kept row.
constexpr int kUnroll = 8;
__global__ __launch_bounds__(kBlock) void permute_kernel(DispatchParams p) {
  const int lane = lane_id();
  const int t = blockIdx.x * kWaves + threadIdx.x / kWave;
  if (t >= p.T) return;
  const int k = p.k;
  const int64_t row_bytes = (int64_t)p.d * p.elem_bytes;
  const int nchunk = (int)(row_bytes / 16);
  const char* src = static_cast<const char*>(p.x) + (int64_t)t * row_bytes;
  char* dst = static_cast<char*>(p.x_perm);
  for (int q0 = 0; q0 < nchunk; q0 += kWave * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int q = q0 + u * kWave + lane;
      if (q < nchunk) v[u] = load16(src + (int64_t)q * 16);
    }
    for (int j = 0; j < k; ++j) {
      const int row = p.row_of[t * k + j];
      if (row < 0) continue;
      char* drow = dst + (int64_t)row * row_bytes;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int q = q0 + u * kWave + lane;
        if (q < nchunk) store16(drow + (int64_t)q * 16, v[u]);
      }
    }
  }
}

}  // namespace

bool dispatch_scans(int64_t T, int N, bool hist32) {
  const int64_t nsrc = hist32 ? (T + kGateHistTokens - 1) / kGateHistTokens : (T + kDispatchTile - 1) / kDispatchTile;
  return nsrc * N > kDispatchDirectMax;
}

hipError_t launch_dispatch(const DispatchParams& p_in, hipStream_t s) {
  const int ntiles = (p_in.T + kDispatchTile - 1) / kDispatchTile;
  DispatchParams p = p_in;
  if (!p.hist32) hipLaunchKernelGGL(count_kernel, dim3(ntiles), dim3(kBlock), 0, s, p);
  if (dispatch_scans(p.T, p.N, p.hist32 != nullptr)) {
    const int nsrc = p.hist32 ? (p.T + kGateHistTokens - 1) / kGateHistTokens : ntiles;
    hipLaunchKernelGGL(scan_kernel, dim3(p.N), dim3(kBlock), 0, s, p, p.hist32 ? p.hist32 : p.tile_counts, nsrc,
                       p.hist32 ? kDispatchTile / kGateHistTokens : 1);
  } else {
    p.tile_start = nullptr;  // every rows block sums the count table itself
  }
  hipLaunchKernelGGL(rows_kernel, dim3(ntiles), dim3(kBlock), 0, s, p, ntiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.x_perm == nullptr) return err;
  return launch_permute(p, s);
}

hipError_t launch_permute(const DispatchParams& p, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3((p.T + kWaves - 1) / kWaves), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
