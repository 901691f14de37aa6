// Backward pass of the MoE layer (bf16 layers; plain and noisy gates).
//
// The gradients of L = sum(dy * y) (+ the load-balance losses) with the
// routing held fixed: gradients flow only through the selected experts'
// gate weights and outputs (sparse gating keeps only the Top-K experts'
// gradient, "MoE稀疏计算加速技术解析与应用实践" §2.1; the auxiliary losses join
// the total loss on the same page's §4.1 and on "MoE架构：突破单卡算力瓶颈的
// 密钥" §3.1). Per kept row r of expert e (token t, choice j, weight w):
//   U = x_perm W1_e + b1_e, H = GELU(U)                 (recomputed)
//   G = dy_t W2_e^T,  dU = w G GELU'(U),  g_tj = G . H (+ dy_t . b2_e)
//   dY = w dy_t, dW2_e = sum H^T dY, dW1_e = sum x^T dU, dx_perm = dU W1_e^T
// and per token: the gate weights' gradients g through the softmax to the
// logits, through the gate to x, w_gate and w_noise.
//
// Kernels:
//   bwd_gemm_kernel    grouped bf16 MFMA GEMM, 128 x 128 tiles of four waves,
//                      four LDS stages filled by direct-to-LDS loads. Either
//                      operand may hold K contiguous (rows of K) or K strided
//                      (rows of M or N): K-contiguous fragments are plain
//                      16-byte LDS reads, K-strided ones gfx950's transposing
//                      LDS reads. Ragged M (groups of output rows, the data
//                      gradients) or ragged K (groups of contraction rows, the
//                      weight gradients, one [M, N] output per group).
//   scale_rows_kernel  dY rows: bf16(w * dy_t) into each kept row of t
//   bwd_token_kernel   one wave per token: gate-weight gradients (partial
//                      dots in a fixed order), softmax and softplus backward
//   bwd_dx_kernel      dx = sum of the token's dx_perm rows + the gate's
//                      part, 4 elements per thread
//   gate_grad_kernels  dW_g = x^T dl, dW_n = x^T dz (one pass over x),
//                      d logit_bias: per 64-token partial sums, then added
//                      in chunk order
//   colsum_kernel      db1, db2: per expert column sums in row order
// Every reduction runs in a fixed order; no floating-point atomics.
#include "common.hpp"
#include "gelu.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kBK = 32;  // K per step
constexpr int kNumXcd = 8;
constexpr int64_t kBwdBigTileMin = 256;  // CUs of the chip
// 256 x 256 tiles with at least this many K-steps run the ping-pong K loop
// (its fixed cost per tile: one more MFMA interval, the second group's)
constexpr int kBwdPingPongMinSteps = 32;

// Output tiles of TS x TS (128 or 256): two waves along M and TS / 64 along
// N, each wave TS / 2 rows x 64 columns (FM x FN fragments of 32 x 32).
// 256 x 256 tiles (8 waves, one block per CU) read half the operand bytes
// per flop of 128 x 128 ones; they are taken where they give every CU a tile.
template <int TS> struct Tile {
  static constexpr int THREADS = TS == 256 ? 512 : 256;
  static constexpr int WN = TS / 64;
  static constexpr int WTM = TS / 2;
  static constexpr int FM = WTM / 32, FN = 2;
  static constexpr int OP_BYTES = TS * kBK * 2;            // one operand's tile of one stage
  static constexpr int LOADS = OP_BYTES / 16 / THREADS;    // 16-byte loads per thread per operand
  static_assert(TS == 128 || TS == 256, "tile size");
};

// 16-byte chunk swizzles (gfx950 LDS: 64 banks of 4 bytes): rows of 4 chunks
// (K-contiguous tiles, 64-byte rows) and rows of 16 or 32 chunks (K-strided
// tiles, 256- or 512-byte rows), each making its fragment reads conflict-free
__device__ inline int swz_rows4(int r) { return (r >> 2) & 3; }
__device__ inline int swz_rows16(int k) { return (2 * (k & 3)) ^ (8 * (k & 1)); }

__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t r, lds_void* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

template <int N>
__device__ inline void wait_loads_and_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2w;

template <BwdLayout L, int TS> struct Operand;

// Tile of TS rows (of M or N) x 32 K, K contiguous: row x at byte x * 64,
// chunk c of it at position c ^ swz_rows4(x).
template <int TS> struct Operand<BwdLayout::kKContig, TS> {
  static constexpr int READS = 1;  // LDS reads per fragment
  // slot i of this thread: row and global chunk
  __device__ static void slot(int s, int& row, int& chunk) {
    row = s >> 2;
    chunk = (s & 3) ^ swz_rows4(row);
  }
  // byte offset in the tile of the lane's fragment (8 consecutive K of row
  // base + 32 f + lane % 32, K half lane / 32 of substep ss)
  __device__ static int frag_off(int base, int f, int ss, int lane) {
    const int x = base + 32 * f + (lane & 31);
    const int c = 2 * ss + (lane >> 5);
    return x * 64 + ((c ^ swz_rows4(x)) * 16);
  }
  __device__ static u32x4 frag(const char* st, int off) { return *(lds_u32x4*)(st + off); }
};

// Tile of 32 K x TS columns (of M or N), K strided: K row k at byte
// k * 2 TS, chunk c of it at position c ^ swz_rows16(k). Fragments by
// transposing reads: in each 16-lane group q, lane r reads the 4 values of
// K row 8 (q / 2) + r / 4 (+ 4 for the second read, + 16 ss) at columns
// 32 f + 16 (q % 2) + 4 (r % 4) .. + 3, and the hardware hands each lane 8
// consecutive K values of one column.
template <int TS> struct Operand<BwdLayout::kKStrided, TS> {
  static constexpr int READS = 2;
  static constexpr int ROW = 2 * TS;  // bytes per K row
  __device__ static void slot(int s, int& row, int& chunk) {
    row = s / (TS / 8);
    chunk = (s % (TS / 8)) ^ swz_rows16(row);
  }
  __device__ static int frag_off(int base, int f, int ss, int lane) {
    const int q = lane >> 4, r = lane & 15;
    const int chunk = (base + 32 * f) / 8 + 2 * (q & 1) + ((r & 3) >> 1);
    const int krow = 16 * ss + 8 * (q >> 1) + (r >> 2);
    return krow * ROW + ((chunk ^ swz_rows16(r >> 2)) * 16) + 8 * (r & 1);
  }
  __device__ static u32x4 frag(const char* st, int off) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(st + off + 4 * ROW));
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    return u32x4{a[0], a[1], b[0], b[1]};
  }
};

// Ragged-M schedule: the block's (group, first row, end row, column tile)
// from seg, over row tiles of all groups (column tiles outermost), XCD by
// XCD in contiguous stretches. Returns false for blocks past the last tile.
template <int TS>
__device__ bool schedule_ragged_m(const BwdGemmParams& p, int* sched) {
  __shared__ int s_sched[4];
  const int lane = lane_id();
  if (threadIdx.x < kWave) {
    constexpr int GPL = 4;  // groups per lane (<= 256 groups)
    int lo[GPL], hi[GPL], nt[GPL], sum = 0;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int g = lane * GPL + i;
      lo[i] = hi[i] = 0;
      if (g < p.groups) {
        lo[i] = min(max(p.seg[g], 0), p.M);
        hi[i] = min(max(p.seg[g + 1], lo[i]), p.M);
      }
      nt[i] = (hi[i] - lo[i] + TS - 1) / TS;
      sum += nt[i];
    }
    int inc = sum;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int o = __shfl_up(inc, m, kWave);
      if (lane >= m) inc += o;
    }
    const int rows_total = __shfl(inc, kWave - 1, kWave);
    const int NT = (p.N + TS - 1) / TS;
    const int tiles = rows_total * NT;
    const int per = (tiles + kNumXcd - 1) / kNumXcd;
    const int b = blockIdx.x;
    const int tile = (b % kNumXcd) * per + b / kNumXcd;
    const bool live = b / kNumXcd < per && tile < tiles;
    if (lane == 0) s_sched[0] = -1;
    const int q = live ? tile % rows_total : -1, col = live ? tile / rows_total : 0;
    int start = inc - sum;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      if (live && q >= start && q < start + nt[i]) {
        s_sched[0] = lane * GPL + i;
        s_sched[1] = lo[i] + (q - start) * TS;
        s_sched[2] = hi[i];
        s_sched[3] = col * TS;
      }
      start += nt[i];
    }
  }
  __syncthreads();
  for (int i = 0; i < 4; ++i) sched[i] = __builtin_amdgcn_readfirstlane(s_sched[i]);
  if (sched[0] >= 0) sched[2] = min(sched[2], sched[1] + TS);
  return sched[0] >= 0;
}

template <int TS, BwdLayout LA, BwdLayout LB, BwdEpi EPI, typename O, bool RAGGED_K>
__global__ __launch_bounds__(Tile<TS>::THREADS) void bwd_gemm_kernel(BwdGemmParams p) {
  using T = Tile<TS>;
  constexpr int THREADS = T::THREADS, FM = T::FM, FN = T::FN, LOADS = T::LOADS, OPB = T::OP_BYTES;
  using OA = Operand<LA, TS>;
  using OB = Operand<LB, TS>;
  // one LDS object per stage (A tile, then B tile), so that the compiler
  // can tell the stage being filled from the one being read
  __shared__ __attribute__((aligned(1024))) char st0[2 * OPB];
  __shared__ __attribute__((aligned(1024))) char st1[2 * OPB];
  __shared__ __attribute__((aligned(1024))) char st2[2 * OPB];
  __shared__ __attribute__((aligned(1024))) char st3[2 * OPB];
  __shared__ float s_dot[T::WN][TS];
  __shared__ float s_w[EPI == BwdEpi::kGeluGrad ? TS : 1];  // the tile's row weights (kGeluGrad)
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int wm = wave / T::WN, wn = wave % T::WN;

  // ---- the tile: group g, output rows [m0, m1) (ragged M: rows of the
  // concatenated groups; ragged K: rows of the group's own output), columns
  // from n0, contraction rows [k_lo, k_hi)
  int g, m0, m1, n0, k_lo, k_hi;
  if constexpr (RAGGED_K) {
    const int MT = (p.M + TS - 1) / TS, NT = (p.N + TS - 1) / TS;
    const int tiles = p.groups * MT * NT, per = (tiles + kNumXcd - 1) / kNumXcd;
    const int b = blockIdx.x, tile = (b % kNumXcd) * per + b / kNumXcd;
    if (b / kNumXcd >= per || tile >= tiles) return;
    g = tile / (MT * NT);
    const int rem = tile % (MT * NT);
    m0 = (rem % MT) * TS;  // row tiles fastest: consecutive blocks share the B panel
    n0 = (rem / MT) * TS;
    m1 = min(m0 + TS, p.M);
    k_lo = min(max(p.seg[g], 0), p.a_rows);
    k_hi = min(max(p.seg[g + 1], k_lo), p.a_rows);
  } else {
    int sc[4];
    if (!schedule_ragged_m<TS>(p, sc)) return;
    g = sc[0], m0 = sc[1], m1 = sc[2], n0 = sc[3];
    k_lo = 0;
    k_hi = p.K;
  }
  const int K = k_hi - k_lo;

  // ---- operand addressing: byte offsets of this thread's 16-byte loads,
  // fixed over K except for the K position, which each step adds
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)p.a_bytes);
  const char* Bg = static_cast<const char*>(p.B) + (int64_t)g * p.strideB * 2;
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bg, (uint32_t)p.b_bytes);
  int a_base[LOADS], a_kc[LOADS], b_base[LOADS], b_kc[LOADS];
  bool a_ok[LOADS], b_ok[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int s = i * THREADS + tid;
    int row, chunk;
    OA::slot(s, row, chunk);
    if constexpr (LA == BwdLayout::kKContig) {
      // row m0 + row of A (gathered: A row gather[m] / gather_div)
      const int m = m0 + row;
      a_ok[i] = m < m1;
      const int arow = p.gather ? (a_ok[i] ? p.gather[m] / p.gather_div : 0) : m;
      a_base[i] = (int)(((int64_t)arow * p.lda + chunk * 8) * 2);
      a_kc[i] = chunk * 8;  // K offset of the chunk
    } else {
      // K row k_lo + row (+ k0), columns m0 + 8 chunk
      a_ok[i] = true;
      a_base[i] = (int)(((int64_t)(k_lo + row) * p.lda + m0 + chunk * 8) * 2);
      a_kc[i] = row;  // K offset of the row
    }
    OB::slot(s, row, chunk);
    if constexpr (LB == BwdLayout::kKContig) {
      const int n = n0 + row;
      b_ok[i] = n < p.N;
      b_base[i] = (int)(((int64_t)n * p.ldb + chunk * 8) * 2);
      b_kc[i] = chunk * 8;
    } else {
      b_ok[i] = true;
      b_base[i] = (int)(((int64_t)(k_lo + row) * p.ldb + n0 + chunk * 8) * 2);
      b_kc[i] = row;
    }
  }
  // loads of K step kt into a stage: a load whose K position lies past K
  // reads zeros (an offset past every range)
  auto issue = [&](char* st, int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const bool ok = a_ok[i] && k0 + a_kc[i] < K;
      const int off = LA == BwdLayout::kKContig ? a_base[i] + k0 * 2 : a_base[i] + (int)((int64_t)k0 * p.lda * 2);
      lds_dma16(ra, (lds_void*)(st + (i * THREADS + wave * kWave) * 16), ok ? off : (int)kOutOfRange);
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const bool ok = b_ok[i] && k0 + b_kc[i] < K;
      const int off = LB == BwdLayout::kKContig ? b_base[i] + k0 * 2 : b_base[i] + (int)((int64_t)k0 * p.ldb * 2);
      lds_dma16(rb, (lds_void*)(st + OPB + (i * THREADS + wave * kWave) * 16), ok ? off : (int)kOutOfRange);
    }
  };

  f32x16 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // the lane's fragment offsets within a stage ([substep][fragment]; B's
  // include the A tile before it), computed once: each fragment read is then
  // one offset from its stage object. (The compiler tells the stages apart
  // only for LDS accesses whose address it traces to one object in a few
  // steps; a read it cannot trace makes it wait for every direct-to-LDS
  // load in flight, which empties the pipeline each step.)
  int oa[2][FM], ob[2][FN];
#pragma unroll
  for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
    for (int f = 0; f < FM; ++f) oa[ss][f] = OA::frag_off(wm * T::WTM, f, ss, lane);
#pragma unroll
    for (int f = 0; f < FN; ++f) ob[ss][f] = OPB + OB::frag_off(wn * 64, f, ss, lane);
  }

  // a step's two 16-deep substeps; the fragment reads of substep 1 are
  // issued before the MFMAs of substep 0
  auto compute = [&](const char* st) {
    u32x4 fa[2][FM], fb[2][FN];  // [substep][fragment]: A (rows m), B (columns n)
    auto read = [&](int ss) {
#pragma unroll
      for (int f = 0; f < FN; ++f) fb[ss][f] = OB::frag(st, ob[ss][f]);
#pragma unroll
      for (int f = 0; f < FM; ++f) fa[ss][f] = OA::frag(st, oa[ss][f]);
    };
    read(0);
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      if (ss == 0) read(1);
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fb[ss][i]),
                                                               __builtin_bit_cast(bf16x8, fa[ss][j]), acc[i][j], 0,
                                                               0, 0);
    }
    if constexpr (TS == 256) {
      // instruction order for the step: the first substep's LDS reads, then
      // each MFMA followed by one of the next substep's LDS reads and, after
      // every second MFMA, one of the step's global->LDS loads
      constexpr int DSR = FM * OA::READS + FN * OB::READS;  // LDS reads per substep
      constexpr int MF = FM * FN;
      constexpr int VM = 2 * LOADS;
      __builtin_amdgcn_sched_group_barrier(0x100, DSR, 0);
#pragma unroll
      for (int ss = 0; ss < 2; ++ss)
#pragma unroll
        for (int m = 0; m < MF; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (ss == 0 && m < DSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if ((ss * MF + m) % 2 == 1 && (ss * MF + m) / 2 < VM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
    }
  };

  // ---- four stages, loads three steps ahead. The prologue's loads go out
  // in program order (scheduling barriers between them), so that counting
  // the loads still in flight tells which steps have landed.
  const int nk = (K + kBK - 1) / kBK;
  issue(st0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue(st1, 1);
  __builtin_amdgcn_sched_barrier(0);
  issue(st2, 2);
  // kGeluGrad: the weight of tile row tid, read while the first stages load
  float w_pre = 0.f;
  if constexpr (EPI == BwdEpi::kGeluGrad)
    if (tid < TS && m0 + tid < m1) w_pre = p.row_w[p.tor[m0 + tid]];
  // one barrier per step: wait until this step's loads have landed and this
  // wave's reads of the previous stage have returned, barrier, load into
  // the stage just freed, compute
  auto one_barrier_loop = [&]() {
    auto step = [&](char* cur, char* nxt, int kt) {
      wait_loads_and_lds<4 * LOADS>();
      __builtin_amdgcn_s_barrier();
      issue(nxt, kt + 3);
      compute(cur);
    };
    int kt = 0;
    for (; kt + 4 <= nk; kt += 4) {
      step(st0, st3, kt);
      step(st1, st0, kt + 1);
      step(st2, st1, kt + 2);
      step(st3, st2, kt + 3);
    }
    if (kt < nk) step(st0, st3, kt);
    if (kt + 1 < nk) step(st1, st0, kt + 1);
    if (kt + 2 < nk) step(st2, st1, kt + 2);
  };
  if constexpr (TS == 256) {
    if (nk >= kBwdPingPongMinSteps) {
      // Ping-pong: waves 0-3 and 4-7 (one of each per SIMD) run the same
      // steps half a step apart, two barriers per step, so that while one
      // wave of a SIMD issues a step's MFMAs (its fragments already in
      // registers) the other reads its next fragments and issues its loads.
      // Group 0: [mem(t) | mma(t)] per step; group 1: [mma(t-1) | mem(t)],
      // its first mma on zero fragments (adds nothing) and its last after
      // the loop. mem(t) loads step t + 3 into the stage of step t - 1,
      // which both groups have read before the barrier that precedes it.
      // Before that barrier every wave waits for its loads of step t: all
      // but the last two steps' (4 LOADS).
      const int grp = wave >> 2;
      u32x4 pa[2][FM], pb[2][FN];
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
        for (int f = 0; f < FM; ++f) pa[ss][f] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int f = 0; f < FN; ++f) pb[ss][f] = u32x4{0u, 0u, 0u, 0u};
      }
      auto stage = [&](auto c) -> char* {
        constexpr int i = decltype(c)::value % 4;
        if constexpr (i == 0) return st0;
        else if constexpr (i == 1) return st1;
        else if constexpr (i == 2) return st2;
        else return st3;
      };
      // the memory phase runs at raised wave priority, so that its reads and
      // loads issue ahead of the other wave's MFMAs
      auto mem = [&](auto c, int kt) {
        constexpr int cur = decltype(c)::value;
        const char* st = stage(c);
        __builtin_amdgcn_s_setprio(1);
        issue(stage(std::integral_constant<int, cur + 3>{}), kt + 3);
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
          for (int f = 0; f < FN; ++f) pb[ss][f] = OB::frag(st, ob[ss][f]);
#pragma unroll
          for (int f = 0; f < FM; ++f) pa[ss][f] = OA::frag(st, oa[ss][f]);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto mma = [&]() {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss)
#pragma unroll
          for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pb[ss][i]),
                                                                   __builtin_bit_cast(bf16x8, pa[ss][j]), acc[i][j],
                                                                   0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto sync_data = [&]() {
        wait_loads_and_lds<4 * LOADS>();
        __builtin_amdgcn_s_barrier();
      };
      auto sync_lds = [&]() {
        wait_loads_and_lds<63>();
        __builtin_amdgcn_s_barrier();
      };
      using J0 = std::integral_constant<int, 0>;
      using J1 = std::integral_constant<int, 1>;
      using J2 = std::integral_constant<int, 2>;
      using J3 = std::integral_constant<int, 3>;
      // Each step opens with its data wait, so that the loop head (where the
      // compiler merges its load tracking) is followed by an explicit wait:
      // with the memory phase there instead, the merged tracking made the
      // first step's fragment reads wait for every load in flight.
      if (grp == 0) {
        auto one = [&](auto c, int kt) {
          sync_data();
          mem(c, kt);
          sync_lds();
          mma();
        };
        int kt = 0;
        for (; kt + 4 <= nk; kt += 4) {
          one(J0{}, kt);
          one(J1{}, kt + 1);
          one(J2{}, kt + 2);
          one(J3{}, kt + 3);
        }
        if (kt < nk) one(J0{}, kt);
        if (kt + 1 < nk) one(J1{}, kt + 1);
        if (kt + 2 < nk) one(J2{}, kt + 2);
        sync_data();
      } else {
        auto one = [&](auto c, int kt) {
          sync_data();
          mma();  // step kt - 1 (zero fragments before step 0)
          sync_lds();
          mem(c, kt);
        };
        int kt = 0;
        for (; kt + 4 <= nk; kt += 4) {
          one(J0{}, kt);
          one(J1{}, kt + 1);
          one(J2{}, kt + 2);
          one(J3{}, kt + 3);
        }
        if (kt < nk) one(J0{}, kt);
        if (kt + 1 < nk) one(J1{}, kt + 1);
        if (kt + 2 < nk) one(J2{}, kt + 2);
        sync_data();
        mma();  // step nk - 1
      }
    } else {
      one_barrier_loop();
    }
  } else {
    one_barrier_loop();
  }
  wait_loads_and_lds<0>();

  // ---- epilogue: the lane holds D[n][m] for rows m = m0 + WTM wm + 32 j +
  // lane % 32 and columns n = n0 + 64 wn + 32 i + 8 q + 4 (lane / 32) + 0..3
  if constexpr (EPI == BwdEpi::kPlain && std::is_same_v<O, float>) {
    // fp32 outputs (dx rows, weight gradients): each 32-row slice of the
    // wave's tile goes through a per-wave LDS region (32 rows of 256 bytes,
    // 16-byte chunk c of row r at c ^ (r % 16)) and back as 16-byte pieces
    // of rows, 16 lanes per row, so that every store instruction writes
    // whole 256-byte row segments (stored from the MFMA layout, one
    // instruction would cover 32 rows with 32 bytes each)
    __syncthreads();  // every wave is done reading the stage buffers
    constexpr int REG = 32 * 64 * 4;
    constexpr int PER = 2 * OPB / REG;  // wave regions per stage buffer
    static_assert(PER >= 1 && (THREADS / kWave) <= 4 * PER, "epilogue regions fit the stage buffers");
    const int bsel = wave / PER;
    char* const reg = (bsel == 0 ? st0 : bsel == 1 ? st1 : bsel == 2 ? st2 : st3) + (wave % PER) * REG;
    const int lrow = lane & 31;
    const int cbase_col = n0 + wn * 64;
    float* const Cf = static_cast<float*>(p.C) + (RAGGED_K ? (int64_t)g * p.strideC : 0);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int frow = m0 + wm * T::WTM + 32 * j;
      if (frow >= m1) break;  // wave-uniform
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = 8 * i + 2 * q + (lane >> 5);  // the lane's 16-byte chunk of its row
          *(lds_f32x4*)(reg + lrow * 256 + ((ch ^ (lrow & 15)) * 16)) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int rr = 4 * t + (lane >> 4), ch = lane & 15;
        const f32x4 v = *(lds_f32x4*)(reg + rr * 256 + ((ch ^ (rr & 15)) * 16));
        const int col = cbase_col + 4 * ch;
        if (frow + rr < m1 && col < p.N) *reinterpret_cast<f32x4*>(Cf + (int64_t)(frow + rr) * p.ldc + col) = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    return;
  }
  if constexpr (EPI == BwdEpi::kGeluGrad) {
    // G = dy W2^T (fp32 in acc): each 32-row slice of the wave's tile goes
    // through a per-wave LDS region (as the fp32 outputs above) into row
    // order; then 16 lanes per row take 4 columns each: U and H are read and
    // dU = bf16(w G GELU'(U)) written as whole 128-byte row segments, and
    // the row's dot G . H over the wave's 64 columns is the lane's 4 terms
    // (fma in column order) summed over the 16 lanes by xor-shuffles in a
    // fixed order; the two waves of each 128 columns are then added, the
    // lower columns' first. The rows' weights w were read before the K loop;
    // a slice's U and H pieces are all requested before any is used (rows
    // and columns past the tile read clamped, in-range positions whose
    // results are dropped), so that the slice waits for one round trip.
    if (tid < TS) s_w[tid] = w_pre;
    __syncthreads();  // every wave is done reading the stage buffers; s_w written
    constexpr int REG = 32 * 64 * 4;
    constexpr int PER = 2 * OPB / REG;
    static_assert(PER >= 1 && (THREADS / kWave) <= 4 * PER, "epilogue regions fit the stage buffers");
    const int bsel = wave / PER;
    char* const reg = (bsel == 0 ? st0 : bsel == 1 ? st1 : bsel == 2 ? st2 : st3) + (wave % PER) * REG;
    const int lrow = lane & 31;
    const int ch = lane & 15;
    const int col = n0 + wn * 64 + 4 * ch;
    const int colc = min(col, p.N - 4);
    const bf16* const Ub = static_cast<const bf16*>(p.U);
    const bf16* const Hb = static_cast<const bf16*>(p.H);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int frow = m0 + wm * T::WTM + 32 * j;
      if (frow >= m1) break;  // wave-uniform
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = 8 * i + 2 * q + (lane >> 5);
          *(lds_f32x4*)(reg + lrow * 256 + ((c ^ (lrow & 15)) * 16)) =
              f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
      u32x2 uu[8], hh[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int mc = min(frow + 4 * t + (lane >> 4), m1 - 1);
        const int64_t at = (int64_t)mc * p.ldc + colc;
        uu[t] = *reinterpret_cast<const u32x2*>(Ub + at);
        hh[t] = *reinterpret_cast<const u32x2*>(Hb + at);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int rr = 4 * t + (lane >> 4);
        const f32x4 gv = *(lds_f32x4*)(reg + rr * 256 + ((ch ^ (rr & 15)) * 16));
        const int m = frow + rr;
        float dot = 0.f;
        if (m < m1 && col < p.N) {
          const float w = s_w[m - m0];
          float du[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float u = chunk_elem<bf16>(u32x4{uu[t][0], uu[t][1], 0u, 0u}, r);
            const float h = chunk_elem<bf16>(u32x4{hh[t][0], hh[t][1], 0u, 0u}, r);
            du[r] = w * gv[r] * gelu_grad(u);
            dot = fmaf(gv[r], h, dot);
          }
          Store<bf16>::four(static_cast<bf16*>(p.C) + (int64_t)m * p.ldc + col, du[0], du[1], du[2], du[3]);
        }
#pragma unroll
        for (int sh = 8; sh >= 1; sh >>= 1) dot += __shfl_xor(dot, sh, kWave);
        if (ch == 0) s_dot[wn][wm * T::WTM + 32 * j + rr] = dot;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
    const int NTc = (p.N + 127) / 128;
    for (int e = tid; e < TS * (TS / 128); e += THREADS) {
      const int r = e % TS, c = e / TS;
      if (m0 + r < m1 && n0 + 128 * c < p.N)
        p.pd[(int64_t)(m0 + r) * NTc + n0 / 128 + c] = s_dot[2 * c][r] + s_dot[2 * c + 1][r];
    }
    return;
  }
  static_assert(EPI != BwdEpi::kPlain || std::is_same_v<O, float>, "plain outputs are fp32");
}

// dY rows: for each kept choice (t, j), row row_of[t k + j] = bf16(w_tj dy_t);
// one wave per token, dy_t read once
__global__ __launch_bounds__(256) void scale_rows_kernel(const bf16* dy, const int32_t* row_of, const float* w,
                                                         bf16* out, int T, int d, int k) {
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  for (int c0 = 0; c0 < d / 8; c0 += kWave) {
    const int c = c0 + lane;
    if (c >= d / 8) break;
    const u32x4 v = load16(dy + (int64_t)t * d + c * 8);
    for (int j = 0; j < k; ++j) {
      const int r = row_of[(int64_t)t * k + j];
      if (r < 0) continue;
      const float wj = w[(int64_t)t * k + j];
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16_bits(wj * chunk_elem<bf16>(v, 2 * i)) |
               (f32_to_bf16_bits(wj * chunk_elem<bf16>(v, 2 * i + 1)) << 16);
      store16(out + (int64_t)r * d + c * 8, o);
    }
  }
}

// d(aux_coef[0] * load_balance_loss + aux_coef[1] * importance_loss) / d
// importance (one wave; N <= 256): 2 (imp - mean) and 0.1 (imp - mean) /
// ((N - 1) std), the latter 0 where std is 0. Sums in a fixed order.
__global__ __launch_bounds__(64) void importance_grad_kernel(const float* imp, float* dimp, int N, float c0,
                                                             float c1) {
  __shared__ float s_mean, s_std;
  const int lane = lane_id();
  if (lane == 0) {
    float sum = 0.f;
    for (int e = 0; e < N; ++e) sum += imp[e];
    const float mean = sum / (float)N;
    float ss = 0.f;
    for (int e = 0; e < N; ++e) ss += (imp[e] - mean) * (imp[e] - mean);
    s_mean = mean;
    s_std = N > 1 ? sqrtf(ss / (float)(N - 1)) : 0.f;
  }
  __syncthreads();
  for (int e = lane; e < N; e += kWave) {
    const float dev = imp[e] - s_mean;
    float gr = c0 * 2.f * dev;
    if (c1 != 0.f && s_std > 0.f) gr += c1 * 0.1f * dev / ((float)(N - 1) * s_std);
    dimp[e] = gr;
  }
}

constexpr int kGateTok = 64;  // tokens per partial sum of the gate's gradients
constexpr int kTokWaves = 4;  // tokens per block of the token kernel, one wave each

// sum and maximum over the wave's 64 lanes, in a fixed (butterfly) order
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// the wave's LDS writes before this point are seen by its reads after it
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave per token t: the gate weights' gradients g_tj (lane j), the
// logits' gradient dl[t] (softmax backward) and, for the noisy gate,
// dz[t] = dl eps sigmoid(x W_n). Reductions over the wave are butterflies.
__global__ __launch_bounds__(kWave * kTokWaves) void bwd_token_kernel(BwdTokenParams p) {
  __shared__ float s_dl[kTokWaves][kMaxExperts], s_dz[kTokWaves][kMaxExperts];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int t = blockIdx.x * kTokWaves + wave;
  if (t >= p.T) return;  // wave-uniform; the waves share no data
  const int k = p.k, N = p.N, d = p.d;
  float* const dl = s_dl[wave];
  float* const dz = s_dz[wave];
  // lane j < k: choice j's expert, weight, row and gate-weight gradient
  // (the row's partial dots G . H over its column tiles, split over the
  // lanes and added by a butterfly)
  int e = 0, r = -1;
  float w = 0.f, g = 0.f;
  if (lane < k) {
    const int64_t i = (int64_t)t * k + lane;
    e = p.topk_idx[i];
    w = p.topk_w[i];
    r = p.row_of[i];
  }
  for (int j = 0; j < k; ++j) {
    const int rj = __shfl(r, j, kWave);
    if (rj < 0) continue;  // wave-uniform
    float part = 0.f;
    for (int c = lane; c < p.ntc; c += kWave) part += p.pd[(int64_t)rj * p.ntc + c];
    part = wave_sum(part);
    if (lane == j) g = part;
  }
  if (p.b2) {
    // + dy_t . b2_e for each kept choice
    for (int j = 0; j < k; ++j) {
      const int rj = __shfl(r, j, kWave), ej = __shfl(e, j, kWave);
      if (rj < 0) continue;  // wave-uniform
      float part = 0.f;
      for (int i = lane; i < d; i += kWave)
        part += (float)p.dy[(int64_t)t * d + i] * (float)p.b2[(int64_t)ej * d + i];
      part = wave_sum(part);
      if (lane == j) g += part;
    }
  }
  if (lane < k && p.dimp) g += p.dimp[e];
  // softmax backward
  if (p.renorm) {
    float sw = 0.f;  // sum over j of w_j g_j, j in order
    for (int j = 0; j < k; ++j) sw += __shfl(w, j, kWave) * __shfl(g, j, kWave);
    for (int n = lane; n < N; n += kWave) dl[n] = 0.f;
    wave_lds_sync();
    if (lane < k) dl[e] = w * (g - sw);
  } else {
    // p = softmax of the logits; G scattered over the experts (in dz)
    const float* l = p.logits + (int64_t)t * N;
    float lv[kMaxExperts / kWave], m = -INFINITY;
#pragma unroll
    for (int q = 0; q < kMaxExperts / kWave; ++q) {
      const int n = lane + kWave * q;
      lv[q] = n < N ? l[n] : -INFINITY;
      m = fmaxf(m, lv[q]);
    }
    m = wave_max(m);
    float ex[kMaxExperts / kWave], zp = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxExperts / kWave; ++q) {
      ex[q] = lane + kWave * q < N ? expf(lv[q] - m) : 0.f;
      zp += ex[q];
    }
    const float z = wave_sum(zp);
    for (int n = lane; n < N; n += kWave) dz[n] = 0.f;
    wave_lds_sync();
    if (lane < k) dz[e] = g;
    wave_lds_sync();
    float sp = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxExperts / kWave; ++q) {
      const int n = lane + kWave * q;
      ex[q] = ex[q] / z;
      if (n < N) sp += ex[q] * dz[n];
    }
    const float sg = wave_sum(sp);
#pragma unroll
    for (int q = 0; q < kMaxExperts / kWave; ++q) {
      const int n = lane + kWave * q;
      if (n < N) dl[n] = ex[q] * (dz[n] - sg);
    }
  }
  wave_lds_sync();
  // noisy gate: dz = dl eps sigmoid(x W_n), x W_n eight experts at a time;
  // with N a multiple of 8 a lane's 8 weights are one 16-byte load, and the
  // loads of 8 of its columns are issued before their FMAs
  if (p.w_noise) {
    const bool vec = N % 8 == 0;
    for (int n0 = 0; n0 < N; n0 += 8) {
      float acc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = 0.f;
      if (vec) {
        for (int i0 = lane; i0 < d; i0 += 8 * kWave) {
          float xv[8];
          u32x4 wc[8];
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const int i = min(i0 + b * kWave, d - 1);
            xv[b] = i0 + b * kWave < d ? (float)p.x[(int64_t)t * d + i] : 0.f;
            wc[b] = *reinterpret_cast<const u32x4*>(p.w_noise + (int64_t)i * N + n0);
          }
          __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the FMAs
#pragma unroll
          for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[u] = fmaf(xv[b], chunk_elem<bf16>(wc[b], u), acc[u]);
        }
      } else {
        for (int i = lane; i < d; i += kWave) {
          const float xv = (float)p.x[(int64_t)t * d + i];
          const bf16* wr = p.w_noise + (int64_t)i * N + n0;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (n0 + u < N) acc[u] = fmaf(xv, (float)wr[u], acc[u]);
        }
      }
      float zsel = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float zu = wave_sum(acc[u]);
        if (lane == u) zsel = zu;
      }
      const int n = n0 + lane;
      if (lane < 8 && n < N) {
        const float ez = expf(-fabsf(zsel));
        const float sig = zsel >= 0.f ? 1.f / (1.f + ez) : ez / (1.f + ez);
        dz[n] = dl[n] * p.noise[(int64_t)t * N + n] * sig;
      }
    }
    wave_lds_sync();
  }
  for (int n = lane; n < N; n += kWave) {
    p.dl[(int64_t)t * N + n] = dl[n];
    if (p.w_noise) p.dz[(int64_t)t * N + n] = dz[n];
  }
}

constexpr int kDxThreads = 256;  // threads of the dx kernel, 4 elements each

// dx[t][i..i+3] = sum over kept j of dx_perm[row_tj][i..] (j order) +
// dl[t] W_g^T + dz[t] W_n^T (experts in order, the noise part after the
// gate part): block (t, y) covers elements 1024 y .. + 1023 of token t,
// with the token's rows, dl and dz in LDS. Dropped choices read row 0 and
// add nothing.
__global__ __launch_bounds__(kDxThreads) void bwd_dx_kernel(BwdTokenParams p) {
  __shared__ float s_sv[2][kMaxExperts];
  __shared__ int s_row[32];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int k = p.k, N = p.N, d = p.d;
  for (int n = tid; n < N; n += kDxThreads) {
    s_sv[0][n] = p.dl[(int64_t)t * N + n];
    if (p.w_noise) s_sv[1][n] = p.dz[(int64_t)t * N + n];
  }
  if (tid < k) s_row[tid] = p.row_of[(int64_t)t * k + tid];
  __syncthreads();
  const int i = (blockIdx.y * kDxThreads + tid) * 4;
  if (i >= d) return;  // d is a multiple of 8: i < d covers i + 3
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < k; j0 += 8) {
    f32x4 a[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int rj = j0 + b < k ? s_row[j0 + b] : -1;
      a[b] = *reinterpret_cast<const f32x4*>(p.dx_perm + (int64_t)max(rj, 0) * d + i);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the adds
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (j0 + b < k && s_row[j0 + b] >= 0)
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] += a[b][u];
  }
  float gs[4] = {0.f, 0.f, 0.f, 0.f};
  const bool vec = N % 8 == 0;  // gate rows of whole 16-byte chunks
  for (int pass = 0; pass < (p.w_noise ? 2 : 1); ++pass) {
    const bf16* W = pass ? p.w_noise : p.w_gate;
    const float* sv = s_sv[pass];
    if (vec) {
      for (int n0 = 0; n0 < N; n0 += 8) {
        u32x4 c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) c[u] = *reinterpret_cast<const u32x4*>(W + (int64_t)(i + u) * N + n0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int q = 0; q < 8; ++q) gs[u] = fmaf(sv[n0 + q], chunk_elem<bf16>(c[u], q), gs[u]);
      }
    } else {
      for (int n = 0; n < N; ++n) {
        const float sn = sv[n];
#pragma unroll
        for (int u = 0; u < 4; ++u) gs[u] = fmaf(sn, (float)W[(int64_t)(i + u) * N + n], gs[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] += gs[u];
  Store<bf16>::four(p.dx + (int64_t)t * d + i, v[0], v[1], v[2], v[3]);
}

// partial[c][n] = sum over the tokens of chunk c of src[t][n] (t ascending)
__global__ __launch_bounds__(256) void column_sum_partial_kernel(const float* src, float* partial, int T, int N) {
  const int c = blockIdx.x;
  const int t0 = c * kGateTok, t1 = min(T, t0 + kGateTok);
  for (int n = threadIdx.x; n < N; n += 256) {
    float s = 0.f;
    for (int t = t0; t < t1; ++t) s += src[(int64_t)t * N + n];
    partial[(int64_t)c * N + n] = s;
  }
}

// partial[c][i][n] = sum over the tokens t of chunk c (ascending) of
// x[t][i] src[t][n], where src is src0 for n < N and src1 (the noisy
// gate's dz, or null) for N <= n < 2N. One wave per block: lane l holds
// IL consecutive columns i (one 8-byte load of x per token) times NL
// experts from blockIdx.z NL; the chunk's src values sit in LDS.
template <int IL, int NL>
__global__ __launch_bounds__(kWave) void gate_grad_partial_kernel(const bf16* x, const float* src0,
                                                                  const float* src1, float* partial, int T, int d,
                                                                  int N) {
  __shared__ float s_src[kGateTok][NL];
  const int Np = src1 ? 2 * N : N;
  const int lane = threadIdx.x;
  const int i0 = (blockIdx.x * kWave + lane) * IL;
  const int c = blockIdx.y, nb = blockIdx.z * NL;
  const int t0 = c * kGateTok, nt = min(T - t0, kGateTok);
  for (int q = lane; q < kGateTok * NL; q += kWave) {
    const int tt = q / NL, n = nb + q % NL;
    float v = 0.f;
    if (tt < nt && n < Np) v = n < N ? src0[(int64_t)(t0 + tt) * N + n] : src1[(int64_t)(t0 + tt) * N + n - N];
    s_src[tt][q % NL] = v;
  }
  __syncthreads();
  const bool live = i0 < d;  // d and i0 multiples of IL: the lane's IL columns are in range
  const bf16* xp = x + (int64_t)t0 * d + (live ? i0 : 0);
  float acc[IL][NL];
#pragma unroll
  for (int u = 0; u < IL; ++u)
#pragma unroll
    for (int n = 0; n < NL; ++n) acc[u][n] = 0.f;
  // batches of 16 tokens: the batch's loads are all issued before its FMAs
  // (rows past the chunk read row t0, in range, and meet zero src values)
  for (int tb = 0; tb < nt; tb += 16) {
    u32x4 raw[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int64_t at = (int64_t)(tb + b < nt ? tb + b : 0) * d;
      if constexpr (IL == 8) {
        raw[b] = *reinterpret_cast<const u32x4*>(xp + at);
      } else {
        const u32x2 r2 = *reinterpret_cast<const u32x2*>(xp + at);
        raw[b] = u32x4{r2[0], r2[1], 0u, 0u};
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the FMAs
#pragma unroll
    for (int b = 0; b < 16; ++b)
#pragma unroll
      for (int u = 0; u < IL; ++u) {
        const float xv = chunk_elem<bf16>(raw[b], u);
#pragma unroll
        for (int n = 0; n < NL; ++n) acc[u][n] = fmaf(xv, s_src[tb + b][n], acc[u][n]);
      }
  }
  if (!live) return;
#pragma unroll
  for (int u = 0; u < IL; ++u)
#pragma unroll
    for (int n = 0; n < NL; ++n)
      if (nb + n < Np) partial[((int64_t)c * d + i0 + u) * Np + nb + n] = acc[u][n];
}

// the chunks' partial sums added in chunk order: column n < N of
// partial[.][i] into out0[i][n], n >= N into out1[i][n - N]. A block takes
// 64 outputs; wave w adds chunks w cs .. (w + 1) cs - 1 in order (cs =
// ceil(chunks / 8)), and wave 0 adds the eight sums in wave order.
constexpr int kFinalWaves = 8;
__global__ __launch_bounds__(kWave * kFinalWaves) void gate_grad_final_kernel(const float* partial, float* out0,
                                                                             float* out1, int chunks, int d, int N,
                                                                             int Np) {
  __shared__ float s_part[kFinalWaves][kWave];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int64_t n_out = (int64_t)d * Np;
  const int64_t q = (int64_t)blockIdx.x * kWave + lane;
  const int cs = (chunks + kFinalWaves - 1) / kFinalWaves;
  const int c0 = w * cs, c1 = min(chunks, c0 + cs);
  float s = 0.f;
  if (q < n_out) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) s += partial[(int64_t)c * n_out + q];
  }
  s_part[w][lane] = s;
  __syncthreads();
  if (w != 0 || q >= n_out) return;
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < kFinalWaves; ++j) t += s_part[j][lane];
  const int i = (int)(q / Np), n = (int)(q % Np);
  if (n < N) out0[(int64_t)i * N + n] = t;
  else out1[(int64_t)i * N + n - N] = t;
}

// out[e][c] = sum over rows [off[e], off[e+1]) of src[row][c], rows in
// order (per expert column sums for the bias gradients)
template <typename S>
__global__ __launch_bounds__(256) void colsum_kernel(const S* src, const int32_t* off, float* out, int cols,
                                                     int rows_bound) {
  const int e = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  const int lo = min(max(off[e], 0), rows_bound), hi = min(max(off[e + 1], lo), rows_bound);
  float s = 0.f;
  for (int r = lo; r < hi; ++r) s += (float)src[(int64_t)r * cols + c];
  out[(int64_t)e * cols + c] = s;
}

// upper bound on the tiles of a launch with TS x TS tiles
template <int TS>
int64_t bwd_tiles(const BwdGemmParams& p, bool ragged_k) {
  const int64_t NT = (p.N + TS - 1) / TS;
  return ragged_k ? (int64_t)p.groups * ((p.M + TS - 1) / TS) * NT : ((int64_t)p.M / TS + p.groups) * NT;
}

template <int TS, BwdLayout LA, BwdLayout LB, BwdEpi EPI, typename O, bool RK>
hipError_t launch_tiles(const BwdGemmParams& p, int64_t tiles, hipStream_t s) {
  const int64_t blocks = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  hipLaunchKernelGGL((bwd_gemm_kernel<TS, LA, LB, EPI, O, RK>), dim3((unsigned)blocks), dim3(Tile<TS>::THREADS), 0,
                     s, p);
  return hipGetLastError();
}

// 256 x 256 tiles where they give at least one per CU and the groups hold
// at least 128 rows on average (fewer rows leave big tiles mostly empty, and
// such layers are bound by their weight and gradient bytes, which two
// blocks per CU of 128 x 128 tiles stream better), else 128 x 128
template <BwdLayout LA, BwdLayout LB, BwdEpi EPI, typename O, bool RK>
hipError_t launch_bwd(const BwdGemmParams& p, hipStream_t s) {
  const int64_t big = bwd_tiles<256>(p, RK);
  const int64_t avg_rows = p.groups > 0 ? (int64_t)(RK ? p.a_rows : p.M) / p.groups : 0;
  if (big >= kBwdBigTileMin && avg_rows >= 128) return launch_tiles<256, LA, LB, EPI, O, RK>(p, big, s);
  const int64_t tiles = bwd_tiles<128>(p, RK);
  if (tiles <= 0) return hipSuccess;
  return launch_tiles<128, LA, LB, EPI, O, RK>(p, tiles, s);
}

}  // namespace

hipError_t launch_bwd_gemm(const BwdGemmParams& p, BwdGemmKind kind, hipStream_t s) {
  using L = BwdLayout;
  switch (kind) {
    case BwdGemmKind::kGeluGrad:  // dU: gathered dy rows, W2_e rows [N][K]
      return launch_bwd<L::kKContig, L::kKContig, BwdEpi::kGeluGrad, bf16, false>(p, s);
    case BwdGemmKind::kDataGrad:  // dx_perm = dU W1_e^T, fp32
      return launch_bwd<L::kKContig, L::kKContig, BwdEpi::kPlain, float, false>(p, s);
    case BwdGemmKind::kWeightGrad:  // dW_e = A_e^T B_e over the group's rows, fp32
      return launch_bwd<L::kKStrided, L::kKStrided, BwdEpi::kPlain, float, true>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scale_rows(const bf16* dy, const int32_t* row_of, const float* w, bf16* out, int T, int d, int k,
                             hipStream_t s) {
  hipLaunchKernelGGL(scale_rows_kernel, dim3((T + 3) / 4), dim3(256), 0, s, dy, row_of, w, out, T, d, k);
  return hipGetLastError();
}

hipError_t launch_importance_grad(const float* imp, float* dimp, int N, float c0, float c1, hipStream_t s) {
  hipLaunchKernelGGL(importance_grad_kernel, dim3(1), dim3(64), 0, s, imp, dimp, N, c0, c1);
  return hipGetLastError();
}

hipError_t launch_bwd_token(const BwdTokenParams& p, hipStream_t s) {
  hipLaunchKernelGGL(bwd_token_kernel, dim3((p.T + kTokWaves - 1) / kTokWaves), dim3(kWave * kTokWaves), 0, s, p);
  hipLaunchKernelGGL(bwd_dx_kernel, dim3(p.T, (p.d + 4 * kDxThreads - 1) / (4 * kDxThreads)), dim3(kDxThreads), 0,
                     s, p);
  return hipGetLastError();
}

int gate_grad_chunks(int64_t T) { return (int)((T + kGateTok - 1) / kGateTok); }

hipError_t launch_gate_grad(const bf16* x, const float* src0, const float* src1, float* partial, float* out0,
                            float* out1, int T, int d, int N, hipStream_t s) {
  const int chunks = gate_grad_chunks(T);
  const int Np = src1 ? 2 * N : N;
  if (Np <= 8)
    hipLaunchKernelGGL((gate_grad_partial_kernel<4, 8>), dim3((d + 4 * kWave - 1) / (4 * kWave), chunks, 1),
                       dim3(kWave), 0, s, x, src0, src1, partial, T, d, N);
  else
    hipLaunchKernelGGL((gate_grad_partial_kernel<4, 16>),
                       dim3((d + 4 * kWave - 1) / (4 * kWave), chunks, (Np + 15) / 16), dim3(kWave), 0, s, x, src0,
                       src1, partial, T, d, N);
  const int64_t n_out = (int64_t)d * Np;
  hipLaunchKernelGGL(gate_grad_final_kernel, dim3((unsigned)((n_out + kWave - 1) / kWave)),
                     dim3(kWave * kFinalWaves), 0, s, partial, out0, out1, chunks, d, N, Np);
  return hipGetLastError();
}

hipError_t launch_colsum_bf16(const bf16* src, const int32_t* off, float* out, int cols, int groups, int rows_bound,
                              hipStream_t s) {
  hipLaunchKernelGGL(colsum_kernel<bf16>, dim3((cols + 255) / 256, groups), dim3(256), 0, s, src, off, out, cols,
                     rows_bound);
  return hipGetLastError();
}

hipError_t launch_column_sum(const float* src, float* partial, float* out, int T, int N, hipStream_t s) {
  const int chunks = gate_grad_chunks(T);
  hipLaunchKernelGGL(column_sum_partial_kernel, dim3(chunks), dim3(256), 0, s, src, partial, T, N);
  hipLaunchKernelGGL(gate_grad_final_kernel, dim3((N + kWave - 1) / kWave), dim3(kWave * kFinalWaves), 0, s, partial,
                     out, out, chunks, 1, N, N);
  return hipGetLastError();
}

}  // namespace moe
