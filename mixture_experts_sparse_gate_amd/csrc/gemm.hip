// Grouped GEMM on MFMA for the experts (and the cosine gate's projection).
//
// For each group g (an expert) and each of its rows r in [seg[g], seg[g+1]):
//     C[r, :] = epilogue(A[r, :] B_g + bias_g)
// with A rows K long, B_g = [K, Ncols] row-major. This is the second stage of
// the two-stage execution on "MoE架构：稀疏激活机制如何提升模型计算效率" §3.1
// (tokens grouped by expert, then one batched matmul per group); the epilogue
// is the expert's GELU (erf form) between its two Linear layers
// ("MoE稀疏计算加速技术解析与应用实践" §3.2).
//
// Design for gfx950:
//  - The block computes a BM x BN tile of C. MFMA 32x32 is used in the
//    transposed sense, D = B^T A^T: the weight tile is the MFMA's first
//    operand and the activation rows its second, so each lane ends up with
//    4 consecutive output columns of one row (8- or 16-byte stores).
//  - Both operands are K-contiguous 16-byte chunks in LDS. A rows are
//    K-contiguous already. B is N-contiguous in memory, so each thread loads
//    an 8x8 (bf16) or 4x4 (fp32) block of it with 16-byte row loads and
//    transposes it in registers before the LDS store.
//  - LDS rows are BK elements = 8 chunks; chunk c of row r is stored at
//    c ^ ((r ^ r>>3) & 7), which keeps both the transposed stores and the
//    MFMA operand reads free of bank conflicts.
//  - Two LDS stages: the next K-step's global loads are in flight while the
//    current one feeds the MFMAs.
//  - Ragged groups: the grid's x dimension is an upper bound on the number
//    of row tiles; each block finds its (group, row range) from seg on the
//    device, so no host synchronisation is needed. Blocks past the last tile
//    exit at once.
//  - No split-K and no atomics: each output element is written once.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <typename E> struct Mfma;
template <> struct Mfma<bf16> {
  // one 32x32x16 MFMA per pair of chunks
  __device__ static inline void step(f32x16& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  // four 32x32x2 MFMAs per pair of chunks: element e of the lane's chunk
  __device__ static inline void step(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc,
                                                 0, 0, 0);
  }
};

// Transposes a CE x CE block held as CE rows of one 16-byte chunk each:
// in[r] = row r (CE consecutive columns), out[c] = column c (CE consecutive rows).
template <typename E> struct Transpose;
template <> struct Transpose<bf16> {
  __device__ static inline void run(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = in[2 * q][c >> 1], hi = in[2 * q + 1][c >> 1];
        out[c][q] = (c & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                            : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      }
  }
};
template <> struct Transpose<float> {
  __device__ static inline void run(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[c][r] = in[r][c];
  }
};

__device__ inline float gelu_erf(float u) { return 0.5f * u * (1.f + erff(u * 0.70710678118654752f)); }

template <typename E, typename O, int BM_, int BN_, int WM_, int WN_, bool GELU_>
struct Cfg {
  using Elem = E;
  using Out = O;
  static constexpr int CE = ElemTraits<E>::kPerChunk;
  static constexpr int KC = 8;  // chunks per LDS row: BK = 8 * CE elements
  static constexpr int BK = KC * CE;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int THREADS = kWave * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr bool GELU = GELU_;
  static constexpr int A_CHUNKS = BM * KC;              // per stage
  static constexpr int B_CHUNKS = BN * KC;
  static constexpr int A_PER_THREAD = (A_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int B_BLOCKS = KC * (BN / CE);       // CE x CE blocks per stage
  static constexpr int B_PER_THREAD = (B_BLOCKS + THREADS - 1) / THREADS;
  static constexpr int LDS_BYTES = 2 * (A_CHUNKS + B_CHUNKS) * 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold at least one 32x32 MFMA tile");
  static_assert(BN % CE == 0, "");
};

__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <class C>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_kernel(GemmParams p) {
  using E = typename C::Elem;
  using O = typename C::Out;
  constexpr int CE = C::CE, KC = C::KC, BK = C::BK, BM = C::BM, BN = C::BN;
  __shared__ u32x4 smem[C::LDS_BYTES / 16];
  __shared__ int sched[3];
  u32x4* As = smem;                      // [2][BM * KC]
  u32x4* Bs = smem + 2 * C::A_CHUNKS;    // [2][BN * KC]

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int mt = blockIdx.x;
  const int n0 = blockIdx.y * BN;

  // ---- find this block's (group, rows)
  if (p.seg == nullptr) {
    if (tid == 0) {
      const int lo = mt * BM;
      sched[0] = lo < p.M ? 0 : -1;
      sched[1] = lo;
      sched[2] = p.M;
    }
  } else if (wave == 0) {
    constexpr int GPL = 4;  // groups per lane (groups <= 256)
    int cnt[GPL];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int g = lane * GPL + i;
      cnt[i] = 0;
      if (g < p.groups) {
        // rows are clamped to [0, M] so that no offset table can address
        // outside the row buffers
        const int lo = min(max(p.seg[g], 0), p.M), hi = min(max(p.seg[g + 1], lo), p.M);
        cnt[i] = (hi - lo + BM - 1) / BM;
      }
      sum += cnt[i];
    }
    int inc = sum;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int o = __shfl_up(inc, m, kWave);
      if (lane >= m) inc += o;
    }
    const int total = __shfl(inc, kWave - 1, kWave);
    if (lane == 0 && mt >= total) sched[0] = -1;
    int start = inc - sum;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      if (mt >= start && mt < start + cnt[i]) {
        const int g = lane * GPL + i;
        const int lo = min(max(p.seg[g], 0), p.M), hi = min(max(p.seg[g + 1], lo), p.M);
        sched[0] = g;
        sched[1] = lo + (mt - start) * BM;
        sched[2] = hi;
      }
      start += cnt[i];
    }
  }
  __syncthreads();
  const int g = sched[0];
  if (g < 0) return;
  const int row_lo = sched[1], row_hi = sched[2];

  const int K = p.K, Ncols = p.Ncols;
  const int lda = (int)p.lda;
  // uniform 64-bit bases, per-thread 32-bit offsets that do not change over K
  const E* At = static_cast<const E*>(p.A) + (int64_t)row_lo * p.lda;
  const E* Bg = static_cast<const E*>(p.B) + (int64_t)g * p.strideB;
  int a_off[C::A_PER_THREAD], a_k[C::A_PER_THREAD];
  bool a_ok[C::A_PER_THREAD];
#pragma unroll
  for (int i = 0; i < C::A_PER_THREAD; ++i) {
    const int idx = tid + i * C::THREADS;
    const int r = idx / KC, c = idx % KC;
    a_k[i] = c * CE;
    a_off[i] = r * lda + c * CE;
    a_ok[i] = idx < C::A_CHUNKS && row_lo + r < row_hi;
  }
  int b_off[C::B_PER_THREAD], b_k[C::B_PER_THREAD];
  bool b_ok[C::B_PER_THREAD];
#pragma unroll
  for (int i = 0; i < C::B_PER_THREAD; ++i) {
    const int idx = tid + i * C::THREADS;
    const int kb = idx / (BN / CE), nb = idx % (BN / CE);
    b_k[i] = kb * CE;
    b_off[i] = kb * CE * Ncols + n0 + nb * CE;
    b_ok[i] = idx < C::B_BLOCKS && n0 + nb * CE < Ncols;
  }

  // ---- global -> register loads of one K-step
  u32x4 ra[C::A_PER_THREAD];
  u32x4 rb[C::B_PER_THREAD][CE];
  auto load_tiles = [&](int k0) {
    const E* Ak = At + k0;
    const E* Bk = Bg + (int64_t)k0 * Ncols;
#pragma unroll
    for (int i = 0; i < C::A_PER_THREAD; ++i) {
      ra[i] = u32x4{0, 0, 0, 0};
      if (a_ok[i] && k0 + a_k[i] < K) ra[i] = load16(Ak + a_off[i]);
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_THREAD; ++i) {
      const bool ok = b_ok[i] && k0 + b_k[i] < K;
#pragma unroll
      for (int r = 0; r < CE; ++r)
        rb[i][r] = ok ? load16(Bk + b_off[i] + r * Ncols) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tiles = [&](int stage) {
    u32x4* as = As + stage * C::A_CHUNKS;
    u32x4* bs = Bs + stage * C::B_CHUNKS;
#pragma unroll
    for (int i = 0; i < C::A_PER_THREAD; ++i) {
      const int idx = tid + i * C::THREADS;
      if (idx < C::A_CHUNKS) {
        const int r = idx / KC, c = idx % KC;
        as[r * KC + (c ^ swz(r))] = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_PER_THREAD; ++i) {
      const int idx = tid + i * C::THREADS;
      if (idx < C::B_BLOCKS) {
        const int kb = idx / (BN / CE), nb = idx % (BN / CE);
        u32x4 t[CE];
        Transpose<E>::run(rb[i], t);
#pragma unroll
        for (int c = 0; c < CE; ++c) {
          const int n = nb * CE + c;
          bs[n * KC + (kb ^ swz(n))] = t[c];
        }
      }
    }
  };

  f32x16 acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  const int lrow = lane & 31, lhalf = lane >> 5;
  // operand fragments of one k-substep (16 bf16 / 8 fp32 of K), double-buffered
  // so that the LDS reads of substep s+1 are in flight during the MFMAs of s
  u32x4 fa[2][C::FN], fb[2][C::FM];
  auto load_frags = [&](const u32x4* as, const u32x4* bs, int s, int buf) {
    const int c = 2 * s + lhalf;
#pragma unroll
    for (int i = 0; i < C::FN; ++i) {
      const int n = wn * C::WTN + i * 32 + lrow;
      fa[buf][i] = bs[n * KC + (c ^ swz(n))];
    }
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int m = wm * C::WTM + j * 32 + lrow;
      fb[buf][j] = as[m * KC + (c ^ swz(m))];
    }
  };
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
    const u32x4* as = As + stage * C::A_CHUNKS;
    const u32x4* bs = Bs + stage * C::B_CHUNKS;
    load_frags(as, bs, 0, 0);
#pragma unroll
    for (int s = 0; s < KC / 2; ++s) {
      if (s + 1 < KC / 2) load_frags(as, bs, s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j) Mfma<E>::step(acc[i][j], fa[s & 1][i], fb[s & 1][j]);
    }
    if (kt + 1 < nk) store_tiles(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds row m = .. + lane%32, columns n = .. + 8*(r/4) + 4*(lane/32) + r%4
  O* Cp = static_cast<O*>(p.C);
  const E* bias = p.bias ? static_cast<const E*>(p.bias) + (int64_t)g * p.strideBias : nullptr;
#pragma unroll
  for (int j = 0; j < C::FM; ++j) {
    const int grow = row_lo + wm * C::WTM + j * 32 + lrow;
    if (grow >= row_hi) continue;
#pragma unroll
    for (int i = 0; i < C::FN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * C::WTN + i * 32 + 8 * q + 4 * lhalf;
        if (col >= Ncols) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[i][j][4 * q + r];
          if (bias) v[r] += ElemTraits<E>::to_f32(bias[col + r]);
          if (C::GELU) v[r] = gelu_erf(v[r]);
        }
        Store<O>::four(Cp + grow * p.ldc + col, v[0], v[1], v[2], v[3]);
      }
    }
  }
}

template <class C>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  int mtiles;
  if (p.seg == nullptr)
    mtiles = (p.M + C::BM - 1) / C::BM;
  else
    mtiles = p.M / C::BM + p.groups + 1;  // >= sum over groups of ceil(rows_g / BM)
  const int ntiles = (p.Ncols + C::BN - 1) / C::BN;
  if (mtiles <= 0 || ntiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_gemm_kernel<C>, dim3(mtiles, ntiles), dim3(C::THREADS), 0, s, p);
  return hipGetLastError();
}

constexpr int kNumCUs = 256;

// Tile shapes (BM x BN with WM x WN waves): the largest tile that still gives
// every CU a block, judged from the row bound M (the routing itself is only
// known on the device). Few rows per expert (decode) take thin row tiles that
// stream the weights.
template <typename E, typename O, bool G>
hipError_t launch_dtype(const GemmParams& p, int avg_rows, hipStream_t s) {
  if (avg_rows < 64) return launch_cfg<Cfg<E, O, 32, 256, 1, 4, G>>(p, s);
  const int groups = p.seg ? p.groups : 0;
  auto tiles = [&](int bm, int bn) {
    return (int64_t)(p.M / bm + groups) * ((p.Ncols + bn - 1) / bn);
  };
  if (tiles(256, 256) >= kNumCUs) return launch_cfg<Cfg<E, O, 256, 256, 2, 2, G>>(p, s);
  if (tiles(256, 128) >= kNumCUs) return launch_cfg<Cfg<E, O, 256, 128, 2, 2, G>>(p, s);
  return launch_cfg<Cfg<E, O, 128, 128, 2, 2, G>>(p, s);
}

}  // namespace

hipError_t launch_grouped_gemm(const GemmParams& p, GemmKind kind, bool bf16_, int avg_rows,
                               hipStream_t s) {
  switch (kind) {
    case GemmKind::kFfn1Gelu:
      return bf16_ ? launch_dtype<bf16, bf16, true>(p, avg_rows, s)
                   : launch_dtype<float, float, true>(p, avg_rows, s);
    case GemmKind::kFfn2:
      return bf16_ ? launch_dtype<bf16, bf16, false>(p, avg_rows, s)
                   : launch_dtype<float, float, false>(p, avg_rows, s);
    case GemmKind::kProjF32:
      return bf16_ ? launch_dtype<bf16, float, false>(p, avg_rows, s)
                   : launch_dtype<float, float, false>(p, avg_rows, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
