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
//  - The block computes a BM x BN tile of C. MFMA 16x16x32 (the ping-pong K
//    loop of long bf16 contractions) or 32x32x16 (every other loop) is used
//    in the transposed sense, D = B^T A^T: the weight tile is the MFMA's
//    first operand and the activation rows its second, so each lane ends up
//    with 4 consecutive output columns of one row (8- or 16-byte stores).
//    Both shapes do the same flops per cycle; 16x16x32 spends less energy
//    per flop, and the chip, held at its power cap by that loop, clocks
//    higher with it.
//  - Both tiles go global -> LDS with buffer_load_dwordx4 ... lds (no staging
//    registers), as they lie in memory: activation rows K-contiguous, weight
//    rows N-contiguous. The MFMA needs 8 consecutive K values of one weight
//    column per lane; gfx950's LDS transpose read (ds_read_b64_tr_b16)
//    delivers exactly that, so the weights are never transposed. The fp32
//    build reads single elements instead (its MFMA takes one K value per lane).
//  - 16-byte chunks are XOR-swizzled (swz_a, swz_b) so that every fragment
//    read is free of bank conflicts on gfx950's LDS.
//  - Four weight stages (three K-steps of loads in flight) and, for 64-byte
//    activation rows, two buffers holding the activation tile of two K-steps
//    each; within a step the fragment reads of substep s+1 overlap the MFMAs
//    of substep s.
//  - Ragged groups: the grid is an upper bound on the number of tiles; each
//    block finds its (group, rows, columns) from seg on the device, so no host
//    synchronisation is needed. A group's remainder of at most BM/2 rows goes
//    to tail tiles of 32 rows per wave, scheduled after all full-height tiles.
//    Blocks past the last tile exit at once.
//  - GEMM1's activation rows can be gathered (row r reads A row
//    gather[r] / gather_div) inside the tile loads.
//  - No split-K and no atomics: each output element is written once.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "gelu.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

#ifdef MOE_FFN_TRACE
__device__ uint64_t g_ffn_trace[kFfnTraceBlocks * kFfnTraceItems * kFfnTraceWords];
#endif

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

// cache-policy operand of the buffer builtins: sc1, agent scope (the access
// is coherent across the XCDs' L2s, the form the compiler gives agent-scope
// atomic loads and stores)
constexpr int kCpolSc1 = 16;

// 16 bytes per lane from the buffer at byte offset voff straight into LDS:
// lane l writes dst + 16 l (dst is wave-uniform). Out-of-range reads write zeros.
__device__ inline void lds_load16(__amdgpu_buffer_rsrc_t r, lds_void* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

// s_waitcnt that waits for at most n outstanding vector-memory operations
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at max).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same with no LDS operation outstanding (lgkmcnt 0). A wave issues it
// before a barrier after which other waves refill LDS it has been reading:
// gfx950's s_barrier does not wait for the wave's own LDS reads to complete
// (and the compiler adds no wait before a bare s_barrier), so a read still
// in flight could otherwise return the refilled data.
template <int N>
__device__ inline void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

constexpr int kNumXcds = 8;  // MI355X: 8 XCDs of 32 CUs, each with its own L2
// The single-launch FFN runs its 256 x 256 bf16 tiles with the two waves of
// each SIMD half a K-step apart (ping-pong, in gemm_tile) where both GEMMs
// have at least this many K-steps; shorter K loops keep one barrier per
// step, as the ping-pong's fixed cost per tile (one more MFMA interval,
// twice the barriers) outweighs its gain there.
constexpr int kPingPongMinSteps = 96;
constexpr int kGroupN = 4;   // n-tiles per run of the tile order
// Single launch with the ping-pong loop (long contractions): an XCD's
// GEMM2 tail items come after this many of its GEMM1 full items (two rounds
// of its 32 CUs, by which time its GEMM1 tail items, first in its queue,
// have completed).
constexpr int kTailsAfter = 64;
// Block-FP8 weights: registers of per-lane block scales a wave holds (64
// scale blocks each), which bounds K at 128 * 64 * kW8ScaleRegs.
constexpr int kW8ScaleRegs = kW8MaxK / (128 * 64);

// W8_: the weights are block-FP8 codes in K-groups of 8 (GemmW8) instead of
// E values; the activations stay E.
// DUAL_: GELU launches also store the pre-activation (GemmParams::C2).
template <typename E, typename O, int BM_, int BN_, int WM_, int WN_, int KC_, int S_, bool GELU_, bool W8_ = false,
          bool DUAL_ = false>
struct Cfg {
  using Elem = E;
  using Out = O;
  static constexpr bool W8 = W8_;
  static constexpr bool DUAL = DUAL_;
  static constexpr int ES = sizeof(E);
  static constexpr int CE = ElemTraits<E>::kPerChunk;   // elements per 16-byte chunk
  static constexpr int KC = KC_;                         // 16-byte chunks of K per activation row per stage
  static constexpr int BK = KC * CE;                     // K per stage
  static constexpr int S = S_;                           // LDS stages
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int THREADS = kWave * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr bool GELU = GELU_;
  // With 64-byte activation rows per K-step (KC = 4) one stage would use
  // half of each 128-byte cache line, and the other half, needed one step
  // later, has usually left the L1 by then. Such configurations load the
  // activation tile for two K-steps at once (AP = 2) into two buffers of
  // 128-byte rows, while the weight tile keeps its ring of S stages.
  static constexpr int AP = (KC == 4 && S == 4) ? 2 : 1;  // K-steps per activation stage
  static constexpr int KCA = KC * AP;                    // 16-byte chunks per activation row per stage
  // weight tile rows: K rows of BN values, or (W8) K-groups of BN x 8 codes
  static constexpr int B_ROWS = W8 ? BK / 8 : BK;
  static constexpr int B_CPR = W8 ? BN * 8 / 16 : BN * ES / 16;  // 16-byte chunks per weight tile row
  static constexpr int A_STAGE = BM * KCA * 16;          // activation tile, K-contiguous rows
  static constexpr int B_STAGE = B_ROWS * B_CPR * 16;    // weight tile
  static constexpr int A_INST = BM * KCA / THREADS;      // 16-byte loads per thread per activation stage
  static constexpr int B_INST = B_ROWS * B_CPR / THREADS;  // ... per weight stage
  static constexpr int LOADS = A_INST + B_INST;
  static constexpr int LDS_BYTES = AP == 1 ? S * (A_STAGE + B_STAGE) : 2 * A_STAGE + S * B_STAGE;
  // Ragged tails: the rows of a group past its last full BM-row tile go to
  // tiles of TBM = 32*WM rows (one 32-row fragment per wave), which load and
  // multiply a quarter (BM = 256) of a full tile's activation rows.
  static constexpr int TBM = 32 * WM;
  static constexpr bool HAS_TAIL = AP == 2 && TBM < BM;
  // bf16 activations and weights with 32-deep K-steps: the ping-pong K loop
  // takes 16x16x32 MFMAs (the same flops per cycle as 32x32x16, at less
  // energy per flop, so that the chip clocks higher under its power cap);
  // every other loop 32x32x16 (32x32x2 for fp32). Both give the same bits.
  static constexpr bool M16_OK = std::is_same_v<E, bf16> && !W8_ && KC_ == 4;
  static constexpr int A_INST_T = HAS_TAIL ? TBM * KCA / THREADS : A_INST;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold at least one 32x32 MFMA tile");
  static_assert(KC == 4 || KC == 8, "activation rows of 4 or 8 chunks");
  static_assert(BM * KCA % THREADS == 0 && B_ROWS * B_CPR % THREADS == 0, "loads must divide evenly");
  static_assert(!W8 || (std::is_same_v<E, bf16> && (128 / BK) * BK == 128 && WTN <= 128),
                "block-FP8 weights: bf16 activations, whole K-steps per 128-deep scale block, a wave's columns in one block");
  static_assert(B_CPR >= (ES == 2 ? 16 : 8) && WTN % 64 == 0, "weight rows of at least 256 (bf16) or 128 (fp32) bytes, wave tiles of 64 columns");
  static_assert(S >= 2 && S <= 4 && LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(LOADS * (S - 2) < 64 && A_INST + 2 * B_INST < 64, "vmcnt range");
  static_assert(!HAS_TAIL || (TBM * KCA % THREADS == 0 && A_INST_T >= 1), "tail tiles: whole loads per thread");
  static_assert(!M16_OK || (KCA == 8 && B_CPR >= 16), "16x16x32 fragments: paired 128-byte activation rows");
};

// Chunk swizzles, for gfx950's LDS as measured with bank-conflict counters:
// 64 banks of 4 bytes (a 256-byte line); a 16-byte read serves 16 lanes per
// pass, lanes {0-3, 12-15, 20-23, 24-27} (and {4-7, 8-11, 16-19, 28-31}, and
// the same sets plus 32); 8-byte reads, transposing or not, serve 32
// consecutive lanes per pass. A pass is conflict-free when its lanes hit
// distinct banks. Activation rows hold KC chunks; chunk c of row r sits at
// c ^ fa(r). A fragment read gives lane l row l%32, so one pass touches rows
// whose r/4 values share a parity: for 64-byte rows fa = (r/4)%4 spreads
// each pass over the 16 chunk slots of a line, for 128-byte rows
// fa = (r%8) ^ ((r/8)%2) does. Weight rows (bf16) hold B_CPR >= 16 chunks;
// chunk c of row k sits at c ^ fb(k), so that the 4 rows x 64 bytes one pass
// of a transpose read touches land in 4 distinct 64-byte windows of a line.
// The fp32 weight reads are 4-byte scalars; their rows take c ^ 2(k%4).
template <int KC> __device__ inline int swz_a(int r) {
  return KC == 8 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3);
}
template <int ES> __device__ inline int swz_b(int k) {
  return ES == 2 ? ((2 * (k & 3)) ^ (8 * (k & 1))) : 2 * (k & 3);
}
// Epilogue slices (32 rows of 8 or 16 chunks): chunk c of row r sits at
// c ^ swz_c(r). Row reads (ds_read_b128, CPR lanes per row) stay free of bank
// conflicts; the fragment writes (one column chunk, 32 rows) go in two passes
// for 8-byte pieces (the minimum for 16 distinct bank pairs) and one per
// 16 lanes for 16-byte pieces.
template <int OB> __device__ inline int swz_c(int r) { return OB == 2 ? ((r >> 1) & 7) : (r & 15); }
// 16x16x32 fragments (M16) read other rows together: lane l of an
// activation read takes row l % 16 of a 16-row block, chunk l / 16, so a
// pass of 16 lanes ({0-3, 12-15, 20-23, 24-27} and the like) reads rows
// 0-3 and 12-15 of one chunk and rows 4-7 and 8-11 of the next; with
// 2 ((r / 2) % 4) each row parity's eight reads land in eight distinct
// chunk slots. A weight read takes K-rows 8q .. 8q + 3 (lane group q) of the
// same 16 columns in all four groups, so rows 8 apart get the chunk slots
// the plain swizzle leaves free (^ 8).
template <int KCA, bool M16> __device__ inline int swz_act(int r) {
  if constexpr (M16) return 2 * ((r >> 1) & 3);
  else return swz_a<KCA>(r);
}
template <int ES, bool M16> __device__ inline int swz_wt(int k) {
  if constexpr (M16) return swz_b<2>(k) ^ (8 * ((k >> 3) & 1));
  else return swz_b<ES>(k);
}
// acc (one 16x16 sub-block of outputs) += weight fragment wf x activation
// fragment af
__device__ inline void mfma16(f32x4& acc, const u32x4& wf, const u32x4& af) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf), __builtin_bit_cast(bf16x8, af), acc, 0,
                                                0, 0);
}

// 4 floats as O into LDS: 8 bytes (bf16) or 16 bytes (fp32)
template <typename O> struct Pack;
template <> struct Pack<bf16> {
  __device__ static inline void four_lds(char* dst, const float* v) {
    u32x2 w;
    w[0] = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
    w[1] = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
    *(__attribute__((address_space(3))) u32x2*)dst = w;
  }
};
template <> struct Pack<float> {
  __device__ static inline void four_lds(char* dst, const float* v) {
    *(__attribute__((address_space(3))) f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
  }
};

// LDS objects of a block of configuration C (declared in each kernel).
#define MOE_GEMM_LDS(C) \
  constexpr int ST = C::AP == 1 ? C::A_STAGE + C::B_STAGE : C::B_STAGE; \
  constexpr int SA = C::AP == 1 ? 16 : C::A_STAGE; \
  __shared__ __attribute__((aligned(1024))) char st0[ST]; \
  __shared__ __attribute__((aligned(1024))) char st1[ST]; \
  __shared__ __attribute__((aligned(1024))) char st2[C::S > 2 ? ST : 16]; \
  __shared__ __attribute__((aligned(1024))) char st3[C::S > 3 ? ST : 16]; \
  __shared__ __attribute__((aligned(1024))) char sa0[SA]; \
  __shared__ __attribute__((aligned(1024))) char sa1[SA];

// One BM x BN output tile (rows [row_lo, row_hi) of group g, columns from
// n0; TBM rows if tail_tile): the K loop and the epilogue, GELU'd if gelu.
// All threads of the block call it with the same arguments; the LDS
// objects are the block's (MOE_GEMM_LDS). at_k_end() runs between the K
// loop and the epilogue. bscale: the block scales of W8 weights (GemmW8),
// else unused. coherent_out: the outputs are stored agent-coherently (sc1),
// for blocks on other XCDs to read once the stores have completed.
// PINGPONG: the K loop of 256 x 256 bf16 tiles runs the ping-pong schedule.
template <class C, bool PINGPONG, class AtKEnd>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, bool gelu, char* st0, char* st1, char* st2,
                                          char* st3, char* sa0, char* sa1, int g, int row_lo, int row_hi,
                                          int n0, bool tail_tile, const float* bscale, AtKEnd&& at_k_end,
                                          bool coherent_out = false) {
  using E = typename C::Elem;
  using O = typename C::Out;
  constexpr int CE = C::CE, KC = C::KC, BK = C::BK, ES = C::ES, S = C::S;
  constexpr int AP = C::AP, KCA = C::KCA;
  // 16x16x32 MFMAs in the ping-pong loop (see Cfg::M16_OK)
  constexpr bool M16 = C::M16_OK && PINGPONG && C::THREADS == 512;
  constexpr int ST = AP == 1 ? C::A_STAGE + C::B_STAGE : C::B_STAGE;  // bytes of st0..st3
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int K = p.K, Ncols = p.Ncols;
  const int lda = (int)p.lda;
  const int rows = row_hi - row_lo;
  // A rows of the tile: contiguous from row_lo, or gathered (then the
  // descriptor spans all of A and each lane's offsets name its rows)
  // weight bytes per element, and per column of a weight tile row (W8:
  // the 8 codes of a K-group; moving k0 rows down moves k0 * Ncols bytes
  // in both layouts, k0 a multiple of 8)
  constexpr int WES = C::W8 ? 1 : ES, WCB = C::W8 ? 8 : ES;
  const char* At = static_cast<const char*>(p.A) + (p.gather ? 0 : (int64_t)row_lo * p.lda * ES);
  const char* Bt = static_cast<const char*>(p.B) + (int64_t)g * p.strideB * WES + (int64_t)n0 * WCB;
  const int64_t a_bytes = (int64_t)(p.gather ? p.a_rows : rows) * lda * ES;
  const int64_t b_bytes = (int64_t)K * Ncols * WES - (int64_t)n0 * WCB;

  // ---- asynchronous global -> LDS loads. Each 16-byte load of a wave lands
  // at (wave's slot base + lane) * 16 in the stage; the lane fetches whichever
  // chunk the swizzle puts in that slot. Offsets are fixed over K; each
  // K-step moves the descriptor base to k0 and shrinks its extent to what
  // remains (zero past K), so the hardware range check supplies zeros for
  // rows past the group and for K past the end. (Activation rows are exactly
  // K long: a load past K in one row reads the next row, which meets zero
  // weights.) Columns past Ncols read neighbouring data and only feed
  // outputs that are never stored.
  int a_off[C::A_INST], b_off[C::B_INST];
#pragma unroll
  for (int i = 0; i < C::A_INST; ++i) {
    const int slot = i * C::THREADS + tid;
    const int r = slot / KCA, c = (slot % KCA) ^ swz_act<KCA, M16>(r);
    if (p.gather) {
      // rows past the group read zeros: an offset past the descriptor's range
      const int grow = row_lo + r;
      a_off[i] = grow < row_hi ? ((p.gather[grow] / p.gather_div) * lda + c * CE) * ES : (int)kOutOfRange;
    } else {
      a_off[i] = (r * lda + c * CE) * ES;
    }
  }
#pragma unroll
  for (int i = 0; i < C::B_INST; ++i) {
    const int slot = i * C::THREADS + tid;
    if constexpr (C::W8) {
      // K-group rows of BN x 8 codes, stored as in memory (the fragment
      // reads of one pass cover 256 contiguous bytes: no swizzle needed)
      b_off[i] = (slot / C::B_CPR) * Ncols * 8 + (slot % C::B_CPR) * 16;
    } else {
      const int k = slot / C::B_CPR, c = (slot % C::B_CPR) ^ swz_wt<ES, M16>(k);
      b_off[i] = (k * Ncols + c * CE) * ES;
    }
  }
  auto issue_b = [&](char* sb, int k0) {
    const int64_t bb = b_bytes - (int64_t)k0 * Ncols * WES;
    const __amdgpu_buffer_rsrc_t br = make_rsrc(Bt + (int64_t)k0 * Ncols * WES, (uint32_t)(bb > 0 ? bb : 0));
#pragma unroll
    for (int i = 0; i < C::B_INST; ++i)
      lds_load16(br, (lds_void*)(sb + (i * C::THREADS + wave * kWave) * 16), b_off[i]);
  };
  // stage i's buffers (i constant, so that each access names its LDS object)
  auto a_stage = [&](auto i) -> char* {
    constexpr int v = decltype(i)::value;
    if constexpr (AP == 2) return (v / 2) % 2 == 0 ? sa0 : sa1;
    else return v == 0 ? st0 : v == 1 ? st1 : v == 2 ? st2 : st3;
  };
  auto b_stage = [&](auto i) -> char* {
    constexpr int v = decltype(i)::value;
    char* const base = v == 0 ? st0 : v == 1 ? st1 : v == 2 ? st2 : st3;
    return AP == 2 ? base : base + C::A_STAGE;
  };

  // The K loop and the epilogue, for full tiles and (TAIL) for ragged-tail
  // tiles of TBM rows: one 32-row fragment per wave and the first A_INST_T
  // activation loads per thread; everything else is the same code.
  auto run = [&](auto tail_c) {
    constexpr bool TAIL = decltype(tail_c)::value;
    constexpr int FM = TAIL ? 1 : C::FM;                 // 32-row fragments per wave
    constexpr int WTM = TAIL ? 32 : C::WTM;              // rows per wave
    constexpr int AI = TAIL ? C::A_INST_T : C::A_INST;   // activation loads per thread per stage
    auto issue_a = [&](char* sa, int k0) {
      const int64_t ab = a_bytes - (int64_t)k0 * ES;
      const __amdgpu_buffer_rsrc_t ar = make_rsrc(At + (int64_t)k0 * ES, (uint32_t)(ab > 0 ? ab : 0));
#pragma unroll
      for (int i = 0; i < AI; ++i)
        lds_load16(ar, (lds_void*)(sa + (i * C::THREADS + wave * kWave) * 16), a_off[i]);
    };

    f32x16 acc[C::FN][FM];
    if constexpr (!M16) {
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }
    // M16: the K loop's accumulators, 16x16 sub-block Q = 2a + b of each
    // 32x32 block (copied into acc[.][.][4Q .. 4Q+3] after the loop)
    f32x4 acq[M16 ? C::FN : 1][M16 ? FM : 1][4];
    if constexpr (M16) {
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) acq[i][j][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // W8: acc holds the current 128-deep block of K; acc8 the scaled total
    f32x16 acc8[C::W8 ? C::FN : 1][C::W8 ? FM : 1];
    // W8: the wave's block scales (one per 128-deep block of K: its columns
    // lie in one scale block; a wave wholly past Ncols, whose outputs are
    // never stored, takes the last block's, so that the reads stay in the
    // array), read before the K loop into lane b % 64 of register b / 64.
    // A read inside the loop would complete behind the step's global->LDS
    // loads, and its wait would drain the whole load pipeline.
    float scl[C::W8 ? kW8ScaleRegs : 1];
    if constexpr (C::W8) {
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc8[i][j][r] = 0.f;
      const int wn_u = __builtin_amdgcn_readfirstlane(wn);
      const int cb = min((n0 + wn_u * C::WTN) / 128, Ncols / 128 - 1);
      const int nkb = K / 128;
#pragma unroll
      for (int r = 0; r < kW8ScaleRegs; ++r) {
        const int b = 64 * r + lane;
        scl[r] = b < nkb ? bscale[((int64_t)g * nkb + b) * (Ncols / 128) + cb] : 0.f;
      }
    }

    // ---- per-lane fragment offsets within a stage
    const int lrow = lane & 31, lhalf = lane >> 5;
    // activation fragment (MFMA second operand): row wm*WTM + 32j + lane%32,
    // chunk 2s + lane/32 (swizzled); one offset per substep
    // (AP == 2: the first K-step of a pair; the second reads chunk + KC, and as
    // the swizzle only permutes the low three chunk bits, that is offset ^ 64)
    int fa_off[KC / 2];
#pragma unroll
    for (int ss = 0; ss < KC / 2; ++ss)
      fa_off[ss] = (wm * WTM + lrow) * KCA * 16 + (((2 * ss + lhalf) ^ swz_act<KCA, M16>(lrow)) * 16);
    // 16x16x32 (M16): the activation fragment of m-half b of 32-row block j
    // is row wm*WTM + 32j + 16b + lane%16, chunk lane/16 (8 consecutive K),
    // at fa16 + (32j + 16b) rows; the weight fragment of n-half a of 32-column
    // block i is column wn*WTN + 32i + 16a + lane%16, K-rows 8(lane/16) + 0..7,
    // two transposing reads of 4 K-rows each from fw16[i][a] (in each 16-lane
    // group, lane 4q + r reads K-row q, columns 4r .. 4r+3 of the group's 16)
    const int l16 = lane & 15, g16 = lane >> 4;
    const int fa16 = (wm * WTM + l16) * KCA * 16 + ((g16 ^ swz_act<KCA, M16>(l16)) * 16);
    int fw16[M16 ? C::FN : 1][2];
    if constexpr (M16) {
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int k = 8 * g16 + (l16 >> 2);
          const int chunk = wn * C::WTN / 8 + 4 * i + 2 * a + ((l16 & 3) >> 1);
          fw16[i][a] = k * C::B_CPR * 16 + ((chunk ^ swz_wt<ES, M16>(k)) * 16) + 8 * (l16 & 1);
        }
    }
    // weight fragment, bf16: 16-lane group q, lane r in it: rows 16s + 8(q/2) + 4p + r/4,
    // columns wn*WTN + 32i + 16(q%2) + 4(r%4) .. +3; the row's swizzle depends on r/4 only
    const int q16 = lane >> 4, r16 = lane & 15;
    int fw[C::FN];
#pragma unroll
    for (int i = 0; i < C::FN; ++i) {
      const int chunk = wn * C::WTN / 8 + 4 * i + 2 * (q16 & 1) + ((r16 & 3) >> 1);
      fw[i] = (8 * (q16 >> 1) + (r16 >> 2)) * C::B_CPR * 16 + (chunk ^ swz_b<ES>(r16 >> 2)) * 16 + 8 * (r16 & 1);
    }
    // weight fragment, fp32: row 8s + 4(lane/32) + e, column wn*WTN + 32i + lane%32
    int fw32[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      fw32[e] = (4 * lhalf + e) * C::B_CPR * 16 + (wn * C::WTN / 4 + ((lrow >> 2) ^ swz_b<ES>(e))) * 16 + (lrow & 3) * 4;

    u32x4 fa[2][C::FN], fb[2][FM];
    auto load_frags = [&](const char* sa, const char* sb, int ss, int buf, int hi) {
      if constexpr (M16) {
        // half ss of the K-step's fragments: m-half ss of every row block,
        // n-half ss of every column block
#pragma unroll
        for (int j = 0; j < FM; ++j)
          fb[buf][j] = *(lds_u32x4*)(sa + (fa16 ^ hi) + (j * 32 + 16 * ss) * KCA * 16);
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
          const char* w = sb + fw16[i][ss];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)w);
          const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(w + 4 * C::B_CPR * 16));
          const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, up);
          fa[buf][i] = u32x4{x[0], x[1], y[0], y[1]};
        }
        return;
      }
#pragma unroll
      for (int j = 0; j < FM; ++j)
        fb[buf][j] = *(lds_u32x4*)(sa + (fa_off[ss] ^ hi) + j * 32 * KCA * 16);
      if constexpr (C::W8) {
        // the lane's 8 codes: K-group 2ss + lane/32 of column lane%32 of
        // fragment i, converted exactly to bf16 (E4M3 values fit bf16)
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
          const u32x2 raw =
              *(const __attribute__((address_space(3))) u32x2*)(sb + ((2 * ss + lhalf) * C::BN + wn * C::WTN +
                                                                      32 * i + lrow) * 8);
          fa[buf][i] = u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[0], 1.f, false)),
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[0], 1.f, true)),
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[1], 1.f, false)),
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw[1], 1.f, true))};
        }
      } else if constexpr (ES == 2) {
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
          const char* w = sb + fw[i];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(w + (16 * ss) * C::B_CPR * 16));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(w + (16 * ss + 4) * C::B_CPR * 16));
          const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
          fa[buf][i] = u32x4{x[0], x[1], y[0], y[1]};
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            fa[buf][i][e] = *(lds_u32*)(sb + fw32[e] + (8 * ss) * C::B_CPR * 16 + i * 128);
      }
    };
    // M16: the K-step's 4 FN FM MFMAs once both halves are in registers;
    // the first quarter needs only half 0
    auto mma16 = [&]() {
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) mfma16(acq[i][j][0], fa[0][i], fb[0][j]);
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) mfma16(acq[i][j][1], fa[0][i], fb[1][j]);
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) mfma16(acq[i][j][2], fa[1][i], fb[0][j]);
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) mfma16(acq[i][j][3], fa[1][i], fb[1][j]);
    };
    auto compute = [&](const char* sa, const char* sb, int hi) {
      if constexpr (M16) {
        load_frags(sa, sb, 0, 0, hi);
        load_frags(sa, sb, 1, 1, hi);
        mma16();
        return;
      }
      load_frags(sa, sb, 0, 0, hi);
#pragma unroll
      for (int ss = 0; ss < KC / 2; ++ss) {
        if (ss + 1 < KC / 2) load_frags(sa, sb, ss + 1, (ss + 1) & 1, hi);
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
          for (int j = 0; j < FM; ++j) Mfma<E>::step(acc[i][j], fa[ss & 1][i], fb[ss & 1][j]);
      }
    };

    // ---- S-stage pipeline, one barrier per K-step: wait until this step's
    // loads have landed (later steps' loads may still be in flight) and this
    // wave's reads of the previous stage have returned, barrier (everyone's
    // loads visible; everyone done with the previous stage), start
    // the loads S-1 steps ahead into the stage just freed, compute.
    // AP == 2 (S == 4): even steps also start the activation pair two steps
    // ahead into the buffer the previous pair used. The counts hold whatever
    // order the compiler gives the loads within a step: an even step waits for
    // everything but the previous step's weight loads (this step's pair was
    // started two steps back), an odd step for everything but the last two
    // steps' loads (its weights were started three steps back, by an even step).
    // (The prologue's loads are issued in program order, scheduling barriers
    // between them.)
    const int nk = (K + BK - 1) / BK;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    issue_a(a_stage(I0{}), 0);
    __builtin_amdgcn_sched_barrier(0);
    issue_b(b_stage(I0{}), 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (S > 2) {
      if constexpr (AP == 1) issue_a(a_stage(I1{}), BK);
      issue_b(b_stage(I1{}), BK);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (S > 3) {
      if constexpr (AP == 1) issue_a(a_stage(I2{}), 2 * BK);
      issue_b(b_stage(I2{}), 2 * BK);
    }
    auto step = [&](auto st, int kt) {
      constexpr int cur = decltype(st)::value;
      constexpr int nxt = (cur + S - 1) % S;
      if constexpr (AP == 1) wait_vmcnt_lds<(AI + C::B_INST) * (S - 2)>();
      else if constexpr (cur % 2 == 0) wait_vmcnt_lds<C::B_INST>();
      else wait_vmcnt_lds<AI + 2 * C::B_INST>();
      __builtin_amdgcn_s_barrier();
      const int kn = (kt + S - 1) * BK;
      if constexpr (AP == 1) issue_a(a_stage(std::integral_constant<int, nxt>{}), kn);
      else if constexpr (cur % 2 == 0) issue_a(a_stage(std::integral_constant<int, (cur + 2) % 4>{}), (kt + 2) * BK);
      issue_b(b_stage(std::integral_constant<int, nxt>{}), kn);
      compute(a_stage(st), b_stage(st), (AP == 2 && (cur & 1)) ? 64 : 0);
      if constexpr (C::W8) {
        constexpr int SPB = 128 / BK;  // K-steps per scale block
        static_assert(S % SPB == 0, "scale blocks end on fixed stages");
        if constexpr ((cur + 1) % SPB == 0) {
          // the end of a 128-deep block of K: its sums, scaled once, join
          // the total
          const int b = __builtin_amdgcn_readfirstlane(kt / SPB);
          float sc = 0.f;
#pragma unroll
          for (int r = 0; r < kW8ScaleRegs; ++r) {
            const float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, scl[r]), b & 63));
            if ((b >> 6) == r) sc = v;
          }
#pragma unroll
          for (int i = 0; i < C::FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                acc8[i][j][r] = fmaf(sc, acc[i][j][r], acc8[i][j][r]);
                acc[i][j][r] = 0.f;
              }
        }
      }
      if constexpr (ES == 2 && C::THREADS == 512 && !M16) {
        // (8-wave tiles) instruction order for the step: the first substep's LDS reads, then
        // each MFMA followed by one of the next substep's LDS reads and, after
        // every second MFMA, one of the step's global->LDS loads, so that the
        // loads reach the address unit evenly spread over the step
        constexpr int DSR = FM + (C::W8 ? 1 : 2) * C::FN;  // LDS reads per substep
        constexpr int MF = FM * C::FN;
        constexpr int VM = (AP == 1 || cur % 2 == 0) ? (AI + C::B_INST) : C::B_INST;
        __builtin_amdgcn_sched_group_barrier(0x100, DSR, 0);
#pragma unroll
        for (int ss = 0; ss < KC / 2; ++ss)
#pragma unroll
          for (int m = 0; m < MF; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (ss + 1 < KC / 2 && m < DSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if ((ss * MF + m) % 2 == 1 && (ss * MF + m) / 2 < VM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
          }
      }
    };
    // whole groups of S steps run as one straight-line loop body: steps guarded
    // by a branch inside the body make the compiler merge its load tracking at
    // the loop head and drain every load in flight there once per iteration
    auto one_barrier_loop = [&]() {
      int kt = 0;
      for (; kt + S <= nk; kt += S) {
        step(std::integral_constant<int, 0>{}, kt);
        step(std::integral_constant<int, 1>{}, kt + 1);
        if constexpr (S > 2) step(std::integral_constant<int, 2 % S>{}, kt + 2);
        if constexpr (S > 3) step(std::integral_constant<int, 3 % S>{}, kt + 3);
      }
      if (kt < nk) step(std::integral_constant<int, 0>{}, kt);
      if constexpr (S > 2) if (kt + 1 < nk) step(std::integral_constant<int, 1>{}, kt + 1);
      if constexpr (S > 3) if (kt + 2 < nk) step(std::integral_constant<int, 2 % S>{}, kt + 2);
    };
    constexpr bool PP = PINGPONG && ES == 2 && !C::W8 && AP == 2 && S == 4 && C::THREADS == 512;
    if constexpr (!PP) {
      one_barrier_loop();
    } else {
      // Ping-pong: waves 0-3 and 4-7 (one of each per SIMD) run the same
      // steps half a step apart, two barriers per step, so that while one
      // wave of a SIMD issues a step's MFMAs (operands already in registers)
      // the other reads its next fragments and issues its loads. Group 0:
      // [mem(s) | mma(s)] per step; group 1: [mma(s-1) | mem(s)], its first
      // mma on zero fragments (adds nothing) and its last after the loop.
      // Every wave passes the same barriers: two per step in either order.
      // Before the barrier that precedes group 0's mem(t), every wave waits
      // for its loads of step t (both groups have then issued mem(0..t-1)):
      // all but the last 2 B_INST loads (t even: mem issues a pair's loads
      // ahead of the weight loads, a scheduling barrier keeping that order,
      // so the last two weight stages were issued after step t's pair) or
      // AI + 2 B_INST (t odd); before the other barrier only for its LDS reads.
      const int grp = wave >> 2;
      // The memory phase runs at raised wave priority, so that its reads and
      // loads issue ahead of the other wave's MFMAs (measured: +0.5 % on the
      // large-expert FFN against no priority change; raising the MFMA phase's
      // priority instead lost 1 %).
      auto mem = [&](auto st, int kt) {
        constexpr int cur = decltype(st)::value;
        constexpr int nxt = (cur + S - 1) % S;
        __builtin_amdgcn_s_setprio(1);
        if constexpr (cur % 2 == 0) {
          issue_a(a_stage(std::integral_constant<int, (cur + 2) % 4>{}), (kt + 2) * BK);
          __builtin_amdgcn_sched_barrier(0);  // the pair's loads ahead of the weight loads
        }
        issue_b(b_stage(std::integral_constant<int, nxt>{}), (kt + S - 1) * BK);
        load_frags(a_stage(st), b_stage(st), 0, 0, (cur & 1) ? 64 : 0);
        load_frags(a_stage(st), b_stage(st), 1, 1, (cur & 1) ? 64 : 0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto mma = [&]() {
        if constexpr (M16) {
          mma16();
        } else {
#pragma unroll
          for (int ss = 0; ss < 2; ++ss)
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
              for (int j = 0; j < FM; ++j) Mfma<E>::step(acc[i][j], fa[ss][i], fb[ss][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      // waits before the barrier ahead of group 0's mem(t)
      auto sync_data = [&](auto t_c) {
        if constexpr (decltype(t_c)::value % 2 == 0) wait_vmcnt_lds<2 * C::B_INST>();
        else wait_vmcnt_lds<AI + 2 * C::B_INST>();
        __builtin_amdgcn_s_barrier();
      };
      auto sync_lds = [&]() {
        wait_vmcnt_lds<63>();
        __builtin_amdgcn_s_barrier();
      };
      using J0 = std::integral_constant<int, 0>;
      using J1 = std::integral_constant<int, 1>;
      using J2 = std::integral_constant<int, 2>;
      using J3 = std::integral_constant<int, 3>;
      sync_data(J0{});
      if (grp == 0) {
        auto one = [&](auto st, int kt) {
          mem(st, kt);
          sync_lds();
          mma();
          sync_data(std::integral_constant<int, (decltype(st)::value + 1) % 2>{});
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
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < C::FN; ++i) fa[b][i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int j = 0; j < FM; ++j) fb[b][j] = u32x4{0u, 0u, 0u, 0u};
        auto one = [&](auto st, int kt) {
          mma();  // step kt - 1 (zero fragments before step 0)
          sync_lds();
          mem(st, kt);
          sync_data(std::integral_constant<int, (decltype(st)::value + 1) % 2>{});
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
        mma();  // step nk - 1
      }
    }
    if constexpr (C::W8) {
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = acc8[i][j];
    }
    if constexpr (M16) {
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][4 * q + r] = acq[i][j][q][r];
    }
    wait_vmcnt<0>();
    at_k_end();

    // The lane's bias values: 4 consecutive columns per (fragment, 8-column
    // group), the same for every row, one buffer load each for the whole
    // tile (columns past Ncols read zeros; d and h are multiples of the
    // 16-byte chunk, so no group of 4 straddles Ncols).
    const bool has_bias = p.bias != nullptr;
    const int ccol0 = n0 + wn * C::WTN;
    u32x4 bv[C::FN][4];
    if (has_bias) {
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(static_cast<const char*>(p.bias) + (int64_t)g * p.strideBias * ES, (uint32_t)(Ncols * ES));
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // M16: the lane's columns are 32i + 16q + 4(lane/16) .. +3 (q < 2)
          if (M16 && q >= 2) continue;
          const int off = (ccol0 + i * 32 + (M16 ? 16 * q + 4 * g16 : 8 * q + 4 * lhalf)) * ES;
          if constexpr (ES == 2) {
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rb, off, 0, 0);
            bv[i][q] = u32x4{w[0], w[1], 0u, 0u};
          } else {
            bv[i][q] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
          }
        }
    }

    // ---- epilogue. The lane holds row .. + lane%32, columns .. + 8*(r/4) +
    // 4*(lane/32) + r%4 of each 32x32 fragment. Stored from there, one store
    // instruction would cover 32 rows with 16 bytes each, and the L2 would see
    // a request per 16 bytes. Instead each 32-row slice of the wave's tile is
    // finished in registers (bias, GELU, conversion), written to a per-wave
    // LDS region, and read back as 16-byte pieces of rows, CPR lanes per row,
    // so that every store writes whole 128- or 256-byte row segments.
    __syncthreads();  // every wave is done reading the stage buffers
    constexpr int OB = sizeof(O);
    constexpr int CPR = C::WTN * OB / 16;  // 16-byte chunks per slice row
    constexpr int RPI = kWave / CPR;       // slice rows per 64-lane read
    constexpr int REG = 32 * CPR * 16;     // bytes of one slice
    // wave w's region: slot w / S of stage buffer w % S while the stage
    // buffers hold every wave's; past that (8-wave 128 x 128 tiles), the
    // activation pair buffers, two regions each
    constexpr int WPS = (C::THREADS / kWave + S - 1) / S;  // waves per stage buffer
    constexpr int PST = ST / REG;                          // regions per stage buffer
    constexpr int PSA = AP == 2 ? C::A_STAGE / REG : 0;    // regions per activation pair buffer
    static_assert(WPS <= PST || (AP == 2 && PST >= 1 && PST * S + 2 * PSA >= C::THREADS / kWave),
                  "epilogue slices fit the stage buffers");
    char* reg;
    const int wsel = wave % S;
    if constexpr (WPS <= PST) {
      reg = (wsel == 0 ? st0 : wsel == 1 ? st1 : wsel == 2 ? st2 : st3) + (wave / S) * REG;
    } else {
      const int w2 = wave - PST * S;
      if (w2 < 0) reg = (wsel == 0 ? st0 : wsel == 1 ? st1 : wsel == 2 ? st2 : st3) + (wave / S) * REG;
      else reg = (w2 / PSA == 0 ? sa0 : sa1) + (w2 % PSA) * REG;
    }
    if constexpr (C::DUAL) {
      // both the pre-activation (C2) and the activation (C), each slice
      // through the same region
      // slice j's values (acc[.][j]) through the wave's region into rows of Dp
      auto store_slice = [&](O* Dp, int j, int frow) {
  #pragma unroll
        for (int i = 0; i < C::FN; ++i) {
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            // slice row and byte offset in it of acc[i][j][4q .. 4q+3]: M32
            // row lane%32, columns 32i + 8q + 4(lane/32); M16 (sub-block q =
            // 2a + b) row 16b + lane%16, columns 32i + 16a + 4(lane/16)
            const int srow = M16 ? 16 * (q & 1) + l16 : lrow;
            const int cb = (i * 32 + (M16 ? 16 * (q >> 1) + 4 * g16 : 8 * q + 4 * lhalf)) * OB;
            float v[4];
  #pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
            Pack<O>::four_lds(reg + srow * CPR * 16 + (((cb / 16) ^ swz_c<OB>(srow)) * 16) + cb % 16, v);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  #pragma unroll
        for (int t = 0; t < 32 / RPI; ++t) {
          const int rr = t * RPI + lane / CPR, ch = lane % CPR;
          const u32x4 val = *(lds_u32x4*)(reg + rr * CPR * 16 + ((ch ^ swz_c<OB>(rr)) * 16));
          const int col = ccol0 + ch * (16 / OB);
          if (frow + rr < row_hi && col < Ncols) {
            if (coherent_out) {
              // the slice's 32 rows as one buffer range
              const __amdgpu_buffer_rsrc_t rc = make_rsrc(Dp + (int64_t)frow * p.ldc, (uint32_t)(32 * p.ldc * OB));
              __builtin_amdgcn_raw_buffer_store_b128(val, rc, (rr * (int)p.ldc + col) * OB, 0, kCpolSc1);
            } else {
              *reinterpret_cast<u32x4*>(Dp + (int64_t)(frow + rr) * p.ldc + col) = val;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      };
  #pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int frow = row_lo + wm * WTM + j * 32;
        if (frow >= row_hi) break;  // wave-uniform
        // bias and GELU over the whole slice, each behind one uniform branch
        if (has_bias) {
  #pragma unroll
          for (int i = 0; i < C::FN; ++i)
  #pragma unroll
            for (int q = 0; q < 4; ++q)
  #pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][j][4 * q + r] += chunk_elem<E>(bv[i][M16 ? q >> 1 : q], r);
        }
        store_slice(static_cast<O*>(p.C2), j, frow);  // the pre-activation
        if (gelu) {
  #pragma unroll
          for (int i = 0; i < C::FN; ++i)
  #pragma unroll
            for (int r = 0; r < 16; ++r)
              acc[i][j][r] = std::is_same_v<O, bf16> ? gelu_erf_bf16(acc[i][j][r]) : gelu_erf(acc[i][j][r]);
        }
        store_slice(static_cast<O*>(p.C), j, frow);
      }
    } else {
      O* Cp = static_cast<O*>(p.C);
  #pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int frow = row_lo + wm * WTM + j * 32;
        if (frow >= row_hi) break;  // wave-uniform
        // bias and GELU over the whole slice, each behind one uniform branch
        if (has_bias) {
  #pragma unroll
          for (int i = 0; i < C::FN; ++i)
  #pragma unroll
            for (int q = 0; q < 4; ++q)
  #pragma unroll
              for (int r = 0; r < 4; ++r) acc[i][j][4 * q + r] += chunk_elem<E>(bv[i][M16 ? q >> 1 : q], r);
        }
        if (gelu) {
  #pragma unroll
          for (int i = 0; i < C::FN; ++i)
  #pragma unroll
            for (int r = 0; r < 16; ++r)
              acc[i][j][r] = std::is_same_v<O, bf16> ? gelu_erf_bf16(acc[i][j][r]) : gelu_erf(acc[i][j][r]);
        }
  #pragma unroll
        for (int i = 0; i < C::FN; ++i) {
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            // slice row and byte offset in it of acc[i][j][4q .. 4q+3]: M32
            // row lane%32, columns 32i + 8q + 4(lane/32); M16 (sub-block q =
            // 2a + b) row 16b + lane%16, columns 32i + 16a + 4(lane/16)
            const int srow = M16 ? 16 * (q & 1) + l16 : lrow;
            const int cb = (i * 32 + (M16 ? 16 * (q >> 1) + 4 * g16 : 8 * q + 4 * lhalf)) * OB;
            float v[4];
  #pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r];
            Pack<O>::four_lds(reg + srow * CPR * 16 + (((cb / 16) ^ swz_c<OB>(srow)) * 16) + cb % 16, v);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  #pragma unroll
        for (int t = 0; t < 32 / RPI; ++t) {
          const int rr = t * RPI + lane / CPR, ch = lane % CPR;
          const u32x4 val = *(lds_u32x4*)(reg + rr * CPR * 16 + ((ch ^ swz_c<OB>(rr)) * 16));
          const int col = ccol0 + ch * (16 / OB);
          if (frow + rr < row_hi && col < Ncols) {
            if (coherent_out) {
              // the slice's 32 rows as one buffer range
              const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cp + (int64_t)frow * p.ldc, (uint32_t)(32 * p.ldc * OB));
              __builtin_amdgcn_raw_buffer_store_b128(val, rc, (rr * (int)p.ldc + col) * OB, 0, kCpolSc1);
            } else {
              *reinterpret_cast<u32x4*>(Cp + (int64_t)(frow + rr) * p.ldc + col) = val;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  };
  if constexpr (C::HAS_TAIL) {
    if (tail_tile) run(std::true_type{});
    else run(std::false_type{});
  } else {
    run(std::false_type{});
  }
}

template <class C, bool PINGPONG>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_kernel(GemmParams p, const float* bscale) {
  constexpr int BM = C::BM, BN = C::BN;
  // one LDS object per stage, so that the compiler can tell a stage being
  // filled by the asynchronous loads from the one being read. AP == 1: stage
  // i holds the activation tile at offset 0 and the weight tile at A_STAGE.
  // AP == 2: st0..st3 hold weight tiles only; sa0/sa1 hold activation tiles
  // for K-step pairs (0,1) and (2,3) of each group of four.
  MOE_GEMM_LDS(C)
  __shared__ int sched[5];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  // ---- tile schedule. A group's rows make full-height tiles of BM rows;
  // with tail tiles (HAS_TAIL), a remainder of at most BM/2 rows makes
  // tiles of TBM rows instead of one partial full-height tile. Phase 0 lists
  // the full-height tiles, phase 1 the tail tiles, each group by group and,
  // within a group, n-tiles in runs of kGroupN with row tiles fastest. Blocks
  // take phase 0 first (the hardware starts blocks in index order), so a
  // second round of tiles on the CUs is made of the cheap tail tiles. The
  // hardware hands blocks to the XCDs round-robin (block b -> XCD b % 8), so
  // within a phase block b takes tile (b % 8) * per + b / 8: each XCD works
  // through one contiguous stretch of the phase, and the ~32 blocks it runs
  // at a time share their weight slabs and activation rows in its own L2.
  if (wave == 0) {
    constexpr int GPL = 4;  // groups per lane (groups <= 256)
    int lo[GPL], hi[GPL], nf[GPL], nt[GPL];
    int sf = 0, st = 0;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int gi = lane * GPL + i;
      lo[i] = 0;
      hi[i] = 0;
      if (p.seg == nullptr) {
        if (gi == 0) hi[i] = p.M;
      } else if (gi < p.groups) {
        // rows are clamped to [0, M] so that no offset table can address
        // outside the row buffers
        lo[i] = min(max(p.seg[gi], 0), p.M);
        hi[i] = min(max(p.seg[gi + 1], lo[i]), p.M);
      }
      const int n = hi[i] - lo[i], t = n % BM;
      const bool small_tail = C::HAS_TAIL && t > 0 && t <= BM / 2;
      nf[i] = n / BM + (t > 0 && !small_tail);
      nt[i] = small_tail ? (t + C::TBM - 1) / C::TBM : 0;
      sf += nf[i];
      st += nt[i];
    }
    int incf = sf, inct = st;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int of = __shfl_up(incf, m, kWave), ot = __shfl_up(inct, m, kWave);
      if (lane >= m) {
        incf += of;
        inct += ot;
      }
    }
    const int NT = (p.Ncols + BN - 1) / BN;
    const int F = __shfl(incf, kWave - 1, kWave) * NT, Tt = __shfl(inct, kWave - 1, kWave) * NT;
    const int BF = (F + kNumXcds - 1) / kNumXcds * kNumXcds;  // blocks of phase 0
    const int phase = (int)blockIdx.x >= BF;
    const int b = blockIdx.x - (phase ? BF : 0);
    const int count = phase ? Tt : F;
    const int per = (count + kNumXcds - 1) / kNumXcds, local = b / kNumXcds;
    const int tile = (b % kNumXcds) * per + local;
    const bool live = local < per && tile < count;
    if (lane == 0 && !live) sched[0] = -1;
    const int q = tile / NT;  // row tile in the concatenated order of the phase
    int start = phase ? inct - st : incf - sf;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int c = phase ? nt[i] : nf[i];
      if (live && q >= start && q < start + c) {
        const int t = tile - start * NT;  // tile within the group's part of the phase
        const int run = c * kGroupN;      // tiles per run of kGroupN n-tiles
        const int ng = t / run, r = t % run;
        const int gn = min(kGroupN, NT - ng * kGroupN);
        const int qr = r / gn;
        const int r0 = phase ? lo[i] + (hi[i] - lo[i]) / BM * BM + qr * C::TBM : lo[i] + qr * BM;
        sched[0] = lane * GPL + i;
        sched[1] = r0;
        sched[2] = min(r0 + (phase ? C::TBM : BM), hi[i]);
        sched[3] = (ng * kGroupN + r % gn) * BN;
        sched[4] = phase;
      }
      start += c;
    }
  }
  __syncthreads();
  // block-uniform: keep them in scalar registers so that the buffer
  // descriptors built from them are uniform too
  const int g = __builtin_amdgcn_readfirstlane(sched[0]);
  if (g < 0) return;
  const int row_lo = __builtin_amdgcn_readfirstlane(sched[1]);
  const int row_hi = __builtin_amdgcn_readfirstlane(sched[2]);
  const int n0 = __builtin_amdgcn_readfirstlane(sched[3]);
  const bool tail_tile = __builtin_amdgcn_readfirstlane(sched[4]) != 0;
  gemm_tile<C, PINGPONG>(p, C::GELU, st0, st1, st2, st3, sa0, sa1, g, row_lo, row_hi, n0, tail_tile, bscale, [] {});
}

// ---- the expert FFN (GEMM1 + GELU, then GEMM2) as one persistent launch.
// Row tiles (each group's full-height tiles, then its tail tiles, as in
// grouped_gemm_kernel) are dealt to the XCDs in contiguous runs; each XCD's
// blocks take work items from that XCD's queue in the order: GEMM1 tiles of
// its full row tiles, of its tail row tiles, then GEMM2 tiles of the same.
// A GEMM2 tile needs all GEMM1 column tiles of its row tile (its K runs over
// all of H's columns): after storing its H tile, a GEMM1 block waits for its
// stores to complete and counts the tile in ready[row tile]; a GEMM2 block
// waits for that count. H is produced and consumed under one XCD's L2, so
// completed stores are what the consumer reads there. The consumer's own
// vector L1 is not coherent with other CUs' stores, but it cannot hold a
// stale line of the rows it reads: it loads H only in GEMM2 tiles, only
// after those rows are complete (and H is not rewritten in the launch), and
// the launch is taken only where an H row is a whole number of 256-byte
// lines (h a multiple of 128), so that no line holds rows of two row tiles;
// the L1 starts each launch empty. (An agent-scope acquire fence after the
// wait instead, which invalidates the L1, cost 5 % of the FFN on the noisy
// top-2 layer and 16 % on the cosine layer.) No block waits on a tile that
// no running block holds: a row tile's items are all in one XCD's queue, and
// each of its GEMM1 tiles is dequeued before any of its GEMM2 tiles, by a
// block that computes it without waiting. The wait is
// bounded all the same; if it ever expires, the GEMM2 tile is not computed
// from an incomplete H: its outputs are set to NaN and the launch's status
// word records the expiry (moe_ffn_status reads it). A block's XCD is read
// from the hardware, so the placement of blocks does not matter for
// correctness; every XCD gets blocks as the grid is a multiple of the XCD
// count.
struct FusedFfn {
  GemmParams g1, g2;  // GEMM1 (GELU) and GEMM2, as for two launches
  // [kNumXcds] queues, the status word (bit 0: a wait for H expired), then
  // ready[row tiles]: zero at launch
  int32_t* counters;
  FusedCombine comb;  // the folded combine (fused_ffn_kernel<C, true>)
#ifdef MOE_FFN_TRACE
  uint32_t trace_launch;  // launch number written into the trace records
#endif
};

// The combine of the tokens a GEMM2 tile completed (fin[0, nfin)), on the
// tile's columns [n0, n0 + 256): y[t, c] = the sum over kept j, in j order,
// of topk_w[t, j] * y_perm[row_of[t, j], c] in fp32 (one fma per term, the
// sequence combine_kernel uses), rounded once to bf16. Each wave takes every
// NW-th token, KB rows per token and 16 / KB tokens per batch with all their
// loads in flight; a lane covers 4 columns. y_perm rows may have been stored
// by blocks on other XCDs: they are read agent-coherently (sc1).
template <int KB, int NW>
__device__ void combine_finished(const int32_t* row_of, const float* topk_w, bf16* y, int k, const bf16* yp,
                                 int ldc, int Ncols, int n0, const int* fin, int nfin, int wave, int lane) {
  constexpr int U = 16 / KB;  // tokens per batch
  const int col = n0 + lane * 4;
  const bool live = col < Ncols;
  for (int f0 = wave; f0 < nfin; f0 += NW * U) {
    int rows[U][KB];
    float w[U][KB];
    u32x2 v[U][KB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int f = f0 + u * NW;
      const int t = f < nfin ? fin[f] : 0;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const bool has = f < nfin && j < k;
        rows[u][j] = has ? row_of[(int64_t)t * k + j] : -1;
        w[u][j] = has ? topk_w[(int64_t)t * k + j] : 0.f;
        v[u][j] = u32x2{0u, 0u};
        if (rows[u][j] >= 0 && live) {
          const uint64_t q = __hip_atomic_load(
              reinterpret_cast<const uint64_t*>(yp + (int64_t)rows[u][j] * ldc + col), __ATOMIC_RELAXED,
              __HIP_MEMORY_SCOPE_AGENT);
          v[u][j] = u32x2{(uint32_t)q, (uint32_t)(q >> 32)};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int f = f0 + u * NW;
      if (f >= nfin) break;  // wave-uniform
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        if (rows[u][j] < 0) continue;  // wave-uniform
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t wd = v[u][j][i >> 1];
          const float yv = __uint_as_float((i & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
          acc[i] = __builtin_fmaf(w[u][j], yv, acc[i]);
        }
      }
      if (live) Store<bf16>::four(y + (int64_t)fin[f] * Ncols + col, acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

constexpr uint32_t kHwRegXccId = (3u << 11) | 20u;  // s_getreg: XCC_ID[3:0]
constexpr int kFusedMaxGroups = 256;
constexpr int kFusedStatus = kNumXcds;      // index of the status word in the counters
constexpr int kFusedReady = kNumXcds + 1;   // index of ready[0]
// polls of a GEMM2 tile's wait (s_sleep 4 each, about 0.1 s in all)
constexpr int kFusedMaxPolls = 1 << 20;

// FOLD: GEMM2 tiles also do the gate-weighted combine (f.comb); see
// FusedCombine. PINGPONG: the tiles' K loops run the ping-pong schedule.
template <class C, bool FOLD, bool PINGPONG>
__global__ __launch_bounds__(C::THREADS) void fused_ffn_kernel(FusedFfn f) {
  constexpr int BM = C::BM, BN = C::BN, TBM = C::TBM;
  static_assert(C::HAS_TAIL, "tail row tiles follow the full ones");
  MOE_GEMM_LDS(C)
  // group table: first row, end row, and how many full / tail row tiles
  // come before the group's (exclusive prefixes)
  __shared__ int g_lo[kFusedMaxGroups], g_hi[kFusedMaxGroups], g_ef[kFusedMaxGroups], g_et[kFusedMaxGroups];
  __shared__ int tot[2];
  __shared__ int sched[9];
  __shared__ int fin[FOLD ? BM : 1];  // tokens a GEMM2 tile completed (FOLD)
  __shared__ int nfin;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int xcc = (int)(__builtin_amdgcn_s_getreg(kHwRegXccId) & (kNumXcds - 1));
  if (wave == 0) {
    const GemmParams& p1 = f.g1;
    const int groups = p1.groups;
    constexpr int GPL = kFusedMaxGroups / kWave;
    int lo[GPL], hi[GPL], nf[GPL], nt[GPL];
    int sf = 0, st = 0;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int gi = lane * GPL + i;
      lo[i] = hi[i] = 0;
      if (gi < groups) {
        lo[i] = min(max(p1.seg[gi], 0), p1.M);
        hi[i] = min(max(p1.seg[gi + 1], lo[i]), p1.M);
      }
      const int n = hi[i] - lo[i], t = n % BM;
      const bool small_tail = t > 0 && t <= BM / 2;
      nf[i] = n / BM + (t > 0 && !small_tail);
      nt[i] = small_tail ? (t + TBM - 1) / TBM : 0;
      sf += nf[i];
      st += nt[i];
    }
    int incf = sf, inct = st;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
      const int of = __shfl_up(incf, m, kWave), ot = __shfl_up(inct, m, kWave);
      if (lane >= m) {
        incf += of;
        inct += ot;
      }
    }
    int ef = incf - sf, et = inct - st;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int gi = lane * GPL + i;
      g_lo[gi] = lo[i];
      g_hi[gi] = hi[i];
      g_ef[gi] = ef;
      g_et[gi] = et;
      ef += nf[i];
      et += nt[i];
    }
    if (lane == kWave - 1) {
      tot[0] = incf;
      tot[1] = inct;
    }
  }
  // item indices: the first taken here, each next one while the current
  // tile's epilogue runs (its result is stored to sched[0] after it)
  if (tid == 0)
    sched[0] = __hip_atomic_fetch_add(f.counters + xcc, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#ifdef MOE_FFN_TRACE
  int tr_n = 0;
#endif
  for (;;) {
    // Everything below reads the arguments through fp, re-read for each
    // tile: the empty asm hides that fp never changes, so that the compiler
    // does not hold the arguments of both GEMMs in registers across the
    // tile's code (it would run out of them). fp points at the kernel
    // argument in the kernel-argument segment (f is the only argument);
    // taking f's address instead would make the compiler copy f to
    // private memory.
    const __attribute__((address_space(4))) FusedFfn* fp =
        (const __attribute__((address_space(4))) FusedFfn*)__builtin_amdgcn_kernarg_segment_ptr();
    __asm__ volatile("" : "+s"(fp));
    const int NT1 = (fp->g1.Ncols + BN - 1) / BN, NT2 = (fp->g2.Ncols + BN - 1) / BN;
    int32_t* const ready = fp->counters + kFusedReady;
    __syncthreads();  // sched[0]: this item's index
    if (wave == 0) {
      const int groups = fp->g1.groups;
      const int Fr = tot[0], Tr = tot[1];
      // this XCD's row tiles: full [fa, fb), tail [ta, tb) (tails dealt in
      // reverse, so that XCDs with fewer full tiles tend to get more tails)
      const int fa = xcc * Fr / kNumXcds, fb = (xcc + 1) * Fr / kNumXcds;
      const int ta = (kNumXcds - 1 - xcc) * Tr / kNumXcds, tb = (kNumXcds - xcc) * Tr / kNumXcds;
      const int nfx = fb - fa, ntx = tb - ta;
      int t = sched[0], kind = 0, tail = 0, NT = 0, c = 0, base = 0;
      if constexpr (PINGPONG) {
        // Long contractions: the XCD's tail items first (GEMM1's, then,
        // after kTailsAfter GEMM1 full items, GEMM2's), then the rest of its
        // GEMM1 full items and its GEMM2 full items. GEMM2 full tiles fill
        // whole rounds of the XCD's CUs; tail tiles taken after them would
        // leave most CUs idle while they finish.
        const int P = min(nfx * NT1, kTailsAfter);
        if (t < ntx * NT1) {
          kind = 1, tail = 1, NT = NT1, c = ntx, base = ta;
        } else if ((t -= ntx * NT1) < P) {
          kind = 1, NT = NT1, c = nfx, base = fa;
        } else if ((t -= P) < ntx * NT2) {
          kind = 2, tail = 1, NT = NT2, c = ntx, base = ta;
        } else if ((t -= ntx * NT2) < nfx * NT1 - P) {
          kind = 1, NT = NT1, c = nfx, base = fa, t += P;
        } else if ((t -= nfx * NT1 - P) < nfx * NT2) {
          kind = 2, NT = NT2, c = nfx, base = fa;
        }
      } else if (t < nfx * NT1) {
        // GEMM1 full items, GEMM1 tail items, GEMM2 full, GEMM2 tail
        kind = 1, NT = NT1, c = nfx, base = fa;
      } else if ((t -= nfx * NT1) < ntx * NT1) {
        kind = 1, tail = 1, NT = NT1, c = ntx, base = ta;
      } else if ((t -= ntx * NT1) < nfx * NT2) {
        kind = 2, NT = NT2, c = nfx, base = fa;
      } else if ((t -= nfx * NT2) < ntx * NT2) {
        kind = 2, tail = 1, NT = NT2, c = ntx, base = ta;
      }
      if (lane == 0) sched[1] = -1;  // done (or no tile found)
      if (kind != 0) {
        // runs of kGroupN column tiles, as in grouped_gemm_kernel
        const int run = c * kGroupN, ng = t / run, r = t % run;
        const int gn = min(kGroupN, NT - ng * kGroupN);
        const int q = base + r / gn, col = ng * kGroupN + r % gn;
#pragma unroll
        for (int i = 0; i < kFusedMaxGroups / kWave; ++i) {
          const int gi = lane * (kFusedMaxGroups / kWave) + i;
          if (gi < groups) {
            const int lo = g_lo[gi], hi = g_hi[gi], n = hi - lo, rem = n % BM;
            const bool small_tail = rem > 0 && rem <= BM / 2;
            const int e = tail ? g_et[gi] : g_ef[gi];
            const int cnt = tail ? (small_tail ? (rem + TBM - 1) / TBM : 0) : n / BM + (rem > 0 && !small_tail);
            if (q >= e && q < e + cnt) {
              const int r0 = tail ? lo + n / BM * BM + (q - e) * TBM : lo + (q - e) * BM;
              sched[1] = kind;
              sched[2] = gi;
              sched[3] = r0;
              sched[4] = min(r0 + (tail ? TBM : BM), hi);
              sched[5] = col * BN;
              sched[6] = tail;
              sched[7] = tail ? Fr + q : q;
            }
          }
        }
      }
    }
    __syncthreads();
    const int kind = __builtin_amdgcn_readfirstlane(sched[1]);
    if (kind < 0) {
      if constexpr (FOLD) {
        // leaving: zero rows of y for the tokens whose every choice was
        // dropped (no tile completes them), every NW-th token of the grid
        constexpr int NW = C::THREADS / kWave;
        const int d = fp->g2.Ncols, T = fp->comb.T, k = fp->comb.k;
        const int32_t* row_of = fp->comb.row_of;
        bf16* y = static_cast<bf16*>(fp->comb.y);
        for (int t = blockIdx.x * NW + wave; t < T; t += gridDim.x * NW) {
          bool any = false;
          for (int j = 0; j < k; ++j) any |= row_of[(int64_t)t * k + j] >= 0;
          if (any) continue;  // wave-uniform
          for (int q = lane; q < d / 8; q += kWave) store16(y + (int64_t)t * d + q * 8, u32x4{0u, 0u, 0u, 0u});
        }
      }
      break;
    }
    const int g = __builtin_amdgcn_readfirstlane(sched[2]);
    const int row_lo = __builtin_amdgcn_readfirstlane(sched[3]);
    const int row_hi = __builtin_amdgcn_readfirstlane(sched[4]);
    const int n0 = __builtin_amdgcn_readfirstlane(sched[5]);
    const bool tail_tile = __builtin_amdgcn_readfirstlane(sched[6]) != 0;
    const int rid = __builtin_amdgcn_readfirstlane(sched[7]);
#ifdef MOE_FFN_TRACE
    const uint64_t tr_t0 = __builtin_amdgcn_s_memrealtime(), tr_c0 = __builtin_readcyclecounter();
#endif
    int expired = 0;
    if (kind == 2) {
      if (tid == 0) {
        int spin = 0;
        for (; spin < kFusedMaxPolls; ++spin) {
          if (__hip_atomic_load(ready + rid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= NT1) break;
          __builtin_amdgcn_s_sleep(4);
        }
        sched[8] = spin == kFusedMaxPolls;
        if (spin == kFusedMaxPolls)
          __hip_atomic_fetch_or(fp->counters + kFusedStatus, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      expired = __builtin_amdgcn_readfirstlane(sched[8]);
    }
#ifdef MOE_FFN_TRACE
    const uint64_t tr_tw = __builtin_amdgcn_s_memrealtime();
#endif
    int next = 0;
    if (expired) {
      // H of these rows may be incomplete: the tile's outputs become NaN
      // (bf16 0x7FC0) instead of a silently wrong product
      const __attribute__((address_space(4))) GemmParams* pp = &fp->g2;
      const int cols = min(BN, pp->Ncols - n0), cpr = cols / 8, rows = row_hi - row_lo;
      bf16* out = static_cast<bf16*>(pp->C);
      for (int i = tid; i < rows * cpr; i += C::THREADS) {
        bf16* q = out + (int64_t)(row_lo + i / cpr) * pp->ldc + n0 + (i % cpr) * 8;
        if constexpr (FOLD) {
          // read by the folded combine, possibly on another XCD
          uint64_t* q8 = reinterpret_cast<uint64_t*>(q);
          __hip_atomic_store(q8, 0x7FC07FC07FC07FC0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(q8 + 1, 0x7FC07FC07FC07FC0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          store16(q, u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u});
        }
      }
      if (tid == 0) next = __hip_atomic_fetch_add(fp->counters + xcc, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // one copy of the tile code for both GEMMs
      const __attribute__((address_space(4))) GemmParams* pp = kind == 1 ? &fp->g1 : &fp->g2;
      gemm_tile<C, PINGPONG>(*(const GemmParams*)pp, kind == 1, st0, st1, st2, st3, sa0, sa1, g, row_lo, row_hi, n0,
                   tail_tile, nullptr, [&] {
                     if (tid == 0)
                       next = __hip_atomic_fetch_add(fp->counters + xcc, 1, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                   }, FOLD && kind == 2);
    }
    if (kind == 1) {
      wait_vmcnt<0>();  // this thread's H stores are in the L2
      __syncthreads();  // ... and every thread's
      if (tid == 0) __hip_atomic_fetch_add(ready + rid, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if constexpr (FOLD) {
      if (kind == 2) {
        // every thread's agent-coherent y_perm stores of the tile have
        // completed; then one arrival per row for its (token, column tile):
        // the arrival that makes a token's count reach its number of kept
        // choices completes that token's combine on these columns
        const int32_t* row_of = fp->comb.row_of;
        const int32_t* tor = fp->comb.token_of_row;
        int32_t* arrive = fp->comb.arrive;
        const int k = fp->comb.k;
        wait_vmcnt<0>();
        if (tid == 0) nfin = 0;
        __syncthreads();
        const int NT2 = (fp->g2.Ncols + BN - 1) / BN, ct = n0 / BN;
        for (int i = tid; i < row_hi - row_lo; i += C::THREADS) {
          const int t = tor[row_lo + i] / k;
          int kept = 0;
          for (int j = 0; j < k; ++j) kept += row_of[(int64_t)t * k + j] >= 0;
          const int before =
              __hip_atomic_fetch_add(arrive + (int64_t)t * NT2 + ct, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (before + 1 == kept) fin[atomicAdd(&nfin, 1)] = t;
        }
        __syncthreads();
        const int n = nfin;
        constexpr int NW = C::THREADS / kWave;
        const bf16* yp = static_cast<const bf16*>(fp->g2.C);
        const float* tw = fp->comb.topk_w;
        bf16* y = static_cast<bf16*>(fp->comb.y);
        const int ldc = (int)fp->g2.ldc, Nc = fp->g2.Ncols;
        if (k <= 2) combine_finished<2, NW>(row_of, tw, y, k, yp, ldc, Nc, n0, fin, n, wave, lane);
        else if (k <= 4) combine_finished<4, NW>(row_of, tw, y, k, yp, ldc, Nc, n0, fin, n, wave, lane);
        else combine_finished<8, NW>(row_of, tw, y, k, yp, ldc, Nc, n0, fin, n, wave, lane);
      }
    }
#ifdef MOE_FFN_TRACE
    if (tid == 0 && tr_n < kFfnTraceItems && (int)blockIdx.x < kFfnTraceBlocks) {
      uint64_t* r = g_ffn_trace + ((size_t)blockIdx.x * kFfnTraceItems + tr_n) * kFfnTraceWords;
      r[0] = tr_t0;
      r[1] = tr_tw;
      r[2] = __builtin_amdgcn_s_memrealtime();
      r[3] = tr_c0;
      r[4] = __builtin_readcyclecounter();
      r[5] = (uint64_t)xcc | ((uint64_t)kind << 4) | ((uint64_t)tail_tile << 8) | ((uint64_t)fp->trace_launch << 32);
      r[6] = (uint64_t)rid;
      r[7] = (uint64_t)n0;
    }
    ++tr_n;
#endif
    if (tid == 0) sched[0] = next;
  }
}

template <class C>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s, LaunchEvents ev, const float* bscale = nullptr) {
  // upper bounds on the row tiles of each phase: per group, the full-height
  // tiles plus at most one partial one, and at most BM/(2 TBM) tail tiles;
  // each phase's blocks are a multiple of the XCD count
  const int groups = p.seg ? p.groups : 1;
  const int64_t full_max = (int64_t)(p.M / C::BM + groups);
  const int64_t tail_max = C::HAS_TAIL ? (int64_t)groups * (C::BM / (2 * C::TBM)) : 0;
  const int ntiles = (p.Ncols + C::BN - 1) / C::BN;
  if (p.M <= 0 || ntiles <= 0) return hipSuccess;
  auto xcd_round = [](int64_t n) { return (n + kNumXcds - 1) / kNumXcds * kNumXcds; };
  const int64_t blocks = xcd_round(full_max * ntiles) + xcd_round(tail_max * ntiles);
  auto launch = [&](auto kernel) {
    if (ev.start || ev.stop)
      hipExtLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(C::THREADS), 0, s, ev.start, ev.stop, 0, p, bscale);
    else
      hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(C::THREADS), 0, s, p, bscale);
  };
  // 256 x 256 bf16 tiles run the single-launch FFN's ping-pong K loop (with
  // its 16x16x32 MFMAs) on long contractions, as that launch does
  constexpr bool kCanPingPong = C::BM == 256 && C::ES == 2 && !C::W8 && C::THREADS == 512;
  if constexpr (kCanPingPong) {
    if ((p.K + C::BK - 1) / C::BK >= kPingPongMinSteps) launch(grouped_gemm_kernel<C, true>);
    else launch(grouped_gemm_kernel<C, false>);
  } else {
    launch(grouped_gemm_kernel<C, false>);
  }
  return hipGetLastError();
}

constexpr int kNumCUs = 256;

// Tile shapes, judged from the rows a group can hold (the routing itself is
// only known on the device): avg_rows = T*k/N, max_rows = the capacity.
// 256 x 256 tiles (8 waves of 128 x 64) when groups can reach ~1536 rows,
// so that the partly filled last row tile of each group wastes little, and
// there are enough tiles to give every CU a block; otherwise 128 x 128
// (2 blocks per CU). Few rows per group on average (decode) take thin row
// tiles that stream the weights with deep prefetch.
// Cfg<elem, out, BM, BN, waves M x N, K chunks per stage, stages, GELU>.
template <typename E, typename O, bool G>
hipError_t launch_dtype(const GemmParams& p, int avg_rows, int max_rows, hipStream_t s, LaunchEvents ev) {
  if (avg_rows < 64) return launch_cfg<Cfg<E, O, 32, 256, 1, 4, 8, 4, G>>(p, s, ev);
  // 256x256 tiles (8 waves, one block per CU) need half the L1 bandwidth per
  // flop of 128x128 ones; with ragged tails in cheap tail tiles run last,
  // they are the faster choice on every FFN shape of the workloads once they
  // give at least half as many tiles as CUs
  const int groups = p.seg ? p.groups : 0;
  const int64_t tiles256 = (int64_t)(p.M / 256 + groups) * ((p.Ncols + 255) / 256);
  if (tiles256 >= kNumCUs / 2)
    return launch_cfg<Cfg<E, O, 256, 256, 2, 4, 4, 4, G>>(p, s, ev);
  // bf16, at most one 128x128 tile per CU (e.g. the cosine gate's
  // projection, a single group of T rows by 256 columns): eight waves of
  // 32 x 64, two per SIMD, so that one wave's waits are covered by the
  // other's MFMAs
  if constexpr (sizeof(E) == 2) {
    const int64_t tiles128 = (int64_t)(p.M / 128 + groups) * ((p.Ncols + 127) / 128);
    if (tiles128 <= kNumCUs) return launch_cfg<Cfg<E, O, 128, 128, 4, 2, 4, 4, G>>(p, s, ev);
  }
  return launch_cfg<Cfg<E, O, 128, 128, 2, 2, 4, 4, G>>(p, s, ev);
}

using FusedCfg = Cfg<bf16, bf16, 256, 256, 2, 4, 4, 4, false>;

// zeros n ints (graph-safe, unlike a memset node)
__global__ __launch_bounds__(256) void fill_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

namespace {
// *out = the fused launch's status word (0 where the layer has none)
__global__ void ffn_status_kernel(const int32_t* counters, int32_t* out) {
  if (threadIdx.x == 0) *out = counters ? counters[kFusedStatus] : 0;
}
}  // namespace

hipError_t launch_ffn_status(const int32_t* counters, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(ffn_status_kernel, dim3(1), dim3(64), 0, s, counters, out);
  return hipGetLastError();
}

int fused_ffn_counters(const GemmParams& g1) {
  const int64_t full_max = (int64_t)g1.M / FusedCfg::BM + g1.groups;
  const int64_t tail_max = (int64_t)g1.groups * (FusedCfg::BM / (2 * FusedCfg::TBM));
  return (int)(kFusedReady + full_max + tail_max);
}

bool fused_ffn_fits(const GemmParams& g1, const GemmParams& g2, bool bf16_, int avg_rows) {
  // the same tile configuration for both GEMMs as the two launches would take
  auto big = [](const GemmParams& p) {
    return (int64_t)(p.M / 256 + p.groups) * ((p.Ncols + 255) / 256) >= kNumCUs / 2;
  };
  // H rows of whole 256-byte lines: no line of H holds rows of two row tiles
  const bool whole_lines = g1.Ncols % 128 == 0;
  return bf16_ && g1.seg && g2.seg && avg_rows >= 64 && g1.groups <= kFusedMaxGroups && big(g1) && big(g2) &&
         g1.M > 0 && whole_lines;
}

int fused_combine_col_tiles(int d) { return (d + FusedCfg::BN - 1) / FusedCfg::BN; }

#ifdef MOE_FFN_TRACE
size_t ffn_trace_bytes() { return sizeof(g_ffn_trace); }
hipError_t ffn_trace_copy(void* host) { return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_ffn_trace), sizeof(g_ffn_trace)); }
#else
size_t ffn_trace_bytes() { return 0; }
hipError_t ffn_trace_copy(void*) { return hipErrorNotSupported; }
#endif

hipError_t launch_fused_ffn(const GemmParams& g1, const GemmParams& g2, int32_t* counters, bool clear,
                            hipStream_t s, LaunchEvents ev, const FusedCombine* comb) {
  if (clear) {
    const int n = fused_ffn_counters(g1);
    hipLaunchKernelGGL(fill_kernel, dim3((n + 255) / 256), dim3(256), 0, s, counters, n);
  }
  if (comb && comb->k > kFusedCombineMaxK) return hipErrorInvalidValue;
  FusedFfn f{g1, g2, counters, comb ? *comb : FusedCombine{}};
#ifdef MOE_FFN_TRACE
  static uint32_t launches = 0;
  f.trace_launch = ++launches;
#endif
  // one block per CU (a multiple of the XCD count)
  auto launch = [&](auto kernel) {
    if (ev.start || ev.stop)
      hipExtLaunchKernelGGL(kernel, dim3(kNumCUs), dim3(FusedCfg::THREADS), 0, s, ev.start, ev.stop, 0, f);
    else
      hipLaunchKernelGGL(kernel, dim3(kNumCUs), dim3(FusedCfg::THREADS), 0, s, f);
  };
  const bool pp = (g1.K + FusedCfg::BK - 1) / FusedCfg::BK >= kPingPongMinSteps &&
                  (g2.K + FusedCfg::BK - 1) / FusedCfg::BK >= kPingPongMinSteps;
  if (comb) {
    if (pp) launch(fused_ffn_kernel<FusedCfg, true, true>);
    else launch(fused_ffn_kernel<FusedCfg, true, false>);
  } else {
    if (pp) launch(fused_ffn_kernel<FusedCfg, false, true>);
    else launch(fused_ffn_kernel<FusedCfg, false, false>);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm_dual(const GemmParams& p, int avg_rows, hipStream_t s) {
  // the tile choice of launch_dtype<bf16, bf16, GELU>
  if (avg_rows < 64) return launch_cfg<Cfg<bf16, bf16, 32, 256, 1, 4, 8, 4, true, false, true>>(p, s, {});
  const int groups = p.seg ? p.groups : 0;
  const int64_t tiles256 = (int64_t)(p.M / 256 + groups) * ((p.Ncols + 255) / 256);
  if (tiles256 >= kNumCUs / 2) return launch_cfg<Cfg<bf16, bf16, 256, 256, 2, 4, 4, 4, true, false, true>>(p, s, {});
  const int64_t tiles128 = (int64_t)(p.M / 128 + groups) * ((p.Ncols + 127) / 128);
  if (tiles128 <= kNumCUs) return launch_cfg<Cfg<bf16, bf16, 128, 128, 4, 2, 4, 4, true, false, true>>(p, s, {});
  return launch_cfg<Cfg<bf16, bf16, 128, 128, 2, 2, 4, 4, true, false, true>>(p, s, {});
}

hipError_t launch_grouped_gemm_w8(const GemmParams& p, GemmW8 w8, GemmKind kind, int avg_rows, hipStream_t s,
                                  LaunchEvents ev) {
  // Few rows per group (decoding): the decode tile (32 rows, 4 waves of 64
  // columns, 64-deep K-steps, 4 stages), the layer's bytes being the
  // weights, streamed once per 32 rows. Otherwise 128 x 128 tiles (4 waves
  // of 64 x 64, paired activation stages, tail tiles): the per-block scale
  // needs a second accumulator set, which the 256 x 256 tile's registers
  // cannot hold.
  const bool gelu = kind == GemmKind::kFfn1Gelu;
  if (p.K % 128 || p.K > kW8MaxK || p.Ncols % 128) return hipErrorInvalidValue;
  if (avg_rows < 64)
    return gelu ? launch_cfg<Cfg<bf16, bf16, 32, 256, 1, 4, 8, 4, true, true>>(p, s, ev, w8.bscale)
                : launch_cfg<Cfg<bf16, bf16, 32, 256, 1, 4, 8, 4, false, true>>(p, s, ev, w8.bscale);
  return gelu ? launch_cfg<Cfg<bf16, bf16, 128, 128, 2, 2, 4, 4, true, true>>(p, s, ev, w8.bscale)
              : launch_cfg<Cfg<bf16, bf16, 128, 128, 2, 2, 4, 4, false, true>>(p, s, ev, w8.bscale);
}

hipError_t launch_grouped_gemm(const GemmParams& p, GemmKind kind, bool bf16_, int avg_rows,
                               int max_rows, hipStream_t s, LaunchEvents ev) {
  switch (kind) {
    case GemmKind::kFfn1Gelu:
      return bf16_ ? launch_dtype<bf16, bf16, true>(p, avg_rows, max_rows, s, ev)
                   : launch_dtype<float, float, true>(p, avg_rows, max_rows, s, ev);
    case GemmKind::kFfn2:
      return bf16_ ? launch_dtype<bf16, bf16, false>(p, avg_rows, max_rows, s, ev)
                   : launch_dtype<float, float, false>(p, avg_rows, max_rows, s, ev);
    case GemmKind::kProjF32:
      return bf16_ ? launch_dtype<bf16, float, false>(p, avg_rows, max_rows, s, ev)
                   : launch_dtype<float, float, false>(p, avg_rows, max_rows, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
