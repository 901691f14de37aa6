// Host-side launchers of the MoE kernels (internal to the library).
// Every launcher enqueues on `stream` and returns the launch status; shapes
// have been validated by the C ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- gate (gate.hip)
struct GateParams {
  const void* x;           // [T, d] X-dtype
  const void* w_gate;      // [d, N]
  const void* w_noise;     // [d, N] or null
  const float* noise;      // [T, N] or null
  const float* logit_bias; // [N] or null
  float* logits;           // [T, N] (required when N exceeds one column block)
  int32_t* topk_idx;       // [T, k]
  float* topk_w;           // [T, k]
  float* partial;          // bf16 only: gate_partial_bytes() of scratch for the split product
  // [ceil(T/32), N] or null: the choices of each 32 tokens per expert
  // (written where gate_writes_hist(): the bf16 single-kernel gate)
  int32_t* hist;
  int T, d, N, k, renorm;
};
bool gate_writes_hist(bool bf16, bool noisy, int N);
constexpr int kGateHistTokens = 32;
hipError_t launch_gate_plain_noisy(const GateParams& p, bool bf16, bool noisy, hipStream_t s);

// How the bf16 plain/noisy gate product x [W_g | W_n] is split: column
// chunks of 32, K slices, and K per slice (a multiple of 64).
struct GateSplit {
  int ncc, ks, kr;
};
GateSplit gate_split(int64_t T, int d, int N, bool noisy);
size_t gate_partial_bytes(int64_t T, int d, int N, bool noisy);

struct CosineParams {
  const float* z;          // [T, p] fp32 projection x P
  const float* emb;        // [N, p] fp32
  const float* logit_bias; // [N] or null
  float inv_temperature;
  float* logits;           // [T, N] or null
  int32_t* topk_idx;
  float* topk_w;
  int T, p, N, k, renorm;
};
hipError_t launch_cosine_select(const CosineParams& p, hipStream_t s);

// ---- dispatch (dispatch.hip)
constexpr int kDispatchTile = 256;  // tokens per dispatch tile (one per thread of a block)
struct DispatchParams {
  const void* x;            // [T, d]
  const int32_t* topk_idx;  // [T, k]
  int32_t* tile_counts;     // [nTiles, N] workspace
  int32_t* expert_count;    // [N]
  int32_t* expert_off;      // [N+1]
  int32_t* row_of;          // [T*k]
  int32_t* token_of_row;    // [R]
  void* x_perm;             // [R, d] or null (skip the copy)
  int32_t* zero;            // zero_n ints to clear on the way (or null)
  int32_t* zero_tok;        // zero_tok_n ints per token to clear on the way (or null)
  int zero_tok_n;
  // the gate's per-32-token choice counts (GateParams::hist), or null: then
  // the dispatch counts them itself
  const int32_t* hist32;
  // [nTiles, N] and [N] workspace for the scan of a large count table
  // (used where dispatch_scans())
  int32_t* tile_start;
  int32_t* totals;
  int T, d, N, k, C, elem_bytes, zero_n;
  // 1: the routing comes from the caller, and a choice that repeats an
  // earlier choice of the same token is dropped like an out-of-range one
  int caller_routing;
};
// Count tables of more entries than this are scanned by their own kernel
// (one block per expert) instead of by every rows block.
constexpr int64_t kDispatchDirectMax = 8192;
bool dispatch_scans(int64_t T, int N, bool hist32);
hipError_t launch_dispatch(const DispatchParams& p, hipStream_t s);
hipError_t launch_permute(const DispatchParams& p, hipStream_t s);

// ---- grouped GEMM (gemm.hip)
// C[r, :] = epilogue(A[r, :] B_g + bias_g) for the rows r of group g.
struct GemmParams {
  const void* A;        // rows of length K, stride lda elements
  const void* B;        // per group [K, Ncols] row-major, group stride strideB elements
  const void* bias;     // per group [Ncols] (stride strideBias) or null
  void* C;              // rows of length Ncols, stride ldc elements
  const int32_t* seg;   // [groups+1] row offsets of each group (device); null = one group of M rows
  // Gathered A rows: output row r reads A row gather[r] / gather_div, A holding
  // a_rows rows (a_rows * lda * element bytes < 2^31). Null: output row r reads A row r.
  const int32_t* gather;
  int gather_div, a_rows;
  int64_t lda, ldc, strideB, strideBias;
  int M;                // rows when seg is null; else the row bound R
  int groups, K, Ncols;
  void* C2;             // launch_grouped_gemm_dual: the pre-activation rows (as C), else unused
};
enum class GemmKind { kFfn1Gelu, kFfn2, kProjF32 };
// Block-FP8 weights (launch_grouped_gemm_w8): B holds E4M3 codes in K-groups
// of 8 (the byte of B[k][n] at (k/8 * Ncols + n) * 8 + k % 8, strideB bytes
// per group) and bscale one fp32 scale per 128 x 128 block,
// [groups, K/128, Ncols/128]; K a multiple of 128, at most kW8MaxK.
constexpr int kW8MaxK = 16384;
struct GemmW8 {
  const float* bscale;
};
// Events a launch records when its kernel starts and when it ends executing
// (hipExtLaunchKernel), each or both null for none.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
// bf16 activations times block-FP8 weights (GELU for kFfn1Gelu); K and
// Ncols multiples of 128. avg_rows: expected rows per group (tile choice:
// 32-row tiles that stream the weights below 64, else 256 x 256).
hipError_t launch_grouped_gemm_w8(const GemmParams& p, GemmW8 w8, GemmKind kind, int avg_rows, hipStream_t s,
                                  LaunchEvents ev = {});
// bf16 GEMM1 of the FFN storing both the pre-activation U = A B + bias (C2)
// and H = GELU(U) (C), with the tiles, K order and GELU of the forward's
// GEMM1 (the backward's recompute of U and H)
hipError_t launch_grouped_gemm_dual(const GemmParams& p, int avg_rows, hipStream_t s);
// E4M3 block quantisation (quant.hip): W [groups, K, Ncols] fp32 or bf16,
// K and Ncols multiples of 128
hipError_t launch_quantize_fp8(const void* W, bool bf16, int groups, int K, int Ncols, uint8_t* codes,
                               float* scales, hipStream_t s);
// avg_rows / max_rows: expected and largest rows per group (tile choice only)
hipError_t launch_grouped_gemm(const GemmParams& p, GemmKind kind, bool bf16, int avg_rows,
                               int max_rows, hipStream_t s, LaunchEvents ev = {});
// The expert FFN (GEMM1 kFfn1Gelu, then GEMM2 kFfn2 on GEMM1's output) in one
// persistent launch, where fused_ffn_fits(); counters: fused_ffn_counters()
// ints, zero at launch (they are consumed): cleared first by a small kernel
// if clear, else by the caller earlier on the stream.
bool fused_ffn_fits(const GemmParams& g1, const GemmParams& g2, bool bf16, int avg_rows);
int fused_ffn_counters(const GemmParams& g1);
// The gate-weighted combine folded into the single-launch FFN: each GEMM2
// tile stores its y_perm rows agent-coherently and counts them per (token,
// column tile); the tile that brings a token's last kept row sums that
// token's kept rows of the column tile in j order, exactly as
// launch_combine does, into y. Blocks leaving the launch write zero rows
// for tokens with every choice dropped. k <= kFusedCombineMaxK.
struct FusedCombine {
  const int32_t* row_of;        // [T*k]
  const int32_t* token_of_row;  // [R]
  const float* topk_w;          // [T, k]
  void* y;                      // [T, d] bf16
  int32_t* arrive;              // [T * fused_combine_col_tiles(d)], zero at launch
  int T, k;
};
constexpr int kFusedCombineMaxK = 8;
int fused_combine_col_tiles(int d);
hipError_t launch_fused_ffn(const GemmParams& g1, const GemmParams& g2, int32_t* counters, bool clear,
                            hipStream_t s, LaunchEvents ev = {}, const FusedCombine* comb = nullptr);
// *out = the status word of the fused launch that last used `counters`
// (bit 0: a GEMM2 tile's wait for its rows of H expired and its outputs were
// set to NaN); counters null: *out = 0
hipError_t launch_ffn_status(const int32_t* counters, int32_t* out, hipStream_t s);
// Per-item trace of the single-launch FFN (measurement build, MOE_FFN_TRACE):
// block b's i-th item (i < kFfnTraceItems) writes record b * kFfnTraceItems + i
// of kFfnTraceWords uint64: wall clock (100 MHz) at the item's start, after
// its wait for H and at its end; shader cycle counter at its start and end;
// XCD | kind << 4 | tail << 8 | launch number << 32; row tile; first column.
// ffn_trace_bytes() is 0 and ffn_trace_copy() fails in other builds.
constexpr int kFfnTraceItems = 64, kFfnTraceWords = 8, kFfnTraceBlocks = 256;
size_t ffn_trace_bytes();
hipError_t ffn_trace_copy(void* host);

// ---- backward pass (backward.hip), bf16 layers
typedef __bf16 bf16;
constexpr int kMaxExperts = 256;
enum class BwdLayout { kKContig, kKStrided };  // an operand's rows hold K (contiguous) or M / N (K strided)
enum class BwdEpi { kPlain, kGeluGrad };
enum class BwdGemmKind {
  kGeluGrad,    // G = dy_perm W2^T: A gathered dy rows, B = W2_e rows [h][d]; C = dU = bf16(w G GELU'(U)),
                // pd = per-row dots G . H over each 128-column tile
  kDataGrad,    // dx_perm = dU W1_e^T: A = dU rows (K = h), B = W1_e rows [d][h]; C fp32
  kWeightGrad,  // per group e: C_e [M, N] = A_e^T B_e over the group's rows; A [rows][M], B [rows][N]; C fp32
};
struct BwdGemmParams {
  const void* A;         // bf16
  const void* B;         // bf16, group g at B + g * strideB elements
  void* C;               // output (group g at C + g * strideC elements for kWeightGrad)
  int64_t lda, ldb, ldc, strideB, strideC;
  int64_t a_bytes, b_bytes;  // byte ranges of A and of one group of B (< 2^31)
  const int32_t* seg;    // [groups + 1]: output rows (ragged M) or contraction rows (kWeightGrad)
  const int32_t* gather; // A row of output row m: gather[m] / gather_div (or null: row m)
  int gather_div;
  int a_rows;            // kWeightGrad: rows of A and B (bound of seg)
  int M, N, K, groups;   // ragged M: M = row bound; kWeightGrad: each group's C is M x N
  const void* U;         // kGeluGrad: [rows, N] bf16
  const void* H;         // kGeluGrad: [rows, N] bf16
  const float* row_w;    // kGeluGrad: gate weight of choice t*k+j
  const int32_t* tor;    // kGeluGrad: choice t*k+j of each row
  float* pd;             // kGeluGrad: [rows, ceil(N / 128)]
};
hipError_t launch_bwd_gemm(const BwdGemmParams& p, BwdGemmKind kind, hipStream_t s);
hipError_t launch_scale_rows(const bf16* dy, const int32_t* row_of, const float* w, bf16* out, int T, int d, int k,
                             hipStream_t s);
hipError_t launch_importance_grad(const float* imp, float* dimp, int N, float c0, float c1, hipStream_t s);
struct BwdTokenParams {
  const float* pd;        // [R, ntc] partial dots G . H
  int ntc;
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* row_of;
  const float* logits;    // [T, N] (renorm = 0)
  const float* dimp;      // [N] or null (no auxiliary losses)
  const bf16* dy;         // [T, d]
  const bf16* b2;         // [N, d] or null
  const bf16* x;          // [T, d]
  const bf16* w_gate;     // [d, N]
  const bf16* w_noise;    // [d, N] or null (plain gate)
  const float* noise;     // [T, N]
  const float* dx_perm;   // [R, d]
  float* dl;              // [T, N] out
  float* dz;              // [T, N] out (noisy)
  bf16* dx;               // [T, d] out
  int T, d, N, k, renorm;
};
hipError_t launch_bwd_token(const BwdTokenParams& p, hipStream_t s);
int gate_grad_chunks(int64_t T);
// out0 [d, N] = x^T src0 and (src1 non-null) out1 [d, N] = x^T src1, src
// [T, N] fp32, through partial [gate_grad_chunks(T), d, N'] (N' = 2N with
// src1, else N)
hipError_t launch_gate_grad(const bf16* x, const float* src0, const float* src1, float* partial, float* out0,
                            float* out1, int T, int d, int N, hipStream_t s);
// out [N] = column sums of src [T, N], through partial [gate_grad_chunks(T), N]
hipError_t launch_column_sum(const float* src, float* partial, float* out, int T, int N, hipStream_t s);
// out [groups, cols] = per group the sums of its rows [off[g], off[g+1]) of src [rows, cols]
hipError_t launch_colsum_bf16(const bf16* src, const int32_t* off, float* out, int cols, int groups, int rows_bound,
                              hipStream_t s);

// ---- measurement aids (probe.hip)
// copies bytes / 16 16-byte chunks from src to dst
hipError_t launch_probe_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);
// iters rounds of MFMAs on registers; sink: probe_mfma_blocks() * 8 floats
hipError_t launch_probe_mfma(int iters, float* sink, hipStream_t s);
int probe_mfma_blocks();
int64_t probe_mfma_flops_per_iter();

// ---- load-balance terms (aux.hip)
constexpr int kAuxTok = 256;  // tokens per partial-sum block
struct AuxParams {
  const int32_t* topk_idx;  // [T, k]
  const float* topk_w;      // [T, k]
  float* partial;           // [aux_blocks(T), N] workspace
  float* importance;        // [N] or null
  float* losses;            // [2] or null
  int T, N, k;
};
int aux_blocks(int64_t T);
hipError_t launch_aux_loss(const AuxParams& p, hipStream_t s);

// ---- combine (combine.hip)
struct CombineParams {
  const void* y_perm;      // [R, d]
  const int32_t* row_of;   // [T*k]
  const float* topk_w;     // [T, k]
  void* y;                 // [T, d]
  int T, d, k;
  int R;                   // rows of y_perm; row_of entries >= R count as dropped
};
hipError_t launch_combine(const CombineParams& p, bool bf16, hipStream_t s);

}  // namespace moe
