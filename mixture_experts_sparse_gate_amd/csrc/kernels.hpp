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
  // the gate's per-32-token choice counts (GateParams::hist), or null: then
  // the dispatch counts them itself
  const int32_t* hist32;
  int T, d, N, k, C, elem_bytes, zero_n;
};
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
};
enum class GemmKind { kFfn1Gelu, kFfn2, kProjF32 };
// Block-FP8 weights (launch_grouped_gemm_w8): B holds E4M3 codes in K-groups
// of 8 (the byte of B[k][n] at (k/8 * Ncols + n) * 8 + k % 8, strideB bytes
// per group) and bscale one fp32 scale per 128 x 128 block,
// [groups, K/128, Ncols/128]; K a multiple of 128.
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
hipError_t launch_fused_ffn(const GemmParams& g1, const GemmParams& g2, int32_t* counters, bool clear,
                            hipStream_t s, LaunchEvents ev = {});

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
