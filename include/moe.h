/*
 * moe.h — C ABI of the sparse-gated Mixture-of-Experts layer forward pass
 * on one MI355X (gfx950).
 *
 * The layer maps tokens x[T, d] to y[T, d]:
 *
 *   1. gate      logits[T, N] from x (plain, noisy or cosine), softmax,
 *                top-k experts per token and their weights g_i(x)
 *   2. dispatch  capacity-limited slots in token order; the kept (token,
 *                expert) pairs are copied into expert-contiguous rows
 *   3. experts   per expert e, on its rows: GELU(x W1[e] + b1[e]) W2[e] + b2[e]
 *   4. combine   y[t] = sum over the kept choices j of g_j(x_t) E_j(x_t)
 *
 * The layer's definition is the weighted sum of expert outputs on the page
 * "MoE架构：突破单卡算力瓶颈的密钥" (§1.2); the gate follows the noisy top-k
 * gating code on "MoE稀疏计算加速技术解析与应用实践" (§2.1) and
 * "MoE架构：稀疏激活机制如何提升模型计算效率" (§2.1); grouping tokens by expert
 * before one batched matmul per group follows the latter page's §3.1; the
 * expert is the Linear-GELU-Linear block of the CANN page's §3.2; the
 * capacity factor appears there and on the Tutel guide
 * ("4大技术模块掌握Tutel MoE…", dynamic routing section).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers to row-major, contiguous arrays,
 *    16-byte aligned. "X-dtype" arrays (x, w_gate, w_noise, proj, W1, b1, W2,
 *    b2, x_perm, H, y_perm, y) hold desc->dtype elements (fp32 or bf16);
 *    noise, expert_emb, logit_bias, logits and topk_w are always fp32; index
 *    arrays are int32.
 *  - The caller owns every buffer, including the workspace. The library
 *    never allocates, frees or synchronises (the one exception is the debug
 *    build's check of caller routing in moe_dispatch), and keeps no pointer
 *    after a call returns.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the default
 *    stream) and runs asynchronously; the call does not wait for it.
 *  - All arguments are checked on the host before anything is enqueued; on
 *    any error nothing is enqueued, the status says which class of error it
 *    was and moe_last_error() gives a message (per thread).
 *  - Results are deterministic: no floating-point atomics anywhere, and a
 *    fixed summation order in every reduction.
 *  - Sizes: 1 <= N <= 256, 1 <= k <= min(N, 32), T*k < 2^31, d and h
 *    multiples of 8 (bf16) or 4 (fp32), cosine proj_dim a multiple of 8 and
 *    at most 256. Outside those: MOE_ERR_INVALID. With s the element bytes,
 *    T*max(d,h)*s, d*h*s and d*N*s (cosine: d*proj_dim*s) must each stay
 *    below 2^31 bytes (the kernels' 32-bit buffer ranges); larger layers
 *    get MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* bad argument: null/misaligned pointer, size out of range */
  MOE_ERR_UNSUPPORTED = 2, /* valid request the library does not implement */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes below moe_workspace_size() */
  MOE_ERR_HIP = 4          /* a HIP launch failed; moe_last_error() has the HIP message */
} moe_status_t;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum moe_gate {
  /* logits = x w_gate (+ logit_bias) */
  MOE_GATE_SOFTMAX = 0,
  /* logits = x w_gate + noise * softplus(x w_noise) (+ logit_bias),
     softplus(z) = max(z, 0) + log1p(exp(-|z|)); noise is the caller's
     standard-normal [T, N] tensor (the pages draw it inside the gate) */
  MOE_GATE_NOISY = 1,
  /* z = x proj; logits_j = cos(z, expert_emb_j) * inv_temperature (+ logit_bias_j),
     both norms clamped below at 1e-12 */
  MOE_GATE_COSINE = 2
} moe_gate_t;

typedef struct moe_desc {
  int64_t T;              /* tokens */
  int32_t d;              /* model dim */
  int32_t h;              /* expert hidden dim */
  int32_t N;              /* experts */
  int32_t k;              /* experts per token */
  double capacity_factor; /* > 0; capacity C = min(T, ceil((cf * (T*k)) / N)) in IEEE double */
  int32_t gate;           /* moe_gate_t */
  int32_t renorm;         /* 1: weights = softmax over the k selected logits;
                             0: weights = full softmax probability of each selected expert */
  int32_t dtype;          /* moe_dtype_t of the X-dtype arrays */
  int32_t proj_dim;       /* cosine gate: p (columns of proj); else 0 */
  float inv_temperature;  /* cosine gate: 1/tau; else ignored */
  int32_t flags;          /* MOE_FLAG_* bits; 0 for the default path */
} moe_desc_t;

/* moe_forward (and moe_forward_noalloc): fold the gate-weighted combine into
 * the single-launch expert FFN. Each GEMM2 tile stores its rows of y_perm
 * agent-coherently and counts them per (token, 256-column tile); the tile
 * that brings a token's last kept row writes that token's y on those
 * columns, summing the kept rows in j order with the sequence moe_combine
 * uses, so y is bit-identical to the default path. (The fusion is the
 * operator fusion and memory reuse of "MoE架构：突破单卡算力瓶颈的密钥" §3.3.)
 * It applies where the single-launch FFN runs (bf16, at least 64 rows per
 * expert on average, h a multiple of 128, enough tiles, the whole chip) and
 * k <= 8; elsewhere the flag changes nothing. The workspace then also holds
 * T * ceil(d / 256) int32 arrival counts. On the measured layers it is
 * slower than the separate combine, so it is off by default. Other entry
 * points ignore it. */
#define MOE_FLAG_COMBINE_IN_FFN 1

/* Which entry point a workspace is sized for. */
typedef enum moe_ws_kind {
  MOE_WS_ROUTE = 0,
  MOE_WS_DISPATCH = 1,
  MOE_WS_FORWARD = 2,
  MOE_WS_FFN = 3,
  MOE_WS_AUX = 4,
  MOE_WS_BACKWARD = 5
} moe_ws_kind_t;

/* Expert capacity C = min(T, ceil((capacity_factor * (T*k)) / N)), evaluated
 * in IEEE double; -1 if desc is invalid. Host only. */
MOE_API int64_t moe_capacity(const moe_desc_t* desc);

/* Row bound R = min(T*k, N*C) of the expert-grouped buffers x_perm, H,
 * y_perm and token_of_row; -1 if desc is invalid. Host only. */
MOE_API int64_t moe_rows_bound(const moe_desc_t* desc);

/* Bytes of device workspace `kind` needs (a multiple of 256). Host only. */
MOE_API moe_status_t moe_workspace_size(const moe_desc_t* desc, moe_ws_kind_t kind, size_t* bytes);

/* Gate: logits, top-k selection and weights. The noisy logits and the
 * top-k with a softmax over the selected logits follow the noisy top-k
 * gating code of "MoE稀疏计算加速技术解析与应用实践" §2.1 (and of
 * "MoE架构：稀疏激活机制如何提升模型计算效率" §2.1); the full-softmax weight of
 * each selected expert (renorm = 0) is the top-1 MOELayer example of
 * "PyTorch-CUDA-v2.6镜像是否支持MoE稀疏激活架构" (section "PyTorch v2.6：为动态
 * 计算而生"); the cosine gate is the cosine_top router named on
 * "4大技术模块掌握Tutel MoE…" (dynamic routing section).
 *   x [T, d] X-dtype; w_gate [d, N] (SOFTMAX, NOISY); w_noise [d, N] and
 *   noise [T, N] fp32 (NOISY); proj [d, p] X-dtype and expert_emb [N, p] fp32
 *   (COSINE); logit_bias [N] fp32 or NULL (any gate).
 * Outputs: logits [T, N] fp32 (the final gate logits, after noise and bias)
 *   or NULL; topk_idx [T, k] int32, experts ordered by logit descending, equal
 *   logits by ascending expert index (-0.0 equals +0.0); topk_w [T, k] fp32.
 * Selection compares the fp32 logits; weights are computed in fp32 from them.
 * ws: MOE_WS_ROUTE bytes (may be NULL when that size is 0). */
MOE_API moe_status_t moe_route(const moe_desc_t* desc, const void* x, const void* w_gate,
                       const void* w_noise, const float* noise, const void* proj,
                       const float* expert_emb, const float* logit_bias, float* logits,
                       int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                       void* stream);

/* Capacity-limited dispatch in token order: tokens grouped by their chosen
 * expert before one batched matmul per group ("MoE架构：稀疏激活机制如何提升
 * 模型计算效率" §3.1), each expert holding at most C = capacity_factor * T*k/N
 * of them (capacity_factor on "MoE稀疏计算加速技术解析与应用实践" §3.2 and the
 * Tutel guide's dynamic routing section).
 *   topk_idx [T, k] int32: each token's experts, which must be distinct and
 *   in [0, N). In a release build an entry outside [0, N), or one that
 *   repeats an earlier expert of the same token, is treated as dropped
 *   (row -1) and counts for no expert. The debug build
 *   (libmoe_gfx950_debug.so, compiled with MOE_DEBUG_CHECKS) copies topk_idx
 *   to the host, synchronising the stream, and returns MOE_ERR_INVALID with
 *   a message naming the first offending (t, j) instead.
 * Outputs: expert_count [N] (demand: choices per expert before the capacity
 *   limit); expert_off [N+1] (exclusive scan of kept = min(count, C);
 *   expert_off[N] = A, the number of kept choices); row_of [T*k] (row of
 *   choice (t, j) in the grouped buffers, or -1 if dropped: the choice is
 *   kept iff fewer than C earlier tokens chose the same expert);
 *   token_of_row [R] (t*k + j of each row < A; rows >= A untouched);
 *   x_perm [R, d] X-dtype (x_perm[row_of[t*k+j]] = x[t] bitwise).
 * ws: MOE_WS_DISPATCH bytes. */
MOE_API moe_status_t moe_dispatch(const moe_desc_t* desc, const void* x, const int32_t* topk_idx,
                          int32_t* expert_count, int32_t* expert_off, int32_t* row_of,
                          int32_t* token_of_row, void* x_perm, void* ws, size_t ws_bytes,
                          void* stream);

/* Grouped expert FFN on the expert-contiguous rows: one batched matmul per
 * group of tokens ("MoE架构：稀疏激活机制如何提升模型计算效率" §3.1), the expert
 * being the Linear-GELU-Linear block of "MoE稀疏计算加速技术解析与应用实践"
 * §3.2.
 *   x_perm [R, d]; expert_off [N+1] (device); W1 [N, d, h]; b1 [N, h] or NULL;
 *   W2 [N, h, d]; b2 [N, d] or NULL. All X-dtype except expert_off.
 * For e < N and off[e] <= r < off[e+1]:
 *   H[r]      = GELU(x_perm[r] W1[e] + b1[e])       fp32 accumulation, rounded once to X-dtype
 *   y_perm[r] = H[r] W2[e] + b2[e]                   fp32 accumulation, rounded once
 * with GELU(u) = u/2 (1 + erf(u / sqrt 2)). H [R, h] and y_perm [R, d] are
 * outputs; rows >= expert_off[N] are not written. The grid is sized from R,
 * so no host read of expert_off is needed.
 * ws: MOE_WS_FFN bytes, or NULL. It holds the work counters of the
 * single-launch form of the two GEMMs (bf16 layers with enough rows and
 * columns for 256x256 tiles), in which GEMM2's tiles wait for the rows of H
 * they read; with NULL the two GEMMs always run as two launches. The values
 * do not depend on which form runs. In the single-launch form a GEMM2 tile's
 * wait for its rows of H is bounded (about 0.1 s); it has never been seen to
 * expire, but if it does, that tile's y_perm values are set to NaN rather
 * than computed from an incomplete H, and moe_ffn_status reports it. */
MOE_API moe_status_t moe_expert_ffn(const moe_desc_t* desc, const void* x_perm, const int32_t* expert_off,
                            const void* W1, const void* b1, const void* W2, const void* b2,
                            void* H, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* Gate-weighted combine, the layer output y = sum_i g_i(x) E_i(x) of
 * "MoE架构：突破单卡算力瓶颈的密钥" §1.2:
 * y[t] = sum over j with row_of[t*k+j] >= 0, in j order,
 * of topk_w[t, j] * y_perm[row_of[t*k+j]], accumulated in fp32 and rounded once;
 * a token with every choice dropped gets a zero row. y [T, d] X-dtype. */
MOE_API moe_status_t moe_combine(const moe_desc_t* desc, const void* y_perm, const int32_t* row_of,
                         const float* topk_w, void* y, void* stream);

/* Every tensor of one layer call. Inputs as for moe_route and moe_expert_ffn;
 * y is the output. The inspection outputs may each be NULL, in which case the
 * value lives only in the workspace. */
typedef struct moe_layer_tensors {
  const void* x;
  const void* w_gate;
  const void* w_noise;
  const float* noise;
  const void* proj;
  const float* expert_emb;
  const float* logit_bias;
  const void* W1;
  const void* b1;
  const void* W2;
  const void* b2;
  void* y;
  /* optional inspection outputs */
  float* logits;          /* [T, N] */
  int32_t* topk_idx;      /* [T, k] */
  float* topk_w;          /* [T, k] */
  int32_t* expert_count;  /* [N]   */
  int32_t* expert_off;    /* [N+1] */
  int32_t* row_of;        /* [T*k] */
  int32_t* token_of_row;  /* [R]   */
} moe_layer_tensors_t;

/* The whole layer: route, dispatch, expert FFN and combine, enqueued on one
 * stream with no host synchronisation (so it can be captured in a HIP
 * graph). Results are those of the four stage calls above, bitwise; the
 * expert rows are gathered from x inside GEMM1's tile loads, so no x_perm
 * copy is made (the row-grouped form of "MoE架构：稀疏激活机制如何提升模型计算
 * 效率" §3.1, fused). ws: MOE_WS_FORWARD bytes; it holds H, y_perm and every
 * routing array the caller does not ask for. */
MOE_API moe_status_t moe_forward(const moe_desc_t* desc, const moe_layer_tensors_t* tensors, void* ws,
                         size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and the same results as moe_forward, with the workspace
 * taken from a fixed device array inside the library instead of the
 * caller's. The array holds moe_noalloc_scratch_bytes() bytes (64 MiB) on
 * each GPU the library's code is loaded on, until the process ends. A layer
 * whose moe_workspace_size(MOE_WS_FORWARD) exceeds that gets
 * MOE_ERR_UNSUPPORTED before anything is enqueued (among the standard
 * shapes: the tiny, noisy top-2 and decode layers fit; the large-expert and
 * cosine layers do not). The call allocates nothing and frees nothing;
 * outputs and inspection outputs are the caller's, as for moe_forward.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (each call clears what it needs cleared), so calls that overlap in
 * time on one GPU (other streams, other threads) race: serialise them. */
MOE_API moe_status_t moe_forward_noalloc(const moe_desc_t* desc, const moe_layer_tensors_t* tensors,
                                         void* stream);
MOE_API size_t moe_noalloc_scratch_bytes(void);

/* Block-FP8 expert weights: FP8 weights shrink the model ("MoE架构：突破单卡
 * 算力瓶颈的密钥" §1.3), held with a scale per block ("Block FP8" serving on
 * MI300 in the CUDA-to-ROCm section of "4大技术模块掌握Tutel MoE…").
 * Quantises a stack W [groups, K, Ncols] of `dtype` values (MOE_F32 or
 * MOE_BF16; finite) in blocks of 128 x 128:
 *   scales [groups, K/128, Ncols/128] fp32: s = amax / 448, amax the
 *   largest |w| of the block (one fp32 division);
 *   codes: the OCP E4M3 byte (bias 7, 3 mantissa bits, largest 448) of the
 *   fp32 quotient w / s rounded to nearest, ties to even, with w's sign
 *   (saturated at 448, which only a block whose scale is an fp32 subnormal
 *   can reach); an all-zero block has s = 0 and zero codes.
 * codes layout: K-groups of 8, the byte of w[g][k][n] at
 *   ((g * K/8 + k/8) * Ncols + n) * 8 + k % 8,
 * so that each column's 8 consecutive K values are contiguous.
 * K and Ncols positive multiples of 128; W and codes 16-byte aligned,
 * scales 4-byte. Any other shape: MOE_ERR_INVALID. */
MOE_API moe_status_t moe_quantize_fp8(const void* W, int32_t dtype, int32_t groups, int32_t K, int32_t Ncols,
                                      uint8_t* codes, float* scales, void* stream);

/* moe_expert_ffn with block-FP8 expert weights (bf16 layers with d and h
 * multiples of 128 and at most 16384, else MOE_ERR_UNSUPPORTED): W1q / S1 are
 * moe_quantize_fp8 of W1 [N, d, h], W2q / S2 of W2 [N, h, d]. With W' the
 * dequantised weights (decoded code times its block's scale):
 *   H[r] = GELU(x_perm[r] W1'[e] + b1[e]), y_perm[r] = H[r] W2'[e] + b2[e],
 * each product accumulated in fp32 over each 128-deep block of K, scaled
 * once and added to the sum in K order; rounded once to bf16. Below 64
 * rows per expert (decoding, where the weight bytes bound the layer) the
 * kernel streams the weights with 32-row tiles; above, it takes 128 x 128
 * tiles. */
MOE_API moe_status_t moe_expert_ffn_fp8(const moe_desc_t* desc, const void* x_perm, const int32_t* expert_off,
                                        const uint8_t* W1q, const float* S1, const void* b1, const uint8_t* W2q,
                                        const float* S2, const void* b2, void* H, void* y_perm, void* stream);

/* A layer's block-FP8 expert weights (moe_quantize_fp8 of W1 and W2). */
typedef struct moe_fp8_weights {
  const uint8_t* W1q;
  const float* S1;
  const uint8_t* W2q;
  const float* S2;
} moe_fp8_weights_t;

/* moe_forward with the expert FFN of moe_expert_ffn_fp8: tensors->W1 and
 * tensors->W2 are not read (they may be NULL); the weights are w8's. The
 * routing and combine are moe_forward's. ws: MOE_WS_FORWARD bytes. */
MOE_API moe_status_t moe_forward_fp8(const moe_desc_t* desc, const moe_layer_tensors_t* tensors,
                                     const moe_fp8_weights_t* w8, void* ws, size_t ws_bytes, void* stream);

/* Load-balance terms of a routing (the topk_idx / topk_w that moe_route or
 * moe_forward produced), for an auxiliary training loss.
 *   importance [N] fp32: importance[e] = the sum over tokens t and choices j
 *   of topk_w[t, j] where topk_idx[t, j] == e, i.e. the column sums of the
 *   [T, N] sparse gate matrix, counted before capacity drops
 *   (gate_output.sum(dim=0) on "MoE架构：突破单卡算力瓶颈的密钥" §3.1,
 *   gates.sum(dim=0) on "MoE稀疏计算加速技术解析与应用实践" §4.1).
 *   losses [2] fp32: losses[0] = the sum over experts of
 *   (mean importance - importance[e])^2 (load_balance_loss of the first
 *   page); losses[1] = 0.1 times the standard deviation of importance with
 *   the N - 1 denominator (expert_importance_loss of the second page; NaN
 *   when N = 1).
 * Sums run in fp32 in a fixed order: repeated calls give the same bits.
 * Either output may be NULL (both NULL: nothing is launched). topk_idx
 * entries outside [0, N) count for no expert. ws: MOE_WS_AUX bytes. */
MOE_API moe_status_t moe_aux_loss(const moe_desc_t* desc, const int32_t* topk_idx, const float* topk_w,
                                  float* importance, float* losses, void* ws, size_t ws_bytes,
                                  void* stream);

/* Status of the expert FFN's single-launch form in the most recent
 * moe_forward (kind MOE_WS_FORWARD) or moe_expert_ffn (kind MOE_WS_FFN) call
 * made with this workspace: enqueues on `stream` a copy of its status word
 * into *status (a DEVICE int32; read it after the stream has reached this
 * point). 0: no GEMM2 tile's wait for its rows of H expired (also where the
 * layer does not use that form); bit 0 set: at least one did, and those
 * tiles' y_perm values (and so y) are NaN. The next layer call on the
 * workspace clears the word. Callers who capture the layer in a graph can
 * capture this call after it. */
MOE_API moe_status_t moe_ffn_status(const moe_desc_t* desc, moe_ws_kind_t kind, const void* ws, size_t ws_bytes,
                                    int32_t* status, void* stream);

/* Tensors of one backward call: the layer's inputs, the routing its forward
 * call produced (moe_forward's inspection outputs), the gradient dy of the
 * output, and the gradients to write. */
typedef struct moe_backward_tensors {
  /* inputs, as for moe_forward (logit_bias is not needed: its gradient does
     not depend on it) */
  const void* x;
  const void* w_gate;
  const void* w_noise;       /* NOISY */
  const float* noise;        /* NOISY */
  const void* W1;
  const void* b1;            /* or NULL */
  const void* W2;
  const void* b2;            /* or NULL */
  /* the forward's routing */
  const float* logits;       /* [T, N] (read when renorm = 0) */
  const int32_t* topk_idx;   /* [T, k] */
  const float* topk_w;       /* [T, k] */
  const int32_t* expert_off; /* [N+1] */
  const int32_t* row_of;     /* [T*k] */
  const int32_t* token_of_row; /* [R] */
  const void* dy;            /* [T, d] X-dtype: dL/dy */
  /* outputs */
  void* dx;                  /* [T, d] X-dtype */
  float* dW1;                /* [N, d, h] */
  float* dW2;                /* [N, h, d] */
  float* db1;                /* [N, h] or NULL (not computed) */
  float* db2;                /* [N, d] or NULL */
  float* dw_gate;            /* [d, N] */
  float* dw_noise;           /* [d, N] (NOISY) */
  float* dlogit_bias;        /* [N] or NULL */
} moe_backward_tensors_t;

/* Backward pass of the layer: the gradients of
 *   L = sum(dy * y) + aux_coef[0] * load_balance_loss + aux_coef[1] * importance_loss
 * (the two losses of moe_aux_loss, on the importance of the same routing)
 * with respect to x, W1, b1, W2, b2, w_gate, w_noise and logit_bias, the
 * routing held fixed: gradients flow only through the selected experts' gate
 * weights and outputs ("MoE稀疏计算加速技术解析与应用实践" §2.1: sparse gating
 * keeps only the Top-K experts' gradient; the auxiliary losses are added to
 * the total loss on its §4.1 and on "MoE架构：突破单卡算力瓶颈的密钥" §3.1). A
 * choice dropped by the capacity limit contributes nothing to y, so its
 * weight gets no gradient from y, but it still counts in the importance.
 * The noise tensor is an input, not a parameter.
 * Per kept row (token t, choice j, expert e, weight w): the expert's
 * pre-activation U = x W1_e + b1_e and H = GELU(U) are recomputed (bf16);
 * dU = bf16(w (dy_t W2_e^T) GELU'(U)); the weight's gradient is
 * (dy_t W2_e^T) . H (+ dy_t . b2_e); dW2_e = sum H^T bf16(w dy_t),
 * dW1_e = sum x^T dU, dx = sum over kept j of dU W1_e^T plus the gate's
 * part (through the softmax over the selected logits, renorm = 1, or over
 * all logits, renorm = 0; through softplus for the noisy gate). All
 * products on bf16 MFMA with fp32 accumulation; every reduction in a fixed
 * order (repeated calls give the same bits).
 * bf16 layers with the SOFTMAX or NOISY gate; others get MOE_ERR_UNSUPPORTED,
 * as do layers with R * max(d, h) * 2 bytes at or above 2^31 (R = the row
 * bound). aux_coef: two host floats, or NULL for none.
 * ws: MOE_WS_BACKWARD bytes. */
MOE_API moe_status_t moe_backward(const moe_desc_t* desc, const moe_backward_tensors_t* tensors,
                                  const float* aux_coef, void* ws, size_t ws_bytes, void* stream);

/* Profiling aid. While set, the expert FFN's kernel launches (in
 * moe_expert_ffn and moe_forward) record start_event (a hipEvent_t) when the
 * FFN's first kernel begins executing and stop_event when its last kernel
 * ends (hipExtLaunchKernel), so that hipEventElapsedTime(start, stop) is the
 * FFN's execution time without launch overheads; with two launches that span
 * includes the gap between them. NULL for both switches it off. The caller
 * creates the events and keeps them alive while they are set. The setting is
 * process-wide and unsynchronised: change it while no other thread enqueues
 * layers. Always returns MOE_OK. */
MOE_API moe_status_t moe_time_ffn_launches(void* start_event, void* stop_event);

/* Per-item trace of the single-launch expert FFN, a measurement aid of the
 * trace build (libmoe_gfx950_trace.so, compiled with MOE_FFN_TRACE; the
 * release and debug builds record nothing). Each block of that launch writes
 * one record per work item it runs (its first 64 items), overwriting those
 * of earlier launches: 8 uint64 per record, block b's item i at record
 * b * 64 + i, for 256 blocks: [0] wall clock (100 MHz counter) when the item
 * starts, [1] after a GEMM2 item's wait for its rows of H, [2] when it ends;
 * [3], [4] the shader cycle counter at its start and end (cycles over wall
 * time give the clock it ran at); [5] XCD | kind << 4 (1: GEMM1, 2: GEMM2)
 * | tail tile << 8 | launch number << 32 (1, 2, ... per process); [6] the
 * row tile; [7] the first output column. Unwritten records are zero.
 * moe_ffn_trace_bytes: the size of the record array (0 in other builds).
 * moe_ffn_trace_read: copies it to host memory of that size, synchronously
 * (after the device's work so far); MOE_ERR_UNSUPPORTED in other builds. */
MOE_API size_t moe_ffn_trace_bytes(void);
MOE_API moe_status_t moe_ffn_trace_read(void* host);

/* Measurement aids, to judge the layer's kernels against the chip's measured
 * ceilings as well as its published ones (run in the same process, timed by
 * the caller with events around the call).
 * moe_probe_copy: copies `bytes` (a positive multiple of 16) from src to dst
 * (device, 16-byte aligned, not overlapping) with 16-byte loads and stores;
 * moved bytes = 2 * bytes (read + write).
 * moe_probe_mfma: `iters` rounds of bf16 32x32x16 MFMAs on register operands
 * over the whole chip, no memory traffic; *flops (host) receives the flops it
 * performs; sink: a device array of moe_probe_mfma_sink_floats() floats that
 * receives meaningless sums (so that the work cannot be removed). */
MOE_API moe_status_t moe_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);
MOE_API moe_status_t moe_probe_mfma(int32_t iters, float* sink, int64_t* flops, void* stream);
MOE_API int64_t moe_probe_mfma_sink_floats(void);

/* Static name of a status code. */
MOE_API const char* moe_status_string(moe_status_t status);

/* Message of this thread's last failed call ("" if none). */
MOE_API const char* moe_last_error(void);

/* Build identification, e.g. "moe gfx950 <date>". */
MOE_API const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
