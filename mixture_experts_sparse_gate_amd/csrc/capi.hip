// C ABI of the MoE layer (declared in include/moe.h): argument checks on the
// host, workspace carve-up and the launch sequence. Nothing here allocates,
// frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "moe.h"
#include "kernels.hpp"
#include "routing_check.h"

namespace {

thread_local char g_last_error[512] = "";

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

moe_status_t hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(const moe_desc_t* d) { return d->dtype == MOE_BF16 ? 2 : 4; }
int chunk_elems(const moe_desc_t* d) { return d->dtype == MOE_BF16 ? 8 : 4; }

int64_t capacity_of(const moe_desc_t* d) {
  const double c = ceil((d->capacity_factor * (double)(d->T * d->k)) / (double)d->N);
  return c < (double)d->T ? (int64_t)c : d->T;
}

int64_t rows_bound_of(const moe_desc_t* d) {
  const int64_t a = d->T * d->k, b = (int64_t)d->N * capacity_of(d);
  return a < b ? a : b;
}

int ntiles_of(const moe_desc_t* d) {
  return (int)((d->T + moe::kDispatchTile - 1) / moe::kDispatchTile);
}

moe_status_t check_desc(const moe_desc_t* d) {
  if (!d) return fail(MOE_ERR_INVALID, "desc is NULL");
  if (d->flags & ~MOE_FLAG_COMBINE_IN_FFN)
    return fail(MOE_ERR_INVALID, "desc->flags: unknown bits 0x%x", (unsigned)(d->flags & ~MOE_FLAG_COMBINE_IN_FFN));
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID, "dtype %d is not MOE_F32 or MOE_BF16", d->dtype);
  if (d->gate < MOE_GATE_SOFTMAX || d->gate > MOE_GATE_COSINE)
    return fail(MOE_ERR_INVALID, "gate %d is not a moe_gate_t", d->gate);
  if (d->renorm != 0 && d->renorm != 1) return fail(MOE_ERR_INVALID, "renorm must be 0 or 1");
  if (d->T < 1) return fail(MOE_ERR_INVALID, "T = %lld must be >= 1", (long long)d->T);
  if (d->N < 1 || d->N > 256) return fail(MOE_ERR_INVALID, "N = %d must be in [1, 256]", d->N);
  if (d->k < 1 || d->k > d->N || d->k > 32)
    return fail(MOE_ERR_INVALID, "k = %d must be in [1, min(N, 32)]", d->k);
  if (d->T * (int64_t)d->k >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID, "T*k must be below 2^31");
  if (!(d->capacity_factor > 0.0) || !isfinite(d->capacity_factor))
    return fail(MOE_ERR_INVALID, "capacity_factor must be finite and > 0");
  const int ce = chunk_elems(d);
  if (d->d < 1 || d->d % ce) return fail(MOE_ERR_INVALID, "d = %d must be a positive multiple of %d", d->d, ce);
  if (d->h < 1 || d->h % ce) return fail(MOE_ERR_INVALID, "h = %d must be a positive multiple of %d", d->h, ce);
  if (d->gate == MOE_GATE_COSINE) {
    if (d->proj_dim < 8 || d->proj_dim > 256 || d->proj_dim % 8)
      return fail(MOE_ERR_INVALID, "proj_dim = %d must be a multiple of 8 in [8, 256]", d->proj_dim);
    if (!isfinite(d->inv_temperature))
      return fail(MOE_ERR_INVALID, "inv_temperature must be finite");
  }
  // the kernels address each operand through buffer descriptors with 32-bit
  // byte ranges and offsets: every operand they cover stays below 2^31 bytes
  const int64_t s = elem_bytes(d), lim = (int64_t)1 << 31;
  const int64_t wide = d->d > d->h ? d->d : d->h;
  const int64_t gate_cols = d->gate == MOE_GATE_COSINE ? d->proj_dim : d->N;
  if (d->T * wide * s >= lim || (int64_t)d->d * d->h * s >= lim || (int64_t)d->d * gate_cols * s >= lim)
    return fail(MOE_ERR_UNSUPPORTED, "T*max(d,h), d*h and d*%s must each stay below 2^31 bytes",
                d->gate == MOE_GATE_COSINE ? "proj_dim" : "N");
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status_t need(const void* p, const char* name, size_t align) {
  if (!p) return fail(MOE_ERR_INVALID, "%s is NULL", name);
  if (!aligned(p, align)) return fail(MOE_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
  return MOE_OK;
}

moe_status_t maybe(const void* p, const char* name, size_t align) {
  if (p && !aligned(p, align)) return fail(MOE_ERR_INVALID, "%s is not %zu-byte aligned", name, align);
  return MOE_OK;
}

#define TRY(expr)                       \
  do {                                  \
    moe_status_t st__ = (expr);         \
    if (st__ != MOE_OK) return st__;    \
  } while (0)

// ---------------------------------------------------------------- workspace

struct RouteWs {
  size_t z, logits, partial, hist, bytes;
  bool has_hist;  // the gate writes per-32-token choice counts (for moe_forward's dispatch)
};
RouteWs route_ws(const moe_desc_t* d) {
  RouteWs w{};
  size_t o = 0;
  w.z = o;
  if (d->gate == MOE_GATE_COSINE) o += align_up((size_t)d->T * d->proj_dim * 4);
  w.logits = o;
  o += align_up((size_t)d->T * d->N * 4);
  w.partial = o;
  if (d->gate != MOE_GATE_COSINE && d->dtype == MOE_BF16)
    o += align_up(moe::gate_partial_bytes(d->T, d->d, d->N, d->gate == MOE_GATE_NOISY));
  w.hist = o;
  w.has_hist = d->gate != MOE_GATE_COSINE &&
               moe::gate_writes_hist(d->dtype == MOE_BF16, d->gate == MOE_GATE_NOISY, d->N);
  if (w.has_hist)
    o += align_up((size_t)((d->T + moe::kGateHistTokens - 1) / moe::kGateHistTokens) * d->N * 4);
  w.bytes = o;
  return w;
}

// per-tile counts, and (for large count tables) the scan's per-tile
// prefixes and totals
struct DispatchWs {
  size_t tile_counts, tile_start, totals, bytes;
};
DispatchWs dispatch_ws(const moe_desc_t* d) {
  DispatchWs w{};
  const size_t t = (size_t)ntiles_of(d) * d->N * 4;
  w.tile_counts = 0;
  w.tile_start = align_up(t);
  w.totals = w.tile_start + align_up(t);
  w.bytes = w.totals + align_up((size_t)d->N * 4);
  return w;
}

struct ForwardWs {
  size_t route, dispatch, ffn_counters, arrive, topk_idx, topk_w, count, off, row_of, token_of_row, H,
      y_perm, bytes;
  int n_counters;
  int arrive_per_token;  // > 0: the single-launch FFN also does the combine
};
int ffn_counters_of(const moe_desc_t* d);
bool combine_in_ffn(const moe_desc_t* d);
ForwardWs forward_ws(const moe_desc_t* d) {
  ForwardWs w{};
  const size_t Tk = (size_t)d->T * d->k, R = (size_t)rows_bound_of(d), s = elem_bytes(d);
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += align_up(n);
    return at;
  };
  w.route = take(route_ws(d).bytes);
  w.dispatch = take(dispatch_ws(d).bytes);
  w.n_counters = ffn_counters_of(d);
  w.ffn_counters = take((size_t)w.n_counters * 4);
  w.arrive_per_token = combine_in_ffn(d) ? moe::fused_combine_col_tiles(d->d) : 0;
  w.arrive = take((size_t)d->T * w.arrive_per_token * 4);
  w.topk_idx = take(Tk * 4);
  w.topk_w = take(Tk * 4);
  w.count = take((size_t)d->N * 4);
  w.off = take((size_t)(d->N + 1) * 4);
  w.row_of = take(Tk * 4);
  w.token_of_row = take(R * 4);
  w.H = take(R * d->h * s);
  w.y_perm = take(R * d->d * s);
  w.bytes = o;
  return w;
}

// the backward pass: expert-ordered rows of x and of w dy, U, H, dU, the
// partial dots, the fp32 dx rows, dl and dz, the load-balance staging and
// the gate gradients' partial sums
struct BackwardWs {
  size_t x_perm, dY, U, H, dU, pd, dx_perm, dl, dz, imp_part, imp, dimp, gpart, bytes;
};
BackwardWs backward_ws(const moe_desc_t* d) {
  BackwardWs w{};
  const size_t R = (size_t)rows_bound_of(d), T = (size_t)d->T;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t a = o;
    o += align_up(n);
    return a;
  };
  w.x_perm = take(R * d->d * 2);
  w.dY = take(R * d->d * 2);
  w.U = take(R * d->h * 2);
  w.H = take(R * d->h * 2);
  w.dU = take(R * d->h * 2);
  w.pd = take(R * (size_t)((d->h + 127) / 128) * 4);
  w.dx_perm = take(R * d->d * 4);
  w.dl = take(T * d->N * 4);
  w.dz = take(T * d->N * 4);
  w.imp_part = take((size_t)moe::aux_blocks(d->T) * d->N * 4);
  w.imp = take((size_t)d->N * 4);
  w.dimp = take((size_t)d->N * 4);
  const size_t chunks = (size_t)moe::gate_grad_chunks(d->T);
  const size_t np = (size_t)d->N * (d->gate == MOE_GATE_NOISY ? 2 : 1);
  const size_t gp = chunks * d->d * np * 4, bp = chunks * d->N * 4;
  w.gpart = take(gp > bp ? gp : bp);
  w.bytes = o;
  return w;
}

// layers the backward serves: bf16, plain or noisy gate, and row buffers
// whose byte ranges fit the kernels' 32-bit buffer descriptors
moe_status_t check_backward(const moe_desc_t* d) {
  TRY(check_desc(d));
  if (d->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_backward needs a bf16 layer");
  if (d->gate == MOE_GATE_COSINE) return fail(MOE_ERR_UNSUPPORTED, "moe_backward covers the plain and noisy gates");
  const int64_t R = rows_bound_of(d), wide = d->d > d->h ? d->d : d->h;
  if (R * wide * 2 >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward: R*max(d,h)*2 = %lld bytes must stay below 2^31",
                (long long)(R * wide * 2));
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// ---------------------------------------------------------------- stages (arguments checked)

// hist: the gate's per-32-token choice counts (route_ws().hist, where
// has_hist), or null
moe_status_t do_route(const moe_desc_t* d, const void* x, const void* w_gate, const void* w_noise,
                      const float* noise, const void* proj, const float* emb, const float* bias,
                      float* logits, int32_t* idx, float* w, void* ws, hipStream_t s,
                      int32_t* hist = nullptr) {
  const RouteWs rw = route_ws(d);
  const bool bf = d->dtype == MOE_BF16;
  if (d->gate == MOE_GATE_COSINE) {
    float* z = at<float>(ws, rw.z);
    moe::GemmParams g{};
    g.A = x;
    g.B = proj;
    g.C = z;
    g.lda = d->d;
    g.ldc = d->proj_dim;
    g.M = (int)d->T;
    g.groups = 1;
    g.K = d->d;
    g.Ncols = d->proj_dim;
    TRY(hip_status(moe::launch_grouped_gemm(g, moe::GemmKind::kProjF32, bf, (int)d->T, (int)d->T, s),
                   "cosine projection"));
    moe::CosineParams c{};
    c.z = z;
    c.emb = emb;
    c.logit_bias = bias;
    c.inv_temperature = d->inv_temperature;
    c.logits = logits;
    c.topk_idx = idx;
    c.topk_w = w;
    c.T = (int)d->T;
    c.p = d->proj_dim;
    c.N = d->N;
    c.k = d->k;
    c.renorm = d->renorm;
    return hip_status(moe::launch_cosine_select(c, s), "cosine gate");
  }
  moe::GateParams g{};
  g.x = x;
  g.w_gate = w_gate;
  g.w_noise = w_noise;
  g.noise = noise;
  g.logit_bias = bias;
  g.logits = logits ? logits : at<float>(ws, rw.logits);
  g.topk_idx = idx;
  g.topk_w = w;
  g.partial = at<float>(ws, rw.partial);
  g.hist = rw.has_hist ? hist : nullptr;
  g.T = (int)d->T;
  g.d = d->d;
  g.N = d->N;
  g.k = d->k;
  g.renorm = d->renorm;
  return hip_status(moe::launch_gate_plain_noisy(g, bf, d->gate == MOE_GATE_NOISY, s), "gate");
}

// zero, zero_n: ints for the dispatch to clear on the way (the fused FFN's
// counters), or null; zero_tok, zero_tok_n: ints per token to clear (the
// folded combine's arrival counts), or null
// hist32: the gate's per-32-token choice counts, or null (counted here)
// caller_routing: idx comes from the caller (moe_dispatch), not the gate
moe_status_t do_dispatch(const moe_desc_t* d, const void* x, const int32_t* idx, int32_t* count,
                         int32_t* off, int32_t* row_of, int32_t* token_of_row, void* x_perm,
                         void* ws, hipStream_t s, int32_t* zero = nullptr, int zero_n = 0,
                         const int32_t* hist32 = nullptr, bool caller_routing = false,
                         int32_t* zero_tok = nullptr, int zero_tok_n = 0) {
  const DispatchWs dw = dispatch_ws(d);
  moe::DispatchParams p{};
  p.x = x;
  p.topk_idx = idx;
  p.tile_counts = at<int32_t>(ws, dw.tile_counts);
  p.tile_start = at<int32_t>(ws, dw.tile_start);
  p.totals = at<int32_t>(ws, dw.totals);
  p.caller_routing = caller_routing ? 1 : 0;
  p.expert_count = count;
  p.expert_off = off;
  p.row_of = row_of;
  p.token_of_row = token_of_row;
  p.x_perm = x_perm;
  p.T = (int)d->T;
  p.d = d->d;
  p.N = d->N;
  p.k = d->k;
  p.C = (int)capacity_of(d);
  p.elem_bytes = elem_bytes(d);
  p.zero = zero;
  p.zero_n = zero_n;
  p.zero_tok = zero_tok;
  p.zero_tok_n = zero_tok_n;
  p.hist32 = hist32;
  return hip_status(moe::launch_dispatch(p, s), "dispatch");
}

// The two expert GEMMs. A1: GEMM1's activation rows. With token_of_row null
// they are the rows of x_perm; otherwise A1 is x itself and row r reads token
// token_of_row[r] / k (the gather fused into GEMM1's tile loads, no x_perm
// round trip). Pointers may be null where only the shapes matter.
void ffn_gemms(const moe_desc_t* d, const void* A1, const int32_t* token_of_row, const int32_t* off,
               const void* W1, const void* b1, const void* W2, const void* b2, void* H, void* y_perm,
               moe::GemmParams* g1, moe::GemmParams* g2) {
  moe::GemmParams& g = *g1;
  g = moe::GemmParams{};
  g.A = A1;
  g.gather = token_of_row;
  g.gather_div = d->k;
  g.a_rows = (int)d->T;
  g.B = W1;
  g.bias = b1;
  g.C = H;
  g.seg = off;
  g.lda = d->d;
  g.ldc = d->h;
  g.strideB = (int64_t)d->d * d->h;
  g.strideBias = d->h;
  g.M = (int)rows_bound_of(d);
  g.groups = d->N;
  g.K = d->d;
  g.Ncols = d->h;
  moe::GemmParams& h = *g2;
  h = g;
  h.A = H;
  h.gather = nullptr;
  h.B = W2;
  h.bias = b2;
  h.C = y_perm;
  h.lda = d->h;
  h.ldc = d->d;
  h.strideB = (int64_t)d->h * d->d;
  h.strideBias = d->d;
  h.K = d->h;
  h.Ncols = d->d;
}

// counters of the fused FFN launch for this layer (0 where it does not apply)
int ffn_counters_of(const moe_desc_t* d) {
  static const int32_t shape_only[1] = {0};  // sizing reads no pointer
  moe::GemmParams g1, g2;
  ffn_gemms(d, nullptr, nullptr, shape_only, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &g1, &g2);
  const int avg_rows = (int)((d->T * d->k) / d->N);
  return moe::fused_ffn_fits(g1, g2, d->dtype == MOE_BF16, avg_rows) ? moe::fused_ffn_counters(g1) : 0;
}

// moe_forward folds the combine into the single-launch FFN where the caller
// asks for it (MOE_FLAG_COMBINE_IN_FFN), that launch applies, and k is
// within its per-token batches
bool combine_in_ffn(const moe_desc_t* d) {
  return (d->flags & MOE_FLAG_COMBINE_IN_FFN) && ffn_counters_of(d) > 0 && d->k <= moe::kFusedCombineMaxK;
}

// The single-launch FFN deals its work to one queue per XCD of the full
// chip (256 CUs in 8 XCDs), each queue drained by the blocks whose hardware
// XCC_ID names it. A device that is a partition of the chip has fewer XCDs,
// so some queues would have no blocks and their tiles would never run: such
// a device takes the two grouped-GEMM launches, whose result does not depend
// on where blocks are placed.
bool whole_chip_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> known[kMaxDevices];  // 0 unknown, 1 whole chip, 2 not
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  int v = known[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    const bool ok =
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus == 256;
    v = ok ? 1 : 2;
    known[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1;
}

// counters: fused-FFN counters (ffn_counters_of ints; cleared here unless
// cleared says the dispatch did it) or null for two grouped-GEMM launches.
// Both give the same bits.
// Events the expert FFN's launches record (moe_time_ffn_launches), or null.
moe::LaunchEvents g_ffn_events;

// comb: the combine to fold into the single-launch form (or null); *combined
// (if given) tells whether it was folded in (else the caller combines).
moe_status_t do_ffn(const moe_desc_t* d, const void* A1, const int32_t* token_of_row,
                    const int32_t* off, const void* W1, const void* b1, const void* W2,
                    const void* b2, void* H, void* y_perm, int32_t* counters, bool cleared, hipStream_t s,
                    const moe::FusedCombine* comb = nullptr, bool* combined = nullptr) {
  const bool bf = d->dtype == MOE_BF16;
  const int avg_rows = (int)((d->T * d->k) / d->N);
  const int max_rows = (int)capacity_of(d);
  moe::GemmParams g1, g2;
  ffn_gemms(d, A1, token_of_row, off, W1, b1, W2, b2, H, y_perm, &g1, &g2);
  const moe::LaunchEvents ev = g_ffn_events;
  if (combined) *combined = false;
  if (counters && moe::fused_ffn_fits(g1, g2, bf, avg_rows) && whole_chip_device()) {
    if (combined) *combined = comb != nullptr;
    return hip_status(moe::launch_fused_ffn(g1, g2, counters, !cleared, s, ev, comb), "expert FFN");
  }
  TRY(hip_status(moe::launch_grouped_gemm(g1, moe::GemmKind::kFfn1Gelu, bf, avg_rows, max_rows, s, {ev.start, nullptr}),
                 "expert GEMM1"));
  return hip_status(moe::launch_grouped_gemm(g2, moe::GemmKind::kFfn2, bf, avg_rows, max_rows, s, {nullptr, ev.stop}),
                    "expert GEMM2");
}

// The expert FFN on block-FP8 weights (moe_expert_ffn_fp8): two launches.
moe_status_t do_ffn_w8(const moe_desc_t* d, const void* A1, const int32_t* token_of_row, const int32_t* off,
                       const uint8_t* W1q, const float* S1, const void* b1, const uint8_t* W2q, const float* S2,
                       const void* b2, void* H, void* y_perm, hipStream_t s) {
  moe::GemmParams g1, g2;
  ffn_gemms(d, A1, token_of_row, off, W1q, b1, W2q, b2, H, y_perm, &g1, &g2);
  const moe::LaunchEvents ev = g_ffn_events;
  const int avg_rows = (int)((d->T * d->k) / d->N);
  TRY(hip_status(moe::launch_grouped_gemm_w8(g1, moe::GemmW8{S1}, moe::GemmKind::kFfn1Gelu, avg_rows, s,
                                             {ev.start, nullptr}),
                 "expert GEMM1 (fp8 weights)"));
  return hip_status(moe::launch_grouped_gemm_w8(g2, moe::GemmW8{S2}, moe::GemmKind::kFfn2, avg_rows, s,
                                                {nullptr, ev.stop}),
                    "expert GEMM2 (fp8 weights)");
}

// layers the block-FP8 FFN serves: bf16, d and h whole 128-wide scale blocks
moe_status_t check_fp8_layer(const moe_desc_t* d) {
  if (d->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "fp8 expert weights need a bf16 layer");
  if (d->d % 128 || d->h % 128)
    return fail(MOE_ERR_UNSUPPORTED, "fp8 expert weights need d and h multiples of 128 (d=%d, h=%d)", d->d, d->h);
  if (d->d > moe::kW8MaxK || d->h > moe::kW8MaxK)
    return fail(MOE_ERR_UNSUPPORTED, "fp8 expert weights need d and h at most %d (d=%d, h=%d)", moe::kW8MaxK, d->d,
                d->h);
  return MOE_OK;
}

moe_status_t do_combine(const moe_desc_t* d, const void* y_perm, const int32_t* row_of,
                        const float* w, void* y, hipStream_t s) {
  moe::CombineParams c{};
  c.y_perm = y_perm;
  c.row_of = row_of;
  c.topk_w = w;
  c.y = y;
  c.T = (int)d->T;
  c.d = d->d;
  c.k = d->k;
  c.R = (int)rows_bound_of(d);
  return hip_status(moe::launch_combine(c, d->dtype == MOE_BF16, s), "combine");
}

moe_status_t check_gate_inputs(const moe_desc_t* d, const void* x, const void* w_gate,
                               const void* w_noise, const float* noise, const void* proj,
                               const float* emb, const float* bias) {
  TRY(need(x, "x", 16));
  if (d->gate == MOE_GATE_SOFTMAX || d->gate == MOE_GATE_NOISY) TRY(need(w_gate, "w_gate", 16));
  if (d->gate == MOE_GATE_NOISY) {
    TRY(need(w_noise, "w_noise", 16));
    TRY(need(noise, "noise", 4));
  }
  if (d->gate == MOE_GATE_COSINE) {
    TRY(need(proj, "proj", 16));
    TRY(need(emb, "expert_emb", 4));
  }
  TRY(maybe(bias, "logit_bias", 4));
  return MOE_OK;
}

moe_status_t check_ws(void* ws, size_t have, size_t want) {
  if (want == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL, %zu bytes needed", want);
  if (!aligned(ws, kAlign)) return fail(MOE_ERR_INVALID, "workspace is not %zu-byte aligned", kAlign);
  if (have < want) return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, want);
  return MOE_OK;
}

// moe_forward, and with w8 non-null moe_forward_fp8
moe_status_t forward_impl(const moe_desc_t* desc, const moe_layer_tensors_t* t, const moe_fp8_weights_t* w8,
                          void* ws, size_t ws_bytes, void* stream) {
  TRY(check_desc(desc));
  if (!t) return fail(MOE_ERR_INVALID, "tensors is NULL");
  TRY(check_gate_inputs(desc, t->x, t->w_gate, t->w_noise, t->noise, t->proj, t->expert_emb,
                        t->logit_bias));
  if (w8) {
    TRY(check_fp8_layer(desc));
    TRY(need(w8->W1q, "W1q", 16));
    TRY(need(w8->S1, "S1", 4));
    TRY(need(w8->W2q, "W2q", 16));
    TRY(need(w8->S2, "S2", 4));
  } else {
    TRY(need(t->W1, "W1", 16));
    TRY(need(t->W2, "W2", 16));
  }
  TRY(maybe(t->b1, "b1", 4));
  TRY(maybe(t->b2, "b2", 4));
  TRY(need(t->y, "y", 16));
  TRY(maybe(t->logits, "logits", 4));
  TRY(maybe(t->topk_idx, "topk_idx", 4));
  TRY(maybe(t->topk_w, "topk_w", 4));
  TRY(maybe(t->expert_count, "expert_count", 4));
  TRY(maybe(t->expert_off, "expert_off", 4));
  TRY(maybe(t->row_of, "row_of", 4));
  TRY(maybe(t->token_of_row, "token_of_row", 4));
  const ForwardWs fw = forward_ws(desc);
  TRY(check_ws(ws, ws_bytes, fw.bytes));
  hipStream_t s = (hipStream_t)stream;
  int32_t* idx = t->topk_idx ? t->topk_idx : at<int32_t>(ws, fw.topk_idx);
  float* w = t->topk_w ? t->topk_w : at<float>(ws, fw.topk_w);
  int32_t* count = t->expert_count ? t->expert_count : at<int32_t>(ws, fw.count);
  int32_t* off = t->expert_off ? t->expert_off : at<int32_t>(ws, fw.off);
  int32_t* row_of = t->row_of ? t->row_of : at<int32_t>(ws, fw.row_of);
  int32_t* tor = t->token_of_row ? t->token_of_row : at<int32_t>(ws, fw.token_of_row);
  void* H = at<char>(ws, fw.H);
  void* y_perm = at<char>(ws, fw.y_perm);
  // the gate also counts each 32 tokens' choices where it can, which
  // spares the dispatch its counting pass
  const RouteWs rw = route_ws(desc);
  int32_t* hist = rw.has_hist ? at<int32_t>(ws, fw.route + rw.hist) : nullptr;
  TRY(do_route(desc, t->x, t->w_gate, t->w_noise, t->noise, t->proj, t->expert_emb, t->logit_bias,
               t->logits, idx, w, at<char>(ws, fw.route), s, hist));
  // routing and row maps only: GEMM1 gathers its rows from x itself
  // (the dispatch also clears the fused FFN's counters)
  int32_t* counters = fw.n_counters ? at<int32_t>(ws, fw.ffn_counters) : nullptr;
  // the combine folded into the single-launch FFN (bf16 weights, on request):
  // its per-(token, column tile) arrival counts are cleared by the dispatch
  const bool fold = !w8 && fw.arrive_per_token > 0;
  int32_t* arrive = fold ? at<int32_t>(ws, fw.arrive) : nullptr;
  TRY(do_dispatch(desc, t->x, idx, count, off, row_of, tor, nullptr, at<char>(ws, fw.dispatch), s, counters,
                  fw.n_counters, hist, false, arrive, fold ? fw.arrive_per_token : 0));
  bool combined = false;
  if (w8) {
    TRY(do_ffn_w8(desc, t->x, tor, off, w8->W1q, w8->S1, t->b1, w8->W2q, w8->S2, t->b2, H, y_perm, s));
  } else {
    const moe::FusedCombine comb{row_of, tor, w, t->y, arrive, (int)desc->T, desc->k};
    TRY(do_ffn(desc, t->x, tor, off, t->W1, t->b1, t->W2, t->b2, H, y_perm, counters, true, s,
               fold ? &comb : nullptr, &combined));
  }
  if (combined) return MOE_OK;
  return do_combine(desc, y_perm, row_of, w, t->y, s);
}

// ---------------------------------------------------------------- no-allocation forward

// moe_forward_noalloc's workspace: a file-scope device array, one copy per
// GPU (held from when the library's code is loaded on that GPU until the
// process ends). Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): it uses the device address
// hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

// The scratch array's device address on the current device, fetched once
// per device (with that device current) and kept.
moe_status_t scratch_on_current_device(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    addr[dev] = p;
  }
  *out = addr[dev];
  return MOE_OK;
}

#ifdef MOE_DEBUG_CHECKS
// Debug builds: the caller's routing is copied to the host (synchronising
// the stream) and checked: every index in [0, N), distinct per token.
moe_status_t debug_check_routing(const moe_desc_t* d, const int32_t* idx, hipStream_t s) {
  const size_t n = (size_t)d->T * d->k;
  std::vector<int32_t> h(n);
  TRY(hip_status(hipMemcpyAsync(h.data(), idx, n * 4, hipMemcpyDeviceToHost, s), "debug routing copy"));
  TRY(hip_status(hipStreamSynchronize(s), "debug routing copy"));
  char msg[256];
  if (moe_check_routing_host(h.data(), d->T, d->k, d->N, msg, sizeof(msg)) != 0)
    return fail(MOE_ERR_INVALID, "topk_idx: %s", msg);
  return MOE_OK;
}
#endif

}  // namespace

extern "C" {

int64_t moe_capacity(const moe_desc_t* desc) {
  if (check_desc(desc) != MOE_OK) return -1;
  return capacity_of(desc);
}

int64_t moe_rows_bound(const moe_desc_t* desc) {
  if (check_desc(desc) != MOE_OK) return -1;
  return rows_bound_of(desc);
}

moe_status_t moe_workspace_size(const moe_desc_t* desc, moe_ws_kind_t kind, size_t* bytes) {
  TRY(check_desc(desc));
  if (!bytes) return fail(MOE_ERR_INVALID, "bytes is NULL");
  switch (kind) {
    case MOE_WS_ROUTE: *bytes = route_ws(desc).bytes; return MOE_OK;
    case MOE_WS_DISPATCH: *bytes = dispatch_ws(desc).bytes; return MOE_OK;
    case MOE_WS_FORWARD: *bytes = forward_ws(desc).bytes; return MOE_OK;
    case MOE_WS_FFN: *bytes = align_up((size_t)ffn_counters_of(desc) * 4); return MOE_OK;
    case MOE_WS_AUX: *bytes = align_up((size_t)moe::aux_blocks(desc->T) * desc->N * 4); return MOE_OK;
    case MOE_WS_BACKWARD: *bytes = backward_ws(desc).bytes; return MOE_OK;
  }
  return fail(MOE_ERR_INVALID, "unknown workspace kind %d", (int)kind);
}

moe_status_t moe_route(const moe_desc_t* desc, const void* x, const void* w_gate,
                       const void* w_noise, const float* noise, const void* proj,
                       const float* expert_emb, const float* logit_bias, float* logits,
                       int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_desc(desc));
  TRY(check_gate_inputs(desc, x, w_gate, w_noise, noise, proj, expert_emb, logit_bias));
  TRY(maybe(logits, "logits", 4));
  TRY(need(topk_idx, "topk_idx", 4));
  TRY(need(topk_w, "topk_w", 4));
  TRY(check_ws(ws, ws_bytes, route_ws(desc).bytes));
  return do_route(desc, x, w_gate, w_noise, noise, proj, expert_emb, logit_bias, logits, topk_idx,
                  topk_w, ws, (hipStream_t)stream);
}

moe_status_t moe_dispatch(const moe_desc_t* desc, const void* x, const int32_t* topk_idx,
                          int32_t* expert_count, int32_t* expert_off, int32_t* row_of,
                          int32_t* token_of_row, void* x_perm, void* ws, size_t ws_bytes,
                          void* stream) {
  TRY(check_desc(desc));
  TRY(need(x, "x", 16));
  TRY(need(topk_idx, "topk_idx", 4));
  TRY(need(expert_count, "expert_count", 4));
  TRY(need(expert_off, "expert_off", 4));
  TRY(need(row_of, "row_of", 4));
  TRY(need(token_of_row, "token_of_row", 4));
  TRY(need(x_perm, "x_perm", 16));
  TRY(check_ws(ws, ws_bytes, dispatch_ws(desc).bytes));
#ifdef MOE_DEBUG_CHECKS
  TRY(debug_check_routing(desc, topk_idx, (hipStream_t)stream));
#endif
  return do_dispatch(desc, x, topk_idx, expert_count, expert_off, row_of, token_of_row, x_perm, ws,
                     (hipStream_t)stream, nullptr, 0, nullptr, true);
}

moe_status_t moe_expert_ffn(const moe_desc_t* desc, const void* x_perm, const int32_t* expert_off,
                            const void* W1, const void* b1, const void* W2, const void* b2,
                            void* H, void* y_perm, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_desc(desc));
  TRY(need(x_perm, "x_perm", 16));
  TRY(need(expert_off, "expert_off", 4));
  TRY(need(W1, "W1", 16));
  TRY(need(W2, "W2", 16));
  TRY(maybe(b1, "b1", 4));
  TRY(maybe(b2, "b2", 4));
  TRY(need(H, "H", 16));
  TRY(need(y_perm, "y_perm", 16));
  // without a workspace the two GEMMs run as two launches
  const int n_counters = ws ? ffn_counters_of(desc) : 0;
  TRY(check_ws(ws, ws_bytes, align_up((size_t)n_counters * 4)));
  return do_ffn(desc, x_perm, nullptr, expert_off, W1, b1, W2, b2, H, y_perm,
                n_counters ? static_cast<int32_t*>(ws) : nullptr, false, (hipStream_t)stream);
}

moe_status_t moe_combine(const moe_desc_t* desc, const void* y_perm, const int32_t* row_of,
                         const float* topk_w, void* y, void* stream) {
  TRY(check_desc(desc));
  TRY(need(y_perm, "y_perm", 16));
  TRY(need(row_of, "row_of", 4));
  TRY(need(topk_w, "topk_w", 4));
  TRY(need(y, "y", 16));
  return do_combine(desc, y_perm, row_of, topk_w, y, (hipStream_t)stream);
}


moe_status_t moe_forward(const moe_desc_t* desc, const moe_layer_tensors_t* t, void* ws, size_t ws_bytes,
                         void* stream) {
  return forward_impl(desc, t, nullptr, ws, ws_bytes, stream);
}

moe_status_t moe_forward_noalloc(const moe_desc_t* desc, const moe_layer_tensors_t* t, void* stream) {
  TRY(check_desc(desc));
  const size_t need_bytes = forward_ws(desc).bytes;
  if (need_bytes > kNoAllocScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_forward_noalloc: the layer needs %zu bytes of workspace, above the %zu-byte scratch array; "
                "call moe_forward with a workspace instead",
                need_bytes, kNoAllocScratchBytes);
  void* ws = nullptr;
  TRY(scratch_on_current_device(&ws));
  return forward_impl(desc, t, nullptr, ws, kNoAllocScratchBytes, stream);
}

size_t moe_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

moe_status_t moe_forward_fp8(const moe_desc_t* desc, const moe_layer_tensors_t* t, const moe_fp8_weights_t* w8,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!w8) return fail(MOE_ERR_INVALID, "w8 is NULL");
  return forward_impl(desc, t, w8, ws, ws_bytes, stream);
}

moe_status_t moe_quantize_fp8(const void* W, int32_t dtype, int32_t groups, int32_t K, int32_t Ncols,
                              uint8_t* codes, float* scales, void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return fail(MOE_ERR_INVALID, "dtype %d is not MOE_F32 or MOE_BF16", dtype);
  if (groups < 1 || groups > 65535 || K < 128 || Ncols < 128 || K % 128 || Ncols % 128)
    return fail(MOE_ERR_INVALID, "quantise [%d, %d, %d]: groups in [1, 65535], K and Ncols positive multiples of 128",
                groups, K, Ncols);
  if ((int64_t)K * Ncols > ((int64_t)1 << 31) - 1)
    return fail(MOE_ERR_INVALID, "K * Ncols = %lld exceeds 2^31 - 1", (long long)K * Ncols);
  TRY(need(W, "W", 16));
  TRY(need(codes, "codes", 16));
  TRY(need(scales, "scales", 4));
  return hip_status(moe::launch_quantize_fp8(W, dtype == MOE_BF16, groups, K, Ncols, codes, scales,
                                             (hipStream_t)stream),
                    "fp8 quantisation");
}

moe_status_t moe_expert_ffn_fp8(const moe_desc_t* desc, const void* x_perm, const int32_t* expert_off,
                                const uint8_t* W1q, const float* S1, const void* b1, const uint8_t* W2q,
                                const float* S2, const void* b2, void* H, void* y_perm, void* stream) {
  TRY(check_desc(desc));
  TRY(check_fp8_layer(desc));
  TRY(need(x_perm, "x_perm", 16));
  TRY(need(expert_off, "expert_off", 4));
  TRY(need(W1q, "W1q", 16));
  TRY(need(S1, "S1", 4));
  TRY(need(W2q, "W2q", 16));
  TRY(need(S2, "S2", 4));
  TRY(maybe(b1, "b1", 4));
  TRY(maybe(b2, "b2", 4));
  TRY(need(H, "H", 16));
  TRY(need(y_perm, "y_perm", 16));
  return do_ffn_w8(desc, x_perm, nullptr, expert_off, W1q, S1, b1, W2q, S2, b2, H, y_perm, (hipStream_t)stream);
}

moe_status_t moe_aux_loss(const moe_desc_t* desc, const int32_t* topk_idx, const float* topk_w,
                          float* importance, float* losses, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_desc(desc));
  TRY(need(topk_idx, "topk_idx", 4));
  TRY(need(topk_w, "topk_w", 4));
  TRY(maybe(importance, "importance", 4));
  TRY(maybe(losses, "losses", 4));
  const size_t need_bytes = align_up((size_t)moe::aux_blocks(desc->T) * desc->N * 4);
  TRY(check_ws(ws, ws_bytes, need_bytes));
  if (!importance && !losses) return MOE_OK;
  moe::AuxParams p{};
  p.topk_idx = topk_idx;
  p.topk_w = topk_w;
  p.partial = static_cast<float*>(ws);
  p.importance = importance;
  p.losses = losses;
  p.T = (int)desc->T;
  p.N = desc->N;
  p.k = desc->k;
  return hip_status(moe::launch_aux_loss(p, (hipStream_t)stream), "load-balance terms");
}

moe_status_t moe_backward(const moe_desc_t* desc, const moe_backward_tensors_t* t, const float* aux_coef, void* ws,
                          size_t ws_bytes, void* stream) {
  TRY(check_backward(desc));
  if (!t) return fail(MOE_ERR_INVALID, "tensors is NULL");
  const bool noisy = desc->gate == MOE_GATE_NOISY;
  TRY(need(t->x, "x", 16));
  TRY(need(t->w_gate, "w_gate", 16));
  if (noisy) {
    TRY(need(t->w_noise, "w_noise", 16));
    TRY(need(t->noise, "noise", 4));
    TRY(need(t->dw_noise, "dw_noise", 16));
  }
  TRY(need(t->W1, "W1", 16));
  TRY(need(t->W2, "W2", 16));
  TRY(maybe(t->b1, "b1", 8));
  TRY(maybe(t->b2, "b2", 8));
  if (!desc->renorm) TRY(need(t->logits, "logits", 4));
  TRY(need(t->topk_idx, "topk_idx", 4));
  TRY(need(t->topk_w, "topk_w", 4));
  TRY(need(t->expert_off, "expert_off", 4));
  TRY(need(t->row_of, "row_of", 4));
  TRY(need(t->token_of_row, "token_of_row", 4));
  TRY(need(t->dy, "dy", 16));
  TRY(need(t->dx, "dx", 16));
  TRY(need(t->dW1, "dW1", 16));
  TRY(need(t->dW2, "dW2", 16));
  TRY(maybe(t->db1, "db1", 4));
  TRY(maybe(t->db2, "db2", 4));
  TRY(need(t->dw_gate, "dw_gate", 16));
  TRY(maybe(t->dlogit_bias, "dlogit_bias", 4));
  const BackwardWs bw = backward_ws(desc);
  TRY(check_ws(ws, ws_bytes, bw.bytes));
  const bool aux = aux_coef && (aux_coef[0] != 0.f || aux_coef[1] != 0.f);
  hipStream_t s = (hipStream_t)stream;
  const int T = (int)desc->T, d = desc->d, h = desc->h, N = desc->N, k = desc->k;
  const int R = (int)rows_bound_of(desc);
  using moe::bf16;
  bf16* x_perm = at<bf16>(ws, bw.x_perm);
  bf16* dY = at<bf16>(ws, bw.dY);
  bf16* U = at<bf16>(ws, bw.U);
  bf16* H = at<bf16>(ws, bw.H);
  bf16* dU = at<bf16>(ws, bw.dU);
  float* pd = at<float>(ws, bw.pd);
  float* dx_perm = at<float>(ws, bw.dx_perm);
  float* dl = at<float>(ws, bw.dl);
  float* dz = at<float>(ws, bw.dz);
  // the rows of x in expert order, and the rows bf16(w dy_t)
  moe::DispatchParams dp{};
  dp.x = t->x;
  dp.row_of = const_cast<int32_t*>(t->row_of);  // read only by the permute
  dp.x_perm = x_perm;
  dp.T = T;
  dp.d = d;
  dp.k = k;
  dp.elem_bytes = 2;
  TRY(hip_status(moe::launch_permute(dp, s), "backward: x rows"));
  TRY(hip_status(moe::launch_scale_rows(static_cast<const bf16*>(t->dy), t->row_of, t->topk_w, dY, T, d, k, s),
                 "backward: dY rows"));
  // U and H (recomputed), then dU and the partial dots G . H
  {
    // U and H on the forward's GEMM1 tiles (same K order and GELU, so H
    // repeats the forward's bits), storing the pre-activation as well
    moe::GemmParams g1, g2;
    ffn_gemms(desc, t->x, t->token_of_row, t->expert_off, t->W1, t->b1, t->W2, t->b2, H, nullptr, &g1, &g2);
    g1.C2 = U;
    const int avg_rows = (int)((desc->T * desc->k) / desc->N);
    TRY(hip_status(moe::launch_grouped_gemm_dual(g1, avg_rows, s), "backward: U, H"));
  }
  // G = dy_perm W2_e^T (dy rows gathered as the x rows are; K = d)
  moe::BwdGemmParams gg{};
  gg.A = t->dy;
  gg.gather = t->token_of_row;
  gg.gather_div = k;
  gg.lda = d;
  gg.a_bytes = (int64_t)T * d * 2;
  gg.B = t->W2;
  gg.ldb = d;
  gg.strideB = (int64_t)h * d;
  gg.b_bytes = (int64_t)d * h * 2;
  gg.C = dU;
  gg.ldc = h;
  gg.seg = t->expert_off;
  gg.M = R;
  gg.N = h;
  gg.K = d;
  gg.groups = N;
  gg.U = U;
  gg.H = H;
  gg.row_w = t->topk_w;
  gg.tor = t->token_of_row;
  gg.pd = pd;
  TRY(hip_status(moe::launch_bwd_gemm(gg, moe::BwdGemmKind::kGeluGrad, s), "backward: dU"));
  // dx_perm = dU W1_e^T
  moe::BwdGemmParams gx{};
  gx.A = dU;
  gx.lda = h;
  gx.a_bytes = (int64_t)R * h * 2;
  gx.B = t->W1;
  gx.ldb = h;
  gx.strideB = (int64_t)d * h;
  gx.b_bytes = (int64_t)d * h * 2;
  gx.C = dx_perm;
  gx.ldc = d;
  gx.seg = t->expert_off;
  gx.M = R;
  gx.N = d;
  gx.K = h;
  gx.groups = N;
  TRY(hip_status(moe::launch_bwd_gemm(gx, moe::BwdGemmKind::kDataGrad, s), "backward: dx rows"));
  // dW2_e = H_e^T dY_e, dW1_e = x_e^T dU_e over each expert's rows
  moe::BwdGemmParams gw{};
  gw.A = H;
  gw.lda = h;
  gw.a_bytes = (int64_t)R * h * 2;
  gw.B = dY;
  gw.ldb = d;
  gw.b_bytes = (int64_t)R * d * 2;
  gw.C = t->dW2;
  gw.ldc = d;
  gw.strideC = (int64_t)h * d;
  gw.seg = t->expert_off;
  gw.a_rows = R;
  gw.M = h;
  gw.N = d;
  gw.groups = N;
  TRY(hip_status(moe::launch_bwd_gemm(gw, moe::BwdGemmKind::kWeightGrad, s), "backward: dW2"));
  gw.A = x_perm;
  gw.lda = d;
  gw.a_bytes = (int64_t)R * d * 2;
  gw.B = dU;
  gw.ldb = h;
  gw.b_bytes = (int64_t)R * h * 2;
  gw.C = t->dW1;
  gw.ldc = h;
  gw.strideC = (int64_t)d * h;
  gw.M = d;
  gw.N = h;
  TRY(hip_status(moe::launch_bwd_gemm(gw, moe::BwdGemmKind::kWeightGrad, s), "backward: dW1"));
  // the load-balance losses' gradient per expert
  float* dimp = nullptr;
  if (aux) {
    moe::AuxParams ap{};
    ap.topk_idx = t->topk_idx;
    ap.topk_w = t->topk_w;
    ap.partial = at<float>(ws, bw.imp_part);
    ap.importance = at<float>(ws, bw.imp);
    ap.T = T;
    ap.N = N;
    ap.k = k;
    TRY(hip_status(moe::launch_aux_loss(ap, s), "backward: importance"));
    dimp = at<float>(ws, bw.dimp);
    TRY(hip_status(moe::launch_importance_grad(ap.importance, dimp, N, aux_coef[0], aux_coef[1], s),
                   "backward: importance gradient"));
  }
  // per token: gate-weight gradients, softmax (and softplus) backward, dx
  moe::BwdTokenParams tp{};
  tp.pd = pd;
  tp.ntc = (h + 127) / 128;
  tp.topk_idx = t->topk_idx;
  tp.topk_w = t->topk_w;
  tp.row_of = t->row_of;
  tp.logits = t->logits;
  tp.dimp = dimp;
  tp.dy = static_cast<const bf16*>(t->dy);
  tp.b2 = static_cast<const bf16*>(t->b2);
  tp.x = static_cast<const bf16*>(t->x);
  tp.w_gate = static_cast<const bf16*>(t->w_gate);
  tp.w_noise = noisy ? static_cast<const bf16*>(t->w_noise) : nullptr;
  tp.noise = t->noise;
  tp.dx_perm = dx_perm;
  tp.dl = dl;
  tp.dz = dz;
  tp.dx = static_cast<bf16*>(t->dx);
  tp.T = T;
  tp.d = d;
  tp.N = N;
  tp.k = k;
  tp.renorm = desc->renorm;
  TRY(hip_status(moe::launch_bwd_token(tp, s), "backward: tokens"));
  // the gate's weights and logit bias
  float* part = at<float>(ws, bw.gpart);
  TRY(hip_status(moe::launch_gate_grad(tp.x, dl, noisy ? dz : nullptr, part, t->dw_gate, noisy ? t->dw_noise : nullptr,
                                       T, d, N, s),
                 "backward: dw_gate, dw_noise"));
  if (t->dlogit_bias)
    TRY(hip_status(moe::launch_column_sum(dl, part, t->dlogit_bias, T, N, s), "backward: dlogit_bias"));
  // the expert biases
  if (t->db1) TRY(hip_status(moe::launch_colsum_bf16(dU, t->expert_off, t->db1, h, N, R, s), "backward: db1"));
  if (t->db2) TRY(hip_status(moe::launch_colsum_bf16(dY, t->expert_off, t->db2, d, N, R, s), "backward: db2"));
  return MOE_OK;
}

moe_status_t moe_ffn_status(const moe_desc_t* desc, moe_ws_kind_t kind, const void* ws, size_t ws_bytes,
                            int32_t* status, void* stream) {
  TRY(check_desc(desc));
  TRY(need(status, "status", 4));
  const int32_t* counters = nullptr;
  if (kind == MOE_WS_FORWARD) {
    const ForwardWs fw = forward_ws(desc);
    TRY(check_ws(const_cast<void*>(ws), ws_bytes, fw.bytes));
    if (fw.n_counters) counters = reinterpret_cast<const int32_t*>(static_cast<const char*>(ws) + fw.ffn_counters);
  } else if (kind == MOE_WS_FFN) {
    const int n = ffn_counters_of(desc);
    TRY(check_ws(const_cast<void*>(ws), ws_bytes, align_up((size_t)n * 4)));
    if (n) counters = static_cast<const int32_t*>(ws);
  } else {
    return fail(MOE_ERR_INVALID, "moe_ffn_status: kind must be MOE_WS_FORWARD or MOE_WS_FFN");
  }
  return hip_status(moe::launch_ffn_status(counters, status, (hipStream_t)stream), "FFN status");
}

moe_status_t moe_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 16 || bytes % 16) return fail(MOE_ERR_INVALID, "moe_probe_copy: bytes must be a positive multiple of 16");
  TRY(need(src, "src", 16));
  TRY(need(dst, "dst", 16));
  return hip_status(moe::launch_probe_copy(src, dst, bytes, (hipStream_t)stream), "probe copy");
}

moe_status_t moe_probe_mfma(int32_t iters, float* sink, int64_t* flops, void* stream) {
  if (iters < 1) return fail(MOE_ERR_INVALID, "moe_probe_mfma: iters must be >= 1");
  TRY(need(sink, "sink", 4));
  if (!flops) return fail(MOE_ERR_INVALID, "flops is NULL");
  *flops = moe::probe_mfma_flops_per_iter() * iters;
  return hip_status(moe::launch_probe_mfma(iters, sink, (hipStream_t)stream), "probe mfma");
}

int64_t moe_probe_mfma_sink_floats(void) { return (int64_t)moe::probe_mfma_blocks() * 8; }

moe_status_t moe_time_ffn_launches(void* start_event, void* stop_event) {
  g_ffn_events.start = static_cast<hipEvent_t>(start_event);
  g_ffn_events.stop = static_cast<hipEvent_t>(stop_event);
  return MOE_OK;
}

size_t moe_ffn_trace_bytes(void) { return moe::ffn_trace_bytes(); }

moe_status_t moe_ffn_trace_read(void* host) {
  if (!host) return fail(MOE_ERR_INVALID, "moe_ffn_trace_read: host is NULL");
  if (moe::ffn_trace_bytes() == 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_ffn_trace_read: this build records no trace (MOE_FFN_TRACE)");
  return hip_status(moe::ffn_trace_copy(host), "moe_ffn_trace_read");
}

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error; }

const char* moe_version(void) { return "moe gfx950 " __DATE__; }

}  // extern "C"
