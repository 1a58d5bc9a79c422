// C ABI of the library: argument validation on the host, then the launchers.
// Nothing here allocates, frees or synchronises (except under
// NVFP4MOE_SYNC_CHECK=1, a debugging aid).
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/nvfp4moe.h"
#include "launch.hpp"

static_assert(NVFP4_NOALLOC_SCRATCH_BYTES == nvfp4::kNoAllocScratchFloats * sizeof(float),
              "the header's scratch limit must match the scratch array");

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool sync_check_enabled() {
  static const bool on = [] {
    const char* v = getenv("NVFP4MOE_SYNC_CHECK");
    return v && v[0] == '1';
  }();
  return on;
}

int32_t finish(const char* who, hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return fail(NVFP4_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  if (sync_check_enabled()) {
    e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(NVFP4_EHIP, "%s: kernel failed: %s", who, hipGetErrorString(e));
  }
  g_last_error.clear();
  return NVFP4_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int elem_size(int32_t dtype) {
  return dtype == NVFP4_DTYPE_F32 ? 4 : (dtype == NVFP4_DTYPE_BF16 ? 2 : 0);
}

}  // namespace

extern "C" {

const char* nvfp4_last_error(void) { return g_last_error.c_str(); }

int32_t nvfp4_version(void) { return 100; }

int32_t nvfp4_quantize(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                       const float* gs, uint8_t* codes, uint8_t* scales, uint16_t* dq, void* stream) {
  const int es = elem_size(x_dtype);
  if (!es) return fail(NVFP4_EINVAL, "nvfp4_quantize: unknown dtype %d", x_dtype);
  if (rows < 0 || cols < 0) return fail(NVFP4_ESHAPE, "nvfp4_quantize: negative size");
  if (cols % 16) return fail(NVFP4_ESHAPE, "nvfp4_quantize: cols=%lld is not a multiple of 16", (long long)cols);
  if (ld_x < cols) return fail(NVFP4_ESHAPE, "nvfp4_quantize: ld_x < cols");
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!x || !gs || !codes || !scales) return fail(NVFP4_EINVAL, "nvfp4_quantize: null pointer");
  if (!aligned(x, 16) || (ld_x * es) % 16 || !aligned(codes, 8) || !aligned(gs, 4) || !aligned(dq, 16))
    return fail(NVFP4_EALIGN, "nvfp4_quantize: x, its row pitch and dq must be 16-byte aligned, codes 8-byte");
  hipStream_t s = (hipStream_t)stream;
  return finish("nvfp4_quantize",
                nvfp4::launch_quantize(x, x_dtype == NVFP4_DTYPE_BF16, rows, cols, ld_x, gs, codes, scales, dq, s),
                s);
}

size_t nvfp4_global_scale_workspace_size(int64_t batch, int64_t n) {
  if (batch <= 0 || n < 0) return 0;
  return (size_t)batch * (size_t)nvfp4::amax_chunks(n) * sizeof(float);
}

int32_t nvfp4_global_scale(const void* x, int32_t x_dtype, int64_t batch, int64_t n, int64_t stride,
                           float* gs_out, void* ws, size_t ws_bytes, void* stream) {
  const int es = elem_size(x_dtype);
  if (!es) return fail(NVFP4_EINVAL, "nvfp4_global_scale: unknown dtype %d", x_dtype);
  if (batch < 0 || n < 0) return fail(NVFP4_ESHAPE, "nvfp4_global_scale: negative size");
  if (batch > 65535) return fail(NVFP4_ESHAPE, "nvfp4_global_scale: batch > 65535");
  if (n % 8) return fail(NVFP4_ESHAPE, "nvfp4_global_scale: n must be a multiple of 8");
  if (stride < n) return fail(NVFP4_ESHAPE, "nvfp4_global_scale: stride < n");
  if (batch == 0) return NVFP4_OK;
  if (!x || !gs_out || !ws) return fail(NVFP4_EINVAL, "nvfp4_global_scale: null pointer");
  if (ws_bytes < nvfp4_global_scale_workspace_size(batch, n))
    return fail(NVFP4_ESHAPE, "nvfp4_global_scale: workspace too small");
  if (!aligned(x, 16) || (stride * es) % 16 || !aligned(ws, 16) || !aligned(gs_out, 4))
    return fail(NVFP4_EALIGN, "nvfp4_global_scale: x, its pitch and ws must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  return finish("nvfp4_global_scale",
                nvfp4::launch_global_scale(x, x_dtype == NVFP4_DTYPE_BF16, batch, n, stride, gs_out,
                                           (float*)ws, s),
                s);
}

int32_t nvfp4_global_scale_noalloc(const void* x, int32_t x_dtype, int64_t batch, int64_t n, int64_t stride,
                                   float* gs_out, void* stream) {
  const char* who = "nvfp4_global_scale_noalloc";
  const int es = elem_size(x_dtype);
  if (!es) return fail(NVFP4_EINVAL, "%s: unknown dtype %d", who, x_dtype);
  if (batch < 0 || n < 0) return fail(NVFP4_ESHAPE, "%s: negative size", who);
  if (batch > 65535) return fail(NVFP4_ESHAPE, "%s: batch > 65535", who);
  if (n % 8) return fail(NVFP4_ESHAPE, "%s: n must be a multiple of 8", who);
  if (stride < n) return fail(NVFP4_ESHAPE, "%s: stride < n", who);
  if (batch == 0) return NVFP4_OK;
  const size_t need = nvfp4_global_scale_workspace_size(batch, n);
  if (need > (size_t)NVFP4_NOALLOC_SCRATCH_BYTES)
    return fail(NVFP4_ESHAPE, "%s: batch=%lld slices of n=%lld need %zu bytes of scratch, above the %d-byte limit",
                who, (long long)batch, (long long)n, need, NVFP4_NOALLOC_SCRATCH_BYTES);
  if (!x || !gs_out) return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(x, 16) || (stride * es) % 16 || !aligned(gs_out, 4))
    return fail(NVFP4_EALIGN, "%s: x and its pitch must be 16-byte aligned", who);
  float* ws = nullptr;
  const hipError_t e = nvfp4::noalloc_scratch(&ws);
  if (e != hipSuccess) return fail(NVFP4_EHIP, "%s: scratch lookup failed: %s", who, hipGetErrorString(e));
  hipStream_t s = (hipStream_t)stream;
  return finish(who, nvfp4::launch_global_scale(x, x_dtype == NVFP4_DTYPE_BF16, batch, n, stride, gs_out, ws, s),
                s);
}

static int32_t route_permute(const char* who, const float* logits, int64_t T, int32_t E, int32_t k,
                             int32_t ns, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                             int32_t* sorted_token_ids, int32_t* inv_perm, void* stream) {
  if (T < 0) return fail(NVFP4_ESHAPE, "%s: T < 0", who);
  if (E < 1 || E > NVFP4_MAX_EXPERTS) return fail(NVFP4_ESHAPE, "%s: E=%d outside [1, %d]", who, E, NVFP4_MAX_EXPERTS);
  if (k < 1 || k > E || k > NVFP4_MAX_TOPK)
    return fail(NVFP4_ESHAPE, "%s: k=%d outside [1, min(E, %d)]", who, k, NVFP4_MAX_TOPK);
  if (ns < 0 || k + ns > NVFP4_MAX_TOPK || E + ns > NVFP4_MAX_EXPERTS)
    return fail(NVFP4_ESHAPE, "%s: n_shared=%d: need n_shared >= 0, k + n_shared <= %d and E + n_shared <= %d", who,
                ns, NVFP4_MAX_TOPK, NVFP4_MAX_EXPERTS);
  if (T * (int64_t)(k + ns) >= ((int64_t)1 << 31)) return fail(NVFP4_ESHAPE, "%s: T*(k+n_shared) >= 2^31", who);
  if (!expert_offsets) return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_token_ids || !inv_perm))
    return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_offsets, 4) ||
      !aligned(sorted_token_ids, 4) || !aligned(inv_perm, 4))
    return fail(NVFP4_EALIGN, "%s: arrays must be 4-byte aligned", who);
  hipStream_t s = (hipStream_t)stream;
  return finish(who,
                nvfp4::launch_route_permute(logits, T, E, k, ns, topk_ids, topk_w, expert_offsets,
                                            sorted_token_ids, inv_perm, s),
                s);
}

int32_t moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids,
                          float* topk_w, int32_t* expert_offsets, int32_t* sorted_token_ids,
                          int32_t* inv_perm, void* stream) {
  return route_permute("moe_route_permute", logits, T, E, k, 0, topk_ids, topk_w, expert_offsets,
                       sorted_token_ids, inv_perm, stream);
}

int32_t moe_route_permute_shared(const float* logits, int64_t T, int32_t E, int32_t k, int32_t n_shared,
                                 int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                 int32_t* sorted_token_ids, int32_t* inv_perm, void* stream) {
  return route_permute("moe_route_permute_shared", logits, T, E, k, n_shared, topk_ids, topk_w, expert_offsets,
                       sorted_token_ids, inv_perm, stream);
}

int32_t nvfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                           int64_t a_rows, const int32_t* a_row_index, const uint16_t* a_dq,
                           const uint8_t* w_codes,
                           const uint8_t* w_scales, int32_t w_layout, const float* w_gs, const int32_t* n_seg,
                           int32_t n_segs, const int32_t* group_offsets, int32_t G, int64_t M, int64_t N,
                           int64_t K, void* out, int32_t out_dtype, int64_t ld_out, void* workspace,
                           size_t ws_bytes, void* stream) {
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return fail(NVFP4_EINVAL, "nvfp4_grouped_gemm: unknown out dtype %d", out_dtype);
  if (w_layout != NVFP4_LAYOUT_ROWS && w_layout != NVFP4_LAYOUT_TILED)
    return fail(NVFP4_EINVAL, "nvfp4_grouped_gemm: unknown weight layout %d", w_layout);
  const bool tiled = w_layout == NVFP4_LAYOUT_TILED;
  if (G < 1 || G > NVFP4_MAX_EXPERTS) return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: G=%d", G);
  if (n_segs < 1 || n_segs > NVFP4_MAX_SEGMENTS)
    return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: n_segs=%d outside [1, %d]", n_segs, NVFP4_MAX_SEGMENTS);
  if (M < 0 || N < 1 || K < 32 || K % 32)
    return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: need M >= 0, N >= 1, K >= 32 and K %% 32 == 0");
  if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
    return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: M and N must be below 2^31");
  if (tiled && (K % 256 || K > nvfp4::kMaxTiledK))
    return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: the tiled layout needs K %% 256 == 0 and K <= 2^24");
  if (ld_out < N) return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: ld_out < N");
  if (a_rows < 0 || (!a_row_index && a_rows < M) || (M > 0 && a_rows < 1))
    return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: a_rows too small");
  if (!n_seg) return fail(NVFP4_EINVAL, "nvfp4_grouped_gemm: null n_seg");
  if (n_seg[0] != 0 || n_seg[n_segs] != N)
    return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: n_seg must run from 0 to N");
  for (int i = 0; i < n_segs; ++i)
    if (n_seg[i + 1] <= n_seg[i]) return fail(NVFP4_ESHAPE, "nvfp4_grouped_gemm: n_seg must increase");
  if (M == 0) return NVFP4_OK;
  if (!a_codes || !a_scales || !a_gs || !w_codes || (!tiled && !w_scales) || !w_gs || !group_offsets || !out)
    return fail(NVFP4_EINVAL, "nvfp4_grouped_gemm: null pointer");
  if (!aligned(a_codes, 16) || !aligned(w_codes, 16) || !aligned(a_scales, 4) || !aligned(w_scales, 4) ||
      !aligned(out, 16) || !aligned(a_gs, 4) || !aligned(w_gs, 4) || !aligned(group_offsets, 4) ||
      !aligned(a_row_index, 4) || !aligned(a_dq, 16))
    return fail(NVFP4_EALIGN, "nvfp4_grouped_gemm: codes, a_dq and out must be 16-byte aligned, scales 4-byte");
  nvfp4::GemmArgs a{};
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.a_gs = a_gs;
  a.a_rows = a_row_index ? a_rows : M;
  a.a_row_index = a_row_index;
  // the direct-to-LDS loads address A with 32-bit byte offsets
  a.a_dq = a_dq && (uint64_t)a.a_rows * (uint64_t)K * 2u < ((uint64_t)1 << 32) ? a_dq : nullptr;
  a.w_codes = w_codes;
  a.w_scales = tiled ? nullptr : w_scales;
  a.w_tiled = tiled ? 1 : 0;
  a.w_gs = w_gs;
  for (int i = 0; i < 5; ++i) a.n_seg[i] = i <= n_segs ? n_seg[i] : (int32_t)N;
  a.n_segs = n_segs;
  a.group_offsets = group_offsets;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.out = out;
  a.out_bf16 = out_dtype == NVFP4_DTYPE_BF16;
  a.ld_out = ld_out;
  // split-K only with a large enough, aligned workspace (else one pass)
  const size_t need = nvfp4::gemm_splitk_bytes(G, M, N, K, tiled);
  if (need && workspace && ws_bytes >= need && aligned(workspace, 16)) {
    a.splits = nvfp4::gemm_splitk_splits(G, M, N, K, tiled);
    a.ws = (float*)workspace;
  }
  hipStream_t s = (hipStream_t)stream;
  return finish("nvfp4_grouped_gemm", nvfp4::launch_grouped_gemm(a, s), s);
}

size_t nvfp4_grouped_gemm_workspace_size(int32_t G, int64_t M, int64_t N, int64_t K, int32_t w_layout) {
  if (G < 1 || M < 1 || N < 1 || K < 32) return 0;
  return nvfp4::gemm_splitk_bytes(G, M, N, K, w_layout == NVFP4_LAYOUT_TILED);
}

// The checks and GemmArgs shared by the two fused first-GEMM calls (h
// re-quantised, or h in float32): sizes, the A and W operands, group offsets.
// Returns NVFP4_OK with *a filled, or the error (set as the last error).
static int32_t fused_gemm_args(const char* who, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                               int64_t a_rows, const int32_t* a_row_index, const uint16_t* a_dq,
                               const uint8_t* w_tiled, const float* w_gs, const int32_t* group_offsets, int32_t G,
                               int64_t M, int64_t I, int64_t K, nvfp4::GemmArgs* a) {
  if (G < 1 || G > NVFP4_MAX_EXPERTS) return fail(NVFP4_ESHAPE, "%s: G=%d", who, G);
  if (M < 0 || I < 32 || I % 32 || K < 256 || K % 256 || K > nvfp4::kMaxTiledK)
    return fail(NVFP4_ESHAPE, "%s: need M >= 0, I >= 32 with I %% 32 == 0, 256 <= K <= 2^24 with K %% 256 == 0",
                who);
  if (M >= ((int64_t)1 << 31) || 2 * I >= ((int64_t)1 << 31))
    return fail(NVFP4_ESHAPE, "%s: M and 2 I must be below 2^31", who);
  if (a_rows < 0 || (!a_row_index && a_rows < M) || (M > 0 && a_rows < 1))
    return fail(NVFP4_ESHAPE, "%s: a_rows too small", who);
  if (M > 0 && (!a_codes || !a_scales || !a_gs || !w_tiled || !w_gs || !group_offsets))
    return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(a_codes, 16) || !aligned(w_tiled, 16) || !aligned(a_scales, 4) || !aligned(a_gs, 4) ||
      !aligned(w_gs, 4) || !aligned(group_offsets, 4) || !aligned(a_row_index, 4) || !aligned(a_dq, 16))
    return fail(NVFP4_EALIGN, "%s: codes, tiled weights and a_dq must be 16-byte aligned, the rest 4-byte", who);
  *a = nvfp4::GemmArgs{};
  a->a_codes = a_codes;
  a->a_scales = a_scales;
  a->a_gs = a_gs;
  a->a_rows = a_row_index ? a_rows : M;
  a->a_row_index = a_row_index;
  a->a_dq = a_dq && (uint64_t)a->a_rows * (uint64_t)K * 2u < ((uint64_t)1 << 32) ? a_dq : nullptr;
  a->w_codes = w_tiled;
  a->w_scales = nullptr;
  a->w_tiled = 1;
  a->w_gs = w_gs;
  a->n_seg[0] = 0;
  a->n_seg[1] = (int32_t)I;
  for (int i = 2; i < 5; ++i) a->n_seg[i] = (int32_t)(2 * I);
  a->n_segs = 2;
  a->group_offsets = group_offsets;
  a->G = G;
  a->M = M;
  a->N = 2 * I;
  a->K = K;
  a->out = nullptr;
  a->out_bf16 = 0;
  a->ld_out = 2 * I;
  a->fuse = 1;
  return NVFP4_OK;
}

int32_t nvfp4_grouped_gemm_silu_requant(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                        int64_t a_rows, const int32_t* a_row_index, const uint16_t* a_dq,
                                        const uint8_t* w_tiled, const float* w_gs, const int32_t* group_offsets,
                                        int32_t G, int64_t M, int64_t I, int64_t K, const float* h_gs,
                                        uint8_t* h_codes, uint8_t* h_scales, uint16_t* h_dq, void* workspace,
                                        size_t ws_bytes, void* stream) {
  const char* who = "nvfp4_grouped_gemm_silu_requant";
  nvfp4::GemmArgs a;
  const int32_t rc = fused_gemm_args(who, a_codes, a_scales, a_gs, a_rows, a_row_index, a_dq, w_tiled, w_gs,
                                     group_offsets, G, M, I, K, &a);
  if (rc != NVFP4_OK) return rc;
  if (M == 0) return NVFP4_OK;
  if (!h_gs || !h_codes || !h_scales) return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(h_gs, 4) || !aligned(h_codes, 16) || !aligned(h_dq, 16))
    return fail(NVFP4_EALIGN, "%s: h_codes and h_dq must be 16-byte aligned, h_gs 4-byte", who);
  a.h_gs = h_gs;
  a.h_codes = h_codes;
  a.h_scales = h_scales;
  a.h_dq = h_dq;
  // split-K as nvfp4_grouped_gemm of the stacked gate_up would (same ranges,
  // same summation order), then SiLU-requant of the reduced sums
  const size_t need = nvfp4::gemm_splitk_bytes(G, M, 2 * I, K, true);
  if (need && workspace && ws_bytes >= need && aligned(workspace, 16)) {
    a.splits = nvfp4::gemm_splitk_splits(G, M, 2 * I, K, true);
    a.ws = (float*)workspace;
  }
  hipStream_t s = (hipStream_t)stream;
  return finish(who, nvfp4::launch_grouped_gemm(a, s), s);
}

size_t nvfp4_grouped_gemm_silu_f32_partials(int32_t G, int64_t M, int64_t I) {
  if (G < 1 || M < 1 || I < 32) return 0;
  return (size_t)nvfp4::gemm_silu_f32_amax_slots(G, M, I);
}

int32_t nvfp4_grouped_gemm_silu_f32(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                    int64_t a_rows, const int32_t* a_row_index, const uint16_t* a_dq,
                                    const uint8_t* w_tiled, const float* w_gs, const int32_t* group_offsets,
                                    int32_t G, int64_t M, int64_t I, int64_t K, float* h, float* amax_partials,
                                    int64_t n_partials, void* stream) {
  const char* who = "nvfp4_grouped_gemm_silu_f32";
  nvfp4::GemmArgs a;
  const int32_t rc = fused_gemm_args(who, a_codes, a_scales, a_gs, a_rows, a_row_index, a_dq, w_tiled, w_gs,
                                     group_offsets, G, M, I, K, &a);
  if (rc != NVFP4_OK) return rc;
  if (M == 0) return NVFP4_OK;
  if (!h || !amax_partials) return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(h, 16) || !aligned(amax_partials, 4))
    return fail(NVFP4_EALIGN, "%s: h must be 16-byte aligned, amax_partials 4-byte", who);
  if (n_partials < nvfp4::gemm_silu_f32_amax_slots(G, M, I))
    return fail(NVFP4_ESHAPE, "%s: n_partials below nvfp4_grouped_gemm_silu_f32_partials", who);
  a.h_f32 = h;
  a.h_amax = amax_partials;
  a.h_amax_n = n_partials;
  hipStream_t s = (hipStream_t)stream;
  return finish(who, nvfp4::launch_grouped_gemm(a, s), s);
}

size_t nvfp4_moe_expert_mlp_workspace_size(int32_t G, int64_t R) {
  if (G < 1 || R < 1) return 0;
  return (size_t)nvfp4::moe_persistent_counters(G, R) * sizeof(int32_t);
}

static int32_t spin_limit_from_env() {
  const char* v = getenv("NVFP4MOE_SPIN_LIMIT");
  if (v && v[0]) {
    const long n = strtol(v, nullptr, 10);
    if (n >= 1 && n <= (1L << 30)) return (int32_t)n;
  }
  return 1 << 22;
}

int32_t nvfp4_moe_expert_mlp(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, int64_t x_rows,
                             const int32_t* sorted_token_ids, const int32_t* expert_offsets, int32_t G, int64_t R,
                             const uint8_t* w1_tiled, const float* w1_gs, const uint8_t* w2_tiled,
                             const float* w2_gs, int64_t H, int64_t I, const float* h_gs, uint8_t* h_codes,
                             uint8_t* h_scales, uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  const char* who = "nvfp4_moe_expert_mlp";
  if (G < 1 || G > NVFP4_MAX_EXPERTS) return fail(NVFP4_ESHAPE, "%s: G=%d", who, G);
  if (R < 0 || H < 256 || H % 256 || I < 256 || I % 256 || H > nvfp4::kMaxTiledK || I > nvfp4::kMaxTiledK)
    return fail(NVFP4_ESHAPE, "%s: need R >= 0, H and I in [256, 2^24] and multiples of 256", who);
  if (R >= ((int64_t)1 << 31) || 2 * I >= ((int64_t)1 << 31) || H >= ((int64_t)1 << 31))
    return fail(NVFP4_ESHAPE, "%s: R, 2 I and H must be below 2^31", who);
  if (x_rows < 0 || (!sorted_token_ids && x_rows < R) || (R > 0 && x_rows < 1))
    return fail(NVFP4_ESHAPE, "%s: x_rows too small", who);
  if (R == 0) return NVFP4_OK;
  if (!x_codes || !x_scales || !x_gs || !expert_offsets || !w1_tiled || !w1_gs || !w2_tiled || !w2_gs || !h_gs ||
      !h_codes || !h_scales || !y || !workspace)
    return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (ws_bytes < nvfp4_moe_expert_mlp_workspace_size(G, R))
    return fail(NVFP4_ESHAPE, "%s: workspace too small", who);
  if (!aligned(x_codes, 16) || !aligned(w1_tiled, 16) || !aligned(w2_tiled, 16) || !aligned(h_codes, 16) ||
      !aligned(y, 16) || !aligned(x_scales, 4) || !aligned(h_scales, 4) || !aligned(x_gs, 4) || !aligned(h_gs, 4) ||
      !aligned(w1_gs, 4) || !aligned(w2_gs, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_token_ids, 4) ||
      !aligned(workspace, 4))
    return fail(NVFP4_EALIGN, "%s: codes, tiled weights and y must be 16-byte aligned, the rest 4-byte", who);
  nvfp4::GemmArgs l1{};
  l1.a_codes = x_codes;
  l1.a_scales = x_scales;
  l1.a_gs = x_gs;
  l1.a_rows = sorted_token_ids ? x_rows : R;
  l1.a_row_index = sorted_token_ids;
  l1.w_codes = w1_tiled;
  l1.w_tiled = 1;
  l1.w_gs = w1_gs;
  l1.n_seg[0] = 0;
  l1.n_seg[1] = (int32_t)I;
  for (int i = 2; i < 5; ++i) l1.n_seg[i] = (int32_t)(2 * I);
  l1.n_segs = 2;
  l1.group_offsets = expert_offsets;
  l1.G = G;
  l1.M = R;
  l1.N = 2 * I;
  l1.K = H;
  l1.ld_out = 2 * I;
  l1.fuse = 1;
  l1.h_gs = h_gs;
  l1.h_codes = h_codes;
  l1.h_scales = h_scales;
  nvfp4::GemmArgs l2{};
  l2.a_codes = h_codes;
  l2.a_scales = h_scales;
  l2.a_gs = h_gs;
  l2.a_rows = R;
  l2.w_codes = w2_tiled;
  l2.w_tiled = 1;
  l2.w_gs = w2_gs;
  l2.n_seg[0] = 0;
  for (int i = 1; i < 5; ++i) l2.n_seg[i] = (int32_t)H;
  l2.n_segs = 1;
  l2.group_offsets = expert_offsets;
  l2.G = G;
  l2.M = R;
  l2.N = H;
  l2.K = I;
  l2.out = y;
  l2.out_bf16 = 1;
  l2.ld_out = H;
  hipStream_t s = (hipStream_t)stream;
  int32_t* ctr = (int32_t*)workspace;
  const int32_t st = finish(who, nvfp4::launch_moe_persistent(l1, l2, ctr, spin_limit_from_env(), s), s);
  if (st == NVFP4_OK && sync_check_enabled()) {
    int32_t status = 0;
    const hipError_t e = hipMemcpy(&status, ctr + 1, sizeof(status), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(NVFP4_EHIP, "%s: status read failed: %s", who, hipGetErrorString(e));
    if (status) return fail(NVFP4_EHIP, "%s: a dependency wait timed out (results unspecified)", who);
  }
  return st;
}

int32_t nvfp4_grouped_gemm_reads_dq(int32_t G, int64_t M, int64_t K, int64_t a_rows, int32_t w_layout) {
  if (G < 1 || M < 1 || K < 256 || K % 256 || a_rows < 1) return 0;
  if ((uint64_t)a_rows * (uint64_t)K * 2u >= ((uint64_t)1 << 32)) return 0;
  const bool tiled = w_layout == NVFP4_LAYOUT_TILED;
  // the 128-row tiles of one small group split over K read it too (N is not
  // known here: a split is assumed whenever one 256-column tile would split,
  // which may report a copy that a very wide GEMM then does not read)
  const bool small = nvfp4::gemm_small_split(G, M, tiled) && nvfp4::gemm_splitk_bytes(G, M, 256, K, tiled) > 0;
  return nvfp4::gemm_uses_big_tiles(G, M, K, tiled) || small ? 1 : 0;
}

size_t nvfp4_prepared_weight_bytes(int64_t G, int64_t N, int64_t K) {
  if (G < 1 || N < 1 || K < 256 || K % 256) return 0;
  return (size_t)nvfp4::prepared_bytes(G, N, K);
}

int32_t nvfp4_prepare_weights(const uint8_t* w_codes, const uint8_t* w_scales, int64_t G, int64_t N, int64_t K,
                              uint8_t* out, void* stream) {
  if (G < 1 || N < 1 || K < 256 || K % 256 || K > nvfp4::kMaxTiledK)
    return fail(NVFP4_ESHAPE, "nvfp4_prepare_weights: need G >= 1, N >= 1, 256 <= K <= 2^24 and K %% 256 == 0");
  if (!w_codes || !w_scales || !out) return fail(NVFP4_EINVAL, "nvfp4_prepare_weights: null pointer");
  if (!aligned(w_codes, 16) || !aligned(w_scales, 16) || !aligned(out, 16))
    return fail(NVFP4_EALIGN, "nvfp4_prepare_weights: buffers must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  return finish("nvfp4_prepare_weights", nvfp4::launch_prepare(w_codes, w_scales, G, N, K, out, s), s);
}

int32_t silu_mul_requant(const void* gate_up, int32_t in_dtype, int64_t M, int64_t I, int64_t ld,
                         const float* gs_h, uint8_t* h_codes, uint8_t* h_scales, uint16_t* h_dq, void* stream) {
  const int es = elem_size(in_dtype);
  if (!es) return fail(NVFP4_EINVAL, "silu_mul_requant: unknown dtype %d", in_dtype);
  if (M < 0 || I < 0) return fail(NVFP4_ESHAPE, "silu_mul_requant: negative size");
  if (I % 16) return fail(NVFP4_ESHAPE, "silu_mul_requant: I must be a multiple of 16");
  if (ld < 2 * I) return fail(NVFP4_ESHAPE, "silu_mul_requant: ld < 2*I");
  if (M == 0 || I == 0) return NVFP4_OK;
  if (!gate_up || !gs_h || !h_codes || !h_scales) return fail(NVFP4_EINVAL, "silu_mul_requant: null pointer");
  if (!aligned(gate_up, 16) || (ld * es) % 16 || !aligned(h_codes, 8) || !aligned(gs_h, 4) || !aligned(h_dq, 16))
    return fail(NVFP4_EALIGN, "silu_mul_requant: gate_up, its pitch and h_dq must be 16-byte aligned, codes 8-byte");
  hipStream_t s = (hipStream_t)stream;
  return finish("silu_mul_requant",
                nvfp4::launch_silu_mul_requant(gate_up, in_dtype == NVFP4_DTYPE_BF16, M, I, ld, gs_h, h_codes,
                                               h_scales, h_dq, s),
                s);
}

int32_t fp8_quantize_weight(const float* w, int64_t N, int64_t K, int64_t ld_w, uint8_t* codes, float* scales,
                            void* stream) {
  const char* who = "fp8_quantize_weight";
  if (N < 0 || K < 128 || K % 128) return fail(NVFP4_ESHAPE, "%s: need N >= 0, K >= 128 with K %% 128 == 0", who);
  if (ld_w < K) return fail(NVFP4_ESHAPE, "%s: ld_w < K", who);
  if (N == 0) return NVFP4_OK;
  if (!w || !codes || !scales) return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(w, 16) || ld_w % 4 || !aligned(codes, 4) || !aligned(scales, 4))
    return fail(NVFP4_EALIGN, "%s: w and its pitch must be 16-byte aligned, codes and scales 4-byte", who);
  hipStream_t s = (hipStream_t)stream;
  return finish(who, nvfp4::launch_fp8_quantize(w, N, K, ld_w, codes, scales, s), s);
}

int32_t fp8_weight_gemm(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint8_t* w_codes,
                        const float* w_scales, int64_t N, void* out, int32_t out_dtype, int64_t ld_out,
                        void* stream) {
  const char* who = "fp8_weight_gemm";
  if (out_dtype != NVFP4_DTYPE_F32 && out_dtype != NVFP4_DTYPE_BF16)
    return fail(NVFP4_EINVAL, "%s: unknown out dtype %d", who, out_dtype);
  if (M < 0 || N < 1 || K < 128 || K % 128)
    return fail(NVFP4_ESHAPE, "%s: need M >= 0, N >= 1, K >= 128 with K %% 128 == 0", who);
  if (ld_x < K || ld_out < N) return fail(NVFP4_ESHAPE, "%s: ld_x < K or ld_out < N", who);
  if (M == 0) return NVFP4_OK;
  if (!x || !w_codes || !w_scales || !out) return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(x, 16) || (ld_x * 2) % 16 || !aligned(w_codes, 16) || !aligned(w_scales, 4) || !aligned(out, 4))
    return fail(NVFP4_EALIGN, "%s: x, its pitch and w_codes must be 16-byte aligned", who);
  hipStream_t s = (hipStream_t)stream;
  return finish(who,
                nvfp4::launch_fp8_gemm(x, M, K, ld_x, w_codes, w_scales, N, out, out_dtype == NVFP4_DTYPE_BF16,
                                       ld_out, s),
                s);
}

size_t silu_mul_global_scale_workspace_size(int64_t M, int64_t I) {
  if (M < 0 || I < 0) return 0;
  return (size_t)nvfp4::silu_amax_chunks(M, I) * sizeof(float);
}

int32_t silu_mul_global_scale(const void* gate_up, int32_t in_dtype, int64_t M, int64_t I, int64_t ld,
                              float* gs_out, void* ws, size_t ws_bytes, void* stream) {
  const int es = elem_size(in_dtype);
  if (!es) return fail(NVFP4_EINVAL, "silu_mul_global_scale: unknown dtype %d", in_dtype);
  if (M < 0 || I < 0) return fail(NVFP4_ESHAPE, "silu_mul_global_scale: negative size");
  if (I % 16) return fail(NVFP4_ESHAPE, "silu_mul_global_scale: I must be a multiple of 16");
  if (ld < 2 * I) return fail(NVFP4_ESHAPE, "silu_mul_global_scale: ld < 2*I");
  if (!gs_out || !ws) return fail(NVFP4_EINVAL, "silu_mul_global_scale: null pointer");
  if (M > 0 && I > 0 && !gate_up) return fail(NVFP4_EINVAL, "silu_mul_global_scale: null pointer");
  if (ws_bytes < silu_mul_global_scale_workspace_size(M, I))
    return fail(NVFP4_ESHAPE, "silu_mul_global_scale: workspace too small");
  if (!aligned(gate_up, 16) || (ld * es) % 16 || !aligned(ws, 16) || !aligned(gs_out, 4))
    return fail(NVFP4_EALIGN, "silu_mul_global_scale: gate_up, its pitch and ws must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  return finish("silu_mul_global_scale",
                nvfp4::launch_silu_mul_global_scale(gate_up, in_dtype == NVFP4_DTYPE_BF16, M, I, ld, gs_out,
                                                    (float*)ws, s),
                s);
}

int32_t moe_combine(const void* y, int32_t y_dtype, const int32_t* inv_perm, const float* topk_w, int64_t T,
                    int32_t k, int64_t H, const uint16_t* residual, uint16_t* out, void* stream) {
  const int es = elem_size(y_dtype);
  if (!es) return fail(NVFP4_EINVAL, "moe_combine: unknown dtype %d", y_dtype);
  if (T < 0 || H < 0) return fail(NVFP4_ESHAPE, "moe_combine: negative size");
  if (k < 1 || k > NVFP4_MAX_TOPK) return fail(NVFP4_ESHAPE, "moe_combine: k=%d outside [1, %d]", k, NVFP4_MAX_TOPK);
  if (H % 8) return fail(NVFP4_ESHAPE, "moe_combine: H must be a multiple of 8");
  if (T == 0 || H == 0) return NVFP4_OK;
  if (!y || !inv_perm || !topk_w || !out) return fail(NVFP4_EINVAL, "moe_combine: null pointer");
  if (!aligned(y, 16) || !aligned(out, 16) || !aligned(residual, 16) || !aligned(inv_perm, 4) ||
      !aligned(topk_w, 4))
    return fail(NVFP4_EALIGN, "moe_combine: y, residual and out must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  return finish("moe_combine",
                nvfp4::launch_combine(y, y_dtype == NVFP4_DTYPE_BF16, inv_perm, topk_w, T, k, H, residual, out, s),
                s);
}

int32_t nvfp4_probe_hbm_read(const void* buf, int64_t bytes, void* sink, void* stream) {
  const char* who = "nvfp4_probe_hbm_read";
  if (bytes < 0 || bytes % 16) return fail(NVFP4_ESHAPE, "%s: bytes must be a non-negative multiple of 16", who);
  if (bytes == 0) return NVFP4_OK;
  if (!buf || !sink) return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(NVFP4_EALIGN, "%s: buf must be 16-byte aligned", who);
  hipStream_t s = (hipStream_t)stream;
  return finish(who, nvfp4::launch_read_probe(buf, bytes, sink, s), s);
}

int32_t nvfp4_probe_mfma_f16(int64_t iters, int64_t workgroups, void* sink, void* stream) {
  const char* who = "nvfp4_probe_mfma_f16";
  if (iters < 0 || workgroups < 0 || workgroups > 65535)
    return fail(NVFP4_ESHAPE, "%s: need iters >= 0 and 0 <= workgroups <= 65535", who);
  if (iters == 0 || workgroups == 0) return NVFP4_OK;
  if (!sink) return fail(NVFP4_EINVAL, "%s: null pointer", who);
  if (!aligned(sink, 4)) return fail(NVFP4_EALIGN, "%s: sink must be 4-byte aligned", who);
  hipStream_t s = (hipStream_t)stream;
  return finish(who, nvfp4::launch_mfma_probe(iters, workgroups, sink, s), s);
}

}  // extern "C"
