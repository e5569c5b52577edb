// Host side of libmoe.so: argument checks, workspace carving, launch order.
// The entry points and their contracts are declared in include/moe.h.
#include <math.h>
#include <string.h>

#include <string>

#include "../../include/moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Returns an empty string when the config is usable, else the reason.
std::string check_config(const moe_config_t* c, int* code) {
  *code = MOE_ERR_INVALID_ARG;
  if (!c) return "config is NULL";
  if (c->T < 1) return "T must be >= 1";
  if (c->n_experts < 1) return "n_experts must be >= 1";
  if (c->top_k < 1 || c->top_k > c->n_experts) return "top_k must satisfy 1 <= K <= N";
  if (c->d_model < 1 || c->d_ff < 1) return "d_model and d_ff must be >= 1";
  if (c->d_ff_shared < 0) return "d_ff_shared must be >= 0";
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return "dtype must be MOE_F32 or MOE_BF16";
  if (!isfinite(c->aux_alpha)) return "aux_alpha must be finite";
  if (c->weight_quant != MOE_WQ_NONE && c->weight_quant != MOE_WQ_INT8)
    return "weight_quant must be MOE_WQ_NONE or MOE_WQ_INT8";
  *code = MOE_ERR_UNSUPPORTED;
  if (c->weight_quant == MOE_WQ_INT8 && c->dtype != MOE_BF16)
    return "INT8 expert weights need dtype MOE_BF16";
  if (c->n_experts > 256) return "n_experts > 256 is not supported";
  if (c->top_k > 64) return "top_k > 64 is not supported";
  if (c->d_model % 64 || c->d_ff % 64 || c->d_ff_shared % 64)
    return "d_model, d_ff and d_ff_shared must be multiples of 64";
  const int64_t mmax = (int64_t)c->T * c->top_k;
  const int64_t wide = c->d_model > c->d_ff ? c->d_model : c->d_ff;
  const int64_t wide_s = c->d_ff_shared > c->d_model ? c->d_ff_shared : c->d_model;
  if (mmax * wide >= (int64_t(1) << 31) || (int64_t)c->T * wide_s >= (int64_t(1) << 31))
    return "T*K*max(d_model, d_ff) must be < 2^31";
  *code = MOE_OK;
  return "";
}

// ---------------------------------------------------------------- workspace
enum GemmPath { PATH_F32 = 0, PATH_TILED = 1, PATH_SKINNY = 2 };

GemmPath gemm_path(const moe_config_t* c) {
  if (c->dtype == MOE_F32) return PATH_F32;
  // Decode-shaped: on average at most 8 rows per routed expert.
  if ((int64_t)c->T * c->top_k <= 8LL * c->n_experts) return PATH_SKINNY;
  return PATH_TILED;
}

// Rows per tile of the tiled GEMMs (the bf16 kernel shrinks its wave layout
// for short tiles by itself).
int gemm_bm(const moe_config_t* c) {
  return gemm_path(c) == PATH_F32 ? moe::gemm_f32_bm() : moe::gemm_bf16_bm();
}
int gemm_bn(const moe_config_t* c) {
  return gemm_path(c) == PATH_F32 ? moe::gemm_f32_bn() : moe::gemm_bf16_bn();
}
// The shared expert rides in the routed launches when its width matches.
// (Not with INT8 routed weights: the shared expert keeps bf16 weights.)
bool fuse_shared(const moe_config_t* c) {
  return c->d_ff_shared > 0 && c->d_ff_shared == c->d_ff && c->weight_quant == MOE_WQ_NONE;
}

struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(bytes);
    return p;
  }
};

struct RouteWs {
  double* part;         // fp64 partial dot products, one slab per model-dim slice
};
struct DispatchWs {
  int32_t* blkcnt;
  int32_t* blkoff;
};
struct FfnWs {
  int4* list[4];        // tile lists: GEMM1, GEMM2, shared GEMM1, shared GEMM2
  int64_t bound[4];     // their capacities (tiles)
  int32_t* count;       // [4] tile counts
  void* h;
  void* h_shared;
};
struct AuxWs {
  double* ppart;
  double* term;
  double* zpart;
  double* spw;          // routing statistics partials
  int32_t* spcnt;
};
struct LayerWs {
  float* logits;
  int32_t* idx;
  float* w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* slot_row;
  int32_t* row_token;
  int32_t* n_dropped;
  void* x_perm;
  void* y_perm;
  void* y_shared;
  RouteWs route;
  DispatchWs disp;
  FfnWs ffn;
  AuxWs aux;
};

void carve_route(Carver& cv, const moe_config_t* c, RouteWs* w) {
  const int S = moe::route_splits(c->T, c->d_model, c->n_experts);
  w->part = cv.take<double>((size_t)S * c->T * c->n_experts * sizeof(double));
}

void carve_dispatch(Carver& cv, const moe_config_t* c, DispatchWs* w) {
  const size_t n = (size_t)moe::dispatch_blocks(c->T) * c->n_experts * sizeof(int32_t);
  w->blkcnt = cv.take<int32_t>(n);
  w->blkoff = cv.take<int32_t>(n);
}

void carve_ffn(Carver& cv, const moe_config_t* c, FfnWs* w) {
  const int64_t mmax = (int64_t)c->T * c->top_k;
  const size_t eb = elem_bytes(c->dtype);
  const int N = c->n_experts, bm = gemm_bm(c), bn = gemm_bn(c);
  const int ts = fuse_shared(c) ? c->T : 0;
  const int tsu = (c->d_ff_shared && !fuse_shared(c)) ? c->T : 0;
  w->bound[0] = moe::max_tiles(mmax, N, ts, bm, bn, c->d_ff);
  w->bound[1] = moe::max_tiles(mmax, N, ts, bm, bn, c->d_model);
  w->bound[2] = tsu ? moe::max_tiles(0, 0, tsu, bm, bn, c->d_ff_shared) : 0;
  w->bound[3] = tsu ? moe::max_tiles(0, 0, tsu, bm, bn, c->d_model) : 0;
  for (int i = 0; i < 4; ++i)
    w->list[i] = cv.take<int4>((size_t)(w->bound[i] > 0 ? w->bound[i] : 1) * sizeof(int4));
  w->count = cv.take<int32_t>(4 * sizeof(int32_t));
  w->h = cv.take<void>((size_t)mmax * c->d_ff * eb);
  w->h_shared = c->d_ff_shared ? cv.take<void>((size_t)c->T * c->d_ff_shared * eb) : nullptr;
}

void carve_aux(Carver& cv, const moe_config_t* c, AuxWs* w) {
  w->ppart = cv.take<double>((size_t)moe::aux_blocks(c->T) * c->n_experts * sizeof(double));
  w->term = cv.take<double>((size_t)c->n_experts * sizeof(double));
  w->zpart = cv.take<double>((size_t)moe::aux_blocks(c->T) * sizeof(double));
  w->spw = cv.take<double>((size_t)moe::stats_blocks(c->T) * c->n_experts * sizeof(double));
  w->spcnt = cv.take<int32_t>((size_t)moe::stats_blocks(c->T) * c->n_experts * sizeof(int32_t));
}

void carve_layer(Carver& cv, const moe_config_t* c, LayerWs* w) {
  const int64_t T = c->T, K = c->top_k, N = c->n_experts, mmax = T * K;
  const size_t eb = elem_bytes(c->dtype);
  w->logits = cv.take<float>(T * N * sizeof(float));
  w->idx = cv.take<int32_t>(mmax * sizeof(int32_t));
  w->w = cv.take<float>(mmax * sizeof(float));
  w->counts = cv.take<int32_t>(N * sizeof(int32_t));
  w->offsets = cv.take<int32_t>((N + 1) * sizeof(int32_t));
  w->slot_row = cv.take<int32_t>(mmax * sizeof(int32_t));
  w->row_token = cv.take<int32_t>(mmax * sizeof(int32_t));
  w->n_dropped = cv.take<int32_t>(sizeof(int32_t));
  w->x_perm = cv.take<void>((size_t)mmax * c->d_model * eb);
  w->y_perm = cv.take<void>((size_t)mmax * c->d_model * eb);
  w->y_shared = c->d_ff_shared ? cv.take<void>((size_t)T * c->d_model * eb) : nullptr;
  carve_route(cv, c, &w->route);
  carve_dispatch(cv, c, &w->disp);
  carve_ffn(cv, c, &w->ffn);
  carve_aux(cv, c, &w->aux);
}

size_t stage_bytes(const moe_config_t* c, moe_stage_t stage) {
  Carver cv{nullptr};
  switch (stage) {
    case MOE_STAGE_COMBINE:
      return 0;
    case MOE_STAGE_ROUTE: {
      RouteWs w;
      carve_route(cv, c, &w);
      return cv.off;
    }
    case MOE_STAGE_DISPATCH: {
      DispatchWs w;
      carve_dispatch(cv, c, &w);
      return cv.off;
    }
    case MOE_STAGE_EXPERT_FFN: {
      FfnWs w;
      carve_ffn(cv, c, &w);
      return cv.off;
    }
    case MOE_STAGE_AUX: {
      AuxWs w;
      carve_aux(cv, c, &w);
      return cv.off;
    }
    case MOE_STAGE_LAYER: {
      LayerWs w;
      carve_layer(cv, c, &w);
      return cv.off;
    }
  }
  return (size_t)-1;
}

int check_ws(const moe_config_t* c, moe_stage_t stage, const void* ws, size_t ws_bytes) {
  const size_t need = stage_bytes(c, stage);
  if (need == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                       " bytes, got " + std::to_string(ws_bytes));
  return MOE_OK;
}

#define MOE_CHECK_CFG(c)                          \
  do {                                            \
    int code_;                                    \
    std::string why_ = check_config((c), &code_); \
    if (code_ != MOE_OK) return fail(code_, why_); \
  } while (0)

#define MOE_REQUIRE_PTR(p, name)                                                 \
  do {                                                                           \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is NULL");  \
    if (!aligned16(p))                                                           \
      return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned"); \
  } while (0)

#define MOE_OPTIONAL_PTR(p, name)                                                \
  do {                                                                           \
    if ((p) && !aligned16(p))                                                    \
      return fail(MOE_ERR_INVALID_ARG, std::string(name) + " is not 16-byte aligned"); \
  } while (0)

int hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
  return MOE_OK;
}

// ---------------------------------------------------------------- stages (checked)
int do_route(const moe_config_t* c, const void* x, const moe_weights_t* w, float* logits,
             int32_t* idx, float* tw, const RouteWs& rw, hipStream_t s) {
  return hip_status(moe::launch_route(c->dtype, x, w->w_router, w->b_router, w->logit_offset,
                                      w->sel_bias, logits, idx, tw, rw.part, c->T, c->d_model,
                                      c->n_experts, c->top_k, s),
                    "moe_route launch");
}

int do_dispatch(const moe_config_t* c, const int32_t* idx, const void* x, int32_t* counts,
                int32_t* offsets, int32_t* slot_row, int32_t* row_token, void* x_perm,
                int32_t* n_dropped, const DispatchWs& dw, hipStream_t s) {
  return hip_status(
      moe::launch_dispatch(idx, x, (size_t)c->d_model * elem_bytes(c->dtype), c->T, c->top_k,
                           c->n_experts, c->capacity, counts, offsets, slot_row, row_token,
                           x_perm, n_dropped, dw.blkcnt, dw.blkoff, s),
      "moe_dispatch launch");
}

int do_ffn(const moe_config_t* c, const void* x_perm, const int32_t* offsets,
           const moe_weights_t* w, const void* x, void* y_perm, void* y_shared, const FfnWs& fw,
           hipStream_t s) {
  const GemmPath path = gemm_path(c);
  const int N = c->n_experts, T = c->T;
  const bool has_shared = c->d_ff_shared > 0;
  const bool fused = fuse_shared(c);
  const int bm = gemm_bm(c), bn = gemm_bn(c);

  // One GEMM launch: build its tile list (tiled kernels), then run it.
  auto gemm = [&](moe::GemmArgs g, int list, const int32_t* offs, int Nr, int Ts, bool gelu,
                  const char* what) -> int {
    hipError_t e = hipSuccess;
    if (path != PATH_SKINNY) {
      const int merge = path == PATH_TILED ? moe::gemm_bf16_merge_rows() : 0;
      e = moe::launch_tile_list(offs, Nr, bm, bn, g.Nd, Ts, merge, fw.list[list],
                                fw.count + list, s);
      if (e != hipSuccess) return hip_status(e, "tile list launch");
      g.tile_list = fw.list[list];
      g.tile_count = fw.count + list;
      g.grid_tiles = fw.bound[list];
    }
    if (path == PATH_F32)
      e = moe::launch_gemm_f32(g, gelu, s);
    else if (path == PATH_SKINNY)
      e = moe::launch_gemm_skinny_bf16(g, gelu, 0, s);
    else
      e = moe::launch_gemm_bf16(g, gelu, s);
    return e == hipSuccess ? MOE_OK : hip_status(e, what);
  };

  moe::GemmArgs g1{};
  g1.A = x_perm;
  g1.W = w->w1;
  g1.bias = w->b1;
  g1.C = fw.h;
  g1.offsets = offsets;
  g1.Kd = c->d_model;
  g1.Nd = c->d_ff;
  g1.E = N;
  const bool q8 = c->weight_quant == MOE_WQ_INT8;
  g1.wscale = q8 ? w->w1_scale : nullptr;
  moe::GemmArgs g2 = g1;
  g2.A = fw.h;
  g2.W = w->w2;
  g2.wscale = q8 ? w->w2_scale : nullptr;
  g2.bias = w->b2;
  g2.C = y_perm;
  g2.Kd = c->d_ff;
  g2.Nd = c->d_model;
  moe::GemmArgs s1{}, s2{};
  if (has_shared) {
    s1.As = x;
    s1.Ws = w->ws1;
    s1.Cs = fw.h_shared;
    s1.Ts = T;
    s1.Kd = c->d_model;
    s1.Nd = c->d_ff_shared;
    s2 = s1;
    s2.As = fw.h_shared;
    s2.Ws = w->ws2;
    s2.Cs = y_shared;
    s2.Kd = c->d_ff_shared;
    s2.Nd = c->d_model;
    if (fused) {
      g1.As = s1.As; g1.Ws = s1.Ws; g1.Cs = s1.Cs; g1.Ts = T;
      g2.As = s2.As; g2.Ws = s2.Ws; g2.Cs = s2.Cs; g2.Ts = T;
    }
  }
  const int tsf = fused ? T : 0;
  int r = gemm(g1, 0, offsets, N, tsf, true, "expert GEMM1 launch");
  if (r != MOE_OK) return r;
  if (has_shared && !fused) {
    r = gemm(s1, 2, nullptr, 0, T, true, "shared GEMM1 launch");
    if (r != MOE_OK) return r;
  }
  r = gemm(g2, 1, offsets, N, tsf, false, "expert GEMM2 launch");
  if (r != MOE_OK) return r;
  if (has_shared && !fused) {
    r = gemm(s2, 3, nullptr, 0, T, false, "shared GEMM2 launch");
    if (r != MOE_OK) return r;
  }
  return MOE_OK;
}

int do_combine(const moe_config_t* c, const void* y_perm, const int32_t* slot_row,
               const float* tw, const void* y_shared, void* out, hipStream_t s) {
  return hip_status(moe::launch_combine(c->dtype, y_perm, slot_row, tw, y_shared, out, c->T,
                                        c->d_model, c->top_k, s),
                    "moe_combine launch");
}

int do_aux(const moe_config_t* c, const float* logits, const int32_t* counts, float* loss,
           const AuxWs& aw, hipStream_t s) {
  return hip_status(moe::launch_aux(logits, counts, c->T, c->n_experts, c->aux_alpha, aw.ppart,
                                    aw.term, loss, s),
                    "moe_aux_loss launch");
}

int check_weights(const moe_config_t* c, const moe_weights_t* w, bool router, bool experts) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (router) {
    MOE_REQUIRE_PTR(w->w_router, "w_router");
    MOE_OPTIONAL_PTR(w->b_router, "b_router");
    MOE_OPTIONAL_PTR(w->logit_offset, "logit_offset");
    MOE_OPTIONAL_PTR(w->sel_bias, "sel_bias");
  }
  if (experts) {
    MOE_REQUIRE_PTR(w->w1, "w1");
    MOE_REQUIRE_PTR(w->w2, "w2");
    if (c->weight_quant == MOE_WQ_INT8) {
      MOE_REQUIRE_PTR(w->w1_scale, "w1_scale");
      MOE_REQUIRE_PTR(w->w2_scale, "w2_scale");
    }
    MOE_OPTIONAL_PTR(w->b1, "b1");
    MOE_OPTIONAL_PTR(w->b2, "b2");
    if (c->d_ff_shared) {
      MOE_REQUIRE_PTR(w->ws1, "ws1");
      MOE_REQUIRE_PTR(w->ws2, "ws2");
    }
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_config_t* cfg, moe_stage_t stage) {
  int code;
  if (!check_config(cfg, &code).empty()) return (size_t)-1;
  if ((int)stage < MOE_STAGE_ROUTE || (int)stage > MOE_STAGE_LAYER) return (size_t)-1;
  return stage_bytes(cfg, stage);
}

int32_t moe_capacity_from_factor(int32_t T, int32_t n_experts, double cf) {
  if (T < 1 || n_experts < 1 || !(cf > 0.0) || !isfinite(cf)) return -1;
  // cf = m * 2^ex exactly, m a 53-bit integer; ceil(T * m * 2^ex / N) in
  // 128-bit integer arithmetic.
  int ex;
  const double fr = frexp(cf, &ex);          // cf = fr * 2^ex, fr in [0.5, 1)
  const unsigned __int128 m = (unsigned __int128)ldexp(fr, 53);
  ex -= 53;
  unsigned __int128 num = m * (unsigned __int128)T;
  unsigned __int128 den = (unsigned __int128)n_experts;
  if (ex >= 0) {
    if (ex > 60) return -1;
    num <<= ex;
  } else {
    if (-ex > 120) return -1;
    den <<= -ex;
  }
  const unsigned __int128 q = (num + den - 1) / den;
  if (q > 0x7fffffff) return -1;
  return (int32_t)q;
}

int moe_route(const moe_config_t* cfg, const void* x, const moe_weights_t* w, float* logits,
              int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(x, "x");
  int r = check_weights(cfg, w, true, false);
  if (r != MOE_OK) return r;
  MOE_OPTIONAL_PTR(logits, "logits");
  MOE_REQUIRE_PTR(topk_idx, "topk_idx");
  MOE_REQUIRE_PTR(topk_w, "topk_w");
  r = check_ws(cfg, MOE_STAGE_ROUTE, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  RouteWs rw;
  carve_route(cv, cfg, &rw);
  return do_route(cfg, x, w, logits, topk_idx, topk_w, rw, stream);
}

int moe_dispatch(const moe_config_t* cfg, const int32_t* topk_idx, const void* x,
                 int32_t* counts, int32_t* expert_offsets, int32_t* slot_row,
                 int32_t* row_token, void* x_perm, int32_t* n_dropped, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(topk_idx, "topk_idx");
  MOE_REQUIRE_PTR(x, "x");
  MOE_REQUIRE_PTR(counts, "counts");
  MOE_REQUIRE_PTR(expert_offsets, "expert_offsets");
  MOE_REQUIRE_PTR(slot_row, "slot_row");
  MOE_REQUIRE_PTR(row_token, "row_token");
  MOE_REQUIRE_PTR(x_perm, "x_perm");
  MOE_REQUIRE_PTR(n_dropped, "n_dropped");
  int r = check_ws(cfg, MOE_STAGE_DISPATCH, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  DispatchWs dw;
  carve_dispatch(cv, cfg, &dw);
  return do_dispatch(cfg, topk_idx, x, counts, expert_offsets, slot_row, row_token, x_perm,
                     n_dropped, dw, stream);
}

int moe_expert_ffn(const moe_config_t* cfg, const void* x_perm, const int32_t* expert_offsets,
                   const moe_weights_t* w, const void* x, void* y_perm, void* y_shared, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(x_perm, "x_perm");
  MOE_REQUIRE_PTR(expert_offsets, "expert_offsets");
  int r = check_weights(cfg, w, false, true);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(y_perm, "y_perm");
  if (cfg->d_ff_shared) {
    MOE_REQUIRE_PTR(x, "x");
    MOE_REQUIRE_PTR(y_shared, "y_shared");
  } else if (y_shared) {
    return fail(MOE_ERR_INVALID_ARG, "y_shared given but the layer has no shared expert");
  }
  r = check_ws(cfg, MOE_STAGE_EXPERT_FFN, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  FfnWs fw;
  carve_ffn(cv, cfg, &fw);
  return do_ffn(cfg, x_perm, expert_offsets, w, x, y_perm, y_shared, fw, stream);
}

int moe_combine(const moe_config_t* cfg, const void* y_perm, const int32_t* slot_row,
                const float* topk_w, const void* y_shared, void* out, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(y_perm, "y_perm");
  MOE_REQUIRE_PTR(slot_row, "slot_row");
  MOE_REQUIRE_PTR(topk_w, "topk_w");
  MOE_OPTIONAL_PTR(y_shared, "y_shared");
  MOE_REQUIRE_PTR(out, "out");
  return do_combine(cfg, y_perm, slot_row, topk_w, y_shared, out, stream);
}

int moe_aux_loss(const moe_config_t* cfg, const float* logits, const int32_t* counts,
                 float* loss_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(logits, "logits");
  MOE_REQUIRE_PTR(counts, "counts");
  if (!loss_out) return fail(MOE_ERR_INVALID_ARG, "loss_out is NULL");
  int r = check_ws(cfg, MOE_STAGE_AUX, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  AuxWs aw;
  carve_aux(cv, cfg, &aw);
  return do_aux(cfg, logits, counts, loss_out, aw, stream);
}

int moe_quantize_int8(const void* w, int32_t dtype, int64_t rows, int32_t cols, int8_t* q,
                      float* scale, hipStream_t stream) {
  MOE_REQUIRE_PTR(w, "w");
  MOE_REQUIRE_PTR(q, "q");
  MOE_REQUIRE_PTR(scale, "scale");
  if (dtype != MOE_F32 && dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_F32 or MOE_BF16");
  if (rows < 1) return fail(MOE_ERR_INVALID_ARG, "rows must be >= 1");
  if (cols < 64 || cols % 64) return fail(MOE_ERR_INVALID_ARG, "cols must be a positive multiple of 64");
  return hip_status(moe::launch_quantize_int8(w, dtype, rows, cols, q, scale, stream),
                    "moe_quantize_int8 launch");
}

int moe_routing_stats(const moe_config_t* cfg, const int32_t* topk_idx, const float* topk_w,
                      int32_t* counts_out, float* weight_mean_out, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(topk_idx, "topk_idx");
  MOE_REQUIRE_PTR(topk_w, "topk_w");
  MOE_OPTIONAL_PTR(counts_out, "counts_out");
  if (!weight_mean_out) return fail(MOE_ERR_INVALID_ARG, "weight_mean_out is NULL");
  int r = check_ws(cfg, MOE_STAGE_AUX, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  AuxWs aw;
  carve_aux(cv, cfg, &aw);
  return hip_status(moe::launch_stats(topk_idx, topk_w, cfg->T, cfg->top_k, cfg->n_experts,
                                      aw.spcnt, aw.spw, counts_out, weight_mean_out, stream),
                    "moe_routing_stats launch");
}

int moe_router_z_loss(const moe_config_t* cfg, const float* logits, float beta, float* loss_out,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(logits, "logits");
  if (!loss_out) return fail(MOE_ERR_INVALID_ARG, "loss_out is NULL");
  if (!isfinite(beta)) return fail(MOE_ERR_INVALID_ARG, "beta is not finite");
  int r = check_ws(cfg, MOE_STAGE_AUX, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  AuxWs aw;
  carve_aux(cv, cfg, &aw);
  return hip_status(moe::launch_zloss(logits, cfg->T, cfg->n_experts, beta, aw.zpart, loss_out,
                                      stream),
                    "moe_router_z_loss launch");
}

int moe_layer_forward(const moe_config_t* cfg, const void* x, const moe_weights_t* w, void* out,
                      float* aux_out, int32_t* counts_out, int32_t* n_dropped_out, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(x, "x");
  int r = check_weights(cfg, w, true, true);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(out, "out");
  MOE_OPTIONAL_PTR(counts_out, "counts_out");
  r = check_ws(cfg, MOE_STAGE_LAYER, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  LayerWs lw;
  carve_layer(cv, cfg, &lw);
  int32_t* counts = counts_out ? counts_out : lw.counts;
  int32_t* ndrop = n_dropped_out ? n_dropped_out : lw.n_dropped;

  r = do_route(cfg, x, w, lw.logits, lw.idx, lw.w, lw.route, stream);
  if (r != MOE_OK) return r;
  r = do_dispatch(cfg, lw.idx, x, counts, lw.offsets, lw.slot_row, lw.row_token, lw.x_perm,
                  ndrop, lw.disp, stream);
  if (r != MOE_OK) return r;
  r = do_ffn(cfg, lw.x_perm, lw.offsets, w, x, lw.y_perm, lw.y_shared, lw.ffn, stream);
  if (r != MOE_OK) return r;
  r = do_combine(cfg, lw.y_perm, lw.slot_row, lw.w, lw.y_shared, out, stream);
  if (r != MOE_OK) return r;
  if (aux_out) {
    r = do_aux(cfg, lw.logits, counts, aux_out, lw.aux, stream);
    if (r != MOE_OK) return r;
  }
  return MOE_OK;
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
