// Host side of libmoe.so: argument checks, workspace carving, launch order.
// The entry points and their contracts are declared in include/moe.h.
#include <math.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "moe_internal.h"

// The workspace of moe_layer_forward_noalloc: a file-scope device array, so
// that call needs no allocation.  Each GPU the library runs on holds its own
// copy (MOE_NOALLOC_SCRATCH_BYTES) until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory: kernels and
// copies get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

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
  if (c->weight_quant != MOE_WQ_NONE && c->weight_quant != MOE_WQ_INT8 &&
      c->weight_quant != MOE_WQ_INT4)
    return "weight_quant must be MOE_WQ_NONE, MOE_WQ_INT8 or MOE_WQ_INT4";
  if (c->router != MOE_ROUTER_AUTO && c->router != MOE_ROUTER_EXACT &&
      c->router != MOE_ROUTER_CERTIFIED)
    return "router must be MOE_ROUTER_AUTO, MOE_ROUTER_EXACT or MOE_ROUTER_CERTIFIED";
  if (c->router == MOE_ROUTER_CERTIFIED && c->dtype != MOE_BF16)
    return "MOE_ROUTER_CERTIFIED needs dtype MOE_BF16";
  *code = MOE_ERR_UNSUPPORTED;
  if (c->weight_quant != MOE_WQ_NONE && c->dtype != MOE_BF16)
    return "INT8 and INT4 expert weights need dtype MOE_BF16";
  if (c->weight_quant == MOE_WQ_INT4 && (c->d_model % 128 || c->d_ff % 128))
    return "INT4 expert weights need d_model and d_ff multiples of 128";
  if (c->n_experts > 256) return "n_experts > 256 is not supported";
  if (c->top_k > 64) return "top_k > 64 is not supported";
  if (c->d_model % 64 || c->d_ff % 64 || c->d_ff_shared % 64)
    return "d_model, d_ff and d_ff_shared must be multiples of 64";
  const int64_t mmax = (int64_t)c->T * c->top_k;
  const int64_t wide = c->d_model > c->d_ff ? c->d_model : c->d_ff;
  const int64_t wide_s = c->d_ff_shared > c->d_model ? c->d_ff_shared : c->d_model;
  if (mmax * wide >= (int64_t(1) << 31) || (int64_t)c->T * wide_s >= (int64_t(1) << 31))
    return "T*K*max(d_model, d_ff) must be < 2^31";
  // (the GEMMs address one expert's weight matrix with 32-bit byte offsets)
  if ((int64_t)c->d_model * c->d_ff >= (int64_t(1) << 31) ||
      (int64_t)c->d_model * c->d_ff_shared >= (int64_t(1) << 31))
    return "d_model*d_ff and d_model*d_ff_shared must be < 2^31";
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

// The certified bf16 router where the fp64 router GEMM would be a visible
// share of the layer (2 T N d >= 2^31 flops), or where asked for.
bool router_certified(const moe_config_t* c) {
  if (c->router == MOE_ROUTER_CERTIFIED) return true;
  if (c->router == MOE_ROUTER_EXACT || c->dtype != MOE_BF16) return false;
  return 2.0 * c->T * c->n_experts * (double)c->d_model >= 2147483648.0;
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
// Its weights stay bf16 under INT8 routed weights: the tiled kernel runs the
// shared tiles through its bf16 path, the decode kernel leaves them to
// launches of their own.
// Few rows per expert (at most 320 on average): the backward's routed GEMMs
// run eight-wavefront workgroups (measured on the same GPU: the Switch-shaped
// backward 7% and the DeepSeek-shaped one 3.5% faster, from the
// weight-gradient GEMMs' short k-segments; the forward GEMMs gain nothing and
// keep four).
bool weight_bound(const moe_config_t* c) {
  return (int64_t)c->T * c->top_k <= 320LL * c->n_experts;
}

bool fuse_shared(const moe_config_t* c) {
  return c->d_ff_shared > 0 && c->d_ff_shared == c->d_ff &&
         (c->weight_quant == MOE_WQ_NONE || gemm_path(c) == PATH_TILED);
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
  void* part;           // partial dot products, one slab per model-dim slice
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
// The routing-partials buffer (moe_route's optional output, and the
// workspace copy the loss / statistics entry points and the layer use):
// ppart [nb, N] fp64, zpart [nb] fp64, spw [nb, N] fp64, spcnt [nb, N] int32,
// nb = aux_blocks(T), each array 256-byte aligned in that order.
struct PartLayout {
  size_t ppart, zpart, spw, spcnt, total;
};
PartLayout part_layout(const moe_config_t* c) {
  const size_t nb = (size_t)moe::aux_blocks(c->T), N = (size_t)c->n_experts;
  PartLayout L;
  size_t off = 0;
  L.ppart = off;
  off = align_up(off + nb * N * sizeof(double));
  L.zpart = off;
  off = align_up(off + nb * sizeof(double));
  L.spw = off;
  off = align_up(off + nb * N * sizeof(double));
  L.spcnt = off;
  off = align_up(off + nb * N * sizeof(int32_t));
  L.total = off;
  return L;
}
moe::RoutePartials partials_at(void* base, const moe_config_t* c) {
  const PartLayout L = part_layout(c);
  char* b = static_cast<char*>(base);
  moe::RoutePartials rp;
  rp.ppart = reinterpret_cast<double*>(b + L.ppart);
  rp.zpart = reinterpret_cast<double*>(b + L.zpart);
  rp.spw = reinterpret_cast<double*>(b + L.spw);
  rp.spcnt = reinterpret_cast<int32_t*>(b + L.spcnt);
  return rp;
}

struct AuxWs {
  moe::RoutePartials rp;  // partials computed here when the caller has none
  double* term;
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
  w->part = cv.take<void>(
      moe::route_ws_bytes(c->T, c->d_model, c->n_experts, router_certified(c)));
}

void carve_dispatch(Carver& cv, const moe_config_t* c, DispatchWs* w) {
  const size_t n = (size_t)moe::dispatch_blocks(c->T) * c->n_experts * sizeof(int32_t);
  w->blkcnt = cv.take<int32_t>(n);
  w->blkoff = cv.take<int32_t>(n);
}

void carve_ffn(Carver& cv, const moe_config_t* c, FfnWs* w, bool hidden = true) {
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
  w->h = hidden ? cv.take<void>((size_t)mmax * c->d_ff * eb) : nullptr;
  w->h_shared =
      (hidden && c->d_ff_shared) ? cv.take<void>((size_t)c->T * c->d_ff_shared * eb) : nullptr;
}

void carve_aux(Carver& cv, const moe_config_t* c, AuxWs* w) {
  char* parts = cv.take<char>(part_layout(c).total);
  w->rp = parts ? partials_at(parts, c) : moe::RoutePartials{};
  w->term = cv.take<double>((size_t)c->n_experts * sizeof(double));
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

// ---------------------------------------------------------------- training workspaces
// Backward GEMMs never take the decode-shaped kernel (it has no k-segment mode).
bool bwd_f32(const moe_config_t* c) { return c->dtype == MOE_F32; }
int bwd_bm(const moe_config_t* c) { return bwd_f32(c) ? moe::gemm_f32_bm() : moe::gemm_bf16_bm(); }
int bwd_bn(const moe_config_t* c) { return bwd_f32(c) ? moe::gemm_f32_bn() : moe::gemm_bf16_bn(); }
int bwd_merge(const moe_config_t* c) { return bwd_f32(c) ? 0 : moe::gemm_bf16_merge_rows(); }
// The routed weight-gradient GEMMs of launches bound by the weight stream run
// narrow tiles, two workgroups per CU (their k-segments are a few k-steps).
bool wg_narrow(const moe_config_t* c) { return !bwd_f32(c) && weight_bound(c); }
int wg_bn(const moe_config_t* c) {
  return wg_narrow(c) ? moe::gemm_bf16_wg_narrow_bn() : bwd_bn(c);
}
// Row stride of the per-expert transposed activations: every expert's rows
// rounded up to 32 (at most T*K + 31 N in all), or the T rows of the shared
// expert, rounded up to 64.
int64_t bwd_ldt(const moe_config_t* c) {
  const int64_t a = (int64_t)c->T * c->top_k + 32LL * c->n_experts, b = (int64_t)c->T + 32;
  return ((a > b ? a : b) + 63) / 64 * 64;
}
int64_t bwd_maxw(const moe_config_t* c) {
  int64_t m = c->d_model > c->d_ff ? c->d_model : c->d_ff;
  return m > c->d_ff_shared ? m : c->d_ff_shared;
}

struct FfnBwdWs {
  void *dh, *dhs;                  // d_h, then d_z in place
  void *tb1, *tb2;                 // transposed activations [maxw, ldt]
  int32_t *kseg, *wr_d, *wr_f;     // routed k-segments and output-row offsets
  int32_t *off2, *kseg2, *wr2_d, *wr2_s;   // the shared expert's single segment
  int4* list[8];                   // dgrad1, dgrad2, wgrad2, wgrad1; the same for the shared expert
  int64_t bound[8];
  int32_t* count;
};
struct RouteBwdWs {
  float* dl;                       // d_logits [T, N]
  float* part;                     // router weight-gradient partials
};
struct LayerTrainWs {
  RouteWs route;
  DispatchWs disp;
  FfnWs ffn;                       // tile lists only
  void* y_shared;
  AuxWs aux;
};
struct LayerBwdWs {
  void* d_y_perm;
  float* d_topk_w;
  void* d_x_perm;
  void* d_x_shared;
  float* d_x_router;
  FfnBwdWs ffn;
  RouteBwdWs route;
};

void carve_ffn_bwd(Carver& cv, const moe_config_t* c, FfnBwdWs* w) {
  const int64_t T = c->T, N = c->n_experts, d = c->d_model, f = c->d_ff, fs = c->d_ff_shared;
  const int64_t M = T * c->top_k;
  const size_t eb = elem_bytes(c->dtype);
  w->dh = cv.take<void>((size_t)(M * f) * eb);
  w->dhs = fs ? cv.take<void>((size_t)(T * fs) * eb) : nullptr;
  const int64_t ldt = bwd_ldt(c), maxw = bwd_maxw(c);
  w->tb1 = cv.take<void>((size_t)(maxw * ldt) * eb);
  w->tb2 = cv.take<void>((size_t)(maxw * ldt) * eb);
  w->kseg = cv.take<int32_t>((N + 1) * sizeof(int32_t));
  w->wr_d = cv.take<int32_t>((N + 1) * sizeof(int32_t));
  w->wr_f = cv.take<int32_t>((N + 1) * sizeof(int32_t));
  w->off2 = cv.take<int32_t>(2 * sizeof(int32_t));
  w->kseg2 = cv.take<int32_t>(2 * sizeof(int32_t));
  w->wr2_d = cv.take<int32_t>(2 * sizeof(int32_t));
  w->wr2_s = cv.take<int32_t>(2 * sizeof(int32_t));
  const int bm = bwd_bm(c), bn = bwd_bn(c);
  w->bound[0] = moe::max_tiles(M, (int)N, 0, bm, bn, f);
  w->bound[1] = moe::max_tiles(M, (int)N, 0, bm, bn, d);
  w->bound[2] = moe::max_tiles(N * d, (int)N, 0, bm, wg_bn(c), f);
  w->bound[3] = moe::max_tiles(N * f, (int)N, 0, bm, wg_bn(c), d);
  w->bound[4] = fs ? moe::max_tiles(0, 0, (int)T, bm, bn, fs) : 0;
  w->bound[5] = fs ? moe::max_tiles(0, 0, (int)T, bm, bn, d) : 0;
  w->bound[6] = fs ? moe::max_tiles(d, 1, 0, bm, bn, fs) : 0;
  w->bound[7] = fs ? moe::max_tiles(fs, 1, 0, bm, bn, d) : 0;
  for (int i = 0; i < 8; ++i)
    w->list[i] = cv.take<int4>((size_t)(w->bound[i] > 0 ? w->bound[i] : 1) * sizeof(int4));
  w->count = cv.take<int32_t>(8 * sizeof(int32_t));
}

void carve_route_bwd(Carver& cv, const moe_config_t* c, RouteBwdWs* w) {
  w->dl = cv.take<float>((size_t)c->T * c->n_experts * sizeof(float));
  w->part = cv.take<float>((size_t)moe::router_dw_slices(c->T, c->n_experts, c->d_model) *
                           c->n_experts * c->d_model * sizeof(float));
}

void carve_layer_train(Carver& cv, const moe_config_t* c, LayerTrainWs* w) {
  carve_route(cv, c, &w->route);
  carve_dispatch(cv, c, &w->disp);
  carve_ffn(cv, c, &w->ffn, false);
  w->y_shared =
      c->d_ff_shared ? cv.take<void>((size_t)c->T * c->d_model * elem_bytes(c->dtype)) : nullptr;
  carve_aux(cv, c, &w->aux);
}

void carve_layer_bwd(Carver& cv, const moe_config_t* c, LayerBwdWs* w) {
  const int64_t T = c->T, M = T * c->top_k, d = c->d_model;
  const size_t eb = elem_bytes(c->dtype);
  w->d_y_perm = cv.take<void>((size_t)(M * d) * eb);
  w->d_topk_w = cv.take<float>((size_t)M * sizeof(float));
  w->d_x_perm = cv.take<void>((size_t)(M * d) * eb);
  w->d_x_shared = c->d_ff_shared ? cv.take<void>((size_t)(T * d) * eb) : nullptr;
  w->d_x_router = cv.take<float>((size_t)(T * d) * sizeof(float));
  carve_ffn_bwd(cv, c, &w->ffn);
  carve_route_bwd(cv, c, &w->route);
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
    case MOE_STAGE_EXPERT_FFN_TRAIN: {
      FfnWs w;
      carve_ffn(cv, c, &w, false);
      return cv.off;
    }
    case MOE_STAGE_LAYER_TRAIN: {
      LayerTrainWs w;
      carve_layer_train(cv, c, &w);
      return cv.off;
    }
    case MOE_STAGE_EXPERT_FFN_BACKWARD: {
      FfnBwdWs w;
      carve_ffn_bwd(cv, c, &w);
      return cv.off;
    }
    case MOE_STAGE_ROUTE_BACKWARD: {
      RouteBwdWs w;
      carve_route_bwd(cv, c, &w);
      return cv.off;
    }
    case MOE_STAGE_LAYER_BACKWARD: {
      LayerBwdWs w;
      carve_layer_bwd(cv, c, &w);
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
// parts: the routing partials to write with the selection, or null.
int do_route(const moe_config_t* c, const void* x, const moe_weights_t* w, float* logits,
             int32_t* idx, float* tw, const RouteWs& rw, hipStream_t s,
             const moe::RoutePartials* parts = nullptr) {
  return hip_status(moe::launch_route(c->dtype, router_certified(c), x, w->w_router, w->b_router,
                                      w->logit_offset, w->sel_bias, logits, idx, tw, rw.part,
                                      c->T, c->d_model, c->n_experts, c->top_k, parts, s),
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

// h / hs: the hidden activations GEMM2 reads.  Training mode (z != null):
// GEMM1 writes the pre-activations z / zs without the GELU, and a GELU pass
// writes h / hs from them, so the backward has both.
int do_ffn(const moe_config_t* c, const void* x_perm, const int32_t* offsets,
           const moe_weights_t* w, const void* x, void* y_perm, void* y_shared, const FfnWs& fw,
           hipStream_t s, void* h, void* hs, void* z = nullptr, void* zs = nullptr) {
  const bool train = z != nullptr;
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
      // Wide tiles for small blocks: with INT8 / INT4 weights, whose A rows
      // are half of a short tile's load bytes (same-GPU: Switch-shaped INT8
      // stage 5% faster), and with bf16 weights in layers of at least 64
      // experts (same-GPU: the DeepSeek-shaped stage 3.71 -> 3.61 ms with
      // 128-row wide tiles, both GEMMs gaining; with the 64- and 96-row wide
      // layouts the Switch shape's 64 experts gain too, 0.994 -> 0.981 ms,
      // where 128-row wide tiles had lost 2%), and only where there are
      // rounds of tiles to spare (about four of the chip's 256 CUs' worth),
      // so that halving the tiles of the small blocks (each twice as long)
      // does not unbalance the last round.
      g.wide_rows = path == PATH_TILED && (g.wscale || c->n_experts >= 64) &&
                            (int64_t)Nr * ((g.Nd + bn - 1) / bn) >= 1024
                        ? moe::gemm_bf16_wide_rows() : 0;
      // Non-temporal loads of bf16 weights where each expert's weights are
      // streamed once (few rows per expert) and the permuted activations are
      // small enough to stay in the 256 MB MALL (same-GPU: the Switch-shaped
      // forward 3.6% faster, its combine 10%; with the DeepSeek shape's
      // 470 MB of activations no gain, Mixtral's weights, re-read per
      // m-tile, 5% slower, and INT8 codes, whose 64-byte rows fill a cache
      // line over two k-steps, 12% slower).  Not with a shared expert in the
      // launch: its weights are re-read by every m-tile of the T tokens.  Not
      // in the training forward either, which keeps z and runs the GELU as a
      // kernel of its own (there the Switch-shaped forward ran 5% slower).
      // (the activations of this launch: its A operand, T*K rows of Kd)
      g.w_stream = path == PATH_TILED && !train && !g.wscale && Ts == 0 && weight_bound(c) &&
                   (int64_t)c->T * c->top_k * g.Kd * (int64_t)elem_bytes(c->dtype) <=
                       (int64_t(128) << 20);
      e = moe::launch_tile_list(offs, Nr, bm, bn, g.Nd, Ts, merge, fw.bound[list],
                                fw.list[list], fw.count + list, s, g.wide_rows);
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
  g1.C = train ? z : h;
  g1.offsets = offsets;
  g1.Kd = c->d_model;
  g1.Nd = c->d_ff;
  g1.E = N;
  const bool quant = c->weight_quant != MOE_WQ_NONE;
  g1.wscale = quant ? w->w1_scale : nullptr;
  g1.w4 = c->weight_quant == MOE_WQ_INT4;
  moe::GemmArgs g2 = g1;
  g2.A = h;
  g2.W = w->w2;
  g2.wscale = quant ? w->w2_scale : nullptr;
  g2.bias = w->b2;
  g2.C = y_perm;
  g2.Kd = c->d_ff;
  g2.Nd = c->d_model;
  moe::GemmArgs s1{}, s2{};
  if (has_shared) {
    s1.As = x;
    s1.Ws = w->ws1;
    s1.Cs = train ? zs : hs;
    s1.Ts = T;
    s1.Kd = c->d_model;
    s1.Nd = c->d_ff_shared;
    s2 = s1;
    s2.As = hs;
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
  int r = gemm(g1, 0, offsets, N, tsf, !train, "expert GEMM1 launch");
  if (r != MOE_OK) return r;
  if (has_shared && !fused) {
    r = gemm(s1, 2, nullptr, 0, T, !train, "shared GEMM1 launch");
    if (r != MOE_OK) return r;
  }
  if (train) {
    r = hip_status(moe::launch_gelu_fwd(c->dtype, z, h, offsets + N, T * c->top_k, c->d_ff, s),
                   "GELU launch");
    if (r != MOE_OK) return r;
    if (has_shared) {
      r = hip_status(moe::launch_gelu_fwd(c->dtype, zs, hs, nullptr, T, c->d_ff_shared, s),
                     "shared GELU launch");
      if (r != MOE_OK) return r;
    }
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

// The aux loss from routing partials (rp), which hold the probability sums
// already, or are first formed from the logits when `logits` is not null.
int do_aux(const moe_config_t* c, const float* logits, const moe::RoutePartials& rp,
           const int32_t* counts, float* loss, const AuxWs& aw, hipStream_t s) {
  if (logits) {
    int r = hip_status(moe::launch_logit_partials(logits, c->T, c->n_experts, rp, s),
                       "aux partials launch");
    if (r != MOE_OK) return r;
  }
  return hip_status(moe::launch_aux_final(rp, counts, c->T, c->n_experts, c->aux_alpha, aw.term,
                                          loss, s),
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
    if (c->weight_quant != MOE_WQ_NONE) {
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


// ---------------------------------------------------------------- training (checked)
// The training entry points: INT8 experts are inference-only, and the
// transposed activations use 32-bit offsets in the GEMM kernels.
std::string check_train(const moe_config_t* c, int* code) {
  std::string why = check_config(c, code);
  if (!why.empty()) return why;
  *code = MOE_ERR_UNSUPPORTED;
  if (c->weight_quant != MOE_WQ_NONE) return "training entry points need weight_quant MOE_WQ_NONE";
  if (bwd_maxw(c) * bwd_ldt(c) >= (int64_t(1) << 31))
    return "max(d_model, d_ff, d_ff_shared) * (T*K + 32N) must be < 2^31 for the backward";
  *code = MOE_OK;
  return "";
}

#define MOE_CHECK_TRAIN(c)                        \
  do {                                            \
    int code_;                                    \
    std::string why_ = check_train((c), &code_);  \
    if (code_ != MOE_OK) return fail(code_, why_); \
  } while (0)

// One backward GEMM: tile list, then the tiled (bf16) or fp32 kernel.
int bwd_gemm(const moe_config_t* c, moe::GemmArgs g, int4* list, int32_t* count, int64_t bound,
             const int32_t* offs, int Nr, int Ts, hipStream_t s, const char* what) {
  hipError_t e = moe::launch_tile_list(offs, Nr, bwd_bm(c), g.wg_narrow ? wg_bn(c) : bwd_bn(c),
                                       g.Nd, Ts, g.wg_narrow ? 0 : bwd_merge(c), bound, list,
                                       count, s);
  if (e != hipSuccess) return hip_status(e, "tile list launch");
  g.tile_list = list;
  g.tile_count = count;
  g.grid_tiles = bound;
  e = bwd_f32(c) ? moe::launch_gemm_f32(g, false, s) : moe::launch_gemm_bf16(g, false, s);
  return e == hipSuccess ? MOE_OK : hip_status(e, what);
}

// One input-gradient GEMM (weights read k-major): on decode-shaped layers the
// weight-streaming kernel (no tile list; same-GPU, the decode-shaped
// backward's two routed input-gradient GEMMs took 0.93 ms on the tiled kernel),
// else bwd_gemm.
int dgrad_gemm(const moe_config_t* c, const moe::GemmArgs& g, int4* list, int32_t* count,
               int64_t bound, const int32_t* offs, int Nr, int Ts, hipStream_t s) {
  if (gemm_path(c) == PATH_SKINNY)
    return hip_status(moe::launch_gemm_skinny_kmaj_bf16(g, s), "dgrad GEMM launch");
  return bwd_gemm(c, g, list, count, bound, offs, Nr, Ts, s, "dgrad GEMM launch");
}

int do_combine_bwd(const moe_config_t* c, const void* d_out, const void* y_perm,
                   const int32_t* slot_row, const float* tw, void* d_y_perm, float* d_tw,
                   hipStream_t s) {
  return hip_status(moe::launch_combine_bwd(c->dtype, d_out, y_perm, slot_row, tw, d_y_perm, d_tw,
                                            c->T, c->d_model, c->top_k, s),
                    "moe_combine_backward launch");
}

// Expert FFN backward (routed experts, then the shared one):
//   d_h = d_y . W2, d_z = d_h * GELU'(z), d_x_perm = d_z . W1 (the GEMMs read
//   the forward's weights k-major),
//   dW2_e = d_y_e^T h_e, db2_e = column sums of d_y_e, dW1_e = d_z_e^T x_e,
//   db1_e = column sums of d_z_e (weight gradients in the k-segment mode).
int do_ffn_bwd(const moe_config_t* c, const void* x_perm, const int32_t* offsets,
               const moe_weights_t* w, const void* x, const void* z, const void* h,
               const void* zs, const void* hs, const void* d_y_perm, const void* d_out,
               void* d_x_perm, void* d_x_shared, const moe_grads_t* g, const FfnBwdWs& fw,
               hipStream_t s) {
  const int dt = c->dtype, T = c->T, N = c->n_experts, d = c->d_model, f = c->d_ff;
  const int fs = c->d_ff_shared;
  const int M = T * c->top_k;
  const int ldt = (int)bwd_ldt(c);
  int r;
#define MOE_TRY(expr, what)                           \
  do {                                                \
    r = hip_status((expr), what);                     \
    if (r != MOE_OK) return r;                        \
  } while (0)
  MOE_TRY(moe::launch_seg_offsets(offsets, N, d, f, fw.kseg, fw.wr_d, fw.wr_f, s), "offsets launch");
  moe::GemmArgs a{};
  a.A = d_y_perm;                       // d_h [M, f] = d_y [M, d] . W2_e [d, f]
  a.W = w->w2;
  a.wkmaj = true;
  a.waves8 = weight_bound(c);
  a.C = fw.dh;
  a.offsets = offsets;
  a.Kd = d;
  a.Nd = f;
  a.E = N;
  r = dgrad_gemm(c, a, fw.list[0], fw.count + 0, fw.bound[0], offsets, N, 0, s);
  if (r != MOE_OK) return r;
  MOE_TRY(moe::launch_gelu_bwd(dt, z, fw.dh, offsets + N, M, f, s), "GELU backward launch");
  a.A = fw.dh;                          // d_x_perm [M, d] = d_z [M, f] . W1_e [f, d]
  a.W = w->w1;
  a.C = d_x_perm;
  a.Kd = f;
  a.Nd = d;
  r = dgrad_gemm(c, a, fw.list[1], fw.count + 1, fw.bound[1], offsets, N, 0, s);
  if (r != MOE_OK) return r;
  // dW2 [N, d, f]: A = d_y^T [d, ldt], W = h^T [f, ldt]
  MOE_TRY(moe::launch_transpose_segments(dt, d_y_perm, offsets, fw.kseg, N, d, ldt, fw.tb1, g->d_b2, s),
          "transpose launch");
  MOE_TRY(moe::launch_transpose_segments(dt, h, offsets, fw.kseg, N, f, ldt, fw.tb2, nullptr, s),
          "transpose launch");
  moe::GemmArgs wg{};
  wg.A = fw.tb1;
  wg.W = fw.tb2;
  wg.C = g->d_w2;
  wg.Kd = ldt;
  wg.Nd = f;
  wg.E = N;
  wg.kseg = fw.kseg;
  wg.wg_rows = d;
  wg.waves8 = weight_bound(c);
  wg.wg_narrow = wg_narrow(c);
  r = bwd_gemm(c, wg, fw.list[2], fw.count + 2, fw.bound[2], fw.wr_d, N, 0, s, "wgrad GEMM launch");
  if (r != MOE_OK) return r;
  // dW1 [N, f, d]: A = d_z^T [f, ldt], W = x_perm^T [d, ldt]
  MOE_TRY(moe::launch_transpose_segments(dt, fw.dh, offsets, fw.kseg, N, f, ldt, fw.tb1, g->d_b1, s),
          "transpose launch");
  MOE_TRY(moe::launch_transpose_segments(dt, x_perm, offsets, fw.kseg, N, d, ldt, fw.tb2, nullptr, s),
          "transpose launch");
  wg.C = g->d_w1;
  wg.Nd = d;
  wg.wg_rows = f;
  r = bwd_gemm(c, wg, fw.list[3], fw.count + 3, fw.bound[3], fw.wr_f, N, 0, s, "wgrad GEMM launch");
  if (r != MOE_OK) return r;
  if (!fs) return MOE_OK;

  // shared expert: upstream gradient d_out for every token, weight 1
  MOE_TRY(moe::launch_dense_offsets(T, d, fs, fw.off2, fw.kseg2, fw.wr2_d, fw.wr2_s, s),
          "offsets launch");
  moe::GemmArgs sa{};
  sa.As = d_out;                        // d_hs [T, fs] = d_out . Ws2 [d, fs]
  sa.Ws = w->ws2;
  sa.wkmaj = true;
  sa.Cs = fw.dhs;
  sa.Ts = T;
  sa.Kd = d;
  sa.Nd = fs;
  r = dgrad_gemm(c, sa, fw.list[4], fw.count + 4, fw.bound[4], nullptr, 0, T, s);
  if (r != MOE_OK) return r;
  MOE_TRY(moe::launch_gelu_bwd(dt, zs, fw.dhs, nullptr, T, fs, s), "GELU backward launch");
  sa.As = fw.dhs;                       // d_x_shared [T, d] = d_zs . Ws1 [fs, d]
  sa.Ws = w->ws1;
  sa.Cs = d_x_shared;
  sa.Kd = fs;
  sa.Nd = d;
  r = dgrad_gemm(c, sa, fw.list[5], fw.count + 5, fw.bound[5], nullptr, 0, T, s);
  if (r != MOE_OK) return r;
  MOE_TRY(moe::launch_transpose_segments(dt, d_out, fw.off2, fw.kseg2, 1, d, ldt, fw.tb1, nullptr, s,
                                          c->T),
          "transpose launch");
  MOE_TRY(moe::launch_transpose_segments(dt, hs, fw.off2, fw.kseg2, 1, fs, ldt, fw.tb2, nullptr, s,
                                          c->T),
          "transpose launch");
  moe::GemmArgs sw{};
  sw.A = fw.tb1;                        // dWs2 [d, fs]
  sw.W = fw.tb2;
  sw.C = g->d_ws2;
  sw.Kd = ldt;
  sw.Nd = fs;
  sw.E = 1;
  sw.kseg = fw.kseg2;
  sw.wg_rows = d;
  r = bwd_gemm(c, sw, fw.list[6], fw.count + 6, fw.bound[6], fw.wr2_d, 1, 0, s, "wgrad GEMM launch");
  if (r != MOE_OK) return r;
  MOE_TRY(moe::launch_transpose_segments(dt, fw.dhs, fw.off2, fw.kseg2, 1, fs, ldt, fw.tb1, nullptr, s,
                                          c->T),
          "transpose launch");
  MOE_TRY(moe::launch_transpose_segments(dt, x, fw.off2, fw.kseg2, 1, d, ldt, fw.tb2, nullptr, s,
                                          c->T),
          "transpose launch");
  sw.C = g->d_ws1;                      // dWs1 [fs, d]
  sw.Nd = d;
  sw.wg_rows = fs;
  r = bwd_gemm(c, sw, fw.list[7], fw.count + 7, fw.bound[7], fw.wr2_s, 1, 0, s, "wgrad GEMM launch");
#undef MOE_TRY
  return r;
}

int do_route_bwd(const moe_config_t* c, const void* x, const moe_weights_t* w, const float* logits,
                 const int32_t* idx, const float* tw, const float* dtw, const int32_t* counts,
                 float aux_grad, float zloss_beta, float zloss_grad, float* dl, float* d_x_router,
                 const moe_grads_t* g, const RouteBwdWs& rw, hipStream_t s) {
  const float aux_coef = (c->aux_alpha != 0.f && aux_grad != 0.f)
                             ? (float)((double)aux_grad * c->aux_alpha * c->n_experts / c->T)
                             : 0.f;
  const float z_coef = (float)((double)zloss_grad * 2.0 * zloss_beta / c->T);
  return hip_status(moe::launch_route_bwd(c->dtype, x, w->w_router, logits, idx, tw, dtw, counts,
                                          aux_coef, z_coef, dl ? dl : rw.dl, rw.part,
                                          g->d_w_router, g->d_b_router, d_x_router, c->T,
                                          c->d_model, c->n_experts, c->top_k, s),
                    "moe_route_backward launch");
}

int check_grads(const moe_config_t* c, const moe_grads_t* g, bool router, bool experts) {
  if (!g) return fail(MOE_ERR_INVALID_ARG, "grads is NULL");
  if (router) {
    MOE_REQUIRE_PTR(g->d_w_router, "d_w_router");
    MOE_OPTIONAL_PTR(g->d_b_router, "d_b_router");
  }
  if (experts) {
    MOE_REQUIRE_PTR(g->d_w1, "d_w1");
    MOE_REQUIRE_PTR(g->d_w2, "d_w2");
    MOE_OPTIONAL_PTR(g->d_b1, "d_b1");
    MOE_OPTIONAL_PTR(g->d_b2, "d_b2");
    if (c->d_ff_shared) {
      MOE_REQUIRE_PTR(g->d_ws1, "d_ws1");
      MOE_REQUIRE_PTR(g->d_ws2, "d_ws2");
    }
  }
  return MOE_OK;
}

int check_saved(const moe_config_t* c, const moe_saved_t* sv) {
  if (!sv) return fail(MOE_ERR_INVALID_ARG, "saved is NULL");
  MOE_REQUIRE_PTR(sv->logits, "saved.logits");
  MOE_REQUIRE_PTR(sv->topk_idx, "saved.topk_idx");
  MOE_REQUIRE_PTR(sv->topk_w, "saved.topk_w");
  MOE_REQUIRE_PTR(sv->counts, "saved.counts");
  MOE_REQUIRE_PTR(sv->expert_offsets, "saved.expert_offsets");
  MOE_REQUIRE_PTR(sv->slot_row, "saved.slot_row");
  MOE_REQUIRE_PTR(sv->row_token, "saved.row_token");
  MOE_REQUIRE_PTR(sv->n_dropped, "saved.n_dropped");
  MOE_REQUIRE_PTR(sv->x_perm, "saved.x_perm");
  MOE_REQUIRE_PTR(sv->z, "saved.z");
  MOE_REQUIRE_PTR(sv->h, "saved.h");
  MOE_REQUIRE_PTR(sv->y_perm, "saved.y_perm");
  if (c->d_ff_shared) {
    MOE_REQUIRE_PTR(sv->zs, "saved.zs");
    MOE_REQUIRE_PTR(sv->hs, "saved.hs");
  }
  return MOE_OK;
}

// The whole layer on a caller-sized workspace (moe_layer_forward and
// moe_layer_forward_noalloc).
// The routing partials are written by the select kernel while it holds each
// token's logits, so the aux loss, the z-loss and the mean routing weights
// only reduce them (no further pass over the logits).
int layer_forward(const moe_config_t* cfg, const void* x, const moe_weights_t* w, void* out,
                  const moe_layer_stats_t& st, void* ws, size_t ws_bytes, hipStream_t stream) {
  int r = check_ws(cfg, MOE_STAGE_LAYER, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  LayerWs lw;
  carve_layer(cv, cfg, &lw);
  int32_t* counts = st.counts_out ? st.counts_out : lw.counts;
  int32_t* ndrop = st.n_dropped_out ? st.n_dropped_out : lw.n_dropped;
  const bool parts = st.aux_out || st.zloss_out || st.weight_mean_out;

  r = do_route(cfg, x, w, lw.logits, lw.idx, lw.w, lw.route, stream,
               parts ? &lw.aux.rp : nullptr);
  if (r != MOE_OK) return r;
  r = do_dispatch(cfg, lw.idx, x, counts, lw.offsets, lw.slot_row, lw.row_token, lw.x_perm,
                  ndrop, lw.disp, stream);
  if (r != MOE_OK) return r;
  r = do_ffn(cfg, lw.x_perm, lw.offsets, w, x, lw.y_perm, lw.y_shared, lw.ffn, stream, lw.ffn.h,
             lw.ffn.h_shared);
  if (r != MOE_OK) return r;
  r = do_combine(cfg, lw.y_perm, lw.slot_row, lw.w, lw.y_shared, out, stream);
  if (r != MOE_OK) return r;
  if (st.aux_out) {
    r = do_aux(cfg, nullptr, lw.aux.rp, counts, st.aux_out, lw.aux, stream);
    if (r != MOE_OK) return r;
  }
  if (st.zloss_out) {
    r = hip_status(moe::launch_zloss_final(lw.aux.rp, cfg->T, st.zloss_beta, st.zloss_out, stream),
                   "z-loss launch");
    if (r != MOE_OK) return r;
  }
  if (st.weight_mean_out) {
    r = hip_status(moe::launch_stats_final(lw.aux.rp, cfg->T, cfg->n_experts, nullptr,
                                           st.weight_mean_out, stream),
                   "routing statistics launch");
    if (r != MOE_OK) return r;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- allocation-free layer
// The address of `scratch` (above) on each device, taken once per device on
// moe_layer_forward_noalloc's first call there.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (nullptr with the error recorded
// on failure).
void* scratch_for_current_device(int* code) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *code = fail(MOE_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *code = fail(MOE_ERR_UNSUPPORTED, "device index beyond the library's scratch table");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *code = fail(MOE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                    (e != hipSuccess ? hipGetErrorString(e) : "null address"));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_config_t* cfg, moe_stage_t stage) {
  int code;
  if (!check_config(cfg, &code).empty()) return (size_t)-1;
  if ((int)stage < MOE_STAGE_ROUTE || (int)stage > MOE_STAGE_LAYER_BACKWARD) return (size_t)-1;
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

int moe_router_path(const moe_config_t* cfg) {
  int code;
  if (!check_config(cfg, &code).empty()) return -1;
  return router_certified(cfg) ? MOE_ROUTER_CERTIFIED : MOE_ROUTER_EXACT;
}

size_t moe_route_partials_size(const moe_config_t* cfg) {
  int code;
  if (!check_config(cfg, &code).empty()) return (size_t)-1;
  return part_layout(cfg).total;
}

int moe_route(const moe_config_t* cfg, const void* x, const moe_weights_t* w, float* logits,
              int32_t* topk_idx, float* topk_w, void* partials, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(x, "x");
  int r = check_weights(cfg, w, true, false);
  if (r != MOE_OK) return r;
  MOE_OPTIONAL_PTR(logits, "logits");
  MOE_REQUIRE_PTR(topk_idx, "topk_idx");
  MOE_REQUIRE_PTR(topk_w, "topk_w");
  if (partials && reinterpret_cast<uintptr_t>(partials) % kAlign)
    return fail(MOE_ERR_INVALID_ARG, "partials must be 256-byte aligned");
  r = check_ws(cfg, MOE_STAGE_ROUTE, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  RouteWs rw;
  carve_route(cv, cfg, &rw);
  if (!partials) return do_route(cfg, x, w, logits, topk_idx, topk_w, rw, stream);
  const moe::RoutePartials rp = partials_at(partials, cfg);
  return do_route(cfg, x, w, logits, topk_idx, topk_w, rw, stream, &rp);
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
  return do_ffn(cfg, x_perm, expert_offsets, w, x, y_perm, y_shared, fw, stream, fw.h, fw.h_shared);
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

// Exactly one of logits / partials.
int check_logits_or_partials(const float* logits, const void* partials) {
  if (!logits == !partials)
    return fail(MOE_ERR_INVALID_ARG, "pass exactly one of logits and partials");
  MOE_OPTIONAL_PTR(logits, "logits");
  if (partials && reinterpret_cast<uintptr_t>(partials) % kAlign)
    return fail(MOE_ERR_INVALID_ARG, "partials must be 256-byte aligned");
  return MOE_OK;
}

int moe_aux_loss(const moe_config_t* cfg, const float* logits, const void* partials,
                 const int32_t* counts, float* loss_out, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  int r = check_logits_or_partials(logits, partials);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(counts, "counts");
  if (!loss_out) return fail(MOE_ERR_INVALID_ARG, "loss_out is NULL");
  r = check_ws(cfg, MOE_STAGE_AUX, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  AuxWs aw;
  carve_aux(cv, cfg, &aw);
  const moe::RoutePartials rp = partials ? partials_at(const_cast<void*>(partials), cfg) : aw.rp;
  return do_aux(cfg, logits, rp, counts, loss_out, aw, stream);
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

int moe_quantize_int4(const void* w, int32_t dtype, int64_t rows, int32_t cols, uint8_t* q,
                      float* scale, hipStream_t stream) {
  MOE_REQUIRE_PTR(w, "w");
  MOE_REQUIRE_PTR(q, "q");
  MOE_REQUIRE_PTR(scale, "scale");
  if (dtype != MOE_F32 && dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_F32 or MOE_BF16");
  if (rows < 1) return fail(MOE_ERR_INVALID_ARG, "rows must be >= 1");
  if (cols < 64 || cols % 64) return fail(MOE_ERR_INVALID_ARG, "cols must be a positive multiple of 64");
  return hip_status(moe::launch_quantize_int4(w, dtype, rows, cols, q, scale, stream),
                    "moe_quantize_int4 launch");
}

int moe_routing_stats(const moe_config_t* cfg, const int32_t* topk_idx, const float* topk_w,
                      const void* partials, int32_t* counts_out, float* weight_mean_out, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  if (partials) {
    if (topk_idx || topk_w)
      return fail(MOE_ERR_INVALID_ARG, "pass either topk_idx and topk_w or partials");
    if (reinterpret_cast<uintptr_t>(partials) % kAlign)
      return fail(MOE_ERR_INVALID_ARG, "partials must be 256-byte aligned");
  } else {
    MOE_REQUIRE_PTR(topk_idx, "topk_idx");
    MOE_REQUIRE_PTR(topk_w, "topk_w");
  }
  MOE_OPTIONAL_PTR(counts_out, "counts_out");
  if (!weight_mean_out) return fail(MOE_ERR_INVALID_ARG, "weight_mean_out is NULL");
  int r = check_ws(cfg, MOE_STAGE_AUX, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  AuxWs aw;
  carve_aux(cv, cfg, &aw);
  moe::RoutePartials rp = aw.rp;
  if (partials) {
    rp = partials_at(const_cast<void*>(partials), cfg);
  } else {
    r = hip_status(moe::launch_routing_partials(topk_idx, topk_w, cfg->T, cfg->top_k,
                                                cfg->n_experts, rp, stream),
                   "routing statistics partials launch");
    if (r != MOE_OK) return r;
  }
  return hip_status(moe::launch_stats_final(rp, cfg->T, cfg->n_experts, counts_out,
                                            weight_mean_out, stream),
                    "moe_routing_stats launch");
}

int moe_router_z_loss(const moe_config_t* cfg, const float* logits, const void* partials,
                      float beta, float* loss_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  int r = check_logits_or_partials(logits, partials);
  if (r != MOE_OK) return r;
  if (!loss_out) return fail(MOE_ERR_INVALID_ARG, "loss_out is NULL");
  if (!isfinite(beta)) return fail(MOE_ERR_INVALID_ARG, "beta is not finite");
  r = check_ws(cfg, MOE_STAGE_AUX, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  AuxWs aw;
  carve_aux(cv, cfg, &aw);
  moe::RoutePartials rp = aw.rp;
  if (partials) {
    rp = partials_at(const_cast<void*>(partials), cfg);
  } else {
    r = hip_status(moe::launch_logit_partials(logits, cfg->T, cfg->n_experts, rp, stream),
                   "z-loss partials launch");
    if (r != MOE_OK) return r;
  }
  return hip_status(moe::launch_zloss_final(rp, cfg->T, beta, loss_out, stream),
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
  const moe_layer_stats_t st{aux_out, 0.f, nullptr, counts_out, n_dropped_out, nullptr};
  return layer_forward(cfg, x, w, out, st, ws, ws_bytes, stream);
}

int moe_layer_forward_stats(const moe_config_t* cfg, const void* x, const moe_weights_t* w,
                            void* out, const moe_layer_stats_t* stats, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(x, "x");
  int r = check_weights(cfg, w, true, true);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(out, "out");
  if (!stats) return fail(MOE_ERR_INVALID_ARG, "stats is NULL");
  MOE_OPTIONAL_PTR(stats->counts_out, "stats.counts_out");
  MOE_OPTIONAL_PTR(stats->weight_mean_out, "stats.weight_mean_out");
  if (stats->zloss_out && !isfinite(stats->zloss_beta))
    return fail(MOE_ERR_INVALID_ARG, "stats.zloss_beta is not finite");
  return layer_forward(cfg, x, w, out, *stats, ws, ws_bytes, stream);
}

int moe_layer_forward_noalloc(const moe_config_t* cfg, const void* x, const moe_weights_t* w,
                              void* out, float* aux_out, int32_t* counts_out,
                              int32_t* n_dropped_out, hipStream_t stream) {
  MOE_CHECK_CFG(cfg);
  MOE_REQUIRE_PTR(x, "x");
  int r = check_weights(cfg, w, true, true);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(out, "out");
  MOE_OPTIONAL_PTR(counts_out, "counts_out");
  const size_t need = stage_bytes(cfg, MOE_STAGE_LAYER);
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "moe_layer_forward_noalloc: this layer needs " + std::to_string(need) +
                    " bytes of workspace, more than the " + std::to_string(kScratchBytes) +
                    " bytes of device scratch the library holds (use moe_layer_forward)");
  int code = MOE_OK;
  void* ptr = scratch_for_current_device(&code);
  if (!ptr) return code;
  const moe_layer_stats_t st{aux_out, 0.f, nullptr, counts_out, n_dropped_out, nullptr};
  return layer_forward(cfg, x, w, out, st, ptr, kScratchBytes, stream);
}

// ---------------------------------------------------------------- training entry points
int moe_expert_ffn_train(const moe_config_t* cfg, const void* x_perm,
                         const int32_t* expert_offsets, const moe_weights_t* w, const void* x,
                         void* z, void* h, void* y_perm, void* zs, void* hs, void* y_shared,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_TRAIN(cfg);
  MOE_REQUIRE_PTR(x_perm, "x_perm");
  MOE_REQUIRE_PTR(expert_offsets, "expert_offsets");
  int r = check_weights(cfg, w, false, true);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(z, "z");
  MOE_REQUIRE_PTR(h, "h");
  MOE_REQUIRE_PTR(y_perm, "y_perm");
  if (cfg->d_ff_shared) {
    MOE_REQUIRE_PTR(x, "x");
    MOE_REQUIRE_PTR(zs, "zs");
    MOE_REQUIRE_PTR(hs, "hs");
    MOE_REQUIRE_PTR(y_shared, "y_shared");
  } else if (y_shared || zs || hs) {
    return fail(MOE_ERR_INVALID_ARG, "shared-expert buffers given but the layer has none");
  }
  r = check_ws(cfg, MOE_STAGE_EXPERT_FFN_TRAIN, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  FfnWs fw;
  carve_ffn(cv, cfg, &fw, false);
  return do_ffn(cfg, x_perm, expert_offsets, w, x, y_perm, y_shared, fw, stream, h, hs, z, zs);
}

int moe_layer_forward_train(const moe_config_t* cfg, const void* x, const moe_weights_t* w,
                            void* out, float* aux_out, const moe_saved_t* saved, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_TRAIN(cfg);
  MOE_REQUIRE_PTR(x, "x");
  int r = check_weights(cfg, w, true, true);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(out, "out");
  r = check_saved(cfg, saved);
  if (r != MOE_OK) return r;
  r = check_ws(cfg, MOE_STAGE_LAYER_TRAIN, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  LayerTrainWs lw;
  carve_layer_train(cv, cfg, &lw);
  const moe_saved_t& sv = *saved;
  r = do_route(cfg, x, w, sv.logits, sv.topk_idx, sv.topk_w, lw.route, stream,
               aux_out ? &lw.aux.rp : nullptr);
  if (r != MOE_OK) return r;
  r = do_dispatch(cfg, sv.topk_idx, x, sv.counts, sv.expert_offsets, sv.slot_row, sv.row_token,
                  sv.x_perm, sv.n_dropped, lw.disp, stream);
  if (r != MOE_OK) return r;
  r = do_ffn(cfg, sv.x_perm, sv.expert_offsets, w, x, sv.y_perm, lw.y_shared, lw.ffn, stream,
             sv.h, sv.hs, sv.z, sv.zs);
  if (r != MOE_OK) return r;
  r = do_combine(cfg, sv.y_perm, sv.slot_row, sv.topk_w, lw.y_shared, out, stream);
  if (r != MOE_OK) return r;
  if (aux_out) return do_aux(cfg, nullptr, lw.aux.rp, sv.counts, aux_out, lw.aux, stream);
  return MOE_OK;
}

int moe_combine_backward(const moe_config_t* cfg, const void* d_out, const void* y_perm,
                         const int32_t* slot_row, const float* topk_w, void* d_y_perm,
                         float* d_topk_w, hipStream_t stream) {
  MOE_CHECK_TRAIN(cfg);
  MOE_REQUIRE_PTR(d_out, "d_out");
  MOE_REQUIRE_PTR(y_perm, "y_perm");
  MOE_REQUIRE_PTR(slot_row, "slot_row");
  MOE_REQUIRE_PTR(topk_w, "topk_w");
  MOE_REQUIRE_PTR(d_y_perm, "d_y_perm");
  MOE_REQUIRE_PTR(d_topk_w, "d_topk_w");
  return do_combine_bwd(cfg, d_out, y_perm, slot_row, topk_w, d_y_perm, d_topk_w, stream);
}

int moe_expert_ffn_backward(const moe_config_t* cfg, const void* x_perm,
                            const int32_t* expert_offsets, const moe_weights_t* w, const void* x,
                            const void* z, const void* h, const void* zs, const void* hs,
                            const void* d_y_perm, const void* d_out, void* d_x_perm,
                            void* d_x_shared, const moe_grads_t* grads, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  MOE_CHECK_TRAIN(cfg);
  MOE_REQUIRE_PTR(x_perm, "x_perm");
  MOE_REQUIRE_PTR(expert_offsets, "expert_offsets");
  int r = check_weights(cfg, w, false, true);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(z, "z");
  MOE_REQUIRE_PTR(h, "h");
  MOE_REQUIRE_PTR(d_y_perm, "d_y_perm");
  MOE_REQUIRE_PTR(d_x_perm, "d_x_perm");
  if (cfg->d_ff_shared) {
    MOE_REQUIRE_PTR(x, "x");
    MOE_REQUIRE_PTR(zs, "zs");
    MOE_REQUIRE_PTR(hs, "hs");
    MOE_REQUIRE_PTR(d_out, "d_out");
    MOE_REQUIRE_PTR(d_x_shared, "d_x_shared");
  } else if (d_x_shared) {
    return fail(MOE_ERR_INVALID_ARG, "d_x_shared given but the layer has no shared expert");
  }
  r = check_grads(cfg, grads, false, true);
  if (r != MOE_OK) return r;
  r = check_ws(cfg, MOE_STAGE_EXPERT_FFN_BACKWARD, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  FfnBwdWs fw;
  carve_ffn_bwd(cv, cfg, &fw);
  return do_ffn_bwd(cfg, x_perm, expert_offsets, w, x, z, h, zs, hs, d_y_perm, d_out, d_x_perm,
                    d_x_shared, grads, fw, stream);
}

int moe_route_backward(const moe_config_t* cfg, const void* x, const moe_weights_t* w,
                       const float* logits, const int32_t* topk_idx, const float* topk_w,
                       const float* d_topk_w, const int32_t* counts, float aux_grad,
                       float zloss_beta, float zloss_grad, float* d_logits, float* d_x_router,
                       const moe_grads_t* grads, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_TRAIN(cfg);
  MOE_REQUIRE_PTR(x, "x");
  int r = check_weights(cfg, w, true, false);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(logits, "logits");
  MOE_REQUIRE_PTR(topk_idx, "topk_idx");
  MOE_REQUIRE_PTR(topk_w, "topk_w");
  MOE_REQUIRE_PTR(d_topk_w, "d_topk_w");
  if (!isfinite(aux_grad) || !isfinite(zloss_beta) || !isfinite(zloss_grad))
    return fail(MOE_ERR_INVALID_ARG, "aux_grad, zloss_beta and zloss_grad must be finite");
  if (cfg->aux_alpha != 0.f && aux_grad != 0.f) MOE_REQUIRE_PTR(counts, "counts");
  MOE_OPTIONAL_PTR(d_logits, "d_logits");
  MOE_OPTIONAL_PTR(d_x_router, "d_x_router");
  r = check_grads(cfg, grads, true, false);
  if (r != MOE_OK) return r;
  r = check_ws(cfg, MOE_STAGE_ROUTE_BACKWARD, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  RouteBwdWs rw;
  carve_route_bwd(cv, cfg, &rw);
  return do_route_bwd(cfg, x, w, logits, topk_idx, topk_w, d_topk_w, counts, aux_grad, zloss_beta,
                      zloss_grad, d_logits, d_x_router, grads, rw, stream);
}

int moe_dispatch_backward(const moe_config_t* cfg, const void* d_x_perm, const int32_t* slot_row,
                          const void* d_x_shared, const float* d_x_router, void* d_x,
                          hipStream_t stream) {
  MOE_CHECK_TRAIN(cfg);
  MOE_REQUIRE_PTR(d_x_perm, "d_x_perm");
  MOE_REQUIRE_PTR(slot_row, "slot_row");
  MOE_OPTIONAL_PTR(d_x_shared, "d_x_shared");
  MOE_OPTIONAL_PTR(d_x_router, "d_x_router");
  MOE_REQUIRE_PTR(d_x, "d_x");
  return hip_status(moe::launch_unpermute(cfg->dtype, d_x_perm, slot_row, d_x_shared, d_x_router,
                                          d_x, cfg->T, cfg->d_model, cfg->top_k, stream),
                    "moe_dispatch_backward launch");
}

int moe_layer_backward(const moe_config_t* cfg, const void* x, const moe_weights_t* w,
                       const moe_saved_t* saved, const void* d_out, float aux_grad,
                       float zloss_beta, float zloss_grad, void* d_x, const moe_grads_t* grads,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_CHECK_TRAIN(cfg);
  MOE_REQUIRE_PTR(x, "x");
  int r = check_weights(cfg, w, true, true);
  if (r != MOE_OK) return r;
  r = check_saved(cfg, saved);
  if (r != MOE_OK) return r;
  MOE_REQUIRE_PTR(d_out, "d_out");
  MOE_REQUIRE_PTR(d_x, "d_x");
  if (!isfinite(aux_grad) || !isfinite(zloss_beta) || !isfinite(zloss_grad))
    return fail(MOE_ERR_INVALID_ARG, "aux_grad, zloss_beta and zloss_grad must be finite");
  r = check_grads(cfg, grads, true, true);
  if (r != MOE_OK) return r;
  r = check_ws(cfg, MOE_STAGE_LAYER_BACKWARD, ws, ws_bytes);
  if (r != MOE_OK) return r;
  Carver cv{static_cast<char*>(ws)};
  LayerBwdWs lw;
  carve_layer_bwd(cv, cfg, &lw);
  const moe_saved_t& sv = *saved;
  r = do_combine_bwd(cfg, d_out, sv.y_perm, sv.slot_row, sv.topk_w, lw.d_y_perm, lw.d_topk_w,
                     stream);
  if (r != MOE_OK) return r;
  r = do_ffn_bwd(cfg, sv.x_perm, sv.expert_offsets, w, x, sv.z, sv.h, sv.zs, sv.hs, lw.d_y_perm,
                 d_out, lw.d_x_perm, lw.d_x_shared, grads, lw.ffn, stream);
  if (r != MOE_OK) return r;
  r = do_route_bwd(cfg, x, w, sv.logits, sv.topk_idx, sv.topk_w, lw.d_topk_w, sv.counts, aux_grad,
                   zloss_beta, zloss_grad, nullptr, lw.d_x_router, grads, lw.route, stream);
  if (r != MOE_OK) return r;
  return hip_status(moe::launch_unpermute(cfg->dtype, lw.d_x_perm, sv.slot_row, lw.d_x_shared,
                                          lw.d_x_router, d_x, cfg->T, cfg->d_model, cfg->top_k,
                                          stream),
                    "unpermute launch");
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
