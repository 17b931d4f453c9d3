// C ABI of the MoE layer forward: argument checks, workspace carve-up and the
// launch sequence.  Every check runs on the host before any HIP call; on an
// error nothing is enqueued.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <functional>

#include "../../include/moe.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_bytes(moe_dtype_t dt) { return dt == MOE_BF16 ? 2 : 4; }

bool dtype_ok(moe_dtype_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }
bool act_ok(moe_act_t a) { return a == MOE_ACT_GELU || a == MOE_ACT_SWIGLU; }

// Workspace carve-up from an (aligned-up) base.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base((char*)p) {
    if (base) base = (char*)(((uintptr_t)base + kAlign - 1) & ~(uintptr_t)(kAlign - 1));
  }
  template <typename T> T* take(size_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += align_up(count * sizeof(T));
    return p;
  }
  size_t bytes() const { return off + kAlign; }  // + slack for aligning the base
};

int64_t capacity_of(int32_t T, int32_t E, int32_t k, float cf) {
  const double c = (double)cf;
  if (!(c > 0.0)) return INT32_MAX;
  const double tpe = (double)((int64_t)k * T) / (double)E;
  const double C = floor(c * tpe);
  if (C < 1.0) return INT32_MAX;
  if (C >= (double)INT32_MAX) return INT32_MAX;
  return (int64_t)C;
}

int rows_max(int32_t T, int32_t E, int32_t k, int64_t C) {
  const int64_t n = (int64_t)T * k;
  if (C == INT32_MAX) return (int)n;
  const int64_t cap = C * E;
  return (int)(cap < n ? cap : n);
}

// Tile height and K splits of the layer's expert GEMMs: from the rows an expert receives
// on average (T k / E, at most the capacity).
FfnPlan layer_plan(bool bf, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, int64_t C) {
  double rpe = (double)T * k / E;
  if (C != INT32_MAX && (double)C < rpe) rpe = (double)C;
  return plan_ffn(bf, rpe, E, rows_max(T, E, k, C), h, f);
}

// Fixed-capacity buckets: the bucket size when it is known on the host (cf > 0:
// max(floor(cf * T * k / E), min_capacity)), INT32_MAX when it is the largest count of
// the step (cf <= 0 or a computed zero); and the bound the buffers are sized for.
int64_t binned_cfixed(int32_t T, int32_t E, int32_t k, float cf, int32_t min_capacity) {
  const double c = (double)cf;
  if (!(c > 0.0)) return INT32_MAX;
  double C = floor(c * ((double)((int64_t)k * T) / (double)E));
  if (C < (double)min_capacity) C = (double)min_capacity;
  if (C < 1.0) return INT32_MAX;
  if (C >= (double)INT32_MAX) return INT32_MAX - 1;
  return (int64_t)C;
}

int64_t binned_cmax(int32_t T, int32_t E, int32_t k, float cf, int32_t min_capacity) {
  const int64_t C = binned_cfixed(T, E, k, cf, min_capacity);
  return C == INT32_MAX ? (int64_t)T : C;  // an expert gets at most one assignment per token
}

moe_status_t common_sizes(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_ARG;
  if ((int64_t)T * k > (int64_t)INT32_MAX / 2) return MOE_ERR_ARG;
  if (E > 256 || k > 16) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The expert GEMMs address their left operand with 32-bit element offsets (row * K):
// x (T rows of h) in the gathered up projection, x_perm (R_max rows of h) and Hm (R_max
// rows of f).  Sizes where one of those products reaches 2^32 are refused.
moe_status_t rows_ok(int64_t rows, int32_t h, int32_t f) {
  if (rows * (int64_t)(h > f ? h : f) >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t dim_ok(int32_t d) {
  if (d <= 0) return MOE_ERR_ARG;
  if (d % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// rows_ok for the layer: the larger of T and R_max rows
moe_status_t size_ok(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, float cf) {
  const int64_t R_max = rows_max(T, E, k, capacity_of(T, E, k, cf));
  return rows_ok(R_max > T ? R_max : (int64_t)T, h, f);
}

// --- workspace layouts (the same carve is used to size and to place)
struct RouteWs { float* prob_part; uint16_t* planes; };
RouteWs carve_route(Carve& c, int32_t T, int32_t h, int32_t E, bool prob, bool planes) {
  RouteWs w;
  w.prob_part = prob ? c.take<float>((size_t)route_blocks(T) * E) : nullptr;
  w.planes = planes ? (uint16_t*)c.take<char>(route_scratch_bytes(T, h, E, true)) : nullptr;
  return w;
}

struct PermWs { int* blk_counts; int* blk_base; int* perm_token; };
PermWs carve_perm(Carve& c, int32_t T, int32_t E, int32_t k) {
  PermWs w;
  const size_t nhb = (size_t)route_blocks(T);
  w.blk_counts = c.take<int>(nhb * E);
  w.blk_base = c.take<int>(nhb * E);
  w.perm_token = c.take<int>((size_t)T * k);
  return w;
}

size_t up_cols(moe_act_t act, int32_t f) { return (size_t)(act == MOE_ACT_SWIGLU ? 2 : 1) * f; }

// Few rows per expert (32-row tiles, the weight-streaming case), bf16 SwiGLU, one K part:
// the up projection writes its raw accumulators [a | g] from tiles of 512 columns of W1
// alone or W3 alone -- 1 KiB weight runs instead of two 512-byte runs -- and
// launch_ffn_finish applies the activation.  (Measured at 16 rows per expert, h = 4096,
// f = 14336, E = 8: the up projection with its finishing pass takes 0.314 ms instead of
// 0.324 ms, the layer 0.484 instead of 0.491 ms.)
bool sep_up(const FfnPlan& pl, moe_act_t act, moe_dtype_t dt) {
  return dt == MOE_BF16 && act == MOE_ACT_SWIGLU && pl.bm == 32 && pl.s_up <= 1;
}
// fp32 parts of the up projection in the workspace (0: it writes Hm directly)
int up_parts(const FfnPlan& pl, moe_act_t act, moe_dtype_t dt) {
  return pl.s_up > 1 ? pl.s_up : (sep_up(pl, act, dt) ? 1 : 0);
}

struct FfnWs { int* tile_off; void* hm; float* part_up; float* part_down; };
FfnWs carve_ffn(Carve& c, const FfnPlan& pl, int R_max, int32_t h, int32_t f, int32_t E, moe_dtype_t dt,
                moe_act_t act) {
  FfnWs w;
  w.tile_off = c.take<int>((size_t)E + 1);
  w.hm = c.take<char>((size_t)R_max * f * elem_bytes(dt));
  w.part_up = up_parts(pl, act, dt) ? c.take<float>((size_t)up_parts(pl, act, dt) * R_max * up_cols(act, f)) : nullptr;
  w.part_down = pl.s_down > 1 ? c.take<float>((size_t)pl.s_down * R_max * h) : nullptr;
  return w;
}

struct LayerWs {
  uint16_t* planes;
  float* logits; int* topk_idx; float* topk_w; float* prob_part; int* blk_counts; int* blk_base;
  int* counts; int* offsets; int* tile_off; float* aux; int* slot_pos; int* sorted_slot;
  int* perm_token; void* hm; float* part_up; float* o;
};
LayerWs carve_layer(Carve& c, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, int R_max,
                    const FfnPlan& pl, moe_dtype_t dt, moe_act_t act) {
  LayerWs w;
  const size_t n = (size_t)T * k;
  const size_t nhb = (size_t)route_blocks(T);
  w.planes = dt == MOE_BF16 ? (uint16_t*)c.take<char>(route_scratch_bytes(T, h, E, true)) : nullptr;
  w.logits = c.take<float>((size_t)T * E);
  w.topk_idx = c.take<int>(n);
  w.topk_w = c.take<float>(n);
  // per histogram block (16 or kSelTokens tokens: route_hist_tokens)
  const size_t nhist = (size_t)route_hist_blocks(T, h, E, dt == MOE_BF16);
  w.prob_part = c.take<float>(nhist * E);
  w.blk_counts = c.take<int>(nhist * E);
  w.blk_base = c.take<int>(nhb * E);
  w.counts = c.take<int>(E);
  w.offsets = c.take<int>((size_t)E + 1);
  w.tile_off = c.take<int>((size_t)E + 1);
  w.aux = c.take<float>(1);
  w.slot_pos = c.take<int>(n);
  // indexed by row: the fixed-capacity layout may have more rows than assignments
  const size_t rows = (size_t)R_max > n ? (size_t)R_max : n;
  w.sorted_slot = c.take<int>(rows);
  w.perm_token = c.take<int>(rows);
  w.hm = c.take<char>((size_t)R_max * f * elem_bytes(dt));
  w.part_up = up_parts(pl, act, dt) ? c.take<float>((size_t)up_parts(pl, act, dt) * R_max * up_cols(act, f)) : nullptr;
  // expert outputs stay fp32 until the combine (s_down K parts of them when the down
  // projection is split; the combine adds the parts)
  w.o = c.take<float>((size_t)pl.s_down * R_max * h);
  return w;
}

#define MOE_TRY(expr)                               \
  do {                                              \
    if ((expr) != hipSuccess) return MOE_ERR_DEVICE; \
  } while (0)

struct BinnedWs { LayerWs l; int* cap; void* x_bins; };
BinnedWs carve_binned(Carve& c, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, int R_max, const FfnPlan& pl,
                      moe_dtype_t dt, moe_act_t act, bool own_bins) {
  BinnedWs w;
  w.l = carve_layer(c, T, h, f, E, k, R_max, pl, dt, act);
  w.cap = c.take<int>(1);
  w.x_bins = own_bins ? c.take<char>((size_t)R_max * h * elem_bytes(dt)) : nullptr;
  return w;
}

// The two expert GEMMs.  up: A (rows through a_rows) x W1 (and W3) -> act -> hm.
// down: hm x W2 -> out (fp32 when out_f32, else dt).  With a K-split down projection and
// out_parts set, the fp32 parts stay in part_down (== out) for the combine to add;
// otherwise they are added into out here.
moe_status_t run_ffn(const void* A, const int* a_rows, const int* offsets, const int* tile_off, const FfnPlan& pl,
                     int R_max, int32_t h, int32_t f, int32_t E, const void* W1, const void* W3, const void* W2,
                     moe_act_t act, moe_dtype_t dt, void* hm, float* part_up, void* out, bool out_f32,
                     float* part_down, bool out_parts, hipStream_t st,
                     const std::function<bool()>& mark = std::function<bool()>(), float* save = nullptr) {
  const bool bf = dt == MOE_BF16;
  const int gact = act == MOE_ACT_SWIGLU ? ACT_SWIGLU : ACT_GELU;
  GemmArgs up{};
  up.A = A;
  up.a_rows = a_rows;
  up.W = W1;
  up.W3 = act == MOE_ACT_SWIGLU ? W3 : nullptr;
  up.K = h;
  up.N = f;
  const bool sep = sep_up(pl, act, dt);
  up.out = pl.s_up > 1 || sep ? (void*)part_up : hm;
  up.offsets = offsets;
  up.tile_off = tile_off;
  up.E = E;
  up.R_max = R_max;
  up.bm = pl.bm;
  up.big = pl.big;
  up.ksplit = pl.s_up;
  up.act = gact;
  up.save = bf && pl.s_up <= 1 && !sep ? save : nullptr;  // bf16 only (fp32: the caller runs preact_gemms)
  up.raw = sep;
  up.sep = sep;
  MOE_TRY(launch_gemm(up, bf, st));
  if (pl.s_up > 1 || sep)
    MOE_TRY(launch_ffn_finish(part_up, pl.s_up > 1 ? pl.s_up : 1, R_max, f, gact, offsets, E, bf, hm, st,
                              bf ? save : nullptr));
  if (mark && !mark()) return MOE_ERR_DEVICE;
  GemmArgs down = up;
  down.save = nullptr;
  down.raw = false;
  down.sep = false;
  down.A = hm;
  down.a_rows = nullptr;
  down.W = W2;
  down.W3 = nullptr;
  down.K = f;
  down.N = h;
  down.out = pl.s_down > 1 ? (void*)part_down : out;
  down.act = ACT_NONE;
  down.out_f32 = out_f32;
  down.ksplit = pl.s_down;
  MOE_TRY(launch_gemm(down, bf, st));
  if (pl.s_down > 1 && !out_parts)
    MOE_TRY(launch_ffn_finish(part_down, pl.s_down, R_max, h, ACT_NONE, offsets, E, bf && !out_f32, out, st));
  if (mark && !mark()) return MOE_ERR_DEVICE;
  return MOE_OK;
}

// The up projection's pre-activations a (| g) as raw fp32 GEMM outputs, into `ag`:
// bf16 [R_max][n_up * f] (a then g in each row), fp32 [n_up][R_max][f].
moe_status_t preact_gemms(const void* A, const int* a_rows, const int* offsets, const int* tile_off,
                          const FfnPlan& pl, int R_max, int32_t h, int32_t f, int32_t E, const void* W1,
                          const void* W3, moe_act_t act, bool bf, float* ag, hipStream_t st) {
  GemmArgs up{};
  up.A = A;
  up.a_rows = a_rows;
  up.K = h;
  up.N = f;
  up.offsets = offsets;
  up.tile_off = tile_off;
  up.E = E;
  up.R_max = R_max;
  up.bm = pl.bm;
  up.big = pl.big;
  up.ksplit = 1;
  up.W = W1;
  up.out = ag;
  if (bf) {
    up.W3 = act == MOE_ACT_SWIGLU ? W3 : nullptr;
    up.act = act == MOE_ACT_SWIGLU ? ACT_SWIGLU : ACT_GELU;
    up.raw = true;
    MOE_TRY(launch_gemm(up, true, st));
  } else {
    up.act = ACT_NONE;
    MOE_TRY(launch_gemm(up, false, st));
    if (act == MOE_ACT_SWIGLU) {
      up.W = W3;
      up.out = ag + (size_t)R_max * f;
      MOE_TRY(launch_gemm(up, false, st));
    }
  }
  return MOE_OK;
}

size_t preact_bytes(int R_max, int32_t f, moe_act_t act) {
  return (size_t)R_max * (act == MOE_ACT_SWIGLU ? 2 : 1) * f * 4;
}

}  // namespace

extern "C" {

int32_t moe_capacity(int32_t T, int32_t E, int32_t k, float capacity_factor) {
  if (T < 0 || E < 1 || k < 1 || !isfinite(capacity_factor)) return -1;
  return (int32_t)capacity_of(T, E, k, capacity_factor);
}

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported size or alignment";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: kernel launch failed";
  }
  return "unknown moe_status_t";
}

size_t moe_workspace_bytes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, float capacity_factor,
                           moe_dtype_t dt, moe_act_t act) {
  if (common_sizes(T, E, k) != MOE_OK || h <= 0 || f <= 0 || !dtype_ok(dt) || !act_ok(act) ||
      !isfinite(capacity_factor))
    return 0;
  const int64_t C = capacity_of(T, E, k, capacity_factor);
  Carve c(nullptr);
  carve_layer(c, T, h, f, E, k, rows_max(T, E, k, C), layer_plan(dt == MOE_BF16, T, h, f, E, k, C), dt, act);
  return c.bytes();
}

size_t moe_route_workspace_bytes(int32_t T, int32_t h, int32_t E, moe_dtype_t dt, uint32_t flags,
                                 int32_t with_prob_sum) {
  if (T < 0 || E < 1 || E > 256 || h < 0 || !dtype_ok(dt)) return 0;
  const bool lin = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  Carve c(nullptr);
  carve_route(c, T, h, E, with_prob_sum != 0, !lin && dt == MOE_BF16);
  return c.bytes();
}

// ---- router variants (moe_router_opts_t)
static moe_status_t opts_ok(const moe_router_opts_t* o, const void* x, bool logits_in) {
  if (o == nullptr) return MOE_OK;
  if (!isfinite(o->temperature) || !(o->temperature > 0.f)) return MOE_ERR_ARG;
  if (o->jitter != nullptr) {
    if (logits_in) return MOE_ERR_ARG;  // the jitter acts on the router input
    if (!aligned16(o->jitter) || !aligned16(x)) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}
static bool has_jitter(const moe_router_opts_t* o) { return o != nullptr && o->jitter != nullptr; }
static void apply_opts(RouteArgs& a, const moe_router_opts_t* o) {
  if (o == nullptr) return;
  a.noise = o->logit_noise;
  a.inv_temp = 1.0f / o->temperature;
  a.uniform = o->uniform_assignment != 0;
  a.soft = o->soft_topk != 0;
}

static moe_status_t route_impl(const void* x, const float* W_gate, const float* logit_bias, int32_t T, int32_t h,
                               int32_t E, int32_t k, moe_dtype_t dt, uint32_t flags,
                               const moe_router_opts_t* opts, float* logits, int32_t* topk_idx, float* topk_w,
                               float* prob_sum, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t s = common_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (!dtype_ok(dt) || (flags & ~MOE_ROUTE_LOGITS_IN) != 0) return MOE_ERR_ARG;
  const bool lin = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_ARG;
  if (!lin) {
    if (!x || !W_gate) return MOE_ERR_ARG;
    if ((s = dim_ok(h)) != MOE_OK) return s;
  }
  if ((s = opts_ok(opts, x, lin)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  Carve c(ws);
  const bool need_planes = !lin && dt == MOE_BF16 && route_scratch_bytes(T, h, E, true) > 0;
  RouteWs w = carve_route(c, T, h, E, prob_sum != nullptr, need_planes);
  void* xj = has_jitter(opts) ? c.take<char>((size_t)T * h * elem_bytes(dt)) : nullptr;
  if ((prob_sum || need_planes || has_jitter(opts)) && (!ws || ws_bytes < c.bytes())) return MOE_ERR_WORKSPACE;
  RouteArgs a{};
  a.x = x;
  a.W_gate = W_gate;
  a.bias = logit_bias;
  a.T = T;
  a.h = h;
  a.E = E;
  a.k = k;
  a.bf16 = dt == MOE_BF16;
  a.logits_in = lin;
  a.logits = logits;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.prob_part = prob_sum ? w.prob_part : nullptr;
  a.blk_counts = nullptr;
  a.planes = w.planes;
  apply_opts(a, opts);
  if (xj != nullptr) {
    MOE_TRY(launch_jitter(x, opts->jitter, (int64_t)T * h, a.bf16, xj, stream));
    a.x = xj;
  }
  MOE_TRY(launch_route(a, stream));
  if (prob_sum) MOE_TRY(launch_reduce_prob(w.prob_part, route_blocks(T), E, prob_sum, stream));
  return MOE_OK;
}

moe_status_t moe_route(const void* x, const float* W_gate, const float* logit_bias, int32_t T, int32_t h,
                       int32_t E, int32_t k, moe_dtype_t dt, uint32_t flags, float* logits,
                       int32_t* topk_idx, float* topk_w, float* prob_sum, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  return route_impl(x, W_gate, logit_bias, T, h, E, k, dt, flags, nullptr, logits, topk_idx, topk_w, prob_sum, ws,
                    ws_bytes, stream);
}

moe_status_t moe_route_ex(const void* x, const float* W_gate, const float* logit_bias, int32_t T, int32_t h,
                          int32_t E, int32_t k, moe_dtype_t dt, uint32_t flags, const moe_router_opts_t* opts,
                          float* logits, int32_t* topk_idx, float* topk_w, float* prob_sum, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  return route_impl(x, W_gate, logit_bias, T, h, E, k, dt, flags, opts, logits, topk_idx, topk_w, prob_sum, ws,
                    ws_bytes, stream);
}

size_t moe_router_opts_workspace_bytes(int32_t T, int32_t h, moe_dtype_t dt, const moe_router_opts_t* opts) {
  if (T < 0 || h < 0 || !dtype_ok(dt) || !has_jitter(opts)) return 0;
  return align_up((size_t)T * h * elem_bytes(dt));
}

size_t moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t k) {
  if (common_sizes(T, E, k) != MOE_OK) return 0;
  Carve c(nullptr);
  carve_perm(c, T, E, k);
  return c.bytes();
}

moe_status_t moe_permute(const int32_t* topk_idx, const void* x, int32_t T, int32_t h, int32_t E, int32_t k,
                         float capacity_factor, moe_dtype_t dt, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_slot, int32_t* slot_pos, void* x_perm, const float* prob_sum,
                         float* aux_loss, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status_t s = common_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (!dtype_ok(dt) || !isfinite(capacity_factor)) return MOE_ERR_ARG;
  if (!topk_idx || !counts || !offsets || !sorted_slot || !slot_pos) return MOE_ERR_ARG;
  if (x_perm) {
    if (!x) return MOE_ERR_ARG;
    if ((s = dim_ok(h)) != MOE_OK) return s;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_UNSUPPORTED;
  }
  if (T == 0) return MOE_OK;
  Carve c(ws);
  PermWs w = carve_perm(c, T, E, k);
  if (!ws || ws_bytes < c.bytes()) return MOE_ERR_WORKSPACE;
  const int64_t C = capacity_of(T, E, k, capacity_factor);
  MOE_TRY(launch_hist(topk_idx, T, k, E, w.blk_counts, stream));
  ScanArgs sa{};
  sa.blk_counts = w.blk_counts;
  sa.nhb = route_blocks(T);
  sa.E = E;
  sa.T = T;
  sa.k = k;
  sa.C = (int)C;
  sa.BM = 0;
  sa.prob_part = nullptr;
  sa.nrb = 0;
  sa.prob_sum = prob_sum;
  sa.counts = counts;
  sa.offsets = offsets;
  sa.blk_base = w.blk_base;
  sa.tile_off = nullptr;
  sa.aux = (prob_sum && aux_loss) ? aux_loss : nullptr;
  if (scan_scatter_fusable(sa.nhb, 0, E)) {
    MOE_TRY(launch_scan_scatter(sa, topk_idx, slot_pos, sorted_slot, w.perm_token, stream));
  } else {
    MOE_TRY(launch_scan(sa, stream));
    MOE_TRY(launch_scatter(topk_idx, T, E, k, (int)C, offsets, w.blk_base, slot_pos, sorted_slot, w.perm_token,
                           stream));
  }
  if (x_perm)
    MOE_TRY(launch_gather(x, w.perm_token, offsets, E, rows_max(T, E, k, C), h, (int)elem_bytes(dt), x_perm,
                          stream));
  return MOE_OK;
}

size_t moe_expert_ffn_workspace_bytes(int32_t R_max, int32_t h, int32_t f, int32_t E, moe_dtype_t dt,
                                      moe_act_t act) {
  if (R_max < 0 || E < 1 || E > 256 || h <= 0 || f <= 0 || !dtype_ok(dt) || !act_ok(act)) return 0;
  const FfnPlan pl = plan_ffn(dt == MOE_BF16, (double)R_max / E, E, R_max, h, f);
  Carve c(nullptr);
  carve_ffn(c, pl, R_max, h, f, E, dt, act);
  return c.bytes();
}

moe_status_t moe_expert_ffn(const void* x_perm, const int32_t* offsets, int32_t R_max, int32_t h, int32_t f,
                            int32_t E, const void* W1, const void* W3, const void* W2, moe_act_t act,
                            moe_dtype_t dt, void* out_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (R_max < 0 || E < 1) return MOE_ERR_ARG;
  if (E > 256) return MOE_ERR_UNSUPPORTED;
  if (!dtype_ok(dt) || !act_ok(act)) return MOE_ERR_ARG;
  moe_status_t s;
  if ((s = dim_ok(h)) != MOE_OK) return s;
  if ((s = dim_ok(f)) != MOE_OK) return s;
  if (!x_perm || !offsets || !W1 || !W2 || !out_perm) return MOE_ERR_ARG;
  if ((act == MOE_ACT_SWIGLU) != (W3 != nullptr)) return MOE_ERR_ARG;
  if (!aligned16(x_perm) || !aligned16(W1) || !aligned16(W2) || (W3 && !aligned16(W3)) || !aligned16(out_perm))
    return MOE_ERR_UNSUPPORTED;
  if ((s = rows_ok(R_max, h, f)) != MOE_OK) return s;
  if (R_max == 0) return MOE_OK;
  const bool bf = dt == MOE_BF16;
  const FfnPlan pl = plan_ffn(bf, (double)R_max / E, E, R_max, h, f);
  Carve c(ws);
  FfnWs w = carve_ffn(c, pl, R_max, h, f, E, dt, act);
  if (!ws || ws_bytes < c.bytes()) return MOE_ERR_WORKSPACE;
  MOE_TRY(launch_tiles(offsets, E, pl.bm, pl.big, w.tile_off, stream));
  return run_ffn(x_perm, nullptr, offsets, w.tile_off, pl, R_max, h, f, E, W1, W3, W2, act, dt, w.hm, w.part_up,
                 out_perm, false, w.part_down, false, stream);
}

moe_status_t moe_unpermute(const void* out_perm, const int32_t* slot_pos, const float* topk_w, int32_t T,
                           int32_t h, int32_t k, moe_dtype_t dt, void* y, hipStream_t stream) {
  if (T < 0 || k < 1) return MOE_ERR_ARG;
  if (k > 16) return MOE_ERR_UNSUPPORTED;
  if (!dtype_ok(dt)) return MOE_ERR_ARG;
  moe_status_t s;
  if ((s = dim_ok(h)) != MOE_OK) return s;
  if (!out_perm || !slot_pos || !topk_w || !y) return MOE_ERR_ARG;
  if (!aligned16(out_perm) || !aligned16(y)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  MOE_TRY(launch_combine(out_perm, dt == MOE_F32, 1, 0, slot_pos, topk_w, T, h, k, dt == MOE_BF16, y, stream));
  return MOE_OK;
}

static moe_status_t layer_forward_impl(const void* x, const float* W_gate, const float* logit_bias,
                                       const void* W1, const void* W3, const void* W2, int32_t T, int32_t h,
                                       int32_t f, int32_t E, int32_t k, float capacity_factor, moe_act_t act,
                                       moe_dtype_t dt, void* y, float* aux_loss, int32_t* counts, void* ws,
                                       size_t ws_bytes, hipStream_t stream, hipEvent_t* ev,
                                       const moe_router_opts_t* opts = nullptr, float* preact = nullptr,
                                       size_t preact_len = 0) {
  moe_status_t s = common_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (!dtype_ok(dt) || !act_ok(act) || !isfinite(capacity_factor)) return MOE_ERR_ARG;
  if ((s = dim_ok(h)) != MOE_OK) return s;
  if ((s = dim_ok(f)) != MOE_OK) return s;
  if (!x || !W_gate || !W1 || !W2 || !y) return MOE_ERR_ARG;
  if ((act == MOE_ACT_SWIGLU) != (W3 != nullptr)) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W2) || (W3 && !aligned16(W3)) || !aligned16(y))
    return MOE_ERR_UNSUPPORTED;
  if ((s = opts_ok(opts, x, false)) != MOE_OK) return s;
  if ((s = size_ok(T, h, f, E, k, capacity_factor)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  const int64_t C = capacity_of(T, E, k, capacity_factor);
  const int R_max = rows_max(T, E, k, C);
  const bool bf = dt == MOE_BF16;
  const FfnPlan pl = layer_plan(bf, T, h, f, E, k, C);
  Carve c(ws);
  LayerWs w = carve_layer(c, T, h, f, E, k, R_max, pl, dt, act);
  void* xj = has_jitter(opts) ? c.take<char>((size_t)T * h * elem_bytes(dt)) : nullptr;
  if (!ws || ws_bytes < c.bytes()) return MOE_ERR_WORKSPACE;
  if (preact != nullptr && preact_len < preact_bytes(R_max, f, act)) return MOE_ERR_WORKSPACE;
  int stage = 0;
  // a null array or a null entry records nothing at that point
  auto mark = [&]() -> bool {
    const hipEvent_t e = ev == nullptr ? nullptr : ev[stage++];
    return e == nullptr || hipEventRecord(e, stream) == hipSuccess;
  };
  if (!mark()) return MOE_ERR_DEVICE;

  RouteArgs ra{};
  ra.x = x;
  ra.W_gate = W_gate;
  ra.bias = logit_bias;
  ra.T = T;
  ra.h = h;
  ra.E = E;
  ra.k = k;
  ra.bf16 = bf;
  ra.logits_in = false;
  ra.logits = w.logits;
  ra.topk_idx = w.topk_idx;
  ra.topk_w = w.topk_w;
  ra.prob_part = w.prob_part;
  ra.blk_counts = w.blk_counts;  // the histogram is counted by the selection (or logits) kernel
  ra.planes = w.planes;
  ra.hist_tokens = route_hist_tokens(T, h, E, bf);
  apply_opts(ra, opts);
  if (xj != nullptr) {  // only the router sees the jittered input
    MOE_TRY(launch_jitter(x, opts->jitter, (int64_t)T * h, bf, xj, stream));
    ra.x = xj;
  }
  // one block of tokens (decode): the selection kernel also does the scan and the scatter
  const bool one_block = route_blocks(T) == 1;
  SmallPermute sp{};
  if (one_block) {
    sp.C = (int)C;
    sp.BM = pl.bm;
    sp.big = pl.big;
    sp.nbits = expert_bits(E);
    sp.counts = counts ? counts : w.counts;
    sp.offsets = w.offsets;
    sp.tile_off = w.tile_off;
    sp.aux = aux_loss ? aux_loss : w.aux;
    sp.slot_pos = w.slot_pos;
    sp.sorted_slot = w.sorted_slot;
    sp.perm_token = w.perm_token;
    ra.permute = &sp;
  }
  MOE_TRY(launch_logits(ra, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  MOE_TRY(launch_select(ra, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  ScanArgs sa{};
  sa.blk_counts = w.blk_counts;
  sa.nhb = route_hist_blocks(T, h, E, bf);
  sa.hpb = kSelTokens / ra.hist_tokens;
  sa.E = E;
  sa.T = T;
  sa.k = k;
  sa.C = (int)C;
  sa.BM = pl.bm;
  sa.big = pl.big;
  sa.prob_part = w.prob_part;
  sa.nrb = sa.nhb;
  sa.prob_sum = nullptr;
  sa.counts = counts ? counts : w.counts;
  sa.offsets = w.offsets;
  sa.blk_base = w.blk_base;
  sa.tile_off = w.tile_off;
  sa.aux = aux_loss ? aux_loss : w.aux;
  // (fused scan + scatter: the scan stage holds both and the scatter stage is empty)
  const bool fused = !one_block && scan_scatter_fusable(sa.nhb, sa.nrb, E);
  if (fused) MOE_TRY(launch_scan_scatter(sa, w.topk_idx, w.slot_pos, w.sorted_slot, w.perm_token, stream));
  else if (!one_block) MOE_TRY(launch_scan(sa, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  if (!one_block && !fused)
    MOE_TRY(launch_scatter(w.topk_idx, T, E, k, (int)C, w.offsets, w.blk_base, w.slot_pos, w.sorted_slot,
                           w.perm_token, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  moe_status_t r = run_ffn(x, w.perm_token, w.offsets, w.tile_off, pl, R_max, h, f, E, W1, W3, W2, act, dt, w.hm,
                           w.part_up, w.o, true, w.o, true, stream,
                           ev ? [&]() { return mark(); } : std::function<bool()>(), preact);
  if (r != MOE_OK) return r;
  if (preact != nullptr && !bf) {  // fp32: the pre-activations from their own GEMMs
    r = preact_gemms(x, w.perm_token, w.offsets, w.tile_off, pl, R_max, h, f, E, W1, W3, act, false, preact, stream);
    if (r != MOE_OK) return r;
  }
  MOE_TRY(launch_combine(w.o, true, pl.s_down, (size_t)R_max * h, w.slot_pos, w.topk_w, T, h, k, bf, y, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  return MOE_OK;
}

moe_status_t moe_layer_routing(const void* ws, size_t ws_bytes, int32_t T, int32_t h, int32_t f, int32_t E,
                               int32_t k, float capacity_factor, moe_dtype_t dt, moe_act_t act,
                               moe_layer_routing_t* out) {
  moe_status_t s = common_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (!dtype_ok(dt) || !act_ok(act) || !isfinite(capacity_factor) || !ws || !out) return MOE_ERR_ARG;
  if ((s = dim_ok(h)) != MOE_OK) return s;
  if ((s = dim_ok(f)) != MOE_OK) return s;
  const int64_t C = capacity_of(T, E, k, capacity_factor);
  Carve c(const_cast<void*>(ws));
  const LayerWs w = carve_layer(c, T, h, f, E, k, rows_max(T, E, k, C), layer_plan(dt == MOE_BF16, T, h, f, E, k, C),
                                dt, act);
  if (ws_bytes < c.bytes()) return MOE_ERR_WORKSPACE;
  out->logits = w.logits;
  out->topk_idx = w.topk_idx;
  out->topk_w = w.topk_w;
  out->counts = w.counts;
  out->offsets = w.offsets;
  out->slot_pos = w.slot_pos;
  out->sorted_slot = w.sorted_slot;
  return MOE_OK;
}

int32_t moe_binned_capacity_max(int32_t T, int32_t E, int32_t k, float capacity_factor, int32_t min_capacity) {
  if (common_sizes(T, E, k) != MOE_OK || !isfinite(capacity_factor) || min_capacity < 0) return -1;
  return (int32_t)binned_cmax(T, E, k, capacity_factor, min_capacity);
}

static moe_status_t binned_sizes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, float cf,
                                 int32_t min_capacity, int64_t* cmax) {
  moe_status_t s = common_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (!isfinite(cf) || min_capacity < 0) return MOE_ERR_ARG;
  if ((s = dim_ok(h)) != MOE_OK) return s;
  if ((s = dim_ok(f)) != MOE_OK) return s;
  *cmax = binned_cmax(T, E, k, cf, min_capacity);
  // bucket rows are int32 and the GEMMs address their operands with 32-bit element offsets
  const int64_t rows = (int64_t)E * *cmax;
  if (rows > INT32_MAX / 2 || rows * (int64_t)(h > f ? h : f) >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_binned_workspace_bytes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, float capacity_factor,
                                  int32_t min_capacity, moe_dtype_t dt, moe_act_t act) {
  int64_t cmax = 0;
  if (!dtype_ok(dt) || !act_ok(act) || binned_sizes(T, h, f, E, k, capacity_factor, min_capacity, &cmax) != MOE_OK)
    return 0;
  const int64_t cfix = binned_cfixed(T, E, k, capacity_factor, min_capacity);
  const double rpe = cfix == INT32_MAX ? (double)T * k / E : (double)cfix;
  const int R_max = (int)(E * cmax);
  const FfnPlan pl = plan_ffn(dt == MOE_BF16, rpe, E, R_max, h, f);
  Carve c(nullptr);
  carve_binned(c, T, h, f, E, k, R_max, pl, dt, act, true);
  return c.bytes();
}

static moe_status_t layer_forward_binned_impl(const void* x, const float* W_gate, const float* logit_bias,
                                              const void* W1, const void* W3, const void* W2, int32_t T, int32_t h,
                                              int32_t f, int32_t E, int32_t k, float capacity_factor,
                                              int32_t min_capacity, moe_act_t act, moe_dtype_t dt, void* y,
                                              float* aux_loss, int32_t* counts, int32_t* capacity, void* x_bins,
                                              void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* ev) {
  int64_t cmax = 0;
  moe_status_t s = binned_sizes(T, h, f, E, k, capacity_factor, min_capacity, &cmax);
  if (s != MOE_OK) return s;
  if (!dtype_ok(dt) || !act_ok(act)) return MOE_ERR_ARG;
  if (!x || !W_gate || !W1 || !W2 || !y) return MOE_ERR_ARG;
  if ((act == MOE_ACT_SWIGLU) != (W3 != nullptr)) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(W1) || !aligned16(W2) || (W3 && !aligned16(W3)) || !aligned16(y) ||
      (x_bins && !aligned16(x_bins)))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const int64_t cfix = binned_cfixed(T, E, k, capacity_factor, min_capacity);
  const double rpe = cfix == INT32_MAX ? (double)T * k / E : (double)cfix;
  const int R_max = (int)(E * cmax);
  const bool bf = dt == MOE_BF16;
  const FfnPlan pl = plan_ffn(bf, rpe, E, R_max, h, f);
  Carve c(ws);
  BinnedWs bw = carve_binned(c, T, h, f, E, k, R_max, pl, dt, act, x_bins == nullptr);
  if (!ws || ws_bytes < c.bytes()) return MOE_ERR_WORKSPACE;
  LayerWs& w = bw.l;
  void* xb = x_bins ? x_bins : bw.x_bins;
  int stage = 0;
  // a null array or a null entry records nothing at that point
  auto mark = [&]() -> bool {
    const hipEvent_t e = ev == nullptr ? nullptr : ev[stage++];
    return e == nullptr || hipEventRecord(e, stream) == hipSuccess;
  };
  if (!mark()) return MOE_ERR_DEVICE;

  RouteArgs ra{};
  ra.x = x;
  ra.W_gate = W_gate;
  ra.bias = logit_bias;
  ra.T = T;
  ra.h = h;
  ra.E = E;
  ra.k = k;
  ra.bf16 = bf;
  ra.logits = w.logits;
  ra.topk_idx = w.topk_idx;
  ra.topk_w = w.topk_w;
  ra.prob_part = w.prob_part;
  ra.blk_counts = w.blk_counts;
  ra.planes = w.planes;
  MOE_TRY(launch_logits(ra, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  MOE_TRY(launch_select(ra, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  ScanArgs sa{};
  sa.blk_counts = w.blk_counts;
  sa.nhb = route_blocks(T);
  sa.E = E;
  sa.T = T;
  sa.k = k;
  sa.C = (int)cfix;
  sa.BM = pl.bm;
  sa.big = pl.big;
  sa.prob_part = w.prob_part;
  sa.nrb = route_blocks(T);
  sa.counts = counts ? counts : w.counts;
  sa.offsets = w.offsets;
  sa.blk_base = w.blk_base;
  sa.tile_off = w.tile_off;
  sa.aux = aux_loss ? aux_loss : w.aux;
  sa.binned = true;
  sa.cap_out = capacity ? capacity : bw.cap;
  MOE_TRY(launch_scan(sa, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  MOE_TRY(launch_scatter(w.topk_idx, T, E, k, (int)cfix, w.offsets, w.blk_base, w.slot_pos, w.sorted_slot,
                         w.perm_token, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  MOE_TRY(launch_binned_gather(x, w.perm_token, w.offsets, sa.counts, E, R_max, h, (int)elem_bytes(dt), xb,
                               stream));
  if (!mark()) return MOE_ERR_DEVICE;
  moe_status_t r = run_ffn(xb, nullptr, w.offsets, w.tile_off, pl, R_max, h, f, E, W1, W3, W2, act, dt,
                           w.hm, w.part_up, w.o, true, w.o, true, stream,
                           ev ? [&]() { return mark(); } : std::function<bool()>());
  if (r != MOE_OK) return r;
  MOE_TRY(launch_combine(w.o, true, pl.s_down, (size_t)R_max * h, w.slot_pos, w.topk_w, T, h, k, bf, y, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  return MOE_OK;
}

moe_status_t moe_layer_forward_binned(const void* x, const float* W_gate, const float* logit_bias, const void* W1,
                                      const void* W3, const void* W2, int32_t T, int32_t h, int32_t f, int32_t E,
                                      int32_t k, float capacity_factor, int32_t min_capacity, moe_act_t act,
                                      moe_dtype_t dt, void* y, float* aux_loss, int32_t* counts, int32_t* capacity,
                                      void* x_bins, void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_forward_binned_impl(x, W_gate, logit_bias, W1, W3, W2, T, h, f, E, k, capacity_factor, min_capacity,
                                   act, dt, y, aux_loss, counts, capacity, x_bins, ws, ws_bytes, stream, nullptr);
}

moe_status_t moe_layer_forward_binned_timed(const void* x, const float* W_gate, const float* logit_bias,
                                            const void* W1, const void* W3, const void* W2, int32_t T, int32_t h,
                                            int32_t f, int32_t E, int32_t k, float capacity_factor,
                                            int32_t min_capacity, moe_act_t act, moe_dtype_t dt, void* y,
                                            float* aux_loss, int32_t* counts, int32_t* capacity, void* x_bins,
                                            void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  if (events == nullptr) return MOE_ERR_ARG;
  return layer_forward_binned_impl(x, W_gate, logit_bias, W1, W3, W2, T, h, f, E, k, capacity_factor, min_capacity,
                                   act, dt, y, aux_loss, counts, capacity, x_bins, ws, ws_bytes, stream, events);
}

moe_status_t moe_layer_forward(const void* x, const float* W_gate, const float* logit_bias, const void* W1,
                               const void* W3, const void* W2, int32_t T, int32_t h, int32_t f, int32_t E,
                               int32_t k, float capacity_factor, moe_act_t act, moe_dtype_t dt, void* y,
                               float* aux_loss, int32_t* counts, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  return layer_forward_impl(x, W_gate, logit_bias, W1, W3, W2, T, h, f, E, k, capacity_factor, act, dt, y,
                            aux_loss, counts, ws, ws_bytes, stream, nullptr);
}

// ---- backward pass
struct BwdWs {
  int* counts;
  int* tile64;
  int* tile_ts;  // data-gradient tile list (ts rows per tile)
  int* seg;
  float* dw;
  float* dl;
  void* dO;
  float* ag;
  void* dag;
  float* dXp;      // [dx_parts][R_max][h]: K parts of the up projection's data gradient
  float* dx_r;
  float* wg_part;  // partial sums of dW_gate over token slices
  void* xp;        // bf16: the gathered rows of x for the up projection's weight gradients
};
// token slices of dW_gate = x^T dl: about 512 tokens each, at most 64
static int wgate_splits(int32_t T) { return std::max(1, std::min(64, (T + 511) / 512)); }
// K parts of the up projection's data gradient (bf16): doubled, up to four, while that
// fills the last round of tiles on the 256 CUs markedly better (by more than 0.12 of a
// round: at the prefill shape 2 parts take the fill from 0.75 to 0.90; 4 parts, filling
// 1.0, measured 5 % slower, and adding them costs the dx kernel 0.08 ms).  Expected m-tiles of the
// ts-row tiles: one per expert when its rows fit one tile, else half a tile of padding per
// expert on top of the rows.
static int dx_parts(bool bf, const FfnPlan& pl, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, int64_t C,
                    int n_up) {
  if (!bf) return 1;
  const double ts = pl.bm == 256 ? 256.0 : 128.0;
  double rpe = (double)T * k / E;
  if (C != INT32_MAX && (double)C < rpe) rpe = (double)C;
  const double mt = rpe <= ts ? E : E * (rpe / ts + 0.5);
  const double tiles = mt * ceil(h / 256.0);
  auto fill = [](double t) {
    const double r = t / 256.0;
    return r / ceil(r);
  };
  const int K = n_up * f;
  int S = 1;
  while (S < 4 && K % (2 * S * 64) == 0 && K / (2 * S) >= 16 * 64 && fill(2 * S * tiles) > fill(S * tiles) + 0.12)
    S *= 2;
  return S;
}
static BwdWs carve_bwd(Carve& c, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, int R_max, moe_dtype_t dt,
                       moe_act_t act, int parts) {
  const int n_up = act == MOE_ACT_SWIGLU ? 2 : 1;
  const size_t es = elem_bytes(dt);
  BwdWs b;
  b.counts = c.take<int>(E);
  b.tile64 = c.take<int>((size_t)E + 1);
  b.tile_ts = c.take<int>((size_t)E + 1);
  b.seg = c.take<int>(4);
  b.dw = c.take<float>((size_t)T * k);
  b.dl = c.take<float>((size_t)T * E);
  b.dO = c.take<char>((size_t)R_max * h * es);
  b.ag = c.take<float>((size_t)R_max * n_up * f);
  b.dag = c.take<char>((size_t)R_max * n_up * f * es);
  b.dXp = c.take<float>((size_t)parts * R_max * h);
  b.dx_r = c.take<float>((size_t)T * h);
  const int S = wgate_splits(T);
  b.wg_part = S > 1 ? c.take<float>((size_t)S * h * E) : nullptr;
  b.xp = dt == MOE_BF16 ? c.take<char>((size_t)R_max * h * es) : nullptr;
  return b;
}

size_t moe_layer_backward_workspace_bytes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                          float capacity_factor, moe_dtype_t dt, moe_act_t act) {
  if (common_sizes(T, E, k) != MOE_OK || !dtype_ok(dt) || !act_ok(act) || !isfinite(capacity_factor)) return 0;
  if (dim_ok(h) != MOE_OK || dim_ok(f) != MOE_OK) return 0;
  const int64_t C = capacity_of(T, E, k, capacity_factor);
  const int R_max = rows_max(T, E, k, C);
  const bool bf = dt == MOE_BF16;
  const int parts = dx_parts(bf, layer_plan(bf, T, h, f, E, k, C), T, h, f, E, k, C, act == MOE_ACT_SWIGLU ? 2 : 1);
  Carve c(nullptr);
  carve_bwd(c, T, h, f, E, k, R_max, dt, act, parts);
  return c.bytes();
}

static moe_status_t layer_backward_impl(const void* x, const float* W_gate, const void* W1, const void* W3,
                                        const void* W2, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                        float capacity_factor, moe_act_t act, moe_dtype_t dt, const void* dy,
                                        float d_aux, const void* fwd_ws, size_t fwd_ws_bytes,
                                        const float* preact, size_t preact_len, void* dx, float* dW_gate,
                                        float* dW1, float* dW3, float* dW2, void* ws, size_t ws_bytes,
                                        hipStream_t stream, hipEvent_t* ev,
                                        const moe_router_opts_t* opts = nullptr) {
  moe_status_t s = common_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (!dtype_ok(dt) || !act_ok(act) || !isfinite(capacity_factor) || !isfinite(d_aux)) return MOE_ERR_ARG;
  if ((s = dim_ok(h)) != MOE_OK) return s;
  if ((s = dim_ok(f)) != MOE_OK) return s;
  if (!x || !W_gate || !W1 || !W2 || !dy || !dx || !dW1 || !dW2) return MOE_ERR_ARG;
  if ((act == MOE_ACT_SWIGLU) != (W3 != nullptr) || (act == MOE_ACT_SWIGLU) != (dW3 != nullptr)) return MOE_ERR_ARG;
  for (const void* p : {x, (const void*)W_gate, W1, W3, W2, dy, (const void*)dx, (const void*)dW_gate,
                        (const void*)dW1, (const void*)dW3, (const void*)dW2, (const void*)preact})
    if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;  // (null passes: the optional ones)
  if ((s = opts_ok(opts, x, false)) != MOE_OK) return s;
  // the training forward takes no router variants, so its pre-activations belong to the plain routing
  if (opts != nullptr && preact != nullptr) return MOE_ERR_ARG;
  // the uniform assignment is a benchmarking mode: its ids are not the router's choice
  if (opts != nullptr && opts->uniform_assignment != 0) return MOE_ERR_UNSUPPORTED;
  if ((s = size_ok(T, h, f, E, k, capacity_factor)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  const int64_t C = capacity_of(T, E, k, capacity_factor);
  const int R_max = rows_max(T, E, k, C);
  const bool bf = dt == MOE_BF16;
  const FfnPlan pl = layer_plan(bf, T, h, f, E, k, C);
  // the forward's workspace, carved as the forward carved it (with jitter: the router's
  // input x * u follows the layer's pieces)
  Carve cf(const_cast<void*>(fwd_ws));
  LayerWs w = carve_layer(cf, T, h, f, E, k, R_max, pl, dt, act);
  const void* xr = has_jitter(opts) ? (const void*)cf.take<char>((size_t)T * h * elem_bytes(dt)) : x;
  if (!fwd_ws || fwd_ws_bytes < cf.bytes()) return MOE_ERR_WORKSPACE;
  Carve c(ws);
  const int parts = dx_parts(bf, pl, T, h, f, E, k, C, act == MOE_ACT_SWIGLU ? 2 : 1);
  BwdWs b = carve_bwd(c, T, h, f, E, k, R_max, dt, act, parts);
  if (!ws || ws_bytes < c.bytes()) return MOE_ERR_WORKSPACE;
  if (preact != nullptr && preact_len < preact_bytes(R_max, f, act)) return MOE_ERR_WORKSPACE;
  const int n_up = act == MOE_ACT_SWIGLU ? 2 : 1;
  const int gact = act == MOE_ACT_SWIGLU ? ACT_SWIGLU : ACT_GELU;
  int stage = 0;
  // a null array or a null entry records nothing at that point
  auto mark = [&]() -> bool {
    const hipEvent_t e = ev == nullptr ? nullptr : ev[stage++];
    return e == nullptr || hipEventRecord(e, stream) == hipSuccess;
  };
  if (!mark()) return MOE_ERR_DEVICE;

  MOE_TRY(launch_counts(w.blk_counts, route_hist_blocks(T, h, E, bf), E, b.counts, stream));
  MOE_TRY(launch_tile_scan(w.offsets, E, 64, b.tile64, stream));
  // data-gradient tile height: 256 rows when the forward's GEMMs take 256-row tiles
  const int ts = pl.bm == 256 ? 256 : 128;
  if (bf) MOE_TRY(launch_tile_scan(w.offsets, E, ts, b.tile_ts, stream));
  MOE_TRY(launch_seg_init(b.seg, T, stream));
  // combine: dw and dO
  MOE_TRY(launch_combine_bwd(dy, w.o, pl.s_down, (size_t)R_max * h, w.slot_pos, w.topk_w, T, h, k, bf, b.dw, b.dO,
                             stream));
  if (!mark()) return MOE_ERR_DEVICE;
  // router: logit gradient of the renormalised selection and of the aux loss
  MOE_TRY(launch_router_bwd(w.logits, opts ? opts->logit_noise : nullptr, w.topk_idx, w.topk_w, b.dw, b.counts, T,
                            E, k, d_aux, opts ? 1.0f / opts->temperature : 1.0f, opts && opts->soft_topk != 0, b.dl,
                            stream));
  if (!mark()) return MOE_ERR_DEVICE;
  // the up projection's pre-activations a (| g): saved by the training forward, else
  // recomputed with the same GEMM
  const float* ag = preact;
  if (ag == nullptr) {
    const moe_status_t r =
        preact_gemms(x, w.perm_token, w.offsets, w.tile_off, pl, R_max, h, f, E, W1, W3, act, bf, b.ag, stream);
    if (r != MOE_OK) return r;
    ag = b.ag;
  }
  const float* pa = ag;
  const float* pg = bf ? ag + f : ag + (size_t)R_max * f;
  const int ld_ag = bf ? n_up * f : f;
  if (!mark()) return MOE_ERR_DEVICE;
  // down projection: dHm = dO W2^T, folded into da (| dg) by the activation's derivative
  BwdNT nt{};
  nt.A = b.dO;
  nt.lda = h;
  nt.a_bf16 = bf;
  nt.B1 = W2;
  nt.B2 = W2;
  nt.K1 = h;
  nt.sbe = (long long)f * h;
  nt.ldb = h;
  nt.b_bf16 = bf;
  nt.K = h;
  nt.N = f;
  nt.offsets = w.offsets;
  nt.tile_off = b.tile64;
  nt.ts = ts;
  nt.tile_off_ts = bf ? b.tile_ts : nullptr;
  nt.E = E;
  nt.R_max = R_max;
  nt.epi = gact;
  nt.pa = pa;
  nt.pg = pg;
  nt.ld_ag = ld_ag;
  nt.DAG = b.dag;
  MOE_TRY(launch_gemm_nt(nt, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  // dW2[e] = Hm^T dO
  BwdTN tn{};
  tn.A = w.hm;
  tn.lda = f;
  tn.a_bf16 = bf;
  tn.B = b.dO;
  tn.ldb = h;
  tn.b_bf16 = bf;
  tn.M = f;
  tn.N = h;
  tn.offsets = w.offsets;
  tn.E = E;
  tn.C1 = dW2;
  tn.C2 = dW2;
  tn.N1 = h;
  tn.sce = (long long)f * h;
  tn.ldc = h;
  MOE_TRY(launch_gemm_tn(tn, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  // up projection: dX = da W1^T (+ dg W3^T)
  nt = BwdNT{};
  nt.A = b.dag;
  nt.lda = n_up * f;
  nt.a_bf16 = bf;
  nt.B1 = W1;
  nt.B2 = act == MOE_ACT_SWIGLU ? W3 : W1;
  nt.K1 = f;
  nt.sbe = (long long)h * f;
  nt.ldb = f;
  nt.b_bf16 = bf;
  nt.K = n_up * f;
  nt.N = h;
  nt.offsets = w.offsets;
  nt.tile_off = b.tile64;
  nt.ts = ts;
  nt.tile_off_ts = bf ? b.tile_ts : nullptr;
  nt.E = E;
  nt.R_max = R_max;
  nt.C = b.dXp;
  nt.ldc = h;
  nt.epi = ACT_NONE;
  nt.ksplit = parts;
  MOE_TRY(launch_gemm_nt(nt, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  // dW1[e] = X^T da, dW3[e] = X^T dg (X rows gathered from x; bf16: into xp first, so
  // that the product reads whole rows)
  tn = BwdTN{};
  tn.A = x;
  tn.lda = h;
  tn.a_rows = w.perm_token;
  if (bf) {
    MOE_TRY(launch_gather_rows(x, w.perm_token, w.offsets, E, R_max, h * 2, b.xp, stream));
    tn.A = b.xp;
    tn.a_rows = nullptr;
  }
  tn.a_bf16 = bf;
  tn.B = b.dag;
  tn.ldb = n_up * f;
  tn.b_bf16 = bf;
  tn.M = h;
  tn.N = n_up * f;
  tn.offsets = w.offsets;
  tn.E = E;
  tn.C1 = dW1;
  tn.C2 = act == MOE_ACT_SWIGLU ? dW3 : dW1;
  tn.N1 = f;
  tn.sce = (long long)h * f;
  tn.ldc = f;
  MOE_TRY(launch_gemm_tn(tn, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  // router: dx += dl W_gate^T (one segment of T rows), dW_gate = x^T dl
  nt = BwdNT{};
  nt.A = b.dl;
  nt.lda = E;
  nt.a_bf16 = false;
  nt.B1 = W_gate;
  nt.B2 = W_gate;
  nt.K1 = E;
  nt.sbe = 0;
  nt.ldb = E;
  nt.b_bf16 = false;
  nt.K = E;
  nt.N = h;
  nt.offsets = b.seg;
  nt.tile_off = b.seg + 2;
  nt.E = 1;
  nt.R_max = T;
  nt.C = b.dx_r;
  nt.ldc = h;
  nt.epi = ACT_NONE;
  MOE_TRY(launch_gemm_nt(nt, stream));
  if (dW_gate) {
    tn = BwdTN{};
    tn.A = xr;  // the router's input
    tn.lda = h;
    tn.a_bf16 = bf;
    tn.B = b.dl;
    tn.ldb = E;
    tn.b_bf16 = false;
    tn.M = h;
    tn.N = E;
    tn.offsets = b.seg;
    tn.E = 1;
    tn.C1 = dW_gate;
    tn.C2 = dW_gate;
    tn.N1 = E;
    tn.sce = 0;
    tn.ldc = E;
    tn.ksplit = wgate_splits(T);
    tn.rows = T;
    tn.part = b.wg_part;
    MOE_TRY(launch_gemm_tn(tn, stream));
  }
  if (!mark()) return MOE_ERR_DEVICE;
  MOE_TRY(launch_dx_final(b.dx_r, has_jitter(opts) ? opts->jitter : nullptr, b.dXp, parts, (size_t)R_max * h,
                          w.slot_pos, T, h, k, bf, dx, stream));
  if (!mark()) return MOE_ERR_DEVICE;
  return MOE_OK;
}

moe_status_t moe_layer_backward(const void* x, const float* W_gate, const void* W1, const void* W3, const void* W2,
                                int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, float capacity_factor,
                                moe_act_t act, moe_dtype_t dt, const void* dy, float d_aux, const void* fwd_ws,
                                size_t fwd_ws_bytes, const float* preact, size_t preact_bytes_, void* dx,
                                float* dW_gate, float* dW1, float* dW3, float* dW2, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  return layer_backward_impl(x, W_gate, W1, W3, W2, T, h, f, E, k, capacity_factor, act, dt, dy, d_aux, fwd_ws,
                             fwd_ws_bytes, preact, preact_bytes_, dx, dW_gate, dW1, dW3, dW2, ws, ws_bytes, stream,
                             nullptr);
}

moe_status_t moe_layer_backward_ex(const void* x, const float* W_gate, const void* W1, const void* W3,
                                   const void* W2, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                   float capacity_factor, moe_act_t act, moe_dtype_t dt,
                                   const moe_router_opts_t* opts, const void* dy, float d_aux, const void* fwd_ws,
                                   size_t fwd_ws_bytes, const float* preact, size_t preact_bytes_, void* dx,
                                   float* dW_gate, float* dW1, float* dW3, float* dW2, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return layer_backward_impl(x, W_gate, W1, W3, W2, T, h, f, E, k, capacity_factor, act, dt, dy, d_aux, fwd_ws,
                             fwd_ws_bytes, preact, preact_bytes_, dx, dW_gate, dW1, dW3, dW2, ws, ws_bytes, stream,
                             nullptr, opts);
}

moe_status_t moe_layer_backward_timed(const void* x, const float* W_gate, const void* W1, const void* W3,
                                      const void* W2, int32_t T, int32_t h, int32_t f, int32_t E, int32_t k,
                                      float capacity_factor, moe_act_t act, moe_dtype_t dt, const void* dy,
                                      float d_aux, const void* fwd_ws, size_t fwd_ws_bytes, const float* preact,
                                      size_t preact_bytes_, void* dx, float* dW_gate, float* dW1, float* dW3,
                                      float* dW2, void* ws, size_t ws_bytes, hipStream_t stream,
                                      hipEvent_t* events) {
  if (events == nullptr) return MOE_ERR_ARG;
  return layer_backward_impl(x, W_gate, W1, W3, W2, T, h, f, E, k, capacity_factor, act, dt, dy, d_aux, fwd_ws,
                             fwd_ws_bytes, preact, preact_bytes_, dx, dW_gate, dW1, dW3, dW2, ws, ws_bytes, stream,
                             events);
}

size_t moe_layer_preact_bytes(int32_t T, int32_t h, int32_t f, int32_t E, int32_t k, float capacity_factor,
                              moe_act_t act) {
  if (common_sizes(T, E, k) != MOE_OK || !act_ok(act) || !isfinite(capacity_factor)) return 0;
  if (dim_ok(h) != MOE_OK || dim_ok(f) != MOE_OK) return 0;
  return preact_bytes(rows_max(T, E, k, capacity_of(T, E, k, capacity_factor)), f, act);
}

moe_status_t moe_layer_forward_train(const void* x, const float* W_gate, const float* logit_bias, const void* W1,
                                     const void* W3, const void* W2, int32_t T, int32_t h, int32_t f, int32_t E,
                                     int32_t k, float capacity_factor, moe_act_t act, moe_dtype_t dt, void* y,
                                     float* aux_loss, int32_t* counts, void* ws, size_t ws_bytes, float* preact,
                                     size_t preact_bytes_, hipStream_t stream, hipEvent_t* events) {
  if (preact == nullptr) return MOE_ERR_ARG;
  if (!aligned16(preact)) return MOE_ERR_UNSUPPORTED;
  return layer_forward_impl(x, W_gate, logit_bias, W1, W3, W2, T, h, f, E, k, capacity_factor, act, dt, y,
                            aux_loss, counts, ws, ws_bytes, stream, events, nullptr, preact, preact_bytes_);
}

moe_status_t moe_layer_forward_ex(const void* x, const float* W_gate, const float* logit_bias, const void* W1,
                                  const void* W3, const void* W2, int32_t T, int32_t h, int32_t f, int32_t E,
                                  int32_t k, float capacity_factor, moe_act_t act, moe_dtype_t dt,
                                  const moe_router_opts_t* opts, void* y, float* aux_loss, int32_t* counts,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_forward_impl(x, W_gate, logit_bias, W1, W3, W2, T, h, f, E, k, capacity_factor, act, dt, y,
                            aux_loss, counts, ws, ws_bytes, stream, nullptr, opts);
}

moe_status_t moe_layer_forward_timed(const void* x, const float* W_gate, const float* logit_bias,
                                     const void* W1, const void* W3, const void* W2, int32_t T, int32_t h,
                                     int32_t f, int32_t E, int32_t k, float capacity_factor, moe_act_t act,
                                     moe_dtype_t dt, void* y, float* aux_loss, int32_t* counts, void* ws,
                                     size_t ws_bytes, hipStream_t stream, hipEvent_t* events) {
  if (events == nullptr) return MOE_ERR_ARG;
  return layer_forward_impl(x, W_gate, logit_bias, W1, W3, W2, T, h, f, E, k, capacity_factor, act, dt, y,
                            aux_loss, counts, ws, ws_bytes, stream, events);
}

}  // extern "C"
