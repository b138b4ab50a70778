// C ABI of the sparse MoE layer forward: argument checks, exact capacity,
// workspace layout and the launch sequence of each entry point.  All launches
// go to the caller's stream; nothing here allocates or synchronises.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return MOE_ERR_HIP;
}

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ceil(k * T * cf / E) on the exact binary value of cf.
int64_t exact_capacity(int64_t T, int32_t E, int32_t k, double cf) {
  int ex = 0;
  const double mant = std::frexp(cf, &ex);  // cf = mant * 2^ex, mant in [0.5, 1)
  const __int128 M = static_cast<__int128>(std::ldexp(mant, 53));  // integer, exact
  const int sh = ex - 53;
  const __int128 P = static_cast<__int128>(k) * T * M;
  __int128 c;
  if (sh >= 0) {
    const __int128 num = P << sh;  // sh is small: cf is bounded by validation
    c = (num + E - 1) / E;
  } else if (-sh > 100) {
    c = P > 0 ? 1 : 0;  // P < 2^87 < E * 2^100: the quotient is in (0, 1)
  } else {
    const __int128 Q = static_cast<__int128>(E) << (-sh);
    c = (P + Q - 1) / Q;
  }
  return static_cast<int64_t>(c);
}

int validate(const moe_config* cfg) {
  if (!cfg) return fail(MOE_ERR_ARG, "cfg is NULL");
  if (cfg->T < 0) return fail(MOE_ERR_ARG, "T must be >= 0");
  if (cfg->E < 1) return fail(MOE_ERR_ARG, "E must be >= 1");
  if (cfg->k < 1 || cfg->k > cfg->E) return fail(MOE_ERR_ARG, "k must be in [1, E]");
  if (cfg->d_model <= 0 || cfg->d_ff <= 0) return fail(MOE_ERR_ARG, "d_model and d_ff must be > 0");
  if (!(cfg->capacity_factor > 0.0) || !std::isfinite(cfg->capacity_factor))
    return fail(MOE_ERR_ARG, "capacity_factor must be finite and > 0");
  if (cfg->dtype != MOE_DTYPE_F32 && cfg->dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_ARG, "dtype must be MOE_DTYPE_F32 or MOE_DTYPE_BF16");
  if (cfg->act < MOE_ACT_RELU || cfg->act > MOE_ACT_GEGLU)
    return fail(MOE_ERR_ARG, "act must be MOE_ACT_RELU, MOE_ACT_GELU, MOE_ACT_REGLU or MOE_ACT_GEGLU");
  if (cfg->route != MOE_ROUTE_TOPK && cfg->route != MOE_ROUTE_RRE)
    return fail(MOE_ERR_ARG, "route must be MOE_ROUTE_TOPK or MOE_ROUTE_RRE");
  if (cfg->route == MOE_ROUTE_RRE) {
    if (cfg->k != 1) return fail(MOE_ERR_ARG, "random routed experts need k == 1");
    if (cfg->n_groups < 1 || cfg->E % cfg->n_groups != 0)
      return fail(MOE_ERR_ARG, "random routed experts need n_groups >= 1 dividing E");
  }
  if (cfg->E > moe::kMaxE) return fail(MOE_ERR_UNSUPPORTED, "E > 512 is not supported");
  if (cfg->k > moe::kMaxK) return fail(MOE_ERR_UNSUPPORTED, "k > 8 is not supported");
  if (cfg->d_model % 64 != 0 || cfg->d_ff % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 64");
  if (cfg->d_model > (1 << 20) || cfg->d_ff > (1 << 20))
    return fail(MOE_ERR_UNSUPPORTED, "d_model and d_ff must be <= 2^20");
  if (cfg->T > (int64_t(1) << 30) / cfg->k) return fail(MOE_ERR_UNSUPPORTED, "k * T must be <= 2^30");
  if (cfg->capacity_factor > 1e6) return fail(MOE_ERR_UNSUPPORTED, "capacity_factor must be <= 1e6");
  const int64_t C = exact_capacity(cfg->T, cfg->E, cfg->k, cfg->capacity_factor);
  if (C > (int64_t(1) << 31) / cfg->E) return fail(MOE_ERR_UNSUPPORTED, "E * capacity must be <= 2^31");
  return MOE_OK;
}

void make_plan(const moe_config* cfg, moe::Plan& p) {
  p.T = cfg->T;
  p.d = cfg->d_model;
  p.f = cfg->d_ff;
  p.E = cfg->E;
  p.k = cfg->k;
  p.C = exact_capacity(cfg->T, cfg->E, cfg->k, cfg->capacity_factor);
  p.Epad = (cfg->E + 31) / 32 * 32;
  // Router block: the bf16 MFMA router takes 32, 64 or 128 tokens per block,
  // aiming at >= 256 blocks (one per CU) and at most 32 tokens when E > 256;
  // the other routers use 64.
  p.TB = 64;
  if (cfg->route == MOE_ROUTE_TOPK && cfg->dtype == MOE_DTYPE_BF16) {
    const int64_t per_cu = cfg->T / 256;
    p.TB = per_cu >= 128 ? 128 : (per_cu >= 64 ? 64 : 32);
    if (p.Epad > 256) p.TB = 32;
  }
  p.NB = static_cast<int>((cfg->T + p.TB - 1) / p.TB);
  p.dtype = cfg->dtype;
  p.act = (cfg->act == MOE_ACT_GELU || cfg->act == MOE_ACT_GEGLU) ? 1 : 0;
  p.glu = cfg->act == MOE_ACT_REGLU || cfg->act == MOE_ACT_GEGLU;
  p.route = cfg->route;
  p.n_groups = cfg->n_groups;
  p.rre_seed = cfg->rre_seed;
  p.elem = cfg->dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const int64_t Tk = p.T * p.k;
  const int64_t EC = static_cast<int64_t>(p.E) * p.C;
  const int64_t sizes[8] = {Tk * 4, Tk * 4, Tk * 4, int64_t(p.E) * 4, EC * 4,
                            EC * p.d * p.elem, EC * p.f * p.elem, EC * p.d * p.elem};
  int64_t off = 0;
  for (int r = 0; r < 8; ++r) {
    p.off_region[r] = off;
    off = align_up(off + sizes[r]);
  }
  const int64_t nh = int64_t(p.E) * p.k * p.NB * 4;
  p.off_hist = off;
  off = align_up(off + nh);
  p.off_offsets = off;
  off = align_up(off + nh);
  p.off_planes = off;
  off = align_up(off + 3LL * p.Epad * p.d * 2);
  p.off_flags = off;
  off = align_up(off + moe::kSplitBlocks * 4);
  p.off_psum = off;  // load-balancing loss: probability sums per router block, range sums
  off = align_up(off + moe::aux_region_bytes(p));
  p.total = off;
}

// Backward scratch (second workspace): byte offsets of its buffers.
struct BwdLayout {
  int64_t idx, gate, dgate, dy_e, zbuf, dz, dx_e, dh, dx_r, dwr_part, clip, total;
};

void bwd_layout(const moe::Plan& p, BwdLayout& L) {
  const int64_t Tk = p.T * p.k, EC = int64_t(p.E) * p.C;
  const bool topk = p.route == MOE_ROUTE_TOPK;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.idx = take(Tk * 4);
  L.gate = take(Tk * 4);
  L.dgate = take(Tk * 4);
  L.dy_e = take(EC * p.d * p.elem);
  // pre-activations recomputed for act': GELU, and both halves for GLU
  L.zbuf = take(p.glu ? EC * 2 * p.f * p.elem : (p.act == 1 ? EC * p.f * p.elem : 0));
  L.dz = take(EC * p.w1_rows() * p.elem);
  L.dx_e = take(EC * p.d * p.elem);
  L.dh = take(topk ? p.T * p.Epad * 4 : 0);
  L.dx_r = take(topk ? p.T * p.d * 4 : 0);
  L.dwr_part = take(topk ? int64_t(moe::kBwdSplit) * p.E * p.d * 4 : 0);
  L.clip = take(moe::kClipScratchBytes);
  L.total = off;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// A required device buffer: non-NULL when it holds bytes, 16-byte aligned.
int need(const void* ptr, int64_t bytes, const char* name) {
  if (bytes > 0 && !ptr) {
    g_last_error = std::string(name) + " is NULL";
    return MOE_ERR_ARG;
  }
  if (ptr && !aligned16(ptr)) {
    g_last_error = std::string(name) + " is not 16-byte aligned";
    return MOE_ERR_ARG;
  }
  return MOE_OK;
}

#define MOE_CHECK(expr)            \
  do {                             \
    const int _rc = (expr);        \
    if (_rc != MOE_OK) return _rc; \
  } while (0)

#define MOE_HIP(expr, where)                          \
  do {                                                \
    const hipError_t _e = (expr);                     \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

int check_router_args(const moe::Plan& p, const void* x, const float* w_r, const int32_t* group_id,
                      const int32_t* expert_idx, const float* gate, const void* ws) {
  const int64_t Tk = p.T * p.k;
  if (p.route == MOE_ROUTE_TOPK) {
    MOE_CHECK(need(x, p.T * p.d * p.elem, "x"));
    MOE_CHECK(need(w_r, 1, "w_r"));
  } else {
    MOE_CHECK(need(group_id, p.T * 4, "group_id"));
  }
  MOE_CHECK(need(expert_idx, Tk * 4, "expert_idx"));
  MOE_CHECK(need(gate, Tk * 4, "gate"));
  MOE_CHECK(need(ws, p.total, "ws"));
  return MOE_OK;
}

int run_router(const moe::Plan& p, const void* x, const float* w_r, const float* bias,
               const int32_t* group_id, int32_t* expert_idx, float* gate, void* ws, hipStream_t s) {
  if (p.route == MOE_ROUTE_TOPK)
    MOE_HIP(moe::launch_router_topk(p, x, w_r, bias, expert_idx, gate, ws, s), "router");
  else
    MOE_HIP(moe::launch_router_rre(p, group_id, expert_idx, gate, ws, s), "router");
  return MOE_OK;
}

}  // namespace

extern "C" {

int64_t moe_capacity(const moe_config* cfg) {
  const int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  return exact_capacity(cfg->T, cfg->E, cfg->k, cfg->capacity_factor);
}

int64_t moe_workspace_bytes(const moe_config* cfg) {
  const int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  moe::Plan p;
  make_plan(cfg, p);
  return p.total;
}

int64_t moe_workspace_offset(const moe_config* cfg, int32_t region) {
  const int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (region < 0 || region >= MOE_WS_N_REGIONS) return fail(MOE_ERR_ARG, "unknown workspace region");
  moe::Plan p;
  make_plan(cfg, p);
  return p.off_region[region];
}

int moe_router(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
               const int32_t* group_id, int32_t* expert_idx, float* gate, void* ws, void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  MOE_CHECK(check_router_args(p, x, w_r, group_id, expert_idx, gate, ws));
  return run_router(p, x, w_r, bias, group_id, expert_idx, gate, ws, static_cast<hipStream_t>(stream));
}

int moe_router_aux(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
                   int32_t* expert_idx, float* gate, double alpha, float* aux, void* ws,
                   void* stream) {
  MOE_CHECK(validate(cfg));
  if (cfg->route != MOE_ROUTE_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "the load-balancing loss needs learned (top-k) routing");
  if (!std::isfinite(alpha)) return fail(MOE_ERR_ARG, "alpha must be finite");
  moe::Plan p;
  make_plan(cfg, p);
  MOE_CHECK(check_router_args(p, x, w_r, nullptr, expert_idx, gate, ws));
  MOE_CHECK(need(aux, (1 + 2 * int64_t(p.E)) * 4, "aux"));
  if (p.T == 0) return fail(MOE_ERR_ARG, "the load-balancing loss needs T >= 1");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_HIP(moe::launch_router_topk(p, x, w_r, bias, expert_idx, gate, ws, s, true), "router");
  MOE_HIP(moe::launch_router_aux(p, alpha, aux, ws, s), "load-balancing loss");
  return MOE_OK;
}

int moe_dispatch(const moe_config* cfg, const void* x, const int32_t* expert_idx, int32_t* slot,
                 int32_t* expert_count, int32_t* slot_token, void* x_e, void* ws, void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  const int64_t Tk = p.T * p.k;
  const int64_t EC = int64_t(p.E) * p.C;
  MOE_CHECK(need(x, p.T * p.d * p.elem, "x"));
  MOE_CHECK(need(expert_idx, Tk * 4, "expert_idx"));
  MOE_CHECK(need(slot, Tk * 4, "slot"));
  MOE_CHECK(need(expert_count, int64_t(p.E) * 4, "expert_count"));
  MOE_CHECK(need(slot_token, EC * 4, "slot_token"));
  MOE_CHECK(need(x_e, EC * p.d * p.elem, "x_e"));
  MOE_CHECK(need(ws, p.total, "ws"));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_HIP(moe::launch_dispatch_hist(p, expert_idx, ws, s), "dispatch histogram");
  MOE_HIP(moe::launch_dispatch_scan(p, expert_count, slot_token, ws, s), "dispatch scan");
  MOE_HIP(moe::launch_dispatch_slot_gather(p, x, expert_idx, slot, slot_token, x_e, ws, s),
          "dispatch slots/gather");
  return MOE_OK;
}

int moe_expert_ffn(const moe_config* cfg, const void* x_e, const int32_t* expert_count,
                   const void* w1, const void* w2, void* y_e, void* ws, void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  const int64_t EC = int64_t(p.E) * p.C;
  const int64_t wbytes = int64_t(p.E) * p.d * p.f * p.elem;
  MOE_CHECK(need(x_e, EC * p.d * p.elem, "x_e"));
  MOE_CHECK(need(expert_count, int64_t(p.E) * 4, "expert_count"));
  MOE_CHECK(need(w1, wbytes / p.f * p.w1_rows(), "w1"));
  MOE_CHECK(need(w2, wbytes, "w2"));
  MOE_CHECK(need(y_e, EC * p.d * p.elem, "y_e"));
  MOE_CHECK(need(ws, p.total, "ws"));
  MOE_HIP(moe::launch_expert_ffn(p, x_e, expert_count, w1, w2, y_e, ws, static_cast<hipStream_t>(stream)),
          "expert ffn");
  return MOE_OK;
}

int moe_expert_ffn_fused(const moe_config* cfg, const void* x_e, const int32_t* expert_count,
                         const void* w1, const void* w2, void* y_e, void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  const int nspl = moe::fused_ffn_split(p);
  if (nspl == 0)
    return fail(MOE_ERR_UNSUPPORTED,
                "fused expert FFN needs bf16, ReLU or GELU, 1 <= capacity <= 64, "
                "d_model % 384 == 0 and d_ff % 128 == 0");
  const int64_t EC = int64_t(p.E) * p.C;
  const int64_t wbytes = int64_t(p.E) * p.d * p.f * p.elem;
  MOE_CHECK(need(x_e, EC * p.d * p.elem, "x_e"));
  MOE_CHECK(need(expert_count, int64_t(p.E) * 4, "expert_count"));
  MOE_CHECK(need(w1, wbytes / p.f * p.w1_rows(), "w1"));
  MOE_CHECK(need(w2, wbytes, "w2"));
  MOE_CHECK(need(y_e, EC * p.d * p.elem, "y_e"));
  MOE_HIP(moe::launch_expert_ffn_fused(p, nspl, x_e, expert_count, w1, w2, y_e,
                                       static_cast<hipStream_t>(stream)),
          "fused expert ffn");
  return MOE_OK;
}

int moe_expert_up(const moe_config* cfg, const void* x_e, const int32_t* expert_count,
                  const void* w1, void* hidden, void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  const int64_t EC = int64_t(p.E) * p.C;
  MOE_CHECK(need(x_e, EC * p.d * p.elem, "x_e"));
  MOE_CHECK(need(expert_count, int64_t(p.E) * 4, "expert_count"));
  MOE_CHECK(need(w1, int64_t(p.E) * p.d * p.w1_rows() * p.elem, "w1"));
  MOE_CHECK(need(hidden, EC * p.f * p.elem, "hidden"));
  MOE_HIP(moe::launch_expert_up(p, x_e, expert_count, w1, hidden, static_cast<hipStream_t>(stream)),
          "expert up-projection");
  return MOE_OK;
}

int moe_expert_down(const moe_config* cfg, const void* hidden, const int32_t* expert_count,
                    const void* w2, void* y_e, void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  const int64_t EC = int64_t(p.E) * p.C;
  MOE_CHECK(need(hidden, EC * p.f * p.elem, "hidden"));
  MOE_CHECK(need(expert_count, int64_t(p.E) * 4, "expert_count"));
  MOE_CHECK(need(w2, int64_t(p.E) * p.d * p.f * p.elem, "w2"));
  MOE_CHECK(need(y_e, EC * p.d * p.elem, "y_e"));
  MOE_HIP(moe::launch_expert_down(p, hidden, expert_count, w2, y_e, static_cast<hipStream_t>(stream)),
          "expert down-projection");
  return MOE_OK;
}

int moe_combine(const moe_config* cfg, const void* y_e, const int32_t* expert_idx,
                const int32_t* slot, const float* gate, void* y, void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  const int64_t Tk = p.T * p.k;
  const int64_t EC = int64_t(p.E) * p.C;
  MOE_CHECK(need(y_e, EC * p.d * p.elem, "y_e"));
  MOE_CHECK(need(expert_idx, Tk * 4, "expert_idx"));
  MOE_CHECK(need(slot, Tk * 4, "slot"));
  MOE_CHECK(need(gate, Tk * 4, "gate"));
  MOE_CHECK(need(y, p.T * p.d * p.elem, "y"));
  MOE_HIP(moe::launch_combine(p, y_e, expert_idx, slot, gate, y, static_cast<hipStream_t>(stream)),
          "combine");
  return MOE_OK;
}

}  // extern "C"

namespace {

int check_forward_args(const moe::Plan& p, const void* x, const float* w_r, const int32_t* group_id,
                       const void* w1, const void* w2, const void* y) {
  const int64_t wbytes = int64_t(p.E) * p.d * p.f * p.elem;
  MOE_CHECK(need(x, p.T * p.d * p.elem, "x"));
  if (p.route == MOE_ROUTE_TOPK) MOE_CHECK(need(w_r, 1, "w_r"));
  else MOE_CHECK(need(group_id, p.T * 4, "group_id"));
  MOE_CHECK(need(w1, wbytes / p.f * p.w1_rows(), "w1"));
  MOE_CHECK(need(w2, wbytes, "w2"));
  MOE_CHECK(need(y, p.T * p.d * p.elem, "y"));
  return MOE_OK;
}

// The launch sequence of the whole layer on the workspace `ws` (validated).
int run_forward(const moe::Plan& p, const void* x, const float* w_r, const float* bias,
                const int32_t* group_id, const void* w1, const void* w2, void* y, void* ws,
                hipStream_t s) {
  char* base = static_cast<char*>(ws);
  auto* expert_idx = reinterpret_cast<int32_t*>(base + p.off_region[MOE_WS_EXPERT_IDX]);
  auto* gate = reinterpret_cast<float*>(base + p.off_region[MOE_WS_GATE]);
  auto* slot = reinterpret_cast<int32_t*>(base + p.off_region[MOE_WS_SLOT]);
  auto* count = reinterpret_cast<int32_t*>(base + p.off_region[MOE_WS_EXPERT_COUNT]);
  auto* slot_token = reinterpret_cast<int32_t*>(base + p.off_region[MOE_WS_SLOT_TOKEN]);
  void* x_e = base + p.off_region[MOE_WS_X_E];
  void* y_e = base + p.off_region[MOE_WS_Y_E];
  MOE_CHECK(run_router(p, x, w_r, bias, group_id, expert_idx, gate, ws, s));
  // the router wrote the per-block histograms; dispatch starts at the scan
  MOE_HIP(moe::launch_dispatch_scan(p, count, slot_token, ws, s), "dispatch scan");
  if (moe::up_reads_token_rows(p)) {
    // the up-projection gathers each slot's row from x itself: slots only, no x_e
    MOE_HIP(moe::launch_dispatch_slot_gather(p, x, expert_idx, slot, slot_token, nullptr, ws, s),
            "dispatch slots");
    MOE_HIP(moe::launch_expert_ffn_rows(p, x, slot_token, count, w1, w2, y_e, ws, s), "expert ffn");
  } else {
    MOE_HIP(moe::launch_dispatch_slot_gather(p, x, expert_idx, slot, slot_token, x_e, ws, s),
            "dispatch slots/gather");
    MOE_HIP(moe::launch_expert_ffn(p, x_e, count, w1, w2, y_e, ws, s), "expert ffn");
  }
  MOE_HIP(moe::launch_combine(p, y_e, expert_idx, slot, gate, y, s), "combine");
  return MOE_OK;
}

static_assert(moe::kNoAllocScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "scratch size");

}  // namespace

extern "C" {

int moe_forward(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
                const int32_t* group_id, const void* w1, const void* w2, void* y, void* ws,
                void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  MOE_CHECK(check_forward_args(p, x, w_r, group_id, w1, w2, y));
  MOE_CHECK(need(ws, p.total, "ws"));
  return run_forward(p, x, w_r, bias, group_id, w1, w2, y, ws, static_cast<hipStream_t>(stream));
}

int moe_forward_noalloc(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
                        const int32_t* group_id, const void* w1, const void* w2, void* y,
                        void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  MOE_CHECK(check_forward_args(p, x, w_r, group_id, w1, w2, y));
  if (p.total > moe::kNoAllocScratchBytes) {
    g_last_error = "moe_forward_noalloc: this configuration needs " + std::to_string(p.total) +
                   " bytes of scratch; the static scratch holds " + std::to_string(moe::kNoAllocScratchBytes) +
                   " (use moe_forward with a workspace)";
    return MOE_ERR_UNSUPPORTED;
  }
  void* ws = nullptr;
  MOE_HIP(moe::noalloc_scratch(&ws), "static scratch address");
  return run_forward(p, x, w_r, bias, group_id, w1, w2, y, ws, static_cast<hipStream_t>(stream));
}

int64_t moe_backward_workspace_bytes(const moe_config* cfg) {
  const int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  moe::Plan p;
  make_plan(cfg, p);
  BwdLayout L;
  bwd_layout(p, L);
  return L.total;
}

int moe_backward(const moe_config* cfg, const void* x, const float* w_r, const float* bias,
                 const void* w1, const void* w2, const void* dy, void* dx, float* dw_r,
                 float* dbias, void* dw1, void* dw2, void* ws, void* bws, void* stream) {
  MOE_CHECK(validate(cfg));
  moe::Plan p;
  make_plan(cfg, p);
  BwdLayout L;
  bwd_layout(p, L);
  const int64_t wbytes = int64_t(p.E) * p.d * p.f * p.elem;
  const int64_t tbytes = p.T * p.d * p.elem;
  const bool topk = p.route == MOE_ROUTE_TOPK;
  MOE_CHECK(need(x, tbytes, "x"));
  if (topk) {
    MOE_CHECK(need(w_r, 1, "w_r"));
    MOE_CHECK(need(dw_r, int64_t(p.E) * p.d * 4, "dw_r"));
  }
  MOE_CHECK(need(w1, wbytes / p.f * p.w1_rows(), "w1"));
  MOE_CHECK(need(w2, wbytes, "w2"));
  MOE_CHECK(need(dy, tbytes, "dy"));
  MOE_CHECK(need(dx, tbytes, "dx"));
  MOE_CHECK(need(dw1, wbytes / p.f * p.w1_rows(), "dw1"));
  MOE_CHECK(need(dw2, wbytes, "dw2"));
  MOE_CHECK(need(ws, p.total, "ws"));
  MOE_CHECK(need(bws, L.total, "bws"));
  char* base = static_cast<char*>(ws);
  char* bb = static_cast<char*>(bws);
  moe::BwdArgs a{};
  a.x = x;
  a.w_r = w_r;
  a.bias = bias;
  a.w1 = w1;
  a.w2 = w2;
  a.dy = dy;
  a.dx = dx;
  a.dw_r = topk ? dw_r : nullptr;
  a.dbias = topk ? dbias : nullptr;
  a.dw1 = dw1;
  a.dw2 = dw2;
  a.expert_idx = reinterpret_cast<const int32_t*>(base + p.off_region[MOE_WS_EXPERT_IDX]);
  a.gate = reinterpret_cast<const float*>(base + p.off_region[MOE_WS_GATE]);
  a.slot = reinterpret_cast<const int32_t*>(base + p.off_region[MOE_WS_SLOT]);
  a.count = reinterpret_cast<const int32_t*>(base + p.off_region[MOE_WS_EXPERT_COUNT]);
  a.x_e = base + p.off_region[MOE_WS_X_E];
  if (moe::up_reads_token_rows(p)) {
    // moe_forward left x_e unwritten (its up-projection read x[slot_token]): the
    // weight gradient of the up-projection needs the gathered rows
    MOE_HIP(moe::launch_gather_slots(p, x, reinterpret_cast<const int32_t*>(base + p.off_region[MOE_WS_SLOT_TOKEN]),
                                     a.count, base + p.off_region[MOE_WS_X_E], static_cast<hipStream_t>(stream)),
            "gather x_e");
  }
  a.hidden = base + p.off_region[MOE_WS_HIDDEN];
  a.y_e = base + p.off_region[MOE_WS_Y_E];
  a.ws = ws;
  a.idx_scratch = reinterpret_cast<int32_t*>(bb + L.idx);
  a.gate_scratch = reinterpret_cast<float*>(bb + L.gate);
  a.dgate = reinterpret_cast<float*>(bb + L.dgate);
  a.dy_e = bb + L.dy_e;
  a.zbuf = bb + L.zbuf;
  a.dz = bb + L.dz;
  a.dx_e = bb + L.dx_e;
  a.dh = reinterpret_cast<float*>(bb + L.dh);
  a.dx_r = reinterpret_cast<float*>(bb + L.dx_r);
  a.dwr_part = reinterpret_cast<float*>(bb + L.dwr_part);
  MOE_HIP(moe::launch_backward(p, a, static_cast<hipStream_t>(stream)), "backward");
  return MOE_OK;
}

int moe_sparse_clip(const moe_config* cfg, float* dw_r, float* dbias, void* dw1, void* dw2,
                    double max_norm, float* norm_coef, void* bws, void* stream) {
  MOE_CHECK(validate(cfg));
  if (!(max_norm > 0.0) || !std::isfinite(max_norm))
    return fail(MOE_ERR_ARG, "max_norm must be finite and > 0");
  moe::Plan p;
  make_plan(cfg, p);
  BwdLayout L;
  bwd_layout(p, L);
  const int64_t wbytes = int64_t(p.E) * p.d * p.f * p.elem;
  MOE_CHECK(need(dw1, wbytes / p.f * p.w1_rows(), "dw1"));
  MOE_CHECK(need(dw2, wbytes, "dw2"));
  MOE_CHECK(need(norm_coef, 8, "norm_coef"));
  MOE_CHECK(need(bws, L.total, "bws"));
  MOE_HIP(moe::launch_sparse_clip(p, dw_r, dbias, dw1, dw2, max_norm, norm_coef,
                                  static_cast<char*>(bws) + L.clip, static_cast<hipStream_t>(stream)),
          "sparse clip");
  return MOE_OK;
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_version(void) { return "moe-mi355x 0.1.0 (gfx950)"; }

}  // extern "C"
