// Host-side launch interface between the C ABI (moe_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxRouterBlock = 128;  // tokens per router block (histogram granularity): 32, 64 or 128
constexpr int kMaxE = 512;
constexpr int kMaxK = 8;
constexpr int kSplitBlocks = 64;   // blocks of the router-weight split kernel

// Sizes derived once from a validated configuration.
struct Plan {
  int64_t T, d, f, C;
  int E, k, Epad, NB;      // Epad: E rounded up to 32; NB: router blocks of TB tokens
  int TB;                  // tokens per router block
  int dtype, act, route, n_groups;  // act: 0 ReLU, 1 GELU (the GLU forms set glu)
  bool glu;                // gated-linear-unit FFN: w1 holds [W; V], 2 f rows
  uint64_t rre_seed;
  int elem;                // bytes per element of dtype
  int64_t w1_rows() const { return glu ? 2 * f : f; }
  // workspace byte offsets
  int64_t off_region[8];
  int64_t off_hist, off_offsets, off_planes, off_flags, off_psum, total;
};

// router.hip
hipError_t launch_router_split(const Plan& p, const float* w_r, void* ws, hipStream_t s);
// with_psum: also write the per-block expert probability sums (load-balancing loss)
// logits (may be null): also write the float32 logits (bias included) [T][Epad]
hipError_t launch_router_topk(const Plan& p, const void* x, const float* w_r, const float* bias,
                              int32_t* expert_idx, float* gate, void* ws, hipStream_t s,
                              bool with_psum = false, float* logits = nullptr);
// aux = [alpha * E * sum_i f_i P_i, f[E], P[E]] from the router's block rows
hipError_t launch_router_aux(const Plan& p, double alpha, float* aux, void* ws, hipStream_t s);
// Load-balancing workspace: per router block a float row of Epad probability
// sums, then kAuxSplit rows of float64 sums and kAuxSplit rows of int64 counts.
constexpr int kAuxSplit = 64;
inline int64_t aux_rows_bytes(const Plan& p) { return (int64_t(p.NB) * p.Epad * 4 + 255) / 256 * 256; }
inline int64_t aux_region_bytes(const Plan& p) { return aux_rows_bytes(p) + int64_t(kAuxSplit) * p.Epad * 16; }
hipError_t launch_router_rre(const Plan& p, const int32_t* group_id, int32_t* expert_idx,
                             float* gate, void* ws, hipStream_t s);

// dispatch.hip
hipError_t launch_dispatch_hist(const Plan& p, const int32_t* expert_idx, void* ws, hipStream_t s);
hipError_t launch_dispatch_scan(const Plan& p, int32_t* expert_count, int32_t* slot_token, void* ws,
                                hipStream_t s);
// x_e null: slots only (slot, slot_token), no row copy
hipError_t launch_dispatch_slot_gather(const Plan& p, const void* x, const int32_t* expert_idx,
                                       int32_t* slot, int32_t* slot_token, void* x_e, void* ws,
                                       hipStream_t s);
// x_e[e, s] = x[slot_token[e, s]] for s < expert_count[e]
hipError_t launch_gather_slots(const Plan& p, const void* x, const int32_t* slot_token,
                               const int32_t* expert_count, void* x_e, hipStream_t s);

// expert_ffn.hip
hipError_t launch_expert_ffn(const Plan& p, const void* x_e, const int32_t* expert_count,
                             const void* w1, const void* w2, void* y_e, void* ws, hipStream_t s);
hipError_t launch_expert_up(const Plan& p, const void* x_e, const int32_t* expert_count,
                            const void* w1, void* hidden, hipStream_t s);
// True where the up-projection can read each slot's activation row from the
// token rows x through slot_token instead of from x_e: the resident-activation
// GEMM (bf16, capacity <= 64, d_model <= 768, E <= 512) and the two-slot ring
// (bf16, capacity > 160, d_model < 2048).
bool up_reads_token_rows(const Plan& p);
// The expert FFN of launch_expert_ffn with the up-projection reading x[slot_token]
// (only where up_reads_token_rows holds; hipErrorInvalidValue elsewhere).
hipError_t launch_expert_ffn_rows(const Plan& p, const void* x, const int32_t* slot_token,
                                  const int32_t* expert_count, const void* w1, const void* w2,
                                  void* y_e, void* ws, hipStream_t s);
// Fused FFN (bf16, capacity <= 64): column groups per expert, 0 if not applicable:
// bf16, capacity <= 64, d_ff a multiple of the 128-column hidden chunk, and d_model a
// multiple of 384 split into column groups of 384 (two 192-column accumulator tiles
// per wave: 64 registers per lane; wider groups spill).
constexpr int kFusedFC = 128;  // d_ff chunk per hidden tile
inline int fused_ffn_split(const Plan& p) {
  if (p.glu || p.dtype != 1 || p.C > 64 || p.C < 1 || p.f % kFusedFC != 0 || p.d % 384 != 0) return 0;
  if (p.d * p.f >= (int64_t(1) << 31)) return 0;  // 32-bit offsets inside one expert
  return static_cast<int>(p.d / 384);
}
// y_e = act(x_e W1) W2 in one launch, the hidden activations kept on chip.
hipError_t launch_expert_ffn_fused(const Plan& p, int nspl, const void* x_e,
                                   const int32_t* expert_count, const void* w1, const void* w2,
                                   void* y_e, hipStream_t s);
hipError_t launch_expert_down(const Plan& p, const void* hidden, const int32_t* expert_count,
                              const void* w2, void* y_e, hipStream_t s);

// Up-projection with an explicit activation (2: none, for the pre-activation).
hipError_t launch_expert_up_act(const Plan& p, const void* x_e, const int32_t* expert_count,
                                const void* w1, void* out, int act, hipStream_t s);
// Backward token-row product out[e][m][n] = sum_k A[e][m][k] B[e][k][n] (A [C][K],
// B [K][N], out [C][N] per expert; rows m < count[e]) on the ping-pong GEMM, times
// act'(aux[e][m][n]) for grad_act 0 (ReLU) or 1 (GELU), plain for grad_act -1.
// hipErrorNotSupported where that kernel does not apply (the caller falls back):
// bf16 only, K >= 1024, capacity > 160 (> 64 when N >= 2048), 32-bit offsets.
hipError_t launch_bwd_rows_pp(const Plan& p, const uint16_t* A, const uint16_t* B, uint16_t* out,
                              const uint16_t* aux, const int32_t* count, int N, int K, int grad_act,
                              hipStream_t s);

// backward.hip
constexpr int kBwdSplit = 64;  // token ranges of the router weight gradient
struct BwdArgs {
  // inputs and outputs of the call
  const void* x;
  const float* w_r;
  const float* bias;
  const void* w1;
  const void* w2;
  const void* dy;
  void* dx;
  float* dw_r;
  float* dbias;
  void* dw1;
  void* dw2;
  // the forward's results (forward workspace)
  const int32_t* expert_idx;
  const float* gate;
  const int32_t* slot;
  const int32_t* count;
  const void* x_e;
  const void* hidden;
  const void* y_e;
  void* ws;
  // backward scratch
  int32_t* idx_scratch;
  float* gate_scratch;
  float* dgate;
  void* dy_e;
  void* zbuf;
  void* dz;
  void* dx_e;
  float* dh;
  float* dx_r;
  float* dwr_part;
};
hipError_t launch_backward(const Plan& p, const BwdArgs& a, hipStream_t s);
// SparseClip in place; norm_coef = [norm, coef] (device floats); part: 4 x 512 doubles
constexpr int64_t kClipScratchBytes = 4 * 512 * 8;
hipError_t launch_sparse_clip(const Plan& p, float* dw_r, float* dbias, void* dw1, void* dw2,
                              double max_norm, float* norm_coef, void* part, hipStream_t s);

// combine.hip
hipError_t launch_combine(const Plan& p, const void* y_e, const int32_t* expert_idx,
                          const int32_t* slot, const float* gate, void* y, hipStream_t s);

// scratch.hip: the static per-device scratch of moe_forward_noalloc.
constexpr int64_t kNoAllocScratchBytes = 80LL << 20;
// Device address of the scratch array on the current device (looked up once per
// device, then cached); hipErrorInvalidDevice for a device ordinal past 63.
hipError_t noalloc_scratch(void** out);

inline char* ws_at(void* ws, int64_t off) { return static_cast<char*>(ws) + off; }

}  // namespace moe
