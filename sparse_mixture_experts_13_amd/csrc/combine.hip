// Combine (Switch Transformers notes, section 2.1, Eq. 2): the layer output of a
// token is the gate-weighted sum of the outputs of the experts it was served by,
// y[t] = sum_c gate[t,c] * y_e[expert_idx[t,c], slot[t,c]] over served choices,
// accumulated in float32 in choice order; a token with no served choice gets 0
// (section 2.2: a dropped token continues only through the residual).
//
// Token-major pull: one wave per token, 16-byte vector loads of each served
// expert row, one coalesced row store.  Every y element is written exactly once.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

// Eight output values with non-temporal stores: y is the layer's result, not read
// again here, and at these sizes it does not stay in L2 for the next reader anyway
// (Switch-Base combine 9.7 -> 9.0 us, step 0.2992 -> 0.2980 ms).
__device__ __forceinline__ void store8_nt(bf16_t* p, const float* v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store8_nt(float* p, const float* v) {
  __builtin_nontemporal_store(floatx4{v[0], v[1], v[2], v[3]}, reinterpret_cast<floatx4*>(p));
  __builtin_nontemporal_store(floatx4{v[4], v[5], v[6], v[7]}, reinterpret_cast<floatx4*>(p + 4));
}

template <typename T, int CH>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y_e,
                                                      const int32_t* __restrict__ expert_idx,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ gate, int ntok,
                                                      int E, int k, int64_t C, int64_t d,
                                                      T* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  // served choices in choice order: lane c loads choice c (one memory round trip
  // for all of them), readlane hands each to the whole wave; fully unrolled so the
  // arrays stay in registers
  int sl = -1, el = -1;
  float gl = 0.f;
  if (lane < k) {
    const int64_t o = static_cast<int64_t>(t) * k + lane;
    sl = slot[o];
    el = expert_idx[o];
    gl = gate[o];
  }
  int64_t off[kMaxK];
  float g[kMaxK];
#pragma unroll
  for (int c = 0; c < kMaxK; ++c) {
    const int s = __builtin_amdgcn_readlane(sl, c);
    const int e = __builtin_amdgcn_readlane(el, c);
    const bool ok = c < k && s >= 0 && s < C && e >= 0 && e < E;
    off[c] = ok ? (e * C + s) * d : -1;
    g[c] = ok ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gl), c)) : 0.f;
  }
  T* dst = y + static_cast<int64_t>(t) * d;
  // CH 8-element chunks per lane: the loads of a choice issue together (a lane
  // past the row end reads the last chunk again and stores nothing), all stores
  // after all loads (a load issued after a store also waits for that store:
  // loads and stores share vmcnt); per element the choices add in choice order
  const int64_t nch = d / 8;
  for (int64_t v0 = lane; v0 < nch; v0 += kWave * CH) {
    float acc[CH][8];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[j][i] = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxK; ++c) {
      if (off[c] >= 0) {
        float r[CH][8];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const int64_t v = min(v0 + j * kWave, nch - 1);
          vec8<T>::load(y_e + off[c] + v * 8, r[j]);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j][i] = fmaf(g[c], r[j][i], acc[j][i]);
      }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int64_t v = v0 + j * kWave;
      if (v < nch) store8_nt(dst + v * 8, acc[j]);
    }
  }
}

template <typename T, int CH>
static void run_combine(const Plan& p, const void* y_e, const int32_t* expert_idx,
                        const int32_t* slot, const float* gate, void* y, hipStream_t s) {
  const int nblk = static_cast<int>((p.T + 3) / 4);
  hipLaunchKernelGGL((combine_kernel<T, CH>), dim3(nblk), dim3(256), 0, s,
                     static_cast<const T*>(y_e), expert_idx, slot, gate, static_cast<int>(p.T), p.E,
                     p.k, p.C, p.d, static_cast<T*>(y));
}

template <typename T>
static void run_combine_typed(const Plan& p, const void* y_e, const int32_t* expert_idx,
                              const int32_t* slot, const float* gate, void* y, hipStream_t s) {
  // chunks per lane: enough for the row in one pass up to 256 chunks (2048 elements)
  const int64_t per_lane = (p.d / 8 + kWave - 1) / kWave;
  if (per_lane <= 1) run_combine<T, 1>(p, y_e, expert_idx, slot, gate, y, s);
  else if (per_lane <= 2) run_combine<T, 2>(p, y_e, expert_idx, slot, gate, y, s);
  else run_combine<T, 4>(p, y_e, expert_idx, slot, gate, y, s);
}

hipError_t launch_combine(const Plan& p, const void* y_e, const int32_t* expert_idx,
                          const int32_t* slot, const float* gate, void* y, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (p.dtype == 1) run_combine_typed<bf16_t>(p, y_e, expert_idx, slot, gate, y, s);
  else run_combine_typed<float>(p, y_e, expert_idx, slot, gate, y, s);
  return hipGetLastError();
}

}  // namespace moe
