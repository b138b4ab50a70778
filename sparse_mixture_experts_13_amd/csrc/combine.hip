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

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y_e,
                                                      const int32_t* __restrict__ expert_idx,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ gate, int ntok,
                                                      int E, int k, int64_t C, int64_t d,
                                                      T* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  // served choices in choice order; fully unrolled so the arrays stay in registers
  int64_t off[kMaxK];
  float g[kMaxK];
#pragma unroll
  for (int c = 0; c < kMaxK; ++c) {
    off[c] = -1;
    g[c] = 0.f;
    if (c < k) {
      const int64_t o = static_cast<int64_t>(t) * k + c;
      const int s = slot[o];
      const int e = expert_idx[o];
      if (s >= 0 && s < C && e >= 0 && e < E) {
        off[c] = (e * C + s) * d;
        g[c] = gate[o];
      }
    }
  }
  T* dst = y + static_cast<int64_t>(t) * d;
  for (int64_t v = lane; v < d / 8; v += kWave) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxK; ++c) {
      if (off[c] >= 0) {
        float r[8];
        vec8<T>::load(y_e + off[c] + v * 8, r);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(g[c], r[i], acc[i]);
      }
    }
    vec8<T>::store(dst + v * 8, acc);
  }
}

hipError_t launch_combine(const Plan& p, const void* y_e, const int32_t* expert_idx,
                          const int32_t* slot, const float* gate, void* y, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const int nblk = static_cast<int>((p.T + 3) / 4);
  if (p.dtype == 1)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3(nblk), dim3(256), 0, s,
                       static_cast<const bf16_t*>(y_e), expert_idx, slot, gate,
                       static_cast<int>(p.T), p.E, p.k, p.C, p.d, static_cast<bf16_t*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(nblk), dim3(256), 0, s,
                       static_cast<const float*>(y_e), expert_idx, slot, gate,
                       static_cast<int>(p.T), p.E, p.k, p.C, p.d, static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace moe
