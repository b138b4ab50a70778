// Grouped expert FFN: y_e = act(x_e W1_e) W2_e for every expert at once
// (Switch Transformers notes, section 2.1: one feed-forward network E_i per
// expert; section 2.2: each expert computes a static-capacity batch, of which
// only the first expert_count[e] rows hold tokens).
//
// Two launches of one grouped GEMM: hidden = act(x_e . w1[e]^T), then
// y_e = hidden . w2[e]^T.  Both operands are stored K-contiguous (activations
// [E][C][K], weights [E][N][K]), so the MFMA A and B fragments are 16-byte row
// reads.  The kernel computes the transposed tile D = W . X^T so that each lane
// ends with four consecutive output columns of one row (8-byte stores).
//
// gfx950: v_mfma_f32_32x32x16_bf16 with float32 accumulation; LDS-staged,
// double-buffered tiles (BK = 64, rows padded to 144 bytes so the fragment reads
// are bank-conflict free); one block per (expert, row tile, column tile); tiles
// whose first row is past the expert's token count exit at once, so the grid is
// static (no device-to-host read of the counts) while dropped capacity costs no
// MFMA work.  float32 workloads use a plain float32 FMA tile kernel.
#include "moe_common.h"
#include "moe_internal.h"

#include <algorithm>

namespace moe {

constexpr int GBK = 64;
constexpr int GLD = GBK + 8;

template <int BM, int BN>
__host__ __device__ constexpr int ffn_lds_bytes() {
  return 2 * (BM + BN) * GLD * 2;
}

template <int BM, int BN, int WM, int WN, int ACT>
__global__ __launch_bounds__(256) void ffn_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, bf16_t* __restrict__ out,
    const int32_t* __restrict__ count, int64_t C, int N, int K, int n_mt, int n_nt) {
  static_assert(WM * WN == 4, "four waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int QL = BM * 8 / 256, PL = BN * 8 / 256;
  static_assert(TM >= 1 && TN >= 1 && QL >= 1 && PL >= 1, "tile shape");

  extern __shared__ __align__(16) unsigned char smem[];
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem);  // [2][BM][GLD] activations
  bf16_t* sP = sQ + 2 * BM * GLD;                // [2][BN][GLD] weights

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int id = blockIdx.x;
  const int per_e = n_mt * n_nt;
  const int e = id / per_e;
  id -= e * per_e;
  const int mt = id / n_nt;
  const int nt = id - mt * n_nt;
  int64_t cnt64 = count[e];
  cnt64 = cnt64 < 0 ? 0 : (cnt64 > C ? C : cnt64);
  const int cnt = static_cast<int>(cnt64);
  const int m0 = mt * BM;
  if (m0 >= cnt) return;
  const int n0 = nt * BN;

  const bf16_t* Ae = A + (static_cast<int64_t>(e) * C + m0) * K;
  const bf16_t* We = W + (static_cast<int64_t>(e) * N + n0) * K;

  u32x4 rq[QL], rp[PL];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const int cid = tid + 256 * i, r = cid >> 3, c = cid & 7;
      rq[i] = m0 + r < cnt ? *reinterpret_cast<const u32x4*>(Ae + static_cast<int64_t>(r) * K + k0 + c * 8)
                           : zero4;
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int cid = tid + 256 * i, r = cid >> 3, c = cid & 7;
      rp[i] = n0 + r < N ? *reinterpret_cast<const u32x4*>(We + static_cast<int64_t>(r) * K + k0 + c * 8)
                         : zero4;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const int cid = tid + 256 * i, r = cid >> 3, c = cid & 7;
      *reinterpret_cast<u32x4*>(sQ + (buf * BM + r) * GLD + c * 8) = rq[i];
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int cid = tid + 256 * i, r = cid >> 3, c = cid & 7;
      *reinterpret_cast<u32x4*>(sP + (buf * BN + r) * GLD + c * 8) = rp[i];
    }
  };

  floatx16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  const int KT = K / GBK;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * GBK);
#pragma unroll
    for (int k16 = 0; k16 < GBK / 16; ++k16) {
      bf16x8 pa[TN], qb[TM];
#pragma unroll
      for (int i = 0; i < TN; ++i)
        pa[i] = *reinterpret_cast<const bf16x8*>(sP + (buf * BN + wn * WTN + i * 32 + fr) * GLD + k16 * 16 + fk);
#pragma unroll
      for (int j = 0; j < TM; ++j)
        qb[j] = *reinterpret_cast<const bf16x8*>(sQ + (buf * BM + wm * WTM + j * 32 + fr) * GLD + k16 * 16 + fk);
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[i], qb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // D[n][m] of each 32x32 tile: lane holds m = lane % 32 and, for accumulator
  // element r, n = 8*(r/4) + 4*(lane/32) + r%4: four consecutive columns per group.
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int m = m0 + wm * WTM + j * 32 + fr;
    if (m < cnt) {
      bf16_t* orow = out + (static_cast<int64_t>(e) * C + m) * N;
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WTN + i * 32 + 8 * g + 4 * (lane >> 5);
          if (n < N) {
            uint2 v;
            v.x = pack_bf16x2(apply_act<ACT>(acc[i][j][4 * g]), apply_act<ACT>(acc[i][j][4 * g + 1]));
            v.y = pack_bf16x2(apply_act<ACT>(acc[i][j][4 * g + 2]), apply_act<ACT>(acc[i][j][4 * g + 3]));
            *reinterpret_cast<uint2*>(orow + n) = v;
          }
        }
    }
  }
}

// float32 grouped GEMM: 64 x 64 tile, 4 x 4 outputs per thread, BK = 16.
template <int ACT>
__global__ __launch_bounds__(256) void ffn_gemm_f32_kernel(const float* __restrict__ A,
                                                           const float* __restrict__ W,
                                                           float* __restrict__ out,
                                                           const int32_t* __restrict__ count,
                                                           int64_t C, int N, int K, int n_mt,
                                                           int n_nt) {
  __shared__ float sA[64][17];
  __shared__ float sB[64][17];
  const int tid = threadIdx.x;
  int id = blockIdx.x;
  const int per_e = n_mt * n_nt;
  const int e = id / per_e;
  id -= e * per_e;
  const int mt = id / n_nt;
  const int nt = id - mt * n_nt;
  int64_t cnt64 = count[e];
  cnt64 = cnt64 < 0 ? 0 : (cnt64 > C ? C : cnt64);
  const int cnt = static_cast<int>(cnt64);
  const int m0 = mt * 64, n0 = nt * 64;
  if (m0 >= cnt) return;
  const float* Ae = A + (static_cast<int64_t>(e) * C + m0) * K;
  const float* We = W + (static_cast<int64_t>(e) * N + n0) * K;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 4, c = q & 15;
      sA[r][c] = m0 + r < cnt ? Ae[static_cast<int64_t>(r) * K + k0 + c] : 0.f;
      sB[r][c] = n0 + r < N ? We[static_cast<int64_t>(r) * K + k0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[ty + 16 * i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[tx + 16 * j][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m < cnt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx + 16 * j;
        if (n < N) out[(static_cast<int64_t>(e) * C + m) * N + n] = apply_act<ACT>(acc[i][j]);
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int ACT>
static hipError_t run_bf16(int E, const bf16_t* A, const bf16_t* W, bf16_t* out,
                           const int32_t* count, int64_t C, int N, int K, hipStream_t s) {
  auto kern = ffn_gemm_bf16_kernel<BM, BN, WM, WN, ACT>;
  constexpr int lds = ffn_lds_bytes<BM, BN>();
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int n_mt = static_cast<int>((C + BM - 1) / BM);
  const int n_nt = (N + BN - 1) / BN;
  const int64_t nblk = static_cast<int64_t>(E) * n_mt * n_nt;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nblk)), dim3(256), lds, s, A, W, out, count,
                     C, N, K, n_mt, n_nt);
  return hipGetLastError();
}

template <int ACT>
static hipError_t run_f32(int E, const float* A, const float* W, float* out, const int32_t* count,
                          int64_t C, int N, int K, hipStream_t s) {
  const int n_mt = static_cast<int>((C + 63) / 64);
  const int n_nt = (N + 63) / 64;
  const int64_t nblk = static_cast<int64_t>(E) * n_mt * n_nt;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(ffn_gemm_f32_kernel<ACT>, dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s,
                     A, W, out, count, C, N, K, n_mt, n_nt);
  return hipGetLastError();
}

template <int ACT>
static hipError_t gemm_bf16(const Plan& p, const bf16_t* A, const bf16_t* W, bf16_t* out,
                            const int32_t* count, int N, int K, hipStream_t s) {
  if (p.C <= 64) return run_bf16<64, 128, 1, 4, ACT>(p.E, A, W, out, count, p.C, N, K, s);
  return run_bf16<128, 128, 2, 2, ACT>(p.E, A, W, out, count, p.C, N, K, s);
}

hipError_t launch_expert_up(const Plan& p, const void* x_e, const int32_t* expert_count,
                            const void* w1, void* hidden, hipStream_t s) {
  if (p.C == 0) return hipSuccess;
  const int d = static_cast<int>(p.d), f = static_cast<int>(p.f);
  if (p.dtype == 1) {
    const bf16_t* xe = static_cast<const bf16_t*>(x_e);
    const bf16_t* w = static_cast<const bf16_t*>(w1);
    bf16_t* h = static_cast<bf16_t*>(hidden);
    return p.act == 0 ? gemm_bf16<0>(p, xe, w, h, expert_count, f, d, s)
                      : gemm_bf16<1>(p, xe, w, h, expert_count, f, d, s);
  }
  const float* xe = static_cast<const float*>(x_e);
  const float* w = static_cast<const float*>(w1);
  float* h = static_cast<float*>(hidden);
  return p.act == 0 ? run_f32<0>(p.E, xe, w, h, expert_count, p.C, f, d, s)
                    : run_f32<1>(p.E, xe, w, h, expert_count, p.C, f, d, s);
}

hipError_t launch_expert_down(const Plan& p, const void* hidden, const int32_t* expert_count,
                              const void* w2, void* y_e, hipStream_t s) {
  if (p.C == 0) return hipSuccess;
  const int d = static_cast<int>(p.d), f = static_cast<int>(p.f);
  if (p.dtype == 1)
    return gemm_bf16<2>(p, static_cast<const bf16_t*>(hidden), static_cast<const bf16_t*>(w2),
                        static_cast<bf16_t*>(y_e), expert_count, d, f, s);
  return run_f32<2>(p.E, static_cast<const float*>(hidden), static_cast<const float*>(w2),
                    static_cast<float*>(y_e), expert_count, p.C, d, f, s);
}

hipError_t launch_expert_ffn(const Plan& p, const void* x_e, const int32_t* expert_count,
                             const void* w1, const void* w2, void* y_e, void* ws, hipStream_t s) {
  void* hidden = ws_at(ws, p.off_region[6]);
  const hipError_t err = launch_expert_up(p, x_e, expert_count, w1, hidden, s);
  if (err != hipSuccess) return err;
  return launch_expert_down(p, hidden, expert_count, w2, y_e, s);
}

}  // namespace moe
