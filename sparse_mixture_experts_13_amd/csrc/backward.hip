// Backward pass of the layer: gradients of y = sum over served choices of
// p_i(x) E_i(x) (Switch Transformers notes, section 2.1, Eq. 2; the gate keeps
// the router differentiable), with E_i(x) = act(x W1_i) W2_i and p = softmax(h)
// of the router logits h = W_r x (+ bias) (Eq. 1).  The chosen set and the
// capacity drop (section 2.2) are piecewise constant: no gradient flows
// through them, and a dropped choice contributes nothing.
//
// Given dy = dL/dy, per served choice (token t, expert e, slot s):
//   dy_e[e,s] = p * dy[t]                    dgate[t,c] = dy[t] . y_e[e,s]
//   dZ = (dy_e W2_e^T-contraction) * act'(Z)  i.e. dZ[s,f] = sum_d dy_e[s,d] w2[e][d][f] * act'(Z[s,f])
//   dx_e[s,d] = sum_f dZ[s,f] w1[e][f][d]
//   dw2[e][d][f] = sum_s dy_e[s,d] H[s,f]    dw1[e][f][d] = sum_s dZ[s,f] x_e[s,d]
//   router: dp_e = sum of dgate over the choices of e, dh = p (dp - <p, dp>),
//           dx += dh W_r, dw_r = dh^T x, dbias = sum_t dh
//   dx[t] = sum over served choices of dx_e[e,s], plus the router term.
// GLU experts (MosaicBERT review, methodology), H = act(Za) * Zb with
// (Za, Zb) = x_e [W; V]^T: dZa = dH * Zb * act'(Za), dZb = dH * act(Za), and
// dZ = (dZa, dZb) takes the place of dZ over the 2 f stacked rows of w1.
//
// gfx950 design.  Scatter, softmax-Jacobian and final gather are one wave per
// token.  All four expert products run on one grouped GEMM kernel with operand
// orientation as template flags: an operand stored k-contiguous is staged in
// LDS as [row][k] and read as 16-byte MFMA fragments; an operand stored
// row-contiguous (the weights in dH = dy_e . w2 and dx_e = dZ . w1, and both
// token-major operands of the weight gradients, whose contraction runs over
// the tokens of an expert) is staged as [k][row] with 16-byte stores and read
// with two LDS transpose reads (ds_read_b64_tr_b16) per fragment.
// Register-staged double buffering, 64-k steps (32 for the token-contracted
// ones), v_mfma_f32_32x32x16_bf16 with float32 accumulation, D = B . A^T
// so each lane stores four consecutive output columns.  act' is applied in the
// dH epilogue (from the hidden activation for ReLU, from the recomputed
// pre-activation for GELU).  The router products (K = E or K = T) and the
// float32 layers use a float32 MFMA tile kernel (v_mfma_f32_32x32x2_f32) with
// the same orientation flags; the token-contracted router weight gradient is
// split over up to 64 token ranges and the ranges are added in order
// (deterministic, no atomics).
#include "moe_common.h"
#include "moe_internal.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace moe {

// ---------------------------------------------------------------------------
// dy_e = gate * dy (expert-major) and dgate = dy . y_e; one wave per token
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_scatter_kernel(
    const T* __restrict__ dy, const T* __restrict__ y_e, const int32_t* __restrict__ expert_idx,
    const int32_t* __restrict__ slot, const float* __restrict__ gate, int ntok, int E, int k,
    int64_t C, int64_t d, T* __restrict__ dy_e, float* __restrict__ dgate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const T* drow = dy + static_cast<int64_t>(t) * d;
  for (int c = 0; c < k; ++c) {
    const int64_t o = static_cast<int64_t>(t) * k + c;
    const int s = slot[o];
    const int e = expert_idx[o];
    if (!(s >= 0 && s < C && e >= 0 && e < E)) {
      if (lane == 0) dgate[o] = 0.f;
      continue;
    }
    const float g = gate[o];
    const int64_t row = (static_cast<int64_t>(e) * C + s) * d;
    float dot = 0.f;
    for (int64_t v = lane; v < d / 8; v += kWave) {
      float a[8], b[8];
      vec8<T>::load(drow + v * 8, a);
      vec8<T>::load(y_e + row + v * 8, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = fmaf(a[i], b[i], dot);
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = g * a[i];
      vec8<T>::store(dy_e + row + v * 8, a);
    }
    dot = wave_sum(dot);
    if (lane == 0) dgate[o] = dot;
  }
}

// ---------------------------------------------------------------------------
// Softmax Jacobian: logits row -> dh = p * (dp - <p, dp>), in place (float32,
// p computed as in the forward router: exp(h - max) / sum); one wave per token
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_router_softmax_kernel(
    float* __restrict__ hrow, int ldh, const int32_t* __restrict__ expert_idx,
    const int32_t* __restrict__ slot, const float* __restrict__ dgate, int ntok, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  float* row = hrow + static_cast<int64_t>(t) * ldh;
  constexpr int NV = kMaxE / kWave;
  float h[NV], dp[NV];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    h[i] = e < E ? row[e] : -INFINITY;
    dp[i] = 0.f;
    m = fmaxf(m, h[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  for (int c = 0; c < k; ++c) {
    const int64_t o = static_cast<int64_t>(t) * k + c;
    const int e = expert_idx[o];
    if (slot[o] >= 0 && e >= 0 && e < E) {
      const float g = dgate[o];
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane + kWave * i == e) dp[i] += g;
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) sum += expf(h[i] - m);  // exp(-inf) = 0
  sum = wave_sum(sum);
  float p[NV], pd = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    p[i] = expf(h[i] - m) / sum;
    pd = fmaf(p[i], dp[i], pd);
  }
  pd = wave_sum(pd);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + kWave * i;
    if (e < ldh) row[e] = e < E ? p[i] * (dp[i] - pd) : 0.f;
  }
}

// ---------------------------------------------------------------------------
// dx[t] = sum over served choices of dx_e[e, s] (+ the router term, float32)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bwd_gather_kernel(
    const T* __restrict__ dx_e, const float* __restrict__ dx_r, const int32_t* __restrict__ expert_idx,
    const int32_t* __restrict__ slot, int ntok, int E, int k, int64_t C, int64_t d,
    T* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  int64_t off[kMaxK];
#pragma unroll
  for (int c = 0; c < kMaxK; ++c) {
    off[c] = -1;
    if (c < k) {
      const int64_t o = static_cast<int64_t>(t) * k + c;
      const int s = slot[o], e = expert_idx[o];
      if (s >= 0 && s < C && e >= 0 && e < E) off[c] = (static_cast<int64_t>(e) * C + s) * d;
    }
  }
  for (int64_t v = lane; v < d / 8; v += kWave) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxK; ++c) {
      if (off[c] >= 0) {
        float r[8];
        vec8<T>::load(dx_e + off[c] + v * 8, r);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += r[i];
      }
    }
    if (dx_r) {
      float r[8];
      vec8<float>::load(dx_r + static_cast<int64_t>(t) * d + v * 8, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += r[i];
    }
    vec8<T>::store(dx + static_cast<int64_t>(t) * d + v * 8, acc);
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM with operand orientation flags (bf16, MFMA).
//   out[e][m][n] = epi( sum_k A(e, m, k) B(e, n, k) )
//   A(e,m,k) = A[e * sAe + (AKC ? m * lda + k : k * lda + m)], same for B.
// Per expert e: rows m < M_e, columns n < N, k < K_e, where either M_e or K_e
// is the expert's token count (clamped to C) and the other is fixed; with
// M_e = count, M is the row extent of the buffers (C), read but not stored past
// the count.  Loads past the valid k range read as zero.  A K_e = 0 expert
// stores zeros (weight gradients of an expert with no tokens).
// EPI 0: store bf16(acc).  EPI 1: bf16(acc * act'(z)) with z read from `aux`
// at the output position (ACT 0: z is the hidden activation, act' = z > 0;
// ACT 1: z is the pre-activation, act' = GELU derivative).  EPI 2 (GLU, acc =
// dH): with za = aux[m][n] and zb = aux[m][N + n] (aux and out have row pitch
// ldo = 2 N), stores bf16(acc * zb * act'(za)) at out[m][n] and
// bf16(acc * act(za)) at out[m][N + n].
// ---------------------------------------------------------------------------

template <int ROWS, bool KC, int BK>
struct OpTile {
  // LDS elements per buffer: [ROWS][BK + 8] (k-contiguous) or [BK][ROWS + 8]
  static constexpr int kPitch = KC ? BK + 8 : ROWS + 8;
  static constexpr int kElems = KC ? ROWS * (BK + 8) : BK * (ROWS + 8);
  static constexpr int kChunks = ROWS * BK / 8;  // 16-byte chunks per tile
};

template <int BM, int BN, int BK, bool AKC, bool BKC, int EPI, int ACT>
__global__ __launch_bounds__(256) void bgemm_kernel(
    const bf16_t* __restrict__ A, int64_t sAe, int lda, const bf16_t* __restrict__ B, int64_t sBe,
    int ldb, bf16_t* __restrict__ out, int64_t sOe, int ldo, const bf16_t* __restrict__ aux,
    const int32_t* __restrict__ count, int64_t C, int M, int N, int K, bool m_is_count) {
  using TA = OpTile<BM, AKC, BK>;
  using TBt = OpTile<BN, BKC, BK>;
  static_assert(TA::kChunks % 256 == 0 && TBt::kChunks % 256 == 0, "chunk split");
  constexpr int CA = TA::kChunks / 256, CB = TBt::kChunks / 256;
  constexpr int TM = BM / 64, TN = BN / 64;  // 32-row MFMA tiles per wave (2 x 2 waves)
  // operand double buffers, reused after the k loop as the output staging tile
  constexpr int OP = BN + 8;  // staging row pitch (elements)
  constexpr int kSmem = 2 * (TA::kElems + TBt::kElems) > BM * OP ? 2 * (TA::kElems + TBt::kElems) : BM * OP;
  __shared__ __align__(16) bf16_t smem_[kSmem];
  bf16_t (*la)[TA::kElems] = reinterpret_cast<bf16_t (*)[TA::kElems]>(smem_);
  bf16_t (*lb)[TBt::kElems] = reinterpret_cast<bf16_t (*)[TBt::kElems]>(smem_ + 2 * TA::kElems);

  const int bx = blockIdx.x, by = blockIdx.y, e = blockIdx.z;
  int64_t cnt = count[e];
  cnt = cnt < 0 ? 0 : (cnt > C ? C : cnt);
  const int Mv = m_is_count ? static_cast<int>(cnt) : M;
  const int Kv = m_is_count ? K : static_cast<int>(cnt);
  const int m0 = by * BM, n0 = bx * BN;
  if (m0 >= Mv) return;
  const bf16_t* Ae = A + e * sAe;
  const bf16_t* Be = B + e * sBe;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, fr = lane & 31;

  u32x4 ra[CA], rb[CB];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = tid + 256 * i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if constexpr (AKC) {
        const int r = q / (BK / 8), kc = q % (BK / 8);
        const int m = m0 + r, kk = k0 + kc * 8;
        if (m < M && kk < Kv) v = *reinterpret_cast<const u32x4*>(Ae + static_cast<int64_t>(m) * lda + kk);
      } else {
        const int kr = q / (BM / 8), mc = q % (BM / 8);
        const int kk = k0 + kr, m = m0 + mc * 8;
        if (kk < Kv && m < M) v = *reinterpret_cast<const u32x4*>(Ae + static_cast<int64_t>(kk) * lda + m);
      }
      ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int q = tid + 256 * i;
      u32x4 v = {0u, 0u, 0u, 0u};
      if constexpr (BKC) {
        const int r = q / (BK / 8), kc = q % (BK / 8);
        const int n = n0 + r, kk = k0 + kc * 8;
        if (n < N && kk < Kv) v = *reinterpret_cast<const u32x4*>(Be + static_cast<int64_t>(n) * ldb + kk);
      } else {
        const int kr = q / (BN / 8), nc = q % (BN / 8);
        const int kk = k0 + kr, n = n0 + nc * 8;
        if (kk < Kv && n < N) v = *reinterpret_cast<const u32x4*>(Be + static_cast<int64_t>(kk) * ldb + n);
      }
      rb[i] = v;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = tid + 256 * i;
      const int idx = AKC ? (q / (BK / 8)) * TA::kPitch + (q % (BK / 8)) * 8
                          : (q / (BM / 8)) * TA::kPitch + (q % (BM / 8)) * 8;
      *reinterpret_cast<u32x4*>(&la[buf][idx]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int q = tid + 256 * i;
      const int idx = BKC ? (q / (BK / 8)) * TBt::kPitch + (q % (BK / 8)) * 8
                          : (q / (BN / 8)) * TBt::kPitch + (q % (BN / 8)) * 8;
      *reinterpret_cast<u32x4*>(&lb[buf][idx]) = rb[i];
    }
  };
  // fragment of operand rows r (32 rows starting at r0), k = 16 j + 8 half .. + 7
  // Fragment of operand rows r0 .. r0 + 31 (lane row r0 + fr), k = 16 j + 8 half .. + 7.
  // A [row][k] tile is read as one 16-byte vector.  A [k][row] tile is read with two
  // ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the
  // 8-byte chunks addressed by lanes 4 q + i / 4 (q = 0..3), so lane 16 g + 4 q + c
  // addresses row chunk r0 + 16 (g % 2) + 4 c of k row 8 (g / 2) + q (+ 4 for the
  // second read) and every lane ends with 4 + 4 consecutive k of its own row.
  const int trq = (lane & 15) >> 2, trc = lane & 3, trg = lane >> 4;
  auto frag = [&](const bf16_t* t, bool kc, int pitch, int r0, int j) {
    const int k = 16 * j + 8 * half;
    if (kc) return *reinterpret_cast<const bf16x8*>(t + (r0 + fr) * pitch + k);
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const bf16_t* src = t + (16 * j + 8 * (trg >> 1) + trq) * pitch + r0 + 16 * (trg & 1) + 4 * trc;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 4 * pitch));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  floatx16 acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;

  const int nk = (Kv + BK - 1) / BK;
  if (nk > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
      for (int j = 0; j < BK / 16; ++j) {
        bf16x8 fa[TM], fb[TN];
#pragma unroll
        for (int t = 0; t < TM; ++t) fa[t] = frag(la[buf], AKC, TA::kPitch, (wm * TM + t) * 32, j);
#pragma unroll
        for (int i = 0; i < TN; ++i) fb[i] = frag(lb[buf], BKC, TBt::kPitch, (wn * TN + i) * 32, j);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int t = 0; t < TM; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[i], fa[t], acc[i][t], 0, 0, 0);
      }
      if (kt + 1 < nk) store(buf ^ 1);
      __syncthreads();
    }
  }
  // D[n][m]: lane holds m = fr and n = 8 * (r / 4) + 4 * half + r % 4 of each 32 x 32 tile.
  // The tile goes through LDS (the operand buffers are free after the last
  // barrier of the k loop), then out with 16-byte stores, four 256-byte row
  // segments per wave instruction.  EPI 2 makes two passes (dZa, then dZb).
  bf16_t* Oe = out + e * sOe;
  const bf16_t* Ze = aux ? aux + e * sOe : nullptr;
  bf16_t* st = smem_;  // [BM][OP]
  auto unpack4 = [](uint2 zz, float* z) {
    z[0] = __uint_as_float(zz.x << 16);
    z[1] = __uint_as_float(zz.x & 0xFFFF0000u);
    z[2] = __uint_as_float(zz.y << 16);
    z[3] = __uint_as_float(zz.y & 0xFFFF0000u);
  };
  constexpr int NPASS = EPI == 2 ? 2 : 1;
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    if (pass > 0) __syncthreads();  // the previous pass's staging reads are done
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int ml = (wm * TM + t) * 32 + fr;
      const int m = m0 + ml;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int nl0 = (wn * TN + i) * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = nl0 + 8 * q + 4 * half;
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = acc[i][t][4 * q + u];
          if constexpr (EPI == 1) {
            if (m < Mv && n0 + nl < N) {
              float z[4];
              unpack4(*reinterpret_cast<const uint2*>(Ze + static_cast<int64_t>(m) * ldo + n0 + nl), z);
#pragma unroll
              for (int u = 0; u < 4; ++u) v[u] *= ACT == 0 ? (z[u] > 0.f ? 1.f : 0.f) : gelu_grad(z[u]);
            }
          } else if constexpr (EPI == 2) {
            if (m < Mv && n0 + nl < N) {
              const bf16_t* zr = Ze + static_cast<int64_t>(m) * ldo + n0 + nl;
              float za[4], zb[4];
              unpack4(*reinterpret_cast<const uint2*>(zr), za);
              unpack4(*reinterpret_cast<const uint2*>(zr + N), zb);
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                if (pass == 0)
                  v[u] *= zb[u] * (ACT == 0 ? (za[u] > 0.f ? 1.f : 0.f) : gelu_grad(za[u]));
                else
                  v[u] *= apply_act<ACT>(za[u]);
              }
            }
          }
          uint2 w;
          w.x = pack_bf16x2(v[0], v[1]);
          w.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(st + ml * OP + nl) = w;
        }
      }
    }
    __syncthreads();
    constexpr int CPRow = BN / 8;  // 16-byte chunks per row
    bf16_t* Op = Oe + (pass ? N : 0);
#pragma unroll
    for (int it = 0; it < BM * CPRow / 256; ++it) {
      const int q = it * 256 + tid;
      const int ml = q / CPRow, c = q % CPRow;
      const int m = m0 + ml, n = n0 + c * 8;
      if (m < Mv && n < N) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + ml * OP + c * 8);
        u32x4* dst = reinterpret_cast<u32x4*>(Op + static_cast<int64_t>(m) * ldo + n);
        // both operands contracted over their leading (token) dimension: the weight
        // gradients, a write stream the backward does not read again; non-temporal
        // stores keep it from allocating in L2 (Switch-Base backward 829 -> 752 us)
        if constexpr (!AKC && !BKC) __builtin_nontemporal_store(v, dst);
        else *dst = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 MFMA tile GEMM with the same orientation flags, 64 x 64 tile of four
// 32 x 32 wave tiles.  Inputs of type TA / TB (float or bf16), float32
// accumulation, output float32 or TO.  Batched over z = e * KS + ks: KS > 1
// splits the k range into KS contiguous pieces, piece ks going to output slice
// ks (out + ks * sOk), added later in order.  Per expert e: M_e / K_e as in
// bgemm_kernel (count == nullptr: every expert has the fixed M and K).
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ float ld_f32(const T* p);
template <> __device__ __forceinline__ float ld_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }
template <typename T> __device__ __forceinline__ void st_f32(T* p, float v);
template <> __device__ __forceinline__ void st_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st_f32<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }

template <typename TA, typename TB, typename TO, bool AKC, bool BKC, int EPI, int ACT>
__global__ __launch_bounds__(256) void fgemm_kernel(
    const TA* __restrict__ A, int64_t sAe, int lda, const TB* __restrict__ B, int64_t sBe, int ldb,
    TO* __restrict__ out, int64_t sOe, int64_t sOk, int ldo, const TO* __restrict__ aux,
    const int32_t* __restrict__ count, int64_t C, int M, int N, int K, bool m_is_count, int KS) {
  // 32-k steps through double-buffered LDS tiles [k][row] (the next step's
  // elements loaded into registers while this step's MFMAs run); wave (wm, wn)
  // owns the 32 x 32 sub-tile; v_mfma_f32_32x32x2_f32 with srcA = rows n of B
  // and srcB = rows m of A gives D[n][m], lane l holding m = l % 32 and
  // n = 8 (r / 4) + 4 (l / 32) + r % 4 of accumulator element r.
  constexpr int FBK = 32, P = 64 + 4, PL = FBK * 64 / 256;
  __shared__ float sa[2][FBK][P];
  __shared__ float sb[2][FBK][P];
  const int bx = blockIdx.x, by = blockIdx.y;
  const int e = blockIdx.z / KS, ks = blockIdx.z % KS;
  int Mv = M, Kv = K;
  if (count) {
    int64_t cnt = count[e];
    cnt = cnt < 0 ? 0 : (cnt > C ? C : cnt);
    if (m_is_count) Mv = static_cast<int>(cnt);
    else Kv = static_cast<int>(cnt);
  }
  const int m0 = by * 64, n0 = bx * 64;
  if (m0 >= Mv) return;
  const int kb = static_cast<int>(static_cast<int64_t>(ks) * Kv / KS);
  const int ke = static_cast<int>(static_cast<int64_t>(ks + 1) * Kv / KS);
  const TA* Ae = A + e * sAe;
  const TB* Be = B + e * sBe;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, fr = lane & 31, kh = lane >> 5;
  // tile element q of a step: (row r in 0..63, k c in 0..FBK-1); which index runs
  // fastest follows the storage so that neighbouring threads read neighbouring memory
  // A row-contiguous operand ([k][row] storage) is read as 8 consecutive rows of
  // one k per thread (one 16-byte load of bf16, two of float; element loads for a
  // chunk that crosses the row extent or sits at an unaligned pitch); a
  // k-contiguous one element by element, k fastest.
  static_assert(PL == 8, "one 8-row chunk of one k per thread");
  float va[PL], vb[PL];
  auto fetch_op = [&](auto* P0, int ld, int r0, int ext, bool kc, int k0, float* v) {
    if (kc) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int q = tid + 256 * i;
        const int r = r0 + q / FBK, kk = k0 + q % FBK;
        v[i] = (r < ext && kk < ke) ? ld_f32(P0 + static_cast<int64_t>(r) * ld + kk) : 0.f;
      }
    } else {
      const int kk = k0 + (tid >> 3), rb = r0 + (tid & 7) * 8;
      const auto* src = P0 + static_cast<int64_t>(kk) * ld + rb;
      if (kk < ke && rb + 8 <= ext && (ld & 7) == 0) {
        vec8<typename std::remove_const<typename std::remove_pointer<decltype(P0)>::type>::type>::load(src, v);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (kk < ke && rb + j < ext) ? ld_f32(src + j) : 0.f;
      }
    }
  };
  auto fetch = [&](int k0) {
    fetch_op(Ae, lda, m0, M, AKC, k0, va);
    fetch_op(Be, ldb, n0, N, BKC, k0, vb);
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int q = tid + 256 * i;
      if constexpr (AKC) sa[buf][q % FBK][q / FBK] = va[i];
      else sa[buf][tid >> 3][(tid & 7) * 8 + i] = va[i];
      if constexpr (BKC) sb[buf][q % FBK][q / FBK] = vb[i];
      else sb[buf][tid >> 3][(tid & 7) * 8 + i] = vb[i];
    }
  };
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (kb < ke) {
    fetch(kb);
    put(0);
  }
  __syncthreads();
  int buf = 0;
  for (int k0 = kb; k0 < ke; k0 += FBK) {
    const bool more = k0 + FBK < ke;
    if (more) fetch(k0 + FBK);
#pragma unroll
    for (int kk = 0; kk < FBK / 2; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sb[buf][2 * kk + kh][wn * 32 + fr],
                                                 sa[buf][2 * kk + kh][wm * 32 + fr], acc, 0, 0, 0);
    if (more) put(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  TO* Oe = out + e * sOe + ks * sOk;
  const TO* Ze = aux ? aux + e * sOe : nullptr;
  const int m = m0 + wm * 32 + fr;
  if (m < Mv) {
    if constexpr (EPI == 0 && sizeof(TO) == 4) {
      if ((ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(Oe) & 15) == 0) {
        // four consecutive columns per lane and group: one 16-byte store
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * 32 + 8 * q + 4 * kh;
          if (n + 3 < N)
            *reinterpret_cast<floatx4*>(Oe + static_cast<int64_t>(m) * ldo + n) =
                floatx4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
          else
            for (int u = 0; u < 4 && n + u < N; ++u) st_f32(Oe + static_cast<int64_t>(m) * ldo + n + u, acc[4 * q + u]);
        }
        return;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = n0 + wn * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (n >= N) continue;
      float v = acc[r];
      if constexpr (EPI == 1) {
        const float z = ld_f32(Ze + static_cast<int64_t>(m) * ldo + n);
        v *= ACT == 0 ? (z > 0.f ? 1.f : 0.f) : gelu_grad(z);
      } else if constexpr (EPI == 2) {
        // GLU: za at column n, zb at column N + n; dZb goes to column N + n
        const float za = ld_f32(Ze + static_cast<int64_t>(m) * ldo + n);
        const float zb = ld_f32(Ze + static_cast<int64_t>(m) * ldo + N + n);
        st_f32(Oe + static_cast<int64_t>(m) * ldo + N + n, v * apply_act<ACT>(za));
        v *= zb * (ACT == 0 ? (za > 0.f ? 1.f : 0.f) : gelu_grad(za));
      }
      st_f32(Oe + static_cast<int64_t>(m) * ldo + n, v);
    }
  }
}

// Add KS float slices in order: out[i] = ((s0 + s1) + s2) + ...
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, int64_t n,
                                                         int KS, float* __restrict__ out) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    float v = part[i];
    for (int s = 1; s < KS; ++s) v += part[s * n + i];
    out[i] = v;
  }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.f;
}

// dbias partials: block (x, y) adds dh[t][e] over token range y of S (fixed by T and
// S only) for experts x*64 .. x*64+63.  The range is cut in four contiguous quarters,
// one per wave, each added in token order with sixteen rows in flight, then the
// quarters in order: part[y][e] = ((q0 + q1) + q2) + q3.  sum_slices_kernel then adds
// the S ranges in order, so the result is the same on every call.
__global__ __launch_bounds__(256) void bwd_bias_partial_kernel(const float* __restrict__ dh, int ldh, int ntok,
                                                               int E, float* __restrict__ part) {
  __shared__ float q[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int y = blockIdx.y, S = gridDim.y;
  const int t0 = static_cast<int>(static_cast<int64_t>(y) * ntok / S);
  const int t1 = static_cast<int>(static_cast<int64_t>(y + 1) * ntok / S);
  const int a = t0 + static_cast<int>(static_cast<int64_t>(wave) * (t1 - t0) / 4);
  const int z = t0 + static_cast<int>(static_cast<int64_t>(wave + 1) * (t1 - t0) / 4);
  float acc = 0.f;
  if (e < E) {
    for (int t = a; t < z; t += 16) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = t + j < z ? dh[static_cast<int64_t>(t + j) * ldh + e] : 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc += v[j];
    }
  }
  q[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && e < E) part[static_cast<int64_t>(y) * E + e] = ((q[0][lane] + q[1][lane]) + q[2][lane]) + q[3][lane];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, bool AKC, bool BKC, int EPI, int ACT>
static hipError_t run_bgemm(const Plan& p, const bf16_t* A, int64_t sAe, int lda, const bf16_t* B,
                            int64_t sBe, int ldb, bf16_t* out, int64_t sOe, int ldo,
                            const bf16_t* aux, const int32_t* count, int M, int N, int K,
                            bool m_is_count, hipStream_t s) {
  const int mtiles = ((m_is_count ? static_cast<int>(p.C) : M) + BM - 1) / BM;
  const dim3 grid((N + BN - 1) / BN, mtiles, p.E);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((bgemm_kernel<BM, BN, BK, AKC, BKC, EPI, ACT>), grid, dim3(256), 0, s, A, sAe, lda, B,
                     sBe, ldb, out, sOe, ldo, aux, count, p.C, M, N, K, m_is_count);
  return hipGetLastError();
}

template <typename TA, typename TB, typename TO, bool AKC, bool BKC, int EPI, int ACT>
static hipError_t run_fgemm(int batch, int64_t C, const TA* A, int64_t sAe, int lda, const TB* B,
                            int64_t sBe, int ldb, TO* out, int64_t sOe, int64_t sOk, int ldo,
                            const TO* aux, const int32_t* count, int M, int N, int K,
                            bool m_is_count, int KS, hipStream_t s) {
  const int mtiles = ((m_is_count && count ? static_cast<int>(C) : M) + 63) / 64;
  const dim3 grid((N + 63) / 64, mtiles, batch * KS);
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  hipLaunchKernelGGL((fgemm_kernel<TA, TB, TO, AKC, BKC, EPI, ACT>), grid, dim3(256), 0, s, A, sAe,
                     lda, B, sBe, ldb, out, sOe, sOk, ldo, aux, count, C, M, N, K, m_is_count, KS);
  return hipGetLastError();
}

#define MOE_TRY(x)                         \
  do {                                     \
    const hipError_t err_ = (x);           \
    if (err_ != hipSuccess) return err_;   \
  } while (0)

// Token-row products (dZ, dx_e): 64-row tiles while one tile holds an expert's
// tokens (capacity <= 64: weight streaming), 128-row tiles above (MFMA-bound;
// 4% faster on the large layer's backward).
template <int EPI, int ACT>
static hipError_t run_bgemm_rows(const Plan& p, const bf16_t* A, int64_t sAe, int lda, const bf16_t* B,
                                 int64_t sBe, int ldb, bf16_t* out, int64_t sOe, int ldo,
                                 const bf16_t* aux, const int32_t* count, int M, int N, int K,
                                 bool m_is_count, hipStream_t s) {
  if (p.C > 64)
    return run_bgemm<128, 128, 64, true, false, EPI, ACT>(p, A, sAe, lda, B, sBe, ldb, out, sOe, ldo, aux,
                                                           count, M, N, K, m_is_count, s);
  return run_bgemm<64, 128, 64, true, false, EPI, ACT>(p, A, sAe, lda, B, sBe, ldb, out, sOe, ldo, aux, count,
                                                        M, N, K, m_is_count, s);
}

// Expert-side products for one dtype.  dZ is staged in the dZ buffer, the
// pre-activation (GELU) in the Z buffer.  GLU: Z = x_e [W; V]^T over the 2 f
// stacked rows in the Z buffer ([C][2 f] per expert), dZ = (dZa, dZb) likewise,
// and the products with w1 run over 2 f rows.

// Plan of the plain product x_e . w1^T over every row of w1 (no activation).
static Plan stacked_plan(const Plan& p) {
  Plan q = p;
  q.f = p.w1_rows();
  q.glu = false;
  return q;
}
template <typename T>
static hipError_t expert_backward(const Plan& p, const T* x_e, const T* hidden, const T* w1,
                                  const T* w2, const int32_t* count, const T* dy_e, T* zbuf,
                                  T* dz, T* dx_e, T* dw1, T* dw2, hipStream_t s);

template <>
hipError_t expert_backward<bf16_t>(const Plan& p, const bf16_t* x_e, const bf16_t* hidden,
                                   const bf16_t* w1, const bf16_t* w2, const int32_t* count,
                                   const bf16_t* dy_e, bf16_t* zbuf, bf16_t* dz, bf16_t* dx_e,
                                   bf16_t* dw1, bf16_t* dw2, hipStream_t s) {
  const int d = static_cast<int>(p.d), f = static_cast<int>(p.f);
  const int r = static_cast<int>(p.w1_rows());  // rows of w1: f, or 2 f for GLU
  const int64_t C = p.C, sX = C * d, sH = C * f, sW = int64_t(d) * f;
  const int64_t sZ = C * r, sW1 = int64_t(d) * r;
  const int Ci = static_cast<int>(C);
  // GELU and GLU: pre-activation Z = x_e . w1^T again (the forward keeps only H)
  if (p.act == 1 || p.glu) MOE_TRY(launch_expert_up_act(stacked_plan(p), x_e, count, w1, zbuf, 2, s));
  const bf16_t* z = (p.act == 1 || p.glu) ? zbuf : hidden;
  // dZ[s][f] = sum_d dy_e[s][d] w2[d][f] * act'(Z)   (A = dy_e k-contiguous, B = w2 [k=d][n=f])
  if (p.glu) {
    if (p.act == 0)
      MOE_TRY((run_bgemm_rows<2, 0>(p, dy_e, sX, d, w2, sW, f, dz, sZ, r, z, count, Ci,
                                                      f, d, true, s)));
    else
      MOE_TRY((run_bgemm_rows<2, 1>(p, dy_e, sX, d, w2, sW, f, dz, sZ, r, z, count, Ci,
                                                      f, d, true, s)));
  } else {
    // the ping-pong GEMM where it applies (large capacities, d_model >= 2048)
    hipError_t err = launch_bwd_rows_pp(p, dy_e, w2, dz, z, count, f, d, p.act, s);
    if (err == hipErrorNotSupported)
      err = p.act == 0 ? run_bgemm_rows<1, 0>(p, dy_e, sX, d, w2, sW, f, dz, sH, f, z, count, Ci, f, d, true, s)
                       : run_bgemm_rows<1, 1>(p, dy_e, sX, d, w2, sW, f, dz, sH, f, z, count, Ci, f, d, true, s);
    MOE_TRY(err);
  }
  // dx_e[s][d] = sum_r dZ[s][r] w1[r][d]   (B = w1 [k=r][n=d]); ping-pong where it applies
  hipError_t err = launch_bwd_rows_pp(p, dz, w1, dx_e, nullptr, count, d, r, -1, s);
  if (err == hipErrorNotSupported)
    err = run_bgemm_rows<0, 0>(p, dz, sZ, r, w1, sW1, d, dx_e, sX, d, nullptr, count, Ci, d, r, true, s);
  MOE_TRY(err);
  // dw2[d][f] = sum_s dy_e[s][d] H[s][f]   (A = dy_e [k=s][m=d], B = H [k=s][n=f])
  MOE_TRY((run_bgemm<128, 128, 32, false, false, 0, 0>(p, dy_e, sX, d, hidden, sH, f, dw2, sW, f, nullptr,
                                                    count, d, f, 0, false, s)));
  // dw1[r][d] = sum_s dZ[s][r] x_e[s][d]
  MOE_TRY((run_bgemm<128, 128, 32, false, false, 0, 0>(p, dz, sZ, r, x_e, sX, d, dw1, sW1, d, nullptr, count,
                                                    r, d, 0, false, s)));
  return hipSuccess;
}

template <>
hipError_t expert_backward<float>(const Plan& p, const float* x_e, const float* hidden,
                                  const float* w1, const float* w2, const int32_t* count,
                                  const float* dy_e, float* zbuf, float* dz, float* dx_e, float* dw1,
                                  float* dw2, hipStream_t s) {
  const int d = static_cast<int>(p.d), f = static_cast<int>(p.f);
  const int r = static_cast<int>(p.w1_rows());
  const int64_t C = p.C, sX = C * d, sH = C * f, sW = int64_t(d) * f;
  const int64_t sZ = C * r, sW1 = int64_t(d) * r;
  const int Ci = static_cast<int>(C);
  if (p.act == 1 || p.glu) MOE_TRY(launch_expert_up_act(stacked_plan(p), x_e, count, w1, zbuf, 2, s));
  const float* z = (p.act == 1 || p.glu) ? zbuf : hidden;
  if (p.glu) {
    if (p.act == 0)
      MOE_TRY((run_fgemm<float, float, float, true, false, 2, 0>(p.E, C, dy_e, sX, d, w2, sW, f, dz, sZ, 0,
                                                                  r, z, count, Ci, f, d, true, 1, s)));
    else
      MOE_TRY((run_fgemm<float, float, float, true, false, 2, 1>(p.E, C, dy_e, sX, d, w2, sW, f, dz, sZ, 0,
                                                                  r, z, count, Ci, f, d, true, 1, s)));
  } else if (p.act == 0) {
    MOE_TRY((run_fgemm<float, float, float, true, false, 1, 0>(p.E, C, dy_e, sX, d, w2, sW, f, dz, sH, 0,
                                                                f, z, count, Ci, f, d, true, 1, s)));
  } else {
    MOE_TRY((run_fgemm<float, float, float, true, false, 1, 1>(p.E, C, dy_e, sX, d, w2, sW, f, dz, sH, 0,
                                                                f, z, count, Ci, f, d, true, 1, s)));
  }
  MOE_TRY((run_fgemm<float, float, float, true, false, 0, 0>(p.E, C, dz, sZ, r, w1, sW1, d, dx_e, sX, 0, d,
                                                              nullptr, count, Ci, d, r, true, 1, s)));
  MOE_TRY((run_fgemm<float, float, float, false, false, 0, 0>(p.E, C, dy_e, sX, d, hidden, sH, f, dw2, sW,
                                                               0, f, nullptr, count, d, f, 0, false, 1, s)));
  MOE_TRY((run_fgemm<float, float, float, false, false, 0, 0>(p.E, C, dz, sZ, r, x_e, sX, d, dw1, sW1, 0,
                                                               d, nullptr, count, r, d, 0, false, 1, s)));
  return hipSuccess;
}

template <typename T>
static hipError_t backward_typed(const Plan& p, const BwdArgs& a, hipStream_t s) {
  const int d = static_cast<int>(p.d);
  const int T_ = static_cast<int>(p.T);
  const int nblk = static_cast<int>((p.T + 3) / 4);
  const T* dy = static_cast<const T*>(a.dy);
  T* dy_e = static_cast<T*>(a.dy_e);
  if (p.T > 0)
    hipLaunchKernelGGL(bwd_scatter_kernel<T>, dim3(nblk), dim3(256), 0, s, dy,
                       static_cast<const T*>(a.y_e), a.expert_idx, a.slot, a.gate, T_, p.E, p.k,
                       p.C, p.d, dy_e, a.dgate);
  MOE_TRY(hipGetLastError());
  if (p.C > 0)
    MOE_TRY(expert_backward<T>(p, static_cast<const T*>(a.x_e), static_cast<const T*>(a.hidden),
                               static_cast<const T*>(a.w1), static_cast<const T*>(a.w2), a.count, dy_e,
                               static_cast<T*>(a.zbuf), static_cast<T*>(a.dz), static_cast<T*>(a.dx_e),
                               static_cast<T*>(a.dw1), static_cast<T*>(a.dw2), s));
  else {
    // no capacity: every weight gradient is zero (sizes are multiples of 64 elements)
    const int64_t n16 = int64_t(p.E) * p.d * p.f * p.elem / 16;
    const int64_t n16w1 = int64_t(p.E) * p.d * p.w1_rows() * p.elem / 16;
    const unsigned g = static_cast<unsigned>(std::min<int64_t>((n16w1 + 255) / 256, 4096));
    hipLaunchKernelGGL(zero_fill_kernel, dim3(g), dim3(256), 0, s, static_cast<u32x4*>(a.dw1), n16w1);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(g), dim3(256), 0, s, static_cast<u32x4*>(a.dw2), n16);
    MOE_TRY(hipGetLastError());
  }
  float* dx_r = nullptr;
  if (p.route == 0 && p.T > 0) {
    // router: logits again (same kernel and arithmetic as the forward), softmax Jacobian
    MOE_TRY(launch_router_topk(p, a.x, a.w_r, a.bias, a.idx_scratch, a.gate_scratch, a.ws, s, false,
                               a.dh));
    hipLaunchKernelGGL(bwd_router_softmax_kernel, dim3(nblk), dim3(256), 0, s, a.dh, p.Epad,
                       a.expert_idx, a.slot, a.dgate, T_, p.E, p.k);
    MOE_TRY(hipGetLastError());
    // dx_r[t][d] = sum_e dh[t][e] w_r[e][d]
    dx_r = a.dx_r;
    MOE_TRY((run_fgemm<float, float, float, true, false, 0, 0>(1, 0, a.dh, 0, p.Epad, a.w_r, 0, d, dx_r, 0,
                                                                0, d, nullptr, nullptr, T_, d, p.E, false, 1,
                                                                s)));
    // dw_r[e][d] = sum_t dh[t][e] x[t][d], in KS token ranges added in order; KS, a
    // function of the sizes only, gives about 384 tiles (16 on Switch-Base), at
    // most kBwdSplit
    const int64_t n = int64_t(p.E) * d;
    const int64_t tiles = int64_t((d + 63) / 64) * ((p.E + 63) / 64);
    const int KS = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kBwdSplit, (384 + tiles - 1) / tiles)));
    MOE_TRY((run_fgemm<float, T, float, false, false, 0, 0>(1, 0, a.dh, 0, p.Epad, static_cast<const T*>(a.x),
                                                             0, d, a.dwr_part, 0, n, d, nullptr, nullptr,
                                                             p.E, d, T_, false, KS, s)));
    hipLaunchKernelGGL(sum_slices_kernel, dim3(static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 1024))),
                       dim3(256), 0, s, a.dwr_part, n, KS, a.dw_r);
    MOE_TRY(hipGetLastError());
    if (a.dbias) {
      // dbias[e] = sum_t dh[t][e]: kBwdSplit token ranges (fewer for short inputs) into
      // the dw_r partial buffer, free again once dw_r is summed (stream order), then
      // the ranges added in order
      const int SB = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kBwdSplit, T_)));
      hipLaunchKernelGGL(bwd_bias_partial_kernel, dim3((p.E + 63) / 64, SB), dim3(256), 0, s, a.dh, p.Epad,
                         T_, p.E, a.dwr_part);
      hipLaunchKernelGGL(sum_slices_kernel, dim3((p.E + 255) / 256), dim3(256), 0, s, a.dwr_part,
                         int64_t(p.E), SB, a.dbias);
      MOE_TRY(hipGetLastError());
    }
  }
  if (p.route == 0 && p.T == 0) {
    // no tokens: the router gradients are zero
    hipLaunchKernelGGL(zero_f32_kernel, dim3(64), dim3(256), 0, s, a.dw_r, int64_t(p.E) * d);
    if (a.dbias) hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(256), 0, s, a.dbias, int64_t(p.E));
    MOE_TRY(hipGetLastError());
  }
  if (p.T > 0)
    hipLaunchKernelGGL(bwd_gather_kernel<T>, dim3(nblk), dim3(256), 0, s,
                       static_cast<const T*>(a.dx_e), dx_r, a.expert_idx, a.slot, T_, p.E, p.k, p.C,
                       p.d, static_cast<T*>(a.dx));
  return hipGetLastError();
}

hipError_t launch_backward(const Plan& p, const BwdArgs& a, hipStream_t s) {
  return p.dtype == 1 ? backward_typed<bf16_t>(p, a, s) : backward_typed<float>(p, a, s);
}

#undef MOE_TRY

}  // namespace moe

// ---------------------------------------------------------------------------
// SparseClip (TorchScale review, methodology): clipping norm with the MoE
// (expert) gradients re-weighted by kappa = 1/sqrt(E),
//   norm = sqrt(|g_dense|^2 + |g_moe|^2 / E),  coef = min(1, max_norm / (norm + 1e-6)),
// every gradient multiplied by coef.  Sums of squares in float64: block b of a
// launch takes the b-th contiguous range of the array; one block adds the
// partials in order.  Dense = router gradients, MoE = expert weight gradients.
// ---------------------------------------------------------------------------
namespace moe {

constexpr int kClipBlocks = 512;

// Sum of squares of one array in float64.  Block b (512 threads) takes the b-th
// contiguous range of its 8-element vectors: full batches of eight 16-byte
// loads per thread issued together (enough bytes in flight to keep HBM busy),
// then the range's remainder one vector per thread; four float64 accumulators
// per thread in a fixed assignment; the last block also takes the n % 8 tail.
// Deterministic: a fixed order throughout.
constexpr int kSumsqThreads = 512;

template <typename T>
__global__ __launch_bounds__(kSumsqThreads) void clip_sumsq_kernel(const T* __restrict__ p, int64_t n,
                                                                   double* __restrict__ part) {
  constexpr int U = 8, NT = kSumsqThreads;
  __shared__ double red[NT];
  const int64_t n8 = n >> 3;
  const int64_t b0 = n8 * blockIdx.x / gridDim.x, b1 = n8 * (blockIdx.x + 1) / gridDim.x;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t i = b0 + threadIdx.x;
  for (; i + NT * (U - 1) < b1; i += NT * U) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) vec8<T>::load(p + 8 * (i + NT * u), v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double x = static_cast<double>(v[u][e]);
        acc[e & 3] = fma(x, x, acc[e & 3]);
      }
  }
  for (; i < b1; i += NT) {
    float v[8];
    vec8<T>::load(p + 8 * i, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = static_cast<double>(v[e]);
      acc[e & 3] = fma(x, x, acc[e & 3]);
    }
  }
  if (blockIdx.x == gridDim.x - 1)
    for (int64_t j = 8 * n8 + threadIdx.x; j < n; j += NT) {
      const double x = static_cast<double>(ld_f32(p + j));
      acc[0] = fma(x, x, acc[0]);
    }
  red[threadIdx.x] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// part: [4][kClipBlocks] (dw_r, dbias, dw1, dw2); out: norm, coef (float).
// Thread t adds partials 2t and 2t + 1 of each array, then a fixed tree.
__global__ __launch_bounds__(256) void clip_coef_kernel(const double* __restrict__ part, int E,
                                                        double max_norm, float* __restrict__ out) {
  static_assert(kClipBlocks == 512, "two partials per thread");
  __shared__ double red[4][256];
  const int t = threadIdx.x;
#pragma unroll
  for (int a = 0; a < 4; ++a) red[a][t] = part[a * kClipBlocks + 2 * t] + part[a * kClipBlocks + 2 * t + 1];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
#pragma unroll
      for (int a = 0; a < 4; ++a) red[a][t] += red[a][t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    const double norm = sqrt((red[0][0] + red[1][0]) + (red[2][0] + red[3][0]) / E);
    const double coef = fmin(1.0, max_norm / (norm + 1e-6));
    out[0] = static_cast<float>(norm);
    out[1] = static_cast<float>(coef);
  }
}

// p *= coef in place.  Block b scales vectors [b, b + 1) * 256 * kScaleVecs of 8
// elements, each thread kScaleVecs of them (all loads before the stores, one pass
// per thread: a load issued after a store would also wait for that store); the
// n % 8 tail by block 0.  coef == 1 leaves every value as it is (x * 1 rounds to
// x), so the pass then reads and writes nothing.
constexpr int kScaleVecs = 4;

template <typename T>
__global__ __launch_bounds__(256) void clip_scale_kernel(T* __restrict__ p, int64_t n,
                                                         const float* __restrict__ nc) {
  constexpr int U = kScaleVecs;
  const float c = nc[1];
  if (c == 1.0f) return;
  const int64_t n8 = n >> 3;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x;
  float v[U][8];
  if (i + 256 * (U - 1) < n8) {
#pragma unroll
    for (int u = 0; u < U; ++u) vec8<T>::load(p + 8 * (i + 256 * u), v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[u][e] *= c;
      vec8<T>::store(p + 8 * (i + 256 * u), v[u]);
    }
  } else {
    for (int u = 0; u < U; ++u)
      if (i + 256 * u < n8) {
        vec8<T>::load(p + 8 * (i + 256 * u), v[0]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[0][e] *= c;
        vec8<T>::store(p + 8 * (i + 256 * u), v[0]);
      }
  }
  if (blockIdx.x == 0)
    for (int64_t j = 8 * n8 + threadIdx.x; j < n; j += 256) st_f32(p + j, ld_f32(p + j) * c);
}

// blocks of clip_scale_kernel for an n-element array (at least one: block 0 takes the tail)
inline unsigned clip_scale_blocks(int64_t n) {
  const int64_t per = 256LL * kScaleVecs;
  return static_cast<unsigned>(std::max<int64_t>(1, ((n >> 3) + per - 1) / per));
}

template <typename T>
static hipError_t clip_typed(const Plan& p, float* dw_r, float* dbias, T* dw1, T* dw2,
                             double max_norm, float* nc, double* part, hipStream_t s) {
  const int64_t nw = int64_t(p.E) * p.d * p.f, nw1 = int64_t(p.E) * p.d * p.w1_rows();
  const int64_t nr = dw_r ? int64_t(p.E) * p.d : 0, nb = dbias ? p.E : 0;
  // empty arrays still write their (zero) partials
  const dim3 sb(kSumsqThreads);
  hipLaunchKernelGGL(clip_sumsq_kernel<float>, dim3(kClipBlocks), sb, 0, s, dw_r, nr, part);
  hipLaunchKernelGGL(clip_sumsq_kernel<float>, dim3(kClipBlocks), sb, 0, s, dbias, nb, part + kClipBlocks);
  hipLaunchKernelGGL(clip_sumsq_kernel<T>, dim3(kClipBlocks), sb, 0, s, dw1, nw1, part + 2 * kClipBlocks);
  hipLaunchKernelGGL(clip_sumsq_kernel<T>, dim3(kClipBlocks), sb, 0, s, dw2, nw, part + 3 * kClipBlocks);
  hipLaunchKernelGGL(clip_coef_kernel, dim3(1), dim3(256), 0, s, part, p.E, max_norm, nc);
  if (nr) hipLaunchKernelGGL(clip_scale_kernel<float>, dim3(clip_scale_blocks(nr)), dim3(256), 0, s, dw_r, nr, nc);
  if (nb) hipLaunchKernelGGL(clip_scale_kernel<float>, dim3(clip_scale_blocks(nb)), dim3(256), 0, s, dbias, nb, nc);
  hipLaunchKernelGGL(clip_scale_kernel<T>, dim3(clip_scale_blocks(nw1)), dim3(256), 0, s, dw1, nw1, nc);
  hipLaunchKernelGGL(clip_scale_kernel<T>, dim3(clip_scale_blocks(nw)), dim3(256), 0, s, dw2, nw, nc);
  return hipGetLastError();
}

hipError_t launch_sparse_clip(const Plan& p, float* dw_r, float* dbias, void* dw1, void* dw2,
                              double max_norm, float* norm_coef, void* part, hipStream_t s) {
  double* pp = static_cast<double*>(part);
  return p.dtype == 1 ? clip_typed<bf16_t>(p, dw_r, dbias, static_cast<bf16_t*>(dw1),
                                           static_cast<bf16_t*>(dw2), max_norm, norm_coef, pp, s)
                      : clip_typed<float>(p, dw_r, dbias, static_cast<float*>(dw1),
                                          static_cast<float*>(dw2), max_norm, norm_coef, pp, s);
}

}  // namespace moe
