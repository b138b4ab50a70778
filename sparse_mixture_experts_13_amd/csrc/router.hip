// Router kernels: fused logits + softmax + top-k (+ per-block expert histogram),
// and the weightless random-routed-experts pick.
//
// Method (Switch Transformers notes, section 2.1): logits h(x) = W_r . x over the
// N experts, gate p_i = exp(h_i) / sum_j exp(h_j) (Eq. 1), the token goes to the
// top-k experts.  Section 2.4 keeps the router arithmetic in float32.  X-MoE
// top-1/top-2 routing (TorchScale review).  Random Routed Experts (PanGu-Sigma
// review): a uniform pick inside the token's expert group, no learned gate.
//
// gfx950 design (bf16 tokens).  A work-group owns a block of TB tokens (32,
// 64 or 128) and every expert.  The logits tile [TB x E] is a skinny GEMM on
// bf16 MFMA (v_mfma_f32_32x32x16_bf16) with float32 accumulation: x is bf16
// already, and the float32 router weight is split once per call into three
// bf16 planes hi + mid + lo that sum to it exactly, so every product is exact;
// when the weight is bf16-exact (mid = lo = 0, detected on the device) only the
// hi plane is used.  Weight and token rows stream through an LDS stage ring fed
// by direct global->LDS loads.  Eight waves per block: four only issue those
// loads and wait for them, four only read fragments and run the MFMAs, so a load
// issue held back by the memory pipeline never stalls the matrix pipe (with one
// wave per SIMD doing both, a stage cost the sum of its load, LDS and MFMA times:
// large-layer router and weight split 60 -> 47 us, Switch-Base 13.0 -> 11.2 us,
// X-MoE 18.5 -> 14.8 us).  The logits tile then goes to LDS, and sixteen
// lanes (one DPP row) rank each token by (logit, then lower index) with
// cross-lane DPP moves.  The block's
// expert histogram is built in LDS for the dispatch scan.  float32 tokens use a
// float32 FMA kernel with the same ranking, 64 tokens per block.
//
// Load-balancing loss (Switch notes 2.2, Eq. 4-6), on request: the epilogue
// also adds up every expert's softmax probability over the block's tokens, in
// a fixed order (lane, then the token groups of a wave, then the waves), into
// one row per router block; a one-block kernel adds the rows in block order
// (float64) for P_i and takes f_i from the first-choice histogram.
#include "moe_common.h"
#include "moe_internal.h"

#include <math.h>

namespace moe {

// ---- ranking inside a 16-lane DPP row: (logit desc, expert asc) ----
// Float comparison ranks -0 equal to +0, so equal logits (either sign of zero)
// fall to the lower expert index.
__device__ __forceinline__ void best_merge(float& v, int& e, float v2, int e2) {
  const bool take = (v2 > v) | ((v2 == v) & (e2 < e));  // bitwise: no branches
  v = take ? v2 : v;
  e = take ? e2 : e;
}

// One exchange step across the row: rotate by 8 or 4 lanes, then swap within
// pairs of lanes of a quad (row_ror:8 and row_ror:4, quad_perm [2,3,0,1] and
// [1,0,3,2]); after the four steps every lane of the row holds the row's
// result.  DPP moves go through the VALU, not the LDS crossbar.
template <int CTRL>
__device__ __forceinline__ int dpp_row(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ void best_step(float& v, int& e) {
  const float v2 = __int_as_float(dpp_row<CTRL>(__float_as_int(v)));
  const int e2 = dpp_row<CTRL>(e);
  best_merge(v, e, v2, e2);
}
__device__ __forceinline__ void row16_best(float& v, int& e) {
  best_step<0x128>(v, e);
  best_step<0x124>(v, e);
  best_step<0x4E>(v, e);
  best_step<0xB1>(v, e);
}
// Sum over the row.  Lanes i and i+8 (then i and i+4, ...) add the same two
// values in either order, so every lane ends with the same bits.
__device__ __forceinline__ float row16_sum(float s) {
  s += __int_as_float(dpp_row<0x128>(__float_as_int(s)));
  s += __int_as_float(dpp_row<0x124>(__float_as_int(s)));
  s += __int_as_float(dpp_row<0x4E>(__float_as_int(s)));
  s += __int_as_float(dpp_row<0xB1>(__float_as_int(s)));
  return s;
}

__device__ __forceinline__ void write_hist(const int* hl, int ldh, int E, int k, int NB, int b,
                                           int* __restrict__ hist, int tid, int nthreads) {
  for (int i = tid; i < E * k; i += nthreads) {
    const int e = i / k, c = i - e * k;
    hist[(static_cast<int64_t>(e) * k + c) * NB + b] = hl[c * ldh + e];
  }
}

// ---------------------------------------------------------------------------
// Split the float32 router weight into bf16 planes hi, mid, lo with
// w = hi + mid + lo exactly (each step rounds the remainder to nearest bf16;
// the remainders are exact in float32).  Rows E..Epad-1 are zero.  Block b
// writes flags[b] = 1 if any mid/lo element of its share is non-zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ w_r, int E,
                                                           int Epad, int d,
                                                           bf16_t* __restrict__ planes,
                                                           int* __restrict__ flags) {
  // eight elements per thread and step (d is a multiple of 64, so E * d and
  // Epad * d are multiples of 8): 16-byte loads, three 16-byte plane stores
  const int64_t n = static_cast<int64_t>(Epad) * d;
  const int64_t lim = static_cast<int64_t>(E) * d;
  int nz = 0;
  for (int64_t i8 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i8 < n / 8;
       i8 += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t i = i8 * 8;
    float w[8];
    vec8<float>::load(w_r + (i < lim ? i : 0), w);
    u32x4 ph, pm, pl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wj = i < lim ? w[j] : 0.f;
      const bf16_t hi = f32_to_bf16(wj);
      const float r1 = wj - bf16_to_f32(hi);
      const bf16_t mid = f32_to_bf16(r1);
      const float r2 = r1 - bf16_to_f32(mid);
      const bf16_t lo = f32_to_bf16(r2);
      const int sh = 16 * (j & 1);
      if (sh == 0) {
        ph[j >> 1] = hi;
        pm[j >> 1] = mid;
        pl[j >> 1] = lo;
      } else {
        ph[j >> 1] |= static_cast<uint32_t>(hi) << 16;
        pm[j >> 1] |= static_cast<uint32_t>(mid) << 16;
        pl[j >> 1] |= static_cast<uint32_t>(lo) << 16;
      }
      nz |= ((mid & 0x7FFF) | (lo & 0x7FFF)) != 0;
    }
    *reinterpret_cast<u32x4*>(planes + i) = ph;
    *reinterpret_cast<u32x4*>(planes + n + i) = pm;
    *reinterpret_cast<u32x4*>(planes + 2 * n + i) = pl;
  }
  nz = __syncthreads_or(nz);
  if (threadIdx.x == 0) flags[blockIdx.x] = nz;
}

// ---------------------------------------------------------------------------
// bf16 router: MFMA logits tile + top-k epilogue.
//
// A block owns TB = 32 * TT tokens and all experts.  Each 64-k stage (router
// weight rows 0..Epad-1, then the block's TB token rows, 128 bytes each) lands
// in an S-deep LDS ring through direct global->LDS loads issued S-1 stages
// ahead; for a non-bf16-exact weight the stages run over the hi, mid and lo
// planes in turn.  Loader waves 4..7 issue the stage loads; MFMA wave w (0..3)
// owns expert tiles w, w+4, ... (up to EW of them) against every token tile:
// D = W_r . x^T with v_mfma_f32_32x32x16_bf16.  All eight waves rank the tokens.
// ---------------------------------------------------------------------------
__host__ __device__ inline int64_t router_ring_bytes(int Epad, int TB, int S) {
  return static_cast<int64_t>(S) * (Epad + TB) * 128;
}
__host__ __device__ inline int64_t router_lg_bytes(int TB, int Epad) {
  return static_cast<int64_t>(TB) * (Epad + 4) * 4;
}

// Rank the tokens of a block from the logits tile lg [TB][ld] in LDS (both
// routers), NWV waves.  Sixteen lanes share a token (a wave ranks four tokens at a
// time); lane `sub` holds experts sub, sub+16, ...  Choices order by (logit desc,
// expert asc).
template <int NV, int NWV>
__device__ __forceinline__ void topk_epilogue16(const float* lg, int ld, int TB, int tok0, int ntok, int E, int k,
                                const float* __restrict__ bias, int32_t* __restrict__ expert_idx,
                                float* __restrict__ gate, int* hl, int ldh, int wave, int lane,
                                float* __restrict__ psum, float* red, float* __restrict__ hout,
                                int ldo) {
  const int grp = lane >> 4, sub = lane & 15;
  float pacc[NV], bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    pacc[i] = 0.f;
    // the lane's bias values once: a global load in the token loop made every
    // round wait for the previous round's stores (loads and stores share vmcnt)
    bv[i] = bias && sub + 16 * i < E ? bias[sub + 16 * i] : 0.f;
  }
  constexpr float kLog2e = 1.4426950408889634f;
  for (int base = 0; base < TB; base += 4 * NWV) {
    const int t = base + wave * 4 + grp;
    const bool valid = t < ntok;
    // every read is inside the tile (t < TB rows, e < Epad <= ld columns); the
    // values past the token count or past E are then replaced by -inf, so the
    // loop has no branches
    const float* row = lg + (valid ? t : 0) * ld;
    float hv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = sub + 16 * i;
      const float h = row[e];
      const float hb = bias ? h + bv[i] : h;  // one float32 rounding after the full dot product
      hv[i] = (valid & (e < E)) ? hb : -INFINITY;
    }
    if (hout && valid) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (sub + 16 * i < E) hout[static_cast<int64_t>(tok0 + t) * ldo + sub + 16 * i] = hv[i];
    }
    // choice c: each lane's best remaining expert (its experts ascend with i, so a
    // strict comparison keeps the lowest index of equal logits), then the row's
    uint32_t removed = 0;
    float hmax = -INFINITY, vmine = -INFINITY;
    int emine = 0;
    for (int c = 0; c < k; ++c) {
      float v = -INFINITY;
      int ev = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const bool take = (((removed >> i) & 1u) == 0u) & (hv[i] > v);
        v = take ? hv[i] : v;
        ev = take ? sub + 16 * i : ev;
      }
      row16_best(v, ev);
      if (ev < E && (ev & 15) == sub) removed |= 1u << (ev >> 4);
      if (c == 0) hmax = v;
      if (sub == c) {
        vmine = v;
        emine = ev;
      }
    }
    // softmax denominator with the native exp2 (one rounding of (h - hmax) log2 e
    // and the instruction's own error: the sum is dominated by terms near the
    // maximum, so its relative error stays near 1e-6); exp(-inf) = 0 past E
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) sum += __builtin_amdgcn_exp2f((hv[i] - hmax) * kLog2e);
    sum = row16_sum(sum);
    if (valid && sub < k) {
      const int64_t o = static_cast<int64_t>(tok0 + t) * k + sub;
      expert_idx[o] = emine;
      gate[o] = expf(vmine - hmax) / sum;
      atomicAdd(&hl[sub * ldh + emine], 1);
    }
    if (psum && valid) {
#pragma unroll
      for (int i = 0; i < NV; ++i) pacc[i] += expf(hv[i] - hmax) / sum;  // 0 past E
    }
  }
  if (psum) {
    // the wave's four token groups: (g0 + g1) + (g2 + g3), the same on every lane
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      pacc[i] += __shfl_xor(pacc[i], 16, kWave);
      pacc[i] += __shfl_xor(pacc[i], 32, kWave);
    }
    __syncthreads();  // every wave is done with the logits tile that red overlays
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = sub + 16 * i;
        if (e < ldh) red[wave * ldh + e] = pacc[i];
      }
    }
    __syncthreads();
    for (int e = wave * kWave + lane; e < E; e += NWV * kWave) {
      float s = red[e];  // the waves' rows in wave order
#pragma unroll
      for (int w = 1; w < NWV; ++w) s += red[w * ldh + e];
      psum[e] = s;
    }
  }
}

template <int TT, int EW, int S>
__global__ __launch_bounds__(512) void router_bf16_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ planes, const int* __restrict__ flags,
    const float* __restrict__ bias, int T, int d, int E, int Epad, int k,
    int32_t* __restrict__ expert_idx, float* __restrict__ gate, int* __restrict__ hist, int NB,
    float* __restrict__ psum, float* __restrict__ hout) {
  constexpr int TB = 32 * TT;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..3 MFMA, 4..7 loads
  const int qw = wave & 3;
  const int half = lane >> 5, fr = lane & 31;
  const int b = blockIdx.x;
  const int tok0 = b * TB;
  const int ntok = min(TB, T - tok0);
  const int n_et = Epad / 32;
  const int rows = Epad + TB;
  const int R = rows / 32;  // direct-to-LDS instructions per loader wave per stage
  const int64_t STAGE = static_cast<int64_t>(rows) * 128;
  const int64_t body = max(router_ring_bytes(Epad, TB, S), router_lg_bytes(TB, Epad));
  int* hl = reinterpret_cast<int*>(smem + body);  // [k][Epad]
  for (int i = tid; i < k * Epad; i += 512) hl[i] = 0;

  // the split kernel's flags, one per lane in a single vector load, then a wave
  // vote (one memory latency)
  static_assert(kSplitBlocks == kWave, "one split flag per lane");
  const int any = __any(flags[lane] != 0) ? 1 : 0;
  const int KS = d / 64;
  const int total = (any ? 3 : 1) * KS;
  const int64_t plane_elems = static_cast<int64_t>(Epad) * d;

  floatx16 acc[EW][TT];
  if (wave >= 4) {
    // Loader waves.  Instruction q of loader wave qw covers rows (4 q + qw) * 8 ..
    // + 7 (lane row (4 q + qw) * 8 + lane / 8) for q < R; RMAX bounds R at compile
    // time so the issue loop unrolls, and each lane's row offsets are computed
    // once: a stage only adds its k offset (and the plane offset).
    constexpr int RMAX = 4 * EW + TT;
    int64_t roff[RMAX];  // element offset of this lane's 16-byte chunk at k = 0
    bool rw[RMAX];       // weight row (else token row)
#pragma unroll
    for (int q = 0; q < RMAX; ++q) {
      const int rbase = (q * 4 + qw) * 8;
      const int row = rbase + (lane >> 3);
      const int c = (lane & 7) ^ lds_swz(row);
      rw[q] = rbase < Epad;
      if (rw[q]) roff[q] = static_cast<int64_t>(row) * d + c * 8;
      else roff[q] = static_cast<int64_t>(min(tok0 + row - Epad, T - 1)) * d + c * 8;
    }
    // (the lambda below reads the arrays through pointers: capturing an array whose
    // size depends on the template arguments leaves the kernel uninstantiated on the host)
    const int64_t* roffp = roff;
    const bool* rwp = rw;
    // Blocks start their k loop at different offsets so that they do not all
    // read the same router-weight rows at the same moment (hot L2 channels).
    const int rot = b % KS;
    auto issue = [&](int st, int slot) {
      const int p = st / KS;
      int ks = st - p * KS + rot;
      ks = ks >= KS ? ks - KS : ks;
      const bf16_t* wp = planes + p * plane_elems + ks * 64;
      const bf16_t* xp = x + ks * 64;
      unsigned char* base = smem + slot * STAGE + qw * 1024;
#pragma unroll
      for (int q = 0; q < RMAX; ++q)
        if (q < R)
          __builtin_amdgcn_global_load_lds((rwp[q] ? wp : xp) + roffp[q], (lds_void*)(base + q * 4096), 16, 0, 0);
    };
#pragma unroll
    for (int i = 0; i < S - 1; ++i)
      if (i < total) issue(i, i);
    // stage st has landed (this wave's share of it) -> barrier -> the slot of stage
    // st - 1, which every MFMA wave has read by now, takes stage st + S - 1
    for (int st = 0; st < total; ++st) {
      wait_vmcnt_dyn(total - 1 - st >= S - 2 ? (S - 2) * R : 0);
      ring_barrier();
      if (st + S - 1 < total) issue(st + S - 1, (st + S - 1) % S);
    }
  } else {
    // MFMA waves: wave w owns expert tiles w, w+4, ... (up to EW of them) against
    // every token tile; the fragments of sub-step j + 1 are read while sub-step j's
    // MFMAs run.  A wave past the last expert tile multiplies a copy of it (its
    // fragments are read clamped) and drops the result at the write-out: a branch
    // around the MFMAs moved every accumulator between AGPRs and VGPRs.
#pragma unroll
    for (int u = 0; u < EW; ++u)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][tt][r] = 0.f;
    for (int st = 0; st < total; ++st) {
      ring_barrier();
      const unsigned char* sb = smem + (st % S) * STAGE;
      bf16x8 bq[2][TT], a[2][EW];
      auto frag = [&](int j, int buf) {
        const int c = 2 * j + half;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const int row = Epad + tt * 32 + fr;
          bq[buf][tt] = *reinterpret_cast<const bf16x8*>(sb + row * 128 + 16 * (c ^ lds_swz(row)));
        }
#pragma unroll
        for (int u = 0; u < EW; ++u) {
          const int row = min(wave + 4 * u, n_et - 1) * 32 + fr;
          a[buf][u] = *reinterpret_cast<const bf16x8*>(sb + row * 128 + 16 * (c ^ lds_swz(row)));
        }
      };
      frag(0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j + 1 < 4) frag(j + 1, (j + 1) & 1);
#pragma unroll
        for (int u = 0; u < EW; ++u)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            acc[u][tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 1][u], bq[j & 1][tt], acc[u][tt], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // ring reads and loads done before the logits tile overwrites it

  // D[i][j] of a 32x32 tile: lane holds column j = lane % 32 (token) and rows
  // i = 8*(r/4) + 4*(lane/32) + r%4 (experts) of accumulator element r.
  float* lg = reinterpret_cast<float*>(smem);
  const int ld = Epad + 4;
  if (wave < 4) {
#pragma unroll
    for (int u = 0; u < EW; ++u) {
      const int et = wave + 4 * u;
      if (et < n_et) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int t = tt * 32 + fr;
            const int e = et * 32 + 8 * g + 4 * half;
            floatx4 v = {acc[u][tt][4 * g], acc[u][tt][4 * g + 1], acc[u][tt][4 * g + 2],
                         acc[u][tt][4 * g + 3]};
            *reinterpret_cast<floatx4*>(lg + t * ld + e) = v;
          }
      }
    }
  }
  __syncthreads();
  topk_epilogue16<8 * EW, 8>(lg, ld, TB, tok0, ntok, E, k, bias, expert_idx, gate, hl, Epad, wave,
                             lane, psum ? psum + static_cast<int64_t>(b) * Epad : nullptr, lg, hout, Epad);
  __syncthreads();
  write_hist(hl, Epad, E, k, NB, b, hist, tid, 512);
}

// ---------------------------------------------------------------------------
// float32 router (float32 token dtype): float32 FMA dot products, 64 tokens per
// block, then the shared ranking epilogue.  NACC = experts per thread; the block
// covers Ecap = 4 * NACC >= E experts.
// ---------------------------------------------------------------------------
constexpr int FBK = 32;
__host__ __device__ inline int64_t router_f32_stage_bytes(int Ecap) {
  return (64LL + Ecap) * (FBK + 1) * 4;
}

template <int NACC>
__global__ __launch_bounds__(256) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ w_r, const float* __restrict__ bias,
    int T, int d, int E, int k, int32_t* __restrict__ expert_idx, float* __restrict__ gate,
    int* __restrict__ hist, int NB, float* __restrict__ psum, int ldp, float* __restrict__ hout) {
  constexpr int Ecap = 4 * NACC;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int tok0 = b * 64;
  const int ntok = min(64, T - tok0);
  float* sx = reinterpret_cast<float*>(smem);  // [64][FBK+1]
  float* sw = sx + 64 * (FBK + 1);             // [Ecap][FBK+1]
  float* lg = reinterpret_cast<float*>(smem);  // [64][Ecap + 4]
  const int64_t body = max(router_f32_stage_bytes(Ecap), router_lg_bytes(64, Ecap));
  int* hl = reinterpret_cast<int*>(smem + body);

  for (int i = tid; i < k * Ecap; i += 256) hl[i] = 0;

  float acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = 0.f;
  const int t = tid & 63, eg = tid >> 6;
  constexpr int XL = 64 * FBK / 256, WL = Ecap * FBK / 256;  // loads per thread and stage
  for (int k0 = 0; k0 < d; k0 += FBK) {
    // every load of the stage in flight before the LDS stores (one memory round trip)
    float xv[XL], wv[WL];
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int id = tid + 256 * i, r = id / FBK, c = id - r * FBK;
      xv[i] = tok0 + r < T ? x[static_cast<int64_t>(tok0 + r) * d + k0 + c] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int id = tid + 256 * i, r = id / FBK, c = id - r * FBK;
      wv[i] = r < E ? w_r[static_cast<int64_t>(r) * d + k0 + c] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int id = tid + 256 * i, r = id / FBK, c = id - r * FBK;
      sx[r * (FBK + 1) + c] = xv[i];
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int id = tid + 256 * i, r = id / FBK, c = id - r * FBK;
      sw[r * (FBK + 1) + c] = wv[i];
    }
    __syncthreads();
#pragma unroll 4
    for (int kk = 0; kk < FBK; ++kk) {
      const float xv = sx[t * (FBK + 1) + kk];
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j] = fmaf(xv, sw[(eg + 4 * j) * (FBK + 1) + kk], acc[j]);
    }
    __syncthreads();
  }
  const int ld = Ecap + 4;
#pragma unroll
  for (int j = 0; j < NACC; ++j) lg[t * ld + eg + 4 * j] = acc[j];
  __syncthreads();
  topk_epilogue16<NACC / 4, 4>(lg, ld, 64, tok0, ntok, E, k, bias, expert_idx, gate, hl, Ecap, wave,
                            lane, psum ? psum + static_cast<int64_t>(b) * ldp : nullptr, lg, hout, ldp);
  __syncthreads();
  write_hist(hl, Ecap, E, k, NB, b, hist, tid, 256);
}

// ---------------------------------------------------------------------------
// Random Routed Experts: expert = g * size + (SplitMix64 output t) mod size.
// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output t of seed s mixes the
// state s + (t+1) * 0x9E3779B97F4A7C15 with two xor-shift-multiply rounds.
// One block of 64 threads per router block of 64 tokens.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t t) {
  uint64_t z = seed + (t + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(64) void router_rre_kernel(const int32_t* __restrict__ group_id, int T,
                                                        int E, int n_groups, uint64_t seed,
                                                        int32_t* __restrict__ expert_idx,
                                                        float* __restrict__ gate,
                                                        int* __restrict__ hist, int NB) {
  __shared__ int hl[kMaxE];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  for (int i = tid; i < E; i += 64) hl[i] = 0;
  __syncthreads();
  const int t = b * 64 + tid;
  if (t < T) {
    const int g = group_id[t];
    const int size = E / n_groups;
    int e = -1;
    if (g >= 0 && g < n_groups) {
      e = g * size + static_cast<int>(splitmix64_at(seed, static_cast<uint64_t>(t)) %
                                      static_cast<uint64_t>(size));
      atomicAdd(&hl[e], 1);
    }
    expert_idx[t] = e;
    gate[t] = e >= 0 ? 1.0f : 0.0f;
  }
  __syncthreads();
  write_hist(hl, kMaxE, E, 1, NB, b, hist, tid, 64);
}

// ---------------------------------------------------------------------------
// Load-balancing loss from the per-block rows: P_i = (sum over blocks of the
// probability sums) / T, f_i = (first choices of expert i) / T, loss =
// alpha * E * sum_i f_i P_i.  Two launches, float64 sums in a fixed order:
//   1. block (x, y): 64 experts x one of kAuxSplit contiguous ranges of router
//      blocks, summed in block order -> part_p[y][e], part_c[y][e];
//   2. one block: the ranges in order, then the loss over the experts.
// aux = [loss, f_0 .. f_{E-1}, P_0 .. P_{E-1}].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void router_aux_partial_kernel(
    const float* __restrict__ psum, int ldp, const int* __restrict__ hist, int E, int k, int NB,
    double* __restrict__ part_p, int64_t* __restrict__ part_c) {
  const int e = blockIdx.x * 64 + threadIdx.x;
  const int y = blockIdx.y, S = gridDim.y;
  if (e >= E) return;
  const int b0 = static_cast<int>(static_cast<int64_t>(y) * NB / S);
  const int b1 = static_cast<int>(static_cast<int64_t>(y + 1) * NB / S);
  double P = 0.0;
  int64_t cnt = 0;
  // sixteen loads in flight, then added in block order
  for (int b = b0; b < b1; b += 16) {
    float v[16];
    int c[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      v[j] = b + j < b1 ? psum[static_cast<int64_t>(b + j) * ldp + e] : 0.f;
      c[j] = b + j < b1 ? hist[(static_cast<int64_t>(e) * k) * NB + b + j] : 0;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      P += static_cast<double>(v[j]);
      cnt += c[j];
    }
  }
  part_p[static_cast<int64_t>(y) * ldp + e] = P;
  part_c[static_cast<int64_t>(y) * ldp + e] = cnt;
}

__global__ __launch_bounds__(256) void router_aux_kernel(const double* __restrict__ part_p,
                                                         const int64_t* __restrict__ part_c,
                                                         int ldp, int S, int T, int E,
                                                         double alpha, float* __restrict__ aux) {
  __shared__ double part[256];
  const int tid = threadIdx.x;
  double acc = 0.0;
  for (int e = tid; e < E; e += 256) {
    double P = 0.0;
    int64_t cnt = 0;
    for (int y = 0; y < S; y += 16) {
      double v[16];
      int64_t c[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        v[j] = y + j < S ? part_p[static_cast<int64_t>(y + j) * ldp + e] : 0.0;
        c[j] = y + j < S ? part_c[static_cast<int64_t>(y + j) * ldp + e] : 0;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        P += v[j];
        cnt += c[j];
      }
    }
    P /= T;
    const double f = static_cast<double>(cnt) / T;
    aux[1 + e] = static_cast<float>(f);
    aux[1 + E + e] = static_cast<float>(P);
    acc += f * P;
  }
  part[tid] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) aux[0] = static_cast<float>(alpha * E * part[0]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_split(const Plan& p, const float* w_r, void* ws, hipStream_t s) {
  bf16_t* planes = reinterpret_cast<bf16_t*>(ws_at(ws, p.off_planes));
  int* flags = reinterpret_cast<int*>(ws_at(ws, p.off_flags));
  hipLaunchKernelGGL(router_split_kernel, dim3(kSplitBlocks), dim3(256), 0, s, w_r, p.E, p.Epad,
                     static_cast<int>(p.d), planes, flags);
  return hipGetLastError();
}

template <typename K>
static hipError_t set_lds(K kernel, int64_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
}

hipError_t launch_router_topk(const Plan& p, const void* x, const float* w_r, const float* bias,
                              int32_t* expert_idx, float* gate, void* ws, hipStream_t s,
                              bool with_psum, float* logits) {
  if (p.T == 0) return hipSuccess;
  int* hist = reinterpret_cast<int*>(ws_at(ws, p.off_hist));
  float* psum = with_psum ? reinterpret_cast<float*>(ws_at(ws, p.off_psum)) : nullptr;
  const int T = static_cast<int>(p.T), d = static_cast<int>(p.d);
  hipError_t err;
  if (p.dtype == 1) {
    err = launch_router_split(p, w_r, ws, s);
    if (err != hipSuccess) return err;
    const bf16_t* planes = reinterpret_cast<const bf16_t*>(ws_at(ws, p.off_planes));
    const int* flags = reinterpret_cast<const int*>(ws_at(ws, p.off_flags));
    const bf16_t* xb = static_cast<const bf16_t*>(x);
#define MOE_ROUTER_BF16(TT, EW, S)                                                               \
  do {                                                                                           \
    const int64_t lds = std::max(router_ring_bytes(p.Epad, 32 * TT, S),                          \
                                 router_lg_bytes(32 * TT, p.Epad)) + 4LL * p.k * p.Epad;         \
    if ((err = set_lds(router_bf16_kernel<TT, EW, S>, lds)) != hipSuccess) return err;           \
    hipLaunchKernelGGL((router_bf16_kernel<TT, EW, S>), dim3(p.NB), dim3(512), lds, s, xb, planes, \
                       flags, bias, T, d, p.E, p.Epad, p.k, expert_idx, gate, hist, p.NB, psum,   \
                       logits);                                                                  \
  } while (0)
    if (p.Epad <= 128) {
      // six ring slots where they fit in LDS (32- and 64-token blocks: 123 / 151 KB):
      // Switch-Base router 15.5 -> 14.9 us, X-MoE 23.6 -> 22.7 us against four
      if (p.TB == 32) MOE_ROUTER_BF16(1, 1, 6);
      else if (p.TB == 64) MOE_ROUTER_BF16(2, 1, 6);
      else MOE_ROUTER_BF16(4, 1, 4);
    } else if (p.Epad <= 256) {
      if (p.TB == 32) MOE_ROUTER_BF16(1, 2, 3);
      else if (p.TB == 64) MOE_ROUTER_BF16(2, 2, 3);
      else MOE_ROUTER_BF16(4, 2, 3);
    } else {
      MOE_ROUTER_BF16(1, 4, 2);
    }
#undef MOE_ROUTER_BF16
  } else {
    const float* xf = static_cast<const float*>(x);
#define MOE_ROUTER_F32(N)                                                                        \
  do {                                                                                           \
    const int64_t lds = std::max(router_f32_stage_bytes(4 * N), router_lg_bytes(64, 4 * N)) +        \
                        4LL * p.k * 4 * N;                                                       \
    if ((err = set_lds(router_f32_kernel<N>, lds)) != hipSuccess) return err;                    \
    hipLaunchKernelGGL(router_f32_kernel<N>, dim3(p.NB), dim3(256), lds, s, xf, w_r, bias, T, d, \
                       p.E, p.k, expert_idx, gate, hist, p.NB, psum, p.Epad, logits);           \
  } while (0)
    if (p.E <= 32) MOE_ROUTER_F32(8);
    else if (p.E <= 64) MOE_ROUTER_F32(16);
    else if (p.E <= 128) MOE_ROUTER_F32(32);
    else if (p.E <= 256) MOE_ROUTER_F32(64);
    else MOE_ROUTER_F32(128);
#undef MOE_ROUTER_F32
  }
  return hipGetLastError();
}

hipError_t launch_router_aux(const Plan& p, double alpha, float* aux, void* ws, hipStream_t s) {
  const float* psum = reinterpret_cast<const float*>(ws_at(ws, p.off_psum));
  const int* hist = reinterpret_cast<const int*>(ws_at(ws, p.off_hist));
  // the range partials follow the block rows in the same region
  double* part_p = reinterpret_cast<double*>(ws_at(ws, p.off_psum + aux_rows_bytes(p)));
  int64_t* part_c = reinterpret_cast<int64_t*>(part_p + static_cast<int64_t>(kAuxSplit) * p.Epad);
  const int S = std::min(kAuxSplit, p.NB);
  hipLaunchKernelGGL(router_aux_partial_kernel, dim3((p.E + 63) / 64, S), dim3(64), 0, s, psum,
                     p.Epad, hist, p.E, p.k, p.NB, part_p, part_c);
  hipLaunchKernelGGL(router_aux_kernel, dim3(1), dim3(256), 0, s, part_p, part_c, p.Epad, S,
                     static_cast<int>(p.T), p.E, alpha, aux);
  return hipGetLastError();
}

hipError_t launch_router_rre(const Plan& p, const int32_t* group_id, int32_t* expert_idx,
                             float* gate, void* ws, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  int* hist = reinterpret_cast<int*>(ws_at(ws, p.off_hist));
  hipLaunchKernelGGL(router_rre_kernel, dim3(p.NB), dim3(64), 0, s, group_id,
                     static_cast<int>(p.T), p.E, p.n_groups, p.rre_seed, expert_idx, gate, hist,
                     p.NB);
  return hipGetLastError();
}

}  // namespace moe
