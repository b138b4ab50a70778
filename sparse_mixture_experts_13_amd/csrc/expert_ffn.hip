// Grouped expert FFN: y_e = act(x_e W1_e) W2_e for every expert at once
// (Switch Transformers notes, section 2.1: one feed-forward network E_i per
// expert; section 2.2: each expert computes a static-capacity batch, of which
// only the first expert_count[e] rows hold tokens).
//
// Two launches of one grouped GEMM: hidden = act(x_e . w1[e]^T), then
// y_e = hidden . w2[e]^T.  Both operands are stored K-contiguous (activations
// [E][C][K], weights [E][N][K]).  The kernel computes the transposed tile
// D = W . X^T so that each lane ends with four consecutive output columns of
// one row (8-byte stores).  bf16 runs on v_mfma_f32_32x32x16_bf16 with float32
// accumulation in persistent kernels over the non-empty tiles only (a stage
// ring kernel, and a ping-pong kernel for MFMA-bound tiles with long
// contractions), so the grid is fixed (no device-to-host read of the counts)
// while dropped or unused capacity costs neither bandwidth nor MFMA work.
// float32 workloads use a plain float32 FMA tile kernel.
//
// Gated-linear-unit experts (MosaicBERT review, methodology: GLU in the
// feed-forward layer, in a fused form): H = act(x W) * (x V) with w1 = [W; V]
// stacked (2 d_ff rows).  The up-projection is one grouped GEMM over the 2 d_ff
// rows in a permuted row order: virtual weight row v is physical row
// glu_row(v), so that every 32-row MFMA tile holds 16 units of W followed by the
// same 16 units of V.  Each lane then holds both halves of its units in its own
// accumulators (rows 8q + 4h + u and 16 + 8q + 4h + u), and the epilogue writes
// act(a) * b once, in bfloat16 from the float32 accumulators: no pre-activation
// reaches memory and no second pass runs.
#include "moe_common.h"
#include "moe_internal.h"

#include <algorithm>

namespace moe {

constexpr int GBK = 64;
constexpr int GLD = GBK + 8;

// Physical w1 row of virtual row v of the GLU up-projection (f = d_ff): 32-row
// groups of 16 rows of W (rows 0 .. f - 1) and the same 16 units of V (rows f ..).
__device__ __forceinline__ int glu_row(int v, int f) {
  return ((v & 16) ? f : 0) + ((v >> 5) << 4) + (v & 15);
}

template <int BM, int BN>
__host__ __device__ constexpr int ffn_lds_bytes() {
  return 2 * (BM + BN) * GLD * 2;
}

// LDS-tiled grouped GEMM, for experts whose panels exceed 32-bit element offsets
// (the persistent kernels address inside an expert with 32-bit offsets): one
// block per (expert, row tile, column tile) of BM x BN, register-staged
// double-buffered LDS tiles (BK = 64, rows padded to 144 bytes: conflict-free
// fragment reads); tiles past the expert's count exit at once.
template <int BM, int BN, int WM, int WN, int ACT, bool GLU>
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
  const bf16_t* We = W + static_cast<int64_t>(e) * N * K;

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
      const int wr = GLU ? glu_row(n0 + r, N >> 1) : n0 + r;
      rp[i] = n0 + r < N ? *reinterpret_cast<const u32x4*>(We + static_cast<int64_t>(wr) * K + k0 + c * 8)
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
  if constexpr (GLU) {
    // GLU: elements 4g + u (g = 0, 1) hold the W half of unit 8g + 4h + u of the
    // tile's 16 units, elements 4g + 8 + u the V half of the same unit
    const int No = N >> 1;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int m = m0 + wm * WTM + j * 32 + fr;
      if (m < cnt) {
        bf16_t* orow = out + (static_cast<int64_t>(e) * C + m) * No;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          const int nt = n0 + wn * WTN + i * 32;
          if (nt < N) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              float h[4];
#pragma unroll
              for (int u = 0; u < 4; ++u) h[u] = apply_act<ACT>(acc[i][j][4 * g + u]) * acc[i][j][4 * g + 8 + u];
              uint2 v;
              v.x = pack_bf16x2(h[0], h[1]);
              v.y = pack_bf16x2(h[2], h[3]);
              *reinterpret_cast<uint2*>(orow + (nt >> 1) + 8 * g + 4 * (lane >> 5)) = v;
            }
          }
        }
      }
    }
    return;
  }
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

// ---------------------------------------------------------------------------
// Persistent grouped GEMM on bf16 MFMA with a direct-to-LDS stage ring.
//
// Tiles are (expert e, row block mb, column block nb) of BM x BN outputs,
// BM = WM * TM * 32 activation rows and BN = WN * TN * 32 weight rows; wave
// (wm, wn) of the WM x WN wave grid owns TM x TN MFMA tiles of 32 x 32.  Only
// tiles holding tokens exist (expert e has ceil(count[e] / BM) row blocks), and
// each block takes an equal contiguous share of them, in (e, mb, nb) order.
//
// A block streams its share as one sequence of 64-k stages:
//   * stages land in an S-deep LDS ring through direct global->LDS 16-byte
//     loads issued S-1 stages ahead, across tile boundaries (no per-tile
//     pipeline fill); weight loads are non-temporal when a weight tile is
//     read by one row block only (each byte read once per launch), and every
//     wave instruction covers whole 128-byte row segments;
//   * LDS rows are 128 bytes with the 16-byte chunk index XORed by
//     (row / 2) % 8, so the MFMA fragment reads hit distinct banks;
//   * blocks are renumbered so that consecutive shares (mostly one expert)
//     run on one XCD and share activations and weights in that L2.
// Rows past the expert's count (and weight rows past N) are loaded from a
// clamped valid row: their products land only in outputs that are never
// stored, so every stage issues the same number of loads and the wait for a
// stage is a fixed memory-counter threshold.
// Inside a 64-k stage, MFMA j (j = 0..3) of lane half h contracts the 16-byte
// chunk 2j + h of each row: A and B fragments use the same k assignment.
// ---------------------------------------------------------------------------
// LDS: stage ring | tile prefix per expert
template <int TM, int TN, int WM, int WN, int S, int BK>
__host__ __device__ constexpr int ffn_ring_lds_bytes() {
  return S * (WN * TN * 32 + WM * TM * 32) * BK * 2 + (kMaxE + 1) * 4;
}

// PAIR: the unit of work is two adjacent column tiles of one row block (column
// blocks 2 u and 2 u + 1), multiplied together: the stages alternate between
// their weight rows at each k-chunk (k-chunk i of half 0, then of half 1), each
// stage carrying the row block's k-chunk i, so the second copy of every
// activation chunk is read while the first is still in L2.
// TOK (the whole-layer forward, two ring slots): A is the token rows x [T][K] and
// row s of expert e is x[tok[e C + s]], so the dispatch copies no rows.  Each lane
// keeps the token of each of its activation-load rows for the loader's current
// tile, loaded when the loader moves to the tile, at the end of a stage: with two
// slots every stage starts by waiting for all loads, so those tokens have landed
// before the next stage's loads use them.
template <int TM, int TN, int WM, int WN, int S, int BK, bool NTW, int ACT, bool GLU, bool PAIR = false,
          bool TOK = false>
__global__ __launch_bounds__(WM * WN * 64) void ffn_ring_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, bf16_t* __restrict__ out,
    const int32_t* __restrict__ count, int E, int64_t C, int N, int K,
    const int32_t* __restrict__ tok = nullptr) {
  static_assert(!TOK || S == 2, "token-row loads rely on the two-slot ring's full wait per stage");
  constexpr int NW = WM * WN;
  constexpr int NH = PAIR ? 2 : 1;  // column tiles per unit
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int RB = BK * 2;         // LDS row bytes
  constexpr int CPR = BK / 8;        // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;     // rows per wave instruction (64 lanes x 16 bytes)
  constexpr int WL = BN / RPI / NW;  // direct-to-LDS instructions per wave per stage (weights)
  constexpr int AL = BM / RPI / NW;  // ... (activations)
  static_assert(BK == 32 || BK == 64, "stage depth");
  static_assert(BN % (RPI * NW) == 0 && BM % (RPI * NW) == 0 && AL >= 1, "stage split");
  constexpr int STAGE = (BN + BM) * RB;
  constexpr int PER_STAGE = WL + AL;
  static_assert((S - 2) * PER_STAGE < 64, "memory counter range");
  extern __shared__ __align__(16) unsigned char smem[];
  int* pre = reinterpret_cast<int*>(smem + S * STAGE);  // [E + 1] tile prefix per expert

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave - (wave / WN) * WN;
  const int half = lane >> 5, fr = lane & 31;
  const int n_nb = (N + BN * NH - 1) / (BN * NH);  // column units (PAIR: N % (2 BN) == 0)
  const int KS = K / BK;

  auto rows_of = [&](int e) {
    int64_t c = count[e];
    return static_cast<int>(c < 0 ? 0 : (c > C ? C : c));
  };
  // prefix of non-empty tiles over experts (wave 0), shared through LDS
  if (wave == 0) {
    int run = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int t = e < E ? (rows_of(e) + BM - 1) / BM * n_nb : 0;
      const int incl = wave_inclusive_scan(t, lane) + run;
      if (e < E) pre[e + 1] = incl;
      run = __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) pre[0] = 0;
  }
  __syncthreads();
  const int V = pre[E];
  const int G = gridDim.x;
  // This block's tiles: v0, v0 + vs, v0 + 2 vs, ... below v1.
  //   * non-temporal weights (each weight tile read by one row block): an equal
  //     contiguous share per block, consecutive shares on one XCD;
  //   * temporal weights (large capacities, MFMA-bound): each XCD takes a
  //     contiguous eighth of the tiles and its blocks take them strided, so all of
  //     an XCD's blocks work on one expert at a time: its activation rows stay in
  //     that XCD's L2 and each weight tile is fetched once while the blocks of its
  //     row blocks read it together (X-MoE top-2: L2 hit rate 51% with shares).
  int v0, v1, vs;
  if constexpr (NTW) {
    const int g = xcd_major_id(blockIdx.x, G);
    v0 = static_cast<int>(static_cast<int64_t>(g) * V / G);
    v1 = static_cast<int>(static_cast<int64_t>(g + 1) * V / G);
    vs = 1;
  } else {
    const int NX = G < 8 ? G : 8;  // XCD groups (blocks are dispatched to XCDs round robin)
    const int x = blockIdx.x % NX, j = blockIdx.x / NX;
    v0 = static_cast<int>(static_cast<int64_t>(x) * V / NX) + j;
    v1 = static_cast<int>(static_cast<int64_t>(x + 1) * V / NX);
    vs = (G - x + NX - 1) / NX;  // blocks in this group
  }
  const int ntile = v0 < v1 ? (v1 - v0 + vs - 1) / vs : 0;
  const int total = ntile * KS * NH;
  if (total == 0) return;

  // a tile cursor: expert, row block, column block of linear non-empty tile v;
  // with temporal weights (row blocks re-read the weight tiles) the row blocks
  // of a weight tile are consecutive, so its re-reads hit L2 (X-MoE top-2: 3-4%
  // faster than column blocks fastest)
  struct Cur { int v, e, mb, nb, cnt; };
  auto seek = [&](Cur& c, int v) {
    c.v = v;
    int e = c.e;  // tiles are visited in increasing order: resume the search
    while (pre[e + 1] <= v) ++e;
    const int local = v - pre[e];
    c.e = e;
    c.cnt = rows_of(e);
    if constexpr (!NTW) {
      const int nmb = (c.cnt + BM - 1) / BM;
      c.nb = local / nmb;
      c.mb = local - c.nb * nmb;
    } else {
      c.mb = local / n_nb;
      c.nb = local - c.mb * n_nb;
    }
  };
  auto next = [&](Cur& c) {
    ++c.v;
    if constexpr (!NTW) {
      if (++c.mb == (c.cnt + BM - 1) / BM) {
        c.mb = 0;
        ++c.nb;
        if (c.v < pre[c.e + 1]) return;
        do { ++c.e; } while (c.e < E && pre[c.e + 1] <= c.v);
        c.nb = 0;
        if (c.e < E) c.cnt = rows_of(c.e);
      }
    } else if (++c.nb == n_nb) {
      c.nb = 0;
      ++c.mb;
      if (c.v < pre[c.e + 1]) return;
      do { ++c.e; } while (c.e < E && pre[c.e + 1] <= c.v);
      c.mb = 0;
      if (c.e < E) c.cnt = rows_of(c.e);
    }
  };

  auto step = [&](Cur& c) {
    if (vs == 1) {
      next(c);
    } else if (c.v + vs >= V) {  // past the last tile: never used, and seek must not scan past pre[E]
      c.v += vs;
      c.e = E;
    } else {
      seek(c, c.v + vs);
    }
  };

  Cur lc, cc;
  lc.e = 0;
  seek(lc, v0);
  cc = lc;
  int lk = 0, lh = 0;  // loader: k-chunk and column half of the stage it issues next
  // TOK: token of this lane's row of activation load q in the loader's tile
  int tokv[AL];
  auto load_tok = [&]() {
    if constexpr (TOK) {
      if (lc.e < E) {
#pragma unroll
        for (int qa = 0; qa < AL; ++qa) {
          const int row = ((wave * AL + qa) * 64 + lane) / CPR;
          tokv[qa] = tok[static_cast<int64_t>(lc.e) * C + min(lc.mb * BM + row, lc.cnt - 1)];
        }
      }
    }
  };
  load_tok();
  // Loads use a block-uniform per-expert base plus 32-bit lane offsets.
  // issue_one(slot, q) issues the q-th of the PER_STAGE direct-to-LDS
  // instructions of the loader's current stage; advance() moves to the next.
  auto issue_one = [&](int slot, int q) {
    unsigned char* base = smem + slot * STAGE;
    if (q < WL) {
      const bf16_t* We = W + static_cast<int64_t>(lc.e) * N * K;
      const int p = (wave * WL + q) * 64 + lane;
      const int row = p / CPR;
      const int c = (p % CPR) ^ lds_swz_n<CPR>(row);
      int wr = min((lc.nb * NH + lh) * BN + row, N - 1);
      if constexpr (GLU) wr = glu_row(wr, N >> 1);
      const uint32_t off = static_cast<uint32_t>(wr) * K + lk * BK + c * 8;
      // non-temporal when each weight tile is read by one row block only
      __builtin_amdgcn_global_load_lds(We + off, (lds_void*)(base + (wave * WL + q) * 1024), 16, 0,
                                       NTW ? 2 : 0);
    } else {
      const int qa = q - WL;
      const int p = (wave * AL + qa) * 64 + lane;
      const int row = p / CPR;
      const int c = (p % CPR) ^ lds_swz_n<CPR>(row);
      const bf16_t* src;
      if constexpr (TOK) {
        src = A + static_cast<int64_t>(tokv[qa]) * K + lk * BK + c * 8;
      } else {
        const bf16_t* Ae = A + static_cast<int64_t>(lc.e) * C * K;
        src = Ae + static_cast<uint32_t>(min(lc.mb * BM + row, lc.cnt - 1)) * K + lk * BK + c * 8;
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + BN * RB + (wave * AL + qa) * 1024),
                                       16, 0, 0);
    }
  };
  auto advance = [&]() {
    if (PAIR && ++lh < NH) return;
    lh = 0;
    if (++lk == KS) {
      lk = 0;
      step(lc);
      load_tok();
    }
  };
  auto issue = [&](int slot) {
#pragma unroll
    for (int q = 0; q < PER_STAGE; ++q) issue_one(slot, q);
    advance();
  };

  floatx16 acc[NH][TN][TM];
  auto zero_acc = [&]() {
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[h][i][t][r] = 0.f;
  };
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < total) issue(i);
  int s = 0;  // stage index over the block's whole sequence
  for (int it = 0; it < ntile; ++it) {
    zero_acc();
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh, ++s) {
        if (total - 1 - s >= S - 2) wait_vmcnt<(S - 2) * PER_STAGE>();
        else wait_vmcnt<0>();
        ring_barrier();
        // the next stage's loads are spread between this stage's MFMAs, so that
        // issuing them does not stall the wave ahead of its math
        const bool pf = s + S - 1 < total;
        const int pslot = (s + S - 1) % S;
        const unsigned char* sw = smem + (s % S) * STAGE;
        const unsigned char* sa = sw + BN * RB;
        // fragments of sub-step j + 1 load while sub-step j's MFMAs run
        bf16x8 fa[2][TN], fb[2][TM];
        auto load_frags = [&](int j, int buf) {
          const int c = 2 * j + half;
#pragma unroll
          for (int t = 0; t < TM; ++t) {
            const int row = (wm * TM + t) * 32 + fr;
            fb[buf][t] = *reinterpret_cast<const bf16x8*>(sa + row * RB + 16 * (c ^ lds_swz_n<CPR>(row)));
          }
#pragma unroll
          for (int i = 0; i < TN; ++i) {
            const int row = (wn * TN + i) * 32 + fr;
            fa[buf][i] = *reinterpret_cast<const bf16x8*>(sw + row * RB + 16 * (c ^ lds_swz_n<CPR>(row)));
          }
        };
        constexpr int NJ = BK / 16;           // MFMA sub-steps per stage
        constexpr int MT = NJ * TN * TM;      // MFMAs per stage
        load_frags(0, 0);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (j + 1 < NJ) load_frags(j + 1, (j + 1) & 1);
#pragma unroll
          for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int t = 0; t < TM; ++t) {
              const int mi = (j * TN + i) * TM + t;
#pragma unroll
              for (int q = 0; q < PER_STAGE; ++q)
                if (q * MT / PER_STAGE == mi && pf) issue_one(pslot, q);
              acc[hh][i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j & 1][i], fb[j & 1][t], acc[hh][i][t], 0, 0, 0);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (pf) advance();
      }
    // tile done: D[n][m], lane holds m = lane % 32 and four consecutive n per group
    const int m0 = cc.mb * BM;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const int n0 = (cc.nb * NH + hh) * BN;
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int m = m0 + (wm * TM + t) * 32 + fr;
        if (GLU && m < cc.cnt) {
          // elements 4q + u (q = 0, 1): W half of unit 8q + 4h + u of the 32-row
          // tile's 16 units; elements 4q + 8 + u: the V half of the same unit
          bf16_t* orow = out + (static_cast<int64_t>(cc.e) * C + m) * (N >> 1);
#pragma unroll
          for (int i = 0; i < TN; ++i) {
            const int nt0 = n0 + (wn * TN + i) * 32;
            if (nt0 < N) {
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                float h[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) h[u] = apply_act<ACT>(acc[hh][i][t][4 * q + u]) * acc[hh][i][t][4 * q + 8 + u];
                uint2 v;
                v.x = pack_bf16x2(h[0], h[1]);
                v.y = pack_bf16x2(h[2], h[3]);
                *reinterpret_cast<uint2*>(orow + (nt0 >> 1) + 8 * q + 4 * half) = v;
              }
            }
          }
        } else if (m < cc.cnt) {
          bf16_t* orow = out + (static_cast<int64_t>(cc.e) * C + m) * N;
#pragma unroll
          for (int i = 0; i < TN; ++i) {
            const int nt0 = n0 + (wn * TN + i) * 32;
            if (nt0 < N) {  // N % 32 == 0: a 32-column tile is wholly valid or not
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int n = nt0 + 8 * q + 4 * half;
                uint2 v;
                v.x = pack_bf16x2(apply_act<ACT>(acc[hh][i][t][4 * q]), apply_act<ACT>(acc[hh][i][t][4 * q + 1]));
                v.y = pack_bf16x2(apply_act<ACT>(acc[hh][i][t][4 * q + 2]), apply_act<ACT>(acc[hh][i][t][4 * q + 3]));
                *reinterpret_cast<uint2*>(orow + n) = v;
              }
            }
          }
        }
      }
    }
    step(cc);
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM with the activation rows resident in LDS, for capacity <= 64 and
// a contraction K <= 768 (the Switch-Base up-projection): every expert's rows
// fit one 64-row block, and each of its column tiles would otherwise re-read
// them with every stage (a fifth of the ring's load stream at 256 weight rows
// per stage).  A block takes a contiguous share of the (expert, 256-column
// block) tiles of the non-empty experts, consecutive shares on one XCD; for each
// run of tiles of one expert it loads that expert's 64 x K activations into LDS
// once (clamped rows past the count), then streams only weight rows: stages of
// 128 weight rows x 64 k (16 KB) through a 3-slot direct-to-LDS ring.  Stage
// 2i + h of a tile carries k-chunk i of its rows 128 h .. + 127; waves 4 h ..
// 4 h + 3 (32 weight rows each, all 64 activation rows: two 32 x 32 MFMA tiles)
// multiply it.  The ring drains at a change of expert (at most a couple of
// times per block).  In a memory-traffic emulation of the Switch-Base
// up-projection (loads only, cold weights) this stream takes 95 us against
// 105 us for the ring's 40 KB stages.
// Output rows leave through a 32-row LDS staging tile as whole 512-byte row
// segments with non-temporal stores: the hidden rows reach memory during this
// kernel, where 8-byte stores left partly written lines in the caches whose
// write-back then slowed the down-projection (Switch-Base, kernel traces of the
// same forward steps: up 122 -> 114 us, down 129 -> 115 us, step 282 -> 262 us).
// Waves 0-3 issue every load and waves 4-7 every output store, so no load wait
// covers a store (gfx9 counts both in one counter).  GLU outputs (half-width
// rows, two halves per unit) keep the direct 8-byte stores of the ring kernel.
// With `tok` (the whole-layer call) A is the token rows x [T][K] and row s of
// expert e is x[tok[e C + s]]: the resident load gathers the rows itself and
// the dispatch writes no x_e.  The block loads the expert's 64 slot tokens with
// one vector load, issues its first weight stages, then the row loads (each
// lane's token from a cross-lane read).
// ---------------------------------------------------------------------------
constexpr int kResRing = 3;                 // ring slots
constexpr int kResStage = 128 * 128;        // 128 weight rows x 128 bytes
constexpr int kResMaxK = 768;               // resident activations: 64 rows x K bf16 <= 96 KB
constexpr int kResStg = 32 * 512;           // output staging: 32 rows x 256 columns bf16
__host__ __device__ constexpr int ffn_res_lds_bytes(int K) {
  return kResRing * kResStage + kResStg + (K / 64) * 8192;
}

template <int ACT, bool GLU>
__global__ __launch_bounds__(512) void ffn_res_bf16_kernel(const bf16_t* __restrict__ A,
                                                           const bf16_t* __restrict__ W,
                                                           bf16_t* __restrict__ out,
                                                           const int32_t* __restrict__ count,
                                                           int E, int64_t C, int N, int K,
                                                           const int32_t* __restrict__ tok) {
  constexpr int S = kResRing, BN = 256, CPR = 8;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* stg = smem + S * kResStage;          // [32 rows][512 bytes], chunk c at c ^ row
  unsigned char* ares = stg + kResStg;                // [K / 64 chunks][64 rows][128 bytes]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, fr = lane & 31;
  const int KS = K / 64;
  const int n_nb = (N + BN - 1) / BN;
  auto rows_of = [&](int e) {
    int64_t c = count[e];
    return static_cast<int>(c < 0 ? 0 : (c > C ? C : c));
  };
  // the non-empty experts as a bit mask (E <= 512), the same in every wave
  uint64_t nz[kMaxE / 64];
  int nne = 0;
#pragma unroll
  for (int i = 0; i < kMaxE / 64; ++i) {
    const int e = i * 64 + lane;
    nz[i] = __ballot(e < E && rows_of(e) > 0);
    nne += __popcll(nz[i]);
  }
  const int V = nne * n_nb;
  const int G = gridDim.x;
  const int g = xcd_major_id(blockIdx.x, G);
  const int v0 = static_cast<int>(static_cast<int64_t>(g) * V / G);
  const int v1 = static_cast<int>(static_cast<int64_t>(g + 1) * V / G);
  // the j-th non-empty expert (wave-uniform scalar search)
  auto nth_expert = [&](int j) {
#pragma unroll
    for (int i = 0; i < kMaxE / 64; ++i) {
      uint64_t m = nz[i];
      const int pc = __popcll(m);
      if (j < pc) {
        for (int r = 0; r < j; ++r) m &= m - 1;  // drop the j lowest set bits
        return i * 64 + __builtin_ctzll(m);
      }
      j -= pc;
    }
    return E;
  };

  floatx16 acc[2];
  for (int v = v0; v < v1;) {
    const int j = v / n_nb;
    const int e = nth_expert(j);
    const int nb0 = v - j * n_nb;
    const int nb1 = min(n_nb, nb0 + (v1 - v));
    v += nb1 - nb0;
    const int cnt = rows_of(e);
    const int nst = (nb1 - nb0) * KS * 2;  // stages of this run of tiles
    const bf16_t* We = W + static_cast<int64_t>(e) * N * K;
    auto issue = [&](int st) {
      const int nb = nb0 + (st >> 1) / KS, kc = (st >> 1) % KS, h = st & 1;
      unsigned char* base = smem + (st % S) * kResStage;
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // loader waves 0-3
        const int p = (wave * 4 + q) * 64 + lane;
        const int row = p / CPR;
        const int c = (p % CPR) ^ lds_swz_n<CPR>(row);
        int wr = min(nb * BN + h * 128 + row, N - 1);
        if constexpr (GLU) wr = glu_row(wr, N >> 1);
        const uint32_t off = static_cast<uint32_t>(wr) * K + kc * 64 + c * 8;
        // non-temporal: each weight byte is read once per launch
        __builtin_amdgcn_global_load_lds(We + off, (lds_void*)(base + (wave * 4 + q) * 1024), 16, 0, 2);
      }
    };
    __syncthreads();  // the previous run is done with the ring and the resident rows
    // resident activations: chunk kc of rows 0..63 at ares + kc * 8 KB, 2 KS loads per wave
    if (tok == nullptr) {
      const bf16_t* Ae = A + static_cast<int64_t>(e) * C * K;
      for (int q = 0; q < 2 * KS && wave < 4; ++q) {
        const int p = (wave * 2 * KS + q) * 64 + lane;  // 16-byte chunk p of [KS][64][8]
        const int kc = p >> 9, row = (p >> 3) & 63;
        const int c = (p % CPR) ^ lds_swz_n<CPR>(row);
        const uint32_t off = static_cast<uint32_t>(min(row, cnt - 1)) * K + kc * 64 + c * 8;
        __builtin_amdgcn_global_load_lds(Ae + off, (lds_void*)(ares + (wave * 2 * KS + q) * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < S - 1; ++i)
        if (i < nst && wave < 4) issue(i);
    } else if (wave < 4) {
      // lane l: the token of slot min(l, cnt - 1); the first weight stages go out
      // while it arrives, the row loads after them (the main loop's first wait
      // then drains every load of the wave)
      const int trow = tok[static_cast<int64_t>(e) * C + min(lane, cnt - 1)];
#pragma unroll
      for (int i = 0; i < S - 1; ++i)
        if (i < nst) issue(i);
      for (int q = 0; q < 2 * KS; ++q) {
        const int p = (wave * 2 * KS + q) * 64 + lane;
        const int kc = p >> 9, row = (p >> 3) & 63;
        const int c = (p % CPR) ^ lds_swz_n<CPR>(row);
        const int t = __shfl(trow, row, kWave);
        const bf16_t* src = A + static_cast<int64_t>(t) * K + kc * 64 + c * 8;
        __builtin_amdgcn_global_load_lds(src, (lds_void*)(ares + (wave * 2 * KS + q) * 1024), 16, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    const int wh = wave >> 2;                 // the half of the tile's rows this wave multiplies
    const int wrow = (wave & 3) * 32 + fr;    // its fragment row within a stage
    for (int st = 0; st < nst; ++st) {
      // this wave's loads of stage st (and, before the first, of the resident rows)
      if (wave < 4) {  // loader waves; waves 4-7 issue only the output stores
        if (nst - 1 - st >= S - 2 && (tok == nullptr || st > 0)) wait_vmcnt<(S - 2) * 4>();
        else wait_vmcnt<0>();
      }
      ring_barrier();
      if (st + S - 1 < nst && wave < 4) issue(st + S - 1);
      const int kc = (st >> 1) % KS;
      if ((st & 1) == wh) {
        const unsigned char* sw = smem + (st % S) * kResStage;
        const unsigned char* sa = ares + kc * 8192;
        bf16x8 fa[4], fb[4][2];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int c = 2 * jj + half;
          fa[jj] = *reinterpret_cast<const bf16x8*>(sw + wrow * 128 + 16 * (c ^ lds_swz_n<CPR>(wrow)));
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int row = t * 32 + fr;
            fb[jj][t] = *reinterpret_cast<const bf16x8*>(sa + row * 128 + 16 * (c ^ lds_swz_n<CPR>(row)));
          }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[jj], fb[jj][t], acc[t], 0, 0, 0);
      }
      if ((st & 1) == 1 && kc == KS - 1) {
        // tile done: D[n][m], lane holds m = lane % 32 and four consecutive n per group
        const int n0t = (nb0 + (st >> 1) / KS) * BN;
        const int nt0 = n0t + wave * 32;
        if constexpr (GLU) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int m = t * 32 + fr;
            if (m < cnt && nt0 < N) {
              bf16_t* orow = out + (static_cast<int64_t>(e) * C + m) * (N >> 1);
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                float hv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) hv[u] = apply_act<ACT>(acc[t][4 * q + u]) * acc[t][4 * q + 8 + u];
                uint2 val;
                val.x = pack_bf16x2(hv[0], hv[1]);
                val.y = pack_bf16x2(hv[2], hv[3]);
                *reinterpret_cast<uint2*>(orow + (nt0 >> 1) + 8 * q + 4 * half) = val;
              }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
          }
        } else {
          // two 32-row passes through the staging tile, then whole 512-byte row
          // segments (four cache lines) per 32 threads, non-temporal: the hidden rows
          // go to memory now instead of being written back during the next kernel
#pragma unroll
          for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int n = wave * 32 + 8 * q + 4 * half;  // column within the tile
              uint2 val;
              val.x = pack_bf16x2(apply_act<ACT>(acc[t][4 * q]), apply_act<ACT>(acc[t][4 * q + 1]));
              val.y = pack_bf16x2(apply_act<ACT>(acc[t][4 * q + 2]), apply_act<ACT>(acc[t][4 * q + 3]));
              *reinterpret_cast<uint2*>(stg + fr * 512 + (((n >> 3) ^ fr) << 4) + (n & 7) * 2) = val;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
            ring_barrier();
            if (wave >= 4) {
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) {
                const int q = (tid - 256) + 256 * ii;
                const int ml = q >> 5, c = q & 31;
                const int m = t * 32 + ml, n = n0t + c * 8;
                if (m < cnt && n < N)
                  __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stg + ml * 512 + ((c ^ ml) << 4)),
                                              reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(e) * C + m) * N + n));
              }
            }
            ring_barrier();  // staging reads done before it is written again
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Ping-pong grouped GEMM for large capacities, where a tile re-reads its weight
// rows for several row blocks and the MFMA pipe, not HBM, sets the pace.
//
// Block tile: BM = 64 TM activation rows x BN = 128 TN weight rows (128 x 256
// with 64-k stages in the forward; 256 x 256 or 128 x 512 with 32-k stages in
// the BT form below), persistent blocks of 8 waves in two groups of four (waves w and
// w + 4 share a SIMD).  Wave (g, wn) owns activation rows g BM / 2 .. and weight
// rows wn BN / 4 .. of the tile: TM x TN MFMA tiles of 32 x 32.  The k loop runs
// in BK-k stages through an R-slot direct-to-LDS ring, and every stage has two
// phases separated by block barriers:
//   * memory phase: read the wave's fragments of the stage from LDS, issue its
//     direct-to-LDS loads of the stage R - 1 ahead, wait for its own loads of
//     the next stage;
//   * MFMA phase: (BK / 16) TM TN MFMAs on the fragments in registers (and the tile's
//     epilogue after its last stage).
// Group 1 runs one phase behind group 0, so on every SIMD one wave issues
// MFMAs while the other feeds LDS and memory: the matrix pipe never waits for
// a fragment read or a barrier of its own wave.  Tiles (expert, row block,
// column block), the per-XCD strided share of them and the clamped rows past
// the count are as in the ring kernel above; the loads of the block's last
// stages re-read its final stage into free slots, so every memory phase issues
// the same loads and waits on one fixed memory-counter threshold.
// BT: the second operand is stored [K][N] per expert (row pitch N) instead of
// [N][K] -- the weights of the backward's token-row products dZ = dy_e w2 and
// dx_e = dZ w1.  Its stage tile is then [32 k rows][BN] and its fragments come
// from two LDS transpose reads (ds_read_b64_tr_b16: within each 16-lane group,
// lane i receives element i % 4 of the 8-byte chunks addressed by lanes
// 4 q + i / 4); the 16-byte chunk c of k row r sits at chunk position
// c ^ 4 (r mod 4), so that every 32 lanes of a transpose read hit 32 distinct
// 8-byte bank slots.  EPI 1 multiplies the product by act'(z), z read from
// `aux` at the output position (the backward's dZ).
// ---------------------------------------------------------------------------
// TM x TN MFMA tiles per wave (activation, weight), R ring slots of BK-k stages.
template <int TM, int TN, int R, int BK = 32>
__host__ __device__ constexpr int ffn_pp_lds_bytes() {
  return R * (2 * TM * 32 + 4 * TN * 32) * BK * 2 + (2 * kMaxE + 1) * 4;
}

template <int TM, int TN, int R, int ACT, bool GLU, bool BT = false, int EPI = 0, int BK = 32>
__global__ __launch_bounds__(512) void ffn_pp_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, bf16_t* __restrict__ out,
    const int32_t* __restrict__ count, int E, int64_t C, int N, int K, const bf16_t* __restrict__ aux) {
  static_assert(!(BT && GLU) && (EPI == 0 || (EPI == 1 && !GLU)), "operand and epilogue forms");
  static_assert(BK == 32 || BK == 64, "stage depth");
  constexpr int BM = 2 * TM * 32, BN = 4 * TN * 32;
  constexpr int NJ = BK / 16;            // MFMA sub-steps per stage
  constexpr int KRB = BN * 2;            // BT: bytes per k row of the weight stage tile
  constexpr int RB = BK * 2;             // LDS row bytes
  constexpr int CPR = BK / 8;            // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;         // rows per wave instruction
  constexpr int WL = BN / RPI / 8;       // weight instructions per wave per stage
  constexpr int AL = BM / RPI / 8;       // activation instructions per wave per stage
  constexpr int PER = WL + AL;
  constexpr int STAGE = (BN + BM) * RB;
  static_assert(BN % (RPI * 8) == 0 && BM % (RPI * 8) == 0 && R >= 3, "stage split");
  extern __shared__ __align__(16) unsigned char smem[];
  int* pre = reinterpret_cast<int*>(smem + R * STAGE);  // [E + 1] tile prefix per expert
  int* cnts = pre + kMaxE + 1;                            // [E] clamped row counts

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wn = wave & 3;
  const int half = lane >> 5, fr = lane & 31;
  const int n_nb = (N + BN - 1) / BN;
  const int KS = K / BK;

  auto rows_of = [&](int e) {
    int64_t c = count[e];
    return static_cast<int>(c < 0 ? 0 : (c > C ? C : c));
  };
  if (wave == 0) {
    int run = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int r = e < E ? rows_of(e) : 0;
      const int t = (r + BM - 1) / BM * n_nb;
      const int incl = wave_inclusive_scan(t, lane) + run;
      if (e < E) {
        pre[e + 1] = incl;
        cnts[e] = r;
      }
      run = __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) pre[0] = 0;
  }
  __syncthreads();
  const int V = pre[E];
  const int G = gridDim.x;
  // each XCD takes a contiguous eighth of the tiles, its blocks take them strided
  const int NX = G < 8 ? G : 8;
  const int xg = blockIdx.x % NX, jb = blockIdx.x / NX;
  const int v0 = static_cast<int>(static_cast<int64_t>(xg) * V / NX) + jb;
  const int v1 = static_cast<int>(static_cast<int64_t>(xg + 1) * V / NX);
  const int vs = (G - xg + NX - 1) / NX;
  const int ntile = v0 < v1 ? (v1 - v0 + vs - 1) / vs : 0;
  const int total = ntile * KS;
  if (total == 0) return;

  // tile cursor; the row blocks of a weight tile are consecutive.  A block visits
  // its tiles in increasing order, so the expert search resumes where the
  // previous tile's expert was (E + tiles steps over the whole launch).
  struct Cur { int v, e, mb, nb, cnt; };
  auto seek = [&](int v, int e) {
    Cur c;
    c.v = v;
    while (pre[e + 1] <= v) ++e;
    const int local = v - pre[e];
    c.e = e;
    c.cnt = cnts[e];
    const int nmb = (c.cnt + BM - 1) / BM;
    c.nb = local / nmb;
    c.mb = local - c.nb * nmb;
    return c;
  };
  // the next tile of this block; past its last tile the cursor is never used
  // for an address, and seek must not scan past pre[E]
  auto step = [&](Cur c) { return c.v + vs < V ? seek(c.v + vs, c.e) : c; };

  Cur lc = seek(v0, 0), cc = lc;
  int lk = 0;
  auto issue_stage = [&](int slot) {
    unsigned char* base = smem + slot * STAGE;
    // buffer loads into LDS: the expert's panels as buffer descriptors (raw, 32-bit
    // data format), byte offsets per lane; the record counts bound every load to its
    // panel (4-7% faster than the equivalent global loads into LDS)
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + static_cast<int64_t>(lc.e) * N * K), (short)0, N * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + static_cast<int64_t>(lc.e) * C * K), (short)0, static_cast<int>(C * K * 2), 0x00020000);
#pragma unroll
    for (int q = 0; q < WL; ++q) {
      const int p = (wave * WL + q) * 64 + lane;
      uint32_t off;
      if constexpr (BT) {  // 16-byte chunk p of the [BK][BN] tile: k row p / (BN / 8)
        const int kr = p / (BN / 8);
        const int c = (p % (BN / 8)) ^ (4 * (kr & 3));
        off = static_cast<uint32_t>(lk * BK + kr) * N + min(lc.nb * BN + c * 8, N - 8);
      } else {
        const int row = p / CPR;
        const int c = (p % CPR) ^ lds_swz_n<CPR>(row);
        int wr = min(lc.nb * BN + row, N - 1);
        if constexpr (GLU) wr = glu_row(wr, N >> 1);
        off = static_cast<uint32_t>(wr) * K + lk * BK + c * 8;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(base + (wave * WL + q) * 1024), 16,
                                               static_cast<int>(off * 2), 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < AL; ++q) {
      const int p = (wave * AL + q) * 64 + lane;
      const int row = p / CPR;
      const int c = (p % CPR) ^ lds_swz_n<CPR>(row);
      const uint32_t off = static_cast<uint32_t>(min(lc.mb * BM + row, lc.cnt - 1)) * K + lk * BK + c * 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(base + BN * RB + (wave * AL + q) * 1024), 16,
                                               static_cast<int>(off * 2), 0, 0, 0);
    }
  };
  // the loader cursor stops on the block's last stage: later issues re-read it
  auto advance = [&]() {
    if (++lk == KS) {
      lk = 0;
      lc = step(lc);
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  floatx16 acc[TN][TM];
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;
  };

#pragma unroll
  for (int x = 0; x < R - 1; ++x) {
    issue_stage(x);
    if (x + 1 < total) advance();
  }
  wait_vmcnt<(R - 2) * PER>();  // this wave's loads of stage 0
  barrier();
  if (grp == 1) barrier();  // group 1 runs one phase behind
  zero_acc();
  int kk = 0;
  for (int s = 0; s < total; ++s) {
    // memory phase
    const unsigned char* sw = smem + (s % R) * STAGE;
    const unsigned char* sa = sw + BN * RB;
    bf16x8 fa[NJ][TN], fb[NJ][TM];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = 2 * j + half;
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int row = (grp * TM + t) * 32 + fr;
        fb[j][t] = *reinterpret_cast<const bf16x8*>(sa + row * RB + 16 * (c ^ lds_swz_n<CPR>(row)));
      }
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        if constexpr (BT) {
          // lane 16 g + 4 q + c' reads k row 16 j + 8 (g / 2) + q (+ 4) at column
          // (wn TN + i) 32 + 16 (g % 2) + 4 c'; every lane ends with its own column
          // (row fr of the fragment) at k = 16 j + 8 half .. + 7
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
          const int trg = lane >> 4;
          const int kr = 16 * j + 8 * (trg >> 1) + ((lane & 15) >> 2);
          const int x = (wn * TN + i) * 32 + 16 * (trg & 1) + 4 * (lane & 3);
          const int cpos = (((x >> 3) ^ (4 * (kr & 3))) << 4) + (x & 7) * 2;  // same for kr + 4
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sw + kr * KRB + cpos));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sw + (kr + 4) * KRB + cpos));
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          fa[j][i] = __builtin_bit_cast(bf16x8, v);
        } else {
          const int row = (wn * TN + i) * 32 + fr;
          fa[j][i] = *reinterpret_cast<const bf16x8*>(sw + row * RB + 16 * (c ^ lds_swz_n<CPR>(row)));
        }
      }
    }
    issue_stage((s + R - 1) % R);
    if (s + R < total) advance();
    wait_vmcnt<(R - 2) * PER>();  // this wave's loads of stage s + 1
    barrier();
    // MFMA phase
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int t = 0; t < TM; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j][i], fb[j][t], acc[i][t], 0, 0, 0);
    if (++kk == KS) {
      kk = 0;
      // tile done: D[n][m], lane holds m = lane % 32 and four consecutive n per group
      const int m0 = cc.mb * BM, n0 = cc.nb * BN;
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int m = m0 + (grp * TM + t) * 32 + fr;
        if (GLU && m < cc.cnt) {
          // elements 4q + u (q = 0, 1): W half of unit 8q + 4h + u of the 32-row
          // tile's 16 units; elements 4q + 8 + u: the V half of the same unit
          bf16_t* orow = out + (static_cast<int64_t>(cc.e) * C + m) * (N >> 1);
#pragma unroll
          for (int i = 0; i < TN; ++i) {
            const int nt0 = n0 + (wn * TN + i) * 32;
            if (nt0 < N) {
#pragma unroll
              for (int q = 0; q < 2; ++q) {
                float h[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) h[u] = apply_act<ACT>(acc[i][t][4 * q + u]) * acc[i][t][4 * q + 8 + u];
                uint2 v;
                v.x = pack_bf16x2(h[0], h[1]);
                v.y = pack_bf16x2(h[2], h[3]);
                *reinterpret_cast<uint2*>(orow + (nt0 >> 1) + 8 * q + 4 * half) = v;
              }
            }
          }
        } else if (m < cc.cnt) {
          bf16_t* orow = out + (static_cast<int64_t>(cc.e) * C + m) * N;
#pragma unroll
          for (int i = 0; i < TN; ++i) {
            const int nt0 = n0 + (wn * TN + i) * 32;
            if (nt0 < N) {  // N % 32 == 0: a 32-column tile is wholly valid or not
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int n = nt0 + 8 * q + 4 * half;
                float h[4];
                if constexpr (EPI == 1) {  // acc * act'(z), z at the output position
                  const uint2 zz = *reinterpret_cast<const uint2*>(
                      aux + (static_cast<int64_t>(cc.e) * C + m) * N + n);
                  const float z[4] = {__uint_as_float(zz.x << 16), __uint_as_float(zz.x & 0xFFFF0000u),
                                      __uint_as_float(zz.y << 16), __uint_as_float(zz.y & 0xFFFF0000u)};
#pragma unroll
                  for (int u = 0; u < 4; ++u) h[u] = acc[i][t][4 * q + u] * act_grad<ACT>(z[u]);
                } else {
#pragma unroll
                  for (int u = 0; u < 4; ++u) h[u] = apply_act<ACT>(acc[i][t][4 * q + u]);
                }
                uint2 v;
                v.x = pack_bf16x2(h[0], h[1]);
                v.y = pack_bf16x2(h[2], h[3]);
                *reinterpret_cast<uint2*>(orow + n) = v;
              }
            }
          }
        }
      }
      cc = step(cc);
      zero_acc();
    }
    barrier();
  }
  if (grp == 0) barrier();
  wait_vmcnt<0>();  // the last stages' repeated loads land before the block's LDS is released
}

// ---------------------------------------------------------------------------
// Fused expert FFN for capacities <= 64, where one 64-row block holds every
// token of an expert: y_e = act(x_e . w1[e]^T) . w2[e]^T with the hidden
// activations kept on chip (the two-launch path writes and re-reads them, and
// those writes, mixed into the weight stream, cost HBM read efficiency).
//
// Work items are (expert e, column group j of y_e) for the non-empty experts,
// NO = 192 * NH columns per group, split evenly over persistent blocks of 8
// waves; the items of one expert are consecutive, so they run on one XCD and
// read w1[e] through one L2 (temporal loads), while each w2 row is read by one
// item only (non-temporal).  An item walks d_ff in chunks of 128:
//   * d_model / 64 up stages: 128 rows of w1 and the 64 activation rows, one
//     64-k slice each; wave w accumulates the 32 x 32 hidden tile
//     (f tile w % 4, row tile w / 4);
//   * the chunk's hidden tile, activated and rounded to bf16, is written to
//     LDS in the stage row layout (two 64-k slices of 64 rows);
//   * 2 * NH down stages: 192 rows of w2 (column group hg of the item) for one
//     64-k slice of the chunk; the four waves whose half matches hg % 2
//     accumulate 3 output tiles each of that group, in registers across chunks.
// Every stage is 192 rows of 128 bytes (three direct-to-LDS instructions per
// wave), so the ring keeps one load count per stage.  Each hidden and output
// element sees the same MFMA operands in the same k order as in the two-launch
// path, so the results are identical to it.
// ---------------------------------------------------------------------------
constexpr int kFusedRows = 192;  // rows per stage: 128 of w1 + 64 activations, or 192 of w2

template <int S>
__host__ __device__ constexpr int ffn_fused_lds_bytes() {
  return S * kFusedRows * 128 + 2 * 64 * 128 + (kMaxE + 1) * 4;
}

template <int ACT, int NH, int S>
__global__ __launch_bounds__(512) void ffn_fused_bf16_kernel(
    const bf16_t* __restrict__ A, const bf16_t* __restrict__ W1, const bf16_t* __restrict__ W2,
    bf16_t* __restrict__ out, const int32_t* __restrict__ count, int E, int64_t C, int d, int f,
    int nspl) {
  static_assert(NH % 2 == 0, "column groups alternate between the two wave halves");
  constexpr int STAGE = kFusedRows * 128;
  constexpr int PER = kFusedRows / 8 / 8;  // direct-to-LDS instructions per wave per stage
  static_assert((S - 2) * PER < 64, "memory counter range");
  constexpr int NO = NH * 192;             // y_e columns per item
  constexpr int YG = NH / 2;               // column groups per wave
  constexpr int KD = 2 * NH;               // down stages per chunk
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* hbuf = smem + S * STAGE;  // hidden tile: [2 slices][64 rows][128 bytes]
  int* pre = reinterpret_cast<int*>(hbuf + 2 * 64 * 128);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, fr = lane & 31;
  const int KU = d / 64;                   // up stages per chunk
  const int SPC = KU + KD;                 // stages per chunk
  const int NCH = f / kFusedFC;

  auto rows_of = [&](int e) {
    int64_t c = count[e];
    return static_cast<int>(c < 0 ? 0 : (c > C ? C : c));
  };
  if (wave == 0) {
    int run = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
      const int e = e0 + lane;
      const int t = (e < E && rows_of(e) > 0) ? nspl : 0;
      const int incl = wave_inclusive_scan(t, lane) + run;
      if (e < E) pre[e + 1] = incl;
      run = __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) pre[0] = 0;
  }
  __syncthreads();
  const int V = pre[E];
  const int G = gridDim.x;
  const int g = xcd_major_id(blockIdx.x, G);
  const int v0 = static_cast<int>(static_cast<int64_t>(g) * V / G);
  const int v1 = static_cast<int>(static_cast<int64_t>(g + 1) * V / G);
  const int total = (v1 - v0) * NCH * SPC;
  if (total == 0) return;

  struct Item { int v, e, j, cnt; };
  auto seek = [&](Item& it, int v) {
    it.v = v;
    int e = 0;
    while (pre[e + 1] <= v) ++e;
    it.e = e;
    it.j = v - pre[e];
    it.cnt = rows_of(e);
  };
  auto next = [&](Item& it) {
    ++it.v;
    if (++it.j == nspl) {
      it.j = 0;
      do { ++it.e; } while (it.e < E && pre[it.e + 1] <= it.v);
      if (it.e < E) it.cnt = rows_of(it.e);
    }
  };

  // loader: item li, chunk lfc, stage lp inside the chunk
  Item li;
  seek(li, v0);
  int lfc = 0, lp = 0;
  auto issue = [&](int slot) {
    unsigned char* base = smem + slot * STAGE;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int ii = wave * PER + q;           // 8 stage rows per instruction
      const int row = ii * 8 + (lane >> 3);
      const int c = (lane & 7) ^ lds_swz_n<8>(row);
      lds_void* dst = (lds_void*)(base + ii * 1024);
      if (lp < KU) {
        if (ii * 8 < kFusedFC) {
          const bf16_t* w = W1 + static_cast<int64_t>(li.e) * f * d;
          const uint32_t off = static_cast<uint32_t>(lfc * kFusedFC + row) * d + lp * 64 + c * 8;
          __builtin_amdgcn_global_load_lds(w + off, dst, 16, 0, 0);
        } else {
          const bf16_t* a = A + static_cast<int64_t>(li.e) * C * d;
          const uint32_t off = static_cast<uint32_t>(min(row - kFusedFC, li.cnt - 1)) * d + lp * 64 + c * 8;
          __builtin_amdgcn_global_load_lds(a + off, dst, 16, 0, 0);
        }
      } else {
        const int pd = lp - KU, kd = pd / NH, hg = pd - kd * NH;
        const bf16_t* w = W2 + static_cast<int64_t>(li.e) * d * f;
        const uint32_t off = static_cast<uint32_t>(li.j * NO + hg * 192 + row) * f +
                             (lfc * 2 + kd) * 64 + c * 8;
        __builtin_amdgcn_global_load_lds(w + off, dst, 16, 0, 2);
      }
    }
    if (++lp == SPC) {
      lp = 0;
      if (++lfc == NCH) {
        lfc = 0;
        next(li);
      }
    }
  };

  floatx16 hacc;
  floatx16 yacc[YG][3];
#pragma unroll
  for (int r = 0; r < 16; ++r) hacc[r] = 0.f;
#pragma unroll
  for (int u = 0; u < YG; ++u)
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) yacc[u][i][r] = 0.f;

  Item ci = li;
  int cfc = 0, cp = 0;
  const int uft = wave & 3, umt = wave >> 2;                // up: f tile, row tile
  const int dgrp = wave >> 2, dmt = (wave >> 1) & 1, dnt = (wave & 1) * 3;  // down
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < total) issue(i);
  for (int s = 0; s < total; ++s) {
    if (total - 1 - s >= S - 2) wait_vmcnt<(S - 2) * PER>();
    else wait_vmcnt<0>();
    ring_barrier();
    if (s + S - 1 < total) issue((s + S - 1) % S);
    const unsigned char* sb = smem + (s % S) * STAGE;
    if (cp < KU) {
      // up: hidden[f][m] += w1 rows . activation rows over this 64-k slice
      const int ra = uft * 32 + fr, rb = kFusedFC + umt * 32 + fr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 2 * j + half;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sb + ra * 128 + 16 * (c ^ lds_swz_n<8>(ra)));
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(sb + rb * 128 + 16 * (c ^ lds_swz_n<8>(rb)));
        hacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, hacc, 0, 0, 0);
      }
      if (cp == KU - 1) {
        // lane holds row m = umt*32 + fr and f = uft*32 + 8q + 4*half + r
        const int m = umt * 32 + fr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int fl = uft * 32 + 8 * q;
          const int c = (fl & 63) >> 3;
          uint2 v;
          v.x = pack_bf16x2(apply_act<ACT>(hacc[4 * q]), apply_act<ACT>(hacc[4 * q + 1]));
          v.y = pack_bf16x2(apply_act<ACT>(hacc[4 * q + 2]), apply_act<ACT>(hacc[4 * q + 3]));
          *reinterpret_cast<uint2*>(hbuf + (fl >> 6) * 8192 + m * 128 + 16 * (c ^ lds_swz_n<8>(m)) + 8 * half) = v;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) hacc[r] = 0.f;
      }
    } else {
      // down: y[n][m] += w2 rows (group hg) . hidden rows over slice kd of the chunk
      const int pd = cp - KU, kd = pd / NH, hg = pd - kd * NH;
      if ((hg & 1) == dgrp) {
        const unsigned char* hb = hbuf + kd * 8192;
        const int rb = dmt * 32 + fr;
#pragma unroll
        for (int u = 0; u < YG; ++u) {
          if (2 * u + dgrp != hg) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int c = 2 * j + half;
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(hb + rb * 128 + 16 * (c ^ lds_swz_n<8>(rb)));
#pragma unroll
            for (int i = 0; i < 3; ++i) {
              const int ra = (dnt + i) * 32 + fr;
              const bf16x8 a = *reinterpret_cast<const bf16x8*>(sb + ra * 128 + 16 * (c ^ lds_swz_n<8>(ra)));
              yacc[u][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, yacc[u][i], 0, 0, 0);
            }
          }
        }
      }
      if (cp == SPC - 1 && cfc == NCH - 1) {
        // item done: lane holds row m and four consecutive columns per group
        const int m = dmt * 32 + fr;
        if (m < ci.cnt) {
#pragma unroll
          for (int u = 0; u < YG; ++u)
#pragma unroll
            for (int i = 0; i < 3; ++i) {
              const int n0 = ci.j * NO + (2 * u + dgrp) * 192 + (dnt + i) * 32 + 4 * half;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int n = n0 + 8 * q;
                uint2 v;
                v.x = pack_bf16x2(yacc[u][i][4 * q], yacc[u][i][4 * q + 1]);
                v.y = pack_bf16x2(yacc[u][i][4 * q + 2], yacc[u][i][4 * q + 3]);
                *reinterpret_cast<uint2*>(out + (static_cast<int64_t>(ci.e) * C + m) * d + n) = v;
              }
            }
        }
#pragma unroll
        for (int u = 0; u < YG; ++u)
#pragma unroll
          for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) yacc[u][i][r] = 0.f;
      }
    }
    if (++cp == SPC) {
      cp = 0;
      if (++cfc == NCH) {
        cfc = 0;
        next(ci);
      }
    }
  }
}

// One 64-k stage of the float32 GEMM's two 64-row operand tiles, in registers.
struct F32Stage {
  float4 a[4], b[4];
};

template <bool GLU>
__device__ __forceinline__ F32Stage f32_stage_load(const float* Ae, const float* We, int K, int k0,
                                                   int tid, int rows, int n0, int N) {
  F32Stage st;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, r = q >> 4, c = (q & 15) * 4;
    st.a[i] = st.b[i] = float4{0.f, 0.f, 0.f, 0.f};
    if (r < rows) st.a[i] = *reinterpret_cast<const float4*>(Ae + static_cast<int64_t>(r) * K + k0 + c);
    const int wr = GLU ? glu_row(n0 + r, N >> 1) : n0 + r;
    if (n0 + r < N) st.b[i] = *reinterpret_cast<const float4*>(We + static_cast<int64_t>(wr) * K + k0 + c);
  }
  return st;
}

// float32 grouped GEMM: 64 x 64 tile, 4 x 4 outputs per thread, 64-k steps loaded
// with 16-byte vectors into registers one step ahead (the next step's loads are in
// flight during this step's FMAs: small layers are latency-bound, a step of 16 k
// with no prefetch paid a memory round trip each).
template <int ACT, bool GLU>
__global__ __launch_bounds__(256) void ffn_gemm_f32_kernel(const float* __restrict__ A,
                                                           const float* __restrict__ W,
                                                           float* __restrict__ out,
                                                           const int32_t* __restrict__ count,
                                                           int64_t C, int N, int K, int n_mt,
                                                           int n_nt) {
  constexpr int BK = 64, LDP = BK + 4;  // rows of 272 bytes: 16-byte aligned vector stores
  __shared__ __align__(16) float sA[64][LDP];
  __shared__ __align__(16) float sB[64][LDP];
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
  const float* We = W + static_cast<int64_t>(e) * N * K;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  // thread q = tid + 256 i loads row q / 16, k chunk 4 (q % 16) of each operand
  F32Stage st = f32_stage_load<GLU>(Ae, We, K, 0, tid, cnt - m0, n0, N);
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, r = q >> 4, c = (q & 15) * 4;
      *reinterpret_cast<float4*>(&sA[r][c]) = st.a[i];
      *reinterpret_cast<float4*>(&sB[r][c]) = st.b[i];
    }
    __syncthreads();
    if (k0 + BK < K) st = f32_stage_load<GLU>(Ae, We, K, k0 + BK, tid, cnt - m0, n0, N);
#pragma unroll 16
    for (int kk = 0; kk < BK; ++kk) {
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
      if constexpr (GLU) {
        // virtual columns n0 + tx + 16 j: j = 0, 2 the W half and j = 1, 3 the V
        // half of units n0 / 2 + tx and n0 / 2 + 16 + tx (N is a multiple of 64)
        float* orow = out + (static_cast<int64_t>(e) * C + m) * (N >> 1) + (n0 >> 1) + tx;
        if (n0 < N) {
          orow[0] = apply_act<ACT>(acc[i][0]) * acc[i][1];
          orow[16] = apply_act<ACT>(acc[i][2]) * acc[i][3];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + tx + 16 * j;
          if (n < N) out[(static_cast<int64_t>(e) * C + m) * N + n] = apply_act<ACT>(acc[i][j]);
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int ACT, bool GLU>
static hipError_t run_bf16(int E, const bf16_t* A, const bf16_t* W, bf16_t* out,
                           const int32_t* count, int64_t C, int N, int K, hipStream_t s) {
  auto kern = ffn_gemm_bf16_kernel<BM, BN, WM, WN, ACT, GLU>;
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

template <int TM, int TN, int WM, int WN, int S, int BK, bool NTW, int ACT, bool GLU, bool PAIR = false,
          bool TOK = false>
static hipError_t run_ring(int E, const bf16_t* A, const bf16_t* W, bf16_t* out,
                           const int32_t* count, int64_t C, int N, int K, hipStream_t s,
                           const int32_t* tok = nullptr) {
  auto kern = ffn_ring_bf16_kernel<TM, TN, WM, WN, S, BK, NTW, ACT, GLU, PAIR, TOK>;
  constexpr int lds = ffn_ring_lds_bytes<TM, TN, WM, WN, S, BK>();
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32 * (PAIR ? 2 : 1);
  if (PAIR && N % BN != 0) return hipErrorInvalidValue;
  const int64_t tiles = static_cast<int64_t>(E) * ((C + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(tiles, 256);  // one persistent block per CU
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(WM * WN * 64), lds, s, A, W,
                     out, count, E, C, N, K, tok);
  return hipGetLastError();
}

template <int ACT, bool GLU>
static hipError_t run_res(int E, const bf16_t* A, const bf16_t* W, bf16_t* out, const int32_t* count,
                          int64_t C, int N, int K, hipStream_t s, const int32_t* tok = nullptr) {
  auto kern = ffn_res_bf16_kernel<ACT, GLU>;
  const int lds = ffn_res_lds_bytes(K);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t tiles = static_cast<int64_t>(E) * ((N + 255) / 256);
  if (tiles == 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(tiles, 256);  // one persistent block per CU
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(512), lds, s, A, W, out, count, E, C,
                     N, K, tok);
  return hipGetLastError();
}

template <int TM, int TN, int R, int ACT, bool GLU, bool BT = false, int EPI = 0, int BK = 32>
static hipError_t run_pp(int E, const bf16_t* A, const bf16_t* W, bf16_t* out, const int32_t* count,
                         int64_t C, int N, int K, hipStream_t s, const bf16_t* aux = nullptr) {
  auto kern = ffn_pp_bf16_kernel<TM, TN, R, ACT, GLU, BT, EPI, BK>;
  constexpr int lds = ffn_pp_lds_bytes<TM, TN, R, BK>();
  constexpr int BM = 2 * TM * 32, BN = 4 * TN * 32;
  static_assert(lds <= 160 * 1024, "LDS budget");
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t tiles = static_cast<int64_t>(E) * ((C + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  const int64_t grid = std::min<int64_t>(tiles, 256);  // one persistent block per CU
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(512), lds, s, A, W, out, count, E,
                     C, N, K, aux);
  return hipGetLastError();
}

template <int ACT, int NH, int S>
static hipError_t run_fused(const Plan& p, int nspl, const bf16_t* A, const bf16_t* W1,
                            const bf16_t* W2, bf16_t* out, const int32_t* count, hipStream_t s) {
  auto kern = ffn_fused_bf16_kernel<ACT, NH, S>;
  constexpr int lds = ffn_fused_lds_bytes<S>();
  static_assert(lds <= 160 * 1024, "LDS budget");
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (err != hipSuccess) return err;
  const int64_t items = static_cast<int64_t>(p.E) * nspl;
  const int64_t grid = std::min<int64_t>(items, 256);  // one persistent block per CU
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(512), lds, s, A, W1, W2, out,
                     count, p.E, p.C, static_cast<int>(p.d), static_cast<int>(p.f), nspl);
  return hipGetLastError();
}

template <int ACT, bool GLU = false>
static hipError_t run_f32(int E, const float* A, const float* W, float* out, const int32_t* count,
                          int64_t C, int N, int K, hipStream_t s) {
  const int n_mt = static_cast<int>((C + 63) / 64);
  const int n_nt = (N + 63) / 64;
  const int64_t nblk = static_cast<int64_t>(E) * n_mt * n_nt;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL((ffn_gemm_f32_kernel<ACT, GLU>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s,
                     A, W, out, count, C, N, K, n_mt, n_nt);
  return hipGetLastError();
}

// Tile shapes by capacity.  Capacity <= 160: one row block holds every token of
// an expert, so the GEMM is bound by streaming the weights once: persistent
// direct-to-LDS ring kernel (8 or 4 waves, 256 weight rows per tile, 3-stage
// ring).  Capacity <= 64 with a contraction of at most 768 (the activation rows
// of an expert fit LDS): the kernel with resident activation rows and a
// weight-only ring, outputs through an LDS staging tile as whole rows (Switch-Base
// up-projection inside the forward: 114 us against 132 us for the ring's 40 KB
// stages, and the down-projection after it 115 against 129 us).  When
// 384-row weight tiles would cover N exactly with at most one tile
// per CU, 192-row tiles (two per CU, 4 waves, a 4-stage ring of 32 KB stages)
// balance the CUs and keep three stages of a cold weight stream in flight
// (Switch-Base down-projection inside the forward: 128-130 us, against 137 us
// for 384-row tiles with a 2-stage ring and 140 us for 256-row tiles), and a
// CU's two tiles run as a pair, their stages alternating at each k-chunk, so
// the second read of each activation chunk hits L2 (115.4 -> 109.5 us in the
// kernel traces of the same forward steps; 384-row tiles with 32-k stages of
// 28 KB instead: 12-15 us slower per step, 60 us with non-temporal weights).
// Other N at capacity <= 64: 256-row tiles (8 waves, 3-stage ring), paired the
// same way where N is a multiple of 512 (a Switch-like layer with d_model 1024,
// d_ff 4096: up / down 226.5 / 236.8 -> 211.1 / 230.2 us, step 505 -> 483 us),
// and likewise the 128 x 256 tiles at capacity <= 128 (E = 64, capacity 128,
// d_ff 4096: up-projection 123.7 -> 117.3 us).  Pairs are taken only where they
// still number at least 256: with half as many units as CUs, that layer's
// down-projection (128 units) took 174.6 us against 137.7 unpaired.
// Capacity > 160 (MFMA-bound: each weight tile is read by every row block of its
// expert, so those loads stay temporal).  With a contraction of at least 2048 the
// ping-pong kernel with 128 x 256 tiles and 64-k stages (3 slots of 48 KB).  The
// stream of a CU into LDS is bound by the L2 read requests it can keep in flight
// (rocprofv3: 80-90 on average in every grouped GEMM, at 400-450 cycles of L2
// latency here), so a stage that reads whole 128-byte rows moves twice the bytes
// per request of the 32-k stages' 64-byte pieces: against 128 x 512 tiles with
// 32-k stages (large Zipf layer, capacity 320) up / down 2.91 / 2.80 ms instead of
// 3.08 / 3.09 ms, against 256 x 256 with 32-k stages (X-MoE top-2
// down-projection, N = 1024, K = 4096) 327 instead of 356 us, same output bits.
// 128-row blocks also waste at most 127 rows of a partly filled last row block
// (X-MoE pads its 32 768 served rows by 26% in 256-row blocks).
// Shorter contractions, where a tile's epilogue is a larger share of its time:
// the ring with 256 x 256 tiles, 8 waves of 4 x 2 MFMA tiles and a 2-stage ring
// of 64 KB stages (X-MoE up-projection, K = 1024: 410 us against 443 us for
// ping-pong).  The
// ring kernels address inside one expert with 32-bit offsets; larger experts
// take the LDS-tiled one.  N is the number of weight rows (2 d_ff for the GLU
// up-projection).
// The resident-activation kernel's shape conditions (N x K and C x K element
// offsets in 32 bits, one 64-row block per expert, the rows of K fit in LDS).
static bool res_ok(const Plan& p, int64_t N, int64_t K) {
  const int64_t lim = int64_t(1) << 32;
  return N * K < lim && p.C * K < lim && p.C <= 64 && K <= kResMaxK && p.E <= kMaxE;
}

// The up-projection of gemm_bf16 on the two-slot 256 x 256 ring (capacity > 160,
// contraction below the ping-pong kernel's 2048, 32-bit panel offsets).
static bool ring2_up(const Plan& p) {
  const int64_t lim = int64_t(1) << 32, N = p.w1_rows(), K = p.d;
  return N * K < lim && p.C * K < lim && p.C > 160 && K < 2048;
}

bool up_reads_token_rows(const Plan& p) {
  return p.dtype == 1 && p.C > 0 && p.T > 0 && (res_ok(p, p.w1_rows(), p.d) || ring2_up(p));
}

template <int ACT, bool GLU = false>
static hipError_t gemm_bf16(const Plan& p, const bf16_t* A, const bf16_t* W, bf16_t* out,
                            const int32_t* count, int N, int K, hipStream_t s) {
  const int64_t lim = int64_t(1) << 32;
  if (int64_t(N) * K >= lim || p.C * K >= lim)
    return run_bf16<128, 128, 2, 2, ACT, GLU>(p.E, A, W, out, count, p.C, N, K, s);
  const bool pp_ok = int64_t(N) * K * 2 < (int64_t(1) << 31) && p.C * K * 2 < (int64_t(1) << 31);
  if (pp_ok && p.C > 160 && K >= 2048)
    return run_pp<2, 2, 3, ACT, GLU, false, 0, 64>(p.E, A, W, out, count, p.C, N, K, s);
  if (p.C > 160) return run_ring<4, 2, 2, 4, 2, 64, false, ACT, GLU>(p.E, A, W, out, count, p.C, N, K, s);
  if (res_ok(p, N, K)) return run_res<ACT, GLU>(p.E, A, W, out, count, p.C, N, K, s);
  // pairing a block's two column tiles halves the work units: only where the pairs
  // still cover the 256 CUs
  auto pairs = [&](int bm, int bn) {
    return N % (2 * bn) == 0 && static_cast<int64_t>(p.E) * ((p.C + bm - 1) / bm) * (N / (2 * bn)) >= 256;
  };
  if (p.C <= 64 && N % 384 == 0 && static_cast<int64_t>(p.E) * (N / 384) <= 256) {
    if (pairs(64, 192))
      return run_ring<1, 3, 2, 2, 4, 64, true, ACT, GLU, true>(p.E, A, W, out, count, p.C, N, K, s);
    return run_ring<1, 3, 2, 2, 4, 64, true, ACT, GLU>(p.E, A, W, out, count, p.C, N, K, s);
  }
  if (p.C <= 64 && pairs(64, 256))
    return run_ring<2, 1, 1, 8, 3, 64, true, ACT, GLU, true>(p.E, A, W, out, count, p.C, N, K, s);
  if (p.C <= 64) return run_ring<2, 1, 1, 8, 3, 64, true, ACT, GLU>(p.E, A, W, out, count, p.C, N, K, s);
  if (p.C <= 128 && pairs(128, 256))
    return run_ring<4, 1, 1, 8, 3, 64, true, ACT, GLU, true>(p.E, A, W, out, count, p.C, N, K, s);
  if (p.C <= 128) return run_ring<4, 1, 1, 8, 3, 64, true, ACT, GLU>(p.E, A, W, out, count, p.C, N, K, s);
  return run_ring<5, 2, 1, 4, 3, 64, true, ACT, GLU>(p.E, A, W, out, count, p.C, N, K, s);
}

hipError_t launch_expert_ffn_fused(const Plan& p, int nspl, const void* x_e,
                                   const int32_t* expert_count, const void* w1, const void* w2,
                                   void* y_e, hipStream_t s) {
  if (p.C == 0) return hipSuccess;
  const bf16_t* a = static_cast<const bf16_t*>(x_e);
  const bf16_t* u = static_cast<const bf16_t*>(w1);
  const bf16_t* v = static_cast<const bf16_t*>(w2);
  bf16_t* o = static_cast<bf16_t*>(y_e);
  if (p.d != static_cast<int64_t>(nspl) * 384) return hipErrorInvalidValue;
  return p.act == 0 ? run_fused<0, 2, 5>(p, nspl, a, u, v, o, expert_count, s)
                    : run_fused<1, 2, 5>(p, nspl, a, u, v, o, expert_count, s);
}

hipError_t launch_expert_up(const Plan& p, const void* x_e, const int32_t* expert_count,
                            const void* w1, void* hidden, hipStream_t s) {
  if (p.C == 0) return hipSuccess;
  const int d = static_cast<int>(p.d), f = static_cast<int>(p.f);
  if (p.dtype == 1) {
    const bf16_t* xe = static_cast<const bf16_t*>(x_e);
    const bf16_t* w = static_cast<const bf16_t*>(w1);
    bf16_t* h = static_cast<bf16_t*>(hidden);
    if (p.glu)
      return p.act == 0 ? gemm_bf16<0, true>(p, xe, w, h, expert_count, 2 * f, d, s)
                        : gemm_bf16<1, true>(p, xe, w, h, expert_count, 2 * f, d, s);
    return p.act == 0 ? gemm_bf16<0>(p, xe, w, h, expert_count, f, d, s)
                      : gemm_bf16<1>(p, xe, w, h, expert_count, f, d, s);
  }
  const float* xe = static_cast<const float*>(x_e);
  const float* w = static_cast<const float*>(w1);
  float* h = static_cast<float*>(hidden);
  if (p.glu)
    return p.act == 0 ? run_f32<0, true>(p.E, xe, w, h, expert_count, p.C, 2 * f, d, s)
                      : run_f32<1, true>(p.E, xe, w, h, expert_count, p.C, 2 * f, d, s);
  return p.act == 0 ? run_f32<0>(p.E, xe, w, h, expert_count, p.C, f, d, s)
                    : run_f32<1>(p.E, xe, w, h, expert_count, p.C, f, d, s);
}

hipError_t launch_expert_up_act(const Plan& p, const void* x_e, const int32_t* expert_count,
                                const void* w1, void* out, int act, hipStream_t s) {
  Plan q = p;
  q.act = act;
  if (act == 2) {  // no activation
    if (p.C == 0) return hipSuccess;
    const int d = static_cast<int>(p.d), f = static_cast<int>(p.f);
    if (p.dtype == 1)
      return gemm_bf16<2>(q, static_cast<const bf16_t*>(x_e), static_cast<const bf16_t*>(w1),
                          static_cast<bf16_t*>(out), expert_count, f, d, s);
    return run_f32<2>(p.E, static_cast<const float*>(x_e), static_cast<const float*>(w1),
                      static_cast<float*>(out), expert_count, p.C, f, d, s);
  }
  return launch_expert_up(q, x_e, expert_count, w1, out, s);
}

// The backward's token-row products on the ping-pong kernel (second operand
// stored [K][N]): contractions of at least 1024, 128 x 512 tiles where N >= 2048
// and the capacity exceeds 64 (RRE 4x16 backward, capacity 160: 5.96 -> 5.54 ms),
// 256 x 256 tiles where the capacity exceeds 160 (X-MoE top-2: 3.12 -> 2.92 ms,
// large Zipf layer 24.2 -> 22.7 ms, against the LDS-tiled backward GEMM);
// hipErrorNotSupported elsewhere (the caller falls back to that kernel).
hipError_t launch_bwd_rows_pp(const Plan& p, const bf16_t* A, const bf16_t* B, bf16_t* out,
                              const bf16_t* aux, const int32_t* count, int N, int K, int grad_act,
                              hipStream_t s) {
  const int64_t lim = int64_t(1) << 31;  // byte offsets inside an expert's panels (buffer loads)
  const bool wide = N >= 2048;
  if (p.dtype != 1 || K < 1024 || p.C <= (wide ? 64 : 160) || int64_t(N) * K * 2 >= lim ||
      p.C * K * 2 >= lim)
    return hipErrorNotSupported;
  if (grad_act < 0)
    return wide ? run_pp<2, 4, 3, 2, false, true, 0>(p.E, A, B, out, count, p.C, N, K, s)
                : run_pp<4, 2, 4, 2, false, true, 0>(p.E, A, B, out, count, p.C, N, K, s);
  if (grad_act == 0)
    return wide ? run_pp<2, 4, 3, 0, false, true, 1>(p.E, A, B, out, count, p.C, N, K, s, aux)
                : run_pp<4, 2, 4, 0, false, true, 1>(p.E, A, B, out, count, p.C, N, K, s, aux);
  return wide ? run_pp<2, 4, 3, 1, false, true, 1>(p.E, A, B, out, count, p.C, N, K, s, aux)
              : run_pp<4, 2, 4, 1, false, true, 1>(p.E, A, B, out, count, p.C, N, K, s, aux);
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

hipError_t launch_expert_ffn_rows(const Plan& p, const void* x, const int32_t* slot_token,
                                  const int32_t* expert_count, const void* w1, const void* w2,
                                  void* y_e, void* ws, hipStream_t s) {
  if (!up_reads_token_rows(p)) return hipErrorInvalidValue;
  void* hidden = ws_at(ws, p.off_region[6]);
  const bf16_t* xr = static_cast<const bf16_t*>(x);
  const bf16_t* w = static_cast<const bf16_t*>(w1);
  bf16_t* h = static_cast<bf16_t*>(hidden);
  const int d = static_cast<int>(p.d), f = static_cast<int>(p.f);
  hipError_t err;
  if (ring2_up(p)) {
    // the ring kernel of gemm_bf16 for this shape, its activation rows read from x
    if (p.glu)
      err = p.act == 0
                ? run_ring<4, 2, 2, 4, 2, 64, false, 0, true, false, true>(p.E, xr, w, h, expert_count, p.C,
                                                                         2 * f, d, s, slot_token)
                : run_ring<4, 2, 2, 4, 2, 64, false, 1, true, false, true>(p.E, xr, w, h, expert_count, p.C,
                                                                         2 * f, d, s, slot_token);
    else
      err = p.act == 0
                ? run_ring<4, 2, 2, 4, 2, 64, false, 0, false, false, true>(p.E, xr, w, h, expert_count, p.C,
                                                                          f, d, s, slot_token)
                : run_ring<4, 2, 2, 4, 2, 64, false, 1, false, false, true>(p.E, xr, w, h, expert_count, p.C,
                                                                          f, d, s, slot_token);
  } else if (p.glu) {
    err = p.act == 0 ? run_res<0, true>(p.E, xr, w, h, expert_count, p.C, 2 * f, d, s, slot_token)
                     : run_res<1, true>(p.E, xr, w, h, expert_count, p.C, 2 * f, d, s, slot_token);
  } else {
    err = p.act == 0 ? run_res<0, false>(p.E, xr, w, h, expert_count, p.C, f, d, s, slot_token)
                     : run_res<1, false>(p.E, xr, w, h, expert_count, p.C, f, d, s, slot_token);
  }
  if (err != hipSuccess) return err;
  return launch_expert_down(p, hidden, expert_count, w2, y_e, s);
}

hipError_t launch_expert_ffn(const Plan& p, const void* x_e, const int32_t* expert_count,
                             const void* w1, const void* w2, void* y_e, void* ws, hipStream_t s) {
  void* hidden = ws_at(ws, p.off_region[6]);
  const hipError_t err = launch_expert_up(p, x_e, expert_count, w1, hidden, s);
  if (err != hipSuccess) return err;
  return launch_expert_down(p, hidden, expert_count, w2, y_e, s);
}

}  // namespace moe
