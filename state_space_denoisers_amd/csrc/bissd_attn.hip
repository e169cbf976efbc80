// bissd_attn.hip -- multi-head softmax attention of the hybrid backbones
// (gfx950): O = softmax(scale Q K^T + M) V per (batch row, head), head dim 64.
//
// The hybrids put attention between the bidirectional Mamba-2 blocks: full
// bidirectional attention ("DiffMamba Checkpoints" model card, Hybrid
// Mamba+attention checkpoints; "DiffuMamba: High-Throughput Diffusion LMs
// with Mamba Backbone", Core Architecture: one multi-head attention block
// every five Mamba blocks), or block-wise attention in block diffusion, where
// a block sees the prefix before it and itself ("Training Hybrid Block
// Diffusion Language Models with Partial Bidirectionality", Methodology, the
// BDLM attention baseline).  M is 0 where a query may see a key and -inf
// elsewhere.
//
// One pass over the keys with a running softmax: each workgroup takes 128
// queries of one (batch, head) and streams 64-key tiles of K and V through
// LDS (copied buffer -> LDS, the next tile in flight while the current one
// is used).  Per tile, each wave forms its 32 queries' scores as S^T = K Q^T
// on the matrix cores, so that a lane holds one query's scores for 16 keys
// in exactly the layout of the A operand of the following P V product; the
// row maximum takes two lane exchanges; the row sums come from the matrix
// cores (P times a column of ones).  Every exponential is one
// exp2 of fma(s, c, -m c) with c = scale * log2(e).  The running maximum m
// of a query only moves when a tile's maximum exceeds it by more than
// kAttnSlack / c (then the output rows are rescaled by exp2((m_old - m_new) c)),
// so after the first tiles a wave usually skips the rescale altogether;
// meanwhile the probabilities stay below 2^kAttnSlack, well inside bf16 and
// the fp32 sums.
#include <math.h>

#include "bissd_device.hpp"
#include "bissd_internal.hpp"

namespace bissd {

constexpr float kAttnSlack = 8.0f;  // log2 units the running maximum may lag
constexpr int kAttnQ = 128;         // queries per workgroup

template <typename T> struct AttnTiles {
  static constexpr int RB = kAttnD * (int)sizeof(T);  // bytes of one head's token row
  using DK = DmaTile<RB, SW_NAT>;  // keys: read as natural rows
  using DV = DmaTile<RB, SW_TR>;   // values: read along the key index
};

// Workgroup = (batch b, head h, 128-query tile); wave w owns queries
// q0 + 32 w + 16 j + (0..15) for j = 0, 1, so every key and value fragment
// read from LDS feeds two products.  Queries past L compute on zeros and are
// not stored; keys past a query group's visible end are masked to -inf.
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 1)))
void k_attn_fwd(AttnArgs a) {
  using DK = typename AttnTiles<T>::DK;
  using DV = typename AttnTiles<T>::DV;
  constexpr int RB = AttnTiles<T>::RB;
  constexpr uint32_t ES = sizeof(T);
  __shared__ __attribute__((aligned(16))) char tK[2][kRB * RB];
  __shared__ __attribute__((aligned(16))) char tV[2][kRB * RB];
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int H = a.H;
  const int64_t L = a.L;
  const int nqt = (int)((L + kAttnQ - 1) / kAttnQ);
  // work item = (b * H + h) * nqt + query tile: the query tiles of one head,
  // which read the same keys and values, run on one XCD
  int bx = xcd_linear_id(blockIdx.x, gridDim.x);
  const int qt = bx % nqt;
  bx /= nqt;
  const int h = bx % H, b = bx / H;
  const int64_t q0 = (int64_t)qt * kAttnQ;
  // visible keys [0, kend_j) of query group j: all, or up to the end of its
  // block (blocks are whole 64-token tiles, so a 16-query group lies in one)
  int64_t kend[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t g0 = q0 + 32 * w + 16 * j;
    kend[j] = a.block > 0 ? min(L, (g0 / a.block + 1) * a.block) : L;
  }
  const int64_t qlast = min(L, q0 + kAttnQ) - 1;
  const int64_t kmax = a.block > 0 ? min(L, (qlast / a.block + 1) * a.block) : L;
  const int nkt = (int)((kmax + kRB - 1) / kRB);
  const uint32_t rs = (uint32_t)H * kAttnD * ES;  // token stride in bytes
  const uint32_t nbytes = (uint32_t)(L * H * kAttnD * ES);
  const int64_t boff = (int64_t)b * L * H * kAttnD;
  const bufres rQ = make_buf(reinterpret_cast<const T *>(a.q) + boff, nbytes);
  const bufres rK = make_buf(reinterpret_cast<const T *>(a.k) + boff, nbytes);
  const bufres rV = make_buf(reinterpret_cast<const T *>(a.v) + boff, nbytes);
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)(((int64_t)kt * kRB * H + h) * kAttnD) * ES;
    DK::load(tK[buf], rK, off, rs, kRB);
    DV::load(tV[buf], rV, off, rs, kRB);
  };

  // this lane's two queries (B operands of S^T = K Q^T), held for the pass
  Frag<T> qf[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t qrow = q0 + 32 * w + 16 * j + r16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      frag_bload(qf[j][ks], rQ, (uint32_t)((qrow * H + h) * kAttnD) * ES + (uint32_t)(32 * ks + 8 * g4) * ES);
  }
  issue(0, 0);

  // o[j][v]: output rows 4 g4 + i of group j, columns 16 v + r16; osum[j]:
  // the same rows' probability sums, formed on the matrix cores as P times a
  // column of ones (so they sit in the output rows' layout and are rescaled
  // with them)
  f32x4 o[2][4], osum[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    zero4(osum[j]);
#pragma unroll
    for (int v = 0; v < 4; ++v) zero4(o[j][v]);
  }
  Frag<T> ones;
  {
    float one8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) one8[e] = 1.0f;
    frag_from(ones, one8);
  }
  const float c = a.scale_log2;
  const float slack = kAttnSlack / c;
  // running reference of query r16 of each group (raw score units)
  float mrow[2] = {-INFINITY, -INFINITY};

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    wait_vmem();
    __syncthreads();  // tile kt is in LDS; every wave is done with tile kt - 1
    if (kt + 1 < nkt) issue(kt + 1, cur ^ 1);
    // s[j][u][i]: score of query r16 of group j against key k0 + 16 u + 4 g4 + i
    f32x4 s[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      zero4(s[0][u]);
      zero4(s[1][u]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag<T> kf;
        frag_ld8_swz<DK>(kf, tK[cur], 16 * u + r16, 32 * ks + 8 * g4);
        mma(s[0][u], kf, qf[0][ks]);
        mma(s[1][u], kf, qf[1][ks]);
      }
    }
    const int64_t k0 = (int64_t)kt * kRB;
    bool move[2];
    float alpha[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (k0 + kRB > kend[j]) {
        // keys past the group's visible end score -inf
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + 16 * u + 4 * g4 + i >= kend[j]) s[j][u][i] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[j][u][i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      // a tile wholly past the group's end has tmax = -inf and moves nothing;
      // the first tile always has a visible key for every group
      move[j] = tmax > mrow[j] + slack;
      const float mnew = move[j] ? tmax : mrow[j];
      alpha[j] = move[j] ? exp2_fast((mrow[j] - mnew) * c) : 1.0f;
      const float nm = -mnew * c;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[j][u][i] = exp2_fast(fmaf(s[j][u][i], c, nm));
      mrow[j] = mnew;
    }
    // output rows 4 g4 + i belong to query 4 g4 + i, whose factor lane
    // 4 g4 + i holds; skipped when no query of the wave moved
    if (__any(move[0] || move[1])) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha[j], 4 * g4 + i, 64);
          osum[j][i] *= ai;
#pragma unroll
          for (int v = 0; v < 4; ++v) o[j][v][i] *= ai;
        }
    }
    // O += P V: P (query r16, keys 32 q + 4 g4 + i and 32 q + 16 + 4 g4 + i)
    // as the A operand, V read along the key index
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      Frag<T> pf[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float m[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          m[i] = s[j][2 * q][i];
          m[4 + i] = s[j][2 * q + 1][i];
        }
        frag_from(pf[j], m);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        Frag<T> vf;
        frag_rows_swz<DV>(vf, tV[cur], 32 * q + 4 * g4, 32 * q + 16 + 4 * g4, 16 * v);
        mma(o[0][v], pf[0], vf);
        mma(o[1][v], pf[1], vf);
      }
      mma(osum[0], pf[0], ones);
      mma(osum[1], pf[1], ones);
    }
  }

  // normalise and store rows q0 + 32 w + 16 j + 4 g4 + i (16 lanes write one
  // contiguous row segment); the lanes of column 0 also write each row's
  // log2-sum-exp of its scaled scores, from which the backward pass rebuilds
  // P = exp2(c s - lse)
  T *og = reinterpret_cast<T *>(a.o) + boff;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv = 1.0f / osum[j][i];
      const float mi = __shfl(mrow[j], 4 * g4 + i, 64);
      const int64_t t = q0 + 32 * w + 16 * j + 4 * g4 + i;
      if (t >= L) continue;
      if (a.lse && r16 == 0) a.lse[((int64_t)b * H + h) * L + t] = mi * c + __builtin_amdgcn_logf(osum[j][i]);
#pragma unroll
      for (int v = 0; v < 4; ++v) og[(t * H + h) * kAttnD + 16 * v + r16] = from_f<T>(o[j][v][i] * inv);
    }
}

// ============================================================== backward
//
// Reverse mode of O = softmax(S) V, S = scale Q K^T + M, for an incoming
// gradient dO (plain matrix calculus):
//   P = exp2(c S_raw - lse),  dV = P^T dO,  dP = dO V^T,
//   dS = P * (dP - D),  D_t = sum_d dO[t][d] O[t][d],
//   dQ = scale dS K,  dK = scale dS^T Q.
// P is rebuilt from the forward's per-query log2-sum-exp (lse).  Two
// launches keep every sum in a fixed order (no atomics): k_attn_dq runs
// over query tiles (dQ, and D as a by-product), then k_attn_dkv over key
// tiles (dK, dV), each recomputing the scores.  As in the forward, every
// product is laid out so that its accumulator is the A operand of the next
// one: per query in k_attn_dq (S^T = K Q^T, dP^T = V dO^T), per key in
// k_attn_dkv (S = Q K^T, dP = dO V^T).

// Workgroup = (batch b, head h, 128-query tile); wave w owns queries
// q0 + 32 w + 16 j + (0..15), j = 0, 1, so every K and V fragment read from
// LDS feeds two products.  K is staged twice (natural rows for the scores,
// along the key index for dQ), V once.
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 1)))
void k_attn_dq(AttnArgs a) {
  using DN = typename AttnTiles<T>::DK;
  using DTR = typename AttnTiles<T>::DV;
  constexpr int RB = AttnTiles<T>::RB;
  constexpr uint32_t ES = sizeof(T);
  __shared__ __attribute__((aligned(16))) char tKn[2][kRB * RB];
  __shared__ __attribute__((aligned(16))) char tKt[2][kRB * RB];
  __shared__ __attribute__((aligned(16))) char tVn[2][kRB * RB];
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int H = a.H;
  const int64_t L = a.L;
  const int nqt = (int)((L + kAttnQ - 1) / kAttnQ);
  int bx = xcd_linear_id(blockIdx.x, gridDim.x);
  const int qt = bx % nqt;
  bx /= nqt;
  const int h = bx % H, b = bx / H;
  const int64_t q0 = (int64_t)qt * kAttnQ;
  int64_t kend[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t g0 = q0 + 32 * w + 16 * j;
    kend[j] = a.block > 0 ? min(L, (g0 / a.block + 1) * a.block) : L;
  }
  const int64_t qlast = min(L, q0 + kAttnQ) - 1;
  const int64_t kmax = a.block > 0 ? min(L, (qlast / a.block + 1) * a.block) : L;
  const int nkt = (int)((kmax + kRB - 1) / kRB);
  const uint32_t rs = (uint32_t)H * kAttnD * ES;
  const uint32_t nbytes = (uint32_t)(L * H * kAttnD * ES);
  const int64_t boff = (int64_t)b * L * H * kAttnD;
  const bufres rQ = make_buf(reinterpret_cast<const T *>(a.q) + boff, nbytes);
  const bufres rK = make_buf(reinterpret_cast<const T *>(a.k) + boff, nbytes);
  const bufres rV = make_buf(reinterpret_cast<const T *>(a.v) + boff, nbytes);
  const bufres rO = make_buf(reinterpret_cast<const T *>(a.o) + boff, nbytes);
  const bufres rG = make_buf(reinterpret_cast<const T *>(a.dout) + boff, nbytes);
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)(((int64_t)kt * kRB * H + h) * kAttnD) * ES;
    DN::load(tKn[buf], rK, off, rs, kRB);
    DTR::load(tKt[buf], rK, off, rs, kRB);
    DN::load(tVn[buf], rV, off, rs, kRB);
  };
  // this lane's two queries: Q and dO fragments (B operands), and
  // D_t = dO_t . O_t (this lane's 16 head-dim entries, then the 4 lanes of
  // the query), written for the dK / dV pass
  const int64_t vrow = ((int64_t)b * H + h) * L;
  Frag<T> qf[2][2], gf[2][2];
  float lse[2], dsum[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t t = q0 + 32 * w + 16 * j + r16;
    const uint32_t roff = (uint32_t)((t * H + h) * kAttnD) * ES;
    float ds = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t off = roff + (uint32_t)(32 * ks + 8 * g4) * ES;
      Frag<T> of;
      frag_bload(qf[j][ks], rQ, off);
      frag_bload(gf[j][ks], rG, off);
      frag_bload(of, rO, off);
#pragma unroll
      for (int e = 0; e < 8; ++e) ds += to_f(gf[j][ks].v[e]) * to_f(of.v[e]);
    }
    ds += __shfl_xor(ds, 16, 64);
    ds += __shfl_xor(ds, 32, 64);
    dsum[j] = ds;
    lse[j] = t < L ? a.lse[vrow + t] : INFINITY;
    if (g4 == 0 && t < L) a.delta[vrow + t] = ds;
  }
  issue(0, 0);
  const float c = a.scale_log2;

  f32x4 dq[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) zero4(dq[j][v]);
  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    wait_vmem();
    __syncthreads();
    if (kt + 1 < nkt) issue(kt + 1, cur ^ 1);
    // s[j][u][i], dp[j][u][i]: query r16 of group j against key k0 + 16 u + 4 g4 + i
    f32x4 s[2][4], dp[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        zero4(s[j][u]);
        zero4(dp[j][u]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag<T> kf, vf;
        frag_ld8_swz<DN>(kf, tKn[cur], 16 * u + r16, 32 * ks + 8 * g4);
        frag_ld8_swz<DN>(vf, tVn[cur], 16 * u + r16, 32 * ks + 8 * g4);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          mma(s[j][u], kf, qf[j][ks]);
          mma(dp[j][u], vf, gf[j][ks]);
        }
      }
    }
    const int64_t k0 = (int64_t)kt * kRB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool ragged = k0 + kRB > kend[j];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float p = exp2_fast(fmaf(s[j][u][i], c, -lse[j]));
          if (ragged && k0 + 16 * u + 4 * g4 + i >= kend[j]) p = 0.0f;
          s[j][u][i] = p * (dp[j][u][i] - dsum[j]);  // dS
        }
    }
    // dQ += dS K
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      Frag<T> df[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float m[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          m[i] = s[j][2 * q][i];
          m[4 + i] = s[j][2 * q + 1][i];
        }
        frag_from(df[j], m);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        Frag<T> kt2;
        frag_rows_swz<DTR>(kt2, tKt[cur], 32 * q + 4 * g4, 32 * q + 16 + 4 * g4, 16 * v);
        mma(dq[0][v], df[0], kt2);
        mma(dq[1][v], df[1], kt2);
      }
    }
  }
  const float sc = a.scale;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tt = q0 + 32 * w + 16 * j + 4 * g4 + i;
      if (tt >= L) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) a.dq[boff + (tt * H + h) * kAttnD + 16 * v + r16] = sc * dq[j][v][i];
    }
}

// Workgroup = (batch b, head h, 128-key tile); wave w owns keys
// k0 + 32 w + 16 j + (0..15), j = 0, 1, so every Q and dO fragment read from
// LDS feeds two products.  Query tiles run from the first key group's block
// on (every later query sees the keys of its block and before); a key group
// whose block starts later skips the tiles before it.  Q and dO are staged
// twice (natural rows for the scores, along the query index for dK and dV),
// lse and D once.
template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1)))
void k_attn_dkv(AttnArgs a) {
  using DN = typename AttnTiles<T>::DK;
  using DTR = typename AttnTiles<T>::DV;
  constexpr int RB = AttnTiles<T>::RB;
  constexpr uint32_t ES = sizeof(T);
  __shared__ __attribute__((aligned(16))) char tQn[2][kRB * RB];
  __shared__ __attribute__((aligned(16))) char tQt[2][kRB * RB];
  __shared__ __attribute__((aligned(16))) char tGn[2][kRB * RB];
  __shared__ __attribute__((aligned(16))) char tGt[2][kRB * RB];
  __shared__ __attribute__((aligned(16))) float tL[2][kRB];  // lse (+inf past L)
  __shared__ __attribute__((aligned(16))) float tD[2][kRB];  // D
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int H = a.H;
  const int64_t L = a.L;
  const int nkt = (int)((L + kAttnQ - 1) / kAttnQ);
  int bx = xcd_linear_id(blockIdx.x, gridDim.x);
  const int kt = bx % nkt;
  bx /= nkt;
  const int h = bx % H, b = bx / H;
  const int64_t k0 = (int64_t)kt * kAttnQ;
  // first query tile each key group needs (its block's start; 0 when full)
  int qbeg[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t g0 = k0 + 32 * w + 16 * j;
    qbeg[j] = a.block > 0 ? (int)((g0 / a.block) * a.block / kRB) : 0;
  }
  const int qt0 = a.block > 0 ? (int)((k0 / a.block) * a.block / kRB) : 0;
  const int nqt = (int)((L + kRB - 1) / kRB);
  const uint32_t rs = (uint32_t)H * kAttnD * ES;
  const uint32_t nbytes = (uint32_t)(L * H * kAttnD * ES);
  const int64_t boff = (int64_t)b * L * H * kAttnD;
  const bufres rQ = make_buf(reinterpret_cast<const T *>(a.q) + boff, nbytes);
  const bufres rK = make_buf(reinterpret_cast<const T *>(a.k) + boff, nbytes);
  const bufres rV = make_buf(reinterpret_cast<const T *>(a.v) + boff, nbytes);
  const bufres rG = make_buf(reinterpret_cast<const T *>(a.dout) + boff, nbytes);
  const int64_t vrow = ((int64_t)b * H + h) * L;
  const bufres rL = make_buf(a.lse + vrow, (uint32_t)(L * 4));
  const bufres rD = make_buf(a.delta + vrow, (uint32_t)(L * 4));
  auto issue = [&](int qt, int buf) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)(((int64_t)qt * kRB * H + h) * kAttnD) * ES;
    DN::load(tQn[buf], rQ, off, rs, kRB);
    DTR::load(tQt[buf], rQ, off, rs, kRB);
    DN::load(tGn[buf], rG, off, rs, kRB);
    DTR::load(tGt[buf], rG, off, rs, kRB);
  };
  // per-query lse and D of a query tile, one value per thread of wave 0
  auto vec_ld = [&](int qt, float &l, float &d) __attribute__((always_inline)) {
    const uint32_t q = (uint32_t)(qt * kRB + lane);
    l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rL, q * 4u, 0, 0));
    d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rD, q * 4u, 0, 0));
    if ((int64_t)q >= L) l = INFINITY;  // queries past L contribute nothing
  };
  // this lane's two keys: K and V fragments (B operands of S = Q K^T, dP = dO V^T)
  Frag<T> kf[2][2], vf[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t s = k0 + 32 * w + 16 * j + r16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t off = (uint32_t)((s * H + h) * kAttnD) * ES + (uint32_t)(32 * ks + 8 * g4) * ES;
      frag_bload(kf[j][ks], rK, off);
      frag_bload(vf[j][ks], rV, off);
    }
  }
  issue(qt0, 0);
  float lnext = 0.0f, dnext = 0.0f;
  if (w == 0) {
    vec_ld(qt0, lnext, dnext);
    wait_vmem();
    tL[0][lane] = lnext;
    tD[0][lane] = dnext;
  }
  const float c = a.scale_log2;

  f32x4 dk[2][4], dv[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      zero4(dk[j][v]);
      zero4(dv[j][v]);
    }
  for (int qt = qt0; qt < nqt; ++qt) {
    const int cur = (qt - qt0) & 1;
    wait_vmem();
    __syncthreads();  // query tile qt staged; every wave is done with the previous one
    if (qt + 1 < nqt) {
      issue(qt + 1, cur ^ 1);
      if (w == 0) vec_ld(qt + 1, lnext, dnext);
    }
    // sv[j][u][i], dp[j][u][i]: key r16 of group j against query q0 + 16 u + 4 g4 + i
    f32x4 sv[2][4], dp[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        zero4(sv[j][u]);
        zero4(dp[j][u]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag<T> qf, gf;
        frag_ld8_swz<DN>(qf, tQn[cur], 16 * u + r16, 32 * ks + 8 * g4);
        frag_ld8_swz<DN>(gf, tGn[cur], 16 * u + r16, 32 * ks + 8 * g4);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          mma(sv[j][u], qf, kf[j][ks]);
          mma(dp[j][u], gf, vf[j][ks]);
        }
      }
    }
    float pm[2][4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&tL[cur][16 * u + 4 * g4]);
      const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&tD[cur][16 * u + 4 * g4]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bool on = qt >= qbeg[j];  // the group's block has begun
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = on ? exp2_fast(fmaf(sv[j][u][i], c, -l4[i])) : 0.0f;
          pm[j][u][i] = p;
          sv[j][u][i] = p * (dp[j][u][i] - d4[i]);  // dS
        }
      }
    }
    // dV += P^T dO, dK += dS^T Q (queries along k)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      Frag<T> pf[2], df[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float mp[8], md[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mp[i] = pm[j][2 * q][i];
          mp[4 + i] = pm[j][2 * q + 1][i];
          md[i] = sv[j][2 * q][i];
          md[4 + i] = sv[j][2 * q + 1][i];
        }
        frag_from(pf[j], mp);
        frag_from(df[j], md);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        Frag<T> gt, qt2;
        frag_rows_swz<DTR>(gt, tGt[cur], 32 * q + 4 * g4, 32 * q + 16 + 4 * g4, 16 * v);
        frag_rows_swz<DTR>(qt2, tQt[cur], 32 * q + 4 * g4, 32 * q + 16 + 4 * g4, 16 * v);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          mma(dv[j][v], pf[j], gt);
          mma(dk[j][v], df[j], qt2);
        }
      }
    }
    if (qt + 1 < nqt && w == 0) {
      // the other buffer's previous readers passed the barrier above
      asm volatile("" : "+v"(lnext), "+v"(dnext) : : "memory");
      tL[cur ^ 1][lane] = lnext;
      tD[cur ^ 1][lane] = dnext;
    }
  }
  const float sc = a.scale;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t ss = k0 + 32 * w + 16 * j + 4 * g4 + i;
      if (ss >= L) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        a.dk[boff + (ss * H + h) * kAttnD + 16 * v + r16] = sc * dk[j][v][i];
        a.dv[boff + (ss * H + h) * kAttnD + 16 * v + r16] = dv[j][v][i];
      }
    }
}

hipError_t launch_attention_backward(const AttnArgs &a, hipStream_t st) {
  dim3 gq((unsigned)(a.Z * a.H * ((a.L + kAttnQ - 1) / kAttnQ)));
  dim3 gk((unsigned)(a.Z * a.H * ((a.L + kAttnQ - 1) / kAttnQ)));
  if (a.dtype == 1) {
    launch_kernel(k_attn_dq<bf16>, gq, dim3(kThreads), 0, st, a);
    launch_kernel(k_attn_dkv<bf16>, gk, dim3(kThreads), 0, st, a);
  } else {
    launch_kernel(k_attn_dq<float>, gq, dim3(kThreads), 0, st, a);
    launch_kernel(k_attn_dkv<float>, gk, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t st) {
  const int64_t nqt = (a.L + kAttnQ - 1) / kAttnQ;
  dim3 g((unsigned)(a.Z * a.H * nqt));
  if (a.dtype == 1) launch_kernel(k_attn_fwd<bf16>, g, dim3(kThreads), 0, st, a);
  else launch_kernel(k_attn_fwd<float>, g, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace bissd
