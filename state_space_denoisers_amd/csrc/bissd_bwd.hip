// bissd_bwd.hip -- backward-only kernels of the bidirectional SSD scan
// (gfx950): the dB / dC panels, the decay gradients, and the final
// deterministic reductions.
//
// Gradients of Loss = sum(dy * y) through the per-direction recurrence
// S_t = exp(dt_t A) S_{t-1} + dt_t x_t (outer) B_t, y_t = S_t C_t ("DiffMamba
// Checkpoints", Model details; the reverse direction runs the same recurrence
// over the flipped sequence).  Write cum_t for the direction's inclusive
// log2-decay sum inside a chunk (forward prefix lam, reverse suffix rho) and
// "s before t" for scan order (s <= t forward, s >= t reverse).  Unrolling the
// chunked recurrence (plain algebra):
//
//   W_h[t][s] = (dy_t . x_s) 2^(cum_t - cum_s) dt_s            (s before t)
//   dC_t = sum_h [ sum_s W_h[t][s] B_s + 2^cum_t dy_t S_in,h ]
//   dB_s = sum_h [ sum_t W_h[t][s] C_t + dt_s 2^(cum_end - cum_s) x_s Gc_h ]
//
// where S_in is the forward carry-in state of the chunk and Gc the adjoint
// carry arriving from the chunks after it in scan order (both P x N per
// head).  Because B and C are shared by the heads of a group, the heads' W
// are summed first and multiplied by B (or C) once per group.
//
// With d_lam_t = dy_t . y_d,t - dt_t x_t . (G_t B_t) (the gradient with
// respect to the cumulative log-decay at t) the decay gradient of token t is
// the sum of d_lam over t and every later token in scan order.  Summed over
// the tokens after the chunk that sum equals <Gc, S_out>, the adjoint carry
// times the state leaving the chunk, so each chunk's sum restarts from that
// exact boundary value:  ddt_t = x_t . (G_t B_t) + A dalpha_t.
//
// dA is taken in forward mode instead (sum_t dy_t . dy_t/dA), which has only
// non-negative weights and so none of the cancellation a sum of dt dalpha
// over every token would carry.  With T_t the cumulative dt in scan order,
// d/dA of 2^(cum_t - cum_s) is (T_t - T_s) times it, and
//   dA = sum_chunks [ sum_{s before t in the chunk} E[t][s] (T_t - T_s)
//                     + <G^T_loc, S_in> + <G_loc, S^A_in> ]
// with E[t][s] = W[t][s] (C_t . B_s), G_loc = sum_t 2^cum_t dy_t (outer) C_t,
// G^T_loc its (T_t - T_chunk start)-weighted version and S^A_in the A-tangent
// of the carry-in state.  The first sum comes from the dy.y_d pass of the
// output kernel (a second product whose Gram operand carries (T_t - T_s) per
// element), the inner products from the chunk-state kernels; they are added
// here.
#include <type_traits>

#include "bissd_device.hpp"
#include "bissd_internal.hpp"

namespace bissd {

// dt post-processing of direction d, head h (off when the direction has no bias)
__device__ __forceinline__ DtPost dt_post_of(const BwdArgs &a, int d, int h) {
  DtPost p;
  if (a.dtb[d]) {
    p.on = true;
    p.bias = a.dtb[d][h];
    p.lo = a.dtlo[d];
    p.hi = a.dthi[d];
  }
  return p;
}


// ============================================================ dB / dC panel

// compute units per XCD (256 in 8 XCDs)
constexpr int kCusPerXcd = 32;

template <typename T, int N> struct PanelLds {
  float lam[2][kQmax];
  float dtv[2][kQmax];
  float colf[2][kQmax]; // column factors of the off-diagonal blocks
};

// Workgroup = (batch b, chunk c, direction d, group g, 64-token row-block j)
// of one panel.  PNL 0 produces dC rows t: the row source is dy, the column
// source x, the columns s run before t in scan order.  PNL 1 produces dB rows
// s: the row source is x, the column source dy, the columns t run after s.
// Wave w owns rows 16 w .. 16 w + 15 of the block.  The carried-state term
// (with the forward carry-in for dC, the adjoint carry for dB) is added by
// k_bwd_state after the panel.
//
// Per head of the group: the Gram tiles D[col][row] = ColSrc_col . RowSrc_row
// come out of the matrix cores already laid out as the A operand of the
// later product, are weighted elementwise by 2^(cum_later - cum_earlier) dt
// and summed over heads in fp32 registers.  Off-diagonal column blocks use
// the factored weight 2^(cum_row - m) 2^(m - cum_col) (or its mirror), m the
// decay sum at the block boundary, so both factors are <= 1: a per-lane row
// factor times a per-column factor formed once per head; the diagonal block
// is weighted exactly per element and masked by selection.  After the last
// head the summed weights multiply the value rows (B for dC, C for dB), one
// 64-row slab at a time.
//
// Every head's column slabs are copied buffer -> LDS directly into a tile.
// With two tiles the copies for head h + 1 are in flight while head h is
// multiplied; with one (used: 38 KB of LDS), three workgroups per CU overlap
// each other's copies.  Each head costs one or two barriers.
template <typename T, int N, int PNL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 4 : 1)))
void k_bwd_panel(BwdArgs a) {
  using Sm = PanelLds<T, N>;
  constexpr uint32_t ES = sizeof(T);
  constexpr int CRB = kP * ES, SRB = N * ES;
  constexpr int CSB = 4 * kRB * CRB;
  // one tile: three workgroups share a CU and overlap each other's copies
  constexpr bool DBUF = false;
  using DC = DmaTile<CRB, SW_NAT>;
  using DS = DmaTile<SRB, SW_TR>;
  __shared__ Sm sm;
  __shared__ __attribute__((aligned(16))) char bufA[CSB];
  __shared__ __attribute__((aligned(16))) char bufB[DBUF ? CSB : 16];
  constexpr int NT = N / 16;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int Q = a.chunk, NRB = Q / kRB, H = a.H, G = a.G, hpg = H / G;
  const int64_t L = a.L;
  // work item = (((b * nchunks + c) * 2 + d) * G + g) * NRB + j', where an
  // XCD hands its consecutive workgroups to its 32 compute units in turn
  // (items 32 apart share one): the row-block j, whose causal column range
  // sets the workgroup's work (1 to NRB column blocks), is j' rotated by the
  // item's group of 32, so that a compute unit holds every row-block instead
  // of four workgroups of one (a bijection: the NRB items of one (b, c, d,
  // g) share their group)
  int bx = xcd_linear_id(blockIdx.x, gridDim.x);
  const int j = (bx + bx / kCusPerXcd) % NRB;
  bx /= NRB;
  const int g = bx % G;
  bx /= G;
  const int d = bx % 2;
  bx /= 2;
  const int c = bx % a.nchunks, b = bx / a.nchunks;
  const int64_t t0 = (int64_t)c * Q;
  const int qlen = (int)((L - t0) < Q ? (L - t0) : Q);
  if (j * kRB >= qlen) return;
  const int klast = (qlen - 1) / kRB;
  // columns before the row in index order: dC forward, dB reverse.  A
  // block-segmented reverse keeps its columns inside the row's block.
  const bool colLE = (PNL == 0) == (d == 0);
  const int segt = d == 1 ? a.rseg_tiles : 0;
  const int kseg0 = segt ? (j & ~(segt - 1)) : 0;
  const int kseg1 = segt ? min(kseg0 + segt - 1, klast) : klast;
  const int kb = colLE ? kseg0 : j, ke = colLE ? j : kseg1;

  const T *rowsrc = reinterpret_cast<const T *>(PNL == 0 ? a.dy : a.x);
  const T *colsrc = reinterpret_cast<const T *>(PNL == 0 ? a.x : a.dy);
  const T *valsrc = reinterpret_cast<const T *>(PNL == 0 ? a.B[d] : a.C[d]);
  const bufres rRow = make_buf(rowsrc + (int64_t)b * L * H * kP, (uint32_t)(L * H * kP * ES));
  const bufres rCol = make_buf(colsrc + (int64_t)b * L * H * kP, (uint32_t)(L * H * kP * ES));
  const bufres rVal = make_buf(valsrc + (int64_t)b * L * G * N, (uint32_t)(L * G * N * ES));
  const uint32_t xrs = (uint32_t)(H * kP * ES), vrs = (uint32_t)(G * N * ES);
  const int rrow = j * kRB + 16 * w + r16;  // this lane's row as Gram operand

  f32x4 wsum[4][4], oacc[NT];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int u = 0; u < 4; ++u) zero4(wsum[k][u]);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) zero4(oacc[nt]);

  // one head's column slabs kb..ke -> a tile
  auto issue_head = [&](int h, char *tile) __attribute__((always_inline)) {
    for (int k = kb; k <= ke; ++k)
      DC::load(tile + k * kRB * CRB, rCol, (uint32_t)((t0 + k * kRB) * H + h) * kP * ES, xrs, kRB);
  };
  auto issue_val = [&](int k, char *tile) __attribute__((always_inline)) {
    DS::load(tile, rVal, (uint32_t)((t0 + k * kRB) * G + g) * N * ES, vrs, kRB);
  };
  // row-source fragments of this lane's row (k = head-dim index)
  auto ld_rows = [&](int h, Frag<T> (&r)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      frag_bload(r[ks], rRow, (uint32_t)((t0 + rrow) * H + h) * kP * ES + (32 * ks + 8 * g4) * ES);
  };

  // Reference for the factored off-diagonal weights: the decay sum at the
  // boundary token between the row block and its off-diagonal columns (dC:
  // the token before the block in scan order; dB: the block's last token in
  // scan order).  Tokens outside the chunk only occur when there are no
  // off-diagonal blocks.
  const int mtok = PNL == 0 ? (d == 0 ? j * kRB - 1 : (j + 1) * kRB) : (d == 0 ? j * kRB + kRB - 1 : j * kRB);
  const bool mok = mtok >= 0 && mtok < Q;
  // Per-token values of one head, thread tid taking token tid of the chunk:
  // the decay sum and cumulative dt the chunk-state kernels kept (fp32,
  // [2][Z][H][L]), dt, and the decay sum at the reference token.  Loaded raw
  // (tokens past L read as zero) well before tok_put turns them into the
  // LDS rows: decay sums, dt, cumulative dt and the column factors
  // (dC 2^(m - cum_s) dt_s, dB 2^(cum_t - m)).
  const int64_t cbase = ((int64_t)d * a.Z + b) * H;
  // dt of one batch row; tokens past L read as zero
  const bufres rDt = make_buf(reinterpret_cast<const T *>(a.dt[d]) + (int64_t)b * L * H,
                              (uint32_t)(L * H * ES));
  auto tok_ld = [&](int h, uint32_t (&raw)[4]) __attribute__((always_inline)) {
    const bufres rl = make_buf(a.lamg + (cbase + h) * L, (uint32_t)(L * 4));
    const uint32_t off = (uint32_t)(t0 + tid) * 4u;
    raw[0] = __builtin_amdgcn_raw_buffer_load_b32(rl, off, 0, 0);
    raw[1] = a.dtb[d] ? __builtin_bit_cast(uint32_t, a.dtb[d][h]) : 0u;  // dt bias of head h
    const uint32_t doff = (uint32_t)((t0 + tid) * H + h) * ES;
    if constexpr (sizeof(T) == 2) raw[2] = __builtin_amdgcn_raw_buffer_load_b16(rDt, doff, 0, 0);
    else raw[2] = __builtin_amdgcn_raw_buffer_load_b32(rDt, doff, 0, 0);
    raw[3] = __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)(t0 + (mok ? mtok : 0)) * 4u, 0, 0);
  };
  DtPost post;
  post.on = a.dtb[d] != nullptr;
  post.lo = a.dtlo[d];
  post.hi = a.dthi[d];
  auto tok_put = [&](const uint32_t (&raw)[4], int buf) __attribute__((always_inline)) {
    if (tid < Q) {
      const float l = __builtin_bit_cast(float, raw[0]);
      DtPost ph = post;
      ph.bias = __builtin_bit_cast(float, raw[1]);
      const float draw = __builtin_bit_cast(float, sizeof(T) == 2 ? raw[2] << 16 : raw[2]);
      // tokens past L keep dt = 0
      const float dtv = t0 + tid < L ? dt_post(draw, ph) : 0.0f;
      const float m = mok ? __builtin_bit_cast(float, raw[3]) : 0.0f;
      sm.lam[buf][tid] = l;
      sm.dtv[buf][tid] = dtv;
      sm.colf[buf][tid] = PNL == 0 ? exp2_fast(fminf(m - l, 0.0f)) * dtv : exp2_fast(fminf(l - m, 0.0f));
    }
  };

  {
    uint32_t r0[4];
    tok_ld(g * hpg, r0);
    tok_put(r0, 0);
  }
  Frag<T> rf[2];
  ld_rows(g * hpg, rf);
  issue_head(g * hpg, bufA);

  auto do_head = [&](int hi, char *cur, char *nxt) __attribute__((always_inline)) {
    const int h = g * hpg + hi, lb = hi & 1;
    wait_vmem();
    __syncthreads();  // head hi's tiles, decay sums and row fragments are ready
    // per-row values are read before the next head's copies are issued (an
    // LDS read the compiler cannot tell apart from their destination would
    // otherwise wait for them)
    const float *lam = sm.lam[lb], *dtv = sm.dtv[lb];
    const float lrow = lam[rrow], drow = dtv[rrow];
    // row factor of the off-diagonal blocks (dC 2^(cum_t - m), dB dt_s 2^(m - cum_s))
    const float mref = mok ? lam[mtok] : 0.0f;
    const float rowf = PNL == 0 ? exp2_fast(fminf(lrow - mref, 0.0f)) : drow * exp2_fast(fminf(mref - lrow, 0.0f));
    Frag<T> rfn[2];
    uint32_t dtn[4];
    // the next head's per-token values, consumed after this head's products
    if (hi + 1 < hpg) tok_ld(h + 1, dtn);
    if (DBUF && hi + 1 < hpg) {
      issue_head(h + 1, nxt);
      ld_rows(h + 1, rfn);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < kb || k > ke) continue;
      const char *cs = cur + k * kRB * CRB;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        f32x4 dg;
        zero4(dg);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          Frag<T> cf;
          frag_ld8_swz<DC>(cf, cs, 16 * u + r16, 32 * ks + 8 * g4);
          mma(dg, cf, rf[ks]);
        }
        // dg[i] = ColSrc[col] . RowSrc[row], col = 64k + 16u + 4 g4 + i
        const int col0 = k * kRB + 16 * u + 4 * g4;
        if (k != j) {
          const f32x4 cf4 = *reinterpret_cast<const f32x4 *>(&sm.colf[lb][col0]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float wv = dg[i] * (rowf * cf4[i]);
            wsum[k][u][i] += wv;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = col0 + i;
            const bool ok = colLE ? (col <= rrow) : (col >= rrow);
            const float lcol = lam[col];
            const float ex = PNL == 0 ? lrow - lcol : lcol - lrow;
            const float dtf = PNL == 0 ? dtv[col] : drow;
            const float wv = ok ? dg[i] * (exp2_fast(fminf(ex, 0.0f)) * dtf) : 0.0f;
            wsum[k][u][i] += wv;
          }
        }
      }
    }

    if (hi + 1 < hpg) {
      if (!DBUF) {
        // single tile: the next head's copies wait for this head's reads
        __syncthreads();
        issue_head(h + 1, cur);
        ld_rows(h + 1, rfn);
      }
      // per-token rows of the next head into the other buffer.  The empty
      // asm keeps their use (and so the wait for their loads, issued before
      // this head's products) here rather than at the top of the head.
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(dtn[i]) : : "memory");
      tok_put(dtn, lb ^ 1);
      rf[0] = rfn[0];
      rf[1] = rfn[1];
    }
  };
  for (int hi = 0; hi < hpg; hi += 2) {
    do_head(hi, bufA, bufB);
    if (hi + 1 < hpg) do_head(hi + 1, DBUF ? bufB : bufA, bufA);
  }
  __syncthreads();

  // summed weights x value rows, one 64-row slab per column block
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k < kb || k > ke) continue;
    issue_val(k, bufA);
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float m[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m[i] = wsum[k][2 * q][i];
        m[4 + i] = wsum[k][2 * q + 1][i];
      }
      Frag<T> mf;
      frag_from(mf, m);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        Frag<T> vf;
        frag_rows_swz<DS>(vf, bufA, 32 * q + 4 * g4, 32 * q + 16 + 4 * g4, 16 * nt);
        mma(oacc[nt], mf, vf);
      }
    }
    __syncthreads();
  }

  float *out = PNL == 0 ? a.dC[d] : a.dB[d];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = j * kRB + 16 * w + 4 * g4 + i;
    if (r >= qlen) continue;
    float *o = out + ((((int64_t)b * L + t0 + r) * G + g) * N);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[16 * nt + r16] = oacc[nt][i];
  }
}

// ============================================ carried-state term of dB / dC

// The panels' carried-state term, summed over a group's heads:
//   dC_t += sum_h 2^cum_t (dy_t . S_in)            (PNL 0, S_in the carry-in)
//   dB_s += sum_h dt_s 2^(cum_end - cum_s) (x_s . Gc)  (PNL 1, Gc the adjoint carry)
// with the head-dim product dy_t . S (a 64-vector times a 64 x N state).
// Workgroup = (batch b, chunk c, direction d, group g, half of the chunk's
// rows), four waves; wave w owns chunk rows 128 half + 32 w .. + 31.  Two
// such workgroups per compute unit keep twice the state copies in flight
// that one eight-wave workgroup over the whole chunk did (train L=2K
// backward 1.073 -> 1.063 ms); each half copies every head's state (the
// second read of a state is an L2 hit: the halves run side by side).  Every head's state goes buffer -> LDS
// (transposed swizzle, as in the panels) into one of NS tiles, so the copies
// of the next NS - 1 heads are in flight while one is multiplied; each state
// tile serves all rows of the chunk.  Added to the panel's output (launched
// after it on the same stream, so the sum has a fixed order).
// an empty asm that takes a fragment's registers: the compiler waits for
// their loads here
__device__ __forceinline__ void hold(Frag<bf16> &f) { asm volatile("" : "+v"(f.v) : : "memory"); }
__device__ __forceinline__ void hold(Frag<float> &f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(f.v[e]) : : "memory");
}
constexpr int kStThreads = 256;
template <typename T, int N, int PNL>
__global__ __launch_bounds__(kStThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1)))
void k_bwd_state(BwdArgs a) {
  constexpr uint32_t ES = sizeof(T);
  constexpr int SRB = N * (int)ES, STB = kP * SRB;
  constexpr int NS = sizeof(T) == 2 ? 3 : 2;  // state tiles (heads) in flight
  constexpr int NT = N / 16;
  constexpr int NWV = kStThreads / 64;
  using DS = DmaTile<SRB, SW_TR>;
  // vector-memory instructions one head's issue() certainly adds per wave:
  // the copy pieces, the row fragments (one 16-byte load each in bf16, two
  // in fp32) and at least one load per row tile of decay sums
  constexpr int kCopyPieces = kP / DS::RPP;
  static_assert(kCopyPieces % NWV == 0, "every wave issues the same number of copy pieces");
  constexpr int kNextMin = kCopyPieces / NWV + (sizeof(T) == 2 ? 4 : 8) + 2;
  __shared__ __attribute__((aligned(16))) char tiles[NS * STB];
  const int tid = threadIdx.x, wv = wave_id(), lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int Q = a.chunk, H = a.H, G = a.G, hpg = H / G;
  const int64_t L = a.L;
  // work item = (((b * nchunks + c) * 2 + d) * G + g) * 2 + half; consecutive
  // items on one XCD, so both halves and both directions of a chunk read its
  // rows and states through the same L2
  int bx = xcd_linear_id(blockIdx.x, gridDim.x);
  const int rb = (bx & 1) * NWV * 32;  // first chunk row of this half
  bx >>= 1;
  const int g = bx % G;
  bx /= G;
  const int d = bx % 2;
  bx /= 2;
  const int c = bx % a.nchunks, b = bx / a.nchunks;
  const int64_t t0 = (int64_t)c * Q;
  const int qlen = (int)((L - t0) < Q ? (L - t0) : Q);
  if (rb >= qlen) return;  // the whole workgroup: no barrier is reached
  const bool rows = rb + 32 * wv < qlen;  // this wave has rows of the chunk

  const T *rowsrc = reinterpret_cast<const T *>(PNL == 0 ? a.dy : a.x);
  const T *stsrc = reinterpret_cast<const T *>(PNL == 0 ? a.sin[d] : a.gin[d]);
  const bufres rRow = make_buf(rowsrc + (int64_t)b * L * H * kP, (uint32_t)(L * H * kP * ES));
  const bufres rDt = make_buf(reinterpret_cast<const T *>(a.dt[d]) + (int64_t)b * L * H, (uint32_t)(L * H * ES));
  const int64_t cbase = ((int64_t)d * a.Z + b) * H;
  DtPost post;
  post.on = a.dtb[d] != nullptr;
  post.lo = a.dtlo[d];
  post.hi = a.dthi[d];

  // per head in flight: row-source fragments of the wave's two 16-row tiles,
  // the decay sums of the lane's 8 rows (rows rb + 32 w + 16 rt + 4 g4 + i), and
  // for dB their raw dt
  Frag<T> rf[NS][2][2];
  f32x4 lm[NS][2];
  uint32_t dtr[NS][2][4];
  // dB: the head's decay sum at the chunk's end and its dt bias (uniform
  // scalars, fetched with the head's other loads)
  float lendv[NS], biasv[NS];
  // Issue order, pinned by compiler fences (no memory access moves across
  // them, in the IR or in the machine scheduler): head after head, and in
  // each head the state copy before the register loads.  The waits below
  // count on it.
  auto fence = []() __attribute__((always_inline)) {
    asm volatile("" : : : "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto issue = [&](int hi, int slot) __attribute__((always_inline)) {
    const int h = g * hpg + hi;
    const int64_t soff = (int64_t)b * a.st_bstride + (int64_t)c * a.st_cstride + (int64_t)h * kP * N;
    fence();
    DS::load(tiles + slot * STB, make_buf(stsrc + soff, (uint32_t)(kP * N * ES)), 0u, (uint32_t)SRB, kP, wv, NWV);
    fence();
    // every wave loads its rows, also past the chunk (the next chunk's
    // tokens, or zeros past L), so that every wave can wait for them
    {
      const bufres rl = make_buf(a.lamg + (cbase + h) * L, (uint32_t)(L * 4));
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int r = rb + 32 * wv + 16 * rt;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          frag_bload(rf[slot][rt][ks], rRow, (uint32_t)((t0 + r + r16) * H + h) * kP * ES + (32 * ks + 8 * g4) * ES);
        // one load per token: tokens past L read as zero
        const uint32_t lo = (uint32_t)(t0 + r + 4 * g4) * 4u;
        lm[slot][rt] = f32x4{__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, lo, 0, 0)),
                             __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, lo + 4u, 0, 0)),
                             __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, lo + 8u, 0, 0)),
                             __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, lo + 12u, 0, 0))};
        if constexpr (PNL == 1) {
          if (rt == 0) {
            lendv[slot] = a.lamg[(cbase + h) * L + t0 + (d == 0 ? qlen - 1 : 0)];
            biasv[slot] = post.on ? a.dtb[d][h] : 0.0f;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t doff = (uint32_t)((t0 + r + 4 * g4 + i) * H + h) * ES;
            if constexpr (sizeof(T) == 2) dtr[slot][rt][i] = __builtin_amdgcn_raw_buffer_load_b16(rDt, doff, 0, 0);
            else dtr[slot][rt][i] = __builtin_amdgcn_raw_buffer_load_b32(rDt, doff, 0, 0);
          }
        }
      }
    }
  };

  f32x4 oacc[2][NT];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) zero4(oacc[rt][nt]);

#pragma unroll
  for (int u = 0; u < NS - 1; ++u)
    if (u < hpg) issue(u, u);
  for (int hi0 = 0; hi0 < hpg; hi0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int hi = hi0 + u;
      if (hi >= hpg) break;
      // This head's state copy (and its register loads) must be complete
      // before the barrier.  Vector-memory loads complete in issue order,
      // and the only loads issued after this head's are the next head's
      // (NS = 3, when there is a next head): at least its copy pieces, its
      // four (fp32: eight) row fragments and two decay-sum loads (the four
      // per-token loads of each row tile may be merged into one).  Waiting
      // until no more than that lower bound is outstanding covers this
      // head's copy and leaves the next head in flight.
      if (NS > 2 && hi + 1 < hpg) wait_vmem_le<kNextMin>();
      else wait_vmem_le<0>();
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) hold(rf[u][rt][ks]);
        asm volatile("" : "+v"(lm[u][rt]) : : "memory");
        if constexpr (PNL == 1)
#pragma unroll
          for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(dtr[u][rt][i]) : : "memory");
      }
      // every wave's part of this head's state is in LDS, and every wave is
      // done with the tile the next copy goes to (read in the last step)
      __syncthreads();
      if (hi + NS - 1 < hpg) issue(hi + NS - 1, (u + NS - 1) % NS);
      if (!rows) continue;
      const char *tile = tiles + u * STB;
      float lend = 0.0f, bias = 0.0f;
      if constexpr (PNL == 1) {
        lend = lendv[u];
        bias = biasv[u];
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        float fr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (PNL == 0) {
            fr[i] = exp2_fast(lm[u][rt][i]);
          } else {
            DtPost ph = post;
            ph.bias = bias;
            const int64_t tok = t0 + rb + 32 * wv + 16 * rt + 4 * g4 + i;
            const float draw = __builtin_bit_cast(float, sizeof(T) == 2 ? dtr[u][rt][i] << 16 : dtr[u][rt][i]);
            const float dtv = tok < L ? dt_post(draw, ph) : 0.0f;
            fr[i] = dtv * exp2_fast(fminf(lend - lm[u][rt][i], 0.0f));
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 t2;
          zero4(t2);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            Frag<T> sf;
            frag_rows_swz<DS>(sf, tile, 32 * ks + 8 * g4, 32 * ks + 8 * g4 + 4, 16 * nt);
            mma(t2, rf[u][rt][ks], sf);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[rt][nt][i] += fr[i] * t2[i];
        }
      }
    }
  }

  if (!rows) return;
  float *out = PNL == 0 ? a.dC[d] : a.dB[d];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb + 32 * wv + 16 * rt + 4 * g4 + i;
      if (r >= qlen) continue;
      float *o = out + ((((int64_t)b * L + t0 + r) * G + g) * N);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[16 * nt + r16] += oacc[rt][nt][i];
    }
}

// ====================================================== decay gradients

// One workgroup per (batch, direction, chunk, group of heads); the chunks
// are independent once their boundary values are known:
// d_lam_t = dy.y_d,t - dt_t x_t.(G_t B_t) (both taken without their common
// t' = t term, which cancels); dalpha_t = the in-chunk sum of d_lam over t
// and the tokens after it in scan order, plus the chunk's boundary value
// (the wave partials of <adjoint carry, state after the chunk>, summed in a
// fixed order); ddt_t = x_t.(G_t B_t) + A dalpha_t.
// Every per-token array is [token][head], so a chunk's rows for a group of
// heads sit together in memory: the workgroup reads and writes them in
// consecutive-element order (each wavefront instruction covers 64
// neighbouring elements) and transposes through an LDS tile [token][head],
// where one wavefront per head runs the sums along the tokens.
#ifndef BISSD_DECAY_HEADS
#define BISSD_DECAY_HEADS 32
#endif
#ifndef BISSD_DECAY_THREADS
#define BISSD_DECAY_THREADS 1024
#endif
constexpr int kDecHeads = BISSD_DECAY_HEADS;  // at most this many heads per workgroup
constexpr int kDecThreads = BISSD_DECAY_THREADS;
constexpr int kDecEpt = 256 * kDecHeads / kDecThreads;  // tile elements per thread
constexpr int kDecHpw = (kDecHeads + kDecThreads / 64 - 1) / (kDecThreads / 64);  // heads per wavefront

__host__ __device__ inline int decay_groups(int H) { return (H + kDecHeads - 1) / kDecHeads; }

// LDS word of (token t, head hl) for an odd row pitch S: a wavefront whose
// lanes take K = 4 consecutive tokens each (lane stride 4 S + 1, odd) and
// one whose lanes take consecutive elements both meet distinct banks
__device__ __forceinline__ int dec_idx(int t, int hl, int S) { return t * S + (t >> 2) + hl; }

template <typename T>
__global__ __launch_bounds__(kDecThreads) void k_bwd_decay(BwdArgs a) {
  __shared__ float sv[256 * (kDecHeads | 1) + 64];
  __shared__ float sA[kDecHeads], sBias[kDecHeads];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, nc = a.nchunks, ngrp = decay_groups(H), hgs = (H + ngrp - 1) / ngrp;
  int item = blockIdx.x;
  const int grp = item % ngrp;
  item /= ngrp;
  const int c = item % nc;
  item /= nc;
  const int d = item & 1, b = item >> 1;
  const int h0 = grp * hgs, hg = min(hgs, H - h0), S = hg | 1;
  const int64_t L = a.L, t0 = (int64_t)c * a.chunk;
  const int Q = a.chunk, K = Q / 64, nwv = kP * a.N / 256;
  const int qlen = (int)min<int64_t>(Q, L - t0);
  const int64_t row0 = (int64_t)b * L + t0;
  const int64_t wrow = ((int64_t)d * a.Z + b) * L + t0;
  const T *dt = reinterpret_cast<const T *>(a.dt[d]) + row0 * H + h0;
  const float *yd = a.ydot + wrow * H + h0, *qx = a.qx + wrow * H + h0, *qxs = a.qxs + wrow * H + h0;
  float *ddt = a.ddt[d] + row0 * H + h0;
  const bool post_on = a.dtb[d] != nullptr;
  if (tid < hg) {
    sA[tid] = a.A[d][h0 + tid];
    sBias[tid] = post_on ? a.dtb[d][h0 + tid] : 0.0f;
  }
  // the boundary values' wave partials of this wavefront's heads (lane k
  // holds partial k), fetched first so their latency hides behind the tile
  const float *rp = a.rpart + ((((int64_t)d * a.Z + b) * nc + c) * H + h0) * nwv;
  float rpv[kDecHpw];
#pragma unroll
  for (int m = 0; m < kDecHpw; ++m) {
    const int hl = wv + m * (kDecThreads / 64);
    rpv[m] = hl < hg && lane < nwv ? rp[hl * nwv + lane] : 0.0f;
  }
  // thread tid takes tile elements tid + j kDecThreads, element e = t hg + hl
  const int dq = kDecThreads / hg, dr = kDecThreads - dq * hg;
  const int tq0 = tid / hg, hr0 = tid - tq0 * hg;
  float rq[kDecEpt], ry[kDecEpt], rs[kDecEpt], rd[kDecEpt];
  {
    int t = tq0, hl = hr0;
#pragma unroll
    for (int j = 0; j < kDecEpt; ++j) {
      const int o = t < qlen ? t * H + hl : 0;
      rq[j] = qx[o];
      ry[j] = yd[o];
      rs[j] = qxs[o];
      rd[j] = to_f(dt[o]);
      t += dq;
      hl += dr;
      if (hl >= hg) {
        hl -= hg;
        ++t;
      }
    }
  }
  __syncthreads();
  float ql[kDecEpt], gr[kDecEpt];
  {
    int t = tq0, hl = hr0;
#pragma unroll
    for (int j = 0; j < kDecEpt; ++j) {
      const bool ok = t < qlen;
      DtPost p;
      p.on = post_on;
      p.bias = sBias[hl];
      p.lo = a.dtlo[d];
      p.hi = a.dthi[d];
      // d dt / d raw of a post-processed dt (1 without), for the chain rule below
      gr[j] = ok ? dt_post_grad(rd[j], p) : 0.0f;
      ql[j] = ok ? rq[j] : 0.0f;
      // dy.y_d and x.(G_t B_t) both without their common t' = t term; rows
      // beyond the sequence end hold 0
      if (t < Q) sv[dec_idx(t, hl, S)] = ok ? ry[j] - dt_post(rd[j], p) * rs[j] : 0.0f;
      t += dq;
      hl += dr;
      if (hl >= hg) {
        hl -= hg;
        ++t;
      }
    }
  }
  __syncthreads();
  // one wavefront per head: lane l holds tokens l K .. l K + K - 1; a sum
  // inside the lane, a scan across the lanes, and the boundary value
#pragma unroll
  for (int m = 0; m < kDecHpw; ++m) {
    const int hl = wv + m * (kDecThreads / 64);
    if (hl >= hg) break;
    // the partials' sum, in lane order, is the top lane of their scan
    const float R = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_scan_up(rpv[m])), 63));
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = i < K ? sv[dec_idx(lane * K + i, hl, S)] : 0.0f;
    float run = 0.0f;
    if (d == 0) {
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        run += x[i];
        x[i] = run;
      }
      const float excl = wave_shift_down1(wave_scan_down(run));
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] += excl + R;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        run += x[i];
        x[i] = run;
      }
      const float excl = wave_shift_up1(wave_scan_up(run));
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] += excl + R;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < K) sv[dec_idx(lane * K + i, hl, S)] = x[i];
  }
  __syncthreads();
  // with dt post-processing, ddt is taken back to the pre-activation and the
  // chunk's sum of it feeds the bias gradient
  {
    int t = tq0, hl = hr0;
#pragma unroll
    for (int j = 0; j < kDecEpt; ++j) {
      if (t < qlen) {
        const int k = dec_idx(t, hl, S);
        const float g = (ql[j] + sA[hl] * sv[k]) * gr[j];
        ddt[t * H + hl] = g;
        sv[k] = g;
      }
      t += dq;
      hl += dr;
      if (hl >= hg) {
        hl -= hg;
        ++t;
      }
    }
  }
  if (!post_on) return;
  __syncthreads();
  for (int hl = wv; hl < hg; hl += kDecThreads / 64) {
    float bsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = lane * K + i;
      if (i < K && t < qlen) bsum += sv[dec_idx(t, hl, S)];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) bsum += __shfl_xor(bsum, o, 64);
    if (lane == 0) a.dbpart[(((int64_t)d * a.Z + b) * nc + c) * H + h0 + hl] = bsum;
  }
}

// dA[d][h]: the cross-chunk inner products of every (batch, chunk) plus the
// within-chunk sums of every (batch, chunk, row-block) that holds tokens;
// dD[h]: the dy.x partials of those row-blocks.  One workgroup per output;
// fixed-order strided sums, then a fixed tree.
__global__ __launch_bounds__(kThreads) void k_bwd_reduce(BwdArgs a) {
  __shared__ float red[kThreads];
  const int tid = threadIdx.x, H = a.H, NRB = a.chunk / kRB;
  // 0 .. 2H-1: dA, 2H .. 3H-1: dD, 3H .. 5H-1: dt bias gradients
  const int o = blockIdx.x;
  if (o >= 3 * H) {
    const int db = (o - 3 * H) / H, hb = (o - 3 * H) % H;
    if (!a.ddtb[db]) return;
    const int64_t nbc = (int64_t)a.Z * a.nchunks;
    float sb = 0.0f;
    for (int64_t i = tid; i < nbc; i += kThreads) sb += a.dbpart[((int64_t)db * nbc + i) * H + hb];
    red[tid] = sb;
    __syncthreads();
    for (int k = kThreads / 2; k > 0; k >>= 1) {
      if (tid < k) red[tid] += red[tid + k];
      __syncthreads();
    }
    if (tid == 0) a.ddtb[db][hb] = red[0];
    return;
  }
  const int d = o < 2 * H ? o / H : 0, h = o < 2 * H ? o % H : o - 2 * H;
  float s = 0.0f;
  if (o < 2 * H) {
    const int64_t nbc = (int64_t)a.Z * a.nchunks;
    for (int64_t i = tid; i < nbc; i += kThreads) {
      const int64_t k = ((int64_t)d * nbc + i) * H + h;
      s += a.dAx1[k];
    }
  }
  const int64_t n = (int64_t)a.Z * a.nchunks * NRB;
  for (int64_t i = tid; i < n; i += kThreads) {
    const int j = (int)(i % NRB);
    const int64_t c = (i / NRB) % a.nchunks;
    const int64_t rem = a.L - c * a.chunk;
    const int qlen = (int)(rem < a.chunk ? rem : a.chunk);
    if (j * kRB >= qlen) continue;
    s += o < 2 * H ? a.dAintra[((int64_t)d * n + i) * H + h] : a.ddpart[i * H + h];
  }
  red[tid] = s;
  __syncthreads();
  for (int k = kThreads / 2; k > 0; k >>= 1) {
    if (tid < k) red[tid] += red[tid + k];
    __syncthreads();
  }
  if (tid == 0) {
    if (o < 2 * H) a.dA[d][h] = red[0];
    else a.dD[h] = red[0];
  }
}

// ============================================================= launchers

template <typename T, int N>
static void launch_panels_t(const BwdArgs &a, hipStream_t st) {
  dim3 g((unsigned)(a.Z * a.nchunks * 2 * a.G * (a.chunk / kRB)));
  dim3 gs((unsigned)(a.Z * a.nchunks * 2 * a.G * 2));
  launch_kernel((k_bwd_panel<T, N, 0>), g, dim3(kThreads), 0, st, a);
  launch_kernel((k_bwd_state<T, N, 0>), gs, dim3(kStThreads), 0, st, a);
  launch_kernel((k_bwd_panel<T, N, 1>), g, dim3(kThreads), 0, st, a);
  launch_kernel((k_bwd_state<T, N, 1>), gs, dim3(kStThreads), 0, st, a);
}

hipError_t launch_bwd_panels(const BwdArgs &a, hipStream_t st) {
  if (a.dtype == 1) {
    if (a.N == 128) launch_panels_t<bf16, 128>(a, st);
    else launch_panels_t<bf16, 64>(a, st);
  } else {
    if (a.N == 128) launch_panels_t<float, 128>(a, st);
    else launch_panels_t<float, 64>(a, st);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_decay(const BwdArgs &a, hipStream_t st) {
  dim3 g((unsigned)((int64_t)a.Z * 2 * a.nchunks * decay_groups(a.H)));
  if (a.dtype == 1) launch_kernel(k_bwd_decay<bf16>, g, dim3(kDecThreads), 0, st, a);
  else launch_kernel(k_bwd_decay<float>, g, dim3(kDecThreads), 0, st, a);
  launch_kernel(k_bwd_reduce, dim3((unsigned)(5 * a.H)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace bissd
