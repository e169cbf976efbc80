// bissd_fwd.hip -- forward kernels of the bidirectional SSD scan (gfx950).
//
// The per-direction recurrence S_t = exp(dt_t A) S_{t-1} + dt_t x_t (outer) B_t,
// y_t = S_t C_t ("DiffMamba Checkpoints", Model details: forward plus
// flipped-reverse Mamba-2; "DiffuMamba", Technical Summary, Methodology /
// Core Architecture: the two directions are added) is evaluated in chunks of
// Q tokens.  With log2-decays a_s = dt_s A log2(e), the inclusive prefix
// lam_t = sum_{k<=t} a_k inside a chunk (forward) and the inclusive suffix
// rho_t = sum_{k>=t} a'_k (reverse), unrolling the recurrence gives
//
//   forward:  y_t = 2^lam_t C_t S_in + sum_{s<=t} (C_t.B_s) 2^(lam_t-lam_s) dt_s x_s
//             S_out = 2^lam_last S_in + sum_s 2^(lam_last-lam_s) dt_s x_s (outer) B_s
//   reverse:  y_t = 2^rho_t C'_t S'_in + sum_{s>=t} (C'_t.B'_s) 2^(rho_t-rho_s) dt'_s x_s
//             S'_out = 2^rho_first S'_in + sum_s 2^(rho_first-rho_s) dt'_s x_s (outer) B'_s
//
// Three launches:
//   K1 chunk_state : per (batch, chunk, direction, head tile) the chunk-local
//                    state sum_s w_s x_s (outer) B_s on the matrix cores, and the
//                    chunk's total log2-decay.
//   K2 state_pass  : per (batch, head, direction) carry the states across
//                    chunks (forward ascending, reverse descending), turning
//                    each chunk-local state into that chunk's carry-in state.
//   K3 chunk_out   : per (batch, chunk, 64-token row-block, head tile) both
//                    directions' intra-chunk and carry-in terms plus D x,
//                    writing y exactly once.
#include "bissd_device.hpp"
#include "bissd_internal.hpp"

namespace bissd {

// =================================================================== K1

template <typename T, int N, int HT> struct K1Lds {
  static constexpr int XP = TokPitch<T>::value;
  float lam[HT][kQmax];
  float dtv[HT][kQmax];
  float scale[HT][kQmax];
  T Bt[N][XP];
  T Xs[HT][kP][XP];
};

// Chunk-local state S_loc = sum_s w_s x_s (outer) B_s with
// w_s = dt_s 2^(lam_last - lam_s) (forward) or dt_s 2^(rho_first - rho_s)
// (reverse), for one (batch, chunk, direction, head tile), plus the chunk's
// total log2-decay.  64-token slabs are fetched into registers one slab
// ahead of the matrix-core work.  Output states[d][b][c][h][p][n] (fp32),
// cdecay[d][b][c][h].  Wave w owns state columns n in [w N/4, (w+1) N/4).
template <typename T, int N, int HT>
__global__ __launch_bounds__(kThreads) void k1_chunk_state(ScanArgs a) {
  using Sm = K1Lds<T, N, HT>;
  using SB = SlabCols<T, N>;
  using SX = SlabCols<T, kP>;
  __shared__ Sm sm;
  constexpr int NT = N / 64;  // 16-wide column tiles per wave
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  int bx = blockIdx.x;
  const int d = a.dir0 + bx % a.ndir;
  bx /= a.ndir;
  const int c = bx % a.nchunks, b = bx / a.nchunks;
  const int h0 = blockIdx.y * HT;
  const int Q = a.chunk, H = a.H, G = a.G;
  const int64_t L = a.L;
  const int64_t t0 = (int64_t)c * Q;
  const int qlen = (int)((L - t0) < Q ? (L - t0) : Q);
  const int gidx = h0 / (H / G);
  const T *dt = reinterpret_cast<const T *>(a.dt[d]);
  const T *Bg = reinterpret_cast<const T *>(a.B[d]) + (((int64_t)b * L + t0) * G + gidx) * N;
  const T *xg = reinterpret_cast<const T *>(a.x) + (((int64_t)b * L + t0) * H + h0) * kP;
  const int64_t brs = (int64_t)G * N, xrs = (int64_t)H * kP;

  u32x4 pfB[SB::NV], pfX[HT][SX::NV];
  SB::prefetch(pfB, Bg, brs, qlen);
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) SX::prefetch(pfX[hh], xg + hh * kP, xrs, qlen);

  for (int hh = w; hh < HT; hh += 4)
    chunk_decay_scan<T>(dt + ((int64_t)b * L + t0) * H + h0 + hh, H, qlen, Q,
                        a.A[d][h0 + hh] * kLog2e, d == 1, sm.lam[hh], sm.dtv[hh]);
  __syncthreads();
  if (tid < HT)
    a.cdecay[(((int64_t)d * a.Z + b) * a.nchunks + c) * H + h0 + tid] =
        d == 0 ? sm.lam[tid][Q - 1] : sm.lam[tid][0];
  for (int it = tid; it < HT * Q; it += kThreads) {
    const int hh = it / Q, s = it % Q;
    const float ref = d == 0 ? sm.lam[hh][Q - 1] : sm.lam[hh][0];
    const float dv = sm.dtv[hh][s];
    sm.scale[hh][s] = dv != 0.0f ? dv * exp2_fast(ref - sm.lam[hh][s]) : 0.0f;
  }

  f32x4 acc[HT][4][NT];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) zero4(acc[hh][pt][nt]);

  const int nb = w * (N / 4);
  const int nslab = (qlen + kRB - 1) / kRB;
  for (int k = 0; k < nslab; ++k) {
    const int s0 = k * kRB;
    __syncthreads();
    SB::commit(&sm.Bt[0][0], pfB, nullptr);
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) SX::commit(&sm.Xs[hh][0][0], pfX[hh], &sm.scale[hh][s0]);
    __syncthreads();
    if (k + 1 < nslab) {
      const int s1 = s0 + kRB;
      SB::prefetch(pfB, Bg + s1 * brs, brs, qlen - s1);
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) SX::prefetch(pfX[hh], xg + s1 * xrs + hh * kP, xrs, qlen - s1);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      Frag<T> bf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        frag_ld4x2(bf[nt], &sm.Bt[nb + 16 * nt + r16][32 * q + 4 * g4],
                   &sm.Bt[nb + 16 * nt + r16][32 * q + 16 + 4 * g4]);
#pragma unroll
      for (int hh = 0; hh < HT; ++hh)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          Frag<T> xf;
          frag_ld4x2(xf, &sm.Xs[hh][16 * pt + r16][32 * q + 4 * g4],
                     &sm.Xs[hh][16 * pt + r16][32 * q + 16 + 4 * g4]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma(acc[hh][pt][nt], xf, bf[nt]);
        }
    }
  }

  float *out = a.states + ((((int64_t)d * a.Z + b) * a.nchunks + c) * H + h0) * (int64_t)(kP * N);
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[(int64_t)hh * kP * N + (16 * pt + 4 * g4 + i) * N + nb + 16 * nt + r16] =
              acc[hh][pt][nt][i];
}

// =================================================================== K2

// Four state elements per thread.  Forward: S_in(0) = init (or 0),
// S_in(c+1) = 2^cdecay(c) S_in(c) + S_loc(c); the reverse runs c downwards
// from zero.  Each chunk's carry-in is written, rounded once to T, to the
// sin_t buffer that the output kernel reads; the carry itself stays fp32 in
// registers and the forward state after the last chunk goes to final_state.
template <typename T>
__global__ __launch_bounds__(kThreads) void k2_state_pass(ScanArgs a, int PN) {
  const int e = (blockIdx.x * kThreads + threadIdx.x) * 4;
  const int h = blockIdx.y;
  const int d = a.dir0 + (int)(blockIdx.z % a.ndir);
  const int b = (int)(blockIdx.z / a.ndir);
  if (e >= PN) return;
  const int nc = a.nchunks, H = a.H;
  const int64_t cs = (int64_t)H * PN;
  const int64_t base = (((int64_t)d * a.Z + b) * nc * H + h) * (int64_t)PN + e;
  const float *src = a.states + base;
  T *dst = a.sin_t ? reinterpret_cast<T *>(a.sin_t) + base : nullptr;
  const float *dec = a.cdecay + ((int64_t)d * a.Z + b) * nc * H + h;
  f32x4 S = {0.0f, 0.0f, 0.0f, 0.0f};
  if (d == 0 && a.init_state)
    S = *reinterpret_cast<const f32x4 *>(a.init_state + ((int64_t)b * H + h) * PN + e);
  const int step = d == 0 ? 1 : -1;
  int c = d == 0 ? 0 : nc - 1;
  for (int n = 0; n < nc; ++n, c += step) {
    const f32x4 loc = *reinterpret_cast<const f32x4 *>(src + c * cs);
    const float g = exp2_fast(dec[(int64_t)c * H]);
    if (dst) {
      if constexpr (sizeof(T) == 2) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (bf16)S[i];
        *reinterpret_cast<bf16x4 *>(dst + c * cs) = o;
      } else {
        *reinterpret_cast<f32x4 *>(dst + c * cs) = S;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) S[i] = g * S[i] + loc[i];
  }
  if (d == 0 && a.final_state)
    *reinterpret_cast<f32x4 *>(a.final_state + ((int64_t)b * H + h) * PN + e) = S;
}

// =================================================================== K3

template <typename T, int N, int HT> struct K3Lds {
  static constexpr int BP = RowPitch<T, N>::value;
  static constexpr int XP = TokPitch<T>::value;
  static constexpr int OP = kP + 4;
  float lam[2][HT][kQmax];
  float dtv[2][HT][kQmax];
  float scale[2][HT][kQmax];
  float refb[2][HT];
  float amax[2][HT];
  union U {
    struct S {
      T Bs[kRB][BP];
      T Xs[HT][kP][XP];
    } s;
    T Sst[kP][BP];
    float Out[kRB][OP];
  } u;
};

template <typename T, int N, int HT> struct K3Pf {
  using SB = SlabRows<T, N>;
  using SX = SlabCols<T, kP>;
  using SS = SlabState<T, T, N>;
  using SF = SlabState<T, float, N>;
  static constexpr int SBLK = SB::NV + HT * SX::NV;
  static constexpr int NPF = SBLK > SF::NV ? SBLK : SF::NV;
};

// Workgroup = (batch b, chunk c, row-block j, head tile).  Wave w owns the 16
// output rows t = 64 j + 16 w + (0..15) of every head in the tile.
//
// Off-diagonal slabs (s-block k != j) and the carry-in term are evaluated in
// factored form around a per-head reference m (forward: lam at the token
// before the row-block; reverse: rho at the token after it):
//   2^(lam_t - lam_s) = 2^(lam_t - m) * 2^(m - lam_s),
// both factors <= 1, so C.B^T feeds the matrix cores unchanged, x is staged
// pre-multiplied by dt_s 2^(m - lam_s), the carry-in state by 2^m, and the
// row factor 2^(lam_t - m) is applied once to the sum.  The diagonal slab
// uses a reference per 16-token tile and is masked elementwise.
//
// Work runs as a pipeline of stages -- the s-blocks and then one carry-in
// stage per head, forward first, then reverse -- and the global loads of
// stage i+1 are issued into registers before the matrix-core work of stage i.
template <typename T, int N, int HT>
__global__ __launch_bounds__(kThreads) void k3_chunk_out(ScanArgs a) {
  using Sm = K3Lds<T, N, HT>;
  using PF = K3Pf<T, N, HT>;
  using SB = typename PF::SB;
  using SX = typename PF::SX;
  using SS = typename PF::SS;
  using SF = typename PF::SF;
  __shared__ Sm sm;
  constexpr int NK = N / 32;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int Q = a.chunk, NRB = Q / kRB, H = a.H, G = a.G;
  const int64_t L = a.L;
  int bx = blockIdx.x;
  const int j = bx % NRB;
  bx /= NRB;
  const int c = bx % a.nchunks, b = bx / a.nchunks;
  const int h0 = blockIdx.y * HT;
  const int64_t t0 = (int64_t)c * Q;
  const int qlen = (int)((L - t0) < Q ? (L - t0) : Q);
  if (j * kRB >= qlen) return;
  const int gidx = h0 / (H / G);
  const T *xg = reinterpret_cast<const T *>(a.x) + (((int64_t)b * L + t0) * H + h0) * kP;
  const int64_t xrs = (int64_t)H * kP, brs = (int64_t)G * N;
  const int klast = (qlen - 1) / kRB;

  // ---- stage list
  const int n0 = j + 1;
  const int n1 = a.sin[0] ? HT : 0;
  const int n2 = klast - j + 1;
  const int n3 = a.sin[1] ? HT : 0;
  const int nst = n0 + n1 + n2 + n3;
  auto decode = [&](int i, int &kind, int &d, int &kk) __attribute__((always_inline)) {
    if (i < n0) { kind = 0; d = 0; kk = i; }
    else if (i < n0 + n1) { kind = 1; d = 0; kk = i - n0; }
    else if (i < n0 + n1 + n2) { kind = 0; d = 1; kk = j + (i - n0 - n1); }
    else { kind = 1; d = 1; kk = i - n0 - n1 - n2; }
  };
  u32x4 pf[PF::NPF];
  auto prefetch = [&](int i) __attribute__((always_inline)) {
    int kind, d, kk;
    decode(i, kind, d, kk);
    if (kind == 0) {
      const int s0 = kk * kRB;
      SB::prefetch(pf, reinterpret_cast<const T *>(a.B[d]) + (((int64_t)b * L + t0 + s0) * G + gidx) * N,
                   brs, qlen - s0);
#pragma unroll
      for (int hh = 0; hh < HT; ++hh)
        SX::prefetch(pf + SB::NV + hh * SX::NV, xg + s0 * xrs + hh * kP, xrs, qlen - s0);
    } else {
      const int64_t off = (int64_t)b * a.sin_bstride[d] + (int64_t)c * a.sin_cstride[d] +
                          (int64_t)(h0 + kk) * kP * N;
      if (a.sin_f32[d]) SF::prefetch(pf, reinterpret_cast<const float *>(a.sin[d]) + off);
      else SS::prefetch(pf, reinterpret_cast<const T *>(a.sin[d]) + off);
    }
  };
  if (nst > 0) prefetch(0);

  // ---- decay scans (forward prefix and reverse suffix) for the whole chunk
  for (int pr = w; pr < 2 * HT; pr += 4) {
    const int d = pr / HT, hh = pr % HT;
    const float am = chunk_decay_scan<T>(
        reinterpret_cast<const T *>(a.dt[d]) + ((int64_t)b * L + t0) * H + h0 + hh, H, qlen, Q,
        a.A[d][h0 + hh] * kLog2e, d == 1, sm.lam[d][hh], sm.dtv[d][hh]);
    if (lane == 0) sm.amax[d][hh] = am;
  }

  // C rows of this wave (operand for both C.B^T and the carry-in product)
  const int trow = j * kRB + 16 * w + r16;
  Frag<T> cf[2][NK];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const T *Cp = reinterpret_cast<const T *>(a.C[d]) + (((int64_t)b * L + t0 + trow) * G + gidx) * N;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      if (trow < qlen) {
        float v[8];
        gload8(v, Cp + 32 * ks + 8 * g4);
        frag_from(cf[d][ks], v);
      } else {
        frag_zero(cf[d][ks]);
      }
    }
  }
  __syncthreads();

  if (tid < 2 * HT) {
    const int d = tid / HT, hh = tid % HT;
    sm.refb[d][hh] = d == 0 ? (j > 0 ? sm.lam[0][hh][j * kRB - 1] : 0.0f)
                            : ((j + 1) * kRB < Q ? sm.lam[1][hh][(j + 1) * kRB] : 0.0f);
  }
  // The factored diagonal slab multiplies by 2^(lam_t - lam_end) <= 2^(15 max|a|)
  // on one side; chunks whose decays could overflow that take the exact
  // per-element path instead (x staged unscaled, full 2^(lam_t - lam_s) dt_s
  // per element).
  bool exact = false;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) exact = exact || (sm.amax[d][hh] >= 8.0f);
  __syncthreads();
  for (int it = tid; it < 2 * HT * Q; it += kThreads) {
    const int d = it / (HT * Q), hh = (it / Q) % HT, s = it % Q;
    const bool dg = (s / kRB) == j;
    const float ref = dg ? (d == 0 ? sm.lam[0][hh][s | 15] : sm.lam[1][hh][s & ~15]) : sm.refb[d][hh];
    const float dv = sm.dtv[d][hh][s];
    sm.scale[d][hh][s] = (dg && exact) ? 1.0f : (dv != 0.0f ? dv * exp2_fast(ref - sm.lam[d][hh][s]) : 0.0f);
  }

  f32x4 acc[HT][4], tmp[HT][4];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      zero4(acc[hh][v]);
      zero4(tmp[hh][v]);
    }

  for (int i = 0; i < nst; ++i) {
    int kind, d, kk;
    decode(i, kind, d, kk);
    __syncthreads();
    // ---- commit stage i to LDS
    if (kind == 0) {
      SB::commit(&sm.u.s.Bs[0][0], pf);
#pragma unroll
      for (int hh = 0; hh < HT; ++hh)
        SX::commit(&sm.u.s.Xs[hh][0][0], pf + SB::NV + hh * SX::NV, &sm.scale[d][hh][kk * kRB]);
    } else {
      const float sc = exp2_fast(sm.refb[d][kk]);
      if (a.sin_f32[d]) SF::commit(&sm.u.Sst[0][0], pf, sc);
      else SS::commit(&sm.u.Sst[0][0], pf, sc);
    }
    __syncthreads();
    if (i + 1 < nst) prefetch(i + 1);

    // ---- compute stage i
    // this direction's C fragments (a select, so no register array is
    // indexed by the runtime direction)
    Frag<T> cd[NK];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) cd[ks] = d ? cf[1][ks] : cf[0][ks];
    if (kind == 0) {
      const bool diag = (kk == j);
      const int s0 = kk * kRB;
      int ulo = 0, uhi = 3;
      if (diag) {
        if (d == 0) uhi = w;
        else ulo = w;
      }
      // cb[u]: lane holds (C.B^T)[t = 16w + r16][s = 16u + 4 g4 + i]
      f32x4 cb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        zero4(cb[u]);
        if (u >= ulo && u <= uhi) {
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            Frag<T> bfr;
            frag_ld8(bfr, &sm.u.s.Bs[16 * u + r16][32 * ks + 8 * g4]);
            mma(cb[u], bfr, cd[ks]);
          }
        }
      }
      if (!diag) {
        Frag<T> mf[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float m[8];
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) {
            m[i2] = cb[2 * q][i2];
            m[4 + i2] = cb[2 * q + 1][i2];
          }
          frag_from(mf[q], m);
        }
#pragma unroll
        for (int hh = 0; hh < HT; ++hh)
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              Frag<T> xf;
              frag_ld4x2(xf, &sm.u.s.Xs[hh][16 * v + r16][32 * q + 4 * g4],
                         &sm.u.s.Xs[hh][16 * v + r16][32 * q + 16 + 4 * g4]);
              mma(tmp[hh][v], mf[q], xf);
            }
      } else {
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          const float lt = sm.lam[d][hh][s0 + 16 * w + r16];
          float f[4];
          if (!exact) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float ru = d == 0 ? sm.lam[0][hh][s0 + 16 * u + 15] : sm.lam[1][hh][s0 + 16 * u];
              f[u] = (u >= ulo && u <= uhi) ? exp2_fast(lt - ru) : 0.0f;
            }
          }
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (2 * q + 1 < ulo || 2 * q > uhi) continue;
            float m[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int u = 2 * q + (e >> 2), i2 = e & 3;
              const int sl = 4 * g4 + i2;  // position inside tile u
              bool ok = (u >= ulo && u <= uhi);
              if (u == w) ok = ok && (d == 0 ? (sl <= r16) : (sl >= r16));
              float wgt;
              if (exact) {
                const int sc = s0 + 16 * u + sl;
                wgt = ok ? exp2_fast(lt - sm.lam[d][hh][sc]) * sm.dtv[d][hh][sc] : 0.0f;
              } else {
                wgt = f[u];
              }
              m[e] = ok ? cb[u][i2] * wgt : 0.0f;
            }
            Frag<T> mf;
            frag_from(mf, m);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              Frag<T> xf;
              frag_ld4x2(xf, &sm.u.s.Xs[hh][16 * v + r16][32 * q + 4 * g4],
                         &sm.u.s.Xs[hh][16 * v + r16][32 * q + 16 + 4 * g4]);
              mma(acc[hh][v], mf, xf);
            }
          }
        }
      }
    } else {
      // carry-in term of head kk: C (16 rows) x (2^m S_in)^T
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) {
        if (hh != kk) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            Frag<T> sf;
            frag_ld8(sf, &sm.u.Sst[16 * v + r16][32 * ks + 8 * g4]);
            mma(tmp[hh][v], cd[ks], sf);
          }
      }
    }

    // ---- end of a direction: row factor 2^(lam_t - m) on the factored part
    const bool last_of_dir = (i == n0 + n1 - 1) || (i == nst - 1);
    if (last_of_dir) {
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) {
        const float rb = sm.refb[d][hh];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const float ut = exp2_fast(sm.lam[d][hh][j * kRB + 16 * w + 4 * g4 + i2] - rb);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc[hh][v][i2] += ut * tmp[hh][v][i2];
            tmp[hh][v][i2] = 0.0f;
          }
        }
      }
    }
  }

  // y = acc + D x, staged through LDS so that every lane writes 16 bytes
  T *yg = reinterpret_cast<T *>(a.y) + (((int64_t)b * L + t0 + j * kRB) * H + h0) * kP;
  const T *xo = xg + (int64_t)j * kRB * xrs;
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) {
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) sm.u.Out[16 * w + 4 * g4 + i2][16 * v + r16] = acc[hh][v][i2];
    __syncthreads();
    const float Dh = a.D[h0 + hh];
    for (int it = tid; it < kRB * 8; it += kThreads) {
      const int r = it >> 3, p0 = (it & 7) * 8;
      if (j * kRB + r >= qlen) continue;
      const int64_t off = (int64_t)r * xrs + hh * kP + p0;
      float xv[8], o[8];
      gload8(xv, xo + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = sm.u.Out[r][p0 + e] + Dh * xv[e];
      gstore8(yg + off, o);
    }
  }
}

// ============================================================= launchers

template <typename T, int N, int HT>
static void launch_t(const ScanArgs &a, int phase, hipStream_t st) {
  if (phase == PHASE_CHUNK_STATE) {
    dim3 g((unsigned)(a.Z * a.nchunks * a.ndir), (unsigned)(a.H / HT));
    hipLaunchKernelGGL((k1_chunk_state<T, N, HT>), g, dim3(kThreads), 0, st, a);
  } else if (phase == PHASE_STATE_PASS) {
    const int PN = kP * N;
    dim3 g2((unsigned)((PN / 4 + kThreads - 1) / kThreads), (unsigned)a.H, (unsigned)(a.Z * a.ndir));
    hipLaunchKernelGGL(k2_state_pass<T>, g2, dim3(kThreads), 0, st, a, PN);
  } else {
    dim3 g((unsigned)(a.Z * a.nchunks * (a.chunk / kRB)), (unsigned)(a.H / HT));
    hipLaunchKernelGGL((k3_chunk_out<T, N, HT>), g, dim3(kThreads), 0, st, a);
  }
}

template <typename T, int N>
static void launch_n(const ScanArgs &a, int phase, hipStream_t st, int HT) {
  if (HT == 4) launch_t<T, N, 4>(a, phase, st);
  else if (HT == 2) launch_t<T, N, 2>(a, phase, st);
  else launch_t<T, N, 1>(a, phase, st);
}

// Heads of one tile must share their B/C group: the tile is 4, 2 or 1 heads,
// whichever divides the heads per group.
#ifndef BISSD_MAX_HEAD_TILE
#define BISSD_MAX_HEAD_TILE 4
#endif

hipError_t launch_scan_phase(const ScanArgs &a, int phase, hipStream_t st) {
  const int hpg = a.H / a.G;
  int HT = (hpg % 4 == 0) ? 4 : (hpg % 2 == 0 ? 2 : 1);
  if (HT > BISSD_MAX_HEAD_TILE) HT = BISSD_MAX_HEAD_TILE;
  if (a.dtype == 0 && HT > 2) HT = 2;  // fp32 tiles of 4 heads exceed the register file
  if (a.dtype == 1) {
    if (a.N == 128) launch_n<bf16, 128>(a, phase, st, HT);
    else launch_n<bf16, 64>(a, phase, st, HT);
  } else {
    if (a.N == 128) launch_n<float, 128>(a, phase, st, HT);
    else launch_n<float, 64>(a, phase, st, HT);
  }
  return hipGetLastError();
}

}  // namespace bissd
