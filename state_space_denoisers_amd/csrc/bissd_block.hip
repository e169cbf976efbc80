// bissd_block.hip -- single-launch block update for active blocks of at most
// 64 tokens (gfx950).
//
// Block-wise denoising with a cached prefix ("Training Hybrid Block Diffusion
// Language Models with Partial Bidirectionality", Methodology and Technical
// Contribution): the forward scan continues from the cached state after the
// prefix, the reverse scan starts from zero at the block end and never
// leaves the block, and y = y_f + y_r + D x.  Committing the block advances
// the cached state over it:
//
//   forward : y_t = 2^lam_t C_t S_in + sum_{s<=t} (C_t.B_s) 2^(lam_t - lam_s) dt_s x_s
//   reverse : y_t =                    sum_{s>=t} (C'_t.B'_s) 2^(rho_t - rho_s) dt'_s x_s
//   S_out   = 2^lam_last S_in + sum_s 2^(lam_last - lam_s) dt_s x_s (outer) B_s
//
// The block is one chunk of the chunked scan, so the work of one (batch,
// head) fits one workgroup, and the call is bound by latency rather than by
// bandwidth or matrix-core time: every input of the workgroup is requested
// at once (B_f, B'_r and x rows and the cached state copied buffer -> LDS,
// C rows and dt into registers), the workgroup waits once, and both
// directions, the skip and the committed state follow without another
// global round trip.  The two directions run side by side in two groups of
// four waves (a batch of a few rows leaves most compute units idle, so each
// workgroup's critical path is what counts): the forward group adds the
// carried state, the reverse outputs reach the forward group through LDS for
// the one write of y, and the two groups form half of the committed state
// each.
//
// With the mixer's convolution (ScanArgs cw / ckw), each direction's scan
// reads its own convolved x, formed in LDS from the block's x tile right after
// it arrives: the forward's taps before the block read the conv state (the
// last ckw - 1 x rows of the prefix), the reverse's past the block read zero.
// The skip reads x itself; the next conv state (the last ckw - 1 rows of
// [conv state | x_blk]) is written at the end, after every read of the old
// one, so it may replace it in place.
#include "bissd_device.hpp"
#include "bissd_internal.hpp"

namespace bissd {

template <typename T, int N> struct BlockLds {
  static constexpr int BRB = N * (int)sizeof(T);
  static constexpr int XRB = kP * (int)sizeof(T);
  static constexpr int SRB = N * 4;
  using DB = DmaTile<BRB, SW_NAT>;
  using DX = DmaTile<XRB, SW_TR>;
  using DS = DmaTile<SRB, SW_NAT>;
  float lam[2][kRB];
  float dtv[2][kRB];
};

constexpr int kBlkThreads = 2 * kThreads;  // two groups of four waves

// Workgroup = (batch b, head h), two groups of four waves: group d takes
// direction d.  Wave w of a group owns block rows t = 16 w .. 16 w + 15 and
// committed state rows p = 16 w .. 16 w + 15 of its group's half of the
// state columns.  Decay
// weights are formed exactly per element (the block is a single 64 x 64
// tile), masked by selection.
template <typename T, int N>
__global__ __launch_bounds__(kBlkThreads) void k_block_update(ScanArgs a) {
  using Sm = BlockLds<T, N>;
  using DB = typename Sm::DB;
  using DX = typename Sm::DX;
  using DS = typename Sm::DS;
  __shared__ Sm sm;
  __shared__ __attribute__((aligned(16))) char tBf[kRB * Sm::BRB];
  __shared__ __attribute__((aligned(16))) char tBr[kRB * Sm::BRB];
  __shared__ __attribute__((aligned(16))) char tX[kRB * Sm::XRB];
  // the directions' convolved x (with the mixer's convolution) and the conv
  // state's rows of this head
  __shared__ __attribute__((aligned(16))) char tXc[2][kRB * Sm::XRB];
  __shared__ float cst[3][kP];
  __shared__ __attribute__((aligned(16))) char tS[kP * Sm::SRB];
  // the reverse group's outputs, [row block of wave w][v][lane] as f32x4;
  // fp32 tiles leave no room for it, so there it takes the reverse's
  // convolved tile (after a barrier: every reverse wave is done reading it)
  constexpr bool XALIAS = sizeof(T) == 4;
  static_assert(!XALIAS || sizeof(f32x4) * 4 * 4 * 64 <= kRB * Sm::XRB, "hand-over fits the tile");
  __shared__ __attribute__((aligned(16))) f32x4 xchg_own[XALIAS ? 1 : 4][4][64];
  f32x4 (*xchg)[4][64] = XALIAS ? reinterpret_cast<f32x4 (*)[4][64]>(tXc[1]) : xchg_own;
  constexpr int NK = N / 32, NT = N / 16;
  constexpr uint32_t ES = sizeof(T);
  const int tid = threadIdx.x, wv = wave_id(), lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int grp = wv >> 2, w = wv & 3;
  const int h = blockIdx.x % a.H, b = blockIdx.x / a.H;
  const int H = a.H, G = a.G, gidx = h / (H / G);
  const int L = (int)a.L;  // block length, 1..64
  const uint32_t brs = (uint32_t)(G * N * ES), xrs = (uint32_t)(H * kP * ES);

  // ---- every load of the workgroup, issued at once: the forward group
  // copies B_f and x, the reverse group B'_r and the cached state; each
  // group loads its own C rows and one of its waves its dt
  const bufres rB = make_buf(reinterpret_cast<const T *>(a.B[grp]) + (int64_t)b * L * G * N, (uint32_t)(L * G * N * ES));
  const bufres rC = make_buf(reinterpret_cast<const T *>(a.C[grp]) + (int64_t)b * L * G * N, (uint32_t)(L * G * N * ES));
  const float *sin = a.init_state + ((int64_t)b * H + h) * kP * N;
  DB::load(grp == 0 ? tBf : tBr, rB, (uint32_t)gidx * N * ES, brs, kRB, w, 4);
  if (grp == 0) {
    const bufres rX = make_buf(reinterpret_cast<const T *>(a.x) + (int64_t)b * L * H * kP, (uint32_t)(L * H * kP * ES));
    DX::load(tX, rX, (uint32_t)h * kP * ES, xrs, kRB, w, 4);
  } else {
    DS::load(tS, make_buf(sin, (uint32_t)(kP * N * 4)), 0u, (uint32_t)Sm::SRB, kP, w, 4);
  }
  const int trow = 16 * w + r16;
  Frag<T> cf[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks)
    frag_bload(cf[ks], rC, (uint32_t)(trow * G + gidx) * N * ES + (32 * ks + 8 * g4) * ES);
  const int K = a.ckw;
  if (K > 1 && tid < (K - 1) * kP) {
    const int j = tid / kP, c = tid % kP;
    cst[j][c] = a.cst_in ? to_f(reinterpret_cast<const T *>(a.cst_in)[(((int64_t)b * (K - 1) + j) * H + h) * kP + c])
                         : 0.0f;
  }
  if (w == 0) {
    DtPost post;
    if (a.dtb[grp]) {
      post.on = true;
      post.bias = a.dtb[grp][h];
      post.lo = a.dtlo[grp];
      post.hi = a.dthi[grp];
    }
    chunk_decay_scan<T>(reinterpret_cast<const T *>(a.dt[grp]) + (int64_t)b * L * H + h, H, L, kRB,
                        a.A[grp][h] * kLog2e, grp == 1, sm.lam[grp], sm.dtv[grp], false, post);
  }
  wait_vmem();
  __syncthreads();

  // ---- the directions' convolved x, [t][c] in the x tile's layout
  const char *tXd[2] = {tX, tX};
  if (K > 0) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (!a.cw[d]) continue;
      const float *wd = a.cw[d] + (int64_t)h * kP * K;
      const float *bd = a.cb[d] ? a.cb[d] + (int64_t)h * kP : nullptr;
      for (int e = tid; e < kRB * kP; e += kBlkThreads) {
        const int t = e / kP, c = e % kP;
        float v = bd ? bd[c] : 0.0f;
        for (int k = 0; k < K; ++k) {
          const int tj = d == 0 ? t - (K - 1) + k : t + (K - 1) - k;
          float xv = 0.0f;
          if (tj >= 0 && tj < L) xv = to_f(*reinterpret_cast<const T *>(tX + DX::at(tj, (int)ES * c)));
          else if (tj < 0) xv = cst[tj + K - 1][c];
          v += wd[c * K + k] * xv;
        }
        if (a.cact[d]) v = v / (1.0f + __expf(-v));
        *reinterpret_cast<T *>(tXc[d] + DX::at(t, (int)ES * c)) = from_f<T>(t < L ? v : 0.0f);
      }
      tXd[d] = tXc[d];
    }
    __syncthreads();
  }

  f32x4 acc[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) zero4(acc[v]);

  // ---- one direction's within-block terms (cf holds this group's C rows)
  auto direction = [&](auto dc) __attribute__((always_inline)) {
    constexpr int d = decltype(dc)::value;
    const char *Bt = d == 0 ? tBf : tBr;
    const int ulo = d == 0 ? 0 : w, uhi = d == 0 ? w : 3;
    // cb[u]: lane holds (C.B^T)[t = 16w + r16][s = 16u + 4 g4 + i]
    f32x4 cb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) zero4(cb[u]);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u < ulo || u > uhi) continue;
        Frag<T> bf;
        frag_ld8_swz<DB>(bf, Bt, 16 * u + r16, 32 * ks + 8 * g4);
        mma(cb[u], bf, cf[ks]);
      }
    }
    const float lt = sm.lam[d][trow];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (2 * q + 1 < ulo || 2 * q > uhi) continue;
      float m[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int u = 2 * q + (e >> 2), i2 = e & 3;
        const int s = 16 * u + 4 * g4 + i2;
        const bool ok = d == 0 ? s <= trow : s >= trow;
        const float wgt = exp2_fast(fminf(lt - sm.lam[d][s], 0.0f)) * sm.dtv[d][s];
        m[e] = ok ? cb[u][i2] * wgt : 0.0f;
      }
      Frag<T> mf;
      frag_from(mf, m);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        Frag<T> xf;
        frag_rows_swz<DX>(xf, tXd[d], 32 * q + 4 * g4, 32 * q + 16 + 4 * g4, 16 * v);
        mma(acc[v], xf, mf);
      }
    }
    if constexpr (d == 0) {
      // carried state: 2^lam_t (S_in C_t^T) for this lane's token t = 16w + r16
      const float et = exp2_fast(sm.lam[0][trow]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        f32x4 t2;
        zero4(t2);
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          Frag<T> sf;
          frag_ld8_swz_f32<DS>(sf, tS, 16 * v + r16, 32 * ks + 8 * g4);
          mma(t2, sf, cf[ks]);
        }
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) acc[v][i2] += et * t2[i2];
      }
    }
  };
  if (grp == 0) {
    direction(std::integral_constant<int, 0>{});
  } else {
    direction(std::integral_constant<int, 1>{});
  }
  if constexpr (XALIAS) __syncthreads();
  if (grp == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) xchg[w][v][lane] = acc[v];
  }

  // the reverse outputs are in LDS for the forward group's write of y; no
  // tile is written after this point
  __syncthreads();

  if (grp == 0) {
    // ---- y = forward + reverse + D x (forward group), x from its tile.  The
    // products are transposed (x^T W^T): the lane holds token t = 16w + r16
    // and four consecutive columns p = 16 v + 4 g4 + i per v, stored at once
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x4 r = xchg[w][v][lane];
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) acc[v][i2] += r[i2];
    }
    const float Dh = a.D[h];
    if (trow < L) {
      T *yg = reinterpret_cast<T *>(a.y) + (((int64_t)b * L + trow) * H + h) * kP;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int p = 16 * v + 4 * g4;
        const T *xp = reinterpret_cast<const T *>(tX + DX::at(trow, (int)ES * p));
        if constexpr (sizeof(T) == 2) {
          const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(xp);
          bf16x4 o;
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) o[i2] = (bf16)(acc[v][i2] + Dh * (float)xv[i2]);
          *reinterpret_cast<bf16x4 *>(yg + p) = o;
        } else {
          const f32x4 xv = *reinterpret_cast<const f32x4 *>(xp);
          f32x4 o;
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) o[i2] = acc[v][i2] + Dh * xv[i2];
          *reinterpret_cast<f32x4 *>(yg + p) = o;
        }
      }
    }
  }

  // ---- committed state: S_out = 2^lam_last S_in + sum_s w_s x_s (outer)
  // B_s, w_s = 2^(lam_last - lam_s) dt_s.  Group g forms columns n of its
  // half (16-column tiles g NT / 2 .. g NT / 2 + NT / 2 - 1); wave w owns
  // state rows p = 16w..16w+15.  Formed transposed (B^T x), so the lane
  // holds row p = 16w + r16 and four consecutive columns n per tile, read
  // from S_in and written as one 16-byte piece each.
  if (a.final_state) {
    constexpr int NH = NT / 2;
    const int nt0 = grp * NH;
    const float lend = sm.lam[0][kRB - 1];  // tokens past the block have dt = 0
    f32x4 sacc[NH];
#pragma unroll
    for (int nt = 0; nt < NH; ++nt) zero4(sacc[nt]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // A operand: x^T rows p = 16w + r16, k = s = 32ks + 8 g4 + e, scaled by w_s
      Frag<T> xa;
      frag_rows_swz<DX>(xa, tXd[0], 32 * ks + 8 * g4, 32 * ks + 8 * g4 + 4, 16 * w);
      float xv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int s = 32 * ks + 8 * g4 + e;
        const float dv = sm.dtv[0][s];
        xv[e] = (float)xa.v[e] * (dv != 0.0f ? dv * exp2_fast(lend - sm.lam[0][s]) : 0.0f);
      }
      frag_from(xa, xv);
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) {
        Frag<T> bfr;
        frag_rows_swz<DB>(bfr, tBf, 32 * ks + 8 * g4, 32 * ks + 8 * g4 + 4, 16 * (nt0 + nt));
        mma(sacc[nt], bfr, xa);
      }
    }
    const float gam = exp2_fast(lend);
    float *so = a.final_state + ((int64_t)b * H + h) * kP * N;
#pragma unroll
    for (int nt = 0; nt < NH; ++nt) {
      const int p = 16 * w + r16, n = 16 * (nt0 + nt) + 4 * g4;
      const f32x4 s0 = *reinterpret_cast<const f32x4 *>(tS + DS::at(p, 4 * n));
      f32x4 o;
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) o[i2] = gam * s0[i2] + sacc[nt][i2];
      *reinterpret_cast<f32x4 *>(so + p * N + n) = o;
    }
  }

  // ---- the next conv state: row j of [conv state | x_blk] at j + L (the old
  // rows were read into LDS before the first barrier)
  if (K > 1 && a.cst_out && tid < (K - 1) * kP) {
    const int j = tid / kP, c = tid % kP;
    const int src = j + L;  // row of [conv state | x_blk]
    const float v = src < K - 1 ? cst[src][c]
                                : to_f(*reinterpret_cast<const T *>(tX + DX::at(src - (K - 1), (int)ES * c)));
    reinterpret_cast<T *>(a.cst_out)[(((int64_t)b * (K - 1) + j) * H + h) * kP + c] = from_f<T>(v);
  }
}

template <typename T, int N>
static void launch_block_t(const ScanArgs &a, hipStream_t st) {
  launch_kernel((k_block_update<T, N>), dim3((unsigned)(a.Z * a.H)), dim3(kBlkThreads), 0, st, a);
}

hipError_t launch_block_update(const ScanArgs &a, hipStream_t st) {
  if (a.dtype == 1) {
    if (a.N == 128) launch_block_t<bf16, 128>(a, st);
    else launch_block_t<bf16, 64>(a, st);
  } else {
    if (a.N == 128) launch_block_t<float, 128>(a, st);
    else launch_block_t<float, 64>(a, st);
  }
  return hipGetLastError();
}

}  // namespace bissd
