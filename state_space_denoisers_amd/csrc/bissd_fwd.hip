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
#include <type_traits>

#include "bissd_device.hpp"
#include "bissd_internal.hpp"

namespace bissd {

// dt post-processing of direction d, head h (off when the direction has no bias)
__device__ __forceinline__ DtPost dt_post_of(const ScanArgs &a, int d, int h) {
  DtPost p;
  if (a.dtb[d]) {
    p.on = true;
    p.bias = a.dtb[d][h];
    p.lo = a.dtlo[d];
    p.hi = a.dthi[d];
  }
  return p;
}


// Gram tile pairs: for slot d, the (row-block j, column-block kb) pairs of
// one chunk that the output kernel reads (kb <= j for d = 0, kb >= j for
// d = 1), numbered row-block by row-block.
__device__ __forceinline__ void gram_pair(int pr, int d, int NRB, int &j, int &kb) {
  j = 0;
  kb = 0;
  for (int jj = 0; jj < NRB; ++jj) {
    const int n = d == 0 ? jj + 1 : NRB - jj;
    if (pr < n) {
      j = jj;
      kb = d == 0 ? pr : jj + pr;
      return;
    }
    pr -= n;
  }
}

// Gram tiles are stored in the compute dtype.  One lane's 16 values
// (accumulator u, element i) are GV = sizeof(T) 16-byte vectors, 64 lanes
// apart: fp32 vector v holds accumulator v; bf16 vector v holds
// accumulators 2v and 2v + 1.  A 16 x 64 tile is 64 GV vectors.
template <typename T> struct GramIO {
  static constexpr int GV = (int)sizeof(T);
  __device__ static __forceinline__ void put(u32x4 *p, const f32x4 (&cb)[4]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = (bf16)cb[2 * v][i];
          o[4 + i] = (bf16)cb[2 * v + 1][i];
        }
        p[v * 64] = __builtin_bit_cast(u32x4, o);
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v * 64] = __builtin_bit_cast(u32x4, cb[v]);
    }
  }
  __device__ static __forceinline__ void get(f32x4 (&cb)[4], const u32x4 *pf) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const bf16x8 o = __builtin_bit_cast(bf16x8, pf[v]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cb[2 * v][i] = (float)o[i];
          cb[2 * v + 1][i] = (float)o[4 + i];
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) cb[v] = __builtin_bit_cast(f32x4, pf[v]);
    }
  }
};

// =================================================================== K1

template <typename T, int N, int HT> struct K1Lds {
  static constexpr int BPT = TrPitch<T, N>::value;
  static constexpr int XPT = TrPitch<T, kP>::value;
  float lam[HT][kQmax];
  float dtv[HT][kQmax];
  float scale[HT][kQmax];
  float cdt[HT][kQmax];  // cumulative dt in scan order (tangent modes)
  float red[4][HT];
  T Bs[kRB][BPT];
  T Xs[HT][kRB][XPT];
};

// Chunk-local state S_loc = sum_s w_s x_s (outer) B_s with
// w_s = dt_s 2^(lam_last - lam_s) (forward) or dt_s 2^(rho_first - rho_s)
// (reverse), for one (batch, chunk, direction, head tile), plus the chunk's
// total log2-decay (MODE 0).  The backward pass reuses the kernel with other
// weights; T_s below is the cumulative dt inside the chunk in scan order
// (the A-derivative of the decay exponent):
//   MODE 1  w_s = 2^cum_s              adjoint state sum_t 2^cum_t dy_t (outer) C_t
//                                      (dy passed as x, C as B), also <state, sin>
//   MODE 2  w_s = dt_s 2^(cum_end - cum_s) (T_end - T_s)   A-tangent state, and
//                                      T_end per chunk to out1
// MODEs 1 and 2 leave the chunk decays as MODE 0 wrote them.  64-token slabs are fetched into registers one slab
// ahead of the matrix-core work and stored row-major; both operands are read
// with k (the token) running down the rows.  Output
// states[d][b][c][h][p][n] (compute dtype, rounded once from the fp32
// accumulators), cdecay[d][b][c][h].  Wave w owns state
// columns n in [w N/4, (w+1) N/4).
// With gram_k1 (MODE 0 over both directions) the workgroup of head tile tg
// within its B/C group also forms the Gram tiles of pair tg of its direction
// (the output kernel's C.B^T, as the Gram kernel below lays them out) while
// the pair's B slab is in LDS; the host sets it only when every pair has a
// workgroup.
template <typename T, int N, int HT, int MODE>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 1)))
void k1_chunk_state(ScanArgs a) {
  using Sm = K1Lds<T, N, HT>;
  using SB = SlabRows<T, N, Sm::BPT>;
  using SX = SlabRowsScaled<T, kP, Sm::XPT>;
  __shared__ Sm sm;
  constexpr int NT = N / 64;  // 16-wide column tiles per wave
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  // work item = ((b * nchunks + c) * ndir + dir) * (H / HT) + head tile
  uint32_t bx = (uint32_t)xcd_linear_id(blockIdx.x, gridDim.x), rem;
  bx = a.fd_tiles.divmod(bx, rem);
  const int h0 = (int)rem * HT;
  const int d = a.dir0 + (a.ndir == 2 ? (int)(bx & 1) : 0);
  bx = a.ndir == 2 ? bx >> 1 : bx;
  bx = a.fd_nc.divmod(bx, rem);
  const int c = (int)rem, b = (int)bx;
  const int Q = a.chunk, H = a.H, G = a.G;
  const int64_t L = a.L;
  const int64_t t0 = (int64_t)c * Q;
  const int qlen = (int)((L - t0) < Q ? (L - t0) : Q);
  const int gidx = (int)a.fd_hpg.div((uint32_t)h0);
  const T *dt = reinterpret_cast<const T *>(a.dt[d]);
  constexpr uint32_t ES = sizeof(T);
  // one buffer per batch row: tokens past L read as zero
  const bufres rB = make_buf(reinterpret_cast<const T *>(a.B[d]) + (int64_t)b * L * G * N,
                             (uint32_t)(L * G * N * ES));
  // the direction's scan input (its convolved x when it has one)
  const void *xsrc = a.xs[d] ? a.xs[d] : a.x;
  const bufres rX = make_buf(reinterpret_cast<const T *>(xsrc) + (int64_t)b * L * H * kP,
                             (uint32_t)(L * H * kP * ES));
  const uint32_t brs = (uint32_t)(G * N * ES), xrs = (uint32_t)(H * kP * ES);
  const uint32_t boff = (uint32_t)(t0 * G + gidx) * N * ES;
  const uint32_t xoff = (uint32_t)(t0 * H + h0) * kP * ES;

  // decay scans, wave w taking head w % HT (waves HT .. 2 HT - 1: the plain
  // cumulative dt of the tangent modes).  The dt loads go out first, raw and
  // unconditional (tokens past L read as zero), then the first slab's loads.
  constexpr bool TAN = MODE == 2;
  constexpr int NPR = (TAN ? 2 : 1) * HT;
  static_assert(NPR <= kThreads / 64, "one decay scan per wave");
  // Gram pair of this workgroup and the C rows of its row-block (raw loads,
  // first in the queue)
  const int NRB = Q / kRB, tpg = (H / G) / HT, tg = h0 / HT - gidx * tpg;
  const bool do_gram = MODE == 0 && a.gram_k1 && tg < NRB * (NRB + 1) / 2;
  int gj = 0, gkb = -1;
  Frag<T> gcf[N / 32];
  if (do_gram) {
    gram_pair(tg, d, NRB, gj, gkb);
    const bufres rC = make_buf(reinterpret_cast<const T *>(a.C[d]) + (int64_t)b * L * G * N,
                               (uint32_t)(L * G * N * ES));
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks)
      frag_bload(gcf[ks], rC, (uint32_t)((t0 + gj * kRB + 16 * w + r16) * G + gidx) * N * ES + (32 * ks + 8 * g4) * ES);
  }
  uint32_t dtraw[4];
  float Ah = 1.0f;
  DtPost post;
  if (w < NPR) {
    chunk_dt_bload<T>(make_buf(dt + (int64_t)b * L * H, (uint32_t)(L * H * ES)),
                      (uint32_t)(t0 * H + h0 + w % HT) * ES, (uint32_t)(H * ES), Q, dtraw);
    if (w < HT) Ah = a.A[d][h0 + w];
    post = dt_post_of(a, d, h0 + w % HT);
  }

  u32x4 pfB[SB::NV], pfX[HT][SX::NV];
  SB::prefetch(pfB, rB, boff, brs);
#pragma unroll
  for (int hh = 0; hh < HT; ++hh) SX::prefetch(pfX[hh], rX, xoff + hh * kP * ES, xrs);

  if (w < NPR) {
    const int hh = w % HT;
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(dtraw[i]) : : "memory");
    asm volatile("" : "+v"(Ah) : : "memory");
    float dv[4];
    chunk_dt_decode<T>(dtraw, Q, dv, post, qlen);
    if (w < HT)
      chunk_decay_scan_vals(dv, Q, Ah * kLog2e, d == 1, sm.lam[hh], sm.dtv[hh]);
    else
      chunk_decay_scan_vals(dv, Q, 1.0f, d == 1, sm.cdt[hh], sm.dtv[hh]);
  }
  __syncthreads();
  const int lq = 31 - __builtin_clz(Q);  // the chunk length is a power of two
  if ((MODE == 0 || MODE == 2) && a.cum_out) {
    // the backward pass keeps the decay sums (MODE 0) and cumulative dt
    // (MODE 2) of every token, [2][Z][H][L], token-contiguous per head
    for (int it = tid; it < HT * Q; it += kThreads) {
      const int hh = it >> lq, s = it & (Q - 1);
      if (s < qlen)
        a.cum_out[(((int64_t)d * a.Z + b) * H + h0 + hh) * L + t0 + s] = MODE == 0 ? sm.lam[hh][s] : sm.cdt[hh][s];
    }
  }
  const int64_t chi = (((int64_t)d * a.Z + b) * a.nchunks + c) * H + h0;  // (d, b, c, h0)
  if (MODE == 0 && tid < HT) a.cdecay[chi + tid] = d == 0 ? sm.lam[tid][Q - 1] : sm.lam[tid][0];
  if (MODE == 2 && tid < HT) a.out1[chi + tid] = d == 0 ? sm.cdt[tid][Q - 1] : sm.cdt[tid][0];
  for (int it = tid; it < HT * Q; it += kThreads) {
    const int hh = it >> lq, s = it & (Q - 1);
    const float ref = d == 0 ? sm.lam[hh][Q - 1] : sm.lam[hh][0];
    const float dv = sm.dtv[hh][s];
    float v;
    if (MODE == 1) {
      v = exp2_fast(sm.lam[hh][s]);
    } else {
      v = dv != 0.0f ? dv * exp2_fast(ref - sm.lam[hh][s]) : 0.0f;
      if (MODE == 2) v *= (d == 0 ? sm.cdt[hh][Q - 1] : sm.cdt[hh][0]) - sm.cdt[hh][s];
    }
    sm.scale[hh][s] = v;
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
    SB::commit(&sm.Bs[0][0], pfB);
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) SX::commit(&sm.Xs[hh][0][0], pfX[hh], &sm.scale[hh][s0]);
    __syncthreads();
    if (k + 1 < nslab) {
      const uint32_t s1 = s0 + kRB;
      SB::prefetch(pfB, rB, boff + s1 * brs, brs);
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) SX::prefetch(pfX[hh], rX, xoff + s1 * xrs + hh * kP * ES, xrs);
    }
    if (do_gram && k == gkb) {
      // Gram tile rows 64 gj + 16 w + (0..15), columns of this slab, in the
      // Gram kernel's order of accumulation and layout
      f32x4 cb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) zero4(cb[u]);
#pragma unroll
      for (int ks = 0; ks < N / 32; ++ks)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          Frag<T> bq;
          frag_ld8(bq, &sm.Bs[16 * u + r16][32 * ks + 8 * g4]);
          mma(cb[u], bq, gcf[ks]);
        }
      constexpr int GV = GramIO<T>::GV;
      u32x4 *go = reinterpret_cast<u32x4 *>(a.gram) +
                  ((((int64_t)d * a.Z + b) * a.nchunks + c) * G + gidx) * (int64_t)Q * Q * GV / 16 +
                  (int64_t)((4 * gj + w) * NRB + gkb) * 64 * GV + lane;
      GramIO<T>::put(go, cb);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r0 = 32 * q + 4 * g4, r1 = r0 + 16;
      Frag<T> bf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) frag_rows(bf[nt], &sm.Bs[0][0], Sm::BPT, r0, r1, nb + 16 * nt);
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) {
        Frag<T> xf[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) frag_rows(xf[pt], &sm.Xs[hh][0][0], Sm::XPT, r0, r1, 16 * pt);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) mma(acc[hh][pt][nt], xf[pt], bf[nt]);
      }
    }
  }

  // Forward calls (skip_edges) leave out the states no later kernel reads:
  // the forward direction's last chunk (unless it feeds final_state) and the
  // reverse direction's first chunk (the last in its scan order).
  const bool unread = MODE == 0 && a.skip_edges &&
                      (d == 0 ? (c == a.nchunks - 1 && a.final_state == nullptr) : c == 0);
  // MODE 1 also forms the Frobenius product of each head's state with the
  // given state of the same (direction, batch, chunk, head), in fp32 from the
  // accumulators: the given state is read in 16-byte pieces (issued before
  // the head's staging) into the same LDS tile, then in the accumulators'
  // layout; the sum is reduced in a fixed order.
  constexpr int EPV = 16 / (int)sizeof(T);
  constexpr int NPV = kP * N / EPV / kThreads;  // 16-byte pieces per thread of one head's state
  static_assert(kP * N * sizeof(T) <= sizeof(sm.Bs), "state tile must fit the B tile");
  T *stile = &sm.Bs[0][0];
  const T *ref = MODE == 1 ? reinterpret_cast<const T *>(a.sin[d]) + (int64_t)b * a.sin_bstride[d] +
                                 (int64_t)c * a.sin_cstride[d] + (int64_t)h0 * kP * N
                           : nullptr;
  if constexpr (MODE <= 2) {
    // one head at a time through LDS (the B tile, no longer read), so that
    // every thread stores (and MODE 1 loads) 16 contiguous bytes
    T *out = reinterpret_cast<T *>(a.states) + chi * (int64_t)(kP * N);
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) {
      u32x4 rp[MODE == 1 ? NPV : 1];
      if constexpr (MODE == 1) {
#pragma unroll
        for (int m = 0; m < NPV; ++m)
          rp[m] = *reinterpret_cast<const u32x4 *>(ref + (int64_t)hh * kP * N + (tid + m * kThreads) * EPV);
      }
      if (!unread) {
        __syncthreads();
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              stile[(16 * pt + 4 * g4 + i) * N + nb + 16 * nt + r16] = from_f<T>(acc[hh][pt][nt][i]);
        __syncthreads();
        for (int v = tid; v < kP * N / EPV; v += kThreads)
          *reinterpret_cast<u32x4 *>(out + (int64_t)hh * kP * N + v * EPV) =
              *reinterpret_cast<const u32x4 *>(stile + v * EPV);
      }
      if constexpr (MODE == 1) {
        __syncthreads();
#pragma unroll
        for (int m = 0; m < NPV; ++m) *reinterpret_cast<u32x4 *>(stile + (tid + m * kThreads) * EPV) = rp[m];
        __syncthreads();
        float v = 0.0f;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              v += acc[hh][pt][nt][i] * to_f(stile[(16 * pt + 4 * g4 + i) * N + nb + 16 * nt + r16]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0) sm.red[w][hh] = v;
      }
    }
  }
  if constexpr (MODE == 1) {
    __syncthreads();
    if (tid < HT) a.out0[chi + tid] = (sm.red[0][tid] + sm.red[1][tid]) + (sm.red[2][tid] + sm.red[3][tid]);
  }
}

// =================================================================== K2

// Four consecutive elements (8- or 16-byte aligned) loaded as raw bits and
// widened to fp32 only when used.  Any arithmetic on a loaded value makes the
// compiler wait for that load where it happens, and since loads complete in
// order that wait also covers every load issued before it; the empty asm in
// widen4 pins the widening at the point of use.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <typename T> struct Raw4 {
  using type = typename std::conditional<sizeof(T) == 2, u32x2, f32x4>::type;
};
template <typename T>
__device__ __forceinline__ typename Raw4<T>::type load4raw(const T *p) {
  return *reinterpret_cast<const typename Raw4<T>::type *>(p);
}
__device__ __forceinline__ f32x4 widen4(u32x2 r) {
  asm volatile("" : "+v"(r));
  return f32x4{__builtin_bit_cast(float, r[0] << 16), __builtin_bit_cast(float, r[0] & 0xffff0000u),
               __builtin_bit_cast(float, r[1] << 16), __builtin_bit_cast(float, r[1] & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 widen4(f32x4 r) {
  asm volatile("" : "+v"(r));
  return r;
}

// Four state elements per thread.  Forward: S_in(0) = init (or 0),
// S_in(c+1) = 2^cdecay(c) S_in(c) + S_loc(c); the reverse runs c downwards
// from zero.  Each chunk's carry-in is written, rounded once to T, to the
// sin_t buffer that the output kernel reads; the carry itself stays fp32 in
// registers and the forward state after the last chunk goes to final_state.
// flip: the adjoint carries of the backward pass, which run against their
// direction (forward: c downwards, reverse: c upwards), from zero.
// Block-segmented reverse: the reverse carry (primal or adjoint) restarts
// from zero at every chunk boundary that is a reverse block boundary.
// With flip, out0 (if set) receives per-wave partial sums of <carry arriving
// at chunk c, primal state after chunk c> (the primal carry-in of the next
// chunk in scan order, from sin[d]): the chunk-boundary value of the decay
// gradient.  Laid out [d][b][c][h][PN / 256].
template <typename T>
__global__ __launch_bounds__(kThreads) void k2_state_pass(ScanArgs a, int PN, int flip) {
  const int e = (blockIdx.x * kThreads + threadIdx.x) * 4;  // PN is a multiple of 1024
  const int h = blockIdx.y;
  const int d = a.dir0 + (int)(blockIdx.z % a.ndir);
  const int b = (int)(blockIdx.z / a.ndir);
  const int nc = a.nchunks, H = a.H;
  const int64_t cs = (int64_t)H * PN;
  const int64_t base = (((int64_t)d * a.Z + b) * nc * H + h) * (int64_t)PN + e;
  const T *src = reinterpret_cast<const T *>(a.states) + base;
  T *dst = a.sin_t ? reinterpret_cast<T *>(a.sin_t) + base : nullptr;
  const float *dec = a.cdecay + ((int64_t)d * a.Z + b) * nc * H + h;
  f32x4 S = {0.0f, 0.0f, 0.0f, 0.0f};
  const bool primal_fwd = d == 0 && !flip;
  if (primal_fwd && a.init_state)
    S = *reinterpret_cast<const f32x4 *>(a.init_state + ((int64_t)b * H + h) * PN + e);
  const bool up = (d == 0) != (flip != 0);
  const int step = up ? 1 : -1;
  const int c0 = up ? 0 : nc - 1;
  const bool rpart = flip && a.out0;
  // block-segmented reverse: index of the chunk boundary the carry arriving
  // at chunk c crosses (c from c - 1 upwards, c + 1 from c + 1 downwards),
  // kept modulo the chunks per block as c steps, so the loop divides nothing
  const int rsc = d == 1 ? a.rseg_chunks : 0;
  int bmod = rsc ? (up ? c0 : c0 + 1) % rsc : 1;
  const int nwv = PN / 256, wv = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const T *sinb = rpart ? reinterpret_cast<const T *>(a.sin[d]) + (int64_t)b * a.sin_bstride[d] +
                              (int64_t)h * PN + e
                        : nullptr;
  // The chunks' inputs are independent of the carry: a ring of D slots keeps
  // the loads of the next D chunks in flight (the loop is latency-bound for
  // long sequences otherwise).  Every load is unconditional: the primal
  // state after chunk c (for the boundary products) is read from a clamped,
  // always valid chunk and discarded by selection where there is none.
  constexpr int D = 8;
  typename Raw4<T>::type rl[D], rn[D];
  float rg[D];
  // Forward calls (skip_edges) leave out what the output kernel never reads:
  // the carry-in of the first chunk in scan order (zero, unless the forward
  // scan starts from init_state) and the state of the last chunk in scan
  // order (it only feeds final_state).
  const bool edge = a.skip_edges && !flip;
  const bool write_first = !edge || (primal_fwd && a.init_state);
  const int nload = (edge && !(primal_fwd && a.final_state)) ? nc - 1 : nc;
#pragma unroll
  for (int i = 0; i < D; ++i) rl[i] = {};
  auto fetch = [&](int slot, int cc) __attribute__((always_inline)) {
    rl[slot] = load4raw(src + cc * cs);
    rg[slot] = dec[(int64_t)cc * H];
    if (rpart) {
      int cn = d == 0 ? cc + 1 : cc - 1;
      cn = cn < 0 ? 0 : (cn >= nc ? nc - 1 : cn);
      rn[slot] = load4raw(sinb + (int64_t)cn * a.sin_cstride[d]);
    }
  };
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < nload) fetch(i, c0 + i * step);
  for (int n = 0; n < nc; n += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int nn = n + i;
      if (nn >= nc) break;
      const int c = c0 + nn * step;
      // widen this slot before refilling it, so the refill can reuse its
      // registers (a copy of an in-flight load would wait for it)
      const f32x4 loc = widen4(rl[i]);
      const f32x4 nb = rpart ? widen4(rn[i]) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const float g = exp2_fast(rg[i]);
      if (nn + D < nload) fetch(i, c + D * step);
      const bool cut = rsc != 0 && bmod == 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) S[k] = cut ? 0.0f : S[k];
      bmod = up ? (bmod + 1 == rsc ? 0 : bmod + 1) : (bmod == 0 ? rsc - 1 : bmod - 1);
      if (rpart) {
        // primal state after chunk c = primal carry-in of chunk c + 1
        // (forward) or c - 1 (reverse)
        const int cn = d == 0 ? c + 1 : c - 1;
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) v += S[k] * nb[k];
        v = (cn >= 0 && cn < nc) ? v : 0.0f;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
        if ((threadIdx.x & 63) == 0)
          a.out0[((((int64_t)d * a.Z + b) * nc + c) * H + h) * nwv + wv] = v;
      }
      if (dst && (nn > 0 || write_first)) {
        if constexpr (sizeof(T) == 2) {
          bf16x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k) o[k] = (bf16)S[k];
          *reinterpret_cast<bf16x4 *>(dst + c * cs) = o;
        } else {
          *reinterpret_cast<f32x4 *>(dst + c * cs) = S;
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) S[k] = g * S[k] + loc[k];
    }
  }
  if (primal_fwd && a.final_state)
    *reinterpret_cast<f32x4 *>(a.final_state + ((int64_t)b * H + h) * PN + e) = S;
}

// The carry passes in bf16 with eight state elements per thread, so every
// load and store moves 16 bytes; otherwise as k2_state_pass, FLIP selecting
// its adjoint mode.  A wave covers 512 consecutive elements, each 32-lane
// half the 256 of one boundary-product partial, so the partials keep the
// [d][b][c][h][PN / 256] layout and the same element groups.
__device__ __forceinline__ void widen8(u32x4 r, f32x4 &lo, f32x4 &hi) {
  asm volatile("" : "+v"(r));
  lo = f32x4{__builtin_bit_cast(float, r[0] << 16), __builtin_bit_cast(float, r[0] & 0xffff0000u),
             __builtin_bit_cast(float, r[1] << 16), __builtin_bit_cast(float, r[1] & 0xffff0000u)};
  hi = f32x4{__builtin_bit_cast(float, r[2] << 16), __builtin_bit_cast(float, r[2] & 0xffff0000u),
             __builtin_bit_cast(float, r[3] << 16), __builtin_bit_cast(float, r[3] & 0xffff0000u)};
}
__device__ __forceinline__ bf16x8 narrow8(const f32x4 &lo, const f32x4 &hi) {
  bf16x8 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = (bf16)lo[k];
    o[4 + k] = (bf16)hi[k];
  }
  return o;
}
template <bool FLIP>
__global__ __launch_bounds__(kThreads) void k2_state_pass8(ScanArgs a, int PN) {
  const int gt = blockIdx.x * kThreads + threadIdx.x;
  const int e = gt * 8;  // PN is a multiple of 2048
  const int h = blockIdx.y;
  const int d = a.dir0 + (int)(blockIdx.z % a.ndir);
  const int b = (int)(blockIdx.z / a.ndir);
  const int nc = a.nchunks, H = a.H;
  const int64_t cs = (int64_t)H * PN;
  const int64_t base = (((int64_t)d * a.Z + b) * nc * H + h) * (int64_t)PN + e;
  const bf16 *src = reinterpret_cast<const bf16 *>(a.states) + base;
  bf16 *dst = a.sin_t ? reinterpret_cast<bf16 *>(a.sin_t) + base : nullptr;
  const float *dec = a.cdecay + ((int64_t)d * a.Z + b) * nc * H + h;
  f32x4 S0 = {0.0f, 0.0f, 0.0f, 0.0f}, S1 = S0;
  const bool primal_fwd = d == 0 && !FLIP;
  if (primal_fwd && a.init_state) {
    const float *in = a.init_state + ((int64_t)b * H + h) * PN + e;
    S0 = *reinterpret_cast<const f32x4 *>(in);
    S1 = *reinterpret_cast<const f32x4 *>(in + 4);
  }
  const bool up = (d == 0) != FLIP;
  const int step = up ? 1 : -1;
  const int c0 = up ? 0 : nc - 1;
  const bool rpart = FLIP && a.out0;
  // block-segmented reverse: boundary index of the incoming carry, stepped
  const int rsc = d == 1 ? a.rseg_chunks : 0;
  int bmod = rsc ? (up ? c0 : c0 + 1) % rsc : 1;
  const int nwv = PN / 256, wv = gt >> 5;
  const bf16 *sinb = rpart ? reinterpret_cast<const bf16 *>(a.sin[d]) + (int64_t)b * a.sin_bstride[d] +
                                 (int64_t)h * PN + e
                           : nullptr;
  // forward calls skip the first chunk's zero carry-in and the last chunk's
  // state when it feeds no final_state
  const bool edge = a.skip_edges && !FLIP;
  const bool write_first = !edge || (primal_fwd && a.init_state);
  const int nload = (edge && !(primal_fwd && a.final_state)) ? nc - 1 : nc;
  constexpr int D = 8;
  u32x4 rl[D], rn[FLIP ? D : 1];
  float rg[D];
#pragma unroll
  for (int i = 0; i < D; ++i) rl[i] = u32x4{0u, 0u, 0u, 0u};
  auto fetch = [&](int slot, int cc) __attribute__((always_inline)) {
    rl[slot] = *reinterpret_cast<const u32x4 *>(src + cc * cs);
    rg[slot] = dec[(int64_t)cc * H];
    if constexpr (FLIP) {
      if (rpart) {
        int cn = d == 0 ? cc + 1 : cc - 1;
        cn = cn < 0 ? 0 : (cn >= nc ? nc - 1 : cn);
        rn[slot] = *reinterpret_cast<const u32x4 *>(sinb + (int64_t)cn * a.sin_cstride[d]);
      }
    }
  };
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < nload) fetch(i, c0 + i * step);
  for (int n = 0; n < nc; n += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int nn = n + i;
      if (nn >= nc) break;
      const int c = c0 + nn * step;
      f32x4 l0, l1, n0 = {0.0f, 0.0f, 0.0f, 0.0f}, n1 = n0;
      widen8(rl[i], l0, l1);
      if constexpr (FLIP) {
        if (rpart) widen8(rn[i], n0, n1);
      }
      const float g = exp2_fast(rg[i]);
      if (nn + D < nload) fetch(i, c + D * step);
      const bool cut = rsc != 0 && bmod == 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        S0[k] = cut ? 0.0f : S0[k];
        S1[k] = cut ? 0.0f : S1[k];
      }
      bmod = up ? (bmod + 1 == rsc ? 0 : bmod + 1) : (bmod == 0 ? rsc - 1 : bmod - 1);
      if constexpr (FLIP) {
        if (rpart) {
          // primal state after chunk c = primal carry-in of chunk c + 1
          // (forward) or c - 1 (reverse)
          const int cn = d == 0 ? c + 1 : c - 1;
          float v = 0.0f;
#pragma unroll
          for (int k = 0; k < 4; ++k) v += S0[k] * n0[k] + S1[k] * n1[k];
          v = (cn >= 0 && cn < nc) ? v : 0.0f;
          // row sums by DPP (lane 15 of each 16-lane row), then each 32-lane
          // half adds its two rows
          v += dpp_f<0x111>(v);
          v += dpp_f<0x112>(v);
          v += dpp_f<0x114>(v);
          v += dpp_f<0x118>(v);
          const int vi = __builtin_bit_cast(int, v);
          const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 15));
          const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 31));
          const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 47));
          const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 63));
          float *po = a.out0 + ((((int64_t)d * a.Z + b) * nc + c) * H + h) * nwv + wv;
          if ((threadIdx.x & 63) == 0) *po = r0 + r1;
          if ((threadIdx.x & 63) == 32) *po = r2 + r3;
        }
      }
      if (dst && (nn > 0 || write_first)) *reinterpret_cast<bf16x8 *>(dst + c * cs) = narrow8(S0, S1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        S0[k] = g * S0[k] + l0[k];
        S1[k] = g * S1[k] + l1[k];
      }
    }
  }
  if (primal_fwd && a.final_state) {
    float *out = a.final_state + ((int64_t)b * H + h) * PN + e;
    *reinterpret_cast<f32x4 *>(out) = S0;
    *reinterpret_cast<f32x4 *>(out + 4) = S1;
  }
}

// A-tangent of the carry-in states, four elements per thread:
// SA_in(c+1) = 2^cdecay(c) (SA_in(c) + Tsum(c) S_in(c)) + ST_loc(c), from zero,
// alongside the primal carry S_in (from init_state or zero), in each
// direction's scan order; SA_in of every chunk goes to sin_t in T (and S_in
// to sin_prim when set, which makes the primal state pass unnecessary).  Loads run
// D chunks ahead as in the state pass.  Both carries of a block-segmented
// reverse restart from zero at its block boundaries.
template <typename T>
__global__ __launch_bounds__(kThreads) void k2_tangent_pass(ScanArgs a, int PN) {
  const int e = (blockIdx.x * kThreads + threadIdx.x) * 4;
  const int h = blockIdx.y;
  const int d = (int)(blockIdx.z % 2);
  const int b = (int)(blockIdx.z / 2);
  const int nc = a.nchunks, H = a.H;
  const int64_t cs = (int64_t)H * PN;
  const int64_t base = (((int64_t)d * a.Z + b) * nc * H + h) * (int64_t)PN + e;
  const T *sl = reinterpret_cast<const T *>(a.states) + base;
  const T *tl = reinterpret_cast<const T *>(a.states2) + base;
  T *dst = reinterpret_cast<T *>(a.sin_t) + base;
  T *pdst = a.sin_prim ? reinterpret_cast<T *>(a.sin_prim) + base : nullptr;
  const float *dec = a.cdecay + ((int64_t)d * a.Z + b) * nc * H + h;
  const float *tsum = a.dtsum + ((int64_t)d * a.Z + b) * nc * H + h;
  f32x4 S = {0.0f, 0.0f, 0.0f, 0.0f}, SA = {0.0f, 0.0f, 0.0f, 0.0f};
  if (d == 0 && a.init_state)
    S = *reinterpret_cast<const f32x4 *>(a.init_state + ((int64_t)b * H + h) * PN + e);
  const int step = d == 0 ? 1 : -1;
  const int c0 = d == 0 ? 0 : nc - 1;
  // block-segmented reverse: the carry into chunk c crosses boundary c + 1,
  // kept modulo the chunks per block as c steps down
  const int rsc = d == 1 ? a.rseg_chunks : 0;
  int bmod = rsc ? (c0 + 1) % rsc : 1;
  constexpr int D = 4;
  typename Raw4<T>::type rl[D], rt[D];
  float rg[D], rs[D];
  auto fetch = [&](int slot, int cc) __attribute__((always_inline)) {
    rl[slot] = load4raw(sl + cc * cs);
    rt[slot] = load4raw(tl + cc * cs);
    rg[slot] = dec[(int64_t)cc * H];
    rs[slot] = tsum[(int64_t)cc * H];
  };
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < nc) fetch(i, c0 + i * step);
  for (int n = 0; n < nc; n += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int nn = n + i;
      if (nn >= nc) break;
      const int c = c0 + nn * step;
      const f32x4 loc = widen4(rl[i]), tloc = widen4(rt[i]);
      const float g = exp2_fast(rg[i]), ts = rs[i];
      if (nn + D < nc) fetch(i, c + D * step);
      const bool cut = rsc != 0 && bmod == 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        S[k] = cut ? 0.0f : S[k];
        SA[k] = cut ? 0.0f : SA[k];
      }
      bmod = bmod == 0 ? rsc - 1 : bmod - 1;
      if constexpr (sizeof(T) == 2) {
        bf16x4 o, op;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[k] = (bf16)SA[k];
          op[k] = (bf16)S[k];
        }
        *reinterpret_cast<bf16x4 *>(dst + c * cs) = o;
        if (pdst) *reinterpret_cast<bf16x4 *>(pdst + c * cs) = op;
      } else {
        *reinterpret_cast<f32x4 *>(dst + c * cs) = SA;
        if (pdst) *reinterpret_cast<f32x4 *>(pdst + c * cs) = S;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        SA[k] = g * (SA[k] + ts * S[k]) + tloc[k];
        S[k] = g * S[k] + loc[k];
      }
    }
  }
}

// The A-tangent pass in bf16 with eight elements per thread (16-byte loads
// and stores); otherwise as k2_tangent_pass.
__global__ __launch_bounds__(kThreads) void k2_tangent_pass8(ScanArgs a, int PN) {
  const int e = (blockIdx.x * kThreads + threadIdx.x) * 8;  // PN is a multiple of 2048
  const int h = blockIdx.y;
  const int d = (int)(blockIdx.z % 2);
  const int b = (int)(blockIdx.z / 2);
  const int nc = a.nchunks, H = a.H;
  const int64_t cs = (int64_t)H * PN;
  const int64_t base = (((int64_t)d * a.Z + b) * nc * H + h) * (int64_t)PN + e;
  const bf16 *sl = reinterpret_cast<const bf16 *>(a.states) + base;
  const bf16 *tl = reinterpret_cast<const bf16 *>(a.states2) + base;
  bf16 *dst = reinterpret_cast<bf16 *>(a.sin_t) + base;
  bf16 *pdst = a.sin_prim ? reinterpret_cast<bf16 *>(a.sin_prim) + base : nullptr;
  const float *dec = a.cdecay + ((int64_t)d * a.Z + b) * nc * H + h;
  const float *tsum = a.dtsum + ((int64_t)d * a.Z + b) * nc * H + h;
  f32x4 S0 = {0.0f, 0.0f, 0.0f, 0.0f}, S1 = S0, A0 = S0, A1 = S0;
  if (d == 0 && a.init_state) {
    const float *in = a.init_state + ((int64_t)b * H + h) * PN + e;
    S0 = *reinterpret_cast<const f32x4 *>(in);
    S1 = *reinterpret_cast<const f32x4 *>(in + 4);
  }
  const int step = d == 0 ? 1 : -1;
  const int c0 = d == 0 ? 0 : nc - 1;
  // block-segmented reverse: the carry into chunk c crosses boundary c + 1,
  // kept modulo the chunks per block as c steps down
  const int rsc = d == 1 ? a.rseg_chunks : 0;
  int bmod = rsc ? (c0 + 1) % rsc : 1;
  constexpr int D = 4;
  u32x4 rl[D], rt[D];
  float rg[D], rs[D];
  auto fetch = [&](int slot, int cc) __attribute__((always_inline)) {
    rl[slot] = *reinterpret_cast<const u32x4 *>(sl + cc * cs);
    rt[slot] = *reinterpret_cast<const u32x4 *>(tl + cc * cs);
    rg[slot] = dec[(int64_t)cc * H];
    rs[slot] = tsum[(int64_t)cc * H];
  };
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < nc) fetch(i, c0 + i * step);
  for (int n = 0; n < nc; n += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int nn = n + i;
      if (nn >= nc) break;
      const int c = c0 + nn * step;
      f32x4 l0, l1, t0, t1;
      widen8(rl[i], l0, l1);
      widen8(rt[i], t0, t1);
      const float g = exp2_fast(rg[i]), ts = rs[i];
      if (nn + D < nc) fetch(i, c + D * step);
      const bool cut = rsc != 0 && bmod == 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        S0[k] = cut ? 0.0f : S0[k];
        S1[k] = cut ? 0.0f : S1[k];
        A0[k] = cut ? 0.0f : A0[k];
        A1[k] = cut ? 0.0f : A1[k];
      }
      bmod = bmod == 0 ? rsc - 1 : bmod - 1;
      *reinterpret_cast<bf16x8 *>(dst + c * cs) = narrow8(A0, A1);
      if (pdst) *reinterpret_cast<bf16x8 *>(pdst + c * cs) = narrow8(S0, S1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        A0[k] = g * (A0[k] + ts * S0[k]) + t0[k];
        A1[k] = g * (A1[k] + ts * S1[k]) + t1[k];
        S0[k] = g * S0[k] + l0[k];
        S1[k] = g * S1[k] + l1[k];
      }
    }
  }
}

// ================================================================= Gram

// The output kernel's C.B^T tiles, computed once per (batch, chunk, group)
// instead of once per head tile.  Workgroup = (batch, chunk, slot d, group,
// one (row-block j, column block kb) pair on the side slot d reads: kb <= j
// for d = 0, kb >= j for d = 1); wave w forms the 16 x 64 tile of rows
// t = 64 j + 16 w + (0..15) and columns s = 64 kb + (0..63).  Lane (r16, g4)
// holds (C.B^T)[t = 64 j + 16 w + r16][s = 64 kb + 16 u + 4 g4 + i] in
// accumulator u, element i -- the lane order in which the output kernel's
// wave needs them -- accumulated in fp32 and rounded once to the compute
// dtype.  Rows and columns past the sequence end are zero.
// Layout: [2][Z][nchunks][G][chunk * chunk] in the compute dtype; tile
// (16-row tile tt, column block kb) at element (tt * (chunk / 64) + kb) * 1024,
// each lane's values as GramIO lays them out, so every store and load moves a
// contiguous kilobyte.
// Work items are grouped so that all the workgroups of one (batch, chunk)
// run on one XCD and share its L2 copy of the B and C rows.
template <typename T, int N>
__global__ __launch_bounds__(kThreads) void k_gram(ScanArgs a) {
  // workgroup = (batch, chunk, slot, group, column block kb); wave w forms
  // rows 16 w .. 16 w + 15 of every row-block j on the slot's side of kb
  // (j >= kb for slot 0, j <= kb for slot 1), holding kb's B rows in
  // registers across them; the heaviest column blocks come first
  constexpr int NK = N / 32;
  constexpr uint32_t ES = sizeof(T);
  const int w = wave_id(), lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
  const int Q = a.chunk, NRB = Q / kRB, G = a.G;
  uint32_t item = (uint32_t)xcd_linear_id(blockIdx.x, gridDim.x), rem;
  const int kr = (int)(item % (uint32_t)NRB);
  item /= (uint32_t)NRB;
  item = a.fd_g.divmod(item, rem);
  const int g = (int)rem;
  const int d = (int)(item & 1);
  item = a.fd_nc.divmod(item >> 1, rem);
  const int c = (int)rem, b = (int)item;
  const int kb = d == 0 ? kr : NRB - 1 - kr;
  const int j0 = d == 0 ? kb : 0, j1 = d == 0 ? NRB - 1 : kb;
  const int64_t L = a.L, t0 = (int64_t)c * Q;
  const bufres rC = make_buf(reinterpret_cast<const T *>(a.C[d]) + (int64_t)b * L * G * N, (uint32_t)(L * G * N * ES));
  const bufres rB = make_buf(reinterpret_cast<const T *>(a.B[d]) + (int64_t)b * L * G * N, (uint32_t)(L * G * N * ES));
  Frag<T> cf[NK], bf[4][NK];
  auto load_c = [&](int j, Frag<T> (&f)[NK]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      frag_bload(f[ks], rC, (uint32_t)((t0 + j * kRB + 16 * w + r16) * G + g) * N * ES + (32 * ks + 8 * g4) * ES);
  };
  load_c(j0, cf);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      frag_bload(bf[u][ks], rB, (uint32_t)((t0 + kb * kRB + 16 * u + r16) * G + g) * N * ES + (32 * ks + 8 * g4) * ES);
  constexpr int GV = GramIO<T>::GV;
  u32x4 *base = reinterpret_cast<u32x4 *>(a.gram) +
                ((((int64_t)d * a.Z + b) * a.nchunks + c) * G + g) * (int64_t)Q * Q * GV / 16 + lane;
  for (int j = j0; j <= j1; ++j) {
    Frag<T> cn[NK];
    if (j < j1) load_c(j + 1, cn);
    f32x4 cb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) zero4(cb[u]);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) mma(cb[u], bf[u][ks], cf[ks]);
    GramIO<T>::put(base + (int64_t)((4 * j + w) * NRB + kb) * 64 * GV, cb);
    if (j < j1)
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) cf[ks] = cn[ks];
  }
}

// =================================================================== K3

template <typename T, int N, int HT> struct K3Lds {
  static constexpr int BP = RowPitch<T, N>::value;  // natural-read rows
  static constexpr int XPT = TrPitch<T, kP>::value; // k-along-rows tile
  static constexpr int OP = kP + 4;
  float lam[2][HT][kQmax];
  alignas(16) float scale[2][HT][kQmax];  // holds dt until the scales are formed
  float dtd[2][HT][kRB];      // dt of the diagonal block (exact path)
  float refb[2][HT];
  float amax[2][HT];
  float red[4][HT];  // per-wave partial sums (PHASE_DX)
  float bcd[2][kRB];  // B_t . C_t of the row-block's tokens (PHASE_DX)
  union U {
    struct S {
      T Xs[HT][kRB][XPT];
    } s;
    T Sst[1][kP][BP];
    float Out[1][kRB][OP];
  } u;
};

template <typename T, int N, int HT, bool SF32> struct K3Pf {
  static constexpr int IH = 1;  // heads per carry-in / output stage (LDS for four workgroups per CU)
  static constexpr int NG = GramIO<T>::GV;    // 16-byte vectors of one lane's Gram tile
  using SX = SlabRows<T, kP, K3Lds<T, N, HT>::XPT>;
  using SS = SlabState<T, typename std::conditional<SF32, float, T>::type, N>;
  static constexpr int SBLK = NG + HT * SX::NV;
  static constexpr int NPF = SBLK > IH * SS::NV ? SBLK : IH * SS::NV;
};

// Workgroup = (batch b, chunk c, row-block j, head tile).  Wave w owns the 16
// output rows t = 64 j + 16 w + (0..15) of every head in the tile.
//
// Off-diagonal slabs (s-block k != j) and the carry-in term are evaluated in
// factored form around a per-head reference m (forward: lam at the token
// before the row-block; reverse: rho at the token after it):
//   2^(lam_t - lam_s) = 2^(lam_t - m) * 2^(m - lam_s),
// both factors <= 1: each lane multiplies its C.B^T values by the row
// factor 2^(lam_t - m) of its row t and by the column factor
// dt_s 2^(m - lam_s) of each column s before they feed the matrix cores,
// with x staged as stored.  The carry-in term 2^lam_t C S_in^T uses the
// states as stored and applies 2^lam_t to its own small accumulator.  The
// diagonal slab uses a reference per 16-token tile and is masked
// elementwise.
//
// The C.B^T tiles come precomputed (chunk-state or Gram kernel), one 16 x 64
// tile per wave and s-block in the compute dtype, already in the lane order
// of the matrix-core accumulators.
//
// Work runs as a pipeline of stages -- the s-blocks, then the carry-in
// states one head per stage, forward first, then reverse -- and the global
// loads of the next stage are issued into registers before the matrix-core
// work of the current one.
// SF32: the carry-in states are fp32 (the block update's cached state)
// rather than the compute dtype written by the state pass.
//
// MODE 0 writes y.  The backward pass runs the same kernel twice more:
// MODE 1 recomputes each direction's output y_d and stores only dy.y_d per
// (token, head), and with a second product of the same x tiles, whose Gram
// operand carries the extra factor (T_t - T_s) per element (T the in-chunk
// cumulative dt in scan order), the within-chunk part of dA:
// sum_{s before t} E[t][s] (T_t - T_s) per (row-block, head); MODE 2 evaluates the adjoint product G_t B_t, where
// G_t = sum_{t' at or after t in scan order} 2^(cum_t' - cum_t) dy_t' (outer) C_t'
// plus the carried adjoint.  That is this kernel's structure with the row
// and column operands swapped (B_t as the row, C_t' as the column), dy in
// place of x, no dt on the staged side, and exclusive cumulative decays; slot
// 0 (causal) carries the reverse direction and slot 1 the forward one.  It
// writes dx = dt_f G_f B + dt_r G_r B + D dy, x.(G_t B_t) per direction and
// partial sums of dy.x.
// In both backward modes the diagonal tile is masked strictly (t' != t):
// the t' = t term is the same product E_tt = dt_t (dy_t.x_t)(B_t.C_t) in
// dy.y_d and in dt_t x.(G_t B_t), and the decay gradient needs only their
// difference, so leaving it out of both removes a cancellation that large
// |A| would amplify.  MODE 2 adds the term back where it is a plain part of
// the result: dy_t (B_t.C_t) into G_t B_t for dx and x.(G_t B_t).
// XCONV (MODE 0): each direction's stages read its own scan input xs[d]
// (the directions' convolved x), and the skip D x is added from x itself in
// the epilogue.
template <typename T, int N, int HT, bool SF32, int MODE, bool XCONV = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? (MODE == 0 ? (SF32 ? 1 : 4) : 4) : 1)))
void k3_chunk_out(ScanArgs a) {
  using Sm = K3Lds<T, N, HT>;
  using PF = K3Pf<T, N, HT, SF32>;
  constexpr int NG = PF::NG;
  using SX = typename PF::SX;
  using SS = typename PF::SS;
  using SSrc = typename std::conditional<SF32, float, T>::type;
  constexpr int IH = PF::IH;
  constexpr bool DAI = MODE == 1;  // the within-chunk dA product
  __shared__ Sm sm;
  // MODE 1: in-chunk cumulative dt of every token, per (direction, head)
  __shared__ __attribute__((aligned(16))) float smcdt[DAI ? 2 : 1][HT][DAI ? kQmax : 4];
  // MODE 1 (one head per workgroup): the row-block's dy rows, staged once
  // and read by both slots' epilogues in the accumulators' layout.  Row
  // pitch 68 elements: the reads (lane rows 4 apart, 16 consecutive
  // columns) meet distinct banks, and the rows stay 8-byte aligned for the
  // staging writes.
  constexpr int kDyP = 68;
  __shared__ __attribute__((aligned(16))) T sdy[MODE == 1 ? kRB : 1][MODE == 1 ? kDyP : 4];
  constexpr int NK = N / 32;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int Q = a.chunk, NRB = Q / kRB, H = a.H, G = a.G;
  const int64_t L = a.L;
  // work item = ((b * nchunks + c) * NRB + j) * (H / HT) + head tile, so all
  // workgroups of one chunk run back to back on one XCD
  uint32_t bx = (uint32_t)xcd_linear_id(blockIdx.x, gridDim.x), rem;
  bx = a.fd_tiles.divmod(bx, rem);
  const int h0 = (int)rem * HT;
  const int j = (int)(bx & (uint32_t)(NRB - 1));  // NRB is 1, 2 or 4
  bx >>= __builtin_ctz((unsigned)NRB);
  bx = a.fd_nc.divmod(bx, rem);
  // the interior chunks of a batch row first, its two edge chunks (one carry-in
  // direction each, so cheaper) last, so that a last partial round of
  // workgroups is made of the cheaper ones
  const int nc = a.nchunks, cp = (int)rem;
  const int c = nc < 3 ? cp : (cp < nc - 2 ? cp + 1 : (cp == nc - 2 ? 0 : nc - 1));
  const int b = (int)bx;
  const int64_t t0 = (int64_t)c * Q;
  const int qlen = (int)((L - t0) < Q ? (L - t0) : Q);
  if (j * kRB >= qlen) return;
  const int gidx = (int)a.fd_hpg.div((uint32_t)h0);
  constexpr uint32_t ES = sizeof(T);
  // one buffer per batch row: tokens past L read as zero
  const bufres rX = make_buf(reinterpret_cast<const T *>(a.x) + (int64_t)b * L * H * kP,
                             (uint32_t)(L * H * kP * ES));
  // the stages' x per slot: the directions' scan inputs with XCONV
  const bufres rXs[2] = {
      XCONV && a.xs[0] ? make_buf(reinterpret_cast<const T *>(a.xs[0]) + (int64_t)b * L * H * kP, (uint32_t)(L * H * kP * ES)) : rX,
      XCONV && a.xs[1] ? make_buf(reinterpret_cast<const T *>(a.xs[1]) + (int64_t)b * L * H * kP, (uint32_t)(L * H * kP * ES)) : rX};
  const bufres rC[2] = {
      make_buf(reinterpret_cast<const T *>(a.C[0]) + (int64_t)b * L * G * N, (uint32_t)(L * G * N * ES)),
      make_buf(reinterpret_cast<const T *>(a.C[1]) + (int64_t)b * L * G * N, (uint32_t)(L * G * N * ES))};
  const uint32_t xrs_b = (uint32_t)(H * kP * ES);
  // this wave's Gram tiles (16-row tile 4 j + w), s-block k at + k * 64 vectors
  const int64_t gslot = (int64_t)a.Z * a.nchunks * G * Q * Q * NG / 16;
  const u32x4 *gt0 = reinterpret_cast<const u32x4 *>(a.gram) +
                     (((int64_t)b * a.nchunks + c) * G + gidx) * (int64_t)Q * Q * NG / 16 +
                     (int64_t)(4 * j + w) * NRB * 64 * NG + lane;
  const uint32_t xoff = (uint32_t)(t0 * H + h0) * kP * ES;
  const int klast = (qlen - 1) / kRB;
  // carry-in terms that can be nonzero: slot 0's carry starts from zero at
  // chunk 0 (the forward scan unless it continues from an initial state;
  // the reverse direction's adjoint in the dx pass), slot 1's at the last
  // chunk (the reverse scan; the forward direction's adjoint)
  // Block-segmented reverse: the slot that carries the reverse direction
  // (slot 1; slot 0 in the dx pass) takes only the s-blocks of the row-block's
  // reverse block, and no carry-in across a block boundary (the reverse's
  // own carry crosses chunk boundary c + 1, its adjoint chunk boundary c).
  constexpr int RSLOT = MODE == 2 ? 0 : 1;
  const int segt = a.rseg_tiles;  // 0, 1 or 2
  const int kseg0 = segt ? (j & ~(segt - 1)) : 0;
  const int kseg1 = segt ? min(kseg0 + segt - 1, klast) : klast;
  const int kf0 = RSLOT == 0 ? kseg0 : 0;      // slot 0's first s-block
  const int kr0 = RSLOT == 1 ? kseg1 : klast;  // slot 1's first s-block
  const bool cut = a.rseg_chunks > 0 && (RSLOT == 0 ? c : c + 1) % a.rseg_chunks == 0;
  const bool has_in0 = a.sin[0] != nullptr && (c > 0 || (MODE != 2 && a.init_state != nullptr)) &&
                       !(RSLOT == 0 && cut);
  const bool has_in1 = a.sin[1] != nullptr && c < a.nchunks - 1 && !(RSLOT == 1 && cut);

  u32x4 pf[PF::NPF];
  auto prefetch_sblock = [&](int d, int k) __attribute__((always_inline)) {
    const uint32_t s0 = k * kRB;
    const u32x4 *gp = gt0 + d * gslot + k * 64 * NG;
#pragma unroll
    for (int u = 0; u < NG; ++u) pf[u] = gp[u * 64];
#pragma unroll
    for (int hh = 0; hh < HT; ++hh)
      SX::prefetch(pf + NG + hh * SX::NV, d ? rXs[1] : rXs[0], xoff + s0 * xrs_b + hh * kP * ES, xrs_b);
  };
  // carry-in states of heads ih*IH .. ih*IH + IH - 1
  auto prefetch_state = [&](int d, int ih) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < IH; ++q) {
      const int64_t off = (int64_t)b * a.sin_bstride[d] + (int64_t)c * a.sin_cstride[d] +
                          (int64_t)(h0 + ih * IH + q) * kP * N;
      SS::prefetch(pf + q * SS::NV, reinterpret_cast<const SSrc *>(a.sin[d]) + off);
    }
  };
  // ---- decay scans (forward prefix and reverse suffix) for the whole
  // chunk, wave w taking (direction w / HT, head w % HT).  The dt loads go
  // out first, raw and unconditional (tokens past L read as zero), then the
  // first stage's loads, so neither waits for the other.
  static_assert(2 * HT <= kThreads / 64, "one decay scan per wave");
  // MODE 1: the row-block's dy rows (aux), in 16-byte pieces (rows past the
  // end read as zero), go out before everything else and reach LDS at the
  // end of the prologue, where the epilogues find them.  (MODE 2 reads its
  // epilogue rows from global memory there, x from aux and dy from x.)
  constexpr int kDyV = (kRB * kP * (int)ES / 16) / kThreads;  // pieces per thread
  const int64_t rowel = (int64_t)L * H * kP;  // elements of one batch row's [L][H][P]
  const bufres rXa = make_buf(reinterpret_cast<const T *>(a.aux) + (int64_t)b * rowel, (uint32_t)(rowel * ES));
  u32x4 dyraw[MODE == 1 ? kDyV : 1];
  if constexpr (MODE == 1) {
#pragma unroll
    for (int m = 0; m < kDyV; ++m) {
      const int it = tid + m * kThreads, r = it / (kP * (int)ES / 16), pc = it % (kP * (int)ES / 16);
      dyraw[m] = bload16(rXa, (uint32_t)(((t0 + j * kRB + r) * H + h0) * kP) * ES + 16u * pc);
    }
  }
  const int pd = w / HT, ph = w % HT;
  uint32_t dtraw[4], cdraw[kQmax / kRB];
  float Ah = 0.0f;
  DtPost post;
  if (w < 2 * HT) {
    chunk_dt_bload<T>(make_buf(reinterpret_cast<const T *>(a.dt[pd]) + (int64_t)b * L * H, (uint32_t)(L * H * ES)),
                      (uint32_t)(t0 * H + h0 + ph) * ES, (uint32_t)(H * ES), Q, dtraw);
    Ah = a.A[pd][h0 + ph];
    post = dt_post_of(a, pd, h0 + ph);
    if constexpr (DAI) {
      // token m 64 + lane of the chunk; past L reads as zero
      const bufres rc = make_buf(a.cdt_in + (((int64_t)pd * a.Z + b) * H + h0 + ph) * L, (uint32_t)(L * 4));
#pragma unroll
      for (int m = 0; m < kQmax / kRB; ++m)
        cdraw[m] = __builtin_amdgcn_raw_buffer_load_b32(rc, (uint32_t)(t0 + m * kRB + lane) * 4u, 0, 0);
    }
  }
  prefetch_sblock(0, kf0);
  if (w < 2 * HT) {
    // the empty asm keeps the decode (and so the wait for the dt loads)
    // behind the stage loads above
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(dtraw[i]) : : "memory");
    asm volatile("" : "+v"(Ah) : : "memory");
    if constexpr (DAI) {
#pragma unroll
      for (int m = 0; m < kQmax / kRB; ++m) {
        asm volatile("" : "+v"(cdraw[m]) : : "memory");
        if (m * kRB < Q) smcdt[pd][ph][m * kRB + lane] = __builtin_bit_cast(float, cdraw[m]);
      }
    }
    float dv[4];
    chunk_dt_decode<T>(dtraw, Q, dv, post, qlen);
    const float am = chunk_decay_scan_vals(dv, Q, Ah * kLog2e, pd == 1, sm.lam[pd][ph],
                                           sm.scale[pd][ph], MODE == 2);
    // The same wave (its LDS accesses complete in order) then forms this
    // pair's references and column factors: the row-block reference m
    // (forward: lam at the token before the row-block; reverse: rho at the
    // token after it), dt of the diagonal block, and for every token s the
    // factor dt_s 2^(ref - lam_s) (no dt in the dx pass), ref = m off the
    // diagonal block and the 16-token tile's end (forward) or start
    // (reverse) on it.
    const float *lm = sm.lam[pd][ph];
    float *sc = sm.scale[pd][ph];
    const float rb = pd == 0 ? (j > 0 ? lm[j * kRB - 1] : 0.0f) : ((j + 1) * kRB < Q ? lm[(j + 1) * kRB] : 0.0f);
    if (lane == 0) {
      sm.amax[pd][ph] = am;
      sm.refb[pd][ph] = rb;
    }
    sm.dtd[pd][ph][lane] = sc[j * kRB + lane];
#pragma unroll
    for (int m = 0; m < kQmax / kRB; ++m) {
      if (m * kRB >= Q) break;
      const int s2 = m * kRB + lane;
      const float ref = m == j ? (pd == 0 ? lm[s2 | 15] : lm[s2 & ~15]) : rb;
      const float dv = sc[s2];
      const float e = exp2_fast(ref - lm[s2]);
      sc[s2] = MODE == 2 ? e : (dv != 0.0f ? dv * e : 0.0f);
    }
  }

  // C rows of this wave (operand of the carry-in product), loaded per
  // direction; rows past the sequence end read as zero
  const int trow = j * kRB + 16 * w + r16;
  auto load_c = [&](int d, Frag<T> (&cfd)[NK]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      frag_bload(cfd[ks], rC[d], (uint32_t)((t0 + trow) * G + gidx) * N * ES + (32 * ks + 8 * g4) * ES);
  };
  if constexpr (MODE == 1) {
#pragma unroll
    for (int m = 0; m < kDyV; ++m) {
      const int it = tid + m * kThreads, r = it / (kP * (int)ES / 16), pc = it % (kP * (int)ES / 16);
      uint2 *dst = reinterpret_cast<uint2 *>(reinterpret_cast<char *>(&sdy[r][0]) + 16 * pc);
      dst[0] = uint2{dyraw[m][0], dyraw[m][1]};
      dst[1] = uint2{dyraw[m][2], dyraw[m][3]};
    }
  }
  __syncthreads();

  // The factored diagonal slab multiplies by 2^(lam_t - lam_end) <= 2^(15 max|a|)
  // on one side; chunks whose decays could overflow that take the exact
  // per-element path instead (column factor 1, full 2^(lam_t - lam_s) dt_s
  // per element).
  bool exact = false;
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) exact = exact || (sm.amax[d][hh] >= 8.0f);

  f32x4 acc[HT][4], acc2[DAI ? HT : 1][4];
#pragma unroll
  for (int hh = 0; hh < HT; ++hh)
#pragma unroll
    for (int v = 0; v < 4; ++v) zero4(acc[hh][v]);
#pragma unroll
  for (int hh = 0; hh < (DAI ? HT : 1); ++hh)
#pragma unroll
    for (int v = 0; v < 4; ++v) zero4(acc2[hh][v]);

  // one direction; D is a compile-time constant so every register array
  // (C fragments, masks, accumulators) is indexed statically
  auto run_direction = [&](auto dc) __attribute__((always_inline)) {
    constexpr int d = decltype(dc)::value;
    // MODE 0 prefetches the reverse's first slab during the forward's last
    // stage; the backward modes finish each slot with an epilogue first and
    // issue it here, so the prefetch registers are not live across it
    if (MODE != 0 && d == 1) prefetch_sblock(1, kr0);
    // per-head row factor 2^(lam_t - m) of this lane's Gram row t = 16w + r16,
    // applied to C.B^T together with the column factors
    float ut[HT], trow[HT];
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) {
      ut[hh] = exp2_fast(sm.lam[d][hh][j * kRB + 16 * w + r16] - sm.refb[d][hh]);
      trow[hh] = 0.0f;
      if constexpr (DAI) trow[hh] = smcdt[d][hh][j * kRB + 16 * w + r16];
    }
    // ---------------- s-blocks of direction d.  One stage: commit the
    // staged x, turn this wave's Gram tile into the masked, decay-weighted
    // operand mf (so the prefetch registers are free again), issue the next
    // stage's loads, then multiply with x from LDS.  Both directions visit
    // their off-diagonal s-blocks first (forward: 0 .. j - 1; reverse:
    // kr0 down to j + 1) and the diagonal one (k = j) last, as an instance
    // of its own: inside the loop the next stage is always an s-block, whose
    // loads go to the same registers.
    auto stage = [&](int k, auto diagc) __attribute__((always_inline)) {
      constexpr bool DIAG = decltype(diagc)::value;
      const int s0 = k * kRB;
      int ulo = 0, uhi = 3;
      if (DIAG) {
        if (d == 0) uhi = w;
        else ulo = w;
      }
      __syncthreads();
      // cb[u]: lane holds (C.B^T)[t = 16w + r16][s = 16u + 4 g4 + i]
      f32x4 cb[4];
      GramIO<T>::get(cb, pf);
#pragma unroll
      for (int hh = 0; hh < HT; ++hh) SX::commit(&sm.u.s.Xs[hh][0][0], pf + NG + hh * SX::NV);
      // column factors (the staged operand's per-token scale) of this lane's
      // 16 columns s = s0 + 16 u + 4 g4 + i
      auto col_scale = [&](int hh, f32x4 (&sc)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          sc[u] = *reinterpret_cast<const f32x4 *>(&sm.scale[d][hh][s0 + 16 * u + 4 * g4]);
      };
      Frag<T> mf[HT][2], mf2[DAI ? HT : 1][2];
      // MODE 1: the same operand times (T_t - T_s), T_s of this lane's 16
      // columns read as the column factors are
      auto dai_frag = [&](int hh, int q, const float (&m)[8]) __attribute__((always_inline)) {
        if constexpr (DAI) {
          const f32x4 ta = *reinterpret_cast<const f32x4 *>(&smcdt[d][hh][s0 + 32 * q + 4 * g4]);
          const f32x4 tb = *reinterpret_cast<const f32x4 *>(&smcdt[d][hh][s0 + 32 * q + 16 + 4 * g4]);
          float m2[8];
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) {
            m2[i2] = m[i2] * (trow[hh] - ta[i2]);
            m2[4 + i2] = m[4 + i2] * (trow[hh] - tb[i2]);
          }
          frag_from(mf2[hh][q], m2);
        }
      };
      if constexpr (!DIAG) {
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          f32x4 sc[4];
          col_scale(hh, sc);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            float m[8];
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
              m[i2] = cb[2 * q][i2] * (ut[hh] * sc[2 * q][i2]);
              m[4 + i2] = cb[2 * q + 1][i2] * (ut[hh] * sc[2 * q + 1][i2]);
            }
            frag_from(mf[hh][q], m);
            dai_frag(hh, q, m);
          }
        }
      } else {
        if (MODE == 2 && g4 == (r16 >> 2)) {
          // this lane holds the diagonal (row t = 16w + r16, column s = t)
          float v = 0.0f;
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2)
              if (u == w && i2 == (r16 & 3)) v = cb[u][i2];
          sm.bcd[d][16 * w + r16] = v;
        }
        // this lane's mask on the diagonal 16 x 16 tile (u == w): causal
        // side of the direction, strict in the backward modes
        bool lm[4];
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int sc = 4 * g4 + i2;
          lm[i2] = MODE == 0 ? (d == 0 ? sc <= r16 : sc >= r16) : (d == 0 ? sc < r16 : sc > r16);
        }
        // masked positions are selected away, never multiplied by a 0/1
        // mask: a large factor must not meet a 0 as 0 * inf.  Tiles u outside
        // [ulo, uhi] get the factor 0 (C.B^T is finite).
        if (!exact) {
#pragma unroll
          for (int hh = 0; hh < HT; ++hh) {
            const float lt = sm.lam[d][hh][s0 + 16 * w + r16];
            float f[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float ru = d == 0 ? sm.lam[0][hh][s0 + 16 * u + 15] : sm.lam[1][hh][s0 + 16 * u];
              const float fu = exp2_fast(fminf(lt - ru, 120.0f));
              f[u] = (u >= ulo && u <= uhi) ? fu : 0.0f;
            }
            f32x4 sc[4];
            col_scale(hh, sc);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              if (2 * q + 1 < ulo || 2 * q > uhi) continue;
              float m[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int u = 2 * q + (e >> 2), i2 = e & 3;
                const float v = cb[u][i2] * (f[u] * sc[u][i2]);
                m[e] = (u == w && !lm[i2]) ? 0.0f : v;
              }
              frag_from(mf[hh][q], m);
              dai_frag(hh, q, m);
            }
          }
        } else {
          // exact per-element weights 2^(lam_t - lam_s) dt_s (column factor 1)
#pragma unroll
          for (int hh = 0; hh < HT; ++hh) {
            const float lt = sm.lam[d][hh][s0 + 16 * w + r16];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              if (2 * q + 1 < ulo || 2 * q > uhi) continue;
              float m[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int u = 2 * q + (e >> 2), i2 = e & 3;
                const int sl = 16 * u + 4 * g4 + i2;
                const float wgt = exp2_fast(fminf(lt - sm.lam[d][hh][s0 + sl], 0.0f)) *
                                  (MODE == 2 ? 1.0f : sm.dtd[d][hh][sl]);
                const bool ok = (u >= ulo && u <= uhi) && !(u == w && !lm[i2]);
                m[e] = ok ? cb[u][i2] * wgt : 0.0f;
              }
              frag_from(mf[hh][q], m);
              dai_frag(hh, q, m);
            }
          }
        }
      }
      __syncthreads();
      if (!DIAG) prefetch_sblock(d, d == 0 ? k + 1 : k - 1);
      else if (d == 0 ? has_in0 : has_in1) prefetch_state(d, 0);
      else if (d == 0 && MODE == 0) prefetch_sblock(1, kr0);
#pragma unroll
      for (int hh = 0; hh < HT; ++hh)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          if (DIAG && (2 * q + 1 < ulo || 2 * q > uhi)) continue;
          Frag<T> xf[4];
#pragma unroll
          for (int v = 0; v < 4; ++v)
            frag_rows(xf[v], &sm.u.s.Xs[hh][0][0], Sm::XPT, 32 * q + 4 * g4, 32 * q + 16 + 4 * g4, 16 * v);
          if constexpr (MODE == 0 && DIAG && d == 0 && !XCONV) {
            // the skip D x: on the diagonal s-block, fragment q = w / 2 holds
            // x at this lane's own accumulator positions (rows 16 w + 4 g4 +
            // i, column 16 v + r16), in its low (even w) or high (odd w) half
            // (frag_half selects whole registers: a per-element index would
            // compile to a selection chain over all eight values)
            if (q == (w >> 1)) {
              const float Dh = a.D[h0 + hh];
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                float xh[4];
                frag_half(xf[v], (w & 1) != 0, xh);
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) acc[hh][v][i2] += Dh * xh[i2];
              }
            }
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) mma(acc[hh][v], mf[hh][q], xf[v]);
          if constexpr (DAI)
#pragma unroll
            for (int v = 0; v < 4; ++v) mma(acc2[hh][v], mf2[hh][q], xf[v]);
        }
    };
    if constexpr (d == 0) {
      for (int k = kf0; k < j; ++k) stage(k, std::false_type{});
    } else {
      for (int k = kr0; k > j; --k) stage(k, std::false_type{});
    }
    stage(j, std::true_type{});
    // ---------------- carry-in term 2^lam_t C S_in^T, one head per stage.
    // The states are staged as stored; the row factor 2^lam_t (<= 1) is
    // applied to a transient accumulator per head.
    if (d == 0 ? has_in0 : has_in1) {
      Frag<T> cfd[NK];
      load_c(d, cfd);
#pragma unroll
      for (int ih = 0; ih < HT / IH; ++ih) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < IH; ++q) {
          if constexpr (SF32) SS::commit(&sm.u.Sst[q][0][0], pf + q * SS::NV, 1.0f);
          else SS::commit_raw(&sm.u.Sst[q][0][0], pf + q * SS::NV);
        }
        __syncthreads();
        if (ih + 1 < HT / IH) prefetch_state(d, ih + 1);
        else if (d == 0 && MODE == 0) prefetch_sblock(1, kr0);
#pragma unroll
        for (int q = 0; q < IH; ++q) {
          const int hh = ih * IH + q;
          f32x4 t2[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) zero4(t2[v]);
#pragma unroll
          for (int ks = 0; ks < NK; ++ks) {
            Frag<T> sf[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) frag_ld8(sf[v], &sm.u.Sst[q][16 * v + r16][32 * ks + 8 * g4]);
#pragma unroll
            for (int v = 0; v < 4; ++v) mma(t2[v], cfd[ks], sf[v]);
          }
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) {
            const int tr = j * kRB + 16 * w + 4 * g4 + i2;
            const float et = exp2_fast(sm.lam[d][hh][tr]);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[hh][v][i2] += et * t2[v][i2];
            if constexpr (DAI) {
              // the carried state's part of dA: T_t 2^lam_t C_t S_in, whose
              // dot with dy summed over the chunk is <sum_t 2^lam_t T_t dy_t
              // (outer) C_t, S_in>, the tangent-weighted adjoint chunk state
              // against the carry-in
              const float tt = smcdt[d][hh][tr] * et;
#pragma unroll
              for (int v = 0; v < 4; ++v) acc2[hh][v][i2] += tt * t2[v][i2];
            }
          }
        }
      }
    }
  };
  if constexpr (MODE == 0) {
    run_direction(std::integral_constant<int, 0>{});
    run_direction(std::integral_constant<int, 1>{});

    // y = acc (the skip D x was added on the forward diagonal s-block; with
    // XCONV it is added below).
    // Each wave stages its own 16 rows through LDS, one head at a time, so
    // that every lane writes 16 contiguous bytes; a wave's LDS accesses
    // complete in order and no other wave touches those rows, so the only
    // barrier is the one that frees the shared region.
    __syncthreads();
    float *ow = &sm.u.Out[0][16 * w][0];
    const int rr = lane >> 2, pc = (lane & 3) * 16;  // row of the wave's 16, first of 16 columns
    const bool rvalid = j * kRB + 16 * w + rr < qlen;
    T *yg = reinterpret_cast<T *>(a.y) + (((int64_t)b * L + t0 + j * kRB + 16 * w + rr) * H + h0) * kP + pc;
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) ow[(4 * g4 + i2) * Sm::OP + 16 * v + r16] = acc[hh][v][i2];
      float o0[8], o1[8];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const f32x4 lo = *reinterpret_cast<const f32x4 *>(&ow[rr * Sm::OP + pc + 8 * m]);
        const f32x4 hi = *reinterpret_cast<const f32x4 *>(&ow[rr * Sm::OP + pc + 8 * m + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          (m ? o1 : o0)[e] = lo[e];
          (m ? o1 : o0)[4 + e] = hi[e];
        }
      }
      if (rvalid) {
        if constexpr (XCONV) {
          // the skip D x from x itself (the stages held the convolved x)
          const T *xr = reinterpret_cast<const T *>(a.x) +
                        (((int64_t)b * L + t0 + j * kRB + 16 * w + rr) * H + h0 + hh) * kP + pc;
          float x0[8], x1[8];
          gload8(x0, xr);
          gload8(x1, xr + 8);
          const float Dh = a.D[h0 + hh];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            o0[e] += Dh * x0[e];
            o1[e] += Dh * x1[e];
          }
        }
        gstore8(yg + hh * kP, o0);
        gstore8(yg + hh * kP + 8, o1);
      }
    }
  } else {
    // Backward modes: each slot's accumulator is finished on its own.
    // MODE 1 (one head per workgroup): dy . y_d per row and the within-chunk
    // dA partial straight from the accumulators, whose lane (r16, g4) of
    // wave w holds rows 16 w + 4 g4 + i2, columns 16 v + r16: dy is read
    // from LDS in that layout, each row's dot product is summed over its 16
    // lanes by DPP, and the dA partial needs no per-row sum at all.
    auto ydot_epilogue = [&](auto dc) __attribute__((always_inline)) {
      constexpr int d = decltype(dc)::value;
      static_assert(HT == 1, "one head per workgroup");
      float part[4], dsum = 0.0f;
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const int r = 16 * w + 4 * g4 + i2;
        float pa = 0.0f, pb = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float dv = to_f(sdy[r][16 * v + r16]);
          pa += acc[0][v][i2] * dv;
          if constexpr (DAI) pb += acc2[0][v][i2] * dv;
        }
        part[i2] = pa;
        if (j * kRB + r < qlen) dsum += pb;
      }
      // row sums: inclusive sums over the 16 lanes of each lane row
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        float v = part[i2];
        v += dpp_f<0x111>(v);
        v += dpp_f<0x112>(v);
        v += dpp_f<0x114>(v);
        v += dpp_f<0x118>(v);
        part[i2] = v;
      }
      const int sd = a.slot_dir[d];
      if (r16 == 15) {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          const int r = j * kRB + 16 * w + 4 * g4 + i2;
          if (r < qlen) a.out0[(((int64_t)sd * a.Z + b) * L + t0 + r) * H + h0] = part[i2];
        }
      }
      // the within-chunk dA partial of this row-block, reduced in a fixed order
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) dsum += __shfl_xor(dsum, o, 64);
      if (lane == 0) sm.red[w][0] = dsum;
      __syncthreads();
      if (tid == 0)
        a.dai_out[((((int64_t)sd * a.Z + b) * a.nchunks + c) * NRB + j) * H + h0] =
            (sm.red[0][0] + sm.red[1][0]) + (sm.red[2][0] + sm.red[3][0]);
#pragma unroll
      for (int v = 0; v < 4; ++v) zero4(acc2[0][v]);
    };
    // MODE 2: each head's accumulator is staged through LDS; 8 consecutive
    // lanes hold one row (8 elements each) and reduce their dot products
    // with shuffles.
    float ddp[HT];
#pragma unroll
    for (int hh = 0; hh < HT; ++hh) ddp[hh] = 0.0f;
    // The epilogue's global inputs of one head: per row pass m2 the 8
    // elements from p0 of row r of the x rows (aux) and of the dy rows.  The
    // input rows come raw through buffer loads (rows past the sequence end
    // read as zero, no branch); each head's are issued before the previous
    // head is finished, so their latency overlaps that work instead of
    // following it.
    constexpr int NRV = sizeof(T) == 2 ? 1 : 2;  // 16-byte pieces of 8 elements
    constexpr int NM2 = (kRB * 8) / kThreads;
    struct EpiRows {
      u32x4 v[NM2][NRV], dy[NM2][NRV];
    };
    // MODE 2: slot 0's part of dx (D dy + dt G B of its direction) for this
    // thread's 8 elements of each row pass and head, kept in registers until
    // slot 1 adds its own and writes dx once
    float dxk[MODE == 2 ? HT : 1][NM2][8];
    const bufres rAux = rXa;
    auto epi_off = [&](int hh, int m2) __attribute__((always_inline)) {
      const int it = tid + m2 * kThreads;
      const int r = it >> 3, p0 = (it & 7) * 8;
      return (uint32_t)(((t0 + j * kRB + r) * H + h0 + hh) * kP + p0);  // element offset in the row
    };
    auto epi_load = [&](int hh, EpiRows &e) __attribute__((always_inline)) {
#pragma unroll
      for (int m2 = 0; m2 < NM2; ++m2) {
        const uint32_t eo = epi_off(hh, m2);
#pragma unroll
        for (int k = 0; k < NRV; ++k) e.v[m2][k] = bload16(rAux, eo * ES + 16 * k);
#pragma unroll
        for (int k = 0; k < NRV; ++k) e.dy[m2][k] = bload16(rX, eo * ES + 16 * k);
      }
    };
    auto raw8 = [&](const u32x4 (&r)[NRV], float (&o)[8]) __attribute__((always_inline)) {
      if constexpr (sizeof(T) == 2) {
        unpack16(o, r[0], (const bf16 *)nullptr);
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (an element of a vector type is copied out before the bit cast:
            // a bit cast of the element itself reads the vector's first one)
            const uint32_t u = r[k][e];
            o[4 * k + e] = __builtin_bit_cast(float, u);
          }
      }
    };
    auto dx_epilogue = [&](auto dc) __attribute__((always_inline)) {
      constexpr int d = decltype(dc)::value;
      const int sd = a.slot_dir[d];
      EpiRows nxt;
      epi_load(0, nxt);
#pragma unroll
      for (int ih = 0; ih < HT / IH; ++ih) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < IH; ++q)
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2)
              sm.u.Out[q][16 * w + 4 * g4 + i2][16 * v + r16] = acc[ih * IH + q][v][i2];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < IH; ++q) {
          const int hh = ih * IH + q;
          const EpiRows cur = nxt;
          if (hh + 1 < HT) epi_load(hh + 1, nxt);
#pragma unroll
          for (int m2 = 0; m2 < NM2; ++m2) {
            const int it = tid + m2 * kThreads;
            const int r = it >> 3, p0 = (it & 7) * 8;
            const int64_t tok = t0 + j * kRB + r;
            const bool valid = j * kRB + r < qlen;
            float o[8], v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = sm.u.Out[q][r][p0 + e];
            raw8(cur.v[m2], v);
            float part = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) part += o[e] * v[e];
            part += __shfl_xor(part, 1, 64);
            part += __shfl_xor(part, 2, 64);
            part += __shfl_xor(part, 4, 64);
            const int64_t oix = (((int64_t)sd * a.Z + b) * L + tok) * H + h0 + hh;
            {
              // part = x.(G_t B_t) without t' = t; add dy_t (B_t.C_t)
              const float dtr = sm.dtd[d][hh][r], bc = sm.bcd[d][r];
              float *dxp = a.out1 + (((int64_t)b * L + tok) * H + h0 + hh) * kP + p0;
              float dyv[8], dxo[8];
              raw8(cur.dy[m2], dyv);
              float pin = 0.0f;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                o[e] += bc * dyv[e];
                pin += o[e] * v[e];
              }
              pin += __shfl_xor(pin, 1, 64);
              pin += __shfl_xor(pin, 2, 64);
              pin += __shfl_xor(pin, 4, 64);
              if ((tid & 7) == 0 && valid) {
                a.out0[oix] = pin;
                a.out3[oix] = part;
              }
              if (d == 0) {
                const float Dh = a.D[h0 + hh];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  dxk[hh][m2][e] = Dh * dyv[e] + dtr * o[e];
                  ddp[hh] += dyv[e] * v[e];
                }
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) dxo[e] = dxk[hh][m2][e] + dtr * o[e];
                if (valid) gstore8(dxp, dxo);
              }
            }
          }
        }
      }
      if constexpr (d == 0) {
        // dy.x of this row-block, per head, in a fixed order
#pragma unroll
        for (int hh = 0; hh < HT; ++hh) {
          float v = ddp[hh];
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
          if (lane == 0) sm.red[w][hh] = v;
        }
        __syncthreads();
        if (tid < HT)
          a.out2[(((int64_t)b * a.nchunks + c) * NRB + j) * H + h0 + tid] =
              (sm.red[0][tid] + sm.red[1][tid]) + (sm.red[2][tid] + sm.red[3][tid]);
      }
    };
    run_direction(std::integral_constant<int, 0>{});
    if constexpr (MODE == 1) ydot_epilogue(std::integral_constant<int, 0>{});
    else dx_epilogue(std::integral_constant<int, 0>{});
#pragma unroll
    for (int hh = 0; hh < HT; ++hh)
#pragma unroll
      for (int v = 0; v < 4; ++v) zero4(acc[hh][v]);
    run_direction(std::integral_constant<int, 1>{});
    if constexpr (MODE == 1) ydot_epilogue(std::integral_constant<int, 1>{});
    else dx_epilogue(std::integral_constant<int, 1>{});
  }
}

// ============================================================= launchers

template <typename T, int N, int HT>
static void launch_t(const ScanArgs &a, int phase, hipStream_t st) {
  if (phase == PHASE_CHUNK_STATE || phase == PHASE_ADJ_STATE || phase == PHASE_TAN_STATE) {
    dim3 g((unsigned)(a.Z * a.nchunks * a.ndir * (a.H / HT)));
    if (phase == PHASE_CHUNK_STATE)
      launch_kernel((k1_chunk_state<T, N, HT, 0>), g, dim3(kThreads), 0, st, a);
    else if (phase == PHASE_ADJ_STATE)
      launch_kernel((k1_chunk_state<T, N, HT, 1>), g, dim3(kThreads), 0, st, a);
    else
      launch_kernel((k1_chunk_state<T, N, HT, 2>), g, dim3(kThreads), 0, st, a);
  } else if (phase == PHASE_GRAM) {
    // one workgroup per (batch, chunk, slot, group, column block), covering
    // the block's row-blocks on the slot's side
    const int nrb = a.chunk / kRB;
    dim3 g((unsigned)((int64_t)a.Z * a.nchunks * 2 * a.G * nrb));
    launch_kernel((k_gram<T, N>), g, dim3(kThreads), 0, st, a);
  } else if (phase == PHASE_TAN_PASS && sizeof(T) == 2) {
    const int PN = kP * N;
    dim3 g2((unsigned)(PN / 8 / kThreads), (unsigned)a.H, (unsigned)(a.Z * 2));
    launch_kernel(k2_tangent_pass8, g2, dim3(kThreads), 0, st, a, PN);
  } else if (phase == PHASE_TAN_PASS) {
    const int PN = kP * N;
    dim3 g2((unsigned)(PN / 4 / kThreads), (unsigned)a.H, (unsigned)(a.Z * 2));
    launch_kernel(k2_tangent_pass<T>, g2, dim3(kThreads), 0, st, a, PN);
  } else if ((phase == PHASE_STATE_PASS || phase == PHASE_ADJ_PASS) && sizeof(T) == 2) {
    const int PN = kP * N;
    dim3 g2((unsigned)(PN / 8 / kThreads), (unsigned)a.H, (unsigned)(a.Z * a.ndir));
    if (phase == PHASE_ADJ_PASS)
      launch_kernel(k2_state_pass8<true>, g2, dim3(kThreads), 0, st, a, PN);
    else
      launch_kernel(k2_state_pass8<false>, g2, dim3(kThreads), 0, st, a, PN);
  } else if (phase == PHASE_STATE_PASS || phase == PHASE_ADJ_PASS) {
    const int PN = kP * N;
    dim3 g2((unsigned)((PN / 4 + kThreads - 1) / kThreads), (unsigned)a.H, (unsigned)(a.Z * a.ndir));
    launch_kernel(k2_state_pass<T>, g2, dim3(kThreads), 0, st, a, PN,
                       phase == PHASE_ADJ_PASS ? 1 : 0);
  } else {
    dim3 g((unsigned)(a.Z * a.nchunks * (a.chunk / kRB) * (a.H / HT)));
    if (phase == PHASE_YDOT || phase == PHASE_DX) {
      // one head per tile (the caller's choice for these passes)
      if constexpr (HT == 1) {
        if (phase == PHASE_YDOT)
          launch_kernel((k3_chunk_out<T, N, 1, false, 1>), g, dim3(kThreads), 0, st, a);
        else
          launch_kernel((k3_chunk_out<T, N, 1, false, 2>), g, dim3(kThreads), 0, st, a);
      }
    } else if (a.xs[0] || a.xs[1]) {
      if (a.sin_f32[0] || a.sin_f32[1])
        launch_kernel((k3_chunk_out<T, N, HT, true, 0, true>), g, dim3(kThreads), 0, st, a);
      else
        launch_kernel((k3_chunk_out<T, N, HT, false, 0, true>), g, dim3(kThreads), 0, st, a);
    } else if (a.sin_f32[0] || a.sin_f32[1])
      launch_kernel((k3_chunk_out<T, N, HT, true, 0>), g, dim3(kThreads), 0, st, a);
    else
      launch_kernel((k3_chunk_out<T, N, HT, false, 0>), g, dim3(kThreads), 0, st, a);
  }
}

template <typename T, int N>
static void launch_n(const ScanArgs &a, int phase, hipStream_t st, int HT) {
  if (HT == 2) launch_t<T, N, 2>(a, phase, st);
  else launch_t<T, N, 1>(a, phase, st);
}

bool gram_in_k1(int H, int G, int chunk) {
  const int hpg = H / G, HT = hpg % 2 == 0 ? 2 : 1, nrb = chunk / kRB;
  return hpg / HT >= nrb * (nrb + 1) / 2;
}

// Compute units of the current device (queried once per device; 0 if the
// query fails).
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

hipError_t launch_scan_phase(const ScanArgs &args, int phase, hipStream_t st) {
  // Heads of one tile share their B/C group: 2 heads when the heads per
  // group are even, else 1.  The dy.y_d pass (two products per stage) takes
  // one head per tile: with two, its accumulators leave too few registers
  // for four waves per SIMD without spilling.  So does the dx pass, whose
  // first slot's part of dx waits in registers for the second: with two
  // heads that takes 218 registers (two waves per SIMD), with one 128
  // (four), and the pass runs faster.  So do the chunk-state and
  // output passes of a problem whose one-head workgroups still run in one
  // round (three per compute unit for the chunk states, four for the
  // output): twice the workgroups, each on a shorter path.  (Whether the
  // chunk-state kernel forms the Gram tiles is decided for two-head tiles,
  // which one-head tiles cover too.)
  const int hpg = args.H / args.G;
  const int64_t ncu = cu_count();
  const int64_t items2 = (int64_t)args.Z * args.nchunks * (args.chunk / kRB) * (args.H / 2);
  const int64_t items1 = (int64_t)args.Z * args.nchunks * args.ndir * (args.H / 2);
  const bool small = (phase == PHASE_CHUNK_OUT && 2 * items2 <= 4 * ncu) ||
                     (phase == PHASE_CHUNK_STATE && 2 * items1 <= 3 * ncu);
  const int HT = (hpg % 2 == 0 && phase != PHASE_YDOT && phase != PHASE_DX && !small) ? 2 : 1;
  ScanArgs a = args;
  const int nrb = a.chunk / kRB;
  a.fd_tiles = FastDiv((uint32_t)(a.H / HT));
  a.fd_nc = FastDiv((uint32_t)a.nchunks);
  a.fd_hpg = FastDiv((uint32_t)hpg);
  a.fd_g = FastDiv((uint32_t)a.G);
  a.fd_pairs = FastDiv((uint32_t)(nrb * (nrb + 1) / 2));
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
