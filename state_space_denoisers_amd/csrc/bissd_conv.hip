// bissd_conv.hip -- the mixer's convolution in front of the scan (gfx950).
//
// Each direction of the bidirectional denoiser is a Mamba-2 layer ("DiffMamba
// Checkpoints", Model details: forward plus flipped-reverse Mamba-2 with
// weight-tied projections), which passes its x through a short causal
// depthwise convolution and a SiLU before the scan.  The directions share the
// pre-convolution x, so one pass reads it once and writes both directions'
// convolved x:
//
//   forward:  xc_f[t][c] = act(b_f[c] + sum_k w_f[c][k] x[t - (K-1) + k][c])
//   reverse:  xc_r[t][c] = act(b_r[c] + sum_k w_r[c][k] x[t + (K-1) - k][c])
//
// (the reverse is the forward convolution of the flipped sequence); bound by
// HBM.
#include <type_traits>

#include "bissd_device.hpp"
#include "bissd_internal.hpp"

namespace bissd {

namespace {

// SiLU on the transcendental unit: z / (1 + e^-z) = z rcp(1 + 2^(-z log2 e)).
// For z very negative 2^(..) overflows to inf and the result is -0 (the
// function's limit); for z very positive it is z.
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-z * kLog2e));
}

// C adjacent channels of one row (C = 2, 4 or 8: one 4- to 16-byte access
// in bf16, 8 to 32 bytes in fp32), as floats
template <int C> struct Vec;
template <> struct Vec<2> { typedef __bf16 b __attribute__((ext_vector_type(2))); typedef float f __attribute__((ext_vector_type(2))); };
template <> struct Vec<4> { typedef __bf16 b __attribute__((ext_vector_type(4))); typedef float f __attribute__((ext_vector_type(4))); };
template <> struct Vec<8> { typedef __bf16 b __attribute__((ext_vector_type(8))); typedef float f __attribute__((ext_vector_type(4))); };

template <int C>
__device__ __forceinline__ void load_ch(float (&o)[C], const bf16 *p) {
  const typename Vec<C>::b v = *reinterpret_cast<const typename Vec<C>::b *>(p);
#pragma unroll
  for (int e = 0; e < C; ++e) o[e] = (float)v[e];
}
template <int C>
__device__ __forceinline__ void load_ch(float (&o)[C], const float *p) {
  constexpr int W = C < 4 ? C : 4;  // floats per access
#pragma unroll
  for (int h = 0; h < C / W; ++h) {
    const typename Vec<W>::f v = *reinterpret_cast<const typename Vec<W>::f *>(p + h * W);
#pragma unroll
    for (int e = 0; e < W; ++e) o[h * W + e] = v[e];
  }
}
template <int C>
__device__ __forceinline__ void store_ch(bf16 *p, const float (&o)[C]) {
  typename Vec<C>::b v;
#pragma unroll
  for (int e = 0; e < C; ++e) v[e] = (bf16)o[e];
  *reinterpret_cast<typename Vec<C>::b *>(p) = v;
}
template <int C>
__device__ __forceinline__ void store_ch(float *p, const float (&o)[C]) {
  constexpr int W = C < 4 ? C : 4;
#pragma unroll
  for (int h = 0; h < C / W; ++h) {
    typename Vec<W>::f v;
#pragma unroll
    for (int e = 0; e < W; ++e) v[e] = o[h * W + e];
    *reinterpret_cast<typename Vec<W>::f *>(p + h * W) = v;
  }
}

}  // namespace

// One thread: the CPL channels c0 .. c0 + CPL - 1 of a run of RUN
// consecutive tokens, both directions.  The run's rows and the K - 1 rows on
// either side are loaded once, all requests issued before any value is used
// and none behind a branch (a row outside the range reads a valid row and is
// then zeroed); consecutive lanes take consecutive channel groups, so a wave
// reads and writes whole row segments, and its taps (channel-major, K per
// channel) are one contiguous block.  Runs start at multiples of RUN (a
// divisor of 64), so a run never straddles a reverse block (a multiple of 64
// tokens): every row at or past min(L, end of the run's reverse block) reads
// as zero, which only the reverse direction's taps can reach.
#ifndef BISSD_CONV_CPL
#define BISSD_CONV_CPL 2
#endif
#ifndef BISSD_CONV_RUN
#define BISSD_CONV_RUN 32
#endif
constexpr int kCpl = BISSD_CONV_CPL;
constexpr int kRun = BISSD_CONV_RUN;
static_assert(64 % kRun == 0 && kCpl >= 2 && kCpl <= 8 && 64 % kCpl == 0, "conv tiling");

template <typename T, int K, int CPL, int RUN>
__global__ __launch_bounds__(256) void k_conv_x(ConvArgs a) {
  constexpr int NR = RUN + 2 * (K - 1);  // rows t0 - (K-1) .. t0 + RUN - 1 + (K-1)
  const int ngrp = a.HP / CPL;
  const int64_t nrun = (a.L + RUN - 1) / RUN;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)a.Z * nrun * ngrp) return;
  const int v = (int)(gid % ngrp);
  const int64_t zr = gid / ngrp;
  const int64_t t0 = (zr % nrun) * RUN;
  const int b = (int)(zr / nrun);
  const int c0 = v * CPL;
  const int64_t HP = a.HP;
  const T *xb = reinterpret_cast<const T *>(a.x) + (int64_t)b * a.L * HP + c0;
  const T *sb = a.state ? reinterpret_cast<const T *>(a.state) + (int64_t)b * (K - 1) * HP + c0 : nullptr;
  const int64_t rend = a.rev_block > 0 ? (t0 / a.rev_block + 1) * a.rev_block : a.L;
  const int64_t lim = rend < a.L ? rend : a.L;
  // row j holds token t0 - (K-1) + j: from x for jlo <= j < jhi, from the
  // state for j < jlo when there is one, else zero
  const int64_t first = t0 - (K - 1);
  const int jlo = first >= 0 ? 0 : (int)(-first);
  const int jhi = (int)((lim - first) < NR ? (lim - first) : NR);
  float row[NR][CPL];
  {
    const T *p = xb + first * HP;  // row 0's address (not read unless valid)
    // rows before the sequence exist only in the first run (t0 = 0, first =
    // -(K-1)), where row j < K-1 is state row j
    const T *q = sb ? sb : xb;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const bool in_x = j >= jlo && j < jhi;
      const bool in_s = j < jlo && sb != nullptr;
      load_ch<CPL>(row[j], in_x ? p : (in_s ? q : xb));
      p += HP;
      q += HP;
    }
  }
  float wv[2][CPL][K], bv[2][CPL];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    // the group's taps: CPL K floats from an offset that is a multiple of 2
    // floats, read as 8-byte pairs
    const float *w = a.w[d] ? a.w[d] + (int64_t)c0 * K : nullptr;
#pragma unroll
    for (int i = 0; i < CPL * K / 2; ++i) {
      typename Vec<2>::f pr = {0.0f, 0.0f};
      if (w) pr = *reinterpret_cast<const typename Vec<2>::f *>(w + 2 * i);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int f = 2 * i + e;  // flat index: channel f / K, tap f % K
        wv[d][f / K][f % K] = pr[e];
      }
    }
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) {
      typename Vec<2>::f bb = {0.0f, 0.0f};
      if (a.b[d]) bb = *reinterpret_cast<const typename Vec<2>::f *>(a.b[d] + c0 + 2 * i);
      bv[d][2 * i] = bb[0];
      bv[d][2 * i + 1] = bb[1];
    }
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const bool keep = (j >= jlo && j < jhi) || (j < jlo && sb != nullptr);
#pragma unroll
    for (int e = 0; e < CPL; ++e) row[j][e] = keep ? row[j][e] : 0.0f;
  }
  const int nst = (int)(a.L - t0 < RUN ? a.L - t0 : RUN);
  auto emit = [&](auto full) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      if (!a.xc[d]) continue;
      T *ob = reinterpret_cast<T *>(a.xc[d]) + ((int64_t)b * a.L + t0) * HP + c0;
      const bool act = a.act[d] != 0;
#pragma unroll
      for (int i = 0; i < RUN; ++i) {
        float o[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) o[e] = bv[d][e];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          // forward tap k reads token t - (K-1) + k (row i + k); reverse tap
          // k reads token t + (K-1) - k (row i + 2(K-1) - k)
          const int j = d == 0 ? i + k : i + 2 * (K - 1) - k;
#pragma unroll
          for (int e = 0; e < CPL; ++e) o[e] += wv[d][e][k] * row[j][e];
        }
        if (act) {
#pragma unroll
          for (int e = 0; e < CPL; ++e) o[e] = silu_f(o[e]);
        }
        if (decltype(full)::value || i < nst) store_ch<CPL>(ob, o);
        ob += HP;
      }
    }
  };
  if (nst == RUN)
    emit(std::true_type{});
  else
    emit(std::false_type{});
}

template <typename T>
__global__ __launch_bounds__(256) void k_conv_state(const T *x, const T *sin, T *sout, int64_t L,
                                                    int Z, int HP, int K) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)Z * HP) return;
  const int c = (int)(gid % HP), b = (int)(gid / HP);
  // row j of [state | x] (the state has K-1 rows)
  auto at = [&](int64_t j) -> T {
    if (j < K - 1) return sin ? sin[((int64_t)b * (K - 1) + j) * HP + c] : from_f<T>(0.0f);
    return x[((int64_t)b * L + (j - (K - 1))) * HP + c];
  };
  T nv[3];
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < K - 1) nv[j] = at(j + L);
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < K - 1) sout[((int64_t)b * (K - 1) + j) * HP + c] = nv[j];
}

hipError_t launch_conv(const ConvArgs &a, hipStream_t st) {
  const int64_t n = (int64_t)a.Z * ((a.L + kRun - 1) / kRun) * (a.HP / kCpl);
  const dim3 g((unsigned)((n + 255) / 256));
#define BISSD_CONV_LAUNCH(TT)                                                           \
  switch (a.K) {                                                                        \
    case 1: launch_kernel((k_conv_x<TT, 1, kCpl, kRun>), g, dim3(256), 0, st, a); break;       \
    case 2: launch_kernel((k_conv_x<TT, 2, kCpl, kRun>), g, dim3(256), 0, st, a); break;       \
    case 3: launch_kernel((k_conv_x<TT, 3, kCpl, kRun>), g, dim3(256), 0, st, a); break;       \
    default: launch_kernel((k_conv_x<TT, 4, kCpl, kRun>), g, dim3(256), 0, st, a); break;      \
  }
  if (a.dtype == 1) {
    BISSD_CONV_LAUNCH(bf16)
  } else {
    BISSD_CONV_LAUNCH(float)
  }
#undef BISSD_CONV_LAUNCH
  return hipGetLastError();
}

hipError_t launch_conv_state(const void *x, const void *state_in, void *state_out, int64_t L,
                             int Z, int HP, int K, int dtype, hipStream_t st) {
  const int64_t n = (int64_t)Z * HP;
  const dim3 g((unsigned)((n + 255) / 256));
  if (dtype == 1)
    launch_kernel(k_conv_state<bf16>, g, dim3(256), 0, st, reinterpret_cast<const bf16 *>(x),
                       reinterpret_cast<const bf16 *>(state_in), reinterpret_cast<bf16 *>(state_out), L, Z, HP, K);
  else
    launch_kernel(k_conv_state<float>, g, dim3(256), 0, st, reinterpret_cast<const float *>(x),
                       reinterpret_cast<const float *>(state_in), reinterpret_cast<float *>(state_out), L, Z, HP, K);
  return hipGetLastError();
}

}  // namespace bissd
