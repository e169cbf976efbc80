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
#include "bissd_device.hpp"
#include "bissd_internal.hpp"

namespace bissd {

namespace {

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace

// One thread: eight channels c0 .. c0 + 7 of a run of kRun consecutive
// tokens, for both directions.  The run's rows and the K - 1 rows on either
// side are loaded once (16-byte vectors, all issued before any is used), the
// taps and biases once per run; consecutive threads take consecutive channel
// vectors of the same rows, so every load and store is coalesced.
constexpr int kRun = 8;
template <typename T, int K>
__global__ __launch_bounds__(256) void k_conv_x(ConvArgs a) {
  constexpr int NR = kRun + 2 * (K - 1);  // rows t0 - (K-1) .. t0 + kRun - 1 + (K-1)
  const int nvec = a.HP / 8;
  const int64_t nrun = (a.L + kRun - 1) / kRun;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)a.Z * nrun * nvec) return;
  const int v = (int)(gid % nvec);
  const int64_t zr = gid / nvec;
  const int64_t t0 = (zr % nrun) * kRun;
  const int b = (int)(zr / nrun);
  const int c0 = v * 8;
  const T *xb = reinterpret_cast<const T *>(a.x) + (int64_t)b * a.L * a.HP + c0;
  const T *sb = a.state ? reinterpret_cast<const T *>(a.state) + (int64_t)b * (K - 1) * a.HP + c0 : nullptr;
  float row[NR][8];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int64_t tj = t0 - (K - 1) + j;
    if (tj >= 0 && tj < a.L) {
      gload8(row[j], xb + tj * a.HP);
    } else if (tj < 0 && sb) {
      gload8(row[j], sb + (tj + (K - 1)) * a.HP);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) row[j][e] = 0.0f;
    }
  }
  // the reverse reads nothing past the end of the run's reverse block (runs
  // never straddle one: reverse blocks are multiples of 64 tokens)
  const int64_t rend = a.rev_block > 0 ? (t0 / a.rev_block + 1) * a.rev_block : a.L;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    if (!a.xc[d]) continue;
    float wv[8][K], bv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int k = 0; k < K; ++k) wv[e][k] = a.w[d][(c0 + e) * K + k];
      bv[e] = a.b[d] ? a.b[d][c0 + e] : 0.0f;
    }
    T *ob = reinterpret_cast<T *>(a.xc[d]) + (int64_t)b * a.L * a.HP + c0;
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const int64_t t = t0 + i;
      if (t >= a.L) break;
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = bv[e];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        // forward tap k reads row t - (K-1) + k (window row i + k); reverse
        // tap k reads row t + (K-1) - k (window row i + 2(K-1) - k)
        const int j = d == 0 ? i + k : i + 2 * (K - 1) - k;
        const bool live = d == 0 || t + (K - 1) - k < rend;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += live ? wv[e][k] * row[j][e] : 0.0f;
      }
      if (a.act[d]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = silu_f(o[e]);
      }
      gstore8(ob + t * a.HP, o);
    }
  }
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
  const int64_t n = (int64_t)a.Z * ((a.L + kRun - 1) / kRun) * (a.HP / 8);
  const dim3 g((unsigned)((n + 255) / 256));
#define BISSD_CONV_LAUNCH(TT)                                                           \
  switch (a.K) {                                                                        \
    case 1: launch_kernel((k_conv_x<TT, 1>), g, dim3(256), 0, st, a); break;       \
    case 2: launch_kernel((k_conv_x<TT, 2>), g, dim3(256), 0, st, a); break;       \
    case 3: launch_kernel((k_conv_x<TT, 3>), g, dim3(256), 0, st, a); break;       \
    default: launch_kernel((k_conv_x<TT, 4>), g, dim3(256), 0, st, a); break;      \
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
