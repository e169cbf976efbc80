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
// (the reverse is the forward convolution of the flipped sequence).  One
// thread forms eight channels of one token for both directions from the 2K-1
// rows around it (16-byte loads, neighbouring tokens' rows served by the
// cache); bound by HBM.
#include "bissd_device.hpp"
#include "bissd_internal.hpp"

namespace bissd {

namespace {

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

template <typename T> __device__ __forceinline__ void load8(float (&o)[8], const T *p) { gload8(o, p); }

}  // namespace

template <typename T, int K>
__global__ __launch_bounds__(256) void k_conv_x(ConvArgs a) {
  const int nvec = a.HP / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t ntok = (int64_t)a.Z * a.L;
  if (gid >= ntok * nvec) return;
  const int v = (int)(gid % nvec);
  const int64_t zt = gid / nvec;
  const int64_t t = zt % a.L;
  const int b = (int)(zt / a.L);
  const int c0 = v * 8;
  const T *xb = reinterpret_cast<const T *>(a.x) + (int64_t)b * a.L * a.HP + c0;
  const T *sb = a.state ? reinterpret_cast<const T *>(a.state) + (int64_t)b * (K - 1) * a.HP + c0 : nullptr;
  // rows t - (K-1) .. t + (K-1); zero outside [0, L) except the forward's
  // left halo from the state
  float row[2 * K - 1][8];
#pragma unroll
  for (int j = 0; j < 2 * K - 1; ++j) {
    const int64_t tj = t - (K - 1) + j;
    if (tj >= 0 && tj < a.L) {
      load8(row[j], xb + tj * a.HP);
    } else if (tj < 0 && sb) {
      load8(row[j], sb + (tj + (K - 1)) * a.HP);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) row[j][e] = 0.0f;
    }
  }
  // the reverse reads nothing past the end of the token's reverse block
  const int64_t rend = a.rev_block > 0 ? (t / a.rev_block + 1) * a.rev_block : a.L;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    if (!a.xc[d]) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = a.b[d] ? a.b[d][c0 + e] : 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      // forward tap k reads row t - (K-1) + k (window index k); reverse tap k
      // reads row t + (K-1) - k (window index 2(K-1) - k)
      const int j = d == 0 ? k : 2 * (K - 1) - k;
      const bool live = d == 0 || t + (K - 1) - k < rend;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float wv = a.w[d][(c0 + e) * K + k];
        o[e] += live ? wv * row[j][e] : 0.0f;
      }
    }
    if (a.act[d]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = silu_f(o[e]);
    }
    gstore8(reinterpret_cast<T *>(a.xc[d]) + ((int64_t)b * a.L + t) * a.HP + c0, o);
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
  const int64_t n = (int64_t)a.Z * a.L * (a.HP / 8);
  const dim3 g((unsigned)((n + 255) / 256));
#define BISSD_CONV_LAUNCH(TT)                                                           \
  switch (a.K) {                                                                        \
    case 1: hipLaunchKernelGGL((k_conv_x<TT, 1>), g, dim3(256), 0, st, a); break;       \
    case 2: hipLaunchKernelGGL((k_conv_x<TT, 2>), g, dim3(256), 0, st, a); break;       \
    case 3: hipLaunchKernelGGL((k_conv_x<TT, 3>), g, dim3(256), 0, st, a); break;       \
    default: hipLaunchKernelGGL((k_conv_x<TT, 4>), g, dim3(256), 0, st, a); break;      \
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
    hipLaunchKernelGGL(k_conv_state<bf16>, g, dim3(256), 0, st, reinterpret_cast<const bf16 *>(x),
                       reinterpret_cast<const bf16 *>(state_in), reinterpret_cast<bf16 *>(state_out), L, Z, HP, K);
  else
    hipLaunchKernelGGL(k_conv_state<float>, g, dim3(256), 0, st, reinterpret_cast<const float *>(x),
                       reinterpret_cast<const float *>(state_in), reinterpret_cast<float *>(state_out), L, Z, HP, K);
  return hipGetLastError();
}

}  // namespace bissd
