// bissd_device.hpp -- device building blocks of the bidirectional SSD scan
// for CDNA4 (gfx950): MFMA fragments, LDS staging and wavefront scans.
//
// Matrix-core convention used throughout.  A 16x16 output tile D = A * B is
// accumulated in 4 fp32 registers per lane: lane l holds D[4*(l/16)+i][l%16]
// for i = 0..3.  A K-step contracts 32 values of k: lane l supplies A[l%16][k]
// and B[k][l%16] for the 8 k values of its lane group l/16.  Which 8 k values
// a group owns only has to agree between A and B, so two mappings are used:
//   natural:  k = 8*(l/16) + e                       (8 contiguous values)
//   paired :  k = 4*(l/16) + e        for e < 4,
//             k = 16 + 4*(l/16) + e-4 for e >= 4     (two runs of 4)
// The paired mapping lets a pair of 16x16 output tiles (two runs of 4 rows per
// lane) be fed straight back in as the A operand of the next product.
// bf16 operands use v_mfma_f32_16x16x32_bf16 (one instruction per K-step);
// fp32 operands use eight v_mfma_f32_16x16x4_f32, element e of every lane in
// instruction e, which covers the same 32 k values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bissd {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kP = 64;        // head dim
constexpr int kRB = 64;       // tokens per row-block (and per staged slab)
constexpr int kThreads = 256; // 4 wavefronts of 64
constexpr int kQmax = 256;    // largest chunk
constexpr float kLog2e = 1.4426950408889634f;

// 2^v on the transcendental unit.  Every decay in the scan is written as
// exp(z) = 2^(z * log2 e); arguments are never positive except where a
// bounded (< 2^40) rescale factor is intended.
__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }

// ------------------------------------------------------------ global I/O

__device__ __forceinline__ void gload8(float (&o)[8], const bf16 *p) {
  const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
}
__device__ __forceinline__ void gload8(float (&o)[8], const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = a[e];
    o[4 + e] = b[e];
  }
}
__device__ __forceinline__ void gstore8(bf16 *p, const float (&o)[8]) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)o[e];
  *reinterpret_cast<bf16x8 *>(p) = v;
}
__device__ __forceinline__ void gstore8(float *p, const float (&o)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = o[e];
    b[e] = o[4 + e];
  }
  *reinterpret_cast<f32x4 *>(p) = a;
  *reinterpret_cast<f32x4 *>(p + 4) = b;
}

// ------------------------------------------------------------- fragments

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

// Elements 0..3 (hi false) or 4..7 (hi true) of a fragment as floats: whole
// registers are selected (two selections in bf16), never single elements,
// so a lane-uniform choice costs no per-element selection chain.
__device__ __forceinline__ void frag_half(const Frag<bf16> &f, bool hi, float (&o)[4]) {
  typedef uint32_t w4 __attribute__((ext_vector_type(4)));
  const w4 r = __builtin_bit_cast(w4, f.v);
  const uint32_t a = hi ? r[2] : r[0], b = hi ? r[3] : r[1];
  o[0] = __builtin_bit_cast(float, a << 16);
  o[1] = __builtin_bit_cast(float, a & 0xffff0000u);
  o[2] = __builtin_bit_cast(float, b << 16);
  o[3] = __builtin_bit_cast(float, b & 0xffff0000u);
}
__device__ __forceinline__ void frag_half(const Frag<float> &f, bool hi, float (&o)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = hi ? f.v[4 + i] : f.v[i];
}

__device__ __forceinline__ void frag_zero(Frag<bf16> &f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)0.0f;
}
__device__ __forceinline__ void frag_zero(Frag<float> &f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = 0.0f;
}
__device__ __forceinline__ void frag_from(Frag<bf16> &f, const float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (bf16)x[e];
}
__device__ __forceinline__ void frag_from(Frag<float> &f, const float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = x[e];
}
// natural mapping: 8 contiguous elements (16-byte aligned)
__device__ __forceinline__ void frag_ld8(Frag<bf16> &f, const bf16 *p) {
  f.v = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void frag_ld8(Frag<float> &f, const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = a[e];
    f.v[4 + e] = b[e];
  }
}
// paired mapping: elements 0..3 from p0, 4..7 from p1
__device__ __forceinline__ void frag_ld4x2(Frag<bf16> &f, const bf16 *p0, const bf16 *p1) {
  const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
  const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_ld4x2(Frag<float> &f, const float *p0, const float *p1) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p0);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p1);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = a[e];
    f.v[4 + e] = b[e];
  }
}

__device__ __forceinline__ void mma(f32x4 &c, const Frag<bf16> &a, const Frag<bf16> &b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &c, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
}

__device__ __forceinline__ void zero4(f32x4 &c) { c = f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// LDS row pitches (elements).  Rows of W contiguous elements read 16 bytes
// per lane (natural mapping) get 16 extra bytes; token rows read as runs of
// 4 (paired mapping) get 4 extra elements.  Both keep a 16-lane read phase
// on distinct banks.
template <typename T, int W> struct RowPitch {
  static constexpr int value = W + 16 / (int)sizeof(T);
};
template <typename T> struct TokPitch {
  static constexpr int value = kRB + 4;
};

// --------------------------------------------------------- LDS staging

// Copy a slab of 64 token rows x W columns (row stride `rs` elements) into
// LDS row-major [token][col] with pitch RowPitch<T,W>.  Rows >= nvalid read
// as zero.
template <typename T, int W>
__device__ __forceinline__ void stage_rows(T *lds, const T *g, int64_t rs, int nvalid) {
  constexpr int CG = W / 8;
  constexpr int PT = RowPitch<T, W>::value;
  for (int it = threadIdx.x; it < kRB * CG; it += kThreads) {
    const int s = it / CG, c0 = (it % CG) * 8;
    float v[8];
    if (s < nvalid) {
      gload8(v, g + (int64_t)s * rs + c0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    if constexpr (sizeof(T) == 2) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
      *reinterpret_cast<bf16x8 *>(lds + s * PT + c0) = o;
    } else {
      gstore8(reinterpret_cast<float *>(lds) + s * PT + c0, v);
    }
  }
}

// Copy a slab of 64 token rows x W columns into LDS transposed, [col][token]
// with pitch TokPitch, multiplying token row s by scale[s] (LDS, or nullptr
// for 1) before the single rounding to T.  Rows >= nvalid read as zero.
template <typename T, int W>
__device__ __forceinline__ void stage_cols(T *lds, const T *g, int64_t rs, int nvalid,
                                           const float *scale) {
  constexpr int CG = W / 8;
  constexpr int PT = TokPitch<T>::value;
  if constexpr (sizeof(T) == 2) {
    // two tokens per item so each LDS write is one 4-byte word
    for (int it = threadIdx.x; it < (kRB / 2) * CG; it += kThreads) {
      const int s = (it / CG) * 2, c0 = (it % CG) * 8;
      float v0[8], v1[8];
      if (s < nvalid) {
        gload8(v0, g + (int64_t)s * rs + c0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v0[e] = 0.0f;
      }
      if (s + 1 < nvalid) {
        gload8(v1, g + (int64_t)(s + 1) * rs + c0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v1[e] = 0.0f;
      }
      const float s0 = scale ? scale[s] : 1.0f;
      const float s1 = scale ? scale[s + 1] : 1.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x2 pr;
        pr[0] = (bf16)(v0[e] * s0);
        pr[1] = (bf16)(v1[e] * s1);
        *reinterpret_cast<bf16x2 *>(lds + (c0 + e) * PT + s) = pr;
      }
    }
  } else {
    for (int it = threadIdx.x; it < kRB * CG; it += kThreads) {
      const int s = it / CG, c0 = (it % CG) * 8;
      float v[8];
      if (s < nvalid) {
        gload8(v, g + (int64_t)s * rs + c0);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
      }
      const float sc = scale ? scale[s] : 1.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) reinterpret_cast<float *>(lds)[(c0 + e) * PT + s] = v[e] * sc;
    }
  }
}

// -------------------------------------------- k-along-rows fragments
//
// ds_read_b64_tr_b16 (gfx950) works on groups of 16 lanes: if lane k of a
// group supplies the address of 4 consecutive 16-bit elements M[k][0..3],
// lane i receives M[4e + i/4][i%4] for e = 0..3.  Lane k therefore points at
// row r0 + k/4, columns c0 + 4(k%4) .. +3 of a row-major tile, and lane i
// receives tile[r0 + e][c0 + i]: four consecutive k values (rows) of its own
// column -- an MFMA operand fragment with k running down the rows, read
// without transposing the tile in LDS.

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 lds_tr4(const bf16 *p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Fragment with k along rows: elements 0..3 = tile[r0 + 0..3][c0 + l%16],
// elements 4..7 = tile[r1 + 0..3][c0 + l%16]  (row-major tile, pitch `pt`).
__device__ __forceinline__ void frag_rows(Frag<bf16> &f, const bf16 *tile, int pt, int r0, int r1,
                                          int c0) {
  const int i = threadIdx.x & 15;
  const int off = (i >> 2) * pt + c0 + 4 * (i & 3);
  const bf16x4 a = lds_tr4(tile + r0 * pt + off);
  const bf16x4 b = lds_tr4(tile + r1 * pt + off);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_rows(Frag<float> &f, const float *tile, int pt, int r0, int r1,
                                          int c0) {
  const int i = threadIdx.x & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = tile[(r0 + e) * pt + c0 + i];
    f.v[4 + e] = tile[(r1 + e) * pt + c0 + i];
  }
}

// Row pitch (elements) of row-major tiles read with frag_rows: a 16-lane
// group reads 4 rows x 32 bytes; a pitch of W + 32 bytes puts the 4 rows on
// disjoint banks.
template <typename T, int W> struct TrPitch {
  static constexpr int value = W + 32 / (int)sizeof(T);
};

// ------------------------------------------------ register-prefetched slabs
//
// A slab is 64 token rows of a row-major global tensor.  Its bytes are
// fetched as 16-byte vectors spread over the workgroup into registers
// (`prefetch`), so the loads of the next slab are in flight while the
// current one is being multiplied, and later written into LDS (`commit`).

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 gload16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// Buffer resource over [base, base + nbytes): raw buffer loads take a 32-bit
// byte offset, and any 16-byte load at or beyond nbytes returns zeros.  A
// resource spans one batch row of a tensor, so tokens past the sequence end
// read as zero without a bounds check.
typedef __amdgpu_buffer_rsrc_t bufres;
__device__ __forceinline__ bufres make_buf(const void *base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(bufres r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 16 raw bytes holding EPV elements of T, widened to fp32
__device__ __forceinline__ void unpack16(float (&o)[8], u32x4 v, const bf16 *) {
  const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (float)b[e];
}
__device__ __forceinline__ void unpack16(float (&o)[8], u32x4 v, const float *) {
  const f32x4 f = __builtin_bit_cast(f32x4, v);
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = f[e];
}

// Row-major slab [64][W] -> LDS [token][col] (pitch PT), no conversion.
// The slab's rows start at byte `off0` of buffer `r`, `rs` bytes apart.
template <typename T, int W, int PT = RowPitch<T, W>::value> struct SlabRows {
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int VPR = W / EPV;
  static constexpr int NV = (kRB * VPR + kThreads - 1) / kThreads;  // vectors per thread
  static constexpr bool FULL = (kRB * VPR) % kThreads == 0;

  __device__ static __forceinline__ void prefetch(u32x4 *pf, bufres r, uint32_t off0, uint32_t rs) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int vi = threadIdx.x + m * kThreads;
      const int s = vi / VPR, c = vi % VPR;
      if (FULL || vi < kRB * VPR) pf[m] = bload16(r, off0 + s * rs + c * 16);
    }
  }
  __device__ static __forceinline__ void commit(T *lds, const u32x4 *pf) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int vi = threadIdx.x + m * kThreads;
      if (FULL || vi < kRB * VPR) {
        const int s = vi / VPR, c = vi % VPR;
        *reinterpret_cast<u32x4 *>(lds + s * PT + c * EPV) = pf[m];
      }
    }
  }
};

// Row-major slab [64][W] -> LDS transposed [col][token] (pitch TokPitch),
// token row s multiplied by scale[s] before the single rounding to T.
// bf16 items carry two consecutive tokens so each LDS write is one word.
template <typename T, int W> struct SlabCols {
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int VPR = W / EPV;
  static constexpr int PAIR = sizeof(T) == 2 ? 2 : 1;
  static constexpr int ITEMS = (kRB / PAIR) * VPR;
  static constexpr int NI = (ITEMS + kThreads - 1) / kThreads;  // items per thread
  static constexpr int NV = NI * PAIR;                          // vectors per thread
  static constexpr int PT = TokPitch<T>::value;

  __device__ static __forceinline__ void prefetch(u32x4 *pf, const T *g, int64_t rs, int nvalid) {
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      const int it = threadIdx.x + m * kThreads;
      const int c = it % VPR, s0 = (it / VPR) * PAIR;
#pragma unroll
      for (int q = 0; q < PAIR; ++q)
        pf[m * PAIR + q] = (it < ITEMS && s0 + q < nvalid)
                               ? gload16(g + (int64_t)(s0 + q) * rs + c * EPV) : zero16();
    }
  }
  __device__ static __forceinline__ void commit(T *lds, const u32x4 *pf, const float *scale) {
#pragma unroll
    for (int m = 0; m < NI; ++m) {
      const int it = threadIdx.x + m * kThreads;
      if (it >= ITEMS) continue;
      const int c = it % VPR, s0 = (it / VPR) * PAIR;
      if constexpr (sizeof(T) == 2) {
        float v0[8], v1[8];
        unpack16(v0, pf[m * 2], (const T *)nullptr);
        unpack16(v1, pf[m * 2 + 1], (const T *)nullptr);
        const float a0 = scale ? scale[s0] : 1.0f, a1 = scale ? scale[s0 + 1] : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16x2 pr;
          pr[0] = (bf16)(v0[e] * a0);
          pr[1] = (bf16)(v1[e] * a1);
          *reinterpret_cast<bf16x2 *>(lds + (c * EPV + e) * PT + s0) = pr;
        }
      } else {
        float v[8];
        unpack16(v, pf[m], (const T *)nullptr);
        const float a0 = scale ? scale[s0] : 1.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) reinterpret_cast<float *>(lds)[(c * EPV + e) * PT + s0] = v[e] * a0;
      }
    }
  }
};

// Row-major slab [64][W] -> LDS row-major [token][col] with pitch PT, token
// row s multiplied by scale[s] before the single rounding to T.  Rows start
// at byte `off0` of buffer `r`, `rs` bytes apart.
template <typename T, int W, int PT> struct SlabRowsScaled {
  static constexpr int EPV = 16 / (int)sizeof(T);
  static constexpr int VPR = W / EPV;
  static constexpr int NV = (kRB * VPR + kThreads - 1) / kThreads;
  static_assert((kRB * VPR) % kThreads == 0, "slab must split evenly");

  __device__ static __forceinline__ void prefetch(u32x4 *pf, bufres r, uint32_t off0, uint32_t rs) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int vi = threadIdx.x + m * kThreads;
      const int s = vi / VPR, c = vi % VPR;
      pf[m] = bload16(r, off0 + s * rs + c * 16);
    }
  }
  __device__ static __forceinline__ void commit(T *lds, const u32x4 *pf, const float *scale) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int vi = threadIdx.x + m * kThreads;
      const int s = vi / VPR, c = vi % VPR;
      const float a0 = scale ? scale[s] : 1.0f;
      float v[8];
      unpack16(v, pf[m], (const T *)nullptr);
      if constexpr (sizeof(T) == 2) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)(v[e] * a0);
        *reinterpret_cast<bf16x8 *>(lds + s * PT + c * EPV) = o;
      } else {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = v[e] * a0;
        *reinterpret_cast<f32x4 *>(lds + s * PT + c * EPV) = o;
      }
    }
  }
};

// A [64][N] state slab (row-major, source type S) -> LDS [row][col] in T
// (pitch RowPitch), every element multiplied by `sc` before rounding.
template <typename T, typename S, int N> struct SlabState {
  static constexpr int EPV = 16 / (int)sizeof(S);
  static constexpr int VPR = N / EPV;
  static constexpr int NV = (kP * VPR + kThreads - 1) / kThreads;
  static constexpr int PT = RowPitch<T, N>::value;
  static_assert((kP * VPR) % kThreads == 0, "state slab must split evenly");

  __device__ static __forceinline__ void prefetch(u32x4 *pf, const S *g) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int vi = threadIdx.x + m * kThreads;
      pf[m] = gload16(g + (int64_t)vi * EPV);
    }
  }
  // the prefetched bytes as they are (S == T)
  __device__ static __forceinline__ void commit_raw(T *lds, const u32x4 *pf) {
    static_assert(sizeof(S) == sizeof(T), "raw commit needs the state in the compute dtype");
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int vi = threadIdx.x + m * kThreads;
      const int r = vi / VPR, c = vi % VPR;
      *reinterpret_cast<u32x4 *>(lds + r * PT + c * EPV) = pf[m];
    }
  }
  __device__ static __forceinline__ void commit(T *lds, const u32x4 *pf, float sc) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int vi = threadIdx.x + m * kThreads;
      const int r = vi / VPR, c = vi % VPR;
      float v[8];
      unpack16(v, pf[m], (const S *)nullptr);
      if constexpr (sizeof(T) == 2 && sizeof(S) == 2) {
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)(v[e] * sc);
        *reinterpret_cast<bf16x8 *>(lds + r * PT + c * EPV) = o;
      } else if constexpr (sizeof(T) == 2) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)(v[e] * sc);
        *reinterpret_cast<bf16x4 *>(lds + r * PT + c * EPV) = o;
      } else {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = v[e] * sc;
        *reinterpret_cast<f32x4 *>(lds + r * PT + c * EPV) = o;
      }
    }
  }
};

// Operand fragment of 8 consecutive elements read straight from a buffer
// resource (zeros past its end).
__device__ __forceinline__ void frag_bload(Frag<bf16> &f, bufres r, uint32_t off) {
  f.v = __builtin_bit_cast(bf16x8, bload16(r, off));
}
__device__ __forceinline__ void frag_bload(Frag<float> &f, bufres r, uint32_t off) {
  const f32x4 a = __builtin_bit_cast(f32x4, bload16(r, off));
  const f32x4 b = __builtin_bit_cast(f32x4, bload16(r, off + 16));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = a[e];
    f.v[4 + e] = b[e];
  }
}

// Index of the calling wavefront in its workgroup, as a wave-uniform
// (scalar) value, so that branches and addresses that depend only on it stay
// on the scalar unit.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ------------------------------------------------- direct buffer -> LDS slabs
//
// gfx950 buffer loads can write LDS directly: each lane's 16 bytes land at
// (wave-uniform base) + 16 * lane, and lanes outside the buffer resource
// write zeros.  A slab of rows of RB bytes is copied as 1 KB pieces into a
// dense tile whose 16-byte chunks are XOR-swizzled by row (chunk c of row y
// is stored at chunk c ^ swz(y)), so that fragment reads hit distinct LDS
// banks without padding.  No registers hold the data in flight; the copies
// are complete once every wave has waited for its vector-memory count and
// the workgroup has passed a barrier.
//
// Swizzle SW_NAT suits natural reads (16 lanes read 16 consecutive rows at
// one chunk); SW_TR suits transpose reads (16 lanes read 4 consecutive rows,
// 32 bytes each).
typedef __attribute__((address_space(3))) void *lds_vptr;
enum { SW_NAT = 0, SW_TR = 1 };

template <int RB, int SW> struct DmaTile {
  static constexpr int CPR = RB / 16;    // 16-byte chunks per row
  static constexpr int RPP = 1024 / RB;  // rows per 1 KB piece
  __device__ static __forceinline__ int swz(int y) {
    if (SW == SW_NAT) return RB == 128 ? ((y >> 1) & 7) : (y & 15);
    return RB == 128 ? 2 * ((y >> 1) & 3) : (RB == 256 ? 2 * (y & 3) : 0);
  }
  // byte offset of logical (row y, byte x) in the tile
  __device__ static __forceinline__ int at(int y, int x) {
    return y * RB + ((((x >> 4) ^ swz(y)) << 4) | (x & 15));
  }
  // copy rows [0, nrows) (nrows a multiple of RPP) of the slab starting at
  // byte off0 of r, rows rs bytes apart; the pieces are spread over nw
  // waves, of which the calling one is wave wv
  __device__ static __forceinline__ void load(char *tile, bufres r, uint32_t off0, uint32_t rs,
                                              int nrows, int wv = wave_id(), int nw = kThreads / 64) {
    const int l = threadIdx.x & 63;
    const int np = nrows / RPP;
    for (int p = wv; p < np; p += nw) {
      const int y = p * RPP + l / CPR, c = l % CPR;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(tile + p * 1024), 16,
                                               off0 + y * rs + 16 * (c ^ swz(y)), 0, 0, 0);
    }
  }
};

// natural-mapping fragment (8 consecutive elements at row y, column x) from
// a swizzled tile
template <class DT>
__device__ __forceinline__ void frag_ld8_swz(Frag<bf16> &f, const char *tile, int y, int x) {
  f.v = *reinterpret_cast<const bf16x8 *>(tile + DT::at(y, 2 * x));
}
template <class DT>
__device__ __forceinline__ void frag_ld8_swz(Frag<float> &f, const char *tile, int y, int x) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(tile + DT::at(y, 4 * x));
  const f32x4 b = *reinterpret_cast<const f32x4 *>(tile + DT::at(y, 4 * x + 16));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = a[e];
    f.v[4 + e] = b[e];
  }
}
// the same from an fp32 tile into a bf16 fragment (one rounding)
template <class DT>
__device__ __forceinline__ void frag_ld8_swz_f32(Frag<bf16> &f, const char *tile, int y, int x) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(tile + DT::at(y, 4 * x));
  const f32x4 b = *reinterpret_cast<const f32x4 *>(tile + DT::at(y, 4 * x + 16));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = (bf16)a[e];
    f.v[4 + e] = (bf16)b[e];
  }
}
template <class DT>
__device__ __forceinline__ void frag_ld8_swz_f32(Frag<float> &f, const char *tile, int y, int x) {
  frag_ld8_swz<DT>(f, tile, y, x);
}
// k-along-rows fragment (frag_rows semantics) from a swizzled tile
template <class DT>
__device__ __forceinline__ void frag_rows_swz(Frag<bf16> &f, const char *tile, int r0, int r1, int c0) {
  const int i = threadIdx.x & 15;
  const int y = i >> 2, x = 2 * (c0 + 4 * (i & 3));
  const bf16x4 a = lds_tr4(reinterpret_cast<const bf16 *>(tile + DT::at(r0 + y, x)));
  const bf16x4 b = lds_tr4(reinterpret_cast<const bf16 *>(tile + DT::at(r1 + y, x)));
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <class DT>
__device__ __forceinline__ void frag_rows_swz(Frag<float> &f, const char *tile, int r0, int r1, int c0) {
  const int i = threadIdx.x & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = *reinterpret_cast<const float *>(tile + DT::at(r0 + e, 4 * (c0 + i)));
    f.v[4 + e] = *reinterpret_cast<const float *>(tile + DT::at(r1 + e, 4 * (c0 + i)));
  }
}

// vector-memory count 0, other counters left alone
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// vector-memory count at most K (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 at their maxima), other counters left alone
template <int K> __device__ __forceinline__ void wait_vmem_le() {
  static_assert(K >= 0 && K < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((K & 15) | ((K >> 4) << 14) | 0x0F70);
}

// ------------------------------------------------------- XCD-aware order
//
// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs,
// each with its own L2.  Remapping the id so that every XCD receives one
// contiguous range of work items keeps workgroups that read the same chunk
// of B, C and x on one XCD, where the second and later reads hit its L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_linear_id(int bid, int nwg) {
  const int per = nwg / kXcds, rem = nwg % kXcds;
  const int xcd = bid % kXcds, slot = bid / kXcds;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// ------------------------------------------------------ wavefront scans

// Cross-lane moves through DPP (no LDS round trip).  Lanes whose source lies
// outside the pattern (or whose row is masked off) read 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, false));
}
// Inclusive sum from lane 0 upwards: steps of 1, 2, 4, 8 lanes inside each
// 16-lane row (row_shr), then each row adds the totals of the rows below it.
__device__ __forceinline__ float wave_scan_up(float v) {
  v += dpp_f<0x111>(v);
  v += dpp_f<0x112>(v);
  v += dpp_f<0x114>(v);
  v += dpp_f<0x118>(v);
  const int row = (threadIdx.x & 63) >> 4;
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
  // the same sums as r0, r0 + r1, (r0 + r1) + r2, formed by selects (no branches)
  const float below = ((row >= 1 ? r0 : 0.0f) + (row >= 2 ? r1 : 0.0f)) + (row >= 3 ? r2 : 0.0f);
  return v + below;
}
// Inclusive sum from lane 63 downwards (row_shl inside the rows, then the
// totals of the rows above).
__device__ __forceinline__ float wave_scan_down(float v) {
  v += dpp_f<0x101>(v);
  v += dpp_f<0x102>(v);
  v += dpp_f<0x104>(v);
  v += dpp_f<0x108>(v);
  const int row = (threadIdx.x & 63) >> 4;
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  const float above = ((row <= 2 ? r3 : 0.0f) + (row <= 1 ? r2 : 0.0f)) + (row == 0 ? r1 : 0.0f);
  return v + above;
}
// lane l receives lane l - 1 (lane 0: 0) / lane l + 1 (lane 63: 0)
__device__ __forceinline__ float wave_shift_up1(float v) { return dpp_f<0x138>(v); }
__device__ __forceinline__ float wave_shift_down1(float v) { return dpp_f<0x130>(v); }

// Largest value over the wave for v >= 0 (row maxima by row_shr, then the
// four row results), in every lane.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  v = fmaxf(v, dpp_f<0x111>(v));
  v = fmaxf(v, dpp_f<0x112>(v));
  v = fmaxf(v, dpp_f<0x114>(v));
  v = fmaxf(v, dpp_f<0x118>(v));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 47));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Mamba-2's dt post-processing, applied wherever a kernel reads dt when the
// direction carries a per-head bias: dt = clamp(softplus(raw + bias), lo, hi).
// softplus(z) = max(z, 0) + log1p(e^-|z|) stays accurate for either sign.
struct DtPost {
  float bias = 0.0f, lo = 0.0f, hi = 0.0f;
  bool on = false;
};
__device__ __forceinline__ float softplus_f(float z) { return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z))); }
__device__ __forceinline__ float dt_post(float raw, const DtPost &p) {
  return p.on ? fminf(fmaxf(softplus_f(raw + p.bias), p.lo), p.hi) : raw;
}
// d dt / d raw: sigmoid(raw + bias) where the softplus lies inside the clamp
// range (ends included), else 0; 1 without post-processing
__device__ __forceinline__ float dt_post_grad(float raw, const DtPost &p) {
  if (!p.on) return 1.0f;
  const float z = raw + p.bias, sp = softplus_f(z);
  return (sp >= p.lo && sp <= p.hi) ? 1.0f / (1.0f + expf(-z)) : 0.0f;
}

// dt of one chunk for one head, in the lane order chunk_decay_scan_vals
// expects: lane l holds tokens l K .. l K + K - 1 (K = Q / 64) in d[0..K-1];
// tokens at or beyond qlen read as 0.  Split from the scan so the loads can
// be issued well before the values are needed.
template <typename T>
__device__ __forceinline__ void chunk_dt_load(const T *dt, int64_t stride, int qlen, int Q,
                                              float (&d)[4], const DtPost &post = DtPost{}) {
  const int lane = threadIdx.x & 63;
  const int K = Q / 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = lane * K + i;
    d[i] = (i < K && s < qlen) ? to_f(dt[(int64_t)s * stride]) : 0.0f;
  }
  if (post.on) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < K && lane * K + i < qlen) d[i] = dt_post(d[i], post);
  }
}

// The same values through a buffer resource, with no branch: tokens past
// the resource read as zero, so every load is issued unconditionally.  The
// raw bits are kept as loaded (any arithmetic on them would make the
// compiler wait for the load at once); chunk_dt_decode turns them into dt.
// off0: byte offset of (first token of the chunk, head); rs: bytes between
// tokens.
template <typename T>
__device__ __forceinline__ void chunk_dt_bload(bufres r, uint32_t off0, uint32_t rs, int Q,
                                               uint32_t (&raw)[4]) {
  const int lane = threadIdx.x & 63;
  const int K = Q / 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t off = off0 + (uint32_t)(lane * K + i) * rs;
    if constexpr (sizeof(T) == 2) raw[i] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    else raw[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
}
// (tokens at or beyond qlen give 0, also after post-processing)
template <typename T>
__device__ __forceinline__ void chunk_dt_decode(const uint32_t (&raw)[4], int Q, float (&d)[4],
                                                const DtPost &post, int qlen) {
  const int K = Q / 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = __builtin_bit_cast(float, sizeof(T) == 2 ? raw[i] << 16 : raw[i]);
    d[i] = i < K ? f : 0.0f;  // tokens past the sequence end read as 0
  }
  if (post.on) {  // uniform: the post-processing costs nothing when off
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d[i] = (i < K && lane * K + i < qlen) ? dt_post(d[i], post) : 0.0f;
  }
}

// Log2-decay cumulative sums of one chunk for one (direction, head), run by
// one wavefront from dt loaded by chunk_dt_load.  a_s = dt_s * A2 (A2 = A
// log2(e), or 1 for plain cumulative dt).  Forward: lam[s] = sum_{k<=s} a_k.
// Reverse: lam[s] = sum_{k>=s} a_k.  With `exclusive` the sums leave out
// a_s itself (sum_{k<s}, sum_{k>s}).  dtv[s] receives dt_s.  Returns the
// largest |a_s| of the chunk (in every lane).
__device__ __forceinline__ float chunk_decay_scan_vals(const float (&d)[4], int Q, float A2,
                                                       bool reverse, float *lam, float *dtv,
                                                       bool exclusive = false) {
  const int lane = threadIdx.x & 63;
  const int K = Q / 64;  // 1, 2 or 4 tokens per lane
  float a[4], amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = d[i] * A2;
    amax = fmaxf(amax, fabsf(a[i]));
  }
  amax = wave_max_nonneg(amax);
  float pre[4];
  if (!reverse) {
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pre[i] = run;
      run += a[i];
      a[i] = run;
    }
    const float incl = wave_scan_up(run);
    const float excl = wave_shift_up1(incl);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < K) {
        lam[lane * K + i] = excl + (exclusive ? pre[i] : a[i]);
        dtv[lane * K + i] = d[i];
      }
  } else {
    float run = 0.0f;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      pre[i] = run;
      if (i < K) {
        run += a[i];
        a[i] = run;
      }
    }
    const float incl = wave_scan_down(run);
    const float excl = wave_shift_down1(incl);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < K) {
        lam[lane * K + i] = excl + (exclusive ? pre[i] : a[i]);
        dtv[lane * K + i] = d[i];
      }
  }
  return amax;
}

// chunk_dt_load followed by chunk_decay_scan_vals.
template <typename T>
__device__ __forceinline__ float chunk_decay_scan(const T *dt, int64_t stride, int qlen, int Q,
                                                  float A2, bool reverse, float *lam,
                                                  float *dtv, bool exclusive = false,
                                                  const DtPost &post = DtPost{}) {
  float d[4];
  chunk_dt_load(dt, stride, qlen, Q, d, post);
  return chunk_decay_scan_vals(d, Q, A2, reverse, lam, dtv, exclusive);
}

}  // namespace bissd
