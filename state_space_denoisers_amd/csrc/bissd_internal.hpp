// bissd_internal.hpp -- launch arguments shared by the ABI layer and the
// kernel launchers (not part of the public interface).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bissd {

// The pair of events armed by bissd_timer_arm, handed to the first launch
// that asks and then disarmed (both nullptr when none is armed).
void take_timer(hipEvent_t *start, hipEvent_t *stop);

// Every kernel launch of the library: hipExtLaunchKernelGGL records the
// dispatch's own start and end timestamps in an armed timer's events.
template <typename F, typename... Args>
inline void launch_kernel(F kern, dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                          Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  take_timer(&e0, &e1);
  hipExtLaunchKernelGGL(kern, grid, block, shmem, st, e0, e1, 0u, args...);
}

// Division by a runtime constant d (1 <= d < 2^31) of numerators n < 2^31 as
// a multiply-high and a shift: with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, n / d = (mulhi(n, m) + n) >> s.  The
// host forms (m, s) once per launch, so the kernels split their workgroup
// index without an integer division.
struct FastDiv {
  uint32_t d = 1, m = 1, s = 0;
  FastDiv() = default;
  explicit FastDiv(uint32_t dv) : d(dv) {
    s = 0;
    while ((1ull << s) < dv) ++s;
    m = (uint32_t)(((1ull << 32) * ((1ull << s) - dv)) / dv + 1);
  }
  __host__ __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint32_t hi = (uint32_t)(((uint64_t)n * m) >> 32);
    return (hi + n) >> s;
  }
  // n / d, leaving n % d in rem
  __host__ __device__ __forceinline__ uint32_t divmod(uint32_t n, uint32_t &rem) const {
    const uint32_t q = div(n);
    rem = n - q * d;
    return q;
  }
};

struct ScanArgs {
  const void *x;
  // the scan's input per direction when it differs from x (the directions'
  // convolved x); nullptr: x.  x itself stays the skip's input.
  const void *xs[2];
  // the block kernel's own convolution (blocks of at most 64 tokens): taps
  // [H][P][ckw] and bias [H][P] per direction (cw[d] nullptr: none), SiLU
  // flags, and the conv state [Z][ckw-1][H][P] in / out (may be equal)
  const float *cw[2], *cb[2];
  int cact[2], ckw;
  const void *cst_in;
  void *cst_out;
  const void *dt[2];  // [0] forward, [1] reverse
  // per-direction dt post-processing: with dtb[d] set, every read of dt[d]
  // becomes clamp(softplus(dt + dtb[d][h]), dtlo[d], dthi[d])
  const float *dtb[2];
  float dtlo[2], dthi[2];
  const float *A[2];
  const void *B[2];
  const void *C[2];
  const float *D;
  void *y;
  void *states;   // [ndir][Z][nchunks][H][P][N] chunk-local states, compute dtype (workspace)
  float *cdecay;  // [ndir][Z][nchunks][H] chunk total log2-decay (workspace)
  const void *sin[2];  // carry-in state of each chunk, per direction (nullptr = none)
  int64_t sin_bstride[2], sin_cstride[2];  // element strides of sin per batch row / chunk
  int sin_f32[2];       // 1: sin is fp32; 0: sin has the compute dtype
  void *sin_t;          // carry-in states in the compute dtype, written by the state pass
  const float *init_state;  // forward start state for the state pass
  float *final_state;       // forward end state written by the state pass
  int64_t L;
  int Z, H, G, N, chunk, nchunks;
  int dir0, ndir;  // directions handled by the chunk-state / state-pass phases
  int dtype;       // 0 fp32, 1 bf16
  // backward phases only
  const void *aux;  // PHASE_YDOT: dy; PHASE_DX: x (x above then holds dy)
  float *out0;      // PHASE_YDOT: dy.y_d; PHASE_DX: x.(G_t B_t); [2][Z][L][H], by direction.
                    // PHASE_ADJ_STATE: <state, sin> per [2][Z][nchunks][H].
                    // PHASE_ADJ_PASS: wave partials of <adjoint carry, state after the chunk>
  float *out1;      // PHASE_DX: dx [Z][L][H][P]; PHASE_TAN_STATE: chunk dt sums [2][Z][nchunks][H]
  float *out2;      // PHASE_DX: partial sums of dy.x per (b, chunk, row-block, head)
  float *out3;      // PHASE_DX: x.(G_t B_t) without the t' = t term, [2][Z][L][H]
  const void *states2;   // PHASE_TAN_PASS: tangent chunk states, compute dtype
  void *sin_prim;        // PHASE_TAN_PASS: if set, also the primal carry-in states it
                         // carries alongside, compute dtype, laid out as sin_t
  const float *dtsum;    // PHASE_TAN_PASS: chunk dt sums
  int slot_dir[2];  // direction under which each output-kernel slot stores out0
  // divisors of the workgroup-index splits (set by launch_scan_phase): head
  // tiles per batch-chunk-row-block, chunks, heads per B/C group, groups,
  // Gram pairs per chunk
  FastDiv fd_tiles, fd_nc, fd_hpg, fd_g, fd_pairs;
  void *gram;       // per slot: the chunk Gram tiles C.B^T in the output kernel's
                    // lane order, compute dtype, [2][Z][nchunks][G][chunk * chunk]; written by
                    // PHASE_GRAM (or by PHASE_CHUNK_STATE when gram_k1 is set), read
                    // by the output kernel (every mode)
  int gram_k1;      // PHASE_CHUNK_STATE over both directions also writes the Gram
                    // tiles (set by the host when gram_in_k1() holds)
  float *cum_out;   // if set, PHASE_CHUNK_STATE writes each token's in-chunk log2-decay
                    // sum and PHASE_TAN_STATE its in-chunk cumulative dt, both in scan
                    // order, fp32 [2][Z][H][L]
  const float *cdt_in;  // PHASE_YDOT: each token's in-chunk cumulative dt (scan order),
                        // fp32 [2][Z][H][L]
  float *dai_out;       // PHASE_YDOT: within-chunk A-tangent sums
                        // sum_{s before t} E[t][s] (T_t - T_s) per (dir, b, chunk,
                        // row-block, head), [2][Z][nchunks][chunk/64][H]
  // Block-segmented reverse scan (0, 0: none).  rseg_chunks: chunks per
  // reverse block, 1 when a block is no longer than a chunk; the reverse
  // carries (primal, A-tangent, adjoint) are zero across every chunk
  // boundary c * chunk with c % rseg_chunks == 0.  rseg_tiles: 64-token tiles
  // per reverse block when a block is shorter than a chunk (1 or 2); the
  // reverse direction's within-chunk pairs then stay inside their block.
  int rseg_chunks, rseg_tiles;
  // Forward calls: skip what no later kernel reads -- PHASE_STATE_PASS the
  // first chunk's zero carry-in in scan order and the last chunk's state
  // unless it feeds final_state, PHASE_CHUNK_STATE the writes of those states
  int skip_edges;
};

enum {
  PHASE_CHUNK_STATE = 0,  // chunk-local states and chunk decays
  PHASE_STATE_PASS = 1,   // carry-in states
  PHASE_CHUNK_OUT = 2,    // y
  PHASE_ADJ_STATE = 3,    // chunk-local adjoint states sum_t 2^cum_t dy_t (outer) C_t
  PHASE_ADJ_PASS = 4,     // adjoint carries, flowing against each direction
  PHASE_YDOT = 5,         // per-direction dy.y_d (forward output recomputed)
  PHASE_DX = 6,           // dx and x.(G_t B_t)
  PHASE_TAN_STATE = 7,    // chunk-local A-tangent states (dt-sum weighted)
  PHASE_TAN_PASS = 8,     // A-tangent carry-in states
  PHASE_GRAM = 10,        // chunk Gram tiles for the output kernel
};

hipError_t launch_scan_phase(const ScanArgs &a, int phase, hipStream_t st);
// True if the chunk-state kernel can form every Gram tile itself: each of
// its workgroups takes one (row-block, column-block) pair of its direction,
// so a group needs at least as many head tiles as there are pairs.
bool gram_in_k1(int H, int G, int chunk);

// Whole block update (both directions, skip, optional committed state) in
// one launch, for blocks of at most 64 tokens: x, dt, A, B, C, D, y as in
// the scan; init_state = the cached state; final_state = the committed
// state or nullptr (may equal init_state); L = block length.
hipError_t launch_block_update(const ScanArgs &a, hipStream_t st);

// The directions' convolutions of x (bissd_conv.hip), one pass over x for
// both: xc[d][t][c] = act_d(b_d[c] + sum_k w_d[c][k] x[t - (K-1) + k][c])
// (forward) and x[t + (K-1) - k] (reverse), c = h P + p.  Rows before the
// sequence come from `state` ([Z][K-1][H][P], nullptr: zeros); rows at or
// past L, or past the end of the token's reverse block (rev_block > 0), are
// zero.
struct ConvArgs {
  const void *x;          // [Z][L][H][P], dtype
  void *xc[2];            // [Z][L][H][P], dtype, per direction (nullptr: not formed)
  const float *w[2], *b[2];
  int act[2];
  const void *state;      // forward left halo or nullptr
  int64_t L;
  int Z, HP, K, dtype, rev_block;
};
hipError_t launch_conv(const ConvArgs &a, hipStream_t st);
// The conv state after a block: state_out[z][j] = row j + L of [state_in | x]
// for j < K-1 (in place allowed: every old row is read before any is written).
hipError_t launch_conv_state(const void *x, const void *state_in, void *state_out, int64_t L,
                             int Z, int HP, int K, int dtype, hipStream_t st);

// Arguments of the backward-only kernels (dB / dC panels, decay gradients,
// final reductions).
struct BwdArgs {
  const void *x, *dy;
  const void *dt[2];
  const float *dtb[2];  // as in ScanArgs
  float dtlo[2], dthi[2];
  float *ddtb[2];       // with dtb[d]: gradient of the bias, [H]
  float *dbpart;        // [2][Z][nchunks][H] per-chunk sums of the pre-activation ddt
  const float *A[2];
  const void *B[2], *C[2];
  const void *sin[2];  // forward carry-in states per direction, compute dtype
  const void *gin[2];  // adjoint carries per direction, compute dtype
  int64_t st_bstride, st_cstride;  // element strides of sin / gin
  const float *ydot, *qx, *qxs;    // [2][Z][L][H]; qxs leaves out the t' = t term
  float *dB[2], *dC[2], *ddt[2], *dA[2], *dD;
  const float *rpart;   // [2][Z][nchunks][H][P N / 256] wave partials of the chunk-boundary dalpha
  float *dAintra;       // [2][Z][nchunks][chunk/64][H] within-chunk A-tangent sums
  const float *dAx1;    // [2][Z][nchunks][H] <adjoint chunk state, A-tangent carry-in>
  const float *ddpart;  // [Z][nchunks][chunk/64][H]
  const float *lamg;    // [2][Z][H][L] in-chunk log2-decay sums (scan order)
  const float *cdtg;    // [2][Z][H][L] in-chunk cumulative dt (scan order)
  int64_t L;
  int Z, H, G, N, chunk, nchunks, dtype;
  int rseg_tiles;  // as in ScanArgs: the reverse panels' column blocks stay in the row's block
};

// Multi-head softmax attention of the hybrid backbones (bissd_attn.hip).
constexpr int kAttnD = 64;  // head dim
struct AttnArgs {
  const void *q, *k, *v;  // [Z][L][H][kAttnD], dtype
  void *o;                // forward: output; backward: the forward's output (read)
  float *lse;             // [Z][H][L] per-query log2-sum-exp of c * scores (forward: written
                          // if set; backward: read)
  const void *dout;       // backward: dO, [Z][L][H][kAttnD], dtype
  float *dq, *dk, *dv;    // backward: fp32 gradients, [Z][L][H][kAttnD]
  float *delta;           // backward: D = rowsum(dO * O), [Z][H][L] (workspace)
  int64_t L, block;       // block: 0 full, > 0 block-wise (a multiple of 64)
  int Z, H, dtype;
  float scale;            // softmax scale
  float scale_log2;       // scale * log2(e)
};
hipError_t launch_attention(const AttnArgs &a, hipStream_t st);
hipError_t launch_attention_backward(const AttnArgs &a, hipStream_t st);

hipError_t launch_bwd_panels(const BwdArgs &a, hipStream_t st);
hipError_t launch_bwd_decay(const BwdArgs &a, hipStream_t st);

}  // namespace bissd
