// bissd_internal.hpp -- launch arguments shared by the ABI layer and the
// kernel launchers (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bissd {

struct ScanArgs {
  const void *x;
  const void *dt[2];  // [0] forward, [1] reverse
  const float *A[2];
  const void *B[2];
  const void *C[2];
  const float *D;
  void *y;
  float *states;  // [ndir][Z][nchunks][H][P][N] chunk states (workspace)
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
};

enum { PHASE_CHUNK_STATE = 0, PHASE_STATE_PASS = 1, PHASE_CHUNK_OUT = 2 };

hipError_t launch_scan_phase(const ScanArgs &a, int phase, hipStream_t st);

}  // namespace bissd
