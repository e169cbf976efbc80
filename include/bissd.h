/*
 * bissd.h -- C ABI of the bidirectional SSD (Mamba-2) scan library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  A bidirectional Mamba-2 mixer runs one selective scan over
 * the sequence and one over the flipped sequence and adds the two ("DiffMamba
 * Checkpoints" model card, Model details: forward plus flipped-reverse
 * Mamba-2; "DiffuMamba: High-Throughput Diffusion LMs with Mamba Backbone",
 * Technical Summary, Methodology / Core Architecture: two Mamba-2 layers, one
 * per direction, fused additively).  Per batch row b and head h, with state
 * S in R^{P x N} and group g = floor(h * G / H):
 *
 *   forward  (t = 0 .. L-1):  S <- exp(dt_f[t] A_f[h]) S + dt_f[t] x[t] (outer) B_f[t]
 *                             yf[t] = S C_f[t]
 *   reverse  (t = L-1 .. 0):  S' <- exp(dt_r[t] A_r[h]) S' + dt_r[t] x[t] (outer) B_r[t]
 *                             yr[t] = S' C_r[t]
 *   y[t] = yf[t] + yr[t] + D[h] x[t]
 *
 * Token t is counted by both directions.  The forward state starts from
 * init_state (or zero); the reverse state always starts from zero after the
 * last token.
 *
 * Block-segmented reverse ("Training Hybrid Block Diffusion Language Models
 * with Partial Bidirectionality", Methodology and Key Results: training with
 * a full-block objective builds the same caches inference uses).  With
 * shape->rev_block = RB > 0, every block of RB tokens of the training
 * sequence is an active block for its own reverse scan: S' restarts from
 * zero after each block's last token, so yr[t] sees only the tokens of t's
 * block from t onwards, while the forward scan -- whose states are the
 * prefix caches -- runs over the whole sequence.  bissd_forward and
 * bissd_backward take it; for RB >= L it is the unsegmented scan.
 *
 * The mixer's convolution (optional, per direction).  A Mamba-2 layer passes
 * its x through a short causal depthwise convolution and a SiLU before the
 * scan; the directions share the pre-convolution x (weight-tied
 * in-projection, "DiffMamba Checkpoints", Model details) and each has its own
 * taps.  With shape->conv_width = K > 0 and dir.conv_w set, that direction's
 * scan reads, per channel c = h * headdim + p,
 *   forward:  xc[t][c] = act(conv_b[c] + sum_{k<K} conv_w[c][k] x[t - (K-1) + k][c])
 *   reverse:  xc[t][c] = act(conv_b[c] + sum_{k<K} conv_w[c][k] x[t + (K-1) - k][c])
 * in place of x (act = SiLU with conv_act, else the identity): the reverse is
 * the forward convolution of the flipped sequence.  x reads as zero before
 * the sequence (a block update's forward convolution continues from the
 * block's conv state instead) and past its end; the reverse never reads past
 * the end of its reverse block.  The skip stays D x on the x given.
 *
 * Block update ("Training Hybrid Block Diffusion Language Models with Partial
 * Bidirectionality", Methodology and Technical Contribution): during
 * block-wise denoising the forward state after the prefix is a cache that is
 * reused exactly, while the reverse scan is confined to the active block.
 * bissd_block_update is the forward above on the block alone, with the
 * forward scan continuing from the cached prefix state and the reverse scan
 * starting from zero at the block end.
 *
 * Layouts (row-major, contiguous, natural token order for both directions):
 *   x, y, dy        [batch][seqlen][nheads][headdim]        dtype
 *   dx              [batch][seqlen][nheads][headdim]        fp32
 *   dt_f, dt_r      [batch][seqlen][nheads]                 dtype
 *   B_*, C_*        [batch][seqlen][ngroups][dstate]        dtype
 *   A_f, A_r, D     [nheads]                                fp32
 *   states          [batch][nheads][headdim][dstate]        fp32
 *   gradients       same layout as their input, fp32
 *
 * Pointers.  Every tensor pointer is a device pointer (from hipMalloc or any
 * device allocator) aligned to 16 bytes; the caller owns every buffer.  The
 * library allocates no device memory and keeps no state between calls: the
 * only scratch memory is the caller's workspace, sized by
 * bissd_workspace_size(), except for bissd_forward_noalloc, whose workspace
 * is a static device array of the library.  Calls are asynchronous on `stream` (a hipStream_t;
 * NULL = the null stream): inputs must stay live and unmodified until the
 * stream reaches the call.  Results are bitwise reproducible for identical
 * inputs and shapes on the same device.
 *
 * Errors.  Every entry point returns a status code.  On any validation
 * failure nothing is launched and no output is touched.  Values are not
 * inspected: NaN/Inf inputs propagate.  No exception, abort or exit crosses
 * the ABI.
 *
 * Support.  headdim == 64; dstate in {64, 128}; chunk in {64, 128, 256};
 * nheads % ngroups == 0; any seqlen >= 1; dtype BISSD_F32 or BISSD_BF16;
 * rev_block 0, or a multiple of 64 that divides chunk or is a multiple of it;
 * conv_width 0..4.
 * All arithmetic accumulates in fp32; bf16 operands feed the matrix cores.
 */
#ifndef BISSD_H
#define BISSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of x, dt, B, C, y and dy. */
enum { BISSD_F32 = 0, BISSD_BF16 = 1 };

/* status codes */
enum {
  BISSD_OK = 0,
  BISSD_ERR_NULL = -1,        /* a required pointer is NULL */
  BISSD_ERR_SHAPE = -2,       /* a dim <= 0, rev_block < 0, nheads % ngroups != 0, or block
                                 longer than chunk */
  BISSD_ERR_UNSUPPORTED = -3, /* headdim, dstate, chunk, rev_block or dtype outside the
                                 supported set */
  BISSD_ERR_ALIGN = -4,       /* a pointer not aligned to 16 bytes */
  BISSD_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than bissd_workspace_size() */
  BISSD_ERR_HIP = -6,         /* a HIP launch failed; see bissd_last_hip_error() */
  BISSD_ERR_ALIAS = -7,       /* an output overlaps an input it may not alias */
  BISSD_ERR_SCRATCH = -8      /* bissd_forward_noalloc: the shape needs more workspace
                                 than BISSD_NOALLOC_SCRATCH_BYTES */
};

/* Size of the device array that serves as bissd_forward_noalloc's workspace
 * (64 MiB; the forward of batch 8 x 1,024 tokens x 24 heads x 64 x d_state
 * 128 in bf16 needs 56 MiB). */
#define BISSD_NOALLOC_SCRATCH_BYTES (64u << 20)

/* operation selector for bissd_workspace_size() */
enum { BISSD_OP_FORWARD = 0, BISSD_OP_BACKWARD = 1, BISSD_OP_BLOCK = 2 };

typedef struct {
  int64_t batch;    /* Z */
  int64_t seqlen;   /* L (the block length for bissd_block_update) */
  int64_t nheads;   /* H */
  int64_t headdim;  /* P */
  int64_t dstate;   /* N */
  int64_t ngroups;  /* G: B and C are shared by nheads/ngroups consecutive heads */
  int64_t chunk;    /* chunk length of the chunked evaluation (a tiling choice;
                       the result does not depend on it beyond rounding) */
  int32_t dtype;    /* BISSD_F32 or BISSD_BF16 */
  int32_t rev_block; /* 0: one reverse scan over the whole sequence.  > 0: the
                        block-segmented reverse scan -- the reverse state
                        restarts from zero after the last token of every
                        block of rev_block tokens (tokens k rev_block ..
                        (k+1) rev_block - 1, the last block possibly shorter),
                        while the forward scan still runs over the whole
                        sequence.  A multiple of 64 that divides chunk or is
                        a multiple of it; bissd_block_update takes 0 only. */
  int32_t conv_width; /* 0: no convolution; 1..4: the width K of the directions'
                         convolutions (each direction with conv_w set uses it;
                         the workspace has room for their outputs) */
  int32_t flags;      /* 0, or BISSD_SAVE for bissd_forward / bissd_backward
                         (and bissd_workspace_size): the forward leaves in its
                         workspace what the backward would otherwise recompute */
} bissd_shape_t;

/* shape->flags: a training step's forward keeps, in its workspace, the chunk
 * states, carry-in states, chunk decays, per-token decay sums and Gram tiles
 * that the backward of the same inputs needs; the backward, given the same
 * workspace with the same flag, takes them from there instead of forming
 * them again.  Only for shapes without a convolution (conv_width 0). */
#define BISSD_SAVE 1

/* One scan direction's parameters.  Without dt_bias, dt is the step itself
 * (already positive).  With dt_bias, dt holds the mixer's pre-activation and
 * every kernel reads the step as Mamba-2 forms it,
 *     dt_step[b][t][h] = clamp(softplus(dt[b][t][h] + dt_bias[h]), dt_min, dt_max),
 * in fp32, without a separate pass over dt. */
typedef struct {
  const void *dt;         /* [Z][L][H] dtype */
  const float *A;         /* [H] fp32, the per-head scalar decay rate (A <= 0) */
  const void *B;          /* [Z][L][G][N] dtype */
  const void *C;          /* [Z][L][G][N] dtype */
  const float *dt_bias;   /* [H] fp32, or NULL: no post-processing */
  float dt_min, dt_max;   /* clamp range with dt_bias: 0 <= dt_min <= dt_max
                             (INFINITY for no upper bound) */
  const float *conv_w;    /* [H][P][conv_width] fp32 taps, or NULL: the scan reads x
                             as given (requires shape->conv_width > 0 when set) */
  const float *conv_b;    /* [H][P] fp32 bias, or NULL: none */
  int32_t conv_act;       /* 1: SiLU after the convolution (Mamba-2's); 0: none */
  int32_t reserved;       /* must be 0 */
} bissd_dir_t;

/* One direction's parameter gradients (all fp32, overwritten). */
typedef struct {
  float *ddt;       /* [Z][L][H]; with dt_bias, the gradient of the pre-activation dt
                       (zero where the clamp holds the step at a bound) */
  float *dA;        /* [H], summed over batch and time */
  float *dB;        /* [Z][L][G][N], summed over the heads of each group */
  float *dC;        /* [Z][L][G][N], summed over the heads of each group */
  float *ddt_bias;  /* [H], summed over batch and time: required when the
                       direction has dt_bias, ignored otherwise */
} bissd_grad_t;

/*
 * Bytes of device workspace that `op` needs for `shape` (0 on a bad shape).
 * The workspace holds the per-chunk states and carries (compute dtype), the
 * chunk decays and the chunk Gram tiles C.B^T (compute dtype), plus the backward
 * pass's adjoint and reduction buffers; it is overwritten by every call and
 * its contents between calls mean nothing -- except with BISSD_SAVE in
 * shape->flags, where BISSD_OP_FORWARD gives the backward's size and a
 * forward call leaves in it what a following bissd_backward reads.
 */
size_t bissd_workspace_size(const bissd_shape_t *shape, int op);

/*
 * Full-sequence bidirectional scan: y = yf + yr + D x.
 *   init_state  [Z][H][P][N] fp32 or NULL (zero): forward start state.
 *   final_state [Z][H][P][N] fp32 or NULL: receives the forward state after
 *               token L-1 (the cache a following block update continues from).
 *               May equal init_state.
 *   fwd.* and rev.* may point to the same buffers (weight-tied directions).
 *   y must not overlap any input.
 * With BISSD_SAVE in shape->flags (forward of a training step) the
 * workspace must hold bissd_workspace_size(shape, BISSD_OP_FORWARD) bytes
 * (the backward's size) and keeps, after the call, the chunk states, carry-in
 * states (forward direction from init_state), chunk decays, per-token decay
 * sums and Gram tiles for bissd_backward; a convolution is then not supported
 * (BISSD_ERR_UNSUPPORTED).
 */
int bissd_forward(const bissd_shape_t *shape, const void *x, bissd_dir_t fwd,
                  bissd_dir_t rev, const float *D, const float *init_state, void *y,
                  float *final_state, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * bissd_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors as
 * bissd_forward; the workspace is a static device array of
 * BISSD_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  Shapes whose workspace
 * (bissd_workspace_size(shape, BISSD_OP_FORWARD)) exceeds it are rejected
 * with BISSD_ERR_SCRATCH before anything is launched.  The call allocates
 * nothing (the array's device address on the current GPU is looked up on the
 * first call on that GPU: make that first call outside graph capture).
 * Runs on the current device, which must be the stream's.  Every call on one
 * GPU shares that GPU's array: calls that may overlap on one GPU (other
 * streams, other host threads) race on it and must be serialised by the
 * caller; calls on one stream are ordered.
 */
/* (shape->flags must be 0 here: the static array is no place to keep values
 * for a backward; BISSD_ERR_UNSUPPORTED otherwise.) */
int bissd_forward_noalloc(const bissd_shape_t *shape, const void *x, bissd_dir_t fwd,
                          bissd_dir_t rev, const float *D, const float *init_state, void *y,
                          float *final_state, void *stream);

/*
 * Training through the scan ("DiffMamba Checkpoints" model card, Model
 * details: the bidirectional backbone is trained end to end with AdamW in
 * bf16-mixed precision; "DiffuMamba", Training & Inference Strategy,
 * Objective: the denoiser is trained on the masked-diffusion objective; "Training Hybrid
 * Block Diffusion Language Models with Partial Bidirectionality",
 * Methodology: the full-block objective trains the same scan with the
 * block-segmented reverse).  The pages give no gradient formulas; these are
 * the plain reverse-mode derivatives of the recurrence above.
 *
 * Gradients of Loss = sum(dy * y) for y = bissd_forward(...) with the same
 * inputs (init_state optional and treated as a constant).  A direction with
 * a convolution (conv_w) is not supported here (BISSD_ERR_UNSUPPORTED):
 *   dx [Z][L][H][P] fp32; gfwd / grev: per-direction ddt, dA, dB, dC (fp32);
 *   dD [H] fp32.  All outputs are overwritten; dA, dB, dC and dD are
 *   reduced deterministically (no floating-point atomics).
 * With BISSD_SAVE in shape->flags the workspace must be the one a
 * bissd_forward call with the same shape (flag included), x, fwd, rev, D
 * and init_state filled, untouched since: its chunk states, carry-ins, decays
 * and Gram tiles are read instead of formed again, with the same results
 * bit for bit.  The library cannot check that contract.  The backward
 * overwrites them (one backward per saving forward).
 */
int bissd_backward(const bissd_shape_t *shape, const void *x, bissd_dir_t fwd,
                   bissd_dir_t rev, const float *D, const float *init_state,
                   const void *dy, float *dx, bissd_grad_t gfwd, bissd_grad_t grev,
                   float *dD, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Block update with partial bidirectionality on an active block of
 * shape->seqlen tokens (seqlen <= chunk):
 *   y_blk = yf(from state_in) + yr(block only) + D x_blk
 *   state_in  [Z][H][P][N] fp32: forward state after the last prefix token.
 *   state_out [Z][H][P][N] fp32 or NULL: forward state after the last block
 *             token (the next block's cache).  May equal state_in.
 *   conv_state_in  [Z][K-1][H][P] dtype or NULL (zeros): with a convolution
 *             (K = shape->conv_width > 1), the last K-1 x rows before the
 *             block, where the forward convolution continues from.
 *   conv_state_out [Z][K-1][H][P] dtype or NULL: receives the last K-1 x rows
 *             of [conv_state_in | x_blk] (the next block's conv state).  May
 *             equal conv_state_in.
 *   Both conv states are ignored when K <= 1.
 */
int bissd_block_update(const bissd_shape_t *shape, const float *state_in,
                       const void *x_blk, bissd_dir_t fwd, bissd_dir_t rev,
                       const float *D, void *y_blk, float *state_out,
                       const void *conv_state_in, void *conv_state_out, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * Diagnostics for timing and profiling single kernels: enqueue only one
 * phase of bissd_forward with the same arguments and validation.
 *   phase 0: per-chunk local states and chunk decays (written to workspace);
 *            with the convolution (conv_width > 0) first the convolution
 *            pass that writes both directions' convolved x to the workspace
 *   phase 3: per-chunk Gram tiles C.B^T of both directions (workspace);
 *            nothing to do when phase 0 forms them itself, which it does
 *            when every B/C group has at least (chunk/64)(chunk/64 + 1)/2
 *            head tiles (a tile is 2 heads if a group's head count is even,
 *            else 1)
 *   phase 1: carry pass over chunks (workspace in place; final_state)
 *   phase 2: fused bidirectional output (reads workspace, writes y)
 * bissd_forward runs them in the order 0, 3, 1, 2.  A phase reads what the
 * phases before it left in the same workspace, so phase 2 repeated after one
 * full bissd_forward recomputes the same y.
 * Phase 1 rewrites the workspace in place and is not idempotent.
 */
int bissd_forward_phase(const bissd_shape_t *shape, const void *x, bissd_dir_t fwd,
                        bissd_dir_t rev, const float *D, const float *init_state, void *y,
                        float *final_state, void *workspace, size_t workspace_bytes,
                        void *stream, int phase);

/*
 * Multi-head softmax attention of the hybrid backbones, which interleave
 * attention blocks with the bidirectional Mamba-2 blocks ("DiffMamba
 * Checkpoints" model card, Hybrid Mamba+attention checkpoints: full
 * bidirectional attention; "DiffuMamba: High-Throughput Diffusion LMs with
 * Mamba Backbone", Core Architecture: one multi-head attention block every
 * five Mamba blocks; "Training Hybrid Block Diffusion Language Models with
 * Partial Bidirectionality", Methodology: the block-wise BDLM attention).
 * Per batch row and head:
 *
 *   O = softmax(scale Q K^T + M) V      (softmax over the keys)
 *
 * M[t][s] = 0 where query t may see key s, -inf elsewhere: everywhere when
 * block == 0 (full bidirectional attention); with block > 0, where
 * floor(s / block) <= floor(t / block) (the query's block and the blocks
 * before it).
 *   shape  headdim == 64; block 0 or a multiple of 64; dtype BISSD_F32 or
 *          BISSD_BF16 (q, k, v and o); reserved 0.
 *   q, k, v, o  [batch][seqlen][nheads][headdim] device pointers, 16-byte
 *          aligned; o must not overlap q, k or v.
 *   scale  > 0, or 0 for 1 / sqrt(headdim).
 *   lse    [batch][nheads][seqlen] fp32 or NULL: receives each query's
 *          log2-sum-exp of its scaled scores, log2 sum_s 2^(scale log2(e) S[t][s]),
 *          which bissd_attention_backward needs.
 * Scores, softmax and the P V accumulation are fp32; o is rounded once.
 * Asynchronous on `stream`; allocates nothing; status codes as above.
 */
typedef struct {
  int64_t batch;    /* Z */
  int64_t seqlen;   /* L */
  int64_t nheads;   /* H (q, k and v have the same heads) */
  int64_t headdim;  /* 64 */
  int64_t block;    /* 0: full bidirectional; > 0: block-wise, blocks of this many tokens */
  int32_t dtype;    /* BISSD_F32 or BISSD_BF16 */
  int32_t reserved; /* must be 0 */
} bissd_attn_shape_t;

int bissd_attention_forward(const bissd_attn_shape_t *shape, const void *q, const void *k,
                            const void *v, float scale, void *o, float *lse, void *stream);

/* Bytes of workspace bissd_attention_backward needs (0 on a bad shape). */
size_t bissd_attention_workspace_size(const bissd_attn_shape_t *shape);

/*
 * Gradients of Loss = sum(dout * o) for o = bissd_attention_forward(q, k, v)
 * (the reverse mode of softmax attention: dV = P^T dO, dS = P (dO V^T - D)
 * with D_t = dO_t . o_t, dQ = scale dS K, dK = scale dS^T Q).
 *   o, lse   the forward's output and log2-sum-exp (same q, k, v, shape, scale)
 *   dout     [batch][seqlen][nheads][headdim], dtype
 *   dq, dk, dv  [batch][seqlen][nheads][headdim] fp32, overwritten
 *   workspace   bissd_attention_workspace_size(shape) bytes
 * Every sum has a fixed order (no atomics): bitwise reproducible.  None of
 * the outputs may overlap an input, the workspace or each other.
 */
int bissd_attention_backward(const bissd_attn_shape_t *shape, const void *q, const void *k,
                             const void *v, const void *o, const void *dout, const float *lse,
                             float scale, float *dq, float *dk, float *dv, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Text of a status code (static storage). */
const char *bissd_status_string(int status);

/* The hipError_t of the last BISSD_ERR_HIP on the calling thread (0 if none). */
int bissd_last_hip_error(void);

/*
 * Kernel timers, for benchmarks that need one kernel's duration inside a
 * sequence of calls without a marker between kernels.  Every kernel the
 * library launches goes through hipExtLaunchKernelGGL; bissd_timer_arm(slot)
 * hands slot `slot`'s pair of HIP events to the NEXT kernel launch the
 * library makes in this process, on any stream and from any call, which
 * records its dispatch's start and end timestamps in them; the slot is then
 * disarmed.  Arming replaces a slot armed before; slot -1 disarms.  The
 * events are created on a slot's first arming on the current device (again
 * when the slot is armed on another device) and kept until the process
 * ends.  bissd_timer_read(slot, &ms) waits for the
 * slot's end event and returns the kernel's duration in milliseconds
 * (BISSD_ERR_HIP if that slot has recorded nothing).  Process-wide state:
 * callers that launch from several threads at once get no defined pairing.
 *   slot  0 <= slot < BISSD_TIMER_SLOTS (or -1 for bissd_timer_arm)
 */
#define BISSD_TIMER_SLOTS 4096
int bissd_timer_arm(int32_t slot);
int bissd_timer_read(int32_t slot, float *ms);

/* ABI version: 4 (3 had a reserved field in place of bissd_shape_t.flags, 2 no
 * convolution fields, 1 no dt post-processing fields). */
int bissd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BISSD_H */
