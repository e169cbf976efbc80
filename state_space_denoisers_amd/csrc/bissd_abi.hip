// bissd_abi.hip -- the C ABI of the bidirectional SSD scan (include/bissd.h):
// argument validation, workspace carving and launch sequencing.  Every check
// runs on the host before anything is enqueued, so a rejected call launches
// nothing and touches no output.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "bissd.h"
#include "bissd_internal.hpp"

using bissd::ScanArgs;

// Workspace of bissd_forward_noalloc, for callers that cannot allocate:
// one array on every GPU the library runs on, held until the process ends.
// In host code `scratch` only names the symbol; its device address on the
// current GPU comes from hipGetSymbolAddress (scratch_address below), and
// only that address is ever handed to a kernel or a copy.
static __device__ __align__(256) char scratch[BISSD_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip = 0;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_at[kMaxDevices] = {};

// Device address of the scratch array on the current GPU, looked up once per
// device (with that device current) and kept.
int scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    return BISSD_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return BISSD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_at[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_hip = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return BISSD_ERR_HIP;
    }
    g_scratch_at[dev] = p;
  }
  *out = g_scratch_at[dev];
  return BISSD_OK;
}

constexpr int64_t kMaxElems = (int64_t)1 << 40;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const bissd_shape_t *s, int op) {
  if (!s) return BISSD_ERR_NULL;
  if (s->batch <= 0 || s->seqlen <= 0 || s->nheads <= 0 || s->headdim <= 0 || s->dstate <= 0 ||
      s->ngroups <= 0 || s->chunk <= 0)
    return BISSD_ERR_SHAPE;
  if (s->nheads % s->ngroups != 0) return BISSD_ERR_SHAPE;
  if (s->rev_block < 0 || s->conv_width < 0 || (s->flags & ~BISSD_SAVE) != 0) return BISSD_ERR_SHAPE;
  if (s->conv_width > 4) return BISSD_ERR_UNSUPPORTED;
  if (op != BISSD_OP_FORWARD && op != BISSD_OP_BACKWARD && op != BISSD_OP_BLOCK)
    return BISSD_ERR_UNSUPPORTED;
  // values kept for a backward: forward and backward only, no convolution
  if ((s->flags & BISSD_SAVE) && (op == BISSD_OP_BLOCK || s->conv_width > 0))
    return BISSD_ERR_UNSUPPORTED;
  // the reverse blocks are whole 64-token tiles and either split a chunk
  // evenly or span whole chunks
  if (s->rev_block > 0 && (op == BISSD_OP_BLOCK || s->rev_block % 64 != 0 ||
                           (s->chunk % s->rev_block != 0 && s->rev_block % s->chunk != 0)))
    return BISSD_ERR_UNSUPPORTED;
  if (s->headdim != 64) return BISSD_ERR_UNSUPPORTED;
  if (s->dstate != 64 && s->dstate != 128) return BISSD_ERR_UNSUPPORTED;
  if (s->chunk != 64 && s->chunk != 128 && s->chunk != 256) return BISSD_ERR_UNSUPPORTED;
  if (s->dtype != BISSD_F32 && s->dtype != BISSD_BF16) return BISSD_ERR_UNSUPPORTED;
  if (op == BISSD_OP_BLOCK && s->seqlen > s->chunk) return BISSD_ERR_SHAPE;
  // grid and index limits
  if (s->batch > (1 << 20) || s->nheads > 4096 || s->seqlen > ((int64_t)1 << 31))
    return BISSD_ERR_UNSUPPORTED;
  const int64_t nc = ceil_div(s->seqlen, s->chunk);
  if (s->batch * nc * (s->chunk / 64) * 2 * s->nheads >= ((int64_t)1 << 31)) return BISSD_ERR_UNSUPPORTED;
  const int64_t nrb = s->chunk / 64;
  if (s->batch * nc * 2 * s->ngroups * (nrb * (nrb + 1) / 2) >= ((int64_t)1 << 31))
    return BISSD_ERR_UNSUPPORTED;
  // per-batch-row buffer resources address at most 4 GiB
  if (s->seqlen * s->nheads * s->headdim * 4 >= ((int64_t)1 << 32)) return BISSD_ERR_UNSUPPORTED;
  if (s->seqlen * s->ngroups * s->dstate * 4 >= ((int64_t)1 << 32)) return BISSD_ERR_UNSUPPORTED;
  if (s->batch * s->seqlen * s->nheads * s->headdim > kMaxElems) return BISSD_ERR_UNSUPPORTED;
  return BISSD_OK;
}

// Workspace: chunk-local states and the carry-in states, both in the compute
// dtype (no carry-in buffer for the block update, which reads its fp32 start
// state directly), the chunk log2-decays, and the chunk Gram tiles C.B^T of
// both slots (compute dtype; none for a block update of at most 64 tokens, whose
// single kernel forms them itself).  The backward pass adds a
// second chunk-state buffer (A-tangent chunk states, then adjoint chunk
// states), the
// A-tangent and adjoint carries (compute dtype), chunk dt sums, the
// per-token dy.y_d and x.(G_t B_t) values (fp32 [2][Z][L][H]), each
// token's in-chunk decay sum and cumulative dt (fp32 [2][Z][H][L]) and the
// partial sums of the reductions.
struct WsLayout {
  size_t states = 0, sin_t = 0, cdecay = 0, gram = 0, xc = 0, xc_bytes = 0;
  size_t tstates = 0, sa_t = 0, gin_t = 0, dtsum = 0, ydot = 0, qx = 0, qxs = 0, ddpart = 0, dAintra = 0,
         dAx1 = 0, rpart = 0, lamg = 0, cdtg = 0, dbpart = 0;
  size_t total = 0;
};

WsLayout ws_layout(const bissd_shape_t *s, int op) {
  WsLayout w;
  // a forward that keeps values for the backward writes them where the
  // backward reads them: it takes the backward's layout
  if (op == BISSD_OP_FORWARD && (s->flags & BISSD_SAVE)) op = BISSD_OP_BACKWARD;
  const int64_t nc = op == BISSD_OP_BLOCK ? 1 : ceil_div(s->seqlen, s->chunk);
  const int64_t ndir = op == BISSD_OP_BLOCK ? 1 : 2;
  const size_t nst = (size_t)(ndir * s->batch * nc * s->nheads * s->headdim * s->dstate);
  const size_t esz = s->dtype == BISSD_BF16 ? 2 : 4;
  const size_t cd = (size_t)(ndir * s->batch * nc * s->nheads) * 4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  w.states = take(nst * esz);
  if (op != BISSD_OP_BLOCK) w.sin_t = take(nst * esz);
  // the directions' convolved x (the convolution pass's output), except for
  // a block of at most 64 tokens, whose single kernel forms it in LDS
  if (s->conv_width > 0 && op != BISSD_OP_BACKWARD && (op == BISSD_OP_FORWARD || s->seqlen > 64)) {
    w.xc_bytes = align256((size_t)(s->batch * s->seqlen * s->nheads * s->headdim) * esz);
    w.xc = take(2 * w.xc_bytes);
  }
  w.cdecay = take(cd);
  if (op != BISSD_OP_BLOCK || s->seqlen > 64)
    w.gram = take((size_t)(2 * s->batch * nc * s->ngroups) * (size_t)(s->chunk * s->chunk) * esz);
  if (op == BISSD_OP_BACKWARD) {
    const size_t tok = (size_t)(2 * s->batch * s->seqlen * s->nheads) * 4;
    const size_t rb = (size_t)(s->batch * nc * (s->chunk / 64) * s->nheads) * 4;
    w.tstates = take(nst * esz);
    w.sa_t = take(nst * esz);
    w.gin_t = take(nst * esz);
    w.dtsum = take(cd);
    w.ydot = take(tok);
    w.qx = take(tok);
    w.qxs = take(tok);
    w.ddpart = take(rb);
    w.dAintra = take(2 * rb);
    w.dAx1 = take(cd);
    w.rpart = take(cd * (size_t)(s->headdim * s->dstate / 256));
    w.lamg = take(tok);
    w.cdtg = take(tok);
    w.dbpart = take(cd);
  }
  w.total = o;
  return w;
}

size_t esize(const bissd_shape_t *s) { return s->dtype == BISSD_BF16 ? 2 : 4; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

struct Sizes {
  size_t x, dt, bc, vec, state, cw, cb, cst;
};

Sizes sizes(const bissd_shape_t *s) {
  Sizes z;
  const size_t e = esize(s);
  z.x = (size_t)(s->batch * s->seqlen * s->nheads * s->headdim) * e;
  z.dt = (size_t)(s->batch * s->seqlen * s->nheads) * e;
  z.bc = (size_t)(s->batch * s->seqlen * s->ngroups * s->dstate) * e;
  z.vec = (size_t)s->nheads * 4;
  z.state = (size_t)(s->batch * s->nheads * s->headdim * s->dstate) * 4;
  z.cw = (size_t)(s->nheads * s->headdim * (s->conv_width > 0 ? s->conv_width : 0)) * 4;
  z.cb = (size_t)(s->nheads * s->headdim) * 4;
  z.cst = (size_t)(s->batch * (s->conv_width > 1 ? s->conv_width - 1 : 0) * s->nheads * s->headdim) * e;
  return z;
}

int check_dir(const bissd_dir_t &d, const bissd_shape_t *s) {
  if (!d.dt || !d.A || !d.B || !d.C) return BISSD_ERR_NULL;
  if (!aligned16(d.dt) || !aligned16(d.A) || !aligned16(d.B) || !aligned16(d.C) ||
      (d.dt_bias && !aligned16(d.dt_bias)) || (d.conv_w && !aligned16(d.conv_w)) ||
      (d.conv_b && !aligned16(d.conv_b)))
    return BISSD_ERR_ALIGN;
  // the convolution: taps need a width; a bias or activation needs taps
  if (d.reserved != 0 || (d.conv_act != 0 && d.conv_act != 1)) return BISSD_ERR_SHAPE;
  if (d.conv_w && s->conv_width <= 0) return BISSD_ERR_SHAPE;
  if (!d.conv_w && (d.conv_b || d.conv_act)) return BISSD_ERR_SHAPE;
  // clamp range of the dt post-processing (NaN fails every comparison)
  if (d.dt_bias && !(d.dt_min >= 0.0f && d.dt_max >= d.dt_min)) return BISSD_ERR_SHAPE;
  return BISSD_OK;
}

// true if `out` (n bytes) overlaps any input of the scan
bool hits_inputs(const void *out, size_t n, const Sizes &z, const void *x, const bissd_dir_t &f,
                 const bissd_dir_t &r, const float *D) {
  const void *bufs[] = {x, f.dt, f.A, f.B, f.C, r.dt, r.A, r.B, r.C, D, f.dt_bias, r.dt_bias,
                        f.conv_w, f.conv_b, r.conv_w, r.conv_b};
  const size_t lens[] = {z.x, z.dt, z.vec, z.bc, z.bc, z.dt, z.vec, z.bc, z.bc, z.vec, z.vec, z.vec,
                         z.cw, z.cb, z.cw, z.cb};
  for (int i = 0; i < 16; ++i)
    if (overlap(out, n, bufs[i], lens[i])) return true;
  return false;
}

// The block-segmented reverse in the kernels' terms: chunks per reverse
// block (1 when a block is no longer than a chunk, so that every chunk
// boundary restarts the reverse scan; 0 without segmentation) and 64-token
// tiles per block when a block is shorter than a chunk (0 otherwise).
void set_rev_blocks(const bissd_shape_t *s, int &chunks, int &tiles) {
  chunks = tiles = 0;
  if (s->rev_block <= 0 || s->rev_block >= s->seqlen) return;
  chunks = s->rev_block >= s->chunk ? (int)(s->rev_block / s->chunk) : 1;
  tiles = s->rev_block < s->chunk ? (int)(s->rev_block / 64) : 0;
}

ScanArgs base_args(const bissd_shape_t *s, const void *x, const bissd_dir_t &f,
                   const bissd_dir_t &r, const float *D) {
  ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.dt[0] = f.dt;
  a.dt[1] = r.dt;
  const bissd_dir_t *dirs[2] = {&f, &r};
  for (int d = 0; d < 2; ++d) {
    a.dtb[d] = dirs[d]->dt_bias;
    a.dtlo[d] = dirs[d]->dt_min;
    a.dthi[d] = dirs[d]->dt_max;
  }
  a.A[0] = f.A;
  a.A[1] = r.A;
  a.B[0] = f.B;
  a.B[1] = r.B;
  a.C[0] = f.C;
  a.C[1] = r.C;
  a.D = D;
  a.L = s->seqlen;
  a.Z = (int)s->batch;
  a.H = (int)s->nheads;
  a.G = (int)s->ngroups;
  a.N = (int)s->dstate;
  a.chunk = (int)s->chunk;
  a.dtype = s->dtype;
  set_rev_blocks(s, a.rseg_chunks, a.rseg_tiles);
  return a;
}

// The directions' convolved x for one call (directions without taps read x
// itself): one pass over x into the workspace's xc region.
hipError_t run_conv(const bissd_shape_t *s, const void *x, const bissd_dir_t &f, const bissd_dir_t &r,
                    const void *state, char *ws, const WsLayout &wl, ScanArgs &a, hipStream_t st) {
  if (!f.conv_w && !r.conv_w) return hipSuccess;
  bissd::ConvArgs c;
  memset(&c, 0, sizeof(c));
  c.x = x;
  const bissd_dir_t *dirs[2] = {&f, &r};
  for (int d = 0; d < 2; ++d) {
    if (!dirs[d]->conv_w) continue;
    c.xc[d] = ws + wl.xc + d * wl.xc_bytes;
    c.w[d] = dirs[d]->conv_w;
    c.b[d] = dirs[d]->conv_b;
    c.act[d] = dirs[d]->conv_act;
    a.xs[d] = c.xc[d];
  }
  c.state = state;
  c.L = s->seqlen;
  c.Z = (int)s->batch;
  c.HP = (int)(s->nheads * s->headdim);
  c.K = (int)s->conv_width;
  c.dtype = s->dtype;
  c.rev_block = (s->rev_block > 0 && s->rev_block < s->seqlen) ? s->rev_block : 0;
  return bissd::launch_conv(c, st);
}

int finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    return BISSD_ERR_HIP;
  }
  return BISSD_OK;
}

// Kernel timers: per slot a pair of events and the device they were created
// on (created on the slot's first arming on that device), and the one armed
// slot (-1: none; read without the lock by every launch, so a launch with
// no timer armed takes no lock).
std::mutex g_timer_mu;
hipEvent_t g_timer_ev[BISSD_TIMER_SLOTS][2] = {};
int g_timer_dev[BISSD_TIMER_SLOTS] = {};
std::atomic<int> g_timer_armed{-1};

}  // namespace

void bissd::take_timer(hipEvent_t *start, hipEvent_t *stop) {
  if (g_timer_armed.load(std::memory_order_relaxed) < 0) return;
  std::lock_guard<std::mutex> lock(g_timer_mu);
  const int slot = g_timer_armed.load(std::memory_order_relaxed);
  if (slot < 0) return;
  *start = g_timer_ev[slot][0];
  *stop = g_timer_ev[slot][1];
  g_timer_armed.store(-1, std::memory_order_relaxed);
}

extern "C" {

int bissd_version(void) { return 4; }

int bissd_last_hip_error(void) { return g_last_hip; }

int bissd_timer_arm(int32_t slot) {
  if (slot < -1 || slot >= BISSD_TIMER_SLOTS) return BISSD_ERR_SHAPE;
  std::lock_guard<std::mutex> lock(g_timer_mu);
  if (slot >= 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
      g_last_hip = (int)e;
      return BISSD_ERR_HIP;
    }
    // events belong to the device they were created on: a slot armed on
    // another device gets new ones
    if (g_timer_ev[slot][0] && g_timer_dev[slot] != dev) {
      for (int i = 0; i < 2; ++i) {
        (void)hipEventDestroy(g_timer_ev[slot][i]);
        g_timer_ev[slot][i] = nullptr;
      }
    }
    for (int i = 0; i < 2; ++i)
      if (!g_timer_ev[slot][i]) {
        e = hipEventCreate(&g_timer_ev[slot][i]);
        if (e != hipSuccess) {
          g_timer_ev[slot][i] = nullptr;
          g_last_hip = (int)e;
          return BISSD_ERR_HIP;
        }
      }
    g_timer_dev[slot] = dev;
  }
  g_timer_armed.store(slot, std::memory_order_relaxed);
  return BISSD_OK;
}

int bissd_timer_read(int32_t slot, float *ms) {
  if (!ms) return BISSD_ERR_NULL;
  if (slot < 0 || slot >= BISSD_TIMER_SLOTS) return BISSD_ERR_SHAPE;
  hipEvent_t e0, e1;
  {
    std::lock_guard<std::mutex> lock(g_timer_mu);
    e0 = g_timer_ev[slot][0];
    e1 = g_timer_ev[slot][1];
  }
  if (!e0 || !e1) return BISSD_ERR_NULL;
  hipError_t e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
  return finish(e);
}

const char *bissd_status_string(int status) {
  switch (status) {
    case BISSD_OK: return "ok";
    case BISSD_ERR_NULL: return "a required pointer is NULL";
    case BISSD_ERR_SHAPE: return "bad shape";
    case BISSD_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case BISSD_ERR_ALIGN: return "pointer not aligned to 16 bytes";
    case BISSD_ERR_WORKSPACE: return "workspace missing or too small";
    case BISSD_ERR_HIP: return "HIP launch failed";
    case BISSD_ERR_ALIAS: return "an output overlaps an input";
    case BISSD_ERR_SCRATCH:
      return "the shape needs more workspace than bissd_forward_noalloc's scratch array "
             "(BISSD_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown status";
  }
}

size_t bissd_workspace_size(const bissd_shape_t *s, int op) {
  if (check_shape(s, op) != BISSD_OK) return 0;
  return ws_layout(s, op).total;
}

static int forward_impl(const bissd_shape_t *s, const void *x, bissd_dir_t fwd, bissd_dir_t rev,
                        const float *D, const float *init_state, void *y, float *final_state,
                        void *workspace, size_t workspace_bytes, void *stream, int phase) {
  int rc = check_shape(s, BISSD_OP_FORWARD);
  if (rc) return rc;
  if (!x || !D || !y) return BISSD_ERR_NULL;
  if ((rc = check_dir(fwd, s)) || (rc = check_dir(rev, s))) return rc;
  if (!aligned16(x) || !aligned16(D) || !aligned16(y) ||
      (init_state && !aligned16(init_state)) || (final_state && !aligned16(final_state)))
    return BISSD_ERR_ALIGN;
  const WsLayout wl = ws_layout(s, BISSD_OP_FORWARD);
  if (!workspace || workspace_bytes < wl.total) return BISSD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BISSD_ERR_ALIGN;
  const Sizes z = sizes(s);
  if (hits_inputs(y, z.x, z, x, fwd, rev, D) || overlap(y, z.x, init_state, z.state) ||
      overlap(y, z.x, final_state, z.state) || overlap(y, z.x, workspace, wl.total))
    return BISSD_ERR_ALIAS;
  if (final_state && (hits_inputs(final_state, z.state, z, x, fwd, rev, D) ||
                      overlap(final_state, z.state, workspace, wl.total)))
    return BISSD_ERR_ALIAS;
  if (hits_inputs(workspace, wl.total, z, x, fwd, rev, D) ||
      overlap(workspace, wl.total, init_state, z.state))
    return BISSD_ERR_ALIAS;

  hipStream_t st = (hipStream_t)stream;
  ScanArgs a = base_args(s, x, fwd, rev, D);
  char *ws = (char *)workspace;
  a.states = (void *)(ws + wl.states);
  a.cdecay = (float *)(ws + wl.cdecay);
  a.gram = (void *)(ws + wl.gram);
  a.gram_k1 = bissd::gram_in_k1(a.H, a.G, a.chunk) ? 1 : 0;
  a.nchunks = (int)ceil_div(s->seqlen, s->chunk);
  a.y = y;
  a.dir0 = 0;
  a.ndir = 2;
  a.init_state = init_state;
  a.final_state = final_state;
  const bool save = (s->flags & BISSD_SAVE) != 0;
  // kept for the backward: every chunk state and carry-in (no edge skipped)
  // and every token's decay sum
  a.skip_edges = save ? 0 : 1;
  if (save) a.cum_out = (float *)(ws + wl.lamg);
  const int64_t PN = s->headdim * s->dstate;
  a.sin_t = ws + wl.sin_t;
  const size_t esz = s->dtype == BISSD_BF16 ? 2 : 4;
  for (int d = 0; d < 2; ++d) {
    a.sin[d] = (const char *)a.sin_t + (size_t)d * a.Z * a.nchunks * a.H * PN * esz;
    a.sin_bstride[d] = (int64_t)a.nchunks * a.H * PN;
    a.sin_cstride[d] = (int64_t)a.H * PN;
    a.sin_f32[d] = 0;
  }
  // chunk states, Gram tiles (phase 3; formed by the chunk-state kernel
  // itself when the head tiles suffice), carry pass, output
  const int order[4][2] = {{0, bissd::PHASE_CHUNK_STATE},
                           {3, bissd::PHASE_GRAM},
                           {1, bissd::PHASE_STATE_PASS},
                           {2, bissd::PHASE_CHUNK_OUT}};
  // the directions' convolved x (part of phase 0 when timing phases)
  hipError_t e = hipSuccess;
  if (phase < 0 || phase == 0) e = run_conv(s, x, fwd, rev, nullptr, ws, wl, a, st);
  else if (fwd.conv_w || rev.conv_w) {
    for (int d = 0; d < 2; ++d)
      if ((d == 0 ? fwd : rev).conv_w) a.xs[d] = ws + wl.xc + d * wl.xc_bytes;
  }
  for (int i = 0; i < 4 && e == hipSuccess; ++i) {
    if (order[i][1] == bissd::PHASE_GRAM && a.gram_k1) continue;
    if (phase < 0 || phase == order[i][0]) e = bissd::launch_scan_phase(a, order[i][1], st);
  }
  return finish(e);
}

int bissd_forward(const bissd_shape_t *s, const void *x, bissd_dir_t fwd, bissd_dir_t rev,
                  const float *D, const float *init_state, void *y, float *final_state,
                  void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(s, x, fwd, rev, D, init_state, y, final_state, workspace, workspace_bytes,
                      stream, -1);
}

int bissd_forward_noalloc(const bissd_shape_t *s, const void *x, bissd_dir_t fwd, bissd_dir_t rev,
                          const float *D, const float *init_state, void *y, float *final_state,
                          void *stream) {
  int rc = check_shape(s, BISSD_OP_FORWARD);
  if (rc) return rc;
  if (s->flags & BISSD_SAVE) return BISSD_ERR_UNSUPPORTED;
  // the forward's workspace needs no zeroing: every kernel writes what a
  // later one reads before it is read, in this call
  const size_t need = ws_layout(s, BISSD_OP_FORWARD).total;
  if (need > (size_t)BISSD_NOALLOC_SCRATCH_BYTES) return BISSD_ERR_SCRATCH;
  void *ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return forward_impl(s, x, fwd, rev, D, init_state, y, final_state, ws,
                      (size_t)BISSD_NOALLOC_SCRATCH_BYTES, stream, -1);
}

int bissd_forward_phase(const bissd_shape_t *s, const void *x, bissd_dir_t fwd, bissd_dir_t rev,
                        const float *D, const float *init_state, void *y, float *final_state,
                        void *workspace, size_t workspace_bytes, void *stream, int phase) {
  if (phase < 0 || phase > 3) return BISSD_ERR_UNSUPPORTED;
  return forward_impl(s, x, fwd, rev, D, init_state, y, final_state, workspace, workspace_bytes,
                      stream, phase);
}

int bissd_block_update(const bissd_shape_t *s, const float *state_in, const void *x_blk,
                       bissd_dir_t fwd, bissd_dir_t rev, const float *D, void *y_blk,
                       float *state_out, const void *conv_state_in, void *conv_state_out,
                       void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_shape(s, BISSD_OP_BLOCK);
  if (rc) return rc;
  if (!state_in || !x_blk || !D || !y_blk) return BISSD_ERR_NULL;
  if ((rc = check_dir(fwd, s)) || (rc = check_dir(rev, s))) return rc;
  if (!aligned16(state_in) || !aligned16(x_blk) || !aligned16(D) || !aligned16(y_blk) ||
      (state_out && !aligned16(state_out)) || (conv_state_in && !aligned16(conv_state_in)) ||
      (conv_state_out && !aligned16(conv_state_out)))
    return BISSD_ERR_ALIGN;
  // the conv states take part only with a convolution wider than one tap
  if (s->conv_width <= 1) conv_state_in = conv_state_out = nullptr;
  const WsLayout wl = ws_layout(s, BISSD_OP_BLOCK);
  if (!workspace || workspace_bytes < wl.total) return BISSD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BISSD_ERR_ALIGN;
  const Sizes z = sizes(s);
  if (hits_inputs(y_blk, z.x, z, x_blk, fwd, rev, D) || overlap(y_blk, z.x, state_in, z.state) ||
      overlap(y_blk, z.x, state_out, z.state) || overlap(y_blk, z.x, workspace, wl.total))
    return BISSD_ERR_ALIAS;
  if (state_out && (hits_inputs(state_out, z.state, z, x_blk, fwd, rev, D) ||
                    overlap(state_out, z.state, workspace, wl.total)))
    return BISSD_ERR_ALIAS;
  // state_out may equal state_in, but may not partially overlap it
  if (state_out && state_out != state_in && overlap(state_out, z.state, state_in, z.state))
    return BISSD_ERR_ALIAS;
  if (hits_inputs(workspace, wl.total, z, x_blk, fwd, rev, D) ||
      overlap(workspace, wl.total, state_in, z.state))
    return BISSD_ERR_ALIAS;
  // conv_state_out may equal conv_state_in, but overlaps no other buffer
  if (conv_state_out) {
    const void *others[] = {y_blk, state_out, state_in, workspace};
    const size_t olens[] = {z.x, z.state, z.state, wl.total};
    if (hits_inputs(conv_state_out, z.cst, z, x_blk, fwd, rev, D)) return BISSD_ERR_ALIAS;
    for (int i = 0; i < 4; ++i)
      if (overlap(conv_state_out, z.cst, others[i], olens[i])) return BISSD_ERR_ALIAS;
    if (conv_state_out != conv_state_in && overlap(conv_state_out, z.cst, conv_state_in, z.cst))
      return BISSD_ERR_ALIAS;
  }
  if (conv_state_in && (overlap(conv_state_in, z.cst, y_blk, z.x) ||
                        overlap(conv_state_in, z.cst, state_out, z.state) ||
                        overlap(conv_state_in, z.cst, workspace, wl.total)))
    return BISSD_ERR_ALIAS;

  hipStream_t st = (hipStream_t)stream;
  ScanArgs a = base_args(s, x_blk, fwd, rev, D);
  char *ws = (char *)workspace;
  a.states = (void *)(ws + wl.states);
  a.cdecay = (float *)(ws + wl.cdecay);
  a.gram = (void *)(ws + wl.gram);
  a.nchunks = 1;
  a.y = y_blk;
  a.dir0 = 0;
  a.ndir = 1;  // the reverse carries nothing in or out of the block
  a.init_state = state_in;
  a.final_state = state_out;
  const int64_t PN = s->headdim * s->dstate;
  a.sin[0] = state_in;
  a.sin_bstride[0] = (int64_t)a.H * PN;
  a.sin_cstride[0] = 0;
  a.sin_f32[0] = 1;
  a.sin[1] = nullptr;
  a.sin_t = nullptr;
  // blocks of at most 64 tokens: one launch does everything
  if (s->seqlen <= 64) {
    if (s->conv_width > 0) {
      const bissd_dir_t *dirs[2] = {&fwd, &rev};
      for (int d = 0; d < 2; ++d) {
        a.cw[d] = dirs[d]->conv_w;
        a.cb[d] = dirs[d]->conv_b;
        a.cact[d] = dirs[d]->conv_act;
      }
      a.ckw = (int)s->conv_width;
      a.cst_in = conv_state_in;
      a.cst_out = conv_state_out;
    }
    return finish(bissd::launch_block_update(a, st));
  }
  // longer blocks: the convolution pass (the forward's taps before the block
  // read the conv state), then the chunked kernels; order matters when
  // state_out == state_in (the output phase reads state_in before the state
  // pass overwrites it) and when conv_state_out == conv_state_in (the
  // convolution pass reads the old conv state before it is replaced, last)
  hipError_t e = run_conv(s, x_blk, fwd, rev, conv_state_in, ws, wl, a, st);
  if (e == hipSuccess && state_out) e = bissd::launch_scan_phase(a, bissd::PHASE_CHUNK_STATE, st);
  if (e == hipSuccess) e = bissd::launch_scan_phase(a, bissd::PHASE_GRAM, st);
  if (e == hipSuccess) e = bissd::launch_scan_phase(a, bissd::PHASE_CHUNK_OUT, st);
  if (e == hipSuccess && state_out) e = bissd::launch_scan_phase(a, bissd::PHASE_STATE_PASS, st);
  if (e == hipSuccess && conv_state_out)
    e = bissd::launch_conv_state(x_blk, conv_state_in, conv_state_out, s->seqlen, (int)s->batch,
                                 (int)(s->nheads * s->headdim), (int)s->conv_width, s->dtype, st);
  return finish(e);
}

int bissd_backward(const bissd_shape_t *s, const void *x, bissd_dir_t fwd, bissd_dir_t rev,
                   const float *D, const float *init_state, const void *dy, float *dx,
                   bissd_grad_t gfwd, bissd_grad_t grev, float *dD, void *workspace,
                   size_t workspace_bytes, void *stream) {
  int rc = check_shape(s, BISSD_OP_BACKWARD);
  if (rc) return rc;
  if (!x || !D || !dy || !dx || !dD) return BISSD_ERR_NULL;
  if ((rc = check_dir(fwd, s)) || (rc = check_dir(rev, s))) return rc;
  // the gradients through the convolution are not formed
  if (fwd.conv_w || rev.conv_w) return BISSD_ERR_UNSUPPORTED;
  if (!gfwd.ddt || !gfwd.dA || !gfwd.dB || !gfwd.dC || !grev.ddt || !grev.dA || !grev.dB ||
      !grev.dC)
    return BISSD_ERR_NULL;
  if ((fwd.dt_bias && !gfwd.ddt_bias) || (rev.dt_bias && !grev.ddt_bias)) return BISSD_ERR_NULL;
  // the bias gradients take part only for directions with a dt bias
  float *dbf = fwd.dt_bias ? gfwd.ddt_bias : nullptr, *dbr = rev.dt_bias ? grev.ddt_bias : nullptr;
  const void *outs[] = {dx, gfwd.ddt, gfwd.dA, gfwd.dB, gfwd.dC,
                        grev.ddt, grev.dA, grev.dB, grev.dC, dD, dbf, dbr};
  if (!aligned16(x) || !aligned16(D) || !aligned16(dy) || (init_state && !aligned16(init_state)))
    return BISSD_ERR_ALIGN;
  for (const void *o : outs)
    if (o && !aligned16(o)) return BISSD_ERR_ALIGN;
  const WsLayout wl = ws_layout(s, BISSD_OP_BACKWARD);
  if (!workspace || workspace_bytes < wl.total) return BISSD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BISSD_ERR_ALIGN;
  const Sizes z = sizes(s);
  const size_t tokh = (size_t)(s->batch * s->seqlen * s->nheads) * 4;
  const size_t bcn = (size_t)(s->batch * s->seqlen * s->ngroups * s->dstate) * 4;
  const size_t olen[] = {z.x / esize(s) * 4, tokh, z.vec, bcn, bcn, tokh, z.vec, bcn, bcn, z.vec,
                         z.vec, z.vec};
  // outputs overlap neither an input, the workspace nor each other (absent
  // bias gradients overlap nothing)
  for (int i = 0; i < 12; ++i) {
    if (hits_inputs(outs[i], olen[i], z, x, fwd, rev, D) || overlap(outs[i], olen[i], dy, z.x) ||
        overlap(outs[i], olen[i], init_state, z.state) ||
        overlap(outs[i], olen[i], workspace, wl.total))
      return BISSD_ERR_ALIAS;
    for (int k = 0; k < i; ++k)
      if (overlap(outs[i], olen[i], outs[k], olen[k])) return BISSD_ERR_ALIAS;
  }
  if (hits_inputs(workspace, wl.total, z, x, fwd, rev, D) || overlap(workspace, wl.total, dy, z.x) ||
      overlap(workspace, wl.total, init_state, z.state))
    return BISSD_ERR_ALIAS;

  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)workspace;
  const int nc = (int)ceil_div(s->seqlen, s->chunk);
  const int64_t PN = s->headdim * s->dstate;
  const size_t esz = esize(s);
  const size_t dirst = (size_t)s->batch * nc * s->nheads * PN * esz;  // bytes per direction

  // primal chunk states and carry-ins
  ScanArgs a = base_args(s, x, fwd, rev, D);
  a.states = (void *)(ws + wl.states);
  a.cdecay = (float *)(ws + wl.cdecay);
  a.gram = (void *)(ws + wl.gram);
  a.gram_k1 = bissd::gram_in_k1(a.H, a.G, a.chunk) ? 1 : 0;
  a.nchunks = nc;
  a.dir0 = 0;
  a.ndir = 2;
  a.init_state = init_state;
  a.sin_t = ws + wl.sin_t;
  for (int d = 0; d < 2; ++d) {
    a.sin[d] = ws + wl.sin_t + d * dirst;
    a.sin_bstride[d] = (int64_t)nc * a.H * PN;
    a.sin_cstride[d] = (int64_t)a.H * PN;
  }
  // the primal chunk states also keep every token's decay sum for the
  // panels; a saving forward has left them (and the chunk decays, the Gram
  // tiles and the carry-ins) in the workspace
  const bool saved = (s->flags & BISSD_SAVE) != 0;
  ScanArgs a0 = a;
  a0.cum_out = (float *)(ws + wl.lamg);
  hipError_t e = saved ? hipSuccess : bissd::launch_scan_phase(a0, bissd::PHASE_CHUNK_STATE, st);

  // A-tangent chunk states (dt-sum weighted), chunk dt sums (and every
  // token's cumulative dt), and the A-tangent carry-ins S^A_in together with
  // the primal carry-ins S_in (the tangent's recurrence carries S_in anyway)
  ScanArgs ta = a;
  ta.states = (void *)(ws + wl.tstates);
  ta.out1 = (float *)(ws + wl.dtsum);
  ta.cum_out = (float *)(ws + wl.cdtg);
  if (e == hipSuccess) e = bissd::launch_scan_phase(ta, bissd::PHASE_TAN_STATE, st);
  ScanArgs tp = a;
  tp.states2 = (const void *)(ws + wl.tstates);
  tp.dtsum = (const float *)(ws + wl.dtsum);
  tp.sin_t = ws + wl.sa_t;
  tp.sin_prim = saved ? nullptr : a.sin_t;
  if (e == hipSuccess) e = bissd::launch_scan_phase(tp, bissd::PHASE_TAN_PASS, st);

  // adjoint chunk states sum_t 2^cum_t dy_t (outer) C_t (into the tangent
  // buffer, now consumed) with <G_loc, S^A_in>, then their carries with the
  // chunk-boundary inner products (the other cross-chunk part of dA,
  // <sum_t 2^cum_t T_t dy_t (outer) C_t, S_in>, comes with the dy.y_d pass)
  ScanArgs g = a;
  g.x = dy;
  g.B[0] = fwd.C;
  g.B[1] = rev.C;
  g.init_state = nullptr;
  g.states = (void *)(ws + wl.tstates);
  for (int d = 0; d < 2; ++d) g.sin[d] = ws + wl.sa_t + d * dirst;
  g.out0 = (float *)(ws + wl.dAx1);
  if (e == hipSuccess) e = bissd::launch_scan_phase(g, bissd::PHASE_ADJ_STATE, st);
  ScanArgs gp = g;
  for (int d = 0; d < 2; ++d) gp.sin[d] = a.sin[d];
  gp.sin_t = ws + wl.gin_t;
  gp.out0 = (float *)(ws + wl.rpart);
  if (e == hipSuccess) e = bissd::launch_scan_phase(gp, bissd::PHASE_ADJ_PASS, st);

  // dy.y_d per direction (forward output recomputed from the carry-ins)
  ScanArgs yd = a;
  yd.aux = dy;
  yd.out0 = (float *)(ws + wl.ydot);
  yd.cdt_in = (const float *)(ws + wl.cdtg);
  yd.dai_out = (float *)(ws + wl.dAintra);
  yd.slot_dir[0] = 0;
  yd.slot_dir[1] = 1;
  // the primal Gram tiles: from the chunk-state launch above, or here
  if (e == hipSuccess && !a.gram_k1 && !saved) e = bissd::launch_scan_phase(yd, bissd::PHASE_GRAM, st);
  if (e == hipSuccess) e = bissd::launch_scan_phase(yd, bissd::PHASE_YDOT, st);

  // dx and x.(G_t B_t): slot 0 (causal) takes the reverse direction's
  // adjoint, slot 1 the forward one; B and C trade places
  ScanArgs q = a;
  q.x = dy;
  q.aux = x;
  q.dt[0] = rev.dt;
  q.dtb[0] = rev.dt_bias;
  q.dtlo[0] = rev.dt_min;
  q.dthi[0] = rev.dt_max;
  q.dtb[1] = fwd.dt_bias;
  q.dtlo[1] = fwd.dt_min;
  q.dthi[1] = fwd.dt_max;
  q.A[0] = rev.A;
  q.B[0] = rev.C;
  q.C[0] = rev.B;
  q.dt[1] = fwd.dt;
  q.A[1] = fwd.A;
  q.B[1] = fwd.C;
  q.C[1] = fwd.B;
  q.sin[0] = ws + wl.gin_t + dirst;
  q.sin[1] = ws + wl.gin_t;
  q.out0 = (float *)(ws + wl.qx);
  q.out1 = dx;
  q.out2 = (float *)(ws + wl.ddpart);
  q.out3 = (float *)(ws + wl.qxs);
  q.slot_dir[0] = 1;
  q.slot_dir[1] = 0;
  // the Gram tiles of the swapped operands overwrite the primal ones, which
  // the dy.y_d launch above has consumed (stream order)
  if (e == hipSuccess) e = bissd::launch_scan_phase(q, bissd::PHASE_GRAM, st);
  if (e == hipSuccess) e = bissd::launch_scan_phase(q, bissd::PHASE_DX, st);

  bissd::BwdArgs b;
  memset(&b, 0, sizeof(b));
  b.x = x;
  b.dy = dy;
  b.dt[0] = fwd.dt;
  b.dt[1] = rev.dt;
  for (int d = 0; d < 2; ++d) {
    b.dtb[d] = a.dtb[d];
    b.dtlo[d] = a.dtlo[d];
    b.dthi[d] = a.dthi[d];
  }
  b.ddtb[0] = dbf;
  b.ddtb[1] = dbr;
  b.dbpart = (float *)(ws + wl.dbpart);
  b.A[0] = fwd.A;
  b.A[1] = rev.A;
  b.B[0] = fwd.B;
  b.B[1] = rev.B;
  b.C[0] = fwd.C;
  b.C[1] = rev.C;
  for (int d = 0; d < 2; ++d) {
    b.sin[d] = ws + wl.sin_t + d * dirst;
    b.gin[d] = ws + wl.gin_t + d * dirst;
  }
  b.st_bstride = (int64_t)nc * a.H * PN;
  b.st_cstride = (int64_t)a.H * PN;
  b.ydot = (const float *)(ws + wl.ydot);
  b.qx = (const float *)(ws + wl.qx);
  b.qxs = (const float *)(ws + wl.qxs);
  b.dB[0] = gfwd.dB;
  b.dB[1] = grev.dB;
  b.dC[0] = gfwd.dC;
  b.dC[1] = grev.dC;
  b.ddt[0] = gfwd.ddt;
  b.ddt[1] = grev.ddt;
  b.dA[0] = gfwd.dA;
  b.dA[1] = grev.dA;
  b.dD = dD;
  b.rpart = (const float *)(ws + wl.rpart);
  b.dAintra = (float *)(ws + wl.dAintra);
  b.dAx1 = (const float *)(ws + wl.dAx1);
  b.ddpart = (const float *)(ws + wl.ddpart);
  b.lamg = (const float *)(ws + wl.lamg);
  b.cdtg = (const float *)(ws + wl.cdtg);
  b.L = s->seqlen;
  b.Z = (int)s->batch;
  b.H = (int)s->nheads;
  b.G = (int)s->ngroups;
  b.N = (int)s->dstate;
  b.chunk = (int)s->chunk;
  b.nchunks = nc;
  b.dtype = s->dtype;
  b.rseg_tiles = a.rseg_tiles;
  if (e == hipSuccess) e = bissd::launch_bwd_panels(b, st);
  if (e == hipSuccess) e = bissd::launch_bwd_decay(b, st);
  return finish(e);
}

static int check_attn(const bissd_attn_shape_t *s, float scale) {
  if (!s) return BISSD_ERR_NULL;
  if (s->batch <= 0 || s->seqlen <= 0 || s->nheads <= 0 || s->headdim <= 0 || s->block < 0 ||
      s->reserved != 0 || !(scale >= 0.0f) || !isfinite(scale))
    return BISSD_ERR_SHAPE;
  if (s->headdim != bissd::kAttnD || s->block % 64 != 0) return BISSD_ERR_UNSUPPORTED;
  if (s->dtype != BISSD_F32 && s->dtype != BISSD_BF16) return BISSD_ERR_UNSUPPORTED;
  // one buffer resource per batch row (< 4 GiB, fp32 gradients included);
  // grid within 2^31
  if (s->batch > (1 << 20) || s->nheads > 4096 || s->seqlen * s->nheads * s->headdim * 4 >= ((int64_t)1 << 32))
    return BISSD_ERR_UNSUPPORTED;
  if (s->batch * s->nheads * ceil_div(s->seqlen, 64) >= ((int64_t)1 << 31)) return BISSD_ERR_UNSUPPORTED;
  return BISSD_OK;
}

static bissd::AttnArgs attn_args(const bissd_attn_shape_t *s, float scale) {
  bissd::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.L = s->seqlen;
  a.block = s->block;
  a.Z = (int)s->batch;
  a.H = (int)s->nheads;
  a.dtype = s->dtype;
  a.scale = scale > 0.0f ? scale : 1.0f / sqrtf((float)s->headdim);
  a.scale_log2 = a.scale * 1.4426950408889634f;
  return a;
}

int bissd_attention_forward(const bissd_attn_shape_t *s, const void *q, const void *k,
                            const void *v, float scale, void *o, float *lse, void *stream) {
  int rc = check_attn(s, scale);
  if (rc) return rc;
  if (!q || !k || !v || !o) return BISSD_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return BISSD_ERR_ALIGN;
  const size_t n = (size_t)(s->batch * s->seqlen * s->nheads * s->headdim * (s->dtype == BISSD_BF16 ? 2 : 4));
  const size_t nl = (size_t)(s->batch * s->nheads * s->seqlen) * 4;
  if (overlap(o, n, q, n) || overlap(o, n, k, n) || overlap(o, n, v, n)) return BISSD_ERR_ALIAS;
  if (lse && (overlap(lse, nl, q, n) || overlap(lse, nl, k, n) || overlap(lse, nl, v, n) ||
              overlap(lse, nl, o, n)))
    return BISSD_ERR_ALIAS;
  bissd::AttnArgs a = attn_args(s, scale);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  return finish(bissd::launch_attention(a, (hipStream_t)stream));
}

size_t bissd_attention_workspace_size(const bissd_attn_shape_t *s) {
  if (check_attn(s, 0.0f) != BISSD_OK) return 0;
  return align256((size_t)(s->batch * s->nheads * s->seqlen) * 4);
}

int bissd_attention_backward(const bissd_attn_shape_t *s, const void *q, const void *k,
                             const void *v, const void *o, const void *dout, const float *lse,
                             float scale, float *dq, float *dk, float *dv, void *workspace,
                             size_t workspace_bytes, void *stream) {
  int rc = check_attn(s, scale);
  if (rc) return rc;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return BISSD_ERR_NULL;
  const void *ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void *p : ptrs)
    if (!aligned16(p)) return BISSD_ERR_ALIGN;
  const size_t nws = bissd_attention_workspace_size(s);
  if (!workspace || workspace_bytes < nws) return BISSD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return BISSD_ERR_ALIGN;
  const size_t n = (size_t)(s->batch * s->seqlen * s->nheads * s->headdim * (s->dtype == BISSD_BF16 ? 2 : 4));
  const size_t n4 = (size_t)(s->batch * s->seqlen * s->nheads * s->headdim) * 4;
  const size_t nl = (size_t)(s->batch * s->nheads * s->seqlen) * 4;
  const void *ins[] = {q, k, v, o, dout, lse, workspace};
  const size_t inl[] = {n, n, n, n, n, nl, nws};
  float *outs[] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlap(outs[i], n4, ins[j], inl[j])) return BISSD_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], n4, outs[j], n4)) return BISSD_ERR_ALIAS;
  }
  for (int j = 0; j < 6; ++j)
    if (overlap(workspace, nws, ins[j], inl[j])) return BISSD_ERR_ALIAS;
  bissd::AttnArgs a = attn_args(s, scale);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = const_cast<void *>(o);
  a.lse = const_cast<float *>(lse);
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = (float *)workspace;
  return finish(bissd::launch_attention_backward(a, (hipStream_t)stream));
}

}  // extern "C"
