/*
 * ssd_oracle.c -- plain, sequential fp64 reference of the bidirectional
 * Mamba-2 (SSD) selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; it exists so that tests, the smoke check and the bench's
 * CPU-baseline leg can compare the GPU library against an obviously correct
 * recurrence.  It shares no code, header or constant with the GPU library.
 *
 * What it computes (each function names the passage it follows):
 *
 *   Per head h and direction d in {forward, reverse}, a state S (P x N)
 *   evolves as  S <- exp(dt_t * A_h) * S + dt_t * x_t (outer) B_t  and each
 *   visited token emits  y_t = S * C_t  (a P-vector).  The forward direction
 *   visits t = 0..L-1; the reverse direction is the same recurrence run over
 *   the flipped sequence (visits t = L-1..0) with its own dt, A, B and C, and
 *   its outputs are written back at their natural positions.  The layer
 *   output is the sum of both directions plus the skip D_h * x_t.
 *
 *   Sources: "DiffMamba Checkpoints" model card, section "Model details"
 *   (the backbone is a forward plus flipped-reverse Mamba-2); "DiffuMamba:
 *   High-Throughput Diffusion LMs with Mamba Backbone", Technical Summary,
 *   section 2 "Methodology / Core Architecture" (one forward and one backward
 *   Mamba-2 layer, combined by addition).  The recurrence, the per-direction
 *   dt/A/B/C and the D skip are the plain Mamba-2 scalar-decay state-space
 *   update that these pages name.
 *
 *   Block update ("Training Hybrid Block Diffusion Language Models with
 *   Partial Bidirectionality", Methodology / Technical Contribution / Novelty):
 *   the forward scan continues from a cached prefix state and the reverse scan
 *   is confined to the active block, starting from zero at the block end.
 *
 *   Block-segmented reverse (same page, Methodology and Key Results: the
 *   full-block training objective builds the same caches as inference).
 *   Read here as: over a whole training sequence every block of RB tokens is
 *   an active block for its own reverse scan, so the reverse state restarts
 *   from zero after the last token of every block (tokens RB k .. RB k + RB - 1,
 *   the last block possibly shorter), while the forward scan runs over the
 *   whole sequence as usual.  RB = 0 means one reverse scan over the whole
 *   sequence.
 *
 *   Backward: reverse-mode differentiation of the same recurrence for the
 *   loss  sum(dy * y), walking the visited order backwards with an adjoint
 *   state G = dLoss/dS.
 *
 * All arithmetic is IEEE fp64 in a fixed order (build without -ffast-math).
 * Work is split over independent (batch, head, direction) units on a pool of
 * POSIX threads; every unit writes disjoint output, so results do not depend
 * on the thread count.
 *
 * Layouts (row-major, contiguous):
 *   x, y, dy, dx : [Z][L][H][P]     dt, ddt : [Z][L][H]
 *   B, C, dB, dC : [Z][L][G][N]     A, D, dA, dD : [H]
 *   states       : [Z][H][P][N]
 * Head h reads group g = floor(h * G / H).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
  int64_t Z, L, H, P, N, G;
  int64_t RB; /* reverse block length (0: the reverse scan spans the sequence) */
} ssdo_shape;

typedef struct {
  const double *dt, *A, *B, *C;
} ssdo_dir;

/* ---------------------------------------------------------------- threads */

typedef void (*unit_fn)(void *ctx, int64_t unit, double *scratch);

typedef struct {
  unit_fn fn;
  void *ctx;
  int64_t nunits;
  int64_t next;
  size_t scratch_doubles;
  pthread_mutex_t mu;
  int failed;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *pl = (pool_t *)arg;
  double *scratch = NULL;
  if (pl->scratch_doubles) {
    scratch = (double *)malloc(pl->scratch_doubles * sizeof(double));
    if (!scratch) {
      pthread_mutex_lock(&pl->mu);
      pl->failed = 1;
      pthread_mutex_unlock(&pl->mu);
      return NULL;
    }
  }
  for (;;) {
    pthread_mutex_lock(&pl->mu);
    int64_t u = pl->next++;
    pthread_mutex_unlock(&pl->mu);
    if (u >= pl->nunits) break;
    pl->fn(pl->ctx, u, scratch);
  }
  free(scratch);
  return NULL;
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

static int run_pool(unit_fn fn, void *ctx, int64_t nunits, size_t scratch_doubles,
                    int nthreads) {
  pool_t pl;
  pl.fn = fn;
  pl.ctx = ctx;
  pl.nunits = nunits;
  pl.next = 0;
  pl.scratch_doubles = scratch_doubles;
  pl.failed = 0;
  pthread_mutex_init(&pl.mu, NULL);
  int nt = resolve_threads(nthreads);
  if (nt > nunits) nt = (int)(nunits > 0 ? nunits : 1);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nt);
  if (!th) return -1;
  int started = 0;
  for (int i = 0; i < nt; ++i) {
    if (pthread_create(&th[i], NULL, pool_worker, &pl) == 0) started++;
    else break;
  }
  if (started == 0) pool_worker(&pl);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&pl.mu);
  return pl.failed ? -1 : 0;
}

int ssdo_thread_count(int nthreads) { return resolve_threads(nthreads); }

/* ------------------------------------------------------------- one scan */

static inline int64_t group_of(const ssdo_shape *s, int64_t h) {
  return h * s->G / s->H;
}

/* 1 if direction d's state restarts from zero just before it visits token t:
 * the reverse scan with RB > 0 at the last token of each block. */
static inline int restarts_at(const ssdo_shape *s, int d, int64_t t) {
  return d == 1 && s->RB > 0 && (t + 1) % s->RB == 0;
}

/*
 * One direction of one head of one batch row: the Mamba-2 recurrence
 *   S <- exp(dt_t A) S + dt_t x_t (outer) B_t,   y_t = S C_t
 * over the visited order (forward: t ascending; reverse: t descending).
 * S starts from S0 (P*N, NULL = zero) and, for a block-segmented reverse
 * scan, is set back to zero before each block's last token is visited; the
 * state after the last visited token is left in S.  Writes this direction's
 * y_t at its natural position.
 */
static void scan_one(const ssdo_shape *s, int64_t b, int64_t h, int reverse,
                     const double *x, ssdo_dir p, const double *S0, double *yd,
                     double *S) {
  const int64_t L = s->L, H = s->H, P = s->P, N = s->N, G = s->G;
  const int64_t g = group_of(s, h);
  const double A = p.A[h];
  if (S0) memcpy(S, S0, sizeof(double) * (size_t)(P * N));
  else memset(S, 0, sizeof(double) * (size_t)(P * N));
  for (int64_t k = 0; k < L; ++k) {
    const int64_t t = reverse ? L - 1 - k : k;
    if (restarts_at(s, reverse, t)) memset(S, 0, sizeof(double) * (size_t)(P * N));
    const double dtv = p.dt[(b * L + t) * H + h];
    const double a = exp(dtv * A);
    const double *xt = x + ((b * L + t) * H + h) * P;
    const double *Bt = p.B + ((b * L + t) * G + g) * N;
    const double *Ct = p.C + ((b * L + t) * G + g) * N;
    double *yt = yd + ((b * L + t) * H + h) * P;
    for (int64_t i = 0; i < P; ++i) {
      double *Si = S + i * N;
      const double u = dtv * xt[i];
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        Si[n] = a * Si[n] + u * Bt[n];
        acc += Si[n] * Ct[n];
      }
      yt[i] = acc;
    }
  }
}

/* ---------------------------------------------------------- forward scan */

typedef struct {
  const ssdo_shape *s;
  const double *x;
  ssdo_dir dir[2];
  const double *init_state; /* fwd start state [Z][H][P][N] or NULL */
  double *yd[2];            /* per-direction outputs [Z][L][H][P] */
  double *final_state;      /* fwd end state or NULL */
} fwd_ctx;

static void fwd_unit(void *vctx, int64_t u, double *S) {
  fwd_ctx *c = (fwd_ctx *)vctx;
  const ssdo_shape *s = c->s;
  const int64_t PN = s->P * s->N;
  const int d = (int)(u % 2);
  const int64_t bh = u / 2;
  const int64_t b = bh / s->H, h = bh % s->H;
  const double *S0 = (d == 0 && c->init_state) ? c->init_state + bh * PN : NULL;
  scan_one(s, b, h, d, c->x, c->dir[d], S0, c->yd[d], S);
  if (d == 0 && c->final_state)
    memcpy(c->final_state + bh * PN, S, sizeof(double) * (size_t)PN);
}

static int shape_ok(const ssdo_shape *s) {
  return s && s->Z > 0 && s->L > 0 && s->H > 0 && s->P > 0 && s->N > 0 &&
         s->G > 0 && s->H % s->G == 0 && s->RB >= 0;
}

/*
 * Bidirectional layer forward:
 *   y = y_fwd + y_rev + D_h x.
 * y_f / y_r (optional, may be NULL) receive the two scan outputs separately.
 * init_state (optional) seeds the forward direction; final_state (optional)
 * receives the forward state after token L-1.  The reverse direction always
 * starts from zero after token L-1 and, with s->RB > 0, again after the last
 * token of every block of RB tokens.
 * Returns 0, or -1 on a bad shape / allocation failure.
 */
int ssdo_forward(const ssdo_shape *s, const double *x, ssdo_dir fwd, ssdo_dir rev,
                 const double *D, const double *init_state, double *y, double *y_f,
                 double *y_r, double *final_state, int nthreads) {
  if (!shape_ok(s)) return -1;
  const int64_t nel = s->Z * s->L * s->H * s->P;
  double *bufs = NULL;
  double *yf = y_f, *yr = y_r;
  if (!yf || !yr) {
    bufs = (double *)malloc(sizeof(double) * (size_t)nel * 2);
    if (!bufs) return -1;
    if (!yf) yf = bufs;
    if (!yr) yr = bufs + nel;
  }
  double *fs = NULL;
  if (final_state) {
    fs = (double *)malloc(sizeof(double) * (size_t)(s->Z * s->H * s->P * s->N));
    if (!fs) { free(bufs); return -1; }
  }
  fwd_ctx c;
  c.s = s;
  c.x = x;
  c.dir[0] = fwd;
  c.dir[1] = rev;
  c.init_state = init_state;
  c.yd[0] = yf;
  c.yd[1] = yr;
  c.final_state = fs;
  int rc = run_pool(fwd_unit, &c, 2 * s->Z * s->H, (size_t)(s->P * s->N), nthreads);
  if (rc == 0) {
    for (int64_t i = 0; i < nel; ++i) {
      const int64_t h = (i / s->P) % s->H;
      y[i] = yf[i] + yr[i] + D[h] * x[i];
    }
    /* copy last so final_state may alias init_state */
    if (final_state)
      memcpy(final_state, fs, sizeof(double) * (size_t)(s->Z * s->H * s->P * s->N));
  }
  free(fs);
  free(bufs);
  return rc;
}

/*
 * Block update with partial bidirectionality: the active block of s->L
 * tokens continues the forward scan from the cached prefix state state_in
 * (the forward state after the last prefix token), while the reverse scan
 * sees only the block and starts from zero after its last token.
 *   y_blk = y_fwd(from state_in) + y_rev(block only) + D x_blk
 * state_out (optional, may equal state_in) receives the forward state after
 * the last block token, i.e. the cache for the next block.
 */
int ssdo_block_update(const ssdo_shape *s, const double *state_in, const double *x_blk,
                      ssdo_dir fwd, ssdo_dir rev, const double *D, double *y_blk,
                      double *state_out, int nthreads) {
  if (!state_in || s->RB != 0) return -1;
  return ssdo_forward(s, x_blk, fwd, rev, D, state_in, y_blk, NULL, NULL, state_out,
                      nthreads);
}

/* --------------------------------------------------------------- backward */

typedef struct {
  const ssdo_shape *s;
  const double *x, *dy;
  ssdo_dir dir[2];
  const double *init_state;
  double *dx;          /* [Z][L][H][P] scan part (both directions) */
  double *ddt[2];      /* [Z][L][H] */
  double *dB[2], *dC[2]; /* [Z][L][G][N] */
  double *dA_part;     /* [Z][2][H] */
  int64_t seg;         /* checkpoint spacing */
} bwd_ctx;

/*
 * Reverse-mode pass for one direction of one head:
 *   forward:  S_k = a_k S_{k-1} + dt_k x_k (outer) B_k,   y_k = S_k C_k
 *   adjoint:  G   = dLoss/dS_k, built from the end:  G += dy_k (outer) C_k,
 *             dC_k += S_k^T dy_k,  dx_k += dt_k G B_k,  dB_k += dt_k G^T x_k,
 *             ddt_k = x_k^T G B_k + A a_k <G, S_{k-1}>,
 *             dA += dt_k a_k <G, S_{k-1}>,   then G <- a_k G.
 * At a restart of a block-segmented reverse scan the factor on S_{k-1} is 0
 * instead of a_k, in the recomputed states, in the two <G, S_{k-1}> terms and
 * in the final G <- 0.
 * States are checkpointed every `seg` visited tokens and each segment is
 * recomputed once, so memory stays (L/seg + seg) * P * N doubles.
 */
static void bwd_one(bwd_ctx *c, int64_t b, int64_t h, int d, double *ws) {
  const ssdo_shape *s = c->s;
  const int64_t L = s->L, H = s->H, P = s->P, N = s->N, G = s->G;
  const int64_t PN = P * N, g = group_of(s, h), seg = c->seg;
  const ssdo_dir p = c->dir[d];
  const double A = p.A[h];
  const int64_t nseg = (L + seg - 1) / seg;
  double *ckpt = ws;                  /* nseg * PN : state before each segment */
  double *segS = ckpt + nseg * PN;    /* (seg + 1) * PN : states inside a segment */
  double *Gm = segS + (seg + 1) * PN; /* PN */
  double *gB = Gm + PN;               /* P */

  /* forward pass: checkpoints */
  double *S = segS; /* reuse as running state */
  if (d == 0 && c->init_state)
    memcpy(S, c->init_state + (b * H + h) * PN, sizeof(double) * (size_t)PN);
  else
    memset(S, 0, sizeof(double) * (size_t)PN);
  for (int64_t k = 0; k < L; ++k) {
    if (k % seg == 0) memcpy(ckpt + (k / seg) * PN, S, sizeof(double) * (size_t)PN);
    const int64_t t = d ? L - 1 - k : k;
    if (restarts_at(s, d, t)) memset(S, 0, sizeof(double) * (size_t)PN);
    const double dtv = p.dt[(b * L + t) * H + h];
    const double a = exp(dtv * A);
    const double *xt = c->x + ((b * L + t) * H + h) * P;
    const double *Bt = p.B + ((b * L + t) * G + g) * N;
    for (int64_t i = 0; i < P; ++i)
      for (int64_t n = 0; n < N; ++n) S[i * N + n] = a * S[i * N + n] + dtv * xt[i] * Bt[n];
  }

  memset(Gm, 0, sizeof(double) * (size_t)PN);
  double dA = 0.0;
  for (int64_t sg = nseg - 1; sg >= 0; --sg) {
    const int64_t k0 = sg * seg;
    const int64_t k1 = (k0 + seg < L) ? k0 + seg : L;
    /* recompute states: segS[j] = state before visited token k0 + j */
    memcpy(segS, ckpt + sg * PN, sizeof(double) * (size_t)PN);
    for (int64_t k = k0; k < k1; ++k) {
      const int64_t t = d ? L - 1 - k : k;
      const double dtv = p.dt[(b * L + t) * H + h];
      const double a = exp(dtv * A);
      const double *xt = c->x + ((b * L + t) * H + h) * P;
      const double *Bt = p.B + ((b * L + t) * G + g) * N;
      const double *Sp = segS + (k - k0) * PN;
      double *Sn = segS + (k - k0 + 1) * PN;
      /* factor on the previous state: zero at a restart */
      const double ap = restarts_at(s, d, t) ? 0.0 : a;
      for (int64_t i = 0; i < P; ++i)
        for (int64_t n = 0; n < N; ++n) Sn[i * N + n] = ap * Sp[i * N + n] + dtv * xt[i] * Bt[n];
    }
    for (int64_t k = k1 - 1; k >= k0; --k) {
      const int64_t t = d ? L - 1 - k : k;
      const double dtv = p.dt[(b * L + t) * H + h];
      const double a = exp(dtv * A);
      const double ap = restarts_at(s, d, t) ? 0.0 : a;
      const double *xt = c->x + ((b * L + t) * H + h) * P;
      const double *dyt = c->dy + ((b * L + t) * H + h) * P;
      const double *Bt = p.B + ((b * L + t) * G + g) * N;
      const double *Ct = p.C + ((b * L + t) * G + g) * N;
      const double *Sprev = segS + (k - k0) * PN;
      const double *Scur = segS + (k - k0 + 1) * PN;
      double *dCt = c->dC[d] + ((b * L + t) * G + g) * N;
      double *dBt = c->dB[d] + ((b * L + t) * G + g) * N;
      double *dxt = c->dx + ((b * L + t) * H + h) * P;
      /* G += dy_t (outer) C_t ; dC_t += S_t^T dy_t */
      for (int64_t i = 0; i < P; ++i)
        for (int64_t n = 0; n < N; ++n) Gm[i * N + n] += dyt[i] * Ct[n];
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t i = 0; i < P; ++i) acc += dyt[i] * Scur[i * N + n];
        dCt[n] += acc;
      }
      /* gB = G B_t ; dx_t += dt gB ; x^T G B */
      double xgb = 0.0;
      for (int64_t i = 0; i < P; ++i) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += Gm[i * N + n] * Bt[n];
        gB[i] = acc;
        dxt[i] += dtv * acc;
        xgb += xt[i] * acc;
      }
      /* dB_t += dt G^T x_t */
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t i = 0; i < P; ++i) acc += Gm[i * N + n] * xt[i];
        dBt[n] += dtv * acc;
      }
      /* <G, S_{t-1}> */
      double ip = 0.0;
      for (int64_t e = 0; e < PN; ++e) ip += Gm[e] * Sprev[e];
      c->ddt[d][(b * L + t) * H + h] = xgb + A * ap * ip;
      dA += dtv * ap * ip;
      for (int64_t e = 0; e < PN; ++e) Gm[e] *= ap;
    }
  }
  c->dA_part[(b * 2 + d) * H + h] = dA;
}

/* One unit = one (batch row, group): its heads' dx rows and its own dB/dC
 * rows are written by this unit only, so no two units touch the same output. */
static void bwd_unit(void *vctx, int64_t u, double *ws) {
  bwd_ctx *c = (bwd_ctx *)vctx;
  const ssdo_shape *s = c->s;
  const int64_t b = u / s->G, g = u % s->G;
  const int64_t hpg = s->H / s->G;
  for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h)
    for (int d = 0; d < 2; ++d) bwd_one(c, b, h, d, ws);
}

/*
 * Gradients of  Loss = sum(dy * y)  with y from ssdo_forward (init_state
 * optional, treated as a constant).  All outputs are overwritten:
 *   dx [Z][L][H][P], ddt_f and ddt_r [Z][L][H], dB and dC per direction [Z][L][G][N],
 *   dA_f/dA_r [H] (summed over batch and time), dD [H].
 */
int ssdo_backward(const ssdo_shape *s, const double *x, ssdo_dir fwd, ssdo_dir rev,
                  const double *D, const double *init_state, const double *dy,
                  double *dx, double *ddt_f, double *dA_f, double *dB_f, double *dC_f,
                  double *ddt_r, double *dA_r, double *dB_r, double *dC_r, double *dD,
                  int nthreads) {
  if (!shape_ok(s)) return -1;
  const int64_t Z = s->Z, L = s->L, H = s->H, P = s->P, N = s->N, G = s->G;
  const int64_t nx = Z * L * H * P, nbc = Z * L * G * N;
  memset(dx, 0, sizeof(double) * (size_t)nx);
  memset(dB_f, 0, sizeof(double) * (size_t)nbc);
  memset(dC_f, 0, sizeof(double) * (size_t)nbc);
  memset(dB_r, 0, sizeof(double) * (size_t)nbc);
  memset(dC_r, 0, sizeof(double) * (size_t)nbc);
  double *dA_part = (double *)calloc((size_t)(Z * 2 * H), sizeof(double));
  if (!dA_part) return -1;
  bwd_ctx c;
  c.s = s;
  c.x = x;
  c.dy = dy;
  c.dir[0] = fwd;
  c.dir[1] = rev;
  c.init_state = init_state;
  c.dx = dx;
  c.ddt[0] = ddt_f;
  c.ddt[1] = ddt_r;
  c.dB[0] = dB_f;
  c.dB[1] = dB_r;
  c.dC[0] = dC_f;
  c.dC[1] = dC_r;
  c.dA_part = dA_part;
  c.seg = 64;
  const int64_t nseg = (L + c.seg - 1) / c.seg;
  const size_t ws = (size_t)((nseg + c.seg + 2) * P * N + P);
  int rc = run_pool(bwd_unit, &c, Z * G, ws, nthreads);
  if (rc == 0) {
    for (int64_t h = 0; h < H; ++h) {
      double af = 0.0, ar = 0.0, dd = 0.0;
      for (int64_t b = 0; b < Z; ++b) {
        af += dA_part[(b * 2 + 0) * H + h];
        ar += dA_part[(b * 2 + 1) * H + h];
      }
      for (int64_t b = 0; b < Z; ++b)
        for (int64_t t = 0; t < L; ++t) {
          const double *xr = x + ((b * L + t) * H + h) * P;
          const double *dr = dy + ((b * L + t) * H + h) * P;
          for (int64_t i = 0; i < P; ++i) dd += dr[i] * xr[i];
        }
      dA_f[h] = af;
      dA_r[h] = ar;
      dD[h] = dd;
    }
    for (int64_t i = 0; i < nx; ++i) {
      const int64_t h = (i / P) % H;
      dx[i] += D[h] * dy[i];
    }
  }
  free(dA_part);
  return rc;
}
