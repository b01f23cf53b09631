/*
 * FP64 CPU oracle for the gated delta rule (Gated DeltaNet, "GDN") training kernel.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the checker, not the product: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it. It shares no
 * code, header, table or helper with the HIP library.
 *
 * What is computed. The pages (flashinfer PR #8172, "non-deterministic context-parallel
 * Cake GDN chunked autograd backend", PR description) name the method, a chunked
 * Gated DeltaNet training kernel with gradients on packed variable-length sequences,
 * and measure every output and gradient against an FP64 reference. They never write the
 * recurrence down. The plainest reading, and the one the chunked saved set in the README
 * table quoted in flashinfer PR #8542 (gamma, gcum, Akk; h tape, v_new, w, u, Aqk) fits,
 * is the gated delta rule with the decay applied before the delta correction:
 *
 *   for each document n, v head h (q/k head j = h / (HV/H)), token t of the document:
 *     qh_t, kh_t = l2norm(q_t), l2norm(k_t)     (identity when the norm is off)
 *     a_t = exp(g_t)                            (g is the log decay), b_t = beta_t
 *     p_t = S_{t-1}^T kh_t                      (S is dk x dv, row = key dim)
 *     e_t = v_t - a_t p_t
 *     S_t = a_t S_{t-1} + b_t kh_t e_t^T
 *     o_t = S_t^T qh_t
 *   S_0 = h0[n,h] (or 0), ht[n,h] = S_L.
 *
 * The q/k L2 norm that the kernel may apply itself (an option listed in the flashinfer
 * PR #8542 description) is l2norm(x) = x / sqrt(x.x + eps). The state is FP32 on the GPU, 64 KiB per v head at
 * d = 128 (PR #8542 description), here FP64.
 *
 * Three entry points:
 *   gdn_oracle_fwd          token-by-token forward (the definition above)
 *   gdn_oracle_bwd          token-by-token reverse mode, derived by hand from the same
 *                           recurrence (states are re-derived from FP64 checkpoints taken
 *                           every ORACLE_BLOCK tokens)
 *   gdn_oracle_chunked_fwd  the same forward in chunked form (chunk = C tokens per
 *                           document): intra-chunk unit-lower-triangular solve, WY factors
 *                           W and U, and the inter-chunk state walk. It also returns the
 *                           chunk intermediates the pages' saved set names (Akk = the
 *                           inverse, gcum = in-chunk cumulative log decay, gamma = the
 *                           chunk's total decay; gdn_oracle_chunked_fwd_full also the full
 *                           set's W, U, v_new, P rows and chunk start states).
 *
 * Inputs are float32 arrays holding the exact values the GPU receives (bf16 values widen
 * to float32 exactly); every operation is in double. Work is split over threads by
 * (document, q/k head) items, longest document first; the G v heads of one q/k head are
 * handled by one thread in fixed order, so dq and dk sums are deterministic.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_BLOCK 64 /* tokens between FP64 state checkpoints in the reverse pass */

typedef struct {
  /* problem */
  int64_t T;
  int N;
  const int32_t* cu;
  int H, HV, dk, dv;
  const float *q, *k, *v, *g, *beta, *h0, *dO, *dht;
  int l2norm;
  double eps;
  /* outputs (any may be NULL unless the entry point needs it) */
  double *o, *ht;
  double *dq, *dkk, *dvv, *dg, *dbeta, *dh0;
  /* chunked-form extras */
  int chunk;
  double *A, *gcum, *gamma;
  double *Wo, *Uo, *Ro, *Po, *Hs; /* full saved set: W, U, R = v_new, P rows, chunk start states */
  int64_t* seq_chunk0; /* first global chunk index of each document */
  /* work queue */
  int n_items;
  int* items; /* item = n * H + j, sorted by document length, longest first */
  int next;
  int status;
} job_t;

/* ------------------------------------------------------------------------------------ */
/* small helpers                                                                         */

/* Row x (length d, float) -> out (double), divided by its L2 norm when l2norm is on. */
static void load_row(const float* x, int d, int l2norm, double eps, double* out, double* inv_norm) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) {
    out[i] = (double)x[i];
    ss += out[i] * out[i];
  }
  double r = 1.0;
  if (l2norm) {
    r = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < d; ++i) out[i] *= r;
  }
  if (inv_norm) *inv_norm = r;
}

static int next_item(job_t* J) { return __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED); }

static int64_t seq_len(const job_t* J, int n) { return (int64_t)J->cu[n + 1] - (int64_t)J->cu[n]; }

/* One forward token step on an FP64 state S (dk x dv, row-major), in place.
 * p and e are scratch of length dv; on return they hold p_t and e_t. */
static void token_step(double* S, int dk, int dv, const double* kh, const double* vv, double a, double b,
                       double* p, double* e) {
  for (int c = 0; c < dv; ++c) p[c] = 0.0;
  for (int r = 0; r < dk; ++r) {
    const double kr = kh[r];
    const double* Sr = S + (size_t)r * dv;
    for (int c = 0; c < dv; ++c) p[c] += Sr[c] * kr;
  }
  for (int c = 0; c < dv; ++c) e[c] = vv[c] - a * p[c];
  for (int r = 0; r < dk; ++r) {
    const double bk = b * kh[r];
    double* Sr = S + (size_t)r * dv;
    for (int c = 0; c < dv; ++c) Sr[c] = a * Sr[c] + bk * e[c];
  }
}

static void init_state(const job_t* J, int n, int h, double* S) {
  const size_t dd = (size_t)J->dk * J->dv;
  if (J->h0) {
    const float* src = J->h0 + ((size_t)n * J->HV + h) * dd;
    for (size_t i = 0; i < dd; ++i) S[i] = (double)src[i];
  } else {
    memset(S, 0, dd * sizeof(double));
  }
}

/* ------------------------------------------------------------------------------------ */
/* recurrent forward                                                                     */

static void fwd_item(job_t* J, int n, int j) {
  const int G = J->HV / J->H, dk = J->dk, dv = J->dv;
  const int64_t L = seq_len(J, n), t0 = J->cu[n];
  const size_t dd = (size_t)dk * dv;
  double* S = (double*)malloc(dd * sizeof(double));
  double* buf = (double*)malloc((size_t)(2 * dk + 3 * dv) * sizeof(double));
  if (!S || !buf) {
    J->status = -2;
    free(S);
    free(buf);
    return;
  }
  double *qh = buf, *kh = buf + dk, *vv = buf + 2 * dk, *p = vv + dv, *e = p + dv;
  for (int gi = 0; gi < G; ++gi) {
    const int h = j * G + gi;
    init_state(J, n, h, S);
    for (int64_t t = 0; t < L; ++t) {
      const int64_t tau = t0 + t;
      load_row(J->q + ((size_t)tau * J->H + j) * dk, dk, J->l2norm, J->eps, qh, NULL);
      load_row(J->k + ((size_t)tau * J->H + j) * dk, dk, J->l2norm, J->eps, kh, NULL);
      const float* vsrc = J->v + ((size_t)tau * J->HV + h) * dv;
      for (int c = 0; c < dv; ++c) vv[c] = (double)vsrc[c];
      const double a = exp((double)J->g[(size_t)tau * J->HV + h]);
      const double b = (double)J->beta[(size_t)tau * J->HV + h];
      token_step(S, dk, dv, kh, vv, a, b, p, e);
      if (J->o) {
        double* out = J->o + ((size_t)tau * J->HV + h) * dv;
        for (int c = 0; c < dv; ++c) out[c] = 0.0;
        for (int r = 0; r < dk; ++r) {
          const double qr = qh[r];
          const double* Sr = S + (size_t)r * dv;
          for (int c = 0; c < dv; ++c) out[c] += Sr[c] * qr;
        }
      }
    }
    if (J->ht) memcpy(J->ht + ((size_t)n * J->HV + h) * dd, S, dd * sizeof(double));
  }
  free(S);
  free(buf);
}

/* ------------------------------------------------------------------------------------ */
/* recurrent reverse mode                                                                */
/*
 * Reverse of one token step (given dS = dLoss/dS_t, including later tokens):
 *   o_t = S_t^T qh          : dS += qh do^T ;      dqh = S_t do
 *   S_t = a S_{t-1} + b kh e^T
 *                           : de = b dS^T kh ;     dbeta = kh^T dS e ;   dkh += b dS e
 *                             dalpha = <dS, S_{t-1}>_F ;  dS_{t-1} = a dS (+ below)
 *   e = v - a p             : dv = de ;            dalpha -= p.de ;      dp = -a de
 *   p = S_{t-1}^T kh        : dkh += S_{t-1} dp ;  dS_{t-1} += kh dp^T
 *   a = exp(g)              : dg = a dalpha
 */
static void bwd_item(job_t* J, int n, int j) {
  const int G = J->HV / J->H, dk = J->dk, dv = J->dv;
  const int64_t L = seq_len(J, n), t0 = J->cu[n];
  const size_t dd = (size_t)dk * dv;
  const int64_t nblk = (L + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
  double* ckpt = (double*)malloc((size_t)(nblk + 1) * dd * sizeof(double));
  double* st = (double*)malloc((size_t)(ORACLE_BLOCK + 1) * dd * sizeof(double));
  double* dS = (double*)malloc(dd * sizeof(double));
  double* acc = (double*)calloc((size_t)(L > 0 ? L : 1) * 2 * dk, sizeof(double)); /* dqh, dkh sums */
  double* buf = (double*)malloc((size_t)(3 * dk + 7 * dv) * sizeof(double));
  if (!ckpt || !st || !dS || !acc || !buf) {
    J->status = -2;
    goto out;
  }
  double *qh = buf, *kh = buf + dk, *dSe = buf + 2 * dk;
  double *vv = buf + 3 * dk, *p = vv + dv, *e = p + dv, *dov = e + dv, *de = dov + dv, *dp = de + dv,
         *tmp = dp + dv;
  double* dqh_acc = acc;
  double* dkh_acc = acc + (size_t)L * dk;

  for (int gi = 0; gi < G; ++gi) {
    const int h = j * G + gi;
    /* forward pass: checkpoint the state before every block */
    init_state(J, n, h, st);
    for (int64_t t = 0; t < L; ++t) {
      if (t % ORACLE_BLOCK == 0) memcpy(ckpt + (size_t)(t / ORACLE_BLOCK) * dd, st, dd * sizeof(double));
      const int64_t tau = t0 + t;
      load_row(J->k + ((size_t)tau * J->H + j) * dk, dk, J->l2norm, J->eps, kh, NULL);
      const float* vsrc = J->v + ((size_t)tau * J->HV + h) * dv;
      for (int c = 0; c < dv; ++c) vv[c] = (double)vsrc[c];
      token_step(st, dk, dv, kh, vv, exp((double)J->g[(size_t)tau * J->HV + h]),
                 (double)J->beta[(size_t)tau * J->HV + h], p, e);
    }
    /* reverse pass */
    if (J->dht) {
      const float* src = J->dht + ((size_t)n * J->HV + h) * dd;
      for (size_t i = 0; i < dd; ++i) dS[i] = (double)src[i];
    } else {
      memset(dS, 0, dd * sizeof(double));
    }
    for (int64_t blk = nblk - 1; blk >= 0; --blk) {
      const int64_t tb = blk * ORACLE_BLOCK;
      const int64_t te = (tb + ORACLE_BLOCK < L) ? tb + ORACLE_BLOCK : L;
      memcpy(st, ckpt + (size_t)blk * dd, dd * sizeof(double));
      for (int64_t t = tb; t < te; ++t) { /* st[i] = state before token tb+i */
        const int64_t tau = t0 + t;
        double* nxt = st + (size_t)(t - tb + 1) * dd;
        memcpy(nxt, st + (size_t)(t - tb) * dd, dd * sizeof(double));
        load_row(J->k + ((size_t)tau * J->H + j) * dk, dk, J->l2norm, J->eps, kh, NULL);
        const float* vsrc = J->v + ((size_t)tau * J->HV + h) * dv;
        for (int c = 0; c < dv; ++c) vv[c] = (double)vsrc[c];
        token_step(nxt, dk, dv, kh, vv, exp((double)J->g[(size_t)tau * J->HV + h]),
                   (double)J->beta[(size_t)tau * J->HV + h], p, e);
      }
      for (int64_t t = te - 1; t >= tb; --t) {
        const int64_t tau = t0 + t;
        const double* Sp = st + (size_t)(t - tb) * dd;     /* S_{t-1} */
        const double* Sc = st + (size_t)(t - tb + 1) * dd; /* S_t */
        load_row(J->q + ((size_t)tau * J->H + j) * dk, dk, J->l2norm, J->eps, qh, NULL);
        load_row(J->k + ((size_t)tau * J->H + j) * dk, dk, J->l2norm, J->eps, kh, NULL);
        const float* vsrc = J->v + ((size_t)tau * J->HV + h) * dv;
        const float* dsrc = J->dO + ((size_t)tau * J->HV + h) * dv;
        for (int c = 0; c < dv; ++c) {
          vv[c] = (double)vsrc[c];
          dov[c] = (double)dsrc[c];
        }
        const double a = exp((double)J->g[(size_t)tau * J->HV + h]);
        const double b = (double)J->beta[(size_t)tau * J->HV + h];
        /* output: dS += qh do^T ; dqh = S_t do */
        double* dq_t = dqh_acc + (size_t)t * dk;
        for (int r = 0; r < dk; ++r) {
          double* dSr = dS + (size_t)r * dv;
          const double* Scr = Sc + (size_t)r * dv;
          double s = 0.0;
          for (int c = 0; c < dv; ++c) {
            dSr[c] += qh[r] * dov[c];
            s += Scr[c] * dov[c];
          }
          dq_t[r] += s;
        }
        /* p, e from S_{t-1} */
        for (int c = 0; c < dv; ++c) p[c] = 0.0;
        for (int r = 0; r < dk; ++r) {
          const double* Spr = Sp + (size_t)r * dv;
          for (int c = 0; c < dv; ++c) p[c] += Spr[c] * kh[r];
        }
        for (int c = 0; c < dv; ++c) e[c] = vv[c] - a * p[c];
        /* de = b dS^T kh ; dSe = dS e ; dalpha = <dS, S_{t-1}> */
        for (int c = 0; c < dv; ++c) tmp[c] = 0.0;
        double dalpha = 0.0, dbeta = 0.0;
        for (int r = 0; r < dk; ++r) {
          const double* dSr = dS + (size_t)r * dv;
          const double* Spr = Sp + (size_t)r * dv;
          double s = 0.0;
          for (int c = 0; c < dv; ++c) {
            tmp[c] += dSr[c] * kh[r];
            s += dSr[c] * e[c];
            dalpha += dSr[c] * Spr[c];
          }
          dSe[r] = s;
          dbeta += kh[r] * s;
        }
        for (int c = 0; c < dv; ++c) {
          de[c] = b * tmp[c];
          dalpha -= p[c] * de[c];
          dp[c] = -a * de[c];
        }
        /* dkh = b dS e + S_{t-1} dp */
        double* dk_t = dkh_acc + (size_t)t * dk;
        for (int r = 0; r < dk; ++r) {
          const double* Spr = Sp + (size_t)r * dv;
          double s = 0.0;
          for (int c = 0; c < dv; ++c) s += Spr[c] * dp[c];
          dk_t[r] += b * dSe[r] + s;
        }
        /* dS_{t-1} = a dS + kh dp^T */
        for (int r = 0; r < dk; ++r) {
          double* dSr = dS + (size_t)r * dv;
          for (int c = 0; c < dv; ++c) dSr[c] = a * dSr[c] + kh[r] * dp[c];
        }
        if (J->dvv) {
          double* out = J->dvv + ((size_t)tau * J->HV + h) * dv;
          for (int c = 0; c < dv; ++c) out[c] = de[c];
        }
        if (J->dg) J->dg[(size_t)tau * J->HV + h] = a * dalpha;
        if (J->dbeta) J->dbeta[(size_t)tau * J->HV + h] = dbeta;
      }
    }
    if (J->dh0) memcpy(J->dh0 + ((size_t)n * J->HV + h) * dd, dS, dd * sizeof(double));
  }
  /* L2-norm backward on the group sums: dx = (dxh - xh (xh . dxh)) / sqrt(x.x + eps) */
  for (int64_t t = 0; t < L; ++t) {
    const int64_t tau = t0 + t;
    for (int which = 0; which < 2; ++which) {
      const float* x = (which == 0 ? J->q : J->k) + ((size_t)tau * J->H + j) * dk;
      const double* dxh = (which == 0 ? dqh_acc : dkh_acc) + (size_t)t * dk;
      double* out = (which == 0 ? J->dq : J->dkk);
      if (!out) continue;
      out += ((size_t)tau * J->H + j) * dk;
      if (!J->l2norm) {
        for (int r = 0; r < dk; ++r) out[r] = dxh[r];
        continue;
      }
      double r_inv;
      load_row(x, dk, 1, J->eps, qh, &r_inv); /* qh <- xh */
      double dot = 0.0;
      for (int r = 0; r < dk; ++r) dot += qh[r] * dxh[r];
      for (int r = 0; r < dk; ++r) out[r] = (dxh[r] - qh[r] * dot) * r_inv;
    }
  }
out:
  free(ckpt);
  free(st);
  free(dS);
  free(acc);
  free(buf);
}

/* ------------------------------------------------------------------------------------ */
/* chunked forward                                                                       */
/*
 * For a chunk of Ce <= C tokens with start state S, per v head:
 *   G_i = sum_{s<=i} g_s ; b_i = exp(G_i) ; gamma = b_{Ce-1}
 *   L_ij = beta_i exp(G_i - G_j) kh_i.kh_j  (i > j) ;  A = (I + L)^{-1}
 *   W = A diag(beta b) Kh ;  U = A diag(beta) V ;  R = U - W S
 *   P_ij = exp(G_i - G_j) qh_i.kh_j  (i >= j)
 *   O = diag(b) Qh S + P R ;  S <- gamma S + Kh^T diag(exp(G_{Ce-1} - G)) R
 * Derivation: write r_t = beta_t (v_t - a_t S_{t-1}^T kh_t) (so S_t = a_t S_{t-1} + kh_t r_t^T)
 * and unroll S_{t-1} back to the chunk start: (I + L) R = diag(beta) V - diag(beta b) Kh S.
 */
static void chunked_item(job_t* J, int n, int j) {
  const int G = J->HV / J->H, dk = J->dk, dv = J->dv, C = J->chunk;
  const int64_t L = seq_len(J, n), t0 = J->cu[n];
  const size_t dd = (size_t)dk * dv;
  const size_t need = dd + (size_t)C * (2 * dk + 4 * dv + 4 * C + 4) + (size_t)C * dk;
  double* mem = (double*)malloc(need * sizeof(double));
  if (!mem) {
    J->status = -2;
    return;
  }
  double* S = mem;
  double* Qh = S + dd;            /* C x dk */
  double* Kh = Qh + (size_t)C * dk; /* C x dk */
  double* V = Kh + (size_t)C * dk;  /* C x dv */
  double* U = V + (size_t)C * dv;   /* C x dv */
  double* R = U + (size_t)C * dv;   /* C x dv */
  double* O = R + (size_t)C * dv;   /* C x dv */
  double* Lm = O + (size_t)C * dv;  /* C x C */
  double* Am = Lm + (size_t)C * C;  /* C x C */
  double* Pm = Am + (size_t)C * C;  /* C x C */
  double* Kk = Pm + (size_t)C * C;  /* C x C */
  double* Gc = Kk + (size_t)C * C;  /* C */
  double* bb = Gc + C;              /* C */
  double* bet = bb + C;             /* C */
  double* col = bet + C;            /* C */
  double* W = col + C;              /* C x dk */

  for (int gi = 0; gi < G; ++gi) {
    const int h = j * G + gi;
    init_state(J, n, h, S);
    int64_t cidx = J->seq_chunk0[n];
    for (int64_t cs = 0; cs < L; cs += C, ++cidx) {
      const int Ce = (int)((L - cs) < C ? (L - cs) : C);
      if (J->Hs) memcpy(J->Hs + ((size_t)cidx * J->HV + h) * dd, S, dd * sizeof(double));
      double run = 0.0;
      for (int i = 0; i < Ce; ++i) {
        const int64_t tau = t0 + cs + i;
        load_row(J->q + ((size_t)tau * J->H + j) * dk, dk, J->l2norm, J->eps, Qh + (size_t)i * dk, NULL);
        load_row(J->k + ((size_t)tau * J->H + j) * dk, dk, J->l2norm, J->eps, Kh + (size_t)i * dk, NULL);
        const float* vsrc = J->v + ((size_t)tau * J->HV + h) * dv;
        for (int c = 0; c < dv; ++c) V[(size_t)i * dv + c] = (double)vsrc[c];
        run += (double)J->g[(size_t)tau * J->HV + h];
        Gc[i] = run;
        bb[i] = exp(run);
        bet[i] = (double)J->beta[(size_t)tau * J->HV + h];
      }
      const double Glast = Gc[Ce - 1];
      /* key-key and query-key products */
      for (int i = 0; i < Ce; ++i)
        for (int jj = 0; jj < Ce; ++jj) {
          double sk = 0.0, sq = 0.0;
          for (int r = 0; r < dk; ++r) {
            sk += Kh[(size_t)i * dk + r] * Kh[(size_t)jj * dk + r];
            sq += Qh[(size_t)i * dk + r] * Kh[(size_t)jj * dk + r];
          }
          Kk[(size_t)i * C + jj] = sk;
          Lm[(size_t)i * C + jj] = (i > jj) ? bet[i] * exp(Gc[i] - Gc[jj]) * sk : 0.0;
          Pm[(size_t)i * C + jj] = (i >= jj) ? exp(Gc[i] - Gc[jj]) * sq : 0.0;
        }
      /* A = (I + L)^{-1}: forward substitution, one unit column at a time */
      for (int c = 0; c < Ce; ++c) {
        for (int i = 0; i < Ce; ++i) {
          if (i < c) {
            col[i] = 0.0;
            continue;
          }
          double x = (i == c) ? 1.0 : 0.0;
          for (int m = c; m < i; ++m) x -= Lm[(size_t)i * C + m] * col[m];
          col[i] = x;
        }
        for (int i = 0; i < Ce; ++i) Am[(size_t)i * C + c] = col[i];
      }
      /* W = A diag(beta b) Kh ; U = A diag(beta) V */
      for (int i = 0; i < Ce; ++i) {
        for (int r = 0; r < dk; ++r) {
          double s = 0.0;
          for (int m = 0; m <= i; ++m) s += Am[(size_t)i * C + m] * bet[m] * bb[m] * Kh[(size_t)m * dk + r];
          W[(size_t)i * dk + r] = s;
        }
        for (int c = 0; c < dv; ++c) {
          double s = 0.0;
          for (int m = 0; m <= i; ++m) s += Am[(size_t)i * C + m] * bet[m] * V[(size_t)m * dv + c];
          U[(size_t)i * dv + c] = s;
        }
      }
      /* R = U - W S */
      for (int i = 0; i < Ce; ++i)
        for (int c = 0; c < dv; ++c) {
          double s = 0.0;
          for (int r = 0; r < dk; ++r) s += W[(size_t)i * dk + r] * S[(size_t)r * dv + c];
          R[(size_t)i * dv + c] = U[(size_t)i * dv + c] - s;
        }
      /* O = diag(b) Qh S + P R */
      for (int i = 0; i < Ce; ++i)
        for (int c = 0; c < dv; ++c) {
          double s = 0.0, s2 = 0.0;
          for (int r = 0; r < dk; ++r) s += Qh[(size_t)i * dk + r] * S[(size_t)r * dv + c];
          for (int m = 0; m <= i; ++m) s2 += Pm[(size_t)i * C + m] * R[(size_t)m * dv + c];
          O[(size_t)i * dv + c] = bb[i] * s + s2;
        }
      /* S <- gamma S + Kh^T diag(exp(Glast - G)) R */
      const double gam = bb[Ce - 1];
      for (int r = 0; r < dk; ++r)
        for (int c = 0; c < dv; ++c) {
          double s = 0.0;
          for (int i = 0; i < Ce; ++i) s += Kh[(size_t)i * dk + r] * exp(Glast - Gc[i]) * R[(size_t)i * dv + c];
          S[(size_t)r * dv + c] = gam * S[(size_t)r * dv + c] + s;
        }
      /* outputs */
      for (int i = 0; i < Ce; ++i) {
        const int64_t tau = t0 + cs + i;
        if (J->o)
          for (int c = 0; c < dv; ++c) J->o[((size_t)tau * J->HV + h) * dv + c] = O[(size_t)i * dv + c];
        if (J->A)
          for (int c = 0; c < C; ++c)
            J->A[((size_t)tau * J->HV + h) * C + c] = (c < Ce) ? Am[(size_t)i * C + c] : 0.0;
        if (J->gcum) J->gcum[(size_t)tau * J->HV + h] = Gc[i];
        const size_t rk_ = ((size_t)tau * J->HV + h) * dk, rv_ = ((size_t)tau * J->HV + h) * dv;
        if (J->Wo) memcpy(J->Wo + rk_, W + (size_t)i * dk, dk * sizeof(double));
        if (J->Uo) memcpy(J->Uo + rv_, U + (size_t)i * dv, dv * sizeof(double));
        if (J->Ro) memcpy(J->Ro + rv_, R + (size_t)i * dv, dv * sizeof(double));
        if (J->Po)
          for (int c = 0; c < C; ++c)
            J->Po[((size_t)tau * J->HV + h) * C + c] = (c < Ce) ? Pm[(size_t)i * C + c] : 0.0;
      }
      if (J->gamma) J->gamma[(size_t)cidx * J->HV + h] = gam;
    }
    if (J->ht) memcpy(J->ht + ((size_t)n * J->HV + h) * dd, S, dd * sizeof(double));
  }
  free(mem);
}

/* ------------------------------------------------------------------------------------ */
/* driver                                                                                */

typedef enum { OP_FWD, OP_BWD, OP_CHUNKED } op_t;
typedef struct {
  job_t* J;
  op_t op;
} worker_arg_t;

static void* worker(void* arg) {
  worker_arg_t* W = (worker_arg_t*)arg;
  job_t* J = W->J;
  for (;;) {
    const int it = next_item(J);
    if (it >= J->n_items) break;
    const int item = J->items[it];
    const int n = item / J->H, j = item % J->H;
    if (W->op == OP_FWD) fwd_item(J, n, j);
    else if (W->op == OP_BWD) bwd_item(J, n, j);
    else chunked_item(J, n, j);
  }
  return NULL;
}

static pthread_mutex_t g_sort_mu = PTHREAD_MUTEX_INITIALIZER;
static const job_t* g_sort_job;
static int cmp_items(const void* a, const void* b) {
  const int ia = *(const int*)a, ib = *(const int*)b;
  const int64_t la = seq_len(g_sort_job, ia / g_sort_job->H), lb = seq_len(g_sort_job, ib / g_sort_job->H);
  if (la != lb) return la > lb ? -1 : 1;
  return ia < ib ? -1 : (ia > ib);
}

static int validate(const job_t* J) {
  if (J->N < 0 || J->H <= 0 || J->HV <= 0 || J->HV % J->H != 0 || J->dk <= 0 || J->dv <= 0) return -1;
  if (!J->cu || J->cu[0] != 0 || (int64_t)J->cu[J->N] != J->T) return -1;
  for (int n = 0; n < J->N; ++n)
    if (J->cu[n + 1] < J->cu[n]) return -1;
  return 0;
}

static int run(job_t* J, op_t op, int nthreads) {
  if (validate(J)) return -1;
  J->n_items = J->N * J->H;
  J->items = (int*)malloc(sizeof(int) * (size_t)(J->n_items > 0 ? J->n_items : 1));
  if (!J->items) return -2;
  for (int i = 0; i < J->n_items; ++i) J->items[i] = i;
  pthread_mutex_lock(&g_sort_mu);
  g_sort_job = J;
  qsort(J->items, (size_t)J->n_items, sizeof(int), cmp_items);
  pthread_mutex_unlock(&g_sort_mu);
  J->next = 0;
  J->status = 0;
  if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
  if (nthreads > J->n_items) nthreads = J->n_items > 0 ? J->n_items : 1;
  worker_arg_t wa = {J, op};
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) {
    free(J->items);
    return -2;
  }
  int started = 0;
  for (int i = 1; i < nthreads; ++i)
    if (pthread_create(&th[started], NULL, worker, &wa) == 0) ++started;
  worker(&wa);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  free(J->items);
  J->items = NULL;
  return J->status;
}

/* Forward, token by token. o: [T,HV,dv]; ht: [N,HV,dk,dv] (nullable). h0 nullable. */
int gdn_oracle_fwd(int64_t T, int N, const int32_t* cu, int H, int HV, int dk, int dv, const float* q,
                   const float* k, const float* v, const float* g, const float* beta, const float* h0, int l2norm,
                   double eps, double* o, double* ht, int nthreads) {
  job_t J;
  memset(&J, 0, sizeof J);
  J.T = T; J.N = N; J.cu = cu; J.H = H; J.HV = HV; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.l2norm = l2norm; J.eps = eps;
  J.o = o; J.ht = ht;
  return run(&J, OP_FWD, nthreads);
}

/* Reverse mode. dO: [T,HV,dv]; dht nullable (= 0). Outputs dq, dk: [T,H,dk]; dv: [T,HV,dv];
 * dg, dbeta: [T,HV]; dh0: [N,HV,dk,dv] (nullable). */
int gdn_oracle_bwd(int64_t T, int N, const int32_t* cu, int H, int HV, int dk, int dv, const float* q,
                   const float* k, const float* v, const float* g, const float* beta, const float* h0, int l2norm,
                   double eps, const float* dO, const float* dht, double* dq, double* dk_out, double* dv_out,
                   double* dg, double* dbeta, double* dh0, int nthreads) {
  job_t J;
  memset(&J, 0, sizeof J);
  J.T = T; J.N = N; J.cu = cu; J.H = H; J.HV = HV; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.l2norm = l2norm; J.eps = eps;
  J.dO = dO; J.dht = dht;
  J.dq = dq; J.dkk = dk_out; J.dvv = dv_out; J.dg = dg; J.dbeta = dbeta; J.dh0 = dh0;
  if (!dO) return -1;
  return run(&J, OP_BWD, nthreads);
}

/* Chunked forward with intermediates. A: [T,HV,chunk] (row i of the chunk's inverse at the
 * token of row i, zero past the chunk's valid length); gcum: [T,HV]; gamma: [NT,HV] with
 * chunks numbered document by document. Any output may be NULL. */
int gdn_oracle_chunked_fwd(int64_t T, int N, const int32_t* cu, int H, int HV, int dk, int dv, const float* q,
                           const float* k, const float* v, const float* g, const float* beta, const float* h0,
                           int l2norm, double eps, int chunk, double* o, double* ht, double* A, double* gcum,
                           double* gamma, int nthreads) {
  job_t J;
  memset(&J, 0, sizeof J);
  J.T = T; J.N = N; J.cu = cu; J.H = H; J.HV = HV; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.l2norm = l2norm; J.eps = eps;
  J.o = o; J.ht = ht; J.chunk = chunk; J.A = A; J.gcum = gcum; J.gamma = gamma;
  if (chunk <= 0 || N < 0 || !cu) return -1;
  J.seq_chunk0 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + 1));
  if (!J.seq_chunk0) return -2;
  J.seq_chunk0[0] = 0;
  for (int n = 0; n < N; ++n)
    J.seq_chunk0[n + 1] = J.seq_chunk0[n] + ((int64_t)cu[n + 1] - cu[n] + chunk - 1) / chunk;
  const int rc = run(&J, OP_CHUNKED, nthreads);
  free(J.seq_chunk0);
  return rc;
}

/* The same, also returning what the full saved set holds besides the light one: W and U
 * ([T,HV,dk], [T,HV,dv]), R = U - W S (v_new, [T,HV,dv]), the rows of P ([T,HV,chunk], zero past
 * the chunk's valid length) and the state at the start of every chunk ([NT,HV,dk,dv]). */
int gdn_oracle_chunked_fwd_full(int64_t T, int N, const int32_t* cu, int H, int HV, int dk, int dv,
                                const float* q, const float* k, const float* v, const float* g, const float* beta,
                                const float* h0, int l2norm, double eps, int chunk, double* o, double* ht,
                                double* A, double* gcum, double* gamma, double* W, double* U, double* R,
                                double* P, double* Hs, int nthreads) {
  job_t J;
  memset(&J, 0, sizeof J);
  J.T = T; J.N = N; J.cu = cu; J.H = H; J.HV = HV; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.h0 = h0; J.l2norm = l2norm; J.eps = eps;
  J.o = o; J.ht = ht; J.chunk = chunk; J.A = A; J.gcum = gcum; J.gamma = gamma;
  J.Wo = W; J.Uo = U; J.Ro = R; J.Po = P; J.Hs = Hs;
  if (chunk <= 0 || N < 0 || !cu) return -1;
  J.seq_chunk0 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + 1));
  if (!J.seq_chunk0) return -2;
  J.seq_chunk0[0] = 0;
  for (int n = 0; n < N; ++n)
    J.seq_chunk0[n + 1] = J.seq_chunk0[n] + ((int64_t)cu[n + 1] - cu[n] + chunk - 1) / chunk;
  const int rc = run(&J, OP_CHUNKED, nthreads);
  free(J.seq_chunk0);
  return rc;
}
