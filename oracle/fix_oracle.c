/*
 * fix_oracle.c -- plain fp64 CPU oracle for FiX parallel attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes (FiX README, section "Quick Start", and the FiX ICML
 * abstract on the icml.cc poster page):
 *   causal softmax attention in which the softmax denominator is dropped
 *   (made redundant by the RMSNorm that follows) and an element-wise,
 *   log-space forget gate g, shaped like v, decays every value vector:
 *
 *     s_ij = scale * <q_i, k_j>                      (j <= i, same sequence)
 *     m_i  = max_{j<=i} s_ij
 *     D_ij = prod_{u=j+1..i} exp(g_u)                (a dv-vector, D_ii = 1)
 *     x_i  = sum_{j<=i} exp(s_ij - m_i) * D_ij (.) v_j
 *     o_i  = x_i * (mean_d x_i^2 + eps)^-1/2 (.) w   if o_norm, else x_i
 *     o_i *= z_i                                      if an output gate is given
 *
 * The decay is evaluated as a running product of per-token gate factors,
 * never as an exponential of a difference of prefix sums.  A walk along the
 * keys (or queries) stops once that product is exactly zero in every channel:
 * every later term is then an exact zero, so no result changes.  The readings
 * taken where the pages are silent (inclusive gate product, m_i the row max
 * of the scaled undecayed logits, contiguous GQA head groups, m held
 * constant in the backward, literal product with the output gate after the
 * norm) are listed with the design notes of this repository.
 *
 * Backward (m held constant):
 *   dz_i = dO_i (.) n_i  with n_i = xhat_i (.) w (o_norm) or x_i
 *   dn_i = dO_i (.) z_i
 *   delta_i = r_i (dn_i(.)w - xhat_i * mean_d(dn_i(.)w(.)xhat_i))  (o_norm)
 *             dn_i                                                (else)
 *   dP_ij = sum_d D_ij,d v_j,d delta_i,d ;  dS_ij = P_ij dP_ij
 *   dq_i = scale sum_j dS_ij k_j ; dk_j = scale sum_{h in group} sum_i dS_ij q_i
 *   dv_j = sum_{h in group} sum_{i>=j} P_ij D_ij (.) delta_i
 *   dG_t = sum_{h in group} delta_t (.) x_t - v_t (.) dv_t
 *   dg_t = sum_{t'>=t, same sequence} dG_t'
 *   dw   = sum over rows and heads of dn (.) xhat
 *
 * Gate given as logits (gate_logits != 0): the argument g holds raw logits
 * x, and the forget gate is g = logsigmoid(x), so the per-token factor is
 * exp(g_u) = sigmoid(x_u) = 1 / (1 + exp(-x_u)) and the reported gradient is
 * the one with respect to x: dx_t = dg_t * dg_t/dx_t = dg_t * sigmoid(-x_t).
 * (The pages fix g as a log-space gate shaped like v; logsigmoid of
 * unconstrained logits is the plainest way to produce one, and it is how
 * every benchmark workload builds g.)
 *
 * Layout: every tensor is token-major and packed, [Ttot, H, D] row-major
 * (a dense [B, T, H, D] batch is Ttot = B*T with sequence b at offset b*T).
 * Inputs arrive as fp64 holding exactly the values the GPU receives (bf16
 * and fp32 values are exact in fp64); all arithmetic is fp64.
 *
 * Sampling for large shapes: unit_mask (bytes [nseq*Hkv], NULL = all)
 * selects (sequence, kv head) units; window > 0 restricts every selected
 * sequence to its last `window` rows.  Forward rows depend only on earlier
 * rows, and dk/dv/dg of a suffix depend only on rows inside that suffix, so
 * the suffix results are exact.  dq is exact for every computed row too.
 * window < 0 (backward only) selects the first -window rows and keys
 * instead: the rows' forward and gradient reaching x are computed for the
 * whole sequence (every later query takes part in the keys' dk and dv),
 * then dq of the first rows and dk, dv of the first keys; dg, a suffix sum
 * over the whole sequence, is not computed in that mode.
 * Outputs outside the computed set are left untouched.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int64_t nseq;
  const int64_t *cu;
  int64_t Hq, Hkv, G, dk, dv;
  double scale, eps;
  int o_norm, gate_logits;
  const double *q, *k, *v, *g, *w, *z;
  const double *m_in;
  const unsigned char *mask;
  int64_t window;
  double *a; /* exp(g) (or sigmoid(x) for logits), [Ttot, Hkv, dv] */
} octx;

typedef struct {
  int64_t s, h, i; /* sequence, q head (or kv head for key items), seq-relative row */
} item;

static int64_t seq_len(const octx *c, int64_t s) { return c->cu[s + 1] - c->cu[s]; }
static int64_t row_lo(const octx *c, int64_t s) {
  int64_t L = seq_len(c, s);
  if (c->window > 0 && c->window < L) return L - c->window;
  return 0;
}
/* Rows whose dq, and keys whose dk and dv, are reported: [out_lo, out_hi). */
static int64_t out_lo(const octx *c, int64_t s) { return row_lo(c, s); }
static int64_t out_hi(const octx *c, int64_t s) {
  int64_t L = seq_len(c, s);
  if (c->window < 0 && -c->window < L) return -c->window;
  return L;
}
static int unit_on(const octx *c, int64_t s, int64_t kvh) {
  return c->mask == NULL || c->mask[s * c->Hkv + kvh] != 0;
}

static const double *Q(const octx *c, int64_t t, int64_t h) { return c->q + (t * c->Hq + h) * c->dk; }
static const double *K(const octx *c, int64_t t, int64_t kh) { return c->k + (t * c->Hkv + kh) * c->dk; }
static const double *V(const octx *c, int64_t t, int64_t kh) { return c->v + (t * c->Hkv + kh) * c->dv; }
static const double *A(const octx *c, int64_t t, int64_t kh) { return c->a + (t * c->Hkv + kh) * c->dv; }

/* 1 when every channel of a running decay product is exactly zero: from then on
 * every later term of the walk is an exact zero (a product of finite factors with
 * 0), so the walk can stop without changing any result. */
static int all_zero(const double *D, int64_t n) {
  for (int64_t d = 0; d < n; ++d)
    if (D[d] != 0.0) return 0;
  return 1;
}

static double dot(const double *x, const double *y, int64_t n) {
  double acc = 0.0;
  for (int64_t e = 0; e < n; ++e) acc += x[e] * y[e];
  return acc;
}

/* Scores s_ij for j = 0..i of row i (sequence-relative), into sc[0..i]; returns m_i. */
static double row_scores(const octx *c, int64_t s, int64_t h, int64_t i, double *sc) {
  int64_t base = c->cu[s], kh = h / c->G;
  const double *qi = Q(c, base + i, h);
  double m = -INFINITY;
  for (int64_t j = 0; j <= i; ++j) {
    sc[j] = c->scale * dot(qi, K(c, base + j, kh), c->dk);
    if (sc[j] > m) m = sc[j];
  }
  if (c->m_in) m = c->m_in[(base + i) * c->Hq + h];
  return m;
}

/* x_i: walk j = i, i-1, ..., 0 carrying D = prod_{u=j+1..i} exp(g_u). */
static void row_x(const octx *c, int64_t s, int64_t h, int64_t i, const double *sc, double m,
                  double *x, double *D) {
  int64_t base = c->cu[s], kh = h / c->G, dv = c->dv;
  for (int64_t d = 0; d < dv; ++d) { x[d] = 0.0; D[d] = 1.0; }
  for (int64_t j = i; j >= 0; --j) {
    double p = exp(sc[j] - m);
    const double *vj = V(c, base + j, kh);
    const double *aj = A(c, base + j, kh);
    for (int64_t d = 0; d < dv; ++d) x[d] += p * D[d] * vj[d];
    for (int64_t d = 0; d < dv; ++d) D[d] *= aj[d];
    if (all_zero(D, dv)) break;
  }
}

static double row_rstd(const octx *c, const double *x) {
  double ss = 0.0;
  for (int64_t d = 0; d < c->dv; ++d) ss += x[d] * x[d];
  return 1.0 / sqrt(ss / c->dv + c->eps);
}

static int setup(octx *c, int64_t nseq, const int64_t *cu, int64_t Hq, int64_t Hkv, int64_t dk,
                 int64_t dv, double scale, double eps, int o_norm, int gate_logits, const double *q, const double *k,
                 const double *v, const double *g, const double *w, const double *z, const double *m_in,
                 const unsigned char *mask, int64_t window) {
  if (nseq < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || dk <= 0 || dv <= 0) return 1;
  c->nseq = nseq; c->cu = cu; c->Hq = Hq; c->Hkv = Hkv; c->G = Hq / Hkv;
  c->dk = dk; c->dv = dv; c->scale = scale; c->eps = eps; c->o_norm = o_norm; c->gate_logits = gate_logits;
  c->q = q; c->k = k; c->v = v; c->g = g; c->w = w; c->z = z; c->m_in = m_in;
  c->mask = mask; c->window = window;
  int64_t Ttot = cu[nseq];
  c->a = (double *)malloc(sizeof(double) * (size_t)(Ttot > 0 ? Ttot : 1) * Hkv * dv);
  if (!c->a) return 2;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < Ttot * Hkv * dv; ++e) c->a[e] = gate_logits ? 1.0 / (1.0 + exp(-g[e])) : exp(g[e]);
  return 0;
}

/* Rows of selected units, one item per (sequence, q head, row). Longest rows first. */
static item *row_items(const octx *c, int64_t *n) {
  int64_t cnt = 0;
  for (int64_t s = 0; s < c->nseq; ++s)
    for (int64_t h = 0; h < c->Hq; ++h)
      if (unit_on(c, s, h / c->G)) cnt += seq_len(c, s) - row_lo(c, s);
  item *it = (item *)malloc(sizeof(item) * (size_t)(cnt > 0 ? cnt : 1));
  int64_t p = 0;
  for (int64_t s = 0; s < c->nseq; ++s)
    for (int64_t h = 0; h < c->Hq; ++h)
      if (unit_on(c, s, h / c->G))
        for (int64_t i = seq_len(c, s) - 1; i >= row_lo(c, s); --i) { it[p].s = s; it[p].h = h; it[p].i = i; ++p; }
  *n = cnt;
  return it;
}

static int64_t max_len(const octx *c) {
  int64_t mx = 1;
  for (int64_t s = 0; s < c->nseq; ++s) if (seq_len(c, s) > mx) mx = seq_len(c, s);
  return mx;
}

int fix_oracle_fwd(int64_t nseq, const int64_t *cu, int64_t Hq, int64_t Hkv, int64_t dk, int64_t dv,
                   double scale, double eps, int o_norm, int gate_logits, const double *q, const double *k,
                   const double *v, const double *g, const double *w, const double *z,
                   const double *m_in, const unsigned char *unit_mask, int64_t window, double *o,
                   double *x_out, double *m_out, double *rstd_out) {
  octx c;
  int st = setup(&c, nseq, cu, Hq, Hkv, dk, dv, scale, eps, o_norm, gate_logits, q, k, v, g, w, z, m_in,
                 unit_mask, window);
  if (st) return st;
  int64_t n;
  item *it = row_items(&c, &n);
  int64_t Lmax = max_len(&c);
#pragma omp parallel
  {
    double *sc = (double *)malloc(sizeof(double) * (size_t)Lmax);
    double *x = (double *)malloc(sizeof(double) * (size_t)dv);
    double *D = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 8)
    for (int64_t e = 0; e < n; ++e) {
      int64_t s = it[e].s, h = it[e].h, i = it[e].i, t = cu[s] + i;
      double m = row_scores(&c, s, h, i, sc);
      row_x(&c, s, h, i, sc, m, x, D);
      double r = row_rstd(&c, x);
      double *orow = o + (t * Hq + h) * dv;
      for (int64_t d = 0; d < dv; ++d) {
        double val = x[d];
        if (o_norm) val = val * r * (w ? w[d] : 1.0);
        if (z) val *= z[(t * Hq + h) * dv + d];
        orow[d] = val;
      }
      if (x_out) memcpy(x_out + (t * Hq + h) * dv, x, sizeof(double) * (size_t)dv);
      if (m_out) m_out[t * Hq + h] = m;
      if (rstd_out) rstd_out[t * Hq + h] = r;
    }
    free(sc); free(x); free(D);
  }
  free(it);
  free(c.a);
  return 0;
}

int fix_oracle_bwd(int64_t nseq, const int64_t *cu, int64_t Hq, int64_t Hkv, int64_t dk, int64_t dv,
                   double scale, double eps, int o_norm, int gate_logits, const double *q, const double *k,
                   const double *v, const double *g, const double *w, const double *z,
                   const double *dO, const double *m_in, const unsigned char *unit_mask,
                   int64_t window, double *dq, double *dk_out, double *dv_out, double *dg,
                   double *dw, double *dz) {
  octx c;
  int st = setup(&c, nseq, cu, Hq, Hkv, dk, dv, scale, eps, o_norm, gate_logits, q, k, v, g, w, z, m_in,
                 unit_mask, window);
  if (st) return st;
  int64_t Ttot = cu[nseq];
  size_t rows = (size_t)(Ttot > 0 ? Ttot : 1) * (size_t)Hq;
  double *X = (double *)calloc(rows * (size_t)dv, sizeof(double));
  double *DL = (double *)calloc(rows * (size_t)dv, sizeof(double));
  double *M = (double *)calloc(rows, sizeof(double));
  double *R = (double *)calloc(rows, sizeof(double));
  if (!X || !DL || !M || !R) return 2;
  int64_t n;
  item *it = row_items(&c, &n);
  int64_t Lmax = max_len(&c);

  /* Pass 1: forward rows, then delta = dL/dx of every computed row. */
#pragma omp parallel
  {
    double *sc = (double *)malloc(sizeof(double) * (size_t)Lmax);
    double *D = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 8)
    for (int64_t e = 0; e < n; ++e) {
      int64_t s = it[e].s, h = it[e].h, i = it[e].i, t = cu[s] + i;
      size_t ro = (size_t)(t * Hq + h);
      double *x = X + ro * dv;
      double m = row_scores(&c, s, h, i, sc);
      row_x(&c, s, h, i, sc, m, x, D);
      double r = row_rstd(&c, x);
      M[ro] = m; R[ro] = r;
      const double *dOr = dO + ro * dv;
      const double *zr = z ? z + ro * dv : NULL;
      double *delta = DL + ro * dv;
      double proj = 0.0;
      for (int64_t d = 0; d < dv; ++d) {
        double dn = dOr[d] * (zr ? zr[d] : 1.0);
        double nval = o_norm ? x[d] * r * (w ? w[d] : 1.0) : x[d];
        if (dz) dz[ro * dv + d] = dOr[d] * nval;
        if (o_norm) {
          double dxh = dn * (w ? w[d] : 1.0);
          delta[d] = dxh;
          proj += dxh * x[d] * r;
        } else {
          delta[d] = dn;
        }
      }
      if (o_norm) {
        proj /= dv;
        for (int64_t d = 0; d < dv; ++d) delta[d] = r * (delta[d] - x[d] * r * proj);
      }
    }
    free(sc); free(D);
  }

  /* dw: fixed-order sum over computed rows, one output channel per iteration. */
  if (dw && o_norm) {
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < dv; ++d) {
      double acc = 0.0;
      for (int64_t s = 0; s < nseq; ++s)
        for (int64_t i = row_lo(&c, s); i < seq_len(&c, s); ++i)
          for (int64_t h = 0; h < Hq; ++h) {
            if (!unit_on(&c, s, h / c.G)) continue;
            size_t ro = (size_t)((cu[s] + i) * Hq + h);
            double dn = dO[ro * dv + d] * (z ? z[ro * dv + d] : 1.0);
            acc += dn * X[ro * dv + d] * R[ro];
          }
      dw[d] = acc;
    }
  } else if (dw) {
    for (int64_t d = 0; d < dv; ++d) dw[d] = 0.0;
  }

  /* Pass 2: dq_i = scale sum_{j<=i} P_ij dP_ij k_j, walking j downward with the running D. */
#pragma omp parallel
  {
    double *sc = (double *)malloc(sizeof(double) * (size_t)Lmax);
    double *D = (double *)malloc(sizeof(double) * (size_t)dv);
    double *acc = (double *)malloc(sizeof(double) * (size_t)dk);
#pragma omp for schedule(dynamic, 8)
    for (int64_t e = 0; e < n; ++e) {
      int64_t s = it[e].s, h = it[e].h, i = it[e].i, t = cu[s] + i, base = cu[s], kh = h / c.G;
      if (i < out_lo(&c, s) || i >= out_hi(&c, s)) continue;
      size_t ro = (size_t)(t * Hq + h);
      (void)row_scores(&c, s, h, i, sc);
      double m = M[ro];
      const double *delta = DL + ro * dv;
      for (int64_t d = 0; d < dv; ++d) D[d] = 1.0;
      for (int64_t e2 = 0; e2 < dk; ++e2) acc[e2] = 0.0;
      for (int64_t j = i; j >= 0; --j) {
        const double *vj = V(&c, base + j, kh);
        const double *aj = A(&c, base + j, kh);
        double dP = 0.0;
        for (int64_t d = 0; d < dv; ++d) dP += D[d] * vj[d] * delta[d];
        double dS = exp(sc[j] - m) * dP;
        const double *kj = K(&c, base + j, kh);
        for (int64_t e2 = 0; e2 < dk; ++e2) acc[e2] += dS * kj[e2];
        for (int64_t d = 0; d < dv; ++d) D[d] *= aj[d];
        if (all_zero(D, dv)) break;
      }
      for (int64_t e2 = 0; e2 < dk; ++e2) dq[ro * dk + e2] = scale * acc[e2];
    }
    free(sc); free(D); free(acc);
  }

  /* Pass 3: per key row j of a unit, walk i upward from j over the group's heads. */
  int64_t nk = 0;
  for (int64_t s = 0; s < nseq; ++s)
    for (int64_t kh = 0; kh < Hkv; ++kh)
      if (unit_on(&c, s, kh)) nk += out_hi(&c, s) - out_lo(&c, s);
  item *kit = (item *)malloc(sizeof(item) * (size_t)(nk > 0 ? nk : 1));
  {
    int64_t p = 0;
    for (int64_t s = 0; s < nseq; ++s)
      for (int64_t kh = 0; kh < Hkv; ++kh)
        if (unit_on(&c, s, kh))
          for (int64_t j = out_lo(&c, s); j < out_hi(&c, s); ++j) { kit[p].s = s; kit[p].h = kh; kit[p].i = j; ++p; }
  }
#pragma omp parallel
  {
    double *D = (double *)malloc(sizeof(double) * (size_t)dv);
    double *adv = (double *)malloc(sizeof(double) * (size_t)dv);
    double *adk = (double *)malloc(sizeof(double) * (size_t)dk);
#pragma omp for schedule(dynamic, 8)
    for (int64_t e = 0; e < nk; ++e) {
      int64_t s = kit[e].s, kh = kit[e].h, j = kit[e].i, base = cu[s], L = seq_len(&c, s);
      const double *kj = K(&c, base + j, kh);
      const double *vj = V(&c, base + j, kh);
      for (int64_t d = 0; d < dv; ++d) adv[d] = 0.0;
      for (int64_t e2 = 0; e2 < dk; ++e2) adk[e2] = 0.0;
      for (int64_t h = kh * c.G; h < (kh + 1) * c.G; ++h) {
        for (int64_t d = 0; d < dv; ++d) D[d] = 1.0;
        for (int64_t i = j; i < L; ++i) {
          if (i > j) {
            const double *ai = A(&c, base + i, kh);
            for (int64_t d = 0; d < dv; ++d) D[d] *= ai[d];
            if (all_zero(D, dv)) break;
          }
          size_t ro = (size_t)((base + i) * Hq + h);
          const double *qi = Q(&c, base + i, h);
          double P = exp(c.scale * dot(qi, kj, dk) - M[ro]);
          const double *delta = DL + ro * dv;
          double dP = 0.0;
          for (int64_t d = 0; d < dv; ++d) {
            dP += D[d] * vj[d] * delta[d];
            adv[d] += P * D[d] * delta[d];
          }
          double dS = P * dP;
          for (int64_t e2 = 0; e2 < dk; ++e2) adk[e2] += dS * qi[e2];
        }
      }
      size_t ko = (size_t)((base + j) * Hkv + kh);
      for (int64_t d = 0; d < dv; ++d) dv_out[ko * dv + d] = adv[d];
      for (int64_t e2 = 0; e2 < dk; ++e2) dk_out[ko * dk + e2] = scale * adk[e2];
    }
    free(D); free(adv); free(adk);
  }
  free(kit);

  /* Pass 4: dG_t = sum_h delta_t x_t - v_t dv_t, then dg_t = sum_{t'>=t} dG_t' per sequence. */
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t s = 0; s < nseq; ++s)
    for (int64_t kh = 0; kh < Hkv; ++kh) {
      if (!unit_on(&c, s, kh) || c.window < 0) continue;
      int64_t base = cu[s], L = seq_len(&c, s), lo = row_lo(&c, s);
      for (int64_t d = 0; d < dv; ++d) {
        double run = 0.0;
        for (int64_t t = L - 1; t >= lo; --t) {
          double dG = 0.0;
          for (int64_t h = kh * c.G; h < (kh + 1) * c.G; ++h) {
            size_t ro = (size_t)((base + t) * Hq + h);
            dG += DL[ro * dv + d] * X[ro * dv + d];
          }
          size_t ko = (size_t)((base + t) * Hkv + kh);
          dG -= v[ko * dv + d] * dv_out[ko * dv + d];
          run += dG;
          /* logits: chain rule through g = logsigmoid(x) */
          dg[ko * dv + d] = c.gate_logits ? run / (1.0 + exp(g[ko * dv + d])) : run;
        }
      }
    }

  free(it); free(X); free(DL); free(M); free(R); free(c.a);
  return 0;
}
