/*
 * pararnn_oracle.c -- plain fp64 CPU oracle for the ParaRNN Newton solve.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the independent checker of the HIP
 * path: only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load it. It shares no code, header, table or helper with the HIP
 * library and includes nothing from it. Everything is computed in double
 * precision with host libm, one channel at a time, in the order the method
 * states its steps; threads only split the independent channels.
 *
 * Sources (web pages on ParaRNN):
 *  - ParaRNN article, cafecomtech.com ("ParaRNN: Apple destrava treino paralelo
 *    de RNNs nao-lineares e escala pra 7B parametros"):
 *      section "O compromisso que SSMs fizeram": the nonlinear recurrence
 *        h_l = sigma_l(h_{l-1}, x_l) versus the linear SSM
 *        h_l = A_l h_{l-1} + B_l x_l;
 *      section "A sacada: metodo de Newton": the whole sequence is one system
 *        whose unknowns are all hidden states; Newton linearises it with the
 *        local Jacobians; the linearised system is a linear SSM with the
 *        Jacobians in the role of A_l; each iteration solves that SSM;
 *      section "Engenharia pra escalar": diagonal cell matrices make the
 *        Jacobian diagonal (ParaGRU) or 2x2 block-diagonal (ParaLSTM).
 *  - ParaRNN article, aifeed.sk ("Apple vracia do hry RNN ..."): Newton
 *    iterations plus parallel reductions; training runs in parallel.
 *
 * The cells are the GRU and LSTM with diagonal recurrent coefficients a (one
 * value per gate and channel), gate inputs u precomputed:
 *   GRU  (gates z, r, c):  z = s(a_z h + u_z), r = s(a_r h + u_r),
 *                          c~ = tanh(a_c (r h) + u_c), h' = (1-z) h + z c~.
 *   LSTM (gates i, f, o, g; state (c, h)): i, f, o = s(a_* h + u_*),
 *                          g = tanh(a_g h + u_g), c' = f c + i g,
 *                          h' = o tanh(c').  The gates read h only.
 * s() is the logistic sigmoid.
 *
 * Array layouts (row-major):
 *   u  [B][L][G][D] float  (bf16 inputs arrive widened to float, exactly)
 *   a  [G][D] float
 *   s0 [NS][B][D] double or NULL (zero initial state)
 *   state arrays [NS][B][L][D] double; state index 0 = h for the GRU,
 *   (0, 1) = (c, h) for the LSTM.
 *   dh [B][L][D] float, du [B][L][G][D] double.
 *
 * Parity is pinned (not self-referential) by the CPU test suite: worked
 * examples with exact values, equivalence with torch.nn.GRUCell / LSTMCell in
 * float64, central finite differences of f, brute-force dense Newton with
 * numpy.linalg.solve, the linear-cell closed form, the fixed point equal to
 * the sequential trajectory, and finite differences of the loss for BPTT.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CELL_GRU 0
#define CELL_LSTM 1
#define MAXG 4
#define MAXS 2

static int n_gates(int cell) { return cell == CELL_GRU ? 3 : 4; }
static int n_state(int cell) { return cell == CELL_GRU ? 1 : 2; }

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* One cell evaluation at previous state s (NS values) and gate inputs u (G
 * values) with coefficients a (G values). Outputs:
 *   f[NS]          the next state f(s, u)
 *   J[NS][NS]      d f / d s   (J[row][col] = d f_row / d s_col)
 *   dfdu[NS][G]    d f / d u
 *   dfda[NS][G]    d f / d a
 */
typedef struct {
  double f[MAXS];
  double J[MAXS][MAXS];
  double dfdu[MAXS][MAXG];
  double dfda[MAXS][MAXG];
} cell_eval;

static void gru_eval(const double* s, const double* u, const double* a, cell_eval* e) {
  double h = s[0];
  double z = sigmoid(a[0] * h + u[0]);
  double r = sigmoid(a[1] * h + u[1]);
  double c = tanh(a[2] * (r * h) + u[2]);
  memset(e, 0, sizeof(*e));
  e->f[0] = (1.0 - z) * h + z * c;
  /* derivatives of the three pre-activations' outputs */
  double dz = z * (1.0 - z);      /* dz / d pre_z */
  double dr = r * (1.0 - r);      /* dr / d pre_r */
  double dc = 1.0 - c * c;        /* dc~ / d pre_c */
  /* d h' / d pre_z, d pre_r, d pre_c */
  double g_z = (c - h) * dz;
  double g_c = z * dc;
  double g_r = g_c * a[2] * h * dr;
  e->dfdu[0][0] = g_z;
  e->dfdu[0][1] = g_r;
  e->dfdu[0][2] = g_c;
  /* pre_z = a_z h + u_z, pre_r = a_r h + u_r, pre_c = a_c (r h) + u_c */
  e->dfda[0][0] = g_z * h;
  e->dfda[0][1] = g_r * h;
  e->dfda[0][2] = g_c * r * h;
  /* d h'/d h = (1 - z) + g_z a_z + g_c a_c (r + h dr a_r) */
  e->J[0][0] = (1.0 - z) + g_z * a[0] + g_c * a[2] * (r + h * dr * a[1]);
}

static void lstm_eval(const double* s, const double* u, const double* a, cell_eval* e) {
  double cp = s[0], hp = s[1];
  double i = sigmoid(a[0] * hp + u[0]);
  double f = sigmoid(a[1] * hp + u[1]);
  double o = sigmoid(a[2] * hp + u[2]);
  double g = tanh(a[3] * hp + u[3]);
  double cn = f * cp + i * g;
  double t = tanh(cn);
  memset(e, 0, sizeof(*e));
  e->f[0] = cn;
  e->f[1] = o * t;
  /* d c' / d pre_{i,f,o,g} */
  double dci = g * i * (1.0 - i);
  double dcf = cp * f * (1.0 - f);
  double dcg = i * (1.0 - g * g);
  double q = o * (1.0 - t * t); /* d h' / d c' */
  double dho = t * o * (1.0 - o);
  e->dfdu[0][0] = dci;
  e->dfdu[0][1] = dcf;
  e->dfdu[0][2] = 0.0;
  e->dfdu[0][3] = dcg;
  e->dfdu[1][0] = q * dci;
  e->dfdu[1][1] = q * dcf;
  e->dfdu[1][2] = dho;
  e->dfdu[1][3] = q * dcg;
  for (int r = 0; r < 2; ++r)
    for (int k = 0; k < 4; ++k) e->dfda[r][k] = e->dfdu[r][k] * hp; /* pre = a h + u */
  /* d c'/d h = sum over gates of d c'/d pre * a */
  double X = dci * a[0] + dcf * a[1] + dcg * a[3];
  e->J[0][0] = f;
  e->J[0][1] = X;
  e->J[1][0] = q * f;
  e->J[1][1] = dho * a[2] + q * X;
}

static void eval_cell(int cell, const double* s, const double* u, const double* a, cell_eval* e) {
  if (cell == CELL_GRU)
    gru_eval(s, u, a, e);
  else
    lstm_eval(s, u, a, e);
}

/* ------------------------------------------------------------------------ */
/* per-channel helpers                                                       */

typedef struct {
  int cell, B, L, D, G, NS;
  const float* u;
  const float* a;
  const double* s0;
} problem;

static size_t idx_u(const problem* p, int b, int l, int g, int d) {
  return (((size_t)b * p->L + l) * p->G + g) * p->D + d;
}
static size_t idx_s(const problem* p, int s, int b, int l, int d) {
  return (((size_t)s * p->B + b) * p->L + l) * p->D + d;
}
static void load_u(const problem* p, int b, int l, int d, double* u) {
  for (int g = 0; g < p->G; ++g) u[g] = (double)p->u[idx_u(p, b, l, g, d)];
}
static void load_a(const problem* p, int d, double* a) {
  for (int g = 0; g < p->G; ++g) a[g] = (double)p->a[(size_t)g * p->D + d];
}
static void load_s0(const problem* p, int b, int d, double* s) {
  for (int k = 0; k < p->NS; ++k) s[k] = p->s0 ? p->s0[((size_t)k * p->B + b) * p->D + d] : 0.0;
}

/* ------------------------------------------------------------------------ */
/* Thread pool over channel ranges. Work items are d-ranges; every item loops
 * over all batch rows, so per-d accumulations (da) have a single owner.      */

typedef void (*chan_fn)(void* ctx, int d_lo, int d_hi);
typedef struct {
  chan_fn fn;
  void* ctx;
  int lo, hi;
} job;

static void* run_job(void* arg) {
  job* j = (job*)arg;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static void parallel_over_d(int D, int nthreads, chan_fn fn, void* ctx) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > D) nthreads = D;
  if (nthreads == 1) {
    fn(ctx, 0, D);
    return;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  job* jobs = (job*)malloc(sizeof(job) * nthreads);
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].lo = (int)((long long)D * t / nthreads);
    jobs[t].hi = (int)((long long)D * (t + 1) / nthreads);
    pthread_create(&th[t], NULL, run_job, &jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
}

static int check_problem(int cell, int B, int L, int D, const float* u, const float* a) {
  if (cell != CELL_GRU && cell != CELL_LSTM) return -1;
  if (B <= 0 || L <= 0 || D <= 0 || !u || !a) return -1;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O1. Sequential application of the recurrence (the fixed point).         */

typedef struct {
  problem p;
  double* out;
} seq_ctx;

static void seq_worker(void* vctx, int d_lo, int d_hi) {
  seq_ctx* c = (seq_ctx*)vctx;
  const problem* p = &c->p;
  double s[MAXS], uu[MAXG], aa[MAXG];
  cell_eval e;
  for (int b = 0; b < p->B; ++b)
    for (int d = d_lo; d < d_hi; ++d) {
      load_a(p, d, aa);
      load_s0(p, b, d, s);
      for (int l = 0; l < p->L; ++l) {
        load_u(p, b, l, d, uu);
        eval_cell(p->cell, s, uu, aa, &e);
        for (int k = 0; k < p->NS; ++k) {
          s[k] = e.f[k];
          c->out[idx_s(p, k, b, l, d)] = s[k];
        }
      }
    }
}

int oracle_seq(int cell, int B, int L, int D, const float* u, const float* a, const double* s0,
               double* out, int nthreads) {
  if (check_problem(cell, B, L, D, u, a) || !out) return -1;
  seq_ctx c = {{cell, B, L, D, n_gates(cell), n_state(cell), u, a, s0}, out};
  parallel_over_d(D, nthreads, seq_worker, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O2. Newton on the whole-sequence system F_l(S) = S_l - f(S_{l-1}, u_l).   */
/* Iteration k -> k+1, for one channel:                                     */
/*   1. linearise at the current iterate: with p = S_{l-1} (S_{-1} = s0),    */
/*      A_l = df/ds(p, u_l) and b_l = f(p, u_l) - A_l p;                     */
/*   2. solve the linear SSM S'_l = A_l S'_{l-1} + b_l from S'_{-1} = s0;     */
/*   3. record max |S' - S| over l and state components.                    */
/* The initial iterate is S = 0 at every l.                                 */

typedef struct {
  problem p;
  int K;
  double* out;       /* [NS][B][L][D] K-th iterate */
  double* iterates;  /* optional [K][NS][B][L][D] */
  double* chan_upd;  /* [K][B][D] per-channel max |S^(k) - S^(k-1)| */
} newton_ctx;

static double nan_max(double m, double v) {
  if (isnan(v) || v > m) return v;
  return m;
}

static void newton_worker(void* vctx, int d_lo, int d_hi) {
  newton_ctx* c = (newton_ctx*)vctx;
  const problem* p = &c->p;
  const int L = p->L, NS = p->NS;
  double* S = (double*)calloc((size_t)L * NS, sizeof(double));   /* current iterate */
  double* Sn = (double*)calloc((size_t)L * NS, sizeof(double));  /* next iterate */
  double* A = (double*)malloc(sizeof(double) * (size_t)L * NS * NS);
  double* bv = (double*)malloc(sizeof(double) * (size_t)L * NS);
  double s0[MAXS], prev[MAXS], uu[MAXG], aa[MAXG];
  cell_eval e;
  for (int b = 0; b < p->B; ++b)
    for (int d = d_lo; d < d_hi; ++d) {
      load_a(p, d, aa);
      load_s0(p, b, d, s0);
      memset(S, 0, sizeof(double) * (size_t)L * NS);
      for (int k = 0; k < c->K; ++k) {
        /* 1. linearise around the current iterate */
        for (int l = 0; l < L; ++l) {
          const double* pp = (l == 0) ? s0 : &S[(size_t)(l - 1) * NS];
          load_u(p, b, l, d, uu);
          eval_cell(p->cell, pp, uu, aa, &e);
          for (int r = 0; r < NS; ++r) {
            double jp = 0.0;
            for (int q = 0; q < NS; ++q) {
              A[((size_t)l * NS + r) * NS + q] = e.J[r][q];
              jp += e.J[r][q] * pp[q];
            }
            bv[(size_t)l * NS + r] = e.f[r] - jp;
          }
        }
        /* 2. solve the linear SSM by a plain sequential loop */
        for (int r = 0; r < NS; ++r) prev[r] = s0[r];
        for (int l = 0; l < L; ++l) {
          for (int r = 0; r < NS; ++r) {
            double acc = bv[(size_t)l * NS + r];
            for (int q = 0; q < NS; ++q) acc += A[((size_t)l * NS + r) * NS + q] * prev[q];
            Sn[(size_t)l * NS + r] = acc;
          }
          for (int r = 0; r < NS; ++r) prev[r] = Sn[(size_t)l * NS + r];
        }
        /* 3. size of the Newton update */
        double m = 0.0;
        for (size_t x = 0; x < (size_t)L * NS; ++x) m = nan_max(m, fabs(Sn[x] - S[x]));
        c->chan_upd[((size_t)k * p->B + b) * p->D + d] = m;
        memcpy(S, Sn, sizeof(double) * (size_t)L * NS);
        if (c->iterates)
          for (int l = 0; l < L; ++l)
            for (int r = 0; r < NS; ++r)
              c->iterates[(size_t)k * NS * p->B * L * p->D + idx_s(p, r, b, l, d)] =
                  S[(size_t)l * NS + r];
      }
      for (int l = 0; l < L; ++l)
        for (int r = 0; r < NS; ++r) c->out[idx_s(p, r, b, l, d)] = S[(size_t)l * NS + r];
    }
  free(S);
  free(Sn);
  free(A);
  free(bv);
}

/* max_update[K][B]: per batch row, max over (l, d, state) of |S^(k+1) - S^(k)|.
 * A NaN anywhere in a row makes that row's entry NaN. */
int oracle_newton(int cell, int B, int L, int D, int K, const float* u, const float* a,
                  const double* s0, double* out, double* max_update, double* iterates,
                  int nthreads) {
  if (check_problem(cell, B, L, D, u, a) || K < 1 || !out) return -1;
  double* chan_upd = (double*)calloc((size_t)K * B * D, sizeof(double));
  if (!chan_upd) return -2;
  newton_ctx c = {{cell, B, L, D, n_gates(cell), n_state(cell), u, a, s0}, K, out, iterates,
                  chan_upd};
  parallel_over_d(D, nthreads, newton_worker, &c);
  if (max_update)
    for (int k = 0; k < K; ++k)
      for (int b = 0; b < B; ++b) {
        double m = 0.0;
        for (int d = 0; d < D; ++d) m = nan_max(m, chan_upd[((size_t)k * B + b) * D + d]);
        max_update[(size_t)k * B + b] = m;
      }
  free(chan_upd);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O3. Adjoint (backpropagation through the recurrence) along a given        */
/* trajectory S, for the loss gradient dh = dL/dh_l:                         */
/*   lambda_{L-1} = G_{L-1};  lambda_{l-1} = G_{l-1} + J_l^T lambda_l,       */
/*   with J_l = df/ds(S_{l-1}, u_l) and G_l = dL/d(state_l) = (0, dh_l) for  */
/*   the LSTM (no upstream gradient on c), dh_l for the GRU;                 */
/*   du_l = (df/du(S_{l-1}, u_l))^T lambda_l;                                */
/*   ds0 = J_0^T lambda_0;  da = sum over b, l of (df/da)^T lambda_l.        */

typedef struct {
  problem p;
  const double* S;
  const float* dh;
  double* du;
  double* ds0;
  double* da;
} adj_ctx;

static void adj_worker(void* vctx, int d_lo, int d_hi) {
  adj_ctx* c = (adj_ctx*)vctx;
  const problem* p = &c->p;
  const int L = p->L, NS = p->NS, G = p->G;
  double lam[MAXS], nl[MAXS], prev[MAXS], s0[MAXS], uu[MAXG], aa[MAXG];
  cell_eval e;
  for (int d = d_lo; d < d_hi; ++d) {
    double da_acc[MAXG] = {0, 0, 0, 0};
    load_a(p, d, aa);
    for (int b = 0; b < p->B; ++b) {
      load_s0(p, b, d, s0);
      for (int r = 0; r < NS; ++r) lam[r] = 0.0;
      lam[NS - 1] = (double)c->dh[((size_t)b * L + (L - 1)) * p->D + d];
      for (int l = L - 1; l >= 0; --l) {
        /* lam holds lambda_l here */
        for (int r = 0; r < NS; ++r) prev[r] = (l == 0) ? s0[r] : c->S[idx_s(p, r, b, l - 1, d)];
        load_u(p, b, l, d, uu);
        eval_cell(p->cell, prev, uu, aa, &e);
        for (int g = 0; g < G; ++g) {
          double acc = 0.0, acca = 0.0;
          for (int r = 0; r < NS; ++r) {
            acc += e.dfdu[r][g] * lam[r];
            acca += e.dfda[r][g] * lam[r];
          }
          c->du[idx_u(p, b, l, g, d)] = acc;
          da_acc[g] += acca;
        }
        /* J_l^T lambda_l */
        for (int q = 0; q < NS; ++q) {
          double acc = 0.0;
          for (int r = 0; r < NS; ++r) acc += e.J[r][q] * lam[r];
          nl[q] = acc;
        }
        if (l > 0) {
          for (int r = 0; r < NS; ++r) lam[r] = nl[r];
          lam[NS - 1] += (double)c->dh[((size_t)b * L + (l - 1)) * p->D + d];
        } else if (c->ds0) {
          for (int r = 0; r < NS; ++r) c->ds0[((size_t)r * p->B + b) * p->D + d] = nl[r];
        }
      }
    }
    if (c->da)
      for (int g = 0; g < G; ++g) c->da[(size_t)g * p->D + d] = da_acc[g];
  }
}

int oracle_adjoint(int cell, int B, int L, int D, const float* u, const float* a,
                   const double* s0, const double* S, const float* dh, double* du, double* ds0,
                   double* da, int nthreads) {
  if (check_problem(cell, B, L, D, u, a) || !S || !dh || !du) return -1;
  adj_ctx c = {{cell, B, L, D, n_gates(cell), n_state(cell), u, a, s0}, S, dh, du, ds0, da};
  parallel_over_d(D, nthreads, adj_worker, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Cell evaluation for n independent channels (pins: finite differences,     */
/* worked examples, library equivalence, dense Newton).                      */
/*   s [NS][n], u [G][n], a [G][n] -> f [NS][n], J [NS][NS][n],              */
/*   dfdu [NS][G][n], dfda [NS][G][n]; any output may be NULL.               */
int oracle_cell(int cell, int n, const double* s, const double* u, const double* a, double* f,
                double* J, double* dfdu, double* dfda) {
  if ((cell != CELL_GRU && cell != CELL_LSTM) || n < 0 || !s || !u || !a) return -1;
  const int G = n_gates(cell), NS = n_state(cell);
  double ss[MAXS], uu[MAXG], aa[MAXG];
  cell_eval e;
  for (int x = 0; x < n; ++x) {
    for (int r = 0; r < NS; ++r) ss[r] = s[(size_t)r * n + x];
    for (int g = 0; g < G; ++g) {
      uu[g] = u[(size_t)g * n + x];
      aa[g] = a[(size_t)g * n + x];
    }
    eval_cell(cell, ss, uu, aa, &e);
    for (int r = 0; r < NS; ++r) {
      if (f) f[(size_t)r * n + x] = e.f[r];
      for (int q = 0; q < NS; ++q)
        if (J) J[((size_t)r * NS + q) * n + x] = e.J[r][q];
      for (int g = 0; g < G; ++g) {
        if (dfdu) dfdu[((size_t)r * G + g) * n + x] = e.dfdu[r][g];
        if (dfda) dfda[((size_t)r * G + g) * n + x] = e.dfda[r][g];
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O4. The linear recurrence alone (the scan tier). The pages' linear SSM    */
/* h_l = A_l h_{l-1} + B_l x_l (ParaRNN article, cafecomtech.com, section    */
/* "O compromisso que SSMs fizeram"), with the input term already formed:    */
/*   s_l = A_l s_{l-1} + b_l,  l = 0 .. L-1,  s_{-1} = s0 (zero when NULL),  */
/* per channel (b, d); A_l is a scalar (ns = 1, diagonal cell) or a 2x2      */
/* block over the channel's two state components (ns = 2), as in section     */
/* "Engenharia pra escalar". Component-major planes:                          */
/*   A [ns*ns][B][L][D] (row-major block entries), b and s [ns][B][L][D],      */
/*   s0 [ns][B][D].                                                           */
typedef struct {
  int ns, B, L, D;
  const double *A, *b, *s0;
  double* s;
} scan_ctx;

static void scan_worker(void* vctx, int d_lo, int d_hi) {
  const scan_ctx* c = (const scan_ctx*)vctx;
  const size_t plane = (size_t)c->B * c->L * c->D;
  for (int d = d_lo; d < d_hi; ++d)
    for (int b = 0; b < c->B; ++b) {
      double prev[MAXS], next[MAXS];
      for (int r = 0; r < c->ns; ++r) prev[r] = c->s0 ? c->s0[((size_t)r * c->B + b) * c->D + d] : 0.0;
      for (int l = 0; l < c->L; ++l) {
        const size_t at = ((size_t)b * c->L + l) * c->D + d;
        for (int r = 0; r < c->ns; ++r) {
          double acc = c->b[(size_t)r * plane + at];
          for (int q = 0; q < c->ns; ++q) acc += c->A[(size_t)(r * c->ns + q) * plane + at] * prev[q];
          next[r] = acc;
        }
        for (int r = 0; r < c->ns; ++r) {
          c->s[(size_t)r * plane + at] = next[r];
          prev[r] = next[r];
        }
      }
    }
}

int oracle_scan(int ns, int B, int L, int D, const double* A, const double* b, const double* s0, double* s,
                int nthreads) {
  if ((ns != 1 && ns != 2) || B <= 0 || L <= 0 || D <= 0 || !A || !b || !s) return -1;
  scan_ctx c = {ns, B, L, D, A, b, s0, s};
  parallel_over_d(D, nthreads, scan_worker, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O5. The linear recurrence with a dense n x n matrix per step: the          */
/* linearised system of a generic RNN, whose Jacobians are dense (ParaRNN     */
/* article, cafecomtech.com, section "Engenharia pra escalar": storage grows  */
/* as n^2 and the products as n^3):                                          */
/*   s_l = A_l s_{l-1} + b_l,  l = 0 .. L-1,  s_{-1} = s0 (zero when NULL).   */
/* Layouts (row-major): A [B][L][n][n] (A_l[r][q] multiplies s_{l-1}[q] into */
/* s_l[r]), b and s [B][L][n], s0 [B][n]. Threads split the batch rows.      */
typedef struct {
  int B, L, n;
  const double *A, *b, *s0;
  double* s;
} dense_ctx;

static void dense_worker(void* vctx, int b_lo, int b_hi) {
  const dense_ctx* c = (const dense_ctx*)vctx;
  const int n = c->n;
  double* prev = (double*)malloc(sizeof(double) * (size_t)n);
  double* next = (double*)malloc(sizeof(double) * (size_t)n);
  for (int b = b_lo; b < b_hi; ++b) {
    for (int r = 0; r < n; ++r) prev[r] = c->s0 ? c->s0[(size_t)b * n + r] : 0.0;
    for (int l = 0; l < c->L; ++l) {
      const size_t step = (size_t)b * c->L + l;
      const double* Al = c->A + step * n * n;
      for (int r = 0; r < n; ++r) {
        double acc = c->b[step * n + r];
        for (int q = 0; q < n; ++q) acc += Al[(size_t)r * n + q] * prev[q];
        next[r] = acc;
      }
      for (int r = 0; r < n; ++r) {
        c->s[step * n + r] = next[r];
        prev[r] = next[r];
      }
    }
  }
  free(prev);
  free(next);
}

int oracle_scan_dense(int B, int L, int n, const double* A, const double* b, const double* s0, double* s,
                      int nthreads) {
  if (B <= 0 || L <= 0 || n <= 0 || !A || !b || !s) return -1;
  dense_ctx c = {B, L, n, A, b, s0, s};
  parallel_over_d(B, nthreads, dense_worker, &c);
  return 0;
}
