/*
 * dsc_oracle.c -- plain, slow, fp64 CPU reference of the dynamic short causal
 * convolution.  TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and
 * the CPU-baseline leg of the benchmark call it; the GPU library never does.
 * It shares no code, header or table with the HIP path.
 *
 * Sources (the pages this follows):
 *   [gist]  gist.science technical summary "Dynamische Korte Convoluties
 *           Verbeteren Transformers", section Methodologie > Dynamische Korte
 *           Convoluties: bullet "Mechanisme" (the defining sum over k < W of
 *           w(t)_k (.) x_{t-k}), bullet "Parametrisatie" (1. low-rank
 *           factorisation of rank R, 2. head-wise tying: one filter shared by H
 *           consecutive channels), bullet "Plaatsing" (residual X + conv(X));
 *           section Efficiente Trainingsimplementatie, bullet "Fused Low-Rank
 *           Kernel" (w is the product zU of the low-rank input z and the
 *           projection matrix U).
 *   [wisp]  wispaper.ai blog "Dynamic Short Convolutions: The 'Locality Bias'
 *           Transformers Were Missing", Methodology > 1. Mathematical Intuition
 *           (static vs dynamic sum), 2. Solving the Parameter Explosion
 *           (rank-16 example, head-wise tying).
 *
 * Readings taken where the pages are silent:
 *   - taps that reach before the start of a sequence (t-k < 0) read zero;
 *     every sequence b is independent and the output has length T;
 *   - tap k = 0 multiplies the current token x_t;
 *   - channel c belongs to group g(c) = floor(c / H), G = D / H groups;
 *   - U has shape (R, G*W) and column g*W + k holds tap k of group g;
 *   - y = act(conv(x)) + rho * x, act in {identity, SiLU}; the SiLU case is a
 *     configuration of the benchmark suite, not of the pages;
 *   - the backward pass is the exact derivative of that forward.
 *
 * Layouts (all row-major, fp64):
 *   x, y, dy, dx : (B, T, D)      w, dw : (B, T, G, W)
 *   z, dz        : (B, T, R)      U, dU : (R, G*W)
 *
 * Parallelism: OpenMP over independent output rows or columns only; every
 * output element is a single sequential sum in a fixed order, so the results
 * do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX3(b, t, c, T, D) ((((int64_t)(b)) * (T) + (t)) * (D) + (c))

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* SiLU and its derivative, written from the definition s * sigmoid(s). */
static double act_fn(double s, int act) {
  if (!act) return s;
  return s / (1.0 + exp(-s));
}

static double act_grad(double s, int act) {
  if (!act) return 1.0;
  double sg = 1.0 / (1.0 + exp(-s));
  return sg * (1.0 + s * (1.0 - sg));
}

/*
 * Pre-activation convolution at one (b, t, c) -- [gist] Mechanisme:
 *   s = sum_{k=0}^{W-1} w[b,t,g(c),k] * x[b,t-k,c], taps with t-k < 0 read 0.
 */
static double conv_at(const double *x, const double *w, int64_t T, int64_t D,
                      int64_t G, int W, int H, int64_t b, int64_t t, int64_t c) {
  int64_t g = c / H;
  const double *wt = w + IDX3(b, t, g, T, G) * W;
  double s = 0.0;
  for (int k = 0; k < W; ++k) {
    if (t - k < 0) break;
    s += wt[k] * x[IDX3(b, t - k, c, T, D)];
  }
  return s;
}

/* Forward, head-wise tying: y = act(s) + rho * x ([gist] Mechanisme,
 * Parametrisatie 2, Plaatsing). */
void oracle_headwise_fwd(const double *x, const double *w, double *y, int64_t B,
                         int64_t T, int64_t D, int W, int H, int residual,
                         int act) {
  int64_t G = D / H;
  int64_t N = B * T;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    int64_t b = n / T, t = n % T;
    for (int64_t c = 0; c < D; ++c) {
      double s = conv_at(x, w, T, D, G, W, H, b, t, c);
      y[n * D + c] = act_fn(s, act) + (residual ? x[n * D + c] : 0.0);
    }
  }
}

/* Same forward, evaluated only at the listed token rows (n = b*T + t);
 * y_rows has shape (nrows, D). */
void oracle_headwise_fwd_rows(const double *x, const double *w, int64_t B,
                              int64_t T, int64_t D, int W, int H, int residual,
                              int act, int64_t nrows, const int64_t *rows,
                              double *y_rows) {
  int64_t G = D / H;
  (void)B;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t n = rows[i], b = n / T, t = n % T;
    for (int64_t c = 0; c < D; ++c) {
      double s = conv_at(x, w, T, D, G, W, H, b, t, c);
      y_rows[i * D + c] = act_fn(s, act) + (residual ? x[n * D + c] : 0.0);
    }
  }
}

/* ds[b,t,c] = dy[b,t,c] * act'(s[b,t,c]): gradient at the pre-activation. */
static double ds_at(const double *x, const double *w, const double *dy,
                    int64_t T, int64_t D, int64_t G, int W, int H, int act,
                    int64_t b, int64_t t, int64_t c) {
  double g = dy[IDX3(b, t, c, T, D)];
  if (!act) return g;
  return g * act_grad(conv_at(x, w, T, D, G, W, H, b, t, c), act);
}

/*
 * dx at one (b, tau, c): every output s[b,t,c] with t = tau + k (k < W,
 * t < T) used x[b,tau,c] with weight w[b,t,g(c),k]; the residual adds dy.
 */
static double dx_at(const double *x, const double *w, const double *dy,
                    int64_t T, int64_t D, int64_t G, int W, int H, int residual,
                    int act, int64_t b, int64_t tau, int64_t c) {
  int64_t g = c / H;
  double acc = 0.0;
  for (int k = 0; k < W; ++k) {
    int64_t t = tau + k;
    if (t >= T) break;
    double wk = w[IDX3(b, t, g, T, G) * W + k];
    acc += wk * ds_at(x, w, dy, T, D, G, W, H, act, b, t, c);
  }
  if (residual) acc += dy[IDX3(b, tau, c, T, D)];
  return acc;
}

/* dw at one (b, t, g, k): sum over the H channels of group g of
 * ds[b,t,c] * x[b,t-k,c]; zero when t-k < 0. */
static double dw_at(const double *x, const double *w, const double *dy,
                    int64_t T, int64_t D, int64_t G, int W, int H, int act,
                    int64_t b, int64_t t, int64_t g, int k) {
  if (t - k < 0) return 0.0;
  double acc = 0.0;
  for (int64_t c = g * H; c < (g + 1) * H; ++c)
    acc += ds_at(x, w, dy, T, D, G, W, H, act, b, t, c) *
           x[IDX3(b, t - k, c, T, D)];
  return acc;
}

/* Backward, head-wise tying: dx (B,T,D) and dw (B,T,G,W). */
void oracle_headwise_bwd(const double *x, const double *w, const double *dy,
                         double *dx, double *dw, int64_t B, int64_t T,
                         int64_t D, int W, int H, int residual, int act) {
  int64_t G = D / H;
  int64_t N = B * T;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    int64_t b = n / T, t = n % T;
    for (int64_t c = 0; c < D; ++c)
      dx[n * D + c] = dx_at(x, w, dy, T, D, G, W, H, residual, act, b, t, c);
    for (int64_t g = 0; g < G; ++g)
      for (int k = 0; k < W; ++k)
        dw[(n * G + g) * W + k] = dw_at(x, w, dy, T, D, G, W, H, act, b, t, g, k);
  }
}

/* Backward at the listed token rows: dx_rows (nrows, D), dw_rows (nrows, G, W). */
void oracle_headwise_bwd_rows(const double *x, const double *w,
                              const double *dy, int64_t B, int64_t T, int64_t D,
                              int W, int H, int residual, int act,
                              int64_t nrows, const int64_t *rows,
                              double *dx_rows, double *dw_rows) {
  int64_t G = D / H;
  (void)B;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t n = rows[i], b = n / T, t = n % T;
    for (int64_t c = 0; c < D; ++c)
      dx_rows[i * D + c] = dx_at(x, w, dy, T, D, G, W, H, residual, act, b, t, c);
    for (int64_t g = 0; g < G; ++g)
      for (int k = 0; k < W; ++k)
        dw_rows[(i * G + g) * W + k] =
            dw_at(x, w, dy, T, D, G, W, H, act, b, t, g, k);
  }
}

/*
 * Low-rank filter generation ([gist] Parametrisatie 1 and "Fused Low-Rank
 * Kernel"; [wisp] 2.): w[b,t,g,k] = sum_r z[b,t,r] * U[r, g*W + k].
 * Materialised here on purpose: the oracle is the plain definition.
 */
void oracle_lowrank_w(const double *z, const double *U, double *w, int64_t B,
                      int64_t T, int64_t G, int W, int R) {
  int64_t N = B * T, GW = G * W;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t col = 0; col < GW; ++col) {
      double acc = 0.0;
      for (int r = 0; r < R; ++r) acc += z[n * R + r] * U[(int64_t)r * GW + col];
      w[n * GW + col] = acc;
    }
}

/* Low-rank forward: w = zU, then the head-wise forward. */
void oracle_lowrank_fwd(const double *x, const double *z, const double *U,
                        double *y, int64_t B, int64_t T, int64_t D, int W,
                        int H, int R, int residual, int act) {
  int64_t G = D / H;
  double *w = (double *)malloc(sizeof(double) * (size_t)(B * T * G * W));
  if (!w) return;
  oracle_lowrank_w(z, U, w, B, T, G, W, R);
  oracle_headwise_fwd(x, w, y, B, T, D, W, H, residual, act);
  free(w);
}

/*
 * Low-rank backward.  With w = zU and dw the head-wise filter gradient:
 *   dz[b,t,r]    = sum_{g,k} dw[b,t,g,k] * U[r, g*W+k]
 *   dU[r, g*W+k] = sum_{b,t} z[b,t,r] * dw[b,t,g,k]
 * dw is materialised in this reference only.
 */
void oracle_lowrank_bwd(const double *x, const double *z, const double *U,
                        const double *dy, double *dx, double *dz, double *dU,
                        int64_t B, int64_t T, int64_t D, int W, int H, int R,
                        int residual, int act) {
  int64_t G = D / H, N = B * T, GW = G * W;
  double *w = (double *)malloc(sizeof(double) * (size_t)(N * GW));
  double *dw = (double *)malloc(sizeof(double) * (size_t)(N * GW));
  if (!w || !dw) { free(w); free(dw); return; }
  oracle_lowrank_w(z, U, w, B, T, G, W, R);
  oracle_headwise_bwd(x, w, dy, dx, dw, B, T, D, W, H, residual, act);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int r = 0; r < R; ++r) {
      double acc = 0.0;
      for (int64_t col = 0; col < GW; ++col)
        acc += dw[n * GW + col] * U[(int64_t)r * GW + col];
      dz[n * R + r] = acc;
    }
#pragma omp parallel for schedule(static)
  for (int64_t col = 0; col < GW; ++col)
    for (int r = 0; r < R; ++r) {
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) acc += z[n * R + r] * dw[n * GW + col];
      dU[(int64_t)r * GW + col] = acc;
    }
  free(w);
  free(dw);
}

/* w[b,t,g,:] for one token, from z and U. */
static void w_row(const double *z, const double *U, int64_t n, int64_t G, int W,
                  int R, double *out) {
  int64_t GW = G * W;
  for (int64_t col = 0; col < GW; ++col) {
    double acc = 0.0;
    for (int r = 0; r < R; ++r) acc += z[n * R + r] * U[(int64_t)r * GW + col];
    out[col] = acc;
  }
}

/*
 * Low-rank forward at listed token rows.  Only the filter rows that the listed
 * outputs read are generated (the token itself), so this scales to the full
 * benchmark shapes.
 */
void oracle_lowrank_fwd_rows(const double *x, const double *z, const double *U,
                             int64_t B, int64_t T, int64_t D, int W, int H,
                             int R, int residual, int act, int64_t nrows,
                             const int64_t *rows, double *y_rows) {
  int64_t G = D / H;
  (void)B;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t n = rows[i], t = n % T;
    double *wr = (double *)malloc(sizeof(double) * (size_t)(G * W));
    if (!wr) continue;
    w_row(z, U, n, G, W, R, wr);
    for (int64_t c = 0; c < D; ++c) {
      int64_t g = c / H;
      double s = 0.0;
      for (int k = 0; k < W; ++k) {
        if (t - k < 0) break;
        s += wr[g * W + k] * x[(n - k) * D + c];
      }
      y_rows[i * D + c] = act_fn(s, act) + (residual ? x[n * D + c] : 0.0);
    }
    free(wr);
  }
}

/*
 * Low-rank backward at listed token rows: dx_rows (nrows, D) and
 * dz_rows (nrows, R).  dx at tau needs filters and ds at tau..tau+W-1; dz at t
 * needs ds at t and x at t-W+1..t, which needs filters at t.
 */
void oracle_lowrank_bwd_rows(const double *x, const double *z, const double *U,
                             const double *dy, int64_t B, int64_t T, int64_t D,
                             int W, int H, int R, int residual, int act,
                             int64_t nrows, const int64_t *rows,
                             double *dx_rows, double *dz_rows) {
  int64_t G = D / H, GW = G * W;
  (void)B;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t n = rows[i], t = n % T;
    /* filters for tokens t .. t+W-1 of the same sequence */
    double *wr = (double *)malloc(sizeof(double) * (size_t)(W * GW));
    if (!wr) continue;
    for (int k = 0; k < W; ++k)
      if (t + k < T) w_row(z, U, n + k, G, W, R, wr + (int64_t)k * GW);
    /* ds at token t+j for channel c, from its own filter row j */
    for (int64_t c = 0; c < D; ++c) {
      int64_t g = c / H;
      double acc = 0.0;
      for (int k = 0; k < W; ++k) {
        int64_t tk = t + k;
        if (tk >= T) break;
        const double *wk = wr + (int64_t)k * GW + g * W;
        double s = 0.0;
        if (act)
          for (int kk = 0; kk < W; ++kk) {
            if (tk - kk < 0) break;
            s += wk[kk] * x[(n + k - kk) * D + c];
          }
        double ds = dy[(n + k) * D + c] * act_grad(s, act);
        acc += wk[k] * ds;
      }
      if (residual) acc += dy[n * D + c];
      dx_rows[i * D + c] = acc;
    }
    /* dz[t, r] = sum_{g,k} dw[t,g,k] U[r, gW+k] with dw from ds at t */
    for (int r = 0; r < R; ++r) dz_rows[i * R + r] = 0.0;
    for (int64_t g = 0; g < G; ++g)
      for (int k = 0; k < W; ++k) {
        if (t - k < 0) continue;
        double dwv = 0.0;
        for (int64_t c = g * H; c < (g + 1) * H; ++c) {
          double s = 0.0;
          if (act)
            for (int kk = 0; kk < W; ++kk) {
              if (t - kk < 0) break;
              s += wr[g * W + kk] * x[(n - kk) * D + c];
            }
          double ds = dy[n * D + c] * act_grad(s, act);
          dwv += ds * x[(n - k) * D + c];
        }
        for (int r = 0; r < R; ++r)
          dz_rows[i * R + r] += dwv * U[(int64_t)r * GW + g * W + k];
      }
    free(wr);
  }
}

/*
 * dU at listed columns col = g*W + k: sum over every token of
 * z[n, r] * dw[n, g, k]; dU_cols has shape (R, ncols).
 */
void oracle_lowrank_dU_cols(const double *x, const double *z, const double *U,
                            const double *dy, int64_t B, int64_t T, int64_t D,
                            int W, int H, int R, int act, int64_t ncols,
                            const int64_t *cols, double *dU_cols) {
  int64_t G = D / H, GW = G * W, N = B * T;
  (void)G;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < ncols; ++j) {
    int64_t col = cols[j], g = col / W;
    int k = (int)(col % W);
    double *acc = (double *)calloc((size_t)R, sizeof(double));
    double *wg = (double *)malloc(sizeof(double) * (size_t)W);
    if (!acc || !wg) { free(acc); free(wg); continue; }
    for (int64_t n = 0; n < N; ++n) {
      int64_t t = n % T;
      if (t - k < 0) continue;
      for (int kk = 0; kk < W; ++kk) {
        double a = 0.0;
        for (int r = 0; r < R; ++r) a += z[n * R + r] * U[(int64_t)r * GW + g * W + kk];
        wg[kk] = a;
      }
      double dwv = 0.0;
      for (int64_t c = g * H; c < (g + 1) * H; ++c) {
        double s = 0.0;
        if (act)
          for (int kk = 0; kk < W; ++kk) {
            if (t - kk < 0) break;
            s += wg[kk] * x[(n - kk) * D + c];
          }
        dwv += dy[n * D + c] * act_grad(s, act) * x[(n - k) * D + c];
      }
      for (int r = 0; r < R; ++r) acc[r] += z[n * R + r] * dwv;
    }
    for (int r = 0; r < R; ++r) dU_cols[(int64_t)r * ncols + j] = acc[r];
    free(acc);
    free(wg);
  }
}

/*
 * Streaming evaluation (one token at a time, for inference).  The pages define
 * the convolution over a whole sequence ([gist] Mechanisme) and leave inference
 * as open work ([wisp] Limitations).  The reading taken here: a step evaluates
 * the same causal sum at the newest position t, with the W-1 previous inputs
 * kept as a state
 *   state[b, j, c] = x[b, t-(W-1)+j, c],  j = 0 .. W-2 (oldest first),
 *                    zero for positions before the start of the sequence;
 *   y[b, c] = act(sum_{k<W} w[b, g(c), k] * x_{t-k}[b, c]) + rho * x_t[b, c],
 *   x_{t-0} = x_t,  x_{t-k} = state[b, W-1-k, c] for k >= 1;
 * afterwards the state drops its oldest row and appends x_t.
 * Layouts: x, y (B, D); w (B, G, W); state_in, state_out (B, W-1, D).
 */
void oracle_headwise_decode(const double *x, const double *w,
                            const double *state_in, double *state_out,
                            double *y, int64_t B, int64_t D, int W, int H,
                            int residual, int act) {
  int64_t G = D / H;
  int S = W - 1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t c = 0; c < D; ++c) {
      int64_t g = c / H;
      double s = w[(b * G + g) * W + 0] * x[b * D + c];
      for (int k = 1; k < W; ++k)
        s += w[(b * G + g) * W + k] * state_in[(b * S + (S - k)) * D + c];
      y[b * D + c] = act_fn(s, act) + (residual ? x[b * D + c] : 0.0);
      for (int j = 0; j + 1 < S; ++j)
        state_out[(b * S + j) * D + c] = state_in[(b * S + j + 1) * D + c];
      if (S > 0) state_out[(b * S + S - 1) * D + c] = x[b * D + c];
    }
  }
}

/* Low-rank step: w[b,g,k] = sum_r z[b,r] * U[r, g*W+k] ([gist] Parametrisatie
 * 1), then the head-wise step.  z (B, R), U (R, G*W). */
void oracle_lowrank_decode(const double *x, const double *z, const double *U,
                           const double *state_in, double *state_out,
                           double *y, int64_t B, int64_t D, int W, int H, int R,
                           int residual, int act) {
  int64_t G = D / H;
  double *w = (double *)malloc(sizeof(double) * (size_t)(B * G * W));
  if (!w) return;
  oracle_lowrank_w(z, U, w, B, 1, G, W, R);
  oracle_headwise_decode(x, w, state_in, state_out, y, B, D, W, H, residual, act);
  free(w);
}

/* State after a prompt x (B, T, D): its last W-1 rows, zero where the prompt
 * is shorter than W-1. */
void oracle_decode_state(const double *x, double *state, int64_t B, int64_t T,
                         int64_t D, int W) {
  int S = W - 1;
  for (int64_t b = 0; b < B; ++b)
    for (int j = 0; j < S; ++j) {
      int64_t t = T - S + j;
      for (int64_t c = 0; c < D; ++c)
        state[(b * S + j) * D + c] = t >= 0 ? x[IDX3(b, t, c, T, D)] : 0.0;
    }
}

/*
 * Static short convolution: the same causal sum with one fixed filter per
 * group for every sequence and position.  [wisp] Methodology > 1.
 * Mathematical Intuition writes it as y_t = sum_k w_k x_{t-k} beside the
 * dynamic form; [thread] describes it as a depthwise-separable causal
 * convolution of small width, and [gist] Prestaties names such kernels as the
 * latency yardstick for the dynamic ones.  Tying over H channels, zero taps
 * before the sequence start, residual and activation follow the dynamic path.
 * Layouts: x, y, dy, dx (B, T, D); w, dw (G, W).
 */
static double static_s(const double *x, const double *w, int64_t T, int64_t D,
                       int W, int H, int64_t b, int64_t t, int64_t c) {
  const double *wg = w + (c / H) * W;
  double s = 0.0;
  for (int k = 0; k < W && t - k >= 0; ++k) s += wg[k] * x[IDX3(b, t - k, c, T, D)];
  return s;
}

void oracle_static_fwd(const double *x, const double *w, double *y, int64_t B,
                       int64_t T, int64_t D, int W, int H, int residual, int act) {
  int64_t N = B * T;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    int64_t b = n / T, t = n % T;
    for (int64_t c = 0; c < D; ++c)
      y[n * D + c] = act_fn(static_s(x, w, T, D, W, H, b, t, c), act) +
                     (residual ? x[n * D + c] : 0.0);
  }
}

/*
 * Its derivative.  With ds = dy * act'(s):
 *   dx[b,tau,c] = sum_{k: tau+k<T} w[g(c),k] * ds[b,tau+k,c] + rho * dy[b,tau,c]
 *   dw[g,k]     = sum_b sum_{t>=k} sum_{c in g} ds[b,t,c] * x[b,t-k,c]
 * dw sums over every sequence and position, because the one filter serves them
 * all; each dw element is one sequential sum in the order (b, t, c).
 */
static double static_ds(const double *x, const double *w, const double *dy,
                        int64_t T, int64_t D, int W, int H, int act, int64_t b,
                        int64_t t, int64_t c) {
  double g = dy[IDX3(b, t, c, T, D)];
  return act ? g * act_grad(static_s(x, w, T, D, W, H, b, t, c), act) : g;
}

void oracle_static_bwd(const double *x, const double *w, const double *dy, double *dx,
                       double *dw, int64_t B, int64_t T, int64_t D, int W, int H,
                       int residual, int act) {
  int64_t G = D / H, N = B * T;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    int64_t b = n / T, tau = n % T;
    for (int64_t c = 0; c < D; ++c) {
      double acc = 0.0;
      for (int k = 0; k < W && tau + k < T; ++k)
        acc += w[(c / H) * W + k] * static_ds(x, w, dy, T, D, W, H, act, b, tau + k, c);
      dx[n * D + c] = acc + (residual ? dy[n * D + c] : 0.0);
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < G * W; ++j) {
    int64_t g = j / W;
    int k = (int)(j % W);
    double acc = 0.0;
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = k; t < T; ++t)
        for (int64_t c = g * H; c < (g + 1) * H; ++c)
          acc += static_ds(x, w, dy, T, D, W, H, act, b, t, c) * x[IDX3(b, t - k, c, T, D)];
    dw[j] = acc;
  }
}

/*
 * Packed variable-length sequences.  The pages train on whole rows; packing
 * several documents into one row (each starting fresh) is a training-side
 * convention they do not discuss.  The reading taken: pos[b,t] (int32) is
 * token t's index inside its document, 0 at a document start, and tap k of
 * token t exists only when k <= pos[b,t], so no tap reaches into the previous
 * document.  With pos[b,t] = t this is the dense operation above.  Masked taps
 * contribute nothing and receive zero gradient.
 * Layouts as above, plus pos (B, T).
 */
static double vl_s(const double *x, const double *w, const int32_t *pos, int64_t T,
                   int64_t D, int64_t G, int W, int H, int64_t n, int64_t c) {
  int64_t t = n % T, g = c / H;
  double s = 0.0;
  for (int k = 0; k < W; ++k)
    if (k <= pos[n] && t - k >= 0) s += w[(n * G + g) * W + k] * x[(n - k) * D + c];
  return s;
}

static double vl_ds(const double *x, const double *w, const int32_t *pos, const double *dy,
                    int64_t T, int64_t D, int64_t G, int W, int H, int act, int64_t n,
                    int64_t c) {
  double gy = dy[n * D + c];
  return act ? gy * act_grad(vl_s(x, w, pos, T, D, G, W, H, n, c), act) : gy;
}

void oracle_headwise_fwd_vl(const double *x, const double *w, const int32_t *pos, double *y,
                            int64_t B, int64_t T, int64_t D, int W, int H, int residual,
                            int act) {
  int64_t G = D / H, N = B * T;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t c = 0; c < D; ++c)
      y[n * D + c] = act_fn(vl_s(x, w, pos, T, D, G, W, H, n, c), act) +
                     (residual ? x[n * D + c] : 0.0);
}

/* dx[b,tau,c] = sum_{k : tau+k < T, k <= pos[b,tau+k]} w[b,tau+k,g,k] ds[b,tau+k,c]
 *               + rho dy[b,tau,c];
 * dw[b,t,g,k] = sum_{c in g} ds[b,t,c] x[b,t-k,c] when tap k of t exists, else 0. */
void oracle_headwise_bwd_vl(const double *x, const double *w, const int32_t *pos,
                            const double *dy, double *dx, double *dw, int64_t B, int64_t T,
                            int64_t D, int W, int H, int residual, int act) {
  int64_t G = D / H, N = B * T;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    int64_t tau = n % T;
    for (int64_t c = 0; c < D; ++c) {
      double acc = 0.0;
      for (int k = 0; k < W && tau + k < T; ++k) {
        int64_t m = n + k;
        if (k <= pos[m])
          acc += w[(m * G + c / H) * W + k] * vl_ds(x, w, pos, dy, T, D, G, W, H, act, m, c);
      }
      dx[n * D + c] = acc + (residual ? dy[n * D + c] : 0.0);
    }
    for (int64_t g = 0; g < G; ++g)
      for (int k = 0; k < W; ++k) {
        double acc = 0.0;
        if (k <= pos[n] && tau - k >= 0)
          for (int64_t c = g * H; c < (g + 1) * H; ++c)
            acc += vl_ds(x, w, pos, dy, T, D, G, W, H, act, n, c) * x[(n - k) * D + c];
        dw[(n * G + g) * W + k] = acc;
      }
  }
}

/* Low-rank forms: w = zU materialised, then the masked head-wise pass;
 * dz = dw U^T and dU = z^T dw with the masked dw. */
void oracle_lowrank_fwd_vl(const double *x, const double *z, const double *U,
                           const int32_t *pos, double *y, int64_t B, int64_t T, int64_t D,
                           int W, int H, int R, int residual, int act) {
  int64_t G = D / H;
  double *w = (double *)malloc(sizeof(double) * (size_t)(B * T * G * W));
  if (!w) return;
  oracle_lowrank_w(z, U, w, B, T, G, W, R);
  oracle_headwise_fwd_vl(x, w, pos, y, B, T, D, W, H, residual, act);
  free(w);
}

void oracle_lowrank_bwd_vl(const double *x, const double *z, const double *U,
                           const int32_t *pos, const double *dy, double *dx, double *dz,
                           double *dU, int64_t B, int64_t T, int64_t D, int W, int H, int R,
                           int residual, int act) {
  int64_t G = D / H, N = B * T, GW = G * W;
  double *w = (double *)malloc(sizeof(double) * (size_t)(N * GW));
  double *gw = (double *)malloc(sizeof(double) * (size_t)(N * GW));
  if (!w || !gw) { free(w); free(gw); return; }
  oracle_lowrank_w(z, U, w, B, T, G, W, R);
  oracle_headwise_bwd_vl(x, w, pos, dy, dx, gw, B, T, D, W, H, residual, act);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int r = 0; r < R; ++r) {
      double s = 0.0;
      for (int64_t j = 0; j < GW; ++j) s += gw[n * GW + j] * U[(int64_t)r * GW + j];
      dz[n * R + r] = s;
    }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < GW; ++j)
    for (int r = 0; r < R; ++r) {
      double s = 0.0;
      for (int64_t n = 0; n < N; ++n) s += z[n * R + r] * gw[n * GW + j];
      dU[(int64_t)r * GW + j] = s;
    }
  free(w);
  free(gw);
}

/*
 * Filter generation fused with the convolution (head-wise, forward).  The
 * filter of token t is a learned linear map of a hidden state ([gist]
 * Parametrisatie): w[b,t,:] = xh[b,t,:] M, with xh (B, T, Dh) and M (Dh, G*W)
 * (column g*W + k), and the convolution then runs as in oracle_headwise_fwd.
 * [wisp] Limitations names merging the convolution into the preceding matrix
 * product as the next step for inference; the oracle simply forms w first.
 */
void oracle_headwise_gen_fwd(const double *x, const double *xh, const double *M, double *y,
                             int64_t B, int64_t T, int64_t D, int64_t Dh, int W, int H,
                             int residual, int act) {
  int64_t G = D / H, GW = G * W, N = B * T;
  double *w = (double *)malloc(sizeof(double) * (size_t)(N * GW));
  if (!w) return;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < GW; ++j) {
      double a = 0.0;
      for (int64_t k = 0; k < Dh; ++k) a += xh[n * Dh + k] * M[k * GW + j];
      w[n * GW + j] = a;
    }
  oracle_headwise_fwd(x, w, y, B, T, D, W, H, residual, act);
  free(w);
}
