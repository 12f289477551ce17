/*
 * atlas_oracle.c -- fp64 CPU oracle for the ATLAS / Titans test-time memory.
 *
 * TEST INFRASTRUCTURE ONLY: the plain, slow, sequential reference the GPU
 * library is checked against.  It shares no code with the GPU library.
 *
 * The update is replayed exactly in the order the pages state it, with the
 * memory weights materialised after every token:
 *
 *   for each chunk of b tokens (ATLAS review, sec. 3.3 "Parallelizing Omega
 *   Rule"; Miras review, chunk-wise parallel training):
 *     theta_c <- current weights            (state at the end of the last chunk)
 *     for every token i whose window reaches into the chunk:
 *        G_i <- gradient of gamma_i * l(theta_c; phi(k_i), v_i)
 *     for every token n of the chunk, in order:
 *        g_n   = sum of G_i over the window i = n-c+1 .. n     (Omega rule,
 *                ATLAS review sec. 3.2; window truncated at the first token)
 *        S     = eta_n * S - theta_n * g_n                      (Titans review,
 *                sec. 3.1, momentum / "past surprise")
 *        W     = (1 - alpha_n) * W + S                          (Titans review,
 *                sec. 3.1, "Forgetting Mechanism")
 *        y_n   = f_W(phi(q_n))                                  (Titans review,
 *                sec. 3.1, "Retrieving a Memory")
 *
 * Memory forms (Titans review sec. 3.1 "Memory Architecture"; ATLAS review
 * sec. 2 "Deep Memory Module"): linear f(x) = M x, or the two-layer MLP
 * f(x) = [r +] W2 gelu(W1 x) with the exact erf GELU and no biases.
 * phi follows ATLAS review sec. 3.1 "Polynomial Feature Mapping".
 * Attentional biases (the loss of one token, e = f - v): squared error, the
 * dot product, and from the Miras review, "Alternative Attentional Biases",
 * the l_p loss |e|_p^p / p and the Huber loss with a threshold delta_t per
 * token (squared error while |e|_2 <= delta_t, else delta_t times the l1
 * error; the choice is made for the token as a whole).
 *
 * The per-token gradient is written out from the chain rule; its
 * factors are the per-token error and hidden activations.  No blocking,
 * fusion or reordering is applied beyond materialising each G_i once per chunk.
 */
#include "atlas_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

static int poly_block(int p) { return p + p * (p + 1) / 2; }

int oracle_feature_dim(const oracle_config* cfg) {
  switch (cfg->feature_map) {
    case ORC_PHI_ID: return cfg->d_k;
    case ORC_PHI_POLY2: return poly_block(cfg->d_k);
    case ORC_PHI_RAW_POLY2: return cfg->d_k + poly_block(cfg->poly_dims);
    default: return -1;
  }
}

long oracle_param_count(const oracle_config* cfg) {
  long D = oracle_feature_dim(cfg);
  if (cfg->memory == ORC_LINEAR) return (long)cfg->d_v * D;
  return (long)cfg->hidden * D * (cfg->gated ? 2 : 1) + (long)cfg->d_v * cfg->hidden;
}

/* [x_0..x_{p-1}, then x_a*x_b for a <= b in row-major upper-triangle order] */
static void poly2(const double* x, int p, double* out) {
  int o = 0;
  for (int a = 0; a < p; ++a) out[o++] = x[a];
  for (int a = 0; a < p; ++a)
    for (int b = a; b < p; ++b) out[o++] = x[a] * x[b];
}

void oracle_phi(const oracle_config* cfg, const double* x, double* out) {
  switch (cfg->feature_map) {
    case ORC_PHI_ID:
      memcpy(out, x, sizeof(double) * cfg->d_k);
      break;
    case ORC_PHI_POLY2:
      poly2(x, cfg->d_k, out);
      break;
    case ORC_PHI_RAW_POLY2:
      memcpy(out, x, sizeof(double) * cfg->d_k);
      poly2(x, cfg->poly_dims, out + cfg->d_k);
      break;
  }
}

static double gelu(double z) { return 0.5 * z * (1.0 + erf(z / sqrt(2.0))); }
/* d/dz of z * Phi(z) = Phi(z) + z * N(z; 0, 1) */
static double gelu_prime(double z) {
  const double pi = 3.14159265358979323846;
  return 0.5 * (1.0 + erf(z / sqrt(2.0))) + z * exp(-0.5 * z * z) / sqrt(2.0 * pi);
}

/* Layer norm of u (n entries) without gain or shift: nhat = (u - mean) / sd,
 * sd = sqrt(var + eps), var the biased variance.  Returns sd.              */
static double layer_norm(const double* u, int n, double eps, double* nhat) {
  double mean = 0.0, var = 0.0;
  for (int o = 0; o < n; ++o) mean += u[o];
  mean /= n;
  for (int o = 0; o < n; ++o) var += (u[o] - mean) * (u[o] - mean);
  var /= n;
  const double sd = sqrt(var + eps);
  for (int o = 0; o < n; ++o) nhat[o] = (u[o] - mean) / sd;
  return sd;
}

/* Forward pass; keeps the hidden pre-activation z when asked (MLP only),
 * and with layer norm the normalised branch nhat and its sd.               */
static void apply_ln(const oracle_config* cfg, const double* th, const double* x,
                     const double* r, double* y, double* z_keep, double* nhat_keep, double* sd_keep);
static void apply(const oracle_config* cfg, const double* th, const double* x,
                  const double* r, double* y, double* z_keep) {
  apply_ln(cfg, th, x, r, y, z_keep, NULL, NULL);
}
static void apply_ln(const oracle_config* cfg, const double* th, const double* x,
                     const double* r, double* y, double* z_keep, double* nhat_keep, double* sd_keep) {
  const int D = oracle_feature_dim(cfg), dv = cfg->d_v, h = cfg->hidden;
  if (cfg->memory == ORC_LINEAR) {
    for (int o = 0; o < dv; ++o) {
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += th[(long)o * D + d] * x[d];
      y[o] = s;
    }
    return;
  }
  /* gated: z keeps W1 x then W3 x (2h entries), a = gelu(W1 x) .* (W3 x) */
  const int gt = cfg->gated;
  const double* W1 = th;
  const double* W2 = th + (long)h * D;
  const double* W3 = W2 + (long)dv * h;
  double* z = z_keep ? z_keep : (double*)malloc(sizeof(double) * h * (gt ? 2 : 1));
  double* a = (double*)malloc(sizeof(double) * h);
  for (int j = 0; j < h; ++j) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += W1[(long)j * D + d] * x[d];
    z[j] = s;
    a[j] = gelu(s);
    if (gt) {
      double s3 = 0.0;
      for (int d = 0; d < D; ++d) s3 += W3[(long)j * D + d] * x[d];
      z[h + j] = s3;
      a[j] *= s3;
    }
  }
  for (int o = 0; o < dv; ++o) {
    double s = 0.0;
    for (int j = 0; j < h; ++j) s += W2[(long)o * h + j] * a[j];
    y[o] = s;   /* the branch u = W2 gelu(W1 x) */
  }
  if (cfg->layernorm) {
    double* nh = nhat_keep ? nhat_keep : (double*)malloc(sizeof(double) * dv);
    const double sd = layer_norm(y, dv, cfg->ln_eps, nh);
    for (int o = 0; o < dv; ++o) y[o] = nh[o];
    if (sd_keep) *sd_keep = sd;
    if (!nhat_keep) free(nh);
  }
  for (int o = 0; o < dv; ++o) y[o] += cfg->residual ? r[o] : 0.0;
  free(a);
  if (!z_keep) free(z);
}

void oracle_memory_apply(const oracle_config* cfg, const double* theta,
                         const double* x, const double* r, double* y) {
  apply(cfg, theta, x, r, y, NULL);
}

static double sgn(double x) { return x > 0.0 ? 1.0 : x < 0.0 ? -1.0 : 0.0; }

/* the sign factor of the l_p and Huber slopes: exact, or tanh(alpha e) */
static double sign_a(double e, double alpha) { return alpha > 0.0 ? tanh(alpha * e) : sgn(e); }

/* derivative of |e|^p / p: sign(e) |e|^(p-1)  (p >= 1; zero at e = 0) */
static double lp_slope(double e, double p, double alpha) {
  return e == 0.0 ? 0.0 : sign_a(e, alpha) * pow(fabs(e), p - 1.0);
}

/* Factors of one token's gradient at theta:
 *   linear: dY (d_v)            G = dY x^T
 *   MLP   : d1 (h), d2 (d_v), a (h)   G = { d1 x^T , d2 a^T }
 *   gated : d1 holds 2h entries, the second half d3 for W3: G = { d1 x^T,
 *           d2 a^T, d3 x^T } with back = W2^T d2, d1 = back .* gelu'(z1) .* z3,
 *           d3 = back .* gelu(z1), a = gelu(z1) .* z3
 * dY / d2 = dLoss/df (with layer norm: dLoss/du of the branch u, through
 * the LN Jacobian (g - mean(g) - nhat mean(g nhat)) / sd), with e = f - v:
 *   L2 -> s*gamma*e;  DOT -> -s*gamma*v;  LP -> s*gamma*sign(e)|e|^(p-1)
 *   (elementwise);  HUBER -> s*gamma*e while |e|_2 <= delta, else
 *   s*gamma*delta*sign(e): one choice for the whole token.                 */
static void grad_factors(const oracle_config* cfg, const double* th,
                         const double* x, const double* r, const double* v,
                         double gamma, double delta, double* d1, double* d2, double* a) {
  const int D = oracle_feature_dim(cfg), dv = cfg->d_v, h = cfg->hidden;
  const double s = cfg->grad_scale;
  double* f = (double*)malloc(sizeof(double) * dv);
  const int gt = cfg->memory == ORC_MLP && cfg->gated;
  double* z = cfg->memory == ORC_MLP ? (double*)malloc(sizeof(double) * h * (gt ? 2 : 1)) : NULL;
  const int ln = cfg->memory == ORC_MLP && cfg->layernorm;
  double* nh = ln ? (double*)malloc(sizeof(double) * dv) : NULL;
  double sd = 1.0;
  apply_ln(cfg, th, x, r, f, z, nh, &sd);
  int huber_small = 0;
  if (cfg->bias == ORC_BIAS_HUBER) {
    double n2 = 0.0;
    for (int o = 0; o < dv; ++o) n2 += (f[o] - v[o]) * (f[o] - v[o]);
    huber_small = sqrt(n2) <= delta;
  }
  for (int o = 0; o < dv; ++o) {
    if (cfg->bias == ORC_BIAS_L2) d2[o] = s * gamma * (f[o] - v[o]);
    else if (cfg->bias == ORC_BIAS_DOT) d2[o] = -s * gamma * v[o];
    else if (cfg->bias == ORC_BIAS_LP) d2[o] = s * gamma * lp_slope(f[o] - v[o], cfg->bias_p, cfg->sign_alpha);
    else d2[o] = s * gamma * (huber_small ? f[o] - v[o] : delta * sign_a(f[o] - v[o], cfg->sign_alpha));
  }
  if (ln) {
    double mg = 0.0, mgn = 0.0;
    for (int o = 0; o < dv; ++o) { mg += d2[o]; mgn += d2[o] * nh[o]; }
    mg /= dv;
    mgn /= dv;
    for (int o = 0; o < dv; ++o) d2[o] = (d2[o] - mg - nh[o] * mgn) / sd;
    free(nh);
  }
  if (cfg->memory == ORC_MLP) {
    const double* W2 = th + (long)h * D;
    for (int j = 0; j < h; ++j) {
      double back = 0.0;
      for (int o = 0; o < dv; ++o) back += W2[(long)o * h + j] * d2[o];
      d1[j] = back * gelu_prime(z[j]) * (gt ? z[h + j] : 1.0);
      a[j] = gelu(z[j]) * (gt ? z[h + j] : 1.0);
      if (gt) d1[h + j] = back * gelu(z[j]);
    }
    free(z);
  }
  free(f);
}

/* g += G(d1, d2, a, x), the outer-product form of one token's gradient,
 * restricted to the weight rows [r0, r1) of the row list W1 (h rows), W2 (d_v
 * rows), W3 (h rows), or M (d_v rows) for a linear memory.  Splitting the rows
 * between threads leaves every element's sum in the same order.            */
static long grad_rows(const oracle_config* cfg) {
  if (cfg->memory == ORC_LINEAR) return cfg->d_v;
  return (long)cfg->hidden * (cfg->gated ? 2 : 1) + cfg->d_v;
}

static void add_grad_rows(const oracle_config* cfg, const double* x, const double* d1,
                          const double* d2, const double* a, double* g, long r0, long r1) {
  const int D = oracle_feature_dim(cfg), dv = cfg->d_v, h = cfg->hidden;
  if (cfg->memory == ORC_LINEAR) {
    for (long o = r0; o < r1; ++o)
      for (int d = 0; d < D; ++d) g[o * D + d] += d2[o] * x[d];
    return;
  }
  double* gW2 = g + (long)h * D;
  double* gW3 = gW2 + (long)dv * h;
  for (long r = r0; r < r1; ++r) {
    if (r < h) {
      const long j = r;
      for (int d = 0; d < D; ++d) g[j * D + d] += d1[j] * x[d];
    } else if (r < h + dv) {
      const long o = r - h;
      for (int j = 0; j < h; ++j) gW2[o * h + j] += d2[o] * a[j];
    } else {
      const long j = r - h - dv;
      for (int d = 0; d < D; ++d) gW3[j * D + d] += d1[h + j] * x[d];
    }
  }
}

static void add_grad(const oracle_config* cfg, const double* x, const double* d1,
                     const double* d2, const double* a, double* g) {
  add_grad_rows(cfg, x, d1, d2, a, g, 0, grad_rows(cfg));
}

/* Threads that work inside one sequence (set per call by oracle_forward_ex
 * when there are fewer sequences than threads).                            */
static int g_inner_threads = 1;

void oracle_token_grad_ex(const oracle_config* cfg, const double* theta,
                          const double* x, const double* r, const double* v,
                          double gamma, double delta, double* grad) {
  const int dv = cfg->d_v, h = cfg->hidden > 0 ? cfg->hidden : 1;
  double* d1 = (double*)malloc(sizeof(double) * h * 2);
  double* d2 = (double*)malloc(sizeof(double) * dv);
  double* a = (double*)malloc(sizeof(double) * h);
  memset(grad, 0, sizeof(double) * oracle_param_count(cfg));
  grad_factors(cfg, theta, x, r, v, gamma, delta, d1, d2, a);
  add_grad(cfg, x, d1, d2, a, grad);
  free(d1); free(d2); free(a);
}

void oracle_token_grad(const oracle_config* cfg, const double* theta,
                       const double* x, const double* r, const double* v,
                       double gamma, double* grad) {
  oracle_token_grad_ex(cfg, theta, x, r, v, gamma, 0.0, grad);
}

/* Muon's orthogonalisation (K. Jordan et al., 2024): X = G / (|G|_F + 1e-7),
 * taken with fewer rows than columns (transposed if needed); then each step
 * X <- a X + (b A + c A A) X with A = X X^T, a, b, c = 3.4445, -4.7750,
 * 2.0315.  Plain triple loops; out is row-major rows x cols like G. */
void oracle_newton_schulz(const double* G, int rows, int cols, int steps, double* out) {
  const double a = 3.4445, b = -4.7750, c = 2.0315;
  const int tr = rows > cols;
  const int r = tr ? cols : rows, n = tr ? rows : cols;
  double* X = (double*)malloc(sizeof(double) * r * n);
  double* Y = (double*)malloc(sizeof(double) * r * n);
  double* A = (double*)malloc(sizeof(double) * r * r);
  double* B = (double*)malloc(sizeof(double) * r * r);
  double nrm = 0.0;
  for (long e = 0; e < (long)rows * cols; ++e) nrm += G[e] * G[e];
  nrm = sqrt(nrm) + 1e-7;
  for (int i = 0; i < rows; ++i)
    for (int j = 0; j < cols; ++j) {
      const double x = G[(long)i * cols + j] / nrm;
      if (tr) X[(long)j * n + i] = x;
      else X[(long)i * n + j] = x;
    }
  for (int s = 0; s < steps; ++s) {
    for (int i = 0; i < r; ++i)
      for (int j = 0; j < r; ++j) {
        double acc = 0.0;
        for (int l = 0; l < n; ++l) acc += X[(long)i * n + l] * X[(long)j * n + l];
        A[i * r + j] = acc;
      }
    for (int i = 0; i < r; ++i)
      for (int j = 0; j < r; ++j) {
        double acc = 0.0;
        for (int l = 0; l < r; ++l) acc += A[i * r + l] * A[l * r + j];
        B[i * r + j] = b * A[i * r + j] + c * acc;
      }
    for (int i = 0; i < r; ++i)
      for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int l = 0; l < r; ++l) acc += B[i * r + l] * X[(long)l * n + j];
        Y[(long)i * n + j] = a * X[(long)i * n + j] + acc;
      }
    memcpy(X, Y, sizeof(double) * r * n);
  }
  for (int i = 0; i < rows; ++i)
    for (int j = 0; j < cols; ++j)
      out[(long)i * cols + j] = tr ? X[(long)j * n + i] : X[(long)i * n + j];
  free(X); free(Y); free(A); free(B);
}

/* The weight matrices of the memory, in their order in theta. */
static int weight_matrices(const oracle_config* cfg, int rows[3], int cols[3]) {
  const int D = oracle_feature_dim(cfg);
  if (cfg->memory == ORC_LINEAR) { rows[0] = cfg->d_v; cols[0] = D; return 1; }
  rows[0] = cfg->hidden; cols[0] = D;
  rows[1] = cfg->d_v; cols[1] = cfg->hidden;
  if (!cfg->gated) return 2;
  rows[2] = cfg->hidden; cols[2] = D;
  return 3;
}

static int config_ok(const oracle_config* c) {
  if (c->n_seq < 0 || c->seq_len < 0 || c->d_k <= 0 || c->d_v <= 0) return 0;
  if (c->window < 1 || c->chunk < 1) return 0;
  if (oracle_feature_dim(c) <= 0) return 0;
  if (c->feature_map == ORC_PHI_RAW_POLY2 && (c->poly_dims < 1 || c->poly_dims > c->d_k)) return 0;
  if (c->memory == ORC_MLP) {
    if (c->hidden < 1) return 0;
    if (c->residual && c->d_k != c->d_v) return 0;
  } else if (c->memory != ORC_LINEAR) {
    return 0;
  }
  if (!(c->sign_alpha >= 0.0 && c->sign_alpha < 1e30)) return 0;
  if (c->layernorm && (c->memory != ORC_MLP || !(c->ln_eps > 0.0 && c->ln_eps < 1.0))) return 0;
  if (c->gated && c->memory != ORC_MLP) return 0;
  if (c->optimizer != ORC_OPT_GD && c->optimizer != ORC_OPT_MUON) return 0;
  if (c->optimizer == ORC_OPT_MUON && c->ns_steps < 1) return 0;
  if (c->bias == ORC_BIAS_LP) return c->bias_p >= 1.0 && c->bias_p < 1e6;
  return c->bias == ORC_BIAS_L2 || c->bias == ORC_BIAS_DOT || c->bias == ORC_BIAS_HUBER;
}

/* One sequence. */
static void run_sequence(const oracle_config* cfg, const double* q, const double* k,
                         const double* v, const double* al, const double* et,
                         const double* th, const double* ga, const double* dl, double* W, double* S,
                         double* hk, double* hv, double* hg, double* hd, int64_t* count,
                         double* out) {
  const int N = cfg->seq_len, dk = cfg->d_k, dv = cfg->d_v, c = cfg->window;
  const int b = cfg->chunk, h = cfg->hidden > 0 ? cfg->hidden : 1;
  const int D = oracle_feature_dim(cfg);
  const long P = oracle_param_count(cfg);
  const int halo = c - 1;
  const int huber = cfg->bias == ORC_BIAS_HUBER;
  /* tokens before this call that still exist (sequence start truncates) */
  const int halo_valid = (int)(*count < halo ? *count : halo);

  double* Wc = (double*)malloc(sizeof(double) * P);
  double* g = (double*)malloc(sizeof(double) * P);
  const int win = b + c - 1;
  double* X = (double*)malloc(sizeof(double) * win * D);
  const int h1 = cfg->gated ? 2 * h : h;   /* d1 (and d3) per window token */
  double* D1 = (double*)malloc(sizeof(double) * win * h1);
  double* D2 = (double*)malloc(sizeof(double) * win * dv);
  double* A = (double*)malloc(sizeof(double) * win * h);
  double* xq = (double*)malloc(sizeof(double) * D);
  double* Sloc = (double*)calloc(P, sizeof(double));
  double* O = cfg->optimizer == ORC_OPT_MUON ? (double*)malloc(sizeof(double) * P) : NULL;

  for (int t0 = 0; t0 < N; t0 += b) {
    const int te = (t0 + b < N ? t0 + b : N) - 1;
    memcpy(Wc, W, sizeof(double) * P);
    /* window tokens i in [lo, te], relative to the call start; i < 0 is halo */
    int lo = t0 - (c - 1);
    if (lo < -halo_valid) lo = -halo_valid;
    /* each window token's factors are independent of the others' */
#pragma omp parallel for num_threads(g_inner_threads) if (g_inner_threads > 1) schedule(dynamic, 1)
    for (int i = lo; i <= te; ++i) {
      const double *ki, *vi;
      double gi, di = 0.0;
      if (i >= 0) {
        ki = k + (long)i * dk; vi = v + (long)i * dv; gi = ga[i];
        if (huber) di = dl[i];
      } else {
        ki = hk + (long)(halo + i) * dk; vi = hv + (long)(halo + i) * dv; gi = hg[halo + i];
        if (huber) di = hd[halo + i];
      }
      const int w = i - lo;
      oracle_phi(cfg, ki, X + (long)w * D);
      grad_factors(cfg, Wc, X + (long)w * D, ki, vi, gi, di, D1 + (long)w * h1,
                   D2 + (long)w * dv, A + (long)w * h);
    }
    for (int n = t0; n <= te; ++n) {
      memset(g, 0, sizeof(double) * P);
      int i0 = n - c + 1;
      if (i0 < lo) i0 = lo;
      /* g_n = sum over the window, oldest token first; threads split the
         weight rows, each row summed in that same order */
      const long nrows = grad_rows(cfg);
#pragma omp parallel num_threads(g_inner_threads) if (g_inner_threads > 1)
      {
        long r0 = 0, r1 = nrows;
#ifdef _OPENMP
        const int nt = omp_get_num_threads(), it = omp_get_thread_num();
        r0 = nrows * it / nt;
        r1 = nrows * (it + 1) / nt;
#endif
        for (int i = i0; i <= n; ++i) {
          const int w = i - lo;
          add_grad_rows(cfg, X + (long)w * D, D1 + (long)w * h1, D2 + (long)w * dv,
                        A + (long)w * h, g, r0, r1);
        }
      }
      const double eta_n = cfg->momentum ? et[n] : 0.0;
      double* Sx = cfg->momentum ? S : Sloc;
      if (cfg->optimizer == ORC_OPT_MUON) {
        for (long p = 0; p < P; ++p) Sx[p] = eta_n * Sx[p] + g[p];
        int rows[3], cols[3];
        const int nm = weight_matrices(cfg, rows, cols);
        long off = 0;
        for (int m = 0; m < nm; ++m) {
          oracle_newton_schulz(Sx + off, rows[m], cols[m], cfg->ns_steps, O + off);
          off += (long)rows[m] * cols[m];
        }
        for (long p = 0; p < P; ++p) W[p] = (1.0 - al[n]) * W[p] - th[n] * O[p];
      } else {
#pragma omp parallel for num_threads(g_inner_threads) if (g_inner_threads > 1) schedule(static)
        for (long p = 0; p < P; ++p) {
          Sx[p] = eta_n * Sx[p] - th[n] * g[p];
          W[p] = (1.0 - al[n]) * W[p] + Sx[p];
        }
      }
      oracle_phi(cfg, q + (long)n * dk, xq);
      apply(cfg, W, xq, q + (long)n * dk, out + (long)n * dv, NULL);
    }
  }

  /* new halo: the last c-1 tokens of (old halo ++ this call) */
  if (halo > 0) {
    double* nk = (double*)malloc(sizeof(double) * halo * dk);
    double* nv = (double*)malloc(sizeof(double) * halo * dv);
    double* ng = (double*)malloc(sizeof(double) * halo);
    double* nd = (double*)malloc(sizeof(double) * halo);
    for (int j = 0; j < halo; ++j) {
      const int i = N - halo + j;
      if (i >= 0) {
        memcpy(nk + (long)j * dk, k + (long)i * dk, sizeof(double) * dk);
        memcpy(nv + (long)j * dv, v + (long)i * dv, sizeof(double) * dv);
        ng[j] = ga[i];
        nd[j] = huber ? dl[i] : 0.0;
      } else {
        memcpy(nk + (long)j * dk, hk + (long)(halo + i) * dk, sizeof(double) * dk);
        memcpy(nv + (long)j * dv, hv + (long)(halo + i) * dv, sizeof(double) * dv);
        ng[j] = hg[halo + i];
        nd[j] = huber ? hd[halo + i] : 0.0;
      }
    }
    memcpy(hk, nk, sizeof(double) * halo * dk);
    memcpy(hv, nv, sizeof(double) * halo * dv);
    memcpy(hg, ng, sizeof(double) * halo);
    if (huber) memcpy(hd, nd, sizeof(double) * halo);
    free(nk); free(nv); free(ng); free(nd);
  }
  *count += N;

  free(Wc); free(g); free(X); free(D1); free(D2); free(A); free(xq); free(Sloc); free(O);
}

int oracle_forward_ex(const oracle_config* cfg,
                      const double* q, const double* k, const double* v,
                      const double* alpha, const double* eta,
                      const double* theta, const double* gamma, const double* delta,
                      double* mem, double* mom,
                      double* halo_k, double* halo_v, double* halo_g, double* halo_d,
                      int64_t* count, double* out) {
  if (!config_ok(cfg)) return -1;
  if (cfg->bias == ORC_BIAS_HUBER && (!delta || (cfg->window > 1 && !halo_d))) return -1;
  const long N = cfg->seq_len, dk = cfg->d_k, dv = cfg->d_v, halo = cfg->window - 1;
  const long P = oracle_param_count(cfg);
  int threads = 1;
  g_inner_threads = 1;
#ifdef _OPENMP
  /* Fewer sequences than threads and large per-token window sums: the
     sequences run one after another, each with every thread splitting the
     weight rows of its window sums and updates.                          */
  const int avail = omp_get_max_threads();
  if (cfg->n_seq < avail && (double)P * cfg->window >= 1.0e6) g_inner_threads = avail;
#endif
  if (g_inner_threads > 1) {
    for (int s = 0; s < cfg->n_seq; ++s)
      run_sequence(cfg, q + s * N * dk, k + s * N * dk, v + s * N * dv,
                   alpha + s * N, eta + s * N, theta + s * N, gamma + s * N,
                   delta ? delta + s * N : NULL,
                   mem + s * P, mom + s * P,
                   halo_k + s * halo * dk, halo_v + s * halo * dv, halo_g + s * halo,
                   halo_d ? halo_d + s * halo : NULL,
                   count + s, out + s * N * dv);
    return g_inner_threads;
  }
#pragma omp parallel
  {
#ifdef _OPENMP
#pragma omp single
    threads = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
    for (int s = 0; s < cfg->n_seq; ++s) {
      run_sequence(cfg, q + s * N * dk, k + s * N * dk, v + s * N * dv,
                   alpha + s * N, eta + s * N, theta + s * N, gamma + s * N,
                   delta ? delta + s * N : NULL,
                   mem + s * P, mom + s * P,
                   halo_k + s * halo * dk, halo_v + s * halo * dv, halo_g + s * halo,
                   halo_d ? halo_d + s * halo : NULL,
                   count + s, out + s * N * dv);
    }
  }
  return threads;
}

int oracle_forward(const oracle_config* cfg,
                   const double* q, const double* k, const double* v,
                   const double* alpha, const double* eta,
                   const double* theta, const double* gamma,
                   double* mem, double* mom,
                   double* halo_k, double* halo_v, double* halo_g,
                   int64_t* count, double* out) {
  if (cfg->bias == ORC_BIAS_HUBER) return -1;   /* needs the thresholds */
  return oracle_forward_ex(cfg, q, k, v, alpha, eta, theta, gamma, NULL, mem, mom,
                           halo_k, halo_v, halo_g, NULL, count, out);
}
