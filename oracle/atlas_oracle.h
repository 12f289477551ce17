/*
 * atlas_oracle.h -- fp64 CPU oracle for the ATLAS / Titans test-time memory.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and atlas_oracle.c are the slow,
 * sequential reference that the GPU library is checked against.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no code, header, constant or helper with the GPU
 * library, and nothing in the library may include or link it.
 *
 * What it computes (per sequence, tokens processed in the order given):
 *   - feature map phi on keys and queries (ATLAS review, section 3.1,
 *     "Polynomial Feature Mapping": all monomials up to degree p; here p<=2,
 *     raw monomials, each unordered pair once, diagonal included);
 *   - the Omega-rule inner loss over the last c tokens,
 *     sum_i gamma_i * l(M; phi(k_i), v_i)  (ATLAS review, section 3.2,
 *     "Sliding window recurrent model" / "Omega Rule");
 *   - chunked gradients: every gradient in a chunk of b tokens is taken at
 *     the memory state left by the previous chunk (ATLAS review, section
 *     3.3 "Parallelizing Omega Rule"; Miras review, "Training"/parallelism);
 *   - Titans momentum S_t = eta_t S_{t-1} - theta_t grad and decay
 *     M_t = (1 - alpha_t) M_{t-1} + S_t (Titans review, section 3.1,
 *     "Learning Process and Surprise Metric" and "Forgetting Mechanism");
 *   - retrieval y_t = M_t(phi(q_t)), a plain forward pass with the memory
 *     after token t's update (Titans review, section 3.1 "Retrieving a
 *     Memory").
 *
 * Memory optimizer Muon (ATLAS summary, section 5, "Memory Optimization": Muon
 * takes the place of plain gradient descent on the memory).  Read as the
 * published Muon optimizer (K. Jordan et al., 2024, "Muon: An optimizer for
 * hidden layers in neural networks"), with the memory's gates in its roles:
 * momentum of the raw window gradients S_t = eta_t S_{t-1} + grad, each
 * weight matrix's S_t orthogonalised by the quintic Newton-Schulz iteration
 * of that optimizer (Frobenius normalisation with eps 1e-7, then ns_steps
 * steps X <- a X + (b A + c A^2) X, A = X X^T, on the orientation with fewer
 * rows; a, b, c = 3.4445, -4.7750, 2.0315), and the step
 * M_t = (1 - alpha_t) M_{t-1} - theta_t NS(S_t).  The learning rate theta
 * scales the orthogonalised step because NS is invariant to the scale of
 * its input.
 *
 * Attentional biases besides the squared error (Miras review, "Alternative
 * Attentional Biases"): the l_p loss, and the Huber loss whose threshold
 * delta_t is an input per token and which picks, per token, the squared
 * error or delta_t times the absolute (l1) error.
 *
 * Parity unpinned: the combination MLP memory + window c > 1 + chunk b > 1 +
 * momentum is fixed by no closed form on the pages; it is pinned only through
 * the special cases that reduce to one (see tests/test_oracle_pins.py).
 */
#ifndef ATLAS_ORACLE_H
#define ATLAS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_LINEAR = 0, ORC_MLP = 1 };
enum { ORC_PHI_ID = 0, ORC_PHI_POLY2 = 1, ORC_PHI_RAW_POLY2 = 2 };
enum { ORC_BIAS_L2 = 0, ORC_BIAS_DOT = 1, ORC_BIAS_LP = 2, ORC_BIAS_HUBER = 3 };
enum { ORC_OPT_GD = 0, ORC_OPT_MUON = 1 };

typedef struct {
  int n_seq;        /* independent sequences (batch * heads)                 */
  int seq_len;      /* tokens per sequence in this call                       */
  int d_k, d_v;     /* raw key/query width, value width                       */
  int memory;       /* ORC_LINEAR: y = M x; ORC_MLP: y = [r] + W2 gelu(W1 x)  */
  int hidden;       /* MLP hidden width                                       */
  int residual;     /* MLP only: add the raw key/query r (needs d_k == d_v)   */
  int feature_map;  /* ORC_PHI_*                                              */
  int poly_dims;    /* p: leading dims fed to the degree-2 map                */
  int window;       /* c >= 1                                                 */
  int chunk;        /* b >= 1                                                 */
  int momentum;     /* 0: eta treated as 0 and S not carried                  */
  int bias;         /* attentional bias of one token (e = f - v), times s*gamma:
                       ORC_BIAS_L2   : |e|_2^2 / 2
                       ORC_BIAS_DOT  : -<f, v>
                       ORC_BIAS_LP   : sum_o |e_o|^p / p
                       ORC_BIAS_HUBER: |e|_2^2 / 2 if |e|_2 <= delta, else
                                       delta * (|e|_1 - delta / 2)          */
  double grad_scale;/* s                                                      */
  double bias_p;    /* p >= 1 of ORC_BIAS_LP                                  */
  double sign_alpha;/* 0: sign(e) exact in the l_p and Huber slopes; > 0:
                       tanh(sign_alpha * e), the smooth sign of the Miras
                       review (Remark 5 under "Alternative Attentional
                       Biases")                                              */
  int layernorm;    /* MLP only: f(x) = [r +] LN(W2 gelu(W1 x)), LN over the
                       d_v outputs without gain or shift (Miras review, the
                       memory of its three models)                           */
  double ln_eps;    /* LN: (u - mean) / sqrt(var + ln_eps)                    */
  int gated;        /* MLP only: the gated memory of three matrices,
                       f(x) = [r +] W2 (gelu(W1 x) .* (W3 x)) (ATLAS summary,
                       Atlas++); weights W1 [h][D], W2 [d_v][h], W3 [h][D]    */
  int optimizer;    /* ORC_OPT_GD: S = eta S - theta g, M = (1-alpha) M + S;
                       ORC_OPT_MUON: S = eta S + g, M = (1-alpha) M - theta NS(S),
                       NS per weight matrix                                    */
  int ns_steps;     /* Muon: Newton-Schulz steps (>= 1)                       */
} oracle_config;

/* Sets the OpenMP thread count used by oracle_forward (n <= 0: default). */
void oracle_set_threads(int n);

/* Width D of phi(x). */
int oracle_feature_dim(const oracle_config* cfg);
/* Number of memory weights P (linear: d_v*D; MLP: hidden*D + d_v*hidden). */
long oracle_param_count(const oracle_config* cfg);

/* phi(x): x has d_k entries, out receives D entries. */
void oracle_phi(const oracle_config* cfg, const double* x, double* out);

/* Memory read f_theta(x, r) for one token; theta laid out as in
 * oracle_forward.  x = phi(key or query) (D), r = raw key or query (d_k). */
void oracle_memory_apply(const oracle_config* cfg, const double* theta,
                         const double* x, const double* r, double* y);

/* Gradient of ONE token's weighted inner loss at theta, written into grad
 * (P entries, same layout as theta):
 *   L2 : gamma * s/2 * |f_theta(x, r) - v|^2
 *   DOT: -gamma * s * <f_theta(x, r), v>                                   */
void oracle_token_grad(const oracle_config* cfg, const double* theta,
                       const double* x, const double* r, const double* v,
                       double gamma, double* grad);
/* The same with the token's Huber threshold delta (ORC_BIAS_HUBER).       */
void oracle_token_grad_ex(const oracle_config* cfg, const double* theta,
                          const double* x, const double* r, const double* v,
                          double gamma, double delta, double* grad);

/* Run the memory over one call's tokens for every sequence.
 *   q, k   [n_seq][seq_len][d_k]     v [n_seq][seq_len][d_v]
 *   alpha, eta, theta, gamma         [n_seq][seq_len]
 *   mem    [n_seq][P]  in: M_0 / theta_0, out: final weights
 *          linear: M [d_v][D];  MLP: W1 [hidden][D] then W2 [d_v][hidden]
 *   mom    [n_seq][P]  in/out momentum S (ignored when momentum == 0)
 *   halo_k [n_seq][c-1][d_k], halo_v [n_seq][c-1][d_v], halo_g [n_seq][c-1]
 *          in/out: the last c-1 tokens seen before this call, oldest first
 *   count  [n_seq]     in/out: tokens seen before this call
 *   out    [n_seq][seq_len][d_v]
 * Chunks start at the call's first token.  Returns the number of OpenMP
 * threads used, or a negative value on a bad configuration.               */
int oracle_forward(const oracle_config* cfg,
                   const double* q, const double* k, const double* v,
                   const double* alpha, const double* eta,
                   const double* theta, const double* gamma,
                   double* mem, double* mom,
                   double* halo_k, double* halo_v, double* halo_g,
                   int64_t* count, double* out);
/* The same with the per-token Huber thresholds delta [n_seq][seq_len] and
 * their halo halo_d [n_seq][c-1] (in/out), both used only by
 * ORC_BIAS_HUBER (which oracle_forward rejects); NULL otherwise.          */
int oracle_forward_ex(const oracle_config* cfg,
                      const double* q, const double* k, const double* v,
                      const double* alpha, const double* eta,
                      const double* theta, const double* gamma, const double* delta,
                      double* mem, double* mom,
                      double* halo_k, double* halo_v, double* halo_g, double* halo_d,
                      int64_t* count, double* out);

/* Muon's Newton-Schulz orthogonalisation of one rows x cols matrix G
 * (row-major) into out; steps >= 0 (0: the normalised input). */
void oracle_newton_schulz(const double* G, int rows, int cols, int steps, double* out);

#ifdef __cplusplus
}
#endif
#endif
