/*
 * atlas_mem.h -- C ABI of the MI355X test-time memory (ATLAS / Titans
 * long-term memory): chunked Omega-rule update with Titans momentum and
 * decay, and retrieval from the updated memory.
 *
 * The operation (for every sequence s = (batch, head), tokens t in order):
 *
 *   x_t   = phi(k_t)      feature map: identity, [k, upper-tri(k k^T)], or
 *                         [k, poly2(k[:p])]            (ATLAS review, sec. 3.1
 *                         "Polynomial Feature Mapping"; raw monomials, each
 *                         unordered pair once, diagonal included)
 *   f(x)  = M x           (linear memory)   or   r + W2 gelu(W1 x)  (2-layer
 *                         MLP memory, exact erf GELU, no biases, r the raw
 *                         key/query; Titans review sec. 3.1 "Memory
 *                         Architecture", ATLAS review sec. 2), optionally
 *                         r + LN(W2 gelu(W1 x)) with a layer norm over the
 *                         d_v outputs, without gain or shift (Miras review,
 *                         the memory of its three models), or the gated
 *                         memory r + W2 (gelu(W1 x) .* (W3 x)) (ATLAS
 *                         summary, Atlas++)
 *   loss  = sum over the last c tokens i of gamma_i * s * l(f(x_i) - v_i)
 *                         (Omega rule, ATLAS review sec. 3.2) with the
 *                         attentional bias l(e) = |e|^2 / 2, or the
 *                         dot-product bias -gamma_i * s * <f(x_i), v_i>, or
 *                         (Miras review, "Alternative Attentional Biases")
 *                         l(e) = sum_o |e_o|^p / p, or the Huber loss with a
 *                         threshold delta_i per token: |e|_2^2 / 2 while
 *                         |e|_2 <= delta_i, else delta_i (|e|_1 - delta_i / 2)
 *   chunks of b tokens:   every gradient of a chunk is taken at the weights
 *                         the previous chunk left (ATLAS review sec. 3.3
 *                         "Parallelizing Omega Rule")
 *   S_t   = eta_t S_{t-1} - theta_t grad_t   (Titans review sec. 3.1,
 *                         momentum / "past surprise")
 *   M_t   = (1 - alpha_t) M_{t-1} + S_t      (Titans review sec. 3.1,
 *                         "Forgetting Mechanism")
 *   y_t   = f_{M_t}(phi(q_t))                 (Titans review sec. 3.1
 *                         "Retrieving a Memory": a forward pass, no update)
 *
 * With the Muon memory optimizer (ATLAS summary sec. 5, "Memory Optimization":
 * Muon in place of plain gradient descent on the memory; per-sequence family,
 * plain linear or 2-layer MLP memory) the two middle lines become
 *   S_t   = eta_t S_{t-1} + grad_t
 *   M_t   = (1 - alpha_t) M_{t-1} - theta_t NS(S_t)
 * per weight matrix, NS the quintic Newton-Schulz orthogonalisation of the
 * published Muon optimizer (K. Jordan et al., 2024): X = S / (|S|_F + 1e-7)
 * on the orientation with fewer rows, then ns_steps times
 * X <- a X + (b A + c A A) X, A = X X^T, (a, b, c) = (3.4445, -4.7750, 2.0315).
 * The gradients keep the chunked semantics (taken at the chunk-start weights);
 * NS runs for every token, in fp32.
 *
 * where grad_t = sum_{i = t-c+1}^{t} grad of token i's term.  The window
 * stops at the first token the sequence has seen.
 *
 * Every function returns an atlas_status (0 = success).  Nothing is thrown
 * across the ABI and nothing aborts.  All device pointers are plain HIP
 * device addresses owned by the caller; the library owns only its handle and
 * the workspace it allocates in atlas_mem_init.
 */
#ifndef ATLAS_MEM_H
#define ATLAS_MEM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATLAS_OK = 0,
  ATLAS_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, aliasing   */
  ATLAS_ERR_UNSUPPORTED = 2,      /* valid config with no kernel built for it      */
  ATLAS_ERR_OUT_OF_MEMORY = 3,    /* workspace allocation failed                   */
  ATLAS_ERR_HIP = 4,              /* a HIP call failed; see atlas_mem_last_hip_error */
  ATLAS_ERR_SCRATCH_TOO_SMALL = 5 /* atlas_mem_forward_noalloc: the call needs more
                                     workspace than the static scratch buffer     */
} atlas_status;

enum { ATLAS_MEM_LINEAR = 0, ATLAS_MEM_MLP = 1 };
enum { ATLAS_PHI_IDENTITY = 0, ATLAS_PHI_POLY2 = 1, ATLAS_PHI_RAW_POLY2 = 2 };
enum { ATLAS_BIAS_L2 = 0, ATLAS_BIAS_DOT = 1, ATLAS_BIAS_LP = 2, ATLAS_BIAS_HUBER = 3 };
enum { ATLAS_BF16 = 0, ATLAS_F32 = 1 };
enum { ATLAS_OPT_GD = 0, ATLAS_OPT_MUON = 1 };
/* Kernel family.  PER_SEQUENCE: one workgroup per sequence, every operand
 * image kept in a global workspace (all memories and feature maps).
 * SHARDED: the hidden units of each sequence split over several workgroups
 * of one XCD, weights resident in registers.  STREAMED: one workgroup per
 * sequence (or a pair of workgroups of one XCD, each with half of the hidden
 * units), the fp32 weights and momentum read and written once per chunk in
 * one fused pass.  SHARDED and STREAMED serve the MLP memory with the
 * identity feature map, d_k == d_v and bf16 io (SHARDED: the l2 and
 * dot-product biases and no layer norm).  GROUPED: phi of every key and
 * query computed once per call into the workspace, the state resident in
 * registers; for the MLP memory the hidden units of each sequence split over
 * a group of workgroups of one XCD (16 per workgroup), for the linear memory
 * one workgroup per sequence runs the chunk chain and the retrieval of every
 * chunk runs afterwards, all chunks at once.  It serves the shapes of its
 * compiled table with the l2 or dot-product bias, bf16 io, chunk 64,
 * c <= 64, no layer norm, no gated memory, gradient descent.  AUTO picks
 * the fastest family measured
 * for the shape: STREAMED where marked so (large hidden layers), else
 * SHARDED, else STREAMED, else GROUPED, else PER_SEQUENCE.                 */
enum { ATLAS_KERNEL_AUTO = 0, ATLAS_KERNEL_PER_SEQUENCE = 1, ATLAS_KERNEL_SHARDED = 2, ATLAS_KERNEL_STREAMED = 3,
       ATLAS_KERNEL_GROUPED = 4 };

typedef struct {
  int batch, heads;   /* B, H: B*H independent sequences                        */
  int seq_len;        /* N: tokens per sequence in every forward call (>= 0)    */
  int d_k, d_v;       /* raw key/query width, value width                       */
  int memory;         /* ATLAS_MEM_LINEAR | ATLAS_MEM_MLP                       */
  int mlp_layers;     /* MLP depth L_M; 2 is the only depth built               */
  int mlp_hidden;     /* MLP hidden width h                                     */
  int mlp_residual;   /* 1: f(x) = r + W2 gelu(W1 x); needs d_k == d_v          */
  int feature_map;    /* ATLAS_PHI_*                                            */
  int poly_dims;      /* p for ATLAS_PHI_RAW_POLY2 (leading key dims)           */
  int window;         /* c >= 1, c <= chunk                                     */
  int chunk;          /* b                                                      */
  int momentum;       /* 0: eta is ignored (treated as 0) and S is not stored   */
  int bias;           /* ATLAS_BIAS_L2 | _DOT | _LP | _HUBER                    */
  int io_dtype;       /* ATLAS_BF16 | ATLAS_F32 for q, k, v, out                */
  float grad_scale;   /* s: 1 matches the printed update rules; 2 is the
                         literal derivative of the squared norm                 */
  int kernel;         /* ATLAS_KERNEL_*                                         */
  float bias_p;       /* p >= 1 of ATLAS_BIAS_LP (ignored otherwise)            */
  float sign_alpha;   /* sign(e) in the l_p and Huber slopes: 0 exact; > 0
                         tanh(sign_alpha * e), the smooth sign of the Miras
                         review (Remark 5 under "Alternative Attentional
                         Biases"), which keeps the result continuous in e    */
  int mlp_layernorm;  /* MLP only, 1: f(x) = r + LN(W2 gelu(W1 x))               */
  float ln_eps;       /* LN: (u - mean) / sqrt(var + ln_eps), 0 < ln_eps < 1    */
  int mlp_gated;      /* MLP only, 1: gated memory of three matrices (weights
                         W1 [h][D], W2 [d_v][h], W3 [h][D]); per-sequence
                         family only                                          */
  int optimizer;      /* ATLAS_OPT_GD (momentum + decay, above) or
                         ATLAS_OPT_MUON (per-sequence family; no layer norm,
                         no gated memory; the momentum slot of the state holds
                         S_t = eta S + grad when momentum is on)              */
  int ns_steps;       /* Muon: Newton-Schulz steps, 1..64 (ignored for GD)   */
} atlas_mem_config;

typedef struct atlas_mem_s* atlas_mem_t;

/* Byte offsets inside ONE sequence's state block, and the block stride.
 * The state buffer is [batch*heads] blocks of seq_stride bytes, sequence
 * index s = b*heads + h, 256-byte aligned.  Inside a block:
 *   weights  fp32  linear: M [d_v][D];  MLP: W1 [h][D] then W2 [d_v][h] (row-major),
 *                  then W3 [h][D] for the gated memory
 *   momentum fp32  same shape as weights (only if momentum)
 *   halo_k   fp32  [c-1][d_k]  raw keys of the last c-1 tokens seen, oldest first
 *   halo_v   fp32  [c-1][d_v]
 *   halo_g   fp32  [c-1]       their gamma
 *   halo_d   fp32  [c-1]       their Huber threshold (ATLAS_BIAS_HUBER only)
 *   count    int64             tokens seen so far
 * The caller writes the initial weights, zeroes everything else, and reads
 * the final weights/momentum back.  D is the width of phi(k).              */
typedef struct {
  size_t seq_stride;
  size_t weights, momentum, halo_k, halo_v, halo_g, count;
  int feature_dim;    /* D */
  long param_count;   /* P: number of weights (floats) */
  size_t halo_d;      /* equal to count when the bias has no threshold */
} atlas_mem_state_layout;

/* Validates cfg, selects the kernels and allocates the device workspace on
 * the current HIP device.  No kernel is launched.  cfg describes one memory
 * per (batch, head) sequence: its form (Titans review sec. 3.1, "Memory
 * Architecture"), the feature map (ATLAS review sec. 3.1), the window c of
 * the Omega rule (ATLAS review sec. 3.2), the chunk b (ATLAS review sec. 3.3)
 * and the attentional bias (Miras review, "Alternative Attentional Biases").
 * On success *out holds a handle that must be released with atlas_mem_free.
 * Errors: INVALID_ARGUMENT (bad or inconsistent sizes, null out),
 * UNSUPPORTED (no kernel for this shape: see atlas_mem_supported),
 * OUT_OF_MEMORY, HIP.                                                      */
atlas_status atlas_mem_init(const atlas_mem_config* cfg, atlas_mem_t* out);

/* Same validation as atlas_mem_init without allocating anything:
 * ATLAS_OK if a kernel exists for cfg.                                     */
atlas_status atlas_mem_supported(const atlas_mem_config* cfg);

/* Size in bytes of the state buffer (all sequences) and its layout.        */
size_t atlas_mem_state_bytes(atlas_mem_t h);
atlas_status atlas_mem_state_layout_of(atlas_mem_t h, atlas_mem_state_layout* out);

/* Runs one call over seq_len tokens of every sequence, enqueued on `stream`
 * (no host synchronisation, no allocation): the chunked update of the
 * memory and the per-token retrieval defined at the top of this file (ATLAS
 * review sec. 3.3 "Parallelizing Omega Rule"; Titans review sec. 3.2 "How to
 * Parallelize the Long-term Memory Training").  stream is a hipStream_t
 * passed as void*, so that this header needs no HIP header (NULL: the
 * default stream).  Chunks start at the call's
 * first token, so a call split in two equals one call when the first part's
 * length is a multiple of the chunk.
 *   q, k   [B][H][N][d_k]   io_dtype, contiguous
 *   v      [B][H][N][d_v]   io_dtype
 *   alpha, eta, theta, gamma  [B][H][N] fp32 (eta may be NULL if !momentum)
 *   state  in/out, layout above (device)
 *   out    [B][H][N][d_v]   io_dtype, must not overlap any input or state
 * All pointers are device pointers, 16-byte aligned (gates: 4-byte); with
 * seq_len == 0 the call does nothing and accepts any pointer.  One handle serves one
 * stream at a time (the workspace is shared by its calls).
 * Errors: INVALID_ARGUMENT (null/misaligned/overlapping pointers, bad
 * handle, a handle with ATLAS_BIAS_HUBER: it needs atlas_mem_forward_ex),
 * HIP (launch failure).  NaN/Inf in the inputs propagate.                  */
atlas_status atlas_mem_forward(atlas_mem_t h,
                               const void* q, const void* k, const void* v,
                               const float* alpha, const float* eta,
                               const float* theta, const float* gamma,
                               void* state, void* out, void* stream /* hipStream_t */);

/* atlas_mem_forward with the per-token Huber thresholds delta [B][H][N]
 * fp32 (device, 4-byte aligned; required with ATLAS_BIAS_HUBER, ignored
 * and may be NULL otherwise).  The Huber bias of the Miras review ("Yaad"):
 * per token, the squared-error gradient while |f(x_i) - v_i|_2 <= delta_i,
 * else delta_i * sign(f(x_i) - v_i).  Same semantics and errors otherwise. */
atlas_status atlas_mem_forward_ex(atlas_mem_t h,
                                  const void* q, const void* k, const void* v,
                                  const float* alpha, const float* eta,
                                  const float* theta, const float* gamma, const float* delta,
                                  void* state, void* out, void* stream /* hipStream_t */);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * call as atlas_mem_forward_ex (same kernels, same results bit for bit, same
 * argument rules), configured by *cfg directly: no handle and no allocation.
 * Its workspace (coefficient blocks, operand images, exchange buffers and
 * control words) lives in one static device buffer of the library, 32 MiB
 * per device, which each device that runs such a call holds until the
 * process ends.  A call whose workspace does not fit returns
 * ATLAS_ERR_SCRATCH_TOO_SMALL and enqueues nothing (for a size, the
 * handle's workspace is what atlas_mem_init would allocate).  Every call on
 * one device shares that buffer, which keeps the last call's contents: calls
 * that overlap on one device (two streams, two threads) race and give wrong
 * results.  errors (device, optional, 4-byte aligned) receives the call's
 * device error word after its kernels (0: none; bit 0: a group barrier timed
 * out and the outputs are invalid; bit 1: the workgroups of one sequence did
 * not all run on one XCD); it replaces atlas_mem_device_errors.
 * Errors: as atlas_mem_forward_ex, plus SCRATCH_TOO_SMALL; UNSUPPORTED /
 * INVALID_ARGUMENT for a config atlas_mem_init would reject.               */
atlas_status atlas_mem_forward_noalloc(const atlas_mem_config* cfg,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* eta,
                                       const float* theta, const float* gamma, const float* delta,
                                       void* state, void* out, unsigned* errors,
                                       void* stream /* hipStream_t */);

/* Optional timing hook for profilers and benchmarks: while set, every
 * atlas_mem_forward records `before` on its stream right before the
 * recurrent chunk kernel and `after` right after it.  Both are hipEvent_t
 * created by the caller, who keeps ownership; NULL, NULL clears the hook.
 * Errors: INVALID_ARGUMENT (bad handle, exactly one event NULL).           */
atlas_status atlas_mem_set_kernel_events(atlas_mem_t h, void* before, void* after);

/* Kernel family the handle runs (ATLAS_KERNEL_PER_SEQUENCE, _SHARDED,
 * _STREAMED or _GROUPED; AUTO is resolved at init).  Returns -1 for an
 * invalid handle.                                                           */
int atlas_mem_kernel_family(atlas_mem_t h);

/* Device-side error word of the handle's last forward call (0: none; bit 0:
 * a group barrier of the sharded, streamed or grouped kernel timed out, its
 * outputs are invalid; bit 1: the workgroups of one sequence (sharded group,
 * streamed pair or grouped group) did not all run on one XCD, so their
 * exchanges were not ordered and the outputs are invalid).
 * Synchronises the device.  Errors: INVALID_ARGUMENT, HIP.                 */
atlas_status atlas_mem_device_errors(atlas_mem_t h, unsigned* flags);

/* Releases the workspace and the handle (NULL is accepted).                */
atlas_status atlas_mem_free(atlas_mem_t h);

/* Static description of a status code.                                     */
const char* atlas_mem_error_string(int code);

/* Text of the last HIP error seen by this thread, "" if none.              */
const char* atlas_mem_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ATLAS_MEM_H */
