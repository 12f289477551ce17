/*
 * atlas_prologue.h -- C ABI of the fused prologue that produces the test-time
 * memory's inputs from a layer's input x (Titans review, sec. 4.4
 * "Architectural Details": SiLU on the query/key/value computation, L2-norm
 * of queries and keys, a 1D depthwise convolution after the q/k/v
 * projections; Miras review, "Training": depthwise convolution across tokens
 * after q, k, v, L2-normalised q and k, gates as per-token values from
 * low-rank projections).
 *
 * Per sequence b and token t:
 *   P_t     = W x_t          W = [Wq; Wk; Wv; U_alpha; U_eta; U_theta; U_gamma]
 *                            (bf16 in, fp32 accumulate, P rounded to bf16)
 *   c_t     = sum_{j<K} w_conv[ch][j] P_{t-(K-1)+j}[ch]    for the 3*H*d q/k/v
 *                            channels; tokens before the sequence start count as
 *                            zero (each call starts its sequences)
 *   q, k, v = SiLU(c),  SiLU(z) = z sigmoid(z)
 *   q, k    <- x / max(|x|_2, 1e-12) per head over its d channels
 *   gate_g  = sigmoid(V_g (U_g x_t) + b_g) per head, g = alpha, eta, theta, gamma
 * The outputs are laid out as atlas_mem_forward takes them.
 *
 * Two paths with the same bits: one kernel that keeps each tile of P on
 * chip and applies the per-token steps to it (the default where it serves
 * the shape: d 64, 128 or 256, 3*H*d a multiple of 256, one sequence of x
 * below 1 GiB), and a projection GEMM into a workspace followed by a
 * per-token kernel (every other shape).
 *
 * Errors as in atlas_mem.h: nothing throws, every call returns a status.
 */
#ifndef ATLAS_PROLOGUE_H
#define ATLAS_PROLOGUE_H

#include "atlas_mem.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int batch;       /* B sequences                                             */
  int seq_len;     /* N tokens per sequence (>= 0)                             */
  int d_model;     /* width of x, a multiple of 8                              */
  int heads;       /* H                                                       */
  int d_head;      /* d: 64, 128 or 256                                       */
  int conv_taps;   /* K, 1 .. 8                                               */
  int gate_rank;   /* r: 1, 2, 4, 8 or 16                                      */
} atlas_prologue_config;

typedef struct atlas_prologue_s* atlas_prologue_t;

/* Validates cfg; on the current device, allocates the projection workspace
 * (B*N rows of 3*H*d + 4*r bf16) if the one-kernel path does not serve it.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (d_head, taps or rank outside the
 * built range), OUT_OF_MEMORY, HIP.                                        */
atlas_status atlas_prologue_init(const atlas_prologue_config* cfg, atlas_prologue_t* out);

/* One call, enqueued on `stream`, no synchronisation, no allocation.
 *   x       [B][N][d_model]            bf16
 *   w       [3*H*d + 4*r][d_model]     bf16 (rows: Wq, Wk, Wv, then U_alpha,
 *                                      U_eta, U_theta, U_gamma with r rows each)
 *   w_conv  [3*H*d][K]                 fp32 (channel order of the q, k, v rows of w)
 *   gate_v  [4][H][r], gate_b [4][H]   fp32
 *   q, k    [B][H][N][d], v [B][H][N][d]   bf16 outputs
 *   alpha, eta, theta, gamma [B][H][N]      fp32 outputs
 * Device pointers, 16-byte aligned (fp32 parameters and gates: 4-byte).
 * Errors: INVALID_ARGUMENT (bad handle or pointer), HIP (launch failure). */
atlas_status atlas_prologue_forward(atlas_prologue_t h, const void* x, const void* w, const float* w_conv,
                                    const float* gate_v, const float* gate_b, void* q, void* k, void* v,
                                    float* alpha, float* eta, float* theta, float* gamma, void* stream);

/* Path selection, for tests and timing: fused = 1 takes the one-kernel path
 * (UNSUPPORTED where it does not serve the shape), 0 the two-kernel path
 * (allocates its workspace on first use: OUT_OF_MEMORY).  Not to be called
 * while a forward of this handle may run.                                  */
atlas_status atlas_prologue_set_fused(atlas_prologue_t h, int fused);

/* Timing hook: while set, each forward records `gemm_before` first, then
 * `before` and `after` (caller-owned hipEvent_t) around the per-token kernel
 * of the two-kernel path, or around the one kernel; NULLs clear it.        */
atlas_status atlas_prologue_set_events(atlas_prologue_t h, void* gemm_before, void* before, void* after);

/* Releases the workspace and the handle (NULL accepted).                    */
atlas_status atlas_prologue_free(atlas_prologue_t h);

#ifdef __cplusplus
}
#endif
#endif
