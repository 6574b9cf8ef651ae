/*
 * pararnn.h -- C ABI of the MI355X (gfx950) ParaRNN Newton solver.
 *
 * The method (ParaRNN articles, cafecomtech.com "ParaRNN: Apple destrava treino
 * paralelo de RNNs nao-lineares ..." and aifeed.sk "Apple vracia do hry RNN ..."):
 * a nonlinear recurrence h_l = f(h_{l-1}, x_l) over a whole sequence is one
 * system of equations in all hidden states (section "A sacada: metodo de
 * Newton"). Newton's method linearises it with the per-step Jacobians; the
 * linearised system is a linear SSM h_l = A_l h_{l-1} + b_l with the Jacobians
 * as A_l, solved by a parallel scan (section "O compromisso que SSMs fizeram").
 * With diagonal cell matrices the Jacobians are diagonal (ParaGRU) or 2x2
 * block-diagonal over (c, h) (ParaLSTM) (section "Engenharia pra escalar").
 *
 * Cells, per channel d, with gate inputs u precomputed and diagonal recurrent
 * coefficients a (s = logistic sigmoid):
 *   GRU,  gates (z, r, c):  z = s(a_z h + u_z), r = s(a_r h + u_r),
 *         c~ = tanh(a_c (r h) + u_c), h' = (1 - z) h + z c~.
 *   LSTM, gates (i, f, o, g), state (c, h): i, f, o = s(a_* h + u_*),
 *         g = tanh(a_g h + u_g), c' = f c + i g, h' = o tanh(c').
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers to caller-owned, contiguous,
 *    row-major buffers. The library never allocates, frees or keeps a pointer
 *    after returning; all scratch lives in the caller's workspace `ws` (the
 *    one exception, pararnn_solve_gru_scratch, uses a scratch array built into
 *    the library instead).
 *  - Layouts: u [B][L][G][D] (fp32 or bf16 per opts.u_dtype), a [G][D] fp32,
 *    states h, c [B][L][D] fp32, initial states h0, c0 [B][D] fp32 (NULL means
 *    zero), dh [B][L][D] fp32, du [B][L][G][D] fp32 (always fp32).
 *  - Pointers must be at least 4-byte aligned (2-byte for bf16 u); 16-byte
 *    alignment with D divisible by 4 selects the widest memory accesses.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *    asynchronous: inputs must stay alive and unmodified, and outputs must not
 *    be read, until the stream reaches the end of the call. Calls on different
 *    streams are safe when each has its own workspace; two calls sharing one
 *    workspace must be ordered on one stream.
 *  - Inputs and outputs must not alias each other or the workspace.
 *  - Return value: PARARNN_OK, or a negative PARARNN_E* code; on an error
 *    nothing has been launched (except PARARNN_EHIP, reported when a launch
 *    itself fails). Numerical trouble is not an error: NaN/Inf propagate into
 *    the states and max_update, and the row is reported as not converged.
 */
#ifndef PARARNN_H
#define PARARNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARARNN_OK 0
#define PARARNN_EINVAL (-1)       /* null pointer, size <= 0, max_iters < 1, bad enum, size overflow */
#define PARARNN_EUNSUPPORTED (-2) /* unsupported dtype or misaligned pointer */
#define PARARNN_EWORKSPACE (-3)   /* ws_bytes smaller than pararnn_workspace_bytes() */
#define PARARNN_EHIP (-4)         /* a HIP launch or runtime call failed */
#define PARARNN_ESCRATCH (-5)     /* the built-in scratch of pararnn_solve_gru_scratch is too small */

typedef enum { PARARNN_F32 = 0, PARARNN_BF16 = 1 } pararnn_dtype;

/* How a solve is laid out in launches (opts.schedule). */
typedef enum {
  PARARNN_SCHEDULE_AUTO = 0,          /* FUSED, or PER_ITERATION when early_exit is set */
  PARARNN_SCHEDULE_FUSED = 1,         /* all K iterations in one launch; the iterate stays on
                                         chip between iterations and only iterate K is written
                                         (ParaRNN article, cafecomtech.com, section "Engenharia
                                         pra escalar": Newton, assembly and reduction fused);
                                         not combinable with early_exit */
  PARARNN_SCHEDULE_PER_ITERATION = 2  /* one fused launch per iteration, iterates through HBM */
} pararnn_schedule;
typedef enum { PARARNN_GRU = 0, PARARNN_LSTM = 1 } pararnn_cell;
typedef enum {
  PARARNN_OP_SOLVE = 0,
  PARARNN_OP_ADJOINT = 1,
  PARARNN_OP_SCAN_DIAG = 2,   /* pararnn_scan_diag; the cell argument is ignored */
  PARARNN_OP_SCAN_BLOCK2 = 3, /* pararnn_scan_block2; the cell argument is ignored */
  PARARNN_OP_SCAN_DENSE = 4   /* pararnn_scan_dense; the cell argument is ignored */
} pararnn_op;

typedef struct {
  int32_t B, L, D;    /* batch rows, sequence length, channels; all >= 1 */
  int32_t max_iters;  /* K: Newton iterations (launches), >= 1 */
  float tol;          /* convergence threshold on max |update| of the last iteration */
  int32_t early_exit; /* 0: always K iterations. 1: stop after the first iteration
                         whose update satisfies tol on every row (later launches copy) */
  int32_t u_dtype;    /* pararnn_dtype of u */
  void* const* events; /* optional, NULL = none: hipEvent_t handles, each NULL
                          or created by the caller. Solve (K + 2): [0] before
                          the workspace reset; [1] the start of the first
                          kernel after it; [k + 1] the end of iteration k's
                          launch (fused schedule: [2] the end of its one
                          launch, [3..K+1] recorded right after). Adjoint and
                          scans (3): before the workspace reset (the dense
                          scan has none), the start of the first kernel, the
                          end of the last. Starts and ends are
                          stamped by the kernel dispatch itself, so an
                          interval between them is execution time without
                          the latency of a separate marker. */
  int32_t schedule;    /* pararnn_schedule of a solve; ignored by the other calls */
} pararnn_opts;

/* Bytes of workspace a call with these options needs (depends on the cell,
 * the operation, B, L, D, max_iters and u_dtype). Returns 0 for invalid
 * options. Host-only; launches nothing. */
size_t pararnn_workspace_bytes(int32_t cell, int32_t op, const pararnn_opts* o);

/* ParaGRU forward solve: K Newton iterations from the zero sequence (the
 * initial state h0 is fixed) on the whole-sequence system S_l = f(S_{l-1}, u_l)
 * (ParaRNN article, cafecomtech.com, section "A sacada: metodo de Newton").
 * Iteration k linearises the system at iterate k-1, assembles the diagonal
 * Jacobian coefficients (section "Engenharia pra escalar": diagonal cell
 * matrices give a diagonal Jacobian) and solves the linear SSM by a parallel
 * scan (section "O compromisso que SSMs fizeram"); by default all K
 * iterations run in one fused launch. Outputs (device):
 *   h          [B][L][D] the K-th iterate (always; also with early exit)
 *   iters      [1] number of iterations performed (K unless early exit fired), or NULL
 *   converged  [B] 1 if max |h^(iters) - h^(iters-1)| <= tol on that row, else 0, or NULL
 *   max_update [K][B] max |h^(k) - h^(k-1)| per iteration and row (0 for skipped
 *              iterations; NaN if the row holds NaN), or NULL */
int32_t pararnn_solve_gru(const void* u, const float* a, const float* h0, float* h, void* ws,
                          size_t ws_bytes, const pararnn_opts* o, int32_t* iters,
                          int32_t* converged, float* max_update, void* stream);

/* The ParaGRU forward solve of pararnn_solve_gru for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no ws / ws_bytes arguments. The workspace
 * is a scratch array built into the library, one per GPU, of
 * pararnn_scratch_bytes() bytes (64 MiB), reserved when the library's code
 * object is loaded on that GPU and held until the process ends. The call
 * allocates and frees nothing; on its first call on a GPU it looks up the
 * array's device address (hipGetSymbolAddress) with that GPU current.
 * Arguments, outputs, asynchrony and numerics are those of pararnn_solve_gru.
 * Errors: as for pararnn_solve_gru; PARARNN_ESCRATCH, before any HIP call,
 * when the workspace of the launch the call makes exceeds the scratch size
 * (that launch's channel group follows from D and the pointers' alignment;
 * pararnn_workspace_bytes(PARARNN_GRU, PARARNN_OP_SOLVE, o), which covers
 * every channel group, bounds it from above). Every call on one GPU uses
 * that GPU's one array, and each call resets what must start at zero; calls
 * on one GPU must therefore be ordered (one stream, or synchronised): calls
 * that overlap in time race on the array and give wrong results. */
int32_t pararnn_solve_gru_scratch(const void* u, const float* a, const float* h0, float* h,
                                  const pararnn_opts* o, int32_t* iters, int32_t* converged,
                                  float* max_update, void* stream);

/* Size in bytes of the built-in scratch of pararnn_solve_gru_scratch. */
size_t pararnn_scratch_bytes(void);

/* ParaLSTM forward solve: as pararnn_solve_gru with the 2x2 block Jacobian over
 * (c, h) (ParaRNN article, cafecomtech.com, section "Engenharia pra escalar":
 * diagonal cell matrices give a 2x2 block-diagonal Jacobian for the LSTM;
 * section "A sacada: metodo de Newton" for the iteration). Outputs c and h,
 * both [B][L][D]; max_update is the max over both state components. */
int32_t pararnn_solve_lstm(const void* u, const float* a, const float* c0, const float* h0,
                           float* c, float* h, void* ws, size_t ws_bytes, const pararnn_opts* o,
                           int32_t* iters, int32_t* converged, float* max_update, void* stream);

/* Adjoint (reverse linear scan) along a given trajectory, e.g. the solve's
 * output, for upstream gradient dh = dL/dh:
 *   lambda_{L-1} = G_{L-1},  lambda_l = G_l + J_{l+1}^T lambda_{l+1},
 *   J_{l+1} = df/ds at (state_l, u_{l+1}), G_l = dh_l (GRU) or (0, dh_l) (LSTM),
 *   du_l = (df/du at (state_{l-1}, u_l))^T lambda_l.
 * c and c0 are ignored for the GRU (pass NULL). Outputs (device, fp32):
 *   du  [B][L][G][D]
 *   ds0 [NS][B][D] gradient of the initial state (NS = 1: h0; NS = 2: c0 then h0), or NULL
 *   da  [G][D] gradient of the coefficients summed over B and L, or NULL
 * opts.max_iters, tol and early_exit are ignored. */
int32_t pararnn_adjoint(int32_t cell, const void* u, const float* a, const float* c0,
                        const float* h0, const float* c, const float* h, const float* dh,
                        float* du, float* ds0, float* da, void* ws, size_t ws_bytes,
                        const pararnn_opts* o, void* stream);

/* The linear scan alone: the solver step of every Newton iteration, for a
 * linear SSM the caller has assembled, e.g. from the Jacobians of a cell this
 * library does not implement (ParaRNN article, cafecomtech.com: section
 * "O compromisso que SSMs fizeram" for the linear recurrence and its parallel
 * scan, section "Como usar" for cells supplied by the user). Per channel
 * (b, d), for l = 0 .. L-1:
 *   s_l = A_l s_{l-1} + b_l,   s_{-1} = s0 (zero when s0 is NULL).
 * pararnn_scan_diag: A_l is a scalar (diagonal Jacobian, NS = 1).
 * pararnn_scan_block2: A_l is a 2x2 block over the channel's two state
 *   components (NS = 2); s_l[r] = sum_q A_l[r][q] s_{l-1}[q] + b_l[r].
 * Layouts: component-major fp32 planes of [B][L][D] each (device):
 *   A  [NS*NS][B][L][D], block entries row-major: A00, A01, A10, A11
 *   b  [NS][B][L][D],  s (output) [NS][B][L][D],  s0 [NS][B][D] or NULL.
 * Workspace: pararnn_workspace_bytes(any cell, PARARNN_OP_SCAN_DIAG or
 * PARARNN_OP_SCAN_BLOCK2, o). opts: B, L, D and events (3 handles, as for
 * the adjoint) are used; the others are ignored. Non-finite coefficients propagate like any other value. Errors as
 * for the solves; 16-byte alignment with D divisible by 4 (diag) or 2 (block2)
 * selects the widest accesses. */
int32_t pararnn_scan_diag(const float* A, const float* b, const float* s0, float* s, void* ws,
                          size_t ws_bytes, const pararnn_opts* o, void* stream);
int32_t pararnn_scan_block2(const float* A, const float* b, const float* s0, float* s, void* ws,
                            size_t ws_bytes, const pararnn_opts* o, void* stream);

/* The linear scan with a dense n x n matrix per step: the linearised system of
 * a generic RNN, whose Jacobians are dense (ParaRNN article, cafecomtech.com,
 * section "Engenharia pra escalar": n^2 storage and n^3 products, hence small
 * n only). Per batch row b, for l = 0 .. L-1:
 *   s_l = A_l s_{l-1} + b_l,   s_{-1} = s0 (zero when s0 is NULL),
 *   s_l[r] = sum_q A_l[r][q] s_{l-1}[q] + b_l[r].
 * Layouts (device, fp32, row-major): A [B][L][n][n], b and s (output)
 * [B][L][n], s0 [B][n] or NULL. n = opts.D, 1 <= n <= 32; opts.B and opts.L
 * as usual; opts.events: 3 handles, as for the adjoint.
 * The chunk transfer products run on the matrix cores in fp32. Workspace:
 * pararnn_workspace_bytes(any cell, PARARNN_OP_SCAN_DENSE, o). Pointers need
 * 4-byte alignment. Errors as for the other calls; n > 32 is EINVAL. */
int32_t pararnn_scan_dense(const float* A, const float* b, const float* s0, float* s, void* ws,
                           size_t ws_bytes, const pararnn_opts* o, void* stream);

/* The launch plan of a call (host-only; launches nothing), for callers and
 * tests that need to know how the work is split: a workgroup covers `chunk`
 * timesteps x `channels` channels, with `vec` channels per lane; `nchunks`
 * chunks along L are chained by the chunk carry, each chunk row holding
 * `tiles_per_row` = B x ceil(D / channels) workgroups. `inclusive_only` = 1
 * when each chunk takes its carry from its neighbour's inclusive carry alone
 * (a fixed composition order: repeated calls give identical bits); 0 when it
 * uses the decoupled look-back over chunk aggregates (repeated calls agree to
 * rounding). `fused` = 1 for the one-launch schedule of a solve. The plan is
 * the one used when every pointer is 16-byte aligned (narrower alignment
 * only lowers `vec`). Returns PARARNN_OK, or PARARNN_EINVAL for invalid
 * options or a NULL plan. */
typedef struct {
  int32_t vec, chunk, channels, nchunks, tiles_per_row, inclusive_only, fused;
} pararnn_plan;
int32_t pararnn_plan_query(int32_t cell, int32_t op, const pararnn_opts* o, pararnn_plan* plan);

/* Static description of a status code. */
const char* pararnn_strerror(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* PARARNN_H */
