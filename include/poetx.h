/*
 * poetx.h -- C ABI of libpoetx.so: forward and backward pass of one POET-X
 * reparameterized linear layer on AMD Instinct MI355X (gfx950).
 *
 * The layer ("Reparameterized LLM Training via Orthogonal Equivalence
 * Transformation", Abstract) computes y = x W^T with W = R W0 P, where W0 is
 * a fixed random [m, n] weight and R, P are learnable orthogonal matrices.
 * Following "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
 * Transformation" (technical summary, sections 2.1-2.4):
 *   - R = Pi_R^T BD(G_R) Pi_R and P = Pi_P^T BD(G_P) Pi_P: block-diagonal
 *     orthogonal matrices with b x b blocks, conjugated by random
 *     permutations; permutation matrix of an index map: Pi[i, pi[i]] = 1;
 *   - each block is G = (I+Q)(I + Q + ... + Q^k), the Cayley transform with
 *     its inverse replaced by the Neumann series cut after Q^k, where Q is
 *     skew-symmetric and only its strict upper triangle is stored (b(b-1)/2
 *     parameters per block, row by row over i < j);
 *   - the evaluation is input-centric: W is never formed; the input passes
 *     through the P-side blocks, the fixed weight, then the R-side blocks;
 *   - permutations are index maps; the two next to W0 are folded into it
 *     once per inner loop: W0f[i, j] = W0[pi_R[i], pi_P[j]].
 * With that fold the forward pass is
 *   U = x[:, pi_P];  V_j = U_j G_Pj^T;  Z = V W0f^T;  S_i = Z_i G_Ri^T;
 *   y[:, pi_R[c]] = S[:, c]
 * (U_j: columns [j b, (j+1) b) of U), and the backward pass is
 *   dS = dy[:, pi_R];  dZ_i = dS_i G_Ri;  dG_Ri = sum_t dS_i^T Z_i;
 *   dV = dZ W0f;  dU_j = dV_j G_Pj;  dG_Pj = sum_t dV_j^T U_j;
 *   dx[:, pi_P[c]] = dU[:, c];  dtheta = CNP^T(theta, dG).
 * W0 is fixed and gets no gradient.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major and contiguous, base
 *     aligned to 16 bytes.  The caller owns every buffer; the library never
 *     allocates or frees device memory.
 *   - Activation storage type `act` (POETX_F32 or POETX_BF16) applies to x,
 *     y, dy, dx, W0, W0f, W0fT, G and GT.  theta, dtheta and dG are float32.
 *     bf16 values are IEEE binary32 truncated to 16 bits; the library rounds
 *     to nearest-even whenever it narrows.  Arithmetic accumulates in fp32.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream);
 *     no call synchronizes the host.  Device faults surface at the caller's
 *     next synchronization.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is written.  Permutations being valid is a
 *     precondition that is not checked on the device.
 *   - Entry points are thread-safe and keep no state between calls, except
 *     poetx_cnp_fwd_noalloc, whose scratch array is shared by its calls.
 *   - poetx_last_error() returns a message for the calling thread's most
 *     recent failure.
 */
#ifndef POETX_H
#define POETX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define POETX_ABI_VERSION 2

typedef enum {
  POETX_OK = 0,
  POETX_ERR_ARG = 1,          /* null pointer, bad size, misalignment      */
  POETX_ERR_UNSUPPORTED = 2,  /* valid but not built (dtype / b pair)       */
  POETX_ERR_WORKSPACE = 3,    /* workspace smaller than required            */
  POETX_ERR_DEVICE = 4        /* HIP launch or device query failed          */
} poetx_status;

typedef enum { POETX_F32 = 0, POETX_BF16 = 1, POETX_I8 = 2 } poetx_dtype;
/* POETX_I8 is a weight storage type only (poetx_fold_perm, poetx_dequant). */

/* Shape of one layer.  m: outputs, n: inputs, b: block size (m % b == 0 and
 * n % b == 0), k: Neumann order (>= 0), T: tokens (>= 1), act: poetx_dtype.
 * Supported b: 8, 16, 32, 64, 128, 256, 512; float32 activations need
 * b <= 64.  1 <= k <= 8 or k = 0. */
typedef struct {
  int32_t m, n, b, k, T;
  int32_t act;
} poetx_shape;

typedef void* poetx_stream_t; /* a hipStream_t */

/* ABI version of the loaded library (POETX_ABI_VERSION). */
int32_t poetx_abi_version(void);

/* Static string naming a status code. */
const char* poetx_status_str(int32_t status);

/* Message describing the calling thread's most recent error ("" if none). */
const char* poetx_last_error(void);

/*
 * poetx_cnp_fwd -- Cayley-Neumann parameterization, forward
 * ("POET-X ...", technical summary 2.4, "Efficient CNP"; the Italian page,
 * "Sommario tecnico" 2, CNP bullet).
 *   theta [nblk][b(b-1)/2] float32: packed strict upper triangle of each
 *         skew-symmetric Q (Q[i][j] = theta[t], Q[j][i] = -theta[t],
 *         t = i*b - i*(i+1)/2 + (j-i-1) for i < j).
 *   G     [nblk][b][b] in g_dtype: G = (I+Q)(I + Q + ... + Q^k).
 *   GT    [nblk][b][b] in g_dtype or NULL: G transposed (= CNP of -Q).
 *   ws    workspace of poetx_cnp_workspace_bytes(nblk, b, k, 0, g_dtype) bytes
 *         (may be NULL when that is 0).
 * Errors: ERR_ARG (nblk < 1, k outside 0..8, b unsupported, null theta/G),
 * ERR_UNSUPPORTED (float32 with b > 64), ERR_WORKSPACE, ERR_DEVICE.
 */
int32_t poetx_cnp_fwd(int32_t nblk, int32_t b, int32_t k, const float* theta,
                      void* G, void* GT, int32_t g_dtype, void* ws,
                      size_t ws_bytes, poetx_stream_t stream);

/*
 * poetx_cnp_fwd_noalloc -- poetx_cnp_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels, bitwise the same G and GT.  The unpacked Q
 * that poetx_cnp_fwd keeps in its workspace goes instead to a library-owned
 * device array of POETX_NOALLOC_SCRATCH_BYTES bytes, one per GPU, which
 * exists from the library's load on that GPU until the process ends; the
 * call itself allocates nothing.  It needs nblk*b*b*2 bytes for bf16 blocks
 * of 64..512 (e.g. up to 64 blocks of 512 or 256 of 256) and none
 * otherwise; more gives ERR_WORKSPACE with nothing enqueued.  Every call on
 * a GPU shares that GPU's array, and each call overwrites what it reads
 * before reading it (nothing needs clearing), so calls that overlap on one
 * GPU -- on different streams, or from different threads -- race and give
 * wrong G.  The array is the one of the calling thread's current device;
 * `stream` must belong to that device.
 * Errors as poetx_cnp_fwd (ERR_WORKSPACE: the blocks exceed the array).
 */
#define POETX_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t poetx_cnp_fwd_noalloc(int32_t nblk, int32_t b, int32_t k, const float* theta,
                              void* G, void* GT, int32_t g_dtype, poetx_stream_t stream);

/*
 * poetx_cnp_bwd -- gradient of the packed parameters (technical summary 2.4:
 * the backward pass reuses on-chip data and fuses, like the forward).
 * Given dG = dL/dG [nblk][b][b] float32, writes
 *   dtheta[t(i,j)] (=|+=) gQ[i][j] - gQ[j][i],  i < j,
 * where gQ = dL/dQ for G(Q) above.  accumulate != 0 adds into dtheta.
 *   prec: POETX_F32 (fp32 arithmetic, b <= 64) or POETX_BF16 (bf16 MFMA
 *         operands with fp32 accumulation), the class of the layer's G.
 *   ws: poetx_cnp_workspace_bytes(nblk, b, k, 1, prec) bytes.
 * Errors as poetx_cnp_fwd (null dG/dtheta -> ERR_ARG).
 */
int32_t poetx_cnp_bwd(int32_t nblk, int32_t b, int32_t k, const float* theta,
                      const float* dG, float* dtheta, int32_t accumulate,
                      int32_t prec, void* ws, size_t ws_bytes,
                      poetx_stream_t stream);

/*
 * poetx_cnp_bwd_after_fwd -- poetx_cnp_bwd for the step's own forward pass:
 * the same arguments and results (bitwise), but `ws` must be the workspace
 * that last served poetx_cnp_fwd with the same nblk, b, k, theta and
 * precision (g_dtype = prec), untouched since.  On the bf16 MFMA path the
 * forward leaves the unpacked Q at the start of its workspace and this call
 * reads it there instead of unpacking theta again (one kernel less); other
 * configurations do exactly what poetx_cnp_bwd does.  ws is sized for the
 * backward, poetx_cnp_workspace_bytes(nblk, b, k, 1, prec), which also
 * serves the forward.  Passing a workspace that does not hold that Q gives
 * wrong dtheta; it is not detected.
 * Errors as poetx_cnp_bwd.
 */
int32_t poetx_cnp_bwd_after_fwd(int32_t nblk, int32_t b, int32_t k, const float* theta,
                                const float* dG, float* dtheta, int32_t accumulate,
                                int32_t prec, void* ws, size_t ws_bytes,
                                poetx_stream_t stream);

/* Workspace bytes for poetx_cnp_fwd (which = 0) or poetx_cnp_bwd (1) with
 * float32 (act = POETX_F32) or bf16 (POETX_BF16) activations;
 * 0 on bad arguments. */
size_t poetx_cnp_workspace_bytes(int32_t nblk, int32_t b, int32_t k,
                                 int32_t which, int32_t act);

/*
 * poetx_fold_perm -- permutation reduction (technical summary 2.2: two of
 * the four forward permutations are merged into the weight before the inner
 * loop).  Pure data movement, bit-exact:
 *   W0f[i][j]  = W0[perm_R[i]][perm_P[j]]        [m][n]
 *   W0fT[j][i] = W0f[i][j]                       [n][m], or NULL
 *   perm_R_inv[perm_R[i]] = i  (m entries), perm_P_inv likewise (n), or NULL.
 * W0fT is the layout the backward dV = dZ W0f product reads.
 * Errors: ERR_ARG (m, n < 1, null W0/perm/W0f, dt not F32/BF16).
 */
int32_t poetx_fold_perm(int32_t m, int32_t n, int32_t dt, const void* W0,
                        const int32_t* perm_R, const int32_t* perm_P, void* W0f,
                        void* W0fT, int32_t* perm_R_inv, int32_t* perm_P_inv,
                        poetx_stream_t stream);

/*
 * POET-XQ ("POET-X ...", technical summary 2.6: training on a low-bit base
 * model, INT8, dequantized on the fly when needed; the high-precision weight
 * is never kept).  The base weight is held as int8 q with one fp32 scale per
 * output row: W0[i][j] = s[i] * q[i][j].  poetx_fold_perm folds q
 * (dt = POETX_I8) into q_f and q_fT; poetx_fold_scale folds the scales.
 * poetx_layer_fwd_q / poetx_layer_bwd_q run the layer on (q_f, q_fT, s_f)
 * directly: the dense kernel widens the int8 operand to bf16 as it reads it
 * (exact) and applies s_f to its fp32 sums, so no high-precision copy of the
 * weight exists at any point.  poetx_dequant (an explicit bf16 copy) remains
 * for callers that want one.
 *
 * poetx_fold_scale -- s_f[i] = s[perm_R[i]], i < m (fp32).
 * poetx_dequant -- out[r][c] = bf16(scale * q[r][c]) for q int8 [rows][cols]
 *   (cols % 16 == 0, 16-byte aligned); per_row = 1: scale[r] (q_f against
 *   s_f gives W0f), per_row = 0: scale[c] (q_fT against s_f gives W0fT).
 *   Rounds to nearest even.
 * Errors: ERR_ARG, ERR_DEVICE.
 */
int32_t poetx_fold_scale(int32_t m, const float* s, const int32_t* perm_R, float* s_f,
                         poetx_stream_t stream);
int32_t poetx_dequant(int32_t rows, int32_t cols, const void* q, const float* scale,
                      int32_t per_row, void* out, poetx_stream_t stream);

/*
 * poetx_layer_fwd_q / poetx_layer_bwd_q -- poetx_layer_fwd / _bwd (xmem = 0)
 * or their memory-saving variants (xmem != 0) on an int8 base weight
 * (technical summary 2.6), with W0f = diag(s_f) q_f in place of the bf16 W0f:
 *   q_f  [m][n] int8, q_fT [n][m] int8 (poetx_fold_perm with POETX_I8),
 *   s_f  [m] fp32 (poetx_fold_scale).
 * The forward forms Z = (V q_f^T) diag(s_f); the backward forms
 * dZ' = dZ diag(s_f) in the R-side block pass and dV = dZ' q_f.  Every
 * other argument, and the saved / workspace sizes (which 0..3 as for the
 * bf16 calls), are those of the bf16 calls.  bwd: G_P and q_f are read only
 * with xmem (may be NULL otherwise).  Needs bf16 activations, b >= 64 and
 * m, n multiples of 256 (ERR_UNSUPPORTED otherwise).
 * Errors: ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE.
 */
int32_t poetx_layer_fwd_q(const poetx_shape* sh, const void* x, const void* G_P, const void* G_R,
                          const int8_t* q_f, const float* s_f, const int32_t* perm_P,
                          const int32_t* perm_R_inv, void* y, void* saved, void* ws,
                          size_t ws_bytes, int32_t xmem, poetx_stream_t stream);
int32_t poetx_layer_bwd_q(const poetx_shape* sh, const void* dy, const void* G_P, const void* GT_P,
                          const void* GT_R, const int8_t* q_f, const int8_t* q_fT,
                          const float* s_f, const int32_t* perm_P_inv, const int32_t* perm_R,
                          const void* saved, void* dx, float* dG_P, float* dG_R, void* ws,
                          size_t ws_bytes, int32_t xmem, poetx_stream_t stream);

/*
 * poetx_layer_fwd -- input-centric forward pass (technical summary 2.1-2.3).
 *   x     [T][n]        input (act)
 *   G_P   [n/b][b][b]   P-side blocks (act), from poetx_cnp_fwd
 *   G_R   [m/b][b][b]   R-side blocks (act)
 *   W0f   [m][n]        folded weight (act), from poetx_fold_perm
 *   perm_P [n], perm_R_inv [m]  int32 index maps
 *   y     [T][m]        output (act)
 *   saved poetx_saved_bytes(sh) bytes: activations kept for the backward
 *         pass (U = x[:, pi_P] then Z, both [T][*] act); the caller keeps it
 *         alive and unmodified until poetx_layer_bwd.
 *   ws    poetx_workspace_bytes(sh, 0) bytes of scratch.
 * Errors: ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE.
 */
int32_t poetx_layer_fwd(const poetx_shape* sh, const void* x, const void* G_P,
                        const void* G_R, const void* W0f, const int32_t* perm_P,
                        const int32_t* perm_R_inv, void* y, void* saved,
                        void* ws, size_t ws_bytes, poetx_stream_t stream);

/*
 * poetx_layer_bwd -- backward pass ("POET-X ...", technical summary 2.1-2.3:
 * the same input-centric chain run in reverse, block products batched,
 * permutations as index maps; 2.5: the default, fast mode keeps the
 * forward's activations for it; "Reparameterized LLM Training ...",
 * Abstract: W0 stays fixed, only the orthogonal factors learn).
 *   dy    [T][m]        dL/dy (act)
 *   GT_P  [n/b][b][b]   P-side blocks transposed (act), from poetx_cnp_fwd
 *   GT_R  [m/b][b][b]   R-side blocks transposed (act)
 *   W0f   [m][n]        folded weight (act), the forward's own
 *   W0fT  [n][m]        its transpose (act) or NULL.  With NULL the dense
 *                       product dV = dZ W0f reads W0f itself (K-major), so
 *                       the fixed weight is held once; with a transposed
 *                       copy it reads that.  Both give bitwise the same
 *                       results.
 *   perm_P_inv [n], perm_R [m]  int32 index maps
 *   saved as written by poetx_layer_fwd for the same shape and inputs
 *   dx    [T][n]        dL/dx (act)
 *   dG_P  [n/b][b][b], dG_R [m/b][b][b]  float32 dL/dG (overwritten)
 *   ws    poetx_workspace_bytes(sh, 1) bytes of scratch.
 * The token reduction of dG is deterministic (no atomics): repeated calls
 * give bitwise-equal results.
 * Errors: ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE.
 */
int32_t poetx_layer_bwd(const poetx_shape* sh, const void* dy, const void* GT_P,
                        const void* GT_R, const void* W0f, const void* W0fT,
                        const int32_t* perm_P_inv, const int32_t* perm_R,
                        const void* saved, void* dx, float* dG_P, float* dG_R,
                        void* ws, size_t ws_bytes, poetx_stream_t stream);

/*
 * poetx_layer_fwd_xmem / poetx_layer_bwd_xmem -- the memory-saving mode
 * ("POET-X ...", technical summary 2.5: recompute in the backward pass
 * instead of keeping intermediates).  The forward keeps only U = x[:, pi_P]
 * in `saved` (poetx_saved_bytes_xmem(sh) bytes) and writes Z to its
 * workspace; the backward first recomputes V = U G_P^T and Z = V W0f^T with
 * the forward's own kernels, then runs as poetx_layer_bwd.  Outputs are
 * bitwise equal to those of poetx_layer_fwd / poetx_layer_bwd; the saved
 * buffer is T*m*sizeof(act) bytes smaller and the backward does one more
 * dense product (2 T m n flops) and one more block product (2 T n b flops).
 *   fwd: arguments as poetx_layer_fwd; ws poetx_workspace_bytes(sh, 2) bytes.
 *   bwd: arguments as poetx_layer_bwd plus G_P [n/b][b][b] (act) (W0fT
 *        may be NULL as there); ws poetx_workspace_bytes(sh, 3) bytes.
 * Errors: ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE.
 */
int32_t poetx_layer_fwd_xmem(const poetx_shape* sh, const void* x, const void* G_P,
                             const void* G_R, const void* W0f, const int32_t* perm_P,
                             const int32_t* perm_R_inv, void* y, void* saved,
                             void* ws, size_t ws_bytes, poetx_stream_t stream);
int32_t poetx_layer_bwd_xmem(const poetx_shape* sh, const void* dy, const void* G_P,
                             const void* GT_P, const void* GT_R, const void* W0f,
                             const void* W0fT, const int32_t* perm_P_inv,
                             const int32_t* perm_R, const void* saved, void* dx,
                             float* dG_P, float* dG_R, void* ws, size_t ws_bytes,
                             poetx_stream_t stream);

/* Bytes of the saved-activation buffer of the xmem mode; 0 on bad arguments. */
size_t poetx_saved_bytes_xmem(const poetx_shape* sh);

/*
 * poetx_merge -- end of an inner loop ("POET-X ...", technical summary 2.1:
 * the learned transforms are merged into the weight, W <- R W P, before new
 * ones start from the identity; 2.2: new permutations are then drawn and
 * folded).  Writes the current effective weight
 *   W0_out = R W0 P = Pi_R^T BD(G_R) W0f BD(G_P) Pi_P,
 *   W0_out[a][c] = M[pi_R^{-1}[a]][pi_P^{-1}[c]],  M = BD(G_R) W0f BD(G_P),
 * with two block products (4 m n b flops), two transposes and the
 * permutation.  The caller then resets theta to 0, draws new permutations
 * and calls poetx_fold_perm on W0_out.  T in `sh` is not used.
 *   W0f   [m][n]        folded weight (act)
 *   G_R   [m/b][b][b]   R-side blocks (act), GT_P [n/b][b][b] P-side blocks
 *                       transposed (act), both from poetx_cnp_fwd
 *   perm_R_inv [m], perm_P_inv [n]  from poetx_fold_perm
 *   W0_out [m][n] (act); must not alias W0f
 *   ws    poetx_workspace_bytes(sh, 4) bytes of scratch.
 * Errors: ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE.
 */
int32_t poetx_merge(const poetx_shape* sh, const void* W0f, const void* G_R,
                    const void* GT_P, const int32_t* perm_R_inv, const int32_t* perm_P_inv,
                    void* W0_out, void* ws, size_t ws_bytes, poetx_stream_t stream);

/*
 * poetx_set_stage_events -- timing hook for profilers and benchmarks.
 * While set, each poetx_layer_fwd / poetx_layer_bwd call on the calling
 * thread records events[i] (hipEvent_t handles owned by the caller) on its
 * stream at stage boundary i:
 *   forward  (count >= 6): 0 | gather x | 1 | P-side blocks | 2 | W0 product
 *            | 3 | R-side blocks | 4 | scatter y | 5
 *   backward (count >= 8): 0 | gather dy | 1 | R-side blocks | 2 | dG_R |
 *            3 | W0 product | 4 | P-side blocks | 5 | dG_P | 6 | scatter dx | 7
 * When two stages run in one kernel their shared boundary is recorded
 * twice, back to back.  With bf16 (b >= 64) the dG_R reduction runs in the
 * same launch as dG_P (for b = 64 and 128 only where that launch splits the
 * tokens): stage 2..3 is then empty and stage 5..6 holds both.
 * events = NULL clears the hook.
 * Errors: ERR_ARG (events non-NULL and count < 8).
 */
int32_t poetx_set_stage_events(void* const* events, int32_t count);

/*
 * poetx_set_fused_gather -- how the layer calls of this process run an
 * input-side gather and the block products that follow it ("POET-X ...",
 * technical summary 2.2: the index map reorders data as it is read; 2.3:
 * batched block products): the forward's U = x[:, pi_P], V = U G_P^T, the
 * backward's dS = dy[:, pi_R], dZ = dS G_R, and the memory-saving
 * backward's recompute of V.  on != 0: one pass that gathers straight into
 * the block products' operands, where the layer is bf16 with b = 256 and
 * the gathered width (n, or m for dy) is a multiple of 512 up to 4096;
 * 0 (the default): a gather pass, then a block pass.  Both forms are exact
 * on the gather and agree with each other to rounding (their block
 * products sum in different orders); on MI355X the one-pass form is the
 * slower of the two at the square 4096 workload.  Workspace sizes depend on
 * the setting: set it before sizing workspaces, and keep it between a
 * forward call and the backward call that uses its saved buffer.  Returns
 * the previous setting (0 or 1).
 */
int32_t poetx_set_fused_gather(int32_t on);

/* Scratch bytes for poetx_layer_fwd (which = 0), poetx_layer_bwd (1),
 * poetx_layer_fwd_xmem (2), poetx_layer_bwd_xmem (3) or poetx_merge (4);
 * 0 on bad arguments. */
size_t poetx_workspace_bytes(const poetx_shape* sh, int32_t which);

/* Bytes of the saved-activation buffer; 0 on bad arguments. */
size_t poetx_saved_bytes(const poetx_shape* sh);

#ifdef __cplusplus
}
#endif

#endif /* POETX_H */
