// Host-side launchers of the POET-X kernels (internal to libpoetx.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace poetx {

// Coefficients of G = sum_p c_p Q^p = (I+Q)(I + ... + Q^k):
// c_0 = 1, c_p = 2 for 1 <= p <= k, c_{k+1} = 1.
__host__ __device__ inline float cnp_coef(int p, int k) {
  if (p == 0 || p == k + 1) return 1.0f;
  return 2.0f;
}
// Backward weights w_p = c_p (-1)^{p-1} (Q^T = -Q folds the transposes).
__host__ __device__ inline float cnp_wcoef(int p, int k) {
  return ((p - 1) & 1) ? -cnp_coef(p, k) : cnp_coef(p, k);
}

// Lets `kern` use `bytes` of dynamic LDS on the calling thread's current
// device (needed above 64 KB).  The attribute belongs to the (kernel,
// device) pair, so it is set once per pair and size; later calls return the
// first call's status (api.hip).
hipError_t lds_opt_in(const void* kern, int bytes);

// ---- permutations (perm.hip); es = element bytes 1 | 2 | 4 ----------------
hipError_t launch_fold(int m, int n, int es, const void* W0, const int32_t* pR,
                       const int32_t* pP, void* W0f, void* W0fT, int32_t* pRinv,
                       int32_t* pPinv, hipStream_t s);
// out[r][c] = in[r][idx[c]] for r < rows, c < width; es = element bytes (2|4);
// nt_store: non-temporal stores (for an output that the next kernel does
// not read; plain stores leave it in the last-level cache for that kernel)
hipError_t launch_permute_cols(int rows, int width, int es, const void* in,
                               const int32_t* idx, void* out, hipStream_t s,
                               bool nt_store = true);
// out[r][c] = in[rmap[r]][idx[c]] ([rows][width], es = element bytes 2|4)
hipError_t launch_permute_rows_cols(int rows, int width, int es, const void* in,
                                    const int32_t* rmap, const int32_t* idx, void* out,
                                    hipStream_t s, bool nt_store = true);
// out[j][i] = in[i][j], in [m][n]
hipError_t launch_transpose(int m, int n, int es, const void* in, void* out, hipStream_t s);
// out = bf16(scale * q) for int8 q [rows][cols] (cols % 16 == 0); the scale
// is indexed by row (per_row) or by column
hipError_t launch_dequant_i8(long rows, int cols, const int8_t* q, const float* scale, int per_row,
                             bf16* out, hipStream_t s);
// dst[i] = src[idx[i]], i < n
hipError_t launch_gather_f32(int n, const float* src, const int32_t* idx, float* dst,
                             hipStream_t s);

// ---- portable tiled kernels (simple.hip) ----------------------------------
// C[bt][i][j] = sum_k A[bt][i][k] * B[bt][j][k]       (row-major, fp32 accumulate);
// bkmajor: B given K-major, element (j, k) at B[bt][k * ldb + j]
template <typename TS>
hipError_t launch_simple_nt(int batch, int M, int N, int K, const TS* A, long lda,
                            long sA, const TS* B, long ldb, long sB, TS* C, long ldc,
                            long sC, hipStream_t s, bool bkmajor = false);
// C[bt][i][j] = sum_k A[bt][k][i] * B[bt][k][j]       (float32 output)
template <typename TS>
hipError_t launch_simple_tn(int batch, int M, int N, int K, const TS* A, long lda,
                            long sA, const TS* B, long ldb, long sB, float* C, long ldc,
                            long sC, hipStream_t s);
// Cayley-Neumann forward/backward for b <= 64: one workgroup per block, the
// block resident in LDS, fp32 arithmetic.
template <typename TS>
hipError_t launch_cnp_small_fwd(int nblk, int b, int k, const float* theta, TS* G, TS* GT,
                                hipStream_t s);
hipError_t launch_cnp_small_bwd(int nblk, int b, int k, const float* theta, const float* dG,
                                float* dtheta, int accumulate, float* ws_F, hipStream_t s);

// ---- bf16 MFMA GEMMs (gemm_mfma.hip) --------------------------------------
// usable when N % 64 == 0 and K % 64 == 0 (M any)
bool mfma_nt_ok(int M, int N, int K);
// C[bt] = A[bt] B[bt]^T; A [M][K] (row pitch lda), B [N][K] (ldb), C [M][N] (ldc);
// cscale (or null): column c of C[bt] scaled by cscale[bt * sS + c] before rounding
hipError_t launch_mfma_nt(int batch, int M, int N, int K, const bf16* A, long lda, long sA,
                          const bf16* B, long ldb, long sB, bf16* C, long ldc, long sC,
                          hipStream_t s, const float* cscale = nullptr, long sS = 0);
// C = A B^T as above (one batch) and, per b-column block g of C (b = 256 or
// 128), E[:, g] = C[:, g] Bk[g]^T with Bk [N/b][b][b].
// E == nullptr: C only, from the same main loop (bitwise the same C).
bool mfma_nt_block_ok(int M, int N, int K, int b);
// ntmask: bit 0 stores C, bit 1 stores E non-temporally (outputs no kernel
// reads soon; they then take no room in the last-level cache).
hipError_t launch_mfma_nt_block(int M, int N, int K, int b, const bf16* A, long lda,
                                const bf16* B, long ldb, bf16* C, long ldc, const bf16* Bk,
                                bf16* E, long lde, hipStream_t s, int ntmask = 0);
// C = A B^T with B given K-major, Bkn = B^T [K][N] (row pitch ldb >= N):
// the dense product of the backward, dV = dZ W0f, read from W0f itself;
// bitwise the result of launch_mfma_nt_block on the transposed copy, block
// epilogue included.  N % 256 == 0, K % 64 == 0, K ldb 2 < 2^31.
bool mfma_nt_kmajor_ok(int M, int N, int K, long lda, long ldb, long ldc);
hipError_t launch_mfma_nt_kmajor(int M, int N, int K, int b, const bf16* A, long lda,
                                 const bf16* Bkn, long ldb, bf16* C, long ldc, const bf16* Bk,
                                 bf16* E, long lde, hipStream_t s, int ntmask = 0);
// C = (A Bq^T) diag(cscale) for an int8 Bq [N][K] (row pitch ldb bytes): the
// dense product on a quantized weight, widened to bf16 inside the kernel's
// operand path (exact) with the per-row weight scale applied to the fp32
// sums; with E, the block epilogue of launch_mfma_nt_block on the scaled C.
bool mfma_nt_q_ok(int M, int N, int K, long lda, long ldb, long ldc);
hipError_t launch_mfma_nt_q(int M, int N, int K, int b, const bf16* A, long lda, const int8_t* Bq,
                            long ldb, bf16* C, long ldc, const float* cscale, const bf16* Bk,
                            bf16* E, long lde, hipStream_t s, int ntmask = 0);
// per-token block products for b in {128, 256}:
// Out[t][j b + n] = sum_k A[t][j b + k] G[j][n][k]  (A, Out row pitch `width`),
// column c of Out scaled by cscale[c] before rounding when cscale is set
bool mfma_blocks_ok(int b);
hipError_t launch_mfma_blocks(int nblk, int T, int width, int b, const bf16* A, const bf16* G,
                              bf16* Out, hipStream_t s, const float* cscale = nullptr);
// out[bt][r][c] = sum_t A[t][bt*sA + r] B[t][bt*sB + c], D x D per batch,
// D in {64, 128, 256, 512}; partials: tn_partial_bytes(batch, D, T,
// max(lda, ldb)) bytes.  D >= 256: sA = sB = D; the token splits are sized
// so that one split of the widest operand spans under 2^31 bytes.
hipError_t launch_mfma_tn(int batch, int D, int T, const bf16* A, long lda, long sA, const bf16* B,
                          long ldb, long sB, float* out, float* partials, hipStream_t s);
size_t tn_partial_bytes(int batch, int D, int T, long width);
// two such reductions in one launch (D = 64, 128 or a multiple of 256,
// sA = sB = D):
// out0 over nb0 blocks of (A0, B0), out1 over nb1 blocks of (A1, B1);
// partials: tn_partial_bytes(nb0 + nb1, D, T, widest pitch) bytes (none
// when the launch does not split the tokens).  b = 64 and 128 only where it
// does (mfma_tn2_ok, width = the widest of the four pitches).
bool mfma_tn2_ok(int nb0, int nb1, int D, int T, long width);
hipError_t launch_mfma_tn2(int nb0, int nb1, int D, int T, const bf16* A0, long lda0,
                           const bf16* B0, long ldb0, float* out0, const bf16* A1, long lda1,
                           const bf16* B1, long ldb1, float* out1, float* partials,
                           hipStream_t s);

// ---- gather-fused block products (gather_blocks.hip), bf16, b = 256 ------
// Ug[t][c] = A[t][perm[c]] (perm null: the identity; Ug null: not stored)
// and Out[t][256 j + n] = sum_k Ug[t][256 j + k] G[j][n][k], column c of Out
// scaled by cscale[c] before rounding when cscale is set; A, Ug, Out [T][W].
// Gf: gather_blocks_ws_bytes(W, b) bytes of scratch (G in operand-fragment
// order).  W a multiple of 512 up to 4096 (gather_blocks_ok).
bool gather_blocks_ok(int W, int b);
size_t gather_blocks_ws_bytes(int W, int b);
hipError_t launch_gather_blocks(int T, int W, const bf16* A, const int32_t* perm, bf16* Ug,
                                const bf16* G, bf16* Gf, bf16* Out, const float* cscale,
                                hipStream_t s);

// ---- MFMA Cayley-Neumann panels (cnp_mfma.hip), bf16, b in {64..512} -------
// ws_Q: nblk*b*b bf16 scratch holding the unpacked skew blocks.
hipError_t launch_cnp_panel_fwd(int nblk, int b, int k, const float* theta, bf16* G,
                                bf16* GT, bf16* ws_Q, hipStream_t s);
// ws_Q as above; ws_F: k*nblk*b*b bf16; ws_dQ: nblk*b*b float.  q_ready:
// ws_Q already holds the unpacked Q of theta (left by launch_cnp_panel_fwd).
hipError_t launch_cnp_panel_bwd(int nblk, int b, int k, const float* theta, const float* dG,
                                float* dtheta, int accumulate, bf16* ws_Q, bf16* ws_F,
                                float* ws_dQ, bool q_ready, hipStream_t s);

}  // namespace poetx
