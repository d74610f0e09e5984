// Portable tiled kernels: any size, float32 or bf16 storage, fp32 arithmetic.
// They carry the float32 layer (fp32 storage has no MFMA-tiled variant here)
// and block sizes b <= 32, and they are the yardstick the MFMA kernels are
// tested beside.
#include "kernels.h"

namespace poetx {

namespace {

constexpr int TILE = 16;

// C[bt][i][j] = sum_k A[bt][i][k] * B[bt][j][k]; bkm: B given K-major,
// element (j, k) at B[bt][k * ldb + j]
template <typename TS>
__global__ __launch_bounds__(256) void k_simple_nt(int M, int N, int K, const TS* __restrict__ A,
                                                   long lda, long sA, const TS* __restrict__ B,
                                                   long ldb, long sB, TS* __restrict__ C, long ldc,
                                                   long sC, int bkm) {
  __shared__ float As[TILE][TILE + 1];
  __shared__ float Bs[TILE][TILE + 1];
  const int bt = blockIdx.z;
  A += bt * sA;
  B += bt * sB;
  C += bt * sC;
  const int tx = threadIdx.x % TILE, ty = threadIdx.x / TILE;
  const int i = blockIdx.y * TILE + ty;  // row of C
  const int j = blockIdx.x * TILE + tx;  // column of C
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += TILE) {
    int ar = blockIdx.y * TILE + ty, ac = k0 + tx;
    As[ty][tx] = (ar < M && ac < K) ? St<TS>::ld(A + ar * lda + ac) : 0.f;
    if (bkm) {  // row k0 + ty of the K-major B, coalesced along j
      const int kr = k0 + ty, jc = blockIdx.x * TILE + tx;
      Bs[tx][ty] = (jc < N && kr < K) ? St<TS>::ld(B + kr * ldb + jc) : 0.f;
    } else {
      const int br = blockIdx.x * TILE + ty, bc = k0 + tx;
      Bs[ty][tx] = (br < N && bc < K) ? St<TS>::ld(B + br * ldb + bc) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TILE; ++kk) acc += As[ty][kk] * Bs[tx][kk];
    __syncthreads();
  }
  if (i < M && j < N) St<TS>::st(C + i * ldc + j, acc);
}

// C[bt][i][j] = sum_k A[bt][k][i] * B[bt][k][j], float32 output
template <typename TS>
__global__ __launch_bounds__(256) void k_simple_tn(int M, int N, int K, const TS* __restrict__ A,
                                                   long lda, long sA, const TS* __restrict__ B,
                                                   long ldb, long sB, float* __restrict__ C,
                                                   long ldc, long sC) {
  __shared__ float As[TILE][TILE + 1];  // [k][i]
  __shared__ float Bs[TILE][TILE + 1];  // [k][j]
  const int bt = blockIdx.z;
  A += bt * sA;
  B += bt * sB;
  C += bt * sC;
  const int tx = threadIdx.x % TILE, ty = threadIdx.x / TILE;
  const int i = blockIdx.y * TILE + ty;
  const int j = blockIdx.x * TILE + tx;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += TILE) {
    int kr = k0 + ty;
    int ac = blockIdx.y * TILE + tx;
    As[ty][tx] = (kr < K && ac < M) ? St<TS>::ld(A + kr * lda + ac) : 0.f;
    int bc = blockIdx.x * TILE + tx;
    Bs[ty][tx] = (kr < K && bc < N) ? St<TS>::ld(B + kr * ldb + bc) : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TILE; ++kk) acc += As[kk][ty] * Bs[kk][tx];
    __syncthreads();
  }
  if (i < M && j < N) C[i * ldc + j] = acc;
}

constexpr int SMALL_B = 64;
constexpr int SP = SMALL_B + 1;  // LDS row pitch (floats)

// X <- alpha * Add + sgn * (L @ R) over b x b LDS matrices (row pitch SP)
__device__ __forceinline__ void small_step(int b, float* __restrict__ out, const float* L,
                                           const float* R, const float* Add, float alpha) {
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
    int i = e / b, j = e % b;
    float acc = alpha * Add[i * SP + j];
    for (int l = 0; l < b; ++l) acc += L[i * SP + l] * R[l * SP + j];
    out[i * SP + j] = acc;
  }
}

// Forward: U_k = Q; U_p = 2Q + Q U_{p+1} (p = k-1..0); G = I + U_0.
template <typename TS>
__global__ __launch_bounds__(256) void k_cnp_small_fwd(int b, int k, const float* __restrict__ theta,
                                                       TS* __restrict__ G, TS* __restrict__ GT) {
  __shared__ float Q[SMALL_B * SP], X[SMALL_B * SP], Xn[SMALL_B * SP];
  const int blk = blockIdx.x;
  const float* th = theta + (long)blk * (b * (b - 1) / 2);
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
    int i = e / b, j = e % b;
    float q = skew_at(th, i, j, b);
    Q[i * SP + j] = q;
    X[i * SP + j] = cnp_coef(k + 1, k) * q;
  }
  __syncthreads();
  float* cur = X;
  float* nxt = Xn;
  for (int p = k - 1; p >= 0; --p) {
    small_step(b, nxt, Q, cur, Q, cnp_coef(p + 1, k));
    __syncthreads();
    float* t = cur; cur = nxt; nxt = t;
  }
  TS* g = G + (long)blk * b * b;
  TS* gt = GT ? GT + (long)blk * b * b : nullptr;
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
    int i = e / b, j = e % b;
    float v = cur[i * SP + j] + (i == j ? 1.f : 0.f);
    St<TS>::st(g + i * b + j, v);
    if (gt) St<TS>::st(gt + j * b + i, v);
  }
}

// Backward.  With D = dG and w_p = c_p (-1)^{p-1}:
//   F_k = w_{k+1} D,  F_a = w_{a+1} D + F_{a+1} Q        (a = k-1..0)
//   Y_k = F_k,        Y_a = F_a + Q Y_{a+1};  gQ = Y_0
//   dtheta = triu1(gQ - gQ^T)
__global__ __launch_bounds__(256) void k_cnp_small_bwd(int b, int k, const float* __restrict__ theta,
                                                       const float* __restrict__ dG,
                                                       float* __restrict__ dtheta, int accumulate,
                                                       float* __restrict__ wsF) {
  __shared__ float Q[SMALL_B * SP], D[SMALL_B * SP], X[SMALL_B * SP], Xn[SMALL_B * SP];
  const int blk = blockIdx.x;
  const int tb = b * (b - 1) / 2;
  const float* th = theta + (long)blk * tb;
  const float* d = dG + (long)blk * b * b;
  float* F = wsF + (long)blk * k * b * b;  // F_a at F + a*b*b, a < k
  const float wk1 = cnp_wcoef(k + 1, k);
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
    int i = e / b, j = e % b;
    Q[i * SP + j] = skew_at(th, i, j, b);
    float dv = d[e];
    D[i * SP + j] = dv;
    X[i * SP + j] = wk1 * dv;
  }
  __syncthreads();
  float* cur = X;
  float* nxt = Xn;
  for (int a = k - 1; a >= 0; --a) {  // F chain: right multiplication by Q
    small_step(b, nxt, cur, Q, D, cnp_wcoef(a + 1, k));
    __syncthreads();
    for (int e = threadIdx.x; e < b * b; e += blockDim.x)
      F[(long)a * b * b + e] = nxt[(e / b) * SP + e % b];
    float* t = cur; cur = nxt; nxt = t;
  }
  __syncthreads();  // the last F store above still reads an LDS buffer
  // Y chain: left multiplication by Q; Y_k = F_k
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
    int i = e / b, j = e % b;
    X[i * SP + j] = wk1 * D[i * SP + j];
  }
  __syncthreads();
  cur = X;
  nxt = Xn;
  for (int a = k - 1; a >= 0; --a) {
    // F_a from global (written by this block above; visible after the barrier)
    for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
      int i = e / b, j = e % b;
      float acc = F[(long)a * b * b + e];
      for (int l = 0; l < b; ++l) acc += Q[i * SP + l] * cur[l * SP + j];
      nxt[i * SP + j] = acc;
    }
    __syncthreads();
    float* t = cur; cur = nxt; nxt = t;
  }
  float* dth = dtheta + (long)blk * tb;
  for (int e = threadIdx.x; e < b * b; e += blockDim.x) {
    int i = e / b, j = e % b;
    if (i < j) {
      float v = cur[i * SP + j] - cur[j * SP + i];
      int t = tri_index(i, j, b);
      dth[t] = accumulate ? dth[t] + v : v;
    }
  }
}

}  // namespace

template <typename TS>
hipError_t launch_simple_nt(int batch, int M, int N, int K, const TS* A, long lda, long sA,
                            const TS* B, long ldb, long sB, TS* C, long ldc, long sC,
                            hipStream_t s, bool bkmajor) {
  dim3 grid((N + TILE - 1) / TILE, (M + TILE - 1) / TILE, batch);
  hipLaunchKernelGGL(k_simple_nt<TS>, grid, dim3(256), 0, s, M, N, K, A, lda, sA, B, ldb, sB, C,
                     ldc, sC, bkmajor ? 1 : 0);
  return hipGetLastError();
}

template <typename TS>
hipError_t launch_simple_tn(int batch, int M, int N, int K, const TS* A, long lda, long sA,
                            const TS* B, long ldb, long sB, float* C, long ldc, long sC,
                            hipStream_t s) {
  dim3 grid((N + TILE - 1) / TILE, (M + TILE - 1) / TILE, batch);
  hipLaunchKernelGGL(k_simple_tn<TS>, grid, dim3(256), 0, s, M, N, K, A, lda, sA, B, ldb, sB, C,
                     ldc, sC);
  return hipGetLastError();
}

template <typename TS>
hipError_t launch_cnp_small_fwd(int nblk, int b, int k, const float* theta, TS* G, TS* GT,
                                hipStream_t s) {
  if (b > SMALL_B) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cnp_small_fwd<TS>, dim3(nblk), dim3(256), 0, s, b, k, theta, G, GT);
  return hipGetLastError();
}

hipError_t launch_cnp_small_bwd(int nblk, int b, int k, const float* theta, const float* dG,
                                float* dtheta, int accumulate, float* ws_F, hipStream_t s) {
  if (b > SMALL_B) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cnp_small_bwd, dim3(nblk), dim3(256), 0, s, b, k, theta, dG, dtheta,
                     accumulate, ws_F);
  return hipGetLastError();
}

template hipError_t launch_simple_nt<float>(int, int, int, int, const float*, long, long,
                                            const float*, long, long, float*, long, long,
                                            hipStream_t, bool);
template hipError_t launch_simple_nt<bf16>(int, int, int, int, const bf16*, long, long,
                                           const bf16*, long, long, bf16*, long, long,
                                           hipStream_t, bool);
template hipError_t launch_simple_tn<float>(int, int, int, int, const float*, long, long,
                                            const float*, long, long, float*, long, long,
                                            hipStream_t);
template hipError_t launch_simple_tn<bf16>(int, int, int, int, const bf16*, long, long,
                                           const bf16*, long, long, float*, long, long,
                                           hipStream_t);
template hipError_t launch_cnp_small_fwd<float>(int, int, int, const float*, float*, float*,
                                                hipStream_t);
template hipError_t launch_cnp_small_fwd<bf16>(int, int, int, const float*, bf16*, bf16*,
                                               hipStream_t);

}  // namespace poetx
