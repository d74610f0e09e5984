// bf16 MFMA GEMMs for the layer's dense contraction and its batched b x b
// block products ("POET-X ...", technical summary 2.1 input-centric form and
// 2.3 batch-parallel blocks: each block is an independent matrix product,
// the block-diagonal matrix is never built).
//
//   gemm_nt:  C[bt] = A[bt] B[bt]^T, A [M][K], B [N][K] (both K-contiguous),
//             bf16 in, fp32 accumulate, bf16 out.  Serves Z = V W0f^T,
//             dV = dZ W0f (B = W0f^T), and every per-token block product
//             (A = a b-column slice of the activations, B = G or G^T).
//   gemm_tn:  P[s][bt] = sum over a token range of A^T B, A [T][*] and
//             B [T][*] token-major, fp32 partial sums (dG = dS^T Z and
//             dG_P = dV^T U); a fixed-order reduction over s follows.
//
// One workgroup = 4 wave64s in a 2 x 2 grid, tile BM x BN, K in slabs of 64
// staged through LDS (double buffered, one barrier per slab).  LDS rows hold
// 64 bf16 (128 B) as eight 16-byte chunks, chunk c of row r stored at
// position c ^ ((r ^ r/8) & 7): MFMA operand reads (16 rows, one chunk) and
// both the row-wise (NT) and the transposing (TN) tile writes are free of
// bank conflicts.
// MFMA: v_mfma_f32_32x32x16_bf16; lane l holds A[l%32][8*(l/32)+i] and
// B[8*(l/32)+i][l%32]; acc[r] = D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include <algorithm>

#include "kernels.h"

namespace poetx {

namespace {

constexpr int BK = 64;
constexpr int ROWB = BK * 2;  // bytes per LDS row
constexpr int NTHR = 256;

__device__ __forceinline__ int lds_off(int r, int c) {
  return r * ROWB + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
}

template <int BM, int BN>
struct Cfg {
  static constexpr int TM = BM / 2, TN = BN / 2;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int STAGE = (BM + BN) * ROWB;
  static constexpr int LDS = 2 * STAGE;
  static_assert(FM >= 1 && FN >= 1, "tile too small");
};

// acc += A_slab(rows of this wave) * B_slab(rows of this wave)^T over BK
template <int BM, int BN>
__device__ __forceinline__ void mma_slab(const char* __restrict__ As, const char* __restrict__ Bs,
                                         f32x16_t (&acc)[Cfg<BM, BN>::FM][Cfg<BM, BN>::FN],
                                         int wm, int wn, int lane) {
  using C = Cfg<BM, BN>;
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int c = ks * 2 + lane / 32;
    bf16x8_t a[C::FM], b[C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      a[i] = as_bf16x8(*reinterpret_cast<const uint4*>(As + lds_off(wm * C::TM + i * 32 + lane % 32, c)));
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      b[j] = as_bf16x8(*reinterpret_cast<const uint4*>(Bs + lds_off(wn * C::TN + j * 32 + lane % 32, c)));
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
  }
}

// XCD-aware order: consecutive workgroup ids are dealt round-robin over the
// 8 XCDs; renumber so each XCD gets a contiguous range of tiles, then walk
// tiles in groups of GROUP tile-rows so neighbours share A and B panels.
__device__ __forceinline__ void tile_of(int wg, int nwg, int tilesM, int tilesN, int& tm, int& tn) {
  constexpr int XCD = 8, GROUP = 8;
  int pid = wg;
  if (nwg % XCD == 0) pid = (wg % XCD) * (nwg / XCD) + wg / XCD;
  const int per_group = GROUP * tilesN;
  const int g = pid / per_group;
  const int first = g * GROUP;
  const int gm = min(tilesM - first, GROUP);
  const int in = pid % per_group;
  tm = first + in % gm;
  tn = in / gm;
}

template <int BM, int BN>
__global__ __launch_bounds__(NTHR, 1) void k_gemm_nt(int M, int N, int K, const bf16* __restrict__ A,
                                                     long lda, long sA, const bf16* __restrict__ B,
                                                     long ldb, long sB, bf16* __restrict__ Cm,
                                                     long ldc, long sC, int tilesM, int tilesN) {
  using C = Cfg<BM, BN>;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const long bt = blockIdx.y;
  A += bt * sA;
  B += bt * sB;
  Cm += bt * sC;

  // loader: 8 threads per 128-byte row slab, 32 rows per pass
  constexpr int PA = BM / 32, PB = BN / 32;
  const int lr = tid / 8, lc = tid % 8;
  uint4 ra0[PA], rb0[PB];
  auto gload = [&](uint4 (&ra)[PA], uint4 (&rb)[PB], int k0) {
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int row = m0 + p * 32 + lr;
      ra[p] = row < M ? *reinterpret_cast<const uint4*>(A + row * lda + k0 + lc * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int row = n0 + p * 32 + lr;
      rb[p] = row < N ? *reinterpret_cast<const uint4*>(B + row * ldb + k0 + lc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](const uint4 (&ra)[PA], const uint4 (&rb)[PB], int buf) {
    char* As = smem + buf * C::STAGE;
    char* Bs = As + C::A_BYTES;
#pragma unroll
    for (int p = 0; p < PA; ++p) *reinterpret_cast<uint4*>(As + lds_off(p * 32 + lr, lc)) = ra[p];
#pragma unroll
    for (int p = 0; p < PB; ++p) *reinterpret_cast<uint4*>(Bs + lds_off(p * 32 + lr, lc)) = rb[p];
  };

  f32x16_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = (f32x16_t){};

  const int nk = K / BK;
  gload(ra0, rb0, 0);
  sstore(ra0, rb0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(ra0, rb0, (kt + 1) * BK);
    const char* As = smem + cur * C::STAGE;
    mma_slab<BM, BN>(As, As + C::A_BYTES, acc, wm, wn, lane);
    if (kt + 1 < nk) sstore(ra0, rb0, cur ^ 1);
    __syncthreads();
  }

  // epilogue: pair lanes l, l^1 so each stores two adjacent bf16 (4 bytes)
  const bool odd = lane & 1;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float v0 = acc[i][j][r], v1 = acc[i][j][r + 1];
        const float got = __shfl_xor(odd ? v0 : v1, 1);
        const int row = m0 + wm * C::TM + i * 32 + acc_row(r, lane) + (odd ? 1 : 0);
        const int col = n0 + wn * C::TN + j * 32 + (lane % 32) - (odd ? 1 : 0);
        const uint32_t pk = odd ? pack2bf(got, v1) : pack2bf(v0, got);
        if (row < M && col < N) *reinterpret_cast<uint32_t*>(Cm + row * ldc + col) = pk;
      }
}

// Partial token reduction: P[s][bt][r][c] = sum_{t in split s} A[t][r] B[t][c]
// (A, B token-major, column offsets folded into the pointers per batch).
template <int BT>
__global__ __launch_bounds__(NTHR, 1) void k_gemm_tn(int T, int tsplit, int tiles1,
                                                     const bf16* __restrict__ A, long lda, long sA,
                                                     const bf16* __restrict__ B, long ldb, long sB,
                                                     float* __restrict__ P, long ldp, long sP,
                                                     long sS) {
  using C = Cfg<BT, BT>;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
  const int tm = blockIdx.x / tiles1, tn = blockIdx.x % tiles1;
  const long bt = blockIdx.y;
  const int s = blockIdx.z;
  A += bt * sA + tm * BT;
  B += bt * sB + tn * BT;
  P += s * sS + bt * sP;
  const int t_begin = s * tsplit, t_end = min(T, t_begin + tsplit);

  // loader: a wave covers 8 tokens x 8 16-byte feature chunks; the LDS write
  // transposes to [feature][token]
  constexpr int COMBOS = 8 * (BT / 64);  // (token group, 64-feature group) pairs
  constexpr int PASSES = (COMBOS + 3) / 4;
  const int tl = lane / 8, fcl = lane % 8;
  uint4 ra[PASSES], rb[PASSES];
  auto gload = [&](int t0) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int ci = p * 4 + wave;
      const int t = t0 + (ci % 8) * 8 + tl;
      const int f = ((ci / 8) * 8 + fcl) * 8;
      const bool ok = ci < COMBOS && t < t_end;
      ra[p] = ok ? *reinterpret_cast<const uint4*>(A + (long)t * lda + f) : make_uint4(0, 0, 0, 0);
      rb[p] = ok ? *reinterpret_cast<const uint4*>(B + (long)t * ldb + f) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    char* As = smem + buf * C::STAGE;
    char* Bs = As + C::A_BYTES;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int ci = p * 4 + wave;
      if (ci >= COMBOS) continue;
      const int tk = (ci % 8) * 8 + tl;  // token within the slab
      const int r0 = ((ci / 8) * 8 + fcl) * 8;
      const uint16_t* ea = reinterpret_cast<const uint16_t*>(&ra[p]);
      const uint16_t* eb = reinterpret_cast<const uint16_t*>(&rb[p]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int off = lds_off(r0 + i, tk / 8) + (tk % 8) * 2;
        *reinterpret_cast<uint16_t*>(As + off) = ea[i];
        *reinterpret_cast<uint16_t*>(Bs + off) = eb[i];
      }
    }
  };

  f32x16_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = (f32x16_t){};

  const int nk = (t_end - t_begin + BK - 1) / BK;
  if (nk > 0) {
    gload(t_begin);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(t_begin + (kt + 1) * BK);
      const char* As = smem + cur * C::STAGE;
      mma_slab<BT, BT>(As, As + C::A_BYTES, acc, wm, wn, lane);
      if (kt + 1 < nk) sstore(cur ^ 1);
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = tm * BT + wm * C::TM + i * 32 + acc_row(r, lane);
        const int col = tn * BT + wn * C::TN + j * 32 + lane % 32;
        P[row * ldp + col] = acc[i][j][r];
      }
}

// out[e] = sum_{s < S} P[s * stride + e], fixed order
__global__ void k_reduce_splits(long n, int S, long stride, const float* __restrict__ P,
                                float* __restrict__ out) {
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    float acc = P[e];
    for (int s = 1; s < S; ++s) acc += P[s * stride + e];
    out[e] = acc;
  }
}

template <typename K>
hipError_t set_lds(K kern, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int BM, int BN>
hipError_t nt_launch(int batch, int M, int N, int K, const bf16* A, long lda, long sA, const bf16* B,
                     long ldb, long sB, bf16* C, long ldc, long sC, hipStream_t s) {
  auto kern = k_gemm_nt<BM, BN>;
  static const hipError_t attr = set_lds(kern, Cfg<BM, BN>::LDS);
  if (attr != hipSuccess) return attr;
  const int tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
  constexpr int lds = Cfg<BM, BN>::LDS;
  hipLaunchKernelGGL(kern, dim3(tilesM * tilesN, batch), dim3(NTHR), lds, s, M, N, K,
                     A, lda, sA, B, ldb, sB, C, ldc, sC, tilesM, tilesN);
  return hipGetLastError();
}

template <int BT>
hipError_t tn_launch(int batch, int D, int T, int S, const bf16* A, long lda, long sA, const bf16* B,
                     long ldb, long sB, float* P, long ldp, long sP, long sS, hipStream_t s) {
  auto kern = k_gemm_tn<BT>;
  static const hipError_t attr = set_lds(kern, Cfg<BT, BT>::LDS);
  if (attr != hipSuccess) return attr;
  const int tiles1 = D / BT;
  const int tsplit = ((T + S - 1) / S + BK - 1) / BK * BK;
  constexpr int lds = Cfg<BT, BT>::LDS;
  hipLaunchKernelGGL(kern, dim3(tiles1 * tiles1, batch, S), dim3(NTHR), lds, s, T,
                     tsplit, tiles1, A, lda, sA, B, ldb, sB, P, ldp, sP, sS);
  return hipGetLastError();
}

constexpr int NUM_CU = 256;

}  // namespace

bool mfma_nt_ok(int M, int N, int K) { return M > 0 && N % 64 == 0 && K % BK == 0; }

hipError_t launch_mfma_nt(int batch, int M, int N, int K, const bf16* A, long lda, long sA,
                          const bf16* B, long ldb, long sB, bf16* C, long ldc, long sC,
                          hipStream_t s) {
  auto tiles = [&](int bm, int bn) { return (long)batch * ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (N % 256 == 0 && tiles(256, 256) >= NUM_CU)
    return nt_launch<256, 256>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s);
  if (N % 128 == 0 && tiles(256, 128) >= NUM_CU)
    return nt_launch<256, 128>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s);
  if (N % 128 == 0)
    return nt_launch<128, 128>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s);
  return nt_launch<128, 64>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s);
}

// splits of the token range for a D x D (per batch) reduction
int tn_splits(int batch, int D, int T) {
  const int BT = D >= 128 ? 128 : 64;
  const long tiles = (long)batch * (D / BT) * (D / BT);
  int S = (int)((NUM_CU + tiles - 1) / tiles);
  const int max_s = (T + 255) / 256;  // keep >= 256 tokens per split
  S = S < max_s ? S : max_s;
  return S < 1 ? 1 : S;
}

size_t tn_partial_bytes(int batch, int D, int T) {
  const int S = tn_splits(batch, D, T);
  return S > 1 ? (size_t)S * batch * D * D * sizeof(float) : 0;
}

hipError_t launch_mfma_tn(int batch, int D, int T, const bf16* A, long lda, long sA, const bf16* B,
                          long ldb, long sB, float* out, float* partials, hipStream_t s) {
  const int S = tn_splits(batch, D, T);
  const long dd = (long)D * D;
  float* P = S > 1 ? partials : out;
  hipError_t e;
  if (D == 64)
    e = tn_launch<64>(batch, D, T, S, A, lda, sA, B, ldb, sB, P, D, dd, dd * batch, s);
  else
    e = tn_launch<128>(batch, D, T, S, A, lda, sA, B, ldb, sB, P, D, dd, dd * batch, s);
  if (e != hipSuccess || S == 1) return e;
  const long n = dd * batch;
  const int grid = (int)std::min<long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_reduce_splits, dim3(grid), dim3(256), 0, s, n, S, n, P, out);
  return hipGetLastError();
}

}  // namespace poetx
