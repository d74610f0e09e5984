// Permutations as index maps ("POET-X ...", technical summary 2.2: data are
// reordered by index instead of multiplying by permutation matrices; two of
// the four forward permutations fold into the fixed weight).
//
// A column permutation of a token-major [rows][width] tensor gathers inside
// each row.  Rows up to 64 KB are staged in LDS with coalesced 16-byte loads,
// gathered from LDS and written back with coalesced 16-byte stores, so HBM
// sees one streaming read and one streaming write per element.
#include "kernels.h"

namespace poetx {

namespace {

constexpr int PERM_THREADS = 256;
constexpr int PERM_LDS_MAX = 64 * 1024;

template <typename E>
__device__ __forceinline__ void copy_row_to_lds(E* lds, const E* __restrict__ src, int width,
                                                bool vec) {
  if (vec) {
    const int nv = width * (int)sizeof(E) / 16;
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    u32x4* l4 = reinterpret_cast<u32x4*>(lds);
    for (int v = threadIdx.x; v < nv; v += blockDim.x) l4[v] = __builtin_nontemporal_load(s4 + v);
  } else {
    for (int c = threadIdx.x; c < width; c += blockDim.x) lds[c] = src[c];
  }
}

// out[r][c] = in[rmap ? rmap[r] : r][idx[c]]
template <typename E>
__global__ __launch_bounds__(PERM_THREADS) void k_permute_rows_lds(
    int rows, int width, const E* __restrict__ in, const int32_t* __restrict__ rmap,
    const int32_t* __restrict__ idx, E* __restrict__ out, int vec) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* row = reinterpret_cast<E*>(smem);
  constexpr int PER = 16 / sizeof(E);  // elements per 16-byte store
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const long src = rmap ? (long)rmap[r] : (long)r;
    copy_row_to_lds(row, in + src * width, width, vec);
    __syncthreads();
    E* dst = out + (long)r * width;
    if (vec) {
      const int nv = width / PER;
      for (int v = threadIdx.x; v < nv; v += blockDim.x) {
        E tmp[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) tmp[e] = row[idx[v * PER + e]];
        uint4 pk;
        __builtin_memcpy(&pk, tmp, 16);
        reinterpret_cast<uint4*>(dst)[v] = pk;
      }
    } else {
      for (int c = threadIdx.x; c < width; c += blockDim.x) dst[c] = row[idx[c]];
    }
    __syncthreads();
  }
}

// The main form: RPW rows per workgroup of NTHR threads, each thread owning
// up to MAXV 16-byte output vectors per row.  Every row load and the
// thread's indices (16-byte vector loads) go out before the first LDS write;
// one barrier, then each thread gathers its vectors of every row from LDS.
// Rows are read non-temporally; NTS: the stores too.
template <typename E, int NTHR, int RPW, int MAXV, bool NTS>
__global__ __launch_bounds__(NTHR) void k_permute_rows_v(int rows, int width,
                                                         const E* __restrict__ in,
                                                         const int32_t* __restrict__ rmap,
                                                         const int32_t* __restrict__ idx,
                                                         E* __restrict__ out) {
  extern __shared__ __align__(16) unsigned char smem[];
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  typedef __attribute__((ext_vector_type(4))) int32_t i32x4;
  constexpr int PER = 16 / sizeof(E);  // elements per vector
  constexpr int IV = PER / 4;          // index vectors per output vector
  const int nv = width / PER;
  const int r0 = blockIdx.x * RPW;
  u32x4 ld[RPW][MAXV];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const long src = r0 + rr < rows ? (rmap ? (long)rmap[r0 + rr] : (long)(r0 + rr)) : 0;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(in + src * width);
#pragma unroll
    for (int u = 0; u < MAXV; ++u) {
      const int v = u * NTHR + threadIdx.x;
      if (v < nv && r0 + rr < rows) ld[rr][u] = __builtin_nontemporal_load(s4 + v);
    }
  }
  i32x4 ix[MAXV][IV];
#pragma unroll
  for (int u = 0; u < MAXV; ++u) {
    const int v = u * NTHR + threadIdx.x;
#pragma unroll
    for (int h = 0; h < IV; ++h)
      if (v < nv) ix[u][h] = reinterpret_cast<const i32x4*>(idx)[v * IV + h];
  }
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
    for (int u = 0; u < MAXV; ++u) {
      const int v = u * NTHR + threadIdx.x;
      if (v < nv && r0 + rr < rows) reinterpret_cast<u32x4*>(smem + (size_t)rr * width * sizeof(E))[v] = ld[rr][u];
    }
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    if (r0 + rr >= rows) break;
    const E* row = reinterpret_cast<const E*>(smem + (size_t)rr * width * sizeof(E));
#pragma unroll
    for (int u = 0; u < MAXV; ++u) {
      const int v = u * NTHR + threadIdx.x;
      if (v < nv) {
        E t[PER];
#pragma unroll
        for (int h = 0; h < IV; ++h) {
          t[4 * h + 0] = row[ix[u][h].x];
          t[4 * h + 1] = row[ix[u][h].y];
          t[4 * h + 2] = row[ix[u][h].z];
          t[4 * h + 3] = row[ix[u][h].w];
        }
        u32x4 pk;
        __builtin_memcpy(&pk, t, 16);
        u32x4* dst = reinterpret_cast<u32x4*>(out + (long)(r0 + rr) * width) + v;
        if constexpr (NTS) __builtin_nontemporal_store(pk, dst);
        else *dst = pk;
      }
    }
  }
}

// rows too wide for LDS: gather straight from global memory
template <typename E>
__global__ __launch_bounds__(PERM_THREADS) void k_permute_rows_direct(
    int rows, int width, const E* __restrict__ in, const int32_t* __restrict__ rmap,
    const int32_t* __restrict__ idx, E* __restrict__ out) {
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const E* src = in + (rmap ? (long)rmap[r] : (long)r) * width;
    E* dst = out + (long)r * width;
    for (int c = threadIdx.x; c < width; c += blockDim.x) dst[c] = src[idx[c]];
  }
}

// out[j][i] = in[i][j], in: [m][n]
template <typename E>
__global__ __launch_bounds__(256) void k_transpose(int m, int n, const E* __restrict__ in,
                                                   E* __restrict__ out) {
  __shared__ E tile[32][33];
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 32 x 8
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  for (int y = ty; y < 32; y += 8) {
    int i = i0 + y, j = j0 + tx;
    if (i < m && j < n) tile[y][tx] = in[(long)i * n + j];
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    int j = j0 + y, i = i0 + tx;
    if (i < m && j < n) out[(long)j * m + i] = tile[tx][y];
  }
}

__global__ void k_inverse_perm(int n, const int32_t* __restrict__ p, int32_t* __restrict__ inv) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) inv[p[i]] = i;
}

template <typename E, int MAXV>
hipError_t permute_v_launch(int rows, int width, const void* in, const int32_t* rmap,
                            const int32_t* idx, void* out, bool nt_store, hipStream_t s) {
  constexpr int NTHR = 512, RPW = 2;
  const int grid = (rows + RPW - 1) / RPW;
  if (nt_store)
    hipLaunchKernelGGL((k_permute_rows_v<E, NTHR, RPW, MAXV, true>), dim3(grid), dim3(NTHR),
                       RPW * width * sizeof(E), s, rows, width, (const E*)in, rmap, idx, (E*)out);
  else
    hipLaunchKernelGGL((k_permute_rows_v<E, NTHR, RPW, MAXV, false>), dim3(grid), dim3(NTHR),
                       RPW * width * sizeof(E), s, rows, width, (const E*)in, rmap, idx, (E*)out);
  return hipGetLastError();
}

template <typename E>
hipError_t permute_impl(int rows, int width, const void* in, const int32_t* rmap,
                        const int32_t* idx, void* out, bool nt_store, hipStream_t s) {
  const size_t bytes = (size_t)width * sizeof(E);
  const int grid = rows < 65536 ? rows : 65536;
  const bool aligned = bytes % 16 == 0 && (uintptr_t)in % 16 == 0 && (uintptr_t)out % 16 == 0 &&
                       (uintptr_t)idx % 16 == 0;
  if (aligned && 2 * bytes <= PERM_LDS_MAX && rows < (1 << 30)) {
    const int nv = (int)(bytes / 16);
    if (nv <= 512) return permute_v_launch<E, 1>(rows, width, in, rmap, idx, out, nt_store, s);
    if (nv <= 1024) return permute_v_launch<E, 2>(rows, width, in, rmap, idx, out, nt_store, s);
    return permute_v_launch<E, 4>(rows, width, in, rmap, idx, out, nt_store, s);
  }
  if (bytes <= PERM_LDS_MAX) {
    int vec = (bytes % 16 == 0) && ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0);
    hipLaunchKernelGGL(k_permute_rows_lds<E>, dim3(grid), dim3(PERM_THREADS), bytes, s, rows,
                       width, (const E*)in, rmap, idx, (E*)out, vec);
  } else {
    hipLaunchKernelGGL(k_permute_rows_direct<E>, dim3(grid), dim3(PERM_THREADS), 0, s, rows,
                       width, (const E*)in, rmap, idx, (E*)out);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t transpose_impl(int m, int n, const void* in, void* out, hipStream_t s) {
  dim3 grid((n + 31) / 32, (m + 31) / 32);
  hipLaunchKernelGGL(k_transpose<E>, grid, dim3(256), 0, s, m, n, (const E*)in, (E*)out);
  return hipGetLastError();
}

__global__ void k_gather_f32(int n, const float* __restrict__ src, const int32_t* __restrict__ idx,
                             float* __restrict__ dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[idx[i]];
}

// out[r][c] = bf16(scale[r or c] * q[r][c]) for an int8 [rows][cols] matrix,
// 16 elements per thread; the scale follows rows (per_row) or columns
__global__ __launch_bounds__(256) void k_dequant_i8(long rows, int cols, const int8_t* __restrict__ q,
                                                    const float* __restrict__ scale, int per_row,
                                                    uint16_t* __restrict__ out) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const int vpr = cols / 16;
  const long v = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= rows * vpr) return;
  const long r = v / vpr;
  const int c0 = (int)(v % vpr) * 16;
  const u32x4 in = *reinterpret_cast<const u32x4*>(q + r * cols + c0);
  const int8_t* b = reinterpret_cast<const int8_t*>(&in);
  uint32_t w[8];
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const float s0 = per_row ? scale[r] : scale[c0 + e];
    const float s1 = per_row ? scale[r] : scale[c0 + e + 1];
    w[e / 2] = pack2bf(s0 * (float)b[e], s1 * (float)b[e + 1]);
  }
  u32x4* o = reinterpret_cast<u32x4*>(out + r * cols + c0);
  o[0] = (u32x4){w[0], w[1], w[2], w[3]};
  o[1] = (u32x4){w[4], w[5], w[6], w[7]};
}

}  // namespace

hipError_t launch_dequant_i8(long rows, int cols, const int8_t* q, const float* scale, int per_row,
                             bf16* out, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const long nv = rows * (cols / 16);
  hipLaunchKernelGGL(k_dequant_i8, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, s, rows, cols,
                     q, scale, per_row, out);
  return hipGetLastError();
}

// element sizes: 1 (int8 weights), 2 (bf16), 4 (fp32)
hipError_t launch_permute_rows_cols(int rows, int width, int es, const void* in,
                                    const int32_t* rmap, const int32_t* idx, void* out,
                                    hipStream_t s, bool nt_store) {
  if (rows <= 0 || width <= 0) return hipSuccess;
  if (es == 1) return permute_impl<uint8_t>(rows, width, in, rmap, idx, out, nt_store, s);
  if (es == 2) return permute_impl<uint16_t>(rows, width, in, rmap, idx, out, nt_store, s);
  return permute_impl<uint32_t>(rows, width, in, rmap, idx, out, nt_store, s);
}

hipError_t launch_permute_cols(int rows, int width, int es, const void* in, const int32_t* idx,
                               void* out, hipStream_t s, bool nt_store) {
  return launch_permute_rows_cols(rows, width, es, in, nullptr, idx, out, s, nt_store);
}

hipError_t launch_transpose(int m, int n, int es, const void* in, void* out, hipStream_t s) {
  if (m <= 0 || n <= 0) return hipSuccess;
  if (es == 1) return transpose_impl<uint8_t>(m, n, in, out, s);
  if (es == 2) return transpose_impl<uint16_t>(m, n, in, out, s);
  return transpose_impl<uint32_t>(m, n, in, out, s);
}

hipError_t launch_gather_f32(int n, const float* src, const int32_t* idx, float* dst,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_f32, dim3((n + 255) / 256), dim3(256), 0, s, n, src, idx, dst);
  return hipGetLastError();
}

hipError_t launch_fold(int m, int n, int es, const void* W0, const int32_t* pR,
                       const int32_t* pP, void* W0f, void* W0fT, int32_t* pRinv,
                       int32_t* pPinv, hipStream_t s) {
  hipError_t e = launch_permute_rows_cols(m, n, es, W0, pR, pP, W0f, s);
  if (e != hipSuccess) return e;
  if (W0fT && (e = launch_transpose(m, n, es, W0f, W0fT, s)) != hipSuccess) return e;
  if (pRinv) {
    hipLaunchKernelGGL(k_inverse_perm, dim3((m + 255) / 256), dim3(256), 0, s, m, pR, pRinv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (pPinv) {
    hipLaunchKernelGGL(k_inverse_perm, dim3((n + 255) / 256), dim3(256), 0, s, n, pP, pPinv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace poetx
