// Gather-fused block products for b = 256 ("POET-X ...", technical summary
// 2.2: the index map reorders the data as it is read, no permutation matrix;
// 2.3: the blocks are independent products, run as one batch):
//
//   Ug[t][c]             = A[t][perm[c]]                    (perm null: A)
//   Out[t][256 j + n]    = sum_k Ug[t][256 j + k] G_j[n][k]
//
// the forward's V = x[:, pi_P] G_P^T (Ug = U, kept for the dG_P reduction)
// and the backward's dZ = dy[:, pi_R] G_R (G := G_R^T, Ug = dS, kept for the
// dG_R reduction), in one pass over A.
//
// A block's 256 columns are spread over the whole row, so a workgroup takes
// whole rows: 32 tokens, staged 16 rows at a time in LDS by LDS-DMA (row
// pitch 2W + 16 bytes, which starts consecutive rows four banks apart).  Each
// lane gathers its MFMA operand fragments for its wave's blocks straight
// out of LDS (2-byte reads at perm's offsets) into registers, and stores
// the same 16 bytes to Ug.  The 32 tokens' fragments of a wave's two blocks
// (128 registers) then meet G_j, which streams from L2 in fragment order:
// one contiguous KB per operand fragment, laid out by k_gfrag just before.
// Every G byte fetched feeds 32 tokens; x is read once, Ug and Out written
// once, so the pass moves 3 T W 2 bytes against the 4 T W 2 of a gather pass
// followed by a block pass; but G crosses from L2 once per 32 tokens, and at
// one 32-token group per CU the row loads, gathers and products run in
// sequence.  The layer calls take this form only when poetx_set_fused_gather
// selects it; the gather pass and block pass are the default.
//
// MFMA: v_mfma_f32_16x16x32_bf16 with the G fragment first: lane l holds
// G_j[16 nf + l%16][32 ks + 8 (l/16) + e] and Ug[t0 + l%16][256 j + 32 ks +
// 8 (l/16) + e], e < 8, so the accumulator's lane l holds Out for token
// l%16 at columns 16 nf + 4 (l/16) + r, r < 4.
#include "kernels.h"

namespace poetx {

namespace {

constexpr int GB_B = 256;              // block size
constexpr int GB_TOK = 32;             // tokens per workgroup
constexpr int GB_RS = 16;              // token rows per LDS stage
constexpr int GB_NTH = 512;            // 8 waves; wave w owns blocks w and w + 8
constexpr int GB_KS = GB_B / 32;       // K-steps of 32 per block
constexpr int GB_NF = GB_B / 16;       // 16-column output fragments per block
constexpr int GB_WMAX = 4096;          // widest row (16 rows of 8 KB staged)

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Gf[((j GB_NF + nf) GB_KS + ks) 64 + l][e] = G[j][16 nf + l%16][32 ks + 8 (l/16) + e]:
// one thread per 16-byte chunk of Gf
__global__ __launch_bounds__(256) void k_gfrag(int nchunks, const bf16* __restrict__ G,
                                               bf16* __restrict__ Gf) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunks) return;
  const int l = c % 64, ks = (c / 64) % GB_KS, nf = (c / (64 * GB_KS)) % GB_NF;
  const long j = c / (64 * GB_KS * GB_NF);
  const uint4 v = *reinterpret_cast<const uint4*>(
      G + (j * GB_B + nf * 16 + l % 16) * GB_B + 32 * ks + 8 * (l / 16));
  reinterpret_cast<uint4*>(Gf)[c] = v;
}

// GATHER false: perm is the identity (the memory-saving backward's recompute
// of V from the saved U, bitwise the forward's V)
template <bool GATHER>
__global__ __launch_bounds__(GB_NTH, 1) void k_gather_blocks(
    int T, int W, const bf16* __restrict__ A, const int32_t* __restrict__ perm,
    bf16* __restrict__ Ug, const bf16* __restrict__ Gf, bf16* __restrict__ Out,
    const float* __restrict__ cscale) {
  extern __shared__ __align__(16) char smem[];
  const int pitch = 2 * W + 16;  // LDS bytes per staged row
  int* pofs = reinterpret_cast<int*>(smem + GB_RS * pitch);  // 2 perm[c]: byte offset in a row
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int r = lane % 16, g = lane / 16;
  const int nblk = W / GB_B;
  const int t0 = blockIdx.x * GB_TOK;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  if constexpr (GATHER) {
    typedef __attribute__((ext_vector_type(4))) int32_t i32x4;
    for (int v = tid; v < W / 4; v += GB_NTH) {
      const i32x4 p = reinterpret_cast<const i32x4*>(perm)[v];
      reinterpret_cast<i32x4*>(pofs)[v] = p * 2;
    }
  }

  bf16x8_t uf[2][GB_KS][2];  // [block of the wave][K-step][token half]
  const int cpr = W / 8;     // 16-byte chunks per row
  const int ndma = W / 256;  // DMA instructions per wave per stage (16 rows x cpr chunks / 64 / 8)
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row0 = t0 + q * GB_RS;
    const int nrows = min(GB_RS, T - row0);  // the same for the whole workgroup
    if (q == 1) {
      // every wave's reads of stage 0 are complete before stage 1 lands
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (nrows > 0) {
      // rows past T are outside the buffer range and land as zeros
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(A + (long)row0 * W), (short)0, nrows * W * 2, 0x00020000);
      for (int i = 0; i < ndma; ++i) {
        // 64 consecutive chunks of one row (cpr is a multiple of 64)
        const int p0 = (i * 8 + wave) * 64;
        const int row = p0 / cpr, c0 = p0 % cpr;
        const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds0 + row * pitch + c0 * 16);
        const int vo = row * W * 2 + (c0 + lane) * 16;
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v),
                     "v"(vo), "s"(rs)
                     : "memory");
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const char* rowp = smem + r * pitch;
    const int trow = row0 + r;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = wave + 8 * jj;
      if (j < nblk) {
#pragma unroll
        for (int ks = 0; ks < GB_KS; ++ks) {
          const int c0 = j * GB_B + 32 * ks + 8 * g;  // first of the lane's 8 columns
          int o[8];
          if constexpr (GATHER) {
            const int4 a = *reinterpret_cast<const int4*>(pofs + c0);
            const int4 b = *reinterpret_cast<const int4*>(pofs + c0 + 4);
            o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
            o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 2 * (c0 + e);
          }
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = *reinterpret_cast<const uint16_t*>(rowp + o[2 * e]);
            const uint32_t hi = *reinterpret_cast<const uint16_t*>(rowp + o[2 * e + 1]);
            w[e] = lo | (hi << 16);
          }
          const uint4 v = make_uint4(w[0], w[1], w[2], w[3]);
          uf[jj][ks][q] = as_bf16x8(v);
          if (Ug && trow < T) *reinterpret_cast<uint4*>(Ug + (long)trow * W + c0) = v;
        }
      }
    }
  }

  // the column scales replace the index table in LDS (read there, they do
  // not wait behind the G loads in the vector-memory counter)
  float* lsc = reinterpret_cast<float*>(pofs);
  if (cscale) {
    __syncthreads();  // every wave is done with the index table
    for (int v = tid; v < W / 4; v += GB_NTH)
      reinterpret_cast<float4*>(lsc)[v] = reinterpret_cast<const float4*>(cscale)[v];
    __syncthreads();
  }

  // the block products, G fragments double-buffered from L2
  const uint4* Gv = reinterpret_cast<const uint4*>(Gf);
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int j = wave + 8 * jj;
    if (j >= nblk) break;
    const uint4* Gj = Gv + (long)j * GB_NF * GB_KS * 64 + lane;
    uint4 gb[2][GB_KS];
#pragma unroll
    for (int ks = 0; ks < GB_KS; ++ks) gb[0][ks] = Gj[ks * 64];
#pragma unroll 2
    for (int nf = 0; nf < GB_NF; ++nf) {
      if (nf + 1 < GB_NF) {
#pragma unroll
        for (int ks = 0; ks < GB_KS; ++ks) gb[(nf + 1) & 1][ks] = Gj[((nf + 1) * GB_KS + ks) * 64];
      }
      f32x4_t acc[2] = {};
#pragma unroll
      for (int ks = 0; ks < GB_KS; ++ks) {
        const bf16x8_t a = as_bf16x8(gb[nf & 1][ks]);
        acc[0] = mfma16x16x32(a, uf[jj][ks][0], acc[0]);
        acc[1] = mfma16x16x32(a, uf[jj][ks][1], acc[1]);
      }
      const int col = j * GB_B + nf * 16 + 4 * g;
      float sc[4] = {1.f, 1.f, 1.f, 1.f};
      if (cscale) {
        const float4 s4 = *reinterpret_cast<const float4*>(lsc + col);
        sc[0] = s4.x; sc[1] = s4.y; sc[2] = s4.z; sc[3] = s4.w;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int t = t0 + q * GB_RS + r;
        if (t < T) {
          const uint2 o = make_uint2(pack2bf(acc[q][0] * sc[0], acc[q][1] * sc[1]),
                                     pack2bf(acc[q][2] * sc[2], acc[q][3] * sc[3]));
          *reinterpret_cast<uint2*>(Out + (long)t * W + col) = o;
        }
      }
    }
  }
}

hipError_t gb_set_lds(const void* kern, int bytes) {
  return lds_opt_in(kern, bytes);
}

}  // namespace

bool gather_blocks_ok(int W, int b) {
  return b == GB_B && W >= 512 && W <= GB_WMAX && W % 512 == 0;
}

size_t gather_blocks_ws_bytes(int W, int b) { return (size_t)W * b * 2; }

hipError_t launch_gather_blocks(int T, int W, const bf16* A, const int32_t* perm, bf16* Ug,
                                const bf16* G, bf16* Gf, bf16* Out, const float* cscale,
                                hipStream_t s) {
  if (!gather_blocks_ok(W, GB_B) || T < 1) return hipErrorInvalidValue;
  const int nblk = W / GB_B;
  const int nchunks = nblk * GB_B * GB_B / 8;
  hipLaunchKernelGGL(k_gfrag, dim3((nchunks + 255) / 256), dim3(256), 0, s, nchunks, G, Gf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int lds = GB_RS * (2 * W + 16) + 4 * W;
  const int ngrp = (T + GB_TOK - 1) / GB_TOK;
  if (perm) {
    const hipError_t attr = gb_set_lds((const void*)k_gather_blocks<true>, GB_RS * (2 * GB_WMAX + 16) + 4 * GB_WMAX);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_gather_blocks<true>, dim3(ngrp), dim3(GB_NTH), lds, s, T, W, A, perm, Ug,
                       Gf, Out, cscale);
  } else {
    const hipError_t attr = gb_set_lds((const void*)k_gather_blocks<false>, GB_RS * (2 * GB_WMAX + 16) + 4 * GB_WMAX);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(k_gather_blocks<false>, dim3(ngrp), dim3(GB_NTH), lds, s, T, W, A, perm, Ug,
                       Gf, Out, cscale);
  }
  return hipGetLastError();
}

}  // namespace poetx
