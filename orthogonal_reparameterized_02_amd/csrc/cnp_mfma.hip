// Cayley-Neumann parameterization on bf16 MFMA, b in {64, 128, 256, 512}
// ("POET-X ...", technical summary 2.4: Q held on-chip, higher powers and the
// sum formed in one pass, the backward likewise fused).
//
// The pages keep Q and Q^2 in shared memory and form Q^3, Q^4 and the sum.
// Here the series is evaluated in Horner form, which needs only Q on chip:
//   G = sum_p c_p Q^p,  c = (1, 2, ..., 2, 1)
//     = I + U_0,  U_k = Q,  U_p = 2Q + Q U_{p+1}   (p = k-1..0)
// Every step is a LEFT multiplication by Q, so each column panel of U evolves
// on its own: one workgroup owns a 32-column panel of one block, keeps Q in
// LDS (b <= 256: 135 KB of the CU's 160 KB) and the panel in registers, and
// runs all k steps without leaving the CU.  k products of b x b x 32 each:
// 2 k b^3 flops per block, as for the power form.
//
// Backward (D = dL/dG, w_p = c_p (-1)^{p-1}, using Q^T = -Q):
//   F_k = w_{k+1} D,  F_a = w_{a+1} D + F_{a+1} Q      -> row-local; its
//       transpose F_a^T = w_{a+1} D^T - Q F_{a+1}^T is the same left-Horner
//       on column panels of D^T (phase 1, stores F_a - w_{a+1} D in bf16)
//   Y_k = F_k,        Y_a = F_a + Q Y_{a+1},  gQ = Y_0   -> column-local
//       (phase 2, writes gQ in fp32)
//   dtheta = triu1(gQ - gQ^T)                           (phase 3, pack)
// 2 k products per block: 4 k b^3 flops.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Operand layout (lane l of 64):
//   A 32x16: A[l%32][8*(l/32) + i], i < 8      B 16x32: B[8*(l/32) + i][l%32]
//   D 32x32: acc[r] = D[8*(r/4) + 4*(l/32) + r%4][l%32]
#include "kernels.h"

namespace poetx {

namespace {

constexpr int PW = 32;        // panel width (columns per workgroup)
constexpr int PAD = 8;        // LDS row padding (bf16) -> conflict-free b128 reads
constexpr int NT = 512;       // threads per workgroup (8 waves: one CU, latency hiding)
constexpr int NWAVE = NT / 64;

enum { MODE_FWD = 0, MODE_BWD1 = 1, MODE_BWD2 = 2 };

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }

// Triangle tiles: a b x b block splits into 64 x 64 tiles (I, J), I <= J;
// tile pair p of a block enumerates them row by row.
constexpr int TT = 64;
__device__ __forceinline__ void tile_pair(int p, int nt, int& I, int& J) {
  I = 0;
  while (p >= nt - I) {
    p -= nt - I;
    ++I;
  }
  J = I + p;
}

// Offset of Q[i][j] in a b x b block of Qg.  Blocks that fit LDS (b <= 256)
// are row-major.  Larger ones are read only as the MFMA A operand, straight
// from L2, so they are stored in operand-fragment order: for row tile i/32
// and K-step j/16, the 32 x 16 fragment is 1 KB laid out as the 64 lanes'
// 16-byte pieces (lane i%32 + 32*((j%16)/8) holds j%16 = 8h .. 8h+7).  One
// wave's fragment load is then 8 whole cache lines instead of 32 partial
// ones.
__device__ __forceinline__ long q_off(int i, int j, int b, bool frag) {
  if (!frag) return (long)i * b + j;
  return ((long)((i >> 5) * (b >> 4) + (j >> 4)) * 64 + (i & 31) + 32 * ((j >> 3) & 1)) * 8 + (j & 7);
}

// Qg[blk] = Q as bf16.  One workgroup per tile pair (I, J): the packed
// parameters of tile (I, J) (row segments, contiguous in theta) go to LDS;
// tile (I, J) of Q is written from it and tile (J, I) = -(tile)^T from the
// transposed LDS reads, both with 16-byte row stores.  Diagonal tiles hold
// both halves and the zero diagonal.
__global__ __launch_bounds__(256) void k_unpack_q(int b, const float* __restrict__ theta,
                                                  bf16* __restrict__ Qg, int frag) {
  __shared__ float tile[TT][TT + 1];
  const int blk = blockIdx.y, nt = b / TT;
  const int tb = b * (b - 1) / 2;
  int I, J;
  tile_pair(blockIdx.x, nt, I, J);
  const float* th = theta + (long)blk * tb;
  bf16* q = Qg + (long)blk * b * b;
  constexpr int PER = TT * TT / 256;
  float v[PER];  // every load in flight before the first LDS write
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = u * 256 + threadIdx.x;
    const int i = I * TT + e / TT, j = J * TT + e % TT;
    v[u] = i < j ? th[tri_index(i, j, b)] : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = u * 256 + threadIdx.x;
    tile[e / TT][e % TT] = v[u];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < TT * TT / 8; e += 256) {
    const int r = e / (TT / 8), c0 = (e % (TT / 8)) * 8;
    const int i = I * TT + r;
    float up[8], lo[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = J * TT + c0 + u;
      // row i of tile (I, J); on a diagonal tile the lower half is -theta(j, i)
      up[u] = i < j ? tile[r][c0 + u] : (i == j ? 0.0f : -tile[c0 + u][r]);
      lo[u] = -tile[c0 + u][r];  // row J*TT + r of tile (J, I)
    }
    uint4 v;
    v.x = pack2bf(up[0], up[1]);
    v.y = pack2bf(up[2], up[3]);
    v.z = pack2bf(up[4], up[5]);
    v.w = pack2bf(up[6], up[7]);
    *reinterpret_cast<uint4*>(q + q_off(i, J * TT + c0, b, frag)) = v;
    if (I != J) {
      v.x = pack2bf(lo[0], lo[1]);
      v.y = pack2bf(lo[2], lo[3]);
      v.z = pack2bf(lo[4], lo[5]);
      v.w = pack2bf(lo[6], lo[7]);
      *reinterpret_cast<uint4*>(q + q_off(J * TT + r, I * TT + c0, b, frag)) = v;
    }
  }
}

// Copy the unpacked block Qg [B][B] into the padded LDS tile (row pitch
// qp).  One workgroup runs per CU, so every 16-byte load is put in flight
// before the first LDS write.
template <int B, int NTH>
__device__ __forceinline__ void q_to_lds(const bf16* __restrict__ Qb, bf16* Qs, int qp) {
  constexpr int VPR = B / 8;                 // 16-byte vectors per row
  constexpr int PER = B * VPR / NTH;         // vectors per thread
  static_assert(B * VPR % NTH == 0, "tile split");
  uint4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int q = u * NTH + threadIdx.x;
    v[u] = *reinterpret_cast<const uint4*>(Qb + (q / VPR) * B + (q % VPR) * 8);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int q = u * NTH + threadIdx.x;
    *reinterpret_cast<uint4*>(Qs + (q / VPR) * qp + (q % VPR) * 8) = v[u];
  }
}

template <int B, bool QLDS, int MODE>
__global__ __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_cnp_panel(int k, const float* __restrict__ theta,
                                                  const bf16* __restrict__ Qg,
                                                  const float* __restrict__ D,
                                                  bf16* __restrict__ out_bf, bf16* __restrict__ out_bfT,
                                                  float* __restrict__ out_f) {
  constexpr int QP = B + PAD;
  constexpr int RT = B / 32;                        // 32-row tiles in a block
  constexpr int RTW = (RT + NWAVE - 1) / NWAVE;     // row tiles per wave
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* Xs = reinterpret_cast<bf16*>(smem);         // [PW][QP]: X^T
  bf16* Qs = Xs + PW * QP;                          // [B][QP] (QLDS only)

  // Workgroups are dealt round-robin over the 8 XCDs; renumber them so each
  // XCD walks a contiguous range of (block, panel) pairs.  The panels of one
  // block then share an XCD (a block may straddle two), its L2 copy of Q
  // (read by every panel) is fetched from MALL/HBM once instead of once per
  // XCD, and an XCD's L2 holds the Q of only the few blocks it has in flight.
  int pan = blockIdx.x, blk = blockIdx.y;
  const int nwg = gridDim.x * gridDim.y;
  if (nwg % 8 == 0) {
    const int id = blockIdx.y * gridDim.x + blockIdx.x;
    const int pid = (id % 8) * (nwg / 8) + id / 8;
    blk = pid / gridDim.x;
    pan = pid % gridDim.x;
  }
  const int J0 = pan * PW;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int col = lane % 32;
  const long boff = (long)blk * B * B;
  const bf16* Qb = Qg + boff;
  const float* Db = D ? D + boff : nullptr;

  // Prologue: every global load (Q, and for phase 1 the band D[J0..J0+31][:])
  // goes out before the first LDS write.
  constexpr int QPER = B * (B / 8) / NT;  // 16-byte Q vectors per thread
  // (native vector types: the HIP vector structs are copied through memcpy,
  // which keeps conditionally stored arrays out of registers)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t qv[QLDS ? QPER : 1];
  if constexpr (QLDS) {
#pragma unroll
    for (int u = 0; u < QPER; ++u) {
      const int q = u * NT + threadIdx.x;
      qv[u] = *reinterpret_cast<const u32x4_t*>(Qb + (q / (B / 8)) * B + (q % (B / 8)) * 8);
    }
  }
  constexpr int DPER = MODE == MODE_BWD1 ? PW * B / 4 / NT : 1;  // float4 of the D band
  f32x4_t dv[DPER];
  if constexpr (MODE == MODE_BWD1) {
#pragma unroll
    for (int u = 0; u < DPER; ++u)
      dv[u] = *reinterpret_cast<const f32x4_t*>(Db + (long)J0 * B + 4 * (u * NT + threadIdx.x));
  }

  // fixed part of the per-step addend, in accumulator layout:
  //   forward  Q[row][J0+c]   (from the bf16 Q in LDS when it is there: the
  //                            products use that same rounded Q)
  //   phase 1  D^T[row][c] = D[J0+c][row]  (the D band, transposed through LDS)
  //   phase 2  D[row][J0+c]                (row-contiguous global loads)
  float base[RTW][16];
#pragma unroll
  for (int t = 0; t < RTW; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) base[t][r] = 0.f;
  if constexpr (MODE == MODE_BWD1) {
    // two passes of 16 band rows through the Xs region as fp32 [16][B + 4]
    float* band = reinterpret_cast<float*>(Xs);
    constexpr int BP = B + 4;
    static_assert(16 * BP * 4 <= PW * QP * 2, "band pass fits in Xs");
#define POETX_BAND_PASS(pass)                                                                  \
  {                                                                                            \
    _Pragma("unroll") for (int u = 0; u < DPER; ++u) {                                         \
      const int e = 4 * (u * NT + threadIdx.x);                                                \
      if (e / B / 16 == (pass))                                                                \
        *reinterpret_cast<f32x4_t*>(band + (e / B - 16 * (pass)) * BP + e % B) = dv[u];        \
    }                                                                                          \
    __syncthreads();                                                                           \
    if (col / 16 == (pass)) {                                                                  \
      _Pragma("unroll") for (int t = 0; t < RTW; ++t) {                                        \
        const int rt = wave + t * NWAVE;                                                       \
        if (rt < RT) {                                                                         \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) base[t][r] =                          \
              band[(col - 16 * (pass)) * BP + rt * 32 + acc_row(r, lane)];                     \
        }                                                                                      \
      }                                                                                        \
    }                                                                                          \
    __syncthreads();                                                                           \
  }
    POETX_BAND_PASS(0);
    POETX_BAND_PASS(1);
#undef POETX_BAND_PASS
  }
  if constexpr (QLDS) {
#pragma unroll
    for (int u = 0; u < QPER; ++u) {
      const int q = u * NT + threadIdx.x;
      *reinterpret_cast<u32x4_t*>(Qs + (q / (B / 8)) * QP + (q % (B / 8)) * 8) = qv[u];
    }
    if constexpr (MODE == MODE_FWD) __syncthreads();  // Q visible for the base
  }
  if constexpr (MODE == MODE_FWD && !QLDS) {
    // Q[row][J0+col] = -Q[J0+col][row]: rows J0.. of Q are one row tile in
    // fragment order, and a lane's four accumulator rows 8a + 4h .. +3 of
    // row tile rt are four consecutive elements of one 16-byte piece
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int rt = min(wave + t * NWAVE, RT - 1);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint2 v = *reinterpret_cast<const uint2*>(
            Qb + q_off(J0 + col, rt * 32 + 8 * a + 4 * (lane / 32), B, true));
        base[t][4 * a + 0] = -bf2f((bf16)(v.x & 0xffff));
        base[t][4 * a + 1] = -bf2f((bf16)(v.x >> 16));
        base[t][4 * a + 2] = -bf2f((bf16)(v.y & 0xffff));
        base[t][4 * a + 3] = -bf2f((bf16)(v.y >> 16));
      }
    }
  }
  f32x16_t X[RTW];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int rt = wave + t * NWAVE;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (rt < RT) {
        const int row = rt * 32 + acc_row(r, lane);
        if constexpr (MODE == MODE_FWD) {
          if constexpr (QLDS) base[t][r] = bf2f(Qs[row * QP + J0 + col]);
        } else if constexpr (MODE == MODE_BWD2) {
          base[t][r] = Db[(long)row * B + J0 + col];
        }
      }
      // initial state: U_k = Q (forward), w_{k+1} D^T or w_{k+1} D (backward)
      X[t][r] = (MODE == MODE_FWD) ? base[t][r] : cnp_wcoef(k + 1, k) * base[t][r];
    }
  }

  auto store_xs = [&]() {
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int rt = wave + t * NWAVE;
      if (rt < RT) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int row = rt * 32 + acc_row(r, lane);  // rows row, row+1
          *reinterpret_cast<uint32_t*>(Xs + col * QP + row) = pack2bf(X[t][r], X[t][r + 1]);
        }
      }
    }
  };
  store_xs();
  __syncthreads();

  for (int step = k - 1; step >= 0; --step) {
    // phase 2 adds F_step - w D: load it before the product so it arrives meanwhile
    float fadd[RTW][16];
    if constexpr (MODE == MODE_BWD2) {
      const bf16* F = out_bf + ((long)step * gridDim.y + blk) * B * B;
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        const int rt = min(wave + t * NWAVE, RT - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) fadd[t][r] = bf2f(F[(long)(rt * 32 + acc_row(r, lane)) * B + J0 + col]);
      }
    }
    // P = Q * X over the panel
    f32x16_t P[RTW];
#pragma unroll
    for (int t = 0; t < RTW; ++t) P[t] = (f32x16_t){};
    if (!QLDS && wave < RT) {
      // Q streamed from L2 in fragment order: each fragment load is 1 KB of
      // whole lines, issued QPF K-steps ahead of its MFMAs (deeper rings
      // measured no faster: the loop is bound by the CU's L2 bandwidth, 512
      // KB of Q per step for eight waves); the X fragments come from LDS one
      // K-step ahead.  Fully unrolled, so every ring index is a constant.
      constexpr int QPF = 2;
      constexpr int NKS = B / 16;
      uint4 bq[2], aq[QPF][RTW];
      // one element offset per row tile (its K-step 0 fragment; K-step ks
      // lies ks KB further).  Q is the same in every step, so the offsets
      // pass through an empty asm each step: otherwise the compiler hoists
      // all of the wave's Q loads out of the step loop and tries to keep its
      // 64 KB of Q in registers.  (An offset, not the pointer: a pointer
      // through asm loses its global address space and the loads become
      // flat ones, which also count against lgkmcnt.)
      int qoff[RTW];
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        qoff[t] = (int)q_off(min(wave + t * NWAVE, RT - 1) * 32 + (lane % 32), 8 * (lane / 32), B, true);
        asm volatile("" : "+v"(qoff[t]));
      }
      const bf16* xrow = Xs + col * QP + 8 * (lane / 32);
      auto fetch_a = [&](int ks, int s) {  // fragment order: K-step ks is 1 KB further
#pragma unroll
        for (int t = 0; t < RTW; ++t)
          aq[s][t] = *reinterpret_cast<const uint4*>(Qb + qoff[t] + ks * 512);
      };
      auto fetch_b = [&](int ks, int s) { bq[s] = *reinterpret_cast<const uint4*>(xrow + ks * 16); };
#pragma unroll
      for (int i = 0; i < QPF; ++i) fetch_a(i, i);
      fetch_b(0, 0);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 1 < NKS) fetch_b(ks + 1, (ks + 1) & 1);
#pragma unroll
        for (int t = 0; t < RTW; ++t)
          if (RTW * NWAVE == RT || wave + t * NWAVE < RT)
            P[t] = mfma32x32x16(as_bf16x8(aq[ks % QPF][t]), as_bf16x8(bq[ks & 1]), P[t]);
        if (ks + QPF < NKS) fetch_a(ks + QPF, ks % QPF);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (QLDS && wave < RT) {  // waves beyond the block's row tiles only join the barriers
      // Q in LDS: operand fragments double-buffered, the reads for k0+16
      // issued before the MFMAs of k0
      uint4 bq[2], aq[2][RTW];
      auto fetch = [&](int k0, int s) {
        const int kk = k0 + 8 * (lane / 32);
        bq[s] = *reinterpret_cast<const uint4*>(Xs + col * QP + kk);
#pragma unroll
        for (int t = 0; t < RTW; ++t) {
          const int arow = min(wave + t * NWAVE, RT - 1) * 32 + (lane % 32);
          aq[s][t] = *reinterpret_cast<const uint4*>(Qs + arow * QP + kk);
        }
      };
      auto mma = [&](int s) {
#pragma unroll
        for (int t = 0; t < RTW; ++t)
          if (wave + t * NWAVE < RT) P[t] = mfma32x32x16(as_bf16x8(aq[s][t]), as_bf16x8(bq[s]), P[t]);
      };
      fetch(0, 0);
#pragma unroll 2
      for (int k0 = 0; k0 < B; k0 += 32) {  // buffer indices stay compile-time
        fetch(k0 + 16, 1);
        mma(0);
        if (k0 + 32 < B) fetch(k0 + 32, 0);
        mma(1);
      }
    }
    __syncthreads();  // every wave finished reading Xs
    const float wstep = (MODE == MODE_FWD) ? cnp_coef(step + 1, k) : cnp_wcoef(step + 1, k);
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int rt = wave + t * NWAVE;
      if (rt >= RT) continue;
      if (MODE == MODE_FWD) {
#pragma unroll
        for (int r = 0; r < 16; ++r) X[t][r] = wstep * base[t][r] + P[t][r];
      } else if (MODE == MODE_BWD1) {
        // F_step - w D = -(Q F_{step+1}^T) transposed: store rows J0+c
        bf16* F = out_bf + ((long)step * gridDim.y + blk) * B * B;
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const int row = rt * 32 + acc_row(r, lane);
          uint2 pk;
          pk.x = pack2bf(-P[t][r], -P[t][r + 1]);
          pk.y = pack2bf(-P[t][r + 2], -P[t][r + 3]);
          *reinterpret_cast<uint2*>(F + (long)(J0 + col) * B + row) = pk;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) X[t][r] = wstep * base[t][r] - P[t][r];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) X[t][r] = wstep * base[t][r] + fadd[t][r] + P[t][r];
      }
    }
    if (step > 0) {
      store_xs();
      __syncthreads();
    }
  }

  // outputs
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int rt = wave + t * NWAVE;
    if (rt >= RT) continue;
    if (MODE == MODE_FWD) {
      bf16* G = out_bf + boff;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rt * 32 + acc_row(r, lane);
        X[t][r] += (row == J0 + col) ? 1.f : 0.f;
        G[(long)row * B + J0 + col] = f2bf(X[t][r]);
      }
      if (out_bfT) {
        bf16* GT = out_bfT + boff;
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const int row = rt * 32 + acc_row(r, lane);
          uint2 pk;
          pk.x = pack2bf(X[t][r], X[t][r + 1]);
          pk.y = pack2bf(X[t][r + 2], X[t][r + 3]);
          *reinterpret_cast<uint2*>(GT + (long)(J0 + col) * B + row) = pk;
        }
      }
    } else if (MODE == MODE_BWD2) {
      float* dQ = out_f + boff;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rt * 32 + acc_row(r, lane);
        dQ[(long)row * B + J0 + col] = X[t][r];
      }
    }
  }
}

// dtheta[t(i,j)] (+)= gQ[i][j] - gQ[j][i], one workgroup per (row i, block)
// dtheta(i, j) = dQ[i][j] - dQ[j][i] for i < j (set or accumulate).  One
// workgroup per tile pair (I, J): tiles (I, J) and (J, I) of dQ are read with
// row-contiguous loads into LDS; the packed outputs of tile (I, J) are row
// segments of dtheta.
__global__ __launch_bounds__(256) void k_pack_skew(int b, const float* __restrict__ dQ,
                                                   float* __restrict__ dtheta, int accumulate) {
  __shared__ float up[TT][TT + 1], lo[TT][TT + 1];
  const int blk = blockIdx.y, nt = b / TT;
  int I, J;
  tile_pair(blockIdx.x, nt, I, J);
  const float* g = dQ + (long)blk * b * b;
  float* dth = dtheta + (long)blk * (b * (b - 1) / 2);
  constexpr int PER = TT * TT / 256;
  float vu[PER], vl[PER];  // every load in flight before the first LDS write
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = u * 256 + threadIdx.x, r = e / TT, c = e % TT;
    vu[u] = g[(long)(I * TT + r) * b + J * TT + c];
    vl[u] = g[(long)(J * TT + r) * b + I * TT + c];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = u * 256 + threadIdx.x;
    up[e / TT][e % TT] = vu[u];
    lo[e / TT][e % TT] = vl[u];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < TT * TT; e += 256) {
    const int r = e / TT, c = e % TT, i = I * TT + r, j = J * TT + c;
    if (i < j) {
      const float v = up[r][c] - lo[c][r];
      float* d = dth + tri_index(i, j, b);
      *d = accumulate ? *d + v : v;
    }
  }
}

template <int B, int MODE>
hipError_t launch_panel(int nblk, int k, const float* theta, const bf16* Qg, const float* D,
                        bf16* out_bf, bf16* out_bfT, float* out_f, hipStream_t s) {
  constexpr bool QLDS = B <= 256;
  constexpr size_t lds = (size_t)(PW + (QLDS ? B : 0)) * (B + PAD) * sizeof(bf16);
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = k_cnp_panel<B, QLDS, MODE>;
  // the LDS opt-in is a host call; make it once per kernel, not per launch
  static const hipError_t attr =
      lds > 64 * 1024 ? hipFuncSetAttribute((const void*)kern,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)
                      : hipSuccess;
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(B / PW, nblk), dim3(NT), lds, s, k, theta, Qg, D, out_bf,
                     out_bfT, out_f);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch_panel(int nblk, int b, int k, const float* theta, const bf16* Qg,
                          const float* D, bf16* out_bf, bf16* out_bfT, float* out_f,
                          hipStream_t s) {
  switch (b) {
    case 64: return launch_panel<64, MODE>(nblk, k, theta, Qg, D, out_bf, out_bfT, out_f, s);
    case 128: return launch_panel<128, MODE>(nblk, k, theta, Qg, D, out_bf, out_bfT, out_f, s);
    case 256: return launch_panel<256, MODE>(nblk, k, theta, Qg, D, out_bf, out_bfT, out_f, s);
    case 512: return launch_panel<512, MODE>(nblk, k, theta, Qg, D, out_bf, out_bfT, out_f, s);
    default: return hipErrorInvalidValue;
  }
}

// every block size reads Q from this bf16 copy: blocks up to 256 stage it in
// LDS, larger ones stream it through L2 as the MFMA A operand
hipError_t unpack(int nblk, int b, const float* theta, bf16* Qg, hipStream_t s) {
  const int nt = b / TT;
  const int frag = b > 256;  // the panel kernel streams these blocks' Q from L2
  hipLaunchKernelGGL(k_unpack_q, dim3(nt * (nt + 1) / 2, nblk), dim3(256), 0, s, b, theta, Qg,
                     frag);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cnp_panel_fwd(int nblk, int b, int k, const float* theta, bf16* G, bf16* GT,
                                bf16* ws_Q, hipStream_t s) {
  hipError_t e = unpack(nblk, b, theta, ws_Q, s);
  if (e != hipSuccess) return e;
  return dispatch_panel<MODE_FWD>(nblk, b, k, theta, ws_Q, nullptr, G, GT, nullptr, s);
}

hipError_t launch_cnp_panel_bwd(int nblk, int b, int k, const float* theta, const float* dG,
                                float* dtheta, int accumulate, bf16* ws_Q, bf16* ws_F,
                                float* ws_dQ, bool q_ready, hipStream_t s) {
  hipError_t e = q_ready ? hipSuccess : unpack(nblk, b, theta, ws_Q, s);
  if (e != hipSuccess) return e;
  if (k > 0) {
    e = dispatch_panel<MODE_BWD1>(nblk, b, k, theta, ws_Q, dG, ws_F, nullptr, nullptr, s);
    if (e != hipSuccess) return e;
  }
  e = dispatch_panel<MODE_BWD2>(nblk, b, k, theta, ws_Q, dG, ws_F, nullptr, ws_dQ, s);
  if (e != hipSuccess) return e;
  const int nt = b / TT;
  hipLaunchKernelGGL(k_pack_skew, dim3(nt * (nt + 1) / 2, nblk), dim3(256), 0, s, b, ws_dQ,
                     dtheta, accumulate);
  return hipGetLastError();
}

}  // namespace poetx
