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
#include <atomic>

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

template <int B, int MODE>
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
  bf16* Qs = Xs + PW * QP;                          // [B][QP]

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
  u32x4_t qv[QPER];
#pragma unroll
  for (int u = 0; u < QPER; ++u) {
    const int q = u * NT + threadIdx.x;
    qv[u] = *reinterpret_cast<const u32x4_t*>(Qb + (q / (B / 8)) * B + (q % (B / 8)) * 8);
  }
  constexpr int DPER = MODE == MODE_BWD1 ? PW * B / 4 / NT : 1;  // float4 of the D band
  f32x4_t dv[DPER];
  if constexpr (MODE == MODE_BWD1) {
#pragma unroll
    for (int u = 0; u < DPER; ++u)
      dv[u] = *reinterpret_cast<const f32x4_t*>(Db + (long)J0 * B + 4 * (u * NT + threadIdx.x));
  }

  // fixed part of the per-step addend, in accumulator layout:
  //   forward  Q[row][J0+c]   (from the bf16 Q in LDS: the products use that
  //                            same rounded Q)
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
#pragma unroll
  for (int u = 0; u < QPER; ++u) {
    const int q = u * NT + threadIdx.x;
    *reinterpret_cast<u32x4_t*>(Qs + (q / (B / 8)) * QP + (q % (B / 8)) * 8) = qv[u];
  }
  if constexpr (MODE == MODE_FWD) __syncthreads();  // Q visible for the base
  f32x16_t X[RTW];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int rt = wave + t * NWAVE;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (rt < RT) {
        const int row = rt * 32 + acc_row(r, lane);
        if constexpr (MODE == MODE_FWD) {
          base[t][r] = bf2f(Qs[row * QP + J0 + col]);
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
    if (wave < RT) {  // waves beyond the block's row tiles only join the barriers
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

// Blocks of 512: panels of 128 columns (forward, phase 2) or 64 (phase 1),
// eight waves of 64 rows each.  Q (512 KB in bf16) does not fit LDS and is
// read straight from L2 as the MFMA A operand in fragment order (q_off), so
// the L2-to-CU traffic of Q bounds a Horner step: a panel streams all of Q
// once per step, and a 128-column panel feeds each Q fragment to four
// MFMAs (a 32-column one to one).  The panel X^T is the B operand in LDS.
// The steps:
//   forward  X_s = c Q[:, panel] + Q X_{s+1}.  The addend is itself a
//            product, Q (c E_panel): after the step's 32 K-steps come 2 CTW
//            more over K = the panel's own columns, each row tile adding one
//            MFMA with c times an identity block as the B fragment;
//   phase 1  X_s = F_s^T = w_{s+1} D^T - Q X_{s+1} (the product with -Q: the
//            A fragments' sign bits flipped).  The panel's D^T stays in
//            registers from the first step on; four consecutive rows of a
//            lane are one 16-byte piece of row J0 + c of D.  F_s goes out
//            from its LDS copy, whose rows are rows of F_s;
//   phase 2  Y_s = F_s + Q Y_{s+1}, Y_k = w_{k+1} D: F_s is loaded into the
//            accumulators at the start of the step.
// Phase 2 reads the bf16 F_s itself, where the narrower panels keep
// F_s - w D (a smaller quantity) in bf16; the rounding of that one term is
// the only difference in arithmetic.
// Phase 1 stores F_s for phase 2 in the latter's accumulator order: the
// 32 x 32 tile (rt, ct) is 2 KB, lane L = 32 h + col holding F_s[rt*32 + 8q
// + 4h + i][ct*32 + col] as its elements 4q + i.  Offset in elements.
__device__ __forceinline__ long f_tile_off(int rt, int ct) { return (long)(rt * 16 + ct) * 1024; }

__device__ __forceinline__ void wide_tile(int id, int nwg, int npan, int& blk, int& pan) {
  // workgroups are dealt round-robin over the 8 XCDs: give each XCD a
  // contiguous range of (block, panel) pairs, so a block's panels share an
  // XCD and its L2 copy of Q (any workgroup count)
  const int x = id % 8, s = id / 8, full = nwg / 8, rem = nwg % 8;
  const int L = x * full + min(x, rem) + s;
  blk = L / npan;
  pan = L % npan;
}

// One panel of 32 * CTW columns of block blk, from column J0; Xs is
// [32 * CTW][QP].
template <int MODE, int CTW>
__device__ __forceinline__ void wide_body(int k, int blk, int J0, int nblk,
                                          const bf16* __restrict__ Qg, const float* __restrict__ D,
                                          bf16* __restrict__ out_bf, bf16* __restrict__ out_bfT,
                                          float* __restrict__ out_f, bf16* __restrict__ Xs) {
  constexpr int B = 512, PWW = 32 * CTW, QP = B + PAD;
  constexpr int RTW = 2;       // row tiles per wave (eight waves: all 512 rows)
  constexpr int NKS = B / 16;  // K-steps of one product
  // Phase 1 keeps its panel of D^T in registers (read once, not once per
  // step): a second accumulator-sized register set, so panels of at most 64.
  constexpr bool DRES = MODE == MODE_BWD1;
  static_assert(!DRES || CTW <= 2, "register budget");
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);  // uniform: scalar offsets
  const int col = lane % 32, h = lane / 32;
  const long boff = (long)blk * B * B;
  const bf16* Qb = Qg + boff;
  f32x16_t P[RTW][CTW];
  float Dr[DRES ? RTW : 1][DRES ? CTW : 1][DRES ? 16 : 1];
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  // The addends are read through buffer resources over one block: a lane's
  // offset is one 32-bit register per column tile, the rest a wave-uniform
  // constant, so no 64-bit address per element stays live.
  const __amdgpu_buffer_rsrc_t rsD = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(D ? D + boff : nullptr), (short)0, D ? B * B * 4 : 0, 0x00020000);

  // P = the addend of step s (s = k: the starting X), every tile at once.
  // inloop: s < k is known (the step loop), so the tiles' loads form one
  // straight run and all go out before the first is waited for.
  auto load_addend = [&](int s, bool inloop) {
    const float w = (MODE == MODE_FWD) ? (s == k ? 1.f : cnp_coef(s + 1, k)) : cnp_wcoef(s + 1, k);
    const bool before_k = inloop || s < k;
    if constexpr (DRES) {
      if (before_k) {
#pragma unroll
        for (int t = 0; t < RTW; ++t)
#pragma unroll
          for (int u = 0; u < CTW; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) P[t][u][r] = w * Dr[t][u][r];
        return;
      }
    }
    int c0 = J0 + col, hh = h;
    asm volatile("" : "+v"(c0), "+v"(hh));  // recomputed per step, not kept
    __amdgpu_buffer_rsrc_t rsF = rsD;
    if constexpr (MODE == MODE_BWD2) {
      if (before_k)
        rsF = __builtin_amdgcn_make_buffer_rsrc((void*)(out_bf + ((long)s * nblk + blk) * B * B),
                                               (short)0, B * B * 2, 0x00020000);
    }
#pragma unroll
    for (int u = 0; u < CTW; ++u) {
      const int c = c0 + u * 32;
#pragma unroll
      for (int t = 0; t < RTW; ++t) {
        const int rt = wave * RTW + t;
        if constexpr (MODE == MODE_FWD) {
          // the c Q[:, panel] term enters through the products (below)
          P[t][u] = (f32x16_t){};
        } else if constexpr (MODE == MODE_BWD1) {
          // D^T[row][c] = D[c][row]: four consecutive rows are 16 bytes of row c
          const int lo = (c * B + 4 * hh) * 4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsD, lo, (rt * 32 + 8 * q) * 4, 0);
            Dr[t][u][4 * q + 0] = __uint_as_float(v.x);
            Dr[t][u][4 * q + 1] = __uint_as_float(v.y);
            Dr[t][u][4 * q + 2] = __uint_as_float(v.z);
            Dr[t][u][4 * q + 3] = __uint_as_float(v.w);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) P[t][u][r] = w * Dr[t][u][r];
        } else if (before_k) {
          // F_s is stored in this lane's accumulator order (f_tile_off):
          // the tile's 16 values are 32 contiguous bytes
          const int so = (int)f_tile_off(rt, J0 / 32 + u) * 2;
          const u32x4_t v0 = __builtin_amdgcn_raw_buffer_load_b128(rsF, lane * 32, so, 0);
          const u32x4_t v1 = __builtin_amdgcn_raw_buffer_load_b128(rsF, lane * 32 + 16, so, 0);
          const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            P[t][u][2 * e] = __uint_as_float(wv[e] << 16);
            P[t][u][2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
          }
        } else {
          // s = k: Y_k = w D
          const int lo = (4 * hh * B + c) * 4;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            P[t][u][r] = w * __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                 rsD, lo, (rt * 32 + 8 * (r / 4) + r % 4) * B * 4, 0));
        }
      }
    }
  };
  // P (bf16) into Xs as X^T: rows r, r+1 of a lane's column are one 4-byte word
  auto store_x = [&]() {
#pragma unroll
    for (int t = 0; t < RTW; ++t)
#pragma unroll
      for (int u = 0; u < CTW; ++u) {
        const int rt = wave * RTW + t, c = u * 32 + col;
#pragma unroll
        for (int r = 0; r < 16; r += 2)
          *reinterpret_cast<uint32_t*>(Xs + c * QP + rt * 32 + acc_row(r, lane)) =
              pack2bf(P[t][u][r], P[t][u][r + 1]);
      }
  };
  // phase 1: rows J0 .. J0 + PWW - 1 of F_s from Xs, 16-byte stores
  // phase 1: rows J0 .. J0 + PWW - 1 of F_s (in Xs) in phase 2's
  // accumulator order, 16-byte stores: chunk v is half v % 2 of lane
  // (v / 2) % 64 of tile v / 128 (row tile J0 / 32 + tile / 16, column
  // tile tile % 16); its eight values come from eight rows of Xs
  auto store_f = [&](int s) {
    bf16* F = out_bf + ((long)s * nblk + blk) * B * B;
    constexpr int NCH = (PWW / 32) * 16 * 128;
#pragma unroll
    for (int v = threadIdx.x; v < NCH; v += 512) {
      const int half = v & 1, L = (v >> 1) & 63, tile = v >> 7;
      const int rtl = tile / 16, ct = tile % 16, cl = L % 32, hl = L / 32;
      const bf16* x = Xs + (rtl * 32 + 4 * hl) * QP + ct * 32 + cl;
      uint4 w;
      uint32_t* wp = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2) {
        // elements 8 half + 2 p2 (+1): q = 2 half + p2 / 2, i = 2 (p2 % 2)
        const int r0 = 8 * (2 * half + p2 / 2) + 2 * (p2 % 2);
        wp[p2] = (uint32_t)x[r0 * QP] | ((uint32_t)x[(r0 + 1) * QP] << 16);
      }
      *reinterpret_cast<uint4*>(F + f_tile_off(J0 / 32 + rtl, ct) + L * 16 + 8 * half) = w;
    }
  };

  load_addend(k, false);
  // one offset per row tile (its K-step 0 fragment; K-step ks lies ks KB
  // further), passed through an empty asm each step so that the compiler
  // does not hoist the wave's Q loads out of the step loop
  int qoff[RTW];
#pragma unroll
  for (int t = 0; t < RTW; ++t) qoff[t] = (int)q_off((wave * RTW + t) * 32 + col, 8 * h, B, true);
  // phase 1 multiplies by -Q: the sign bits of its bf16 fragments flip as
  // the products take them (flipped at the load, each load would be waited
  // for at once instead of two K-steps later)
  const uint32_t qsign = (MODE == MODE_BWD1) ? 0x80008000u : 0u;
  auto qfrag = [&](uint4 v) {
    v.x ^= qsign;
    v.y ^= qsign;
    v.z ^= qsign;
    v.w ^= qsign;
    return as_bf16x8(v);
  };
  // The forward's addend c Q[:, panel] = Q (c E_panel) is a product too:
  // after the step's own K-steps come 2 CTW more over K = the panel's
  // columns, each row tile taking one product with c times an identity
  // block as the B fragment.  Exact (c is 1 or 2, Q is bf16), and no load
  // of the addend stands before the step's first product.
  constexpr int NID = MODE == MODE_FWD ? 2 * CTW : 0;  // identity K-steps
  const int kb = J0 / 16;                              // the panel's first K-step
  // lane (col, h) of the identity fragment of panel K-step m has its one
  // nonzero at element col - 16 (m % 2) - 8h (if in 0..7)
  auto id_frag = [&](int m, uint32_t wbits) {
    const int i = col - 16 * (m & 1) - 8 * h;
    uint4 v;
    v.x = (i == 0 ? wbits : 0u) | (i == 1 ? wbits << 16 : 0u);
    v.y = (i == 2 ? wbits : 0u) | (i == 3 ? wbits << 16 : 0u);
    v.z = (i == 4 ? wbits : 0u) | (i == 5 ? wbits << 16 : 0u);
    v.w = (i == 6 ? wbits : 0u) | (i == 7 ? wbits << 16 : 0u);
    return v;
  };
  // K-step ks of the extended order: the product's NKS, then the identity's
  auto fetch_q = [&](int ks, uint4 (&dst)[RTW]) {
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int off = ks < NKS ? ks * 512 : (kb + ks - NKS) * 512;
      dst[t] = *reinterpret_cast<const uint4*>(Qb + qoff[t] + off);
    }
  };
  if constexpr (NID > 0) {
    // X_k = Q[:, panel]: the identity products alone (c = 1)
#pragma unroll
    for (int m = 0; m < NID; ++m) {
      uint4 aq[RTW];
      fetch_q(NKS + m, aq);
      const uint4 bi = id_frag(m, 0x3F80u);
#pragma unroll
      for (int t = 0; t < RTW; ++t) P[t][m / 2] = mfma32x32x16(as_bf16x8(aq[t]), as_bf16x8(bi), P[t][m / 2]);
    }
  }

  for (int s = k - 1; s >= 0; --s) {
    store_x();
    __syncthreads();
    load_addend(s, true);
#pragma unroll
    for (int t = 0; t < RTW; ++t) asm volatile("" : "+v"(qoff[t]));
    {
      // P += (+-Q) X: Q fragments from L2 two K-steps ahead (three in
      // phase 1, whose Q fragments feed half as many products per byte), X
      // fragments from LDS one K-step ahead
      constexpr int QPF = MODE == MODE_BWD1 ? 3 : 2, NKX = NKS + NID;
      uint4 aq[QPF][RTW], bq[2][CTW];
      const uint32_t wbits = cnp_coef(s + 1, k) == 2.f ? 0x4000u : 0x3F80u;
      auto fetch_b = [&](int ks, int sl) {
#pragma unroll
        for (int u = 0; u < CTW; ++u)
          bq[sl][u] = *reinterpret_cast<const uint4*>(Xs + (u * 32 + col) * QP + ks * 16 + 8 * h);
      };
#pragma unroll
      for (int i = 0; i < QPF; ++i) fetch_q(i, aq[i]);
      fetch_b(0, 0);
#pragma unroll
      for (int ks = 0; ks < NKX; ++ks) {
        if (ks + 1 < NKS) fetch_b(ks + 1, (ks + 1) & 1);
        if (ks < NKS) {
#pragma unroll
          for (int t = 0; t < RTW; ++t)
#pragma unroll
            for (int u = 0; u < CTW; ++u)
              P[t][u] = mfma32x32x16(qfrag(aq[ks % QPF][t]), as_bf16x8(bq[ks & 1][u]), P[t][u]);
        } else {
          const int m = ks - NKS;
          const uint4 bi = id_frag(m, wbits);
#pragma unroll
          for (int t = 0; t < RTW; ++t)
            P[t][m / 2] = mfma32x32x16(as_bf16x8(aq[ks % QPF][t]), as_bf16x8(bi), P[t][m / 2]);
        }
        if (ks + QPF < NKX) fetch_q(ks + QPF, aq[ks % QPF]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // phase 1: F_{s+1} (this step's B operand, in Xs; F_k = w D is not
    // stored) goes out after the step's last Q loads, so that no Q load
    // waits behind these stores
    if constexpr (MODE == MODE_BWD1) {
      if (s + 1 < k) store_f(s + 1);
    }
    __syncthreads();  // every wave finished reading Xs
  }

  // outputs: G = I + X_0 and G^T (forward), F_0 (phase 1), dQ = Y_0 (phase 2)
  if constexpr (MODE == MODE_FWD) {
#pragma unroll
    for (int t = 0; t < RTW; ++t)
#pragma unroll
      for (int u = 0; u < CTW; ++u) {
        const int rt = wave * RTW + t, c = J0 + u * 32 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rt * 32 + acc_row(r, lane);
          P[t][u][r] += (row == c) ? 1.f : 0.f;
          out_bf[boff + (long)row * B + c] = f2bf(P[t][u][r]);
        }
      }
    if (out_bfT) {  // rows J0 .. J0 + PWW - 1 of G^T, through Xs
      store_x();
      __syncthreads();
      bf16* GT = out_bfT + boff;
      constexpr int VPR = B / 8;
#pragma unroll
      for (int v = threadIdx.x; v < PWW * VPR; v += 512) {
        const int r = v / VPR, c8 = (v % VPR) * 8;
        *reinterpret_cast<uint4*>(GT + (long)(J0 + r) * B + c8) = *reinterpret_cast<const uint4*>(Xs + r * QP + c8);
      }
    }
  } else if constexpr (MODE == MODE_BWD1) {
    store_x();
    __syncthreads();
    store_f(0);
  } else {
#pragma unroll
    for (int t = 0; t < RTW; ++t)
#pragma unroll
      for (int u = 0; u < CTW; ++u) {
        const int rt = wave * RTW + t, c = J0 + u * 32 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) out_f[boff + (long)(rt * 32 + acc_row(r, lane)) * B + c] = P[t][u][r];
      }
  }
}

// Workgroups 0 .. (16 / CTM) nmain - 1 take blocks 0 .. nmain - 1 in
// 32 * CTM-column panels; the rest take the remaining blocks in
// 32 * CTT-column panels.  A block count that leaves a partial last round
// of wide panels (74 blocks: 296 panels of 128 columns on 256 CUs) would
// otherwise run two full panel times; the narrower tail panels fill that
// round in a fraction of one.
template <int MODE, int CTM, int CTT>
__global__ __launch_bounds__(512, 1) void k_cnp_wide(int k, int nmain, int nblk,
                                                     const bf16* __restrict__ Qg,
                                                     const float* __restrict__ D,
                                                     bf16* __restrict__ out_bf,
                                                     bf16* __restrict__ out_bfT,
                                                     float* __restrict__ out_f) {
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* Xs = reinterpret_cast<bf16*>(smem);
  const int id = blockIdx.x, wm = (16 / CTM) * nmain;
  int blk, pan;
  if (CTM != CTT && id < wm) {
    wide_tile(id, wm, 16 / CTM, blk, pan);
    wide_body<MODE, CTM>(k, blk, pan * 32 * CTM, nblk, Qg, D, out_bf, out_bfT, out_f, Xs);
  } else {
    wide_tile(id - wm, (int)gridDim.x - wm, 16 / CTT, blk, pan);
    wide_body<MODE, CTT>(k, nmain + blk, pan * 32 * CTT, nblk, Qg, D, out_bf, out_bfT, out_f, Xs);
  }
}

// Every block in six panels: four of 96 columns, then two of 64 (the
// forward and phase 2; phase 1 has no registers for a 96-column panel of
// D^T).  Between 33 and 42 blocks (the Llama-13B MLP's 37) uniform panels
// waste the CUs: 128-column ones leave 256 - 4 nblk idle, 64-column ones
// take two rounds.  Six panels a block fill one round, which lasts a
// 96-column panel.
template <int MODE>
__global__ __launch_bounds__(512, 1) void k_cnp_wide6(int k, int nblk,
                                                      const bf16* __restrict__ Qg,
                                                      const float* __restrict__ D,
                                                      bf16* __restrict__ out_bf,
                                                      bf16* __restrict__ out_bfT,
                                                      float* __restrict__ out_f) {
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* Xs = reinterpret_cast<bf16*>(smem);
  int blk, pan;
  wide_tile(blockIdx.x, (int)gridDim.x, 6, blk, pan);
  if (pan < 4)
    wide_body<MODE, 3>(k, blk, pan * 96, nblk, Qg, D, out_bf, out_bfT, out_f, Xs);
  else
    wide_body<MODE, 2>(k, blk, 384 + (pan - 4) * 64, nblk, Qg, D, out_bf, out_bfT, out_f, Xs);
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
  constexpr size_t lds = (size_t)(PW + B) * (B + PAD) * sizeof(bf16);
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = k_cnp_panel<B, MODE>;
  const hipError_t attr = lds_opt_in((const void*)kern, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(B / PW, nblk), dim3(NT), lds, s, k, theta, Qg, D, out_bf,
                     out_bfT, out_f);
  return hipGetLastError();
}

// CUs of the current device, asked once per device (256 on MI355X)
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v < 1) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Blocks given the wider panels (pm per block; the rest get pt narrower
// ones): the split with the fewest panel times, counting a narrower panel
// as tcost of a wider one (it streams all of Q per step for fewer columns)
// and one panel per CU at a time.
int wide_split(int nblk, int ncu, int pm, int pt, double tcost, double* time = nullptr) {
  auto rounds = [&](long wg) { return (double)((wg + ncu - 1) / ncu); };
  int best = nblk;
  double tbest = rounds((long)pm * nblk);
  for (int r = 0; (long)r * ncu <= (long)pm * nblk; ++r) {
    const int M = (int)((long)r * ncu / pm);
    if (M > nblk) break;
    const double t = rounds((long)pm * M) + tcost * rounds((long)pt * (nblk - M));
    if (t < tbest - 1e-9) {
      tbest = t;
      best = M;
    }
  }
  if (time) *time = tbest;
  return best;
}

template <int MODE>
hipError_t launch_wide(int nblk, int k, const bf16* Qg, const float* D, bf16* out_bf,
                       bf16* out_bfT, float* out_f, hipStream_t s) {
  // the forward and phase 2: 128-column panels where they fill whole rounds
  // of the CUs, 64-column ones for the rest; phase 1 (which keeps D^T in
  // registers): 64 and 32
  constexpr int CTM = MODE == MODE_BWD1 ? 2 : 4, CTT = CTM / 2;
  constexpr double TCOST = MODE == MODE_BWD1 ? 0.6 : 0.55;
  // a round of six-panel blocks (k_cnp_wide6) in 128-column panel times
  // (measured at 37 blocks: the forward 64 against 77 us)
  constexpr double T6 = 0.8;
  constexpr size_t lds = (size_t)32 * CTM * (512 + PAD) * sizeof(bf16);
  constexpr size_t lds6 = (size_t)96 * (512 + PAD) * sizeof(bf16);
  static_assert(lds <= 160 * 1024 && lds6 <= 160 * 1024, "LDS budget");
  const int ncu = cu_count();
  double tsplit = 0;
  const int nmain = wide_split(nblk, ncu, 16 / CTM, 16 / CTT, TCOST, &tsplit);
  if constexpr (MODE != MODE_BWD1) {
    if (T6 * (double)((6L * nblk + ncu - 1) / ncu) < tsplit - 1e-9) {
      auto kern6 = k_cnp_wide6<MODE>;
      const hipError_t attr6 = lds_opt_in((const void*)kern6, (int)lds6);
      if (attr6 != hipSuccess) return attr6;
      hipLaunchKernelGGL(kern6, dim3((unsigned)(6L * nblk)), dim3(512), lds6, s, k, nblk, Qg, D,
                         out_bf, out_bfT, out_f);
      return hipGetLastError();
    }
  }
  auto kern = k_cnp_wide<MODE, CTM, CTT>;
  const hipError_t attr = lds_opt_in((const void*)kern, (int)lds);
  if (attr != hipSuccess) return attr;
  const long nwg = (long)(16 / CTM) * nmain + (long)(16 / CTT) * (nblk - nmain);
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(512), lds, s, k, nmain, nblk, Qg, D, out_bf,
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
    case 512: return launch_wide<MODE>(nblk, k, Qg, D, out_bf, out_bfT, out_f, s);
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
