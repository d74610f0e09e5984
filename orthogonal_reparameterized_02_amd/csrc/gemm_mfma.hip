// bf16 MFMA GEMMs for the layer's dense contraction and its batched b x b
// block products ("POET-X ...", technical summary 2.1 input-centric form and
// 2.3 batch-parallel blocks: each block is an independent matrix product,
// the block-diagonal matrix is never built).
//
//   k_nt4:      C = A B^T on 256 x 256 tiles, 4 waves, K fed by
//               buffer_load ... lds into a ring of five 32 KB slots (the dense products
//               Z = V W0f^T and dV = dZ W0f, and large batched products).
//               EPI 1 and 2 add the block epilogue: when the tile's 256
//               columns are one b = 256 orthogonal block g (EPI 1) or two
//               b = 128 blocks (EPI 2), E = C_tile blockdiag(Bk)^T is formed
//               from the tile staged in LDS, so Z -> S_i = Z_i G_Ri^T and
//               dV -> dU_j = dV_j G_Pj leave the CU without a second pass
//               over HBM.
//   k_gemm_nt:  the same product with register-staged loads, for small or
//               narrow shapes (fewer tiles than CUs, N % 256 != 0).
//   k_blocks:   per-token block products with G_j resident in LDS
//               (V = U G_P^T, dZ = dS G_R, b in {128, 256}).
//   k_tn4 / k_gemm_tn: P[s][bt] = sum over a token range of A^T B, A [T][*]
//               and B [T][*] token-major, fp32 partial sums (dG_R = dS^T Z,
//               dG_P = dV^T U); a fixed-order reduction over s follows.
//
// LDS rows of 64 bf16 (128 B) hold eight 16-byte chunks, chunk c of row r
// stored at position c ^ ((r ^ r/8) & 7), which keeps the 16 rows an MFMA
// operand read touches per phase on distinct banks.
// MFMA: v_mfma_f32_32x32x16_bf16; lane l holds A[l%32][8*(l/32)+i] and
// B[8*(l/32)+i][l%32]; acc[r] = D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include <algorithm>

#include "kernels.h"

namespace poetx {

namespace {

constexpr int BK = 64;
constexpr int ROWB = BK * 2;  // bytes per LDS row

__device__ __forceinline__ int lds_off(int r, int c) {
  return r * ROWB + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
}

template <int BM, int BN, int WM, int WN>
struct Cfg {
  static constexpr int NTH = 64 * WM * WN;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int STAGE = (BM + BN) * ROWB;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int RPP = NTH / 8;               // rows per load pass
  static constexpr int PA = BM / RPP, PB = BN / RPP;
  static_assert(FM >= 1 && FN >= 1 && PA >= 1 && PB >= 1, "tile too small");
};

template <int FM, int FN, int TM, int TN>
__device__ __forceinline__ void frag_load(const char* __restrict__ As, const char* __restrict__ Bs,
                                          bf16x8_t (&a)[FM], bf16x8_t (&b)[FN], int ks, int wm,
                                          int wn, int lane) {
  const int c = ks * 2 + lane / 32;
#pragma unroll
  for (int i = 0; i < FM; ++i)
    a[i] = as_bf16x8(*reinterpret_cast<const uint4*>(As + lds_off(wm * TM + i * 32 + lane % 32, c)));
#pragma unroll
  for (int j = 0; j < FN; ++j)
    b[j] = as_bf16x8(*reinterpret_cast<const uint4*>(Bs + lds_off(wn * TN + j * 32 + lane % 32, c)));
}

template <int FM, int FN>
__device__ __forceinline__ void frag_mma(const bf16x8_t (&a)[FM], const bf16x8_t (&b)[FN],
                                         f32x16_t (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
}

// acc += A_slab(rows of this wave) * B_slab(rows of this wave)^T over BK;
// the LDS reads of sub-step ks+1 are issued before the MFMAs of ks
template <class C>
__device__ __forceinline__ void mma_slab(const char* __restrict__ As, const char* __restrict__ Bs,
                                         f32x16_t (&acc)[C::FM][C::FN], int wm, int wn, int lane) {
  bf16x8_t a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
  frag_load<C::FM, C::FN, C::TM, C::TN>(As, Bs, a0, b0, 0, wm, wn, lane);
  frag_load<C::FM, C::FN, C::TM, C::TN>(As, Bs, a1, b1, 1, wm, wn, lane);
  frag_mma<C::FM, C::FN>(a0, b0, acc);
  frag_load<C::FM, C::FN, C::TM, C::TN>(As, Bs, a0, b0, 2, wm, wn, lane);
  frag_mma<C::FM, C::FN>(a1, b1, acc);
  frag_load<C::FM, C::FN, C::TM, C::TN>(As, Bs, a1, b1, 3, wm, wn, lane);
  frag_mma<C::FM, C::FN>(a0, b0, acc);
  frag_mma<C::FM, C::FN>(a1, b1, acc);
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

// Write a wave's accumulators as bf16 into LDS laid out as 64-column slabs
// [col/64][row][64] (the MFMA operand layout).  Only fragments whose 32 rows
// lie in [r_lo, r_hi) are written (partial staging); rbase and r_lo are
// multiples of 32, so a fragment's swizzle keys are fixed per lane.  Each
// lane packs its row pair (r, r+1) of one column; lanes l and l^1 swap
// halves (DPP quad permute) so each writes two adjacent columns of one row.
// With SC, column c of the tile is scaled by cs[c] (fp32, before rounding).
template <int FM, int FN, bool SC>
__device__ __forceinline__ void acc_to_slabs_impl(const f32x16_t (&acc)[FM][FN], char* lds,
                                                  int slab_bytes, int rbase, int cbase, int lane,
                                                  int r_lo, int r_hi, const float* __restrict__ cs) {
  const int odd = lane & 1;
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
  const int rl = 4 * (lane >> 5) + odd;  // row within an 8-row group for r % 4 == 0
  const int cl = (lane & 31) - odd;      // first column of the written pair
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int fr = rbase + i * 32 - r_lo;  // fragment's first row in the staging buffer
    if (fr < 0 || fr >= r_hi - r_lo) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = cbase + j * 32 + cl;
      char* base = lds + (col >> 6) * slab_bytes + (fr + rl) * ROWB + (col & 7) * 2;
      const int chx = ((col >> 3) & 7) ^ ((fr >> 3) & 4);
      const float sc = SC ? cs[cbase + j * 32 + (lane & 31)] : 1.0f;  // this lane's column
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const uint32_t p = SC ? pack2bf(acc[i][j][r] * sc, acc[i][j][r + 1] * sc)
                              : pack2bf(acc[i][j][r], acc[i][j][r + 1]);
        const uint32_t q = (uint32_t)__builtin_amdgcn_mov_dpp((int)p, 0xB1, 0xF, 0xF, true);
        const uint32_t v = __builtin_amdgcn_perm(q, p, sel);
        const int key = chx ^ ((r & 3) + rl) ^ (r >> 2);
        *reinterpret_cast<uint32_t*>(base + (8 * (r >> 2) + (r & 3)) * ROWB + (key << 4)) = v;
      }
    }
  }
}

template <int FM, int FN>
__device__ __forceinline__ void acc_to_slabs(const f32x16_t (&acc)[FM][FN], char* lds, int slab_bytes,
                                             int rbase, int cbase, int lane, int r_lo, int r_hi,
                                             const float* __restrict__ cs = nullptr) {
  if (cs)
    acc_to_slabs_impl<FM, FN, true>(acc, lds, slab_bytes, rbase, cbase, lane, r_lo, r_hi, cs);
  else
    acc_to_slabs_impl<FM, FN, false>(acc, lds, slab_bytes, rbase, cbase, lane, r_lo, r_hi, cs);
}

// Copy ROWS x COLS bf16 from the slab layout to global memory with 16-byte
// stores: consecutive lanes cover whole 128-byte row segments.
template <int ROWS, int COLS, int NTH>
__device__ __forceinline__ void slabs_to_global(const char* lds, bf16* __restrict__ C, long ldc,
                                                int row0, int col0, int M, int N) {
  constexpr int CHUNKS = ROWS * COLS / 8;
  static_assert(CHUNKS % NTH == 0, "store split");
#pragma unroll
  for (int u = 0; u < CHUNKS / NTH; ++u) {
    const int q = u * NTH + threadIdx.x;
    const int s = q / (ROWS * 8), r = (q / 8) % ROWS, c = q % 8;
    const uint4 v = *reinterpret_cast<const uint4*>(lds + s * ROWS * ROWB + lds_off(r, c));
    const int row = row0 + r, col = col0 + s * BK + c * 8;
    if (row < M && col < N) *reinterpret_cast<uint4*>(C + (long)row * ldc + col) = v;
  }
}

// Transposed accumulator layout (k_nt4 swaps the MFMA operands): acc[i][j]
// holds the 32 x 32 block of rows rbase + 32 i (lane l: row rbase + 32 i +
// l % 32) and columns cbase + 32 j; register r holds column
// 8 (r/4) + 4 (l/32) + r % 4 of it.  So four consecutive registers are four
// consecutive columns of one row: one 8-byte LDS write per four values, into
// the same [col/64][row][64] slab layout as acc_to_slabs.
template <int FM, int FN, bool SC>
__device__ __forceinline__ void acc_to_slabsT_impl(const f32x16_t (&acc)[FM][FN], char* lds,
                                                   int slab_bytes, int rbase, int cbase, int lane,
                                                   const float* __restrict__ cs) {
  const int h = lane >> 5;
  if constexpr (SC) {
    // one scale vector (the lane's four columns c0 + 4 h .. + 3) at a time,
    // used for every row fragment before the next is loaded
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c0 = cbase + j * 32 + 8 * q;
        const float4 sc = *reinterpret_cast<const float4*>(cs + c0 + 4 * h);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = rbase + i * 32 + (lane & 31);
          const int key = (row ^ (row >> 3)) & 7;
          uint2 v;
          v.x = pack2bf(acc[i][j][4 * q] * sc.x, acc[i][j][4 * q + 1] * sc.y);
          v.y = pack2bf(acc[i][j][4 * q + 2] * sc.z, acc[i][j][4 * q + 3] * sc.w);
          *reinterpret_cast<uint2*>(lds + row * ROWB + 8 * h + (c0 >> 6) * slab_bytes +
                                    ((((c0 & 63) >> 3) ^ key) << 4)) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = rbase + i * 32 + (lane & 31);
    const int key = (row ^ (row >> 3)) & 7;
    char* rowp = lds + row * ROWB + 8 * h;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c0 = cbase + j * 32 + 8 * q;  // the lane's columns: c0 + 4 h .. + 3
        uint2 v;
        v.x = pack2bf(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
        v.y = pack2bf(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        *reinterpret_cast<uint2*>(rowp + (c0 >> 6) * slab_bytes + ((((c0 & 63) >> 3) ^ key) << 4)) = v;
      }
  }
}

// cs (or null): column c of the tile scaled by cs[c] before rounding.
template <int FM, int FN>
__device__ __forceinline__ void acc_to_slabsT(const f32x16_t (&acc)[FM][FN], char* lds, int slab_bytes,
                                              int rbase, int cbase, int lane,
                                              const float* __restrict__ cs = nullptr) {
  if (cs) {
    acc_to_slabsT_impl<FM, FN, true>(acc, lds, slab_bytes, rbase, cbase, lane, cs);
  } else {
    acc_to_slabsT_impl<FM, FN, false>(acc, lds, slab_bytes, rbase, cbase, lane, cs);
  }
}

// Slabs to global with buffer stores: rows past M fall outside the buffer
// range and are dropped by the hardware, so there is no branch; every column
// of the tile must exist (callers have N % COLS == 0).  Offsets stay below
// ROWS * ldc * 2 < 2^31 (host-checked).  The range is clamped at zero rows:
// a negative count would wrap to an unbounded range.  nt: non-temporal
// stores, for outputs that no kernel reads soon (they then hold no space in
// the last-level cache that the next kernels' reads would have to evict).
template <int ROWS, int COLS, int NTH>
__device__ __forceinline__ void slabs_to_global_buf(const char* lds, bf16* __restrict__ C, long ldc,
                                                    int row0, int col0, int M, bool nt = false) {
  constexpr int CHUNKS = ROWS * COLS / 8;
  static_assert(CHUNKS % NTH == 0 && (ROWS & (ROWS - 1)) == 0, "store split");
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  // a pass may start at or past M (the last token tile of k_blocks): its
  // range is then empty, not negative, and every store is dropped
  // (base and count are uniform; readfirstlane keeps the resource in SGPRs)
  const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(ROWS, M - row0)));
  const uint64_t base = (uint64_t)(uintptr_t)(C + (long)row0 * ldc + col0);
  const uint64_t ubase = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(uintptr_t)ubase, (short)0, nrows * (int)ldc * 2, 0x00020000);
  constexpr int RSTEP = NTH / 8;  // rows one pass of the workgroup covers
  const int c = threadIdx.x % 8;
  if constexpr (ROWS % RSTEP == 0) {  // each pass stays in one slab: offsets affine in u
    const int r0 = threadIdx.x / 8, vbase = (r0 * (int)ldc + c * 8) * 2;
#pragma unroll
    for (int u = 0; u < CHUNKS / NTH; ++u) {
      const int s = u / (ROWS / RSTEP), ru = (u % (ROWS / RSTEP)) * RSTEP;
      const u32x4v v = *reinterpret_cast<const u32x4v*>(lds + s * ROWS * ROWB + lds_off(ru + r0, c));
      if (nt) __builtin_amdgcn_raw_buffer_store_b128(v, rs, vbase + (ru * (int)ldc + s * 64) * 2, 0, 2);
      else __builtin_amdgcn_raw_buffer_store_b128(v, rs, vbase + (ru * (int)ldc + s * 64) * 2, 0, 0);
    }
  } else {
#pragma unroll
    for (int u = 0; u < CHUNKS / NTH; ++u) {
      const int q = u * NTH + threadIdx.x;
      const int s = q / (ROWS * 8), r = (q >> 3) & (ROWS - 1);
      const u32x4v v = *reinterpret_cast<const u32x4v*>(lds + s * ROWS * ROWB + lds_off(r, c));
      if (nt) __builtin_amdgcn_raw_buffer_store_b128(v, rs, (r * (int)ldc + s * 64 + c * 8) * 2, 0, 2);
      else __builtin_amdgcn_raw_buffer_store_b128(v, rs, (r * (int)ldc + s * 64 + c * 8) * 2, 0, 0);
    }
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// two transposed 4 x 16 reads -> one 8-value MFMA operand
__device__ __forceinline__ bf16x8_t frag_tr(const char* p0, const char* p1) {
  const s16x4_t h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<char*>(p0)));
  const s16x4_t h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(const_cast<char*>(p1)));
  const s16x8_t w = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, w);
}

// eight int8 values (K order, lowest byte first) as a bf16 MFMA operand;
// exact, since every int8 value has at most 8 significant bits
__device__ __forceinline__ bf16x8_t i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const int32_t a = (int32_t)lo, b = (int32_t)hi;
  uint4 u;
  u.x = pack2bf((float)((a << 24) >> 24), (float)((a << 16) >> 24));
  u.y = pack2bf((float)((a << 8) >> 24), (float)(a >> 24));
  u.z = pack2bf((float)((b << 24) >> 24), (float)((b << 16) >> 24));
  u.w = pack2bf((float)((b << 8) >> 24), (float)(b >> 24));
  return as_bf16x8(u);
}

// C = A B^T with register-staged loads (two LDS stages), for shapes k_nt4
// does not take: fewer 256 x 256 tiles than CUs, or N % 256 != 0.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void k_gemm_nt(
    int M, int N, int K, const bf16* __restrict__ A, long lda, long sA, const bf16* __restrict__ B,
    long ldb, long sB, bf16* __restrict__ Cm, long ldc, long sC, int tilesM, int tilesN,
    const float* __restrict__ cscale, long sS) {
  using C = Cfg<BM, BN, WM, WN>;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / WN, wn = wave % WN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const long bt = blockIdx.y;
  A += bt * sA;
  B += bt * sB;
  Cm += bt * sC;

  const int lr = tid / 8, lc = tid % 8;
  uint4 ra[C::PA], rb[C::PB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int p = 0; p < C::PA; ++p) {
      const int row = m0 + p * C::RPP + lr;
      ra[p] = row < M ? *reinterpret_cast<const uint4*>(A + row * lda + k0 + lc * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < C::PB; ++p) {
      const int row = n0 + p * C::RPP + lr;
      rb[p] = row < N ? *reinterpret_cast<const uint4*>(B + row * ldb + k0 + lc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    char* As = smem + buf * C::STAGE;
    char* Bs = As + C::A_BYTES;
#pragma unroll
    for (int p = 0; p < C::PA; ++p) *reinterpret_cast<uint4*>(As + lds_off(p * C::RPP + lr, lc)) = ra[p];
#pragma unroll
    for (int p = 0; p < C::PB; ++p) *reinterpret_cast<uint4*>(Bs + lds_off(p * C::RPP + lr, lc)) = rb[p];
  };

  f32x16_t acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = (f32x16_t){};

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const char* As = smem + cur * C::STAGE;
    mma_slab<C>(As, As + C::A_BYTES, acc, wm, wn, lane);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // C tile -> LDS (64-column slabs; the main loop's last barrier freed the
  // stage buffers) -> global with 16-byte stores over whole row segments
  constexpr int SLAB = BM * ROWB;
  static_assert(BN * SLAB / BK <= C::LDS, "staging fits in the stage buffers");
  acc_to_slabs<C::FM, C::FN>(acc, smem, SLAB, wm * C::TM, wn * C::TN, lane, 0, BM,
                             cscale ? cscale + bt * sS + n0 : nullptr);
  __syncthreads();
  slabs_to_global<BM, BN, C::NTH>(smem, Cm, ldc, m0, n0, M, N);
}

// C = A B^T on a 256 x 256 tile with 4 waves (128 x 128 each, accumulators
// in AGPRs).  K advances in slabs of 64: a slab row is 128 bytes, one whole
// cache line, and eight lanes of a buffer_load_dwordx4 ... lds fetch it, so
// every L2 request is a full line.  The data go from L2 straight into LDS
// (no staging registers); the loads are issued from inline asm (they have no
// register results) and completion is tracked by hand with vmcnt, so the
// compiler puts no conservative wait in front of the LDS operand reads.
// Operands live in a ring of five 32 KB slots (all 160 KB of LDS): slab j's
// A rows in slot 2j mod 5, its B rows in slot 2j+1 mod 5.  While slab kt is
// multiplied, slab kt+1 sits in two slots and A of slab kt+2 streams into the
// fifth (during K-steps 0 and 1); B of slab kt+2 follows into A_kt's slot in
// K-step 3, after the slab's one barrier, by which point every wave has
// read slab kt (its last fragments are read during K-step 2).  With one wave
// per SIMD nothing else hides a stall of the MFMA pipe, so the issue order
// is fixed by hand (sched_barrier): each pair of MFMAs is followed by one
// operand read for the next K-step and, where scheduled, one load.  Rows
// past M or N read as zero through the buffer range check and are masked on
// store (buffer stores whose range covers the tile's existing rows).  The K
// order of the MFMAs is plain ascending, as in k_gemm_nt.  EPI 1 adds the
// block epilogue (described at its code below).
//
// BMODE selects B's storage: 0 bf16 [N][K] (as above), 1 int8 [N][K], 2 bf16
// [K][N] (K-major: the weight as stored for the other product, so one copy
// serves both).
// K-major B (BMODE 2): a 64-row K slab of the tile's 256 columns lands in the
// B slot as 64 rows of 512 bytes, 16-byte chunk c of row k stored at
// position c ^ 2 (k mod 4), and the fragments are read with
// ds_read_b64_tr_b16: each 16-lane group receives a 4-K x 16-column tile
// transposed, and two reads give a lane its eight consecutive K values of
// one column, the same values in the same K order as the N-major read, so
// the products are bitwise those of BMODE 0 on the transposed weight.
// int8 B (BMODE 1; a quantized weight; ldb, sB in bytes).  Its
// 64-wide K slabs land in the B slots as 64-byte rows (16 KB of the 32 KB
// slot), 16-byte chunk c of row r stored at position c ^ ((r >> 2) & 3), and
// are widened to bf16 when the fragments are read: every int8 value is
// exact in bf16, so the products are those of the integer weight.  One
// 16-byte read per row gives a lane the B values of two K-steps, so within
// a slab a K-step pair 2j, 2j+1 takes, for lane half h, the K ranges
// 32 j + 16 h + [0, 8) and + [8, 16); the A reads follow the same K order.
// SC: column c of C is multiplied by cscale[bt * sS + c] (fp32, before
// rounding), which applies a per-output-row weight scale.
// ntmask: bit 0 stores C, bit 1 stores E non-temporally.
template <int EPI, int BMODE, bool SC>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_nt4(
    int M, int N, int K, const bf16* __restrict__ A, long lda, long sA, const void* __restrict__ Bv,
    long ldb, long sB, bf16* __restrict__ Cm, long ldc, long sC, int tilesM, int tilesN,
    const bf16* __restrict__ Bk, bf16* __restrict__ E, long lde, const float* __restrict__ cscale,
    long sS, int ntmask) {
  constexpr int BM = 256, BN = 256, TM = 128, TN = 128, FM = 4, FN = 4, NTH = 256;
  constexpr int OPB = 256 * ROWB;  // one operand's 256 rows of a 64-wide slab: 32 KB
  constexpr bool BQ = BMODE == 1, BNN = BMODE == 2;
  constexpr int BES = BQ ? 1 : 2;  // bytes per B element
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, tilesM, tilesN, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const long bt = blockIdx.y;
  Cm += bt * sC;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  // buffer ranges cover the tile's rows that exist (fewer than 256 at the
  // bottom edge); offsets stay below 256 * ld * 2 < 2^31 (host-checked)
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + bt * sA + (long)m0 * lda), (short)0, min(BM, M - m0) * (int)lda * 2, 0x00020000);
  // K-major B: the tile's columns from n0, every K row (K * ldb * 2 < 2^31,
  // host-checked); N-major: the tile's rows that exist
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(reinterpret_cast<const char*>(Bv) +
              (bt * sB + (BNN ? (long)n0 : (long)n0 * ldb)) * BES),
      (short)0, BNN ? K * (int)ldb * 2 : min(BN, N - n0) * (int)ldb * BES, 0x00020000);
  // Load q (0..7) of this wave fills rows 32 q + 8 wave .. +7 of a slot
  // (1 KB): lane l lands at byte 16 l, i.e. row 32 q + 8 wave + l/8, slot
  // position l % 8, which holds logical chunk (l%8) ^ (l/8) ^ wave ^ 4 (q&1)
  // under lds_off's swizzle.
  const int rl = wave * 8 + lane / 8;
  const int cx = (lane % 8) ^ (lane / 8) ^ wave;
  int voA[2], voB[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    voA[p] = rl * (int)lda * 2 + ((cx ^ (4 * p)) << 4);
    voB[p] = rl * (int)ldb * 2 + ((cx ^ (4 * p)) << 4);
  }
  const int gA = 32 * (int)lda * 2, gB = 32 * (int)ldb * 2;  // bytes per 32 rows
  // int8 B: load q (0..3) of this wave fills rows 64 q + 16 wave + l/4 of a
  // slot (1 KB of 64-byte rows), lane l at position l % 4, which holds
  // logical chunk (l % 4) ^ (l / 16) under the int8 swizzle
  int voQ[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    voQ[q] = (64 * q + 16 * wave + lane / 4) * (int)ldb + 16 * ((lane & 3) ^ (lane >> 4));
  // K-major B: load q (0..7) of this wave fills K rows 2 (4 q + wave) + l/32
  // of the slab, lane l at chunk position l % 32, which holds logical chunk
  // (l % 32) ^ 2 (row mod 4); a slab is 64 K rows further
  int voN[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int row = 2 * (4 * q + wave) + lane / 32;
    voN[q] = row * (int)ldb * 2 + 16 * ((lane & 31) ^ ((row & 3) << 1));
  }
  const int slabN = 64 * (int)ldb * 2;
  // K-major fragment reads: lane l supplies K row 8 (l/32) + (l%16)/4 and
  // columns 16 ((l>>4)&1) + 4 (l&3) .. +3 of a 32-column fragment
  const int tk_l = 8 * (lane / 32) + (lane % 16) / 4;
  const int ft_l = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // load q of slab `from` into the slot at byte offset slotb.  M0 (the LDS
  // destination) is set inside the same asm statement; nothing else in these
  // kernels reads M0 (no indirect register indexing, no LDS-DMA builtins),
  // so the asm does not declare it.
#define POETX_DMA1(slotb, from, q, vo, g, rs)                                                  \
  {                                                                                            \
    const uint32_t m0v_ =                                                                      \
        __builtin_amdgcn_readfirstlane(lds0 + (slotb) + ((q) * 4 + wave) * 1024);              \
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v_),    \
                 "v"(vo[(q) & 1] + (q) * (g) + (from) * 128), "s"(rs)                          \
                 : "memory");                                                                 \
  }
  // int8 B, slab `from`, load q into the slot at byte offset slotb
#define POETX_DMAQ(slotb, from, q)                                                             \
  {                                                                                            \
    const uint32_t m0v_ =                                                                      \
        __builtin_amdgcn_readfirstlane(lds0 + (slotb) + ((q) * 4 + wave) * 1024);              \
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v_),    \
                 "v"(voQ[q] + (from) * 64), "s"(rsB)                                           \
                 : "memory");                                                                 \
  }
  // K-major bf16 B, slab `from`, load q into the slot at byte offset slotb
#define POETX_DMAN(slotb, from, q)                                                             \
  {                                                                                            \
    const uint32_t m0v_ =                                                                      \
        __builtin_amdgcn_readfirstlane(lds0 + (slotb) + ((q) * 4 + wave) * 1024);              \
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v_),    \
                 "v"(voN[q] + (from) * slabN), "s"(rsB)                                        \
                 : "memory");                                                                 \
  }
  // operand fragment g of K-step ks from slots sa (A) / sb (B): g < 4 reads A
  // rows, else B rows.  int8 B: the even K-step of a pair reads both steps'
  // bytes, widens its own half and keeps the other for the odd step.
  // K-major B: two transposed reads, K rows t0 and t0 + 4.
#define POETX_FRAG(F, sa, sb, ks, g)                                                           \
  {                                                                                            \
    if ((g) < 4) {                                                                             \
      const int c_ = BQ ? 4 * ((ks) >> 1) + 2 * (lane / 32) + ((ks) & 1) : (ks) * 2 + lane / 32; \
      fa[F][(g) & 3] = as_bf16x8(*reinterpret_cast<const uint4*>(                              \
          smem + (sa) + lds_off(wm * TM + ((g) & 3) * 32 + lane % 32, c_)));                    \
    } else if (BNN) {                                                                          \
      const int ft_ = wn * TN + ((g) & 3) * 32 + ft_l;                                         \
      const int t0_ = 16 * (ks) + tk_l, t1_ = t0_ + 4;                                         \
      fb[F][(g) & 3] = frag_tr(                                                                \
          smem + (sb) + t0_ * 512 + ((((ft_ >> 3) ^ ((t0_ & 3) << 1))) << 4) + (ft_ & 7) * 2,  \
          smem + (sb) + t1_ * 512 + ((((ft_ >> 3) ^ ((t1_ & 3) << 1))) << 4) + (ft_ & 7) * 2); \
    } else if (!BQ) {                                                                          \
      fb[F][(g) & 3] = as_bf16x8(*reinterpret_cast<const uint4*>(                              \
          smem + (sb) + lds_off(wn * TN + ((g) & 3) * 32 + lane % 32, (ks) * 2 + lane / 32)));  \
    } else if (((ks) & 1) == 0) {                                                              \
      const int r_ = wn * TN + ((g) & 3) * 32 + lane % 32;                                     \
      const uint4 raw_ = *reinterpret_cast<const uint4*>(                                      \
          smem + (sb) + r_ * 64 + 16 * (((ks) + lane / 32) ^ ((r_ >> 2) & 3)));                \
      fb[F][(g) & 3] = i8x8_to_bf16(raw_.x, raw_.y);                                           \
      fbq[(g) & 3] = make_uint2(raw_.z, raw_.w);                                               \
    } else {                                                                                   \
      fb[F][(g) & 3] = i8x8_to_bf16(fbq[(g) & 3].x, fbq[(g) & 3].y);                           \
    }                                                                                          \
  }
  // MFMAs 2g, 2g+1 of a K-step: row fragment g/2 against two column
  // fragments, which run 0..3 for even rows and 3..0 for odd ones, so that
  // consecutive MFMAs change one operand (less switching power: the card is
  // power-limited here).  Each accumulator still sums its K-steps in order.
  // The B fragment is the MFMA's first operand, so acc[i][j] holds its block
  // transposed (acc_to_slabsT's layout).
#define POETX_MMA2(F, g)                                                                       \
  {                                                                                            \
    const int i_ = (g) / 2;                                                                    \
    const int j0_ = (i_ & 1) ? 3 - 2 * ((g) % 2) : 2 * ((g) % 2);                              \
    const int j1_ = (i_ & 1) ? j0_ - 1 : j0_ + 1;                                              \
    acc[i_][j0_] = mfma32x32x16(fb[F][j0_], fa[F][i_], acc[i_][j0_]);                          \
    acc[i_][j1_] = mfma32x32x16(fb[F][j1_], fa[F][i_], acc[i_][j1_]);                          \
  }
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16_t){};
  bf16x8_t fa[2][FM], fb[2][FN];
  uint2 fbq[FN];  // int8 B: the odd K-step's raw bytes
  const int nk = K / 64;
  // Slab numbers past the end are clamped to the last slab; those copies land
  // in slots that are never read again, so every wave always has the same
  // number of loads in flight and the vmcnt thresholds are constants.
  {
    const int s1 = min(1, nk - 1);
#pragma unroll
    for (int q = 0; q < 8; ++q) POETX_DMA1(0 * OPB, 0, q, voA, gA, rsA);
    if constexpr (BQ) {
#pragma unroll
      for (int q = 0; q < 4; ++q) POETX_DMAQ(1 * OPB, 0, q);
    } else if constexpr (BNN) {
#pragma unroll
      for (int q = 0; q < 8; ++q) POETX_DMAN(1 * OPB, 0, q);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) POETX_DMA1(1 * OPB, 0, q, voB, gB, rsB);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) POETX_DMA1(2 * OPB, s1, q, voA, gA, rsA);
    if constexpr (BQ) {
#pragma unroll
      for (int q = 0; q < 4; ++q) POETX_DMAQ(3 * OPB, s1, q);
    } else if constexpr (BNN) {
#pragma unroll
      for (int q = 0; q < 8; ++q) POETX_DMAN(3 * OPB, s1, q);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) POETX_DMA1(3 * OPB, s1, q, voB, gB, rsB);
    }
  }
  // slab 0 has landed (this wave's part): at most slab 1's loads are pending
  if constexpr (BQ) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int g = 0; g < 8; ++g) POETX_FRAG(0, 0, OPB, 0, g);
  int sl = 0;  // slot of A_kt (B_kt: sl+1, A_kt+1: sl+2, B_kt+1: sl+3, A_kt+2: sl+4, mod 5)
  for (int kt = 0; kt < nk; ++kt) {
    const int sa = sl * OPB, sb = (sl + 1 >= 5 ? sl - 4 : sl + 1) * OPB;
    const int na = (sl + 2 >= 5 ? sl - 3 : sl + 2) * OPB, nb = (sl + 3 >= 5 ? sl - 2 : sl + 3) * OPB;
    const int a2 = (sl + 4 >= 5 ? sl - 1 : sl + 4) * OPB;
    const int pre = min(kt + 2, nk - 1);
    // K-steps 0 and 1, each with the next K-step's fragments and half of A_kt+2
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      POETX_FRAG(1, sa, sb, 1, g);
      POETX_MMA2(0, g);
      if (g & 1) POETX_DMA1(a2, pre, g / 2, voA, gA, rsA);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      POETX_FRAG(0, sa, sb, 2, g);
      POETX_MMA2(1, g);
      if (g & 1) POETX_DMA1(a2, pre, 4 + g / 2, voA, gA, rsA);
      __builtin_amdgcn_sched_barrier(0);
    }
    // K-step 2 with the last fragments of slab kt
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      POETX_FRAG(1, sa, sb, 3, g);
      POETX_MMA2(0, g);
      __builtin_amdgcn_sched_barrier(0);
    }
    // slab kt+1 has landed when at most A_kt+2's eight loads are pending;
    // lgkmcnt(0): this wave's reads of slab kt are complete, so after the
    // barrier A_kt's slot can be refilled
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    // K-step 3, with slab kt+1's first fragments and B_kt+2 into A_kt's slot
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      POETX_FRAG(0, na, nb, 0, g);
      POETX_MMA2(1, g);
      if constexpr (BQ) {
        if ((g & 1) == 0) POETX_DMAQ(sa, pre, g / 2);
      } else if constexpr (BNN) {
        POETX_DMAN(sa, pre, g);
      } else {
        POETX_DMA1(sa, pre, g, voB, gB, rsB);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    sl = sl + 2 >= 5 ? sl - 3 : sl + 2;
  }
#undef POETX_DMA1
#undef POETX_DMAQ
#undef POETX_DMAN
#undef POETX_FRAG
#undef POETX_MMA2
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  constexpr int SLAB = BM * ROWB;
  if constexpr (SC)
    acc_to_slabsT_impl<FM, FN, true>(acc, smem, SLAB, wm * TM, wn * TN, lane,
                                     cscale + bt * sS + n0);
  else
    acc_to_slabsT<FM, FN>(acc, smem, SLAB, wm * TM, wn * TN, lane);
  // Block epilogue, E = C_tile blockdiag(G)^T, formed transposed like C.
  // EPI 1 (blocks of 256): the tile's columns are one block, so every wave
  // sums over all 256 columns of the C tile with G block tn.  EPI 2 (blocks
  // of 128): a wave's 128 output columns (half wn of the tile) are exactly
  // block 2 tn + wn, so it sums over that half of the C tile only.  The
  // MFMA's first operand is a G fragment (rows of the block's G, straight
  // from global memory: G is read by every tile of its column, so it sits in
  // L2; two K-steps ahead, so the loop has no barrier), the second a fragment
  // of the C tile just staged in LDS (four 64-wide K slabs).  The first loads
  // go out before the C stores: vmcnt is in order, and a wait for loads
  // issued after the stores would wait for the stores too.
  constexpr int EB = EPI == 2 ? 128 : 256;  // block size
  constexpr int EKS = EB / 16;               // K-steps of the block product
  const int ek0 = EPI == 2 ? wn * 8 : 0;     // first K-step within the C tile
  const bf16* Gw = nullptr;
  bf16x8_t gb[3][FN];
  if constexpr (EPI != 0) {
    const long gblk = EPI == 2 ? 2L * tn + wn : (long)tn;
    const int grow = EPI == 2 ? lane % 32 : wn * TN + lane % 32;
    Gw = Bk + gblk * EB * EB + (long)grow * EB + 8 * (lane / 32);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        gb[f][j] = as_bf16x8(*reinterpret_cast<const uint4*>(Gw + j * 32 * EB + f * 16));
  }
  __syncthreads();
  slabs_to_global_buf<BM, BN, NTH>(smem, Cm, ldc, m0, n0, M, (ntmask & 1) != 0);
  if constexpr (EPI != 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16_t){};
    bf16x8_t ca[2][FM];
#define POETX_CFRAG(F, ks)                                                                     \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) ca[F][i] = as_bf16x8(                       \
        *reinterpret_cast<const uint4*>(smem + ((ek0 + (ks)) / 4) * SLAB +                     \
                                        lds_off(wm * TM + i * 32 + lane % 32,                  \
                                                ((ks) % 4) * 2 + lane / 32)));
    POETX_CFRAG(0, 0);
#pragma unroll
    for (int ks = 0; ks < EKS; ++ks) {
      if (ks + 2 < EKS) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          gb[(ks + 2) % 3][j] =
              as_bf16x8(*reinterpret_cast<const uint4*>(Gw + j * 32 * EB + (ks + 2) * 16));
      }
      if (ks + 1 < EKS) { POETX_CFRAG((ks + 1) & 1, ks + 1); }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
          const int j = (i & 1) ? FN - 1 - jj : jj;  // one operand changes per MFMA
          acc[i][j] = mfma32x32x16(gb[ks % 3][j], ca[ks & 1][i], acc[i][j]);
        }
    }
#undef POETX_CFRAG
    __syncthreads();  // every wave is done with the C tile
    acc_to_slabsT<FM, FN>(acc, smem, SLAB, wm * TM, wn * TN, lane);
    __syncthreads();
    slabs_to_global_buf<BM, BN, NTH>(smem, E, lde, m0, n0, M, (ntmask & 2) != 0);
  }
}


// vmcnt(N), optionally with lgkmcnt(0), as an s_waitcnt immediate (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N, bool LGKM0>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8) | ((N >> 4) << 14));
}

// Token reduction P[s][bt][r][c] = sum over split s's tokens of
// A[t][bt*sA + tr*TM + r] * B[t][bt*sB + tc*TN + c]  (dG = dS^T Z, dV^T U).
// A 4-wave, DMA-fed MFMA pipeline like k_nt4's (hand-fixed issue order, vmcnt
// counted by hand), here with K slabs of 32 tokens in four LDS stages and
// the operands' roles transposed: both operands are token-major, so a K
// slab lands in LDS as [token][feature]
// rows (buffer_load ... lds: rows past the split's end read as zero), and
// the MFMA fragments are read across tokens with ds_read_b64_tr_b16, which
// hands lane i of each 16-lane group feature i of a 4-token x 16-feature
// tile.  Two transposed reads give the eight consecutive tokens (K values) a
// lane holds.  The 16-byte chunk index of a token row is XORed with
// 2 * (token % 4), so the four rows one read touches fall on distinct banks.
// Output: an fp32 TM x TN partial, staged through LDS for 16-byte stores.
// A TM x TN tile of a D x D product: TN = TM / 2 or TM / 4 gives two or
// four times the workgroups of square tiles for the same token splits (and
// fp32 partials); the column parts of a block read the same A slabs, and
// the renumbering below puts them on one XCD, so that A comes from its L2.
// One launch can serve two operand pairs of the same D (dG_R and dG_P):
// batch entries below nb0 read (A0, B0), the rest (A1, B1).  With one token
// split and P1 set, the second pair writes its sums to P1 instead of after
// the first pair's in P (two output buffers, no reduction pass).
template <int TM, int TN, int NSTG>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_tn4(
    int T, int tsplit, int tilesN, int ntiles, int nbatch, const bf16* __restrict__ A0, long lda0,
    long sA, const bf16* __restrict__ B0, long ldb0, long sB, float* __restrict__ P, long ldp,
    long sP, long sS, int nb0, const bf16* __restrict__ A1, long lda1, const bf16* __restrict__ B1,
    long ldb1, float* __restrict__ P1) {
  constexpr int WTM = TM / 2, WTN = TN / 2, FM = WTM / 32, FN = WTN / 32, NF = FM + FN;
  constexpr int NMMA = FM * FN;                   // MFMAs per K-step, spread over NF groups
  constexpr int ROWA = TM * 2, ROWB = TN * 2;     // LDS bytes per token row
  constexpr int A_BYTES = 32 * ROWA, STG = A_BYTES + 32 * ROWB;
  constexpr int NQ = STG / 1024 / 4;              // DMA instructions per wave per slab
  static_assert(NQ == NF, "one DMA per group");
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
  // workgroups are dealt round-robin over the 8 XCDs: number them so each
  // XCD takes a contiguous range of (tile, batch, split), tiles fastest
  int L;
  {
    const int nwg = gridDim.x;
    const int x = blockIdx.x % 8, q = blockIdx.x / 8, full = nwg / 8, rem = nwg % 8;
    L = x * full + min(x, rem) + q;
  }
  const int tile = L % ntiles, by = (L / ntiles) % nbatch, s = L / (ntiles * nbatch);
  const int tr = tile / tilesN, tc = tile % tilesN;
  // batch entries from nb0 on belong to the second operand pair (A1, B1);
  // the partials are indexed over both
  const bool second = by >= nb0;
  const long bt = second ? (long)by - nb0 : (long)by;
  const bf16* __restrict__ A = second ? A1 : A0;
  const bf16* __restrict__ B = second ? B1 : B0;
  const long lda = second ? lda1 : lda0, ldb = second ? ldb1 : ldb0;
  const int t_begin = s * tsplit, t_end = min(T, t_begin + tsplit);
  // P1 set: one token split, each pair straight into its own output
  P = P1 && second ? P1 + bt * sP : P + s * sS + (long)by * sP;
  const int ntok = max(0, t_end - t_begin);
  const int nk = max(1, (ntok + 31) / 32);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (long)t_begin * lda + bt * sA + tr * TM), (short)0, ntok * (int)lda * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + (long)t_begin * ldb + bt * sB + tc * TN), (short)0, ntok * (int)ldb * 2, 0x00020000);
  int vo[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int off = (q * 4 + wave) * 1024 + 16 * lane;
    const bool isA = off < A_BYTES;
    const int o = isA ? off : off - A_BYTES, rb = isA ? ROWA : ROWB;
    const int row = o / rb, pc = (o % rb) / 16;
    const int lc = pc ^ ((row & 3) << 1);
    vo[q] = row * (int)(isA ? lda : ldb) * 2 + lc * 16;
  }
  const int slabA = 32 * (int)lda * 2, slabB = 32 * (int)ldb * 2;
#define DMA1(slot, from, q)                                                                   \
  {                                                                                           \
    const uint32_t m0v_ = __builtin_amdgcn_readfirstlane(                                     \
        lds0 + ((slot) % NSTG) * STG + ((q) * 4 + wave) * 1024);                              \
    if ((q) * 4 < A_BYTES / 1024)                                                             \
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v_),  \
                   "v"(vo[q] + (from) * slabA), "s"(rsA) : "memory");                         \
    else                                                                                      \
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v_),  \
                   "v"(vo[q] + (from) * slabB), "s"(rsB) : "memory");                         \
  }
  const int tk_l = 8 * (lane / 32) + (lane % 16) / 4;
  const int ft_l = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#define FRAG(F, slab, ks, g)                                                                  \
  {                                                                                           \
    const char* S_ = smem + ((slab) % NSTG) * STG + ((g) < FM ? 0 : A_BYTES);                 \
    const int rb_ = (g) < FM ? ROWA : ROWB;                                                   \
    const int ft_ = ((g) < FM ? wm * WTM + (g) * 32 : wn * WTN + ((g) - FM) * 32) + ft_l;      \
    const int t0_ = 16 * (ks) + tk_l, t1_ = t0_ + 4;                                           \
    const char* p0_ = S_ + t0_ * rb_ + (((ft_ >> 3) ^ ((t0_ & 3) << 1)) << 4) + (ft_ & 7) * 2;  \
    const char* p1_ = S_ + t1_ * rb_ + (((ft_ >> 3) ^ ((t1_ & 3) << 1)) << 4) + (ft_ & 7) * 2;  \
    if ((g) < FM) fa[F][(g)] = frag_tr(p0_, p1_);                                             \
    else fb[F][(g) - FM] = frag_tr(p0_, p1_);                                                 \
  }
  // group g issues MFMAs g NMMA / NF .. (g + 1) NMMA / NF - 1 of the K-step
#define MMAG(F, g)                                                                            \
  _Pragma("unroll") for (int m_ = (g) * NMMA / NF; m_ < ((g) + 1) * NMMA / NF; ++m_) {         \
    acc[m_ / FN][m_ % FN] = mfma32x32x16(fa[F][m_ / FN], fb[F][m_ % FN], acc[m_ / FN][m_ % FN]); \
  }
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16_t){};
  bf16x8_t fa[2][FM], fb[2][FN];
#pragma unroll
  for (int p = 0; p < NSTG; ++p)
#pragma unroll
    for (int q = 0; q < NQ; ++q) DMA1(p, min(p, nk - 1), q);
  wait_vm<(NSTG - 1) * NQ, false>();  // stage 0 has landed
  __syncthreads();
#pragma unroll
  for (int g = 0; g < NF; ++g) FRAG(0, 0, 0, g);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int g = 0; g < NF; ++g) {
      FRAG(1, kt, 1, g);
      MMAG(0, g);
      __builtin_amdgcn_sched_barrier(0);
    }
    // stage kt + 1 has landed; this wave's reads of stage kt are complete
    wait_vm<(NSTG - 2) * NQ, true>();
    __syncthreads();
    const int refill = min(kt + NSTG, nk - 1);
#pragma unroll
    for (int g = 0; g < NF; ++g) {
      FRAG(0, kt + 1, 0, g);
      MMAG(1, g);
      DMA1(kt, refill, g);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef DMA1
#undef FRAG
#undef MMAG
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // fp32 tile out through LDS in passes of PR rows: [row][TN] with the
  // 16-byte chunk index XOR (row & 7), then 16-byte row stores
  constexpr int PR0 = (NSTG * STG) / (TN * 4);
  constexpr int PR = PR0 >= TM ? TM : (PR0 >= 128 ? 128 : 64);
  static_assert(TM % PR == 0 && PR * TN * 4 <= NSTG * STG, "output passes");
  float* st = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int pass = 0; pass < TM / PR; ++pass) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = wm * WTM + i * 32;
      if (rb < pass * PR || rb >= (pass + 1) * PR) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rb - pass * PR + acc_row(r, lane);
          const int col = wn * WTN + j * 32 + lane % 32;
          st[row * TN + (((col >> 2) ^ (row & 7)) << 2) + (col & 3)] = acc[i][j][r];
        }
    }
    __syncthreads();
    constexpr int CH = PR * TN / 4;  // 16-byte chunks in the pass
#pragma unroll
    for (int u = 0; u < CH / 256; ++u) {
      const int q = u * 256 + tid, row = q / (TN / 4), c4 = q % (TN / 4);
      const float4 v = *reinterpret_cast<const float4*>(st + row * TN + ((c4 ^ (row & 7)) << 2));
      *reinterpret_cast<float4*>(P + (long)(tr * TM + pass * PR + row) * ldp + tc * TN + c4 * 4) = v;
    }
    __syncthreads();
  }
}

// Partial token reduction: P[s][bt][r][c] = sum_{t in split s} A[t][r] B[t][c]
// (A, B token-major, column offsets folded into the pointers per batch).
// Batch entries from nb0 on read the second operand pair (A1, B1), as in
// k_tn4; the partials are indexed over both.
template <int BT>
__global__ __launch_bounds__(256, 1) void k_gemm_tn(int T, int tsplit, int tiles1,
                                                    const bf16* __restrict__ A0, long lda0, long sA,
                                                    const bf16* __restrict__ B0, long ldb0, long sB,
                                                    float* __restrict__ P, long ldp, long sP,
                                                    long sS, int nb0, const bf16* __restrict__ A1,
                                                    long lda1, const bf16* __restrict__ B1,
                                                    long ldb1) {
  using C = Cfg<BT, BT, 2, 2>;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
  const int tm = blockIdx.x / tiles1, tn = blockIdx.x % tiles1;
  const bool second = (int)blockIdx.y >= nb0;
  const long bt = second ? (long)blockIdx.y - nb0 : (long)blockIdx.y;
  const long lda = second ? lda1 : lda0, ldb = second ? ldb1 : ldb0;
  const int s = blockIdx.z;
  const bf16* __restrict__ A = (second ? A1 : A0) + bt * sA + tm * BT;
  const bf16* __restrict__ B = (second ? B1 : B0) + bt * sB + tn * BT;
  P += s * sS + (long)blockIdx.y * sP;
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
      mma_slab<C>(As, As + C::A_BYTES, acc, wm, wn, lane);
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

// Per-token block products, out[:, jB + n] = sum_k A[:, jB + k] G_j[n][k]
// (V = U G_P^T, dZ = dS G_R with G := G_R^T).  One workgroup per (block j,
// token range): G_j stays resident in LDS (B/64 K-slabs of [B][64]) while
// token tiles of TOK rows stream through a double-buffered A slab, so the
// operand pipeline never restarts between tiles and G_j is read once.
template <int B, int TOK, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void k_blocks(int T, int width, int tiles_per_wg,
                                                            const bf16* __restrict__ A,
                                                            const bf16* __restrict__ G,
                                                            bf16* __restrict__ Out,
                                                            const float* __restrict__ cscale) {
  constexpr int NTH = 64 * WM * WN;
  constexpr int TM = TOK / WM, TN = B / WN, FM = TM / 32, FN = TN / 32;
  constexpr int NS = B / BK;                    // K-slabs per token tile
  constexpr int G_BYTES = B * B * 2;            // NS slabs of [B][64]
  constexpr int A_SLAB = TOK * ROWB;
  constexpr int RPP = NTH / 8;                  // rows per load pass
  constexpr int PA = TOK / RPP, PG = B / RPP;
  static_assert(PA >= 1 && PG >= 1 && FM >= 1 && FN >= 1, "shape");
  using CF = Cfg<TOK, B, WM, WN>;
  extern __shared__ __align__(16) char smem[];
  char* Gs = smem;
  char* As0 = smem + G_BYTES;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = tid / 8, lc = tid % 8;
  const int j = blockIdx.x;
  const int tile0 = blockIdx.y * tiles_per_wg;
  const int ntiles_total = (T + TOK - 1) / TOK;
  const int ntiles = min(tiles_per_wg, ntiles_total - tile0);
  if (ntiles <= 0) return;
  const bf16* Aj = A + (long)j * B;
  bf16* Oj = Out + (long)j * B;
  // G_j -> registers first (from L2); the first A slabs (from HBM) go out
  // before G's LDS writes wait for G
  const bf16* Gj = G + (long)j * B * B;
  uint4 gv[NS][PG];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int p = 0; p < PG; ++p)
      gv[s][p] = *reinterpret_cast<const uint4*>(Gj + (long)(p * RPP + lr) * B + s * BK + lc * 8);
  // A slabs stream through a ring of four register sets: slab st+5 is
  // requested as soon as slab st+1 leaves its set for LDS, so four slabs are
  // in flight per workgroup while G_j stays resident.  Every step issues the
  // same loads (buffer loads: rows past T read as zeros, steps past the end
  // reload the last slab), a token tile leaves at a fixed step of the ring's
  // turn and the column scales sit in registers, so the wait for a slab
  // counts only the loads issued after it instead of draining the ring.
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const int nsteps = ntiles * NS;
  const int wrows = min(ntiles * TOK, T - tile0 * TOK);
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Aj + (long)tile0 * TOK * width), (short)0, wrows * width * 2, 0x00020000);
  uint4 ra[4][PA];
  auto aload = [&](uint4 (&r)[PA], int step) {  // step = tile * NS + slab
    const int stc = min(step, nsteps - 1);
    const int tr = (stc / NS) * TOK, k0 = (stc % NS) * BK;
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int row = tr + p * RPP + lr;
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsA, (row * width + k0 + lc * 8) * 2, 0, 0);
      r[p] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto astore = [&](const uint4 (&r)[PA], int buf) {
    char* As = As0 + buf * A_SLAB;
#pragma unroll
    for (int p = 0; p < PA; ++p) *reinterpret_cast<uint4*>(As + lds_off(p * RPP + lr, lc)) = r[p];
  };
  // the lane's column scales (b = 256; with b = 128 the registers are
  // short, and the staging below reads them)
  constexpr bool SCV = B == 256;
  float scv[FN];
#pragma unroll
  for (int jj = 0; jj < FN; ++jj)
    scv[jj] = SCV && cscale ? cscale[(long)j * B + wn * TN + jj * 32 + lane % 32] : 1.0f;
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) acc[i][jj] = (f32x16_t){};
  aload(ra[0], 0);
  aload(ra[1], 1);
  aload(ra[2], 2);
  aload(ra[3], 3);
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int p = 0; p < PG; ++p)
      *reinterpret_cast<uint4*>(Gs + s * B * ROWB + lds_off(p * RPP + lr, lc)) = gv[s][p];
  astore(ra[0], 0);
  aload(ra[0], 4);
  __syncthreads();
  constexpr int TPI = 4 / NS;  // token tiles per turn of the ring (four steps)
  static_assert(NS * TPI == 4, "four steps per turn");
  for (int tile = 0; tile < ntiles; tile += TPI) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int st = tile * NS + u;
      mma_slab<CF>(As0 + (u & 1) * A_SLAB, Gs + (u % NS) * B * ROWB, acc, wm, wn, lane);
      // slab st+1 into the other A buffer (free since the last barrier)
      astore(ra[(u + 1) & 3], (u + 1) & 1);
      aload(ra[(u + 1) & 3], st + 5);
      if (u % NS == NS - 1 && (TPI == 1 || tile + u / NS < ntiles)) {
        // token tile complete: the A buffer just consumed stages it in
        // passes of PROWS rows so the global stores cover whole 128-byte
        // row segments; then the accumulators restart
        const int t0 = (tile0 + tile + u / NS) * TOK;
        constexpr int PROWS = A_SLAB / (B * 2);
        char* stg = As0 + (u & 1) * A_SLAB;
        // column scales on the fp32 sums (1 without cscale: x * 1.0f is x)
        if constexpr (SCV) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) acc[i][jj] *= scv[jj];
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < TOK / PROWS; ++p) {
          acc_to_slabs<FM, FN>(acc, stg, PROWS * ROWB, wm * TM, wn * TN, lane, p * PROWS,
                               (p + 1) * PROWS, SCV || !cscale ? nullptr : cscale + (long)j * B);
          __syncthreads();
          slabs_to_global_buf<PROWS, B, NTH>(stg, Oj, width, t0 + p * PROWS, 0, T);
          __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jj = 0; jj < FN; ++jj) acc[i][jj] = (f32x16_t){};
      }
      __syncthreads();
    }
  }
}



// out[e] = sum_{s < S} P[s * stride + e], fixed order
// (n, n0 and stride multiples of 4 and every buffer 16-byte aligned: the
// sums go four at a time, each still in split order)
__global__ void k_reduce_splits(long n, int S, long stride, const float* __restrict__ P,
                                float* __restrict__ out, long n0, float* __restrict__ out1) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  for (long e = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4; e < n;
       e += (long)gridDim.x * blockDim.x * 4) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(P + e);
    for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const f32x4*>(P + s * stride + e);
    if (e < n0) *reinterpret_cast<f32x4*>(out + e) = acc;
    else *reinterpret_cast<f32x4*>(out1 + (e - n0)) = acc;
  }
}

template <typename K>
hipError_t set_lds(K kern, int bytes) {
  return lds_opt_in((const void*)kern, bytes);
}

template <int BM, int BN, int WM, int WN>
hipError_t nt_launch(int batch, int M, int N, int K, const bf16* A, long lda, long sA, const bf16* B,
                     long ldb, long sB, bf16* C, long ldc, long sC, hipStream_t s,
                     const float* cscale, long sS) {
  using CF = Cfg<BM, BN, WM, WN>;
  auto kern = k_gemm_nt<BM, BN, WM, WN>;
  if (cscale && N % BN) return hipErrorInvalidValue;  // the scale is read for whole tiles
  constexpr int lds = CF::LDS;
  static_assert(lds <= 160 * 1024, "LDS budget");
  const hipError_t attr = set_lds(kern, lds);
  if (attr != hipSuccess) return attr;
  const int tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
  hipLaunchKernelGGL(kern, dim3(tilesM * tilesN, batch), dim3(CF::NTH), lds, s, M, N, K, A, lda,
                     sA, B, ldb, sB, C, ldc, sC, tilesM, tilesN, cscale, sS);
  return hipGetLastError();
}

template <int BT>
hipError_t tn_launch(int batch, int D, int T, int S, const bf16* A, long lda, long sA, const bf16* B,
                     long ldb, long sB, float* P, long ldp, long sP, long sS, hipStream_t s,
                     int nb0 = -1, const bf16* A1 = nullptr, long lda1 = 0,
                     const bf16* B1 = nullptr, long ldb1 = 0) {
  using CF = Cfg<BT, BT, 2, 2>;
  auto kern = k_gemm_tn<BT>;
  const hipError_t attr = set_lds(kern, CF::LDS);
  if (attr != hipSuccess) return attr;
  if (nb0 < 0) {  // one operand pair
    nb0 = batch;
    A1 = A, lda1 = lda, B1 = B, ldb1 = ldb;
  }
  const int tiles1 = D / BT;
  const int tsplit = ((T + S - 1) / S + BK - 1) / BK * BK;
  constexpr int lds = CF::LDS;
  hipLaunchKernelGGL(kern, dim3(tiles1 * tiles1, batch, S), dim3(256), lds, s, T, tsplit, tiles1,
                     A, lda, sA, B, ldb, sB, P, ldp, sP, sS, nb0, A1, lda1, B1, ldb1);
  return hipGetLastError();
}

constexpr int NUM_CU = 256;

}  // namespace

bool mfma_nt_ok(int M, int N, int K) { return M > 0 && N % 64 == 0 && K % BK == 0; }

// k_nt4's buffer offsets reach 256 rows * ld * 2 bytes, kept below 2^31
bool nt4_ld_ok(long lda, long ldb, long ldc) {
  return lda > 0 && ldb > 0 && ldc > 0 && lda < (1L << 21) && ldb < (1L << 21) && ldc < (1L << 21);
}

// 4-wave 256 x 256 launcher; LDS: the five 32 KB operand slots (the block
// epilogue stages its tile in the first 128 KB).  BMODE: B's storage (k_nt4).
template <int EPI, int BMODE = 0, bool SC = false>
hipError_t nt4_launch_t(int batch, int M, int N, int K, const bf16* A, long lda, long sA,
                        const void* B, long ldb, long sB, bf16* C, long ldc, long sC,
                        const bf16* Bk, bf16* E, long lde, hipStream_t s, const float* cscale,
                        long sS, int ntmask) {
  auto kern = k_nt4<EPI, BMODE, SC>;
  constexpr int lds = 5 * 256 * ROWB;
  static_assert(lds <= 160 * 1024, "LDS budget");
  const hipError_t attr = set_lds(kern, lds);
  if (attr != hipSuccess) return attr;
  const int tM = (M + 255) / 256, tN = (N + 255) / 256;
  hipLaunchKernelGGL(kern, dim3(tM * tN, batch), dim3(256), lds, s, M, N, K, A, lda, sA, B, ldb,
                     sB, C, ldc, sC, tM, tN, Bk, E, lde, cscale, sS, ntmask);
  return hipGetLastError();
}

// the column scale is a compile-time choice: the scaled staging costs
// registers the plain kernels do not spend
template <int EPI, int BMODE = 0>
hipError_t nt4_launch(int batch, int M, int N, int K, const bf16* A, long lda, long sA,
                      const void* B, long ldb, long sB, bf16* C, long ldc, long sC, const bf16* Bk,
                      bf16* E, long lde, hipStream_t s, const float* cscale = nullptr,
                      long sS = 0, int ntmask = 0) {
  if (cscale)
    return nt4_launch_t<EPI, BMODE, true>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, Bk, E,
                                       lde, s, cscale, sS, ntmask);
  return nt4_launch_t<EPI, BMODE, false>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, Bk, E,
                                      lde, s, nullptr, 0, ntmask);
}

hipError_t launch_mfma_nt(int batch, int M, int N, int K, const bf16* A, long lda, long sA,
                          const bf16* B, long ldb, long sB, bf16* C, long ldc, long sC,
                          hipStream_t s, const float* cscale, long sS) {
  auto tiles = [&](int bm, int bn) { return (long)batch * ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  // the 256 x 256 kernel stays ahead of the 256 x 128 one down to half a
  // tile per CU (4096 x 2048 x 2048: 43 against 52 us)
  if (N % 256 == 0 && tiles(256, 256) >= NUM_CU / 2 && nt4_ld_ok(lda, ldb, ldc))
    return nt4_launch<0>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, nullptr, nullptr, 0,
                         s, cscale, sS);
  if (N % 128 == 0 && tiles(256, 128) >= NUM_CU)
    return nt_launch<256, 128, 2, 2>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s, cscale,
                                     sS);
  if (N % 128 == 0)
    return nt_launch<128, 128, 2, 2>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s, cscale,
                                     sS);
  return nt_launch<128, 64, 2, 2>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s, cscale, sS);
}

bool mfma_nt_block_ok(int M, int N, int K, int b) {
  return (b == 256 || b == 128) && N % 256 == 0 && K % BK == 0 && M > 0 && K < (1 << 21);
}

hipError_t launch_mfma_nt_block(int M, int N, int K, int b, const bf16* A, long lda,
                                const bf16* B, long ldb, bf16* C, long ldc, const bf16* Bk,
                                bf16* E, long lde, hipStream_t s, int ntmask) {
  if (!nt4_ld_ok(lda, ldb, ldc) || (E && !nt4_ld_ok(lda, ldb, lde))) return hipErrorInvalidValue;
  if (!E)
    return nt4_launch<0>(1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, nullptr, nullptr, 0, s,
                         nullptr, 0, ntmask);
  if (b == 128)
    return nt4_launch<2>(1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, Bk, E, lde, s, nullptr, 0,
                         ntmask);
  if (b != 256) return hipErrorInvalidValue;
  return nt4_launch<1>(1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, Bk, E, lde, s, nullptr, 0,
                       ntmask);
}

bool mfma_nt_kmajor_ok(int M, int N, int K, long lda, long ldb, long ldc) {
  return M > 0 && N % 256 == 0 && K % BK == 0 && nt4_ld_ok(lda, ldb, ldc) && ldb >= N &&
         (long)K * ldb * 2 < (1L << 31);
}

hipError_t launch_mfma_nt_kmajor(int M, int N, int K, int b, const bf16* A, long lda,
                                 const bf16* Bkn, long ldb, bf16* C, long ldc, const bf16* Bk,
                                 bf16* E, long lde, hipStream_t s, int ntmask) {
  if (!mfma_nt_kmajor_ok(M, N, K, lda, ldb, ldc) || (E && !nt4_ld_ok(lda, ldb, lde)))
    return hipErrorInvalidValue;
  if (!E)
    return nt4_launch<0, 2>(1, M, N, K, A, lda, 0, Bkn, ldb, 0, C, ldc, 0, nullptr, nullptr, 0, s,
                            nullptr, 0, ntmask);
  if (b == 128)
    return nt4_launch<2, 2>(1, M, N, K, A, lda, 0, Bkn, ldb, 0, C, ldc, 0, Bk, E, lde, s, nullptr,
                            0, ntmask);
  if (b != 256) return hipErrorInvalidValue;
  return nt4_launch<1, 2>(1, M, N, K, A, lda, 0, Bkn, ldb, 0, C, ldc, 0, Bk, E, lde, s, nullptr, 0,
                          ntmask);
}

bool mfma_nt_q_ok(int M, int N, int K, long lda, long ldb, long ldc) {
  return M > 0 && N % 256 == 0 && K % BK == 0 && nt4_ld_ok(lda, ldb, ldc);
}

hipError_t launch_mfma_nt_q(int M, int N, int K, int b, const bf16* A, long lda, const int8_t* Bq,
                            long ldb, bf16* C, long ldc, const float* cscale, const bf16* Bk,
                            bf16* E, long lde, hipStream_t s, int ntmask) {
  if (!mfma_nt_q_ok(M, N, K, lda, ldb, ldc) || (E && !nt4_ld_ok(lda, ldb, lde)))
    return hipErrorInvalidValue;
  if (!E)
    return nt4_launch<0, 1>(1, M, N, K, A, lda, 0, Bq, ldb, 0, C, ldc, 0, nullptr, nullptr, 0, s,
                               cscale, 0, ntmask);
  if (b == 128)
    return nt4_launch<2, 1>(1, M, N, K, A, lda, 0, Bq, ldb, 0, C, ldc, 0, Bk, E, lde, s, cscale, 0,
                            ntmask);
  if (b != 256) return hipErrorInvalidValue;
  return nt4_launch<1, 1>(1, M, N, K, A, lda, 0, Bq, ldb, 0, C, ldc, 0, Bk, E, lde, s, cscale, 0,
                          ntmask);
}

bool mfma_blocks_ok(int b) { return b == 128 || b == 256; }

template <int B, int TOK, int WM, int WN>
hipError_t blocks_launch(int nblk, int T, int width, const bf16* A, const bf16* G, bf16* Out,
                         hipStream_t s, const float* cscale) {
  auto kern = k_blocks<B, TOK, WM, WN>;
  constexpr int lds = B * B * 2 + 2 * TOK * ROWB;
  static_assert(lds <= 160 * 1024, "LDS budget");
  const hipError_t attr = set_lds(kern, lds);
  if (attr != hipSuccess) return attr;
  // token splits per block: each workgroup loads its G_j (about two token
  // tiles' time) and then streams its tiles, one workgroup per CU, so the
  // time goes as rounds of workgroups x (tiles each + 2); take the cheapest
  // (56 blocks: 4 splits in one round rather than 5 in two)
  const int tiles = (T + TOK - 1) / TOK;
  int per = tiles, splits = 1;
  long best = -1;
  for (int want = 1; want <= tiles; ++want) {
    const int p = (tiles + want - 1) / want, sp = (tiles + p - 1) / p;
    const long rounds = ((long)nblk * sp + NUM_CU - 1) / NUM_CU;
    const long cost = rounds * (p + 2);
    if (best < 0 || cost < best || (cost == best && sp < splits)) best = cost, per = p, splits = sp;
  }
  // a workgroup's rows of A lie in one buffer range: per TOK width 2 < 2^31
  while (per > 1 && (long)per * TOK * width * 2 >= (1L << 31)) per = (per + 1) / 2;
  splits = (tiles + per - 1) / per;
  hipLaunchKernelGGL(kern, dim3(nblk, splits), dim3(64 * WM * WN), lds, s, T, width, per, A, G,
                     Out, cscale);
  return hipGetLastError();
}

hipError_t launch_mfma_blocks(int nblk, int T, int width, int b, const bf16* A, const bf16* G,
                              bf16* Out, hipStream_t s, const float* cscale) {
  if (width <= 0 || width >= (1 << 21)) return hipErrorInvalidValue;  // 32-bit buffer offsets
  if (b == 256) return blocks_launch<256, 128, 2, 4>(nblk, T, width, A, G, Out, s, cscale);
  if (b == 128) return blocks_launch<128, 256, 4, 2>(nblk, T, width, A, G, Out, s, cscale);
  return hipErrorInvalidValue;
}

// Tile width of the D >= 256 reduction (k_tn4): the narrowest of 64, 128
// and 256 columns whose tiles still fit one round of the CUs; then as many
// token splits as fill the CUs.  Narrower tiles mean fewer splits, so fewer
// fp32 partials to write and reduce (the tiles of a block share their A
// rows through L2): 32 blocks of 256 take 256 x 64 tiles in 2 splits.
int tn4_width(int batch, int D) {
  const long tiles256 = (long)batch * (D / 256) * (D / 256);
  if (4 * tiles256 <= NUM_CU) return 64;
  return 2 * tiles256 <= NUM_CU ? 128 : 256;
}

// splits of the token range for a D x D (per batch) reduction whose widest
// operand has row pitch `width` (elements)
int tn_splits(int batch, int D, int T, long width) {
  int S;
  if (D >= 256) {
    // k_tn4: fill the CUs once; more splits only add fp32 partials
    const long tiles = (long)batch * (D / 256) * (D / tn4_width(batch, D));
    S = (int)std::max<long>(1, NUM_CU / tiles);
  } else {
    const int BT = D >= 128 ? 128 : 64;
    const long tiles = (long)batch * (D / BT) * (D / BT);
    S = (int)((NUM_CU + tiles - 1) / tiles);
  }
  const int max_s = (T + 255) / 256;  // keep >= 256 tokens per split
  S = S < max_s ? S : max_s;
  if (S < 1) S = 1;
  if (D >= 256 && width > 0) {
    // k_tn4 addresses a split through one buffer range: its tokens (rounded
    // up to 32) times the row pitch stay below 2^31 bytes
    const long tmax = ((1L << 31) - 1) / (2 * width) / 32 * 32;
    const long smin = tmax > 0 ? ((long)T + tmax - 1) / tmax : T;
    if (S < smin) S = (int)smin;
  }
  return S;
}

size_t tn_partial_bytes(int batch, int D, int T, long width) {
  const int S = tn_splits(batch, D, T, width);
  return S > 1 ? (size_t)S * batch * D * D * sizeof(float) : 0;
}

namespace {

template <int TN>
hipError_t tn4_launch_w(int batch, int nb0, int D, int T, int S, const bf16* A0, long lda0,
                        const bf16* B0, long ldb0, const bf16* A1, long lda1, const bf16* B1,
                        long ldb1, float* P, hipStream_t s, float* P1) {
  // four stages: five or six (up to 144 KB of LDS) measured no faster in the
  // layer step, where the reads meet the write-back of the preceding passes
  constexpr int NSTG = 4;
  constexpr int lds = NSTG * 32 * (256 + TN) * 2;  // stages of 32 tokens x (A, B) rows
  static_assert(lds <= 160 * 1024, "LDS budget");
  const hipError_t attr = set_lds(k_tn4<256, TN, NSTG>, lds);
  if (attr != hipSuccess) return attr;
  const long dd = (long)D * D;
  const int tilesN = D / TN, ntiles = (D / 256) * tilesN;
  const int tsplit = ((T + S - 1) / S + 31) / 32 * 32;
  // a split's buffer range (tsplit rows of the widest operand) stays below
  // 2^31 bytes; tn_splits chose S for that, this only guards the invariant
  if ((long)tsplit * std::max(std::max(lda0, ldb0), std::max(lda1, ldb1)) * 2 >= (1L << 31))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_tn4<256, TN, NSTG>), dim3(ntiles * batch * S), dim3(256), lds, s, T, tsplit,
                     tilesN, ntiles, batch, A0, lda0, (long)D, B0, ldb0, (long)D, P, (long)D, dd,
                     dd * batch, nb0, A1, lda1, B1, ldb1, P1);
  return hipGetLastError();
}

// k_tn4 over `batch` D x D products (D a multiple of 256) in S token splits;
// entries from nb0 on read (A1, B1).  Writes P[s][batch][D][D].
hipError_t tn4_launch(int batch, int nb0, int D, int T, int S, const bf16* A0, long lda0,
                      const bf16* B0, long ldb0, const bf16* A1, long lda1, const bf16* B1,
                      long ldb1, float* P, hipStream_t s, float* P1 = nullptr) {
  const int w = tn4_width(batch, D);
  if (w == 64)
    return tn4_launch_w<64>(batch, nb0, D, T, S, A0, lda0, B0, ldb0, A1, lda1, B1, ldb1, P, s, P1);
  if (w == 128)
    return tn4_launch_w<128>(batch, nb0, D, T, S, A0, lda0, B0, ldb0, A1, lda1, B1, ldb1, P, s, P1);
  return tn4_launch_w<256>(batch, nb0, D, T, S, A0, lda0, B0, ldb0, A1, lda1, B1, ldb1, P, s, P1);
}

// out0 = the first n0 sums over S partials of stride n, out1 = the rest
hipError_t reduce_launch(long n, int S, const float* P, float* out0, long n0, float* out1,
                         hipStream_t s) {
  if (n % 4 || n0 % 4) return hipErrorInvalidValue;
  const int grid = (int)std::min<long>((n / 4 + 255) / 256, 4096);
  hipLaunchKernelGGL(k_reduce_splits, dim3(grid), dim3(256), 0, s, n, S, n, P, out0, n0, out1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_tn(int batch, int D, int T, const bf16* A, long lda, long sA, const bf16* B,
                          long ldb, long sB, float* out, float* partials, hipStream_t s) {
  const int S = tn_splits(batch, D, T, std::max(lda, ldb));
  const long dd = (long)D * D;
  float* P = S > 1 ? partials : out;
  hipError_t e;
  if (D >= 256) {
    if (sA != D || sB != D) return hipErrorInvalidValue;
    e = tn4_launch(batch, batch, D, T, S, A, lda, B, ldb, A, lda, B, ldb, P, s);
  } else if (D == 64) {
    e = tn_launch<64>(batch, D, T, S, A, lda, sA, B, ldb, sB, P, D, dd, dd * batch, s);
  } else {
    e = tn_launch<128>(batch, D, T, S, A, lda, sA, B, ldb, sB, P, D, dd, dd * batch, s);
  }
  if (e != hipSuccess || S == 1) return e;
  return reduce_launch(dd * batch, S, P, out, dd * batch, nullptr, s);
}

bool mfma_tn2_ok(int nb0, int nb1, int D, int T, long width) {
  return D % 256 == 0 || ((D == 64 || D == 128) && tn_splits(nb0 + nb1, D, T, width) > 1);
}

hipError_t launch_mfma_tn2(int nb0, int nb1, int D, int T, const bf16* A0, long lda0,
                           const bf16* B0, long ldb0, float* out0, const bf16* A1, long lda1,
                           const bf16* B1, long ldb1, float* out1, float* partials,
                           hipStream_t s) {
  const long width = std::max(std::max(lda0, ldb0), std::max(lda1, ldb1));
  if (!mfma_tn2_ok(nb0, nb1, D, T, width)) return hipErrorInvalidValue;
  const int batch = nb0 + nb1;
  const int S = tn_splits(batch, D, T, width);
  const long dd = (long)D * D;
  if (S == 1)  // enough tiles without splitting the tokens: sums straight to out0, out1
    return tn4_launch(batch, nb0, D, T, 1, A0, lda0, B0, ldb0, A1, lda1, B1, ldb1, out0, s, out1);
  hipError_t e;
  if (D >= 256)
    e = tn4_launch(batch, nb0, D, T, S, A0, lda0, B0, ldb0, A1, lda1, B1, ldb1, partials, s);
  else if (D == 64)
    e = tn_launch<64>(batch, D, T, S, A0, lda0, D, B0, ldb0, D, partials, D, dd, dd * batch, s, nb0,
                      A1, lda1, B1, ldb1);
  else
    e = tn_launch<128>(batch, D, T, S, A0, lda0, D, B0, ldb0, D, partials, D, dd, dd * batch, s,
                       nb0, A1, lda1, B1, ldb1);
  if (e != hipSuccess) return e;
  return reduce_launch(dd * batch, S, partials, out0, dd * nb0, out1, s);
}

}  // namespace poetx
