// C ABI of libpoetx.so: host-side validation, workspace layout and dispatch.
// Declarations and argument documentation: include/poetx.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include "../../include/poetx.h"
#include "kernels.h"

namespace poetx {

hipError_t lds_opt_in(const void* kern, int bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  int dev = 0;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) return ge;
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int>, hipError_t> done;
  const std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(kern, dev, bytes);
  const auto it = done.find(key);
  if (it != done.end()) return it->second;
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  done.emplace(key, e);
  return e;
}

}  // namespace poetx

using namespace poetx;

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

int32_t ok() {
  g_err[0] = '\0';
  return POETX_OK;
}

int32_t dev_fail(hipError_t e, const char* where) {
  return fail(POETX_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define NEED_PTR(p)                                                                  \
  do {                                                                               \
    if (!(p)) return fail(POETX_ERR_ARG, "%s: null pointer '%s'", fn, #p);           \
    if (!aligned16(p)) return fail(POETX_ERR_ARG, "%s: '%s' not 16-byte aligned", fn, #p); \
  } while (0)
#define OPT_PTR(p)                                                                   \
  do {                                                                               \
    if ((p) && !aligned16(p))                                                        \
      return fail(POETX_ERR_ARG, "%s: '%s' not 16-byte aligned", fn, #p);            \
  } while (0)

bool b_supported(int b) {
  return b == 8 || b == 16 || b == 32 || b == 64 || b == 128 || b == 256 || b == 512;
}

constexpr int K_MAX = 8;
constexpr int SMALL_B_MAX = 64;  // LDS-resident fp32 Cayley-Neumann kernels

size_t es_of(int act) { return act == POETX_BF16 ? 2 : 4; }

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// the MFMA Cayley-Neumann panels run for bf16 blocks of 64..512
bool cnp_uses_panel(int b, int act) { return act == POETX_BF16 && b >= 64; }

int32_t check_cnp_args(const char* fn, int32_t nblk, int32_t b, int32_t k, int32_t act) {
  if (nblk < 1) return fail(POETX_ERR_ARG, "%s: nblk=%d < 1", fn, nblk);
  if (!b_supported(b)) return fail(POETX_ERR_ARG, "%s: b=%d not in {8,16,32,64,128,256,512}", fn, b);
  if (k < 0 || k > K_MAX) return fail(POETX_ERR_ARG, "%s: k=%d outside 0..%d", fn, k, K_MAX);
  if (act != POETX_F32 && act != POETX_BF16) return fail(POETX_ERR_ARG, "%s: dtype %d", fn, act);
  if (act == POETX_F32 && b > SMALL_B_MAX)
    return fail(POETX_ERR_UNSUPPORTED, "%s: float32 blocks need b <= %d (b=%d)", fn, SMALL_B_MAX, b);
  return POETX_OK;
}

int32_t check_shape(const char* fn, const poetx_shape* sh) {
  if (!sh) return fail(POETX_ERR_ARG, "%s: null shape", fn);
  if (sh->m < 1 || sh->n < 1 || sh->T < 1)
    return fail(POETX_ERR_ARG, "%s: m=%d n=%d T=%d must be >= 1", fn, sh->m, sh->n, sh->T);
  if (!b_supported(sh->b))
    return fail(POETX_ERR_ARG, "%s: b=%d not in {8,16,32,64,128,256,512}", fn, sh->b);
  if (sh->m % sh->b || sh->n % sh->b)
    return fail(POETX_ERR_ARG, "%s: m=%d and n=%d must be multiples of b=%d", fn, sh->m, sh->n, sh->b);
  if (sh->k < 0 || sh->k > K_MAX) return fail(POETX_ERR_ARG, "%s: k=%d outside 0..%d", fn, sh->k, K_MAX);
  if (sh->act != POETX_F32 && sh->act != POETX_BF16)
    return fail(POETX_ERR_ARG, "%s: act dtype %d", fn, sh->act);
  if (sh->act == POETX_F32 && sh->b > SMALL_B_MAX)
    return fail(POETX_ERR_UNSUPPORTED, "%s: float32 layers need b <= %d (b=%d)", fn, SMALL_B_MAX, sh->b);
  return POETX_OK;
}

size_t cnp_ws(int nblk, int b, int k, int which, int act) {
  const size_t bb = (size_t)b * b;
  if (!cnp_uses_panel(b, act)) return which == 0 ? 0 : align_up((size_t)nblk * k * bb * 4);
  if (which == 0) return align_up(nblk * bb * 2);
  return align_up(nblk * bb * 2) + align_up((size_t)k * nblk * bb * 2) + align_up(nblk * bb * 4);
}


// ---- timing hook: stage-boundary events, per calling thread ---------------
thread_local hipEvent_t g_stage_ev[8];
thread_local int g_stage_on = 0;

inline void mark(int i, hipStream_t s) {
  if (g_stage_on) (void)hipEventRecord(g_stage_ev[i], s);
}

// MFMA kernels carry bf16 layers with b >= 64; everything else takes the
// portable tiled kernels
inline bool use_mfma(const poetx_shape* sh) { return sh->act == POETX_BF16 && sh->b >= 64; }

// workspace layout of the layer calls
// (xmem: the forward's Z, or the backward's recomputed Z, lives in the
// workspace instead of the saved buffer)
struct FwdWs { size_t V, S, Z, Gf, total; };
struct BwdWs { size_t dS, dZ, dV, dU, part, Z, Gf, total; };

// poetx_set_fused_gather: the gather and its block products as one pass
std::atomic<int> g_fused_gather{0};

// a side of width W gathers and forms its block products in one pass
// (gather_blocks.hip: bf16, b = 256, W a multiple of 512 up to 4096) when
// that form is selected
inline bool fused_gather(const poetx_shape* sh, int W) {
  return g_fused_gather.load(std::memory_order_relaxed) && use_mfma(sh) &&
         gather_blocks_ok(W, sh->b);
}

FwdWs fwd_ws(const poetx_shape* sh, bool xmem = false) {
  const size_t es = es_of(sh->act), T = sh->T;
  FwdWs w;
  w.V = 0;
  w.S = w.V + align_up(T * sh->n * es);
  w.Z = w.S + align_up(T * sh->m * es);
  w.Gf = w.Z + (xmem ? align_up(T * sh->m * es) : 0);
  w.total = w.Gf + (fused_gather(sh, sh->n) ? align_up(gather_blocks_ws_bytes(sh->n, sh->b)) : 0);
  return w;
}

BwdWs bwd_ws(const poetx_shape* sh, bool xmem = false) {
  const size_t es = es_of(sh->act), T = sh->T;
  BwdWs w;
  w.dS = 0;
  w.dZ = w.dS + align_up(T * sh->m * es);
  w.dV = w.dZ + align_up(T * sh->m * es);
  w.dU = w.dV + align_up(T * sh->n * es);
  w.part = w.dU + align_up(T * sh->n * es);
  size_t part = 0;
  if (use_mfma(sh)) {
    const long wmax = std::max(sh->m, sh->n);  // the widest operand pitch of each reduction
    const size_t pr = tn_partial_bytes(sh->m / sh->b, sh->b, sh->T, sh->m);
    const size_t pp = tn_partial_bytes(sh->n / sh->b, sh->b, sh->T, sh->n);
    const size_t pb = tn_partial_bytes(sh->m / sh->b + sh->n / sh->b, sh->b, sh->T, wmax);
    part = align_up(std::max(pb, std::max(pr, pp)));
  }
  w.Z = w.part + part;
  w.Gf = w.Z + (xmem ? align_up((size_t)sh->T * sh->m * es) : 0);
  // G in fragment order: the R side's for dy, and in the memory-saving mode
  // the P side's for the recompute of V (one after the other)
  size_t gf = fused_gather(sh, sh->m) ? gather_blocks_ws_bytes(sh->m, sh->b) : 0;
  if (xmem && fused_gather(sh, sh->n)) gf = std::max(gf, gather_blocks_ws_bytes(sh->n, sh->b));
  w.total = w.Gf + align_up(gf);
  return w;
}

// merge: two [m][n] scratch matrices
size_t merge_ws(const poetx_shape* sh) {
  return 2 * align_up((size_t)sh->m * sh->n * es_of(sh->act));
}

// saved activations: U = x[:, pi_P] then Z
size_t saved_U(const poetx_shape*) { return 0; }
size_t saved_Z(const poetx_shape* sh) { return align_up((size_t)sh->T * sh->n * es_of(sh->act)); }
size_t saved_total(const poetx_shape* sh, bool xmem = false) {
  return xmem ? saved_Z(sh) : saved_Z(sh) + align_up((size_t)sh->T * sh->m * es_of(sh->act));
}

template <typename TS> TS* at(void* base, size_t off) {
  return reinterpret_cast<TS*>(reinterpret_cast<char*>(base) + off);
}
template <typename TS> const TS* at(const void* base, size_t off) {
  return reinterpret_cast<const TS*>(reinterpret_cast<const char*>(base) + off);
}

// ---- the layer passes, per storage type ---------------------------------
// The fixed weight of a layer call: W0f (and W0fT) in the activation type,
// or an int8 pair q_f / q_fT with one fp32 scale per output row, s_f.
template <typename TS>
struct Weight {
  const TS* f = nullptr;       // W0f  [m][n]
  const TS* fT = nullptr;      // W0fT [n][m]
  const int8_t* q = nullptr;   // q_f  [m][n]
  const int8_t* qT = nullptr;  // q_fT [n][m]
  const float* s = nullptr;    // s_f  [m]
  bool quant() const { return s != nullptr; }
};

// C[bt] = A[bt] B[bt]^T (column c of C[bt] scaled by cscale[bt * sS + c]
// when cscale is set: MFMA path only)
template <typename TS>
hipError_t nt(bool mfma, int batch, int M, int N, int K, const TS* A, long lda, long sA,
              const TS* B, long ldb, long sB, TS* C, long ldc, long sC, hipStream_t s,
              const float* cscale = nullptr, long sS = 0) {
  if constexpr (sizeof(TS) == 2) {
    if (mfma && mfma_nt_ok(M, N, K))
      return launch_mfma_nt(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s, cscale, sS);
  }
  if (cscale) return hipErrorInvalidValue;
  return launch_simple_nt<TS>(batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, s);
}

// Out[:, jb + n] = sum_k A[:, jb + k] Gb[j][n][k] for every block j (A and
// Out row pitch `width`): the per-token block products (output column c
// scaled by cscale[c] when cscale is set)
template <typename TS>
hipError_t blocks(bool mfma, int nblk, int T, int width, int b, const TS* A, const TS* Gb, TS* Out,
                  hipStream_t s, const float* cscale = nullptr) {
  if constexpr (sizeof(TS) == 2) {
    if (mfma && mfma_blocks_ok(b))
      return launch_mfma_blocks(nblk, T, width, b, A, Gb, Out, s, cscale);
  }
  return nt<TS>(mfma, nblk, T, b, b, A, width, b, Gb, b, (long)b * b, Out, width, b, s, cscale, b);
}

// Z = V W0f^T (T x m), and with the block epilogue (b = 128 or 256, S
// set) S_i = Z_i G_Ri^T in the same kernel; false from `fused` when the
// caller must form S itself
template <typename TS>
hipError_t dense_fwd(bool mf, const poetx_shape* sh, const TS* V, const Weight<TS>& W, TS* Z,
                     const TS* G_R, TS* S, bool& fused, hipStream_t s) {
  const int m = sh->m, n = sh->n, b = sh->b, T = sh->T;
  fused = false;
  if constexpr (sizeof(TS) == 2) {
    if (W.quant()) {
      fused = S && mfma_nt_block_ok(T, m, n, b);
      return launch_mfma_nt_q(T, m, n, b, V, n, W.q, n, Z, m, W.s, fused ? G_R : nullptr,
                              fused ? S : nullptr, m, s);
    }
    if (mf && mfma_nt_block_ok(T, m, n, b)) {
      fused = S != nullptr;
      return launch_mfma_nt_block(T, m, n, b, V, n, W.f, n, Z, m, fused ? G_R : nullptr,
                                  fused ? S : nullptr, m, s);
    }
  }
  return nt<TS>(mf, 1, T, m, n, V, n, 0, W.f, n, 0, Z, m, 0, s);
}

// out[bt] = A_bt^T B_bt over T tokens, D x D blocks at column offsets bt*D
template <typename TS>
hipError_t tn(bool mfma, int batch, int D, int T, const TS* A, long lda, const TS* B, long ldb,
              float* out, float* partials, hipStream_t s) {
  if constexpr (sizeof(TS) == 2) {
    if (mfma) return launch_mfma_tn(batch, D, T, A, lda, D, B, ldb, D, out, partials, s);
  }
  return launch_simple_tn<TS>(batch, D, D, T, A, lda, D, B, ldb, D, out, D, (long)D * D, s);
}

template <typename TS>
int32_t layer_fwd_impl(const poetx_shape* sh, const TS* x, const TS* G_P, const TS* G_R,
                       const Weight<TS>& W, const int32_t* perm_P, const int32_t* perm_R_inv, TS* y,
                       void* saved, void* ws, hipStream_t s, bool xmem) {
  const int m = sh->m, n = sh->n, b = sh->b, T = sh->T;
  const int es = (int)sizeof(TS);
  const bool mf = use_mfma(sh);
  const FwdWs w = fwd_ws(sh, xmem);
  TS* U = at<TS>(saved, saved_U(sh));
  TS* Z = xmem ? at<TS>(ws, w.Z) : at<TS>(saved, saved_Z(sh));
  TS* V = at<TS>(ws, w.V);
  TS* S = at<TS>(ws, w.S);
  const long bb = (long)b * b;
  hipError_t e;
  mark(0, s);
  bool gathered = false;
  if constexpr (sizeof(TS) == 2) {
    if (fused_gather(sh, n)) {
      // U = x[:, pi_P] and V_j = U_j G_Pj^T in one pass
      if ((e = launch_gather_blocks(T, n, x, perm_P, U, G_P, at<TS>(ws, w.Gf), V, nullptr, s)) !=
          hipSuccess)
        return dev_fail(e, "gather x + P-side blocks");
      gathered = true;
    }
  }
  if (!gathered) {
    // U = x[:, pi_P] (plain stores: the block pass reads U next)
    if ((e = launch_permute_cols(T, n, es, x, perm_P, U, s, false)) != hipSuccess)
      return dev_fail(e, "gather x");
  }
  mark(1, s);
  // V_j = U_j G_Pj^T
  if (!gathered && (e = blocks<TS>(mf, n / b, T, n, b, U, G_P, V, s)) != hipSuccess)
    return dev_fail(e, "P-side blocks");
  mark(2, s);
  {
    // Z = V W0f^T and, where the dense kernel carries the block epilogue,
    // S_i = Z_i G_Ri^T in the same kernel
    bool fused = false;
    if ((e = dense_fwd<TS>(mf, sh, V, W, Z, G_R, S, fused, s)) != hipSuccess)
      return dev_fail(e, "W0 product");
    mark(3, s);
    // S_i = Z_i G_Ri^T
    if (!fused && (e = blocks<TS>(mf, m / b, T, m, b, Z, G_R, S, s)) != hipSuccess)
      return dev_fail(e, "R-side blocks");
    mark(4, s);
  }
  // y[:, pi_R[c]] = S[:, c]  <=>  y = S[:, pi_R^{-1}]
  if ((e = launch_permute_cols(T, m, es, S, perm_R_inv, y, s)) != hipSuccess)
    return dev_fail(e, "scatter y");
  mark(5, s);
  return ok();
}

template <typename TS>
int32_t layer_bwd_impl(const poetx_shape* sh, const TS* dy, const TS* GT_P, const TS* GT_R,
                       const Weight<TS>& W, const int32_t* perm_P_inv, const int32_t* perm_R,
                       const void* saved, TS* dx, float* dG_P, float* dG_R, void* ws,
                       hipStream_t s, const TS* G_P = nullptr) {
  const int m = sh->m, n = sh->n, b = sh->b, T = sh->T;
  const int es = (int)sizeof(TS);
  const bool mf = use_mfma(sh);
  const bool xmem = G_P != nullptr;
  const BwdWs w = bwd_ws(sh, xmem);
  const TS* U = at<TS>(saved, saved_U(sh));
  TS* dS = at<TS>(ws, w.dS);
  TS* dZ = at<TS>(ws, w.dZ);
  TS* dV = at<TS>(ws, w.dV);
  TS* dU = at<TS>(ws, w.dU);
  float* part = at<float>(ws, w.part);
  const long bb = (long)b * b;
  hipError_t e;
  const TS* Z;
  if (xmem) {
    // recompute V = U G_P^T (into dU's space, free until the end) and
    // Z = V W0f^T with the kernels the forward used, so Z is bitwise the same
    TS* V = dU;
    TS* Zr = at<TS>(ws, w.Z);
    bool done = false;
    if constexpr (sizeof(TS) == 2) {
      if (fused_gather(sh, n)) {
        // the forward's kernel with the identity map: bitwise its V
        if ((e = launch_gather_blocks(T, n, U, nullptr, nullptr, G_P, at<TS>(ws, w.Gf), V,
                                      nullptr, s)) != hipSuccess)
          return dev_fail(e, "recompute V");
        done = true;
      }
    }
    if (!done && (e = blocks<TS>(mf, n / b, T, n, b, U, G_P, V, s)) != hipSuccess)
      return dev_fail(e, "recompute V");
    bool fused = false;
    if ((e = dense_fwd<TS>(mf, sh, V, W, Zr, nullptr, nullptr, fused, s)) != hipSuccess)
      return dev_fail(e, "recompute Z");
    Z = Zr;
  } else {
    Z = at<TS>(saved, saved_Z(sh));
  }
  mark(0, s);
  // dS = dy[:, pi_R], then dZ_i = dS_i G_Ri (B operand G_Ri^T).  An int8
  // weight W0f = diag(s_f) q_f gives dV = dZ W0f = (dZ diag(s_f)) q_f: the
  // scale goes on dZ's columns here, where it is one multiply per element
  // before rounding.
  bool gathered = false;
  if constexpr (sizeof(TS) == 2) {
    if (fused_gather(sh, m)) {
      if ((e = launch_gather_blocks(T, m, dy, perm_R, dS, GT_R, at<TS>(ws, w.Gf), dZ, W.s, s)) !=
          hipSuccess)
        return dev_fail(e, "gather dy + R-side blocks (bwd)");
      gathered = true;
    }
  }
  if (!gathered && (e = launch_permute_cols(T, m, es, dy, perm_R, dS, s, false)) != hipSuccess)
    return dev_fail(e, "gather dy");
  mark(1, s);
  if (!gathered && (e = blocks<TS>(mf, m / b, T, m, b, dS, GT_R, dZ, s, W.s)) != hipSuccess)
    return dev_fail(e, "R-side blocks (bwd)");
  mark(2, s);
  // dG_Ri = dS_i^T Z_i.  On the MFMA path dG_R waits for dG_P and the two
  // run as one launch (mfma_tn2_ok): half the fp32 partials of two launches
  // and one reduction pass, or none when the launch needs no token split
  // (dS and Z stay untouched in between).
  bool dg_joint = false;
  if constexpr (sizeof(TS) == 2) dg_joint = mf && mfma_tn2_ok(m / b, n / b, b, T, std::max(m, n));
  if (!dg_joint && (e = tn<TS>(mf, m / b, b, T, dS, m, Z, m, dG_R, part, s)) != hipSuccess)
    return dev_fail(e, "dG_R");
  mark(3, s);
  {
    // dV = dZ W0f and, where the dense kernel carries the block epilogue
    // (b = 128, 256), dU_j = dV_j G_Pj in the same kernel.  dU goes out
    // non-temporally: the dG reduction runs between it and the dx scatter,
    // and dirty dU lines in the last-level cache would have to be written
    // back to make room for that pass's reads.  The weight is
    // read as W0fT (N-major) when the caller keeps that copy, else straight
    // from W0f (K-major): the same products in the same order.
    bool fused = false, dv_done = false;
    if constexpr (sizeof(TS) == 2) {
      const bool epi = mfma_nt_block_ok(T, n, m, b);
      if (W.quant()) {
        // dV = dZ' q_f (B operand q_fT)
        fused = epi;
        if ((e = launch_mfma_nt_q(T, n, m, b, dZ, m, W.qT, m, dV, n, nullptr,
                                  fused ? GT_P : nullptr, fused ? dU : nullptr, n, s, 2)) !=
            hipSuccess)
          return dev_fail(e, "W0 product (bwd)");
        dv_done = true;
      } else if (mf && W.fT && epi) {
        if ((e = launch_mfma_nt_block(T, n, m, b, dZ, m, W.fT, m, dV, n, GT_P, dU, n, s, 2)) !=
            hipSuccess)
          return dev_fail(e, "W0 product + P-side blocks (bwd)");
        fused = dv_done = true;
      } else if (mf && !W.fT && mfma_nt_kmajor_ok(T, n, m, m, n, n)) {
        fused = epi;
        if ((e = launch_mfma_nt_kmajor(T, n, m, b, dZ, m, W.f, n, dV, n, fused ? GT_P : nullptr,
                                       fused ? dU : nullptr, n, s, 2)) != hipSuccess)
          return dev_fail(e, "W0 product (bwd)");
        dv_done = true;
      }
    }
    if (!dv_done) {
      e = W.fT ? nt<TS>(mf, 1, T, n, m, dZ, m, 0, W.fT, m, 0, dV, n, 0, s)
               : launch_simple_nt<TS>(1, T, n, m, dZ, m, 0, W.f, n, 0, dV, n, 0, s, true);
      if (e != hipSuccess) return dev_fail(e, "W0 product (bwd)");
    }
    mark(4, s);
    // dU_j = dV_j G_Pj
    if (!fused && (e = blocks<TS>(mf, n / b, T, n, b, dV, GT_P, dU, s)) != hipSuccess)
      return dev_fail(e, "P-side blocks (bwd)");
  }
  mark(5, s);
  // dG_Pj = dV_j^T U_j
  if constexpr (sizeof(TS) == 2) {
    if (dg_joint) {
      if ((e = launch_mfma_tn2(m / b, n / b, b, T, dS, m, Z, m, dG_R, dV, n, U, n, dG_P, part, s)) !=
          hipSuccess)
        return dev_fail(e, "dG_R and dG_P");
    }
  }
  if (!dg_joint && (e = tn<TS>(mf, n / b, b, T, dV, n, U, n, dG_P, part, s)) != hipSuccess)
    return dev_fail(e, "dG_P");
  mark(6, s);
  // dx[:, pi_P[c]] = dU[:, c]  <=>  dx = dU[:, pi_P^{-1}]
  if ((e = launch_permute_cols(T, n, es, dU, perm_P_inv, dx, s)) != hipSuccess)
    return dev_fail(e, "scatter dx");
  mark(7, s);
  return ok();
}

// W0_out = Pi_R^T BD(G_R) W0f BD(G_P) Pi_P
template <typename TS>
int32_t merge_impl(const poetx_shape* sh, const TS* W0f, const TS* G_R, const TS* GT_P,
                   const int32_t* perm_R_inv, const int32_t* perm_P_inv, TS* W0_out, void* ws,
                   hipStream_t s) {
  const int m = sh->m, n = sh->n, b = sh->b;
  const int es = (int)sizeof(TS);
  const bool mf = use_mfma(sh);
  TS* A = at<TS>(ws, 0);
  TS* Bm = at<TS>(ws, align_up((size_t)m * n * es));
  hipError_t e;
  // A = W0f BD(G_P): the rows of W0f are the "tokens" of a P-side block
  // product with B operand G_P^T
  if ((e = blocks<TS>(mf, n / b, m, n, b, W0f, GT_P, A, s)) != hipSuccess)
    return dev_fail(e, "merge: W0f BD(G_P)");
  if ((e = launch_transpose(m, n, es, A, Bm, s)) != hipSuccess) return dev_fail(e, "merge: transpose");
  // A = (BD(G_R) W0f BD(G_P))^T = Bm BD(G_R)^T, [n][m]
  if ((e = blocks<TS>(mf, m / b, n, m, b, Bm, G_R, A, s)) != hipSuccess)
    return dev_fail(e, "merge: BD(G_R) rows");
  if ((e = launch_transpose(n, m, es, A, Bm, s)) != hipSuccess) return dev_fail(e, "merge: transpose");
  if ((e = launch_permute_rows_cols(m, n, es, Bm, perm_R_inv, perm_P_inv, W0_out, s)) != hipSuccess)
    return dev_fail(e, "merge: unfold");
  return ok();
}

// the CNP backward; q_ready: ws already holds the forward's unpacked Q
int32_t cnp_bwd_impl(const char* fn, int32_t nblk, int32_t b, int32_t k, const float* theta,
                     const float* dG, float* dtheta, int32_t accumulate, int32_t prec, void* ws,
                     size_t ws_bytes, poetx_stream_t stream, bool q_ready) {
  const int32_t act = prec;
  int32_t st = check_cnp_args(fn, nblk, b, k, act);
  if (st != POETX_OK) return st;
  NEED_PTR(theta);
  NEED_PTR(dG);
  NEED_PTR(dtheta);
  const size_t need = cnp_ws(nblk, b, k, 1, act);
  if (need) {
    NEED_PTR(ws);
    if (ws_bytes < need) return fail(POETX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (cnp_uses_panel(b, act)) {
    const size_t bb = (size_t)b * b;
    bf16* Qg = (bf16*)ws;  // the forward's workspace holds the same Q at the same place
    bf16* F = at<bf16>(ws, align_up(nblk * bb * 2));
    float* dQ = at<float>(ws, align_up(nblk * bb * 2) + align_up((size_t)k * nblk * bb * 2));
    e = launch_cnp_panel_bwd(nblk, b, k, theta, dG, dtheta, accumulate, Qg, F, dQ, q_ready, s);
  } else {
    e = launch_cnp_small_bwd(nblk, b, k, theta, dG, dtheta, accumulate, (float*)ws, s);
  }
  if (e != hipSuccess) return dev_fail(e, fn);
  return ok();
}

// dispatch of the CNP forward once the arguments are checked (ws: the
// unpacked-Q scratch, at least cnp_ws(nblk, b, k, 0, g_dtype) bytes)
int32_t cnp_fwd_launch(const char* fn, int32_t nblk, int32_t b, int32_t k, const float* theta,
                       void* G, void* GT, int32_t g_dtype, void* ws, hipStream_t s) {
  hipError_t e;
  if (cnp_uses_panel(b, g_dtype))
    e = launch_cnp_panel_fwd(nblk, b, k, theta, (bf16*)G, (bf16*)GT, (bf16*)ws, s);
  else if (g_dtype == POETX_F32)
    e = launch_cnp_small_fwd<float>(nblk, b, k, theta, (float*)G, (float*)GT, s);
  else
    e = launch_cnp_small_fwd<bf16>(nblk, b, k, theta, (bf16*)G, (bf16*)GT, s);
  if (e != hipSuccess) return dev_fail(e, fn);
  return ok();
}

}  // namespace

// ---- library-owned scratch of poetx_cnp_fwd_noalloc -----------------------
// One copy per GPU, part of the library's code object: it exists on a device
// from the library's load there until the process ends.  In host code the
// name `scratch` stands for a host-side shadow, not device memory, so host
// code never hands it to a kernel, a memset or a copy: every use goes
// through the device address hipGetSymbolAddress returns, looked up once per
// device with that device current.
static __device__ __align__(256) unsigned char scratch[POETX_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};

// the device address of `scratch` on the calling thread's current device
int32_t scratch_on_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dev_fail(e, fn);
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(POETX_ERR_DEVICE, "%s: device %d outside 0..%d", fn, dev, SCRATCH_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return dev_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(POETX_ERR_DEVICE, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return POETX_OK;
}

}  // namespace

extern "C" {

int32_t poetx_abi_version(void) { return POETX_ABI_VERSION; }

const char* poetx_status_str(int32_t st) {
  switch (st) {
    case POETX_OK: return "POETX_OK";
    case POETX_ERR_ARG: return "POETX_ERR_ARG";
    case POETX_ERR_UNSUPPORTED: return "POETX_ERR_UNSUPPORTED";
    case POETX_ERR_WORKSPACE: return "POETX_ERR_WORKSPACE";
    case POETX_ERR_DEVICE: return "POETX_ERR_DEVICE";
    default: return "POETX_UNKNOWN_STATUS";
  }
}

const char* poetx_last_error(void) { return g_err; }

size_t poetx_cnp_workspace_bytes(int32_t nblk, int32_t b, int32_t k, int32_t which, int32_t act) {
  if (which != 0 && which != 1) return 0;
  if (check_cnp_args("poetx_cnp_workspace_bytes", nblk, b, k, act) != POETX_OK) return 0;
  return cnp_ws(nblk, b, k, which, act);
}

int32_t poetx_cnp_fwd(int32_t nblk, int32_t b, int32_t k, const float* theta, void* G, void* GT,
                      int32_t g_dtype, void* ws, size_t ws_bytes, poetx_stream_t stream) {
  const char* fn = "poetx_cnp_fwd";
  int32_t st = check_cnp_args(fn, nblk, b, k, g_dtype);
  if (st != POETX_OK) return st;
  NEED_PTR(theta);
  NEED_PTR(G);
  OPT_PTR(GT);
  const size_t need = cnp_ws(nblk, b, k, 0, g_dtype);
  if (need) {
    NEED_PTR(ws);
    if (ws_bytes < need) return fail(POETX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  }
  return cnp_fwd_launch(fn, nblk, b, k, theta, G, GT, g_dtype, ws, (hipStream_t)stream);
}

int32_t poetx_cnp_fwd_noalloc(int32_t nblk, int32_t b, int32_t k, const float* theta, void* G,
                              void* GT, int32_t g_dtype, poetx_stream_t stream) {
  const char* fn = "poetx_cnp_fwd_noalloc";
  int32_t st = check_cnp_args(fn, nblk, b, k, g_dtype);
  if (st != POETX_OK) return st;
  NEED_PTR(theta);
  NEED_PTR(G);
  OPT_PTR(GT);
  const size_t need = cnp_ws(nblk, b, k, 0, g_dtype);
  if (need > (size_t)POETX_NOALLOC_SCRATCH_BYTES)
    return fail(POETX_ERR_WORKSPACE, "%s: %zu bytes of scratch needed, the library's array holds %zu",
                fn, need, (size_t)POETX_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need) {
    st = scratch_on_current_device(fn, &ws);
    if (st != POETX_OK) return st;
  }
  return cnp_fwd_launch(fn, nblk, b, k, theta, G, GT, g_dtype, ws, (hipStream_t)stream);
}


int32_t poetx_cnp_bwd(int32_t nblk, int32_t b, int32_t k, const float* theta, const float* dG,
                      float* dtheta, int32_t accumulate, int32_t prec, void* ws,
                      size_t ws_bytes, poetx_stream_t stream) {
  return cnp_bwd_impl("poetx_cnp_bwd", nblk, b, k, theta, dG, dtheta, accumulate, prec, ws,
                      ws_bytes, stream, false);
}

int32_t poetx_cnp_bwd_after_fwd(int32_t nblk, int32_t b, int32_t k, const float* theta,
                                const float* dG, float* dtheta, int32_t accumulate, int32_t prec,
                                void* ws, size_t ws_bytes, poetx_stream_t stream) {
  return cnp_bwd_impl("poetx_cnp_bwd_after_fwd", nblk, b, k, theta, dG, dtheta, accumulate, prec,
                      ws, ws_bytes, stream, true);
}

int32_t poetx_fold_perm(int32_t m, int32_t n, int32_t dt, const void* W0, const int32_t* perm_R,
                        const int32_t* perm_P, void* W0f, void* W0fT, int32_t* perm_R_inv,
                        int32_t* perm_P_inv, poetx_stream_t stream) {
  const char* fn = "poetx_fold_perm";
  if (m < 1 || n < 1) return fail(POETX_ERR_ARG, "%s: m=%d n=%d must be >= 1", fn, m, n);
  if (dt != POETX_F32 && dt != POETX_BF16 && dt != POETX_I8)
    return fail(POETX_ERR_ARG, "%s: dtype %d", fn, dt);
  NEED_PTR(W0);
  NEED_PTR(perm_R);
  NEED_PTR(perm_P);
  NEED_PTR(W0f);
  OPT_PTR(W0fT);
  OPT_PTR(perm_R_inv);
  OPT_PTR(perm_P_inv);
  hipError_t e = launch_fold(m, n, dt == POETX_I8 ? 1 : (int)es_of(dt), W0, perm_R, perm_P, W0f, W0fT, perm_R_inv,
                             perm_P_inv, (hipStream_t)stream);
  if (e != hipSuccess) return dev_fail(e, fn);
  return ok();
}

int32_t poetx_fold_scale(int32_t m, const float* s, const int32_t* perm_R, float* s_f,
                         poetx_stream_t stream) {
  const char* fn = "poetx_fold_scale";
  if (m < 1) return fail(POETX_ERR_ARG, "%s: m=%d must be >= 1", fn, m);
  NEED_PTR(s);
  NEED_PTR(perm_R);
  NEED_PTR(s_f);
  hipError_t e = launch_gather_f32(m, s, perm_R, s_f, (hipStream_t)stream);
  if (e != hipSuccess) return dev_fail(e, fn);
  return ok();
}

int32_t poetx_dequant(int32_t rows, int32_t cols, const void* q, const float* scale,
                      int32_t per_row, void* out, poetx_stream_t stream) {
  const char* fn = "poetx_dequant";
  if (rows < 1 || cols < 1 || cols % 16)
    return fail(POETX_ERR_ARG, "%s: rows=%d cols=%d (cols must be a positive multiple of 16)", fn,
                rows, cols);
  NEED_PTR(q);
  NEED_PTR(scale);
  NEED_PTR(out);
  if ((uintptr_t)q % 16 || (uintptr_t)out % 16)
    return fail(POETX_ERR_ARG, "%s: q and out must be 16-byte aligned", fn);
  hipError_t e = launch_dequant_i8(rows, cols, (const int8_t*)q, scale, per_row ? 1 : 0,
                                   (bf16*)out, (hipStream_t)stream);
  if (e != hipSuccess) return dev_fail(e, fn);
  return ok();
}

size_t poetx_workspace_bytes(const poetx_shape* sh, int32_t which) {
  if (check_shape("poetx_workspace_bytes", sh) != POETX_OK) return 0;
  if (which == 0) return fwd_ws(sh).total;
  if (which == 1) return bwd_ws(sh).total;
  if (which == 2) return fwd_ws(sh, true).total;
  if (which == 3) return bwd_ws(sh, true).total;
  if (which == 4) return merge_ws(sh);
  return 0;
}

size_t poetx_saved_bytes(const poetx_shape* sh) {
  if (check_shape("poetx_saved_bytes", sh) != POETX_OK) return 0;
  return saved_total(sh);
}

size_t poetx_saved_bytes_xmem(const poetx_shape* sh) {
  if (check_shape("poetx_saved_bytes_xmem", sh) != POETX_OK) return 0;
  return saved_total(sh, true);
}

// an int8 weight runs on the MFMA path, whose dense kernel needs both
// widths to be whole 256-column tiles
static int32_t check_quant(const char* fn, const poetx_shape* sh) {
  if (sh->act != POETX_BF16)
    return fail(POETX_ERR_UNSUPPORTED, "%s: an int8 weight needs bf16 activations", fn);
  if (sh->b < 64 || sh->m % 256 || sh->n % 256 || sh->m >= (1 << 21) || sh->n >= (1 << 21))
    return fail(POETX_ERR_UNSUPPORTED,
                "%s: an int8 weight needs b >= 64 and m, n multiples of 256 below 2^21 "
                "(m=%d n=%d b=%d)", fn, sh->m, sh->n, sh->b);
  return POETX_OK;
}

// W0f set: the activation-type weight; s_f set: the int8 pair (q_f, s_f)
static int32_t layer_fwd_entry(const char* fn, bool xmem, const poetx_shape* sh, const void* x,
                               const void* G_P, const void* G_R, const void* W0f,
                               const int8_t* q_f, const float* s_f, const int32_t* perm_P,
                               const int32_t* perm_R_inv, void* y, void* saved, void* ws,
                               size_t ws_bytes, poetx_stream_t stream) {
  int32_t st = check_shape(fn, sh);
  if (st != POETX_OK) return st;
  const bool quant = s_f != nullptr || q_f != nullptr;
  if (quant && (st = check_quant(fn, sh)) != POETX_OK) return st;
  NEED_PTR(x);
  NEED_PTR(G_P);
  NEED_PTR(G_R);
  if (quant) {
    NEED_PTR(q_f);
    NEED_PTR(s_f);
  } else {
    NEED_PTR(W0f);
  }
  NEED_PTR(perm_P);
  NEED_PTR(perm_R_inv);
  NEED_PTR(y);
  NEED_PTR(saved);
  NEED_PTR(ws);
  const size_t need = fwd_ws(sh, xmem).total;
  if (ws_bytes < need) return fail(POETX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  if (sh->act == POETX_BF16) {
    Weight<bf16> W;
    W.f = (const bf16*)W0f;
    W.q = q_f;
    W.s = s_f;
    return layer_fwd_impl<bf16>(sh, (const bf16*)x, (const bf16*)G_P, (const bf16*)G_R, W, perm_P,
                                perm_R_inv, (bf16*)y, saved, ws, s, xmem);
  }
  Weight<float> W;
  W.f = (const float*)W0f;
  return layer_fwd_impl<float>(sh, (const float*)x, (const float*)G_P, (const float*)G_R, W,
                               perm_P, perm_R_inv, (float*)y, saved, ws, s, xmem);
}

int32_t poetx_layer_fwd(const poetx_shape* sh, const void* x, const void* G_P, const void* G_R,
                        const void* W0f, const int32_t* perm_P, const int32_t* perm_R_inv,
                        void* y, void* saved, void* ws, size_t ws_bytes, poetx_stream_t stream) {
  return layer_fwd_entry("poetx_layer_fwd", false, sh, x, G_P, G_R, W0f, nullptr, nullptr, perm_P,
                         perm_R_inv, y, saved, ws, ws_bytes, stream);
}

int32_t poetx_layer_fwd_xmem(const poetx_shape* sh, const void* x, const void* G_P,
                             const void* G_R, const void* W0f, const int32_t* perm_P,
                             const int32_t* perm_R_inv, void* y, void* saved, void* ws,
                             size_t ws_bytes, poetx_stream_t stream) {
  return layer_fwd_entry("poetx_layer_fwd_xmem", true, sh, x, G_P, G_R, W0f, nullptr, nullptr,
                         perm_P, perm_R_inv, y, saved, ws, ws_bytes, stream);
}

int32_t poetx_layer_fwd_q(const poetx_shape* sh, const void* x, const void* G_P, const void* G_R,
                          const int8_t* q_f, const float* s_f, const int32_t* perm_P,
                          const int32_t* perm_R_inv, void* y, void* saved, void* ws,
                          size_t ws_bytes, int32_t xmem, poetx_stream_t stream) {
  if (!s_f) return fail(POETX_ERR_ARG, "poetx_layer_fwd_q: null pointer 's_f'");
  return layer_fwd_entry("poetx_layer_fwd_q", xmem != 0, sh, x, G_P, G_R, nullptr, q_f, s_f,
                         perm_P, perm_R_inv, y, saved, ws, ws_bytes, stream);
}

// W0f / W0fT set: the activation-type weight; s_f set: the int8 pair
// (q_f, q_fT, s_f); G_P and W0f / q_f only for the memory-saving mode
static int32_t layer_bwd_entry(const char* fn, bool xmem, const poetx_shape* sh, const void* dy,
                               const void* G_P, const void* GT_P, const void* GT_R,
                               const void* W0f, const void* W0fT, const int8_t* q_f,
                               const int8_t* q_fT, const float* s_f, const int32_t* perm_P_inv,
                               const int32_t* perm_R, const void* saved, void* dx, float* dG_P,
                               float* dG_R, void* ws, size_t ws_bytes, poetx_stream_t stream) {
  int32_t st = check_shape(fn, sh);
  if (st != POETX_OK) return st;
  const bool quant = s_f != nullptr;
  if (quant && (st = check_quant(fn, sh)) != POETX_OK) return st;
  NEED_PTR(dy);
  if (xmem) {
    NEED_PTR(G_P);
    if (quant) NEED_PTR(q_f);
  }
  NEED_PTR(GT_P);
  NEED_PTR(GT_R);
  if (quant) {
    NEED_PTR(q_fT);
    NEED_PTR(s_f);
  } else {
    NEED_PTR(W0f);
    OPT_PTR(W0fT);
  }
  NEED_PTR(perm_P_inv);
  NEED_PTR(perm_R);
  NEED_PTR(saved);
  NEED_PTR(dx);
  NEED_PTR(dG_P);
  NEED_PTR(dG_R);
  NEED_PTR(ws);
  const size_t need = bwd_ws(sh, xmem).total;
  if (ws_bytes < need) return fail(POETX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  if (sh->act == POETX_BF16) {
    Weight<bf16> W;
    W.f = (const bf16*)W0f;
    W.fT = (const bf16*)W0fT;
    W.q = q_f;
    W.qT = q_fT;
    W.s = s_f;
    return layer_bwd_impl<bf16>(sh, (const bf16*)dy, (const bf16*)GT_P, (const bf16*)GT_R, W,
                                perm_P_inv, perm_R, saved, (bf16*)dx, dG_P, dG_R, ws, s,
                                xmem ? (const bf16*)G_P : nullptr);
  }
  Weight<float> W;
  W.f = (const float*)W0f;
  W.fT = (const float*)W0fT;
  return layer_bwd_impl<float>(sh, (const float*)dy, (const float*)GT_P, (const float*)GT_R, W,
                               perm_P_inv, perm_R, saved, (float*)dx, dG_P, dG_R, ws, s,
                               xmem ? (const float*)G_P : nullptr);
}

int32_t poetx_layer_bwd(const poetx_shape* sh, const void* dy, const void* GT_P, const void* GT_R,
                        const void* W0f, const void* W0fT, const int32_t* perm_P_inv,
                        const int32_t* perm_R, const void* saved, void* dx, float* dG_P,
                        float* dG_R, void* ws, size_t ws_bytes, poetx_stream_t stream) {
  return layer_bwd_entry("poetx_layer_bwd", false, sh, dy, nullptr, GT_P, GT_R, W0f, W0fT,
                         nullptr, nullptr, nullptr, perm_P_inv, perm_R, saved, dx, dG_P, dG_R, ws,
                         ws_bytes, stream);
}

int32_t poetx_layer_bwd_xmem(const poetx_shape* sh, const void* dy, const void* G_P,
                             const void* GT_P, const void* GT_R, const void* W0f,
                             const void* W0fT, const int32_t* perm_P_inv, const int32_t* perm_R,
                             const void* saved, void* dx, float* dG_P, float* dG_R, void* ws,
                             size_t ws_bytes, poetx_stream_t stream) {
  return layer_bwd_entry("poetx_layer_bwd_xmem", true, sh, dy, G_P, GT_P, GT_R, W0f, W0fT, nullptr,
                         nullptr, nullptr, perm_P_inv, perm_R, saved, dx, dG_P, dG_R, ws, ws_bytes,
                         stream);
}

int32_t poetx_layer_bwd_q(const poetx_shape* sh, const void* dy, const void* G_P, const void* GT_P,
                          const void* GT_R, const int8_t* q_f, const int8_t* q_fT,
                          const float* s_f, const int32_t* perm_P_inv, const int32_t* perm_R,
                          const void* saved, void* dx, float* dG_P, float* dG_R, void* ws,
                          size_t ws_bytes, int32_t xmem, poetx_stream_t stream) {
  if (!s_f) return fail(POETX_ERR_ARG, "poetx_layer_bwd_q: null pointer 's_f'");
  return layer_bwd_entry("poetx_layer_bwd_q", xmem != 0, sh, dy, G_P, GT_P, GT_R, nullptr, nullptr,
                         q_f, q_fT, s_f, perm_P_inv, perm_R, saved, dx, dG_P, dG_R, ws, ws_bytes,
                         stream);
}

int32_t poetx_merge(const poetx_shape* sh, const void* W0f, const void* G_R, const void* GT_P,
                    const int32_t* perm_R_inv, const int32_t* perm_P_inv, void* W0_out, void* ws,
                    size_t ws_bytes, poetx_stream_t stream) {
  const char* fn = "poetx_merge";
  int32_t st = check_shape(fn, sh);
  if (st != POETX_OK) return st;
  NEED_PTR(W0f);
  NEED_PTR(G_R);
  NEED_PTR(GT_P);
  NEED_PTR(perm_R_inv);
  NEED_PTR(perm_P_inv);
  NEED_PTR(W0_out);
  NEED_PTR(ws);
  if (W0_out == W0f) return fail(POETX_ERR_ARG, "%s: W0_out must not alias W0f", fn);
  const size_t need = merge_ws(sh);
  if (ws_bytes < need) return fail(POETX_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  if (sh->act == POETX_BF16)
    return merge_impl<bf16>(sh, (const bf16*)W0f, (const bf16*)G_R, (const bf16*)GT_P, perm_R_inv,
                            perm_P_inv, (bf16*)W0_out, ws, s);
  return merge_impl<float>(sh, (const float*)W0f, (const float*)G_R, (const float*)GT_P,
                           perm_R_inv, perm_P_inv, (float*)W0_out, ws, s);
}

}  // extern "C"

extern "C" int32_t poetx_set_fused_gather(int32_t on) {
  return g_fused_gather.exchange(on != 0 ? 1 : 0);
}

extern "C" int32_t poetx_set_stage_events(void* const* events, int32_t count) {
  if (!events) {
    g_stage_on = 0;
    return ok();
  }
  if (count < 8) return fail(POETX_ERR_ARG, "poetx_set_stage_events: count=%d < 8", count);
  for (int i = 0; i < 8; ++i) {
    if (!events[i]) return fail(POETX_ERR_ARG, "poetx_set_stage_events: null event %d", i);
    g_stage_ev[i] = (hipEvent_t)events[i];
  }
  g_stage_on = 1;
  return ok();
}
