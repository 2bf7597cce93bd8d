// Co-batched dense projections (ConfluxServe §4 and App. B: the QKV, O and FFN
// projections run once over the concatenated [prefill-chunk || decode] rows
// against one weight read): launch-shape selection for the MFMA GEMM of
// gemm_core.h.
//
// Which tile shape is fastest depends mostly on how many tiles a shape yields
// compared with the 256 CUs: a grid of 1.1 rounds of resident workgroups takes as
// long as 2 full rounds.  Each candidate below carries its measured full-occupancy
// rate on MI355X and how many of its workgroups fit on one CU (LDS-limited); the
// launcher estimates rounds x time-per-tile for each and takes the smallest.
#include "gemm_core.h"
#include "xp_internal.h"

namespace xp {

namespace {

using gemm::gemm_kernel;

template <typename T, int BM, int BN, int WGM, int WGN, int EPI, int ST>
xp_status launch_cfg(const void* A, const void* B, const void* B2, const void* R, void* C, int M, int N, int K,
                     hipStream_t s) {
  const int tm = cdiv(M, BM), tn = cdiv(N, BN);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WGM, WGN, EPI, ST>), dim3(tm * tn), dim3(64 * WGM * WGN), 0, s,
                     static_cast<const char*>(A), static_cast<const char*>(B), static_cast<const char*>(B2), R, C,
                     M, N, K, tm, tn);
  XP_CHECK_LAUNCH();
  return XP_OK;
}

struct Candidate {
  int id, bm, bn, per_cu;   // tile, workgroups resident per CU (LDS-limited)
  double tflops;            // measured rate of one resident workgroup (bf16, TFLOP/s)
};

// Per epilogue kind: single weight (plain / residual epilogues) and dual weight
// (SwiGLU).  Rates are per resident workgroup, fitted over the layer shapes' QKV, O,
// gate/up and down projections at 128 to 1040 rows; a workgroup's time is then
// rounds x (tile flops / rate).
constexpr Candidate kSingle[] = {
    {0, 128, 128, 2, 3.14},   // 2x4 waves, 2-stage ring (64 KB LDS)
    {1, 128, 128, 1, 4.74},   // 2x4 waves, 3-stage ring (96 KB)
    {2, 128, 256, 1, 5.19},   // 2x4 waves, 2-stage ring (96 KB)
    {3, 64, 128, 2, 2.16},    // 1x4 waves, 3-stage ring (72 KB)
    {4, 128, 256, 1, 6.12},   // 2x4 waves, 3-stage ring (144 KB)
    {5, 64, 128, 1, 3.11},    // 1x4 waves, 4-stage ring (96 KB)
    {6, 128, 64, 2, 2.24},    // 2x2 waves, 3-stage ring (72 KB)
};
constexpr Candidate kDual[] = {
    {0, 128, 128, 1, 3.62},   // 2x4 waves, 2-stage ring (96 KB)
    {1, 128, 128, 1, 4.55},   // 2x4 waves, 3-stage ring (144 KB)
    {2, 128, 256, 1, 4.39},   // 2x4 waves, 2-stage ring (160 KB)
    {3, 64, 128, 1, 3.32},    // 1x4 waves, 3-stage ring (120 KB)
    {4, 256, 128, 1, 5.73},   // 4x2 waves, 2-stage ring (128 KB)
    {5, 128, 64, 1, 3.77},    // 2x2 waves, 3-stage ring (96 KB)
};

template <size_t NC>
int pick(const Candidate (&c)[NC], int M, int N, int K, int n_cus, int nb) {
  double best = 1e300;
  int id = 0;
  for (const Candidate& x : c) {
    const long tiles = long(cdiv(M, x.bm)) * cdiv(N, x.bn);
    const long slots = long(n_cus) * x.per_cu;
    const double rounds = double((tiles + slots - 1) / slots);
    const double t = rounds * 2.0 * x.bm * x.bn * nb * K / (x.tflops * 1e12);
    if (t < best) {
      best = t;
      id = x.id;
    }
  }
  return id;
}

int n_cus_of_current_device() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <typename T, int EPI>
xp_status launch_epi(const void* A, const void* B, const void* B2, const void* R, void* C, int M, int N, int K,
                     hipStream_t s) {
  const int cus = n_cus_of_current_device();
  if constexpr (EPI == XP_EPI_SWIGLU) {
    switch (pick(kDual, M, N, K, cus, 2)) {
      case 1: return launch_cfg<T, 128, 128, 2, 4, EPI, 3>(A, B, B2, R, C, M, N, K, s);
      case 2: return launch_cfg<T, 128, 256, 2, 4, EPI, 2>(A, B, B2, R, C, M, N, K, s);
      case 3: return launch_cfg<T, 64, 128, 1, 4, EPI, 3>(A, B, B2, R, C, M, N, K, s);
      case 4: return launch_cfg<T, 256, 128, 4, 2, EPI, 2>(A, B, B2, R, C, M, N, K, s);
      case 5: return launch_cfg<T, 128, 64, 2, 2, EPI, 3>(A, B, B2, R, C, M, N, K, s);
      default: return launch_cfg<T, 128, 128, 2, 4, EPI, 2>(A, B, B2, R, C, M, N, K, s);
    }
  } else {
    switch (pick(kSingle, M, N, K, cus, 1)) {
      case 1: return launch_cfg<T, 128, 128, 2, 4, EPI, 3>(A, B, B2, R, C, M, N, K, s);
      case 2: return launch_cfg<T, 128, 256, 2, 4, EPI, 2>(A, B, B2, R, C, M, N, K, s);
      case 3: return launch_cfg<T, 64, 128, 1, 4, EPI, 3>(A, B, B2, R, C, M, N, K, s);
      case 4: return launch_cfg<T, 128, 256, 2, 4, EPI, 3>(A, B, B2, R, C, M, N, K, s);
      case 5: return launch_cfg<T, 64, 128, 1, 4, EPI, 4>(A, B, B2, R, C, M, N, K, s);
      case 6: return launch_cfg<T, 128, 64, 2, 2, EPI, 3>(A, B, B2, R, C, M, N, K, s);
      default: return launch_cfg<T, 128, 128, 2, 4, EPI, 2>(A, B, B2, R, C, M, N, K, s);
    }
  }
}

template <typename T>
xp_status launch_type(int epi, const void* A, const void* B, const void* B2, const void* R, void* C, int M, int N,
                      int K, hipStream_t s) {
  switch (epi) {
    case XP_EPI_F32: return launch_epi<T, XP_EPI_F32>(A, B, B2, R, C, M, N, K, s);
    case XP_EPI_ADD_T: return launch_epi<T, XP_EPI_ADD_T>(A, B, B2, R, C, M, N, K, s);
    case XP_EPI_ADD_F32: return launch_epi<T, XP_EPI_ADD_F32>(A, B, B2, R, C, M, N, K, s);
    case XP_EPI_SWIGLU: return launch_epi<T, XP_EPI_SWIGLU>(A, B, B2, R, C, M, N, K, s);
  }
  return fail(XP_EINVAL, "xp_gemm: unknown epilogue %d", epi);
}

}  // namespace

xp_status launch_gemm(int dtype, int epi, const void* A, const void* B, const void* B2, const void* R, void* C,
                      int M, int N, int K, hipStream_t s) {
  if (dtype != XP_BF16 && dtype != XP_F32) return fail(XP_EINVAL, "xp_gemm: dtype %d", dtype);
  if (M < 0 || N <= 0 || K <= 0) return fail(XP_ESHAPE, "xp_gemm: M=%d N=%d K=%d", M, N, K);
  const int bk = gemm::kRowBytes / dtype_bytes(dtype);
  if (K % bk) return fail(XP_EUNSUPPORTED, "xp_gemm: K=%d is not a multiple of %d", K, bk);
  // a buffer resource covers one tile's rows (<= 256), so its byte offsets must stay below 2^31
  if (256L * K * dtype_bytes(dtype) >= (1L << 31)) return fail(XP_EUNSUPPORTED, "xp_gemm: K=%d too large", K);
  if (!A || !B || !C) return fail(XP_EINVAL, "xp_gemm: null operand");
  if ((epi == XP_EPI_ADD_T || epi == XP_EPI_ADD_F32) && !R) return fail(XP_EINVAL, "xp_gemm: null residual");
  if (epi == XP_EPI_SWIGLU && !B2) return fail(XP_EINVAL, "xp_gemm: null second weight");
  if (M == 0) return XP_OK;
  if (dtype == XP_BF16) return launch_type<bf16_t>(epi, A, B, B2, R, C, M, N, K, s);
  return launch_type<float>(epi, A, B, B2, R, C, M, N, K, s);
}

}  // namespace xp
