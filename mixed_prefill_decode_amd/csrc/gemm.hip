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

template <typename T, int BM, int BN, int WGM, int WGN, int EPI, int ST, bool FOLD = false>
xp_status launch_cfg(const void* A, const void* B, const void* B2, const void* R, void* C, int M, int N, int K,
                     int splits, int chunks, float* part, hipStream_t s,
                     const typename gemm::EpiArg<EPI>::type& ea = {}) {
  const int tm = cdiv(M, BM), tn = cdiv(N, BN);
  const int stages = K / gemm::Cfg<T, BM, BN, WGM, WGN, EPI>::BK;
  const int per = cdiv(stages, chunks);     // stages per K chunk
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WGM, WGN, EPI, ST, 128, FOLD>), dim3(tm * tn * splits),
                     dim3(64 * WGM * WGN), 0, s, static_cast<const char*>(A), static_cast<const char*>(B),
                     static_cast<const char*>(B2), R, C, M, N, K, tm, tn, splits, per, part, ea);
  XP_CHECK_LAUNCH();
  if constexpr (EPI == gemm::kEpiRope) return XP_OK;   // one unit per tile, no partials
  if (splits > 1) {
    const long mn = long(M) * N;
    if (mn % 4 == 0) {
      const int blocks = int(std::min<long>((mn / 4 + 255) / 256, 4096));
      hipLaunchKernelGGL((gemm::gemm_reduce_kernel<T, EPI, true>), dim3(blocks), dim3(256), 0, s, part, R, C, mn,
                         splits);
    } else {
      const int blocks = int(std::min<long>((mn + 255) / 256, 4096));
      hipLaunchKernelGGL((gemm::gemm_reduce_kernel<T, EPI, false>), dim3(blocks), dim3(256), 0, s, part, R, C, mn,
                         splits);
    }
    XP_CHECK_LAUNCH();
  }
  return XP_OK;
}

struct Candidate {
  int id, bm, bn, per_cu;   // tile, workgroups resident per CU (LDS- and wave-limited)
  double tflops;            // fitted rate of one resident workgroup (bf16, TFLOP/s)
};

// Per epilogue kind: single weight (plain / residual epilogues) and dual weight
// (SwiGLU).  A call is modelled as rounds x (work-unit flops / rate), rounds counting
// waves of resident workgroups (a grid of 1.1 rounds takes as long as 2).  The rates
// are fitted so that the model's pick is the fastest measured candidate on the QKV,
// O, gate/up and down projections of the 8B, 14B and 32B layer shapes at 128 to 1040
// rows and the 14B shape at 8216 rows (all picks within 1% of the best measured); they
// rank the candidates rather than describe them.  Tiles of 96 and 192 rows exist for
// row counts such as 1040 = 1024 + 16, where 128-row tiles leave a nearly empty extra
// tile row (and so a second round of workgroups).
constexpr Candidate kSingle[] = {
    {0, 64, 128, 1, 4.59},    // 1x4 waves, 4-stage ring (96 KB LDS)
    {1, 96, 128, 1, 5.50},    // 1x4 waves, 4-stage ring (112 KB)
    {2, 128, 256, 1, 6.65},   // 2x4 waves, 3-stage ring (144 KB)
    {3, 192, 128, 1, 7.03},   // 2x4 waves, 4-stage ring (160 KB)
    {4, 192, 192, 1, 6.88},   // 2x2 waves, 3-stage ring (144 KB)
    {5, 256, 256, 1, 11.61},  // 2x4 waves, 2-stage ring (128 KB)
};
// Unsplit units that fold K chunks hold a second set of accumulators: the tiles
// that keep it in registers.
constexpr Candidate kSingleFold[] = {
    {0, 64, 128, 1, 4.59},
    {1, 96, 128, 1, 5.50},
    {2, 128, 256, 1, 6.65},
    {3, 192, 128, 1, 7.03},
};
// The fused RoPE epilogue stages a tile of whole heads in the ring: tiles whose width
// is a multiple of 128 (so of d = 64 and 128) and whose [BM][BN + 4] fp32 image fits.
constexpr Candidate kSingleRope[] = {
    {0, 64, 128, 1, 4.59},
    {1, 96, 128, 1, 5.50},
    {2, 128, 256, 1, 6.65},
    {3, 192, 128, 1, 7.03},
};
constexpr Candidate kDual[] = {
    {0, 128, 64, 1, 8.03},    // 2x2 waves, 3-stage ring (96 KB)
    {4, 128, 128, 1, 10.32},  // 2x4 waves, 3-stage ring (144 KB)
    {1, 192, 64, 1, 8.98},    // 2x2 waves, 3-stage ring (120 KB)
    {2, 192, 128, 1, 10.32},  // 2x4 waves, 2-stage ring (112 KB)
    {3, 256, 128, 1, 11.05},  // 4x2 waves, 2-stage ring (128 KB)
};

template <size_t NC>
int pick(const Candidate (&c)[NC], int M, int N, int K, int n_cus, int nb, int splits) {
  double best = 1e300;
  int id = 0;
  for (const Candidate& x : c) {
    const long units = long(cdiv(M, x.bm)) * cdiv(N, x.bn) * splits;
    const long slots = long(n_cus) * x.per_cu;
    const double rounds = double((units + slots - 1) / slots);
    const double t = rounds * 2.0 * x.bm * x.bn * nb * (double(K) / splits) / (x.tflops * 1e12);
    if (t < best) {
      best = t;
      id = x.id;
    }
  }
  return id;
}


template <typename T, int EPI>
xp_status launch_epi(const void* A, const void* B, const void* B2, const void* R, void* C, int M, int N, int K,
                     int splits, int chunks, float* part, hipStream_t s) {
  const int cus = device_cus();
#define XP_GEMM_ARGS A, B, B2, R, C, M, N, K, splits, chunks, part, s
  if constexpr (EPI == XP_EPI_SWIGLU) {
    switch (pick(kDual, M, N, K, cus, 2, splits)) {
      case 1: return launch_cfg<T, 192, 64, 2, 2, EPI, 3>(XP_GEMM_ARGS);
      case 2: return launch_cfg<T, 192, 128, 2, 4, EPI, 2>(XP_GEMM_ARGS);
      case 3: return launch_cfg<T, 256, 128, 4, 2, EPI, 2>(XP_GEMM_ARGS);
      case 4: return launch_cfg<T, 128, 128, 2, 4, EPI, 3>(XP_GEMM_ARGS);
      default: return launch_cfg<T, 128, 64, 2, 2, EPI, 3>(XP_GEMM_ARGS);
    }
  } else if (splits == 1 && chunks > 1) {
    switch (pick(kSingleFold, M, N, K, cus, 1, splits)) {
      case 1: return launch_cfg<T, 96, 128, 1, 4, EPI, 4, true>(XP_GEMM_ARGS);
      case 2: return launch_cfg<T, 128, 256, 2, 4, EPI, 3, true>(XP_GEMM_ARGS);
      case 3: return launch_cfg<T, 192, 128, 2, 4, EPI, 4, true>(XP_GEMM_ARGS);
      default: return launch_cfg<T, 64, 128, 1, 4, EPI, 4, true>(XP_GEMM_ARGS);
    }
  } else {
    switch (pick(kSingle, M, N, K, cus, 1, splits)) {
      case 1: return launch_cfg<T, 96, 128, 1, 4, EPI, 4>(XP_GEMM_ARGS);
      case 2: return launch_cfg<T, 128, 256, 2, 4, EPI, 3>(XP_GEMM_ARGS);
      case 3: return launch_cfg<T, 192, 128, 2, 4, EPI, 4>(XP_GEMM_ARGS);
      case 4: return launch_cfg<T, 192, 192, 2, 2, EPI, 3>(XP_GEMM_ARGS);
      case 5: return launch_cfg<T, 256, 256, 2, 4, EPI, 2>(XP_GEMM_ARGS);
      default: return launch_cfg<T, 64, 128, 1, 4, EPI, 4>(XP_GEMM_ARGS);
    }
  }
#undef XP_GEMM_ARGS
}

template <typename T>
xp_status launch_type(int epi, const void* A, const void* B, const void* B2, const void* R, void* C, int M, int N,
                      int K, int splits, int chunks, float* part, hipStream_t s) {
  switch (epi) {
    case XP_EPI_F32: return launch_epi<T, XP_EPI_F32>(A, B, B2, R, C, M, N, K, splits, chunks, part, s);
    case XP_EPI_ADD_T: return launch_epi<T, XP_EPI_ADD_T>(A, B, B2, R, C, M, N, K, splits, chunks, part, s);
    case XP_EPI_ADD_F32: return launch_epi<T, XP_EPI_ADD_F32>(A, B, B2, R, C, M, N, K, splits, chunks, part, s);
    case XP_EPI_SWIGLU: return launch_epi<T, XP_EPI_SWIGLU>(A, B, B2, R, C, M, N, K, splits, chunks, part, s);
  }
  return fail(XP_EINVAL, "xp_gemm: unknown epilogue %d", epi);
}

template <typename T>
xp_status launch_rope_type(const void* A, const void* B, int M, int N, int K, const PostQkvArgs& ra, hipStream_t s) {
  constexpr int E = gemm::kEpiRope;
#define XP_ROPE_ARGS A, B, nullptr, nullptr, nullptr, M, N, K, 1, 1, nullptr, s, ra
  switch (pick(kSingleRope, M, N, K, device_cus(), 1, 1)) {
    case 1: return launch_cfg<T, 96, 128, 1, 4, E, 4>(XP_ROPE_ARGS);
    case 2: return launch_cfg<T, 128, 256, 2, 4, E, 3>(XP_ROPE_ARGS);
    case 3: return launch_cfg<T, 192, 128, 2, 4, E, 4>(XP_ROPE_ARGS);
    default: return launch_cfg<T, 64, 128, 1, 4, E, 4>(XP_ROPE_ARGS);
  }
#undef XP_ROPE_ARGS
}

}  // namespace

bool gemm_rope_supported(int dtype, int d) {
  return (dtype == XP_BF16 || dtype == XP_F32) && (d == 64 || d == 128);
}

xp_status launch_gemm_rope(int dtype, const void* A, const void* B, int M, int N, int K, const PostQkvArgs& ra,
                           hipStream_t s) {
  if (!gemm_rope_supported(dtype, ra.d)) return fail(XP_EUNSUPPORTED, "fused RoPE epilogue: head_dim %d", ra.d);
  if (M < 0 || N != (ra.Hq + 2 * ra.Hkv) * ra.d || K <= 0) return fail(XP_ESHAPE, "fused RoPE epilogue: M=%d N=%d", M, N);
  const int bk = 128 / dtype_bytes(dtype);
  if (K % bk || 256L * K * dtype_bytes(dtype) >= (1L << 31)) return fail(XP_EUNSUPPORTED, "fused RoPE epilogue: K=%d", K);
  if (!A || !B || !ra.rope_tab) return fail(XP_EINVAL, "fused RoPE epilogue: null operand");
  if (M == 0) return XP_OK;
  // the rotation frequencies are not needed here (the table holds cos and sin)
  xp_status st = dtype == XP_BF16 ? launch_rope_type<bf16_t>(A, B, M, N, K, ra, s)
                                  : launch_rope_type<float>(A, B, M, N, K, ra, s);
  return st;
}

int device_cus() {
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

// K chunks of a GEMM against an [N, K] weight: a function of the weight's shape only.
// Only long-K, narrow products (K >= 3N, the FFN down projection) are chunked: their
// sum runs over C fixed K ranges in order, whether the chunks are separate work units
// (few rows cannot fill the chip otherwise: 128 rows of an 8B down projection take 27
// us split, 61 unsplit) or one unit folds them (gemm_kernel's FOLD), so a row's result
// never depends on how many rows share the call.  Aim: with 256-row tiles and about
// 1024 rows, (N / 256) x 4 x C ~ 256 work units; at least 16 K stages per chunk; at
// most 4 chunks.
int gemm_chunks(int dtype, int epi, int N, int K) {
  const int nb = epi == XP_EPI_SWIGLU ? 2 : 1;
  const int stages = K / (128 / dtype_bytes(dtype));
  if (long(K) < 3L * N * nb) return 1;
  int sp = int(16384.0 / (double(N) * nb) + 0.5);
  sp = std::max(1, std::min(4, sp));
  while (sp > 1 && stages / sp < 16) --sp;
  return sp;
}

// Work units per chunked product: one per chunk (plus the reduction) when the unsplit
// product would keep fewer than 70% of the CUs busy with 192 x 128 tiles, else one
// folding unit per tile.  Measured on the down projections of the layer shapes: 1040
// rows run unsplit in 127 us vs 145 split; 128 to 544 rows split in 27-154 us vs
// 61-205 unsplit.  Chunked SwiGLU products always split.
int gemm_split_count(int dtype, int epi, int M, int N, int K) {
  const int c = gemm_chunks(dtype, epi, N, K);
  if (c <= 1 || epi == XP_EPI_SWIGLU) return c;
  const long tiles = long(cdiv(M, 192)) * cdiv(N, 128);
  return tiles * 10 < long(device_cus()) * 7 ? c : 1;
}

void gemm_tile(int dtype, int epi, int M, int N, int K, int* bm, int* bn, int* splits) {
  const int sp = gemm_split_count(dtype, epi, M, N, K);
  const int cus = device_cus();
  const Candidate* c = nullptr;
  if (epi == XP_EPI_SWIGLU) {
    const int id = pick(kDual, M, N, K, cus, 2, sp);
    for (const Candidate& x : kDual) if (x.id == id) c = &x;
  } else if (sp == 1 && gemm_chunks(dtype, epi, N, K) > 1) {
    const int id = pick(kSingleFold, M, N, K, cus, 1, sp);
    for (const Candidate& x : kSingleFold) if (x.id == id) c = &x;
  } else {
    const int id = pick(kSingle, M, N, K, cus, 1, sp);
    for (const Candidate& x : kSingle) if (x.id == id) c = &x;
  }
  *bm = c ? c->bm : 0;
  *bn = c ? c->bn : 0;
  *splits = sp;
}

size_t gemm_ws_bytes(int dtype, int epi, int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const int sp = gemm_split_count(dtype, epi, M, N, K);
  if (sp <= 1) return 0;
  return size_t(sp) * (epi == XP_EPI_SWIGLU ? 2 : 1) * size_t(M) * N * sizeof(float);
}

xp_status launch_gemm(int dtype, int epi, const void* A, const void* B, const void* B2, const void* R, void* C,
                      int M, int N, int K, void* ws, size_t ws_bytes, hipStream_t s) {
  if (dtype != XP_BF16 && dtype != XP_F32) return fail(XP_EINVAL, "xp_gemm: dtype %d", dtype);
  if (M < 0 || N <= 0 || K <= 0) return fail(XP_ESHAPE, "xp_gemm: M=%d N=%d K=%d", M, N, K);
  if (epi < XP_EPI_F32 || epi > XP_EPI_SWIGLU) return fail(XP_EINVAL, "xp_gemm: unknown epilogue %d", epi);
  const int bk = 128 / dtype_bytes(dtype);
  if (K % bk) return fail(XP_EUNSUPPORTED, "xp_gemm: K=%d is not a multiple of %d", K, bk);
  // a buffer resource covers one tile's rows (<= 256), so its byte offsets must stay below 2^31
  if (256L * K * dtype_bytes(dtype) >= (1L << 31)) return fail(XP_EUNSUPPORTED, "xp_gemm: K=%d too large", K);
  if (!A || !B || !C) return fail(XP_EINVAL, "xp_gemm: null operand");
  if ((epi == XP_EPI_ADD_T || epi == XP_EPI_ADD_F32) && !R) return fail(XP_EINVAL, "xp_gemm: null residual");
  if (epi == XP_EPI_SWIGLU && !B2) return fail(XP_EINVAL, "xp_gemm: null second weight");
  if (M == 0) return XP_OK;
  const int splits = gemm_split_count(dtype, epi, M, N, K), chunks = gemm_chunks(dtype, epi, N, K);
  const size_t need = gemm_ws_bytes(dtype, epi, M, N, K);
  if (need && (!ws || ws_bytes < need))
    return fail(XP_EWORKSPACE, "xp_gemm: needs %zu bytes of workspace (got %zu)", need, ws ? ws_bytes : size_t(0));
  float* part = static_cast<float*>(ws);
  if (dtype == XP_BF16) return launch_type<bf16_t>(epi, A, B, B2, R, C, M, N, K, splits, chunks, part, s);
  return launch_type<float>(epi, A, B, B2, R, C, M, N, K, splits, chunks, part, s);
}

}  // namespace xp
