// Co-batched dense projections: C = epilogue(A B^T) with MFMA and fp32
// accumulation (ConfluxServe §4 and App. B: QKV, O and FFN projections run once
// over the concatenated [prefill-chunk || decode] rows against one weight read).
//
// Tiling: 256 threads = 4 waves in a 2x2 grid; block tile BM x BN, wave tile
// (BM/2) x (BN/2) made of 32x32 MFMA blocks.  Each stage moves a 128-byte
// slice of K per row (64 bf16 or 32 fp32) from HBM into a double-buffered LDS
// tile whose 16-byte chunks are XOR-swizzled by (row & 7), so the eight lanes
// an LDS read serves together hit eight different bank groups.  The SwiGLU
// epilogue reads two weight tiles (gate, up) against the same A tile and keeps
// both accumulators, so silu(g) * u is formed in registers.
//
// Block order is XCD-aware: workgroups are dealt to the 8 XCDs round-robin, so
// block b is remapped to tile (b % 8) * per_xcd + b / 8 with tiles ordered
// M-fastest; the M tiles that share one weight tile then run on one XCD and
// share its L2.
//
// The K loop order is the same for every M, so a row's result does not depend
// on which other rows are co-batched with it.
#include "xp_device.h"
#include "xp_internal.h"

namespace xp {

namespace {

constexpr int kRowBytes = 128;
constexpr int kChunks = 8;  // 16-byte chunks per LDS row

__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunks + (chunk ^ (row & 7)); }

template <typename T>
__device__ __forceinline__ void lds_frag(Frag8<T>& f, const uint4* buf, int row, int chunk);
template <>
__device__ __forceinline__ void lds_frag(Frag8<bf16_t>& f, const uint4* buf, int row, int chunk) {
  f.v = buf[swz(row, chunk)];
}
template <>
__device__ __forceinline__ void lds_frag(Frag8<float>& f, const uint4* buf, int row, int chunk) {
  uint4 a = buf[swz(row, chunk)], b = buf[swz(row, chunk + 1)];
  f.lo = __builtin_bit_cast(float4, a);
  f.hi = __builtin_bit_cast(float4, b);
}

template <typename T, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const char* __restrict__ A, const char* __restrict__ B,
                                                   const char* __restrict__ B2, const void* __restrict__ R,
                                                   void* __restrict__ C, int M, int N, int K, int tiles_m,
                                                   int tiles_n) {
  constexpr int EB = St<T>::bytes;
  constexpr int BK = kRowBytes / EB;
  constexpr int NB = (EPI == XP_EPI_SWIGLU) ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int ROWS = BM + NB * BN;
  constexpr int A_IT = BM / 32, B_IT = BN / 32;
  constexpr int CPK = 16 * EB / 16;  // 16-byte chunks per 16-deep k step (2 bf16, 4 fp32)
  __shared__ uint4 lds[2][ROWS * kChunks];

  // XCD-aware tile order
  const int n_tiles = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int q = n_tiles / 8, rem = n_tiles % 8, x = b % 8;
  const int t = x * q + min(x, rem) + b / 8;
  const int m0 = (t % tiles_m) * BM, n0 = (t / tiles_m) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid >> 3, lchunk = tid & 7;
  const long kbytes = long(K) * EB;

  uint4 ra[A_IT], rb[NB][B_IT];
  auto gload = [&](int kt) {
    const long koff = long(kt) * kRowBytes + lchunk * 16;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      int row = m0 + lrow + 32 * i;
      ra[i] = row < M ? *reinterpret_cast<const uint4*>(A + row * kbytes + koff) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const char* Bp = nb == 0 ? B : B2;
#pragma unroll
      for (int i = 0; i < B_IT; ++i) {
        int row = n0 + lrow + 32 * i;
        rb[nb][i] = row < N ? *reinterpret_cast<const uint4*>(Bp + row * kbytes + koff) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_IT; ++i) lds[buf][swz(lrow + 32 * i, lchunk)] = ra[i];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < B_IT; ++i) lds[buf][swz(BM + nb * BN + lrow + 32 * i, lchunk)] = rb[nb][i];
  };

  f32x16 acc[NB][FM][FN];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[nb][i][j] = f32x16{};

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lr = lane & 31, kg = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint4* buf = lds[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = ks * CPK + kg * (CPK / 2);
      Frag8<T> fa[FM], fb[NB][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) lds_frag<T>(fa[i], buf, wm * WM + i * 32 + lr, chunk);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < FN; ++j) lds_frag<T>(fb[nb][j], buf, BM + nb * BN + wn * WN + j * 32 + lr, chunk);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mma32x32_k16(acc[nb][i][j], fa[i], fb[nb][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * WN + j * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
        if (row >= M || col >= N) continue;
        const long idx = long(row) * N + col;
        const float v = acc[0][i][j][r];
        if constexpr (EPI == XP_EPI_F32) {
          reinterpret_cast<float*>(C)[idx] = v;
        } else if constexpr (EPI == XP_EPI_ADD_T) {
          reinterpret_cast<float*>(C)[idx] = St<T>::load(R, idx) + v;
        } else if constexpr (EPI == XP_EPI_ADD_F32) {
          reinterpret_cast<float*>(C)[idx] = reinterpret_cast<const float*>(R)[idx] + v;
        } else {
          const float u = acc[NB - 1][i][j][r];
          St<T>::store(C, idx, v / (1.0f + __expf(-v)) * u);
        }
      }
    }
}

template <typename T, int BM, int BN, int EPI>
xp_status launch_t(const void* A, const void* B, const void* B2, const void* R, void* C, int M, int N,
                   int K, hipStream_t s) {
  const int tm = cdiv(M, BM), tn = cdiv(N, BN);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, EPI>), dim3(tm * tn), dim3(256), 0, s,
                     static_cast<const char*>(A), static_cast<const char*>(B),
                     static_cast<const char*>(B2), R, C, M, N, K, tm, tn);
  XP_CHECK_LAUNCH();
  return XP_OK;
}

template <typename T, int EPI>
xp_status launch_epi(const void* A, const void* B, const void* B2, const void* R, void* C, int M, int N,
                     int K, hipStream_t s) {
  if (M <= 64) return launch_t<T, 64, 128, EPI>(A, B, B2, R, C, M, N, K, s);
  return launch_t<T, 128, 128, EPI>(A, B, B2, R, C, M, N, K, s);
}

template <typename T>
xp_status launch_type(int epi, const void* A, const void* B, const void* B2, const void* R, void* C, int M,
                      int N, int K, hipStream_t s) {
  switch (epi) {
    case XP_EPI_F32: return launch_epi<T, XP_EPI_F32>(A, B, B2, R, C, M, N, K, s);
    case XP_EPI_ADD_T: return launch_epi<T, XP_EPI_ADD_T>(A, B, B2, R, C, M, N, K, s);
    case XP_EPI_ADD_F32: return launch_epi<T, XP_EPI_ADD_F32>(A, B, B2, R, C, M, N, K, s);
    case XP_EPI_SWIGLU: return launch_epi<T, XP_EPI_SWIGLU>(A, B, B2, R, C, M, N, K, s);
  }
  return fail(XP_EINVAL, "xp_gemm: unknown epilogue %d", epi);
}

}  // namespace

xp_status launch_gemm(int dtype, int epi, const void* A, const void* B, const void* B2, const void* R,
                      void* C, int M, int N, int K, hipStream_t s) {
  if (dtype != XP_BF16 && dtype != XP_F32) return fail(XP_EINVAL, "xp_gemm: dtype %d", dtype);
  if (M < 0 || N <= 0 || K <= 0) return fail(XP_ESHAPE, "xp_gemm: M=%d N=%d K=%d", M, N, K);
  const int bk = kRowBytes / dtype_bytes(dtype);
  if (K % bk) return fail(XP_EUNSUPPORTED, "xp_gemm: K=%d is not a multiple of %d", K, bk);
  if (!A || !B || !C) return fail(XP_EINVAL, "xp_gemm: null operand");
  if ((epi == XP_EPI_ADD_T || epi == XP_EPI_ADD_F32) && !R) return fail(XP_EINVAL, "xp_gemm: null residual");
  if (epi == XP_EPI_SWIGLU && !B2) return fail(XP_EINVAL, "xp_gemm: null second weight");
  if (M == 0) return XP_OK;
  if (dtype == XP_BF16) return launch_type<bf16_t>(epi, A, B, B2, R, C, M, N, K, s);
  return launch_type<float>(epi, A, B, B2, R, C, M, N, K, s);
}

}  // namespace xp
