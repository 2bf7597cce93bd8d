// The MFMA GEMM, as a template over block tile, wave grid and LDS ring depth.
//
// C = epilogue(A B^T): A [M, K] and B [N, K] (K contiguous), fp32 accumulation.
// Block tile BM x BN, WGM x WGN waves, wave tile (BM/WGM) x (BN/WGN) made of
// 32x32 MFMA blocks.  Each stage is a 128-byte slice of K per row (64 bf16 or 32
// fp32), copied from HBM straight into an LDS ring (buffer_load ... lds: no staging
// registers, no LDS store instructions) whose 16-byte chunks are XOR-swizzled by
// ((row >> 1) & 7).  gfx950's LDS serves a 16-byte-per-lane read 16 lanes at a time
// across 64 four-byte banks (256 bytes): the 16 rows such a group reads are 8
// row pairs, and a pair spans the 64 banks once, so the swizzle gives the 8 pairs
// 8 different chunk positions and the group hits every bank exactly once.  The
// SwiGLU epilogue reads two weight tiles (gate, up) against the same A tile and
// keeps both accumulators, so silu(g) * u is formed in registers.
//
// Block order is XCD-aware: workgroups are dealt to the 8 XCDs round-robin, so
// block b is remapped to tile (b % 8) * per_xcd + b / 8 with tiles ordered
// M-fastest; the M tiles that share one weight tile then run on one XCD and
// share its L2.
//
// The K loop order (128-byte stages, 16-deep MFMA steps, in order) is the same for
// every M and every tile shape, so a row's result does not depend on which other
// rows are co-batched with it.
#pragma once
#include "xp_device.h"
#include "../../include/xp.h"

namespace xp {
namespace gemm {

constexpr int kRowBytes = 128;
constexpr int kChunks = 8;  // 16-byte chunks per LDS row

__device__ __forceinline__ int swz_of(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunks + (chunk ^ swz_of(row)); }

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

template <typename T, int BM, int BN, int WGM, int WGN, int EPI>
struct Cfg {
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int EB = St<T>::bytes;
  static constexpr int BK = kRowBytes / EB;
  static constexpr int NB = (EPI == XP_EPI_SWIGLU) ? 2 : 1;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int ROWS = BM + NB * BN;
  static constexpr int CPK = 16 * EB / 16;       // 16-byte chunks per 16-deep k step
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be made of 32x32 blocks");
};

// ---------------------------------------------------------------------------
// Loads: a wave instruction fills 8 consecutive LDS rows (64 lanes x 16 B,
// lane-contiguous); lane l fetches global chunk (l % 8) ^ swz_of(row) of its row so
// the LDS image is the XOR-swizzled layout the fragment reads expect.  Each operand's
// buffer resource starts at the tile's first row and covers only its valid rows, so
// rows past M or N read as zero without any per-load check.  STAGES-deep ring:
// stage kt + STAGES - 1 is issued right after the barrier that ends the reads of the
// buffer it overwrites.
// ---------------------------------------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

template <bool V>
struct LiveTag {
  static constexpr bool value = V;
};

// Buffer resource over `rows` rows of `row_bytes` starting at `base` (gfx9 layout: 48-bit
// base, stride 0, num_records in bytes, default format word); reads past it return 0.
__device__ __forceinline__ i32x4 rsrc_rows(const char* base, long rows, long row_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const long n = rows > 0 ? rows * row_bytes : 0;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(int32_t(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane(int32_t((a >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(int32_t(n));
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane from buffer `r` at byte offset `voff` into LDS at `lds_addr` + 16 * lane.
// Issued as inline asm so the compiler's wait-count pass does not see an LDS write it cannot
// disambiguate (it would otherwise drain every load in flight before each LDS read); the
// caller waits on vmcnt itself.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds16(i32x4 r, uint32_t lds_addr, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r)
               : "memory", "m0");
}
// as load_lds16, plus a wave-uniform byte offset `soff` added to the address
__device__ __forceinline__ void load_lds16_so(i32x4 r, uint32_t lds_addr, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <typename T, int BM, int BN, int WGM, int WGN, int EPI, int STAGES>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(const char* __restrict__ A, const char* __restrict__ B,
                                                                 const char* __restrict__ B2, const void* __restrict__ R,
                                                                 void* __restrict__ C, int M, int N, int K, int tiles_m,
                                                                 int tiles_n, int splits, int kt_per_split,
                                                                 float* __restrict__ part) {
  using G = Cfg<T, BM, BN, WGM, WGN, EPI>;
  constexpr int NB = G::NB, FM = G::FM, FN = G::FN, CPK = G::CPK;
  constexpr int ROWS = G::ROWS, BK = G::BK, WM = G::WM, WN = G::WN;
  constexpr int W = WGM * WGN;
  constexpr int INSTR = ROWS / 8;        // wave instructions per stage
  static_assert(INSTR % W == 0, "stage rows must split evenly over the waves");
  constexpr int IPW = INSTR / W;
  __shared__ uint4 lds[STAGES][ROWS * kChunks];

  // work units: (tile, K split), M tiles fastest, then N tiles, then splits
  const int n_tiles = tiles_m * tiles_n;
  const int n_units = n_tiles * splits;
  const int b = blockIdx.x;
  const int q = n_units / 8, rem = n_units % 8, x = b % 8;
  const int t = x * q + min(x, rem) + b / 8;
  const int tile = t % n_tiles, sp = t / n_tiles;
  const int m0 = (tile % tiles_m) * BM, n0 = (tile / tiles_m) * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches below
  const int wm = wave / WGN, wn = wave % WGN;
  const long kbytes = long(K) * G::EB;
  const auto ra = rsrc_rows(A + m0 * kbytes, min(BM, M - m0), kbytes);
  const auto rb = rsrc_rows(B + n0 * kbytes, min(BN, N - n0), kbytes);
  const auto rb2 = rsrc_rows((NB == 2 ? B2 : B) + n0 * kbytes, min(BN, N - n0), kbytes);
  const int lrow = lane >> 3;

  // Load instruction i of a wave fills LDS rows (i * W + wave) * 8 .. + 7 of a stage.
  // W * 8 divides BM and BN, so whether instruction i reads A, B or B2 depends on i
  // alone; its per-lane byte offset inside the operand is fixed for the whole K loop
  // and the stage's K position is added as a scalar offset.
  constexpr int RPI = 8 * W;
  static_assert(BM % RPI == 0 && BN % RPI == 0, "tile rows must split evenly over the waves");
  int voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = i * RPI + wave * 8 + lrow;                 // LDS row of this lane's chunk
    const int orow = (i * RPI < BM) ? row : (NB == 1 || i * RPI < BM + BN) ? row - BM : row - BM - BN;
    voff[i] = int(orow * kbytes) + (((lane & 7) ^ swz_of(row)) << 4);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(&lds[0][0])));
  constexpr uint32_t SLOT = ROWS * kRowBytes;
  // instructions [i0, i1) of stage kt into ring slot buf
  auto issue = [&](int kt, int buf, int i0, int i1) {
    const int soff = kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      if (i < i0 || i >= i1) continue;
      const uint32_t dst = lds0 + buf * SLOT + uint32_t((i * RPI + wave * 8) * kRowBytes);
      if (i * RPI < BM) load_lds16_so(ra, dst, voff[i], soff);
      else if (NB == 1 || i * RPI < BM + BN) load_lds16_so(rb, dst, voff[i], soff);
      else load_lds16_so(rb2, dst, voff[i], soff);
    }
  };

  f32x16 acc[NB][FM][FN];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[nb][i][j] = f32x16{};

  const int lr = lane & 31, kg = lane >> 5;
  // this unit's K stages [kt0, kt0 + nk)
  const int kt0 = sp * kt_per_split;
  const int nk = min(K / BK - kt0, kt_per_split);
  constexpr int KS = BK / 16;     // 16-deep MFMA steps per stage
  // A wave whose rows all lie past M (the last M tile of a ragged M) still issues
  // its share of the loads and meets every barrier, but skips the LDS reads and MFMAs.
  const bool live = m0 + wm * WM < M;
  auto k_loop = [&](auto live_tag) {
    constexpr bool LIVE = decltype(live_tag)::value;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(kt0 + s, s, 0, IPW);
    for (int kt = 0; kt < nk; ++kt) {
      // stage kt must have landed: the stages issued after it may stay in flight
      const int after = min(STAGES - 2, nk - 1 - kt);
      if constexpr (STAGES >= 3) {
        if (after >= 1) wait_vmcnt<IPW>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<0>();
      }
      // A bare barrier: every wave has waited for its own loads of stage kt above, and
      // its reads of the slot refilled during this stage were consumed by MFMAs before
      // it arrived.  (A fence here would also drain the stages still in flight.)
      __builtin_amdgcn_s_barrier();
      const bool refill = kt + STAGES - 1 < nk;
      const int kn = kt0 + kt + STAGES - 1, bn = (kt + STAGES - 1) % STAGES;
      const uint4* buf = lds[kt % STAGES];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int chunk = ks * CPK + kg * (CPK / 2);
        Frag8<T> fa[FM], fb[NB][FN];
        if constexpr (LIVE) {
#pragma unroll
          for (int i = 0; i < FM; ++i) lds_frag<T>(fa[i], buf, wm * WM + i * 32 + lr, chunk);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < FN; ++j) lds_frag<T>(fb[nb][j], buf, BM + nb * BN + wn * WN + j * 32 + lr, chunk);
        }
        // The next stage's loads, spread over the MFMA steps of this one.  With a
        // two-slot ring they must land before the next barrier, so they go out in the
        // first half of the steps; deeper rings spread them over all of them.
        constexpr int SPREAD = STAGES == 2 ? (KS + 1) / 2 : KS;
        if (refill && ks < SPREAD) issue(kn, bn, (IPW * ks) / SPREAD, (IPW * (ks + 1)) / SPREAD);
        if constexpr (LIVE) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j) mma32x32_k16(acc[nb][i][j], fa[i], fb[nb][j]);
        }
      }
    }
  };
  if (live) k_loop(LiveTag<true>{});
  else k_loop(LiveTag<false>{});
  if (!live) return;

  if (splits > 1) {
    // fp32 partial of this K split: part[sp][nb][row][col]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WN + j * 32 + lr;
          float* pp = part + (long(sp) * NB + nb) * long(M) * N;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * kg + (r & 3);
            if (row < M && col < N) pp[long(row) * N + col] = acc[nb][i][j][r];
          }
        }
    return;
  }

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

// Sums the K-split partials of gemm_kernel in split order and applies the epilogue:
// C = epi(sum_s part[s][0]) (SwiGLU: silu(sum_s part[s][0]) * sum_s part[s][1]).
template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, const void* __restrict__ R,
                                                          void* __restrict__ C, long MN, int splits) {
  constexpr int NB = (EPI == XP_EPI_SWIGLU) ? 2 : 1;
  for (long idx = long(blockIdx.x) * 256 + threadIdx.x; idx < MN; idx += long(gridDim.x) * 256) {
    float v = part[idx];
    for (int s = 1; s < splits; ++s) v += part[long(s) * NB * MN + idx];
    if constexpr (EPI == XP_EPI_F32) {
      reinterpret_cast<float*>(C)[idx] = v;
    } else if constexpr (EPI == XP_EPI_ADD_T) {
      reinterpret_cast<float*>(C)[idx] = St<T>::load(R, idx) + v;
    } else if constexpr (EPI == XP_EPI_ADD_F32) {
      reinterpret_cast<float*>(C)[idx] = reinterpret_cast<const float*>(R)[idx] + v;
    } else {
      float u = part[MN + idx];
      for (int s = 1; s < splits; ++s) u += part[(long(s) * NB + 1) * MN + idx];
      St<T>::store(C, idx, v / (1.0f + __expf(-v)) * u);
    }
  }
}

}  // namespace gemm
}  // namespace xp
