// The MFMA GEMM, as a template over block tile, wave grid, LDS ring depth and stage
// row size.
//
// C = epilogue(A B^T): A [M, K] and B [N, K] (K contiguous), fp32 accumulation.
// Block tile BM x BN, WGM x WGN waves, wave tile (BM/WGM) x (BN/WGN) made of
// 32x32 MFMA blocks.  Each stage is an RB-byte slice of K per row (RB = 128: 64 bf16
// or 32 fp32), copied from HBM straight into an LDS ring (buffer_load ... lds: no
// staging registers, no LDS store instructions) whose 16-byte chunks are
// XOR-swizzled per row (see Rows).  The SwiGLU epilogue reads two weight tiles
// (gate, up) against the same A tile and keeps both accumulators, so silu(g) * u is
// formed in registers.
//
// Inside a stage the fragments of the next 16-deep step are read from LDS while the
// current step's MFMAs run.  Measured on MI355X, these kernels are bound by the vector
// memory path that fills the ring (the address and data units are 85-90% busy, mostly
// waiting on L2 reads of about 600 cycles), then by LDS reads; with both taken out the
// same loop reaches 0.8 of the bf16 peak.
//
// Block order is XCD-aware: workgroups are dealt to the 8 XCDs round-robin, so
// block b is remapped to tile (b % 8) * per_xcd + b / 8 with tiles ordered
// M-fastest; the M tiles that share one weight tile then run on one XCD and
// share its L2.
//
// The K loop order (16-deep MFMA steps, in order) is the same for every M and every
// tile shape, so a row's result does not depend on which other rows are co-batched
// with it.
#pragma once
#include "rope.h"
#include "xp_device.h"
#include "../../include/xp.h"

namespace xp {
namespace gemm {

// Stage rows are RB bytes of K: 128 (8 chunks of 16 bytes) or 64 (4 chunks).  The
// chunk position of a row is XOR-swizzled so that the 16 consecutive rows one
// 16-lane group of a fragment read touches cover the 64 banks once: with 128-byte
// rows a row pair spans the banks and the 8 pairs get 8 positions ((row >> 1) & 7);
// with 64-byte rows 4 rows span them and the 4 quads get 4 positions ((row >> 2) & 3).
template <int RB>
struct Rows {
  static constexpr int chunks = RB / 16;
  static_assert(RB == 64 || RB == 128, "stage rows are 64 or 128 bytes");
  __device__ static __forceinline__ int swz_of(int row) { return RB == 128 ? (row >> 1) & 7 : (row >> 2) & 3; }
  __device__ static __forceinline__ int swz(int row, int chunk) { return row * chunks + (chunk ^ swz_of(row)); }
};

template <typename T, int RB>
__device__ __forceinline__ void lds_frag(Frag8<T>& f, const uint4* buf, int row, int chunk) {
  using Rw = Rows<RB>;
  if constexpr (sizeof(Frag8<T>) == 16) {
    f.v = buf[Rw::swz(row, chunk)];
  } else {
    uint4 a = buf[Rw::swz(row, chunk)], b = buf[Rw::swz(row, chunk + 1)];
    f.lo = __builtin_bit_cast(float4, a);
    f.hi = __builtin_bit_cast(float4, b);
  }
}

// Internal epilogue of the QKV projection: RoPE and the step's appends (rope.h) instead
// of an fp32 store; its kernel argument is the step's PostQkvArgs.
constexpr int kEpiRope = 16;
struct NoEpiArg {};
template <int EPI> struct EpiArg { using type = NoEpiArg; };
template <> struct EpiArg<kEpiRope> { using type = PostQkvArgs; };

template <typename T, int BM, int BN, int WGM, int WGN, int EPI, int RB = 128>
struct Cfg {
  static constexpr int THREADS = 64 * WGM * WGN;
  static constexpr int EB = St<T>::bytes;
  static constexpr int BK = RB / EB;
  static constexpr int NB = (EPI == XP_EPI_SWIGLU) ? 2 : 1;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int ROWS = BM + NB * BN;
  static constexpr int CPK = 16 * EB / 16;       // 16-byte chunks per 16-deep k step
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be made of 32x32 blocks");
};

// ---------------------------------------------------------------------------
// Loads: a wave instruction fills 1024 bytes of consecutive LDS rows (64 lanes x 16 B,
// lane-contiguous); lane l fetches global chunk (l % chunks) ^ swz_of(row) of its row
// so the LDS image is the XOR-swizzled layout the fragment reads expect.  Each
// operand's buffer resource starts at the tile's first row and covers only its valid
// rows, so rows past M or N read as zero without any per-load check.  STAGES-deep
// ring: stage kt + STAGES - 1 is issued after the barrier that ends the reads of the
// slot it overwrites.
// ---------------------------------------------------------------------------

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// s_barrier with compiler fences on both sides: no LDS access moves across it.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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

// the resource itself (mask -1) or the same resource with no records (mask 0)
__device__ __forceinline__ i32x4 gate(i32x4 r, int mask) {
  r.z &= mask;
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

template <typename T, int BM, int BN, int WGM, int WGN, int EPI, int STAGES, int RB = 128, bool FOLD = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(const char* __restrict__ A, const char* __restrict__ B,
                                                                 const char* __restrict__ B2, const void* __restrict__ R,
                                                                 void* __restrict__ C, int M, int N, int K, int tiles_m,
                                                                 int tiles_n, int splits, int kt_per_split,
                                                                 float* __restrict__ part,
                                                                 typename EpiArg<EPI>::type ea) {
  using G = Cfg<T, BM, BN, WGM, WGN, EPI, RB>;
  using Rw = Rows<RB>;
  constexpr int NB = G::NB, FM = G::FM, FN = G::FN, CPK = G::CPK;
  constexpr int ROWS = G::ROWS, BK = G::BK, WM = G::WM, WN = G::WN;
  constexpr int W = WGM * WGN;
  constexpr int CH = Rw::chunks;
  constexpr int LR = 64 / CH;            // LDS rows one wave instruction fills
  constexpr int INSTR = ROWS / LR;       // wave instructions per stage
  static_assert(INSTR % W == 0, "stage rows must split evenly over the waves");
  constexpr int IPW = INSTR / W;
  __shared__ uint4 lds[STAGES][ROWS * CH];

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
  const int lrow = lane / CH;

  // The RoPE epilogue's lookups (each row's position and page ids, each item's cos/sin
  // pairs) depend only on the tile, so they are issued here and land during the K loop.
  [[maybe_unused]] constexpr int RHPT = BN / 64;                      // heads per tile, at most
  [[maybe_unused]] constexpr int RIPT = (BM * BN / 8 + G::THREADS - 1) / G::THREADS;   // items per thread
  [[maybe_unused]] int rope_pos_r = 0, rope_page_r[RHPT > 0 ? RHPT : 1] = {};
  [[maybe_unused]] constexpr bool RPRE = RIPT <= 6;                   // cos/sin prefetched (register budget)
  [[maybe_unused]] float4 rope_c[RPRE ? RIPT : 1][2];
  if constexpr (EPI == kEpiRope) {
    const PostQkvArgs& ra = ea;
    const int d = ra.d, half = d / 2, pq = d / 8, hpt = BN / d, head0 = n0 / d, n_heads = ra.Hq + 2 * ra.Hkv;
    static_assert(BM <= G::THREADS, "one thread per tile row");
    const int rr = threadIdx.x;
    if (rr < BM && m0 + rr < M) {
      const int row = m0 + rr;
      rope_pos_r = rope_pos(ra, row);
#pragma unroll
      for (int hl = 0; hl < RHPT; ++hl) {
        const int h = head0 + hl;
        const int g = h >= ra.Hq + ra.Hkv ? h - ra.Hq - ra.Hkv : h - ra.Hq;
        if (hl < hpt && h >= ra.Hq && h < n_heads) rope_page_r[hl] = rope_page(ra, row, g, rope_pos_r);
      }
    }
#pragma unroll
    for (int k = 0; k < (RPRE ? RIPT : 0); ++k) {
      const int e = threadIdx.x + k * G::THREADS;
      const int er = e / (hpt * pq), hl = (e / pq) % hpt, j = 4 * (e % pq);
      const int row = m0 + er, h = head0 + hl;
      rope_c[k][0] = rope_c[k][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < BM * hpt * pq && row < M && h < ra.Hq + ra.Hkv) {
        rope_c[k][0] = *reinterpret_cast<const float4*>(ra.rope_tab + long(row) * half + j);
        rope_c[k][1] = *reinterpret_cast<const float4*>(ra.rope_tab + long(row) * half + j + 2);
      }
    }
  }

  // Load instruction i of a wave fills LDS rows (i * W + wave) * LR .. + LR - 1 of a
  // stage.  W * LR divides BM and BN, so whether instruction i reads A, B or B2 depends
  // on i alone; its per-lane byte offset inside the operand is fixed for the whole K
  // loop and the stage's K position is added as a scalar offset.
  constexpr int RPI = LR * W;
  static_assert(BM % RPI == 0 && BN % RPI == 0, "tile rows must split evenly over the waves");
  int voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int row = i * RPI + wave * LR + lrow;                // LDS row of this lane's chunk
    const int orow = (i * RPI < BM) ? row : (NB == 1 || i * RPI < BM + BN) ? row - BM : row - BM - BN;
    voff[i] = int(orow * kbytes) + (((lane % CH) ^ Rw::swz_of(row)) << 4);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(&lds[0][0])));
  constexpr uint32_t SLOT = ROWS * RB;
  // instructions [i0, i1) of stage kt into ring slot buf; with on == false the loads
  // use zero-record resources (they return zeros and fetch nothing)
  auto issue = [&](int kt, int buf, int i0, int i1, bool on) {
    const int soff = kt * RB;
    const int nr = on ? -1 : 0;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      if (i < i0 || i >= i1) continue;
      const uint32_t dst = lds0 + buf * SLOT + uint32_t((i * RPI + wave * LR) * RB);
      if (i * RPI < BM) load_lds16_so(gate(ra, nr), dst, voff[i], soff);
      else if (NB == 1 || i * RPI < BM + BN) load_lds16_so(gate(rb, nr), dst, voff[i], soff);
      else load_lds16_so(gate(rb2, nr), dst, voff[i], soff);
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
  // this unit's K stages [kt0, kt0 + nk); with FOLD the unit covers all of K as
  // consecutive chunks of kt_per_split stages (see the fold below)
  const int kt0 = FOLD ? 0 : sp * kt_per_split;
  const int nk = FOLD ? K / BK : min(K / BK - kt0, kt_per_split);
  constexpr int KS = BK / 16;     // 16-deep MFMA steps per stage
  static_assert(KS % 2 == 0, "fragment double buffer alternates over an even number of steps");
  constexpr int NF = FM + NB * FN;                        // fragments per 16-deep step
  // The refill of a stage is spread over the first SPREAD steps of the stage before it.
  // With a two-slot ring it must land by the next stage's start, so it goes out early.
  constexpr int SPREAD = STAGES == 2 ? KS / 2 : KS - 1;
  // A wave whose rows all lie past M (the last M tile of a ragged M) still issues
  // its share of the loads and meets every barrier, but skips the LDS reads and MFMAs.
  const bool live = m0 + wm * WM < M;
  auto read = [&](Frag8<T>* dst, const uint4* buf, int ks) {
    const int chunk = ks * CPK + kg * (CPK / 2);
#pragma unroll
    for (int i = 0; i < FM; ++i) lds_frag<T, RB>(dst[i], buf, wm * WM + i * 32 + lr, chunk);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < FN; ++j) lds_frag<T, RB>(dst[FM + nb * FN + j], buf, BM + nb * BN + wn * WN + j * 32 + lr, chunk);
  };
  // Software pipeline: the fragments of step ks + 1 are read while the MFMAs of step ks
  // run (two register sets).  With a ring of three or more slots the barrier that hands
  // the next stage over is taken in the last step of a stage, after this stage's reads
  // have all returned, so the first fragments of the next stage are in flight during
  // that step's MFMAs.  A two-slot ring keeps the barrier at the start of each stage
  // instead: its refill then has the whole stage to land.  Refill loads are
  // unconditional (the stages past the unit's range read nothing: their resource has no
  // records), so each stage is one straight-line block.
  constexpr bool EARLY = STAGES >= 3;
  // FOLD: a long-K product is summed over fixed K chunks in chunk order.  Split into
  // units, each chunk is a unit and the reduction adds the chunk results in order;
  // unsplit, one unit accumulates chunk by chunk and folds each finished chunk into a
  // running total, in the same order: ((c0 + c1) + c2) + ...  Both give the same bits,
  // so the launcher may choose either for any row count.
  [[maybe_unused]] f32x16 tot[NB][FM][FN];
  auto fold = [&](bool first) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          tot[nb][i][j] = first ? acc[nb][i][j] : tot[nb][i][j] + acc[nb][i][j];
          acc[nb][i][j] = f32x16{};
        }
  };
  auto k_loop = [&](auto live_tag) {
    constexpr bool LIVE = decltype(live_tag)::value;
    [[maybe_unused]] int chunk_left = kt_per_split, chunks_done = 0;
    Frag8<T> f[2][NF];
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(kt0 + s, s, 0, IPW, s < nk);
    if constexpr (EARLY) {
      wait_vmcnt<IPW * (STAGES - 2)>();
      barrier();
      if constexpr (LIVE) read(f[0], lds[0], 0);
    }
    for (int kt = 0; kt < nk; ++kt) {
      const uint4* buf = lds[kt % STAGES];
      const int kn = kt0 + kt + STAGES - 1, bn = (kt + STAGES - 1) % STAGES;
      const bool refill = kt + STAGES - 1 < nk;
      if constexpr (!EARLY) {
        // stage kt has landed and every wave is done with the slot refilled below
        wait_vmcnt<0>();
        barrier();
        if constexpr (LIVE) read(f[0], buf, 0);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag8<T>* cur = f[ks & 1];
        Frag8<T>* nxt = f[(ks + 1) & 1];
        if (ks < KS - 1) {
          if constexpr (LIVE) read(nxt, buf, ks + 1);
          if (ks < SPREAD) issue(kn, bn, (IPW * ks) / SPREAD, (IPW * (ks + 1)) / SPREAD, refill);
        } else if constexpr (EARLY) {
          // this stage's fragments are all in registers before its slot is released;
          // the next stage's own loads have landed (the later stages may stay in flight)
          wait_lgkmcnt0();
          wait_vmcnt<IPW * (STAGES - 2)>();
          barrier();
          if constexpr (LIVE) read(nxt, lds[(kt + 1) % STAGES], 0);
        }
        // the reads above go out before this step's MFMAs (no reordering across)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (LIVE) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
              for (int j = 0; j < FN; ++j) mma32x32_k16(acc[nb][i][j], cur[i], cur[FM + nb * FN + j]);
        }
      }
      if constexpr (FOLD && LIVE) {
        if (--chunk_left == 0 && kt + 1 < nk) {
          fold(chunks_done == 0);
          ++chunks_done;
          chunk_left = kt_per_split;
        }
      }
    }
    if constexpr (FOLD && LIVE) {
      if (chunks_done > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[nb][i][j] = tot[nb][i][j] + acc[nb][i][j];
      }
    }
    // the loads of the stages past the range still write the ring: drain them
    wait_vmcnt<0>();
  };
  if (live) k_loop(LiveTag<true>{});
  else k_loop(LiveTag<false>{});

  // ---- epilogue ----
  // Each 32x32 accumulator block goes through a wave-private LDS patch (the ring is
  // free once every wave is past this barrier: all reads are consumed and all loads
  // drained) and is read back as rows of 4 consecutive columns per lane, so the
  // residual loads and the output stores move whole 16-byte (fp32) or 8-byte (bf16)
  // pieces of a row instead of single elements.  Patch rows are 40 floats apart: the
  // two rows one MFMA-layout store instruction writes (r and r + 4) then fall in
  // opposite halves of the 64 banks, and each 16-lane group of a read takes rows r and
  // r + 4 as well.  The arithmetic per element is unchanged.
  barrier();
  if constexpr (EPI == kEpiRope) {
    // RoPE + appends of the QKV projection.  The tile goes through the drained ring as
    // [BM][BN + 8] fp32 (rows 8 floats apart put the two half-waves of an MFMA-layout
    // store on disjoint banks), so a rotation pair (dims j and j + d/2 of one head, held
    // by different waves) is in one place; BN is a multiple of d, so a tile holds whole
    // heads.  Each row's position and, per key/value head of the tile, the page of its
    // slot (looked up before the K loop) go to LDS beside the tile.  Items of the first
    // pass are (row, head, dims j .. j + 3 < d/2 and their partners j + d/2) of query and
    // key heads, rotated and stored; value heads, stored as they are, take a second pass.
    const PostQkvArgs& ra = ea;
    constexpr int TP = BN + 8;
    constexpr int HPT_MAX = BN / 64;                         // heads per tile, at most (d >= 64)
    static_assert(BM * TP * 4 + BM * (1 + HPT_MAX) * 4 <= STAGES * SLOT, "the staged tile fits in the ring");
    float* tile = reinterpret_cast<float*>(&lds[0][0]);
    int* rpos = reinterpret_cast<int*>(tile + BM * TP);      // [BM] positions
    int* rpage = rpos + BM;                                  // [BM][HPT_MAX] pages
    const int d = ra.d, half = d / 2, pq = d / 8, hpt = BN / d, head0 = n0 / d;
    const int n_heads = ra.Hq + 2 * ra.Hkv;
    if (live) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            tile[(wm * WM + i * 32 + 8 * (r >> 2) + 4 * kg + (r & 3)) * TP + wn * WN + j * 32 + lr] = acc[0][i][j][r];
    }
    if (threadIdx.x < BM) {
      rpos[threadIdx.x] = rope_pos_r;
#pragma unroll
      for (int hl = 0; hl < RHPT; ++hl) rpage[threadIdx.x * HPT_MAX + hl] = rope_page_r[hl];
    }
    barrier();
#pragma unroll
    for (int k = 0; k < RIPT; ++k) {
      const int e = threadIdx.x + k * G::THREADS;
      if (e >= BM * hpt * pq) break;
      const int rr = e / (hpt * pq), hl = (e / pq) % hpt, j = 4 * (e % pq);
      const int row = m0 + rr, h = head0 + hl;
      if (row >= M || h >= ra.Hq + ra.Hkv) continue;       // value heads: the pass below
      const int pos = rpos[rr], page = rpage[rr * HPT_MAX + hl];
      const float* src = tile + rr * TP + hl * d;
      const float4 x0 = *reinterpret_cast<const float4*>(src + j), x1 = *reinterpret_cast<const float4*>(src + j + half);
      float4 c01, c23;
      if constexpr (RPRE) {
        c01 = rope_c[k][0];
        c23 = rope_c[k][1];
      } else {
        c01 = *reinterpret_cast<const float4*>(ra.rope_tab + long(row) * half + j);
        c23 = *reinterpret_cast<const float4*>(ra.rope_tab + long(row) * half + j + 2);
      }
      const float2 cs[4] = {make_float2(c01.x, c01.y), make_float2(c01.z, c01.w), make_float2(c23.x, c23.y),
                            make_float2(c23.z, c23.w)};
      float4 y0, y1;
      rope_pair4(x0, x1, cs, y0, y1);
      rope_store4<T>(ra, row, h, j, y0, pos, page);
      rope_store4<T>(ra, row, h, j + half, y1, pos, page);
    }
    // Value heads, whose page plane is dim-major: an item is 4 rows x 4 dims, so that
    // rows on consecutive slots of one page leave as one 4-slot store per dim.  Lanes
    // take the four row quads of 16 rows first, then the dim quads.
    static_assert(BM % 16 == 0, "value pass walks 16-row groups");
    if (head0 + hpt > ra.Hq + ra.Hkv) {
      const int n_items = BM / 4 * hpt * (d / 4);
      for (int e = threadIdx.x; e < n_items; e += G::THREADS) {
        const int qd = e & 3, g = (e >> 2) % (d / 4), rest = e / d;
        const int rr0 = (rest % (BM / 16)) * 16 + qd * 4, hl = rest / (BM / 16);
        const int row0 = m0 + rr0, h = head0 + hl;
        if (row0 >= M || h < ra.Hq + ra.Hkv || h >= n_heads) continue;
        float4 x[4];
        int pos[4], page[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = *reinterpret_cast<const float4*>(tile + (rr0 + i) * TP + hl * d + 4 * g);
          pos[i] = rpos[rr0 + i];
          page[i] = rpage[(rr0 + i) * HPT_MAX + hl];
        }
        const bool run = row0 + 3 < M && (ra.S & 3) == 0 && (pos[0] & 3) == 0 && page[0] >= 0 &&
                         page[0] < ra.n_pages && page[1] == page[0] && page[2] == page[0] && page[3] == page[0] &&
                         pos[1] == pos[0] + 1 && pos[2] == pos[0] + 2 && pos[3] == pos[0] + 3;
        if (run) {
          const int S = ra.S;
          const long vb = long(page[0]) * 2 * S * d + long(S) * d + long(4 * g) * S + pos[0] % S;
          St4<T>::store(ra.pool, vb, make_float4(x[0].x, x[1].x, x[2].x, x[3].x));
          St4<T>::store(ra.pool, vb + S, make_float4(x[0].y, x[1].y, x[2].y, x[3].y));
          St4<T>::store(ra.pool, vb + 2 * S, make_float4(x[0].z, x[1].z, x[2].z, x[3].z));
          St4<T>::store(ra.pool, vb + 3 * S, make_float4(x[0].w, x[1].w, x[2].w, x[3].w));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (row0 + i < M) rope_store4<T>(ra, row0 + i, h, 4 * g, x[i], pos[i], page[i]);
        }
      }
    }
    return;
  }
  if (!live) return;
  constexpr int PS = 40;                                   // patch row stride (floats)
  float* patch = reinterpret_cast<float*>(&lds[0][0]) + wave * (32 * PS);
  const bool vec = (N & 3) == 0;
  const int rsub = lane >> 3, c4 = (lane & 7) * 4;
  const int rperm = (rsub >> 1) + 4 * (rsub & 1);          // 16-lane group: rows r, r + 4
  // stores a 32x32 block `v` (MFMA layout) at rows r0.., cols c0.. through f(row, col, x4)
  auto emit = [&](const f32x16& v, int r0, int c0, auto&& f) {
#pragma unroll
    for (int r = 0; r < 16; ++r) patch[(8 * (r >> 2) + 4 * kg + (r & 3)) * PS + lr] = v[r];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int pr = it * 8 + rperm;
      const float4 x = *reinterpret_cast<const float4*>(&patch[pr * PS + c4]);
      const int row = r0 + pr, col = c0 + c4;
      if (row < M) f(row, col, x);
    }
  };
  // writes 4 consecutive values of row `row` from column `col` (vector when whole and
  // aligned, else element by element inside N)
  auto put4 = [&](auto* out, int row, int col, float4 x, auto&& g) {
    const long idx = long(row) * N + col;
    if (vec && col + 3 < N) {
      g(out, idx, x, true);
    } else {
      const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (col + q < N) g(out, idx + q, make_float4(e[q], 0.f, 0.f, 0.f), false);
    }
  };
  auto store_f32 = [](float* out, long idx, float4 x, bool v4) {
    if (v4) *reinterpret_cast<float4*>(out + idx) = x;
    else out[idx] = x.x;
  };

  if (splits > 1) {
    // fp32 partial of this K split: part[sp][nb][row][col]
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float* pp = part + (long(sp) * NB + nb) * long(M) * N;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          emit(acc[nb][i][j], m0 + wm * WM + i * 32, n0 + wn * WN + j * 32,
               [&](int row, int col, float4 x) { put4(pp, row, col, x, store_f32); });
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r0 = m0 + wm * WM + i * 32, c0 = n0 + wn * WN + j * 32;
      if constexpr (EPI == XP_EPI_F32) {
        emit(acc[0][i][j], r0, c0,
             [&](int row, int col, float4 x) { put4(reinterpret_cast<float*>(C), row, col, x, store_f32); });
      } else if constexpr (EPI == XP_EPI_ADD_T || EPI == XP_EPI_ADD_F32) {
        emit(acc[0][i][j], r0, c0, [&](int row, int col, float4 x) {
          put4(reinterpret_cast<float*>(C), row, col, x, [&](float* out, long idx, float4 y, bool v4) {
            if (v4) {
              const float4 rr = EPI == XP_EPI_ADD_F32 ? St4<float>::load(R, idx) : St4<T>::load(R, idx);
              *reinterpret_cast<float4*>(out + idx) = make_float4(rr.x + y.x, rr.y + y.y, rr.z + y.z, rr.w + y.w);
            } else {
              const float rv = EPI == XP_EPI_ADD_F32 ? reinterpret_cast<const float*>(R)[idx] : St<T>::load(R, idx);
              out[idx] = rv + y.x;
            }
          });
        });
      } else {
        f32x16 h;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = acc[0][i][j][r], u = acc[NB - 1][i][j][r];
          h[r] = v / (1.0f + __expf(-v)) * u;
        }
        emit(h, r0, c0, [&](int row, int col, float4 x) {
          put4(C, row, col, x, [&](void* out, long idx, float4 y, bool v4) {
            if (v4) St4<T>::store(out, idx, y);
            else St<T>::store(out, idx, y.x);
          });
        });
      }
    }
}

// Sums the K-split partials of gemm_kernel in split order and applies the epilogue:
// C = epi(sum_s part[s][0]) (SwiGLU: silu(sum_s part[s][0]) * sum_s part[s][1]).
// V4: four consecutive elements per thread (MN a multiple of 4), the same sums.
template <typename T, int EPI, bool V4>
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part, const void* __restrict__ R,
                                                          void* __restrict__ C, long MN, int splits) {
  constexpr int NB = (EPI == XP_EPI_SWIGLU) ? 2 : 1;
  if constexpr (V4) {
    const float4* p4 = reinterpret_cast<const float4*>(part);
    const long MN4 = MN / 4;
    auto add = [](float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); };
    for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < MN4; i += long(gridDim.x) * 256) {
      float4 v = p4[i];
      for (int s = 1; s < splits; ++s) v = add(v, p4[long(s) * NB * MN4 + i]);
      if constexpr (EPI == XP_EPI_F32) {
        reinterpret_cast<float4*>(C)[i] = v;
      } else if constexpr (EPI == XP_EPI_ADD_T) {
        reinterpret_cast<float4*>(C)[i] = add(St4<T>::load(R, 4 * i), v);
      } else if constexpr (EPI == XP_EPI_ADD_F32) {
        reinterpret_cast<float4*>(C)[i] = add(reinterpret_cast<const float4*>(R)[i], v);
      } else {
        float4 u = p4[MN4 + i];
        for (int s = 1; s < splits; ++s) u = add(u, p4[(long(s) * NB + 1) * MN4 + i]);
        St4<T>::store(C, 4 * i,
                      make_float4(v.x / (1.0f + __expf(-v.x)) * u.x, v.y / (1.0f + __expf(-v.y)) * u.y,
                                  v.z / (1.0f + __expf(-v.z)) * u.z, v.w / (1.0f + __expf(-v.w)) * u.w));
      }
    }
  } else {
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
}

}  // namespace gemm
}  // namespace xp
