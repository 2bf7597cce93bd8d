// Causal chunked-prefill attention on one SP rank's head subset, over the
// cached prior keys plus the chunk (ConfluxServe §4 and App. A: with Ulysses SP
// each rank computes complete attention for the heads it owns over the whole
// chunk, and later chunks reuse the head-sharded history; the mask is the
// inclusive causal mask of Adaptive Context Parallelism §2.1).  All keys are
// read from the paged pool: the chunk's own K/V were appended before.
//
// Work decomposition: a workgroup owns one KV head g, one query tile of 32*NQ
// chunk rows and one split of the tile's key range (`bps` 32-key blocks), with
// one wave per query head of g's GQA group (up to 8), so each K/V block is read
// from HBM once for the whole group.  A wave covers the whole query tile for its
// head, as NQ 32-query MFMA column blocks: every K or V fragment it reads from
// LDS feeds NQ MFMAs, and the NQ accumulation chains are independent.  Blocks
// (two pages: 8 KB of K rows + 8 KB of V^T rows for d = 128 bf16) are copied
// straight into an LDS ring of two-block stages with buffer_load ... lds.  A
// workgroup of a small grid may hold two waves per head (two key sets), each set
// taking every other block of the split, merged in LDS at the end.  gfx950's LDS serves
// 16-byte reads 16 lanes at a time over 64 banks (256 bytes): the K plane's chunk-major
// page layout already puts one dim chunk of 16 keys in 256 consecutive bytes, and the
// V^T plane is XOR-swizzled in 16-byte chunks so 16 dim rows of a read land on
// distinct banks.  Splitting the key range gives
// long prior contexts enough workgroups; a tile whose keys fit in one split
// writes its output directly, the others write fp32 (max, sum, output) partials
// that `prefill_combine_kernel` merges (the log-sum-exp merge of Decode Token
// Parallelism Eq. 4).
//
// Per wave, block and query column block j, 32x32 MFMA tiles:
//   S^T[32 keys x 32 queries] = K[32 x d] . Q_j^T[d x 32]      (16-deep k steps)
//   O_j^T[d x 32 queries]   += V^T[d x 32 keys] . P_j^T        (16-deep k steps)
// Queries are the MFMA columns, so lane l owns query l % 32 of each column block
// for both the scores and the output: the row max needs one exchange with lane
// l ^ 32 and the rescale is per lane.  Row i of the K operand holds key kappa(i)
// of the block (bits 2 and 3 of i swapped), which makes accumulator elements
// 0..7 of lane l the keys 8*(l/32) .. +7 of the first page and elements 8..15 the
// same slots of the second page -- exactly the k-slots the PV step's P operand
// supplies, and the V^T operand is then 8 consecutive slots of one dim row.
#include "gemm_core.h"
#include <algorithm>
#include <type_traits>
#include <vector>

#include "xp_device.h"
#include "xp_internal.h"

namespace xp {

namespace {

constexpr int kPage = 16;
constexpr int kNQ = 1;               // 32-query column blocks per wave
constexpr int kMaxW = 8;             // waves (query heads) per workgroup
constexpr int kStages = 2;           // LDS ring stages, one key set
constexpr int kStagesKS2 = 3;        // LDS ring stages, two key sets
constexpr int kStagesPipe = 3;       // LDS ring stages, the block-pipelined loop
constexpr int kBlocksPerStage = 2;   // 32-key blocks per stage
constexpr int kBlocksPerStagePipe = 3;   // 32-key blocks per stage, the block-pipelined loop
constexpr int kMaxBps = 256;   // key blocks per split (its page ids are staged in LDS)
constexpr int kXcds = 8;       // XCDs the hardware deals consecutive workgroups to, in turn

__device__ __forceinline__ int kappa(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ void zero_from(Frag8<bf16_t>& f, int nvalid) {
  uint32_t w[4] = {f.v.x, f.v.y, f.v.z, f.v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
  f.v = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void zero_from(Frag8<float>& f, int nvalid) {
  if (nvalid <= 0) f.lo.x = 0.f;
  if (nvalid <= 1) f.lo.y = 0.f;
  if (nvalid <= 2) f.lo.z = 0.f;
  if (nvalid <= 3) f.lo.w = 0.f;
  if (nvalid <= 4) f.hi.x = 0.f;
  if (nvalid <= 5) f.hi.y = 0.f;
  if (nvalid <= 6) f.hi.z = 0.f;
  if (nvalid <= 7) f.hi.w = 0.f;
}

// Maximum of two scores as one v_med3 (the median of a, b and +inf).  fmaxf costs an
// extra quieting instruction per operand produced by an MFMA; scores are never
// signalling NaNs (slots past the table end are replaced by -inf before any maximum),
// so the median gives the same value.  The +inf comes from a scalar register the
// compiler cannot see through (with a literal +inf it turns the median back into
// fmaxf).
__device__ __forceinline__ float opaque_inf() {
  float v;
  asm("s_mov_b32 %0, 0x7f800000" : "=s"(v));
  return v;
}
__device__ __forceinline__ float smax(float a, float b, float inf) { return __builtin_amdgcn_fmed3f(a, b, inf); }
// the maximum of 16 scores
template <typename V>
__device__ __forceinline__ float max16(const V& v, float inf) {
  const float lo = smax(smax(smax(v[0], v[1], inf), smax(v[2], v[3], inf), inf),
                        smax(smax(v[4], v[5], inf), smax(v[6], v[7], inf), inf), inf);
  const float hi = smax(smax(smax(v[8], v[9], inf), smax(v[10], v[11], inf), inf),
                        smax(smax(v[12], v[13], inf), smax(v[14], v[15], inf), inf), inf);
  return smax(lo, hi, inf);
}

// log2-domain margin by which a row maximum may exceed the softmax reference
// before O and l are rescaled
constexpr float kLazy = 8.0f;

// Packs 8 weights into a PV operand fragment (rounding them to the operand type)
// and returns the sum of the rounded weights, so the normaliser sums exactly the
// weights the PV product uses.
__device__ __forceinline__ float pack_and_sum(Frag8<bf16_t>& f, const float* p) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  set_frag8(f, p);
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, f.v.x), one2, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, f.v.y), one2, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, f.v.z), one2, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, f.v.w), one2, s, false);
}
__device__ __forceinline__ float pack_and_sum(Frag8<float>& f, const float* p) {
  set_frag8(f, p);
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// LDS planes.  K: the page's K plane copied as it is stored, 16-byte chunks of dims
// chunk-major over the page's 16 slots (chunk c of key k at (c * 16 + k) * 16), so a
// 16-lane group reading one chunk of 16 keys reads 256 consecutive bytes: all 64
// banks once.  V^T: rows of VROW_CH chunks, one per dim; dim row r's chunk c sits at
// c ^ vswz(r), which alternates every 256 bytes of rows.
template <int VROW_CH>
__device__ __forceinline__ int vswz(int r) {
  constexpr int ROWS256 = 16 / VROW_CH;                       // V^T rows per 256-byte bank line
  return (r / ROWS256) & (VROW_CH - 1);
}
__device__ __forceinline__ const uint4* kchunk(const char* plane, int k, int c) {
  return reinterpret_cast<const uint4*>(plane + (c * kPage + k) * 16);
}
// K fragment of key k: dims [elem0, elem0 + 8)
__device__ __forceinline__ void kfrag(Frag8<bf16_t>& f, const char* plane, int k, int elem0) {
  f.v = *kchunk(plane, k, elem0 / 8);
}
__device__ __forceinline__ void kfrag(Frag8<float>& f, const char* plane, int k, int elem0) {
  f.lo = __builtin_bit_cast(float4, *kchunk(plane, k, elem0 / 4));
  f.hi = __builtin_bit_cast(float4, *kchunk(plane, k, elem0 / 4 + 1));
}
// V^T fragment: 8 consecutive key slots [8*hf, 8*hf + 8) of dim row r
template <int VROW_CH>
__device__ __forceinline__ void vfrag(Frag8<bf16_t>& f, const char* plane, int r, int hf) {
  f.v = *reinterpret_cast<const uint4*>(plane + (r * VROW_CH + (hf ^ vswz<VROW_CH>(r))) * 16);
}
template <int VROW_CH>
__device__ __forceinline__ void vfrag(Frag8<float>& f, const char* plane, int r, int hf) {
  f.lo = *reinterpret_cast<const float4*>(plane + (r * VROW_CH + ((2 * hf) ^ vswz<VROW_CH>(r))) * 16);
  f.hi = *reinterpret_cast<const float4*>(plane + (r * VROW_CH + ((2 * hf + 1) ^ vswz<VROW_CH>(r))) * 16);
}

struct PrefillArgs {
  const void* q;
  const char* pool;
  int n_pages;
  const int32_t* pre_pages;
  int pre_max_blocks;
  int hq, hkv, prior, chunk, off, n_local;
  void* out_local;
  int out_local_stride;
  void* out_peer;
  int out_peer_stride;
  float scale_log2;
  uint32_t* status;
  int bps;        // 32-key blocks per split
  int n_split;    // splits in the grid (the longest tile's)
  int wpg;        // waves per workgroup (query heads of the group it covers)
  int qt_rows;    // queries per tile (32 * NQ)
  float* part_ml; // [n_qt, hq, n_split, qt_rows, 2]
  float* part_o;  // [n_qt, hq, n_split, qt_rows, D]
};

// s_waitcnt vmcnt(min(n, 63)) for a wave-uniform n (gfx950's counter holds 6 bits;
// a larger n waits for more than necessary, never less)
__device__ __forceinline__ void wait_vm_le(int n) {
#define XP_VM_CASE(k) \
  case k: gemm::wait_vmcnt<k>(); break;
#define XP_VM_CASE8(k) XP_VM_CASE(k) XP_VM_CASE(k + 1) XP_VM_CASE(k + 2) XP_VM_CASE(k + 3) \
  XP_VM_CASE(k + 4) XP_VM_CASE(k + 5) XP_VM_CASE(k + 6) XP_VM_CASE(k + 7)
  switch (n < 63 ? n : 63) {
    XP_VM_CASE8(0) XP_VM_CASE8(8) XP_VM_CASE8(16) XP_VM_CASE8(24)
    XP_VM_CASE8(32) XP_VM_CASE8(40) XP_VM_CASE8(48) XP_VM_CASE8(56)
    default: gemm::wait_vmcnt<0>(); break;
  }
#undef XP_VM_CASE8
#undef XP_VM_CASE
}

// output row pointer of chunk row t (local rows and peer rows go to different buffers)
__device__ __forceinline__ void out_row(const PrefillArgs& a, int t, void*& dst, long& row_off) {
  if (t >= a.off && t < a.off + a.n_local) {
    dst = a.out_local;
    row_off = long(t - a.off) * a.out_local_stride;
  } else {
    dst = a.out_peer;
    row_off = long(t < a.off ? t : t - a.n_local) * a.out_peer_stride;
  }
}

// PIPE: the block-pipelined loop (one key set, one query column block, 16-bit
// operands; below).
template <typename T, int D, int NQ, int MAXW, int KS, bool PIPE = false>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int bx, int by) {
  constexpr int EB = St<T>::bytes;
  constexpr int QT = 32 * NQ;                     // queries per tile
  constexpr int PLANE = kPage * D * EB;           // bytes of one K or V plane of a page
  constexpr long PAGE_BYTES = 2L * PLANE;
  constexpr int BLK = 4 * PLANE;                  // one 32-key block: K_A | K_B | V_A | V_B
  constexpr int CH_PER_PLANE = PLANE / 16;        // 16-byte chunks per plane
  constexpr int INSTR_BLK = 4 * CH_PER_PLANE / 64;  // 64-lane load instructions per block
  constexpr int VROW_CH = kPage * EB / 16;        // 16-byte chunks per V^T row
  // blocks per stage and ring depth, within the LDS budget
  constexpr int kBudget = 144 * 1024;
  static_assert(!PIPE || (KS == 1 && NQ == 1 && sizeof(T) == 2), "the pipelined loop: one key set, NQ = 1, bf16");
  constexpr int kSt = KS == 2 ? kStagesKS2 : (PIPE ? kStagesPipe : kStages);
  constexpr int kBps = PIPE ? kBlocksPerStagePipe : kBlocksPerStage;
  constexpr int SB = kBps * kSt * BLK <= kBudget ? kBps
                     : kBlocksPerStage * 2 * BLK <= kBudget
                         ? kBlocksPerStage
                         : (kBudget / (2 * BLK) > 0 ? kBudget / (2 * BLK) : 1);
  constexpr int NST = kSt * SB * BLK <= kBudget ? kSt : (kBudget / (SB * BLK) > 2 ? kBudget / (SB * BLK) : 2);
  constexpr int STAGE = SB * BLK;
  __shared__ uint4 ring[NST][STAGE / 16];
  __shared__ int32_t pids[2 * kMaxBps];
  // KS key sets: with KS = 2 the workgroup holds two waves per query head; set k
  // consumes the blocks at odd or even positions of the split's key range, and the
  // two partial softmax states are merged through LDS at the end.
  static_assert(KS == 1 || (KS == 2 && SB % 2 == 0 && MAXW * NQ * D * 128 <= NST * STAGE),
                "two key sets need an even number of blocks per stage and a ring that holds one set's state");

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kset = KS == 1 ? 0 : wave_all / a.wpg;
  const int wave = KS == 1 ? wave_all : wave_all % a.wpg;   // query head of the group
  const int G = a.hq / a.hkv;
  const int n_qt = (a.chunk + QT - 1) / QT;
  // Work units (query tile, key split), longest tiles first, in groups of kXcds adjacent
  // tiles with the tile fastest: the hardware deals consecutive workgroups to the XCDs
  // in turn, so each XCD takes one tile of every group with all of its splits.  (With
  // the split fastest, split s would always land on XCD s mod kXcds, and the later
  // splits of short causal tiles hold no keys: the first XCDs would get most of the work.)
  const int grp = bx / (kXcds * a.n_split), rem = bx % (kXcds * a.n_split);
  const int s = rem / kXcds;
  const int qt = n_qt - 1 - (grp * kXcds + rem % kXcds);
  if (qt < 0) return;                                       // padding of the last group
  const int groups_per_kv = (G + a.wpg - 1) / a.wpg;
  const int g = by / groups_per_kv;
  const int h0 = g * G + (by % groups_per_kv) * a.wpg;   // first query head of this workgroup
  const int waves = min(a.wpg, g * G + G - h0);
  const int t0 = qt * QT;
  const int q_last = min(t0 + QT - 1, a.chunk - 1);
  const int n_keys = a.prior + a.chunk;                     // keys in the table
  const int nkb = (a.prior + q_last + 1 + 31) / 32;         // key blocks this tile needs
  const int kb0 = s * a.bps;
  if (kb0 >= nkb) return;                                   // uniform over the workgroup
  const int kb1 = min(nkb, kb0 + a.bps);
  const int ns = (nkb + a.bps - 1) / a.bps;
  const bool active = wave < waves;
  const int h = h0 + (active ? wave : 0);
  const int32_t* tbl = a.pre_pages + long(g) * a.pre_max_blocks;

  // The split's page ids, staged once and validated: table reads inside the pipeline
  // would be vector loads, and waiting for one of them would also wait for every
  // ring load before it.  An id outside the pool is staged as -1 (its page then
  // reads as zeros) and flags the workgroup.
  __shared__ int bad_s;
  if (threadIdx.x == 0) bad_s = 0;
  __syncthreads();
  const int n_tbl = (n_keys + kPage - 1) / kPage;
  for (int i = int(threadIdx.x); i < 2 * (kb1 - kb0); i += int(blockDim.x)) {
    const int b = 2 * kb0 + i;
    const int pid = b < n_tbl ? tbl[b] : -1;
    const bool ok = pid >= 0 && pid < a.n_pages;
    if (b < n_tbl && !ok) bad_s = 1;
    pids[i] = ok ? pid : -1;
  }
  __syncthreads();
  const bool bad = bad_s != 0;

  // Loads are issued a whole block at a time by one wave: block b of every stage by
  // wave b % waves, so its page resources are set up once and its 64-lane load
  // instructions have fixed LDS destinations.  Blocks past the split load through
  // empty resources (moving no data), so each wave issues the same number of
  // instructions for every stage and the wait counts below are exact.
  const int nl = KS * waves, lw = kset * waves + wave;     // loading waves, this wave's index
  int my_blocks = 0;
  for (int b = lw; b < SB; b += nl) ++my_blocks;
  const int my_instr = wave < waves ? my_blocks * INSTR_BLK : 0;   // per stage
  auto issue_block = [&](int sg, int b, int buf) {
    const int kb = kb0 + sg * SB + b;
    const bool in = kb < kb1;
    const int2 pp = in ? *reinterpret_cast<const int2*>(&pids[2 * (kb - kb0)]) : make_int2(-1, -1);
    const int pa = __builtin_amdgcn_readfirstlane(pp.x), pb = __builtin_amdgcn_readfirstlane(pp.y);
    const gemm::i32x4 ra = gemm::rsrc_rows(a.pool + (pa >= 0 ? long(pa) : 0L) * PAGE_BYTES, pa >= 0 ? 1 : 0, PAGE_BYTES);
    const gemm::i32x4 rb = gemm::rsrc_rows(a.pool + (pb >= 0 ? long(pb) : 0L) * PAGE_BYTES, pb >= 0 ? 1 : 0, PAGE_BYTES);
    const uint32_t dst0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(&ring[buf][(b * BLK) / 16])));
#pragma unroll
    for (int i = 0; i < INSTR_BLK; ++i) {
      const int region = i / (CH_PER_PLANE / 64);         // 0 K_A, 1 K_B, 2 V_A, 3 V_B
      const int p = (i % (CH_PER_PLANE / 64)) * 64 + lane;  // chunk position inside the plane
      int src;
      if (region < 2) {
        src = p * 16;                 // the K plane as stored
      } else {
        const int row = p / VROW_CH, c = (p % VROW_CH) ^ vswz<VROW_CH>(row);
        src = PLANE + (row * VROW_CH + c) * 16;
      }
      gemm::load_lds16((region & 1) ? rb : ra, dst0 + (region * CH_PER_PLANE + (i % (CH_PER_PLANE / 64)) * 64) * 16, src);
    }
  };

  const int ql = lane & 31, hf = lane >> 5;

  Frag8<T> qf[NQ][D / 16];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const char* qrow = static_cast<const char*>(a.q) + (long(h) * a.chunk + min(t0 + 32 * j + ql, a.chunk - 1)) * D * EB;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) load_frag8(qf[j][st], qrow + (16 * st + 8 * hf) * EB);
  }
  // Settle these loads before any ring load is issued: the compiler waits for them at
  // their first use inside the loop, and with in-order completion such a wait would
  // also drain the ring stages in flight.
  gemm::wait_vmcnt<0>();

  f32x16 o[NQ][D / 32];
  float ms[NQ], lsum[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
#pragma unroll
    for (int n = 0; n < D / 32; ++n) o[j][n] = f32x16{};
    ms[j] = -__builtin_inff();
    lsum[j] = 0.f;
  }

  const int krow = kappa(ql);
  if constexpr (PIPE) {
    // Block-pipelined loop.  Each step issues the PV MFMAs of the previous block
    // between the masking and maximum of this block's scores, and the QK MFMAs of the
    // next block between this block's exponentials and packing, so a wave keeps its
    // matrix pipe fed through its own softmax instead of leaving that to the other
    // wave of its SIMD.  The rescale of block i still precedes block i's PV product
    // and every sum runs in the plain loop's order: both loops give the same bits.
    // The last block of a stage has its V^T fragments read after the barrier that
    // opens the next stage, so that barrier refills the slot of the stage before
    // (a three-slot ring), with the next stage's loads issued as it opens.
    constexpr int NM = D / 16;                    // MFMAs of each product per block
    const int n = kb1 - kb0;
    const int n_sg = (n + SB - 1) / SB;
    auto open_stage = [&](int sg) {
      gemm::wait_vmcnt<0>();                      // this wave's loads of stage sg landed
      __builtin_amdgcn_s_barrier();
      if (sg + 1 < n_sg && wave < waves)
        for (int b = lw; b < SB; b += nl) issue_block(sg + 1, b, (sg + 1) % NST);
    };
    if (wave < waves)
      for (int b = lw; b < SB; b += nl) issue_block(0, b, 0);
    if (!active) {
      for (int sg = 0; sg < n_sg; ++sg) open_stage(sg);
    } else {
      open_stage(0);
      auto blk = [&](int i) { return reinterpret_cast<const char*>(ring[(i / SB) % NST]) + (i % SB) * BLK; };
      const int kofs = krow < kPage ? 0 : PLANE, kr = krow & 15;
      Frag8<T> kf[NM], vf[2][D / 32], pf[2];
      // the first step's PV product adds zeros
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pf[u].v = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int nn = 0; nn < D / 32; ++nn) vf[u][nn].v = make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int st = 0; st < NM; ++st) kfrag(kf[st], blk(0) + kofs, kr, 16 * st + 8 * hf);
      f32x16 sc = f32x16{};
#pragma unroll
      for (int st = 0; st < NM; ++st) mma32x32_k16(sc, kf[st], qf[0][st]);
      for (int sg = 0; sg < n_sg; ++sg) {
#pragma unroll
        for (int b = 0; b < SB; ++b) {
          const int i = sg * SB + b;
          if (i >= n) break;
          const int key0 = (kb0 + i) * 32;
          // causal mask (blocks that cross the diagonal)
          if (key0 + 31 > a.prior + t0) {
            const int lim = a.prior + min(t0 + ql, a.chunk - 1) - (key0 + 8 * hf);
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] = (16 * (r >> 3) + (r & 7) > lim) ? -__builtin_inff() : sc[r];
          }
          // PV of block i - 1 | K fragments of block i + 1 (same stage) | block maximum
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nn = 0; nn < D / 32; ++nn) mma32x32_k16(o[0][nn], vf[u][nn], pf[u]);
          if (b + 1 < SB) {
#pragma unroll
            for (int st = 0; st < NM; ++st) kfrag(kf[st], blk(i + 1) + kofs, kr, 16 * st + 8 * hf);
          }
          const float inf = opaque_inf();
          float mb = max16(sc, inf);
          float m0, m1;
          halves_xor32(mb, m0, m1);
          mb = smax(m0, m1, inf) * a.scale_log2;
#pragma unroll
          for (int k = 0; k < NM; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
          }
          if (__builtin_amdgcn_ballot_w64(mb > ms[0] + kLazy) != 0) {
            const float mn = fmaxf(ms[0], mb);
            const float alpha = ms[0] == -__builtin_inff() ? 0.f : fast_exp2(ms[0] - mn);
            ms[0] = mn;
            lsum[0] *= alpha;
#pragma unroll
            for (int nn = 0; nn < D / 32; ++nn) o[0][nn] *= alpha;
          }
          const float mref = ms[0] == -__builtin_inff() ? 0.f : ms[0];
          if (b + 1 == SB && sg + 1 < n_sg) open_stage(sg + 1);
          // QK of block i + 1 | weights of block i | V^T fragments of block i.  Past the
          // last block the K fragments are stale and that product goes unused.
          if (b + 1 == SB) {
#pragma unroll
            for (int st = 0; st < NM; ++st) kfrag(kf[st], blk(i + 1) + kofs, kr, 16 * st + 8 * hf);
          }
          f32x16 sn = f32x16{};
#pragma unroll
          for (int st = 0; st < NM; ++st) mma32x32_k16(sn, kf[st], qf[0][st]);
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            float pu[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) pu[r] = fast_exp2(__builtin_fmaf(sc[8 * u + r], a.scale_log2, -mref));
            lsum[0] += pack_and_sum(pf[u], pu);
          }
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nn = 0; nn < D / 32; ++nn) vfrag<VROW_CH>(vf[u][nn], blk(i) + (2 + u) * PLANE, 32 * nn + ql, hf);
          if (b + 1 == SB) __builtin_amdgcn_sched_group_barrier(0x100, NM, 0);
#pragma unroll
          for (int k = 0; k < NM; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          sc = sn;
        }
      }
      // slots at or past the table end hold no key (their V^T columns may hold
      // anything, including NaN): only the table's last block has them, and it can
      // only be the last block of a split
      const int key_last = (kb1 - 1) * 32;
      if (key_last + 32 > n_keys) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int nn = 0; nn < D / 32; ++nn) zero_from(vf[u][nn], n_keys - (key_last + 16 * u + 8 * hf));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int nn = 0; nn < D / 32; ++nn) mma32x32_k16(o[0][nn], vf[u][nn], pf[u]);
    }
  } else {
  // stages 0 .. NST - 2 in flight before the first one is consumed; stage
  // sg + NST - 1 is then issued block by block while stage sg is consumed, into the
  // ring slot every wave finished reading before the barrier that opened stage sg
  const int n_sg = (kb1 - kb0 + SB - 1) / SB;
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (i < n_sg && wave < waves)
      for (int b = lw; b < SB; b += nl) issue_block(i, b, i);
  for (int sg = 0; sg < n_sg; ++sg) {
    // stage sg has landed once no more than the later stages' loads are outstanding
    wait_vm_le(min(NST - 2, n_sg - 1 - sg) * my_instr);
    __builtin_amdgcn_s_barrier();
    const bool refill = sg + NST - 1 < n_sg;
#pragma unroll 1
    for (int b = 0; b < SB; ++b) {
      if (refill && wave < waves && b % nl == lw) issue_block(sg + NST - 1, b, (sg + NST - 1) % NST);
      const int kb = kb0 + sg * SB + b;
      if (!active || kb >= kb1 || (KS == 2 && (b & 1) != kset)) continue;
      const char* st_base = reinterpret_cast<const char*>(ring[sg % NST]) + b * BLK;
      const int key0 = kb * 32;
      // All K fragments of the block are read up front, then the V^T fragments right
      // after the QK MFMAs are issued, so the LDS latency hides behind MFMAs and the
      // softmax instead of stalling each MFMA on its own read.
      const char* kplane = st_base + (krow < kPage ? 0 : PLANE);
      const int kr = krow & 15;
      Frag8<T> kf[D / 16];
#pragma unroll
      for (int st = 0; st < D / 16; ++st) kfrag(kf[st], kplane, kr, 16 * st + 8 * hf);
      // S^T = K . Q^T; K operand row ql holds key kappa(ql) of the block
      f32x16 sacc[NQ];
#pragma unroll
      for (int j = 0; j < NQ; ++j) sacc[j] = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
#pragma unroll
        for (int j = 0; j < NQ; ++j) mma32x32_k16(sacc[j], kf[st], qf[j][st]);
      Frag8<T> vf[2][D / 32];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int n = 0; n < D / 32; ++n) vfrag<VROW_CH>(vf[u][n], st_base + (2 + u) * PLANE, 32 * n + ql, hf);
      // issue order: the K reads, the QK MFMAs, then the V^T reads
      constexpr int KREADS = (D / 16) * (sizeof(Frag8<T>) / 16), VREADS = D / 16 * (sizeof(Frag8<T>) / 16);
      __builtin_amdgcn_sched_group_barrier(0x100, KREADS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NQ * (D / 16) * (sizeof(Frag8<T>) / 16 == 2 ? 8 : 1), 0);
      __builtin_amdgcn_sched_group_barrier(0x100, VREADS, 0);

      // Online softmax in the exp2 domain with a lazily moved reference: ms is the
      // row maximum (scaled) a rescale last set, and the weights exp2(s c - ms) stay
      // below 2^kLazy while no new score exceeds ms by more than kLazy, so O and l
      // are rescaled only when some row of the wave crosses that margin (the result
      // is the same function of the scores; only the rounding points move).  Only
      // blocks that cross the causal diagonal are masked.
      const bool masked = key0 + 31 > a.prior + t0;       // uniform over the wave
      Frag8<T> pf[NQ][2];   // the weights as PV operands: slots 8u .. 8u + 7 of the block
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        // element r: key key0 + 16*(r/8) + 8*hf + r%8 for query t0 + 32 j + ql
        float sv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = sacc[j][r];
        if (masked) {
          const int lim = a.prior + min(t0 + 32 * j + ql, a.chunk - 1) - (key0 + 8 * hf);
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[r] = (16 * (r >> 3) + (r & 7) > lim) ? -__builtin_inff() : sv[r];
        }
        const float inf = opaque_inf();
        float mb = max16(sv, inf);
        float m0, m1;
        halves_xor32(mb, m0, m1);
        mb = smax(m0, m1, inf) * a.scale_log2;
        if (__builtin_amdgcn_ballot_w64(mb > ms[j] + kLazy) != 0) {
          const float mn = fmaxf(ms[j], mb);
          const float alpha = ms[j] == -__builtin_inff() ? 0.f : fast_exp2(ms[j] - mn);
          ms[j] = mn;
          lsum[j] *= alpha;
#pragma unroll
          for (int n = 0; n < D / 32; ++n) o[j][n] *= alpha;
        }
        const float mref = ms[j] == -__builtin_inff() ? 0.f : ms[j];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float pu[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) pu[r] = fast_exp2(__builtin_fmaf(sv[8 * u + r], a.scale_log2, -mref));
          lsum[j] += pack_and_sum(pf[j][u], pu);
        }
      }
      // slots at or past the table end hold no key (their V^T columns may hold
      // anything, including NaN): only the last block of the table has them
      if (key0 + 32 > n_keys) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int n = 0; n < D / 32; ++n) zero_from(vf[u][n], n_keys - (key0 + 16 * u + 8 * hf));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
#pragma unroll
          for (int j = 0; j < NQ; ++j) mma32x32_k16(o[j][n], vf[u][n], pf[j][u]);
    }
  }
  }
  if (bad && a.status && lane == 0 && wave_all == 0) atomicOr(a.status, XP_DEV_BAD_PAGE);
  if constexpr (KS == 2) {
    // set 1 hands its state to set 0 through the drained ring: o as [head][j][n][r][lane]
    // floats, (reference, sum) beside it; set 0 rescales both to the larger reference
    __shared__ float xml[MAXW * NQ * 2 * 64];
    float* xo = reinterpret_cast<float*>(&ring[0][0]);
    __syncthreads();
    if (kset == 1 && active) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) xo[(((wave * NQ + j) * (D / 32) + n) * 16 + r) * 64 + lane] = o[j][n][r];
        xml[((wave * NQ + j) * 2) * 64 + lane] = ms[j];
        xml[((wave * NQ + j) * 2 + 1) * 64 + lane] = lsum[j];
      }
    }
    __syncthreads();
    if (kset == 1) return;
    if (active) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const float m1 = xml[((wave * NQ + j) * 2) * 64 + lane], l1 = xml[((wave * NQ + j) * 2 + 1) * 64 + lane];
        const float mn = fmaxf(ms[j], m1);
        const float a0 = ms[j] == -__builtin_inff() ? 0.f : fast_exp2(ms[j] - mn);
        const float a1 = m1 == -__builtin_inff() ? 0.f : fast_exp2(m1 - mn);
        ms[j] = mn;
        lsum[j] = lsum[j] * a0 + l1 * a1;
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            o[j][n][r] = o[j][n][r] * a0 + xo[(((wave * NQ + j) * (D / 32) + n) * 16 + r) * 64 + lane] * a1;
      }
    }
  }
  if (!active) return;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int t = t0 + 32 * j + ql;
    const float ls = lsum[j] + shfl_xor(lsum[j], 32);
    if (ns == 1) {
      if (t >= a.chunk) continue;
      const float inv = bad ? __builtin_nanf("") : 1.0f / ls;
      void* dst;
      long row_off;
      out_row(a, t, dst, row_off);
      const long base = row_off + long(h) * D;
      // element r of o[j][n]: dim 32*n + 8*(r/4) + 4*hf + r%4
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          St<T>::store(dst, base + 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3), o[j][n][r] * inv);
      continue;
    }
    const long unit = ((long(qt) * a.hq + h) * a.n_split + s) * QT + 32 * j + ql;
    if (hf == 0) {
      a.part_ml[2 * unit] = bad ? __builtin_nanf("") : ms[j];
      a.part_ml[2 * unit + 1] = ls;
    }
    float* po = a.part_o + unit * D;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(po + 32 * n + 8 * r4 + 4 * hf) =
            make_float4(o[j][n][4 * r4], o[j][n][4 * r4 + 1], o[j][n][4 * r4 + 2], o[j][n][4 * r4 + 3]);
  }
}

// merges the split partials of the tiles that were split (scores in the exp2 domain):
// the split weights of each query are formed once, then every thread sums float4
// slices of the partial outputs with independent loads.
constexpr int kMaxSplits = 64;
constexpr int kMaxQT = 64;          // queries per tile, at most

template <typename T, int D>
__device__ __forceinline__ void prefill_combine_tile(const PrefillArgs& a, int qt, int h) {
  __shared__ float wts[kMaxSplits][kMaxQT];
  const int QT = a.qt_rows;
  const int q_last = min(qt * QT + QT - 1, a.chunk - 1);
  const int nkb = (a.prior + q_last + 1 + 31) / 32;
  const int ns = (nkb + a.bps - 1) / a.bps;
  if (ns <= 1) return;
  const long u0 = ((long(qt) * a.hq + h) * a.n_split) * QT;   // unit of (split 0, query 0)
  if (int(threadIdx.x) < QT) {
    const int ql = threadIdx.x;
    float mx = -__builtin_inff();
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.part_ml[2 * (u0 + s * QT + ql)]);
    float L = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float w = fast_exp2(a.part_ml[2 * (u0 + s * QT + ql)] - mx);
      wts[s][ql] = w;
      L += a.part_ml[2 * (u0 + s * QT + ql) + 1] * w;
    }
    const float inv = 1.0f / L;
    for (int s = 0; s < ns; ++s) wts[s][ql] *= inv;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < QT * (D / 4); e += 256) {
    const int ql = e / (D / 4), j4 = e % (D / 4);
    const int t = qt * QT + ql;
    if (t >= a.chunk) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < ns; ++s) {
      const float4 v = reinterpret_cast<const float4*>(a.part_o + (u0 + s * QT + ql) * D)[j4];
      const float w = wts[s][ql];
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    void* dst;
    long row_off;
    out_row(a, t, dst, row_off);
    const long o = row_off + long(h) * D + 4 * j4;
    St<T>::store(dst, o, acc.x);
    St<T>::store(dst, o + 1, acc.y);
    St<T>::store(dst, o + 2, acc.z);
    St<T>::store(dst, o + 3, acc.w);
  }
}

template <typename T, int D, int NQ, int MAXW, int KS, bool PIPE = false>
__global__ __launch_bounds__(64 * MAXW * KS) void prefill_kernel(PrefillArgs a) {
  prefill_tile<T, D, NQ, MAXW, KS, PIPE>(a, int(blockIdx.x), int(blockIdx.y));
}

// The co-resident form, for prefill running beside decode attention on the same CUs:
// the same tiles within 168 registers per wave, so that a SIMD holds two prefill waves
// and one of decode's co-resident waves.  Its waves issue at a raised priority: decode
// waiting on its page loads then fills the issue slots prefill leaves, instead of
// competing for them (measured: C5 step 1035 -> 1003 us, C3 719 -> 684 us; the other way
// round, decode first, 1099 and 745 us).
template <typename T, int D, int NQ, int MAXW, int KS>
__global__ __launch_bounds__(64 * MAXW * KS) __attribute__((amdgpu_waves_per_eu(3))) void prefill_cores_kernel(
    PrefillArgs a) {
  __builtin_amdgcn_s_setprio(2);
  prefill_tile<T, D, NQ, MAXW, KS>(a, int(blockIdx.x), int(blockIdx.y));
}

template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
  prefill_combine_tile<T, D>(a, int(blockIdx.x), int(blockIdx.y));
}

// Several chunks' prefill attention in one launch (the scheduled prefills of one
// step, ConfluxServe §6.2 Eq. 6): member j owns the flat workgroups [start[j],
// start[j + 1]) and lays them out as its own grid of width gx[j]; its combine owns
// [cstart[j], cstart[j + 1]) with width cgx[j].  A small chunk alone leaves most CUs
// idle; in one launch the chunks' tiles share the device.
constexpr int kMaxGroup = 8;
struct PrefillGroup {
  int n;
  int start[kMaxGroup + 1], gx[kMaxGroup];
  int cstart[kMaxGroup + 1], cgx[kMaxGroup];
  PrefillArgs a[kMaxGroup];
};

// Member of flat workgroup b (uniform): every read of the kernel arguments uses a
// constant index, so they stay scalar loads of the argument segment.
__device__ __forceinline__ void group_member(const PrefillGroup& g, int b, bool combine, PrefillArgs& a, int& x,
                                             int& y) {
  int j = 0;
#pragma unroll
  for (int k = 1; k < kMaxGroup; ++k) j += (k < g.n && b >= (combine ? g.cstart[k] : g.start[k])) ? 1 : 0;
  int s0 = 0, w = 1;
  switch (j) {
#define XP_MEMBER(k) \
  case k: a = g.a[k]; s0 = combine ? g.cstart[k] : g.start[k]; w = combine ? g.cgx[k] : g.gx[k]; break;
    XP_MEMBER(0) XP_MEMBER(1) XP_MEMBER(2) XP_MEMBER(3) XP_MEMBER(4) XP_MEMBER(5) XP_MEMBER(6) XP_MEMBER(7)
#undef XP_MEMBER
  }
  x = (b - s0) % w;
  y = (b - s0) / w;
}

template <typename T, int D, int NQ, int MAXW, int KS, bool PIPE = false>
__global__ __launch_bounds__(64 * MAXW * KS) void prefill_group_kernel(PrefillGroup g) {
  PrefillArgs a;
  int x, y;
  group_member(g, int(blockIdx.x), false, a, x, y);
  prefill_tile<T, D, NQ, MAXW, KS, PIPE>(a, x, y);
}

template <typename T, int D, int NQ, int MAXW, int KS>
__global__ __launch_bounds__(64 * MAXW * KS) __attribute__((amdgpu_waves_per_eu(3))) void prefill_group_cores_kernel(
    PrefillGroup g) {
  __builtin_amdgcn_s_setprio(2);
  PrefillArgs a;
  int x, y;
  group_member(g, int(blockIdx.x), false, a, x, y);
  prefill_tile<T, D, NQ, MAXW, KS>(a, x, y);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_group_combine_kernel(PrefillGroup g) {
  PrefillArgs a;
  int x, y;
  group_member(g, int(blockIdx.x), true, a, x, y);
  prefill_combine_tile<T, D>(a, x, y);
}

struct Plan {
  int bps, n_split, wpg, nq, qt;
};

// Query column blocks per wave and waves per workgroup.
struct Shape {
  int nq, maxw;
};
Shape pick_shape(int d, int G) {
  (void)d;
  (void)G;
  return {kNQ, kMaxW};
}

// Key blocks per split (planned for the whole device in every split-attention mode, so
// the mode never changes the summation).  A candidate split count gives work units of at most bps
// 32-key blocks (a tile's key range cut into ceil(nkb / bps) pieces); the launch
// takes about max(total work / CUs, longest unit) plus half a longest unit when units
// outnumber the CUs, and every split unit adds its fp32 partials to the combine's
// reads.  The estimate (microseconds, per-block and per-unit costs measured on
// MI355X for d = 128 bf16) picks the candidate; on the 8B, 14B and 32B prefill
// batches it matches the longest-first schedule of the units over the CUs and the
// measured best split within a few percent (8B chunk: no split, 33 us vs 48 us at
// the previous fixed target of 8192 waves; 14B: 2 splits, 154 vs 192 us).
Plan plan(int hq, int hkv, int d, int prior, int chunk, int cus) {
  const int G = hq / hkv;
  const Shape sh = pick_shape(d, G);
  const int kQT = 32 * sh.nq;
  const int n_qt = (chunk + kQT - 1) / kQT;
  const int max_nkb = (prior + chunk + 31) / 32;
  const int wpg = std::min(G, sh.maxw);
  const long groups = long(hkv) * ((G + wpg - 1) / wpg);
  const double t_blk = 0.75 + 0.065 * wpg, t_unit = 2.0;
  cus = std::max(1, cus);
  static constexpr int kCand[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
  double best = 1e300;
  Plan out{std::min(max_nkb, kMaxBps), (max_nkb + kMaxBps - 1) / kMaxBps, wpg, sh.nq, kQT};
  int last_bps = -1;
  for (int ns : kCand) {
    if (ns > kMaxSplits) break;
    const int bps = (max_nkb + ns - 1) / ns;
    if (bps > kMaxBps || bps == last_bps) continue;
    last_bps = bps;
    double total = 0.0, longest = 0.0;
    long n_units = 0, split_units = 0;
    for (int qt = 0; qt < n_qt; ++qt) {
      const int nkb = (prior + std::min(qt * kQT + kQT - 1, chunk - 1) + 1 + 31) / 32;
      const int n = (nkb + bps - 1) / bps;
      total += nkb * t_blk + n * t_unit;
      longest = std::max(longest, std::min(bps, nkb) * t_blk + t_unit);
      n_units += n;
      if (n > 1) split_units += n;
    }
    total *= double(groups);
    n_units *= groups;
    split_units *= groups;
    double t = std::max(total / cus, longest);
    if (n_units > cus) t = std::max(t, total / cus + 0.5 * longest);
    if (split_units) t += 3.0 + double(split_units) * kQT * wpg * (d + 2) * 4.0 / 5e12 * 1e6;
    if (t < best) {
      best = t;
      out.bps = bps;
      out.n_split = (max_nkb + bps - 1) / bps;
    }
  }
  return out;
}

}  // namespace

size_t prefill_ws_bytes(int hq, int hkv, int d, int prior, int chunk, int cus) {
  if (chunk <= 0) return 0;
  const Plan p = plan(hq, hkv, d, prior, chunk, cus);
  if (p.n_split <= 1) return 0;
  const size_t units = size_t((chunk + p.qt - 1) / p.qt) * hq * p.n_split * p.qt;
  return align_up(units * 2 * sizeof(float), 256) + align_up(units * d * sizeof(float), 256);
}

namespace {

// One chunk's launch: host checks, its key-split plan, kernel arguments and grids.
struct Prepared {
  PrefillArgs a;
  Plan p;
  int n_qt, gy, cus;
};

// Workgroups along x of one chunk's launch: whole groups of kXcds tiles, every split
int unit_grid(const Prepared& pr) { return cdiv(pr.n_qt, kXcds) * kXcds * pr.p.n_split; }

// Two key sets per workgroup (two waves per query head), for 32-bit operands, when the
// group has at most four heads, the grid has no more workgroups than CUs and the
// longest work unit spans at least 16 key blocks: each CU then holds one four-wave
// workgroup, and a second set of waves on the other half of the keys shortens the
// longest unit (1024-token 8B chunk, plain loop: 33 -> 29.5 us).  Larger grids already
// keep two workgroups per CU, and on short units the merge costs more than it saves
// (a 256-token chunk: 19.4 vs 21.2 us).  16-bit operands always take the pipelined
// loop with one key set, which overlaps a wave's own softmax with its MFMAs (the 8B
// chunk: 30.2 us against 31.2 with two key sets).
bool two_key_sets(const Prepared& pr, long workgroups) {
  const int nkb = (pr.a.prior + pr.a.chunk + 31) / 32;
  return pr.p.wpg <= 4 && workgroups <= pr.cus && std::min(nkb, pr.p.bps) >= 16;
}

xp_status prepare(const void* pool, int n_pages, int S, int hq, int hkv, int d, const PrefillJob& j, uint32_t* status,
                  int cus, Prepared& out) {
  if (S != kPage) return fail(XP_EUNSUPPORTED, "prefill attention: page_size %d (supported: 16)", S);
  if (hkv <= 0 || hq % hkv) return fail(XP_ESHAPE, "prefill attention: hq=%d hkv=%d", hq, hkv);
  if (d != 64 && d != 128) return fail(XP_EUNSUPPORTED, "prefill attention: head_dim %d", d);
  if (long(j.pre_max_blocks) * kPage < long(j.prior) + j.chunk)
    return fail(XP_EPAGE, "prefill attention: table of %d blocks < %d keys", j.pre_max_blocks, j.prior + j.chunk);
  if (j.off < 0 || j.n_local < 0 || j.off + j.n_local > j.chunk) return fail(XP_ESHAPE, "prefill attention: off/n_local");
  if ((long(j.prior) + j.chunk + 31) / 32 > long(kMaxBps) * kMaxSplits)
    return fail(XP_EUNSUPPORTED, "prefill attention: %d keys exceed %d", j.prior + j.chunk, 32 * kMaxBps * kMaxSplits);
  const Plan p = plan(hq, hkv, d, j.prior, j.chunk, cus);
  const size_t need = prefill_ws_bytes(hq, hkv, d, j.prior, j.chunk, cus);
  if (need && !j.ws) return fail(XP_EWORKSPACE, "prefill attention: needs %zu bytes of workspace", need);
  const size_t units = size_t((j.chunk + p.qt - 1) / p.qt) * hq * p.n_split * p.qt;
  float* ml = static_cast<float*>(j.ws);
  float* po = j.ws ? reinterpret_cast<float*>(static_cast<char*>(j.ws) + align_up(units * 2 * sizeof(float), 256)) : nullptr;
  out.a = PrefillArgs{j.q, static_cast<const char*>(pool), n_pages, j.pre_pages, j.pre_max_blocks, hq, hkv, j.prior,
                      j.chunk, j.off, j.n_local, j.out_local, j.out_local_stride, j.out_peer, j.out_peer_stride,
                      float(1.4426950408889634 / __builtin_sqrt(double(d))), status, p.bps, p.n_split, p.wpg, p.qt,
                      ml, po};
  out.p = p;
  out.n_qt = (j.chunk + p.qt - 1) / p.qt;
  const int G = hq / hkv;
  out.gy = hkv * ((G + p.wpg - 1) / p.wpg);
  out.cus = cus;
  return XP_OK;
}

// `cores`: decode runs beside this launch on the same CUs (its co-resident form), so
// the tiles take the co-resident kernel and one key set
template <typename T, int D>
void launch_one(const Prepared& pr, bool cores, hipStream_t s) {
  const dim3 grid(unit_grid(pr), pr.gy), block(64 * pr.p.wpg), cgrid(pr.n_qt, pr.a.hq);
  if (cores && sizeof(T) == 2) {
    // the co-resident form exists for 16-bit operands only (the step never asks for others)
    if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((prefill_cores_kernel<T, D, kNQ, kMaxW, 1>), grid, block, 0, s, pr.a);
  } else if (sizeof(T) != 2 && two_key_sets(pr, long(grid.x) * grid.y))
    hipLaunchKernelGGL((prefill_kernel<T, D, kNQ, 4, 2>), grid, dim3(2 * block.x), 0, s, pr.a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, D, kNQ, kMaxW, 1, sizeof(T) == 2>), grid, block, 0, s, pr.a);
  if (pr.p.n_split > 1) hipLaunchKernelGGL((prefill_combine_kernel<T, D>), cgrid, dim3(256), 0, s, pr.a);
}

template <typename T, int D>
void launch_group(const Prepared* pr, int n, bool cores, hipStream_t s) {
  PrefillGroup g{};
  g.n = n;
  bool split = false;
  for (int k = 0; k < n; ++k) {
    g.a[k] = pr[k].a;
    g.gx[k] = unit_grid(pr[k]);
    g.start[k + 1] = g.start[k] + g.gx[k] * pr[k].gy;
    const bool sk = pr[k].p.n_split > 1;
    split = split || sk;
    g.cgx[k] = pr[k].n_qt;
    g.cstart[k + 1] = g.cstart[k] + (sk ? pr[k].n_qt * pr[k].a.hq : 0);
  }
  if (cores && sizeof(T) == 2) {
    if constexpr (sizeof(T) == 2)
      hipLaunchKernelGGL((prefill_group_cores_kernel<T, D, kNQ, kMaxW, 1>), dim3(g.start[n]),
                         dim3(64 * pr[0].p.wpg), 0, s, g);
  } else if (sizeof(T) != 2 && two_key_sets(pr[0], g.start[n]))
    hipLaunchKernelGGL((prefill_group_kernel<T, D, kNQ, 4, 2>), dim3(g.start[n]), dim3(128 * pr[0].p.wpg), 0,
                       s, g);
  else
    hipLaunchKernelGGL((prefill_group_kernel<T, D, kNQ, kMaxW, 1, sizeof(T) == 2>), dim3(g.start[n]),
                       dim3(64 * pr[0].p.wpg), 0, s, g);
  if (split) hipLaunchKernelGGL((prefill_group_combine_kernel<T, D>), dim3(g.cstart[n]), dim3(256), 0, s, g);
}

template <typename F>
xp_status dispatch(int dtype, int d, F&& f) {
  if (dtype == XP_BF16) {
    if (d == 128) f(bf16_t{}, std::integral_constant<int, 128>{});
    else f(bf16_t{}, std::integral_constant<int, 64>{});
  } else if (dtype == XP_F32) {
    if (d == 128) f(float{}, std::integral_constant<int, 128>{});
    else f(float{}, std::integral_constant<int, 64>{});
  } else {
    return fail(XP_EINVAL, "prefill attention: dtype %d", dtype);
  }
  XP_CHECK_LAUNCH();
  return XP_OK;
}

}  // namespace

xp_status launch_prefill(int dtype, const void* q, const void* pool, int n_pages, int S, const int32_t* pre_pages,
                         int pre_max_blocks, int hq, int hkv, int d, int prior, int chunk, int off, int n_local,
                         void* out_local, int out_local_stride, void* out_peer, int out_peer_stride, void* ws,
                         uint32_t* status, int cus, hipStream_t s, bool cores) {
  if (chunk == 0) return XP_OK;
  const PrefillJob j{q, pre_pages, pre_max_blocks, prior, chunk, off, n_local, out_local, out_local_stride, out_peer,
                     out_peer_stride, ws};
  Prepared pr;
  xp_status st = prepare(pool, n_pages, S, hq, hkv, d, j, status, cus, pr);
  if (st) return st;
  return dispatch(dtype, d, [&](auto t, auto dd) { launch_one<decltype(t), decltype(dd)::value>(pr, cores, s); });
}

xp_status launch_prefill_group(int dtype, const void* pool, int n_pages, int S, int hq, int hkv, int d, int n,
                               const PrefillJob* jobs, uint32_t* status, int cus, hipStream_t s, bool cores) {
  std::vector<Prepared> pr;
  for (int k = 0; k < n; ++k) {
    if (jobs[k].chunk == 0) continue;
    Prepared one;
    xp_status st = prepare(pool, n_pages, S, hq, hkv, d, jobs[k], status, cus, one);
    if (st) return st;
    pr.push_back(one);
  }
  // the longest key ranges first, so their tiles start before the short ones
  std::stable_sort(pr.begin(), pr.end(), [](const Prepared& x, const Prepared& y) {
    return x.a.prior + x.a.chunk > y.a.prior + y.a.chunk;
  });
  for (size_t k0 = 0; k0 < pr.size(); k0 += kMaxGroup) {
    const int m = int(std::min<size_t>(kMaxGroup, pr.size() - k0));
    xp_status st = m == 1 ? dispatch(dtype, d, [&](auto t, auto dd) {
                              launch_one<decltype(t), decltype(dd)::value>(pr[k0], cores, s);
                            })
                          : dispatch(dtype, d, [&](auto t, auto dd) {
                              launch_group<decltype(t), decltype(dd)::value>(pr.data() + k0, m, cores, s);
                            });
    if (st) return st;
  }
  return XP_OK;
}

}  // namespace xp
