// Causal chunked-prefill attention on one SP rank's head subset, over the
// cached prior keys plus the chunk (ConfluxServe §4 and App. A: with Ulysses SP
// each rank computes complete attention for the heads it owns over the whole
// chunk, and later chunks reuse the head-sharded history; the mask is the
// inclusive causal mask of Adaptive Context Parallelism §2.1).  All keys are
// read from the paged pool: the chunk's own K/V were appended before.
//
// Work decomposition: a workgroup owns one KV head g, one 32-query tile and one
// split of the tile's key range (`bps` 32-key blocks), with one wave per query
// head of g's GQA group (up to 8), so each K/V block is read from HBM once for
// the whole group.  Blocks (two pages: 8 KB of K rows + 8 KB of V^T rows for
// d = 128) are copied straight into a 3-stage LDS ring with buffer_load ... lds;
// K rows are stored with their 16-byte chunks XOR-swizzled by (key & 15) so the
// eight keys an LDS read serves together hit different banks.  Splitting the key
// range gives long prior contexts enough workgroups; a tile whose keys fit in one
// split writes its output directly, the others write fp32 (max, sum, output)
// partials that `prefill_combine_kernel` merges (the log-sum-exp merge of Decode
// Token Parallelism Eq. 4).
//
// Per wave and block, 32x32 MFMA tiles:
//   S^T[32 keys x 32 queries] = K[32 x d] . Q^T[d x 32]      (16-deep k steps)
//   O^T[d x 32 queries]     += V^T[d x 32 keys] . P^T        (16-deep k steps)
// Queries are the MFMA columns, so lane l owns query l % 32 for both the scores
// and the output: the row max needs one exchange with lane l ^ 32 and the
// rescale is per lane.  Row i of the K operand holds key kappa(i) of the block
// (bits 2 and 3 of i swapped), which makes accumulator elements 0..7 of lane l
// the keys 8*(l/32) .. +7 of the first page and elements 8..15 the same slots of
// the second page -- exactly the k-slots the PV step's P operand supplies, and
// the V^T operand is then 8 consecutive slots of one dim row (16 bytes for bf16).
#include "gemm_core.h"
#include "xp_device.h"
#include "xp_internal.h"

namespace xp {

namespace {

constexpr int kPage = 16;
constexpr int kMaxWaves = 8;
constexpr int kStages = 3;
constexpr int kMaxBps = 256;   // key blocks per split (its page ids are staged in LDS)

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

// K rows are stored with 16-byte chunk c of key k at position c ^ (k & (chunks - 1)).
template <int KROW_CH>
__device__ __forceinline__ const uint4* kchunk(const char* plane, int k, int c, int row_bytes) {
  return reinterpret_cast<const uint4*>(plane + k * row_bytes + ((c ^ (k & (KROW_CH - 1))) & (KROW_CH - 1)) * 16);
}
template <int KROW_CH>
__device__ __forceinline__ void kfrag(Frag8<bf16_t>& f, const char* plane, int k, int elem0, int row_bytes) {
  f.v = *kchunk<KROW_CH>(plane, k, elem0 * 2 / 16, row_bytes);
}
template <int KROW_CH>
__device__ __forceinline__ void kfrag(Frag8<float>& f, const char* plane, int k, int elem0, int row_bytes) {
  const int c = elem0 * 4 / 16;
  f.lo = __builtin_bit_cast(float4, *kchunk<KROW_CH>(plane, k, c, row_bytes));
  f.hi = __builtin_bit_cast(float4, *kchunk<KROW_CH>(plane, k, c + 1, row_bytes));
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
  float* part_ml; // [n_qt, hq, n_split, 32, 2]
  float* part_o;  // [n_qt, hq, n_split, 32, D]
};

__device__ __forceinline__ void wait_vm_upto16(int n) {
  switch (n) {
    case 0: gemm::wait_vmcnt<0>(); break;
    case 1: gemm::wait_vmcnt<1>(); break;
    case 2: gemm::wait_vmcnt<2>(); break;
    case 3: gemm::wait_vmcnt<3>(); break;
    case 4: gemm::wait_vmcnt<4>(); break;
    case 5: gemm::wait_vmcnt<5>(); break;
    case 6: gemm::wait_vmcnt<6>(); break;
    case 7: gemm::wait_vmcnt<7>(); break;
    default: gemm::wait_vmcnt<8>(); break;
  }
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

template <typename T, int D>
__global__ __launch_bounds__(64 * kMaxWaves) void prefill_kernel(PrefillArgs a) {
  constexpr int EB = St<T>::bytes;
  constexpr int PLANE = kPage * D * EB;           // bytes of one K or V plane of a page
  constexpr long PAGE_BYTES = 2L * PLANE;
  constexpr int STAGE = 4 * PLANE;                // K_A | K_B | V_A | V_B
  constexpr int CH_PER_PLANE = PLANE / 16;        // 16-byte chunks per plane
  constexpr int INSTR = 4 * CH_PER_PLANE / 64;    // 64-lane load instructions per stage
  constexpr int KROW_CH = D * EB / 16;            // 16-byte chunks per K row
  constexpr int VROW_B = kPage * EB;              // bytes per V^T row of a page
  __shared__ uint4 ring[kStages][STAGE / 16];
  __shared__ int32_t pids[2 * kMaxBps];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.hq / a.hkv;
  const int n_qt = (a.chunk + 31) / 32;
  const int qt = n_qt - 1 - int(blockIdx.x) / a.n_split;   // longest tiles first
  const int s = int(blockIdx.x) % a.n_split;
  const int groups_per_kv = (G + a.wpg - 1) / a.wpg;
  const int g = int(blockIdx.y) / groups_per_kv;
  const int h0 = g * G + (int(blockIdx.y) % groups_per_kv) * a.wpg;   // first query head of this workgroup
  const int waves = min(a.wpg, g * G + G - h0);
  const int t0 = qt * 32;
  const int q_last = min(t0 + 31, a.chunk - 1);
  const int n_keys = a.prior + a.chunk;                     // keys in the table
  const int nkb = (a.prior + q_last + 1 + 31) / 32;         // key blocks this tile needs
  const int kb0 = s * a.bps;
  if (kb0 >= nkb) return;                                   // uniform over the workgroup
  const int kb1 = min(nkb, kb0 + a.bps);
  const int ns = (nkb + a.bps - 1) / a.bps;
  const bool active = wave < waves;
  const int h = h0 + (active ? wave : 0);
  const int32_t* tbl = a.pre_pages + long(g) * a.pre_max_blocks;

  // The split's page ids, staged once: table reads inside the pipeline would be vector
  // loads, and waiting for one of them would also wait for every ring load before it.
  const int n_tbl = (n_keys + kPage - 1) / kPage;
  for (int i = int(threadIdx.x); i < 2 * (kb1 - kb0); i += int(blockDim.x)) {
    const int b = 2 * kb0 + i;
    pids[i] = b < n_tbl ? tbl[b] : -1;
  }
  __syncthreads();

  // my load instructions per stage: i = wave, wave + waves, ...
  const int my_instr = wave < waves ? (INSTR - wave + waves - 1) / waves : 0;
  bool bad = false;
  auto issue = [&](int kb, int buf) {
    if (wave >= waves) return;
    const int key0 = kb * 32;
    const int pa = __builtin_amdgcn_readfirstlane(pids[2 * (kb - kb0)]);
    const bool has_b = key0 + kPage < n_keys;
    const int pb = has_b ? __builtin_amdgcn_readfirstlane(pids[2 * (kb - kb0) + 1]) : -1;
    const bool ok_a = pa >= 0 && pa < a.n_pages;
    const bool ok_b = pb >= 0 && pb < a.n_pages;
    if (!ok_a || (has_b && !ok_b)) bad = true;
    const gemm::i32x4 ra = gemm::rsrc_rows(a.pool + (ok_a ? long(pa) : 0L) * PAGE_BYTES, ok_a ? 1 : 0, PAGE_BYTES);
    const gemm::i32x4 rb = gemm::rsrc_rows(a.pool + (ok_b ? long(pb) : 0L) * PAGE_BYTES, ok_b ? 1 : 0, PAGE_BYTES);
    for (int i = wave; i < INSTR; i += waves) {
      const int region = i / (CH_PER_PLANE / 64);         // 0 K_A, 1 K_B, 2 V_A, 3 V_B
      const int p = (i % (CH_PER_PLANE / 64)) * 64 + lane;  // chunk position inside the plane
      int src;
      if (region < 2) {
        const int row = p / KROW_CH, c = (p % KROW_CH) ^ (row & (KROW_CH - 1));
        src = row * (D * EB) + c * 16;
      } else {
        src = PLANE + p * 16;
      }
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          uint32_t(reinterpret_cast<uintptr_t>(&ring[buf][region * CH_PER_PLANE + (i % (CH_PER_PLANE / 64)) * 64])));
      gemm::load_lds16((region & 1) ? rb : ra, dst, src);
    }
  };

  const int ql = lane & 31, hf = lane >> 5;
  const int t = t0 + ql;
  const bool qvalid = t < a.chunk;
  const int qpos = a.prior + min(t, a.chunk - 1);

  Frag8<T> qf[D / 16];
  const char* qrow = static_cast<const char*>(a.q) + (long(h) * a.chunk + min(t, a.chunk - 1)) * D * EB;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) load_frag8(qf[st], qrow + (16 * st + 8 * hf) * EB);
  // Settle these loads before any ring load is issued: the compiler waits for them at
  // their first use inside the loop, and with in-order completion such a wait would
  // also drain the ring stages in flight.
  gemm::wait_vmcnt<0>();

  f32x16 o[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) o[n] = f32x16{};
  float m = -__builtin_inff(), lsum = 0.f;

  issue(kb0, 0);
  if (kb0 + 1 < kb1) issue(kb0 + 1, 1);
  const int krow = kappa(ql);
  for (int kb = kb0; kb < kb1; ++kb) {
    const int it = kb - kb0;
    if (kb + 1 < kb1) wait_vm_upto16(my_instr);
    else gemm::wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kb + 2 < kb1) issue(kb + 2, (it + 2) % kStages);
    if (!active) continue;
    const char* st_base = reinterpret_cast<const char*>(ring[it % kStages]);
    const int key0 = kb * 32;
    // S^T = K . Q^T; K operand row ql holds key kappa(ql) of the block
    const char* kplane = st_base + (krow < kPage ? 0 : PLANE);
    const int kr = krow & 15;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      Frag8<T> kf;
      kfrag<KROW_CH>(kf, kplane, kr, 16 * st + 8 * hf, D * EB);
      mma32x32_k16(sacc, kf, qf[st]);
    }
    // element r: key key0 + 16*(r/8) + 8*hf + r%8
    float sv[16];
    float mb = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kpos = key0 + 16 * (r >> 3) + 8 * hf + (r & 7);
      sv[r] = (kpos <= qpos) ? sacc[r] * a.scale_log2 : -__builtin_inff();
      mb = fmaxf(mb, sv[r]);
    }
    mb = fmaxf(mb, shfl_xor(mb, 32));
    const float mn = fmaxf(m, mb);
    const float mref = (mn == -__builtin_inff()) ? 0.f : mn;
    const float alpha = fast_exp2(m - mref);
    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = round_st<T>(fast_exp2(sv[r] - mref));
      ps += p[r];
    }
    lsum = lsum * alpha + ps;
    m = mn;
#pragma unroll
    for (int n = 0; n < D / 32; ++n) o[n] *= alpha;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      Frag8<T> pf;
      set_frag8(pf, &p[8 * u]);
      const char* vplane = st_base + (2 + u) * PLANE;
      const int nvalid = n_keys - (key0 + 16 * u + 8 * hf);   // slots at or past the table end hold no key
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        Frag8<T> vf;
        load_frag8(vf, vplane + (32 * n + ql) * VROW_B + 8 * hf * EB);
        if (nvalid < 8) zero_from(vf, nvalid);
        mma32x32_k16(o[n], vf, pf);
      }
    }
  }
  if (bad && a.status && lane == 0 && wave == 0) atomicOr(a.status, XP_DEV_BAD_PAGE);
  if (!active) return;
  lsum += shfl_xor(lsum, 32);
  if (ns == 1) {
    if (!qvalid) return;
    const float inv = bad ? __builtin_nanf("") : 1.0f / lsum;
    void* dst;
    long row_off;
    out_row(a, t, dst, row_off);
    const long base = row_off + long(h) * D;
    // element r of o[n]: dim 32*n + 8*(r/4) + 4*hf + r%4
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) St<T>::store(dst, base + 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3), o[n][r] * inv);
    return;
  }
  const long unit = ((long(qt) * a.hq + h) * a.n_split + s) * 32 + ql;
  if (hf == 0) {
    a.part_ml[2 * unit] = bad ? __builtin_nanf("") : m;
    a.part_ml[2 * unit + 1] = lsum;
  }
  float* po = a.part_o + unit * D;
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<float4*>(po + 32 * n + 8 * r4 + 4 * hf) =
          make_float4(o[n][4 * r4], o[n][4 * r4 + 1], o[n][4 * r4 + 2], o[n][4 * r4 + 3]);
}

// merges the split partials of the tiles that were split (scores in the exp2 domain):
// the split weights of each query are formed once, then every thread sums float4
// slices of the partial outputs with independent loads.
constexpr int kMaxSplits = 64;

template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
  __shared__ float wts[kMaxSplits][32];
  const int qt = blockIdx.x, h = blockIdx.y;
  const int q_last = min(qt * 32 + 31, a.chunk - 1);
  const int nkb = (a.prior + q_last + 1 + 31) / 32;
  const int ns = (nkb + a.bps - 1) / a.bps;
  if (ns <= 1) return;
  const long u0 = ((long(qt) * a.hq + h) * a.n_split) * 32;   // unit of (split 0, query 0)
  if (threadIdx.x < 32) {
    const int ql = threadIdx.x;
    float mx = -__builtin_inff();
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.part_ml[2 * (u0 + s * 32 + ql)]);
    float L = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float w = fast_exp2(a.part_ml[2 * (u0 + s * 32 + ql)] - mx);
      wts[s][ql] = w;
      L += a.part_ml[2 * (u0 + s * 32 + ql) + 1] * w;
    }
    const float inv = 1.0f / L;
    for (int s = 0; s < ns; ++s) wts[s][ql] *= inv;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 32 * (D / 4); e += 256) {
    const int ql = e / (D / 4), j4 = e % (D / 4);
    const int t = qt * 32 + ql;
    if (t >= a.chunk) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < ns; ++s) {
      const float4 v = reinterpret_cast<const float4*>(a.part_o + (u0 + s * 32 + ql) * D)[j4];
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

struct Plan {
  int bps, n_split, wpg;
};

Plan plan(int hq, int hkv, int prior, int chunk) {
  const int G = hq / hkv;
  const int n_qt = (chunk + 31) / 32;
  const int max_nkb = (prior + chunk + 31) / 32;
  long total = 0;  // key blocks over all tiles
  for (int qt = 0; qt < n_qt; ++qt) total += (prior + std::min(qt * 32 + 31, chunk - 1) + 1 + 31) / 32;
  const int wpg = std::min(G, kMaxWaves);
  const long wgs_per_tile = long(hkv) * ((G + wpg - 1) / wpg);
  // aim at about two waves per SIMD over the whole launch (more splits cost fp32 partial
  // traffic), splits of >= 8 blocks
  const long target = std::max<long>(1, 2048 / wpg);
  long bps = (total * wgs_per_tile + target - 1) / target;
  bps = std::max<long>(8, bps);
  bps = std::min<long>(bps, max_nkb);
  bps = std::min<long>(bps, kMaxBps);
  int n_split = int((max_nkb + bps - 1) / bps);
  if (n_split > kMaxSplits) {
    bps = (max_nkb + kMaxSplits - 1) / kMaxSplits;
    n_split = int((max_nkb + bps - 1) / bps);
  }
  return {int(bps), n_split, wpg};
}

}  // namespace

size_t prefill_ws_bytes(int hq, int hkv, int d, int prior, int chunk) {
  if (chunk <= 0) return 0;
  const Plan p = plan(hq, hkv, prior, chunk);
  if (p.n_split <= 1) return 0;
  const size_t units = size_t((chunk + 31) / 32) * hq * p.n_split * 32;
  return align_up(units * 2 * sizeof(float), 256) + align_up(units * d * sizeof(float), 256);
}

xp_status launch_prefill(int dtype, const void* q, const void* pool, int n_pages, int S, const int32_t* pre_pages,
                         int pre_max_blocks, int hq, int hkv, int d, int prior, int chunk, int off, int n_local,
                         void* out_local, int out_local_stride, void* out_peer, int out_peer_stride, void* ws,
                         uint32_t* status, hipStream_t s) {
  if (chunk == 0) return XP_OK;
  if (S != kPage) return fail(XP_EUNSUPPORTED, "prefill attention: page_size %d (supported: 16)", S);
  if (hkv <= 0 || hq % hkv) return fail(XP_ESHAPE, "prefill attention: hq=%d hkv=%d", hq, hkv);
  if (long(pre_max_blocks) * kPage < long(prior) + chunk)
    return fail(XP_EPAGE, "prefill attention: table of %d blocks < %d keys", pre_max_blocks, prior + chunk);
  if (off < 0 || n_local < 0 || off + n_local > chunk) return fail(XP_ESHAPE, "prefill attention: off/n_local");
  if ((long(prior) + chunk + 31) / 32 > long(kMaxBps) * kMaxSplits)
    return fail(XP_EUNSUPPORTED, "prefill attention: %d keys exceed %d", prior + chunk, 32 * kMaxBps * kMaxSplits);
  const Plan p = plan(hq, hkv, prior, chunk);
  const size_t need = prefill_ws_bytes(hq, hkv, d, prior, chunk);
  if (need && !ws) return fail(XP_EWORKSPACE, "prefill attention: needs %zu bytes of workspace", need);
  const size_t units = size_t((chunk + 31) / 32) * hq * p.n_split * 32;
  float* ml = static_cast<float*>(ws);
  float* po = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(units * 2 * sizeof(float), 256)) : nullptr;
  PrefillArgs a{q, static_cast<const char*>(pool), n_pages, pre_pages, pre_max_blocks, hq, hkv, prior, chunk, off,
                n_local, out_local, out_local_stride, out_peer, out_peer_stride,
                float(1.4426950408889634 / __builtin_sqrt(double(d))), status, p.bps, p.n_split, p.wpg, ml, po};
  const int n_qt = (chunk + 31) / 32;
  const int G = hq / hkv;
  const dim3 grid(n_qt * p.n_split, hkv * ((G + p.wpg - 1) / p.wpg));
  const dim3 block(64 * p.wpg);
  const dim3 cgrid(n_qt, hq);
  if (dtype == XP_BF16) {
    if (d == 128) {
      hipLaunchKernelGGL((prefill_kernel<bf16_t, 128>), grid, block, 0, s, a);
      if (p.n_split > 1) hipLaunchKernelGGL((prefill_combine_kernel<bf16_t, 128>), cgrid, dim3(256), 0, s, a);
    } else if (d == 64) {
      hipLaunchKernelGGL((prefill_kernel<bf16_t, 64>), grid, block, 0, s, a);
      if (p.n_split > 1) hipLaunchKernelGGL((prefill_combine_kernel<bf16_t, 64>), cgrid, dim3(256), 0, s, a);
    } else {
      return fail(XP_EUNSUPPORTED, "prefill attention: head_dim %d", d);
    }
  } else if (dtype == XP_F32) {
    if (d == 128) {
      hipLaunchKernelGGL((prefill_kernel<float, 128>), grid, block, 0, s, a);
      if (p.n_split > 1) hipLaunchKernelGGL((prefill_combine_kernel<float, 128>), cgrid, dim3(256), 0, s, a);
    } else if (d == 64) {
      hipLaunchKernelGGL((prefill_kernel<float, 64>), grid, block, 0, s, a);
      if (p.n_split > 1) hipLaunchKernelGGL((prefill_combine_kernel<float, 64>), cgrid, dim3(256), 0, s, a);
    } else {
      return fail(XP_EUNSUPPORTED, "prefill attention: head_dim %d", d);
    }
  } else {
    return fail(XP_EINVAL, "prefill attention: dtype %d", dtype);
  }
  XP_CHECK_LAUNCH();
  return XP_OK;
}

}  // namespace xp
