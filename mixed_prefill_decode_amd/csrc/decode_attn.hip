// Paged GQA decode attention, split-K over the context, with an fp32
// log-sum-exp merge of the partials.
//
// ConfluxServe §4: decode attention stays rank-local and each request reads
// only its own KV, so the step is bound by HBM bandwidth (App. B, Table 7:
// its arithmetic intensity does not grow with batch).  The merge of partial
// results uses the (output, fp32 log-sum-exp) partial form of Decode Token
// Parallelism Eq. 4.
//
// One wave handles one (request, KV head, split) and reads each page of the
// split exactly once for all G query heads of the group:
//   S^T[16 keys x 16 heads] = K_page[16 x d] . Q^T[d x 16]   (16x16 MFMA, 32-deep k)
//   O^T[d x 16 heads]     += V^T_page[d x 16 keys] . P^T     (16x16 MFMA, 16-deep k)
// Query heads are the MFMA columns (G <= 16, unused columns are zero), so lane
// l owns head l % 16 for both the scores and the output, and the online-softmax
// rescale needs no cross-lane traffic beyond the 16-key max.  The V plane of a
// page is stored dim-major, so the V^T operand of lane l is 4 consecutive keys
// of one dim row (8 contiguous bytes for bf16).  Scores are kept in the exp2
// domain (scale * log2(e) folded in).  Each wave keeps a few pages of K/V
// fragments in flight ahead of the page it consumes.
#include <mutex>

#include "xp_device.h"
#include "xp_internal.h"

namespace xp {

namespace {

constexpr int kPage = 16;
// pages in flight per wave while one is consumed
constexpr int kDepth = 1;
// Cache policy of the page loads: non-temporal (the buffer instructions' nt bit).
// Every K/V byte is read once per step, so keeping it out of the caches' recency
// costs nothing; measured on MI355X it raises the decode stream from 5.16 to 5.79
// TB/s on the 8B batch (6.03 on the 32K-context one) and shortens the 8B layer step
// by 4%, the following GEMMs finding more of their operands cached.
constexpr int kLoadAux = 2;
// log2-domain margin by which a head's maximum may exceed the softmax reference
// before O and l are rescaled
constexpr float kLazy = 8.0f;

// Packs 4 weights into a PV operand fragment (rounding them to the operand type)
// and returns the sum of the rounded weights.
__device__ __forceinline__ float pack4_and_sum(Frag4<bf16_t>& f, const float* p) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  set_frag4(f, p[0], p[1], p[2], p[3]);
  const bf16x2 one2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  const float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, f.v.x), one2, 0.f, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, f.v.y), one2, s, false);
}
__device__ __forceinline__ float pack4_and_sum(Frag4<float>& f, const float* p) {
  set_frag4(f, p[0], p[1], p[2], p[3]);
  return (p[0] + p[1]) + (p[2] + p[3]);
}

__device__ __forceinline__ void zero_tail(Frag4<bf16_t>& f, int nvalid) {
  uint32_t x = f.v.x, y = f.v.y;
  if (nvalid <= 0) x = 0;
  else if (nvalid == 1) x &= 0xffffu;
  if (nvalid <= 2) y = 0;
  else if (nvalid == 3) y &= 0xffffu;
  f.v = make_uint2(x, y);
}
__device__ __forceinline__ void zero_tail(Frag4<float>& f, int nvalid) {
  if (nvalid <= 0) f.v.x = 0.f;
  if (nvalid <= 1) f.v.y = 0.f;
  if (nvalid <= 2) f.v.z = 0.f;
  if (nvalid <= 3) f.v.w = 0.f;
}

template <typename T, int D>
struct PageFrags {
  Frag8<T> k[D / 32];
  Frag4<T> v[D / 16];
};

// Buffer resource over one page: a page outside the split or with an id
// outside the pool gets zero records, so its loads return zeros and touch no
// memory.  The loads of the pipeline are therefore unconditional.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* page, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(page), (short)0, nbytes, 0x00020000);
}

__device__ __forceinline__ void bload(Frag4<bf16_t>& f, __amdgpu_buffer_rsrc_t r, int off) {
  f.v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadAux));
}
__device__ __forceinline__ void bload(Frag4<float>& f, __amdgpu_buffer_rsrc_t r, int off) {
  f.v = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadAux));
}

// byte offset of slot `key`, dim j inside a page's K plane (chunk-major, k_elem)
template <typename T>
__device__ __forceinline__ int k_byte(int key, int j) {
  return int(k_elem<T>(key, j, kPage)) * St<T>::bytes;
}

// K fragment of one key: dims [j0, j0 + 8) (one 16-byte chunk for bf16, two for fp32)
__device__ __forceinline__ void bload_k(Frag8<bf16_t>& f, __amdgpu_buffer_rsrc_t r, int key, int j0) {
  f.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, k_byte<bf16_t>(key, j0), 0, kLoadAux));
}
__device__ __forceinline__ void bload_k(Frag8<float>& f, __amdgpu_buffer_rsrc_t r, int key, int j0) {
  f.lo = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, k_byte<float>(key, j0), 0, kLoadAux));
  f.hi = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, k_byte<float>(key, j0 + 4), 0, kLoadAux));
}

// K plane chunk-major (k_elem): lane l reads key l%16, dims [32*st + 8*(l/16), +8); for
// bf16 the 64 lanes of fragment st read the plane's bytes [1024 st, 1024 (st + 1))
// in lane order, one contiguous run per load instruction.
// V plane dim-major [D][16]: lane l reads dim 16*n + l%16, keys [4*(l/16), +4).
template <typename T, int D>
__device__ __forceinline__ void load_page(PageFrags<T, D>& f, __amdgpu_buffer_rsrc_t r, int lane) {
  constexpr int EB = St<T>::bytes;
  const int key = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int st = 0; st < D / 32; ++st) bload_k(f.k[st], r, key, 32 * st + 8 * grp);
#pragma unroll
  for (int n = 0; n < D / 16; ++n) bload(f.v[n], r, (kPage * D + (16 * n + key) * kPage + 4 * grp) * EB);
}

// One unit of work: split s of request i's context on KV head g.  DEPTH pages
// are in flight while one is consumed; the register ring has DEPTH + 1 page
// buffers and the loop is unrolled over the ring so every buffer index is static.
template <typename T, int D, int DEPTH>
__device__ __forceinline__ void decode_unit(const void* __restrict__ q, const char* __restrict__ pool, int n_pages,
                                            const int32_t* __restrict__ dec_pages, int max_blocks,
                                            const int32_t* __restrict__ dec_ctx, int Hq, int Hkv, int pps,
                                            int n_splits, float* __restrict__ part_ml, float* __restrict__ part_o,
                                            float scale_log2, uint32_t* __restrict__ status, int i, int g, int s) {
  constexpr int EB = St<T>::bytes;
  constexpr int PAGE_BYTES = 2 * kPage * D * EB;
  constexpr int NB = DEPTH + 1;
  const int lane = threadIdx.x & 63;
  const int G = Hq / Hkv;
  const int b0 = s * pps;
  // the table slice is read before anything that depends on the context length
  const int32_t* tbl = dec_pages + (long(i) * Hkv + g) * max_blocks;
  const int my_pid = (lane < pps && b0 + lane < max_blocks) ? tbl[b0 + lane] : -1;
  const int hh = lane & 15, grp = lane >> 4;
  Frag8<T> qf[D / 32];
#pragma unroll
  for (int st = 0; st < D / 32; ++st) {
    if (hh < G) {
      load_frag8(qf[st], static_cast<const char*>(q) + ((long(i) * Hq + g * G + hh) * D + 32 * st + 8 * grp) * EB);
    } else {
      zero_frag(qf[st]);
    }
  }
  const int n_keys = dec_ctx[i] + 1;
  const int nb_need = (n_keys + kPage - 1) / kPage;
  const int nb = min(nb_need, max_blocks);
  if (b0 >= nb_need && !(s == 0 && n_keys <= 0)) return;  // this split has no keys
  const int b1 = min(nb, b0 + pps);
  bool bad = nb_need > max_blocks || n_keys <= 0;

  auto rsrc_of = [&](int b) {
    const bool in = b < b1;
    const int pid = __builtin_amdgcn_readlane(my_pid, in ? b - b0 : 0);
    const bool ok = in && pid >= 0 && pid < n_pages;
    bad |= in && !ok;
    return page_rsrc(pool + (ok ? long(pid) : 0L) * PAGE_BYTES, ok ? PAGE_BYTES : 0);
  };

  f32x4 o[D / 16];
#pragma unroll
  for (int n = 0; n < D / 16; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), lsum = 0.f;

  PageFrags<T, D> buf[NB];
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) {
    load_page<T, D>(buf[j], rsrc_of(b0 + j), lane);
    // keep the pages' loads in issue order: the waits below count on it
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int bb = b0; bb < b1; bb += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int b = bb + u;
      load_page<T, D>(buf[(u + DEPTH) % NB], rsrc_of(b + DEPTH), lane);
      __builtin_amdgcn_sched_barrier(0);
      if (b < b1) {
        PageFrags<T, D>& cur = buf[u];
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < D / 32; ++st) mma16x16_k32(sacc, cur.k[st], qf[st]);
        // element r: key b*16 + 4*grp + r of head hh; only the context's last page
        // has slots past the newest key (their V^T columns may hold anything)
        float sv[4] = {sacc[0], sacc[1], sacc[2], sacc[3]};
        if ((b + 1) * kPage > n_keys) {
          const int k0 = b * kPage + 4 * grp;
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[r] = (k0 + r < n_keys) ? sv[r] : -__builtin_inff();
#pragma unroll
          for (int n = 0; n < D / 16; ++n) zero_tail(cur.v[n], n_keys - k0);
        }
        float mb = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        float x0, x1;
        halves_xor16(mb, x0, x1);                         // register lane swaps, not the LDS queue
        halves_xor32(fmaxf(x0, x1), x0, x1);
        mb = fmaxf(x0, x1) * scale_log2;                  // finite: every visited page holds a key
        // Lazily moved softmax reference (exp2 domain): O and l are rescaled only when
        // some head's maximum exceeds the reference by more than kLazy, so the
        // weights stay below 2^kLazy; the result is the same function of the scores.
        if (__builtin_amdgcn_ballot_w64(mb > m + kLazy) != 0) {
          const float mn = fmaxf(m, mb);
          const float alpha = m == -__builtin_inff() ? 0.f : fast_exp2(m - mn);
          m = mn;
          lsum *= alpha;
#pragma unroll
          for (int n = 0; n < D / 16; ++n) o[n] *= alpha;
        }
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = fast_exp2(__builtin_fmaf(sv[r], scale_log2, -m));
        // the weights are rounded to the operand type first, so the normaliser sums
        // exactly the weights the PV product uses
        Frag4<T> pf;
        lsum += pack4_and_sum(pf, p);
#pragma unroll
        for (int n = 0; n < D / 16; ++n) mma16x16_k16(o[n], cur.v[n], pf);
      }
    }
  }
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  if (bad && status && lane == 0) atomicOr(status, XP_DEV_BAD_PAGE);
  if (hh < G) {
    const long base = (long(i) * Hq + g * G + hh) * n_splits + s;
    if (grp == 0) {
      part_ml[2 * base] = bad ? __builtin_nanf("") : m;
      part_ml[2 * base + 1] = lsum;
    }
    float* po = part_o + base * D;
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) po[16 * n + 4 * grp + r] = o[n][r];
  }
}

// The split waves of a batch as one compact list: unit u enumerates (request i,
// split s, KV head g) with i slowest and g fastest, over only the splits that hold
// keys (a request of nb pages has ceil(nb / pps) of them), and workgroup w takes
// units w, w + W, w + 2W, ... of the W workgroups launched.  Short requests then
// cost nothing and the splits of long ones spread over the whole grid; the
// partials keep their (i, h, s) layout for the combine.
// A workgroup holds one wave (its own unit list position) or, in the co-resident form,
// four independent waves: wave w of workgroup b then takes list position 4 b + w.
template <typename T, int D, int DEPTH>
__device__ __forceinline__ void decode_units(const void* __restrict__ q, const char* __restrict__ pool, int n_pages,
                                             const int32_t* __restrict__ dec_pages, int max_blocks,
                                             const int32_t* __restrict__ dec_ctx, int n_d, int Hq, int Hkv, int pps,
                                             int n_splits, float* __restrict__ part_ml, float* __restrict__ part_o,
                                             float scale_log2, uint32_t* __restrict__ status) {
  const int wpb = int(blockDim.x) >> 6;
  const int W = int(gridDim.x) * wpb;
  int u = int(blockIdx.x) * wpb + __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  int base = 0;
  for (int i = 0; i < n_d; ++i) {
    const int nb_need = (dec_ctx[i] + kPage) / kPage;               // pages of ctx + 1 keys
    const int ns = max(1, min(n_splits, (nb_need + pps - 1) / pps));
    const int cnt = ns * Hkv;
    for (; u < base + cnt; u += W) {
      const int r = u - base;
      decode_unit<T, D, DEPTH>(q, pool, n_pages, dec_pages, max_blocks, dec_ctx, Hq, Hkv, pps, n_splits,
                                    part_ml, part_o, scale_log2, status, i, r % Hkv, r / Hkv);
    }
    base += cnt;
  }
}

template <typename T, int D, int DEPTH>
__global__ __launch_bounds__(64) void decode_split_kernel(const void* __restrict__ q, const char* __restrict__ pool,
                                                          int n_pages, const int32_t* __restrict__ dec_pages,
                                                          int max_blocks, const int32_t* __restrict__ dec_ctx, int n_d,
                                                          int Hq, int Hkv, int pps, int n_splits,
                                                          float* __restrict__ part_ml, float* __restrict__ part_o,
                                                          float scale_log2, uint32_t* __restrict__ status) {
  decode_units<T, D, DEPTH>(q, pool, n_pages, dec_pages, max_blocks, dec_ctx, n_d, Hq, Hkv, pps, n_splits,
                                 part_ml, part_o, scale_log2, status);
}

// The co-resident form, for decode running beside prefill attention on the same CUs:
// four-wave workgroups of at most 168 registers per wave (three waves per SIMD), each
// launched with kCoresLds bytes of LDS it does not use, so that a CU holds at most one
// of them (four decode waves, one per SIMD) next to one prefill workgroup (two waves
// per SIMD of at most 168 registers, 68 KB of LDS).  The units and their arithmetic are
// those of decode_split_kernel: the results are the same bits.
constexpr int kCoresWaves = 4;
constexpr size_t kCoresLds = 84 * 1024;
template <typename T, int D, int DEPTH>
__global__ __launch_bounds__(64 * kCoresWaves) __attribute__((amdgpu_waves_per_eu(3))) void decode_split_cores_kernel(
    const void* __restrict__ q, const char* __restrict__ pool, int n_pages, const int32_t* __restrict__ dec_pages,
    int max_blocks, const int32_t* __restrict__ dec_ctx, int n_d, int Hq, int Hkv, int pps, int n_splits,
    float* __restrict__ part_ml, float* __restrict__ part_o, float scale_log2, uint32_t* __restrict__ status) {
  decode_units<T, D, DEPTH>(q, pool, n_pages, dec_pages, max_blocks, dec_ctx, n_d, Hq, Hkv, pps, n_splits,
                                 part_ml, part_o, scale_log2, status);
}

// out[i, h*D + j] = sum_s 2^(m_s - m*) o_s[j] / sum_s 2^(m_s - m*) l_s
// One 256-thread workgroup per (query head, request): thread t accumulates dim
// t % D over every (256 / D)-th split with several partial loads in flight,
// and the split groups are summed in LDS at the end.
constexpr int kCombineThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const float* __restrict__ part_ml,
                                                                         const float* __restrict__ part_o,
                                                                         const int32_t* __restrict__ dec_ctx, int Hq,
                                                                         int pps, int n_splits, void* __restrict__ out,
                                                                         int out_stride) {
  constexpr int R = kCombineThreads / D;  // split groups
  __shared__ float red[kCombineThreads / 64];
  __shared__ float acc_s[R][D];
  __shared__ float l_s[R];
  const int h = blockIdx.x, i = blockIdx.y, t = threadIdx.x;
  const int nb = (dec_ctx[i] + 1 + kPage - 1) / kPage;
  const int ns = max(1, min(n_splits, (nb + pps - 1) / pps));
  const float* ml = part_ml + 2L * (long(i) * Hq + h) * n_splits;
  const float* po = part_o + (long(i) * Hq + h) * n_splits * long(D);
  // m* over the splits (a NaN maximum of a flagged split is ignored here and
  // poisons the weights below)
  float mx = -__builtin_inff();
  for (int s = t; s < ns; s += kCombineThreads) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) mx = fmaxf(mx, shfl_xor(mx, w));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < kCombineThreads / 64; ++w) mx = fmaxf(mx, red[w]);
  const int j = t % D, r = t / D;
  float acc = 0.f, L = 0.f;
  constexpr int U = 4;
  int s = r;
  for (; s + (U - 1) * R < ns; s += U * R) {
    float m4[U], l4[U], o4[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      m4[u] = ml[2 * (s + u * R)];
      l4[u] = ml[2 * (s + u * R) + 1];
      o4[u] = po[long(s + u * R) * D + j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = fast_exp2(m4[u] - mx);
      L += l4[u] * w;
      acc += o4[u] * w;
    }
  }
  for (; s < ns; s += R) {
    const float w = fast_exp2(ml[2 * s] - mx);
    L += ml[2 * s + 1] * w;
    acc += po[long(s) * D + j] * w;
  }
  acc_s[r][j] = acc;
  if (j == 0) l_s[r] = L;
  __syncthreads();
  if (r == 0) {
#pragma unroll
    for (int q = 1; q < R; ++q) {
      acc += acc_s[q][j];
      L += l_s[q];
    }
    St<T>::store(out, long(i) * out_stride + long(h) * D + j, acc / L);
  }
}

template <typename T, int D>
xp_status launch_dec_t(const void* q, const void* pool, int n_pages, const int32_t* dec_pages, int max_blocks,
                       const int32_t* dec_ctx, int n_d, int Hq, int Hkv, void* out, int out_stride, float* part_ml,
                       float* part_o, int pps, uint32_t* status, bool cores, hipStream_t s) {
  const int n_splits = decode_splits(max_blocks, pps);
  const float scale_log2 = float(1.4426950408889634 / __builtin_sqrt(double(D)));
  const int waves = decode_grid(n_d, Hkv, n_splits);
  if (cores)
    hipLaunchKernelGGL((decode_split_cores_kernel<T, D, kDepth>), dim3(cdiv(waves, kCoresWaves)),
                       dim3(64 * kCoresWaves), kCoresLds, s, q, static_cast<const char*>(pool), n_pages, dec_pages,
                       max_blocks, dec_ctx, n_d, Hq, Hkv, pps, n_splits, part_ml, part_o, scale_log2, status);
  else
    hipLaunchKernelGGL((decode_split_kernel<T, D, kDepth>), dim3(waves), dim3(64), 0, s, q,
                       static_cast<const char*>(pool), n_pages, dec_pages, max_blocks, dec_ctx, n_d, Hq, Hkv, pps,
                       n_splits, part_ml, part_o, scale_log2, status);
  XP_CHECK_LAUNCH();
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(Hq, n_d), dim3(kCombineThreads), 0, s, part_ml, part_o, dec_ctx, Hq, pps,
                     n_splits, out, out_stride);
  XP_CHECK_LAUNCH();
  return XP_OK;
}

}  // namespace

int decode_splits(int dec_max_blocks, int pps) { return std::max(1, cdiv(dec_max_blocks, pps)); }

// Workgroups of the split kernel.  Up to kGridWaves units (counting every request
// as filling its table) each unit gets a workgroup of its own, so the hardware
// dispatcher balances uniform batches; beyond that the count is the largest one
// that gives every workgroup the same number of units.  Measured on MI355X over the
// 8B, 14B and 32B decode batches: as fast as one workgroup per split for uniform
// contexts, and 1.26x faster for the lognormal 32B batch, whose short requests no
// longer leave most of a table-wide grid empty.
constexpr long kGridWaves = 16384;
int decode_grid(int n_d, int Hkv, int n_splits) {
  const long units = long(n_d) * Hkv * n_splits;   // when every request fills its table
  const long per = (units + kGridWaves - 1) / kGridWaves;
  return int(std::max(1L, (units + per - 1) / per));
}

// Pages per split when the caller leaves it open (0): about kTargetWaves split
// waves over the batch's (request, KV head) pairs at their table width, i.e.
// some six resident waves per CU, and between 8 and 64 pages per wave.  Fewer,
// longer splits write fewer partials; more splits keep more pages in flight.
constexpr long kTargetWaves = 1600;
int decode_pick_pps(int requested, int n_d, int Hkv, int dec_max_blocks) {
  if (requested > 0) return requested;
  const long work = long(n_d) * Hkv * dec_max_blocks;
  return int(std::min(64L, std::max(8L, work / kTargetWaves)));
}

size_t decode_ws_bytes(int n_d, int Hq, int d, int n_splits) {
  const size_t units = size_t(n_d) * Hq * n_splits;
  return align_up(units * 2 * sizeof(float), 256) + align_up(units * d * sizeof(float), 256);
}

xp_status launch_decode(int dtype, const void* q, const void* pool, int n_pages, int S, const int32_t* dec_pages,
                        int dec_max_blocks, const int32_t* dec_ctx, int n_d, int Hq, int Hkv, int d, void* out,
                        int out_stride, float* part_ml, float* part_o, int pps, uint32_t* status, hipStream_t s,
                        bool cores) {
  if (n_d == 0) return XP_OK;
  if (S != kPage) return fail(XP_EUNSUPPORTED, "decode attention: page_size %d (supported: 16)", S);
  if (Hkv <= 0 || Hq % Hkv || Hq / Hkv > 16) return fail(XP_EUNSUPPORTED, "decode attention: Hq=%d Hkv=%d", Hq, Hkv);
  if (pps < 1 || pps > 64) return fail(XP_EINVAL, "decode attention: pages_per_split %d (1..64)", pps);
  if (dec_max_blocks < 1) return fail(XP_ESHAPE, "decode attention: dec_max_blocks %d", dec_max_blocks);
  if (dtype == XP_BF16) {
    if (d == 128) return launch_dec_t<bf16_t, 128>(q, pool, n_pages, dec_pages, dec_max_blocks, dec_ctx, n_d, Hq, Hkv, out, out_stride, part_ml, part_o, pps, status, cores, s);
    if (d == 64) return launch_dec_t<bf16_t, 64>(q, pool, n_pages, dec_pages, dec_max_blocks, dec_ctx, n_d, Hq, Hkv, out, out_stride, part_ml, part_o, pps, status, cores, s);
  } else if (dtype == XP_F32) {
    if (d == 128) return launch_dec_t<float, 128>(q, pool, n_pages, dec_pages, dec_max_blocks, dec_ctx, n_d, Hq, Hkv, out, out_stride, part_ml, part_o, pps, status, cores, s);
    if (d == 64) return launch_dec_t<float, 64>(q, pool, n_pages, dec_pages, dec_max_blocks, dec_ctx, n_d, Hq, Hkv, out, out_stride, part_ml, part_o, pps, status, cores, s);
  }
  return fail(XP_EUNSUPPORTED, "decode attention: dtype %d head_dim %d", dtype, d);
}

}  // namespace xp

namespace xp {

// ---- the entry point that allocates nothing ----------------------------------------
//
// The split partials of xp_decode_attention_static live in this file-scope device
// array, one copy per GPU the library runs on, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in symbol, not a
// device address): the device address of each GPU's copy is looked up once per device,
// with that device current, and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[XP_DECODE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on the device's first call).
xp_status scratch_of_current_device(char** out) {
  int dev = -1;
  XP_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(XP_EUNSUPPORTED, "xp_decode_attention_static: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(XP_EHIP, "xp_decode_attention_static: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return XP_OK;
}
}  // namespace

}  // namespace xp

extern "C" xp_status xp_decode_attention_static(int32_t dtype, const void* q, const void* pool, int32_t n_pages,
                                                int32_t S, const int32_t* dec_pages, int32_t max_blocks,
                                                const int32_t* dec_ctx, int32_t n_d, int32_t Hq, int32_t Hkv,
                                                int32_t d, void* out, int32_t out_stride, int32_t pps,
                                                void* stream) {
  using namespace xp;
  if (n_d < 0) return fail(XP_ESHAPE, "xp_decode_attention_static: n_decode %d", n_d);
  if (n_d == 0) return XP_OK;
  if (!q || !pool || !dec_pages || !dec_ctx || !out) return fail(XP_EINVAL, "xp_decode_attention_static: null pointer");
  if (out_stride < Hq * d) return fail(XP_ESHAPE, "xp_decode_attention_static: out_stride %d < Hq*d", out_stride);
  if (pps < 0) return fail(XP_EINVAL, "xp_decode_attention_static: pages_per_split %d", pps);
  if (Hq <= 0 || Hkv <= 0 || d <= 0 || max_blocks <= 0)
    return fail(XP_ESHAPE, "xp_decode_attention_static: Hq %d Hkv %d d %d max_blocks %d", Hq, Hkv, d, max_blocks);
  pps = decode_pick_pps(pps, n_d, Hkv, max_blocks);
  const int splits = decode_splits(max_blocks, pps);
  const size_t need = decode_ws_bytes(n_d, Hq, d, splits);
  if (need > size_t(XP_DECODE_STATIC_SCRATCH_BYTES))
    return fail(XP_EWORKSPACE, "xp_decode_attention_static: the split partials need %zu bytes, more than the %zu "
                "of its static scratch (use xp_decode_attention with a workspace)", need,
                size_t(XP_DECODE_STATIC_SCRATCH_BYTES));
  char* ws = nullptr;
  xp_status st = scratch_of_current_device(&ws);
  if (st) return st;
  const size_t ml_bytes = align_up(size_t(n_d) * Hq * splits * 2 * sizeof(float), 256);
  return launch_decode(dtype, q, pool, n_pages, S, dec_pages, max_blocks, dec_ctx, n_d, Hq, Hkv, d, out, out_stride,
                       reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws + ml_bytes), pps, nullptr,
                       static_cast<hipStream_t>(stream));
}
