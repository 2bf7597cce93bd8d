// Causal chunked-prefill attention on one SP rank's head subset, over the
// cached prior keys plus the chunk (ConfluxServe §4 and App. A: with Ulysses SP
// each rank computes complete attention for the heads it owns over the whole
// chunk, and later chunks reuse the head-sharded history; the mask is the
// inclusive causal mask of Adaptive Context Parallelism §2.1).  All keys are
// read from the paged pool: the chunk's own K/V were appended before.
//
// One wave owns 32 queries of one head and walks 32-key blocks (two pages):
//   S^T[32 keys x 32 queries] = K[32 x d] . Q^T[d x 32]      (32x32 MFMA, 16-deep k)
//   O^T[d x 32 queries]     += V^T[d x 32 keys] . P^T        (32x32 MFMA, 16-deep k)
// Queries are the MFMA columns, so lane l owns query l % 32 for both the
// scores and the output: the row max needs one exchange with lane l ^ 32 and
// the rescale is per lane.  Row i of the K operand holds key kappa(i) of the
// block (bits 2 and 3 of i swapped), which makes accumulator elements 0..7 of
// lane l the keys 8*(l/32) .. +7 of the first page and elements 8..15 the same
// slots of the second page -- exactly the k-slots the PV step's P operand must
// supply, and the V^T operand is then 8 consecutive slots of one dim row of a
// dim-major V plane (16 contiguous bytes for bf16).
//
// Waves are independent (no LDS, no barriers); a workgroup packs four
// consecutive 32-query tiles of one head, and the workgroups with the most
// keys are dispatched first.
#include "xp_device.h"
#include "xp_internal.h"

namespace xp {

namespace {

constexpr int kPage = 16;

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
};

template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  constexpr int EB = St<T>::bytes;
  constexpr long PAGE_BYTES = 2L * kPage * D * EB;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_qt = (a.chunk + 127) / 128;
  const int qt = n_qt - 1 - int(blockIdx.x);
  const int h = blockIdx.y;
  const int g = h / (a.hq / a.hkv);
  const int t0 = qt * 128 + wave * 32;
  if (t0 >= a.chunk) return;
  const int ql = lane & 31, hf = lane >> 5;
  const int t = t0 + ql;
  const bool qvalid = t < a.chunk;
  const int n_keys = a.prior + a.chunk;                  // keys in the table
  const int qpos = a.prior + min(t, a.chunk - 1);        // this lane's query position

  Frag8<T> qf[D / 16];
  const char* qrow = static_cast<const char*>(a.q) + (long(h) * a.chunk + min(t, a.chunk - 1)) * D * EB;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) load_frag8(qf[st], qrow + (16 * st + 8 * hf) * EB);

  f32x16 o[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) o[n] = f32x16{};
  float m = -__builtin_inff(), lsum = 0.f;
  bool bad = false;

  const int32_t* tbl = a.pre_pages + long(g) * a.pre_max_blocks;
  const int kend = a.prior + min(t0 + 31, a.chunk - 1) + 1;  // keys this wave needs: [0, kend)
  const int n_kb = (kend + 31) / 32;
  const int krow = kappa(ql);
  for (int kb = 0; kb < n_kb; ++kb) {
    const int key0 = kb * 32;
    const int pa = tbl[key0 / kPage];
    const bool has_b = key0 + kPage < n_keys;
    const int pb = has_b ? tbl[key0 / kPage + 1] : pa;
    if (pa < 0 || pa >= a.n_pages || pb < 0 || pb >= a.n_pages) {
      bad = true;
      continue;
    }
    const char* pga = a.pool + pa * PAGE_BYTES;
    const char* pgb = a.pool + pb * PAGE_BYTES;
    // S^T = K . Q^T ; K operand row ql holds key kappa(ql) of the block
    const char* krp = (krow < kPage ? pga : pgb) + (krow & 15) * D * EB;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      Frag8<T> kf;
      load_frag8(kf, krp + (16 * st + 8 * hf) * EB);
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
    // O^T += V^T . P^T, one 16-deep step per page
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      Frag8<T> pf;
      set_frag8(pf, &p[8 * u]);
      const char* vp = (u ? pgb : pga) + kPage * D * EB;
      const int nvalid = n_keys - (key0 + 16 * u + 8 * hf);   // slots at or past the table end hold no key
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        Frag8<T> vf;
        load_frag8(vf, vp + ((32 * n + ql) * kPage + 8 * hf) * EB);
        if (nvalid < 8) zero_from(vf, nvalid);
        mma32x32_k16(o[n], vf, pf);
      }
    }
  }
  lsum += shfl_xor(lsum, 32);
  if (bad && a.status && lane == 0) atomicOr(a.status, XP_DEV_BAD_PAGE);
  if (!qvalid) return;
  const float inv = bad ? __builtin_nanf("") : 1.0f / lsum;
  void* dst;
  long row_off;
  if (t >= a.off && t < a.off + a.n_local) {
    dst = a.out_local;
    row_off = long(t - a.off) * a.out_local_stride;
  } else {
    dst = a.out_peer;
    row_off = long(t < a.off ? t : t - a.n_local) * a.out_peer_stride;
  }
  const long base = row_off + long(h) * D;
  // element r of o[n]: dim 32*n + 8*(r/4) + 4*hf + r%4
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) St<T>::store(dst, base + 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3), o[n][r] * inv);
}

}  // namespace

xp_status launch_prefill(int dtype, const void* q, const void* pool, int n_pages, int S, const int32_t* pre_pages,
                         int pre_max_blocks, int hq, int hkv, int d, int prior, int chunk, int off, int n_local,
                         void* out_local, int out_local_stride, void* out_peer, int out_peer_stride,
                         uint32_t* status, hipStream_t s) {
  if (chunk == 0) return XP_OK;
  if (S != kPage) return fail(XP_EUNSUPPORTED, "prefill attention: page_size %d (supported: 16)", S);
  if (hkv <= 0 || hq % hkv) return fail(XP_ESHAPE, "prefill attention: hq=%d hkv=%d", hq, hkv);
  if (pre_max_blocks * kPage < prior + chunk)
    return fail(XP_EPAGE, "prefill attention: table of %d blocks < %d keys", pre_max_blocks, prior + chunk);
  if (off < 0 || n_local < 0 || off + n_local > chunk) return fail(XP_ESHAPE, "prefill attention: off/n_local");
  PrefillArgs a{q, static_cast<const char*>(pool), n_pages, pre_pages, pre_max_blocks, hq, hkv, prior, chunk,
                off, n_local, out_local, out_local_stride, out_peer, out_peer_stride,
                float(1.4426950408889634 / __builtin_sqrt(double(d))), status};
  const dim3 grid(cdiv(chunk, 128), hq);
  if (dtype == XP_BF16) {
    if (d == 128) hipLaunchKernelGGL((prefill_kernel<bf16_t, 128>), grid, dim3(256), 0, s, a);
    else if (d == 64) hipLaunchKernelGGL((prefill_kernel<bf16_t, 64>), grid, dim3(256), 0, s, a);
    else return fail(XP_EUNSUPPORTED, "prefill attention: head_dim %d", d);
  } else if (dtype == XP_F32) {
    if (d == 128) hipLaunchKernelGGL((prefill_kernel<float, 128>), grid, dim3(256), 0, s, a);
    else if (d == 64) hipLaunchKernelGGL((prefill_kernel<float, 64>), grid, dim3(256), 0, s, a);
    else return fail(XP_EUNSUPPORTED, "prefill attention: head_dim %d", d);
  } else {
    return fail(XP_EINVAL, "prefill attention: dtype %d", dtype);
  }
  XP_CHECK_LAUNCH();
  return XP_OK;
}

}  // namespace xp
