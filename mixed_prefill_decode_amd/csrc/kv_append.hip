// RoPE + KV append for one layer step, and the paged-pool append/gather kernels.
//
// Decode Token Parallelism §4.3 fixes the order for a decode token: rotary
// embedding, append the new K/V to the local cache, then attention.  ConfluxServe
// §4 (KV residency, Fig. 8): decode requests extend their rank-local cache on
// every KV head, while the prefill chunk appends to its head-sharded cache, i.e.
// to this rank's KV heads only, for all chunk rows (local rows from this rank's
// projection, peer rows from the All-to-All stand-in buffer).  A step with at most one
// chunk rotates and appends its local rows in the QKV projection's epilogue
// (gemm_core.h); this kernel then only copies the peer rows and the peer_attn_in rows.
// The rotation and routing helpers are shared (rope.h).
//
// Pool layout: page = [K plane: 16-byte chunks of dims, chunk-major over the slots
// (k_elem) | V plane: d x page_size dim-major]; position p of a table row is slot
// p % page_size of page table[p / page_size].
//
// RoPE angles pos * base^(-2i/d) are formed and reduced in fp64 once per row
// (positions reach 65536, where an fp32 product would already be off by
// several milliradians; the frequencies base^(-2i/d) come from the host, also in
// fp64) and the rotation itself runs in fp32.
#include <algorithm>
#include <cmath>

#include "rope.h"
#include "xp_device.h"
#include "xp_internal.h"

namespace xp {

namespace {

template <typename T>
__device__ __forceinline__ void put_kv(void* pool, int n_pages, int S, int d, int page, int slot, int j,
                                       float kval, float vval, uint32_t* status) {
  if (page < 0 || page >= n_pages) {
    if (status) atomicOr(status, XP_DEV_BAD_PAGE);
    return;
  }
  const long base = long(page) * 2 * S * d;
  St<T>::store(pool, base + k_elem<T>(slot, j, S), kval);
  St<T>::store(pool, base + long(S) * d + long(j) * S + slot, vval);
}

// dims j .. j + 3 (j a multiple of 4) of one slot: the four K values are consecutive
// inside one 16-byte chunk of the K plane, the V values are S apart
template <typename T>
__device__ __forceinline__ void put_kv4(void* pool, int n_pages, int S, int d, int page, int slot, int j, float4 k,
                                        float4 v, uint32_t* status) {
  if (page < 0 || page >= n_pages) {
    if (status) atomicOr(status, XP_DEV_BAD_PAGE);
    return;
  }
  const long base = long(page) * 2 * S * d;
  St4<T>::store(pool, base + k_elem<T>(slot, j, S), k);
  const long vb = base + long(S) * d + long(j) * S + slot;
  St<T>::store(pool, vb, v.x);
  St<T>::store(pool, vb + S, v.y);
  St<T>::store(pool, vb + 2 * S, v.z);
  St<T>::store(pool, vb + 3 * S, v.w);
}

// copies elements [si, si + 8) of src to [di, di + 8) of dst unchanged (16 or 32 bytes)
template <typename T>
__device__ __forceinline__ void copy8(void* dst, long di, const void* src, long si) {
  const uint4* s4 = reinterpret_cast<const uint4*>(static_cast<const T*>(src) + si);
  uint4* d4 = reinterpret_cast<uint4*>(static_cast<T*>(dst) + di);
  d4[0] = s4[0];
  if constexpr (sizeof(T) == 4) d4[1] = s4[1];
}

// One workgroup per row task: tasks [0, M) are this rank's rows; the chunk's peer
// rows, which are only copied, go kPeerRowsPerTask to a task after them.  Every
// thread moves 4 consecutive dims of a head (and their rotation partners d/2 away) or
// 8 consecutive elements of a copy per access.
constexpr int kPeerRowsPerTask = 8;

template <typename T>
__global__ __launch_bounds__(256) void post_qkv_kernel(PostQkvArgs a) {
  extern __shared__ float cs[];  // [d/2] cos, [d/2] sin
  const int task = int(blockIdx.x) + a.task0, tid = threadIdx.x;
  const int M = a.n_pl + a.n_d;
  const int d = a.d, half = d / 2, S = a.S;
  const int hq_loc = a.Hq / a.P, hkv_loc = a.Hkv / a.P;
  const int q0 = a.r * hq_loc;
  const int ldq = (a.Hq + 2 * a.Hkv) * d;

  if (task >= M) {  // peer chunk rows: copy their (already rotated) q | k | v on this rank's heads
    // the task's rows flattened: q items of 8 elements, then K/V items of 4 dims; every
    // thread loads all its items before it stores any
    const int n_peer = a.chunk - a.n_pl;
    const int pr0 = (task - M) * kPeerRowsPerTask, nr = min(n_peer - pr0, kPeerRowsPerTask);
    const int w = (hq_loc + 2 * hkv_loc) * d;
    const int qi = hq_loc * d / 8, ki = hkv_loc * d / 4;   // items per row
    constexpr int kQ = 4, kK = 2;
    uint4 qv[kQ][sizeof(T) / 2];
    float4 kv[kK], vv[kK];
#pragma unroll
    for (int u = 0; u < kQ; ++u) {
      const int e = tid + 256 * u;
      if (e < nr * qi) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const T*>(a.peer_qkv_in) +
                                                          long(pr0 + e / qi) * w + 8 * (e % qi));
#pragma unroll
        for (int c = 0; c < int(sizeof(T) / 2); ++c) qv[u][c] = src[c];
      }
    }
#pragma unroll
    for (int u = 0; u < kK; ++u) {
      const int e = tid + 256 * u;
      if (e < nr * ki) {
        const long src = long(pr0 + e / ki) * w + 4 * (e % ki);
        kv[u] = St4<T>::load(a.peer_qkv_in, src + hq_loc * d);
        vv[u] = St4<T>::load(a.peer_qkv_in, src + (hq_loc + hkv_loc) * d);
      }
    }
    // items past the unrolled batches (shapes larger than the 32B layer's), one at a time
    for (int e = tid + 256 * kQ; e < nr * qi; e += 256) {
      const int p = pr0 + e / qi, t = p < a.off ? p : p + a.n_pl, f = 8 * (e % qi);
      copy8<T>(a.q_pre, (long(f / d) * a.chunk + t) * d + f % d, a.peer_qkv_in, long(p) * w + f);
    }
    for (int e = tid + 256 * kK; e < nr * ki; e += 256) {
      const int p = pr0 + e / ki, t = p < a.off ? p : p + a.n_pl, pos = a.prior + t, f = 4 * (e % ki);
      const int g = f / d, page = a.pre_pages[long(g) * a.pre_max_blocks + pos / S];
      put_kv4<T>(a.pool, a.n_pages, S, d, page, pos % S, f % d, St4<T>::load(a.peer_qkv_in, long(p) * w + hq_loc * d + f),
                 St4<T>::load(a.peer_qkv_in, long(p) * w + (hq_loc + hkv_loc) * d + f), a.status);
    }
#pragma unroll
    for (int u = 0; u < kQ; ++u) {
      const int e = tid + 256 * u;
      if (e < nr * qi) {
        const int p = pr0 + e / qi, t = p < a.off ? p : p + a.n_pl, f = 8 * (e % qi);
        uint4* dst = reinterpret_cast<uint4*>(static_cast<T*>(a.q_pre) + (long(f / d) * a.chunk + t) * d + f % d);
#pragma unroll
        for (int c = 0; c < int(sizeof(T) / 2); ++c) dst[c] = qv[u][c];
      }
    }
#pragma unroll
    for (int u = 0; u < kK; ++u) {
      const int e = tid + 256 * u;
      if (e < nr * ki) {
        const int p = pr0 + e / ki, t = p < a.off ? p : p + a.n_pl, pos = a.prior + t, f = 4 * (e % ki);
        const int g = f / d, page = a.pre_pages[long(g) * a.pre_max_blocks + pos / S];
        put_kv4<T>(a.pool, a.n_pages, S, d, page, pos % S, f % d, kv[u], vv[u], a.status);
      }
    }
    return;
  }

  const bool is_dec = task >= a.n_pl;
  const int row = task;                 // local row: the chunk's local rows, then the decodes
  const int oq_w = (a.Hq - hq_loc) * d;
  // local prefill rows: attention outputs of the heads other ranks own arrive as peer_attn_in
  auto copy_peer_attn = [&] {
    if (is_dec || oq_w == 0) return;
    for (int e = 8 * tid; e < oq_w; e += 256 * 8) {
      const int hi = e / d, j = e % d;
      const int h = hi < q0 ? hi : hi + hq_loc;
      copy8<T>(a.attn, long(task) * a.Hq * d + long(h) * d + j, a.peer_attn_in, long(task) * oq_w + e);
    }
  };
  if (a.rope_done) {   // the QKV projection's epilogue rotated and appended this row
    copy_peer_attn();
    return;
  }
  const int pos = rope_pos(a, row);
  float2* cs2 = reinterpret_cast<float2*>(cs);   // [d/2] (cos, sin)
  int* pg = reinterpret_cast<int*>(cs + d);      // [Hkv] page of this row's slot per kv head (rope_page)
  const float* qrow = a.qkv + long(task) * ldq;

  // rotated q and k: item (head h, dims j .. j + 3 < d/2) with partners j + d/2.  Each
  // thread loads a batch of items before storing any of them (the compiler cannot prove
  // the stores leave the row alone, so loads interleaved with stores would each wait a
  // full memory round trip); the first batch goes out before the angles are formed.
  constexpr int kBatch = 5;
  const int quads = half / 4;
  const int n_items = (a.Hq + a.Hkv) * quads;
  float4 x0[kBatch], x1[kBatch], v0[kBatch], v1[kBatch];
  auto load_batch = [&](int e0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = e0 + 256 * u;
      x0[u] = x1[u] = v0[u] = v1[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e < n_items) {
        const int h = e / quads, j = 4 * (e % quads);
        x0[u] = *reinterpret_cast<const float4*>(qrow + h * d + j);
        x1[u] = *reinterpret_cast<const float4*>(qrow + h * d + j + half);
        if (h >= a.Hq) {  // the value row of kv head h - Hq
          v0[u] = *reinterpret_cast<const float4*>(qrow + (a.Hkv + h) * d + j);
          v1[u] = *reinterpret_cast<const float4*>(qrow + (a.Hkv + h) * d + j + half);
        }
      }
    }
  };
  load_batch(tid);
  if (tid < half) cs2[tid] = rope_cs(pos, a.inv_freq[tid]);
  for (int g = tid; g < a.Hkv; g += 256) pg[g] = rope_page(a, row, g, pos);
  __syncthreads();
  for (int e0 = tid; e0 < n_items; e0 += 256 * kBatch) {
    if (e0 != tid) load_batch(e0);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = e0 + 256 * u;
      if (e >= n_items) break;
      const int h = e / quads, j = 4 * (e % quads);
      const float2 c4[4] = {cs2[j], cs2[j + 1], cs2[j + 2], cs2[j + 3]};
      float4 y0, y1;
      rope_pair4(x0[u], x1[u], c4, y0, y1);
      const int page = h >= a.Hq ? pg[h - a.Hq] : 0;
      rope_store4<T>(a, row, h, j, y0, pos, page);
      rope_store4<T>(a, row, h, j + half, y1, pos, page);
      if (h >= a.Hq) {
        rope_store4<T>(a, row, h + a.Hkv, j, v0[u], pos, page);
        rope_store4<T>(a, row, h + a.Hkv, j + half, v1[u], pos, page);
      }
    }
  }
  copy_peer_attn();
}

template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(void* pool, int n_pages, int S, int d, const int32_t* table,
                                                        int table_stride, const int32_t* seq, const int32_t* pos,
                                                        const void* k, const void* v, int n, uint32_t* status) {
  const long e = long(blockIdx.x) * 256 + threadIdx.x;
  if (e >= long(n) * d) return;
  const int t = int(e / d), j = int(e % d);
  const int p = pos[t];
  const int page = (p >= 0 && p / S < table_stride) ? table[long(seq[t]) * table_stride + p / S] : -1;
  put_kv<T>(pool, n_pages, S, d, page, p % S, j, St<T>::load(k, e), St<T>::load(v, e), status);
}

template <typename T>
__global__ __launch_bounds__(256) void kv_gather_kernel(const void* pool, int n_pages, int S, int d, const int32_t* table,
                                                        int table_stride, const int32_t* len, int max_len,
                                                        void* k_out, void* v_out) {
  const int sq = blockIdx.y;
  const long e = long(blockIdx.x) * 256 + threadIdx.x;
  const int n = min(len[sq], max_len);
  if (e >= long(n) * d) return;
  const int p = int(e / d), j = int(e % d);
  const int page = p / S < table_stride ? table[long(sq) * table_stride + p / S] : -1;
  const long o = (long(sq) * max_len + p) * d + j;
  if (page < 0 || page >= n_pages) {
    St<T>::store(k_out, o, __builtin_nanf(""));
    St<T>::store(v_out, o, __builtin_nanf(""));
    return;
  }
  const long base = long(page) * 2 * S * d;
  St<T>::store(k_out, o, St<T>::load(pool, base + k_elem<T>(p % S, j, S)));
  St<T>::store(v_out, o, St<T>::load(pool, base + long(S) * d + long(j) * S + p % S));
}

}  // namespace

void rope_frequencies(double base, int d, double* inv_freq) {
  for (int i = 0; i < d / 2 && i < 64; ++i) inv_freq[i] = std::pow(base, -2.0 * double(i) / double(d));
}

xp_status launch_post_qkv(int dtype, const PostQkvArgs& args, hipStream_t s) {
  const int n_peer_tasks = cdiv(args.chunk - args.n_pl, kPeerRowsPerTask);
  const int M = args.n_pl + args.n_d;
  int lo = args.only == 2 ? M : 0, hi = args.only == 1 ? M : M + n_peer_tasks;
  // with the rotation done by the QKV epilogue a local row's task only copies its
  // peer_attn_in heads (none without sequence parallelism)
  if (args.rope_done && args.P == 1) lo = std::max(lo, M);
  if (args.rope_done && args.only == 1) hi = std::min(hi, args.n_pl);   // decode rows have no peer heads
  if (hi <= lo) return XP_OK;
  if (args.d % 8 || args.d / 2 > 64) return fail(XP_EUNSUPPORTED, "RoPE: head_dim %d", args.d);
  // the rotation frequencies base^(-2i/d), formed once in fp64 on the host
  PostQkvArgs a = args;
  a.task0 = lo;
  const int tasks = hi - lo;
  rope_frequencies(a.rope_base, a.d, a.inv_freq);
  const size_t shm = size_t(a.d) * sizeof(float) + size_t(a.Hkv) * sizeof(int);
  if (dtype == XP_BF16)
    hipLaunchKernelGGL(post_qkv_kernel<bf16_t>, dim3(tasks), dim3(256), shm, s, a);
  else
    hipLaunchKernelGGL(post_qkv_kernel<float>, dim3(tasks), dim3(256), shm, s, a);
  XP_CHECK_LAUNCH();
  return XP_OK;
}

xp_status launch_kv_append(int dtype, void* pool, int n_pages, int S, int d, const int32_t* table, int table_stride,
                           const int32_t* seq, const int32_t* pos, const void* k, const void* v, int n,
                           uint32_t* status, hipStream_t s) {
  if (n == 0) return XP_OK;
  const int blocks = cdiv(long(n) * d, 256);
  if (dtype == XP_BF16)
    hipLaunchKernelGGL(kv_append_kernel<bf16_t>, dim3(blocks), dim3(256), 0, s, pool, n_pages, S, d, table,
                       table_stride, seq, pos, k, v, n, status);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(blocks), dim3(256), 0, s, pool, n_pages, S, d, table,
                       table_stride, seq, pos, k, v, n, status);
  XP_CHECK_LAUNCH();
  return XP_OK;
}

xp_status launch_kv_gather(int dtype, const void* pool, int n_pages, int S, int d, const int32_t* table,
                           int table_stride, const int32_t* len, int n_seq, int max_len, void* k_out, void* v_out,
                           hipStream_t s) {
  if (n_seq == 0 || max_len == 0) return XP_OK;
  const dim3 grid(cdiv(long(max_len) * d, 256), n_seq);
  if (dtype == XP_BF16)
    hipLaunchKernelGGL(kv_gather_kernel<bf16_t>, grid, dim3(256), 0, s, pool, n_pages, S, d, table, table_stride,
                       len, max_len, k_out, v_out);
  else
    hipLaunchKernelGGL(kv_gather_kernel<float>, grid, dim3(256), 0, s, pool, n_pages, S, d, table, table_stride,
                       len, max_len, k_out, v_out);
  XP_CHECK_LAUNCH();
  return XP_OK;
}

}  // namespace xp
