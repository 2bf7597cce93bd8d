// RoPE + KV append for one layer step, and the paged-pool append/gather kernels.
//
// Decode Token Parallelism §4.3 fixes the order for a decode token: rotary
// embedding, append the new K/V to the local cache, then attention.  ConfluxServe
// §4 (KV residency, Fig. 8): decode requests extend their rank-local cache on
// every KV head, while the prefill chunk appends to its head-sharded cache, i.e.
// to this rank's KV heads only, for all chunk rows (local rows from this rank's
// projection, peer rows from the All-to-All stand-in buffer).
//
// Pool layout: page = [K plane: 16-byte chunks of dims, chunk-major over the slots
// (k_elem) | V plane: d x page_size dim-major]; position p of a table row is slot
// p % page_size of page table[p / page_size].
//
// RoPE angles pos * base^(-2i/d) are formed and reduced in fp64 once per row
// (positions reach 65536, where an fp32 product would already be off by
// several milliradians) and the rotation itself runs in fp32.
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

// One workgroup per row task: tasks [0, M) are this rank's rows; the chunk's peer
// rows, which are only copied, go kPeerRowsPerTask to a task after them.
constexpr int kPeerRowsPerTask = 8;

template <typename T>
__global__ __launch_bounds__(256) void post_qkv_kernel(PostQkvArgs a) {
  extern __shared__ float cs[];  // [d/2] cos, [d/2] sin
  const int task = blockIdx.x, tid = threadIdx.x;
  const int M = a.n_pl + a.n_d;
  const int d = a.d, half = d / 2, S = a.S;
  const int hq_loc = a.Hq / a.P, hkv_loc = a.Hkv / a.P;
  const int q0 = a.r * hq_loc, k0 = a.r * hkv_loc;
  const int ldq = (a.Hq + 2 * a.Hkv) * d;

  if (task >= M) {  // peer chunk rows: copy their (already rotated) q | k | v on this rank's heads
    const int n_peer = a.chunk - a.n_pl;
    const int p1 = min(n_peer, (task - M + 1) * kPeerRowsPerTask);
    for (int p = (task - M) * kPeerRowsPerTask; p < p1; ++p) {
      const int t = p < a.off ? p : p + a.n_pl;
      const int pos = a.prior + t;
      const int w = (hq_loc + 2 * hkv_loc) * d;
      const long src = long(p) * w;
      for (int e0 = tid; e0 < hq_loc * d; e0 += 256 * 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = e0 + 256 * u < hq_loc * d ? St<T>::load(a.peer_qkv_in, src + e0 + 256 * u) : 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + 256 * u;
          if (e >= hq_loc * d) break;
          St<T>::store(a.q_pre, (long(e / d) * a.chunk + t) * d + e % d, v[u]);
        }
      }
      for (int e = tid; e < hkv_loc * d; e += 256) {
        const int g = e / d, j = e % d;
        const int page = a.pre_pages[long(g) * a.pre_max_blocks + pos / S];
        put_kv<T>(a.pool, a.n_pages, S, d, page, pos % S, j,
                  St<T>::load(a.peer_qkv_in, src + hq_loc * d + e),
                  St<T>::load(a.peer_qkv_in, src + (hq_loc + hkv_loc) * d + e), a.status);
      }
    }
    return;
  }

  const bool is_dec = task >= a.n_pl;
  const int i = task - a.n_pl;          // decode request
  const int t = a.off + task;           // chunk row of a local prefill row
  const int pos = is_dec ? a.dec_ctx[i] : a.prior + t;
  int* pg = reinterpret_cast<int*>(cs + d);  // [Hkv] page of this row's slot per kv head, -2: not appended here
  if (tid < half) {
    const double theta = pow(a.rope_base, -2.0 * double(tid) / double(d));
    double sn, cn;
    sincos(double(pos) * theta, &sn, &cn);
    cs[tid] = float(cn);
    cs[half + tid] = float(sn);
  }
  for (int g = tid; g < a.Hkv; g += 256) {
    int page = -2;
    if (is_dec) {
      page = (pos >= 0 && pos / S < a.dec_max_blocks) ? a.dec_pages[(long(i) * a.Hkv + g) * a.dec_max_blocks + pos / S]
                                                       : -1;
    } else if (g >= k0 && g < k0 + hkv_loc) {
      page = a.pre_pages[long(g - k0) * a.pre_max_blocks + pos / S];
    }
    pg[g] = page;
  }
  __syncthreads();
  const float* row = a.qkv + long(task) * ldq;
  const int oq_w = (a.Hq - hq_loc) * d, ok_w = (a.Hkv - hkv_loc) * d;
  const long pq_out = long(task) * (oq_w + 2 * ok_w);

  // rotated q and k: pairs (j, j + d/2).  Each thread loads a batch of pairs before
  // storing any of them: the compiler cannot prove the stores leave the row alone, so
  // loads interleaved with stores would each wait a full memory round trip.
  constexpr int kBatch = 8;
  const int n_pairs = (a.Hq + a.Hkv) * half;
  for (int e0 = tid; e0 < n_pairs; e0 += 256 * kBatch) {
    float x0[kBatch], x1[kBatch], v0[kBatch], v1[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = e0 + 256 * u;
      x0[u] = x1[u] = v0[u] = v1[u] = 0.f;
      if (e < n_pairs) {
        const int h = e / half, j = e % half;
        x0[u] = row[h * d + j];
        x1[u] = row[h * d + j + half];
        if (h >= a.Hq) {  // the value row of kv head h - Hq
          v0[u] = row[(a.Hkv + h) * d + j];
          v1[u] = row[(a.Hkv + h) * d + j + half];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = e0 + 256 * u;
      if (e >= n_pairs) break;
      const int h = e / half, j = e % half;
      const float c = cs[j], s = cs[half + j];
      const float y0 = x0[u] * c - x1[u] * s, y1 = x1[u] * c + x0[u] * s;
      if (h < a.Hq) {
        if (is_dec) {
          const long o = (long(i) * a.Hq + h) * d;
          St<T>::store(a.q_dec, o + j, y0);
          St<T>::store(a.q_dec, o + j + half, y1);
        } else if (h >= q0 && h < q0 + hq_loc) {
          const long o = (long(h - q0) * a.chunk + t) * d;
          St<T>::store(a.q_pre, o + j, y0);
          St<T>::store(a.q_pre, o + j + half, y1);
        } else {
          const long o = pq_out + long(h < q0 ? h : h - hq_loc) * d;
          St<T>::store(a.peer_qkv_out, o + j, y0);
          St<T>::store(a.peer_qkv_out, o + j + half, y1);
        }
      } else {
        const int g = h - a.Hq;
        const int page = pg[g];
        if (page != -2) {
          put_kv<T>(a.pool, a.n_pages, S, d, page, pos % S, j, y0, v0[u], a.status);
          put_kv<T>(a.pool, a.n_pages, S, d, page, pos % S, j + half, y1, v1[u], a.status);
        } else {
          const int gi = g < k0 ? g : g - hkv_loc;
          const long ok = pq_out + oq_w + long(gi) * d;
          const long ov = pq_out + oq_w + ok_w + long(gi) * d;
          St<T>::store(a.peer_qkv_out, ok + j, y0);
          St<T>::store(a.peer_qkv_out, ok + j + half, y1);
          St<T>::store(a.peer_qkv_out, ov + j, v0[u]);
          St<T>::store(a.peer_qkv_out, ov + j + half, v1[u]);
        }
      }
    }
  }
  // local prefill rows: attention outputs of the heads other ranks own arrive as peer_attn_in
  // (batched like the pairs above, so the loads do not wait on the stores)
  if (!is_dec && oq_w > 0) {
    for (int e0 = tid; e0 < oq_w; e0 += 256 * kBatch) {
      float v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = e0 + 256 * u;
        v[u] = e < oq_w ? St<T>::load(a.peer_attn_in, long(task) * oq_w + e) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = e0 + 256 * u;
        if (e >= oq_w) break;
        const int hi = e / d, j = e % d;
        const int h = hi < q0 ? hi : hi + hq_loc;
        St<T>::store(a.attn, long(task) * a.Hq * d + long(h) * d + j, v[u]);
      }
    }
  }
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

xp_status launch_post_qkv(int dtype, const PostQkvArgs& a, hipStream_t s) {
  const int tasks = a.n_pl + a.n_d + cdiv(a.chunk - a.n_pl, kPeerRowsPerTask);
  if (tasks == 0) return XP_OK;
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
