// Rotary embedding and the step's appends, shared by the stand-alone RoPE/append kernel
// (post_qkv_kernel) and the QKV GEMM's fused epilogue, so both produce the same bits.
//
// Decode Token Parallelism §4.3 fixes the order for a decode token: rotary embedding,
// append the new K/V to the local cache, then attention.  ConfluxServe §4 (KV
// residency, Fig. 8): decode requests extend their rank-local cache on every KV head,
// while the prefill chunk appends to its head-sharded cache, i.e. to this rank's KV
// heads only; the local rows' other heads leave through the All-to-All stand-in.
#pragma once
#include "xp_device.h"
#include "xp_internal.h"

namespace xp {

// sin and cos of x (radians, |x| < 2^40) in fp64.  x is first reduced modulo 2 pi by
// Cody and Waite's two-constant method (2 pi = P1 + P2, P1 the double nearest 2 pi; for
// these magnitudes k P1 is exact inside the fma and the remainder is good to a few
// units in the last place), so the library's sincos only ever sees |r| <= pi.
__device__ __forceinline__ void sincos_2pi(double x, double* sn, double* cn) {
  constexpr double P1 = 6.283185307179586;        // 0x1.921fb54442d18p+2
  constexpr double P2 = 2.4492935982947064e-16;   // 2 pi - P1
  const double k = rint(x * (1.0 / P1));
  const double r = fma(-k, P2, fma(-k, P1, x));
  sincos(r, sn, cn);
}

// (cos, sin) of position pos at frequency inv_freq, rounded to fp32
__device__ __forceinline__ float2 rope_cs(int pos, double inv_freq) {
  double sn, cn;
  sincos_2pi(double(pos) * inv_freq, &sn, &cn);
  return make_float2(float(cn), float(sn));
}

// the rotation of the pair (x0, x1) = (dim j, dim j + d/2), written with explicit fmas
// so every caller rounds the same way
__device__ __forceinline__ void rope_pair(float x0, float x1, float c, float s, float& y0, float& y1) {
  y0 = __builtin_fmaf(x0, c, -(x1 * s));
  y1 = __builtin_fmaf(x1, c, x0 * s);
}
__device__ __forceinline__ void rope_pair4(float4 x0, float4 x1, const float2 (&cs)[4], float4& y0, float4& y1) {
  rope_pair(x0.x, x1.x, cs[0].x, cs[0].y, y0.x, y1.x);
  rope_pair(x0.y, x1.y, cs[1].x, cs[1].y, y0.y, y1.y);
  rope_pair(x0.z, x1.z, cs[2].x, cs[2].y, y0.z, y1.z);
  rope_pair(x0.w, x1.w, cs[3].x, cs[3].y, y0.w, y1.w);
}

// Page of local row `row`'s slot on KV head g: -2 when the row does not append on g
// here (a prefill row on another rank's head), -1 when the table has no such block.
__device__ __forceinline__ int rope_page(const PostQkvArgs& a, int row, int g, int pos) {
  const int hkv_loc = a.Hkv / a.P, k0 = a.r * hkv_loc;
  if (row >= a.n_pl) {
    const int i = row - a.n_pl;
    return (pos >= 0 && pos / a.S < a.dec_max_blocks) ? a.dec_pages[(long(i) * a.Hkv + g) * a.dec_max_blocks + pos / a.S]
                                                       : -1;
  }
  if (g >= k0 && g < k0 + hkv_loc) return a.pre_pages[long(g - k0) * a.pre_max_blocks + pos / a.S];
  return -2;
}

// position of local row `row` (prefill rows first, then decode rows)
__device__ __forceinline__ int rope_pos(const PostQkvArgs& a, int row) {
  return row >= a.n_pl ? a.dec_ctx[row - a.n_pl] : a.prior + a.off + row;
}

// Stores dims j .. j + 3 (j a multiple of 4) of head h of local row `row` where the
// step puts them: a query head to the decode queries, the rank's chunk queries or the
// export; a key (h in [Hq, Hq + Hkv)) or value (h in [Hq + Hkv, Hq + 2 Hkv)) head to its
// page's K plane (16-byte chunks, chunk-major over the slots) or V plane (dim-major), or
// to the export when the row does not append on that head here.  `page` is
// rope_page(...) for key and value heads (ignored for queries).
template <typename T>
__device__ __forceinline__ void rope_store4(const PostQkvArgs& a, int row, int h, int j, float4 v, int pos,
                                            int page) {
  const int d = a.d, hq_loc = a.Hq / a.P, hkv_loc = a.Hkv / a.P;
  const int q0 = a.r * hq_loc, k0 = a.r * hkv_loc;
  const int oq_w = (a.Hq - hq_loc) * d, ok_w = (a.Hkv - hkv_loc) * d;
  const long pq_out = long(row) * (oq_w + 2 * ok_w);
  if (h < a.Hq) {
    if (row >= a.n_pl) St4<T>::store(a.q_dec, (long(row - a.n_pl) * a.Hq + h) * d + j, v);
    else if (h >= q0 && h < q0 + hq_loc) St4<T>::store(a.q_pre, (long(h - q0) * a.chunk + a.off + row) * d + j, v);
    else St4<T>::store(a.peer_qkv_out, pq_out + long(h < q0 ? h : h - hq_loc) * d + j, v);
    return;
  }
  const bool is_v = h >= a.Hq + a.Hkv;
  const int g = is_v ? h - a.Hq - a.Hkv : h - a.Hq;
  if (page == -2) {
    const int gi = g < k0 ? g : g - hkv_loc;
    St4<T>::store(a.peer_qkv_out, pq_out + oq_w + (is_v ? ok_w : 0) + long(gi) * d + j, v);
    return;
  }
  if (page < 0 || page >= a.n_pages) {
    if (a.status) atomicOr(a.status, XP_DEV_BAD_PAGE);
    return;
  }
  const int S = a.S, slot = pos % S;
  const long base = long(page) * 2 * S * d;
  if (!is_v) {
    St4<T>::store(a.pool, base + k_elem<T>(slot, j, S), v);
  } else {
    const long vb = base + long(S) * d + long(j) * S + slot;
    St<T>::store(a.pool, vb, v.x);
    St<T>::store(a.pool, vb + S, v.y);
    St<T>::store(a.pool, vb + 2 * S, v.z);
    St<T>::store(a.pool, vb + 3 * S, v.w);
  }
}

}  // namespace xp
