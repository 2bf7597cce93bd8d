// RMSNorm of a row block: y = x / sqrt(mean(x^2) + eps) * gamma, written in the
// storage type as the next projection's MFMA operand (pre-norm block; Decode
// Token Parallelism §4.3 lists normalization between attention and the MLP).
// One workgroup per row; the sum of squares is accumulated in fp32.  The first RMSNorm
// of a step also forms each row's RoPE (cos, sin) table for the QKV projection's
// fused epilogue (rope.h).
#include "rope.h"
#include "xp_device.h"
#include "xp_internal.h"

namespace xp {

namespace {

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ x, const void* __restrict__ gamma,
                                                      void* __restrict__ y, int H, float eps,
                                                      uint32_t* __restrict__ status_clear, RopeTab rope) {
  // 16-byte vectors of the input; the row is read twice (the second pass hits L2)
  constexpr int V = 16 / St<TI>::bytes;
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (status_clear && row == 0 && tid == 0) *status_clear = 0u;
  // the row's RoPE (cos, sin) pairs for the QKV projection's epilogue
  if (rope.tab && tid < rope.half) {
    const int pos = row < rope.n_pl ? rope.pos0 + row : rope.dec_ctx[row - rope.n_pl];
    rope.tab[long(row) * rope.half + tid] = rope_cs(pos, rope.inv_freq[tid]);
  }
  const char* xr = static_cast<const char*>(x) + long(row) * H * St<TI>::bytes;
  const int nv = H / V;
  float ss = 0.f;
  for (int v = tid; v < nv; v += 256) {
    const uint4 u = reinterpret_cast<const uint4*>(xr)[v];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float f = St<TI>::load(&u, e);
      ss += f * f;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor(ss, m);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float rstd = 1.0f / sqrtf(tot / float(H) + eps);
  char* yr = static_cast<char*>(y) + long(row) * H * St<TO>::bytes;
  for (int v = tid; v < nv; v += 256) {
    const uint4 u = reinterpret_cast<const uint4*>(xr)[v];
    float f[V];
#pragma unroll
    for (int e = 0; e < V; ++e) f[e] = St<TI>::load(&u, e) * rstd * St<TO>::load(gamma, long(v) * V + e);
    if constexpr (St<TO>::bytes == 2) {
      uint32_t w[V / 2];
#pragma unroll
      for (int e = 0; e < V / 2; ++e) w[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
      if constexpr (V == 8)
        reinterpret_cast<uint4*>(yr)[v] = make_uint4(w[0], w[1], w[2], w[3]);
      else
        reinterpret_cast<uint2*>(yr)[v] = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int e = 0; e < V; ++e) reinterpret_cast<float*>(yr)[long(v) * V + e] = f[e];
    }
  }
}

__global__ void clear_status_kernel(uint32_t* status) { *status = 0u; }

}  // namespace

xp_status launch_rmsnorm(int dtype, const void* x, int x_is_f32, const void* gamma, void* y, int M, int H,
                         float eps, uint32_t* status_clear, hipStream_t s, const RopeTab* rope) {
  if (dtype != XP_BF16 && dtype != XP_F32) return fail(XP_EINVAL, "xp_rmsnorm: dtype %d", dtype);
  if (M < 0 || H <= 0 || H % 8) return fail(XP_ESHAPE, "xp_rmsnorm: M=%d H=%d (H a multiple of 8)", M, H);
  if (!x || !gamma || !y) return fail(XP_EINVAL, "xp_rmsnorm: null pointer");
  if (M == 0) {
    if (status_clear) {
      hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, s, status_clear);
      XP_CHECK_LAUNCH();
    }
    return XP_OK;
  }
  RopeTab rt{};
  if (rope) rt = *rope;
  if (rt.tab && (rt.half <= 0 || rt.half > 64)) return fail(XP_EUNSUPPORTED, "RoPE table: d/2 = %d", rt.half);
  if (dtype == XP_BF16) {
    if (x_is_f32)
      hipLaunchKernelGGL((rmsnorm_kernel<float, bf16_t>), dim3(M), dim3(256), 0, s, x, gamma, y, H, eps, status_clear, rt);
    else
      hipLaunchKernelGGL((rmsnorm_kernel<bf16_t, bf16_t>), dim3(M), dim3(256), 0, s, x, gamma, y, H, eps, status_clear,
                         rt);
  } else {
    hipLaunchKernelGGL((rmsnorm_kernel<float, float>), dim3(M), dim3(256), 0, s, x, gamma, y, H, eps, status_clear, rt);
  }
  XP_CHECK_LAUNCH();
  return XP_OK;
}

}  // namespace xp
