// Measurement probes.  Hardware placement: which XCC / SE / CU each workgroup of a
// launch ran on (to check how a stream's CU mask maps onto the XCDs).  Streaming
// read: every byte of a buffer read once, the ceiling HBM-bound kernels are compared
// with.
#include "xp_device.h"
#include "xp_internal.h"

namespace xp {
namespace {

__global__ void probe_kernel(int32_t* out) {
  if (threadIdx.x != 0) return;
  // s_getreg fields: HW_ID (id 4): CU_ID bits 11:8, SH_ID bit 12, SE_ID bits 15:13;
  // XCC_ID (id 20): bits 3:0.
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
  const uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20);
  int32_t* o = out + 4 * blockIdx.x;
  o[0] = int32_t(xcc & 0xf);
  o[1] = int32_t((hw >> 13) & 0x7);
  o[2] = int32_t((hw >> 8) & 0xf) | (int32_t((hw >> 12) & 1) << 4);
  o[3] = int32_t(hw);
  // keep the workgroup resident briefly so the launch spreads over the mask
  uint64_t t0 = __builtin_readcyclecounter();
  while (__builtin_readcyclecounter() - t0 < 20000) {
  }
}

// Each thread reads U = 4 independent 16-byte pieces per iteration of a grid-stride
// loop, non-temporal (measured on MI355X: 6.05 TB/s, against 5.55 with plain loads and
// 5.3-5.4 with 8 or 16 pieces); the XOR of everything a thread read reaches memory only
// if it equals a value that random data essentially never gives, which keeps the
// loads without adding traffic.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t fold16(const uint4* p) {
  const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return a.x ^ a.y ^ a.z ^ a.w;
}
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, long n16,
                                                         uint32_t* __restrict__ sink) {
  constexpr int U = 4;
  const long stride = long(gridDim.x) * 256;
  uint32_t acc = 0;
  long i = long(blockIdx.x) * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = fold16(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= fold16(src + i);
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace
}  // namespace xp

extern "C" xp_status xp_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16) return xp::fail(XP_EINVAL, "xp_probe_read: bad argument");
  const int blocks = 8 * xp::device_cus();
  hipLaunchKernelGGL(xp::read_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), long(bytes / 16), sink);
  XP_CHECK_LAUNCH();
  return XP_OK;
}

extern "C" xp_status xp_probe_hw_ids(int32_t n_blocks, int32_t* out, void* stream) {
  if (n_blocks <= 0 || !out) return xp::fail(XP_EINVAL, "xp_probe_hw_ids: bad argument");
  hipLaunchKernelGGL(xp::probe_kernel, dim3(n_blocks), dim3(64), 0, static_cast<hipStream_t>(stream), out);
  XP_CHECK_LAUNCH();
  return XP_OK;
}
