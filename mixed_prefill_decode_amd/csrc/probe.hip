// Hardware placement probe: which XCC / SE / CU each workgroup of a launch ran
// on.  Used to check how a stream's CU mask maps onto the XCDs.
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

}  // namespace
}  // namespace xp

extern "C" xp_status xp_probe_hw_ids(int32_t n_blocks, int32_t* out, void* stream) {
  if (n_blocks <= 0 || !out) return xp::fail(XP_EINVAL, "xp_probe_hw_ids: bad argument");
  hipLaunchKernelGGL(xp::probe_kernel, dim3(n_blocks), dim3(64), 0, static_cast<hipStream_t>(stream), out);
  XP_CHECK_LAUNCH();
  return XP_OK;
}
