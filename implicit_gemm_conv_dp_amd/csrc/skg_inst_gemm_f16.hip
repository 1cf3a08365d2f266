// fp16 GEMM kernel instances.
#include "skg_inst_gemm_common.hpp"

namespace skg {
GemmInst gemm_instance_f16(int tile_id, bool tensor_scales) {
  return gemm_inst::by_tile<DT_F16>(tile_id, tensor_scales);
}
hipError_t wait_timeouts_gemm_f16(uint32_t* out, bool reset) { return unit_wait_timeouts(out, reset); }
}  // namespace skg
