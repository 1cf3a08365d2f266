// fp8 (OCP E4M3) and bf8 (OCP E5M2) GEMM kernel instances: 256x256x128 tiles.
#include "skg_inst_gemm_common.hpp"

namespace skg {
GemmInst gemm_instance_f8(int tile_id, int dtype, bool tensor_scales) {
  if (tile_id != SKG_TILE_256x256x128) return {nullptr, nullptr};
  if (dtype == SKG_F8E4M3)
    return gemm_inst::make<TileCfg<DT_F8, 256, 256, 128, 2, 2, 32, 128>>(tensor_scales);
  if (dtype == SKG_F8E5M2)
    return gemm_inst::make<TileCfg<DT_BF8, 256, 256, 128, 2, 2, 32, 128>>(tensor_scales);
  return {nullptr, nullptr};
}
hipError_t wait_timeouts_gemm_f8(uint32_t* out, bool reset) { return unit_wait_timeouts(out, reset); }
}  // namespace skg
