// fp8 (OCP E4M3) and bf8 (OCP E5M2) GEMM kernel instances: 256x256x128 and
// 128x128x128 tiles; the latter also with OCP MX block scales.
#include "skg_inst_gemm_common.hpp"

namespace skg {
namespace {
template <int DT>
GemmInst f8_by_tile(int tile_id, int scale_mode) {
  const bool tensor = scale_mode == SKG_SCALE_TENSOR;
  if (tile_id == SKG_TILE_256x256x128) {
    if (scale_mode == SKG_SCALE_MX_E8M0) {
      typedef TileCfg<DT, 256, 256, 128, 2, 2, 32, 128, true> Cfg;
      return {&launch_instance<Cfg, GemmMxProblem<Cfg>>, &occupancy_instance<Cfg, GemmMxProblem<Cfg>>};
    }
    return gemm_inst::make<TileCfg<DT, 256, 256, 128, 2, 2, 32, 128>>(tensor);
  }
  if (tile_id == SKG_TILE_128x128x128) {
    if (scale_mode == SKG_SCALE_MX_E8M0) {
      typedef TileCfg<DT, 128, 128, 128, 2, 2, 32, 128, true> Cfg;
      return {&launch_instance<Cfg, GemmMxProblem<Cfg>>, &occupancy_instance<Cfg, GemmMxProblem<Cfg>>};
    }
    return gemm_inst::make<TileCfg<DT, 128, 128, 128, 2, 2, 32, 128>>(tensor);
  }
  return {nullptr, nullptr};
}
}  // namespace

GemmInst gemm_instance_f8(int tile_id, int dtype, int scale_mode) {
  if (dtype == SKG_F8E4M3) return f8_by_tile<DT_F8>(tile_id, scale_mode);
  if (dtype == SKG_F8E5M2) return f8_by_tile<DT_BF8>(tile_id, scale_mode);
  return {nullptr, nullptr};
}
hipError_t wait_timeouts_gemm_f8(uint32_t* out, bool reset) { return unit_wait_timeouts(out, reset); }
}  // namespace skg
