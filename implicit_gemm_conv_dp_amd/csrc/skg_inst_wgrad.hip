// Conv wgrad (implicit GEMM) kernel instances.  Tile shapes per enum skg_tile.
#include "skg_launch.hpp"
#include "skgemm.h"

namespace skg {

namespace {
template <class Cfg>
WgradInst make() {
  return {&launch_instance<Cfg, WgradProblem<Cfg>>, &occupancy_instance<Cfg, WgradProblem<Cfg>>};
}
template <class Cfg>
WgradInst make_bd() {
  return {&launch_instance<Cfg, WgradBdProblem<Cfg>>, &occupancy_instance<Cfg, WgradBdProblem<Cfg>>};
}
template <int DT>
WgradInst by_tile(int tile_id) {
  switch (tile_id) {
    case SKG_TILE_64x144x32: return make_bd<TileCfg<DT, 64, 144, 32, 4, 1, 16, 64, false, 4>>();
    case SKG_TILE_128x128x32: return make<TileCfg<DT, 128, 128, 32, 2, 2, 32>>();
    case SKG_TILE_32x64x64: return make<TileCfg<DT, 32, 64, 64, 2, 2, 16>>();
    case SKG_TILE_128x128x64: return make<TileCfg<DT, 128, 128, 64, 2, 2, 32>>();
    case SKG_TILE_256x128x64: return make<TileCfg<DT, 256, 128, 64, 2, 2, 32>>();
    case SKG_TILE_256x256x64: return make<TileCfg<DT, 256, 256, 64, 2, 2, 32>>();
    default: return {nullptr, nullptr};
  }
}
}  // namespace

WgradInst wgrad_instance(int tile_id, int dtype) {
  if (dtype == SKG_F16) return by_tile<DT_F16>(tile_id);
  if (dtype == SKG_BF16) return by_tile<DT_BF16>(tile_id);
  return {nullptr, nullptr};
}

hipError_t wait_timeouts_wgrad(uint32_t* out, bool reset) { return unit_wait_timeouts(out, reset); }
}  // namespace skg
