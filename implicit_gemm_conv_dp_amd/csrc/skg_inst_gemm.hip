// GEMM kernel instances (rcr).  Tile shapes per enum skg_tile.
#include "skg_launch.hpp"
#include "skgemm.h"

namespace skg {

namespace {
template <class Cfg>
GemmInst make() {
  return {&launch_instance<Cfg, GemmProblem<Cfg>>, &occupancy_instance<Cfg, GemmProblem<Cfg>>};
}
template <int DT>
GemmInst by_tile(int tile_id) {
  switch (tile_id) {
    case SKG_TILE_128x128x32: return make<TileCfg<DT, 128, 128, 32, 2, 2, 32>>();
    case SKG_TILE_256x256x64: return make<TileCfg<DT, 256, 256, 64, 2, 2, 32>>();
    case SKG_TILE_128x128x64: return make<TileCfg<DT, 128, 128, 64, 2, 2, 32>>();
    case SKG_TILE_256x128x64: return make<TileCfg<DT, 256, 128, 64, 2, 2, 32>>();
    default: return {nullptr, nullptr};
  }
}
}  // namespace

GemmInst gemm_instance(int tile_id, int dtype) {
  if (dtype == SKG_F16) return by_tile<DT_F16>(tile_id);
  if (dtype == SKG_BF16) return by_tile<DT_BF16>(tile_id);
  if (dtype == SKG_F8E4M3 && tile_id == SKG_TILE_256x256x128)
    return make<TileCfg<DT_F8, 256, 256, 128, 2, 2, 32, 128>>();
  return {nullptr, nullptr};
}

}  // namespace skg
