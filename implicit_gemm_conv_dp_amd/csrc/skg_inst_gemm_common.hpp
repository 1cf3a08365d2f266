// Shared pieces of the GEMM instance units.
#pragma once

#include "skg_launch.hpp"
#include "skgemm.h"

namespace skg {
namespace gemm_inst {

template <class Cfg, bool TENSOR>
GemmInst make() {
  typedef GemmProblem<Cfg, TENSOR> Prob;
  return {&launch_instance<Cfg, Prob>, &occupancy_instance<Cfg, Prob>};
}

template <class Cfg>
GemmInst make(bool tensor_scales) {
  return tensor_scales ? make<Cfg, true>() : make<Cfg, false>();
}

// fp16 / bf16 tile shapes per enum skg_tile.
template <int DT>
GemmInst by_tile(int tile_id, bool tensor_scales) {
  switch (tile_id) {
    case SKG_TILE_128x128x32: return make<TileCfg<DT, 128, 128, 32, 2, 2, 32>>(tensor_scales);
    case SKG_TILE_256x256x64: return make<TileCfg<DT, 256, 256, 64, 2, 2, 32>>(tensor_scales);
    case SKG_TILE_128x128x64: return make<TileCfg<DT, 128, 128, 64, 2, 2, 32>>(tensor_scales);
    case SKG_TILE_256x128x64: return make<TileCfg<DT, 256, 128, 64, 2, 2, 32>>(tensor_scales);
    default: return {nullptr, nullptr};
  }
}

}  // namespace gemm_inst
}  // namespace skg
