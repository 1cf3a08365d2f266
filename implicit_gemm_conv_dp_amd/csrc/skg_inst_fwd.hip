// Forward convolution kernel instances (implicit GEMM, 16-bit inputs): the
// tiles whose LDS rows are whole 128-byte lines.
#include "skg_launch.hpp"
#include "skgemm.h"

namespace skg {

namespace {
template <class Cfg>
ConvInst make() {
  typedef ConvProblem<Cfg, false> Prob;
  return {&launch_instance<Cfg, Prob>, &occupancy_instance<Cfg, Prob>};
}
template <class Cfg>
ConvInst make_bd() {
  typedef ConvBdProblem<Cfg, false> Prob;
  return {&launch_instance<Cfg, Prob>, &occupancy_instance<Cfg, Prob>};
}
template <int DT>
ConvInst by_tile(int tile_id) {
  switch (tile_id) {
    case SKG_TILE_128x64x32: return make_bd<TileCfg<DT, 128, 64, 32, 1, 4, 16, 64, false, 4, 2>>();
    case SKG_TILE_256x256x64: return make<TileCfg<DT, 256, 256, 64, 2, 2, 32>>();
    case SKG_TILE_128x128x64: return make<TileCfg<DT, 128, 128, 64, 2, 2, 32>>();
    case SKG_TILE_256x128x64: return make<TileCfg<DT, 256, 128, 64, 2, 2, 32>>();
    default: return {nullptr, nullptr};
  }
}
}  // namespace

ConvInst fwd_instance(int tile_id, int dtype) {
  if (dtype == SKG_F16) return by_tile<DT_F16>(tile_id);
  if (dtype == SKG_BF16) return by_tile<DT_BF16>(tile_id);
  return {nullptr, nullptr};
}

hipError_t wait_timeouts_fwd(uint32_t* out, bool reset) { return unit_wait_timeouts(out, reset); }
}  // namespace skg
