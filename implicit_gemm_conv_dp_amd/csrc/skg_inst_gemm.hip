// GEMM kernel instances (rcr): dispatch by input type.  Each type's
// instances live in a unit of their own so that they compile in parallel.
#include "skg_launch.hpp"
#include "skgemm.h"

namespace skg {

GemmInst gemm_instance(int tile_id, int dtype, int scale_mode) {
  const bool tensor = scale_mode == SKG_SCALE_TENSOR;
  switch (dtype) {
    case SKG_F16: return scale_mode == SKG_SCALE_MX_E8M0 ? GemmInst{nullptr, nullptr} : gemm_instance_f16(tile_id, tensor);
    case SKG_BF16: return scale_mode == SKG_SCALE_MX_E8M0 ? GemmInst{nullptr, nullptr} : gemm_instance_bf16(tile_id, tensor);
    case SKG_F8E4M3:
    case SKG_F8E5M2: return gemm_instance_f8(tile_id, dtype, scale_mode);
    default: return {nullptr, nullptr};
  }
}

}  // namespace skg
