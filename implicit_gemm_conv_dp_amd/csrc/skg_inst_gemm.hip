// GEMM kernel instances (rcr): dispatch by input type.  Each type's
// instances live in a unit of their own so that they compile in parallel.
#include "skg_launch.hpp"
#include "skgemm.h"

namespace skg {

GemmInst gemm_instance(int tile_id, int dtype, bool tensor_scales) {
  switch (dtype) {
    case SKG_F16: return gemm_instance_f16(tile_id, tensor_scales);
    case SKG_BF16: return gemm_instance_bf16(tile_id, tensor_scales);
    case SKG_F8E4M3:
    case SKG_F8E5M2: return gemm_instance_f8(tile_id, dtype, tensor_scales);
    default: return {nullptr, nullptr};
  }
}

}  // namespace skg
