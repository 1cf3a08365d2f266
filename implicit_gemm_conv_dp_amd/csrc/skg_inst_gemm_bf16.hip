// bf16 GEMM kernel instances.
#include "skg_inst_gemm_common.hpp"

namespace skg {
GemmInst gemm_instance_bf16(int tile_id, bool tensor_scales) {
  return gemm_inst::by_tile<DT_BF16>(tile_id, tensor_scales);
}
}  // namespace skg
