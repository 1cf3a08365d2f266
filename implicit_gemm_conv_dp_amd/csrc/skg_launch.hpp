// Kernel instance table shared by the launch code and the instance units.
#pragma once

#include <hip/hip_runtime.h>

#include "skg_conv.hpp"
#include "skg_kernels.hpp"

namespace skg {

struct GemmInst {
  hipError_t (*launch)(const GemmParams&, const KPlan&, const Scratch&, hipStream_t, hipEvent_t,
                       hipEvent_t);
  hipError_t (*occupancy)(int*);
};

struct WgradInst {
  hipError_t (*launch)(const WgradParams&, const KPlan&, const Scratch&, hipStream_t, hipEvent_t,
                       hipEvent_t);
  hipError_t (*occupancy)(int*);
};

struct ConvInst {
  hipError_t (*launch)(const ConvParams&, const KPlan&, const Scratch&, hipStream_t, hipEvent_t,
                       hipEvent_t);
  hipError_t (*occupancy)(int*);
};

// {nullptr, nullptr} when the (tile, dtype, scale mode) has no compiled
// instance; scale_mode is an enum skg_scale_mode.
GemmInst gemm_instance(int tile_id, int dtype, int scale_mode);
GemmInst gemm_instance_f16(int tile_id, bool tensor_scales);
GemmInst gemm_instance_bf16(int tile_id, bool tensor_scales);
GemmInst gemm_instance_f8(int tile_id, int dtype, int scale_mode);
WgradInst wgrad_instance(int tile_id, int dtype);
ConvInst fwd_instance(int tile_id, int dtype);
ConvInst dgrad_instance(int tile_id, int dtype);

// Flag-wait give-ups counted by the kernels of one instance unit (read, and
// reset to zero when `reset`); skg_fixup_timeouts sums the units.
hipError_t wait_timeouts_gemm_f16(uint32_t* out, bool reset);
hipError_t wait_timeouts_gemm_bf16(uint32_t* out, bool reset);
hipError_t wait_timeouts_gemm_f8(uint32_t* out, bool reset);
hipError_t wait_timeouts_wgrad(uint32_t* out, bool reset);
hipError_t wait_timeouts_fwd(uint32_t* out, bool reset);
hipError_t wait_timeouts_dgrad(uint32_t* out, bool reset);

// The calling unit's own counter (each unit has its copy of the symbol).
static inline hipError_t unit_wait_timeouts(uint32_t* out, bool reset) {
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_skg_wait_timeouts), sizeof(uint32_t), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess || !reset) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_skg_wait_timeouts), &zero, sizeof(uint32_t), 0,
                           hipMemcpyHostToDevice);
}

// Launches the stream-K kernel of the plan's fix-up family (bracketed by ev0
// / ev1 when they are set) and, for the workspace reduction, the second
// stage.
template <class Cfg, class Prob>
hipError_t launch_instance(const typename Prob::Params& prm, const KPlan& p, const Scratch& s,
                           hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e;
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  // A plan without stream-K CTAs runs no fix-up, whatever reduction it
  // names, so it may take either family.  It takes the atomic one, whose
  // fix-up code is the smaller: fewer registers live around the copy-out
  // and fewer spilled (grouped forward / dgrad 10-18 % faster, fp8 GEMM
  // 2 %), except on the MX-scaled tiles, where that family spills more.
  const bool sk_atomic = (p.reduction == RED_ATOMIC || p.reduction == RED_WORKSPACE) && p.sk_ctas > 0;
  const bool dp_only = p.sk_ctas == 0;
  if (sk_atomic || (dp_only && !Cfg::MX))
    hipLaunchKernelGGL((sk_kernel<Cfg, Prob, FIX_ATOMIC>), dim3(p.grid), dim3(Cfg::THREADS), 0, st,
                       prm, p, s);
  else
    hipLaunchKernelGGL((sk_kernel<Cfg, Prob, FIX_HANDOFF>), dim3(p.grid), dim3(Cfg::THREADS), 0, st,
                       prm, p, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, st)) != hipSuccess) return e;
  if (p.reduction == RED_WORKSPACE && p.sk_tiles > 0) {
    const dim3 g2(p.sk_tiles, (Cfg::TM * Cfg::TN + 1023) / 1024);
    hipLaunchKernelGGL((stage2_kernel<Cfg, Prob>), g2, dim3(256), 0, st, prm, p, s);
    e = hipGetLastError();
  }
  return e;
}

template <class Cfg, class Prob>
hipError_t occupancy_instance(int* out) {
  // Both families are built with the same launch bounds and LDS; the
  // smaller of the two residencies is reported.
  int h = 0, a = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&h, sk_kernel<Cfg, Prob, FIX_HANDOFF>,
                                                              Cfg::THREADS, 0);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, sk_kernel<Cfg, Prob, FIX_ATOMIC>, Cfg::THREADS, 0);
  *out = h < a ? h : a;
  return e;
}

}  // namespace skg
