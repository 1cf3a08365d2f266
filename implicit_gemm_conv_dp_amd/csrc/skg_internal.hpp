// Host-side internals shared by the planner/validator (skg_host.cpp) and the
// launch code (skg_api.hip).  No device code here.
#pragma once

#include <cstdint>
#include <string>

#include "skgemm.h"

namespace skg {

// Per-thread reason for the last non-zero status.
void set_error(const std::string& msg);
void clear_error();

// Returns -2 after recording msg.
int unsupported(const std::string& msg);
// Returns -1 after recording msg.
int hip_failure(const std::string& msg);

struct TileDesc {
  int tm, tn, tk, n_waves;
  int gemm_mask;   // 1 << skg_dtype accepted as GEMM A/B
  int wgrad_mask;  // 1 << skg_dtype accepted as wgrad X/dY
  int conv_mask;   // 1 << skg_dtype accepted for forward conv / dgrad
  int group_block; // block-diagonal wgrad tile: whole 16-channel groups per tile (0: dense)
};

const TileDesc* tile_desc(int tile_id);

// Fix-ups whose CTAs hand partials on through flags (flags + partials in the
// workspace, every stream-K CTA resident at once).
inline bool handoff_reduction(int r) {
  return r == SKG_RED_LINEAR || r == SKG_RED_TREE || r == SKG_RED_SCATTER;
}
// A resolved reduction (AUTO excluded).
inline bool known_reduction(int r) {
  return (r >= SKG_RED_LINEAR && r <= SKG_RED_WORKSPACE) || r == SKG_RED_SCATTER;
}
// Every stream-K CTA holds one whole slice of one tile.
inline bool whole_slices(const skg_plan_t& p) {
  return p.sk_ctas > 0 && p.extra_iters == 0 && p.iters_per_tile % p.iters_per_sk_cta == 0 &&
         p.sk_ctas == p.sk_tiles * (p.iters_per_tile / p.iters_per_sk_cta);
}

int elem_bytes(int dtype);

// GEMM-shaped view of a problem: what the partitioner needs.
struct GemmShape {
  int64_t tiles_m, tiles_n, iters_per_tile;
};

// Resolves the plan of a GEMM-shaped problem.  pool_default_cus /
// resident_per_cu are only read when ctas == -1.
int make_plan(const GemmShape& g, const TileDesc& t, int mode, int reduction,
              int ctas, int num_cus, int resident_per_cu, skg_plan_t* out);
// make_plan after resolving SKG_MODE_AUTO / SKG_MODE_SPLITK / SKG_RED_AUTO;
// sk_order is already resolved (resolve_sk_order) and copied into the plan.
int plan_launch(const GemmShape& g, const TileDesc& t, int mode, int reduction,
                int ctas, int sk_order, int num_cus, int resident_per_cu, skg_plan_t* out);
// SKG_SK_ORDER_AUTO -> XCD for wgrad, BLOCK for GEMM; others unchanged.
int resolve_sk_order(int requested, bool wgrad);

// Argument checks that need no device (a0 of the hot path).
int validate_gemm(const skg_gemm_args_t* a);
int validate_wgrad(const skg_wgrad_args_t* a);
int validate_conv(const skg_conv_args_t* a, bool dgrad);

GemmShape gemm_shape(const skg_gemm_args_t* a, const TileDesc& t);
GemmShape wgrad_shape(const skg_wgrad_args_t* a, const TileDesc& t);
GemmShape conv_shape(const skg_conv_args_t* a, const TileDesc& t, bool dgrad);
// Bytes of the per-group transposed filter a dgrad run writes into the
// workspace after the fix-up region (multiple of 256).
int64_t dgrad_filter_bytes(const skg_conv_args_t* a);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Stride phases of the input gradient, row phase major: phase (a, b) holds
// the pixels with (h + pad_h) mod stride_h == a and (w + pad_w) mod
// stride_w == b (rows h0, h0 + stride_h, ..., hc of them; columns w0, ...,
// wc) and meets exactly the taps r = a + stride_h * ri (ri < rc), s = b +
// stride_w * si (si < sc).  Returns the number of phases written to out.
struct DgradPhase {
  int a, b, h0, w0, hc, wc, rc, sc;
};
inline int dgrad_phases(const skg_conv_args_t* c, DgradPhase* out) {
  int n = 0;
  for (int a = 0; a < c->stride_h; ++a)
    for (int b = 0; b < c->stride_w; ++b) {
      DgradPhase p;
      p.a = a;
      p.b = b;
      p.h0 = ((a - c->pad_h) % c->stride_h + c->stride_h) % c->stride_h;
      p.w0 = ((b - c->pad_w) % c->stride_w + c->stride_w) % c->stride_w;
      p.hc = c->h > p.h0 ? (int)ceil_div(c->h - p.h0, c->stride_h) : 0;
      p.wc = c->w > p.w0 ? (int)ceil_div(c->w - p.w0, c->stride_w) : 0;
      p.rc = c->r > a ? (int)ceil_div(c->r - a, c->stride_h) : 0;
      p.sc = c->s > b ? (int)ceil_div(c->s - b, c->stride_w) : 0;
      out[n++] = p;
    }
  return n;
}
// Stride phases a block-diagonal dgrad can carry.
constexpr int kMaxDgradPhases = 16;

}  // namespace skg
