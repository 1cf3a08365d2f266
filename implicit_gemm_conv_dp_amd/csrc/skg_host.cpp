// Host planner, validator and tile table of the stream-K engine.
//
// The partition follows rocm-libraries PR #13151 ("feat(rocke): stream-K for
// implicit-GEMM conv wgrad"): Technical Details (Partitioner), the commit
// adding the iteration partitioner (data-parallel waves of whole tiles, the
// remainder's MAC iterations as contiguous balanced ranges that may straddle
// tiles, the plan resolved once and returned by value), review item 1 (the
// iterations-per-CTA clamp), review item 2 (one flag per CTA and wave), the
// commits sizing the default pool, and the bot comment on automatic selection
// (a remainder with fewer iterations than the pool gives no stream-K CTAs).
#include <climits>
#include <cstring>

#include <algorithm>

#include "skg_internal.hpp"

namespace skg {

namespace {
thread_local std::string g_last_error;

constexpr int M_F16 = 1 << SKG_F16;
constexpr int M_BF16 = 1 << SKG_BF16;
constexpr int M_F8 = 1 << SKG_F8E4M3 | 1 << SKG_F8E5M2;

// Must agree with the kernel instances compiled in skg_api.hip.
const TileDesc kTiles[SKG_TILE_COUNT] = {
    /* 128x128x32  */ {128, 128, 32, 4, M_F16 | M_BF16, M_F16 | M_BF16, 0},
    /* 256x256x64  */ {256, 256, 64, 4, M_F16 | M_BF16, M_F16 | M_BF16, M_F16 | M_BF16},
    /* 256x256x128 */ {256, 256, 128, 4, M_F8, 0, 0},
    /* 32x64x64    */ {32, 64, 64, 4, 0, M_F16 | M_BF16, 0},
    /* 128x128x64  */ {128, 128, 64, 4, M_F16 | M_BF16, M_F16 | M_BF16, M_F16 | M_BF16},
    /* 256x128x64  */ {256, 128, 64, 4, M_F16 | M_BF16, M_F16 | M_BF16, M_F16 | M_BF16},
    /* 128x128x128 */ {128, 128, 128, 4, M_F8, 0, 0},
    /* 64x144x32   */ {64, 144, 32, 4, 0, M_F16 | M_BF16, 0, 4},
    /* 128x64x32   */ {128, 64, 32, 4, 0, 0, M_F16 | M_BF16, 4},
};

// Offsets inside one buffer are 32-bit on the device (buffer resources).
constexpr int64_t kMaxBufferBytes = INT32_MAX;
}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
int unsupported(const std::string& msg) {
  set_error(msg);
  return SKG_ERR_UNSUPPORTED;
}
int hip_failure(const std::string& msg) {
  set_error(msg);
  return SKG_ERR_HIP;
}

const TileDesc* tile_desc(int tile_id) {
  if (tile_id < 0 || tile_id >= SKG_TILE_COUNT) return nullptr;
  return &kTiles[tile_id];
}

int elem_bytes(int dtype) {
  switch (dtype) {
    case SKG_F16:
    case SKG_BF16:
      return 2;
    case SKG_F8E4M3:
    case SKG_F8E5M2:
      return 1;
    case SKG_F32:
      return 4;
    default:
      return 0;
  }
}

// Automatic launch choice and the split-K comparator (PR #13151, commit
// making stream-K the "auto" default and its review follow-up): stream-K
// for tiles that leave a ragged wave of the pool over a long reduction
// when that partition has stream-K CTAs, split-K otherwise; "auto"
// reduction = workspace.  Split-K runs as dp_sk with a pool of tiles x
// slices; default slices fill the pool but stay at least kLongReduction
// iterations long (a slice's fp32 partial tile round trip costs about as
// many bytes as that many iterations' operand tiles).  Same steps as the
// oracle's resolve_launch.
constexpr int64_t kLongReduction = 8;

static int resolve_launch(const GemmShape& g, int& mode, int& reduction, int& ctas, int num_cus,
                          int resident_per_cu, int& slices) {
  slices = 1;
  if (reduction == SKG_RED_AUTO) reduction = SKG_RED_WORKSPACE;
  if (!known_reduction(reduction)) return unsupported("unknown stream-K reduction");
  if (ctas == 0 || ctas < -1) return unsupported("streamk ctas must be -1 or positive");
  if (g.tiles_m <= 0 || g.tiles_n <= 0 || g.iters_per_tile <= 0) return unsupported("empty problem");
  const int64_t T = g.tiles_m * g.tiles_n, ipt = g.iters_per_tile;
  auto pool = [&](int64_t* P) {
    if (ctas > 0) {
      *P = ctas;
      return SKG_OK;
    }
    int32_t d = 0;
    const int rc = skg_default_pool(reduction, num_cus, resident_per_cu, &d);
    *P = d;
    return rc;
  };
  int64_t S = 1;
  if (mode == SKG_MODE_AUTO) {
    int64_t P = 0;
    int rc = pool(&P);
    if (rc) return rc;
    if (T % P != 0 && T < 2 * P && ipt >= kLongReduction && (T - (T / P) * P) * ipt >= P) {
      mode = SKG_MODE_DP_SK;
      ctas = (int)P;
      return SKG_OK;
    }
    S = std::min<int64_t>(P / T, ipt / kLongReduction);  // split-K filling the same pool
  } else if (mode == SKG_MODE_SPLITK) {
    if (ctas == -1) {
      int64_t P = 0;
      int rc = pool(&P);
      if (rc) return rc;
      S = std::min<int64_t>(P / T, ipt / kLongReduction);
    } else {
      S = ctas;
    }
  }
  if (mode == SKG_MODE_AUTO || mode == SKG_MODE_SPLITK) {
    if (S > ipt) S = ipt;
    if (S < 1) S = 1;
    if (T * S > INT32_MAX) return unsupported("too many split-K CTAs");
    slices = (int)S;
    mode = S == 1 ? SKG_MODE_DP : SKG_MODE_DP_SK;
    ctas = (int)(T * S);
  }
  return SKG_OK;
}

int resolve_sk_order(int requested, bool wgrad) {
  if (requested != SKG_SK_ORDER_AUTO) return requested;
  return wgrad ? SKG_SK_ORDER_KMAJOR : SKG_SK_ORDER_BLOCK;
}

int plan_launch(const GemmShape& g, const TileDesc& t, int mode, int reduction, int ctas,
                int sk_order, int num_cus, int resident_per_cu, skg_plan_t* out) {
  const int requested = mode;
  int slices = 1;
  int rc = resolve_launch(g, mode, reduction, ctas, num_cus, resident_per_cu, slices);
  if (rc) return rc;
  rc = make_plan(g, t, mode, reduction, ctas, num_cus, resident_per_cu, out);
  if (rc) return rc;
  out->requested_mode = requested;
  out->slices = slices;
  // Slice-major order needs every stream-K CTA to hold one whole slice of
  // one tile; otherwise the XCD runs are taken over the CTAs themselves.
  if (sk_order == SKG_SK_ORDER_KMAJOR && !whole_slices(*out)) sk_order = SKG_SK_ORDER_XCD;
  out->sk_order = sk_order;
  if (reduction == SKG_RED_SCATTER && out->sk_ctas > 0 && !whole_slices(*out))
    return unsupported("the scatter fix-up needs every stream-K CTA to hold one whole slice of "
                       "one tile (split-K with the slice count dividing the iterations per tile)");
  return SKG_OK;
}

// `requested`: the caller's knobs (AUTO / SPLITK allowed); otherwise the
// resolved launch the planner plans.
static int check_launch_knobs(int mode, int reduction, int ctas, bool requested) {
  const int max_mode = requested ? SKG_MODE_AUTO : SKG_MODE_PERSISTENT;
  if (mode < SKG_MODE_DP || mode > max_mode) return unsupported("unknown launch mode");
  if (!known_reduction(reduction) && !(requested && reduction == SKG_RED_AUTO))
    return unsupported("unknown stream-K reduction");
  if (ctas == 0 || ctas < -1) return unsupported("streamk ctas must be -1 or positive");
  return SKG_OK;
}

int make_plan(const GemmShape& g, const TileDesc& t, int mode, int reduction, int ctas,
              int num_cus, int resident_per_cu, skg_plan_t* out) {
  int rc = check_launch_knobs(mode, reduction, ctas, false);
  if (rc) return rc;
  if (g.tiles_m <= 0 || g.tiles_n <= 0 || g.iters_per_tile <= 0) return unsupported("empty problem");
  skg_plan_t p;
  std::memset(&p, 0, sizeof(p));
  p.tm = t.tm;
  p.tn = t.tn;
  p.tk = t.tk;
  p.n_waves = t.n_waves;
  p.mode = mode;
  p.reduction = reduction;
  // 1. Tiles.
  p.tiles_m = g.tiles_m;
  p.tiles_n = g.tiles_n;
  p.tiles = g.tiles_m * g.tiles_n;
  p.iters_per_tile = g.iters_per_tile;
  const int64_t T = p.tiles, ipt = p.iters_per_tile;
  if (T > INT32_MAX / 2 || ipt > INT32_MAX / 2 || T * ipt > INT32_MAX)
    return unsupported("problem has too many MAC iterations");
  // 2. Pool.
  int64_t P;
  if (ctas == -1) {
    int32_t d = 0;
    rc = skg_default_pool(reduction, num_cus, resident_per_cu, &d);
    if (rc) return rc;
    P = d;
  } else {
    P = ctas;
  }
  p.pool = P;
  // 3./4. Data-parallel / stream-K split.
  int64_t dp_tiles, sk_tiles, sk_ctas;
  if (mode == SKG_MODE_DP) {
    dp_tiles = T;
    sk_tiles = 0;
    sk_ctas = 0;
  } else {
    dp_tiles = (T / P) * P;
    sk_tiles = T - dp_tiles;
    if (sk_tiles == 0 || sk_tiles * ipt < P) {
      dp_tiles = T;
      sk_tiles = 0;
      sk_ctas = 0;
    } else {
      sk_ctas = P;
    }
  }
  p.dp_tiles = dp_tiles;
  p.sk_tiles = sk_tiles;
  p.sk_ctas = sk_ctas;
  p.sk_iters = sk_tiles * ipt;
  // 5. Iterations per stream-K CTA, clamped so no divisor is ever zero.
  const int64_t ipc_raw = sk_ctas ? p.sk_iters / sk_ctas : 0;
  p.extra_iters = sk_ctas ? p.sk_iters % sk_ctas : 0;
  p.iters_per_sk_cta = ipc_raw > 1 ? ipc_raw : 1;
  // 9. Grid.
  if (mode == SKG_MODE_DP)
    p.grid = T;
  else if (mode == SKG_MODE_DP_SK)
    p.grid = sk_ctas + dp_tiles;
  else
    p.grid = sk_ctas ? P : (P < T ? P : T);
  if (p.grid > INT32_MAX) return unsupported("grid too large");
  // 8. Most contributors to one stream-K tile; the owner of a tile is the
  // CTA running its first iteration.
  const int64_t ipc = p.iters_per_sk_cta, extra = p.extra_iters;
  auto cta_of = [&](int64_t it) {
    const int64_t boundary = extra * (ipc + 1);
    return it < boundary ? it / (ipc + 1) : extra + (it - boundary) / ipc;
  };
  int64_t max_contrib = 1;
  for (int64_t s = 0; s < sk_tiles; ++s) {
    const int64_t n = cta_of((s + 1) * ipt - 1) - cta_of(s * ipt) + 1;
    if (n > max_contrib) max_contrib = n;
  }
  p.max_contrib = max_contrib;
  p.linear_partners = max_contrib - 1;
  int64_t rounds = 0;
  while ((int64_t(1) << rounds) < max_contrib) ++rounds;
  p.tree_rounds = rounds;
  // 10. Bytes: flags (one i32 per CTA and wave, 256-byte aligned) then one
  // fp32 partial tile per stream-K CTA; or the fp32 scratch of the workspace
  // reduction (one tile per stream-K tile).
  if (sk_ctas && handoff_reduction(reduction)) {
    p.flags_bytes = ceil_div(4 * sk_ctas * t.n_waves, 256) * 256;
    p.partials_bytes = sk_ctas * int64_t(t.tm) * t.tn * 4;
    p.workspace_bytes = p.flags_bytes + p.partials_bytes;
  } else if (sk_ctas && reduction == SKG_RED_WORKSPACE) {
    p.workspace_bytes = sk_tiles * int64_t(t.tm) * t.tn * 4;
  }
  *out = p;
  return SKG_OK;
}

GemmShape gemm_shape(const skg_gemm_args_t* a, const TileDesc& t) {
  return {ceil_div(a->M, t.tm), ceil_div(a->N, t.tn), ceil_div(a->K, t.tk)};
}

GemmShape wgrad_shape(const skg_wgrad_args_t* a, const TileDesc& t) {
  const int64_t ho = (int64_t(a->h) + 2 * a->pad_h - a->r) / a->stride_h + 1;
  const int64_t wo = (int64_t(a->w) + 2 * a->pad_w - a->s) / a->stride_w + 1;
  const int64_t kpg = a->k / a->groups, cpg = a->c / a->groups;
  // Groups fold into GEMM-M: dense tiles are counted per group, a
  // block-diagonal tile holds group_block whole groups.
  const int64_t tiles_m = t.group_block ? ceil_div(a->groups, t.group_block)
                                        : int64_t(a->groups) * ceil_div(kpg, t.tm);
  return {tiles_m, ceil_div(cpg * a->r * a->s, t.tn), ceil_div(int64_t(a->n) * ho * wo, t.tk)};
}

GemmShape conv_shape(const skg_conv_args_t* a, const TileDesc& t, bool dgrad) {
  const int64_t ho = (int64_t(a->h) + 2 * a->pad_h - a->r) / a->stride_h + 1;
  const int64_t wo = (int64_t(a->w) + 2 * a->pad_w - a->s) / a->stride_w + 1;
  const int64_t kpg = a->k / a->groups, cpg = a->c / a->groups;
  if (t.group_block) {
    // Block-diagonal: group_block whole groups per N tile, the reduction
    // per group (16 channels at every tap).  dgrad runs GEMM-M stride phase
    // by phase, each with its own taps: M tiles per phase, the iterations of
    // the phase with the most taps.
    if (!dgrad)
      return {ceil_div(int64_t(a->n) * ho * wo, t.tm), ceil_div(a->groups, t.group_block),
              ceil_div(a->r * a->s * 16, t.tk)};
    DgradPhase ph[kMaxDgradPhases];
    const int np = dgrad_phases(a, ph);
    int64_t tiles_m = 0, taps = 0;
    for (int i = 0; i < np; ++i) {
      tiles_m += ceil_div(int64_t(a->n) * ph[i].hc * ph[i].wc, t.tm);
      taps = std::max<int64_t>(taps, int64_t(ph[i].rc) * ph[i].sc);
    }
    return {tiles_m, ceil_div(a->groups, t.group_block), std::max<int64_t>(1, ceil_div(taps * 16, t.tk))};
  }
  // Groups fold into GEMM-N with the tile count per group.
  if (!dgrad)
    return {ceil_div(int64_t(a->n) * ho * wo, t.tm), int64_t(a->groups) * ceil_div(kpg, t.tn),
            ceil_div(a->r * a->s * cpg, t.tk)};
  return {ceil_div(int64_t(a->n) * a->h * a->w, t.tm), int64_t(a->groups) * ceil_div(cpg, t.tn),
          ceil_div(a->r * a->s * kpg, t.tk)};
}

int64_t dgrad_filter_bytes(const skg_conv_args_t* a) {
  return ceil_div(int64_t(a->k) * a->r * a->s * (a->c / a->groups) * 2, 256) * 256;
}

int validate_gemm(const skg_gemm_args_t* a) {
  if (!a) return unsupported("null arguments");
  const TileDesc* t = tile_desc(a->tile_id);
  if (!t) return unsupported("unknown tile id");
  if (a->dtype_ab != SKG_F16 && a->dtype_ab != SKG_BF16 && a->dtype_ab != SKG_F8E4M3 &&
      a->dtype_ab != SKG_F8E5M2)
    return unsupported("unsupported A/B dtype");
  if (a->scale_mode != SKG_SCALE_ROWCOL && a->scale_mode != SKG_SCALE_TENSOR &&
      a->scale_mode != SKG_SCALE_MX_E8M0)
    return unsupported("unknown scale mode");
  if (a->scale_mode == SKG_SCALE_MX_E8M0) {
    if (a->dtype_ab != SKG_F8E4M3 && a->dtype_ab != SKG_F8E5M2)
      return unsupported("MX block scales need fp8 or bf8 inputs");
    if (a->tile_id != SKG_TILE_128x128x128 && a->tile_id != SKG_TILE_256x256x128)
      return unsupported("MX block scales need the 128x128x128 or 256x256x128 tile");
    if (a->K % 128) return unsupported("MX block scales need K to be a multiple of 128");
  }
  if (a->sk_order < SKG_SK_ORDER_AUTO || a->sk_order > SKG_SK_ORDER_KMAJOR)
    return unsupported("unknown stream-K CTA order");
  if (a->dtype_c != SKG_F16 && a->dtype_c != SKG_BF16 && a->dtype_c != SKG_F32)
    return unsupported("unsupported C dtype");
  if (!(t->gemm_mask & (1 << a->dtype_ab))) return unsupported("tile has no GEMM instance for this A/B dtype");
  int rc = check_launch_knobs(a->mode, a->reduction, a->ctas, true);
  if (rc) return rc;
  if (a->reduction == SKG_RED_ATOMIC && a->dtype_c != SKG_F32)
    return unsupported("atomic reduction needs an fp32 output");
  if (a->M <= 0 || a->N <= 0 || a->K <= 0) return unsupported("M, N and K must be positive");
  if (a->M > INT32_MAX || a->N > INT32_MAX || a->K > INT32_MAX) return unsupported("dimension too large");
  if (a->lda < a->K || a->ldb < a->K || a->ldc < a->N) return unsupported("leading dimension too small");
  const int eb = elem_bytes(a->dtype_ab), ec = elem_bytes(a->dtype_c);
  if ((a->K * eb) % 16 || (a->lda * eb) % 16 || (a->ldb * eb) % 16)
    return unsupported("K, lda and ldb must be multiples of 16 bytes");
  if ((a->ldc * ec) % 16) return unsupported("ldc must be a multiple of 16 bytes");
  if (int64_t(t->tm) * a->lda * eb > kMaxBufferBytes || int64_t(t->tn) * a->ldb * eb > kMaxBufferBytes)
    return unsupported("row pitch too large for 32-bit tile offsets");
  return SKG_OK;
}

int validate_wgrad(const skg_wgrad_args_t* a) {
  if (!a) return unsupported("null arguments");
  const TileDesc* t = tile_desc(a->tile_id);
  if (!t) return unsupported("unknown tile id");
  if (a->dtype != SKG_F16 && a->dtype != SKG_BF16) return unsupported("unsupported wgrad dtype");
  if (a->sk_order < SKG_SK_ORDER_AUTO || a->sk_order > SKG_SK_ORDER_KMAJOR)
    return unsupported("unknown stream-K CTA order");
  if (!(t->wgrad_mask & (1 << a->dtype))) return unsupported("tile has no wgrad instance for this dtype");
  int rc = check_launch_knobs(a->mode, a->reduction, a->ctas, true);
  if (rc) return rc;
  if (a->n <= 0 || a->h <= 0 || a->w <= 0 || a->c <= 0 || a->k <= 0 || a->r <= 0 || a->s <= 0)
    return unsupported("sizes must be positive");
  if (a->stride_h <= 0 || a->stride_w <= 0 || a->pad_h < 0 || a->pad_w < 0)
    return unsupported("bad stride or padding");
  if (a->groups <= 0 || a->c % a->groups || a->k % a->groups)
    return unsupported("groups must divide C and K");
  const int64_t cpg = a->c / a->groups, kpg = a->k / a->groups;
  if (cpg % 8 || kpg % 8) return unsupported("channels per group must be multiples of 8");
  if (t->group_block && (cpg != 16 || kpg != 16))
    return unsupported("the block-diagonal tile needs 16 input and 16 output channels per group");
  const int64_t ho = (int64_t(a->h) + 2 * a->pad_h - a->r) / a->stride_h + 1;
  const int64_t wo = (int64_t(a->w) + 2 * a->pad_w - a->s) / a->stride_w + 1;
  if (int64_t(a->h) + 2 * a->pad_h < a->r || int64_t(a->w) + 2 * a->pad_w < a->s || ho <= 0 || wo <= 0)
    return unsupported("empty output image");
  const int eb = elem_bytes(a->dtype);
  const int64_t xbytes = int64_t(a->n) * a->h * a->w * a->c * eb;
  const int64_t dybytes = int64_t(a->n) * ho * wo * a->k * eb;
  if (xbytes > kMaxBufferBytes || dybytes > kMaxBufferBytes)
    return unsupported("activation tensor too large for 32-bit offsets");
  if (int64_t(a->k) * a->r * a->s * cpg * 4 > kMaxBufferBytes) return unsupported("filter too large");
  return SKG_OK;
}

int validate_conv(const skg_conv_args_t* a, bool dgrad) {
  if (!a) return unsupported("null arguments");
  const TileDesc* t = tile_desc(a->tile_id);
  if (!t) return unsupported("unknown tile id");
  if (a->dtype != SKG_F16 && a->dtype != SKG_BF16) return unsupported("unsupported convolution dtype");
  if (a->dtype_out != SKG_F16 && a->dtype_out != SKG_BF16 && a->dtype_out != SKG_F32)
    return unsupported("unsupported output dtype");
  if (a->sk_order < SKG_SK_ORDER_AUTO || a->sk_order > SKG_SK_ORDER_KMAJOR)
    return unsupported("unknown stream-K CTA order");
  if (!(t->conv_mask & (1 << a->dtype))) return unsupported("tile has no convolution instance for this dtype");
  int rc = check_launch_knobs(a->mode, a->reduction, a->ctas, true);
  if (rc) return rc;
  if (a->reduction == SKG_RED_ATOMIC && a->dtype_out != SKG_F32)
    return unsupported("atomic reduction needs an fp32 output");
  if (a->n <= 0 || a->h <= 0 || a->w <= 0 || a->c <= 0 || a->k <= 0 || a->r <= 0 || a->s <= 0)
    return unsupported("sizes must be positive");
  if (a->stride_h <= 0 || a->stride_w <= 0 || a->pad_h < 0 || a->pad_w < 0)
    return unsupported("bad stride or padding");
  if (a->groups <= 0 || a->c % a->groups || a->k % a->groups)
    return unsupported("groups must divide C and K");
  const int64_t cpg = a->c / a->groups, kpg = a->k / a->groups;
  if (cpg % 8 || kpg % 8) return unsupported("channels per group must be multiples of 8");
  if (t->group_block && (cpg != 16 || kpg != 16))
    return unsupported("the block-diagonal tile needs 16 input and 16 output channels per group");
  if (t->group_block && dgrad && int64_t(a->stride_h) * a->stride_w > kMaxDgradPhases)
    return unsupported("the block-diagonal dgrad tile takes strides with at most 16 phases (stride_h * stride_w)");
  const int64_t ho = (int64_t(a->h) + 2 * a->pad_h - a->r) / a->stride_h + 1;
  const int64_t wo = (int64_t(a->w) + 2 * a->pad_w - a->s) / a->stride_w + 1;
  if (int64_t(a->h) + 2 * a->pad_h < a->r || int64_t(a->w) + 2 * a->pad_w < a->s || ho <= 0 || wo <= 0)
    return unsupported("empty output image");
  const int eb = elem_bytes(a->dtype), eo = elem_bytes(a->dtype_out);
  const int64_t xpix = int64_t(a->n) * a->h * a->w, ypix = int64_t(a->n) * ho * wo;
  const int64_t act = (dgrad ? ypix * a->k : xpix * a->c) * eb;
  const int64_t out = (dgrad ? xpix * a->c : ypix * a->k) * eo;
  if (act > kMaxBufferBytes || out > kMaxBufferBytes)
    return unsupported("activation tensor too large for 32-bit offsets");
  if (int64_t(a->k) * a->r * a->s * cpg * eb > kMaxBufferBytes) return unsupported("filter too large");
  return SKG_OK;
}

}  // namespace skg

using namespace skg;

extern "C" {

const char* skg_last_error(void) { return g_last_error.c_str(); }

int skg_tile_info(int32_t tile_id, skg_tile_info_t* out) {
  clear_error();
  const TileDesc* t = tile_desc(tile_id);
  if (!t) return unsupported("unknown tile id");
  if (!out) return unsupported("null output");
  out->tm = t->tm;
  out->tn = t->tn;
  out->tk = t->tk;
  out->n_waves = t->n_waves;
  out->gemm_dtypes = t->gemm_mask;
  out->wgrad_dtypes = t->wgrad_mask;
  out->conv_dtypes = t->conv_mask;
  out->group_block = t->group_block;
  return SKG_OK;
}

int skg_default_pool(int32_t reduction, int32_t num_cus, int32_t resident_per_cu, int32_t* out) {
  if (!known_reduction(reduction)) return unsupported("unknown stream-K reduction");
  if (num_cus <= 0 || resident_per_cu <= 0) return unsupported("device has no resident capacity");
  if (!out) return unsupported("null output");
  const int per_cu = handoff_reduction(reduction) ? 1 : 4;
  *out = num_cus * (per_cu < resident_per_cu ? per_cu : resident_per_cu);
  return SKG_OK;
}

}  // extern "C"
