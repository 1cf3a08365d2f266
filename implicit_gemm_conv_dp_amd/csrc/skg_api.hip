// C ABI of the engine: device queries, plans and the run calls.
//
// Status convention of the stream-K GEMM bridge (composable_kernel commit
// "feat(ck-tile): stream-K GEMM TE to dispatcher bridge", Changes): 0, -1 for
// a HIP error or a C++ exception, -2 for arguments the engine does not
// support, decided before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "skg_internal.hpp"
#include "skg_launch.hpp"

namespace skg {
namespace {

struct DeviceRec {
  bool valid = false;
  bool gfx950 = false;
  int cus = 0;
  std::string arch;
};

std::mutex g_dev_mu;
std::vector<DeviceRec> g_devs;

// Optional timing hook (skg_profile_events), per host thread.
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

int current_device(DeviceRec* out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failure(std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_devs.size() <= dev) g_devs.resize(dev + 1);
  DeviceRec& r = g_devs[dev];
  if (!r.valid) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_failure(std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    r.arch = prop.gcnArchName;
    r.gfx950 = r.arch.compare(0, 6, "gfx950") == 0;
    r.cus = prop.multiProcessorCount;
    r.valid = true;
  }
  *out = r;
  return SKG_OK;
}

// CU count and resident CTAs per CU of one instance on the current device.
int device_capacity(int op, int tile_id, int dtype, int* cus, int* per_cu) {
  DeviceRec d;
  int rc = current_device(&d);
  if (rc) return rc;
  if (!d.gfx950) return unsupported("unsupported arch " + d.arch + " (the engine is built for gfx950)");
  int occ = 0;
  hipError_t e;
  if (op == SKG_OP_GEMM) {
    GemmInst in = gemm_instance(tile_id, dtype, SKG_SCALE_ROWCOL);
    if (!in.occupancy) return unsupported("no GEMM instance for this tile and dtype");
    e = in.occupancy(&occ);
  } else if (op == SKG_OP_WGRAD) {
    WgradInst in = wgrad_instance(tile_id, dtype);
    if (!in.occupancy) return unsupported("no wgrad instance for this tile and dtype");
    e = in.occupancy(&occ);
  } else if (op == SKG_OP_FWD || op == SKG_OP_DGRAD) {
    ConvInst in = op == SKG_OP_FWD ? fwd_instance(tile_id, dtype) : dgrad_instance(tile_id, dtype);
    if (!in.occupancy) return unsupported("no convolution instance for this tile and dtype");
    e = in.occupancy(&occ);
  } else {
    return unsupported("unknown op");
  }
  if (e != hipSuccess) return hip_failure(std::string("occupancy query: ") + hipGetErrorString(e));
  if (occ <= 0) return unsupported("kernel instance cannot be resident on this device");
  *cus = d.cus;
  *per_cu = occ;
  return SKG_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Fault injection for tests of the error paths, read from the environment on
// every run call: SKG_FAULT=launch makes the call fail with -1 where it would
// launch the stream-K kernel (after its resets are enqueued, like a real
// launch failure); SKG_FAULT=handoff runs the kernel with stream-K CTAs that
// never raise their flags and a spin limit of kFaultSpin polls, so every
// hand-off wait gives up (counted, and its tile poisoned with NaN) and the
// kernel still ends.
enum { INJECT_NONE = 0, INJECT_LAUNCH = 1, INJECT_HANDOFF = 2 };
constexpr uint32_t kFaultSpin = 64;

int injected_fault() {
  const char* v = std::getenv("SKG_FAULT");
  if (!v) return INJECT_NONE;
  if (std::strcmp(v, "launch") == 0) return INJECT_LAUNCH;
  if (std::strcmp(v, "handoff") == 0) return INJECT_HANDOFF;
  return INJECT_NONE;
}

FastDiv make_fastdiv(uint32_t d);

KPlan to_kplan(const skg_plan_t& pl, int inject) {
  KPlan k;
  k.tiles_m = (int)pl.tiles_m;
  k.tiles_n = (int)pl.tiles_n;
  k.ipt = (int)pl.iters_per_tile;
  k.dp_tiles = (int)pl.dp_tiles;
  k.sk_tiles = (int)pl.sk_tiles;
  k.sk_ctas = (int)pl.sk_ctas;
  k.ipc = (int)pl.iters_per_sk_cta;
  k.extra = (int)pl.extra_iters;
  k.grid = (int)pl.grid;
  k.mode = pl.mode;
  k.reduction = pl.reduction;
  k.sk_order = pl.sk_order == SKG_SK_ORDER_XCD      ? SK_ORDER_XCD
               : pl.sk_order == SKG_SK_ORDER_KMAJOR ? SK_ORDER_KMAJOR
                                                    : SK_ORDER_BLOCK;
  k.sk_slices = whole_slices(pl) ? (int)(pl.iters_per_tile / pl.iters_per_sk_cta) : 1;
  k.spin_limit = inject == INJECT_HANDOFF ? kFaultSpin : kSpinLimit;
  k.fault = inject == INJECT_HANDOFF ? FAULT_NO_PUBLISH : FAULT_NONE;
  const int tn = k.tiles_n > 0 ? k.tiles_n : 1;
  k.dp_rows = k.dp_tiles / tn;
  k.div_tiles_n = make_fastdiv((uint32_t)tn);
  k.div_groups = make_fastdiv((uint32_t)(kDpGroupRows * tn));
  return k;
}

Scratch carve(const skg_plan_t& pl, void* ws) {
  Scratch s{nullptr, nullptr, nullptr};
  char* base = static_cast<char*>(ws);
  if (pl.sk_ctas && handoff_reduction(pl.reduction)) {
    s.flags = reinterpret_cast<uint32_t*>(base);
    s.partials = reinterpret_cast<float*>(base + pl.flags_bytes);  // partials after the flags
  } else if (pl.sk_ctas && pl.reduction == SKG_RED_WORKSPACE) {
    s.ws = reinterpret_cast<float*>(base);
  }
  return s;
}

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  f.shift = s;
  f.magic = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
  return f;
}

// Checks shared by both run calls once the plan is known: the workspace
// covers the plan, and a linear/tree pool fits on the device at once (its
// CTAs wait on each other, so all of them must be resident).
int check_run(const skg_plan_t& pl, void* ws, size_t ws_bytes, int cus, int per_cu) {
  if ((size_t)pl.workspace_bytes > ws_bytes) return unsupported("workspace too small for this plan");
  if (pl.workspace_bytes && (!ws || !aligned(ws, 256))) return unsupported("workspace must be 256-byte aligned device memory");
  if (handoff_reduction(pl.reduction) && pl.sk_ctas > (int64_t)cus * per_cu)
    return unsupported("linear/tree/scatter stream-K pool exceeds the resident capacity of the device");
  return SKG_OK;
}

// The conv plan once the device capacity is known (used only for ctas = -1).
int plan_conv_with(const skg_conv_args_t* a, bool dgrad, const TileDesc& t, int cus, int per_cu,
                   skg_plan_t* out) {
  const int rc = plan_launch(conv_shape(a, t, dgrad), t, a->mode, a->reduction, a->ctas,
                             resolve_sk_order(a->sk_order, false), cus, per_cu, out);
  if (rc) return rc;
  if (dgrad) {
    out->aux_bytes = dgrad_filter_bytes(a);
    out->workspace_bytes += out->aux_bytes;
  }
  return SKG_OK;
}

int reset_scratch(const skg_plan_t& pl, void* ws, hipStream_t st) {
  if (!pl.sk_ctas) return SKG_OK;
  hipError_t e = hipSuccess;
  if (handoff_reduction(pl.reduction))
    e = hipMemsetAsync(ws, 0, (size_t)pl.flags_bytes, st);
  else if (pl.reduction == SKG_RED_WORKSPACE)
    e = hipMemsetAsync(ws, 0, (size_t)(pl.workspace_bytes - pl.aux_bytes), st);
  if (e != hipSuccess) return hip_failure(std::string("reset: ") + hipGetErrorString(e));
  return SKG_OK;
}

// Fills `words` 32-bit words with zero.  The allocation-free entry point
// clears its scratch and outputs with this kernel instead of
// hipMemsetAsync: a caller may capture the call into a HIP graph, where
// memset nodes are best avoided.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t words) {
  const size_t step = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += step) p[i] = 0u;
}

hipError_t zero_fill(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;  // every cleared region is a multiple of 4 bytes
  if (!words) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

// Scratch of skg_run_wgrad_static: a file-scope device array (one copy per
// device the library runs on, held until the process ends).  Host code
// never uses the array's name as a device address: the address of each
// device's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and kept in g_static_scratch.
constexpr size_t kStaticScratchBytes = SKG_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_static_scratch;  // per device; nullptr until first use

int static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_failure(std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_static_scratch.size() <= dev) g_static_scratch.resize(dev + 1, nullptr);
  if (!g_static_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return hip_failure(std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_static_scratch[dev] = ptr;
  }
  *out = g_static_scratch[dev];
  return SKG_OK;
}

// The wgrad run call.  kernel_resets: clear flags, scratch and (atomic) dW
// with zero_fill instead of hipMemsetAsync.
int run_wgrad(const skg_wgrad_args_t* a, void* ws, size_t ws_bytes, hipStream_t st,
              bool kernel_resets) {
  int rc = validate_wgrad(a);
  if (rc) return rc;
  if (!a->x || !a->dy || !a->dw) return unsupported("null x, dy or dw");
  if (!aligned(a->x, 16) || !aligned(a->dy, 16) || !aligned(a->dw, 16))
    return unsupported("x, dy and dw must be 16-byte aligned");
  const TileDesc* t = tile_desc(a->tile_id);
  WgradInst inst = wgrad_instance(a->tile_id, a->dtype);
  if (!inst.launch) return unsupported("no wgrad instance for this tile and dtype");
  int cus = 0, per_cu = 0;
  rc = device_capacity(SKG_OP_WGRAD, a->tile_id, a->dtype, &cus, &per_cu);
  if (rc) return rc;
  skg_plan_t pl;
  rc = plan_launch(wgrad_shape(a, *t), *t, a->mode, a->reduction, a->ctas,
                   resolve_sk_order(a->sk_order, true), cus, per_cu, &pl);
  if (rc) return rc;
  if (kernel_resets && (size_t)pl.workspace_bytes > ws_bytes)
    return unsupported("the plan needs " + std::to_string(pl.workspace_bytes) +
                       " bytes of scratch; the static scratch holds " + std::to_string(ws_bytes));
  rc = check_run(pl, ws, ws_bytes, cus, per_cu);
  if (rc) return rc;
  if (kernel_resets) {
    size_t bytes = 0;
    if (pl.sk_ctas && handoff_reduction(pl.reduction))
      bytes = (size_t)pl.flags_bytes;
    else if (pl.sk_ctas && pl.reduction == SKG_RED_WORKSPACE)
      bytes = (size_t)(pl.workspace_bytes - pl.aux_bytes);
    hipError_t e = zero_fill(ws, bytes, st);
    if (e != hipSuccess) return hip_failure(std::string("reset: ") + hipGetErrorString(e));
  } else {
    rc = reset_scratch(pl, ws, st);
    if (rc) return rc;
  }
  WgradParams w;
  w.X = static_cast<const char*>(a->x);
  w.dY = static_cast<const char*>(a->dy);
  w.dW = a->dw;
  w.N = a->n;
  w.H = a->h;
  w.W = a->w;
  w.C = a->c;
  w.K = a->k;
  w.R = a->r;
  w.S = a->s;
  w.sh = a->stride_h;
  w.sw = a->stride_w;
  w.ph = a->pad_h;
  w.pw = a->pad_w;
  w.Ho = (a->h + 2 * a->pad_h - a->r) / a->stride_h + 1;
  w.Wo = (a->w + 2 * a->pad_w - a->s) / a->stride_w + 1;
  w.cpg = a->c / a->groups;
  w.kpg = a->k / a->groups;
  w.mt_per_group = (int)ceil_div(w.kpg, t->tm);
  w.gemm_n = w.cpg * a->r * a->s;
  w.kred = a->n * w.Ho * w.Wo;
  w.x_bytes = (uint32_t)((int64_t)a->n * a->h * a->w * a->c * 2);
  w.dy_bytes = (uint32_t)((int64_t)w.kred * a->k * 2);
  w.div_howo = make_fastdiv((uint32_t)(w.Ho * w.Wo));
  w.div_wo = make_fastdiv((uint32_t)w.Wo);
  w.div_ho = make_fastdiv((uint32_t)w.Ho);
  w.div_cpg = make_fastdiv((uint32_t)w.cpg);
  w.div_s = make_fastdiv((uint32_t)a->s);
  if (pl.reduction == SKG_RED_ATOMIC && pl.sk_ctas) {
    const size_t bytes = (size_t)a->k * w.gemm_n * 4;
    hipError_t e = kernel_resets ? zero_fill(a->dw, bytes, st) : hipMemsetAsync(a->dw, 0, bytes, st);
    if (e != hipSuccess) return hip_failure(std::string("zeroing dW: ") + hipGetErrorString(e));
  }
  const int inject = injected_fault();
  if (inject == INJECT_LAUNCH) return hip_failure("launch: failure injected by SKG_FAULT=launch");
  hipError_t e = inst.launch(w, to_kplan(pl, inject), carve(pl, ws), st, g_ev_start, g_ev_stop);
  if (e != hipSuccess) return hip_failure(std::string("launch: ") + hipGetErrorString(e));
  return SKG_OK;
}

// Wt[g][c][r][s][k'] = W[g*Kpg + k'][r][s][c]: per group and tap, a Kpg x Cpg
// block transposed through a 32x33 LDS tile (reads along c, writes along k',
// both coalesced).  Grid: (ceil(Cpg/32), ceil(Kpg/32), groups*R*S), 32x8 threads.
__global__ __launch_bounds__(256) void transpose_filter_kernel(const uint16_t* __restrict__ w,
                                                              uint16_t* __restrict__ wt, int kpg,
                                                              int cpg, int rs) {
  __shared__ uint16_t t[32][33];
  const int g = blockIdx.z / rs, tap = blockIdx.z - g * rs;
  const int c0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int k = k0 + ty + i, c = c0 + tx;
    if (k < kpg && c < cpg) t[ty + i][tx] = w[((size_t)(g * kpg + k) * rs + tap) * cpg + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    const int c = c0 + ty + i, k = k0 + tx;
    if (k < kpg && c < cpg) wt[((size_t)(g * cpg + c) * rs + tap) * kpg + k] = t[tx][ty + i];
  }
}


int plan_conv(const skg_conv_args_t* a, bool dgrad, skg_plan_t* out) {
  int rc = validate_conv(a, dgrad);
  if (rc) return rc;
  if (!out) return unsupported("null output");
  const TileDesc* t = tile_desc(a->tile_id);
  int cus = 0, per_cu = 0;
  if (a->ctas == -1) {
    rc = device_capacity(dgrad ? SKG_OP_DGRAD : SKG_OP_FWD, a->tile_id, a->dtype, &cus, &per_cu);
    if (rc) return rc;
  }
  return plan_conv_with(a, dgrad, *t, cus, per_cu, out);
}

int run_conv(const skg_conv_args_t* a, bool dgrad, void* ws, size_t ws_bytes, hipStream_t st) {
  int rc = validate_conv(a, dgrad);
  if (rc) return rc;
  if (!a->act || !a->filt || !a->out) return unsupported("null act, filt or out");
  if (!aligned(a->act, 16) || !aligned(a->filt, 16) || !aligned(a->out, 16))
    return unsupported("act, filt and out must be 16-byte aligned");
  const TileDesc* t = tile_desc(a->tile_id);
  ConvInst inst = dgrad ? dgrad_instance(a->tile_id, a->dtype) : fwd_instance(a->tile_id, a->dtype);
  if (!inst.launch) return unsupported("no convolution instance for this tile and dtype");
  int cus = 0, per_cu = 0;
  rc = device_capacity(dgrad ? SKG_OP_DGRAD : SKG_OP_FWD, a->tile_id, a->dtype, &cus, &per_cu);
  if (rc) return rc;
  skg_plan_t pl;
  rc = plan_conv_with(a, dgrad, *t, cus, per_cu, &pl);
  if (rc) return rc;
  rc = check_run(pl, ws, ws_bytes, cus, per_cu);
  if (rc) return rc;
  rc = reset_scratch(pl, ws, st);
  if (rc) return rc;
  const int ho = (a->h + 2 * a->pad_h - a->r) / a->stride_h + 1;
  const int wo = (a->w + 2 * a->pad_w - a->s) / a->stride_w + 1;
  const int cpg = a->c / a->groups, kpg = a->k / a->groups;
  ConvParams c;
  c.act = static_cast<const char*>(a->act);
  c.out = static_cast<char*>(a->out);
  c.dtype_out = a->dtype_out == SKG_F32 ? DT_F32 : (a->dtype_out == SKG_F16 ? DT_F16 : DT_BF16);
  c.S = a->s;
  c.sh = a->stride_h;
  c.sw = a->stride_w;
  c.ph = a->pad_h;
  c.pw = a->pad_w;
  const int eo = a->dtype_out == SKG_F32 ? 4 : 2;
  if (!dgrad) {
    c.filt = static_cast<const char*>(a->filt);
    c.gm = a->n * ho * wo;
    c.npg = kpg;
    c.kred = a->r * a->s * cpg;
    c.cin = cpg;
    c.act_c = a->c;
    c.out_c = a->k;
    c.act_h = a->h;
    c.act_w = a->w;
    c.pix_w = wo;
    c.div_pix_hw = make_fastdiv((uint32_t)(ho * wo));
    c.act_bytes = (uint32_t)((int64_t)a->n * a->h * a->w * a->c * 2);
  } else {
    // The filter transposed per group into the workspace after the fix-up
    // region: Wt[g][c][r][s][k'] = W[g*Kpg + k'][r][s][c].
    char* wt = static_cast<char*>(ws) + (pl.workspace_bytes - pl.aux_bytes);
    const dim3 grid((unsigned)ceil_div(cpg, 32), (unsigned)ceil_div(kpg, 32), (unsigned)(a->groups * a->r * a->s));
    hipLaunchKernelGGL(transpose_filter_kernel, grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(a->filt), reinterpret_cast<uint16_t*>(wt), kpg, cpg,
                       a->r * a->s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_failure(std::string("filter transpose: ") + hipGetErrorString(e));
    c.filt = wt;
    c.gm = a->n * a->h * a->w;
    c.npg = cpg;
    c.kred = a->r * a->s * kpg;
    c.cin = kpg;
    c.act_c = a->k;
    c.out_c = a->c;
    c.act_h = ho;
    c.act_w = wo;
    c.pix_w = a->w;
    c.div_pix_hw = make_fastdiv((uint32_t)(a->h * a->w));
    c.act_bytes = (uint32_t)((int64_t)a->n * ho * wo * a->k * 2);
  }
  c.pix_h = dgrad ? a->h : ho;
  c.nimg = a->n;
  c.nph = 0;
  if (dgrad && t->group_block) {
    // Stride phases of the block-diagonal dgrad: M tiles phase by phase.
    DgradPhase ph[kMaxDgradPhases];
    c.nph = dgrad_phases(a, ph);
    int tiles = 0;
    for (int i = 0; i < c.nph; ++i) {
      const DgradPhase& q = ph[i];
      c.ph_tile[i] = tiles;
      tiles += (int)ceil_div(int64_t(a->n) * q.hc * q.wc, t->tm);
      DgradPhaseRec& r = c.phase[i];
      r = DgradPhaseRec{};
      r.h0 = q.h0;
      r.w0 = q.w0;
      r.hc = q.hc;
      r.wc = q.wc;
      r.a = q.a;
      r.b = q.b;
      r.rc = q.rc;
      r.sc = q.sc;
      // h0 + pad_h and a agree modulo the stride: exact divisions
      r.qh = (q.h0 + a->pad_h - q.a) / a->stride_h;
      r.qw = (q.w0 + a->pad_w - q.b) / a->stride_w;
      r.div_hw = make_fastdiv((uint32_t)std::max(1, q.hc * q.wc));
      r.div_w = make_fastdiv((uint32_t)std::max(1, q.wc));
      r.div_sc = make_fastdiv((uint32_t)std::max(1, q.sc));
    }
    c.ph_tile[c.nph] = tiles;
  }
  c.nt_per_group = (int)ceil_div(c.npg, t->tn);
  c.filt_bytes = (uint32_t)((int64_t)a->k * a->r * a->s * cpg * 2);
  c.div_pix_w = make_fastdiv((uint32_t)c.pix_w);
  c.div_cin = make_fastdiv((uint32_t)c.cin);
  c.div_s = make_fastdiv((uint32_t)a->s);
  c.div_sh = make_fastdiv((uint32_t)a->stride_h);
  c.div_sw = make_fastdiv((uint32_t)a->stride_w);
  if (pl.reduction == SKG_RED_ATOMIC && pl.sk_ctas) {
    hipError_t e = hipMemsetAsync(a->out, 0, (size_t)c.gm * c.out_c * eo, st);
    if (e != hipSuccess) return hip_failure(std::string("zeroing the output: ") + hipGetErrorString(e));
  }
  const int inject = injected_fault();
  if (inject == INJECT_LAUNCH) return hip_failure("launch: failure injected by SKG_FAULT=launch");
  hipError_t e = inst.launch(c, to_kplan(pl, inject), carve(pl, ws), st, g_ev_start, g_ev_stop);
  if (e != hipSuccess) return hip_failure(std::string("launch: ") + hipGetErrorString(e));
  return SKG_OK;
}

}  // namespace
}  // namespace skg

using namespace skg;

extern "C" {

int skg_device_info(int32_t op, int32_t tile_id, int32_t dtype_ab, int32_t* num_cus,
                    int32_t* resident_per_cu) {
  try {
    clear_error();
    if (!num_cus || !resident_per_cu) return unsupported("null output");
    int c = 0, r = 0;
    int rc = device_capacity(op, tile_id, dtype_ab, &c, &r);
    if (rc) return rc;
    *num_cus = c;
    *resident_per_cu = r;
    return SKG_OK;
  } catch (const std::exception& ex) {
    return hip_failure(std::string("exception: ") + ex.what());
  } catch (...) {
    return hip_failure("unknown exception");
  }
}

int skg_profile_events(void* start, void* stop) {
  clear_error();
  if ((start == nullptr) != (stop == nullptr)) return unsupported("set both events or neither");
  g_ev_start = static_cast<hipEvent_t>(start);
  g_ev_stop = static_cast<hipEvent_t>(stop);
  return SKG_OK;
}

int skg_plan_gemm(const skg_gemm_args_t* a, skg_plan_t* out) {
  try {
    clear_error();
    int rc = validate_gemm(a);
    if (rc) return rc;
    if (!out) return unsupported("null output");
    const TileDesc* t = tile_desc(a->tile_id);
    int cus = 0, per_cu = 0;
    if (a->ctas == -1) {
      rc = device_capacity(SKG_OP_GEMM, a->tile_id, a->dtype_ab, &cus, &per_cu);
      if (rc) return rc;
    }
    return plan_launch(gemm_shape(a, *t), *t, a->mode, a->reduction, a->ctas,
                       resolve_sk_order(a->sk_order, false), cus, per_cu, out);
  } catch (...) {
    return hip_failure("exception in skg_plan_gemm");
  }
}

int skg_plan_wgrad(const skg_wgrad_args_t* a, skg_plan_t* out) {
  try {
    clear_error();
    int rc = validate_wgrad(a);
    if (rc) return rc;
    if (!out) return unsupported("null output");
    const TileDesc* t = tile_desc(a->tile_id);
    int cus = 0, per_cu = 0;
    if (a->ctas == -1) {
      rc = device_capacity(SKG_OP_WGRAD, a->tile_id, a->dtype, &cus, &per_cu);
      if (rc) return rc;
    }
    return plan_launch(wgrad_shape(a, *t), *t, a->mode, a->reduction, a->ctas,
                       resolve_sk_order(a->sk_order, true), cus, per_cu, out);
  } catch (...) {
    return hip_failure("exception in skg_plan_wgrad");
  }
}

int skg_gemm_workspace_bytes(const skg_gemm_args_t* a, size_t* out) {
  if (!out) {
    clear_error();
    return unsupported("null output");
  }
  skg_plan_t pl;
  const int rc = skg_plan_gemm(a, &pl);
  if (rc) return rc;
  *out = (size_t)pl.workspace_bytes;
  return SKG_OK;
}

int skg_wgrad_workspace_bytes(const skg_wgrad_args_t* a, size_t* out) {
  if (!out) {
    clear_error();
    return unsupported("null output");
  }
  skg_plan_t pl;
  const int rc = skg_plan_wgrad(a, &pl);
  if (rc) return rc;
  *out = (size_t)pl.workspace_bytes;
  return SKG_OK;
}

int skg_fixup_timeouts(uint32_t* count, int32_t reset) {
  try {
    clear_error();
    if (!count) return unsupported("null output");
    hipError_t (*const units[])(uint32_t*, bool) = {wait_timeouts_gemm_f16, wait_timeouts_gemm_bf16,
                                                    wait_timeouts_gemm_f8,  wait_timeouts_wgrad,
                                                    wait_timeouts_fwd,      wait_timeouts_dgrad};
    uint32_t total = 0;
    for (auto fn : units) {
      uint32_t c = 0;
      const hipError_t e = fn(&c, reset != 0);
      if (e != hipSuccess) return hip_failure(std::string("reading the wait counters: ") + hipGetErrorString(e));
      total += c;
    }
    *count = total;
    return SKG_OK;
  } catch (...) {
    return hip_failure("exception in skg_fixup_timeouts");
  }
}

int skg_run_gemm(const skg_gemm_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    int rc = validate_gemm(a);
    if (rc) return rc;
    if (!a->A || !a->B || !a->C) return unsupported("null A, B or C");
    if (!aligned(a->A, 16) || !aligned(a->B, 16) || !aligned(a->C, 16))
      return unsupported("A, B and C must be 16-byte aligned");
    if ((a->scale_a && !aligned(a->scale_a, 16)) || (a->scale_b && !aligned(a->scale_b, 16)))
      return unsupported("scales must be 16-byte aligned");
    const TileDesc* t = tile_desc(a->tile_id);
    if (a->scale_mode == SKG_SCALE_MX_E8M0 && (!a->scale_a || !a->scale_b))
      return unsupported("MX block scales need both scale arrays");
    GemmInst inst = gemm_instance(a->tile_id, a->dtype_ab, a->scale_mode);
    if (!inst.launch) return unsupported("no GEMM instance for this tile and dtype");
    int cus = 0, per_cu = 0;
    rc = device_capacity(SKG_OP_GEMM, a->tile_id, a->dtype_ab, &cus, &per_cu);
    if (rc) return rc;
    skg_plan_t pl;
    rc = plan_launch(gemm_shape(a, *t), *t, a->mode, a->reduction, a->ctas,
                     resolve_sk_order(a->sk_order, false), cus, per_cu, &pl);
    if (rc) return rc;
    rc = check_run(pl, ws, ws_bytes, cus, per_cu);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    rc = reset_scratch(pl, ws, st);
    if (rc) return rc;
    if (pl.reduction == SKG_RED_ATOMIC && pl.sk_ctas) {
      hipError_t e = hipMemset2DAsync(a->C, (size_t)a->ldc * 4, 0, (size_t)a->N * 4, (size_t)a->M, st);
      if (e != hipSuccess) return hip_failure(std::string("zeroing C: ") + hipGetErrorString(e));
    }
    GemmParams g;
    g.A = static_cast<const char*>(a->A);
    g.B = static_cast<const char*>(a->B);
    g.C = static_cast<char*>(a->C);
    g.M = (int)a->M;
    g.N = (int)a->N;
    g.K = (int)a->K;
    g.lda_b = (uint32_t)(a->lda * elem_bytes(a->dtype_ab));
    g.ldb_b = (uint32_t)(a->ldb * elem_bytes(a->dtype_ab));
    g.ldc = (int)a->ldc;
    g.sa = a->scale_a;
    g.sb = a->scale_b;
    g.dtype_c = a->dtype_c == SKG_F32 ? DT_F32 : (a->dtype_c == SKG_F16 ? DT_F16 : DT_BF16);
    const int inject = injected_fault();
    if (inject == INJECT_LAUNCH) return hip_failure("launch: failure injected by SKG_FAULT=launch");
    hipError_t e = inst.launch(g, to_kplan(pl, inject), carve(pl, ws), st, g_ev_start, g_ev_stop);
    if (e != hipSuccess) return hip_failure(std::string("launch: ") + hipGetErrorString(e));
    return SKG_OK;
  } catch (const std::exception& ex) {
    return hip_failure(std::string("exception: ") + ex.what());
  } catch (...) {
    return hip_failure("unknown exception");
  }
}

int skg_run_wgrad(const skg_wgrad_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    return run_wgrad(a, ws, ws_bytes, static_cast<hipStream_t>(stream), false);
  } catch (const std::exception& ex) {
    return hip_failure(std::string("exception: ") + ex.what());
  } catch (...) {
    return hip_failure("unknown exception");
  }
}

int skg_plan_fwd(const skg_conv_args_t* a, skg_plan_t* out) {
  try {
    clear_error();
    return plan_conv(a, false, out);
  } catch (...) {
    return hip_failure("exception in skg_plan_fwd");
  }
}

int skg_plan_dgrad(const skg_conv_args_t* a, skg_plan_t* out) {
  try {
    clear_error();
    return plan_conv(a, true, out);
  } catch (...) {
    return hip_failure("exception in skg_plan_dgrad");
  }
}

int skg_run_fwd(const skg_conv_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    return run_conv(a, false, ws, ws_bytes, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return hip_failure(std::string("exception: ") + ex.what());
  } catch (...) {
    return hip_failure("unknown exception");
  }
}

int skg_run_dgrad(const skg_conv_args_t* a, void* ws, size_t ws_bytes, void* stream) {
  try {
    clear_error();
    return run_conv(a, true, ws, ws_bytes, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return hip_failure(std::string("exception: ") + ex.what());
  } catch (...) {
    return hip_failure("unknown exception");
  }
}

int skg_run_wgrad_static(const skg_wgrad_args_t* a, void* stream) {
  try {
    clear_error();
    if (!a) return unsupported("null arguments");
    void* ws = nullptr;
    const int rc = static_scratch(&ws);
    if (rc) return rc;
    return run_wgrad(a, ws, kStaticScratchBytes, static_cast<hipStream_t>(stream), true);
  } catch (const std::exception& ex) {
    return hip_failure(std::string("exception: ") + ex.what());
  } catch (...) {
    return hip_failure("unknown exception");
  }
}

}  // extern "C"
