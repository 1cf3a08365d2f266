// Forward convolution and input gradient (dgrad) as implicit GEMMs on the
// stream-K engine (rocm-libraries PR #13151 "feat(rocke): stream-K for
// implicit-GEMM conv wgrad": the docs commit points the forward-convolution
// future-work note at the stream-K port, review items 2-3 ask for forward
// convolution on the family-agnostic partitioner).
//
// Both are GEMMs whose operands are K-contiguous in NHWC / KRSC memory, so
// they run the GEMM mainloop (whole 128-byte rows per MAC iteration straight
// into LDS, ds_read_b128 fragments):
//   forward  Y[m][k]  = sum_q A[m][q] * W[k][q]   m = (n, ho, wo), q = (r, s, c')
//            A[m][q]  = X[n][ho*sh - ph + r][wo*sw - pw + s][g*Cpg + c'] (0 outside)
//   dgrad    dX[m][c] = sum_q A[m][q] * Wt[c][q]  m = (n, h, w),   q = (r, s, k')
//            A[m][q]  = dY[n][(h + ph - r)/sh][(w + pw - s)/sw][g*Kpg + k'] when both
//                       divisions are exact and inside the output image, else 0
//            Wt[g][c][r][s][k'] = W[g*Kpg + k'][r][s][c]   (written into the workspace
//                       by the run call before the stream-K kernel)
// Groups fold into GEMM-N with the tile count per group, so an N tile never
// crosses a group.  The reduction index q runs over (r, s) taps with the
// channel fastest, so a 16-byte chunk (8 channels; channels per group are
// multiples of 8) lies inside one tap.
#pragma once

#include "skg_kernels.hpp"

namespace skg {

constexpr int kMaxPhases = 16;  // stride phases of a block-diagonal dgrad (sh * sw)

// One stride phase of a block-diagonal dgrad: the pixels h = h0 + sh*i
// (i < hc), w = w0 + sw*j (j < wc) of every image, and the taps
// r = a + sh*ri (ri < rc), s = b + sw*si (si < sc); pixel (i, j) meets dY
// at (i + qh - ri, j + qw - si).  One record per phase, so that a tile's
// set-up reads its phase in one round of scalar loads.
struct alignas(16) DgradPhaseRec {
  int h0, w0, hc, wc;
  int a, b, rc, sc;
  int qh, qw, pad0, pad1;
  FastDiv div_hw, div_w, div_sc;  // by hc * wc, wc, sc
  int pad2[3];
};
static_assert(sizeof(DgradPhaseRec) == 96, "phase record");

struct ConvParams {
  const char* act;    // forward: X (N,H,W,C); dgrad: dY (N,Ho,Wo,K)
  const char* filt;   // forward: W (K,R,S,Cpg); dgrad: Wt (groups,Cpg,R,S,Kpg)
  char* out;          // forward: Y (N,Ho,Wo,K); dgrad: dX (N,H,W,C)
  int dtype_out;
  int gm;             // GEMM-M: output pixels (forward) or input pixels (dgrad)
  int npg;            // GEMM-N per group: Kpg (forward) or Cpg (dgrad)
  int nt_per_group;   // ceil(npg / TN)
  int kred;           // reduction: R*S*Cpg (forward) or R*S*Kpg (dgrad)
  int cin;            // gathered channels per group: Cpg (forward) or Kpg (dgrad)
  int act_c, out_c;   // channels of the activation and of the output tensor
  int act_h, act_w;   // spatial size of the activation tensor
  int pix_w;          // row length of the GEMM-M pixel grid (Wo forward, W dgrad)
  int pix_h;          // its height (Ho forward, H dgrad)
  int S, sh, sw, ph, pw;
  uint32_t act_bytes, filt_bytes;
  FastDiv div_pix_hw, div_pix_w, div_cin, div_s, div_sh, div_sw;
  // Stride phases of a block-diagonal dgrad, whose GEMM-M runs phase by
  // phase: phase p owns M tiles [ph_tile[p], ph_tile[p+1]), described by
  // phase[p].
  int nph, nimg;
  int ph_tile[kMaxPhases + 1];
  DgradPhaseRec phase[kMaxPhases];
};

// Operand loader of the grouped pipeline.  Group j of a segment is the A
// tile (j even: TM rows of the gathered activation, 128 bytes of the
// reduction each) or the B tile (j odd: TN filter rows) of MAC iteration
// j/2.  A thread owns one 16-byte chunk position of a row and the rows
// row(tid) + u*STEP; the pixel of each of its A rows is decomposed once per
// tile, the tap and channel of its chunk once per group.  Padding, pixels
// past GEMM-M, filter rows past the group and the reduction tail come back
// as zero (out-of-range buffer offsets).
template <class Cfg, bool DGRAD>
struct ConvGrpLoader {
  static constexpr bool kDma = true, kGrouped = true, kTrans = false;
  static_assert(Cfg::RB == 128 && Cfg::ESZ == 2, "whole-line rows of 16-bit elements");
  static constexpr int CPR = Cfg::RB / 16;
  static constexpr int STEP = Cfg::THREADS / CPR;
  static constexpr int UA = Cfg::TM / STEP, UB = Cfg::TN / STEP;
  static_assert(UA * STEP == Cfg::TM && UB * STEP == Cfg::TN, "DMA mapping");

  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t offb, stepb, limb;  // B: this thread's first chunk, STEP rows, K limit (bytes)
  int wave, chunk;
  int pn[UA];                  // n * act_h, or -1 for a row past GEMM-M
  int py[UA], px[UA];          // forward: ho*sh - ph, wo*sw - pw; dgrad: h + ph, w + pw
  int act_h, act_w, kred, cin, S, sh, sw;
  uint32_t act_c2, chan0;      // bytes per activation pixel; byte offset of the group's channels
  FastDiv div_cin, div_s, div_sh, div_sw;

  SKG_DEV void init(const ConvParams& c, int group, int m0, int n0, int tid) {
    ra = make_rsrc(c.act, c.act_bytes);
    const uint32_t rowb = (uint32_t)c.kred * 2;
    const int rows_b = c.npg - n0;
    // The filter is below 2 GiB: a 32-bit offset, kept scalar so the
    // resource stays in SGPRs.
    const uint32_t boff = __builtin_amdgcn_readfirstlane((uint32_t)(group * c.npg + n0) * rowb);
    const uint32_t brec = __builtin_amdgcn_readfirstlane((uint32_t)rows_b * rowb);
    rb = make_rsrc(c.filt + boff, brec);
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int row;
    lds_slot<128>(tid, row, chunk);
    offb = (uint32_t)row * rowb + chunk * 16;
    stepb = STEP * rowb;
    limb = rowb > (uint32_t)chunk * 16 ? rowb - chunk * 16 : 0;  // a chunk past a short reduction reads nothing
    act_h = c.act_h;
    act_w = c.act_w;
    kred = c.kred;
    cin = c.cin;
    S = c.S;
    sh = c.sh;
    sw = c.sw;
    act_c2 = (uint32_t)c.act_c * 2;
    chan0 = (uint32_t)(group * c.cin) * 2;
    div_cin = c.div_cin;
    div_s = c.div_s;
    div_sh = c.div_sh;
    div_sw = c.div_sw;
    const int pix_w = c.pix_w;
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int m = m0 + row + u * STEP;
      const uint32_t n = fdiv((uint32_t)m, c.div_pix_hw);
      const int rem = m - (int)n * (int)c.div_pix_hw.d;
      const int y = (int)fdiv((uint32_t)rem, c.div_pix_w);
      const int x = rem - y * pix_w;
      pn[u] = m < c.gm ? (int)n * act_h : -1;
      py[u] = DGRAD ? y + c.ph : y * c.sh - c.ph;
      px[u] = DGRAD ? x + c.pw : x * c.sw - c.pw;
    }
  }

  // Tap and channel of this thread's chunk in MAC iteration `it`.
  struct Tap {
    int r, s;
    uint32_t cofs;  // byte offset of the chunk's channels within a pixel
    bool ok;        // inside the reduction
  };
  SKG_DEV Tap tap_of(int it) const {
    const int kk = it * Cfg::TK + chunk * 8;
    const uint32_t t = fdiv((uint32_t)kk, div_cin);
    const int ci = kk - (int)t * cin;
    const uint32_t r = fdiv(t, div_s);
    Tap tp;
    tp.r = (int)r;
    tp.s = (int)t - (int)r * S;
    tp.cofs = chan0 + (uint32_t)ci * 2;
    tp.ok = kk < kred;
    return tp;
  }

  // Activation row u of this thread for tap tp, or kOOB.  Evaluated without
  // branches.
  SKG_DEV uint32_t a_off(int u, const Tap& tp, bool live) const {
    int hi, wi;
    bool ok = live & tp.ok & (pn[u] >= 0);
    if constexpr (!DGRAD) {
      hi = py[u] + tp.r;
      wi = px[u] + tp.s;
    } else {
      const int t = py[u] - tp.r, v = px[u] - tp.s;
      hi = (int)fdiv((uint32_t)t, div_sh);
      wi = (int)fdiv((uint32_t)v, div_sw);
      ok = ok & (t >= 0) & (v >= 0) & (hi * sh == t) & (wi * sw == v);
    }
    ok = ok & ((uint32_t)hi < (uint32_t)act_h) & ((uint32_t)wi < (uint32_t)act_w);
    uint32_t off = (uint32_t)((pn[u] + hi) * act_w + wi) * act_c2 + tp.cofs;
    asm volatile("" : "+v"(off));
    return ok ? off : kOOB;
  }

  template <bool IS_A>
  SKG_DEV void issue_group(int it, SKG_LDS char* slot, bool live) const {
    if constexpr (IS_A) {
      const Tap tp = tap_of(it);
#pragma unroll
      for (int u = 0; u < UA; ++u)
        dma16(ra, lds_addr(slot + u * Cfg::THREADS * 16 + wave * 1024), a_off(u, tp, live));
    } else {
      const uint32_t kb = (uint32_t)it * Cfg::RB;
      const bool ok = live && kb < limb;
#pragma unroll
      for (int u = 0; u < UB; ++u)
        dma16(rb, lds_addr(slot + u * Cfg::THREADS * 16 + wave * 1024), ok ? offb + u * stepb + kb : kOOB);
    }
  }

  SKG_DEV void issue_live(int j, int it, SKG_LDS char* slot, bool live) const {
    if ((j & 1) == 0)
      issue_group<true>(it, slot, live);
    else
      issue_group<false>(it, slot, live);
  }
  SKG_DEV void issue(int j, int it, SKG_LDS char* slot) const { issue_live(j, it, slot, true); }

  // Spread refill (256x256 tiles): B group of one iteration, A group of the
  // next, one DMA instruction at a time among the MFMAs.
  struct Refill {
    SKG_LDS char* slot_b;
    SKG_LDS char* slot_a;
    int it_b, it_a;
    bool live_b, live_a;
    Tap tap_a;
  };
  SKG_DEV void finish_refill(Refill& r) const { r.tap_a = tap_of(r.it_a); }
  template <int N>
  SKG_DEV void refill(const Refill& r) const {
    if constexpr (N < UB) {
      const uint32_t kb = (uint32_t)r.it_b * Cfg::RB;
      const bool ok = r.live_b && kb < limb;
      dma16(rb, lds_addr(r.slot_b + N * Cfg::THREADS * 16 + wave * 1024), ok ? offb + N * stepb + kb : kOOB);
    } else {
      constexpr int U = N - UB;
      dma16(ra, lds_addr(r.slot_a + U * Cfg::THREADS * 16 + wave * 1024), a_off(U, r.tap_a, r.live_a));
    }
  }
};

template <class Cfg, bool DGRAD>
struct ConvProblem {
  typedef ConvParams Params;
  static constexpr int kScaleInc = 1;  // no scales
  typedef ConvGrpLoader<Cfg, DGRAD> Loader;

  SKG_DEV static void coords(const Params& c, const KPlan& p, int tile, int& group, int& m0, int& n0) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    group = tn / c.nt_per_group;
    n0 = (tn - group * c.nt_per_group) * Cfg::TN;
    m0 = tm * Cfg::TM;
  }
  SKG_DEV static void setup(const Params& c, const KPlan& p, int tile, Loader& ld, OutTile& out, int tid) {
    int group, m0, n0;
    coords(c, p, tile, group, m0, n0);
    ld.init(c, group, m0, n0, tid);
    out = out_tile(c, p, tile);
  }
  SKG_DEV static OutTile out_tile(const Params& c, const KPlan& p, int tile) {
    int group, m0, n0;
    coords(c, p, tile, group, m0, n0);
    const int esz = c.dtype_out == DT_F32 ? 4 : 2;
    OutTile o;
    // The output is GEMM-M rows of out_c channels; the group's GEMM-N
    // columns start at channel group * npg.
    o.base = c.out + ((size_t)m0 * c.out_c + group * c.npg + n0) * esz;
    o.sa = nullptr;
    o.sb = nullptr;
    o.ld = c.out_c;
    o.rows = c.gm - m0;
    o.cols = c.npg - n0;
    return o;
  }
  SKG_DEV static int dtype_c(const Params& c) { return c.dtype_out; }
};

// Stride phase of GEMM-M tile tm of a block-diagonal dgrad: the number of
// phase boundaries at or below it (every boundary is compared, so the
// table is fetched in one go instead of one dependent load per step).
SKG_DEV int phase_of(const ConvParams& c, int tm) {
  int p = 0;
#pragma unroll
  for (int q = 1; q < kMaxPhases; ++q) p += (q < c.nph) & (tm >= c.ph_tile[q]);
  return p;
}

// Block-diagonal grouped tile for 16 input and 16 output channels per group
// (so C == K): the tile's TN = 16 * BDG channels are BDG whole groups, one
// wave per group, over TM pixels.  A MAC iteration covers TK / 16 filter
// taps of every group's 16 channels: the A side is one plane per tap, TM
// pixel rows of the tile's TN channels gathered at that tap (a whole
// 128-byte line per row for TN = 64), the B side TN filter rows (W for the
// forward pass, the per-group transposed Wt for dgrad) of TK reduction
// elements; the filter rows of consecutive groups are consecutive, so B is
// one dense slab.  dgrad tiles hold the pixels of one stride phase (see
// ConvParams) and walk only that phase's taps.  Wave w multiplies its group's 32-byte slice of every A
// row by its group's 16 filter rows.  Two CTAs share a CU (two ring entries
// each): the loads of a CU are bound by the requests its waves keep in
// flight, and the short per-tile reduction leaves little to pipeline.
template <class Cfg, bool DGRAD>
struct ConvBdLoader {
  static constexpr bool kDma = true, kGrouped = false, kTrans = false;
  static_assert(Cfg::ESZ == 2 && Cfg::BDG > 0 && Cfg::TN == 64, "block-diagonal conv tile");
  static constexpr int PA = Cfg::TN * 2;        // bytes per A row (pixel at one tap)
  static constexpr int RBB = Cfg::TK * 2;       // bytes per B row and iteration
  static constexpr int NPL = Cfg::TK / 16;      // taps (A planes) per iteration
  static constexpr int PLANE = Cfg::TM * PA;
  static constexpr int B_OFF = NPL * PLANE;
  static constexpr int ENTRY = B_OFF + Cfg::TN * RBB;
  static constexpr int EPI = 64 * PA;  // copy-out staging beside the ring: 64 rows of 16-bit outputs
  static constexpr int D = (Cfg::BD_LDS - EPI) / ENTRY > 6 ? 6 : (Cfg::BD_LDS - EPI) / ENTRY;
  static_assert(D >= 2 && PA == 128 && (RBB == 64 || RBB == 128), "ring entries");
  static constexpr int STEP = Cfg::THREADS / (PA / 16);  // A rows per DMA instruction
  static constexpr int UPL = Cfg::TM / STEP;              // DMA instructions per plane
  static constexpr int UA = NPL * UPL, UB = Cfg::TN * RBB / (Cfg::THREADS * 16);
  static_assert(UPL * STEP == Cfg::TM && UB * Cfg::THREADS * 16 == Cfg::TN * RBB && UB >= 1,
                "DMA mapping");

  __amdgpu_buffer_rsrc_t ra, rb;
  int wave;
  uint32_t cofs;               // A: byte offset of this thread's channels within a pixel
  bool chan_ok;                // its channels lie inside the activation
  int pn[UPL];                 // n * act_h, or -1 for a row past the tile's pixels
  int py[UPL], px[UPL];        // forward: ho*sh - ph, wo*sw - pw; dgrad: dY row, column at tap (a, b)
  uint32_t offb[UB], limb[UB]; // B: this thread's filter row (bytes), and its length (0 past the channels)
  uint32_t bch[UB];            // B: this thread's 16-byte chunk within the iteration's row slice
  int act_h, act_w, S, RS, ntap;
  uint32_t act_c2;
  FastDiv div_s, div_sc;
  // dgrad: the tile's stride phase (first tap (a, b), strides, taps per row)
  int pa, pb, sc, sh, sw;

  // Tile tm of GEMM-M (forward: pixels tm*TM..; dgrad: the tm-th tile of
  // the phase-major order), channels k0.. .
  SKG_DEV void init(const ConvParams& c, int tm, int k0, int tid) {
    ra = make_rsrc(c.act, c.act_bytes);
    rb = make_rsrc(c.filt, c.filt_bytes);
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    act_h = c.act_h;
    act_w = c.act_w;
    S = c.S;
    RS = c.kred / 16;
    act_c2 = (uint32_t)c.act_c * 2;
    div_s = c.div_s;
    int row, chunk;
    lds_slot<PA>(tid, row, chunk);
    const int ch = k0 + chunk * 8;
    chan_ok = ch < c.act_c;
    cofs = (uint32_t)ch * 2;
    if constexpr (!DGRAD) {
      const int m0 = tm * Cfg::TM, pix_w = c.pix_w;
      ntap = RS;
#pragma unroll
      for (int u = 0; u < UPL; ++u) {
        const int m = m0 + row + u * STEP;
        const uint32_t n = fdiv((uint32_t)m, c.div_pix_hw);
        const int rem = m - (int)n * (int)c.div_pix_hw.d;
        const int y = (int)fdiv((uint32_t)rem, c.div_pix_w);
        const int x = rem - y * pix_w;
        pn[u] = m < c.gm ? (int)n * act_h : -1;
        py[u] = y * c.sh - c.ph;
        px[u] = x * c.sw - c.pw;
      }
    } else {
      const int p = phase_of(c, tm);
      const DgradPhaseRec& r = c.phase[p];
      const int p0 = (tm - c.ph_tile[p]) * Cfg::TM;
      const int hw = r.hc * r.wc;
      const int total = c.nimg * hw;  // the phase's pixels over all images
      pa = r.a;
      pb = r.b;
      sc = r.sc;
      sh = c.sh;
      sw = c.sw;
      div_sc = r.div_sc;
      ntap = r.rc * r.sc;
#pragma unroll
      for (int u = 0; u < UPL; ++u) {
        const int m = p0 + row + u * STEP;
        const uint32_t n = fdiv((uint32_t)m, r.div_hw);
        const int rem = m - (int)n * hw;
        const int i = (int)fdiv((uint32_t)rem, r.div_w);
        const int j = rem - i * r.wc;
        pn[u] = m < total ? (int)n * act_h : -1;
        py[u] = i + r.qh;
        px[u] = j + r.qw;
      }
    }
    const uint32_t rowb = (uint32_t)c.kred * 2;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      int br, bc;
      lds_slot<RBB>(tid + u * Cfg::THREADS, br, bc);
      const int frow = k0 + br;
      offb[u] = (uint32_t)frow * rowb;
      limb[u] = frow < c.out_c ? rowb : 0u;
      bch[u] = (uint32_t)bc;
    }
  }

  // MAC iterations that hold at least one of the tile's taps.
  SKG_DEV int iters() const { return (ntap * 16 + Cfg::TK - 1) / Cfg::TK; }

  // Tap jj of the tile (forward: of the filter; dgrad: of its stride
  // phase): filter position (r, s) and, for dgrad, the dY offset (ri, si)
  // from the phase's first tap.
  struct Tap {
    int r, s, ri, si;
    bool ok;
  };
  SKG_DEV Tap tap_of(int jj) const {
    Tap t;
    t.ok = jj < ntap;
    if constexpr (!DGRAD) {
      t.r = (int)fdiv((uint32_t)jj, div_s);
      t.s = jj - t.r * S;
      t.ri = t.si = 0;
    } else {
      t.ri = (int)fdiv((uint32_t)jj, div_sc);
      t.si = jj - t.ri * sc;
      t.r = pa + sh * t.ri;
      t.s = pb + sw * t.si;
    }
    return t;
  }

  // Activation row u of this thread at tap t, or kOOB.
  SKG_DEV uint32_t a_off(int u, const Tap& t) const {
    const int hi = DGRAD ? py[u] - t.ri : py[u] + t.r;
    const int wi = DGRAD ? px[u] - t.si : px[u] + t.s;
    const bool ok = chan_ok & t.ok & (pn[u] >= 0) & ((uint32_t)hi < (uint32_t)act_h) &
                    ((uint32_t)wi < (uint32_t)act_w);
    const uint32_t off = (uint32_t)((pn[u] + hi) * act_w + wi) * act_c2 + cofs;
    return ok ? off : kOOB;
  }

  // MAC iteration `it` into the ring entry at `e`: the A planes, then the
  // B slab (the filter rows' entries of the iteration's taps; dgrad: the
  // phase's taps, which are not consecutive in the filter row).
  SKG_DEV void issue_iter(int it, SKG_LDS char* e) const {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const Tap t = tap_of(it * NPL + j);
#pragma unroll
      for (int u = 0; u < UPL; ++u)
        dma16(ra, lds_addr(e + j * PLANE + u * Cfg::THREADS * 16 + wave * 1024), a_off(u, t));
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      uint32_t off;
      if constexpr (!DGRAD) {
        const uint32_t kb = (uint32_t)it * RBB + bch[u] * 16u;
        off = kb < limb[u] ? offb[u] + kb : kOOB;
      } else {
        // Chunk bch of the iteration's slice: half bch % 2 of the 16
        // channels of tap it * NPL + bch / 2 of the phase.
        const Tap t = tap_of(it * NPL + (int)(bch[u] >> 1));
        const uint32_t kb = (uint32_t)(t.r * S + t.s) * 32u + (bch[u] & 1u) * 16u;
        off = (t.ok && limb[u] != 0u) ? offb[u] + kb : kOOB;
      }
      dma16(rb, lds_addr(e + B_OFF + u * Cfg::THREADS * 16 + wave * 1024), off);
    }
  }
};

template <class Cfg, bool DGRAD>
struct ConvBdProblem {
  typedef ConvParams Params;
  static constexpr int kScaleInc = 1;  // no scales
  typedef ConvBdLoader<Cfg, DGRAD> Loader;

  // dgrad: tile rows are pixels of one stride phase (out_row remaps them)
  static constexpr bool kRowRemap = DGRAD;

  SKG_DEV static void setup(const Params& c, const KPlan& p, int tile, Loader& ld, OutTile& out, int tid) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    ld.init(c, tm, tn * Cfg::TN, tid);
    out = out_tile(c, p, tile);
  }
  SKG_DEV static OutTile out_tile(const Params& c, const KPlan& p, int tile) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    const int k0 = tn * Cfg::TN;
    const int esz = c.dtype_out == DT_F32 ? 4 : 2;
    OutTile o;
    o.sa = nullptr;
    o.sb = nullptr;
    o.ld = c.out_c;
    o.cols = c.out_c - k0;
    if constexpr (!DGRAD) {
      // Pixel rows of out_c channels; the tile's channels start at k0.
      const int m0 = tm * Cfg::TM;
      o.base = c.out + ((size_t)m0 * c.out_c + k0) * esz;
      o.rows = c.gm - m0;
    } else {
      const int ph = phase_of(c, tm);
      const DgradPhaseRec& r = c.phase[ph];
      const int p0 = (tm - c.ph_tile[ph]) * Cfg::TM;
      o.base = c.out + (size_t)k0 * esz;
      o.rows = c.nimg * r.hc * r.wc - p0;
      o.rm = RowRemap{p0, r.hc * r.wc, r.wc, r.h0, r.w0, c.sh, c.sw, r.div_hw, r.div_w, c.pix_h, c.pix_w};
    }
    return o;
  }
  SKG_DEV static int dtype_c(const Params& c) { return c.dtype_out; }
};

}  // namespace skg
