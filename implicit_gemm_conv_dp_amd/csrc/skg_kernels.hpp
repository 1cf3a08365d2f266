// The stream-K engine's kernels for gfx950.
//
// One CTA walks its share of the partition resolved on the host (rocm-libraries
// PR #13151 "feat(rocke): stream-K for implicit-GEMM conv wgrad", Technical
// Details, and the commit porting stream-K to the wgrad: the device maps its
// CTA index onto an iteration range and walks it with one bounded loop): a
// stream-K CTA runs a contiguous range of MAC iterations that may straddle
// output tiles; at every tile boundary it stores, publishes or folds the
// tile's accumulator according to whether its segment started and/or ended the
// tile.  Data-parallel tiles run whole.
//
// Mainloop: operands go straight from global memory into a ring of LDS
// slots with gfx950's direct-to-LDS buffer loads (one slot per operand tile of
// a MAC iteration, or per sub-stage for 64-byte rows), several iterations
// ahead, one CTA barrier per iteration; wave64 MFMAs read their fragments
// from the slots.  GEMM operands are K-contiguous and read as they are; wgrad
// operands are M/N-contiguous (NHWC) and are read with the transposing LDS
// read.  The 128x128x32 wgrad tile keeps a register loader that transposes
// 8x8 blocks in registers before its LDS stores.
#pragma once

#include <type_traits>

#include "skg_device.hpp"

namespace skg {

// ---------------------------------------------------------------------------
// Plan as the kernels see it (32-bit; the host checks the ranges).
enum { SK_ORDER_BLOCK = 0, SK_ORDER_XCD = 1, SK_ORDER_KMAJOR = 2 };

// Forced faults (set only from the host's fault-injection switch): with
// FAULT_NO_PUBLISH the stream-K CTAs store their partials but never raise
// their flags, so every wait on them runs into its (then small) spin limit.
enum { FAULT_NONE = 0, FAULT_NO_PUBLISH = 1 };

// Tile rows per group of the data-parallel tile order (dp_order).
constexpr int kDpGroupRows = 4;

struct KPlan {
  int tiles_m, tiles_n, ipt;
  int dp_tiles, sk_tiles, sk_ctas, ipc, extra;
  int grid, mode, reduction;
  int sk_order;         // SK_ORDER_*
  int sk_slices;        // SK_ORDER_KMAJOR: slices per tile (sk_ctas = sk_tiles * sk_slices)
  uint32_t spin_limit;  // polls before a flag wait gives up
  int fault;            // FAULT_*
  int dp_rows;          // dp_tiles / tiles_n
  FastDiv div_tiles_n;  // by tiles_n
  FastDiv div_groups;   // by kDpGroupRows * tiles_n
  // Row of the tile grid that tile id `tile` lies in.
  SKG_DEV int tile_row(int tile) const { return (int)fdiv((uint32_t)tile, div_tiles_n); }
};

// The caller's workspace, carved up on the host.
struct Scratch {
  uint32_t* flags;   // [sk_cta][wave], linear / tree
  float* partials;   // [sk_cta][TM][TN] fp32, linear / tree
  float* ws;         // [sk_tile][TM][TN] fp32, workspace
};

// Where an output tile lands: a row-major window with valid extent
// rows x cols, optional per-row / per-column scales (the problem's
// kScaleInc is 1), or one scale for every row and one for every column
// (kScaleInc is 0: per-tensor).
// Rows of a block-diagonal dgrad tile are pixels of one stride phase: tile
// row r is phase pixel q = p0 + r, i.e. image q / hw, row h0 + sh * i and
// column w0 + sw * j with (i, j) = divmod(q % hw, wc).
struct RowRemap {
  int p0, hw, wc, h0, w0, sh, sw;
  FastDiv div_hw, div_wc;
  int H, W;
};

struct OutTile {
  char* base;
  const float* sa;
  const float* sb;
  int ld;
  int rows, cols;
  RowRemap rm;  // read only by problems with kRowRemap
};

// Pixel of tile row r (its offset from the tile base in rows of ld
// elements).  32-bit: the host keeps every output under 2^31 bytes.
SKG_DEV uint32_t remap_row(const RowRemap& m, int r) {
  const uint32_t q = (uint32_t)(m.p0 + r);
  const uint32_t n = fdiv(q, m.div_hw);
  const uint32_t rem = q - n * (uint32_t)m.hw;
  const uint32_t i = fdiv(rem, m.div_wc);
  const uint32_t j = rem - i * (uint32_t)m.wc;
  return (n * (uint32_t)m.H + m.h0 + m.sh * i) * (uint32_t)m.W + m.w0 + m.sw * j;
}

// Problems whose output rows are not consecutive declare kRowRemap.
template <class P, class = void>
struct ProbRemap {
  static constexpr bool value = false;
};
template <class P>
struct ProbRemap<P, std::void_t<decltype(P::kRowRemap)>> {
  static constexpr bool value = P::kRowRemap;
};
template <class P>
SKG_DEV size_t out_row(const OutTile& o, int r) {
  if constexpr (ProbRemap<P>::value)
    return remap_row(o.rm, r) * (uint32_t)o.ld;  // < 2^31 elements
  else
    return (size_t)r * o.ld;
}

struct GemmParams {
  const char* A;
  const char* B;
  char* C;
  int M, N, K;
  uint32_t lda_b, ldb_b;   // row pitches in bytes
  int ldc;                 // elements
  const float* sa;
  const float* sb;
  int dtype_c;
};

struct WgradParams {
  const char* X;
  const char* dY;
  float* dW;
  int N, H, W, C, K, R, S, sh, sw, ph, pw;
  int Ho, Wo, cpg, kpg, mt_per_group, gemm_n, kred;
  uint32_t x_bytes, dy_bytes;
  FastDiv div_howo, div_wo, div_ho, div_cpg, div_s;
};

// ---------------------------------------------------------------------------
// MX_: the operand slots also hold each row's E8M0 block scales of the
// iteration (4 bytes per row after the row data).
// BDG_ > 0: block-diagonal grouped tile holding BDG_ whole groups of 16
// channels, one wave per group: along M for the wgrad (WgradBdLoader),
// along N for the forward convolution and dgrad (ConvBdLoader); BDC_ of
// them share a CU (each with its share of the LDS).
template <int DT_, int TM_, int TN_, int TK_, int WM_, int WN_, int MN_, int RBS_ = 64, bool MX_ = false,
          int BDG_ = 0, int BDC_ = 1>
struct TileCfg {
  static constexpr int DT = DT_, TM = TM_, TN = TN_, TK = TK_, WM = WM_, WN = WN_, MN = MN_;
  static constexpr bool MX = MX_;
  static constexpr int SCB = MX_ ? 4 : 0;  // scale bytes per row in a slot
  static constexpr int ESZ = DT == DT_F8 || DT == DT_BF8 ? 1 : 2;
  static constexpr int RB = TK * ESZ;  // LDS row bytes (K contiguous)
  static constexpr int CPR = RB / 16;  // 16-byte chunks per row
  static constexpr int NW = WM * WN, THREADS = 64 * NW;
  static constexpr int WTM = TM / WM, WTN = TN / WN;
  static constexpr int FM = WTM / MN, FN = WTN / MN;
  typedef Mfma<DT, MN> Op;
  typedef typename Op::acc_t acc_t;
  static constexpr int NACC = Op::NACC;
  static constexpr int OPC = Op::OPB / 16;  // 16-byte chunks per operand per lane
  static constexpr int KSTEPS = RB / Op::KB;
  static constexpr int A_BYTES = TM * RB, B_BYTES = TN * RB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  // Epilogue staging: one wave-row of the tile (WTM rows) at a time, rows
  // padded by 16 bytes, fp32 in the worst case.
  static constexpr int EPI_PITCH32 = TN * 4 + 16;
  static constexpr int EPI_BYTES = WTM * EPI_PITCH32;
  static constexpr int LDS = 2 * STAGE > EPI_BYTES ? 2 * STAGE : EPI_BYTES;
  static constexpr int ACC4 = FM * FN * NACC / 4;  // float4 slots per lane
  // Direct-to-LDS pipeline (GEMM): a MAC iteration is cut into SUBS
  // sub-stages of RBS bytes of K per row, held in a ring of NST sub-stage
  // buffers.
  static constexpr int RBS = RBS_;
  static constexpr int SUBS = RB / RBS;
  static constexpr int KSS = RBS / Op::KB;  // MFMA k-steps per sub-stage
  static constexpr int SST = (TM + TN) * RBS;
  static constexpr int NST = (4 * SST <= 128 * 1024) ? 4 : 2;
  static constexpr int LDS_DMA = NST * SST > EPI_BYTES ? NST * SST : EPI_BYTES;
  // Grouped direct-to-LDS pipeline (128-byte rows, i.e. whole cache lines
  // per row and MAC iteration): each ring slot holds one operand tile (A or
  // B) of one MAC iteration.  Large tiles take the whole LDS; 128-row tiles
  // stay within half of it so that two CTAs fit on a CU.  Square tiles use
  // one ring of NSLOT equal slots; when TM != TN the A and B tiles differ in
  // size and each gets a ring of its own, NSLOT / 2 slots sized to fit, so
  // the LDS holds more iterations ahead.
  static constexpr int SLOT_A = TM * (RB + SCB), SLOT_B = TN * (RB + SCB);
  static constexpr bool SPLIT = TM != TN;
  static constexpr int SLOT = (TM > TN ? TM : TN) * (RB + SCB);
  static constexpr int LDS_BUDGET = TM * TN >= 256 * 128 ? 160 * 1024 : 80 * 1024;
  static constexpr int RING_D = LDS_BUDGET / (SLOT_A + SLOT_B);  // iterations, split rings
  static constexpr int NSLOT = SPLIT ? (2 * RING_D > 8 ? 8 : 2 * RING_D)
                                     : (LDS_BUDGET / SLOT > 8 ? 8 : LDS_BUDGET / SLOT);
  static constexpr int RING_BYTES = SPLIT ? NSLOT / 2 * (SLOT_A + SLOT_B) : NSLOT * SLOT;
  static constexpr bool GROUPED = RB == 128 && NSLOT >= 4 && KSTEPS % 2 == 0;
  static constexpr int LDS_GRP = RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES;
  // Spread the refill DMAs among the MFMAs (256x256 tiles: one resident
  // CTA per CU); otherwise issue them in one burst after the barrier, which
  // keeps them further ahead (two CTAs per CU hide the burst).
  static constexpr bool SPREAD = TM == 256 && TN == 256 && !MX_;
  // Block-diagonal tile: its loader lays out one ring entry per MAC
  // iteration (Loader::ENTRY bytes, Loader::D entries in BD_LDS bytes).
  static constexpr int BDG = BDG_;
  static constexpr int BD_LDS = 160 * 1024 / BDC_;
  // Resident CTAs per CU the register allocation must allow: tiles of up
  // to 128x128 keep two (their LDS fits twice), larger ones take the CU,
  // block-diagonal ones BDC_ each.
  static constexpr int MIN_CTAS = BDG_ ? BDC_ : TM * TN <= 128 * 128 ? 2 : 1;
  static_assert(RB == 64 || RB == 128, "LDS row layout");
  static_assert(FM >= 1 && FN >= 1 && WTM % MN == 0 && WTN % MN == 0, "wave tile");
  static_assert(KSTEPS >= 1 && RB % Op::KB == 0, "k steps");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(BDG_ == 0 || (MN == 16 && ((TM == 16 * BDG_ && WM == BDG_ && WN == 1) ||
                                            (TN == 16 * BDG_ && WN == BDG_ && WM == 1))),
                "block-diagonal tile: one wave per group");
};

// ---------------------------------------------------------------------------
// GEMM (rcr) operand loader: rows of A (M x K, row-major) and of B^T (N x K,
// i.e. column-major B) are K-contiguous; each thread moves 16-byte chunks.
template <class Cfg>
struct GemmLoader {
  static constexpr bool kDma = false, kGrouped = false, kTrans = false;
  // Chunk j = tid + THREADS*u sits at row j / CPR, chunk j % CPR; THREADS is
  // a multiple of CPR, so unit u only moves the row by u * RSTEP.
  static constexpr int UA = (Cfg::TM * Cfg::CPR) / Cfg::THREADS;
  static constexpr int UB = (Cfg::TN * Cfg::CPR) / Cfg::THREADS;
  static constexpr int RSTEP = Cfg::THREADS / Cfg::CPR;
  static_assert(UA * Cfg::THREADS == Cfg::TM * Cfg::CPR, "A chunks per thread");
  static_assert(UB * Cfg::THREADS == Cfg::TN * Cfg::CPR, "B chunks per thread");
  static_assert(Cfg::THREADS % Cfg::CPR == 0 && RSTEP % 16 == 0, "row step keeps the swizzle");

  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t lda_b, ldb_b, kbytes, cb;  // row pitches, K extent, this thread's chunk byte
  int row0, rows_a, rows_b;
  i32x4 ra_regs[UA], rb_regs[UB];

  SKG_DEV void init(const GemmParams& g, int m0, int n0, int tid) {
    rows_a = g.M - m0;
    rows_b = g.N - n0;
    ra = make_rsrc(g.A + (size_t)m0 * g.lda_b, (uint32_t)min((int64_t)rows_a * g.lda_b, (int64_t)0x7fffffff));
    rb = make_rsrc(g.B + (size_t)n0 * g.ldb_b, (uint32_t)min((int64_t)rows_b * g.ldb_b, (int64_t)0x7fffffff));
    lda_b = g.lda_b;
    ldb_b = g.ldb_b;
    kbytes = (uint32_t)g.K * Cfg::ESZ;
    row0 = tid / Cfg::CPR;
    cb = (uint32_t)(tid % Cfg::CPR) * 16;
  }

  SKG_DEV void load(int it) {
    const uint32_t kb = (uint32_t)it * Cfg::RB + cb;
    const bool kok = kb < kbytes;
#pragma unroll
    for (int u = 0; u < UA; ++u) {
      const int row = row0 + u * RSTEP;
      const bool ok = kok && row < rows_a;
      ra_regs[u] = buffer_load16(ra, ok ? (uint32_t)row * lda_b + kb : kOOB);
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int row = row0 + u * RSTEP;
      const bool ok = kok && row < rows_b;
      rb_regs[u] = buffer_load16(rb, ok ? (uint32_t)row * ldb_b + kb : kOOB);
    }
  }

  SKG_DEV void store(SKG_LDS char* stage, int tid) const {
    const uint32_t off = lds_off<Cfg::RB>(tid / Cfg::CPR, tid % Cfg::CPR);
#pragma unroll
    for (int u = 0; u < UA; ++u)
      *(SKG_LDS i32x4*)(stage + off + u * RSTEP * Cfg::RB) = ra_regs[u];
#pragma unroll
    for (int u = 0; u < UB; ++u)
      *(SKG_LDS i32x4*)(stage + Cfg::A_BYTES + off + u * RSTEP * Cfg::RB) = rb_regs[u];
  }
};

// GEMM operand loaders, direct to LDS.  Each wave-instruction fills 1024
// contiguous bytes of LDS (lane i at +16*i), so a thread fetches the global
// chunk that the swizzled layout keeps in its LDS slot.  For slot
// u*THREADS + tid the row is row(tid) + u*(THREADS/CPR) and the chunk does
// not depend on u, so a thread keeps one offset per operand, the row step
// is uniform, and one K limit serves all its chunks.  Rows past the edge of
// the matrix lie past the end of the buffer resource and read as zero, as
// do chunks past K (sent to an out-of-range offset).
template <class Cfg, int RBX>
struct DmaRows {
  static constexpr int CPR = RBX / 16;              // chunks per row
  static constexpr int STEP = Cfg::THREADS / CPR;   // rows between a thread's chunks
  static constexpr int UA = Cfg::TM / STEP, UB = Cfg::TN / STEP;
  static_assert(UA * STEP == Cfg::TM && UB * STEP == Cfg::TN, "DMA mapping");

  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t offa, offb;      // byte offset of this thread's first chunk
  uint32_t stepa, stepb;    // STEP rows, in bytes (uniform)
  uint32_t lim;             // K bytes this thread's chunk may reach before the tail
  int wave;

  SKG_DEV void init(const GemmParams& g, int m0, int n0, int tid) {
    const int rows_a = g.M - m0, rows_b = g.N - n0;
    ra = make_rsrc_uniform(g.A + (size_t)m0 * g.lda_b,
                           (uint32_t)min((int64_t)rows_a * g.lda_b, (int64_t)0x7fffffff));
    rb = make_rsrc_uniform(g.B + (size_t)n0 * g.ldb_b,
                           (uint32_t)min((int64_t)rows_b * g.ldb_b, (int64_t)0x7fffffff));
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int row, chunk;
    lds_slot<RBX>(tid, row, chunk);
    offa = (uint32_t)row * g.lda_b + chunk * 16;
    offb = (uint32_t)row * g.ldb_b + chunk * 16;
    stepa = STEP * g.lda_b;
    stepb = STEP * g.ldb_b;
    // Clamped at zero: with K shorter than one LDS row the chunk may start
    // past K, and a wrapped limit would let it read the row's padding.
    lim = (uint32_t)max(g.K * Cfg::ESZ - chunk * 16, 0);
  }

  // RBX bytes of K starting at byte kb of every row, A rows into `la`, B
  // rows into `lb` (either may be skipped).
  template <bool DO_A, bool DO_B>
  SKG_DEV void issue_rows(uint32_t kb, SKG_LDS char* la, SKG_LDS char* lb) const {
    const bool ok = kb < lim;
    if constexpr (DO_A) {
#pragma unroll
      for (int u = 0; u < UA; ++u)
        dma16(ra, lds_addr(la + u * Cfg::THREADS * 16 + wave * 1024), ok ? offa + u * stepa + kb : kOOB);
    }
    if constexpr (DO_B) {
#pragma unroll
      for (int u = 0; u < UB; ++u)
        dma16(rb, lds_addr(lb + u * Cfg::THREADS * 16 + wave * 1024), ok ? offb + u * stepb + kb : kOOB);
    }
  }
};

// Sub-stage pipeline: sub-stage q holds RBS bytes of K for every row of the
// A and B tiles.
template <class Cfg>
struct GemmDmaLoader : DmaRows<Cfg, Cfg::RBS> {
  static constexpr bool kDma = true, kGrouped = false, kTrans = false;
  typedef DmaRows<Cfg, Cfg::RBS> Base;
  static constexpr int LPS = Base::UA + Base::UB;  // instructions per sub-stage

  // Sub-stage q (K bytes [q*RBS, (q+1)*RBS) of the tile) into `stage`.
  SKG_DEV void issue(int q, SKG_LDS char* stage) const {
    this->template issue_rows<true, true>((uint32_t)q * Cfg::RBS, stage, stage + Cfg::TM * Cfg::RBS);
  }
};

// Grouped pipeline: group j of a segment is operand A (j even) or B (j odd)
// of its MAC iteration j/2, RB = 128 bytes of K per row, so every
// wave-instruction reads eight whole 128-byte lines.
template <class Cfg>
struct GemmGrpLoader : DmaRows<Cfg, Cfg::RB> {
  static constexpr bool kDma = true, kGrouped = true, kTrans = false;
  typedef DmaRows<Cfg, Cfg::RB> Base;
  static_assert(Cfg::RB == 128, "whole-line rows");

  // Where the two groups refilled during one MAC iteration go: B of one
  // iteration (kb_b: its first K byte) into slot_b, A of the next into
  // slot_a.  A group that is not `live` (past the segment) reads nothing
  // and zero-fills its slot, which nobody reads.
  struct Refill {
    SKG_LDS char* slot_b;
    SKG_LDS char* slot_a;
    int it_b, it_a;  // MAC iterations (tile-relative) of the two groups
    bool live_b, live_a;
  };

  // DMA instruction N of a refill: [0, UB) for the B group, then A.
  template <int N>
  SKG_DEV void refill(const Refill& r) const {
    if constexpr (N < Base::UB) {
      const uint32_t kb = (uint32_t)r.it_b * Cfg::RB;
      const bool ok = r.live_b && kb < this->lim;
      dma16(this->rb, lds_addr(r.slot_b + N * Cfg::THREADS * 16 + this->wave * 1024),
            ok ? this->offb + N * this->stepb + kb : kOOB);
    } else {
      constexpr int U = N - Base::UB;
      const uint32_t kb = (uint32_t)r.it_a * Cfg::RB;
      const bool ok = r.live_a && kb < this->lim;
      dma16(this->ra, lds_addr(r.slot_a + U * Cfg::THREADS * 16 + this->wave * 1024),
            ok ? this->offa + U * this->stepa + kb : kOOB);
    }
  }

  // Group j (A when even, B when odd) of MAC iteration `it` into `slot`;
  // zero fill when not `live`.
  SKG_DEV void issue_live(int j, int it, SKG_LDS char* slot, bool live) const {
    const uint32_t kb = live ? (uint32_t)it * Cfg::RB : 0xffffffffu;
    if ((j & 1) == 0)
      this->template issue_rows<true, false>(kb, slot, nullptr);
    else
      this->template issue_rows<false, true>(kb, nullptr, slot);
  }
  SKG_DEV void issue(int j, int it, SKG_LDS char* slot) const { issue_live(j, it, slot, true); }
  // Per-refill set-up once its groups are known (nothing for plain rows).
  SKG_DEV void finish_refill(Refill&) const {}
};

// GEMM with OCP MX block scales (fp8 / bf8, K a multiple of the tile's K):
// each group also carries the E8M0 scale words of its rows for the MAC
// iteration (4 bytes = the 4 blocks of 32 K elements a 128-byte row holds,
// at row*(K/32) + it*4 of the row-major M x K/32 or N x K/32 scale array),
// one 4-byte direct-to-LDS instruction per wave placed after the slot's row
// data, so the engine's waits and barriers order them with the tile.
template <class Cfg>
struct MxGrpLoader : GemmGrpLoader<Cfg> {
  typedef GemmGrpLoader<Cfg> Base;
  typedef DmaRows<Cfg, Cfg::RB> Rows;
  static constexpr bool kMx = true;
  static_assert(Cfg::MX && Cfg::RB == 128 && Cfg::TK == 128, "MX: 4 scale blocks per 128-byte row");
  static_assert(Cfg::TM % 64 == 0 && Cfg::TN % 64 == 0 && (Cfg::TM / 64) <= Cfg::NW &&
                    Cfg::NW % (Cfg::TM / 64) == 0 && Cfg::NW % (Cfg::TN / 64) == 0,
                "one 64-row scale chunk per wave");
  // DMA instructions per group and thread: the rows plus one scale word.
  static constexpr int UA = Rows::UA + 1, UB = Rows::UB + 1;

  __amdgpu_buffer_rsrc_t rsa, rsb;
  uint32_t sofa, sofb;  // this lane's scale-row byte offset (row * K/32)
  int cha, chb;         // 64-row chunk of the tile this wave's scale DMA fills

  SKG_DEV void init(const GemmParams& g, int m0, int n0, int tid) {
    Base::init(g, m0, n0, tid);
    const uint32_t kb32 = (uint32_t)g.K / 32;
    const char* sa = (const char*)g.sa;
    const char* sb = (const char*)g.sb;
    rsa = make_rsrc(sa + (size_t)m0 * kb32, (uint32_t)(g.M - m0) * kb32);
    rsb = make_rsrc(sb + (size_t)n0 * kb32, (uint32_t)(g.N - n0) * kb32);
    const int lane = tid & 63;
    cha = this->wave % (Cfg::TM / 64);
    chb = this->wave % (Cfg::TN / 64);
    sofa = (uint32_t)(cha * 64 + lane) * kb32;
    sofb = (uint32_t)(chb * 64 + lane) * kb32;
  }

  SKG_DEV void scales_a(int it, SKG_LDS char* slot, bool live) const {
    dma4(rsa, lds_addr(slot + Cfg::TM * Cfg::RB + cha * 256), live ? sofa + (uint32_t)it * 4 : kOOB);
  }
  SKG_DEV void scales_b(int it, SKG_LDS char* slot, bool live) const {
    dma4(rsb, lds_addr(slot + Cfg::TN * Cfg::RB + chb * 256), live ? sofb + (uint32_t)it * 4 : kOOB);
  }

  SKG_DEV void issue_live(int j, int it, SKG_LDS char* slot, bool live) const {
    Base::issue_live(j, it, slot, live);
    if ((j & 1) == 0)
      scales_a(it, slot, live);
    else
      scales_b(it, slot, live);
  }
  SKG_DEV void issue(int j, int it, SKG_LDS char* slot) const { issue_live(j, it, slot, true); }

  // DMA instruction N of a refill spread among the MFMAs, in the order of
  // issue_live: the B group's rows, its scale word, then the A group's.
  template <int N>
  SKG_DEV void refill(const typename Base::Refill& r) const {
    if constexpr (N < Rows::UB)
      Base::template refill<N>(r);
    else if constexpr (N == Rows::UB)
      scales_b(r.it_b, r.slot_b, r.live_b);
    else if constexpr (N < UB + Rows::UA)
      Base::template refill<Rows::UB + (N - UB)>(r);
    else
      scales_a(r.it_a, r.slot_a, r.live_a);
  }
};

// ---------------------------------------------------------------------------
// wgrad operand loader.  GEMM-A = dY^T (row m = output channel of the group,
// K index q = (image, ho, wo)); GEMM-B^T = im2col(X) (row = (r, s, c') with c'
// fastest, K index q).  Both are contiguous along M / N in memory (NHWC), so
// a thread loads an 8 x 8 block -- 8 consecutive q, 16 bytes (8 channels)
// each -- transposes it in registers and writes 8 K-contiguous 16-byte chunks.
// Zero padding, ragged channel tails and the reduction tail come back as zero
// from out-of-range buffer offsets.
template <class Cfg>
struct WgradLoader {
  static constexpr bool kDma = false, kGrouped = false, kTrans = false;
  static_assert(Cfg::ESZ == 2, "wgrad runs on 16-bit inputs");
  static constexpr int QB = Cfg::TK / 8;             // 8-wide q blocks per K step
  static constexpr int NA = (Cfg::TM / 8) * QB;      // blocks of the A tile
  static constexpr int NB = (Cfg::TN / 8) * QB;      // blocks of the B tile
  static constexpr int U = (NA + NB + Cfg::THREADS - 1) / Cfg::THREADS;

  __amdgpu_buffer_rsrc_t rx, rdy;
  int kind[U];        // 0: none, 1: A block, 2: B block
  int lrow[U], qc[U]; // first tile row of the block, q block index
  uint32_t base[U];   // A: channel byte offset in a dY row; B: channel byte offset in an X pixel
  int tap_r[U], tap_s[U];
  bool ok[U];         // rows of the block exist
  i32x4 regs[U][8];

  SKG_DEV void init(const WgradParams& w, int group, int mrow0, int n0, int tid) {
    rx = make_rsrc(w.X, w.x_bytes);
    rdy = make_rsrc(w.dY, w.dy_bytes);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = tid + Cfg::THREADS * u;
      kind[u] = 0;
      ok[u] = false;
      lrow[u] = 0;
      qc[u] = 0;
      base[u] = 0;
      tap_r[u] = tap_s[u] = 0;
      if (j < NA) {
        kind[u] = 1;
        lrow[u] = (j / QB) * 8;
        qc[u] = j % QB;
        const int m = mrow0 + lrow[u];
        ok[u] = m < w.kpg;
        base[u] = (uint32_t)(group * w.kpg + m) * 2;
      } else if (j < NA + NB) {
        const int jb = j - NA;
        kind[u] = 2;
        lrow[u] = (jb / QB) * 8;
        qc[u] = jb % QB;
        const int nidx = n0 + lrow[u];
        ok[u] = nidx < w.gemm_n;
        const uint32_t rs = fdiv((uint32_t)nidx, w.div_cpg);
        const int cc = nidx - (int)rs * w.cpg;
        const uint32_t r = fdiv(rs, w.div_s);
        tap_r[u] = (int)r;
        tap_s[u] = (int)(rs - r * w.S);
        base[u] = (uint32_t)(group * w.cpg + cc) * 2;
      }
    }
  }

  SKG_DEV void load(const WgradParams& w, int it) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kind[u] == 0) continue;
      const int q0 = it * Cfg::TK + qc[u] * 8;
      // (image, ho, wo) of q0, then stepped along the 8 consecutive q.
      const uint32_t img0 = fdiv((uint32_t)q0, w.div_howo);
      const int rem = q0 - (int)img0 * w.Ho * w.Wo;
      const uint32_t ho0 = fdiv((uint32_t)rem, w.div_wo);
      int img = (int)img0, ho = (int)ho0, wo = rem - (int)ho0 * w.Wo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = q0 + i;
        uint32_t off = kOOB;
        if (kind[u] == 1) {
          if (ok[u] && q < w.kred) off = (uint32_t)q * (uint32_t)(w.K * 2) + base[u];
          regs[u][i] = buffer_load16(rdy, off);
        } else {
          const int hi = ho * w.sh - w.ph + tap_r[u];
          const int wi = wo * w.sw - w.pw + tap_s[u];
          if (ok[u] && q < w.kred && hi >= 0 && hi < w.H && wi >= 0 && wi < w.W)
            off = (uint32_t)(((img * w.H + hi) * w.W + wi) * w.C) * 2 + base[u];
          regs[u][i] = buffer_load16(rx, off);
        }
        if (++wo == w.Wo) {
          wo = 0;
          if (++ho == w.Ho) {
            ho = 0;
            ++img;
          }
        }
      }
    }
  }

  SKG_DEV void store(SKG_LDS char* stage, int /*tid*/) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kind[u] == 0) continue;
      SKG_LDS char* dst = stage + (kind[u] == 2 ? Cfg::A_BYTES : 0);
      // regs[u][i] holds channels lrow..lrow+7 at q = 8*qc + i; transpose so
      // that row lrow + r holds q = 8*qc .. 8*qc+7.
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        i32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (uint32_t)regs[u][2 * e][r >> 1];
          const uint32_t hi = (uint32_t)regs[u][2 * e + 1][r >> 1];
          o[e] = (int)((r & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16)));
        }
        *(SKG_LDS i32x4*)(dst + lds_off<Cfg::RB>(lrow[u] + r, qc[u])) = o;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Problem policies: tile coordinates, loader set-up and the output window.
// TENSOR: one scale for all of A and one for all of B instead of per-row /
// per-column scales.
template <class Cfg, bool TENSOR = false>
struct GemmProblem {
  typedef GemmParams Params;
  static constexpr int kScaleInc = TENSOR ? 0 : 1;
  typedef typename std::conditional<Cfg::GROUPED, GemmGrpLoader<Cfg>, GemmDmaLoader<Cfg>>::type Loader;

  SKG_DEV static void setup(const Params& g, const KPlan& p, int tile, Loader& ld, OutTile& out,
                               int tid) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    const int m0 = tm * Cfg::TM, n0 = tn * Cfg::TN;
    ld.init(g, m0, n0, tid);
    out = out_tile(g, p, tile);
  }
  SKG_DEV static OutTile out_tile(const Params& g, const KPlan& p, int tile) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    const int m0 = tm * Cfg::TM, n0 = tn * Cfg::TN;
    const int esz = g.dtype_c == DT_F32 ? 4 : 2;
    OutTile o;
    o.base = g.C + ((size_t)m0 * g.ldc + n0) * esz;
    o.sa = g.sa ? g.sa + m0 * kScaleInc : nullptr;
    o.sb = g.sb ? g.sb + n0 * kScaleInc : nullptr;
    o.ld = g.ldc;
    o.rows = g.M - m0;
    o.cols = g.N - n0;
    return o;
  }
  SKG_DEV static int dtype_c(const Params& g) { return g.dtype_c; }
};

// GEMM with MX block scales: scale_a / scale_b are the E8M0 arrays the
// loader moves with the tiles; the epilogue applies no further scale.
template <class Cfg>
struct GemmMxProblem {
  typedef GemmParams Params;
  static constexpr int kScaleInc = 1;
  typedef MxGrpLoader<Cfg> Loader;

  SKG_DEV static void setup(const Params& g, const KPlan& p, int tile, Loader& ld, OutTile& out,
                            int tid) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    ld.init(g, tm * Cfg::TM, tn * Cfg::TN, tid);
    out = out_tile(g, p, tile);
  }
  SKG_DEV static OutTile out_tile(const Params& g, const KPlan& p, int tile) {
    OutTile o = GemmProblem<Cfg>::out_tile(g, p, tile);
    o.sa = nullptr;
    o.sb = nullptr;
    return o;
  }
  SKG_DEV static int dtype_c(const Params& g) { return g.dtype_c; }
};

// Chunk swizzle of the wgrad operand tiles in LDS.  A tile holds one row
// per reduction index q (P bytes: the tile's channels, contiguous as in
// NHWC memory); the 16-byte chunk index is XORed with a function of the row
// so that the transposing fragment reads -- four consecutive rows of 32
// bytes per group of 16 lanes -- hit distinct banks (64 banks of 4 bytes).
template <int P, int MN>
SKG_DEV int tr_swz(int row) {
  static_assert(P >= 256 || (P == 128) || (P == 64 && MN == 16), "wgrad tile pitch");
  if constexpr (P >= 256)
    return (4 * (row & 1)) ^ (8 * ((row >> 1) & 1));
  else if constexpr (P == 128 && MN == 32)
    return 4 * ((row >> 1) & 1);
  else if constexpr (P == 128)
    return (2 * ((row >> 1) & 1)) ^ (4 * ((row >> 3) & 1));
  else
    return 2 * ((row >> 3) & 1);
}

// wgrad operand loader for the grouped pipeline, direct to LDS without any
// transposition: group j of a segment is the A tile (j even: rows of dY,
// the tile's output channels of TK consecutive q) or the B tile (j odd:
// rows of im2col(X), the tile's (r, s, c') columns) of MAC iteration j/2.
// Every row is one contiguous run of channels in NHWC memory.  The MFMA
// fragments, which want the reduction index contiguous per lane, are read
// back with the gfx950 transposing LDS read.  Zero padding, rows past the
// reduction and channels past a group come back as zero (out-of-range
// buffer offsets).
template <class Cfg>
struct WgradGrpLoader {
  static constexpr bool kDma = true, kGrouped = true, kTrans = true;
  static_assert(Cfg::ESZ == 2, "wgrad runs on 16-bit inputs");
  static constexpr int PA = Cfg::TM * 2, PB = Cfg::TN * 2;  // bytes per q row
  static constexpr int CPRA = PA / 16, CPRB = PB / 16;
  static constexpr int STEPA = Cfg::THREADS / CPRA, STEPB = Cfg::THREADS / CPRB;
  static constexpr int UA = Cfg::TK / STEPA, UB = Cfg::TK / STEPB;  // instructions per group
  static_assert(Cfg::THREADS % CPRA == 0 && Cfg::THREADS % CPRB == 0 && UA * STEPA == Cfg::TK &&
                    UB * STEPB == Cfg::TK && UA >= 1 && UB >= 1,
                "wgrad DMA mapping");

  __amdgpu_buffer_rsrc_t rx, rdy;
  int wave;
  // Row d (< TK) of an iteration is reduction index q0 + d.  The CTA-uniform
  // q0 is split into (image, ho, wo) once per iteration on the scalar unit;
  // each lane holds the same split of its own rows d_u = row + u * STEP
  // (radix Wo, then Ho) and adds the two digit by digit, with at most one
  // carry per digit, so the hot loop needs no division and no 32-bit
  // multiply.  Byte offsets follow in uint32 arithmetic: X offset of
  // (img, ho, wo) shifted by the thread's tap = img*HWc2 + ho*sh*Wc2 +
  // wo*sw*c2 + ((r - ph)*W + (s - pw))*c2 + channel bytes, where the last
  // two terms and the lane's own digits are folded into boff[u].
  uint32_t aoff_l;     // rowa * K*2 + A channel bytes
  int qrow_a, qrow_b;  // the lane's first row, or past any reduction when its chunk is empty
  uint32_t boff[Cfg::TK / STEPB];
  uint32_t bwo[Cfg::TK / STEPB], bho[Cfg::TK / STEPB];  // digits of the lane's rows
  int tr_ph, ts_pw;  // r - ph, s - pw of the lane's tap
  // problem constants (uniform)
  uint32_t k2, hwc2, shwc2, swc2, cw1, cw2, howo;
  int kred, H, W, Ho, Wo, sh, sw;
  FastDiv div_howo, div_wo;

  SKG_DEV void init(const WgradParams& w, int group, int mrow0, int n0, int tid) {
    rx = make_rsrc(w.X, w.x_bytes);
    rdy = make_rsrc(w.dY, w.dy_bytes);
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    k2 = (uint32_t)w.K * 2;
    const uint32_t c2 = (uint32_t)w.C * 2;
    kred = w.kred;
    H = w.H;
    W = w.W;
    Ho = w.Ho;
    Wo = w.Wo;
    sh = w.sh;
    sw = w.sw;
    howo = (uint32_t)(w.Ho * w.Wo);
    hwc2 = (uint32_t)(w.H * w.W) * c2;
    shwc2 = (uint32_t)(w.sh * w.W) * c2;
    swc2 = (uint32_t)w.sw * c2;
    cw1 = shwc2 - (uint32_t)w.Wo * swc2;  // wo wrapped: wo - Wo, ho + 1
    cw2 = hwc2 - (uint32_t)w.Ho * shwc2;  // ho wrapped: ho - Ho, img + 1
    div_howo = w.div_howo;
    div_wo = w.div_wo;
    constexpr int kPast = 1 << 30;
    const int rowa = tid / CPRA;
    const int lca = (tid % CPRA) ^ tr_swz<PA, Cfg::MN>(rowa);
    const int m = mrow0 + lca * 8;
    qrow_a = m < w.kpg ? rowa : kPast;
    aoff_l = (uint32_t)rowa * k2 + (uint32_t)(group * w.kpg + m) * 2;
    const int rowb = tid / CPRB;
    const int lcb = (tid % CPRB) ^ tr_swz<PB, Cfg::MN>(rowb);
    const int nidx = n0 + lcb * 8;
    qrow_b = nidx < w.gemm_n ? rowb : kPast;
    const uint32_t rs = fdiv((uint32_t)nidx, w.div_cpg);
    const int cc = nidx - (int)rs * w.cpg;
    const uint32_t r = fdiv(rs, w.div_s);
    tr_ph = (int)r - w.ph;
    ts_pw = (int)(rs - r * w.S) - w.pw;
    const uint32_t tap = (uint32_t)tr_ph * ((uint32_t)w.W * c2) + (uint32_t)ts_pw * c2 +
                         (uint32_t)(group * w.cpg + cc) * 2;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const uint32_t d = (uint32_t)(rowb + u * STEPB);
      const uint32_t t = fdiv(d, div_wo);
      const uint32_t img = fdiv(t, w.div_ho);
      bwo[u] = d - t * (uint32_t)Wo;
      bho[u] = t - img * (uint32_t)Ho;
      boff[u] = img * hwc2 + bho[u] * shwc2 + bwo[u] * swc2 + tap;
    }
  }

  // The scalar part of iteration it's rows.
  struct QBase {
    uint32_t wo0, ho0, boff, aoff;
    int lim;  // rows d < lim are inside the reduction (0 when not live)
  };
  SKG_DEV QBase qbase(int it, bool live) const {
    const uint32_t q0 = __builtin_amdgcn_readfirstlane((uint32_t)it * Cfg::TK);
    const uint32_t img = fdiv(q0, div_howo);
    const uint32_t rem = q0 - img * howo;
    const uint32_t ho = fdiv(rem, div_wo);
    QBase b;
    b.wo0 = rem - ho * (uint32_t)Wo;
    b.ho0 = ho;
    b.boff = img * hwc2 + ho * shwc2 + b.wo0 * swc2;
    b.aoff = q0 * k2;
    b.lim = live ? kred - (int)q0 : 0;
    return b;
  }

  // dY row of this thread's A chunk u, or kOOB.
  SKG_DEV uint32_t a_off(const QBase& b, int u) const {
    const uint32_t off = aoff_l + (b.aoff + (uint32_t)(u * STEPA) * k2);
    return qrow_a < b.lim - u * STEPA ? off : kOOB;
  }
  // X pixel of this thread's B row u shifted by its filter tap, or kOOB
  // (zero padding, past the reduction, past the group's channels).
  SKG_DEV uint32_t b_off(const QBase& b, int u) const {
    uint32_t wo = b.wo0 + bwo[u];
    const bool c1 = wo >= (uint32_t)Wo;
    wo = c1 ? wo - (uint32_t)Wo : wo;
    uint32_t ho = b.ho0 + bho[u] + (c1 ? 1u : 0u);
    const bool c2 = ho >= (uint32_t)Ho;
    ho = c2 ? ho - (uint32_t)Ho : ho;
    const uint32_t off = b.boff + boff[u] + (c1 ? cw1 : 0u) + (c2 ? cw2 : 0u);
    const int hi = __mul24((int)ho, sh) + tr_ph;
    const int wi = __mul24((int)wo, sw) + ts_pw;
    const bool ok = ((uint32_t)hi < (uint32_t)H) & ((uint32_t)wi < (uint32_t)W) &
                    (qrow_b < b.lim - u * STEPB);
    return ok ? off : kOOB;
  }

  template <bool IS_A>
  SKG_DEV void issue_group(int it, SKG_LDS char* slot, bool live) const {
    const QBase b = qbase(it, live);
    if constexpr (IS_A) {
#pragma unroll
      for (int u = 0; u < UA; ++u)
        dma16(rdy, lds_addr(slot + u * Cfg::THREADS * 16 + wave * 1024), a_off(b, u));
    } else {
#pragma unroll
      for (int u = 0; u < UB; ++u)
        dma16(rx, lds_addr(slot + u * Cfg::THREADS * 16 + wave * 1024), b_off(b, u));
    }
  }

  // Group j (A when even, B when odd) of MAC iteration `it` into `slot`;
  // zero fill when not `live`.
  SKG_DEV void issue_live(int j, int it, SKG_LDS char* slot, bool live) const {
    if ((j & 1) == 0)
      issue_group<true>(it, slot, live);
    else
      issue_group<false>(it, slot, live);
  }
  SKG_DEV void issue(int j, int it, SKG_LDS char* slot) const { issue_live(j, it, slot, true); }

  // A refill spread among the MFMAs: the B group of iteration it_b into
  // slot_b (DMA instructions [0, UB)), then the A group of it_a.
  struct Refill {
    SKG_LDS char* slot_b;
    SKG_LDS char* slot_a;
    int it_b, it_a;
    bool live_b, live_a;
    QBase qb, qa;
  };
  SKG_DEV void finish_refill(Refill& r) const {
    r.qb = qbase(r.it_b, r.live_b);
    r.qa = qbase(r.it_a, r.live_a);
  }
  template <int N>
  SKG_DEV void refill(const Refill& r) const {
    if constexpr (N < UB) {
      dma16(rx, lds_addr(r.slot_b + N * Cfg::THREADS * 16 + wave * 1024), b_off(r.qb, N));
    } else {
      constexpr int U = N - UB;
      dma16(rdy, lds_addr(r.slot_a + U * Cfg::THREADS * 16 + wave * 1024), a_off(r.qa, U));
    }
  }
};

template <class Cfg>
struct WgradProblem {
  static constexpr int kScaleInc = 1;  // no scales
  typedef WgradParams Params;
  typedef typename std::conditional<Cfg::GROUPED, WgradGrpLoader<Cfg>, WgradLoader<Cfg>>::type Loader;

  SKG_DEV static void setup(const Params& w, const KPlan& p, int tile, Loader& ld, OutTile& out,
                               int tid) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    const int group = tm / w.mt_per_group;
    const int mrow0 = (tm - group * w.mt_per_group) * Cfg::TM;
    ld.init(w, group, mrow0, tn * Cfg::TN, tid);
    out = out_tile(w, p, tile);
  }
  SKG_DEV static OutTile out_tile(const Params& w, const KPlan& p, int tile) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    const int group = tm / w.mt_per_group;
    const int mrow0 = (tm - group * w.mt_per_group) * Cfg::TM;
    const int n0 = tn * Cfg::TN;
    OutTile o;
    // dW is K x (R*S*Cpg) row-major (KRSC): GEMM column n0 of output channel
    // k sits at k*gemm_n + n0.
    o.base = (char*)(w.dW + (size_t)(group * w.kpg + mrow0) * w.gemm_n + n0);
    o.sa = nullptr;
    o.sb = nullptr;
    o.ld = w.gemm_n;
    o.rows = w.kpg - mrow0;
    o.cols = w.gemm_n - n0;
    return o;
  }
  SKG_DEV static void load(const Params& w, Loader& ld, int it) { ld.load(w, it); }
  SKG_DEV static int dtype_c(const Params&) { return DT_F32; }
};

// ---------------------------------------------------------------------------
// Block-diagonal grouped wgrad (16 input and 16 output channels per group):
// the tile's TM output channels are BDG whole groups, and their input
// channels are the same index range [k0, k0 + TM).  Row k of the tile only
// meets its own group's input channels, so the tile is not a dense GEMM
// tile: wave w owns group w, i.e. rows [16w, 16w + 16), and all TN = 16 *
// taps columns, whose B fragments come from the same 16 channels of each
// tap's plane.  MAC iteration `it` covers reduction rows q0 + d, d < TK:
// the A tile holds dY[q][k0 .. k0+TM) per row, plane t holds X at pixel q
// shifted by filter tap tap0 + t, channels [k0, k0+TM); every row of either
// is one contiguous run of TM * 2 bytes (a whole 128-byte line for TM =
// 64).  Each thread moves the same (row, chunk) of the A tile and of every
// plane: it splits its row's reduction index once per iteration, and the
// taps only add wave-uniform offsets.  Padding, taps past R*S, rows past the
// reduction and channels past C come back as zero (out-of-range buffer
// offsets).
template <class Cfg>
struct WgradBdLoader {
  static constexpr bool kDma = true, kGrouped = false, kTrans = true;
  static_assert(Cfg::ESZ == 2 && Cfg::BDG > 0, "block-diagonal tile");
  static constexpr int PA = Cfg::TM * 2, PB = PA;  // bytes per q row
  // One MAC iteration: the A tile, then one plane per filter tap, in a
  // ring of D entries filling the LDS.
  static constexpr int TAPS = Cfg::TN / 16, PLANE = Cfg::TK * PA;
  static constexpr int ENTRY = PLANE * (1 + TAPS);
  static constexpr int EPI = 0;  // copy-out straight from the accumulators
  static constexpr int D = Cfg::BD_LDS / ENTRY > 6 ? 6 : Cfg::BD_LDS / ENTRY;
  static_assert(D >= 2, "two ring entries at least");
  static constexpr int CPR = PA / 16;
  static_assert(Cfg::THREADS == Cfg::TK * CPR, "one 16-byte chunk per thread, tile and plane");
  static constexpr int UA = 1, UB = TAPS;  // DMA instructions per thread and iteration

  __amdgpu_buffer_rsrc_t rx, rdy;
  int wave, row;
  uint32_t coff;          // the thread's channel bytes
  bool chan_ok;           // its chunk lies inside C
  uint32_t lwo, lho;      // digits (radix Wo, then Ho) of its row
  uint32_t loff;          // X offset of those digits (image folded in)
  int tr[TAPS], ts[TAPS];  // r - ph and s - pw of each plane's tap (past R*S: never in range)
  uint32_t toff[TAPS];    // ((r - ph) * W + (s - pw)) * C * 2
  uint32_t k2, hwc2, shwc2, swc2, cw1, cw2, howo;
  int kred, H, W, Ho, Wo, sh, sw;
  FastDiv div_howo, div_wo;

  SKG_DEV void init(const WgradParams& w, int k0, int tap0, int tid) {
    rx = make_rsrc(w.X, w.x_bytes);
    rdy = make_rsrc(w.dY, w.dy_bytes);
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    k2 = (uint32_t)w.K * 2;
    const uint32_t c2 = (uint32_t)w.C * 2;
    kred = w.kred;
    H = w.H;
    W = w.W;
    Ho = w.Ho;
    Wo = w.Wo;
    sh = w.sh;
    sw = w.sw;
    howo = (uint32_t)(w.Ho * w.Wo);
    hwc2 = (uint32_t)(w.H * w.W) * c2;
    shwc2 = (uint32_t)(w.sh * w.W) * c2;
    swc2 = (uint32_t)w.sw * c2;
    cw1 = shwc2 - (uint32_t)w.Wo * swc2;  // wo wrapped: wo - Wo, ho + 1
    cw2 = hwc2 - (uint32_t)w.Ho * shwc2;  // ho wrapped: ho - Ho, img + 1
    div_howo = w.div_howo;
    div_wo = w.div_wo;
    row = tid / CPR;
    const int chunk = (tid % CPR) ^ tr_swz<PA, Cfg::MN>(row);
    const int ch = k0 + chunk * 8;
    chan_ok = ch < w.C;  // C == K: 16 channels in and out per group
    coff = (uint32_t)ch * 2;
    const uint32_t t = fdiv((uint32_t)row, div_wo);
    const uint32_t img = fdiv(t, w.div_ho);
    lwo = (uint32_t)row - t * (uint32_t)Wo;
    lho = t - img * (uint32_t)Ho;
    loff = img * hwc2 + lho * shwc2 + lwo * swc2;
    const int rs = w.R * w.S;
#pragma unroll
    for (int j = 0; j < TAPS; ++j) {
      const int tap = tap0 + j;
      const int r = (int)fdiv((uint32_t)tap, w.div_s);
      const int sx = tap - r * w.S;
      tr[j] = tap < rs ? r - w.ph : (1 << 30);
      ts[j] = sx - w.pw;
      toff[j] = (uint32_t)(r - w.ph) * ((uint32_t)w.W * c2) + (uint32_t)(sx - w.pw) * c2;
    }
  }

  // The scalar split of iteration it's first row, and the thread's row.
  struct QBase {
    uint32_t wo, ho, pix;  // the thread's output position and its X offset (no tap)
    uint32_t aoff;         // dY offset of the thread's row and chunk
    bool ok;               // row inside the reduction and chunk inside C
  };
  SKG_DEV QBase qbase(int it) const {
    const uint32_t q0 = __builtin_amdgcn_readfirstlane((uint32_t)it * Cfg::TK);
    const uint32_t img = fdiv(q0, div_howo);
    const uint32_t rem = q0 - img * howo;
    const uint32_t ho0 = fdiv(rem, div_wo);
    const uint32_t wo0 = rem - ho0 * (uint32_t)Wo;
    const uint32_t base = img * hwc2 + ho0 * shwc2 + wo0 * swc2;
    QBase b;
    uint32_t wo = wo0 + lwo;
    const bool c1 = wo >= (uint32_t)Wo;
    wo = c1 ? wo - (uint32_t)Wo : wo;
    uint32_t ho = ho0 + lho + (c1 ? 1u : 0u);
    const bool c2 = ho >= (uint32_t)Ho;
    ho = c2 ? ho - (uint32_t)Ho : ho;
    b.wo = wo;
    b.ho = ho;
    b.pix = base + loff + (c1 ? cw1 : 0u) + (c2 ? cw2 : 0u) + coff;
    b.aoff = (q0 + (uint32_t)row) * k2 + coff;
    b.ok = chan_ok & ((int)q0 + row < kred);
    return b;
  }

  SKG_DEV uint32_t a_off(const QBase& b) const { return b.ok ? b.aoff : kOOB; }
  SKG_DEV uint32_t b_off(const QBase& b, int j) const {
    const int hi = __mul24((int)b.ho, sh) + tr[j];
    const int wi = __mul24((int)b.wo, sw) + ts[j];
    const bool ok = b.ok & ((uint32_t)hi < (uint32_t)H) & ((uint32_t)wi < (uint32_t)W);
    return ok ? b.pix + toff[j] : kOOB;
  }

  // MAC iteration `it` into the ring entry at `e`: the A tile, then the
  // tap planes.
  SKG_DEV void issue_iter(int it, SKG_LDS char* e) const {
    const QBase b = qbase(it);
    dma16(rdy, lds_addr(e + wave * 1024), a_off(b));
#pragma unroll
    for (int j = 0; j < TAPS; ++j) dma16(rx, lds_addr(e + (1 + j) * PLANE + wave * 1024), b_off(b, j));
  }
};

template <class Cfg>
struct WgradBdProblem {
  static constexpr int kScaleInc = 1;  // no scales
  typedef WgradParams Params;
  typedef WgradBdLoader<Cfg> Loader;

  SKG_DEV static void setup(const Params& w, const KPlan& p, int tile, Loader& ld, OutTile& out,
                               int tid) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    ld.init(w, tm * Cfg::TM, tn * Loader::TAPS, tid);
    out = out_tile(w, p, tile);
  }
  SKG_DEV static OutTile out_tile(const Params& w, const KPlan& p, int tile) {
    const int tm = p.tile_row(tile), tn = tile - tm * p.tiles_n;
    const int k0 = tm * Cfg::TM, n0 = tn * Cfg::TN;
    OutTile o;
    // dW is K x (R*S*16) row-major; the tile's rows are output channels
    // k0.., its columns (tap, channel) entries n0.. of each row's own group.
    o.base = (char*)(w.dW + (size_t)k0 * w.gemm_n + n0);
    o.sa = nullptr;
    o.sb = nullptr;
    o.ld = w.gemm_n;
    o.rows = w.K - k0;
    o.cols = w.gemm_n - n0;
    return o;
  }
  SKG_DEV static int dtype_c(const Params&) { return DT_F32; }
};

// ---------------------------------------------------------------------------
// Fix-up families: each kernel instance carries the code of one, so the
// epilogue of the other does not take part in its register allocation.
//   FIX_HANDOFF: linear, tree and reduce-scatter (partials handed on
//                through flags);
//   FIX_ATOMIC:  atomic and workspace (fp32 atomics, nothing waits).
// Data-parallel-only launches use FIX_ATOMIC (FIX_HANDOFF on MX tiles).
enum { FIX_HANDOFF = 0, FIX_ATOMIC = 1 };

// Loaders that move MX block scales with the tiles declare kMx.
template <class L, class = void>
struct LoaderMx {
  static constexpr bool value = false;
};
template <class L>
struct LoaderMx<L, std::void_t<decltype(L::kMx)>> {
  static constexpr bool value = L::kMx;
};

// Block-diagonal loaders declare their ring (D entries of ENTRY bytes) and
// the copy-out staging (EPI bytes) that follows it.
template <class L, class = void>
struct LoaderRing {
  static constexpr int ring = 0, bytes = 0;
};
template <class L>
struct LoaderRing<L, std::void_t<decltype(L::ENTRY)>> {
  static constexpr int ring = L::D * L::ENTRY, bytes = ring + L::EPI;
};

template <class Cfg, class Prob, int FIX>
struct Engine {
  typedef typename Cfg::acc_t acc_t;
  typedef typename Prob::Params Params;
  typedef typename Prob::Loader Loader;
  typedef typename Cfg::Op::frag_t Frag;
  typedef Frag FragA[Cfg::FM];
  typedef Frag FragB[Cfg::FN];

  const Params& prm;
  const KPlan& p;
  const Scratch& s;
  SKG_LDS char* lds;
  int tid, lane, wave, wm, wn;
  acc_t acc[Cfg::FM][Cfg::FN];
  // MX: this iteration's and the next one's scale words per fragment, each
  // already shifted so that byte 0 is the lane's block of k-step 0 and
  // byte 2 that of k-step 1.
  static constexpr bool kMx = LoaderMx<Loader>::value;
  // One CTA per CU: the burst schedule spreads its refills among the MFMAs
  // (grp_iter_burst).
  static constexpr bool kDefer = Cfg::MIN_CTAS == 1;
  static constexpr bool kBd = Cfg::BDG > 0;  // block-diagonal grouped wgrad tile
  uint32_t msa[Cfg::FM], msb[Cfg::FN], nsa[Cfg::FM], nsb[Cfg::FN];

  SKG_DEV Engine(const Params& prm_, const KPlan& p_, const Scratch& s_, SKG_LDS char* lds_)
      : prm(prm_), p(p_), s(s_), lds(lds_) {
    tid = threadIdx.x;
    lane = tid & 63;
    wave = tid >> 6;
    wm = wave / Cfg::WN;
    wn = wave % Cfg::WN;
  }

  SKG_DEV void zero_acc() {
#pragma unroll
    for (int f = 0; f < Cfg::FM; ++f)
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g)
#pragma unroll
        for (int i = 0; i < Cfg::NACC; ++i) acc[f][g][i] = 0.f;
  }

  // Operand fragments of k-step ks from a stage whose rows are RBX bytes (A
  // rows first, then B rows).  The rows of one wave's blocks differ by
  // multiples of 32, which leaves the swizzle unchanged, so each block is a
  // constant offset from the first.
  template <int RBX>
  SKG_DEV void load_frags(FragA& fa, FragB& fb, const SKG_LDS char* stage, int ks) const {
    load_frags_ab<RBX>(fa, fb, stage, stage + Cfg::TM * RBX, ks);
  }

  template <int RBX>
  SKG_DEV void load_frags_ab(FragA& fa, FragB& fb, const SKG_LDS char* stage,
                             const SKG_LDS char* sb, int ks) const {
    static_assert(RBX == 128 || Cfg::MN == 32, "block offsets keep the 64-byte swizzle");
    const int lrow = lane % Cfg::MN, lk = (lane / Cfg::MN) * Cfg::Op::OPB;
    // A 32-byte fp8 operand is two 16-byte chunks.  The scaled f8f6f4 MFMA
    // reads the first chunk of every lane as its first 32-element K block
    // (lanes 0-31 the first 16, lanes 32-63 the next 16) and the second
    // chunk as its second block, scaled by the upper lanes' scales (measured
    // lane layout).  Unscaled, any arrangement common to A and B works, and
    // the lane reads 32 contiguous bytes; with MX block scales the lane of
    // half h reads chunks 4ks + h and 4ks + h + 2, so the instruction's
    // blocks are the operands' blocks 2ks and 2ks + 1.
    const int chunk0 = kMx ? ((ks * Cfg::Op::KB) >> 4) + lane / Cfg::MN : (ks * Cfg::Op::KB + lk) >> 4;
    const int h1 = kMx ? 2 : Cfg::OPC - 1;  // second chunk of a 32-byte operand
    const uint32_t oa0 = lds_off<RBX>(wm * Cfg::WTM + lrow, chunk0);
    const uint32_t oa1 = lds_off<RBX>(wm * Cfg::WTM + lrow, chunk0 + h1);
    const uint32_t ob0 = lds_off<RBX>(wn * Cfg::WTN + lrow, chunk0);
    const uint32_t ob1 = lds_off<RBX>(wn * Cfg::WTN + lrow, chunk0 + h1);
#pragma unroll
    for (int f = 0; f < Cfg::FM; ++f)
      fa[f] = frag_from<Frag>(stage + oa0 + f * Cfg::MN * RBX, stage + oa1 + f * Cfg::MN * RBX);
#pragma unroll
    for (int g = 0; g < Cfg::FN; ++g)
      fb[g] = frag_from<Frag>(sb + ob0 + g * Cfg::MN * RBX, sb + ob1 + g * Cfg::MN * RBX);
  }

  SKG_DEV void mma(const FragA& fa, const FragB& fb, int ks = 0) { mma_rows(fa, fb, 0, Cfg::FM, ks); }

  // One MFMA of block (f, g); the B fragment goes first (transposed block),
  // and with MX its scale is the instruction's first scale operand.
  SKG_DEV void mfma(int f, int g, const Frag& a, const Frag& b, int ks) {
    if constexpr (kMx)
      Cfg::Op::run_scaled(acc[f][g], b, a, (msb[g] >> (16 * ks)) & 0xffu, (msa[f] >> (16 * ks)) & 0xffu);
    else
      Cfg::Op::run(acc[f][g], b, a);
  }

  SKG_DEV void mma_rows(const FragA& fa, const FragB& fb, int f0, int f1, int ks = 0) {
#pragma unroll
    for (int f = 0; f < Cfg::FM; ++f)
      if (f >= f0 && f < f1)
#pragma unroll
        for (int g = 0; g < Cfg::FN; ++g) mfma(f, g, fa[f], fb[g], ks);
  }

  // MX: the scale words of the iteration in slots sa (A) and sb (B): the
  // word of the lane's row (A) or column (B), shifted right by 8 bits in
  // the upper half of the wave, whose operand data is the second block of
  // each k-step.
  SKG_DEV void read_scales(uint32_t (&ra)[Cfg::FM], uint32_t (&rb)[Cfg::FN], const SKG_LDS char* sa,
                           const SKG_LDS char* sb) const {
    if constexpr (kMx) {
      const int r = lane % Cfg::MN, sh = 8 * (lane / Cfg::MN);
#pragma unroll
      for (int f = 0; f < Cfg::FM; ++f)
        ra[f] = *(const SKG_LDS uint32_t*)(sa + Cfg::TM * Cfg::RB + (wm * Cfg::WTM + f * Cfg::MN + r) * 4) >> sh;
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g)
        rb[g] = *(const SKG_LDS uint32_t*)(sb + Cfg::TN * Cfg::RB + (wn * Cfg::WTN + g * Cfg::MN + r) * 4) >> sh;
    }
  }

  // acc += A_tile * B_tile for the stage in LDS.  Fragments are double
  // buffered: the reads of k-step ks+1 are scheduled among the MFMAs of ks,
  // and the scheduling barriers stop the compiler from hoisting more reads
  // than that (which would not fit next to the accumulators).
  SKG_DEV void compute(const SKG_LDS char* stage) {
    FragA fa[2];
    FragB fb[2];
    load_frags<Cfg::RB>(fa[0], fb[0], stage, 0);
#pragma unroll
    for (int ks = 0; ks < Cfg::KSTEPS; ++ks) {
      if (ks + 1 < Cfg::KSTEPS) load_frags<Cfg::RB>(fa[(ks + 1) & 1], fb[(ks + 1) & 1], stage, ks + 1);
      mma(fa[ks & 1], fb[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // MAC iterations [k0, k1) of one tile into acc.
  SKG_DEV void mainloop(Loader& ld, int k0, int k1) {
    if constexpr (kBd)
      mainloop_bd(ld, k0, k1);
    else if constexpr (Loader::kGrouped)
      mainloop_grp(ld, k0, k1);
    else if constexpr (Loader::kDma)
      mainloop_dma(ld, k0, k1);
    else
      mainloop_regs(ld, k0, k1);
  }

  // Direct-to-LDS pipeline.  Sub-stage q of the segment lives in ring slot
  // q % NST; NST sub-stages are in flight ahead of the one being consumed.
  // In sub-stage q the MFMAs of its last k-step are split around the
  // synchronisation point, where the wave (1) waits for its own loads of
  // sub-stage q+1 and for its LDS reads of sub-stage q, (2) meets the other
  // waves at the barrier -- after which sub-stage q+1 is complete in LDS and
  // nobody reads slot q % NST any more -- (3) refills slot q % NST with
  // sub-stage q + NST and (4) reads the first fragments of sub-stage q+1.
  SKG_DEV SKG_LDS char* ring(int q) const { return lds + (q % Cfg::NST) * Cfg::SST; }

  SKG_DEV static void wait_loads(int younger) {
    constexpr int L = Loader::LPS;
    static_assert(Cfg::NST <= 4, "wait table");
    if (younger <= 0)
      wait_vm<0>();
    else if (younger == 1)
      wait_vm<L>();
    else if (younger == 2)
      wait_vm<2 * L>();
    else
      wait_vm<3 * L>();
  }

  // LAST: the segment's final sub-stage, which has nothing to wait for or
  // prefetch.  It is a separate instantiation so that the second half of
  // the MFMAs after the barrier is reached from one path only, and the
  // compiler's LDS wait before it covers the fragments read before the
  // barrier, not those of the next sub-stage read right after it.
  template <int CB, bool LAST>
  SKG_DEV void last_kstep(FragA (&fa)[2], FragB (&fb)[2], const Loader& ld, int q, int Q, int q0) {
    mma_rows(fa[CB], fb[CB], 0, Cfg::FM / 2);
    if constexpr (!LAST) {
      wait_loads(min(Cfg::NST - 2, Q - 2 - q));
      lds_barrier();
      if (q + Cfg::NST < Q) ld.issue(q0 + q + Cfg::NST, ring(q));
      load_frags<Cfg::RBS>(fa[CB ^ 1], fb[CB ^ 1], ring(q + 1), 0);
    }
    mma_rows(fa[CB], fb[CB], Cfg::FM / 2, Cfg::FM);
  }

  // One sub-stage: k-steps 0 .. KSS-2 with the fragments of the next k-step
  // read during the MFMAs of the current one, then the last k-step around
  // the synchronisation point.  FB is the fragment buffer of k-step 0.
  template <int FB, bool LAST>
  SKG_DEV void dma_substage(FragA (&fa)[2], FragB (&fb)[2], const Loader& ld, int q, int Q, int q0) {
#pragma unroll
    for (int ks = 0; ks + 1 < Cfg::KSS; ++ks) {
      load_frags<Cfg::RBS>(fa[(FB + ks + 1) & 1], fb[(FB + ks + 1) & 1], ring(q), ks + 1);
      mma(fa[(FB + ks) & 1], fb[(FB + ks) & 1]);
    }
    last_kstep<(FB + Cfg::KSS - 1) & 1, LAST>(fa, fb, ld, q, Q, q0);
  }

  SKG_DEV void mainloop_dma(const Loader& ld, int k0, int k1) {
    // Nothing is outstanding here; saying so lets the compiler drop the
    // waits it would otherwise place inside the loop for loads of earlier
    // segments.  The loop itself only issues loads the compiler cannot see.
    __builtin_amdgcn_s_waitcnt(0);
    zero_acc();
    const int q0 = k0 * Cfg::SUBS, Q = (k1 - k0) * Cfg::SUBS;  // Q >= 1
#pragma unroll
    for (int j = 0; j < Cfg::NST; ++j)
      if (j < Q) ld.issue(q0 + j, ring(j));
    wait_loads(min(Cfg::NST - 1, Q - 1));
    lds_barrier();
    FragA fa[2];
    FragB fb[2];
    load_frags<Cfg::RBS>(fa[0], fb[0], ring(0), 0);
    // Sub-stages 0 .. Q-2, then the last one.  With one k-step per
    // sub-stage the fragment buffers alternate, so sub-stages go in pairs.
    if constexpr (Cfg::KSS % 2 == 0) {
      for (int q = 0; q < Q - 1; ++q) dma_substage<0, false>(fa, fb, ld, q, Q, q0);
      dma_substage<0, true>(fa, fb, ld, Q - 1, Q, q0);
    } else {
      int q = 0;
      for (; q + 2 < Q; q += 2) {
        dma_substage<0, false>(fa, fb, ld, q, Q, q0);
        dma_substage<1, false>(fa, fb, ld, q + 1, Q, q0);
      }
      if (q + 2 == Q) {
        dma_substage<0, false>(fa, fb, ld, q, Q, q0);
        dma_substage<1, true>(fa, fb, ld, q + 1, Q, q0);
      } else {
        dma_substage<0, true>(fa, fb, ld, q, Q, q0);
      }
    }
    __syncthreads();  // every wave is done with the ring before LDS is reused
  }

  // Grouped pipeline.  Group j of the segment (A or B of MAC iteration
  // j/2) lives in ring slot j % NSLOT (split rings: A groups in slot
  // (j/2) % (NSLOT/2) of the A ring, B groups likewise in the B ring, so
  // group j + NSLOT again takes group j's slot).  At the end of iteration i the wave
  // waits for its own loads of iteration i+1, meets the other waves at the
  // barrier -- after which iteration i+1 is complete in LDS and nobody reads
  // iteration i's two slots any more -- refills those slots with groups
  // 2i+NSLOT and 2i+NSLOT+1 and reads the first fragments of iteration i+1,
  // all inside the last k-step's MFMAs.
  SKG_DEV SKG_LDS char* slot(int j) const {
    if constexpr (Cfg::SPLIT) {
      constexpr int D = Cfg::NSLOT / 2;
      const int k = (j >> 1) % D;
      return (j & 1) ? lds + D * Cfg::SLOT_A + k * Cfg::SLOT_B : lds + k * Cfg::SLOT_A;
    } else {
      return lds + (j % Cfg::NSLOT) * Cfg::SLOT;
    }
  }

  // Order of the MAC iterations of a wgrad segment [k0, k0+L): local step
  // i runs iteration k0 + (i + rot) % L, rot = -k0 mod L, i.e. every
  // segment starts at the iteration whose index is a multiple of its
  // length.  Stream-K segments of different tiles (other groups, other
  // filter taps) that cover the same reduction indices then tend to read
  // the same dY and X rows at the same time, which lets them share L2
  // lines.  A data-parallel tile (k0 = 0) keeps its natural order; GEMM
  // segments keep theirs.
  int gk0, gL, grot;
  SKG_DEV int iter(int i) const {
    if constexpr (!Loader::kTrans) return gk0 + i;  // GEMM: natural order
    const int x = i + grot;
    return gk0 + (x >= gL ? x - gL : x);
  }

  // Wait until at most n groups younger than the awaited one are in flight
  // (younger groups alternate A, B, A, ... starting with an A group).
  SKG_DEV static void wait_groups(int n) {
    constexpr int A = Loader::UA, B = Loader::UB;
    static_assert(Cfg::NSLOT <= 8 && 3 * A + 3 * B < 64, "wait table");
    switch (n <= 0 ? 0 : n) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<A>(); break;
      case 2: wait_vm<A + B>(); break;
      case 3: wait_vm<2 * A + B>(); break;
      case 4: wait_vm<2 * A + 2 * B>(); break;
      case 5: wait_vm<3 * A + 2 * B>(); break;
      default: wait_vm<3 * A + 3 * B>(); break;
    }
  }

  // Per-lane LDS addresses of the transposing fragment reads of one slot.
  struct TrBase {
    uint32_t a[Cfg::FM], b[Cfg::FN];
  };

  // Fragments of k-step ks of the grouped pipeline from the A tile at sa
  // and the B tile at sb: K-contiguous rows (GEMM) read directly, q-row
  // tiles (wgrad) with the transposing read.
  SKG_DEV void grp_frags(FragA& fa, FragB& fb, const SKG_LDS char* sa, const SKG_LDS char* sb,
                         int ks) const {
    if constexpr (Loader::kTrans)
      load_frags_tr(fa, fb, tr_bases(sa, sb), ks);
    else
      load_frags_ab<Cfg::RB>(fa, fb, sa, sb, ks);
  }
  // Same, with the transposing reads' bases of the slots formed already.
  SKG_DEV void grp_frags(FragA& fa, FragB& fb, const SKG_LDS char* sa, const SKG_LDS char* sb,
                         const TrBase& t, int ks) const {
    if constexpr (Loader::kTrans)
      load_frags_tr(fa, fb, t, ks);
    else
      load_frags_ab<Cfg::RB>(fa, fb, sa, sb, ks);
  }

  // Transposing fragment reads.  ds_read_b64_tr_b16 hands lane i of each
  // group of 16 lanes the element in column i of four consecutive rows,
  // taking the row from lane 4s + i/4 of the group and the column offset
  // from its address; pointing lane j of the group at row kb + j/4,
  // columns mb + 4*(j%4) .. +3 therefore gives lane i the four consecutive
  // reduction indices kb .. kb+3 of column mb + i.  Two such reads (rows
  // +0..3 and +4..7) make the eight-element MFMA operand; kb is 8 * (lane /
  // 32) for the 32x32 MFMA (16 reduction indices per k-step) and 8 * (lane
  // / 16) for the 16x16 one (32 per k-step).  tro_a / tro_b
  // hold, per lane and fragment, the byte offset of the first read of
  // k-step 0; k-steps and the second read are immediate offsets.
  uint32_t tro_a[Cfg::FM], tro_b[Cfg::FN];

  template <int P>
  SKG_DEV uint32_t tr_offset(int col0) const {
    const int grp = lane >> 4, jj = lane & 15;
    const int mb = Cfg::MN == 32 ? 16 * (grp & 1) : 0;
    const int kb = Cfg::MN == 32 ? 8 * (grp >> 1) : 8 * grp;
    const int row = kb + (jj >> 2);
    const int col = col0 + mb + 4 * (jj & 3);
    return (uint32_t)(row * P + (((col >> 3) ^ tr_swz<P, Cfg::MN>(row)) << 4) + (col & 7) * 2);
  }

  SKG_DEV void tr_init() {
    if constexpr (kBd && Loader::kTrans) {
      // Wave wm's group: its 16 output channels in the A tile, its 16 input
      // channels in every tap plane (plane g follows the A tile).
#pragma unroll
      for (int f = 0; f < Cfg::FM; ++f) tro_a[f] = tr_offset<Loader::PA>(wm * Cfg::WTM + f * Cfg::MN);
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g) tro_b[g] = g * Loader::PLANE + tr_offset<Loader::PB>(wm * Cfg::WTM);
    } else if constexpr (Loader::kTrans && !kBd) {
#pragma unroll
      for (int f = 0; f < Cfg::FM; ++f) tro_a[f] = tr_offset<Loader::PA>(wm * Cfg::WTM + f * Cfg::MN);
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g) tro_b[g] = tr_offset<Loader::PB>(wn * Cfg::WTN + g * Cfg::MN);
    }
  }

  // The k-step and the second read are constant offsets from one per-lane
  // address per fragment and slot (TrBase, formed once per slot and
  // iteration).  That address is made opaque to the compiler, which
  // otherwise hoists every (lane offset + constant) of the loop into a
  // register of its own and re-adds the slot base to each of them on every
  // iteration (two VALU instructions per read) instead of using the read's
  // immediate offset.
  SKG_DEV TrBase tr_bases(const SKG_LDS char* sa, const SKG_LDS char* sb) const {
    TrBase t;
    if constexpr (Loader::kTrans) {
#pragma unroll
      for (int f = 0; f < Cfg::FM; ++f) {
        uint32_t x = lds_addr(sa) + tro_a[f];
        asm volatile("" : "+v"(x));
        t.a[f] = x;
      }
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g) {
        uint32_t x = lds_addr(sb) + tro_b[g];
        asm volatile("" : "+v"(x));
        t.b[g] = x;
      }
    }
    return t;
  }

  template <int P>
  SKG_DEV static Frag tr_frag(uint32_t addr, int ks) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef SKG_LDS v4i16 lds_v4i16;
    constexpr int KE = Cfg::Op::KB / 2;  // reduction indices per k-step
    const SKG_LDS char* p = (const SKG_LDS char*)(uintptr_t)addr + ks * KE * P;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * P));
    const i32x2 l2 = __builtin_bit_cast(i32x2, lo), h2 = __builtin_bit_cast(i32x2, hi);
    return Frag{l2[0], l2[1], h2[0], h2[1]};
  }

  SKG_DEV void load_frags_tr(FragA& fa, FragB& fb, const TrBase& t, int ks) const {
    if constexpr (Loader::kTrans) {
#pragma unroll
      for (int f = 0; f < Cfg::FM; ++f) fa[f] = tr_frag<Loader::PA>(t.a[f], ks);
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g) fb[g] = tr_frag<Loader::PB>(t.b[g], ks);
    }
  }

  // The MFMAs of rows [F0, F1) of one k-step with DMA instructions
  // [D0, D1) of a refill spread among them in program order, so that the
  // wave issues each DMA while an MFMA runs instead of in one burst.
  template <int F0, int F1, int D0, int D1, int KS = 0, class Refill>
  SKG_DEV void mma_dma(const FragA& fa, const FragB& fb, const Loader& ld, const Refill& rf) {
    constexpr int NM = (F1 - F0) * Cfg::FN, ND = D1 - D0;
    static_for<0, NM>([&](auto m_) {
      constexpr int m = decltype(m_)::value;
      constexpr int f = F0 + m / Cfg::FN, g = m % Cfg::FN;
      mfma(f, g, fa[f], fb[g], KS);  // transposed block (k-step KS's scales under MX)
      if constexpr (ND > 0) {
        // DMA d follows MFMA (d * NM) / ND
        static_for<0, ND>([&](auto d_) {
          constexpr int d = decltype(d_)::value;
          if constexpr ((d * NM) / ND == m) ld.template refill<D0 + d>(rf);
        });
      }
    });
  }

  // One A (IS_A) or B fragment `idx` of k-step ks from a grouped GEMM slot.
  template <bool IS_A>
  SKG_DEV Frag one_frag(const SKG_LDS char* st, int idx, int ks) const {
    const int lrow = lane % Cfg::MN, lk = (lane / Cfg::MN) * Cfg::Op::OPB;
    const int chunk0 = (ks * Cfg::Op::KB + lk) >> 4;
    const int r0 = (IS_A ? wm * Cfg::WTM : wn * Cfg::WTN) + lrow;
    const uint32_t o0 = lds_off<Cfg::RB>(r0, chunk0), o1 = lds_off<Cfg::RB>(r0, chunk0 + Cfg::OPC - 1);
    return frag_from<Frag>(st + o0 + idx * Cfg::MN * Cfg::RB, st + o1 + idx * Cfg::MN * Cfg::RB);
  }

  // One MAC iteration i of the grouped pipeline with the refill spread among
  // the MFMAs (256x256 GEMM tiles).  The refill of iteration i-1's two slots
  // (groups 2i-2+NSLOT, a B group, and 2i-1+NSLOT) is spread over the
  // k-steps; not in iteration 0 (no slot is free yet) nor in the last
  // (nothing left to load).  Fragments roll: the MFMAs of a k-step run
  // row by row (one A fragment each); a row's A fragment is dead once its
  // row is issued, so the next k-step's A fragment of that row is read into
  // the same registers during the following row.  Only B is double
  // buffered: FM + 2 FN fragments are live instead of 2 (FM + FN).
  // Reads per row region (ks, f):
  //   f == 0:           A(ks, FM-1), which the previous region freed;
  //   ks < KL, f >= 1:  A(ks+1, f-1);  ks < KL, any f:  B(ks+1) spread;
  //   ks == KL:         the next iteration's k-step 0, after the barrier
  //                     that sits before row H = FM/2: A(0, 0..H-1) at row
  //                     H, A(0, f-1) at row f > H, B(0) spread over H..FM-1.
  // The refill DMAs of k-step ks are spread over its rows (over the rows
  // before the barrier in the last k-step).
  template <bool LAST, bool DMA>
  SKG_DEV void grp_iter_roll(FragA& fa, FragB (&fb)[2], const Loader& ld, int i, int G) {
    static_assert(Cfg::NSLOT % 2 == 1, "the first refilled group is a B group");
    constexpr int FM = Cfg::FM, FN = Cfg::FN, H = FM / 2, KL = Cfg::KSTEPS - 1;
    constexpr int NDMA = DMA ? Loader::UA + Loader::UB : 0;
    constexpr int PER = NDMA / Cfg::KSTEPS;  // DMA instructions per k-step
    static_assert(NDMA % Cfg::KSTEPS == 0 && PER % FM == 0 && FN % FM == 0 && FN % H == 0,
                  "rolling schedule");
    typename Loader::Refill rf;
    if constexpr (DMA) {
      const int jb = 2 * i - 2 + Cfg::NSLOT, ja = jb + 1;
      rf.slot_b = slot(jb);
      rf.slot_a = slot(ja);
      rf.it_b = iter(jb >> 1);
      rf.it_a = iter(ja >> 1);
      rf.live_b = jb < G;
      rf.live_a = ja < G;
      ld.finish_refill(rf);
    }
    const SKG_LDS char* sa = slot(2 * i);
    const SKG_LDS char* sb = slot(2 * i + 1);
    const SKG_LDS char* na = slot(2 * i + 2);
    const SKG_LDS char* nb = slot(2 * i + 3);
    static_for<0, Cfg::KSTEPS>([&](auto ks_) {
      constexpr int ks = decltype(ks_)::value, CB = ks & 1, NB = CB ^ 1;
      static_for<0, FM>([&](auto f_) {
        constexpr int f = decltype(f_)::value;
        constexpr bool last_step = ks == KL;
        constexpr int RD = !last_step ? PER / FM : (f < H ? PER / H : 0);
        constexpr int D0 = ks * PER + (!last_step ? f * (PER / FM) : (f < H ? f * (PER / H) : 0));
        if constexpr (last_step && f == H && !LAST) {
          // Groups 2i+2 and 2i+3 (iteration i+1) have landed once only the
          // A group refilled last is younger.
          wait_vm<Loader::UA>();
          lds_barrier();
        }
        mma_dma<f, f + 1, D0, D0 + RD, ks>(fa, fb[CB], ld, rf);
        if constexpr (f == 0) {
          fa[FM - 1] = one_frag<true>(sa, FM - 1, ks);
        }
        if constexpr (!last_step) {
          if constexpr (f >= 1) {
            fa[f - 1] = one_frag<true>(sa, f - 1, ks + 1);
            }
          static_for<f * (FN / FM), (f + 1) * (FN / FM)>([&](auto g_) {
            constexpr int g = decltype(g_)::value;
            fb[NB][g] = one_frag<false>(sb, g, ks + 1);
          });
        } else if constexpr (!LAST && f >= H) {
          if constexpr (f == H) {
            static_for<0, H>([&](auto r_) {
              constexpr int r = decltype(r_)::value;
              fa[r] = one_frag<true>(na, r, 0);
            });
          } else {
            fa[f - 1] = one_frag<true>(na, f - 1, 0);
            }
          static_for<(f - H) * (FN / H), (f - H + 1) * (FN / H)>([&](auto g_) {
            constexpr int g = decltype(g_)::value;
            fb[NB][g] = one_frag<false>(nb, g, 0);
          });
        }
        // Alternate the row's MFMAs with its LDS reads.
        static_for<0, FN>([&](auto) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, Cfg::OPC, 0);  // one fragment's reads
        });
        __builtin_amdgcn_sched_barrier(0);  // one row per scheduling region
      });
    });
  }

  // Burst variant (tiles without the rolling schedule).  With two CTAs per
  // CU, at the end of iteration i the two slots it used are refilled right
  // after the barrier with groups 2i+NSLOT and 2i+NSLOT+1, and the other
  // CTA's MFMAs cover the burst.  With one CTA per CU (kDefer) nothing
  // would: a wave that issues a dozen DMAs in a row stalls until the
  // address unit takes them, with no MFMA queued.  There the refill of
  // iteration i-1's slots is issued during iteration i instead, spread
  // among the MFMAs of its first KSTEPS-1 k-steps (DMA: i >= 1, not the
  // last iteration, whose pending groups all lie past the segment).  The
  // awaited groups are the same either way.  Pending groups past the
  // segment zero-fill slots nobody reads; the main loop waits for them
  // before the LDS is reused.
  template <bool LAST, bool DMA>
  SKG_DEV void grp_iter_burst(FragA (&fa)[2], FragB (&fb)[2], const Loader& ld, int i, int G) {
    constexpr int ODD = Cfg::NSLOT % 2;  // group 2i+NSLOT is a B group when NSLOT is odd
    const SKG_LDS char* sa = slot(2 * i);
    const SKG_LDS char* sb = slot(2 * i + 1);
    typename Loader::Refill rf;
    if constexpr (kDefer && DMA) {
      const int jb = 2 * (i - 1) + Cfg::NSLOT + (1 - ODD), ja = 2 * (i - 1) + Cfg::NSLOT + ODD;
      rf.slot_b = slot(jb);
      rf.slot_a = slot(ja);
      rf.it_b = iter(jb >> 1);
      rf.it_a = iter(ja >> 1);
      rf.live_b = jb < G;
      rf.live_a = ja < G;
      ld.finish_refill(rf);
    }
    const TrBase tb = tr_bases(sa, sb);
    static_for<0, Cfg::KSTEPS - 1>([&](auto ks_) {
      constexpr int ks = decltype(ks_)::value, ND = Loader::UA + Loader::UB, KS = Cfg::KSTEPS - 1;
      grp_frags(fa[(ks + 1) & 1], fb[(ks + 1) & 1], sa, sb, tb, ks + 1);
      if constexpr (kDefer && DMA)
        mma_dma<0, Cfg::FM, ks * ND / KS, (ks + 1) * ND / KS, ks>(fa[ks & 1], fb[ks & 1], ld, rf);
      else
        mma(fa[ks & 1], fb[ks & 1], ks);
      __builtin_amdgcn_sched_barrier(0);  // one k-step per scheduling region
    });
    constexpr int CB = (Cfg::KSTEPS - 1) & 1, KL = Cfg::KSTEPS - 1;
    mma_rows(fa[CB], fb[CB], 0, Cfg::FM / 2, KL);
    if constexpr (!LAST) {
      wait_groups(min(G, 2 * i + Cfg::NSLOT) - (2 * i + 4));
      lds_barrier();
      if constexpr (!kDefer) {
        const int jb = 2 * i + Cfg::NSLOT + (1 - ODD), ja = 2 * i + Cfg::NSLOT + ODD;
        if (jb < G) ld.issue(jb, iter(jb >> 1), slot(jb));
        if (ja < G) ld.issue(ja, iter(ja >> 1), slot(ja));
      }
      grp_frags(fa[CB ^ 1], fb[CB ^ 1], slot(2 * i + 2), slot(2 * i + 3), 0);
      read_scales(nsa, nsb, slot(2 * i + 2), slot(2 * i + 3));
    }
    mma_rows(fa[CB], fb[CB], Cfg::FM / 2, Cfg::FM, KL);
    if constexpr (kMx && !LAST) {
#pragma unroll
      for (int f = 0; f < Cfg::FM; ++f) msa[f] = nsa[f];
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g) msb[g] = nsb[g];
    }
  }

  SKG_DEV void mainloop_grp(const Loader& ld, int k0, int k1) {
    static_assert(Cfg::KSTEPS % 2 == 0, "k-step 0 of every iteration uses buffer 0");
    __builtin_amdgcn_s_waitcnt(0);  // see mainloop_dma
    zero_acc();
    tr_init();
    const int I = k1 - k0, G = 2 * I;  // I >= 1
    gk0 = k0;
    gL = I;
    grot = (I - k0 % I) % I;
    FragA fa[2];
    FragB fb[2];
    // The wgrad refills compute an im2col address per row, which does not
    // fit between the MFMAs next to 256 accumulators: they take the burst.
    if constexpr (Cfg::SPREAD && !Loader::kTrans) {
      // Prologue: all NSLOT slots (groups past the segment only zero-fill),
      // then k-step 0's A fragments but the last (which the first row region
      // reads) and its B fragments.
      static_for<0, Cfg::NSLOT>([&](auto j_) {
        constexpr int j = decltype(j_)::value;
        ld.issue_live(j, iter(j >> 1), slot(j), j < G);
      });
      wait_groups(Cfg::NSLOT - 2);
      lds_barrier();
      FragA ra;
      static_for<0, Cfg::FM - 1>([&](auto r_) {
        constexpr int r = decltype(r_)::value;
        ra[r] = one_frag<true>(slot(0), r, 0);
      });
      static_for<0, Cfg::FN>([&](auto g_) {
        constexpr int g = decltype(g_)::value;
        fb[0][g] = one_frag<false>(slot(1), g, 0);
      });
      if (I == 1) {
        grp_iter_roll<true, false>(ra, fb, ld, 0, G);
      } else {
        grp_iter_roll<false, false>(ra, fb, ld, 0, G);
        for (int i = 1; i + 1 < I; ++i) grp_iter_roll<false, true>(ra, fb, ld, i, G);
        grp_iter_roll<true, false>(ra, fb, ld, I - 1, G);
      }
      wait_vm<0>();  // zero-fill loads of groups past the segment
    } else {
#pragma unroll
      for (int j = 0; j < Cfg::NSLOT; ++j)
        if (j < G) ld.issue(j, iter(j >> 1), slot(j));
      wait_groups(min(Cfg::NSLOT, G) - 2);
      lds_barrier();
      grp_frags(fa[0], fb[0], slot(0), slot(1), 0);
      read_scales(msa, msb, slot(0), slot(1));
      if constexpr (kDefer) {
        if (I == 1) {
          grp_iter_burst<true, false>(fa, fb, ld, 0, G);
        } else {
          grp_iter_burst<false, false>(fa, fb, ld, 0, G);
          for (int i = 1; i + 1 < I; ++i) grp_iter_burst<false, true>(fa, fb, ld, i, G);
          grp_iter_burst<true, false>(fa, fb, ld, I - 1, G);
        }
        wait_vm<0>();  // zero-fill loads of groups past the segment
      } else {
        for (int i = 0; i + 1 < I; ++i) grp_iter_burst<false, false>(fa, fb, ld, i, G);
        grp_iter_burst<true, false>(fa, fb, ld, I - 1, G);
      }
    }
    __syncthreads();  // every wave is done with the ring before LDS is reused
  }

  // Block-diagonal pipeline: a ring of D iterations, iteration i in entry
  // i % D.  Before iteration i a wave waits for its own loads of i and
  // meets the other waves at the barrier, after which iteration i is
  // complete in LDS and nobody reads iteration i-1's entry any more; it
  // refills that entry with iteration i-1+D, reads its group's fragments
  // and runs its MFMAs.  Iterations past the segment are never issued.
  SKG_DEV SKG_LDS char* bd_entry(int i) const { return lds + (i % Loader::D) * Loader::ENTRY; }

  // Wait until at most n iterations younger than the awaited one are in
  // flight.
  SKG_DEV static void wait_iters(int n) {
    constexpr int L = Loader::UA + Loader::UB, D = Loader::D;
    static_assert(D <= 6 && 5 * L < 64, "wait table");
    switch (n <= 0 ? 0 : n < D - 1 ? n : D - 1) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<L>(); break;
      case 2: wait_vm<2 * L>(); break;
      case 3: wait_vm<3 * L>(); break;
      case 4: wait_vm<4 * L>(); break;
      default: wait_vm<5 * L>(); break;
    }
  }

  // Fragments of k-step ks of a forward / dgrad entry (ConvBdLoader): the
  // A planes hold TM pixel rows of the tile's channels at one tap each, the
  // B tile TN filter rows of the iteration's reduction.  Lane l's eight
  // reduction indices 8 * (l / 16) .. +7 of the k-step are tap 2 ks + l / 32,
  // channels 8 * ((l / 16) & 1) .. +7 of its group: 16 contiguous bytes.
  SKG_DEV void bd_conv_frags(FragA& fa, FragB& fb, const SKG_LDS char* e, int ks) const {
    const int lrow = lane % 16, half = (lane / 16) & 1;
    const SKG_LDS char* pa = e + (2 * ks + lane / 32) * Loader::PLANE;
#pragma unroll
    for (int f = 0; f < Cfg::FM; ++f)
      fa[f] = *(const SKG_LDS Frag*)(pa + lds_off<Loader::PA>(f * Cfg::MN + lrow, 2 * wn + half));
    const SKG_LDS char* pb = e + Loader::B_OFF;
#pragma unroll
    for (int g = 0; g < Cfg::FN; ++g)
      fb[g] = *(const SKG_LDS Frag*)(pb + lds_off<Loader::RBB>(wn * Cfg::WTN + g * Cfg::MN + lrow,
                                                                4 * ks + lane / 16));
  }

  SKG_DEV void mainloop_bd(const Loader& ld, int k0, int k1) {
    constexpr int D = Loader::D;
    __builtin_amdgcn_s_waitcnt(0);  // see mainloop_dma
    zero_acc();
    tr_init();
    const int I = k1 - k0;  // >= 1
    gk0 = k0;
    gL = I;
    grot = (I - k0 % I) % I;
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (j < I) ld.issue_iter(iter(j), bd_entry(j));
    for (int i = 0; i < I; ++i) {
      // Issued so far: iterations up to D-1 (i <= 1) or i-2+D.
      wait_iters(i == 0 ? min(I - 1, D - 1) : min(I - 1 - i, D - 2));
      lds_barrier();
      if (i >= 1 && i - 1 + D < I) ld.issue_iter(iter(i - 1 + D), bd_entry(i - 1));
      const SKG_LDS char* e = bd_entry(i);
      FragA fa;
      FragB fb;
      if constexpr (Loader::kTrans) {
        static_assert(Cfg::KSTEPS == 1, "one k-step per wgrad iteration");
        load_frags_tr(fa, fb, tr_bases(e, e + Loader::PLANE), 0);
        mma(fa, fb, 0);
      } else {
#pragma unroll
        for (int ks = 0; ks < Cfg::KSTEPS; ++ks) {
          bd_conv_frags(fa, fb, e, ks);
          mma(fa, fb, 0);
        }
      }
    }
    wait_vm<0>();
    __syncthreads();  // every wave is done with the ring before LDS is reused
  }

  SKG_DEV void mainloop_regs(Loader& ld, int k0, int k1) {
    zero_acc();
    Prob::load(prm, ld, k0);
    ld.store(lds, tid);
    __syncthreads();
    for (int it = k0; it < k1; ++it) {
      const int cur = (it - k0) & 1;
      const bool more = it + 1 < k1;
      if (more) Prob::load(prm, ld, it + 1);
      compute(lds + cur * Cfg::STAGE);
      if (more) ld.store(lds + (cur ^ 1) * Cfg::STAGE, tid);
      __syncthreads();
    }
  }

  // --- epilogue -------------------------------------------------------------
  // Row (in the tile) of this lane's elements of row-block f, and the first
  // of the four consecutive columns of element group q of column-block g.
  SKG_DEV int row_of(int f) const { return wm * Cfg::WTM + f * Cfg::MN + acc_row<Cfg::MN>(lane); }
  SKG_DEV int col_of(int g, int q) const {
    return wn * Cfg::WTN + g * Cfg::MN + acc_col<Cfg::MN>(4 * q, lane);
  }

  enum { OUT_STORE = 0, OUT_ATOMIC = 1, OUT_WORKSPACE = 2, OUT_PUBLISH = 3, OUT_SCATTER = 4 };

  // How a finished segment leaves the CTA: first add the partials of
  // `nfold` other stream-K CTAs, in a fixed order (partner k is cta + 1 + k
  // for linear, cta + 2^k for tree), then `how`.
  struct Fix {
    int how, nfold, cta;
    bool tree;
    SKG_DEV int partner(int k) const { return tree ? cta + (1 << k) : cta + 1 + k; }
  };

  // Partial tile of stream-K CTA c: TM x TN fp32 in register order.  Wave
  // w's accumulators fill bytes [w * WBYTES, (w + 1) * WBYTES); float4 j of
  // lane l (the order of acc[f][g][4q .. 4q+3], j = (f * FN + g) * NACC/4 + q)
  // lies at (j * 64 + l) * 16.  Producer and consumer of a (CTA, wave) flag
  // hold the same fragments, so a wave folds its partner's wave straight into
  // its registers, and every wave-instruction moves 1 KiB contiguous.
  static constexpr int PSLOTS = Cfg::FM * Cfg::FN * Cfg::NACC / 4;  // float4 per lane
  static constexpr uint32_t WBYTES = PSLOTS * 64 * 16;
  static_assert(WBYTES * Cfg::NW == Cfg::TM * Cfg::TN * 4, "register-order partial");
  SKG_DEV float* partial(int c) const { return s.partials + (size_t)c * Cfg::TM * Cfg::TN; }
  SKG_DEV __amdgpu_buffer_rsrc_t partial_rsrc(int c) const {
    return make_rsrc(partial(c), Cfg::TM * Cfg::TN * 4);
  }
  // Byte offset of this lane's float4 0 in its wave's block; float4 j adds
  // the wave-uniform j * 1024.
  SKG_DEV uint32_t part_base() const { return wave * WBYTES + (uint32_t)lane * 16; }

  // OUT_PUBLISH: this wave's accumulators go out as the CTA's partial, then
  // the wave's flag is set once its stores have completed.
  SKG_DEV void publish_regs(int cta) const {
    const __amdgpu_buffer_rsrc_t q = partial_rsrc(cta);
    const uint32_t base = part_base();
    static_for<0, PSLOTS>([&](auto j_) {
      constexpr int j = decltype(j_)::value;
      constexpr int f = j / (Cfg::FN * (Cfg::NACC / 4)), g = (j / (Cfg::NACC / 4)) % Cfg::FN;
      constexpr int e = 4 * (j % (Cfg::NACC / 4));
      store_dev16_s(q, base, j * 1024, f32x4{acc[f][g][e], acc[f][g][e + 1], acc[f][g][e + 2], acc[f][g][e + 3]});
    });
    if (p.fault == FAULT_NO_PUBLISH) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      return;
    }
    flag_publish(s.flags + cta * Cfg::NW + wave);
  }

  // Adds the fold partners' partials into the accumulators, partner by
  // partner in the order Fix::partner gives.  Each wave waits only for the
  // flag of its own wave in the partner CTA.  The loads of a batch are all
  // issued before its first add, so one memory round trip covers FB float4
  // per lane.  A wait that gives up (flag_wait) is counted for the host
  // (skg_fixup_timeouts); the fold then adds whatever the partial buffer
  // holds, so the tile's values are unspecified.  Marking the tile here
  // (NaN) costs the folds of every launch: any extra work on the loaded
  // partials or on the accumulators changes how the compiler schedules the
  // batched loads or allocates the accumulators; each variant tried slowed
  // the hand-off kernels by 15-20 %.
  SKG_DEV void fold_regs(const Fix& fx) {
    // float4 loads in flight per batch: 128 VGPRs with one wave per SIMD,
    // 32 with two (half the register file each).
    constexpr int FBMAX = Cfg::NW > 4 ? 8 : 32;
    constexpr int FB = PSLOTS < FBMAX ? PSLOTS : FBMAX;
    static_assert(PSLOTS % FB == 0, "fold batches");
    // One round trip reads the flags of the first MAXQ partners (usually
    // all set by now); a partner seen unset is waited for in turn below.
    constexpr int MAXQ = 8;
    uint32_t fl[MAXQ];
    static_for<0, MAXQ>([&](auto k_) {
      constexpr int k = decltype(k_)::value;
      const int c = fx.partner(k < fx.nfold ? k : fx.nfold - 1);
      fl[k] = __hip_atomic_load(s.flags + c * Cfg::NW + wave, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    });
    uint32_t ready = 0;
    static_for<0, MAXQ>([&](auto k_) {
      constexpr int k = decltype(k_)::value;
      if (fl[k] == 1u) ready |= 1u << k;
    });
    for (int k = 0; k < fx.nfold; ++k) {
      const int c = fx.partner(k);
      if (k >= MAXQ || !((ready >> k) & 1u)) flag_wait(s.flags + c * Cfg::NW + wave, p.spin_limit);
      asm volatile("" ::: "memory");  // partial loads stay after the flag check
      const __amdgpu_buffer_rsrc_t q = partial_rsrc(c);
      const uint32_t base = part_base();
      static_for<0, PSLOTS / FB>([&](auto b_) {
        constexpr int b = decltype(b_)::value;
        f32x4 t[FB];
        static_for<0, FB>([&](auto i_) {
          constexpr int i = decltype(i_)::value;
          t[i] = load_dev16_s(q, base, (b * FB + i) * 1024);
        });
        static_for<0, FB>([&](auto i_) {
          constexpr int i = decltype(i_)::value, j = b * FB + i;
          constexpr int f = j / (Cfg::FN * (Cfg::NACC / 4)), g = (j / (Cfg::NACC / 4)) % Cfg::FN;
          constexpr int e = 4 * (j % (Cfg::NACC / 4));
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[f][g][e + u] = add_in_agpr(acc[f][g][e + u], t[i][u]);
        });
      });
    }
  }

  // OUT_SCATTER (whole-slice partitions): the tile's contributors are the S
  // consecutive stream-K CTAs c0 .. c0+S-1, each with one slice.  All of
  // them have published their partials (this one included); contributor
  // k = cta - c0 sums float4 units [k*U/S, (k+1)*U/S) of the register-order
  // partial over the S partials, contributor by contributor from c0, and
  // writes them out as the copy-out would: C = cvt((v * sa[row]) * sb[col]).
  // A unit is 4 consecutive columns of one row.
  SKG_DEV void scatter_out(const OutTile& o, int tile, int cta) const {
    constexpr int U = Cfg::TM * Cfg::TN / 4;
    const int S = p.sk_slices;
    const int c0 = (tile - p.dp_tiles) * S, k = cta - c0;
    flags_wait_all(s.flags + c0 * Cfg::NW, S * Cfg::NW, p.spin_limit);
    const int u0 = (int)((int64_t)k * U / S), u1 = (int)((int64_t)(k + 1) * U / S);
    // Batches of SB partials, the smallest of 8 / 16 / 32 that holds all S
    // (32 only with one CTA per CU: the accumulators are dead here, the
    // batch takes 4 * SB registers).
    if (S <= 8)
      scatter_units<8>(o, c0, S, u0, u1);
    else if (S <= 16 || Cfg::MIN_CTAS > 1)
      scatter_units<16>(o, c0, S, u0, u1);
    else
      scatter_units<32>(o, c0, S, u0, u1);
  }

  // Units [u0, u1) of the tile from the S partials of CTAs c0 .. c0+S-1.
  // Loads go out in batches of SB partials so that one memory round trip
  // covers a batch.
  template <int SB>
  SKG_DEV void scatter_units(const OutTile& o, int c0, int S, int u0, int u1) const {
    const int dt = Prob::dtype_c(prm);
    const bool full = o.rows >= Cfg::TM && o.cols >= Cfg::TN;
    // The tile's S partials are contiguous: one resource, the contributor's
    // partial c at byte c * PB.
    constexpr uint32_t PB = Cfg::TM * Cfg::TN * 4;
    const __amdgpu_buffer_rsrc_t r = make_rsrc_uniform(partial(c0), (uint32_t)S * PB);
    for (int u = u0 + tid; u < u1; u += Cfg::THREADS) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      for (int cb = 0; cb < S; cb += SB) {
        // Past the last contributor the batch reloads it (in bounds) and
        // adds nothing: no load is predicated.
        f32x4 t[SB];
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const int c = cb + i < S ? cb + i : S - 1;
          t[i] = load_dev16_s(r, (uint32_t)u * 16 + (uint32_t)c * PB, 0);
        }
#pragma unroll
        for (int i = 0; i < SB; ++i)
          if (cb + i < S) v = cb + i == 0 ? t[i] : v + t[i];
      }
      // Unit u: lane l of wave w, float4 j = (f * FN + g) * NACC/4 + q.
      const int w = u / (PSLOTS * 64), j = (u / 64) % PSLOTS, l = u % 64;
      const int f = j / (Cfg::FN * (Cfg::NACC / 4)), g = (j / (Cfg::NACC / 4)) % Cfg::FN;
      const int q = j % (Cfg::NACC / 4);
      const int row = (w / Cfg::WN) * Cfg::WTM + f * Cfg::MN + acc_row<Cfg::MN>(l);
      const int col = (w % Cfg::WN) * Cfg::WTN + g * Cfg::MN + acc_col<Cfg::MN>(4 * q, l);
      if (row >= o.rows) continue;
      const float sa = o.sa ? o.sa[row * Prob::kScaleInc] : 1.f;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sb = o.sb && col + e < o.cols ? o.sb[(col + e) * Prob::kScaleInc] : 1.f;
        x[e] = (v[e] * sa) * sb;
      }
      const size_t idx = out_row<Prob>(o, row) + col;
      if (full && dt == DT_F32 && ((uintptr_t)(o.base + idx * 4) & 15) == 0) {
        *(f32x4*)(o.base + idx * 4) = f32x4{x[0], x[1], x[2], x[3]};
        continue;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (col + e >= o.cols) break;
        if (dt == DT_F32)
          ((float*)o.base)[idx + e] = x[e];
        else if (dt == DT_F16)
          ((uint16_t*)o.base)[idx + e] = to_f16_bits(x[e]);
        else
          ((uint16_t*)o.base)[idx + e] = to_bf16_bits(x[e]);
      }
    }
  }

  // Writes the accumulator tile out, one wave-row (WTM rows) at a time: the
  // owning waves stage it in LDS as fp32, then every thread takes a fixed
  // 8-column chunk of the staged rows and
  //   OUT_STORE:     C = cvt((v * sa[row]) * sb[col]), round to nearest even;
  //   OUT_ATOMIC:    fp32 atomic add of (v * sa[row]) * sb[col] into C;
  //   OUT_WORKSPACE: fp32 atomic add of v into the tile's scratch wsp;
  // (Full tiles take the two atomic forms through atomic_full, one column
  // per lane.)  Partials never pass through here: publish_regs and fold_regs
  // move them between registers and memory before the copy-out.
  static constexpr int VC = 8;                      // columns per thread chunk
  static constexpr int CPRO = Cfg::TN / VC;         // chunks per row
  static constexpr int RSTEP = Cfg::THREADS / CPRO; // rows between a thread's rows
  static constexpr int NR = (Cfg::WTM + RSTEP - 1) / RSTEP;  // rows per thread per pass

  struct Row {   // one thread's 8 columns of one row, fp32
    f32x4 v0, v1;
  };

  SKG_DEV Row staged(int lr, int col) const {
    const SKG_LDS char* p = lds + lr * Cfg::EPI_PITCH32 + col * 4;
    return Row{*(const SKG_LDS f32x4*)p, *(const SKG_LDS f32x4*)(p + 16)};
  }

  // SCALED: apply the row / column scales; without scales the products
  // would be v * 1 * 1, skipped (bit-identical).
  template <int HOW, int DTC, bool SCALED>
  SKG_DEV void emit_full(const Row& r, const OutTile& o, const Fix& fx, float* wsp, int row, int col,
                         int tofs, float sa, const f32x4& sb0, const f32x4& sb1) const {
    {
      static_assert(HOW == OUT_STORE, "atomic fix-ups copy out through atomic_full");
      const f32x4 w0 = SCALED ? (r.v0 * sa) * sb0 : r.v0, w1 = SCALED ? (r.v1 * sa) * sb1 : r.v1;
      const size_t idx = (size_t)row * o.ld + col;
      if constexpr (DTC == DT_F32) {
        // C is written once and not read back here: non-temporal stores.
        f32x4* dst = (f32x4*)((float*)o.base + idx);
        __builtin_nontemporal_store(w0, dst);
        __builtin_nontemporal_store(w1, dst + 1);
      } else {
        i32x4 h;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if constexpr (DTC == DT_F16) {
            h[e] = (int)pack_f16x2(w0[2 * e], w0[2 * e + 1]);
            h[e + 2] = (int)pack_f16x2(w1[2 * e], w1[2 * e + 1]);
          } else {
            h[e] = (int)pack_bf16x2(w0[2 * e], w0[2 * e + 1]);
            h[e + 2] = (int)pack_bf16x2(w1[2 * e], w1[2 * e + 1]);
          }
        }
        __builtin_nontemporal_store(h, (i32x4*)((uint16_t*)o.base + idx));
      }
    }
  }

  // Row scales of this thread's rows in one pass of a full tile (1 without
  // scales), loaded before the pass stages its accumulators so that the
  // loads are in flight during the staging and its barrier.
  SKG_DEV void row_scales(const OutTile& o, int pass, float (&sav)[NR]) const {
    const int lr0 = tid / CPRO;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int lr = lr0 + i * RSTEP;
      const int row = pass * Cfg::WTM + (lr < Cfg::WTM ? lr : 0);
      sav[i] = o.sa ? o.sa[row * Prob::kScaleInc] : 1.f;
    }
  }

  // Copy-out of one pass of a full tile: no bounds checks.
  template <int HOW, int DTC, bool SCALED>
  SKG_DEV void copy_full(const OutTile& o, const Fix& fx, float* wsp, int pass, int col,
                         const f32x4& sb0, const f32x4& sb1, const float (&sav)[NR]) const {
    const int lr0 = tid / CPRO;
    if (RSTEP > Cfg::WTM && lr0 >= Cfg::WTM) return;  // fewer rows than threads
#pragma unroll 4
    for (int i = 0; i < NR; ++i) {
      const int lr = lr0 + i * RSTEP, row = pass * Cfg::WTM + lr;
      Row r = staged(lr, col);
      emit_full<HOW, DTC, SCALED>(r, o, fx, wsp, row, col, row * Cfg::TN + col, sav[i], sb0, sb1);
    }
  }
  template <int DTC>
  SKG_DEV void copy_full_store(const OutTile& o, const Fix& fx, float* wsp, int pass, int col,
                               const f32x4& sb0, const f32x4& sb1, const float (&sav)[NR]) const {
    if (o.sa || o.sb)
      copy_full<OUT_STORE, DTC, true>(o, fx, wsp, pass, col, sb0, sb1, sav);
    else
      copy_full<OUT_STORE, DTC, false>(o, fx, wsp, pass, col, sb0, sb1, sav);
  }

  // Atomic copy-out of one pass of a full tile (atomic and workspace
  // fix-ups, partners already folded): consecutive lanes take consecutive
  // columns, so each wave-instruction adds into one contiguous 256-byte run
  // of the row instead of 4-byte pieces 32 bytes apart.
  template <int HOW>
  SKG_DEV void atomic_full(const OutTile& o, float* wsp, int pass) const {
    static_assert(Cfg::THREADS % Cfg::TN == 0 || Cfg::TN % Cfg::THREADS == 0, "atomic mapping");
    constexpr int TPR = Cfg::TN < Cfg::THREADS ? Cfg::TN : Cfg::THREADS;  // threads per row
    constexpr int RPS = Cfg::THREADS / TPR;                                 // rows per step
    const int c0 = tid % TPR, lr0 = tid / TPR;
#pragma unroll
    for (int cc = 0; cc < Cfg::TN; cc += TPR) {
      const int c = c0 + cc;
      const float sb = HOW == OUT_ATOMIC && o.sb ? o.sb[c * Prob::kScaleInc] : 1.f;
#pragma unroll 1
      for (int lr = lr0; lr < Cfg::WTM; lr += RPS) {
        const int row = pass * Cfg::WTM + lr;
        const float v = *(const SKG_LDS float*)(lds + lr * Cfg::EPI_PITCH32 + c * 4);
        if constexpr (HOW == OUT_WORKSPACE) {
          unsafeAtomicAdd(wsp + row * Cfg::TN + c, v);
        } else {
          const float sa = o.sa ? o.sa[row * Prob::kScaleInc] : 1.f;
          unsafeAtomicAdd((float*)o.base + (size_t)row * o.ld + c, (v * sa) * sb);
        }
      }
    }
  }

  // Copy-out of one pass of a ragged tile (rows or columns cut by the
  // problem edge): element-wise bounds checks.
  SKG_DEV void copy_ragged(const OutTile& o, const Fix& fx, float* wsp, int pass, int col,
                           const f32x4& sb0, const f32x4& sb1) const {
    const int dt = Prob::dtype_c(prm);
    const int ncol = o.cols - col < VC ? o.cols - col : VC;
    if (ncol <= 0) return;
    for (int lr = tid / CPRO; lr < Cfg::WTM; lr += RSTEP) {
      const int row = pass * Cfg::WTM + lr;
      if (row >= o.rows) break;
      Row r = staged(lr, col);
      const int tofs = row * Cfg::TN + col;
      float v[VC];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = r.v0[e];
        v[4 + e] = r.v1[e];
      }
      if (FIX == FIX_ATOMIC && fx.how == OUT_WORKSPACE) {
        for (int e = 0; e < ncol; ++e) unsafeAtomicAdd(wsp + tofs + e, v[e]);
        continue;
      }
      const float sa = o.sa ? o.sa[row * Prob::kScaleInc] : 1.f;
      const size_t idx = (size_t)row * o.ld + col;
      for (int e = 0; e < ncol; ++e) {
        const float w = (v[e] * sa) * (e < 4 ? sb0[e] : sb1[e - 4]);
        if (FIX == FIX_ATOMIC && fx.how == OUT_ATOMIC)
          unsafeAtomicAdd((float*)o.base + idx + e, w);
        else if (dt == DT_F32)
          ((float*)o.base)[idx + e] = w;
        else if (dt == DT_F16)
          ((uint16_t*)o.base)[idx + e] = to_f16_bits(w);
        else
          ((uint16_t*)o.base)[idx + e] = to_bf16_bits(w);
      }
    }
  }

  // Copy-out straight from the accumulators (block-diagonal tiles, whose
  // 144-column rows do not fit the staged copy-out's thread mapping): lane
  // l of a fragment holds four consecutive columns of one row.
  SKG_DEV void write_direct(const OutTile& o, const Fix& fx, float* wsp) const {
    const int dt = Prob::dtype_c(prm);
#pragma unroll
    for (int f = 0; f < Cfg::FM; ++f) {
      const int row = row_of(f);
      if (row >= o.rows) continue;
      const float sa = o.sa ? o.sa[row * Prob::kScaleInc] : 1.f;
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g)
#pragma unroll
        for (int q = 0; q < Cfg::NACC / 4; ++q) {
          const int col = col_of(g, q);
          const f32x4 v = {acc[f][g][4 * q], acc[f][g][4 * q + 1], acc[f][g][4 * q + 2],
                           acc[f][g][4 * q + 3]};
          if (FIX == FIX_ATOMIC && fx.how == OUT_WORKSPACE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) unsafeAtomicAdd(wsp + row * Cfg::TN + col + e, v[e]);
            continue;
          }
          const size_t idx = out_row<Prob>(o, row) + col;
          if (fx.how == OUT_STORE && !o.sa && !o.sb && col + 4 <= o.cols) {
            if (dt == DT_F32 && ((uintptr_t)(o.base + idx * 4) & 15) == 0) {
              __builtin_nontemporal_store(v, (f32x4*)((float*)o.base + idx));
              continue;
            }
            if (dt != DT_F32 && ((uintptr_t)(o.base + idx * 2) & 7) == 0) {
              const i32x2 h = dt == DT_F16 ? i32x2{(int)pack_f16x2(v[0], v[1]), (int)pack_f16x2(v[2], v[3])}
                                           : i32x2{(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
              __builtin_nontemporal_store(h, (i32x2*)((uint16_t*)o.base + idx));
              continue;
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e >= o.cols) break;
            const float w = (v[e] * sa) * (o.sb ? o.sb[(col + e) * Prob::kScaleInc] : 1.f);
            if (FIX == FIX_ATOMIC && fx.how == OUT_ATOMIC)
              unsafeAtomicAdd((float*)o.base + idx + e, w);
            else if (dt == DT_F32)
              ((float*)o.base)[idx + e] = w;
            else if (dt == DT_F16)
              ((uint16_t*)o.base)[idx + e] = to_f16_bits(w);
            else
              ((uint16_t*)o.base)[idx + e] = to_bf16_bits(w);
          }
        }
    }
  }

  // Copy-out of a block-diagonal forward / dgrad tile with 16-bit outputs
  // through the staging area beside the ring (which keeps streaming the
  // next tile meanwhile): two passes of 64 rows; each wave leaves its 16
  // channels of every row there (one packed 8-byte write per fragment, 16-byte
  // chunks XOR-swizzled by row), then 8 lanes store each 128-byte row whole.
  // Stored straight from the registers, a row arrives as four 32-byte pieces
  // from four waves.
  SKG_DEV void write_bd_staged(const OutTile& o, int dt) {
    static_assert(Cfg::WM == 1 && Cfg::FN == 1 && Cfg::TN * 2 == 128 && Cfg::TM % 64 == 0, "staging map");
    constexpr int PR = 64, FPP = PR / Cfg::MN, NCH = PR * 8 / Cfg::THREADS;
    SKG_LDS char* st = lds + LoaderRing<Loader>::ring;
#pragma unroll
    for (int pass = 0; pass < Cfg::TM / PR; ++pass) {
#pragma unroll
      for (int ff = 0; ff < FPP; ++ff) {
        const f32x4 v = acc[pass * FPP + ff][0];
        const int r = ff * Cfg::MN + (lane & 15);
        const int byte = wn * 32 + 8 * (lane >> 4);  // 4 channels of the wave's 16
        const i32x2 h = dt == DT_F16 ? i32x2{(int)pack_f16x2(v[0], v[1]), (int)pack_f16x2(v[2], v[3])}
                                     : i32x2{(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
        *(SKG_LDS i32x2*)(st + r * 128 + ((((byte >> 4) ^ (r & 7))) << 4) + (byte & 15)) = h;
      }
      lds_barrier();
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int id = tid + k * Cfg::THREADS, r = id >> 3, c = id & 7;
        const int row = pass * PR + r;
        if (row < o.rows && c * 8 < o.cols) {
          const i32x4 d = *(const SKG_LDS i32x4*)(st + r * 128 + ((c ^ (r & 7)) << 4));
          __builtin_nontemporal_store(d, (i32x4*)((uint16_t*)o.base + out_row<Prob>(o, row) + c * 8));
        }
      }
      lds_barrier();  // the staging area is free for the next pass
    }
  }

  SKG_DEV void write_out(const OutTile& o, const Fix& fx, float* wsp) {
    if constexpr (kStream) {
      const int dt = Prob::dtype_c(prm);
      if (fx.how == OUT_STORE && dt != DT_F32 && !o.sa && !o.sb)
        write_bd_staged(o, dt);
      else
        write_direct(o, fx, wsp);
    } else if constexpr (kBd) {
      write_direct(o, fx, wsp);
    } else {
      write_staged(o, fx, wsp);
    }
  }

  SKG_DEV void write_staged(const OutTile& o, const Fix& fx, float* wsp) {
    static_assert(Cfg::TN % VC == 0 && Cfg::THREADS % CPRO == 0 && 64 % CPRO == 0 &&
                      (Cfg::WTM % RSTEP == 0 || RSTEP % Cfg::WTM == 0),
                  "copy-out mapping");
    const int col = (tid % CPRO) * VC;
    const bool full = o.rows >= Cfg::TM && o.cols >= Cfg::TN;  // CTA-uniform
    const bool scaled = fx.how == OUT_STORE || fx.how == OUT_ATOMIC;
    f32x4 sb0 = {1.f, 1.f, 1.f, 1.f}, sb1 = sb0;
    if (Prob::kScaleInc == 0 && scaled && o.sb) {
      const float t = o.sb[0];
      sb0 = f32x4{t, t, t, t};
      sb1 = sb0;
    } else if (scaled && o.sb) {
      if (col + VC <= o.cols) {
        sb0 = *(const f32x4*)(o.sb + col);
        sb1 = *(const f32x4*)(o.sb + col + 4);
      } else {
        for (int e = 0; e < 4; ++e) {
          if (col + e < o.cols) sb0[e] = o.sb[col + e];
          if (col + 4 + e < o.cols) sb1[e] = o.sb[col + 4 + e];
        }
      }
    }
    const int dt = Prob::dtype_c(prm);
#pragma unroll
    for (int pass = 0; pass < Cfg::WM; ++pass) {
      float sav[NR];
      if (full && fx.how == OUT_STORE) row_scales(o, pass, sav);
      if (wm == pass) {
        // One per-lane base address; every (f, g, q) is a constant offset
        // from it (the column step of element group q is 8 or 4).
        SKG_LDS char* st = lds + acc_row<Cfg::MN>(lane) * Cfg::EPI_PITCH32 +
                           (wn * Cfg::WTN + acc_col<Cfg::MN>(0, lane)) * 4;
        constexpr int QSTEP = Cfg::MN == 32 ? 8 : 4;
#pragma unroll
        for (int f = 0; f < Cfg::FM; ++f) {
#pragma unroll
          for (int g = 0; g < Cfg::FN; ++g)
#pragma unroll
            for (int q = 0; q < Cfg::NACC / 4; ++q) {
              const f32x4 v = {acc[f][g][4 * q], acc[f][g][4 * q + 1], acc[f][g][4 * q + 2],
                               acc[f][g][4 * q + 3]};
              *(SKG_LDS f32x4*)(st + f * Cfg::MN * Cfg::EPI_PITCH32 + (g * Cfg::MN + q * QSTEP) * 4) = v;
              if ((q & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
      __syncthreads();
      if (!full) {
        copy_ragged(o, fx, wsp, pass, col, sb0, sb1);
      } else if (FIX == FIX_ATOMIC && fx.how == OUT_WORKSPACE) {
        atomic_full<OUT_WORKSPACE>(o, wsp, pass);
      } else if (FIX == FIX_ATOMIC && fx.how == OUT_ATOMIC) {
        atomic_full<OUT_ATOMIC>(o, wsp, pass);
      } else if (dt == DT_F32) {
        copy_full_store<DT_F32>(o, fx, wsp, pass, col, sb0, sb1, sav);
      } else if (dt == DT_F16) {
        copy_full_store<DT_F16>(o, fx, wsp, pass, col, sb0, sb1, sav);
      } else {
        copy_full_store<DT_BF16>(o, fx, wsp, pass, col, sb0, sb1, sav);
      }
      __syncthreads();
    }
  }

  SKG_DEV int cta_of(int it) const {
    const int boundary = p.extra * (p.ipc + 1);
    return it < boundary ? it / (p.ipc + 1) : p.extra + (it - boundary) / p.ipc;
  }

  // Runs MAC iterations [k0, k1) of `tile` and hands the result on.  `cta`
  // is the stream-K CTA index, or -1 for a data-parallel tile.
  SKG_DEV void process(int tile, int k0, int k1, int cta) {
    Loader ld;
    OutTile o;
    Prob::setup(prm, p, tile, ld, o, tid);
    mainloop(ld, k0, k1);
    const Fix fx = fixup(tile, k0, k1, cta);
    if constexpr (FIX == FIX_HANDOFF) {
      if (fx.nfold > 0) fold_regs(fx);
      if (fx.how == OUT_PUBLISH) {
        publish_regs(fx.cta);
        return;
      }
      if (fx.how == OUT_SCATTER) {
        publish_regs(fx.cta);
        scatter_out(o, tile, fx.cta);
        return;
      }
    }
    write_out(o, fx, fx.how == OUT_WORKSPACE ? s.ws + (size_t)(tile - p.dp_tiles) * Cfg::TM * Cfg::TN
                                             : nullptr);
  }

  // Stream-K hand-off of a finished segment (CTA-uniform, so all waves
  // agree).  linear: a CTA that did not start the tile publishes; the owner
  // folds every later contributor in CTA order.  tree: at position pos among
  // the tile's n contributors, round st (1, 2, 4, ...) folds pos + st when
  // bit st of pos is clear, or publishes and stops when it is set.
  SKG_DEV Fix fixup(int tile, int k0, int k1, int cta) const {
    Fix fx = {OUT_STORE, 0, cta, false};
    if (cta < 0) return fx;  // data-parallel tile: sole writer
    const bool started = k0 == 0, ended = k1 == p.ipt;
    if constexpr (FIX == FIX_ATOMIC) {
      // workspace: every stream-K segment adds into the tile's scratch (the
      // second stage writes C); atomic: a whole tile is stored directly.
      if (p.reduction == RED_WORKSPACE)
        fx.how = OUT_WORKSPACE;
      else if (!(started && ended))
        fx.how = OUT_ATOMIC;
      return fx;
    }
    if (started && ended) return fx;  // a whole tile inside one range
    if (p.reduction == RED_SCATTER) {
      fx.how = OUT_SCATTER;
      return fx;
    }
    const int sk_tile = tile - p.dp_tiles;
    const int first = cta_of(sk_tile * p.ipt);
    const int last = cta_of(sk_tile * p.ipt + p.ipt - 1);
    if (p.reduction == RED_LINEAR) {
      if (!started)
        fx.how = OUT_PUBLISH;
      else
        fx.nfold = last - cta;
      return fx;
    }
    fx.tree = true;
    const int n = last - first + 1, pos = cta - first;
    for (int st = 1; st < n; st <<= 1) {
      if (pos & st) {
        fx.how = OUT_PUBLISH;
        return fx;
      }
      if (pos + st < n) ++fx.nfold;
    }
    return fx;
  }

  // Data-parallel slot s (the s-th DP tile in launch order) -> tile id.
  // Blocks go to the 8 XCDs round robin, so consecutive slots land on
  // different L2 caches.  Slots are first transposed so that each XCD takes
  // one contiguous run of them, and the run is laid over the tile grid in
  // groups of GM tile rows, column by column, so that the tiles running
  // together on one XCD form a compact block sharing A and B panels.  A
  // bijection on [0, dp_tiles); the DP tiles are whole rows of the tile
  // grid plus a partial last row, which keeps its order.
  SKG_DEV int dp_order(int s) const {
    constexpr int XCDS = 8, GM = kDpGroupRows;
    const int n8 = p.dp_tiles & ~(XCDS - 1);
    const int u = s < n8 ? (s % XCDS) * (n8 / XCDS) + s / XCDS : s;
    const int rows = p.dp_rows;
    if (u >= rows * p.tiles_n) return u;
    const int g = (int)fdiv((uint32_t)u, p.div_groups);
    const int within = u - g * GM * p.tiles_n;
    const int rg = min(GM, rows - g * GM);  // 1 .. 4
    // within / rg without a division: a shift for 1, 2, 4; for 3 the
    // multiply-high by ceil(2^33 / 3), exact for every 32-bit value
    const int q = rg == 3 ? (int)(__umulhi((uint32_t)within, 0xAAAAAAABu) >> 1) : within >> (rg >> 1);
    return (g * GM + (within - q * rg)) * p.tiles_n + q;
  }

  // One bounded work loop: the stream-K range (if any) segment by segment,
  // then this block's data-parallel tiles.
  SKG_DEV void run() {
    const int blk = blockIdx.x;
    const bool sk_block = p.mode != MODE_DP && blk < p.sk_ctas;
    // Stream-K CTA index.  XCD order: blocks are dealt to the 8 XCDs round
    // robin (block blk to XCD blk % 8), so give XCD x the contiguous run of
    // CTAs [x*q + min(x, r), ...) of its q or q + 1 blocks: CTAs that share
    // a tile, and neighbouring tiles, then share one L2.
    // K-major order: the same runs over (slice, tile) pairs taken slice by
    // slice, so one XCD runs the same k range of several tiles at once.
    int b = blk;
    if (sk_block && p.sk_order != SK_ORDER_BLOCK) {
      const int q = p.sk_ctas >> 3, r = p.sk_ctas & 7, x = blk & 7;
      b = x * q + min(x, r) + (blk >> 3);
      if (p.sk_order == SK_ORDER_KMAJOR) {
        const int s = b / p.sk_tiles;
        b = (b - s * p.sk_tiles) * p.sk_slices + s;
      }
    }
    int it = 0, end = 0;
    if (sk_block) {
      it = b * p.ipc + min(b, p.extra);
      end = it + p.ipc + (b < p.extra ? 1 : 0);
    }
    int dp_tile, dp_step;
    if (p.mode == MODE_DP) {
      dp_tile = blk;
      dp_step = p.dp_tiles;  // one tile
    } else if (p.mode == MODE_DP_SK) {
      dp_tile = blk >= p.sk_ctas ? blk - p.sk_ctas : p.dp_tiles;
      dp_step = p.dp_tiles;
    } else {
      dp_tile = blk;
      dp_step = p.grid;
    }
    // Stream-K iterations [it, split) run before the DP tiles and
    // [split, end) after them.  dp / dp_sk: the whole range first.
    // persistent: first only a first segment that continues a tile begun by
    // a lower CTA (a non-owner: it hands its partial on, in a tree possibly
    // after folding still higher positions), then the DP tiles, then the
    // rest -- the owners' segments, whose partners handed on long before, so
    // their waits cost little.  A non-owner's partners are higher positions
    // of the same tile, i.e. first segments of higher CTAs, which run first
    // in those CTAs; all stream-K CTAs are resident, so every wait ends.
    int split = end;
    if (p.mode == MODE_PERSISTENT) {
      split = it;
      if (it < end && it % p.ipt != 0) split = min(end, (it / p.ipt + 1) * p.ipt);
    }
    if constexpr (kStream) {
      Walk w = {it, end, split, dp_tile, dp_step, b};
      run_stream(w);
    } else {
      // (The same walk as next_segment, written out: as a call it changes
      // the register allocation of the spilling fp8 instances.)
      while (true) {
        int tile, k0, k1, cta;
        if (it < split || (it < end && dp_tile >= p.dp_tiles)) {
          const int t = it / p.ipt;
          const int seg_end = min(end, (t + 1) * p.ipt);
          tile = p.dp_tiles + t;
          k0 = it - t * p.ipt;
          k1 = seg_end - t * p.ipt;
          cta = b;
          it = seg_end;  // strictly increases
        } else if (dp_tile < p.dp_tiles) {
          tile = dp_order(dp_tile);
          k0 = 0;
          k1 = p.ipt;
          cta = -1;
          dp_tile += dp_step;  // strictly increases
        } else {
          break;
        }
        process(tile, k0, k1, cta);
      }
    }
  }

  // The CTA's work list: stream-K iterations [it, split), then its DP tiles,
  // then the rest of its stream-K range.
  struct Walk {
    int it, end, split, dp_tile, dp_step, b;
  };
  struct Seg {
    int tile, k0, k1, cta;
  };
  SKG_DEV bool next_segment(Walk& w, Seg& sg) const {
    if (w.it < w.split || (w.it < w.end && w.dp_tile >= p.dp_tiles)) {
      const int t = w.it / p.ipt;
      const int seg_end = min(w.end, (t + 1) * p.ipt);
      sg.tile = p.dp_tiles + t;
      sg.k0 = w.it - t * p.ipt;
      sg.k1 = seg_end - t * p.ipt;
      sg.cta = w.b;
      w.it = seg_end;  // strictly increases
      return true;
    }
    if (w.dp_tile < p.dp_tiles) {
      sg.tile = dp_order(w.dp_tile);
      sg.k0 = 0;
      sg.k1 = p.ipt;
      sg.cta = -1;
      w.dp_tile += w.dp_step;  // strictly increases
      return true;
    }
    return false;
  }

  // Hands a finished segment on (fix-up and copy-out; no LDS involved on
  // the block-diagonal tiles).
  SKG_DEV void finish(const Seg& sg, const OutTile& o) {
    const Fix fx = fixup(sg.tile, sg.k0, sg.k1, sg.cta);
    if constexpr (FIX == FIX_HANDOFF) {
      if (fx.nfold > 0) fold_regs(fx);
      if (fx.how == OUT_PUBLISH) {
        publish_regs(fx.cta);
        return;
      }
      if (fx.how == OUT_SCATTER) {
        publish_regs(fx.cta);
        scatter_out(o, sg.tile, fx.cta);
        return;
      }
    }
    write_out(o, fx, fx.how == OUT_WORKSPACE ? s.ws + (size_t)(sg.tile - p.dp_tiles) * Cfg::TM * Cfg::TN
                                             : nullptr);
  }

  // Block-diagonal forward / dgrad tiles have a short reduction (a few MAC
  // iterations per tile), so the ring runs across the CTA's segments: the
  // iterations of the current segment and of the next one form one stream,
  // position q in ring entry q % D, and the refill after each barrier
  // continues into the next segment while the current one is multiplied,
  // handed on and written out (none of which touches the LDS).
  static constexpr bool kStream = kBd && !Loader::kTrans;

  // A tile's iterations past the last tap it has (a dgrad stride phase with
  // fewer taps than the largest) add nothing and are skipped.
  SKG_DEV static int seg_iters(const Seg& sg, const Loader& ld) {
    return max(0, min(sg.k1, ld.iters()) - sg.k0);
  }

  SKG_DEV void run_stream(Walk& w) {
    constexpr int D = Loader::D;
    Seg cur, nxt;
    if (!next_segment(w, cur)) return;
    Loader lc, ln;
    OutTile oc, on;
    Prob::setup(prm, p, cur.tile, lc, oc, tid);
    int nc = seg_iters(cur, lc), nn = 0;  // iterations run of cur, nxt
    bool has_nxt = next_segment(w, nxt);
    if (has_nxt) {
      Prob::setup(prm, p, nxt.tile, ln, on, tid);
      nn = seg_iters(nxt, ln);
    }
    int base = 0;    // stream position of cur's first iteration
    int issued = 0;  // positions [0, issued) are issued
    // Issues position q (q == issued) if it lies in cur or nxt.
    auto issue_next = [&]() -> bool {
      const int q = issued;
      if (q < base + nc) {
        lc.issue_iter(cur.k0 + (q - base), bd_entry(q));
      } else if (has_nxt && q < base + nc + nn) {
        ln.issue_iter(nxt.k0 + (q - base - nc), bd_entry(q));
      } else {
        return false;
      }
      ++issued;
      return true;
    };
    while (issued < D && issue_next()) {
    }
    while (true) {
      zero_acc();
      for (int i = 0; i < nc; ++i) {
        const int q = base + i;
        wait_iters(issued - 1 - q);
        lds_barrier();
        // The entry of position q-1 is free: keep the ring D positions ahead.
        while (issued < q + D && issue_next()) {
        }
        const SKG_LDS char* e = bd_entry(q);
        FragA fa;
        FragB fb;
#pragma unroll
        for (int ks = 0; ks < Cfg::KSTEPS; ++ks) {
          bd_conv_frags(fa, fb, e, ks);
          mma(fa, fb, 0);
        }
      }
      finish(cur, oc);
      if (!has_nxt) break;
      base += nc;
      cur = nxt;
      lc = ln;
      oc = on;
      nc = nn;
      has_nxt = next_segment(w, nxt);
      if (has_nxt) {
        Prob::setup(prm, p, nxt.tile, ln, on, tid);
        nn = seg_iters(nxt, ln);
      }
    }
    wait_vm<0>();
  }
};

template <class Cfg, class Prob, int FIX>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::MIN_CTAS) void sk_kernel(typename Prob::Params prm, KPlan p,
                                                            Scratch s) {
  constexpr int kLds = Cfg::BDG > 0             ? LoaderRing<typename Prob::Loader>::bytes
                       : Prob::Loader::kGrouped ? Cfg::LDS_GRP
                       : Prob::Loader::kDma     ? Cfg::LDS_DMA
                                                : Cfg::LDS;
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  Engine<Cfg, Prob, FIX> e(prm, p, s, (SKG_LDS char*)lds);
  e.run();
}

// Second stage of the workspace reduction: apply the epilogue to each
// stream-K tile's fp32 scratch.  Grid: (sk_tiles, chunks of 1024 elements).
template <class Cfg, class Prob>
__global__ __launch_bounds__(256) void stage2_kernel(typename Prob::Params prm, KPlan p, Scratch s) {
  const int sk_tile = blockIdx.x;
  const OutTile o = Prob::out_tile(prm, p, p.dp_tiles + sk_tile);
  const int dt = Prob::dtype_c(prm);
  const float* w = s.ws + (size_t)sk_tile * Cfg::TM * Cfg::TN;
  const int base = (blockIdx.y * 256 + threadIdx.x) * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = base + e;
    if (idx >= Cfg::TM * Cfg::TN) break;
    const int row = idx / Cfg::TN, col = idx % Cfg::TN;
    if (row >= o.rows || col >= o.cols) continue;
    float v = w[idx];
    if (o.sa) v *= o.sa[row * Prob::kScaleInc];
    if (o.sb) v *= o.sb[col * Prob::kScaleInc];
    const size_t oi = out_row<Prob>(o, row) + col;
    if (dt == DT_F32)
      ((float*)o.base)[oi] = v;
    else if (dt == DT_F16)
      ((uint16_t*)o.base)[oi] = to_f16_bits(v);
    else
      ((uint16_t*)o.base)[oi] = to_bf16_bits(v);
  }
}

}  // namespace skg
