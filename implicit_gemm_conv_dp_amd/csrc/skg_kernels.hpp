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
// Mainloop: operands are staged global -> registers -> LDS (double-buffered,
// one barrier per MAC iteration) and fed to wave64 MFMA from LDS with the
// register prefetch of iteration i+1 in flight while iteration i computes.
// GEMM operands are K-contiguous and copied as 16-byte chunks; wgrad operands
// are M/N-contiguous (NHWC) and go through an 8x8 register transpose so that
// LDS always holds K-contiguous rows.
#pragma once

#include "skg_device.hpp"

namespace skg {

// ---------------------------------------------------------------------------
// Plan as the kernels see it (32-bit; the host checks the ranges).
struct KPlan {
  int tiles_m, tiles_n, ipt;
  int dp_tiles, sk_tiles, sk_ctas, ipc, extra;
  int grid, mode, reduction;
};

// The caller's workspace, carved up on the host.
struct Scratch {
  uint32_t* flags;   // [sk_cta][wave], linear / tree
  float* partials;   // [sk_cta][TM][TN] fp32, linear / tree
  float* ws;         // [sk_tile][TM][TN] fp32, workspace
};

// Where an output tile lands: a row-major window with valid extent
// rows x cols, optional per-row / per-column scales.
struct OutTile {
  char* base;
  const float* sa;
  const float* sb;
  int ld;
  int rows, cols;
};

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
  FastDiv div_howo, div_wo, div_cpg, div_s;
};

// ---------------------------------------------------------------------------
template <int DT_, int TM_, int TN_, int TK_, int WM_, int WN_, int MN_>
struct TileCfg {
  static constexpr int DT = DT_, TM = TM_, TN = TN_, TK = TK_, WM = WM_, WN = WN_, MN = MN_;
  static constexpr int ESZ = DT == DT_F8 ? 1 : 2;
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
  static_assert(RB == 64 || RB == 128, "LDS row layout");
  static_assert(FM >= 1 && FN >= 1 && WTM % MN == 0 && WTN % MN == 0, "wave tile");
  static_assert(KSTEPS >= 1 && RB % Op::KB == 0, "k steps");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// ---------------------------------------------------------------------------
// GEMM (rcr) operand loader: rows of A (M x K, row-major) and of B^T (N x K,
// i.e. column-major B) are K-contiguous; each thread moves 16-byte chunks.
template <class Cfg>
struct GemmLoader {
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
template <class Cfg>
struct GemmProblem {
  typedef GemmParams Params;
  typedef GemmLoader<Cfg> Loader;

  SKG_DEV static void setup(const Params& g, const KPlan& p, int tile, Loader& ld, OutTile& out,
                               int tid) {
    const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
    const int m0 = tm * Cfg::TM, n0 = tn * Cfg::TN;
    ld.init(g, m0, n0, tid);
    out = out_tile(g, p, tile);
  }
  SKG_DEV static OutTile out_tile(const Params& g, const KPlan& p, int tile) {
    const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
    const int m0 = tm * Cfg::TM, n0 = tn * Cfg::TN;
    const int esz = g.dtype_c == DT_F32 ? 4 : 2;
    OutTile o;
    o.base = g.C + ((size_t)m0 * g.ldc + n0) * esz;
    o.sa = g.sa ? g.sa + m0 : nullptr;
    o.sb = g.sb ? g.sb + n0 : nullptr;
    o.ld = g.ldc;
    o.rows = g.M - m0;
    o.cols = g.N - n0;
    return o;
  }
  SKG_DEV static void load(const Params&, Loader& ld, int it) { ld.load(it); }
  SKG_DEV static int dtype_c(const Params& g) { return g.dtype_c; }
};

template <class Cfg>
struct WgradProblem {
  typedef WgradParams Params;
  typedef WgradLoader<Cfg> Loader;

  SKG_DEV static void setup(const Params& w, const KPlan& p, int tile, Loader& ld, OutTile& out,
                               int tid) {
    const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
    const int group = tm / w.mt_per_group;
    const int mrow0 = (tm - group * w.mt_per_group) * Cfg::TM;
    ld.init(w, group, mrow0, tn * Cfg::TN, tid);
    out = out_tile(w, p, tile);
  }
  SKG_DEV static OutTile out_tile(const Params& w, const KPlan& p, int tile) {
    const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
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
template <class Cfg, class Prob>
struct Engine {
  typedef typename Cfg::acc_t acc_t;
  typedef typename Prob::Params Params;
  typedef typename Prob::Loader Loader;
  typedef i32x4 FragA[Cfg::FM][Cfg::OPC];
  typedef i32x4 FragB[Cfg::FN][Cfg::OPC];

  const Params& prm;
  const KPlan& p;
  const Scratch& s;
  SKG_LDS char* lds;
  int tid, lane, wave, wm, wn;
  acc_t acc[Cfg::FM][Cfg::FN];

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

  // Operand fragments of k-step ks.  The rows of one wave's blocks differ by
  // multiples of 32, which leaves the swizzle unchanged, so each block is a
  // constant offset from the first.
  SKG_DEV void load_frags(FragA& fa, FragB& fb, const SKG_LDS char* stage, int ks) const {
    const int lrow = lane % Cfg::MN, lk = (lane / Cfg::MN) * Cfg::Op::OPB;
    const int chunk0 = (ks * Cfg::Op::KB + lk) >> 4;
#pragma unroll
    for (int h = 0; h < Cfg::OPC; ++h) {
      const uint32_t oa = lds_off<Cfg::RB>(wm * Cfg::WTM + lrow, chunk0 + h);
      const uint32_t ob = lds_off<Cfg::RB>(wn * Cfg::WTN + lrow, chunk0 + h);
#pragma unroll
      for (int f = 0; f < Cfg::FM; ++f)
        fa[f][h] = *(const SKG_LDS i32x4*)(stage + oa + f * Cfg::MN * Cfg::RB);
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g)
        fb[g][h] = *(const SKG_LDS i32x4*)(stage + Cfg::A_BYTES + ob + g * Cfg::MN * Cfg::RB);
    }
  }

  SKG_DEV void mma(const FragA& fa, const FragB& fb) {
#pragma unroll
    for (int f = 0; f < Cfg::FM; ++f)
#pragma unroll
      for (int g = 0; g < Cfg::FN; ++g) Cfg::Op::run(acc[f][g], fb[g], fa[f]);  // transposed block
  }

  // acc += A_tile * B_tile for the stage in LDS.  Fragments are double
  // buffered: the reads of k-step ks+1 are scheduled among the MFMAs of ks,
  // and the scheduling barriers stop the compiler from hoisting more reads
  // than that (which would not fit next to the accumulators).
  SKG_DEV void compute(const SKG_LDS char* stage) {
    FragA fa[2];
    FragB fb[2];
    load_frags(fa[0], fb[0], stage, 0);
#pragma unroll
    for (int ks = 0; ks < Cfg::KSTEPS; ++ks) {
      if (ks + 1 < Cfg::KSTEPS) load_frags(fa[(ks + 1) & 1], fb[(ks + 1) & 1], stage, ks + 1);
      mma(fa[ks & 1], fb[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // MAC iterations [k0, k1) of one tile into acc.
  SKG_DEV void mainloop(Loader& ld, int k0, int k1) {
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

  enum { OUT_STORE = 0, OUT_ATOMIC = 1, OUT_WORKSPACE = 2, OUT_PUBLISH = 3 };

  // How a finished segment leaves the CTA: first add the partials of
  // `nfold` other stream-K CTAs, in a fixed order (partner k is cta + 1 + k
  // for linear, cta + 2^k for tree), then `how`.
  struct Fix {
    int how, nfold, cta;
    bool tree;
    SKG_DEV int partner(int k) const { return tree ? cta + (1 << k) : cta + 1 + k; }
  };

  // Partial tile of stream-K CTA c: fp32, tile order [row][TN].
  SKG_DEV float* partial(int c) const { return s.partials + (size_t)c * Cfg::TM * Cfg::TN; }

  // Writes the accumulator tile out, one wave-row (WTM rows) at a time: the
  // owning waves stage it in LDS as fp32, then every thread takes a fixed
  // 4-column chunk of the staged rows, adds the partners' partials and
  //   OUT_STORE:     C = cvt((v * sa[row]) * sb[col]), round to nearest even;
  //   OUT_ATOMIC:    fp32 atomic add of (v * sa[row]) * sb[col] into C;
  //   OUT_WORKSPACE: fp32 atomic add of v into the tile's scratch wsp;
  //   OUT_PUBLISH:   stores v as this CTA's partial.
  // A wave reads and writes partials only in the rows its threads own, so
  // one flag per (CTA, wave) orders each hand-off: the producer's wave w
  // releases its flag after its last partial store; the consumer's wave w
  // acquires that flag before its first partial load.
  SKG_DEV void write_out(const OutTile& o, const Fix& fx, float* wsp) {
    constexpr int PITCH = Cfg::EPI_PITCH32;
    constexpr int CPRO = Cfg::TN / 4;                // 4-column chunks per row
    constexpr int RSTEP = Cfg::THREADS / CPRO;       // rows between a thread's chunks
    static_assert(Cfg::THREADS % CPRO == 0 && 64 % CPRO == 0, "copy-out mapping");
    const int dt = Prob::dtype_c(prm);
    const int ch = tid % CPRO, col = ch * 4;
    const bool col_ok = col < o.cols;
    const bool scaled = fx.how == OUT_STORE || fx.how == OUT_ATOMIC;
    f32x4 sb = {1.f, 1.f, 1.f, 1.f};
    if (scaled && o.sb && col_ok) {
      if (col + 4 <= o.cols) {
        sb = *(const f32x4*)(o.sb + col);
      } else {
        for (int e = 0; e < o.cols - col; ++e) sb[e] = o.sb[col + e];
      }
    }
    for (int k = 0; k < fx.nfold; ++k) flag_wait(s.flags + fx.partner(k) * Cfg::NW + wave);
#pragma unroll
    for (int pass = 0; pass < Cfg::WM; ++pass) {
      if (wm == pass) {
#pragma unroll
        for (int f = 0; f < Cfg::FM; ++f) {
          const int lrow = f * Cfg::MN + acc_row<Cfg::MN>(lane);
#pragma unroll
          for (int g = 0; g < Cfg::FN; ++g)
#pragma unroll
            for (int q = 0; q < Cfg::NACC / 4; ++q) {
              const f32x4 v = {acc[f][g][4 * q], acc[f][g][4 * q + 1], acc[f][g][4 * q + 2],
                               acc[f][g][4 * q + 3]};
              *(SKG_LDS f32x4*)(lds + lrow * PITCH + col_of(g, q) * 4) = v;
              if ((q & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
      __syncthreads();
      if (col_ok) {
        for (int lr = tid / CPRO; lr < Cfg::WTM; lr += RSTEP) {
          const int row = pass * Cfg::WTM + lr;
          if (row >= o.rows) break;
          f32x4 v = *(const SKG_LDS f32x4*)(lds + lr * PITCH + col * 4);
          const int tofs = row * Cfg::TN + col;
          for (int k = 0; k < fx.nfold; ++k) v += *(const f32x4*)(partial(fx.partner(k)) + tofs);
          const int ncol = o.cols - col < 4 ? o.cols - col : 4;
          if (fx.how == OUT_PUBLISH) {
            *(f32x4*)(partial(fx.cta) + tofs) = v;
            continue;
          }
          if (fx.how == OUT_WORKSPACE) {
            for (int e = 0; e < ncol; ++e) unsafeAtomicAdd(wsp + tofs + e, v[e]);
            continue;
          }
          const float sa = o.sa ? o.sa[row] : 1.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (v[e] * sa) * sb[e];
          const size_t idx = (size_t)row * o.ld + col;
          if (fx.how == OUT_ATOMIC) {
            float* dst = (float*)o.base + idx;
            for (int e = 0; e < ncol; ++e) unsafeAtomicAdd(dst + e, v[e]);
          } else if (dt == DT_F32) {
            float* dst = (float*)o.base + idx;
            if (ncol == 4)
              *(f32x4*)dst = v;
            else
              for (int e = 0; e < ncol; ++e) dst[e] = v[e];
          } else {
            uint16_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = dt == DT_F16 ? to_f16_bits(v[e]) : to_bf16_bits(v[e]);
            uint16_t* dst = (uint16_t*)o.base + idx;
            if (ncol == 4)
              *(uint2*)dst = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
            else
              for (int e = 0; e < ncol; ++e) dst[e] = h[e];
          }
        }
      }
      __syncthreads();
    }
    if (fx.how == OUT_PUBLISH) flag_publish(s.flags + fx.cta * Cfg::NW + wave);
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
    if (p.reduction == RED_WORKSPACE) {
      fx.how = OUT_WORKSPACE;
      return fx;
    }
    if (started && ended) return fx;  // a whole tile inside one range
    if (p.reduction == RED_ATOMIC) {
      fx.how = OUT_ATOMIC;
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

  // One bounded work loop: the stream-K range (if any) segment by segment,
  // then this block's data-parallel tiles.
  SKG_DEV void run() {
    const int b = blockIdx.x;
    int it = 0, end = 0;
    if (p.mode != MODE_DP && b < p.sk_ctas) {
      it = b * p.ipc + min(b, p.extra);
      end = it + p.ipc + (b < p.extra ? 1 : 0);
    }
    int dp_tile, dp_step;
    if (p.mode == MODE_DP) {
      dp_tile = b;
      dp_step = p.dp_tiles;  // one tile
    } else if (p.mode == MODE_DP_SK) {
      dp_tile = b >= p.sk_ctas ? b - p.sk_ctas : p.dp_tiles;
      dp_step = p.dp_tiles;
    } else {
      dp_tile = b;
      dp_step = p.grid;
    }
    while (true) {
      int tile, k0, k1, cta;
      if (it < end) {
        const int t = it / p.ipt;
        const int seg_end = min(end, (t + 1) * p.ipt);
        tile = p.dp_tiles + t;
        k0 = it - t * p.ipt;
        k1 = seg_end - t * p.ipt;
        cta = b;
        it = seg_end;  // strictly increases
      } else if (dp_tile < p.dp_tiles) {
        tile = dp_tile;
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
};

template <class Cfg, class Prob>
__global__ __launch_bounds__(Cfg::THREADS, 1) void sk_kernel(typename Prob::Params prm, KPlan p,
                                                            Scratch s) {
  __shared__ __attribute__((aligned(16))) char lds[Cfg::LDS];
  Engine<Cfg, Prob> e(prm, p, s, (SKG_LDS char*)lds);
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
    if (o.sa) v *= o.sa[row];
    if (o.sb) v *= o.sb[col];
    const size_t oi = (size_t)row * o.ld + col;
    if (dt == DT_F32)
      ((float*)o.base)[oi] = v;
    else if (dt == DT_F16)
      ((uint16_t*)o.base)[oi] = to_f16_bits(v);
    else
      ((uint16_t*)o.base)[oi] = to_bf16_bits(v);
  }
}

}  // namespace skg
