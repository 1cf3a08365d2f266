// Device primitives for gfx950 (CDNA4, wave64): MFMA wrappers, buffer
// resources, cross-CTA flags, fast integer division.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#define SKG_DEV __device__ __forceinline__
#define SKG_LDS __attribute__((address_space(3)))
#define SKG_GLOBAL __attribute__((address_space(1)))

namespace skg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum { DT_F16 = 0, DT_BF16 = 1, DT_F8 = 2, DT_F32 = 3, DT_BF8 = 4 };
enum { MODE_DP = 0, MODE_DP_SK = 1, MODE_PERSISTENT = 2 };
enum { RED_LINEAR = 0, RED_TREE = 1, RED_ATOMIC = 2, RED_WORKSPACE = 3, RED_SCATTER = 5 };

// ---------------------------------------------------------------------------
// Buffer resources.  A load whose byte offset is at or beyond num_records
// returns zero, which the loaders use for padding and ragged tails.
constexpr uint32_t kOOB = 0x80000000u;

SKG_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // 0x00020000: raw (untyped) 32-bit data format for the gfx9 descriptor.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                           0x00020000);
}

// make_rsrc of a base and size the caller knows to be wave-uniform, made
// scalar explicitly (the direct-to-LDS loads take the resource in SGPRs,
// and the compiler cannot always prove that values derived from the tile
// index are uniform).
SKG_DEV __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return make_rsrc((const void*)(uintptr_t)(((uint64_t)hi << 32) | lo), n);
}

SKG_DEV i32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// 16 bytes per lane from buffer offset voff straight into LDS: lane i lands
// at LDS byte address lds_base + 16*i (lds_base is wave-uniform).  Written
// as assembly so that the compiler does not track it: its own conservative
// wait before every later LDS read would serialise the pipeline, and the
// engine orders these loads with explicit vmcnt waits and barriers instead.
// (Loads the compiler cannot see only make its own vmcnt waits stricter.)
SKG_DEV void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :
               : "v"(voff), "s"(lds_base), "s"(r)
               : "memory", "m0");
}

// 4 bytes per lane straight into LDS (lane i at lds_base + 4*i); ordered
// like dma16, by the engine's own vmcnt waits.
SKG_DEV void dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dword %0, %2, 0 offen lds"
               :
               : "v"(voff), "s"(lds_base), "s"(r)
               : "memory", "m0");
}

SKG_DEV uint32_t lds_addr(const SKG_LDS void* p) { return (uint32_t)(uintptr_t)p; }

// Compile-time loop: f(std::integral_constant<int, i>) for i in [B, E).
template <int B, int E, class F>
SKG_DEV void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// Cross-CTA hand-off (rocm-libraries PR #13151, commit adding the fence and
// flag leaf ops: a release publish, an acquire wait, both at agent scope).
// The L2 caches of the eight XCDs are not coherent with one another, so the
// partial tiles themselves are stored and loaded at device scope (cache
// policy sc1: the stores write through to, and the loads read from, the
// level every XCD sees).  A contributor then only has to wait for its own
// partial stores to complete before it stores the flag (device scope); the
// consumer polls the flag with device-scope loads and reads the partials
// with device-scope loads.  This gives the release/acquire ordering of the
// hand-off without writing back or invalidating a whole L2, which would
// also throw away every other CTA's cached operands.  Every lane of the
// wave performs the store and the poll on the same flag word.
//
// The poll is bounded: after `limit` polls the wave gives up, counts the event
// once in g_skg_wait_timeouts and returns false, so a broken plan or a pool
// that is not resident ends as a counted failure the host can read
// (skg_fixup_timeouts) rather than a hung device.  The default limit,
// kSpinLimit, is 2^22 polls; each poll is a device-scope load (a round trip
// past the L2) followed by a short sleep, so the bound is in the order of
// seconds, far beyond any legitimate wait.
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kDeviceScope = 16;  // cache-policy bits of a buffer access: sc1

// One counter per translation unit that instantiates kernels (the library
// is built without relocatable device code); each unit exports a host
// accessor, and skg_fixup_timeouts sums them.
static __device__ uint32_t g_skg_wait_timeouts = 0;

// a + b for an accumulator that lives in an AGPR: read, add and write back
// in place, so the register allocator keeps the accumulators in AGPRs (a
// plain VALU add would move all of them to VGPRs, which do not hold them
// next to the operands).
SKG_DEV float add_in_agpr(float a, float b) {
  float t;
  asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_add_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
               : "+a"(a), "=&v"(t)
               : "v"(b));
  return a;
}
// Device-scope 16-byte store / load of a partial: per-lane byte offset
// `off` plus a wave-uniform one `soff` (an SGPR), so a run of 16-byte slots
// shares one VGPR offset.
SKG_DEV void store_dev16_s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, soff, kDeviceScope);
}
SKG_DEV f32x4 load_dev16_s(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kDeviceScope));
}

SKG_DEV void flag_publish(uint32_t* flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are done
  __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns false when the wait gave up.
SKG_DEV bool flag_wait(const uint32_t* flag, uint32_t limit) {
  uint32_t n = 0;
  bool ok = true;
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 1u) {
    __builtin_amdgcn_s_sleep(2);
    if (++n >= limit) {
      // one count per wave: every lane runs this loop
      if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(&g_skg_wait_timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = false;
      break;
    }
  }
  asm volatile("" ::: "memory");  // partial loads stay after the poll
  return ok;
}

// Waits until all n flags at `flags` are set: lane i of the wave polls flags
// i, i + 64, ...  A lane that gives up stops polling; the wave counts one
// give-up (as flag_wait does) and returns false.
SKG_DEV bool flags_wait_all(const uint32_t* flags, int n, uint32_t limit) {
  bool ok = true;
  for (int i = threadIdx.x & 63; i < n; i += 64) {
    uint32_t t = 0;
    while (__hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 1u) {
      __builtin_amdgcn_s_sleep(2);
      if (++t >= limit) {
        ok = false;
        break;
      }
    }
  }
  const bool all = __builtin_amdgcn_ballot_w64(!ok) == 0;
  if (!all && (threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(&g_skg_wait_timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::: "memory");  // partial loads stay after the polls
  return all;
}

// ---------------------------------------------------------------------------
// Unsigned division by a run-time constant (Granlund & Montgomery, "Division
// by invariant integers using multiplication", 1994): q = (hi32(n*magic) + n)
// >> shift, exact for n < 2^31.
struct FastDiv {
  uint32_t d, magic, shift;
};

SKG_DEV uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t t = __umulhi(n, f.magic);
  return (t + n) >> f.shift;
}

// ---------------------------------------------------------------------------
// MFMA instruction wrappers.  Operand layout shared by A and B: lane l feeds
// row (or column) l % MN and the OPB bytes of K starting at (l / MN) * OPB
// within the instruction's K extent.  Accumulator layout, 32x32: element i of
// lane l is row 8*(i/4) + 4*(l/32) + i%4, column l%32; 16x16: element i is
// row 4*(l/16) + i, column l%16.
template <int DT, int MN>
struct Mfma;

template <>
struct Mfma<DT_F16, 32> {
  static constexpr int OPB = 16, KB = 32, NACC = 16;
  typedef f32x16 acc_t;
  typedef i32x4 frag_t;
  SKG_DEV static void run(acc_t& c, const frag_t& a, const frag_t& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<DT_BF16, 32> {
  static constexpr int OPB = 16, KB = 32, NACC = 16;
  typedef f32x16 acc_t;
  typedef i32x4 frag_t;
  SKG_DEV static void run(acc_t& c, const frag_t& a, const frag_t& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<DT_F16, 16> {
  static constexpr int OPB = 16, KB = 64, NACC = 4;
  typedef f32x4 acc_t;
  typedef i32x4 frag_t;
  SKG_DEV static void run(acc_t& c, const frag_t& a, const frag_t& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                               __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<DT_BF16, 16> {
  static constexpr int OPB = 16, KB = 64, NACC = 4;
  typedef f32x4 acc_t;
  typedef i32x4 frag_t;
  SKG_DEV static void run(acc_t& c, const frag_t& a, const frag_t& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
// fp8 (OCP E4M3, DT_F8) and bf8 (OCP E5M2, DT_BF8) on gfx950: the f8f6f4
// family with K = 64 (32x32) or 128 (16x16) per instruction; format code 0
// selects E4M3, 1 selects E5M2, the same for both operands.  Zero scale
// operands select the unscaled instruction (no block scales, and it keeps its
// accumulator in AGPRs); the row and column scales are applied in the
// epilogue instead.
template <int FMT>
struct MfmaF8x32 {
  static constexpr int OPB = 32, KB = 64, NACC = 16;
  typedef f32x16 acc_t;
  typedef i32x8 frag_t;
  SKG_DEV static void run(acc_t& c, const frag_t& a, const frag_t& b) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
  }
  // With OCP MX block scales: each lane's operand data is one 32-element
  // block along K (32 bytes), and the lane's E8M0 scale byte (bits 7:0 of
  // sa / sb) multiplies that block: 2^(code - 127).
  SKG_DEV static void run_scaled(acc_t& c, const frag_t& a, const frag_t& b, uint32_t sa, uint32_t sb) {
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, (int)sa, 0, (int)sb);
  }
};
template <int FMT>
struct MfmaF8x16 {
  static constexpr int OPB = 32, KB = 128, NACC = 4;
  typedef f32x4 acc_t;
  typedef i32x8 frag_t;
  SKG_DEV static void run(acc_t& c, const frag_t& a, const frag_t& b) {
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, 0, 0, 0, 0);
  }
};
template <>
struct Mfma<DT_F8, 32> : MfmaF8x32<0> {};
template <>
struct Mfma<DT_F8, 16> : MfmaF8x16<0> {};
template <>
struct Mfma<DT_BF8, 32> : MfmaF8x32<1> {};
template <>
struct Mfma<DT_BF8, 16> : MfmaF8x16<1> {};

// One operand fragment from two 16-byte LDS reads (OPB = 32) or one.
template <class FragT>
SKG_DEV FragT frag_from(const SKG_LDS char* p0, const SKG_LDS char* p1) {
  if constexpr (sizeof(FragT) == 32) {
    const i32x4 lo = *(const SKG_LDS i32x4*)p0, hi = *(const SKG_LDS i32x4*)p1;
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    return *(const SKG_LDS FragT*)p0;
  }
}

// The engine calls the MFMA with the B fragment first, so it computes the
// transposed block: accumulator element e of lane l is output row l % MN and
// output column 8*(e/4) + 4*(l/32) + e%4 (32x32) or 4*(l/16) + e (16x16);
// each group of four elements is four consecutive columns of one row.
template <int MN>
SKG_DEV int acc_row(int lane) {
  return lane & (MN - 1);
}
template <int MN>
SKG_DEV int acc_col(int e, int lane) {
  return MN == 32 ? 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3) : 4 * (lane >> 4) + e;
}

// ---------------------------------------------------------------------------
// LDS tile layout: rows of RB bytes (one row per M or N index, K contiguous),
// 16-byte chunks permuted within a row so that the MFMA operand reads (16
// consecutive rows, one chunk) and the transposing loader's writes (rows
// i, i+8, i+16, ... one chunk each) spread over the banks.
template <int RB>
SKG_DEV uint32_t lds_off(int row, int chunk);

template <>
SKG_DEV uint32_t lds_off<128>(int row, int chunk) {
  const int prow = row ^ ((row >> 3) & 1);
  return (uint32_t)(prow * 128 + ((chunk ^ (row & 7)) << 4));
}
template <>
SKG_DEV uint32_t lds_off<64>(int row, int chunk) {
  return (uint32_t)(row * 64 + ((chunk ^ (((row >> 1) ^ (row >> 3)) & 3)) << 4));
}
// Inverse of lds_off<RB>: the (row, chunk) stored in 16-byte slot s of a
// stage (both permutations are involutions).
template <int RB>
SKG_DEV void lds_slot(int s, int& row, int& chunk);
template <>
SKG_DEV void lds_slot<64>(int s, int& row, int& chunk) {
  row = s >> 2;
  chunk = (s & 3) ^ (((row >> 1) ^ (row >> 3)) & 3);
}
template <>
SKG_DEV void lds_slot<128>(int s, int& row, int& chunk) {
  const int prow = s >> 3;
  row = prow ^ ((prow >> 3) & 1);
  chunk = (s & 7) ^ (row & 7);
}

// Waits written as inline assembly with a memory clobber, so the compiler
// neither moves memory operations across them nor adds waits of its own:
// wait_vm<n>() returns once at most n vector memory operations of this wave
// are outstanding; lds_barrier() completes this wave's LDS reads and then
// synchronises the workgroup.
template <int N>
SKG_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
SKG_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Conversions used by the epilogue (round to nearest even).
SKG_DEV uint16_t to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
SKG_DEV uint16_t to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}
// Two values rounded to nearest even and packed (a in the low half): one
// v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 on gfx950.
SKG_DEV uint32_t pack_f16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), f16x2));
}
SKG_DEV uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

}  // namespace skg
