// Device primitives for gfx950 (CDNA4, wave64): MFMA wrappers, buffer
// resources, cross-CTA flags, fast integer division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SKG_DEV __device__ __forceinline__
#define SKG_LDS __attribute__((address_space(3)))
#define SKG_GLOBAL __attribute__((address_space(1)))

namespace skg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum { DT_F16 = 0, DT_BF16 = 1, DT_F8 = 2, DT_F32 = 3 };
enum { MODE_DP = 0, MODE_DP_SK = 1, MODE_PERSISTENT = 2 };
enum { RED_LINEAR = 0, RED_TREE = 1, RED_ATOMIC = 2, RED_WORKSPACE = 3 };

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

SKG_DEV i32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// ---------------------------------------------------------------------------
// Cross-CTA hand-off (rocm-libraries PR #13151, commit adding the fence and
// flag leaf ops): a contributor's release store at agent scope makes its
// partial visible across the per-XCD L2s (the compiler emits the L2
// write-back before the store); the consumer polls with relaxed agent-scope
// loads and then takes an agent-scope acquire fence (the L2 invalidate)
// before it reads the partial.  Every lane of the wave performs the store and
// the poll on the same flag word.
//
// The poll is bounded: after kSpinLimit polls (a fraction of a second) the wave gives
// up, counts the event in g_skg_wait_timeouts and continues, so a broken plan
// produces wrong numbers rather than a hung device.
constexpr uint32_t kSpinLimit = 1u << 22;

static __device__ uint32_t g_skg_wait_timeouts = 0;

SKG_DEV void flag_publish(uint32_t* flag) {
  __hip_atomic_store(flag, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

SKG_DEV void flag_wait(const uint32_t* flag) {
  uint32_t n = 0;
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 1u) {
    __builtin_amdgcn_s_sleep(2);
    if (++n == kSpinLimit) {
      __hip_atomic_fetch_add(&g_skg_wait_timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
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
  SKG_DEV static void run(acc_t& c, const i32x4* a, const i32x4* b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[0]),
                                               __builtin_bit_cast(f16x8, b[0]), c, 0, 0, 0);
  }
};
template <>
struct Mfma<DT_BF16, 32> {
  static constexpr int OPB = 16, KB = 32, NACC = 16;
  typedef f32x16 acc_t;
  SKG_DEV static void run(acc_t& c, const i32x4* a, const i32x4* b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
  }
};
template <>
struct Mfma<DT_F16, 16> {
  static constexpr int OPB = 16, KB = 64, NACC = 4;
  typedef f32x4 acc_t;
  SKG_DEV static void run(acc_t& c, const i32x4* a, const i32x4* b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[0]),
                                               __builtin_bit_cast(f16x8, b[0]), c, 0, 0, 0);
  }
};
template <>
struct Mfma<DT_BF16, 16> {
  static constexpr int OPB = 16, KB = 64, NACC = 4;
  typedef f32x4 acc_t;
  SKG_DEV static void run(acc_t& c, const i32x4* a, const i32x4* b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
  }
};
// fp8 (OCP E4M3 on gfx950): the f8f6f4 family with K = 64 (32x32) or 128
// (16x16) per instruction; format code 0 selects E4M3 for both operands and
// the e8m0 block scales are fixed at 127 (2^0): the row and column scales are
// applied in the epilogue instead.
template <>
struct Mfma<DT_F8, 32> {
  static constexpr int OPB = 32, KB = 64, NACC = 16;
  typedef f32x16 acc_t;
  SKG_DEV static void run(acc_t& c, const i32x4* a, const i32x4* b) {
    const i32x8 av = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
    const i32x8 bv = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
  }
};
template <>
struct Mfma<DT_F8, 16> {
  static constexpr int OPB = 32, KB = 128, NACC = 4;
  typedef f32x4 acc_t;
  SKG_DEV static void run(acc_t& c, const i32x4* a, const i32x4* b) {
    const i32x8 av = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
    const i32x8 bv = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
  }
};

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
  return (uint32_t)(row * 64 + ((chunk ^ ((row >> 1) & 3)) << 4));
}

// ---------------------------------------------------------------------------
// Conversions used by the epilogue (round to nearest even).
SKG_DEV uint16_t to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
SKG_DEV uint16_t to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

}  // namespace skg
