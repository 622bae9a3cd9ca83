// Device-side building blocks for the gfx950 (CDNA4, wave64) kernels:
// element codecs, 16-byte lane-vector loads/stores, DPP reductions across
// lanes, and the fp8 / fp4 conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rn_internal.h"

namespace rn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct DTypeInfo;
template <>
struct DTypeInfo<kBF16> { static constexpr int bits = 16; };
template <>
struct DTypeInfo<kF32> { static constexpr int bits = 32; };
template <>
struct DTypeInfo<kFP8> { static constexpr int bits = 8; };
template <>
struct DTypeInfo<kFP4> { static constexpr int bits = 4; };

// dwords that hold N elements of dtype DT (at least one)
template <int DT, int N>
constexpr int words_for() { return (N * DTypeInfo<DT>::bits + 31) / 32; }

// ---------------------------------------------------------------------------
// Raw words: a lane vector of N elements of one dtype is N * bytes / 4 dwords.
// ---------------------------------------------------------------------------

template <int BYTES, bool NT = false>
__device__ __forceinline__ void load_words(const void* p, uint32_t (&w)[BYTES / 4]) {
  static_assert(BYTES == 4 || BYTES == 8 || BYTES == 16 || BYTES == 32, "lane vector size");
  if constexpr (BYTES == 32) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    const u32x4 a = NT ? __builtin_nontemporal_load(q) : q[0];
    const u32x4 b = NT ? __builtin_nontemporal_load(q + 1) : q[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (BYTES == 16) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    const u32x4 a = NT ? __builtin_nontemporal_load(q) : *q;
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  } else if constexpr (BYTES == 8) {
    const u32x2* q = reinterpret_cast<const u32x2*>(p);
    const u32x2 a = NT ? __builtin_nontemporal_load(q) : *q;
    w[0] = a.x; w[1] = a.y;
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    w[0] = NT ? __builtin_nontemporal_load(q) : *q;
  }
}

// Stores of write-once outputs use the nontemporal hint: they are not re-read
// by this kernel and would only evict useful lines from L2.
template <int BYTES>
__device__ __forceinline__ void store_words(void* p, const uint32_t (&w)[BYTES / 4]) {
  static_assert(BYTES == 4 || BYTES == 8 || BYTES == 16 || BYTES == 32, "lane vector size");
  if constexpr (BYTES == 32) {
    u32x4 a = {w[0], w[1], w[2], w[3]};
    u32x4 b = {w[4], w[5], w[6], w[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<u32x4*>(p) + 1);
  } else if constexpr (BYTES == 16) {
    u32x4 a = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(p));
  } else if constexpr (BYTES == 8) {
    u32x2 a = {w[0], w[1]};
    __builtin_nontemporal_store(a, reinterpret_cast<u32x2*>(p));
  } else {
    __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
  }
}

// ---------------------------------------------------------------------------
// Buffer addressing.  A buffer resource (four scalar registers) holds a base
// address and a size in bytes; raw buffer loads and stores take a 32-bit lane
// offset from that base, and the hardware range check turns an access at or
// past the size into a load of zeros or a dropped store.  A row's tail
// therefore needs no branch: lanes whose chunk lies past the end of the row
// load zeros (neutral for the sum of squares and the max) and store nothing.
// The fourth descriptor dword is the gfx9-family buffer format word (32-bit
// data format, no swizzle, stride 0: raw byte addressing).
// ---------------------------------------------------------------------------

constexpr int kBufferFormatWord = 0x00020000;
constexpr int kCachePolicyNontemporal = 2;  // "nt" on gfx94x/gfx950 (the former slc bit)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kBufferFormatWord);
}

// NT selects the nontemporal hint for data read exactly once (x, residual):
// on MI355X streaming reads with it measured 7.5 TB/s against 6.2 TB/s without
// (1.6 GB read-only probe).  Data that every row re-reads (the weight) is
// loaded without it so that it stays in the caches.
template <int BYTES, bool NT>
__device__ __forceinline__ void buffer_load_words(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                  uint32_t (&w)[BYTES / 4]) {
  static_assert(BYTES == 4 || BYTES == 8 || BYTES == 16 || BYTES == 32, "lane vector size");
  constexpr int aux = NT ? kCachePolicyNontemporal : 0;
  const int o = static_cast<int>(off);
  if constexpr (BYTES == 32) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, aux);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, o + 16, 0, aux);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (BYTES == 16) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, aux);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  } else if constexpr (BYTES == 8) {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, aux);
    w[0] = a.x; w[1] = a.y;
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, aux);
  }
}

// Write-once outputs carry the nontemporal hint: this kernel never re-reads
// them, and on MI355X the hint measured faster than plain stores for these
// streams (when each store instruction writes one contiguous run).
template <int BYTES>
__device__ __forceinline__ void buffer_store_words(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   const uint32_t (&w)[(BYTES + 3) / 4]) {
  static_assert(BYTES == 2 || BYTES == 4 || BYTES == 8 || BYTES == 16 || BYTES == 32, "lane vector size");
  const int o = static_cast<int>(off);
  if constexpr (BYTES == 32) {
    const u32x4 a = {w[0], w[1], w[2], w[3]};
    const u32x4 b = {w[4], w[5], w[6], w[7]};
    __builtin_amdgcn_raw_buffer_store_b128(a, r, o, 0, kCachePolicyNontemporal);
    __builtin_amdgcn_raw_buffer_store_b128(b, r, o + 16, 0, kCachePolicyNontemporal);
  } else if constexpr (BYTES == 16) {
    const u32x4 a = {w[0], w[1], w[2], w[3]};
    __builtin_amdgcn_raw_buffer_store_b128(a, r, o, 0, kCachePolicyNontemporal);
  } else if constexpr (BYTES == 8) {
    const u32x2 a = {w[0], w[1]};
    __builtin_amdgcn_raw_buffer_store_b64(a, r, o, 0, kCachePolicyNontemporal);
  } else if constexpr (BYTES == 4) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], r, o, 0, kCachePolicyNontemporal);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(w[0]), r, o, 0,
                                          kCachePolicyNontemporal);
  }
}

// One float or one byte at a byte offset (per-group scales).
__device__ __forceinline__ void buffer_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(off), 0, 0);
}
__device__ __forceinline__ void buffer_store_u8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(static_cast<unsigned char>(v), r, static_cast<int>(off), 0, 0);
}

// ---------------------------------------------------------------------------
// Element codecs (float32 in registers).
// ---------------------------------------------------------------------------

// bfloat16 is the upper half of a binary32: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> two bfloat16 (round to nearest even) in one dword, element 0
// in the low half: v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// float32 -> OCP fp8 E4M3FN (bias 7, 3 fraction bits, largest finite 448 =
// code 0x7E) and OCP MX fp4 E2M1 (values 0, 0.5, 1, 1.5, 2, 3, 4, 6) use the
// gfx950 conversion instructions, two elements per instruction, first operand
// in the low byte / low nibble.  Both round to nearest even.  The fp8
// conversion turns magnitudes past the format into NaN (0x7F), so values are
// first clamped to +-448 (v_med3), which makes it the saturating conversion;
// the fp4 conversion saturates at 6 by itself.  On MI355X both matched an
// encoder written from the format definitions bit for bit on every code, on
// every midpoint between neighbouring codes and its float32 neighbours, on
// out-of-range values and on 400k random values.
template <int BYTE>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, BYTE);
}

template <bool HIGH_HALF>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HIGH_HALF));
}

// Unpack a lane vector of VEC elements of dtype DT to floats.
template <int DT, int VEC>
__device__ __forceinline__ void unpack(const uint32_t (&w)[words_for<DT, VEC>()], float (&f)[VEC]) {
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
    static_assert(DT == kF32, "inputs are bf16 or f32");
#pragma unroll
    for (int i = 0; i < VEC; ++i) f[i] = __uint_as_float(w[i]);
  }
}

// Element i of a lane vector of dtype DT (bf16 or f32) as a float.
template <int DT, int N>
__device__ __forceinline__ float element(const uint32_t (&w)[N], int i) {
  if constexpr (DT == kBF16) {
    return (i & 1) ? bf16_hi(w[i / 2]) : bf16_lo(w[i / 2]);
  } else {
    static_assert(DT == kF32, "inputs are bf16 or f32");
    return __uint_as_float(w[i]);
  }
}

// Pack floats to a lane vector of dtype DT: bf16/f32 round to nearest even;
// fp8 e4m3fn and fp4 e2m1 take values already scaled into the format's range
// (codes in element order from the low byte / low nibble up).
template <int DT, int VEC>
__device__ __forceinline__ void pack(const float (&f)[VEC], uint32_t (&w)[words_for<DT, VEC>()]) {
  if constexpr (DT == kBF16) {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  } else if constexpr (DT == kF32) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) w[i] = __float_as_uint(f[i]);
  } else if constexpr (DT == kFP8) {
    static_assert(VEC % 4 == 0, "fp8 lane vectors are whole dwords");
#pragma unroll
    for (int i = 0; i < VEC / 4; ++i) {
      const uint32_t lo = cvt_fp8x2<false>(f[4 * i], f[4 * i + 1], 0u);
      w[i] = cvt_fp8x2<true>(f[4 * i + 2], f[4 * i + 3], lo);
    }
  } else {
    static_assert(DT == kFP4, "outputs are bf16, f32, fp8 or fp4");
    static_assert(VEC == 4 || VEC == 8, "fp4 lane vectors are 16 or 32 bits");
    uint32_t word = cvt_fp4x2<0>(0u, f[0], f[1]);
    word = cvt_fp4x2<1>(word, f[2], f[3]);
    if constexpr (VEC == 8) {
      word = cvt_fp4x2<2>(word, f[4], f[5]);
      word = cvt_fp4x2<3>(word, f[6], f[7]);
    }
    w[0] = word;
  }
}

// ---------------------------------------------------------------------------
// Cross-lane reductions (wave64).  DPP moves stay inside a 16-lane row:
//   quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
//   row_half_mirror (lane i of 8 <- 7 - i), row_mirror (lane i of 16 <- 15 - i).
// After these four steps every lane of a row holds the row's total, bitwise
// identical in all 16 lanes (each step adds the same two values in either
// order).  Wider groups continue with ds_swizzle (lane ^ 16 inside 32) or
// readlane of the four row totals (uniform result).
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kSwizzleXor16 = 0x401F;  // bitmask mode: and 0x1F, or 0, xor 0x10

struct OpSum {
  __device__ __forceinline__ static float apply(float a, float b) { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ static float apply(float a, float b) { return __builtin_fmaxf(a, b); }
};

// Reduce over aligned groups of G lanes (G = 2, 4, 8, 16, 32 or 64); every
// lane of a group receives the group's result.
template <int G, class Op>
__device__ __forceinline__ float group_reduce(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
  v = Op::apply(v, dpp_mov<kDppQuadXor1>(v));
  if constexpr (G >= 4) v = Op::apply(v, dpp_mov<kDppQuadXor2>(v));
  if constexpr (G >= 8) v = Op::apply(v, dpp_mov<kDppRowHalfMirror>(v));
  if constexpr (G >= 16) v = Op::apply(v, dpp_mov<kDppRowMirror>(v));
  if constexpr (G == 32) {
    v = Op::apply(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                           kSwizzleXor16)));
  }
  if constexpr (G == 64) {
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    v = Op::apply(Op::apply(r0, r1), Op::apply(r2, r3));
  }
  return v;
}

// ---------------------------------------------------------------------------
// Exact sums of float32 terms (the partial inputs and the residual).
//
// The running sum s is a float32 value and every addition goes through
// Knuth's TwoSum, an error-free transformation: t = fl(s + v) and
// e = (s + v) - t exactly, in six float32 additions and no branch.  The
// errors are summed in a double c.  The exact sum is s + c provided that sum
// of errors is itself exact, which holds whenever the largest running sum is
// below 2^74 times the last significant bit of the smallest nonzero term:
// every error is a multiple of that bit and at most 2^-24 of the running sum,
// so the sums of up to eight of them stay within 53 bits.  For nine terms or
// fewer with 8 significant bits (bf16 values) that is any set of terms within
// 2^63 of one another in magnitude; with 24 (float32), within 2^47.  (bf16
// terms within 2^12 of one another are summed exactly in float32 and c stays
// zero.)
//
// Rounding the exact sum once to a narrower format goes through round-to-odd
// at an intermediate precision: rounding to odd with at least two more bits
// than the target and then to nearest even is the same as rounding the exact
// value to nearest even once (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", IEEE
// Transactions on Computers, 2008).  Double has 53 bits, float32 24, bfloat16
// 8, so double -> float32 needs one such step and double -> bfloat16 two.
// When no addition but the last one rounded in a wave, the last float32
// addition alone rounds the exact sum (no step is needed for float32).
// ---------------------------------------------------------------------------

struct ExactSum {
  float s;   // running sum, rounded
  double c;  // exact sum of the rounding errors (within the range above)
  __device__ __forceinline__ void init(float v) {
    s = v;
    c = 0.0;
  }
  __device__ __forceinline__ void add(float v) {
    const float t = s + v;
    const float bv = t - s;
    const float e = (s - (t - bv)) + (v - bv);
    s = t;
    c += static_cast<double>(e);
  }
};

// Step a value one unit in the last place toward the exact value it
// approximates: away from zero when `away`, else toward zero (bit patterns of
// one sign are ordered like the magnitudes).
__device__ __forceinline__ double step_ulp(double t, bool away) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(t));
  return __longlong_as_double(static_cast<long long>(away ? b + 1u : b - 1u));
}
__device__ __forceinline__ float step_ulp(float f, bool away) {
  const uint32_t b = __float_as_uint(f);
  return __uint_as_float(away ? b + 1u : b - 1u);
}

// The exact sum of the accumulated terms and a last term v, rounded once to
// float32: to nearest even (ODD == false), or to odd (ODD == true) for a later
// nearest-even rounding to bfloat16.
//
// When no earlier addition of the wave rounded (c == 0 in every lane), the
// exact sum is s + v: float32 addition rounds it correctly by itself, and
// only the round-to-odd form needs that addition's error.  Otherwise the
// double-precision path: t + r == s + c exactly (a double TwoSum), t rounded
// to odd at double precision stands for s + c in any rounding to 51 bits or
// fewer.
template <bool ODD>
__device__ __forceinline__ float add_last_and_round(const ExactSum& a, float v) {
  const float t = a.s + v;
  const float bv = t - a.s;
  if (__builtin_amdgcn_ballot_w64(a.c != 0.0) == 0) {  // every earlier addition of the wave was exact
    if constexpr (!ODD) {
      return t;
    } else {
      const float e = (a.s - (t - bv)) + (v - bv);
      // t != 0 when e != 0: a zero sum of two floats is exact
      return e != 0.f && (__float_as_uint(t) & 1u) == 0 ? step_ulp(t, (e > 0.f) == (t > 0.f)) : t;
    }
  }
  const double c = a.c + static_cast<double>((a.s - (t - bv)) + (v - bv));
  const double sd = static_cast<double>(t);
  double u = sd + c;
  const double bu = u - sd;
  const double r = (sd - (u - bu)) + (c - bu);
  if (c == 0.0) u = sd;  // sd + 0 would turn a -0 sum into +0
  if (r != 0.0 && (__double_as_longlong(u) & 1) == 0) u = step_ulp(u, (r > 0.0) == (u > 0.0));
  float f = static_cast<float>(u);  // nearest even of the exact sum
  if constexpr (ODD) {
    // nonzero: the terms are multiples of 2^-149, so a nonzero sum is at
    // least 2^-149 in magnitude and never rounds to zero
    const double back = static_cast<double>(f);
    if (back != u && (__float_as_uint(f) & 1u) == 0) f = step_ulp(f, (u > back) == (f > 0.f));
  }
  return f;
}

}  // namespace rn

namespace rn {

// ---------------------------------------------------------------------------
// Block-scaled quantization of one chunk of U consecutive elements whose
// scale group spans GL = group / U neighbouring lanes (group = 128 for the
// per-128 fp8 scheme, 32 for MX, 16 for NVFP4).  The values to quantize are
// v[i] * mul with mul > 0; the group's amax is max|v| over the group times mul
// (multiplying by a positive number is monotone, so this is the max of the
// products).  Writes the scaled values into y (ready for pack<OD>) and, from
// the group's first lane, the scale (float32 amax / 448, E8M0 byte e + 127, or
// NVFP4's E4M3FN block-scale code) at index gidx of the row's scale resource,
// and the amax when requested.
// ---------------------------------------------------------------------------

template <int QS>
constexpr int scale_group() { return QS == kQGroup128 ? 128 : QS == kQMx32 ? 32 : QS == kQNv16 ? 16 : 0; }

// Value of a non-negative OCP E4M3FN code (bias 7; subnormals m * 2^-9), exact.
__device__ __forceinline__ float e4m3fn_value(uint32_t code) {
  const int e = static_cast<int>((code >> 3) & 0xF);
  const int m = static_cast<int>(code & 0x7);
  return e == 0 ? __builtin_amdgcn_ldexpf(static_cast<float>(m), -9)
                : __builtin_amdgcn_ldexpf(static_cast<float>(8 + m), e - 10);
}

template <int OD, int QS, int U>
__device__ __forceinline__ void quantize_group_chunk(const float (&v)[U], float mul, int lane, uint32_t gidx,
                                                     __amdgpu_buffer_rsrc_t sr, __amdgpu_buffer_rsrc_t ar,
                                                     bool want_amax, float (&y)[U], float tensor_scale = 0.f) {
  constexpr int QG = scale_group<QS>();
  constexpr int GL = QG / U;
  constexpr int EMAX = OD == kFP8 ? 8 : 2;  // MX: exponent of the element format's top binade
  static_assert(QG % U == 0 && GL <= 64, "scale groups");
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < U; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  const float gamax = group_reduce<GL, OpMax>(m) * mul;
  const bool leader = (lane % GL) == 0;
  if constexpr (QS == kQGroup128) {
    const float gq = gamax > 0.f ? 448.0f / gamax : 0.f;
#pragma unroll
    for (int i = 0; i < U; ++i) y[i] = (v[i] * mul) * gq;
    if (leader) buffer_store_f32(sr, gidx * 4, gamax / 448.0f);
  } else if constexpr (QS == kQNv16) {
    // NVFP4: block scale code RNE_e4m3fn(amax / (6 s_t)) (saturating), element
    // codes of v / (s_b s_t) through the hardware reciprocal (within an ulp of
    // float32, far below E2M1's steps); a zero block scale gives zero codes.
    const uint32_t sc = cvt_fp8x2<false>(gamax / (6.0f * tensor_scale), 0.f, 0u) & 0xFFu;
    const float d = e4m3fn_value(sc) * tensor_scale;
    const float r = d > 0.f ? __builtin_amdgcn_rcpf(d) : 0.f;
#pragma unroll
    for (int i = 0; i < U; ++i) y[i] = (v[i] * mul) * r;
    if (leader) buffer_store_u8(sr, gidx, sc);
  } else {
    // MX: shared exponent floor(log2 amax) - EMAX, clamped to E8M0's range;
    // an all-zero block takes the smallest scale, 2^-127.
    int se = gamax > 0.f ? __builtin_amdgcn_frexp_expf(gamax) - 1 - EMAX : -127;
    se = se < -127 ? -127 : (se > 127 ? 127 : se);
#pragma unroll
    for (int i = 0; i < U; ++i) y[i] = __builtin_amdgcn_ldexpf(v[i] * mul, -se);
    if (leader) buffer_store_u8(sr, gidx, static_cast<uint32_t>(se + 127));
  }
  if (leader && want_amax) buffer_store_f32(ar, gidx * 4, gamax);
}

}  // namespace rn
