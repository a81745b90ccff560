// Device-side building blocks shared by the kernel files of the RaggedShard /
// DBuffer layout library (gfx950): vector types, nontemporal loads, the
// stores and their cache policies, the 8-bit code formats, wavefront
// reductions, the division-free index walks and the XCD-aware renumbering of
// work items. Everything here is in an anonymous namespace: each kernel file
// gets its own copy.
//
// Every kernel is HBM-bound streaming work over plan-indexed work lists made
// once by rs_plan_load, with 16-byte vector loads (nontemporal) and stores
// (nontemporal, or with nt and sc1 set where that measured faster). The
// streaming transforms split each work item over small, short-lived
// workgroups (64-128 threads, one or two vectors each), which keep more
// independent streams in flight on gfx950 than one large workgroup per item;
// piece_index can keep runs of consecutive pieces on one XCD. No MFMA: nothing
// here is a dense contraction.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "rs_internal.h"

namespace rs {
namespace {

constexpr int kThreads = 256;
constexpr int kWave = 64;

#ifndef RS_NT
#define RS_NT 1
#endif
// Streamed data is touched once: load and store it with the nontemporal hint
// so it does not displace anything in L2 / MALL.
constexpr bool kNT = RS_NT != 0;

template <typename T>
__device__ __forceinline__ T ldg(const T* p) {
  if constexpr (kNT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <typename T>
__device__ __forceinline__ void stg(T* p, T v) {
  if constexpr (kNT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// stg for a pointer read from a table: the compiler cannot tell that it
// addresses global memory and would issue a flat store, which also counts
// against the LDS/scalar-load counter; the cast makes it a global store.
// Every buffer the library writes is device memory.
template <typename T>
__device__ __forceinline__ void stg_global(T* p, T v) {
  typedef __attribute__((address_space(1))) T* GT;
  const GT g = (GT)p;
  if constexpr (kNT) __builtin_nontemporal_store(v, g);
  else *g = v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Cache policy of a streamed store. kStoreNT is stg above (a global store,
// nontemporal). kStoreNtSc1 is a buffer store with nt and sc1 set (the
// cache-policy immediate: bit 0 sc0, bit 1 nt, bit 4 sc1). On gfx950 a cold
// 1 GiB copy ran at 6.70 TB/s with nt-sc1 stores against 6.62 with
// nontemporal ones, and each kernel takes the policy that measured faster
// for it.
constexpr int kStoreNT = 0;
constexpr int kStoreNtSc1 = 18;

// Word 3 of a raw (byte-addressed, stride 0) buffer descriptor on gfx9-family
// parts: data format 32 bits, no swizzle. The range is 2^32 - 1 bytes; every
// caller keeps its offsets under 2^31.
constexpr int kRawBufferWord3 = 0x00020000;

// The first active lane's value of a 64-bit address, in scalar registers.
// readfirstlane is int -> int: each half is widened through uint32_t, so a
// low word with bit 31 set does not spill into the high word.
__device__ __forceinline__ uint64_t first_lane(uint64_t a) {
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu)));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Store of a 4-, 8- or 16-byte value at byte offset off from base with cache
// policy SC, as a buffer store. The caller guarantees that base is the same
// in every lane of the wave and that 0 <= off < 2^31. Where a kernel has such
// a base (a block's or a run's start) this is the cheaper form: no per-store
// vote.
template <int SC, typename T>
__device__ __forceinline__ void sts_at(const void* base, int off, T v) {
  const uint64_t a0 = first_lane(reinterpret_cast<uint64_t>(base));
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(a0), 0, -1, kRawBufferWord3);
  if constexpr (sizeof(T) == 16) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, SC);
  } else if constexpr (sizeof(T) == 8) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, SC);
  } else {
    static_assert(sizeof(T) == 4, "4-, 8- or 16-byte stores");
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, SC);
  }
}

// Store of a 4-, 8- or 16-byte value with cache policy SC. A buffer store
// addresses base + 32-bit offset, with the base the same in every lane: here
// the first active lane's address. When some active lane's address is below
// it or 2 GiB or more above it, the wave takes the global store instead, so
// every lane writes exactly at p whatever the layout.
template <int SC, typename T>
__device__ __forceinline__ void sts(T* p, T v) {
  if constexpr (SC == 0) {
    stg(p, v);
  } else {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t a0 = first_lane(a);
    const uint64_t off = a - a0;
    if (__all(off < 0x80000000ull))
      sts_at<SC>(reinterpret_cast<const void*>(a0), static_cast<int>(off), v);
    else
      stg_global(p, v);
  }
}

enum Fmt { FMT_E4M3 = 0, FMT_I8 = 1, FMT_U8 = 2 };

template <int FMT>
struct QMax;
template <> struct QMax<FMT_E4M3> { static constexpr float v = 448.0f; };
template <> struct QMax<FMT_I8> { static constexpr float v = 127.0f; };
template <> struct QMax<FMT_U8> { static constexpr float v = 255.0f; };

// ------------------------------------------------------------------ codes

// OCP E4M3, saturating, round to nearest even, sign kept. In the normal range
// the fp32 significand is rounded to 3 bits by adding 0x7ffff plus the kept
// lsb at bit 20, and the exponent rebiased from 127 to 7 (120 << 3 in code
// units); below 2^-6 the code is the number of 2^-9 steps, rounded to even.
__device__ __forceinline__ uint32_t e4m3_sw(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t a = u & 0x7fffffffu;
  const uint32_t normal = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  const uint32_t sub = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  uint32_t c = a < 0x3c800000u ? sub : normal;
  c = c < 0x7eu ? c : 0x7eu;
  return c | ((u >> 24) & 0x80u);
}

__device__ __forceinline__ uint32_t i8_code(float y) {
  float r = __builtin_rintf(y);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu;
}

__device__ __forceinline__ uint32_t u8_code(float y) {
  float r = __builtin_rintf(y);
  r = fminf(fmaxf(r, 0.0f), 255.0f);
  return static_cast<uint32_t>(r);
}

// Four values -> four code bytes in one word (value k in byte k).
template <int FMT, bool HW>
__device__ __forceinline__ uint32_t encode4(float y0, float y1, float y2, float y3) {
  if constexpr (FMT == FMT_E4M3 && HW) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
    return static_cast<uint32_t>(w);
  } else if constexpr (FMT == FMT_E4M3) {
    return e4m3_sw(y0) | (e4m3_sw(y1) << 8) | (e4m3_sw(y2) << 16) | (e4m3_sw(y3) << 24);
  } else if constexpr (FMT == FMT_I8) {
    return i8_code(y0) | (i8_code(y1) << 8) | (i8_code(y2) << 16) | (i8_code(y3) << 24);
  } else {
    return u8_code(y0) | (u8_code(y1) << 8) | (u8_code(y2) << 16) | (u8_code(y3) << 24);
  }
}

template <int FMT, bool HW>
__device__ __forceinline__ uint32_t encode1(float y) {
  return encode4<FMT, HW>(y, 0.0f, 0.0f, 0.0f) & 0xffu;
}

__device__ __forceinline__ float e4m3_value_sw(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                : static_cast<float>(m) * 0.001953125f;  // m * 2^-9
  if ((c & 0x7fu) == 0x7fu) mag = __uint_as_float(0x7fc00000u);
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

template <int FMT>
__device__ __forceinline__ float decode_sw(uint32_t c) {
  if constexpr (FMT == FMT_E4M3) {
    return e4m3_value_sw(c);
  } else if constexpr (FMT == FMT_I8) {
    return static_cast<float>(static_cast<int8_t>(c));
  } else {
    return static_cast<float>(c);
  }
}

// Four code bytes of a word -> their exact values.
template <int FMT, bool HW>
__device__ __forceinline__ f32x4 decode4(uint32_t word) {
  if constexpr (FMT == FMT_E4M3 && HW) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(word), true);
    return f32x4{lo.x, lo.y, hi.x, hi.y};
  } else {
    return f32x4{decode_sw<FMT>(word & 0xffu), decode_sw<FMT>((word >> 8) & 0xffu),
                 decode_sw<FMT>((word >> 16) & 0xffu), decode_sw<FMT>(word >> 24)};
  }
}

template <int FMT, bool HW>
__device__ __forceinline__ float decode1(uint32_t c) {
  return decode4<FMT, HW>(c & 0xffu).x;
}

// ------------------------------------------------------------------ input types

// fp32 or bf16 input: elements per 16-byte vector, widening, |x| bits.
template <bool BF16>
struct In;

template <>
struct In<false> {
  static constexpr int VE = 4;
  static constexpr int EB = 4;
  __device__ static float elem(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static uint32_t absmax(const u32x4& r) {
    const uint32_t a = max(r.x & 0x7fffffffu, r.y & 0x7fffffffu);
    const uint32_t b = max(r.z & 0x7fffffffu, r.w & 0x7fffffffu);
    return max(a, b);
  }
  __device__ static void widen(const u32x4& r, float (&x)[4]) {
    x[0] = __uint_as_float(r.x); x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z); x[3] = __uint_as_float(r.w);
  }
};

template <>
struct In<true> {
  static constexpr int VE = 8;
  static constexpr int EB = 2;
  __device__ static float elem(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  // max |x| as fp32 bits: low halves compared before the shift, high halves in place
  __device__ static uint32_t absmax(const u32x4& r) {
    const uint32_t lo = max(max(r.x & 0x7fffu, r.y & 0x7fffu), max(r.z & 0x7fffu, r.w & 0x7fffu));
    const uint32_t hi = max(max(r.x & 0x7fff0000u, r.y & 0x7fff0000u),
                            max(r.z & 0x7fff0000u, r.w & 0x7fff0000u));
    return max(lo << 16, hi);
  }
  __device__ static void widen(const u32x4& r, float (&x)[8]) {
    x[0] = __uint_as_float(r.x << 16); x[1] = __uint_as_float(r.x & 0xffff0000u);
    x[2] = __uint_as_float(r.y << 16); x[3] = __uint_as_float(r.y & 0xffff0000u);
    x[4] = __uint_as_float(r.z << 16); x[5] = __uint_as_float(r.z & 0xffff0000u);
    x[6] = __uint_as_float(r.w << 16); x[7] = __uint_as_float(r.w & 0xffff0000u);
  }
};

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, kWave)));
  return v;
}

// Max over a group of NT threads (a wave, or a 256-thread workgroup via LDS).
template <int NT>
__device__ __forceinline__ uint32_t group_max(uint32_t v, int tid, uint32_t* red) {
  v = wave_max(v);
  if constexpr (NT > kWave) {
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < NT / kWave; ++w) v = max(v, red[w]);
  }
  return v;
}

// Walks vector indices tid, tid + NT, ... of a rows x vpr grid without a
// division per step: (row, col) advance by (NT / vpr, NT % vpr) with a carry.
struct GridWalk {
  int row, col, drow, dcol, vpr;
  __device__ GridWalk(int tid, int vpr_, int nt) : vpr(vpr_) {
    row = tid / vpr; col = tid - row * vpr;
    drow = nt / vpr; dcol = nt - drow * vpr;
  }
  __device__ void next() {
    row += drow; col += dcol;
    if (col >= vpr) { col -= vpr; row += 1; }
  }
};

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8). piece_index renumbers them so that G consecutive pieces of
// the buffer run on one XCD (and share its L2 and TLB), while neighbouring
// groups still alternate between XCDs. The last partial round keeps the
// identity order. A permutation of [0, n): correctness never depends on it.
template <unsigned G>
__device__ __forceinline__ unsigned piece_index(unsigned b, unsigned n) {
  if constexpr (G <= 1) {
    return b;
  } else {
    constexpr unsigned kRound = 8u * G;
    if (b >= n - n % kRound) return b;
    const unsigned slot = b / 8u, xcd = b % 8u;
    return (slot / G) * kRound + xcd * G + slot % G;
  }
}

// Nearest bf16 of an fp32, ties to even: add 0x7fff plus the kept lsb, keep
// the top half (a finite value past the overflow midpoint carries into
// infinity; infinities stay). A NaN keeps its sign and top payload bits with
// the quiet bit set: the rounding add would carry some NaN payloads into the
// exponent and sign (0x7fffffff would become -0.0).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Scale and reciprocal of a quantisation block with absmax amax (>= 0, or
// NaN) for code range Q. A finite, positive amax gives scale = fl32(amax / Q)
// and r = min(fl32(Q / amax), FLT_MAX); amax 0 gives scale 1. A block holding
// a NaN (amax NaN: the max over |x| bits lets a NaN win) or an infinity (amax
// +inf) cannot be scaled: scale is a quiet NaN 0x7FC00000 or +inf. Every
// block that is not finite and positive gets r = 0, which marks codes that
// are all 0x00; such a block dequantises to NaN (0 x NaN, 0 x inf).
__device__ __forceinline__ void block_scale(float amax, float Q, float& scale, float& r) {
  if (amax > 0.0f && amax <= FLT_MAX) {
    scale = __fdiv_rn(amax, Q);
    r = fminf(__fdiv_rn(Q, amax), FLT_MAX);
  } else {
    scale = amax == 0.0f ? 1.0f : (amax != amax ? __uint_as_float(0x7fc00000u) : amax);
    r = 0.0f;
  }
}

// Square root rounded to nearest even, for x in [kSqrtShortMin, FLT_MAX]:
// gfx950's v_sqrt_f32 estimate s is within one ulp of the root there, and
// the rounded root is s or one of its neighbours sd, su, chosen by the signs
// of the residuals x - sd*s and x - su*s (Tuckerman's rounding test), each
// from one fma, whose rounding keeps the sign of the exact residual. This
// skips the scaling of tiny inputs and the zero and infinity cases of the
// general correctly rounded sequence. Every fp32 of the range gives the same
// bits as __builtin_sqrtf under -fhip-fp32-correctly-rounded-divide-sqrt
// (rs_bench_sqrt_check); callers use that one outside the range.
constexpr float kSqrtShortMin = 0x1p-96f;
__device__ __forceinline__ float sqrt_rn_short(float x) {
  const float s = __builtin_amdgcn_sqrtf(x);
  const float sd = __uint_as_float(__float_as_uint(s) - 1u);
  const float su = __uint_as_float(__float_as_uint(s) + 1u);
  const float rd = __builtin_fmaf(-sd, s, x);
  const float ru = __builtin_fmaf(-su, s, x);
  const float r = rd <= 0.0f ? sd : s;
  return ru > 0.0f ? su : r;
}

// floor(n / d) for n < 2^16 and 1 <= d < 2^16 with m = magic_u16(d) =
// ceil(2^32 / d): n*m / 2^32 exceeds n/d by less than 2^-16 < 1/d, which
// never carries past the next integer.
__device__ __forceinline__ uint32_t magic_u16(uint32_t d) { return d == 1 ? 0u : 0xFFFFFFFFu / d + 1u; }
__device__ __forceinline__ uint32_t div_u16(uint32_t n, uint32_t d, uint32_t m) {
  return d == 1 ? n : __umulhi(n, m);
}

}  // namespace
}  // namespace rs
