// HIP kernels for gfx950 (CDNA4) and the transform entry points of the
// RaggedShard / DBuffer layout library.
//
// Every kernel is HBM-bound streaming work over plan-indexed work lists made
// once by rs_plan_load, with 16-byte nontemporal vector loads and stores.
// The streaming transforms (unpack, pack, the row-run gather, the tile-major
// reorder) split each work item over small, short-lived workgroups (64-128
// threads, one or two vectors each), which keep more independent streams in
// flight on gfx950 than one large workgroup per item; piece_index can keep
// runs of consecutive pieces on one XCD. Quantisation keeps a whole tile
// (512 threads) or a whole flat block (one wave) in registers, so each input
// byte is read from HBM once; the block absmax is a wave shuffle reduction
// plus, for tiles, an LDS combine over the waves. No MFMA: nothing here is a
// dense contraction.
//
// Arithmetic follows "veScale-FSDP: flexible, structure-aware sharding at
// 10K-GPU scale" (feynmanwiki walkthrough, DBuffer paragraph on fused add /
// scale / zero / copy; the block-wise quantisation and 8-bit Adam
// paragraphs) with IEEE fp32 round-to-nearest-even operations written out
// (__fmul_rn, __fadd_rn, __fdiv_rn) and no contraction into FMA.
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// ------------------------------------------------------------------ quant

// One quantisation block: element (r, c) at base + r*stride + c, r < rows,
// c < cols, handled by NT threads (tid in [0, NT)). Fast path: every vector
// of the block stays in registers (at most NT*MAXV 16-byte vectors, rows and
// base aligned to a vector). Otherwise: two passes over memory, element by
// element.
template <bool BF16, int FMT, bool HW, int NT, int MAXV>
__device__ void quant_block(const void* __restrict__ src, uint8_t* __restrict__ q,
                            float* __restrict__ scales, int64_t base, int64_t stride, int rows,
                            int cols, int64_t sidx, int tid, uint32_t* red) {
  using I = In<BF16>;
  constexpr int VE = I::VE;
  constexpr float Q = QMax<FMT>::v;
  const int vpr = cols / VE;
  const int nvec = rows * vpr;
  const bool fast = (base % VE == 0) && (stride % VE == 0) && (cols % VE == 0) && nvec <= NT * MAXV;
  const char* sb = static_cast<const char*>(src);

  if (fast) {
    u32x4 raw[MAXV];
    uint32_t m = 0;
    {
      GridWalk w(tid, vpr, NT);
#pragma unroll
      for (int k = 0; k < MAXV; ++k) {
        if (tid + k * NT < nvec) {
          const int64_t e = base + static_cast<int64_t>(w.row) * stride + static_cast<int64_t>(w.col) * VE;
          raw[k] = ldg(reinterpret_cast<const u32x4*>(sb + e * I::EB));
          m = max(m, I::absmax(raw[k]));
        }
        w.next();
      }
    }
    const float amax = __uint_as_float(group_max<NT>(m, tid, red));
    const bool zero = amax == 0.0f;
    const float r = zero ? 0.0f : fminf(__fdiv_rn(Q, amax), FLT_MAX);
    if (tid == 0) scales[sidx] = zero ? 1.0f : __fdiv_rn(amax, Q);
    GridWalk w(tid, vpr, NT);
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
      if (tid + k * NT < nvec) {
        const int64_t e = base + static_cast<int64_t>(w.row) * stride + static_cast<int64_t>(w.col) * VE;
        float x[VE];
        I::widen(raw[k], x);
        uint32_t words[VE / 4];
#pragma unroll
        for (int h = 0; h < VE / 4; ++h) {
          words[h] = zero ? 0u
                          : encode4<FMT, HW>(__fmul_rn(x[4 * h], r), __fmul_rn(x[4 * h + 1], r),
                                             __fmul_rn(x[4 * h + 2], r), __fmul_rn(x[4 * h + 3], r));
        }
        if constexpr (VE == 8) {
          stg(reinterpret_cast<u32x2*>(q + e), u32x2{words[0], words[1]});
        } else {
          stg(reinterpret_cast<uint32_t*>(q + e), words[0]);
        }
      }
      w.next();
    }
    return;
  }

  // general path: any alignment, any block size
  const int64_t total = static_cast<int64_t>(rows) * cols;
  uint32_t m = 0;
  for (int64_t i = tid; i < total; i += NT) {
    const int64_t rr = i / cols, cc = i - rr * cols;
    m = max(m, __float_as_uint(I::elem(src, base + rr * stride + cc)) & 0x7fffffffu);
  }
  const float amax = __uint_as_float(group_max<NT>(m, tid, red));
  const bool zero = amax == 0.0f;
  const float r = zero ? 0.0f : fminf(__fdiv_rn(Q, amax), FLT_MAX);
  if (tid == 0) scales[sidx] = zero ? 1.0f : __fdiv_rn(amax, Q);
  for (int64_t i = tid; i < total; i += NT) {
    const int64_t rr = i / cols, cc = i - rr * cols;
    const int64_t e = base + rr * stride + cc;
    q[e] = zero ? 0 : static_cast<uint8_t>(encode1<FMT, HW>(__fmul_rn(I::elem(src, e), r)));
  }
}

// Zero [base, base + len) of a byte array (codes) with 16-byte stores in the
// middle, by NT threads.
template <int NT = kThreads>
__device__ void zero_bytes(uint8_t* q, int64_t base, int64_t len, int tid) {
  const int64_t end = base + len;
  const int64_t a0 = (base + 15) & ~int64_t(15);
  const int64_t a1 = end & ~int64_t(15);
  if (a0 >= a1) {
    for (int64_t i = base + tid; i < end; i += NT) q[i] = 0;
    return;
  }
  for (int64_t i = base + tid; i < a0; i += NT) q[i] = 0;
  for (int64_t i = a1 + tid; i < end; i += NT) q[i] = 0;
  u32x4* v = reinterpret_cast<u32x4*>(q + a0);
  const int64_t nv = (a1 - a0) >> 4;
  for (int64_t i = tid; i < nv; i += NT) stg(v + i, u32x4{0u, 0u, 0u, 0u});
}

// Zero [base, base + len) of an fp32 array with 16-byte stores in the
// middle, by NT threads.
template <int NT = kThreads>
__device__ void zero_f32(float* o, int64_t base, int64_t len, int tid) {
  const int64_t end = base + len;
  const int64_t a0 = (base + 3) & ~int64_t(3);
  const int64_t a1 = end & ~int64_t(3);
  if (a0 >= a1) {
    for (int64_t i = base + tid; i < end; i += NT) o[i] = 0.0f;
    return;
  }
  for (int64_t i = base + tid; i < a0; i += NT) o[i] = 0.0f;
  for (int64_t i = a1 + tid; i < end; i += NT) o[i] = 0.0f;
  f32x4* v = reinterpret_cast<f32x4*>(o + a0);
  const int64_t nv = (a1 - a0) >> 2;
  for (int64_t i = tid; i < nv; i += NT) stg(v + i, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
}

// One workgroup per tile. Workgroups from n_main on take the zero-range jobs
// that follow the tiles in the list and clear code bytes outside every block,
// so the whole call is one launch.
// kQuantThreads threads per tile; the register path holds a whole tile of up
// to 16384 elements (2048 16-byte vectors of bf16, 4096 of fp32).
template <bool BF16, int FMT, bool HW>
__device__ __forceinline__ void quant_tile_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs, int64_t n_main,
                                                                   const void* __restrict__ src,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ scales) {
  __shared__ uint32_t red[kQuantThreads / kWave];
  const unsigned b = piece_index<kTileXcdGroup>(jb, n_jobs);
  const QJob j = jobs[b];
  if (static_cast<int64_t>(b) >= n_main) {
    zero_bytes<kQuantThreads>(q, j.base, j.stride, threadIdx.x);
    return;
  }
  quant_block<BF16, FMT, HW, kQuantThreads, (BF16 ? 2048 : 4096) / kQuantThreads>(
      src, q, scales, j.base, j.stride, j.rows, j.cols, j.scale, threadIdx.x, red);
}

template <bool BF16, int FMT, bool HW>
__global__ __launch_bounds__(kQuantThreads) void quant_tile_kernel(const QJob* __restrict__ jobs, int64_t n_main,
                                                                   const void* __restrict__ src,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ scales, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    quant_tile_kernel_job<BF16, FMT, HW>(jb, n_jobs, jobs, n_main, src, q, scales);
    __syncthreads();   // the next job reuses this workgroup's LDS
  }
}

// One wave per flat block, kFlatPerGroup blocks per workgroup; zero-range jobs
// from n_main on, as in the tile kernel.
template <bool BF16, int FMT, bool HW>
__device__ __forceinline__ void quant_flat_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs, int64_t n_main,
                                                              const void* __restrict__ src,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ scales) {
  const unsigned b = piece_index<kFlatXcdGroup>(jb, n_jobs);
  const QJob j = jobs[b];
  if (static_cast<int64_t>(b) >= n_main) {
    zero_bytes<kFlatThreads>(q, j.base, j.stride, threadIdx.x);
    return;
  }
  const int wave = threadIdx.x / kWave;
  if (wave >= j.rows) return;
  const int len = wave == j.rows - 1 ? j.last : j.cols;
  quant_block<BF16, FMT, HW, kWave, 8>(src, q, scales, j.base + static_cast<int64_t>(wave) * j.cols, len,
                                       1, len, j.scale + wave, threadIdx.x & (kWave - 1), nullptr);
}

template <bool BF16, int FMT, bool HW>
__global__ __launch_bounds__(kFlatThreads) void quant_flat_kernel(const QJob* __restrict__ jobs, int64_t n_main,
                                                              const void* __restrict__ src,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ scales, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    quant_flat_kernel_job<BF16, FMT, HW>(jb, n_jobs, jobs, n_main, src, q, scales);
  }
}

// Code bytes of positions outside every block (a plan with no block at all).
__device__ __forceinline__ void zero_codes_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs,
                                                              uint8_t* __restrict__ q) {
  const QJob j = jobs[jb];
  zero_bytes(q, j.base, j.stride, threadIdx.x);
}

__global__ __launch_bounds__(kThreads) void zero_codes_kernel(const QJob* __restrict__ jobs,
                                                              uint8_t* __restrict__ q, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    zero_codes_kernel_job(jb, n_jobs, jobs, q);
  }
}

// ------------------------------------------------------------------ dequant

template <int FMT, bool HW, int NT>
__device__ void dequant_block(const uint8_t* __restrict__ q, float* __restrict__ out, float s,
                              int64_t base, int64_t stride, int rows, int cols, int tid) {
  if ((base % 4 == 0) && (stride % 4 == 0) && (cols % 4 == 0)) {
    const int vpr = cols / 4;
    const int nvec = rows * vpr;
    GridWalk w(tid, vpr, NT);
    for (int i = tid; i < nvec; i += NT) {
      const int64_t e = base + static_cast<int64_t>(w.row) * stride + static_cast<int64_t>(w.col) * 4;
      const f32x4 d = decode4<FMT, HW>(ldg(reinterpret_cast<const uint32_t*>(q + e)));
      stg(reinterpret_cast<f32x4*>(out + e),
          f32x4{__fmul_rn(d.x, s), __fmul_rn(d.y, s), __fmul_rn(d.z, s), __fmul_rn(d.w, s)});
      w.next();
    }
    return;
  }
  const int64_t total = static_cast<int64_t>(rows) * cols;
  for (int64_t i = tid; i < total; i += NT) {
    const int64_t rr = i / cols, cc = i - rr * cols;
    const int64_t e = base + rr * stride + cc;
    out[e] = __fmul_rn(decode1<FMT, HW>(q[e]), s);
  }
}

// Workgroups from n_main on clear the values outside every block (zero-range
// jobs), as in the quant kernels.
template <int FMT, bool HW>
__device__ __forceinline__ void dequant_tile_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs, int64_t n_main,
                                                                const uint8_t* __restrict__ q,
                                                                const float* __restrict__ scales,
                                                                float* __restrict__ out) {
  const unsigned b = piece_index<kTileXcdGroup>(jb, n_jobs);
  const QJob j = jobs[b];
  if (static_cast<int64_t>(b) >= n_main) {
    zero_f32(out, j.base, j.stride, threadIdx.x);
    return;
  }
  dequant_block<FMT, HW, kThreads>(q, out, scales[j.scale], j.base, j.stride, j.rows, j.cols,
                                   threadIdx.x);
}

template <int FMT, bool HW>
__global__ __launch_bounds__(kThreads) void dequant_tile_kernel(const QJob* __restrict__ jobs, int64_t n_main,
                                                                const uint8_t* __restrict__ q,
                                                                const float* __restrict__ scales,
                                                                float* __restrict__ out, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    dequant_tile_kernel_job<FMT, HW>(jb, n_jobs, jobs, n_main, q, scales, out);
  }
}

template <int FMT, bool HW>
__device__ __forceinline__ void dequant_flat_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs, int64_t n_main,
                                                                const uint8_t* __restrict__ q,
                                                                const float* __restrict__ scales,
                                                                float* __restrict__ out) {
  const unsigned b = piece_index<kFlatXcdGroup>(jb, n_jobs);
  const QJob j = jobs[b];
  if (static_cast<int64_t>(b) >= n_main) {
    zero_f32<kFlatThreads>(out, j.base, j.stride, threadIdx.x);
    return;
  }
  const int wave = threadIdx.x / kWave;
  if (wave >= j.rows) return;
  const int len = wave == j.rows - 1 ? j.last : j.cols;
  dequant_block<FMT, HW, kWave>(q, out, scales[j.scale + wave], j.base + static_cast<int64_t>(wave) * j.cols,
                                len, 1, len, threadIdx.x & (kWave - 1));
}

template <int FMT, bool HW>
__global__ __launch_bounds__(kFlatThreads) void dequant_flat_kernel(const QJob* __restrict__ jobs, int64_t n_main,
                                                                const uint8_t* __restrict__ q,
                                                                const float* __restrict__ scales,
                                                                float* __restrict__ out, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    dequant_flat_kernel_job<FMT, HW>(jb, n_jobs, jobs, n_main, q, scales, out);
  }
}

// Dequantised values of positions outside every block (a plan with no block at all).
__device__ __forceinline__ void zero_values_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs,
                                                               float* __restrict__ out) {
  const QJob j = jobs[jb];
  zero_f32(out, j.base, j.stride, threadIdx.x);
}

__global__ __launch_bounds__(kThreads) void zero_values_kernel(const QJob* __restrict__ jobs,
                                                               float* __restrict__ out, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    zero_values_kernel_job(jb, n_jobs, jobs, out);
  }
}

// ------------------------------------------------------------------ gather side

// Nearest bf16 of a finite fp32, ties to even: add 0x7fff plus the kept lsb,
// keep the top half.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One block of gathered codes -> its values inside the full tensor: element
// (r, c) comes from q[qbase + r*stride + c] and goes to dst[dbase + r*stride + c]
// as fl32(decode * s), rounded to bf16 when BF16OUT. Eight codes per 8-byte
// load, four loads in flight per thread.
template <int FMT, bool HW, bool BF16OUT, int NT>
__device__ void gather_block(const uint8_t* __restrict__ q, void* __restrict__ dst, float s,
                             int64_t qbase, int64_t dbase, int64_t stride, int64_t dstride, int rows,
                             int cols, int tid) {
  if ((qbase % 8 == 0) && (dbase % 8 == 0) && (stride % 8 == 0) && (dstride % 8 == 0) && (cols % 8 == 0)) {
    constexpr int U = 4;
    const int vpr = cols / 8;
    const int nvec = rows * vpr;
    GridWalk w(tid, vpr, NT);
    for (int i0 = tid; i0 < nvec; i0 += NT * U) {
      u32x2 c[U];
      int64_t off[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        off[u] = static_cast<int64_t>(w.row) * dstride + static_cast<int64_t>(w.col) * 8;
        if (i0 + u * NT < nvec)
          c[u] = ldg(reinterpret_cast<const u32x2*>(q + qbase + static_cast<int64_t>(w.row) * stride +
                                                     static_cast<int64_t>(w.col) * 8));
        w.next();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i0 + u * NT >= nvec) continue;
        const f32x4 a = decode4<FMT, HW>(c[u].x), b = decode4<FMT, HW>(c[u].y);
        const float v[8] = {__fmul_rn(a.x, s), __fmul_rn(a.y, s), __fmul_rn(a.z, s), __fmul_rn(a.w, s),
                            __fmul_rn(b.x, s), __fmul_rn(b.y, s), __fmul_rn(b.z, s), __fmul_rn(b.w, s)};
        if constexpr (BF16OUT) {
          const u32x4 o{bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16),
                        bf16_rne(v[4]) | (bf16_rne(v[5]) << 16), bf16_rne(v[6]) | (bf16_rne(v[7]) << 16)};
          stg(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + dbase + off[u]), o);
        } else {
          f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(dst) + dbase + off[u]);
          stg(o, f32x4{v[0], v[1], v[2], v[3]});
          stg(o + 1, f32x4{v[4], v[5], v[6], v[7]});
        }
      }
    }
    return;
  }
  const int64_t total = static_cast<int64_t>(rows) * cols;
  for (int64_t i = tid; i < total; i += NT) {
    const int64_t rr = i / cols, cc = i - rr * cols;
    const float v = __fmul_rn(decode1<FMT, HW>(q[qbase + rr * stride + cc]), s);
    const int64_t d = dbase + rr * dstride + cc;
    if constexpr (BF16OUT)
      static_cast<uint16_t*>(dst)[d] = static_cast<uint16_t>(bf16_rne(v));
    else
      static_cast<float*>(dst)[d] = v;
  }
}

// floor(n / d) for n < 2^16 and 1 <= d < 2^16 with m = magic_u16(d) =
// ceil(2^32 / d): n*m / 2^32 exceeds n/d by less than 2^-16 < 1/d, which
// never carries past the next integer.
__device__ __forceinline__ uint32_t magic_u16(uint32_t d) { return d == 1 ? 0u : 0xFFFFFFFFu / d + 1u; }
__device__ __forceinline__ uint32_t div_u16(uint32_t n, uint32_t d, uint32_t m) {
  return d == 1 ? n : __umulhi(n, m);
}

// Contiguous row runs of a quantised tensor (see GatherChunk). Each lane turns
// VEC codes into one 16-byte store (8 codes -> 8 bf16, 4 codes -> 4 fp32), so
// the lanes of a wave read and write one contiguous range each. Workgroup b
// takes piece b % split of run b / split: kGatherVec vectors per thread, and
// again split pieces further on while the run lasts. A run of several rows
// holds fewer than 2^16 vectors (the lowering keeps it under 16384 elements),
// so its row and tile-column indices come from div_u16.
template <int FMT, bool HW, bool BF16OUT>
__device__ __forceinline__ void gather_rows_kernel_piece(unsigned b, const GatherChunk* __restrict__ chunks,
                                                                    const uint8_t* __restrict__ q,
                                                                    const float* __restrict__ scales,
                                                                    void* const* __restrict__ dst, int split) {
  constexpr int VEC = BF16OUT ? 8 : 4;
  constexpr int U = kGatherVec;
  const unsigned cu = b / static_cast<unsigned>(split);
  const int ci = static_cast<int>(cu);
  const int piece = static_cast<int>(b - cu * static_cast<unsigned>(split));
  const GatherChunk c = chunks[ci];
  void* out = dst[c.tensor];
  const uint32_t vpr = static_cast<uint32_t>(c.cols / VEC);
  const int nvec = c.rows * static_cast<int>(vpr);
  const uint8_t* qb = q + c.qbase;
  const bool band = c.rstep == 0;
  const uint32_t mv = magic_u16(vpr);
  const uint32_t cpt = band ? static_cast<uint32_t>(c.bc / VEC) : 1u;   // vectors per tile column
  const uint32_t mc = magic_u16(cpt);
  const int pass = split * static_cast<int>(kGatherPiece);
  for (int i0 = piece * static_cast<int>(kGatherPiece) + static_cast<int>(threadIdx.x); i0 < nvec; i0 += pass) {
    uint32_t code[U][VEC / 4];
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kGatherThreads;
      if (i < nvec) {
        if constexpr (VEC == 8) {
          const u32x2 t = ldg(reinterpret_cast<const u32x2*>(qb) + i);
          code[u][0] = t.x;
          code[u][1] = t.y;
        } else {
          code[u][0] = ldg(reinterpret_cast<const uint32_t*>(qb) + i);
        }
        const uint32_t row = c.rows == 1 ? 0u : div_u16(static_cast<uint32_t>(i), vpr, mv);
        if (band) {
          const uint32_t col = static_cast<uint32_t>(i) - row * vpr;
          sc[u] = scales[c.scale0 + div_u16(col, cpt, mc)];
        } else {
          sc[u] = scales[c.scale0 + row];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kGatherThreads;
      if (i >= nvec) continue;
      const int64_t e = c.toff + static_cast<int64_t>(i) * VEC;
      float v[VEC];
#pragma unroll
      for (int h = 0; h < VEC / 4; ++h) {
        const f32x4 d = decode4<FMT, HW>(code[u][h]);
        v[4 * h] = __fmul_rn(d.x, sc[u]);
        v[4 * h + 1] = __fmul_rn(d.y, sc[u]);
        v[4 * h + 2] = __fmul_rn(d.z, sc[u]);
        v[4 * h + 3] = __fmul_rn(d.w, sc[u]);
      }
      if constexpr (BF16OUT) {
        stg(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + e),
            u32x4{bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16),
                  bf16_rne(v[4]) | (bf16_rne(v[5]) << 16), bf16_rne(v[6]) | (bf16_rne(v[7]) << 16)});
      } else {
        stg(reinterpret_cast<f32x4*>(static_cast<float*>(out) + e), f32x4{v[0], v[1], v[2], v[3]});
      }
    }
  }
}

template <int FMT, bool HW, bool BF16OUT>
__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(const GatherChunk* __restrict__ chunks,
                                                                    const uint8_t* __restrict__ q,
                                                                    const float* __restrict__ scales,
                                                                    void* const* __restrict__ dst, int split, unsigned n_pieces) {
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    gather_rows_kernel_piece<FMT, HW, BF16OUT>(piece_index<kGatherXcdGroup>(p, n_pieces), chunks, q, scales, dst, split);
}

template <int FMT, bool HW, bool BF16OUT>
__device__ __forceinline__ void gather_tile_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs,
                                                               const uint8_t* __restrict__ q,
                                                               const float* __restrict__ scales,
                                                               void* const* __restrict__ dst) {
  const QJob j = jobs[jb];
  gather_block<FMT, HW, BF16OUT, kThreads>(q, dst[j.tensor], scales[j.scale], j.base, j.toff, j.stride,
                                           j.tstride, j.rows, j.cols, threadIdx.x);
}

template <int FMT, bool HW, bool BF16OUT>
__global__ __launch_bounds__(kThreads) void gather_tile_kernel(const QJob* __restrict__ jobs,
                                                               const uint8_t* __restrict__ q,
                                                               const float* __restrict__ scales,
                                                               void* const* __restrict__ dst, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    gather_tile_kernel_job<FMT, HW, BF16OUT>(jb, n_jobs, jobs, q, scales, dst);
  }
}

template <int FMT, bool HW, bool BF16OUT>
__device__ __forceinline__ void gather_flat_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs,
                                                               const uint8_t* __restrict__ q,
                                                               const float* __restrict__ scales,
                                                               void* const* __restrict__ dst) {
  const QJob j = jobs[jb];
  const int wave = threadIdx.x / kWave;
  if (wave >= j.rows) return;
  const int len = wave == j.rows - 1 ? j.last : j.cols;
  const int64_t step = static_cast<int64_t>(wave) * j.cols;
  gather_block<FMT, HW, BF16OUT, kWave>(q, dst[j.tensor], scales[j.scale + wave], j.base + step,
                                        j.toff + step, len, len, 1, len, threadIdx.x & (kWave - 1));
}

template <int FMT, bool HW, bool BF16OUT>
__global__ __launch_bounds__(kFlatThreads) void gather_flat_kernel(const QJob* __restrict__ jobs,
                                                               const uint8_t* __restrict__ q,
                                                               const float* __restrict__ scales,
                                                               void* const* __restrict__ dst, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    gather_flat_kernel_job<FMT, HW, BF16OUT>(jb, n_jobs, jobs, q, scales, dst);
  }
}

// ------------------------------------------------------------------ 8-bit Adam step

struct AdamK {
  float b1, b2, c1, c2, eps, step_size, inv_bc2_sqrt, decay;
};

// m1, v1 and the new parameter of one element (every operation rounded).
// The square root is __builtin_sqrtf, which this build (correctly rounded
// divide and sqrt) lowers to a correctly rounded sequence; __fsqrt_rn is not
// correctly rounded on this toolchain (about 15% of inputs differ by an ulp).
__device__ __forceinline__ void adam_elem(float p, float g, float m0, float v0, const AdamK& k,
                                          float& p1, float& m1, float& v1) {
  m1 = __fadd_rn(__fmul_rn(k.b1, m0), __fmul_rn(k.c1, g));
  v1 = __fadd_rn(__fmul_rn(k.b2, v0), __fmul_rn(k.c2, __fmul_rn(g, g)));
  const float den = __fadd_rn(__fmul_rn(__builtin_sqrtf(v1), k.inv_bc2_sqrt), k.eps);
  p1 = __fsub_rn(__fmul_rn(p, k.decay), __fmul_rn(k.step_size, __fdiv_rn(m1, den)));
}

// Scale and reciprocal of a block with absmax `amax` for code range Q.
__device__ __forceinline__ void block_scale(float amax, float Q, float& scale, float& r) {
  const bool zero = amax == 0.0f;
  scale = zero ? 1.0f : __fdiv_rn(amax, Q);
  r = zero ? 0.0f : fminf(__fdiv_rn(Q, amax), FLT_MAX);
}

// One quantisation block (element (r, c) at base + r*stride + c) handled by
// NT threads. The old scales are read before the block's max is reduced and
// the new ones written after it. Fast path: 4-element vectors, every updated
// m and v kept in registers; otherwise two passes (the second recomputes m1
// and v1 from the old codes, which it then overwrites).
template <int NT, int MAXV>
__device__ void adam_block(float* __restrict__ param, const float* __restrict__ grad,
                           uint8_t* __restrict__ qm, float* __restrict__ sm, uint8_t* __restrict__ qv,
                           float* __restrict__ sv, int64_t base, int64_t stride, int rows, int cols,
                           int64_t sidx, int tid, uint32_t* red, const AdamK& k) {
  const float sm0 = sm[sidx], sv0 = sv[sidx];
  const int vpr = cols / 4;
  const int nvec = rows * vpr;
  if ((base % 4 == 0) && (stride % 4 == 0) && (cols % 4 == 0) && nvec <= NT * MAXV) {
    f32x4 m1[MAXV], v1[MAXV];
    uint32_t am = 0, av = 0;
    GridWalk w(tid, vpr, NT);
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      if (tid + j * NT < nvec) {
        const int64_t e = base + static_cast<int64_t>(w.row) * stride + static_cast<int64_t>(w.col) * 4;
        const f32x4 p = ldg(reinterpret_cast<const f32x4*>(param + e));
        const f32x4 g = ldg(reinterpret_cast<const f32x4*>(grad + e));
        const uint32_t cm = ldg(reinterpret_cast<const uint32_t*>(qm + e));
        const uint32_t cv = ldg(reinterpret_cast<const uint32_t*>(qv + e));
        const f32x4 dm = decode4<FMT_I8, false>(cm), dv = decode4<FMT_U8, false>(cv);
        const float pin[4] = {p.x, p.y, p.z, p.w}, gin[4] = {g.x, g.y, g.z, g.w};
        const float dmi[4] = {dm.x, dm.y, dm.z, dm.w}, dvi[4] = {dv.x, dv.y, dv.z, dv.w};
        float po[4], mo[4], vo[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          adam_elem(pin[h], gin[h], __fmul_rn(dmi[h], sm0), __fmul_rn(dvi[h], sv0), k, po[h], mo[h], vo[h]);
        m1[j] = f32x4{mo[0], mo[1], mo[2], mo[3]};
        v1[j] = f32x4{vo[0], vo[1], vo[2], vo[3]};
        stg(reinterpret_cast<f32x4*>(param + e), f32x4{po[0], po[1], po[2], po[3]});
        am = max(am, max(max(__float_as_uint(m1[j].x) & 0x7fffffffu, __float_as_uint(m1[j].y) & 0x7fffffffu),
                         max(__float_as_uint(m1[j].z) & 0x7fffffffu, __float_as_uint(m1[j].w) & 0x7fffffffu)));
        av = max(av, max(max(__float_as_uint(v1[j].x) & 0x7fffffffu, __float_as_uint(v1[j].y) & 0x7fffffffu),
                         max(__float_as_uint(v1[j].z) & 0x7fffffffu, __float_as_uint(v1[j].w) & 0x7fffffffu)));
      }
      w.next();
    }
    const float amax_m = __uint_as_float(group_max<NT>(am, tid, red));
    const float amax_v = __uint_as_float(group_max<NT>(av, tid, NT > kWave ? red + NT / kWave : nullptr));
    float scm, rm, scv, rv;
    block_scale(amax_m, 127.0f, scm, rm);
    block_scale(amax_v, 255.0f, scv, rv);
    if (tid == 0) {
      sm[sidx] = scm;
      sv[sidx] = scv;
    }
    GridWalk w2(tid, vpr, NT);
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      if (tid + j * NT < nvec) {
        const int64_t e = base + static_cast<int64_t>(w2.row) * stride + static_cast<int64_t>(w2.col) * 4;
        const uint32_t cm = amax_m == 0.0f ? 0u
            : encode4<FMT_I8, false>(__fmul_rn(m1[j].x, rm), __fmul_rn(m1[j].y, rm), __fmul_rn(m1[j].z, rm), __fmul_rn(m1[j].w, rm));
        const uint32_t cv = amax_v == 0.0f ? 0u
            : encode4<FMT_U8, false>(__fmul_rn(v1[j].x, rv), __fmul_rn(v1[j].y, rv), __fmul_rn(v1[j].z, rv), __fmul_rn(v1[j].w, rv));
        stg(reinterpret_cast<uint32_t*>(qm + e), cm);
        stg(reinterpret_cast<uint32_t*>(qv + e), cv);
      }
      w2.next();
    }
    return;
  }
  // general path
  const int64_t total = static_cast<int64_t>(rows) * cols;
  uint32_t am = 0, av = 0;
  for (int64_t i = tid; i < total; i += NT) {
    const int64_t rr = i / cols, cc = i - rr * cols;
    const int64_t e = base + rr * stride + cc;
    float p1, m1, v1;
    adam_elem(param[e], grad[e], __fmul_rn(decode1<FMT_I8, false>(qm[e]), sm0),
              __fmul_rn(decode1<FMT_U8, false>(qv[e]), sv0), k, p1, m1, v1);
    param[e] = p1;
    am = max(am, __float_as_uint(m1) & 0x7fffffffu);
    av = max(av, __float_as_uint(v1) & 0x7fffffffu);
  }
  const float amax_m = __uint_as_float(group_max<NT>(am, tid, red));
  const float amax_v = __uint_as_float(group_max<NT>(av, tid, NT > kWave ? red + NT / kWave : nullptr));
  float scm, rm, scv, rv;
  block_scale(amax_m, 127.0f, scm, rm);
  block_scale(amax_v, 255.0f, scv, rv);
  if (tid == 0) {
    sm[sidx] = scm;
    sv[sidx] = scv;
  }
  for (int64_t i = tid; i < total; i += NT) {
    const int64_t rr = i / cols, cc = i - rr * cols;
    const int64_t e = base + rr * stride + cc;
    float p1, m1, v1;  // m1 and v1 again, from the old codes (p1 is discarded)
    adam_elem(0.0f, grad[e], __fmul_rn(decode1<FMT_I8, false>(qm[e]), sm0),
              __fmul_rn(decode1<FMT_U8, false>(qv[e]), sv0), k, p1, m1, v1);
    qm[e] = amax_m == 0.0f ? 0 : static_cast<uint8_t>(encode1<FMT_I8, false>(__fmul_rn(m1, rm)));
    qv[e] = amax_v == 0.0f ? 0 : static_cast<uint8_t>(encode1<FMT_U8, false>(__fmul_rn(v1, rv)));
  }
}

__device__ __forceinline__ void adam_tile_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs, float* param,
                                                             const float* grad, uint8_t* qm, float* sm,
                                                             uint8_t* qv, float* sv, AdamK k) {
  __shared__ uint32_t red[2 * kThreads / kWave];
  const unsigned b = piece_index<kTileXcdGroup>(jb, n_jobs);
  const QJob j = jobs[b];
  adam_block<kThreads, 4>(param, grad, qm, sm, qv, sv, j.base, j.stride, j.rows, j.cols, j.scale,
                          threadIdx.x, red, k);
}

__global__ __launch_bounds__(kThreads) void adam_tile_kernel(const QJob* __restrict__ jobs, float* param,
                                                             const float* grad, uint8_t* qm, float* sm,
                                                             uint8_t* qv, float* sv, AdamK k, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    adam_tile_kernel_job(jb, n_jobs, jobs, param, grad, qm, sm, qv, sv, k);
    __syncthreads();   // the next job reuses this workgroup's LDS
  }
}

__device__ __forceinline__ void adam_flat_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs, float* param,
                                                             const float* grad, uint8_t* qm, float* sm,
                                                             uint8_t* qv, float* sv, AdamK k) {
  const unsigned b = piece_index<kFlatXcdGroup>(jb, n_jobs);
  const QJob j = jobs[b];
  const int wave = threadIdx.x / kWave;
  if (wave >= j.rows) return;
  const int len = wave == j.rows - 1 ? j.last : j.cols;
  adam_block<kWave, 8>(param, grad, qm, sm, qv, sv, j.base + static_cast<int64_t>(wave) * j.cols, len, 1,
                       len, j.scale + wave, threadIdx.x & (kWave - 1), nullptr, k);
}

__global__ __launch_bounds__(kFlatThreads) void adam_flat_kernel(const QJob* __restrict__ jobs, float* param,
                                                             const float* grad, uint8_t* qm, float* sm,
                                                             uint8_t* qv, float* sv, AdamK k, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    adam_flat_kernel_job(jb, n_jobs, jobs, param, grad, qm, sm, qv, sv, k);
  }
}

// ------------------------------------------------------------------ unpack

// Workgroup b copies piece b % split (kUnpackPiece vectors) of chunk b / split.
__device__ __forceinline__ void unpack_kernel_piece(unsigned b, const CopyChunk* __restrict__ chunks,
                                                               const uint8_t* __restrict__ gathered,
                                                               void* const* __restrict__ dst, int eb,
                                                               int split) {
  const unsigned cu = b / static_cast<unsigned>(split);
  const int ci = static_cast<int>(cu);
  const int piece = static_cast<int>(b - cu * static_cast<unsigned>(split));
  const CopyChunk c = chunks[ci];
  const uint8_t* s = gathered + c.src * eb;
  uint8_t* d = static_cast<uint8_t*>(dst[c.tensor]) + c.off * eb;
  const int nbytes = c.len * eb;
  const int nvec = nbytes >> 4;
  const int v0 = piece * static_cast<int>(kUnpackPiece) + static_cast<int>(threadIdx.x);
  const u32x4* s4 = reinterpret_cast<const u32x4*>(s);
  u32x4* d4 = reinterpret_cast<u32x4*>(d);
  u32x4 r[kUnpackVec];
#pragma unroll
  for (int u = 0; u < kUnpackVec; ++u)
    if (v0 + u * kUnpackThreads < nvec) r[u] = ldg(s4 + v0 + u * kUnpackThreads);
#pragma unroll
  for (int u = 0; u < kUnpackVec; ++u)
    if (v0 + u * kUnpackThreads < nvec) stg(d4 + v0 + u * kUnpackThreads, r[u]);
  const int tail = nbytes & 15;
  if (piece == 0 && static_cast<int>(threadIdx.x) < tail) d[(nvec << 4) + threadIdx.x] = s[(nvec << 4) + threadIdx.x];
}

__global__ __launch_bounds__(kUnpackThreads) void unpack_kernel(const CopyChunk* __restrict__ chunks,
                                                               const uint8_t* __restrict__ gathered,
                                                               void* const* __restrict__ dst, int eb,
                                                               int split, unsigned n_pieces) {
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    unpack_kernel_piece(piece_index<kUnpackXcdGroup>(p, n_pieces), chunks, gathered, dst, eb, split);
}

// ------------------------------------------------------------------ pack

template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* p, int64_t e) {
  if constexpr (BF16) {
    const u32x2 w = ldg(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + e));
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
  } else {
    return ldg(reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + e));
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* p, int64_t e) {
  if constexpr (BF16)
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[e]) << 16);
  else
    return static_cast<const float*>(p)[e];
}

// packed = acc ? prev + src*sigma : src*sigma on tensor data, +0.0 on padding.
// Workgroup b writes piece b % kPackSplit (kPackPiece output vectors) of
// chunk b / kPackSplit. `prev` may alias `out`: every element is read before
// it is written, by the same thread.
template <bool BF16, bool ACC>
__device__ __forceinline__ void pack_kernel_piece(unsigned b, const PackChunk* __restrict__ chunks,
                                                             const void* const* __restrict__ src,
                                                             const float* prev, float* out, float sigma) {
  const unsigned cu = b / static_cast<unsigned>(kPackSplit);
  const int ci = static_cast<int>(cu);
  const int piece = static_cast<int>(b - cu * static_cast<unsigned>(kPackSplit));
  const PackChunk c = chunks[ci];
  f32x4* o4 = reinterpret_cast<f32x4*>(out + c.out);
  const int nv = c.n_total >> 2;
  const int v0 = piece * static_cast<int>(kPackPiece) + static_cast<int>(threadIdx.x);
  if (c.tensor < 0) {
#pragma unroll
    for (int u = 0; u < kPackVec; ++u)
      if (v0 + u * kPackThreads < nv) stg(o4 + v0 + u * kPackThreads, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
    return;
  }
  const void* g = src[c.tensor];
  const int nd = c.n_data;
  const f32x4* p4 = reinterpret_cast<const f32x4*>(prev + c.out);
  f32x4 gv[kPackVec], pv[kPackVec];
#pragma unroll
  for (int u = 0; u < kPackVec; ++u) {
    const int i = v0 + u * kPackThreads;
    if (i < nv && 4 * i + 4 <= nd) {
      gv[u] = load4<BF16>(g, c.off + 4 * i);
      if constexpr (ACC) pv[u] = ldg(p4 + i);
    }
  }
#pragma unroll
  for (int u = 0; u < kPackVec; ++u) {
    const int i = v0 + u * kPackThreads;
    if (i >= nv) continue;
    f32x4 y;
    if (4 * i + 4 <= nd) {
      y.x = __fmul_rn(gv[u].x, sigma);
      y.y = __fmul_rn(gv[u].y, sigma);
      y.z = __fmul_rn(gv[u].z, sigma);
      y.w = __fmul_rn(gv[u].w, sigma);
      if constexpr (ACC) {
        y.x = __fadd_rn(pv[u].x, y.x);
        y.y = __fadd_rn(pv[u].y, y.y);
        y.z = __fadd_rn(pv[u].z, y.z);
        y.w = __fadd_rn(pv[u].w, y.w);
      }
    } else {
      float t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 4 * i + k;
        if (e < nd) {
          float v = __fmul_rn(load1<BF16>(g, c.off + e), sigma);
          if constexpr (ACC) v = __fadd_rn(prev[c.out + e], v);
          t[k] = v;
        } else {
          t[k] = 0.0f;
        }
      }
      y = f32x4{t[0], t[1], t[2], t[3]};
    }
    stg(o4 + i, y);
  }
}

template <bool BF16, bool ACC>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const PackChunk* __restrict__ chunks,
                                                             const void* const* __restrict__ src,
                                                             const float* prev, float* out, float sigma, unsigned n_pieces) {
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    pack_kernel_piece<BF16, ACC>(piece_index<kPackXcdGroup>(p, n_pieces), chunks, src, prev, out, sigma);
}

// ------------------------------------------------------------------ tile-major layout

// Tile-major -> row-major (unpack of a TILEMAJOR tensor), one TmJob per
// workgroup: the job's k runs of h*bc elements (one per tile, contiguous in
// the buffer) are staged in LDS as h rows of k*bc elements, which are then
// written as h contiguous row segments of the tensor. Both global sides move
// long contiguous ranges; the reorder happens in LDS.
template <int EB>
__device__ __forceinline__ void unpack_tm_kernel_job(unsigned jb, unsigned n_jobs, const TmJob* __restrict__ jobs,
                                                             const uint8_t* __restrict__ gathered,
                                                             void* const* __restrict__ dst) {
  extern __shared__ __attribute__((aligned(16))) uint8_t tm_stage_bytes[];   // the plan's largest strip
  uint8_t* stage = tm_stage_bytes;
  const TmJob j = jobs[jb];
  const int bc = j.bc, h = j.h, k = j.k, tid = threadIdx.x;
  const int run = h * bc, width = k * bc;
  const uint8_t* src = gathered + j.base * EB;
  uint8_t* out = static_cast<uint8_t*>(dst[j.tensor]) + j.toff * EB;
  if ((bc * EB) % 16 == 0 && (j.cols * EB) % 16 == 0) {
    constexpr int VE = 16 / EB;
    const int rv = run / VE, total = k * rv;
    for (int v = tid; v < total; v += kTmLdsThreads) {
      const int t = v / rv, e = (v - t * rv) * VE, r = e / bc, c = e - r * bc;
      *reinterpret_cast<u32x4*>(stage + (r * width + t * bc + c) * EB) =
          ldg(reinterpret_cast<const u32x4*>(src + (static_cast<int64_t>(t) * j.tile_elems + e) * EB));
    }
    __syncthreads();
    const int wv = width / VE, total2 = h * wv;
    for (int v = tid; v < total2; v += kTmLdsThreads) {
      const int r = v / wv, w = v - r * wv;
      stg(reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(r) * j.cols + w * VE) * EB),
          *reinterpret_cast<const u32x4*>(stage + (r * width + w * VE) * EB));
    }
    return;
  }
  for (int v = tid; v < k * run; v += kTmLdsThreads) {
    const int t = v / run, e = v - t * run, r = e / bc, c = e - r * bc;
    const uint8_t* from = src + (static_cast<int64_t>(t) * j.tile_elems + e) * EB;
    uint8_t* to = stage + (r * width + t * bc + c) * EB;
    for (int b = 0; b < EB; ++b) to[b] = from[b];
  }
  __syncthreads();
  for (int v = tid; v < h * width; v += kTmLdsThreads) {
    const int r = v / width, w = v - r * width;
    uint8_t* to = out + (static_cast<int64_t>(r) * j.cols + w) * EB;
    const uint8_t* from = stage + v * EB;
    for (int b = 0; b < EB; ++b) to[b] = from[b];
  }
}

template <int EB>
__global__ __launch_bounds__(kTmLdsThreads) void unpack_tm_kernel(const TmJob* __restrict__ jobs,
                                                             const uint8_t* __restrict__ gathered,
                                                             void* const* __restrict__ dst, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    unpack_tm_kernel_job<EB>(jb, n_jobs, jobs, gathered, dst);
    __syncthreads();   // the next job reuses this workgroup's LDS
  }
}

// Row-major -> tile-major with the pack arithmetic (pack of a TILEMAJOR
// tensor): h rows of k*bc gradients are staged in LDS as fp32, then each
// tile's run of h*bc elements is written contiguously as
// [prev +] fl32(g * sigma). `prev` may alias `out` (each element is read and
// written by the same thread).
template <bool BF16, bool ACC>
__device__ __forceinline__ void pack_tm_kernel_job(unsigned jb, unsigned n_jobs, const TmJob* __restrict__ jobs,
                                                           const void* const* __restrict__ src,
                                                           const float* prev, float* out, float sigma) {
  extern __shared__ __attribute__((aligned(16))) float tm_stage_f32[];   // the plan's largest strip
  float* stage = tm_stage_f32;
  const TmJob j = jobs[jb];
  const int bc = j.bc, h = j.h, k = j.k, tid = threadIdx.x;
  const int run = h * bc, width = k * bc;
  const void* g = src[j.tensor];
  if (bc % 4 == 0 && j.cols % 4 == 0) {
    const int wv = width / 4, total = h * wv;
    for (int v = tid; v < total; v += kTmLdsThreads) {
      const int r = v / wv, w = v - r * wv;
      *reinterpret_cast<f32x4*>(stage + r * width + 4 * w) = load4<BF16>(g, j.toff + static_cast<int64_t>(r) * j.cols + 4 * w);
    }
    __syncthreads();
    const int rv = run / 4, total2 = k * rv;
    for (int v = tid; v < total2; v += kTmLdsThreads) {
      const int t = v / rv, e = (v - t * rv) * 4, r = e / bc, c = e - r * bc;
      const int64_t pos = j.base + static_cast<int64_t>(t) * j.tile_elems + e;
      const f32x4 x = *reinterpret_cast<const f32x4*>(stage + r * width + t * bc + c);
      f32x4 y{__fmul_rn(x.x, sigma), __fmul_rn(x.y, sigma), __fmul_rn(x.z, sigma), __fmul_rn(x.w, sigma)};
      if constexpr (ACC) {
        const f32x4 pv = ldg(reinterpret_cast<const f32x4*>(prev + pos));
        y = f32x4{__fadd_rn(pv.x, y.x), __fadd_rn(pv.y, y.y), __fadd_rn(pv.z, y.z), __fadd_rn(pv.w, y.w)};
      }
      stg(reinterpret_cast<f32x4*>(out + pos), y);
    }
    return;
  }
  for (int v = tid; v < h * width; v += kTmLdsThreads) {
    const int r = v / width, w = v - r * width;
    stage[v] = load1<BF16>(g, j.toff + static_cast<int64_t>(r) * j.cols + w);
  }
  __syncthreads();
  for (int v = tid; v < k * run; v += kTmLdsThreads) {
    const int t = v / run, e = v - t * run, r = e / bc, c = e - r * bc;
    const int64_t pos = j.base + static_cast<int64_t>(t) * j.tile_elems + e;
    float y = __fmul_rn(stage[r * width + t * bc + c], sigma);
    if constexpr (ACC) y = __fadd_rn(prev[pos], y);
    out[pos] = y;
  }
}

template <bool BF16, bool ACC>
__global__ __launch_bounds__(kTmLdsThreads) void pack_tm_kernel(const TmJob* __restrict__ jobs,
                                                           const void* const* __restrict__ src,
                                                           const float* prev, float* out, float sigma, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    pack_tm_kernel_job<BF16, ACC>(jb, n_jobs, jobs, src, prev, out, sigma);
    __syncthreads();   // the next job reuses this workgroup's LDS
  }
}

// Direct tile-major reorder, no LDS: workgroup b takes piece b % split of
// strip b / split, kTmThreads vectors (one per thread). Unpack walks the strip
// in row-major order: consecutive lanes write one contiguous row segment and
// read bc-element runs of consecutive tiles (256 bytes for 128 bf16 columns).
// Pack walks it in buffer order: writes and prev reads are contiguous, grad
// reads are bc-element row runs. Strips hold at most kTmStage elements, so
// every index below stays under 2^16 and div_u16 applies.
template <int EB>
__device__ __forceinline__ void unpack_tm_direct_kernel_piece(unsigned b, const TmJob* __restrict__ jobs,
                                                                      const uint8_t* __restrict__ gathered,
                                                                      void* const* __restrict__ dst, int split) {
  constexpr int VE = 16 / EB;   // elements per 16-byte vector
  const unsigned ju = b / static_cast<unsigned>(split);
  const int ji = static_cast<int>(ju);
  const int piece = static_cast<int>(b - ju * static_cast<unsigned>(split));
  const TmJob j = jobs[ji];
  const uint32_t bc = static_cast<uint32_t>(j.bc), width = static_cast<uint32_t>(j.k) * bc;
  const uint32_t mbc = magic_u16(bc);
  const uint8_t* src = gathered + j.base * EB;
  uint8_t* out = static_cast<uint8_t*>(dst[j.tensor]) + j.toff * EB;
  const int stride = split * kTmThreads;
  if (bc % VE == 0 && j.cols % VE == 0) {
    const uint32_t wv = width / VE, mw = magic_u16(wv);
    const int nvec = j.h * static_cast<int>(wv);
    for (int v = piece * kTmThreads + static_cast<int>(threadIdx.x); v < nvec; v += stride) {
      const uint32_t r = div_u16(static_cast<uint32_t>(v), wv, mw);
      const uint32_t col = (static_cast<uint32_t>(v) - r * wv) * VE;
      const uint32_t t = div_u16(col, bc, mbc), c = col - t * bc;
      const u32x4 x = ldg(reinterpret_cast<const u32x4*>(src + (static_cast<int64_t>(t) * j.tile_elems + r * bc + c) * EB));
      stg(reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(r) * j.cols + col) * EB), x);
    }
    return;
  }
  const int n = j.h * static_cast<int>(width);
  const uint32_t mw = magic_u16(width);
  for (int e = piece * kTmThreads + static_cast<int>(threadIdx.x); e < n; e += stride) {
    const uint32_t r = div_u16(static_cast<uint32_t>(e), width, mw);
    const uint32_t col = static_cast<uint32_t>(e) - r * width;
    const uint32_t t = div_u16(col, bc, mbc), c = col - t * bc;
    const uint8_t* from = src + (static_cast<int64_t>(t) * j.tile_elems + r * bc + c) * EB;
    uint8_t* to = out + (static_cast<int64_t>(r) * j.cols + col) * EB;
    for (int b = 0; b < EB; ++b) to[b] = from[b];
  }
}

template <int EB>
__global__ __launch_bounds__(kTmThreads) void unpack_tm_direct_kernel(const TmJob* __restrict__ jobs,
                                                                      const uint8_t* __restrict__ gathered,
                                                                      void* const* __restrict__ dst, int split, unsigned n_pieces) {
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    unpack_tm_direct_kernel_piece<EB>(p, jobs, gathered, dst, split);
}

template <bool BF16, bool ACC>
__device__ __forceinline__ void pack_tm_direct_kernel_piece(unsigned b, const TmJob* __restrict__ jobs,
                                                                    const void* const* __restrict__ src,
                                                                    const float* prev, float* out, float sigma,
                                                                    int split) {
  const unsigned ju = b / static_cast<unsigned>(split);
  const int ji = static_cast<int>(ju);
  const int piece = static_cast<int>(b - ju * static_cast<unsigned>(split));
  const TmJob j = jobs[ji];
  const uint32_t bc = static_cast<uint32_t>(j.bc), run = static_cast<uint32_t>(j.h) * bc;
  const uint32_t mbc = magic_u16(bc);
  const void* g = src[j.tensor];
  const int stride = split * kTmThreads;
  if (bc % 4 == 0 && j.cols % 4 == 0) {
    const uint32_t rv = run / 4, mr = magic_u16(rv);
    const int nvec = j.k * static_cast<int>(rv);
    for (int o = piece * kTmThreads + static_cast<int>(threadIdx.x); o < nvec; o += stride) {
      const uint32_t t = div_u16(static_cast<uint32_t>(o), rv, mr);
      const uint32_t e = (static_cast<uint32_t>(o) - t * rv) * 4;
      const uint32_t r = div_u16(e, bc, mbc), c = e - r * bc;
      const int64_t pos = j.base + static_cast<int64_t>(t) * j.tile_elems + e;
      const f32x4 x = load4<BF16>(g, j.toff + static_cast<int64_t>(r) * j.cols + t * bc + c);
      f32x4 y{__fmul_rn(x.x, sigma), __fmul_rn(x.y, sigma), __fmul_rn(x.z, sigma), __fmul_rn(x.w, sigma)};
      if constexpr (ACC) {
        const f32x4 pv = ldg(reinterpret_cast<const f32x4*>(prev + pos));
        y = f32x4{__fadd_rn(pv.x, y.x), __fadd_rn(pv.y, y.y), __fadd_rn(pv.z, y.z), __fadd_rn(pv.w, y.w)};
      }
      stg(reinterpret_cast<f32x4*>(out + pos), y);
    }
    return;
  }
  const int n = j.k * static_cast<int>(run);
  const uint32_t mr = magic_u16(run);
  for (int o = piece * kTmThreads + static_cast<int>(threadIdx.x); o < n; o += stride) {
    const uint32_t t = div_u16(static_cast<uint32_t>(o), run, mr);
    const uint32_t e = static_cast<uint32_t>(o) - t * run;
    const uint32_t r = div_u16(e, bc, mbc), c = e - r * bc;
    const int64_t pos = j.base + static_cast<int64_t>(t) * j.tile_elems + e;
    float y = __fmul_rn(load1<BF16>(g, j.toff + static_cast<int64_t>(r) * j.cols + t * bc + c), sigma);
    if constexpr (ACC) y = __fadd_rn(prev[pos], y);
    out[pos] = y;
  }
}

template <bool BF16, bool ACC>
__global__ __launch_bounds__(kTmThreads) void pack_tm_direct_kernel(const TmJob* __restrict__ jobs,
                                                                    const void* const* __restrict__ src,
                                                                    const float* prev, float* out, float sigma,
                                                                    int split, unsigned n_pieces) {
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    pack_tm_direct_kernel_piece<BF16, ACC>(p, jobs, src, prev, out, sigma, split);
}

// Gather side of a tile-major tensor, over the same strips: each lane turns
// VEC codes of one tile row into one 16-byte store of the row-major tensor
// (8 codes -> 8 bf16, 4 -> 4 fp32), kGatherVec vectors per thread; tile t of
// the strip uses scale scale0 + t.
template <int FMT, bool HW, bool BF16OUT>
__device__ __forceinline__ void gather_tm_kernel_piece(unsigned b, const TmJob* __restrict__ jobs,
                                                                  const uint8_t* __restrict__ q,
                                                                  const float* __restrict__ scales,
                                                                  void* const* __restrict__ dst, int split) {
  constexpr int VEC = BF16OUT ? 8 : 4;
  constexpr int U = kGatherVec;
  const unsigned ju = b / static_cast<unsigned>(split);
  const int ji = static_cast<int>(ju);
  const int piece = static_cast<int>(b - ju * static_cast<unsigned>(split));
  const TmJob j = jobs[ji];
  const uint32_t bc = static_cast<uint32_t>(j.bc), width = static_cast<uint32_t>(j.k) * bc;
  const uint32_t mbc = magic_u16(bc);
  const uint8_t* qb = q + j.base;
  void* out = dst[j.tensor];
  const int pass = split * static_cast<int>(kGatherPiece);
  if (bc % VEC == 0 && j.cols % VEC == 0) {
    const uint32_t wv = width / VEC, mw = magic_u16(wv);
    const int nvec = j.h * static_cast<int>(wv);
    for (int i0 = piece * static_cast<int>(kGatherPiece) + static_cast<int>(threadIdx.x); i0 < nvec; i0 += pass) {
      uint32_t code[U][VEC / 4];
      float sc[U];
      int64_t dpos[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kGatherThreads;
        if (i < nvec) {
          const uint32_t r = div_u16(static_cast<uint32_t>(i), wv, mw);
          const uint32_t col = (static_cast<uint32_t>(i) - r * wv) * VEC;
          const uint32_t t = div_u16(col, bc, mbc), c = col - t * bc;
          const uint8_t* from = qb + static_cast<int64_t>(t) * j.tile_elems + r * bc + c;
          if constexpr (VEC == 8) {
            const u32x2 w = ldg(reinterpret_cast<const u32x2*>(from));
            code[u][0] = w.x;
            code[u][1] = w.y;
          } else {
            code[u][0] = ldg(reinterpret_cast<const uint32_t*>(from));
          }
          sc[u] = scales[j.scale0 + t];
          dpos[u] = j.toff + static_cast<int64_t>(r) * j.cols + col;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i0 + u * kGatherThreads >= nvec) continue;
        float v[VEC];
#pragma unroll
        for (int h = 0; h < VEC / 4; ++h) {
          const f32x4 d = decode4<FMT, HW>(code[u][h]);
          v[4 * h] = __fmul_rn(d.x, sc[u]);
          v[4 * h + 1] = __fmul_rn(d.y, sc[u]);
          v[4 * h + 2] = __fmul_rn(d.z, sc[u]);
          v[4 * h + 3] = __fmul_rn(d.w, sc[u]);
        }
        if constexpr (BF16OUT) {
          stg(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + dpos[u]),
              u32x4{bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16),
                    bf16_rne(v[4]) | (bf16_rne(v[5]) << 16), bf16_rne(v[6]) | (bf16_rne(v[7]) << 16)});
        } else {
          stg(reinterpret_cast<f32x4*>(static_cast<float*>(out) + dpos[u]), f32x4{v[0], v[1], v[2], v[3]});
        }
      }
    }
    return;
  }
  // element path: a piece is kGatherPiece elements, U per thread
  const int n = j.h * static_cast<int>(width);
  const uint32_t mw = magic_u16(width);
  for (int e0 = piece * static_cast<int>(kGatherPiece) + static_cast<int>(threadIdx.x); e0 < n; e0 += pass) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * kGatherThreads;
      if (e >= n) break;
      const uint32_t r = div_u16(static_cast<uint32_t>(e), width, mw);
      const uint32_t col = static_cast<uint32_t>(e) - r * width;
      const uint32_t t = div_u16(col, bc, mbc), c = col - t * bc;
      const float v = __fmul_rn(decode1<FMT, HW>(qb[static_cast<int64_t>(t) * j.tile_elems + r * bc + c]),
                                scales[j.scale0 + t]);
      const int64_t d = j.toff + static_cast<int64_t>(r) * j.cols + col;
      if constexpr (BF16OUT)
        static_cast<uint16_t*>(out)[d] = static_cast<uint16_t>(bf16_rne(v));
      else
        static_cast<float*>(out)[d] = v;
    }
  }
}

template <int FMT, bool HW, bool BF16OUT>
__global__ __launch_bounds__(kGatherThreads) void gather_tm_kernel(const TmJob* __restrict__ jobs,
                                                                  const uint8_t* __restrict__ q,
                                                                  const float* __restrict__ scales,
                                                                  void* const* __restrict__ dst, int split, unsigned n_pieces) {
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    gather_tm_kernel_piece<FMT, HW, BF16OUT>(p, jobs, q, scales, dst, split);
}

// ------------------------------------------------------------------ host side

// Grid of a launch: one workgroup per work item up to the plan's max_grid
// (kMaxGrid unless RS_MAX_GRID lowers it), beyond which every workgroup loops
// over items p, p + grid, ... (max_grid is a multiple of 8, so item p still
// runs on XCD p % 8).
dim3 grid_of(const rs_plan* p, int64_t n_items) {
  return dim3(static_cast<unsigned>(std::min<int64_t>(n_items, p->max_grid)));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_call(const rs_plan* p, const char* who) {
  if (!p) return fail(RS_EINVAL, std::string(who) + ": null plan");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return fail(RS_EHIP, std::string(who) + ": hipGetDevice failed");
  if (cur != p->device)
    return fail(RS_EINVAL, std::string(who) + ": current device " + std::to_string(cur) +
                               " differs from the plan's device " + std::to_string(p->device));
  return RS_OK;
}

int launched(const char* who) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RS_EHIP, std::string(who) + ": launch failed: " + hipGetErrorString(e));
  return RS_OK;
}

// Upload a per-tensor pointer table on `stream` if it differs from the last one.
int sync_table(rs_plan* p, PtrTable* tab, const void* const* ptrs, hipStream_t stream, const char* who) {
  const size_t bytes = sizeof(void*) * static_cast<size_t>(p->n);
  if (tab->valid && std::memcmp(tab->seen.data(), ptrs, bytes) == 0) return RS_OK;
  if (tab->pending && hipEventSynchronize(tab->done) != hipSuccess)
    return fail(RS_EHIP, std::string(who) + ": waiting for the previous table upload failed");
  std::memcpy(tab->stage, ptrs, bytes);
  if (hipMemcpyAsync(tab->dev, tab->stage, bytes, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(tab->done, stream) != hipSuccess) {
    tab->valid = false;
    return fail(RS_EHIP, std::string(who) + ": pointer table upload failed");
  }
  tab->pending = true;
  std::memcpy(tab->seen.data(), ptrs, bytes);
  tab->valid = true;
  return RS_OK;
}

int elem_bytes(int32_t dt) {
  switch (dt) {
    case RS_F32: return 4;
    case RS_BF16: return 2;
    case RS_E4M3: case RS_I8: case RS_U8: return 1;
    default: return 0;
  }
}

}  // namespace
}  // namespace rs

using namespace rs;

extern "C" int rs_unpack_gathered(rs_plan* p, const void* gathered, int32_t dt, void* const* dst,
                                  void* stream) {
  const char* who = "rs_unpack_gathered";
  clear_error();
  int st = check_call(p, who);
  if (st != RS_OK) return st;
  const int eb = elem_bytes(dt);
  if (eb == 0) return fail(RS_EDTYPE, std::string(who) + ": unknown dtype");
  if (!gathered || !dst) return fail(RS_EINVAL, std::string(who) + ": null buffer");
  if (!aligned16(gathered)) return fail(RS_EALIGN, std::string(who) + ": gathered buffer not 16-byte aligned");
  for (int64_t i = 0; i < p->n; ++i) {
    if (!dst[i]) return fail(RS_EINVAL, std::string(who) + ": null destination " + std::to_string(i));
    if (!aligned16(dst[i])) return fail(RS_EALIGN, std::string(who) + ": destination " + std::to_string(i) + " not 16-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = sync_table(p, &p->dst, dst, s, who);
  if (st != RS_OK) return st;
  const uint8_t* gb = static_cast<const uint8_t*>(gathered);
  if (p->n_unpack) {
    const int64_t split = unpack_split(eb);
    const int64_t n = p->n_unpack * split;
    hipLaunchKernelGGL(unpack_kernel, grid_of(p, n), dim3(kUnpackThreads), 0, s, p->unpack, gb, p->dst.dev, eb,
                       static_cast<int>(split), static_cast<unsigned>(n));
  }
  if (p->n_tm && !p->tm_unpack_lds) {
    const int64_t split = tm_pieces(p->tm_max_strip, 16 / eb, kTmThreads);
    const int64_t n = p->n_tm * split;
    const dim3 g = grid_of(p, n), b(kTmThreads);
    const int sp = static_cast<int>(split);
    const unsigned np = static_cast<unsigned>(n);
    if (eb == 4) hipLaunchKernelGGL(unpack_tm_direct_kernel<4>, g, b, 0, s, p->tmjobs, gb, p->dst.dev, sp, np);
    else if (eb == 2) hipLaunchKernelGGL(unpack_tm_direct_kernel<2>, g, b, 0, s, p->tmjobs, gb, p->dst.dev, sp, np);
    else hipLaunchKernelGGL(unpack_tm_direct_kernel<1>, g, b, 0, s, p->tmjobs, gb, p->dst.dev, sp, np);
  } else if (p->n_tm) {
    const dim3 g = grid_of(p, p->n_tm);
    const unsigned nj = static_cast<unsigned>(p->n_tm);
    const unsigned lds = static_cast<unsigned>(p->tm_max_strip * eb);
    if (eb == 4) hipLaunchKernelGGL(unpack_tm_kernel<4>, g, dim3(kTmLdsThreads), lds, s, p->tmjobs, gb, p->dst.dev, nj);
    else if (eb == 2) hipLaunchKernelGGL(unpack_tm_kernel<2>, g, dim3(kTmLdsThreads), lds, s, p->tmjobs, gb, p->dst.dev, nj);
    else hipLaunchKernelGGL(unpack_tm_kernel<1>, g, dim3(kTmLdsThreads), lds, s, p->tmjobs, gb, p->dst.dev, nj);
  }
  return launched(who);
}

extern "C" int rs_pack_scatter(rs_plan* p, const void* const* src, int32_t src_dt, const float* prev,
                               float* packed, int32_t scale_mode, float scale, void* stream) {
  const char* who = "rs_pack_scatter";
  clear_error();
  int st = check_call(p, who);
  if (st != RS_OK) return st;
  if (src_dt != RS_F32 && src_dt != RS_BF16) return fail(RS_EDTYPE, std::string(who) + ": src must be fp32 or bf16");
  if (!src || !packed) return fail(RS_EINVAL, std::string(who) + ": null buffer");
  if (!aligned16(packed) || (prev && !aligned16(prev)))
    return fail(RS_EALIGN, std::string(who) + ": packed / prev not 16-byte aligned");
  for (int64_t i = 0; i < p->n; ++i) {
    if (!src[i]) return fail(RS_EINVAL, std::string(who) + ": null source " + std::to_string(i));
    if (!aligned16(src[i])) return fail(RS_EALIGN, std::string(who) + ": source " + std::to_string(i) + " not 16-byte aligned");
  }
  float sigma;
  if (scale_mode == RS_SCALE_INV_V)
    sigma = 1.0f / static_cast<float>(p->V);   // IEEE fp32 division on the host: fl32(1/V) for V < 2^24
  else if (scale_mode == RS_SCALE_GIVEN)
    sigma = scale;
  else
    return fail(RS_EINVAL, std::string(who) + ": unknown scale mode");
  if (scale_mode == RS_SCALE_INV_V && p->V >= (int64_t(1) << 24))
    return fail(RS_ERANGE, std::string(who) + ": V too large for an exact fp32 1/V");
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = sync_table(p, &p->src, src, s, who);
  if (st != RS_OK) return st;
  const int64_t n_pieces = p->n_pack * kPackSplit;
  const unsigned np = static_cast<unsigned>(n_pieces);
  const dim3 grid = grid_of(p, n_pieces), sblock(kPackThreads);
  void** tab = p->src.dev;
  if (p->n_pack) {
    if (src_dt == RS_F32) {
      if (prev) hipLaunchKernelGGL((pack_kernel<false, true>), grid, sblock, 0, s, p->pack, tab, prev, packed, sigma, np);
      else hipLaunchKernelGGL((pack_kernel<false, false>), grid, sblock, 0, s, p->pack, tab, prev, packed, sigma, np);
    } else {
      if (prev) hipLaunchKernelGGL((pack_kernel<true, true>), grid, sblock, 0, s, p->pack, tab, prev, packed, sigma, np);
      else hipLaunchKernelGGL((pack_kernel<true, false>), grid, sblock, 0, s, p->pack, tab, prev, packed, sigma, np);
    }
  }
  if (p->n_tm && !p->tm_pack_lds) {
    const int64_t split = tm_pieces(p->tm_max_strip, 4, kTmThreads);
    const int64_t n = p->n_tm * split;
    const dim3 g = grid_of(p, n), b(kTmThreads);
    const int sp = static_cast<int>(split);
    const unsigned ntp = static_cast<unsigned>(n);
    if (src_dt == RS_F32) {
      if (prev) hipLaunchKernelGGL((pack_tm_direct_kernel<false, true>), g, b, 0, s, p->tmjobs, tab, prev, packed, sigma, sp, ntp);
      else hipLaunchKernelGGL((pack_tm_direct_kernel<false, false>), g, b, 0, s, p->tmjobs, tab, prev, packed, sigma, sp, ntp);
    } else {
      if (prev) hipLaunchKernelGGL((pack_tm_direct_kernel<true, true>), g, b, 0, s, p->tmjobs, tab, prev, packed, sigma, sp, ntp);
      else hipLaunchKernelGGL((pack_tm_direct_kernel<true, false>), g, b, 0, s, p->tmjobs, tab, prev, packed, sigma, sp, ntp);
    }
  } else if (p->n_tm) {
    const dim3 g = grid_of(p, p->n_tm);
    const unsigned nj = static_cast<unsigned>(p->n_tm);
    const unsigned lds = static_cast<unsigned>(p->tm_max_strip * 4);
    if (src_dt == RS_F32) {
      if (prev) hipLaunchKernelGGL((pack_tm_kernel<false, true>), g, dim3(kTmLdsThreads), lds, s, p->tmjobs, tab, prev, packed, sigma, nj);
      else hipLaunchKernelGGL((pack_tm_kernel<false, false>), g, dim3(kTmLdsThreads), lds, s, p->tmjobs, tab, prev, packed, sigma, nj);
    } else {
      if (prev) hipLaunchKernelGGL((pack_tm_kernel<true, true>), g, dim3(kTmLdsThreads), lds, s, p->tmjobs, tab, prev, packed, sigma, nj);
      else hipLaunchKernelGGL((pack_tm_kernel<true, false>), g, dim3(kTmLdsThreads), lds, s, p->tmjobs, tab, prev, packed, sigma, nj);
    }
  }
  return launched(who);
}

namespace {

// The zero-range jobs follow the flat groups, which follow the tiles: they ride
// at the end of the last launch that has blocks, or get their own launch.
template <bool BF16, int FMT, bool HW>
void launch_quant_kinds(const rs_plan* p, const void* src, uint8_t* q, float* scales, hipStream_t s) {
  const dim3 block(kThreads);
  const QJob* tiles = p->qjobs;
  const QJob* flats = tiles + p->n_qtile;
  const int64_t nz = p->n_qzero;
  if (p->n_qtile) {
    const int64_t n = p->n_qtile + (p->n_qflat ? 0 : nz);
    hipLaunchKernelGGL((quant_tile_kernel<BF16, FMT, HW>), grid_of(p, n), dim3(kQuantThreads), 0, s, tiles,
                       p->n_qtile, src, q, scales, static_cast<unsigned>(n));
  }
  if (p->n_qflat)
    hipLaunchKernelGGL((quant_flat_kernel<BF16, FMT, HW>), grid_of(p, p->n_qflat + nz), dim3(kFlatThreads), 0, s, flats,
                       p->n_qflat, src, q, scales, static_cast<unsigned>(p->n_qflat + nz));
  if (!p->n_qtile && !p->n_qflat && nz)
    hipLaunchKernelGGL(zero_codes_kernel, grid_of(p, nz), block, 0, s, flats, q, static_cast<unsigned>(nz));
}

template <bool BF16>
void launch_quant(const rs_plan* p, const void* src, int fmt, bool hw, uint8_t* q, float* scales,
                  hipStream_t s) {
  if (fmt == FMT_E4M3 && hw)
    launch_quant_kinds<BF16, FMT_E4M3, true>(p, src, q, scales, s);
  else if (fmt == FMT_E4M3)
    launch_quant_kinds<BF16, FMT_E4M3, false>(p, src, q, scales, s);
  else if (fmt == FMT_I8)
    launch_quant_kinds<BF16, FMT_I8, false>(p, src, q, scales, s);
  else
    launch_quant_kinds<BF16, FMT_U8, false>(p, src, q, scales, s);
}

template <int FMT, bool HW>
void launch_dequant(const rs_plan* p, const uint8_t* q, const float* scales, float* out, hipStream_t s) {
  const dim3 block(kThreads);
  const QJob* tiles = p->qjobs;
  const QJob* flats = tiles + p->n_qtile;
  const int64_t nz = p->n_qzero;
  if (p->n_qtile) {
    const int64_t n = p->n_qtile + (p->n_qflat ? 0 : nz);
    hipLaunchKernelGGL((dequant_tile_kernel<FMT, HW>), grid_of(p, n), block, 0, s, tiles, p->n_qtile, q, scales, out,
                       static_cast<unsigned>(n));
  }
  if (p->n_qflat)
    hipLaunchKernelGGL((dequant_flat_kernel<FMT, HW>), grid_of(p, p->n_qflat + nz), dim3(kFlatThreads), 0, s, flats,
                       p->n_qflat, q, scales, out, static_cast<unsigned>(p->n_qflat + nz));
  if (!p->n_qtile && !p->n_qflat && nz)
    hipLaunchKernelGGL(zero_values_kernel, grid_of(p, nz), block, 0, s, flats, out, static_cast<unsigned>(nz));
}

int fmt_of(int32_t q_dt) {
  switch (q_dt) {
    case RS_E4M3: return FMT_E4M3;
    case RS_I8: return FMT_I8;
    case RS_U8: return FMT_U8;
    default: return -1;
  }
}

}  // namespace

extern "C" int rs_block_quant(rs_plan* p, const void* src, int32_t src_dt, void* q, int32_t q_dt,
                              float* scales, void* stream) {
  const char* who = "rs_block_quant";
  clear_error();
  int st = check_call(p, who);
  if (st != RS_OK) return st;
  if (src_dt != RS_F32 && src_dt != RS_BF16) return fail(RS_EDTYPE, std::string(who) + ": src must be fp32 or bf16");
  const int fmt = fmt_of(q_dt);
  if (fmt < 0) return fail(RS_EDTYPE, std::string(who) + ": code format must be E4M3, I8 or U8");
  if (!src || !q || (!scales && p->n_qblocks > 0)) return fail(RS_EINVAL, std::string(who) + ": null buffer");
  if (!aligned16(src) || !aligned16(q)) return fail(RS_EALIGN, std::string(who) + ": src / q not 16-byte aligned");
  if (p->n_qjobs == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (src_dt == RS_BF16)
    launch_quant<true>(p, src, fmt, p->e4m3_hw, static_cast<uint8_t*>(q), scales, s);
  else
    launch_quant<false>(p, src, fmt, p->e4m3_hw, static_cast<uint8_t*>(q), scales, s);
  return launched(who);
}

extern "C" int rs_block_dequant(rs_plan* p, const void* q, int32_t q_dt, const float* scales,
                                float* out, void* stream) {
  const char* who = "rs_block_dequant";
  clear_error();
  int st = check_call(p, who);
  if (st != RS_OK) return st;
  const int fmt = fmt_of(q_dt);
  if (fmt < 0) return fail(RS_EDTYPE, std::string(who) + ": code format must be E4M3, I8 or U8");
  if (!q || !out || (!scales && p->n_qblocks > 0)) return fail(RS_EINVAL, std::string(who) + ": null buffer");
  if (!aligned16(q) || !aligned16(out)) return fail(RS_EALIGN, std::string(who) + ": q / out not 16-byte aligned");
  if (p->n_qjobs == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  if (fmt == FMT_E4M3 && p->e4m3_hw)
    launch_dequant<FMT_E4M3, true>(p, qb, scales, out, s);
  else if (fmt == FMT_E4M3)
    launch_dequant<FMT_E4M3, false>(p, qb, scales, out, s);
  else if (fmt == FMT_I8)
    launch_dequant<FMT_I8, false>(p, qb, scales, out, s);
  else
    launch_dequant<FMT_U8, false>(p, qb, scales, out, s);
  return launched(who);
}

namespace {

template <int FMT, bool HW, bool BF16OUT>
void launch_gather(const rs_plan* p, const uint8_t* q, const float* scales, hipStream_t s) {
  const dim3 block(kThreads);
  const QJob* tiles = p->gjobs;
  const QJob* flats = tiles + p->n_gtile;
  if (p->n_gchunks) {
    const int64_t split = gather_split(BF16OUT ? 8 : 4);
    const int64_t n = p->n_gchunks * split;
    hipLaunchKernelGGL((gather_rows_kernel<FMT, HW, BF16OUT>), grid_of(p, n), dim3(kGatherThreads), 0, s, p->gchunks, q,
                       scales, p->gdst.dev, static_cast<int>(split), static_cast<unsigned>(n));
  }
  if (p->n_gtile)
    hipLaunchKernelGGL((gather_tile_kernel<FMT, HW, BF16OUT>), grid_of(p, p->n_gtile), block, 0, s, tiles, q, scales,
                       p->gdst.dev, static_cast<unsigned>(p->n_gtile));
  if (p->n_gflat)
    hipLaunchKernelGGL((gather_flat_kernel<FMT, HW, BF16OUT>), grid_of(p, p->n_gflat), dim3(kFlatThreads), 0, s, flats, q,
                       scales, p->gdst.dev, static_cast<unsigned>(p->n_gflat));
  if (p->n_tm) {
    const int64_t split = tm_pieces(p->tm_max_strip, BF16OUT ? 8 : 4, kGatherPiece);
    const int64_t n = p->n_tm * split;
    hipLaunchKernelGGL((gather_tm_kernel<FMT, HW, BF16OUT>), grid_of(p, n), dim3(kGatherThreads), 0, s, p->tmjobs, q,
                       scales, p->gdst.dev, static_cast<int>(split), static_cast<unsigned>(n));
  }
}

template <bool BF16OUT>
void launch_gather_fmt(const rs_plan* p, int fmt, const uint8_t* q, const float* scales, hipStream_t s) {
  if (fmt == FMT_E4M3 && p->e4m3_hw)
    launch_gather<FMT_E4M3, true, BF16OUT>(p, q, scales, s);
  else if (fmt == FMT_E4M3)
    launch_gather<FMT_E4M3, false, BF16OUT>(p, q, scales, s);
  else if (fmt == FMT_I8)
    launch_gather<FMT_I8, false, BF16OUT>(p, q, scales, s);
  else
    launch_gather<FMT_U8, false, BF16OUT>(p, q, scales, s);
}

}  // namespace

extern "C" int rs_unpack_dequant(rs_plan* p, const void* q, int32_t q_dt, const float* scales,
                                 void* const* dst, int32_t dst_dt, void* stream) {
  const char* who = "rs_unpack_dequant";
  clear_error();
  int st = check_call(p, who);
  if (st != RS_OK) return st;
  const int fmt = fmt_of(q_dt);
  if (fmt < 0) return fail(RS_EDTYPE, std::string(who) + ": code format must be E4M3, I8 or U8");
  if (dst_dt != RS_F32 && dst_dt != RS_BF16) return fail(RS_EDTYPE, std::string(who) + ": dst must be fp32 or bf16");
  if (!q || !dst || (!scales && p->n_qblocks > 0)) return fail(RS_EINVAL, std::string(who) + ": null buffer");
  if (!aligned16(q)) return fail(RS_EALIGN, std::string(who) + ": q not 16-byte aligned");
  for (int64_t i = 0; i < p->n; ++i) {
    if (p->t[i].kind != RS_TILE && p->t[i].kind != RS_FLAT && p->t[i].kind != RS_TILEMAJOR) continue;
    if (!dst[i]) return fail(RS_EINVAL, std::string(who) + ": null destination " + std::to_string(i));
    if (!aligned16(dst[i])) return fail(RS_EALIGN, std::string(who) + ": destination " + std::to_string(i) + " not 16-byte aligned");
  }
  if (p->n_gchunks + p->n_gtile + p->n_gflat + p->n_tm == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = sync_table(p, &p->gdst, dst, s, who);
  if (st != RS_OK) return st;
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  if (dst_dt == RS_BF16)
    launch_gather_fmt<true>(p, fmt, qb, scales, s);
  else
    launch_gather_fmt<false>(p, fmt, qb, scales, s);
  return launched(who);
}

extern "C" int rs_adam8_step(rs_plan* p, float* param, const float* grad, void* q_m, float* s_m,
                             void* q_v, float* s_v, const rs_adam_hparams* hp, void* stream) {
  const char* who = "rs_adam8_step";
  clear_error();
  int st = check_call(p, who);
  if (st != RS_OK) return st;
  if (!param || !grad || !q_m || !q_v || !hp || (p->n_qblocks > 0 && (!s_m || !s_v)))
    return fail(RS_EINVAL, std::string(who) + ": null argument");
  if (hp->step < 1 || !(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f) ||
      !(hp->eps >= 0.0f) || !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay) || hp->reserved != 0)
    return fail(RS_EINVAL, std::string(who) + ": bad hyper-parameters");
  if (!aligned16(param) || !aligned16(grad) || !aligned16(q_m) || !aligned16(q_v))
    return fail(RS_EALIGN, std::string(who) + ": buffers must be 16-byte aligned");
  const double b1 = hp->beta1, b2 = hp->beta2, lr = hp->lr, wd = hp->weight_decay;
  const double t = static_cast<double>(hp->step);
  AdamK k;
  k.b1 = hp->beta1;
  k.b2 = hp->beta2;
  k.eps = hp->eps;
  k.c1 = static_cast<float>(1.0 - b1);
  k.c2 = static_cast<float>(1.0 - b2);
  k.step_size = static_cast<float>(lr / (1.0 - std::pow(b1, t)));
  k.inv_bc2_sqrt = static_cast<float>(1.0 / std::sqrt(1.0 - std::pow(b2, t)));
  k.decay = static_cast<float>(1.0 - lr * wd);
  if (p->n_qtile + p->n_qflat == 0) return RS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* qmb = static_cast<uint8_t*>(q_m);
  uint8_t* qvb = static_cast<uint8_t*>(q_v);
  if (p->n_qtile)
    hipLaunchKernelGGL(adam_tile_kernel, grid_of(p, p->n_qtile), dim3(kThreads), 0, s, p->qjobs, param, grad, qmb, s_m,
                       qvb, s_v, k, static_cast<unsigned>(p->n_qtile));
  if (p->n_qflat)
    hipLaunchKernelGGL(adam_flat_kernel, grid_of(p, p->n_qflat), dim3(kFlatThreads), 0, s, p->qjobs + p->n_qtile, param,
                       grad, qmb, s_m, qvb, s_v, k, static_cast<unsigned>(p->n_qflat));
  return launched(who);
}
