// Block quantisation and dequantisation of the flat buffer on gfx950: kernels
// and the rs_block_quant / rs_block_dequant entry points.
//
// Every locally whole block (a tile, or a flat block) is quantised by its own
// absmax: scale = fl32(amax / Q), codes of fl32(x * fl32(Q / amax))
// ("veScale-FSDP: flexible, structure-aware sharding at 10K-GPU scale",
// feynmanwiki walkthrough, the block-quantisation and 8-bit Adam paragraphs).
// A tile stays in the registers of one 512-thread workgroup, a flat block in
// those of one 128-thread workgroup (quant) or one wave (dequant), so each
// input byte is read once; the absmax is a wave shuffle
// reduction plus, across the waves of a workgroup, an LDS combine.
#include "host_common.h"

#include <cstdlib>
#include <mutex>
#include <vector>

// Work-list memory of rs_block_quant_noalloc, for callers that cannot
// allocate: a static device array, so the library never allocates for that
// call. Each GPU the library runs on holds its own copy at its own address
// until the process ends. In host code the array's name is only a host-side
// stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr int64_t kNoallocScratchBytes = int64_t(16) << 20;   // 262,144 work items of 64 bytes
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace rs {
namespace {

// ------------------------------------------------------------------ quant

// One quantisation block: element (r, c) at base + r*stride + c, r < rows,
// c < cols, handled by NT threads (tid in [0, NT)). Fast path: every vector
// of the block stays in registers (at most NT*MAXV 16-byte vectors, rows and
// base aligned to a vector). Otherwise: two passes over memory, element by
// element.
// BATCH: every load of the block is issued before the first is used (loads past
// the block read its first vector and count as zero); otherwise each vector's
// absmax is taken as it arrives, which keeps one load per lane in flight.
// Measured on gfx950 (interleaved, cold): issuing them all lifts the flat
// blocks (5.81 -> 6.05 TB/s) and the MoE layer's 2880-wide tiles (5.69 ->
// 5.81), and costs the 8B layer's tiles 2% (6.07 -> 5.96), which therefore
// keep the one-at-a-time order.
// SC: the codes' store policy. nt-sc1 stores quantise the 8B layer's tiles 1%
// and flat blocks 2% faster cold than nontemporal ones, but tiles that share
// lines of codes with their neighbours (the MoE layer's 2880-wide tensors) 1%
// slower, so those keep nontemporal stores.
template <bool BF16, int FMT, bool HW, int NT, int MAXV, bool BATCH, int SC>
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
    if constexpr (BATCH) {
      GridWalk w(tid, vpr, NT);
#pragma unroll
      for (int k = 0; k < MAXV; ++k) {
        const bool valid = tid + k * NT < nvec;
        const int64_t e = valid ? base + static_cast<int64_t>(w.row) * stride + static_cast<int64_t>(w.col) * VE : base;
        raw[k] = ldg(reinterpret_cast<const u32x4*>(sb + e * I::EB));
        w.next();
      }
#pragma unroll
      for (int k = 0; k < MAXV; ++k)
        if (tid + k * NT < nvec) m = max(m, I::absmax(raw[k]));
    } else {
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
    float sc, r;
    block_scale(amax, Q, sc, r);
    const bool blank = r == 0.0f;   // a zero or non-finite block: every code 0x00
    if (tid == 0) scales[sidx] = sc;
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
          words[h] = blank ? 0u
                          : encode4<FMT, HW>(__fmul_rn(x[4 * h], r), __fmul_rn(x[4 * h + 1], r),
                                             __fmul_rn(x[4 * h + 2], r), __fmul_rn(x[4 * h + 3], r));
        }
        if constexpr (VE == 8) {
          sts<SC>(reinterpret_cast<u32x2*>(q + e), u32x2{words[0], words[1]});
        } else {
          sts<SC>(reinterpret_cast<uint32_t*>(q + e), words[0]);
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
  float sc, r;
  block_scale(amax, Q, sc, r);
  const bool blank = r == 0.0f;
  if (tid == 0) scales[sidx] = sc;
  for (int64_t i = tid; i < total; i += NT) {
    const int64_t rr = i / cols, cc = i - rr * cols;
    const int64_t e = base + rr * stride + cc;
    q[e] = blank ? 0 : static_cast<uint8_t>(encode1<FMT, HW>(__fmul_rn(I::elem(src, e), r)));
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
  for (int64_t i = tid; i < nv; i += NT) sts<kStoreNtSc1>(v + i, u32x4{0u, 0u, 0u, 0u});
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
template <bool BF16, int FMT, bool HW, unsigned XG>
__device__ __forceinline__ void quant_tile_kernel_job(unsigned jb, unsigned n_jobs, const QJob* __restrict__ jobs, int64_t n_main,
                                                                   const void* __restrict__ src,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ scales) {
  __shared__ uint32_t red[kQuantThreads / kWave];
  const unsigned b = piece_index<XG>(jb, n_jobs);
  const QJob j = jobs[b];
  if (static_cast<int64_t>(b) >= n_main) {
    zero_bytes<kQuantThreads>(q, j.base, j.stride, threadIdx.x);
    return;
  }
  quant_block<BF16, FMT, HW, kQuantThreads, (BF16 ? 2048 : 4096) / kQuantThreads, XG == kTileXcdGroupSplit,
              XG == kTileXcdGroupSplit ? kStoreNT : kStoreNtSc1>(
      src, q, scales, j.base, j.stride, j.rows, j.cols, j.scale, threadIdx.x, red);
}

template <bool BF16, int FMT, bool HW, unsigned XG>
__global__ __launch_bounds__(kQuantThreads) void quant_tile_kernel(const QJob* __restrict__ jobs, int64_t n_main,
                                                                   const void* __restrict__ src,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ scales, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    quant_tile_kernel_job<BF16, FMT, HW, XG>(jb, n_jobs, jobs, n_main, src, q, scales);
    __syncthreads();   // the next job reuses this workgroup's LDS
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

// Up to NT*MAXV code words are all loaded before the first is decoded (past
// the block: its first word, unused); larger blocks loop one word at a time.
// The all-loaded path stores with nt and sc1 set, addressed from the block's
// start (sts_at; the block must span under 2 GiB of out, else nontemporal
// global stores): 2.5% faster cold on flat blocks than nontemporal stores,
// where the per-lane-address form (sts) was 13% slower.
template <int FMT, bool HW, int NT, int MAXV = 8>
__device__ void dequant_block(const uint8_t* __restrict__ q, float* __restrict__ out, float s,
                              int64_t base, int64_t stride, int rows, int cols, int tid) {
  if ((base % 4 == 0) && (stride % 4 == 0) && (cols % 4 == 0)) {
    const int vpr = cols / 4;
    const int nvec = rows * vpr;
    if (nvec <= NT * MAXV) {   // every code word loaded before any is decoded
      const bool rel = (static_cast<int64_t>(rows - 1) * stride + cols) * 4 < (int64_t(1) << 31);   // uniform
      uint32_t c[MAXV];
      int64_t at[MAXV];
      GridWalk w(tid, vpr, NT);
#pragma unroll
      for (int k = 0; k < MAXV; ++k) {
        at[k] = tid + k * NT < nvec ? base + static_cast<int64_t>(w.row) * stride + static_cast<int64_t>(w.col) * 4
                                    : base;
        c[k] = ldg(reinterpret_cast<const uint32_t*>(q + at[k]));
        w.next();
      }
#pragma unroll
      for (int k = 0; k < MAXV; ++k) {
        if (tid + k * NT < nvec) {
          const f32x4 d = decode4<FMT, HW>(c[k]);
          const f32x4 o{__fmul_rn(d.x, s), __fmul_rn(d.y, s), __fmul_rn(d.z, s), __fmul_rn(d.w, s)};
          if (rel)
            sts_at<kStoreNtSc1>(out + base, static_cast<int>((at[k] - base) * 4), o);
          else
            stg(reinterpret_cast<f32x4*>(out + at[k]), o);
        }
      }
      return;
    }
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
  dequant_block<FMT, HW, kThreads, 16>(q, out, scales[j.scale], j.base, j.stride, j.rows, j.cols,
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

// Flat blocks, one 128-thread workgroup per block: workgroup b < n_flat *
// kFlatPerGroup takes block b % kFlatPerGroup of flat group b / kFlatPerGroup
// (a 2048-element fp32 block is 4 vectors per thread, all loaded before the
// first is used); the rest take the zero-range jobs that follow the flat
// groups. Measured on gfx950 (Adam-state workload, int8 / uint8 codes, three
// interleaved rounds, cold): one wave per block (8 vectors per lane, 84
// VGPRs) 6.04-6.08 TB/s, 128 threads 6.22-6.28, 256 threads 5.80-5.83.
// Dequant keeps one wave per block: 6.00-6.05 against 5.85-5.92 (128) and
// 5.65-5.68 (256).
constexpr int kQuantFlatThreads = 128;

template <bool BF16, int FMT, bool HW>
__global__ __launch_bounds__(kQuantFlatThreads) void quant_flat_kernel(const QJob* __restrict__ jobs, int64_t n_flat,
                                                                       const void* __restrict__ src,
                                                                       uint8_t* __restrict__ q,
                                                                       float* __restrict__ scales, unsigned n_pieces) {
  __shared__ uint32_t red[kQuantFlatThreads / kWave];
  const int64_t n_main = n_flat * kFlatPerGroup;
  for (unsigned pb = blockIdx.x; pb < n_pieces; pb += gridDim.x) {
    const unsigned b = piece_index<kFlatXcdGroup>(pb, n_pieces);
    if (static_cast<int64_t>(b) >= n_main) {
      const QJob j = jobs[n_flat + (static_cast<int64_t>(b) - n_main)];
      zero_bytes<kQuantFlatThreads>(q, j.base, j.stride, threadIdx.x);
    } else {
      const QJob j = jobs[b / kFlatPerGroup];
      const int blk = static_cast<int>(b % kFlatPerGroup);
      if (blk < j.rows) {   // uniform over the workgroup
        const int len = blk == j.rows - 1 ? j.last : j.cols;
        // fp32: blocks of up to 2048 elements in registers; bf16: 4096
        quant_block<BF16, FMT, HW, kQuantFlatThreads, 512 / kQuantFlatThreads, true, kStoreNtSc1>(
            src, q, scales, j.base + static_cast<int64_t>(blk) * j.cols, len, 1, len, j.scale + blk, threadIdx.x, red);
      }
    }
    __syncthreads();   // the next block reuses `red`
  }
}

}  // namespace
}  // namespace rs

using namespace rs;

namespace {

// What one quant call launches: the job list (tiles, then flat groups, then
// zero ranges) in device memory, and the launch limits.
struct QuantLaunch {
  const QJob* jobs;
  int64_t n_tile, n_flat, n_zero;
  bool split_code_lines;
  int64_t max_grid;
};

dim3 grid_for(const QuantLaunch& L, int64_t n_items) {
  return dim3(static_cast<unsigned>(std::min<int64_t>(n_items, L.max_grid)));
}

// The zero-range jobs follow the flat groups, which follow the tiles: they ride
// at the end of the last launch that has blocks, or get their own launch.
template <bool BF16, int FMT, bool HW>
void launch_quant_kinds(const QuantLaunch& L, const void* src, uint8_t* q, float* scales, hipStream_t s) {
  const dim3 block(kThreads);
  const QJob* tiles = L.jobs;
  const QJob* flats = tiles + L.n_tile;
  const int64_t nz = L.n_zero;
  if (L.n_tile) {
    const int64_t n = L.n_tile + (L.n_flat ? 0 : nz);
    if (L.split_code_lines)
      hipLaunchKernelGGL((quant_tile_kernel<BF16, FMT, HW, kTileXcdGroupSplit>), grid_for(L, n), dim3(kQuantThreads), 0,
                         s, tiles, L.n_tile, src, q, scales, static_cast<unsigned>(n));
    else
      hipLaunchKernelGGL((quant_tile_kernel<BF16, FMT, HW, kTileXcdGroup>), grid_for(L, n), dim3(kQuantThreads), 0, s,
                         tiles, L.n_tile, src, q, scales, static_cast<unsigned>(n));
  }
  if (L.n_flat) {
    const int64_t n = L.n_flat * kFlatPerGroup + nz;   // one workgroup per flat block, then the zero ranges
    hipLaunchKernelGGL((quant_flat_kernel<BF16, FMT, HW>), grid_for(L, n), dim3(kQuantFlatThreads), 0, s, flats,
                       L.n_flat, src, q, scales, static_cast<unsigned>(n));
  }
  if (!L.n_tile && !L.n_flat && nz)
    hipLaunchKernelGGL(zero_codes_kernel, grid_for(L, nz), block, 0, s, flats, q, static_cast<unsigned>(nz));
}

template <bool BF16>
void launch_quant(const QuantLaunch& L, const void* src, int fmt, bool hw, uint8_t* q, float* scales,
                  hipStream_t s) {
  if (fmt == FMT_E4M3 && hw)
    launch_quant_kinds<BF16, FMT_E4M3, true>(L, src, q, scales, s);
  else if (fmt == FMT_E4M3)
    launch_quant_kinds<BF16, FMT_E4M3, false>(L, src, q, scales, s);
  else if (fmt == FMT_I8)
    launch_quant_kinds<BF16, FMT_I8, false>(L, src, q, scales, s);
  else
    launch_quant_kinds<BF16, FMT_U8, false>(L, src, q, scales, s);
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
  const QuantLaunch L{p->qjobs, p->n_qtile, p->n_qflat, p->n_qzero, p->split_code_lines, p->max_grid};
  if (src_dt == RS_BF16)
    launch_quant<true>(L, src, fmt, p->e4m3_hw, static_cast<uint8_t*>(q), scales, s);
  else
    launch_quant<false>(L, src, fmt, p->e4m3_hw, static_cast<uint8_t*>(q), scales, s);
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

// ------------------------------------------------------------------ allocation-free quant

namespace {

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on device `dev`, which is current; taken once per device.
int scratch_on(int dev, void** out, const char* who) {
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(RS_EINVAL, std::string(who) + ": device index " + std::to_string(dev) + " out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(RS_EHIP, std::string(who) + ": hipGetSymbolAddress of the work-list memory failed: " +
                               hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RS_OK;
}

}  // namespace

extern "C" int rs_block_quant_noalloc(const rs_tensor_spec* specs, int64_t n, int64_t V, int64_t S,
                                      const int64_t* starts, int64_t R_mat, const void* src, int32_t src_dt,
                                      void* q, int32_t q_dt, float* scales, int64_t scales_len, void* stream) {
  const char* who = "rs_block_quant_noalloc";
  try {
    clear_error();
    if (src_dt != RS_F32 && src_dt != RS_BF16) return fail(RS_EDTYPE, std::string(who) + ": src must be fp32 or bf16");
    const int fmt = fmt_of(q_dt);
    if (fmt < 0) return fail(RS_EDTYPE, std::string(who) + ": code format must be E4M3, I8 or U8");
    if (!src || !q) return fail(RS_EINVAL, std::string(who) + ": null buffer");
    if (!aligned16(src) || !aligned16(q)) return fail(RS_EALIGN, std::string(who) + ": src / q not 16-byte aligned");
    if (scales_len < 0) return fail(RS_EINVAL, std::string(who) + ": negative scales_len");
    std::vector<Tensor> t;
    int64_t R_used = 0;
    int st = validate_plan(who, specs, n, V, S, starts, R_mat, &t, &R_used);
    if (st != RS_OK) return st;
    QuantList ql;
    lower_quant(t, R_mat * S, &ql);
    if (ql.n_blocks > scales_len || (ql.n_blocks > 0 && !scales))
      return fail(RS_EINVAL, std::string(who) + ": the plan has " + std::to_string(ql.n_blocks) +
                                 " quantisation blocks; scales holds " + std::to_string(scales ? scales_len : 0));
    const int64_t bytes = static_cast<int64_t>(sizeof(QJob)) * static_cast<int64_t>(ql.jobs.size());
    if (bytes > kNoallocScratchBytes)
      return fail(RS_ERANGE, std::string(who) + ": the plan needs " + std::to_string(ql.jobs.size()) +
                                 " quant work items (" + std::to_string(bytes) + " bytes); the static work-list "
                                 "memory holds " + std::to_string(kNoallocScratchBytes / int64_t(sizeof(QJob))) +
                                 " (" + std::to_string(kNoallocScratchBytes) + " bytes): use rs_plan_load and "
                                 "rs_block_quant");
    if (ql.jobs.empty()) return RS_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(RS_EHIP, std::string(who) + ": hipGetDevice failed");
    void* ptr = nullptr;
    st = scratch_on(dev, &ptr, who);
    if (st != RS_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // The list goes in on the call's stream, after the work already queued there
    // (a previous call on this stream may still be reading it). The copy reads this
    // call's pageable host memory, so the call waits for it before returning.
    if (hipMemcpyAsync(ptr, ql.jobs.data(), static_cast<size_t>(bytes), hipMemcpyHostToDevice, s) != hipSuccess)
      return fail(RS_EHIP, std::string(who) + ": upload of the work list failed");
    if (hipStreamSynchronize(s) != hipSuccess)
      return fail(RS_EHIP, std::string(who) + ": waiting for the work-list upload failed");
    const char* enc = std::getenv("RS_E4M3_ENCODER");
    const bool hw = !(enc && std::strcmp(enc, "sw") == 0);
    int64_t max_grid = kMaxGrid;
    if (const char* mg = std::getenv("RS_MAX_GRID")) {
      const long long v = std::strtoll(mg, nullptr, 10);
      max_grid = std::max<int64_t>(8, std::min<int64_t>(kMaxGrid, v) / 8 * 8);
    }
    const QuantLaunch L{static_cast<const QJob*>(ptr), ql.n_tile, ql.n_flat, ql.n_zero, ql.split_code_lines,
                        max_grid};
    if (src_dt == RS_BF16)
      launch_quant<true>(L, src, fmt, hw, static_cast<uint8_t*>(q), scales, s);
    else
      launch_quant<false>(L, src, fmt, hw, static_cast<uint8_t*>(q), scales, s);
    return launched(who);
  } catch (const std::exception& ex) {
    return fail(RS_ENOMEM, std::string(who) + ": " + ex.what());
  }
}
