// One AdamW step on block-quantised 8-bit state on gfx950: kernels and the
// rs_adam8_step entry point.
//
// Per quantisation block: dequantise int8 m and uint8 v, update them and the
// fp32 parameters with the packed gradient, requantise m and v with fresh
// block scales ("veScale-FSDP: flexible, structure-aware sharding at 10K-GPU
// scale", feynmanwiki walkthrough, 8-bit Adam paragraph: each device
// quantises its own whole blocks). Every operation is one IEEE fp32 rounding.
#include "host_common.h"

namespace rs {
namespace {

// ------------------------------------------------------------------ 8-bit Adam step

struct AdamK {
  float b1, b2, c1, c2, eps, step_size, inv_bc2_sqrt, decay;
};

// sqrt(v1), correctly rounded: the short sequence where it holds, else
// __builtin_sqrtf, which the library's compile flags
// (-fhip-fp32-correctly-rounded-divide-sqrt) lower to the general correctly
// rounded sequence (v1 = 0, subnormal or tiny, infinite or NaN); __fsqrt_rn
// is not correctly rounded with this compiler (about 15% of inputs differ by
// an ulp). On the Adam-state workload the flat-block step went from
// 5.94-6.00 to 6.11-6.14 TB/s cold with the short sequence (three interleaved
// rounds; that kernel's VALU was 98% busy); the 32x32-strip step did not move.
__device__ __forceinline__ float adam_sqrt(float x) {
  return (x >= kSqrtShortMin && x <= FLT_MAX) ? sqrt_rn_short(x) : __builtin_sqrtf(x);
}

// m1, v1 and the new parameter of one element (every operation rounded).
__device__ __forceinline__ void adam_elem(float p, float g, float m0, float v0, const AdamK& k,
                                          float& p1, float& m1, float& v1) {
  m1 = __fadd_rn(__fmul_rn(k.b1, m0), __fmul_rn(k.c1, g));
  v1 = __fadd_rn(__fmul_rn(k.b2, v0), __fmul_rn(k.c2, __fmul_rn(g, g)));
  const float den = __fadd_rn(__fmul_rn(adam_sqrt(v1), k.inv_bc2_sqrt), k.eps);
  p1 = __fsub_rn(__fmul_rn(p, k.decay), __fmul_rn(k.step_size, __fdiv_rn(m1, den)));
}

// One quantisation block (element (r, c) at base + r*stride + c) handled by
// NT threads. The old scales are read before the block's max is reduced and
// the new ones written after it. Fast path: 4-element vectors, every updated
// m and v kept in registers, the loads issued B vectors at a time; otherwise
// two passes (the second recomputes m1 and v1 from the old codes, which it
// then overwrites). The tile kernels load one vector at a time (B = 1); the
// flat-block kernel, with two vectors per thread, loads both first.
// Nontemporal stores: with nt-sc1 ones the flat-block step ran 3% slower.
template <int NT, int MAXV, int B = 1>
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
    // vectors in batches of B: every load of a batch is issued before the first is
    // used (a lane past the block reads the block's first vector and ignores it)
#pragma unroll
    for (int j0 = 0; j0 < MAXV; j0 += B) {
      f32x4 p[B], g[B];
      uint32_t cm[B], cv[B];
      int64_t at[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        at[b] = tid + (j0 + b) * NT < nvec
                    ? base + static_cast<int64_t>(w.row) * stride + static_cast<int64_t>(w.col) * 4 : base;
        p[b] = ldg(reinterpret_cast<const f32x4*>(param + at[b]));
        g[b] = ldg(reinterpret_cast<const f32x4*>(grad + at[b]));
        cm[b] = ldg(reinterpret_cast<const uint32_t*>(qm + at[b]));
        cv[b] = ldg(reinterpret_cast<const uint32_t*>(qv + at[b]));
        w.next();
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int j = j0 + b;
        if (tid + j * NT >= nvec) continue;
        const f32x4 dm = decode4<FMT_I8, false>(cm[b]), dv = decode4<FMT_U8, false>(cv[b]);
        const float pin[4] = {p[b].x, p[b].y, p[b].z, p[b].w}, gin[4] = {g[b].x, g[b].y, g[b].z, g[b].w};
        const float dmi[4] = {dm.x, dm.y, dm.z, dm.w}, dvi[4] = {dv.x, dv.y, dv.z, dv.w};
        float po[4], mo[4], vo[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          adam_elem(pin[h], gin[h], __fmul_rn(dmi[h], sm0), __fmul_rn(dvi[h], sv0), k, po[h], mo[h], vo[h]);
        m1[j] = f32x4{mo[0], mo[1], mo[2], mo[3]};
        v1[j] = f32x4{vo[0], vo[1], vo[2], vo[3]};
        stg(reinterpret_cast<f32x4*>(param + at[b]), f32x4{po[0], po[1], po[2], po[3]});
        am = max(am, max(max(__float_as_uint(m1[j].x) & 0x7fffffffu, __float_as_uint(m1[j].y) & 0x7fffffffu),
                         max(__float_as_uint(m1[j].z) & 0x7fffffffu, __float_as_uint(m1[j].w) & 0x7fffffffu)));
        av = max(av, max(max(__float_as_uint(v1[j].x) & 0x7fffffffu, __float_as_uint(v1[j].y) & 0x7fffffffu),
                         max(__float_as_uint(v1[j].z) & 0x7fffffffu, __float_as_uint(v1[j].w) & 0x7fffffffu)));
      }
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
        const uint32_t cm = rm == 0.0f ? 0u
            : encode4<FMT_I8, false>(__fmul_rn(m1[j].x, rm), __fmul_rn(m1[j].y, rm), __fmul_rn(m1[j].z, rm), __fmul_rn(m1[j].w, rm));
        const uint32_t cv = rv == 0.0f ? 0u
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
    qm[e] = rm == 0.0f ? 0 : static_cast<uint8_t>(encode1<FMT_I8, false>(__fmul_rn(m1, rm)));
    qv[e] = rv == 0.0f ? 0 : static_cast<uint8_t>(encode1<FMT_U8, false>(__fmul_rn(v1, rv)));
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

// Tiles of at most 1024 elements (the pages' 32x32 blocks): one wave per tile,
// kAdamWaveTiles tiles per workgroup, the block's absmax a wave reduction
// only (no LDS, no barrier). Tile jobs b*kAdamWaveTiles + wave.
constexpr int kAdamWaveTiles = kAdamStripTiles;

//
// Four 32x32 tiles side by side in one band (the usual case: the workgroup's
// four jobs are consecutive tiles of a band) form a 32 x 128 strip whose rows
// of 1-byte codes are whole 128-byte runs, while each tile alone has only 32
// bytes of codes per row, a quarter of a line shared with three other tiles.
// The workgroup then moves the strip's codes through LDS with 16-byte lane
// accesses, eight lanes per 128-byte row, and each wave updates its own tile
// from there; the fp32 parameters and gradients (128 bytes per tile row) go
// straight to and from memory. Other groups of four jobs take one wave per
// tile directly.
constexpr int kStripRows = kAdamStripRows, kStripTileCols = kAdamStripTileCols;
constexpr int kStripCols = kAdamWaveTiles * kStripTileCols;

// One 32x32 tile of a strip by one wave: codes read from and written back to
// the strip's LDS copy (cm, cv: kStripRows rows of kStripCols bytes; this
// tile's columns start at c0). The arithmetic and the order of every
// operation are adam_block's.
constexpr int kAdamStripThreads = kAdamWaveTiles * kWave;
constexpr int kStripVPR = kStripTileCols / 4;             // 4-element vectors per tile row
constexpr int kStripNV = kStripRows * kStripVPR / kWave;  // vectors per lane

// Parameters and gradients of one lane's vectors of a strip tile, loaded
// while the workgroup stages the strip's codes. The strip kernels store with
// nt and sc1 set: 1-3% faster cold than with nontemporal stores.
__device__ __forceinline__ void adam_strip_loads(const float* __restrict__ param, const float* __restrict__ grad,
                                                 int64_t base, int64_t stride, int lane, f32x4 (&p)[kStripNV],
                                                 f32x4 (&g)[kStripNV]) {
#pragma unroll
  for (int j = 0; j < kStripNV; ++j) {
    const int i = lane + j * kWave, row = i / kStripVPR, col = (i % kStripVPR) * 4;
    const int64_t e = base + row * stride + col;
    p[j] = ldg(reinterpret_cast<const f32x4*>(param + e));
    g[j] = ldg(reinterpret_cast<const f32x4*>(grad + e));
  }
}

__device__ void adam_strip_tile(float* __restrict__ param, const f32x4 (&pv)[kStripNV], const f32x4 (&gv)[kStripNV],
                                uint8_t* cm, uint8_t* cv, float* __restrict__ sm, float* __restrict__ sv,
                                int64_t base, int64_t stride, int c0, int64_t sidx, int lane, const AdamK& k) {
  constexpr int VPR = kStripVPR;
  constexpr int NV = kStripNV;
  const float sm0 = sm[sidx], sv0 = sv[sidx];
  f32x4 m1[NV], v1[NV];
  uint32_t am = 0, av = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = lane + j * kWave, row = i / VPR, col = (i % VPR) * 4;
    const int64_t e = base + row * stride + col;
    const f32x4 p = pv[j];
    const f32x4 g = gv[j];
    const f32x4 dm = decode4<FMT_I8, false>(*reinterpret_cast<const uint32_t*>(cm + row * kStripCols + c0 + col));
    const f32x4 dv = decode4<FMT_U8, false>(*reinterpret_cast<const uint32_t*>(cv + row * kStripCols + c0 + col));
    const float pin[4] = {p.x, p.y, p.z, p.w}, gin[4] = {g.x, g.y, g.z, g.w};
    const float dmi[4] = {dm.x, dm.y, dm.z, dm.w}, dvi[4] = {dv.x, dv.y, dv.z, dv.w};
    float po[4], mo[4], vo[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      adam_elem(pin[h], gin[h], __fmul_rn(dmi[h], sm0), __fmul_rn(dvi[h], sv0), k, po[h], mo[h], vo[h]);
    m1[j] = f32x4{mo[0], mo[1], mo[2], mo[3]};
    v1[j] = f32x4{vo[0], vo[1], vo[2], vo[3]};
    sts<kStoreNtSc1>(reinterpret_cast<f32x4*>(param + e), f32x4{po[0], po[1], po[2], po[3]});
    am = max(am, max(max(__float_as_uint(mo[0]) & 0x7fffffffu, __float_as_uint(mo[1]) & 0x7fffffffu),
                     max(__float_as_uint(mo[2]) & 0x7fffffffu, __float_as_uint(mo[3]) & 0x7fffffffu)));
    av = max(av, max(max(__float_as_uint(vo[0]) & 0x7fffffffu, __float_as_uint(vo[1]) & 0x7fffffffu),
                     max(__float_as_uint(vo[2]) & 0x7fffffffu, __float_as_uint(vo[3]) & 0x7fffffffu)));
  }
  const float amax_m = __uint_as_float(wave_max(am));
  const float amax_v = __uint_as_float(wave_max(av));
  float scm, rm, scv, rv;
  block_scale(amax_m, 127.0f, scm, rm);
  block_scale(amax_v, 255.0f, scv, rv);
  if (lane == 0) {
    sm[sidx] = scm;
    sv[sidx] = scv;
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = lane + j * kWave, row = i / VPR, col = (i % VPR) * 4;
    *reinterpret_cast<uint32_t*>(cm + row * kStripCols + c0 + col) = rm == 0.0f ? 0u
        : encode4<FMT_I8, false>(__fmul_rn(m1[j].x, rm), __fmul_rn(m1[j].y, rm), __fmul_rn(m1[j].z, rm), __fmul_rn(m1[j].w, rm));
    *reinterpret_cast<uint32_t*>(cv + row * kStripCols + c0 + col) = rv == 0.0f ? 0u
        : encode4<FMT_U8, false>(__fmul_rn(v1[j].x, rv), __fmul_rn(v1[j].y, rv), __fmul_rn(v1[j].z, rv), __fmul_rn(v1[j].w, rv));
  }
}

// ALL_STRIPS: the plan's lowering found every group to be a strip, so the
// kernel neither checks nor carries the one-wave-per-tile path, whose
// registers would otherwise set the kernel's count (115 VGPRs instead of 124;
// the 8B layer's states in 32x32 tiles: 5.95-5.99 -> 6.04-6.09 TB/s cold,
// three interleaved rounds). Two waves per tile (512-thread strips, the
// tile's maxima combined through LDS; 94 VGPRs, but still 4 waves per SIMD
// with 8-wave workgroups) ran at 5.09-5.10.
template <bool ALL_STRIPS>
__global__ __launch_bounds__(kAdamStripThreads) void adam_wave_tile_kernel(
    const QJob* __restrict__ jobs, float* param, const float* grad, uint8_t* qm, float* sm, uint8_t* qv, float* sv,
    AdamK k, unsigned n_jobs, unsigned n_groups) {
  __shared__ __align__(16) uint8_t cm[kStripRows * kStripCols];
  __shared__ __align__(16) uint8_t cv[kStripRows * kStripCols];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  for (unsigned gb = blockIdx.x; gb < n_groups; gb += gridDim.x) {
    const unsigned t0 = piece_index<kTileXcdGroup>(gb, n_groups) * kAdamWaveTiles;
    // a strip: four full 32x32 tiles of one tensor side by side, 16-byte aligned
    // (every thread reads the four jobs, so the choice is the same for all waves)
    const QJob j0 = jobs[min(t0, n_jobs - 1)];
    bool strip = ALL_STRIPS;
    if constexpr (!ALL_STRIPS) {
      strip = t0 + kAdamWaveTiles <= n_jobs && j0.rows == kStripRows && j0.cols == kStripTileCols &&
              j0.base % 16 == 0 && j0.stride % 16 == 0;
#pragma unroll
      for (int w = 1; w < kAdamWaveTiles; ++w) {
        if (!strip) break;
        const QJob jw = jobs[t0 + w];
        strip = jw.tensor == j0.tensor && jw.rows == kStripRows && jw.cols == kStripTileCols &&
                jw.stride == j0.stride && jw.base == j0.base + w * kStripTileCols && jw.scale == j0.scale + w;
      }
    }
    if (!ALL_STRIPS && !strip) {   // one wave per tile
      const unsigned t = t0 + wave;
      if (wave < kAdamWaveTiles && t < n_jobs) {
        const QJob j = jobs[t];
        adam_block<kWave, 4>(param, grad, qm, sm, qv, sv, j.base, j.stride, j.rows, j.cols, j.scale, lane, nullptr, k);
      }
      continue;
    }
    // codes of the strip in: thread i moves 16 bytes of row i / 8
    const int row = threadIdx.x / (kStripCols / 16), chunk = threadIdx.x % (kStripCols / 16);
    const int64_t ge = j0.base + row * j0.stride + chunk * 16;
    const u32x4 codes_m = ldg(reinterpret_cast<const u32x4*>(qm + ge));
    const u32x4 codes_v = ldg(reinterpret_cast<const u32x4*>(qv + ge));
    f32x4 pv[kStripNV], gv[kStripNV];
    const int64_t tb = j0.base + wave * kStripTileCols;
    adam_strip_loads(param, grad, tb, j0.stride, lane, pv, gv);
    *reinterpret_cast<u32x4*>(cm + row * kStripCols + chunk * 16) = codes_m;
    *reinterpret_cast<u32x4*>(cv + row * kStripCols + chunk * 16) = codes_v;
    __syncthreads();
    adam_strip_tile(param, pv, gv, cm, cv, sm, sv, tb, j0.stride, wave * kStripTileCols, j0.scale + wave, lane, k);
    __syncthreads();
    sts<kStoreNtSc1>(reinterpret_cast<u32x4*>(qm + ge), *reinterpret_cast<const u32x4*>(cm + row * kStripCols + chunk * 16));
    sts<kStoreNtSc1>(reinterpret_cast<u32x4*>(qv + ge), *reinterpret_cast<const u32x4*>(cv + row * kStripCols + chunk * 16));
    __syncthreads();   // the next group reuses the LDS copy
  }
}

// Tiles of up to 16384 elements (128x128): 1024 threads per tile, four
// 4-element vectors each in registers.
constexpr int kAdamBigTileThreads = 1024;

__global__ __launch_bounds__(kAdamBigTileThreads) void adam_big_tile_kernel(
    const QJob* __restrict__ jobs, float* param, const float* grad, uint8_t* qm, float* sm, uint8_t* qv, float* sv,
    AdamK k, unsigned n_jobs) {
  __shared__ uint32_t red[2 * kAdamBigTileThreads / kWave];
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    const QJob j = jobs[piece_index<kTileXcdGroup>(jb, n_jobs)];
    adam_block<kAdamBigTileThreads, 4>(param, grad, qm, sm, qv, sv, j.base, j.stride, j.rows, j.cols, j.scale,
                                       threadIdx.x, red, k);
    __syncthreads();   // the next job reuses this workgroup's LDS
  }
}

// Flat blocks, one 256-thread workgroup per block (workgroup b takes block
// b % kFlatPerGroup of flat group b / kFlatPerGroup): a 2048-element block is
// two 4-element vectors per thread, both loaded before either is used.
// Measured on gfx950 against one wave per block (8 vectors per lane, 122
// VGPRs, 4 waves per SIMD), three interleaved rounds on the Adam-state
// workload, cold: 5.74-5.82 TB/s one wave, 5.78-5.84 with 128 threads,
// 5.79-5.85 with 256 threads one vector at a time, 5.85-5.94 with 256 threads
// and both vectors' loads first (57 VGPRs, 8 waves per SIMD).
constexpr int kAdamFlatThreads = 256;
constexpr int kAdamFlatVec = (2048 / 4 + kAdamFlatThreads - 1) / kAdamFlatThreads;

__global__ __launch_bounds__(kAdamFlatThreads) void adam_flat_kernel(const QJob* __restrict__ jobs, float* param,
                                                                     const float* grad, uint8_t* qm, float* sm,
                                                                     uint8_t* qv, float* sv, AdamK k,
                                                                     unsigned n_pieces) {
  __shared__ uint32_t red[2 * (kAdamFlatThreads / kWave)];
  for (unsigned pb = blockIdx.x; pb < n_pieces; pb += gridDim.x) {
    const unsigned b = piece_index<kFlatXcdGroup>(pb, n_pieces);
    const QJob j = jobs[b / kFlatPerGroup];
    const int blk = static_cast<int>(b % kFlatPerGroup);
    if (blk < j.rows) {   // uniform over the workgroup
      const int len = blk == j.rows - 1 ? j.last : j.cols;
      adam_block<kAdamFlatThreads, kAdamFlatVec, kAdamFlatVec>(param, grad, qm, sm, qv, sv,
                                                               j.base + static_cast<int64_t>(blk) * j.cols, len, 1,
                                                               len, j.scale + blk, threadIdx.x, red, k);
    }
    __syncthreads();   // the next block reuses `red`
  }
}

}  // namespace
}  // namespace rs

using namespace rs;

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
  // tiles: the register path sized to the plan's largest tile (16-byte vectors of fp32)
  const int64_t nt = p->n_qtile;
  if (nt && p->adam_wave_tiles && p->max_tile_vec16 <= kWave * 4) {
    const int64_t groups = (nt + kAdamWaveTiles - 1) / kAdamWaveTiles;
    if (p->adam_all_strips)
      hipLaunchKernelGGL(adam_wave_tile_kernel<true>, grid_of(p, groups), dim3(kAdamStripThreads), 0, s, p->qjobs,
                         param, grad, qmb, s_m, qvb, s_v, k, static_cast<unsigned>(nt), static_cast<unsigned>(groups));
    else
      hipLaunchKernelGGL(adam_wave_tile_kernel<false>, grid_of(p, groups), dim3(kAdamStripThreads), 0, s, p->qjobs,
                         param, grad, qmb, s_m, qvb, s_v, k, static_cast<unsigned>(nt), static_cast<unsigned>(groups));
  } else if (nt && p->max_tile_vec16 > kThreads * 4 && p->max_tile_vec16 <= kAdamBigTileThreads * 4) {
    hipLaunchKernelGGL(adam_big_tile_kernel, grid_of(p, nt), dim3(kAdamBigTileThreads), 0, s, p->qjobs, param, grad,
                       qmb, s_m, qvb, s_v, k, static_cast<unsigned>(nt));
  } else if (nt) {
    hipLaunchKernelGGL(adam_tile_kernel, grid_of(p, nt), dim3(kThreads), 0, s, p->qjobs, param, grad, qmb, s_m,
                       qvb, s_v, k, static_cast<unsigned>(nt));
  }
  if (p->n_qflat) {
    const int64_t n = p->n_qflat * kFlatPerGroup;   // one workgroup per flat block
    hipLaunchKernelGGL(adam_flat_kernel, grid_of(p, n), dim3(kAdamFlatThreads), 0, s, p->qjobs + p->n_qtile, param,
                       grad, qmb, s_m, qvb, s_v, k, static_cast<unsigned>(n));
  }
  return launched(who);
}

