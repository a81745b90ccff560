// Unpack and pack of a RaggedShard / DBuffer group on gfx950: kernels and the
// rs_unpack_gathered / rs_pack_scatter entry points.
//
// Unpack copies each tensor out of the gathered flat buffer, bit for bit
// ("veScale-FSDP: flexible, structure-aware sharding at 10K-GPU scale",
// feynmanwiki walkthrough, DBuffer paragraphs: a tensor is its planned
// slice). Pack writes the gradients into the flat buffer with the fused
// pre-communication ops of the DBuffer paragraph: scale by sigma, then add the
// previous buffer, as two IEEE round-to-nearest-even operations (__fmul_rn,
// __fadd_rn, never an FMA), and +0.0 in the padding. Both split each plan item
// over small, short-lived workgroups. Tile-major tensors are reordered through
// an LDS stage per strip, or directly per lane.
#include "host_common.h"

namespace rs {
namespace {

// ------------------------------------------------------------------ unpack

// Workgroup b copies piece b % split (kUnpackPiece vectors) of chunk b / split.
// Stores with nt and sc1 set: 3% faster cold than nontemporal ones (8B and
// MoE layers), the same warm.
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
    if (v0 + u * kUnpackThreads < nvec) sts<kStoreNtSc1>(d4 + v0 + u * kUnpackThreads, r[u]);
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

// Four (or one) packed values at element `pos` of the packed buffer: fp32, or,
// for a bf16 buffer (OB), each fp32 result rounded once to the nearest bf16
// (ties to even). Stores with nt and sc1 set: 2-3% faster cold than
// nontemporal ones for every pack measured (fp32, with and without
// accumulation; row-major and tile-major).
template <bool OB>
__device__ __forceinline__ void store_packed4(void* out, int64_t pos, const f32x4& y) {
  if constexpr (OB)
    sts<kStoreNtSc1>(reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + pos),
        u32x2{bf16_rne(y.x) | (bf16_rne(y.y) << 16), bf16_rne(y.z) | (bf16_rne(y.w) << 16)});
  else
    sts<kStoreNtSc1>(reinterpret_cast<f32x4*>(static_cast<float*>(out) + pos), y);
}

template <bool OB>
__device__ __forceinline__ void store_packed1(void* out, int64_t pos, float y) {
  if constexpr (OB)
    static_cast<uint16_t*>(out)[pos] = static_cast<uint16_t>(bf16_rne(y));
  else
    static_cast<float*>(out)[pos] = y;
}

// packed = acc ? prev + src*sigma : src*sigma on tensor data, +0.0 on padding.
// Workgroup b (NT threads) writes piece b % split (NT * kPackVec output
// vectors) of chunk b / split, split = pack_split(NT). `prev` may alias `out`:
// every element is read before it is written, by the same thread (fp32 output
// only).
template <bool BF16, bool ACC, bool OB, int NT>
__device__ __forceinline__ void pack_kernel_piece(unsigned b, const PackChunk* __restrict__ chunks,
                                                             const void* const* __restrict__ src,
                                                             const float* prev, void* out, float sigma) {
  constexpr unsigned kSplit = static_cast<unsigned>(pack_split(NT));
  const unsigned cu = b / kSplit;
  const int ci = static_cast<int>(cu);
  const int piece = static_cast<int>(b - cu * kSplit);
  const PackChunk c = chunks[ci];
  const int nv = c.n_total >> 2;
  const int v0 = piece * NT * kPackVec + static_cast<int>(threadIdx.x);
  if (c.tensor < 0) {
#pragma unroll
    for (int u = 0; u < kPackVec; ++u)
      if (v0 + u * NT < nv)
        store_packed4<OB>(out, c.out + 4 * static_cast<int64_t>(v0 + u * NT), f32x4{0.0f, 0.0f, 0.0f, 0.0f});
    return;
  }
  const void* g = src[c.tensor];
  const int nd = c.n_data;
  const f32x4* p4 = reinterpret_cast<const f32x4*>(prev + c.out);
  f32x4 gv[kPackVec], pv[kPackVec];
#pragma unroll
  for (int u = 0; u < kPackVec; ++u) {
    const int i = v0 + u * NT;
    if (i < nv && 4 * i + 4 <= nd) {
      gv[u] = load4<BF16>(g, c.off + 4 * i);
      if constexpr (ACC) pv[u] = ldg(p4 + i);
    }
  }
#pragma unroll
  for (int u = 0; u < kPackVec; ++u) {
    const int i = v0 + u * NT;
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
    store_packed4<OB>(out, c.out + 4 * static_cast<int64_t>(i), y);
  }
}

// Workgroup shape: the accumulating pack kPackThreads threads, runs of
// kPackXcdGroup pieces per XCD; without accumulation kPack1Threads, runs of
// kPack1XcdGroup.
template <bool ACC>
struct PackShape {
  static constexpr int NT = ACC ? kPackThreads : kPack1Threads;
  static constexpr unsigned XG = ACC ? kPackXcdGroup : kPack1XcdGroup;
};

template <bool BF16, bool ACC, bool OB>
__global__ __launch_bounds__(PackShape<ACC>::NT) void pack_kernel(const PackChunk* __restrict__ chunks,
                                                                  const void* const* __restrict__ src,
                                                                  const float* prev, void* out, float sigma,
                                                                  unsigned n_pieces) {
  using Sh = PackShape<ACC>;
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    pack_kernel_piece<BF16, ACC, OB, Sh::NT>(piece_index<Sh::XG>(p, n_pieces), chunks, src, prev, out, sigma);
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
      sts<kStoreNtSc1>(reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(r) * j.cols + w * VE) * EB),
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
template <bool BF16, bool ACC, bool OB>
__device__ __forceinline__ void pack_tm_kernel_job(unsigned jb, unsigned n_jobs, const TmJob* __restrict__ jobs,
                                                           const void* const* __restrict__ src,
                                                           const float* prev, void* out, float sigma) {
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
      store_packed4<OB>(out, pos, y);
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
    store_packed1<OB>(out, pos, y);
  }
}

template <bool BF16, bool ACC, bool OB>
__global__ __launch_bounds__(kTmLdsThreads) void pack_tm_kernel(const TmJob* __restrict__ jobs,
                                                           const void* const* __restrict__ src,
                                                           const float* prev, void* out, float sigma, unsigned n_jobs) {
  for (unsigned jb = blockIdx.x; jb < n_jobs; jb += gridDim.x) {
    pack_tm_kernel_job<BF16, ACC, OB>(jb, n_jobs, jobs, src, prev, out, sigma);
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
      sts<kStoreNtSc1>(reinterpret_cast<u32x4*>(out + (static_cast<int64_t>(r) * j.cols + col) * EB), x);
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

template <bool BF16, bool ACC, bool OB>
__device__ __forceinline__ void pack_tm_direct_kernel_piece(unsigned b, const TmJob* __restrict__ jobs,
                                                                    const void* const* __restrict__ src,
                                                                    const float* prev, void* out, float sigma,
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
      store_packed4<OB>(out, pos, y);
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
    store_packed1<OB>(out, pos, y);
  }
}

template <bool BF16, bool ACC, bool OB>
__global__ __launch_bounds__(kTmThreads) void pack_tm_direct_kernel(const TmJob* __restrict__ jobs,
                                                                    const void* const* __restrict__ src,
                                                                    const float* prev, void* out, float sigma,
                                                                    int split, unsigned n_pieces) {
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    pack_tm_direct_kernel_piece<BF16, ACC, OB>(p, jobs, src, prev, out, sigma, split);
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

namespace {

template <bool BF16, bool ACC, bool OB>
void launch_pack(const rs_plan* p, void** tab, const float* prev, void* packed, float sigma, hipStream_t s) {
  if (p->n_pack) {
    const int64_t n_pieces = p->n_pack * pack_split(PackShape<ACC>::NT);
    hipLaunchKernelGGL((pack_kernel<BF16, ACC, OB>), grid_of(p, n_pieces), dim3(PackShape<ACC>::NT), 0, s, p->pack,
                       tab, prev, packed, sigma, static_cast<unsigned>(n_pieces));
  }
  if (p->n_tm && !p->tm_pack_lds) {
    const int64_t split = tm_pieces(p->tm_max_strip, 4, kTmThreads);
    const int64_t n = p->n_tm * split;
    hipLaunchKernelGGL((pack_tm_direct_kernel<BF16, ACC, OB>), grid_of(p, n), dim3(kTmThreads), 0, s, p->tmjobs, tab,
                       prev, packed, sigma, static_cast<int>(split), static_cast<unsigned>(n));
  } else if (p->n_tm) {
    const unsigned lds = static_cast<unsigned>(p->tm_max_strip * 4);
    hipLaunchKernelGGL((pack_tm_kernel<BF16, ACC, OB>), grid_of(p, p->n_tm), dim3(kTmLdsThreads), lds, s, p->tmjobs,
                       tab, prev, packed, sigma, static_cast<unsigned>(p->n_tm));
  }
}

template <bool BF16, bool OB>
void launch_pack_acc(const rs_plan* p, void** tab, const float* prev, void* packed, float sigma, hipStream_t s) {
  if (prev) launch_pack<BF16, true, OB>(p, tab, prev, packed, sigma, s);
  else launch_pack<BF16, false, OB>(p, tab, prev, packed, sigma, s);
}

}  // namespace

extern "C" int rs_pack_scatter(rs_plan* p, const void* const* src, int32_t src_dt, const float* prev,
                               void* packed, int32_t packed_dt, int32_t scale_mode, float scale, void* stream) {
  const char* who = "rs_pack_scatter";
  clear_error();
  int st = check_call(p, who);
  if (st != RS_OK) return st;
  if (src_dt != RS_F32 && src_dt != RS_BF16) return fail(RS_EDTYPE, std::string(who) + ": src must be fp32 or bf16");
  if (packed_dt != RS_F32 && packed_dt != RS_BF16)
    return fail(RS_EDTYPE, std::string(who) + ": packed must be fp32 or bf16");
  if (!src || !packed) return fail(RS_EINVAL, std::string(who) + ": null buffer");
  if (packed_dt == RS_BF16 && prev && static_cast<const void*>(prev) == packed)
    return fail(RS_EINVAL, std::string(who) + ": in-place accumulation needs an fp32 packed buffer");
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
  void** tab = p->src.dev;
  if (src_dt == RS_F32 && packed_dt == RS_F32) launch_pack_acc<false, false>(p, tab, prev, packed, sigma, s);
  else if (src_dt == RS_F32) launch_pack_acc<false, true>(p, tab, prev, packed, sigma, s);
  else if (packed_dt == RS_F32) launch_pack_acc<true, false>(p, tab, prev, packed, sigma, s);
  else launch_pack_acc<true, true>(p, tab, prev, packed, sigma, s);
  return launched(who);
}
