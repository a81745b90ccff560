// The FP8 gather side on gfx950: kernels and the rs_unpack_dequant entry point.
//
// After the codes and scales are gathered, each quantised tensor is rebuilt
// as fl32(decode(code) * scale), rounded to bf16 for a bf16 tensor, in one
// pass over the codes (DeepSeek-V3-style block-wise FP8 training, as in
// "veScale-FSDP: Flexible and High-Performance FSDP at Scale", TL;DR and Key
// claims). Row runs and tile-major strips are split over small workgroups.
#include "host_common.h"

namespace rs {
namespace {

// ------------------------------------------------------------------ gather side

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
          stg_global(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(dst) + dbase + off[u]), o);
        } else {
          f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(dst) + dbase + off[u]);
          stg_global(o, f32x4{v[0], v[1], v[2], v[3]});
          stg_global(o + 1, f32x4{v[4], v[5], v[6], v[7]});
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


// Contiguous row runs of a quantised tensor (see GatherChunk). Each lane turns
// VEC codes into one 16-byte store (8 codes -> 8 bf16, 4 codes -> 4 fp32), so
// the lanes of a wave read and write one contiguous range each. Workgroup b
// takes piece b % split of run b / split: U vectors per thread (the plan's
// gather_vec, 2 or 4), and again split pieces further on while the run lasts.
// A run of several rows holds at most kGatherMaxRun elements, fewer than 2^16
// vectors, so its row and tile-column indices come from div_u16; a one-row
// run needs no division. Stores have nt and sc1 set and are addressed
// from the run's start (sts_at, when the run spans under 2 GiB of the tensor,
// as every run of a TILE tensor does; otherwise nontemporal global stores):
// 1-2% faster cold than nontemporal global stores, where the per-lane-address
// form (sts) was 1-7% slower and the flat stores that the table's pointer
// gave before a global cast 2-5% slower.
template <int FMT, bool HW, bool BF16OUT, int U>
__device__ __forceinline__ void gather_rows_kernel_piece(unsigned b, const GatherChunk* __restrict__ chunks,
                                                                    const uint8_t* __restrict__ q,
                                                                    const float* __restrict__ scales,
                                                                    void* const* __restrict__ dst, int split) {
  constexpr int VEC = BF16OUT ? 8 : 4;
  constexpr int kPiece = static_cast<int>(gather_piece(U));
  const unsigned cu = b / static_cast<unsigned>(split);
  const int ci = static_cast<int>(cu);
  const int piece = static_cast<int>(b - cu * static_cast<unsigned>(split));
  const GatherChunk c = chunks[ci];
  void* out = dst[c.tensor];
  const uint32_t vpr = static_cast<uint32_t>(c.cols / VEC);
  const int nvec = c.rows * static_cast<int>(vpr);
  const uint8_t* qb = q + c.qbase;
  const bool band = c.rstep == 0;
  const bool rel = static_cast<int64_t>(nvec) * 16 < (int64_t(1) << 31);   // uniform
  const uint32_t mv = magic_u16(vpr);
  const uint32_t cpt = band ? static_cast<uint32_t>(c.bc / VEC) : 1u;   // vectors per tile column
  const uint32_t mc = magic_u16(cpt);
  const int pass = split * kPiece;
  for (int i0 = piece * kPiece + static_cast<int>(threadIdx.x); i0 < nvec; i0 += pass) {
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
      // 16 bytes per vector: vector i of the run at byte 16 i of its start
      if constexpr (BF16OUT) {
        const u32x4 o{bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16),
                      bf16_rne(v[4]) | (bf16_rne(v[5]) << 16), bf16_rne(v[6]) | (bf16_rne(v[7]) << 16)};
        if (rel)
          sts_at<kStoreNtSc1>(static_cast<uint16_t*>(out) + c.toff, i * 16, o);
        else
          stg_global(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + e), o);
      } else {
        const f32x4 o{v[0], v[1], v[2], v[3]};
        if (rel)
          sts_at<kStoreNtSc1>(static_cast<float*>(out) + c.toff, i * 16, o);
        else
          stg_global(reinterpret_cast<f32x4*>(static_cast<float*>(out) + e), o);
      }
    }
  }
}

template <int FMT, bool HW, bool BF16OUT, int U>
__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(const GatherChunk* __restrict__ chunks,
                                                                    const uint8_t* __restrict__ q,
                                                                    const float* __restrict__ scales,
                                                                    void* const* __restrict__ dst, int split, unsigned n_pieces) {
  for (unsigned p = blockIdx.x; p < n_pieces; p += gridDim.x)
    gather_rows_kernel_piece<FMT, HW, BF16OUT, U>(piece_index<kGatherXcdGroup>(p, n_pieces), chunks, q, scales, dst, split);
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

// Gather side of a tile-major tensor, over the same strips: each lane turns
// VEC codes of one tile row into one 16-byte store of the row-major tensor
// (8 codes -> 8 bf16, 4 -> 4 fp32), kGatherTmVec vectors per thread; tile t
// of the strip uses scale scale0 + t. Stores with nt and sc1 set: 2-3% faster
// cold than nontemporal ones.
template <int FMT, bool HW, bool BF16OUT>
__device__ __forceinline__ void gather_tm_kernel_piece(unsigned b, const TmJob* __restrict__ jobs,
                                                                  const uint8_t* __restrict__ q,
                                                                  const float* __restrict__ scales,
                                                                  void* const* __restrict__ dst, int split) {
  constexpr int VEC = BF16OUT ? 8 : 4;
  constexpr int U = kGatherTmVec;
  const unsigned ju = b / static_cast<unsigned>(split);
  const int ji = static_cast<int>(ju);
  const int piece = static_cast<int>(b - ju * static_cast<unsigned>(split));
  const TmJob j = jobs[ji];
  const uint32_t bc = static_cast<uint32_t>(j.bc), width = static_cast<uint32_t>(j.k) * bc;
  const uint32_t mbc = magic_u16(bc);
  const uint8_t* qb = q + j.base;
  void* out = dst[j.tensor];
  const int pass = split * static_cast<int>(kGatherTmPiece);
  if (bc % VEC == 0 && j.cols % VEC == 0) {
    // vectors in buffer order: tile t's run of h rows of bc codes, row by row
    // (a wave reads contiguous codes; in row order, interleaved on gfx950,
    // 5.59-5.64 against 5.66-5.67 TB/s cold)
    const uint32_t rv = static_cast<uint32_t>(j.h) * bc / VEC, mrv = magic_u16(rv);   // vectors per tile run
    const int nvec = static_cast<int>(j.k * rv);
    for (int i0 = piece * static_cast<int>(kGatherTmPiece) + static_cast<int>(threadIdx.x); i0 < nvec; i0 += pass) {
      uint32_t code[U][VEC / 4];
      float sc[U];
      int64_t dpos[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kGatherThreads;
        if (i < nvec) {
          const uint32_t t = div_u16(static_cast<uint32_t>(i), rv, mrv);
          const uint32_t e = (static_cast<uint32_t>(i) - t * rv) * VEC;
          const uint32_t r = div_u16(e, bc, mbc), c = e - r * bc, col = t * bc + c;
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
          sts<kStoreNtSc1>(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + dpos[u]),
              u32x4{bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16),
                    bf16_rne(v[4]) | (bf16_rne(v[5]) << 16), bf16_rne(v[6]) | (bf16_rne(v[7]) << 16)});
        } else {
          sts<kStoreNtSc1>(reinterpret_cast<f32x4*>(static_cast<float*>(out) + dpos[u]), f32x4{v[0], v[1], v[2], v[3]});
        }
      }
    }
    return;
  }
  // element path: a piece is kGatherTmPiece elements, U per thread
  const int n = j.h * static_cast<int>(width);
  const uint32_t mw = magic_u16(width);
  for (int e0 = piece * static_cast<int>(kGatherTmPiece) + static_cast<int>(threadIdx.x); e0 < n; e0 += pass) {
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
    gather_tm_kernel_piece<FMT, HW, BF16OUT>(piece_index<kGatherXcdGroup>(p, n_pieces), jobs, q, scales, dst, split);
}

}  // namespace
}  // namespace rs

using namespace rs;

namespace {

template <int FMT, bool HW, bool BF16OUT>
void launch_gather(const rs_plan* p, const uint8_t* q, const float* scales, hipStream_t s) {
  const dim3 block(kThreads);
  const QJob* tiles = p->gjobs;
  const QJob* flats = tiles + p->n_gtile;
  if (p->n_gchunks) {
    const int64_t split = BF16OUT ? p->gather_split8 : p->gather_split4;
    const int64_t n = p->n_gchunks * split;
    if (p->gather_vec == kGatherVecShort)
      hipLaunchKernelGGL((gather_rows_kernel<FMT, HW, BF16OUT, kGatherVecShort>), grid_of(p, n), dim3(kGatherThreads), 0,
                         s, p->gchunks, q, scales, p->gdst.dev, static_cast<int>(split), static_cast<unsigned>(n));
    else
      hipLaunchKernelGGL((gather_rows_kernel<FMT, HW, BF16OUT, kGatherVecLong>), grid_of(p, n), dim3(kGatherThreads), 0,
                         s, p->gchunks, q, scales, p->gdst.dev, static_cast<int>(split), static_cast<unsigned>(n));
  }
  if (p->n_gtile)
    hipLaunchKernelGGL((gather_tile_kernel<FMT, HW, BF16OUT>), grid_of(p, p->n_gtile), block, 0, s, tiles, q, scales,
                       p->gdst.dev, static_cast<unsigned>(p->n_gtile));
  if (p->n_gflat)
    hipLaunchKernelGGL((gather_flat_kernel<FMT, HW, BF16OUT>), grid_of(p, p->n_gflat), dim3(kFlatThreads), 0, s, flats, q,
                       scales, p->gdst.dev, static_cast<unsigned>(p->n_gflat));
  if (p->n_tm) {
    const int64_t split = tm_pieces(p->tm_max_strip, BF16OUT ? 8 : 4, kGatherTmPiece);
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
