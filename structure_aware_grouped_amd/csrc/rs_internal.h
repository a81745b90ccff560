// Internal types shared by the host planner, the plan lowering and the HIP
// kernels of the RaggedShard / DBuffer layout library.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include <algorithm>

#include "rs.h"

namespace rs {

// Elements per work item (tuned on gfx950; all multiples of 16 so every item
// starts 16-element aligned when its tensor does). Small items spread the
// streams of the concurrently running workgroups over all HBM channels.
#ifndef RS_UNPACK_CHUNK
#define RS_UNPACK_CHUNK 8192
#endif
#ifndef RS_PACK_CHUNK
#define RS_PACK_CHUNK 4096
#endif
#ifndef RS_ZERO_CHUNK
#define RS_ZERO_CHUNK 65536
#endif
constexpr int64_t kUnpackChunk = RS_UNPACK_CHUNK;   // elements per unpack work item
constexpr int64_t kPackChunk = RS_PACK_CHUNK;       // output elements per pack work item
constexpr int64_t kZeroChunk = RS_ZERO_CHUNK;       // elements per zero-fill work item
static_assert(kUnpackChunk % 16 == 0 && kPackChunk % 16 == 0, "work items keep 16-element alignment");
// The unpack and pack launches split every work item into pieces of
// threads * vec 16-byte vectors, one small workgroup per piece. Short-lived
// workgroups that each move 1-2 KiB keep more independent streams in flight
// across the HBM channels than one 256-thread workgroup per 16 KiB item: on
// gfx950 unpack went from 6.2 to 6.6 TB/s and pack from 6.0 to 6.5 TB/s.
#ifndef RS_UNPACK_THREADS
#define RS_UNPACK_THREADS 64
#endif
#ifndef RS_UNPACK_VEC
#define RS_UNPACK_VEC 1
#endif
#ifndef RS_PACK_THREADS
#define RS_PACK_THREADS 128
#endif
#ifndef RS_PACK_VEC
#define RS_PACK_VEC 1
#endif
// A pack that does not accumulate (one read and one write stream, the shape
// of unpack) is fastest with unpack's shape too: 64 threads, plain
// round-robin over the XCDs. On the Adam-state workload's 1.75 GB packs,
// interleaved and cold: 5.88-5.94 TB/s with the accumulating pack's 128
// threads and runs of 256, 6.04-6.09 with 128 threads round-robin, 6.25-6.28
// with 64 round-robin. The accumulating pack kept its shape: 64 threads
// round-robin gave it +0.5% cold and -2.5% warm on the 8B layer.
#ifndef RS_PACK1_THREADS
#define RS_PACK1_THREADS 64
#endif
constexpr int kUnpackThreads = RS_UNPACK_THREADS, kUnpackVec = RS_UNPACK_VEC;
constexpr int kPackThreads = RS_PACK_THREADS, kPackVec = RS_PACK_VEC;
constexpr int kPack1Threads = RS_PACK1_THREADS;
constexpr int64_t kUnpackPiece = int64_t(kUnpackThreads) * kUnpackVec;   // vectors per workgroup
// pieces per unpack item for element size eb; per pack item (fp32 output) for
// a pack workgroup of nt threads
constexpr int64_t unpack_split(int64_t eb) { return (kUnpackChunk * eb / 16 + kUnpackPiece - 1) / kUnpackPiece; }
constexpr int64_t pack_split(int nt) { return (kPackChunk / 4 + int64_t(nt) * kPackVec - 1) / (int64_t(nt) * kPackVec); }
constexpr int64_t kPackSplit = pack_split(kPackThreads);
constexpr int64_t kPack1Split = pack_split(kPack1Threads);
// Consecutive pieces of a split launch kept on one XCD (1: plain round-robin).
// Pack, with three streams, gains from runs of 256 pieces (512 KiB of output)
// per XCD: 6.52 -> 6.67 TB/s on the Llama-3-8B layer, 5.97 -> 6.59 TB/s on the
// 55 GB MoE layer. Unpack is fastest with plain round-robin; the row-run
// gather of the MoE layer gains 7% from runs of 128, and the tile-major gather
// of the 8B layer 6% (5.72 -> 6.09 TB/s; each strip's two pieces then read its
// job and scales from one L2).
#ifndef RS_UNPACK_XCD_GROUP
#define RS_UNPACK_XCD_GROUP 1
#endif
#ifndef RS_PACK_XCD_GROUP
#define RS_PACK_XCD_GROUP 256
#endif
#ifndef RS_PACK1_XCD_GROUP
#define RS_PACK1_XCD_GROUP 1
#endif
#ifndef RS_GATHER_XCD_GROUP
#define RS_GATHER_XCD_GROUP 128
#endif
constexpr unsigned kUnpackXcdGroup = RS_UNPACK_XCD_GROUP;
constexpr unsigned kPackXcdGroup = RS_PACK_XCD_GROUP;
constexpr unsigned kPack1XcdGroup = RS_PACK1_XCD_GROUP;   // pack without accumulation
constexpr unsigned kGatherXcdGroup = RS_GATHER_XCD_GROUP;
// the same for the per-block kernels (quant, dequant, Adam): consecutive tiles
// per XCD (4: tile quant 5.98 -> 6.32 TB/s on the 8B layer), consecutive
// flat-block groups per XCD (1: grouping slowed the Adam-state kernels)
#ifndef RS_TILE_XCD_GROUP
#define RS_TILE_XCD_GROUP 4
#endif
#ifndef RS_FLAT_XCD_GROUP
#define RS_FLAT_XCD_GROUP 1
#endif
// Tile quant of a plan whose code rows share 128-byte lines between
// neighbouring tiles (a TILE tensor whose start, width or tile width is not a
// multiple of 128 codes, such as the MoE layer's 2880-wide tensors). Such
// tensors quantise slower: 128x128 tiles of bf16 ran at 5.6 TB/s on
// 2880-wide tensors, 6.1 on 2944-wide and 6.3 on 4096-wide. Longer runs of
// consecutive tiles per XCD recover part of it, on measurement rather than a
// model (the write counter did not fall): on the MoE layer 5.50 TB/s at 4,
// 5.65 at 32, 5.75 at 64 and 128, 5.70 at 256.
#ifndef RS_TILE_XCD_GROUP_SPLIT
#define RS_TILE_XCD_GROUP_SPLIT 64
#endif
constexpr unsigned kTileXcdGroup = RS_TILE_XCD_GROUP;
constexpr unsigned kTileXcdGroupSplit = RS_TILE_XCD_GROUP_SPLIT;
constexpr unsigned kFlatXcdGroup = RS_FLAT_XCD_GROUP;
// Threads per tile in the tile quant kernel.
#ifndef RS_QUANT_THREADS
#define RS_QUANT_THREADS 512
#endif
constexpr int kQuantThreads = RS_QUANT_THREADS;
static_assert(kQuantThreads % 64 == 0 && 2048 % kQuantThreads == 0, "tile quant thread count");
// Split launches use at most kMaxGrid workgroups and loop over further pieces
// (a multiple of 8: one round of the XCD dispatch).
constexpr int64_t kMaxGrid = int64_t(1) << 24;
// Largest materialised buffer, R_mat * S elements (4 TiB of fp32, far beyond
// one device); it keeps every work-item index within 32 bits.
constexpr int64_t kMaxElems = int64_t(1) << 39;
// Flat quantisation blocks per workgroup, one 64-lane wave each.
#ifndef RS_FLAT_PER_GROUP
#define RS_FLAT_PER_GROUP 2
#endif
constexpr int kFlatPerGroup = RS_FLAT_PER_GROUP;
constexpr int kFlatThreads = kFlatPerGroup * 64;

// One tensor of a loaded plan.
struct Tensor {
  int64_t rows, cols, n, g, start;
  int64_t p0, p1;
  int32_t kind;
};

// Unpack work item: `len` consecutive elements of one tensor.
struct CopyChunk {
  int64_t src;      // element offset in the flat buffer
  int64_t off;      // element offset inside the tensor
  int32_t len;      // elements
  int32_t tensor;
};

// Pack work item: an aligned run of the flat output. The first n_data
// elements come from tensor `tensor` (starting at its element `off`); the
// remaining n_total - n_data elements are padding. tensor < 0: all padding.
struct PackChunk {
  int64_t out;      // element offset in the flat buffer (multiple of 16)
  int64_t off;
  int32_t n_total;  // multiple of 16
  int32_t n_data;
  int32_t tensor;
  int32_t unused;
};

enum QJobKind : int32_t { QJOB_TILE = 0, QJOB_FLAT = 1, QJOB_ZERO = 2 };

// Quant / dequant work item.
//   TILE: one tile: element (r, c) sits at base + r*stride + c, r < rows, c < cols.
//   FLAT: `rows` (1..kFlatPerGroup) consecutive flat blocks of `cols` elements
//         from base; the last one has `last` elements. Scales scale..scale+rows-1.
//   ZERO: elements [base, base + stride) lie in no block (codes 0, values +0.0).
// TILE and FLAT jobs also name their tensor and where the block's element
// (0, 0) sits in the full row-major tensor (toff) with the tensor's row
// stride (tstride), for kernels that write the full tensors. For a
// row-major tensor toff = base - s_tensor and tstride = stride; a TILEMAJOR
// tile has stride = bc in the buffer but tstride = cols in the tensor.
struct QJob {
  int64_t base;
  int64_t stride;
  int64_t scale;
  int64_t toff;
  int64_t tstride;
  int32_t rows;
  int32_t cols;
  int32_t kind;
  int32_t last;
  int32_t tensor;
  int32_t unused;
};

// Tile-major reorder work item: rows [r0, r0 + h) of tiles tc0 .. tc0 + k - 1
// of tile row tr of a TILEMAJOR tensor, staged through LDS. In the buffer
// those are k runs of h*bc elements (one per tile, tile_elems apart) from
// `base`; in the row-major tensor, h rows of k*bc elements from `toff`.
struct TmJob {
  int64_t base;        // flat position of row r0 of tile (tr, tc0)
  int64_t toff;        // row-major offset of element (tr*br + r0, tc0*bc)
  int64_t cols;        // tensor columns (row stride of the tensor)
  int64_t tile_elems;  // br * bc
  int64_t scale0;      // scale index of tile (tr, tc0); tile t of the job uses scale0 + t
  int32_t tensor;
  int32_t k;
  int32_t h;
  int32_t bc;
};

#ifndef RS_TM_STRIP
#define RS_TM_STRIP 2048
#endif
#ifndef RS_TM_ROWS
#define RS_TM_ROWS 2
#endif
#ifndef RS_TM_LDS_THREADS
#define RS_TM_LDS_THREADS 128
#endif
// A tile-major job is a strip of up to kTmRows rows of consecutive tiles of
// one tile row, about kTmStrip elements; a single row of the widest allowed
// tile (8192 columns) is the largest strip.
constexpr int64_t kTmStrip = RS_TM_STRIP;
constexpr int64_t kTmStage = 8192;          // largest strip, in elements
constexpr int64_t kTmRows = RS_TM_ROWS;
constexpr int kTmLdsThreads = RS_TM_LDS_THREADS;
static_assert(kTmStrip <= kTmStage && kTmStage <= 16384, "tile-major strips: indices stay under 2^16");
// Tile-major reorder: staged through LDS (one kTmLdsThreads workgroup per
// strip; the default) or direct (each lane maps its own 16-byte vector between
// the two layouts, on small split workgroups; RS_TM_KERNEL=direct at
// rs_plan_load). Both give the same results.
#ifndef RS_TM_THREADS
#define RS_TM_THREADS 64
#endif
constexpr int kTmThreads = RS_TM_THREADS;
// pieces per job for vectors of vec elements (direct kernels)
// pieces per job: the plan's largest strip in vectors of vec elements, per_piece vectors each
inline int64_t tm_pieces(int64_t max_strip, int64_t vec, int64_t per_piece) {
  return std::max<int64_t>(1, (max_strip / vec + per_piece - 1) / per_piece);
}

// Gather-side work item: a contiguous run of whole rows of one quantised
// tensor, inside one band of tiles (TILE) or made of whole flat blocks (FLAT,
// a "row" being one block). Element (r, c) of the run sits at r*cols + c and
// its scale is scales[scale0 + r*rstep + c/bc]. Only tensors whose rows and
// tile widths are multiples of 16 elements (TILE: at most kGatherMaxCols
// columns) or whose flat blocks are, use these.
struct GatherChunk {
  int64_t qbase;   // flat position of the first element
  int64_t toff;    // the same element's offset inside the tensor
  int64_t scale0;
  int32_t rows;
  int32_t cols;    // a multiple of 8
  int32_t bc;      // width sharing one scale: tile columns, or the flat block
  int32_t rstep;   // 0: every row of the run shares the band's scales; 1: one block per row
  int32_t tensor;
  int32_t unused;
};

// A gather run is split over `split` workgroups of gather_piece(vec) vectors, the
// same number for every run of a launch, so a run shorter than the longest
// leaves workgroups idle. The lowering therefore picks one target length for
// the whole plan, P pieces of gather_piece(vec) * 8 codes with P in
// [kGatherMinPieces, kGatherMaxPieces], that launches the fewest workgroups:
// on the MoE layer (2880-wide rows, 128-row bands) 16-row runs of exactly 45
// pieces ran the gather at 6.28 TB/s, against 5.79 for runs of about 16K codes.
// Runs of at least 48 pieces (P from 48 instead of 8) were faster again, in
// eight interleaved pairs: the MoE layer 6.59 -> 6.68 TB/s (22-row runs), the
// 8B layer 5.86 -> 5.94 (14-row runs, 4-row runs of the 14336-wide tensor,
// 56 pieces each, where P from 8 gave 28-piece runs).
constexpr int64_t kGatherMinPieces = 48;
constexpr int64_t kGatherMaxPieces = 64;
constexpr int64_t kGatherMaxCols = 16384;           // widest TILE tensor handled as row runs
// Gather runs are split like unpack items: kGatherThreads threads of `vec`
// vectors each per workgroup, vec chosen per plan. A short launch (a row-run
// gather of fewer than kGatherShortElems elements, a few hundred µs) takes 4
// vectors per thread, half the workgroups; a longer one 2. Measured cold,
// three interleaved rounds: 4 against 2 vectors gave +2.3% on 0.2G elements
// of 2880-wide rows and +1-5% on 0.18G of 4096-wide rows (and +3-7% on the
// 8B layer's 0.22G), the same on 0.8G of 2880-wide rows, -2% on 2.8G of
// 4096-wide rows and -8% on the MoE layer's 3.2G: what decides is the
// length of the launch, not the row width. RS_GATHER_VEC=2|4 forces one.
#ifndef RS_GATHER_THREADS
#define RS_GATHER_THREADS 64
#endif
constexpr int kGatherThreads = RS_GATHER_THREADS;
constexpr int kGatherVecShort = 4, kGatherVecLong = 2;
constexpr int64_t kGatherShortElems = int64_t(1) << 29;
constexpr int64_t gather_piece(int vec) { return int64_t(kGatherThreads) * vec; }   // vectors per workgroup
// The gather side of tile-major strips takes 8 vectors per thread: on the 8B
// layer stored tile-major, cold, 4 against 2 gave 5.38-5.42 -> 5.62-5.64 TB/s
// and, with nt-sc1 stores, 8 against 4 5.74-5.79 -> 5.85-6.05 in three
// interleaved rounds (warm 2-3% slower). With 128x128 tiles a bf16 strip is
// 256 vectors, one workgroup either way; an fp32 strip takes one instead of two.
#ifndef RS_GATHER_TM_VEC
#define RS_GATHER_TM_VEC 8
#endif
constexpr int kGatherTmVec = RS_GATHER_TM_VEC;
constexpr int64_t kGatherTmPiece = int64_t(kGatherThreads) * kGatherTmVec;
// the longest run: kGatherMaxPieces pieces of 8-code vectors (of the larger
// piece), or one row of kGatherMaxCols codes; as 4-code vectors its indices
// stay under 2^16
constexpr int64_t kGatherMaxRun =
    std::max<int64_t>(kGatherMaxPieces * gather_piece(kGatherVecShort) * 8, kGatherMaxCols);
static_assert(kGatherMaxRun / 4 < 65536, "a run of several rows keeps its vector indices under 2^16");


// Device copy of a per-tensor pointer table plus the host state that decides
// when it must be uploaded again.
struct PtrTable {
  void** dev = nullptr;          // n device-side pointers (inside the plan's allocation)
  void** stage = nullptr;        // pinned host staging for the upload
  hipEvent_t done = nullptr;     // recorded after the last upload from `stage`
  std::vector<const void*> seen; // pointers of the last upload
  bool valid = false;
  bool pending = false;
};

// Granularity and spec checks shared by the planner and the loader.
int64_t granularity(const rs_tensor_spec& s);
bool spec_ok(const rs_tensor_spec& s, std::string* why);

// Checks a plan (the arguments of rs_plan_load) against the layout
// constraints and fills the tensor table; returns an rs_status, with a
// message that starts with `who` (the entry point called).
int validate_plan(const char* who, const rs_tensor_spec* specs, int64_t n, int64_t V, int64_t S,
                  const int64_t* starts, int64_t R_mat, std::vector<Tensor>* out, int64_t* R_used);

// The Adam step takes tile jobs in groups of kAdamStripTiles; a group of four
// 32x32 tiles side by side in one band of one tensor (codes 16-byte aligned)
// is a 32 x 128 strip whose code rows are whole 128-byte runs.
constexpr int kAdamStripTiles = 4, kAdamStripRows = 32, kAdamStripTileCols = 32;

// The block quant / dequant work list of a validated plan.
struct QuantList {
  std::vector<QJob> jobs;   // tiles, then flat groups, then zero ranges
  int64_t n_tile = 0, n_flat = 0, n_zero = 0, n_blocks = 0;
  int32_t max_tile_vec16 = 0;     // largest tile, in 16-byte vectors of 4-byte input
  bool split_code_lines = false;  // neighbouring tiles share 128-byte lines of codes
  bool all_strips = false;        // the tile jobs are whole Adam strips, group after group
};
void lower_quant(const std::vector<Tensor>& t, int64_t top, QuantList* ql);

// Thread-local error reporting: record a message, return the status.
int fail(int status, const std::string& msg);
void clear_error();

}  // namespace rs

struct rs_plan {
  int device = 0;
  int64_t V = 0, S = 0, R_mat = 0, R_used = 0, n = 0, padding = 0;
  std::vector<rs::Tensor> t;

  void* dmem = nullptr;  // one device allocation holding every table below
  rs::CopyChunk* unpack = nullptr;
  int64_t n_unpack = 0;
  rs::PackChunk* pack = nullptr;
  int64_t n_pack = 0;
  rs::QJob* qjobs = nullptr;   // tile jobs, then flat-group jobs, then zero ranges
  int64_t n_qjobs = 0;
  int64_t n_qtile = 0, n_qflat = 0, n_qzero = 0;
  int64_t n_qblocks = 0;
  int32_t max_tile_vec16 = 0;  // largest tile (TILE or TILEMAJOR), in 16-byte vectors of 4-byte input
  bool split_code_lines = false;  // neighbouring tiles share 128-byte lines of codes
  int gather_vec = rs::kGatherVecLong;   // vectors per thread of the row-run gather
  int64_t gather_split8 = 0;      // workgroups per gather run, 8 codes per vector (bf16 out)
  int64_t gather_split4 = 0;      // the same, 4 codes per vector (fp32 out)

  rs::TmJob* tmjobs = nullptr;         // unpack / pack of TILEMAJOR tensors
  int64_t n_tm = 0;
  rs::GatherChunk* gchunks = nullptr;  // gather side, vector-friendly tensors
  int64_t n_gchunks = 0;
  rs::QJob* gjobs = nullptr;           // gather side, other tensors: tile jobs, then flat groups
  int64_t n_gtile = 0, n_gflat = 0;

  rs::PtrTable dst;   // unpack destinations
  rs::PtrTable src;   // pack sources
  rs::PtrTable gdst;  // unpack-dequant destinations
  bool e4m3_hw = false;  // use gfx950's FP8 conversion instructions
  int64_t tm_max_strip = 0;    // elements of the largest tile-major job (LDS stage, piece count)
  bool tm_unpack_lds = true;   // tile-major unpack staged through LDS (else the direct kernel)
  bool tm_pack_lds = true;     // tile-major pack staged through LDS (else the direct kernel)
  int64_t max_grid = rs::kMaxGrid;   // workgroups per launch; beyond it workgroups loop over items
  bool adam_wave_tiles = true;       // Adam step: one wave per tile when every tile fits one wave's registers
  bool adam_all_strips = false;      // Adam step: every group of kAdamStripTiles tile jobs is a strip
};
