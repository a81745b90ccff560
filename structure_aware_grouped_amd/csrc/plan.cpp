// Plan validation and lowering: a plan (specs, V, S, starts, R_mat) becomes
// device work lists for unpack, pack and block quant / dequant, built once
// and kept for the plan's lifetime (the DBuffer's persistent per-tensor
// address mapping: "veScale-FSDP: flexible, structure-aware sharding at
// 10K-GPU scale", feynmanwiki walkthrough, DBuffer paragraphs).
#include <algorithm>
#include <cassert>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "rs_internal.h"

namespace rs {

namespace {
thread_local std::string g_error;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Tables {
  std::vector<TmJob> tm;
  std::vector<CopyChunk> unpack;
  std::vector<PackChunk> pack;
  std::vector<QJob> qjobs;          // sorted by kind: tiles, flat groups, zero ranges
  int64_t n_qtile = 0, n_qflat = 0, n_qzero = 0;
  int64_t tm_max_strip = 0;
  std::vector<GatherChunk> gchunks;
  std::vector<QJob> gjobs;          // tiles, then flat groups
  int64_t n_gtile = 0, n_gflat = 0;
  int64_t n_qblocks = 0;
  int64_t padding = 0;
  int32_t max_tile_vec16 = 0;
  bool split_code_lines = false;
  bool adam_all_strips = false;
  int gather_vec = kGatherVecLong;
  int64_t gather_split8 = 0, gather_split4 = 0;
};

// Gather runs of one tensor: `unit` codes per row (TILE) or per flat block
// (FLAT), grouped into bands of `band` units (`n_full` full bands and one of
// `last` units if last > 0) that no run crosses.
struct RunGroups {
  int64_t unit, band, n_full, last;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Units per run for a target of P pieces of pc codes.
int64_t run_units(const RunGroups& g, int64_t P, int64_t pc) {
  return std::max<int64_t>(1, std::min<int64_t>(g.band, P * pc / g.unit));
}

// Runs and the largest run (in pieces of pc codes) of a tensor for `per` units per run.
void run_stats(const RunGroups& g, int64_t per, int64_t pc, int64_t* runs, int64_t* max_pieces) {
  auto band_runs = [&](int64_t units) {
    if (units <= 0) return;
    *runs += ceil_div(units, per);
    *max_pieces = std::max(*max_pieces, ceil_div(std::min(per, units) * g.unit, pc));
  };
  if (g.n_full > 0) {
    *runs += ceil_div(g.band, per) * (g.n_full - 1);   // band_runs adds the last full band
    band_runs(g.band);
  }
  band_runs(g.last);
}

// Target pieces per run for the whole plan: the one that launches the fewest
// workgroups (runs x the largest run), the longer target on ties.
int64_t pick_run_pieces(const std::vector<RunGroups>& gs, int64_t pc) {
  int64_t best_P = kGatherMinPieces, best = -1;
  for (int64_t P = kGatherMinPieces; P <= kGatherMaxPieces; ++P) {
    int64_t runs = 0, maxp = 0;
    for (const RunGroups& g : gs) run_stats(g, run_units(g, P, pc), pc, &runs, &maxp);
    const int64_t cost = runs * maxp;
    if (best < 0 || cost <= best) {
      best = cost;
      best_P = P;
    }
  }
  return best_P;
}

void lower(const std::vector<Tensor>& t, int64_t S, int64_t R_mat, Tables* tb) {
  const int64_t top = R_mat * S;
  const int64_t n = static_cast<int64_t>(t.size());

  // first scale index of every tensor (tensors in order; tiles row-major, flat blocks in order)
  std::vector<int64_t> first_scale(n + 1, 0);
  for (int64_t i = 0; i < n; ++i) {
    const Tensor& x = t[i];
    int64_t nb = 0;
    if (x.kind == RS_TILE) nb = ((x.rows + x.p0 - 1) / x.p0) * ((x.cols + x.p1 - 1) / x.p1);
    else if (x.kind == RS_TILEMAJOR) nb = x.n / (x.p0 * x.p1);
    else if (x.kind == RS_FLAT) nb = (x.n + x.p0 - 1) / x.p0;
    first_scale[i + 1] = first_scale[i] + nb;
  }

  // unpack: every row-major tensor in chunks; TILEMAJOR tensors in strips of
  // rows across up to k tiles of one tile row (unpack, pack and the gather side
  // share them)
  for (int64_t i = 0; i < n; ++i) {
    const Tensor& x = t[i];
    if (x.kind == RS_TILEMAJOR) {
      const int64_t br = x.p0, bc = x.p1, ntc = x.cols / bc;
      const int64_t h = std::min<int64_t>(br, std::max<int64_t>(1, std::min<int64_t>(kTmRows, kTmStrip / bc)));
      const int64_t k = std::max<int64_t>(1, std::min(ntc, kTmStrip / (h * bc)));
      tb->tm_max_strip = std::max(tb->tm_max_strip, h * k * bc);   // <= max(kTmStrip, bc) <= kTmStage
      for (int64_t tr = 0; tr < x.rows / br; ++tr)
        for (int64_t tc0 = 0; tc0 < ntc; tc0 += k)
          for (int64_t r0 = 0; r0 < br; r0 += h) {
            TmJob j{};
            j.base = x.start + (tr * ntc + tc0) * br * bc + r0 * bc;
            j.toff = (tr * br + r0) * x.cols + tc0 * bc;
            j.cols = x.cols;
            j.tile_elems = br * bc;
            j.scale0 = first_scale[i] + tr * ntc + tc0;
            j.tensor = static_cast<int32_t>(i);
            j.k = static_cast<int32_t>(std::min(k, ntc - tc0));
            j.h = static_cast<int32_t>(std::min(h, br - r0));
            j.bc = static_cast<int32_t>(bc);
            tb->tm.push_back(j);
          }
      continue;
    }
    for (int64_t off = 0; off < x.n; off += kUnpackChunk)
      tb->unpack.push_back({x.start + off, off, static_cast<int32_t>(std::min(kUnpackChunk, x.n - off)),
                            static_cast<int32_t>(i)});
  }

  // pack: walk the buffer in address order; data chunks own the padding up
  // to the next 16-element boundary after their tensor ends
  std::vector<int64_t> by_start(n);
  for (int64_t i = 0; i < n; ++i) by_start[i] = i;
  std::sort(by_start.begin(), by_start.end(), [&](int64_t a, int64_t b) { return t[a].start < t[b].start; });
  auto pad = [&](int64_t from, int64_t to) {
    for (int64_t p = from; p < to; p += kPackChunk)
      tb->pack.push_back({p, 0, static_cast<int32_t>(std::min(kPackChunk, to - p)), 0, -1, 0});
  };
  int64_t pos = 0;
  for (int64_t k : by_start) {
    const Tensor& x = t[k];
    pad(pos, x.start);
    const int64_t end16 = align_up(x.start + x.n, 16);
    if (x.kind == RS_TILEMAJOR) {   // packed by the tile-major jobs; n is a multiple of 16
      pos = end16;
      continue;
    }
    for (int64_t off = 0; off < x.n; off += kPackChunk) {
      const int64_t n_data = std::min(kPackChunk, x.n - off);
      const int64_t n_total = (off + kPackChunk >= x.n) ? end16 - (x.start + off) : n_data;
      tb->pack.push_back({x.start + off, off, static_cast<int32_t>(n_total),
                          static_cast<int32_t>(n_data), static_cast<int32_t>(k), 0});
    }
    pos = end16;
  }
  pad(pos, top);

  int64_t covered = 0;
  for (const Tensor& x : t) covered += x.n;
  tb->padding = top - covered;

  // quant / dequant: tiles and flat blocks in scale order, then zero ranges
  QuantList ql;
  lower_quant(t, top, &ql);
  tb->qjobs = std::move(ql.jobs);
  tb->n_qtile = ql.n_tile;
  tb->n_qflat = ql.n_flat;
  tb->n_qzero = ql.n_zero;
  tb->n_qblocks = ql.n_blocks;
  tb->max_tile_vec16 = ql.max_tile_vec16;
  tb->split_code_lines = ql.split_code_lines;
  tb->adam_all_strips = ql.all_strips;
  assert(tb->n_qblocks == first_scale[n]);

  // gather side: contiguous row runs where every 16-element vector has one
  // scale; per-block jobs (as for quant) for everything else
  std::vector<char> tile_vec(n, 0);
  for (int64_t ti = 0; ti < n; ++ti)
    tile_vec[ti] = t[ti].kind == RS_TILE && t[ti].cols % 16 == 0 && t[ti].p1 % 16 == 0 &&
                   t[ti].cols <= kGatherMaxCols;
  for (const QJob& j : tb->qjobs)
    if (j.kind == QJOB_TILE && !tile_vec[j.tensor] && t[j.tensor].kind != RS_TILEMAJOR)
      tb->gjobs.push_back(j);   // TILEMAJOR tensors use the tile-major strips
  // vectors per thread, from the length of the launch (rs_internal.h) unless
  // RS_GATHER_VEC=2|4 forces it; then one run length for the plan (8-code
  // pieces: gather_piece(vec) vectors of 8 codes)
  int64_t run_elems = 0;
  for (int64_t ti = 0; ti < n; ++ti) {
    const Tensor& x = t[ti];
    if (x.kind == RS_TILE && tile_vec[ti]) run_elems += x.n;
    else if (x.kind == RS_FLAT && x.p0 % 16 == 0) run_elems += (x.n / x.p0) * x.p0;
  }
  tb->gather_vec = run_elems < kGatherShortElems ? kGatherVecShort : kGatherVecLong;
  if (const char* gv = std::getenv("RS_GATHER_VEC")) {
    const int f = std::atoi(gv);
    if (f == kGatherVecShort || f == kGatherVecLong) tb->gather_vec = f;
  }
  const int64_t pc8 = gather_piece(tb->gather_vec) * 8;
  std::vector<RunGroups> groups(n, RunGroups{0, 0, 0, 0});
  std::vector<RunGroups> used;
  for (int64_t ti = 0; ti < n; ++ti) {
    const Tensor& x = t[ti];
    if (x.kind == RS_TILE && tile_vec[ti]) groups[ti] = {x.cols, x.p0, x.rows / x.p0, x.rows % x.p0};
    else if (x.kind == RS_FLAT && x.p0 % 16 == 0 && x.n / x.p0 > 0) groups[ti] = {x.p0, x.n / x.p0, 1, 0};
    if (groups[ti].unit) used.push_back(groups[ti]);
  }
  const int64_t P = pick_run_pieces(used, pc8);
  int64_t q = 0;
  {
    int64_t runs = 0, m8 = 0, m4 = 0;
    for (const RunGroups& g : used) {
      run_stats(g, run_units(g, P, pc8), pc8, &runs, &m8);
      run_stats(g, run_units(g, P, pc8), pc8 / 2, &runs, &m4);
    }
    tb->gather_split8 = m8;
    tb->gather_split4 = m4;
  }
  for (int64_t ti = 0; ti < n; ++ti) {
    const Tensor& x = t[ti];
    if (x.kind == RS_TILE) {
      const int64_t ntc = (x.cols + x.p1 - 1) / x.p1;
      if (tile_vec[ti]) {
        const int64_t per = run_units(groups[ti], P, pc8);
        for (int64_t r0 = 0; r0 < x.rows; r0 += x.p0) {
          const int64_t band_end = std::min(x.rows, r0 + x.p0);
          for (int64_t r = r0; r < band_end; r += per) {
            GatherChunk c{};
            c.qbase = x.start + r * x.cols;
            c.toff = r * x.cols;
            c.scale0 = q + (r0 / x.p0) * ntc;
            c.rows = static_cast<int32_t>(std::min(per, band_end - r));
            c.cols = static_cast<int32_t>(x.cols);
            c.bc = static_cast<int32_t>(x.p1);
            c.rstep = 0;
            c.tensor = static_cast<int32_t>(ti);
            tb->gchunks.push_back(c);
          }
        }
      }
      q += ((x.rows + x.p0 - 1) / x.p0) * ntc;
    } else if (x.kind == RS_TILEMAJOR) {
      q += x.n / (x.p0 * x.p1);
    } else if (x.kind == RS_FLAT) {
      const int64_t nfull = x.n / x.p0;            // whole blocks
      int64_t done = 0;
      if (groups[ti].unit) {
        const int64_t per = run_units(groups[ti], P, pc8);
        for (; done < nfull; done += per) {
          GatherChunk c{};
          c.qbase = x.start + done * x.p0;
          c.toff = done * x.p0;
          c.scale0 = q + done;
          c.rows = static_cast<int32_t>(std::min(per, nfull - done));
          c.cols = static_cast<int32_t>(x.p0);
          c.bc = static_cast<int32_t>(x.p0);
          c.rstep = 1;
          c.tensor = static_cast<int32_t>(ti);
          tb->gchunks.push_back(c);
        }
        done = nfull;
      }
      // remaining blocks (all of them, or the partial last one) as flat groups
      const int64_t nblk = (x.n + x.p0 - 1) / x.p0;
      for (int64_t b0 = done; b0 < nblk; b0 += kFlatPerGroup) {
        const int64_t cnt = std::min<int64_t>(kFlatPerGroup, nblk - b0);
        QJob j{};
        j.base = x.start + b0 * x.p0;
        j.stride = x.p0;
        j.scale = q + b0;
        j.rows = static_cast<int32_t>(cnt);
        j.cols = static_cast<int32_t>(x.p0);
        j.kind = QJOB_FLAT;
        j.last = static_cast<int32_t>(std::min(x.p0, x.n - (b0 + cnt - 1) * x.p0));
        j.tensor = static_cast<int32_t>(ti);
        j.toff = j.base - x.start;
        j.tstride = x.p0;
        tb->gjobs.push_back(j);
      }
      q += nblk;
    }
  }
  std::stable_sort(tb->gjobs.begin(), tb->gjobs.end(),
                   [](const QJob& a, const QJob& b) { return a.kind < b.kind; });
  for (const QJob& j : tb->gjobs) (j.kind == QJOB_TILE ? tb->n_gtile : tb->n_gflat)++;
}

template <typename T>
T* carve(char*& p, int64_t count) {
  T* out = reinterpret_cast<T*>(p);
  p += align_up(static_cast<int64_t>(sizeof(T)) * std::max<int64_t>(count, 1), 256);
  return out;
}

}  // namespace

int fail(int status, const std::string& msg) {
  g_error = msg;
  return status;
}

void clear_error() { g_error.clear(); }

// Checks a plan against the constraints; fills the tensor table. Messages
// start with `who`, the entry point that was called.
int validate_plan(const char* who, const rs_tensor_spec* specs, int64_t n, int64_t V, int64_t S,
                  const int64_t* starts, int64_t R_mat, std::vector<Tensor>* out, int64_t* R_used) {
  const std::string w = who;
  if (!specs || !starts) return fail(RS_EINVAL, w + ": null specs or starts");
  if (n < 1 || n > (int64_t(1) << 31)) return fail(RS_EINVAL, w + ": bad tensor count");
  if (V < 1) return fail(RS_EINVAL, w + ": V must be >= 1");
  if (S <= 0) return fail(RS_EINVAL, w + ": S must be > 0");
  if (S % 16 != 0) return fail(RS_EALIGN, w + ": S must be a multiple of 16");
  const int64_t kLimit = int64_t(1) << 62;
  if (V > kLimit / S) return fail(RS_ERANGE, w + ": V * S overflows");
  const int64_t total = V * S;

  out->resize(n);
  std::vector<std::pair<int64_t, int64_t>> iv(n);
  int64_t max_end = 0;
  for (int64_t i = 0; i < n; ++i) {
    std::string why;
    if (!spec_ok(specs[i], &why))
      return fail(RS_EINVAL, w + ": tensor " + std::to_string(i) + ": " + why);
    Tensor& t = (*out)[i];
    t.rows = specs[i].rows;
    t.cols = specs[i].cols;
    t.n = t.rows * t.cols;
    t.g = granularity(specs[i]);
    t.kind = specs[i].kind;
    t.p0 = specs[i].p0;
    t.p1 = specs[i].p1;
    t.start = starts[i];
    const std::string tag = w + ": tensor " + std::to_string(i);
    if (t.start % 16 != 0) return fail(RS_EALIGN, tag + ": start not a multiple of 16");
    if (t.start < 0 || t.start > total - t.n)
      return fail(RS_EPLAN, tag + ": interval outside [0, V*S)");
    // rank boundaries strictly inside the tensor: the first one at b, then every S
    const int64_t b = (t.start / S + 1) * S;
    if (b < t.start + t.n) {
      if ((b - t.start) % t.g != 0) return fail(RS_EPLAN, tag + ": a rank boundary cuts an atomic block");
      if (b + S < t.start + t.n && S % t.g != 0)
        return fail(RS_EPLAN, tag + ": a rank boundary cuts an atomic block");
    }
    iv[i] = {t.start, t.start + t.n};
    max_end = std::max(max_end, t.start + t.n);
  }
  std::sort(iv.begin(), iv.end());
  for (int64_t i = 1; i < n; ++i)
    if (iv[i].first < iv[i - 1].second) return fail(RS_EPLAN, w + ": tensors overlap");
  *R_used = (max_end + S - 1) / S;
  if (R_mat < *R_used || R_mat > V)
    return fail(RS_ERANGE, w + ": R_mat must lie in [R_used, V] (R_used = " +
                               std::to_string(*R_used) + ")");
  if (R_mat > kMaxElems / S)
    return fail(RS_ERANGE, w + ": R_mat * S exceeds 2^39 elements, more than one device holds");
  return RS_OK;
}

// Quant / dequant work list of a validated plan over [0, top): one job per
// tile (TILE: a br x bc tile of the row-major tensor, partial at the edges;
// TILEMAJOR: one contiguous tile) and per group of up to kFlatPerGroup flat
// blocks, in scale order (tensors in spec order, tiles row-major), then
// zero-range jobs for every position outside all blocks; the list is sorted
// by job kind (stable), so each kind is one contiguous run for its kernel.
void lower_quant(const std::vector<Tensor>& t, int64_t top, QuantList* ql) {
  const int64_t n = static_cast<int64_t>(t.size());
  int64_t q = 0;
  for (int64_t ti = 0; ti < n; ++ti) {
    const Tensor& x = t[ti];
    if (x.kind == RS_TILE) {
      // a code row of one tile then starts or ends inside a 128-byte line that
      // the tile next to it also writes
      if (x.cols > x.p1 && ((x.start | x.cols | x.p1) & 127) != 0) ql->split_code_lines = true;
      for (int64_t r0 = 0; r0 < x.rows; r0 += x.p0) {
        for (int64_t c0 = 0; c0 < x.cols; c0 += x.p1) {
          QJob j{};
          j.base = x.start + r0 * x.cols + c0;
          j.stride = x.cols;
          j.scale = q++;
          j.rows = static_cast<int32_t>(std::min(x.p0, x.rows - r0));
          j.cols = static_cast<int32_t>(std::min(x.p1, x.cols - c0));
          j.kind = QJOB_TILE;
          j.last = 0;
          j.tensor = static_cast<int32_t>(ti);
          j.toff = j.base - x.start;
          j.tstride = x.cols;
          ql->jobs.push_back(j);
          const int64_t v16 = int64_t(j.rows) * ((int64_t(j.cols) * 4 + 15) / 16);
          ql->max_tile_vec16 = static_cast<int32_t>(std::max<int64_t>(ql->max_tile_vec16, std::min<int64_t>(v16, 1 << 30)));
        }
      }
    } else if (x.kind == RS_TILEMAJOR) {
      const int64_t br = x.p0, bc = x.p1, ntc = x.cols / bc;
      for (int64_t tr = 0; tr < x.rows / br; ++tr) {
        for (int64_t tc = 0; tc < ntc; ++tc) {
          QJob j{};
          j.base = x.start + (tr * ntc + tc) * br * bc;   // the tile is contiguous
          j.stride = bc;
          j.scale = q++;
          j.rows = static_cast<int32_t>(br);
          j.cols = static_cast<int32_t>(bc);
          j.kind = QJOB_TILE;
          j.last = 0;
          j.tensor = static_cast<int32_t>(ti);
          j.toff = tr * br * x.cols + tc * bc;
          j.tstride = x.cols;
          ql->jobs.push_back(j);
        }
      }
      const int64_t v16 = br * ((bc * 4 + 15) / 16);
      ql->max_tile_vec16 = static_cast<int32_t>(std::max<int64_t>(ql->max_tile_vec16, std::min<int64_t>(v16, 1 << 30)));
    } else if (x.kind == RS_FLAT) {
      const int64_t nblk = (x.n + x.p0 - 1) / x.p0;
      for (int64_t b0 = 0; b0 < nblk; b0 += kFlatPerGroup) {
        const int64_t cnt = std::min<int64_t>(kFlatPerGroup, nblk - b0);
        QJob j{};
        j.base = x.start + b0 * x.p0;
        j.stride = x.p0;
        j.scale = q;
        j.rows = static_cast<int32_t>(cnt);
        j.cols = static_cast<int32_t>(x.p0);
        j.kind = QJOB_FLAT;
        j.last = static_cast<int32_t>(std::min(x.p0, x.n - (b0 + cnt - 1) * x.p0));
        j.tensor = static_cast<int32_t>(ti);
        j.toff = j.base - x.start;
        j.tstride = x.p0;
        ql->jobs.push_back(j);
        q += cnt;
      }
    }
  }
  ql->n_blocks = q;
  std::vector<std::pair<int64_t, int64_t>> qiv;
  for (const Tensor& x : t)
    if (x.kind == RS_TILE || x.kind == RS_FLAT || x.kind == RS_TILEMAJOR) qiv.push_back({x.start, x.start + x.n});
  std::sort(qiv.begin(), qiv.end());
  auto zero = [&](int64_t from, int64_t to) {
    for (int64_t p = from; p < to; p += kZeroChunk) {
      QJob j{};
      j.base = p;
      j.stride = std::min(kZeroChunk, to - p);
      j.kind = QJOB_ZERO;
      j.tensor = -1;
      ql->jobs.push_back(j);
    }
  };
  int64_t pos = 0;
  for (auto& r : qiv) {
    zero(pos, r.first);
    pos = r.second;
  }
  zero(pos, top);
  // one kernel per job kind: keep each kind contiguous
  std::stable_sort(ql->jobs.begin(), ql->jobs.end(),
                   [](const QJob& a, const QJob& b) { return a.kind < b.kind; });
  for (const QJob& j : ql->jobs) {
    if (j.kind == QJOB_TILE) ++ql->n_tile;
    else if (j.kind == QJOB_FLAT) ++ql->n_flat;
    else ++ql->n_zero;
  }
  // Adam strips: tile jobs 4g .. 4g+3 are four full 32x32 tiles of one tensor
  // side by side (consecutive in the buffer and in scale order), 16-byte
  // aligned, for every group g
  ql->all_strips = ql->n_tile > 0 && ql->n_tile % kAdamStripTiles == 0;
  for (int64_t g = 0; ql->all_strips && g < ql->n_tile; g += kAdamStripTiles) {
    const QJob& j0 = ql->jobs[g];
    for (int w = 0; w < kAdamStripTiles && ql->all_strips; ++w) {
      const QJob& jw = ql->jobs[g + w];
      ql->all_strips = jw.tensor == j0.tensor && jw.rows == kAdamStripRows && jw.cols == kAdamStripTileCols &&
                       jw.stride == j0.stride && jw.stride % 16 == 0 && jw.base % 16 == 0 &&
                       jw.base == j0.base + w * kAdamStripTileCols && jw.scale == j0.scale + w;
    }
  }
}


}  // namespace rs

using namespace rs;

static void release(rs_plan* p) {
  if (!p) return;
  int prev = 0;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(p->device);
  (void)hipDeviceSynchronize();
  for (PtrTable* tab : {&p->dst, &p->src, &p->gdst}) {
    if (tab->done) (void)hipEventDestroy(tab->done);
    if (tab->stage) (void)hipHostFree(tab->stage);
  }
  if (p->dmem) (void)hipFree(p->dmem);
  (void)hipSetDevice(prev);
  delete p;
}

static int init_table(PtrTable* tab, void** dev, int64_t n) {
  tab->dev = dev;
  tab->seen.assign(n, nullptr);
  if (hipHostMalloc(reinterpret_cast<void**>(&tab->stage), sizeof(void*) * n, hipHostMallocDefault) != hipSuccess)
    return fail(RS_ENOMEM, "rs_plan_load: pinned staging allocation failed");
  if (hipEventCreateWithFlags(&tab->done, hipEventDisableTiming) != hipSuccess)
    return fail(RS_EHIP, "rs_plan_load: hipEventCreate failed");
  return RS_OK;
}

extern "C" int rs_plan_load(const rs_tensor_spec* specs, int64_t n, int64_t V, int64_t S,
                            const int64_t* starts, int64_t R_mat, int32_t device, rs_plan** out) {
  try {
    clear_error();
    if (!out) return fail(RS_EINVAL, "rs_plan_load: null output");
    *out = nullptr;
    if (device < 0) return fail(RS_EINVAL, "rs_plan_load: bad device");
    std::vector<Tensor> t;
    int64_t R_used = 0;
    int st = validate_plan("rs_plan_load", specs, n, V, S, starts, R_mat, &t, &R_used);
    if (st != RS_OK) return st;

    Tables tb;
    lower(t, S, R_mat, &tb);
    // Every launch loops over its work items beyond kMaxGrid workgroups; item
    // and piece indices are 32-bit. Under the 2^39-element limit this holds
    // for any plan but one made of tiny tiles.
    const int64_t items = std::max({static_cast<int64_t>(tb.unpack.size()) * unpack_split(4),
                                    static_cast<int64_t>(tb.pack.size()) * std::max(kPackSplit, kPack1Split),
                                    static_cast<int64_t>(tb.gchunks.size()) * tb.gather_split4,
                                    static_cast<int64_t>(tb.tm.size()) * tm_pieces(tb.tm_max_strip, 4, kTmThreads),
                                    static_cast<int64_t>(tb.qjobs.size()), static_cast<int64_t>(tb.gjobs.size()),
                                    tb.n_qflat * kFlatPerGroup + tb.n_qzero});
    if (items > 0xFFFFFFFFll)
      return fail(RS_ERANGE, "rs_plan_load: the plan needs " + std::to_string(items) +
                                 " work items in one launch; indices are 32-bit");

    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return fail(RS_EHIP, "rs_plan_load: no HIP device");
    if (hipSetDevice(device) != hipSuccess) return fail(RS_EHIP, "rs_plan_load: hipSetDevice failed");

    rs_plan* p = new rs_plan();
    p->device = device;
    p->V = V;
    p->S = S;
    p->R_mat = R_mat;
    p->R_used = R_used;
    p->n = n;
    p->padding = tb.padding;
    p->t = t;
    p->n_unpack = static_cast<int64_t>(tb.unpack.size());
    p->n_tm = static_cast<int64_t>(tb.tm.size());
    p->n_pack = static_cast<int64_t>(tb.pack.size());
    p->n_qjobs = static_cast<int64_t>(tb.qjobs.size());
    p->n_qblocks = tb.n_qblocks;
    p->n_qtile = tb.n_qtile;
    p->n_qflat = tb.n_qflat;
    p->n_qzero = tb.n_qzero;
    p->tm_max_strip = tb.tm_max_strip;
    p->n_gchunks = static_cast<int64_t>(tb.gchunks.size());
    p->n_gtile = tb.n_gtile;
    p->n_gflat = tb.n_gflat;
    p->max_tile_vec16 = tb.max_tile_vec16;
    p->split_code_lines = tb.split_code_lines;
    p->adam_all_strips = tb.adam_all_strips;
    p->gather_vec = tb.gather_vec;
    p->gather_split8 = tb.gather_split8;
    p->gather_split4 = tb.gather_split4;
    // gfx950's FP8 conversion (OCP E4M3, round to nearest even) by default;
    // RS_E4M3_ENCODER=sw selects the integer encoder, which gives the same codes.
    const char* enc = std::getenv("RS_E4M3_ENCODER");
    p->e4m3_hw = !(enc && std::strcmp(enc, "sw") == 0);
    // Tile-major reorder: staged through LDS by default; RS_TM_KERNEL=direct
    // selects the direct kernels (=lds the staged ones) for unpack and pack.
    // Both give the same results.
    if (const char* tmk = std::getenv("RS_TM_KERNEL")) {
      if (std::strcmp(tmk, "lds") == 0) p->tm_unpack_lds = p->tm_pack_lds = true;
      if (std::strcmp(tmk, "direct") == 0) p->tm_unpack_lds = p->tm_pack_lds = false;
    }
    // RS_ADAM_TILE_KERNEL=workgroup: the Adam step gives every tile a 256-thread
    // workgroup even when one wave would hold it (=wave: the default choice)
    if (const char* ak = std::getenv("RS_ADAM_TILE_KERNEL")) p->adam_wave_tiles = std::strcmp(ak, "workgroup") != 0;
    // RS_MAX_GRID=n caps every launch at n workgroups (rounded down to a
    // multiple of 8, at least 8), so the workgroups loop over work items; the
    // results do not change.
    if (const char* mg = std::getenv("RS_MAX_GRID")) {
      const long long v = std::strtoll(mg, nullptr, 10);
      p->max_grid = std::max<int64_t>(8, std::min<int64_t>(kMaxGrid, v) / 8 * 8);
    }

    const int64_t bytes = align_up(sizeof(TmJob) * std::max<int64_t>(p->n_tm, 1), 256) +
                          align_up(sizeof(CopyChunk) * std::max<int64_t>(p->n_unpack, 1), 256) +
                          align_up(sizeof(PackChunk) * std::max<int64_t>(p->n_pack, 1), 256) +
                          align_up(sizeof(QJob) * std::max<int64_t>(p->n_qjobs, 1), 256) +
                          align_up(sizeof(GatherChunk) * std::max<int64_t>(p->n_gchunks, 1), 256) +
                          align_up(sizeof(QJob) * std::max<int64_t>(p->n_gtile + p->n_gflat, 1), 256) +
                          3 * align_up(sizeof(void*) * n, 256);
    if (hipMalloc(&p->dmem, bytes) != hipSuccess) {
      p->dmem = nullptr;
      release(p);
      (void)hipSetDevice(prev);
      return fail(RS_ENOMEM, "rs_plan_load: device allocation of the work lists failed");
    }
    char* cur = static_cast<char*>(p->dmem);
    p->tmjobs = carve<TmJob>(cur, p->n_tm);
    p->unpack = carve<CopyChunk>(cur, p->n_unpack);
    p->pack = carve<PackChunk>(cur, p->n_pack);
    p->qjobs = carve<QJob>(cur, p->n_qjobs);
    p->gchunks = carve<GatherChunk>(cur, p->n_gchunks);
    p->gjobs = carve<QJob>(cur, p->n_gtile + p->n_gflat);
    void** dst_dev = carve<void*>(cur, n);
    void** src_dev = carve<void*>(cur, n);
    void** gdst_dev = carve<void*>(cur, n);

    bool ok = (p->n_tm == 0 || hipMemcpy(p->tmjobs, tb.tm.data(), sizeof(TmJob) * p->n_tm, hipMemcpyHostToDevice) == hipSuccess) &&
              (p->n_unpack == 0 || hipMemcpy(p->unpack, tb.unpack.data(), sizeof(CopyChunk) * p->n_unpack, hipMemcpyHostToDevice) == hipSuccess) &&
              (p->n_pack == 0 || hipMemcpy(p->pack, tb.pack.data(), sizeof(PackChunk) * p->n_pack, hipMemcpyHostToDevice) == hipSuccess) &&
              (p->n_qjobs == 0 || hipMemcpy(p->qjobs, tb.qjobs.data(), sizeof(QJob) * p->n_qjobs, hipMemcpyHostToDevice) == hipSuccess) &&
              (p->n_gchunks == 0 || hipMemcpy(p->gchunks, tb.gchunks.data(), sizeof(GatherChunk) * p->n_gchunks, hipMemcpyHostToDevice) == hipSuccess) &&
              (tb.gjobs.empty() || hipMemcpy(p->gjobs, tb.gjobs.data(), sizeof(QJob) * tb.gjobs.size(), hipMemcpyHostToDevice) == hipSuccess);
    if (!ok) {
      release(p);
      (void)hipSetDevice(prev);
      return fail(RS_EHIP, "rs_plan_load: upload of the work lists failed");
    }
    st = init_table(&p->dst, dst_dev, n);
    if (st == RS_OK) st = init_table(&p->src, src_dev, n);
    if (st == RS_OK) st = init_table(&p->gdst, gdst_dev, n);
    if (st != RS_OK) {
      std::string msg = rs_last_error();
      release(p);
      (void)hipSetDevice(prev);
      return fail(st, msg);
    }
    (void)hipSetDevice(prev);
    *out = p;
    return RS_OK;
  } catch (const std::exception& ex) {
    return fail(RS_ENOMEM, std::string("rs_plan_load: ") + ex.what());
  }
}

extern "C" int rs_plan_info(const rs_plan* p, int64_t* R_used, int64_t* n_qblocks, int64_t* padding) {
  clear_error();
  if (!p) return fail(RS_EINVAL, "rs_plan_info: null plan");
  if (R_used) *R_used = p->R_used;
  if (n_qblocks) *n_qblocks = p->n_qblocks;
  if (padding) *padding = p->padding;
  return RS_OK;
}

extern "C" void rs_plan_free(rs_plan* p) { release(p); }

extern "C" const char* rs_last_error(void) { return rs::g_error.c_str(); }
