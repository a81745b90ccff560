// Host check of the lowering that rs_plan_load uploads: from the work lists
// alone, every kernel writes every element of its output exactly once, reads
// it from the right place and uses the right scale. The work lists are
// simulated element by element, independently of the kernels.
//
// Reads "n V S R_mat" and n lines "rows cols kind p0 p1 start" on stdin;
// prints "ok" or the first violation. With an argument 1-4 it first plants
// one mistake in the lists (a pack chunk dropped, a quant job doubled, a
// gather scale shifted, an unpack source shifted), which must be reported.
// With the argument "shape" it only lowers the plan and prints the gather
// side's shape (for plans too large to check element by element). This file includes plan.cpp so that it
// can call validate_plan() and the file-local lower(); link it with planner.cpp.
#include "plan.cpp"

#include <cstdio>

namespace {

using namespace rs;

std::string fail_msg;
#define CHECK(cond, ...)                                                   \
  do {                                                                     \
    if (!(cond)) {                                                         \
      char b_[512];                                                        \
      std::snprintf(b_, sizeof b_, __VA_ARGS__);                           \
      fail_msg = std::string(b_) + " [" #cond "]";                         \
      return false;                                                        \
    }                                                                      \
  } while (0)

bool quantised(const Tensor& x) { return x.kind == RS_TILE || x.kind == RS_FLAT || x.kind == RS_TILEMAJOR; }

// Flat position of row-major element e of tensor x (TILEMAJOR: tile by tile).
int64_t flat_of(const Tensor& x, int64_t e) {
  if (x.kind != RS_TILEMAJOR) return x.start + e;
  const int64_t R = e / x.cols, C = e % x.cols, br = x.p0, bc = x.p1, ntc = x.cols / bc;
  return x.start + ((R / br) * ntc + C / bc) * br * bc + (R % br) * bc + C % bc;
}

// Scale index of row-major element e of quantised tensor x, given its first scale.
int64_t scale_of(const Tensor& x, int64_t first, int64_t e) {
  const int64_t R = e / x.cols, C = e % x.cols;
  if (x.kind == RS_FLAT) return first + e / x.p0;
  const int64_t ntc = (x.cols + x.p1 - 1) / x.p1;
  return first + (R / x.p0) * ntc + C / x.p1;
}

int64_t g_split8 = 0, g_split4 = 0, g_runs = 0, g_vec = 0;
bool g_strips = false;

// The Adam step's whole-strip launch, decided from the tensors rather than
// the job list: some tensor has tiles, and every tiled tensor is a row-major
// TILE(32, 32) tensor of whole 32-row bands whose width is a multiple of 128
// (so each band's tiles fall into groups of four side by side).
bool strips_from_tensors(const std::vector<Tensor>& t) {
  bool any = false;
  for (const Tensor& x : t) {
    if (x.kind == RS_TILEMAJOR) return false;
    if (x.kind != RS_TILE) continue;
    if (x.p0 != 32 || x.p1 != 32 || x.rows % 32 != 0 || x.cols % 128 != 0) return false;
    any = true;
  }
  return any;
}

bool check(const std::vector<Tensor>& t, int64_t S, int64_t R, int plant) {
  Tables tb;
  lower(t, S, R, &tb);
  g_split8 = tb.gather_split8;
  g_split4 = tb.gather_split4;
  g_runs = static_cast<int64_t>(tb.gchunks.size());
  g_vec = tb.gather_vec;
  g_strips = tb.adam_all_strips;
  CHECK(tb.adam_all_strips == strips_from_tensors(t), "Adam strip launch %d, from the tensors %d",
        int(tb.adam_all_strips), int(strips_from_tensors(t)));
  if (plant == 1 && !tb.pack.empty()) tb.pack.pop_back();
  if (plant == 2 && !tb.qjobs.empty()) tb.qjobs.insert(tb.qjobs.begin(), tb.qjobs.front());
  if (plant == 3 && !tb.gchunks.empty()) tb.gchunks.back().scale0 += 1;
  if (plant == 4 && !tb.unpack.empty()) tb.unpack.back().src += 16;
  const int64_t top = R * S;
  const int64_t n = static_cast<int64_t>(t.size());
  std::vector<int64_t> first(n + 1, 0);
  for (int64_t i = 0; i < n; ++i) {
    const Tensor& x = t[i];
    int64_t nb = 0;
    if (x.kind == RS_TILE) nb = ((x.rows + x.p0 - 1) / x.p0) * ((x.cols + x.p1 - 1) / x.p1);
    if (x.kind == RS_TILEMAJOR) nb = x.n / (x.p0 * x.p1);
    if (x.kind == RS_FLAT) nb = (x.n + x.p0 - 1) / x.p0;
    first[i + 1] = first[i] + nb;
  }
  CHECK(tb.n_qblocks == first[n], "scale count %lld, expected %lld", (long long)tb.n_qblocks, (long long)first[n]);
  std::vector<int32_t> owner(top, -1);   // tensor owning each flat position
  for (int64_t i = 0; i < n; ++i)
    for (int64_t e = 0; e < t[i].n; ++e) owner[flat_of(t[i], e)] = static_cast<int32_t>(i);

  std::vector<std::vector<uint8_t>> cnt(n);
  auto reset = [&]() { for (int64_t i = 0; i < n; ++i) cnt[i].assign(t[i].n, 0); };
  auto all_once = [&](const char* what, bool only_quantised) -> bool {
    for (int64_t i = 0; i < n; ++i) {
      const uint8_t want = (!only_quantised || quantised(t[i])) ? 1 : 0;
      for (int64_t e = 0; e < t[i].n; ++e)
        CHECK(cnt[i][e] == want, "%s: tensor %lld element %lld written %d times", what, (long long)i, (long long)e,
              cnt[i][e]);
    }
    return true;
  };
  // a tile-major strip: k tiles x h rows of bc elements; element (r, c) of tile t
  auto strip = [&](const TmJob& j, bool scales) -> bool {
    const Tensor& x = t[j.tensor];
    CHECK(x.kind == RS_TILEMAJOR, "strip of tensor %d", j.tensor);
    for (int64_t tt = 0; tt < j.k; ++tt)
      for (int64_t r = 0; r < j.h; ++r)
        for (int64_t c = 0; c < j.bc; ++c) {
          const int64_t e = j.toff + r * j.cols + tt * j.bc + c;
          const int64_t p = j.base + tt * j.tile_elems + r * j.bc + c;
          CHECK(e >= 0 && e < x.n && flat_of(x, e) == p, "strip maps element %lld to %lld", (long long)e, (long long)p);
          if (scales) CHECK(scale_of(x, first[j.tensor], e) == j.scale0 + tt, "strip scale of element %lld", (long long)e);
          cnt[j.tensor][e]++;
        }
    return true;
  };

  // unpack: tensor element e comes from flat position flat_of(e)
  reset();
  for (const CopyChunk& c : tb.unpack) {
    const Tensor& x = t[c.tensor];
    CHECK(x.kind != RS_TILEMAJOR && c.src == x.start + c.off && c.off >= 0 && c.off + c.len <= x.n,
          "unpack chunk of tensor %d at %lld", c.tensor, (long long)c.off);
    for (int64_t e = c.off; e < c.off + c.len; ++e) cnt[c.tensor][e]++;
  }
  for (const TmJob& j : tb.tm)
    if (!strip(j, false)) return false;
  if (!all_once("unpack", false)) return false;

  // pack: every flat position once; data from its own tensor element; the rest is padding
  std::vector<uint8_t> pc(top, 0);
  for (const PackChunk& c : tb.pack) {
    CHECK(c.out % 16 == 0 && c.n_total % 16 == 0 && c.out + c.n_total <= top && c.n_data <= c.n_total,
          "pack chunk at %lld", (long long)c.out);
    for (int64_t k = 0; k < c.n_total; ++k) {
      const int64_t p = c.out + k;
      if (c.tensor >= 0 && k < c.n_data)
        CHECK(owner[p] == c.tensor && p == t[c.tensor].start + c.off + k, "pack data at %lld", (long long)p);
      else
        CHECK(owner[p] == -1, "pack writes padding over tensor %d at %lld", owner[p], (long long)p);
      pc[p]++;
    }
  }
  for (const TmJob& j : tb.tm)
    for (int64_t tt = 0; tt < j.k; ++tt)
      for (int64_t r = 0; r < j.h; ++r)
        for (int64_t c = 0; c < j.bc; ++c) pc[j.base + tt * j.tile_elems + r * j.bc + c]++;
  for (int64_t p = 0; p < top; ++p) CHECK(pc[p] == 1, "pack: position %lld written %d times", (long long)p, pc[p]);

  // quant: every code position once (blocks or zero ranges), every scale once, blocks whole
  std::vector<uint8_t> qc(top, 0), sc(first[n] + 1, 0);
  int64_t seen_tile = 0, seen_flat = 0, seen_zero = 0;
  for (const QJob& j : tb.qjobs) {
    if (j.kind == QJOB_ZERO) {
      ++seen_zero;
      for (int64_t p = j.base; p < j.base + j.stride; ++p) {
        CHECK(p >= 0 && p < top && (owner[p] == -1 || !quantised(t[owner[p]])), "zero range over a block at %lld",
              (long long)p);
        qc[p]++;
      }
      continue;
    }
    const Tensor& x = t[j.tensor];
    CHECK(quantised(x), "quant job on tensor %d", j.tensor);
    if (j.kind == QJOB_TILE) {
      ++seen_tile;
      CHECK(x.kind == RS_TILE || x.kind == RS_TILEMAJOR, "tile job on tensor %d", j.tensor);
      for (int64_t r = 0; r < j.rows; ++r)
        for (int64_t c = 0; c < j.cols; ++c) {
          const int64_t p = j.base + r * j.stride + c, e = j.toff + r * j.tstride + c;
          CHECK(owner[p] == j.tensor && flat_of(x, e) == p && scale_of(x, first[j.tensor], e) == j.scale,
                "tile job element (%lld, %lld) of tensor %d", (long long)r, (long long)c, j.tensor);
          qc[p]++;
        }
      sc[j.scale]++;
    } else {
      ++seen_flat;
      CHECK(x.kind == RS_FLAT && j.rows >= 1 && j.rows <= kFlatPerGroup, "flat job on tensor %d", j.tensor);
      for (int64_t b = 0; b < j.rows; ++b) {
        const int64_t len = b == j.rows - 1 ? j.last : j.cols;
        for (int64_t k = 0; k < len; ++k) {
          const int64_t p = j.base + b * j.cols + k, e = j.toff + b * j.cols + k;
          CHECK(owner[p] == j.tensor && flat_of(x, e) == p && scale_of(x, first[j.tensor], e) == j.scale + b,
                "flat job element %lld of tensor %d", (long long)e, j.tensor);
          qc[p]++;
        }
        sc[j.scale + b]++;
      }
    }
  }
  CHECK(seen_tile == tb.n_qtile && seen_flat == tb.n_qflat && seen_zero == tb.n_qzero, "job kinds out of order");
  for (size_t k = 1; k < tb.qjobs.size(); ++k) CHECK(tb.qjobs[k - 1].kind <= tb.qjobs[k].kind, "job kinds not sorted");
  for (int64_t p = 0; p < top; ++p) CHECK(qc[p] == 1, "quant: code %lld written %d times", (long long)p, qc[p]);
  for (int64_t s = 0; s < first[n]; ++s) CHECK(sc[s] == 1, "quant: scale %lld written %d times", (long long)s, sc[s]);

  // gather side: every element of every quantised tensor once, with its own scale;
  // no run longer than its launch's split covers
  reset();
  for (const GatherChunk& c : tb.gchunks) {
    const Tensor& x = t[c.tensor];
    CHECK(ceil_div(int64_t(c.rows) * c.cols, gather_piece(tb.gather_vec) * 8) <= tb.gather_split8 &&
              ceil_div(int64_t(c.rows) * c.cols, gather_piece(tb.gather_vec) * 4) <= tb.gather_split4,
          "gather run of %lld codes longer than the split", (long long)c.rows * c.cols);
    CHECK(c.qbase == x.start + c.toff && c.cols % 8 == 0, "gather run of tensor %d", c.tensor);
    for (int64_t r = 0; r < c.rows; ++r)
      for (int64_t k = 0; k < c.cols; ++k) {
        const int64_t e = c.toff + r * c.cols + k;
        CHECK(e < x.n && scale_of(x, first[c.tensor], e) == c.scale0 + r * c.rstep + k / c.bc,
              "gather run element %lld of tensor %d", (long long)e, c.tensor);
        cnt[c.tensor][e]++;
      }
  }
  for (const QJob& j : tb.gjobs) {
    const Tensor& x = t[j.tensor];
    const int64_t nb = j.kind == QJOB_TILE ? 1 : j.rows;
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t rows = j.kind == QJOB_TILE ? j.rows : 1;
      const int64_t cols = j.kind == QJOB_TILE ? j.cols : (b == j.rows - 1 ? j.last : j.cols);
      for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
          const int64_t e = j.toff + (j.kind == QJOB_TILE ? r * j.tstride + c : b * j.cols + c);
          const int64_t p = j.base + (j.kind == QJOB_TILE ? r * j.stride + c : b * j.cols + c);
          CHECK(flat_of(x, e) == p && scale_of(x, first[j.tensor], e) == j.scale + b,
                "gather job element %lld of tensor %d", (long long)e, j.tensor);
          cnt[j.tensor][e]++;
        }
    }
  }
  for (const TmJob& j : tb.tm)
    if (!strip(j, true)) return false;
  return all_once("gather", true);
}

}  // namespace

int main(int argc, char** argv) {
  const bool shape_only = argc > 1 && std::strcmp(argv[1], "shape") == 0;
  const int plant = argc > 1 && !shape_only ? std::atoi(argv[1]) : 0;
  long long n, V, S, R;
  if (std::scanf("%lld %lld %lld %lld", &n, &V, &S, &R) != 4 || n < 1) return 2;
  std::vector<rs_tensor_spec> specs(n);
  std::vector<int64_t> starts(n);
  for (long long i = 0; i < n; ++i) {
    long long r, c, k, p0, p1, s;
    if (std::scanf("%lld %lld %lld %lld %lld %lld", &r, &c, &k, &p0, &p1, &s) != 6) return 2;
    specs[i] = rs_tensor_spec{};
    specs[i].rows = r;
    specs[i].cols = c;
    specs[i].kind = static_cast<int32_t>(k);
    specs[i].p0 = p0;
    specs[i].p1 = p1;
    starts[i] = s;
  }
  std::vector<Tensor> t;
  int64_t R_used = 0;
  if (validate_plan("rs_plan_load", specs.data(), n, V, S, starts.data(), R, &t, &R_used) != RS_OK) {
    std::printf("invalid plan: %s\n", rs_last_error());
    return 0;
  }
  if (shape_only) {
    Tables tb;
    lower(t, S, R, &tb);
    std::printf("ok\ngather runs %lld split8 %lld split4 %lld vec %d\n", (long long)tb.gchunks.size(),
                (long long)tb.gather_split8, (long long)tb.gather_split4, tb.gather_vec);
    return 0;
  }
  if (!check(t, S, R, plant)) {
    std::printf("FAIL %s\n", fail_msg.c_str());
    return 0;
  }
  std::printf("ok\n");
  std::printf("gather runs %lld split8 %lld split4 %lld vec %lld\n", (long long)g_runs, (long long)g_split8,
              (long long)g_split4, (long long)g_vec);
  std::printf("adam strips %d\n", int(g_strips));
  return 0;
}
