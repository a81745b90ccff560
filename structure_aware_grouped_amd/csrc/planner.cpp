// Host planner: shard size S and tensor starts for a RaggedShard group.
//
// Problem ("veScale-FSDP: flexible, structure-aware sharding at 10K-GPU
// scale", feynmanwiki walkthrough, the planner-as-packing paragraph): place
// every tensor in a contiguous interval of a buffer of V*S elements, disjoint,
// padding only between tensors, such that every rank boundary inside a tensor
// lies a multiple of its atomic block size g from the tensor's start, with S
// as small as possible.
//
// Method (same walkthrough, the planner's tensor-order paragraph and the two
// paragraphs after it; bud-325 summary, Method (2)):
//   * three orders: the caller's, block size descending, shape descending;
//   * for one order and one S, feasibility is decided by placing each tensor
//     at the first valid start after the previous one (the DP's state f(i, j)
//     only grows with j, and a tensor's constraint depends on its own start
//     alone, so first-fit reaches every state's minimum);
//   * candidate S values start at the lower bound and step by the alignment
//     (an order after the first stops at the best S found so far); after a
//     short sequential start, candidates are checked in batches on host
//     threads and the smallest feasible one is kept, which gives the same S
//     as a sequential scan;
//     a tensor longer than 2S always holds two boundaries, so S must then be a
//     multiple of its g (the pages' case of a tensor that fully contains a
//     shard): such S values are skipped in one jump. The pages binary-search
//     over aligned candidates; feasibility is not monotone there in general,
//     so this planner scans upward and returns the exact smallest S per order.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "rs_internal.h"

namespace rs {

int64_t granularity(const rs_tensor_spec& s) {
  switch (s.kind) {
    case RS_ELEM: return 1;
    case RS_ROWS: return s.p0 * s.cols;
    case RS_TILE: return s.p0 * s.cols;
    case RS_FLAT: return s.p0;
    case RS_WHOLE: return s.rows * s.cols;
    case RS_TILEMAJOR: return s.p0 * s.p1;
    default: return 0;
  }
}

bool spec_ok(const rs_tensor_spec& s, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return false; };
  if (s.rows < 1 || s.cols < 1) return bad("rows and cols must be >= 1");
  if (s.rows > (int64_t(1) << 40) / s.cols) return bad("tensor too large");
  if (s.reserved != 0) return bad("reserved field must be 0");
  switch (s.kind) {
    case RS_ELEM:
    case RS_WHOLE:
      if (s.p0 != 0 || s.p1 != 0) return bad("ELEM/WHOLE take no block parameters");
      break;
    case RS_ROWS:
      if (s.p0 < 1 || s.p1 != 0) return bad("ROWS needs p0 >= 1 rows and p1 = 0");
      break;
    case RS_FLAT:
      if (s.p0 < 1 || s.p1 != 0) return bad("FLAT needs p0 >= 1 elements and p1 = 0");
      if (s.p0 > (int64_t(1) << 24)) return bad("flat block larger than 2^24 elements");
      break;
    case RS_TILE:
      if (s.p0 < 1 || s.p1 < 1) return bad("TILE needs p0, p1 >= 1");
      if (s.p0 > (int64_t(1) << 24) || s.p1 > (int64_t(1) << 24) || s.p0 * s.p1 > (int64_t(1) << 24))
        return bad("tile larger than 2^24 elements");
      break;
    case RS_TILEMAJOR:
      if (s.p0 < 1 || s.p1 < 1) return bad("TILEMAJOR needs p0, p1 >= 1");
      if (s.p0 > (int64_t(1) << 24) || s.p1 > 8192 || s.p1 > kTmStage || s.p0 * s.p1 > (int64_t(1) << 24))
        return bad("TILEMAJOR tiles hold at most 2^24 elements and 8192 columns");
      if (s.rows % s.p0 != 0 || s.cols % s.p1 != 0) return bad("TILEMAJOR tiles must cover the tensor exactly");
      if ((s.p0 * s.p1) % 16 != 0) return bad("TILEMAJOR tile size must be a multiple of 16 elements");
      break;
    default:
      return bad("unknown block kind");
  }
  if (s.p0 > (int64_t(1) << 40)) return bad("block too large");
  return true;
}

namespace {

struct Item {
  int64_t n, g, rows, L;  // L = lcm(align, g)
};

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// lcm with saturation at `cap` (anything above cap can never divide a
// candidate S <= cap, so its exact value does not matter)
int64_t lcm_cap(int64_t a, int64_t b, int64_t cap) {
  int64_t g = std::gcd(a, b);
  int64_t q = a / g;
  if (q > cap / b) return cap + 1;
  return q * b;
}

// First valid start >= e inside [0, cap) for a tensor, or -1. Starting from
// the first aligned position, look at the first rank boundary b after s: if
// the tensor ends by b, s works. If b - s is not a multiple of g, move s to
// the next position congruent to b modulo lcm(align, g) (at most b itself).
// If b is legal but the tensor also spans b + S while S is not a multiple of
// g, no start before b works: continue from b.
int64_t first_fit(int64_t e, const Item& it, int64_t S, int64_t a, int64_t cap) {
  int64_t s = align_up(e, a);
  for (;;) {
    if (s > cap - it.n) return -1;
    const int64_t b = (s / S + 1) * S;
    if (b >= s + it.n) return s;
    const int64_t off = b - s;
    if (off % it.g != 0) {
      s += off % it.L;
      continue;
    }
    if (s + it.n > b + S && S % it.g != 0) {
      s = b;
      continue;
    }
    return s;
  }
}

// First fit of every tensor in `order`; false as soon as the tensors still to
// place cannot fit after the current end even without padding (`rest[k]` is
// the total size of order[k..]).
bool place(const std::vector<Item>& items, const std::vector<int>& order,
           const std::vector<int64_t>& rest, int64_t S, int64_t V, int64_t a,
           std::vector<int64_t>* starts, int64_t* end) {
  const int64_t cap = V * S;
  int64_t e = 0;
  for (size_t k = 0; k < order.size(); ++k) {
    if (e > cap - rest[k]) return false;
    const int i = order[k];
    const int64_t s = first_fit(e, items[i], S, a, cap);
    if (s < 0) return false;
    if (starts) (*starts)[i] = s;
    e = s + items[i].n;
  }
  if (end) *end = e;
  return true;
}

// Candidate shard sizes in increasing order: multiples of the alignment from
// the lower bound, skipping every S that a tensor longer than 2S forces to be
// a multiple of its g (by_n: tensors by size, largest first; prefix_lcm[p]:
// lcm of the alignment and the g of the first p of them).
struct Candidates {
  const std::vector<Item>* items;
  const std::vector<int>* by_n;
  const std::vector<int64_t>* prefix_lcm;
  int64_t align, s_max;

  // smallest admissible candidate >= S
  int64_t next(int64_t S) const {
    const int64_t n = static_cast<int64_t>(by_n->size());
    for (;;) {
      int64_t p = 0;
      while (p < n && (*items)[(*by_n)[p]].n > 2 * S) ++p;
      const int64_t A = (*prefix_lcm)[p];
      if (S % A == 0) return S;
      // the next multiple of A, or where the smallest forced tensor stops being
      // forced, whichever comes first
      const int64_t to_a = A <= s_max ? align_up(S, A) : s_max + align;
      const int64_t release = align_up(((*items)[(*by_n)[p - 1]].n + 1) / 2, align);
      S = std::max(S + align, std::min(to_a, release));
    }
  }
};

// Smallest feasible candidate in [from, bound] for one order, or -1.
int64_t scan(const std::vector<Item>& items, const std::vector<int>& order,
             const std::vector<int64_t>& rest, const Candidates& cand, int64_t from, int64_t bound,
             int64_t V) {
  const int64_t a = cand.align;
  int64_t S = from;
  for (int k = 0; k < 64; ++k) {  // most groups are settled by the first few candidates
    S = cand.next(S);
    if (S > bound) return -1;
    if (place(items, order, rest, S, V, a, nullptr, nullptr)) return S;
    S += a;
  }
  const unsigned hw = std::thread::hardware_concurrency();
  const int T = static_cast<int>(std::max(1u, std::min(16u, hw)));
  int64_t batch = 256;
  while (S <= bound) {
    std::vector<int64_t> list;
    list.reserve(batch);
    while (static_cast<int64_t>(list.size()) < batch) {
      S = cand.next(S);
      if (S > bound) break;
      list.push_back(S);
      S += a;
    }
    if (list.empty()) return -1;
    std::atomic<int64_t> first(static_cast<int64_t>(list.size()));
    auto work = [&](int t) {
      for (int64_t i = t; i < static_cast<int64_t>(list.size()); i += T) {
        if (i > first.load(std::memory_order_relaxed)) break;
        if (place(items, order, rest, list[i], V, a, nullptr, nullptr)) {
          int64_t cur = first.load();
          while (i < cur && !first.compare_exchange_weak(cur, i)) {
          }
          break;
        }
      }
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < T; ++t) pool.emplace_back(work, t);
    work(0);
    for (auto& th : pool) th.join();
    if (first.load() < static_cast<int64_t>(list.size())) return list[first.load()];
    batch = std::min<int64_t>(batch * 4, 1 << 16);
  }
  return -1;
}

}  // namespace
}  // namespace rs

extern "C" int rs_plan_build(const rs_tensor_spec* specs, int64_t n, int64_t V, int64_t align,
                             int32_t policy, int64_t* S_out, int64_t* starts_out,
                             int64_t* order_out, int32_t* order_kind_out) {
  using namespace rs;
  try {
    clear_error();
    if (!specs || !S_out || !starts_out) return fail(RS_EINVAL, "rs_plan_build: null argument");
    if (n < 1) return fail(RS_EINVAL, "rs_plan_build: need at least one tensor");
    if (V < 1) return fail(RS_EINVAL, "rs_plan_build: V must be >= 1");
    if (align < 1) return fail(RS_EINVAL, "rs_plan_build: align must be >= 1");
    if (policy != RS_ORDER_BEST && policy != RS_ORDER_DEFAULT && policy != RS_ORDER_BLOCK_SIZE &&
        policy != RS_ORDER_SHAPE)
      return fail(RS_EINVAL, "rs_plan_build: unknown order policy");

    std::vector<Item> items(n);
    int64_t total = 0, biggest = 0, s_max = 0;
    const int64_t kLimit = int64_t(1) << 60;
    for (int64_t i = 0; i < n; ++i) {
      std::string why;
      if (!spec_ok(specs[i], &why))
        return fail(RS_EINVAL, "rs_plan_build: tensor " + std::to_string(i) + ": " + why);
      Item& it = items[i];
      it.n = specs[i].rows * specs[i].cols;
      it.g = granularity(specs[i]);
      it.rows = specs[i].rows;
      it.L = lcm_cap(align, it.g, kLimit);
      if (it.L > kLimit) return fail(RS_ERANGE, "rs_plan_build: lcm(align, g) overflows");
      total += it.n;
      biggest = std::max(biggest, std::min(it.g, it.n));
      s_max += align_up(it.n, align);
      if (total > kLimit || s_max > kLimit) return fail(RS_ERANGE, "rs_plan_build: group too large");
    }
    s_max = align_up(s_max, align);  // one shard holding every tensor is always feasible
    const int64_t LB = align_up(std::max((total + V - 1) / V, biggest), align);
    if (V > kLimit / std::max<int64_t>(s_max, 1))
      return fail(RS_ERANGE, "rs_plan_build: V * S may overflow int64");

    // Tensors by element count, largest first, with the running lcm of their
    // g: the first p of them are exactly those longer than 2S for some S.
    std::vector<int> by_n(n);
    std::iota(by_n.begin(), by_n.end(), 0);
    std::stable_sort(by_n.begin(), by_n.end(), [&](int x, int y) { return items[x].n > items[y].n; });
    std::vector<int64_t> prefix_lcm(n + 1);
    prefix_lcm[0] = align;
    for (int64_t p = 0; p < n; ++p)
      prefix_lcm[p + 1] = lcm_cap(prefix_lcm[p], items[by_n[p]].g, s_max);

    // the three orders (kind RS_ORDER_KIND_*), or the one the policy names
    std::vector<int> ident(n);
    std::iota(ident.begin(), ident.end(), 0);
    std::vector<int> by_block = ident;
    std::stable_sort(by_block.begin(), by_block.end(), [&](int x, int y) { return items[x].g > items[y].g; });
    std::vector<int> by_shape = ident;
    std::stable_sort(by_shape.begin(), by_shape.end(), [&](int x, int y) {
      if (items[x].n != items[y].n) return items[x].n > items[y].n;
      return items[x].rows > items[y].rows;
    });
    std::vector<std::vector<int>> orders;
    std::vector<int32_t> kinds;
    auto take = [&](int32_t pol, const std::vector<int>& order, int32_t kind) {
      if (policy == RS_ORDER_BEST || policy == pol) {
        orders.push_back(order);
        kinds.push_back(kind);
      }
    };
    take(RS_ORDER_DEFAULT, ident, RS_ORDER_KIND_DEFAULT);
    take(RS_ORDER_BLOCK_SIZE, by_block, RS_ORDER_KIND_BLOCK);
    take(RS_ORDER_SHAPE, by_shape, RS_ORDER_KIND_SHAPE);

    const Candidates cand{&items, &by_n, &prefix_lcm, align, s_max};
    int64_t best_S = -1, best_end = -1;
    int best_o = -1;
    std::vector<int64_t> starts(n), best_starts(n);
    for (size_t o = 0; o < orders.size(); ++o) {
      std::vector<int64_t> rest(n + 1, 0);
      for (int64_t k = n - 1; k >= 0; --k) rest[k] = rest[k + 1] + items[orders[o][k]].n;
      // an order can only win with an S no larger than the best one so far
      const int64_t bound = best_o < 0 ? s_max : best_S;
      const int64_t S = scan(items, orders[o], rest, cand, LB, bound, V);
      if (S < 0) {
        if (best_o < 0) return fail(RS_EPLAN, "rs_plan_build: internal error, no feasible S");
        continue;
      }
      int64_t end = 0;
      place(items, orders[o], rest, S, V, align, &starts, &end);
      if (best_o < 0 || S < best_S || (S == best_S && end < best_end)) {
        best_S = S;
        best_end = end;
        best_o = static_cast<int>(o);
        best_starts = starts;
      }
    }
    *S_out = best_S;
    std::memcpy(starts_out, best_starts.data(), sizeof(int64_t) * n);
    if (order_out)
      for (int64_t i = 0; i < n; ++i) order_out[i] = orders[best_o][i];
    if (order_kind_out) *order_kind_out = kinds[best_o];
    return RS_OK;
  } catch (const std::exception& ex) {
    return fail(RS_ENOMEM, std::string("rs_plan_build: ") + ex.what());
  }
}
