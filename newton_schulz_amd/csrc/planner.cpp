// Host scheduler: same-shape buckets cut into micro-buckets under a cap.
//
// The blog "Muon Optimizer + FSDP" recommends processing XTuner-style same-
// shape buckets (introduction; section "Chunked communication") in micro-
// buckets of whole matrices under a dedicated Muon cap (section "Memory
// control", item 1, estimate_muon_peak(bucket) <= workspace cap), merging
// same-shape matrices across layers (item 6) and planning buffer addresses
// once (section "DBuffer").  Pure host code, no HIP calls.
#include <algorithm>
#include <map>
#include <new>
#include <utility>
#include <vector>

#include "muon.h"
#include "ns_layout.h"

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A round of 128-tiles (two workgroups of four waves per CU) takes about
// this fraction of the time of a round of 256-tiles at the same K (MI355X:
// 0.58 for the update and 0.49 for the symmetric square at K = 768, many
// rounds each); the margin keeps 256-tiles wherever the two are close.
constexpr double kRound128 = 0.6;

// Model of the Newton-Schulz time of one micro-bucket of U units of
// canonical shape (m, n) on `cus` compute units, in k-elements processed per
// 256-tile slot: every product launch takes ceil(tiles / slots) rounds, a
// round as long as its contraction (Gram: n, symmetric square and update:
// m), a round of 128-tiles kRound128 of that.  Tile side and slots per CU
// follow the launches: bf16 products take ns_mfma_tile's side (one 256-tile
// or two 128-tiles per CU), fp32 runs 64 x 64 tiles (four per CU).

double ns_time_model(int64_t m, int64_t n, int64_t units, int cus, int32_t compute) {
  // rounds of tiles of one launch, a round of 128-tiles weighted kRound128
  auto rounds = [&](int64_t rows, int64_t cols, bool upper) -> double {
    const int64_t tile = compute == MUON_F32 ? 64 : ns_mfma_tile(rows, cols, upper, units, cus);
    const int64_t slots = static_cast<int64_t>(cus) * (tile == 256 ? 1 : (tile == 128 ? 2 : 4));
    const int64_t tm = ceil_div(rows, tile), tn = ceil_div(cols, tile);
    const int64_t r = ceil_div(units * (upper ? tm * (tm + 1) / 2 : tm * tn), slots);
    return static_cast<double>(r) * (tile == 128 ? kRound128 : 1.0);
  };
  // Gram (K = n) and symmetric square (K = m) over the m x m upper tiles,
  // update (K = m) over the m x n tiles
  return rounds(m, m, true) * static_cast<double>(n + m) + rounds(m, n, false) * static_cast<double>(m);
}

// Fixed cost of one more micro-bucket in the same units: about 20 dependent
// launches (momentum, norm, the products, apply) at a few microseconds each,
// with ~19 ns per k-element of a 256-wide tile round.
constexpr double kBucketOverhead = 3000.0;

}  // namespace

int ns_mfma_tile(int64_t rows, int64_t cols, bool upper, int64_t units, int cus) {
  if (std::min(rows, cols) < 256) return 128;
  const int64_t c = cus > 0 ? cus : 256;
  auto tiles = [&](int64_t t) {
    const int64_t tm = ceil_div(rows, t), tn = ceil_div(cols, t);
    return units * (upper ? tm * (tm + 1) / 2 : tm * tn);
  };
  const int64_t r256 = ceil_div(tiles(256), c), r128 = ceil_div(tiles(128), 2 * c);
  return kRound128 * static_cast<double>(r128) < static_cast<double>(r256) ? 128 : 256;
}

// Shared with muon_api.hip, so the reported size and the carve-up agree.
bool ns_layout(const muon_shape_t& s, int64_t count, int32_t compute, NsLayout* L) {
  if (s.rows <= 0 || s.cols <= 0 || s.head_rows < 0 || count < 0) return false;
  if (s.head_rows > 0 && s.rows % s.head_rows != 0) return false;
  if (compute != MUON_BF16 && compute != MUON_F32) return false;
  const size_t e = compute == MUON_BF16 ? 2 : 4;
  NsLayout l;
  const int64_t per = s.head_rows > 0 ? s.rows / s.head_rows : 1;
  l.units = count * per;
  l.ur = s.head_rows > 0 ? s.head_rows : s.rows;
  l.uc = s.cols;
  l.m = std::min(l.ur, l.uc);
  l.n = std::max(l.ur, l.uc);
  const int64_t ue = l.ur * l.uc;
  // norm partial sums: about 32K elements per part, at most 512 parts
  int64_t parts = (ue + 32767) / 32768;
  if (parts < 1) parts = 1;
  if (parts > 512) parts = 512;
  int64_t chunk = (ue + parts - 1) / parts;
  chunk = (chunk + 7) / 8 * 8;
  parts = (ue + chunk - 1) / chunk;
  l.parts = static_cast<int>(parts);
  const size_t U = static_cast<size_t>(l.units);
  const size_t xbytes = align_up(U * static_cast<size_t>(l.m * l.n) * e);
  const size_t abytes = align_up(U * static_cast<size_t>(l.m * l.m) * e);
  size_t off = 0;
  l.xa = off; off += xbytes;
  l.xb = off; off += xbytes;
  l.a = off; off += abytes;
  l.b = off; off += abytes;
  l.scale = off; off += align_up(U * 4);
  l.zflag = off; off += align_up(U * 4);
  l.partial = off; off += align_up(U * static_cast<size_t>(l.parts) * 8);
  if (compute == MUON_BF16) {
    const int64_t t = l.m >= 256 ? 256 : 128;
    l.lo_unit = static_cast<size_t>(ceil_div(l.m, t) * t) * static_cast<size_t>(ceil_div(l.n, t) * t) * 2;
    l.lo = off; off += align_up(U * l.lo_unit);
    l.dvec = off; off += align_up(U * static_cast<size_t>(l.m) * 4);
  }
  if (compute == MUON_BF16 && l.m < kNsTinySide) {
    // the fp32 iteration of small units: their widened inputs, then the
    // fp32 layout of the same call
    NsLayout f;
    const muon_shape_t one{l.ur, l.uc, 0};
    if (!ns_layout(one, l.units, MUON_F32, &f)) return false;
    l.stage = 0;
    l.sub = align_up(U * static_cast<size_t>(ue) * 4);
    off = std::max(off, l.sub + f.total);
  }
  l.total = count == 0 ? 0 : off;
  *L = l;
  return true;
}

extern "C" size_t muon_ns_workspace_bytes(muon_shape_t shape, int64_t count, int32_t compute) {
  NsLayout l;
  if (!ns_layout(shape, count, compute, &l)) return 0;
  return l.total;
}

struct MicroBucket {
  muon_bucket_info_t info;
  std::vector<int64_t> idx;
  std::vector<int64_t> off;  // element offset of each member in the flat layout
};

struct muon_plan_s {
  std::vector<MicroBucket> buckets;
  size_t max_ws = 0;
  int64_t total = 0;  // elements of the flat layout
};

static bool same_shape(const muon_shape_t& x, const muon_shape_t& y) {
  return x.rows == y.rows && x.cols == y.cols && x.head_rows == y.head_rows;
}

// a tall unit (more rows than columns) runs the other orientation of the
// products (Y' = Y B'), in launches of its own
static bool is_tall(const muon_shape_t& s) {
  return (s.head_rows > 0 ? s.head_rows : s.rows) > s.cols;
}

extern "C" muon_status_t muon_plan_create(const muon_shape_t* shapes, int64_t count,
                                          size_t cap_bytes, int32_t cap_kind, int32_t compute,
                                          int32_t compute_units, muon_plan_t** out) {
  if (out == nullptr || (count > 0 && shapes == nullptr) || count < 0) return MUON_EINVAL;
  if (cap_kind != MUON_CAP_FULL_BYTES && cap_kind != MUON_CAP_WORKSPACE) return MUON_EINVAL;
  if (compute != MUON_BF16 && compute != MUON_F32) return MUON_EDTYPE;
  *out = nullptr;
  const size_t e = compute == MUON_BF16 ? 2 : 4;
  for (int64_t i = 0; i < count; ++i) {
    NsLayout l;
    if (!ns_layout(shapes[i], 1, compute, &l)) return MUON_ESHAPE;
  }
  muon_plan_t* plan = new (std::nothrow) muon_plan_t;
  if (plan == nullptr) return MUON_ENOMEM;
  try {
    // buckets by canonical unit shape, in order of first appearance
    std::vector<std::pair<int64_t, int64_t>> keys;
    std::map<std::pair<int64_t, int64_t>, size_t> key_id;
    std::vector<std::vector<int64_t>> members;
    for (int64_t i = 0; i < count; ++i) {
      const muon_shape_t& s = shapes[i];
      const int64_t ur = s.head_rows > 0 ? s.head_rows : s.rows;
      const std::pair<int64_t, int64_t> k(std::min(ur, s.cols), std::max(ur, s.cols));
      auto it = key_id.find(k);
      if (it == key_id.end()) {
        key_id[k] = keys.size();
        keys.push_back(k);
        members.emplace_back();
        it = key_id.find(k);
      }
      members[it->second].push_back(i);
    }
    for (size_t b = 0; b < keys.size(); ++b) {
      // order members by orientation (that of the bucket's first member
      // first), then by exact shape, shapes in order of first appearance:
      // units of one orientation have one shape, and the members that give
      // them lie together, so a caller can pass them as one call
      std::vector<muon_shape_t> order;
      for (int64_t i : members[b]) {
        bool seen = false;
        for (const auto& o : order) seen = seen || same_shape(o, shapes[i]);
        if (!seen) order.push_back(shapes[i]);
      }
      const bool tall0 = is_tall(shapes[members[b][0]]);
      std::stable_partition(order.begin(), order.end(),
                            [&](const muon_shape_t& o) { return is_tall(o) == tall0; });
      std::vector<int64_t> sorted;
      for (const auto& o : order)
        for (int64_t i : members[b])
          if (same_shape(o, shapes[i])) sorted.push_back(i);

      auto cost = [&](int64_t i) -> size_t {
        const muon_shape_t& s = shapes[i];
        return cap_kind == MUON_CAP_FULL_BYTES
                   ? e * static_cast<size_t>(s.rows * s.cols)
                   : muon_ns_workspace_bytes(s, 1, compute);
      };
      std::vector<int64_t> cur;
      size_t cur_cost = 0;
      auto flush = [&]() {
        if (cur.empty()) return;
        MicroBucket mb;
        mb.idx = cur;
        muon_bucket_info_t& in = mb.info;
        in.m = keys[b].first;
        in.n = keys[b].second;
        in.count = static_cast<int64_t>(cur.size());
        in.units = 0;
        in.numel = 0;
        in.workspace_bytes = 0;
        in.shape_groups = 0;
        in.over_cap = (cur.size() == 1 && cur_cost > cap_bytes) ? 1 : 0;
        size_t r = 0;
        while (r < cur.size()) {
          size_t q = r;
          while (q < cur.size() && same_shape(shapes[cur[q]], shapes[cur[r]])) ++q;
          const muon_shape_t& s = shapes[cur[r]];
          const int64_t run = static_cast<int64_t>(q - r);
          in.units += run * (s.head_rows > 0 ? s.rows / s.head_rows : 1);
          in.numel += run * s.rows * s.cols;
          in.workspace_bytes += muon_ns_workspace_bytes(s, run, compute);
          in.shape_groups += 1;
          r = q;
        }
        in.full_bytes = e * static_cast<size_t>(in.numel);
        // flat layout: micro-buckets one after another, members packed in
        // execution order
        in.elem_offset = plan->total;
        for (int64_t i : cur) {
          mb.off.push_back(plan->total);
          plan->total += shapes[i].rows * shapes[i].cols;
        }
        plan->max_ws = std::max(plan->max_ws, in.workspace_bytes);
        plan->buckets.push_back(std::move(mb));
        cur.clear();
        cur_cost = 0;
      };
      if (compute_units <= 0) {
        for (int64_t i : sorted) {
          const size_t c = cost(i);
          if (!cur.empty() && cur_cost + c > cap_bytes) flush();
          cur.push_back(i);
          cur_cost += c;
        }
        flush();
      } else {
        // cut points minimising the time model: best[i] = cheapest plan of
        // the first i members, each micro-bucket a run within the cap (or a
        // single matrix)
        // (a micro-bucket's two orientations are separate chains of
        // launches, each with its own rounds of tiles)
        const size_t N = sorted.size();
        std::vector<size_t> c(N);
        std::vector<int64_t> u(N);
        std::vector<char> tall(N);
        for (size_t i = 0; i < N; ++i) {
          const muon_shape_t& sh = shapes[sorted[i]];
          c[i] = cost(sorted[i]);
          u[i] = sh.head_rows > 0 ? sh.rows / sh.head_rows : 1;
          tall[i] = is_tall(sh) ? 1 : 0;
        }
        std::vector<double> best(N + 1, 0.0);
        std::vector<size_t> from(N + 1, 0);
        for (size_t i = 1; i <= N; ++i) {
          best[i] = -1.0;
          size_t bytes = 0;
          int64_t units[2] = {0, 0};
          for (size_t j = i; j-- > 0;) {
            bytes += c[j];
            units[tall[j]] += u[j];
            if (j + 1 < i && bytes > cap_bytes) break;
            double t = best[j];
            for (int o = 0; o < 2; ++o)
              if (units[o] > 0)
                t += kBucketOverhead +
                     ns_time_model(keys[b].first, keys[b].second, units[o], compute_units, compute);
            if (best[i] < 0.0 || t < best[i]) {
              best[i] = t;
              from[i] = j;
            }
          }
        }
        std::vector<size_t> cuts;
        for (size_t i = N; i > 0; i = from[i]) cuts.push_back(i);
        std::reverse(cuts.begin(), cuts.end());
        size_t start = 0;
        for (size_t end : cuts) {
          for (size_t q = start; q < end; ++q) {
            cur.push_back(sorted[q]);
            cur_cost += c[q];
          }
          flush();
          start = end;
        }
      }
    }
  } catch (...) {
    delete plan;
    return MUON_ENOMEM;
  }
  *out = plan;
  return MUON_OK;
}

extern "C" int64_t muon_plan_num_buckets(const muon_plan_t* plan) {
  return plan ? static_cast<int64_t>(plan->buckets.size()) : 0;
}

extern "C" muon_status_t muon_plan(const muon_shape_t* shapes, int64_t count, size_t cap_bytes,
                                   int32_t cap_kind, muon_plan_t** out) {
  return muon_plan_create(shapes, count, cap_bytes, cap_kind, MUON_BF16, 0, out);
}

extern "C" muon_status_t muon_plan_bucket(const muon_plan_t* plan, int64_t b,
                                          muon_bucket_info_t* info, int64_t* indices,
                                          int64_t* offsets) {
  if (plan == nullptr || info == nullptr) return MUON_EINVAL;
  if (b < 0 || b >= static_cast<int64_t>(plan->buckets.size())) return MUON_EINVAL;
  const MicroBucket& mb = plan->buckets[static_cast<size_t>(b)];
  *info = mb.info;
  if (indices)
    for (size_t i = 0; i < mb.idx.size(); ++i) indices[i] = mb.idx[i];
  if (offsets)
    for (size_t i = 0; i < mb.off.size(); ++i) offsets[i] = mb.off[i];
  return MUON_OK;
}

extern "C" int64_t muon_plan_total_elems(const muon_plan_t* plan) { return plan ? plan->total : 0; }

extern "C" size_t muon_workspace_bytes(const muon_shape_t* shapes, int64_t count, int32_t compute) {
  if (count <= 0 || shapes == nullptr) return 0;
  // one Newton-Schulz call per shape group, run one after another on one
  // context: the largest group's need
  size_t need = 0;
  std::vector<char> done(static_cast<size_t>(count), 0);
  for (int64_t i = 0; i < count; ++i) {
    if (done[i]) continue;
    int64_t n = 0;
    for (int64_t j = i; j < count; ++j)
      if (!done[j] && same_shape(shapes[i], shapes[j])) {
        done[j] = 1;
        ++n;
      }
    const size_t w = muon_ns_workspace_bytes(shapes[i], n, compute);
    if (w == 0) return 0;
    need = std::max(need, w);
  }
  return need;
}

extern "C" size_t muon_plan_max_workspace(const muon_plan_t* plan) {
  return plan ? plan->max_ws : 0;
}

extern "C" void muon_plan_destroy(muon_plan_t* plan) { delete plan; }
