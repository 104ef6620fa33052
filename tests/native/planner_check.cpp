// Randomised check of the host planner (planner.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py. No GPU and no HIP runtime call:
// only the pure integer planning code is linked.
//
// For random shapes, lengths, page sizes and head policies (GLOBAL, LOCAL, context-adaptive
// LOCAL, RETRIEVAL) it runs argument validation, single-layer, several-layer and growable
// layouts, the table writer, the attention work list (paged and dense-plus-mask modes, and the
// table-driven decode form) and the plan serialiser, and checks their invariants:
// - every head's segments hold kv_len tokens on ceil(ntok / P) pages (growable: at least that
//   many owned pages), virtual pages handed out contiguously in (request, layer, head,
//   segment) order, summing to n_virt;
// - the work items' query blocks partition each (request, KV head)'s queries, and the KV
//   steps of each block's items cover exactly the stored slots that some query of the block
//   sees (visibility written out here from the head-policy rules), each slot once;
// - split items form one combine group per block over distinct partial slots, and the queue
//   bounds and serialised offsets stay inside the workspace the plan sizes.
// Invalid arguments must come back as status codes. Exit status 0 = every check passed.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <set>
#include <tuple>
#include <vector>

#include "planner.h"

using namespace sp;

namespace {

uint64_t g_state = 0;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
int rnd(int n) { return int(next_u64() % uint64_t(n)); }
template <class T>
T pick(std::initializer_list<T> v) {
  return *(v.begin() + rnd(int(v.size())));
}

int g_fail = 0;
#define CHECK(c, ...)                                       \
  do {                                                      \
    if (!(c)) {                                             \
      fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #c); \
      fprintf(stderr, __VA_ARGS__);                         \
      fprintf(stderr, "\n");                                \
      if (++g_fail > 20) exit(1);                           \
    }                                                       \
  } while (0)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

sp_head_policy random_policy() {
  const int r = rnd(100);
  if (r < 30) return sp_head_policy{SP_GLOBAL, 0, 1};
  if (r < 42) return sp_head_policy{SP_RETRIEVAL, pick({0, 4}), pick({1, 100, 999, 1000})};
  if (r < 50) return sp_head_policy{SP_LOCAL_ADAPTIVE, pick({0, 4}), pick({1, 2, 5, 40})};
  return sp_head_policy{SP_LOCAL, pick({0, 1, 4, 70}), pick({1, 33, 64, 500, 2000})};
}

// Policy of a head for a request of context L (adaptive heads take window L / divisor).
sp_head_policy eff(const sp_head_policy& p, int L) {
  if (p.kind != SP_LOCAL_ADAPTIVE) return p;
  return sp_head_policy{SP_LOCAL, p.sink, std::max(1, L / p.window)};
}

// Stored slots (segment, slot) some query at positions [pmin, pmax] of (L, q) sees.
std::set<std::pair<int, int>> visible_slots(const HeadLayout& hl, const sp_head_policy& pol_in,
                                            int L, int q, int pmin, int pmax) {
  const sp_head_policy pol = eff(pol_in, L);
  std::set<std::pair<int, int>> out;
  for (int s = 0; s < hl.nseg; ++s) {
    const Segment& sg = hl.seg[s];
    const bool chunk = pol.kind == SP_RETRIEVAL && q > 0 && s == hl.nseg - 1 && sg.pos == L - q;
    for (int i = 0; i < sg.ntok; ++i) {
      bool vis = false;
      if (pol.kind == SP_RETRIEVAL) {
        vis = chunk ? sg.pos + i <= pmax : true;
      } else {
        const int j = sg.pos + i;
        for (int p = pmin; p <= pmax && !vis; ++p)
          vis = j <= p && (pol.kind == SP_GLOBAL || j < pol.sink || j > p - pol.window);
      }
      if (vis) out.insert({s, i});
    }
  }
  return out;
}

// (segment, slot) pairs of the KV steps [c_begin, c_end) of one item.
std::vector<std::pair<int, int>> item_slots(const WorkItem& w) {
  std::vector<std::pair<int, int>> out;
  const int n_ra = w.ra_end > w.ra_begin ? int(cdiv(w.ra_end, kChunk) - w.ra_begin / kChunk) : 0;
  for (int c = w.c_begin; c < w.c_end; ++c) {
    int seg, lo, hi, base;
    if (c < n_ra) {
      seg = w.ra_seg, lo = w.ra_begin, hi = w.ra_end, base = w.ra_begin / kChunk + c;
    } else {
      seg = w.rb_seg, lo = w.rb_begin, hi = w.rb_end, base = w.rb_begin / kChunk + (c - n_ra);
    }
    for (int i = std::max(lo, base * kChunk); i < std::min(hi, base * kChunk + kChunk); ++i)
      out.push_back({seg, i});
  }
  return out;
}

void check_layout(const Layout& lay, int n_layers, int B, int Hkv, const int32_t* ctx,
                  const int32_t* ql, const std::vector<sp_head_policy>& pol, int P,
                  const int32_t* reserve) {
  int64_t v = 0;
  for (int b = 0; b < B; ++b)
    for (int l = 0; l < n_layers; ++l)
      for (int h = 0; h < Hkv; ++h) {
        const HeadLayout& hl = lay.heads[(size_t(l) * B + b) * Hkv + h];
        int pos[2] = {0, 0}, nt[2] = {0, 0};
        const int nseg = head_segments(pol[size_t(l) * Hkv + h], ctx[b], ql[b], pos, nt);
        CHECK(nseg == hl.nseg, "b %d l %d h %d", b, l, h);
        int kl = 0;
        for (int s = 0; s < 2; ++s) {
          const Segment& sg = hl.seg[s];
          CHECK(sg.vstart == v, "vstart %d != %lld", sg.vstart, (long long)v);
          if (s < hl.nseg) {
            CHECK(sg.pos == pos[s] && sg.ntok == nt[s], "segment %d", s);
            CHECK(sg.ntok >= 0 && sg.pos >= 0 && sg.pos + sg.ntok <= ctx[b], "segment range kind %d pos %d ntok %d L %d q %d", pol[size_t(l) * Hkv + h].kind, sg.pos, sg.ntok, ctx[b], ql[b]);
            if (reserve == nullptr || reserve[b] == 0)
              CHECK(sg.npages == cdiv(sg.ntok, P), "pages %d", sg.npages);
            else
              CHECK(sg.npages >= cdiv(sg.ntok, P), "owned pages %d", sg.npages);
            v += sg.npages;
            kl += sg.ntok;
          } else {
            CHECK(sg.pos == 0 && sg.ntok == 0 && sg.npages == 0, "unused slot");
          }
        }
        if (hl.nseg == 2) CHECK(hl.seg[0].pos + hl.seg[0].ntok <= hl.seg[1].pos, "order");
        CHECK(kl == hl.kv_len, "kv_len");
      }
  CHECK(v == lay.n_virt, "n_virt %lld %lld", (long long)v, (long long)lay.n_virt);
  std::vector<int32_t> tab(size_t(n_layers) * B * Hkv * 8 + 1, -7), kv(size_t(n_layers) * B * Hkv + 1, -7);
  layout_tables(lay, n_layers * B * Hkv, tab.data(), kv.data());
  CHECK(tab.back() == -7 && kv.back() == -7, "table writer overran");
  for (size_t i = 0; i + 1 < kv.size(); ++i) CHECK(kv[i] == lay.heads[i].kv_len, "kv table");
}

void check_plan(const Shape& s, const std::vector<sp_head_policy>& pol, int slots, bool table) {
  Plan plan;
  const sp_status st = make_plan(s, slots, slots, &plan, table);
  CHECK(st == SP_OK, "make_plan %d", int(st));
  if (st != SP_OK) return;
  const WsHeader& hd = plan.hdr;
  for (int x = 0; x < kXcds; ++x) {
    CHECK(hd.prefill_q[x] <= hd.prefill_q[x + 1] && hd.decode_q[x] <= hd.decode_q[x + 1], "queues");
  }
  CHECK(hd.prefill_q[0] == 0 && hd.prefill_q[kXcds] == int(plan.prefill.size()), "prefill queue");
  CHECK(hd.decode_q[0] == 0 && hd.decode_q[kXcds] == int(plan.decode.size()), "decode queue");
  CHECK(plan.upload_bytes <= plan.bytes && hd.bytes == plan.bytes, "sizes");
  CHECK(size_t(hd.off_ml_dec) + size_t(hd.n_part_dec) * kDecodeRows * 8 <= plan.bytes, "partials");
  std::vector<uint8_t> buf;
  serialize_plan(plan, &buf);
  CHECK(buf.size() == plan.upload_bytes, "serialised size");
  if (table) {  // table-driven decode items: (split k of n), no ranges
    for (const WorkItem& w : plan.decode) CHECK(w.ra_seg == -1 && w.c_begin < w.c_end, "table item");
    return;
  }
  Layout lay;
  if (s.mode == kModePaged) CHECK(make_layout(s.B, s.ctx_len, s.q_len, s.Hkv, s.pol, s.P, &lay) == SP_OK, "layout");
  const int G = s.Hq / s.Hkv;
  std::map<std::tuple<int, int, int, int>, std::vector<WorkItem>> blocks;
  for (const std::vector<WorkItem>* v : {&plan.prefill, &plan.decode})
    for (const WorkItem& w : *v) {
      CHECK(w.b >= 0 && w.b < s.B && w.h >= 0 && w.h < s.Hkv && w.nq > 0, "item ids");
      CHECK(w.c_begin < w.c_end, "empty item");
      CHECK(w.p0 == s.ctx_len[w.b] - s.q_len[w.b], "p0");
      CHECK(int64_t(w.nq) * G <= (v == &plan.prefill ? kTileRows : kDecodeRows), "rows");
      blocks[{w.b, w.h, w.tq0, w.nq}].push_back(w);
    }
  std::map<std::tuple<int, int, int, int>, std::vector<int>> parts;
  for (auto& kv : blocks) {
    const int b = std::get<0>(kv.first), h = std::get<1>(kv.first);
    const int t0 = std::get<2>(kv.first), nq = std::get<3>(kv.first);
    const int L = s.ctx_len[b], q = s.q_len[b];
    std::vector<std::pair<int, int>> cov;
    for (const WorkItem& w : kv.second) {
      std::vector<std::pair<int, int>> c = item_slots(w);
      cov.insert(cov.end(), c.begin(), c.end());
    }
    std::set<std::pair<int, int>> covs(cov.begin(), cov.end());
    CHECK(covs.size() == cov.size(), "a slot covered twice (b %d h %d)", b, h);
    if (s.mode == kModePaged) {
      const HeadLayout& hl = lay.heads[size_t(b) * s.Hkv + h];
      const auto want = visible_slots(hl, pol[h], L, q, L - q + t0, L - q + t0 + nq - 1);
      CHECK(covs == want, "coverage b %d h %d t0 %d: %zu vs %zu", b, h, t0, covs.size(), want.size());
    } else {  // dense: rows of the request up to the block's last query
      const int pmax = L - q + t0 + nq - 1;
      for (const auto& c : cov) CHECK(c.second >= 0 && c.second <= pmax, "dense range");
    }
    if (kv.second.size() == 1) {
      CHECK(kv.second[0].part == -1, "unsplit item writes O");
    } else {
      std::vector<int> sp;
      for (const WorkItem& w : kv.second) sp.push_back(w.part);
      std::sort(sp.begin(), sp.end());
      CHECK(sp.front() >= 0 && std::adjacent_find(sp.begin(), sp.end()) == sp.end(), "parts");
      parts[kv.first] = sp;
    }
  }
  CHECK(plan.combine.size() == parts.size(), "combine groups");
  for (const CombineItem& c : plan.combine) {
    auto it = parts.find({c.b, c.h, c.tq0, c.nq});
    CHECK(it != parts.end(), "combine group without items");
    if (it == parts.end()) continue;
    for (int k = 0; k < c.nsplit; ++k) CHECK(it->second[size_t(k)] == c.part0 + k, "combine slots");
    CHECK(c.part0 + c.nsplit <= (c.kind == 0 ? hd.n_part_pre : hd.n_part_dec), "slot range");
  }
  // query blocks partition every (request, head)'s queries that see anything
  for (int b = 0; b < s.B; ++b)
    for (int h = 0; h < s.Hkv; ++h) {
      int got = 0;
      for (auto& kv : blocks)
        if (std::get<0>(kv.first) == b && std::get<1>(kv.first) == h) {
          CHECK(std::get<2>(kv.first) == got, "block order");
          got += std::get<3>(kv.first);
        }
      CHECK(got == 0 || got == s.q_len[b], "blocks cover the chunk");
    }
}

void invalid_arguments() {
  const int32_t ctx[2] = {10, 5}, ql[2] = {3, 6};  // q > ctx for request 1
  sp_head_policy pol[2] = {{SP_GLOBAL, 0, 1}, {SP_LOCAL, 4, 8}};
  CHECK(check_lengths_policy(2, ctx, ql, 2, pol) == SP_ERR_INVALID_ARG, "q > ctx");
  CHECK(check_lengths_policy(2, nullptr, ql, 2, pol) == SP_ERR_INVALID_ARG, "null ctx");
  CHECK(check_lengths_policy(1, ctx, ql, 0, pol) == SP_ERR_INVALID_ARG, "Hkv 0");
  sp_head_policy bad[3] = {{SP_LOCAL, -1, 8}, {SP_LOCAL, 0, 0}, {SP_RETRIEVAL, 0, 1001}};
  for (auto& p : bad) CHECK(check_lengths_policy(1, ctx, ctx, 1, &p) == SP_ERR_INVALID_ARG, "policy");
  sp_head_policy k9{9, 0, 1};
  CHECK(check_lengths_policy(1, ctx, ctx, 1, &k9) == SP_ERR_INVALID_ARG, "kind");
  const int32_t big[2] = {0x7fffff00, 0x7fffff00}, zq[2] = {0, 0};
  CHECK(check_lengths_policy(2, big, zq, 1, pol) == SP_ERR_UNSUPPORTED, "total context");
  CHECK(check_dtype_dim(SP_BF16, 96) == SP_ERR_UNSUPPORTED && check_dtype_dim(7, 64) == SP_ERR_UNSUPPORTED, "dtype/D");
  CHECK(check_page_size(48) == SP_ERR_UNSUPPORTED && check_page_size(0) == SP_ERR_UNSUPPORTED, "page size");
  Shape s{};
  s.mode = kModePaged, s.dtype = SP_BF16, s.B = 1, s.Hq = 3, s.Hkv = 2, s.D = 64, s.P = 64;
  s.ctx_len = ctx, s.q_len = ctx, s.pol = pol;
  CHECK(check_shape(s) == SP_ERR_INVALID_ARG, "Hq %% Hkv");
  s.Hq = 2 * 256;
  CHECK(check_shape(s) == SP_ERR_UNSUPPORTED, "G > 128");
  const int32_t res[1] = {-1};
  CHECK(check_growable(1, ctx, ctx, res, 2, pol) == SP_ERR_INVALID_ARG, "negative reserve");
  sp_head_policy ad{SP_LOCAL_ADAPTIVE, 0, 2};
  const int32_t r0[1] = {0};
  CHECK(check_growable(1, ctx, ctx, r0, 1, &ad) == SP_ERR_UNSUPPORTED, "adaptive growth");
}

}  // namespace

int main(int argc, char** argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 300;
  g_state = argc > 2 ? strtoull(argv[2], nullptr, 10) : 12345;
  invalid_arguments();
  int plans = 0;
  for (int t = 0; t < trials; ++t) {
    const int B = rnd(5);
    const int Hkv = pick({1, 2, 3, 4});
    const int G = pick({1, 2, 4, 8, 16, 32});
    const int P = pick({16, 32, 64, 128, 256});
    const int n_layers = 1 + rnd(3);
    std::vector<int32_t> ctx(size_t(B) + 1), ql(size_t(B) + 1), reserve(size_t(B) + 1);
    for (int b = 0; b < B; ++b) {
      ctx[b] = rnd(4) == 0 ? rnd(70) : rnd(2600);
      ql[b] = std::min(ctx[b], pick({0, 1, 2, 7, 64, 300, 5000}));
      reserve[b] = pick({0, 0, 1, 37, 700});
    }
    std::vector<sp_head_policy> pol(size_t(n_layers) * Hkv);
    for (auto& p : pol) p = random_policy();
    CHECK(check_lengths_policy(B, ctx.data(), ql.data(), Hkv, pol.data()) == SP_OK, "valid args");
    Layout lay;
    CHECK(make_layout_layers(n_layers, B, ctx.data(), ql.data(), Hkv, pol.data(), P, nullptr, &lay) == SP_OK, "layers");
    check_layout(lay, n_layers, B, Hkv, ctx.data(), ql.data(), pol, P, nullptr);
    // growable (one layer, no adaptive heads; growing retrieval heads need a query chunk)
    std::vector<sp_head_policy> gpol(pol.begin(), pol.begin() + Hkv);
    for (auto& p : gpol)
      if (p.kind == SP_LOCAL_ADAPTIVE) p = sp_head_policy{SP_LOCAL, p.sink, 100};
    for (int b = 0; b < B; ++b)
      if (ctx[b] < 1 || ql[b] < 1) reserve[b] = 0;
    if (check_growable(B, ctx.data(), ql.data(), reserve.data(), Hkv, gpol.data()) == SP_OK) {
      Layout g;
      CHECK(make_layout_layers(1, B, ctx.data(), ql.data(), Hkv, gpol.data(), P, reserve.data(), &g) == SP_OK, "growable");
      check_layout(g, 1, B, Hkv, ctx.data(), ql.data(), gpol, P, reserve.data());
    }
    Shape s{};
    s.mode = kModePaged, s.dtype = pick({0, 1}), s.B = B, s.Hq = Hkv * G, s.Hkv = Hkv;
    s.D = pick({64, 128}), s.P = P, s.ctx_len = ctx.data(), s.q_len = ql.data(), s.pol = pol.data();
    CHECK(check_shape(s) == SP_OK, "shape");
    const int slots = pick({1, 7, 512, 2048});
    check_plan(s, pol, slots, false);
    bool retrieval = false;
    for (int h = 0; h < Hkv; ++h) retrieval |= pol[size_t(h)].kind == SP_RETRIEVAL;
    if (!retrieval) {
      Shape d = s;
      d.mode = kModeDense, d.P = 64;
      check_plan(d, pol, slots, false);
    }
    if (G <= kDecodeRows) {
      std::vector<int32_t> ones(size_t(B) + 1, 1), hint(size_t(B) + 1, 1);
      for (int b = 0; b < B; ++b) hint[b] = std::max(1, ctx[b]);
      Shape td = s;
      td.ctx_len = hint.data(), td.q_len = ones.data();
      check_plan(td, pol, slots, true);
    }
    plans += 1;
  }
  printf("planner_check: %d trials, %d failures\n", plans, g_fail);
  return g_fail == 0 ? 0 : 1;
}
