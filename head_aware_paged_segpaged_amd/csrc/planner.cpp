// Host planning: validation, per-head page layout, attention work list.
//
// Layout rules (page "RedKnot SegPagedAttention runtime design", section 3): every (layer,
// head, segment) owns contiguous virtual pages; GLOBAL heads keep the whole context, LOCAL
// heads only the sink and the recent tokens any query of the chunk can see. The work list
// realises section 4 of the same page: every (query head, KV head) pair in one launch, each
// head walking only its own stored tokens.
#include "planner.h"

#include <algorithm>
#include <cstring>
#include <numeric>

namespace sp {

namespace {

constexpr int64_t kInt32Max = 0x7fffffffLL;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Number of 64-aligned KV steps covering [begin, end) of a segment.
int32_t range_steps(const Range& r) {
  if (r.end <= r.begin) return 0;
  return int32_t(ceil_div(r.end, kChunk) - r.begin / kChunk);
}

uint64_t fnv(uint64_t h, uint64_t v) {
  for (int i = 0; i < 8; ++i) {
    h ^= (v >> (8 * i)) & 0xff;
    h *= 0x100000001b3ull;
  }
  return h;
}

}  // namespace

sp_status check_dtype_dim(int32_t dtype, int32_t D) {
  if (dtype != SP_BF16 && dtype != SP_F32) return SP_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return SP_ERR_UNSUPPORTED;
  return SP_OK;
}

sp_status check_page_size(int32_t P) {
  if (P != 16 && P != 32 && P != 64 && P != 128 && P != 256) return SP_ERR_UNSUPPORTED;
  return SP_OK;
}

sp_status check_lengths_policy(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                               int32_t Hkv, const sp_head_policy* pol) {
  if (B < 0 || Hkv < 1) return SP_ERR_INVALID_ARG;
  if (B > 0 && (ctx_len == nullptr || q_len == nullptr)) return SP_ERR_INVALID_ARG;
  if (pol == nullptr) return SP_ERR_INVALID_ARG;
  for (int32_t h = 0; h < Hkv; ++h) {
    if (pol[h].kind == SP_GLOBAL) continue;
    if (pol[h].kind != SP_LOCAL && pol[h].kind != SP_LOCAL_ADAPTIVE &&
        pol[h].kind != SP_RETRIEVAL)
      return SP_ERR_INVALID_ARG;
    if (pol[h].sink < 0 || pol[h].window < 1) return SP_ERR_INVALID_ARG;
    if (pol[h].kind == SP_RETRIEVAL && pol[h].window > 1000) return SP_ERR_INVALID_ARG;
  }
  int64_t tot_ctx = 0, tot_q = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (ctx_len[b] < 0 || q_len[b] < 0 || q_len[b] > ctx_len[b]) return SP_ERR_INVALID_ARG;
    tot_ctx += ctx_len[b];
    tot_q += q_len[b];
  }
  if (tot_ctx > kInt32Max || tot_q > kInt32Max) return SP_ERR_UNSUPPORTED;
  return SP_OK;
}

sp_status check_shape(const Shape& s) {
  sp_status st = check_dtype_dim(s.dtype, s.D);
  if (st != SP_OK) return st;
  if (s.mode == kModePaged) {
    st = check_page_size(s.P);
    if (st != SP_OK) return st;
  }
  if (s.Hkv < 1 || s.Hq < 1 || s.Hq % s.Hkv != 0) return SP_ERR_INVALID_ARG;
  if (s.mode == kModeDense && s.pol != nullptr) {  // its mask is positional only
    for (int32_t h = 0; h < s.Hkv; ++h)
      if (s.pol[h].kind == SP_RETRIEVAL) return SP_ERR_UNSUPPORTED;
  }
  if (s.Hq / s.Hkv > kTileRows) return SP_ERR_UNSUPPORTED;
  st = check_lengths_policy(s.B, s.ctx_len, s.q_len, s.Hkv, s.pol);
  if (st != SP_OK) return st;
  int64_t tot_q = 0;
  for (int32_t b = 0; b < s.B; ++b) tot_q += s.q_len[b];
  if (tot_q * s.Hq > kInt32Max) return SP_ERR_UNSUPPORTED;  // int32 O/Q row ids in kernels
  return SP_OK;
}

sp_head_policy effective_policy(const sp_head_policy& pol, int32_t L) {
  if (pol.kind != SP_LOCAL_ADAPTIVE) return pol;
  return sp_head_policy{SP_LOCAL, pol.sink, std::max<int32_t>(1, L / pol.window)};
}

void retrieval_counts(const sp_head_policy& pol, int32_t L, int32_t q, int32_t* n_sink,
                      int32_t* n_kept) {
  const int64_t prefix = std::max<int64_t>(0, int64_t(L) - q);
  const int64_t s = std::min<int64_t>(pol.sink, prefix);
  *n_sink = int32_t(s);
  *n_kept = int32_t(ceil_div(int64_t(pol.window) * (prefix - s), 1000));
}

int head_segments(const sp_head_policy& pol_in, int32_t L, int32_t q, int32_t out_pos[2],
                  int32_t out_ntok[2]) {
  const sp_head_policy pol = effective_policy(pol_in, L);
  if (L <= 0) return 0;
  if (pol.kind == SP_GLOBAL) {
    out_pos[0] = 0;
    out_ntok[0] = L;
    return 1;
  }
  if (pol.kind == SP_RETRIEVAL) {
    // The kept prefix tokens, compacted (positions come from the build's keep list), then
    // the query chunk.
    int32_t s = 0, k = 0, n = 0;
    retrieval_counts(pol, L, q, &s, &k);
    if (s + k > 0) {
      out_pos[n] = 0;
      out_ntok[n++] = s + k;
    }
    if (q > 0) {
      out_pos[n] = L - q;
      out_ntok[n++] = q;
    }
    return n;
  }
  const int64_t s = std::min<int64_t>(pol.sink, L);
  const int64_t r0 = std::max<int64_t>(0, int64_t(L) - q - pol.window + 1);
  if (r0 <= s) {
    out_pos[0] = 0;
    out_ntok[0] = L;
    return 1;
  }
  if (s == 0) {
    out_pos[0] = int32_t(r0);
    out_ntok[0] = int32_t(L - r0);
    return 1;
  }
  out_pos[0] = 0;
  out_ntok[0] = int32_t(s);
  out_pos[1] = int32_t(r0);
  out_ntok[1] = int32_t(L - r0);
  return 2;
}

sp_status check_growable(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                         const int32_t* reserve, int32_t Hkv, const sp_head_policy* pol) {
  if (B > 0 && reserve == nullptr) return SP_ERR_INVALID_ARG;
  bool retrieval = false;
  for (int32_t h = 0; h < Hkv; ++h) {
    if (pol[h].kind == SP_LOCAL_ADAPTIVE) return SP_ERR_UNSUPPORTED;
    retrieval |= pol[h].kind == SP_RETRIEVAL;
  }
  for (int32_t b = 0; b < B; ++b) {
    if (reserve[b] < 0 || (reserve[b] > 0 && ctx_len[b] < 1)) return SP_ERR_INVALID_ARG;
    // a growing retrieval head appends to its query chunk, which must exist
    if (retrieval && reserve[b] > 0 && q_len[b] < 1) return SP_ERR_INVALID_ARG;
    if (int64_t(ctx_len[b]) + reserve[b] > kInt32Max) return SP_ERR_UNSUPPORTED;
  }
  return SP_OK;
}

void owned_pages(const sp_head_policy& pol, int nseg, const int32_t pos[2],
                 const int32_t ntok[2], int64_t L, int64_t lmax, int32_t P, int64_t own[2]) {
  for (int s = 0; s < nseg; ++s) own[s] = ceil_div(ntok[s], P);
  if (nseg == 0 || lmax <= L) return;
  if (pol.kind == SP_GLOBAL) {
    own[0] = ceil_div(lmax, P);
    return;
  }
  if (pol.kind == SP_RETRIEVAL) {  // the query chunk (last segment) grows, the kept prefix not
    own[nseg - 1] = ceil_div(int64_t(ntok[nseg - 1]) + (lmax - L), P);
    return;
  }
  const int64_t W = pol.window, S = pol.sink;
  const int64_t ring_max = W + P - 1;  // most tokens a ring holds once it recycles pages
  if (S > 0 && nseg == 1) {
    // Sink and window in one segment (0, L): grows whole until the window start reaches the
    // first page boundary past the sink, then becomes sink pages + a ring from that boundary.
    const int64_t s_pages = ceil_div(S, P), s_pg = s_pages * P;
    int64_t o = std::max(own[0], ceil_div(std::min(lmax, s_pg + W - 1), P));
    if (lmax >= s_pg + W) o = std::max(o, s_pages + ceil_div(std::min(lmax - s_pg, ring_max), P));
    own[0] = o;
    return;
  }
  const int r = nseg - 1;  // the ring: the only segment (sink 0) or the one after the sink
  own[r] = std::max(own[r], ceil_div(std::min(lmax - pos[r], ring_max), P));
}

sp_status make_layout(int32_t B, const int32_t* ctx_len, const int32_t* q_len, int32_t Hkv,
                      const sp_head_policy* pol, int32_t P, Layout* out) {
  return make_layout_layers(1, B, ctx_len, q_len, Hkv, pol, P, nullptr, out);
}

sp_status make_layout_layers(int32_t n_layers, int32_t B, const int32_t* ctx_len,
                             const int32_t* q_len, int32_t Hkv, const sp_head_policy* pol,
                             int32_t P, const int32_t* reserve, Layout* out) {
  out->heads.assign(size_t(n_layers) * B * Hkv, HeadLayout{});
  int64_t v = 0;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t l = 0; l < n_layers; ++l) {
      for (int32_t h = 0; h < Hkv; ++h) {
        HeadLayout& hl = out->heads[(size_t(l) * B + b) * Hkv + h];
        int32_t pos[2] = {0, 0}, ntok[2] = {0, 0};
        const sp_head_policy& hp = pol[size_t(l) * Hkv + h];
        hl.nseg = head_segments(hp, ctx_len[b], q_len[b], pos, ntok);
        hl.kv_len = 0;
        int64_t own[2] = {0, 0};
        owned_pages(hp, hl.nseg, pos, ntok, ctx_len[b],
                    int64_t(ctx_len[b]) + (reserve ? reserve[b] : 0), P, own);
        for (int s = 0; s < 2; ++s) {
          Segment& sg = hl.seg[s];
          if (s < hl.nseg) {
            if (v + own[s] > kInt32Max) return SP_ERR_UNSUPPORTED;
            sg.pos = pos[s];
            sg.ntok = ntok[s];
            sg.vstart = int32_t(v);
            sg.npages = int32_t(own[s]);
            v += sg.npages;
            hl.kv_len += ntok[s];
          } else {
            sg = Segment{0, 0, int32_t(v), 0};
          }
          if (v > kInt32Max) return SP_ERR_UNSUPPORTED;
        }
      }
    }
  }
  out->n_virt = v;
  return SP_OK;
}

void layout_tables(const Layout& lay, int32_t n_heads_total, int32_t* seg_table,
                   int32_t* kv_len) {
  for (int32_t i = 0; i < n_heads_total; ++i) {
    const HeadLayout& hl = lay.heads[i];
    for (int s = 0; s < 2; ++s) {
      int32_t* e = seg_table + (size_t(i) * 2 + s) * 4;
      e[0] = hl.seg[s].pos;
      e[1] = hl.seg[s].ntok;
      e[2] = hl.seg[s].vstart;
      e[3] = hl.seg[s].npages;
    }
    kv_len[i] = hl.kv_len;
  }
}

uint64_t shape_signature(const Shape& s, int32_t slots_prefill, int32_t slots_decode) {
  uint64_t h = 0xcbf29ce484222325ull;
  const int64_t fields[] = {s.mode, s.dtype, s.B, s.Hq, s.Hkv, s.D,
                            s.mode == kModePaged ? s.P : 0, slots_prefill, slots_decode};
  for (int64_t f : fields) h = fnv(h, uint64_t(f));
  for (int32_t b = 0; b < s.B; ++b) h = fnv(h, (uint64_t(uint32_t(s.ctx_len[b])) << 32) |
                                                   uint32_t(s.q_len[b]));
  for (int32_t i = 0; i < s.Hkv; ++i) {
    h = fnv(h, uint64_t(uint32_t(s.pol[i].kind)));
    if (s.pol[i].kind != SP_GLOBAL)
      h = fnv(h, (uint64_t(uint32_t(s.pol[i].sink)) << 32) | uint32_t(s.pol[i].window));
  }
  return h;
}

uint64_t table_decode_signature(const Shape& s, int32_t slots_decode) {
  uint64_t h = 0xcbf29ce484222325ull;
  const int64_t fields[] = {kModeTableDecode, s.dtype, s.B, s.Hq, s.Hkv, s.D, s.P, slots_decode};
  for (int64_t f : fields) h = fnv(h, uint64_t(f));
  for (int32_t i = 0; i < s.Hkv; ++i) {
    h = fnv(h, uint64_t(uint32_t(s.pol[i].kind)));
    if (s.pol[i].kind != SP_GLOBAL)
      h = fnv(h, (uint64_t(uint32_t(s.pol[i].sink)) << 32) | uint32_t(s.pol[i].window));
  }
  return h;
}

void needed_kernels(const Shape& s, bool* prefill, bool* decode) {
  const int32_t G = s.Hq / s.Hkv;
  *prefill = *decode = false;
  for (int32_t b = 0; b < s.B; ++b) {
    if (s.q_len[b] == 0) continue;
    if (int64_t(s.q_len[b]) * G <= kDecodeRows)
      *decode = true;
    else
      *prefill = true;
  }
}

namespace {

// The KV ranges a block of queries at positions [pmin, pmax] of one head must read.
void tile_ranges(const Shape& s, const HeadLayout* hl, const sp_head_policy& pol, int32_t pmin,
                 int32_t pmax, int32_t L, Range* ra, Range* rb) {
  *ra = Range{0, 0, 0};
  *rb = Range{0, 0, 0};
  if (s.mode == kModeDense || pol.kind == SP_GLOBAL) {
    *ra = Range{0, 0, pmax + 1};
    return;
  }
  if (pol.kind == SP_RETRIEVAL) {
    // Every kept prefix token is visible to every query of the chunk; the chunk (the last
    // segment, starting at position L - q) is read up to the block's last query.
    const Segment& chunk = hl->seg[hl->nseg - 1];
    if (hl->nseg == 2) {
      *ra = Range{0, 0, hl->seg[0].ntok};
      *rb = Range{1, 0, pmax + 1 - chunk.pos};
    } else {
      *ra = Range{0, 0, pmax + 1 - chunk.pos};
    }
    return;
  }
  const int32_t sink = std::min(pol.sink, L);
  const int32_t lo = int32_t(std::max<int64_t>(0, int64_t(pmin) - pol.window + 1));
  if (hl->nseg == 1 && hl->seg[0].pos == 0) {  // one merged segment (0, L)
    if (lo <= sink) {
      *ra = Range{0, 0, pmax + 1};
    } else {
      if (sink > 0) *ra = Range{0, 0, sink};
      *rb = Range{0, lo, pmax + 1};
    }
  } else if (hl->nseg == 1) {  // recent part only (sink 0)
    const int32_t r0 = hl->seg[0].pos;
    *ra = Range{0, lo - r0, pmax + 1 - r0};
  } else {  // sink segment + recent segment
    const int32_t r0 = hl->seg[1].pos;
    *ra = Range{0, 0, sink};
    *rb = Range{1, lo - r0, pmax + 1 - r0};
  }
  if (ra->end <= ra->begin) {
    *ra = *rb;
    *rb = Range{0, 0, 0};
  }
}

struct Tile {
  WorkItem w;
  int32_t steps;
  int32_t split;   // index of this split within its tile
  int32_t nsplit;  // splits of its tile
};

// Splits long tiles along KV so that no item is much longer than the average load of one
// work-group slot (and no shorter than min_split steps), then returns the items and the
// combine list. Decode items are cut to half that average when it is long (above 64 steps):
// the last items of the launch then end closer together, which outweighs the extra partials
// (32K-128K contexts: -3.7 %; with shorter contexts the finer cut costs more than it saves).
// Small decode batches, whose average is below 32 steps, get items down to 8 steps, so that a
// few long heads still spread over the whole chip (one 94K-context request: 0.113 -> 0.054 ms;
// four requests: 0.117 -> 0.081 ms; 64 requests unchanged).
void split_tiles(std::vector<Tile>& tiles, int32_t slots, int32_t min_split, int32_t kind,
                 std::vector<Tile>* items, std::vector<CombineItem>* combine, int32_t* n_part) {
  int64_t total = 0;
  for (const Tile& t : tiles) total += t.steps + kItemOverhead;
  int64_t avg = slots > 0 ? ceil_div(total, slots) : total;
  if (kind == 1 && avg > 64) avg /= 2;
  const int32_t target = int32_t(std::max<int64_t>(min_split, avg));
  for (const Tile& t : tiles) {
    const int32_t ns = int32_t(std::max<int64_t>(1, ceil_div(t.steps, target)));
    if (ns == 1) {
      Tile x = t;
      x.w.part = -1;
      x.nsplit = 1;
      items->push_back(x);
      continue;
    }
    const int32_t part0 = *n_part;
    *n_part += ns;
    for (int32_t k = 0; k < ns; ++k) {
      Tile x = t;
      const int32_t c0 = int32_t(int64_t(t.steps) * k / ns);
      const int32_t c1 = int32_t(int64_t(t.steps) * (k + 1) / ns);
      x.w.c_begin = c0;
      x.w.c_end = c1;
      x.w.part = part0 + k;
      x.steps = c1 - c0;
      x.split = k;
      x.nsplit = ns;
      items->push_back(x);
    }
    combine->push_back(CombineItem{t.w.b, t.w.h, t.w.tq0, t.w.nq, part0, ns, t.w.q_row0, kind});
  }
}

// Cuts the locality-ordered items into kXcds contiguous runs of about equal cost (one queue
// per XCD, so tiles that read the same KV share an L2), then orders each queue longest first.
void make_queues(std::vector<Tile>& items, std::vector<WorkItem>* out, int32_t* bounds) {
  std::stable_sort(items.begin(), items.end(), [](const Tile& a, const Tile& b) {
    if (a.w.b != b.w.b) return a.w.b < b.w.b;
    if (a.w.h != b.w.h) return a.w.h < b.w.h;
    if (a.split != b.split) return a.split < b.split;
    return a.w.tq0 < b.w.tq0;
  });
  int64_t total = 0;
  for (const Tile& t : items) total += t.steps + kItemOverhead;
  std::vector<int32_t> cut(kXcds + 1, int32_t(items.size()));
  cut[0] = 0;
  int64_t acc = 0;
  int x = 1;
  for (size_t i = 0; i < items.size() && x < kXcds; ++i) {
    acc += items[i].steps + kItemOverhead;
    while (x < kXcds && acc * kXcds >= total * x) cut[x++] = int32_t(i + 1);
  }
  out->clear();
  for (int q = 0; q < kXcds; ++q) {
    std::stable_sort(items.begin() + cut[q], items.begin() + cut[q + 1],
                     [](const Tile& a, const Tile& b) { return a.steps > b.steps; });
    bounds[q] = int32_t(out->size());
    for (int32_t i = cut[q]; i < cut[q + 1]; ++i) out->push_back(items[i].w);
  }
  bounds[kXcds] = int32_t(out->size());
}

}  // namespace

sp_status make_plan(const Shape& s, int32_t slots_prefill, int32_t slots_decode, Plan* out,
                    bool table_decode) {
  Layout lay;
  if (s.mode == kModePaged) {
    sp_status st = make_layout(s.B, s.ctx_len, s.q_len, s.Hkv, s.pol, s.P, &lay);
    if (st != SP_OK) return st;
  }
  const int32_t G = s.Hq / s.Hkv;
  std::vector<Tile> pre_tiles, dec_tiles;
  int32_t q_row0 = 0, kv_row0 = 0;
  for (int32_t b = 0; b < s.B; ++b) {
    const int32_t L = s.ctx_len[b], nq = s.q_len[b];
    if (nq > 0) {
      const bool dec = int64_t(nq) * G <= kDecodeRows;
      const int32_t bq = dec ? nq : std::max(1, kTileRows / G);
      const int32_t p0 = L - nq;
      for (int32_t h = 0; h < s.Hkv; ++h) {
        const HeadLayout* hl =
            s.mode == kModePaged ? &lay.heads[size_t(b) * s.Hkv + h] : nullptr;
        for (int32_t t0 = 0; t0 < nq; t0 += bq) {
          const int32_t nt = std::min(bq, nq - t0);
          const int32_t pmin = p0 + t0, pmax = pmin + nt - 1;
          Range ra, rb;
          tile_ranges(s, hl, effective_policy(s.pol[h], L), pmin, pmax, L, &ra, &rb);
          Tile t{};
          WorkItem& w = t.w;
          w.b = b;
          w.h = h;
          w.tq0 = t0;
          w.nq = nt;
          w.ra_seg = ra.seg;
          w.ra_begin = ra.begin;
          w.ra_end = ra.end;
          w.rb_seg = rb.seg;
          w.rb_begin = rb.begin;
          w.rb_end = rb.end;
          t.steps = range_steps(ra) + range_steps(rb);
          w.c_begin = 0;
          w.c_end = t.steps;
          w.part = -1;
          w.q_row0 = q_row0;
          w.p0 = p0;
          w.kv_row0 = kv_row0;
          t.split = 0;
          (dec ? dec_tiles : pre_tiles).push_back(t);
        }
      }
    }
    q_row0 += nq;
    kv_row0 += L;
  }

  std::vector<Tile> pre_items, dec_items;
  std::vector<CombineItem> combine;
  int32_t n_part_pre = 0, n_part_dec = 0;
  split_tiles(pre_tiles, slots_prefill, /*min_split=*/8, 0, &pre_items, &combine, &n_part_pre);
  split_tiles(dec_tiles, slots_decode, /*min_split=*/8, 1, &dec_items, &combine, &n_part_dec);
  if (table_decode) {
    // Each item keeps only its split fraction (split c_begin of c_end); the kernel takes the
    // head's stored tokens and query position from the device tables when it runs. Groups of
    // up to kDecodeRows query heads are decode items; larger groups (one query, G rows) are
    // tiles of the prefill kernel.
    for (std::vector<Tile>* v : {&pre_items, &dec_items}) {
      for (Tile& t : *v) {
        WorkItem& w = t.w;
        w.ra_seg = -1;
        w.ra_begin = w.ra_end = 0;
        w.rb_seg = 0;
        w.rb_begin = w.rb_end = 0;
        w.c_begin = t.split;
        w.c_end = t.nsplit;
        w.p0 = 0;
      }
    }
  }

  WsHeader& hd = out->hdr;
  std::memset(&hd, 0, sizeof(hd));
  make_queues(pre_items, &out->prefill, hd.prefill_q);
  make_queues(dec_items, &out->decode, hd.decode_q);
  out->combine = combine;
  // The kernels' policy table: one effective (kind, sink, window) per (request, KV head).
  out->policy.resize(size_t(std::max(s.B, 1)) * s.Hkv * 3);
  for (int32_t b = 0; b < s.B; ++b) {
    for (int32_t h = 0; h < s.Hkv; ++h) {
      const sp_head_policy e = effective_policy(s.pol[h], s.ctx_len[b]);
      int32_t* d = &out->policy[(size_t(b) * s.Hkv + h) * 3];
      // A RETRIEVAL head stores only tokens its queries may see, bar the chunk's causal edge.
      d[0] = e.kind == SP_RETRIEVAL ? int32_t(SP_GLOBAL) : e.kind;
      d[1] = e.kind == SP_LOCAL ? e.sink : 0;
      d[2] = e.kind == SP_LOCAL ? e.window : 1;
    }
  }

  hd.magic = kMagic;
  hd.signature = table_decode ? table_decode_signature(s, slots_decode)
                              : shape_signature(s, slots_prefill, slots_decode);
  hd.n_prefill = int32_t(out->prefill.size());
  hd.n_decode = int32_t(out->decode.size());
  hd.n_combine = int32_t(out->combine.size());
  hd.n_part_pre = n_part_pre;
  hd.n_part_dec = n_part_dec;
  size_t off = kHeaderBytes;
  hd.off_prefill = int64_t(off);
  off = align256(off + out->prefill.size() * sizeof(WorkItem));
  hd.off_decode = int64_t(off);
  off = align256(off + out->decode.size() * sizeof(WorkItem));
  hd.off_combine = int64_t(off);
  off = align256(off + out->combine.size() * sizeof(CombineItem));
  hd.off_policy = int64_t(off);
  off = align256(off + out->policy.size() * sizeof(int32_t));
  out->upload_bytes = off;
  const size_t fbytes = 4;
  hd.off_part_pre = int64_t(off);
  off = align256(off + size_t(n_part_pre) * kTileRows * s.D * fbytes);
  hd.off_ml_pre = int64_t(off);
  off = align256(off + size_t(n_part_pre) * kTileRows * 2 * fbytes);
  hd.off_part_dec = int64_t(off);
  off = align256(off + size_t(n_part_dec) * kDecodeRows * s.D * fbytes);
  hd.off_ml_dec = int64_t(off);
  off = align256(off + size_t(n_part_dec) * kDecodeRows * 2 * fbytes);
  out->bytes = off;
  hd.bytes = off;
  return SP_OK;
}

void serialize_plan(const Plan& plan, std::vector<uint8_t>* buf) {
  buf->assign(plan.upload_bytes, 0);
  uint8_t* p = buf->data();
  std::memcpy(p, &plan.hdr, sizeof(WsHeader));
  if (!plan.prefill.empty())
    std::memcpy(p + plan.hdr.off_prefill, plan.prefill.data(),
                plan.prefill.size() * sizeof(WorkItem));
  if (!plan.decode.empty())
    std::memcpy(p + plan.hdr.off_decode, plan.decode.data(),
                plan.decode.size() * sizeof(WorkItem));
  if (!plan.combine.empty())
    std::memcpy(p + plan.hdr.off_combine, plan.combine.data(),
                plan.combine.size() * sizeof(CombineItem));
  std::memcpy(p + plan.hdr.off_policy, plan.policy.data(), plan.policy.size() * sizeof(int32_t));
}

}  // namespace sp
