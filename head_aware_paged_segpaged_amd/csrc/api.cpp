// C ABI of libsegpaged (declared in include/segpaged.h): argument validation, table uploads
// and kernel launches. Every argument is checked before anything is queued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "launch.h"
#include "planner.h"
#include "segpaged.h"

using namespace sp;

namespace {

sp_status device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SP_ERR_HIP;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return SP_ERR_HIP;
  *cus = n > 0 ? n : 1;
  return SP_OK;
}

// A stream of the library's own per device, with two events to fork it from a caller's stream
// and join it back (RETRIEVAL selection runs there, beside the scatter). Default priority;
// created on first use and kept until the process ends. `mu` orders the fork / join sequences
// of concurrent calls.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};

sp_status side_stream(SideStream** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static SideStream sides[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(mu);
  SideStream& s = sides[dev];
  if (s.stream == nullptr) {
    if (hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess ||
        hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess)
      return SP_ERR_HIP;
  }
  *out = &s;
  return SP_OK;
}

// Persistent grid sizes for one shape: resident work groups of each kernel.
sp_status grids(const Shape& s, int32_t* g_pre, int32_t* g_dec) {
  int cus = 0;
  sp_status st = device_cus(&cus);
  if (st != SP_OK) return st;
  *g_pre = cus * attention_occupancy(s.dtype, s.D, s.mode, false);
  *g_dec = cus * attention_occupancy(s.dtype, s.D, s.mode, true);
  return SP_OK;
}

Shape make_shape(int32_t mode, sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                 int32_t P, const int32_t* ctx_len, const int32_t* q_len,
                 const sp_head_policy* pol) {
  Shape s;
  s.mode = mode;
  s.dtype = int32_t(dtype);
  s.B = B;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.D = D;
  s.P = mode == kModePaged ? P : 64;
  s.ctx_len = ctx_len;
  s.q_len = q_len;
  s.pol = pol;
  return s;
}

sp_status workspace_size(const Shape& s, size_t* bytes) {
  if (bytes == nullptr) return SP_ERR_INVALID_ARG;
  sp_status st = check_shape(s);
  if (st != SP_OK) return st;
  int32_t gp = 0, gd = 0;
  st = grids(s, &gp, &gd);
  if (st != SP_OK) return st;
  Plan plan;
  st = make_plan(s, gp, gd, &plan);
  if (st != SP_OK) return st;
  *bytes = plan.bytes;
  return SP_OK;
}

// Item counts of recently planned shapes, by plan signature. segpaged_attention skips the
// combine launch for a signature planned here with no KV-split item, and sizes the decode grid
// by its decode item count (see decode_grid). The plan is a function of what the signature
// hashes (shapes, lengths, policies, grid sizes), so an entry never goes stale; a signature not
// found here (evicted, or planned in another process) launches the full decode grid and the
// combine, whose kernel reads the item count from the workspace and returns at once.
class PlanCounts {
 public:
  struct Counts {
    int32_t n_combine, n_decode;
  };
  void put(uint64_t sig, Counts c) {
    std::lock_guard<std::mutex> g(mu_);
    for (Entry& e : ent_)
      if (e.used && e.sig == sig) {
        e.c = c;
        return;
      }
    ent_[next_] = Entry{sig, c, true};
    next_ = (next_ + 1) % kEntries;
  }
  bool get(uint64_t sig, Counts* c) {
    std::lock_guard<std::mutex> g(mu_);
    for (const Entry& e : ent_)
      if (e.used && e.sig == sig) {
        *c = e.c;
        return true;
      }
    return false;
  }

 private:
  static constexpr int kEntries = 64;
  struct Entry {
    uint64_t sig;
    Counts c;
    bool used;
  };
  std::mutex mu_;
  Entry ent_[kEntries] = {};
  int next_ = 0;
};

PlanCounts& plan_counts() {
  static PlanCounts c;
  return c;
}

void remember_plan(const Plan& plan) {
  plan_counts().put(plan.hdr.signature, PlanCounts::Counts{plan.hdr.n_combine, plan.hdr.n_decode});
}

// Work groups of a decode launch. The plan cuts decode items for gd slots (two one-wave work
// groups per SIMD), and a launch with at most gd items runs them all at once. With more items
// than that the launch has one work group per SIMD instead: the second wave of a SIMD gets its
// issue slots only after the first (measured 1.5-2.5x slower per KV step), so a second wave
// helps only while it has an item of its own, and the queues balance the rest.
constexpr int32_t kSimdsPerCu = 4;  // CDNA compute units: four SIMDs each

int32_t decode_grid(uint64_t sig, int32_t gd) {
  PlanCounts::Counts c{0, 0};
  int cus = 0;
  if (!plan_counts().get(sig, &c) || c.n_decode <= gd || device_cus(&cus) != SP_OK) return gd;
  return std::max<int32_t>(1, std::min<int32_t>(gd, cus * kSimdsPerCu));
}

sp_status plan_into(const Shape& s, void* workspace, size_t ws_bytes, hipStream_t stream) {
  sp_status st = check_shape(s);
  if (st != SP_OK) return st;
  if (workspace == nullptr) return SP_ERR_INVALID_ARG;
  int32_t gp = 0, gd = 0;
  st = grids(s, &gp, &gd);
  if (st != SP_OK) return st;
  Plan plan;
  st = make_plan(s, gp, gd, &plan);
  if (st != SP_OK) return st;
  if (ws_bytes < plan.bytes) return SP_ERR_WORKSPACE_TOO_SMALL;
  std::vector<uint8_t> buf;
  serialize_plan(plan, &buf);
  if (hipMemcpyAsync(workspace, buf.data(), buf.size(), hipMemcpyHostToDevice, stream) !=
      hipSuccess)
    return SP_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SP_ERR_HIP;
  remember_plan(plan);
  return SP_OK;
}

sp_status run_attention(const Shape& s, const void* q, const void* k, const void* v,
                        int64_t n_phys, const int32_t* seg_table, const int32_t* kv_len,
                        const int32_t* v2p, float scale, void* o, void* workspace,
                        size_t ws_bytes, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  sp_status st = check_shape(s);
  if (st != SP_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return SP_ERR_INVALID_ARG;
  bool need_pre = false, need_dec = false;
  needed_kernels(s, &need_pre, &need_dec);
  if (!need_pre && !need_dec) {
    if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return SP_ERR_HIP;
    if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return SP_ERR_HIP;
    return SP_OK;
  }
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || workspace == nullptr)
    return SP_ERR_INVALID_ARG;
  if (s.mode == kModePaged &&
      (seg_table == nullptr || kv_len == nullptr || v2p == nullptr || n_phys < 1))
    return SP_ERR_INVALID_ARG;
  if (ws_bytes < size_t(kHeaderBytes)) return SP_ERR_WORKSPACE_TOO_SMALL;
  // Prefill with pages smaller than a KV step addresses rows from the pool start with 32-bit
  // byte offsets.
  if (need_pre && s.mode == kModePaged && s.P < kChunk &&
      n_phys * int64_t(s.P) * s.D * (s.dtype == SP_BF16 ? 2 : 4) > int64_t(0x7fffffff))
    return SP_ERR_UNSUPPORTED;
  int32_t gp = 0, gd = 0;
  st = grids(s, &gp, &gd);
  if (st != SP_OK) return st;

  AttnParams p;
  p.q = q;
  p.o = o;
  p.k = k;
  p.v = v;
  p.seg_table = seg_table;
  p.kv_len = kv_len;
  p.v2p = v2p;
  p.n_phys = n_phys;
  p.ws = static_cast<uint8_t*>(workspace);
  p.signature = shape_signature(s, gp, gd);
  p.ws_bytes = ws_bytes;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.G = s.Hq / s.Hkv;
  p.P = s.P;
  p.scale_log2 = scale * 1.4426950408889634f;

  if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return SP_ERR_HIP;
  if (need_pre && launch_attention(s.dtype, s.D, s.mode, false, gp, p, stream) != hipSuccess)
    return SP_ERR_HIP;
  if (need_dec && launch_attention(s.dtype, s.D, s.mode, true, decode_grid(p.signature, gd), p,
                                   stream) != hipSuccess)
    return SP_ERR_HIP;
  if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return SP_ERR_HIP;
  PlanCounts::Counts counts{0, 0};
  if (plan_counts().get(p.signature, &counts) && counts.n_combine == 0) return SP_OK;
  int cus = 0;
  st = device_cus(&cus);
  if (st != SP_OK) return st;
  if (launch_combine(s.dtype, s.D, 4 * cus, p, stream) != hipSuccess) return SP_ERR_HIP;
  return SP_OK;
}

// Arguments shared by the layout calls, for n_layers layers whose policies are [n_layers][Hkv].
sp_status check_layers(int32_t n_layers, int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                       int32_t Hkv, const sp_head_policy* pol, int32_t page_size) {
  if (n_layers < 1 || pol == nullptr) return SP_ERR_INVALID_ARG;
  sp_status st = check_page_size(page_size);
  if (st != SP_OK) return st;
  for (int32_t l = 0; l < n_layers; ++l) {
    st = check_lengths_policy(B, ctx_len, q_len, Hkv, pol + size_t(l) * Hkv);
    if (st != SP_OK) return st;
  }
  return SP_OK;
}

// Checks and layout of n_layers layers; growable (single layer) when `reserve` is not null.
sp_status layout_impl(int32_t n_layers, int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                      const int32_t* reserve, int32_t Hkv, const sp_head_policy* pol,
                      int32_t page_size, Layout* lay) {
  sp_status st = check_layers(n_layers, B, ctx_len, q_len, Hkv, pol, page_size);
  if (st != SP_OK) return st;
  if (reserve != nullptr) {
    if (n_layers != 1) return SP_ERR_INVALID_ARG;
    st = check_growable(B, ctx_len, q_len, reserve, Hkv, pol);
    if (st != SP_OK) return st;
  }
  return make_layout_layers(n_layers, B, ctx_len, q_len, Hkv, pol, page_size, reserve, lay);
}

// The kept lists of the RETRIEVAL heads of a single-layer layout, in (request, head) order:
// per (request, head) with a non-empty list, one selection task (its sink, then the top
// fraction of the other prefix tokens by importance, ascending; chosen on the device).
// offsets[b * Hkv + h] = start of (b, h) in row_pos (-1: none); *total = entries of row_pos.
void retrieval_tasks(int32_t B, const int32_t* ctx_len, const int32_t* q_len, int32_t Hkv,
                     const sp_head_policy* pol, std::vector<SelectTask>* tasks,
                     std::vector<int64_t>* offsets, int64_t* total) {
  offsets->assign(size_t(B) * Hkv, -1);
  int64_t row0 = 0, acc = 0;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t h = 0; h < Hkv; ++h) {
      if (pol[h].kind != SP_RETRIEVAL) continue;
      int32_t s = 0, k = 0;
      retrieval_counts(pol[h], ctx_len[b], q_len[b], &s, &k);
      if (s + k == 0) continue;
      (*offsets)[size_t(b) * Hkv + h] = acc;
      tasks->push_back(SelectTask{int32_t(acc), int32_t(row0), h, s, k, ctx_len[b] - q_len[b] - s});
      acc += s + k;
    }
    row0 += ctx_len[b];
  }
  *total = acc;
}

// Build of n_layers layers (growable when `reserve` is not null: single layer only).
sp_status build_impl(sp_dtype dtype, int32_t n_layers, int32_t B, int32_t Hkv, int32_t D,
                     int32_t page_size, const int32_t* ctx_len, const int32_t* q_len,
                     const int32_t* reserve, const sp_head_policy* pol, const void* k_dense,
                     const void* v_dense, const int32_t* free_pages, int64_t n_free,
                     int64_t n_phys, void* k_pool, void* v_pool, int32_t* seg_table,
                     int32_t* kv_len, int32_t* v2p, hipStream_t stream,
                     const float* importance = nullptr, int32_t* row_pos = nullptr) {
  sp_status st = check_dtype_dim(dtype, D);
  if (st != SP_OK) return st;
  if (n_free < 0 || n_phys < 0) return SP_ERR_INVALID_ARG;
  Layout lay;
  st = layout_impl(n_layers, B, ctx_len, q_len, reserve, Hkv, pol, page_size, &lay);
  if (st != SP_OK) return st;
  int64_t t_total = 0;
  for (int32_t b = 0; b < B; ++b) t_total += ctx_len[b];
  if (int64_t(n_layers) * t_total > 0x7fffffffLL) return SP_ERR_UNSUPPORTED;  // int32 rows
  if (B == 0) return SP_OK;
  if (seg_table == nullptr || kv_len == nullptr) return SP_ERR_INVALID_ARG;
  std::vector<SelectTask> tasks;
  std::vector<int64_t> keep_off;
  int64_t n_keep = 0;
  bool retrieval = false;
  for (size_t i = 0; i < size_t(n_layers) * Hkv; ++i) retrieval |= pol[i].kind == SP_RETRIEVAL;
  if (retrieval) {
    if (n_layers != 1) return SP_ERR_INVALID_ARG;
    retrieval_tasks(B, ctx_len, q_len, Hkv, pol, &tasks, &keep_off, &n_keep);
    if (n_keep > 0 && (importance == nullptr || row_pos == nullptr)) return SP_ERR_INVALID_ARG;
    if (n_keep > 0x7fffffffLL) return SP_ERR_UNSUPPORTED;
  }
  const int64_t n_virt = lay.n_virt;
  if (n_free < n_virt) return SP_ERR_POOL_TOO_SMALL;
  if (n_virt > 0) {
    if (free_pages == nullptr || v2p == nullptr || k_pool == nullptr || v_pool == nullptr ||
        k_dense == nullptr || v_dense == nullptr)
      return SP_ERR_INVALID_ARG;
    std::vector<uint8_t> seen(size_t(n_phys), 0);
    for (int64_t i = 0; i < n_virt; ++i) {
      const int32_t f = free_pages[i];
      if (f < 0 || f >= n_phys || seen[size_t(f)]) return SP_ERR_INVALID_ARG;
      seen[size_t(f)] = 1;
    }
  }
  // Tables: seg_table, kv_len and v2p. When the caller placed them back to back in one
  // allocation they go up in a single host-to-device copy (each copy from pageable memory
  // costs tens of microseconds of fixed overhead), else in three. A copy from pageable host
  // memory returns once the source has been staged, so the host buffer may go out of scope.
  const size_t n_heads = size_t(n_layers) * B * Hkv;
  const size_t n_tab = n_heads * 8, n_kl = n_heads;
  const bool adjacent = kv_len == seg_table + n_tab && (n_virt == 0 || v2p == kv_len + n_kl);
  std::vector<int32_t> host(n_tab + n_kl + (adjacent ? size_t(n_virt) : 0));
  layout_tables(lay, int32_t(n_heads), host.data(), host.data() + n_tab);
  if (adjacent) {
    if (n_virt > 0) std::memcpy(host.data() + n_tab + n_kl, free_pages, size_t(n_virt) * 4);
    if (hipMemcpyAsync(seg_table, host.data(), host.size() * 4, hipMemcpyHostToDevice,
                       stream) != hipSuccess)
      return SP_ERR_HIP;
  } else {
    if (hipMemcpyAsync(seg_table, host.data(), n_tab * 4, hipMemcpyHostToDevice, stream) !=
            hipSuccess ||
        hipMemcpyAsync(kv_len, host.data() + n_tab, n_kl * 4, hipMemcpyHostToDevice, stream) !=
            hipSuccess)
      return SP_ERR_HIP;
    if (n_virt > 0 && hipMemcpyAsync(v2p, free_pages, size_t(n_virt) * 4,
                                     hipMemcpyHostToDevice, stream) != hipSuccess)
      return SP_ERR_HIP;
  }
  // RETRIEVAL heads: the kept lists are chosen on the device by the selection kernel, on a
  // side stream forked from `stream`, while the scatter copies every other segment; the kept
  // prefixes are copied once the selection has joined back.
  SideStream* side = nullptr;
  if (!tasks.empty()) {
    st = side_stream(&side);
    if (st != SP_OK) return st;
  }
  std::unique_lock<std::mutex> side_lock;
  if (side != nullptr) {
    side_lock = std::unique_lock<std::mutex>(side->mu);
    if (hipEventRecord(side->fork, stream) != hipSuccess ||
        hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess)
      return SP_ERR_HIP;
    SelectParams sp_;
    std::memset(&sp_, 0, sizeof(sp_));
    sp_.imp = importance;
    sp_.row_pos = row_pos;
    sp_.t_total = int32_t(t_total);
    for (size_t t0 = 0; t0 < tasks.size(); t0 += kMaxSelectTasks) {
      sp_.n_tasks = int32_t(std::min<size_t>(kMaxSelectTasks, tasks.size() - t0));
      std::memcpy(sp_.t, tasks.data() + t0, size_t(sp_.n_tasks) * sizeof(SelectTask));
      if (launch_select(sp_, side->stream) != hipSuccess) return SP_ERR_HIP;
    }
    if (hipEventRecord(side->join, side->stream) != hipSuccess) return SP_ERR_HIP;
  }

  // Scatter: the chunks of each (layer, request) group are counted on the host; the groups'
  // chunk offsets, first dense rows and (retrieval) kept-prefix offsets travel in the kernel
  // arguments, so one launch covers as many groups as fit there (every workload here: all).
  const int32_t n_groups_all = n_layers * B;
  const bool gather = !keep_off.empty();
  // per group: chunks of the segments copied straight (phase 0/1) and of the kept prefixes
  std::vector<int32_t> g_plain(size_t(n_groups_all), 0), g_kept(size_t(n_groups_all), 0);
  std::vector<int32_t> g_row0(size_t(n_groups_all), 0);
  for (int32_t l = 0; l < n_layers; ++l) {
    int64_t row0 = int64_t(l) * t_total;  // dense K/V of layer l start at row l * sum(ctx_len)
    for (int32_t b = 0; b < B; ++b) {
      const size_t g = size_t(l) * B + b;
      int64_t plain = 0, kept = 0;
      for (int32_t h = 0; h < Hkv; ++h) {
        const HeadLayout& hl = lay.heads[g * Hkv + h];
        const bool has_kept = gather && keep_off[size_t(b) * Hkv + h] >= 0;
        for (int s_ = 0; s_ < hl.nseg; ++s_) {
          const int64_t c = (hl.seg[s_].ntok + kChunk - 1) / kChunk;
          (has_kept && s_ == 0 ? kept : plain) += c;
        }
      }
      g_plain[g] = int32_t(plain);
      g_kept[g] = int32_t(kept);
      g_row0[g] = int32_t(row0);
      row0 += ctx_len[b];
    }
  }
  BuildParams bp;
  std::memset(&bp, 0, sizeof(bp));
  bp.k = k_dense;
  bp.v = v_dense;
  bp.kp = k_pool;
  bp.vp = v_pool;
  bp.v2p = v2p;
  bp.row_pos = row_pos;
  bp.seg_table = seg_table;
  bp.Hkv = Hkv;
  bp.P = page_size;
  const int32_t per_group = 2 + (gather ? Hkv : 0);  // ints of kernel arguments per group
  auto scatter = [&](int32_t phase, const std::vector<int32_t>& g_chunks) -> sp_status {
    bp.phase = phase;
    for (int32_t g0 = 0; g0 < n_groups_all;) {
      int32_t n = 0;
      int64_t total = 0;
      while (g0 + n < n_groups_all && 1 + (n + 1) * per_group <= kBuildArgInts &&
             total + g_chunks[size_t(g0 + n)] <= 0x7fffffffLL) {
        total += g_chunks[size_t(g0 + n)];
        ++n;
      }
      if (n == 0) return SP_ERR_UNSUPPORTED;  // one group's descriptors do not fit
      bp.group0 = g0;
      bp.n_groups = n;
      int32_t* cb = bp.arr;
      int32_t* r0 = bp.arr + n + 1;
      int32_t* go = r0 + n;
      int32_t acc = 0;
      for (int32_t i = 0; i < n; ++i) {
        cb[i] = acc;
        acc += g_chunks[size_t(g0 + i)];
        r0[i] = g_row0[size_t(g0 + i)];
        if (gather) {
          const int32_t b = (g0 + i) % B;  // retrieval builds have one layer
          for (int32_t h = 0; h < Hkv; ++h) {
            const int64_t o = keep_off[size_t(b) * Hkv + h];
            go[size_t(i) * Hkv + h] = o < 0 ? -1 : int32_t(o);
          }
        }
      }
      cb[n] = acc;
      if (acc > 0 && launch_build(dtype, D, bp, acc, stream) != hipSuccess) return SP_ERR_HIP;
      g0 += n;
    }
    return SP_OK;
  };
  st = scatter(gather ? 1 : 0, g_plain);
  if (st != SP_OK) return st;
  if (side != nullptr && hipStreamWaitEvent(stream, side->join, 0) != hipSuccess)
    return SP_ERR_HIP;
  if (gather) return scatter(2, g_kept);
  return SP_OK;
}

// Shape of a table-driven decode call: one query per request; ctx_hint only balances the
// plan's KV splits (null: every request gets the same weight).
sp_status table_decode_shape(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t P, const int32_t* ctx_hint, const sp_head_policy* pol,
                             std::vector<int32_t>* hint, std::vector<int32_t>* ones, Shape* s) {
  if (B < 0) return SP_ERR_INVALID_ARG;
  hint->assign(size_t(B), 1);
  ones->assign(size_t(B), 1);
  for (int32_t b = 0; b < B; ++b) {
    if (ctx_hint != nullptr) {
      if (ctx_hint[b] < 1) return SP_ERR_INVALID_ARG;
      (*hint)[size_t(b)] = ctx_hint[b];
    }
  }
  *s = make_shape(kModePaged, dtype, B, Hq, Hkv, D, P, hint->data(), ones->data(), pol);
  sp_status st = check_shape(*s);
  if (st != SP_OK) return st;
  // Groups of up to kDecodeRows query heads run as decode items (one wave each), larger ones
  // (up to kTileRows, checked with the shape) as tiles of the prefill kernel.
  for (int32_t h = 0; h < Hkv; ++h)
    if (pol[h].kind == SP_LOCAL_ADAPTIVE) return SP_ERR_UNSUPPORTED;
  return SP_OK;
}

sp_status table_decode_plan(const Shape& s, Plan* plan) {
  int32_t gp = 0, gd = 0;
  sp_status st = grids(s, &gp, &gd);
  if (st != SP_OK) return st;
  return make_plan(s, gp, gd, plan, /*table_decode=*/true);
}

}  // namespace

extern "C" {

const char* segpaged_status_string(int status) {
  switch (status) {
    case SP_OK: return "SP_OK";
    case SP_ERR_INVALID_ARG: return "SP_ERR_INVALID_ARG: invalid argument";
    case SP_ERR_UNSUPPORTED: return "SP_ERR_UNSUPPORTED: unsupported shape, dtype or size";
    case SP_ERR_POOL_TOO_SMALL: return "SP_ERR_POOL_TOO_SMALL: free list shorter than needed";
    case SP_ERR_WORKSPACE_TOO_SMALL: return "SP_ERR_WORKSPACE_TOO_SMALL: workspace too small";
    case SP_ERR_HIP: return "SP_ERR_HIP: HIP runtime error";
    case SP_ERR_PLAN_MISMATCH: return "SP_ERR_PLAN_MISMATCH: workspace planned for other arguments";
    case SP_ERR_SEGMENT_FULL: return "SP_ERR_SEGMENT_FULL: no owned page left for an appended token";
    default: return "unknown status";
  }
}

sp_status segpaged_plan_pages(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                              int32_t Hkv, const sp_head_policy* pol, int32_t page_size,
                              int64_t* n_pages_needed) {
  return segpaged_plan_pages_layers(1, B, ctx_len, q_len, Hkv, pol, page_size, n_pages_needed);
}

sp_status segpaged_plan_pages_layers(int32_t n_layers, int32_t B, const int32_t* ctx_len,
                                     const int32_t* q_len, int32_t Hkv,
                                     const sp_head_policy* pol, int32_t page_size,
                                     int64_t* n_pages_needed) {
  if (n_pages_needed == nullptr) return SP_ERR_INVALID_ARG;
  Layout lay;
  sp_status st = layout_impl(n_layers, B, ctx_len, q_len, nullptr, Hkv, pol, page_size, &lay);
  if (st != SP_OK) return st;
  *n_pages_needed = lay.n_virt;
  return SP_OK;
}

sp_status segpaged_layout_tables(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                                 int32_t Hkv, const sp_head_policy* pol, int32_t page_size,
                                 int32_t* seg_table, int32_t* kv_len) {
  return segpaged_layout_tables_layers(1, B, ctx_len, q_len, Hkv, pol, page_size, seg_table,
                                       kv_len);
}

sp_status segpaged_layout_tables_layers(int32_t n_layers, int32_t B, const int32_t* ctx_len,
                                        const int32_t* q_len, int32_t Hkv,
                                        const sp_head_policy* pol, int32_t page_size,
                                        int32_t* seg_table, int32_t* kv_len) {
  if (seg_table == nullptr || kv_len == nullptr) return SP_ERR_INVALID_ARG;
  Layout lay;
  sp_status st = layout_impl(n_layers, B, ctx_len, q_len, nullptr, Hkv, pol, page_size, &lay);
  if (st != SP_OK) return st;
  layout_tables(lay, n_layers * B * Hkv, seg_table, kv_len);
  return SP_OK;
}

sp_status segpaged_retrieval_rows(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                                  int32_t Hkv, const sp_head_policy* pol, int64_t* n_rows) {
  if (n_rows == nullptr) return SP_ERR_INVALID_ARG;
  sp_status st = check_lengths_policy(B, ctx_len, q_len, Hkv, pol);
  if (st != SP_OK) return st;
  int64_t n = 0;
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t h = 0; h < Hkv; ++h) {
      if (pol[h].kind != SP_RETRIEVAL) continue;
      int32_t s = 0, k = 0;
      retrieval_counts(pol[h], ctx_len[b], q_len[b], &s, &k);
      n += s + k;
    }
  }
  *n_rows = n;
  return SP_OK;
}

sp_status segpaged_build_scored(sp_dtype dtype, int32_t B, int32_t Hkv, int32_t D,
                                int32_t page_size, const int32_t* ctx_len, const int32_t* q_len,
                                const int32_t* reserve, const sp_head_policy* pol,
                                const float* importance, const void* k_dense,
                                const void* v_dense, const int32_t* free_pages, int64_t n_free,
                                int64_t n_phys, void* k_pool, void* v_pool, int32_t* seg_table,
                                int32_t* kv_len, int32_t* v2p, int32_t* row_pos,
                                hipStream_t stream) {
  return build_impl(dtype, 1, B, Hkv, D, page_size, ctx_len, q_len, reserve, pol, k_dense,
                    v_dense, free_pages, n_free, n_phys, k_pool, v_pool, seg_table, kv_len, v2p,
                    stream, importance, row_pos);
}

sp_status segpaged_plan_pages_growable(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                                       const int32_t* reserve, int32_t Hkv,
                                       const sp_head_policy* pol, int32_t page_size,
                                       int64_t* n_pages_needed) {
  if (n_pages_needed == nullptr || reserve == nullptr) return SP_ERR_INVALID_ARG;
  Layout lay;
  sp_status st = layout_impl(1, B, ctx_len, q_len, reserve, Hkv, pol, page_size, &lay);
  if (st != SP_OK) return st;
  *n_pages_needed = lay.n_virt;
  return SP_OK;
}

sp_status segpaged_layout_tables_growable(int32_t B, const int32_t* ctx_len,
                                          const int32_t* q_len, const int32_t* reserve,
                                          int32_t Hkv, const sp_head_policy* pol,
                                          int32_t page_size, int32_t* seg_table,
                                          int32_t* kv_len) {
  if (seg_table == nullptr || kv_len == nullptr || reserve == nullptr) return SP_ERR_INVALID_ARG;
  Layout lay;
  sp_status st = layout_impl(1, B, ctx_len, q_len, reserve, Hkv, pol, page_size, &lay);
  if (st != SP_OK) return st;
  layout_tables(lay, B * Hkv, seg_table, kv_len);
  return SP_OK;
}

sp_status segpaged_build_growable(sp_dtype dtype, int32_t B, int32_t Hkv, int32_t D,
                                  int32_t page_size, const int32_t* ctx_len,
                                  const int32_t* q_len, const int32_t* reserve,
                                  const sp_head_policy* pol, const void* k_dense,
                                  const void* v_dense, const int32_t* free_pages, int64_t n_free,
                                  int64_t n_phys, void* k_pool, void* v_pool,
                                  int32_t* seg_table, int32_t* kv_len, int32_t* v2p,
                                  hipStream_t stream) {
  if (reserve == nullptr) return SP_ERR_INVALID_ARG;
  return build_impl(dtype, 1, B, Hkv, D, page_size, ctx_len, q_len, reserve, pol, k_dense,
                    v_dense, free_pages, n_free, n_phys, k_pool, v_pool, seg_table, kv_len, v2p,
                    stream);
}

sp_status segpaged_build(sp_dtype dtype, int32_t B, int32_t Hkv, int32_t D, int32_t page_size,
                         const int32_t* ctx_len, const int32_t* q_len, const sp_head_policy* pol,
                         const void* k_dense, const void* v_dense, const int32_t* free_pages,
                         int64_t n_free, int64_t n_phys, void* k_pool, void* v_pool,
                         int32_t* seg_table, int32_t* kv_len, int32_t* v2p, hipStream_t stream) {
  return segpaged_build_layers(dtype, 1, B, Hkv, D, page_size, ctx_len, q_len, pol, k_dense,
                               v_dense, free_pages, n_free, n_phys, k_pool, v_pool, seg_table,
                               kv_len, v2p, stream);
}

sp_status segpaged_build_layers(sp_dtype dtype, int32_t n_layers, int32_t B, int32_t Hkv,
                                int32_t D, int32_t page_size, const int32_t* ctx_len,
                                const int32_t* q_len, const sp_head_policy* pol,
                                const void* k_dense, const void* v_dense,
                                const int32_t* free_pages, int64_t n_free, int64_t n_phys,
                                void* k_pool, void* v_pool, int32_t* seg_table, int32_t* kv_len,
                                int32_t* v2p, hipStream_t stream) {
  return build_impl(dtype, n_layers, B, Hkv, D, page_size, ctx_len, q_len, nullptr, pol, k_dense,
                    v_dense, free_pages, n_free, n_phys, k_pool, v_pool, seg_table, kv_len, v2p,
                    stream);
}

sp_status segpaged_attention_workspace_size(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                            int32_t D, int32_t page_size,
                                            const int32_t* ctx_len, const int32_t* q_len,
                                            const sp_head_policy* pol, size_t* bytes) {
  return workspace_size(
      make_shape(kModePaged, dtype, B, Hq, Hkv, D, page_size, ctx_len, q_len, pol), bytes);
}

sp_status segpaged_attention_plan(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t page_size, const int32_t* ctx_len,
                                  const int32_t* q_len, const sp_head_policy* pol,
                                  void* workspace, size_t ws_bytes, hipStream_t stream) {
  return plan_into(make_shape(kModePaged, dtype, B, Hq, Hkv, D, page_size, ctx_len, q_len, pol),
                   workspace, ws_bytes, stream);
}

sp_status segpaged_attention(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t page_size, const int32_t* ctx_len, const int32_t* q_len,
                             const sp_head_policy* pol, const void* q, const void* k_pool,
                             const void* v_pool, int64_t n_phys, const int32_t* seg_table,
                             const int32_t* kv_len, const int32_t* v2p, float softmax_scale,
                             void* o, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return run_attention(
      make_shape(kModePaged, dtype, B, Hq, Hkv, D, page_size, ctx_len, q_len, pol), q, k_pool,
      v_pool, n_phys, seg_table, kv_len, v2p, softmax_scale, o, workspace, ws_bytes, stream,
      nullptr, nullptr);
}

sp_status segpaged_attention_static(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t page_size, const int32_t* ctx_len,
                                    const int32_t* q_len, const sp_head_policy* pol,
                                    const void* q, const void* k_pool, const void* v_pool,
                                    int64_t n_phys, const int32_t* seg_table,
                                    const int32_t* kv_len, const int32_t* v2p,
                                    float softmax_scale, void* o, int32_t* error,
                                    hipStream_t stream) {
  const Shape s = make_shape(kModePaged, dtype, B, Hq, Hkv, D, page_size, ctx_len, q_len, pol);
  sp_status st = check_shape(s);
  if (st != SP_OK) return st;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return SP_ERR_INVALID_ARG;
  bool need_pre = false, need_dec = false;
  needed_kernels(s, &need_pre, &need_dec);
  if (!need_pre && !need_dec) return SP_OK;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || o == nullptr ||
      seg_table == nullptr || kv_len == nullptr || v2p == nullptr || n_phys < 1)
    return SP_ERR_INVALID_ARG;
  if (need_pre && s.P < kChunk &&
      n_phys * int64_t(s.P) * s.D * (s.dtype == SP_BF16 ? 2 : 4) > int64_t(0x7fffffff))
    return SP_ERR_UNSUPPORTED;
  int32_t gp = 0, gd = 0;
  st = grids(s, &gp, &gd);
  if (st != SP_OK) return st;
  Plan plan;
  st = make_plan(s, gp, gd, &plan);
  if (st != SP_OK) return st;
  if (plan.bytes > kStaticWorkspaceBytes) return SP_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (static_workspace(&ws) != hipSuccess) return SP_ERR_HIP;
  // The upload rewrites the header: the error word and the queue counters start at zero.
  std::vector<uint8_t> buf;
  serialize_plan(plan, &buf);
  if (hipMemcpyAsync(ws, buf.data(), buf.size(), hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return SP_ERR_HIP;
  remember_plan(plan);
  st = run_attention(s, q, k_pool, v_pool, n_phys, seg_table, kv_len, v2p, softmax_scale, o, ws,
                     kStaticWorkspaceBytes, stream, nullptr, nullptr);
  if (st != SP_OK) return st;
  if (error != nullptr &&
      hipMemcpyAsync(error, static_cast<uint8_t*>(ws) + kOffError, sizeof(int32_t),
                     hipMemcpyDeviceToDevice, stream) != hipSuccess)
    return SP_ERR_HIP;
  return SP_OK;
}

sp_status segpaged_attention_profiled(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t page_size, const int32_t* ctx_len,
                                      const int32_t* q_len, const sp_head_policy* pol,
                                      const void* q, const void* k_pool, const void* v_pool,
                                      int64_t n_phys, const int32_t* seg_table,
                                      const int32_t* kv_len, const int32_t* v2p,
                                      float softmax_scale, void* o, void* workspace,
                                      size_t ws_bytes, hipStream_t stream,
                                      hipEvent_t main_begin, hipEvent_t main_end) {
  return run_attention(
      make_shape(kModePaged, dtype, B, Hq, Hkv, D, page_size, ctx_len, q_len, pol), q, k_pool,
      v_pool, n_phys, seg_table, kv_len, v2p, softmax_scale, o, workspace, ws_bytes, stream,
      main_begin, main_end);
}

sp_status segpaged_attention_plan_host(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t D, int32_t page_size, int32_t dense_mask,
                                       const int32_t* ctx_len, const int32_t* q_len,
                                       const sp_head_policy* pol, int32_t slots_prefill,
                                       int32_t slots_decode, void* host_buf, size_t buf_bytes,
                                       size_t* plan_bytes, size_t* workspace_bytes) {
  const Shape s = make_shape(dense_mask ? kModeDense : kModePaged, dtype, B, Hq, Hkv, D,
                             page_size, ctx_len, q_len, pol);
  sp_status st = check_shape(s);
  if (st != SP_OK) return st;
  if (slots_prefill < 1 || slots_decode < 1 || plan_bytes == nullptr) return SP_ERR_INVALID_ARG;
  Plan plan;
  st = make_plan(s, slots_prefill, slots_decode, &plan);
  if (st != SP_OK) return st;
  *plan_bytes = plan.upload_bytes;
  if (workspace_bytes) *workspace_bytes = plan.bytes;
  if (host_buf == nullptr) return SP_OK;
  if (buf_bytes < plan.upload_bytes) return SP_ERR_WORKSPACE_TOO_SMALL;
  std::vector<uint8_t> buf;
  serialize_plan(plan, &buf);
  std::memcpy(host_buf, buf.data(), buf.size());
  return SP_OK;
}

sp_status segpaged_attention_check(void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (workspace == nullptr || ws_bytes < size_t(kHeaderBytes)) return SP_ERR_INVALID_ARG;
  int32_t word = 0;
  uint8_t* w = static_cast<uint8_t*>(workspace) + kOffError;
  if (hipMemcpyAsync(&word, w, 4, hipMemcpyDeviceToHost, stream) != hipSuccess)
    return SP_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SP_ERR_HIP;
  if (word != 0) {
    const int32_t zero = 0;
    if (hipMemcpyAsync(w, &zero, 4, hipMemcpyHostToDevice, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return SP_ERR_HIP;
  }
  return sp_status(word);
}

sp_status segpaged_dense_mask_workspace_size(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                             int32_t D, const int32_t* ctx_len,
                                             const int32_t* q_len, const sp_head_policy* pol,
                                             size_t* bytes) {
  return workspace_size(make_shape(kModeDense, dtype, B, Hq, Hkv, D, 64, ctx_len, q_len, pol),
                        bytes);
}

sp_status segpaged_dense_mask_plan(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                   const int32_t* ctx_len, const int32_t* q_len,
                                   const sp_head_policy* pol, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  return plan_into(make_shape(kModeDense, dtype, B, Hq, Hkv, D, 64, ctx_len, q_len, pol),
                   workspace, ws_bytes, stream);
}

sp_status segpaged_dense_mask_attention(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                        int32_t D, const int32_t* ctx_len, const int32_t* q_len,
                                        const sp_head_policy* pol, const void* q,
                                        const void* k_dense, const void* v_dense,
                                        float softmax_scale, void* o, void* workspace,
                                        size_t ws_bytes, hipStream_t stream) {
  return run_attention(make_shape(kModeDense, dtype, B, Hq, Hkv, D, 64, ctx_len, q_len, pol), q,
                       k_dense, v_dense, 0, nullptr, nullptr, nullptr, softmax_scale, o,
                       workspace, ws_bytes, stream, nullptr, nullptr);
}

sp_status segpaged_decode_workspace_size(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                         int32_t D, int32_t page_size, const int32_t* ctx_hint,
                                         const sp_head_policy* pol, size_t* bytes) {
  if (bytes == nullptr) return SP_ERR_INVALID_ARG;
  std::vector<int32_t> hint, ones;
  Shape s;
  sp_status st = table_decode_shape(dtype, B, Hq, Hkv, D, page_size, ctx_hint, pol, &hint,
                                    &ones, &s);
  if (st != SP_OK) return st;
  Plan plan;
  st = table_decode_plan(s, &plan);
  if (st != SP_OK) return st;
  *bytes = plan.bytes;
  return SP_OK;
}

sp_status segpaged_decode_plan(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t page_size, const int32_t* ctx_hint,
                               const sp_head_policy* pol, void* workspace, size_t ws_bytes,
                               hipStream_t stream) {
  std::vector<int32_t> hint, ones;
  Shape s;
  sp_status st = table_decode_shape(dtype, B, Hq, Hkv, D, page_size, ctx_hint, pol, &hint,
                                    &ones, &s);
  if (st != SP_OK) return st;
  if (workspace == nullptr) return SP_ERR_INVALID_ARG;
  Plan plan;
  st = table_decode_plan(s, &plan);
  if (st != SP_OK) return st;
  if (ws_bytes < plan.bytes) return SP_ERR_WORKSPACE_TOO_SMALL;
  std::vector<uint8_t> buf;
  serialize_plan(plan, &buf);
  if (hipMemcpyAsync(workspace, buf.data(), buf.size(), hipMemcpyHostToDevice, stream) !=
      hipSuccess)
    return SP_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return SP_ERR_HIP;
  remember_plan(plan);
  return SP_OK;
}

sp_status segpaged_decode(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t page_size, const sp_head_policy* pol, const void* q,
                          const void* k_pool, const void* v_pool, int64_t n_phys,
                          const int32_t* seg_table, const int32_t* kv_len, const int32_t* v2p,
                          float softmax_scale, void* o, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  std::vector<int32_t> hint, ones;
  Shape s;
  sp_status st = table_decode_shape(dtype, B, Hq, Hkv, D, page_size, nullptr, pol, &hint,
                                    &ones, &s);
  if (st != SP_OK) return st;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return SP_ERR_INVALID_ARG;
  if (B == 0) return SP_OK;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || o == nullptr ||
      workspace == nullptr || seg_table == nullptr || kv_len == nullptr || v2p == nullptr ||
      n_phys < 1)
    return SP_ERR_INVALID_ARG;
  if (ws_bytes < size_t(kHeaderBytes)) return SP_ERR_WORKSPACE_TOO_SMALL;
  // Every request has one query, so either every item is a decode item (G <= kDecodeRows) or
  // every item is a tile of the prefill kernel; only that kernel is launched.
  const bool tiles = Hq / Hkv > kDecodeRows;
  // The prefill kernel with pages smaller than a KV step addresses rows from the pool start
  // with 32-bit byte offsets.
  if (tiles && page_size < kChunk &&
      n_phys * int64_t(page_size) * D * (dtype == SP_BF16 ? 2 : 4) > int64_t(0x7fffffff))
    return SP_ERR_UNSUPPORTED;
  int32_t gp = 0, gd = 0;
  st = grids(s, &gp, &gd);
  if (st != SP_OK) return st;
  AttnParams p;
  p.q = q;
  p.o = o;
  p.k = k_pool;
  p.v = v_pool;
  p.seg_table = seg_table;
  p.kv_len = kv_len;
  p.v2p = v2p;
  p.n_phys = n_phys;
  p.ws = static_cast<uint8_t*>(workspace);
  p.signature = table_decode_signature(s, gd);
  p.ws_bytes = ws_bytes;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.G = s.Hq / s.Hkv;
  p.P = s.P;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  if (launch_attention(s.dtype, s.D, kModePaged, !tiles,
                       tiles ? gp : decode_grid(p.signature, gd), p, stream) != hipSuccess)
    return SP_ERR_HIP;
  int cus = 0;
  st = device_cus(&cus);
  if (st != SP_OK) return st;
  if (launch_combine(s.dtype, s.D, 4 * cus, p, stream) != hipSuccess) return SP_ERR_HIP;
  return SP_OK;
}

sp_status segpaged_append(sp_dtype dtype, int32_t B, int32_t Hkv, int32_t D, int32_t page_size,
                          const sp_head_policy* pol, const int32_t* n_new, const void* k_new,
                          const void* v_new, void* k_pool, void* v_pool, int64_t n_phys,
                          int32_t* seg_table, int32_t* kv_len, int32_t* v2p, int64_t n_virt,
                          int32_t* error, hipStream_t stream) {
  sp_status st = check_dtype_dim(dtype, D);
  if (st != SP_OK) return st;
  st = check_page_size(page_size);
  if (st != SP_OK) return st;
  if (B < 0 || Hkv < 1 || pol == nullptr) return SP_ERR_INVALID_ARG;
  if (Hkv > kMaxAppendHeads) return SP_ERR_UNSUPPORTED;
  for (int32_t h = 0; h < Hkv; ++h) {
    if (pol[h].kind == SP_LOCAL_ADAPTIVE) return SP_ERR_UNSUPPORTED;
    if (pol[h].kind != SP_GLOBAL && pol[h].kind != SP_LOCAL && pol[h].kind != SP_RETRIEVAL)
      return SP_ERR_INVALID_ARG;
    if (pol[h].kind == SP_LOCAL && (pol[h].sink < 0 || pol[h].window < 1))
      return SP_ERR_INVALID_ARG;
  }
  if (int64_t(B) * Hkv > 0x7fffffffLL) return SP_ERR_UNSUPPORTED;
  if (B == 0) return SP_OK;
  if (k_new == nullptr || v_new == nullptr || k_pool == nullptr || v_pool == nullptr ||
      seg_table == nullptr || kv_len == nullptr || v2p == nullptr || error == nullptr ||
      n_phys < 1 || n_virt < 1 || n_virt > 0x7fffffffLL)
    return SP_ERR_INVALID_ARG;
  AppendParams p;
  std::memset(&p, 0, sizeof(p));
  p.k_new = k_new;
  p.v_new = v_new;
  p.n_new = n_new;
  p.kp = k_pool;
  p.vp = v_pool;
  p.seg_table = seg_table;
  p.kv_len = kv_len;
  p.v2p = v2p;
  p.error = error;
  p.n_phys = n_phys;
  p.n_virt = n_virt;
  p.Hkv = Hkv;
  p.P = page_size;
  for (int32_t h = 0; h < Hkv; ++h) {
    p.pol[h][0] = pol[h].kind;
    p.pol[h][1] = pol[h].kind == SP_LOCAL ? pol[h].sink : 0;
    p.pol[h][2] = pol[h].kind == SP_LOCAL ? pol[h].window : 1;
  }
  if (launch_append(dtype, D, B * Hkv, p, stream) != hipSuccess) return SP_ERR_HIP;
  return SP_OK;
}

}  // extern "C"
