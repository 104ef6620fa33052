// Host-side planning for libsegpaged: argument validation, the per-head page layout and the
// attention work list. Pure integer C++; no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "segpaged.h"
#include "sp_common.h"

namespace sp {

struct Segment {
  int32_t pos, ntok, vstart, npages;
};

struct HeadLayout {
  Segment seg[2];
  int32_t nseg;
  int32_t kv_len;
};

// Page layout of one batch over n_layers layers: heads[(layer * B + b) * Hkv + h] (layer-major,
// so each layer's tables are contiguous); virtual pages are numbered in (request, layer, head,
// segment) order.
struct Layout {
  std::vector<HeadLayout> heads;
  int64_t n_virt = 0;
};

// Shape arguments common to the attention calls.
struct Shape {
  int32_t mode;  // kModePaged or kModeDense
  int32_t dtype;
  int32_t B, Hq, Hkv, D, P;
  const int32_t* ctx_len;
  const int32_t* q_len;
  const sp_head_policy* pol;
};

sp_status check_dtype_dim(int32_t dtype, int32_t D);
sp_status check_page_size(int32_t P);
sp_status check_lengths_policy(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                               int32_t Hkv, const sp_head_policy* pol);
sp_status check_shape(const Shape& s);

// Policy of one head for a request of context length L: an SP_LOCAL_ADAPTIVE head becomes a
// LOCAL head with window max(1, L / divisor); other heads are returned unchanged.
sp_head_policy effective_policy(const sp_head_policy& pol, int32_t L);
// Tokens a RETRIEVAL head keeps of its prefix: its sink, and the top fraction of the rest.
void retrieval_counts(const sp_head_policy& pol, int32_t L, int32_t q, int32_t* n_sink,
                      int32_t* n_kept);
// Segments of one (request, KV head) following the layout rules of include/segpaged.h.
int head_segments(const sp_head_policy& pol, int32_t L, int32_t q, int32_t out_pos[2],
                  int32_t out_ntok[2]);

sp_status make_layout(int32_t B, const int32_t* ctx_len, const int32_t* q_len, int32_t Hkv,
                      const sp_head_policy* pol, int32_t P, Layout* out);
// The same for n_layers layers sharing one page pool; pol is [n_layers][Hkv]. With `reserve`
// (host [B], or null) the layout is growable: each segment owns the pages it needs while its
// request's context grows by reserve[b] decode tokens (Segment::npages = pages owned).
sp_status make_layout_layers(int32_t n_layers, int32_t B, const int32_t* ctx_len,
                             const int32_t* q_len, int32_t Hkv, const sp_head_policy* pol,
                             int32_t P, const int32_t* reserve, Layout* out);

// Arguments of a growable layout: reserve[b] >= 0, a non-empty context (and, with retrieval
// heads, a non-empty query chunk) where reserve[b] > 0, no context-adaptive heads (their
// window moves with the context).
sp_status check_growable(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                         const int32_t* reserve, int32_t Hkv, const sp_head_policy* pol);
// Pages owned by each of the nseg segments of one head whose context L may grow to lmax.
void owned_pages(const sp_head_policy& pol, int nseg, const int32_t pos[2],
                 const int32_t ntok[2], int64_t L, int64_t lmax, int32_t P, int64_t own[2]);

// Fills seg_table [B][Hkv][2][4] and kv_len [B][Hkv] from a layout.
// seg_table [n_layers][B][Hkv][2][4] and kv_len [n_layers][B][Hkv] of a layout.
void layout_tables(const Layout& lay, int32_t n_heads_total, int32_t* seg_table,
                   int32_t* kv_len);

uint64_t shape_signature(const Shape& s, int32_t slots_prefill, int32_t slots_decode);
// Signature of a table-driven decode plan: shapes and policies, no lengths.
uint64_t table_decode_signature(const Shape& s, int32_t slots_decode);

struct Plan {
  WsHeader hdr;
  std::vector<WorkItem> prefill, decode;
  std::vector<CombineItem> combine;
  std::vector<int32_t> policy;  // [Hkv][3]
  size_t bytes = 0;             // whole workspace
  size_t upload_bytes = 0;      // header + item arrays + policy (what the plan call copies)
};

// table_decode: every request has one query (q_len all 1); the decode items are written in
// their table-driven form (ra_seg = -1, split c_begin of c_end) and the plan carries
// table_decode_signature. Lengths only balance the splits.
sp_status make_plan(const Shape& s, int32_t slots_prefill, int32_t slots_decode, Plan* out,
                    bool table_decode = false);

// Header, counters (zero), item arrays and policy table as one host buffer of
// plan.upload_bytes bytes, laid out exactly as in the workspace.
void serialize_plan(const Plan& plan, std::vector<uint8_t>* buf);

// Which kernels a call needs (cheap, from the host arrays only).
void needed_kernels(const Shape& s, bool* prefill, bool* decode);

}  // namespace sp
