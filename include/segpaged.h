/*
 * segpaged.h -- C ABI of libsegpaged.so: head-aware SegPaged attention on AMD CDNA4 (gfx950).
 *
 * Method (page "RedKnot SegPagedAttention runtime design", sections 1-4): every KV head owns
 * its own page table over one shared physical page pool. A GLOBAL head stores and reads the
 * whole context. A LOCAL head stores and reads only its first S "sink" tokens plus a recent
 * window of W tokens. A RETRIEVAL head stores its sink, the most important part of its prefix
 * and its query chunk. Attention then packs every (query head, KV head) pair into one
 * variable-length launch in which each head walks only its own stored pages, so LOCAL heads
 * neither hold nor move KV they cannot see.
 *
 * Calls, in the order a caller makes them:
 *   segpaged_plan_pages           host only: how many pages a layout needs
 *   segpaged_layout_tables        host only: the tables segpaged_build will write
 *   segpaged_build                once per layout: page tables + fill the pool from dense K/V
 *                                 (segpaged_build_scored when RETRIEVAL heads need importance;
 *                                 segpaged_build_layers for several layers in one pool)
 *   segpaged_attention_workspace_size / segpaged_attention_plan
 *                                 once per layout: the work list the attention kernels pop
 *   segpaged_attention            every call: O = attention(Q, paged K/V)
 * Decode over a layout that grows by one token per step:
 *   segpaged_build_growable       once: the layout with pages reserved for decode tokens
 *                                 (segpaged_build_scored with a reserve for RETRIEVAL heads)
 *   segpaged_decode_workspace_size / segpaged_decode_plan
 *                                 once (re-plan at will): a work list that reads lengths from
 *                                 the device tables when it runs
 *   segpaged_append               every step: store each request's new token
 *   segpaged_decode               every step: O = attention(Q, paged K/V), one query each
 * The dense-plus-mask comparison path (segpaged_dense_mask_*) reads dense K/V directly.
 *
 * Conventions shared by every call
 * --------------------------------
 * - B requests; request b has ctx_len[b] context tokens and a query chunk of q_len[b] tokens,
 *   the LAST q_len[b] positions of its context: query token t sits at absolute position
 *   p = ctx_len[b] - q_len[b] + t. 0 <= q_len[b] <= ctx_len[b].
 * - Hq query heads over Hkv KV heads, G = Hq / Hkv an integer; query head hq reads KV head
 *   hq / G (contiguous groups).
 * - Visibility of key position j to a query at position p:
 *     GLOBAL: j <= p;   LOCAL: j <= p and (j < sink or j > p - window).
 *   A LOCAL_ADAPTIVE head is a LOCAL head whose window, for request b, is
 *   max(1, ctx_len[b] / window) (integer division; its `window` field is the divisor).
 * - Dense K/V are token-major with requests concatenated: [sum(ctx_len), Hkv, D], request b's
 *   rows start at sum_{b'<b} ctx_len[b']. Q and O are [sum(q_len), Hq, D]. Rows are dense
 *   (row stride Hkv*D or Hq*D elements).
 * - Element type: SP_BF16 (bfloat16 storage, fp32 accumulation and softmax, probabilities
 *   rounded to bf16 before P*V, O rounded to nearest even) or SP_F32 (fp32 throughout).
 * - Supported: D in {64, 128}; page_size in {16, 32, 64, 128, 256}; 1 <= G <= 128;
 *   sink >= 0; window >= 1.
 * - Pointers named "host" are read before the call returns. Pointers named "device" are
 *   device memory owned by the caller; the library allocates no device memory and keeps no
 *   state between calls. Device work is queued on `stream` and is asynchronous unless a call
 *   says otherwise.
 * - Errors: every argument is validated on the host before anything is queued; a call that
 *   returns an error has written nothing. The library never aborts and never throws.
 *
 * Page layout written by segpaged_build (page "RedKnot SegPagedAttention runtime design",
 * section 3: (layer, head, segment) -> contiguous virtual pages; a virtual -> physical map
 * over a shared pool; LOCAL heads keep only sink + recent tokens):
 * - A LOCAL head's recent part starts at R0 = max(0, L - q - W + 1), the earliest position
 *   any query of the chunk can see. Its segments, in position order, are
 *     (0, L) when R0 <= min(S, L);  (R0, L - R0) when S == 0;  else (0, S) and (R0, L - R0).
 *   A GLOBAL head has the single segment (0, L). L == 0 stores nothing.
 * - A RETRIEVAL head (sink S, window = p in thousandths) keeps, of its prefix [0, L - q): the
 *   first min(S, L - q) tokens and, of the n others, the ceil(p * n / 1000) with the highest
 *   importance (an input: one float per (token, KV head); ties go to the lower position); and
 *   the whole query chunk [L - q, L). Segments: the kept prefix tokens compacted in position
 *   order (slot i holds the i-th kept position; its pos_start reads 0; the positions are
 *   written to row_pos by segpaged_build_scored), then the chunk (L - q, q); with an empty
 *   prefix the chunk alone. The tables depend only on (L, q, S, p); which tokens fill the first
 *   segment depends on the importance. Every stored token is visible to every query of the
 *   chunk up to the causal edge, so attention reads exactly its stored tokens. Not supported
 *   by the dense-plus-mask path or several layers per build.
 * - seg_table int32 [B][Hkv][2][4] = {pos_start, n_tok, vpage_start, n_pages} per segment
 *   slot; an unused slot is {0, 0, running page total, 0}.
 * - Each segment starts on a fresh page; slot i of the segment's k-th page holds position
 *   pos_start + k*page_size + i. n_pages = ceil(n_tok / page_size).
 * - Virtual pages are numbered in (request, head, segment) order from 0; v2p[v] is the
 *   physical page of virtual page v, taken from the caller's free list in order.
 * - kv_len int32 [B][Hkv] = number of stored tokens of the head (its true KV length).
 * - Pools: [n_phys][page_size][D] elements; tail slots of a segment's last page are left
 *   untouched and never read.
 */
#ifndef SEGPAGED_H
#define SEGPAGED_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sp_status {
  SP_OK = 0,
  SP_ERR_INVALID_ARG = -1,         /* null pointer, negative size, inconsistent lengths  */
  SP_ERR_UNSUPPORTED = -2,         /* D, page size, dtype or G outside the supported set */
  SP_ERR_POOL_TOO_SMALL = -3,      /* fewer free pages than the layout needs             */
  SP_ERR_WORKSPACE_TOO_SMALL = -4, /* ws_bytes below what the workspace query returned   */
  SP_ERR_HIP = -5,                 /* a HIP runtime call failed                          */
  SP_ERR_PLAN_MISMATCH = -6,       /* workspace holds no plan for these arguments        */
  SP_ERR_SEGMENT_FULL = -7         /* segpaged_append: a segment owns no page left       */
} sp_status;

typedef enum sp_dtype { SP_BF16 = 0, SP_F32 = 1 } sp_dtype;

typedef enum sp_head_kind {
  SP_GLOBAL = 0,
  SP_LOCAL = 1,
  SP_LOCAL_ADAPTIVE = 2,
  SP_RETRIEVAL = 3
} sp_head_kind;

/* One per KV head (page "RedKnot head classification": head types, defaults window 512 and
 * sink 4). `sink` and `window` are ignored for SP_GLOBAL heads. SP_LOCAL_ADAPTIVE follows the
 * same page's passage on windows that adapt to each request's context length (its example:
 * half the context): the head is LOCAL with window max(1, ctx_len[b] / window) for request b,
 * so `window` is a divisor >= 1. SP_RETRIEVAL follows the same page's retrieval heads (full KV
 * of which only the top-p important tokens are kept) and the closing summary of page "RedKnot
 * SegPagedAttention runtime design" (retrieval heads take pages on demand): `window` is the
 * kept fraction p in thousandths (1..1000); see the layout rules. Any other kind is
 * SP_ERR_INVALID_ARG. */
typedef struct sp_head_policy {
  int32_t kind;   /* sp_head_kind                         */
  int32_t sink;   /* S >= 0                               */
  int32_t window; /* W >= 1 (SP_LOCAL_ADAPTIVE: divisor >= 1) */
} sp_head_policy;

/* Human-readable name of a status code. Never NULL. */
const char* segpaged_status_string(int status);

/* Pages the layout needs (the n_virt of segpaged_build). Host only; touches no GPU.
 * ctx_len, q_len: host [B]; pol: host [Hkv]. Writes *n_pages_needed on success. */
sp_status segpaged_plan_pages(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                              int32_t Hkv, const sp_head_policy* pol, int32_t page_size,
                              int64_t* n_pages_needed);

/* Host copy of the tables segpaged_build writes (same rules, no GPU touched).
 *   seg_table: host int32 [B][Hkv][2][4]; kv_len: host int32 [B][Hkv]. */
sp_status segpaged_layout_tables(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                                 int32_t Hkv, const sp_head_policy* pol, int32_t page_size,
                                 int32_t* seg_table, int32_t* kv_len);

/* Build the per-head page tables and fill the pool (page "RedKnot SegPagedAttention runtime
 * design", section 3: building per-head storage from dense KV keeps only the tokens each
 * LOCAL head can see; section 5: the layout is built once at KV-write time and reused).
 *   k_dense, v_dense : device [sum(ctx_len)][Hkv][D]
 *   free_pages       : host [n_free], distinct ids in [0, n_phys); the first n_virt are used
 *   k_pool, v_pool   : device [n_phys][page_size][D]
 *   seg_table        : device int32 [B][Hkv][2][4]   (written)
 *   kv_len           : device int32 [B][Hkv]         (written)
 *   v2p              : device int32 [n_virt]         (written; n_virt = segpaged_plan_pages)
 * The tables go up in one host-to-device copy on `stream` when kv_len directly follows
 * seg_table and v2p directly follows kv_len in memory (else three); host arrays are read
 * before return. Then one scatter launch (a work group per 64 stored tokens of a segment,
 * finding its segment from the uploaded seg_table) copies every stored row; it runs
 * asynchronously on `stream`. Batches with more (layer, request) groups than one launch's
 * arguments hold (about 470, or 940 / (Hkv + 2) with RETRIEVAL heads) take one launch per
 * such run of groups. Errors: SP_ERR_POOL_TOO_SMALL if n_free < n_virt, SP_ERR_INVALID_ARG
 * for duplicate or out-of-range free-list entries. */
sp_status segpaged_build(sp_dtype dtype, int32_t B, int32_t Hkv, int32_t D, int32_t page_size,
                         const int32_t* ctx_len, const int32_t* q_len, const sp_head_policy* pol,
                         const void* k_dense, const void* v_dense,
                         const int32_t* free_pages, int64_t n_free, int64_t n_phys,
                         void* k_pool, void* v_pool,
                         int32_t* seg_table, int32_t* kv_len, int32_t* v2p, hipStream_t stream);

/* The layout of n_layers layers of one batch in ONE page pool and one v2p (page "RedKnot
 * SegPagedAttention runtime design", section 3: the page table is keyed by (layer, head,
 * segment)). Virtual pages are numbered in (request, layer, head, segment) order; each layer's
 * segments follow the single-layer rules with that layer's policies. n_layers = 1 gives exactly
 * segpaged_plan_pages / segpaged_layout_tables / segpaged_build.
 *   pol              : host [n_layers][Hkv]
 *   k_dense, v_dense : device [n_layers][sum(ctx_len)][Hkv][D] (layers stacked)
 *   seg_table        : int32 [n_layers][B][Hkv][2][4]   (device for build, host for tables)
 *   kv_len           : int32 [n_layers][B][Hkv]
 *   v2p              : device int32 [n_virt] (n_virt from segpaged_plan_pages_layers)
 * Layer l is then served by segpaged_attention with pol + l*Hkv, seg_table + l*B*Hkv*8,
 * kv_len + l*B*Hkv and the shared v2p and pools. Errors as the single-layer calls, plus
 * SP_ERR_INVALID_ARG for n_layers < 1 and SP_ERR_UNSUPPORTED when n_layers * sum(ctx_len)
 * exceeds 2^31 - 1 rows. */
sp_status segpaged_plan_pages_layers(int32_t n_layers, int32_t B, const int32_t* ctx_len,
                                     const int32_t* q_len, int32_t Hkv,
                                     const sp_head_policy* pol, int32_t page_size,
                                     int64_t* n_pages_needed);
sp_status segpaged_layout_tables_layers(int32_t n_layers, int32_t B, const int32_t* ctx_len,
                                        const int32_t* q_len, int32_t Hkv,
                                        const sp_head_policy* pol, int32_t page_size,
                                        int32_t* seg_table, int32_t* kv_len);
sp_status segpaged_build_layers(sp_dtype dtype, int32_t n_layers, int32_t B, int32_t Hkv,
                                int32_t D, int32_t page_size, const int32_t* ctx_len,
                                const int32_t* q_len, const sp_head_policy* pol,
                                const void* k_dense, const void* v_dense,
                                const int32_t* free_pages, int64_t n_free, int64_t n_phys,
                                void* k_pool, void* v_pool, int32_t* seg_table, int32_t* kv_len,
                                int32_t* v2p, hipStream_t stream);

/* ---------------------------------------------------------------------------------------
 * Decode-time growth (page "RedKnot SegPagedAttention runtime design", section 3: LOCAL heads
 * hold only sink and recent pages, so their storage does not grow with the context; section
 * 5: layout work is done when KV is written; the product overview page "RedKnot：小红书开源的
 * 长上下文LLM推理优化工具…", section 3.2, items (1) and (3): LOCAL heads cache a bounded
 * length of KV and idle pages are reclaimed).
 *
 * Growable layout: the segments and page order of segpaged_build for (ctx_len, q_len), but each
 * segment OWNS enough contiguous virtual pages for reserve[b] more tokens of request b, all
 * mapped at build (v2p[v] = free_pages[v]); field 3 of a segment row (n_pages above) is the
 * number of pages it owns. reserve[b] == 0 for all b gives exactly segpaged_build's layout.
 * Let L be the context, Lmax = L + reserve[b], W the window, S the sink, P the page size:
 *   GLOBAL            owns ceil(Lmax / P).
 *   ring              (the recent segment of a LOCAL head: its only segment when S == 0, its
 *                     second when the head has two) with build pos_start o owns
 *                     max(ceil((L - o) / P), ceil(min(Lmax - o, W + P - 1) / P)).
 *   (0, L), S > 0     (sink and window in one segment) owns the largest of ceil(L / P),
 *                     ceil(min(Lmax, Sp + W - 1) / P) and, if Lmax >= Sp + W,
 *                     ceil(S / P) + ceil(min(Lmax - Sp, W + P - 1) / P), Sp = ceil(S/P) * P.
 *   sink segment      owns its pages.
 * Append (one token per request, at position L = the old context length; the context becomes
 * L + 1 and the next decode query sits at position L):
 *   GLOBAL            the token goes to the end of its segment.
 *   (0, L), S > 0     the token goes to the end of the segment; once the window start
 *                     L + 1 - W reaches Sp the segment first splits into the sink (0, S) on its
 *                     first ceil(S / P) pages and a ring starting at Sp on the other pages.
 *   ring              first its k = floor((L + 1 - W - pos_start) / P) oldest pages (if k > 0)
 *                     are dropped: pos_start += k*P, n_tok -= k*P, and the segment's v2p
 *                     entries rotate left by k (the dropped physical pages move to its end,
 *                     where later tokens reuse them); then the token goes to its end.
 *   RETRIEVAL         the token goes to the end of its last segment, the query chunk, which
 *                     owns ceil((q + reserve[b]) / P) pages; its kept prefix never changes (a
 *                     growing request needs q_len[b] >= 1; layouts with retrieval heads are
 *                     built by segpaged_build_scored with a reserve).
 * A ring thus keeps at most W + P - 1 tokens; fewer than P of them (all older than the window)
 * are stale, and attention masks them by position. Context-adaptive heads are not growable
 * (SP_ERR_UNSUPPORTED).
 * --------------------------------------------------------------------------------------- */

/* Number of kept-prefix rows of all SP_RETRIEVAL heads (the size of row_pos), in
 * (request, head) order. Host only. */
sp_status segpaged_retrieval_rows(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                                  int32_t Hkv, const sp_head_policy* pol, int64_t* n_rows);

/* segpaged_build for layouts with SP_RETRIEVAL heads (page "RedKnot head classification":
 * retrieval heads keep only the top-p important tokens; the selection happens once, at
 * KV-write time, like the rest of the layout). Same arguments and errors as segpaged_build,
 * plus:
 *   reserve    : host int32 [B] or NULL: with it the layout is the growable one of
 *                segpaged_build_growable (below), RETRIEVAL heads included
 *   importance : device float [Hkv][sum(ctx_len)], head-major (each head's scores of all
 *                tokens contiguous, requests concatenated as in k_dense); only the prefix
 *                tokens of RETRIEVAL heads are read, on the device, by one selection work
 *                group per (request, retrieval head). The selection runs on a stream of the
 *                library's own (one per device, default priority, created on first use), forked
 *                from `stream` after the table upload and joined back before the kept
 *                prefixes are copied, so it overlaps the copy of every other segment; the call
 *                stays ordered on `stream` like segpaged_build. Values must be finite (a NaN
 *                orders by its bits: a valid but unspecified selection).
 *   row_pos    : device int32 [segpaged_retrieval_rows] (written): the kept positions of each
 *                RETRIEVAL head, ascending, heads in (request, head) order; may be NULL when
 *                that count is 0.
 * segpaged_build (and the _layers build) returns SP_ERR_INVALID_ARG for layouts that keep
 * RETRIEVAL rows, since it has no importance. */
sp_status segpaged_build_scored(sp_dtype dtype, int32_t B, int32_t Hkv, int32_t D,
                                int32_t page_size, const int32_t* ctx_len, const int32_t* q_len,
                                const int32_t* reserve, const sp_head_policy* pol,
                                const float* importance, const void* k_dense,
                                const void* v_dense, const int32_t* free_pages, int64_t n_free,
                                int64_t n_phys, void* k_pool, void* v_pool, int32_t* seg_table,
                                int32_t* kv_len, int32_t* v2p, int32_t* row_pos,
                                hipStream_t stream);

/* Pages (n_virt) and host tables of the growable layout. reserve: host int32 [B] >= 0; a
 * request with reserve[b] > 0 needs ctx_len[b] >= 1. Errors as segpaged_plan_pages /
 * segpaged_layout_tables, plus SP_ERR_UNSUPPORTED for SP_LOCAL_ADAPTIVE heads or
 * ctx_len[b] + reserve[b] >= 2^31. */
sp_status segpaged_plan_pages_growable(int32_t B, const int32_t* ctx_len, const int32_t* q_len,
                                       const int32_t* reserve, int32_t Hkv,
                                       const sp_head_policy* pol, int32_t page_size,
                                       int64_t* n_pages_needed);
sp_status segpaged_layout_tables_growable(int32_t B, const int32_t* ctx_len,
                                          const int32_t* q_len, const int32_t* reserve,
                                          int32_t Hkv, const sp_head_policy* pol,
                                          int32_t page_size, int32_t* seg_table,
                                          int32_t* kv_len);

/* segpaged_build for the growable layout (same arguments, same errors, plus reserve). The
 * first build attention call can be segpaged_attention (its segments are segpaged_build's);
 * after the first segpaged_append only segpaged_decode reads the tables. */
sp_status segpaged_build_growable(sp_dtype dtype, int32_t B, int32_t Hkv, int32_t D,
                                  int32_t page_size, const int32_t* ctx_len,
                                  const int32_t* q_len, const int32_t* reserve,
                                  const sp_head_policy* pol, const void* k_dense,
                                  const void* v_dense, const int32_t* free_pages, int64_t n_free,
                                  int64_t n_phys, void* k_pool, void* v_pool,
                                  int32_t* seg_table, int32_t* kv_len, int32_t* v2p,
                                  hipStream_t stream);

/* Appends one token to every request with n_new[b] == 1 (n_new: device int32 [B] of 0 / 1, or
 * NULL for all), following the rules above; one work group per (request, KV head), all state on
 * the device, nothing read back, no host synchronisation.
 *   pol          : host [Hkv], SP_GLOBAL, SP_LOCAL or SP_RETRIEVAL (Hkv <= 128)
 *   k_new, v_new : device [B][Hkv][D], row (b, h) is request b's new token for KV head h
 *   k_pool, v_pool, n_phys, seg_table, kv_len, v2p : a growable layout (updated in place)
 *   n_virt       : number of v2p entries (segpaged_plan_pages_growable)
 *   error        : device int32; the first failing (request, head) writes its code there with
 *                  an atomic compare-and-swap from 0 (the caller clears it): SP_ERR_SEGMENT_FULL
 *                  when the token needs a page the segment does not own (appending past the
 *                  reserve), SP_ERR_INVALID_ARG for an empty head, n_new not 0 or 1, or a page
 *                  id outside the pool. A failing (request, head) is left unchanged; the others
 *                  of the launch are appended.
 * The context length of each request is not passed: it is one past the newest stored token. */
sp_status segpaged_append(sp_dtype dtype, int32_t B, int32_t Hkv, int32_t D, int32_t page_size,
                          const sp_head_policy* pol, const int32_t* n_new, const void* k_new,
                          const void* v_new, void* k_pool, void* v_pool, int64_t n_phys,
                          int32_t* seg_table, int32_t* kv_len, int32_t* v2p, int64_t n_virt,
                          int32_t* error, hipStream_t stream);

/* Table-driven decode (page "RedKnot SegPagedAttention runtime design", section 4: each head's
 * true KV length comes from its page table; section 5: no layout work per call). One query per
 * request, Q and O [B][Hq][D]; query b sits at request b's newest stored position. The work
 * list holds (request, KV head, split k of n) items; the kernel takes each head's segments and
 * lengths from the device seg_table / kv_len when it runs, so one plan serves every decode step
 * of a growing layout (and any layout segpaged_build writes). ctx_hint (host [B] >= 1, or NULL)
 * only sizes the KV splits; re-plan when the lengths have drifted far. The workspace, the
 * combine and reproducibility are as for segpaged_attention; errors likewise, plus
 * SP_ERR_UNSUPPORTED for SP_LOCAL_ADAPTIVE heads. Groups of G = Hq / Hkv <= 16 query heads run
 * as decode items (one wave per item); larger groups (G <= 128) as 128-row tiles of the prefill
 * kernel, one per (request, KV head, split), each reading the head's KV once for all G rows. */
sp_status segpaged_decode_workspace_size(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                         int32_t D, int32_t page_size, const int32_t* ctx_hint,
                                         const sp_head_policy* pol, size_t* bytes);
sp_status segpaged_decode_plan(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t page_size, const int32_t* ctx_hint,
                               const sp_head_policy* pol, void* workspace, size_t ws_bytes,
                               hipStream_t stream);
sp_status segpaged_decode(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                          int32_t page_size, const sp_head_policy* pol, const void* q,
                          const void* k_pool, const void* v_pool, int64_t n_phys,
                          const int32_t* seg_table, const int32_t* kv_len, const int32_t* v2p,
                          float softmax_scale, void* o, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/* Bytes of device workspace segpaged_attention needs for these arguments (host only). The
 * workspace holds the work list (one item per (request, KV head, query block, KV split),
 * per-XCD queues and counters) and the fp32 partial results of KV-split items. */
sp_status segpaged_attention_workspace_size(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                            int32_t D, int32_t page_size,
                                            const int32_t* ctx_len, const int32_t* q_len,
                                            const sp_head_policy* pol, size_t* bytes);

/* Plan the attention launch into `workspace` (device, >= the size above). The work list
 * balances long GLOBAL-head tiles against short LOCAL-head tiles: long tiles are split along
 * KV, items are grouped by KV head onto per-XCD queues and ordered longest first. Done once
 * per layout (page "RedKnot SegPagedAttention runtime design", section 5: recomputing layout
 * work on every attention call costs more than it saves). Synchronous: the plan is in place
 * when this returns. */
sp_status segpaged_attention_plan(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t page_size, const int32_t* ctx_len,
                                  const int32_t* q_len, const sp_head_policy* pol,
                                  void* workspace, size_t ws_bytes, hipStream_t stream);

/* O = SegPaged attention (page "RedKnot SegPagedAttention runtime design", section 4: each
 * head's true KV length comes from its page table; all (query head, KV head) pairs go into
 * one variable-length launch, each head with its own length).
 *   q        : device [sum(q_len)][Hq][D]
 *   k_pool, v_pool, n_phys, seg_table, kv_len, v2p : as written by segpaged_build
 *   o        : device [sum(q_len)][Hq][D] (written)
 *   workspace: device, planned by segpaged_attention_plan with the same shape arguments;
 *              reused across calls (its counters return to zero when the kernels finish).
 * Query requests with q_len * G <= 16 take the split-KV decode kernel; the others take the
 * prefill kernel; KV-split items are merged by a fixed-order combine kernel, so O is bitwise
 * reproducible. Calls that share one workspace must not overlap in time.
 * Errors: SP_ERR_PLAN_MISMATCH if the workspace was planned for other arguments (checked on
 * the device; the kernels then write nothing -- see segpaged_attention_check);
 * SP_ERR_UNSUPPORTED if page_size < 64, some request takes the prefill kernel and a pool is
 * larger than 2 GiB (that path addresses pool rows with 32-bit offsets). O is unspecified when
 * the device-side error word reports SP_ERR_INVALID_ARG (a page id >= n_phys in v2p). */
sp_status segpaged_attention(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t page_size, const int32_t* ctx_len, const int32_t* q_len,
                             const sp_head_policy* pol, const void* q, const void* k_pool,
                             const void* v_pool, int64_t n_phys, const int32_t* seg_table,
                             const int32_t* kv_len, const int32_t* v2p, float softmax_scale,
                             void* o, void* workspace, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code that must not call hipMalloc, tight
 * serving loops, harnesses that forbid allocation): segpaged_attention with no workspace
 * argument. It plans on the host and uploads the plan (synchronising `stream`) into a
 * library-owned device array of 64 MiB per GPU, held until the process ends, then runs the
 * same kernels on it. It allocates no device memory. Plans larger than 64 MiB (many KV-split
 * partial results) return SP_ERR_WORKSPACE_TOO_SMALL before anything is written. Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (any streams) race
 * and give undefined results. Planning on every call is host work that segpaged_attention
 * keeps out of the call (it plans once per layout).
 *   error : device int32 or NULL; after the kernels, the call's device-side status (SP_OK,
 *           SP_ERR_INVALID_ARG for a page id >= n_phys) is copied there on `stream`.
 * Other arguments, errors and O: as segpaged_attention, bit for bit. */
sp_status segpaged_attention_static(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t page_size, const int32_t* ctx_len,
                                    const int32_t* q_len, const sp_head_policy* pol,
                                    const void* q, const void* k_pool, const void* v_pool,
                                    int64_t n_phys, const int32_t* seg_table,
                                    const int32_t* kv_len, const int32_t* v2p,
                                    float softmax_scale, void* o, int32_t* error,
                                    hipStream_t stream);

/* Same as segpaged_attention, and records `main_begin` / `main_end` (may be NULL) on
 * `stream` right before and after the attention kernel(s), before any combine kernel, so a
 * caller can time the main kernel alone. */
sp_status segpaged_attention_profiled(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t page_size, const int32_t* ctx_len,
                                      const int32_t* q_len, const sp_head_policy* pol,
                                      const void* q, const void* k_pool, const void* v_pool,
                                      int64_t n_phys, const int32_t* seg_table,
                                      const int32_t* kv_len, const int32_t* v2p,
                                      float softmax_scale, void* o, void* workspace,
                                      size_t ws_bytes, hipStream_t stream,
                                      hipEvent_t main_begin, hipEvent_t main_end);

/* Host-only copy of the plan segpaged_attention_plan (dense_mask = 0) or
 * segpaged_dense_mask_plan (dense_mask = 1) would upload, for inspection and testing, with the
 * persistent grid sizes given explicitly instead of read from the current device. Writes
 * *plan_bytes (bytes of header + work lists) and, if non-NULL, *workspace_bytes; fills
 * host_buf (buf_bytes >= *plan_bytes) unless it is NULL. Layout of the buffer: a 4096-byte
 * header, then 64-byte work items and 32-byte combine items, as described in the
 * library's csrc/sp_common.h. */
sp_status segpaged_attention_plan_host(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                       int32_t D, int32_t page_size, int32_t dense_mask,
                                       const int32_t* ctx_len, const int32_t* q_len,
                                       const sp_head_policy* pol, int32_t slots_prefill,
                                       int32_t slots_decode, void* host_buf, size_t buf_bytes,
                                       size_t* plan_bytes, size_t* workspace_bytes);

/* Reads back (synchronising `stream`) the device-side error word of a workspace: SP_OK, or
 * SP_ERR_PLAN_MISMATCH / SP_ERR_INVALID_ARG if a kernel found a plan for other arguments or a
 * page id >= n_phys in v2p. Clears the word. */
sp_status segpaged_attention_check(void* workspace, size_t ws_bytes, hipStream_t stream);

/* Dense-plus-mask comparison path (page "RedKnot SegPagedAttention runtime design",
 * sections 4 and 6: the dense + mask baseline the SegPaged result is checked and timed
 * against). Same tile engine and scheduling, but every head walks its full causal range of
 * the dense [sum(ctx_len)][Hkv][D] K/V and applies its visibility as an elementwise mask.
 * Workspace query and plan as above. */
sp_status segpaged_dense_mask_workspace_size(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                             int32_t D, const int32_t* ctx_len,
                                             const int32_t* q_len, const sp_head_policy* pol,
                                             size_t* bytes);
sp_status segpaged_dense_mask_plan(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                   const int32_t* ctx_len, const int32_t* q_len,
                                   const sp_head_policy* pol, void* workspace, size_t ws_bytes,
                                   hipStream_t stream);
sp_status segpaged_dense_mask_attention(sp_dtype dtype, int32_t B, int32_t Hq, int32_t Hkv,
                                        int32_t D, const int32_t* ctx_len, const int32_t* q_len,
                                        const sp_head_policy* pol, const void* q,
                                        const void* k_dense, const void* v_dense,
                                        float softmax_scale, void* o, void* workspace,
                                        size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SEGPAGED_H */
