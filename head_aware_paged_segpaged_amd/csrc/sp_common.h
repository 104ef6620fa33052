// Internal layout shared by the host planner and the HIP kernels of libsegpaged.
// Not part of the public ABI (include/segpaged.h is).
#pragma once

#include <stdint.h>

namespace sp {

// KV tokens per inner step of every kernel. A step never crosses a segment, and inside a
// segment it covers stored indices [64k, 64k + 64), so with page sizes >= 64 it lies in one
// page and with smaller pages it covers 64 / page_size whole pages.
constexpr int kChunk = 64;
// Rows (query head x query token pairs of one KV head) of one prefill tile: 4 waves x 32.
constexpr int kTileRows = 128;
// Rows of one decode item; requests with q_len * G <= kDecodeRows take the decode kernel.
constexpr int kDecodeRows = 16;
// AMD Instinct MI355X has 8 accelerator complex dies (XCDs), each with its own L2. Work
// groups are dispatched to them round-robin, so queue x is popped first by work groups with
// blockIdx.x % 8 == x.
constexpr int kXcds = 8;
// Fixed cost of one work item in units of KV steps (Q load, epilogue, queue pop).
constexpr int kItemOverhead = 2;

constexpr uint64_t kMagic = 0x5350414745445631ull;  // "SPAGEDV1"
constexpr int kHeaderBytes = 4096;

enum Mode : int32_t { kModePaged = 0, kModeDense = 1, kModeTableDecode = 2 };

// One contiguous range of stored tokens of one segment: indices [begin, end) counted from the
// segment's first stored token (for the dense path: dense rows of the request).
struct Range {
  int32_t seg;
  int32_t begin;
  int32_t end;
};

// One unit of attention work: a block of query rows of one (request, KV head) against the
// KV steps [c_begin, c_end) of its step list. The step list is the 64-aligned steps of range
// `ra` followed by those of range `rb`.
struct WorkItem {
  int32_t b, h;          // request, KV head
  int32_t tq0, nq;       // first query token (within the request's chunk) and token count
  int32_t ra_seg, ra_begin, ra_end;
  int32_t rb_seg, rb_begin, rb_end;
  int32_t c_begin, c_end;  // KV steps of this item
  int32_t part;          // partial-result slot, or -1 to write O directly
  int32_t q_row0;        // Q/O row of the request's first query token
  int32_t p0;            // absolute position of the request's first query token
  int32_t kv_row0;       // dense path: first dense K/V row of the request
};
static_assert(sizeof(WorkItem) == 64, "WorkItem is 64 bytes");

// Merges the partial results of one KV-split block of rows, in split order.
struct CombineItem {
  int32_t b, h, tq0, nq;
  int32_t part0, nsplit;  // partial slots part0 .. part0 + nsplit - 1
  int32_t q_row0, kind;   // kind 0: prefill partial pool, 1: decode partial pool
};
static_assert(sizeof(CombineItem) == 32, "CombineItem is 32 bytes");

struct WsHeader {
  uint64_t magic;
  uint64_t signature;
  uint64_t bytes;          // workspace bytes the plan uses
  int32_t n_prefill, n_decode, n_combine, pad0;
  int32_t prefill_q[kXcds + 1];  // queue x = items [prefill_q[x], prefill_q[x+1])
  int32_t decode_q[kXcds + 1];
  int64_t off_prefill, off_decode, off_combine;  // byte offsets of the item arrays
  int64_t off_part_pre, off_ml_pre;              // prefill partials: o [n][128][D], ml [n][128][2]
  int64_t off_part_dec, off_ml_dec;              // decode partials:  o [n][16][D],  ml [n][16][2]
  int64_t off_policy;                            // int32 [Hkv][3] = (kind, sink, window)
  int32_t n_part_pre, n_part_dec;
};
static_assert(sizeof(WsHeader) <= 1024, "header fits its first kilobyte");

// Device-side words, each in its own 128-byte line after the header's first kilobyte.
constexpr int kOffError = 1024;
constexpr int kOffPrefillCnt = 1024 + 128;                   // kXcds counters
constexpr int kOffPrefillDone = kOffPrefillCnt + kXcds * 128;
constexpr int kOffDecodeCnt = kOffPrefillDone + 128;
constexpr int kOffDecodeDone = kOffDecodeCnt + kXcds * 128;
static_assert(kOffDecodeDone + 128 <= kHeaderBytes, "counters fit the header");

}  // namespace sp
