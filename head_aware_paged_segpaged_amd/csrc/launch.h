// Kernel parameter blocks and launchers of libsegpaged (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sp_common.h"

namespace sp {

struct AttnParams {
  const void* q;
  void* o;
  const void* k;  // K pool [n_phys][P][D] (paged) or dense K [T][Hkv][D]
  const void* v;
  const int32_t* seg_table;  // paged only
  const int32_t* kv_len;     // paged only
  const int32_t* v2p;        // paged only
  int64_t n_phys;
  uint8_t* ws;
  uint64_t signature;
  uint64_t ws_bytes;
  int32_t Hq, Hkv, G, P;
  float scale_log2;  // softmax_scale * log2(e)
};

// Build: the kernel arguments carry, for each (layer, request) group of one launch, its first
// chunk (64 stored tokens of one segment) among the launch's chunks, the dense row of the
// group's first token and, for RETRIEVAL layouts, the kept-list offset of each head's kept
// segment (-1: none). Heads and segments come from the uploaded seg_table.
constexpr int kBuildArgInts = 944;

struct BuildParams {
  const void* k;  // dense [n_layers][T][Hkv][D]
  const void* v;
  void* kp;  // pools [n_phys][P][D]
  void* vp;
  const int32_t* v2p;
  const int32_t* row_pos;    // kept positions of RETRIEVAL segments (gather layouts only)
  const int32_t* seg_table;  // device [n_layers][B][Hkv][2][4], uploaded before the launch
  int32_t Hkv, P, n_groups, group0;
  // 0: every segment; 1: every segment but the kept prefixes of RETRIEVAL heads (their
  // positions are still being chosen); 2: only those kept prefixes (a gather through row_pos)
  int32_t phase, pad;
  // chunk offsets [n_groups + 1], first dense rows [n_groups], gather offsets [n_groups][Hkv]
  // (phases 1 and 2: -1 for heads without a kept prefix)
  int32_t arr[kBuildArgInts];
};
static_assert(sizeof(BuildParams) <= 4000, "build arguments fit the kernel argument segment");

// RETRIEVAL selection: one task per (request, retrieval head) with a non-empty kept list.
struct SelectTask {
  int32_t out;   // first entry of the task's kept list in row_pos
  int32_t row0;  // dense row of the request's position 0
  int32_t h, sink, k, n;  // KV head, sink tokens, kept candidates, candidates (sink .. prefix-1)
};
constexpr int kMaxSelectTasks = 160;

struct SelectParams {
  const float* imp;  // device [Hkv][T], T = rows of the dense K/V
  int32_t* row_pos;
  int32_t t_total, n_tasks;
  SelectTask t[kMaxSelectTasks];
};
static_assert(sizeof(SelectParams) <= 4000, "selection arguments fit the kernel argument segment");

constexpr int kMaxAppendHeads = 128;

struct AppendParams {
  const void* k_new;    // [B][Hkv][D]: the new token of every request
  const void* v_new;
  const int32_t* n_new;  // [B] 0 or 1, or null (every request appends)
  void* kp;
  void* vp;
  int32_t* seg_table;
  int32_t* kv_len;
  int32_t* v2p;
  int32_t* error;  // device word: first error code of the launch
  int64_t n_phys, n_virt;
  int32_t Hkv, P;
  int32_t pol[kMaxAppendHeads][3];  // (kind, sink, window) per KV head
};

// Bytes of the library-owned device workspace of segpaged_attention_static (one per GPU).
constexpr size_t kStaticWorkspaceBytes = size_t(64) << 20;
// Device address of that workspace on the current device (looked up once per device).
hipError_t static_workspace(void** ptr);

// Resident work groups per compute unit of the persistent attention kernels.
int attention_occupancy(int32_t dtype, int32_t D, int32_t mode, bool decode);
hipError_t launch_attention(int32_t dtype, int32_t D, int32_t mode, bool decode, int grid,
                            const AttnParams& p, hipStream_t stream);
hipError_t launch_combine(int32_t dtype, int32_t D, int grid, const AttnParams& p,
                          hipStream_t stream);
hipError_t launch_build(int32_t dtype, int32_t D, const BuildParams& p, int n_chunks,
                        hipStream_t stream);
hipError_t launch_select(const SelectParams& p, hipStream_t stream);
hipError_t launch_append(int32_t dtype, int32_t D, int grid, const AppendParams& p,
                         hipStream_t stream);

}  // namespace sp
