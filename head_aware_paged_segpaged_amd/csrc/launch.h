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

struct BuildSeg {
  int32_t chunk0;    // first 64-token copy unit of this segment in the launch
  int32_t src_row0;  // dense row of the segment's first stored token (gather: of position 0)
  int32_t vstart;    // first virtual page of the segment
  int32_t ntok;
  int32_t h;
  int32_t pos_off;  // -1: tokens are consecutive; else token i is at position row_pos[pos_off + i]
};

constexpr int kMaxBuildSegs = 128;

struct BuildParams {
  const void* k;
  const void* v;
  void* kp;
  void* vp;
  const int32_t* v2p;
  const int32_t* row_pos;  // kept positions of RETRIEVAL segments (gather segments only)
  int32_t Hkv, P, nseg, nchunks;
  BuildSeg seg[kMaxBuildSegs];
};

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
hipError_t launch_build(int32_t dtype, int32_t D, const BuildParams& p, hipStream_t stream);
hipError_t launch_append(int32_t dtype, int32_t D, int grid, const AppendParams& p,
                         hipStream_t stream);

}  // namespace sp
