// HIP kernels of libsegpaged for CDNA4 (gfx950): build/scatter, varlen prefill attention,
// split-KV decode attention and the fixed-order cross-split combine.
//
// Method: page "RedKnot SegPagedAttention runtime design", sections 3-4. Each (request, KV
// head) walks only its own stored tokens through its page table; GLOBAL heads walk the whole
// prefix, LOCAL heads the sink and the recent window. All (query head, KV head) pairs of a
// batch run in one persistent launch that pops work items from per-XCD queues.
//
// Data layout in the kernels:
// - Prefill: one KV step = 64 stored tokens of one segment (64-aligned in the segment). K and V
//   of a step arrive by LDS-DMA into row-major LDS tiles whose 16-byte chunks are XOR-swizzled
//   by row (conflict-free fragment and transposed reads); two K and two V stages. A tile is
//   128 rows = (query token, query head of the GQA group) pairs of one KV head; wave w owns
//   rows 32w..32w+31. S^T = K * Q^T on 32x32 MFMA puts one query row per lane column, so the
//   softmax row statistics are per lane (plus one cross-half exchange) and the O^T
//   accumulators are rescaled in-lane; V^T comes from the LDS transpose reads.
// - Decode: one wave per item of up to 16 rows, in sub-steps of 16 keys: K straight into
//   registers, V into a wave-private LDS ring, three sub-steps ahead, no work-group barrier.
// Softmax runs in base 2 with scale*log2(e) folded into one FMA, against a per-row reference
// that moves only when a row maximum passes it by more than 2^kSlack; masks are evaluated only
// on steps that straddle a visibility edge or are not full.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "launch.h"
#include "segpaged.h"

namespace sp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
// Headroom of the prefill softmax reference, in log2 units (exponentials stay <= 2^kSlack).
constexpr float kSlack = 8.f;

struct BF16 {
  using S = uint16_t;
  static constexpr int kVec = 8;  // elements per 16-byte access
  static constexpr int KPL = 8;   // reduction elements per lane of one MFMA
  using Frag = bf16x8_t;
};

struct F32 {
  using S = float;
  static constexpr int kVec = 4;
  static constexpr int KPL = 1;
  using Frag = float;
};

__device__ __forceinline__ f32x16_t mma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mma32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma16(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <class E>
__device__ __forceinline__ typename E::Frag load_frag(const typename E::S* p) {
  if constexpr (E::KPL == 8) {
    return *reinterpret_cast<const bf16x8_t*>(p);
  } else {
    return *p;
  }
}

template <class E>
__device__ __forceinline__ typename E::Frag zero_frag() {
  if constexpr (E::KPL == 8) {
    u32x4_t z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8_t, z);
  } else {
    return 0.f;
  }
}

__device__ __forceinline__ bf16x8_t to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
  f32x8_t f = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(f, bf16x8_t);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Instruction interleave of one prefill step, for the machine scheduler: `pre` LDS reads, then
// nA S^T MFMAs each followed by one LDS read, vA VALU and tA transcendental instructions, then
// nC P*V MFMAs each followed by two LDS reads and vC VALU. On gfx950 a few independent VALU
// instructions placed between MFMAs run almost for free, while the same work gathered into a
// block between MFMA blocks adds its full length to the step.
template <int nA, int vA, int tA, int nC, int vC, int pre>
__device__ __forceinline__ void step_schedule() {
  __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);
#pragma unroll
  for (int m = 0; m < nA; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, vA, 0);
    __builtin_amdgcn_sched_group_barrier(0x400, tA, 0);
  }
#pragma unroll
  for (int m = 0; m < nC; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, vC, 0);
  }
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ void set_error(uint8_t* ws, int code) {
  atomicCAS(reinterpret_cast<int*>(ws + kOffError), 0, code);
}

// Work groups the round-robin dispatch places on XCD x (work group i runs on XCD i % kXcds).
__device__ __forceinline__ int wgs_on_xcd(int x) {
  return (int(gridDim.x) - x + kXcds - 1) / kXcds;
}

// The work queues as one work group sees them, read once when it starts: queue (xcd + k) %
// kXcds at index k, its own XCD's first. In a one-round launch every queue fits the work groups
// of its XCD, so each work group's first (static) pop is its only item and the queue counters
// are never touched.
struct Queues {
  int32_t lo[kXcds], n[kXcds];  // first item and item count of queue (xcd + k) % kXcds
  bool one_round;
};

__device__ __forceinline__ Queues load_queues(const int32_t* qb, int xcd) {
  Queues q;
  q.one_round = true;
#pragma unroll
  for (int k = 0; k < kXcds; ++k) {
    const int x = (xcd + k) & (kXcds - 1);
    q.lo[k] = qb[x];
    q.n[k] = qb[x + 1] - qb[x];
    q.one_round = q.one_round && q.n[k] <= wgs_on_xcd(x);
  }
  return q;
}

// Pops the next work item, one thread per work group. The first pop is static: the k-th work
// group of an XCD takes item k of that XCD's queue, so the launch starts without a burst of
// atomics on the queue counters. Later pops take the queue's counter (past the items handed
// out statically): own XCD's queue first, then the others. Bit k of `exhausted` marks queue
// (xcd + k) % kXcds as empty.
__device__ __forceinline__ int pop_item(uint8_t* ws, const Queues& q, int cnt_off, int xcd,
                                        uint32_t& exhausted, bool& first) {
  if (first) {
    first = false;
    const int k = int(blockIdx.x) / kXcds;
    if (k < q.n[0]) return q.lo[0] + k;
  }
#pragma unroll
  for (int k = 0; k < kXcds; ++k) {
    if (exhausted & (1u << k)) continue;
    const int x = (xcd + k) & (kXcds - 1);
    const int s = min(q.n[k], wgs_on_xcd(x));
    if (q.n[k] > s) {
      const int t = atomicAdd(reinterpret_cast<int*>(ws + cnt_off + x * 128), 1);
      if (s + t < q.n[k]) return q.lo[k] + s + t;
    }
    exhausted |= 1u << k;
  }
  return -1;
}

// The last work group to finish returns the queue counters to zero for the next launch (not
// called in one-round launches, which leave the counters at zero).
__device__ __forceinline__ void retire(uint8_t* ws, int cnt_off, int done_off) {
  const int d = atomicAdd(reinterpret_cast<int*>(ws + done_off), 1);
  if (d == int(gridDim.x) - 1) {
    for (int x = 0; x < kXcds; ++x) atomicExch(reinterpret_cast<int*>(ws + cnt_off + x * 128), 0);
    atomicExch(reinterpret_cast<int*>(ws + done_off), 0);
  }
}

// Per-item view of the KV source: segment table of (b, h) and the step list.
struct ItemKV {
  int pos0, ntok0, vstart0;
  int pos1, ntok1, vstart1;
  int n_ra;
};

// One KV step of an item: 64 token slots of one segment. `off` is the element offset of the
// step's first row in the pool (paged layout, pages of at least one step) or in the dense K/V.
struct Step {
  int seg, ti0, vlo, vhi, pos0;
  int64_t off;
};

// Segment, slot range and key positions of step c (no memory access).
__device__ __forceinline__ Step step_range(const WorkItem& w, const ItemKV& kv, int c,
                                           bool dense) {
  Step s;
  int base, lo, hi;
  if (c < kv.n_ra) {
    s.seg = w.ra_seg;
    base = w.ra_begin / kChunk + c;
    lo = w.ra_begin;
    hi = w.ra_end;
  } else {
    s.seg = w.rb_seg;
    base = w.rb_begin / kChunk + (c - kv.n_ra);
    lo = w.rb_begin;
    hi = w.rb_end;
  }
  s.ti0 = base * kChunk;
  s.vlo = max(0, lo - s.ti0);
  s.vhi = min(kChunk, hi - s.ti0);
  s.pos0 = dense ? s.ti0 : (s.seg == 0 ? kv.pos0 : kv.pos1) + s.ti0;
  s.off = 0;
  return s;
}

// ---------------------------------------------------------------------------------------
// LDS tile of one KV step: 64 rows x D elements, row-major, with the 16-byte chunks of a row
// XOR-swizzled by the row index, so that the same column of 16 consecutive rows lands in 16
// different bank groups. K and V of a step arrive by LDS-DMA (buffer_load ... lds): each lane
// of a wave writes 16 bytes at wave_base + 16 * lane, so a lane fetches the source chunk that
// belongs at its destination slot. No register staging, no ds_write.
// ---------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

template <class E, int D>
struct KVTile {
  using S = typename E::S;
  static constexpr int kRowBytes = D * int(sizeof(S));
  static constexpr int kChunks = kRowBytes / 16;           // 16-byte chunks per row
  static constexpr int kBytes = kChunk * kRowBytes;        // K (or V) of one step
  static constexpr int kLoads = kChunk * kChunks / 256;    // DMA pieces per thread per tensor
  static constexpr uint32_t kOut = 0x80000000u;            // offset past num_records: reads 0

  // Chunk permutation of row `row`. With 16 chunks per row the XOR key swaps the two 2-bit
  // halves of row % 16: any 16 consecutive rows get 16 different keys (row-major fragment reads
  // are conflict-free) and any 4 consecutive rows get keys in 4 different quarters of the row
  // (the transposed V reads, 4 rows x 64 bytes per half-wave, are conflict-free too).
  __device__ __forceinline__ static int swz(int row, int chunk) {
    if constexpr (kChunks == 16) {
      return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3));
    } else {
      return chunk ^ (row & (kChunks - 1));
    }
  }
  // Byte offset of byte `byte` of row `row` inside a tile.
  __device__ __forceinline__ static int off(int row, int byte) {
    return row * kRowBytes + (swz(row, byte >> 4) << 4) + (byte & 15);
  }
  // Row and source chunk of this thread's DMA piece j.
  __device__ __forceinline__ static int piece_row(int j) { return (j * 256 + int(threadIdx.x)) / kChunks; }
  __device__ __forceinline__ static int piece_chunk(int j) {
    const int n = j * 256 + int(threadIdx.x);
    return swz(n / kChunks, n % kChunks);
  }
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                             0x00020000);
  }
  // DMA of the 64 rows of K and V whose first rows start at kb / vb, `rs` bytes apart; rows
  // outside [vlo, vhi) are written as zero.
  template <bool kK, bool kV>
  __device__ __forceinline__ static void dma_strided(const void* kb, const void* vb, uint32_t rs,
                                                     int vlo, int vhi, bool full, char* lk,
                                                     char* lv) {
    const __amdgpu_buffer_rsrc_t rk = rsrc(kb), rv = rsrc(vb);
    const int wbase = uniform(int(threadIdx.x >> 6)) * 1024;
    auto issue = [&](int j, uint32_t o) {
      if constexpr (kK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(lk + j * 4096 + wbase), 16, o,
                                                 0, 0, 0);
      if constexpr (kV)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(lv + j * 4096 + wbase), 16, o,
                                                 0, 0, 0);
    };
    if (full) {  // uniform: the common case takes no per-row test
#pragma unroll
      for (int j = 0; j < kLoads; ++j)
        issue(j, uint32_t(piece_row(j)) * rs + uint32_t(piece_chunk(j)) * 16u);
    } else {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int row = piece_row(j);
        const bool in = row >= vlo && row < vhi;
        issue(j, in ? uint32_t(row) * rs + uint32_t(piece_chunk(j)) * 16u : kOut);
      }
    }
  }
  // Full step of a pool whose pages hold at least one step: its 64 rows are contiguous
  // (kBytes from `kb`). Wave w fills tile bytes [w * kWave, (w + 1) * kWave) with kLoads
  // transfers that share one LDS base (M0) and one per-lane offset each: transfer j adds
  // 1024 * j through the instruction's immediate offset, which the hardware adds to both the
  // memory and the LDS address. `vo[j]` = memory offset of this lane's 16 bytes of transfer j,
  // relative to the step's first row, minus 1024 * j (fast_voff).
  static constexpr int kWave = kLoads * 1024;
  static constexpr bool kFast = kLoads <= 4;  // immediate offsets up to 3072
  __device__ __forceinline__ static uint32_t fast_voff(int j) {
    const int byte = int(threadIdx.x >> 6) * kWave + 1024 * j + 16 * int(threadIdx.x & 63);
    const int row = byte / kRowBytes, pc = (byte % kRowBytes) / 16;
    return uint32_t(row * kRowBytes + swz(row, pc) * 16 - 1024 * j);
  }
  template <int J>
  __device__ __forceinline__ static void dma_at(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t vo) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, vo, 0, 1024 * J, 0);
  }
  // `wb` = this wave's byte offset in the tile (wave * kWave, uniform).
  __device__ __forceinline__ static void dma_fast(const void* src, const uint32_t (&vo)[4],
                                                  char* lds, int wb) {
    static_assert(kFast, "fast transfers need kLoads <= 4");
    const __amdgpu_buffer_rsrc_t r = rsrc(src);
    char* dst = lds + wb;
    dma_at<0>(r, dst, vo[0]);
    if constexpr (kLoads > 1) dma_at<1>(r, dst, vo[1]);
    if constexpr (kLoads > 2) dma_at<2>(r, dst, vo[2]);
    if constexpr (kLoads > 3) dma_at<3>(r, dst, vo[3]);
  }
  // Pages smaller than a step: every row looks up its own page; offsets are taken from the
  // pool start (pools under 2 GiB, checked on the host).
  template <bool kK, bool kV>
  __device__ __forceinline__ static void dma_small_pages(const AttnParams& p, int vstart, int ti0,
                                                         int vlo, int vhi, char* lk, char* lv) {
    const __amdgpu_buffer_rsrc_t rk = rsrc(p.k), rv = rsrc(p.v);
    const int wbase = uniform(int(threadIdx.x >> 6)) * 1024;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int row = piece_row(j);
      uint32_t o = kOut;
      if (row >= vlo && row < vhi) {
        const int ti = ti0 + row;
        const int phys = p.v2p[vstart + ti / p.P];
        if (uint32_t(phys) < uint64_t(p.n_phys))
          o = uint32_t((phys * p.P + (ti & (p.P - 1))) * kRowBytes + piece_chunk(j) * 16);
      }
      if constexpr (kK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(lk + j * 4096 + wbase), 16, o,
                                                 0, 0, 0);
      if constexpr (kV)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(lv + j * 4096 + wbase), 16, o,
                                                 0, 0, 0);
    }
  }
};

// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave still in flight. They
// complete in issue order, so every operation issued before the last N has landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Work-group barrier for the KV pipeline: this wave's LDS reads are done (lgkmcnt 0) and at
// most N of its DMAs are in flight, then all waves meet. Unlike __syncthreads it carries no
// release fence, which would drain every in-flight LDS-DMA (vmcnt 0) and defeat the
// prefetch; the "memory" clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void kv_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

// Uniform load through the scalar data cache (read-only use): keeps page-table lookups off
// the vector-memory counter that tracks the KV DMAs.
__device__ __forceinline__ int scalar_ld(const int32_t* p, int idx) {
  typedef __attribute__((address_space(4))) const int32_t cint;
  return ((cint*)(p))[idx];
}

// Step c of item w with its source offset. For pages of at least one step the page-table
// lookup happens here, once per step, through the scalar cache; a physical page outside the
// pool flags SP_ERR_INVALID_ARG and the step becomes empty.
template <int D, bool kDense>
__device__ __forceinline__ Step describe_step(const AttnParams& p, const WorkItem& w,
                                              const ItemKV& kv, int c) {
  Step s = step_range(w, kv, c, kDense);
  if constexpr (kDense) {
    s.off = (int64_t(w.kv_row0 + s.ti0) * p.Hkv + w.h) * D;
  } else {
    if (p.P >= kChunk && s.vhi > s.vlo) {
      const int vs = s.seg == 0 ? kv.vstart0 : kv.vstart1;
      const int phys = scalar_ld(p.v2p, uniform(vs + s.ti0 / p.P));
      if (uint32_t(phys) >= uint64_t(p.n_phys)) {
        if (threadIdx.x == 0) set_error(p.ws, SP_ERR_INVALID_ARG);
        s.vlo = s.vhi = 0;
      } else {
        s.off = (int64_t(phys) * p.P + (s.ti0 & (p.P - 1))) * D;
      }
    }
  }
  return s;
}

__device__ __forceinline__ void load_item_kv(const AttnParams& p, const WorkItem& w, bool dense,
                                             ItemKV& kv, uint8_t* ws) {
  if (!dense) {
    const int32_t* e = p.seg_table + (int64_t(w.b) * p.Hkv + w.h) * 8;
    kv.pos0 = uniform(e[0]);
    kv.ntok0 = uniform(e[1]);
    kv.vstart0 = uniform(e[2]);
    kv.pos1 = uniform(e[4]);
    kv.ntok1 = uniform(e[5]);
    kv.vstart1 = uniform(e[6]);
    const int kl = uniform(p.kv_len[int64_t(w.b) * p.Hkv + w.h]);
    const int na = w.ra_seg == 0 ? kv.ntok0 : kv.ntok1;
    const int nb = w.rb_seg == 0 ? kv.ntok0 : kv.ntok1;
    const bool bad = kl != kv.ntok0 + kv.ntok1 || (w.ra_end > w.ra_begin && w.ra_end > na) ||
                     (w.rb_end > w.rb_begin && w.rb_end > nb);
    if (bad && threadIdx.x == 0) set_error(ws, SP_ERR_INVALID_ARG);
  } else {
    kv.pos0 = kv.pos1 = 0;
    kv.ntok0 = kv.ntok1 = 0;
    kv.vstart0 = kv.vstart1 = 0;
  }
  kv.n_ra = w.ra_end > w.ra_begin ? (w.ra_end + kChunk - 1) / kChunk - w.ra_begin / kChunk : 0;
}

__device__ __forceinline__ WorkItem load_item(const WorkItem* items, int it) {
  const int32_t* src = reinterpret_cast<const int32_t*>(items + it);
  WorkItem w;
  int32_t* dst = reinterpret_cast<int32_t*>(&w);
#pragma unroll
  for (int i = 0; i < 16; ++i) dst[i] = uniform(src[i]);
  return w;
}

__device__ __forceinline__ bool header_ok(const AttnParams& p) {
  const WsHeader* hd = reinterpret_cast<const WsHeader*>(p.ws);
  return hd->magic == kMagic && hd->signature == p.signature && hd->bytes <= p.ws_bytes;
}

// Issues the LDS-DMA of step `st` of item `w` into the tile at lk / lv.
// An empty step: no rows. Its DMA writes zeros and touches no page table entry; issuing it
// keeps the count of vector-memory operations per iteration uniform.
__device__ __forceinline__ Step empty_step() { return Step{0, 0, 0, 0, 0, 0}; }

// Issues the LDS-DMA of K (kK) and/or V (kV) of step `st` of item `w` into lk / lv.
template <class E, int D, bool kDense, bool kK, bool kV>
__device__ __forceinline__ void issue_step(const AttnParams& p, const WorkItem& w,
                                           const ItemKV& kv, const Step& st, char* lk, char* lv) {
  using T = KVTile<E, D>;
  using S = typename E::S;
  if (st.vhi <= st.vlo) {
    T::template dma_strided<kK, kV>(p.k, p.v, 0, 0, 0, false, lk, lv);
    return;
  }
  const bool full = st.vlo == 0 && st.vhi == kChunk;
  const S* kb = static_cast<const S*>(p.k) + st.off;
  const S* vb = static_cast<const S*>(p.v) + st.off;
  if constexpr (kDense) {
    T::template dma_strided<kK, kV>(kb, vb, uint32_t(p.Hkv) * T::kRowBytes, st.vlo, st.vhi, full,
                                    lk, lv);
  } else {
    if (p.P >= kChunk) {
      T::template dma_strided<kK, kV>(kb, vb, T::kRowBytes, st.vlo, st.vhi, full, lk, lv);
    } else {
      const int vs = st.seg == 0 ? kv.vstart0 : kv.vstart1;
      T::template dma_small_pages<kK, kV>(p, vs, st.ti0, st.vlo, st.vhi, lk, lv);
    }
  }
}

// The KV steps of a prefill item, 64 at a time in one register per field: lane j describes
// step win + j of the item. Read per step with v_readlane (no memory access, no wait), so the
// step loop carries no page lookups or range arithmetic; refilled every 64 steps.
//   lo, hi : paged, pages of at least one step: byte offset of the step's first row in the
//            pool (64 bits); smaller pages: the step's first stored index and the segment's
//            first virtual page; dense: byte offset of the step's first row in the dense K/V
//   pos    : key position of slot 0
//   rng    : valid slots vlo | vhi << 8; 0 for an empty step (past the item's end)
struct StepLane {
  uint32_t lo, hi;
  int pos, rng;
};
constexpr int kFullRange = kChunk << 8;  // vlo 0, vhi 64

// Bit of StepLane::rng: the step straddles a causal or window edge, or is not full, so its
// scores need the visibility mask (the dense comparison path masks every step).
constexpr int kNeedsMask = 1 << 16;

template <int D, bool kDense, int RB>
__device__ __forceinline__ StepLane fill_steps(const AttnParams& p, const WorkItem& w,
                                               const ItemKV& kv, int n, int win, int kind,
                                               int sink, int window, int pmin, int pmax) {
  const int i = win + int(threadIdx.x & 63);
  const int c = w.c_begin + i;
  const bool ia = c < kv.n_ra;
  const int lo = ia ? w.ra_begin : w.rb_begin;
  const int hi = ia ? w.ra_end : w.rb_end;
  const int base = ia ? w.ra_begin / kChunk + c : w.rb_begin / kChunk + (c - kv.n_ra);
  const int seg = ia ? w.ra_seg : w.rb_seg;
  const int ti0 = base * kChunk;
  int vlo = max(0, lo - ti0), vhi = min(kChunk, hi - ti0);
  if (i >= n || vhi <= vlo) vlo = vhi = 0;
  StepLane s;
  s.pos = kDense ? ti0 : (seg == 0 ? kv.pos0 : kv.pos1) + ti0;
  uint64_t off = 0;
  if constexpr (kDense) {
    off = uint64_t((int64_t(w.kv_row0 + ti0) * p.Hkv + w.h) * RB);
  } else {
    const int vs = seg == 0 ? kv.vstart0 : kv.vstart1;
    if (p.P >= kChunk) {
      if (vhi > vlo) {
        const int phys = p.v2p[vs + ti0 / p.P];
        if (uint32_t(phys) >= uint64_t(p.n_phys)) {
          set_error(p.ws, SP_ERR_INVALID_ARG);
          vlo = vhi = 0;
        } else {
          off = uint64_t((int64_t(phys) * p.P + (ti0 & (p.P - 1))) * RB);
        }
      }
    } else {
      off = uint64_t(uint32_t(ti0)) | (uint64_t(uint32_t(vs)) << 32);
    }
  }
  s.lo = uint32_t(off);
  s.hi = uint32_t(off >> 32);
  const int last = s.pos + kChunk - 1;
  const bool clear = vlo == 0 && vhi == kChunk && last <= pmin &&
                     (kind == SP_GLOBAL || last < sink || s.pos > pmax - window);
  s.rng = vhi > vlo ? vlo | (vhi << 8) | (kDense || !clear ? kNeedsMask : 0) : 0;
  return s;
}

__device__ __forceinline__ StepLane read_step(const StepLane& t, int lane) {
  StepLane s;
  s.lo = uint32_t(__builtin_amdgcn_readlane(int(t.lo), lane));
  s.hi = uint32_t(__builtin_amdgcn_readlane(int(t.hi), lane));
  s.pos = __builtin_amdgcn_readlane(t.pos, lane);
  s.rng = __builtin_amdgcn_readlane(t.rng, lane);
  return s;
}

__device__ __forceinline__ StepLane no_step() { return StepLane{0u, 0u, 0, 0}; }

__device__ __forceinline__ Step as_step(const StepLane& s) {
  return Step{0, 0, s.rng & 0xff, (s.rng >> 8) & 0xff, s.pos, 0};
}

// LDS-DMA of K (kK) or V of one step from its table entry. Full steps of a paged pool with
// pages of at least one step take the fast transfers; partial steps (rows outside the valid
// range read as zero), small pages and the dense path take the general ones; empty steps
// issue nothing (their tile is never read).
template <class E, int D, bool kDense, bool kK>
__device__ __forceinline__ void issue_table_step(const AttnParams& p, const StepLane& s,
                                                 const uint32_t (&vo)[4], int wb, char* lds) {
  using T = KVTile<E, D>;
  if (s.rng == 0) return;
  const void* pool = kK ? p.k : p.v;
  const uint64_t off = uint64_t(s.lo) | (uint64_t(s.hi) << 32);
  const int vlo = s.rng & 0xff, vhi = (s.rng >> 8) & 0xff;
  const bool full = (s.rng & 0xffff) == kFullRange;
  if constexpr (!kDense && T::kFast) {
    if (p.P >= kChunk && full) {
      T::dma_fast(static_cast<const char*>(pool) + off, vo, lds, wb);
      return;
    }
  }
  if constexpr (kDense) {
    const char* b = static_cast<const char*>(pool) + off;
    T::template dma_strided<kK, !kK>(b, b, uint32_t(p.Hkv) * T::kRowBytes, vlo, vhi, full, lds,
                                     lds);
  } else {
    if (p.P >= kChunk) {
      const char* b = static_cast<const char*>(pool) + off;
      T::template dma_strided<kK, !kK>(b, b, T::kRowBytes, vlo, vhi, full, lds, lds);
    } else {
      T::template dma_small_pages<kK, !kK>(p, int(s.hi), int(s.lo), vlo, vhi, lds, lds);
    }
  }
}

template <class T>
__device__ __forceinline__ T lds_ld(const char* p) {
  return *reinterpret_cast<const T*>(p);
}

// Four bf16 of V transposed by the LDS unit: lane j of each 16-lane group receives element
// j % 4 of the 8-byte rows addressed by lanes 4e + j / 4 of its group, e = 0..3.
__device__ __forceinline__ s16x4_t lds_tr4(const char* p) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

// Visible keys of one step for one query row, as slot intervals. A step holds positions
// pos0 .. pos0+63 (slots outside [vlo, vhi) are empty). For a query at p_row the visible slots
// are those <= p_row - pos0 that are sink positions (< sink) or inside the window
// (> p_row - window); GLOBAL heads drop the second condition. A step is "dual" when it holds
// sink positions and may also hold window positions; then two intervals are needed, otherwise
// one. Intervals are (start, length) and tested as (unsigned)(key - start) < length.
struct KeyMask {
  int a0, n0, a1, n1;
};

__device__ __forceinline__ bool step_is_dual(const Step& st, int kind, int sink, int window,
                                             int pmin) {
  return kind != SP_GLOBAL && st.pos0 < sink && st.pos0 + kChunk - 1 > pmin - window;
}

__device__ __forceinline__ KeyMask key_mask(const Step& st, int p_row, int kind, int sink,
                                            int window, bool dual, int lane_off) {
  const int hi = min(st.vhi - 1, p_row - st.pos0);
  int lo0 = st.vlo, hi0 = hi, lo1 = 1, hi1 = 0;
  if (kind != SP_GLOBAL) {
    const int band = p_row - window + 1 - st.pos0;  // first window slot
    const int sk = sink - st.pos0;                  // first slot past the sink
    if (dual) {
      hi0 = min(hi, sk - 1);
      lo1 = max(st.vlo, band);
      hi1 = hi;
    } else if (st.pos0 >= sink) {
      lo0 = max(st.vlo, band);
    } else {
      hi0 = min(hi, sk - 1);
    }
  }
  KeyMask m;
  m.a0 = lo0 - lane_off;
  m.n0 = max(0, hi0 - lo0 + 1);
  m.a1 = lo1 - lane_off;
  m.n1 = max(0, hi1 - lo1 + 1);
  return m;
}

__device__ __forceinline__ bool in_mask(const KeyMask& m, int c, bool dual) {
  const bool v = uint32_t(c - m.a0) < uint32_t(m.n0);
  return dual ? (v || uint32_t(c - m.a1) < uint32_t(m.n1)) : v;
}

// The same mask as 64 bits, bit c for value position c (positions outside 0..63 are never
// visible): built once per row and step, then each of a lane's 32 values costs two bit
// operations (sign-extend bit c, then select the value's bits or -inf's) instead of a
// subtract, compare and select per interval.
__device__ __forceinline__ uint64_t range_bits(int a, int n) {
  const int lo = max(a, 0), hi = min(a + n, 64);
  if (hi <= lo) return 0ull;
  const uint64_t ones = hi - lo >= 64 ? ~0ull : (1ull << (hi - lo)) - 1ull;
  return ones << lo;
}

__device__ __forceinline__ uint64_t mask_bits(const KeyMask& m, bool dual) {
  const uint64_t b = range_bits(m.a0, m.n0);
  return dual ? b | range_bits(m.a1, m.n1) : b;
}

// x if bit c of `bits` is set, else -inf.
__device__ __forceinline__ float keep_if(uint32_t bits, int c, float x) {
  const uint32_t k = uint32_t(int32_t(bits << (31 - c)) >> 31);
  return __uint_as_float((k & __float_as_uint(x)) | (~k & 0xff800000u));
}

// An item of a table-driven decode plan (ra_seg < 0) carries only its split: split c_begin of
// c_end over all tokens its (request, KV head) stores, as the device tables hold them when the
// kernel runs (segment 0, then segment 1). The query is the newest stored token: in decode the
// request's last context position, which every head stores.
__device__ __forceinline__ void table_item(WorkItem& w, ItemKV& kv) {
  const int na = kv.ntok0, nb = kv.ntok1;
  const int sa = (na + kChunk - 1) / kChunk, sb = (nb + kChunk - 1) / kChunk;
  const int64_t n = sa + sb;
  const int k = w.c_begin, ns = max(w.c_end, 1);
  w.ra_seg = 0;
  w.ra_begin = 0;
  w.ra_end = na;
  w.rb_seg = 1;
  w.rb_begin = 0;
  w.rb_end = nb;
  w.c_begin = int(n * k / ns);
  w.c_end = int(n * (k + 1) / ns);
  w.p0 = (nb > 0 ? kv.pos1 + nb : kv.pos0 + na) - 1;
  kv.n_ra = sa;
}

// ---------------------------------------------------------------------------------------
// Prefill: persistent, 256 threads, 128-row tiles.
// ---------------------------------------------------------------------------------------
template <class E, int D, int MODE>
__global__ void __launch_bounds__(256, (sizeof(typename E::S) == 2 ? 2 : 1))
    prefill_kernel(AttnParams p) {
  using S = typename E::S;
  using T = KVTile<E, D>;
  constexpr int KPL = E::KPL;
  constexpr bool kBf16 = KPL == 8;
  constexpr int NQK = D / (2 * KPL);  // MFMAs per 32-key block for S^T = K Q^T
  constexpr int ND = D / 32;          // 32-dim blocks of O^T
  constexpr bool kDense = MODE == kModeDense;
  constexpr int RB = T::kRowBytes;

  // Two K and two V stages as four separate objects, so that the compiler can tell an LDS
  // read of one stage from a DMA into another and does not wait for the DMA.
  __shared__ __attribute__((aligned(16))) char lk0[T::kBytes];
  __shared__ __attribute__((aligned(16))) char lk1[T::kBytes];
  __shared__ __attribute__((aligned(16))) char lv0[T::kBytes];
  __shared__ __attribute__((aligned(16))) char lv1[T::kBytes];
  __shared__ int s_item;

  if (!header_ok(p)) {
    if (threadIdx.x == 0 && blockIdx.x == 0) set_error(p.ws, SP_ERR_PLAN_MISMATCH);
    return;
  }
  const WsHeader* hd = reinterpret_cast<const WsHeader*>(p.ws);
  const WorkItem* items = reinterpret_cast<const WorkItem*>(p.ws + hd->off_prefill);
  const int32_t* pol = reinterpret_cast<const int32_t*>(p.ws + hd->off_policy);
  float* part_o = reinterpret_cast<float*>(p.ws + hd->off_part_pre);
  float* part_ml = reinterpret_cast<float*>(p.ws + hd->off_ml_pre);

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 31, hh = lane >> 5;
  const int xcd = blockIdx.x % kXcds;
  const Queues queues = load_queues(hd->prefill_q, xcd);
  uint32_t exhausted = 0;
  bool first = true;
  const S* qbase = static_cast<const S*>(p.q);
  S* obase = static_cast<S*>(p.o);

  // Per-lane LDS offsets inside a tile.
  int kaddr[NQK];  // K fragment c of key row lq (add 32 * RB for the second key block)
#pragma unroll
  for (int c = 0; c < NQK; ++c) kaddr[c] = T::off(lq, (2 * KPL * c + KPL * hh) * int(sizeof(S)));
  int vaddr[2][ND];  // bf16: transposed V reads, half r of the 8 keys of one P*V MFMA
  if constexpr (kBf16) {
    const int s = lane & 15, g = lane >> 4;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int d = 0; d < ND; ++d)
        vaddr[r][d] = T::off(8 * r + 4 * (g >> 1) + (s >> 2), 2 * (32 * d + 16 * (g & 1) + 4 * (s & 3)));
  }

  // Per-lane memory offsets of the fast step transfers (shared by K and V), and this wave's
  // byte offset in a tile.
  const int wb = wave * T::kWave;
  uint32_t vo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vo[j] = T::kFast && j < T::kLoads ? T::fast_voff(j) : 0u;

  for (;;) {
    if (tid == 0) s_item = pop_item(p.ws, queues, kOffPrefillCnt, xcd, exhausted, first);
    __syncthreads();
    const int it = uniform(s_item);
    if (it < 0) break;
    WorkItem w = load_item(items, it);
    ItemKV kv;
    load_item_kv(p, w, kDense, kv, p.ws);
    if constexpr (!kDense) {
      if (w.ra_seg < 0) table_item(w, kv);  // a decode query of more than 16 rows
    }
    const int32_t* ph = pol + (w.b * p.Hkv + w.h) * 3;  // effective policy of (request, head)
    const int kind = uniform(ph[0]);
    const int sink = uniform(ph[1]);
    const int window = uniform(ph[2]);

    // This lane's query row.
    const int r = wave * 32 + lq;
    const int tl = r / p.G, g = r - tl * p.G;
    const bool row_ok = tl < w.nq;
    const int p_row = w.p0 + w.tq0 + tl;
    const int64_t orow = int64_t(w.q_row0 + w.tq0 + tl) * p.Hq + int64_t(w.h) * p.G + g;
    typename E::Frag qf[NQK];
#pragma unroll
    for (int c = 0; c < NQK; ++c) {
      qf[c] = row_ok ? load_frag<E>(qbase + orow * D + 2 * KPL * c + KPL * hh) : zero_frag<E>();
    }
    const int pmin = w.p0 + w.tq0, pmax = pmin + w.nq - 1;

    f32x16_t oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x16_t{};
    float m_run = kNegInf, l_run = 0.f;

    // Software pipeline over the item's KV steps. Iteration i runs S^T of step i on the
    // matrix cores alongside the softmax of step i-1 on the vector ALUs (independent work in
    // one instruction stream), then P*V of step i-1. K(i+1) and V(i) are in flight during
    // iteration i; K stage j & 1 holds K(j), V stage j & 1 holds V(j). One barrier per step.
    using F = typename E::Frag;
    auto qk = [&](const char* lk, f32x16_t& a0, f32x16_t& a1) {
      a0 = f32x16_t{};
      a1 = f32x16_t{};
      constexpr int kAhead = 2;  // K fragment pairs in flight ahead of the MFMAs
      F fa[kAhead + 1][2];
#pragma unroll
      for (int c = 0; c < kAhead && c < NQK; ++c) {
        fa[c][0] = lds_ld<F>(lk + kaddr[c]);
        fa[c][1] = lds_ld<F>(lk + 32 * RB + kaddr[c]);
      }
#pragma unroll
      for (int c = 0; c < NQK; ++c) {
        if (c + kAhead < NQK) {
          fa[(c + kAhead) % (kAhead + 1)][0] = lds_ld<F>(lk + kaddr[c + kAhead]);
          fa[(c + kAhead) % (kAhead + 1)][1] = lds_ld<F>(lk + 32 * RB + kaddr[c + kAhead]);
        }
        a0 = mma32(fa[c % (kAhead + 1)][0], qf[c], a0);
        a1 = mma32(fa[c % (kAhead + 1)][1], qf[c], a1);
      }
    };
    // Masks step st where it straddles a causal or window edge or is not full.
    auto mask = [&](const StepLane& sl, f32x16_t& a0, f32x16_t& a1) {
      if (sl.rng & kNeedsMask) {
        const Step st = as_step(sl);
        const bool dual = step_is_dual(st, kind, sink, window, pmin);
        const uint64_t mb = mask_bits(key_mask(st, p_row, kind, sink, window, dual, 4 * hh), dual);
        const uint32_t m_lo = uint32_t(mb), m_hi = uint32_t(mb >> 32);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int c = 8 * (rr >> 2) + (rr & 3);
          a0[rr] = keep_if(m_lo, c, a0[rr]);
          a1[rr] = keep_if(m_hi, c, a1[rr]);  // value position 32 + c
        }
      }
    };
    // Softmax reference: m_run is a per-row reference, not the exact running maximum. It
    // moves (and O and l are rescaled to it) only when some row's maximum passes it by more
    // than kSlack, so every exponential stays at most 2^kSlack; with logits of ordinary spread
    // that happens on a row's first steps only, and the O rescale drops out of the loop.
    // Returns the reference the step's exponentials use.
    auto update_max = [&](const f32x16_t& a0, const f32x16_t& a1) -> float {
      // two chains of three-input maxima, then the other half-wave's value (rows of lane l
      // and lane l ^ 32 are the same query row) through a half swap, no LDS round trip
      float ma = fmaxf(fmaxf(a0[0], a0[1]), a0[2]), mb = fmaxf(fmaxf(a1[0], a1[1]), a1[2]);
#pragma unroll
      for (int t = 3; t < 15; t += 2) {
        ma = fmaxf(fmaxf(ma, a0[t]), a0[t + 1]);
        mb = fmaxf(fmaxf(mb, a1[t]), a1[t + 1]);
      }
      ma = fmaxf(fmaxf(ma, a0[15]), fmaxf(mb, a1[15]));
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ma), __float_as_uint(ma),
                                                       false, false);
      float mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * p.scale_log2;
      if (__ballot(mx > m_run + kSlack) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast(m_run - (m_new == kNegInf ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
      }
      return m_run == kNegInf ? 0.f : m_run;
    };
    // Probabilities of one step against reference m_use: the P operand, and l += row sums.
    auto probs = [&](f32x16_t& a0, f32x16_t& a1, float m_use, F (&pb)[2][16 / KPL]) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        a0[rr] = exp2_fast(__builtin_fmaf(a0[rr], p.scale_log2, -m_use));
        a1[rr] = exp2_fast(__builtin_fmaf(a1[rr], p.scale_log2, -m_use));
      }
      if constexpr (kBf16) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          pb[0][ii] = to_bf16x8(a0[8 * ii + 0], a0[8 * ii + 1], a0[8 * ii + 2], a0[8 * ii + 3],
                                a0[8 * ii + 4], a0[8 * ii + 5], a0[8 * ii + 6], a0[8 * ii + 7]);
          pb[1][ii] = to_bf16x8(a1[8 * ii + 0], a1[8 * ii + 1], a1[8 * ii + 2], a1[8 * ii + 3],
                                a1[8 * ii + 4], a1[8 * ii + 5], a1[8 * ii + 6], a1[8 * ii + 7]);
        }
        // l += the row sums of the bf16 probabilities the P*V product uses, two per dot2.
        // (The pairs are taken with shufflevector: taking them as bit casts of the vector's
        // 32-bit words is folded wrongly by this compiler, into one word summed four times.)
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int ii = 0; ii < 2; ++ii) {
            const bf16x8_t x = pb[kb][ii];
            acc[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), ones,
                                                     acc[0], false);
            acc[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), ones,
                                                     acc[1], false);
            acc[2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), ones,
                                                     acc[2], false);
            acc[3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), ones,
                                                     acc[3], false);
          }
        l_run += (acc[0] + acc[1]) + (acc[2] + acc[3]);
      } else {
        float r8[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
          r8[t] = (a0[2 * t] + a0[2 * t + 1]) + (a1[2 * t] + a1[2 * t + 1]);
#pragma unroll
        for (int t = 0; t < 4; ++t) r8[t] += r8[t + 4];
        l_run += (r8[0] + r8[1]) + (r8[2] + r8[3]);
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          pb[0][ii] = a0[ii];
          pb[1][ii] = a1[ii];
        }
      }
    };
    // O^T[dim][row] += V^T P^T for one step.
    auto pv = [&](const char* lv, const F (&pb)[2][16 / KPL]) {
      if constexpr (kBf16) {
        constexpr int kN = 4 * ND;  // P*V MFMAs per step: (key block, half) x dim block
        constexpr int kAhead = 2;
        s16x4_t tv[kAhead + 1][2];
        auto vread = [&](int m, s16x4_t* t) {
          const int kb = m / (2 * ND), ii = (m / ND) & 1, d = m % ND;
          const char* base = lv + (32 * kb + 16 * ii) * RB;
          t[0] = lds_tr4(base + vaddr[0][d]);
          t[1] = lds_tr4(base + vaddr[1][d]);
        };
#pragma unroll
        for (int m = 0; m < kAhead; ++m) vread(m, tv[m]);
#pragma unroll
        for (int m = 0; m < kN; ++m) {
          if (m + kAhead < kN) vread(m + kAhead, tv[(m + kAhead) % (kAhead + 1)]);
          const int kb = m / (2 * ND), ii = (m / ND) & 1, d = m % ND;
          const s16x4_t* t = tv[m % (kAhead + 1)];
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[d] = mma32(a, pb[kb][ii], oacc[d]);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int ii = 0; ii < 16; ++ii) {
            const int key = 32 * kb + 8 * (ii >> 2) + 4 * hh + (ii & 3);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
              const float a = lds_ld<float>(lv + T::off(key, 4 * (32 * d + lq)));
              oacc[d] = mma32(a, pb[kb][ii], oacc[d]);
            }
          }
        }
      }
    };

    const int n = w.c_end - w.c_begin;
    StepLane tab = fill_steps<D, kDense, RB>(p, w, kv, n, 0, kind, sink, window, pmin, pmax);
    // Prologue: S^T, mask and row maximum of step 0; K(1) and V(0) land meanwhile.
    const StepLane s0 = read_step(tab, 0);
    StepLane cur = n > 1 ? read_step(tab, 1) : no_step();  // step 1
    issue_table_step<E, D, kDense, true>(p, s0, vo, wb, lk0);
    kv_barrier<0>();
    issue_table_step<E, D, kDense, true>(p, cur, vo, wb, lk1);
    issue_table_step<E, D, kDense, false>(p, s0, vo, wb, lv0);
    f32x16_t sp0, sp1;
    qk(lk0, sp0, sp1);
    mask(s0, sp0, sp1);
    float mp = update_max(sp0, sp1);
    kv_barrier<0>();

    // Iteration i: S^T(i) on the matrix cores interleaved with the exponentials of step i-1,
    // then P*V(i-1) (one basic block, instruction mix set by step_schedule); then the mask and
    // row maximum of step i, and O and l move to the new reference if needed. K(i+1) and V(i)
    // are in flight. `cur` is step i; step i+1 comes from the step table (refilled when it
    // starts a new window of 64).
    auto run_step = [&](auto stage_c, int i) {
      constexpr int stg = decltype(stage_c)::value;  // i & 1
      StepLane nxt = no_step();
      if (i + 1 < n) {
        if (((i + 1) & 63) == 0) tab = fill_steps<D, kDense, RB>(p, w, kv, n, i + 1, kind, sink, window, pmin,
                                         pmax);
        nxt = read_step(tab, (i + 1) & 63);
      }
      issue_table_step<E, D, kDense, true>(p, nxt, vo, wb, stg ? lk0 : lk1);
      issue_table_step<E, D, kDense, false>(p, cur, vo, wb, stg ? lv1 : lv0);
      f32x16_t sc0, sc1;
      qk(stg ? lk1 : lk0, sc0, sc1);
      F pb[2][16 / KPL];
      probs(sp0, sp1, mp, pb);
      pv(stg ? lv0 : lv1, pb);
      // 32 scores per lane: 32 FMA + 16 packs + 16 dot2 and 32 exponentials; the exponentials
      // and four VALU per S^T MFMA, the rest among the P*V MFMAs (measured best of the
      // interleaves tried, by about 1 % over three VALU per S^T MFMA)
      if constexpr (kBf16)
        step_schedule<2 * NQK, 64 / (2 * NQK), 32 / (2 * NQK), 4 * ND, 16 / (4 * ND), 3>();
      mask(cur, sc0, sc1);
      mp = update_max(sc0, sc1);
      kv_barrier<0>();
      sp0 = sc0;
      sp1 = sc1;
      cur = nxt;
    };
    for (int i = 1; i < n; i += 2) {
      run_step(std::integral_constant<int, 1>{}, i);
      if (i + 1 < n) run_step(std::integral_constant<int, 0>{}, i + 1);
    }
    {
      // Last step: its V landed at the final barrier.
      F pb[2][16 / KPL];
      probs(sp0, sp1, mp, pb);
      pv(((n - 1) & 1) ? lv1 : lv0, pb);
    }

    // Epilogue.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (w.part < 0) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      if (row_ok) {
        S* dst = obase + orow * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int dim = 32 * d + 8 * g4 + 4 * hh;
            const float o0 = oacc[d][4 * g4 + 0] * inv, o1 = oacc[d][4 * g4 + 1] * inv;
            const float o2 = oacc[d][4 * g4 + 2] * inv, o3 = oacc[d][4 * g4 + 3] * inv;
            if constexpr (kBf16) {
              u32x2_t v = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
              *reinterpret_cast<u32x2_t*>(dst + dim) = v;
            } else {
              f32x4_t v = {o0, o1, o2, o3};
              *reinterpret_cast<f32x4_t*>(dst + dim) = v;
            }
          }
        }
      }
    } else {
      float* po = part_o + (int64_t(w.part) * kTileRows + r) * D;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dim = 32 * d + 8 * g4 + 4 * hh;
          f32x4_t v = {oacc[d][4 * g4 + 0], oacc[d][4 * g4 + 1], oacc[d][4 * g4 + 2],
                       oacc[d][4 * g4 + 3]};
          *reinterpret_cast<f32x4_t*>(po + dim) = v;
        }
      }
      if (hh == 0) {
        float* pm = part_ml + (int64_t(w.part) * kTileRows + r) * 2;
        pm[0] = m_run;
        pm[1] = l_tot;
      }
    }
    __syncthreads();
  }
  if (tid == 0 && !queues.one_round) retire(p.ws, kOffPrefillCnt, kOffPrefillDone);
}

// ---------------------------------------------------------------------------------------
// Decode: persistent, one wave per work group and per work item, up to 16 query rows,
// split-KV. The wave walks its item in sub-steps of 16 keys; every page size is a multiple
// of 16, so a sub-step never straddles a page and needs one page-table lookup. K goes from
// memory straight into registers, already in MFMA operand layout; V goes by LDS-DMA into the
// wave's own ring of 16-row tiles (read back transposed). Both run kDecAhead sub-steps ahead
// of the arithmetic. Nothing is shared between waves, so the wave's own vector-memory
// counter orders every transfer and there is no work-group barrier: decode is bound by how
// many bytes are in flight, and this keeps several times more of them in flight per CU than
// a 256-thread tile shared through LDS can.
// ---------------------------------------------------------------------------------------
constexpr int kSub = 16;      // keys per decode sub-step
constexpr int kDecAhead = 3;  // sub-steps of K and V in flight ahead of the one computed

// One decode sub-step: rows [vlo, vhi) of 16 are valid; `off` is the element offset of row 0
// in the pool or the dense K/V (0 when there is no valid row).
struct Sub {
  int vlo, vhi, pos0;
  int64_t off;
};

// Source of a decode item's two slot ranges (A, then B): first step, valid slot bounds, first
// virtual page and first key position of each, resolved per item into plain integers. Per
// sub-step the range is picked arithmetically rather than by a select between fields, which
// the compiler can turn into a load through a selected address and so into scratch memory.
struct SubSrc {
  int n_ra, log2_p;
  int a_base, a_lo, a_hi, a_vs, a_pos;
  int b_base, b_lo, b_hi, b_vs, b_pos;
};

__device__ __forceinline__ SubSrc sub_source(const WorkItem& w, const ItemKV& kv, bool dense,
                                             int page_size) {
  SubSrc r;
  r.n_ra = kv.n_ra;
  r.log2_p = dense ? 0 : int(__builtin_ctz(uint32_t(page_size)));
  r.a_base = w.ra_begin / kChunk;
  r.a_lo = w.ra_begin;
  r.a_hi = w.ra_end;
  r.a_vs = w.ra_seg == 0 ? kv.vstart0 : kv.vstart1;
  r.a_pos = dense ? 0 : (w.ra_seg == 0 ? kv.pos0 : kv.pos1);
  r.b_base = w.rb_begin / kChunk - kv.n_ra;
  r.b_lo = w.rb_begin;
  r.b_hi = w.rb_end;
  r.b_vs = w.rb_seg == 0 ? kv.vstart0 : kv.vstart1;
  r.b_pos = dense ? 0 : (w.rb_seg == 0 ? kv.pos0 : kv.pos1);
  return r;
}

template <int D, bool kDense>
__device__ __forceinline__ Sub describe_sub(const AttnParams& p, const WorkItem& w,
                                            const SubSrc& r, int s) {
  const int c = w.c_begin + (s >> 2);
  const int ia = int(c < r.n_ra);  // 1: range A, 0: range B
  const int base = r.b_base + ia * (r.a_base - r.b_base) + c;
  const int lo = r.b_lo + ia * (r.a_lo - r.b_lo);
  const int hi = r.b_hi + ia * (r.a_hi - r.b_hi);
  const int vs = r.b_vs + ia * (r.a_vs - r.b_vs);
  const int pos = r.b_pos + ia * (r.a_pos - r.b_pos);
  const int t0 = base * kChunk + kSub * (s & 3);  // first slot of the sub-step
  Sub u;
  u.vlo = min(max(lo - t0, 0), kSub);
  u.vhi = min(max(hi - t0, 0), kSub);
  u.pos0 = pos + t0;
  u.off = 0;
  if (u.vhi > u.vlo) {
    if constexpr (kDense) {
      u.off = (int64_t(w.kv_row0 + t0) * p.Hkv + w.h) * D;
    } else {
      const int phys = scalar_ld(p.v2p, uniform(vs + (t0 >> r.log2_p)));
      if (uint32_t(phys) >= uint64_t(p.n_phys)) {
        if (__lane_id() == 0) set_error(p.ws, SP_ERR_INVALID_ARG);
        u.vlo = u.vhi = 0;
      } else {
        u.off = ((int64_t(phys) << r.log2_p) + (t0 & (p.P - 1))) * D;
      }
    }
  }
  return u;
}

// 16 bytes per lane from a buffer into registers / into LDS at lds + 16 * lane (device-only
// builtins kept out of the kernel body, which the host pass also parses). Decode reads every
// stored K/V byte exactly once, so these loads carry the non-temporal cache policy (NT, bit 1
// of the buffer instruction's cache-policy operand): the stream neither allocates in nor
// evicts from the L2s and the MALL, which lets it run closer to the HBM read rate.
constexpr int kPolicyStream = 2;
__device__ __forceinline__ u32x4_t buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicyStream);
}
__device__ __forceinline__ void buffer_dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, off, 0, 0, kPolicyStream);
}

template <class E, int D, int MODE>
__global__ void __launch_bounds__(64) decode_kernel(AttnParams p) {
  using S = typename E::S;
  using T = KVTile<E, D>;  // same row pitch and chunk swizzle, 16 rows used
  constexpr bool kBf16 = E::KPL == 8;
  constexpr bool kDense = MODE == kModeDense;
  constexpr int kTileBytes = kSub * T::kRowBytes;
  constexpr int kL = kTileBytes / 1024;  // 16-byte-per-lane transfers per K or V sub-step
  constexpr int ND = D / 16;             // 16-dim blocks of O^T
  constexpr int kStages = kDecAhead + 1;
  static_assert(kL >= 1 && kTileBytes % 1024 == 0, "sub-step tile is whole wave transfers");

  // The V ring as four separate objects: the compiler then tells a transposed read of one
  // stage from a DMA into another and does not wait for the DMA.
  __shared__ __attribute__((aligned(16))) char lv0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char lv1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char lv2[kTileBytes];
  __shared__ __attribute__((aligned(16))) char lv3[kTileBytes];
  auto ring = [&](int i) -> char* { return i == 0 ? lv0 : i == 1 ? lv1 : i == 2 ? lv2 : lv3; };

  if (!header_ok(p)) {
    if (__lane_id() == 0 && blockIdx.x == 0) set_error(p.ws, SP_ERR_PLAN_MISMATCH);
    return;
  }
  const WsHeader* hd = reinterpret_cast<const WsHeader*>(p.ws);
  const WorkItem* items = reinterpret_cast<const WorkItem*>(p.ws + hd->off_decode);
  const int32_t* pol = reinterpret_cast<const int32_t*>(p.ws + hd->off_policy);
  float* part_o = reinterpret_cast<float*>(p.ws + hd->off_part_dec);
  float* part_ml = reinterpret_cast<float*>(p.ws + hd->off_ml_dec);

  const int lane = __lane_id();
  const int lc = lane & 15, k4 = lane >> 4;
  const int xcd = blockIdx.x % kXcds;
  const Queues queues = load_queues(hd->decode_q, xcd);
  uint32_t exhausted = 0;
  bool first = true;
  const S* qbase = static_cast<const S*>(p.q);
  S* obase = static_cast<S*>(p.o);
  const uint32_t rs = kDense ? uint32_t(p.Hkv) * T::kRowBytes : uint32_t(T::kRowBytes);

  // K transfer j of a sub-step: lane (row lc, group k4) fetches bytes [64j + 16k4, +16) of
  // key row lc. bf16: that is the A operand of 16x16x32 MFMA j (dims 32j + 8k4 .. +7).
  // fp32: four floats, dims 16j + 4k4 + e, the A operands of 16x16x4 MFMAs 4j + e; the Q
  // operands below use the same dimension order, so the products sum over every dimension.
  const uint32_t k_lane = uint32_t(lc) * rs + 16u * uint32_t(k4);
  // V DMA j: lane writes LDS bytes [1024j + 16 lane, +16) = row (64j + lane) / kChunks, and so
  // fetches the source chunk the swizzle puts there.
  uint32_t v_lane[kL];
#pragma unroll
  for (int j = 0; j < kL; ++j) {
    const int n = 64 * j + lane;
    const int row = n / T::kChunks;
    v_lane[j] = uint32_t(row) * rs + uint32_t(T::swz(row, n % T::kChunks)) * 16u;
  }
  // bf16: transposed V reads, one per 16-dim block (see the prefill kernel for the layout).
  int vaddr[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
    vaddr[d] = kBf16 ? T::off(4 * k4 + (lc >> 2), 2 * (16 * d + 4 * (lc & 3))) : 0;

  for (;;) {
    int it = 0;
    if (lane == 0) it = pop_item(p.ws, queues, kOffDecodeCnt, xcd, exhausted, first);
    it = uniform(it);
    if (it < 0) break;
    WorkItem w = load_item(items, it);
    SubSrc src;
    {
      ItemKV kv;
      load_item_kv(p, w, kDense, kv, p.ws);
      if constexpr (!kDense) {
        if (w.ra_seg < 0) table_item(w, kv);
      }
      src = sub_source(w, kv, kDense, p.P);
    }
    const int32_t* ph = pol + (w.b * p.Hkv + w.h) * 3;  // effective policy of (request, head)
    const int kind = uniform(ph[0]);
    const int sink = uniform(ph[1]);
    const int window = uniform(ph[2]);
    const int rows = w.nq * p.G;

    // Query row of this lane's MFMA column.
    const int tl = lc / p.G, g = lc - tl * p.G;
    const bool row_ok = lc < rows;
    const int p_row = w.p0 + w.tq0 + tl;
    const int64_t orow = int64_t(w.q_row0 + w.tq0 + tl) * p.Hq + int64_t(w.h) * p.G + g;
    typename E::Frag qf[kBf16 ? kL : 4 * kL];
#pragma unroll
    for (int j = 0; j < kL; ++j) {
      if constexpr (kBf16) {
        qf[j] = row_ok ? load_frag<E>(qbase + orow * D + 32 * j + 8 * k4) : zero_frag<E>();
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qf[4 * j + e] = row_ok ? load_frag<E>(qbase + orow * D + 16 * j + 4 * k4 + e) : 0.f;
      }
    }
    const int pmin = w.p0 + w.tq0, pmax = pmin + w.nq - 1;

    f32x4_t oacc[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] = f32x4_t{};
    float m_run = kNegInf, l_run = 0.f;

    // Every sub-step issues kL K loads then kL V DMAs, so the counts below are exact: when
    // sub-step s is computed, K(s) has 2*kL*kDecAhead + kL transfers issued after it and V(s)
    // has 2*kL*kDecAhead.
    const int n_sub = 4 * (w.c_end - w.c_begin);
    u32x4_t kr[kStages][kL];
    auto issue = [&](int s, u32x4_t (&kdst)[kL], char* vdst) {
      const Sub u = s < n_sub ? describe_sub<D, kDense>(p, w, src, s) : Sub{0, 0, 0, 0};
      // Rows outside [vlo, vhi) read past the buffer's end and so as zeros (one compare and
      // one select per transfer; no branch, so the transfer count never varies).
      const __amdgpu_buffer_rsrc_t rk = T::rsrc(static_cast<const S*>(p.k) + u.off);
      const __amdgpu_buffer_rsrc_t rv = T::rsrc(static_cast<const S*>(p.v) + u.off);
      // (The offsets stay below 2^31; setting bit 31 moves them out of range. Written as an OR
      // rather than a select, which the compiler may turn into two predicated loads.)
      const uint32_t nv = uint32_t(u.vhi - u.vlo);
      const uint32_t kout = uint32_t(uint32_t(lc - u.vlo) >= nv) << 31;
#pragma unroll
      for (int j = 0; j < kL; ++j)
        kdst[j] = buffer_ld16(rk, (k_lane + 64u * j) | kout);
#pragma unroll
      for (int j = 0; j < kL; ++j) {
        const int row = (64 * j + lane) / T::kChunks;
        const uint32_t vout = uint32_t(uint32_t(row - u.vlo) >= nv) << 31;
        buffer_dma16(rv, vdst + 1024 * j, v_lane[j] | vout);
      }
    };
#pragma unroll
    for (int s = 0; s < kDecAhead; ++s) issue(s, kr[s], ring(s));

    auto run_sub = [&](auto stage_c, int s) {
      constexpr int stg = decltype(stage_c)::value;  // s % kStages
      constexpr int nxt = (stg + kDecAhead) % kStages;
      issue(s + kDecAhead, kr[nxt], ring(nxt));
      const Sub u = describe_sub<D, kDense>(p, w, src, s);
      wait_vm<2 * kL * kDecAhead + kL>();
      // S^T[key][row] for the sub-step's 16 keys: lane holds keys 4*k4 .. 4*k4+3 of row lc.
      f32x4_t sc = f32x4_t{};
#pragma unroll
      for (int j = 0; j < kL; ++j) {
        if constexpr (kBf16) {
          sc = mma16(__builtin_bit_cast(bf16x8_t, kr[stg][j]), qf[j], sc);
        } else {
          const f32x4_t kf = __builtin_bit_cast(f32x4_t, kr[stg][j]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc = mma16(kf[e], qf[4 * j + e], sc);
        }
      }
      const bool full = u.vlo == 0 && u.vhi == kSub;
      const int last = u.pos0 + kSub - 1;
      const bool clear = full && last <= pmin &&
                         (kind == SP_GLOBAL || last < sink || u.pos0 > pmax - window);
      if (kDense || !clear) {
        const Step st{0, 0, u.vlo, u.vhi, u.pos0, 0};
        const KeyMask km = key_mask(st, p_row, kind, sink, window, true, 4 * k4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sc[rr] = in_mask(km, rr, true) ? sc[rr] : kNegInf;
      }
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * p.scale_log2;
      // Softmax reference with 2^kSlack headroom, as in the prefill kernel.
      if (__ballot(mx > m_run + kSlack) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast(m_run - (m_new == kNegInf ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sc[rr] = exp2_fast(__builtin_fmaf(sc[rr], p.scale_log2, -m_use));
      l_run += (sc[0] + sc[1]) + (sc[2] + sc[3]);
      wait_vm<2 * kL * kDecAhead>();
      const char* lv = ring(stg);
      // O^T[dim][row] += V^T P^T over the sub-step's 16 keys.
      if constexpr (kBf16) {
        const s16x4_t b = __builtin_bit_cast(
            s16x4_t, u32x2_t{pack_bf16x2(sc[0], sc[1]), pack_bf16x2(sc[2], sc[3])});
#pragma unroll
        for (int d = 0; d < ND; ++d)
          oacc[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lds_tr4(lv + vaddr[d]), b, oacc[d],
                                                              0, 0, 0);
      } else {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const float a = lds_ld<float>(lv + T::off(4 * k4 + rr, 4 * (16 * d + lc)));
            oacc[d] = mma16(a, sc[rr], oacc[d]);
          }
        }
      }
    };
    static_assert(kStages == 4, "the sub-step loop below is unrolled for four stages");
    for (int s = 0; s < n_sub; s += 4) {
      run_sub(std::integral_constant<int, 0>{}, s);
      run_sub(std::integral_constant<int, 1>{}, s + 1);
      run_sub(std::integral_constant<int, 2>{}, s + 2);
      run_sub(std::integral_constant<int, 3>{}, s + 3);
    }
    // The trailing transfers (zero fills past the last sub-step) must land before the ring is
    // written by the next item.
    wait_vm<0>();

    // Epilogue: lane holds dims 16d + 4*k4 + r of query row lc.
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (row_ok) {
      const int q = lc;
      if (w.part < 0) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        S* dst = obase + orow * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const int dim = 16 * d + 4 * k4;
          if constexpr (kBf16) {
            *reinterpret_cast<u32x2_t*>(dst + dim) =
                u32x2_t{pack_bf16x2(oacc[d][0] * inv, oacc[d][1] * inv),
                        pack_bf16x2(oacc[d][2] * inv, oacc[d][3] * inv)};
          } else {
            *reinterpret_cast<f32x4_t*>(dst + dim) = oacc[d] * inv;
          }
        }
      } else {
        float* po = part_o + (int64_t(w.part) * kDecodeRows + q) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d)
          *reinterpret_cast<f32x4_t*>(po + 16 * d + 4 * k4) = oacc[d];
        if (k4 == 0) {
          part_ml[(int64_t(w.part) * kDecodeRows + q) * 2 + 0] = m_run;
          part_ml[(int64_t(w.part) * kDecodeRows + q) * 2 + 1] = l_tot;
        }
      }
    }
  }
  if (lane == 0 && !queues.one_round) retire(p.ws, kOffDecodeCnt, kOffDecodeDone);
}

// ---------------------------------------------------------------------------------------
// Combine: merges the partials of each KV-split block. A work group is 16 lanes x D/8
// dimension groups and takes one of 8 units of a block. Blocks with at most 8 splits or
// more than 16 rows (prefill): unit k merges rows 16k .. 16k+15, a lane per row. Blocks of
// up to 16 rows with more splits (decode): unit k merges rows 2k and 2k+1, 8 split lanes per
// row; split lane j folds splits j, j + 8, ... and the lanes are then folded in lane order.
// Every fold is an online rescale whose loads do not wait on earlier results, and the order
// is fixed, so O is bitwise reproducible.
// ---------------------------------------------------------------------------------------
struct MergeState {
  float m, l;
  f32x4_t a0, a1;
};

__device__ __forceinline__ void merge_into(MergeState& s, float m, float l, f32x4_t o0,
                                           f32x4_t o1) {
  const float mn = fmaxf(s.m, m);
  const float mu = mn == kNegInf ? 0.f : mn;
  const float fa = exp2_fast(s.m - mu), fb = exp2_fast(m - mu);
  s.l = s.l * fa + l * fb;
  s.a0 = s.a0 * fa + o0 * fb;
  s.a1 = s.a1 * fa + o1 * fb;
  s.m = mn;
}

template <class E, int D>
__global__ void __launch_bounds__(256) combine_kernel(AttnParams p) {
  using S = typename E::S;
  constexpr int kTpr = D / 8;                 // dimension groups of 8
  constexpr int kLanes = 16;                  // lanes (threads past 16 * kTpr idle)
  constexpr int kUnits = kTileRows / kLanes;  // 8 units per block
  static_assert(kLanes * kTpr <= 256, "a unit fits the work group");
  __shared__ MergeState s_state[kLanes][kTpr];
  if (!header_ok(p)) return;
  const WsHeader* hd = reinterpret_cast<const WsHeader*>(p.ws);
  const CombineItem* items = reinterpret_cast<const CombineItem*>(p.ws + hd->off_combine);
  S* obase = static_cast<S*>(p.o);
  const int n_units = hd->n_combine * kUnits;
  const bool act = threadIdx.x < kLanes * kTpr;
  const int ln = act ? threadIdx.x / kTpr : 0, dg = threadIdx.x % kTpr, d0 = dg * 8;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const CombineItem c = items[u / kUnits];
    const int k = u % kUnits;
    const int rows = c.nq * p.G;
    const bool by_split = rows <= kDecodeRows && c.nsplit > kUnits;  // uniform per unit
    const int r = by_split ? 2 * k + (ln >> 3) : kLanes * k + ln;
    const int j0 = by_split ? (ln & 7) : 0, js = by_split ? 8 : 1;
    const int rows_max = c.kind == 0 ? kTileRows : kDecodeRows;
    const float* po = reinterpret_cast<const float*>(p.ws + (c.kind == 0 ? hd->off_part_pre
                                                                        : hd->off_part_dec));
    const float* pm = reinterpret_cast<const float*>(p.ws + (c.kind == 0 ? hd->off_ml_pre
                                                                        : hd->off_ml_dec));
    MergeState st{kNegInf, 0.f, f32x4_t{}, f32x4_t{}};
    if (act && r < rows) {
#pragma unroll 8
      for (int s = j0; s < c.nsplit; s += js) {
        const int64_t slot = int64_t(c.part0 + s) * rows_max + r;
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(po + slot * D + d0);
        merge_into(st, pm[slot * 2], pm[slot * 2 + 1], src[0], src[1]);
      }
    }
    bool write = act && r < rows;
    if (by_split) {
      if (act) s_state[ln][dg] = st;
      __syncthreads();
      write = write && (ln & 7) == 0;
      if (write) {
        for (int j = 1; j < 8 && j < c.nsplit; ++j) {
          const MergeState& o = s_state[ln + j][dg];
          merge_into(st, o.m, o.l, o.a0, o.a1);
        }
      }
      __syncthreads();
    }
    if (write) {
      const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
      const f32x4_t a0 = st.a0 * inv, a1 = st.a1 * inv;
      const int tq = r / p.G, g = r - tq * p.G;
      const int64_t orow = int64_t(c.q_row0 + c.tq0 + tq) * p.Hq + int64_t(c.h) * p.G + g;
      if constexpr (sizeof(S) == 2) {
        u32x4_t v = {pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]),
                     pack_bf16x2(a1[0], a1[1]), pack_bf16x2(a1[2], a1[3])};
        *reinterpret_cast<u32x4_t*>(obase + orow * D + d0) = v;
      } else {
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(obase + orow * D + d0);
        dst[0] = a0;
        dst[1] = a1;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// Build / scatter: one launch copies every stored (token, head) row of every layer of the
// batch from the dense [layer][T][Hkv][D] K/V into its pool page. A work group copies one
// 64-token chunk of one segment. Chunks are numbered per (layer, request) group in (head,
// segment) order; the group comes from a search of the per-group chunk offsets in the kernel
// arguments, the head and segment from a wave-wide prefix sum over the group's rows of the
// (already uploaded) seg_table. A RETRIEVAL head's kept-prefix segment takes its tokens'
// positions from a list (a gather): layouts with such segments copy them in a launch of their
// own (phase 2), after the selection that writes the list, and everything else before
// (phase 1), so that the selection overlaps the bulk of the copy. Reads are whole D-rows,
// streaming (non-temporal: each byte is read once); writes are whole contiguous page rows,
// ordinary stores, which leave the caches free to gather the pages' lines before they go out.
// ---------------------------------------------------------------------------------------
template <class E, int D>
__global__ void __launch_bounds__(256) build_kernel(BuildParams p) {
  using S = typename E::S;
  constexpr int kVec = E::kVec;
  constexpr int kCols = D / kVec;
  constexpr int kLoads = kChunk * kCols / 256;
  const int c = blockIdx.x;
  const int32_t* cb = p.arr;                     // chunk offsets of the groups [n_groups + 1]
  const int32_t* row0 = p.arr + p.n_groups + 1;  // first dense row of each group [n_groups]
  const int32_t* gofs = row0 + p.n_groups;       // gather offsets [n_groups][Hkv] (retrieval)
  // group: last g with cb[g] <= c (kernel arguments, uniform)
  int lo = 0, hi = p.n_groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cb[mid] <= c) lo = mid; else hi = mid - 1;
  }
  const int g = lo, lc = c - cb[g];
  // Head and segment of the group's chunk lc: the wave takes the heads 64 at a time, lane l
  // head 64 * r + l in round r, counts their chunks (segment 0, then 1), and a prefix sum
  // over the lanes orders them.
  const int lane = __lane_id();
  const int32_t* rows = p.seg_table + int64_t(p.group0 + g) * p.Hkv * 8;
  int h = -1, s = 0, chunk = 0, base = 0;
  for (int r = 0; r < (p.Hkv + 63) / 64 && h < 0; ++r) {
    const int hh = lane + 64 * r;
    int n0 = 0, n1 = 0;
    if (hh < p.Hkv) {
      n0 = (rows[hh * 8 + 1] + kChunk - 1) / kChunk;
      n1 = (rows[hh * 8 + 5] + kChunk - 1) / kChunk;
      if (p.phase != 0) {  // segment 0 of a head with a kept prefix is its gather segment
        const bool kept = gofs[g * p.Hkv + hh] >= 0;
        if (p.phase == 1 && kept) n0 = 0;
        if (p.phase == 2) {
          n0 = kept ? n0 : 0;
          n1 = 0;
        }
      }
    }
    int incl = n0 + n1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    const int excl = base + incl - (n0 + n1);
    const uint64_t hit = __ballot(lc >= excl && lc < base + incl);
    if (hit != 0) {
      const int l = int(__builtin_ctzll(hit));
      const int e = __shfl(excl, l), m0 = __shfl(n0, l);
      h = l + 64 * r;
      s = lc - e < m0 ? 0 : 1;
      chunk = lc - e - (s ? m0 : 0);
    }
    base += __shfl(incl, 63);
  }
  h = uniform(h);
  if (h < 0) return;  // past the group's chunks (never for a launch the host sized)
  s = uniform(s);
  chunk = uniform(chunk);
  const int32_t* sr = rows + h * 8 + 4 * s;
  const int pos = uniform(sr[0]), ntok = uniform(sr[1]), vstart = uniform(sr[2]);
  const int pos_off = p.phase == 2 ? uniform(gofs[g * p.Hkv + h]) : -1;
  const int src_row0 = row0[g] + (pos_off < 0 ? pos : 0);
  const int ti0 = chunk * kChunk;
  const int lp = __builtin_ctz(unsigned(p.P));  // page size: a power of two
  const S* kd = static_cast<const S*>(p.k);
  const S* vd = static_cast<const S*>(p.v);
  S* kp = static_cast<S*>(p.kp);
  S* vp = static_cast<S*>(p.vp);
  // Every load is issued before any store, with no branch: lanes past the segment's end copy
  // the segment's last token again (the same bytes to the same slot as the lane that owns it,
  // in this work group), so all loads are unconditional and in flight at once.
  u32x4_t kr[kLoads], vr[kLoads];
  int64_t dst[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int idx = threadIdx.x + 256 * j;
    const int row = idx / kCols, col = idx % kCols;
    const int ti = min(ti0 + row, ntok - 1);
    const int tok = pos_off < 0 ? ti : p.row_pos[pos_off + ti];
    const int64_t src = (int64_t(src_row0 + tok) * p.Hkv + h) * D + col * kVec;
    kr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kd + src));
    vr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vd + src));
    const int phys = p.v2p[vstart + (ti >> lp)];
    dst[j] = ((int64_t(phys) << lp) + (ti & (p.P - 1))) * D + col * kVec;
  }
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    *reinterpret_cast<u32x4_t*>(kp + dst[j]) = kr[j];
    *reinterpret_cast<u32x4_t*>(vp + dst[j]) = vr[j];
  }
}

// ---------------------------------------------------------------------------------------
// RETRIEVAL selection (page "RedKnot head classification", the four head types: a retrieval
// head keeps only the top fraction of tokens by importance). One work group per (request,
// retrieval head) task writes the head's kept positions ascending: its sink, then the k most
// important of the other n prefix tokens, ties going to the lower position. Importance values
// map to unsigned keys in the same order; the k-th largest key T comes from a radix select
// over three digits (10, 11 and 11 bits, one histogram pass each), then one pass in position
// order takes every key above T and the first (k - count above T) keys equal to T.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_sum(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(x, d);
    if (lane >= d) x += t;
  }
  return x;
}

constexpr int kSelectThreads = 1024;

__global__ void __launch_bounds__(kSelectThreads) select_kernel(SelectParams p) {
  // Histogram words in LDS: passes of 10, 11 and 11 key bits, each histogram held in several
  // copies (lane l adds to copy l % copies) so that lanes of one wave whose keys share a bin
  // rarely hit the same word: importance values crowd into few bins of the top bits.
  constexpr int kWords = 16384;
  constexpr int kWaves = kSelectThreads / 64;
  constexpr int kBatch = 8;  // keys per thread in flight in the histogram passes
  __shared__ uint32_t hist[kWords];
  __shared__ int s_pick[2];
  __shared__ int s_wave[kWaves];
  const SelectTask t = p.t[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* out = p.row_pos + t.out;
  for (int i = tid; i < t.sink; i += kSelectThreads) out[i] = i;
  if (t.k <= 0) return;
  const float* col = p.imp + int64_t(t.h) * p.t_total + t.row0 + t.sink;  // candidate j: col[j]
  uint32_t prefix = 0, pmask = 0;
  int remaining = t.k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int bits = pass == 0 ? 10 : 11;
    const int shift = pass == 0 ? 22 : pass == 1 ? 11 : 0;
    const int nb = 1 << bits, copies = kWords >> bits;
    uint32_t* mine = hist + (lane & (copies - 1)) * nb;
    for (int i = tid; i < kWords; i += kSelectThreads) hist[i] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < t.n; j0 += kSelectThreads * kBatch) {
      uint32_t key[kBatch];
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        const int j = j0 + e * kSelectThreads + tid;
        key[e] = j < t.n ? order_key(col[j]) : 0u;
      }
#pragma unroll
      for (int e = 0; e < kBatch; ++e) {
        const int j = j0 + e * kSelectThreads + tid;
        if (j < t.n && (key[e] & pmask) == prefix)
          atomicAdd(&mine[(key[e] >> shift) & uint32_t(nb - 1)], 1u);
      }
    }
    __syncthreads();
    for (int b = tid; b < nb; b += kSelectThreads) {  // fold the copies into copy 0
      uint32_t sum = hist[b];
      for (int c = 1; c < copies; ++c) sum += hist[c * nb + b];
      hist[b] = sum;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l sums its run of bins, taken from the top: nb-1-per*l down to nb-per*(l+1)
      const int per = nb / 64;
      int sum = 0;
      for (int i = 0; i < per; ++i) sum += int(hist[nb - 1 - per * lane - i]);
      const int incl = wave_incl_sum(sum);  // keys in the top runs, through this lane's
      const uint64_t hit = __ballot(incl >= remaining && incl - sum < remaining);
      const int l = hit ? int(__builtin_ctzll(hit)) : 63;
      if (lane == l) {
        int above = incl - sum, d = nb - 1 - per * l;
        for (int i = 0; i < per - 1; ++i, --d) {
          const int c = int(hist[d]);
          if (above + c >= remaining) break;
          above += c;
        }
        s_pick[0] = d;
        s_pick[1] = remaining - above;
      }
    }
    __syncthreads();
    prefix |= uint32_t(s_pick[0]) << shift;
    pmask |= uint32_t(nb - 1) << shift;
    remaining = s_pick[1];
    __syncthreads();
  }
  // prefix = T, the k-th largest key; `remaining` keys equal to T are taken (the lowest).
  const uint32_t T = prefix;
  const int ties = remaining;
  constexpr int kPer = 8;  // consecutive candidates per thread and tile
  int gt_base = 0, eq_base = 0;
  for (int j0 = 0; j0 < t.n; j0 += kSelectThreads * kPer) {
    uint32_t gt = 0, eq = 0;  // bit e: candidate j0 + kPer * tid + e
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = j0 + kPer * tid + e;
      if (j < t.n) {
        const uint32_t key = order_key(col[j]);
        gt |= uint32_t(key > T) << e;
        eq |= uint32_t(key == T) << e;
      }
    }
    // prefix counts of (above, equal) over the threads of the tile, packed in one int (each
    // count is at most kSelectThreads * kPer < 2^16)
    const int mine = (__builtin_popcount(gt) << 16) | __builtin_popcount(eq);
    const int incl = wave_incl_sum(mine);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = incl - mine, tot = 0;
    for (int w = 0; w < kWaves; ++w) {
      const int x = s_wave[w];
      before += w < wave ? x : 0;
      tot += x;
    }
    __syncthreads();
    int g_before = gt_base + (before >> 16), e_before = eq_base + (before & 0xffff);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const bool is_gt = (gt >> e) & 1, is_eq = (eq >> e) & 1;
      if (is_gt || (is_eq && e_before < ties)) {
        const int slot = g_before + min(e_before, ties);
        out[t.sink + slot] = t.sink + j0 + kPer * tid + e;
      }
      g_before += is_gt;
      e_before += is_eq;
    }
    gt_base += tot >> 16;
    eq_base += tot & 0xffff;
  }
}

// ---------------------------------------------------------------------------------------
// Decode append: one wave per (request, KV head) writes the request's new token into the
// head's pages and updates its table row (growable layout, see include/segpaged.h). LOCAL
// heads keep their recent segment as a ring of whole pages: pages whose tokens all fell out of
// the window are dropped from its front and their physical pages rotate to its back, so the
// head's page use stays constant.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void append_error(int32_t* err, int code) {
  if (threadIdx.x == 0) atomicCAS(reinterpret_cast<int*>(err), 0, code);
}

// Rotates x[0 .. n) left by k (0 < k < n) with the 64 lanes of one wave. Up to 256 entries:
// every lane loads its four sources, the wave waits, then stores. Longer rings: three
// reversals (of [0, k), [k, n), then [0, n)); within a reversal every pair of entries belongs
// to one lane and one iteration.
__device__ void rotate_left(int32_t* x, int n, int k) {
  const int lane = threadIdx.x;
  if (n <= 256) {
    int v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = lane + 64 * c;
      int src = j + k;
      if (src >= n) src -= n;
      v[c] = j < n ? x[src] : 0;
    }
    __syncthreads();  // every load has returned before any entry is overwritten
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = lane + 64 * c;
      if (j < n) x[j] = v[c];
    }
    return;
  }
  auto reverse = [&](int a, int m) {
    for (int i = lane; i < m / 2; i += 64) {
      const int l = x[a + i], r = x[a + m - 1 - i];
      x[a + i] = r;
      x[a + m - 1 - i] = l;
    }
  };
  reverse(0, k);
  reverse(k, n - k);
  __syncthreads();
  reverse(0, n);
}

template <class E, int D>
__global__ void __launch_bounds__(64) append_kernel(AppendParams p) {
  using S = typename E::S;
  const int b = blockIdx.x / p.Hkv, h = blockIdx.x - b * p.Hkv;
  if (p.n_new != nullptr) {
    const int nn = uniform(p.n_new[b]);
    if (nn == 0) return;
    if (nn != 1) {
      append_error(p.error, SP_ERR_INVALID_ARG);
      return;
    }
  }
  int32_t* e = p.seg_table + (int64_t(b) * p.Hkv + h) * 8;
  int pos[2], ntok[2], vs[2], own[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    pos[s] = uniform(e[4 * s + 0]);
    ntok[s] = uniform(e[4 * s + 1]);
    vs[s] = uniform(e[4 * s + 2]);
    own[s] = uniform(e[4 * s + 3]);
  }
  const int kind = p.pol[h][0], sink = p.pol[h][1], window = p.pol[h][2];
  const int P = p.P;
  // Old context length: one past the newest stored token.
  int L = -1;
#pragma unroll
  for (int s = 0; s < 2; ++s)
    if (ntok[s] > 0) L = max(L, pos[s] + ntok[s]);
  if (L < 0 || ntok[0] < 0 || ntok[1] < 0) {
    append_error(p.error, SP_ERR_INVALID_ARG);
    return;
  }
  const int r0 = max(0, L + 1 - window);  // first window position of the query at L
  int ring = -1;
  int t = 0;                                // segment that takes the token
  if (kind == SP_RETRIEVAL) t = own[1] > 0;  // its query chunk; the kept prefix is fixed
  if (kind == SP_LOCAL) {
    if (sink == 0) {
      ring = 0;
    } else if (own[1] > 0) {
      ring = 1;
    } else {
      // One segment (0, L) holding sink and window: split once the window start reaches the
      // first page boundary past the sink.
      const int s_pages = (sink + P - 1) / P, s_pg = s_pages * P;
      if (r0 >= s_pg) {
        pos[1] = s_pg;
        ntok[1] = ntok[0] - s_pg;
        vs[1] = vs[0] + s_pages;
        own[1] = own[0] - s_pages;
        ntok[0] = sink;
        own[0] = s_pages;
        ring = 1;
      }
    }
  }
  int k = 0;  // ring pages dropped by this append
  if (ring >= 0) {
    const int lag = r0 - pos[ring];
    k = lag > 0 ? lag / P : 0;
    pos[ring] += k * P;
    ntok[ring] -= k * P;
  }
  if (ring >= 0) t = ring;
  const int slot_idx = ntok[t];
  const int page = slot_idx / P;
  if (own[t] < 0 || k > own[t] || vs[t] < 0 || int64_t(vs[t]) + own[t] > p.n_virt) {
    append_error(p.error, SP_ERR_INVALID_ARG);
    return;
  }
  if (page >= own[t]) {  // no owned page left for the token (appending past the reserve)
    append_error(p.error, SP_ERR_SEGMENT_FULL);
    return;
  }
  // Physical page of the new token, read before the rotation: after rotating left by k,
  // position j of the segment's page list holds what was at (j + k) mod own.
  int src = page + k;
  if (src >= own[t]) src -= own[t];
  const int phys = uniform(p.v2p[vs[t] + src]);
  if (uint32_t(phys) >= uint64_t(p.n_phys)) {
    append_error(p.error, SP_ERR_INVALID_ARG);
    return;
  }
  if (k > 0 && k < own[t]) rotate_left(p.v2p + vs[t], own[t], k);

  // The token's K and V rows: D elements each, as 4-byte words.
  constexpr int kWords = D * int(sizeof(S)) / 4;
  const int64_t row = (int64_t(b) * p.Hkv + h) * D;
  const int64_t dst = (int64_t(phys) * P + (slot_idx - page * P)) * D;
  const uint32_t* ks = reinterpret_cast<const uint32_t*>(static_cast<const S*>(p.k_new) + row);
  const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(static_cast<const S*>(p.v_new) + row);
  uint32_t* kd = reinterpret_cast<uint32_t*>(static_cast<S*>(p.kp) + dst);
  uint32_t* vd = reinterpret_cast<uint32_t*>(static_cast<S*>(p.vp) + dst);
  for (int i = threadIdx.x; i < kWords; i += 64) {
    kd[i] = ks[i];
    vd[i] = vsrc[i];
  }
  ntok[t] += 1;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      e[4 * s + 0] = pos[s];
      e[4 * s + 1] = ntok[s];
      e[4 * s + 2] = vs[s];
      e[4 * s + 3] = own[s];
    }
    p.kv_len[int64_t(b) * p.Hkv + h] = ntok[0] + ntok[1];
  }
}

template <class E, int D, int MODE>
int occ_of(bool decode) {
  int n = 0;
  hipError_t e;
  if (decode)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<E, D, MODE>, 64, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_kernel<E, D, MODE>, 256, 0);
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

template <class E, int D, int MODE>
hipError_t launch_attn_t(bool decode, int grid, const AttnParams& p, hipStream_t st) {
  if (decode)
    decode_kernel<E, D, MODE><<<grid, 64, 0, st>>>(p);
  else
    prefill_kernel<E, D, MODE><<<grid, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

#define SP_DISPATCH(DTYPE, DIM, MODE, CALL)                                  \
  do {                                                                       \
    if ((DTYPE) == SP_BF16) {                                                \
      if ((DIM) == 64) {                                                     \
        if ((MODE) == kModePaged) { CALL(BF16, 64, kModePaged); }            \
        else { CALL(BF16, 64, kModeDense); }                                 \
      } else {                                                               \
        if ((MODE) == kModePaged) { CALL(BF16, 128, kModePaged); }           \
        else { CALL(BF16, 128, kModeDense); }                                \
      }                                                                      \
    } else {                                                                 \
      if ((DIM) == 64) {                                                     \
        if ((MODE) == kModePaged) { CALL(F32, 64, kModePaged); }             \
        else { CALL(F32, 64, kModeDense); }                                  \
      } else {                                                               \
        if ((MODE) == kModePaged) { CALL(F32, 128, kModePaged); }            \
        else { CALL(F32, 128, kModeDense); }                                 \
      }                                                                      \
    }                                                                        \
  } while (0)

int attention_occupancy(int32_t dtype, int32_t D, int32_t mode, bool decode) {
  int n = 1;
#define SP_OCC(E, DD, M) n = occ_of<E, DD, M>(decode)
  SP_DISPATCH(dtype, D, mode, SP_OCC);
#undef SP_OCC
  return n;
}

hipError_t launch_attention(int32_t dtype, int32_t D, int32_t mode, bool decode, int grid,
                            const AttnParams& p, hipStream_t stream) {
  hipError_t e = hipSuccess;
#define SP_LAUNCH(E, DD, M) e = launch_attn_t<E, DD, M>(decode, grid, p, stream)
  SP_DISPATCH(dtype, D, mode, SP_LAUNCH);
#undef SP_LAUNCH
  return e;
}

hipError_t launch_combine(int32_t dtype, int32_t D, int grid, const AttnParams& p,
                          hipStream_t stream) {
  if (dtype == SP_BF16) {
    if (D == 64) combine_kernel<BF16, 64><<<grid, 256, 0, stream>>>(p);
    else combine_kernel<BF16, 128><<<grid, 256, 0, stream>>>(p);
  } else {
    if (D == 64) combine_kernel<F32, 64><<<grid, 256, 0, stream>>>(p);
    else combine_kernel<F32, 128><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_append(int32_t dtype, int32_t D, int grid, const AppendParams& p,
                         hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (dtype == SP_BF16) {
    if (D == 64) append_kernel<BF16, 64><<<grid, 64, 0, stream>>>(p);
    else append_kernel<BF16, 128><<<grid, 64, 0, stream>>>(p);
  } else {
    if (D == 64) append_kernel<F32, 64><<<grid, 64, 0, stream>>>(p);
    else append_kernel<F32, 128><<<grid, 64, 0, stream>>>(p);
  }
  return hipGetLastError();
}

// Library-owned workspace for callers that cannot allocate device memory. Each GPU the library
// runs on holds its own copy until the process ends. In host code `scratch` names a host-side
// stand-in, not the device array: its device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is handed to kernels and copies.
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;

hipError_t static_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_build(int32_t dtype, int32_t D, const BuildParams& p, int n_chunks,
                        hipStream_t stream) {
  if (n_chunks <= 0) return hipSuccess;
  if (dtype == SP_BF16) {
    if (D == 64) build_kernel<BF16, 64><<<n_chunks, 256, 0, stream>>>(p);
    else build_kernel<BF16, 128><<<n_chunks, 256, 0, stream>>>(p);
  } else {
    if (D == 64) build_kernel<F32, 64><<<n_chunks, 256, 0, stream>>>(p);
    else build_kernel<F32, 128><<<n_chunks, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  if (p.n_tasks <= 0) return hipSuccess;
  select_kernel<<<p.n_tasks, kSelectThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace sp
