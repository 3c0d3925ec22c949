// dsatopk.hip - windowed per-row top-k selection with fused RAGGED / PAGED
// emit for gfx950, and the C ABI declared in include/dsatopk.h.
//
// Operation (sglang PR #35175 digest, "Key source excerpts",
// topk_ragged_kernel and TopKProblem): row b selects the k largest scores
// in columns [row_start_b, row_start_b + seq_len_b); rows with
// seq_len_b <= k take every position without reading scores; selected
// window position j is emitted as j + out_offset_b (RAGGED) or
// page_table[b][j / page_size] * page_size + j % page_size (PAGED); slots
// past min(k, seq_len_b) hold -1. Ties: lower position first.
//
// Work decomposition, by the row's aligned span (seq_len plus the row
// start's residue mod 4) and the batch's score stride (no span exceeds it):
//   - trivial rows (seq_len <= k) write their positions and read no score;
//   - register rows: one workgroup per row loads the whole span once with
//     16-byte loads and keeps it as keys, in registers and for the last
//     slices of the longest ones in LDS (loaded there directly); every
//     later pass runs over those. 512 threads per row for small batches of
//     short strides, 256 threads up to a 16384 stride, 512 threads up to
//     40960-float spans for longer strides, and 1024-thread workgroups of
//     the long-row kernel up to 65536 (without a plan; with one, for a
//     batch of 1024 rows or more whose stride is at most 57344, every row
//     of it);
//   - long rows of batches with few of them (split rows): cut into
//     segments of 4096 or 8192 floats, each held in registers by one
//     workgroup of the register kernel; the segments merge their digit
//     histograms through an exchange area in the plan buffer;
//   - the other long rows: with a plan, read in pieces of 16384 floats by
//     a 512-thread workgroup of the register kernel; without one, streamed
//     by a 1024-thread workgroup above 65536. Both keep the pairs above a
//     running threshold in LDS (a two-pass re-read serves the rare rows
//     that defeat it).
// The pages' CUDA design (register rows up to 8192 / 16384, a streaming
// template, thread-block clusters for very long rows; PR #26788 and
// PR #36684 digests) is prior art here: the widths and the capacities are
// chosen for 64-wide waves, 160 KB of LDS and 512 VGPRs per SIMD lane.
//
// An unaligned window start is handled by reading from the 16-byte aligned
// column below it and giving the (at most 3) columns before the window the
// reserved key 0 in registers: the scores are never written (the pages'
// kernel overwrites them in place; PR #35175 digest, same excerpt).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "dsatopk.h"
#include "select_device.h"

namespace dsatopk {

constexpr int kSmallVec = 8;          // float4 per thread: 8192-float spans
constexpr int kLargeVec = 16;         // float4 per thread: 16384-float spans
constexpr int kBigBlock = 512;        // threads per big register row
constexpr int kBigVec = 16;           // float4 per thread of those: 32768-float spans
constexpr int kBigLds = 4;            // and 4 more per thread in LDS: 40960-float spans
constexpr int kBigCap = (kBigVec + kBigLds) * 4 * kBigBlock;  // 40960
constexpr int kStreamVec = 8;         // float4 per thread per streaming chunk
constexpr int kStreamCandCap = 2048;  // streaming path: threshold-bin pairs in LDS
constexpr int kPtCap = 512;           // page-table entries staged in LDS
// 1024-thread rows stage more (their LDS has room): one entry per thread,
// the table of a register row of 65536 floats at a page size of 64 (a
// second entry per thread took a VGPR that the long rows' registers need:
// one spilled register, reloaded in every row's cut)
template <int BS>
constexpr int pt_cap() {
  return BS >= 1024 ? 1024 : kPtCap;
}

struct Params {
  const float* scores;
  int64_t stride;
  const int32_t* seq_lens;
  const int32_t* row_starts;   // may be null
  const int32_t* out_offsets;  // RAGGED
  const int32_t* page_table;   // PAGED
  int64_t pt_stride;
  int32_t page_bits;
  int32_t num_rows;
  int32_t k;
  int32_t* out;
  int32_t* plan;  // plan words (header, class lists, classes, exchange areas) or null
  // PAGED only: row b maps window position j through page-table row
  // table_rows[b] (b if null) at table position table_starts[b] + j (j if
  // null), and also writes j to out_raw (if not null), slot for slot
  const int32_t* table_rows;
  const int32_t* table_starts;
  int32_t* out_raw;
  // register kernel: its first `workers` workgroups serve split segments
  // (claimed from the plan), the others one row each
  int32_t workers;
  // who reads the long rows that are not split (see LongMode)
  int32_t long_mode;
  // register kernel with a plan: row workgroup g serves the plan's
  // class-list entry num_rows - 1 - g (the longest classes first)
  int32_t ordered;
};

// The long rows that are not split: with no plan, the long-row kernel
// (one 1024-thread workgroup per row of the batch); with a plan, the
// register kernel, in pieces (three rows per CU), and the long-row kernel
// is not launched. kLongAll: a large batch whose stride keeps every row in
// 1024 threads' registers and is at most kLongAllStride (see launch_rows):
// the long-row kernel alone serves every row, one workgroup per row, and
// no row is split.
enum LongMode : int32_t { kLongPerRow = 0, kLongInPieces = 1, kLongAll = 2 };

// Row classes by aligned span. A row's class is recomputed by every kernel
// from the current seq_lens / row_starts; the plan only packs the rows of a
// class into the first workgroups of that class's launch.
enum RowClass : int32_t { kClassShort = 0, kClassMid = 1, kClassBig = 2, kClassLong = 3 };
constexpr int kNumClasses = 4;

// Plan layout (int32 words): a 64-word header; the rows of each class
// (class order); each row's class, segment count and exchange slot; the
// (row, segment) work items of split rows; one exchange area per split
// row.
constexpr int kPlanMagic = 0x44534b33;  // "DSK3"
constexpr int kPlanHeaderWords = 64;
enum PlanWord : int32_t {
  kPlanWordMagic = 0,
  kPlanWordRows = 1,
  kPlanWordK = 2,
  kPlanWordCount = 4,        // [4] rows per class
  kPlanWordOffset = 8,       // [4] first list index per class
  kPlanWordSplit = 12,       // long rows cut into segments (each owns an exchange area)
  kPlanWordItems = 13,       // (row, segment) work items of those rows
  kPlanWordError = 14,       // set when a split segment gave up waiting for its row
  kPlanWordSpin = 15,        // polls before such a wait gives up (0: kSpinLimit)
  kPlanWordSegLen = 16,      // floats per segment of the split rows
};

// Long rows are cut into segments of 4096 or 8192 aligned floats, one
// workgroup each, holding its segment in registers like a short row. The
// segments of a row merge their digit histograms through the row's exchange
// area in the plan buffer (this replaces the pages' thread-block cluster
// path: CDNA has no clusters or distributed shared memory). Segments are
// 8192 floats unless the batch's long rows would then give fewer segments
// than the chip has CUs.
constexpr int kSegShort = 4096;
constexpr int kSegLong = 8192;
constexpr int kChipCUs = 256;
constexpr int kMaxSeg = (DSATOPK_MAX_SEQ_LEN + 3 + kSegShort - 1) / kSegShort;  // 33
// A batch's long rows are split only if there are at most this many (about
// one per CU): each then gets the whole GPU's help. With more, one
// workgroup per long row already fills the GPU and does less work per
// element than the split rows' merge rounds.
constexpr int kMaxSplitRows = 256;
// Split workers per launch: at most the register kernel's three
// workgroups per CU, so that the workers, the first workgroups of the grid,
// are resident together (see SplitSync).
constexpr int kMaxWorkers = 3 * kChipCUs;
constexpr uint32_t kSpinLimit = 1u << 20;  // about a second of polling

// Exchange area of one split row (int32 words). The histogram and the
// counters are zero at the start of a call: the plan zeroes them, every
// round's last arriver re-zeroes the bins it read, and the row's last
// segment to finish resets the counters.
constexpr int kCandCapG = 2048;  // threshold-bin elements resolved by the last segment
// Each counter has a 128-byte line of its own: the device-scope atomics on
// one address are serialized (about 12 ns each on MI355X), and the polls of
// the round word should not queue behind the arrivals.
enum XWord : int32_t {
  kXHist = 0,       // 4096 bins: the current digit round's merged histogram
  kXCand = 4096,     // kCandCapG (key, position) pairs of the level-1 bin
  kXVal = 8192,      // their emitted values (page-mapped or offset), pair for pair
  kXFlag = 10240,    // 64-bit: last published round and its result
  kXArrive = 10272,  // segments arrived (all rounds)
  kXOut = 10336,     // 64-bit: output slots taken (low), candidate pairs written (high)
  kXDone = 10368,    // segments finished
  kXFail = 10400,    // a segment of the row gave up waiting
  kXWords = 10432,   // multiple of 64 words (256 bytes)
};

__host__ __device__ constexpr int64_t plan_split_cap(int64_t rows) {
  return rows < kMaxSplitRows ? rows : kMaxSplitRows;
}
__host__ __device__ constexpr int64_t plan_cls_word(int64_t rows) { return kPlanHeaderWords + rows; }
__host__ __device__ constexpr int64_t plan_nseg_word(int64_t rows) { return kPlanHeaderWords + 2 * rows; }
__host__ __device__ constexpr int64_t plan_slot_word(int64_t rows) { return kPlanHeaderWords + 3 * rows; }
__host__ __device__ constexpr int64_t plan_items_word(int64_t rows) { return kPlanHeaderWords + 4 * rows; }
__host__ __device__ constexpr int64_t plan_xarea_word(int64_t rows) {
  return (plan_items_word(rows) + 2 * plan_split_cap(rows) * kMaxSeg + 63) / 64 * 64;
}
__host__ __device__ constexpr int64_t plan_words(int64_t rows) {
  return plan_xarea_word(rows) + plan_split_cap(rows) * kXWords;
}
__host__ __device__ constexpr int32_t segments_for(int32_t span, int32_t seg_len) {
  return (span + seg_len - 1) / seg_len;
}

// Output of one row: window position j -> emitted value. In PAGED mode the
// row's page-table entries may be staged in LDS first (short windows).
template <bool kPaged>
struct Emit {
  int32_t* out;
  int32_t* out_raw;   // PAGED: also the window positions, slot for slot (or null)
  const int32_t* pt;  // the row's page-table row (global)
  int32_t pt_off;     // table position of window position 0 (packed rows)
  int32_t pt_first;   // first entry of the LDS copy, when staged
  int32_t page_bits;
  int32_t offset;
  bool staged;        // entries pt_first .. sit in the workgroup's LDS table

  __device__ __forceinline__ int32_t map(int32_t q, int32_t page) const {
    return (int32_t)(((uint32_t)page << page_bits) | ((uint32_t)q & ((1u << page_bits) - 1u)));
  }

  // The emitted value of window position j, with the page-table entry read
  // from global memory.
  __device__ __forceinline__ int32_t value(int32_t j) const {
    if constexpr (kPaged) {
      const int32_t q = j + pt_off;
      return map(q, pt[q >> page_bits]);
    } else {
      return j + offset;
    }
  }

  // Same, with the entry read from the staged LDS copy `lds`.
  __device__ __forceinline__ int32_t value_lds(int32_t j, const int32_t* lds) const {
    if constexpr (kPaged) {
      // an LDS pointer by type, so that the read is an LDS read even where
      // the compiler merges this path with the global one
      // entry q >> page_bits sits at lds[(q >> page_bits) - pt_first]: its
      // LDS byte address is one shift-add onto a scalar base
      using lds_i32 = const __attribute__((address_space(3))) int32_t;
      const uint32_t base =
          (uint32_t)(uintptr_t)(lds_i32*)lds - (uint32_t)pt_first * 4u;
      const uint32_t q = (uint32_t)(j + pt_off);
      lds_i32* e = (lds_i32*)(uintptr_t)(((q >> page_bits) << 2) + base);
      return map((int32_t)q, *e);
    } else {
      return j + offset;
    }
  }

  // Output slot t takes value v of window position j (j = -1: padding).
  __device__ __forceinline__ void put(int32_t t, int32_t j, int32_t v) const {
    out[t] = v;
    if (kPaged && out_raw) out_raw[t] = j;
  }

  // Page-table entries of window positions [0, L): first entry, count.
  __device__ __forceinline__ int2 table_span(int32_t L) const {
    const int32_t e0 = pt_off >> page_bits;
    return make_int2(e0, L > 0 ? ((pt_off + L - 1) >> page_bits) - e0 + 1 : 0);
  }

  // Stage the first ceil(L / page_size) table entries into `lds` when they
  // fit; issued early so the loads overlap the score loads.
  __device__ __forceinline__ void stage_table(int32_t* lds, int32_t L) {
    stage_table_range(lds, 0, L);
  }

  // Same for the entries of window positions [j0, j1) only (clamped to the
  // window [0, L)).
  __device__ __forceinline__ void stage_table_range(int32_t* lds, int32_t j0, int32_t j1) {
    if constexpr (kPaged) {
      j0 = j0 < 0 ? 0 : j0;
      if (j1 <= j0) return;
      const int32_t e0 = (j0 + pt_off) >> page_bits;
      const int32_t n = ((j1 - 1 + pt_off) >> page_bits) - e0 + 1;
      if (n <= kPtCap) {
        for (int32_t e = tix(); e < n; e += (int32_t)blockDim.x) lds[e] = pt[e0 + e];
        staged = true;
        pt_first = e0;
      }
    }
  }
};

// Shared memory of the register path.
constexpr int kWideBlock = 512;  // threads per row when rows are too few to fill the chip
static_assert(kMaxK + kBlock <= kBins, "a split segment's output stage and its dummies fit the histogram");

// NB: bins of the first key digit (4096, or 16384 for the rows of the
// latency-bound wide kernel, whose first digit then takes 14 key bits).
template <int BS, int NB = kBins>
struct SmemRegB {
  uint32_t hist[NB];           // every histogram of the row's digits; finally the output stage
  int32_t pt[pt_cap<BS>()];    // the row's page-table entries (PAGED)
  uint32_t wave_cnt[BS / 64];  // per wave: selected elements
  uint32_t bcast[4];           // a bin search's result, when one wave searches
  // per-lane and per-wave running sums of a search shared by all waves
  // (register-row layouts of 256 threads and more)
  uint32_t lsum[BS >= kBlock ? BS : 1];
  uint32_t wsum[BS / 64];
  uint32_t tie_n;  // slots taken by a small tie class's positions
};
using SmemReg = SmemRegB<kBlock>;

// A split segment's workgroup (the register kernel's 512 threads) also
// keeps an 8-bit digit histogram, the positions of a small tie class and
// the words of its row's rounds and of its claims.
template <int BS>
struct SmemSplitB : SmemRegB<BS> {
  uint32_t h2[256];
  uint32_t tie[64];
  uint32_t word[8];
};

// Shared memory of the streaming path.
struct SmemStream {
  uint32_t hist[kBins];
  int32_t stage[kMaxK];
  uint2 cand[kStreamCandCap];
  uint32_t nstage;
  uint32_t ncand;
};

// The long-row kernel: 1024 threads per row.
constexpr int kLongBlock = 1024;

// Shared memory of the single-pass streaming path: the candidate list and
// one digit histogram. A chunk is one float4 per thread (4096 elements),
// kS1Depth chunks are in flight (64 KiB). Two workgroups fit a CU; after a
// compaction about 2000 pairs of room stay above k + one chunk, so on rows
// in random order the list is compacted a handful of times per row.
constexpr int kS1Chunk = 4 * kLongBlock;

// The opening chunks of the streamed row that is likely to start next on
// this workgroup's XCD: two streaming workgroups per CU on a 256-CU part
// run rows b .. b + 511 at once, and workgroups start in row order, so row
// b + 512 follows about when row b ends (its XCD is row b's: workgroups go
// to the XCDs round-robin). A streamed row touches one word per 64-byte
// line of that row's first 16384 columns during its own final cut, with
// the default cache policy, so the next row's first loads find them in the
// caches instead of waiting a full HBM round trip under load. A guess only
// about timing: every row is still read by its own workgroup.
constexpr int kPrefetchAhead = 512;
struct Prefetch {
  const float* base;  // first aligned column of the row's window, or null
  int32_t bytes;      // bytes to touch from base
};
constexpr int kS1Depth = 4;
constexpr int kS1Sample = 2;  // chunks whose histogram sets the list's opening threshold
constexpr int kS1Cap = 8160;

// The list's length lives in registers, never in one shared counter that
// a fast wave could bump for the next chunk before a slow wave has read it
// for this one. Chunk c takes slots from ccnt[c % 4], which holds only that
// chunk's appends: after the chunk's barrier every wave adds it to its
// length, and thread 0 zeroes the counter of chunk c - 2 (read by everyone
// before the barrier of chunk c - 1, next used by chunk c + 2 after the
// barrier of chunk c + 1). A compaction ranks its kept pairs by per-wave
// counts in wave_cnt; the warm start, which appends once between barriers,
// counts in n0. After the last chunk the final cut reads the list in place.
template <int BS, int CAP>
struct SmemListB {
  static constexpr int kCap = CAP;
  uint2 cand[CAP];
  uint32_t hist[kBins];                 // digit histograms; finally the output stage
  uint32_t wave_cnt[BS / 64];           // per-wave counts (compaction, stage)
  uint32_t ccnt[4];
  uint32_t n0;
  uint32_t tie_n;
  uint32_t bcast[4];
};
using SmemS1 = SmemListB<kLongBlock, kS1Cap>;

// Window of one row, addressed from the 16-byte aligned column at or below
// row_start: aligned index a holds window position a - rem, and only
// rem <= a < span are in the window.
struct RowView {
  const float4* base4;
  int32_t rem;
  int32_t span;
};

__device__ __forceinline__ uint32_t key_at(float x, int32_t a, const RowView& rv) {
  return ((a >= rv.rem) & (a < rv.span)) ? order_key(x) : 0u;
}

__device__ __forceinline__ float lane_of(const float4& v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// Register-resident elements of one workgroup: element (i, c) of thread t is
// aligned index (i * kBlock + t) * 4 + c.
template <int NV, int BS = kBlock>
struct RegSrc {
  static constexpr int kPerThread = 4 * NV;  // elements per thread
  const uint32_t (&key)[NV][4];
  int32_t origin;  // window position of register element (0, 0) of thread 0
  int32_t ilast;   // last register slice that holds columns (workgroup-uniform)

  // Positions are rebuilt from one opaque base in every pass: the compiler
  // cannot keep NV * 4 position registers alive across passes.
  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    int32_t base = tix() * 4 + origin;
    asm volatile("" : "+v"(base));
    // the slice bound as an opaque scalar: every slice test is one scalar
    // compare, not a lane mask rebuilt in VGPRs for each pass
    int32_t il = ilast;
    asm volatile("" : "+s"(il));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i <= il) {
#pragma unroll
        for (int c = 0; c < 4; ++c) f(key[i][c], base + i * BS * 4 + c);
      }
      // keep the scheduler from hoisting every slot's compare masks (one
      // SGPR pair each) to the top of the pass
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// (key, position) pairs in LDS, enumerated to one wave.
struct WaveCandSrc {
  const uint2* cand;
  uint32_t n;

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    for (uint32_t i = lane_id(); i < n; i += 64) {
      const uint2 e = cand[i];
      f(e.x, (int32_t)e.y);
    }
  }
};

// The row re-read from global memory in chunks of kStreamVec float4 per
// thread. Every thread calls f the same number of times.
template <int BS>
struct StreamSrc {
  RowView rv;

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int32_t nvec = (rv.span + 3) >> 2;
    for (int32_t v0 = 0; v0 < nvec; v0 += BS * kStreamVec) {
      float4 x[kStreamVec];
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u) {
        const int32_t v = v0 + u * BS + tix();
        x[u] = v < nvec ? rv.base4[v] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u) {
        const int32_t a0 = (v0 + u * BS + tix()) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) f(key_at(lane_of(x[u], c), a0 + c, rv), a0 + c - rv.rem);
      }
    }
  }
};

// Candidate (key, position) pairs held in registers, NP per thread.
template <int NP>
struct CandRegSrc {
  const uint32_t (&key)[NP];
  const int32_t (&pos)[NP];

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
#pragma unroll
    for (int j = 0; j < NP; ++j) f(key[j], pos[j]);
  }
};

// The (key, position) pairs of a streamed row's LDS list, as they stand:
// thread t takes entries t, t + BS, ... . With `offsets` the key is the
// pair's offset above T, min(key - T, 2^24 - 2) + 1, moved to bits 31..8:
// the pairs just above T spread over the digits, and every offset that
// reaches the bound compares above all the others.
template <int BS>
struct ListSrc {
  const uint2* cand;
  uint32_t n;
  uint32_t T;
  bool offsets;

  static constexpr uint32_t kSat = (1u << 24) - 2u;

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    for (uint32_t i = (uint32_t)tix(); i < n; i += BS) {
      const uint2 e = cand[i];
      uint32_t key = e.x;
      if (offsets) {
        const uint32_t r = key - T;
        key = ((r < kSat ? r : kSat) + 1u) << 8;
      }
      f(key, (int32_t)e.y);
    }
  }
};

// A raw buffer over the n int32 words at p. Stores through it take their
// address from one VGPR offset (plus the instruction's immediate offset),
// and the hardware drops a store whose offset is at or past n words, so the
// slots past k need no lane compare.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t words_buffer(int32_t* p, int32_t n) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(n * 4),
                                           0x00020000);
}

// Cache policy of the output stores: non-temporal, like the score loads
// (the outputs are not read back by this library). On MI355X this takes
// 2-4% off the short, big-register and streaming kernels' launches; the
// mid kernel's 16 float4 x 256-thread rows ran 5% slower with it, so that
// configuration stores with the default policy.
constexpr int kStreamingStore = 2;
constexpr int kDefaultStore = 0;

// Slot i * BS + t of a row's output (t = this thread's index): the slot's
// byte offset is in the VGPR offset, where the range check sees it.
template <int BS, int kPolicy = kStreamingStore>
__device__ __forceinline__ void store_slot(__amdgpu_buffer_rsrc_t r, int32_t t, int i, int32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (t + i * BS) * 4, 0, kPolicy);
}

template <bool kPaged, int BS = kBlock>
__device__ __forceinline__ void write_trivial(const Emit<kPaged>& em, int32_t L, int32_t k) {
  // all table loads before any store: one memory round trip, not one per
  // slot. Every slot loads (a slot past the window looks up the window's
  // last position, which is in bounds, and its value is replaced), so no
  // load sits behind a branch and its own wait.
  constexpr int kIter = kMaxK / BS;
  const int32_t t = tix();
  int32_t v[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) v[i] = -1;
  if (L > 0) {
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      const int32_t s = i * BS + t;
      v[i] = em.value(s < L ? s : L - 1);
    }
  }
  const __amdgpu_buffer_rsrc_t ro = words_buffer(em.out, k);
#pragma unroll
  for (int i = 0; i < kIter; ++i) store_slot<BS>(ro, t, i, i * BS + t < L ? v[i] : -1);
  if (kPaged && em.out_raw) {
    const __amdgpu_buffer_rsrc_t rr = words_buffer(em.out_raw, k);
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      const int32_t s = i * BS + t;
      store_slot<BS>(rr, t, i, s < L ? s : -1);
    }
  }
}

// Final coalesced store of the k staged positions. A position outside
// [0, L) cannot come out of a correct cut; it is written as -1 rather than
// used to index the page table.
// Fully unrolled (k <= kMaxK) in three straight-line phases: every stage
// read (the stage holds at least kMaxK words, so slots past k are read but
// not used), then every page-table lookup, then the stores. All reads of a
// phase are in flight together, not one dependent pair per slot.
template <bool kPaged, int BS, int kPolicy, class V>
__device__ __forceinline__ void write_stage_with(const Emit<kPaged>& em, const int32_t* stage,
                                                 int32_t L, int32_t k, V value) {
  static_assert(kMaxK % BS == 0, "whole iterations");
  constexpr int kIter = kMaxK / BS;
  // one thread index for every phase: the stage reads and the stores take
  // their slot from an immediate offset
  const int32_t t = tix();
  int32_t j[kIter];
  int32_t v[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) j[i] = stage[i * BS + t];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const bool ok = (uint32_t)j[i] < (uint32_t)L;  // a valid window position
    const int32_t vv = value(ok ? j[i] : 0);
    j[i] = ok ? j[i] : -1;
    v[i] = ok ? vv : -1;
  }
  const __amdgpu_buffer_rsrc_t ro = words_buffer(em.out, k);
#pragma unroll
  for (int i = 0; i < kIter; ++i) store_slot<BS, kPolicy>(ro, t, i, v[i]);
  if (kPaged && em.out_raw) {
    const __amdgpu_buffer_rsrc_t rr = words_buffer(em.out_raw, k);
#pragma unroll
    for (int i = 0; i < kIter; ++i) store_slot<BS, kPolicy>(rr, t, i, j[i]);
  }
}

// The k staged positions, mapped, to the row's output. `lds_table` is the
// workgroup's LDS copy of the page table, used when the emit staged it.
template <bool kPaged, int BS = kBlock, int kPolicy = kStreamingStore>
__device__ __forceinline__ void write_stage(const Emit<kPaged>& em, const int32_t* stage,
                                            int32_t L, int32_t k, const int32_t* lds_table) {
  if (kPaged && em.staged)
    write_stage_with<kPaged, BS, kPolicy>(em, stage, L, k,
                                          [&](int32_t j) { return em.value_lds(j, lds_table); });
  else
    write_stage_with<kPaged, BS, kPolicy>(em, stage, L, k,
                                          [&](int32_t j) { return em.value(j); });
}

// A bin search whose result every thread needs: wave 0 searches and the
// result goes through LDS (one barrier). Used where a layout holds no
// all-wave running sums (the streaming list's compactions, small digits).
template <int NB, bool kDesc, class Sm>
__device__ __forceinline__ BinHit wave0_find(const uint32_t* hist, uint32_t need, Sm& sm) {
  if (wave_id() == 0) {
    const BinHit h = wave_find<NB, kDesc>(hist, need);
    if (lane_id() == 0) {
      sm.bcast[0] = h.bin;
      sm.bcast[1] = h.before;
      sm.bcast[2] = h.cnt;
    }
  }
  __syncthreads();
  return BinHit{(uint32_t)__builtin_amdgcn_readfirstlane(sm.bcast[0]),
                (uint32_t)__builtin_amdgcn_readfirstlane(sm.bcast[1]),
                (uint32_t)__builtin_amdgcn_readfirstlane(sm.bcast[2])};
}

// The same search by all W = BS / 64 waves of a workgroup that runs alone
// on its CU (a latency-bound launch): lane u = 64 w + l sums the run of
// PER = NB / BS bins at scan positions [u PER, (u + 1) PER); the per-lane
// running sums of each wave and the wave totals go through LDS; after one
// barrier every wave finds the crossing wave, then lane, then bin by
// itself. Its second-level reads of the histogram need a closing barrier
// before anyone may write it again.
template <int NB, bool kDesc, int BS, class Sm>
__device__ __forceinline__ BinHit all_waves_find(const uint32_t* hist, uint32_t need, Sm& sm) {
  constexpr int W = BS / 64;
  constexpr int PER = NB / BS;
  static_assert(PER >= 4 && PER % 4 == 0 && PER <= 64 && W <= 64, "one 16-byte read per run step");
  const int lane = lane_id();
  const int w = wave_id();
  const int u = w * 64 + lane;
  auto bin_of = [](int r) { return kDesc ? NB - 1 - r : r; };  // scan position -> bin
  uint32_t sum = 0;
  {
    // Runs of 32 bins and more are 128 bytes apart or more: read in step,
    // every lane's chunk would sit on the same LDS banks, so each lane
    // starts at another 16-byte chunk of its run (the sum does not care
    // about the order). Shorter runs read in step: there the rotation's
    // address arithmetic cost more than the conflicts (mid-kernel rows
    // 4.5% slower with it).
    constexpr int CH = PER / 4;
    const int lo = kDesc ? NB - (u + 1) * PER : u * PER;
    const uint4* h4 = reinterpret_cast<const uint4*>(hist + lo);
    const int rot = CH >= 8 ? (lane & (CH - 1)) : 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const uint4 q = h4[CH >= 8 ? ((i + rot) & (CH - 1)) : i];
      sum += q.x + q.y + q.z + q.w;
    }
  }
  const uint32_t incl = wave_inclusive_sum(sum);
  sm.lsum[u] = incl;
  if (lane == 63) sm.wsum[w] = incl;
  __syncthreads();
  const uint32_t tw = lane < W ? sm.wsum[lane] : 0u;
  const uint32_t iw = wave_inclusive_sum(tw);
  const uint64_t mw = __ballot(iw >= need);
  const int wc = mw ? __builtin_ctzll(mw) : W - 1;
  const uint32_t basew = read_lane(iw - tw, wc);
  const uint32_t il = basew + sm.lsum[wc * 64 + lane];
  const uint64_t ml = __ballot(il >= need);
  const int l1 = ml ? __builtin_ctzll(ml) : 63;
  const uint32_t before1 = l1 ? read_lane(il, l1 - 1) : basew;
  const int r0 = (wc * 64 + l1) * PER;
  const uint32_t v = lane < PER ? hist[bin_of(r0 + lane)] : 0u;
  const uint32_t incl2 = before1 + wave_inclusive_sum(v);
  const uint64_t m2 = __ballot((lane < PER) & (incl2 >= need));
  const int l2 = m2 ? __builtin_ctzll(m2) : 0;
  BinHit h;
  h.bin = (uint32_t)bin_of(r0 + l2);
  h.cnt = read_lane(v, l2);
  h.before = read_lane(incl2, l2) - h.cnt;
  __syncthreads();
  return h;
}

// Whether a shared-memory layout holds the running sums of an all-wave
// search (the register-row layouts do). Register rows search their
// 4096-bin digits with every wave: the rows are latency-bound, not
// VALU-bound, and the search by wave 0 alone kept a 256-thread row's cut
// at 38 % of its workgroup's life (8192-float rows: 232 -> 216 us per
// 32768-row launch; 16384-float rows: 211 -> 201 us, at one workgroup
// per CU fewer for the VGPRs the search adds).
template <class Sm>
struct HasWaveSums {
  static constexpr bool value = false;
};
template <int BS, int NB>
struct HasWaveSums<SmemRegB<BS, NB>> {
  static constexpr bool value = BS >= kBlock;
};
template <int BS>
struct HasWaveSums<SmemSplitB<BS>> {
  static constexpr bool value = BS >= kBlock;
};

template <int NB, bool kDesc, int BS, class Sm>
__device__ __forceinline__ BinHit group_find(const uint32_t* hist, uint32_t need, Sm& sm) {
  if constexpr (BS >= kBlock && NB >= 4 * BS && HasWaveSums<Sm>::value)
    return all_waves_find<NB, kDesc, BS, Sm>(hist, need, sm);
  else
    return wave0_find<NB, kDesc>(hist, need, sm);
}

// The need-th lowest window position among the elements whose key is tau
// (not 0: window elements only, so positions are >= 0 and below 2^17),
// when cnt <= 64 hold it. Their positions go to LDS, one atomic slot each;
// then every wave picks the need-th lowest by itself, one position bit at
// a time from the top, on lane masks (positions are distinct). The caller
// has zeroed sm.tie_n behind at least one barrier, and the histogram is
// free. The positions are read before the caller's next barrier, so the
// histogram may be written after it.
template <class Src, class Sm>
__device__ __forceinline__ int32_t small_tie_pos(const Src& src, Sm& sm, uint32_t tau,
                                                 uint32_t cnt, uint32_t need) {
  uint32_t* tie = sm.hist;
  src.for_each([&](uint32_t kk, int32_t j) {
    if (kk == tau) {
      const uint32_t slot = atomicAdd(&sm.tie_n, 1u);
      if (slot < 64u) tie[slot] = (uint32_t)j;
    }
  });
  __syncthreads();
  const int lane = lane_id();
  const uint32_t p = lane < (int)cnt ? tie[lane] : 0u;
  uint64_t live = cnt >= 64u ? ~0ull : (1ull << cnt) - 1ull;
#pragma unroll
  for (int b = 16; b >= 0; --b) {
    const uint64_t zeros = __ballot(((p >> b) & 1u) == 0u) & live;
    const uint32_t c0 = (uint32_t)__builtin_popcountll(zeros);
    if (need <= c0) {
      live = zeros;
    } else {
      need -= c0;
      live &= ~zeros;
    }
  }
  return (int32_t)read_lane(p, live ? __builtin_ctzll(live) : 0);
}

// Whether a register source holds many elements per thread (above 32): the
// level-1 threshold bin then holds a small share of a long row (about 1%
// at 65536 floats and k = 2048), and most 64-lane groups of a pass hold
// none of it. Measured: 1-1.5% faster at 32768..65536 floats, 2.5% slower
// at 32 per thread (8192 floats), where most groups hold one.
template <class Src, class = void>
struct SparseBin {
  static constexpr bool value = false;
};
template <class Src>
struct SparseBin<Src, decltype(void(Src::kPerThread))> {
  static constexpr bool value = Src::kPerThread > 32;
};

// The cut of a register-resident row. Level 1 (key bits 31..20) was
// histogrammed into sm.hist by the caller. Level 2 takes the next 12 bits
// (19..8) in the same array, cleared once its level-1 search is done;
// level 3 the last 8 bits, unless the caller knows them to be zero in every
// key (low8_zero). Each level costs one filtered pass over the registers
// and a search. Ties at the k-th key: a class of at most 64 elements is
// ranked by position in one pass; a larger one takes two position digits.
// refine_from_level1 takes the level-1 search's result h (need = k minus
// h.before elements still to take from bin h.bin), with sm.tie_n zeroed
// behind that search's barrier.
template <int BS, class Src, class Sm>
__device__ __forceinline__ Cut refine_from_level1(const Src& src, Sm& sm, BinHit h, uint32_t need,
                                                  bool low8_zero = false) {
  uint32_t prefix = h.bin;  // key bits 31..20
  if (h.cnt == need) return Cut{20, prefix, kAllPos};
  // every wave is past the search's barrier: the level-1 counts are dead
  clear_bins<kBins, BS>(sm.hist);
  __syncthreads();
  {
    const uint32_t p = prefix;
    const uint32_t one = opaque_one();
    src.for_each([&](uint32_t kk, int32_t) {
      const bool in = (kk >> 20) == p;
      if constexpr (SparseBin<Src>::value) {
        // a wave with no element of the bin here branches past the add's
        // address arithmetic (the empty asm keeps this wave-uniform test a
        // branch of its own)
        if (__builtin_amdgcn_ballot_w64(in) != 0u) {
          asm volatile("");
          if (in) lds_add(&sm.hist[(kk >> 8) & 0xfffu], one);
        }
      } else if (in) {
        lds_add(&sm.hist[(kk >> 8) & 0xfffu], one);
      }
    });
  }
  __syncthreads();
  h = group_find<kBins, true, BS>(sm.hist, need, sm);
  need -= h.before;
  prefix = (prefix << 12) | h.bin;  // bits 31..8
  if (h.cnt == need) return Cut{8, prefix, kAllPos};
  uint32_t tau = prefix << 8;  // every key of the bin, when bits 7..0 are zero
  if (!low8_zero) {
    clear_bins<256, BS>(sm.hist);
    __syncthreads();
    {
      const uint32_t p = prefix;
      const uint32_t one = opaque_one();
      src.for_each([&](uint32_t kk, int32_t) {
        if ((kk >> 8) == p) lds_add(&sm.hist[kk & 0xffu], one);
      });
    }
    __syncthreads();
    h = group_find<256, true, BS>(sm.hist, need, sm);
    need -= h.before;
    tau |= h.bin;
    if (h.cnt == need) return Cut{0, tau, kAllPos};
  }
  if (h.cnt <= 64u && tau != 0u) return Cut{0, tau, small_tie_pos(src, sm, tau, h.cnt, need)};

  // Several elements hold exactly the key tau and only `need` of them are
  // taken: the lowest positions. Window positions are < 2^17: two ascending
  // digits (bits 16..5, then 4..0) find the need-th lowest. Columns before
  // the window have negative positions and key 0; they are left out so that
  // every bin index stays inside the histogram.
  clear_bins<kBins, BS>(sm.hist);
  __syncthreads();
  src.for_each([&](uint32_t kk, int32_t j) {
    if ((kk == tau) & (j >= 0)) lds_inc(&sm.hist[(uint32_t)j >> 5]);
  });
  __syncthreads();
  h = group_find<kBins, false, BS>(sm.hist, need, sm);
  need -= h.before;
  const uint32_t hi = h.bin;
  clear_bins<32, BS>(sm.hist);
  __syncthreads();
  src.for_each([&](uint32_t kk, int32_t j) {
    if ((kk == tau) & (j >= 0) & (((uint32_t)j >> 5) == hi)) lds_inc(&sm.hist[(uint32_t)j & 31u]);
  });
  __syncthreads();
  h = group_find<32, false, BS>(sm.hist, need, sm);
  return Cut{0, tau, (int32_t)((hi << 5) | h.bin)};
}

template <int BS, class Src, class Sm>
__device__ __forceinline__ Cut refine_in_registers(const Src& src, Sm& sm, uint32_t k,
                                                   bool low8_zero = false) {
  if (tix() == 0) sm.tie_n = 0u;  // the first search's barrier publishes it
  const BinHit h = group_find<kBins, true, BS>(sm.hist, k, sm);
  return refine_from_level1<BS>(src, sm, h, k - h.before, low8_zero);
}

// Whole span in registers (span <= NV * 4 * BS).
//
// Every pass over the registers is budgeted in VALU operations per score:
// at 8 TB/s a CU sees about 3.3 scores per clock against 64 lane-ops per
// clock, i.e. about 19 operations per score for everything. The passes are
// key (4 ops), level-1 histogram (2 ops + 1 LDS atomic), one filtered pass
// per further digit (2 ops; the rare matches add an LDS atomic), the
// output count (2) and the staging of the selection (3).
//
// Every wave finds each threshold bin itself (no broadcast barrier). The
// emit order is (wave, lane, register slot): a fixed function of the input.
// The k selected positions are staged in LDS and mapped and stored in one
// coalesced pass.
// Cache policy of the score loads: non-temporal. Scores are read once;
// streaming them past the caches leaves L2 and the Infinity Cache to the
// output writes, which raises the combined read+write rate of a launch by
// about a fifth on MI355X.
constexpr int kStreamingLoad = 2;

// A raw buffer over the row's nvec aligned vectors: the hardware returns
// zeros for vectors past the end instead of reading them, so no load needs a
// compare. Every load puts its whole offset (thread and slice) in the VGPR
// offset, which the range check covers; the scalar offset is left at 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buffer(const float4* base4, int32_t nvec) {
  const uint64_t a = reinterpret_cast<uint64_t>(base4);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  // dword 3: 32-bit data format, the setting of untyped loads on gfx9-class GPUs
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0,
                                           __builtin_amdgcn_readfirstlane(nvec * 16), 0x00020000);
}

// Vector v0 + i * BS + t of the row into x[i] (zeros past the row's last vector).
template <int NV, int BS>
__device__ __forceinline__ void load_vectors(const float4* base4, int32_t nvec, int32_t v0,
                                             float4 (&x)[NV]) {
  const __amdgpu_buffer_rsrc_t r = row_buffer(base4, nvec);
  const int32_t off = (v0 + tix()) * 16;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    x[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off + i * BS * 16, 0,
                                                                            kStreamingLoad));
}

template <int NV, int BS>
__device__ __forceinline__ void load_row(const RowView& rv, float4 (&x)[NV]) {
  load_vectors<NV, BS>(rv.base4, (rv.span + 3) >> 2, 0, x);
}

// The page-table entries of window [0, L) into registers (entry e in
// v[e / BS] of thread e % BS) when they fit the LDS table, then into the
// table. The loads are issued before the row's score loads, so the wait for
// them before the LDS store does not also wait for the scores.
template <int BS>
constexpr int table_per_thread() {
  return (pt_cap<BS>() + BS - 1) / BS;
}

template <bool kPaged, int BS>
__device__ __forceinline__ void load_table(const Emit<kPaged>& em, int32_t L,
                                           int32_t (&v)[table_per_thread<BS>()]) {
  if constexpr (kPaged) {
    const int2 sp = em.table_span(L);
    if (sp.y <= pt_cap<BS>()) {
#pragma unroll
      for (int q = 0; q < table_per_thread<BS>(); ++q) {
        const int32_t e = q * BS + tix();
        v[q] = e < sp.y ? em.pt[sp.x + e] : 0;
      }
    }
  }
}

template <bool kPaged, int BS>
__device__ __forceinline__ void store_table(Emit<kPaged>& em, int32_t* lds, int32_t L,
                                            const int32_t (&v)[table_per_thread<BS>()]) {
  if constexpr (kPaged) {
    const int2 sp = em.table_span(L);
    if (sp.y <= pt_cap<BS>()) {
#pragma unroll
      for (int q = 0; q < table_per_thread<BS>(); ++q) {
        const int32_t e = q * BS + tix();
        if (e < sp.y) lds[e] = v[q];
      }
      em.staged = true;
      em.pt_first = sp.x;
    }
  }
}

// Positions of the elements `sel` takes, into stage[0 ..) in register
// order: each thread counts its own, a scan over the workgroup gives its
// first slot, and a second pass writes them. Without kGuard the caller
// guarantees that at most k elements are taken.
template <int BS, bool kGuard, class Src, class Sel, class Sm>
__device__ __forceinline__ void stage_selected(const Src& src, Sel sel, uint32_t k,
                                               int32_t* stage, Sm& sm) {
  const int lane = lane_id();
  const int w = wave_id();
  uint32_t mine = 0;
  src.for_each([&](uint32_t kk, int32_t j) { mine = add_lane_bit(mine, __ballot(sel(kk, j))); });
  const uint32_t incl = wave_inclusive_sum(mine);
  if (lane == 63) sm.wave_cnt[w] = incl;
  __syncthreads();
  uint32_t slot = incl - mine;
  if constexpr (BS > kBlock) {
    // the counts of the waves before this one: one read per lane and a scan
    const uint32_t c = lane < BS / 64 ? sm.wave_cnt[lane] : 0u;
    const uint32_t ic = wave_inclusive_sum(c);
    slot += w ? read_lane(ic, w - 1) : 0u;
  } else {
    for (int v = 0; v < w; ++v) slot += sm.wave_cnt[v];
  }
  src.for_each([&](uint32_t kk, int32_t j) {
    const bool s = sel(kk, j);
    const uint64_t m = __ballot(s);
    if (kGuard ? (s & (slot < k)) : s) stage[slot] = j;
    slot = add_lane_bit(slot, m);
  });
}

// How many register elements of the workgroup have key >= thr (every
// thread gets the total). wave_cnt is free on entry and again on return.
template <int BS, class Src>
__device__ __forceinline__ uint32_t count_at_least(const Src& src, uint32_t thr,
                                                   uint32_t* wave_cnt) {
  uint32_t mine = 0;  // this wave's count (scalar)
  src.for_each([&](uint32_t kk, int32_t) {
    mine += (uint32_t)__builtin_popcountll(__ballot(kk >= thr));
  });
  if (lane_id() == 0) wave_cnt[wave_id()] = mine;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int v = 0; v < BS / 64; ++v) tot += wave_cnt[v];
  tot = __builtin_amdgcn_readfirstlane(tot);
  __syncthreads();
  return tot;
}

// The elements of the k-th key's first-digit bin are ranked directly when
// there are at most this many of them (a pair compare per element pair).
constexpr uint32_t kRankCap = 256;

// Stage the k selected positions of a register row when the k-th largest
// key lies in the first-digit bin [lo, hi] with `before` keys above it and
// `need` of its elements to take. One pass counts, per thread, the keys
// above hi (taken) and the window keys in the bin (candidates); a second
// writes the taken positions to stage[0 .. before) and the candidates to
// LDS as 64-bit (key, ~position) words, whose order is the selection
// order (higher key, then lower position). A candidate's rank is the
// number of candidates with a larger word (1 to 4 lanes share one
// candidate's compares); ranks below need take stage slot before + rank.
// Key 0 (columns outside the window) is never a candidate. The caller's
// search has closed with a barrier (the histogram is free).
template <int BS, class Src, class Sm>
__device__ __forceinline__ void stage_by_rank(const Src& src, uint32_t lo, uint32_t hi,
                                              uint32_t before, uint32_t need, int32_t* stage,
                                              Sm& sm) {
  constexpr int W = BS / 64;
  const int lane = lane_id();
  const int w = wave_id();
  const uint32_t clo = lo ? lo : 1u;
  // per lane: keys above hi; per wave (scalar): candidates
  uint32_t n_win = 0;
  uint32_t c_wave = 0;
  src.for_each([&](uint32_t kk, int32_t) {
    const uint64_t m_win = __ballot(kk > hi);
    n_win = add_lane_bit(n_win, m_win);
    c_wave += (uint32_t)__builtin_popcountll(__ballot(kk >= clo) & ~m_win);
  });
  const uint32_t iw = wave_inclusive_sum(n_win);
  // one word per wave: winners (below k <= 2048) in the low half,
  // candidates (at most kRankCap) in the high half
  if (lane == 63) sm.wave_cnt[w] = iw | (c_wave << 16);
  __syncthreads();
  uint32_t sw = iw - n_win;
  uint32_t sc;
  uint32_t n;
  {
    const uint32_t a = lane < W ? sm.wave_cnt[lane] : 0u;
    const uint32_t ia = wave_inclusive_sum(a);
    const uint32_t pre = w ? read_lane(ia, w - 1) : 0u;
    sw += pre & 0xffffu;
    sc = pre >> 16;
    n = read_lane(ia, W - 1) >> 16;
  }
  uint64_t* cand = reinterpret_cast<uint64_t*>(stage + kMaxK);
  // zero words after the last candidate: the rank loop reads in groups
  // of four (a zero word is below every candidate's)
  if (tix() < 16) cand[n + tix()] = 0ull;
  // a lane whose element is not taken writes its own spare word instead
  // of branching around the store
  const int32_t spare = kMaxK + 2 * ((int32_t)kRankCap + 16) + lane;
  src.for_each([&](uint32_t kk, int32_t j) {
    const bool win = kk > hi;
    const uint64_t m_win = __ballot(win);
    stage[win ? (int32_t)sw : spare] = j;
    sw = add_lane_bit(sw, m_win);
    const uint64_t m_c = __ballot(kk >= clo) & ~m_win;
    if (m_c) {
      const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m_c >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m_c, 0u));
      if ((kk >= clo) & !win) cand[sc + r] = ((uint64_t)kk << 32) | (uint32_t)~j;
      sc += (uint32_t)__builtin_popcountll(m_c);
    }
  });
  __syncthreads();
  const uint32_t lg = n * 4 <= (uint32_t)BS ? 2u : n * 2 <= (uint32_t)BS ? 1u : 0u;
  const uint32_t g = 1u << lg;
  const uint32_t t = (uint32_t)tix();
  const uint32_t i = t >> lg;
  const uint32_t part = t & (g - 1u);
  uint32_t r = 0;
  uint64_t mine = 0;
  if (i < n) {
    mine = cand[i];
    // four reads in flight per step
    for (uint32_t q = part; q < n; q += 4 * g) {
      const uint64_t c0 = cand[q], c1 = cand[q + g], c2 = cand[q + 2 * g], c3 = cand[q + 3 * g];
      r += (c0 > mine ? 1u : 0u) + (c1 > mine ? 1u : 0u) + (c2 > mine ? 1u : 0u) +
           (c3 > mine ? 1u : 0u);
    }
  }
  // a candidate's lanes are adjacent: sum them within pairs, then quads
  if (lg >= 1) r += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, 0xb1, 0xf, 0xf, false);
  if (lg >= 2) r += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, 0x4e, 0xf, 0xf, false);
  if (i < n && part == 0 && r < need) stage[before + r] = (int32_t)~(uint32_t)mine;
}

// The cut of a register row whose level-1 histogram is in sm.hist, then
// the stage and the emit. The selected positions go to LDS (the
// histogram's space, free after the cut), then one coalesced pass maps and
// stores the k outputs. Without a partial tie class (the usual case) the
// selection is key >= thr, and the cut's counts make that at most k
// elements. With one (several elements hold exactly the k-th key tau and
// only those at positions <= pos are taken) the rare second form applies,
// with a guard on the slot.
template <bool kPaged, int BS, int kPolicy, class Src, int NB>
__device__ __forceinline__ void cut_stage_emit(const Src& src, const Emit<kPaged>& em, int32_t L,
                                               int32_t k, SmemRegB<BS, NB>& sm) {
  int32_t* stage = reinterpret_cast<int32_t*>(sm.hist);
  Cut cut;
  if constexpr (NB == kBins) {
    cut = refine_in_registers<BS>(src, sm, (uint32_t)k);
  } else {
    // A 14-bit first digit (bits 31..18): its threshold bin holds about a
    // quarter of a 12-bit one's elements, so that for most rows the bin's
    // elements are ranked directly instead of taking a second digit.
    static_assert(NB == 4 * kBins, "a 14-bit first digit");
    constexpr uint32_t kShift = 18;
    if (tix() == 0) sm.tie_n = 0u;  // the search's barrier publishes it
    const BinHit h = group_find<NB, true, BS>(sm.hist, (uint32_t)k, sm);
    const uint32_t need = (uint32_t)k - h.before;
    if (h.cnt == need) {
      cut = Cut{kShift, h.bin, kAllPos};
    } else if (h.cnt <= kRankCap) {
      stage_by_rank<BS>(src, h.bin << kShift, (h.bin << kShift) | ((1u << kShift) - 1u),
                        h.before, need, stage, sm);
      __syncthreads();
      write_stage<kPaged, BS, kPolicy>(em, stage, L, k, sm.pt);
      return;
    } else {
      // Too many for ranking: the 12-bit digit's result from the four
      // 14-bit bins of its bin, then the 12-bit refinement.
      const uint32_t b12 = h.bin >> 2;
      uint32_t cnt12 = 0, above = 0;
#pragma unroll
      for (uint32_t q = 0; q < 4; ++q) {
        const uint32_t c = sm.hist[4 * b12 + q];
        cnt12 += c;
        above += 4 * b12 + q > h.bin ? c : 0u;
      }
      const BinHit h12{b12, h.before - above, cnt12};
      __syncthreads();  // the counts are read before the refinement clears them
      cut = refine_from_level1<BS>(src, sm, h12, (uint32_t)k - h12.before);
    }
  }
  if (cut.pos == kAllPos) {
    const uint32_t lo = cut.prefix << cut.shift;
    const uint32_t thr = lo ? lo : 1u;
    stage_selected<BS, false>(
        src, [thr](uint32_t kk, int32_t) { return kk >= thr; }, (uint32_t)k, stage, sm);
  } else {
    const uint32_t tau = cut.prefix;
    const int32_t pos = cut.pos;
    stage_selected<BS, true>(
        src,
        [tau, pos](uint32_t kk, int32_t j) {
          return (kk != 0u) & ((kk > tau) | ((kk == tau) & (j <= pos)));
        },
        (uint32_t)k, stage, sm);
  }
  __syncthreads();
  write_stage<kPaged, BS, kPolicy>(em, stage, L, k, sm.pt);
}

// The rest of the register path, once the row's vectors are in x (and the
// caller has staged the page table, if it stages it).
template <int NV, bool kPaged, int BS, int NB>
__device__ __forceinline__ void row_from_vectors(const RowView& rv, const float4 (&x)[NV],
                                                 const int32_t (&tv)[table_per_thread<BS>()],
                                                 int32_t k, Emit<kPaged> em,
                                                 SmemRegB<BS, NB>& sm) {
  // first digit: the top 12 (or 14) key bits
  constexpr uint32_t kShift1 = NB == kBins ? 20 : 18;
  const int32_t t = tix();
  const int32_t L = rv.span - rv.rem;
  // Register slices 0 .. ilast hold the span's vectors; later slices hold
  // nothing of the row, and every pass skips them.
  const int32_t ilast = __builtin_amdgcn_readfirstlane((((rv.span + 3) >> 2) - 1) / BS);
  uint32_t key[NV][4];
  if constexpr (BS <= kBlock) store_table<kPaged, BS>(em, sm.pt, L, tv);
  clear_bins<NB, BS>(sm.hist);
  __syncthreads();
  // Slice by slice as its loads land: keys, then the level-1 histogram.
  // Columns outside the window get key 0, below every float's key except
  // the all-ones NaN: in the first vector the columns before the window
  // start, and in slice ilast every column at or past the span. All other
  // columns of slices 0 .. ilast lie inside the window. The outside columns
  // count in bin 0 like in every later pass, so the counts of all passes
  // agree.
  {
    const uint32_t one = opaque_one();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i <= ilast) {
#pragma unroll
        for (int c = 0; c < 4; ++c) key[i][c] = order_key(lane_of(x[i], c));
        if (i == 0 && t == 0) {
          if (rv.rem > 0) key[0][0] = 0u;
          if (rv.rem > 1) key[0][1] = 0u;
          if (rv.rem > 2) key[0][2] = 0u;
        }
        if (i == ilast) {
          const int32_t a = 4 * (i * BS + t);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (a + c >= rv.span) key[i][c] = 0u;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) lds_add(&sm.hist[key[i][c] >> kShift1], one);
      }
    }
  }
  // A 1024-thread workgroup runs alone on its CU and waits for everything:
  // it stores the table now, when its loads (issued before the scores) are
  // in, instead of stalling on them before the clear. Workgroups sharing a
  // CU hide that stall and keep the registers instead.
  if constexpr (BS > kBlock) store_table<kPaged, BS>(em, sm.pt, L, tv);
  __syncthreads();
  const RegSrc<NV, BS> src{key, -rv.rem, ilast};
  cut_stage_emit<kPaged, BS, (NV == kLargeVec && BS == kBlock) ? kDefaultStore : kStreamingStore>(
      src, em, L, k, sm);
}

template <int NV, bool kPaged, int BS = kBlock, int NB = kBins>
__device__ __forceinline__ void row_in_registers(const RowView& rv, int32_t k, Emit<kPaged> em,
                                                 SmemRegB<BS, NB>& sm) {
  // Nothing of this row is in flight: this wait costs nothing and keeps the
  // compiler from draining the table load before the score loads (a load
  // another path leaves pending into a register it reuses here).
  __builtin_amdgcn_s_waitcnt(0x0f70);
  int32_t tv[table_per_thread<BS>()];
  load_table<kPaged, BS>(em, rv.span - rv.rem, tv);
  float4 x[NV];
  load_row<NV, BS>(rv, x);
  row_from_vectors<NV, kPaged, BS, NB>(rv, x, tv, k, em, sm);
}

// Rows longer than the registers hold: NL more slices of the row, loaded
// straight into LDS (16 bytes per lane, no VGPRs; the VGPRs are what limits
// the workgroups per CU) and turned into keys there. Element (i, c) of
// thread t is aligned index (i * BS + t) * 4 + c for slices i < NV + NL;
// slice NV + q is lkeys[q * BS + t].
template <int BS, int NL>
struct SmemRegL : SmemRegB<BS> {
  uint4 lkeys[NL * BS];
};

template <int NV, int NL, int BS>
struct RegLdsSrc {
  static constexpr int kPerThread = 4 * (NV + NL);  // elements per thread
  const uint32_t (&key)[NV][4];
  const uint4* lkeys;
  int32_t origin;  // window position of element (0, 0) of thread 0
  int32_t ilast;   // last slice that holds columns (workgroup-uniform)

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    int32_t base = tix() * 4 + origin;
    asm volatile("" : "+v"(base));
    int32_t il = ilast;
    asm volatile("" : "+s"(il));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i <= il) {
#pragma unroll
        for (int c = 0; c < 4; ++c) f(key[i][c], base + i * BS * 4 + c);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      if (NV + q <= il) {
        const uint4 v = lkeys[q * BS + tix()];
        const int32_t j = base + (NV + q) * BS * 4;
        f(v.x, j);
        f(v.y, j + 1);
        f(v.z, j + 2);
        f(v.w, j + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

template <int NV, int NL, bool kPaged, int BS>
__device__ __forceinline__ void row_in_registers_lds(const RowView& rv, int32_t k, Emit<kPaged> em,
                                                     SmemRegL<BS, NL>& sm) {
  const int32_t t = tix();
  const int32_t L = rv.span - rv.rem;
  const int32_t nvec = (rv.span + 3) >> 2;
  const int32_t ilast = __builtin_amdgcn_readfirstlane((nvec - 1) / BS);
  // the LDS slices' loads first (the row's last columns): lane l of wave w
  // lands at lkeys[q * BS + 64 w + l]. Every slice's load takes the same
  // VGPR offset (this thread's 16 bytes) in a buffer that starts at the
  // slice: when the offset VGPR was rewritten between them, the compiler
  // drained every load in flight before the next slice's (one memory round
  // trip per slice instead of one for all).
  {
    // Nothing of this row is in flight yet: this wait (vmcnt 0, the other
    // counters left alone) costs nothing, and it tells the compiler so. A
    // load that another path leaves pending into a register it reuses here
    // would otherwise make it drain the row's own loads at every reuse.
    __builtin_amdgcn_s_waitcnt(0x0f70);
    using lds_void = __attribute__((address_space(3))) void;
    const int32_t off = t * 16;
    // the wave's index straight from the thread index (no VGPR copy that
    // the compiler might place in a register a load in flight still writes)
    const int32_t w = __builtin_amdgcn_readfirstlane((int)threadIdx.x) >> 6;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      if (NV + q <= ilast) {
        const int32_t v0 = (NV + q) * BS;  // the slice's first vector
        __builtin_amdgcn_raw_ptr_buffer_load_lds(row_buffer(rv.base4 + v0, nvec - v0),
                                                 (lds_void*)&sm.lkeys[q * BS + w * 64], 16, off,
                                                 0, 0, kStreamingLoad);
      }
    }
  }
  int32_t tv[table_per_thread<BS>()];
  load_table<kPaged, BS>(em, L, tv);
  float4 x[NV];
  load_vectors<NV, BS>(rv.base4, nvec, 0, x);
  uint32_t key[NV][4];
  clear_bins<kBins, BS>(sm.hist);
  __syncthreads();
  const uint32_t one = opaque_one();
  // register slices as their loads land (as in row_from_vectors)
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (i <= ilast) {
#pragma unroll
      for (int c = 0; c < 4; ++c) key[i][c] = order_key(lane_of(x[i], c));
      if (i == 0 && t == 0) {
        if (rv.rem > 0) key[0][0] = 0u;
        if (rv.rem > 1) key[0][1] = 0u;
        if (rv.rem > 2) key[0][2] = 0u;
      }
      if (i == ilast) {
        const int32_t a = 4 * (i * BS + t);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (a + c >= rv.span) key[i][c] = 0u;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) lds_add(&sm.hist[key[i][c] >> 20], one);
    }
  }
  // the LDS slices, once this wave's loads (issued first) have all landed:
  // each thread turns its own vectors into keys (columns past the span get
  // key 0) and counts them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int q = 0; q < NL; ++q) {
    if (NV + q <= ilast) {
      uint4 v = sm.lkeys[q * BS + t];
      const int32_t a = 4 * ((NV + q) * BS + t);
      uint32_t kv[4] = {order_key(__uint_as_float(v.x)), order_key(__uint_as_float(v.y)),
                        order_key(__uint_as_float(v.z)), order_key(__uint_as_float(v.w))};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kv[c] = a + c < rv.span ? kv[c] : 0u;
        lds_add(&sm.hist[kv[c] >> 20], one);
      }
      sm.lkeys[q * BS + t] = make_uint4(kv[0], kv[1], kv[2], kv[3]);
    }
  }
  store_table<kPaged, BS>(em, sm.pt, L, tv);
  __syncthreads();
  const RegLdsSrc<NV, NL, BS> src{key, sm.lkeys, -rv.rem, ilast};
  cut_stage_emit<kPaged, BS, kStreamingStore>(src, em, L, k, sm);
}

// Span too long for registers: stream it. Pass 1 builds the level-1
// histogram; pass 2 sends the elements above the threshold bin to the
// stage and the threshold bin's elements to LDS, where one wave resolves
// the cut. A threshold bin larger than the LDS buffer is resolved by
// re-reading the span once per digit instead.
template <bool kPaged, int BS>
__device__ __forceinline__ void row_streaming(const RowView& rv, int32_t k, const Emit<kPaged>& em,
                                              SmemStream& sm) {
  const StreamSrc<BS> src{rv};
  const int32_t L = rv.span - rv.rem;
  clear_bins<kBins, BS>(sm.hist);
  if (tix() == 0) {
    sm.nstage = 0;
    sm.ncand = 0;
  }
  __syncthreads();
  src.for_each([&](uint32_t key, int32_t) {
    if (key) lds_inc(&sm.hist[key >> 20]);
  });
  __syncthreads();
  const BinHit h1 = wave_find<kBins, true>(sm.hist, (uint32_t)k);
  const uint32_t t1 = h1.bin;
  const uint32_t need = (uint32_t)k - h1.before;
  const uint32_t cnt = h1.cnt;

  if (cnt != need && cnt <= (uint32_t)kStreamCandCap) {
    src.for_each([&](uint32_t key, int32_t j) {
      const uint32_t bin = key >> 20;
      wave_append((key != 0u) & (bin > t1), j, sm.stage, &sm.nstage, kMaxK);
      wave_append_pair((key != 0u) & (bin == t1), key, j, sm.cand, &sm.ncand, kStreamCandCap);
    });
    __syncthreads();
    if (wave_id() == 0) {
      const WaveCandSrc cs{sm.cand, cnt};
      const Cut cut = refine_cut<true>(cs, sm.hist, t1, need, cnt);
      for (uint32_t i0 = 0; i0 < cnt; i0 += 64) {
        const uint32_t i = i0 + lane_id();
        uint2 e = make_uint2(0, 0);
        if (i < cnt) e = sm.cand[i];
        wave_append((i < cnt) & is_selected(cut, e.x, (int32_t)e.y), (int32_t)e.y, sm.stage,
                    &sm.nstage, kMaxK);
      }
    }
  } else {
    // The whole bin is taken, or it is too large for LDS.
    const Cut cut = refine_cut<false, StreamSrc<BS>, BS>(src, sm.hist, t1, need, cnt);
    src.for_each([&](uint32_t key, int32_t j) {
      wave_append(is_selected(cut, key, j), j, sm.stage, &sm.nstage, kMaxK);
    });
  }
  __syncthreads();
  write_stage<kPaged, BS>(em, sm.stage, L, k, nullptr);
}

// A long row in one pass over its scores. The workgroup streams the row
// in chunks, kS1Depth chunks in flight, and keeps in LDS the (key,
// position) pairs of every element with key >= T. T opens at a key found
// from the row's first chunks (below) and only rises: when the list could
// not take another chunk, T becomes a key no higher than the k-th largest
// of the list (its 24-bit prefix), and only the pairs >= T stay. The k-th
// largest of a subset never exceeds the k-th largest of the row, so once
// at least k pairs reached T, every pair the row's top k needs is in the
// list. After the last chunk the register path resolves the exact cut over
// the list (ties included) and emits. Returns false, having written
// nothing, when the opening pairs overflow the list, when ties keep the
// list too full to take another chunk, or when fewer than k keys of the
// row reached T; the caller then runs the two-pass path.
// From per-wave counts cnt[0 .. W) (written before a barrier the caller
// has passed): x = the count of the waves before this one, y = the total.
template <int W>
__device__ __forceinline__ uint2 wave_slots(const uint32_t* cnt) {
  const uint32_t c = lane_id() < W ? cnt[lane_id()] : 0u;
  const uint32_t inc = wave_inclusive_sum(c);
  const int w = wave_id();
  return make_uint2(w ? read_lane(inc, w - 1) : 0u, read_lane(inc, W - 1));
}

template <int BS>
__device__ __forceinline__ bool compact_candidates(SmemS1& sm, uint32_t k, uint32_t& T,
                                                   uint32_t& n) {
  // Digits of the offset above T, not of the key: the list's keys all sit
  // just above T, so their top bits share a few bins (LDS atomic
  // contention), while their offsets spread. Bin (key - T) >> 12, the last
  // bin taking every larger offset; the lowest key of any bin is a valid
  // new T, the bin holding the k-th largest giving the highest one.
  const int t = tix();
  clear_bins<kBins, BS>(sm.hist);
  __syncthreads();
  for (uint32_t i = t; i < n; i += BS) {
    const uint32_t r = (sm.cand[i].x - T) >> 12;
    lds_inc(&sm.hist[r < (uint32_t)kBins ? r : (uint32_t)kBins - 1u]);
  }
  __syncthreads();
  const BinHit h = wave0_find<kBins, true>(sm.hist, k, sm);
  uint32_t Tn = T + (h.bin << 12);
  if (h.cnt > 64 && h.bin < (uint32_t)kBins - 1u) {
    clear_bins<kBins, BS>(sm.hist);
    __syncthreads();
    for (uint32_t i = t; i < n; i += BS) {
      const uint32_t r = sm.cand[i].x - T;
      if ((r >> 12) == h.bin) lds_inc(&sm.hist[r & 0xfffu]);
    }
    __syncthreads();
    const BinHit h2 = wave0_find<kBins, true>(sm.hist, k - h.before, sm);
    Tn += h2.bin;
  }
  constexpr int kPer = (kS1Cap + BS - 1) / BS;
  uint2 mine[kPer];
  uint32_t total = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t i = (uint32_t)(j * BS + t);
    mine[j] = i < n ? sm.cand[i] : make_uint2(0u, 0u);
    total += (uint32_t)__builtin_popcountll(__ballot(mine[j].x >= Tn));
  }
  if (lane_id() == 0) sm.wave_cnt[wave_id()] = total;
  __syncthreads();  // counts written, and every pair is in registers
  const uint2 st = wave_slots<BS / 64>(sm.wave_cnt);
  uint32_t base = st.x;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const bool keep = mine[j].x >= Tn;
    const uint64_t m = __ballot(keep);
    const uint32_t rank =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (keep) sm.cand[base + rank] = mine[j];
    base += (uint32_t)__builtin_popcountll(m);
  }
  n = st.y;
  T = Tn;
  return n + (uint32_t)kS1Chunk <= (uint32_t)kS1Cap;
}

// The exact cut over a row's (key, position) list in LDS (n >= k pairs,
// every key >= T, every pair the row's top k needs among them), then the
// stage and the emit of the k selected positions.
template <bool kPaged, int BS, class Sm>
__device__ __forceinline__ void list_cut_emit(const RowView& rv, int32_t k, const Emit<kPaged>& em,
                                              Sm& sm, uint32_t n, uint32_t T) {
  // The cut and the stage run on the list where it stands (at least k
  // pairs). On offsets above T when fewer than k pairs reach the offset
  // bound (those are then all above the cut, where their order does not
  // matter); on the keys themselves otherwise.
  const uint32_t kk = (uint32_t)k;
  // The row's page-table entries, when at most kBins - kMaxK, into registers
  // now (their loads overlap the cut), and into the histogram's upper part
  // once the cut is found: the stage below it takes at most kMaxK words.
  // The emit then looks them up in LDS instead of waiting on global loads.
  constexpr int kTabCap = kBins - kMaxK;
  constexpr int kTabPer = kTabCap / BS;
  static_assert(kTabCap % BS == 0, "whole table entries per thread");
  const int32_t L = rv.span - rv.rem;
  const int2 tsp = em.table_span(L);
  const bool tab = kPaged && tsp.y <= kTabCap;
  int32_t tv[kTabPer];
  if (tab) {
#pragma unroll
    for (int q = 0; q < kTabPer; ++q) {
      const int32_t e = q * BS + tix();
      tv[q] = e < tsp.y ? em.pt[tsp.x + e] : 0;
    }
  }
  clear_bins<kBins, BS>(sm.hist);
  __syncthreads();
  int32_t* stage = reinterpret_cast<int32_t*>(sm.hist);
  // Level 1 on the offsets first: every offset at the bound lands in the
  // top bin (with the offsets just below it), so a top bin of fewer than
  // k pairs means fewer than k at the bound. Otherwise (keys far above T)
  // the histogram is rebuilt on the keys.
  const uint32_t one = opaque_one();
  {
    const ListSrc<BS> so{sm.cand, n, T, true};
    so.for_each([&](uint32_t kv, int32_t) { lds_add(&sm.hist[kv >> 20], one); });
  }
  __syncthreads();
  const bool offsets = __builtin_amdgcn_readfirstlane(sm.hist[kBins - 1]) < kk;
  const ListSrc<BS> src{sm.cand, n, T, offsets};
  if (!offsets) {
    __syncthreads();  // every wave has read the top bin
    clear_bins<kBins, BS>(sm.hist);
    __syncthreads();
    src.for_each([&](uint32_t kv, int32_t) { lds_add(&sm.hist[kv >> 20], one); });
    __syncthreads();
  }
  const Cut cut = refine_in_registers<BS>(src, sm, kk, offsets);
  // every search of the cut ended with a barrier after its last histogram
  // read; the tie ranking reads only the first 64 words
  int32_t* table = stage + kMaxK;
  Emit<kPaged> et = em;
  if (tab) {
#pragma unroll
    for (int q = 0; q < kTabPer; ++q) {
      const int32_t e = q * BS + tix();
      if (e < tsp.y) table[e] = tv[q];
    }
    et.staged = true;
    et.pt_first = tsp.x;
  }
  if (cut.pos == kAllPos) {
    const uint32_t lo = cut.prefix << cut.shift;
    const uint32_t thr = lo ? lo : 1u;
    stage_selected<BS, false>(
        src, [thr](uint32_t kv, int32_t) { return kv >= thr; }, kk, stage, sm);
  } else {
    const uint32_t tau = cut.prefix;
    const int32_t pos = cut.pos;
    stage_selected<BS, true>(
        src,
        [tau, pos](uint32_t kv, int32_t j) {
          return (kv != 0u) & ((kv > tau) | ((kv == tau) & (j <= pos)));
        },
        kk, stage, sm);
  }
  __syncthreads();
  write_stage<kPaged, BS>(et, stage, L, k, table);
}

template <bool kPaged, int BS>
__device__ __forceinline__ bool row_stream1(const RowView& rv, int32_t k, const Emit<kPaged>& em,
                                            SmemS1& sm, SmemRegB<BS>& fin, const Prefetch pf) {
  static_assert(kS1Chunk == 4 * BS, "one float4 per thread per chunk");
  const int t = tix();
  const int32_t nvec = (rv.span + 3) >> 2;
  const int32_t nchunk = (nvec + BS - 1) / BS;
  const __amdgpu_buffer_rsrc_t rs = row_buffer(rv.base4, nvec);
  const int32_t off = t * 16;
  if (t < 4) sm.ccnt[t] = 0;
  if (t == 0) sm.n0 = 0;
  uint32_t T = 1;
  uint32_t n = 0;
  float4 buf[kS1Depth];
  auto issue = [&](float4& b, int32_t c) {
    b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + c * BS * 16, 0,
                                                                         kStreamingLoad));
  };
  // Chunk c's pairs (key[q], a0 + q - rem) with sel[q] to the list after
  // position n: one ccnt[c % 4] atomic per wave for the four, then the
  // chunk's barrier, after which n is the new length in every wave.
  auto append4 = [&](const uint32_t (&key)[4], const bool (&sel)[4], int32_t a0, int c4) {
    uint64_t m[4];
    uint32_t total = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m[q] = __ballot(sel[q]);
      total += (uint32_t)__builtin_popcountll(m[q]);
    }
    if (total) {
      uint32_t base = 0;
      if (lane_id() == 0) base = atomicAdd(&sm.ccnt[c4], total);
      base = n + read_lane(base, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m[q] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[q], 0u));
        if (sel[q]) sm.cand[base + rank] = make_uint2(key[q], (uint32_t)(a0 + q - rv.rem));
        base += (uint32_t)__builtin_popcountll(m[q]);
      }
    }
    __syncthreads();
    n += __builtin_amdgcn_readfirstlane(sm.ccnt[c4]);
    if (tix() == 0) sm.ccnt[(c4 + 2) & 3] = 0;
  };
  // The warm-start subset's pairs that `sel` takes open the list: one
  // n0 atomic per wave and half, lane masks in scalar registers; then the
  // barrier that ends the step (the caller has made sure that nothing reads
  // the aliased final-cut space any more).
  auto append_all = [&](const uint32_t (&wk)[kS1Depth][4], auto sel) {
    constexpr int kHalf = kS1Depth / 2;  // two batches: fewer live lane masks
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint64_t m[kHalf][4];
      uint32_t total = 0;
#pragma unroll
      for (int e = 0; e < kHalf; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d = h * kHalf + e;
          m[e][q] = __ballot(sel(wk[d][q], (d * BS + t) * 4 + q - rv.rem));
          total += (uint32_t)__builtin_popcountll(m[e][q]);
        }
      uint32_t base = 0;
      if (lane_id() == 0 && total) base = atomicAdd(&sm.n0, total);
      base = read_lane(base, 0);
#pragma unroll
      for (int e = 0; e < kHalf; ++e)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d = h * kHalf + e;
          const uint64_t mm = m[e][q];
          const uint32_t rank = __builtin_amdgcn_mbcnt_hi(
              (uint32_t)(mm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0u));
          // slots past the list are dropped; the caller sees n > kS1Cap
          if (((mm >> lane_id()) & 1ull) && base + rank < (uint32_t)kS1Cap)
            sm.cand[base + rank] =
                make_uint2(wk[d][q], (uint32_t)((d * BS + t) * 4 + q - rv.rem));
          base += (uint32_t)__builtin_popcountll(mm);
        }
    }
    __syncthreads();
    n = __builtin_amdgcn_readfirstlane(sm.n0);
  };
#pragma unroll
  for (int d = 0; d < kS1Depth; ++d) issue(buf[d], d);

  // Warm start: the first kS1Depth chunks (16384 elements; a long span has
  // more) are held as keys. T opens at the lowest key of the level-1 bin
  // that holds the kt-th largest key of the first kS1Sample chunks, and
  // every pair of the kS1Depth chunks at or above it opens the list, with
  // kt the count that, at the sample's rate, puts about 1.25 k keys of the
  // whole span at or above the kt-th key (the rest of the bin adds a fifth
  // or more on N(0,1) rows: about 1.5 k in all). Histogramming half the
  // held chunks took 2-3 % off streamed launches; kt is then 320 (65536
  // columns) or 160 (131072). On rows whose large keys are spread along the
  // span the list then never reaches the compaction mark (opening at the
  // subset's k-th key, the list of a 131072-column row took about 4000
  // appends and two compactions). A span where fewer than k keys reach T
  // (its largest keys crowd its first columns) is found after the last
  // chunk and re-read by the two-pass path. When the subset's pairs at or
  // above T might not fit the list (a huge bin), the list opens with the
  // subset's exact top k instead, T being its k-th key.
  {
    uint32_t wk[kS1Depth][4];
#pragma unroll
    for (int d = 0; d < kS1Depth; ++d) {
      const int32_t a0 = (d * BS + t) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x = lane_of(buf[d], q);
        wk[d][q] = d == 0 ? key_at(x, a0 + q, rv) : order_key(x);
      }
    }
#pragma unroll
    for (int d = 0; d < kS1Depth; ++d) issue(buf[d], kS1Depth + d);
    clear_bins<kBins, BS>(fin.hist);
    __syncthreads();
    {
      const uint32_t one = opaque_one();
#pragma unroll
      for (int d = 0; d < kS1Sample; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q) lds_add(&fin.hist[wk[d][q] >> 20], one);
    }
    __syncthreads();
    constexpr int32_t kWarm = kS1Sample * kS1Chunk;
    const uint32_t kt = (uint32_t)min(
        k, max(1, (int32_t)((5 * k * kWarm + 4 * rv.span - 1) / (4 * rv.span))));
    const BinHit h = group_find<kBins, true, BS>(fin.hist, kt, fin);
    uint32_t tau;
    // (the sample's pairs at or above T fit; the other held chunks' pairs
    // are checked against the list's size after the append)
    if (h.before + h.cnt <= (uint32_t)(kS1Cap - kS1Chunk)) {
      // the search closed with a barrier: nothing reads the final-cut space
      tau = h.bin << 20;
      tau = tau ? tau : 1u;
      append_all(wk, [tau](uint32_t kv, int32_t) { return kv >= tau; });
    } else {
      // the held chunks past the sample join the histogram (every wave is
      // past the search's closing barrier): the exact cut of all of them
      {
        const uint32_t one = opaque_one();
#pragma unroll
        for (int d = kS1Sample; d < kS1Depth; ++d)
#pragma unroll
          for (int q = 0; q < 4; ++q) lds_add(&fin.hist[wk[d][q] >> 20], one);
      }
      __syncthreads();
      const RegSrc<kS1Depth, BS> src{wk, -rv.rem, kS1Depth - 1};
      const Cut cut = refine_in_registers<BS>(src, fin, (uint32_t)k);
      __syncthreads();  // the final-cut space aliases the list
      if (cut.pos == kAllPos) {
        const uint32_t lo = cut.prefix << cut.shift;
        tau = lo ? lo : 1u;
        append_all(wk, [tau](uint32_t kv, int32_t) { return kv >= tau; });
      } else {
        tau = cut.prefix;
        const int32_t pos = cut.pos;
        append_all(wk, [tau, pos](uint32_t kv, int32_t j) {
          return (kv != 0u) & ((kv > tau) | ((kv == tau) & (j <= pos)));
        });
      }
    }
    T = tau > 1u ? tau : 1u;
  }
  // Set when a compaction cannot make room for a chunk (heavy ties): the
  // chunk loop stops appending and ends at its next turn. No exit from
  // inside the unrolled body, whose waits for the loads in flight the
  // compiler counts exactly only on straight-line paths; for the same
  // reason every buffered chunk is processed and refilled (chunks past the
  // row are all masked, and loads past the buffer's end return zeros
  // without touching memory).
  // The sample bounds only its own chunks' pairs: when the held chunks
  // brought more pairs than the list holds (keys rising along the row),
  // some were dropped and the row takes the two-pass path.
  bool overflow = n > (uint32_t)kS1Cap;
  for (int32_t c0 = kS1Depth; c0 < nchunk && !overflow; c0 += kS1Depth) {
#pragma unroll
    for (int d = 0; d < kS1Depth; ++d) {
      const int32_t c = c0 + d;
      if (c < nchunk && !overflow && n + (uint32_t)kS1Chunk > (uint32_t)kS1Cap)
        overflow = !compact_candidates<BS>(sm, (uint32_t)k, T, n);
      const uint32_t Tc = overflow ? 0xffffffffu : T;  // no key reaches all ones
      const bool edge = (c + 1) * kS1Chunk > rv.span;
      const int32_t a0 = (c * BS + t) * 4;
      uint32_t key[4];
      bool sel[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x = lane_of(buf[d], q);
        key[q] = edge ? key_at(x, a0 + q, rv) : order_key(x);
        sel[q] = key[q] >= Tc;
      }
      // the chunk is in registers as keys: its buffer refills before the
      // append's barrier, not after it
      issue(buf[d], c + kS1Depth);
      append4(key, sel, a0, d);  // c0 is a multiple of 4: c % 4 == d
    }
  }
  __syncthreads();  // every wave's last pairs are in the list
  // fewer than k pairs: T opened above the span's k-th key (or the window
  // holds keys below every threshold, i.e. all-ones NaNs): two passes
  if (overflow || n < (uint32_t)k) return false;
  // the next row's opening lines (see kPrefetchAhead): one word per 64-byte
  // line, loads past pf.bytes return zero without touching memory
  uint32_t touched = 0;
  if (pf.base) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(pf.base), (short)0, pf.bytes, 0x00020000);
    touched = __builtin_amdgcn_raw_buffer_load_b32(r, tix() * 64, 0, 0);
  }

  list_cut_emit<kPaged, BS>(rv, k, em, sm, n, T);
  asm volatile("" ::"v"(touched));  // keeps the touch (landed long before)
  return true;
}

// Long rows in register pieces (the 512-thread register kernel). A long
// row that is not split is read in pieces of kPiece floats, each held in
// registers while it is scanned (8 float4 per thread: with more, the
// pieces' bookkeeping no longer fits the kernel's 80 VGPRs). T opens at the
// key of rank kt in the first piece, kt the count that, at the piece's
// rate, puts about 1.25 k keys of the whole span at or above it (kt = k
// when the span is at most 1.25 pieces); the 24-bit prefix of that key
// (level-1 and level-2 digits) gives T. Every piece's pairs with key >= T
// go to an LDS list. When a piece's pairs would overflow the list, T rises
// to the floor of the offset bin that holds the k-th largest key of the
// list and the piece together, and the list keeps its pairs >= T. Once the
// last piece is in and at least k pairs reached T, every key of the row's
// top k is in the list, and the final cut runs on it. A row where fewer
// than k keys reached T (its largest keys crowd its first piece), or whose
// pairs overflow the list at every threshold it can reach (heavy ties), is
// re-read by the two-pass path.
constexpr int kPieceVec = 8;
constexpr int kPiece = kPieceVec * 4 * kBigBlock;  // 16384
constexpr int kListCap = 4352;
// The list with the running sums of all-wave searches (the keys of a piece
// stay in registers through the searches, which a one-wave search of 4096
// bins would push into spills): three fit a CU's 160 KB of LDS.
struct SmemPieces : SmemListB<kBigBlock, kListCap> {
  uint32_t lsum[kBigBlock];
  uint32_t wsum[kBigBlock / 64];
};
template <>
struct HasWaveSums<SmemPieces> {
  static constexpr bool value = true;
};

// Appends the register elements with key >= thr to cand[n ..) in register
// order (slots at or past CAP are dropped: the caller has checked the
// count) and returns the new length.
template <int BS, int CAP, class Src>
__device__ __forceinline__ uint32_t append_at_least(const Src& src, uint32_t thr, uint2* cand,
                                                    uint32_t n, uint32_t* wave_cnt) {
  const int lane = lane_id();
  const int w = wave_id();
  uint32_t mine = 0;
  src.for_each([&](uint32_t kk, int32_t) { mine = add_lane_bit(mine, __ballot(kk >= thr)); });
  const uint32_t incl = wave_inclusive_sum(mine);
  if (lane == 63) wave_cnt[w] = incl;
  __syncthreads();
  const uint32_t c = lane < BS / 64 ? wave_cnt[lane] : 0u;
  const uint32_t ic = wave_inclusive_sum(c);
  uint32_t slot = n + incl - mine + (w ? read_lane(ic, w - 1) : 0u);
  const uint32_t tot = read_lane(ic, BS / 64 - 1);
  src.for_each([&](uint32_t kk, int32_t j) {
    const bool s = kk >= thr;
    const uint64_t m = __ballot(s);
    if (s & (slot < (uint32_t)CAP)) cand[slot] = make_uint2(kk, (uint32_t)j);
    slot = add_lane_bit(slot, m);
  });
  __syncthreads();
  return n + tot;
}

// Keeps the list's pairs with key >= Tn, in order, in place, and returns
// the new length. One pair per thread at a time: each block of BS pairs is
// read, ranked and written at or below its own start (all of a block's
// reads come before its writes, and its writes land below the next block).
template <int BS>
__device__ __forceinline__ uint32_t compact_inplace(uint2* cand, uint32_t n, uint32_t Tn,
                                                    uint32_t* wave_cnt) {
  const int lane = lane_id();
  const int w = wave_id();
  uint32_t out = 0;
  for (uint32_t b0 = 0; b0 < n; b0 += BS) {
    const uint32_t i = b0 + (uint32_t)tix();
    const uint2 e = i < n ? cand[i] : make_uint2(0u, 0u);
    const bool keep = (i < n) & (e.x >= Tn);
    const uint64_t m = __ballot(keep);
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (lane == 0) wave_cnt[w] = (uint32_t)__builtin_popcountll(m);
    __syncthreads();
    const uint32_t c = lane < BS / 64 ? wave_cnt[lane] : 0u;
    const uint32_t ic = wave_inclusive_sum(c);
    const uint32_t pre = w ? read_lane(ic, w - 1) : 0u;
    if (keep) cand[out + pre + rank] = e;
    out += read_lane(ic, BS / 64 - 1);
    __syncthreads();
  }
  return out;
}

// T rises to the floor of the offset bin holding the k-th largest key of
// the list and of the register keys >= T together (offsets key - T in
// 12-bit digits, the top bin taking every larger offset; inside a bin of
// more than 64 pairs the next 12 offset bits), and the list keeps its pairs
// >= the new T. At least k keys of the two reach it.
template <int BS, class Src, class Sm>
__device__ __forceinline__ void raise_threshold(const Src& src, Sm& sm, uint32_t k, uint32_t& T,
                                                uint32_t& n) {
  const uint32_t t = (uint32_t)tix();
  const uint32_t T0 = T;
  const uint32_t one = opaque_one();
  auto bin1 = [T0](uint32_t kk) {
    const uint32_t r = (kk - T0) >> 12;
    return r < (uint32_t)kBins ? r : (uint32_t)kBins - 1u;
  };
  clear_bins<kBins, BS>(sm.hist);
  __syncthreads();
  for (uint32_t i = t; i < n; i += BS) lds_add(&sm.hist[bin1(sm.cand[i].x)], one);
  src.for_each([&](uint32_t kk, int32_t) {
    if (kk >= T0) lds_add(&sm.hist[bin1(kk)], one);
  });
  __syncthreads();
  const BinHit h = group_find<kBins, true, BS>(sm.hist, k, sm);
  uint32_t Tn = T0 + (h.bin << 12);
  if (h.cnt > 64u && h.bin < (uint32_t)kBins - 1u) {
    clear_bins<kBins, BS>(sm.hist);
    __syncthreads();
    const uint32_t hb = h.bin;
    for (uint32_t i = t; i < n; i += BS) {
      const uint32_t r = sm.cand[i].x - T0;
      if ((r >> 12) == hb) lds_add(&sm.hist[r & 0xfffu], one);
    }
    src.for_each([&](uint32_t kk, int32_t) {
      const uint32_t r = kk - T0;
      if ((kk >= T0) & ((r >> 12) == hb)) lds_add(&sm.hist[r & 0xfffu], one);
    });
    __syncthreads();
    const BinHit h2 = group_find<kBins, true, BS>(sm.hist, k - h.before, sm);
    Tn += h2.bin;
  }
  n = compact_inplace<BS>(sm.cand, n, Tn, sm.wave_cnt);
  T = Tn;
}

// A long row in pieces (span > 2 * kPiece). Returns false, having written
// nothing, when fewer than k keys reach T or the list cannot hold the
// pairs at or above any threshold it can reach (the caller then runs the
// two-pass path).
template <bool kPaged>
__device__ __forceinline__ bool row_in_pieces(const RowView& rv, int32_t k, const Emit<kPaged>& em,
                                              SmemPieces& sm) {
  constexpr int BS = kBigBlock;
  constexpr int NV = kPieceVec;
  const int32_t t = tix();
  const int32_t nvec = (rv.span + 3) >> 2;
  const int32_t npiece = (rv.span + kPiece - 1) / kPiece;
  const uint32_t kk = (uint32_t)k;
  uint32_t T = 1;
  uint32_t n = 0;
  for (int32_t pc = 0; pc < npiece; ++pc) {
    const int32_t v0 = pc * (kPiece / 4);
    float4 x[NV];
    load_vectors<NV, BS>(rv.base4, nvec, v0, x);
    // register slices 0 .. ilast hold the piece's columns
    const int32_t rest = (nvec - v0 - 1) / BS;
    const int32_t ilast = __builtin_amdgcn_readfirstlane(rest < NV - 1 ? rest : NV - 1);
    // keys, with key 0 for every column outside the window (a branch-free
    // range test per element: the piece's columns before the window start,
    // or at or past the span)
    uint32_t key[NV][4];
    {
      const uint32_t lim = (uint32_t)(rv.span - rv.rem);
      int32_t a = 4 * (v0 + t) - rv.rem;  // window position of element (0, 0)
      asm volatile("" : "+v"(a));
#pragma unroll
      for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t kv = order_key(lane_of(x[i], c));
          key[i][c] = (uint32_t)(a + i * BS * 4 + c) < lim ? kv : 0u;
        }
    }
    const RegSrc<NV, BS> src{key, v0 * 4 - rv.rem, ilast};
    if (pc == 0) {
      clear_bins<kBins, BS>(sm.hist);
      __syncthreads();
      {
        const uint32_t one = opaque_one();
        src.for_each([&](uint32_t kv, int32_t) { lds_add(&sm.hist[kv >> 20], one); });
      }
      __syncthreads();
      // T: the floor of the 24-bit prefix bin holding the piece's kt-th key
      const uint32_t kt = (uint32_t)min(
          k, max(1, (int32_t)((5 * (int64_t)k * kPiece + 4 * rv.span - 1) / (4 * rv.span))));
      const BinHit h = group_find<kBins, true, BS>(sm.hist, kt, sm);
      clear_bins<kBins, BS>(sm.hist);
      __syncthreads();
      {
        const uint32_t one = opaque_one();
        const uint32_t b1 = h.bin;
        src.for_each([&](uint32_t kv, int32_t) {
          if ((kv >> 20) == b1) lds_add(&sm.hist[(kv >> 8) & 0xfffu], one);
        });
      }
      __syncthreads();
      const BinHit h2 = group_find<kBins, true, BS>(sm.hist, kt - h.before, sm);
      T = (h.bin << 20) | (h2.bin << 8);
      T = T ? T : 1u;
      if (h.before + h2.before + h2.cnt > (uint32_t)kListCap) return false;
    } else if (n + count_at_least<BS>(src, T, sm.wave_cnt) > (uint32_t)kListCap) {
      raise_threshold<BS>(src, sm, kk, T, n);
      if (n + count_at_least<BS>(src, T, sm.wave_cnt) > (uint32_t)kListCap) return false;
    }
    n = append_at_least<BS, kListCap>(src, T, sm.cand, n, sm.wave_cnt);
  }
  // fewer than k keys of the span reached T (its largest keys crowd its
  // first piece, or the window holds keys below every threshold, i.e.
  // all-ones NaNs): the two-pass path
  if (n < kk) return false;
  list_cut_emit<kPaged, BS>(rv, k, em, sm, n, T);
  return true;
}

template <bool kPaged>
__device__ __forceinline__ Emit<kPaged> row_emit(const Params& p, int64_t b) {
  Emit<kPaged> em;
  em.out = p.out + b * p.k;
  em.out_raw = nullptr;
  em.page_bits = p.page_bits;
  em.staged = false;
  em.pt_first = 0;
  em.pt_off = 0;
  if constexpr (kPaged) {
    const int64_t tr = p.table_rows ? p.table_rows[b] : b;
    em.pt = p.page_table + tr * p.pt_stride;
    em.pt_off = p.table_starts ? p.table_starts[b] : 0;
    if (p.out_raw) em.out_raw = p.out_raw + b * p.k;
    em.offset = 0;
  } else {
    em.pt = nullptr;
    em.offset = p.out_offsets[b];
  }
  return em;
}

struct RowInfo {
  int32_t L;
  int32_t s;
  int32_t span;
  int32_t cls;
};

// Class of a row from its length word and start: short = trivial (L <= k)
// or span <= 8192 floats; mid = span <= 16384; big = span <= 32768; long =
// the rest. The one rule every kernel, the plan and the next-row touch use,
// so that each row is served by exactly one kernel.
__device__ __forceinline__ RowInfo classify(int32_t len, int32_t s, int32_t k) {
  RowInfo r;
  r.L = len < 0 ? 0 : (len > DSATOPK_MAX_SEQ_LEN ? DSATOPK_MAX_SEQ_LEN : len);
  r.s = s;
  r.span = r.L + (r.s & 3);
  r.cls = (r.L <= k || r.span <= kSmallVec * 4 * kBlock) ? kClassShort
          : (r.span <= kLargeVec * 4 * kBlock)            ? kClassMid
          : (r.span <= kBigCap)                           ? kClassBig
                                                          : kClassLong;
  return r;
}

__device__ __forceinline__ RowInfo row_info(const int32_t* seq_lens, const int32_t* row_starts,
                                            int32_t k, int64_t b) {
  return classify(seq_lens[b], row_starts ? row_starts[b] : 0, k);
}

// A word that no kernel of this library writes while it runs (row lengths
// and starts, table rows and starts, out offsets, the plan's header, row
// entries and work items), read as constant memory: a scalar load through
// the scalar cache. The compiler issues such loads together, where vector
// loads of these words, under register pressure, went through one VGPR and
// each waited for the one before.
__device__ __forceinline__ int32_t ld_const(const int32_t* a) {
  return *(const __attribute__((address_space(4))) int32_t*)a;
}

// Every word a row's workgroup reads before its scores, loaded together:
// one memory round trip before the first score load instead of a chain of
// dependent ones (under a full-chip load each round trip costs
// microseconds). An optional array that is absent is read at a valid
// stand-in address (the row's length) and its value replaced afterwards, so
// no load waits on the test of another. The plan words are read only when
// with_plan; a plan passed to a call is at least dsatopk_plan_bytes long
// (checked on the host), so its row words are in bounds whatever it holds.
struct RowMeta {
  RowInfo r;
  int32_t trow;     // PAGED: page-table row
  int32_t tstart;   // PAGED: table position of window position 0
  int32_t offset;   // RAGGED: the row's out offset
  int32_t nseg;     // plan: the row's segments (split rows)
  int32_t slot;     // plan: the row's exchange area (split rows)
  int32_t seg_len;  // plan: floats per segment
  bool split;       // the plan sends the row to the split workers
};

template <bool kPaged>
__device__ __forceinline__ RowMeta row_meta(const Params& p, int64_t b, bool with_plan) {
  const int32_t* a_len = p.seq_lens + b;
  const int32_t* a_rs = p.row_starts ? p.row_starts + b : a_len;
  const int32_t* a_tr = (kPaged && p.table_rows) ? p.table_rows + b : a_len;
  const int32_t* a_ts = (kPaged && p.table_starts) ? p.table_starts + b : a_len;
  const int32_t* a_of = kPaged ? a_len : p.out_offsets + b;
  const bool hp = with_plan && p.plan != nullptr;
  const int32_t* a_pm = hp ? p.plan + kPlanWordMagic : a_len;
  const int32_t* a_pr = hp ? p.plan + kPlanWordRows : a_len;
  const int32_t* a_pg = hp ? p.plan + kPlanWordSegLen : a_len;
  const int32_t* a_ps = hp ? p.plan + plan_nseg_word(p.num_rows) + b : a_len;
  const int32_t* a_pl = hp ? p.plan + plan_slot_word(p.num_rows) + b : a_len;
  // (readfirstlane: a no-op on scalar loads; a vector load, where the
  // compiler cannot prove the words unchanged, still ends in an SGPR)
  auto rd = [](const int32_t* a) { return __builtin_amdgcn_readfirstlane(ld_const(a)); };
  int32_t len = rd(a_len), rs = rd(a_rs), tr = rd(a_tr), ts = rd(a_ts), of = rd(a_of);
  int32_t pm = rd(a_pm), pr = rd(a_pr), pg = rd(a_pg), ps = rd(a_ps), pl = rd(a_pl);
  // every value is needed here: the compiler may not sink a load into the
  // branch that uses it (which would put it behind another load's wait)
  asm volatile("" : "+s"(len), "+s"(rs), "+s"(tr), "+s"(ts), "+s"(of), "+s"(pm), "+s"(pr),
               "+s"(pg), "+s"(ps), "+s"(pl));
  RowMeta m;
  RowInfo& r = m.r;
  r = classify(len, p.row_starts ? rs : 0, p.k);
  r.L = __builtin_amdgcn_readfirstlane(r.L);
  r.s = __builtin_amdgcn_readfirstlane(r.s);
  r.span = __builtin_amdgcn_readfirstlane(r.span);
  r.cls = __builtin_amdgcn_readfirstlane(r.cls);
  m.trow = __builtin_amdgcn_readfirstlane((kPaged && p.table_rows) ? tr : (int32_t)b);
  m.tstart = __builtin_amdgcn_readfirstlane((kPaged && p.table_starts) ? ts : 0);
  m.offset = __builtin_amdgcn_readfirstlane(kPaged ? 0 : of);
  m.nseg = ps;
  m.slot = pl;
  m.seg_len = pg;
  const bool ours = hp && pm == kPlanMagic && pr == p.num_rows;
  m.split = ours && r.cls == kClassLong && (pg == kSegShort || pg == kSegLong) && ps >= 2 &&
            ps == segments_for(r.span, pg) && pl >= 0 && pl < plan_split_cap(p.num_rows);
  return m;
}

// row_emit from words already loaded.
template <bool kPaged>
__device__ __forceinline__ Emit<kPaged> row_emit(const Params& p, int64_t b, const RowMeta& m) {
  Emit<kPaged> em;
  em.out = p.out + b * p.k;
  em.out_raw = nullptr;
  em.page_bits = p.page_bits;
  em.staged = false;
  em.pt_first = 0;
  em.pt_off = 0;
  if constexpr (kPaged) {
    em.pt = p.page_table + (int64_t)m.trow * p.pt_stride;
    em.pt_off = m.tstart;
    if (p.out_raw) em.out_raw = p.out_raw + b * p.k;
    em.offset = 0;
  } else {
    em.pt = nullptr;
    em.offset = m.offset;
  }
  return em;
}

__device__ __forceinline__ RowView row_view(const Params& p, int64_t b, const RowInfo& r) {
  RowView rv;
  const int32_t rem = r.s & 3;
  rv.base4 = reinterpret_cast<const float4*>(p.scores + b * p.stride + (r.s - rem));
  rv.rem = rem;
  rv.span = r.span;
  return rv;
}



// Trivial rows and spans <= 8192 floats, kept in registers.
template <bool kPaged>
__global__ __launch_bounds__(kBlock) void rows_short_kernel(const Params p) {
  const int64_t b = blockIdx.x;
  const RowMeta m = row_meta<kPaged>(p, b, false);
  const RowInfo& r = m.r;
  if (r.cls != kClassShort) return;
  const Emit<kPaged> em = row_emit<kPaged>(p, b, m);
  if (r.L <= p.k) {
    write_trivial(em, r.L, p.k);
    return;
  }
  __shared__ SmemReg sm;
  row_in_registers<kSmallVec>(row_view(p, b, r), p.k, em, sm);
}

// Same rows with 512 threads per row (4 float4 per thread), for batches
// too small to fill the chip: a row's latency, not the rows in flight,
// sets the time. 512 threads put two waves of the row on each SIMD, where
// 1024 put four that all run the searches' dependent steps (128 rows of
// 8192 floats: 6.65 us per launch against 6.75 at 1024 threads and 8.1 at
// 256; 4 rows of 3000: 6.0 us against 7.1 at 1024).
// The first key digit takes 14 bits (a 64 KiB histogram: one workgroup per
// CU at these batch sizes has the LDS): its threshold bin holds about 40 of
// a decode row's 8192 keys, which are ranked directly instead of taking a
// second 12-bit digit and a separate stage pass (128 rows of 8192 floats:
// 6.60 -> 6.17 us per launch; 4 rows of 3000: 6.00 -> 5.90 us).
template <bool kPaged>
__global__ __launch_bounds__(kWideBlock) void rows_wide_kernel(const Params p) {
  const int64_t b = blockIdx.x;
  const RowMeta m = row_meta<kPaged>(p, b, false);
  const RowInfo& r = m.r;
  if (r.cls != kClassShort) return;
  const Emit<kPaged> em = row_emit<kPaged>(p, b, m);
  if (r.L <= p.k) {
    write_trivial<kPaged, kWideBlock>(em, r.L, p.k);
    return;
  }
  __shared__ SmemRegB<kWideBlock, 4 * kBins> sm;
  row_in_registers<kSmallVec * kBlock / kWideBlock, kPaged, kWideBlock, 4 * kBins>(
      row_view(p, b, r), p.k, em, sm);
}

// Every row of a batch with a score stride of 8193 .. 16384 floats, in one
// launch: 256 threads per row, holding 8 or 16 float4 each by the row's
// span. Five rows share a CU (86 VGPRs); 512 threads with 8 float4 each
// (three rows per CU) ran 6-12% slower on such rows.
template <bool kPaged>
__global__ __launch_bounds__(kBlock) void rows_mid_kernel(const Params p) {
  const int64_t b = blockIdx.x;
  const RowMeta m = row_meta<kPaged>(p, b, false);
  const RowInfo& r = m.r;
  if (r.cls != kClassShort && r.cls != kClassMid) return;
  const Emit<kPaged> em = row_emit<kPaged>(p, b, m);
  if (r.L <= p.k) {
    write_trivial(em, r.L, p.k);
    return;
  }
  __shared__ SmemReg sm;
  const RowView rv = row_view(p, b, r);
  if (r.span <= kSmallVec * 4 * kBlock)
    row_in_registers<kSmallVec>(rv, p.k, em, sm);
  else
    row_in_registers<kLargeVec>(rv, p.k, em, sm);
}

// A published round result: round number in bits 63..56, the payload in
// the low 56 bits (a bin search: bin << 36 | before << 18 | count, each
// count < 2^18).
__device__ __forceinline__ uint64_t pack_round(uint32_t round, uint64_t payload) {
  return ((uint64_t)round << 56) | payload;
}
__device__ __forceinline__ uint64_t pack_hit(const BinHit& h) {
  return ((uint64_t)h.bin << 36) | ((uint64_t)h.before << 18) | (uint64_t)h.cnt;
}
__device__ __forceinline__ BinHit unpack_hit(uint64_t w) {
  BinHit h;
  h.bin = (uint32_t)(w >> 36) & 0xfffffu;
  h.before = (uint32_t)(w >> 18) & 0x3ffffu;
  h.cnt = (uint32_t)w & 0x3ffffu;
  return h;
}

// Split-row synchronisation. Every access to a row's exchange area is a
// device-scope atomic (read-modify-write, load or store), and device-scope
// atomics are coherent across the chip's XCDs; none of them needs the L2
// write-back or invalidation that release / acquire fences would add at
// every round. Ordering comes from waiting: before a segment arrives, each
// of its waves waits until its own accesses have completed, so whoever
// sees the arrival count complete also sees every contribution. Every
// segment arrives once per round; the last to arrive computes the round's
// result and publishes it in one 64-bit word, which the others poll.
// Polls are bounded: a segment that gives up marks its row and the plan as
// failed and takes no further part in the row (the row's outputs become
// -1, see split_finish), so no wave can hang.
//
// Forward progress: the W split workers are the first W <= 768 workgroups
// of the register kernel's grid (three fit a CU), worker w serving work
// items w, w + W, ... in order, and a row's segments are consecutive items.
// When the workers are resident together, every row completes: a row's
// segments are served in the same pass over the items, or a row that
// straddles two passes waits for workers that finish rows of the earlier
// pass first. Workgroups are dispatched in grid order on an otherwise idle
// GPU, which makes the workers resident together; HIP does not promise
// that, and where it does not hold the bounded waits give up instead of
// hanging, and the plan's error word and the row's -1 outputs report it.
// (A counter that workers claim items from would not need the promise, but
// each claim is a device-scope atomic on one address, and hundreds of them
// serialize for tens of microseconds.)
struct SplitSync {
  uint32_t* x;       // the row's exchange area
  int32_t S;         // segments of the row
  int32_t* err;      // the plan's error word
  uint32_t spin;     // polls before a wait gives up
  uint32_t* word;    // LDS: [0] arrival, [1] [2] round result, [3] gave up

  // Returns true in the last segment to arrive at `round` (whole workgroup).
  __device__ __forceinline__ bool arrive(uint32_t round) const {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's accesses completed
    __syncthreads();
    if (tix() == 0) {
      const uint32_t prev =
          __hip_atomic_fetch_add(&x[kXArrive], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      word[0] = prev == (uint32_t)S * round - 1u;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(word[0]) != 0u;
  }

  // Last arriver, whole workgroup: once every thread's exchange accesses
  // have completed, make `payload` the result of `round`.
  __device__ __forceinline__ void publish(uint32_t round, uint64_t payload) const {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tix() == 0)
      __hip_atomic_store(reinterpret_cast<uint64_t*>(x + kXFlag), pack_round(round, payload),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Everyone: the published result of `round` into res (the last arriver
  // passes `mine`, which it just published). False when the wait gave up.
  __device__ __forceinline__ bool result(uint32_t round, bool last, uint64_t mine,
                                         uint64_t& res) const {
    if (tix() == 0) {
      uint64_t w = mine;
      uint32_t gave_up = 0u;
      if (!last) {
        const uint64_t* f = reinterpret_cast<const uint64_t*>(x + kXFlag);
        uint32_t n = 0;
        while (((w = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >> 56) <
               round) {
          if (++n > spin) {
            gave_up = 1u;
            __hip_atomic_store(&x[kXFail], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
      }
      word[1] = (uint32_t)w;
      word[2] = (uint32_t)(w >> 32);
      word[3] = gave_up;
    }
    __syncthreads();
    res = (((uint64_t)word[2] << 32) | word[1]) & ((1ull << 56) - 1ull);
    return __builtin_amdgcn_readfirstlane(word[3]) == 0u;
  }
};

// One histogram round: every segment adds its local LDS histogram (NB
// bins) into the row's global one; the last to arrive gathers the totals
// into its LDS (one coalesced read), finds the bin where the running count
// reaches `need`, zeroes the global bins it found set and publishes. A
// later round adds into the same bins, so they are zero before the publish
// when one may follow; when none can (the bin is taken whole, or it holds
// at most later_cap elements, which go to the candidate buffer instead) the
// zeroing follows the publish, off the other segments' path. False when the
// wait gave up.
template <int NB, bool kDesc, int BS>
__device__ __forceinline__ bool histogram_round(uint32_t* lds_hist, uint32_t* g_hist,
                                                uint32_t round, uint32_t need,
                                                uint32_t later_cap, const SplitSync& sy,
                                                SmemSplitB<BS>& sm, BinHit& hit) {
  const int32_t t = tix();
  __syncthreads();  // local histogram complete
  for (int32_t i = t; i < NB; i += BS) {
    const uint32_t v = lds_hist[i];
    if (v) __hip_atomic_fetch_add(&g_hist[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const bool last = sy.arrive(round);
  uint64_t mine = 0;
  if (last) {
    if constexpr (NB % (4 * BS) == 0) {
      // 16 bytes per load, with the cache policy of a relaxed device-scope
      // atomic load (sc1): the totals as the other segments' atomics left them
      const __amdgpu_buffer_rsrc_t rh = words_buffer(reinterpret_cast<int32_t*>(g_hist), NB);
#pragma unroll
      for (int q = 0; q < NB / (4 * BS); ++q) {
        const int32_t i4 = q * BS + t;
        reinterpret_cast<uint4*>(lds_hist)[i4] =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, i4 * 16, 0, 16));
      }
    } else {
      for (int32_t i = t; i < NB; i += BS)
        lds_hist[i] = __hip_atomic_load(&g_hist[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    // (4096 bins: every wave searches a part; fewer: one wave each)
    const BinHit f = group_find<NB, kDesc, BS>(lds_hist, need, sm);
    mine = pack_hit(f);
    auto zero = [&]() {
      for (int32_t i = t; i < NB; i += BS)
        if (lds_hist[i])
          __hip_atomic_store(&g_hist[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    const bool later = (f.cnt != need - f.before) && (f.cnt > later_cap);
    if (later) zero();
    sy.publish(round, mine);
    if (!later) zero();
  }
  uint64_t res;
  const bool ok = sy.result(round, last, mine, res);
  hit = unpack_hit(res);
  return ok;
}

// AND / OR of v over the wave, in lane 63 (DPP row shifts, then the row
// broadcasts; a lane with no source keeps its own value).
__device__ __forceinline__ uint32_t wave_and63(uint32_t v) {
  v &= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xf, 0xf, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xf, 0xf, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xf, 0xf, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xf, 0xf, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false);
  v &= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false);
  return v;
}
__device__ __forceinline__ uint32_t wave_or63(uint32_t v) {
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xf, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false);
  v |= (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false);
  return v;
}

// The exact cut among the candidate (key, position) pairs of one level-1
// bin, NP per thread in registers (key 0: no candidate), taking `need` of
// them; the whole workgroup. The keys' AND and OR give the bits in which
// they differ: 8-bit digit rounds run over those bits only (the bits below
// them are the same in every key), each a histogram of the candidates
// still matching the digits fixed so far, searched by every wave. Ties at
// the k-th key take the lowest positions: a tie class of at most 64
// elements is gathered and ranked on lane masks by wave 0, a larger one
// takes position digits (8, 8 and 1 bits). The result selects key > tau,
// or key == tau at position <= pos (pos == kAllPos: every such key).
template <int BS, int NP>
__device__ __forceinline__ Cut resolve_pairs_regs(const uint32_t (&ck)[NP], const int32_t (&cp)[NP],
                                                  uint32_t n, uint32_t need, SmemSplitB<BS>& sm) {
  const int32_t t = tix();
  const int lane = lane_id();
  uint32_t a = 0xffffffffu, o = 0u;
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    if (ck[q]) {
      a &= ck[q];
      o |= ck[q];
    }
  }
  a = wave_and63(a);
  o = wave_or63(o);
  if (t == 0) {
    sm.bcast[0] = 0xffffffffu;
    sm.bcast[1] = 0u;
    sm.tie_n = 0u;
  }
  if (t < 256) sm.h2[t] = 0u;  // the first digit round's histogram
  __syncthreads();
  if (lane == 63) {
    atomicAnd(&sm.bcast[0], a);
    atomicOr(&sm.bcast[1], o);
  }
  __syncthreads();
  const uint32_t all_and = __builtin_amdgcn_readfirstlane(sm.bcast[0]);
  const uint32_t diff = all_and ^ __builtin_amdgcn_readfirstlane(sm.bcast[1]);
  uint32_t fixed = all_and & ~diff;  // the key bits decided so far
  uint32_t cnt = n;
  if (diff) {
    const int lo_bit = __builtin_ctz(diff);
    bool first = true;
    for (int top = 31 - __builtin_clz(diff); top >= lo_bit; top -= 8) {
      const int width = top - lo_bit + 1 < 8 ? top - lo_bit + 1 : 8;
      const int sh = top - width + 1;
      const uint32_t above = top == 31 ? 0u : fixed >> (top + 1);
      if (!first) {
        __syncthreads();  // every wave's search of the last round is done
        if (t < 256) sm.h2[t] = 0u;
        __syncthreads();
      }
      first = false;
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const uint32_t kk = ck[q];
        if ((kk != 0u) & ((top == 31) | ((kk >> (top + 1)) == above)))
          lds_inc(&sm.h2[(kk >> sh) & ((1u << width) - 1u)]);
      }
      __syncthreads();
      const BinHit b = wave_find<256, true>(sm.h2, need);
      need -= b.before;
      fixed |= b.bin << sh;
      cnt = b.cnt;
      // every key of this digit bin is taken: the cut is its lowest key
      if (b.cnt == need) return Cut{0, (fixed >> sh) << sh, kAllPos};
    }
  } else if (cnt == need) {
    return Cut{0, fixed, kAllPos};
  }
  const uint32_t tau = fixed;  // every key bit decided: the tied key
  if (cnt <= 64u) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      if ((ck[q] == tau) & (ck[q] != 0u)) {
        const uint32_t slot = atomicAdd(&sm.tie_n, 1u);
        if (slot < 64u) sm.tie[slot] = (uint32_t)cp[q];
      }
    }
    __syncthreads();
    if (wave_id() == 0) {
      const uint32_t p = lane < (int)cnt ? sm.tie[lane] : 0u;
      uint64_t live = cnt >= 64u ? ~0ull : (1ull << cnt) - 1ull;
#pragma unroll
      for (int b = 16; b >= 0; --b) {
        const uint64_t zeros = __ballot(((p >> b) & 1u) == 0u) & live;
        const uint32_t c0 = (uint32_t)__builtin_popcountll(zeros);
        if (need <= c0) {
          live = zeros;
        } else {
          need -= c0;
          live &= ~zeros;
        }
      }
      const uint32_t pos = read_lane(p, live ? __builtin_ctzll(live) : 0);
      if (lane == 0) sm.bcast[2] = pos;
    }
    __syncthreads();
    return Cut{0, tau, (int32_t)__builtin_amdgcn_readfirstlane(sm.bcast[2])};
  }
  // a large tie class: position digits 16..9, 8..1, 0
  uint32_t pprefix = 0;
  const int pos_shift[3] = {9, 1, 0};
  const int pos_width[3] = {8, 8, 1};
  for (int d = 0; d < 3; ++d) {
    const int sh = pos_shift[d];
    const int wd = pos_width[d];
    __syncthreads();  // the last search's reads of h2 are done
    if (t < 256) sm.h2[t] = 0u;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const uint32_t j = (uint32_t)cp[q];
      if ((ck[q] == tau) & (ck[q] != 0u) & ((j >> (sh + wd)) == pprefix))
        lds_inc(&sm.h2[(j >> sh) & ((1u << wd) - 1u)]);
    }
    __syncthreads();
    const BinHit b = wave_find<256, false>(sm.h2, need);
    need -= b.before;
    pprefix = (pprefix << wd) | b.bin;
  }
  return Cut{0, tau, (int32_t)pprefix};
}

// The register elements that `sel` takes, to the row's output at slots
// taken from the row's output counter (one atomic per call): staged in LDS
// in register order, then mapped and stored in one coalesced pass. The
// histogram space must be free.
template <bool kPaged, int BS, class Src, class Sel>
__device__ __forceinline__ void split_emit(const Src& src, Sel sel, const Emit<kPaged>& em,
                                           int32_t L, uint32_t k, uint32_t* x,
                                           SmemSplitB<BS>& sm) {
  const int lane = lane_id();
  const int w = wave_id();
  const int32_t t = tix();
  uint32_t mine = 0;
  src.for_each([&](uint32_t kk, int32_t j) { mine = add_lane_bit(mine, __ballot(sel(kk, j))); });
  const uint32_t incl = wave_inclusive_sum(mine);
  if (lane == 63) sm.wave_cnt[w] = incl;
  __syncthreads();
  const uint32_t c = lane < BS / 64 ? sm.wave_cnt[lane] : 0u;
  const uint32_t ic = wave_inclusive_sum(c);
  uint32_t slot = incl - mine + (w ? read_lane(ic, w - 1) : 0u);
  const uint32_t total = read_lane(ic, BS / 64 - 1);
  if (t == 0)
    sm.word[5] = total ? __hip_atomic_fetch_add(&x[kXOut], total, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                       : 0u;
  int32_t* stage = reinterpret_cast<int32_t*>(sm.hist);
  src.for_each([&](uint32_t kk, int32_t j) {
    const bool s = sel(kk, j);
    const uint64_t m = __ballot(s);
    if (s & (slot < (uint32_t)kMaxK)) stage[slot] = j;
    slot = add_lane_bit(slot, m);
  });
  __syncthreads();
  const uint32_t base = __builtin_amdgcn_readfirstlane(sm.word[5]);
  auto put = [&](auto value) {
    for (uint32_t i = (uint32_t)t; i < total; i += BS) {
      const int32_t j = stage[i];
      if (((uint32_t)j < (uint32_t)L) & (base + i < k)) em.put((int32_t)(base + i), j, value(j));
    }
  };
  if (kPaged && em.staged)
    put([&](int32_t j) { return em.value_lds(j, sm.pt); });
  else
    put([&](int32_t j) { return em.value(j); });
  __syncthreads();  // the stage and wave_cnt are free again
}

// The winners of a segment (keys above the threshold bin T) to the row's
// output, and the bin's elements (the candidates) to the row's candidate
// buffer: one counting pass for both, and one 64-bit atomic on the words
// kXOut (output slots, low half) and kXOut + 1 (candidate slots, high half)
// takes both ranges. The winners go through the LDS stage as in
// split_emit; the candidates are stored straight from the registers.
template <bool kPaged, int BS, class Src>
__device__ __forceinline__ void split_emit_cands(const Src& src, uint32_t T,
                                                 const Emit<kPaged>& em, int32_t L, uint32_t k,
                                                 uint32_t* x, SmemSplitB<BS>& sm) {
  const int lane = lane_id();
  const int w = wave_id();
  const int32_t t = tix();
  auto win = [T](uint32_t kk) { return (kk != 0u) & ((kk >> 20) > T); };
  auto cand = [T](uint32_t kk) { return (kk != 0u) & ((kk >> 20) == T); };
  uint32_t mw = 0, mc = 0;
  src.for_each([&](uint32_t kk, int32_t) {
    mw = add_lane_bit(mw, __ballot(win(kk)));
    mc = add_lane_bit(mc, __ballot(cand(kk)));
  });
  const uint32_t iw = wave_inclusive_sum(mw);
  const uint32_t ic = wave_inclusive_sum(mc);
  if (lane == 63) {
    sm.wave_cnt[w] = iw;
    sm.tie[w] = ic;  // (the tie positions' space is free until a resolve)
  }
  __syncthreads();
  const uint32_t cw = lane < BS / 64 ? sm.wave_cnt[lane] : 0u;
  const uint32_t cc = lane < BS / 64 ? sm.tie[lane] : 0u;
  const uint32_t sw = wave_inclusive_sum(cw);
  const uint32_t sc = wave_inclusive_sum(cc);
  uint32_t slot = iw - mw + (w ? read_lane(sw, w - 1) : 0u);
  uint32_t at = ic - mc + (w ? read_lane(sc, w - 1) : 0u);
  const uint32_t tw = read_lane(sw, BS / 64 - 1);
  const uint32_t tc = read_lane(sc, BS / 64 - 1);
  if (t == 0) {
    const uint64_t add = (uint64_t)tw | ((uint64_t)tc << 32);
    const uint64_t got =
        add ? __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(x + kXOut), add,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
            : 0ull;
    sm.word[5] = (uint32_t)got;
    sm.word[6] = (uint32_t)(got >> 32);
  }
  int32_t* stage = reinterpret_cast<int32_t*>(sm.hist);
  src.for_each([&](uint32_t kk, int32_t j) {
    const bool s = win(kk);
    const uint64_t m = __ballot(s);
    if (s & (slot < (uint32_t)kMaxK)) stage[slot] = j;
    slot = add_lane_bit(slot, m);
  });
  __syncthreads();
  const uint32_t base = __builtin_amdgcn_readfirstlane(sm.word[5]);
  at += __builtin_amdgcn_readfirstlane(sm.word[6]);
  uint64_t* gcand = reinterpret_cast<uint64_t*>(x + kXCand);
  // a candidate's emitted value goes with it, so the row's last segment
  // reads it with the pair instead of looking it up after the pair
  auto cand_value = [&](int32_t j) -> int32_t {
    if ((uint32_t)j >= (uint32_t)L) return -1;
    if constexpr (kPaged) return em.staged ? em.value_lds(j, sm.pt) : em.value(j);
    else return em.value(j);
  };
  src.for_each([&](uint32_t kk, int32_t j) {
    const bool s = cand(kk);
    const uint64_t m = __ballot(s);
    if (s & (at < (uint32_t)kCandCapG)) {
      __hip_atomic_store(&gcand[at], ((uint64_t)(uint32_t)j << 32) | kk, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&x[kXVal + at], (uint32_t)cand_value(j), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    at = add_lane_bit(at, m);
  });
  auto put = [&](auto value) {
    for (uint32_t i = (uint32_t)t; i < tw; i += BS) {
      const int32_t j = stage[i];
      if (((uint32_t)j < (uint32_t)L) & (base + i < k)) em.put((int32_t)(base + i), j, value(j));
    }
  };
  if (kPaged && em.staged)
    put([&](int32_t j) { return em.value_lds(j, sm.pt); });
  else
    put([&](int32_t j) { return em.value(j); });
  __syncthreads();  // the stage and wave_cnt are free again
}

// -1 in every output slot of the row (a row whose segments gave up).
template <bool kPaged, int BS>
__device__ __forceinline__ void split_fail_row(const Emit<kPaged>& em, uint32_t k) {
  for (uint32_t i = (uint32_t)tix(); i < k; i += BS) em.put((int32_t)i, -1, -1);
}

// The end of a segment: it counts itself done once its stores have
// completed; the row's last segment to finish resets the counters (and,
// when a segment of the row gave up, writes -1 over the whole row, after
// every other segment's stores, and clears the histogram). A segment that
// gave up writes -1 over the row itself too: if a segment of its row never
// runs, no last segment comes.
template <bool kPaged, int BS>
__device__ __forceinline__ void split_finish(const Emit<kPaged>& em, uint32_t k, uint32_t* x,
                                             int32_t S, bool gave_up, SmemSplitB<BS>& sm) {
  const int32_t t = tix();
  if (gave_up) split_fail_row<kPaged, BS>(em, k);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (t == 0) {
    const uint32_t d =
        __hip_atomic_fetch_add(&x[kXDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.word[0] = d == (uint32_t)S - 1u;
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(sm.word[0]) == 0u) return;
  const bool failed =
      __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(&x[kXFail], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0u;
  if (failed) {
    split_fail_row<kPaged, BS>(em, k);
    for (int32_t i = t; i < kXCand; i += BS)
      __hip_atomic_store(&x[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int32_t i = kXFlag + t; i < kXWords; i += BS)
    __hip_atomic_store(&x[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One segment of a split row (SEG = NV * 4 * 512 floats) in the register
// kernel. The segment sits in registers like a short row. Round 1 merges
// the level-1 histogram over the row; every segment then emits its keys
// above the threshold bin at once (winners). When the bin's elements of the
// whole row fit the candidate buffer (kCandCapG), each segment writes its
// own there, arrives and leaves, and the last to arrive resolves the exact
// cut among them and emits the winners of the bin: no segment waits after
// round 1. A larger bin takes one more merged round per further digit (12
// and 8 key bits, 12 and 5 position bits), after which each segment emits
// its winners of the bin. Output slots come from the row's shared counter.
template <bool kPaged, int NV>
__device__ __forceinline__ void split_segment(const Params& p, int64_t b, const RowMeta& m,
                                              int32_t seg, uint32_t* x, uint32_t spin,
                                              SmemSplitB<kBigBlock>& sm) {
  constexpr int BS = kBigBlock;
  constexpr int SEG = NV * 4 * BS;
  const RowInfo& r = m.r;
  const int32_t t = tix();
  const int lane = lane_id();
  const uint32_t k = (uint32_t)p.k;
  const int32_t S = m.nseg;
  const SplitSync sy{x, S, p.plan + kPlanWordError, spin, sm.word};
  const int32_t rem = r.s & 3;
  const float4* base4 = reinterpret_cast<const float4*>(p.scores + b * p.stride + (r.s - rem));
  const int32_t nvec = (r.span + 3) >> 2;
  const int32_t v0 = seg * (SEG / 4);  // first aligned vector of the segment
  Emit<kPaged> em = row_emit<kPaged>(p, b, m);
  uint32_t key[NV][4];
  {
    float4 xv[NV];
    load_vectors<NV, BS>(base4, nvec, v0, xv);
    const int32_t j0 = v0 * 4 - rem;
    const int32_t j1 = j0 + SEG < r.L ? j0 + SEG : r.L;
    em.stage_table_range(sm.pt, j0, j1);
    clear_bins<kBins, BS>(sm.hist);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int32_t v = v0 + i * BS + t;
#pragma unroll
      for (int c = 0; c < 4; ++c) key[i][c] = order_key(lane_of(xv[i], c));
      if ((v == 0) | (v * 4 + 4 > r.span)) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int32_t a = v * 4 + c;
          if ((a < rem) | (a >= r.span)) key[i][c] = 0u;
        }
      }
    }
  }
  const RegSrc<NV, BS> src{key, v0 * 4 - rem, NV - 1};
  __syncthreads();
  {
    const uint32_t one = opaque_one();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (v0 + i * BS + t < nvec) {
#pragma unroll
        for (int c = 0; c < 4; ++c) lds_add(&sm.hist[key[i][c] >> 20], one);
      }
    }
  }
  uint32_t round = 1;
  BinHit h;
  bool ok =
      histogram_round<kBins, true, BS>(sm.hist, x + kXHist, round++, k, kCandCapG, sy, sm, h);
  if (ok) {
    uint32_t need = k - h.before;
    const uint32_t T = h.bin;
    const bool whole = h.cnt == need;
    if (!whole && h.cnt <= (uint32_t)kCandCapG) {
      // the winners above the bin to the output and the bin's elements to
      // the row's candidate buffer
      split_emit_cands<kPaged, BS>(src, T, em, r.L, k, x, sm);
      if (sy.arrive(round++)) {
        // the last segment: every candidate is in; resolve and emit them
        const uint32_t n = h.cnt;
        const uint64_t* gcand = reinterpret_cast<const uint64_t*>(x + kXCand);
        // Each thread's candidates (i = t + q BS) and their emitted values
        // in registers (the values' loads land during the resolve).
        constexpr int kCandPer = kCandCapG / BS;
        uint32_t ck[kCandPer];
        int32_t cp[kCandPer];
        int32_t cval[kCandPer];
#pragma unroll
        for (int q = 0; q < kCandPer; ++q) {
          const uint32_t i = (uint32_t)(q * BS + t);
          ck[q] = 0u;
          cp[q] = -1;
          cval[q] = 0;
          if (i < n) {
            const uint64_t e =
                __hip_atomic_load(&gcand[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ck[q] = (uint32_t)e;
            cp[q] = (int32_t)(e >> 32);
            cval[q] = (int32_t)__hip_atomic_load(&x[kXVal + i], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        // Every segment of the row has arrived, so none gave up: this one
        // counts itself done now (issued after its loads, so their waits do
        // not wait for it) and reads the count at the end, the round trip
        // hidden behind the resolve. Nothing after this touches the words
        // a last finisher resets.
        uint32_t done_prev = 0u;
        if (t == 0)
          done_prev =
              __hip_atomic_fetch_add(&x[kXDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (t == 0) sm.word[6] = 0u;  // published by the resolve's barriers
        const Cut cut = resolve_pairs_regs<BS, kCandPer>(ck, cp, n, need, sm);
        // the segments' winners above the bin number h.before (the merged
        // count): they took slots [0, h.before), the bin's take the rest.
        // One LDS atomic per wave takes the wave's slots.
        const uint32_t base = h.before;
        uint64_t ms[kCandPer];
        uint32_t wtot = 0;
#pragma unroll
        for (int q = 0; q < kCandPer; ++q) {
          ms[q] = __ballot(is_selected(cut, ck[q], cp[q]));
          wtot += (uint32_t)__builtin_popcountll(ms[q]);
        }
        if (wtot) {
          uint32_t wb = 0;
          if (lane == 0) wb = atomicAdd(&sm.word[6], wtot);
          wb = read_lane(wb, 0);
#pragma unroll
          for (int q = 0; q < kCandPer; ++q) {
            const uint64_t mm = ms[q];
            const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(mm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mm, wb));
            const int32_t j = cp[q];
            if (((mm >> lane) & 1ull) & (slot < need) & ((uint32_t)j < (uint32_t)r.L) &
                (base + slot < k))
              em.put((int32_t)(base + slot), j, cval[q]);
            wb += (uint32_t)__builtin_popcountll(mm);
          }
        }
        if (t == 0) sm.word[0] = done_prev == (uint32_t)S - 1u;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(sm.word[0]) != 0u) {
          // the row's last segment to finish: reset the counters
          for (int32_t i = kXFlag + t; i < kXWords; i += BS)
            __hip_atomic_store(&x[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;  // counted done above
      }
    } else {
      // the winners above the threshold bin (with it, when it is taken whole)
      split_emit<kPaged, BS>(
          src,
          [T, whole](uint32_t kk, int32_t) {
            const uint32_t d = kk >> 20;
            return (kk != 0u) & ((d > T) | (whole & (d == T)));
          },
          em, r.L, k, x, sm);
    }
    if (!whole && h.cnt > (uint32_t)kCandCapG) {
      // The bin is too large for the buffer: one merged round per digit.
      clear_bins<kBins, BS>(sm.hist);
      __syncthreads();
      {
        src.for_each([&](uint32_t kk, int32_t) {
          if ((kk != 0u) & ((kk >> 20) == T)) lds_inc(&sm.hist[(kk >> 8) & 0xfffu]);
        });
      }
      ok = histogram_round<kBins, true, BS>(sm.hist, x + kXHist, round++, need, 0u, sy, sm,
                                            h);
      Cut cut{8, (T << 12) | h.bin, kAllPos};
      need -= h.before;
      if (ok && h.cnt != need) {
        if (t < 256) sm.h2[t] = 0u;
        __syncthreads();
        {
          const uint32_t pre = cut.prefix;
          src.for_each([&](uint32_t kk, int32_t) {
            if ((kk != 0u) & ((kk >> 8) == pre)) lds_inc(&sm.h2[kk & 0xffu]);
          });
        }
        ok = histogram_round<256, true, BS>(sm.h2, x + kXHist, round++, need, 0u, sy, sm, h);
        cut = Cut{0, (cut.prefix << 8) | h.bin, kAllPos};
        need -= h.before;
        if (ok && h.cnt != need) {
          const uint32_t tau = cut.prefix;
          clear_bins<kBins, BS>(sm.hist);
          __syncthreads();
          src.for_each([&](uint32_t kk, int32_t j) {
            if ((kk == tau) & (j >= 0)) lds_inc(&sm.hist[(uint32_t)j >> 5]);
          });
          ok = histogram_round<kBins, false, BS>(sm.hist, x + kXHist, round++, need, 0u, sy,
                                                 sm, h);
          need -= h.before;
          const uint32_t hi = h.bin;
          if (ok) {
            if (t < 256) sm.h2[t] = 0u;
            __syncthreads();
            src.for_each([&](uint32_t kk, int32_t j) {
              if ((kk == tau) & (j >= 0) & (((uint32_t)j >> 5) == hi))
                lds_inc(&sm.h2[(uint32_t)j & 31u]);
            });
            ok = histogram_round<32, false, BS>(sm.h2, x + kXHist, round++, need, 0u, sy, sm,
                                               h);
            cut.pos = (int32_t)((hi << 5) | h.bin);
          }
        }
      }
      if (ok) {
        __syncthreads();  // the last searches' reads of the histogram are done
        split_emit<kPaged, BS>(
            src,
            [T, cut](uint32_t kk, int32_t j) {
              return ((kk >> 20) == T) & is_selected(cut, kk, j);
            },
            em, r.L, k, x, sm);
      }
    }
  }
  split_finish<kPaged, BS>(em, k, x, S, !ok, sm);
}

// The split workers of the register kernel: worker w serves work items w,
// w + W, ... (W workers, the first workgroups of the grid).
template <bool kPaged>
__device__ __forceinline__ void split_worker(const Params& p, SmemSplitB<kBigBlock>& sm) {
  if (!p.plan) return;
  int32_t* plan = p.plan;
  const int64_t R = p.num_rows;
  const int64_t cap_items = plan_split_cap(R) * kMaxSeg;
  // the header words in one round trip
  const int32_t pm = __builtin_amdgcn_readfirstlane(ld_const(plan + kPlanWordMagic));
  const int32_t pr = __builtin_amdgcn_readfirstlane(ld_const(plan + kPlanWordRows));
  const int32_t ni = __builtin_amdgcn_readfirstlane(ld_const(plan + kPlanWordItems));
  const int32_t sp = __builtin_amdgcn_readfirstlane(ld_const(plan + kPlanWordSpin));
  if (pm != kPlanMagic || pr != p.num_rows) return;
  const uint32_t n_items = (uint32_t)(ni < 0 ? 0 : (ni > cap_items ? cap_items : ni));
  const uint32_t spin = sp > 0 ? (uint32_t)sp : kSpinLimit;
  const int32_t* items = plan + plan_items_word(R);
  for (uint32_t it = blockIdx.x; it < n_items; it += (uint32_t)p.workers) {
    const int64_t b = __builtin_amdgcn_readfirstlane(ld_const(items + 2 * it));
    const int32_t seg = __builtin_amdgcn_readfirstlane(ld_const(items + 2 * it + 1));
    if ((uint64_t)b < (uint64_t)R) {
      const RowMeta m = row_meta<kPaged>(p, b, true);
      if (m.split && seg >= 0 && seg < m.nseg) {
        uint32_t* x =
            reinterpret_cast<uint32_t*>(plan + plan_xarea_word(R) + (int64_t)m.slot * kXWords);
        if (m.seg_len == kSegShort)
          split_segment<kPaged, kSegShort / (4 * kBigBlock)>(p, b, m, seg, x, spin, sm);
        else
          split_segment<kPaged, kSegLong / (4 * kBigBlock)>(p, b, m, seg, x, spin, sm);
      }
    }
    __syncthreads();  // the next item reuses the LDS
  }
}

// Every row of a batch with a score stride above 16384 floats, in one
// launch (a launch costs about 1.6 us even when its workgroups have
// nothing to do): 512 threads per row, holding 4, 8 or 16 float4 each by
// the row's span, or a long row in pieces of 16 float4 per thread. At 80
// VGPRs three rows share a CU, so one row's searches overlap the others'
// loads (for spans above 16384, two rows of 1024 threads with 8 float4
// each ran 10-50% slower). With a plan, the first p.workers workgroups are
// the split workers.
template <bool kPaged>
__global__ __launch_bounds__(kBigBlock) __attribute__((amdgpu_waves_per_eu(6))) void
rows_reg_kernel(const Params p) {
  __shared__ union {
    SmemRegB<kBigBlock> reg;
    SmemRegL<kBigBlock, kBigLds> regl;
    SmemSplitB<kBigBlock> split;
    SmemPieces pieces;
    SmemStream two;
  } sm;
  if ((int32_t)blockIdx.x < p.workers) {
    split_worker<kPaged>(p, sm.split);
    return;
  }
  int64_t b = (int64_t)blockIdx.x - p.workers;
  if (p.ordered) {
    // The plan lists the rows by class, shortest class first: read from the
    // end, the longest rows start first and the last workgroups to be
    // dispatched (after the split workers free their slots) serve short
    // and trivial rows. A plan of another batch size leaves the order as
    // it is.
    const int32_t R = p.num_rows;
    const int32_t pm = __builtin_amdgcn_readfirstlane(ld_const(p.plan + kPlanWordMagic));
    const int32_t pr = __builtin_amdgcn_readfirstlane(ld_const(p.plan + kPlanWordRows));
    const int32_t e = __builtin_amdgcn_readfirstlane(
        ld_const(p.plan + kPlanHeaderWords + (R - 1 - (int32_t)b)));
    if (pm == kPlanMagic && pr == R && (uint32_t)e < (uint32_t)R) b = e;
  }
  const RowMeta m = row_meta<kPaged>(p, b, true);
  const RowInfo& r = m.r;
  // long rows: the split workers', or without a plan the long-row kernel's
  if (r.cls == kClassLong && (m.split || p.long_mode == kLongPerRow)) return;
  const Emit<kPaged> em = row_emit<kPaged>(p, b, m);
  if (r.L <= p.k) {
    write_trivial<kPaged, kBigBlock>(em, r.L, p.k);
    return;
  }
  const RowView rv = row_view(p, b, r);
  if (r.span <= kBigVec * kBigBlock) {
    row_in_registers<kBigVec / 4, kPaged, kBigBlock>(rv, p.k, em, sm.reg);
  } else if (r.span <= kBigVec * 2 * kBigBlock) {
    row_in_registers<kBigVec / 2, kPaged, kBigBlock>(rv, p.k, em, sm.reg);
  } else if (r.span <= kBigVec * 4 * kBigBlock) {
    row_in_registers<kBigVec, kPaged, kBigBlock>(rv, p.k, em, sm.reg);
  } else if (r.span <= kBigCap) {
    row_in_registers_lds<kBigVec, kBigLds, kPaged, kBigBlock>(rv, p.k, em, sm.regl);
  } else if (!row_in_pieces<kPaged>(rv, p.k, em, sm.pieces)) {
    __syncthreads();
    row_streaming<kPaged, kBigBlock>(rv, p.k, em, sm.two);
  }
}

// Long rows up to 65536 floats are register rows of a 1024-thread
// workgroup: 13 float4 per thread in registers (the most that fits the 64
// VGPRs of two workgroups per CU without spills) and 3 in LDS (the 80 KB of
// the streaming path's list hold them); longer ones are streamed.
constexpr int kLongRegVec = 13;
constexpr int kLongLds = 3;
constexpr int kLongRegCap = (kLongRegVec + kLongLds) * 4 * kLongBlock;  // 65536

// Long rows read whole, one 1024-thread workgroup per row of the batch
// (the workgroups of other rows leave at once): from registers up to 65536
// floats, else streamed, each streamed row touching during its final cut
// the opening lines of the row likely to start next.
template <bool kPaged>
__device__ __forceinline__ void long_row(const Params& p, int64_t b, const RowMeta& m,
                                         const Prefetch pf) {
  const RowInfo& r = m.r;
  const Emit<kPaged> em = row_emit<kPaged>(p, b, m);
  __shared__ union {
    SmemS1 one;
    SmemRegB<kLongBlock> fin;
    SmemRegL<kLongBlock, kLongLds> regl;
    SmemStream two;
  } sm;
  const RowView rv = row_view(p, b, r);
  if (r.span <= kLongRegCap) {
    row_in_registers_lds<kLongRegVec, kLongLds, kPaged, kLongBlock>(rv, p.k, em, sm.regl);
    return;
  }
  if (!row_stream1<kPaged, kLongBlock>(rv, p.k, em, sm.one, sm.fin, pf)) {
    __syncthreads();
    row_streaming<kPaged, kLongBlock>(rv, p.k, em, sm.two);
  }
}

template <bool kPaged>
__global__ __launch_bounds__(kLongBlock) __attribute__((amdgpu_waves_per_eu(8))) void
rows_long_kernel(const Params p) {
  // Workgroup g reads row g of the batch; the launch takes no plan. (A
  // persistent grid would launch fewer workgroups, but its loop keeps
  // values the compiler hoists out of it live through the row's body,
  // which spills at the 64 VGPRs of two workgroups per CU.)
  const int64_t b = blockIdx.x;
  const int64_t b2 = b + kPrefetchAhead;  // the row likely to start next on this XCD
  const int32_t R = p.num_rows;
  // the touched row's words, loaded with the row's own
  const bool t2 = (uint64_t)b2 < (uint64_t)R;
  const int32_t* a_l2 = t2 ? p.seq_lens + b2 : p.seq_lens + b;
  const int32_t* a_s2 = (t2 && p.row_starts) ? p.row_starts + b2 : a_l2;
  int32_t l2 = __builtin_amdgcn_readfirstlane(ld_const(a_l2));
  int32_t s2 = __builtin_amdgcn_readfirstlane(ld_const(a_s2));
  const RowMeta m = row_meta<kPaged>(p, b, false);
  asm volatile("" : "+s"(l2), "+s"(s2));
  if (p.long_mode == kLongAll) {
    if (m.r.L <= p.k) {
      write_trivial<kPaged, kLongBlock>(row_emit<kPaged>(p, b, m), m.r.L, p.k);
      return;
    }
  } else if (m.r.cls != kClassLong) {
    return;
  }
  Prefetch pf{nullptr, 0};
  if (t2) {
    const RowInfo r2 = classify(l2, p.row_starts ? s2 : 0, p.k);
    if (r2.cls == kClassLong) {
      const int32_t st2 = p.row_starts ? s2 : 0;
      pf.base = p.scores + b2 * p.stride + (st2 - (st2 & 3));
      pf.bytes = 4 * (r2.span < kS1Depth * kS1Chunk ? r2.span : kS1Depth * kS1Chunk);
    }
  }
  long_row<kPaged>(p, b, m, pf);
}

// Plan: classify every row and list the rows of each class (workgroup 0).
// Workgroups of up to this many threads: a batch of at most that many rows
// takes the least multiple of 64 threads that covers its rows, and at least
// kPlanMinBlock (the exchange areas' zeroing keeps enough threads).
constexpr int kPlanBlock = 1024;
constexpr int kPlanMinBlock = 256;

// Up to this many rows the plan is one launch: its workgroups after the
// first zero the exchange areas, each counting the batch's long rows by
// itself (one row per thread) to learn whether its area is assigned. Larger
// batches zero them in a second launch that reads the count from the plan.
constexpr int kFusedClearRows = kPlanBlock;

// The words of split row q's exchange area that must be zero at the start
// of a call: the histogram and the counters (the candidate pairs are
// written before they are read).
__device__ __forceinline__ void zero_area(int32_t num_rows, int32_t* plan, int32_t q,
                                          int32_t block) {
  int32_t* x = plan + plan_xarea_word(num_rows) + (int64_t)q * kXWords;
  for (int32_t i = tix(); i < kXCand; i += block) x[i] = 0;
  for (int32_t i = kXFlag + tix(); i < kXWords; i += block) x[i] = 0;
}

__global__ __launch_bounds__(kPlanBlock) void plan_kernel(const int32_t* seq_lens,
                                                         const int32_t* row_starts,
                                                         int32_t num_rows, int32_t k,
                                                         int32_t* plan) {
  if (blockIdx.x > 0) {
    // area q of the split rows: the first min(long rows, cap) are assigned
    __shared__ uint32_t n_long;
    if (tix() == 0) n_long = 0;
    __syncthreads();
    const int32_t b = tix();
    const bool lng =
        b < num_rows && row_info(seq_lens, row_starts, k, b).cls == kClassLong;
    const uint64_t m = __ballot(lng);
    if (lane_id() == 0 && m) atomicAdd(&n_long, (uint32_t)__builtin_popcountll(m));
    __syncthreads();
    const int64_t cap = plan_split_cap(num_rows);
    const int32_t q = (int32_t)blockIdx.x - 1;
    if ((int64_t)n_long <= cap && (int64_t)q < (int64_t)n_long)
      zero_area(num_rows, plan, q, (int32_t)blockDim.x);
    return;
  }
  __shared__ uint32_t count[kNumClasses];
  __shared__ uint32_t fill[kNumClasses];
  __shared__ uint32_t n_split;
  __shared__ uint32_t n_items;
  __shared__ uint32_t n_seg_long;  // segments of the long rows at kSegLong floats
  if (tix() < kNumClasses) {
    count[tix()] = 0;
    fill[tix()] = 0;
  }
  if (tix() == 0) {
    n_split = 0;
    n_items = 0;
    n_seg_long = 0;
  }
  __syncthreads();
  int32_t* cls = plan + plan_cls_word(num_rows);
  int32_t* nseg = plan + plan_nseg_word(num_rows);
  int32_t* slot = plan + plan_slot_word(num_rows);
  int32_t* items = plan + plan_items_word(num_rows);
  const uint32_t cap = (uint32_t)plan_split_cap(num_rows);
  // With one row per thread, each thread keeps its row's class in a
  // register for the later passes; otherwise they read it back from the
  // plan (a round trip to L2 after each barrier).
  const int32_t nb = (int32_t)blockDim.x;
  const bool one_each = num_rows <= nb;
  int32_t my_cls = -1;
  for (int32_t b = tix(); b < num_rows; b += nb) {
    const RowInfo r = row_info(seq_lens, row_starts, k, b);
    cls[b] = r.cls;
    my_cls = r.cls;
    atomicAdd(&count[r.cls], 1u);
    if (r.cls == kClassLong) atomicAdd(&n_seg_long, (uint32_t)segments_for(r.span, kSegLong));
  }
  __syncthreads();
  // the long rows are split all (at most cap of them) or none; in short
  // segments when long ones would leave CUs idle
  const bool split = count[kClassLong] <= cap;
  const int32_t seg_len = n_seg_long < (uint32_t)kChipCUs ? kSegShort : kSegLong;
  for (int32_t b = tix(); b < num_rows; b += nb) {
    int32_t S = 0;
    int32_t q = -1;
    if (split && (one_each ? my_cls : cls[b]) == kClassLong) {
      const RowInfo r = row_info(seq_lens, row_starts, k, b);
      S = segments_for(r.span, seg_len);
      q = (int32_t)atomicAdd(&n_split, 1u);
      // a row's segments are consecutive work items
      const uint32_t at = atomicAdd(&n_items, (uint32_t)S);
      for (int32_t sg = 0; sg < S; ++sg) {
        items[2 * (at + sg)] = b;
        items[2 * (at + sg) + 1] = sg;
      }
    }
    nseg[b] = S;
    slot[b] = q;
  }
  __syncthreads();
  uint32_t off[kNumClasses];
  off[0] = 0u;
#pragma unroll
  for (int c = 1; c < kNumClasses; ++c) off[c] = off[c - 1] + count[c - 1];
  int32_t* list = plan + kPlanHeaderWords;
  for (int32_t b = tix(); b < num_rows; b += nb) {
    const int32_t c = one_each ? my_cls : cls[b];
    const uint32_t at = atomicAdd(&fill[c], 1u);
    list[off[c] + at] = b;
  }
  if (tix() == 0) {
    plan[kPlanWordMagic] = kPlanMagic;
    plan[kPlanWordRows] = num_rows;
    plan[kPlanWordK] = k;
    for (int c = 0; c < kNumClasses; ++c) {
      plan[kPlanWordCount + c] = (int32_t)count[c];
      plan[kPlanWordOffset + c] = (int32_t)off[c];
    }
    plan[kPlanWordSplit] = (int32_t)n_split;
    plan[kPlanWordItems] = (int32_t)n_items;
    plan[kPlanWordError] = 0;
    plan[kPlanWordSpin] = 0;
    plan[kPlanWordSegLen] = seg_len;
  }
}

// Zero the exchange areas of the planned split rows (one workgroup each).
__global__ __launch_bounds__(kBlock) void plan_clear_kernel(int32_t num_rows, int32_t* plan) {
  const int32_t q = blockIdx.x;
  if (q >= plan[kPlanWordSplit]) return;
  zero_area(num_rows, plan, q, kBlock);
}

}  // namespace dsatopk

using namespace dsatopk;

namespace {

bool is_pow2(int64_t v) { return v >= 1 && (v & (v - 1)) == 0; }

int log2_exact(int64_t v) {
  int b = 0;
  while ((int64_t(1) << b) < v) ++b;
  return b;
}

int check_common(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                 int32_t num_rows, int32_t k, const int32_t* out, const void* plan,
                 size_t plan_bytes) {
  if (k < 1 || k > DSATOPK_MAX_K || num_rows < 0) return DSATOPK_ERR_INVALID_ARG;
  if (num_rows == 0) return DSATOPK_OK;
  if (!scores || !seq_lens || !out || score_stride < 1) return DSATOPK_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(scores) & 15u) != 0 || (score_stride & 3) != 0)
    return DSATOPK_ERR_ALIGNMENT;
  if (plan && (reinterpret_cast<uintptr_t>(plan) & 15u) != 0) return DSATOPK_ERR_ALIGNMENT;
  if (plan && plan_bytes < dsatopk_plan_bytes(num_rows)) return DSATOPK_ERR_PLAN_TOO_SMALL;
  return DSATOPK_OK;
}

// Up to this many rows, short rows use 1024 threads each: with fewer rows
// than about two per CU, per-row latency sets the time.
constexpr int32_t kWideRows = 512;

// From this many rows, a batch whose stride admits long rows but no row
// beyond 1024 threads' registers (40961 .. 65536 floats) runs in the
// long-row kernel alone, every row in one workgroup. The register kernel's
// launch would otherwise cost one workgroup per row even where the long
// rows are all of the batch (13 us of 235 at 5462 rows of 49152 floats;
// the long rows took 223). Rows of 40960 floats and less then run at 1024
// threads instead of 512, and long rows are not split: a smaller batch
// (few long rows among many short ones: 300 rows at 20 us split, 29 us
// whole) keeps the split path.
constexpr int32_t kLongAllRows = 1024;
// ... and, with a plan, for strides up to this. Longer rows hold more of
// their span in the long kernel's LDS slices and cut and stage over more
// keys: from 61440 columns the register kernel's pieces (three rows per
// CU) take less time (rows of 57344 / 61440 / 65536 floats, 1 GiB of
// scores per launch: 213 / 217 / 220 us in the long kernel, 219 / 212 /
// 208 us in pieces; at 49152, 214 against 219).
constexpr int64_t kLongAllStride = 57344;

// Up to this many rows, a register kernel launch with a plan serves the
// rows in the plan's class order, longest first: in a small batch of
// mixed lengths the rows that start last set the launch's end, and with
// split rows those start only when the split workers free their slots
// (512 rows of log-uniform lengths up to 131072: 27.2 -> 23.9 us). The
// order costs each row one more scalar round trip; larger batches keep the
// plain order.
constexpr int32_t kOrderedRows = 1024;

struct KernelLaunch {
  void (*fn)(Params);
  dim3 grid;
  dim3 block;
};

// The kernels for a batch, in stream order, chosen by the score stride (a
// row's span never exceeds it). Up to 8192 floats every row is short: the
// short-row kernel (or the wide one, for few rows) serves the batch alone;
// up to 16384 the mid kernel alone; up to 40960 the register kernel alone;
// from kLongAllRows rows, up to kLongAllStride (without a plan, up to
// 65536) the long-row kernel alone (the plan is not used). Other strides: the register kernel, whose first
// workgroups are the split workers when a plan is given and which then
// also reads the long rows that are not split, in pieces; without a plan
// the long-row kernel follows it for the long rows (many long rows of
// 98304 or 131072 floats, 1 GiB per launch: 215 / 211 us with the
// long-row kernel's 1024-thread streamed rows, 199 / 198 us in pieces).
// Each launch reports its own status.
template <bool kPaged>
int launch_rows(Params p, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_rows);
  const bool lng = p.stride > (int64_t)kBigCap;
  if (!lng) p.plan = nullptr;
  p.workers = 0;
  p.ordered = 0;
  p.long_mode = p.plan ? kLongInPieces : kLongPerRow;
  KernelLaunch ls[2];
  int n = 0;
  if (p.stride <= (int64_t)kSmallVec * 4 * kBlock) {
    if (p.num_rows <= kWideRows)
      ls[n++] = {rows_wide_kernel<kPaged>, grid, dim3(kWideBlock)};
    else
      ls[n++] = {rows_short_kernel<kPaged>, grid, dim3(kBlock)};
  } else if (p.stride <= (int64_t)kLargeVec * 4 * kBlock) {
    ls[n++] = {rows_mid_kernel<kPaged>, grid, dim3(kBlock)};
  } else if (lng && p.num_rows >= kLongAllRows &&
             p.stride <= (p.plan ? kLongAllStride : (int64_t)kLongRegCap)) {
    p.plan = nullptr;
    p.long_mode = kLongAll;
    ls[n++] = {rows_long_kernel<kPaged>, grid, dim3(kLongBlock)};
  } else {
    if (p.plan) {
      const int64_t w = plan_split_cap(p.num_rows) * kMaxSeg;
      p.workers = (int32_t)(w < kMaxWorkers ? w : kMaxWorkers);
      p.ordered = p.num_rows <= kOrderedRows;
    }
    ls[n++] = {rows_reg_kernel<kPaged>, dim3((unsigned)(p.workers + p.num_rows)),
               dim3(kBigBlock)};
    if (lng && p.long_mode != kLongInPieces)
      ls[n++] = {rows_long_kernel<kPaged>, grid, dim3(kLongBlock)};
  }
  for (int i = 0; i < n; ++i) {
    void* args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void*>(ls[i].fn), ls[i].grid, ls[i].block, args, 0,
                        stream) != hipSuccess)
      return DSATOPK_ERR_HIP;
  }
  return DSATOPK_OK;
}

// The plan of dsatopk_paged_noalloc: a file-scope device array (each GPU
// that loads the library holds its own copy until the process ends). Host
// code never uses its name as an address: the address comes from
// hipGetSymbolAddress, once per device with that device current.
constexpr size_t kNoAllocBytes = size_t(16) << 20;
static_assert((size_t)plan_words(DSATOPK_NOALLOC_MAX_ROWS) * sizeof(int32_t) <= kNoAllocBytes,
              "the largest accepted batch's plan fits the static scratch");
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address (found on the first call there).
int noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSATOPK_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSATOPK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return DSATOPK_OK;
}

}  // namespace

extern "C" {

const char* dsatopk_status_string(int status) {
  switch (status) {
    case DSATOPK_OK: return "ok";
    case DSATOPK_ERR_INVALID_ARG: return "invalid argument";
    case DSATOPK_ERR_ALIGNMENT: return "scores not 16-byte aligned or stride not a multiple of 4";
    case DSATOPK_ERR_PLAN_TOO_SMALL: return "plan buffer too small";
    case DSATOPK_ERR_HIP: return "HIP runtime error";
    case DSATOPK_ERR_TOO_LARGE:
      return "num_rows above DSATOPK_NOALLOC_MAX_ROWS (the static scratch of dsatopk_paged_noalloc)";
    default: return "unknown status";
  }
}

size_t dsatopk_plan_bytes(int32_t num_rows) {
  if (num_rows < 0) return 0;
  return sizeof(int32_t) * (size_t)plan_words(num_rows);
}

int dsatopk_plan(const int32_t* seq_lens, const int32_t* row_starts, int32_t num_rows, int32_t k,
                 void* plan, size_t plan_bytes, void* stream) {
  if (num_rows < 0 || k < 1 || k > DSATOPK_MAX_K) return DSATOPK_ERR_INVALID_ARG;
  if (num_rows == 0) return DSATOPK_OK;
  if (!seq_lens || !plan) return DSATOPK_ERR_INVALID_ARG;
  if (plan_bytes < dsatopk_plan_bytes(num_rows)) return DSATOPK_ERR_PLAN_TOO_SMALL;
  if ((reinterpret_cast<uintptr_t>(plan) & 15u) != 0) return DSATOPK_ERR_ALIGNMENT;
  const int64_t cap = plan_split_cap(num_rows);
  const bool fused = num_rows <= kFusedClearRows;
  // a fused launch's counting workgroups need a thread per row
  const int32_t cover = (num_rows + 63) / 64 * 64;
  const int32_t pb = !fused ? kPlanBlock : (cover < kPlanMinBlock ? kPlanMinBlock : cover);
  int32_t* pl = static_cast<int32_t*>(plan);
  {
    void* args[] = {&seq_lens, &row_starts, &num_rows, &k, &pl};
    if (hipLaunchKernel(reinterpret_cast<const void*>(plan_kernel),
                        dim3(fused ? (unsigned)(1 + cap) : 1u), dim3((unsigned)pb), args, 0,
                        (hipStream_t)stream) != hipSuccess)
      return DSATOPK_ERR_HIP;
  }
  if (!fused) {
    void* args[] = {&num_rows, &pl};
    if (hipLaunchKernel(reinterpret_cast<const void*>(plan_clear_kernel), dim3((unsigned)cap),
                        dim3(kBlock), args, 0, (hipStream_t)stream) != hipSuccess)
      return DSATOPK_ERR_HIP;
  }
  return DSATOPK_OK;
}

int dsatopk_plan_error(const void* plan, size_t plan_bytes, int32_t* error, void* stream) {
  if (!plan || !error) return DSATOPK_ERR_INVALID_ARG;
  if (plan_bytes < (size_t)kPlanHeaderWords * sizeof(int32_t)) return DSATOPK_ERR_PLAN_TOO_SMALL;
  int32_t w = 0;
  if (hipMemcpyAsync(&w, static_cast<const int32_t*>(plan) + kPlanWordError, sizeof(w),
                     hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
      hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return DSATOPK_ERR_HIP;
  *error = w;
  return DSATOPK_OK;
}

int dsatopk_paged(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                  const int32_t* row_starts, const int32_t* page_table,
                  int64_t page_table_stride, int32_t page_size, int32_t num_rows, int32_t k,
                  void* plan, size_t plan_bytes, int32_t* out, void* stream) {
  return dsatopk_paged_packed(scores, score_stride, seq_lens, row_starts, page_table,
                              page_table_stride, page_size, nullptr, nullptr, num_rows, k, plan,
                              plan_bytes, out, nullptr, stream);
}

int dsatopk_paged_packed(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                         const int32_t* row_starts, const int32_t* page_table,
                         int64_t page_table_stride, int32_t page_size,
                         const int32_t* table_rows, const int32_t* table_starts,
                         int32_t num_rows, int32_t k, void* plan, size_t plan_bytes,
                         int32_t* out, int32_t* out_raw, void* stream) {
  int st = check_common(scores, score_stride, seq_lens, num_rows, k, out, plan, plan_bytes);
  if (st != DSATOPK_OK || num_rows == 0) return st;
  if (!page_table || page_table_stride < 1 || !is_pow2(page_size) || page_size > (1 << 20))
    return DSATOPK_ERR_INVALID_ARG;
  Params p{};
  p.scores = scores;
  p.stride = score_stride;
  p.seq_lens = seq_lens;
  p.row_starts = row_starts;
  p.out_offsets = nullptr;
  p.page_table = page_table;
  p.pt_stride = page_table_stride;
  p.page_bits = log2_exact(page_size);
  p.num_rows = num_rows;
  p.k = k;
  p.out = out;
  p.plan = (int32_t*)plan;
  p.table_rows = table_rows;
  p.table_starts = table_starts;
  p.out_raw = out_raw;
  return launch_rows<true>(p, (hipStream_t)stream);
}

int dsatopk_ragged(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                   const int32_t* row_starts, const int32_t* out_offsets, int32_t num_rows,
                   int32_t k, void* plan, size_t plan_bytes, int32_t* out, void* stream) {
  int st = check_common(scores, score_stride, seq_lens, num_rows, k, out, plan, plan_bytes);
  if (st != DSATOPK_OK || num_rows == 0) return st;
  if (!out_offsets) return DSATOPK_ERR_INVALID_ARG;
  Params p{};
  p.scores = scores;
  p.stride = score_stride;
  p.seq_lens = seq_lens;
  p.row_starts = row_starts;
  p.out_offsets = out_offsets;
  p.page_table = nullptr;
  p.pt_stride = 0;
  p.page_bits = 0;
  p.num_rows = num_rows;
  p.k = k;
  p.out = out;
  p.plan = (int32_t*)plan;
  return launch_rows<false>(p, (hipStream_t)stream);
}

int dsatopk_paged_noalloc(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                          const int32_t* row_starts, const int32_t* page_table,
                          int64_t page_table_stride, int32_t page_size, int32_t num_rows,
                          int32_t k, int32_t* out, void* stream) {
  if (num_rows > DSATOPK_NOALLOC_MAX_ROWS) return DSATOPK_ERR_TOO_LARGE;
  int st = check_common(scores, score_stride, seq_lens, num_rows, k, out, nullptr, 0);
  if (st != DSATOPK_OK || num_rows == 0) return st;
  if (!page_table || page_table_stride < 1 || !is_pow2(page_size) || page_size > (1 << 20))
    return DSATOPK_ERR_INVALID_ARG;
  void* plan = nullptr;
  st = noalloc_scratch(&plan);
  if (st != DSATOPK_OK) return st;
  const size_t bytes = dsatopk_plan_bytes(num_rows);
  st = dsatopk_plan(seq_lens, row_starts, num_rows, k, plan, bytes, stream);
  if (st != DSATOPK_OK) return st;
  return dsatopk_paged(scores, score_stride, seq_lens, row_starts, page_table, page_table_stride,
                       page_size, num_rows, k, plan, bytes, out, stream);
}

}  // extern "C"
