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
// Work decomposition: one 512-thread workgroup per row. By the row's
// aligned span (seq_len plus the row start's residue mod 4) the workgroup
// takes one of
//   - the trivial path (seq_len <= k): writes positions, reads no score;
//   - a register path: the whole span is loaded once with 16-byte loads
//     into registers as keys (up to 8192 or 18432 floats), every later
//     pass runs over registers;
//   - a streaming path for longer spans: pass 1 builds the level-1
//     histogram from global memory; pass 2 re-reads the span, writes the
//     elements above the threshold bin straight to the output stage and
//     collects the threshold bin's elements in LDS, where the remaining
//     digits are resolved. If that bin holds more than the LDS candidate
//     capacity, the remaining digits re-read the span instead.
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

#include "dsatopk.h"
#include "select_device.h"

namespace dsatopk {

constexpr int kSmallVec = 8;          // float4 per thread: 8192-float spans
constexpr int kLargeVec = 16;         // float4 per thread: 16384-float spans
constexpr int kStreamVec = 8;         // float4 per thread per streaming chunk
constexpr int kStreamCandCap = 2048;  // streaming path: threshold-bin pairs in LDS
constexpr int kPtCap = 512;           // page-table entries staged in LDS

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
  const int32_t* plan;  // plan words (header, class lists, classes) or null
};

// Row classes by aligned span. A row's class is recomputed by every kernel
// from the current seq_lens / row_starts; the plan only packs the rows of a
// class into the first workgroups of that class's launch.
enum RowClass : int32_t { kClassShort = 0, kClassMid = 1, kClassLong = 2 };

// Plan layout (int32 words): header, then the rows of each class
// (segments in class order), then each row's class at planning time.
constexpr int kPlanMagic = 0x44534b32;  // "DSK2"
constexpr int kPlanHeaderWords = 64;
enum PlanWord : int32_t {
  kPlanWordMagic = 0,
  kPlanWordRows = 1,
  kPlanWordK = 2,
  kPlanWordCount = 4,   // [3] rows per class
  kPlanWordOffset = 8,  // [3] first list index per class
};

// Output of one row: window position j -> emitted value. In PAGED mode the
// row's page-table entries may be staged in LDS first (short windows).
template <bool kPaged>
struct Emit {
  int32_t* out;
  const int32_t* pt;      // the row's page-table entries (global)
  const int32_t* pt_lds;  // staged copy, or null
  int32_t page_bits;
  int32_t offset;

  __device__ __forceinline__ int32_t value(int32_t j) const {
    if constexpr (kPaged) {
      const int32_t e = j >> page_bits;
      const int32_t page = pt_lds ? pt_lds[e] : pt[e];
      return (int32_t)(((uint32_t)page << page_bits) | ((uint32_t)j & ((1u << page_bits) - 1u)));
    } else {
      return j + offset;
    }
  }

  // Stage the first ceil(L / page_size) table entries into `lds` when they
  // fit; issued early so the loads overlap the score loads.
  __device__ __forceinline__ void stage_table(int32_t* lds, int32_t L) {
    if constexpr (kPaged) {
      const int32_t n = (int32_t)(((uint32_t)L + (1u << page_bits) - 1u) >> page_bits);
      if (n <= kPtCap) {
        for (int32_t e = threadIdx.x; e < n; e += kBlock) lds[e] = pt[e];
        pt_lds = lds;
      }
    }
  }
};

// Shared memory of the register path.
static_assert(kMaxK + kBlock <= kBins, "output stage and its dummies fit the histogram");

struct SmemReg {
  uint32_t hist[kBins];       // level-1 histogram; position digits; finally the output stage
  uint32_t h2[256];           // key bits 19..12 inside the level-1 bin
  uint32_t h3[256];           // key bits 11..4
  uint32_t h4[16];            // key bits 3..0
  int32_t pt[kPtCap];         // the row's page-table entries (PAGED)
  uint32_t wave_cnt[kWaves];  // per wave: selected elements
};

// Shared memory of the streaming path.
struct SmemStream {
  uint32_t hist[kBins];
  int32_t stage[kMaxK];
  uint2 cand[kStreamCandCap];
  uint32_t nstage;
  uint32_t ncand;
};

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
template <int NV>
struct RegSrc {
  const uint32_t (&key)[NV][4];
  int32_t rem;

  // Positions are rebuilt from one opaque base in every pass: the compiler
  // cannot keep NV * 4 position registers alive across passes.
  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    int32_t base = (int32_t)threadIdx.x * 4 - rem;
    asm volatile("" : "+v"(base));
#pragma unroll
    for (int i = 0; i < NV; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) f(key[i][c], base + i * kBlock * 4 + c);
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
struct StreamSrc {
  RowView rv;

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int32_t nvec = (rv.span + 3) >> 2;
    for (int32_t v0 = 0; v0 < nvec; v0 += kBlock * kStreamVec) {
      float4 x[kStreamVec];
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u) {
        const int32_t v = v0 + u * kBlock + (int32_t)threadIdx.x;
        x[u] = v < nvec ? rv.base4[v] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kStreamVec; ++u) {
        const int32_t a0 = (v0 + u * kBlock + (int32_t)threadIdx.x) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) f(key_at(lane_of(x[u], c), a0 + c, rv), a0 + c - rv.rem);
      }
    }
  }
};

template <bool kPaged>
__device__ __forceinline__ void write_trivial(const Emit<kPaged>& em, int32_t L, int32_t k) {
  for (int32_t t = threadIdx.x; t < k; t += kBlock) em.out[t] = t < L ? em.value(t) : -1;
}

// Final coalesced store of the k staged positions. A position outside
// [0, L) cannot come out of a correct cut; it is written as -1 rather than
// used to index the page table.
// Fully unrolled (k <= kMaxK) with unconditional loads, so the stage and
// page-table lookups of all iterations are in flight together.
template <bool kPaged>
__device__ __forceinline__ void write_stage(const Emit<kPaged>& em, const int32_t* stage,
                                            int32_t L, int32_t k) {
  static_assert(kMaxK % kBlock == 0, "whole iterations");
#pragma unroll
  for (int i = 0; i < kMaxK / kBlock; ++i) {
    const int32_t t = i * kBlock + (int32_t)threadIdx.x;
    const int32_t j = stage[t];
    const bool ok = (j >= 0) & (j < L);
    const int32_t v = em.value(ok ? j : 0);
    if (t < k) em.out[t] = ok ? v : -1;
  }
}

// The cut of a register-resident row. Level 1 (key bits 31..20) was
// histogrammed into sm.hist by the caller. The remaining key digits are 8,
// 8 and 4 bits wide: their histograms are small, cleared when the row was
// loaded, and each level costs one filtered pass over the registers, one
// barrier and a 256-bin search. Ties at the k-th key take two position
// digits in sm.hist (rare). Every wave computes every bin itself.
template <class Src>
__device__ __forceinline__ Cut refine_in_registers(const Src& src, SmemReg& sm, uint32_t k) {
  BinHit h = wave_find<kBins, true>(sm.hist, k);
  uint32_t need = k - h.before;
  uint32_t prefix = h.bin;  // key bits 31..20
  if (h.cnt == need) return Cut{20, prefix, kAllPos};
  {
    const uint32_t p = prefix;
    src.for_each([&](uint32_t kk, int32_t) {
      if ((kk >> 20) == p) lds_inc(&sm.h2[(kk >> 12) & 0xffu]);
    });
  }
  __syncthreads();
  h = wave_find<256, true>(sm.h2, need);
  need -= h.before;
  prefix = (prefix << 8) | h.bin;  // bits 31..12
  if (h.cnt == need) return Cut{12, prefix, kAllPos};
  {
    const uint32_t p = prefix;
    src.for_each([&](uint32_t kk, int32_t) {
      if ((kk >> 12) == p) lds_inc(&sm.h3[(kk >> 4) & 0xffu]);
    });
  }
  __syncthreads();
  h = wave_find<256, true>(sm.h3, need);
  need -= h.before;
  prefix = (prefix << 8) | h.bin;  // bits 31..4
  if (h.cnt == need) return Cut{4, prefix, kAllPos};
  {
    const uint32_t p = prefix;
    src.for_each([&](uint32_t kk, int32_t) {
      if ((kk >> 4) == p) lds_inc(&sm.h4[kk & 0xfu]);
    });
  }
  __syncthreads();
  h = wave_find<16, true>(sm.h4, need);
  need -= h.before;
  const uint32_t tau = (prefix << 4) | h.bin;
  if (h.cnt == need) return Cut{0, tau, kAllPos};

  // Several elements hold exactly the key tau and only `need` of them are
  // taken: the lowest positions. Window positions are < 2^17: two ascending
  // digits (bits 16..5, then 4..0) find the need-th lowest. The level-1
  // histogram is free (all its readers passed the barriers above).
  clear_bins<kBins>(sm.hist);
  __syncthreads();
  src.for_each([&](uint32_t kk, int32_t j) {
    if (kk == tau) lds_inc(&sm.hist[(uint32_t)j >> 5]);
  });
  __syncthreads();
  h = wave_find<kBins, false>(sm.hist, need);
  need -= h.before;
  const uint32_t hi = h.bin;
  __syncthreads();
  clear_bins<32>(sm.hist);
  __syncthreads();
  src.for_each([&](uint32_t kk, int32_t j) {
    if ((kk == tau) & (((uint32_t)j >> 5) == hi)) lds_inc(&sm.hist[(uint32_t)j & 31u]);
  });
  __syncthreads();
  h = wave_find<32, false>(sm.hist, need);
  return Cut{0, tau, (int32_t)((hi << 5) | h.bin)};
}

// Whole span in registers (span <= NV * 4 * kBlock).
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
template <int NV, bool kPaged>
__device__ __forceinline__ void row_in_registers(const RowView& rv, int32_t k, Emit<kPaged> em,
                                                 SmemReg& sm) {
  const int lane = lane_id();
  const int w = wave_id();
  const int32_t t = threadIdx.x;
  const int32_t L = rv.span - rv.rem;
  const int32_t nvec = (rv.span + 3) >> 2;
  uint32_t key[NV][4];
  {
    float4 x[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int32_t v = i * kBlock + t;
      x[i] = v < nvec ? rv.base4[v] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    em.stage_table(sm.pt, L);
    clear_bins<kBins>(sm.hist);
    sm.h2[t] = 0;  // kBlock == 256 == the size of h2 and h3
    sm.h3[t] = 0;
    if (t < 16) sm.h4[t] = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int32_t v = i * kBlock + t;
#pragma unroll
      for (int c = 0; c < 4; ++c) key[i][c] = order_key(lane_of(x[i], c));
      // only the vectors holding the window's first or last columns (or
      // none of it) carry columns outside the window
      if ((v == 0) | (v * 4 + 4 > rv.span)) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int32_t a = v * 4 + c;
          if ((a < rv.rem) | (a >= rv.span)) key[i][c] = 0;
        }
      }
    }
  }
  __syncthreads();
  // Level-1 histogram. Vectors past the span are skipped; the few columns
  // outside the window inside the edge vectors land in bin 0, which the
  // descending scan never reaches (bin 0 holds no float's key, and more
  // than k in-window keys sit above it).
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (i * kBlock + t < nvec) {
#pragma unroll
      for (int c = 0; c < 4; ++c) lds_inc(&sm.hist[key[i][c] >> 20]);
    }
  }
  __syncthreads();
  const RegSrc<NV> src{key, rv.rem};
  const Cut cut = refine_in_registers(src, sm, (uint32_t)k);

  // Selection becomes one compare, key >= thr. Without a partial tie class
  // (the usual case) thr is the cut's lowest key. With one (several
  // elements hold exactly the k-th key tau, and only those at positions
  // <= pos are taken), a rare extra pass raises the taken tied keys to
  // tau + 1 and thr = tau + 1. (tau + 1 cannot wrap: no float's key is
  // all ones.)
  uint32_t thr;
  if (cut.pos == kAllPos) {
    const uint32_t lo = cut.prefix << cut.shift;
    thr = lo ? lo : 1u;
  } else {
    const uint32_t tau = cut.prefix;
    const int32_t pos = cut.pos;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int32_t j = (i * kBlock + t) * 4 + c - rv.rem;
        if ((key[i][c] == tau) & (j <= pos)) key[i][c] = tau + 1u;
      }
    }
    thr = tau + 1u;
  }

  // Each thread's output count, then its first output slot: lane l of wave
  // w writes after all lower waves and after lanes < l of its wave.
  uint32_t mine = 0;
  src.for_each([&](uint32_t kk, int32_t) { mine += (kk >= thr) ? 1u : 0u; });
  const uint32_t mine_incl = wave_inclusive_sum(mine);
  if (lane == 63) sm.wave_cnt[w] = mine_incl;
  __syncthreads();
  uint32_t slot = mine_incl - mine;
  for (int v = 0; v < w; ++v) slot += sm.wave_cnt[v];

  // Stage the selected positions in LDS (the histogram's space, free now),
  // branch-free: unselected elements go to a dummy slot past the k real
  // ones. Then one coalesced pass maps and stores the k outputs.
  int32_t* stage = reinterpret_cast<int32_t*>(sm.hist);
  const uint32_t dummy = (uint32_t)kMaxK + (uint32_t)t;  // kMaxK + kBlock <= kBins
  src.for_each([&](uint32_t kk, int32_t j) {
    const bool sel = kk >= thr;
    stage[(sel & (slot < (uint32_t)k)) ? slot : dummy] = j;
    slot += sel ? 1u : 0u;
  });
  __syncthreads();
  write_stage(em, stage, L, k);
}

// Span too long for registers: stream it. Pass 1 builds the level-1
// histogram; pass 2 sends the elements above the threshold bin to the
// stage and the threshold bin's elements to LDS, where one wave resolves
// the cut. A threshold bin larger than the LDS buffer is resolved by
// re-reading the span once per digit instead.
template <bool kPaged>
__device__ __forceinline__ void row_streaming(const RowView& rv, int32_t k, const Emit<kPaged>& em,
                                              SmemStream& sm) {
  const StreamSrc src{rv};
  const int32_t L = rv.span - rv.rem;
  clear_bins<kBins>(sm.hist);
  if (threadIdx.x == 0) {
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
    const Cut cut = refine_cut<false>(src, sm.hist, t1, need, cnt);
    src.for_each([&](uint32_t key, int32_t j) {
      wave_append(is_selected(cut, key, j), j, sm.stage, &sm.nstage, kMaxK);
    });
  }
  __syncthreads();
  write_stage(em, sm.stage, L, k);
}

template <bool kPaged>
__device__ __forceinline__ Emit<kPaged> row_emit(const Params& p, int64_t b) {
  Emit<kPaged> em;
  em.out = p.out + b * p.k;
  em.page_bits = p.page_bits;
  em.pt_lds = nullptr;
  if constexpr (kPaged) {
    em.pt = p.page_table + b * p.pt_stride;
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

// Class of a row: short = trivial (L <= k) or span <= 8192 floats; mid =
// span <= 16384; long = the rest.
__device__ __forceinline__ RowInfo row_info(const int32_t* seq_lens, const int32_t* row_starts,
                                            int32_t k, int64_t b) {
  RowInfo r;
  int32_t L = seq_lens[b];
  r.L = L < 0 ? 0 : (L > DSATOPK_MAX_SEQ_LEN ? DSATOPK_MAX_SEQ_LEN : L);
  r.s = row_starts ? row_starts[b] : 0;
  r.span = r.L + (r.s & 3);
  r.cls = (r.L <= k || r.span <= kSmallVec * 4 * kBlock) ? kClassShort
          : (r.span <= kLargeVec * 4 * kBlock)            ? kClassMid
                                                          : kClassLong;
  return r;
}

__device__ __forceinline__ RowView row_view(const Params& p, int64_t b, const RowInfo& r) {
  RowView rv;
  const int32_t rem = r.s & 3;
  rv.base4 = reinterpret_cast<const float4*>(p.scores + b * p.stride + (r.s - rem));
  rv.rem = rem;
  rv.span = r.span;
  return rv;
}

// The row this workgroup serves in a launch for class kClass, or -1.
// With a plan, workgroup i takes the i-th planned row of the class; a row
// whose class changed since planning is skipped here and served by the
// long-row launch instead. Without a plan, workgroup i looks at row i.
// A plan is used only if it was built for this many rows; every kernel of a
// call takes the same decision, so each row is served exactly once.
__device__ __forceinline__ bool plan_ok(const Params& p) {
  return p.plan && p.plan[kPlanWordMagic] == kPlanMagic && p.plan[kPlanWordRows] == p.num_rows;
}

template <int kClass>
__device__ __forceinline__ int64_t class_row(const Params& p, RowInfo& r) {
  int64_t b = blockIdx.x;
  if (plan_ok(p)) {
    const uint32_t i = (uint32_t)p.plan[kPlanWordOffset + kClass] + blockIdx.x;
    if ((int32_t)blockIdx.x >= p.plan[kPlanWordCount + kClass] || i >= (uint32_t)p.num_rows)
      return -1;
    b = p.plan[kPlanHeaderWords + i];
    if ((uint64_t)b >= (uint64_t)p.num_rows) return -1;
  }
  r = row_info(p.seq_lens, p.row_starts, p.k, b);
  return r.cls == kClass ? b : -1;
}

// Trivial rows and spans <= 8192 floats, kept in registers.
template <bool kPaged>
__global__ __launch_bounds__(kBlock) void rows_short_kernel(const Params p) {
  RowInfo r;
  const int64_t b = class_row<kClassShort>(p, r);
  if (b < 0) return;
  const Emit<kPaged> em = row_emit<kPaged>(p, b);
  if (r.L <= p.k) {
    write_trivial(em, r.L, p.k);
    return;
  }
  __shared__ SmemReg sm;
  row_in_registers<kSmallVec>(row_view(p, b, r), p.k, em, sm);
}

// Spans of 8193 .. 16384 floats, kept in registers.
template <bool kPaged>
__global__ __launch_bounds__(kBlock) void rows_mid_kernel(const Params p) {
  RowInfo r;
  const int64_t b = class_row<kClassMid>(p, r);
  if (b < 0) return;
  __shared__ SmemReg sm;
  row_in_registers<kLargeVec>(row_view(p, b, r), p.k, row_emit<kPaged>(p, b), sm);
}

// Longer spans, streamed; also any row whose class differs from the plan's
// (such a row is skipped by the other launches). One workgroup per row.
template <bool kPaged>
__global__ __launch_bounds__(kBlock) void rows_long_kernel(const Params p) {
  const int64_t b = blockIdx.x;
  const RowInfo r = row_info(p.seq_lens, p.row_starts, p.k, b);
  const int32_t* planned = plan_ok(p) ? p.plan + kPlanHeaderWords + p.num_rows : nullptr;
  const bool stale = planned && planned[b] != r.cls;
  if (r.cls != kClassLong && !stale) return;
  const Emit<kPaged> em = row_emit<kPaged>(p, b);
  if (r.L <= p.k) {
    write_trivial(em, r.L, p.k);
    return;
  }
  __shared__ SmemStream sm;
  row_streaming(row_view(p, b, r), p.k, em, sm);
}

// Plan: classify every row and list the rows of each class. One workgroup.
constexpr int kPlanBlock = 1024;

__global__ __launch_bounds__(kPlanBlock) void plan_kernel(const int32_t* seq_lens,
                                                         const int32_t* row_starts,
                                                         int32_t num_rows, int32_t k,
                                                         int32_t* plan) {
  __shared__ uint32_t count[3];
  __shared__ uint32_t fill[3];
  if (threadIdx.x < 3) {
    count[threadIdx.x] = 0;
    fill[threadIdx.x] = 0;
  }
  __syncthreads();
  int32_t* cls = plan + kPlanHeaderWords + num_rows;
  for (int32_t b = threadIdx.x; b < num_rows; b += kPlanBlock) {
    const int32_t c = row_info(seq_lens, row_starts, k, b).cls;
    cls[b] = c;
    atomicAdd(&count[c], 1u);
  }
  __syncthreads();
  const uint32_t off[3] = {0u, count[0], count[0] + count[1]};
  int32_t* list = plan + kPlanHeaderWords;
  for (int32_t b = threadIdx.x; b < num_rows; b += kPlanBlock) {
    const int32_t c = cls[b];
    list[off[c] + atomicAdd(&fill[c], 1u)] = b;
  }
  if (threadIdx.x == 0) {
    plan[kPlanWordMagic] = kPlanMagic;
    plan[kPlanWordRows] = num_rows;
    plan[kPlanWordK] = k;
    for (int c = 0; c < 3; ++c) {
      plan[kPlanWordCount + c] = (int32_t)count[c];
      plan[kPlanWordOffset + c] = (int32_t)off[c];
    }
  }
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
  if (plan && plan_bytes < dsatopk_plan_bytes(num_rows)) return DSATOPK_ERR_PLAN_TOO_SMALL;
  return DSATOPK_OK;
}

// Launch the class kernels the score stride allows (a row's span never
// exceeds score_stride). The plan's row lists are used only when every
// class is launched: a row whose class changed since planning then still
// reaches the long-row launch.
template <bool kPaged>
int launch_rows(Params p, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_rows);
  const dim3 block(kBlock);
  const bool mid = p.stride > (int64_t)kSmallVec * 4 * kBlock;
  const bool lng = p.stride > (int64_t)kLargeVec * 4 * kBlock;
  if (!lng) p.plan = nullptr;
  if (lng) hipLaunchKernelGGL((rows_long_kernel<kPaged>), grid, block, 0, stream, p);
  hipLaunchKernelGGL((rows_short_kernel<kPaged>), grid, block, 0, stream, p);
  if (mid) hipLaunchKernelGGL((rows_mid_kernel<kPaged>), grid, block, 0, stream, p);
  return hipGetLastError() == hipSuccess ? DSATOPK_OK : DSATOPK_ERR_HIP;
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
    default: return "unknown status";
  }
}

size_t dsatopk_plan_bytes(int32_t num_rows) {
  if (num_rows < 0) return 0;
  return sizeof(int32_t) * ((size_t)kPlanHeaderWords + 2u * (size_t)num_rows);
}

int dsatopk_plan(const int32_t* seq_lens, const int32_t* row_starts, int32_t num_rows, int32_t k,
                 void* plan, size_t plan_bytes, void* stream) {
  if (num_rows < 0 || k < 1 || k > DSATOPK_MAX_K) return DSATOPK_ERR_INVALID_ARG;
  if (num_rows == 0) return DSATOPK_OK;
  if (!seq_lens || !plan) return DSATOPK_ERR_INVALID_ARG;
  if (plan_bytes < dsatopk_plan_bytes(num_rows)) return DSATOPK_ERR_PLAN_TOO_SMALL;
  if ((reinterpret_cast<uintptr_t>(plan) & 15u) != 0) return DSATOPK_ERR_ALIGNMENT;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanBlock), 0, (hipStream_t)stream, seq_lens,
                     row_starts, num_rows, k, (int32_t*)plan);
  return hipGetLastError() == hipSuccess ? DSATOPK_OK : DSATOPK_ERR_HIP;
}

int dsatopk_paged(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                  const int32_t* row_starts, const int32_t* page_table,
                  int64_t page_table_stride, int32_t page_size, int32_t num_rows, int32_t k,
                  const void* plan, size_t plan_bytes, int32_t* out, void* stream) {
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
  p.plan = (const int32_t*)plan;
  return launch_rows<true>(p, (hipStream_t)stream);
}

int dsatopk_ragged(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                   const int32_t* row_starts, const int32_t* out_offsets, int32_t num_rows,
                   int32_t k, const void* plan, size_t plan_bytes, int32_t* out, void* stream) {
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
  p.plan = (const int32_t*)plan;
  return launch_rows<false>(p, (hipStream_t)stream);
}

}  // extern "C"
