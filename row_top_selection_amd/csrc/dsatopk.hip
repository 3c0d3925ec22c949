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

constexpr int kSmallVec = 4;   // float4 per thread: 8192-float spans
constexpr int kLargeVec = 9;   // float4 per thread: 18432-float spans
constexpr int kStreamVec = 4;  // float4 per thread per streaming chunk
constexpr int kCandCap = 2048; // LDS candidate pairs on the streaming path

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
};

// Output of one row: position j -> emitted value.
template <bool kPaged>
struct Emit {
  int32_t* out;
  const int32_t* pt;
  int32_t page_bits;
  int32_t offset;

  __device__ __forceinline__ int32_t value(int32_t j) const {
    if constexpr (kPaged) {
      const int32_t page = pt[j >> page_bits];
      return (int32_t)(((uint32_t)page << page_bits) | ((uint32_t)j & ((1u << page_bits) - 1u)));
    } else {
      return j + offset;
    }
  }
};

// Shared memory of the register path: the histogram, reused as the output
// stage once the cut is known.
struct SmemReg {
  uint32_t hist[kBins];
  uint32_t wave_tot[kWaves];
  uint32_t res[4];
};

// Shared memory of the streaming path.
struct SmemStream {
  uint32_t hist[kBins];
  int32_t stage[kMaxK];
  uint2 cand[kCandCap];
  uint32_t wave_tot[kWaves];
  uint32_t res[4];
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
  return (a >= rv.rem && a < rv.span) ? order_key(x) : 0u;
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

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int32_t a0 = (i * kBlock + (int32_t)threadIdx.x) * 4 - rem;
#pragma unroll
      for (int c = 0; c < 4; ++c) f(key[i][c], a0 + c);
    }
  }
};

// Candidates held in LDS as (key, position) pairs.
struct CandSrc {
  const uint2* cand;
  uint32_t n;

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
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
template <bool kPaged>
__device__ __forceinline__ void write_stage(const Emit<kPaged>& em, const int32_t* stage,
                                            int32_t L, int32_t k) {
  for (int32_t t = threadIdx.x; t < k; t += kBlock) {
    const int32_t j = stage[t];
    em.out[t] = (j >= 0 && j < L) ? em.value(j) : -1;
  }
}

// Whole span in registers (span <= NV * 4 * kBlock).
template <int NV, bool kPaged>
__device__ __forceinline__ void row_in_registers(const RowView& rv, int32_t k,
                                                 const Emit<kPaged>& em, SmemReg& sm) {
  uint32_t key[NV][4];
  {
    const int32_t nvec = (rv.span + 3) >> 2;
    float4 x[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int32_t v = i * kBlock + (int32_t)threadIdx.x;
      x[i] = v < nvec ? rv.base4[v] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    clear_bins<kBins>(sm.hist);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int32_t a0 = (i * kBlock + (int32_t)threadIdx.x) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) key[i][c] = key_at(lane_of(x[i], c), a0 + c, rv);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (key[i][c]) lds_inc(&sm.hist[key[i][c] >> 20]);
  }
  __syncthreads();
  const Scratch sc{sm.hist, sm.wave_tot, sm.res};
  find_bin<kBins, true>(sm.hist, (uint32_t)k, sm.wave_tot, sm.res);
  const RegSrc<NV> src{key, rv.rem};
  const Cut cut = refine_cut(src, sc, sm.res[0], (uint32_t)k - sm.res[1], sm.res[2]);

  // Deterministic emit: each thread's selected elements go to consecutive
  // stage slots after those of lower threads. The stage reuses the
  // histogram, which no thread reads any more.
  uint32_t mine = 0;
  src.for_each([&](uint32_t kk, int32_t j) { mine += is_selected(cut, kk, j) ? 1u : 0u; });
  uint32_t slot = block_exclusive_sum(mine, sm.wave_tot);
  int32_t* stage = reinterpret_cast<int32_t*>(sm.hist);
  src.for_each([&](uint32_t kk, int32_t j) {
    if (is_selected(cut, kk, j) && slot < (uint32_t)kMaxK) stage[slot++] = j;
  });
  __syncthreads();
  write_stage(em, stage, rv.span - rv.rem, k);
}

// Span too long for registers: stream it.
template <bool kPaged>
__device__ __forceinline__ void row_streaming(const RowView& rv, int32_t k, const Emit<kPaged>& em,
                                           SmemStream& sm) {
  const StreamSrc src{rv};
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
  const Scratch sc{sm.hist, sm.wave_tot, sm.res};
  find_bin<kBins, true>(sm.hist, (uint32_t)k, sm.wave_tot, sm.res);
  const uint32_t t1 = sm.res[0];
  const uint32_t need = (uint32_t)k - sm.res[1];
  const uint32_t cnt = sm.res[2];

  if (cnt != need && cnt <= (uint32_t)kCandCap) {
    // Pass 2: elements above bin t1 are selected; bin t1 goes to LDS.
    src.for_each([&](uint32_t key, int32_t j) {
      const uint32_t bin = key >> 20;
      wave_append(key != 0u && bin > t1, j, sm.stage, &sm.nstage, kMaxK);
      wave_append_pair(key != 0u && bin == t1, key, j, sm.cand, &sm.ncand, kCandCap);
    });
    __syncthreads();
    const CandSrc cs{sm.cand, cnt};
    const Cut cut = refine_cut(cs, sc, t1, need, cnt);
    for (uint32_t i0 = 0; i0 < cnt; i0 += kBlock) {
      const uint32_t i = i0 + threadIdx.x;
      uint2 e = make_uint2(0, 0);
      if (i < cnt) e = sm.cand[i];
      wave_append(i < cnt && is_selected(cut, e.x, (int32_t)e.y), (int32_t)e.y, sm.stage,
                  &sm.nstage, kMaxK);
    }
  } else {
    // Either the whole bin is taken, or it is too large for LDS: resolve
    // the cut by re-reading the span, then emit in one more pass.
    const Cut cut = refine_cut(src, sc, t1, need, cnt);
    src.for_each([&](uint32_t key, int32_t j) {
      wave_append(is_selected(cut, key, j), j, sm.stage, &sm.nstage, kMaxK);
    });
  }
  __syncthreads();
  write_stage(em, sm.stage, rv.span - rv.rem, k);
}

template <bool kPaged>
__device__ __forceinline__ Emit<kPaged> row_emit(const Params& p, int64_t b) {
  Emit<kPaged> em;
  em.out = p.out + b * p.k;
  em.page_bits = p.page_bits;
  if constexpr (kPaged) {
    em.pt = p.page_table + b * p.pt_stride;
    em.offset = 0;
  } else {
    em.pt = nullptr;
    em.offset = p.out_offsets[b];
  }
  return em;
}

// One workgroup per row. kLong: the launch may hold spans longer than
// kSmallVec * 4 * kBlock floats (the host knows spans <= score_stride).
template <bool kPaged, bool kLong>
__global__ __launch_bounds__(kBlock) void rows_kernel(const Params p) {
  const int64_t b = blockIdx.x;
  int32_t L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > DSATOPK_MAX_SEQ_LEN ? DSATOPK_MAX_SEQ_LEN : L);
  const int32_t s = p.row_starts ? p.row_starts[b] : 0;
  const Emit<kPaged> em = row_emit<kPaged>(p, b);
  const int32_t k = p.k;
  if (L <= k) {
    write_trivial(em, L, k);
    return;
  }
  const int32_t rem = s & 3;
  RowView rv;
  rv.base4 = reinterpret_cast<const float4*>(p.scores + b * p.stride + (s - rem));
  rv.rem = rem;
  rv.span = L + rem;

  if constexpr (kLong) {
    __shared__ union {
      SmemReg reg;
      SmemStream stream;
    } sm;
    if (rv.span <= kSmallVec * 4 * kBlock) {
      row_in_registers<kSmallVec>(rv, k, em, sm.reg);
    } else if (rv.span <= kLargeVec * 4 * kBlock) {
      row_in_registers<kLargeVec>(rv, k, em, sm.reg);
    } else {
      row_streaming(rv, k, em, sm.stream);
    }
  } else {
    __shared__ SmemReg sm;
    if (rv.span <= kSmallVec * 4 * kBlock) {
      row_in_registers<kSmallVec>(rv, k, em, sm);
    } else {
      // Unreachable when the host's bound holds; keep the row defined.
      write_trivial(em, 0, k);
    }
  }
}

// Plan: header only for now (see dsatopk_plan_bytes).
__global__ void plan_kernel(const int32_t* seq_lens, int32_t num_rows, int32_t k, int32_t* plan,
                            int32_t plan_words) {
  (void)seq_lens;
  for (int32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < plan_words;
       i += gridDim.x * blockDim.x) {
    int32_t v = 0;
    if (i == 0) v = 0x44534b31;  // "DSK1"
    if (i == 1) v = num_rows;
    if (i == 2) v = k;
    plan[i] = v;
  }
}

}  // namespace dsatopk

using namespace dsatopk;

namespace {

constexpr size_t kPlanHeaderBytes = 256;

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

template <bool kPaged>
int launch_rows(const Params& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_rows);
  const dim3 block(kBlock);
  if (p.stride <= kSmallVec * 4 * kBlock) {
    hipLaunchKernelGGL((rows_kernel<kPaged, false>), grid, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL((rows_kernel<kPaged, true>), grid, block, 0, stream, p);
  }
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
  return kPlanHeaderBytes + (size_t)num_rows * 8u;
}

int dsatopk_plan(const int32_t* seq_lens, int32_t num_rows, int32_t k, void* plan,
                 size_t plan_bytes, void* stream) {
  if (num_rows < 0 || k < 1 || k > DSATOPK_MAX_K) return DSATOPK_ERR_INVALID_ARG;
  if (num_rows == 0) return DSATOPK_OK;
  if (!seq_lens || !plan) return DSATOPK_ERR_INVALID_ARG;
  if (plan_bytes < dsatopk_plan_bytes(num_rows)) return DSATOPK_ERR_PLAN_TOO_SMALL;
  if ((reinterpret_cast<uintptr_t>(plan) & 15u) != 0) return DSATOPK_ERR_ALIGNMENT;
  const int32_t words = (int32_t)(dsatopk_plan_bytes(num_rows) / 4);
  const int32_t blocks = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
  hipLaunchKernelGGL(plan_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, seq_lens,
                     num_rows, k, (int32_t*)plan, words);
  return hipGetLastError() == hipSuccess ? DSATOPK_OK : DSATOPK_ERR_HIP;
}

int dsatopk_paged(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                  const int32_t* row_starts, const int32_t* page_table,
                  int64_t page_table_stride, int32_t page_size, int32_t num_rows, int32_t k,
                  void* plan, size_t plan_bytes, int32_t* out, void* stream) {
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
  return launch_rows<false>(p, (hipStream_t)stream);
}

}  // extern "C"
