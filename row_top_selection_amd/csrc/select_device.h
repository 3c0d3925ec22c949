// select_device.h - device building blocks of the dsatopk kernels (gfx950).
//
// Selection scheme: every in-window score is mapped to a 32-bit key whose
// unsigned order is the float order; the k-th largest key is found digit by
// digit with LDS histograms (12, 12 and 8 bits), and when several elements
// share that exact key, two more digits over the window position (12 and 5
// bits) find the position cut so that the lowest positions win. The result
// is a cut (shift, prefix, pos): an element is selected iff its key's high
// bits exceed the prefix, or equal it with position <= pos.
//
// The pages describe the same two-stage idea (a coarse key histogram finds
// the threshold bin, then a refinement pass inside that bin) with a 12-bit
// first key (sglang PR #36684 digest, "Motivation": 12-bit key instead of
// 8-bit, so fewer candidates reach refinement; PR #26788 digest, "Executive
// summary": histogram + threshold two-stage algorithm). The tie rule and the
// position digits are this library's: the pages leave ties unordered.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsatopk {

constexpr int kBlock = 512;          // threads per workgroup: 8 wave64s
constexpr int kWaves = kBlock / 64;
constexpr int kBins = 4096;          // 12-bit digit
constexpr int kMaxK = 2048;
constexpr int kAllPos = 0x7fffffff;  // "every tied position" in a cut

// Order-preserving key: unsigned order of the key equals the numeric order
// of the float. -0.0 is folded onto +0.0 first so that the two tie. The key
// 0 is reserved for "not in the window"; the one float that would map to it
// (the all-ones negative NaN) is moved to 1.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  u = (u == 0x80000000u) ? 0u : u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return key ? key : 1u;
}

__device__ __forceinline__ void lds_inc(uint32_t* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Inclusive prefix sum across one wave64.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t n = __shfl_up(v, d, 64);
    if (lane >= d) v += n;
  }
  return v;
}

// Exclusive prefix sum across the workgroup in thread order. Contains one
// barrier; the caller must pass another barrier before wave_tot is reused.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* wave_tot) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_sum(v);
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) base += (w < wave) ? wave_tot[w] : 0u;
  return base + inc - v;
}

template <int NB>
__device__ __forceinline__ void clear_bins(uint32_t* hist) {
  if constexpr (NB >= 4 * kBlock) {
    uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
    for (int i = threadIdx.x; i < NB / 4; i += kBlock) h4[i] = make_uint4(0, 0, 0, 0);
  } else {
    for (int i = threadIdx.x; i < NB; i += kBlock) hist[i] = 0;
  }
}

// Scan NB bins in descending (kDesc) or ascending bin order and find the bin
// where the running count first reaches `need` (1 <= need <= total).
// res[0] = that bin, res[1] = count of all bins before it in scan order,
// res[2] = count in the bin. Ends with a barrier, after which every thread
// may read res.
template <int NB, bool kDesc>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t need, uint32_t* wave_tot,
                                         uint32_t* res) {
  constexpr int PER = NB >= kBlock ? NB / kBlock : 1;
  const int r0 = threadIdx.x * PER;
  uint32_t c[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int r = r0 + i;
    uint32_t h = 0;
    if (r < NB) h = hist[kDesc ? NB - 1 - r : r];
    c[i] = h;
    sum += h;
  }
  const uint32_t base = block_exclusive_sum(sum, wave_tot);
  if (base < need && need <= base + sum) {
    uint32_t acc = base;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc < need && need <= acc + c[i]) {
        const int r = r0 + i;
        res[0] = kDesc ? NB - 1 - r : r;
        res[1] = acc;
        res[2] = c[i];
      }
      acc += c[i];
    }
  }
  __syncthreads();
}

// Selection cut: key's bits above `shift` compared with `prefix`; on
// equality the window position decides (<= pos).
struct Cut {
  uint32_t shift;
  uint32_t prefix;
  int32_t pos;
};

__device__ __forceinline__ bool is_selected(const Cut& c, uint32_t key, int32_t j) {
  const uint32_t hi = key >> c.shift;
  return key != 0u && (hi > c.prefix || (hi == c.prefix && j <= c.pos));
}

// LDS working set shared by the refinement levels.
struct Scratch {
  uint32_t* hist;      // kBins counters
  uint32_t* wave_tot;  // kWaves
  uint32_t* res;       // 4
};

// Given the level-1 result (bin T1 of the top 12 key bits, `need` elements
// still to take from it, `cnt` elements in it), resolve the exact cut over
// the elements produced by `src` (any superset of the elements of bin T1:
// others are filtered out here). Every thread of the workgroup must call it.
template <class Src>
__device__ __forceinline__ Cut refine_cut(const Src src, const Scratch sc, uint32_t prefix,
                                          uint32_t need, uint32_t cnt) {
  uint32_t* hist = sc.hist;
  if (cnt == need) return Cut{20, prefix, kAllPos};

  // level 2: key bits 19..8 inside bin T1
  clear_bins<kBins>(hist);
  __syncthreads();
  {
    const uint32_t p = prefix;
    src.for_each([&](uint32_t key, int32_t) {
      if (key != 0u && (key >> 20) == p) lds_inc(&hist[(key >> 8) & 0xfffu]);
    });
  }
  __syncthreads();
  find_bin<kBins, true>(hist, need, sc.wave_tot, sc.res);
  need -= sc.res[1];
  cnt = sc.res[2];
  prefix = (prefix << 12) | sc.res[0];
  if (cnt == need) return Cut{8, prefix, kAllPos};

  // level 3: key bits 7..0
  clear_bins<256>(hist);
  __syncthreads();
  {
    const uint32_t p = prefix;
    src.for_each([&](uint32_t key, int32_t) {
      if (key != 0u && (key >> 8) == p) lds_inc(&hist[key & 0xffu]);
    });
  }
  __syncthreads();
  find_bin<256, true>(hist, need, sc.wave_tot, sc.res);
  need -= sc.res[1];
  cnt = sc.res[2];
  const uint32_t tau = (prefix << 8) | sc.res[0];
  if (cnt == need) return Cut{0, tau, kAllPos};

  // Several elements hold exactly the key tau and only `need` of them are
  // taken: the lowest positions. Window positions are < 2^17, so two
  // ascending digits (bits 16..5, then 4..0) find the need-th lowest.
  clear_bins<kBins>(hist);
  __syncthreads();
  src.for_each([&](uint32_t key, int32_t j) {
    if (key == tau) lds_inc(&hist[(uint32_t)j >> 5]);
  });
  __syncthreads();
  find_bin<kBins, false>(hist, need, sc.wave_tot, sc.res);
  need -= sc.res[1];
  const uint32_t hi = sc.res[0];
  clear_bins<32>(hist);
  __syncthreads();
  src.for_each([&](uint32_t key, int32_t j) {
    if (key == tau && ((uint32_t)j >> 5) == hi) lds_inc(&hist[(uint32_t)j & 31u]);
  });
  __syncthreads();
  find_bin<32, false>(hist, need, sc.wave_tot, sc.res);
  return Cut{0, tau, (int32_t)((hi << 5) | sc.res[0])};
}

// Append `val` for every lane with `pred` to buf at slots taken from
// *counter, one LDS atomic per wave. Slots at or past `cap` are dropped.
// Must be called by the whole wave.
__device__ __forceinline__ void wave_append(bool pred, int32_t val, int32_t* buf,
                                            uint32_t* counter, uint32_t cap) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  const int leader = __builtin_ctzll(m);
  uint32_t base = 0;
  if ((int)lane == leader) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(m));
  base = __shfl(base, leader, 64);
  if (pred && base + rank < cap) buf[base + rank] = val;
}

// Same for (key, position) pairs.
__device__ __forceinline__ void wave_append_pair(bool pred, uint32_t key, int32_t j, uint2* buf,
                                                 uint32_t* counter, uint32_t cap) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  const int leader = __builtin_ctzll(m);
  uint32_t base = 0;
  if ((int)lane == leader) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(m));
  base = __shfl(base, leader, 64);
  if (pred && base + rank < cap) buf[base + rank] = make_uint2(key, (uint32_t)j);
}

}  // namespace dsatopk
