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
//
// All cross-lane work is native wave64: DPP row shifts and row broadcasts
// for scans, 64-bit ballots with mbcnt for ordered compaction (the pages'
// CUDA code emulates 32-lane warps on wave64; PR #36684 digest,
// topk_impl.cuh excerpt).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsatopk {

constexpr int kBlock = 256;          // threads per workgroup: 4 wave64s
constexpr int kWaves = kBlock / 64;
constexpr int kBins = 4096;          // 12-bit digit
constexpr int kMaxK = 2048;
constexpr int kAllPos = 0x7fffffff;  // "every tied position" in a cut

// Order-preserving key: unsigned order of the key equals the numeric order
// of the float, and -0.0 and +0.0 get the same key. Negative floats map to
// ~u (so -0.0 -> 0x7fffffff); non-negative floats map to (u | 2^31) - 1
// (so +0.0 -> 0x7fffffff too; the shift by one keeps the order). Key 0 is
// reserved for "not in the window": no float maps to it except the
// all-ones negative NaN, and NaNs are outside the contract. Written as
// (u ^ s) + (~s & 0x7fffffff) with s the sign mask: for a negative float
// that is ~u + 0, for a non-negative one u + 2^31 - 1, the same key; it
// compiles to three VALU ops (shift, bit select, xor-add).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = (uint32_t)((int32_t)u >> 31);  // all ones if negative
  return (u ^ s) + (~s & 0x7fffffffu);
}

__device__ __forceinline__ void lds_inc(uint32_t* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Adds v to an LDS counter. With v from opaque_one() the constant stays in
// one VGPR for a whole pass; a literal 1 is rebuilt in every exec-masked
// block of a filtered pass.
__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t opaque_one() {
  uint32_t one = 1u;
  asm volatile("" : "+v"(one));
  return one;
}

// x + (this lane's bit of the lane mask m), as one add-with-carry that
// takes the mask (a compare's result) as its carry-in.
__device__ __forceinline__ uint32_t add_lane_bit(uint32_t x, uint64_t m) {
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, 0, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(x), "s"(m));
  return r;
}

// threadIdx.x, opaque to the optimizer: values derived from it are rebuilt
// where they are used instead of being hoisted out of a row loop and held
// in VGPRs for the whole kernel (which cost the persistent kernel a third
// of its occupancy).
__device__ __forceinline__ int tix() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ int lane_id() { return tix() & 63; }
// The wave's index in the workgroup, as a scalar (the same for all lanes).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(tix() >> 6);
}

// Orders this wave's LDS accesses: everything issued before is complete and
// visible to every lane of the wave afterwards.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t read_lane(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Inclusive prefix sum across one wave64 with DPP: shifts by 1, 2, 4, 8
// inside each 16-lane row, then the row-15 and row-31 broadcasts carry the
// row totals into the rows above.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

template <int NB, int BS = kBlock>
__device__ __forceinline__ void clear_bins(uint32_t* hist) {
  if constexpr (NB >= 4 * BS) {
    uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
    for (int i = tix(); i < NB / 4; i += BS) h4[i] = make_uint4(0, 0, 0, 0);
  } else {
    for (int i = tix(); i < NB; i += BS) hist[i] = 0;
  }
}

// Same, by one wave.
template <int NB>
__device__ __forceinline__ void wave_clear_bins(uint32_t* hist) {
  if constexpr (NB >= 256) {
    uint4* h4 = reinterpret_cast<uint4*>(hist);
#pragma unroll
    for (int i = lane_id(); i < NB / 4; i += 64) h4[i] = make_uint4(0, 0, 0, 0);
  } else {
    for (int i = lane_id(); i < NB; i += 64) hist[i] = 0;
  }
}

struct BinHit {
  uint32_t bin;     // the bin where the running count reaches `need`
  uint32_t before;  // count of all bins before it in scan order
  uint32_t cnt;     // count in the bin
};

// One wave scans NB bins in descending (kDesc) or ascending order and finds
// the bin where the running count first reaches need (1 <= need <= total).
// Two levels: lane l sums scan positions [l*PER, (l+1)*PER); the lane where
// the running sum crosses `need` is found with a DPP scan and a ballot; then
// the 64 lanes take one scan position each inside that lane's run (PER is
// at most 64) and a second scan finds the bin. The result is wave-uniform.
template <int NB, bool kDesc>
__device__ __forceinline__ BinHit wave_find(const uint32_t* hist, uint32_t need) {
  constexpr int PER = NB >= 64 ? NB / 64 : 1;
  static_assert(PER <= 64, "one lane run per second-level lane");
  const int lane = lane_id();
  auto at = [&](int r) -> uint32_t { return r < NB ? hist[kDesc ? NB - 1 - r : r] : 0u; };
  uint32_t sum = 0;
  if constexpr (PER >= 4) {
    // scan run of this lane = bins [lo, lo + PER) in memory, either order.
    // Lanes' runs are PER * 4 bytes apart, so reading them in step would
    // put every lane on the same LDS banks; each lane starts its run at a
    // different 16-byte chunk instead (the sum does not care).
    constexpr int CH = PER / 4;
    const int lo = kDesc ? NB - (lane + 1) * PER : lane * PER;
    const uint4* h4 = reinterpret_cast<const uint4*>(hist + lo);
    // at most four 16-byte reads in flight: the caller's keys stay in VGPRs
#pragma unroll 4
    for (int i = 0; i < CH; ++i) {
      const uint4 q = h4[(i + lane) & (CH - 1)];
      sum += q.x + q.y + q.z + q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) sum += at(lane * PER + i);
  }
  const uint32_t incl = wave_inclusive_sum(sum);
  const uint64_t m1 = __ballot(incl >= need);
  const int l1 = m1 ? __builtin_ctzll(m1) : 63;
  const uint32_t base = read_lane(incl - sum, l1);
  BinHit h;
  if constexpr (PER == 1) {
    const uint32_t r = (uint32_t)l1;
    h.bin = kDesc ? NB - 1 - r : r;
    h.before = base;
    h.cnt = read_lane(sum, l1);
  } else {
    const uint32_t v = lane < PER ? at(l1 * PER + lane) : 0u;
    const uint32_t incl2 = base + wave_inclusive_sum(v);
    const uint64_t m2 = __ballot((lane < PER) & (incl2 >= need));
    const int l2 = m2 ? __builtin_ctzll(m2) : 0;
    const uint32_t rr = (uint32_t)(l1 * PER + l2);
    h.bin = kDesc ? NB - 1 - rr : rr;
    h.cnt = read_lane(v, l2);
    h.before = read_lane(incl2, l2) - h.cnt;
  }
  return h;
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
  return (key != 0u) & ((hi > c.prefix) | ((hi == c.prefix) & (j <= c.pos)));
}

// Resolve the exact cut given the level-1 result (bin t1 of the top 12 key
// bits, `need` elements still to take from it, `cnt` elements in it), over
// the elements produced by `src` (any superset of bin t1's elements: the
// rest is filtered out here).
//
// kWave: executed by one wave alone (no workgroup barriers), src must
// enumerate every element to that wave. Otherwise executed by the whole
// workgroup, every wave finding each bin redundantly; it begins and ends
// with a barrier.
template <bool kWave, class Src, int BS = kBlock>
__device__ __forceinline__ Cut refine_cut(const Src src, uint32_t* hist, uint32_t prefix,
                                          uint32_t need, uint32_t cnt) {
  if (cnt == need) return Cut{20, prefix, kAllPos};
  auto sync = [] {
    if constexpr (kWave) wave_lds_sync(); else __syncthreads();
  };
  auto clear4096 = [&] {
    if constexpr (kWave) wave_clear_bins<kBins>(hist); else clear_bins<kBins, BS>(hist);
  };

  // level 2: key bits 19..8 inside bin t1
  sync();  // earlier readers of hist are done
  clear4096();
  sync();
  {
    const uint32_t p = prefix;
    src.for_each([&](uint32_t key, int32_t) {
      if ((key != 0u) & ((key >> 20) == p)) lds_inc(&hist[(key >> 8) & 0xfffu]);
    });
  }
  sync();
  BinHit h = wave_find<kBins, true>(hist, need);
  need -= h.before;
  prefix = (prefix << 12) | h.bin;
  Cut cut{8, prefix, kAllPos};
  if (h.cnt != need) {
    // level 3: key bits 7..0
    sync();
    if constexpr (kWave) wave_clear_bins<256>(hist); else clear_bins<256, BS>(hist);
    sync();
    {
      const uint32_t p = prefix;
      src.for_each([&](uint32_t key, int32_t) {
        if ((key != 0u) & ((key >> 8) == p)) lds_inc(&hist[key & 0xffu]);
      });
    }
    sync();
    h = wave_find<256, true>(hist, need);
    need -= h.before;
    const uint32_t tau = (prefix << 8) | h.bin;
    cut = Cut{0, tau, kAllPos};
    if (h.cnt != need) {
      // Several elements hold exactly the key tau and only `need` of them
      // are taken: the lowest positions. Window positions are < 2^17, so two
      // ascending digits (bits 16..5, then 4..0) find the need-th lowest.
      sync();
      clear4096();
      sync();
      src.for_each([&](uint32_t key, int32_t j) {
        if (key == tau) lds_inc(&hist[(uint32_t)j >> 5]);
      });
      sync();
      h = wave_find<kBins, false>(hist, need);
      need -= h.before;
      const uint32_t hi = h.bin;
      sync();
      if constexpr (kWave) wave_clear_bins<32>(hist); else clear_bins<32, BS>(hist);
      sync();
      src.for_each([&](uint32_t key, int32_t j) {
        if ((key == tau) & (((uint32_t)j >> 5) == hi)) lds_inc(&hist[(uint32_t)j & 31u]);
      });
      sync();
      h = wave_find<32, false>(hist, need);
      cut.pos = (int32_t)((hi << 5) | h.bin);
    }
  }
  sync();  // hist readers done before reuse
  return cut;
}

// Append `val` for every lane with `pred` to buf at slots taken from
// *counter, one LDS atomic per wave. Slots at or past `cap` are dropped.
// Must be called by the whole wave.
__device__ __forceinline__ void wave_append(bool pred, int32_t val, int32_t* buf,
                                            uint32_t* counter, uint32_t cap) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return;
  const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  const int leader = __builtin_ctzll(m);
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(m));
  base = read_lane(base, leader);
  if (pred && base + rank < cap) buf[base + rank] = val;
}

// Same for (key, position) pairs.
__device__ __forceinline__ void wave_append_pair(bool pred, uint32_t key, int32_t j, uint2* buf,
                                                 uint32_t* counter, uint32_t cap) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return;
  const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  const int leader = __builtin_ctzll(m);
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(m));
  base = read_lane(base, leader);
  if (pred && base + rank < cap) buf[base + rank] = make_uint2(key, (uint32_t)j);
}

}  // namespace dsatopk
