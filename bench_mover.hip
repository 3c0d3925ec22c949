// The bytes of a selection launch, moved with no selection: the benchmark's
// ceiling for a launch of the same shape. One 256-thread workgroup per row
// reads the row's window of scores (16-byte non-temporal loads from the
// aligned column at or below the window's start, as the selection kernels
// read it) when the row has more than k columns, and writes k int32 to the
// row's outputs (non-temporal stores), each thread's values depending on
// its own loads so that no load is dropped. No barrier, no LDS, a few VALU
// per float4: its time is what HBM takes for these reads and writes in
// this launch shape.
//
// Built by __graft_entry__.build() into bench_mover.so beside this file and
// called by bench.py through ctypes; the library under row_top_selection_amd
// does not contain it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // float4 loads in flight per thread

__global__ __launch_bounds__(kThreads) void mover_kernel(const float* __restrict__ scores,
                                                         int64_t stride,
                                                         const int32_t* __restrict__ lens,
                                                         const int32_t* __restrict__ starts,
                                                         int32_t k, int32_t* __restrict__ out) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x;
  int32_t L = lens[b];
  int32_t s = starts ? starts[b] : 0;
  s = s < 0 ? 0 : (s > stride ? (int32_t)stride : s);
  L = L < 0 ? 0 : (L > stride - s ? (int32_t)(stride - s) : L);
  float acc = 0.f;
  if (L > k) {
    // the aligned column below the start; stride % 4 == 0, so every float4
    // of the span [s - s % 4, s + L) lies in the row
    const int32_t a = s & ~3;
    const v4f* row = reinterpret_cast<const v4f*>(scores + b * stride + a);
    const int32_t nv = (s + L - a + 3) >> 2;
    for (int32_t v0 = 0; v0 < nv; v0 += kUnroll * kThreads) {
      v4f x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t v = v0 + u * kThreads + t;
        x[u] = v < nv ? __builtin_nontemporal_load(row + v) : v4f{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc += (x[u].x + x[u].y) + (x[u].z + x[u].w);
    }
  }
  const int32_t base = (int32_t)__float_as_uint(acc) & 0xffff;
  int32_t* o = out + b * k;
  for (int32_t i = t; i < k; i += kThreads) __builtin_nontemporal_store(base + i, o + i);
}

}  // namespace

// scores: device fp32 [rows, stride] (16-byte aligned, stride % 4 == 0);
// lens: device int32 [rows]; starts: device int32 [rows] window starts, or
// NULL for 0 (clamped to the row like the lengths); out: device int32
// [rows, k]. Launches on `stream` and returns the launch status (0 on
// success, 1 on bad sizes).
extern "C" int bench_mover(const float* scores, int64_t stride, const int32_t* lens,
                           const int32_t* starts, int32_t rows, int32_t k, int32_t* out,
                           void* stream) {
  if (rows < 0 || k < 1 || stride < 0 || stride % 4 != 0) return 1;
  if (rows == 0) return 0;
  hipLaunchKernelGGL(mover_kernel, dim3(rows), dim3(kThreads), 0, (hipStream_t)stream, scores,
                     stride, lens, starts, k, out);
  return (int)hipPeekAtLastError();
}
