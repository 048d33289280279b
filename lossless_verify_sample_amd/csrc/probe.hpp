// Plain streaming-read probe (a measurement aid, not part of the method):
// reads a buffer once with 16-byte loads and folds the words into one value
// per workgroup, so that the read bandwidth the streaming passes could reach
// on this part is measured by the same library.  Layouts: one-shot grids
// (each workgroup one chunk of WGT * L 16-byte loads, all issued before any
// is used) and persistent grids (a fixed set of workgroups looping over the
// chunks, the next chunk's loads issued before the current one is folded).
#pragma once

#include "device.hpp"

namespace ssd {

template <int L>
__device__ __forceinline__ uint32_t fold(const u32x4 (&v)[L]) {
  uint32_t a = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) a ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  return a;
}

template <int WGT, int L, bool NT>
__device__ __forceinline__ void probe_load(const u32x4* p, int64_t chunk, int64_t n16, u32x4 (&v)[L]) {
  const int64_t base = chunk * (int64_t)(WGT * L) + threadIdx.x;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int64_t k = min(base + (int64_t)i * WGT, n16 - 1);
    v[i] = NT ? __builtin_nontemporal_load(p + k) : p[k];
  }
}

template <int WGT, int L, bool NT, bool XCD>
__global__ __launch_bounds__(WGT) void k_probe_once(const u32x4* p, int64_t n16, uint32_t* out) {
  int64_t chunk = blockIdx.x;
  if constexpr (XCD) {
    // consecutive chunks on one XCD: workgroups are dealt to the 8 XCDs in turn
    const int64_t g = gridDim.x, per = (g + 7) / 8;
    const int64_t c = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
    chunk = c < g ? c : blockIdx.x;
  }
  u32x4 v[L];
  probe_load<WGT, L, NT>(p, chunk, n16, v);
  const uint32_t a = fold<L>(v);
  if (a == 0x9e3779b9u) out[blockIdx.x] = a;  // keeps the loads live; almost never stores
}

template <int WGT, int L, bool NT>
__global__ __launch_bounds__(WGT) void k_probe_persist(const u32x4* p, int64_t n16, int64_t nchunk, uint32_t* out) {
  u32x4 a[L], b[L];
  uint32_t acc = 0;
  int64_t c = blockIdx.x;
  if (c < nchunk) probe_load<WGT, L, NT>(p, c, n16, a);
  while (c < nchunk) {
    const int64_t nx = c + gridDim.x;
    if (nx < nchunk) probe_load<WGT, L, NT>(p, nx, n16, b);
    acc ^= fold<L>(a);
#pragma unroll
    for (int i = 0; i < L; ++i) a[i] = b[i];
    c = nx;
  }
  if (acc == 0x9e3779b9u) out[blockIdx.x] = acc;
}

}  // namespace ssd
