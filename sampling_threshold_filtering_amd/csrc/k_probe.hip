// Practical read ceiling of the filter's roofline: one streaming read of x with the
// filter's loads (dwordx4, non-temporal) and nothing else.  The filter of stage 3 of
// Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k Selection", §3
// stage 3; App. C) reads each input value once; its time cannot drop below this
// kernel's on the same buffer, which is what the measurement reports beside the
// published 8 TB/s.
//
// Each wavefront streams wave-tiles of 64 lanes x U float4 (U = 8: 8 KB) in a
// grid-stride order, with the next tile's loads issued before the current one is
// folded (two register sets), so every wavefront keeps U dwordx4 loads in flight.  The
// values are folded into an XOR of their bits (so the loads stay live), reduced per
// block and XORed into *out with one atomic per block: *out ends up XORed with the XOR
// of all N values' bits, which a test can check.
#include "launch.h"

namespace profk {

namespace {
constexpr int kProbeThreads = 256;
constexpr int kProbeU = 8;
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32 fold4(const f4& v) {
  return __float_as_uint(v.x) ^ __float_as_uint(v.y) ^ __float_as_uint(v.z) ^ __float_as_uint(v.w);
}
}  // namespace

__global__ __launch_bounds__(kProbeThreads) void read_ceiling_kernel(const float* x, u64 N, unsigned long long* out) {
  __shared__ u32 s_acc[kProbeThreads / kWave];
  const u32 lane = lane_id(), wid = threadIdx.x / kWave;
  const f4* xv = reinterpret_cast<const f4*>(x);
  const u64 nvec = N >> 2;
  const u64 per_tile = (u64)kProbeU * kWave;
  const u64 ntiles = (nvec + per_tile - 1) / per_tile;
  const u64 nw = (u64)gridDim.x * (kProbeThreads / kWave);
  u64 tile = (u64)blockIdx.x * (kProbeThreads / kWave) + wid;
  u32 acc = 0;
  f4 a[kProbeU], b[kProbeU];
  auto load = [&](u64 tl, f4 (&v)[kProbeU]) {
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) {
      const u64 vi = tl * per_tile + (u64)u * kWave + lane;
      v[u] = vi < nvec ? __builtin_nontemporal_load(xv + vi) : f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto fold = [&](const f4 (&v)[kProbeU]) {
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) acc ^= fold4(v[u]);
  };
  if (tile < ntiles) load(tile, a);
  while (tile < ntiles) {
    const u64 t1 = tile + nw;
    if (t1 < ntiles) load(t1, b);
    fold(a);
    if (t1 >= ntiles) break;
    const u64 t2 = t1 + nw;
    if (t2 < ntiles) load(t2, a);
    fold(b);
    tile = t2;
  }
  // the scalar tail (N mod 4 values)
  if (blockIdx.x == 0 && wid == 0) {
    const u64 i = 4 * nvec + lane;
    if (i < N) acc ^= __float_as_uint(x[i]);
  }
  acc = wave_reduce_u32(acc, [](u32 p, u32 q) { return p ^ q; });
  if (lane == 0) s_acc[wid] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32 t = 0;
    for (int w = 0; w < kProbeThreads / kWave; ++w) t ^= s_acc[w];
    atomicXor(out, (unsigned long long)t);
  }
}

hipError_t launch_read_ceiling(const float* x, u64 N, u32 blocks_per_cu, unsigned long long* out, hipStream_t s) {
  const u32 bpc = blocks_per_cu ? blocks_per_cu : 4u;
  read_ceiling_kernel<<<bpc * device_cu_count(), kProbeThreads, 0, s>>>(x, N, out);
  return hipGetLastError();
}

}  // namespace profk
