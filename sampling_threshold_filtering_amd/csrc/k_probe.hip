// Practical read ceiling of the filter's roofline: one streaming read of x with the
// filter's loads (dwordx4, non-temporal) and nothing else.  The filter of stage 3 of
// Prof-K ("Prof-K: Probabilistic One-Pass Filtering for Efficient Top-k Selection", §3
// stage 3; App. C) reads each input value once; its time cannot drop below this
// kernel's on the same buffer, which is what the measurement reports beside the
// published 8 TB/s.
//
// The read order is the filter's: the blocks of die x (b mod 8 = x, which the
// dispatcher places round-robin on the dies) own a contiguous range of wave-tiles (64
// lanes x U float4, U = 4: 4 KB) and deal it block-cyclically over their wavefronts, so
// the die's wavefronts sweep it together; the next tile's loads are issued before the
// current one is folded (two register sets).  The values are folded into an XOR of
// their bits (so the loads stay live), reduced per block and XORed into *out with one
// atomic per block: *out ends up XORed with the XOR of all N values' bits, which a test
// can check.
#include "launch.h"

namespace profk {

namespace {
constexpr int kProbeThreads = 256;
constexpr int kProbeWaves = kProbeThreads / kWave;
constexpr int kProbeU = 4;
typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32 fold4(const f4& v) {
  return __float_as_uint(v.x) ^ __float_as_uint(v.y) ^ __float_as_uint(v.z) ^ __float_as_uint(v.w);
}
}  // namespace

__global__ __launch_bounds__(kProbeThreads) void read_ceiling_kernel(const float* x, u64 N, unsigned long long* out) {
  __shared__ u32 s_acc[kProbeWaves];
  const u32 lane = lane_id(), wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const f4* xv = reinterpret_cast<const f4*>(x);
  const u64 nvec = N >> 2;
  const u64 per_tile = (u64)kProbeU * kWave;
  const u64 ntiles = (nvec + per_tile - 1) / per_tile;
  // die x's tile range and its wavefronts
  const u32 xcd = blockIdx.x % kXcds;
  const u64 nbx = (gridDim.x - xcd + kXcds - 1) / kXcds;
  const u64 nwx = nbx * kProbeWaves;
  const u64 wx = (u64)(blockIdx.x / kXcds) * kProbeWaves + wid;
  const u64 t0 = ntiles * xcd / kXcds, t1 = ntiles * (xcd + 1) / kXcds;
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
  u64 tile = t0 + wx;
  if (tile < t1) load(tile, a);
  while (tile < t1) {
    const u64 n1 = tile + nwx;
    if (n1 < t1) load(n1, b);
    fold(a);
    if (n1 >= t1) break;
    const u64 n2 = n1 + nwx;
    if (n2 < t1) load(n2, a);
    fold(b);
    tile = n2;
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
    for (int w = 0; w < kProbeWaves; ++w) t ^= s_acc[w];
    atomicXor(out, (unsigned long long)t);
  }
}

hipError_t launch_read_ceiling(const float* x, u64 N, u32 blocks_per_cu, unsigned long long* out, hipStream_t s) {
  const u32 bpc = blocks_per_cu ? blocks_per_cu : 2u;
  read_ceiling_kernel<<<bpc * device_cu_count(), kProbeThreads, 0, s>>>(x, N, out);
  return hipGetLastError();
}

}  // namespace profk
