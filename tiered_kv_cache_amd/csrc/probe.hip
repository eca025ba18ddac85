// Read-bandwidth probe (a benchmark aid, not part of the method): how fast this GPU
// streams a buffer with the access pattern of the decode-attention kernel.
//
// One wave per SIMD (workgroups of four waves), wave w reading the contiguous byte
// range [w*B/W, (w+1)*B/W) in units of 16 KB, each unit sixteen 1 KB wave loads
// (16 bytes per lane, non-temporal), the next unit requested before the current
// one is consumed (up to two units in flight per wave) -- the geometry and load
// width of the attention kernel's key/value stream, without its arithmetic.  Each wave folds
// what it read into one word and stores it, so no load can be dropped.
#include "common.h"
#include "kernels.h"

namespace tkv {

constexpr int kProbeUnitBytes = 16 * 1024;

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

__global__ __launch_bounds__(256, 1) void read_probe_kernel(const uint4* buf, long units,
                                                            long waves, unsigned* sink) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= waves) return;
  const long u0 = w * units / waves, u1 = (w + 1) * units / waves;
  constexpr int kLoads = kProbeUnitBytes / 1024;  // 1 KB wave loads per unit
  uint4 cur[kLoads];
  unsigned acc = 0;
  if (u0 < u1) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) cur[i] = ld_nt(buf + u0 * (kProbeUnitBytes / 16) + i * 64 + lane);
  }
  for (long u = u0; u < u1; ++u) {
    uint4 nxt[kLoads];
    const bool more = u + 1 < u1;
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      nxt[i] = more ? ld_nt(buf + (u + 1) * (kProbeUnitBytes / 16) + i * 64 + lane)
                    : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) acc ^= cur[i].x ^ cur[i].y ^ cur[i].z ^ cur[i].w;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) cur[i] = nxt[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) sink[w] = acc;
}

void launch_read_probe(const void* buf, long units, long waves, unsigned* sink, hipStream_t s) {
  KernelTimer timer("read_probe", s);
  hipExtLaunchKernelGGL(read_probe_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s,
                        timer.start(), timer.stop(), 0, (const uint4*)buf, units, waves, sink);
}

}  // namespace tkv

using namespace tkv;

extern "C" tkv_status tkv_read_probe(const void* buf, size_t bytes, int32_t waves, uint32_t* sink,
                                     hipStream_t stream) {
  if (!buf || !sink) return fail(TKV_ERR_ARG, "null pointer");
  if (waves < 1 || waves > kMaxWorkers) return fail(TKV_ERR_ARG, "waves must be in [1, 8192]");
  if (bytes % kProbeUnitBytes || ((uintptr_t)buf & 15))
    return fail(TKV_ERR_ARG, "bytes must be a multiple of 16 KB and buf 16-byte aligned");
  launch_read_probe(buf, (long)(bytes / kProbeUnitBytes), waves, sink, stream);
  return hip_check(hipGetLastError(), "read_probe launch");
}
