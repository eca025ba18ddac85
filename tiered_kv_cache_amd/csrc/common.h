// Internal helpers of libtkv (device math, launch bookkeeping).  Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <string>
#include <thread>
#include <vector>

#include "../../include/tkv.h"

namespace tkv {

// Sequences handled by one launch; larger batches are split on the host.
constexpr int kMaxSeqPerLaunch = 64;
constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// element access: bf16 bit patterns (uint16_t) or float32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float to_f32(float f) { return f; }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// wave64 reductions (cross-lane through ds_swizzle/bpermute as the compiler picks)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// Block-wide exclusive scan of one int per thread (blockDim.x a multiple of 64,
// at most 1024).  `tmp` holds at least blockDim.x/64 + 1 ints of LDS.  Returns
// the exclusive prefix; *total receives the block sum.  Contains barriers: every
// thread of the block must call it.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int incl = wave_incl_scan_i(v);
  if (lane == kWave - 1) tmp[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      int t = tmp[w];
      tmp[w] = run;
      run += t;
    }
    tmp[nw] = run;
  }
  __syncthreads();
  int res = tmp[wid] + incl - v;
  *total = tmp[nw];
  __syncthreads();
  return res;
}

__device__ __forceinline__ int block_sum_i(int v, int* tmp) {
  int total;
  (void)block_excl_scan(v, tmp, &total);
  return total;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
void set_error(const std::string& msg);
tkv_status fail(tkv_status code, const std::string& msg);
tkv_status hip_check(hipError_t e, const char* what);

// Optional event timing around each launch (see tkv_timing_*).
// The two events go to hipExtLaunchKernelGGL, which records them when the
// kernel itself starts and ends (no launch gap inside the interval).
struct KernelTimer {
  KernelTimer(const char* name, hipStream_t s);
  ~KernelTimer();
  hipEvent_t start() const { return start_; }
  hipEvent_t stop() const { return stop_; }
  const char* name_;
  hipEvent_t start_, stop_;  // null when timing is off
};

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Host threads for the library's host-side copies: the process's CPU affinity,
// at most 16.
int host_threads();

// Runs f(lo, hi) over [0, total) split into at most `nt` contiguous ranges, on
// the calling thread and nt - 1 helpers.
template <class F>
void parallel_ranges(long total, int nt, F f) {
  nt = (int)std::max<long>(1, std::min<long>(nt, total));
  if (nt == 1) {
    if (total > 0) f(0L, total);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(nt - 1);
  for (int t = 1; t < nt; ++t) pool.emplace_back([&, t] { f(total * t / nt, total * (t + 1) / nt); });
  f(0L, total / nt);
  for (auto& th : pool) th.join();
}

}  // namespace tkv
