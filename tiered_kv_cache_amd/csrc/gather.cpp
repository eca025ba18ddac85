// T1 gather: host pack of a sequence's T1 rows into pinned staging, then the
// host-to-device copy of the staging on a side stream.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490), Methodologie section 1: T1 tokens live in host DDR at full
// precision and are brought to the GPU before each attention step.  The pack
// writes the rows in the device window's storage order (K-tiles, V-tiles) so the
// copy is one strided 2D transfer per tensor, served by the DMA engines from
// pinned memory.
#include <sched.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <type_traits>
#include <vector>

#include "common.h"
#include "layout.h"

namespace {

int pack_threads() {
  cpu_set_t set;
  int n = 0;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) n = CPU_COUNT(&set);
  if (n <= 0) n = (int)std::thread::hardware_concurrency();
  return std::max(1, std::min(n, 16));
}

}  // namespace

using namespace tkv;

extern "C" tkv_status tkv_gather_t1(const tkv_model* model, const void* host_k,
                                    const void* host_v, int32_t max_ctx,
                                    const int32_t* positions, int32_t n_t1, void* staging_k,
                                    void* staging_v, int32_t cap1, void* dev_k_t1,
                                    void* dev_v_t1, hipStream_t side_stream, hipEvent_t ready) {
  if (!model) return fail(TKV_ERR_ARG, "model is null");
  if (model->num_layers < 1 || model->num_kv_heads < 1 ||
      (model->head_dim != 64 && model->head_dim != 128) ||
      (model->kv_dtype != TKV_BF16 && model->kv_dtype != TKV_F32))
    return fail(TKV_ERR_ARG, "bad model shape");
  if (n_t1 < 0 || cap1 < 0 || max_ctx < 0) return fail(TKV_ERR_ARG, "negative size");
  if (n_t1 > cap1) return fail(TKV_ERR_CAPACITY, "n_t1 > cap1");
  if (cap1 % 32) return fail(TKV_ERR_ARG, "cap1 must be a multiple of 32");
  if (!staging_k || !staging_v) return fail(TKV_ERR_ARG, "staging is null");
  if ((dev_k_t1 == nullptr) != (dev_v_t1 == nullptr))
    return fail(TKV_ERR_ARG, "both or neither device windows must be given");
  if (positions) {
    if (!host_k || !host_v) return fail(TKV_ERR_ARG, "host store is null");
    for (int i = 0; i < n_t1; ++i) {
      if (positions[i] < 0 || positions[i] >= max_ctx)
        return fail(TKV_ERR_ARG, "position outside [0, max_ctx)");
      if (i > 0 && positions[i] <= positions[i - 1])
        return fail(TKV_ERR_ARG, "positions must be strictly ascending");
    }
  }
  const size_t esz = model->kv_dtype == TKV_BF16 ? 2 : 4;
  const size_t row = esz * model->head_dim;
  const long lgs = (long)model->num_layers * model->num_kv_heads;

  const int D = model->head_dim;
  const long nblocks = (n_t1 + 31) / 32;  // 32-slot blocks of the tile layouts
  if (positions && n_t1 > 0) {
    const long krows = lgs * n_t1;
    const long vpanels = lgs * nblocks * 4;
    const long total = krows + vpanels * 8;  // work units: K rows, then V panels (8 rows each)
    const int nt = (int)std::min<long>(pack_threads(), std::max<long>(1, total / 2048));
    auto pack = [&](auto* sk_base, auto* sv_base, const auto* hk_base, const auto* hv_base,
                    long lo, long hi) {
      using E = std::remove_const_t<std::remove_pointer_t<decltype(hk_base)>>;
      // K rows in [0, krows): 8-element chunks to their K-tile places
      for (long i = lo; i < std::min(hi, krows); ++i) {
        const long lg = i / n_t1;
        const long r = i - lg * n_t1;
        const E* from = hk_base + ((size_t)lg * max_ctx + positions[r]) * D;
        E* to = sk_base + (size_t)lg * cap1 * D;
        for (int c = 0; c < D; c += 8) memcpy(to + k_off(r, c, D), from + c, 8 * sizeof(E));
      }
      // V panels: units [krows, total) in steps of 8
      const long vlo = std::max(lo, krows);
      if (hi <= vlo) return;
      const long plo = (vlo - krows + 7) / 8, phi = (hi - krows + 7) / 8;
      for (long i = plo; i < phi; ++i) {
        const long lg = i / (nblocks * 4);
        const long p = i - lg * nblocks * 4;  // panel: slots 8p .. 8p+7
        E* to = sv_base + (size_t)lg * cap1 * D;
        for (int e = 0; e < 8; ++e) {
          const long r = 8 * p + e;
          if (r < n_t1) {
            const E* from = hv_base + ((size_t)lg * max_ctx + positions[r]) * D;
            for (int d = 0; d < D; ++d) to[v_off(r, d, D)] = from[d];
          } else {
            for (int d = 0; d < D; ++d) to[v_off(r, d, D)] = E(0);
          }
        }
      }
    };
    auto work = [&](int t) {
      const long lo = total * t / nt, hi = total * (t + 1) / nt;
      if (esz == 2)
        pack((uint16_t*)staging_k, (uint16_t*)staging_v, (const uint16_t*)host_k,
             (const uint16_t*)host_v, lo, hi);
      else
        pack((uint32_t*)staging_k, (uint32_t*)staging_v, (const uint32_t*)host_k,
             (const uint32_t*)host_v, lo, hi);
    };
    if (nt == 1) {
      work(0);
    } else {
      std::vector<std::thread> pool;
      pool.reserve(nt - 1);
      for (int t = 1; t < nt; ++t) pool.emplace_back(work, t);
      work(0);
      for (auto& th : pool) th.join();
    }
  }
  if (dev_k_t1 && n_t1 > 0) {
    const size_t pitch = (size_t)cap1 * row;
    KernelTimer timer("gather_t1_h2d", side_stream);
    const size_t width = (size_t)nblocks * 32 * row;  // whole 32-slot blocks
    tkv_status st = hip_check(hipMemcpy2DAsync(dev_k_t1, pitch, staging_k, pitch, width, lgs,
                                               hipMemcpyHostToDevice, side_stream),
                              "T1 key copy");
    if (st) return st;
    st = hip_check(hipMemcpy2DAsync(dev_v_t1, pitch, staging_v, pitch, width, lgs,
                                    hipMemcpyHostToDevice, side_stream),
                   "T1 value copy");
    if (st) return st;
  }
  if (ready) return hip_check(hipEventRecord(ready, side_stream), "event record");
  return TKV_OK;
}
