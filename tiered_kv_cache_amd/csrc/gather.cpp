// T1 gather: host pack of a sequence's T1 rows into pinned staging, then the
// host-to-device copy of the staging on a side stream.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490), Methodologie section 1: T1 tokens live in host DDR at full
// precision and are brought to the GPU before each attention step.  The pack
// writes the rows in the device window's storage order (K-tiles, V-tiles) so the
// copy is one strided 2D transfer per tensor, served by the DMA engines from
// pinned memory.
#include <emmintrin.h>
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

// One 8-slot value panel group: dims [dg, dg + 16) of 8 source rows, written as
// 16 dimensions x 8 slots (256 contiguous bytes).  bf16: an SSE2 8x8 transpose of
// 16-bit lanes, twice; other element types: element by element.
template <typename E>
inline void panel16(E* out, const E* const* rows, int nr, int dg) {
  for (int d = 0; d < 16; ++d) {
    E vals[8];
    for (int e = 0; e < 8; ++e) vals[e] = e < nr ? rows[e][dg + d] : E(0);
    memcpy(out + d * 8, vals, sizeof(vals));
  }
}

template <>
inline void panel16<uint16_t>(uint16_t* out, const uint16_t* const* rows, int nr, int dg) {
  for (int half = 0; half < 2; ++half) {
    __m128i a[8];
    for (int e = 0; e < 8; ++e)
      a[e] = e < nr ? _mm_loadu_si128(reinterpret_cast<const __m128i*>(rows[e] + dg + 8 * half))
                    : _mm_setzero_si128();
    const __m128i t0 = _mm_unpacklo_epi16(a[0], a[1]), t1 = _mm_unpackhi_epi16(a[0], a[1]);
    const __m128i t2 = _mm_unpacklo_epi16(a[2], a[3]), t3 = _mm_unpackhi_epi16(a[2], a[3]);
    const __m128i t4 = _mm_unpacklo_epi16(a[4], a[5]), t5 = _mm_unpackhi_epi16(a[4], a[5]);
    const __m128i t6 = _mm_unpacklo_epi16(a[6], a[7]), t7 = _mm_unpackhi_epi16(a[6], a[7]);
    const __m128i u0 = _mm_unpacklo_epi32(t0, t2), u1 = _mm_unpackhi_epi32(t0, t2);
    const __m128i u2 = _mm_unpacklo_epi32(t1, t3), u3 = _mm_unpackhi_epi32(t1, t3);
    const __m128i u4 = _mm_unpacklo_epi32(t4, t6), u5 = _mm_unpackhi_epi32(t4, t6);
    const __m128i u6 = _mm_unpacklo_epi32(t5, t7), u7 = _mm_unpackhi_epi32(t5, t7);
    __m128i* o = reinterpret_cast<__m128i*>(out + 64 * half);  // dims 8 half + 0..7
    _mm_storeu_si128(o + 0, _mm_unpacklo_epi64(u0, u4));
    _mm_storeu_si128(o + 1, _mm_unpackhi_epi64(u0, u4));
    _mm_storeu_si128(o + 2, _mm_unpacklo_epi64(u1, u5));
    _mm_storeu_si128(o + 3, _mm_unpackhi_epi64(u1, u5));
    _mm_storeu_si128(o + 4, _mm_unpacklo_epi64(u2, u6));
    _mm_storeu_si128(o + 5, _mm_unpackhi_epi64(u2, u6));
    _mm_storeu_si128(o + 6, _mm_unpacklo_epi64(u3, u7));
    _mm_storeu_si128(o + 7, _mm_unpackhi_epi64(u3, u7));
  }
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
    std::vector<uint8_t> seen((size_t)max_ctx, 0);
    for (int i = 0; i < n_t1; ++i) {
      if (positions[i] < 0 || positions[i] >= max_ctx)
        return fail(TKV_ERR_ARG, "position outside [0, max_ctx)");
      if (seen[positions[i]]++) return fail(TKV_ERR_ARG, "repeated position");
    }
  }
  const size_t esz = model->kv_dtype == TKV_BF16 ? 2 : 4;
  const size_t row = esz * model->head_dim;
  const long lgs = (long)model->num_layers * model->num_kv_heads;

  const int D = model->head_dim;
  const long nblocks = (n_t1 + 31) / 32;  // 32-slot blocks of the tile layouts
  if (positions && n_t1 > 0) {
    // Work item: one 32-slot block of one (layer, KV head), keys and values.  Both
    // are written in storage order -- a K-tile as [tile][chunk][16 rows] of 8-element
    // chunks, a V-tile as [dim group][panel][16 dims] of 8-slot panels -- so the
    // staging stores are sequential and the 32 source rows stay in the L1 cache.
    const long total = lgs * nblocks;
    const int nt = (int)std::min<long>(pack_threads(), std::max<long>(1, total / 16));
    auto pack = [&](auto* sk_base, auto* sv_base, const auto* hk_base, const auto* hv_base,
                    long lo, long hi) {
      using E = std::remove_const_t<std::remove_pointer_t<decltype(hk_base)>>;
      const E* rk[32];
      const E* rv[32];
      for (long it = lo; it < hi; ++it) {
        const long lg = it / nblocks;
        const long blk = it - lg * nblocks;
        const long r0 = blk * 32;
        const int nr = (int)std::min<long>(32, n_t1 - r0);
        for (int i = 0; i < nr; ++i) {
          const size_t src = ((size_t)lg * max_ctx + positions[r0 + i]) * D;
          rk[i] = hk_base + src;
          rv[i] = hv_base + src;
        }
        E* tk = sk_base + ((size_t)lg * cap1 + r0) * D;
        E* tv = sv_base + ((size_t)lg * cap1 + r0) * D;
        // keys: slot r = 8j + 4u + i is row 4j + i of tile u
        for (int u = 0; u < 2; ++u)
          for (int c = 0; c < D; c += 8)
            for (int row = 0; row < 16; ++row) {
              const int r = ((row >> 2) << 3) + 4 * u + (row & 3);
              E* to = tk + k_off(r, c, D);
              if (r < nr) memcpy(to, rk[r] + c, 8 * sizeof(E));
              else memset(to, 0, 8 * sizeof(E));
            }
        // values: the 8 slots of a panel for one dimension are contiguous
        for (int dg = 0; dg < D; dg += 16)
          for (int pn = 0; pn < 4; ++pn)
            panel16<E>(tv + v_off(8 * pn, dg, D), rv + 8 * pn, nr - 8 * pn, dg);
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
