// T1 gather: host pack of a sequence's T1 rows into pinned staging, then the
// host-to-device copy of the staging on a side stream.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490), Methodologie section 1: T1 tokens live in host DDR at full
// precision and are brought to the GPU before each attention step.  The pack
// writes the rows in the device window's storage order (K-tiles, V-tiles),
// each (layer, KV head) row holding its cap1 key slots and then its cap1 value
// slots, so the copy is one strided 2D transfer served by the DMA engines from
// pinned memory.
//
// Two packers share the layout code:
//   pack_t1_blocks -- every slot [0, n) of a window from a list of positions,
//                     32-slot block by block (tkv_gather_t1);
//   pack_t1_slots  -- a list of (slot, position) pairs, slot by slot (the
//                     differential refresh after a reassignment: only the slots
//                     whose position changed are rewritten).
#include <emmintrin.h>
#include <sched.h>
#include <string.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace tkv {

int host_threads() {
  cpu_set_t set;
  int n = 0;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) n = CPU_COUNT(&set);
  if (n <= 0) n = (int)std::thread::hardware_concurrency();
  return std::max(1, std::min(n, 16));
}

namespace {

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

// Work item: one 32-slot block of one (layer, KV head) row of the window, keys
// and values.  Both are written in storage order -- a K-tile as [tile][chunk][16
// rows] of 8-element chunks, a V-tile as [dim group][panel][16 dims] of 8-slot
// panels -- so the staging stores are sequential and the 32 source rows stay in
// the L1 cache.  Slots past n of the last block are zero.
template <typename E>
void pack_blocks(E* stg, const E* hk, const E* hv, long store_rs, long lgs, int D, int cap1,
                 const int32_t* positions, int n, long lo, long hi) {
  const long nblocks = (n + 31) / 32;
  const E* rk[32];
  const E* rv[32];
  for (long it = lo; it < hi; ++it) {
    const long lg = it / nblocks;
    const long blk = it - lg * nblocks;
    const long r0 = blk * 32;
    const int nr = (int)std::min<long>(32, n - r0);
    for (int i = 0; i < nr; ++i) {
      const size_t src = (size_t)lg * store_rs + (size_t)positions[r0 + i] * D;
      rk[i] = hk + src;
      rv[i] = hv + src;
    }
    E* tk = stg + (size_t)lg * 2 * cap1 * D + (size_t)r0 * D;
    E* tv = tk + (size_t)cap1 * D;
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
      for (int pn = 0; pn < 4; ++pn) panel16<E>(tv + v_off(8 * pn, dg, D), rv + 8 * pn, nr - 8 * pn, dg);
  }
}

// Work item: one (layer, KV head) row; every listed slot of it is rewritten.
template <typename E>
void pack_slots(E* stg, const E* hk, const E* hv, long store_rs, int D, int cap1,
                const int32_t* slots, const int32_t* positions, int n, long lo, long hi) {
  for (long lg = lo; lg < hi; ++lg) {
    E* tk = stg + (size_t)lg * 2 * cap1 * D;
    E* tv = tk + (size_t)cap1 * D;
    for (int i = 0; i < n; ++i) {
      const long s = slots[i];
      const E* k = hk + (size_t)lg * store_rs + (size_t)positions[i] * D;
      const E* v = hv + (size_t)lg * store_rs + (size_t)positions[i] * D;
      for (int c = 0; c < D; c += 8) memcpy(tk + k_off(s, c, D), k + c, 8 * sizeof(E));
      for (int d = 0; d < D; ++d) tv[v_off(s, d, D)] = v[d];
    }
  }
}

}  // namespace

void pack_t1_blocks(const tkv_model* m, const void* store_k, const void* store_v, int max_ctx,
                    const int32_t* positions, int n, void* staging, int cap1) {
  const long lgs = (long)m->num_layers * m->num_kv_heads;
  const long total = lgs * ((n + 31) / 32);
  if (total == 0) return;
  const int D = m->head_dim;
  const long rs = (long)max_ctx * D;
  const int nt = (int)std::min<long>(host_threads(), std::max<long>(1, total / 16));
  parallel_ranges(total, nt, [&](long lo, long hi) {
    if (m->kv_dtype == TKV_BF16)
      pack_blocks((uint16_t*)staging, (const uint16_t*)store_k, (const uint16_t*)store_v, rs, lgs,
                  D, cap1, positions, n, lo, hi);
    else
      pack_blocks((uint32_t*)staging, (const uint32_t*)store_k, (const uint32_t*)store_v, rs, lgs,
                  D, cap1, positions, n, lo, hi);
  });
}

void pack_t1_slots(const tkv_model* m, const void* store_k, const void* store_v, int max_ctx,
                   const int32_t* slots, const int32_t* positions, int n, void* staging,
                   int cap1) {
  if (n == 0) return;
  const long lgs = (long)m->num_layers * m->num_kv_heads;
  const int D = m->head_dim;
  const long rs = (long)max_ctx * D;
  const int nt = (int)std::min<long>(host_threads(), std::max<long>(1, lgs * n / 512));
  parallel_ranges(lgs, nt, [&](long lo, long hi) {
    if (m->kv_dtype == TKV_BF16)
      pack_slots((uint16_t*)staging, (const uint16_t*)store_k, (const uint16_t*)store_v, rs, D,
                 cap1, slots, positions, n, lo, hi);
    else
      pack_slots((uint32_t*)staging, (const uint32_t*)store_k, (const uint32_t*)store_v, rs, D,
                 cap1, slots, positions, n, lo, hi);
  });
}

}  // namespace tkv

using namespace tkv;

extern "C" tkv_status tkv_gather_t1(const tkv_model* model, const void* host_k,
                                    const void* host_v, int32_t max_ctx,
                                    const int32_t* positions, int32_t n_t1, void* staging,
                                    int32_t cap1, void* dev_t1, hipStream_t side_stream,
                                    hipEvent_t ready) {
  if (!model) return fail(TKV_ERR_ARG, "model is null");
  if (model->num_layers < 1 || model->num_kv_heads < 1 ||
      (model->head_dim != 64 && model->head_dim != 128) ||
      (model->kv_dtype != TKV_BF16 && model->kv_dtype != TKV_F32))
    return fail(TKV_ERR_ARG, "bad model shape");
  if (n_t1 < 0 || cap1 < 0 || max_ctx < 0) return fail(TKV_ERR_ARG, "negative size");
  if (n_t1 > cap1) return fail(TKV_ERR_CAPACITY, "n_t1 > cap1");
  if (cap1 % 32) return fail(TKV_ERR_ARG, "cap1 must be a multiple of 32");
  if (!staging) return fail(TKV_ERR_ARG, "staging is null");
  if (positions) {
    if (!host_k || !host_v) return fail(TKV_ERR_ARG, "host store is null");
    std::vector<uint8_t> seen((size_t)max_ctx, 0);
    for (int i = 0; i < n_t1; ++i) {
      if (positions[i] < 0 || positions[i] >= max_ctx)
        return fail(TKV_ERR_ARG, "position outside [0, max_ctx)");
      if (seen[positions[i]]++) return fail(TKV_ERR_ARG, "repeated position");
    }
  }
  const size_t slot_bytes = (model->kv_dtype == TKV_BF16 ? 2 : 4) * (size_t)model->head_dim;
  const long lgs = (long)model->num_layers * model->num_kv_heads;
  if (positions && n_t1 > 0) {
    // an earlier copy queued on the side stream may still be reading the staging (a
    // pack-only call leaves that ordering to its caller)
    if (dev_t1) {
      tkv_status st = hip_check(hipStreamSynchronize(side_stream), "side stream sync");
      if (st) return st;
    }
    pack_t1_blocks(model, host_k, host_v, max_ctx, positions, n_t1, staging, cap1);
  }
  if (dev_t1 && n_t1 > 0) {
    KernelTimer timer("gather_t1_h2d", side_stream);
    const size_t pitch = (size_t)cap1 * slot_bytes;
    const size_t width = (size_t)((n_t1 + 31) / 32 * 32) * slot_bytes;  // whole 32-slot blocks
    tkv_status st = hip_check(hipMemcpy2DAsync(dev_t1, pitch, staging, pitch, width, 2 * lgs,
                                               hipMemcpyHostToDevice, side_stream),
                              "T1 copy");
    if (st) return st;
  }
  if (ready) return hip_check(hipEventRecord(ready, side_stream), "event record");
  return TKV_OK;
}
