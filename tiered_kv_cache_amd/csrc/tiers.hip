// Tier assignment, pool compaction and the append of a new token.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490).  Methodologie section 1: protected prompt/sink/recent tokens and
// the most important tokens stay in T0, medium ones go to T1, low ones to T2,
// and only the least important tail is dropped (T3).  Section 4: tiers are
// recomputed every Delta steps.  Each generated token adds one key/value pair
// (Enonce du probleme).
//
// assign_tiers  -- one workgroup per sequence.  The ranking the method sorts by
//                  is realised as three order-statistic selections (evict,
//                  then T2, then T1), each an 8-bit LDS radix select over a
//                  monotone uint32 key of the float32 score, with ties at the
//                  threshold resolved by position (the higher positions leave
//                  first) through a block scan.  No sort is materialised.
// compact_scan  -- one workgroup per sequence: block scans over positions map
//                  every new T0/T1 slot to its source slot in the previous
//                  pool/window and list the positions newly in T2.
// compact_copy  -- moves the rows into the new pool/window (K-tile chunks and
//                  V-tile panels, written in destination order).
// append        -- writes the new token's K/V row into its T0 slot.
#include <limits.h>

#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace tkv {

constexpr int kTierThreads = 1024;

// Ascending key order == ascending score order; -0 ranks as +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A selection of the k least important candidates: key < T, or key == T and
// position >= cut.  The empty selection is T = 0, cut = INT_MAX.
struct Sel {
  uint32_t T;
  int cut;
};
__device__ __forceinline__ bool in_sel(const Sel& s, uint32_t key, int p) {
  return key < s.T || (key == s.T && p >= s.cut);
}

// k (block-uniform) least important candidates among positions [0, n).
template <class Cand>
__device__ Sel radix_select(int k, int n, const float* sc, const uint8_t* tp, Cand cand,
                            unsigned* hist, int* tmp, int* sh) {
  Sel r;
  r.T = 0u;
  r.cut = INT_MAX;
  if (k <= 0) return r;
  const int tid = threadIdx.x;
  uint32_t prefix = 0u;
  int kk = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kTierThreads) hist[i] = 0u;
    __syncthreads();
    const uint32_t himask = (shift == 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int p = tid; p < n; p += kTierThreads) {
      const uint32_t key = score_key(sc[p]);
      if ((key & himask) == prefix && cand(p, tp[p], key))
        atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, d = 0;
      for (; d < 255; ++d) {
        const int h = (int)hist[d];
        if (cum + h >= kk) break;
        cum += h;
      }
      sh[0] = d;
      sh[1] = kk - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)sh[0] << shift;
    kk = sh[1];
    __syncthreads();
  }
  // kk candidates with key == prefix remain to be taken: the highest positions.
  // Thread t owns positions [n - (t+1)*seg, n - t*seg): a forward scan over
  // threads counts ties above each segment.
  const int seg = (n + kTierThreads - 1) / kTierThreads;
  const int hi = max(0, n - tid * seg);
  const int lo = max(0, n - (tid + 1) * seg);
  int cnt = 0;
  for (int p = lo; p < hi; ++p) {
    const uint32_t key = score_key(sc[p]);
    if (key == prefix && cand(p, tp[p], key)) ++cnt;
  }
  int total;
  const int excl = block_excl_scan(cnt, tmp, &total);
  if (excl < kk && kk <= excl + cnt) {
    int need = kk - excl;
    for (int p = hi - 1; p >= lo; --p) {
      const uint32_t key = score_key(sc[p]);
      if (key == prefix && cand(p, tp[p], key)) {
        if (--need == 0) {
          sh[2] = p;
          break;
        }
      }
    }
  }
  __syncthreads();
  r.T = prefix;
  r.cut = sh[2];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTierThreads) void assign_tiers_kernel(TierArgs a) {
  __shared__ unsigned hist[256];
  __shared__ int tmp[kTierThreads / kWave + 1];
  __shared__ int sh[4];
  const int tid = threadIdx.x;
  const int bl = blockIdx.x;
  const long b = a.b_offset + bl;
  const int n = a.n[bl];
  const float* sc = a.scores + b * a.max_ctx;
  const uint8_t* tp = a.tprev + b * a.max_ctx;
  uint8_t* tn = a.tnext + b * a.max_ctx;
  int* counts = a.counts + b * 4;
  const int prot_lo = a.prot_lo;
  const int prot_hi = n - a.recent;  // positions >= prot_hi are the recent window
  auto prot = [=](int p) { return p < prot_lo || p >= prot_hi; };

  int cE = 0, cT2 = 0, cPool = 0, cBad = 0;
  for (int p = tid; p < n; p += kTierThreads) {
    const int t = tp[p];
    if (t > 3) ++cBad;
    else if (t == 3) ++cE;
    else {
      if (t == 2) ++cT2;
      if (!prot(p)) ++cPool;
    }
  }
  cBad = block_sum_i(cBad, tmp);
  if (cBad) {
    if (tid < 4) counts[tid] = -1;
    return;
  }
  cE = block_sum_i(cE, tmp);
  cT2 = block_sum_i(cT2, tmp);
  cPool = block_sum_i(cPool, tmp);

  // 1. eviction from the pool (non-protected T0/T1/T2)
  const int e = min(max(a.n3[bl] - cE, 0), cPool);
  auto cand1 = [=](int p, int t, uint32_t) { return t <= 2 && !prot(p); };
  const Sel s1 = radix_select(e, n, sc, tp, cand1, hist, tmp, sh);

  int cEvT2 = 0, cLive = 0;
  for (int p = tid; p < n; p += kTierThreads) {
    const int t = tp[p];
    if (t > 2 || prot(p)) continue;
    const bool ev = in_sel(s1, score_key(sc[p]), p);
    if (t == 2 && ev) ++cEvT2;
    if (t <= 1 && !ev) ++cLive;
  }
  cEvT2 = block_sum_i(cEvT2, tmp);
  cLive = block_sum_i(cLive, tmp);

  // 2. T2 from live (non-protected T0/T1 not just evicted)
  const int survivors = cT2 - cEvT2;
  const int q = min(max(a.n2[bl] - survivors, 0), cLive);
  auto cand2 = [=](int p, int t, uint32_t key) {
    return t <= 1 && !prot(p) && !in_sel(s1, key, p);
  };
  const Sel s2 = radix_select(q, n, sc, tp, cand2, hist, tmp, sh);

  // 3. T1 from what is left of live
  const int r1 = min(a.n1[bl], cLive - q);
  auto cand3 = [=](int p, int t, uint32_t key) {
    return t <= 1 && !prot(p) && !in_sel(s1, key, p) && !in_sel(s2, key, p);
  };
  const Sel s3 = radix_select(r1, n, sc, tp, cand3, hist, tmp, sh);

  int c[4] = {0, 0, 0, 0};
  for (int p = tid; p < n; p += kTierThreads) {
    const int t = tp[p];
    const uint32_t key = score_key(sc[p]);
    const bool np = !prot(p);
    int nt;
    if (t == 3) nt = 3;
    else if (np && in_sel(s1, key, p)) nt = 3;
    else if (t == 2) nt = 2;
    else if (np && in_sel(s2, key, p)) nt = 2;
    else if (np && in_sel(s3, key, p)) nt = 1;
    else nt = 0;
    tn[p] = (uint8_t)nt;
    ++c[nt];
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int v = block_sum_i(c[t], tmp);
    if (tid == 0) counts[t] = v;
  }
}

void launch_assign_tiers(const TierArgs& a, int nb, hipStream_t s) {
  KernelTimer timer("assign_tiers", s);
  hipLaunchKernelGGL(assign_tiers_kernel, dim3(nb), dim3(kTierThreads), 0, s, a);
}

// ---------------------------------------------------------------------------
// compaction
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kTierThreads) void compact_scan_kernel(CompactArgs a) {
  __shared__ int tmp[kTierThreads / kWave + 1];
  const int tid = threadIdx.x;
  const int bl = blockIdx.x;
  const long b = a.b_offset + bl;
  const int n = a.n[bl];
  const uint8_t* tp = a.tprev + b * a.max_ctx;
  const uint8_t* tn = a.tnext + b * a.max_ctx;
  const int seg = (n + kTierThreads - 1) / kTierThreads;
  const int lo = min(n, tid * seg);
  const int hi = min(n, lo + seg);

  int cp0 = 0, cp1 = 0, cn0 = 0, cn1 = 0, ct2 = 0, bad = 0;
  for (int p = lo; p < hi; ++p) {
    const int o = tp[p], w = tn[p];
    if (o > 3 || w > 3) ++bad;
    if (o == 0) ++cp0;
    else if (o == 1) ++cp1;
    if (w == 0) ++cn0;
    else if (w == 1) ++cn1;
    else if (w == 2 && o <= 1) ++ct2;
    if (w <= 1 && o > 1) ++bad;  // T2/T3 never return to full precision
  }
  int tp0, tp1, tn0, tn1, tt2;
  int bp0 = block_excl_scan(cp0, tmp, &tp0);
  int bp1 = block_excl_scan(cp1, tmp, &tp1);
  int bn0 = block_excl_scan(cn0, tmp, &tn0);
  int bn1 = block_excl_scan(cn1, tmp, &tn1);
  int bt2 = block_excl_scan(ct2, tmp, &tt2);
  bad = block_sum_i(bad, tmp);
  int* lens = a.new_lens + b * 3;
  if (bad || tp0 != a.len0[bl] || tp1 != a.len1[bl] || tn0 > a.cap0 || tn1 > a.cap1 ||
      tt2 > a.t2_cap) {
    if (tid < 3) lens[tid] = -1;
    return;
  }
  int* pos0 = a.t0_pos_dst + b * a.cap0;
  int* pos1 = a.t1_pos_dst + b * a.cap1;
  int* src0 = a.src0 + b * a.cap0;
  int* src1 = a.src1 + b * a.cap1;
  int* t2s = a.t2_src + b * a.t2_cap;
  int* t2p = a.t2_pos + b * a.t2_cap;
  for (int p = lo; p < hi; ++p) {
    const int o = tp[p], w = tn[p];
    int loc = 0;
    if (o == 0) loc = bp0++;
    else if (o == 1) loc = -(bp1++) - 1;
    if (w == 0) {
      pos0[bn0] = p;
      src0[bn0++] = loc;
    } else if (w == 1) {
      pos1[bn1] = p;
      src1[bn1++] = loc;
    } else if (w == 2 && o <= 1) {
      t2s[bt2] = loc;
      t2p[bt2++] = p;
    }
  }
  if (tid == 0) {
    lens[0] = tn0;
    lens[1] = tn1;
    lens[2] = tt2;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void compact_copy_kernel(CopyArgs c) {
  constexpr int ROWS = 64;  // destination slots per workgroup (two 32-slot blocks)
  const int z = blockIdx.z;  // 0: T0 destination, 1: T1 destination
  const int lgs = c.L * c.hkv;
  const int bl = blockIdx.y / lgs;
  const long lg = blockIdx.y - (long)bl * lgs;
  const long b = c.b_offset + bl;
  const int len = c.new_lens[b * 3 + z];
  const int r0 = blockIdx.x * ROWS;
  if (len <= r0) return;
  const int cap_d = z ? c.cap1 : c.cap0;
  const int* src = z ? c.src1 + b * c.cap1 : c.src0 + b * c.cap0;
  const long blk0 = (b * lgs + lg) * c.cap0 * D;  // element offset of this (b, l, g) block
  const long blk1 = (b * lgs + lg) * c.cap1 * D;
  const long blkd = (b * lgs + lg) * (long)cap_d * D;
  // K: 8-element chunks; items ordered like the destination (block, tile, chunk, row)
  {
    const T* ks0 = (const T*)c.k0s + blk0;
    const T* ks1 = (const T*)c.k1s + blk1;
    T* kd = (T*)(z ? c.k1d : c.k0d) + blkd;
    constexpr int CH = D / 8;
    for (int i = threadIdx.x; i < ROWS * CH; i += 256) {
      const int row = i & 15;
      const int cc = (i >> 4) % CH;
      const int u = (i / (16 * CH)) & 1;
      const int bk = i / (32 * CH);
      const int r = r0 + bk * 32 + 8 * (row >> 2) + 4 * u + (row & 3);
      if (r >= len) continue;
      const int sidx = src[r];
      const long ss = sidx >= 0 ? sidx : -sidx - 1;
      const T* from = (sidx >= 0 ? ks0 : ks1) + k_off(ss, 8 * cc, D);
      T* to = kd + k_off(r, 8 * cc, D);
#pragma unroll
      for (int e = 0; e < 8; ++e) to[e] = from[e];
    }
  }
  // V: 8-slot panels of one dimension; items ordered like the destination
  {
    const T* vs0 = (const T*)c.v0s + blk0;
    const T* vs1 = (const T*)c.v1s + blk1;
    T* vd = (T*)(z ? c.v1d : c.v0d) + blkd;
    for (int i = threadIdx.x; i < (ROWS / 8) * D; i += 256) {
      const int d15 = i & 15;
      const int pnl = (i >> 4) & 3;
      const int dh = (i >> 6) % (D / 16);
      const int bk = i / (4 * D);
      const int d = dh * 16 + d15;
      const int rb = r0 + bk * 32 + pnl * 8;
      if (rb >= len) continue;
      T vals[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vals[e] = T(0);
        if (rb + e < len) {
          const int sidx = src[rb + e];
          const long ss = sidx >= 0 ? sidx : -sidx - 1;
          vals[e] = (sidx >= 0 ? vs0 : vs1)[v_off(ss, d, D)];
        }
      }
      T* to = vd + v_off(rb, d, D);
#pragma unroll
      for (int e = 0; e < 8; ++e) to[e] = vals[e];
    }
  }
}

void launch_compact(const CompactArgs& a, const CopyArgs& c, int kv_dtype, int head_dim, int nb,
                    int max_n, hipStream_t s) {
  {
    KernelTimer timer("compact_scan", s);
    hipLaunchKernelGGL(compact_scan_kernel, dim3(nb), dim3(kTierThreads), 0, s, a);
  }
  const int rows = max(1, min(max_n, max(c.cap0, c.cap1)));
  dim3 grid(ceil_div(rows, 64), nb * c.L * c.hkv, 2);
  KernelTimer timer("compact_copy", s);
  if (kv_dtype == TKV_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((compact_copy_kernel<uint16_t, 128>), grid, dim3(256), 0, s, c);
    else
      hipLaunchKernelGGL((compact_copy_kernel<uint16_t, 64>), grid, dim3(256), 0, s, c);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((compact_copy_kernel<float, 128>), grid, dim3(256), 0, s, c);
    else
      hipLaunchKernelGGL((compact_copy_kernel<float, 64>), grid, dim3(256), 0, s, c);
  }
}

// ---------------------------------------------------------------------------
// append
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const long lg = blockIdx.x;
  const int bl = blockIdx.y;
  const long b = a.b_offset + bl;
  const int lgs = a.L * a.hkv;
  const int slot = a.slot[bl];
  const int pos = a.pos[bl];
  const T* ks = (const T*)a.kn + (b * lgs + lg) * D;
  const T* vs = (const T*)a.vn + (b * lgs + lg) * D;
  T* kd = (T*)a.k0 + (b * lgs + lg) * a.cap0 * D;
  T* vd = (T*)a.v0 + (b * lgs + lg) * a.cap0 * D;
  for (int d = threadIdx.x; d < D; d += 64) {  // K-tiles / V-tiles storage order
    kd[k_off(slot, d, D)] = ks[d];
    vd[v_off(slot, d, D)] = vs[d];
  }
  if (lg == 0 && threadIdx.x == 0) {
    a.t0_pos[b * a.cap0 + slot] = pos;
    if (a.scores) a.scores[b * a.max_ctx + pos] = 0.f;
    if (a.tier) a.tier[b * a.max_ctx + pos] = 0;
  }
}

void launch_append(const AppendArgs& a, int kv_dtype, int head_dim, int nb, hipStream_t s) {
  KernelTimer timer("append", s);
  dim3 grid(a.L * a.hkv, nb);
  if (kv_dtype == TKV_BF16) {
    if (head_dim == 128) hipLaunchKernelGGL((append_kernel<uint16_t, 128>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((append_kernel<uint16_t, 64>), grid, dim3(64), 0, s, a);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((append_kernel<float, 128>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((append_kernel<float, 64>), grid, dim3(64), 0, s, a);
  }
}

}  // namespace tkv
