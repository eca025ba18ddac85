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
// compact_copy  -- moves the rows into the new pool/window, one 32-slot
//                  destination block per workgroup: 16-byte key chunks and
//                  8-slot value panels, written in destination order.
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

// hist[bin] += 1 for every active lane, one LDS atomic per distinct bin of the
// wave (scores of a tail cluster in few bins of the leading digits).
__device__ __forceinline__ void wave_hist_add(unsigned* hist, unsigned bin, bool active) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t todo = __ballot(active);
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const unsigned lb = (unsigned)__shfl((int)bin, leader, kWave);
    const uint64_t same = __ballot(active && bin == lb);
    if (lane == leader) atomicAdd(&hist[lb], (unsigned)__popcll(same));
    todo &= ~same;
    if (bin == lb) active = false;
  }
}

// Digit of the k-th smallest key: the first bin whose inclusive prefix count
// reaches kk.  sh[0] = bin, sh[1] = kk minus the count below that bin.
// Every thread of the block calls it (barriers); hist holds 256 counts.
__device__ __forceinline__ void pick_digit(const unsigned* hist, int kk, int* tmp, int* sh) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int v = tid < 256 ? (int)hist[tid] : 0;
  int incl = wave_incl_scan_i(v);
  if (wid < 256 / kWave && lane == kWave - 1) tmp[wid] = incl;
  if (tid == 0) {
    sh[0] = 255;
    sh[1] = kk;
  }
  __syncthreads();
  if (tid < 256) {
    for (int w = 0; w < wid; ++w) incl += tmp[w];
    const int excl = incl - v;
    if (excl < kk && kk <= incl) {
      sh[0] = tid;
      sh[1] = kk - excl;
    }
  }
  __syncthreads();
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
    // the trip count is the same for every lane of a wave (n is block-uniform and
    // the stride is the block size), so the ballots below see the whole wave
    for (int p0 = tid - (tid & (kWave - 1)); p0 < n; p0 += kTierThreads) {
      const int p = p0 + (tid & (kWave - 1));
      bool act = false;
      uint32_t key = 0u;
      if (p < n) {
        key = score_key(sc[p]);
        act = (key & himask) == prefix && cand(p, tp[p], key);
      }
      wave_hist_add(hist, (key >> shift) & 255u, act);
    }
    __syncthreads();
    pick_digit(hist, kk, tmp, sh);
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
  constexpr int kBatch = 16;  // positions whose loads are issued together
  int cnt = 0;
  for (int base = lo; base < hi; base += kBatch) {
    bool tie[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = base + i;
      tie[i] = false;
      if (p < hi) {
        const uint32_t key = score_key(sc[p]);
        tie[i] = key == prefix && cand(p, tp[p], key);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) cnt += tie[i] ? 1 : 0;
  }
  int total;
  const int excl = block_excl_scan(cnt, tmp, &total);
  if (excl < kk && kk <= excl + cnt) {
    int need = kk - excl;  // the need-th tie counted from the top of this segment
    for (int top = hi - 1; top >= lo && need > 0; top -= kBatch) {
      bool tie[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int p = top - i;
        tie[i] = false;
        if (p >= lo) {
          const uint32_t key = score_key(sc[p]);
          tie[i] = key == prefix && cand(p, tp[p], key);
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (need > 0 && tie[i] && --need == 0) sh[2] = top - i;
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

// Eight consecutive elements: one 16-byte vector for bf16, two for float32.
template <typename T>
struct Vec8 {
  uint4 w[sizeof(T) / 2];
};

template <typename T>
__device__ __forceinline__ Vec8<T> load8(const T* p) {
  Vec8<T> v;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) v.w[i] = reinterpret_cast<const uint4*>(p)[i];
  return v;
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const Vec8<T>& v) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) reinterpret_cast<uint4*>(p)[i] = v.w[i];
}

// One workgroup per destination 32-slot block of one (sequence, layer, KV head).
// Keys move as 8-element chunks (a chunk of a row is contiguous in a K-tile);
// values are gathered 8 slots at a time into one V-tile panel of one dimension.
// Items are numbered in destination order, so the stores of a wave are
// contiguous; slots at or past the new length are written as zero.
template <typename T, int D>
__global__ __launch_bounds__(256) void compact_copy_kernel(CopyArgs c) {
  constexpr int CH = D / 8;  // 8-element key chunks per row
  const int z = blockIdx.z;  // 0: T0 destination, 1: T1 destination
  const int lgs = c.L * c.hkv;
  const int bl = blockIdx.y / lgs;
  const long lg = blockIdx.y - (long)bl * lgs;
  const long b = c.b_offset + bl;
  const int len = c.new_lens[b * 3 + z];
  const int r0 = blockIdx.x * 32;
  if (len <= r0) return;
  const int cap_d = z ? c.cap1 : c.cap0;
  const int* src = (z ? c.src1 + b * c.cap1 : c.src0 + b * c.cap0) + r0;
  const int nrow = min(32, len - r0);
  const long blk0 = (b * lgs + lg) * c.cap0 * D;  // element offset of this (b, l, g) block
  const long blk1 = (b * lgs + lg) * c.cap1 * D;
  const long blkd = (b * lgs + lg) * (long)cap_d * D + (long)r0 * D;
  // keys: item i -> (tile u, chunk cc, tile row) in destination order
  {
    const T* ks0 = (const T*)c.k0s + blk0;
    const T* ks1 = (const T*)c.k1s + blk1;
    T* kd = (T*)(z ? c.k1d : c.k0d) + blkd;
    for (int i = threadIdx.x; i < 32 * CH; i += 256) {
      const int row = i & 15;
      const int cc = (i >> 4) % CH;
      const int u = i / (16 * CH);
      const int r = 8 * (row >> 2) + 4 * u + (row & 3);
      Vec8<T> v;
      if (r < nrow) {
        const int sidx = src[r];
        const long ss = sidx >= 0 ? sidx : -sidx - 1;
        v = load8((sidx >= 0 ? ks0 : ks1) + k_off(ss, 8 * cc, D));
      } else {
#pragma unroll
        for (int w = 0; w < (int)(sizeof(T) / 2); ++w) v.w[w] = make_uint4(0, 0, 0, 0);
      }
      store8(kd + k_off(r, 8 * cc, D), v);
    }
  }
  // values: item i -> (dimension group dh, panel, dimension) in destination order
  {
    const T* vs0 = (const T*)c.v0s + blk0;
    const T* vs1 = (const T*)c.v1s + blk1;
    T* vd = (T*)(z ? c.v1d : c.v0d) + blkd;
    for (int i = threadIdx.x; i < 4 * D; i += 256) {
      const int d15 = i & 15;
      const int pnl = (i >> 4) & 3;
      const int dh = i >> 6;
      const int d = dh * 16 + d15;
      T vals[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = pnl * 8 + e;
        vals[e] = T(0);
        if (r < nrow) {
          const int sidx = src[r];
          const long ss = sidx >= 0 ? sidx : -sidx - 1;
          vals[e] = (sidx >= 0 ? vs0 : vs1)[v_off(ss, d, D)];
        }
      }
      Vec8<T> packed;
      __builtin_memcpy(&packed, vals, sizeof(packed));
      store8(vd + v_off(pnl * 8, d, D), packed);
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
  dim3 grid(ceil_div(rows, 32), nb * c.L * c.hkv, 2);
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
