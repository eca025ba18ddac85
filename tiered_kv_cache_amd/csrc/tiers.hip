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
// reloc_scan    -- one workgroup per sequence: block scans over positions and
//                  slots list the holes of the pool and window, the rows that
//                  move into them, and the positions newly in T2.  The slot ->
//                  position maps are updated in place.
// reloc_move    -- copies the listed rows (one wave per row and layer x KV
//                  head); three launches: promoted T1 rows to staging, rows
//                  into the T1 window, rows into the T0 pool.
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

// hist[bin] += 1 for every active lane.  Lanes that share the bin of the first
// active lane add their count with one atomic (up to kHistPeel such rounds, while
// a round takes at least a quarter of the wave); the others add one each.  Keys
// of similar scores share their leading byte, and 64 same-address LDS atomics of
// one instruction would be serialised; after the leading digit the candidates
// spread over many bins and the plain atomics do not collide.
constexpr int kHistPeel = 3;

__device__ __forceinline__ void hist_add(unsigned* hist, unsigned bin, bool active) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int r = 0; r < kHistPeel; ++r) {
    const uint64_t act = __ballot(active);
    if (act == 0) return;
    const int leader = __ffsll((unsigned long long)act) - 1;
    const unsigned lb = (unsigned)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t same = __ballot(active && bin == lb);
    const int c = __popcll(same);
    if (lane == leader) atomicAdd(&hist[lb], (unsigned)c);
    active = active && bin != lb;
    if (c < kWave / 4) break;
  }
  if (active) atomicAdd(&hist[bin], 1u);
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

// Positions [0, n) of the block in strides of its size, kPassBatch per thread
// at a time: the score and tier loads of a batch are issued before any is used.
constexpr int kPassBatch = 8;

template <class F>
__device__ __forceinline__ void for_positions(int n, const float* sc, const uint8_t* tp, F f) {
  for (int p0 = threadIdx.x; p0 < n; p0 += kTierThreads * kPassBatch) {
    uint32_t key[kPassBatch];
    int t[kPassBatch];
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i) {
      const int p = p0 + i * kTierThreads;
      key[i] = 0u;
      t[i] = 0;
      if (p < n) {
        key[i] = score_key(sc[p]);
        t[i] = tp[p];
      }
    }
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i) {
      const int p = p0 + i * kTierThreads;
      if (p < n) f(p, t[i], key[i]);
    }
  }
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
    for_positions(n, sc, tp, [&](int p, int t, uint32_t key) {
      hist_add(hist, (key >> shift) & 255u, (key & himask) == prefix && cand(p, t, key));
    });
    __syncthreads();
    pick_digit(hist, kk, tmp, sh);
    prefix |= (uint32_t)sh[0] << shift;
    kk = sh[1];
    __syncthreads();
  }
  // kk candidates with key == prefix remain to be taken: the highest positions.
  // The last histogram still holds how many candidates have key == prefix; when
  // all of them are taken (the usual case for distinct scores) no scan is needed.
  const int ties = (int)hist[prefix & 255u];
  __syncthreads();
  if (kk == ties) {
    r.T = prefix;
    r.cut = 0;
    return r;
  }
  // Otherwise thread t owns positions [n - (t+1)*seg, n - t*seg): a forward scan
  // over threads counts ties above each segment.
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
  for_positions(n, sc, tp, [&](int p, int t, uint32_t) {
    cBad += t > 3;
    cE += t == 3;
    cT2 += t == 2;
    cPool += t <= 2 && !prot(p);
  });
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
  for_positions(n, sc, tp, [&](int p, int t, uint32_t key) {
    const bool pool = t <= 2 && !prot(p);
    const bool ev = in_sel(s1, key, p);
    cEvT2 += pool && t == 2 && ev;
    cLive += pool && t <= 1 && !ev;
  });
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

  int c0 = 0, c1 = 0, c2 = 0, c3 = 0;
  for_positions(n, sc, tp, [&](int p, int t, uint32_t key) {
    const bool np = !prot(p);
    int nt;
    if (t == 3) nt = 3;
    else if (np && in_sel(s1, key, p)) nt = 3;
    else if (t == 2) nt = 2;
    else if (np && in_sel(s2, key, p)) nt = 2;
    else if (np && in_sel(s3, key, p)) nt = 1;
    else nt = 0;
    tn[p] = (uint8_t)nt;
    c0 += nt == 0;
    c1 += nt == 1;
    c2 += nt == 2;
    c3 += nt == 3;
  });
  c0 = block_sum_i(c0, tmp);
  c1 = block_sum_i(c1, tmp);
  c2 = block_sum_i(c2, tmp);
  c3 = block_sum_i(c3, tmp);
  if (tid == 0) {
    counts[0] = c0;
    counts[1] = c1;
    counts[2] = c2;
    counts[3] = c3;
  }
}

// ---------------------------------------------------------------------------
// the same selection with every key in registers (n <= 1024 * PPT)
// ---------------------------------------------------------------------------
// The positions are cut into chunks of PPT from position 0 and thread t owns chunk
// ceil(n / PPT) - 1 - t (positions >= n absent): thread 0 holds the highest
// positions, so a block scan over threads counts what lies above a thread's chunk.  The scores and previous tiers
// are read once; the keys stay in registers and every per-position condition is a
// bit mask over the owned positions (bit i: position base + i), so the radix passes
// touch no memory but the LDS histogram.
template <int PPT>
struct Owned {
  uint32_t key[PPT];
  int base;  // position of key[0]
};

// Bit i set for the owned positions that are candidates (mask), have key == T and
// lie at or above cut: the ties a selection (T, cut) takes.
template <int PPT>
__device__ __forceinline__ uint64_t sel_mask(const Owned<PPT>& o, uint64_t cand, const Sel& s) {
  uint64_t m = 0;
#pragma unroll
  for (int i = 0; i < PPT; ++i)
    m |= (uint64_t)((cand >> i & 1) && in_sel(s, o.key[i], o.base + i)) << i;
  return m;
}

// k (block-uniform) least important positions among the owned candidates (bits of
// cand).  The same digits, counts and tie rule as radix_select.
template <int PPT>
__device__ __forceinline__ Sel radix_select_owned(int k, const Owned<PPT>& o, uint64_t cand,
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
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      hist_add(hist, (o.key[i] >> shift) & 255u, (cand >> i & 1) && (o.key[i] & himask) == prefix);
    __syncthreads();
    pick_digit(hist, kk, tmp, sh);
    prefix |= (uint32_t)sh[0] << shift;
    kk = sh[1];
    __syncthreads();
  }
  const int ties = (int)hist[prefix & 255u];
  __syncthreads();
  if (kk == ties) {  // every candidate with key == prefix is taken
    r.T = prefix;
    r.cut = 0;
    return r;
  }
  // kk of the ties are taken: the highest positions
  uint64_t tie = 0;
#pragma unroll
  for (int i = 0; i < PPT; ++i) tie |= (uint64_t)((cand >> i & 1) && o.key[i] == prefix) << i;
  const int cnt = __popcll(tie);
  int total;
  const int excl = block_excl_scan(cnt, tmp, &total);
  if (excl < kk && kk <= excl + cnt) {
    // the (kk - excl)-th tie counted from the top of this chunk
    for (int need = kk - excl; need > 1; --need) tie &= ~(1ull << (63 - __clzll(tie)));
    sh[2] = o.base + 63 - __clzll(tie);
  }
  __syncthreads();
  r.T = prefix;
  r.cut = sh[2];
  __syncthreads();
  return r;
}

template <int PPT>
__global__ __launch_bounds__(kTierThreads) void assign_tiers_reg_kernel(TierArgs a) {
  static_assert(PPT <= 64 && PPT % 16 == 0, "one bit per owned position in a 64-bit mask");
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

  Owned<PPT> o;
  const int chunks = (n + PPT - 1) / PPT;
  o.base = (chunks - 1 - tid) * PPT;  // chunk-aligned: thread 0 owns the top chunk
  uint32_t tw[PPT / 4];               // previous tiers, four per word
  const bool aligned = (((uintptr_t)(sc + o.base) | (uintptr_t)(tp + o.base)) & 15) == 0;
  if (o.base >= 0 && o.base + PPT <= n && aligned) {  // whole chunk: vector loads
    const uint4* s4 = reinterpret_cast<const uint4*>(sc + o.base);
    const uint4* t4 = reinterpret_cast<const uint4*>(tp + o.base);
#pragma unroll
    for (int i = 0; i < PPT / 4; ++i) {
      const uint4 v = s4[i];
      o.key[4 * i] = v.x;
      o.key[4 * i + 1] = v.y;
      o.key[4 * i + 2] = v.z;
      o.key[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < PPT / 16; ++i) {
      const uint4 v = t4[i];
      tw[4 * i] = v.x;
      tw[4 * i + 1] = v.y;
      tw[4 * i + 2] = v.z;
      tw[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PPT / 4; ++i) tw[i] = 0u;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = o.base + i;
      const bool in = p >= 0 && p < n;
      o.key[i] = in ? __float_as_uint(sc[p]) : 0u;
      tw[i / 4] |= (in ? (uint32_t)tp[p] : 0u) << (8 * (i % 4));
    }
  }
  // masks over the owned positions
  uint64_t valid = 0, m3 = 0, m2 = 0, m01 = 0, bad = 0, np = 0;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int p = o.base + i;
    const uint32_t t = (tw[i / 4] >> (8 * (i % 4))) & 0xFFu;
    o.key[i] = score_key(__uint_as_float(o.key[i]));
    const uint64_t bit = 1ull << i;
    if (p >= 0 && p < n) {
      valid |= bit;
      if (t > 3) bad |= bit;
      if (t == 3) m3 |= bit;
      if (t == 2) m2 |= bit;
      if (t <= 1) m01 |= bit;
      if (p >= prot_lo && p < prot_hi) np |= bit;
    }
  }
  const int cBad = block_sum_i(__popcll(bad), tmp);
  if (cBad) {
    if (tid < 4) counts[tid] = -1;
    return;
  }
  const uint64_t pool = np & (m2 | m01);  // non-protected T0/T1/T2
  const int cE = block_sum_i(__popcll(m3), tmp);
  const int cT2 = block_sum_i(__popcll(m2), tmp);
  const int cPool = block_sum_i(__popcll(pool), tmp);

  // 1. eviction from the pool
  const int e = min(max(a.n3[bl] - cE, 0), cPool);
  const Sel s1 = radix_select_owned(e, o, pool, hist, tmp, sh);
  const uint64_t ev = sel_mask(o, pool, s1);
  const uint64_t live = pool & m01 & ~ev;  // non-protected T0/T1 not just evicted
  const int cEvT2 = block_sum_i(__popcll(ev & m2), tmp);
  const int cLive = block_sum_i(__popcll(live), tmp);

  // 2. T2 from live
  const int survivors = cT2 - cEvT2;
  const int q = min(max(a.n2[bl] - survivors, 0), cLive);
  const Sel s2 = radix_select_owned(q, o, live, hist, tmp, sh);
  const uint64_t to2 = sel_mask(o, live, s2);

  // 3. T1 from what is left of live
  const int r1 = min(a.n1[bl], cLive - q);
  const Sel s3 = radix_select_owned(r1, o, live & ~to2, hist, tmp, sh);
  const uint64_t to1 = sel_mask(o, live & ~to2, s3);

  const uint64_t n3 = (m3 | ev) & valid;
  const uint64_t n2 = (m2 & ~ev) | to2;
  const uint64_t n1 = to1;
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    if (valid >> i & 1)
      tn[o.base + i] = (uint8_t)((n3 >> i & 1) ? 3 : (n2 >> i & 1) ? 2 : (n1 >> i & 1) ? 1 : 0);
  }
  const int c3 = block_sum_i(__popcll(n3), tmp);
  const int c2 = block_sum_i(__popcll(n2), tmp);
  const int c1 = block_sum_i(__popcll(n1), tmp);
  const int c0 = block_sum_i(__popcll(valid), tmp) - c1 - c2 - c3;
  if (tid == 0) {
    counts[0] = c0;
    counts[1] = c1;
    counts[2] = c2;
    counts[3] = c3;
  }
}

// Keys in registers when the longest sequence of the launch fits; the kernel that
// streams them from memory on every pass otherwise.
void launch_assign_tiers(const TierArgs& a, int nb, hipStream_t s) {
  KernelTimer timer("assign_tiers", s);
  int nmax = 0;
  for (int i = 0; i < nb; ++i) nmax = max(nmax, a.n[i]);
  const dim3 grid(nb), block(kTierThreads);
  if (nmax <= kTierThreads * 16)
    hipExtLaunchKernelGGL(assign_tiers_reg_kernel<16>, grid, block, 0, s, timer.start(), timer.stop(), 0, a);
  else if (nmax <= kTierThreads * 32)
    hipExtLaunchKernelGGL(assign_tiers_reg_kernel<32>, grid, block, 0, s, timer.start(), timer.stop(), 0, a);
  else if (nmax <= kTierThreads * 48)
    hipExtLaunchKernelGGL(assign_tiers_reg_kernel<48>, grid, block, 0, s, timer.start(), timer.stop(), 0, a);
  else if (nmax <= kTierThreads * 64)
    hipExtLaunchKernelGGL(assign_tiers_reg_kernel<64>, grid, block, 0, s, timer.start(), timer.stop(), 0, a);
  else
    hipExtLaunchKernelGGL(assign_tiers_kernel, grid, block, 0, s, timer.start(), timer.stop(), 0, a);
}

// ---------------------------------------------------------------------------
// relocation (in place)
// ---------------------------------------------------------------------------
constexpr int kNoSlot = INT_MIN;

// Helpers of the relocation scan: kPassBatch entries per thread at a time, the
// loads of a batch issued before any is used, f called in index order.

// Slot -> position map entries [0, len), strided by the block: f(slot, position).
template <class F>
__device__ __forceinline__ void for_map(int len, const int* pos, F f) {
  for (int s0 = threadIdx.x; s0 < len; s0 += kTierThreads * kPassBatch) {
    int p[kPassBatch];
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i) {
      const int s = s0 + i * kTierThreads;
      p[i] = s < len ? pos[s] : 0;
    }
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i)
      if (s0 + i * kTierThreads < len) f(s0 + i * kTierThreads, p[i]);
  }
}

// Positions [lo, hi): f(position, previous tier, new tier, slot code).
template <class F>
__device__ __forceinline__ void for_segment(int lo, int hi, const uint8_t* tp, const uint8_t* tn,
                                            const int* inv, F f) {
  for (int base = lo; base < hi; base += kPassBatch) {
    int o[kPassBatch], w[kPassBatch], v[kPassBatch];
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i) {
      const int p = base + i;
      o[i] = 0;
      w[i] = 0;
      v[i] = kNoSlot;
      if (p < hi) {
        o[i] = tp[p];
        w[i] = tn[p];
        v[i] = inv[p];
      }
    }
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i)
      if (base + i < hi) f(base + i, o[i], w[i], v[i]);
  }
}

// Slots [s0, s1) of a pool with `len` rows: f(slot, hole).  A hole is a slot at
// or past the old length, or one whose row leaves `tier`.  Positions of slots
// below len are known to lie in [0, n).
template <class F>
__device__ __forceinline__ void for_slots(int s0, int s1, int len, const int* pos,
                                          const uint8_t* tn, int tier, F f) {
  for (int base = s0; base < s1; base += kPassBatch) {
    int p[kPassBatch];
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i) {
      const int s = base + i;
      p[i] = (s < s1 && s < len) ? pos[s] : -1;
    }
    int t[kPassBatch];
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i) t[i] = p[i] >= 0 ? (int)tn[p[i]] : -1;
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i)
      if (base + i < s1) f(base + i, t[i] != tier);
  }
}

// One workgroup per sequence.  Only the rows whose tier changed, and the rows
// left above the new length of their pool, move: each fills a "hole", a slot
// below the new length whose row left (or which was past the old length).
// The i-th mover in position order takes the i-th hole in slot order.
__global__ __launch_bounds__(kTierThreads) void reloc_scan_kernel(RelocArgs a) {
  __shared__ int tmp[kTierThreads / kWave + 1];
  const int tid = threadIdx.x;
  const int bl = blockIdx.x;
  const long b = a.b_offset + bl;
  const int n = a.n[bl], len0 = a.len0[bl], len1 = a.len1[bl];
  const uint8_t* tp = a.tprev + b * a.max_ctx;
  const uint8_t* tn = a.tnext + b * a.max_ctx;
  int* pos0 = a.t0_pos + b * a.cap0;
  int* pos1 = a.t1_pos + b * a.cap1;
  int* inv = a.inv + b * a.max_ctx;
  int* cnt = a.cnt + b * 4;
  int* lens = a.new_lens + b * 4;

  // inverse map of the current pool and window
  for (int p = tid; p < n; p += kTierThreads) inv[p] = kNoSlot;
  __syncthreads();
  int bad = 0;
  for_map(len0, pos0, [&](int s, int p) {
    if (p < 0 || p >= n) ++bad;
    else inv[p] = s;
  });
  for_map(len1, pos1, [&](int s, int p) {
    if (p < 0 || p >= n) ++bad;
    else inv[p] = -s - 1;
  });
  __syncthreads();

  // new sizes, and a consistency check of the maps against the previous tiers:
  // with len0 T0 slots and len0 T0 positions, every T0 position holding a T0
  // slot makes the map a bijection (likewise for T1)
  const int seg = (n + kTierThreads - 1) / kTierThreads;
  const int lo = min(n, tid * seg);
  const int hi = min(n, lo + seg);
  int cp0 = 0, cp1 = 0, cn0 = 0, cn1 = 0, ct2 = 0, ct2h = 0;
  for_segment(lo, hi, tp, tn, inv, [&](int, int o, int w, int v) {
    bad += o > 3 || w > 3 || (w <= 1 && o > 1);  // T2/T3 never return to full precision
    bad += o == 0 && v < 0;
    bad += o == 1 && (v >= 0 || v == kNoSlot);
    bad += o > 1 && v != kNoSlot;
    cp0 += o == 0;
    cp1 += o == 1;
    cn0 += w == 0;
    cn1 += w == 1;
    ct2 += w == 2 && o <= 1;
    ct2h += w == 2 && o == 1;  // new T2 rows that leave T1
  });
  bad = block_sum_i(bad, tmp);
  cp0 = block_sum_i(cp0, tmp);
  cp1 = block_sum_i(cp1, tmp);
  const int n0 = block_sum_i(cn0, tmp);
  const int n1 = block_sum_i(cn1, tmp);
  const int nt2 = block_sum_i(ct2, tmp);
  if (bad || cp0 != len0 || cp1 != len1 || n0 > a.lim0[bl] || n1 > a.lim1[bl] || nt2 > a.t2_cap) {
    if (tid < 4) lens[tid] = -1;
    if (tid < 4) cnt[tid] = 0;
    return;
  }

  // holes, in slot order
  int* holes0 = a.holes0 + b * a.cap0;
  int* holes1 = a.holes1 + b * a.cap1;
  int h0, h1;
  {
    const int sg = (n0 + kTierThreads - 1) / kTierThreads;
    const int s0 = min(n0, tid * sg), s1 = min(n0, s0 + sg);
    int c = 0;
    for_slots(s0, s1, len0, pos0, tn, 0, [&](int, bool hole) { c += hole; });
    int k = block_excl_scan(c, tmp, &h0);
    for_slots(s0, s1, len0, pos0, tn, 0, [&](int s, bool hole) {
      if (hole) holes0[k++] = s;
    });
  }
  {
    const int sg = (n1 + kTierThreads - 1) / kTierThreads;
    const int s0 = min(n1, tid * sg), s1 = min(n1, s0 + sg);
    int c = 0;
    for_slots(s0, s1, len1, pos1, tn, 1, [&](int, bool hole) { c += hole; });
    int k = block_excl_scan(c, tmp, &h1);
    for_slots(s0, s1, len1, pos1, tn, 1, [&](int s, bool hole) {
      if (hole) holes1[k++] = s;
    });
  }

  // movers, in position order
  int m0 = 0, m1 = 0, mp = 0;
  for_segment(lo, hi, tp, tn, inv, [&](int, int o, int w, int v) {
    m0 += w == 0 && (o == 1 || (o == 0 && v >= n0));
    m1 += w == 1 && (o == 0 || (o == 1 && -v - 1 >= n1));
    mp += w == 0 && o == 1;
  });
  int M0, M1, MP, T2, T2H;
  int i0 = block_excl_scan(m0, tmp, &M0);
  int i1 = block_excl_scan(m1, tmp, &M1);
  int ip = block_excl_scan(mp, tmp, &MP);
  int it2 = block_excl_scan(ct2, tmp, &T2);
  int ih = block_excl_scan(ct2h, tmp, &T2H);
  if (M0 != h0 || M1 != h1) {  // cannot happen once the checks above hold
    if (tid < 4) lens[tid] = -1;
    if (tid < 4) cnt[tid] = 0;
    return;
  }
  __syncthreads();  // every read of the old slot -> position maps is done
  int2* to0 = a.to_t0 + b * a.cap0;
  int2* to1 = a.to_t1 + b * a.cap1;
  int2* stg = a.staged + b * a.cap1;
  int* t2s = a.t2_src + b * a.t2_cap;
  int* t2p = a.t2_pos + b * a.t2_cap;
  for_segment(lo, hi, tp, tn, inv, [&](int p, int o, int w, int v) {
    if (w == 0 && o == 1) {
      const int j = ip++;
      stg[j] = make_int2(v, j);
      const int d = holes0[i0];
      to0[i0++] = make_int2(-j - 1, d);
      pos0[d] = p;
    } else if (w == 0 && o == 0 && v >= n0) {
      const int d = holes0[i0];
      to0[i0++] = make_int2(v, d);
      pos0[d] = p;
    } else if (w == 1 && (o == 0 || -v - 1 >= n1)) {
      const int d = holes1[i1];
      to1[i1++] = make_int2(v, d);
      pos1[d] = p;
    } else if (w == 2 && o <= 1) {
      // host-resident T1: the row reaches the device in staging row MP + (its rank
      // among the new T2 rows that leave T1), after the promoted rows
      t2s[it2] = (a.host_t1 && o == 1) ? -(MP + ih++) - 1 : v;
      t2p[it2++] = p;
    }
  });
  if (tid == 0) {
    lens[0] = n0;
    lens[1] = n1;
    lens[2] = nt2;
    lens[3] = M0 + M1 + MP;
    cnt[kMoveToT0] = M0;
    cnt[kMoveToT1] = M1;
    cnt[kMoveStage] = MP;
    cnt[3] = 0;
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

// One row of one (layer, KV head): a slot of a pool (K-tile / V-tile order) or
// a plain staging row (D keys then D values).
template <typename T>
struct RowRef {
  T* k;
  T* v;
  long slot;  // < 0: plain row
};

// Source and destination rows of one move of one (layer, KV head).
template <typename T, int D>
__device__ __forceinline__ void move_rows(const MoveArgs& m, long b, int lg, int2 mv, long idx,
                                          RowRef<T>& src, RowRef<T>& dst) {
  const int bl = (int)(b - m.b_offset);
  const long o0 = pool_row(m.pool.blk0, m.pool.cap0, bl, lg, D);
  const long o1 = pool_row(m.pool.blk1, m.pool.cap1, bl, lg, D);
  T* p0k = (T*)m.k0 + o0;
  T* p0v = (T*)m.v0 + o0;
  T* p1k = (T*)m.k1 + o1;
  T* p1v = (T*)m.v1 + o1;
  if (m.which == kMoveStage) {  // T1 slot -> staging row
    src = {p1k, p1v, (long)(-mv.x - 1)};
    T* r = (T*)m.staging + ((b * m.cap1 + mv.y) * m.lgs + lg) * 2 * D;
    dst = {r, r + D, -1};
  } else if (m.which == kMoveDown) {  // T0 slot -> staging row (the entry's list index)
    src = {p0k, p0v, (long)mv.x};
    T* r = (T*)m.staging + ((b * m.cap1 + idx) * m.lgs + lg) * 2 * D;
    dst = {r, r + D, -1};
  } else if (m.which == kMoveToT1) {  // T0 or T1 slot -> T1 slot
    src = mv.x >= 0 ? RowRef<T>{p0k, p0v, (long)mv.x} : RowRef<T>{p1k, p1v, (long)(-mv.x - 1)};
    dst = {p1k, p1v, (long)mv.y};
  } else {  // T0 slot or staging row -> T0 slot
    if (mv.x >= 0) {
      src = {p0k, p0v, (long)mv.x};
    } else {
      T* r = (T*)m.staging + ((b * m.cap1 + (-mv.x - 1)) * m.lgs + lg) * 2 * D;
      src = {r, r + D, -1};
    }
    dst = {p0k, p0v, (long)mv.y};
  }
}

// One wave per (move, layer x KV head) item, kMoveBatch items of a wave in
// flight together (list entries first, then every row load, then the stores);
// consecutive waves take consecutive moves of one (layer, KV head), whose
// destinations are in slot order.
constexpr int kMoveBatch = 4;

template <typename T, int D>
__global__ __launch_bounds__(256) void reloc_move_kernel(MoveArgs m) {
  constexpr int VE = D / kWave;  // value elements per lane
  const int lane = threadIdx.x & (kWave - 1);
  const long gw = (long)blockIdx.x * (256 / kWave) + (threadIdx.x / kWave);
  const long nw = (long)gridDim.x * (256 / kWave);
  for (int bl = 0; bl < m.nb; ++bl) {
    const long b = m.b_offset + bl;
    // the down list is the T1-destination list; it moves only the entries whose
    // source is a T0 slot
    const bool down = m.which == kMoveDown;
    const int cnt = m.cnt[b * 4 + (down ? kMoveToT1 : m.which)];
    const long items = (long)cnt * m.lgs;
    const int2* list = m.list + b * m.list_stride;
    for (long it0 = gw; it0 < items; it0 += nw * kMoveBatch) {
      int2 mv[kMoveBatch];
      int lg[kMoveBatch];
      long li[kMoveBatch];
      bool on[kMoveBatch];
#pragma unroll
      for (int k = 0; k < kMoveBatch; ++k) {
        const long it = it0 + k * nw;
        lg[k] = 0;
        li[k] = 0;
        mv[k] = make_int2(0, 0);
        if (it < items) {
          lg[k] = (int)(it / cnt);
          li[k] = it - (long)lg[k] * cnt;
          mv[k] = list[li[k]];
        }
        on[k] = it < items && !(down && mv[k].x < 0);
      }
      RowRef<T> src[kMoveBatch], dst[kMoveBatch];
      Vec8<T> kv[kMoveBatch];
      T x[kMoveBatch][VE];
#pragma unroll
      for (int k = 0; k < kMoveBatch; ++k) {
        if (!on[k]) continue;
        move_rows<T, D>(m, b, lg[k], mv[k], li[k], src[k], dst[k]);
        if (lane < D / 8) {
          const int d = 8 * lane;
          kv[k] = load8(src[k].slot >= 0 ? src[k].k + k_off(src[k].slot, d, D) : src[k].k + d);
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const int d = lane + e * kWave;
          x[k][e] = src[k].slot >= 0 ? src[k].v[v_off(src[k].slot, d, D)] : src[k].v[d];
        }
      }
#pragma unroll
      for (int k = 0; k < kMoveBatch; ++k) {
        if (!on[k]) continue;
        if (lane < D / 8) {
          const int d = 8 * lane;
          store8(dst[k].slot >= 0 ? dst[k].k + k_off(dst[k].slot, d, D) : dst[k].k + d, kv[k]);
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const int d = lane + e * kWave;
          if (dst[k].slot >= 0) dst[k].v[v_off(dst[k].slot, d, D)] = x[k][e];
          else dst[k].v[d] = x[k][e];
        }
      }
    }
  }
}

void launch_reloc_scan(const RelocArgs& a, int nb, hipStream_t s) {
  KernelTimer timer("reloc_scan", s);
  hipExtLaunchKernelGGL(reloc_scan_kernel, dim3(nb), dim3(kTierThreads), 0, s,
                        timer.start(), timer.stop(), 0, a);
}

void launch_reloc_move(const MoveArgs& m, int kv_dtype, int head_dim, hipStream_t s) {
  static const char* names[4] = {"reloc_stage", "reloc_to_t1", "reloc_to_t0", "reloc_down"};
  KernelTimer timer(names[m.which], s);
  const dim3 grid(2048);
  if (kv_dtype == TKV_BF16) {
    if (head_dim == 128) hipExtLaunchKernelGGL((reloc_move_kernel<uint16_t, 128>), grid, dim3(256), 0, s,
                                               timer.start(), timer.stop(), 0, m);
    else hipExtLaunchKernelGGL((reloc_move_kernel<uint16_t, 64>), grid, dim3(256), 0, s,
                               timer.start(), timer.stop(), 0, m);
  } else {
    if (head_dim == 128) hipExtLaunchKernelGGL((reloc_move_kernel<float, 128>), grid, dim3(256), 0, s,
                                               timer.start(), timer.stop(), 0, m);
    else hipExtLaunchKernelGGL((reloc_move_kernel<float, 64>), grid, dim3(256), 0, s,
                               timer.start(), timer.stop(), 0, m);
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
  const long o0 = pool_row(a.pool.blk0, a.pool.cap0, (int)(b - a.b_offset), lg, D);
  T* kd = (T*)a.k0 + o0;
  T* vd = (T*)a.v0 + o0;
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
    if (head_dim == 128) hipExtLaunchKernelGGL((append_kernel<uint16_t, 128>), grid, dim3(64), 0, s,
                                               timer.start(), timer.stop(), 0, a);
    else hipExtLaunchKernelGGL((append_kernel<uint16_t, 64>), grid, dim3(64), 0, s,
                               timer.start(), timer.stop(), 0, a);
  } else {
    if (head_dim == 128) hipExtLaunchKernelGGL((append_kernel<float, 128>), grid, dim3(64), 0, s,
                                               timer.start(), timer.stop(), 0, a);
    else hipExtLaunchKernelGGL((append_kernel<float, 64>), grid, dim3(64), 0, s,
                               timer.start(), timer.stop(), 0, a);
  }
}

}  // namespace tkv
