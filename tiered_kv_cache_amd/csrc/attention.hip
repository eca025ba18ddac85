// Decode attention over T0 u T1 (with the append of the step's new token), and
// its two variants: the 8-bit T2 rows attended after T1, and a T1 window that
// holds only the call's layers (streamed from host memory chunk by chunk).
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490).  Methodologie section 1: T1 rows reach the GPU before the
// attention step; section 3: they then enter the softmax exactly like resident
// rows, so attention runs over the T0 pool and the T1 window as one attended
// set.  Section 2: the score of a position grows by its attention weight
// averaged over heads and layers.
//
// Work decomposition (stream-K): each (sequence, layer, KV head) "group" has a
// T0 segment, a T1 segment and, when the caller attends T2, a T2 segment of
// 8-bit rows (Methodologie section 1 keeps T2 at reduced precision: each row is
// attended as code x scale of its stored int8 codes and float32 scale), cut
// into work units of U tokens (U = 32 on the
// matrix-core path, 256 on the float32 path); units are numbered group after
// group.  Worker w of W owns units [w*P/W, (w+1)*P/W) -- an equal share, so the
// launch has no tail -- runs one online softmax per group it touches and writes
// one split record per group, at record index w + group (unique, and at most
// W + groups records).
//
// Kernels:
//   attn_partial_mfma<D, T2, GEO> -- bf16 path; T2: the launch has T2 units and
//       walks its work as runs of one unit format; GEO: the window geometry.
//       A worker is one wave, one wave per SIMD
//       (the grid is resident at once).  Per 32-token unit:
//       S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (the group's query heads padded
//       to 16 columns), an online softmax with lazy rescaling, and O += P V on
//       the same MFMA with P split into a bf16 high part and a bf16 remainder
//       (P V is then exact to ~2^-17 relative).  The token order inside a unit
//       is permuted so that the S^T accumulator is already the A operand of
//       P V, and keys and values are stored in the operand order (K-tiles,
//       V-tiles: layout.h), so every operand load is one contiguous 1 KB wave
//       access, marked non-temporal (read once).  The next unit's keys and
//       values are requested as soon as this unit has consumed its own.  The
//       logits of a wave's units are staged in LDS and written in bursts once
//       its key/value stream is done (stores interleaved with the stream slow
//       its reads down; a stage that fills before then is written with
//       non-temporal stores).  The logits are kept in base 2 (q.k * softmax_scale *
//       log2 e), so every weight is one v_exp_f32; they go to `alpha` and are
//       normalised there by the merge kernels.  With a new token, the wave
//       whose range holds the T0 unit of its slot also writes its key and
//       value rows there (and its position, score 0, tier T0).
//   attn_partial_valu -- float32 path (plain FMAs); a worker is a workgroup.
// The records are merged, and the logits normalised into alpha, by the merge
// kernels (merge.hip).
#include "attn_args.h"
#include "common.h"
#include "layout.h"

namespace tkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// ---------------------------------------------------------------------------
// work units
// ---------------------------------------------------------------------------
struct Unit {
  long b;      // sequence in the caller's batch
  long group;  // group index within the launch
  int lr, g;   // layer (relative) and KV head
  int seg;     // 0: T0 pool, 1: T1 window, 2: T2 pool (int8)
  int c0, c1;  // slot range inside the segment
  int off;     // attended index of the segment's slot 0
};

__device__ __forceinline__ Unit decode_unit(const AttnArgs& a, long p) {
  int bl = 0;
  while (bl + 1 < a.seq.nb && a.seq.base[bl + 1] <= p) ++bl;
  Unit u;
  u.b = a.seq.b_offset + bl;
  const int n0 = a.seq.t0_len[bl], n1 = a.seq.t1_len[bl], n2 = a.seq.t2_len[bl];
  const long local = p - a.seq.base[bl];
  const int per = a.seq.units[bl];
  const int lgl = (int)(local / per);
  const int q = (int)(local - (long)lgl * per);
  u.lr = lgl / a.hkv;
  u.g = lgl - u.lr * a.hkv;
  u.group = (long)bl * a.Lr * a.hkv + lgl;
  const int nu0 = (n0 + a.unit - 1) / a.unit;
  const int nu1 = (n1 + a.unit - 1) / a.unit;
  if (q < nu0) {
    u.seg = 0;
    u.c0 = q * a.unit;
    u.c1 = min(n0, u.c0 + a.unit);
    u.off = 0;
  } else if (q < nu0 + nu1) {
    u.seg = 1;
    u.c0 = (q - nu0) * a.unit;
    u.c1 = min(n1, u.c0 + a.unit);
    u.off = n0;
  } else {
    u.seg = 2;
    u.c0 = (q - nu0 - nu1) * a.unit;
    u.c1 = min(n2, u.c0 + a.unit);
    u.off = n0 + n1;
  }
  return u;
}

// ---------------------------------------------------------------------------
// bf16 path: MFMA partial attention, one worker per wave
// ---------------------------------------------------------------------------
// Walks the units of a worker's range in order.  Everything here is uniform
// across the wave (scalar registers); only the first position needs a division.
struct Cursor {
  int bl;      // sequence within the launch
  int lgl;     // group within the sequence: layer * Hkv + KV head
  int lr, g;
  int seg;     // 0: T0 pool, 1: T1 window, 2: T2 pool (int8)
  int c0;      // first slot of the unit inside the segment
  int n0, n1, n2;
};

// Segment geometry of a unit whose format is known at compile time: Q8 units are
// T2 units, the others T0 (seg 0) or T1 (seg 1) units.  Every loop over units
// runs over units of one format, so no three-way segment select sits in the
// loop (one there measurably slowed the key/value stream on chain-8K sizes).
template <bool Q8>
__device__ __forceinline__ int seg_len(const Cursor& c) {
  if constexpr (Q8) return c.n2;
  else return c.seg ? c.n1 : c.n0;
}

// attended index of the unit's segment slot 0: T0, then T1, then T2
template <bool Q8>
__device__ __forceinline__ int seg_off(const Cursor& c) {
  if constexpr (Q8) return c.n0 + c.n1;
  else return c.seg ? c.n0 : 0;
}

// T2: the launch has T2 units (three segments per group)
template <bool T2>
__device__ __forceinline__ Cursor cursor_at(const AttnArgs& a, long p) {
  Cursor c;
  int bl = 0;
  while (bl + 1 < a.seq.nb && a.seq.base[bl + 1] <= p) ++bl;
  c.bl = bl;
  c.n0 = a.seq.t0_len[bl];
  c.n1 = a.seq.t1_len[bl];
  c.n2 = T2 ? a.seq.t2_len[bl] : 0;
  const long local = p - a.seq.base[bl];
  const int per = a.seq.units[bl];
  c.lgl = (int)(local / per);
  const int q = (int)(local - (long)c.lgl * per);
  c.lr = c.lgl / a.hkv;
  c.g = c.lgl - c.lr * a.hkv;
  const int nu0 = (c.n0 + kUnitMfma - 1) / kUnitMfma;
  if constexpr (T2) {
    const int nu1 = (c.n1 + kUnitMfma - 1) / kUnitMfma;
    c.seg = q < nu0 ? 0 : (q < nu0 + nu1 ? 1 : 2);
    c.c0 = (q < nu0 ? q : (q < nu0 + nu1 ? q - nu0 : q - nu0 - nu1)) * kUnitMfma;
  } else {
    c.seg = q < nu0 ? 0 : 1;
    c.c0 = (q < nu0 ? q : q - nu0) * kUnitMfma;
  }
  return c;
}

// Next unit in the global order of a launch without T2 units (T0 units, then
// T1 units, group after group).
__device__ __forceinline__ void cursor_next(const AttnArgs& a, Cursor& c) {
  c.c0 += kUnitMfma;
  if (c.c0 < seg_len<false>(c)) return;
  c.c0 = 0;
  if (c.seg == 0 && c.n1 > 0) {
    c.seg = 1;
    return;
  }
  if (++c.g == a.hkv) {
    c.g = 0;
    ++c.lr;
  }
  ++c.lgl;
  if (c.lgl == a.Lr * a.hkv) {  // next sequence with work
    c.lgl = c.lr = c.g = 0;
    do {
      ++c.bl;
    } while (c.bl < a.seq.nb && a.seq.units[c.bl] == 0);
    if (c.bl < a.seq.nb) {
      c.n0 = a.seq.t0_len[c.bl];
      c.n1 = a.seq.t1_len[c.bl];
    }
  }
  c.seg = c.n0 > 0 ? 0 : 1;
}

// Operand registers of one unit.  T2 units hold 8 int8 codes per operand in
// .x/.y (widened to bf16 when consumed) and the key / value scales of the
// lane's 8 tokens.
template <int D>
struct UnitLoads {
  uint4 k[2][D / 32];
  uint4 v[D / 16];
  float4 ks[2], vs[2];
};

template <int D>
struct WaveState {
  f32x4_t acc[D / 16];
  bf16x8_t qop[D / 32];
  float m, lsum;  // running max (base-2 logits) and partial sum of this lane's 8 columns
  long group;     // group index within the launch of the current softmax
  long lrow0;     // element offset in `alpha` of the group's first query head row
};

// Logits are staged in LDS and written in bursts: stores interleaved with the
// key/value stream cost this GPU about a fifth of its read bandwidth, while a
// burst after the last load costs only its own bytes.  Per wave: up to
// kStageUnits units of [G heads][32 tokens] floats, with each unit's destination.
// 36 KB per wave (four waves per workgroup, one per SIMD: 147 KB of LDS) holds 41
// units of seven heads: at chain-8K sizes (27 units per wave) every logit goes out
// after the wave's last load; larger launches (a ragged 16-sequence batch: ~200
// units per wave) flush a third less often than with 24 KB (1% faster there).
constexpr int kStageFloats = 9216;
constexpr int kStageUnits = 64;

struct Stage {
  float* buf;   // this wave's slice of LDS
  long* dst;    // per staged unit: element offset of (head 0, first token) in alpha
  int* count;   // per staged unit: valid tokens
  int n;        // units staged
  int cap;      // capacity in units for this group size
};

// GEO: q and alpha rows may belong to arrays of every layer (io_L, io_l0).
template <int D, bool GEO>
__device__ __forceinline__ void begin_group(const AttnArgs& a, const Cursor& c, int h, int grp,
                                            int G, WaveState<D>& st) {
  constexpr int KB = D / 32, NB = D / 16;
  const long b = a.seq.b_offset + c.bl;
  st.group = (long)c.bl * a.Lr * a.hkv + c.lgl;
  long row0;
  if constexpr (GEO) row0 = (b * a.io_L + a.io_l0 + c.lr) * a.hq + (long)c.g * G;
  else row0 = (b * a.Lr + c.lr) * a.hq + (long)c.g * G;
  const uint16_t* qrow = (const uint16_t*)a.q + (row0 + h) * D;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (h < G) v = *(const uint4*)(qrow + kb * 32 + grp * 8);
    st.qop[kb] = as_bf16x8(v);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) st.acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.lsum = 0.f;
  st.lrow0 = row0 * a.alpha_stride;
}

// Split record of (worker, group): per head of the group, (m, l) and the partial P.V.
template <int D>
__device__ __forceinline__ void flush_record(const AttnArgs& a, long worker, int h, int grp, int G,
                                             WaveState<D>& st) {
  constexpr int NB = D / 16;
  float l = st.lsum;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const long rec = (worker + st.group) * G;
  if (grp == 0 && h < G) {
    a.ml[(rec + h) * 2] = st.m;
    a.ml[(rec + h) * 2 + 1] = l;
  }
  if (grp < (G + 3) / 4) {  // lane groups holding real heads; one whole row per store
    float* base = a.part + (worker + st.group) * part_rec_floats(G, D);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) base[part_off(G, D, grp * 4 + r, nb * 16 + h)] = st.acc[nb][r];
  }
}

// Write every staged unit.  Units go in batches of kFlushBatch whose LDS reads are
// all issued before the first store needs one: a store per LDS round trip would leave
// every wave ~5 round trips per unit at the end of the launch, when nothing else hides
// them.  A store covers one head of two consecutive units (lanes 0-31 and 32-63): 256
// contiguous bytes of a logit row when the units are consecutive.  NT: a flush made
// while the wave still streams keys and values (its stage full) uses non-temporal
// stores -- lines written with normal stores are held in the caches and written back in
// the middle of the read stream, which on large launches cost more than the stores
// themselves; the last flush of a wave uses normal stores, as the merge reads those
// lines back next.  Whether the first kind goes out non-temporal is the launch's
// `stage_nt`, set on the host (see launch_attn_partial).
constexpr int kFlushBatch = 8;

template <bool NT>
__device__ __forceinline__ void flush_stage(const AttnArgs& a, int lane, int G, Stage& sg) {
  constexpr int J = kFlushBatch / 2;  // unit pairs per batch
  const int t = lane & 31;
  const int half = lane >> 5;
  for (int u0 = 0; u0 < sg.n; u0 += kFlushBatch) {
    int src[J], cnt[J];
    long dst[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      src[j] = min(u0 + 2 * j + half, sg.n - 1);  // reads stay inside the staged units
      dst[j] = sg.dst[src[j]];
      cnt[j] = sg.count[src[j]];
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (u0 + 2 * j + half >= sg.n) cnt[j] = 0;  // past the last staged unit: nothing to write
    for (int h0 = 0; h0 < G; h0 += 2) {
      float v[2][J];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < J; ++j) v[e][j] = sg.buf[(src[j] * G + min(h0 + e, G - 1)) * 32 + t];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (h0 + e < G && t < cnt[j]) {
            float* p = a.alpha + dst[j] + (h0 + e) * a.alpha_stride + t;
            if constexpr (NT) __builtin_nontemporal_store(v[e][j], p);
            else *p = v[e][j];
          }
    }
  }
  sg.n = 0;
}

// Loads of one unit: with K-tiles and V-tiles every operand is one contiguous
// 1 KB wave access at lane offset kb*64 + lane (K) or nb*64 + lane (V).  The
// 32-slot block is always inside the allocation (capacities are multiples of
// 32); slots past the segment end are masked when consumed.
// Key and value loads are marked non-temporal: every K/V byte is read exactly
// once per step, and a normal load lets that stream (hundreds of MB) push out of
// the caches the lines that are written during the launch (staged logits, split
// records), which then go back to HBM in the middle of the read stream.  On
// MI355X this alone took the chain-8K launch from ~87 us to ~77 us.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

// 8 int8 codes of a T2 operand (the same element order at one byte each: every
// operand load is one contiguous 512-byte wave access), kept in .x/.y.
__device__ __forceinline__ uint4 ld_stream8(const uint2* p) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint4(x.x, x.y, 0u, 0u);
}

// int8 codes -> bf16, exactly (|code| <= 127 needs 7 significant bits): the
// float32 conversion of the code, truncated to its upper half.
__device__ __forceinline__ uint32_t bf16_pair_of_codes(uint32_t w, int sh) {
  const float lo = (float)(int)(int8_t)(w >> sh);
  const float hi = (float)(int)(int8_t)(w >> (sh + 8));
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

__device__ __forceinline__ bf16x8_t widen_codes(const uint4& x) {
  return as_bf16x8(make_uint4(bf16_pair_of_codes(x.x, 0), bf16_pair_of_codes(x.x, 16),
                              bf16_pair_of_codes(x.y, 0), bf16_pair_of_codes(x.y, 16)));
}

// Row index (sequence, layer, KV head) of the unit's group in a uniform pool (the
// T2 pool), and its pool row inside the sequence (layer * Hkv + KV head).
__device__ __forceinline__ long unit_row(const AttnArgs& a, const Cursor& c) {
  const long b = a.seq.b_offset + c.bl;
  return (b * a.L + a.layer_begin + c.lr) * a.hkv + c.g;
}
__device__ __forceinline__ long unit_lg(const AttnArgs& a, const Cursor& c) {
  return (long)(a.layer_begin + c.lr) * a.hkv + c.g;
}

// The T1 window of a call may hold every layer of a sequence (t1_L = L,
// t1_l0 = layer_begin) or only the call's layers (t1_L = Lr, t1_l0 = 0: a
// window streamed layer by layer from host memory).  Consecutive (sequence,
// layer, KV head) rows of the window lie t1_rs elements apart (cap1 * D for
// separate key and value arrays; 2 * cap1 * D when each row's keys are followed
// by its values, the layout of a streamed window).
template <int D, bool Q8, bool GEO>
__device__ __forceinline__ long unit_base(const AttnArgs& a, const Cursor& c) {
  if constexpr (Q8) {
    return unit_row(a, c) * (long)a.cap2 * D + (long)c.c0 * D;
  } else if constexpr (GEO) {
    const long b = a.seq.b_offset + c.bl;
    if (c.seg == 1)
      return ((b * a.t1_L + a.t1_l0 + c.lr) * a.hkv + c.g) * a.t1_rs + (long)c.c0 * D;
    return pool_row(a.pool.blk0, a.pool.cap0, c.bl, unit_lg(a, c), D) + (long)c.c0 * D;
  } else {
    return (c.seg ? pool_row(a.pool.blk1, a.pool.cap1, c.bl, unit_lg(a, c), D)
                  : pool_row(a.pool.blk0, a.pool.cap0, c.bl, unit_lg(a, c), D)) +
           (long)c.c0 * D;
  }
}

// Q8: the unit is a T2 unit.  The format is a compile-time property of every
// load loop: loads of two formats into the same prefetch registers behind a
// branch make the compiler wait for them early and the stream loses its overlap.
template <int D, bool Q8, bool GEO>
__device__ __forceinline__ void issue_k(const AttnArgs& a, const Cursor& c, int lane, int grp,
                                        UnitLoads<D>& L) {
  constexpr int KB = D / 32;
  if constexpr (Q8) {  // int8 codes, and both scales of the lane's 8 tokens
    const uint2* Ku = (const uint2*)(a.k2 + unit_base<D, Q8, GEO>(a, c));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) L.k[u][kb] = ld_stream8(&Ku[u * 2 * D + kb * 64 + lane]);
    const long so = unit_row(a, c) * (long)a.cap2 + c.c0 + 8 * grp;
    const float4* ks = (const float4*)(a.ks2 + so);
    const float4* vs = (const float4*)(a.vs2 + so);
    L.ks[0] = ks[0];
    L.ks[1] = ks[1];
    L.vs[0] = vs[0];
    L.vs[1] = vs[1];
    return;
  }
  const uint4* Ku = (const uint4*)((const uint16_t*)(c.seg ? a.k1 : a.k0) + unit_base<D, Q8, GEO>(a, c));
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) L.k[u][kb] = ld_stream(&Ku[u * 2 * D + kb * 64 + lane]);
}

template <int D, bool Q8, bool GEO>
__device__ __forceinline__ void issue_v(const AttnArgs& a, const Cursor& c, int lane,
                                        UnitLoads<D>& L) {
  constexpr int NB = D / 16;
  if constexpr (Q8) {
    const uint2* Vu = (const uint2*)(a.v2 + unit_base<D, Q8, GEO>(a, c));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) L.v[nb] = ld_stream8(&Vu[nb * 64 + lane]);
    return;
  }
  const uint4* Vu = (const uint4*)((const uint16_t*)(c.seg ? a.v1 : a.v0) + unit_base<D, Q8, GEO>(a, c));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) L.v[nb] = ld_stream(&Vu[nb * 64 + lane]);
}

// Append fused into the attention launch: the wave that owns the T0 unit holding
// a sequence's new slot writes the new key/value rows of that (layer, KV head)
// into the pool; only that wave reads the unit.  The rows are fetched first, the
// wave's first unit is requested, and only then are the rows stored (the store
// waits for the fetch, not for the unit), so the stream starts without a bubble.
// A wave reads the stored rows with later instructions of its own (in order for
// the same wave), except when the appended unit is its very first unit: then the
// rows are stored before that unit is requested.  The wave of layer 0 / KV head
// 0 also records the token's position, score 0 and tier T0.
struct AppendRow {
  long blk;     // element offset of the 32-slot pool block
  long row;     // element offset of the new row in k_new / v_new
  int rn;       // slot within the block
  int bl, lgl;  // sequence within the launch; layer * Hkv + KV head
};

// The appended row in this wave's unit range (a range holds at most one T0 tail
// unit per group; the first one is taken, the others are written at once).
template <int D, bool T2>
__device__ bool find_append(const AttnArgs& a, long p0, long p1, int lane, AppendRow& r,
                            long& pu_first) {
  const int per_seq = a.Lr * a.hkv;
  const Cursor first = cursor_at<T2>(a, p0);
  const Cursor last = cursor_at<T2>(a, p1 - 1);
  const long g0 = (long)first.bl * per_seq + first.lgl;
  const long g1 = (long)last.bl * per_seq + last.lgl;
  bool found = false;
  for (long g = g0; g <= g1; ++g) {
    const int bl = (int)(g / per_seq);
    const int lgl = (int)(g - (long)bl * per_seq);
    const int per = a.seq.units[bl];
    if (per == 0) continue;
    const int slot = a.app_slot[bl];
    const long pu = a.seq.base[bl] + (long)lgl * per + slot / kUnitMfma;  // unit holding it
    if (pu < p0 || pu >= p1) continue;
    const long b = a.seq.b_offset + bl;
    const int lr = lgl / a.hkv, gk = lgl - lr * a.hkv;
    AppendRow x;
    x.row = ((b * a.L + a.layer_begin + lr) * a.hkv + gk) * (long)D;
    x.blk = pool_row(a.pool.blk0, a.pool.cap0, bl, (long)(a.layer_begin + lr) * a.hkv + gk, D) +
            (long)(slot & ~(kUnitMfma - 1)) * D;
    x.rn = slot & (kUnitMfma - 1);
    x.bl = bl;
    x.lgl = lgl;
    if (!found) {
      r = x;
      pu_first = pu;
      found = true;
    } else {  // more than one (short segments): write it now, blocking
      const uint16_t* kn = (const uint16_t*)a.kn + x.row;
      const uint16_t* vn = (const uint16_t*)a.vn + x.row;
      if (lane < D / 8)
        *reinterpret_cast<uint4*>((uint16_t*)a.k0 + x.blk + k_off(x.rn, 8 * lane, D)) =
            *reinterpret_cast<const uint4*>(kn + 8 * lane);
#pragma unroll
      for (int d = lane; d < D; d += 64) ((uint16_t*)a.v0)[x.blk + v_off(x.rn, d, D)] = vn[d];
      if (lgl == 0 && lane == 0) {
        const int pos = a.app_pos[bl];
        a.app_t0_pos[b * a.cap0 + slot] = pos;
        if (a.app_scores) a.app_scores[b * a.app_max_ctx + pos] = 0.f;
        if (a.app_tier) a.app_tier[b * a.app_max_ctx + pos] = 0;
      }
    }
  }
  return found;
}

template <int D>
__device__ __forceinline__ void store_append(const AttnArgs& a, const AppendRow& r, int lane,
                                             const uint4& kx, const uint16_t (&vx)[D / 64]) {
  if (lane < D / 8)
    *reinterpret_cast<uint4*>((uint16_t*)a.k0 + r.blk + k_off(r.rn, 8 * lane, D)) = kx;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) ((uint16_t*)a.v0)[r.blk + v_off(r.rn, lane + 64 * i, D)] = vx[i];
  if (r.lgl == 0 && lane == 0) {
    const long b = a.seq.b_offset + r.bl;
    const int pos = a.app_pos[r.bl];
    a.app_t0_pos[b * a.cap0 + a.app_slot[r.bl]] = pos;
    if (a.app_scores) a.app_scores[b * a.app_max_ctx + pos] = 0.f;
    if (a.app_tier) a.app_tier[b * a.app_max_ctx + pos] = 0;
  }
}

template <int D, bool Q8, bool GEO>
__device__ __forceinline__ void issue_loads(const AttnArgs& a, const Cursor& c, int lane, int grp,
                                            UnitLoads<D>& L) {
  issue_k<D, Q8, GEO>(a, c, lane, grp, L);
  issue_v<D, Q8, GEO>(a, c, lane, L);
}

// Logits of one unit from its keys: S^T = K Q^T, staged in LDS, the online
// softmax update, and P (bf16 high part + bf16 remainder) for P.V.
// Q8 (a T2 unit): the keys are int8 codes, widened exactly to bf16, so the
// product is q.code; the row's key scale turns it into q.(code x scale).  The
// values are codes too: P enters P.V multiplied by each row's value scale,
// while the softmax sum keeps the plain weights.
template <int D, bool FULL, bool Q8>
__device__ __forceinline__ void unit_scores(const AttnArgs& a, const Cursor& c, UnitLoads<D>& L,
                                            int h, int grp, int G, WaveState<D>& st, Stage& sg,
                                            bf16x8_t& phi, bf16x8_t& plo) {
  constexpr int KB = D / 32, NB = D / 16;
  constexpr float kLazy = 8.0f;  // rescale only when the max grows by more than 2^8
  const int c1 = seg_len<Q8>(c);
  const int tb = c.c0 + 8 * grp;  // first of this lane's 8 tokens
  // S^T = K Q^T: this lane gets tokens tb + e (e = 0..7) of head h
  f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const bf16x8_t k0 = Q8 ? widen_codes(L.k[0][kb]) : as_bf16x8(L.k[0][kb]);
    const bf16x8_t k1 = Q8 ? widen_codes(L.k[1][kb]) : as_bf16x8(L.k[1][kb]);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, st.qop[kb], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, st.qop[kb], s1, 0, 0, 0);
  }
  float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  if (Q8) {
    const float ks[8] = {L.ks[0].x, L.ks[0].y, L.ks[0].z, L.ks[0].w,
                         L.ks[1].x, L.ks[1].y, L.ks[1].z, L.ks[1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] *= ks[e];
  }
  float pm = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sv[e] *= a.scale;  // base-2 logit: q.k * softmax_scale * log2(e)
    if (!FULL && tb + e >= c1) sv[e] = -INFINITY;
    pm = fmaxf(pm, sv[e]);
  }
  // stage the logits of this unit: [head][32 tokens]
  if (h < G) {
    float4* dst = reinterpret_cast<float4*>(sg.buf + (sg.n * G + h) * 32 + 8 * grp);
    dst[0] = make_float4(sv[0], sv[1], sv[2], sv[3]);
    dst[1] = make_float4(sv[4], sv[5], sv[6], sv[7]);
  }
  if ((threadIdx.x & 63) == 0) {
    sg.dst[sg.n] = st.lrow0 + seg_off<Q8>(c) + c.c0;
    sg.count[sg.n] = min(kUnitMfma, c1 - c.c0);
  }
  ++sg.n;
  pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
  pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
  if (__ballot(pm > st.m + kLazy) != 0ull) {
    const float mn = fmaxf(st.m, pm);
    const float corr = __builtin_amdgcn_exp2f(st.m - mn);  // 0 on the first unit (m = -inf)
    st.lsum *= corr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float cr = __shfl(corr, grp * 4 + r, 64);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) st.acc[nb][r] *= cr;
    }
    st.m = mn;
  }
  float vsc[8];
  if (Q8) {
    vsc[0] = L.vs[0].x; vsc[1] = L.vs[0].y; vsc[2] = L.vs[0].z; vsc[3] = L.vs[0].w;
    vsc[4] = L.vs[1].x; vsc[5] = L.vs[1].y; vsc[6] = L.vs[1].z; vsc[7] = L.vs[1].w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float pe = __builtin_amdgcn_exp2f(sv[e] - st.m);  // masked slots: exp2(-inf) = 0
    st.lsum += pe;
    float pv = pe;
    // masked T2 slots: P is 0 whatever the stale scale past the segment end holds
    if (Q8) pv = (FULL || tb + e < c1) ? pe * vsc[e] : 0.f;
    const __bf16 hb = (__bf16)pv;
    phi[e] = hb;
    plo[e] = (__bf16)(pv - (float)hb);
  }
}

// O += P V (high part, then the remainder).  Q8: the values are int8 codes,
// widened exactly; P already carries the value scales.
template <int D, bool FULL, bool Q8>
__device__ __forceinline__ void unit_values(const Cursor& c, UnitLoads<D>& L, int grp,
                                            const bf16x8_t& phi, const bf16x8_t& plo,
                                            WaveState<D>& st) {
  constexpr int NB = D / 16;
  if (Q8) {  // codes are finite, and P is 0 on masked slots: nothing to clear
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8_t v = widen_codes(L.v[nb]);
      st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, v, st.acc[nb], 0, 0, 0);
      st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, v, st.acc[nb], 0, 0, 0);
    }
    return;
  }
  if (!FULL) {  // tail: zero the value slots past the end of the segment (they may hold NaN)
    const int valid = seg_len<Q8>(c) - (c.c0 + 8 * grp);
    if (valid < 8) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        uint32_t* wds = (uint32_t*)&L.v[nb];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= valid) wds[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, as_bf16x8(L.v[nb]), st.acc[nb], 0, 0, 0);
    st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, as_bf16x8(L.v[nb]), st.acc[nb], 0, 0, 0);
  }
}


template <bool Q8>
__device__ __forceinline__ bool unit_full(const Cursor& c) {
  return c.c0 + kUnitMfma <= seg_len<Q8>(c);
}

// One unit of format Q8: group change, staging, Q.K, the next unit's keys (the
// next unit, when `more`, has the same format), P.V, its values.
template <int D, bool Q8, bool GEO>
__device__ __forceinline__ void process_unit(const AttnArgs& a, const Cursor& c, UnitLoads<D>& L,
                                             const Cursor& cn, bool more, long w, int lane,
                                             int h, int grp, int G, WaveState<D>& st, Stage& sg) {
  const long group = (long)c.bl * a.Lr * a.hkv + c.lgl;
  if (group != st.group) {
    flush_record<D>(a, w, h, grp, G, st);
    begin_group<D, GEO>(a, c, h, grp, G, st);
  }
  if (sg.n == sg.cap) {  // two instances: a store hint chosen at run time would be merged away
    if (a.stage_nt) flush_stage<true>(a, lane, G, sg);
    else flush_stage<false>(a, lane, G, sg);
  }
  bf16x8_t phi, plo;
  const bool full = unit_full<Q8>(c);
  if constexpr (Q8) {  // 8-bit T2 rows (codes are finite: no tail clearing of values)
    if (full) unit_scores<D, true, true>(a, c, L, h, grp, G, st, sg, phi, plo);
    else unit_scores<D, false, true>(a, c, L, h, grp, G, st, sg, phi, plo);
    if (more) issue_k<D, Q8, GEO>(a, cn, lane, grp, L);
    unit_values<D, true, true>(c, L, grp, phi, plo, st);
    if (more) issue_v<D, Q8, GEO>(a, cn, lane, L);
  } else {
    if (full) unit_scores<D, true, false>(a, c, L, h, grp, G, st, sg, phi, plo);
    else unit_scores<D, false, false>(a, c, L, h, grp, G, st, sg, phi, plo);
    if (more) issue_k<D, Q8, GEO>(a, cn, lane, grp, L);
    if (full) unit_values<D, true, false>(c, L, grp, phi, plo, st);
    else unit_values<D, false, false>(c, L, grp, phi, plo, st);
    if (more) issue_v<D, Q8, GEO>(a, cn, lane, L);
  }
}

// A run of n units of one format inside one group, starting at c (left at the
// run's last unit), with its own rolling prefetch.  Launches with T2 units walk
// their work as such runs: a group's T0 and T1 units, then its T2 units.
template <int D, bool Q8, bool GEO>
__device__ __forceinline__ void run_units(const AttnArgs& a, Cursor& c, long n, long w, int lane,
                                          int h, int grp, int G, WaveState<D>& st, Stage& sg) {
  UnitLoads<D> L;
  issue_loads<D, Q8, GEO>(a, c, lane, grp, L);
  for (long i = 0; i < n; ++i) {
    const bool more = i + 1 < n;
    Cursor cn = c;
    if (more) {  // the next unit of the run: same group, T0 -> T1 at most
      cn.c0 += kUnitMfma;
      if constexpr (!Q8) {
        if (cn.c0 >= (cn.seg ? cn.n1 : cn.n0)) {
          cn.seg = 1;
          cn.c0 = 0;
        }
      }
    }
    process_unit<D, Q8, GEO>(a, c, L, cn, more, w, lane, h, grp, G, st, sg);
    c = cn;
  }
}


// T2: the launch has T2 units (walked as runs of one format); GEO: the T1
// window and the q / out / alpha rows use the geometry of a window call.
// One workgroup per CU: the logit stage takes 147 KB of the CU's 160 KB of LDS.
template <int D, bool T2, bool GEO>
__global__ __launch_bounds__(256, 1) void attn_partial_mfma_kernel(AttnArgs a) {
  __shared__ float stage_buf[4][kStageFloats];
  __shared__ long stage_dst[4][kStageUnits];
  __shared__ int stage_cnt[4][kStageUnits];
  const int lane = threadIdx.x & 63;
  const int h = lane & 15;    // head column of S^T / P row; token row of the K operand
  const int grp = lane >> 4;  // k-slice of the operands; 8-token block of the unit
  // The worker index is uniform across the wave; saying so keeps the whole unit
  // cursor in scalar registers (scalar loads of the sequence table, no vector
  // memory waits for bookkeeping).
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long w = (long)blockIdx.x * 4 + wv;
  const long P = a.total_units, W = a.workers;
  if (w >= W) return;  // the last workgroup may hold waves past the worker count
  const long p0 = w * P / W, p1 = (w + 1) * P / W;
  if (p0 >= p1) return;  // this wave has no work (small launches)
  const int G = a.hq / a.hkv;
  Stage sg;
  sg.buf = stage_buf[wv];
  sg.dst = stage_dst[wv];
  sg.count = stage_cnt[wv];
  sg.n = 0;
  sg.cap = min(kStageUnits, kStageFloats / (32 * G));
  AppendRow ar;
  long pu = -1;
  const bool app = a.kn && find_append<D, T2>(a, p0, p1, lane, ar, pu);
  uint4 kx = make_uint4(0, 0, 0, 0);
  uint16_t vx[D / 64];
  if (app) {  // fetch the new rows
    if (lane < D / 8) kx = *reinterpret_cast<const uint4*>((const uint16_t*)a.kn + ar.row + 8 * lane);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) vx[i] = ((const uint16_t*)a.vn)[ar.row + lane + 64 * i];
    // the appended unit is the first one requested: in place before it is
    if (pu == p0) {
      store_append<D>(a, ar, lane, kx, vx);
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
  WaveState<D> st;
  Cursor c = cursor_at<T2>(a, p0);
  begin_group<D, GEO>(a, c, h, grp, G, st);
  if constexpr (!T2) {
    // Rolling prefetch: the next unit's keys are requested as soon as Q.K of this
    // unit has consumed the key registers, its values as soon as P.V has consumed
    // the value registers, so a unit's worth of loads stays in flight.
    UnitLoads<D> L;
    issue_loads<D, false, GEO>(a, c, lane, grp, L);
    if (app && pu != p0) store_append<D>(a, ar, lane, kx, vx);  // read back units later
    for (long p = p0; p < p1; ++p) {
      const bool more = p + 1 < p1;
      Cursor cn = c;
      if (more) cursor_next(a, cn);
      process_unit<D, false, GEO>(a, c, L, cn, more, w, lane, h, grp, G, st, sg);
      c = cn;
    }
  } else {
    if (app && pu != p0) {  // before any unit is requested
      store_append<D>(a, ar, lane, kx, vx);
      __builtin_amdgcn_s_waitcnt(0);
    }
    long p = p0;
    for (;;) {
      const int nu0 = (c.n0 + kUnitMfma - 1) / kUnitMfma;
      const int nu1 = (c.n1 + kUnitMfma - 1) / kUnitMfma;
      const int nu2 = (c.n2 + kUnitMfma - 1) / kUnitMfma;
      const int u = c.c0 / kUnitMfma;
      const int q = c.seg == 0 ? u : (c.seg == 1 ? nu0 + u : nu0 + nu1 + u);  // unit in group
      const int end = c.seg == 2 ? nu0 + nu1 + nu2 : nu0 + nu1;              // end of the run
      const long n = min((long)(end - q), p1 - p);
      if (c.seg == 2) run_units<D, true, GEO>(a, c, n, w, lane, h, grp, G, st, sg);
      else run_units<D, false, GEO>(a, c, n, w, lane, h, grp, G, st, sg);
      p += n;
      if (p >= p1) break;
      c = cursor_at<true>(a, p);
    }
  }
  flush_record<D>(a, w, h, grp, G, st);
  flush_stage<false>(a, lane, G, sg);
}

// ---------------------------------------------------------------------------
// float32 path: VALU partial attention, one worker per workgroup, one token per
// thread for Q.K, units of 256 tokens
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(256) void attn_partial_valu_kernel(AttnArgs a) {
  constexpr int NT = 256;
  constexpr int DP = D / 2;    // d pairs in the P.V phase
  constexpr int NG = NT / DP;  // token groups in the P.V phase
  constexpr int TPG = NT / NG; // tokens per group
  __shared__ float4 qs4[G][D / 4];
  __shared__ float ps[G][NT];
  __shared__ float red[G][NT / kWave];
  __shared__ float mfin[G], lfin[G];
  __shared__ float pv[NG][G][D];
  __shared__ float orun[G][D];  // running (unnormalised) output of the current group
  __shared__ float mrun[G], lrun[G];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const long w = blockIdx.x;
  const long P = a.total_units, W = a.workers;
  const long p0 = w * P / W, p1 = (w + 1) * P / W;
  long cur_group = -1;

  auto flush = [&]() {
    const long rec = (w + cur_group) * G;
    float* base = a.part + (w + cur_group) * part_rec_floats(G, D);
    for (int i = tid; i < G * D; i += NT) {
      const int hh = i / D;
      base[part_off(G, D, hh, i - hh * D)] = orun[hh][i - hh * D];
    }
    if (tid < G) {
      a.ml[(rec + tid) * 2] = mrun[tid];
      a.ml[(rec + tid) * 2 + 1] = lrun[tid];
    }
  };

  for (long p = p0; p < p1; ++p) {
    const Unit u = decode_unit(a, p);
    if (u.group != cur_group) {
      if (cur_group >= 0) flush();
      __syncthreads();
      cur_group = u.group;
      const float* qp =
          (const float*)a.q + ((u.b * a.io_L + a.io_l0 + u.lr) * a.hq + (long)u.g * G) * D;
      float* qsf = (float*)&qs4[0][0];
      for (int i = tid; i < G * D; i += NT) {
        qsf[i] = qp[i];
        orun[i / D][i % D] = 0.f;
      }
      if (tid < G) {
        mrun[tid] = -INFINITY;
        lrun[tid] = 0.f;
      }
      __syncthreads();
    }
    const bool q8 = u.seg == 2;  // 8-bit T2 rows: code x scale
    const long lg = (u.b * a.L + a.layer_begin + u.lr) * a.hkv + u.g;  // T2 pool row
    const long lgs = (long)(a.layer_begin + u.lr) * a.hkv + u.g;       // row in the sequence
    const int bl = (int)(u.b - a.seq.b_offset);
    // T1: a window of the call's layers (t1_rs apart), or the T1 pool
    const long t1o = a.t1_L != a.L || a.t1_l0 != a.layer_begin || a.t1_rs != (long)a.cap1 * D
                         ? ((u.b * a.t1_L + a.t1_l0 + u.lr) * a.hkv + u.g) * a.t1_rs
                         : pool_row(a.pool.blk1, a.pool.cap1, bl, lgs, D);
    const long t0o = pool_row(a.pool.blk0, a.pool.cap0, bl, lgs, D);
    const float* Kb = u.seg ? (const float*)a.k1 + t1o : (const float*)a.k0 + t0o;
    const float* Vb = u.seg ? (const float*)a.v1 + t1o : (const float*)a.v0 + t0o;
    const int8_t* Kc = a.k2 + lg * a.cap2 * D;
    const int8_t* Vc = a.v2 + lg * a.cap2 * D;
    const int t = u.c0 + tid;
    const bool valid = t < u.c1;
    float s[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) s[hh] = 0.f;
    if (valid) {
#pragma unroll 2
      for (int c = 0; c < D / 4; ++c) {
        // K-tiles keep 8 consecutive dimensions of a row together
        float4 k4;
        if (q8) {
          const char4 k8 = *(const char4*)(Kc + k_off(t, 4 * c, D));
          k4 = make_float4((float)k8.x, (float)k8.y, (float)k8.z, (float)k8.w);
        } else {
          k4 = *(const float4*)(Kb + k_off(t, 4 * c, D));
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float4 qa = qs4[hh][c];
          float x = s[hh];
          x = fmaf(qa.x, k4.x, x);
          x = fmaf(qa.y, k4.y, x);
          x = fmaf(qa.z, k4.z, x);
          x = fmaf(qa.w, k4.w, x);
          s[hh] = x;
        }
      }
      if (q8) {  // q.code x key scale
        const float ksc = a.ks2[lg * a.cap2 + t];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) s[hh] *= ksc;
      }
    }
    float* lg_out = a.alpha + ((u.b * a.io_L + a.io_l0 + u.lr) * a.hq + (long)u.g * G) * a.alpha_stride +
                    u.off;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float v = valid ? s[hh] * a.scale : -INFINITY;  // base-2 logit
      s[hh] = v;
      if (valid) lg_out[hh * a.alpha_stride + t] = v;
      const float mx = wave_max(v);
      if (lane == 0) red[hh][wid] = mx;
    }
    __syncthreads();
    if (tid < G) {
      float mx = red[tid][0];
      for (int ww = 1; ww < NT / kWave; ++ww) mx = fmaxf(mx, red[tid][ww]);
      mfin[tid] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float pe = valid ? __builtin_amdgcn_exp2f(s[hh] - mfin[hh]) : 0.f;
      ps[hh][tid] = pe;
      const float l = wave_sum(pe);
      if (lane == 0) red[hh][wid] = l;
    }
    __syncthreads();
    if (tid < G) {
      float l = 0.f;
      for (int ww = 0; ww < NT / kWave; ++ww) l += red[tid][ww];
      lfin[tid] = l;
    }
    // P.V over V-tiles
    const int dp = tid % DP;
    const int tg = tid / DP;
    float acc[G][2];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) acc[hh][0] = acc[hh][1] = 0.f;
    const int tend = min(TPG, u.c1 - u.c0 - tg * TPG);
    for (int i = 0; i < tend; ++i) {
      const int tt = tg * TPG + i;
      const long slot = u.c0 + tt;
      float v0, v1;
      if (q8) {  // code x value scale
        const float vsc = a.vs2[lg * a.cap2 + slot];
        v0 = (float)Vc[v_off(slot, 2 * dp, D)] * vsc;
        v1 = (float)Vc[v_off(slot, 2 * dp + 1, D)] * vsc;
      } else {
        v0 = Vb[v_off(slot, 2 * dp, D)];
        v1 = Vb[v_off(slot, 2 * dp + 1, D)];
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pe = ps[hh][tt];
        acc[hh][0] = fmaf(pe, v0, acc[hh][0]);
        acc[hh][1] = fmaf(pe, v1, acc[hh][1]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      pv[tg][hh][2 * dp] = acc[hh][0];
      pv[tg][hh][2 * dp + 1] = acc[hh][1];
    }
    __syncthreads();
    // merge this unit into the running state of the group
    for (int i = tid; i < G * D; i += NT) {
      const int hh = i / D;
      const int d = i - hh * D;
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < NG; ++q) sum += pv[q][hh][d];
      const float mo = mrun[hh], mu = mfin[hh];
      const float mn = fmaxf(mo, mu);
      const float co = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
      const float cu = mu == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mu - mn);
      orun[hh][d] = orun[hh][d] * co + sum * cu;
    }
    __syncthreads();
    if (tid < G) {
      const float mo = mrun[tid], mu = mfin[tid];
      const float mn = fmaxf(mo, mu);
      const float co = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
      const float cu = mu == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mu - mn);
      lrun[tid] = lrun[tid] * co + lfin[tid] * cu;
      mrun[tid] = mn;
    }
    __syncthreads();
  }
  if (cur_group >= 0) flush();
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int D>
static bool launch_valu(const AttnArgs& a, int group, dim3 grid, hipStream_t s,
                        const KernelTimer& timer) {
  switch (group) {
#define TKV_CASE(G)                                                                 \
  case G:                                                                           \
    hipExtLaunchKernelGGL((attn_partial_valu_kernel<D, G>), grid, dim3(256), 0, s,    \
                          timer.start(), timer.stop(), 0, a);                     \
    return true;
    TKV_CASE(1) TKV_CASE(2) TKV_CASE(3) TKV_CASE(4) TKV_CASE(5) TKV_CASE(6) TKV_CASE(7)
    TKV_CASE(8) TKV_CASE(16)
#undef TKV_CASE
    default:
      return false;
  }
}

bool attn_group_supported(int group) { return (group >= 1 && group <= 8) || group == 16; }

// Worker count of attn_partial_mfma: one wave per SIMD (4 per CU).  The kernel
// fits two waves per SIMD, but one streams the keys and values as fast (measured
// on chain8k: 76.1 us against 77.4 us), halves the split records and the work
// of the merge, and leaves LDS for a logit stage that holds a whole wave's share.
int mfma_resident_waves(int head_dim) {
  static int cached = 0;
  (void)head_dim;
  if (cached) return cached;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  cached = cus * 4 < kMaxWorkers ? cus * 4 : kMaxWorkers;
  return cached;
}

// Logit stages that fill before a wave's last load are written with non-temporal
// stores when the launch's logits exceed the memory-side cache (256 MB on MI355X):
// then their lines would only churn it, and written back in the middle of the
// key/value stream they cost more than the stores (a 4 x 32K chain: 2.50 -> 2.22 ms).
// Logits that fit stay cached until the merge reads them back (a 16-sequence batch
// with 158 MB of logits: 0.54 ms, 0.57 ms with non-temporal stores).
constexpr double kMemorySideCacheBytes = 256.0 * 1024 * 1024;

void launch_attn_partial(const AttnArgs& args, int kv_dtype, int head_dim, int group,
                         hipStream_t s) {
  KernelTimer timer("attn_partial", s);
  AttnArgs a = args;
  a.stage_nt = (double)a.total_units * a.unit * (a.hq / a.hkv) * sizeof(float) >
               kMemorySideCacheBytes;
  if (kv_dtype == TKV_BF16) {
    dim3 grid((unsigned)((a.workers + 3) / 4));
    // variants: a T2 pool with rows in this launch; a T1 window of the call's layers
    // only (with q / out / alpha rows of every layer)
    const bool t2 = a.k2 != nullptr;
    const bool geo = a.t1_L != a.L || a.t1_l0 != a.layer_begin || a.io_L != a.Lr || a.io_l0 != 0 ||
                     a.t1_rs != (long)a.cap1 * head_dim;
#define TKV_MFMA(DD, TT, GG)                                                             \
  hipExtLaunchKernelGGL((attn_partial_mfma_kernel<DD, TT, GG>), grid, dim3(256), 0, s,   \
                        timer.start(), timer.stop(), 0, a)
#define TKV_MFMA_D(DD)                     \
  if (t2 && geo) TKV_MFMA(DD, true, true);  \
  else if (t2) TKV_MFMA(DD, true, false);   \
  else if (geo) TKV_MFMA(DD, false, true);  \
  else TKV_MFMA(DD, false, false);
    if (head_dim == 128) {
      TKV_MFMA_D(128)
    } else {
      TKV_MFMA_D(64)
    }
#undef TKV_MFMA_D
#undef TKV_MFMA
  } else {
    dim3 grid((unsigned)a.workers);
    if (head_dim == 128) launch_valu<128>(a, group, grid, s, timer);
    else launch_valu<64>(a, group, grid, s, timer);
  }
}

}  // namespace tkv
