// Second half of the decode step: merge the split records of the attention
// kernel into the output O, normalise the weights alpha in place, and add
// their mean over layers and query heads into the importance scores.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490).  Methodologie section 2: the score of a position grows, every
// decode step, by its attention weight averaged over the heads and the layers;
// section 3: T1 rows are attended exactly like T0 rows, so one softmax runs over
// the attended set T0 u T1 (followed, when the caller attends them, by the
// 8-bit T2 rows).
//
// Every (sequence, layer, KV head) group was split between consecutive waves of
// the attention kernel; wave w left, per query head of the group, a record
// (m, l, acc[D]) at index w + group: its running max m (base-2 logits), its sum
// l = sum 2^(S - m) and its unnormalised P.V.  With M = max m and
// Lambda = sum l 2^(m - M):
//   O     = sum acc 2^(m - M) / Lambda
//   alpha = 2^(S - M) / Lambda        (S: the raw base-2 logits left in alpha)
//
// Kernels:
//   attn_merge -- one grid, two kinds of workgroups.  The first `out_blocks`
//       workgroups merge O, one wave per (sequence, layer, query head): the
//       (m, l) of all records are loaded at once (one record per lane) and
//       reduced across the wave, then the acc rows are summed four records at
//       a time.  Every other workgroup owns 1024 consecutive attended slots of
//       one group: it issues the loads of the G logit rows first, works out
//       (M, Lambda) of its G heads from the records while those loads are in
//       flight, then writes alpha (unless the caller keeps the alpha buffer as
//       scratch) and, if scores are kept, the per-slot sum of alpha over the G
//       heads into a [group][slot] array.
//   score_rows -- per 64 attended slots: the float64 sum over the rows of such
//       an array (the group sums of the fused step, or a caller's normalised
//       alpha rows for tkv_update_scores), weighted 1/(num_layers * Hq) and
//       added to the score of each slot's position.  A fixed summation order:
//       the result does not depend on timing.
#include "common.h"
#include "kernels.h"

namespace tkv {

constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 4 * kMergeThreads;  // attended slots per alpha workgroup
constexpr int kScoreThreads = 1024;
constexpr int kScoreRowGroups = kScoreThreads / kScoreSlots;

// Records of the waves that worked on units [s, e) of one group, reduced across
// one wave: M = max m, Lambda = sum l 2^(m - M).  Every lane gets the result.
__device__ __forceinline__ void split_stats(const float* ml, long group, int G, int hh, long s,
                                            long e, long P, long W, float& M, float& lam) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY, l = 0.f;
  if (e > s) {
    const long wf = ((s + 1) * W - 1) / P;  // worker holding unit s
    const long wl = (e * W - 1) / P;        // worker holding unit e - 1
    for (long w = wf + lane; w <= wl; w += kWave) {
      const long ws = w * P / W, we = (w + 1) * P / W;
      if (ws >= we || ws >= e || we <= s) continue;  // no unit of this group
      const long rec = (w + group) * G + hh;
      const float mw = ml[rec * 2], lw = ml[rec * 2 + 1];
      if (mw == -INFINITY) continue;
      if (mw > m) {
        l = fmaf(l, __builtin_amdgcn_exp2f(m - mw), lw);
        m = mw;
      } else {
        l = fmaf(lw, __builtin_amdgcn_exp2f(mw - m), l);
      }
    }
  }
  M = wave_max(m);
  lam = wave_sum(m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - M));
}

// Group geometry shared by both kinds of workgroup.
struct GroupRef {
  long group;  // record group index within the launch
  long s, e;   // its units [s, e)
};

__device__ __forceinline__ GroupRef group_ref(const MergeArgs& a, int bl, int lr, int g) {
  GroupRef r;
  const int gi = lr * a.hkv + g;
  r.group = (long)bl * a.Lr * a.hkv + gi;
  const int per = a.seq.units[bl];
  r.s = a.seq.base[bl] + (long)gi * per;
  r.e = r.s + per;
  return r;
}

template <int D>
__device__ void merge_output_row(const MergeArgs& a, int row_in_launch) {
  constexpr int PER = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int rows = a.Lr * a.hq;
  const int G = a.hq / a.hkv;
  const int bl = row_in_launch / rows;
  const int r = row_in_launch - bl * rows;
  const int lr = r / a.hq;
  const int hd = r - lr * a.hq;
  const int g = hd / G;
  const int hh = hd - g * G;
  const GroupRef ref = group_ref(a, bl, lr, g);
  const long P = a.total_units, W = a.workers;
  float M, lam;
  split_stats(a.ml, ref.group, G, hh, ref.s, ref.e, P, W, M, lam);
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  if (lam > 0.f) {
    const long wf = ((ref.s + 1) * W - 1) / P;
    const long wl = (ref.e * W - 1) / P;
    for (long w0 = wf; w0 <= wl; w0 += kWave) {
      // lane k describes record k of this batch of up to 64 workers
      const long w = w0 + lane;
      int rec = 0;
      float c = 0.f;
      if (w <= wl) {
        const long ws = w * P / W, we = (w + 1) * P / W;
        if (!(ws >= we || ws >= ref.e || we <= ref.s)) {
          rec = (int)((w + ref.group) * G + hh);
          const float mw = a.ml[rec * 2];
          c = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        }
      }
      const int cnt = (int)(wl - w0 + 1 < kWave ? wl - w0 + 1 : kWave);
      for (int k = 0; k < cnt; k += 4) {
        float v[4][PER], cu[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int src = k + u < cnt ? k + u : k;
          const int ru = __shfl(rec, src, kWave);
          cu[u] = k + u < cnt ? __shfl(c, src, kWave) : 0.f;
          const float* pp = a.part + (long)(ru / G) * part_rec_floats(G, D);
#pragma unroll
          for (int i = 0; i < PER; ++i)
            v[u][i] = cu[u] != 0.f ? pp[part_off(G, D, hh, lane + kWave * i)] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < PER; ++i) o[i] = fmaf(v[u][i], cu[u], o[i]);
      }
    }
  }
  const long orow = ((long)(a.seq.b_offset + bl) * a.io_L + a.io_l0 + lr) * a.hq + hd;
  const float inv = lam > 0.f ? 1.0f / lam : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) a.out[orow * D + lane + kWave * i] = o[i] * inv;
}

// The logits are read once and alpha is written once per step: both go
// through non-temporal accesses, so they do not displace lines in the caches
// (measured: ~2 us of the ~15 us launch at chain 8K).
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld_stream4(const float* p) {
  const f32x4v_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void st_stream4(float* p, const float4& y) {
  const f32x4v_t v = {y.x, y.y, y.z, y.w};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4v_t*>(p));
}

template <int GM>
__device__ void normalise_chunk(const MergeArgs& a, int cb) {
  __shared__ float sM[GM], sI[GM];
  int bl = 0;
  while (bl + 1 < a.seq.nb && a.cbase[bl + 1] <= cb) ++bl;
  const int natt = a.seq.t0_len[bl] + a.seq.t1_len[bl] + a.seq.t2_len[bl];
  const int nch = (natt + kMergeChunk - 1) / kMergeChunk;
  const int local = cb - a.cbase[bl];
  const int gi = local / nch;
  const int ch = local - gi * nch;
  const int lr = gi / a.hkv;
  const int g = gi - lr * a.hkv;
  const int G = a.hq / a.hkv;
  const long b = a.seq.b_offset + bl;
  const int j0 = ch * kMergeChunk + 4 * (int)threadIdx.x;
  const bool full = j0 + 3 < natt;
  float* arow = a.alpha + ((b * a.io_L + a.io_l0 + lr) * a.hq + (long)g * G) * a.alpha_stride + j0;

  // 1. logits of the G heads for this thread's 4 slots (loads in flight during 2.)
  float4 x[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    x[h] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (h < G) {
      const float* p = arow + (long)h * a.alpha_stride;
      if (full) {
        x[h] = ld_stream4(p);
      } else if (j0 < natt) {
        x[h].x = p[0];
        if (j0 + 1 < natt) x[h].y = p[1];
        if (j0 + 2 < natt) x[h].z = p[2];
      }
    }
  }
  // 2. (M, 1/Lambda) of the group's heads, wave h % 4 computing head h
  const GroupRef ref = group_ref(a, bl, lr, g);
  const int wv = threadIdx.x / kWave;
  for (int h = wv; h < G; h += kMergeThreads / kWave) {
    float M, lam;
    split_stats(a.ml, ref.group, G, h, ref.s, ref.e, a.total_units, a.workers, M, lam);
    if ((threadIdx.x & (kWave - 1)) == 0) {
      sM[h] = M;
      sI[h] = lam > 0.f ? 1.0f / lam : 0.f;
    }
  }
  __syncthreads();
  if (j0 >= natt) return;
  // 3. alpha in place, and the sum over the group's heads
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G) {
      const float m = sM[h], inv = sI[h];
      float4 y;
      y.x = __builtin_amdgcn_exp2f(x[h].x - m) * inv;
      y.y = __builtin_amdgcn_exp2f(x[h].y - m) * inv;
      y.z = __builtin_amdgcn_exp2f(x[h].z - m) * inv;
      y.w = __builtin_amdgcn_exp2f(x[h].w - m) * inv;
      if (a.alpha_out) {
        float* p = arow + (long)h * a.alpha_stride;
        if (full) {
          st_stream4(p, y);
        } else {
          p[0] = y.x;
          if (j0 + 1 < natt) p[1] = y.y;
          if (j0 + 2 < natt) p[2] = y.z;
        }
      }
      sum.x += y.x;
      sum.y += y.y;
      sum.z += y.z;
      sum.w += y.w;
    }
  }
  if (!a.gsum) return;
  float* gp = a.gsum + ((long)bl * a.gs_seq_rows + a.gs_row0 + gi) * a.gs_stride + j0;
  if (full) {
    *reinterpret_cast<float4*>(gp) = sum;
  } else {
    gp[0] = sum.x;
    if (j0 + 1 < natt) gp[1] = sum.y;
    if (j0 + 2 < natt) gp[2] = sum.z;
  }
}

template <int D, int GM>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(MergeArgs a) {
  if ((int)blockIdx.x < a.out_blocks) {
    const int row = (int)blockIdx.x * (kMergeThreads / kWave) + (int)(threadIdx.x / kWave);
    if (row < a.out_rows) merge_output_row<D>(a, row);
    return;
  }
  normalise_chunk<GM>(a, (int)blockIdx.x - a.out_blocks);
}

// ---------------------------------------------------------------------------
// score accumulation: s[pos(j)] += weight * sum_r src[r][j]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kScoreThreads) void score_rows_kernel(ScoreArgs a) {
  __shared__ double red[kScoreRowGroups][kScoreSlots];
  const int tid = threadIdx.x;
  const int lane = tid % kScoreSlots;
  const int rg = tid / kScoreSlots;
  const int blk = blockIdx.x;
  int bl = 0;
  while (bl + 1 < a.seq.nb && a.seq.base[bl + 1] <= blk) ++bl;
  const long b = a.seq.b_offset + bl;
  const int n0 = a.seq.t0_len[bl];
  const int n01 = n0 + a.seq.t1_len[bl];
  const int natt = n01 + a.seq.t2_len[bl];
  const int j = (blk - a.seq.base[bl]) * kScoreSlots + lane;
  // the first row group also owns the score of its slot: its position and the
  // current score are fetched before the rows, so the three loads overlap
  float* sp = nullptr;
  float s_old = 0.f;
  if (rg == 0 && j < natt) {
    const int pos = j < n0    ? a.t0_pos[b * a.cap0 + j]
                    : j < n01 ? a.t1_pos[b * a.cap1 + (j - n0)]
                              : a.t2_pos[b * a.cap2 + (j - n01)];
    if ((unsigned)pos < (unsigned)a.max_ctx) {  // slot maps hold positions < max_ctx
      sp = a.scores + b * a.max_ctx + pos;
      s_old = *sp;
    }
  }
  double acc = 0.0;
  if (j < natt) {
    const float* src = a.src + (long)bl * a.seq_stride + j;
    for (int r0 = rg; r0 < a.rows; r0 += 8 * kScoreRowGroups) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = r0 + u * kScoreRowGroups;
        x[u] = r < a.rows ? src[(long)r * a.row_stride] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += (double)x[u];
    }
  }
  red[rg][lane] = acc;
  __syncthreads();
  if (sp) {
    double t = 0.0;
    for (int q = 0; q < kScoreRowGroups; ++q) t += red[q][tid];
    *sp = s_old + (float)(t * a.weight);
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int merge_alpha_blocks(int natt) { return (natt + kMergeChunk - 1) / kMergeChunk; }
int merge_output_blocks(int rows) { return (rows + kMergeThreads / kWave - 1) / (kMergeThreads / kWave); }

void launch_attn_merge(const MergeArgs& a, int head_dim, int nblocks, hipStream_t s) {
  KernelTimer timer("attn_merge", s);
  const int G = a.hq / a.hkv;
  dim3 grid(nblocks), block(kMergeThreads);
  if (head_dim == 128) {
    if (G <= 8) hipExtLaunchKernelGGL((attn_merge_kernel<128, 8>), grid, block, 0, s,
                                      timer.start(), timer.stop(), 0, a);
    else hipExtLaunchKernelGGL((attn_merge_kernel<128, 16>), grid, block, 0, s,
                               timer.start(), timer.stop(), 0, a);
  } else {
    if (G <= 8) hipExtLaunchKernelGGL((attn_merge_kernel<64, 8>), grid, block, 0, s,
                                      timer.start(), timer.stop(), 0, a);
    else hipExtLaunchKernelGGL((attn_merge_kernel<64, 16>), grid, block, 0, s,
                               timer.start(), timer.stop(), 0, a);
  }
}

void launch_score_rows(const ScoreArgs& a, int nblocks, const char* name, hipStream_t s) {
  KernelTimer timer(name, s);
  hipExtLaunchKernelGGL(score_rows_kernel, dim3(nblocks), dim3(kScoreThreads), 0, s,
                        timer.start(), timer.stop(), 0, a);
}

}  // namespace tkv
