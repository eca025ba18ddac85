// Decode attention over T0 u T1 and the importance-score accumulation.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490).  Methodologie section 1: T1 rows reach the GPU before the
// attention step; section 3: they then enter the softmax exactly like resident
// rows, so attention runs over the concatenation of the T0 pool and the T1
// window.  Section 2: the score of a position grows by its attention weight
// averaged over heads and layers.
//
// Kernels (one decode step, all requested layers in one launch each):
//   attn_partial  -- split-K over the attended index: per (sequence, layer, KV
//                    head, chunk of CH tokens) the logits of the group's query
//                    heads, their chunk max m, l = sum exp(S - m) and
//                    acc = sum exp(S - m) V.  Raw scaled logits go to `alpha`.
//   attn_combine  -- per (sequence, layer, query head): M = max m, Lambda =
//                    sum l exp(m - M), O = sum acc exp(m - M) / Lambda; stores
//                    (M, 1/Lambda).
//   alpha_score   -- per block of 64 attended slots: alpha = exp(S - M)/Lambda
//                    written in place, summed over every (layer, head) in
//                    float64 and added, weighted 1/(num_layers*Hq), to the
//                    score of the slot's position.  Also the standalone score
//                    update (alpha already normalised).
#include "common.h"
#include "kernels.h"

namespace tkv {

// ---------------------------------------------------------------------------
// K1: split-K partial attention (VALU; one token per thread for Q.K)
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(AttnArgs a) {
  constexpr int NT = kAttnThreads;
  constexpr int CH = kAttnChunk;
  constexpr int DP = D / 2;       // d pairs: one per thread in the P.V phase
  constexpr int NG = NT / DP;     // token groups in the P.V phase
  constexpr int TPG = CH / NG;    // tokens per group
  static_assert(CH == NT, "one token per thread in the Q.K phase");

  __shared__ float4 qs4[G][D / 4];
  __shared__ float ps[G][CH];
  __shared__ float red[G][NT / kWave];
  __shared__ float mfin[G], lfin[G];
  __shared__ const T* vrow[CH];
  __shared__ float pv[NG][G][D];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int chunk = blockIdx.x;
  int bl = 0;
  while (bl + 1 < a.seq.nb && a.seq.base[bl + 1] <= chunk) ++bl;
  const int split = chunk - a.seq.base[bl];
  const long b = a.seq.b_offset + bl;
  const int lr = blockIdx.y / a.hkv;
  const int g = blockIdx.y - lr * a.hkv;
  const long layer = a.layer_begin + lr;
  const int n0 = a.seq.t0_len[bl];
  const int natt = n0 + a.seq.t1_len[bl];
  const int j0 = split * CH;

  const T* qp = (const T*)a.q + ((b * a.Lr + lr) * a.hq + (long)g * G) * D;
  float* qsf = (float*)&qs4[0][0];
  for (int i = tid; i < G * D; i += NT) qsf[i] = to_f32(qp[i]);

  const int j = j0 + tid;
  const bool valid = j < natt;
  const T* krow = nullptr;
  const T* vr = nullptr;
  if (valid) {
    const long lg = (b * a.L + layer) * a.hkv + g;
    if (j < n0) {
      const long off = (lg * a.cap0 + j) * D;
      krow = (const T*)a.k0 + off;
      vr = (const T*)a.v0 + off;
    } else {
      const long off = (lg * a.cap1 + (j - n0)) * D;
      krow = (const T*)a.k1 + off;
      vr = (const T*)a.v1 + off;
    }
  }
  vrow[tid] = vr;
  __syncthreads();

  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = 0.f;
  if (valid) {
    if constexpr (sizeof(T) == 2) {
      const uint4* kp = (const uint4*)krow;
#pragma unroll 2
      for (int c = 0; c < D / 8; ++c) {
        const uint4 w = kp[c];
        const float k8[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                             bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float4 qa = qs4[h][2 * c];
          const float4 qb = qs4[h][2 * c + 1];
          float t = s[h];
          t = fmaf(qa.x, k8[0], t);
          t = fmaf(qa.y, k8[1], t);
          t = fmaf(qa.z, k8[2], t);
          t = fmaf(qa.w, k8[3], t);
          t = fmaf(qb.x, k8[4], t);
          t = fmaf(qb.y, k8[5], t);
          t = fmaf(qb.z, k8[6], t);
          t = fmaf(qb.w, k8[7], t);
          s[h] = t;
        }
      }
    } else {
      const float4* kp = (const float4*)krow;
#pragma unroll 2
      for (int c = 0; c < D / 4; ++c) {
        const float4 k4 = kp[c];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float4 qa = qs4[h][c];
          float t = s[h];
          t = fmaf(qa.x, k4.x, t);
          t = fmaf(qa.y, k4.y, t);
          t = fmaf(qa.z, k4.z, t);
          t = fmaf(qa.w, k4.w, t);
          s[h] = t;
        }
      }
    }
  }

  float* lg_out = a.alpha + ((b * a.Lr + lr) * a.hq + (long)g * G) * a.alpha_stride;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float v = valid ? s[h] * a.scale : -INFINITY;
    s[h] = v;
    if (valid) lg_out[h * a.alpha_stride + j] = v;
    const float m = wave_max(v);
    if (lane == 0) red[h][wid] = m;
  }
  __syncthreads();
  if (tid < G) {
    float m = red[tid][0];
    for (int w = 1; w < NT / kWave; ++w) m = fmaxf(m, red[tid][w]);
    mfin[tid] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float p = valid ? exp_acc(s[h] - mfin[h]) : 0.f;
    ps[h][tid] = p;
    const float l = wave_sum(p);
    if (lane == 0) red[h][wid] = l;
  }
  __syncthreads();
  if (tid < G) {
    float l = 0.f;
    for (int w = 0; w < NT / kWave; ++w) l += red[tid][w];
    lfin[tid] = l;
  }

  // P.V: thread (dp, tg) accumulates d = 2dp, 2dp+1 over its token group
  const int dp = tid % DP;
  const int tg = tid / DP;
  float acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = 0.f;
  const int tend = min(TPG, natt - j0 - tg * TPG);
  for (int t = 0; t < tend; ++t) {
    const int tt = tg * TPG + t;
    const T* vp = vrow[tt];
    float v0, v1;
    if constexpr (sizeof(T) == 2) {
      const uint32_t w = ((const uint32_t*)vp)[dp];
      v0 = bf16_lo(w);
      v1 = bf16_hi(w);
    } else {
      const float2 f = ((const float2*)vp)[dp];
      v0 = f.x;
      v1 = f.y;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = ps[h][tt];
      acc[h][0] = fmaf(p, v0, acc[h][0]);
      acc[h][1] = fmaf(p, v1, acc[h][1]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    pv[tg][h][2 * dp] = acc[h][0];
    pv[tg][h][2 * dp + 1] = acc[h][1];
  }
  __syncthreads();

  const long row0 = (b * a.Lr + lr) * a.hq + (long)g * G;
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D;
    const int d = i - h * D;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < NG; ++q) sum += pv[q][h][d];
    a.part[((row0 + h) * a.max_splits + split) * D + d] = sum;
  }
  if (tid < G) {
    float* mlp = a.ml + ((row0 + tid) * a.max_splits + split) * 2;
    mlp[0] = mfin[tid];
    mlp[1] = lfin[tid];
  }
}

// ---------------------------------------------------------------------------
// K2: combine the splits of every (sequence, layer, query head)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnArgs a) {
  const int rows = a.Lr * a.hq;
  const int bl = blockIdx.x / rows;
  const int r = blockIdx.x - bl * rows;
  const long b = a.seq.b_offset + bl;
  const int natt = a.seq.t0_len[bl] + a.seq.t1_len[bl];
  const int ns = (natt + kAttnChunk - 1) / kAttnChunk;
  const long row = b * rows + r;
  const float* mlp = a.ml + row * a.max_splits * 2;
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, mlp[2 * s]);
  float lam = 0.f, o = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = exp_acc(mlp[2 * s] - M);
    lam = fmaf(mlp[2 * s + 1], w, lam);
    o = fmaf(a.part[(row * a.max_splits + s) * D + d], w, o);
  }
  a.out[row * D + d] = ns ? o / lam : 0.f;
  if (d == 0) {
    a.stat[row * 2] = M;
    a.stat[row * 2 + 1] = ns ? 1.0f / lam : 0.f;
  }
}

// ---------------------------------------------------------------------------
// K3: alpha normalisation (optional) + score accumulation over (layer, head)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void alpha_score_kernel(ScoreArgs a) {
  constexpr int SLOTS = 64;
  constexpr int GRPS = 256 / SLOTS;
  __shared__ double red[GRPS][SLOTS];
  const int tid = threadIdx.x;
  const int lane = tid & (SLOTS - 1);
  const int grp = tid / SLOTS;
  const int blk = blockIdx.x;
  int bl = 0;
  while (bl + 1 < a.seq.nb && a.seq.base[bl + 1] <= blk) ++bl;
  const long b = a.seq.b_offset + bl;
  const int n0 = a.seq.t0_len[bl];
  const int natt = n0 + a.seq.t1_len[bl];
  const int j = (blk - a.seq.base[bl]) * SLOTS + lane;
  const int rows = a.rows;
  double acc = 0.0;
  if (j < natt) {
    float* ap = a.alpha + b * rows * a.alpha_stride + j;
    const float* st = a.stat + b * rows * 2;
    int r = grp;
    if (a.normalise) {
      for (; r + 3 * GRPS < rows; r += 4 * GRPS) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = ap[(long)(r + u * GRPS) * a.alpha_stride];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int rr = r + u * GRPS;
          const float v = exp_acc(x[u] - st[2 * rr]) * st[2 * rr + 1];
          ap[(long)rr * a.alpha_stride] = v;
          acc += (double)v;
        }
      }
      for (; r < rows; r += GRPS) {
        const float v = exp_acc(ap[(long)r * a.alpha_stride] - st[2 * r]) * st[2 * r + 1];
        ap[(long)r * a.alpha_stride] = v;
        acc += (double)v;
      }
    } else {
      for (; r + 3 * GRPS < rows; r += 4 * GRPS) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = ap[(long)(r + u * GRPS) * a.alpha_stride];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += (double)x[u];
      }
      for (; r < rows; r += GRPS) acc += (double)ap[(long)r * a.alpha_stride];
    }
  }
  if (!a.scores) return;  // normalisation only (block-uniform)
  red[grp][lane] = acc;
  __syncthreads();
  if (grp == 0 && j < natt) {
    double t = red[0][lane];
#pragma unroll
    for (int q = 1; q < GRPS; ++q) t += red[q][lane];
    const int pos = j < n0 ? a.t0_pos[b * a.cap0 + j] : a.t1_pos[b * a.cap1 + (j - n0)];
    if ((unsigned)pos < (unsigned)a.max_ctx) {  // slot maps hold positions < max_ctx
      float* sp = a.scores + b * a.max_ctx + pos;
      *sp = *sp + (float)(t * a.weight);
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
static void launch_partial(const AttnArgs& a, int nchunks, hipStream_t s) {
  dim3 grid(nchunks, a.Lr * a.hkv);
  hipLaunchKernelGGL((attn_partial_kernel<T, D, G>), grid, dim3(kAttnThreads), 0, s, a);
}

template <typename T, int D>
static bool dispatch_group(const AttnArgs& a, int group, int nchunks, hipStream_t s) {
  switch (group) {
    case 1: launch_partial<T, D, 1>(a, nchunks, s); return true;
    case 2: launch_partial<T, D, 2>(a, nchunks, s); return true;
    case 3: launch_partial<T, D, 3>(a, nchunks, s); return true;
    case 4: launch_partial<T, D, 4>(a, nchunks, s); return true;
    case 5: launch_partial<T, D, 5>(a, nchunks, s); return true;
    case 6: launch_partial<T, D, 6>(a, nchunks, s); return true;
    case 7: launch_partial<T, D, 7>(a, nchunks, s); return true;
    case 8: launch_partial<T, D, 8>(a, nchunks, s); return true;
    case 16: launch_partial<T, D, 16>(a, nchunks, s); return true;
    default: return false;
  }
}

bool attn_group_supported(int group) {
  return (group >= 1 && group <= 8) || group == 16;
}

void launch_attn_partial(const AttnArgs& a, int kv_dtype, int head_dim, int group,
                         int nchunks, hipStream_t s) {
  KernelTimer timer("attn_partial", s);
  if (kv_dtype == TKV_BF16) {
    if (head_dim == 128) dispatch_group<uint16_t, 128>(a, group, nchunks, s);
    else dispatch_group<uint16_t, 64>(a, group, nchunks, s);
  } else {
    if (head_dim == 128) dispatch_group<float, 128>(a, group, nchunks, s);
    else dispatch_group<float, 64>(a, group, nchunks, s);
  }
}

void launch_attn_combine(const AttnArgs& a, int head_dim, int nb, hipStream_t s) {
  KernelTimer timer("attn_combine", s);
  dim3 grid(nb * a.Lr * a.hq);
  if (head_dim == 128)
    hipLaunchKernelGGL((attn_combine_kernel<128>), grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<64>), grid, dim3(64), 0, s, a);
}

void launch_alpha_score(const ScoreArgs& a, int nblocks, hipStream_t s) {
  KernelTimer timer(a.normalise ? "alpha_score" : "update_scores", s);
  hipLaunchKernelGGL(alpha_score_kernel, dim3(nblocks), dim3(256), 0, s, a);
}

}  // namespace tkv
