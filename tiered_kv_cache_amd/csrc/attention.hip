// Decode attention over T0 u T1 and the importance-score accumulation.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490).  Methodologie section 1: T1 rows reach the GPU before the
// attention step; section 3: they then enter the softmax exactly like resident
// rows, so attention runs over the T0 pool and the T1 window as one attended
// set.  Section 2: the score of a position grows by its attention weight
// averaged over heads and layers.
//
// Kernels (one decode step; every requested layer in one launch each):
//   attn_partial_mfma -- bf16 path.  A workgroup (4 waves) owns a chunk of one
//       segment (T0 pool or T1 window) of one (sequence, layer, KV head).  Each
//       wave walks 32-token pairs: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (the
//       group's query heads padded to 16 columns), an online softmax with lazy
//       rescaling, and O += P V on the same MFMA with P split into a bf16 high
//       part and a bf16 remainder (P V is then exact to ~2^-17 relative).  The
//       token order inside a pair is permuted so that the S^T accumulator is
//       already the A operand of P V, and V is stored in 8-slot panels
//       (head_dim-major inside a panel) so its B operand is one 16-byte load:
//       no LDS transpose, no shuffles.  The raw scaled logits go to `alpha`.
//   attn_partial_valu -- float32 path (plain FMAs), same work decomposition.
//   Both end with a split record (m, l, acc) and the last workgroup of each
//   (sequence, layer, KV head) -- found with a device-scope counter -- merges
//   the splits: M = max m, Lambda = sum l e^(m-M), O = sum acc e^(m-M) / Lambda,
//   and stores (M, 1/Lambda).
//   alpha_score -- per 16 attended slots (8 waves, 32 row groups): alpha = e^(S-M)/Lambda written in
//       place, summed in float64 over every (layer, head) and added, weighted
//       1/(num_layers*Hq), to the score of the slot's position.  Also the
//       standalone score update (alpha already normalised).
#include "common.h"
#include "kernels.h"

namespace tkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// ---------------------------------------------------------------------------
// work decomposition: per sequence, ceil(t0_len/chunk) T0 tasks then
// ceil(t1_len/chunk) T1 tasks (one empty task for an empty sequence)
// ---------------------------------------------------------------------------
struct Task {
  int bl;
  long b;
  int seg;    // 0: T0 pool, 1: T1 window
  int c0, c1; // slot range inside the segment
  int split;  // index among the sequence's tasks
  int nsplit;
  int n0, n1;
};

__device__ __forceinline__ Task decode_task(const AttnArgs& a, int t) {
  int bl = 0;
  while (bl + 1 < a.seq.nb && a.seq.base[bl + 1] <= t) ++bl;
  Task k;
  k.bl = bl;
  k.b = a.seq.b_offset + bl;
  k.n0 = a.seq.t0_len[bl];
  k.n1 = a.seq.t1_len[bl];
  k.split = t - a.seq.base[bl];
  k.nsplit = a.seq.base[bl + 1] - a.seq.base[bl];
  const int nt0 = (k.n0 + a.chunk - 1) / a.chunk;
  if (k.split < nt0) {
    k.seg = 0;
    k.c0 = k.split * a.chunk;
    k.c1 = min(k.n0, k.c0 + a.chunk);
  } else if (k.n1 > 0) {
    k.seg = 1;
    k.c0 = (k.split - nt0) * a.chunk;
    k.c1 = min(k.n1, k.c0 + a.chunk);
  } else {
    k.seg = 0;
    k.c0 = 0;
    k.c1 = 0;
  }
  return k;
}

// Every workgroup calls this after writing its split record (all threads, with
// `flag` in LDS).  The last one to arrive for its (sequence, layer, KV head)
// merges the splits into the output and the softmax statistics, and resets the
// counter for the next call.
__device__ void merge_if_last(const AttnArgs& a, const Task& k, int lr, int g, int D, int* flag) {
  const int G = a.hq / a.hkv;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int* ctr = a.counters + (k.b * a.Lr + lr) * a.hkv + g;
    const int prev = atomicAdd(ctr, 1);
    const int last = prev == k.nsplit - 1;
    if (last) atomicExch(ctr, 0);
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  __threadfence();
  const long row0 = (k.b * a.Lr + lr) * a.hq + (long)g * G;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int h = i / D;
    const int d = i - h * D;
    const long row = row0 + h;
    const float* mlp = a.ml + row * a.max_splits * 2;
    const float* pp = a.part + row * a.max_splits * D + d;
    float M = -INFINITY;
    for (int s = 0; s < k.nsplit; ++s) M = fmaxf(M, mlp[2 * s]);
    float lam = 0.f, o = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < k.nsplit; ++s) {
        const float ms = mlp[2 * s];
        if (ms == -INFINITY) continue;
        const float w = exp_acc(ms - M);
        lam = fmaf(mlp[2 * s + 1], w, lam);
        o = fmaf(pp[(long)s * D], w, o);
      }
    }
    a.out[row * D + d] = lam > 0.f ? o / lam : 0.f;
    if (d == 0) {
      a.stat[row * 2] = M;
      a.stat[row * 2 + 1] = lam > 0.f ? 1.0f / lam : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 path: MFMA partial attention
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_partial_mfma_kernel(AttnArgs a) {
  constexpr int KB = D / 32;  // k-blocks of S^T = K Q^T
  constexpr int NB = D / 16;  // n-blocks of O = P V
  constexpr float kLazy = 8.0f;  // rescale only when a new max exceeds the old by this
  __shared__ float o_lds[4][16][D + 4];
  __shared__ float m_lds[4][16], l_lds[4][16];
  __shared__ int flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane & 15;    // head column of S^T / P row; token row of the K operand
  const int grp = lane >> 4;  // k-slice of the operands; 8-token block of the pair
  const int lr = blockIdx.y / a.hkv;
  const int g = blockIdx.y - lr * a.hkv;
  const Task k = decode_task(a, blockIdx.x);
  const int G = a.hq / a.hkv;
  const long layer = a.layer_begin + lr;
  const int cap = k.seg ? a.cap1 : a.cap0;
  const long lg = (k.b * a.L + layer) * a.hkv + g;
  const uint16_t* Kb = (const uint16_t*)(k.seg ? a.k1 : a.k0) + lg * cap * D;
  const uint4* Vb = (const uint4*)((const uint16_t*)(k.seg ? a.v1 : a.v0) + lg * cap * D);
  const long jofs = k.seg ? k.n0 : 0;

  // B operand of S^T: lane holds Q[h][kb*32 + grp*8 + e]; heads >= G are zero
  bf16x8_t qop[KB];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((k.b * a.Lr + lr) * a.hq + (long)g * G + h) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (h < G) v = *(const uint4*)(qrow + kb * 32 + grp * 8);
      qop[kb] = as_bf16x8(v);
    }
  }
  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  float* lg_out = a.alpha + ((k.b * a.Lr + lr) * a.hq + (long)g * G + h) * a.alpha_stride + jofs;
  const bool write_logits = h < G;

  for (int pb = k.c0 + 32 * w; pb < k.c1; pb += 128) {
    // --- loads: K rows of the permuted tiles, V panels ---------------------
    uint4 kr[2][KB];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = pb + 8 * (h >> 2) + 4 * u + (h & 3);
      if (t < k.c1) {
        const uint4* src = (const uint4*)(Kb + (long)t * D + grp * 8);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kr[u][kb] = src[kb * 4];
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kr[u][kb] = make_uint4(0, 0, 0, 0);
      }
    }
    const int p = (pb >> 3) + grp;  // this lane's V panel (slots 8p .. 8p+7)
    uint4 vr[NB];
    if (8 * p < k.c1) {
      const uint4* vsrc = Vb + (long)p * D + h;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vr[nb] = vsrc[nb * 16];
      const int valid = k.c1 - 8 * p;
      if (valid < 8) {  // tail panel: zero the slots past the end
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          uint32_t* wds = (uint32_t*)&vr[nb];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= valid) wds[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vr[nb] = make_uint4(0, 0, 0, 0);
    }

    // --- S^T = K Q^T: lane gets tokens pb+8grp+e (e = 0..7) of head h -----
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[0][kb]), qop[kb], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[1][kb]), qop[kb], s1, 0, 0, 0);
    }
    const int tb = pb + 8 * grp;
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float pm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = (tb + e < k.c1) ? sv[e] * a.scale : -INFINITY;
      pm = fmaxf(pm, sv[e]);
    }
    if (write_logits) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (tb + e < k.c1) lg_out[tb + e] = sv[e];
    }
    pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
    pm = fmaxf(pm, __shfl_xor(pm, 32, 64));

    // --- online softmax, rescaling only when the max moves by > kLazy ------
    if (__ballot(pm > m + kLazy) != 0ull) {
      const float mn = fmaxf(m, pm);
      const float corr = (m == -INFINITY) ? 0.f : exp_acc(m - mn);
      lsum *= corr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float cr = __shfl(corr, grp * 4 + r, 64);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb][r] *= cr;
      }
      m = mn;
    }
    bf16x8_t phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = (sv[e] == -INFINITY) ? 0.f : exp_acc(sv[e] - m);
      lsum += pe;
      const __bf16 hb = (__bf16)pe;
      phi[e] = hb;
      plo[e] = (__bf16)(pe - (float)hb);
    }
    // --- O += P V (high part, then the remainder) --------------------------
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, as_bf16x8(vr[nb]), acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, as_bf16x8(vr[nb]), acc[nb], 0, 0, 0);
    }
  }

  // --- merge the 4 waves into this workgroup's split record --------------
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (lane < 16) {
    m_lds[w][lane] = m;
    l_lds[w][lane] = lsum;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) o_lds[w][grp * 4 + r][nb * 16 + h] = acc[nb][r];
  __syncthreads();
  const long row0 = (k.b * a.Lr + lr) * a.hq + (long)g * G;
  for (int i = tid; i < G * D; i += 256) {
    const int hh = i / D;
    const int d = i - hh * D;
    float M = fmaxf(fmaxf(m_lds[0][hh], m_lds[1][hh]), fmaxf(m_lds[2][hh], m_lds[3][hh]));
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = m_lds[ww][hh];
        if (mw == -INFINITY) continue;
        const float c = exp_acc(mw - M);
        o = fmaf(o_lds[ww][hh][d], c, o);
        l = fmaf(l_lds[ww][hh], c, l);
      }
    }
    const long row = row0 + hh;
    a.part[(row * a.max_splits + k.split) * D + d] = o;
    if (d == 0) {
      a.ml[(row * a.max_splits + k.split) * 2] = M;
      a.ml[(row * a.max_splits + k.split) * 2 + 1] = l;
    }
  }
  merge_if_last(a, k, lr, g, D, &flag);
}

// ---------------------------------------------------------------------------
// float32 path: VALU partial attention, one token per thread for Q.K
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
  __shared__ int flag;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int lr = blockIdx.y / a.hkv;
  const int g = blockIdx.y - lr * a.hkv;
  const Task k = decode_task(a, blockIdx.x);
  const long layer = a.layer_begin + lr;
  const int cap = k.seg ? a.cap1 : a.cap0;
  const long lg = (k.b * a.L + layer) * a.hkv + g;
  const float* Kb = (const float*)(k.seg ? a.k1 : a.k0) + lg * cap * D;
  const float* Vb = (const float*)(k.seg ? a.v1 : a.v0) + lg * cap * D;
  const long jofs = k.seg ? k.n0 : 0;

  const float* qp = (const float*)a.q + ((k.b * a.Lr + lr) * a.hq + (long)g * G) * D;
  float* qsf = (float*)&qs4[0][0];
  for (int i = tid; i < G * D; i += NT) qsf[i] = qp[i];
  __syncthreads();

  const int t = k.c0 + tid;
  const bool valid = t < k.c1;
  float s[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) s[hh] = 0.f;
  if (valid) {
    const float4* kp = (const float4*)(Kb + (long)t * D);
#pragma unroll 2
    for (int c = 0; c < D / 4; ++c) {
      const float4 k4 = kp[c];
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
  }
  float* lg_out = a.alpha + ((k.b * a.Lr + lr) * a.hq + (long)g * G) * a.alpha_stride + jofs;
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float v = valid ? s[hh] * a.scale : -INFINITY;
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
    const float pe = valid ? exp_acc(s[hh] - mfin[hh]) : 0.f;
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
  // P.V with V in 8-slot panels: element (slot, d) at ((slot/8)*D + d)*8 + slot%8
  const int dp = tid % DP;
  const int tg = tid / DP;
  float acc[G][2];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) acc[hh][0] = acc[hh][1] = 0.f;
  const int tend = min(TPG, k.c1 - k.c0 - tg * TPG);
  for (int i = 0; i < tend; ++i) {
    const int tt = tg * TPG + i;
    const long slot = k.c0 + tt;
    const float* vp = Vb + ((slot >> 3) * D + 2 * dp) * 8 + (slot & 7);
    const float v0 = vp[0], v1 = vp[8];
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
  const long row0 = (k.b * a.Lr + lr) * a.hq + (long)g * G;
  const bool any = k.c1 > k.c0;
  for (int i = tid; i < G * D; i += NT) {
    const int hh = i / D;
    const int d = i - hh * D;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < NG; ++q) sum += pv[q][hh][d];
    a.part[((row0 + hh) * a.max_splits + k.split) * D + d] = any ? sum : 0.f;
    if (d == 0) {
      a.ml[((row0 + hh) * a.max_splits + k.split) * 2] = any ? mfin[hh] : -INFINITY;
      a.ml[((row0 + hh) * a.max_splits + k.split) * 2 + 1] = any ? lfin[hh] : 0.f;
    }
  }
  merge_if_last(a, k, lr, g, D, &flag);
}

// ---------------------------------------------------------------------------
// alpha normalisation (optional) + score accumulation over (layer, head)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void alpha_score_kernel(ScoreArgs a) {
  constexpr int SL = kScoreSlots;  // slots per workgroup
  constexpr int RG = 32;           // row groups (8 waves x 4 lane groups)
  __shared__ double red[RG][SL];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int rg = (tid >> 6) * 4 + (lane >> 4);
  const int blk = blockIdx.x;
  int bl = 0;
  while (bl + 1 < a.seq.nb && a.seq.base[bl + 1] <= blk) ++bl;
  const long b = a.seq.b_offset + bl;
  const int n0 = a.seq.t0_len[bl];
  const int natt = n0 + a.seq.t1_len[bl];
  const int j = (blk - a.seq.base[bl]) * SL + (lane & 15);
  const int rows = a.rows;
  double acc = 0.0;
  if (j < natt) {
    float* ap = a.alpha + b * rows * a.alpha_stride + j;
    const float* st = a.stat + b * rows * 2;
    int r = rg;
    if (a.normalise) {
      for (; r + 3 * RG < rows; r += 4 * RG) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = ap[(long)(r + u * RG) * a.alpha_stride];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int rr = r + u * RG;
          const float v = exp_acc(x[u] - st[2 * rr]) * st[2 * rr + 1];
          ap[(long)rr * a.alpha_stride] = v;
          acc += (double)v;
        }
      }
      for (; r < rows; r += RG) {
        const float v = exp_acc(ap[(long)r * a.alpha_stride] - st[2 * r]) * st[2 * r + 1];
        ap[(long)r * a.alpha_stride] = v;
        acc += (double)v;
      }
    } else {
      for (; r + 3 * RG < rows; r += 4 * RG) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = ap[(long)(r + u * RG) * a.alpha_stride];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += (double)x[u];
      }
      for (; r < rows; r += RG) acc += (double)ap[(long)r * a.alpha_stride];
    }
  }
  if (!a.scores) return;  // normalisation only (block-uniform)
  red[rg][lane & 15] = acc;
  __syncthreads();
  if (tid < SL && j < natt) {
    double t = 0.0;
    for (int q = 0; q < RG; ++q) t += red[q][tid];
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
template <int D>
static bool launch_valu(const AttnArgs& a, int group, dim3 grid, hipStream_t s) {
  switch (group) {
#define TKV_CASE(G)                                                                 \
  case G:                                                                           \
    hipLaunchKernelGGL((attn_partial_valu_kernel<D, G>), grid, dim3(256), 0, s, a); \
    return true;
    TKV_CASE(1) TKV_CASE(2) TKV_CASE(3) TKV_CASE(4) TKV_CASE(5) TKV_CASE(6) TKV_CASE(7)
    TKV_CASE(8) TKV_CASE(16)
#undef TKV_CASE
    default:
      return false;
  }
}

bool attn_group_supported(int group) { return (group >= 1 && group <= 8) || group == 16; }

void launch_attn_partial(const AttnArgs& a, int kv_dtype, int head_dim, int group, int ntasks,
                         hipStream_t s) {
  KernelTimer timer("attn_partial", s);
  dim3 grid(ntasks, a.Lr * a.hkv);
  if (kv_dtype == TKV_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_partial_mfma_kernel<128>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((attn_partial_mfma_kernel<64>), grid, dim3(256), 0, s, a);
  } else {
    if (head_dim == 128) launch_valu<128>(a, group, grid, s);
    else launch_valu<64>(a, group, grid, s);
  }
}

void launch_alpha_score(const ScoreArgs& a, int nblocks, hipStream_t s) {
  KernelTimer timer(a.normalise ? "alpha_score" : "update_scores", s);
  hipLaunchKernelGGL(alpha_score_kernel, dim3(nblocks), dim3(512), 0, s, a);
}

}  // namespace tkv
