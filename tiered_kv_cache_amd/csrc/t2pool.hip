// The attended T2 pool: 8-bit rows kept on the device after a reassignment.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490).  Methodologie section 1: T2 holds low-importance tokens at
// reduced precision (8-bit quantisation); section 4: tiers change every Delta
// steps and only the tokens whose tier changed move.  T2 is left only for T3
// (its full precision is gone), and it receives the rows a reassignment has
// just quantised.
//
// Storage: per (sequence, layer, KV head) `cap2` slots of D int8 codes in the
// K-tile / V-tile element order of the bf16 pools (layout.h, one byte per
// element), and one float32 scale per (slot, layer, KV head) for keys and one
// for values.  A slot -> position map says which position each slot holds.
//
// Update, in place (two launches):
//   t2_scan -- one 1024-thread workgroup per sequence.  Checks the state first
//       (every old slot maps to a position < n whose new tier is T2 or T3, the
//       new row count is in range, the new length fits cap2 and equals the
//       number of T2 positions of the new map); on failure it reports -1 and
//       changes nothing.  Then: holes = slots below the new length whose row
//       left or which were past the old length (slot order); movers = rows that
//       stay but sit at or past the new length (slot order), then the new rows
//       (their list order).  The i-th mover fills the i-th hole; the map is
//       rewritten for the holes only.
//   t2_move -- one wave per (move, layer x KV head, K or V): the codes and the
//       scale of one row.  Sources are slots at or past the new length or new
//       rows, destinations lie below it, so no move reads a slot another move
//       writes.
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace tkv {

constexpr int kT2ScanThreads = 1024;

__global__ __launch_bounds__(kT2ScanThreads) void t2_scan_kernel(T2ScanArgs a) {
  __shared__ int tmp[kT2ScanThreads / kWave + 1];
  __shared__ int s_bad;
  const int bl = blockIdx.x;
  const long b = a.b_offset + bl;
  const int tid = threadIdx.x;
  const int n = a.n[bl];
  const int len2 = a.len2[bl];
  int* pos = a.t2_pos + b * a.cap2;
  const uint8_t* tn = a.tnext + b * a.max_ctx;
  if (tid == 0) s_bad = 0;
  __syncthreads();

  // 1. checks, and the rows that stay
  int kept = 0, bad = 0;
  for (int j = tid; j < len2; j += kT2ScanThreads) {
    const int p = pos[j];
    if ((unsigned)p >= (unsigned)n) {
      bad = 1;
      continue;
    }
    const int t = tn[p];
    if (t == 2) ++kept;
    else if (t != 3) bad = 1;
  }
  int in_map = 0;  // T2 positions of the new map
  for (int i = tid; i < n; i += kT2ScanThreads) in_map += tn[i] == 2;
  if (bad) s_bad = 1;
  kept = block_sum_i(kept, tmp);
  in_map = block_sum_i(in_map, tmp);
  const int nn = a.n_new[b * a.n_new_stride];
  const int new_len = kept + nn;
  if (s_bad || nn < 0 || nn > a.max_rows || new_len > a.cap2 || new_len != in_map) {
    if (tid == 0) {
      a.cnt[b] = 0;
      a.out_len[b * 2] = -1;
      a.out_len[b * 2 + 1] = -1;
    }
    return;
  }
  int* holes = a.holes + b * a.cap2;
  int2* list = a.list + b * a.cap2;

  // 2. holes below the new length, in slot order
  int nh = 0;
  for (int j0 = 0; j0 < new_len; j0 += kT2ScanThreads) {
    const int j = j0 + tid;
    int f = 0;
    if (j < new_len) f = j >= len2 || tn[pos[j]] != 2;
    int tot;
    const int at = block_excl_scan(f, tmp, &tot);
    if (f) holes[nh + at] = j;
    nh += tot;
  }
  __syncthreads();  // the hole list is read by other threads below

  // 3. rows that stay but sit at or past the new length (slot order), then
  //    the new rows; the map is read at j >= new_len and written below it
  int nm = 0;
  for (int j0 = new_len; j0 < len2; j0 += kT2ScanThreads) {
    const int j = j0 + tid;
    int f = 0, p = 0;
    if (j < len2) {
      p = pos[j];
      f = tn[p] == 2;
    }
    int tot;
    const int at = block_excl_scan(f, tmp, &tot);
    if (f) {
      const int d = holes[nm + at];
      list[nm + at] = make_int2(j, d);
      pos[d] = p;
    }
    nm += tot;
  }
  const int* np = a.new_pos + b * a.max_rows;
  for (int r = tid; r < nn; r += kT2ScanThreads) {
    const int d = holes[nm + r];
    list[nm + r] = make_int2(-r - 1, d);
    pos[d] = np[r];
  }
  if (tid == 0) {
    a.cnt[b] = nm + nn;  // == nh
    a.out_len[b * 2] = new_len;
    a.out_len[b * 2 + 1] = nm + nn;
  }
}

template <int D>
__global__ __launch_bounds__(256) void t2_move_kernel(T2MoveArgs a) {
  constexpr int PER = D / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const long wave = (long)blockIdx.x * 4 + threadIdx.x / kWave;
  const long nwaves = (long)gridDim.x * 4;
  const long per_move = (long)a.lgs * 2;
  for (int bl = 0; bl < a.nb; ++bl) {
    const long b = a.b_offset + bl;
    const long items = (long)a.cnt[b] * per_move;
    for (long it = wave; it < items; it += nwaves) {
      const long mi = it / per_move;
      const int rest = (int)(it - mi * per_move);
      const int lg = rest >> 1, kv = rest & 1;
      const int2 mv = a.list[b * a.cap2 + mi];
      const long row = b * a.lgs + lg;  // (sequence, layer x KV head)
      int8_t* pool = (kv ? a.v2 : a.k2) + row * a.cap2 * D;
      float* sc = (kv ? a.vs2 : a.ks2) + row * a.cap2;
      int8_t x[PER];
      float s;
      if (mv.x >= 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int d = lane + kWave * i;
          x[i] = pool[kv ? v_off(mv.x, d, D) : k_off(mv.x, d, D)];
        }
        s = sc[mv.x];
      } else {
        const long r = -mv.x - 1;
        const long src = ((b * a.max_rows + r) * a.lgs + lg) * 2 + kv;
#pragma unroll
        for (int i = 0; i < PER; ++i) x[i] = a.new_codes[src * D + lane + kWave * i];
        s = a.new_scales[src];
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int d = lane + kWave * i;
        pool[kv ? v_off(mv.y, d, D) : k_off(mv.y, d, D)] = x[i];
      }
      if (lane == 0) sc[mv.y] = s;
    }
  }
}

void launch_t2_scan(const T2ScanArgs& a, int nb, hipStream_t s) {
  KernelTimer timer("t2_scan", s);
  hipExtLaunchKernelGGL(t2_scan_kernel, dim3(nb), dim3(kT2ScanThreads), 0, s, timer.start(),
                        timer.stop(), 0, a);
}

void launch_t2_move(const T2MoveArgs& a, int head_dim, hipStream_t s) {
  KernelTimer timer("t2_move", s);
  const dim3 grid(1024), block(256);
  if (head_dim == 128)
    hipExtLaunchKernelGGL((t2_move_kernel<128>), grid, block, 0, s, timer.start(), timer.stop(),
                          0, a);
  else
    hipExtLaunchKernelGGL((t2_move_kernel<64>), grid, block, 0, s, timer.start(), timer.stop(),
                          0, a);
}

}  // namespace tkv
