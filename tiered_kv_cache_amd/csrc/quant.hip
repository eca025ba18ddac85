// 8-bit rows of the tokens that enter T2.
//
// Method: "Not All Thoughts Need HBM" summary pages (gist.science, paper
// 2605.09490), Methodologie section 1: T2 keeps low-importance tokens on the
// host at reduced precision, 8-bit quantisation being the example.  Format
// (symmetric, one float32 scale per row of head_dim values): scale =
// absmax / 127, code = round-half-even(x / scale) clamped to [-127, 127], both
// divisions IEEE float32 (the library is built with correctly rounded float32
// division); an all-zero row has scale 0 and codes 0.
//
// One wave per (row, layer, KV head, K or V): coalesced load of the row, a
// wave max-reduction for absmax, one division per element.
#include "common.h"
#include "kernels.h"
#include "layout.h"

namespace tkv {

template <typename T, int D>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  constexpr int PER = D / kWave;  // elements per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int combo = blockIdx.x * 4 + threadIdx.x / kWave;  // (layer, KV head, K|V)
  const int lgs = a.L * a.hkv;
  if (combo >= lgs * 2) return;
  const int r = blockIdx.y;
  const long b = a.b_offset + blockIdx.z;
  const int nr = a.n_rows[b * a.n_rows_stride];
  if (r >= nr || r >= a.max_rows) return;
  const int kv = combo & 1;
  const long lg = combo >> 1;
  const int s = a.src[b * a.max_rows + r];
  if ((a.only == 1 && s < 0) || (a.only == 2 && s >= 0)) return;
  float v[PER];
  float am = 0.f;
  if (s < 0 && a.staging) {  // a plain staging row: D keys, then D values
    const T* row = (const T*)a.staging + (((b * a.cap1 + (-s - 1)) * lgs + lg) * 2 + kv) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      v[i] = to_f32(row[lane * PER + i]);
      am = fmaxf(am, fabsf(v[i]));
    }
  } else {
    const long slot = s >= 0 ? s : -s - 1;
    const int bl = blockIdx.z;
    const T* blk = (const T*)(kv ? (s >= 0 ? a.v0 : a.v1) : (s >= 0 ? a.k0 : a.k1)) +
                   (s >= 0 ? pool_row(a.pool.blk0, a.pool.cap0, bl, lg, D)
                           : pool_row(a.pool.blk1, a.pool.cap1, bl, lg, D));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int d = lane * PER + i;
      const long off = kv ? v_off(slot, d, D) : k_off(slot, d, D);  // tile storage order
      v[i] = to_f32(blk[off]);
      am = fmaxf(am, fabsf(v[i]));
    }
  }
  am = wave_max(am);
  const float scale = am / 127.0f;
  const long orow = ((b * a.max_rows + r) * lgs + lg) * 2 + kv;
  int8_t* out = a.codes + orow * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    float c = 0.f;
    if (scale > 0.f) c = fminf(fmaxf(rintf(v[i] / scale), -127.f), 127.f);
    out[lane * PER + i] = (int8_t)(int)c;
  }
  if (lane == 0) a.scales[orow] = scale;
}

void launch_quantize(const QuantArgs& a, int kv_dtype, int head_dim, int nb, hipStream_t s) {
  KernelTimer timer("quantize_t2", s);
  dim3 grid(ceil_div(a.L * a.hkv * 2, 4), a.max_rows, nb);
  if (kv_dtype == TKV_BF16) {
    if (head_dim == 128) hipExtLaunchKernelGGL((quantize_kernel<uint16_t, 128>), grid, dim3(256), 0, s,
                                               timer.start(), timer.stop(), 0, a);
    else hipExtLaunchKernelGGL((quantize_kernel<uint16_t, 64>), grid, dim3(256), 0, s,
                               timer.start(), timer.stop(), 0, a);
  } else {
    if (head_dim == 128) hipExtLaunchKernelGGL((quantize_kernel<float, 128>), grid, dim3(256), 0, s,
                                               timer.start(), timer.stop(), 0, a);
    else hipExtLaunchKernelGGL((quantize_kernel<float, 64>), grid, dim3(256), 0, s,
                               timer.start(), timer.stop(), 0, a);
  }
}

}  // namespace tkv
