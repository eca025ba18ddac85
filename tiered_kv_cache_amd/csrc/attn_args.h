// Argument block of the decode-attention launch and the layouts it shares with
// the merge (internal).  Kept apart from the other kernels' arguments: the
// attention kernel compiles from this header, layout.h, common.h and
// attention.hip only.
#pragma once

#include "common.h"

namespace tkv {

constexpr int kUnitMfma = 32;        // tokens per work unit, bf16 matrix-core path (a pair of 16-token tiles)
constexpr int kUnitValu = 256;       // tokens per work unit, float32 path (one token per thread)
constexpr int kMaxWorkers = 8192;    // bound on attention workers (split records <= workers + groups)

// Per-launch sequence table: lengths and the prefix of work blocks per sequence.
struct SeqTable {
  int nb;        // sequences in this launch
  int b_offset;  // index of the first one in the caller's batch
  int t0_len[kMaxSeqPerLaunch];
  int t1_len[kMaxSeqPerLaunch];
  int t2_len[kMaxSeqPerLaunch];    // attended 8-bit T2 rows (0 unless a T2 pool is given)
  int base[kMaxSeqPerLaunch + 1];  // first work unit (attention) or slot block (scores)
  int units[kMaxSeqPerLaunch];     // attention: work units per (layer, KV head) group
};

// Where the T0 pool and T1 window blocks of the sequences of one launch start, in
// 32-slot blocks of 32 * D elements from the start of the pool, and how many slots
// each (layer, KV head) row of a sequence holds.  Uniform pools: blk = b * L * Hkv *
// cap / 32 and cap the same for every sequence; per-sequence capacities pack the
// sequences' blocks one after the other.
struct PoolTable {
  int blk0[kMaxSeqPerLaunch];
  int cap0[kMaxSeqPerLaunch];
  int blk1[kMaxSeqPerLaunch];
  int cap1[kMaxSeqPerLaunch];
};

// Element offset of slot 0 of pool row lg (= layer * Hkv + KV head) of sequence bl.
__host__ __device__ inline long pool_row(const int* blk, const int* cap, int bl, long lg, int D) {
  return ((long)blk[bl] * 32 + lg * (long)cap[bl]) * D;
}

// Split records of the partial P.V: per record (worker + group) the G heads'
// D values, stored in the order the matrix-core kernel holds them, so that its
// stores are whole 64-byte (G <= 4), 128-byte (G <= 8) or 256-byte rows:
// [head % 4][D / 16][ceil(G / 4)][16], head h at (h % 4, h / 4), dim d at
// (d / 16, d % 16).  Heads past G (padding up to 4 * ceil(G / 4)) are written
// but never read.
__host__ __device__ inline long part_rec_floats(int G, int D) { return 4L * D * ((G + 3) / 4); }
__host__ __device__ inline long part_off(int G, int D, int head, int d) {
  const int GR = (G + 3) / 4;
  return ((long)((head & 3) * (D / 16) + (d >> 4)) * GR + (head >> 2)) * 16 + (d & 15);
}

struct AttnArgs {
  const void* q;
  const void* k0;
  const void* v0;
  const void* k1;
  const void* v1;
  // attended T2 pool (null when no sequence has T2 rows): int8 codes in the
  // K-tile / V-tile order of the pools, one float32 scale per row
  const int8_t* k2;
  const int8_t* v2;
  const float* ks2;  // [B][L][Hkv][cap2]
  const float* vs2;  // [B][L][Hkv][cap2]
  float* out;
  float* alpha;   // raw scaled logits on exit of attn_partial
  float* part;    // split records: [worker + group][part_rec_floats] partial P.V
  float* ml;      // split records: [worker + group][head in group][2] (m, l)
  long alpha_stride;
  long total_units;  // work units of this launch
  long workers;      // workers sharing them (record index = worker + group)
  int unit;          // tokens per work unit
  int cap0, cap1, cap2;
  int L, Lr, layer_begin, hq, hkv;
  int t1_L, t1_l0;   // T1 window: layers it holds per sequence, index of the call's first
  long t1_rs;        // T1 window: elements between consecutive (sequence, layer, KV head) rows
  int io_L, io_l0;   // q / out / alpha rows: layers they hold per sequence, the call's first
  float scale;       // softmax_scale * log2(e): logits are kept in base 2
  int stage_nt;      // logit stages that fill before a wave's last load go out non-temporal
  SeqTable seq;
  PoolTable pool;    // the T0 pool and (unless a window call) the T1 pool rows
  // append fused into the bf16 kernel (kn null: none).  The new row of sequence i
  // sits at T0 slot app_slot[i] (< seq.t0_len[i]); the kernel reads it from kn/vn
  // ([B][L][Hkv][D]), writes it into the pool, and records its position.
  const void* kn;
  const void* vn;
  int* app_t0_pos;
  float* app_scores;
  uint8_t* app_tier;
  int app_max_ctx;
  int app_slot[kMaxSeqPerLaunch];
  int app_pos[kMaxSeqPerLaunch];
};

bool attn_group_supported(int group);
int mfma_resident_waves(int head_dim);
void launch_attn_partial(const AttnArgs& a, int kv_dtype, int head_dim, int group, hipStream_t s);

}  // namespace tkv
