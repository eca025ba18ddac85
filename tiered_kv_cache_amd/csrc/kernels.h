// Kernel argument blocks and launchers of libtkv (internal).
#pragma once

#include "attn_args.h"
#include "common.h"

namespace tkv {

constexpr int kScoreSlots = 64;      // attended slots per score workgroup

// Score accumulation: s[pos(j)] += weight * sum over r of src[r][j], for the
// attended slots j of every sequence (row r of sequence bl at
// src + bl * seq_stride + r * row_stride).
struct ScoreArgs {
  const float* src;
  long row_stride, seq_stride;
  int rows;
  const int* t0_pos;
  const int* t1_pos;
  const int* t2_pos;  // attended T2 slots (after T1), or null
  float* scores;
  int cap0, cap1, cap2, max_ctx;
  double weight;  // 1 / (num_layers * Hq)
  SeqTable seq;   // base[] counts kScoreSlots-slot blocks
};

// Merge of the split records (output O), alpha normalisation, group sums.
struct MergeArgs {
  const float* part;
  const float* ml;
  float* out;
  float* alpha;
  int alpha_out;  // 0: alpha holds the logits only, the normalised weights are not stored
  float* gsum;  // [nb][gs_seq_rows][gs_stride] sums of alpha over a group's heads, or null
  long alpha_stride, gs_stride;
  long gs_seq_rows;           // gsum rows per sequence (Lr * Hkv, or L * Hkv for a whole step)
  int gs_row0;                // gsum row of the launch's first (layer, KV head)
  long total_units, workers;  // as in the attention launch
  int Lr, hq, hkv;
  int io_L, io_l0;            // out / alpha rows: layers they hold per sequence, the call's first
  int out_rows, out_blocks;   // O rows of the launch; workgroups merging them (first)
  SeqTable seq;               // base[] / units[] as in the attention launch
  int cbase[kMaxSeqPerLaunch + 1];  // alpha workgroups: prefix over sequences
};

struct AppendArgs {
  const void* kn;
  const void* vn;
  void* k0;
  void* v0;
  int* t0_pos;
  float* scores;
  uint8_t* tier;
  int cap0, max_ctx, L, hkv, b_offset;
  int slot[kMaxSeqPerLaunch];
  int pos[kMaxSeqPerLaunch];
  PoolTable pool;  // T0 rows of the launch's sequences
};

struct TierArgs {
  const float* scores;
  const uint8_t* tprev;
  uint8_t* tnext;
  int* counts;
  int max_ctx, prot_lo, recent, b_offset;
  int n[kMaxSeqPerLaunch];
  int n1[kMaxSeqPerLaunch];
  int n2[kMaxSeqPerLaunch];
  int n3[kMaxSeqPerLaunch];
};

// Relocation after a reassignment, in place.  Per sequence the workspace holds
// an inverse map (position -> slot code), the low holes of the T0 pool and of
// the T1 window, three move lists of (source, destination) pairs and their
// counts.  Slot codes: s >= 0 is T0 slot s, s < 0 is T1 slot -s-1; in the
// T0-destination list a negative source is staging row -s-1.
struct RelocArgs {
  const uint8_t* tprev;
  const uint8_t* tnext;
  int* t0_pos;   // in/out [B][cap0]
  int* t1_pos;   // in/out [B][cap1]
  int* inv;      // [B][max_ctx]
  int* holes0;   // [B][cap0]
  int* holes1;   // [B][cap1]
  int2* to_t0;   // [B][cap0]  (T0 slot or staging row, T0 slot)
  int2* to_t1;   // [B][cap1]  (T0 or T1 slot code, T1 slot)
  int2* staged;  // [B][cap1]  (T1 slot code, staging row): promotions
  int* cnt;      // [B][4]  |to_t0|, |to_t1|, |staged|, 0
  int* t2_src;
  int* t2_pos;
  int* new_lens;
  int max_ctx, cap0, cap1, t2_cap, b_offset;
  // T1 rows live in host memory: new T2 rows that leave T1 are listed by a
  // staging row after the promoted rows (t2_src = -(row) - 1) instead of by
  // their T1 slot; the T1 side of the moves is the host's
  int host_t1;
  int n[kMaxSeqPerLaunch];
  int len0[kMaxSeqPerLaunch];
  int len1[kMaxSeqPerLaunch];
  int lim0[kMaxSeqPerLaunch];  // the sequence's T0 pool capacity (<= cap0)
  int lim1[kMaxSeqPerLaunch];  // its T1 window capacity (<= cap1)
};

// kMoveDown (T1 rows in host memory): the rows of the T1-destination list that
// come from the T0 pool go to staging row = their list index.
enum MoveList { kMoveStage = 0, kMoveToT1 = 1, kMoveToT0 = 2, kMoveDown = 3 };

struct MoveArgs {
  void* k0;
  void* v0;
  void* k1;
  void* v1;
  void* staging;      // [B][cap1][L * Hkv][2][D] elements, plain rows (K then V)
  const int2* list;   // [B][list_stride]
  const int* cnt;     // [B][4]
  int list_stride, which, cap0, cap1, lgs, b_offset, nb;
  PoolTable pool;     // T0 pool and T1 window rows of the launch's sequences
};

struct QuantArgs {
  const void* k0;
  const void* v0;
  const void* k1;
  const void* v1;
  // with staging set, a source s < 0 is staging row -s-1 ([B][cap1][L * Hkv][2][D]
  // plain rows) rather than T1 slot -s-1; `only` = 1 takes only the T0 sources,
  // 2 only the negative ones, 0 every row
  const void* staging;
  int only;
  const int* src;
  const int* n_rows;
  int8_t* codes;
  float* scales;
  int n_rows_stride, max_rows, cap0, cap1, L, hkv, b_offset;
  PoolTable pool;  // T0 pool and T1 window rows of the launch's sequences
};

// In-place update of the attended T2 pool after a reassignment: rows whose
// position left T2 (for T3) free their slots; rows left at or past the new
// length and the newly quantised rows fill the holes below it.  Move list
// entries are (source, destination slot): source >= 0 an old pool slot,
// source < 0 new row -source-1.
struct T2ScanArgs {
  const uint8_t* tnext;     // [B][max_ctx]
  int* t2_pos;              // in/out [B][cap2]
  const int* new_pos;       // [B][max_rows] positions of the new rows
  const int* n_new;         // element b * n_new_stride: new row count of sequence b
  int* holes;               // [B][cap2]
  int2* list;               // [B][cap2]
  int* cnt;                 // [B]
  int* out_len;             // [B][2]: new length, moves (or -1, -1)
  int max_ctx, cap2, max_rows, n_new_stride, b_offset;
  int n[kMaxSeqPerLaunch];
  int len2[kMaxSeqPerLaunch];
};

struct T2MoveArgs {
  int8_t* k2;
  int8_t* v2;
  float* ks2;
  float* vs2;
  const int8_t* new_codes;  // [B][max_rows][L * Hkv][2][D]
  const float* new_scales;  // [B][max_rows][L * Hkv][2]
  const int2* list;
  const int* cnt;
  int cap2, max_rows, lgs, b_offset, nb;
};

// Host-side T1 packers (gather.cpp): every slot [0, n) of a window of one
// sequence from its positions, or only the listed (slot, position) pairs.  The
// store is [L][Hkv][max_ctx][D] rows by position; the staging [L][Hkv][2][cap1][D]
// tiles (each row's key slots, then its value slots).
void pack_t1_blocks(const tkv_model* m, const void* store_k, const void* store_v, int max_ctx,
                    const int32_t* positions, int n, void* staging, int cap1);
void pack_t1_slots(const tkv_model* m, const void* store_k, const void* store_v, int max_ctx,
                   const int32_t* slots, const int32_t* positions, int n, void* staging,
                   int cap1);

int merge_alpha_blocks(int natt);    // alpha workgroups per (layer, KV head) group
int merge_output_blocks(int rows);   // workgroups merging `rows` output rows
void launch_attn_merge(const MergeArgs& a, int head_dim, int nblocks, hipStream_t s);
void launch_score_rows(const ScoreArgs& a, int nblocks, const char* name, hipStream_t s);
void launch_append(const AppendArgs& a, int kv_dtype, int head_dim, int nb, hipStream_t s);
void launch_assign_tiers(const TierArgs& a, int nb, hipStream_t s);
void launch_reloc_scan(const RelocArgs& a, int nb, hipStream_t s);
void launch_reloc_move(const MoveArgs& m, int kv_dtype, int head_dim, hipStream_t s);
void launch_quantize(const QuantArgs& a, int kv_dtype, int head_dim, int nb, hipStream_t s);
void launch_t2_scan(const T2ScanArgs& a, int nb, hipStream_t s);
void launch_t2_move(const T2MoveArgs& a, int head_dim, hipStream_t s);

}  // namespace tkv
