// C ABI of libtkv: argument validation, batch splitting, kernel dispatch.
// Every check runs before the first HIP call of an entry point.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace tkv {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

tkv_status fail(tkv_status code, const std::string& msg) {
  set_error(msg);
  return code;
}

tkv_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return TKV_OK;
  return fail(TKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// kernel timers (benchmark aid)
// ---------------------------------------------------------------------------
namespace {
struct TimerRec {
  std::string name;
  hipEvent_t start, stop;
};
struct TimerState {
  bool enabled = false;
  std::set<std::string> only;  // empty: every kernel
  std::vector<TimerRec> pending;
  std::vector<hipEvent_t> free_events;
  std::map<std::string, std::pair<double, long long>> totals;
};
TimerState& timers() {
  static TimerState t;
  return t;
}
hipEvent_t take_event() {
  auto& t = timers();
  if (!t.free_events.empty()) {
    hipEvent_t e = t.free_events.back();
    t.free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
void drain_timers() {
  auto& t = timers();
  for (auto& r : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      auto& tot = t.totals[r.name];
      tot.first += ms;
      tot.second += 1;
    }
    t.free_events.push_back(r.start);
    t.free_events.push_back(r.stop);
  }
  t.pending.clear();
}
}  // namespace

KernelTimer::KernelTimer(const char* name, hipStream_t)
    : name_(name), start_(nullptr), stop_(nullptr) {
  if (!timers().enabled) return;
  if (!timers().only.empty() && !timers().only.count(name)) return;
  start_ = take_event();
  stop_ = take_event();
  if (!start_ || !stop_) {
    if (start_) timers().free_events.push_back(start_);
    if (stop_) timers().free_events.push_back(stop_);
    start_ = stop_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  timers().pending.push_back({name_, start_, stop_});
  if (timers().pending.size() > 4096) drain_timers();
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
static tkv_status check_model(const tkv_model* m) {
  if (!m) return fail(TKV_ERR_ARG, "model is null");
  if (m->num_layers < 1 || m->num_q_heads < 1 || m->num_kv_heads < 1)
    return fail(TKV_ERR_ARG, "layers and heads must be positive");
  if (m->num_q_heads % m->num_kv_heads != 0)
    return fail(TKV_ERR_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (!attn_group_supported(m->num_q_heads / m->num_kv_heads))
    return fail(TKV_ERR_ARG, "query heads per KV head must be 1..8 or 16");
  if (m->head_dim != 64 && m->head_dim != 128) return fail(TKV_ERR_ARG, "head_dim must be 64 or 128");
  if (m->kv_dtype != TKV_BF16 && m->kv_dtype != TKV_F32) return fail(TKV_ERR_ARG, "bad kv_dtype");
  if (!(m->softmax_scale == m->softmax_scale) || isinf(m->softmax_scale))
    return fail(TKV_ERR_ARG, "softmax_scale must be finite");
  if (m->alpha_scratch != 0 && m->alpha_scratch != 1) return fail(TKV_ERR_ARG, "alpha_scratch must be 0 or 1");
  return TKV_OK;
}

// Per-sequence pool capacities (tkv_model.t0_caps / t1_caps, or the call's cap for
// every sequence).
static int cap0_of(const tkv_model* m, int b, int cap0) { return m->t0_caps ? m->t0_caps[b] : cap0; }
static int cap1_of(const tkv_model* m, int b, int cap1) { return m->t1_caps ? m->t1_caps[b] : cap1; }

// The per-sequence capacities of a call over `batch` sequences: multiples of 32, at
// most the call's cap0 / cap1, and pools of fewer than 2^31 32-slot blocks (t1: the
// call addresses a device T1 pool through t1_caps).
static tkv_status check_caps(const tkv_model* m, int batch, int cap0, int cap1, bool t1) {
  const long per = (long)m->num_layers * m->num_kv_heads;
  long blk0 = 0, blk1 = 0;
  for (int b = 0; b < batch; ++b) {
    const int c0 = cap0_of(m, b, cap0), c1 = t1 ? cap1_of(m, b, cap1) : 0;
    if (c0 < 0 || c0 % 32 || c0 > cap0 || c1 < 0 || c1 % 32 || c1 > cap1)
      return fail(TKV_ERR_ARG, "per-sequence capacities must be multiples of 32 within cap0 / cap1");
    blk0 += per * (c0 / 32);
    blk1 += per * (c1 / 32);
  }
  if (blk0 >= (1L << 31) || blk1 >= (1L << 31))
    return fail(TKV_ERR_CAPACITY, "a pool of 2^31 or more 32-slot blocks");
  return TKV_OK;
}

// Pool table of sequences [b0, b0 + nb): their capacities and the first block of
// each (the blocks of the sequences before b0 come first).
static void fill_pool(PoolTable& t, const tkv_model* m, int b0, int nb, int cap0, int cap1) {
  const long per = (long)m->num_layers * m->num_kv_heads;
  long s0 = 0, s1 = 0;
  if (m->t0_caps || m->t1_caps) {
    for (int b = 0; b < b0; ++b) {
      s0 += per * (cap0_of(m, b, cap0) / 32);
      s1 += per * (cap1_of(m, b, cap1) / 32);
    }
  } else {
    s0 = per * (long)b0 * (cap0 / 32);
    s1 = per * (long)b0 * (cap1 / 32);
  }
  for (int i = 0; i < nb; ++i) {
    const int c0 = cap0_of(m, b0 + i, cap0), c1 = cap1_of(m, b0 + i, cap1);
    t.blk0[i] = (int)s0;
    t.cap0[i] = c0;
    t.blk1[i] = (int)s1;
    t.cap1[i] = c1;
    s0 += per * (c0 / 32);
    s1 += per * (c1 / 32);
  }
}

static float scale_of(const tkv_model* m) {
  return m->softmax_scale > 0.f ? m->softmax_scale : 1.0f / sqrtf((float)m->head_dim);
}

// Split records of one launch: at most workers + groups (see attention.hip).
static size_t max_records(int batch, int n_layers, int hkv) {
  const int nb = batch < kMaxSeqPerLaunch ? batch : kMaxSeqPerLaunch;
  return (size_t)kMaxWorkers + (size_t)nb * n_layers * hkv;
}

static size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

// Decode workspace, in floats, every region 256-byte aligned:
//   part [records][G][D] | ml [records][G][2] | gsum [nb][Lr * Hkv][gs_stride]
struct DecodeWorkspace {
  size_t part, ml, gsum, total, gs_stride;
};

static DecodeWorkspace decode_workspace(const tkv_model* m, int batch, int n_layers, int cap0,
                                        int cap1) {
  const size_t G = (size_t)(m->num_q_heads / m->num_kv_heads);
  const size_t D = (size_t)m->head_dim;
  const size_t recs = max_records(batch, n_layers, m->num_kv_heads);
  const size_t nb = (size_t)(batch < kMaxSeqPerLaunch ? batch : kMaxSeqPerLaunch);
  DecodeWorkspace w;
  w.gs_stride = round_up((size_t)cap0 + (size_t)cap1, 4);
  w.part = 0;
  w.ml = round_up(w.part + recs * (size_t)part_rec_floats((int)G, (int)D), 64);
  w.gsum = round_up(w.ml + recs * G * 2, 64);
  w.total = round_up(w.gsum + nb * n_layers * m->num_kv_heads * w.gs_stride, 64);
  return w;
}

}  // namespace tkv

using namespace tkv;

extern "C" {

int32_t tkv_abi_version(void) { return TKV_ABI_VERSION; }

const char* tkv_last_error(void) { return g_last_error.c_str(); }

tkv_status tkv_timing_enable(int32_t enable) {
  timers().enabled = enable != 0;
  return TKV_OK;
}

tkv_status tkv_timing_select(const char* kernels) {
  auto& only = timers().only;
  only.clear();
  if (!kernels) return TKV_OK;
  std::string cur;
  for (const char* c = kernels;; ++c) {
    if (*c == ',' || *c == '\0') {
      if (!cur.empty()) only.insert(cur);
      cur.clear();
      if (*c == '\0') break;
    } else if (*c != ' ') {
      cur += *c;
    }
  }
  return TKV_OK;
}

tkv_status tkv_timing_reset(void) {
  drain_timers();
  timers().totals.clear();
  return TKV_OK;
}

tkv_status tkv_timing_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return fail(TKV_ERR_ARG, "null argument");
  drain_timers();
  auto it = timers().totals.find(kernel);
  *total_ms = it == timers().totals.end() ? 0.0 : it->second.first;
  *launches = it == timers().totals.end() ? 0 : it->second.second;
  return TKV_OK;
}

// ---------------------------------------------------------------------------
tkv_status tkv_append(const tkv_model* model, int32_t batch, const void* k_new, const void* v_new,
                      void* k_t0, void* v_t0, int32_t cap0, const int32_t* t0_len,
                      int32_t* t0_pos, const int32_t* position, float* scores, uint8_t* tier,
                      int32_t max_ctx, hipStream_t stream) {
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0) return fail(TKV_ERR_ARG, "batch < 0");
  if (batch == 0) return TKV_OK;
  if (!k_new || !v_new || !k_t0 || !v_t0 || !t0_len || !t0_pos || !position)
    return fail(TKV_ERR_ARG, "null pointer");
  if (cap0 < 1 || cap0 % 32) return fail(TKV_ERR_ARG, "cap0 must be a positive multiple of 32");
  if ((st = check_caps(model, batch, cap0, 0, false))) return st;
  for (int b = 0; b < batch; ++b) {
    if (t0_len[b] < 0 || position[b] < 0) return fail(TKV_ERR_ARG, "negative length or position");
    if (t0_len[b] >= cap0_of(model, b, cap0))
      return fail(TKV_ERR_CAPACITY, "T0 pool full (t0_len >= its capacity)");
    if ((scores || tier) && position[b] >= max_ctx)
      return fail(TKV_ERR_CAPACITY, "position >= max_ctx");
  }
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    AppendArgs a{};
    a.kn = k_new;
    a.vn = v_new;
    a.k0 = k_t0;
    a.v0 = v_t0;
    a.t0_pos = t0_pos;
    a.scores = scores;
    a.tier = tier;
    a.cap0 = cap0;
    a.max_ctx = max_ctx;
    a.L = model->num_layers;
    a.hkv = model->num_kv_heads;
    a.b_offset = b0;
    for (int i = 0; i < nb; ++i) {
      a.slot[i] = t0_len[b0 + i];
      a.pos[i] = position[b0 + i];
    }
    fill_pool(a.pool, model, b0, nb, cap0, 0);
    launch_append(a, model->kv_dtype, model->head_dim, nb, stream);
    if ((st = hip_check(hipGetLastError(), "append launch"))) return st;
  }
  return TKV_OK;
}

size_t tkv_decode_workspace_bytes(const tkv_model* model, int32_t batch, int32_t n_layers,
                                  int32_t cap0, int32_t cap1) {
  if (!model || batch < 0 || n_layers < 0 || cap0 < 0 || cap1 < 0) return 0;
  if (model->num_kv_heads < 1 || model->num_q_heads < 1) return 0;
  const DecodeWorkspace w = decode_workspace(model, batch, n_layers, cap0, cap1);
  return w.total * sizeof(float);
}

}  // extern "C"

namespace tkv {

// The token each sequence appends in this call (tkv_append_decode_step).
struct AppendInfo {
  const void* k_new;
  const void* v_new;
  const int32_t* position;  // host [B]
  int32_t* t0_pos;
  uint8_t* tier;
};

// The per-slot group sums of a call that covers only some layers of a step,
// written into a region that covers every layer; the score launch is left to the
// caller, which adds the whole step's increment once (tkv_decode_step_streamed).
struct DeferredScore {
  float* gsum;      // [nb][L * Hkv][gs_stride]
  int row0;         // first (layer, KV head) row of the call
};

// tkv_decode_step; with `app`, t0_len are the lengths before the append and the
// attention kernel performs the append (bf16; the float32 path appends first);
// with `t2`, the 8-bit T2 rows are attended after T1.
static tkv_status decode_step(const tkv_model* model, int32_t batch, int32_t layer_begin,
                              int32_t layer_end, const void* q, const void* k_t0,
                              const void* v_t0, const int32_t* t0_len, int32_t cap0,
                              const void* k_t1, const void* v_t1, const int32_t* t1_len,
                              int32_t cap1, float* out, float* alpha, int32_t alpha_stride,
                              const int32_t* t0_pos, const int32_t* t1_pos, float* scores,
                              int32_t max_ctx, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, const AppendInfo* app,
                              const tkv_t2_pool* t2, bool t1_window = false,
                              bool validate_only = false, long t1_rs = 0,
                              const DeferredScore* deferred = nullptr) {
  // t1_window: the T1 window holds only the call's layers, and q / out / alpha hold
  // every layer (the call reads and writes the rows of its own layers); t1_rs: the
  // elements between consecutive rows of the window (0: cap1 * head_dim)
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0) return fail(TKV_ERR_ARG, "batch < 0");
  if (layer_begin < 0 || layer_end > model->num_layers || layer_begin >= layer_end)
    return fail(TKV_ERR_ARG, "need 0 <= layer_begin < layer_end <= num_layers");
  if (batch == 0) return TKV_OK;
  if (!q || !k_t0 || !v_t0 || !t0_len || !t1_len || !out || !alpha || !workspace)
    return fail(TKV_ERR_ARG, "null pointer");
  if (cap0 < 0 || cap1 < 0 || alpha_stride < 1) return fail(TKV_ERR_ARG, "bad capacity or stride");
  if (cap0 % 32 || cap1 % 32) return fail(TKV_ERR_ARG, "cap0 and cap1 must be multiples of 32");
  const int cap2 = t2 ? t2->cap2 : 0;
  if (t2 && (!t2->t2_len || cap2 < 0 || cap2 % 32))
    return fail(TKV_ERR_ARG, "T2 pool: t2_len is null or cap2 is not a multiple of 32");
  bool any_t1 = false, any_t2 = false;
  const int grow = app ? 1 : 0;  // T0 rows added by the append
  if ((st = check_caps(model, batch, cap0, cap1, !t1_window))) return st;
  for (int b = 0; b < batch; ++b) {
    const int n2 = t2 ? t2->t2_len[b] : 0;
    if (t0_len[b] < 0 || t1_len[b] < 0 || n2 < 0) return fail(TKV_ERR_ARG, "negative length");
    if (t0_len[b] + grow > cap0_of(model, b, cap0) ||
        t1_len[b] > (t1_window ? cap1 : cap1_of(model, b, cap1)) || n2 > cap2)
      return fail(TKV_ERR_CAPACITY, "length > capacity");
    if ((long)t0_len[b] + grow + t1_len[b] + n2 > alpha_stride)
      return fail(TKV_ERR_CAPACITY, "alpha_stride < t0_len + t1_len + t2_len");
    any_t1 |= t1_len[b] > 0;
    any_t2 |= n2 > 0;
  }
  if (any_t2) {
    if (!t2->k_codes || !t2->v_codes || !t2->k_scale || !t2->v_scale)
      return fail(TKV_ERR_ARG, "T2 pool pointer is null but t2_len > 0");
    if (((uintptr_t)t2->k_codes | (uintptr_t)t2->v_codes | (uintptr_t)t2->k_scale |
         (uintptr_t)t2->v_scale) & 15)
      return fail(TKV_ERR_ARG, "T2 codes and scales must be 16-byte aligned");
    if (scores && !t2->t2_pos) return fail(TKV_ERR_ARG, "fused score update needs t2_pos");
  }
  if (app) {
    if (layer_begin != 0 || layer_end != model->num_layers)
      return fail(TKV_ERR_ARG, "the fused append needs all layers");
    if (!app->k_new || !app->v_new || !app->position || !app->t0_pos)
      return fail(TKV_ERR_ARG, "null pointer");
    for (int b = 0; b < batch; ++b) {
      if (app->position[b] < 0) return fail(TKV_ERR_ARG, "negative position");
      if ((scores || app->tier) && app->position[b] >= max_ctx)
        return fail(TKV_ERR_CAPACITY, "position >= max_ctx");
    }
  }
  if (any_t1 && (!k_t1 || !v_t1)) return fail(TKV_ERR_ARG, "T1 window is null but t1_len > 0");
  if (scores && (!t0_pos || (any_t1 && !t1_pos) || max_ctx < 1))
    return fail(TKV_ERR_ARG, "fused score update needs t0_pos, t1_pos and max_ctx");
  if (alpha_stride % 4 || ((uintptr_t)alpha & 15) || ((uintptr_t)workspace & 255))
    return fail(TKV_ERR_ARG,
                "alpha_stride must be a multiple of 4, alpha 16-byte and workspace 256-byte aligned");
  const int Lr = layer_end - layer_begin;
  // the group sums cover every attended slot: T2 slots follow T1 (a deferred score
  // keeps the group sums of every layer)
  if (workspace_bytes < tkv_decode_workspace_bytes(model, batch, deferred ? model->num_layers : Lr,
                                                   cap0, cap1 + cap2))
    return fail(TKV_ERR_CAPACITY, "workspace too small");
  if (validate_only) return TKV_OK;

  const int hq = model->num_q_heads;
  const int hkv = model->num_kv_heads;
  const int D = model->head_dim;
  const int G = hq / hkv;
  const bool mfma = model->kv_dtype == TKV_BF16;
  std::vector<int32_t> len_after;
  if (app) {
    len_after.assign(t0_len, t0_len + batch);
    for (auto& n : len_after) ++n;
    if (!mfma) {  // float32 path: the separate append kernel first
      if ((st = tkv_append(model, batch, app->k_new, app->v_new, const_cast<void*>(k_t0),
                           const_cast<void*>(v_t0), cap0, t0_len, app->t0_pos, app->position,
                           scores, app->tier, max_ctx, stream)))
        return st;
    }
  }
  const int32_t* att_len = app ? len_after.data() : t0_len;  // attended T0 rows
  const int unit = mfma ? kUnitMfma : kUnitValu;
  const DecodeWorkspace wl =
      decode_workspace(model, batch, deferred ? model->num_layers : Lr, cap0, cap1 + cap2);
  float* part = (float*)workspace + wl.part;
  float* ml = (float*)workspace + wl.ml;
  float* gsum = (float*)workspace + wl.gsum;
  int resident = 0;
  if (mfma) {
    resident = mfma_resident_waves(D);
    if (resident < 1) return fail(TKV_ERR_HIP, "cannot query the device for its occupancy");
    static const int override_workers = [] {  // tuning sweeps: TKV_ATTN_WORKERS
      const char* e = getenv("TKV_ATTN_WORKERS");
      return e ? atoi(e) : 0;
    }();
    if (override_workers > 0) resident = std::min(override_workers, kMaxWorkers);
  }

  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    AttnArgs a{};
    a.q = q;
    a.k0 = k_t0;
    a.v0 = v_t0;
    a.k1 = k_t1;
    a.v1 = v_t1;
    if (any_t2) {
      a.k2 = t2->k_codes;
      a.v2 = t2->v_codes;
      a.ks2 = t2->k_scale;
      a.vs2 = t2->v_scale;
    }
    a.out = out;
    a.alpha = alpha;
    a.part = part;
    a.ml = ml;
    a.alpha_stride = alpha_stride;
    a.unit = unit;
    a.cap0 = cap0;
    a.cap1 = cap1;
    a.cap2 = cap2;
    a.L = model->num_layers;
    a.Lr = Lr;
    a.layer_begin = layer_begin;
    a.hq = hq;
    a.hkv = hkv;
    a.t1_L = t1_window ? Lr : model->num_layers;
    a.t1_l0 = t1_window ? 0 : layer_begin;
    a.t1_rs = t1_rs > 0 ? t1_rs : (long)cap1 * D;
    a.io_L = t1_window ? model->num_layers : Lr;
    a.io_l0 = t1_window ? layer_begin : 0;
    // logits are kept in base 2: q.k * softmax_scale * log2(e)
    a.scale = (float)((double)scale_of(model) * 1.4426950408889634074);
    a.seq.nb = nb;
    a.seq.b_offset = b0;
    fill_pool(a.pool, model, b0, nb, cap0, cap1);
    MergeArgs m{};
    ScoreArgs sa{};
    long units = 0;
    int cblocks = 0, sblocks = 0;
    if (app && mfma) {
      a.kn = app->k_new;
      a.vn = app->v_new;
      a.app_t0_pos = app->t0_pos;
      a.app_scores = scores;
      a.app_tier = app->tier;
      a.app_max_ctx = max_ctx;
      for (int i = 0; i < nb; ++i) {
        a.app_slot[i] = t0_len[b0 + i];
        a.app_pos[i] = app->position[b0 + i];
      }
    }
    for (int i = 0; i < nb; ++i) {
      const int n0 = att_len[b0 + i], n1 = t1_len[b0 + i];
      const int n2 = t2 ? t2->t2_len[b0 + i] : 0;
      a.seq.t0_len[i] = n0;
      a.seq.t1_len[i] = n1;
      a.seq.t2_len[i] = n2;
      a.seq.base[i] = (int)units;
      a.seq.units[i] = ceil_div(n0, unit) + ceil_div(n1, unit) + ceil_div(n2, unit);
      units += (long)Lr * hkv * a.seq.units[i];
      m.cbase[i] = cblocks;
      cblocks += Lr * hkv * merge_alpha_blocks(n0 + n1 + n2);
      sa.seq.t0_len[i] = n0;
      sa.seq.t1_len[i] = n1;
      sa.seq.t2_len[i] = n2;
      sa.seq.base[i] = sblocks;
      sblocks += ceil_div(n0 + n1 + n2, kScoreSlots);
    }
    if (units > (1L << 30)) return fail(TKV_ERR_CAPACITY, "too many attention work units");
    a.seq.base[nb] = (int)units;
    a.total_units = units;
    // at least two units per wave: a small launch (one layer of a streamed step)
    // spread over every SIMD leaves each group split into hundreds of records,
    // which the merge then walks one output row at a time
    a.workers = mfma ? std::min<long>(resident, std::max<long>(1, (units + 1) / 2))
                     : std::min<long>(units, kMaxWorkers);
    if (units > 0) {
      launch_attn_partial(a, model->kv_dtype, D, G, stream);
      if ((st = hip_check(hipGetLastError(), "attn_partial launch"))) return st;
    }

    m.part = part;
    m.ml = ml;
    m.out = out;
    m.alpha = alpha;
    m.alpha_out = !model->alpha_scratch;
    m.gsum = deferred ? deferred->gsum : (scores ? gsum : nullptr);
    m.alpha_stride = alpha_stride;
    m.gs_stride = (long)wl.gs_stride;
    m.gs_seq_rows = (long)(deferred ? model->num_layers : Lr) * hkv;
    m.gs_row0 = deferred ? deferred->row0 : 0;
    m.total_units = a.total_units;
    m.workers = a.workers > 0 ? a.workers : 1;
    m.Lr = Lr;
    m.hq = hq;
    m.hkv = hkv;
    m.io_L = a.io_L;
    m.io_l0 = a.io_l0;
    m.out_rows = nb * Lr * hq;
    m.out_blocks = merge_output_blocks(m.out_rows);
    m.seq = a.seq;
    m.cbase[nb] = cblocks;
    launch_attn_merge(m, D, m.out_blocks + cblocks, stream);
    if ((st = hip_check(hipGetLastError(), "attn_merge launch"))) return st;

    if (scores && sblocks > 0 && !deferred) {
      sa.src = gsum;
      sa.row_stride = (long)wl.gs_stride;
      sa.seq_stride = (long)Lr * hkv * (long)wl.gs_stride;
      sa.rows = Lr * hkv;
      sa.t0_pos = t0_pos;
      sa.t1_pos = t1_pos;
      sa.t2_pos = any_t2 ? t2->t2_pos : nullptr;
      sa.scores = scores;
      sa.cap0 = cap0;
      sa.cap1 = cap1;
      sa.cap2 = cap2;
      sa.max_ctx = max_ctx;
      sa.weight = 1.0 / ((double)model->num_layers * hq);
      sa.seq.nb = nb;
      sa.seq.b_offset = b0;
      sa.seq.base[nb] = sblocks;
      launch_score_rows(sa, sblocks, "score_update", stream);
      if ((st = hip_check(hipGetLastError(), "score_update launch"))) return st;
    }
  }
  return TKV_OK;
}

}  // namespace tkv

namespace tkv {

// Workspace of tkv_decode_step_noalloc: one array per GPU, held until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device memory:
// its device address is looked up once per device and used from then on.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device ordinal

// The device address of `scratch` on the current device (looked up on the first call
// made with that device current).
static tkv_status scratch_on_current_device(void** out) {
  int dev = -1;
  tkv_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(TKV_ERR_HIP, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((st = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address")))
      return st;
    if (!p) return fail(TKV_ERR_HIP, "scratch address is null");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TKV_OK;
}

}  // namespace tkv

extern "C" {

tkv_status tkv_decode_step_noalloc(const tkv_model* model, int32_t batch, int32_t layer_begin,
                                   int32_t layer_end, const void* q, const void* k_t0,
                                   const void* v_t0, const int32_t* t0_len, int32_t cap0,
                                   const void* k_t1, const void* v_t1, const int32_t* t1_len,
                                   int32_t cap1, float* out, float* alpha, int32_t alpha_stride,
                                   const int32_t* t0_pos, const int32_t* t1_pos, float* scores,
                                   int32_t max_ctx, hipStream_t stream) {
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0 || layer_begin < 0 || layer_end > model->num_layers || layer_begin >= layer_end ||
      cap0 < 0 || cap1 < 0)
    return fail(TKV_ERR_ARG, "bad batch, layer range or capacity");
  const size_t need = tkv_decode_workspace_bytes(model, batch, layer_end - layer_begin, cap0, cap1);
  if (need > kNoAllocScratchBytes)
    return fail(TKV_ERR_CAPACITY, "the call needs " + std::to_string(need) +
                                      " bytes of workspace; tkv_decode_step_noalloc holds " +
                                      std::to_string(kNoAllocScratchBytes));
  if (batch == 0) return TKV_OK;
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws))) return st;
  return decode_step(model, batch, layer_begin, layer_end, q, k_t0, v_t0, t0_len, cap0, k_t1,
                     v_t1, t1_len, cap1, out, alpha, alpha_stride, t0_pos, t1_pos, scores,
                     max_ctx, ws, kNoAllocScratchBytes, stream, nullptr, nullptr);
}

tkv_status tkv_decode_step(const tkv_model* model, int32_t batch, int32_t layer_begin,
                           int32_t layer_end, const void* q, const void* k_t0, const void* v_t0,
                           const int32_t* t0_len, int32_t cap0, const void* k_t1,
                           const void* v_t1, const int32_t* t1_len, int32_t cap1, float* out,
                           float* alpha, int32_t alpha_stride, const int32_t* t0_pos,
                           const int32_t* t1_pos, float* scores, int32_t max_ctx,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_step(model, batch, layer_begin, layer_end, q, k_t0, v_t0, t0_len, cap0, k_t1,
                     v_t1, t1_len, cap1, out, alpha, alpha_stride, t0_pos, t1_pos, scores,
                     max_ctx, workspace, workspace_bytes, stream, nullptr, nullptr);
}

tkv_status tkv_decode_step_window(const tkv_model* model, int32_t batch, int32_t layer_begin,
                                  int32_t layer_end, const void* q, const void* k_t0,
                                  const void* v_t0, const int32_t* t0_len, int32_t cap0,
                                  const void* t1_win, const int32_t* t1_len, int32_t cap1,
                                  float* out, float* alpha, int32_t alpha_stride,
                                  const int32_t* t0_pos, const int32_t* t1_pos, float* scores,
                                  int32_t max_ctx, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  if (!model) return fail(TKV_ERR_ARG, "model is null");
  if (cap1 < 0 || cap1 % 32) return fail(TKV_ERR_ARG, "cap1 must be a multiple of 32");
  // each (sequence, layer, KV head) row of the window: cap1 key slots, then cap1 value slots
  const size_t e = model->kv_dtype == TKV_BF16 ? 2 : 4;
  const void* v_win = t1_win ? (const char*)t1_win + (size_t)cap1 * model->head_dim * e : nullptr;
  return decode_step(model, batch, layer_begin, layer_end, q, k_t0, v_t0, t0_len, cap0, t1_win,
                     v_win, t1_len, cap1, out, alpha, alpha_stride, t0_pos, t1_pos, scores,
                     max_ctx, workspace, workspace_bytes, stream, nullptr, nullptr, true, false,
                     2L * cap1 * model->head_dim);
}

tkv_status tkv_decode_step_streamed(const tkv_model* model, int32_t batch, const void* q,
                                    const void* k_t0, const void* v_t0, const int32_t* t0_len,
                                    int32_t cap0, const void* host_t1, const int32_t* t1_len,
                                    int32_t cap1, void* win, int32_t chunk_layers, float* out,
                                    float* alpha, int32_t alpha_stride, const int32_t* t0_pos,
                                    const int32_t* t1_pos, float* scores, int32_t max_ctx,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    hipStream_t side_stream, hipStream_t side_stream2,
                                    hipEvent_t* events, int64_t* link_bytes) {
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0) return fail(TKV_ERR_ARG, "batch < 0");
  if (batch == 0) return TKV_OK;
  if (batch > kMaxSeqPerLaunch)
    return fail(TKV_ERR_CAPACITY, "the streamed step takes at most 64 sequences per call");
  if (!host_t1 || !win || !events || !t1_len) return fail(TKV_ERR_ARG, "null pointer");
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return fail(TKV_ERR_ARG, "null event");
  const int L = model->num_layers;
  if (chunk_layers < 1 || chunk_layers > L) return fail(TKV_ERR_ARG, "need 1 <= chunk_layers <= L");
  if (cap1 < 0 || cap1 % 32) return fail(TKV_ERR_ARG, "cap1 must be a multiple of 32");
  const int hkv = model->num_kv_heads, D = model->head_dim;
  const size_t e = model->kv_dtype == TKV_BF16 ? 2 : 4;
  const size_t slot_bytes = (size_t)D * e;
  const size_t row_bytes = 2 * (size_t)cap1 * slot_bytes;        // keys then values of one row
  const size_t layer_bytes = (size_t)hkv * row_bytes;             // one layer of one sequence
  const size_t buf_bytes = (size_t)batch * chunk_layers * layer_bytes;
  const int n_chunks = (L + chunk_layers - 1) / chunk_layers;
  const long t1_rs = 2L * cap1 * D;
  // every check of the per-chunk calls before anything is queued (the chunks differ
  // only in their layer range)
  const DecodeWorkspace wfull = decode_workspace(model, batch, L, cap0, cap1);
  float* gsum = (float*)workspace + wfull.gsum;
  DeferredScore ds{gsum, 0};
  if ((st = decode_step(model, batch, 0, chunk_layers, q, k_t0, v_t0, t0_len, cap0, win,
                        (const char*)win + cap1 * slot_bytes, t1_len, cap1, out, alpha,
                        alpha_stride, t0_pos, t1_pos, scores, max_ctx, workspace,
                        workspace_bytes, stream, nullptr, nullptr, true, true, t1_rs,
                        scores ? &ds : nullptr)))
    return st;
  hipEvent_t* loaded = events;
  hipEvent_t* read = events + 2;
  int64_t link = 0;
  // everything queued on `stream` before this call (the previous step's reads of the
  // two buffers among it) happens before the first copies
  if ((st = hip_check(hipEventRecord(read[0], stream), "event record"))) return st;
  if ((st = hip_check(hipEventRecord(read[1], stream), "event record"))) return st;
  // chunk c goes on side stream c % 2 when two are given: the next copy is then
  // already queued when the running one ends (each buffer is always filled from
  // the same stream).  Only whole 32-slot blocks holding live T1 rows move: one
  // 2-D copy per sequence of its n * Hkv * 2 rows (keys, values), each
  // ceil32(t1_len) slots wide.
  auto copy_chunk = [&](int c) -> tkv_status {
    const int buf = c & 1;
    const int l0 = c * chunk_layers;
    const int n = std::min(chunk_layers, L - l0);
    hipStream_t ss = (side_stream2 && buf) ? side_stream2 : side_stream;
    tkv_status s2 = hip_check(hipStreamWaitEvent(ss, read[buf], 0), "stream wait");
    if (s2) return s2;
    char* dbuf = (char*)win + (size_t)buf * buf_bytes;
    for (int b = 0; b < batch; ++b) {
      const size_t live = (size_t)((t1_len[b] + 31) / 32 * 32) * slot_bytes;
      if (live == 0) continue;
      const char* src = (const char*)host_t1 + ((size_t)b * L + l0) * layer_bytes;
      char* dst = dbuf + (size_t)b * n * layer_bytes;     // a partial last chunk packs with pitch n
      s2 = hip_check(hipMemcpy2DAsync(dst, cap1 * slot_bytes, src, cap1 * slot_bytes, live,
                                      (size_t)n * hkv * 2, hipMemcpyHostToDevice, ss),
                     "T1 chunk copy");
      if (s2) return s2;
      link += (int64_t)(live * n * hkv * 2);
    }
    return hip_check(hipEventRecord(loaded[buf], ss), "event record");
  };
  for (int c = 0; c < std::min(2, n_chunks); ++c)
    if ((st = copy_chunk(c))) return st;
  for (int c = 0; c < n_chunks; ++c) {
    const int buf = c & 1;
    const int l0 = c * chunk_layers;
    const int n = std::min(chunk_layers, L - l0);
    if ((st = hip_check(hipStreamWaitEvent(stream, loaded[buf], 0), "stream wait"))) return st;
    const char* wk = (const char*)win + (size_t)buf * buf_bytes;
    ds.row0 = l0 * hkv;
    if ((st = decode_step(model, batch, l0, l0 + n, q, k_t0, v_t0, t0_len, cap0, wk,
                          wk + cap1 * slot_bytes, t1_len, cap1, out, alpha, alpha_stride,
                          t0_pos, t1_pos, scores, max_ctx, workspace, workspace_bytes, stream,
                          nullptr, nullptr, true, false, t1_rs, scores ? &ds : nullptr)))
      return st;
    if ((st = hip_check(hipEventRecord(read[buf], stream), "event record"))) return st;
    if (c + 2 < n_chunks && (st = copy_chunk(c + 2))) return st;
  }
  // the whole step's score increment, added once: the group sums of every layer in
  // the order of a single-call step
  if (scores) {
    ScoreArgs sa{};
    int sblocks = 0;
    for (int i = 0; i < batch; ++i) {
      sa.seq.t0_len[i] = t0_len[i];
      sa.seq.t1_len[i] = t1_len[i];
      sa.seq.base[i] = sblocks;
      sblocks += ceil_div(t0_len[i] + t1_len[i], kScoreSlots);
    }
    sa.seq.nb = batch;
    sa.seq.b_offset = 0;
    sa.seq.base[batch] = sblocks;
    sa.src = gsum;
    sa.row_stride = (long)wfull.gs_stride;
    sa.seq_stride = (long)L * hkv * (long)wfull.gs_stride;
    sa.rows = L * hkv;
    sa.t0_pos = t0_pos;
    sa.t1_pos = t1_pos;
    sa.scores = scores;
    sa.cap0 = cap0;
    sa.cap1 = cap1;
    sa.max_ctx = max_ctx;
    sa.weight = 1.0 / ((double)L * model->num_q_heads);
    if (sblocks > 0) {
      launch_score_rows(sa, sblocks, "score_update", stream);
      if ((st = hip_check(hipGetLastError(), "score_update launch"))) return st;
    }
  }
  if (link_bytes) *link_bytes = link;
  return TKV_OK;
}

tkv_status tkv_decode_step_t2(const tkv_model* model, int32_t batch, int32_t layer_begin,
                              int32_t layer_end, const void* q, const void* k_t0,
                              const void* v_t0, const int32_t* t0_len, int32_t cap0,
                              const void* k_t1, const void* v_t1, const int32_t* t1_len,
                              int32_t cap1, const tkv_t2_pool* t2, float* out, float* alpha,
                              int32_t alpha_stride, const int32_t* t0_pos,
                              const int32_t* t1_pos, float* scores, int32_t max_ctx,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!t2) return fail(TKV_ERR_ARG, "T2 pool is null");
  return decode_step(model, batch, layer_begin, layer_end, q, k_t0, v_t0, t0_len, cap0, k_t1,
                     v_t1, t1_len, cap1, out, alpha, alpha_stride, t0_pos, t1_pos, scores,
                     max_ctx, workspace, workspace_bytes, stream, nullptr, t2);
}

tkv_status tkv_append_decode_step(const tkv_model* model, int32_t batch, const void* k_new,
                                  const void* v_new, const int32_t* position, uint8_t* tier,
                                  const void* q, void* k_t0, void* v_t0, const int32_t* t0_len,
                                  int32_t cap0, const void* k_t1, const void* v_t1,
                                  const int32_t* t1_len, int32_t cap1, float* out, float* alpha,
                                  int32_t alpha_stride, int32_t* t0_pos, const int32_t* t1_pos,
                                  float* scores, int32_t max_ctx, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (!model) return fail(TKV_ERR_ARG, "model is null");
  const AppendInfo app{k_new, v_new, position, t0_pos, tier};
  return decode_step(model, batch, 0, model->num_layers, q, k_t0, v_t0, t0_len, cap0, k_t1, v_t1,
                     t1_len, cap1, out, alpha, alpha_stride, t0_pos, t1_pos, scores, max_ctx,
                     workspace, workspace_bytes, stream, &app, nullptr);
}

tkv_status tkv_append_decode_step_t2(const tkv_model* model, int32_t batch, const void* k_new,
                                     const void* v_new, const int32_t* position, uint8_t* tier,
                                     const void* q, void* k_t0, void* v_t0,
                                     const int32_t* t0_len, int32_t cap0, const void* k_t1,
                                     const void* v_t1, const int32_t* t1_len, int32_t cap1,
                                     const tkv_t2_pool* t2, float* out, float* alpha,
                                     int32_t alpha_stride, int32_t* t0_pos,
                                     const int32_t* t1_pos, float* scores, int32_t max_ctx,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (!model) return fail(TKV_ERR_ARG, "model is null");
  if (!t2) return fail(TKV_ERR_ARG, "T2 pool is null");
  const AppendInfo app{k_new, v_new, position, t0_pos, tier};
  return decode_step(model, batch, 0, model->num_layers, q, k_t0, v_t0, t0_len, cap0, k_t1, v_t1,
                     t1_len, cap1, out, alpha, alpha_stride, t0_pos, t1_pos, scores, max_ctx,
                     workspace, workspace_bytes, stream, &app, t2);
}

tkv_status tkv_update_scores(const tkv_model* model, int32_t batch, int32_t layer_begin,
                             int32_t layer_end, const float* alpha, int32_t alpha_stride,
                             const int32_t* t0_pos, const int32_t* t0_len, int32_t cap0,
                             const int32_t* t1_pos, const int32_t* t1_len, int32_t cap1,
                             float* scores, int32_t max_ctx, hipStream_t stream) {
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0) return fail(TKV_ERR_ARG, "batch < 0");
  if (layer_begin < 0 || layer_end > model->num_layers || layer_begin >= layer_end)
    return fail(TKV_ERR_ARG, "need 0 <= layer_begin < layer_end <= num_layers");
  if (batch == 0) return TKV_OK;
  if (!alpha || !t0_pos || !t0_len || !t1_len || !scores) return fail(TKV_ERR_ARG, "null pointer");
  if (alpha_stride < 1 || max_ctx < 1 || cap0 < 0 || cap1 < 0)
    return fail(TKV_ERR_ARG, "bad capacity or stride");
  bool any_t1 = false;
  for (int b = 0; b < batch; ++b) {
    if (t0_len[b] < 0 || t1_len[b] < 0) return fail(TKV_ERR_ARG, "negative length");
    if (t0_len[b] > cap0 || t1_len[b] > cap1) return fail(TKV_ERR_CAPACITY, "length > capacity");
    if ((long)t0_len[b] + t1_len[b] > alpha_stride)
      return fail(TKV_ERR_CAPACITY, "alpha_stride < t0_len + t1_len");
    any_t1 |= t1_len[b] > 0;
  }
  if (any_t1 && !t1_pos) return fail(TKV_ERR_ARG, "t1_pos is null but t1_len > 0");
  const int Lr = layer_end - layer_begin;
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    ScoreArgs sa{};
    const int rows = Lr * model->num_q_heads;
    sa.src = alpha + (size_t)b0 * rows * alpha_stride;
    sa.row_stride = alpha_stride;
    sa.seq_stride = (long)rows * alpha_stride;
    sa.rows = rows;
    sa.t0_pos = t0_pos;
    sa.t1_pos = t1_pos;
    sa.scores = scores;
    sa.cap0 = cap0;
    sa.cap1 = cap1;
    sa.max_ctx = max_ctx;
    sa.weight = 1.0 / ((double)model->num_layers * model->num_q_heads);
    sa.seq.nb = nb;
    sa.seq.b_offset = b0;
    int sblocks = 0;
    for (int i = 0; i < nb; ++i) {
      sa.seq.t0_len[i] = t0_len[b0 + i];
      sa.seq.t1_len[i] = t1_len[b0 + i];
      sa.seq.base[i] = sblocks;
      sblocks += ceil_div(t0_len[b0 + i] + t1_len[b0 + i], kScoreSlots);
    }
    sa.seq.base[nb] = sblocks;
    if (sblocks > 0) {
      launch_score_rows(sa, sblocks, "update_scores", stream);
      if ((st = hip_check(hipGetLastError(), "update_scores launch"))) return st;
    }
  }
  return TKV_OK;
}

tkv_status tkv_assign_tiers(int32_t batch, const int32_t* ctx_len, int32_t max_ctx,
                            const float* scores, const tkv_policy* policy,
                            const uint8_t* tier_prev, uint8_t* tier_next, int32_t* counts,
                            hipStream_t stream) {
  if (batch < 0) return fail(TKV_ERR_ARG, "batch < 0");
  if (!policy) return fail(TKV_ERR_ARG, "policy is null");
  const float f1 = policy->frac_t1, f2 = policy->frac_t2, f3 = policy->frac_t3;
  if (!(f1 >= 0.f && f2 >= 0.f && f3 >= 0.f) || (double)f1 + f2 + f3 > 1.0)
    return fail(TKV_ERR_ARG, "tier fractions must be >= 0 and sum to <= 1");
  if (policy->prompt_len < 0 || policy->num_sinks < 0 || policy->recent_window < 0)
    return fail(TKV_ERR_ARG, "negative protected size");
  if (policy->delta < 1) return fail(TKV_ERR_ARG, "delta < 1");
  if (batch == 0) return TKV_OK;
  if (!ctx_len || !scores || !tier_prev || !tier_next || !counts)
    return fail(TKV_ERR_ARG, "null pointer");
  if (max_ctx < 1) return fail(TKV_ERR_ARG, "max_ctx < 1");
  for (int b = 0; b < batch; ++b) {
    if (ctx_len[b] < 0) return fail(TKV_ERR_ARG, "negative length");
    if (ctx_len[b] > max_ctx) return fail(TKV_ERR_CAPACITY, "ctx_len > max_ctx");
  }
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    TierArgs a{};
    a.scores = scores;
    a.tprev = tier_prev;
    a.tnext = tier_next;
    a.counts = counts;
    a.max_ctx = max_ctx;
    a.prot_lo = std::max(policy->prompt_len, policy->num_sinks);
    a.recent = policy->recent_window;
    a.b_offset = b0;
    for (int i = 0; i < nb; ++i) {
      const int n = ctx_len[b0 + i];
      a.n[i] = n;
      a.n1[i] = (int)floor((double)f1 * (double)n);
      a.n2[i] = (int)floor((double)f2 * (double)n);
      a.n3[i] = (int)floor((double)f3 * (double)n);
    }
    launch_assign_tiers(a, nb, stream);
    tkv_status st = hip_check(hipGetLastError(), "assign_tiers launch");
    if (st) return st;
  }
  return TKV_OK;
}

// Relocation workspace, every region 256-byte aligned:
//   inv [B][max_ctx] | holes0 [B][cap0] | holes1 [B][cap1] | to_t0 [B][cap0] int2 |
//   to_t1 [B][cap1] int2 | staged [B][cap1] int2 | cnt [B][4] | staging [B][cap1][L*Hkv][2][D]
struct RelocWorkspace {
  size_t inv, holes0, holes1, to_t0, to_t1, staged, cnt, staging, total;
};

static RelocWorkspace reloc_workspace(const tkv_model* m, int batch, int max_ctx, int cap0,
                                      int cap1) {
  const size_t B = (size_t)batch;
  const size_t elem = m->kv_dtype == TKV_BF16 ? 2 : 4;
  RelocWorkspace w;
  w.inv = 0;
  w.holes0 = round_up(w.inv + B * max_ctx * 4, 256);
  w.holes1 = round_up(w.holes0 + B * cap0 * 4, 256);
  w.to_t0 = round_up(w.holes1 + B * cap1 * 4, 256);
  w.to_t1 = round_up(w.to_t0 + B * cap0 * 8, 256);
  w.staged = round_up(w.to_t1 + B * cap1 * 8, 256);
  w.cnt = round_up(w.staged + B * cap1 * 8, 256);
  w.staging = round_up(w.cnt + B * 16, 256);
  w.total = round_up(w.staging + B * cap1 * (size_t)m->num_layers * m->num_kv_heads * 2 *
                                     m->head_dim * elem,
                     256);
  return w;
}

size_t tkv_compact_workspace_bytes(const tkv_model* model, int32_t batch, int32_t max_ctx,
                                   int32_t cap0, int32_t cap1) {
  if (check_model(model) || batch < 0 || max_ctx < 0 || cap0 < 0 || cap1 < 0) return 0;
  return reloc_workspace(model, batch, max_ctx, cap0, cap1).total;
}

tkv_status tkv_compact(const tkv_model* model, int32_t batch, const int32_t* ctx_len,
                       int32_t max_ctx, const uint8_t* tier_prev, const uint8_t* tier_next,
                       void* k_t0, void* v_t0, int32_t* t0_pos, const int32_t* t0_len,
                       int32_t cap0, void* k_t1, void* v_t1, int32_t* t1_pos,
                       const int32_t* t1_len, int32_t cap1, int32_t* t2_src, int32_t* t2_pos,
                       int32_t t2_cap, int8_t* t2_codes, float* t2_scales, int32_t* new_lens,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0) return fail(TKV_ERR_ARG, "batch < 0");
  if (batch == 0) return TKV_OK;
  if (!ctx_len || !tier_prev || !tier_next || !k_t0 || !v_t0 || !t0_pos || !t0_len || !t1_len ||
      !t2_src || !t2_pos || !new_lens || !workspace)
    return fail(TKV_ERR_ARG, "null pointer");
  if (cap1 > 0 && (!k_t1 || !v_t1 || !t1_pos))
    return fail(TKV_ERR_ARG, "null T1 pointer with cap1 > 0");
  if (t2_cap > 0 && (!t2_codes || !t2_scales))
    return fail(TKV_ERR_ARG, "null T2 codes or scales with t2_cap > 0");
  if (cap0 < 1 || cap1 < 0 || t2_cap < 0 || max_ctx < 1 || cap0 % 32 || cap1 % 32)
    return fail(TKV_ERR_ARG, "bad capacity (cap0, cap1 multiples of 32)");
  if (t2_cap > 65535) return fail(TKV_ERR_CAPACITY, "t2_cap above 65535");
  if (tier_prev == tier_next) return fail(TKV_ERR_ARG, "tier_prev and tier_next must differ");
  for (int b = 0; b < batch; ++b) {
    if (ctx_len[b] < 0 || t0_len[b] < 0 || t1_len[b] < 0)
      return fail(TKV_ERR_ARG, "negative length");
    if (ctx_len[b] > max_ctx) return fail(TKV_ERR_CAPACITY, "ctx_len > max_ctx");
    if (t0_len[b] > cap0_of(model, b, cap0) || t1_len[b] > cap1_of(model, b, cap1))
      return fail(TKV_ERR_CAPACITY, "length > capacity");
    if ((long)t0_len[b] + t1_len[b] > ctx_len[b])
      return fail(TKV_ERR_STATE, "t0_len + t1_len > ctx_len");
  }
  if ((st = check_caps(model, batch, cap0, cap1, true))) return st;
  const RelocWorkspace w = reloc_workspace(model, batch, max_ctx, cap0, cap1);
  if (workspace_bytes < w.total) return fail(TKV_ERR_CAPACITY, "workspace too small");
  char* base = (char*)workspace;
  const int lgs = model->num_layers * model->num_kv_heads;
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    RelocArgs a{};
    a.tprev = tier_prev;
    a.tnext = tier_next;
    a.t0_pos = t0_pos;
    a.t1_pos = t1_pos;
    a.inv = (int*)(base + w.inv);
    a.holes0 = (int*)(base + w.holes0);
    a.holes1 = (int*)(base + w.holes1);
    a.to_t0 = (int2*)(base + w.to_t0);
    a.to_t1 = (int2*)(base + w.to_t1);
    a.staged = (int2*)(base + w.staged);
    a.cnt = (int*)(base + w.cnt);
    a.t2_src = t2_src;
    a.t2_pos = t2_pos;
    a.new_lens = new_lens;
    a.max_ctx = max_ctx;
    a.cap0 = cap0;
    a.cap1 = cap1;
    a.t2_cap = t2_cap;
    a.b_offset = b0;
    a.host_t1 = 0;
    for (int i = 0; i < nb; ++i) {
      a.n[i] = ctx_len[b0 + i];
      a.len0[i] = t0_len[b0 + i];
      a.len1[i] = t1_len[b0 + i];
      a.lim0[i] = cap0_of(model, b0 + i, cap0);
      a.lim1[i] = cap1_of(model, b0 + i, cap1);
    }
    launch_reloc_scan(a, nb, stream);
    if ((st = hip_check(hipGetLastError(), "reloc_scan launch"))) return st;
    // the rows entering T2 are quantised from their old slots, before any row moves
    if (t2_cap > 0) {
      QuantArgs q{};
      q.k0 = k_t0;
      q.v0 = v_t0;
      q.k1 = k_t1;
      q.v1 = v_t1;
      q.staging = nullptr;
      q.only = 0;
      q.src = t2_src;
      q.n_rows = new_lens + 2;
      q.codes = t2_codes;
      q.scales = t2_scales;
      q.n_rows_stride = 4;
      q.max_rows = t2_cap;
      q.cap0 = cap0;
      q.cap1 = cap1;
      q.L = model->num_layers;
      q.hkv = model->num_kv_heads;
      q.b_offset = b0;
      fill_pool(q.pool, model, b0, nb, cap0, cap1);
      launch_quantize(q, model->kv_dtype, model->head_dim, nb, stream);
      if ((st = hip_check(hipGetLastError(), "quantize launch"))) return st;
    }
    // promoted T1 rows to staging, then every row into the T1 window (its
    // sources are T0 slots and T1 slots at or past the new T1 length, never a
    // T1 hole), then every row into the T0 pool (sources: T0 slots at or past
    // the new T0 length, and staging)
    MoveArgs mv{};
    mv.k0 = k_t0;
    mv.v0 = v_t0;
    mv.k1 = k_t1;
    mv.v1 = v_t1;
    mv.staging = base + w.staging;
    mv.cnt = a.cnt;
    mv.cap0 = cap0;
    mv.cap1 = cap1;
    mv.lgs = lgs;
    mv.b_offset = b0;
    mv.nb = nb;
    fill_pool(mv.pool, model, b0, nb, cap0, cap1);
    const int2* lists[3] = {a.staged, a.to_t1, a.to_t0};
    const int strides[3] = {cap1, cap1, cap0};
    const int order[3] = {kMoveStage, kMoveToT1, kMoveToT0};
    for (int k = 0; k < 3; ++k) {
      if (cap1 == 0 && order[k] != kMoveToT0) continue;
      mv.which = order[k];
      mv.list = lists[order[k]];
      mv.list_stride = strides[order[k]];
      launch_reloc_move(mv, model->kv_dtype, model->head_dim, stream);
      if ((st = hip_check(hipGetLastError(), "reloc_move launch"))) return st;
    }
  }
  return TKV_OK;
}

// Pinned host scratch of tkv_compact_host_t1, every region 256-byte aligned:
//   rows [B][cap1][L*Hkv][2][D] | tier_prev, tier_next [B][max_ctx] u8 |
//   pos1 before, after [B][cap1] | to_t1 [B][cap1] int2 | lens, cnt [B][4]
struct HostT1Scratch {
  size_t rows, tprev, tnext, pos_old, pos_new, to_t1, lens, cnt, total;
};

static HostT1Scratch host_t1_scratch(const tkv_model* m, int batch, int max_ctx, int cap1) {
  const size_t B = (size_t)batch;
  const size_t elem = m->kv_dtype == TKV_BF16 ? 2 : 4;
  HostT1Scratch h;
  h.rows = 0;
  h.tprev = round_up(B * cap1 * (size_t)m->num_layers * m->num_kv_heads * 2 * m->head_dim * elem, 256);
  h.tnext = round_up(h.tprev + B * max_ctx, 256);
  h.pos_old = round_up(h.tnext + B * max_ctx, 256);
  h.pos_new = round_up(h.pos_old + B * cap1 * 4, 256);
  h.to_t1 = round_up(h.pos_new + B * cap1 * 4, 256);
  h.lens = round_up(h.to_t1 + B * cap1 * 8, 256);
  h.cnt = round_up(h.lens + B * 16, 256);
  h.total = round_up(h.cnt + B * 16, 256);
  return h;
}

size_t tkv_compact_host_t1_workspace_bytes(const tkv_model* model, int32_t batch, int32_t max_ctx,
                                           int32_t cap0, int32_t cap1) {
  if (check_model(model) || batch < 0 || max_ctx < 0 || cap0 < 0 || cap1 < 0) return 0;
  return reloc_workspace(model, batch, max_ctx, cap0, cap1).staging;  // no device staging
}

size_t tkv_compact_host_t1_scratch_bytes(const tkv_model* model, int32_t batch, int32_t max_ctx,
                                         int32_t cap1) {
  if (check_model(model) || batch < 0 || max_ctx < 0 || cap1 < 0) return 0;
  return host_t1_scratch(model, batch, max_ctx, cap1).total;
}

int32_t tkv_t0_capacity(const tkv_policy* policy, int32_t n_from, int32_t n_to) {
  if (!policy || n_from < 0 || n_to < n_from || policy->delta < 1) return -1;
  const float f1 = policy->frac_t1, f2 = policy->frac_t2, f3 = policy->frac_t3;
  if (!(f1 >= 0.f && f2 >= 0.f && f3 >= 0.f) || (double)f1 + f2 + f3 > 1.0) return -1;
  if (policy->prompt_len < 0 || policy->num_sinks < 0 || policy->recent_window < 0) return -1;
  // after a reassignment at length n, T0 holds at most max(N0(n), |protected(n)|) rows:
  // either every budget of T1..T3 is met (T0 = N0 or fewer, T2/T3 being absorbing), or
  // the non-protected candidates ran out (T0 = the protected T0/T1 rows); then Delta
  // appended rows before the next reassignment
  long best = 0;
  const long lo = std::max(policy->prompt_len, policy->num_sinks);
  for (long n = n_from; n <= n_to; ++n) {
    const long n0 = n - (long)floor((double)f1 * n) - (long)floor((double)f2 * n) -
                    (long)floor((double)f3 * n);
    const long head = std::min(n, lo);
    const long tail = std::max(head, std::max(0L, n - (long)policy->recent_window));
    const long prot = head + (n - tail);
    best = std::max(best, std::max(n0, prot));
  }
  const long cap = (best + policy->delta + 31) / 32 * 32;
  return cap > INT32_MAX ? -1 : (int32_t)cap;
}

tkv_status tkv_compact_host_t1(const tkv_model* model, int32_t batch, const int32_t* ctx_len,
                               int32_t max_ctx, const uint8_t* tier_prev,
                               const uint8_t* tier_next, void* k_t0, void* v_t0,
                               int32_t* t0_pos, const int32_t* t0_len, int32_t cap0,
                               int32_t* t1_pos, const int32_t* t1_len, int32_t cap1,
                               void* store_k, void* store_v, void* t1_host, int32_t* t2_src,
                               int32_t* t2_pos, int32_t t2_cap, int8_t* t2_codes,
                               float* t2_scales, int32_t* new_lens, int32_t* new_lens_host,
                               void* workspace, size_t workspace_bytes, void* host_scratch,
                               size_t host_scratch_bytes, int64_t* link_bytes,
                               hipStream_t stream) {
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0) return fail(TKV_ERR_ARG, "batch < 0");
  if (batch == 0) return TKV_OK;
  if (!ctx_len || !tier_prev || !tier_next || !k_t0 || !v_t0 || !t0_pos || !t0_len || !t1_pos ||
      !t1_len || !store_k || !store_v || !t1_host || !t2_src || !t2_pos || !new_lens ||
      !new_lens_host || !workspace || !host_scratch)
    return fail(TKV_ERR_ARG, "null pointer");
  if (t2_cap > 0 && (!t2_codes || !t2_scales))
    return fail(TKV_ERR_ARG, "null T2 codes or scales with t2_cap > 0");
  if (cap0 < 1 || cap1 < 0 || t2_cap < 0 || max_ctx < 1 || cap0 % 32 || cap1 % 32)
    return fail(TKV_ERR_ARG, "bad capacity (cap0, cap1 multiples of 32)");
  if (t2_cap > 65535) return fail(TKV_ERR_CAPACITY, "t2_cap above 65535");
  if (tier_prev == tier_next) return fail(TKV_ERR_ARG, "tier_prev and tier_next must differ");
  for (int b = 0; b < batch; ++b) {
    if (ctx_len[b] < 0 || t0_len[b] < 0 || t1_len[b] < 0)
      return fail(TKV_ERR_ARG, "negative length");
    if (ctx_len[b] > max_ctx) return fail(TKV_ERR_CAPACITY, "ctx_len > max_ctx");
    if (t0_len[b] > cap0_of(model, b, cap0) || t1_len[b] > cap1)
      return fail(TKV_ERR_CAPACITY, "length > capacity");
    if ((long)t0_len[b] + t1_len[b] > ctx_len[b])
      return fail(TKV_ERR_STATE, "t0_len + t1_len > ctx_len");
  }
  if ((st = check_caps(model, batch, cap0, cap1, false))) return st;
  const RelocWorkspace w = reloc_workspace(model, batch, max_ctx, cap0, cap1);
  if (workspace_bytes < w.staging) return fail(TKV_ERR_CAPACITY, "workspace too small");
  const HostT1Scratch hs = host_t1_scratch(model, batch, max_ctx, cap1);
  if (host_scratch_bytes < hs.total) return fail(TKV_ERR_CAPACITY, "host scratch too small");
  char* hb = (char*)host_scratch;
  // the row staging is read and written by the kernels in place (pinned host memory)
  void* rows_dev = nullptr;
  if ((st = hip_check(hipHostGetDevicePointer(&rows_dev, hb + hs.rows, 0),
                      "host scratch is not pinned, device-mapped memory")))
    return st;
  char* base = (char*)workspace;
  const int L = model->num_layers, hkv = model->num_kv_heads, D = model->head_dim;
  const int lgs = L * hkv;
  const size_t elem = model->kv_dtype == TKV_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)lgs * 2 * D * elem;  // one position: K and V of every (l, g)
  int32_t* pos_old = (int32_t*)(hb + hs.pos_old);
  int32_t* pos_new = (int32_t*)(hb + hs.pos_new);
  uint8_t* tp_h = (uint8_t*)(hb + hs.tprev);
  uint8_t* tn_h = (uint8_t*)(hb + hs.tnext);
  int2* to1_h = (int2*)(hb + hs.to_t1);
  int32_t* lens_h = (int32_t*)(hb + hs.lens);
  int32_t* cnt_h = (int32_t*)(hb + hs.cnt);
  const size_t B = (size_t)batch;
  int64_t link = 0;
  // 1. the slot -> position map of the T1 window before the relocation
  if ((st = hip_check(hipMemcpyAsync(pos_old, t1_pos, B * cap1 * 4, hipMemcpyDeviceToHost, stream),
                      "T1 map copy")))
    return st;
  link += (int64_t)(B * cap1 * 4);
  // 2. the scan, the new T2 rows that leave T0, and the rows that enter T1 from T0
  //    written to host memory (the only rows that go device -> host)
  RelocArgs a{};
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    a = RelocArgs{};
    a.tprev = tier_prev;
    a.tnext = tier_next;
    a.t0_pos = t0_pos;
    a.t1_pos = t1_pos;
    a.inv = (int*)(base + w.inv);
    a.holes0 = (int*)(base + w.holes0);
    a.holes1 = (int*)(base + w.holes1);
    a.to_t0 = (int2*)(base + w.to_t0);
    a.to_t1 = (int2*)(base + w.to_t1);
    a.staged = (int2*)(base + w.staged);
    a.cnt = (int*)(base + w.cnt);
    a.t2_src = t2_src;
    a.t2_pos = t2_pos;
    a.new_lens = new_lens;
    a.max_ctx = max_ctx;
    a.cap0 = cap0;
    a.cap1 = cap1;
    a.t2_cap = t2_cap;
    a.b_offset = b0;
    a.host_t1 = 1;
    for (int i = 0; i < nb; ++i) {
      a.n[i] = ctx_len[b0 + i];
      a.len0[i] = t0_len[b0 + i];
      a.len1[i] = t1_len[b0 + i];
      a.lim0[i] = cap0_of(model, b0 + i, cap0);
      a.lim1[i] = cap1;  // the host window
    }
    launch_reloc_scan(a, nb, stream);
    if ((st = hip_check(hipGetLastError(), "reloc_scan launch"))) return st;
    if (t2_cap > 0) {
      QuantArgs q{};
      q.k0 = k_t0;
      q.v0 = v_t0;
      q.staging = rows_dev;
      q.only = 1;
      q.src = t2_src;
      q.n_rows = new_lens + 2;
      q.codes = t2_codes;
      q.scales = t2_scales;
      q.n_rows_stride = 4;
      q.max_rows = t2_cap;
      q.cap0 = cap0;
      q.cap1 = cap1;
      q.L = L;
      q.hkv = hkv;
      q.b_offset = b0;
      fill_pool(q.pool, model, b0, nb, cap0, 0);
      launch_quantize(q, model->kv_dtype, D, nb, stream);
      if ((st = hip_check(hipGetLastError(), "quantize launch"))) return st;
    }
    if (cap1 > 0) {
      MoveArgs mv{};
      mv.k0 = k_t0;
      mv.v0 = v_t0;
      mv.staging = rows_dev;
      mv.cnt = a.cnt;
      mv.cap0 = cap0;
      mv.cap1 = cap1;
      mv.lgs = lgs;
      mv.b_offset = b0;
      mv.nb = nb;
      fill_pool(mv.pool, model, b0, nb, cap0, 0);
      mv.which = kMoveDown;
      mv.list = a.to_t1;
      mv.list_stride = cap1;
      launch_reloc_move(mv, model->kv_dtype, D, stream);
      if ((st = hip_check(hipGetLastError(), "reloc_move launch"))) return st;
    }
  }
  // 3. the maps the host side needs, then one sync
  struct Cp {
    void* dst;
    const void* src;
    size_t bytes;
  } cps[] = {{tp_h, tier_prev, B * max_ctx},           {tn_h, tier_next, B * max_ctx},
             {pos_new, t1_pos, B * cap1 * 4},          {to1_h, base + w.to_t1, B * cap1 * 8},
             {lens_h, new_lens, B * 16},               {cnt_h, base + w.cnt, B * 16}};
  for (const Cp& c : cps) {
    if ((st = hip_check(hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyDeviceToHost, stream),
                        "map copy")))
      return st;
    link += (int64_t)c.bytes;
  }
  if ((st = hip_check(hipStreamSynchronize(stream), "stream sync"))) return st;
  // 4. host: rows that entered T1 from T0 into the store; the rows that leave T1 for
  //    T0 (promoted, ascending position) and for T2 (after them) into the staging rows
  const size_t store_rs = (size_t)max_ctx * D * elem;  // one (l, g) row of the store
  char* rows_h = hb + hs.rows;
  std::vector<int> ok(batch, 1);
  std::vector<std::vector<int32_t>> up(batch);
  std::vector<std::vector<std::pair<int32_t, int32_t>>> down(batch);  // (staging row, position)
  for (int b = 0; b < batch; ++b) {
    memcpy(new_lens_host + 4 * b, lens_h + 4 * b, 16);
    if (lens_h[4 * b] < 0) {
      ok[b] = 0;
      continue;
    }
    const int n = ctx_len[b];
    const uint8_t* tp = tp_h + (size_t)b * max_ctx;
    const uint8_t* tn = tn_h + (size_t)b * max_ctx;
    for (int p = 0; p < n; ++p)
      if (tp[p] == 1 && tn[p] == 0) up[b].push_back(p);
    const int mp = (int)up[b].size();
    for (int p = 0; p < n; ++p)
      if (tp[p] == 1 && tn[p] == 2) up[b].push_back(p);
    if (mp != cnt_h[4 * b + kMoveStage] || (long)up[b].size() > cap1)
      return fail(TKV_ERR_STATE, "promoted rows disagree with the device relocation lists");
    const int m1 = cnt_h[4 * b + kMoveToT1];
    const int2* l1 = to1_h + (size_t)b * cap1;
    for (int i = 0; i < m1; ++i)
      if (l1[i].x >= 0) down[b].push_back({i, pos_new[(size_t)b * cap1 + l1[i].y]});
  }
  std::vector<std::pair<int, int>> jobs;  // (sequence, index) over down then up rows
  for (int b = 0; b < batch; ++b)
    for (int i = 0; i < (int)down[b].size(); ++i) jobs.push_back({b, i});
  const size_t n_down = jobs.size();
  parallel_ranges((long)n_down, std::min<long>(host_threads(), 1 + (long)n_down / 64),
                  [&](long lo, long hi) {
    for (long j = lo; j < hi; ++j) {
      const int b = jobs[j].first;
      const auto& d = down[b][jobs[j].second];
      const char* src = rows_h + ((size_t)b * cap1 + d.first) * row_bytes;
      for (int lg = 0; lg < lgs; ++lg) {
        const size_t so = ((size_t)b * lgs + lg) * store_rs + (size_t)d.second * D * elem;
        memcpy((char*)store_k + so, src + (size_t)lg * 2 * D * elem, D * elem);
        memcpy((char*)store_v + so, src + ((size_t)lg * 2 + 1) * D * elem, D * elem);
      }
    }
  });
  jobs.clear();
  for (int b = 0; b < batch; ++b)
    for (int i = 0; i < (int)up[b].size(); ++i) jobs.push_back({b, i});
  parallel_ranges((long)jobs.size(), std::min<long>(host_threads(), 1 + (long)jobs.size() / 64),
                  [&](long lo, long hi) {
    for (long j = lo; j < hi; ++j) {
      const int b = jobs[j].first, i = jobs[j].second;
      const int p = up[b][i];
      char* dst = rows_h + ((size_t)b * cap1 + i) * row_bytes;
      for (int lg = 0; lg < lgs; ++lg) {
        const size_t so = ((size_t)b * lgs + lg) * store_rs + (size_t)p * D * elem;
        memcpy(dst + (size_t)lg * 2 * D * elem, (const char*)store_k + so, D * elem);
        memcpy(dst + ((size_t)lg * 2 + 1) * D * elem, (const char*)store_v + so, D * elem);
      }
    }
  });
  link += (int64_t)((n_down + jobs.size()) * row_bytes);
  // 5. device: the new T2 rows that left T1, then every row into the T0 pool (the
  //    promoted rows straight from the staging rows)
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    if (t2_cap > 0) {
      QuantArgs q{};
      q.k0 = k_t0;
      q.v0 = v_t0;
      q.staging = rows_dev;
      q.only = 2;
      q.src = t2_src;
      q.n_rows = new_lens + 2;
      q.codes = t2_codes;
      q.scales = t2_scales;
      q.n_rows_stride = 4;
      q.max_rows = t2_cap;
      q.cap0 = cap0;
      q.cap1 = cap1;
      q.L = L;
      q.hkv = hkv;
      q.b_offset = b0;
      fill_pool(q.pool, model, b0, nb, cap0, 0);
      launch_quantize(q, model->kv_dtype, D, nb, stream);
      if ((st = hip_check(hipGetLastError(), "quantize launch"))) return st;
    }
    MoveArgs mv{};
    mv.k0 = k_t0;
    mv.v0 = v_t0;
    mv.staging = rows_dev;
    mv.cnt = (int*)(base + w.cnt);
    mv.cap0 = cap0;
    mv.cap1 = cap1;
    mv.lgs = lgs;
    mv.b_offset = b0;
    mv.nb = nb;
    fill_pool(mv.pool, model, b0, nb, cap0, 0);
    mv.which = kMoveToT0;
    mv.list = (int2*)(base + w.to_t0);
    mv.list_stride = cap0;
    launch_reloc_move(mv, model->kv_dtype, D, stream);
    if ((st = hip_check(hipGetLastError(), "reloc_move launch"))) return st;
  }
  // 6. host, while the device moves rows: the streamed T1 window takes the rows of the
  //    slots whose position changed (holes refilled), from the store
  const size_t seq_t1 = (size_t)lgs * 2 * cap1 * D * elem;
  for (int b = 0; b < batch; ++b) {
    if (!ok[b]) continue;
    const int n1 = lens_h[4 * b + 1];
    std::vector<int32_t> slots, poss;
    for (int s2 = 0; s2 < n1; ++s2) {
      const int32_t pn = pos_new[(size_t)b * cap1 + s2];
      if (s2 >= t1_len[b] || pn != pos_old[(size_t)b * cap1 + s2]) {
        slots.push_back(s2);
        poss.push_back(pn);
      }
    }
    pack_t1_slots(model, (const char*)store_k + (size_t)b * lgs * store_rs,
                  (const char*)store_v + (size_t)b * lgs * store_rs, max_ctx, slots.data(),
                  poss.data(), (int)slots.size(), (char*)t1_host + b * seq_t1, cap1);
  }
  if ((st = hip_check(hipStreamSynchronize(stream), "stream sync"))) return st;
  if (link_bytes) *link_bytes = link;
  return TKV_OK;
}

tkv_status tkv_quantize_t2(const tkv_model* model, int32_t batch, const void* k_t0,
                           const void* v_t0, int32_t cap0, const void* k_t1, const void* v_t1,
                           int32_t cap1, const int32_t* src, const int32_t* n_rows,
                           int32_t n_rows_stride, int32_t max_rows, int8_t* codes,
                           float* scales, hipStream_t stream) {
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0 || max_rows < 0) return fail(TKV_ERR_ARG, "negative batch or max_rows");
  if (batch == 0 || max_rows == 0) return TKV_OK;
  if (!k_t0 || !v_t0 || !src || !n_rows || !codes || !scales)
    return fail(TKV_ERR_ARG, "null pointer");
  if (cap1 > 0 && (!k_t1 || !v_t1)) return fail(TKV_ERR_ARG, "null T1 window with cap1 > 0");
  if (n_rows_stride < 1 || cap0 < 0 || cap1 < 0 || cap0 % 32 || cap1 % 32)
    return fail(TKV_ERR_ARG, "bad stride or capacity (cap0, cap1 multiples of 32)");
  if (max_rows > 65535) return fail(TKV_ERR_CAPACITY, "max_rows above 65535");
  if ((st = check_caps(model, batch, cap0, cap1, true))) return st;
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    QuantArgs a{};
    a.k0 = k_t0;
    a.v0 = v_t0;
    a.k1 = k_t1;
    a.v1 = v_t1;
    a.staging = nullptr;
    a.only = 0;
    a.src = src;
    a.n_rows = n_rows;
    a.codes = codes;
    a.scales = scales;
    a.n_rows_stride = n_rows_stride;
    a.max_rows = max_rows;
    a.cap0 = cap0;
    a.cap1 = cap1;
    a.L = model->num_layers;
    a.hkv = model->num_kv_heads;
    a.b_offset = b0;
    fill_pool(a.pool, model, b0, nb, cap0, cap1);
    launch_quantize(a, model->kv_dtype, model->head_dim, nb, stream);
    if ((st = hip_check(hipGetLastError(), "quantize launch"))) return st;
  }
  return TKV_OK;
}

// T2 update workspace, 256-byte aligned regions: holes [B][cap2] | list [B][cap2] int2 | cnt [B]
static size_t t2_ws_list(int batch, int cap2) { return round_up((size_t)batch * cap2 * 4, 256); }
static size_t t2_ws_cnt(int batch, int cap2) {
  return round_up(t2_ws_list(batch, cap2) + (size_t)batch * cap2 * 8, 256);
}

size_t tkv_t2_update_workspace_bytes(int32_t batch, int32_t cap2) {
  if (batch < 0 || cap2 < 0) return 0;
  return round_up(t2_ws_cnt(batch, cap2) + (size_t)batch * 4, 256);
}

tkv_status tkv_t2_update(const tkv_model* model, int32_t batch, const int32_t* ctx_len,
                         int32_t max_ctx, const uint8_t* tier_next, int8_t* k_codes,
                         int8_t* v_codes, float* k_scale, float* v_scale, int32_t* t2_pos,
                         const int32_t* t2_len, int32_t cap2, const int32_t* new_pos,
                         const int8_t* new_codes, const float* new_scales, const int32_t* n_new,
                         int32_t n_new_stride, int32_t max_rows, int32_t* new_t2_len,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  tkv_status st = check_model(model);
  if (st) return st;
  if (batch < 0) return fail(TKV_ERR_ARG, "batch < 0");
  if (batch == 0) return TKV_OK;
  if (!ctx_len || !tier_next || !k_codes || !v_codes || !k_scale || !v_scale || !t2_pos ||
      !t2_len || !new_pos || !n_new || !new_t2_len || !workspace)
    return fail(TKV_ERR_ARG, "null pointer");
  if (max_rows > 0 && (!new_codes || !new_scales))
    return fail(TKV_ERR_ARG, "null new codes or scales with max_rows > 0");
  if (cap2 < 1 || cap2 % 32 || max_ctx < 1 || max_rows < 0 || n_new_stride < 1)
    return fail(TKV_ERR_ARG, "bad capacity, size or stride (cap2 a positive multiple of 32)");
  for (int b = 0; b < batch; ++b) {
    if (ctx_len[b] < 0 || t2_len[b] < 0) return fail(TKV_ERR_ARG, "negative length");
    if (ctx_len[b] > max_ctx || t2_len[b] > cap2)
      return fail(TKV_ERR_CAPACITY, "ctx_len > max_ctx or t2_len > cap2");
  }
  if (workspace_bytes < tkv_t2_update_workspace_bytes(batch, cap2))
    return fail(TKV_ERR_CAPACITY, "workspace too small");
  char* base = (char*)workspace;
  for (int b0 = 0; b0 < batch; b0 += kMaxSeqPerLaunch) {
    const int nb = std::min(kMaxSeqPerLaunch, batch - b0);
    T2ScanArgs a{};
    a.tnext = tier_next;
    a.t2_pos = t2_pos;
    a.new_pos = new_pos;
    a.n_new = n_new;
    a.holes = (int*)base;
    a.list = (int2*)(base + t2_ws_list(batch, cap2));
    a.cnt = (int*)(base + t2_ws_cnt(batch, cap2));
    a.out_len = new_t2_len;
    a.max_ctx = max_ctx;
    a.cap2 = cap2;
    a.max_rows = max_rows;
    a.n_new_stride = n_new_stride;
    a.b_offset = b0;
    for (int i = 0; i < nb; ++i) {
      a.n[i] = ctx_len[b0 + i];
      a.len2[i] = t2_len[b0 + i];
    }
    launch_t2_scan(a, nb, stream);
    if ((st = hip_check(hipGetLastError(), "t2_scan launch"))) return st;
    T2MoveArgs m{};
    m.k2 = k_codes;
    m.v2 = v_codes;
    m.ks2 = k_scale;
    m.vs2 = v_scale;
    m.new_codes = new_codes;
    m.new_scales = new_scales;
    m.list = a.list;
    m.cnt = a.cnt;
    m.cap2 = cap2;
    m.max_rows = max_rows;
    m.lgs = model->num_layers * model->num_kv_heads;
    m.b_offset = b0;
    m.nb = nb;
    launch_t2_move(m, model->head_dim, stream);
    if ((st = hip_check(hipGetLastError(), "t2_move launch"))) return st;
  }
  return TKV_OK;
}

}  // extern "C"
