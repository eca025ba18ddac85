"""The C ABI (include/tkv.h) on the host: the library loads, exports every declared
entry point, and rejects bad arguments with the documented status before any HIP call
(so these run without a GPU; no compute call is made)."""
import ctypes
import os
import re

import numpy as np
import pytest

from tiered_kv_cache_amd import tkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NULL = None


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "tkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tkv_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return tkv.lib()


def test_exports_every_declared_symbol(L):
    names = declared_symbols()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tkv.EXPORTED)
    assert tkv.tkv_abi_version() == 4 == tkv.ABI_VERSION
    with open(os.path.join(ROOT, "include", "tkv.h")) as f:
        header = re.search(r"#define TKV_ABI_VERSION (\d+)", f.read())
    assert header and int(header.group(1)) == tkv.ABI_VERSION


def model(**kw):
    d = dict(layers=2, q_heads=8, kv_heads=2, head_dim=128, kv_dtype=tkv.TKV_BF16)
    d.update(kw)
    return tkv.make_model(**d)


def policy(**kw):
    d = dict(prompt=4, sinks=2, recent=4, f1=0.3, f2=0.2, f3=0.1, delta=4)
    d.update(kw)
    return tkv.make_policy(**d)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def decode(m, **kw):
    args = dict(batch=1, layer_begin=0, layer_end=m.num_layers, q=FAKE, k_t0=FAKE, v_t0=FAKE,
                t0_len=[10], cap0=32, k_t1=FAKE, v_t1=FAKE, t1_len=[2], cap1=32, out=FAKE,
                alpha=FAKE, alpha_stride=24, t0_pos=FAKE, t1_pos=FAKE, scores=FAKE, max_ctx=64,
                workspace=FAKE, workspace_bytes=1 << 30, stream=0)
    args.update(kw)
    return tkv.tkv_decode_step(m, **args)


def status_of(fn, *a, **kw):
    with pytest.raises(tkv.TkvError) as e:
        fn(*a, **kw)
    return e.value.status


def test_model_validation():
    assert status_of(decode, model(q_heads=7, kv_heads=2)) == tkv.TKV_ERR_ARG
    assert status_of(decode, model(head_dim=96)) == tkv.TKV_ERR_ARG
    assert status_of(decode, model(kv_dtype=7)) == tkv.TKV_ERR_ARG
    assert status_of(decode, model(q_heads=24, kv_heads=2)) == tkv.TKV_ERR_ARG  # group 12
    assert status_of(decode, model(layers=0)) == tkv.TKV_ERR_ARG
    bad = model()
    bad.alpha_scratch = 2
    assert status_of(decode, bad) == tkv.TKV_ERR_ARG


def test_decode_step_validation():
    m = model()
    assert status_of(decode, m, layer_begin=1, layer_end=1) == tkv.TKV_ERR_ARG
    assert status_of(decode, m, layer_end=3) == tkv.TKV_ERR_ARG
    assert status_of(decode, m, q=NULL) == tkv.TKV_ERR_ARG
    assert status_of(decode, m, t0_len=[33]) == tkv.TKV_ERR_CAPACITY
    assert status_of(decode, m, t1_len=[33]) == tkv.TKV_ERR_CAPACITY
    assert status_of(decode, m, cap0=48) == tkv.TKV_ERR_ARG      # tile blocks of 32 slots
    assert status_of(decode, m, alpha_stride=11) == tkv.TKV_ERR_CAPACITY
    assert status_of(decode, m, workspace_bytes=16) == tkv.TKV_ERR_CAPACITY
    assert status_of(decode, m, k_t1=NULL) == tkv.TKV_ERR_ARG
    assert status_of(decode, m, t1_pos=NULL) == tkv.TKV_ERR_ARG
    assert status_of(decode, m, t0_len=[-1]) == tkv.TKV_ERR_ARG
    msg = tkv.lib().tkv_last_error().decode()
    assert "negative" in msg


def test_per_sequence_capacity_validation():
    # tkv_model.t0_caps / t1_caps: multiples of 32 within cap0 / cap1, and each sequence's
    # lengths within its own capacities
    def caps_model(t0, t1):
        return model(t0_caps=t0, t1_caps=t1)
    two = dict(batch=2, t0_len=[10, 40], t1_len=[2, 3], cap0=64, cap1=32, alpha_stride=128)
    assert status_of(decode, caps_model([48, 64], None), **two) == tkv.TKV_ERR_ARG
    assert status_of(decode, caps_model([32, 96], None), **two) == tkv.TKV_ERR_ARG
    assert status_of(decode, caps_model(None, [32, 16]), **two) == tkv.TKV_ERR_ARG
    assert status_of(decode, caps_model([32, 32], None), **two) == tkv.TKV_ERR_CAPACITY  # 40 > 32
    assert status_of(decode, caps_model([64, 64], [0, 32]), **two) == tkv.TKV_ERR_CAPACITY
    # the same layout with fitting capacities gets past the checks to the workspace one
    assert status_of(decode, caps_model([32, 64], [32, 32]), workspace_bytes=16,
                     **two) == tkv.TKV_ERR_CAPACITY
    msg = tkv.lib().tkv_last_error().decode()
    assert "workspace" in msg


def append_decode(m, **kw):
    args = dict(batch=1, k_new=FAKE, v_new=FAKE, position=[10], tier=FAKE, q=FAKE, k_t0=FAKE,
                v_t0=FAKE, t0_len=[10], cap0=32, k_t1=FAKE, v_t1=FAKE, t1_len=[2], cap1=32,
                out=FAKE, alpha=FAKE, alpha_stride=24, t0_pos=FAKE, t1_pos=FAKE, scores=FAKE,
                max_ctx=64, workspace=FAKE, workspace_bytes=1 << 30, stream=0)
    args.update(kw)
    return tkv.tkv_append_decode_step(m, **args)


def test_append_decode_step_validation():
    m = model()
    assert status_of(append_decode, m, t0_len=[32]) == tkv.TKV_ERR_CAPACITY   # no slot left
    assert status_of(append_decode, m, k_new=NULL) == tkv.TKV_ERR_ARG
    assert status_of(append_decode, m, t0_pos=NULL) == tkv.TKV_ERR_ARG
    assert status_of(append_decode, m, position=[-1]) == tkv.TKV_ERR_ARG
    assert status_of(append_decode, m, position=[64]) == tkv.TKV_ERR_CAPACITY
    assert status_of(append_decode, m, alpha_stride=12) == tkv.TKV_ERR_CAPACITY  # 10 + 1 + 2
    assert status_of(append_decode, model(head_dim=96)) == tkv.TKV_ERR_ARG


def test_workspace_size_formula():
    m = model()
    a = tkv.tkv_decode_workspace_bytes(m, 1, 2, 256, 256)
    b = tkv.tkv_decode_workspace_bytes(m, 2, 2, 256, 256)
    assert b > a > 0
    assert tkv.tkv_decode_workspace_bytes(m, -1, 2, 256, 256) == 0


def test_assign_tiers_validation():
    args = dict(batch=1, ctx_len=[10], max_ctx=16, scores=FAKE, tier_prev=FAKE,
                tier_next=FAKE, counts=FAKE, stream=0)
    for bad in (policy(f1=-0.1), policy(f1=0.5, f2=0.4, f3=0.2), policy(delta=0),
                policy(recent=-1)):
        assert status_of(tkv.tkv_assign_tiers, policy=bad, **args) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_assign_tiers, policy=policy(),
                     **{**args, "ctx_len": [17]}) == tkv.TKV_ERR_CAPACITY
    assert status_of(tkv.tkv_assign_tiers, policy=policy(),
                     **{**args, "scores": NULL}) == tkv.TKV_ERR_ARG


def test_compact_and_quant_validation():
    m = model()
    ws = tkv.tkv_compact_workspace_bytes(m, 1, 16, 32, 32)
    args = dict(model=m, batch=1, ctx_len=[10], max_ctx=16, tier_prev=FAKE, tier_next=FAKE + 64,
                k_t0=FAKE, v_t0=FAKE, t0_pos=FAKE, t0_len=[6], cap0=32, k_t1=FAKE, v_t1=FAKE,
                t1_pos=FAKE, t1_len=[3], cap1=32, t2_src=FAKE, t2_pos=FAKE, t2_cap=8,
                t2_codes=FAKE, t2_scales=FAKE, new_lens=FAKE, workspace=FAKE,
                workspace_bytes=ws, stream=0)
    assert ws > 0 and tkv.tkv_compact_workspace_bytes(m, -1, 16, 32, 32) == 0
    assert status_of(tkv.tkv_compact, **{**args, "t0_len": [8]}) == tkv.TKV_ERR_STATE
    assert status_of(tkv.tkv_compact, **{**args, "t1_len": [33], "ctx_len": [40],
                                          "max_ctx": 64}) == tkv.TKV_ERR_CAPACITY
    assert status_of(tkv.tkv_compact, **{**args, "tier_next": FAKE}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_compact, **{**args, "t2_codes": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_compact, **{**args, "t1_pos": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_compact, **{**args, "cap0": 40}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_compact, **{**args, "workspace_bytes": ws - 1}) == \
        tkv.TKV_ERR_CAPACITY
    qargs = dict(model=m, batch=1, k_t0=FAKE, v_t0=FAKE, cap0=32, k_t1=FAKE, v_t1=FAKE, cap1=32,
                 src=FAKE, n_rows=FAKE, n_rows_stride=3, max_rows=4, codes=FAKE, scales=FAKE,
                 stream=0)
    assert status_of(tkv.tkv_quantize_t2, **{**qargs, "src": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_quantize_t2, **{**qargs, "n_rows_stride": 0}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_quantize_t2, **{**qargs, "max_rows": 70000}) == tkv.TKV_ERR_CAPACITY


def t2pool(**kw):
    d = dict(k_codes=FAKE, v_codes=FAKE, k_scale=FAKE, v_scale=FAKE, t2_pos=FAKE, t2_len=[5],
             cap2=32)
    d.update(kw)
    return tkv.T2Pool(**d)


def test_decode_step_t2_validation():
    m = model()

    def call(t2, fused_append=False, **kw):
        if fused_append:
            args = dict(batch=1, k_new=FAKE, v_new=FAKE, position=[10], tier=FAKE, q=FAKE,
                        k_t0=FAKE, v_t0=FAKE, t0_len=[10], cap0=32, k_t1=FAKE, v_t1=FAKE,
                        t1_len=[2], cap1=32, t2=t2, out=FAKE, alpha=FAKE, alpha_stride=24,
                        t0_pos=FAKE, t1_pos=FAKE, scores=FAKE, max_ctx=64, workspace=FAKE,
                        workspace_bytes=1 << 30, stream=0)
            args.update(kw)
            return tkv.tkv_append_decode_step_t2(m, **args)
        args = dict(batch=1, layer_begin=0, layer_end=2, q=FAKE, k_t0=FAKE, v_t0=FAKE,
                    t0_len=[10], cap0=32, k_t1=FAKE, v_t1=FAKE, t1_len=[2], cap1=32, t2=t2,
                    out=FAKE, alpha=FAKE, alpha_stride=24, t0_pos=FAKE, t1_pos=FAKE,
                    scores=FAKE, max_ctx=64, workspace=FAKE, workspace_bytes=1 << 30, stream=0)
        args.update(kw)
        return tkv.tkv_decode_step_t2(m, **args)

    assert status_of(call, None) == tkv.TKV_ERR_ARG                         # pool required
    assert status_of(call, t2pool(t2_len=[33])) == tkv.TKV_ERR_CAPACITY     # > cap2
    assert status_of(call, t2pool(cap2=40)) == tkv.TKV_ERR_ARG              # 32-slot blocks
    assert status_of(call, t2pool(t2_len=[-1])) == tkv.TKV_ERR_ARG
    assert status_of(call, t2pool(k_codes=NULL)) == tkv.TKV_ERR_ARG
    assert status_of(call, t2pool(v_scale=FAKE + 4)) == tkv.TKV_ERR_ARG     # 16-byte aligned
    assert status_of(call, t2pool(t2_pos=NULL)) == tkv.TKV_ERR_ARG          # fused scores
    assert status_of(call, t2pool(t2_len=[13])) == tkv.TKV_ERR_CAPACITY     # stride < 10+2+13
    ws = tkv.tkv_decode_workspace_bytes(m, 1, 2, 32, 32)
    assert status_of(call, t2pool(), alpha_stride=64,
                     workspace_bytes=ws) == tkv.TKV_ERR_CAPACITY            # gsum covers T2
    assert status_of(call, t2pool(), fused_append=True, t0_len=[32]) == tkv.TKV_ERR_CAPACITY
    assert status_of(call, t2pool(t2_len=[12]), fused_append=True) == tkv.TKV_ERR_CAPACITY
    assert status_of(call, None, fused_append=True) == tkv.TKV_ERR_ARG


def test_window_and_streamed_validation():
    m = model()
    wargs = dict(batch=1, layer_begin=1, layer_end=2, q=FAKE, k_t0=FAKE, v_t0=FAKE, t0_len=[10],
                 cap0=32, t1_win=FAKE, t1_len=[2], cap1=32, out=FAKE,
                 alpha=FAKE, alpha_stride=24, t0_pos=FAKE, t1_pos=FAKE, scores=FAKE, max_ctx=64,
                 workspace=FAKE, workspace_bytes=1 << 30, stream=0)
    assert status_of(tkv.tkv_decode_step_window, m, **{**wargs, "t1_win": NULL}) == \
        tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_decode_step_window, m, **{**wargs, "cap1": 48}) == \
        tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_decode_step_window, m, **{**wargs, "layer_end": 3}) == \
        tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_decode_step_window, m, **{**wargs, "t1_len": [40]}) == \
        tkv.TKV_ERR_CAPACITY
    sargs = dict(batch=1, q=FAKE, k_t0=FAKE, v_t0=FAKE, t0_len=[10], cap0=32, host_t1=FAKE,
                 t1_len=[2], cap1=32, win=FAKE, chunk_layers=1, out=FAKE, alpha=FAKE,
                 alpha_stride=24, t0_pos=FAKE, t1_pos=FAKE, scores=FAKE, max_ctx=64,
                 workspace=FAKE, workspace_bytes=1 << 30, stream=0, side_stream=0,
                 events=[FAKE] * 4, side_stream2=None)
    st = tkv.tkv_decode_step_streamed
    assert status_of(st, m, **{**sargs, "host_t1": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(st, m, **{**sargs, "win": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(st, m, **{**sargs, "chunk_layers": 0}) == tkv.TKV_ERR_ARG
    assert status_of(st, m, **{**sargs, "chunk_layers": 3}) == tkv.TKV_ERR_ARG     # > L
    assert status_of(st, m, **{**sargs, "events": [FAKE, NULL, FAKE, FAKE]}) == tkv.TKV_ERR_ARG
    assert status_of(st, m, **{**sargs, "cap1": 40}) == tkv.TKV_ERR_ARG
    # the per-chunk checks run before any event is recorded or copy queued (the fake
    # events would fail a HIP call with another status)
    assert status_of(st, m, **{**sargs, "t0_len": [33]}) == tkv.TKV_ERR_CAPACITY
    assert status_of(st, m, **{**sargs, "alpha_stride": 8}) == tkv.TKV_ERR_CAPACITY
    assert status_of(st, m, **{**sargs, "workspace_bytes": 16}) == tkv.TKV_ERR_CAPACITY
    # the score update covers every layer after the last chunk: its group sums need the
    # workspace of a whole-step call
    ws_chunk = tkv.tkv_decode_workspace_bytes(m, 1, 1, 32, 32)
    assert ws_chunk < tkv.tkv_decode_workspace_bytes(m, 1, 2, 32, 32)
    assert status_of(st, m, **{**sargs, "workspace_bytes": ws_chunk}) == tkv.TKV_ERR_CAPACITY
    big = {**sargs, "batch": 65, "t0_len": [10] * 65, "t1_len": [2] * 65}
    assert status_of(st, m, **big) == tkv.TKV_ERR_CAPACITY                         # > 64


def test_t0_capacity_bounds_the_oracle_assignment():
    # after any reassignment the T0 count stays within tkv_t0_capacity - delta, whatever
    # the scores and the tier history (T2/T3 absorbing), including policies whose
    # protected set exceeds the T0 budget
    from oracle import Policy, assign_tiers
    r = np.random.default_rng(5)
    for case in range(300):
        n = int(r.integers(1, 400))
        pol = Policy(int(r.integers(0, 40)), int(r.integers(0, 8)), int(r.integers(0, 40)),
                     *r.dirichlet([1, 1, 1, 1])[1:].astype(np.float32).tolist(),
                     int(r.integers(1, 9)))
        if sum(np.float32(f) for f in (pol.frac_t1, pol.frac_t2, pol.frac_t3)) > 1:
            continue
        prev = r.choice(4, size=n, p=[0.5, 0.2, 0.2, 0.1]).astype(np.uint8) if case % 2 else \
            np.zeros(n, np.uint8)
        scores = r.choice([0.0, 0.5, 1.0], size=n) if case % 3 == 0 else r.random(n)
        tier, counts = assign_tiers(scores, prev, n, pol)
        tp = tkv.make_policy(pol.prompt, pol.sinks, pol.recent, pol.frac_t1, pol.frac_t2,
                             pol.frac_t3, pol.delta)
        cap = tkv.tkv_t0_capacity(tp, n, n)
        assert cap % 32 == 0 and counts[0] + pol.delta <= cap, (case, counts, cap)
        assert tkv.tkv_t0_capacity(tp, max(0, n - 5), n + 5) >= cap      # a range: the maximum
    # the 7B-class chain after its first reassignment: N0 = n - N1 - N2 - N3 bounds T0
    tp = tkv.make_policy(256, 4, 128, 0.3, 0.15, 0.05, 64)
    n0 = [n - int(np.floor(np.float64(np.float32(0.3)) * n)) - int(np.floor(np.float64(np.float32(0.15)) * n))
          - int(np.floor(np.float64(np.float32(0.05)) * n)) for n in range(8256, 8513)]
    assert tkv.tkv_t0_capacity(tp, 8256, 8512) == -(-(max(n0) + 64) // 32) * 32
    assert tkv.lib().tkv_t0_capacity(ctypes.byref(tp), 10, 5) == -1


def test_compact_host_t1_validation():
    m = model()
    ws = tkv.tkv_compact_host_t1_workspace_bytes(m, 1, 64, 32, 32)
    assert 0 < ws < tkv.tkv_compact_workspace_bytes(m, 1, 64, 32, 32)   # no device row staging
    hs = tkv.tkv_compact_host_t1_scratch_bytes(m, 1, 64, 32)
    # the row staging of the host scratch holds cap1 rows of every (layer, KV head)
    assert hs >= 32 * 2 * 2 * 2 * 128 * 2
    args = dict(model=m, batch=1, ctx_len=[60], max_ctx=64, tier_prev=FAKE, tier_next=FAKE + 64,
                k_t0=FAKE, v_t0=FAKE, t0_pos=FAKE, t0_len=[40], cap0=64, t1_pos=FAKE,
                t1_len=[10], cap1=32, store_k=FAKE, store_v=FAKE, t1_host=FAKE, t2_src=FAKE,
                t2_pos=FAKE, t2_cap=16, t2_codes=FAKE, t2_scales=FAKE, new_lens=FAKE,
                workspace=FAKE, workspace_bytes=ws, host_scratch=FAKE, host_scratch_bytes=hs,
                stream=0)
    call = tkv.tkv_compact_host_t1
    assert status_of(call, **{**args, "store_k": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(call, **{**args, "t1_host": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(call, **{**args, "host_scratch": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(call, **{**args, "tier_next": FAKE}) == tkv.TKV_ERR_ARG     # distinct maps
    assert status_of(call, **{**args, "cap1": 40}) == tkv.TKV_ERR_ARG
    assert status_of(call, **{**args, "t1_len": [33]}) == tkv.TKV_ERR_CAPACITY
    assert status_of(call, **{**args, "t0_len": [55]}) == tkv.TKV_ERR_STATE      # > ctx_len
    assert status_of(call, **{**args, "workspace_bytes": ws - 1}) == tkv.TKV_ERR_CAPACITY
    assert status_of(call, **{**args, "host_scratch_bytes": hs - 1}) == tkv.TKV_ERR_CAPACITY


def test_t2_update_validation():
    m = model()
    ws = tkv.tkv_t2_update_workspace_bytes(2, 64)
    assert ws > tkv.tkv_t2_update_workspace_bytes(1, 64) > 0
    assert tkv.tkv_t2_update_workspace_bytes(-1, 64) == 0
    args = dict(model=m, batch=2, ctx_len=[100, 50], max_ctx=128, tier_next=FAKE, k_codes=FAKE,
                v_codes=FAKE, k_scale=FAKE, v_scale=FAKE, t2_pos=FAKE, t2_len=[10, 0], cap2=64,
                new_pos=FAKE, new_codes=FAKE, new_scales=FAKE, n_new=FAKE, n_new_stride=4,
                max_rows=16, new_t2_len=FAKE, workspace=FAKE, workspace_bytes=ws, stream=0)
    assert status_of(tkv.tkv_t2_update, **{**args, "t2_len": [65, 0]}) == tkv.TKV_ERR_CAPACITY
    assert status_of(tkv.tkv_t2_update, **{**args, "ctx_len": [129, 0]}) == tkv.TKV_ERR_CAPACITY
    assert status_of(tkv.tkv_t2_update, **{**args, "cap2": 48}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_t2_update, **{**args, "n_new_stride": 0}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_t2_update, **{**args, "new_codes": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_t2_update, **{**args, "t2_pos": NULL}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_t2_update, **{**args, "t2_len": [-2, 0]}) == tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_t2_update, **{**args, "workspace_bytes": ws - 1}) == \
        tkv.TKV_ERR_CAPACITY


def test_append_validation():
    m = model()
    args = dict(model=m, batch=1, k_new=FAKE, v_new=FAKE, k_t0=FAKE, v_t0=FAKE, cap0=32,
                t0_len=[32], t0_pos=FAKE, position=[40], scores=FAKE, tier=FAKE, max_ctx=64,
                stream=0)
    assert status_of(tkv.tkv_append, **args) == tkv.TKV_ERR_CAPACITY
    assert status_of(tkv.tkv_append, **{**args, "t0_len": [3], "position": [64]}) == \
        tkv.TKV_ERR_CAPACITY
    assert status_of(tkv.tkv_append, **{**args, "k_new": NULL}) == tkv.TKV_ERR_ARG


def test_gather_host_pack_without_device():
    # position checks (repeats, range, capacity), then a pack-only call (no device
    # pointer -> no HIP call) with positions in window-slot order, not sorted
    m = model(layers=2, kv_heads=2, q_heads=2, head_dim=64)
    r = np.random.default_rng(0)
    max_ctx, cap1 = 40, 32
    hk = r.integers(0, 65535, size=(2, 2, max_ctx, 64)).astype(np.uint16)
    hv = r.integers(0, 65535, size=(2, 2, max_ctx, 64)).astype(np.uint16)
    stg = np.zeros((2, 2, 2, cap1, 64), np.uint16)        # per row: key slots, value slots
    assert status_of(tkv.tkv_gather_t1, m, hk, hv, max_ctx, [3, 2, 3], 3, stg, cap1) == \
        tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_gather_t1, m, hk, hv, max_ctx, [3, 40], 2, stg, cap1) == \
        tkv.TKV_ERR_ARG
    assert status_of(tkv.tkv_gather_t1, m, hk, hv, max_ctx, list(range(33)), 33, stg, cap1) == \
        tkv.TKV_ERR_CAPACITY
    pos = [17, 5, 39, 1, 6]
    tkv.tkv_gather_t1(m, hk, hv, max_ctx, pos, len(pos), stg, cap1)
    sk = stg[:, :, 0].reshape(2, 2, -1)
    sv = stg[:, :, 1].reshape(2, 2, -1)
    # storage order of 32-slot blocks: K-tiles and V-tiles (element-wise definition)
    for r in range(len(pos)):
        for d in range(64):
            jj, u, i = (r % 32) // 8, (r % 32) // 4 % 2, r % 4
            ko = (r // 32) * 32 * 64 + u * 16 * 64 + ((d // 8) * 16 + 4 * jj + i) * 8 + d % 8
            vo = (r // 32) * 32 * 64 + ((d // 16) * 4 + (r % 32) // 8) * 128 + (d % 16) * 8 + r % 8
            assert sk[:, :, ko].tolist() == hk[:, :, pos[r], d].tolist()
            assert sv[:, :, vo].tolist() == hv[:, :, pos[r], d].tolist()
    for r in range(len(pos), 8):                 # the rest of the last value panel is cleared
        vo = [((d // 16) * 4 + r // 8) * 128 + (d % 16) * 8 + r % 8 for d in range(64)]
        assert not sv[:, :, vo].any()


def test_gather_host_pack_blocks_d128():
    # several 32-slot blocks with a ragged last one, head_dim 128: every staged element
    # against the element-wise storage order, padding slots zero
    m = model(layers=3, kv_heads=2, q_heads=4, head_dim=128)
    r = np.random.default_rng(1)
    max_ctx, cap1, D = 300, 96, 128
    hk = r.integers(0, 65535, size=(3, 2, max_ctx, D)).astype(np.uint16)
    hv = r.integers(0, 65535, size=(3, 2, max_ctx, D)).astype(np.uint16)
    stg = np.full((3, 2, 2, cap1, D), 7, np.uint16)
    pos = sorted(r.choice(max_ctx, 77, replace=False).tolist())
    tkv.tkv_gather_t1(m, hk, hv, max_ctx, pos, len(pos), stg, cap1)
    n = len(pos)
    slots = np.arange(96)[:, None]
    d = np.arange(D)[None, :]
    rr = slots % 32
    ko = (slots // 32) * 32 * D + ((rr // 4) % 2) * 16 * D + ((d // 8) * 16 + 4 * (rr // 8) + rr % 4) * 8 + d % 8
    vo = (slots // 32) * 32 * D + ((d // 16) * 4 + rr // 8) * 128 + (d % 16) * 8 + rr % 8
    exp_k = np.zeros((3, 2, 96, D), np.uint16)
    exp_v = np.zeros((3, 2, 96, D), np.uint16)
    exp_k[:, :, :n] = hk[:, :, pos]
    exp_v[:, :, :n] = hv[:, :, pos]
    got_k = stg[:, :, 0].reshape(3, 2, -1)[:, :, ko]
    got_v = stg[:, :, 1].reshape(3, 2, -1)[:, :, vo]
    assert np.array_equal(got_k, exp_k)          # slots past n of the last block cleared
    assert np.array_equal(got_v, exp_v)
