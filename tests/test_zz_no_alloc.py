"""tkv_decode_step_noalloc (workspace inside the library, for callers that cannot
allocate) against tkv_decode_step with a caller workspace, through the C ABI: the same
kernels on the same inputs give the same bits (output, weights, scores).  Two calls in a
row, the second with a smaller input, so the second runs on the scratch contents the
first left behind; then a call whose workspace would exceed the library's array is
rejected before anything is queued.  The first call's two sequences have pools of their
own capacities (tkv_model.t0_caps / t1_caps)."""
import pytest
import torch

from tests.parity import say
from tiered_kv_cache_amd import tkv
from tiered_kv_cache_amd.synth import WORKLOADS
from tiered_kv_cache_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu


def one_call(wl, per_sequence=False):
    dw = DeviceWorkload(wl)
    cache = dw.make_cache(per_sequence=per_sequence)
    cache.reassign()                       # T0 and T1 both populated
    qd, _, _ = dw.device_step(1)
    B = wl.batch
    s0 = cache.scores.clone()
    tkv.tkv_decode_step(cache.model, B, 0, wl.layers, qd, cache.k_t0, cache.v_t0, cache.t0_len,
                        cache.cap0, cache.k_t1, cache.v_t1, cache.t1_len, cache.cap1, cache.out,
                        cache.alpha, cache.alpha_stride, cache.t0_pos, cache.t1_pos,
                        cache.scores, cache.max_ctx, cache.ws, cache.ws_bytes)
    torch.cuda.synchronize()
    ref = (cache.out.clone(), cache.alpha.clone(), cache.scores.clone())
    cache.scores.copy_(s0)
    cache.out.fill_(float("nan"))
    cache.alpha.fill_(float("nan"))
    tkv.tkv_decode_step_noalloc(cache.model, B, 0, wl.layers, qd, cache.k_t0, cache.v_t0,
                                cache.t0_len, cache.cap0, cache.k_t1, cache.v_t1, cache.t1_len,
                                cache.cap1, cache.out, cache.alpha, cache.alpha_stride,
                                cache.t0_pos, cache.t1_pos, cache.scores, cache.max_ctx)
    torch.cuda.synchronize()
    assert torch.equal(cache.out, ref[0]), "output"
    for b in range(B):
        m = cache.t0_len[b] + cache.t1_len[b]
        assert torch.equal(cache.alpha[b, :, :, :m], ref[1][b, :, :, :m]), f"weights, sequence {b}"
    assert torch.equal(cache.scores, ref[2]), "scores"
    return sum(cache.t0_len) + sum(cache.t1_len)


def test_noalloc_matches_the_workspace_call_twice():
    big = WORKLOADS["small"].scaled(name="noalloc_big", batch=2, ctx=(2048, 1500),
                                    planted=(8, 6), warmup=0, steps=1, delta=1)
    small = WORKLOADS["small"].scaled(name="noalloc_small", layers=2, batch=1, ctx=(300,),
                                      planted=(2,), warmup=0, steps=1, delta=1)
    n1 = one_call(big, per_sequence=True)
    n2 = one_call(small)
    assert n2 < n1
    say(f"[noalloc] identical bits on two calls ({n1} then {n2} attended rows)")


def test_noalloc_rejects_a_call_above_its_array():
    # 16 sequences of 32K-token capacity, 32 layers x 8 KV heads: far above 64 MiB
    m = tkv.make_model(32, 32, 8, 128, tkv.TKV_BF16)
    assert tkv.tkv_decode_workspace_bytes(m, 16, 32, 32768, 16384) > 64 << 20
    with pytest.raises(tkv.TkvError) as e:
        tkv.tkv_decode_step_noalloc(m, 16, 0, 32, 0x1000, 0x1000, 0x1000, [10] * 16, 32768,
                                    0x1000, 0x1000, [2] * 16, 16384, 0x1000, 0x1000, 64,
                                    0x1000, 0x1000, 0x1000, 40000)
    assert e.value.status == tkv.TKV_ERR_CAPACITY
