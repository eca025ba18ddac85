"""The T1 gather end to end on the GPU (Methodologie section 1 of "Toutes les pensees
n'ont pas besoin de HBM": T1 stays in host memory at full precision and is brought to
the GPU before the attention step).

tkv_gather_t1 packs a host store's rows, at a shuffled list of positions, into pinned
staging with host threads, copies the staging into a device window on a side stream and
records an event there; the compute stream waits on the event.  The window, read back
and put in row order, must hold exactly the bytes of the oracle's gather of the same
store at the same positions; then one attention call over that window alone
(tkv_decode_step_window, no T0 rows) must match the oracle's attention over those rows.
A second gather into the same staging and window (other positions, fewer rows) checks
that the pack waits for the earlier copy and that the window holds the new rows.
"""
from collections import defaultdict

import numpy as np
import pytest
import torch

from oracle import attention, gather_rows
from tests.parity import check_alpha, check_output, check_scores, say
from tiered_kv_cache_amd import tkv
from tiered_kv_cache_amd.driver import k_tiles_to_rows, to_device, to_host_bits, v_tiles_to_rows
from tiered_kv_cache_amd.synth import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def host_tensor(x: np.ndarray, dtype) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))


@pytest.mark.parametrize("dtype,D,hq,hkv", [("bf16", 128, 8, 2), ("f32", 64, 4, 4)],
                         ids=["bf16_d128_gqa4", "f32_d64"])
def test_gather_t1_end_to_end(dtype, D, hq, hkv):
    L, max_ctx, cap1 = 3, 500, 128
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = tkv.TKV_BF16 if dtype == "bf16" else tkv.TKV_F32
    m = tkv.make_model(L, hq, hkv, D, code)
    r = np.random.default_rng(42)

    def draw(shape):
        x = r.standard_normal(shape, dtype=np.float32)
        return f32_to_bf16_bits(x) if dtype == "bf16" else x

    store_k, store_v = draw((L, hkv, max_ctx, D)), draw((L, hkv, max_ctx, D))
    hk, hv = host_tensor(store_k, tdt), host_tensor(store_v, tdt)
    staging = torch.empty((L, hkv, 2, cap1, D), dtype=tdt, pin_memory=True)
    window = torch.full((1, L, hkv, 2, cap1, D), float("nan"), dtype=tdt, device="cuda")
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    main = torch.cuda.current_stream()
    stats = defaultdict(float)
    for n in (101, 37):                     # a second gather reuses staging and window
        pos = r.choice(max_ctx, n, replace=False).astype(np.int64)   # window-slot order
        say(f"[gather {dtype} D{D}] n = {n}")
        tkv.tkv_gather_t1(m, hk, hv, max_ctx, pos, n, staging, cap1, window, side, ready)
        main.wait_event(ready)
        k_rows = to_host_bits(k_tiles_to_rows(window[0, :, :, 0], n))
        v_rows = to_host_bits(v_tiles_to_rows(window[0, :, :, 1], n))
        assert k_rows.tobytes() == gather_rows(store_k, pos).tobytes(), "window keys"
        assert v_rows.tobytes() == gather_rows(store_v, pos).tobytes(), "window values"

        # one attention call over that window alone (T0 empty)
        q = draw((1, L, hq, D))
        qd = to_device(q, tdt, "cuda")
        k0 = torch.zeros((1, L, hkv, 32, D), dtype=tdt, device="cuda")
        t0_pos = torch.zeros((1, 32), dtype=torch.int32, device="cuda")
        t1_pos = torch.zeros((1, cap1), dtype=torch.int32, device="cuda")
        t1_pos[0, :n] = torch.from_numpy(pos.astype(np.int32))
        scores = torch.zeros((1, max_ctx), dtype=torch.float32, device="cuda")
        stride = 32 + cap1
        out = torch.full((1, L, hq, D), float("nan"), dtype=torch.float32, device="cuda")
        alpha = torch.zeros((1, L, hq, stride), dtype=torch.float32, device="cuda")
        ws_bytes = tkv.tkv_decode_workspace_bytes(m, 1, L, 32, cap1)
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        tkv.tkv_decode_step_window(m, 1, 0, L, qd, k0, k0, [0], 32, window, [n], cap1, out,
                                   alpha, stride, t0_pos, t1_pos, scores, max_ctx, ws, ws_bytes)
        torch.cuda.synchronize()
        o = out[0].cpu().numpy()
        a = alpha[0, :, :, :n].cpu().numpy()
        inc = np.zeros(max_ctx)
        K, V = gather_rows(store_k, pos), gather_rows(store_v, pos)
        for l in range(L):
            O, al = attention(q[0][l], K[l], V[l], 1.0 / np.sqrt(D))
            check_output(o[l], O, stats)
            check_alpha(a[l], al, stats)
            inc[pos] += al.sum(axis=0)
        check_scores(scores[0].cpu().numpy(), inc / (L * hq), stats)
    say(f"[gather {dtype} D{D}] ok: " + ", ".join(f"{k}={v:.3g}" for k, v in sorted(stats.items())))
