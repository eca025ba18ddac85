"""tkv_compact (the in-place relocation after a reassignment) called directly on
adversarial tier transitions, against expectations computed here from the maps:
shuffled slot orders, mass promotion T1 -> T0 (every promoted row goes through the
staging area), T0 shrinking while T1 fills to capacity, everything leaving for T2/T3,
no change at all, and a sequence whose maps are inconsistent.  Rows are compared
byte for byte by position; the newly-T2 rows against the oracle's quantizer."""
import numpy as np
import pytest
import torch

from oracle import quantize_rows, widen
from tests.parity import say
from tiered_kv_cache_amd import tkv
from tiered_kv_cache_amd.driver import (k_rows_to_tiles, k_tiles_to_rows, to_host_bits,
                                        v_rows_to_tiles, v_tiles_to_rows)

pytestmark = pytest.mark.gpu

L, HKV, HQ = 2, 2, 4
CAP0, CAP1, T2CAP = 704, 320, 256
MAX_CTX = 704


def transitions(rng, kind, n):
    """(tier_prev, tier_next) of one sequence of length n."""
    prev = rng.choice(4, size=n, p=[0.45, 0.3, 0.15, 0.1]).astype(np.uint8)
    # keep the window within its capacity
    t1 = np.nonzero(prev == 1)[0]
    if len(t1) > CAP1 - 40:
        prev[t1[CAP1 - 40:]] = 0
    nxt = prev.copy()
    live = prev <= 1
    if kind == "mixed":
        r = rng.random(n)
        nxt[live & (r < 0.25)] = 0
        nxt[live & (r >= 0.25) & (r < 0.5)] = 1
        nxt[live & (r >= 0.5) & (r < 0.6)] = 2
        nxt[live & (r >= 0.6) & (r < 0.65)] = 3
        nxt[(prev == 2) & (r < 0.3)] = 3
    elif kind == "mass_promotion":          # nearly every T1 row goes to T0
        nxt[prev == 1] = 0
        back = np.nonzero(prev == 0)[0]
        nxt[rng.choice(back, size=min(30, len(back)), replace=False)] = 1
    elif kind == "t1_fills":                # T0 shrinks, T1 filled to capacity
        t0 = np.nonzero(prev == 0)[0]
        room = CAP1 - int((prev == 1).sum())
        nxt[rng.choice(t0, size=min(room, len(t0)), replace=False)] = 1
    elif kind == "all_leave":               # the pool and the window empty out
        nxt[live] = np.where(rng.random(int(live.sum())) < 0.5, 2, 3).astype(np.uint8)
        over = np.nonzero(nxt == 2)[0]
        over = over[prev[over] <= 1]
        nxt[over[T2CAP:]] = 3
    elif kind == "no_change":
        pass
    return prev, nxt


def build_case(rng, lens_n, kinds, dtype):
    B = len(lens_n)
    D = 128 if dtype == torch.bfloat16 else 64
    seqs = []
    for b in range(B):
        n = lens_n[b]
        prev, nxt = transitions(rng, kinds[b], n)
        if dtype == torch.bfloat16:  # finite values: N(0, 1) truncated to bf16 bit patterns
            K = (rng.standard_normal((L, HKV, n, D)).astype(np.float32).view(np.uint32)
                 >> 16).astype(np.uint16)
            V = (rng.standard_normal((L, HKV, n, D)).astype(np.float32).view(np.uint32)
                 >> 16).astype(np.uint16)
        else:
            K = rng.standard_normal((L, HKV, n, D)).astype(np.float32)
            V = rng.standard_normal((L, HKV, n, D)).astype(np.float32)
        p0 = rng.permutation(np.nonzero(prev == 0)[0]).astype(np.int32)
        p1 = rng.permutation(np.nonzero(prev == 1)[0]).astype(np.int32)
        seqs.append(dict(n=n, prev=prev, nxt=nxt, K=K, V=V, p0=p0, p1=p1))
    return seqs, D


def pools(seqs, D, dtype):
    """Device pool / window in tile order with the rows of each slot (garbage past the
    lengths), their slot -> position maps and the tier maps."""
    B = len(seqs)
    rows_t = np.uint16 if dtype == torch.bfloat16 else np.float32
    rng = np.random.default_rng(7)
    out = {}
    for name, cap, key in (("0", CAP0, "p0"), ("1", CAP1, "p1")):
        Kr = rng.integers(0, 1 << 15, size=(B, L, HKV, cap, D)).astype(rows_t)
        Vr = rng.integers(0, 1 << 15, size=(B, L, HKV, cap, D)).astype(rows_t)
        pos = np.full((B, cap), -7, np.int32)
        for b, sq in enumerate(seqs):
            p = sq[key]
            Kr[b, :, :, :len(p)] = sq["K"][:, :, p]
            Vr[b, :, :, :len(p)] = sq["V"][:, :, p]
            pos[b, :len(p)] = p
        kt = k_rows_to_tiles(torch.from_numpy(Kr.view(np.int16) if rows_t == np.uint16 else Kr))
        vt = v_rows_to_tiles(torch.from_numpy(Vr.view(np.int16) if rows_t == np.uint16 else Vr))
        if dtype == torch.bfloat16:
            kt, vt = kt.view(torch.bfloat16), vt.view(torch.bfloat16)
        out["k" + name] = kt.to("cuda")
        out["v" + name] = vt.to("cuda")
        out["pos" + name] = torch.from_numpy(pos).to("cuda")
    tp = np.zeros((B, MAX_CTX), np.uint8)
    tn = np.zeros((B, MAX_CTX), np.uint8)
    for b, sq in enumerate(seqs):
        tp[b, :sq["n"]] = sq["prev"]
        tn[b, :sq["n"]] = sq["nxt"]
    out["tp"] = torch.from_numpy(tp).to("cuda")
    out["tn"] = torch.from_numpy(tn).to("cuda")
    return out


def expected_copies(sq):
    prev, nxt = sq["prev"], sq["nxt"]
    n0, n1 = int((nxt == 0).sum()), int((nxt == 1).sum())
    slot0 = {int(p): s for s, p in enumerate(sq["p0"])}
    slot1 = {int(p): s for s, p in enumerate(sq["p1"])}
    m0 = sum(1 for p in np.nonzero(nxt == 0)[0] if prev[p] == 1 or slot0[int(p)] >= n0)
    m1 = sum(1 for p in np.nonzero(nxt == 1)[0] if prev[p] == 0 or slot1[int(p)] >= n1)
    mp = int(((nxt == 0) & (prev == 1)).sum())
    return m0 + m1 + mp


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16_d128", "f32_d64"])
def test_relocation_adversarial(dtype):
    rng = np.random.default_rng(20261214)
    kinds = ["mixed", "mass_promotion", "t1_fills", "all_leave", "no_change"]
    lens_n = [700, 650, 611, 333, 97]
    seqs, D = build_case(rng, lens_n, kinds, dtype)
    # a sixth sequence whose T0 map lists a T2 position: must be rejected untouched
    bad_seq, _ = build_case(rng, [400], ["mixed"], dtype)
    bad = bad_seq[0]
    t2p = np.nonzero(bad["prev"] == 2)[0]
    bad["p0"] = bad["p0"].copy()
    bad["p0"][0] = t2p[0]
    seqs.append(bad)
    B = len(seqs)
    dev = pools(seqs, D, dtype)
    before = {k: v.clone() for k, v in dev.items()}
    code = tkv.TKV_BF16 if dtype == torch.bfloat16 else tkv.TKV_F32
    model = tkv.make_model(L, HQ, HKV, D, code)
    ws_bytes = tkv.tkv_compact_workspace_bytes(model, B, MAX_CTX, CAP0, CAP1)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    t2_src = torch.zeros((B, T2CAP), dtype=torch.int32, device="cuda")
    t2_pos = torch.zeros((B, T2CAP), dtype=torch.int32, device="cuda")
    codes = torch.zeros((B, T2CAP, L, HKV, 2, D), dtype=torch.int8, device="cuda")
    scales = torch.zeros((B, T2CAP, L, HKV, 2), dtype=torch.float32, device="cuda")
    new_lens = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
    tkv.tkv_compact(model, B, [s["n"] for s in seqs], MAX_CTX, dev["tp"], dev["tn"],
                    dev["k0"], dev["v0"], dev["pos0"], [len(s["p0"]) for s in seqs], CAP0,
                    dev["k1"], dev["v1"], dev["pos1"], [len(s["p1"]) for s in seqs], CAP1,
                    t2_src, t2_pos, T2CAP, codes, scales, new_lens, ws, ws_bytes)
    torch.cuda.synchronize()
    lens = new_lens.cpu().numpy()
    k0 = to_host_bits(k_tiles_to_rows(dev["k0"], CAP0))
    v0 = to_host_bits(v_tiles_to_rows(dev["v0"], CAP0))
    k1 = to_host_bits(k_tiles_to_rows(dev["k1"], CAP1))
    v1 = to_host_bits(v_tiles_to_rows(dev["v1"], CAP1))
    pos0 = dev["pos0"].cpu().numpy()
    pos1 = dev["pos1"].cpu().numpy()
    for b, sq in enumerate(seqs[:-1]):
        prev, nxt = sq["prev"], sq["nxt"]
        n0, n1 = int((nxt == 0).sum()), int((nxt == 1).sum())
        new_t2 = np.nonzero((nxt == 2) & (prev <= 1))[0]
        assert lens[b].tolist() == [n0, n1, len(new_t2), expected_copies(sq)], kinds[b]
        for tier, n_new, pos, kk, vv, old in ((0, n0, pos0, k0, v0, sq["p0"]),
                                               (1, n1, pos1, k1, v1, sq["p1"])):
            got = pos[b, :n_new]
            assert np.array_equal(np.sort(got), np.nonzero(nxt == tier)[0]), (kinds[b], tier)
            assert kk[b][:, :, :n_new].tobytes() == sq["K"][:, :, got].tobytes(), (kinds[b], tier)
            assert vv[b][:, :, :n_new].tobytes() == sq["V"][:, :, got].tobytes(), (kinds[b], tier)
            # rows that keep their tier below the new length keep their slot
            for s, p in enumerate(old[:n_new]):
                if nxt[p] == tier:
                    assert got[s] == p, (kinds[b], tier, s)
        r = len(new_t2)
        assert np.array_equal(t2_pos[b, :r].cpu().numpy(), new_t2), kinds[b]
        if r:
            f = (lambda x: widen(x).astype(np.float32)) if dtype == torch.bfloat16 else \
                (lambda x: x.astype(np.float32))
            ck, sk = quantize_rows(f(sq["K"][:, :, new_t2]))
            cv, sv = quantize_rows(f(sq["V"][:, :, new_t2]))
            ref_codes = np.stack([ck, cv], axis=3).transpose(2, 0, 1, 3, 4)
            ref_scales = np.stack([sk, sv], axis=3).transpose(2, 0, 1, 3)
            assert np.array_equal(codes[b, :r].cpu().numpy(), ref_codes), kinds[b]
            assert np.array_equal(scales[b, :r].cpu().numpy().view(np.uint32),
                                  ref_scales.view(np.uint32)), kinds[b]
    # the inconsistent sequence: reported, and its pool, window and maps untouched
    b = B - 1
    assert lens[b].tolist() == [-1, -1, -1, -1]
    for k in ("k0", "v0", "pos0", "k1", "v1", "pos1"):  # bitwise (garbage slots hold NaN bits)
        assert torch.equal(dev[k][b].contiguous().view(torch.uint8),
                           before[k][b].contiguous().view(torch.uint8)), k
    say(f"[relocation {dtype}] {B - 1} sequences exact, inconsistent one rejected; copies "
        f"{lens[:-1, 3].tolist()}")
