"""Pins of the oracle's decode attention (CPU only).

* A library routine: torch's scaled_dot_product_attention in float64 on the CPU,
  with the KV heads repeated per query group, must give the oracle's output.  This
  pins the logit scale, the softmax and the contiguous grouping g(h) = h // (Hq/Hkv).
* Proposition 1 ("Toutes les pensees n'ont pas besoin de HBM", gist.science, paper
  2605.09490, Methodologie section 3): with T1 at full precision the output depends
  only on the evicted set T3.  With nothing in T2 or T3 the tiered step equals full
  attention over the whole cache, and moving the T0/T1 split at a fixed T3 changes
  nothing.
"""
import math

import numpy as np
import pytest
import torch

from oracle import Policy, TieredSequence, attention, widen
from tiered_kv_cache_amd.synth import SequenceStream, WORKLOADS, f32_to_bf16_bits


def sdpa(q, K, V):
    """Library attention: q [Hq][D], K/V [Hkv][m][D] -> O [Hq][D] (float64, CPU)."""
    q = torch.from_numpy(widen(q))
    K = torch.from_numpy(widen(K))
    V = torch.from_numpy(widen(V))
    g = q.shape[0] // K.shape[0]
    Kr = K.repeat_interleave(g, dim=0).contiguous()
    Vr = V.repeat_interleave(g, dim=0).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], Kr, Vr, attn_mask=None, dropout_p=0.0, is_causal=False)
    return out[:, 0, :].numpy()


@pytest.mark.parametrize("hq,hkv,d,m,bf16", [(2, 2, 64, 37, False), (8, 2, 128, 300, True),
                                              (28, 4, 128, 129, True), (7, 1, 64, 1, True)])
def test_matches_library_sdpa(hq, hkv, d, m, bf16):
    r = np.random.default_rng(1234 + hq + m)
    q = r.standard_normal((hq, d), dtype=np.float32) * 2
    K = r.standard_normal((hkv, m, d), dtype=np.float32)
    V = r.standard_normal((hkv, m, d), dtype=np.float32)
    if bf16:
        q, K, V = f32_to_bf16_bits(q), f32_to_bf16_bits(K), f32_to_bf16_bits(V)
    O, alpha = attention(q, K, V, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(O, sdpa(q, K, V), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(alpha.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    # weight ratios are exp of logit differences (closed form)
    Kf, qf = widen(K), widen(q)
    for h in range(hq):
        z = Kf[h // (hq // hkv)] @ qf[h] / math.sqrt(d)
        np.testing.assert_allclose(np.log(alpha[h] / alpha[h][0]), z - z[0], atol=1e-9)


def test_group_mapping_is_contiguous():
    # Hq=4, Hkv=2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1.
    d, m = 4, 3
    q = np.zeros((4, d))
    K = np.zeros((2, m, d))
    V = np.zeros((2, m, d))
    V[0] = 1.0
    V[1] = 2.0
    O, _ = attention(q, K, V, 1.0)
    np.testing.assert_array_equal(O[:, 0], [1.0, 1.0, 2.0, 2.0])


def _run(wl, f1, f2, f3, steps=None):
    st = SequenceStream(wl, 0)
    K0, V0 = st.context()
    pol = Policy(wl.prompt, wl.sinks, wl.recent, f1, f2, f3, wl.delta)
    seq = TieredSequence(K0, V0, pol, cap=wl.max_ctx)
    outs = []
    for k in range(1, (steps or wl.total_steps) + 1):
        q = st.query(k)
        att_tiers = np.append(seq.tier[:seq.n], 0)       # tiers the attention of step k sees
        O, alpha, pos = seq.step(q, *st.new_kv(k))
        outs.append((O, q, pos, att_tiers))
    return seq, outs


def test_prop1_nothing_evicted_equals_full_attention():
    wl = WORKLOADS["tiny"]                  # 40/60/0/0 variant: T1 non-empty, T2 = T3 = 0
    seq, outs = _run(wl, 0.6, 0.0, 0.0)
    assert (seq.tier[:seq.n] == 1).sum() > 0
    st = SequenceStream(wl, 0)
    K0, V0 = st.context()
    Kall, Vall = [K0], [V0]
    for k, (O, q, pos, tiers) in enumerate(outs, start=1):
        kn, vn = st.new_kv(k)
        Kall.append(kn[:, :, None, :])
        Vall.append(vn[:, :, None, :])
        Kf = np.concatenate(Kall, axis=2)
        Vf = np.concatenate(Vall, axis=2)
        for l in range(wl.layers):
            np.testing.assert_allclose(O[l], sdpa(q[l], Kf[l], Vf[l]), rtol=1e-12, atol=1e-12)


def test_prop1_hbm_split_does_not_matter_at_fixed_eviction():
    wl = WORKLOADS["small"].scaled(ctx=(320,), warmup=0, steps=12, delta=4, prompt=16,
                                   recent=16, sinks=4, planted=(8,))
    runs = [_run(wl, f1, 0.0, 0.1) for f1 in (0.7, 0.5, 0.3)]      # HBM 20/40/60 %, T3 10 %
    n_t1 = [(seq.tier[:seq.n] == 1).sum() for seq, _ in runs]
    assert len(set(n_t1)) == 3                                      # different splits
    base = runs[0][1]
    for _, outs in runs[1:]:
        for (Oa, _, _, ta), (Ob, _, _, tb) in zip(base, outs):
            np.testing.assert_array_equal(ta == 3, tb == 3)          # same evicted set
            np.testing.assert_allclose(Oa, Ob, rtol=1e-12, atol=1e-12)
    # and the output is attention over everything except T3, computed by the library
    seq, outs = runs[1]
    st = SequenceStream(wl, 0)
    K0, V0 = st.context()
    Kall, Vall = [K0], [V0]
    for k, (O, q, pos, tiers) in enumerate(outs, start=1):
        kn, vn = st.new_kv(k)
        Kall.append(kn[:, :, None, :])
        Vall.append(vn[:, :, None, :])
        keep = np.nonzero(tiers != 3)[0]
        Kf = np.concatenate(Kall, axis=2)[:, :, keep]
        Vf = np.concatenate(Vall, axis=2)[:, :, keep]
        for l in range(wl.layers):
            np.testing.assert_allclose(O[l], sdpa(q[l], Kf[l], Vf[l]), rtol=1e-11, atol=1e-11)


def test_t2_t3_rows_are_poisoned_and_never_attended():
    wl = WORKLOADS["tiny"]
    seq, outs = _run(wl, 0.3, 0.2, 0.1)
    t = seq.tier[:seq.n]
    assert (t == 2).any() and (t == 3).any()
    assert np.isnan(widen(seq.K[:, :, np.nonzero(t >= 2)[0]])).all()
    for O, *_ in outs:
        assert np.all(np.isfinite(O))


def _exact_rows(r, shape):
    """Rows of multiples of 2^-7 with |x| <= 127 * 2^-7 and the bound reached in every
    row: the 8-bit format holds them exactly (scale 2^-7, codes the integers)."""
    k = r.integers(-127, 128, size=shape)
    k[..., 0] = np.where(r.random(shape[:-1]) < 0.5, 127, -127)
    return (k / 128.0).astype(np.float32)


def test_attended_t2_exact_rows_equal_full_attention():
    # attend_t2 rebuilds T2 rows from their 8-bit codes; with rows the format holds
    # exactly and nothing evicted, every step must equal full attention over the whole
    # cache (library SDPA), whatever the T0/T1/T2 split
    L, hkv, hq, d, n0 = 2, 2, 4, 64, 48
    r = np.random.default_rng(99)
    K0 = _exact_rows(r, (L, hkv, n0, d))
    V0 = _exact_rows(r, (L, hkv, n0, d))
    pol = Policy(4, 2, 4, 0.25, 0.30, 0.0, 2)
    seq = TieredSequence(K0, V0, pol, cap=64, attend_t2=True)
    Kall, Vall = [K0], [V0]
    seen_t2 = 0
    for step in range(1, 9):
        q = r.standard_normal((L, hq, d)).astype(np.float32)
        kn = _exact_rows(r, (L, hkv, d))
        vn = _exact_rows(r, (L, hkv, d))
        O, alpha, pos = seq.step(q, kn, vn)
        Kall.append(kn[:, :, None, :])
        Vall.append(vn[:, :, None, :])
        Kf = np.concatenate(Kall, axis=2)
        Vf = np.concatenate(Vall, axis=2)
        assert sorted(pos.tolist()) == list(range(seq.n))            # nothing evicted
        for l in range(L):
            np.testing.assert_allclose(O[l], sdpa(q[l], Kf[l], Vf[l]), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(alpha.sum(axis=2), 1.0, atol=1e-12)
        seen_t2 = max(seen_t2, int((seq.tier[:seq.n] == 2).sum()))
    assert seen_t2 > 0                                               # T2 rows were attended


def test_attended_t2_rows_are_the_dequantised_codes():
    # with arbitrary rows, the attended T2 rows are code * scale of the quantiser,
    # not the full-precision rows: the output equals library attention over T0/T1
    # at full precision and T2 rebuilt by hand from quantize_rows
    from oracle import quantize_rows
    L, hkv, hq, d, n0 = 1, 2, 4, 64, 40
    r = np.random.default_rng(5)
    K0 = r.standard_normal((L, hkv, n0, d)).astype(np.float32)
    V0 = r.standard_normal((L, hkv, n0, d)).astype(np.float32)
    pol = Policy(4, 2, 4, 0.2, 0.4, 0.0, 2)
    seq = TieredSequence(K0, V0, pol, cap=48, attend_t2=True)
    Kf, Vf = K0.copy(), V0.copy()
    for step in range(1, 5):
        q = r.standard_normal((L, hq, d)).astype(np.float32)
        kn = r.standard_normal((L, hkv, d)).astype(np.float32)
        vn = r.standard_normal((L, hkv, d)).astype(np.float32)
        tiers_before = seq.tier[:seq.n].copy()
        O, alpha, pos = seq.step(q, kn, vn, reassign=False)
        Kf = np.concatenate([Kf, kn[:, :, None, :]], axis=2)
        Vf = np.concatenate([Vf, vn[:, :, None, :]], axis=2)
        t2 = np.nonzero(tiers_before == 2)[0]
        Kh, Vh = Kf[:, :, pos].astype(np.float64), Vf[:, :, pos].astype(np.float64)
        for j, p in enumerate(pos.tolist()):
            if p in set(t2.tolist()):
                ck, sk = quantize_rows(Kf[:, :, p])
                cv, sv = quantize_rows(Vf[:, :, p])
                Kh[:, :, j] = ck.astype(np.float64) * sk[..., None].astype(np.float64)
                Vh[:, :, j] = cv.astype(np.float64) * sv[..., None].astype(np.float64)
        np.testing.assert_allclose(O[0], sdpa(q[0], Kh[0], Vh[0]), rtol=1e-12, atol=1e-12)
        if step % 2 == 0:
            seq.reassign()
    assert (seq.tier[:seq.n] == 2).sum() > 0
