"""The shared seeded input generator: determinism, formats and workload structure."""
import numpy as np
import torch

from tiered_kv_cache_amd.synth import (SequenceStream, WORKLOADS, bf16_bits_to_f32,
                                       f32_to_bf16_bits)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, 3.4e38, -3.4e38, np.inf, -np.inf,
                                  1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .float().numpy())


def test_streams_are_deterministic_and_independent():
    wl = WORKLOADS["small"]
    a, b = SequenceStream(wl, 0), SequenceStream(wl, 0)
    assert np.array_equal(a.query(5), b.query(5))
    assert not np.array_equal(a.query(5), a.query(6))
    assert np.array_equal(a.new_kv(3)[0], b.new_kv(3)[0])
    assert np.array_equal(a.context_layer(2)[0], b.context_layer(2)[0])
    assert a.query(5).dtype == np.uint16 and a.query(5).shape == (4, 8, 128)


def test_structure_sinks_and_planted():
    wl = WORKLOADS["small"]
    st = SequenceStream(wl, 0)
    pos, tgt = st.planted()
    assert len(pos) == 64 and len(set(pos.tolist())) == 64
    assert pos.min() >= max(wl.prompt, wl.sinks) and pos.max() < wl.ctx[0] - wl.recent
    assert tgt.min() > wl.warmup and tgt.max() <= wl.warmup + wl.steps
    K, _ = st.context_layer(0)
    Kf = bf16_bits_to_f32(K)
    u = st.directions()[0]
    along = np.einsum("gnd,gd->gn", Kf, u)
    assert along[:, :wl.sinks].min() > 15.0                    # sinks: 8 * 3 = 24 along u
    plain = np.delete(along, np.r_[0:wl.sinks, pos], axis=1)
    assert abs(plain.mean()) < 0.2
    # planted keys carry +3 along the unit group-mean query of their target step
    proj = []
    for p, t in zip(pos.tolist(), tgt.tolist()):
        q = bf16_bits_to_f32(st.query(int(t)))[0].reshape(2, 4, 128).mean(axis=1)
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        proj.append(np.einsum("gd,gd->g", Kf[:, p], q))
    assert abs(np.mean(proj) - 3.0) < 0.3


def test_workload_shapes():
    c = WORKLOADS["chain8k"]
    assert (c.layers, c.q_heads, c.kv_heads, c.head_dim, c.ctx, c.batch) == (28, 28, 4, 128, (8192,), 1)
    b = WORKLOADS["batch16"]
    assert len(b.ctx) == 16 and min(b.ctx) >= 1024 and max(b.ctx) <= 8192
    t = WORKLOADS["tiny"]
    assert t.dtype == "f32" and t.delta == 4 and t.total_steps == 16
