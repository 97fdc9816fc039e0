"""The seeded synthetic workloads: determinism and the configurations' structure."""

import numpy as np
import pytest

from oracle import hogwild_oracle as O
from shared_kv_cache_amd import workloads as W


@pytest.mark.parametrize("name", W.CONFIGS)
def test_views_follow_the_combined_layout(name):
    wl = W.make(name, n_layers=1)
    for w, view in enumerate(wl.views()):
        assert view == O.canonical_view(w, wl.history, wl.inprogress)


def test_structure_of_each_config():
    t = W.make("tiny_fp32")
    assert (t.n_workers, t.n_q_heads, t.n_kv_heads, t.head_dim, t.kv_dtype) == (2, 4, 2, 64, "f32")
    assert [t.lengths[b] for b in t.blocks()] == [256, 32, 27] and t.seed == 0

    c2 = W.make("w2_4k")
    assert [c2.lengths[b] for b in c2.blocks()] == [4096, 256, 193] and c2.value_scale == 0.5

    c3 = W.make("w4_16k")
    hist = [c3.lengths[b] for b in c3.history]
    assert hist[0] == 8192 and sum(hist[1:]) == 8192 and c3.n_layers == 64
    assert all(64 <= x <= 512 for x in hist[1:-1]) and 1 <= hist[-1] <= 512
    assert all(1 <= c3.lengths[b] <= 512 for b in c3.inprogress)
    owners = [c3.owners[b] for b in c3.history[1:]]
    assert owners == [i % 4 for i in range(len(owners))]
    offs = [O.default_offsets(v, c3.lengths) for v in c3.views()]
    assert len({tuple(o[-4:]) for o in offs}) > 1          # workers' offsets differ

    c4 = W.make("w8_32k")
    assert c4.lengths[0] == 32768 and c4.page_seed != 0
    assert all(1 <= c4.lengths[b] <= 1024 for b in c4.inprogress)
    assert c4.n_pages >= 2 * (32768 // 256)

    c5 = W.make("w4_128k_sinks", n_layers=1)
    assert c5.lengths[0] == 131072 and c5.sink == (7, 4, 8.0)


def test_draws_are_seeded_per_tensor_and_bf16_exact():
    a = W.make("w2_4k", n_layers=2)
    b = W.make("w2_4k", n_layers=2)
    ka, va = a.kv(1, a.inprogress[1])
    kb, vb = b.kv(1, b.inprogress[1])
    np.testing.assert_array_equal(ka, kb)
    np.testing.assert_array_equal(va, vb)
    k0, _ = a.kv(0, a.inprogress[1])
    assert not np.array_equal(k0, ka)
    np.testing.assert_array_equal(W.round_to_bf16_values(ka), ka)
    assert np.array_equal(a.q(0), b.q(0)) and not np.array_equal(a.q(0), a.q(1))
    sk, sv = a.step_kv(0, 1)
    assert sk.shape == (2, 8, 128) and not np.array_equal(sk, a.step_kv(0, 2)[0])


def test_sink_keys_scaled():
    c5 = W.make("w4_128k_sinks", n_layers=1)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([c5.seed, 0, 1])))
    raw = rng.standard_normal((8, 8, 128), dtype=np.float32)
    k, _ = c5.kv(0, 0, length=8)
    np.testing.assert_array_equal(k[:4, 7], W.round_to_bf16_values(raw[:4, 7] * 8))
    np.testing.assert_array_equal(k[4:, 7], W.round_to_bf16_values(raw[4:, 7]))
    np.testing.assert_array_equal(k[:, :7], W.round_to_bf16_values(raw[:, :7]))
