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


def _two_worker_structure():
    """Prompt P, finished steps A1 (worker 0), B1 (worker 1), A2 (worker 0) in history order;
    unfinished steps A3 (worker 0) and B2 (worker 1). Ids 0..6 = P A1 B1 A2 A3 B2."""
    base = W.make("tiny_fp32")
    P, A1, B1, A2, A3, B2 = range(6)
    lengths = {b: 8 for b in range(6)}
    owners = {P: -1, A1: 0, B1: 1, A2: 0, A3: 0, B2: 1}
    wl = W.Workload(**{**base.__dict__, "history": [P, A1, B1, A2], "inprogress": [A3, B2],
                       "lengths": lengths, "owners": owners})
    return wl, (P, A1, B1, A2, A3, B2)


def test_layout_views_printed_orders():
    # gentlecold.top summary s6 (combined layout; layout table) and s10 (no sync / step-wise /
    # token-wise): the views written out by hand for a two-worker history
    wl, (P, A1, B1, A2, A3, B2) = _two_worker_structure()
    assert wl.views("combined") == [[P, A1, B1, A2, B2, A3], [P, A1, B1, A2, A3, B2]]
    assert wl.views("stepwise") == [[P, A1, B1, A2, A3], [P, A1, B1, A2, B2]]
    assert wl.views("contiguous") == [[P, B1, B2, A1, A2, A3], [P, A1, A2, A3, B1, B2]]
    assert wl.views("nosync") == [[P, A1, A2, A3], [P, B1, B2]]
    assert wl.views() == wl.views("combined")
    with pytest.raises(ValueError):
        wl.views("token")


@pytest.mark.parametrize("name", ["w4_16k", "w8_32k", "tiny_fp32"])
def test_layout_views_properties(name):
    wl = W.make(name, n_layers=1)
    comb = wl.views("combined")
    for layout in ("combined", "stepwise", "contiguous", "nosync"):
        for w, v in enumerate(wl.views(layout)):
            assert len(v) == len(set(v)) and v[-1] == wl.inprogress[w]
            if layout == "contiguous":
                assert sorted(v) == sorted(comb[w])           # same blocks, other order
            if layout in ("stepwise", "nosync"):
                assert set(v) <= set(comb[w])
                assert not set(v) & {wl.inprogress[u] for u in range(wl.n_workers) if u != w}
            if layout == "nosync":
                assert all(wl.owners.get(b, -1) in (-1, w) for b in v)
            if layout == "contiguous":   # each worker's blocks form one span
                owner_seq = [wl.owners.get(b, -1) for b in v]
                spans = [o for i, o in enumerate(owner_seq) if i == 0 or o != owner_seq[i - 1]]
                assert len(spans) == len(set(spans))
