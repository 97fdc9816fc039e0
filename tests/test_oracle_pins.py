"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with the GPU path. Each test pins the oracle
to something other than itself: printed worked examples (tests/golden/),
closed forms, an independently written re-encoding brute force, textbook
single-sequence causal decode in complex form plus torch's SDPA, invariants,
and a mutation check showing that plausible slips in the oracle fail a pin.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import hogwild_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, n_workers=3, hq=4, hkv=2, d=8, max_len=6, gaps=False):
    """Random tiny multi-worker case with one history block and per-worker blocks."""
    n_hist = 2
    history = list(range(n_hist))
    inprog = [n_hist + w for w in range(n_workers)]
    blocks = {}
    for b in history + inprog:
        n = int(rng.integers(1 if b == inprog[0] else 0, max_len + 1))
        if b == history[0]:
            n = max(n, 1)
        blocks[b] = (rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d)))
    views = [O.canonical_view(w, history, inprog) for w in range(n_workers)]
    lengths = {b: kv[0].shape[0] for b, kv in blocks.items()}
    offsets = None
    if gaps:
        offsets = []
        for v in views:
            off, acc = [], int(rng.integers(0, 3))
            for b in v:
                off.append(acc)
                acc += lengths[b] + int(rng.integers(0, 4))
            offsets.append(off)
    q = rng.standard_normal((n_workers, hq, d))
    return q, blocks, views, offsets


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


# ---------------------------------------------------------------- RoPE pins

def test_rope_known_answers_pairing_frequency_sign():
    """d = 4, theta = 1e4: closed-form scores fix the pairing (j, j+d/2), the
    frequency ladder theta^(-2j/d) and the direction of rotation."""
    d, theta = 4, 1e4
    e = np.eye(d)
    iq, ik = 5, 2

    def score(qv, kv):
        return float(O.rope(qv, iq, theta) @ O.rope(kv, ik, theta))

    assert score(e[0], e[0]) == pytest.approx(math.cos(3.0), abs=1e-15)
    assert score(e[1], e[1]) == pytest.approx(math.cos(3.0 * 0.01), abs=1e-15)
    # partner of component 0 is component d/2 = 2; rho(q,iq).rho(k,ik) = q R(ik-iq) k
    assert score(e[0], e[2]) == pytest.approx(math.sin(3.0), abs=1e-15)
    assert score(e[2], e[0]) == pytest.approx(-math.sin(3.0), abs=1e-15)
    assert score(e[0], e[1]) == 0.0 and score(e[0], e[3]) == 0.0


def test_rope_relative_position_and_isometry():
    """Scores depend only on the position difference, and rho preserves norms
    (Hogwild! summary s5; ocdem.com article s2.2: R(D)q.R(D)k = q.k)."""
    rng = np.random.default_rng(1)
    for d in (2, 8, 64, 128):
        q, k = rng.standard_normal(d), rng.standard_normal(d)
        for a, b, c in [(7, 3, 11), (100, 0, 2500), (131071, 5, -5), (0, 0, 999)]:
            s1 = O.rope(q, a, 1e4) @ O.rope(k, b, 1e4)
            s2 = O.rope(q, a + c, 1e4) @ O.rope(k, b + c, 1e4)
            s3 = O.rope(q, a - b, 1e4) @ k
            # fp64 angles carry an absolute error ~ position * 2^-53 per term
            tol = 1e-12 + 4e-16 * max(abs(a), abs(b), abs(a + c), abs(b + c)) * (
                np.linalg.norm(q) * np.linalg.norm(k))
            assert abs(s1 - s2) <= tol
            assert abs(s1 - s3) <= tol
        assert np.linalg.norm(O.rope(q, 12345, 1e4)) == pytest.approx(np.linalg.norm(q), rel=1e-14)
        assert np.array_equal(O.rope(q, 0, 1e4), q)   # Delta = 0 gives the identity


# ----------------------------------------------------------- identity (s5)

def _query_rotation_form(q, blocks, views, offsets, q_pos, theta):
    """Right-hand side of the concatenation identity, written with dense
    rotation matrices: keys stay at local positions; the query is rotated by
    q_pos - offset once per block; one softmax over all blocks."""
    n_workers, hq, d = q.shape
    lengths = {b: kv[0].shape[0] for b, kv in blocks.items()}
    hkv = next(iter(blocks.values()))[0].shape[1]
    group = hq // hkv
    out = np.zeros_like(q)
    for w in range(n_workers):
        offs = offsets[w] if offsets else O.default_offsets(views[w], lengths)
        qp = q_pos[w] if q_pos else O.default_q_pos(views[w], offs, lengths)
        for h in range(hq):
            g = h // group
            scores, vals = [], []
            for b, off in zip(views[w], offs):
                kb, vb = blocks[b]
                q_b = O._rotation_matrix(qp - off, d, theta) @ q[w, h]
                for j in range(lengths[b]):
                    k_local = O._rotation_matrix(j, d, theta) @ kb[j, g]
                    scores.append(q_b @ k_local / math.sqrt(d))
                    vals.append(vb[j, g])
            s = np.array(scores)
            p = np.exp(s - s.max())
            out[w, h] = p @ np.array(vals) / p.sum()
    return out


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("gaps", [False, True])
def test_concatenation_identity(seed, gaps):
    """Attention with keys re-rotated to their view positions equals attention
    with block-local keys and a per-block rotated query (summary s5)."""
    rng = np.random.default_rng(seed)
    q, blocks, views, offsets = _rand_case(rng, gaps=gaps)
    ref, _ = O.concurrent_attention(q, blocks, views, offsets=offsets)
    rhs = _query_rotation_form(q, blocks, views, offsets, None, 1e4)
    assert _rel(ref, rhs) <= 1e-12


# ------------------------------------------------------ brute force (s4, s9)

@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("gaps", [False, True])
def test_reencode_bruteforce(seed, gaps):
    rng = np.random.default_rng(100 + seed)
    q, blocks, views, offsets = _rand_case(rng, n_workers=2 + seed % 3, gaps=gaps)
    q_pos = None
    if gaps:  # query one past the last key (allowed: q_pos >= every key position)
        lengths = {b: kv[0].shape[0] for b, kv in blocks.items()}
        q_pos = [offsets[w][-1] + lengths[v[-1]] + 1 for w, v in enumerate(views)]
    ref, lse = O.concurrent_attention(q, blocks, views, offsets=offsets, q_pos=q_pos)
    bf, bf_lse = O.reencode_bruteforce(q, blocks, views, offsets=offsets, q_pos=q_pos)
    assert _rel(ref, bf) <= 1e-12
    assert np.max(np.abs(lse - bf_lse)) <= 1e-12


# --------------------------------------------- one worker = causal decode

@pytest.mark.parametrize("seed", range(3))
def test_one_worker_is_ordinary_causal_decode(seed):
    rng = np.random.default_rng(200 + seed)
    hq, hkv, d = 6, 2, 16
    n_common, n_own = 9 + seed, 4 + seed
    kc, vc = rng.standard_normal((n_common, hkv, d)), rng.standard_normal((n_common, hkv, d))
    ko, vo = rng.standard_normal((n_own, hkv, d)), rng.standard_normal((n_own, hkv, d))
    q = rng.standard_normal((1, hq, d))
    blocks = {10: (kc, vc), 20: (ko, vo)}
    views = [O.canonical_view(0, [10], [20])]
    assert views == [[10, 20]]
    out, lse = O.concurrent_attention(q, blocks, views)
    k_seq, v_seq = np.concatenate([kc, ko]), np.concatenate([vc, vo])
    tb_out, tb_lse = O.causal_decode_textbook(q[0], k_seq, v_seq)
    assert _rel(out[0], tb_out) <= 1e-12
    assert np.max(np.abs(lse[0] - tb_lse)) <= 1e-12

    # and against torch's SDPA (fp64, CPU) with an explicit causal mask
    t = n_common + n_own
    ang = np.arange(t)[:, None] * np.array([1e4 ** (-(2.0 * j) / d) for j in range(d // 2)])
    zk = (k_seq[..., :d // 2] + 1j * k_seq[..., d // 2:]) * np.exp(1j * ang)[:, None, :]
    k_rot = np.concatenate([zk.real, zk.imag], axis=-1)                    # [T, Hkv, D]
    zq = (q[0, :, :d // 2] + 1j * q[0, :, d // 2:]) * np.exp(1j * ang[-1])[None, :]
    q_rot = np.concatenate([zq.real, zq.imag], axis=-1)                    # [Hq, D]
    kq = torch.from_numpy(np.repeat(k_rot, hq // hkv, axis=1)).permute(1, 0, 2)   # [Hq, T, D]
    vq = torch.from_numpy(np.repeat(v_seq, hq // hkv, axis=1)).permute(1, 0, 2)
    qq = torch.from_numpy(np.repeat(q_rot[:, None, :], t, axis=1))               # all rows
    mask = torch.ones(t, t, dtype=torch.bool).tril()
    sdpa = torch.nn.functional.scaled_dot_product_attention(qq, kq.contiguous(), vq.contiguous(),
                                                            attn_mask=mask)
    assert _rel(out[0], sdpa[:, -1, :].numpy()) <= 1e-12


# ------------------------------------------------------------ closed forms

def test_closed_forms():
    rng = np.random.default_rng(7)
    q, blocks, views, offsets = _rand_case(rng, n_workers=3)
    lengths = {b: kv[0].shape[0] for b, kv in blocks.items()}
    # K = 0: uniform weights -> mean of the view's values; lse = log T
    zero_k = {b: (np.zeros_like(k), v) for b, (k, v) in blocks.items()}
    out, lse = O.concurrent_attention(q, zero_k, views)
    for w, view in enumerate(views):
        vals = np.concatenate([blocks[b][1] for b in view])
        t = sum(lengths[b] for b in view)
        for h in range(q.shape[1]):
            g = h // (q.shape[1] // vals.shape[1])
            np.testing.assert_allclose(out[w, h], vals[:, g].mean(axis=0), rtol=0, atol=1e-14)
            assert lse[w, h] == pytest.approx(math.log(t), abs=1e-14)
    # q = 0: same
    out0, _ = O.concurrent_attention(np.zeros_like(q), blocks, views)
    np.testing.assert_allclose(out0, out, rtol=0, atol=1e-14)
    # a view of one token: out = v, lse = score
    one = {0: (rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 2, 8)))}
    o1, l1 = O.concurrent_attention(q[:1], one, [[0]])
    for h in range(4):
        np.testing.assert_array_equal(o1[0, h], one[0][1][0, h // 2])
        assert l1[0, h] == pytest.approx(float(q[0, h] @ one[0][0][0, h // 2]) / math.sqrt(8), abs=1e-13)


def test_shift_and_order_invariance():
    rng = np.random.default_rng(8)
    q, blocks, views, offsets = _rand_case(rng, gaps=True)
    base, lse = O.concurrent_attention(q, blocks, views, offsets=offsets)
    shifted = [[o + 1000 for o in offs] for offs in offsets]
    lengths = {b: kv[0].shape[0] for b, kv in blocks.items()}
    q_pos = [O.default_q_pos(v, offsets[w], lengths) + 1000 for w, v in enumerate(views)]
    out, lse2 = O.concurrent_attention(q, blocks, views, offsets=shifted, q_pos=q_pos)
    assert _rel(out, base) <= 1e-12
    # listing a view's blocks in another order with the same offsets changes nothing
    rev_views = [list(reversed(v)) for v in views]
    rev_offs = [list(reversed(o)) for o in offsets]
    q_pos0 = [O.default_q_pos(v, offsets[w], lengths) for w, v in enumerate(views)]
    out3, _ = O.concurrent_attention(q, blocks, rev_views, offsets=rev_offs, q_pos=q_pos0)
    assert _rel(out3, base) <= 1e-12


def test_view_error_cases():
    L = {0: 4, 1: 3, 2: 2}
    assert O.view_error([0, 1, 2], [0, 4, 7], L, 8) is None
    assert O.view_error([0, 1, 2], [0, 3, 7], L, 8) == "overlapping blocks"
    assert O.view_error([0, 1, 2], [0, 4, 7], L, 7) == "key after query"
    assert O.view_error([0, 1, 2], [0, 10, 20], L, 21) is None        # gaps allowed
    assert O.view_error([0, 0], [0, 4], L, 9) == "block repeated in view"
    assert O.view_error([0, 1], [0, 4], {0: 4, 1: 0}, 3) is None      # empty block
    with pytest.raises(ValueError):
        O.concurrent_attention(np.zeros((1, 2, 4)),
                               {0: (np.zeros((2, 1, 4)), np.zeros((2, 1, 4)))},
                               [[0]], q_pos=[0])


# --------------------------------------------------------- golden fixtures

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_kv_bytes_worked_examples():
    rows = _golden("kv_bytes_p5.txt")
    assert len(rows) == 5
    for ln in rows:
        s, b, gib = ln.split()
        got = O.kv_cache_bytes(32, 32, int(s), int(b), 128, 2)
        assert got == float(gib) * 2 ** 30


def test_view_orders_printed_examples():
    rows = _golden("view_orders_p1.txt")
    assert len(rows) >= 2
    for ln in rows:
        hist, cur, rest = [x.strip() for x in ln.split("|")]
        worker, expect = [x.strip() for x in rest.split(":")]
        got = O.canonical_view(int(worker), hist.split(), cur.split())
        assert got == expect.split(), ln


def test_commit_step_moves_block_to_history_end():
    hist, cur = O.commit_step_views(["C", "H1"], ["A", "B"], 1, "B2")
    assert hist == ["C", "H1", "B"] and cur == ["A", "B2"]
    assert O.canonical_view(0, hist, cur) == ["C", "H1", "B", "B2", "A"]


# ------------------------------------------------------ stored-key reference

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        # exact ties between two bf16 values, both parities
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], np.float32)])
    ours = O.bf16_bits_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_rope_store_reference_within_rounding_of_fp64(kv_dtype):
    rng = np.random.default_rng(10)
    k = rng.standard_normal((64, 2, 128)).astype(np.float32)
    pos = rng.integers(0, 140000, size=64)
    got = O.rope_store_reference(k, pos, 1e4, kv_dtype)
    got = O.bf16_bits_to_f32(got) if kv_dtype == "bf16" else got
    exact = O.rope(k.astype(np.float64), pos[:, None], 1e4)
    err = np.abs(got - exact)
    bound = (2.0 ** -8 if kv_dtype == "bf16" else 2.0 ** -22) * (np.abs(exact) + 1e-3) + 4e-7 * 4
    assert np.all(err <= bound)


# ----------------------------------------------------------- mutation check

def _pin_suite():
    """A compact run of the pins above; returns the names of those that fail."""
    failed = []
    checks = {
        "known_answers": test_rope_known_answers_pairing_frequency_sign,
        "identity": lambda: test_concatenation_identity(0, True),
        "bruteforce": lambda: test_reencode_bruteforce(1, False),
        "textbook": lambda: test_one_worker_is_ordinary_causal_decode(0),
        "closed_forms": test_closed_forms,
        "views": test_view_orders_printed_examples,
    }
    for name, fn in checks.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


def _mut_rope_interleaved(x, pos, theta):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, np.float64)[..., None] * O.rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = a * c - b * s, b * c + a * s
    return out


def _mut_rope_sign(x, pos, theta):
    return _ORIG_ROPE(x, -np.asarray(pos, np.float64), theta)


def _mut_inv_freq(d, theta):
    return np.array([math.pow(theta, -j / d) for j in range(d // 2)])


def _mut_view_own_first(worker, history, inprogress):
    others = [inprogress[u] for u in range(len(inprogress)) if u != worker]
    return list(history) + [inprogress[worker]] + others


def _mut_view_descending(worker, history, inprogress):
    others = [inprogress[u] for u in range(len(inprogress)) if u != worker]
    return list(history) + others[::-1] + [inprogress[worker]]


def _mut_qpos(view, offsets, lengths):
    return offsets[-1] + lengths[view[-1]]


_ORIG_ROPE = O.rope
_ORIG_CA = O.concurrent_attention


def _mut_no_scale(q, blocks, views, offsets=None, q_pos=None, theta=1e4, scale=None, heads=None):
    return _ORIG_CA(q, blocks, views, offsets, q_pos, theta, 1.0, heads)


def _mut_gqa_modulo(q, blocks, views, offsets=None, q_pos=None, theta=1e4, scale=None, heads=None):
    hq = q.shape[1]
    hkv = next(iter(blocks.values()))[0].shape[1]
    g = hq // hkv
    perm = [(h % hkv) * g + h // hkv for h in range(hq)]   # head h read as head perm[h]
    out, lse = _ORIG_CA(np.asarray(q)[:, np.argsort(perm)], blocks, views, offsets, q_pos,
                        theta, scale, None)
    return out[:, perm], lse[:, perm]


@pytest.mark.parametrize("target,mutant", [
    ("rope", _mut_rope_interleaved),
    ("rope", _mut_rope_sign),
    ("rope_inv_freq", _mut_inv_freq),
    ("canonical_view", _mut_view_own_first),
    ("canonical_view", _mut_view_descending),
    ("default_q_pos", _mut_qpos),
    ("concurrent_attention", _mut_no_scale),
    ("concurrent_attention", _mut_gqa_modulo),
])
def test_planted_oracle_mistakes_fail_a_pin(monkeypatch, target, mutant):
    assert _pin_suite() == []
    monkeypatch.setattr(O, target, mutant)
    assert _pin_suite() != [], f"mutant {mutant.__name__} of {target} passed every pin"


# ------------------------------------------- several query tokens per worker

def _truncated_case(q_tok, blocks, views, offsets, pos):
    """The one-token problem of a token at position pos[w]: every block of every view cut
    down to its keys at or before pos[w] (new block ids, explicit offsets kept)."""
    new_blocks, new_views, new_offs = {}, [], []
    for w, view in enumerate(views):
        v2, o2 = [], []
        for b, off in zip(view, offsets[w]):
            k, v = blocks[b]
            keep = max(0, min(len(k), pos[w] - off + 1))
            nb = (w, b)
            new_blocks[nb] = (k[:keep], v[:keep])
            v2.append(nb)
            o2.append(off)
        new_views.append(v2)
        new_offs.append(o2)
    return new_blocks, new_views, new_offs


@pytest.mark.parametrize("seed", range(4))
def test_several_tokens_equal_one_token_problems_cut_at_each_token(seed):
    # [P1] s8 step 4: a fresh block starts with a paragraph header, several tokens
    # processed at once. Token t (position q_pos - (n_new - 1 - t)) must equal the
    # one-token oracle over the views cut at its position: a different code path (cut
    # blocks instead of a mask), so a wrong shift, sign or mask edge fails here.
    rng = np.random.default_rng(500 + seed)
    q1, blocks, views, _ = _rand_case(rng, n_workers=3)
    n_new = 1 + seed
    # grow each worker's own (last) block so that it holds the n_new tokens
    for w, view in enumerate(views):
        b = view[-1]
        k, v = blocks[b]
        extra = max(0, n_new - len(k))
        if extra:
            blocks[b] = (np.concatenate([k, rng.standard_normal((extra,) + k.shape[1:])]),
                         np.concatenate([v, rng.standard_normal((extra,) + v.shape[1:])]))
    lengths = {b: len(kv[0]) for b, kv in blocks.items()}
    offsets = []
    for v in views:   # running sums, with random gaps for odd seeds
        off, acc = [], int(rng.integers(0, 3)) if seed % 2 else 0
        for b in v:
            off.append(acc)
            acc += lengths[b] + (int(rng.integers(0, 4)) if seed % 2 else 0)
        offsets.append(off)
    q = rng.standard_normal((3, n_new) + q1.shape[1:])
    out, lse = O.concurrent_attention(q, blocks, views, offsets=offsets)
    assert out.shape == q.shape and lse.shape == q.shape[:3]
    qps = [offsets[w][-1] + lengths[v[-1]] - 1 for w, v in enumerate(views)]
    for t in range(n_new):
        pos = [p - (n_new - 1 - t) for p in qps]
        nb, nv, no = _truncated_case(q[:, t], blocks, views, offsets, pos)
        ref, ref_lse = O.concurrent_attention(q[:, t], nb, nv, offsets=no, q_pos=pos)
        assert np.array_equal(out[:, t], ref), t
        assert np.array_equal(lse[:, t], ref_lse), t


def test_several_tokens_one_token_case_and_interleaved_keys():
    rng = np.random.default_rng(77)
    q1, blocks, views, offsets = _rand_case(rng, n_workers=2)
    out1, lse1 = O.concurrent_attention(q1, blocks, views, offsets=offsets)
    out, lse = O.concurrent_attention(q1[:, None], blocks, views, offsets=offsets)
    assert np.array_equal(out[:, 0], out1) and np.array_equal(lse[:, 0], lse1)

    # Keys between the query tokens: with an explicit q_pos the tokens need not be stored
    # keys. Worker 0's block 5 holds positions 100..106, block 7 holds 107..108 and the
    # queries sit at 107, 108, 109: the token at 107 sees block 7's first key only, the one
    # at 109 sees both. Written out by hand.
    d, hkv = 8, 1
    k_own, v_own = rng.standard_normal((7, hkv, d)), rng.standard_normal((7, hkv, d))
    k7, v7 = rng.standard_normal((2, hkv, d)), rng.standard_normal((2, hkv, d))
    qq = rng.standard_normal((1, 3, 1, d))
    bl = {5: (k_own, v_own), 7: (k7, v7)}
    out, lse = O.concurrent_attention(qq, bl, [[5, 7]], offsets=[[100, 107]], q_pos=[109])
    for t, p in enumerate((107, 108, 109)):
        n7 = min(2, p - 107 + 1)
        keys = np.concatenate([k_own, k7[:n7]])
        vals = np.concatenate([v_own, v7[:n7]])
        kpos = np.concatenate([100 + np.arange(7), 107 + np.arange(n7)])
        s = O.rope(keys[:, 0], kpos, 1e4) @ O.rope(qq[0, t], p, 1e4)[0] / math.sqrt(d)
        w_ = np.exp(s - s.max())
        assert _rel(out[0, t, 0], (w_ @ vals[:, 0]) / w_.sum()) <= 1e-12
        assert abs(lse[0, t, 0] - (s.max() + math.log(w_.sum()))) <= 1e-12

    # a token with no key at or before it: out 0, lse -inf
    out, lse = O.concurrent_attention(qq, {7: (k7, v7)}, [[7]], offsets=[[107]], q_pos=[108])
    assert np.all(out[0, 0] == 0) and lse[0, 0, 0] == -np.inf   # the token at 106
    assert np.isfinite(lse[0, 1:]).all()
    with pytest.raises(ValueError):   # a query position below 0
        O.concurrent_attention(rng.standard_normal((1, 3, 1, d)), {7: (k7[:1], v7[:1])}, [[7]],
                               offsets=[[0]], q_pos=[1])
