"""Several query tokens per worker in one decode (hw_concurrent_decode_tokens), against the
fp64 oracle's causal several-token attention, through the C ABI.

Token t of worker w sits at q_pos(w) - (n_new - 1 - t) and sees only the keys of w's view
at or before it (paper summary s8 step 4: a worker that opens a fresh block appends its
paragraph header, and the header's tokens are attended together). Rows of a KV head are
(worker, token, head), in blocks of at most 32 rows (bf16) or 16 (fp32) on the 8-wave
kernels: these shapes take one to six row blocks, one and two row tiles, both head sizes.
Tolerances as for one token: relative L2 <= 1e-2 (bf16 K/V), <= 1e-5 (fp32).
"""

import numpy as np
import pytest
import torch

from oracle import hogwild_oracle as O
from shared_kv_cache_amd import hogwild as H
from shared_kv_cache_amd import workloads as W

from hw_testlib import (DEV, TOL, assert_parity, decode_np, decode_tokens_np, fill_layer, kv_tensor,
                        make_cache, oracle_blocks, rel_l2, variant_workload)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _compare(name, out, lse, ref, ref_lse, tol):
    # every (worker, token, head) row within tol (rel L2 and absolute lse); a token with no
    # key at or before it: zero output, lse -inf
    assert_parity(name, out, lse, ref, ref_lse, tol, _say)


@pytest.mark.parametrize("head_dim,n_workers,group,n_new,kv_dtype", [
    (128, 2, 8, 2, "bf16"),    # 32 rows: one block of two row tiles, 4-int descriptors
    (64, 4, 8, 2, "bf16"),     # 64 rows: two blocks
    (64, 3, 5, 5, "bf16"),     # 75 rows: blocks of 32, 32, 11; a token's heads straddle blocks
    (128, 16, 2, 3, "bf16"),   # 96 rows of 16 workers: three blocks
    (64, 1, 1, 7, "bf16"),     # one worker, one head per KV head: 7 rows, one tile
    (128, 6, 8, 4, "bf16"),    # 192 rows: six blocks
    (128, 3, 2, 3, "f32"),     # fp32 pools: 18 rows in blocks of 16 and 2
])
def test_several_query_tokens_per_worker(head_dim, n_workers, group, n_new, kv_dtype):
    # The variant workload's own blocks hold 33, 1, 64, 65, 7, 0, 31, 32 tokens: a worker
    # whose block is shorter than n_new has early tokens inside the previous block (cut
    # causally), and one whose block is empty queries from the end of the previous block.
    wl = variant_workload(head_dim, n_workers, group)
    wl = W.Workload(**{**wl.__dict__, "kv_dtype": kv_dtype})
    cache = make_cache(wl, max_blocks=n_workers + 2, max_splits=128, max_query_tokens=8)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    q = wl.q_tokens(0, n_new)
    ref, ref_lse = O.concurrent_attention(q.astype(np.float64), oracle_blocks(wl, 0), wl.views(),
                                          theta=wl.theta)
    for splits in (0, 1, 3, 40):
        H.hw_set_split(cache.ctx, splits)
        out, lse = decode_tokens_np(cache, 0, q)
        _compare(f"{wl.name} n_new {n_new} {kv_dtype} splits {splits}", out, lse, ref, ref_lse,
                 TOL[kv_dtype])
    # one token through either entry point: the same launch, the same bits
    H.hw_set_split(cache.ctx, 0)
    q1 = np.ascontiguousarray(q[:, -1])
    one, one_lse = decode_np(cache, 0, q1)
    tok, tok_lse = decode_tokens_np(cache, 0, q1[:, None])
    np.testing.assert_array_equal(one, tok[:, 0])
    np.testing.assert_array_equal(one_lse, tok_lse[:, 0])
    cache.close()


def test_several_tokens_explicit_offsets_gaps_and_qpos():
    # Offsets with gaps between blocks and a query position past the last key: some tokens
    # sit in a gap, the earliest ones before the end of the previous block.
    wl = variant_workload(128, 4, 8)
    cache = make_cache(wl, max_blocks=8, max_splits=64, max_query_tokens=6)
    fill_layer(cache, wl, 0)
    views = wl.views()
    L = wl.lengths
    offsets, q_pos = [], []
    for v in views:
        off, acc = [], 5
        for b in v:
            off.append(acc)
            acc += L[b] + 3
        offsets.append(off)
        q_pos.append(off[-1] + L[v[-1]] + 1)
    cache.set_views(views, offsets, q_pos)
    q = wl.q_tokens(0, 6)
    ref, ref_lse = O.concurrent_attention(q.astype(np.float64), oracle_blocks(wl, 0), views,
                                          offsets=offsets, q_pos=q_pos, theta=wl.theta)
    for splits in (0, 1, 7):
        H.hw_set_split(cache.ctx, splits)
        out, lse = decode_tokens_np(cache, 0, q)
        _compare(f"offsets and gaps splits {splits}", out, lse, ref, ref_lse, TOL["bf16"])
    cache.close()


def test_paragraph_header_flow():
    # Every worker opens a fresh block with a 4-token paragraph header (paper summary s8
    # step 4): the old unfinished steps are committed to the history, the headers appended,
    # the views rebuilt and the headers' tokens attended together; then one more token each.
    wl = variant_workload(128, 4, 8)
    n_new = 4
    cache = make_cache(wl, max_blocks=16, n_pages=wl.n_pages + 8, max_query_tokens=n_new)
    fill_layer(cache, wl, 0)
    hist = [wl.history[0]] + list(wl.inprogress)
    fresh = [10 + w for w in range(4)]
    host = {b: wl.kv(0, b) for b in wl.blocks()}
    kh, vh = zip(*(wl.kv(0, b, length=n_new) for b in fresh))
    cache.append(0, fresh, [n_new] * 4, kv_tensor(np.concatenate(kh), "bf16"),
                 kv_tensor(np.concatenate(vh), "bf16"))
    for b, k, v in zip(fresh, kh, vh):
        host[b] = (k, v)
    views = [hist + [fresh[u] for u in range(4) if u != w] + [fresh[w]] for w in range(4)]
    cache.set_views(views)
    blocks = {b: (np.asarray(k, np.float64), np.asarray(v, np.float64)) for b, (k, v) in host.items()}
    q = wl.q_tokens(0, n_new)
    ref, ref_lse = O.concurrent_attention(q.astype(np.float64), blocks, views, theta=wl.theta)
    out, lse = decode_tokens_np(cache, 0, q)
    _compare("header tokens", out, lse, ref, ref_lse, TOL["bf16"])
    # the header's last token is the one-token decode of the same state
    ref1, _ = O.concurrent_attention(q[:, -1].astype(np.float64), blocks, views, theta=wl.theta)
    np.testing.assert_allclose(ref[:, -1], ref1, rtol=0, atol=1e-12)
    one, one_lse = decode_np(cache, 0, np.ascontiguousarray(q[:, -1]))
    _compare("header last token, one-token decode", one, one_lse, ref1, ref_lse[:, -1], TOL["bf16"])
    # next step: one token per worker after the header
    k, v = wl.step_kv(0, 1)
    cache.append(0, fresh, [1] * 4, kv_tensor(k, "bf16"), kv_tensor(v, "bf16"))
    for w, b in enumerate(fresh):
        blocks[b] = tuple(np.concatenate([x, y[w:w + 1].astype(np.float64)])
                          for x, y in zip(blocks[b], (k, v)))
    cache.set_views(views)
    q1 = wl.q(0, 1)
    ref, ref_lse = O.concurrent_attention(q1.astype(np.float64), blocks, views, theta=wl.theta)
    out, lse = decode_np(cache, 0, q1)
    _compare("token after the header", out, lse, ref, ref_lse, TOL["bf16"])
    cache.close()


def test_several_tokens_errors_and_empty_view():
    wl = variant_workload(128, 2, 8)
    cache = make_cache(wl, max_blocks=6, max_query_tokens=4)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    q = wl.q_tokens(0, 4)
    before = decode_tokens_np(cache, 0, q)
    with pytest.raises(H.HwError) as e:             # more tokens than the context allows
        decode_tokens_np(cache, 0, wl.q_tokens(0, 5))
    assert e.value.status == H.HW_ERR_INVALID_ARG
    # block 2 holds one token: a view of it alone queries at position 0, so with 4 tokens
    # the first would sit at -3
    cache.set_views([[2], [0, 2]])
    with pytest.raises(H.HwError) as e:
        decode_tokens_np(cache, 0, q)
    assert e.value.status == H.HW_ERR_STALE_VIEW
    # a worker whose view holds no token: zero output and lse -inf for every token
    cache.set_views([wl.views()[0], []])
    out, lse = decode_tokens_np(cache, 0, q)
    assert np.all(out[1] == 0.0) and np.all(np.isneginf(lse[1]))
    ref, ref_lse = O.concurrent_attention(q[:1].astype(np.float64), oracle_blocks(wl, 0),
                                          wl.views()[:1], theta=wl.theta)
    _compare("worker 0 beside an empty view", out[:1], lse[:1], ref, ref_lse, TOL["bf16"])
    cache.set_views(wl.views())
    after = decode_tokens_np(cache, 0, q)
    np.testing.assert_array_equal(before[0], after[0])
    np.testing.assert_array_equal(before[1], after[1])
    cache.close()


def test_w4_16k_header_tokens_sampled_heads():
    # The w4_16k cache (16k-token history of 64-token pages, 40 query heads over 8 KV
    # heads), four tokens per worker, in the launch configuration of the one-token decode.
    wl = W.make("w4_16k", n_layers=1)
    cache = make_cache(wl, max_query_tokens=4)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    q = wl.q_tokens(0, 4)
    rng = np.random.default_rng(wl.seed + 4)
    heads = sorted(int(x) for x in rng.choice(wl.n_q_heads, size=6, replace=False))
    ref, ref_lse = O.concurrent_attention(q.astype(np.float64), oracle_blocks(wl, 0), wl.views(),
                                          theta=wl.theta, heads=heads)
    out, lse = decode_tokens_np(cache, 0, q)
    _compare("w4_16k 4 tokens", out[:, :, heads], lse[:, :, heads], ref[:, :, heads],
             ref_lse[:, :, heads], TOL["bf16"])
    cache.close()


def test_w8_32k_header_tokens_sampled_heads():
    # The w8_32k cache (32k-token common history in scattered 256-token pages, 64 query heads
    # over 8 KV heads, 8 workers): four tokens per worker make 256 rows per KV head, eight
    # row blocks, in the launch configuration the bench times.
    wl = W.make("w8_32k", n_layers=1)
    cache = make_cache(wl, max_query_tokens=4)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    q = wl.q_tokens(0, 4)
    out, lse = decode_tokens_np(cache, 0, q)
    # the oracle on sampled workers (first, middle, last) and heads: each worker's result
    # depends only on its own view
    rng = np.random.default_rng(wl.seed + 8)
    heads = sorted(int(x) for x in rng.choice(wl.n_q_heads, size=4, replace=False))
    sel = [0, 3, 7]
    views = wl.views()
    ref, ref_lse = O.concurrent_attention(q[sel].astype(np.float64), oracle_blocks(wl, 0),
                                          [views[w] for w in sel], theta=wl.theta, heads=heads)
    _compare("w8_32k 4 tokens", out[sel][:, :, heads], lse[sel][:, :, heads], ref[:, :, heads],
             ref_lse[:, :, heads], TOL["bf16"])
    cache.close()


def test_several_tokens_graph_replays_equal_eager():
    # A two-layer several-token decode captured as one HIP graph (after the tables are
    # uploaded): every replay, with eager work in between, equals the eager result bit for bit.
    wl = variant_workload(128, 4, 8)
    wl = W.Workload(**{**wl.__dict__, "n_layers": 2})
    cache = make_cache(wl, max_blocks=8, max_query_tokens=3)
    for layer in range(2):
        fill_layer(cache, wl, layer)
    cache.set_views(wl.views())
    qs = [torch.from_numpy(wl.q_tokens(layer, 3)).to(DEV) for layer in range(2)]
    outs = [torch.empty_like(q) for q in qs]
    lses = [torch.empty(q.shape[:3], device=DEV) for q in qs]

    def step():
        for layer in range(2):
            cache.decode_tokens(layer, qs[layer], out=outs[layer], lse=lses[layer])

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs], [x.clone() for x in lses]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer in range(2):
            assert torch.equal(outs[layer], eager[0][layer]), (rep, layer)
            assert torch.equal(lses[layer], eager[1][layer]), (rep, layer)
        step()
        torch.cuda.synchronize()
    cache.close()
