"""Parity of the gfx950 path against the fp64 oracle, through the C ABI.

Tolerances (hw_testlib.assert_parity): relative L2 over all (worker, head, dim)
of a layer <= 1e-5 for the fp32 configuration and <= 1e-2 for bf16 K/V, the
same bound on every single (worker, head) row, and |lse - lse_ref| <= the same
number in absolute terms; the stored pool bytes are bit-exact (V copied, K =
the oracle's stored-key reference).
"""

import math

import numpy as np
import pytest
import torch

from oracle import hogwild_oracle as O
from shared_kv_cache_amd import hogwild as H
from shared_kv_cache_amd import workloads as W

from hw_testlib import (DEV, TOL, assert_parity, decode_np, fill_layer, k_pool_token, kv_tensor,
                        make_cache, oracle_blocks, rel_l2, v_pool_token, variant_workload)

pytestmark = pytest.mark.gpu

# Agreement of one decode under different partition counts (bf16 pools). Each partition
# rounds its probabilities to bf16 against its own running maximum, so two partition
# counts round different numbers: relative 2^-9 per probability, independent across keys,
# which averages to about 2e-3 over a layer (measured 2.2e-3 on w2_4k between 1 and 256
# partitions). Twice that is the bound; fp32 pools agree to 1e-6.
SPLIT_TOL_BF16 = 5e-3


def _say(*a):
    print(*a, flush=True)


def _check_layer(cache, wl, layer, heads=None, tol=None, offsets=None, q_pos=None, views=None):
    views = wl.views() if views is None else views
    q = wl.q(layer)
    out, lse = decode_np(cache, layer, q)
    ref, ref_lse = O.concurrent_attention(q.astype(np.float64), oracle_blocks(wl, layer), views,
                                          offsets=offsets, q_pos=q_pos, theta=wl.theta, heads=heads)
    hs = list(range(wl.n_q_heads)) if heads is None else list(heads)
    tol = TOL[wl.kv_dtype] if tol is None else tol
    assert_parity(f"{wl.name} layer {layer}", out[:, hs], lse[:, hs], ref[:, hs], ref_lse[:, hs],
                  tol, _say)
    return out, lse


# ------------------------------------------------------------- small configs

def test_tiny_fp32_parity():
    wl = W.make("tiny_fp32")
    cache = make_cache(wl)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    _check_layer(cache, wl, 0)
    cache.close()


@pytest.mark.parametrize("page_size", [32, 256, 8192])   # 8192: the largest page the library takes
def test_tiny_fp32_page_sizes_and_splits(page_size):
    wl = W.make("tiny_fp32", page_size=page_size)
    cache = make_cache(wl)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    outs = []
    for splits in (1, 3, 11):
        H.hw_set_split(cache.ctx, splits)
        outs.append(_check_layer(cache, wl, 0)[0])
    assert rel_l2(outs[0], outs[2]) <= 1e-6
    cache.close()


def test_pool_bytes_bit_exact_fp32_and_bf16():
    for name in ("tiny_fp32", "w2_4k"):
        wl = W.make(name, n_layers=2)
        cache = make_cache(wl)
        blocks = fill_layer(cache, wl, 1)
        torch.cuda.synchronize()
        kp = cache.k_pool.cpu()
        vp = cache.v_pool.cpu()
        if wl.kv_dtype == "bf16":
            kp = kp.view(torch.int16).numpy().view(np.uint16)
            vp = vp.view(torch.int16).numpy().view(np.uint16)
        else:
            kp, vp = kp.numpy(), vp.numpy()
        rng = np.random.default_rng(0)
        for b in wl.blocks():
            length, pages = cache.block_info(b, 1)
            assert length == wl.lengths[b]
            toks = np.unique(np.concatenate([[0, length - 1], rng.integers(0, length, 40)]))
            k_raw, v_raw = blocks[b]
            expect_k = O.rope_store_reference(k_raw[toks], toks, wl.theta, wl.kv_dtype)
            for i, t in enumerate(toks):
                page, slot = pages[t // wl.page_size], t % wl.page_size
                for h in range(wl.n_kv_heads):
                    got_k = kp[k_pool_token(cache, 1, page, h, slot)]
                    got_v = vp[v_pool_token(cache, 1, page, h, slot)]
                    np.testing.assert_array_equal(got_k, expect_k[i, h])
                    want_v = (v_raw[t, h] if wl.kv_dtype == "f32"
                              else O.bf16_bits_rne(v_raw[t, h]))
                    np.testing.assert_array_equal(got_v, want_v)
        _say(f"{name}: pool bytes bit-exact")
        cache.close()


def test_w2_4k_parity_and_split_invariance():
    wl = W.make("w2_4k", n_layers=2)
    cache = make_cache(wl)
    for layer in range(2):
        fill_layer(cache, wl, layer)
    cache.set_views(wl.views())
    for layer in range(2):
        _check_layer(cache, wl, layer)
    q = wl.q(1)
    H.hw_set_split(cache.ctx, 1)
    o1, l1 = decode_np(cache, 1, q)
    H.hw_set_split(cache.ctx, 256)
    o256, l256 = decode_np(cache, 1, q)
    H.hw_set_split(cache.ctx, 0)
    _say(f"split 1 vs 256: {rel_l2(o256, o1):.3e}")
    assert rel_l2(o256, o1) <= SPLIT_TOL_BF16
    assert np.max(np.abs(l256 - l1)) <= 1e-4
    cache.close()


def test_fp32_results_across_partition_counts():
    # fp32 pools keep fp32 probabilities: the partition count changes only the order of fp32
    # sums, so 1 and 5 partitions agree to fp32 rounding (the bf16 bound above comes from
    # bf16 probabilities rounded against each partition's own running maximum).
    wl = W.make("tiny_fp32")
    cache = make_cache(wl)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    q = wl.q(0)
    H.hw_set_split(cache.ctx, 1)
    o1, l1 = decode_np(cache, 0, q)
    H.hw_set_split(cache.ctx, 5)
    o5, l5 = decode_np(cache, 0, q)
    H.hw_set_split(cache.ctx, 0)
    _say(f"fp32 split 1 vs 5: {rel_l2(o5, o1):.3e}, lse {np.max(np.abs(l5 - l1)):.3e}")
    assert rel_l2(o5, o1) <= TOL["f32"]
    assert np.max(np.abs(l5 - l1)) <= TOL["f32"]
    cache.close()


def test_page_scatter_invariance_is_bitwise():
    wl = W.make("w2_4k", n_layers=1)
    outs = []
    for seed in (0, 0xABC):
        cache = make_cache(wl, page_seed=seed, n_pages=2 * wl.n_pages)
        fill_layer(cache, wl, 0)
        cache.set_views(wl.views())
        outs.append(decode_np(cache, 0, wl.q(0)))
        cache.close()
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_explicit_offsets_gaps_qpos_and_subset_views():
    wl = W.make("w2_4k", n_layers=1)
    cache = make_cache(wl)
    fill_layer(cache, wl, 0)
    views = wl.views()
    L = wl.lengths
    offsets, q_pos = [], []
    for v in views:
        off, acc = [], 7
        for b in v:
            off.append(acc)
            acc += L[b] + 13
        offsets.append(off)
        q_pos.append(off[-1] + L[v[-1]] + 2)
    cache.set_views(views, offsets, q_pos)
    _check_layer(cache, wl, 0, offsets=offsets, q_pos=q_pos, views=views)
    # no-sync style: each worker sees the common block and its own block only
    sub = [[wl.history[0], wl.inprogress[w]] for w in range(wl.n_workers)]
    cache.set_views(sub)
    _check_layer(cache, wl, 0, views=sub)
    cache.close()


def test_many_rows_multiple_row_blocks_and_empty_view():
    # 5 workers x G = 16 rows each = 80 rows: two row blocks of the decode grid
    wl = W.make("tiny_fp32")
    wl = W.Workload(**{**wl.__dict__, "name": "rows80", "n_workers": 5, "n_q_heads": 32,
                       "n_kv_heads": 2, "kv_dtype": "bf16",
                       "inprogress": [1, 2, 3, 4, 5],
                       "lengths": {0: 300, 1: 33, 2: 1, 3: 64, 4: 65, 5: 0},
                       "owners": {0: -1, 1: 0, 2: 1, 3: 2, 4: 3, 5: 4}, "n_pages": 40})
    cache = make_cache(wl, max_blocks=8)
    fill_layer(cache, wl, 0, blocks=[0, 1, 2, 3, 4])
    views = wl.views()
    views[4] = [5]                                 # a worker whose view holds no token
    cache.set_views(views)
    q = wl.q(0)
    out, lse = decode_np(cache, 0, q)
    assert np.all(out[4] == 0.0) and np.all(np.isneginf(lse[4]))
    blocks = {b: tuple(np.asarray(x, np.float64) for x in wl.kv(0, b)) for b in range(6)}
    ref, ref_lse = O.concurrent_attention(q[:4].astype(np.float64), blocks, views[:4], theta=wl.theta)
    assert_parity("rows80", out[:4], lse[:4], ref, ref_lse, TOL["bf16"], _say)
    cache.close()


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("n_workers,group", [(2, 8), (4, 8), (5, 8), (8, 8), (3, 5), (6, 8),
                                             (7, 6), (16, 2), (9, 7), (32, 2), (64, 1), (13, 5),
                                             (128, 2)])
def test_every_bf16_kernel_variant(head_dim, n_workers, group):
    # 15 to 65 rows per KV head: one to four 16-row tiles, i.e. the 8-wave single-stage
    # kernels (wide descriptors up to 6 workers, narrow beyond) and the 4-wave two-stage
    # kernels; 128 workers of 2 heads make 256 rows, four row blocks of the 4-wave kernel.
    # Each under automatic and forced KV partitions: 1 (several rotation phases in one
    # workgroup), 3, 40 and 80 (bounds chosen by the host; many partitions empty at 80).
    wl = variant_workload(head_dim, n_workers, group)
    cache = make_cache(wl, max_blocks=n_workers + 2, max_splits=128)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    q = wl.q(0)
    ref, ref_lse = O.concurrent_attention(q.astype(np.float64), oracle_blocks(wl, 0), wl.views(),
                                          theta=wl.theta)
    for splits in (0, 1, 3, 40, 80):
        H.hw_set_split(cache.ctx, splits)
        out, lse = decode_np(cache, 0, q)
        assert_parity(f"{wl.name} splits {splits}", out, lse, ref, ref_lse, TOL["bf16"], _say)
    cache.close()


def _layout_workload(n_workers, n_q_heads, seed):
    """bf16, 8 KV heads x 128: a 600-token prompt, ten paragraphs of U{40..200} tokens owned
    round-robin (the shape of the w4_16k history, shortened) and unfinished steps of
    U{1..150} tokens, 64-token pages."""
    base = W.make("w4_16k", n_layers=1)
    rng = np.random.default_rng(seed)
    paras = [int(x) for x in rng.integers(40, 201, size=10)]
    cur = [int(x) for x in rng.integers(1, 151, size=n_workers)]
    history = list(range(11))
    inprog = [11 + w for w in range(n_workers)]
    lengths = {0: 600, **{1 + i: n for i, n in enumerate(paras)}, **{b: n for b, n in zip(inprog, cur)}}
    owners = {0: -1, **{1 + i: i % n_workers for i in range(10)}, **{b: w for w, b in enumerate(inprog)}}
    pages = sum(-(-n // 64) for n in lengths.values()) + 4
    return W.Workload(**{**base.__dict__, "name": f"layouts_{n_workers}w", "seed": seed,
                         "n_workers": n_workers, "n_q_heads": n_q_heads, "n_kv_heads": 8,
                         "page_size": 64, "history": history, "inprogress": inprog,
                         "lengths": lengths, "owners": owners, "n_pages": pages,
                         "max_position": 4096})


@pytest.mark.parametrize("n_workers,n_q_heads", [(4, 40), (8, 64)])
def test_cache_layouts_as_views(n_workers, n_q_heads):
    # The layouts the paper summary compares (s6 table; s10 sync levels) are block orders
    # over the same stored blocks: combined (the method), step-wise (other workers'
    # unfinished steps invisible, so rows of one tile differ in visibility), contiguous
    # (each worker's output one span) and no-sync. 20 rows per KV head run the 8-wave
    # kernels, 64 rows the cooperative ones; each layout under automatic and forced splits.
    wl = _layout_workload(n_workers, n_q_heads, seed=11 + n_workers)
    cache = make_cache(wl, max_splits=64)
    fill_layer(cache, wl, 0)
    q = wl.q(0)
    blocks = oracle_blocks(wl, 0)
    for layout in ("combined", "stepwise", "contiguous", "nosync"):
        views = wl.views(layout)
        ref, ref_lse = O.concurrent_attention(q.astype(np.float64), blocks, views, theta=wl.theta)
        cache.set_views(views)
        for splits in (0, 1, 7):
            H.hw_set_split(cache.ctx, splits)
            out, lse = decode_np(cache, 0, q)
            assert_parity(f"{wl.name} {layout} splits {splits}", out, lse, ref, ref_lse,
                          TOL["bf16"], _say)
    cache.close()


def test_step_commit_flow_with_block_reuse():
    # Steps of a run (paper summary s8): every worker appends its token, the views are
    # rebuilt, attention runs. At step 3 worker 1's step is committed: its block moves to
    # the end of the common history and the worker continues in block 20, whose earlier
    # contents were freed with hw_reset_block (its pages return to the free list and are
    # handed out again); at step 5 worker 3 commits into the fresh block 21. Each step is
    # checked against the oracle over the blocks' current contents.
    wl = _layout_workload(4, 40, seed=23)
    cache = make_cache(wl, max_blocks=32, n_pages=wl.n_pages + 16)
    fill_layer(cache, wl, 0)
    host = {b: [list(x) for x in wl.kv(0, b)] for b in wl.blocks()}   # b -> [K rows, V rows]
    scratch_k, scratch_v = wl.kv(0, wl.history[1])                   # fill block 20, unused
    cache.append(0, [20], [len(scratch_k)], kv_tensor(scratch_k, "bf16"), kv_tensor(scratch_v, "bf16"))
    hist, cur = list(wl.history), list(wl.inprogress)
    for step in range(1, 7):
        if step == 3:
            free0 = H.hw_free_pages(cache.ctx)
            H.hw_reset_block(cache.ctx, 20)
            assert H.hw_free_pages(cache.ctx) == free0 + -(-len(scratch_k) // wl.page_size)
            hist, cur = O.commit_step_views(hist, cur, 1, 20)
            host[20] = [[], []]
        if step == 5:
            hist, cur = O.commit_step_views(hist, cur, 3, 21)
            host[21] = [[], []]
        k, v = wl.step_kv(0, step)
        cache.append(0, cur, [1] * 4, kv_tensor(k, "bf16"), kv_tensor(v, "bf16"))
        for w, b in enumerate(cur):
            host[b][0].append(k[w])
            host[b][1].append(v[w])
        views = [hist + [cur[u] for u in range(4) if u != w] + [cur[w]] for w in range(4)]
        cache.set_views(views)
        blocks = {b: (np.asarray(kk, np.float64), np.asarray(vv, np.float64))
                  for b, (kk, vv) in host.items() if any(b in vw for vw in views)}
        q = wl.q(0, step)
        ref, ref_lse = O.concurrent_attention(q.astype(np.float64), blocks, views, theta=wl.theta)
        out, lse = decode_np(cache, 0, q)
        assert_parity(f"commit flow step {step} ({len(hist)} history blocks)", out, lse, ref,
                      ref_lse, TOL["bf16"], _say)
    cache.close()


def test_decode_step_graph_replays_equal_eager():
    # A whole decode step (every layer) captured as one HIP graph: kernels only once the
    # views' tables are uploaded (no memset nodes). Each replay, with eager work and
    # synchronisations in between, must equal the eager step bit for bit.
    wl = _layout_workload(4, 40, seed=31)
    wl = W.Workload(**{**wl.__dict__, "n_layers": 4})
    cache = make_cache(wl)
    for layer in range(4):
        fill_layer(cache, wl, layer)
    cache.set_views(wl.views())
    qs = [torch.from_numpy(wl.q(layer)).to(DEV) for layer in range(4)]
    outs = [torch.empty_like(q) for q in qs]
    lses = [torch.empty(q.shape[:2], device=DEV) for q in qs]

    def step():
        for layer in range(4):
            cache.decode(layer, qs[layer], out=outs[layer], lse=lses[layer])

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs], [x.clone() for x in lses]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer in range(4):
            assert torch.equal(outs[layer], eager[0][layer]), (rep, layer)
            assert torch.equal(lses[layer], eager[1][layer]), (rep, layer)
        step()   # eager work between replays
        torch.cuda.synchronize()
    _say("graph replays equal the eager step")
    cache.close()


def test_errors_leave_gpu_state_unchanged():
    wl = W.make("w2_4k", n_layers=1)
    cache = make_cache(wl)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    before = decode_np(cache, 0, wl.q(0))
    free0 = H.hw_free_pages(cache.ctx)
    big = torch.zeros((free0 * wl.page_size + 1, wl.n_kv_heads, wl.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    with pytest.raises(H.HwError) as e:
        cache.append(0, [wl.inprogress[0]], [big.shape[0]], big, big)
    assert e.value.status == H.HW_ERR_OUT_OF_PAGES
    with pytest.raises(H.HwError) as e:
        cache.set_views([[0, 0]])
    assert e.value.status == H.HW_ERR_INVALID_ARG
    bad_off = [[0, 10, 20]] * wl.n_workers
    cache.set_views(wl.views(), bad_off)
    with pytest.raises(H.HwError) as e:
        cache.decode(0, torch.from_numpy(wl.q(0)).cuda())
    assert e.value.status == H.HW_ERR_STALE_VIEW
    cache.set_views(wl.views())
    after = decode_np(cache, 0, wl.q(0))
    assert H.hw_free_pages(cache.ctx) == free0
    np.testing.assert_array_equal(before[0], after[0])
    cache.close()


@pytest.mark.parametrize("name", ["tiny_fp32", "variant"])
def test_pools_holding_nan_bits(name):
    # Pools that were never initialised may hold any bits. Fill both with NaN patterns
    # before the appends: the unoccupied slots of every block's last group then hold NaN,
    # and the decode must still match the oracle (masked scores, zeroed values).
    wl = W.make("tiny_fp32") if name == "tiny_fp32" else variant_workload(128, 4, 8)
    cache = make_cache(wl, max_splits=64)
    for pool in (cache.k_pool, cache.v_pool):
        (pool.view(torch.int16) if pool.dtype == torch.bfloat16 else pool.view(torch.int32)).fill_(-1)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    q = wl.q(0)
    ref, ref_lse = O.concurrent_attention(q.astype(np.float64), oracle_blocks(wl, 0), wl.views(),
                                          theta=wl.theta)
    for splits in (0, 1, 5):
        H.hw_set_split(cache.ctx, splits)
        out, lse = decode_np(cache, 0, q)
        assert np.all(np.isfinite(out))
        assert_parity(f"{wl.name} NaN pools splits {splits}", out, lse, ref, ref_lse,
                      TOL[wl.kv_dtype], _say)
    cache.close()


def test_capture_refuses_a_table_upload():
    # A decode whose views' tables must be uploaded (views or lengths changed) cannot sit in
    # a stream capture: it returns an error and enqueues nothing; the same decode after an
    # eager one (tables current) captures and replays to the eager result.
    wl = _layout_workload(4, 40, seed=37)
    cache = make_cache(wl)
    fill_layer(cache, wl, 0)
    q = torch.from_numpy(wl.q(0)).to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], device=DEV)
    cache.set_views(wl.views("stepwise"))
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with pytest.raises(H.HwError) as e:
        with torch.cuda.graph(g, stream=side):
            cache.decode(0, q, out=out, lse=lse)
    assert e.value.status == H.HW_ERR_INVALID_ARG
    assert "capture" in e.value.message
    torch.cuda.synchronize()
    cache.decode(0, q, out=out, lse=lse)               # eager: uploads the tables
    torch.cuda.synchronize()
    eager = out.clone(), lse.clone()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=side):
        cache.decode(0, q, out=out, lse=lse)
    for _ in range(2):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]) and torch.equal(lse, eager[1])
    cache.close()


# ------------------------------------------------------- full-size configs

def test_w4_16k_parity_sampled_layers():
    wl = W.make("w4_16k")                 # 64 layers, as timed
    cache = make_cache(wl)
    for layer in range(wl.n_layers):
        fill_layer(cache, wl, layer)
    cache.set_views(wl.views())
    for layer in (0, 21, 42, 63):
        _check_layer(cache, wl, layer)
    cache.close()


def test_w8_32k_parity_across_steps():
    steps = 3
    wl = W.make("w8_32k", steps=steps)
    cache = make_cache(wl)
    for layer in range(wl.n_layers):
        fill_layer(cache, wl, layer)
    lengths = dict(wl.lengths)
    hist = {layer: {} for layer in (0, 5)}
    for step in range(1, steps + 1):
        cache.set_views(wl.views())
        for layer in range(wl.n_layers):
            k, v = wl.step_kv(layer, step)
            cache.append(layer, wl.inprogress, [1] * wl.n_workers, kv_tensor(k, "bf16"),
                         kv_tensor(v, "bf16"))
            if layer in hist:
                hist[layer][step] = (k, v)
        for b in wl.inprogress:
            lengths[b] += 1
        for layer in (0, 5):
            blocks = {}
            for b in wl.blocks():
                k0, v0 = wl.kv(layer, b)
                if b in wl.inprogress:
                    w = wl.inprogress.index(b)
                    k0 = np.concatenate([k0] + [hist[layer][s][0][w:w + 1] for s in range(1, step + 1)])
                    v0 = np.concatenate([v0] + [hist[layer][s][1][w:w + 1] for s in range(1, step + 1)])
                blocks[b] = (k0.astype(np.float64), v0.astype(np.float64))
            q = wl.q(layer, step)
            out, lse = decode_np(cache, layer, q)
            ref, ref_lse = O.concurrent_attention(q.astype(np.float64), blocks, wl.views(), theta=wl.theta)
            assert_parity(f"w8_32k step {step} layer {layer}", out, lse, ref, ref_lse,
                          TOL["bf16"], _say)
    cache.close()


def _sink_heads(wl, salt):
    """Four query heads of the 131k-token case: three seeded heads outside the sink group and
    one inside it (KV head 7 holds the four keys scaled x8, query heads 35..39)."""
    rng = np.random.default_rng(wl.seed + salt)
    return sorted(set(int(x) for x in rng.choice(35, size=3, replace=False)) |
                  {int(rng.integers(35, 40))})


def test_w4_128k_sinks_automatic_splits_two_layer_pools():
    # The launch configuration the bench times: the automatic partition count with
    # host-chosen bounds (the bounded-partition path), on two of the four layer pools.
    wl = W.make("w4_128k_sinks", n_layers=2)
    cache = make_cache(wl)
    for layer in range(2):
        fill_layer(cache, wl, layer)
    cache.set_views(wl.views())
    n_splits = H.hw_debug_resolve(cache.ctx, 0, wl.n_workers)["n_splits"]
    _say(f"w4_128k_sinks: automatic split count {n_splits}")
    assert 1 < n_splits <= 255
    for layer in range(2):
        heads = _sink_heads(wl, layer)
        assert any(35 <= h < 40 for h in heads)
        _check_layer(cache, wl, layer, heads=heads)
    cache.close()


def test_w4_128k_sinks_split256_sampled_heads():
    # 256 partitions: beyond the 255 whose bounds ride in the launch arguments, so the
    # uniform cuts p * n_groups / 256 (about two pages a partition).
    wl = W.make("w4_128k_sinks", n_layers=1)
    cache = make_cache(wl, max_splits=512)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    H.hw_set_split(cache.ctx, 256)
    assert H.hw_debug_resolve(cache.ctx, 0, wl.n_workers)["n_splits"] == 256
    _check_layer(cache, wl, 0, heads=_sink_heads(wl, 0))
    cache.close()
