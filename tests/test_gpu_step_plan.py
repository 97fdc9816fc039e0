"""Step plans (hw_plan_steps / hw_append_step / hw_plan_end): whole decode steps, appends
included, whose positions, group sizes and query offsets the device derives from its own
per-layer count of planned appends, so that a step can be captured once as a HIP graph.

Paper summary (gentlecold.top) s8: in every step each worker appends its token, the views
are rebuilt, then attention runs; s5: blocks stored once at local positions, queries
rotated per block. Each step is checked against the fp64 oracle over the blocks' current
contents (hw_testlib.assert_parity: rel L2, every row, lse), and graph replays against the
same steps run eagerly, bit for bit.
"""

import numpy as np
import pytest
import torch

from oracle import hogwild_oracle as O
from shared_kv_cache_amd import hogwild as H
from shared_kv_cache_amd import workloads as W

from hw_testlib import (DEV, TOL, assert_parity, decode_np, fill_layer, k_pool_token, kv_tensor,
                        make_cache, v_pool_token)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _small_workload(n_layers):
    """bf16, 4 workers, 8 KV heads x 128, 40 query heads: a 300-token prompt, three
    paragraphs, and unfinished steps of 62 (two tokens short of a 64-token page), 31 (one
    short of a 32-token group), 0 (empty) and 5 tokens; 64-token pages."""
    base = W.make("w4_16k", n_layers=n_layers)
    history = [0, 1, 2, 3]
    inprog = [4, 5, 6, 7]
    lengths = {0: 300, 1: 77, 2: 130, 3: 41, 4: 62, 5: 31, 6: 0, 7: 5}
    owners = {0: -1, 1: 0, 2: 1, 3: 2, 4: 0, 5: 1, 6: 2, 7: 3}
    return W.Workload(**{**base.__dict__, "name": "plan_small", "seed": 41, "n_workers": 4,
                         "page_size": 64, "history": history, "inprogress": inprog,
                         "lengths": lengths, "owners": owners, "n_pages": 40,
                         "max_position": 2048})


def test_planned_steps_match_the_oracle():
    # Six planned steps on two layers. Worker blocks grow by 1, 1, 1 and 2 tokens a step:
    # they cross a page boundary (62 -> 68), a group boundary (31 -> 37), start from empty
    # (0 -> 6) and take two tokens at once (5 -> 17). Each layer's append precedes its decode.
    wl = _small_workload(2)
    cache = make_cache(wl, max_splits=64)
    for layer in range(2):
        fill_layer(cache, wl, layer)
    views = wl.views()
    cache.set_views(views)
    tps = [1, 1, 1, 2]
    steps = 6
    free0 = H.hw_free_pages(cache.ctx)
    cache.plan_steps(steps, wl.inprogress, tps)
    host = {layer: {b: [np.asarray(x, np.float64) for x in wl.kv(layer, b)] for b in wl.blocks()}
            for layer in range(2)}
    with pytest.raises(H.HwError) as e:          # the views are fixed while the plan runs
        cache.set_views(views)
    assert e.value.status == H.HW_ERR_INVALID_ARG
    with pytest.raises(H.HwError) as e:
        cache.append(0, [4], [1], kv_tensor(np.zeros((1, 8, 128), np.float32), "bf16"),
                     kv_tensor(np.zeros((1, 8, 128), np.float32), "bf16"))
    assert e.value.status == H.HW_ERR_INVALID_ARG
    rng = np.random.default_rng(5)
    for step in range(1, steps + 1):
        for layer in range(2):
            k = W.round_to_bf16_values(rng.standard_normal((sum(tps), 8, 128), dtype=np.float32))
            v = W.round_to_bf16_values(rng.standard_normal((sum(tps), 8, 128), dtype=np.float32))
            cache.append_step(layer, kv_tensor(k, "bf16"), kv_tensor(v, "bf16"))
            r = 0
            for b, t in zip(wl.inprogress, tps):
                host[layer][b][0] = np.concatenate([host[layer][b][0], k[r:r + t].astype(np.float64)])
                host[layer][b][1] = np.concatenate([host[layer][b][1], v[r:r + t].astype(np.float64)])
                r += t
            q = wl.q(layer, step)
            out, lse = decode_np(cache, layer, q)
            blocks = {b: tuple(x) for b, x in host[layer].items()}
            ref, ref_lse = O.concurrent_attention(q.astype(np.float64), blocks, views, theta=wl.theta)
            assert_parity(f"planned step {step} layer {layer}", out, lse, ref, ref_lse,
                          TOL["bf16"], _say)
    cache.plan_end()
    for b, t in zip(wl.inprogress, tps):
        for layer in range(2):
            assert cache.block_info(b, layer)[0] == wl.lengths[b] + steps * t
    # pages the blocks did not fill went back; the pool holds exactly the grown blocks
    used = sum(-(-(wl.lengths[b] + steps * t) // 64) - -(-wl.lengths[b] // 64)
               for b, t in zip(wl.inprogress, tps))
    assert H.hw_free_pages(cache.ctx) == free0 - used
    # the appended keys and values are the pool bytes hw_append_kv would have written
    torch.cuda.synchronize()
    kp = cache.k_pool.cpu().view(torch.int16).numpy().view(np.uint16)
    vp = cache.v_pool.cpu().view(torch.int16).numpy().view(np.uint16)
    for b in wl.inprogress:
        length, pages = cache.block_info(b, 1)
        toks = np.arange(wl.lengths[b], length)
        kraw = host[1][b][0][toks].astype(np.float32)
        expect_k = O.rope_store_reference(kraw, toks, wl.theta, "bf16")
        for i, t in enumerate(toks):
            for h in range(8):
                np.testing.assert_array_equal(
                    kp[k_pool_token(cache, 1, pages[t // 64], h, t % 64)], expect_k[i, h])
                np.testing.assert_array_equal(
                    vp[v_pool_token(cache, 1, pages[t // 64], h, t % 64)],
                    O.bf16_bits_rne(host[1][b][1][t, h].astype(np.float32)))
    # after the plan, ordinary decodes upload fresh tables and still match
    cache.set_views(views)
    q = wl.q(1, 99)
    out, lse = decode_np(cache, 1, q)
    ref, ref_lse = O.concurrent_attention(q.astype(np.float64),
                                          {b: tuple(x) for b, x in host[1].items()}, views,
                                          theta=wl.theta)
    assert_parity("after the plan", out, lse, ref, ref_lse, TOL["bf16"], _say)
    cache.close()


def _w8_cache(steps):
    wl = W.make("w8_32k", steps=steps)
    cache = make_cache(wl)
    for layer in range(wl.n_layers):
        fill_layer(cache, wl, layer)
    cache.set_views(wl.views())
    cache.plan_steps(steps, wl.inprogress, [1] * wl.n_workers)
    return wl, cache


def test_w8_32k_step_graph_replays_equal_eager_and_the_oracle():
    # The w8_32k step as the bench times it: per layer (8 layer pools) each worker appends
    # one token, then the concurrent decode runs. Cache A runs three steps eagerly; cache B,
    # in the same state, captures ONE step as a HIP graph and replays it three times. The
    # replays must equal the eager steps bit for bit, and match the oracle (layers 0 and 5).
    plan = 4
    wl, ca = _w8_cache(plan)
    _, cb = _w8_cache(plan)
    L, n = wl.n_layers, wl.n_workers
    kv = [[tuple(kv_tensor(x, "bf16") for x in wl.step_kv(layer, s)) for layer in range(L)]
          for s in range(1, 4)]
    qs = [[torch.from_numpy(wl.q(layer, s)).to(DEV) for layer in range(L)] for s in range(1, 4)]
    outs = [torch.empty((n, wl.n_q_heads, wl.head_dim), device=DEV) for _ in range(L)]
    lses = [torch.empty((n, wl.n_q_heads), device=DEV) for _ in range(L)]
    eager = []
    for s in range(3):
        for layer in range(L):
            ca.append_step(layer, *kv[s][layer])
            ca.decode(layer, qs[s][layer], out=outs[layer], lse=lses[layer])
        torch.cuda.synchronize()
        eager.append(([o.clone() for o in outs], [x.clone() for x in lses]))
    # graph: inputs staged in fixed buffers that the host refills between replays
    kbuf = [torch.empty_like(kv[0][layer][0]) for layer in range(L)]
    vbuf = [torch.empty_like(kv[0][layer][1]) for layer in range(L)]
    qbuf = [torch.empty_like(qs[0][layer]) for layer in range(L)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        for layer in range(L):
            cb.append_step(layer, kbuf[layer], vbuf[layer])
            cb.decode(layer, qbuf[layer], out=outs[layer], lse=lses[layer])
    torch.cuda.synchronize()
    hist = {layer: {} for layer in (0, 5)}
    for s in range(3):
        for layer in range(L):
            kbuf[layer].copy_(kv[s][layer][0])
            vbuf[layer].copy_(kv[s][layer][1])
            qbuf[layer].copy_(qs[s][layer])
            outs[layer].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer in range(L):
            assert torch.equal(outs[layer], eager[s][0][layer]), (s, layer)
            assert torch.equal(lses[layer], eager[s][1][layer]), (s, layer)
        for layer in (0, 5):
            hist[layer][s + 1] = wl.step_kv(layer, s + 1)
            blocks = {}
            for b in wl.blocks():
                k0, v0 = wl.kv(layer, b)
                if b in wl.inprogress:
                    w = wl.inprogress.index(b)
                    k0 = np.concatenate([k0] + [hist[layer][t][0][w:w + 1] for t in range(1, s + 2)])
                    v0 = np.concatenate([v0] + [hist[layer][t][1][w:w + 1] for t in range(1, s + 2)])
                blocks[b] = (k0.astype(np.float64), v0.astype(np.float64))
            q = wl.q(layer, s + 1)
            ref, ref_lse = O.concurrent_attention(q.astype(np.float64), blocks, wl.views(),
                                                  theta=wl.theta)
            assert_parity(f"w8_32k replay {s + 1} layer {layer}", outs[layer].cpu().numpy(),
                          lses[layer].cpu().numpy(), ref, ref_lse, TOL["bf16"], _say)
        _say(f"replay {s + 1}: equal to the eager step")
    # two more replays run past the 4-step window: the fifth append is dropped and
    # reported when the plan ends; lengths advance by the 4 planned steps only
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    with pytest.raises(H.HwError) as e:
        cb.plan_end()
    assert e.value.status == H.HW_ERR_INVALID_ARG and "dropped" in e.value.message
    ca.plan_end()
    for b in wl.inprogress:
        for layer in range(L):
            assert cb.block_info(b, layer)[0] == wl.lengths[b] + plan
            assert ca.block_info(b, layer)[0] == wl.lengths[b] + 3
    ca.close()
    cb.close()


def test_plan_step_order_rules():
    # A layer's planned step is append, then decode; the decode's kernels advance the
    # layer's count. A second append before the decode is refused; a decode without an
    # append sees the state as it is (bitwise the same output twice); a step appended but
    # not decoded when the plan ends still counts.
    wl = _small_workload(1)
    cache = make_cache(wl, max_splits=64)
    fill_layer(cache, wl, 0)
    cache.set_views(wl.views())
    cache.plan_steps(3, wl.inprogress, [1, 1, 1, 1])
    rng = np.random.default_rng(9)

    def kv():
        return [kv_tensor(W.round_to_bf16_values(rng.standard_normal((4, 8, 128), dtype=np.float32)),
                          "bf16") for _ in range(2)]

    q = wl.q(0, 1)
    cache.append_step(0, *kv())
    with pytest.raises(H.HwError) as e:
        cache.append_step(0, *kv())
    assert e.value.status == H.HW_ERR_INVALID_ARG
    a1 = decode_np(cache, 0, q)
    a2 = decode_np(cache, 0, q)          # no append in between: same state, same bits
    np.testing.assert_array_equal(a1[0], a2[0])
    np.testing.assert_array_equal(a1[1], a2[1])
    cache.append_step(0, *kv())
    decode_np(cache, 0, q)
    cache.append_step(0, *kv())          # third step appended, never decoded
    torch.cuda.synchronize()
    cache.plan_end()
    for b in wl.inprogress:
        assert cache.block_info(b, 0)[0] == wl.lengths[b] + 3
    cache.close()


def _pool_bits(cache):
    torch.cuda.synchronize()
    return (cache.k_pool.view(torch.int16).cpu(), cache.v_pool.view(torch.int16).cpu())


def test_fused_step_equals_append_then_decode():
    # hw_decode_step against hw_append_step + hw_concurrent_decode on two caches in the same
    # state: six steps on two layers of the small workload (blocks crossing a page and a
    # group boundary, starting empty, taking two tokens a step; 20 rows: the 8-wave kernel).
    # Outputs, lse and every pool byte must agree bit for bit, and the lengths after the plan.
    wl = _small_workload(2)
    caches = [make_cache(wl, max_splits=64) for _ in range(2)]
    tps = [1, 1, 1, 2]
    for c in caches:
        for layer in range(2):
            fill_layer(c, wl, layer)
        c.set_views(wl.views())
        c.plan_steps(6, wl.inprogress, tps)
    rng = np.random.default_rng(11)
    for step in range(1, 7):
        for layer in range(2):
            k, v = (kv_tensor(W.round_to_bf16_values(rng.standard_normal((sum(tps), 8, 128),
                                                                       dtype=np.float32)), "bf16")
                    for _ in range(2))
            q = torch.from_numpy(wl.q(layer, step)).to(DEV)
            caches[0].append_step(layer, k, v)
            o0, l0 = caches[0].decode(layer, q)
            o1, l1 = caches[1].decode_step(layer, k, v, q)
            torch.cuda.synchronize()
            assert torch.equal(o0, o1) and torch.equal(l0, l1), (step, layer)
    a, b = _pool_bits(caches[0]), _pool_bits(caches[1])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    for c in caches:
        c.plan_end()
    for blk, t in zip(wl.inprogress, tps):
        for layer in range(2):
            assert caches[1].block_info(blk, layer)[0] == wl.lengths[blk] + 6 * t
    _say("fused small: 12 steps bitwise equal to append + decode, pools equal")
    for c in caches:
        c.close()


def test_w8_32k_fused_step_graph_equals_two_call_steps():
    # The w8_32k step with its appends fused into the decodes (40 rows: the cooperative
    # kernel), captured once as a HIP graph and replayed three times, against the same steps
    # run eagerly with hw_append_step + hw_concurrent_decode: bitwise equal outputs and pools.
    plan = 4
    wl, ca = _w8_cache(plan)
    _, cb = _w8_cache(plan)
    L, n = wl.n_layers, wl.n_workers
    kv = [[tuple(kv_tensor(x, "bf16") for x in wl.step_kv(layer, s)) for layer in range(L)]
          for s in range(1, 4)]
    qs = [[torch.from_numpy(wl.q(layer, s)).to(DEV) for layer in range(L)] for s in range(1, 4)]
    outs = [torch.empty((n, wl.n_q_heads, wl.head_dim), device=DEV) for _ in range(L)]
    lses = [torch.empty((n, wl.n_q_heads), device=DEV) for _ in range(L)]
    eager = []
    for s in range(3):
        for layer in range(L):
            ca.append_step(layer, *kv[s][layer])
            ca.decode(layer, qs[s][layer], out=outs[layer], lse=lses[layer])
        torch.cuda.synchronize()
        eager.append(([o.clone() for o in outs], [x.clone() for x in lses]))
    kbuf = [torch.empty_like(kv[0][layer][0]) for layer in range(L)]
    vbuf = [torch.empty_like(kv[0][layer][1]) for layer in range(L)]
    qbuf = [torch.empty_like(qs[0][layer]) for layer in range(L)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        for layer in range(L):
            cb.decode_step(layer, kbuf[layer], vbuf[layer], qbuf[layer], out=outs[layer],
                           lse=lses[layer])
    torch.cuda.synchronize()
    for s in range(3):
        for layer in range(L):
            kbuf[layer].copy_(kv[s][layer][0])
            vbuf[layer].copy_(kv[s][layer][1])
            qbuf[layer].copy_(qs[s][layer])
            outs[layer].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer in range(L):
            assert torch.equal(outs[layer], eager[s][0][layer]), (s, layer)
            assert torch.equal(lses[layer], eager[s][1][layer]), (s, layer)
        _say(f"fused replay {s + 1}: equal to the two-call eager step")
    a, b = _pool_bits(ca), _pool_bits(cb)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # past the window: the fifth fused step writes nothing and is reported
    g.replay()
    g.replay()
    torch.cuda.synchronize()
    with pytest.raises(H.HwError) as e:
        cb.plan_end()
    assert e.value.status == H.HW_ERR_INVALID_ARG and "dropped" in e.value.message
    ca.plan_end()
    for blk in wl.inprogress:
        for layer in range(L):
            assert cb.block_info(blk, layer)[0] == wl.lengths[blk] + plan
    ca.close()
    cb.close()
