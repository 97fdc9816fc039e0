"""hw_concurrent_decode_noalloc: the decode with its split partials in the library's static
device array instead of the workspace, for callers that cannot allocate. It must give what
hw_concurrent_decode gives (the same kernels and tables: bit for bit), call after call on
the same array, including a smaller input after a larger one, and refuse a partition count
whose partials do not fit the array.
"""

import numpy as np
import pytest
import torch

from oracle import hogwild_oracle as O
from shared_kv_cache_amd import hogwild as H
from shared_kv_cache_amd import workloads as W

from hw_testlib import DEV, TOL, assert_parity, fill_layer, make_cache, oracle_blocks

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _both(cache, q):
    """The same decode through both entry points (C ABI): (workspace result, static result)."""
    n, hq, d = q.shape
    stream = torch.cuda.current_stream().cuda_stream
    res = []
    for fn in (H.hw_concurrent_decode, H.hw_concurrent_decode_noalloc):
        out = torch.full((n, hq, d), float("nan"), device=DEV)
        lse = torch.full((n, hq), float("nan"), device=DEV)
        fn(cache.ctx, 0, q.data_ptr(), out.data_ptr(), lse.data_ptr(), stream)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    return res


def test_noalloc_decode_equals_the_workspace_decode():
    # The w8_32k layer (8 workers x 8 heads = 64 rows per KV head, 32 partitions: 8.5 MB
    # of partials), then a smaller input on the same array: three workers' views.
    wl = W.make("w8_32k", n_layers=1)
    cache = make_cache(wl)
    fill_layer(cache, wl, 0)
    views = wl.views()
    q_all = wl.q(0)
    heads = [0, 9, 63]
    for name, nw in (("8 workers", 8), ("3 workers", 3)):
        cache.set_views(views[:nw])
        q = torch.from_numpy(np.ascontiguousarray(q_all[:nw])).to(DEV)
        (o_ws, l_ws), (o_na, l_na) = _both(cache, q)
        np.testing.assert_array_equal(o_na, o_ws)
        np.testing.assert_array_equal(l_na, l_ws)
        ref, ref_lse = O.concurrent_attention(q_all[:nw].astype(np.float64), oracle_blocks(wl, 0),
                                              views[:nw], theta=wl.theta, heads=heads)
        assert_parity(f"noalloc, {name}", o_na[:, heads], l_na[:, heads], ref[:, heads],
                      ref_lse[:, heads], TOL["bf16"], _say)
    # captured in a HIP graph (the tables of these views are current) and replayed twice
    q = torch.from_numpy(np.ascontiguousarray(q_all[:3])).to(DEV)
    out = torch.empty((3, wl.n_q_heads, wl.head_dim), device=DEV)
    lse = torch.empty((3, wl.n_q_heads), device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        H.hw_concurrent_decode_noalloc(cache.ctx, 0, q.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                       side.cuda_stream)
    for _ in range(2):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), o_ws)
        np.testing.assert_array_equal(lse.cpu().numpy(), l_ws)
    # partials beyond the array: refused before anything is enqueued
    cache.set_views(views)
    H.hw_set_split(cache.ctx, 200)          # 200 x 8 x 64 x 129 x 4 B = 52.8 MB > 16 MiB
    out8 = torch.zeros((8, wl.n_q_heads, wl.head_dim), device=DEV)
    q8 = torch.from_numpy(q_all).to(DEV)
    with pytest.raises(H.HwError) as e:
        H.hw_concurrent_decode_noalloc(cache.ctx, 0, q8.data_ptr(), out8.data_ptr(), None,
                                       torch.cuda.current_stream().cuda_stream)
    assert e.value.status == H.HW_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out8).item() == 0
    cache.close()
