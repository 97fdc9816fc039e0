"""Host logic of the C-ABI library, checked on a machine without a GPU.

The library is loaded through its C ABI; only host-only entry points are
called (no kernel launches, no device memory). Slot assignment, page
allocation and view resolution are compared bit-exactly with a small Python
model written here from the header's specification, and every error path is
forced from the host and shown to leave the state unchanged.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import hogwild_oracle as O
from shared_kv_cache_amd import hogwild as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_K, FAKE_V = 1 << 20, 2 << 20       # never dereferenced by host-only calls


def make_cfg(**kw):
    base = dict(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, page_size=64, n_pages=16,
                max_blocks=16, max_workers=4, max_position=4096, max_splits=0,
                max_query_tokens=0, kv_dtype=H.HW_BF16, page_seed=0, rope_theta=1e4, softmax_scale=0.0,
                k_pool=FAKE_K, v_pool=FAKE_V)
    base.update(kw)
    return H.HwConfig(**base)


@pytest.fixture
def ctx():
    c = H.hw_create(make_cfg())
    yield c
    H.hw_destroy(c)


# ------------------------------------------------------------------- exports

def test_library_exports_every_declared_symbol():
    lib = H.load_library()
    declared = set()
    for name in ("hogwild.h", "hogwild_debug.h"):
        text = open(os.path.join(ROOT, "include", name)).read()
        declared |= set(re.findall(r"\b(hw_[a-z_]+)\s*\(", text))
    assert declared == set(H.EXPORTS)
    for sym in declared:
        assert hasattr(lib, sym), sym          # dlsym succeeds


# ----------------------------------------------------------------- creation

@pytest.mark.parametrize("field,value", [
    ("n_layers", 0), ("n_q_heads", 7), ("n_kv_heads", 0), ("head_dim", 96), ("page_size", 48),
    ("n_pages", 0), ("max_blocks", 0), ("max_workers", 0), ("max_position", 0),
    ("max_splits", -1), ("max_query_tokens", -1), ("max_query_tokens", 1025),
    ("kv_dtype", 7), ("rope_theta", 1.0), ("softmax_scale", -1.0),
    ("k_pool", 0), ("v_pool", FAKE_V + 8),
])
def test_create_rejects_bad_config(field, value):
    with pytest.raises(H.HwError) as e:
        H.hw_create(make_cfg(**{field: value}))
    assert e.value.status == H.HW_ERR_INVALID_ARG and e.value.message


def test_create_bounds_stacked_rows():
    # (worker, query token, head) rows of one KV head must stay below 2^22 (the kernels'
    # fp32 row -> (token, worker) division is exact there)
    H.hw_destroy(H.hw_create(make_cfg(max_workers=1024, max_query_tokens=1023, n_q_heads=8)))
    with pytest.raises(H.HwError) as e:
        H.hw_create(make_cfg(max_workers=1024, max_query_tokens=1024, n_q_heads=8))
    assert e.value.status == H.HW_ERR_INVALID_ARG


def test_workspace_size_formula(ctx):
    d, half, max_pos = 128, 64, 4096
    al = lambda x: (x + 255) // 256 * 256
    max_groups = 16 * (64 // 32)
    rows = 4 * 4
    expect = al(max_pos * half * 8) + al(half * 8)
    expect += al(al(16 * 4 * 4) + al(max_groups * 8 * 4))   # up to 8 ints per group descriptor
    expect += al(256 * 2 * rows * d * 4)
    expect += al(256 * 2 * rows * 4)
    # step-plan region: counters (2 layers + overflow flag), the fused step's table (64
    # blocks x 4 ints), {d0, rate} offsets, 4-int descriptors
    expect += al(al(3 * 4) + al(64 * 4 * 4) + al(16 * 4 * 2 * 4) + al(max_groups * 4 * 4))
    assert H.hw_workspace_bytes(ctx) == expect
    # several query tokens per worker: partials for every (worker, token, head) row
    c3 = H.hw_create(make_cfg(max_query_tokens=3))
    rows3 = 4 * 3 * 4
    expect3 = expect - al(256 * 2 * rows * d * 4) - al(256 * 2 * rows * 4)
    expect3 += al(256 * 2 * rows3 * d * 4) + al(256 * 2 * rows3 * 4)
    assert H.hw_workspace_bytes(c3) == expect3
    H.hw_destroy(c3)


def test_calls_without_workspace_or_views(ctx):
    with pytest.raises(H.HwError) as e:
        H.hw_append_kv(ctx, 0, [0], [4], FAKE_K, FAKE_V, 0)
    assert e.value.status == H.HW_ERR_WORKSPACE
    with pytest.raises(H.HwError) as e:
        H.hw_concurrent_decode(ctx, 0, FAKE_K, FAKE_V, None, 0)
    assert e.value.status == H.HW_ERR_WORKSPACE
    with pytest.raises(H.HwError) as e:
        H.hw_concurrent_decode_tokens(ctx, 0, 1, FAKE_K, FAKE_V, None, 0)
    assert e.value.status == H.HW_ERR_WORKSPACE
    for n_new in (0, 2):          # max_query_tokens is 1 here
        with pytest.raises(H.HwError) as e:
            H.hw_concurrent_decode_tokens(ctx, 0, n_new, FAKE_K, FAKE_V, None, 0)
        assert e.value.status == H.HW_ERR_INVALID_ARG
    with pytest.raises(H.HwError) as e:
        H.hw_debug_resolve(ctx, 0, 1)
    assert e.value.status == H.HW_ERR_STALE_VIEW


# ------------------------------------------------------ page allocation model

def splitmix_shuffle(n, seed):
    """Fisher-Yates over 0..n-1 driven by splitmix64 (Steele, Lea, Flood)."""
    mask = (1 << 64) - 1
    state = seed
    order = list(range(n))
    for i in range(n - 1, 0, -1):
        state = (state + 0x9E3779B97F4A7C15) & mask
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        z ^= z >> 31
        j = z % (i + 1)
        order[i], order[j] = order[j], order[i]
    return order


class HostModel:
    """Python model of the header's slot-assignment and page rules."""

    def __init__(self, n_layers, page_size, n_pages, seed):
        order = splitmix_shuffle(n_pages, seed) if seed else list(range(n_pages))
        self.free = list(reversed(order))       # pop() hands out order[0] first
        self.ps = page_size
        self.n_layers = n_layers
        self.pages, self.len = {}, {}

    def reserve(self, layer, ids, counts):
        runs, row = [], 0
        need_total = 0
        for b, n in zip(ids, counts):
            lens = self.len.setdefault(b, [0] * self.n_layers)
            pages = self.pages.setdefault(b, [])
            need = -(-max(max(lens), lens[layer] + n) // self.ps)
            need_total += max(0, need - len(pages))
        if need_total > len(self.free):
            return None
        for b, n in zip(ids, counts):
            lens, pages = self.len[b], self.pages[b]
            need = -(-max(max(lens), lens[layer] + n) // self.ps)
            while len(pages) < need:
                pages.append(self.free.pop())
            pos, left = lens[layer], n
            while left:
                slot = pos % self.ps
                cnt = min(left, self.ps - slot)
                runs.append((row, pages[pos // self.ps], slot, cnt, pos))
                row, pos, left = row + cnt, pos + cnt, left - cnt
            lens[layer] += n
        return runs

    def reset(self, b):
        for p in reversed(self.pages.get(b, [])):
            self.free.append(p)
        self.pages[b] = []
        self.len[b] = [0] * self.n_layers


@pytest.mark.parametrize("seed", [0, 1, 0xDEADBEEF])
def test_slot_assignment_and_pages_bit_exact(seed):
    cfg = make_cfg(n_pages=40, page_size=64, page_seed=seed, max_blocks=8)
    c = H.hw_create(cfg)
    model = HostModel(2, 64, 40, seed)
    rng = np.random.default_rng(seed)
    try:
        for step in range(60):
            layer = int(rng.integers(0, 2))
            k = int(rng.integers(1, 4))
            ids = [int(x) for x in rng.choice(8, size=k, replace=False)]
            counts = [int(x) for x in rng.integers(0, 90, size=k)]
            expect = model.reserve(layer, ids, counts)
            if expect is None:
                free0 = H.hw_free_pages(c)
                with pytest.raises(H.HwError) as e:
                    H.hw_debug_reserve(c, layer, ids, counts)
                assert e.value.status == H.HW_ERR_OUT_OF_PAGES
                assert H.hw_free_pages(c) == free0
                victim = ids[0]
                model.reset(victim)
                H.hw_reset_block(c, victim)
                continue
            got = H.hw_debug_reserve(c, layer, ids, counts)
            assert got == expect
            assert H.hw_free_pages(c) == len(model.free)
            for b in ids:
                for lay in range(2):
                    length, pages = H.hw_block_info(c, b, lay)
                    assert length == model.len[b][lay] and pages == model.pages[b]
    finally:
        H.hw_destroy(c)


def test_scattered_pages_are_a_permutation():
    c = H.hw_create(make_cfg(n_pages=64, page_size=32, page_seed=0x5EED, max_blocks=2))
    runs = H.hw_debug_reserve(c, 0, [0], [64 * 32])
    pages = [r[1] for r in runs]
    assert sorted(pages) == list(range(64)) and pages != list(range(64))
    assert pages == splitmix_shuffle(64, 0x5EED)
    H.hw_destroy(c)


@pytest.mark.parametrize("ids,counts,status", [
    ([16], [1], H.HW_ERR_INVALID_ARG),           # id out of range
    ([-1], [1], H.HW_ERR_INVALID_ARG),
    ([3, 3], [1, 1], H.HW_ERR_INVALID_ARG),      # repeated id
    ([2], [-1], H.HW_ERR_INVALID_ARG),           # negative count
    ([2], [4097], H.HW_ERR_INVALID_ARG),         # reaches max_position
    ([2, 3], [600, 600], H.HW_ERR_OUT_OF_PAGES), # 10 + 10 pages > 16
])
def test_append_errors_leave_state_unchanged(ctx, ids, counts, status):
    H.hw_debug_reserve(ctx, 0, [5], [70])
    before = (H.hw_free_pages(ctx), H.hw_block_info(ctx, 5, 0), H.hw_block_info(ctx, 2, 0))
    with pytest.raises(H.HwError) as e:
        H.hw_debug_reserve(ctx, 0, ids, counts)
    assert e.value.status == status
    assert (H.hw_free_pages(ctx), H.hw_block_info(ctx, 5, 0), H.hw_block_info(ctx, 2, 0)) == before
    with pytest.raises(H.HwError):
        H.hw_debug_reserve(ctx, 2, [1], [1])      # layer out of range


def test_pages_shared_across_layers(ctx):
    r0 = H.hw_debug_reserve(ctx, 0, [1], [100])   # 2 pages
    r1 = H.hw_debug_reserve(ctx, 1, [1], [30])    # same pages, no new ones
    assert [r[1] for r in r1] == [r0[0][1]] and H.hw_free_pages(ctx) == 14
    r2 = H.hw_debug_reserve(ctx, 1, [1], [100])   # layer 1 grows to 130 -> 3rd page
    assert H.hw_free_pages(ctx) == 13
    assert r2[0][1:] == (r0[0][1], 30, 34, 30) and r2[1][2:] == (0, 64, 64) and r2[2][2:] == (0, 2, 128)


# ------------------------------------------------------------- view model

def model_resolve(lengths, pages, views, offsets, q_pos, page_size, max_position):
    """Python model of the resolution specified in hogwild_debug.h."""
    n = len(views)
    segs = []
    all_offs, all_q = [], []
    for w, v in enumerate(views):
        offs = offsets[w] if offsets is not None else O.default_offsets(v, lengths)
        if q_pos is not None:
            qp = q_pos[w]
        else:
            qp = offs[-1] + lengths[v[-1]] - 1 if v else -1
        err = O.view_error(v, offs, lengths, qp)
        if err:
            return err
        for b, o in zip(v, offs):
            if lengths[b] and qp - o >= max_position:
                return "delta"
        all_offs.append(offs)
        all_q.append(qp)
        for b in v:
            if lengths[b] > 0 and b not in segs:
                segs.append(b)
    delta = [[-1] * n for _ in segs]
    for w, v in enumerate(views):
        for b, o in zip(v, all_offs[w]):
            if b in segs:
                delta[segs.index(b)][w] = all_q[w] - o
    groups = []
    for s, b in enumerate(segs):
        for t in range(0, lengths[b], 32):
            groups.append((pages[b][t // page_size], (t % page_size) // 32, s, min(32, lengths[b] - t)))
    return segs, delta, groups


def _fill(c, layer, lens):
    for b, n in lens.items():
        if n:
            H.hw_debug_reserve(c, layer, [b], [n])


def _pages_of(c, blocks, layer=0):
    info = {b: H.hw_block_info(c, b, layer) for b in blocks}
    return {b: i[0] for b, i in info.items()}, {b: i[1] for b, i in info.items()}


@pytest.mark.parametrize("seed", range(6))
def test_resolution_bit_exact(seed):
    rng = np.random.default_rng(50 + seed)
    c = H.hw_create(make_cfg(n_pages=64, page_size=64, max_blocks=12, max_workers=4,
                             page_seed=seed))
    try:
        n = int(rng.integers(1, 5))
        history = [0, 1, 2]
        inprog = [3 + w for w in range(n)]
        lens = {b: int(rng.integers(1, 200)) for b in history}
        lens.update({b: int(rng.integers(0 if w else 1, 70)) for w, b in enumerate(inprog)})
        _fill(c, 0, lens)
        views = [O.canonical_view(w, history, inprog) for w in range(n)]
        lengths, pages = _pages_of(c, history + inprog)
        offsets = q_pos = None
        if seed % 2:        # explicit offsets with gaps and a later query
            offsets = []
            for v in views:
                acc, off = int(rng.integers(0, 5)), []
                for b in v:
                    off.append(acc)
                    acc += lengths[b] + int(rng.integers(0, 9))
                offsets.append(off)
            q_pos = [offsets[w][-1] + lengths[v[-1]] + int(rng.integers(0, 3)) for w, v in enumerate(views)]
        H.hw_set_views(c, views, offsets, q_pos)
        got = H.hw_debug_resolve(c, 0, n)
        segs, delta, groups = model_resolve(lengths, pages, views, offsets, q_pos, 64, 4096)
        assert got["segs"] == segs and got["delta"] == delta and got["groups"] == groups
        assert got["n_groups"] == len(groups)
        # layer 1 holds nothing yet: every view is empty there
        empty = H.hw_debug_resolve(c, 1, n)
        assert empty["n_groups"] == 0 and empty["n_segs"] == 0
    finally:
        H.hw_destroy(c)


def test_subset_views_and_visibility(ctx):
    _fill(ctx, 0, {0: 40, 1: 10, 2: 12})
    # worker 0 sees only the common block and its own (no-sync style view)
    H.hw_set_views(ctx, [[0, 1], [0, 1, 2]])
    got = H.hw_debug_resolve(ctx, 0, 2)
    assert got["segs"] == [0, 1, 2]
    assert got["delta"] == [[49, 61], [9, 21], [-1, 11]]


@pytest.mark.parametrize("offsets,q_pos,why", [
    ([[0, 30, 40]], None, "overlapping blocks"),
    ([[0, 40, 50]], [55], "key after query"),
    ([[0, 40, 4000]], [4100], "delta"),
])
def test_stale_views_rejected_like_the_oracle(ctx, offsets, q_pos, why):
    _fill(ctx, 0, {0: 40, 1: 10, 2: 12})
    H.hw_set_views(ctx, [[0, 1, 2]], offsets, q_pos)
    lengths, pages = _pages_of(ctx, [0, 1, 2])
    assert model_resolve(lengths, pages, [[0, 1, 2]], offsets, q_pos, 64, 4096) == why
    with pytest.raises(H.HwError) as e:
        H.hw_debug_resolve(ctx, 0, 1)
    assert e.value.status == H.HW_ERR_STALE_VIEW


@pytest.mark.parametrize("views,offsets,q_pos", [
    ([[0, 0]], None, None),                   # repeated block
    ([[0, 99]], None, None),                  # id out of range
    ([[0]] * 5, None, None),                  # more workers than max_workers
    ([[0, 1]], [[0, -4]], None),              # negative offset
    ([[0, 1]], None, [-2]),                   # bad q_pos
    ([], None, None),                         # no workers
])
def test_set_views_rejects_bad_input(ctx, views, offsets, q_pos):
    H.hw_set_views(ctx, [[0]])
    with pytest.raises(H.HwError) as e:
        H.hw_set_views(ctx, views, offsets, q_pos)
    assert e.value.status == H.HW_ERR_INVALID_ARG
    _fill(ctx, 0, {0: 5})
    assert H.hw_debug_resolve(ctx, 0, 1)["segs"] == [0]      # previous views kept


def test_split_choice_and_override(ctx):
    _fill(ctx, 0, {0: 900, 1: 24})
    H.hw_set_views(ctx, [[0, 1]])
    auto = H.hw_debug_resolve(ctx, 0, 1)["n_splits"]
    # 30 groups: min(3/4 of 256 CUs / (2 KV heads * 1 row block), 30 // 4) = 7 without a GPU,
    # then the fewest workgroups that give each of their 8 waves at most one group: ceil(30 / 8)
    assert auto == 4
    H.hw_set_split(ctx, 5)
    assert H.hw_debug_resolve(ctx, 0, 1)["n_splits"] == 5
    with pytest.raises(H.HwError):
        H.hw_set_split(ctx, 257)
    H.hw_set_split(ctx, 0)
    assert H.hw_debug_resolve(ctx, 0, 1)["n_splits"] == auto


@pytest.mark.parametrize("tokens", [16 * 32, 17 * 32, 30 * 32, 100 * 32, 142 * 32 - 5, 190 * 32])
def test_auto_split_count_rules(tokens):
    # Without a GPU the library assumes 256 CUs: 3/4 of them over 2 KV heads is 96 partitions,
    # at least 4 groups each; one partition for at most 16 groups; and a small cache takes the
    # fewest workgroups whose 8 waves get at most one group each.
    c = H.hw_create(make_cfg(n_pages=96, max_position=8192))
    try:
        _fill(c, 0, {0: tokens})
        H.hw_set_views(c, [[0]])
        g = (tokens + 31) // 32
        want = 1 if g <= 16 else min(96, max(1, g // 4), (g + 7) // 8)
        assert H.hw_debug_resolve(c, 0, 1)["n_splits"] == want
    finally:
        H.hw_destroy(c)


@pytest.mark.parametrize("src,nbytes,sink,n_blocks", [
    (0, 1 << 20, 4096, 4),          # no source
    (4096, 1 << 20, 0, 4),          # no sink
    (4100, 1 << 20, 4096, 4),       # source not 16-byte aligned
    (4096, 1000, 4096, 4),          # size not a multiple of 16
    (4096, 0, 4096, 4),             # empty
    (4096, 1 << 20, 4096, 0),       # no workgroups
    (4096, 1 << 20, 4096, 65536),   # too many workgroups
])
def test_stream_read_probe_rejects_bad_arguments(src, nbytes, sink, n_blocks):
    # validated on the host before any HIP call, so no GPU is needed and nothing is enqueued
    with pytest.raises(H.HwError) as e:
        H.hw_debug_stream_read(src, nbytes, sink, n_blocks, 0)
    assert e.value.status == H.HW_ERR_INVALID_ARG
    assert "hw_debug_stream_read" in H.hw_last_error(None)


# ---- KV partitioning (host only) ----------------------------------------------------------

def _partition_cost(first, a, b, alpha):
    """Cost of partition [a, b): one per group plus alpha per block it touches."""
    if b <= a:
        return 0.0
    return (b - a) + alpha * sum(1 for i in range(a, b) if i == a or first[i])


def _best_max_cost(first, n, alpha):
    """Brute force: the smallest largest-partition cost over all cut vectors."""
    import itertools
    g = len(first)
    best = float("inf")
    for cuts in itertools.combinations_with_replacement(range(g + 1), n - 1):
        b = [0, *cuts, g]
        best = min(best, max(_partition_cost(first, b[i], b[i + 1], alpha) for i in range(n)))
    return best


def test_partition_bounds_are_min_max_optimal():
    rng = np.random.default_rng(7)
    for case in range(60):
        g = int(rng.integers(0, 13))
        n = int(rng.integers(1, 5))
        first = [1 if (i == 0 or rng.random() < 0.3) else 0 for i in range(g)]
        alpha = float(rng.choice([0.0, 0.5, 2.0, 3.0]))
        b = H.hw_debug_partition(first, n, alpha)
        assert len(b) == n + 1 and b[0] == 0 and b[-1] == g
        assert all(b[i] <= b[i + 1] for i in range(n)), b
        got = max(_partition_cost(first, b[i], b[i + 1], alpha) for i in range(n)) if g else 0.0
        want = _best_max_cost(first, n, alpha) if g else 0.0
        assert got <= want + 1e-4, (case, first, n, alpha, b, got, want)


def test_partition_without_block_weight_is_balanced():
    # alpha 0: partitions of floor(G / n) or ceil(G / n) groups (the even split)
    for g, n in [(1149, 24), (541, 24), (560, 24), (7, 3), (5, 8), (256, 256), (1000, 7)]:
        b = H.hw_debug_partition([1] + [0] * (g - 1), n, 0.0)
        sizes = [b[i + 1] - b[i] for i in range(n)]
        assert max(sizes) == -(-g // n) and min(sizes) == g // n and sum(sizes) == g, sizes


def test_partition_gives_block_rich_ranges_fewer_groups():
    # a long block, then eight short ones (the shape of a common history followed by the
    # workers' in-progress blocks): weighting blocks shrinks the partitions that hold them
    lens = [1024, 11, 22, 18, 15, 22, 16, 3, 18]
    first = []
    for n_g in lens:
        first += [1] + [0] * (n_g - 1)
    b = H.hw_debug_partition(first, 24, 3.0)
    sizes = [b[i + 1] - b[i] for i in range(24)]
    assert max(sizes[-3:]) < min(sizes[:20])
    worst = max(_partition_cost(first, b[i], b[i + 1], 3.0) for i in range(24))
    assert worst <= 52.0 + 1e-6


def test_partition_rejects_bad_arguments():
    for args in [([1, 0], 0, 1.0), ([1, 0], 2, -1.0), ([1, 0], 2, float("nan"))]:
        with pytest.raises(H.HwError) as e:
            H.hw_debug_partition(*args)
        assert e.value.status == H.HW_ERR_INVALID_ARG


# ------------------------------------------------------------------ step plans

def test_step_plan_validation_before_any_change(ctx):
    # hw_plan_steps checks its arguments before it needs the workspace or touches a page
    with pytest.raises(H.HwError) as e:                      # no views yet
        H.hw_plan_steps(ctx, 4, [1], [1], 0)
    assert e.value.status == H.HW_ERR_STALE_VIEW
    H.hw_debug_reserve(ctx, 0, [0, 1], [40, 7])
    H.hw_debug_reserve(ctx, 1, [0, 1], [40, 7])
    H.hw_set_views(ctx, [[0, 1]])
    free0 = H.hw_free_pages(ctx)
    bad = [
        (dict(n_steps=0, ids=[1], tps=[1]), H.HW_ERR_INVALID_ARG),
        (dict(n_steps=4, ids=[1, 1], tps=[1, 1]), H.HW_ERR_INVALID_ARG),
        (dict(n_steps=4, ids=[99], tps=[1]), H.HW_ERR_INVALID_ARG),
        (dict(n_steps=4, ids=[1], tps=[-1]), H.HW_ERR_INVALID_ARG),
        (dict(n_steps=5000, ids=[1], tps=[1]), H.HW_ERR_INVALID_ARG),    # past max_position
        (dict(n_steps=4, ids=[1], tps=[1]), H.HW_ERR_WORKSPACE),         # valid, no workspace
    ]
    for kw, status in bad:
        with pytest.raises(H.HwError) as e:
            H.hw_plan_steps(ctx, kw["n_steps"], kw["ids"], kw["tps"], 0)
        assert e.value.status == status, kw
        assert H.hw_free_pages(ctx) == free0
    # explicit offsets or query positions cannot grow with the plan
    H.hw_set_views(ctx, [[0, 1]], offsets=[[0, 40]])
    with pytest.raises(H.HwError) as e:
        H.hw_plan_steps(ctx, 4, [1], [1], 0)
    assert e.value.status == H.HW_ERR_INVALID_ARG
    # lengths that differ between layers
    H.hw_set_views(ctx, [[0, 1]])
    H.hw_debug_reserve(ctx, 1, [1], [1])
    with pytest.raises(H.HwError) as e:
        H.hw_plan_steps(ctx, 4, [1], [1], 0)
    assert e.value.status == H.HW_ERR_INVALID_ARG and "layers" in e.value.message
    # no plan active: the step calls refuse
    with pytest.raises(H.HwError) as e:
        H.hw_append_step(ctx, 0, FAKE_K, FAKE_V, 0)
    assert e.value.status == H.HW_ERR_INVALID_ARG
    with pytest.raises(H.HwError) as e:
        H.hw_decode_step(ctx, 0, FAKE_K, FAKE_V, FAKE_K, FAKE_V, None, 0)
    assert e.value.status == H.HW_ERR_INVALID_ARG and "no step plan" in e.value.message
    with pytest.raises(H.HwError) as e:
        H.hw_plan_end(ctx, 0)
    assert e.value.status == H.HW_ERR_INVALID_ARG


def test_step_plan_needs_bf16():
    c = H.hw_create(make_cfg(kv_dtype=H.HW_F32))
    H.hw_debug_reserve(c, 0, [0], [8])
    H.hw_debug_reserve(c, 1, [0], [8])
    H.hw_set_views(c, [[0]])
    with pytest.raises(H.HwError) as e:
        H.hw_plan_steps(c, 2, [0], [1], 0)
    assert e.value.status == H.HW_ERR_INVALID_ARG and "bf16" in e.value.message
    H.hw_destroy(c)
