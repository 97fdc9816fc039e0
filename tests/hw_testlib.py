"""Helpers shared by the GPU tests: fill a cache from a workload, run the oracle."""

from __future__ import annotations

import numpy as np
import torch

from oracle import hogwild_oracle as O
from shared_kv_cache_amd import hogwild as H
from shared_kv_cache_amd import workloads as W

DEV = "cuda"


def kv_tensor(x: np.ndarray, kv_dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=DEV, dtype=torch.bfloat16 if kv_dtype == "bf16" else torch.float32)


def make_cache(wl: W.Workload, n_layers=None, page_seed=None, max_splits=0, n_pages=None,
               max_blocks=None, max_position=None, max_workers=None,
               max_query_tokens=0) -> H.HogwildCache:
    return H.HogwildCache(
        n_layers=wl.n_layers if n_layers is None else n_layers,
        n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
        page_size=wl.page_size, n_pages=wl.n_pages if n_pages is None else n_pages,
        max_blocks=len(wl.blocks()) + 4 if max_blocks is None else max_blocks,
        max_workers=wl.n_workers if max_workers is None else max_workers,
        max_position=wl.max_position if max_position is None else max_position,
        kv_dtype=wl.kv_dtype, page_seed=wl.page_seed if page_seed is None else page_seed,
        rope_theta=wl.theta, max_splits=max_splits, max_query_tokens=max_query_tokens)


def fill_layer(cache: H.HogwildCache, wl: W.Workload, layer: int, blocks=None):
    """Append every block of the workload (step-0 contents) to one layer, one call."""
    blocks = wl.blocks() if blocks is None else blocks
    ks, vs = zip(*(wl.kv(layer, b) for b in blocks))
    k = kv_tensor(np.concatenate(ks), wl.kv_dtype)
    v = kv_tensor(np.concatenate(vs), wl.kv_dtype)
    cache.append(layer, blocks, [wl.lengths[b] for b in blocks], k, v)
    return {b: (kk, vv) for b, kk, vv in zip(blocks, ks, vs)}


def oracle_blocks(wl: W.Workload, layer: int):
    return {b: tuple(np.asarray(x, np.float64) for x in wl.kv(layer, b)) for b in wl.blocks()}


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def max_row_rel(got, ref) -> float:
    """Largest per-(worker, head) relative L2 error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / den))


# Parity bar of the GPU path against the oracle: relative L2 over the whole output, and the
# same bound on every (worker, [token,] head) row; lse in absolute terms (natural log).
TOL = {"f32": 1e-5, "bf16": 1e-2}


def assert_parity(name, out, lse, ref, ref_lse, tol, say=print):
    """out/ref [..., D], lse/ref_lse [...]. Rows whose reference lse is -inf (no key) must be
    exactly 0 with lse -inf; every other row is held to tol, in rel L2 and in lse."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    lse = np.asarray(lse, np.float64)
    ref_lse = np.asarray(ref_lse, np.float64)
    fin = np.isfinite(ref_lse)
    assert np.all(np.isneginf(lse[~fin])) and np.all(out[~fin] == 0.0), f"{name}: empty rows"
    err = rel_l2(out[fin], ref[fin])
    row = max_row_rel(out[fin], ref[fin])
    lse_err = float(np.max(np.abs(lse[fin] - ref_lse[fin])))
    say(f"{name}: rel_l2 {err:.3e} max_row {row:.3e} lse_abs {lse_err:.3e} (tol {tol:g})")
    assert err <= tol, f"{name}: rel_l2 {err}"
    assert row <= tol, f"{name}: max_row {row}"
    assert lse_err <= tol, f"{name}: lse {lse_err}"
    return err, row, lse_err


def decode_np(cache: H.HogwildCache, layer: int, q: np.ndarray):
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).to(DEV)
    out, lse = cache.decode(layer, qt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def decode_tokens_np(cache: H.HogwildCache, layer: int, q: np.ndarray):
    """Several query tokens per worker: q [N, n_new, Hq, D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).to(DEV)
    out, lse = cache.decode_tokens(layer, qt)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


VARIANT_LENGTHS = [33, 1, 64, 65, 7, 0, 31, 32]


def variant_workload(head_dim, n_workers, group):
    """bf16 workload with n_workers * group rows per KV head: a ragged 300-token history and
    ragged in-progress blocks (one of them empty), 32-token pages."""
    base = W.make("tiny_fp32")
    inprog = list(range(1, n_workers + 1))
    lengths = {0: 300}
    lengths.update({b: VARIANT_LENGTHS[(b - 1) % len(VARIANT_LENGTHS)] for b in inprog})
    owners = {0: -1}
    owners.update({b: b - 1 for b in inprog})
    pages = sum(-(-n // 32) for n in lengths.values()) + 4
    return W.Workload(**{**base.__dict__, "name": f"d{head_dim}_rows{n_workers * group}",
                         "n_workers": n_workers, "n_q_heads": 2 * group, "n_kv_heads": 2,
                         "head_dim": head_dim, "kv_dtype": "bf16", "value_scale": 1.0,
                         "inprogress": inprog, "lengths": lengths, "owners": owners,
                         "n_pages": pages,
                         "max_position": max(2048, -(-(sum(lengths.values()) + 1) // 1024) * 1024)})


def k_pool_token(cache: H.HogwildCache, layer: int, page: int, head: int, slot: int):
    """Read one stored key back from the pool using the header's K layout."""
    d = cache.head_dim
    g, u = slot // 32, slot % 32
    base = ((((layer * cache.n_pages + page) * cache.n_kv_heads + head) *
             (cache.page_size // 32) + g) * 32 * d)
    idx = [(((i // 32) * 2 + (u // 4) % 2) * 4 + (i % 32) // 8) * 128 + (4 * (u // 8) + u % 4) * 8
           + i % 8 for i in range(d)]
    return base + np.array(idx)


def v_pool_token(cache: H.HogwildCache, layer: int, page: int, head: int, slot: int):
    d = cache.head_dim
    g, u = slot // 32, slot % 32
    base = ((((layer * cache.n_pages + page) * cache.n_kv_heads + head) *
             (cache.page_size // 32) + g) * 32 * d)
    idx = [(((i // 16) * 4 + u // 8) * 16 + i % 16) * 8 + u % 8 for i in range(d)]
    return base + np.array(idx)
