"""Seeded synthetic workloads shaped like the Hogwild! decode configurations.

This module only draws numbers and lays out block structure; it holds none of
the method's arithmetic (no RoPE, no attention), so the oracle and the GPU
path can both be fed from it. Every tensor is drawn from its own stream,
``SeedSequence([config_seed, layer, tensor_id])``, so any one layer or block
can be regenerated alone (per-unit derived seeds instead of one shared global
generator; kwkr.cn essay on KV-cache sharing vs isolation, s2.3).

Block structure follows the combined layout of the Hogwild! Inference paper
summary (gentlecold.top), s6: a common prompt, a common history of finished
steps (paragraphs), and one unfinished block per worker. Views are listed in
that layout's order (history, other workers ascending, own block last).
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

_STRUCTURE = 0xFFFF_FFFF  # tensor id reserved for structural draws
_Q_ID = 0
_STEP_BASE = 1 << 24      # tensor ids of per-step appended tokens
_TOKENS_BASE = 1 << 23    # tensor ids of several-token queries


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words))))


def round_to_bf16_values(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value (ties to even), kept as fp32.

    Used only to make the inputs exactly representable in the cache dtype, so
    that both sides of a parity test start from identical numbers.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    n_workers: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kv_dtype: str                 # "bf16" or "f32"
    page_size: int
    theta: float
    value_scale: float            # every draw is value_scale * N(0, 1)
    history: List[int]            # common blocks in history order (prompt first)
    inprogress: List[int]         # inprogress[w] = worker w's current block
    lengths: Dict[int, int]       # block id -> tokens (at step 0)
    owners: Dict[int, int]        # block id -> owning worker (-1: prompt)
    n_pages: int                  # pool pages
    page_seed: int                # 0: pages handed out in order; else shuffled
    max_position: int             # largest position + 1 the cache must rotate to
    sink: Optional[Tuple[int, int, float]] = None   # (kv head, first n tokens, key factor)
    steps: int = 0                # decode steps the workload grows by (1 token/worker/step)

    # ---- structure -----------------------------------------------------
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def views(self, layout: str = "combined") -> List[List[int]]:
        """Every worker's view (block order) under one of the cache layouts the paper
        summary (gentlecold.top) compares in s6 and whose synchronisation levels s10
        contrasts:

        combined    the method's own: the common history (prompt, then finished steps in
                    history order), the other workers' unfinished steps in ascending
                    worker ID, the worker's own unfinished step last.
        stepwise    ("interleaved" / step-wise): only finished steps enter the history;
                    other workers' unfinished steps are not visible.
        contiguous  each worker's output kept in one contiguous span: the prompt, then
                    every other worker's finished steps and unfinished step in ascending
                    worker ID, the worker's own span last.
        nosync      no synchronisation: the prompt, the worker's own finished steps and
                    its unfinished step.

        The prompt is every history block without an owner (owner -1).
        """
        prompt = [b for b in self.history if self.owners.get(b, -1) < 0]
        own_done = lambda u: [b for b in self.history if self.owners.get(b, -1) == u]
        out = []
        for w in range(self.n_workers):
            others = [u for u in range(self.n_workers) if u != w]
            if layout == "combined":
                v = list(self.history) + [self.inprogress[u] for u in others]
            elif layout == "stepwise":
                v = list(self.history)
            elif layout == "contiguous":
                v = list(prompt)
                for u in others:
                    v += own_done(u) + [self.inprogress[u]]
                v += own_done(w)
            elif layout == "nosync":
                v = list(prompt) + own_done(w)
            else:
                raise ValueError(layout)
            out.append(v + [self.inprogress[w]])
        return out

    def blocks(self) -> List[int]:
        return list(self.history) + list(self.inprogress)

    def total_tokens(self, lengths: Optional[Dict[int, int]] = None) -> int:
        lengths = self.lengths if lengths is None else lengths
        return sum(lengths[b] for b in self.blocks())

    # ---- tensors -------------------------------------------------------
    def _draw(self, layer: int, tensor_id: int, shape) -> np.ndarray:
        x = _rng(self.seed, layer, tensor_id).standard_normal(shape, dtype=np.float32)
        if self.value_scale != 1.0:
            x *= np.float32(self.value_scale)
        return x

    def _as_cache_values(self, x: np.ndarray) -> np.ndarray:
        return round_to_bf16_values(x) if self.kv_dtype == "bf16" else x

    def kv(self, layer: int, block: int, length: Optional[int] = None):
        """Raw (unrotated) K and V of a block at step 0: fp32 [len, Hkv, D]."""
        n = self.lengths[block] if length is None else length
        shape = (n, self.n_kv_heads, self.head_dim)
        k = self._draw(layer, 1 + 2 * block, shape)
        v = self._draw(layer, 2 + 2 * block, shape)
        if self.sink is not None and block == self.history[0]:
            head, count, factor = self.sink
            k[:count, head, :] *= np.float32(factor)
        return self._as_cache_values(k), self._as_cache_values(v)

    def q(self, layer: int, step: int = 0) -> np.ndarray:
        """Raw queries [N, Hq, D] fp32 (the query dtype is always fp32)."""
        tid = _Q_ID if step == 0 else _STEP_BASE + 2 * step + 1
        return self._draw(layer, tid, (self.n_workers, self.n_q_heads, self.head_dim))

    def q_tokens(self, layer: int, n_new: int) -> np.ndarray:
        """Raw queries of n_new tokens per worker [N, n_new, Hq, D] fp32 (the tokens a worker
        appends together, e.g. a paragraph header opening a fresh block)."""
        return self._draw(layer, _TOKENS_BASE + n_new,
                          (self.n_workers, n_new, self.n_q_heads, self.head_dim))

    def step_kv(self, layer: int, step: int):
        """The one new token each worker appends at decode step ``step`` >= 1:
        raw K and V [N, Hkv, D] (row w goes to worker w's block)."""
        shape = (self.n_workers, self.n_kv_heads, self.head_dim)
        k = self._draw(layer, _STEP_BASE + 2 * step, shape)
        v = self._draw(layer, _STEP_BASE + 2 * step + (1 << 22), shape)
        return self._as_cache_values(k), self._as_cache_values(v)


def _pages_for(lengths, blocks, page_size) -> int:
    return sum(-(-lengths[b] // page_size) for b in blocks)


def make(name: str, n_layers: Optional[int] = None, steps: int = 0,
         page_size: Optional[int] = None) -> Workload:
    """Build one of the named configurations.

    tiny_fp32      2 workers, 1 layer, 4/2 heads, d 64, fp32, common 256,
                   in-progress 32 and 27, N(0,1) from seed 0.
    w2_4k          2 workers, 40/8 x 128 bf16, common 4096 in 256-token pages,
                   in-progress 256 and 193, values 0.5 N(0,1).
    w4_16k         4 workers, 40/8 x 128 bf16, 8192-token prompt + 8192 tokens
                   of paragraphs U{64..512} (owners round-robin), in-progress
                   U{1..512}, 64 layers.
    w8_32k         8 workers, 64/8 x 128 bf16, common 32768 in 256-token pages
                   scattered in a pool twice the size needed, in-progress
                   U{1..1024}; grows by one token per worker per step.
    w4_128k_sinks  4 workers, 40/8 x 128 bf16, 131072-token history whose KV
                   head 7 has 4 sink keys scaled x8, in-progress 1024 each.
    """
    if name == "tiny_fp32":
        seed, n, hq, hkv, d, dt, ps, vs = 0, 2, 4, 2, 64, "f32", 32, 1.0
        hist_lens = [256]
        cur_lens = [32, 27]
        layers = 1
    elif name == "w2_4k":
        seed, n, hq, hkv, d, dt, ps, vs = 1, 2, 40, 8, 128, "bf16", 256, 0.5
        hist_lens = [4096]
        cur_lens = [256, 193]
        layers = 32
    elif name == "w4_16k":
        seed, n, hq, hkv, d, dt, ps, vs = 2, 4, 40, 8, 128, "bf16", 256, 1.0
        r = _rng(seed, _STRUCTURE, 0)
        paras, total = [], 0
        while total < 8192:
            x = int(r.integers(64, 513))
            x = min(x, 8192 - total)
            paras.append(x)
            total += x
        hist_lens = [8192] + paras
        cur_lens = [int(x) for x in r.integers(1, 513, size=n)]
        layers = 64
    elif name == "w8_32k":
        seed, n, hq, hkv, d, dt, ps, vs = 3, 8, 64, 8, 128, "bf16", 256, 1.0
        r = _rng(seed, _STRUCTURE, 0)
        hist_lens = [32768]
        cur_lens = [int(x) for x in r.integers(1, 1025, size=n)]
        layers = 8
    elif name == "w4_128k_sinks":
        seed, n, hq, hkv, d, dt, ps, vs = 4, 4, 40, 8, 128, "bf16", 256, 1.0
        hist_lens = [131072]
        cur_lens = [1024] * n
        layers = 4
    else:
        raise KeyError(name)
    if page_size is not None:
        ps = page_size
    history = list(range(len(hist_lens)))
    inprogress = [len(hist_lens) + w for w in range(n)]
    lengths = {b: l for b, l in zip(history, hist_lens)}
    lengths.update({b: l for b, l in zip(inprogress, cur_lens)})
    owners = {0: -1}
    for i in range(1, len(hist_lens)):
        owners[i] = (i - 1) % n
    for w, b in enumerate(inprogress):
        owners[b] = w
    grown = dict(lengths)
    for b in inprogress:
        grown[b] += steps
    needed = _pages_for(grown, history + inprogress, ps)
    scattered = name == "w8_32k"
    n_pages = 2 * needed if scattered else needed + n
    total = sum(grown.values())
    max_pos = ((total + 1 + 1023) // 1024) * 1024
    return Workload(
        name=name, seed=seed, n_workers=n, n_layers=layers if n_layers is None else n_layers,
        n_q_heads=hq, n_kv_heads=hkv, head_dim=d, kv_dtype=dt, page_size=ps,
        theta=1e4, value_scale=vs, history=history, inprogress=inprogress,
        lengths=lengths, owners=owners, n_pages=n_pages,
        page_seed=0x5EED if scattered else 0, max_position=max_pos,
        sink=(7, 4, 8.0) if name == "w4_128k_sinks" else None, steps=steps)


CONFIGS = ["tiny_fp32", "w2_4k", "w4_16k", "w8_32k", "w4_128k_sinks"]
