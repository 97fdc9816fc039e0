"""fp64 CPU oracle for the Hogwild! concurrent-attention decode step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It imports nothing
from the product package and the product package imports nothing from it.

What it computes is the method's *exact* result, written out the plain way:
for every worker, concatenate the raw (unrotated) keys and values of the
blocks in that worker's view order, give every key its true position in that
view, apply RoPE to the keys at those positions and to the query at the query
position, and run ordinary softmax attention. The method reaches the same
number faster by storing each block once at block-local positions and rotating
the query per block instead of the keys (Hogwild! Inference paper summary,
gentlecold.top, section 5 "RoPE position rearrangement", the concatenation
identity); this oracle deliberately does NOT use that shortcut.

Sources (pages' titles, section on the page):

* [P1] "Hogwild! Inference论文调研" -- gentlecold.top summary of *Hogwild!
  Inference: Parallel LLM Generation via Concurrent Attention*.
  s4 (shared KV cache problem, Alice/Bob view orders), s5 (RoPE
  rearrangement, the concatenation identity and the five-step procedure),
  s6 (combined layout: common history, other workers' unfinished steps, own
  step last), s8 (step order: append before attention), s9 (blocks hold all
  layers at local positions 0..len-1; view computed at attention time).
* [P2] ocdem.com article on Hogwild! Inference, s2.1 (neighbour blocks in
  ascending worker ID), s2.2 (rotation isometry).
* [P5] kwkr.cn essay on KV-cache sharing vs isolation, s3.2 (KV-cache size
  formula), s6.1 (worked size table).

Readings taken where the pages are silent:
rotate-half RoPE pairing (j, j + d/2); frequencies theta^(-2j/d) in fp64;
softmax scale 1/sqrt(d); GQA mapping kv_head = h // (Hq / Hkv); default
offsets = running sum of block lengths in view order; default query position =
last token of the worker's own block (its token of this step is appended
before attention, [P1] s8).

Parity: every function here is pinned by ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "rope_inv_freq",
    "rope",
    "canonical_view",
    "default_offsets",
    "default_q_pos",
    "view_error",
    "concurrent_attention",
    "reencode_bruteforce",
    "causal_decode_textbook",
    "kv_cache_bytes",
    "rope_store_reference",
    "bf16_bits_rne",
    "bf16_bits_to_f32",
    "commit_step_views",
]


# --------------------------------------------------------------------------
# RoPE  rho(x, i)   [P1] s5: the rotation applied to a query/key at position i
# --------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Rotation frequencies theta_j = theta^(-2j/d), j = 0 .. d/2-1, in fp64.

    The pages only write rho(x, i); the frequency ladder is the standard RoPE
    one (a reading). Each entry is a libm ``pow`` call so that a C
    implementation calling ``pow`` with the same arguments gets the same bits.
    """
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    return np.array([math.pow(theta, -(2.0 * j) / head_dim)
                     for j in range(head_dim // 2)], dtype=np.float64)


def rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """rho(x, i) in fp64 ([P1] s5).

    ``x`` has the head dimension last; ``pos`` broadcasts against
    ``x.shape[:-1]``. Pair (j, j + d/2) is rotated by angle pos * theta_j:
    (a, b) -> (a cos - b sin, b cos + a sin).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# --------------------------------------------------------------------------
# Views   [P1] s4, s6 ; [P2] s2.1
# --------------------------------------------------------------------------

def canonical_view(worker: int, history: Sequence[int],
                   inprogress: Sequence[int]) -> List[int]:
    """Block order seen by ``worker`` in the combined (token-wise) layout.

    Common history blocks in history order ([P1] s6), then every other
    worker's unfinished block in ascending worker ID ([P2] s2.1), then the
    worker's own block last ([P1] s4: Alice sees C+B+A, Bob sees C+A+B).
    ``inprogress[u]`` is worker u's current block.
    """
    others = [inprogress[u] for u in range(len(inprogress)) if u != worker]
    return list(history) + others + [inprogress[worker]]


def default_offsets(view: Sequence[int], lengths: Dict[int, int]) -> List[int]:
    """Start position of each block in the view: running sum of lengths."""
    out, acc = [], 0
    for b in view:
        out.append(acc)
        acc += lengths[b]
    return out


def default_q_pos(view: Sequence[int], offsets: Sequence[int],
                  lengths: Dict[int, int]) -> int:
    """The query is the last token of the last (own) block of the view."""
    return offsets[-1] + lengths[view[-1]] - 1


def view_error(view: Sequence[int], offsets: Sequence[int],
               lengths: Dict[int, int], q_pos: int) -> Optional[str]:
    """Why a view cannot be attended, or None.

    Two true positions may not coincide (intervals [off, off + len) of the
    blocks must not overlap; gaps are allowed), a block may appear once, and
    the query may not precede any key it attends to (decode is causal).
    """
    if len(set(view)) != len(view):
        return "block repeated in view"
    spans = sorted((o, o + lengths[b]) for b, o in zip(view, offsets) if lengths[b] > 0)
    for (a0, a1), (b0, _) in zip(spans, spans[1:]):
        if b0 < a1:
            return "overlapping blocks"
    for b, o in zip(view, offsets):
        if o < 0:
            return "negative offset"
        if lengths[b] > 0 and o + lengths[b] - 1 > q_pos:
            return "key after query"
    return None


# --------------------------------------------------------------------------
# The oracle proper
# --------------------------------------------------------------------------

def _resolve(views, lengths, offsets, q_pos):
    offs = [list(default_offsets(v, lengths)) if offsets is None or offsets[w] is None
            else list(offsets[w]) for w, v in enumerate(views)]
    qps = [default_q_pos(v, offs[w], lengths) if q_pos is None or q_pos[w] is None
           else int(q_pos[w]) for w, v in enumerate(views)]
    return offs, qps


def concurrent_attention(q: np.ndarray,
                         blocks: Dict[int, Tuple[np.ndarray, np.ndarray]],
                         views: Sequence[Sequence[int]],
                         offsets=None, q_pos=None, theta: float = 1e4,
                         scale: Optional[float] = None,
                         heads: Optional[Sequence[int]] = None):
    """Exact concurrent attention for one decode step of one layer.

    q       [N, Hq, D] raw (unrotated) queries, one token per worker; or
            [N, n_new, Hq, D]: n_new tokens per worker processed together (a
            paragraph header inserted into a fresh block, [P1] s8 step 4). Token t
            sits at position q_pos - (n_new - 1 - t) and attends to the keys at or
            before its own position only (causal), so the last token is the one-token
            case and earlier tokens do not see the ones after them.
    blocks  block id -> (K [len, Hkv, D], V [len, Hkv, D]) raw, unrotated.
    views   per worker, block ids in view order.
    offsets per worker, start position of each view block (None: running sum).
    q_pos   per worker, query position (None: last token of the view).
    heads   query heads to compute (None: all); others stay NaN.

    Returns (out [N, Hq, D], lse [N, Hq]) in fp64 (with n_new: [N, n_new, Hq, D] and
    [N, n_new, Hq]); lse is the natural-log normaliser log(sum_t exp(s_t)). A token
    with no key at or before it gets out = 0 and lse = -inf.

    Steps ([P1] s5, s8): concatenate the view's keys and values; give token j
    of a block at offset o the true position o + j; rho every key at its true
    position and the query at q_pos; scores s_t = rho(q)·rho(k_t) * scale;
    softmax over every token of the view; out = sum_t softmax_t v_t.
    """
    q = np.asarray(q, dtype=np.float64)
    lengths = {b: int(kv[0].shape[0]) for b, kv in blocks.items()}
    offs, qps = _resolve(views, lengths, offsets, q_pos)
    if q.ndim == 4:   # several tokens per worker: each token on its own, causally
        n_new = q.shape[1]
        outs, lses = [], []
        for t in range(n_new):
            back = n_new - 1 - t
            o, l_ = _attend(q[:, t], blocks, views, lengths, offs, [p - back for p in qps],
                            qps, theta, scale, heads, causal=True)
            outs.append(o)
            lses.append(l_)
        return np.stack(outs, axis=1), np.stack(lses, axis=1)
    return _attend(q, blocks, views, lengths, offs, qps, qps, theta, scale, heads, causal=False)


def _attend(q, blocks, views, lengths, offs, qps, last_qps, theta, scale, heads, causal):
    """One query token per worker, at qps[w], over the worker's view (validated against
    last_qps[w], the position of the worker's last query token). causal: keys after the
    token are left out."""
    n_workers, hq, d = q.shape
    hkv = next(iter(blocks.values()))[0].shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    heads = list(range(hq)) if heads is None else list(heads)
    out = np.full((n_workers, hq, d), np.nan)
    lse = np.full((n_workers, hq), np.nan)
    for w in range(n_workers):
        view = list(views[w])
        err = view_error(view, offs[w], lengths, last_qps[w])
        if err:
            raise ValueError(f"worker {w}: {err}")
        if qps[w] < 0:
            raise ValueError(f"worker {w}: query position below 0")
        if sum(lengths[b] for b in view) == 0:
            out[w, heads] = 0.0
            lse[w, heads] = -np.inf
            continue
        pos = np.concatenate([o + np.arange(lengths[b]) for b, o in zip(view, offs[w])])
        keys = np.concatenate([np.asarray(blocks[b][0], np.float64) for b in view])
        vals = np.concatenate([np.asarray(blocks[b][1], np.float64) for b in view])
        if causal:
            keep = pos <= qps[w]
            pos, keys, vals = pos[keep], keys[keep], vals[keep]
            if len(pos) == 0:
                out[w, heads] = 0.0
                lse[w, heads] = -np.inf
                continue
        q_rot = rope(q[w], qps[w], theta)
        for kvh in sorted({h // group for h in heads}):
            k_rot = rope(keys[:, kvh, :], pos, theta)
            for h in heads:
                if h // group != kvh:
                    continue
                s = (k_rot @ q_rot[h]) * scale
                m = s.max()
                p = np.exp(s - m)
                l_sum = p.sum()
                out[w, h] = (p @ vals[:, kvh, :]) / l_sum
                lse[w, h] = m + math.log(l_sum)
    return out, lse


# --------------------------------------------------------------------------
# Independent cross-checks used to pin the oracle (small inputs only)
# --------------------------------------------------------------------------

def _rotation_matrix(position: float, d: int, theta: float) -> np.ndarray:
    """Dense d x d matrix of rho(., position): 2x2 rotations on (j, j + d/2)."""
    h = d // 2
    m = np.zeros((d, d))
    for j in range(h):
        a = position * math.pow(theta, -(2.0 * j) / d)
        c, s = math.cos(a), math.sin(a)
        m[j, j], m[j, j + h] = c, -s
        m[j + h, j], m[j + h, j + h] = s, c
    return m


def reencode_bruteforce(q, blocks, views, offsets=None, q_pos=None,
                        theta: float = 1e4, scale: Optional[float] = None):
    """The naive alternative the method avoids ([P1] s4, s9: re-encode / re-prefill).

    Starts from each block stored rotated at block-local positions, undoes the
    local rotation and re-rotates every key to its true position with dense
    rotation matrices, then builds the full causal attention matrix of the
    concatenated sequence (one query row per key, plus the worker's query as
    the last row) and returns that last row's output. Tiny inputs only.
    """
    q = np.asarray(q, dtype=np.float64)
    n_workers, hq, d = q.shape
    lengths = {b: int(kv[0].shape[0]) for b, kv in blocks.items()}
    hkv = next(iter(blocks.values()))[0].shape[1]
    group = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    offs, qps = _resolve(views, lengths, offsets, q_pos)
    out = np.zeros((n_workers, hq, d))
    lse = np.zeros((n_workers, hq))
    for w in range(n_workers):
        keys, vals, pos = [], [], []
        for b, o in zip(views[w], offs[w]):
            kb, vb = blocks[b]
            for j in range(lengths[b]):
                stored = [_rotation_matrix(j, d, theta) @ np.asarray(kb[j, g], float)
                          for g in range(hkv)]
                back = _rotation_matrix(-j, d, theta)
                fwd = _rotation_matrix(o + j, d, theta)
                keys.append([fwd @ (back @ stored[g]) for g in range(hkv)])
                vals.append(np.asarray(vb[j], float))
                pos.append(o + j)
        keys = np.array(keys)          # [T, Hkv, D] re-encoded
        vals = np.array(vals)
        pos = np.array(pos, dtype=np.float64)
        t_len = len(pos)
        q_fwd = _rotation_matrix(qps[w], d, theta)
        for h in range(hq):
            g = h // group
            rows = np.vstack([keys[:, g, :], q_fwd @ q[w, h]])      # [T+1, D]
            row_pos = np.concatenate([pos, [qps[w]]])
            logits = (rows @ keys[:, g, :].T) * scale                # [T+1, T]
            mask = pos[None, :] <= row_pos[:, None]
            logits = np.where(mask, logits, -np.inf)
            mx = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - mx)
            probs = e / e.sum(axis=1, keepdims=True)
            out[w, h] = probs[t_len] @ vals[:, g, :]
            lse[w, h] = mx[t_len, 0] + math.log(e[t_len].sum())
    return out, lse


def causal_decode_textbook(q_last, k_seq, v_seq, theta: float = 1e4,
                           scale: Optional[float] = None):
    """Ordinary single-sequence causal decode of the last token (tiny inputs).

    q_last [Hq, D] is the query of the token at position T-1; k_seq, v_seq
    [T, Hkv, D] hold raw keys/values at positions 0..T-1. RoPE is written in
    its complex form: pair (j, j + d/2) is the complex number x_j + i x_{j+d/2}
    multiplied by exp(i * pos * theta_j); a real dot product is the real part
    of sum_j z_q,j * conj(z_k,j). Pure Python loops.
    """
    hq, d = len(q_last), len(q_last[0])
    t_len, hkv = len(k_seq), len(k_seq[0])
    half = d // 2
    group = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    freqs = [theta ** (-(2.0 * j) / d) for j in range(half)]

    def as_complex(vec, position):
        return [complex(float(vec[j]), float(vec[j + half]))
                * complex(math.cos(position * freqs[j]), math.sin(position * freqs[j]))
                for j in range(half)]

    out, lse = [], []
    for h in range(hq):
        g = h // group
        zq = as_complex(q_last[h], t_len - 1)
        scores = []
        for t in range(t_len):
            zk = as_complex(k_seq[t][g], t)
            scores.append(sum((a * b.conjugate()).real for a, b in zip(zq, zk)) * scale)
        mx = max(scores)
        weights = [math.exp(s - mx) for s in scores]
        total = sum(weights)
        out.append([sum(weights[t] * float(v_seq[t][g][i]) for t in range(t_len)) / total
                    for i in range(d)])
        lse.append(mx + math.log(total))
    return np.array(out), np.array(lse)


# --------------------------------------------------------------------------
# Byte accounting  [P5] s3.2 formula, s6.1 worked table
# --------------------------------------------------------------------------

def kv_cache_bytes(n_layers: int, n_heads: int, seq_len: int, batch: int,
                   head_dim: int, bytes_per_elem: int) -> int:
    """KV-cache size: 2 (K and V) * L * H * S * B * D * bytes per element."""
    return 2 * n_layers * n_heads * seq_len * batch * head_dim * bytes_per_elem


# --------------------------------------------------------------------------
# Stored-key reference: what RoPE-on-insert writes, in the stated precision
# --------------------------------------------------------------------------

def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rope_store_reference(k_raw: np.ndarray, positions: np.ndarray, theta: float,
                         kv_dtype: str) -> np.ndarray:
    """Keys as a block stores them: rho(k, local position) in fp32, then rounded.

    [P1] s5 steps (1)-(2) and s9: each block's keys are stored once, rotated
    at block-local positions 0..len-1. Precision (a reading; the pages fix
    none): angle = position * theta_j in fp64, cos/sin in fp64 (libm), each
    rounded once to fp32; then a*c - b*s and b*c + a*s with every product and
    sum rounded to fp32 (no fused multiply-add); bf16 storage rounds to nearest
    even. k_raw [n, Hkv, D] is fp32 (already the stored dtype's values);
    positions [n]. Returns float32 for kv_dtype 'f32', uint16 bf16 bits for
    'bf16'.
    """
    k = np.asarray(k_raw, dtype=np.float32)
    n, _, d = k.shape
    h = d // 2
    inv = rope_inv_freq(d, theta)
    cos_t = np.empty((n, h), np.float32)
    sin_t = np.empty((n, h), np.float32)
    cache = {}
    for i, p in enumerate(np.asarray(positions).tolist()):
        if p not in cache:
            ang = [float(p) * inv[j] for j in range(h)]
            cache[p] = (np.array([math.cos(a) for a in ang], np.float32),
                        np.array([math.sin(a) for a in ang], np.float32))
        cos_t[i], sin_t[i] = cache[p]
    c = cos_t[:, None, :]
    s = sin_t[:, None, :]
    a, b = k[..., :h], k[..., h:]
    lo = (a * c) - (b * s)
    hi = (b * c) + (a * s)
    rot = np.concatenate([lo, hi], axis=-1).astype(np.float32)
    if kv_dtype == "f32":
        return rot
    if kv_dtype == "bf16":
        return bf16_bits_rne(rot)
    raise ValueError(kv_dtype)


# --------------------------------------------------------------------------
# Step commit (history merge)  [P1] s8: a finished step joins the history
# --------------------------------------------------------------------------

def commit_step_views(history: Sequence[int], inprogress: Sequence[int],
                      worker: int, new_block: int):
    """History and in-progress lists after ``worker`` finishes its step.

    The finished block moves to the end of the common history and the worker
    continues in a fresh, empty block ([P1] s8). Keys are not touched: the
    block's new position is only a new offset in every view.
    """
    hist = list(history) + [inprogress[worker]]
    cur = list(inprogress)
    cur[worker] = new_block
    return hist, cur
