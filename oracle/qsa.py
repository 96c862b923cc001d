"""QSA compressed indexer -- TEST INFRASTRUCTURE ONLY (plain numpy, fp64).  Only the tests, the
smoke check and the benchmark's CPU-baseline leg use this module; the library never does.

Follows the explainer page "論文解説: Qwen3.8-Next の設計" (ta-paperlens.web.app), section
"部品②: QSA": keys are cut into blocks of r tokens and mean-pooled *before* the position
encoding, each block gets one position (its first token's), the indexer is multi-query
attention with Hq query heads over one shared key head, with rotary position encoding on
part of the head dimension, and a token budget K (K / r blocks) picks the blocks to keep.

Readings where the page leaves a step open (each one is a parameter or documented choice):
  - block j covers tokens j*r .. min((j+1)*r, T) - 1; its pooled key is the mean of those
    keys; it is eligible for the query at position t when its last token is <= t (no future
    key enters a mean the query sees);
  - rotary encoding on the first `rope_dims` dimensions, rotate-half pairing (dimension i with
    i + rope_dims/2), angle = position * base^(-2i / rope_dims); the rest is not rotated;
  - the per-head score of block j for the query at t is a softmax over the eligible blocks of
    q_{t,h} . kbar_j / sqrt(d); a block's importance is the sum over the Hq heads (the page
    says the indexer is first distilled from the backbone's attention distribution, so it
    outputs attention-like distributions);
  - the selection keeps the min(K / r, #eligible) most important blocks (ties: lower block
    index first) and returns them in ascending order, padded with -1.
"""
from __future__ import annotations

import numpy as np


def pool_keys(k, r):
    """k: [B, T, d] -> pooled keys [B, nb, d] (fp64), nb = ceil(T / r); block j is the mean of
    keys j*r .. min((j+1)*r, T) - 1."""
    k = np.asarray(k, dtype=np.float64)
    B, T, d = k.shape
    nb = -(-T // r)
    out = np.zeros((B, nb, d))
    for j in range(nb):
        a, b = j * r, min((j + 1) * r, T)
        out[:, j] = k[:, a:b].mean(axis=1)
    return out


def rope(x, pos, rope_dims, base=10000.0):
    """Rotate the first rope_dims dimensions of x[..., d] at positions pos (broadcast over the
    last axis): pairs (i, i + rope_dims/2), angle pos * base^(-2i/rope_dims)."""
    x = np.array(x, dtype=np.float64)
    h = rope_dims // 2
    i = np.arange(h, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * base ** (-2.0 * i / rope_dims)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h].copy(), x[..., h:rope_dims].copy()
    x[..., :h] = a * c - b * s
    x[..., h:rope_dims] = a * s + b * c
    return x


def importance(q, k, r, rope_dims=64, base=10000.0, scale=None, rows=None):
    """q: [B, T, Hq, d]; k: [B, T, d] (the shared key head).  Returns (imp [B, n, nb] fp64,
    eligible mask [n, nb]) for the query positions `rows` (all T by default; n of them):
    imp[b, i, j] = sum_h softmax_j(scale * q_{t,h} . kbar_j) over the blocks eligible for
    t = rows[i], 0 elsewhere; scale defaults to 1/sqrt(d)."""
    q = np.asarray(q, dtype=np.float64)
    B, T, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    kb = pool_keys(k, r)
    nb = kb.shape[1]
    kb = rope(kb, np.arange(nb) * r, rope_dims, base)                # a block sits at its first
    qr = rope(q[:, rows], rows[None, :, None], rope_dims, base)      # token; a query at its own
    last = np.minimum((np.arange(nb) + 1) * r, T) - 1
    elig = last[None, :] <= rows[:, None]                            # [n, nb]
    s = np.einsum("bthd,bjd->bthj", qr, kb) * scale
    s = np.where(elig[None, :, None, :], s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    den = p.sum(axis=-1, keepdims=True)
    p = np.where(den > 0, p / np.where(den > 0, den, 1.0), 0.0)
    return p.sum(axis=2), elig


def select(imp, elig, nsel):
    """The min(nsel, #eligible) most important eligible blocks of every query (ties to the
    lower index), ascending, padded with -1.  imp: [B, T, nb] -> [B, T, nsel] int64."""
    B, T, nb = imp.shape
    out = np.full((B, T, nsel), -1, dtype=np.int64)
    for b in range(B):
        for t in range(T):
            cand = np.nonzero(elig[t])[0]
            if cand.size == 0:
                continue
            # stable sort on (-importance, index)
            order = cand[np.lexsort((cand, -imp[b, t, cand]))]
            keep = np.sort(order[:nsel])
            out[b, t, :keep.size] = keep
    return out


def expand_tokens(sel, r, T):
    """Selected blocks back to token positions: block j stands for tokens j*r .. min((j+1)*r,
    T) - 1.  sel [..., nsel] -> [..., nsel * r], ascending, padded with -1."""
    sel = np.asarray(sel)
    out = np.full(sel.shape[:-1] + (sel.shape[-1] * r,), -1, dtype=np.int64)
    for idx in np.ndindex(*sel.shape[:-1]):
        toks = [t for j in sel[idx] if j >= 0 for t in range(j * r, min((j + 1) * r, T))]
        out[idx][:len(toks)] = toks
    return out


def qsa_index(q, k, r=4, budget_tokens=2048, rope_dims=64, base=10000.0, scale=None):
    """The whole indexer: (selected block indices [B, T, budget/r], importance [B, T, nb])."""
    imp, elig = importance(q, k, r, rope_dims, base, scale)
    return select(imp, elig, budget_tokens // r), imp
