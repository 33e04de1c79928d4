"""CPU fp64 oracle for TTT sparse tree attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never touches it, and it
imports nothing from the product.

What it computes is the plain definition, written out densely:

* The mask is the one the SpecForge paper review gives under
  "§3 Technical architecture -> Compute optimisation -> Sparse Tree Attention ->
  BlockMask construction algorithm", restated as formulas in
  "§4 Core formulas -> BlockMask construction":
  a query i sees key j if (i >= j and j < T)  [the causal part]
  or (j >= Q_LEN and j mod Q_LEN < T and (j - i) mod Q_LEN == 0)  [the suffix].
* Attention is softmax attention restricted to that mask (the review's
  "§3 -> Sparse Tree Attention -> streaming computation": FlexAttention streams
  the very same masked softmax, so the dense result is what a streaming kernel
  must reach, up to rounding order).  The softmax is the one printed under
  "§4 Core formulas -> Masked softmax loss".
* The backward pass is the softmax Jacobian identity
  (dS = P * (dP - rowsum(P * dP))), the same identity the review uses for the
  loss gradient in "§4 Core formulas -> In-place backward".

Readings where the pages are silent:
  - queries index the current TTT step's Q_LEN rows; keys of step t sit in rows
    [t*Q_LEN, (t+1)*Q_LEN) of the stacked K/V, block 0 is the prefix;
  - padded query rows (i >= T) follow the formula literally: they see keys
    [0, T) and are computed and receive gradient;
  - a row with no visible key (only possible when T == 0) gives O = 0,
    lse = -inf and no gradient;
  - GQA heads map to KV heads in contiguous groups: kv head = h // (Hq // Hkv);
  - lse is the natural-log log-sum-exp of the scaled logits over the mask.

Every function here is pinned by ``tests/test_oracle.py`` against brute force,
library routines, closed forms and finite differences; none is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024  # rows per block of the dense computation (memory bound only)


def mask_rows(q_len: int, ttt_step: int, valid_len: int, r0: int, r1: int) -> np.ndarray:
    """Rows [r0, r1) of the boolean mask M of shape [Q_LEN, (ttt_step + 1) * Q_LEN].

    The formula of the BlockMask construction (review §3 "BlockMask construction algorithm",
    restated in §4 "BlockMask construction"), evaluated on the global query index i (r0..r1-1)
    and key index j (0..KV-1):  M = causal | suffix, with
        causal = (i >= j) & (j < T)
        suffix = (j >= Q_LEN) & (j mod Q_LEN < T) & ((j - i) mod Q_LEN == 0).
    ``%`` on numpy integers is the non-negative (floored) modulus.
    """
    L, T = int(q_len), int(valid_len)
    i = np.arange(r0, r1, dtype=np.int64)[:, None]
    j = np.arange((int(ttt_step) + 1) * L, dtype=np.int64)[None, :]
    causal = (i >= j) & (j < T)
    suffix = (j >= L) & (j % L < T) & ((j - i) % L == 0)
    return causal | suffix


def mask(q_len: int, ttt_step: int, valid_len: int) -> np.ndarray:
    """The whole mask M, shape [Q_LEN, (ttt_step + 1) * Q_LEN]."""
    return mask_rows(q_len, ttt_step, valid_len, 0, int(q_len))


def _chunk(q_len, ttt_step, valid_len, r0, r1):
    """Mask rows [r0, r1) restricted to the key columns that at least one of those rows may
    see.  Every other column holds exp(-inf) = 0 in each softmax sum and gradient, so leaving
    it out changes no result; it only keeps the dense blocks small."""
    Mr = mask_rows(q_len, ttt_step, valid_len, r0, r1)
    cols = np.nonzero(Mr.any(axis=0))[0]
    return Mr[:, cols], cols


def _check_shapes(q, k, v, seq_T):
    B, Hq, L, d = q.shape
    Bk, Hkv, KV, dk = k.shape
    # V may carry its own feature width (the pins feed V = identity columns)
    assert v.shape[:3] == k.shape[:3] and Bk == B and dk == d
    assert Hq % Hkv == 0 and KV % L == 0
    assert len(seq_T) == B
    return B, Hq, Hkv, L, d, KV // L - 1


def forward(q, k, v, seq_T, scale):
    """Masked softmax attention.  Returns (o, lse) in fp64.

    q [B, Hq, L, d]; k, v [B, Hkv, (step+1)*L, d]; seq_T [B] ints.
    o [B, Hq, L, d]; lse [B, Hq, L] natural log (-inf on empty rows).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, L, d, step = _check_shapes(q, k, v, seq_T)
    G = Hq // Hkv
    o = np.zeros((B, Hq, L, v.shape[3]))
    lse = np.full((B, Hq, L), -np.inf)
    for b in range(B):
        for r0 in range(0, L, ROW_CHUNK):
            r1 = min(L, r0 + ROW_CHUNK)
            Mr, cols = _chunk(L, step, int(seq_T[b]), r0, r1)
            for h in range(Hq):
                g = h // G
                S = scale * (q[b, h, r0:r1] @ k[b, g, cols].T)
                S = np.where(Mr, S, -np.inf)
                nonempty = Mr.any(axis=1)
                m = np.where(nonempty, S.max(axis=1, initial=-np.inf), 0.0)
                P = np.exp(S - m[:, None])  # exp(-inf) = 0 off the mask
                l = P.sum(axis=1)
                safe_l = np.where(nonempty, l, 1.0)
                P = P / safe_l[:, None]
                o[b, h, r0:r1] = P @ v[b, g, cols]
                lse[b, h, r0:r1] = np.where(nonempty, m + np.log(safe_l), -np.inf)
    return o, lse


def backward(q, k, v, seq_T, scale, do, o=None):
    """Gradients of sum(do * o) with respect to q, k, v, in fp64.

    P is recomputed from the dense masked logits; D = rowsum(do * o);
    dP = do @ V^T; dS = P * (dP - D); dQ = scale * dS @ K;
    dK = scale * sum_h dS^T @ Q_h; dV = sum_h P^T @ dO_h (sums over the query
    heads of a KV group, in head order).  Rows of dK/dV that no query sees are 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Hkv, L, d, step = _check_shapes(q, k, v, seq_T)
    G = Hq // Hkv
    if o is None:
        o, _ = forward(q, k, v, seq_T, scale)
    o = np.asarray(o, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for r0 in range(0, L, ROW_CHUNK):
            r1 = min(L, r0 + ROW_CHUNK)
            Mr, cols = _chunk(L, step, int(seq_T[b]), r0, r1)
            for h in range(Hq):
                g = h // G
                Kc, Vc = k[b, g, cols], v[b, g, cols]
                S = np.where(Mr, scale * (q[b, h, r0:r1] @ Kc.T), -np.inf)
                nonempty = Mr.any(axis=1)
                m = np.where(nonempty, S.max(axis=1, initial=-np.inf), 0.0)
                P = np.exp(S - m[:, None])
                l = np.where(nonempty, P.sum(axis=1), 1.0)
                P = P / l[:, None]
                dO = do[b, h, r0:r1]
                D = (dO * o[b, h, r0:r1]).sum(axis=1)
                dP = dO @ Vc.T
                dS = P * (dP - D[:, None])
                dq[b, h, r0:r1] = scale * (dS @ Kc)
                dk[b, g, cols] += scale * (dS.T @ q[b, h, r0:r1])
                dv[b, g, cols] += P.T @ dO
    return dq, dk, dv


def unmasked_pairs(q_len: int, ttt_step: int, valid_len: int) -> int:
    """Number of (query, key) pairs in M for one (batch, head): |M| summed.

    Counted from the mask itself (no closed form), so it is a definition, not a
    shortcut; the closed form used by the benchmark is pinned against it.
    """
    return int(mask(q_len, ttt_step, valid_len).sum())
