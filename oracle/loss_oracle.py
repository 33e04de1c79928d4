"""CPU fp64 oracle for the in-place masked softmax-loss gradient.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never touches it, and it
imports nothing from the product.

What it computes (the kernel the review's "§3 -> Memory-efficient gradient
computation" describes; formulas in "§4 Core formulas -> Masked softmax loss"
and "-> In-place backward"):

* the loss of a row, L = -sum_i p_i log softmax(z)_i, with p the target
  distribution;
* the gradient of sum_n g_n L_n with respect to the logits, which the kernel
  writes over z.

Readings where the pages are silent:
  - z, p are [N, V] (one row per token, V draft-vocabulary columns) and the
    upstream gradient is one weight per row, g [N], broadcast along the row
    (a per-token loss has one scalar gradient per token; the loss mask and the
    1 / normaliser live in it, so a masked row has g = 0 and gets a zero
    gradient); then s = g * sum_i p_i;
  - p need not sum to one (targets restricted to a draft vocabulary);
  - the loss is returned per row, unweighted by g.

Pinned by ``tests/test_loss_oracle.py`` against a hand-derived fixture,
torch's cross entropy with probability targets (a library routine) and its
autograd, central finite differences, and invariants; not "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """pi = exp(z_i) / sum_j exp(z_j) per row (review §4 "Masked softmax loss"), with the
    row maximum subtracted first (the same quotient, without overflow)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def loss_rows(z: np.ndarray, p: np.ndarray) -> np.ndarray:
    """L = -sum_i p_i log softmax(z)_i per row (review §4 "Masked softmax loss").
    log softmax(z)_i is z_i - log sum_j exp(z_j); terms with p_i = 0 contribute 0."""
    z = np.asarray(z, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True))
    return -(p * (z - lse)).sum(axis=-1)


def grad_inplace(z: np.ndarray, p: np.ndarray, g: np.ndarray) -> np.ndarray:
    """The value the kernel leaves in z: the gradient of sum_n g_n L_n with respect to the
    logits of row n, g_n (softmax(z_n) sum_i p_ni - p_n), which is the review's §4
    "In-place backward" expression with its s = sum_i p_i g_i (g [N] broadcast over each row).
    """
    z = np.asarray(z, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    g_row = np.asarray(g, dtype=np.float64)[..., None]
    return g_row * (softmax_rows(z) * p.sum(axis=-1, keepdims=True) - p)


def loss_and_grad(z, p, g):
    """(per-row loss [N], gradient [N, V]) in fp64."""
    return loss_rows(z, p), grad_inplace(z, p, g)
