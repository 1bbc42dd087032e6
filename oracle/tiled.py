"""Online-softmax tile recurrence in fp64 (numpy). TEST INFRASTRUCTURE ONLY.

This is the FlashAttention-2 forward as the pages derive it, written with
numpy matmuls as the only library primitive and no other reordering:

* the outer loop walks query tiles of ``block_m`` rows; for each, the running
  state is m = -inf, l = 0, acc = 0 ("Triton: FlashAttention-2 Forward Pass",
  The online-softmax state and its shapes);
* the inner loop walks key tiles of ``block_n`` keys up to the key length, and
  for causal attention stops after the tile's last query row ("A09 - Advanced
  Triton & FlashAttention", section 3, Causal masking: skipping beats masking);
* per key tile: scores scale*Q K^T; masked keys (beyond the key length, or
  later than the query under the causal mask) get -inf; m_new = max(m,
  rowmax); alpha = exp(m - m_new); p = exp(s - m_new); l = alpha*l + rowsum(p);
  acc = alpha*acc + p V; m = m_new ("A09", section 3, The rescaling update,
  written out; "Building a Verifiable FlashAttention Forward from PyTorch to
  Triton", Part 2);
* after the loop: O = acc / l once, LSE = m + log(l) ("FlashAttention 2 from
  PyTorch to Triton", What I am building).

Where the pages differ on the sentinel for a row that has seen no visible key
(-1e6, -1e9 or -inf with a guard), this follows the -inf reading with the guard
("Triton: FlashAttention-2 Forward Pass", The rescale direction; "Building a
Verifiable FlashAttention Forward", Part 3 Step 2): while m_new is -inf the
exponent reference is taken as 0, so alpha and p are exactly 0 and no NaN
appears; a row that never sees a key ends with l = 0, O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np


def tiled_attention(q, k, v, scale, causal, block_m, block_n, n_kv=None):
    """q, k, v: [BH, N, D] (any float dtype). Returns (O, LSE) in fp64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    BH, N, D = q.shape
    if n_kv is None:
        n_kv = N
    out = np.zeros((BH, N, D))
    lse = np.full((BH, N), -np.inf)
    for bh in range(BH):
        for m_start in range(0, N, block_m):
            m_end = min(m_start + block_m, N)
            q_pos = np.arange(m_start, m_end)
            q_tile = q[bh, m_start:m_end]
            m_run = np.full(m_end - m_start, -np.inf)
            l_run = np.zeros(m_end - m_start)
            acc = np.zeros((m_end - m_start, D))
            end_n = min(n_kv, m_end) if causal else n_kv
            for n_start in range(0, end_n, block_n):
                n_end = min(n_start + block_n, N)
                kv_pos = np.arange(n_start, n_end)
                s = (q_tile @ k[bh, n_start:n_end].T) * scale
                masked = (kv_pos[None, :] >= n_kv)
                if causal:
                    masked = masked | (kv_pos[None, :] > q_pos[:, None])
                s = np.where(masked, -np.inf, s)
                m_new = np.maximum(m_run, s.max(axis=1))
                m_ref = np.where(np.isneginf(m_new), 0.0, m_new)
                alpha = np.exp(m_run - m_ref)
                p = np.exp(s - m_ref[:, None])
                l_run = alpha * l_run + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[bh, n_start:n_end]
                m_run = m_new
            seen = l_run > 0
            safe_l = np.where(seen, l_run, 1.0)
            out[bh, m_start:m_end] = np.where(seen[:, None], acc / safe_l[:, None], 0.0)
            lse[bh, m_start:m_end] = np.where(seen, m_run + np.log(safe_l), -np.inf)
    return out, lse
