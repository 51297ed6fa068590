"""Independent formulations used to pin the oracle (test helpers only).

Neither of these touches oracle.c or the GPU library:
  * ``dense_numpy``: per request, the key/value sequence is assembled straight
    from the inputs (prior positions from the *initial* cache through the page
    table, new positions from k_new/v_new), then softmax(Q K^T * scale + mask) V
    is evaluated as fp64 matrix products.
  * ``sdpa_torch``: the same sequences fed to torch's CPU
    scaled_dot_product_attention in float64, with GQA expanded by
    repeat_interleave and an explicit bottom-right boolean mask.
"""
from __future__ import annotations

import numpy as np
import torch


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def request_sequences(b, r):
    """(K, V) of request r as float64 [L, Hkv, D], built from the call inputs."""
    from ragged_paged_attention_amd.inputs import u16

    S = b.page_size
    c = int(b.context_lens[r])
    t0, t1 = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1])
    L = c + (t1 - t0)
    P, _, Hkv, D = b.k_cache.shape
    kc = widen(u16(b.k_cache)).reshape(P * S, Hkv, D)
    vc = widen(u16(b.v_cache)).reshape(P * S, Hkv, D)
    pos = np.arange(c)
    rows = b.page_table[r].numpy().astype(np.int64)[pos // S] * S + pos % S
    K = np.concatenate([kc[rows], widen(u16(b.k_new))[t0:t1]], axis=0)
    V = np.concatenate([vc[rows], widen(u16(b.v_new))[t0:t1]], axis=0)
    assert K.shape[0] == L
    return K, V


def visible_mask(c, q, L, causal):
    """[q, L] boolean: query i (position c+i) sees key j."""
    i = np.arange(q)[:, None]
    j = np.arange(L)[None, :]
    if causal:
        return j <= c + i
    return np.ones((q, L), dtype=bool)


def dense_numpy(b):
    """float64 [T, Hq, D] by dense matrix softmax attention per request."""
    from ragged_paged_attention_amd.inputs import u16

    T, Hq, D = b.q.shape
    Hkv = b.num_kv_heads
    G = Hq // Hkv
    scale = b.effective_scale()
    Q = widen(u16(b.q))
    out = np.zeros((T, Hq, D))
    for r in range(b.num_reqs):
        t0, t1 = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1])
        if t1 == t0:
            continue
        K, V = request_sequences(b, r)
        c, L = int(b.context_lens[r]), K.shape[0]
        mask = visible_mask(c, t1 - t0, L, b.causal)
        for h in range(Hq):
            hk = h // G
            s = Q[t0:t1, h, :] @ K[:, hk, :].T * scale
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w /= w.sum(axis=1, keepdims=True)
            out[t0:t1, h, :] = w @ V[:, hk, :]
    return out


def sdpa_torch(b):
    """float64 [T, Hq, D] from torch.nn.functional.scaled_dot_product_attention."""
    from ragged_paged_attention_amd.inputs import u16

    T, Hq, D = b.q.shape
    G = Hq // b.num_kv_heads
    Q = torch.from_numpy(widen(u16(b.q)))
    out = torch.zeros((T, Hq, D), dtype=torch.float64)
    for r in range(b.num_reqs):
        t0, t1 = int(b.cu_q_lens[r]), int(b.cu_q_lens[r + 1])
        if t1 == t0:
            continue
        K, V = request_sequences(b, r)
        c, L = int(b.context_lens[r]), K.shape[0]
        k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D]
        v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
        q = Q[t0:t1].permute(1, 0, 2)  # [Hq, q, D]
        mask = torch.from_numpy(visible_mask(c, t1 - t0, L, b.causal))
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=mask, scale=b.effective_scale())
        out[t0:t1] = o.permute(1, 0, 2)
    return out.numpy()
