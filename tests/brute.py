"""Double-precision brute-force attention: the textbook definition, used to pin
the oracle (never the GPU path's arithmetic, never the oracle's code).

    O = softmax(scale * Q K^T + mask, causal) V,   L = logsumexp of the same row

in natural exp/log, with key j visible to query row i under the causal rule
iff j <= max(kl - ql, 0) + i (the page's bottom-right alignment, offset
clamped at zero). A row with no visible key gives O = 0 and L = -inf.
GQA: query head h reads kv head h // (H // Hkv).
"""
import numpy as np


def attention_f64(q, k, v, mask, scale, causal):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, ql, D = q.shape
    Hkv, kl = k.shape[1], k.shape[2]
    group = H // Hkv
    O = np.zeros((B, H, ql, D))
    L = np.full((B, H, ql), -np.inf)
    off = max(kl - ql, 0)
    for b in range(B):
        for h in range(H):
            kvh = h // group
            s = scale * (q[b, h] @ k[b, kvh].T)
            if mask is not None:
                s = s + np.asarray(mask[b, h], dtype=np.float64)
            if causal:
                i = np.arange(ql)[:, None]
                j = np.arange(kl)[None, :]
                s = np.where(j > off + i, -np.inf, s)
            for i in range(ql):
                row = s[i]
                if kl == 0 or not np.isfinite(row).any():
                    continue
                m = row[np.isfinite(row)].max()
                e = np.exp(row - m)
                z = e.sum()
                L[b, h, i] = m + np.log(z)
                O[b, h, i] = (e @ v[b, kvh]) / z
    return O, L
