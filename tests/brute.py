"""Double-precision brute-force attention: the textbook definition, used to pin
the oracle (never the GPU path's arithmetic, never the oracle's code).

    O = softmax(scale * Q K^T + mask, causal) V,   L = logsumexp of the same row

in natural exp/log, with key j visible to query row i under the causal rule
iff j <= max(kl - ql, 0) + i (the page's bottom-right alignment, offset
clamped at zero). With a sliding window w (which implies the causal rule),
key j is visible iff off + i - w <= j <= off + i, off = max(kl - ql, 0).
A row with no visible key gives O = 0 and L = -inf.
GQA: query head h reads kv head h // (H // Hkv). V (and O) may be wider or
narrower than Q and K.
"""
import numpy as np


def attention_f64(q, k, v, mask, scale, causal, window=None, sinks=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, ql, D = q.shape
    Hkv, kl = k.shape[1], k.shape[2]
    Dv = v.shape[3]
    group = H // Hkv
    O = np.zeros((B, H, ql, Dv))
    L = np.full((B, H, ql), -np.inf)
    off = max(kl - ql, 0)
    for b in range(B):
        for h in range(H):
            kvh = h // group
            s = scale * (q[b, h] @ k[b, kvh].T)
            if mask is not None:
                s = s + np.asarray(mask[b, h], dtype=np.float64)
            i = np.arange(ql)[:, None]
            j = np.arange(kl)[None, :]
            if causal or window is not None:
                s = np.where(j > off + i, -np.inf, s)
            if window is not None:
                s = np.where(j < off + i - window, -np.inf, s)
            # a sink: one more logit in the row's softmax, with a zero value
            sink = -np.inf if sinks is None else float(sinks[h])
            for i in range(ql):
                row = s[i]
                if (kl == 0 or not np.isfinite(row).any()) and not np.isfinite(sink):
                    continue
                m = max(row[np.isfinite(row)].max() if np.isfinite(row).any() else -np.inf,
                        sink)
                e = np.exp(row - m)
                z = e.sum() + np.exp(sink - m)
                L[b, h, i] = m + np.log(z)
                O[b, h, i] = (e @ v[b, kvh]) / z
    return O, L


def attention_grads_f64(q, k, v, mask, dO, scale, causal, window=None, sinks=None):
    """Gradients of sum(O * dO) with respect to q, k, v for the same textbook
    definition, by torch's autograd in float64 on the CPU (a library routine
    serving as the differentiation step). Rows with no visible key have O = 0
    and contribute nothing. Returns numpy (dQ, dK, dV); with sinks (one logit
    per query head, one more softmax term with a zero value), also dsinks [H]."""
    import torch
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float64)
    qt, kt, vt = t(q).requires_grad_(), t(k).requires_grad_(), t(v).requires_grad_()
    st = None if sinks is None else t(sinks).requires_grad_()
    B, H, ql, D = qt.shape
    Hkv, kl = kt.shape[1], kt.shape[2]
    group = H // Hkv
    idx = torch.arange(H) // group
    kr, vr = kt[:, idx], vt[:, idx]                       # [B, H, kl, D]
    s = scale * torch.matmul(qt, kr.transpose(-1, -2).contiguous())
    if mask is not None:
        s = s + t(mask)
    off = max(kl - ql, 0)
    q_abs = off + torch.arange(ql)[:, None]
    if causal or window is not None:
        s = s.masked_fill(torch.arange(kl)[None, :] > q_abs, float("-inf"))
    if window is not None:
        s = s.masked_fill(torch.arange(kl)[None, :] < q_abs - window, float("-inf"))
    if st is not None:
        # the sink as one more column of every row's logits; its weight is
        # dropped from the weighted sum (a zero value)
        col = st[None, :, None, None].expand(s.shape[0], s.shape[1], s.shape[2], 1)
        s = torch.cat([s, col], dim=-1)
    live = torch.isfinite(s).any(dim=-1, keepdim=True)
    s = torch.where(live, s, torch.zeros_like(s))
    p = torch.softmax(s, dim=-1) * live
    if st is not None:
        p = p[..., :kl]
    O = torch.matmul(p, vr)
    (O * t(dO)).sum().backward()
    if st is None:
        return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), st.grad.numpy()
