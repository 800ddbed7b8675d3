"""Helpers of the GPU tests: upload generated inputs, run the HIP forward
through the binding, and compare with the oracle element by element."""
import numpy as np

import flash_attention_forward_fa_amd as fa


def to_dev(bits_or_f32, dev):
    import torch
    a = np.ascontiguousarray(bits_or_f32)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a.astype(np.float32)).to(dev)


def run(inputs, w, dev="cuda:0", scale=None):
    """HIP forward on the generated inputs of workload-like `w`; returns
    (O as float32 numpy, L numpy, raw O bits)."""
    import torch
    q, k, v = (to_dev(inputs[n], dev) for n in ("q", "k", "v"))
    mask = None if inputs.get("mask") is None else to_dev(inputs["mask"], dev)
    O, L = fa.train_fwd(q, k, v, mask=mask, scale=w.scale if scale is None else scale,
                        causal=w.causal)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    return widen(bits), L.cpu().numpy(), bits


def widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def tolerances(kl):
    """Absolute bounds on O and L: 5e-3 / 3e-3 up to 256 keys, 1e-2 / 1e-2 beyond."""
    return (5e-3, 3e-3) if kl <= 256 else (1e-2, 1e-2)


def bf16_step(x):
    """Size of one bf16 rounding step (2^-7 relative) at |x| (float32 array)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float32)), np.float32(2.0 ** -126))
    return np.exp2(np.floor(np.log2(ax)) - 7)


def compare(o_gpu, l_gpu, o_bits, ob_ref, l_ref, tol_o, tol_l, label="", o_ref_f32=None):
    """Element-wise parity: fully masked rows exact (O = +0 bits, L = -inf),
    every other element within the absolute bounds; no NaN anywhere.

    O is compared with the oracle's O rounded to bf16 (as the method's page
    compares it), within tol_o. Where one bf16 step of the reference value
    exceeds tol_o (|O| >= 1 at 5e-3, |O| >= 2 at 1e-2), that comparison is
    ill-posed: two correct f32 results a few ulps apart can round to bf16
    values one step apart, more than the tolerance. There (given o_ref_f32,
    the oracle's unrounded O) the GPU's bf16 O is bounded against the
    unrounded value: tol_o plus half a bf16 step (the rounding of the GPU's
    own f32 result). Returns (max |dO| against the rounded oracle, max |dL|,
    relative RMS of dO)."""
    o_ref = widen(ob_ref)
    assert not np.isnan(o_gpu).any() and not np.isnan(l_gpu).any(), f"{label}: NaN in output"
    dead = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_gpu), dead), f"{label}: -inf rows of L differ"
    assert np.all(o_bits[dead] == 0), f"{label}: fully masked rows must be +0 bits"
    live = ~dead
    if not live.any():
        return 0.0, 0.0, 0.0
    d_o = np.abs(o_gpu[live] - o_ref[live])
    d_l = np.abs(l_gpu[live] - l_ref[live])
    err_o, err_l = float(d_o.max()), float(d_l.max())
    rms = float(np.sqrt((d_o ** 2).mean() / max((o_ref[live] ** 2).mean(), 1e-30)))
    if o_ref_f32 is not None:
        of = np.asarray(o_ref_f32, np.float32)[live]
        g = o_gpu[live]
        coarse = bf16_step(of) > tol_o
        mag = np.maximum(np.abs(of) + tol_o, np.abs(g))
        excess = np.where(coarse, np.abs(g - of) - (tol_o + 0.5 * bf16_step(mag)), d_o - tol_o)
        worst = float(excess.max())
        assert worst <= 0, (f"{label}: |dO| beyond the bound by {worst:.3e} (tol {tol_o:.1e}; "
                            f"{int(coarse.sum())} elements where a bf16 step exceeds it are "
                            "bounded against the unrounded oracle)")
    else:
        assert err_o <= tol_o, f"{label}: max|dO| = {err_o:.3e} > {tol_o:.1e}"
    assert err_l <= tol_l, f"{label}: max|dL| = {err_l:.3e} > {tol_l:.1e}"
    return err_o, err_l, rms
