"""GPU parity of the paged-KV forward (fa_paged_fwd) against the CPU oracle
(marked gpu). The layout and the check follow the adjacent attention API on
the pages (paged caches [n_blocks, Hkv, block_size, D] filled in a shuffled
block order with a few unused blocks, a block table, a key count per
sequence): the paged result must equal attention over each sequence's first
seq_lens[b] keys, which the oracle computes from the contiguous keys. Bounds
as for the plain forward (by each sequence's key count); a sequence with no
key gives O = +0 and L = -inf exactly. Sequences of more than 256 keys run
plain tiles (with the compensated redo) where the accuracy rule allows.
"""
import math

import numpy as np
import pytest

import fagen
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _paged(keys, values, bs, seed):
    """keys, values: bf16 bits [B, Hkv, N, D] -> (k_cache, v_cache, table) with
    the blocks of every sequence in a seeded shuffled order plus 3 unused ones."""
    B, Hkv, N, D = keys.shape
    per = -(-N // bs)
    blocks = B * per + 3
    order = np.random.default_rng(seed).permutation(blocks)
    kc = np.zeros((blocks, Hkv, bs, D), np.uint16)
    vc = np.zeros((blocks, Hkv, bs, D), np.uint16)
    for b in range(B):
        for j in range(per):
            blk, n = order[b * per + j], min(bs, N - j * bs)
            kc[blk, :, :n] = keys[b, :, j * bs:j * bs + n]
            vc[blk, :, :n] = values[b, :, j * bs:j * bs + n]
    table = order[:B * per].reshape(B, per).astype(np.int32)
    return kc, vc, table


def _run(case, n_split, seed, with_sinks=False):
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, Hkv, ql, D, bs, lens, causal = case
    N = max(max(lens), 1)
    s = fagen.SEED_BASE + seed
    q = fagen.normal_bf16(s, 0, (B, H, ql, D))
    keys = fagen.normal_bf16(s, 1, (B, Hkv, N, D))
    values = fagen.normal_bf16(s, 2, (B, Hkv, N, D))
    kc, vc, table = _paged(keys, values, bs, seed)
    dev = "cuda:0"
    # sinks: log(longest sequence) + N(0, 2^2), rounded through bf16
    sinks = None
    if with_sinks:
        z = fagen.bf16_bits_to_f32(fagen.normal_bf16(s, 5, (H,), sigma=2.0))
        sinks = (np.float32(math.log(N)) + z).astype(np.float32)
    O, L = fa.paged_fwd(gu.to_dev(q, dev), gu.to_dev(kc, dev), gu.to_dev(vc, dev),
                        torch.from_numpy(table).to(dev),
                        torch.tensor(lens, dtype=torch.int32, device=dev), causal=causal,
                        n_split=n_split,
                        sinks=None if sinks is None else torch.from_numpy(sinks).to(dev))
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    o, l = gu.widen(bits), L.cpu().numpy()
    scale = 1.0 / math.sqrt(D)
    for b, n in enumerate(lens):
        of, ob, lr = oracle.fwd_dv(q[b:b + 1], keys[b:b + 1, :, :n].copy(),
                                   values[b:b + 1, :, :n].copy(), None, 1, H, Hkv, ql, n, D, D,
                                   scale, causal, sinks=sinks)
        tol_o, tol_l = gu.tolerances(n)
        eo, el, _ = gu.compare(o[b:b + 1], l[b:b + 1], bits[b:b + 1], ob, lr, tol_o, tol_l,
                               f"paged {case} seq {b}", o_ref_f32=of)
        print(f"paged {case} n_split={n_split} seq {b} (len {n}): dO={eo:.3e} dL={el:.3e}")
    return o, l


CASES = [
    # (B, H, Hkv, ql, D, block_size, seq_lens, causal)
    (1, 4, 4, 1, 128, 64, [37], True),
    (3, 8, 2, 1, 128, 64, [1, 64, 300], True),
    (2, 4, 1, 4, 64, 64, [4, 77], True),
    (2, 2, 2, 1, 256, 128, [9, 513], True),
    (2, 8, 2, 1, 128, 64, [1500, 3000], True),
    (1, 8, 2, 4, 128, 64, [2100], True),
    (1, 4, 2, 1, 256, 64, [1100], True),
    (2, 4, 2, 300, 128, 128, [1000, 450], True),   # prefill against a cache
    (2, 4, 4, 70, 64, 64, [300, 200], False),
    (2, 4, 2, 1, 64, 64, [0, 200], True),          # a sequence with no key
    # blocks shorter than a 64-key tile (looked up per copy instruction)
    (1, 4, 4, 1, 128, 16, [37], True),
    (3, 8, 2, 1, 128, 16, [1, 64, 300], True),
    (2, 4, 1, 4, 64, 32, [4, 77], True),
    (2, 2, 2, 1, 256, 16, [9, 513], True),
    (2, 8, 2, 1, 128, 48, [1500, 3000], True),
    (2, 4, 2, 300, 128, 16, [1000, 450], True),
    (2, 4, 4, 70, 64, 96, [300, 200], False),
    (2, 4, 2, 1, 256, 32, [0, 200], True),
]


@pytest.mark.parametrize("n_split", [0, 8])
@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_paged_matches_contiguous_oracle(case, n_split):
    print(f"case paged {case} n_split={n_split}", flush=True)
    _run(case, n_split, seed=11000 + CASES.index(case))


@pytest.mark.parametrize("n_split", [0, 6])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_paged_plain_tiles_and_redo(D, n_split):
    """Sequences of more than 256 keys run plain tiles (pre-scaled Q, bf16 P)
    where every row of a tile (chunk) sees none or at least 128 of its keys.
    V times 16 (exact in bf16) at the usual scale makes many rows reach
    |O| >= 1 and take the compensated redo; a 200-key sequence stays
    compensated. Every row against the oracle."""
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, Hkv, ql, bs = 3, 4, 2, 200, 64
    lens = [1500, 200, 700]
    N = max(lens)
    s = fagen.SEED_BASE + 11900 + D + n_split
    print(f"case paged plain/redo D={D} n_split={n_split}", flush=True)
    q = fagen.normal_bf16(s, 0, (B, H, ql, D))
    keys = fagen.normal_bf16(s, 1, (B, Hkv, N, D))
    vb = fagen.normal_bf16(s, 2, (B, Hkv, N, D))
    e = (vb >> 7) & 0xFF
    assert np.all(e < 250)
    values = np.where(e != 0, vb + np.uint16(4 << 7), vb).astype(np.uint16)  # exponent + 4
    kc, vc, table = _paged(keys, values, bs, 11900 + D)
    dev = "cuda:0"
    O, L = fa.paged_fwd(gu.to_dev(q, dev), gu.to_dev(kc, dev), gu.to_dev(vc, dev),
                        torch.from_numpy(table).to(dev),
                        torch.tensor(lens, dtype=torch.int32, device=dev),
                        causal=True, n_split=n_split)
    torch.cuda.synchronize()
    bits = O.view(torch.int16).cpu().numpy().view(np.uint16)
    o, l = gu.widen(bits), L.cpu().numpy()
    big = 0
    for b, n in enumerate(lens):
        of, ob, lr = oracle.fwd(q[b:b + 1], keys[b:b + 1, :, :n].copy(),
                               values[b:b + 1, :, :n].copy(), None, 1, H, Hkv, ql, n, D,
                               1.0 / math.sqrt(D), True)
        big += int((np.abs(of) >= 1).any(axis=-1).sum())
        tol_o, tol_l = gu.tolerances(n)
        eo, el, rms = gu.compare(o[b:b + 1], l[b:b + 1], bits[b:b + 1], ob, lr, tol_o, tol_l,
                                 f"paged plain D={D} seq {b}", o_ref_f32=of)
        print(f"paged plain/redo D={D} n_split={n_split} seq {b} (len {n}): dO={eo:.3e} "
              f"dL={el:.3e} relRMS={rms:.2e}")
        assert rms <= 5e-3
    assert big > 0


@pytest.mark.parametrize("n_split", [0, 8])
@pytest.mark.parametrize("case", [CASES[i] for i in (1, 3, 7, 9, 12, 15, 17)],
                         ids=[str(i) for i in (1, 3, 7, 9, 12, 15, 17)])
def test_paged_sinks_match_contiguous_oracle(case, n_split):
    """Sinks through the paged forward (packed GQA decode, prefill, a sequence
    with no key: O = +0 and L = its head's sink), plain and split-KV."""
    print(f"case paged sinks {case} n_split={n_split}", flush=True)
    _run(case, n_split, seed=11500 + CASES.index(case), with_sinks=True)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_small_blocks_give_the_bits_of_whole_tile_blocks(D):
    """The same sequences in blocks of 16 and of 64 keys: only the copies'
    addressing differs, so O and L agree bit for bit (plain and split)."""
    import torch
    import flash_attention_forward_fa_amd as fa
    B, H, Hkv, ql, lens = 3, 8, 2, 1, [700, 1, 2049]
    print(f"case paged small vs whole blocks D={D}", flush=True)
    s = fagen.SEED_BASE + 11800 + D
    N = max(lens)
    q = gu.to_dev(fagen.normal_bf16(s, 0, (B, H, ql, D)), "cuda:0")
    keys = fagen.normal_bf16(s, 1, (B, Hkv, N, D))
    values = fagen.normal_bf16(s, 2, (B, Hkv, N, D))
    n = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    outs = []
    for bs in (16, 64):
        kc, vc, table = _paged(keys, values, bs, 11800 + D + bs)
        args = (q, gu.to_dev(kc, "cuda:0"), gu.to_dev(vc, "cuda:0"),
                torch.from_numpy(table).to("cuda:0"), n)
        outs.append([fa.paged_fwd(*args, causal=True, n_split=ns) for ns in (0, 8)])
    torch.cuda.synchronize()
    for (o1, l1), (o2, l2) in zip(*outs):
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_paged_table_entries_outside_the_cache_are_clamped():
    """A table entry outside 0..n_blocks-1 reads a clamped block: the call
    completes with finite output (the keys it read are not that sequence's)."""
    import torch
    import flash_attention_forward_fa_amd as fa
    print("case paged clamp", flush=True)
    B, H, Hkv, ql, D, bs = 2, 4, 2, 1, 64, 64
    s = fagen.SEED_BASE + 11900
    q = gu.to_dev(fagen.normal_bf16(s, 0, (B, H, ql, D)), "cuda:0")
    kc = gu.to_dev(fagen.normal_bf16(s, 1, (5, Hkv, bs, D)), "cuda:0")
    vc = gu.to_dev(fagen.normal_bf16(s, 2, (5, Hkv, bs, D)), "cuda:0")
    table = torch.tensor([[0, 10 ** 9], [-5, 2]], dtype=torch.int32, device="cuda:0")
    lens = torch.tensor([128, 100], dtype=torch.int32, device="cuda:0")
    O, L = fa.paged_fwd(q, kc, vc, table, lens, causal=True)
    # blocks of 16 keys: the same clamping on the per-instruction lookup
    k16, v16 = kc.view(5 * 4, Hkv, 16, D), vc.view(5 * 4, Hkv, 16, D)
    t16 = torch.tensor([[0, 1, 2, 3, 10 ** 9, -7, 19, 4], [-5, 2, 3, 1 << 30, 0, 0, 0, 0]],
                       dtype=torch.int32, device="cuda:0")
    O16, L16 = fa.paged_fwd(q, k16, v16, t16, lens, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(O.float()).all() and torch.isfinite(L).all()
    assert torch.isfinite(O16.float()).all() and torch.isfinite(L16).all()


def test_paged_errors_raise_from_binding():
    import torch
    import flash_attention_forward_fa_amd as fa
    q = torch.zeros(1, 2, 1, 64, device="cuda:0", dtype=torch.bfloat16)
    c = torch.zeros(4, 2, 40, 64, device="cuda:0", dtype=torch.bfloat16)
    t = torch.zeros(1, 2, dtype=torch.int32, device="cuda:0")
    n = torch.tensor([40], dtype=torch.int32, device="cuda:0")
    with pytest.raises(fa.FAError) as e:
        fa.paged_fwd(q, c, c, t, n)
    assert e.value.status == 12
    with pytest.raises(ValueError):
        fa.paged_fwd(q, c, c, t.float(), n)


def _draw_paged(i):
    """A seeded random paged configuration (a pure function of i)."""
    r = np.random.default_rng(0xFA9E + 15485863 * i)
    D = int(r.choice([64, 128, 256]))
    B = int(r.integers(1, 4))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4]))
    ql = int(r.choice([1, int(r.integers(2, 17)), int(r.integers(17, 260))], p=[0.4, 0.2, 0.4]))
    bs = int(16 * r.integers(1, 9))
    lens = [int(r.choice([0, int(r.integers(1, 300)), int(r.integers(300, 2500))],
                         p=[0.1, 0.4, 0.5])) for _ in range(B)]
    causal = bool(r.random() < 0.7)
    n_split = int(r.choice([0, 0, 2, 8, 24]))
    sinks = bool(r.random() < 0.3)
    return (B, Hkv * G, Hkv, ql, D, bs, lens, causal), n_split, sinks


@pytest.mark.parametrize("i", range(24))
def test_paged_random_configs(i):
    """24 seeded random paged configurations (block sizes of 16 to 128 keys,
    per-sequence lengths from 0 to 2500, one to 259 query rows, split-KV,
    sinks) against the oracle per sequence."""
    case, n_split, sinks = _draw_paged(i)
    print(f"case paged random {i}: {case} n_split={n_split} sinks={sinks}", flush=True)
    _run(case, n_split, seed=12000 + i, with_sinks=sinks)
