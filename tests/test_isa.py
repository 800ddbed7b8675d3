"""Checks on the gfx950 machine code of the forward and backward kernels (no GPU needed:
hipcc cross-compiles the kernels to assembly here).

- No v_mfma instruction may be reachable inside an EXEC-masked region
  (between an s_*_saveexec and the instruction that restores EXEC), on any
  path through the kernel's basic blocks. Such an MFMA still accumulates when
  EXEC is zero, so a wave-uniform condition that the compiler could not prove
  uniform silently corrupts O.
- The key-tile loop (the innermost loop: the deepest "Depth=N" in the
  compiler's block annotations) must not touch scratch memory (register
  spills) in any variant.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    from flash_attention_forward_fa_amd import build
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    text = ""
    outs, procs = [], []
    for src in build.SOURCES:  # (compiled in parallel)
        out = tmp_path_factory.mktemp("isa") / (os.path.basename(src) + ".s")
        outs.append(out)
        procs.append(subprocess.Popen([build.HIPCC, *flags, "--cuda-device-only", "-S", "-o",
                                       str(out), src], stdout=subprocess.DEVNULL,
                                      stderr=subprocess.DEVNULL))
    assert all(p.wait() == 0 for p in procs), "hipcc failed"
    for out in outs:
        text += out.read_text() + "\n"
    kernels = {}
    name = None
    for line in text.split("\n"):
        m = re.match(r"^(_Z\w*fa_(?:fwd|bwd)_kernel\w+):", line)
        if m:
            name = m.group(1)
            kernels[name] = []
        elif name is not None:
            kernels[name].append(line)
    return kernels


def test_all_variants_present(isa):
    fwd = [n for n in isa if "fa_fwd_kernel" in n]
    bwd = [n for n in isa if "fa_bwd_kernel" in n]
    # head_dim (64, 128, 256) x {none, causal, window} x {mixed, compensated f32 mask, bf16 mask}
    # + split-KV, paged (whole-tile and short blocks), paged split-KV (head_dim x causal
    # each), bool masks: 66; the (key, value) pairs (80, 80), (96, 96), (96, 64),
    # (192, 192), (192, 128) x {none, causal, window} x {mixed, three mask kinds}: 60
    # + the narrow split-KV kernels (at most 16 query rows) of head_dim 64 and 128:
    # {split, paged split, short-block paged split} x causal x 2 = 12
    assert len(fwd) == 138
    assert len(bwd) == 72  # head_dim (3) x {dQ, dKV} x {none, causal, window} x mask (4 kinds)


_OPEN = (re.compile(r"s_(?:and|andn2|or)_saveexec_b64 (s\[\d+:\d+\])"),
         re.compile(r"^s_mov_b64 (s\[\d+:\d+\]), exec$"))
_CLOSE = (re.compile(r"^s_or_b64 exec, exec, (s\[\d+:\d+\])"),
          re.compile(r"^s_mov_b64 exec, (s\[\d+:\d+\])"))
# s_xor_b64 sY, exec, sX with sX a saved EXEC: sY holds the lanes the region
# left out, and the region is closed by OR-ing them back from sY
_RENAME = re.compile(r"^s_xor_b64 (s\[\d+:\d+\]), exec, (s\[\d+:\d+\])")
# s_or_saveexec_b64 sY, sX with sX the lanes an if left out (the else of an
# if/else): EXEC becomes the region's lanes again, sY saves the then-lanes and
# the region goes on (the else) until EXEC is OR-ed back from sY
_ELSE = re.compile(r"^s_or_saveexec_b64 (s\[\d+:\d+\]), (s\[\d+:\d+\])")


def mfma_under_exec_mask(lines):
    """MFMAs reachable while an EXEC-masked region is open, by dataflow over
    the kernel's basic blocks. A region opens with s_*_saveexec_b64 sX or
    s_mov_b64 sX, exec (the old EXEC saved in sX) and closes when EXEC is
    restored from sX (or from the register that an s_xor_b64 with EXEC turned
    sX into), which also closes every region opened after it, so the state on
    a path is a stack of saved registers. Blocks end at labels and
    after branches; a block's entry states are those of all its predecessors,
    so an MFMA is reported if any path reaches it inside a region."""
    blocks, label, body = [], "<entry>", []
    for raw in lines:
        m = re.match(r"^(\.L\w+):", raw)
        if m:
            blocks.append((label, body))
            label, body = m.group(1), []
            continue
        t = raw.strip()
        if not t or t.startswith((";", ".")):
            continue
        body.append(t)
        if t.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append((label, body))
            label, body = None, []
    blocks.append((label, body))
    blocks = [blk for blk in blocks if blk[0] is not None or blk[1]]
    index = {blk[0]: i for i, blk in enumerate(blocks) if blk[0]}

    def successors(i):
        last = blocks[i][1][-1] if blocks[i][1] else ""
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if last.startswith("s_branch"):
            return [index[last.split()[1]]]
        if last.startswith("s_cbranch"):
            return [index[last.split()[1]]] + nxt
        if last.startswith(("s_endpgm", "s_setpc")):
            return []
        return nxt

    states, work, found = {0: {()}}, [0], []
    while work:
        i = work.pop()
        for entry in list(states[i]):
            stack = list(entry)
            for t in blocks[i][1]:
                rn = _RENAME.search(t) or _ELSE.search(t)
                if rn and rn.group(2) in stack:
                    stack[stack.index(rn.group(2))] = rn.group(1)
                    continue
                op = next((m for r in _OPEN for m in [r.search(t)] if m), None)
                cl = next((m for r in _CLOSE for m in [r.search(t)] if m), None)
                if op:
                    stack.append(op.group(1))
                elif cl:
                    if cl.group(1) in stack:
                        del stack[stack.index(cl.group(1)):]
                elif "v_mfma" in t and stack:
                    found.append(t)
            out = tuple(stack[-8:])
            for j in successors(i):
                seen = states.setdefault(j, set())
                if out not in seen and len(seen) < 32:
                    seen.add(out)
                    work.append(j)
    return found


def test_exec_check_finds_masked_mfma():
    # the checker itself: a masked MFMA in line, one reached by a branch from
    # inside a region, and the layout the compiler emits (a region whose body
    # sits after an s_endpgm, an unmasked MFMA after it reached from elsewhere)
    mf = "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]"
    assert mfma_under_exec_mask(["s_and_saveexec_b64 s[0:1], vcc", mf,
                                 "s_or_b64 exec, exec, s[0:1]"])
    assert mfma_under_exec_mask(["s_and_saveexec_b64 s[0:1], vcc", "s_cbranch_execnz .LBB0_2",
                                 "s_or_b64 exec, exec, s[0:1]", "s_endpgm", ".LBB0_2:", mf,
                                 "s_branch .LBB0_3", ".LBB0_3:", "s_endpgm"])
    assert not mfma_under_exec_mask(["s_cbranch_scc1 .LBB0_4", "s_and_saveexec_b64 s[0:1], vcc",
                                     "s_cbranch_execnz .LBB0_5", "s_endpgm", ".LBB0_4:", mf,
                                     "s_endpgm", ".LBB0_5:", "v_mov_b32 v1, 0",
                                     "s_or_b64 exec, exec, s[0:1]", "s_endpgm"])
    assert not mfma_under_exec_mask(["s_and_saveexec_b64 s[0:1], vcc", "v_mov_b32 v1, 0",
                                     "s_or_b64 exec, exec, s[0:1]", mf])
    # the if/else form: the region is closed through the register the xor wrote
    ifelse = ["s_and_saveexec_b64 s[4:5], s[2:3]", "s_xor_b64 s[2:3], exec, s[4:5]",
              "s_cbranch_execz .LBB0_7", "v_mov_b32 v1, 0", ".LBB0_7:",
              "s_or_b64 exec, exec, s[2:3]"]
    assert not mfma_under_exec_mask(ifelse + [mf])
    assert mfma_under_exec_mask(ifelse[:4] + [mf] + ifelse[4:])
    # the full if/else with the else entered through s_or_saveexec into another
    # register: closed by OR-ing that register back; an MFMA in the else is masked
    full = ["s_and_saveexec_b64 s[8:9], vcc", "s_xor_b64 s[8:9], exec, s[8:9]",
            "v_mov_b32 v1, 0", "s_or_saveexec_b64 s[48:49], s[8:9]",
            "s_xor_b64 exec, exec, s[48:49]", "v_mov_b32 v2, 0", "s_or_b64 exec, exec, s[48:49]"]
    assert not mfma_under_exec_mask(full + [mf])
    assert mfma_under_exec_mask(full[:6] + [mf] + full[6:])


def test_no_mfma_under_exec_mask(isa):
    for name, lines in isa.items():
        found = mfma_under_exec_mask(lines)
        assert not found, f"{name}: MFMA inside an EXEC-masked region: {found[0]}"


def test_key_loop_does_not_spill(isa):
    for name, lines in isa.items():
        depths = [int(m.group(1)) for line in lines for m in [re.search(r"Depth=(\d+)", line)] if m]
        assert depths, f"{name}: no loop found"
        deepest = f"Depth={max(depths)}"
        in_inner = False
        for line in lines:
            if re.match(r"^\.LBB\w+:", line) or re.match(r"^; %bb\.\d+:", line):
                in_inner = deepest in line
            elif in_inner and re.search(r"\bscratch_(load|store)", line):
                raise AssertionError(f"{name}: spill in the key loop: {line.strip()}")
