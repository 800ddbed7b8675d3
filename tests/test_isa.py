"""Checks on the gfx950 machine code of the forward kernels (no GPU needed:
hipcc cross-compiles the kernels to assembly here).

- No v_mfma instruction may sit inside an EXEC-masked region (between an
  s_*_saveexec and the s_or_b64 exec that restores EXEC). Such an MFMA still
  accumulates when EXEC is zero, so a wave-uniform condition that the compiler
  could not prove uniform silently corrupts O.
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
    out = tmp_path_factory.mktemp("isa") / "fa_fwd.s"
    flags = [f for f in build.FLAGS if f not in ("-fPIC", "-shared")]
    subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out),
                    *build.SOURCES], check=True, capture_output=True)
    text = out.read_text()
    kernels = {}
    name = None
    for line in text.split("\n"):
        m = re.match(r"^(_Z\w*fa_(?:fwd|rescue)_kernel\w+):", line)
        if m:
            name = m.group(1)
            kernels[name] = []
        elif name is not None:
            kernels[name].append(line)
    return kernels


def test_all_variants_present(isa):
    assert len(isa) == 12  # head_dim x causal x {mixed plain/compensated, compensated masked, rescue}


def test_no_mfma_under_exec_mask(isa):
    # A masked region opens with s_*_saveexec_b64 sX or s_mov_b64 sX, exec
    # (the old EXEC saved in sX) and closes with s_or_b64 exec, exec, sX. Regions may be closed by
    # restoring an outer saved mask, which also closes every region opened
    # after it, so the open regions are kept as a stack of saved registers.
    for name, lines in isa.items():
        open_regions = []
        for line in lines:
            m = (re.search(r"s_(?:and|andn2|or)_saveexec_b64 (s\[\d+:\d+\])", line)
                 or re.search(r"s_mov_b64 (s\[\d+:\d+\]), exec$", line.strip()))
            c = re.search(r"s_or_b64 exec, exec, (s\[\d+:\d+\])", line)
            if m:
                open_regions.append(m.group(1))
            elif c:
                if c.group(1) in open_regions:
                    del open_regions[open_regions.index(c.group(1)):]
            elif "v_mfma" in line:
                assert not open_regions, f"{name}: MFMA inside an EXEC-masked region: {line.strip()}"


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
