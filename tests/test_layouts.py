"""The LDS tile layouts of fa_common.h, checked on the host (no GPU needed):
tests/layout_check.hip includes the header, builds as a host program and
checks, for every row width the kernels use (64, 80, 96, 128, 192, 256), that
each K and V layout is a bijection between (row, 16-byte chunk) and the
tile's slots, that the copy's inverse agrees with it, and that the per-lane
piece addresses of the forward kernel's reads agree with the layout. It also
reports a bank model's worst case per access pattern (64 four-byte banks;
ds_read_b128 served 8 lanes at a time, 64-bit reads 32 lanes at a time); the
layouts of 64, 128 and 256, measured conflict-free on the hardware, come out
conflict-free in it, and the panel layouts of 80, 96 and 192 were designed to.
"""
import os
import re
import subprocess

from flash_attention_forward_fa_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_layouts(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.run([build.HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
                    "-I" + os.path.join(build.ROOT, "include"),
                    "-I" + os.path.join(build.HERE, "csrc"), "-o", str(exe),
                    os.path.join(HERE, "layout_check.hip")], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip().endswith("ok"), out.stdout
    widths = set()
    for m in re.finditer(r"model W=(\d+) k_b128=(\d+) k_tail=(\d+) v_tr=(\d+)", out.stdout):
        widths.add(int(m.group(1)))
        assert m.groups()[1:] == ("1", "1", "1"), m.group(0)
    assert widths == {64, 80, 96, 128, 192, 256}
