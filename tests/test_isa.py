"""Checks on the gfx950 ISA of the attention kernels (CPU only: hipcc cross-compiles).

The d = 128 forward kernels and the backward kernels copy tiles with LDS-DMA
instructions written as inline assembly that set M0 themselves.  The compiler treats M0 as reserved and does
not save it around inline assembly, so the kernels are only correct while
nothing else in them reads or writes M0: every M0 write must be one of those
copies (``s_mov_b32 m0, sN`` directly followed by the buffer load to LDS).
The kernels must also keep every value in registers (no scratch).
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from tiled_attention_13_amd import build as fa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", params=["fa_fwd.hip", "fa_bwd.hip"])
def isa(request, tmp_path_factory):
    try:
        cc = fa_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / (request.param + ".s")
    flags = [f for f in fa_build.HIP_FLAGS if f != "-fPIC"]
    cmd = [cc, *flags, "--cuda-device-only", "-S", "-I", fa_build.INCLUDE, "-I", fa_build.CSRC,
           os.path.join(fa_build.CSRC, request.param), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().splitlines()


def test_m0_only_set_by_tile_copies(isa):
    """Every M0 write is `s_mov_b32 m0, sN` or `s_add_u32 m0, sN, imm`, followed by
    the LDS-DMA load (with an optional `s_mov_b32 sK, imm` for its scalar offset)."""
    lines = [l.strip() for l in isa]
    copies = 0
    for i, l in enumerate(lines):
        if l.startswith(";") or not re.search(r"\bm0\b", l):
            continue
        assert re.match(r"(s_mov_b32 m0, s\d+|s_add_u32 m0, s\d+, (0x[0-9a-f]+|\d+))$", l), \
            f"M0 used outside a tile copy: {l}"
        nxt = lines[i + 1]
        so = re.match(r"s_mov_b32 (s\d+), (0x[0-9a-f]+|\d+)$", nxt)
        if so:
            nxt = lines[i + 2]
            assert re.match(rf"buffer_load_dwordx4 v\d+, s\[\d+:\d+\], {so.group(1)} offen lds$", nxt), \
                f"M0 write not followed by an LDS-DMA load: {l} / {lines[i + 1]} / {nxt}"
        else:
            assert re.match(r"buffer_load_dwordx4 v\d+, s\[\d+:\d+\], 0 offen lds$", nxt), \
                f"M0 write not followed by an LDS-DMA load: {l} / {nxt}"
        copies += 1
    assert copies > 0, "no LDS-DMA tile copies found"


def test_attention_kernels_use_no_scratch(isa):
    sizes = {}
    for l in isa:
        m = re.match(r"\s*\.set (_ZN\S*(?:fwd_pp_kernel|bwd_kv_kernel|bwd_dq_kernel)\S*)\.private_seg_size, (\d+)", l)
        if m:
            sizes[m.group(1)] = int(m.group(2))
    assert sizes, "no attention kernel instances found"
    spilled = {k: v for k, v in sizes.items() if v}
    assert not spilled, f"scratch in {spilled}"
