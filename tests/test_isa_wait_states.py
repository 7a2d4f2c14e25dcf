"""The library's inline-asm buffer instructions carry the wait states the hardware requires
after a VALU write of their SGPR operands and after an m0 write (checked on the gfx950
assembly of every source, compiled with the library's own flags; no GPU needed)."""

import concurrent.futures as cf
import glob
import os
import subprocess
import tempfile

import pytest

from fp8_block_scaled_quant_amd import build as B
from isa_scan import scan

_PLANTED = """_Zk:
	v_readfirstlane_b32 s40, v98
	;;#ASMSTART
	buffer_load_dwordx4 v[34:37], v38, s[40:43], 0 offen
	;;#ASMEND
	s_mov_b32 s20, 0
	;;#ASMSTART
	s_mov_b32 m0, s21
	buffer_load_dword v1, s[8:11], 0 offen lds
	;;#ASMEND
	s_endpgm
"""

_PADDED = """_Zk:
	v_readfirstlane_b32 s40, v98
	;;#ASMSTART
	s_nop 4
	buffer_load_dwordx4 v[34:37], v38, s[40:43], 0 offen
	;;#ASMEND
	;;#ASMSTART
	s_mov_b32 m0, s21
	s_nop 4
	buffer_load_dword v1, s[8:11], 0 offen lds
	;;#ASMEND
	s_endpgm
"""


def test_scan_finds_planted_hazards():
    found = scan(_PLANTED)
    assert len(found) == 2, found
    assert "0 wait states after a VALU write" in found[0]
    assert "m0 write" in found[1]
    assert scan(_PADDED) == []


def _device_asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *[f for f in B.CFLAGS if f != "-Wall"], "--offload-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr[-2000:]}")
    with open(out) as f:
        return f.read()


def test_library_asm_wait_states():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
    with tempfile.TemporaryDirectory() as d, cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        texts = list(ex.map(lambda s: _device_asm(s, d), srcs))
    problems = [f"{os.path.basename(s)}: {p}" for s, t in zip(srcs, texts) for p in scan(t)]
    assert not problems, f"{len(problems)} hazards, first: {problems[:3]}"
