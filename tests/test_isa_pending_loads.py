"""The decode kernel's weight loads are inline assembly waited for explicitly: no compiled
instruction may name a weight register between its load and the wait that covers it (no
read, copy, spill or reuse). Checked on the gfx950 assembly of every library source,
compiled with the library's own flags (no GPU needed), after the scanner itself is shown to
find planted cases."""

import concurrent.futures as cf
import glob
import os
import tempfile

import pytest

from fp8_block_scaled_quant_amd import build as B
from isa_pending import scan
from test_isa_wait_states import _device_asm

_HEAD = "_Zk:\n"


def _fn(body):
    return _HEAD + body + "\ts_endpgm\n"


_LOAD = "\t;;#ASMSTART\n\tbuffer_load_dwordx4 v[4:7], v1, s[8:11], 0 offen\n\t;;#ASMEND\n"
_OTHER = "\t;;#ASMSTART\n\tbuffer_load_dwordx4 v[8:11], v1, s[8:11], 0 offen\n\t;;#ASMEND\n"


def test_waited_use_is_clean():
    assert scan(_fn(_LOAD + _OTHER + "\ts_waitcnt vmcnt(1)\n\tv_mov_b32 v20, v4\n")) == []


def test_use_before_wait_is_found():
    assert len(scan(_fn(_LOAD + _OTHER + "\ts_waitcnt vmcnt(2)\n\tv_mov_b32 v20, v5\n"))) == 1


def test_overwrite_and_spill_are_found():
    found = scan(_fn(_LOAD + "\tv_mov_b32 v6, 0\n\tscratch_store_dwordx4 off, v[4:7], off\n\ts_waitcnt vmcnt(0)\n"))
    assert len(found) == 2, found


def test_wait_on_one_branch_only_is_found():
    body = (_LOAD + "\ts_cbranch_scc1 .LBB0_2\n\ts_waitcnt vmcnt(0)\n.LBB0_2:\n\tv_add_f32_e32 v20, v4, v4\n")
    assert len(scan(_fn(body))) == 1
    both = (_LOAD + "\ts_cbranch_scc1 .LBB0_2\n\ts_waitcnt vmcnt(0)\n\ts_branch .LBB0_3\n.LBB0_2:\n"
            "\ts_waitcnt vmcnt(0)\n.LBB0_3:\n\tv_add_f32_e32 v20, v4, v4\n")
    assert scan(_fn(both)) == []


def test_conditional_operation_does_not_count():
    # the copy after the load may be skipped, so vmcnt(1) does not cover the load on that path
    body = (_LOAD + "\ts_cbranch_scc1 .LBB0_2\n\tbuffer_load_dword v30, s[8:11], 0 offen lds\n.LBB0_2:\n"
            "\ts_waitcnt vmcnt(1)\n\tv_mov_b32 v20, v4\n")
    assert len(scan(_fn(body))) == 1


def test_loop_carried_load_is_followed():
    # loaded at the bottom of the loop, used at the top of the next iteration with the
    # wait in between, and after the loop past a vmcnt(0)
    body = (".LBB0_1:\n\ts_waitcnt vmcnt(0)\n\tv_mov_b32 v20, v4\n" + _LOAD +
            "\ts_cbranch_scc1 .LBB0_1\n\ts_waitcnt vmcnt(0)\n\tv_mov_b32 v21, v4\n")
    assert scan(_fn(body)) == []
    early = (".LBB0_1:\n\tv_mov_b32 v20, v4\n\ts_waitcnt vmcnt(0)\n" + _LOAD + "\ts_cbranch_scc1 .LBB0_1\n")
    assert len(scan(_fn(early))) == 1


def test_library_weight_registers_untouched_until_waited():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    srcs = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
    with tempfile.TemporaryDirectory() as d, cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        texts = list(ex.map(lambda s: _device_asm(s, d), srcs))
    assert any("k_gemm_decode" in t and "offen offset:" in t for t in texts), "decode kernel not found"
    problems = [f"{os.path.basename(s)}: {p}" for s, t in zip(srcs, texts) for p in scan(t)]
    assert not problems, f"{len(problems)} early accesses, first: {problems[:3]}"
