"""No instruction of any kernel touches a register whose LDS or global load is still in flight.

Many LDS operand reads are written in inline assembly and waited for by explicit ``s_waitcnt`` in
later statements; the compiler does not know that their destinations are written late, so only
its assembly shows whether it copied or reused one too early (tests/_isa_loads.py).  The first
tests pin the checker on small hand-written sequences (each with the mistake it must catch or the
pattern it must accept); the last compiles the library's sources for gfx950 with the library's
own flags and checks every kernel.  CPU only: hipcc cross-compiles.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests import _isa_loads as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def issues(text: str):
    return I.check_function([l for l in text.strip().split("\n")])


def test_read_before_wait_is_caught():
    assert issues("""
        ds_read_b128 v[0:3], v10
        v_add_f32_e32 v5, v0, v1
    """)


def test_wait_covers_the_read():
    assert not issues("""
        ds_read_b128 v[0:3], v10
        s_waitcnt lgkmcnt(0)
        v_add_f32_e32 v5, v0, v1
    """)


def test_partial_wait_covers_only_the_older_reads():
    seq = """
        ds_read_b128 v[0:3], v10
        ds_read_b128 v[4:7], v11
        s_waitcnt lgkmcnt(1)
        v_add_f32_e32 v20, v{r}, v1
    """
    assert not issues(seq.format(r=2))
    assert issues(seq.format(r=5))


def test_copy_to_agpr_before_wait_is_caught():
    # what a register allocator that moves an operand to another register class would emit
    assert issues("""
        ds_read_b64_tr_b16 v[148:149], v254 offset:0x4100
        v_accvgpr_write_b32 a6, v148
        s_waitcnt lgkmcnt(0)
    """)


def test_overwrite_before_wait_is_caught():
    assert issues("""
        ds_read_b128 v[0:3], v10
        v_mov_b32_e32 v2, 0
        s_waitcnt lgkmcnt(0)
    """)


def test_mfma_reading_pending_operand_is_caught():
    assert issues("""
        ds_read_b128 v[32:35], v84 offset:0
        v_mfma_f32_32x32x16_bf16 a[0:15], v[32:35], v[228:231], a[0:15]
    """)


def test_same_counter_reload_is_in_order():
    # a ring slot read again while its previous read is in flight: LDS returns in order
    assert not issues("""
        ds_read_b128 v[0:3], v10
        ds_read_b128 v[0:3], v11
        s_waitcnt lgkmcnt(0)
        v_add_f32_e32 v5, v0, v1
    """)


def test_cross_counter_overwrite_is_caught():
    assert issues("""
        global_load_dwordx4 v[0:3], v[8:9], off
        ds_read_b128 v[0:3], v10
        s_waitcnt vmcnt(0) lgkmcnt(0)
    """)


def test_direct_to_lds_load_has_no_register_destination():
    assert not issues("""
        global_load_lds_dwordx4 v[8:9], off
        v_add_u32_e32 v8, 16, v8
        v_mov_b32_e32 v0, v9
    """)


def test_path_that_skips_the_wait_is_caught():
    assert issues("""
        ds_read_b32 v0, v10
        s_cbranch_scc1 .LBB0_2
        s_waitcnt lgkmcnt(0)
    .LBB0_2:
        v_add_f32_e32 v5, v0, v1
        s_endpgm
    """)


def test_loop_carried_read_is_caught():
    # the read issued at the end of one iteration is used at the top of the next without a wait
    assert issues("""
        s_waitcnt lgkmcnt(0)
    .LBB0_1:
        v_add_f32_e32 v5, v0, v1
        ds_read_b32 v0, v10
        s_cbranch_scc1 .LBB0_1
        s_waitcnt lgkmcnt(0)
        s_endpgm
    """)


def test_loop_carried_read_with_wait_at_the_top_is_accepted():
    assert not issues("""
        ds_read_b32 v0, v10
    .LBB0_1:
        s_waitcnt lgkmcnt(0)
        v_add_f32_e32 v5, v0, v1
        ds_read_b32 v0, v10
        s_cbranch_scc1 .LBB0_1
        s_waitcnt lgkmcnt(0)
        s_endpgm
    """)


def _device_asm(src: str, out_dir: str) -> str:
    sys.path.insert(0, ROOT)
    from attention_forward_flashattention_amd import build as B

    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    subprocess.check_call([B.hipcc(), *B.HIPCC_FLAGS, "-I", B.INCLUDE, "--cuda-device-only", "-S", src, "-o", out],
                          stderr=subprocess.DEVNULL)
    return out


@pytest.mark.slow
def test_no_kernel_touches_a_register_in_flight():
    from attention_forward_flashattention_amd import build as B

    if not os.path.exists(B.hipcc()):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=len(B.SRCS)) as ex:
            asm = list(ex.map(lambda s: _device_asm(s, d), B.SRCS))
        n_kernels = n_asm_reads = 0
        found = {}
        for path in asm:
            text = open(path).read()
            for name, lines in I.functions(text).items():
                n_kernels += 1
                n_asm_reads += sum(1 for l in lines if "ds_read_b64_tr_b16" in l)
                bad = I.check_function(lines)
                if bad:
                    found[name] = bad[:3]
    # the check is not vacuous: every kernel source was parsed and the transpose reads were seen
    assert n_kernels >= 60 and n_asm_reads > 1000, (n_kernels, n_asm_reads)
    assert not found, found
