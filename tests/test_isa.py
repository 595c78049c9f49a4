"""CPU checks on the compiled gfx950 kernels: no scratch or spills, no use of
a register before the load that writes it has been waited for, and the
balanced GEMV's slot fold shifts every accumulator element."""

import os
import subprocess
from pathlib import Path

import pytest

from isa_check import kernels, load_hazards, metadata

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "bit_block_quantized_q4_amd" / "csrc"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asm(src, extra=()):
    from bit_block_quantized_q4_amd.build import COMMON_FLAGS, PER_FILE_FLAGS
    cmd = [HIPCC, *COMMON_FLAGS, *PER_FILE_FLAGS.get(src, []), *extra, "--cuda-device-only",
           "-S", str(CSRC / src), "-o", "-"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stdout


_CACHE = {}


def asm(src):
    if src not in _CACHE:
        _CACHE[src] = _asm(src)
    return _CACHE[src]


pytestmark = pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not available")


@pytest.mark.parametrize("src", sorted(p.name for p in CSRC.glob("*.hip")))
def test_no_scratch_or_spills(src):
    meta = metadata(asm(src))
    if src == "q4_api.hip":  # host code only
        assert not meta
        return
    assert meta, "no kernels found"
    for name, m in meta.items():
        assert m["private_segment_fixed_size"] == 0, name
        assert m["vgpr_spill_count"] == 0, name


@pytest.mark.parametrize("src,pattern", [("q4_gemv.hip", "gemv_bal_kernel"),
                                         ("q4_gemv_tile.hip", "gemv_tile")])
def test_dynamic_lds_kernels_have_no_static_lds(src, pattern):
    """The decode kernels launch with all 160 KB of a CU's LDS as dynamic
    shared memory, so any static LDS (for example the reduction buffer behind
    __syncthreads_or) would make every such launch invalid."""
    meta = metadata(asm(src))
    names = [nm for nm in meta if pattern in nm]
    assert names, pattern
    for nm in names:
        assert meta[nm]["group_segment_fixed_size"] == 0, nm


@pytest.mark.parametrize("src,pattern", [("q4_gemm.hip", "gemm_mfma_kernel"),
                                         ("q4_gemv.hip", "gemv_bal_kernel"),
                                         ("q4_gemv.hip", "gemv_stream_kernel"),
                                         ("q4_gemv_tile.hip", "gemv_tile")])
def test_no_register_used_before_its_load_lands(src, pattern):
    ks = kernels(asm(src), pattern)
    assert ks, pattern
    for name, body in ks:
        assert load_hazards(body) == [], name


def test_balanced_fold_shifts_every_element():
    """Two row shifts (8, then 4) of every accumulated activation row per fold:
    the kernel instantiated for MR rows shifts a multiple of MR values."""
    import re
    seen = set()
    for name, body in kernels(asm("q4_gemv.hip"), "gemv_bal_kernel"):
        mr = int(re.search(r"gemv_bal_kernelILi\d+ELi\d+ELi(\d+)E", name).group(1))
        seen.add(mr)
        text = "\n".join(body)
        n8 = text.count("row_shr:8")
        n4 = text.count("row_shr:4")
        assert n8 > 0 and n8 % mr == 0 and n4 == n8, (name, n8, n4)
        if mr > 1:  # distinct source registers for the first fold's shifts
            lines = [ln.split("row_shr")[0] for ln in text.splitlines() if "row_shr:8" in ln][:mr]
            assert len(set(lines)) == mr, lines
    assert seen == {1, 2, 4}


def test_checker_flags_a_planted_early_read():
    body = ["global_load_dword v4, v[0:1], off", "v_add_u32_e32 v5, v4, v6", "s_endpgm"]
    assert load_hazards(body)
    ok = ["global_load_dword v4, v[0:1], off", "s_waitcnt vmcnt(0)", "v_add_u32_e32 v5, v4, v6",
          "s_endpgm"]
    assert load_hazards(ok) == []
