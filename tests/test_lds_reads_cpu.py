"""The compiled DMA kernels never touch a register an LDS read in flight will
still write (see tests/lds_read_check.py), checked on the device assembly the
build writes; the check itself is pinned on hand-written snippets."""
import os

import pytest

from invariant_matmul_amd import build
from tests.lds_read_check import file_hazards, kernel_hazards


def test_built_dma_kernels_have_no_in_flight_read_hazard():
    if not os.path.exists(build.DMA_ASM):
        pytest.skip("device assembly not built (run invariant_matmul_amd.build)")
    with open(build.DMA_ASM) as f:
        hazards, n = file_hazards(f.read())
    assert n > 100, n
    assert not hazards, {k[:90]: list(v.items())[:3] for k, v in list(hazards.items())[:5]}


SAFE = """
  ds_read_b128 v[0:3], v10 offset:0
  v_add_u32_e32 v11, 4, v12
  s_waitcnt lgkmcnt(0)
  v_mov_b32_e32 v1, v0
  s_endpgm
"""
# the data of the read lands after v2 was written for another purpose
WRITE_BEFORE_WAIT = """
  ds_read_b128 v[0:3], v10 offset:0
  v_mov_b32_e32 v2, 0
  s_waitcnt lgkmcnt(0)
  s_endpgm
"""
# after lgkmcnt(1) the older of two reads has landed (in-order completion):
# using its result is fine, using the newer one's is not
IN_ORDER = """
  ds_read_b64 v[0:1], v10
  ds_read_b64 v[2:3], v10 offset:8
  s_waitcnt lgkmcnt(1)
  v_add_u32_e32 v4, v0, v1
  v_add_u32_e32 v5, v2, v4
  s_waitcnt lgkmcnt(0)
  s_endpgm
"""
# a wait on one side of a branch only: the fall-through path is a hazard
ONE_SIDED = """
  ds_read_b64 v[0:1], v10
  s_cbranch_scc1 .LBB0_2
  s_waitcnt lgkmcnt(0)
.LBB0_2:
  v_mov_b32_e32 v0, 1
  s_endpgm
"""
# a later read into the same registers lands later: not a hazard; its
# address register being a pending destination is
REREAD = """
  ds_read_b64 v[0:1], v10
  ds_read_b64 v[0:1], v11
  ds_read_b64 v[4:5], v1
  s_waitcnt lgkmcnt(0)
  s_endpgm
"""
# a loop whose body reads for the next iteration and waits at its head
LOOP_OK = """
.LBB0_1:
  s_waitcnt lgkmcnt(0)
  v_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]
  ds_read_b128 v[0:3], v10
  s_cbranch_scc0 .LBB0_1
  s_waitcnt lgkmcnt(0)
  v_mov_b32_e32 v0, 0
  s_endpgm
"""
LOOP_EXIT_BAD = """
.LBB0_1:
  s_waitcnt lgkmcnt(0)
  v_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]
  ds_read_b128 v[0:3], v10
  s_cbranch_scc0 .LBB0_1
  v_accvgpr_read_b32 v2, a2
  s_waitcnt lgkmcnt(0)
  s_endpgm
"""


def _h(text):
    return kernel_hazards(text.strip().split("\n"))


def test_checker_pins():
    assert _h(SAFE) == {}
    assert list(_h(WRITE_BEFORE_WAIT)) == ["v_mov_b32_e32 v2, 0"]
    assert list(_h(IN_ORDER)) == ["v_add_u32_e32 v5, v2, v4"]
    assert list(_h(ONE_SIDED)) == ["v_mov_b32_e32 v0, 1"]
    assert list(_h(REREAD)) == ["ds_read_b64 v[4:5], v1"]
    assert _h(LOOP_OK) == {}
    assert list(_h(LOOP_EXIT_BAD)) == ["v_accvgpr_read_b32 v2, a2"]
