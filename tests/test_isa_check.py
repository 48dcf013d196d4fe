"""The assembly checks of gqa_causal_prefill_amd.isa_check on small hand-written streams:
each rule finds the hazard it is written for and passes the same stream made safe.
(The run over the kernels themselves compiles the whole source and is not part of the
CPU suite: python -m gqa_causal_prefill_amd.isa_check.)"""

import pytest

from gqa_causal_prefill_amd import isa_check

HEAD = "_ZN12_GLOBAL__N_118gqa_prefill_kernelILb0ELb0ELi3ELb0EEEvNS_6ParamsE:\n"
TAIL = ".Lfunc_end0:\n"


def run(body):
    kernels = isa_check.parse(HEAD + body + TAIL)
    assert len(kernels) == 1
    (name, insts), = kernels.items()
    return isa_check.check(name, insts)


def test_registers():
    assert isa_check.registers("v[4:7]") == {("v", 4), ("v", 5), ("v", 6), ("v", 7)}
    assert isa_check.registers("a12,") == {("a", 12)}
    assert isa_check.registers("-v9") == {("v", 9)}
    assert isa_check.registers("s[2:3]") == set()
    assert isa_check.registers("0x3f800000") == set()


# A conversion writes a P register and an MFMA reads it as its B operand.
P_WRITE = "\tv_cvt_pk_bf16_f32 v46, v46, v58\n"
MFMA_P = "\tv_mfma_f32_16x16x32_bf16 a[120:123], v[26:29], v[46:49], a[120:123]\n"
MFMA_OTHER = "\tv_mfma_f32_16x16x32_bf16 a[184:187], v[26:29], v[38:41], a[184:187]\n"


def test_valu_then_mfma_read_is_flagged():
    assert len(run(P_WRITE + MFMA_P).violations["valu_mfma"]) == 1


def test_one_mfma_between_is_one_wait_state():
    # the case found in the library before the first MFMA on each P register carried P:
    # another step's MFMA between the conversion and the reader is only one wait state
    assert len(run(P_WRITE + MFMA_OTHER + MFMA_P).violations["valu_mfma"]) == 1


@pytest.mark.parametrize("gap", ["\ts_nop 1\n", "\ts_nop 0\n\tv_add_f32 v1, v2, v3\n",
                                 "\tv_add_f32 v1, v2, v3\n\tv_add_f32 v4, v2, v3\n"])
def test_two_wait_states_are_enough(gap):
    assert run(P_WRITE + gap + MFMA_P).ok()


def test_accumulator_operand_is_not_an_a_or_b_read():
    # a VALU write of a register the MFMA only uses as its C operand is another rule
    assert run("\tv_mov_b32 v2, 0\n\tv_mfma_f32_16x16x32_bf16 v[2:5], v[8:11], v[12:15], v[2:5]\n").ok()


READ = "\tds_read_b128 v[4:7], v1 offset:0\n"
READ2 = "\tds_read_b128 v[8:11], v1 offset:16\n"


def test_use_before_the_lds_wait_is_flagged():
    assert len(run(READ + "\tv_add_f32 v20, v5, v9\n").violations["lds_pending"]) == 1


def test_overwrite_before_the_lds_wait_is_flagged():
    assert len(run(READ + "\tv_mov_b32 v6, 0\n").violations["lds_pending"]) == 1


def test_wait_counts_in_order():
    # lgkmcnt(1): the older read is complete, the younger may not be
    assert run(READ + READ2 + "\ts_waitcnt lgkmcnt(1)\n\tv_add_f32 v20, v5, v12\n").ok()
    rep = run(READ + READ2 + "\ts_waitcnt lgkmcnt(1)\n\tv_add_f32 v20, v9, v9\n")
    assert len(rep.violations["lds_pending"]) == 1


def test_scalar_loads_share_the_counter():
    # a scalar load issued after the read keeps lgkmcnt(1) from covering the read
    body = READ + "\ts_load_dwordx2 s[4:5], s[0:1], 0x0\n\ts_waitcnt lgkmcnt(1)\n\tv_add_f32 v20, v5, v12\n"
    assert run(body).ok()
    body = "\ts_load_dwordx2 s[4:5], s[0:1], 0x0\n" + READ + "\ts_waitcnt lgkmcnt(1)\n\tv_add_f32 v20, v5, v12\n"
    assert len(run(body).violations["lds_pending"]) == 1


QK = "\tv_mfma_i32_16x16x64_i8 v[36:39], v[112:115], v[42:45], v[36:39]\n"
CARRY = "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[120:123], v[64:67], a[0:3] ; carry v37 v80\n"


def test_carrying_an_mfma_result_is_flagged():
    rep = run(QK + CARRY)
    assert len(rep.violations["carried_mfma_write"]) == 1
    assert rep.carried == 2


def test_holding_an_mfma_result_in_an_empty_statement_is_flagged():
    rep = run(QK + "\t; hold v[36:39]\n\tv_cvt_f32_i32 v40, v36\n")
    assert len(rep.violations["carried_mfma_write"]) == 4


def test_carrying_a_vector_result_is_fine():
    # once a vector instruction has rewritten the register, the MFMA is no longer its writer
    assert run(QK + "\tv_cvt_f32_i32 v37, v37\n" + CARRY).ok()
    assert run("\tv_mul_f32 v80, v55, v76\n" + CARRY).ok()
