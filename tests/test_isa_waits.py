"""The compiled attention kernels leave at least 20 issue slots between every scaled FP8
matrix instruction and the first read of its result, on every control path (host-side check
of the gfx950 assembly; no GPU needed)."""
import os
import shutil

import pytest

from precision_causal_attention_token_amd import build
from tests import isa_waits

# (source, symbol pattern, instantiations: head dims 64 and 128, times causal and non-causal for
# the forward and key-tile kernels, with and without 4-bit scores (and the causal precision-option
# variants of both), times the forward's two workgroup shapes; the precision options' dQ kernel
# per head dim)
KERNELS = [("attn_fwd.hip", r"_ZN6flamia12_GLOBAL__N_110fwd_kernelI\w+", 20),
           ("attn_bwd.hip", r"_ZN6flamia12_GLOBAL__N_110bwd_kernelI\w+", 10),
           ("attn_bwd.hip", r"_ZN6flamia12_GLOBAL__N_19dq_kernelI\w+", 2),
           ("attn_dqp.hip", r"_ZN6flamia12_GLOBAL__N_110dqp_kernelI\w+", 2)]


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src,pattern,count", KERNELS)
def test_matrix_results_read_after_full_latency(tmp_path, src, pattern, count):
    asm = isa_waits.compile_to_asm(os.path.join(build.CSRC, src), str(tmp_path / (src + ".s")), build.HIPCC,
                                   build.FLAGS)
    syms = isa_waits.kernel_symbols(asm, pattern)
    assert len(syms) == count, syms
    for sym in syms:
        close, n = isa_waits.close_reads(asm, sym)
        assert n > 0, sym
        assert not close, (sym, close)


def test_checker_flags_a_short_distance():
    """The checker itself: a read after 19 slots (scalar fill) is reported, after 20 it is not,
    chained accumulation is not a read, and a branch path is followed."""
    def kern(body):
        return "k:\n" + body + "\ts_endpgm\n.Lfunc_end0:\n"
    mf = "\tv_mfma_scale_f32_32x32x64_f8f6f4 a[0:15], v[2:9], v[10:17], 0, v20, v21 op_sel_hi:[0,0,0]\n"
    read = "\tv_accvgpr_read_b32 v30, a15\n"
    salu = "\ts_add_i32 s0, s0, 1\n"
    assert isa_waits.close_reads(kern(mf + salu * 19 + read), "k")[0][0][1] == 19
    assert isa_waits.close_reads(kern(mf + salu * 20 + read), "k")[0] == []
    assert isa_waits.close_reads(kern(mf + "\ts_nop 15\n\ts_nop 3\n" + read), "k")[0] == []
    chain = "\tv_mfma_scale_f32_32x32x64_f8f6f4 a[0:15], v[2:9], v[10:17], a[0:15], v20, v21 op_sel_hi:[0,0,0]\n"
    res, n = isa_waits.close_reads(kern(mf + chain + "\ts_nop 15\n\ts_nop 3\n" + read), "k")
    assert n == 2 and res == []
    branchy = mf + "\ts_cbranch_scc1 .LBB0_1\n" + "\ts_nop 15\n\ts_nop 7\n" + ".LBB0_1:\n" + read
    res, _ = isa_waits.close_reads(kern(branchy), "k")
    assert [r[1] for r in res] == [1]


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("src,pattern,count", KERNELS)
def test_m0_only_in_direct_load_sequences(tmp_path, src, pattern, count):
    """M0 is written only by the direct-load sequence, which always writes it right before its
    load: no compiler-placed M0 value can be live across it."""
    asm = isa_waits.compile_to_asm(os.path.join(build.CSRC, src), str(tmp_path / (src + ".s")), build.HIPCC,
                                   build.FLAGS)
    for sym in isa_waits.kernel_symbols(asm, pattern):
        assert isa_waits.stray_m0_uses(asm, sym) == [], sym


def test_m0_checker_flags_a_stray_use():
    k = lambda body: "k:\n" + body + "\ts_endpgm\n.Lfunc_end0:\n"
    good = "\ts_mov_b32 m0, s4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v[0:1], off\n"
    assert isa_waits.stray_m0_uses(k(good), "k") == []
    assert isa_waits.stray_m0_uses(k("\ts_mov_b32 m0, s5\n" + good), "k") != []
    assert isa_waits.stray_m0_uses(k("\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v[0:1], off\n"), "k") != []
