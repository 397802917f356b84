"""The C-ABI library loads and exports every entry point declared in include/flamia.h, and
its host-side argument checks return the documented statuses.  No kernel is launched."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np

import pytest

import precision_causal_attention_token_amd as fl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "flamia.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flamia_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fl.LIB_PATH):
        pytest.fail("libflamia.so is not built; run __graft_entry__.build()")
    return fl.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) >= {"flamia_quantize", "flamia_fwd", "flamia_bwd", "flamia_build_worklist"}
    for nm in names:
        assert hasattr(lib, nm), nm
    assert set(fl.EXPORTED_SYMBOLS) <= set(names)


def test_status_strings(lib):
    for s, txt in ((0, b"ok"), (1, b"null pointer"), (4, b"buffer too small")):
        assert lib.flamia_status_str(s) == txt


def test_size_queries(lib):
    assert lib.flamia_worklist_bytes(3, 1000, 0) == 16 + 16 * (8 + 3) + 64   # header, items, forward counters
    assert lib.flamia_worklist_bytes(-1, 10, 0) == 0
    T, Hq, d = 1000, 4, 64
    blk = 8192 + 128
    # the smallest workspace depends on the sizes only: tables plus twice the largest key tile
    lo = lib.flamia_bwd_workspace_bytes(4, T, Hq, d, 0)
    assert lo >= 256 + T * Hq * 2 + 2 * ((T + 63) // 64) * Hq * blk
    assert lib.flamia_bwd_workspace_bytes(4, T, Hq, d, 10 * Hq * blk) == lo           # clamped up
    mid = lib.flamia_bwd_workspace_bytes(4, T, Hq, d, 100 * Hq * blk)
    assert mid - lo == (100 - 2 * 16) * Hq * blk                                      # budget honoured
    hi = lib.flamia_bwd_workspace_bytes(4, T, Hq, d, 1 << 40)
    worst_nc = (T * T) // 8192 + 5 * T // 64 + 3 + (T + 63) // 64           # one chunk, non-causal bound
    assert hi - lo == (worst_nc - 2 * 16) * Hq * blk                                  # clamped down
    assert lib.flamia_bwd_workspace_bytes(4, T, Hq, 96, 0) == 0                       # bad d
    # one chunk for known lengths: the call's stored blocks plus the largest key tile
    cu = np.array([0, 100, 100, 612, 1000], np.int32)       # lengths 100, 0, 512, 388
    blocks = 0 + 0 + (4 * 8 - 4 * 3) + (4 * 7 - 4 * 3)     # n_kt n_qt - n_kt (n_kt - 1), 1-tile docs: 0
    got = lib.flamia_bwd_workspace_bytes_for(cu.ctypes.data_as(ctypes.c_void_p), 4, T, Hq, d, 0)
    assert got - (lo - 2 * 16 * Hq * blk) == (blocks + 16) * Hq * blk
    blocks_nc = 0 + 0 + 4 * 8 + 4 * 7                        # non-causal: every (query tile, key tile) pair
    got_nc = lib.flamia_bwd_workspace_bytes_for(cu.ctypes.data_as(ctypes.c_void_p), 4, T, Hq, d, 1)
    assert got_nc - (lo - 2 * 16 * Hq * blk) == (blocks_nc + 16) * Hq * blk
    assert lib.flamia_bwd_workspace_bytes_for(None, 3, T, Hq, d, 0) == 0               # host lengths required
    assert fl.bwd_workspace_bytes_for(cu, T, Hq, d) == got
    assert fl.bwd_workspace_bytes_for(cu, T, Hq, d, causal=False) == got_nc
    assert fl.bwd_workspace_bytes(4, T, Hq, d, 0) == lo


def test_host_validation_errors(lib):
    # null argument blocks
    assert lib.flamia_fwd(None, None) == 1
    assert lib.flamia_bwd(None, None) == 1
    assert lib.flamia_build_worklist(None, 1, 10, 0, 4, None, 0, None) == 1
    # unsupported head dim / head ratio and small buffers are rejected before any launch
    fake = 1 << 20  # never dereferenced: validation fails first
    a = fl._FwdArgs(fake, fake, fake, fake, fake, fake, 100, 4, 3, 128, 0.0, fake, 1, fake, fake, 512, 128, fake)
    assert lib.flamia_fwd(ctypes.byref(a), None) == 3          # Hq % Hkv != 0
    a.Hkv, a.d = 2, 96
    assert lib.flamia_fwd(ctypes.byref(a), None) == 3          # d not in {64, 128}
    a.d, a.o_stride_t = 128, 3
    assert lib.flamia_fwd(ctypes.byref(a), None) == 2          # misaligned output stride
    assert lib.flamia_build_worklist(fake, 1, 1000, 0, 4, fake, 16, None) == 4
    assert lib.flamia_build_worklist(fake, 1, 1 << 21, 0, 4, fake, 1 << 30, None) == 3
    b = fl._BwdArgs()
    for f, _ in fl._BwdArgs._fields_:
        if f in ("q", "k", "v", "dO", "sq", "sk", "sv", "sdO", "lse", "D", "cu_seqlens", "fwd_list", "bwd_list",
                 "dq", "dk", "dv", "workspace"):
            setattr(b, f, fake)
    b.T, b.Hq, b.Hkv, b.d, b.n_docs = 100, 4, 2, 64, 1
    b.workspace_bytes = 16
    assert lib.flamia_bwd(ctypes.byref(b), None) == 4          # workspace too small
    b.workspace_bytes = lib.flamia_bwd_workspace_bytes(1, 100, 4, 64, 0) - 1
    assert lib.flamia_bwd(ctypes.byref(b), None) == 4          # one byte short of the smallest
    b.workspace_bytes = lib.flamia_bwd_workspace_bytes(1, 100, 4, 64, 0)
    b.non_causal, b.causal_dq_scale = 1, 1
    assert lib.flamia_bwd(ctypes.byref(b), None) == 3          # causal dQ prescale needs causal attention
    b.non_causal, b.causal_dq_scale, b.hadamard = 0, 0, 1
    b.dq_stride_t, b.dq_stride_h = 4 * 64 + 4, 64               # 8-byte aligned, not a multiple of 8 elements
    b.dk_stride_t, b.dk_stride_h, b.dv_stride_t, b.dv_stride_h = 128, 64, 128, 64
    assert lib.flamia_bwd(ctypes.byref(b), None) == 2          # the un-rotation needs 16-byte rows
    b.hadamard, b.non_causal, b.precise = 0, 1, 1
    assert lib.flamia_bwd(ctypes.byref(b), None) == 3          # the precision options are causal
    # the dO pass is never rotated
    t = (fl._QTensor * 1)()
    t[0] = fl._QTensor(fake, 512, 128, 4, fake, fake, 1)
    assert lib.flamia_quantize(t, 1, 100, 128, fake, 1, fake, 512, 128, fake, None) == 3


def test_list_kinds(lib):
    fake = 1 << 20
    for kind in (0, 1, 2, 3):      # causal and non-causal forward / backward lists
        assert lib.flamia_build_worklist(fake, 1, 1000, kind, 4, fake, 16, None) == 4
    assert lib.flamia_build_worklist(fake, 1, 1000, 4, 4, fake, 1 << 20, None) == 2   # unknown kind
    assert lib.flamia_status_str(6) == b"call too large for the static scratch"


@pytest.mark.skipif(not shutil.which("gcc"), reason="gcc not installed")
def test_binding_structs_match_the_header(tmp_path):
    """Every argument struct of the Python binding has the C header's layout: the same size and,
    field by field, the same offsets (the header compiled by gcc, offsetof printed)."""
    structs = {"flamia_qtensor": fl._QTensor, "flamia_fwd_args": fl._FwdArgs, "flamia_bwd_args": fl._BwdArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "flamia.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append('  printf("%s sizeof %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('  printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[cname + " sizeof"]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(got["%s %s" % (cname, f)]) == getattr(py, f).offset, (cname, f)
