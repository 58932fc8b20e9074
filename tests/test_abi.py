"""The C ABI boundary, checked without a GPU.

* libsa.so loads and exports every function include/sa.h declares;
* the ctypes mirrors have the C layout (a gcc-compiled probe prints sizeof /
  offsetof from the header itself);
* invalid arguments are rejected on the host with the documented status and
  a message, before anything touches a device.
"""

import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_attention_sa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsa.so is not built (run python -m block_sparse_attention_sa_amd.build)")
    L = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert _lib.lib().sa_abi_version() == _lib.ABI_VERSION


def test_struct_layout_matches_header(tmp_path):
    probe = tmp_path / "layout.c"
    fields_p = [f for f, _ in _lib.SaPattern._fields_]
    fields_a = [f for f, _ in _lib.SaAttnArgs._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){",
             'printf("P %zu\\n", sizeof(sa_pattern));', 'printf("A %zu\\n", sizeof(sa_attn_args));']
    for f in fields_p:
        lines.append(f'printf("p.{f} %zu\\n", offsetof(sa_pattern, {f}));')
    for f in fields_a:
        lines.append(f'printf("a.{f} %zu\\n", offsetof(sa_attn_args, {f}));')
    lines.append("return 0;}")
    probe.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-o", str(exe), str(probe)])
    out = dict(line.split() for line in subprocess.check_output([str(exe)], text=True).splitlines())
    assert int(out["P"]) == ctypes.sizeof(_lib.SaPattern)
    assert int(out["A"]) == ctypes.sizeof(_lib.SaAttnArgs)
    for f in fields_p:
        assert int(out[f"p.{f}"]) == getattr(_lib.SaPattern, f).offset, f
    for f in fields_a:
        assert int(out[f"a.{f}"]) == getattr(_lib.SaAttnArgs, f).offset, f


def _err():
    return _lib.lib().sa_last_error().decode()


def test_block_mask_argument_errors():
    L = _lib.lib()
    p = _lib.SaPattern(causal=1, window_left=8, window_right=0, sinks=0, unit_window=-1)
    fake = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation
    st = L.sa_build_block_mask(None, 64, 64, 64, 64, fake, fake, fake, fake, None)
    assert st == _lib.SA_ERR_INVALID_ARG and "pattern" in _err()
    st = L.sa_build_block_mask(ctypes.byref(p), 64, 64, 48, 64, fake, fake, fake, fake, None)
    assert st == _lib.SA_ERR_INVALID_ARG and "block" in _err()
    st = L.sa_build_block_mask(ctypes.byref(p), -1, 64, 64, 64, fake, fake, fake, fake, None)
    assert st == _lib.SA_ERR_INVALID_ARG
    st = L.sa_build_block_mask(ctypes.byref(p), 64, 64, 64, 64, fake, fake, fake, None, None)
    assert st == _lib.SA_ERR_INVALID_ARG and "live_pairs" in _err()
    bad = _lib.SaPattern(stride=4, stride_phase=4, unit_window=-1, window_left=-1)
    st = L.sa_build_block_mask(ctypes.byref(bad), 64, 64, 64, 64, fake, fake, fake, fake, None)
    assert st == _lib.SA_ERR_INVALID_ARG and "stride_phase" in _err()
    bad = _lib.SaPattern(unit=0, unit_window=1, window_left=-1)
    st = L.sa_build_block_mask(ctypes.byref(bad), 64, 64, 64, 64, fake, fake, fake, fake, None)
    assert st == _lib.SA_ERR_INVALID_ARG and "unit" in _err()
    bad = _lib.SaPattern(unit=64, unit_window=-1, n_rand=9, window_left=-1, rand_units=16)
    st = L.sa_build_block_mask(ctypes.byref(bad), 64, 64, 64, 64, fake, fake, fake, fake, None)
    assert st == _lib.SA_ERR_UNSUPPORTED and "n_rand" in _err()
    bad = _lib.SaPattern(q_offset=2**31, window_left=-1, unit_window=-1)
    st = L.sa_build_block_mask(ctypes.byref(bad), 64, 64, 64, 64, fake, fake, fake, fake, None)
    assert st == _lib.SA_ERR_UNSUPPORTED


def _args(**kw):
    a = _lib.SaAttnArgs()
    a.q = a.k = a.v = a.o = 4096
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = 1, 1, 64, 64, 64
    for s in (a.q_strides, a.k_strides, a.v_strides, a.o_strides):
        s[:] = [4096, 4096, 64]
    a.mode = _lib.SA_MODE_BLOCKS
    a.block_q = a.block_kv = 64
    a.kv_count = a.kv_index = a.kv_partial = 4096
    a.pattern = _lib.SaPattern(causal=1, window_left=-1, unit_window=-1)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status,word", [
    (dict(head_dim=96), _lib.SA_ERR_UNSUPPORTED, "head_dim"),
    (dict(o_dtype=7), _lib.SA_ERR_INVALID_ARG, "o_dtype"),
    (dict(mode=3), _lib.SA_ERR_INVALID_ARG, "mode"),
    (dict(q=0), _lib.SA_ERR_INVALID_ARG, "NULL"),
    (dict(k=4100), _lib.SA_ERR_INVALID_ARG, "aligned"),
    (dict(lse=4098), _lib.SA_ERR_INVALID_ARG, "lse"),
    (dict(block_q=32), _lib.SA_ERR_UNSUPPORTED, "block"),
    (dict(kv_count=0), _lib.SA_ERR_INVALID_ARG, "block lists"),
    (dict(mode=_lib.SA_MODE_GATHER, gather_idx=0), _lib.SA_ERR_INVALID_ARG, "gather_idx"),
    (dict(mode=_lib.SA_MODE_GATHER, gather_idx=4096, topk=0), _lib.SA_ERR_UNSUPPORTED, "topk"),
    (dict(batch=-1), _lib.SA_ERR_INVALID_ARG, "batch"),
])
def test_attn_argument_errors(kw, status, word):
    a = _args(**kw)
    st = _lib.lib().sa_attn_fwd(ctypes.byref(a), None)
    assert st == status
    assert word in _err()


def test_attn_stride_errors():
    a = _args()
    a.k_strides[2] = 60
    assert _lib.lib().sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG
    a = _args()
    a.q_strides[2] = 32
    assert _lib.lib().sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG


def test_attn_empty_is_ok_without_launch():
    a = _args(n_q=0)
    assert _lib.lib().sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_OK


def test_indexer_topk_argument_errors():
    L = _lib.lib()
    f = ctypes.c_void_p(4096)
    assert L.sa_indexer_scores(f, f, 4, 64, 12, 0, f, None) == _lib.SA_ERR_UNSUPPORTED
    assert L.sa_indexer_scores(f, f, 4, 64, 64, -1, f, None) == _lib.SA_ERR_INVALID_ARG
    assert L.sa_topk(f, 4, 64, 0, 0, f, None) == _lib.SA_ERR_UNSUPPORTED
    assert L.sa_topk(f, 4, 70000, 0, 16, f, None) == _lib.SA_ERR_UNSUPPORTED
    assert L.sa_topk(None, 4, 64, 0, 16, f, None) == _lib.SA_ERR_INVALID_ARG
    assert L.sa_indexer_topk(f, f, 4, 64, 64, 0, 5000, f, f, None) == _lib.SA_ERR_UNSUPPORTED
    assert L.sa_topk(f, 0, 64, 0, 16, f, None) == _lib.SA_OK  # empty: nothing launched


def test_attn_offset_range_error():
    # key tiles are addressed with 32-bit byte offsets per (batch, head)
    a = _args(n_kv=1 << 24)
    for s in (a.k_strides, a.v_strides):
        s[:] = [1 << 32, 1 << 32, 128]
    assert _lib.lib().sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_UNSUPPORTED
    assert "2^31 bytes" in _err()
    # gathered rows too
    g = _args(mode=_lib.SA_MODE_GATHER, gather_idx=4096, topk=64, n_kv=1 << 24)
    for s in (g.k_strides, g.v_strides):
        s[:] = [1 << 32, 1 << 32, 128]
    assert _lib.lib().sa_attn_fwd(ctypes.byref(g), None) == _lib.SA_ERR_UNSUPPORTED
    assert "2^31 bytes" in _err()


def test_gather_workspace_size_and_errors():
    L = _lib.lib()
    a = _args(mode=_lib.SA_MODE_GATHER, gather_idx=4096, topk=64, head_dim=128, n_kv=1000)
    for s in (a.q_strides, a.k_strides, a.v_strides, a.o_strides):
        s[:] = [1 << 24, 1 << 24, 128]
    assert L.sa_attn_workspace_bytes(ctypes.byref(a)) == 0      # one key range: no split form
    a.n_kv = 20000                                              # 5 ranges of 4096 keys
    need = L.sa_attn_workspace_bytes(ctypes.byref(a))
    rows, items, nch = 64, 64, 5
    up = lambda x: (x + 255) // 256 * 256
    exp = up(up(up(up(rows * 64 * 4) + rows * (nch + 1) * 4) + items * nch * 128 * 4) + items * nch * 2 * 4)
    assert need == exp
    a.workspace, a.workspace_bytes = 1 << 20, need - 1
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "workspace" in _err()
    a.workspace, a.workspace_bytes = (1 << 20) + 16, need
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "aligned" in _err()
    b = _args()
    assert L.sa_attn_workspace_bytes(ctypes.byref(b)) == 0      # block mode needs none


def test_merge_partial_argument_errors():
    L = _lib.lib()
    f = ctypes.c_void_p(4096)
    st3 = (ctypes.c_int64 * 3)(1 << 20, 1 << 16, 128)
    assert L.sa_merge_partial(f, f, f, f, 1, 1, 64, 96, st3, st3, 1, 0, 64, None) == _lib.SA_ERR_UNSUPPORTED
    assert "head_dim" in _err()
    assert L.sa_merge_partial(f, f, f, f, 1, 1, 64, 128, st3, st3, 0, 0, 64, None) == _lib.SA_ERR_INVALID_ARG
    assert L.sa_merge_partial(f, f, f, f, 1, 1, 64, 128, st3, st3, 16, -1, 2, None) == _lib.SA_ERR_INVALID_ARG
    # every call below fails validation before any launch (the pointers are fake)
    assert L.sa_merge_partial(f, f, f, f, 1, 1, 64, 128, st3, st3, 16, 31, 4, None) == _lib.SA_ERR_INVALID_ARG
    assert "below n" in _err()                                   # 31 + 3*16 = 79 >= 64
    assert L.sa_merge_partial(f, f, f, f, 1, 1, 64, 128, st3, st3, 16, 49, 2, None) == _lib.SA_ERR_INVALID_ARG
    assert L.sa_merge_partial(None, f, f, f, 1, 1, 64, 128, st3, st3, 16, 31, 2, None) == _lib.SA_ERR_INVALID_ARG
    assert "NULL" in _err()
    bad = (ctypes.c_int64 * 3)(1 << 20, 1 << 16, 130)          # row stride not a multiple of 4
    assert L.sa_merge_partial(f, f, f, f, 1, 1, 64, 128, st3, bad, 16, 31, 2, None) == _lib.SA_ERR_INVALID_ARG
    assert "multiples of 4" in _err()
    g = ctypes.c_void_p(4100)                                     # not 16-byte aligned
    assert L.sa_merge_partial(g, f, f, f, 1, 1, 64, 128, st3, st3, 16, 31, 2, None) == _lib.SA_ERR_INVALID_ARG
    assert "aligned" in _err()
    assert L.sa_merge_partial(None, None, None, None, 0, 1, 64, 128, None, None, 16, 31, 2, None) == _lib.SA_OK


def test_strided_form_detection():
    import block_sparse_attention_sa_amd as sa
    pat = dict(causal=1, window_left=127, window_right=0, stride=128, stride_phase=127)
    assert sa.strided_stride(pat, 16384, 16384) == 128
    assert sa.strided_stride(pat, 16384, 16000) == 0            # n_q != n_kv
    assert sa.strided_stride(pat, 16300, 16300) == 0            # not a multiple of the stride
    assert sa.strided_stride(pat, 256, 256) == 0                # fewer than three groups
    assert sa.strided_stride(dict(pat, sinks=4), 16384, 16384) == 0
    assert sa.strided_stride(dict(pat, stride_phase=3), 16384, 16384) == 0
    assert sa.strided_stride(dict(pat, window_left=64), 16384, 16384) == 0
    assert sa.strided_stride(dict(pat, causal=0), 16384, 16384) == 0


def test_plan_strided_rejects_other_patterns():
    import block_sparse_attention_sa_amd as sa
    pat = dict(causal=1, window_left=127, window_right=0, stride=128, stride_phase=127)
    for bad, n in ((dict(pat, sinks=1), 16384), (pat, 16300), (dict(causal=1, window_left=127), 16384)):
        with pytest.raises(ValueError):
            sa.plan_strided(bad, n)        # raises before any device work
