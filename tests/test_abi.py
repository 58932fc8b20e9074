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
    fields_s = [f for f, _ in _lib.SaSelectArgs._fields_]
    fields_b = [f for f, _ in _lib.SaAttnBwdArgs._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){",
             'printf("P %zu\\n", sizeof(sa_pattern));', 'printf("A %zu\\n", sizeof(sa_attn_args));',
             'printf("S %zu\\n", sizeof(sa_select_args));', 'printf("B %zu\\n", sizeof(sa_attn_bwd_args));']
    for f in fields_b:
        lines.append(f'printf("b.{f} %zu\\n", offsetof(sa_attn_bwd_args, {f}));')
    for f in fields_s:
        lines.append(f'printf("s.{f} %zu\\n", offsetof(sa_select_args, {f}));')
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
    for f in fields_s:
        assert int(out[f"s.{f}"]) == getattr(_lib.SaSelectArgs, f).offset, f
    assert int(out["S"]) == ctypes.sizeof(_lib.SaSelectArgs)
    for f in fields_b:
        assert int(out[f"b.{f}"]) == getattr(_lib.SaAttnBwdArgs, f).offset, f
    assert int(out["B"]) == ctypes.sizeof(_lib.SaAttnBwdArgs)


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
    assert L.sa_indexer_topk(f, f, 4, 64, 64, 0, 5000, f, f, None, 0, None) == _lib.SA_ERR_UNSUPPORTED
    assert L.sa_topk(f, 0, 64, 0, 16, f, None) == _lib.SA_OK  # empty: nothing launched
    # streaming form (scores_out NULL): the workspace is checked before any launch
    need = L.sa_indexer_topk_workspace(4, 64, 16)
    assert need > 0
    assert L.sa_indexer_topk(f, f, 4, 64, 64, 0, 16, None, f, None, 0, None) == _lib.SA_ERR_INVALID_ARG
    assert "workspace" in _err()
    assert L.sa_indexer_topk(f, f, 4, 64, 64, 0, 16, None, f, f, need - 1, None) == _lib.SA_ERR_INVALID_ARG
    assert L.sa_indexer_topk(f, f, 4, 64, 64, 0, 16, None, f, ctypes.c_void_p(4096 + 16), need,
                             None) == _lib.SA_ERR_INVALID_ARG
    assert "aligned" in _err()
    assert L.sa_indexer_topk(f, f, 4, 70000, 64, 0, 16, None, f, f, need, None) == _lib.SA_ERR_UNSUPPORTED
    assert L.sa_indexer_topk(f, f, 4, 64, 64, 0, 16, None, None, f, need, None) == _lib.SA_ERR_INVALID_ARG
    assert L.sa_indexer_topk(f, f, 0, 64, 64, 0, 16, None, None, None, 0, None) == _lib.SA_OK


def test_indexer_topk_workspace_sizes():
    """The streaming scratch: per row a 1/32 sample (64 keys of every 2,048), a
    threshold, one largest key norm per 64-key tile, and per 512-key chunk two
    counts and 72 kept 4-byte slots (approximate score, 9-bit position);
    each array 256-byte aligned."""
    L = _lib.lib()
    up = lambda x: (x + 255) // 256 * 256

    def expect(n_q, n_kv):
        s_max = 64 * -(-n_kv // 2048)
        reg = n_q * -(-n_kv // 512)
        return up(up(up(up(up(n_q * s_max * 4) + n_q * 4) + reg * 2 * 4) + -(-n_kv // 64) * 4) + reg * 72 * 4)

    for n_q, n_kv in ((1024, 65536), (1, 1), (77, 5000), (3, 65535)):
        assert L.sa_indexer_topk_workspace(n_q, n_kv, 2048) == expect(n_q, n_kv)
    assert L.sa_indexer_topk_workspace(1024, 65536, 2048) < 64 << 20
    assert L.sa_indexer_topk_workspace(0, 100, 16) == 0
    assert L.sa_indexer_topk_workspace(4, 65537, 16) == 0
    assert L.sa_indexer_topk_workspace(4, 100, 0) == 0
    assert L.sa_indexer_topk_workspace(4, 100, 4097) == 0


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
    a.n_kv = 40000                                              # 5 ranges of 8192 keys
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
    assert L.sa_attn_workspace_bytes(ctypes.byref(b)) == 0      # causal block mode needs none


def test_block_long_row_split_workspace_size_and_errors():
    """Block mode without causality and with global tokens: the query blocks of global
    rows list every key block and, past 8 key blocks, take the chunked form, whose
    partial O rows and LSEs need scratch."""
    L = _lib.lib()
    up = lambda x: (x + 255) // 256 * 256
    pat = lambda **kw: _lib.SaPattern(**{**dict(causal=0, window_left=-1, unit_window=-1, global_tokens=130), **kw})
    a = _args(batch=2, heads=3, n_q=1000, n_kv=2000, pattern=pat())
    for s in (a.q_strides, a.k_strides, a.v_strides, a.o_strides):
        s[:] = [1 << 24, 1 << 20, 64]
    gq, chunks = 3, 4                                  # ceil(130 / 64) blocks; 32 key blocks in chunks of 8
    slots = 2 * 3 * gq * chunks * 64
    need = L.sa_attn_workspace_bytes(ctypes.byref(a))
    assert need == up(slots * 64 * 4) + up(slots * 4)
    for kw in (dict(pattern=pat(causal=1)), dict(pattern=pat(global_tokens=0)), dict(per_head_lists=1),
               dict(n_kv=512), dict(pattern=pat(q_offset=130))):
        assert L.sa_attn_workspace_bytes(ctypes.byref(_args(batch=2, heads=3, n_q=1000,
                                                            **{"n_kv": 2000, **kw}))) == 0, kw
    a.workspace, a.workspace_bytes = 1 << 20, need - 1
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "workspace" in _err()
    a.workspace, a.workspace_bytes = (1 << 20) + 16, need
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "aligned" in _err()


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


def test_strided_form_detection_and_workspace():
    """SA_MODE_STRIDED accepts only the strided template (its workspace query is 0
    otherwise) and its scratch holds the two parts' block lists, 64 x 64 tiles."""
    import block_sparse_attention_sa_amd as sa
    pat = dict(causal=1, window_left=127, window_right=0, stride=128, stride_phase=127)
    up = lambda x: (x + 255) // 256 * 256

    def lists(at, nq, nkv):
        nqb, nkb = -(-nq // 64), -(-nkv // 64)
        return up(up(up(up(at + 4 * nqb) + 4 * nqb * nkb) + nqb * nkb) + 8)

    n, S = 16384, 128
    G = n // S
    exp = lists(lists(0, n, n), G - 1, G)
    assert sa.attn_workspace_bytes_strided(pat, 1, 16, n, 64) == exp
    assert sa.attn_workspace_bytes_strided(pat, 1, 16, 16300, 64) == 0           # not a multiple of the stride
    assert sa.attn_workspace_bytes_strided(pat, 1, 16, 256, 64) == 0             # fewer than three groups
    for bad in (dict(pat, sinks=4), dict(pat, stride_phase=3), dict(pat, window_left=64), dict(pat, causal=0),
                dict(pat, global_tokens=1), dict(pat, q_offset=5)):
        assert sa.attn_workspace_bytes_strided(bad, 1, 16, n, 64) == 0, bad


def test_strided_mode_argument_errors():
    L = _lib.lib()
    a = _args(mode=_lib.SA_MODE_STRIDED, n_q=1024, n_kv=1024, o_dtype=_lib.SA_DTYPE_F32, lse=8192)
    a.pattern = _lib.SaPattern(causal=1, window_left=127, window_right=0, stride=128, stride_phase=127,
                               unit_window=-1)
    for st in (a.q_strides, a.k_strides, a.v_strides, a.o_strides):
        st[:] = [1 << 20, 1 << 16, 64]
    need = L.sa_attn_workspace_bytes(ctypes.byref(a))
    assert need > 0
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "workspace" in _err()
    a.workspace, a.workspace_bytes = 1 << 20, need - 1
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG
    a.workspace, a.workspace_bytes = (1 << 20) + 16, need
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "aligned" in _err()
    a.workspace = 1 << 20
    a.o_dtype = _lib.SA_DTYPE_BF16
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_UNSUPPORTED and "float32" in _err()
    a.o_dtype = _lib.SA_DTYPE_F32
    a.lse = None
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "lse" in _err()
    a.lse = 8192
    a.pattern.sinks = 2
    assert L.sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "template" in _err()
    assert L.sa_attn_strided_plan(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "template" in _err()
    a.pattern.sinks = 0
    a.workspace_bytes = need - 1
    assert L.sa_attn_strided_plan(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "workspace" in _err()
    a.mode = _lib.SA_MODE_BLOCKS
    assert L.sa_attn_strided_plan(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "mode" in _err()


def _sel_args(**kw):
    a = _lib.SaSelectArgs()
    a.q = a.k = 4096
    a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = 1, 2, 512, 512, 64
    a.q_strides[:] = a.k_strides[:] = [2 * 512 * 64, 512 * 64, 64]
    a.block_q = a.block_kv = 64
    a.n_select = 2
    a.kv_count = a.kv_index = a.kv_partial = a.live_pairs = 4096
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_select_blocks_workspace_and_errors():
    L = _lib.lib()
    a = _sel_args()
    assert L.sa_select_blocks_workspace(ctypes.byref(a)) == 2 * 8 * 64 * 8 * 2   # fp64 means of q and k blocks
    for kw, status, word in ((dict(head_dim=96), _lib.SA_ERR_UNSUPPORTED, "head_dim"),
                             (dict(block_q=32), _lib.SA_ERR_UNSUPPORTED, "block"),
                             (dict(n_kv=64 * 1025), _lib.SA_ERR_UNSUPPORTED, "key blocks"),
                             (dict(n_select=-1), _lib.SA_ERR_INVALID_ARG, "negative"),
                             (dict(live_pairs=None), _lib.SA_ERR_INVALID_ARG, "live_pairs"),
                             (dict(), _lib.SA_ERR_INVALID_ARG, "workspace")):
        b = _sel_args(**kw)
        assert L.sa_select_blocks(ctypes.byref(b), None) == status, kw
        assert word in _err(), (kw, _err())
    b = _sel_args(workspace=4096 + 16, workspace_bytes=1 << 20)
    assert L.sa_select_blocks(ctypes.byref(b), None) == _lib.SA_ERR_INVALID_ARG and "aligned" in _err()
    assert L.sa_select_blocks_workspace(ctypes.byref(_sel_args(head_dim=96))) == 0


def test_attn_per_head_lists_flag_checked():
    a = _args(per_head_lists=2)
    assert _lib.lib().sa_attn_fwd(ctypes.byref(a), None) == _lib.SA_ERR_INVALID_ARG and "per_head_lists" in _err()


def test_attn_bwd_workspace_and_errors():
    L = _lib.lib()

    def bwd(**kw):
        a = _lib.SaAttnBwdArgs()
        a.q = a.k = a.v = a.o = a.lse = a.dout = a.dq = a.dk = a.dv = 4096
        a.batch, a.heads, a.n_q, a.n_kv, a.head_dim = 1, 2, 300, 300, 64
        a.block_q = a.block_kv = 64
        a.kv_count = a.kv_index = a.kv_partial = 4096
        a.pattern = _lib.SaPattern(causal=1, window_left=50, window_right=0, unit_window=-1)
        for k_, v_ in kw.items():
            setattr(a, k_, v_)
        return a

    up = lambda x: (x + 255) // 256 * 256
    nqb = nkb = 5
    q_partial = up(up(up(2 * 300 * 4) + nkb * 4) + nkb * nqb * 4)
    order_q = up(q_partial + nkb * nqb)
    order_k = up(order_q + nqb * 4)
    assert L.sa_attn_bwd_workspace(ctypes.byref(bwd())) == up(order_k + nkb * 4)
    for kw, status, word in ((dict(head_dim=96), _lib.SA_ERR_UNSUPPORTED, "head_dim"),
                             (dict(block_kv=32), _lib.SA_ERR_UNSUPPORTED, "block"),
                             (dict(per_head_lists=3), _lib.SA_ERR_INVALID_ARG, "per_head_lists"),
                             (dict(dq=None), _lib.SA_ERR_INVALID_ARG, "NULL"),
                             (dict(k=4100), _lib.SA_ERR_INVALID_ARG, "aligned"),
                             (dict(), _lib.SA_ERR_INVALID_ARG, "workspace")):
        assert L.sa_attn_bwd(ctypes.byref(bwd(**kw)), None) == status, kw
        assert word in _err(), (kw, _err())
    assert L.sa_attn_bwd_workspace(ctypes.byref(bwd(head_dim=96))) == 0
