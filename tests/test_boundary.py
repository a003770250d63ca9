"""The C ABI on the host: exports, config rules, and every status a call can
return before it touches the GPU.  Pointers here are fake addresses; every
case is rejected by host-side validation, so no kernel is ever launched."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")

dfs = pytest.importorskip("block_drafter_grouped_amd")
import workloads as wl  # noqa: E402

OK, NULL, SHAPE, UNSUP, MISAL, WS, HIP = range(7)
A = 0x7F0000000000  # 256-B aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dfs_\w+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert set(names) == set(dfs.dflash2.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", dfs.dflash2.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dfs_\w+)$", out, re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(dfs.lib(), n)
    # and nothing else: the library's internal functions stay hidden
    every_text_symbol = set(re.findall(r"\bT (\S+)$", out, re.M))
    assert every_text_symbol == set(names), sorted(every_text_symbol - set(names))[:5]


def test_status_strings():
    for st in range(7):
        s = dfs.lib().dfs_status_string(st)
        assert isinstance(s, bytes) and len(s) > 0
    assert dfs.lib().dfs_status_string(99) == b"unknown status"


def cfg_of(cfg_id=2, **kw):
    c = dfs.Config.of(wl.shape_of(cfg_id))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("cfg_id", sorted(wl.WORKLOADS))
def test_workload_configs_are_valid(cfg_id):
    c = cfg_of(cfg_id)
    assert dfs.validate_config(c) == OK
    assert dfs.workspace_size(c) > 0


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, SHAPE), ("block_size", 1, SHAPE), ("block_size", 65, SHAPE),
    ("hidden", 48, SHAPE), ("hidden", 0, SHAPE), ("hidden", 16384, UNSUP),
    ("conv_group_size", 0, SHAPE), ("conv_group_size", 48, SHAPE),
    ("conv_kernel_size", 0, SHAPE), ("conv_kernel_size", 3, UNSUP), ("conv_kernel_size", 8, UNSUP),
    ("top_k", 0, SHAPE), ("top_k", 65, UNSUP), ("vocab", 15, SHAPE), ("vocab", (1 << 21) + 1, UNSUP),
    ("rank", 0, SHAPE), ("rank", 12, SHAPE), ("rank", 8192, SHAPE), ("dtype", 7, UNSUP),
])
def test_config_rules(field, value, status):
    c = cfg_of(2, **{field: value})
    assert dfs.validate_config(c) == status
    assert dfs.workspace_size(c) == 0


def test_config_rule_allowed_edges():
    assert dfs.validate_config(cfg_of(2, block_size=2)) == OK
    assert dfs.validate_config(cfg_of(2, block_size=64)) == OK
    assert dfs.validate_config(cfg_of(2, top_k=64)) == OK
    assert dfs.validate_config(cfg_of(2, conv_kernel_size=1)) == OK
    assert dfs.validate_config(cfg_of(2, conv_kernel_size=4)) == OK
    assert dfs.validate_config(cfg_of(2, vocab=16)) == OK
    assert dfs.validate_config(cfg_of(2, vocab=1 << 21)) == OK
    assert dfs.validate_config(cfg_of(0, hidden=16384, conv_group_size=16)) == OK  # fp32 has no LDS-resident head
    assert dfs.validate_config(cfg_of(2, batch=8192, block_size=8)) == OK
    assert dfs.validate_config(cfg_of(2, batch=8193, block_size=8)) == SHAPE


def test_workspace_grows_with_shape():
    small = dfs.workspace_size(cfg_of(2))
    big = dfs.workspace_size(cfg_of(3))
    assert big > small > 0
    # K > 16 on bf16 and every fp32 shape keep the logits in the workspace
    assert dfs.workspace_size(cfg_of(2, top_k=17)) >= 8 * 248320 * 4


L = dfs.lib()


def call(name, *args):
    return getattr(L, name)(*args)


def conv_args(cfg, h=A, wg=A, y=A, yf=None, ws=A, nbytes=None):
    if nbytes is None:
        nbytes = dfs.workspace_size(cfg) if dfs.validate_config(cfg) == OK else 0
    return (C.byref(cfg), h, wg, y, yf, ws, nbytes, None)


def test_conv_validation():
    c = cfg_of(2)
    assert L.dfs_conv(None, A, A, A, None, A, 1 << 20, None) == NULL
    assert call("dfs_conv", *conv_args(c, h=None)) == NULL
    assert call("dfs_conv", *conv_args(c, wg=None)) == NULL
    assert call("dfs_conv", *conv_args(c, y=None)) == NULL
    assert call("dfs_conv", *conv_args(c, h=A + 8)) == MISAL
    assert call("dfs_conv", *conv_args(c, yf=A + 4)) == MISAL
    assert call("dfs_conv", *conv_args(cfg_of(2, conv_kernel_size=3))) == UNSUP
    assert call("dfs_conv", *conv_args(cfg_of(2, hidden=100))) == SHAPE
    assert call("dfs_conv", *conv_args(c, nbytes=dfs.workspace_size(c) - 1)) == WS
    assert call("dfs_conv", *conv_args(c, ws=None)) == NULL
    assert call("dfs_conv", *conv_args(c, ws=A + 16)) == MISAL


def test_conv_layers_validation():
    c = cfg_of(2)
    n = dfs.conv_layers_workspace_size(c, 5)
    assert n >= dfs.conv_layers_workspace_size(c, 1) > 0
    # the split-D generator of many rows keeps partials per layer
    c3 = cfg_of(3)
    assert dfs.conv_layers_workspace_size(c3, 5) > dfs.conv_layers_workspace_size(c3, 1) > 0
    assert dfs.conv_layers_workspace_size(c, 0) == 0 and dfs.conv_layers_workspace_size(c, 65) == 0
    assert dfs.conv_layers_workspace_size(cfg_of(2, block_size=1), 5) == 0
    assert L.dfs_conv_layers(C.byref(c), 0, A, A, A, A, n, None) == SHAPE
    assert L.dfs_conv_layers(C.byref(c), 65, A, A, A, A, n, None) == SHAPE
    assert L.dfs_conv_layers(C.byref(c), 5, None, A, A, A, n, None) == NULL
    assert L.dfs_conv_layers(C.byref(c), 5, A, A, A, None, n, None) == NULL
    assert L.dfs_conv_layers(C.byref(c), 5, A, A + 8, A, A, n, None) == MISAL
    assert L.dfs_conv_layers(C.byref(c), 5, A, A, A, A + 16, n, None) == MISAL
    assert L.dfs_conv_layers(C.byref(c), 5, A, A, A, A, n - 1, None) == WS


def test_head_topk_validation():
    c = cfg_of(2)
    ws = dfs.workspace_size(c)
    base = [C.byref(c), A, A, A, A, A, None, A, ws, None]

    def with_(i, v):
        a = list(base)
        a[i] = v
        return a

    for i in (1, 2, 3, 4, 5, 7):
        assert L.dfs_head_topk(*with_(i, None)) == NULL, i
    for i in (1, 2, 3, 4, 5, 6):
        assert L.dfs_head_topk(*with_(i, A + 8)) == MISAL, i
    assert L.dfs_head_topk(*with_(7, A + 64)) == MISAL  # workspace wants 256 B
    assert L.dfs_head_topk(*with_(8, ws - 1)) == WS
    assert L.dfs_head_topk(*with_(0, C.byref(cfg_of(2, top_k=0)))) == SHAPE


def test_topk_logits_validation():
    c = cfg_of(1)
    ws = dfs.workspace_size(c)
    assert L.dfs_topk_logits(C.byref(c), None, A, A, A, A, ws, None) == NULL
    assert L.dfs_topk_logits(C.byref(c), A, A, A + 4, A, A, ws, None) == MISAL
    assert L.dfs_topk_logits(C.byref(c), A, A, A, A, A, 0, None) == WS
    assert L.dfs_topk_logits(C.byref(cfg_of(1, vocab=3)), A, A, A, A, A, ws, None) == SHAPE


def test_select_validation():
    c = cfg_of(3)
    ws = dfs.workspace_size(c)
    base = [C.byref(c), None, A, A, A, A, A, A, A, None, A, ws, None]
    for i in (2, 3, 4, 5, 6, 7, 8, 10):
        a = list(base)
        a[i] = None
        assert L.dfs_select(*a) == NULL, i
    for i in (2, 3, 4, 5, 6, 7, 8, 9):
        a = list(base)
        a[i] = A + 8
        assert L.dfs_select(*a) == MISAL, i
    a = list(base)
    a[11] = 16
    assert L.dfs_select(*a) == WS


def opts(**kw):
    o = dfs.dflash2.SelectOpts(None, 0, 1.0, None)
    for k, v in kw.items():
        setattr(o, k, v)
    return C.byref(o)


@pytest.mark.parametrize("o,status", [
    (dict(walk=3), UNSUP), (dict(walk=-1), UNSUP),
    (dict(walk=2), NULL),                                   # sampling needs the uniforms
    (dict(walk=2, uniforms=A, temperature=0.0), SHAPE),
    (dict(walk=2, uniforms=A, temperature=-1.0), SHAPE),
    (dict(walk=2, uniforms=A, temperature=float("inf")), SHAPE),
    (dict(walk=2, uniforms=A, temperature=float("nan")), SHAPE),
    (dict(walk=2, uniforms=A + 4), MISAL),
    (dict(gate=A + 8), MISAL),
])
def test_select_options_validation(o, status):
    c = cfg_of(3)
    ws = dfs.workspace_size(c)
    assert L.dfs_select(C.byref(c), opts(**o), A, A, A, A, A, A, A, None, A, ws, None) == status
    assert L.dfs_draft_block(C.byref(c), opts(**o), A, A, A, A, A, A, A, A, None, None, A, ws, None) == status


def test_select_options_unused_fields_ignored():
    """Uniforms and temperature are read only by the sampling walk: a greedy
    call with a bad temperature and no uniforms is still valid (it reaches
    the workspace check, the last host-side rule)."""
    c = cfg_of(3)
    o = opts(walk=1, temperature=0.0)
    assert L.dfs_select(C.byref(c), o, A, A, A, A, A, A, A, None, A, 16, None) == WS


def test_draft_block_validation():
    c = cfg_of(2)
    ws = dfs.workspace_size(c)
    base = [C.byref(c), None, A, A, A, A, A, A, A, A, None, None, A, ws, None]
    for i in (2, 3, 4, 5, 6, 7, 8, 9, 12):
        a = list(base)
        a[i] = None
        assert L.dfs_draft_block(*a) == NULL, i
    for i in (2, 3, 4, 5, 6, 7, 8, 9, 10, 11):
        a = list(base)
        a[i] = A + 2
        assert L.dfs_draft_block(*a) == MISAL, i
    a = list(base)
    a[13] = ws // 2
    assert L.dfs_draft_block(*a) == WS
    assert L.dfs_draft_block(C.byref(cfg_of(2, block_size=1)), *base[1:]) == SHAPE


def test_binding_raises_typed_error():
    c = cfg_of(2, block_size=1)
    with pytest.raises(dfs.DFSError) as e:
        dfs.conv(c, A, A, A, None, stream=0)
    assert e.value.status == SHAPE and "DFS_ERR_SHAPE" in str(e.value)


def test_static_entry_point_host_checks():
    """dfs_draft_block_static: the same host checks as dfs_draft_block, and a
    configuration whose workspace exceeds the static buffer is refused with
    DFS_ERR_WORKSPACE before any HIP call (fake pointers: nothing launches)."""
    import re as _re
    m = _re.search(r"#define DFS_STATIC_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == dfs.STATIC_WORKSPACE_BYTES
    f = dfs.lib().dfs_draft_block_static
    big = cfg_of(3)  # batch 32 at the page vocabulary: written logits of 254 MB
    assert dfs.workspace_size(big) > dfs.STATIC_WORKSPACE_BYTES
    args = [A] * 10 + [None, None, None]  # h, anchor, wg, W, P, Q, path, score; cand buffers; stream
    assert f(C.byref(big), None, *args[:8], None, None, None) == WS
    small = cfg_of(2)
    assert dfs.workspace_size(small) <= dfs.STATIC_WORKSPACE_BYTES
    assert f(C.byref(small), None, None, *args[1:8], None, None, None) == NULL
    assert f(C.byref(small), None, A + 8, *args[1:8], None, None, None) == MISAL
    assert f(C.byref(cfg_of(2, top_k=0)), None, *args[:8], None, None, None) == SHAPE
    bad_walk = dfs.SelectOpts(None, 7, 1.0, None)
    assert f(C.byref(small), C.byref(bad_walk), *args[:8], None, None, None) == UNSUP
