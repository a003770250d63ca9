"""ctypes binding of libdflash2 (argument marshalling only).

Every function takes torch tensors already on the GPU (or None for optional
outputs) and enqueues the library's kernels on the current torch stream,
unless ``stream`` gives another ``torch.cuda.Stream``.  Nothing here computes:
if the shared library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdflash2.so")

DFS_F32 = 0
DFS_BF16 = 1

STATUS = {
    0: "DFS_OK",
    1: "DFS_ERR_NULL",
    2: "DFS_ERR_SHAPE",
    3: "DFS_ERR_UNSUPPORTED",
    4: "DFS_ERR_MISALIGNED",
    5: "DFS_ERR_WORKSPACE",
    6: "DFS_ERR_HIP",
}

EXPORTS = ("dfs_workspace_size", "dfs_status_string", "dfs_validate_config", "dfs_conv",
           "dfs_conv_layers", "dfs_conv_layers_workspace_size",
           "dfs_head_topk", "dfs_topk_logits", "dfs_select", "dfs_draft_block", "dfs_draft_block_static")

STATIC_WORKSPACE_BYTES = 64 << 20  # DFS_STATIC_WORKSPACE_BYTES


class Config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("batch", "block_size", "hidden", "vocab", "top_k", "rank",
                 "conv_group_size", "conv_kernel_size", "dtype")]

    @classmethod
    def of(cls, shape) -> "Config":
        """From a ``workloads.Shape``-like object."""
        return cls(shape.batch, shape.block, shape.hidden, shape.vocab, shape.top_k, shape.rank,
                   shape.group, shape.ksize, DFS_BF16 if shape.dtype == "bf16" else DFS_F32)

    @property
    def rows(self) -> int:
        return self.batch * self.block_size


WALKS = {"viterbi": 0, "greedy": 1, "sample": 2}


class SelectOpts(C.Structure):
    """dfs_select_opts: context gate, walk rule, temperature, uniforms."""
    _fields_ = [("gate", C.c_void_p), ("walk", C.c_int32), ("temperature", C.c_float),
                ("uniforms", C.c_void_p)]


def _opts(gate, walk, temperature, uniforms):
    if gate is None and walk == "viterbi" and uniforms is None:
        return None
    return C.byref(SelectOpts(_ptr(gate), WALKS[walk], float(temperature), _ptr(uniforms)))


class DFSError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({_lib.dfs_status_string(status).decode()})")


def _load():
    # PyTorch ships its own HIP runtime with the same soname as the system
    # one.  Importing torch first makes the dynamic loader bind this library
    # to that already-loaded runtime; loading the library first would put two
    # HIP runtimes in one process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python block_drafter_grouped_amd/build.py`")
    lib_ = C.CDLL(LIB_PATH)
    P, S, I = C.c_void_p, C.c_size_t, C.c_int
    cfg = C.POINTER(Config)
    lib_.dfs_workspace_size.argtypes = [cfg]
    lib_.dfs_workspace_size.restype = S
    lib_.dfs_status_string.argtypes = [I]
    lib_.dfs_status_string.restype = C.c_char_p
    lib_.dfs_validate_config.argtypes = [cfg]
    lib_.dfs_conv.argtypes = [cfg, P, P, P, P, P, S, P]
    lib_.dfs_conv_layers.argtypes = [cfg, I, P, P, P, P, S, P]
    lib_.dfs_conv_layers_workspace_size.restype = S
    lib_.dfs_conv_layers_workspace_size.argtypes = [cfg, I]
    lib_.dfs_head_topk.argtypes = [cfg, P, P, P, P, P, P, P, S, P]
    lib_.dfs_topk_logits.argtypes = [cfg, P, P, P, P, P, S, P]
    lib_.dfs_select.argtypes = [cfg, P, P, P, P, P, P, P, P, P, P, S, P]
    lib_.dfs_draft_block.argtypes = [cfg, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib_.dfs_draft_block_static.argtypes = [cfg, P, P, P, P, P, P, P, P, P, P, P, P]
    for n in EXPORTS[2:]:
        getattr(lib_, n).restype = I
    return lib_


_lib = _load()


def lib():
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if isinstance(stream, int):
        return stream
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _nbytes(ws):
    if ws is None:
        return 0
    return ws.numel() * ws.element_size()


def _check(st: int, fn: str):
    if st != 0:
        raise DFSError(st, fn)


def workspace_size(cfg: Config) -> int:
    return int(_lib.dfs_workspace_size(C.byref(cfg)))


def validate_config(cfg: Config) -> int:
    return int(_lib.dfs_validate_config(C.byref(cfg)))


def conv(cfg, h, wg_cm, y, ws, y_f32=None, stream=None):
    _check(_lib.dfs_conv(C.byref(cfg), _ptr(h), _ptr(wg_cm), _ptr(y), _ptr(y_f32), _ptr(ws), _nbytes(ws),
                         _stream(stream)), "dfs_conv")


def conv_layers_workspace_size(cfg: Config, layers: int) -> int:
    return _lib.dfs_conv_layers_workspace_size(C.byref(cfg), layers)


def conv_layers(cfg, layers, h, wg_cm, y, ws, stream=None):
    """dfs_conv_layers: h [layers, rows, D], wg_cm [layers, G*ks, D] -> y
    [layers, rows, D]; ws of conv_layers_workspace_size(cfg, layers) bytes."""
    _check(_lib.dfs_conv_layers(C.byref(cfg), layers, _ptr(h), _ptr(wg_cm), _ptr(y), _ptr(ws), _nbytes(ws),
                                _stream(stream)), "dfs_conv_layers")


def head_topk(cfg, y, W, cand_ids, cand_logp, lse, ws, logits_f32=None, stream=None):
    _check(_lib.dfs_head_topk(C.byref(cfg), _ptr(y), _ptr(W), _ptr(cand_ids), _ptr(cand_logp), _ptr(lse),
                              _ptr(logits_f32), _ptr(ws), _nbytes(ws), _stream(stream)), "dfs_head_topk")


def topk_logits(cfg, logits, cand_ids, cand_logp, lse, ws, stream=None):
    _check(_lib.dfs_topk_logits(C.byref(cfg), _ptr(logits), _ptr(cand_ids), _ptr(cand_logp), _ptr(lse),
                                _ptr(ws), _nbytes(ws), _stream(stream)), "dfs_topk_logits")


def select(cfg, anchor, cand_ids, cand_logp, P, Q, path, path_score, ws, path_idx=None, stream=None,
           gate=None, walk="viterbi", temperature=1.0, uniforms=None):
    """dfs_select.  gate: fp32 [rows, r] context gate or None; walk: "viterbi",
    "greedy" or "sample" (then temperature > 0 and fp32 uniforms [batch, B])."""
    _check(_lib.dfs_select(C.byref(cfg), _opts(gate, walk, temperature, uniforms), _ptr(anchor), _ptr(cand_ids),
                           _ptr(cand_logp), _ptr(P), _ptr(Q), _ptr(path), _ptr(path_score), _ptr(path_idx),
                           _ptr(ws), _nbytes(ws), _stream(stream)), "dfs_select")


def draft_block(cfg, h, anchor, wg_cm, W, P, Q, path, path_score, ws, cand_ids=None, cand_logp=None,
                stream=None, gate=None, walk="viterbi", temperature=1.0, uniforms=None):
    """dfs_draft_block: conv, head + top-K and selector on one stream; the
    selector options as for select()."""
    _check(_lib.dfs_draft_block(C.byref(cfg), _opts(gate, walk, temperature, uniforms), _ptr(h), _ptr(anchor),
                                _ptr(wg_cm), _ptr(W), _ptr(P), _ptr(Q), _ptr(path), _ptr(path_score),
                                _ptr(cand_ids), _ptr(cand_logp), _ptr(ws), _nbytes(ws), _stream(stream)),
           "dfs_draft_block")


def draft_block_static(cfg, h, anchor, wg_cm, W, P, Q, path, path_score, cand_ids=None, cand_logp=None,
                       stream=None, gate=None, walk="viterbi", temperature=1.0, uniforms=None):
    """dfs_draft_block_static: draft_block() on the library's static
    per-device workspace (no workspace argument, nothing allocated)."""
    _check(_lib.dfs_draft_block_static(C.byref(cfg), _opts(gate, walk, temperature, uniforms), _ptr(h),
                                       _ptr(anchor), _ptr(wg_cm), _ptr(W), _ptr(P), _ptr(Q), _ptr(path),
                                       _ptr(path_score), _ptr(cand_ids), _ptr(cand_logp), _stream(stream)),
           "dfs_draft_block_static")
