"""Python binding of libeagle_verify.so (the C ABI in include/eagle_verify.h).

Argument marshalling only: every step of the verification runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
HIP stream.  If the shared library is missing, every call raises; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libeagle_verify.so"

EAGLE_OK = 0
EAGLE_ERR_INVALID_ARGUMENT = 1
EAGLE_ERR_UNSUPPORTED = 2
EAGLE_ERR_HIP = 3
EAGLE_ERR_WORKSPACE = 4

FLAG_BAD_PARENT = 1
FLAG_BAD_KV_LEN = 2
FLAG_BAD_TOKEN = 4
FLAG_NONFINITE = 8
FLAG_BAD_PATH = 32
FLAG_BAD_ROW = 64


class EagleError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"eagle status {status}: {message}")
        self.status = status


_LIB = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "eagle_last_error": (ctypes.c_char_p, []),
    "eagle_abi_version": (_I, []),
    "eagle_validate_tree_host": (_I, [_P, _I, _I]),
    "eagle_workspace_clear": (_I, [_P, _SZ, _P]),
    "eagle_testing_attn_plan": (_I, [_I, _I]),
    "eagle_testing_read_floor": (_I, [_P, _SZ, _I, _P, _P]),
    "eagle_tree_build": (_I, [_P, _P, _I, _I, _P, _P, _P, _P, _P]),
    "eagle_tree_attn_workspace": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "eagle_tree_attn": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _P, _P]),
    "eagle_tree_attn_parents": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P,
                                     _P, _P, _SZ, _P, _P]),
    "eagle_tree_attn_parents_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P,
                                             _P, _P, _P, _P, _P]),
    "eagle_verify_accept_workspace": (_SZ, [_I, _I, _I]),
    "eagle_verify_accept": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P, _P,
                                 _P, _P, _P, _P, _P, _SZ, _P, _P]),
    "eagle_verify_accept_compact": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P, _P,
                                         _P, _P, _P, _P, _I, _I, _I, _P, _P, _SZ, _P, _P]),
    "eagle_kv_compact": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "eagle_feature_gather": (_I, [_P, _P, _P, _I, _I, ctypes.c_int64, _P, _P, _P]),
    "eagle_dtree_expand": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P]),
    "eagle_dtree_select": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "eagle_dtree_rerank": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
}


def library_path() -> str:
    return os.environ.get("EAGLE_VERIFY_LIB") or os.path.join(PKG_DIR, LIB_NAME)


def lib():
    """The loaded C library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m "
                               "tree_attention_verification_parent_amd.build` first")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def _check(status: int) -> None:
    if status != EAGLE_OK:
        raise EagleError(status, lib().eagle_last_error().decode())


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _expect(t: Optional[torch.Tensor], shape, name: str) -> None:
    """The kernels index these buffers by the sizes passed beside them, so a
    tensor of another shape would be read or written out of its bounds."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_cache(q, k_cache, v_cache, kv_len, seq_flags):
    B, N, Hq, d = q.shape
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError(f"k_cache must be [B, Hkv, Lmax, d] with B = {B}, d = {d}, "
                         f"got {tuple(k_cache.shape)}")
    _expect(v_cache, k_cache.shape, "v_cache")
    _expect(kv_len, (B,), "kv_len")
    _expect(seq_flags, (B,), "seq_flags")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def abi_version() -> int:
    return lib().eagle_abi_version()


def validate_tree_host(parents) -> None:
    """Host-side check of a [B, N] int32 parent array (numpy or CPU tensor)."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    if arr.ndim == 1:
        arr = arr[None]
    B, N = arr.shape
    _check(lib().eagle_validate_tree_host(arr.ctypes.data, B, N))


ATTN_KERNELS = {"auto": 0, "ring": 1, "group": 2}


def testing_attn_plan(kernel: str = "auto", pieces: int = 0) -> None:
    """Testing hook: force the attention kernel ("auto", "ring", "group") and
    the pieces per (sequence, KV head) at full cache length (0 = planner) of
    later attention calls in this process."""
    _check(lib().eagle_testing_attn_plan(ATTN_KERNELS[kernel], int(pieces)))


def testing_read_floor(src: torch.Tensor, workgroups: int, sink: torch.Tensor,
                       stream=None) -> None:
    """Measurement hook: read all of `src` (a contiguous device tensor) with
    the ring attention kernel's load structure and nothing else, split over
    `workgroups` workgroups; `sink` (int32, workgroups * 512) receives what
    was read, XOR-ed per thread."""
    nbytes = src.numel() * src.element_size()
    if sink.numel() * sink.element_size() < workgroups * 512 * 4:
        raise ValueError("sink must hold workgroups * 512 int32")
    _check(lib().eagle_testing_read_floor(_ptr(src, name="src"), nbytes, int(workgroups),
                                          _ptr(sink, torch.int32, "sink"), _stream(stream)))


class attn_plan:
    """Context manager around testing_attn_plan that restores the planner."""

    def __init__(self, kernel: str = "auto", pieces: int = 0):
        self.kernel, self.pieces = kernel, pieces

    def __enter__(self):
        testing_attn_plan(self.kernel, self.pieces)
        return self

    def __exit__(self, *exc):
        testing_attn_plan("auto", 0)
        return False


def workspace_clear(ws: torch.Tensor, stream=None) -> None:
    _check(lib().eagle_workspace_clear(_ptr(ws, name="workspace"), ws.numel() * ws.element_size(),
                                       _stream(stream)))


def tree_build(parents: torch.Tensor, kv_len: Optional[torch.Tensor] = None, *, anc=None,
               depth=None, pos=None, seq_flags=None, stream=None):
    """Ancestor masks (int64 tensor holding the uint64 bits), depth and position ids."""
    B, N = parents.shape
    _expect(kv_len, (B,), "kv_len")
    for t, name in ((anc, "anc"), (depth, "depth"), (pos, "pos")):
        _expect(t, (B, N), name)
    _expect(seq_flags, (B,), "seq_flags")
    if anc is None:
        anc = torch.empty((B, N), dtype=torch.int64, device=parents.device)
        depth = torch.empty((B, N), dtype=torch.int32, device=parents.device)
        if kv_len is not None:
            pos = torch.empty((B, N), dtype=torch.int32, device=parents.device)
    _check(lib().eagle_tree_build(_ptr(parents, torch.int32, "parents"),
                                  _ptr(kv_len, torch.int32, "kv_len"), B, N, _ptr(anc), _ptr(depth),
                                  _ptr(pos), _ptr(seq_flags, torch.int32, "seq_flags"),
                                  _stream(stream)))
    return anc, depth, pos


def tree_attn_workspace_bytes(B, N, Hq, Hkv, d, Lmax) -> int:
    return int(lib().eagle_tree_attn_workspace(B, N, Hq, Hkv, d, Lmax))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Device workspace of `nbytes` (zero-filled, as the verification
    workspace requires before its first use)."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def tree_attn(q, k_cache, v_cache, kv_len, anc, *, sm_scale: float = 0.0, out=None,
              workspace=None, seq_flags=None, stream=None):
    """q [B,N,Hq,d] bf16; k/v [B,Hkv,Lmax,d] bf16; kv_len [B] int32; anc [B,N] int64."""
    B, N, Hq, d = q.shape
    _check_cache(q, k_cache, v_cache, kv_len, seq_flags)
    _expect(anc, (B, N), "anc")
    _expect(out, q.shape, "out")
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(tree_attn_workspace_bytes(B, N, Hq, Hkv, d, Lmax), q.device)
    _check(lib().eagle_tree_attn(
        _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(kv_len, torch.int32, "kv_len"),
        _ptr(anc, torch.int64, "anc"), B, N, Hq, Hkv, d, Lmax, float(sm_scale),
        _ptr(out, torch.bfloat16, "out"), _ptr(workspace, name="workspace"),
        workspace.numel() * workspace.element_size(), _ptr(seq_flags, torch.int32, "seq_flags"),
        _stream(stream)))
    return out


def tree_attn_parents(q, k_cache, v_cache, kv_len, parents, *, sm_scale: float = 0.0, out=None,
                      anc=None, depth=None, pos=None, workspace=None, seq_flags=None, stream=None):
    """Tree mask built from parents [B,N] int32 inside the attention launch; anc [B,N] int64,
    depth and pos [B,N] int32 are optional outputs.  Returns out."""
    B, N, Hq, d = q.shape
    _check_cache(q, k_cache, v_cache, kv_len, seq_flags)
    for t, name in ((parents, "parents"), (anc, "anc"), (depth, "depth"), (pos, "pos")):
        _expect(t, (B, N), name)
    _expect(out, q.shape, "out")
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(tree_attn_workspace_bytes(B, N, Hq, Hkv, d, Lmax), q.device)
    _check(lib().eagle_tree_attn_parents(
        _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(kv_len, torch.int32, "kv_len"),
        _ptr(parents, torch.int32, "parents"), B, N, Hq, Hkv, d, Lmax, float(sm_scale),
        _ptr(out, torch.bfloat16, "out"), _ptr(anc, torch.int64, "anc"),
        _ptr(depth, torch.int32, "depth"), _ptr(pos, torch.int32, "pos"),
        _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
        _ptr(seq_flags, torch.int32, "seq_flags"), _stream(stream)))
    return out


def tree_attn_parents_noalloc(q, k_cache, v_cache, kv_len, parents, *, sm_scale: float = 0.0,
                              out=None, anc=None, depth=None, pos=None, seq_flags=None,
                              stream=None):
    """tree_attn_parents with the library's static scratch instead of a
    workspace (eagle_tree_attn_parents_noalloc).  Returns out."""
    B, N, Hq, d = q.shape
    _check_cache(q, k_cache, v_cache, kv_len, seq_flags)
    for t, name in ((parents, "parents"), (anc, "anc"), (depth, "depth"), (pos, "pos")):
        _expect(t, (B, N), name)
    _expect(out, q.shape, "out")
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _check(lib().eagle_tree_attn_parents_noalloc(
        _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(kv_len, torch.int32, "kv_len"),
        _ptr(parents, torch.int32, "parents"), B, N, Hq, Hkv, d, Lmax, float(sm_scale),
        _ptr(out, torch.bfloat16, "out"), _ptr(anc, torch.int64, "anc"),
        _ptr(depth, torch.int32, "depth"), _ptr(pos, torch.int32, "pos"),
        _ptr(seq_flags, torch.int32, "seq_flags"), _stream(stream)))
    return out


def _check_walk_inputs(draft_tokens, draft_probs, target_logits, parents, kv_len, uniforms,
                       outputs, seq_flags, draft_row=None):
    B, N, V = target_logits.shape
    for t, name in ((draft_tokens, "draft_tokens"), (parents, "parents"), (uniforms, "uniforms"),
                    (draft_row, "draft_row")):
        _expect(t, (B, N), name)
    _expect(draft_probs, (B, N, V), "draft_probs")
    _expect(kv_len, (B,), "kv_len")
    _expect(seq_flags, (B,), "seq_flags")
    shapes = {"accept_len": (B,), "bonus": (B,), "new_kv_len": (B,), "path": (B, N),
              "accepted_tokens": (B, N), "kv_src": (B, N), "ratio": (B, N),
              "probs": (B, N, V), "final_dist": (B, V)}
    for key, t in (outputs or {}).items():
        if key in shapes:
            _expect(t, shapes[key], key)


def verify_accept_workspace_bytes(B, N, V) -> int:
    return int(lib().eagle_verify_accept_workspace(B, N, V))


def verify_accept(draft_tokens, draft_probs, target_logits, parents, kv_len, temperature, uniforms,
                  *, draft_row=None, want_probs=False, want_final_dist=False, want_ratio=False,
                  outputs=None, workspace=None, seq_flags=None, stream=None):
    """Acceptance walk; returns a dict of device tensors (see include/eagle_verify.h).
    draft_row [B, N] int32 (optional): the row of draft_probs each node was drawn from."""
    B, N, V = target_logits.shape
    _check_walk_inputs(draft_tokens, draft_probs, target_logits, parents, kv_len, uniforms,
                       outputs, seq_flags, draft_row)
    dev = target_logits.device
    o = outputs or {}
    if not o:
        o["accept_len"] = torch.empty(B, dtype=torch.int32, device=dev)
        o["path"] = torch.empty((B, N), dtype=torch.int32, device=dev)
        o["accepted_tokens"] = torch.empty((B, N), dtype=torch.int32, device=dev)
        o["bonus"] = torch.empty(B, dtype=torch.int32, device=dev)
        o["kv_src"] = torch.empty((B, N), dtype=torch.int32, device=dev)
        if want_probs:
            o["probs"] = torch.empty((B, N, V), dtype=torch.float32, device=dev)
        if want_final_dist:
            o["final_dist"] = torch.empty((B, V), dtype=torch.float32, device=dev)
        if want_ratio:
            o["ratio"] = torch.empty((B, N), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(verify_accept_workspace_bytes(B, N, V), dev)
    _check(lib().eagle_verify_accept(
        _ptr(draft_tokens, torch.int32, "draft_tokens"), _ptr(draft_probs, torch.float32, "draft_probs"),
        _ptr(draft_row, torch.int32, "draft_row"),
        _ptr(target_logits, torch.float32, "target_logits"), _ptr(parents, torch.int32, "parents"),
        _ptr(kv_len, torch.int32, "kv_len"), B, N, V, float(temperature),
        _ptr(uniforms, torch.float32, "uniforms"),
        _ptr(o["accept_len"]), _ptr(o["path"]), _ptr(o["accepted_tokens"]), _ptr(o["bonus"]),
        _ptr(o["kv_src"]), _ptr(o.get("probs")), _ptr(o.get("final_dist")), _ptr(o.get("ratio")),
        _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
        _ptr(seq_flags, torch.int32, "seq_flags"), _stream(stream)))
    return o


def verify_accept_compact(draft_tokens, draft_probs, target_logits, parents, kv_len, temperature,
                          uniforms, k_cache, v_cache, *, draft_row=None, outputs=None,
                          new_kv_len=None, workspace=None, seq_flags=None, stream=None):
    """Acceptance walk and KV compaction in one launch; returns the walk's
    outputs (as verify_accept) plus "new_kv_len"."""
    B, N, V = target_logits.shape
    _check_walk_inputs(draft_tokens, draft_probs, target_logits, parents, kv_len, uniforms,
                       outputs, seq_flags, draft_row)
    if k_cache.dim() != 4 or k_cache.shape[0] != B:
        raise ValueError(f"k_cache must be [B, Hkv, Lmax, d] with B = {B}, got {tuple(k_cache.shape)}")
    _expect(v_cache, k_cache.shape, "v_cache")
    _expect(new_kv_len, (B,), "new_kv_len")
    _, Hkv, Lmax, d = k_cache.shape
    dev = target_logits.device
    o = dict(outputs) if outputs else {}
    if "accept_len" not in o:
        o["accept_len"] = torch.empty(B, dtype=torch.int32, device=dev)
        o["path"] = torch.empty((B, N), dtype=torch.int32, device=dev)
        o["accepted_tokens"] = torch.empty((B, N), dtype=torch.int32, device=dev)
        o["bonus"] = torch.empty(B, dtype=torch.int32, device=dev)
        o["kv_src"] = torch.empty((B, N), dtype=torch.int32, device=dev)
    if new_kv_len is None:
        new_kv_len = o.get("new_kv_len")
    if new_kv_len is None:
        new_kv_len = torch.empty_like(kv_len)
    o["new_kv_len"] = new_kv_len
    if workspace is None:
        workspace = alloc_workspace(verify_accept_workspace_bytes(B, N, V), dev)
    _check(lib().eagle_verify_accept_compact(
        _ptr(draft_tokens, torch.int32, "draft_tokens"), _ptr(draft_probs, torch.float32, "draft_probs"),
        _ptr(draft_row, torch.int32, "draft_row"),
        _ptr(target_logits, torch.float32, "target_logits"), _ptr(parents, torch.int32, "parents"),
        _ptr(kv_len, torch.int32, "kv_len"), B, N, V, float(temperature),
        _ptr(uniforms, torch.float32, "uniforms"),
        _ptr(o["accept_len"]), _ptr(o["path"]), _ptr(o["accepted_tokens"]), _ptr(o["bonus"]),
        _ptr(o["kv_src"]), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), Hkv, d, Lmax,
        _ptr(new_kv_len, torch.int32, "new_kv_len"),
        _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
        _ptr(seq_flags, torch.int32, "seq_flags"), _stream(stream)))
    return o


def kv_compact(k_cache, v_cache, kv_len, kv_src, accept_len, *, new_kv_len=None, seq_flags=None,
               stream=None):
    B, Hkv, Lmax, d = k_cache.shape
    if kv_src.dim() != 2 or kv_src.shape[0] != B:
        raise ValueError(f"kv_src must be [B, N] with B = {B}, got {tuple(kv_src.shape)}")
    N = kv_src.shape[1]
    _expect(v_cache, k_cache.shape, "v_cache")
    for t, name in ((kv_len, "kv_len"), (accept_len, "accept_len"), (new_kv_len, "new_kv_len"),
                    (seq_flags, "seq_flags")):
        _expect(t, (B,), name)
    if new_kv_len is None:
        new_kv_len = torch.empty_like(kv_len)
    _check(lib().eagle_kv_compact(
        _ptr(k_cache, torch.bfloat16, "k_cache"), _ptr(v_cache, torch.bfloat16, "v_cache"),
        _ptr(kv_len, torch.int32, "kv_len"), _ptr(kv_src, torch.int32, "kv_src"),
        _ptr(accept_len, torch.int32, "accept_len"), B, N, Hkv, d, Lmax,
        _ptr(new_kv_len, torch.int32, "new_kv_len"), _ptr(seq_flags, torch.int32, "seq_flags"),
        _stream(stream)))
    return new_kv_len


def feature_gather(features, path, accept_len, *, out=None, seq_flags=None, stream=None):
    """out[b, j] = features[b, path[b, j]] for j = 0..accept_len[b] (rows
    copied as bytes); features [B, N, ...] contiguous, any dtype.  Returns out
    (rows past accept_len[b] are left as they were)."""
    B, N = path.shape
    if features.dim() < 2 or tuple(features.shape[:2]) != (B, N):
        raise ValueError(f"features must be [B, N, ...] with B, N = {B}, {N}")
    _expect(accept_len, (B,), "accept_len")
    _expect(seq_flags, (B,), "seq_flags")
    row_bytes = features[0, 0].numel() * features.element_size()
    if out is None:
        out = torch.empty_like(features)
    if out.shape != features.shape or out.dtype != features.dtype:
        raise ValueError("out must have the shape and dtype of features")
    _check(lib().eagle_feature_gather(
        _ptr(features, None, "features"), _ptr(path, torch.int32, "path"),
        _ptr(accept_len, torch.int32, "accept_len"), B, N, row_bytes, _ptr(out, None, "out"),
        _ptr(seq_flags, torch.int32, "seq_flags"), _stream(stream)))
    return out


# ---- EAGLE-2 dynamic tree: created nodes are [B, T] arrays (parent, token, value)
def dtree_expand(q, parent_node, parent_value, k, created_parent, created_token, created_value,
                 base, *, stream=None):
    """Children of the R expanded rows of q [B, R, V]: created nodes
    base + r*k + j take the row's j-th most probable token (ties: lower id),
    parent parent_node[b, r] and value parent_value[b, r] * q[b, r, token]."""
    B, R, V = q.shape
    if created_parent.dim() != 2 or created_parent.shape[0] != B:
        raise ValueError(f"created arrays must be [B, T] with B = {B}")
    T = created_parent.shape[1]
    _expect(parent_node, (B, R), "parent_node")
    _expect(parent_value, (B, R), "parent_value")
    _expect(created_token, (B, T), "created_token")
    _expect(created_value, (B, T), "created_value")
    _check(lib().eagle_dtree_expand(
        _ptr(q, torch.float32, "q"), B, R, V, k, _ptr(parent_node, torch.int32, "parent_node"),
        _ptr(parent_value, torch.float32, "parent_value"),
        _ptr(created_parent, torch.int32, "created_parent"),
        _ptr(created_token, torch.int32, "created_token"),
        _ptr(created_value, torch.float32, "created_value"), T, base, _stream(stream)))


def dtree_select(created_value, first, count, k, *, out_node=None, out_value=None, stream=None):
    """The k most valuable created nodes among ids [first, first + count)
    (ties: lower id), most valuable first: (node ids [B, k], values [B, k])."""
    B, T = created_value.shape
    _expect(out_node, (B, k), "out_node")
    _expect(out_value, (B, k), "out_value")
    dev = created_value.device
    if out_node is None:
        out_node = torch.empty((B, k), dtype=torch.int32, device=dev)
    if out_value is None:
        out_value = torch.empty((B, k), dtype=torch.float32, device=dev)
    _check(lib().eagle_dtree_select(
        _ptr(created_value, torch.float32, "created_value"), B, T, first, count, k,
        _ptr(out_node, torch.int32, "out_node"), _ptr(out_value, torch.float32, "out_value"),
        _stream(stream)))
    return out_node, out_value


def dtree_rerank(created_parent, created_token, created_value, used, N, *, seq_flags=None,
                 stream=None):
    """Keep the root and the N - 1 most valuable of created nodes [1, used),
    renumbered in creation order: (parents [B, N], tokens [B, N], kept created
    ids [B, N])."""
    B, T = created_parent.shape
    _expect(created_token, (B, T), "created_token")
    _expect(created_value, (B, T), "created_value")
    _expect(seq_flags, (B,), "seq_flags")
    dev = created_parent.device
    parents = torch.empty((B, N), dtype=torch.int32, device=dev)
    tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    kept = torch.empty((B, N), dtype=torch.int32, device=dev)
    _check(lib().eagle_dtree_rerank(
        _ptr(created_parent, torch.int32, "created_parent"),
        _ptr(created_token, torch.int32, "created_token"),
        _ptr(created_value, torch.float32, "created_value"), B, T, used, N,
        _ptr(parents, torch.int32, "parents"), _ptr(tokens, torch.int32, "tokens"),
        _ptr(kept, torch.int32, "kept"), _ptr(seq_flags, torch.int32, "seq_flags"),
        _stream(stream)))
    return parents, tokens, kept
