"""Python binding of libtpshard.so (one GPU's share of a tensor-parallel layer).

Argument marshalling only: every function checks dtypes, devices, shapes and
contiguity of torch tensors, passes their device pointers and the current
torch stream to the C entry point of the same name (include/tpshard.h), and
allocates missing outputs with torch. All arithmetic runs in the HIP kernels
of libtpshard.so; there is no fallback: if the library is not built, or no
GPU is present, the calls raise.

Errors: INVALID_ARG / NOT_DIVISIBLE -> ValueError, UNSUPPORTED ->
NotImplementedError, HIP -> RuntimeError (message from tp_last_error).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib_path", "load", "tp_version", "tp_last_error", "tp_col_linear",
    "tp_row_linear_partial", "tp_mlp_shard_fwd", "tp_mlp_shard_bwd",
    "tp_col_linear_bwd", "tp_row_linear_bwd", "tp_qkv_regroup", "tp_shard_shape",
    "tp_row_linear_partial_chunked", "tp_col_linear_bwd_chunked", "tp_kv_grad_accumulate", "tp_vocab_ce_fwd",
    "tp_vocab_ce_combine", "tp_vocab_ce_bwd", "tp_vocab_embed_fwd", "tp_vocab_embed_bwd",
    "tp_col_linear_noalloc", "workspace_size", "regroup_width", "ACT", "TPError",
]

ACT = {"none": 0, "gelu": 1, "swiglu": 2}
_STATUS = {0: "TP_OK", 1: "TP_ERR_INVALID_ARG", 2: "TP_ERR_NOT_DIVISIBLE",
           3: "TP_ERR_UNSUPPORTED", 4: "TP_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class TPError(RuntimeError):
    pass


def lib_path() -> str:
    return os.path.join(_HERE, "libtpshard.so")


def load():
    """Load libtpshard.so (torch is imported first so both share one HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m tensor_sharded_matmul_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sz, psz = ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)
    i = ctypes.c_int
    sigs = {
        "tp_version": ([], i),
        "tp_last_error": ([], ctypes.c_char_p),
        "tp_col_linear_workspace_size": ([i64, i64, i64, i, psz], i),
        "tp_col_linear": ([vp, vp, vp, i64, i64, i64, i, vp, vp, sz, vp], i),
        "tp_col_linear_noalloc": ([vp, vp, vp, i64, i64, i64, i, vp, vp], i),
        "tp_row_linear_partial_workspace_size": ([i64, i64, i64, psz], i),
        "tp_row_linear_partial": ([vp, vp, vp, i64, i64, i64, i, vp, sz, vp], i),
        "tp_row_linear_partial_chunked_workspace_size": ([i64, i64, i64, i32, psz], i),
        "tp_row_linear_partial_chunked": ([vp, vp, vp, i64, i64, i64, i, i32, ctypes.POINTER(vp), vp, sz, vp], i),
        "tp_mlp_shard_fwd_workspace_size": ([i64, i64, i64, i, psz], i),
        "tp_mlp_shard_fwd": ([vp, vp, vp, i64, i64, i64, i, vp, vp, vp, i, vp, sz, vp], i),
        "tp_mlp_shard_bwd_workspace_size": ([i64, i64, i64, i, psz], i),
        "tp_mlp_shard_bwd": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i, vp, vp, vp, vp, i, vp, sz, vp], i),
        "tp_col_linear_bwd_workspace_size": ([i64, i64, i64, psz], i),
        "tp_col_linear_bwd": ([vp, vp, vp, vp, vp, i64, i64, i64, i, vp, sz, vp], i),
        "tp_col_linear_bwd_chunked_workspace_size": ([i64, i64, i64, i32, psz], i),
        "tp_col_linear_bwd_chunked": ([vp, vp, vp, vp, vp, i64, i64, i64, i, i32, ctypes.POINTER(vp), vp, sz,
                                       vp], i),
        "tp_row_linear_bwd_workspace_size": ([i64, i64, i64, psz], i),
        "tp_row_linear_bwd": ([vp, vp, vp, vp, vp, i64, i64, i64, vp, sz, vp], i),
        "tp_qkv_regroup": ([vp, vp, i64, i32, i32, i32, i32, i32, vp], i),
        "tp_kv_grad_accumulate": ([vp, vp, i64, i32, i32, i32, i32, vp], i),
        "tp_vocab_embed_fwd": ([vp, vp, i64, i64, i64, i64, vp, i, vp], i),
        "tp_vocab_embed_bwd_workspace_size": ([i64, i64, i64, psz], i),
        "tp_vocab_embed_bwd": ([vp, vp, i64, i64, i64, i64, vp, vp, sz, vp], i),
        "tp_vocab_ce_fwd_workspace_size": ([i64, i64, i64, psz], i),
        "tp_vocab_ce_fwd": ([vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, sz, vp], i),
        "tp_vocab_ce_combine": ([vp, vp, vp, i32, i64, vp, vp, vp, vp], i),
        "tp_vocab_ce_bwd_workspace_size": ([i64, i64, i64, psz], i),
        "tp_vocab_ce_bwd": ([vp, vp, vp, i64, vp, vp, vp, i64, i64, i64, vp, vp, vp, i, vp, sz, vp], i),
        "tp_shard_shape": ([i32, ctypes.POINTER(i64), i32, i32, ctypes.POINTER(i64),
                            ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(i64),
                            ctypes.POINTER(i64), ctypes.POINTER(i64)], i),
    }
    for name, (args, res) in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _LIB = lib
    return lib


def _check(status: int):
    if status == 0:
        return
    msg = load().tp_last_error().decode(errors="replace")
    name = _STATUS.get(status, str(status))
    if status in (1, 2):
        raise ValueError(f"{name}: {msg}")
    if status == 3:
        raise NotImplementedError(f"{name}: {msg}")
    raise TPError(f"{name}: {msg}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t, name, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out(t, name, dtype, shape, like):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    return _dev(t, name, dtype, shape)


_bf16, _f32 = torch.bfloat16, torch.float32


def workspace_size(entry: str, *sizes) -> int:
    """Bytes of workspace the C call `entry` needs for these sizes on the
    current device (its host-only `<entry>_workspace_size` query)."""
    n = ctypes.c_size_t(0)
    _check(getattr(load(), entry + "_workspace_size")(*sizes, ctypes.byref(n)))
    return n.value


def _workspace(entry, sizes, like, stream, workspace=None):
    """(pointer, bytes, tensor) of the workspace for one call: the caller's
    `workspace` tensor if given (any dtype, contiguous, on the GPU), else a
    torch allocation of exactly the queried size (none if it is 0). A tensor
    allocated here is kept by the caching allocator for the stream the call
    runs on until that stream's work is done."""
    if workspace is not None:
        if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda and workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous GPU tensor")
        return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(), workspace
    n = workspace_size(entry, *sizes)
    if n == 0:
        return ctypes.c_void_p(0), 0, None
    ws = torch.empty(n, dtype=torch.uint8, device=like.device)
    if stream is not None and stream != torch.cuda.current_stream(like.device):
        ws.record_stream(stream)
    return ctypes.c_void_p(ws.data_ptr()), n, ws


def tp_version() -> int:
    return load().tp_version()


def tp_last_error() -> str:
    return load().tp_last_error().decode(errors="replace")


def tp_col_linear(X, W, act="none", Y=None, H_save=None, want_h=False, workspace=None, stream=None):
    """Y = act(X W) (SwiGLU: W = [gate | up]); returns (Y, H_save or None)."""
    lib = load()
    a = ACT[act]
    N, k = X.shape
    n_w = W.shape[1]
    n_out = n_w // 2 if act == "swiglu" else n_w
    _dev(X, "X", _bf16, (N, k))
    _dev(W, "W", _bf16, (k, n_w))
    Y = _out(Y, "Y", _bf16, (N, n_out), X)
    if want_h and H_save is None and act != "none":
        H_save = torch.empty((N, n_w), dtype=_bf16, device=X.device)
    if H_save is not None:
        _dev(H_save, "H_save", _bf16, (N, n_w))
    wp, wn, _keep = _workspace("tp_col_linear", (N, k, n_out, a), X, stream, workspace)
    _check(lib.tp_col_linear(_ptr(X), _ptr(W), _ptr(Y), N, k, n_out, a, _ptr(H_save), wp, wn,
                             _stream(stream)))
    return Y, H_save


def tp_col_linear_noalloc(X, W, Y, act="none", H_save=None, stream=None):
    """tp_col_linear with the library's device scratch instead of a workspace
    (the C call allocates nothing; Y and H_save must be given)."""
    lib = load()
    a = ACT[act]
    N, k = X.shape
    n_w = W.shape[1]
    n_out = n_w // 2 if act == "swiglu" else n_w
    _dev(X, "X", _bf16, (N, k))
    _dev(W, "W", _bf16, (k, n_w))
    _dev(Y, "Y", _bf16, (N, n_out))
    if H_save is not None:
        _dev(H_save, "H_save", _bf16, (N, n_w))
    _check(lib.tp_col_linear_noalloc(_ptr(X), _ptr(W), _ptr(Y), N, k, n_out, a, _ptr(H_save), _stream(stream)))
    return Y, H_save


def tp_row_linear_partial(Z, W, P=None, accumulate=False, workspace=None, stream=None):
    """P = Z W (or P += Z W), f32 partial sum; returns P."""
    lib = load()
    N, k_loc = Z.shape
    n = W.shape[1]
    _dev(Z, "Z", _bf16, (N, k_loc))
    _dev(W, "W", _bf16, (k_loc, n))
    P = _out(P, "P", _f32, (N, n), Z)
    wp, wn, _keep = _workspace("tp_row_linear_partial", (N, k_loc, n), Z, stream, workspace)
    _check(lib.tp_row_linear_partial(_ptr(Z), _ptr(W), _ptr(P), N, k_loc, n, int(bool(accumulate)), wp, wn,
                                     _stream(stream)))
    return P


def _events(events, nchunks):
    """None, or a C array of the HIP events of `events` (nchunks torch.cuda.Event)."""
    if events is None:
        return None
    if len(events) != nchunks:
        raise ValueError(f"{len(events)} events for {nchunks} chunks")
    for e in events:
        if not e.cuda_event:  # torch creates the HIP event on its first record
            e.record()
    return (ctypes.c_void_p * nchunks)(*[e.cuda_event for e in events])


def tp_row_linear_partial_chunked(Z, W, nchunks, P=None, accumulate=False, events=None, workspace=None,
                                  stream=None):
    """P = Z W (or P += Z W) in nchunks token-row chunks; events: None or nchunks
    torch.cuda.Event objects, each recorded after its chunk. Returns P."""
    lib = load()
    N, k_loc = Z.shape
    n = W.shape[1]
    _dev(Z, "Z", _bf16, (N, k_loc))
    _dev(W, "W", _bf16, (k_loc, n))
    P = _out(P, "P", _f32, (N, n), Z)
    ev = _events(events, nchunks)
    wp, wn, _keep = _workspace("tp_row_linear_partial_chunked", (N, k_loc, n, nchunks), Z, stream, workspace)
    _check(lib.tp_row_linear_partial_chunked(_ptr(Z), _ptr(W), _ptr(P), N, k_loc, n, int(bool(accumulate)),
                                             nchunks, ev, wp, wn, _stream(stream)))
    return P


def tp_mlp_shard_fwd(X, W_in, W_out, act, Z=None, H_save=None, P=None, want_h=True,
                     accumulate=False, workspace=None, stream=None):
    """One rank's MLP forward; returns (Z, H_save or None, P)."""
    lib = load()
    a = ACT[act]
    N, h = X.shape
    f = W_out.shape[0]
    n_w = 2 * f if act == "swiglu" else f
    _dev(X, "X", _bf16, (N, h))
    _dev(W_in, "W_in", _bf16, (h, n_w))
    _dev(W_out, "W_out", _bf16, (f, h))
    Z = _out(Z, "Z", _bf16, (N, f), X)
    if want_h and H_save is None:
        H_save = torch.empty((N, n_w), dtype=_bf16, device=X.device)
    if H_save is not None:
        _dev(H_save, "H_save", _bf16, (N, n_w))
    P = _out(P, "P", _f32, (N, h), X)
    wp, wn, _keep = _workspace("tp_mlp_shard_fwd", (N, h, f, a), X, stream, workspace)
    _check(lib.tp_mlp_shard_fwd(_ptr(X), _ptr(W_in), _ptr(W_out), N, h, f, a, _ptr(Z), _ptr(H_save),
                                _ptr(P), int(bool(accumulate)), wp, wn, _stream(stream)))
    return Z, H_save, P


def tp_mlp_shard_bwd(X, W_in, W_out, H_save, Z, dY, act, dH=None, dX_part=None, dW_in=None,
                     dW_out=None, accumulate=False, want=("dX_part", "dW_in", "dW_out"), workspace=None,
                     stream=None):
    """One rank's MLP backward; returns (dH, dX_part, dW_in, dW_out). Outputs
    not named in `want` are skipped (returned as None)."""
    lib = load()
    a = ACT[act]
    N, h = X.shape
    f = W_out.shape[0]
    n_w = 2 * f if act == "swiglu" else f
    _dev(X, "X", _bf16, (N, h))
    _dev(W_in, "W_in", _bf16, (h, n_w))
    _dev(W_out, "W_out", _bf16, (f, h))
    _dev(H_save, "H_save", _bf16, (N, n_w))
    _dev(Z, "Z", _bf16, (N, f))
    _dev(dY, "dY", _bf16, (N, h))
    unknown = set(want) - {"dX_part", "dW_in", "dW_out"}
    if unknown:
        raise ValueError(f"unknown outputs {sorted(unknown)}")
    dH = _out(dH, "dH", _bf16, (N, n_w), X)
    dX_part = _out(dX_part, "dX_part", _f32, (N, h), X) if "dX_part" in want else None
    dW_in = _out(dW_in, "dW_in", _f32, (h, n_w), X) if "dW_in" in want else None
    dW_out = _out(dW_out, "dW_out", _f32, (f, h), X) if "dW_out" in want else None
    wp, wn, _keep = _workspace("tp_mlp_shard_bwd", (N, h, f, a), X, stream, workspace)
    _check(lib.tp_mlp_shard_bwd(_ptr(X), _ptr(W_in), _ptr(W_out), _ptr(H_save), _ptr(Z), _ptr(dY),
                                N, h, f, a, _ptr(dH), _ptr(dX_part), _ptr(dW_in), _ptr(dW_out),
                                int(bool(accumulate)), wp, wn, _stream(stream)))
    return dH, dX_part, dW_in, dW_out


def tp_col_linear_bwd(X, W, dY, dX_part=None, dW=None, want_dx=True, want_dw=True,
                      accumulate=False, workspace=None, stream=None):
    """dX_part = dY W^T ({U}), dW = X^T dY; returns (dX_part, dW)."""
    lib = load()
    N, k = X.shape
    n = W.shape[1]
    _dev(X, "X", _bf16, (N, k))
    _dev(W, "W", _bf16, (k, n))
    _dev(dY, "dY", _bf16, (N, n))
    if want_dx:
        dX_part = _out(dX_part, "dX_part", _f32, (N, k), X)
    if want_dw:
        dW = _out(dW, "dW", _f32, (k, n), X)
    wp, wn, _keep = _workspace("tp_col_linear_bwd", (N, k, n), X, stream, workspace)
    _check(lib.tp_col_linear_bwd(_ptr(X), _ptr(W), _ptr(dY), _ptr(dX_part if want_dx else None),
                                 _ptr(dW if want_dw else None), N, k, n, int(bool(accumulate)), wp, wn,
                                 _stream(stream)))
    return (dX_part if want_dx else None), (dW if want_dw else None)


def tp_col_linear_bwd_chunked(X, W, dY, nchunks, dX_part=None, dW=None, want_dw=True, accumulate=False,
                              events=None, workspace=None, stream=None):
    """dX_part = dY W^T ({U}; accumulate adds) in nchunks token-row chunks,
    events[c] recorded after chunk c, then dW = X^T dY over all tokens;
    returns (dX_part, dW)."""
    lib = load()
    N, k = X.shape
    n = W.shape[1]
    _dev(X, "X", _bf16, (N, k))
    _dev(W, "W", _bf16, (k, n))
    _dev(dY, "dY", _bf16, (N, n))
    dX_part = _out(dX_part, "dX_part", _f32, (N, k), X)
    if want_dw:
        dW = _out(dW, "dW", _f32, (k, n), X)
    ev = _events(events, nchunks)
    wp, wn, _keep = _workspace("tp_col_linear_bwd_chunked", (N, k, n, nchunks), X, stream, workspace)
    _check(lib.tp_col_linear_bwd_chunked(_ptr(X), _ptr(W), _ptr(dY), _ptr(dX_part), _ptr(dW if want_dw else None),
                                         N, k, n, int(bool(accumulate)), nchunks, ev, wp, wn, _stream(stream)))
    return dX_part, (dW if want_dw else None)


def tp_row_linear_bwd(Z, W, dY, dZ=None, dW=None, want_dz=True, want_dw=True, workspace=None, stream=None):
    """dZ = dY W^T (bf16), dW = Z^T dY (f32); returns (dZ, dW)."""
    lib = load()
    N, k_loc = Z.shape
    n = W.shape[1]
    _dev(Z, "Z", _bf16, (N, k_loc))
    _dev(W, "W", _bf16, (k_loc, n))
    _dev(dY, "dY", _bf16, (N, n))
    if want_dz:
        dZ = _out(dZ, "dZ", _bf16, (N, k_loc), Z)
    if want_dw:
        dW = _out(dW, "dW", _f32, (k_loc, n), Z)
    wp, wn, _keep = _workspace("tp_row_linear_bwd", (N, k_loc, n), Z, stream, workspace)
    _check(lib.tp_row_linear_bwd(_ptr(Z), _ptr(W), _ptr(dY), _ptr(dZ if want_dz else None),
                                 _ptr(dW if want_dw else None), N, k_loc, n, wp, wn, _stream(stream)))
    return (dZ if want_dz else None), (dW if want_dw else None)


def regroup_width(n_h, n_kv, d_h, t):
    """Columns of one rank's W_r: its n_h/t query heads plus n_kv/t K and V heads
    (one replicated K and V head when n_kv < t); 0 for an invalid t."""
    if t <= 0 or n_h % t:
        return 0
    kv = n_kv // t if t <= n_kv else 1
    return (n_h // t + 2 * kv) * d_h


def tp_qkv_regroup(W_qkv, n_h, n_kv, d_h, t, rank, W_r=None, stream=None):
    """Rank-local [Q_r | K_r | V_r] columns of the fused QKV weight; returns W_r."""
    lib = load()
    h, width = W_qkv.shape
    if width != (n_h + 2 * n_kv) * d_h:
        raise ValueError(f"W_qkv width {width} != (n_h + 2 n_kv) d_h = {(n_h + 2 * n_kv) * d_h}")
    _dev(W_qkv, "W_qkv", _bf16, (h, width))
    out_w = regroup_width(n_h, n_kv, d_h, t)
    if W_r is None:
        W_r = torch.empty((h, out_w), dtype=_bf16, device=W_qkv.device)
    else:
        _dev(W_r, "W_r", _bf16, (h, out_w))
    _check(lib.tp_qkv_regroup(_ptr(W_qkv), _ptr(W_r), h, n_h, n_kv, d_h, t, rank, _stream(stream)))
    return W_r


def tp_kv_grad_accumulate(dW_dst, dW_src, n_h, n_kv, d_h, t, stream=None):
    """dW_dst[:, K|V columns] += dW_src[:, K|V columns] for two replica ranks'
    weight-gradient shards (n_kv < t); returns dW_dst."""
    lib = load()
    h = dW_dst.shape[0]
    w = (n_h // t + 2) * d_h if t > 0 else 0
    _dev(dW_dst, "dW_dst", _f32, (h, w))
    _dev(dW_src, "dW_src", _f32, (h, w))
    _check(lib.tp_kv_grad_accumulate(_ptr(dW_dst), _ptr(dW_src), h, n_h, n_kv, d_h, t, _stream(stream)))
    return dW_dst


def tp_vocab_ce_fwd(X, W_i, targets, vocab_start, workspace=None, stream=None):
    """One rank's local cross-entropy statistics; returns (m_i, s_i, zy_i), f32 [N]."""
    lib = load()
    N, h = X.shape
    v_loc = W_i.shape[1]
    _dev(X, "X", _bf16, (N, h))
    _dev(W_i, "W_i", _bf16, (h, v_loc))
    _dev(targets, "targets", torch.int32, (N,))
    m, s, zy = (torch.empty((N,), dtype=_f32, device=X.device) for _ in range(3))
    wp, wn, _keep = _workspace("tp_vocab_ce_fwd", (N, h, v_loc), X, stream, workspace)
    _check(lib.tp_vocab_ce_fwd(_ptr(X), _ptr(W_i), _ptr(targets), vocab_start, N, h, v_loc, _ptr(m), _ptr(s),
                               _ptr(zy), wp, wn, _stream(stream)))
    return m, s, zy


def tp_vocab_ce_combine(m_parts, s_parts, zy_parts, stream=None):
    """Stacked [t, N] local statistics -> (loss, m, S), f32 [N]."""
    lib = load()
    t, N = m_parts.shape
    for name, x in (("m_parts", m_parts), ("s_parts", s_parts), ("zy_parts", zy_parts)):
        _dev(x, name, _f32, (t, N))
    loss, m, S = (torch.empty((N,), dtype=_f32, device=m_parts.device) for _ in range(3))
    _check(lib.tp_vocab_ce_combine(_ptr(m_parts), _ptr(s_parts), _ptr(zy_parts), t, N, _ptr(loss), _ptr(m),
                                   _ptr(S), _stream(stream)))
    return loss, m, S


def tp_vocab_ce_bwd(X, W_i, targets, vocab_start, m, S, dloss, dZ=None, dX_part=None, dW_i=None,
                    accumulate=False, workspace=None, stream=None):
    """One rank's backward; returns (dZ, dX_part, dW_i)."""
    lib = load()
    N, h = X.shape
    v_loc = W_i.shape[1]
    _dev(X, "X", _bf16, (N, h))
    _dev(W_i, "W_i", _bf16, (h, v_loc))
    _dev(targets, "targets", torch.int32, (N,))
    for name, x in (("m", m), ("S", S), ("dloss", dloss)):
        _dev(x, name, _f32, (N,))
    dZ = _out(dZ, "dZ", _bf16, (N, v_loc), X)
    dX_part = _out(dX_part, "dX_part", _f32, (N, h), X)
    dW_i = _out(dW_i, "dW_i", _f32, (h, v_loc), X)
    wp, wn, _keep = _workspace("tp_vocab_ce_bwd", (N, h, v_loc), X, stream, workspace)
    _check(lib.tp_vocab_ce_bwd(_ptr(X), _ptr(W_i), _ptr(targets), vocab_start, _ptr(m), _ptr(S), _ptr(dloss), N,
                               h, v_loc, _ptr(dZ), _ptr(dX_part), _ptr(dW_i), int(bool(accumulate)), wp, wn,
                               _stream(stream)))
    return dZ, dX_part, dW_i


def tp_vocab_embed_fwd(ids, E_i, vocab_start, out=None, accumulate=False, stream=None):
    """Masked lookup of this rank's table rows; returns out bf16 [N, h]."""
    lib = load()
    N = ids.shape[0]
    v_loc, h = E_i.shape
    _dev(ids, "ids", torch.int32, (N,))
    _dev(E_i, "E_i", _bf16, (v_loc, h))
    if out is None:
        out = (torch.zeros if accumulate else torch.empty)((N, h), dtype=_bf16, device=E_i.device)
    else:
        _dev(out, "out", _bf16, (N, h))
    _check(lib.tp_vocab_embed_fwd(_ptr(ids), _ptr(E_i), vocab_start, N, v_loc, h, _ptr(out),
                                  int(bool(accumulate)), _stream(stream)))
    return out


def tp_vocab_embed_bwd(ids, dY, vocab_start, v_loc, dE_i=None, workspace=None, stream=None):
    """Gradient of this rank's table rows; returns dE_i f32 [v_loc, h]."""
    lib = load()
    N, h = dY.shape
    _dev(ids, "ids", torch.int32, (N,))
    _dev(dY, "dY", _f32, (N, h))
    dE_i = _out(dE_i, "dE_i", _f32, (v_loc, h), dY)
    wp, wn, _keep = _workspace("tp_vocab_embed_bwd", (N, v_loc, h), dY, stream, workspace)
    _check(lib.tp_vocab_embed_bwd(_ptr(ids), _ptr(dY), vocab_start, N, v_loc, h, _ptr(dE_i), wp, wn,
                                  _stream(stream)))
    return dE_i


def tp_shard_shape(shape, elem_bytes, axis_sizes, dim_axis_mask):
    """Host-only shard arithmetic; returns (local_shape, local_bytes, total_bytes)."""
    lib = load()
    nd, na = len(shape), len(axis_sizes)
    I64 = ctypes.c_int64
    sh = (I64 * max(nd, 1))(*shape)
    ax = (I64 * max(na, 1))(*axis_sizes)
    mk = (ctypes.c_uint32 * max(nd, 1))(*dim_axis_mask)
    loc = (I64 * max(nd, 1))()
    lb, tb = I64(), I64()
    _check(lib.tp_shard_shape(nd, sh, elem_bytes, na, ax, mk, loc, ctypes.byref(lb), ctypes.byref(tb)))
    return tuple(loc[i] for i in range(nd)), lb.value, tb.value
