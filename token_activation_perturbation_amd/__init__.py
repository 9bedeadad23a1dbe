"""Dust per-token zeroth-order weight-gradient estimator on MI355X (gfx950).

A thin ctypes binding over libdust.so: every function here only checks and
marshals arguments (torch device tensors -> device pointers, the current HIP
stream, a workspace tensor) and calls the C entry point of the same name
declared in include/dust.h.  All arithmetic runs in the library's kernels.
If libdust.so is missing the calls raise; nothing falls back to the CPU.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["DustError", "dust_workspace_bytes", "dust_workspace_bytes_seq", "dust_validate", "dust_estimate",
           "dust_validate_local", "dust_estimate_local", "dust_validate_head",
           "dust_estimate_head", "dust_embedding_workspace_bytes",
           "dust_reassemble_workspace_bytes", "dust_validate_embedding", "dust_estimate_embedding",
           "dust_validate_reassemble", "dust_reassemble_embedding", "dust_noise_fill",
           "dust_estimate_noalloc", "dust_noalloc_workspace_capacity",
           "dust_attention_workspace_bytes", "dust_validate_attention", "dust_estimate_attention",
           "dust_set_timing_events", "dust_profile_begin", "dust_profile_end", "dust_last_error",
           "library_path", "DUST_F32", "DUST_BF16", "ATTENTION_SITES"]

DUST_F32 = 0
DUST_BF16 = 1
# dust_attn_site_t: which of the cached queries, keys and values is jittered
ATTENTION_SITES = {"query": 0, "key": 1, "value": 2}
_STATUS = {0: "DUST_OK", 1: "DUST_ERR_INVALID_ARG", 2: "DUST_ERR_UNSUPPORTED",
           3: "DUST_ERR_WORKSPACE", 4: "DUST_ERR_HIP"}
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdust.so")
_lib = None


class DustError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m token_activation_perturbation_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                             ctypes.c_float, ctypes.c_size_t)
    lib.dust_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.dust_workspace_bytes.restype = sz
    lib.dust_workspace_bytes_seq.argtypes = [i64, i64, i64, i64, i32, f32, i32, i32]
    lib.dust_workspace_bytes_seq.restype = sz
    lib.dust_validate.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, f32, i32,
                                  vp, vp, sz]
    lib.dust_validate.restype = ctypes.c_int
    lib.dust_estimate.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, f32,
                                  ctypes.c_uint64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dust_estimate.restype = ctypes.c_int
    lib.dust_estimate_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, f32,
                                          ctypes.c_uint64, i32, vp, vp, vp, vp, vp, vp]
    lib.dust_estimate_noalloc.restype = ctypes.c_int
    lib.dust_noalloc_workspace_capacity.argtypes = []
    lib.dust_noalloc_workspace_capacity.restype = sz
    lib.dust_validate_local.argtypes = [vp, vp, i64, i64, i64, i64, i32, i32, f32, f32, i32,
                                        vp, vp, sz]
    lib.dust_validate_local.restype = ctypes.c_int
    lib.dust_estimate_local.argtypes = [vp, vp, i64, i64, i64, i64, i32, i32, f32, f32,
                                        ctypes.c_uint64, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.dust_estimate_local.restype = ctypes.c_int
    lib.dust_validate_head.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, f32, i32, vp, vp,
                                       sz]
    lib.dust_validate_head.restype = ctypes.c_int
    lib.dust_estimate_head.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, f32,
                                       ctypes.c_uint64, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.dust_estimate_head.restype = ctypes.c_int
    lib.dust_embedding_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32]
    lib.dust_embedding_workspace_bytes.restype = sz
    lib.dust_reassemble_workspace_bytes.argtypes = [i64, i64, i64]
    lib.dust_reassemble_workspace_bytes.restype = sz
    lib.dust_validate_embedding.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, f32,
                                            i32, f32, vp, vp, sz]
    lib.dust_validate_embedding.restype = ctypes.c_int
    lib.dust_estimate_embedding.argtypes = [vp, vp, vp, i64, i64, i64, i64, i32, i32, f32, f32,
                                            ctypes.c_uint64, i32, f32, vp, vp, vp, vp, vp, vp,
                                            sz, vp]
    lib.dust_estimate_embedding.restype = ctypes.c_int
    lib.dust_validate_reassemble.argtypes = [vp, vp, i64, i64, i64, f32, vp, vp, sz]
    lib.dust_validate_reassemble.restype = ctypes.c_int
    lib.dust_reassemble_embedding.argtypes = [vp, vp, i64, i64, i64, f32, vp, vp, sz, vp]
    lib.dust_reassemble_embedding.restype = ctypes.c_int
    lib.dust_attention_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32, i32]
    lib.dust_attention_workspace_bytes.restype = sz
    lib.dust_validate_attention.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                                            i32, i32, f32, f32, i32, vp, vp, sz]
    lib.dust_validate_attention.restype = ctypes.c_int
    lib.dust_estimate_attention.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                                            i32, i32, f32, f32, ctypes.c_uint64, i32, vp, vp,
                                            vp, vp, vp, sz, vp]
    lib.dust_estimate_attention.restype = ctypes.c_int
    lib.dust_noise_fill.argtypes = [ctypes.c_uint64, i64, i64, i64, i64, i64, vp, vp, vp]
    lib.dust_noise_fill.restype = ctypes.c_int
    vpp = ctypes.POINTER(ctypes.c_void_p)
    lib.dust_set_timing_events.argtypes = [vpp, vpp, i32]
    lib.dust_set_timing_events.restype = ctypes.c_int
    lib.dust_profile_begin.argtypes = [i32]
    lib.dust_profile_begin.restype = ctypes.c_int
    lib.dust_profile_end.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(f32),
                                     ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double), i32,
                                     ctypes.POINTER(i32)]
    lib.dust_profile_end.restype = ctypes.c_int
    lib.dust_last_error.argtypes = []
    lib.dust_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def dust_last_error() -> str:
    return _load().dust_last_error().decode()


def _check(status: int):
    if status != 0:
        raise DustError(status, dust_last_error())


def dust_workspace_bytes(T: int, d_in: int, d_out: int, K: int, antithetic: bool,
                         dtype: int) -> int:
    return int(_load().dust_workspace_bytes(T, d_in, d_out, K, int(bool(antithetic)), dtype))


def dust_workspace_bytes_seq(T: int, d_in: int, d_out: int, seq_len: int, K: int, gamma: float,
                             antithetic: bool, dtype: int) -> int:
    """Workspace bytes with which a gamma > 0 call with antithetic pairs
    generates each noise value once (equal to dust_workspace_bytes where
    that path does not apply to these sizes)."""
    return int(_load().dust_workspace_bytes_seq(T, d_in, d_out, seq_len, K, gamma,
                                                int(bool(antithetic)), dtype))


def dust_validate(X_ptr, W_ptr, target_ptr, T, d_in, d_out, seq_len, dtype, K, sigma, gamma,
                  antithetic, G_ptr, workspace_ptr, workspace_bytes) -> int:
    """Raw host-side validation (no device memory touched); returns the status."""
    return int(_load().dust_validate(X_ptr, W_ptr, target_ptr, T, d_in, d_out, seq_len, dtype,
                                     K, sigma, gamma, int(bool(antithetic)), G_ptr,
                                     workspace_ptr, workspace_bytes))


def dust_validate_local(X_ptr, E_ptr, T, d_in, d_out, seq_len, dtype, K, sigma, gamma,
                        antithetic, G_ptr, workspace_ptr, workspace_bytes) -> int:
    """Raw host-side validation of dust_estimate_local's arguments; returns the status."""
    return int(_load().dust_validate_local(X_ptr, E_ptr, T, d_in, d_out, seq_len, dtype, K,
                                           sigma, gamma, int(bool(antithetic)), G_ptr,
                                           workspace_ptr, workspace_bytes))


def dust_validate_head(X_ptr, W_ptr, labels_ptr, T, d_in, V, dtype, K, sigma, antithetic,
                       G_ptr, workspace_ptr, workspace_bytes) -> int:
    """Raw host-side validation of dust_estimate_head's arguments; returns the status."""
    return int(_load().dust_validate_head(X_ptr, W_ptr, labels_ptr, T, d_in, V, dtype, K, sigma,
                                          int(bool(antithetic)), G_ptr, workspace_ptr,
                                          workspace_bytes))


def _output_getter(res: dict, dev):
    """A function (name, shape) -> the fp32 output tensor res[name], created
    on `dev` when absent, else checked (contiguous float32 of that shape)."""
    import torch

    def _get(name, shape):
        t = res.get(name)
        if t is None:
            t = torch.empty(shape, dtype=torch.float32, device=dev)
            res[name] = t
        elif (tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous()
              or t.device != dev):
            raise ValueError(f"out[{name!r}] must be a contiguous float32 {tuple(shape)} "
                             f"tensor on {dev}")
        return t
    return _get


def _check_tensors(dev, **tensors):
    """Each given tensor (None skipped) must be a contiguous device tensor on
    `dev` (the first tensor's device when `dev` is None); returns the device."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")
    return dev


def _workspace(workspace, need: int, dev):
    """The caller's workspace (a contiguous device tensor on `dev`; its byte
    size is checked by the library) or a new uint8 tensor of `need` bytes;
    returns (tensor, its size in bytes)."""
    import torch
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _check_tensors(dev, workspace=workspace)
    return workspace, workspace.numel() * workspace.element_size()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DUST_BF16
    if t.dtype == torch.float32:
        return DUST_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bfloat16 or float32")


def _stream_ptr(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def dust_estimate(X, W, target, *, K: int, sigma: float, gamma: float, seed: int,
                  antithetic: bool, seq_len: int, want_loss: bool = False,
                  want_rho: bool = False, want_reward: bool = False, want_g: bool = False,
                  out: dict | None = None, workspace=None):
    """Enqueue dust_estimate on the current stream of X's device.

    X [T,d_in], W [d_out,d_in], target [T,d_out]: contiguous device tensors,
    all bfloat16 or all float32.  Returns a dict of fp32 device tensors: "G_W"
    [d_out,d_in] and the requested optional outputs "loss" [T], "rho" [T,K],
    "reward" [T,K], "g" [T,d_out].  ``out`` may supply preallocated output
    tensors and ``workspace`` a uint8 device tensor of dust_workspace_bytes.
    """
    dev = _check_tensors(None, X=X, W=W, target=target)
    if not (X.dtype == W.dtype == target.dtype):
        raise TypeError("X, W and target must share one dtype")
    if X.dim() != 2 or W.dim() != 2 or target.dim() != 2:
        raise ValueError("X, W and target must be 2-D")
    T, d_in = X.shape
    d_out = W.shape[0]
    if W.shape[1] != d_in or tuple(target.shape) != (T, d_out):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}, "
                         f"target {tuple(target.shape)}")
    dt = _dtype_code(X)
    res = dict(out or {})
    _get = _output_getter(res, dev)

    G = _get("G_W", (d_out, d_in))
    loss = _get("loss", (T,)) if want_loss else None
    rho = _get("rho", (T, K)) if want_rho else None
    reward = _get("reward", (T, K)) if want_reward else None
    g = _get("g", (T, d_out)) if want_g else None
    # per-draw outputs need the two-pass path: its workspace suffices then
    need = (dust_workspace_bytes(T, d_in, d_out, K, antithetic, dt) if want_rho or want_reward
            else dust_workspace_bytes_seq(T, d_in, d_out, seq_len, K, gamma, antithetic, dt))
    ws, ws_bytes = _workspace(workspace, need, dev)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    status = _load().dust_estimate(
        X.data_ptr(), W.data_ptr(), target.data_ptr(), T, d_in, d_out, seq_len, dt, K,
        sigma, gamma, ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), int(bool(antithetic)),
        G.data_ptr(), ptr(loss), ptr(rho), ptr(reward), ptr(g), ws.data_ptr(), ws_bytes,
        _stream_ptr(dev))
    _check(status)
    return res


def dust_noalloc_workspace_capacity() -> int:
    """Bytes of the static workspace dust_estimate_noalloc runs in."""
    return int(_load().dust_noalloc_workspace_capacity())


def dust_estimate_noalloc(X, W, target, *, K: int, sigma: float, gamma: float, seed: int,
                          antithetic: bool, seq_len: int, want_loss: bool = False,
                          want_rho: bool = False, want_reward: bool = False,
                          want_g: bool = False, out: dict | None = None):
    """Enqueue dust_estimate_noalloc (dust_estimate in the library's static
    workspace: the library allocates nothing) on the current stream of X's
    device.  Arguments and outputs as for dust_estimate, without a
    workspace; pass every output in ``out`` for a call that allocates
    nothing at all (missing ones are created here, before the call)."""
    dev = _check_tensors(None, X=X, W=W, target=target)
    if not (X.dtype == W.dtype == target.dtype):
        raise TypeError("X, W and target must share one dtype")
    if X.dim() != 2 or W.dim() != 2 or target.dim() != 2:
        raise ValueError("X, W and target must be 2-D")
    T, d_in = X.shape
    d_out = W.shape[0]
    if W.shape[1] != d_in or tuple(target.shape) != (T, d_out):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}, "
                         f"target {tuple(target.shape)}")
    dt = _dtype_code(X)
    res = dict(out or {})
    _get = _output_getter(res, dev)
    G = _get("G_W", (d_out, d_in))
    loss = _get("loss", (T,)) if want_loss else None
    rho = _get("rho", (T, K)) if want_rho else None
    reward = _get("reward", (T, K)) if want_reward else None
    g = _get("g", (T, d_out)) if want_g else None
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    status = _load().dust_estimate_noalloc(
        X.data_ptr(), W.data_ptr(), target.data_ptr(), T, d_in, d_out, seq_len, dt, K,
        sigma, gamma, ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), int(bool(antithetic)),
        G.data_ptr(), ptr(loss), ptr(rho), ptr(reward), ptr(g), _stream_ptr(dev))
    _check(status)
    return res


def dust_estimate_local(X, E, *, K: int, sigma: float, gamma: float, seed: int,
                        antithetic: bool, seq_len: int, want_rho: bool = False,
                        want_reward: bool = False, want_g: bool = False,
                        out: dict | None = None, workspace=None):
    """Enqueue dust_estimate_local (local scoring against the error estimate
    E) on the current stream of E's device.

    X [T,d_in] (bfloat16 or float32) and E [T,d_out] (float32): contiguous
    device tensors; X may be None for a site with no input matrix (a value
    embedding): then no G_W is formed, and g (want_g) is the result.  Returns
    a dict of fp32 device tensors: "G_W" [d_out,d_in] (with X) and the
    requested optional outputs "rho" [T,K] (the scores), "reward" [T,K],
    "g" [T,d_out].  ``out`` and ``workspace`` as for dust_estimate.
    """
    import torch
    dev = _check_tensors(None, E=E, X=X)
    if E.dtype != torch.float32:
        raise TypeError("E must be float32")
    if E.dim() != 2 or (X is not None and (X.dim() != 2 or X.shape[0] != E.shape[0])):
        raise ValueError(f"shape mismatch: X {None if X is None else tuple(X.shape)}, "
                         f"E {tuple(E.shape)}")
    T, d_out = E.shape
    d_in = 1 if X is None else X.shape[1]
    dt = DUST_F32 if X is None else _dtype_code(X)
    res = dict(out or {})
    _get = _output_getter(res, dev)
    G = None if X is None else _get("G_W", (d_out, d_in))
    rho = _get("rho", (T, K)) if want_rho else None
    reward = _get("reward", (T, K)) if want_reward else None
    g = _get("g", (T, d_out)) if want_g else None
    need = (dust_workspace_bytes(T, d_in, d_out, K, antithetic, dt) if want_rho or want_reward
            else dust_workspace_bytes_seq(T, d_in, d_out, seq_len, K, gamma, antithetic, dt))
    ws, ws_bytes = _workspace(workspace, need, dev)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    status = _load().dust_estimate_local(
        ptr(X), E.data_ptr(), T, d_in, d_out, seq_len, dt, K, sigma, gamma,
        ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), int(bool(antithetic)), ptr(G),
        ptr(rho), ptr(reward), ptr(g), ws.data_ptr(), ws_bytes, _stream_ptr(dev))
    _check(status)
    return res


def dust_attention_workspace_bytes(T: int, d_in: int, heads: int, d_head: int, seq_len: int,
                                   site: str, K: int, antithetic: bool) -> int:
    """Bytes of workspace dust_estimate_attention needs (0 if invalid)."""
    return int(_load().dust_attention_workspace_bytes(T, d_in, heads, d_head, seq_len,
                                                      ATTENTION_SITES[site], K,
                                                      int(bool(antithetic)), DUST_BF16))


def dust_validate_attention(X_ptr, Q_ptr, K_ptr, V_ptr, E_ptr, T, d_in, heads, d_head, seq_len,
                            site, dtype, K, sigma, gamma, antithetic, G_ptr, workspace_ptr,
                            workspace_bytes) -> int:
    """Raw host-side validation of dust_estimate_attention's arguments (site
    as its integer code); returns the status."""
    return int(_load().dust_validate_attention(X_ptr, Q_ptr, K_ptr, V_ptr, E_ptr, T, d_in, heads,
                                               d_head, seq_len, site, dtype, K, sigma, gamma,
                                               int(bool(antithetic)), G_ptr, workspace_ptr,
                                               workspace_bytes))


def dust_estimate_attention(X, q, k, v, E, *, heads: int, site: str, K: int, sigma: float,
                            gamma: float, seed: int, antithetic: bool, seq_len: int,
                            want_rho: bool = False, want_reward: bool = False,
                            want_g: bool = False, out: dict | None = None, workspace=None):
    """Enqueue dust_estimate_attention (scores through a recomputed causal
    attention) on the current stream of q's device.

    q, k, v [T, heads*d_head] (bfloat16): the block's cached queries, keys
    and values; E [T, heads*d_head] (float32): the error estimate of the
    attention output; site: "query", "key" or "value" (the one jittered); X
    [T, d_in] (bfloat16) the block's input, or None (no G_W).  Returns a dict
    of fp32 device tensors: "G_W" [heads*d_head, d_in] (with X) and the
    requested "rho" [T,K] (the scores), "reward" [T,K], "g" [T,heads*d_head].
    """
    import torch
    dev = _check_tensors(None, q=q, k=k, v=v, E=E, X=X)
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16) or (
            X is not None and X.dtype != torch.bfloat16):
        raise TypeError("q, k, v and X must be bfloat16")
    if E.dtype != torch.float32:
        raise TypeError("E must be float32")
    if q.dim() != 2 or tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape) \
            or tuple(E.shape) != tuple(q.shape) or q.shape[1] % heads != 0:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}, E {tuple(E.shape)}, heads {heads}")
    T, D = q.shape
    if X is not None and (X.dim() != 2 or X.shape[0] != T):
        raise ValueError(f"X {tuple(X.shape)} must be [T={T}, d_in]")
    d_in = 1 if X is None else X.shape[1]
    res = dict(out or {})
    _get = _output_getter(res, dev)
    G = None if X is None else _get("G_W", (D, d_in))
    rho = _get("rho", (T, K)) if want_rho else None
    reward = _get("reward", (T, K)) if want_reward else None
    g = _get("g", (T, D)) if want_g else None
    need = dust_attention_workspace_bytes(T, d_in, heads, D // heads, seq_len, site, K,
                                          antithetic)
    ws, ws_bytes = _workspace(workspace, need, dev)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    status = _load().dust_estimate_attention(
        ptr(X), q.data_ptr(), k.data_ptr(), v.data_ptr(), E.data_ptr(), T, d_in, heads,
        D // heads, seq_len, ATTENTION_SITES[site], DUST_BF16, K, sigma, gamma,
        ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), int(bool(antithetic)), ptr(G), ptr(rho),
        ptr(reward), ptr(g), ws.data_ptr(), ws_bytes, _stream_ptr(dev))
    _check(status)
    return res


def dust_estimate_head(X, W, labels, *, K: int, sigma: float, seed: int, antithetic: bool,
                       want_loss: bool = False, want_rho: bool = False, want_g: bool = False,
                       out: dict | None = None, workspace=None):
    """Enqueue dust_estimate_head (the cross-entropy head, jittered one
    256-column slab of the vocabulary at a time) on the current stream of
    X's device.

    X [T,d_in] and W [V,d_in] (both bfloat16 or both float32) and labels [T]
    (int32): contiguous device tensors; V a multiple of 256.  Returns a dict
    of fp32 device tensors: "G_W" [V,d_in] and the requested optional outputs
    "loss" [T] (clean cross-entropy), "rho" [T,V//256,K] (loss reductions per
    slab and draw), "g" [T,V].  ``out`` and ``workspace`` as for
    dust_estimate.
    """
    import torch
    dev = _check_tensors(None, X=X, W=W, labels=labels)
    if X.dtype != W.dtype:
        raise TypeError("X and W must share a dtype")
    if labels.dtype != torch.int32:
        raise TypeError("labels must be int32")
    if X.dim() != 2 or W.dim() != 2 or labels.dim() != 1 or X.shape[1] != W.shape[1] \
            or labels.shape[0] != X.shape[0]:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}, "
                         f"labels {tuple(labels.shape)}")
    T, d_in = X.shape
    V = W.shape[0]
    dt = _dtype_code(X)
    res = dict(out or {})
    _get = _output_getter(res, dev)

    G = _get("G_W", (V, d_in))
    loss = _get("loss", (T,)) if want_loss else None
    rho = _get("rho", (T, V // 256, K)) if want_rho else None
    g = _get("g", (T, V)) if want_g else None
    ws, ws_bytes = _workspace(workspace, dust_workspace_bytes(T, d_in, V, K, antithetic, dt), dev)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    status = _load().dust_estimate_head(
        X.data_ptr(), W.data_ptr(), labels.data_ptr(), T, d_in, V, dt, K, sigma,
        ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), int(bool(antithetic)), G.data_ptr(),
        ptr(loss), ptr(rho), ptr(g), ws.data_ptr(), ws_bytes, _stream_ptr(dev))
    _check(status)
    return res


def dust_embedding_workspace_bytes(T: int, V: int, d: int, K: int, antithetic: bool,
                                   dtype: int) -> int:
    return int(_load().dust_embedding_workspace_bytes(T, V, d, K, int(bool(antithetic)), dtype))


def dust_reassemble_workspace_bytes(T: int, V: int, d: int) -> int:
    return int(_load().dust_reassemble_workspace_bytes(T, V, d))


def dust_validate_embedding(table_ptr, ids_ptr, target_ptr, T, V, d, seq_len, dtype, K, sigma,
                            gamma, antithetic, scale, G_ptr, workspace_ptr,
                            workspace_bytes) -> int:
    """Raw host-side validation of dust_estimate_embedding's arguments; returns the status."""
    return int(_load().dust_validate_embedding(table_ptr, ids_ptr, target_ptr, T, V, d, seq_len,
                                               dtype, K, sigma, gamma, int(bool(antithetic)),
                                               scale, G_ptr, workspace_ptr, workspace_bytes))


def dust_validate_reassemble(ids_ptr, g_ptr, T, V, d, scale, G_ptr, workspace_ptr,
                             workspace_bytes) -> int:
    """Raw host-side validation of dust_reassemble_embedding's arguments; returns the status."""
    return int(_load().dust_validate_reassemble(ids_ptr, g_ptr, T, V, d, scale, G_ptr,
                                                workspace_ptr, workspace_bytes))


def dust_estimate_embedding(table, ids, target, *, K: int, sigma: float, gamma: float, seed: int,
                            antithetic: bool, seq_len: int, scale: float = 1.0,
                            want_loss: bool = False, want_rho: bool = False,
                            want_reward: bool = False, want_g: bool = False,
                            out: dict | None = None, workspace=None):
    """Enqueue dust_estimate_embedding (a token embedding: the gather of
    table rows, the estimator, the scatter-add of g by id times `scale`) on
    the current stream of the table's device.

    table [V,d] and target [T,d] (both bfloat16 or both float32), ids [T]
    (int32): contiguous device tensors.  Returns a dict of fp32 device
    tensors: "G_E" [V,d] and the requested optional outputs "loss" [T],
    "rho" [T,K], "reward" [T,K], "g" [T,d].  ``workspace``: a uint8 device
    tensor of dust_embedding_workspace_bytes.
    """
    import torch
    dev = _check_tensors(None, table=table, ids=ids, target=target)
    if table.dtype != target.dtype:
        raise TypeError("table and target must share one dtype")
    if ids.dtype != torch.int32:
        raise TypeError("ids must be int32")
    if table.dim() != 2 or ids.dim() != 1 or target.dim() != 2 \
            or tuple(target.shape) != (ids.shape[0], table.shape[1]):
        raise ValueError(f"shape mismatch: table {tuple(table.shape)}, ids {tuple(ids.shape)}, "
                         f"target {tuple(target.shape)}")
    V, d = table.shape
    T = ids.shape[0]
    dt = _dtype_code(table)
    res = dict(out or {})
    _get = _output_getter(res, dev)
    G = _get("G_E", (V, d))
    loss = _get("loss", (T,)) if want_loss else None
    rho = _get("rho", (T, K)) if want_rho else None
    reward = _get("reward", (T, K)) if want_reward else None
    g = _get("g", (T, d)) if want_g else None
    ws, ws_bytes = _workspace(workspace,
                              dust_embedding_workspace_bytes(T, V, d, K, antithetic, dt), dev)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    status = _load().dust_estimate_embedding(
        table.data_ptr(), ids.data_ptr(), target.data_ptr(), T, V, d, seq_len, dt, K, sigma,
        gamma, ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), int(bool(antithetic)), scale,
        G.data_ptr(), ptr(loss), ptr(rho), ptr(reward), ptr(g), ws.data_ptr(), ws_bytes,
        _stream_ptr(dev))
    _check(status)
    return res


def dust_reassemble_embedding(ids, g, V: int, *, scale: float = 1.0, out=None, workspace=None):
    """Enqueue dust_reassemble_embedding: G_E [V,d] = scale * the sum of the
    rows of g [T,d] (float32) whose ids [T] (int32) select row v, in a fixed
    order.  Returns G_E (``out`` if given: a contiguous float32 [V,d] tensor)."""
    import torch
    dev = _check_tensors(None, g=g, ids=ids)
    if ids.dtype != torch.int32 or g.dtype != torch.float32:
        raise TypeError("ids must be int32 and g float32")
    if ids.dim() != 1 or g.dim() != 2 or g.shape[0] != ids.shape[0]:
        raise ValueError(f"shape mismatch: ids {tuple(ids.shape)}, g {tuple(g.shape)}")
    T, d = g.shape
    G = _output_getter({} if out is None else {"G_E": out}, dev)("G_E", (V, d))
    ws, ws_bytes = _workspace(workspace, dust_reassemble_workspace_bytes(T, V, d), dev)
    status = _load().dust_reassemble_embedding(ids.data_ptr(), g.data_ptr(), T, V, d, scale,
                                               G.data_ptr(), ws.data_ptr(), ws_bytes,
                                               _stream_ptr(dev))
    _check(status)
    return G


def dust_noise_fill(seed: int, n0: int, n_cnt: int, t0: int, t_cnt: int, d_out: int, *,
                    words: bool = True, gauss: bool = True, device="cuda"):
    """The estimator's noise written out: words [n_cnt,t_cnt,4*ceil(d_out/4)]
    (int32 tensor holding the uint32 bits) and Gaussians [n_cnt,t_cnt,d_out]
    (float32), on the current stream of `device`."""
    import torch
    nq = (d_out + 3) // 4
    w = torch.empty((n_cnt, t_cnt, 4 * nq), dtype=torch.int32, device=device) if words else None
    g = torch.empty((n_cnt, t_cnt, d_out), dtype=torch.float32, device=device) if gauss else None
    status = _load().dust_noise_fill(
        ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), n0, n_cnt, t0, t_cnt, d_out,
        None if w is None else w.data_ptr(), None if g is None else g.data_ptr(),
        _stream_ptr(torch.device(device)))
    _check(status)
    return w, g


def dust_set_timing_events(starts, stops) -> None:
    """Register event pairs (torch.cuda.Event with enable_timing=True, already
    recorded once so their HIP events exist) that the dispatch of the next
    estimate calls' noise kernel stamps at its start and end, pair i on call
    i.  Pass empty lists to turn the hook off."""
    n = len(starts)
    if len(stops) != n:
        raise ValueError("starts and stops must have the same length")
    if n == 0:
        _check(_load().dust_set_timing_events(None, None, 0))
        return
    arr = ctypes.c_void_p * n
    handles_s = [e.cuda_event for e in starts]
    handles_e = [e.cuda_event for e in stops]
    if not all(handles_s) or not all(handles_e):
        raise ValueError("record every event once before registering it")
    _check(_load().dust_set_timing_events(arr(*handles_s), arr(*handles_e), n))


_profile_cap = 0


def dust_profile_begin(max_launches: int) -> None:
    """Turn on the per-launch profile for this thread: each kernel launch of
    the next library calls (up to max_launches) is stamped by its own pair
    of library-owned events."""
    global _profile_cap
    _check(_load().dust_profile_begin(int(max_launches)))
    _profile_cap = int(max_launches)


def dust_profile_end() -> list:
    """Turn the profile off (waiting for the recorded launches) and return
    one dict per recorded launch, in launch order: kernel (stage name), ms,
    flops (the method's MFMA flops), bytes (least HBM bytes it must move)."""
    global _profile_cap
    cap = max(_profile_cap, 1)
    _profile_cap = 0
    lib = _load()
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    flops = (ctypes.c_double * cap)()
    nbytes = (ctypes.c_double * cap)()
    count = ctypes.c_int32(0)
    _check(lib.dust_profile_end(names, ms, flops, nbytes, cap, ctypes.byref(count)))
    n = min(cap, count.value)
    return [{"kernel": names[i].decode(), "ms": float(ms[i]), "flops": float(flops[i]),
             "bytes": float(nbytes[i])} for i in range(n)]
