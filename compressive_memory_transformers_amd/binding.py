"""ctypes binding of libinfini_attn.so (include/infini_attn.h).

Argument marshalling only: shapes are read off torch tensors, data pointers and
the current HIP stream are passed to the C entry points, and a non-OK status
becomes an exception. Every step of the computation runs in the library's HIP
kernels; nothing here computes a result, and there is no fallback: if the
library is missing or a call fails, an error is raised.
"""

import ctypes
import os

import torch

from .build import LIB_PATH

RULES = {"linear": 0, "delta": 1}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_p = ctypes.c_void_p
_c_size = ctypes.c_size_t

# (name, restype, argtypes) of every entry point the header declares
SIGNATURES = {
    "infini_attn_workspace_size": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32, ctypes.POINTER(_c_size), ctypes.POINTER(_c_size)]),
    "infini_attn_forward": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]),
    "infini_attn_forward_noalloc": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p]),
    "infini_attn_workspace_size_kv": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32, ctypes.POINTER(_c_size), ctypes.POINTER(_c_size)]),
    "infini_attn_forward_kv": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]),
    "infini_attn_forward_kv_timed": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]
        + [ctypes.POINTER(_c_p), _c_i32]),
    "infini_attn_forward_timed": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]
        + [ctypes.POINTER(_c_p), _c_i32]),
    "infini_attn_forward_train": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32] + [_c_p] * 10 + [_c_p, _c_size, _c_p]),
    "infini_attn_forward_train_kv": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32] + [_c_p] * 10 + [_c_p, _c_size, _c_p]),
    "infini_attn_backward_workspace_size_kv": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32, ctypes.POINTER(_c_size)]),
    "infini_attn_backward_kv": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32] + [_c_p] * 17 + [_c_p, _c_size, _c_p]),
    "infini_attn_backward_workspace_size": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32, ctypes.POINTER(_c_size)]),
    "infini_attn_backward": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32] + [_c_p] * 17 + [_c_p, _c_size, _c_p]),
    "infini_attn_decode_workspace_size": (
        _c_i32, [_c_i64] * 5 + [_c_i32, _c_i32, ctypes.POINTER(_c_size)]),
    "infini_attn_decode_step": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]),
    "infini_attn_decode_workspace_size_kv": (
        _c_i32, [_c_i64] * 6 + [_c_i32, _c_i32, ctypes.POINTER(_c_size)]),
    "infini_attn_decode_step_kv": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]),
    "infini_attn_block_workspace_size": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32, ctypes.POINTER(_c_size)]),
    "infini_attn_block_forward": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]),
    "infini_attn_block_workspace_size_kv": (
        _c_i32, [_c_i64] * 8 + [_c_i32, _c_i32, ctypes.POINTER(_c_size)]),
    "infini_attn_block_forward_kv": (
        _c_i32, [_c_i64] * 8 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]),
    "infini_attn_block_forward_timed": (
        _c_i32, [_c_i64] * 7 + [_c_i32, _c_i32] + [_c_p] * 9 + [_c_p, _c_size, _c_p]
        + [ctypes.POINTER(_c_p), _c_i32]),
    "infini_attn_status_string": (ctypes.c_char_p, [_c_i32]),
    "infini_attn_error_string": (ctypes.c_char_p, [_c_i32]),
    "infini_attn_version": (_c_i32, []),
}

_lib = None


class InfiniAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path():
    return os.environ.get("INFINI_ATTN_LIB", LIB_PATH)


def load_library():
    """Load libinfini_attn.so once; raise ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python compressive_memory_transformers_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status):
    return load_library().infini_attn_status_string(int(status)).decode()


def version():
    return int(load_library().infini_attn_version())


def workspace_size(B, Hq, Hkv, L, d, seg_len, rule, dtype):
    """(full_bytes, min_bytes) of the workspace for these sizes."""
    lib = load_library()
    full, least = _c_size(0), _c_size(0)
    st = lib.infini_attn_workspace_size(B, Hq, Hkv, L, d, seg_len, RULES[rule], DTYPES[dtype],
                                        ctypes.byref(full), ctypes.byref(least))
    if st != 0:
        raise InfiniAttnError(st, "infini_attn_workspace_size")
    return int(full.value), int(least.value)


def workspace_size_kv(B, Hq, Hkv, L, d_key, d_value, seg_len, rule, dtype):
    """(full_bytes, min_bytes) of the workspace with separate key and value widths."""
    lib = load_library()
    full, least = _c_size(0), _c_size(0)
    st = lib.infini_attn_workspace_size_kv(B, Hq, Hkv, L, d_key, d_value, seg_len, RULES[rule],
                                           DTYPES[dtype], ctypes.byref(full), ctypes.byref(least))
    if st != 0:
        raise InfiniAttnError(st, "infini_attn_workspace_size_kv")
    return int(full.value), int(least.value)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def forward(q, k, v, beta, M0, z0, seg_len, rule, *, out=None, M_final=None, z_final=None,
            workspace=None, stream=None, events=None, lse=None):
    """Infini-attention block forward on the GPU.

    q [B,Hq,L,d], k and v [B,Hkv,L,d] (float32 or bfloat16, contiguous, on one
    GPU), beta [Hq] float32, M0 [B,Hkv,d,d] float32, z0 [B,Hkv,d] float32.
    v may have another width dv than q and k (then M0 is [B,Hkv,d,dv] and out
    [B,Hq,L,dv]): infini_attn_forward_kv, without ``lse``.
    Returns (out, M_final, z_final). Output buffers and a workspace (a uint8
    tensor) may be passed in; M_final may be M0 and z_final may be z0. Runs on
    ``stream`` (a torch.cuda.Stream) or torch's current stream, asynchronously.
    ``events``: optional list of torch.cuda.Event to record around each phase
    (see infini_attn_forward_timed); each must have been recorded once so that
    its HIP event exists. ``lse``: a float32 [B,Hq,L] tensor to receive the
    softmax statistics (infini_attn_forward_train, _kv with two widths); not
    with ``events``.
    """
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dv = v.shape[-1] if v.dim() == 4 else -1
    if not (k.shape == (B, Hkv, L, d) and v.shape == (B, Hkv, L, dv)):
        raise ValueError(f"k must be [B,Hkv,L,d] and v [B,Hkv,L,dv]; got {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    if beta.shape != (Hq,) or M0.shape != (B, Hkv, d, dv) or z0.shape != (B, Hkv, d):
        raise ValueError("beta, M0 or z0 has the wrong shape")
    if q.dtype not in DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype, float32 or bfloat16")
    if beta.dtype != torch.float32 or M0.dtype != torch.float32 or z0.dtype != torch.float32:
        raise TypeError("beta, M0 and z0 must be float32")
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)}")
    tensors = [q, k, v, beta, M0, z0]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    for t in tensors:
        if t.device != dev:
            raise ValueError("all tensors must be on one GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = torch.empty((B, Hq, L, dv), dtype=q.dtype, device=dev)
    if M_final is None:
        M_final = torch.empty_like(M0)
    if z_final is None:
        z_final = torch.empty_like(z0)
    if out.shape != (B, Hq, L, dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,Hq,L,dv] tensor of q's dtype")
    if M_final.shape != M0.shape or z_final.shape != z0.shape:
        raise ValueError("M_final / z_final must have the shapes of M0 / z0")
    if workspace is None:
        full, _ = workspace_size_kv(B, Hq, Hkv, L, d, dv, seg_len, rule, q.dtype)
        workspace = torch.empty(full, dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    lib = load_library()
    with torch.cuda.device(dev):
        return _forward_call(lib, B, Hq, Hkv, L, d, dv, seg_len, rule, q, k, v, beta, M0, z0,
                             out, M_final, z_final, workspace, stream, events, lse)


def _forward_call(lib, B, Hq, Hkv, L, d, dv, seg_len, rule, q, k, v, beta, M0, z0, out,
                  M_final, z_final, workspace, stream, events, lse):
    dev = q.device
    args = [B, Hq, Hkv, L, d, seg_len, RULES[rule], DTYPES[q.dtype],
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(M0), _ptr(z0),
            _ptr(out), _ptr(M_final), _ptr(z_final),
            _ptr(workspace), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(stream.cuda_stream)]
    if lse is not None:
        if events:
            raise ValueError("lse and events cannot be combined")
        if lse.shape != (B, Hq, L) or lse.dtype != torch.float32 or not lse.is_contiguous() \
                or lse.device != dev:
            raise ValueError("lse must be a contiguous float32 [B,Hq,L] tensor on the GPU of q")
        if dv != d:
            st = lib.infini_attn_forward_train_kv(*args[:5], dv, *args[5:17], _ptr(lse),
                                                  *args[17:])
            name = "infini_attn_forward_train_kv"
        else:
            st = lib.infini_attn_forward_train(*args[:17], _ptr(lse), *args[17:])
            name = "infini_attn_forward_train"
    elif events:
        handles = (_c_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
        if dv != d:
            st = lib.infini_attn_forward_kv_timed(*args[:5], dv, *args[5:], handles, len(events))
            name = "infini_attn_forward_kv_timed"
        else:
            st = lib.infini_attn_forward_timed(*args, handles, len(events))
            name = "infini_attn_forward_timed"
    elif dv != d:
        st = lib.infini_attn_forward_kv(*args[:5], dv, *args[5:])
        name = "infini_attn_forward_kv"
    else:
        st = lib.infini_attn_forward(*args)
        name = "infini_attn_forward"
    if st != 0:
        raise InfiniAttnError(st, name)
    return out, M_final, z_final


NOALLOC_SCRATCH_BYTES = 64 << 20  # INFINI_NOALLOC_SCRATCH_BYTES


def forward_noalloc(q, k, v, beta, M0, z0, seg_len, rule, *, out, M_final, z_final,
                    stream=None):
    """infini_attn_forward_noalloc: the forward with the library's per-GPU
    scratch array as its workspace. q, k, v share one width d here. Every
    output buffer is the caller's (nothing is allocated, here or in the
    library); M_final may be M0 and z_final may be z0. Calls that can run at
    the same time on one GPU race on the scratch array."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, L, d) or v.shape != (B, Hkv, L, d):
        raise ValueError("k and v must be [B,Hkv,L,d] with q's d")
    if beta.shape != (Hq,) or M0.shape != (B, Hkv, d, d) or z0.shape != (B, Hkv, d):
        raise ValueError("beta, M0 or z0 has the wrong shape")
    if out.shape != (B, Hq, L, d) or M_final.shape != M0.shape or z_final.shape != z0.shape:
        raise ValueError("out, M_final or z_final has the wrong shape")
    if q.dtype not in DTYPES or k.dtype != q.dtype or v.dtype != q.dtype or \
            out.dtype != q.dtype:
        raise TypeError("q, k, v and out must share one dtype, float32 or bfloat16")
    for t in (beta, M0, z0, M_final, z_final):
        if t.dtype != torch.float32:
            raise TypeError("beta, M0, z0, M_final and z_final must be float32")
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)}")
    dev = q.device
    for t in (q, k, v, beta, M0, z0, out, M_final, z_final):
        if t.device != dev or dev.type != "cuda" or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous and on one GPU")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.infini_attn_forward_noalloc(
            B, Hq, Hkv, L, d, seg_len, RULES[rule], DTYPES[q.dtype],
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(M0), _ptr(z0),
            _ptr(out), _ptr(M_final), _ptr(z_final), ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise InfiniAttnError(st, "infini_attn_forward_noalloc")
    return out, M_final, z_final


def decode_workspace_size(B, Hq, Hkv, d, seg_len, rule, dtype):
    """Workspace bytes of a decode step with these sizes."""
    lib = load_library()
    n = _c_size(0)
    st = lib.infini_attn_decode_workspace_size(B, Hq, Hkv, d, seg_len, RULES[rule], DTYPES[dtype],
                                               ctypes.byref(n))
    if st != 0:
        raise InfiniAttnError(st, "infini_attn_decode_workspace_size")
    return int(n.value)


def decode_step(q, k, v, beta, k_cache, v_cache, M, z, pos, rule, *, out=None, workspace=None,
                stream=None):
    """One streaming decode step on the GPU (infini_attn_decode_step).

    q [B,Hq,d], k and v [B,Hkv,d] (float32 or bfloat16) for the token at
    position ``pos`` of its segment; k_cache, v_cache [B,Hkv,seg_len,d] of the
    same dtype; M [B,Hkv,d,d] and z [B,Hkv,d] float32, the state before the
    segment. Writes the token into the caches and, when pos == seg_len - 1,
    folds the segment into M and z in place. Returns out [B,Hq,d].
    v, v_cache and M's columns may have another width dv than q and k (then
    out is [B,Hq,dv]: infini_attn_decode_step_kv).
    Asynchronous on ``stream`` (or torch's current stream).
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    seg_len = k_cache.shape[2]
    dv = v.shape[-1] if v.dim() == 3 else -1
    if k.shape != (B, Hkv, d) or v.shape != (B, Hkv, dv):
        raise ValueError("k must be [B,Hkv,d] and v [B,Hkv,dv]")
    if k_cache.shape != (B, Hkv, seg_len, d) or v_cache.shape != (B, Hkv, seg_len, dv):
        raise ValueError("k_cache must be [B,Hkv,seg_len,d] and v_cache [B,Hkv,seg_len,dv]")
    if beta.shape != (Hq,) or M.shape != (B, Hkv, d, dv) or z.shape != (B, Hkv, d):
        raise ValueError("beta, M or z has the wrong shape")
    if q.dtype not in DTYPES or any(t.dtype != q.dtype for t in (k, v, k_cache, v_cache)):
        raise TypeError("q, k, v and the caches must share one dtype, float32 or bfloat16")
    if beta.dtype != torch.float32 or M.dtype != torch.float32 or z.dtype != torch.float32:
        raise TypeError("beta, M and z must be float32")
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)}")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    for t in (q, k, v, beta, k_cache, v_cache, M, z):
        if t.device != dev:
            raise ValueError("all tensors must be on one GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = torch.empty((B, Hq, dv), dtype=q.dtype, device=dev)
    if out.shape != (B, Hq, dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,Hq,dv] tensor of q's dtype")
    lib = load_library()
    if workspace is None:
        n = _c_size(0)
        st = lib.infini_attn_decode_workspace_size_kv(B, Hq, Hkv, d, dv, seg_len, RULES[rule],
                                                      DTYPES[q.dtype], ctypes.byref(n))
        if st != 0:
            raise InfiniAttnError(st, "infini_attn_decode_workspace_size_kv")
        workspace = torch.empty(int(n.value), dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(k_cache), _ptr(v_cache), _ptr(M),
            _ptr(z), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(stream.cuda_stream)]
    if dv != d:
        st = lib.infini_attn_decode_step_kv(B, Hq, Hkv, d, dv, seg_len, int(pos), RULES[rule],
                                            DTYPES[q.dtype], *args)
        name = "infini_attn_decode_step_kv"
    else:
        st = lib.infini_attn_decode_step(B, Hq, Hkv, d, seg_len, int(pos), RULES[rule],
                                         DTYPES[q.dtype], *args)
        name = "infini_attn_decode_step"
    if st != 0:
        raise InfiniAttnError(st, name)
    return out


def forward_train(q, k, v, beta, M0, z0, seg_len, rule, **kw):
    """forward() that also returns the softmax statistics the backward pass
    needs: (out, M_final, z_final, lse) with lse [B,Hq,L] float32."""
    B, Hq, L, _ = q.shape
    lse = torch.empty(B, Hq, L, dtype=torch.float32, device=q.device)
    out, M_final, z_final = forward(q, k, v, beta, M0, z0, seg_len, rule, lse=lse, **kw)
    return out, M_final, z_final, lse


def backward_workspace_size(B, Hq, Hkv, L, d, seg_len, rule, dtype, d_value=None):
    """Workspace bytes of a backward call with these sizes (of
    infini_attn_backward_kv when d_value is given and differs from d)."""
    n = _c_size(0)
    lib = load_library()
    if d_value is None or d_value == d:
        st = lib.infini_attn_backward_workspace_size(B, Hq, Hkv, L, d, seg_len, RULES[rule],
                                                     DTYPES[dtype], ctypes.byref(n))
        name = "infini_attn_backward_workspace_size"
    else:
        st = lib.infini_attn_backward_workspace_size_kv(B, Hq, Hkv, L, d, d_value, seg_len,
                                                        RULES[rule], DTYPES[dtype],
                                                        ctypes.byref(n))
        name = "infini_attn_backward_workspace_size_kv"
    if st != 0:
        raise InfiniAttnError(st, name)
    return int(n.value)


def backward(q, k, v, beta, M0, z0, seg_len, rule, out, lse, d_out, dM_final=None,
             dz_final=None, *, workspace=None, stream=None):
    """Gradients of the block (infini_attn_backward).

    The forward's inputs, its out and lse (forward_train), and the gradients
    d_out (like out), dM_final (like M0) and dz_final (like z0; either may be
    None for zero). Returns (dq, dk, dv, dbeta, dM0, dz0). Asynchronous on
    ``stream`` (or torch's current stream). v may have another width dv than
    q and k (out, d_out [B,Hq,L,dv], M0 [B,Hkv,d,dv]): infini_attn_backward_kv.
    """
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dv_w = v.shape[-1] if v.dim() == 4 else -1
    if not (k.shape == (B, Hkv, L, d) and v.shape == (B, Hkv, L, dv_w)):
        raise ValueError("k must be [B,Hkv,L,d] and v [B,Hkv,L,dv]")
    if beta.shape != (Hq,) or M0.shape != (B, Hkv, d, dv_w) or z0.shape != (B, Hkv, d):
        raise ValueError("beta, M0 or z0 has the wrong shape")
    if out.shape != (B, Hq, L, dv_w) or d_out.shape != out.shape or lse.shape != (B, Hq, L):
        raise ValueError("out and d_out must be [B,Hq,L,dv], lse [B,Hq,L]")
    if q.dtype not in DTYPES or any(t.dtype != q.dtype for t in (k, v, out, d_out)):
        raise TypeError("q, k, v, out and d_out must share one dtype, float32 or bfloat16")
    f32 = [beta, M0, z0, lse] + [t for t in (dM_final, dz_final) if t is not None]
    if any(t.dtype != torch.float32 for t in f32):
        raise TypeError("beta, M0, z0, lse, dM_final and dz_final must be float32")
    if dM_final is not None and dM_final.shape != M0.shape:
        raise ValueError("dM_final must be like M0")
    if dz_final is not None and dz_final.shape != z0.shape:
        raise ValueError("dz_final must be like z0")
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)}")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    for t in [q, k, v, out, d_out] + f32:
        if t.device != dev:
            raise ValueError("all tensors must be on one GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbeta, dM0, dz0 = torch.empty_like(beta), torch.empty_like(M0), torch.empty_like(z0)
    if workspace is None:
        workspace = torch.empty(backward_workspace_size(B, Hq, Hkv, L, d, seg_len, rule, q.dtype,
                                                        d_value=dv_w),
                                dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    opt = lambda t: _ptr(t) if t is not None else ctypes.c_void_p(0)
    args = [RULES[rule], DTYPES[q.dtype],
            _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(M0), _ptr(z0),
            _ptr(out), _ptr(lse), _ptr(d_out), opt(dM_final), opt(dz_final),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbeta), _ptr(dM0), _ptr(dz0),
            _ptr(workspace), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(stream.cuda_stream)]
    lib = load_library()
    if dv_w != d:
        st = lib.infini_attn_backward_kv(B, Hq, Hkv, L, d, dv_w, seg_len, *args)
        name = "infini_attn_backward_kv"
    else:
        st = lib.infini_attn_backward(B, Hq, Hkv, L, d, seg_len, *args)
        name = "infini_attn_backward"
    if st != 0:
        raise InfiniAttnError(st, name)
    return dq, dk, dv, dbeta, dM0, dz0


def block_workspace_size(B, L, d_model, Hq, Hkv, d, seg_len, rule, dtype=torch.bfloat16,
                         d_value=None):
    """Workspace bytes of infini_attn_block_forward with these sizes (of
    infini_attn_block_forward_kv when d_value is given and differs from d)."""
    n = _c_size(0)
    lib = load_library()
    if d_value is None or d_value == d:
        st = lib.infini_attn_block_workspace_size(B, L, d_model, Hq, Hkv, d, seg_len,
                                                  RULES[rule], DTYPES[dtype], ctypes.byref(n))
        name = "infini_attn_block_workspace_size"
    else:
        st = lib.infini_attn_block_workspace_size_kv(B, L, d_model, Hq, Hkv, d, d_value,
                                                     seg_len, RULES[rule], DTYPES[dtype],
                                                     ctypes.byref(n))
        name = "infini_attn_block_workspace_size_kv"
    if st != 0:
        raise InfiniAttnError(st, name)
    return int(n.value)


def block_forward(x, w_qkv, w_o, beta, M0, z0, seg_len, rule, Hq, Hkv, *, y=None, M_final=None,
                  z_final=None, workspace=None, stream=None, events=None):
    """The block with its projections on the GPU (infini_attn_block_forward).

    x [B,L,d_model] bfloat16; w_qkv [(Hq+2Hkv)*d, d_model] and w_o
    [d_model, Hq*d] bfloat16 (linear-layer layout); beta [Hq], M0 [B,Hkv,d,d],
    z0 [B,Hkv,d] float32. Returns (y [B,L,d_model], M_final, z_final).
    With a value width dv other than the key width d (M0 [B,Hkv,d,dv]), w_qkv
    is [(Hq+Hkv)*d + Hkv*dv, d_model] and w_o [d_model, Hq*dv]
    (infini_attn_block_forward_kv, without ``events``).
    ``events`` (up to 4 torch.cuda.Event) are recorded before the input
    projection, after it, after the block and after the output projection.
    Asynchronous on ``stream`` (or torch's current stream).
    """
    B, L, d_model = x.shape
    if M0.dim() != 4:
        raise ValueError("M0 must be [B,Hkv,d,dv]")
    d, dv = M0.shape[2], M0.shape[3]
    if w_qkv.shape != ((Hq + Hkv) * d + Hkv * dv, d_model):
        raise ValueError("w_qkv must be [(Hq+Hkv)*d + Hkv*dv, d_model]")
    if w_o.shape != (d_model, Hq * dv):
        raise ValueError("w_o must be [d_model, Hq*dv]")
    if beta.shape != (Hq,) or M0.shape != (B, Hkv, d, dv) or z0.shape != (B, Hkv, d):
        raise ValueError("beta, M0 or z0 has the wrong shape")
    if dv != d and events:
        raise ValueError("events need d_value == d_key")
    if any(t.dtype != torch.bfloat16 for t in (x, w_qkv, w_o)):
        raise TypeError("x, w_qkv and w_o must be bfloat16")
    if any(t.dtype != torch.float32 for t in (beta, M0, z0)):
        raise TypeError("beta, M0 and z0 must be float32")
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)}")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    for t in (x, w_qkv, w_o, beta, M0, z0):
        if t.device != dev:
            raise ValueError("all tensors must be on one GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if y is None:
        y = torch.empty_like(x)
    if M_final is None:
        M_final = torch.empty_like(M0)
    if z_final is None:
        z_final = torch.empty_like(z0)
    if y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous():
        raise ValueError("y must be a contiguous tensor like x")
    if workspace is None:
        workspace = torch.empty(block_workspace_size(B, L, d_model, Hq, Hkv, d, seg_len, rule,
                                                     d_value=dv),
                                dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    lib = load_library()
    args = [B, L, d_model, Hq, Hkv, d, seg_len, RULES[rule], DTYPES[x.dtype],
            _ptr(x), _ptr(w_qkv), _ptr(w_o), _ptr(beta), _ptr(M0), _ptr(z0),
            _ptr(y), _ptr(M_final), _ptr(z_final),
            _ptr(workspace), workspace.numel() * workspace.element_size(),
            ctypes.c_void_p(stream.cuda_stream)]
    if events:
        if any(e.cuda_event == 0 for e in events):
            raise ValueError("record every event once before passing it (torch creates the "
                             "HIP event at its first record)")
        handles = (_c_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
        st = lib.infini_attn_block_forward_timed(*args, handles, len(events))
        name = "infini_attn_block_forward_timed"
    elif dv != d:
        st = lib.infini_attn_block_forward_kv(*args[:6], dv, *args[6:])
        name = "infini_attn_block_forward_kv"
    else:
        st = lib.infini_attn_block_forward(*args)
        name = "infini_attn_block_forward"
    if st != 0:
        raise InfiniAttnError(st, name)
    return y, M_final, z_final
