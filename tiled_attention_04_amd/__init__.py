"""MI355X (gfx950) fused attention: thin ctypes binding of libfa_mi355x.so.

The binding only marshals arguments: every step of the attention forward and
backward runs in the library's HIP kernels.  PyTorch supplies device memory
and the stream.  There is no CPU fallback -- calling into the binding without
the built library raises.

``fa_fwd`` and ``fa_bwd`` mirror the C entry points of the same names (raw
pointers, sizes and per-tensor element strides); ``forward`` and ``backward``
are the tensor-level convenience wrappers.
"""
import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa_mi355x.so")

FA_DTYPE_F32, FA_DTYPE_F16, FA_DTYPE_BF16, FA_DTYPE_E5M2 = 0, 1, 2, 3
STATUS = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_DTYPE",
          4: "FA_ERR_HEAD_DIM", 5: "FA_ERR_LAYOUT", 6: "FA_ERR_HIP", 7: "FA_ERR_SCALE",
          8: "FA_ERR_WORKSPACE"}
EXPORTS = ("fa_fwd", "fa_fwd_splitk", "fa_fwd_splitk_choose", "fa_fwd_splitk_workspace",
           "fa_fwd_splitk_static", "fa_bwd", "fa_status_string", "fa_last_error", "fa_version")
SPLITK_STATIC_MAX_BYTES = 32 << 20  # FA_SPLITK_STATIC_MAX_BYTES of include/fa.h


class FaStrides(ctypes.Structure):
    """Element strides of one tensor for (batch, head, seq, dim)."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64),
                ("seq", ctypes.c_int64), ("dim", ctypes.c_int64)]


class FaError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


_lib = None


def lib():
    """Load libfa_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m tiled_attention_04_amd.build` "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.fa_fwd.restype = ctypes.c_int
        L.fa_fwd.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [FaStrides] * 4 +
                             [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p])
        L.fa_fwd_splitk.restype = ctypes.c_int
        L.fa_fwd_splitk.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [FaStrides] * 4 +
                                    [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p])
        L.fa_fwd_splitk_static.restype = ctypes.c_int
        L.fa_fwd_splitk_static.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 +
                                           [FaStrides] * 4 +
                                           [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p])
        L.fa_fwd_splitk_choose.restype = ctypes.c_int
        L.fa_fwd_splitk_choose.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int]
        L.fa_fwd_splitk_workspace.restype = ctypes.c_size_t
        L.fa_fwd_splitk_workspace.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
        L.fa_bwd.restype = ctypes.c_int
        L.fa_bwd.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int64] * 5 + [FaStrides] * 8 +
                             [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p])
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_status_string.argtypes = [ctypes.c_int]
        L.fa_last_error.restype = ctypes.c_char_p
        L.fa_last_error.argtypes = []
        L.fa_version.restype = ctypes.c_int
        L.fa_version.argtypes = []
        _lib = L
    return _lib


def fa_fwd(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, q_st, k_st, v_st, o_st,
           sm_scale, causal, dtype, stream):
    """Direct call of the C entry point; returns the integer status."""
    st = [s if isinstance(s, FaStrides) else FaStrides(*s) for s in (q_st, k_st, v_st, o_st)]
    return lib().fa_fwd(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, *st,
                        float(sm_scale), int(causal), int(dtype), stream)


def fa_fwd_splitk(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, q_st, k_st, v_st, o_st,
                  sm_scale, causal, dtype, num_splits, workspace, workspace_bytes, stream):
    """Direct call of the C entry point; returns the integer status."""
    st = [s if isinstance(s, FaStrides) else FaStrides(*s) for s in (q_st, k_st, v_st, o_st)]
    return lib().fa_fwd_splitk(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, *st,
                               float(sm_scale), int(causal), int(dtype), int(num_splits),
                               workspace, int(workspace_bytes), stream)


def fa_fwd_splitk_static(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, q_st, k_st, v_st,
                         o_st, sm_scale, causal, dtype, num_splits, stream):
    """Direct call of the C entry point; returns the integer status."""
    st = [s if isinstance(s, FaStrides) else FaStrides(*s) for s in (q_st, k_st, v_st, o_st)]
    return lib().fa_fwd_splitk_static(q, k, v, o, lse, batch, heads, seq_q, seq_k, head_dim, *st,
                                      float(sm_scale), int(causal), int(dtype), int(num_splits),
                                      stream)


def fa_fwd_splitk_choose(batch, heads, seq_q, seq_k, head_dim, causal):
    return lib().fa_fwd_splitk_choose(batch, heads, seq_q, seq_k, head_dim, int(causal))


def fa_fwd_splitk_workspace(batch, heads, seq_q, head_dim, num_splits):
    return lib().fa_fwd_splitk_workspace(batch, heads, seq_q, head_dim, int(num_splits))


def fa_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, batch, heads, seq_q, seq_k, head_dim,
           q_st, k_st, v_st, o_st, do_st, dq_st, dk_st, dv_st, sm_scale, causal, dtype, stream):
    """Direct call of the C entry point; returns the integer status."""
    st = [s if isinstance(s, FaStrides) else FaStrides(*s)
          for s in (q_st, k_st, v_st, o_st, do_st, dq_st, dk_st, dv_st)]
    return lib().fa_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, batch, heads, seq_q, seq_k,
                        head_dim, *st, float(sm_scale), int(causal), int(dtype), stream)


def last_error():
    return lib().fa_last_error().decode()


def _check_device(device, **tensors):
    """Every tensor given must live on `device` (a CUDA device): a host
    pointer handed to a kernel would fault the GPU, so nothing is launched."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor (got {t.device})")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, q on {device}")


def _check_like(name, t, shape, dtype):
    """A caller-supplied output: exactly `shape` and `dtype` (the C ABI cannot
    see sizes, so an undersized buffer would be written past its end)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _check_rows(name, t, B, H, Sq):
    """lse / delta: contiguous fp32 [B, H, Sq]."""
    import torch
    if t.dtype != torch.float32 or tuple(t.shape) != (B, H, Sq) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 [{B}, {H}, {Sq}] tensor")


def _dtype_code(t):
    import torch
    codes = {torch.float32: FA_DTYPE_F32, torch.float16: FA_DTYPE_F16,
             torch.bfloat16: FA_DTYPE_BF16, torch.float8_e5m2: FA_DTYPE_E5M2}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _dims(t, layout):
    """(batch, heads, seq, dim) sizes and element strides of t under `layout`."""
    if layout == "bhsd":
        B, H, S, D = t.shape
        sb, sh, ss, sd = t.stride()
    elif layout == "bshd":
        B, S, H, D = t.shape
        sb, ss, sh, sd = t.stride()
    elif layout == "shd":
        S, H, D = t.shape
        ss, sh, sd = t.stride()
        B, sb = 1, 0
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return (B, H, S, D), FaStrides(sb, sh, ss, sd)


def _dims_vt(vt, layout):
    """Sizes and strides of a key-major V ([B, H, D, Sv], or [H, D, Sv] for "shd")."""
    if layout == "shd":
        H, D, S = vt.shape
        sh, sd, ss = vt.stride()
        B, sb = 1, 0
    elif layout in ("bhsd", "bshd"):
        B, H, D, S = vt.shape
        sb, sh, sd, ss = vt.stride()
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return (B, H, S, D), FaStrides(sb, sh, ss, sd)


def forward(q, k, v, causal=False, sm_scale=None, layout="bhsd", out=None, lse=None,
            return_lse=True):
    """Attention forward on the current HIP stream.

    q: [B, H, Sq, D] ("bhsd"), [B, Sq, H, D] ("bshd") or [Sq, H, D] ("shd");
    k, v: the same with Sk.  sm_scale defaults to 1/sqrt(D).
    For torch.float8_e5m2 inputs v is passed key-major instead: [B, H, D, Sv]
    ([H, D, Sv] for "shd") with unit key stride and Sv >= Sk (keys past Sk
    are padding and must be finite), e.g. ``v.transpose(-2, -1)`` of a
    contiguous copy padded to a multiple of 16 keys.
    Returns (o, lse) with o like q and lse fp32 [B, H, Sq]; or o alone when
    return_lse is False (then lse is not computed unless passed in).
    """
    import torch
    if not q.is_cuda:
        raise ValueError("q, k and v must be device tensors")
    _check_device(q.device, k=k, v=v, out=out, lse=lse)
    (B, H, Sq, D), q_st = _dims(q, layout)
    (Bk, Hk, Sk, Dk), k_st = _dims(k, layout)
    if q.dtype == torch.float8_e5m2:
        (Bv, Hv, Sv, Dv), v_st = _dims_vt(v, layout)
        if (Bv, Hv, Dv) != (B, H, D) or Sv < Sk:
            raise ValueError("key-major v must be [B, H, D, Sv] with Sv >= Sk")
    else:
        (Bv, Hv, Sv, Dv), v_st = _dims(v, layout)
        if (Bv, Hv, Sv, Dv) != (B, H, Sk, D):
            raise ValueError("q, k, v shapes disagree")
    if (Bk, Hk, Dk) != (B, H, D):
        raise ValueError("q, k, v shapes disagree")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check_like("out", out, q.shape, q.dtype)
    (_, _, _, _), o_st = _dims(out, layout)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_rows("lse", lse, B, H, Sq)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                lse.data_ptr() if lse is not None else None, B, H, Sq, Sk, D,
                q_st, k_st, v_st, o_st, sm_scale, causal, _dtype_code(q), stream)
    if rc != 0:
        raise FaError(rc, last_error())
    return (out, lse) if return_lse else out


def forward_splitk(q, k, v, causal=False, sm_scale=None, layout="bhsd", num_splits=0,
                   out=None, lse=None, workspace=None):
    """``forward`` with the keys split over ``num_splits`` workgroups per query
    tile (0: the library's choice) and merged by logsumexp.  ``workspace`` is a
    device tensor of at least fa_fwd_splitk_workspace(...) bytes (allocated
    when None).  Returns (o, lse)."""
    import torch
    if not q.is_cuda:
        raise ValueError("q, k and v must be device tensors")
    _check_device(q.device, k=k, v=v, out=out, lse=lse, workspace=workspace)
    (B, H, Sq, D), q_st = _dims(q, layout)
    (Bk, Hk, Sk, Dk), k_st = _dims(k, layout)
    (Bv, Hv, Sv, Dv), v_st = _dims(v, layout)
    if (Bk, Hk, Dk) != (B, H, D) or (Bv, Hv, Sv, Dv) != (B, H, Sk, D):
        raise ValueError("q, k, v shapes disagree")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if num_splits == 0:
        num_splits = fa_fwd_splitk_choose(B, H, Sq, Sk, D, causal)
    out = torch.empty_like(q) if out is None else out
    _check_like("out", out, q.shape, q.dtype)
    (_, _, _, _), o_st = _dims(out, layout)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_rows("lse", lse, B, H, Sq)
    need = fa_fwd_splitk_workspace(B, H, Sq, D, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_fwd_splitk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       B, H, Sq, Sk, D, q_st, k_st, v_st, o_st, sm_scale, causal, _dtype_code(q),
                       num_splits, ws_ptr, ws_bytes, stream)
    if rc != 0:
        raise FaError(rc, last_error())
    return out, lse


def backward(q, k, v, o, dout, lse, causal=False, sm_scale=None, layout="bhsd",
             dq=None, dk=None, dv=None, delta=None):
    """Gradients of ``forward`` on the current HIP stream.

    o and lse are the forward's outputs for (q, k, v); dout is the gradient
    of the loss with respect to o (same shape as q).  Returns (dq, dk, dv),
    each like its input; ``delta`` (fp32 [B, H, Sq], allocated when None)
    receives rowsum(dout * o).
    """
    import torch
    if not q.is_cuda:
        raise ValueError("all tensors must be device tensors")
    _check_device(q.device, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)
    (B, H, Sq, D), q_st = _dims(q, layout)
    (Bk, Hk, Sk, Dk), k_st = _dims(k, layout)
    (_, _, Sv, _), v_st = _dims(v, layout)
    (_, _, So, _), o_st = _dims(o, layout)
    (_, _, Sd, _), do_st = _dims(dout, layout)
    if (Bk, Hk, Dk) != (B, H, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, o, dout shapes disagree")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise TypeError("q, k, v, o and dout must share a dtype")
    _check_rows("lse", lse, B, H, Sq)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check_like("dq", dq, q.shape, q.dtype)
    _check_like("dk", dk, k.shape, q.dtype)
    _check_like("dv", dv, v.shape, q.dtype)
    if delta is None:
        delta = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_rows("delta", delta, B, H, Sq)
    (_, _, _, _), dq_st = _dims(dq, layout)
    (_, _, _, _), dk_st = _dims(dk, layout)
    (_, _, _, _), dv_st = _dims(dv, layout)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                B, H, Sq, Sk, D, q_st, k_st, v_st, o_st, do_st, dq_st, dk_st, dv_st,
                sm_scale, causal, _dtype_code(q), stream)
    if rc != 0:
        raise FaError(rc, last_error())
    return dq, dk, dv
