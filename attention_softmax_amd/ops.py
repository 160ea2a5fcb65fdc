"""Tensor-level binding of sms_forward / sms_backward and the autograd wrapper.

Argument marshalling only: shapes, strides, dtype, mask mode and the current
stream are read from the tensors and passed to libsms.so. Nothing here computes
any part of the softmax, and there is no CPU path: a tensor that is not on the
GPU is an error.
"""

import torch

from . import _lib

_DTYPES = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
           torch.float64: "f64"}


def _dtype_code(t, what):
    try:
        return _lib.DTYPE_CODES[_DTYPES[t.dtype]]
    except KeyError:
        raise TypeError(
            f"{what}: dtype {t.dtype} is not float32, float16, bfloat16 or float64") from None


def _require_gpu(t, what):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor (there is no CPU path)")


def _require_4d_rows(t, what):
    if t.dim() != 4:
        raise ValueError(f"{what} must be 4-D [B, H, Sq, Sk], got shape {tuple(t.shape)}")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{what}: the key axis must be contiguous (stride 1)")


def _strides(t):
    st = list(t.stride())
    if t.shape[-1] <= 1:
        st[-1] = 1
    return _lib.strides4(st)


_INT_DTYPES = (torch.int32, torch.int64)
_BOOL_DTYPES = (torch.bool, torch.uint8)


def mask_kind_of(mask):
    """"none", "bool" (torch.bool / uint8: nonzero excludes the key), "lengths"
    (an integer tensor of per-batch key lengths) or "additive"."""
    if mask is None:
        return "none"
    if mask.dtype in _BOOL_DTYPES:
        return "bool"
    if mask.dtype in _INT_DTYPES:
        return "lengths"
    return "additive"


def mask_mode_of(mask, shape):
    """Mask shape mode for ``mask`` against x of ``shape``.

    [Sq,Sk] or [1,1,Sq,Sk] -> "sq_sk"; [B,Sq,Sk] or [B,1,Sq,Sk] -> "b_sq_sk";
    [B,1,Sk] or [B,1,1,Sk] -> "b_1_sk"; [B,H,Sq,Sk] -> "full"; an integer
    tensor of shape [B] -> "key_lengths".
    """
    if mask is None:
        return "none"
    B, H, Sq, Sk = shape
    ms = tuple(mask.shape)
    if mask_kind_of(mask) == "lengths":
        if ms != (B,):
            raise ValueError(f"key lengths must have shape [B] = ({B},), got {ms}")
        return "key_lengths"
    table = [
        ((Sq, Sk), "sq_sk"), ((1, 1, Sq, Sk), "sq_sk"),
        ((B, Sq, Sk), "b_sq_sk"), ((B, 1, Sq, Sk), "b_sq_sk"),
        ((B, 1, Sk), "b_1_sk"), ((B, 1, 1, Sk), "b_1_sk"),
        ((B, H, Sq, Sk), "full"),
    ]
    for s, mode in table:
        if ms == s:
            return mode
    raise ValueError(f"mask shape {ms} is none of [Sq,Sk], [B,Sq,Sk], [B,1,Sk], [B,H,Sq,Sk] "
                     f"for x of shape {tuple(shape)}")


def causal_code(is_causal):
    """False / None / "none" -> 0; True / "top_left" -> 1 (key k > q excluded);
    "bottom_right" -> 2 (key k > q + Sk - Sq excluded)."""
    if is_causal is None or is_causal is False:
        return 0
    if is_causal is True:
        return 1
    if isinstance(is_causal, str) and is_causal in _lib.CAUSAL_CODES:
        return _lib.CAUSAL_CODES[is_causal]
    if isinstance(is_causal, int) and is_causal in (0, 1, 2):
        return is_causal
    raise ValueError(f"is_causal must be False, True, 'top_left' or 'bottom_right', "
                     f"got {is_causal!r}")


def _stream_of(device, stream):
    return stream if stream is not None else torch.cuda.current_stream(device)


def sms_workspace_bytes(dtype, shape, backward=False):
    """Workspace bytes sms_forward / sms_backward use for split rows (0: none)."""
    B, H, Sq, Sk = shape
    n = int(_lib.lib().sms_workspace_bytes(_lib.DTYPE_CODES[_DTYPES[dtype]], B, H, Sq, Sk,
                                           int(backward)))
    if n < 0:
        raise ValueError(f"no workspace size for dtype {dtype} and shape {tuple(shape)}")
    return n


def _workspace(dtype, shape, backward, device, stream, workspace):
    """(pointer, bytes) of the workspace for a call: the caller's tensor, or a
    fresh one from torch's allocator on the launch stream when rows split."""
    if workspace is not None:
        _require_gpu(workspace, "workspace")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()
    B, H, Sq, Sk = shape
    need = int(_lib.lib().sms_workspace_bytes(_lib.DTYPE_CODES[_DTYPES[dtype]], B, H, Sq, Sk,
                                              int(backward)))
    if need <= 0:  # no split; invalid sizes are reported by the call itself
        return None, None, 0
    with torch.cuda.stream(stream):
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.data_ptr(), need


def _forward_args(x, mask, y):
    """Checks of a forward call's tensors; (dtype code, mask pointer, C mask mode)."""
    _require_gpu(x, "x")
    _require_gpu(y, "y")
    _require_4d_rows(x, "x")
    _require_4d_rows(y, "y")
    if y.shape != x.shape or y.dtype != x.dtype or y.device != x.device:
        raise ValueError("y must have x's shape, dtype and device")
    code = _dtype_code(x, "x")
    mode = mask_mode_of(mask, tuple(x.shape))
    kind = mask_kind_of(mask)
    mode_code = _lib.MASK_MODES[mode]
    mptr = None
    if mask is not None:
        _require_gpu(mask, "mask")
        if kind == "additive" and mask.dtype != x.dtype:
            raise TypeError(f"additive mask dtype {mask.dtype} must equal x dtype {x.dtype}")
        if kind == "lengths" and mask.dtype != torch.int32:
            raise TypeError("key lengths must be int32")
        if kind == "bool":
            mode_code |= _lib.MASK_BOOL
        if mask.device != x.device:
            raise ValueError("mask must be on x's device")
        if not mask.is_contiguous():
            raise ValueError("mask must be contiguous in its own shape")
        mptr = mask.data_ptr()
    return code, mptr, mode_code


def sms_forward(x, mask, y, scale=1.0, is_causal=False, stream=None, workspace=None):
    """y <- softmax(x*scale + mask) over the last axis (C ABI sms_forward_ws).

    x, y: 4-D GPU tensors of one shape and dtype (float32/float16/bfloat16), key
    axis contiguous; y may be x itself (in place). mask: None; an additive mask
    of x's dtype; a boolean mask (torch.bool or uint8, nonzero = key excluded);
    both contiguous, in one of the shapes ``mask_mode_of`` accepts; or int32 key
    lengths of shape [B]. is_causal: see ``causal_code``. Enqueued on ``stream``
    (default: the current stream); returns y. Few long rows are split across
    workgroups through a workspace: ``workspace`` (a GPU tensor of at least
    ``sms_workspace_bytes`` bytes) or, by default, one taken from torch's
    allocator on the launch stream.
    """
    code, mptr, mode_code = _forward_args(x, mask, y)
    B, H, Sq, Sk = x.shape
    L = _lib.lib()
    with torch.cuda.device(x.device):
        s = _stream_of(x.device, stream)
        keep, wptr, wbytes = _workspace(x.dtype, x.shape, False, x.device, s, workspace)
        st = L.sms_forward_ws(x.data_ptr(), _strides(x), mptr, mode_code, y.data_ptr(),
                              _strides(y), code, B, H, Sq, Sk, float(scale),
                              causal_code(is_causal), wptr, wbytes, s.cuda_stream)
        del keep  # torch reuses the block only for later work on this stream, after the launch
    _lib.check("sms_forward", st)
    return y


def sms_forward_noalloc(x, mask, y, scale=1.0, is_causal=False, stream=None):
    """sms_forward that allocates nothing (C ABI sms_forward_noalloc): a split
    of few long rows keeps its partials in the library's per-GPU scratch
    instead of a workspace. Arguments as for ``sms_forward``; calls that may
    overlap on one GPU share that scratch and must be ordered by the caller."""
    code, mptr, mode_code = _forward_args(x, mask, y)
    B, H, Sq, Sk = x.shape
    L = _lib.lib()
    with torch.cuda.device(x.device):
        s = _stream_of(x.device, stream)
        st = L.sms_forward_noalloc(x.data_ptr(), _strides(x), mptr, mode_code, y.data_ptr(),
                                   _strides(y), code, B, H, Sq, Sk, float(scale),
                                   causal_code(is_causal), s.cuda_stream)
    _lib.check("sms_forward_noalloc", st)
    return y


def sms_noalloc_scratch_bytes():
    """Bytes of the per-GPU scratch ``sms_forward_noalloc`` uses."""
    return int(_lib.lib().sms_noalloc_scratch_bytes())


def sms_backward(y, dy, dx, scale=1.0, is_causal=False, stream=None, workspace=None):
    """dx <- scale * y * (dy - sum_k dy_k y_k) row by row (C ABI sms_backward_ws).

    y, dy, dx: 4-D GPU tensors of one shape and dtype, key axis contiguous; dx
    may be dy or y itself. A causal ``is_causal`` (see ``causal_code``) promises
    y == 0 at the keys that rule excludes (true for y from a forward with the
    same rule); those keys are then skipped. ``workspace``: as for sms_forward.
    """
    for t, n in ((y, "y"), (dy, "dy"), (dx, "dx")):
        _require_gpu(t, n)
        _require_4d_rows(t, n)
        if t.shape != y.shape or t.dtype != y.dtype or t.device != y.device:
            raise ValueError("y, dy and dx must share shape, dtype and device")
    code = _dtype_code(y, "y")
    B, H, Sq, Sk = y.shape
    L = _lib.lib()
    with torch.cuda.device(y.device):
        s = _stream_of(y.device, stream)
        keep, wptr, wbytes = _workspace(y.dtype, y.shape, True, y.device, s, workspace)
        st = L.sms_backward_ws(y.data_ptr(), _strides(y), dy.data_ptr(), _strides(dy),
                               dx.data_ptr(), _strides(dx), code, B, H, Sq, Sk, float(scale),
                               causal_code(is_causal), wptr, wbytes, s.cuda_stream)
        del keep
    _lib.check("sms_backward", st)
    return dx


def _attn_check(tensors, q):
    for t, n in tensors:
        _require_gpu(t, n)
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{n} must be 4-D with a contiguous last axis")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{n} must share q's dtype and device")
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("attention takes float16 or bfloat16")


def _attn_shapes(q, k, v):
    B, H, Sq, D = q.shape
    Bk, Hk, Sk, Dk = k.shape
    if tuple(v.shape) != (Bk, Hk, Sk, Dk) or Bk != B or Dk != D:
        raise ValueError(f"shapes q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    return B, H, Hk, Sq, Sk, D


def _attn_mask(mask, q, scores_shape):
    """(pointer, C mask mode) of an attention mask over [B, H, Sq, Sk] scores."""
    mode_code = _lib.MASK_MODES[mask_mode_of(mask, scores_shape)]
    if mask is None:
        return None, mode_code
    _require_gpu(mask, "mask")
    kind = mask_kind_of(mask)
    if kind == "additive" and mask.dtype != q.dtype:
        raise TypeError("additive mask dtype must equal q's")
    if kind == "lengths" and mask.dtype != torch.int32:
        raise TypeError("key lengths must be int32")
    if kind == "bool":
        mode_code |= _lib.MASK_BOOL
    if not mask.is_contiguous():
        raise ValueError("mask must be contiguous in its own shape")
    return mask.data_ptr(), mode_code


def sms_attention_forward(q, k, v, mask=None, scale=None, is_causal=False, o=None,
                          return_lse=False, stream=None, lse=None):
    """O = softmax(Q K^T * scale + mask) V, fused on the matrix cores (C ABI
    sms_attention_forward).

    q [B,H,Sq,D], k and v [B,Hk,Sk,D] (Hk divides H), float16 or bfloat16 GPU
    tensors with the head dim contiguous and every row 16-byte aligned; D = 64
    or 128. ``mask``: as for ``sms_forward`` (shapes over [B,H,Sq,Sk], additive
    of q's dtype, boolean, or int32 key lengths [B]). ``scale`` defaults to
    1/sqrt(D). Returns O (``o`` if given), and the fp32 log-sum-exp [B,H,Sq]
    too when ``return_lse`` (written into ``lse`` if given, a contiguous
    float32 [B,H,Sq] GPU tensor; giving it implies ``return_lse``).
    """
    _attn_check(((q, "q"), (k, "k"), (v, "v")), q)
    B, H, Hk, Sq, Sk, D = _attn_shapes(q, k, v)
    if o is None:
        o = torch.empty_like(q, memory_format=torch.contiguous_format)
    _require_gpu(o, "o")
    if o.shape != q.shape or o.dtype != q.dtype or o.stride(-1) != 1:
        raise ValueError("o must have q's shape and dtype, last axis contiguous")
    if lse is not None:
        _require_gpu(lse, "lse")
        if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq)
                or not lse.is_contiguous() or lse.device != q.device):
            raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor on q's device")
        return_lse = True
    elif return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    mptr, mode_code = _attn_mask(mask, q, (B, H, Sq, Sk))
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    L = _lib.lib()
    with torch.cuda.device(q.device):
        s = _stream_of(q.device, stream)
        st = L.sms_attention_forward(
            q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
            mptr, mode_code, o.data_ptr(), _strides(o),
            lse.data_ptr() if lse is not None else None, _dtype_code(q, "q"), B, H, Hk, Sq, Sk,
            D, float(scale), causal_code(is_causal), s.cuda_stream)
    _lib.check("sms_attention_forward", st)
    return (o, lse) if return_lse else o


def sms_attention_workspace_bytes(B, H, Sq):
    """Bytes of device workspace ``sms_attention_backward`` needs (4 * B * H * Sq)."""
    n = int(_lib.lib().sms_attention_workspace_bytes(int(B), int(H), int(Sq)))
    if n < 0:
        raise ValueError(f"invalid attention sizes B={B} H={H} Sq={Sq}")
    return n


def sms_attention_backward(q, k, v, o, lse, do, mask=None, scale=None, is_causal=False,
                           dq=None, dk=None, dv=None, workspace=None, stream=None):
    """(dQ, dK, dV) of the fused attention (C ABI sms_attention_backward).

    q, k, v, mask, scale, is_causal: as passed to ``sms_attention_forward``;
    o and lse: its output and fp32 log-sum-exp; do: the upstream gradient
    (q's shape and dtype). The probabilities are recomputed from lse. Outputs
    are allocated unless given; ``workspace`` (a GPU tensor of at least
    ``sms_attention_workspace_bytes(B, H, Sq)`` bytes) likewise.
    """
    _attn_check(((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")), q)
    B, H, Hk, Sq, Sk, D = _attn_shapes(q, k, v)
    if o.shape != q.shape or do.shape != q.shape:
        raise ValueError("o and do must have q's shape")
    _require_gpu(lse, "lse")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
    outs = []
    for t, like, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if t is None:
            t = torch.empty_like(like, memory_format=torch.contiguous_format)
        _require_gpu(t, n)
        if t.shape != like.shape or t.dtype != like.dtype or t.stride(-1) != 1:
            raise ValueError(f"{n} must match its input's shape and dtype, last axis contiguous")
        outs.append(t)
    dq, dk, dv = outs
    mptr, mode_code = _attn_mask(mask, q, (B, H, Sq, Sk))
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    L = _lib.lib()
    need = sms_attention_workspace_bytes(B, H, Sq)
    with torch.cuda.device(q.device):
        s = _stream_of(q.device, stream)
        if workspace is None and need > 0:
            with torch.cuda.stream(s):
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        wptr, wbytes = None, 0
        if workspace is not None:
            _require_gpu(workspace, "workspace")
            wptr, wbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        st = L.sms_attention_backward(
            q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
            o.data_ptr(), _strides(o), do.data_ptr(), _strides(do), lse.data_ptr(), mptr,
            mode_code, dq.data_ptr(), _strides(dq), dk.data_ptr(), _strides(dk), dv.data_ptr(),
            _strides(dv), _dtype_code(q, "q"), B, H, Hk, Sq, Sk, D, float(scale),
            causal_code(is_causal), wptr, wbytes, s.cuda_stream)
    _lib.check("sms_attention_backward", st)
    return dq, dk, dv


def sms_max_sk(dtype):
    """Largest key length the library runs for a torch dtype."""
    return int(_lib.lib().sms_max_sk(_lib.DTYPE_CODES[_DTYPES[dtype]]))


def sms_path(dtype, Sk, backward=False):
    """Kernel family for (dtype, Sk): 0 rows-per-wave, 1 wave-per-row, 2 multi-wave."""
    return int(_lib.lib().sms_path(_lib.DTYPE_CODES[_DTYPES[dtype]], int(Sk), int(backward)))


def sms_copy_reference(src, dst, stream=None):
    """dst <- src as raw bytes through the library's plain 16-byte copy kernel
    (C ABI sms_copy_reference): the bandwidth reference for the softmax
    kernels, not part of the method. Both tensors contiguous, on the GPU, of
    the same byte size (a multiple of 16)."""
    _require_gpu(src, "src")
    _require_gpu(dst, "dst")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst must hold the same number of bytes")
    s = _stream_of(src.device, stream)
    _lib.check("sms_copy_reference",
               _lib.lib().sms_copy_reference(src.data_ptr(), dst.data_ptr(), n, s.cuda_stream))


def _rows_view(t):
    """t itself when its key axis is contiguous, else a contiguous copy."""
    return t if (t.shape[-1] <= 1 or t.stride(-1) == 1) else t.contiguous()


class ScaledMaskSoftmaxFunction(torch.autograd.Function):
    """Autograd wrapper: forward saves y only; backward returns (dx, None, None, None)."""

    @staticmethod
    def forward(ctx, x, mask, scale, is_causal):
        x = _rows_view(x)
        if mask is not None:
            if mask.dtype == torch.int64:  # key lengths: the C ABI takes int32
                mask = mask.to(torch.int32)
            if not mask.is_contiguous():
                mask = mask.contiguous()
        y = torch.empty_like(x, memory_format=torch.contiguous_format)
        sms_forward(x, mask, y, scale, is_causal)
        ctx.scale = float(scale)
        ctx.is_causal = causal_code(is_causal)
        ctx.save_for_backward(y)
        return y

    @staticmethod
    def backward(ctx, dy):
        (y,) = ctx.saved_tensors
        dy = _rows_view(dy)
        dx = torch.empty_like(y)
        sms_backward(y, dy, dx, ctx.scale, ctx.is_causal)
        return dx, None, None, None


def scaled_mask_softmax(x, mask=None, scale=1.0, is_causal=False):
    """softmax(x*scale + mask) over the last axis of a 4-D GPU tensor, differentiable in x.

    mask: None, an additive mask (x's dtype), a boolean mask (True = excluded)
    or integer key lengths [B]; is_causal: False, True ("top_left") or
    "bottom_right".
    """
    return ScaledMaskSoftmaxFunction.apply(x, mask, scale, is_causal)


class AttentionFunction(torch.autograd.Function):
    """Autograd wrapper of the fused attention: forward saves q, k, v, O and
    the log-sum-exp (no probabilities); backward returns (dQ, dK, dV, None...)."""

    @staticmethod
    def forward(ctx, q, k, v, mask, scale, is_causal):
        if mask is not None:
            if mask.dtype == torch.int64:  # key lengths: the C ABI takes int32
                mask = mask.to(torch.int32)
            if not mask.is_contiguous():
                mask = mask.contiguous()
        if scale is None:
            scale = 1.0 / float(q.shape[-1]) ** 0.5
        o, lse = sms_attention_forward(q, k, v, mask, scale, is_causal, return_lse=True)
        ctx.scale = float(scale)
        ctx.is_causal = causal_code(is_causal)
        ctx.save_for_backward(q, k, v, o, lse, mask)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, mask = ctx.saved_tensors
        if do.stride(-1) != 1 or do.data_ptr() % 16:
            do = do.contiguous()
        dq, dk, dv = sms_attention_backward(q, k, v, o, lse, do, mask, ctx.scale, ctx.is_causal)
        return dq, dk, dv, None, None, None


def attention(q, k, v, mask=None, scale=None, is_causal=False):
    """softmax(Q K^T * scale + mask) V on the fused kernels, differentiable in q, k and v.

    Shapes and mask forms as for ``sms_attention_forward``; ``scale`` defaults
    to 1/sqrt(D).
    """
    return AttentionFunction.apply(q, k, v, mask, scale, is_causal)
