"""Fused scaled-masked softmax for AMD MI355X (gfx950).

    y = softmax(x * scale + mask) over the key axis of x[B, H, Sq, Sk],
    optional causal rule (key k > query q masked), and its backward
    dx = scale * y * (dy - sum_k dy_k y_k).

``sms_forward`` / ``sms_backward`` are thin marshalling wrappers over the C ABI
functions of the same names in libsms.so (include/sms.h): every step of the
computation runs in the HIP kernels. ``scaled_mask_softmax`` wraps them in a
``torch.autograd.Function`` that saves only y for the backward, as in lmnt.cn
"Custom fused Softmax operator in CUDA, wrapped into PyTorch", sec. 4.3.

``sms_attention_forward`` / ``sms_attention_backward`` run the fused attention
softmax(Q K^T * scale + mask) V and its gradients on the matrix cores;
``attention`` is the differentiable wrapper.
"""

from ._lib import SmsError, lib  # noqa: F401
from .ops import (  # noqa: F401
    AttentionFunction,
    ScaledMaskSoftmaxFunction,
    attention,
    causal_code,
    mask_kind_of,
    mask_mode_of,
    scaled_mask_softmax,
    sms_attention_backward,
    sms_attention_forward,
    sms_attention_workspace_bytes,
    sms_backward,
    sms_copy_reference,
    sms_forward,
    sms_forward_noalloc,
    sms_max_sk,
    sms_noalloc_scratch_bytes,
    sms_path,
    sms_workspace_bytes,
)
