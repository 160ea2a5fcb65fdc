"""Float64 CPU oracle for the fused scaled-masked softmax and its backward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or loads
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (``attention_softmax_amd``) and never imports it.

What it computes is the plain definition of the operation, evaluated in float64
from the exact values of the typed inputs (every fp32, fp16 and bf16 value is
exactly representable as a float64):

* forward  -- lmnt.cn "Custom fused Softmax operator in CUDA, wrapped into
  PyTorch", sec. 1.2 (score = x*scale + mask, softmax over keys) and sec. 2.1
  (subtract the row maximum before exponentiating); the causal rule (key j > query
  i is masked) from sec. 1.2, applied after the additive mask as in sec. 3.1,
  with a bottom-right variant (offset Sk - Sq) for Sq != Sk; boolean masks
  that exclude keys inside the operator (pnsm.cn ScaledMaskSoftmax article,
  sec. 2.3) and key padding given as per-batch lengths;
* backward -- the same page, sec. 3.3: dx_i = scale * y_i * (dy_i - sum_j dy_j*y_j);
* fully-masked rows -- pnsm.cn article on a custom ScaledMaskSoftmax operator,
  sec. 4.2 / 4.3: such a row must not divide 0 by 0; it returns all zeros;
* fused attention (``oracle.attention``) -- O = softmax(Q K^T * scale + mask) V
  and the rows' log-sum-exp, the fusion of the QK^T product into the operator
  that the pnsm.cn article proposes in sec. 4.4, with the softmax step taken
  from this package's softmax oracle.

Every function here is pinned by tests in ``tests/test_oracle_pins.py``
(closed forms, invariants, brute force, finite differences, the explicit
Jacobian). Nothing in this package is "parity unpinned".
"""

from . import attention  # noqa: F401
from .softmax import (  # noqa: F401
    DTYPES,
    causal_offset,
    decode,
    forward,
    forward_row,
    forward_rows,
    backward,
    backward_row,
    backward_rows,
    row_index,
)
