"""CPU oracle for the Mamba-2 SSD chunked forward.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path (the HIP library and
its Python binding) never does, and shares no code with it.

Contents
  recurrence : ``ssd_recurrence`` -- the token-by-token recurrence in plain C
               (fp64), the definition every other result is checked against;
               ``ssd_recurrence_f32``, its float instance, is the CPU
               baseline the benchmark times (not a parity reference).
  forms      : two independent restatements used to pin the recurrence --
               the quadratic semiseparable-matrix form and the four-stage
               chunked form -- plus the A = 0 closed form.
  rmsnorm    : ``rmsnorm_gated`` -- the gated grouped RMSNorm that follows
               chunk_scan in the chain (fp64 NumPy).
  varlen     : ``ssd_varlen`` -- packed variable-length sequences (state reset
               at each cu_seqlens start), the recurrence per sequence, and
               ``ssd_quadratic_seq_idx``, the same as one masked matrix.
  conv1d     : ``causal_conv1d`` -- the depthwise causal conv1d + bias + SiLU
               that precedes the SSD (fp64 NumPy).
  backward   : ``ssd_grads`` -- the gradients of the SSD forward, by
               autograd over the token recurrence in PyTorch fp64.

Parity status: every function here is pinned by ``tests/test_oracle.py``,
``tests/test_oracle_rmsnorm.py``, ``tests/test_oracle_varlen.py``,
``tests/test_oracle_conv1d.py`` or ``tests/test_oracle_backward.py``
(hand-derived golden values, closed forms, cross-form equality and
invariants); none is "parity unpinned".
"""
from .recurrence import (ssd_recurrence, ssd_recurrence_f32, build_oracle,  # noqa: F401
                         oracle_max_threads)
from .forms import (ssd_quadratic, ssd_chunked, ssd_linear_attention_closed_form,  # noqa: F401
                    discretize)
from .rmsnorm import rmsnorm_gated  # noqa: F401
from .varlen import ssd_quadratic_seq_idx, ssd_varlen  # noqa: F401
from .conv1d import causal_conv1d  # noqa: F401
from .backward import ssd_grads  # noqa: F401
