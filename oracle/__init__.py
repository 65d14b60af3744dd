"""Float64 CPU oracle for the mLSTM forward pass and its gradients.

Test infrastructure only: the tests, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports, links or runs anything here, and nothing here imports the GPU
library.
"""
from .mlstm_oracle import (  # noqa: F401
    log_sigmoid,
    sigmoid,
    recurrent_fw,
    quadratic_fw,
    chunkwise_fw,
)
from .mlstm_q8 import q8_decode, q8_encode, q8_scaled, recurrent_step_q8  # noqa: F401,E402


def __getattr__(name):
    # The gradient oracle needs torch; it is imported on first use only, so
    # that the numpy forward oracle stays free of it.
    if name in ("grad_fw", "quadratic_fw_torch"):
        from . import mlstm_grad
        return getattr(mlstm_grad, name)
    raise AttributeError(name)
