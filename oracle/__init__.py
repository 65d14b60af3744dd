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
from .mlstm_grad import grad_fw, quadratic_fw_torch  # noqa: F401,E402
