"""The tests' handle on the HIP path: the package's step runner (upload, buffers, one step,
host snapshot).  Imports no oracle code: the parity tests compare what it returns with the oracle."""
from mixture_experts_top_amd.runner import (Buffers, DevInputs, act_code, aux, bwd, dev_act, fwd, fwd_aux,  # noqa: F401
                                            run, snapshot, step, to_host, upload, wrap)
