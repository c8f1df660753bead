"""Input marshalling for the oracle: anything array-like becomes exact numpy.

Floating inputs are widened to float64 (exact for bf16 and fp32 values);
metadata becomes int64 so position differences cannot overflow.  Test
infrastructure only.
"""

import numpy as np


def f64(x):
    if hasattr(x, "detach"):  # a torch tensor; widening is exact
        import torch
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def i64(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu", torch.int64).numpy()
    return np.asarray(x, dtype=np.int64)
