"""Per-head oracle comparisons for a process pool (numpy and the oracle only;
the workers never touch the GPU). Used by the parity tests to check full-size
workloads element by element across the host cores."""

import numpy as np

from oracle import attend_head


def limit_blas_threads():
    """Pool initializer: one BLAS thread per worker process."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def head_errors(job):
    """job = (tag, q, k, v, o_gpu, lse_gpu, scale, causal) for one head, the
    inputs as float32 holding the exact bf16 values. Returns (tag, max |dO|,
    max |dlse|, all outputs finite)."""
    tag, q, k, v, o, lse, scale, causal = job
    o_ref, lse_ref = attend_head(q.astype(np.float64), k.astype(np.float64),
                                 v.astype(np.float64), scale, causal)
    finite = bool(np.all(np.isfinite(o)) and np.all(np.isfinite(lse)))
    return (tag, float(np.abs(o - o_ref).max()), float(np.abs(lse - lse_ref).max()), finite)
