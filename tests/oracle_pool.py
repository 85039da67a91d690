"""Per-head oracle comparisons for a process pool (numpy and the oracle only;
the workers never touch the GPU). Used by the parity tests to check full-size
workloads element by element across the host cores."""

import numpy as np

from oracle import attend_head


def limit_blas_threads(threads=1):
    """Pool initializer: `threads` BLAS threads per worker process."""
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(threads)
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


def head_grad_errors(job):
    """job = (tag, q, k, v, do, dq, dk, dv, scale, causal) for one head (float32
    holding exact bf16 values). Returns (tag, [(max |err|, max |ref|,
    ||err||_F, ||ref||_F, all finite)] for dq, dk, dv)."""
    from oracle import attend_head_grad

    tag, q, k, v, do, dq, dk, dv, scale, causal = job
    refs = attend_head_grad(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            do.astype(np.float64), scale, causal)
    out = []
    for got, ref in zip((dq, dk, dv), refs):
        diff = got.astype(np.float64) - ref
        out.append((float(np.abs(diff).max()), float(np.abs(ref).max()),
                    float(np.linalg.norm(diff)), float(np.linalg.norm(ref)),
                    bool(np.all(np.isfinite(got)))))
    return tag, out
