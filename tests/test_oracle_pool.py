"""The process-pool helper the full-size parity tests use (CPU only): under
pytest, spawned workers run the oracle per head and report its errors."""

import multiprocessing as mp

import numpy as np

from oracle import attend_head
from tests.oracle_pool import head_errors, limit_blas_threads


def test_pool_reports_oracle_errors_per_head():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((300, 64)).astype(np.float32) for _ in range(3))
    o, lse = attend_head(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                         0.125, True)
    o32, l32 = o.astype(np.float32), lse.astype(np.float32)
    jobs = [("exact", q, k, v, o32, l32, 0.125, True),
            ("off", q, k, v, o32 + 0.1, l32, 0.125, True),
            ("nan", q, k, v, np.full_like(o32, np.nan), l32, 0.125, True)]
    with mp.get_context("spawn").Pool(2, initializer=limit_blas_threads) as pool:
        res = {r[0]: r for r in pool.imap_unordered(head_errors, jobs)}
    assert res["exact"][1] < 1e-6 and res["exact"][2] < 1e-5 and res["exact"][3]
    assert abs(res["off"][1] - 0.1) < 1e-5
    assert not res["nan"][3]
