"""Independent fp64 blockwise (online-softmax) attention, used only as a pin.

The kernel does not compute the softmax row in one piece: it walks the keys in
blocks, keeping a running maximum m, a running sum l and an unnormalised output
accumulator, and rescales both by exp(m_old - m_new) whenever the maximum grows.
The pages name this blockwise, fused computation ("[GPU] Deep Learning for
HPC", section "Flash Attention": tile the score matrix and keep it on chip) but
do not print the recurrence; this file writes the plain reading out in fp64 so
that a test can show it equals the oracle's one-piece definition up to
rounding. It shares no code with the oracle or with the HIP path.
"""

import math

import numpy as np


def blockwise_head(q, k, v, scale, causal, block):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, n_k = q.shape[0], k.shape[0]
    o = np.zeros((n_q, v.shape[1]))
    lse = np.zeros(n_q)
    for i in range(n_q):
        run_max = -math.inf
        run_sum = 0.0
        acc = np.zeros(v.shape[1])
        last = min(i, n_k - 1) if causal else n_k - 1
        for j0 in range(0, last + 1, block):
            j1 = min(j0 + block, last + 1)
            s = scale * (k[j0:j1] @ q[i])
            new_max = max(run_max, float(s.max()))
            alpha = math.exp(run_max - new_max) if run_max != -math.inf else 0.0
            p = np.exp(s - new_max)
            run_sum = run_sum * alpha + float(p.sum())
            acc = acc * alpha + p @ v[j0:j1]
            run_max = new_max
        o[i] = acc / run_sum
        lse[i] = run_max + math.log(run_sum)
    return o, lse
