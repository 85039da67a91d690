"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

None of these retypes the oracle's formula. They use hand-derived exact
examples (tests/golden/hand_examples.txt), closed forms (Q = 0, scale = 0,
constant V, causal row 0), invariants (key/value permutation, key shift,
linearity, convex bounds), an independent blockwise recurrence, and library
routines (torch softmax / logsumexp / scaled_dot_product_attention in fp64).
The last test plants plausible mistakes in copies of the oracle and shows that
each one trips at least one pin.
"""

import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attend_head, attention_ref
from tests.blockwise_ref import blockwise_head

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.txt")


# ---------------------------------------------------------------- fixtures --

def _entry(tok):
    tok = tok.strip()
    if tok == "-inf":
        return -math.inf
    if tok.startswith("ln(") and tok.endswith(")"):
        return math.log(float(Fraction(tok[3:-1])))
    return float(Fraction(tok))


def _matrix(text):
    return np.array([[_entry(t) for t in row.split(",")] for row in text.split(";")],
                    dtype=np.float64)


def load_golden():
    cases = []
    for block in re.split(r"^---$", open(GOLDEN).read(), flags=re.M):
        fields = {}
        for line in block.splitlines():
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
        if not fields:
            continue
        cases.append({
            "name": fields["name"],
            "scale": float(Fraction(fields["scale"])),
            "causal": bool(int(fields["causal"])),
            "Q": _matrix(fields["Q"]), "K": _matrix(fields["K"]),
            "V": _matrix(fields["V"]), "O": _matrix(fields["O"]),
            "lse": _matrix(fields["lse"])[:, 0],
        })
    return cases


GOLDEN_CASES = load_golden()


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# -------------------------------------------------------------------- pins --
# Each pin takes an attention function with attend_head's signature and
# returns True when it behaves as the pages and the mathematics require.

def pin_golden(attend):
    for c in GOLDEN_CASES:
        o, lse = attend(c["Q"], c["K"], c["V"], c["scale"], c["causal"])
        finite = np.isfinite(c["lse"])
        if not (np.allclose(o, c["O"], rtol=0, atol=1e-13)
                and np.array_equal(np.isfinite(lse), finite)
                and np.allclose(lse[finite], c["lse"][finite], rtol=0, atol=1e-13)
                and np.all(lse[~finite] == -np.inf)):
            return False
    return True


def pin_rows_are_distributions(attend):
    """Weights are distributions; causal weights vanish above the diagonal
    that ends both axes together (19 queries, 23 keys: query i at key i+4)."""
    q, k, v = _rand((19, 8), 1), _rand((23, 8), 2), _rand((23, 5), 3)
    for causal in (False, True):
        _, _, w = attend(q, k, v, 0.7, causal, return_weights=True)
        if np.abs(w.sum(axis=1) - 1).max() > 1e-14 or w.min() < 0:
            return False
        if causal and np.any(np.triu(w, 1 + 23 - 19) != 0):
            return False
        if causal and np.any(np.diagonal(w, 23 - 19) == 0):
            return False
    return True


def pin_uniform_when_scores_vanish(attend):
    """Q = 0 or scale = 0: every visible key gets the same weight."""
    n, d = 17, 6
    k, v = _rand((n, d), 4), _rand((n, 3), 5)
    for q, scale in ((np.zeros((n, d)), 0.9), (_rand((n, d), 6), 0.0)):
        o, lse = attend(q, k, v, scale, False)
        if not (np.allclose(o, v.mean(axis=0)[None, :], atol=1e-14)
                and np.allclose(lse, math.log(n), atol=1e-14)):
            return False
        o, lse = attend(q, k, v, scale, True)
        prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
        if not (np.allclose(o, prefix, atol=1e-14)
                and np.allclose(lse, np.log(np.arange(1, n + 1)), atol=1e-14)):
            return False
    return True


def pin_constant_values(attend):
    q, k = _rand((13, 4), 7, 3.0), _rand((13, 4), 8, 3.0)
    v = np.tile(np.array([[1.25, -3.5, 7.0]]), (13, 1))
    for causal in (False, True):
        o, _ = attend(q, k, v, 1.3, causal)
        if not np.allclose(o, v, atol=1e-13):
            return False
    return True


def pin_causal_first_row(attend):
    q, k, v = _rand((9, 4), 9), _rand((9, 4), 10), _rand((9, 2), 11)
    o, lse = attend(q, k, v, 0.45, True)
    return (np.allclose(o[0], v[0], atol=1e-15)
            and abs(lse[0] - 0.45 * float(q[0] @ k[0])) < 1e-14)


def pin_permutations(attend):
    q, k, v = _rand((11, 6), 12), _rand((15, 6), 13), _rand((15, 4), 14)
    o, lse = attend(q, k, v, 0.8, False)
    perm_kv = np.random.default_rng(15).permutation(15)
    o2, lse2 = attend(q, k[perm_kv], v[perm_kv], 0.8, False)
    perm_q = np.random.default_rng(16).permutation(11)
    o3, lse3 = attend(q[perm_q], k, v, 0.8, False)
    return (np.allclose(o2, o, atol=1e-13) and np.allclose(lse2, lse, atol=1e-13)
            and np.allclose(o3, o[perm_q], atol=1e-13)
            and np.allclose(lse3, lse[perm_q], atol=1e-13))


def pin_key_shift(attend):
    """K + 1 u^T: O unchanged, lse_i shifted by scale * <q_i, u>.

    A shift of size 1e3 puts the scores near +-1e3, far beyond exp's range,
    so this also pins the maximum subtraction."""
    q, k, v = _rand((10, 5), 17), _rand((12, 5), 18), _rand((12, 3), 19)
    for u_size in (1.0, 1e3):
        u = _rand((5,), 20, u_size)
        for causal in (False, True):
            o, lse = attend(q, k, v, 0.6, causal)
            o2, lse2 = attend(q, k + u[None, :], v, 0.6, causal)
            if not np.all(np.isfinite(o2)) or not np.all(np.isfinite(lse2)):
                return False
            tol = 1e-12 * max(1.0, u_size * 10)
            if not (np.allclose(o2, o, atol=1e-9)
                    and np.allclose(lse2, lse + 0.6 * (q @ u), atol=tol)):
                return False
    return True


def pin_linearity_and_bounds(attend):
    q, k = _rand((14, 4), 21), _rand((14, 4), 22)
    v1, v2 = _rand((14, 3), 23), _rand((14, 3), 24)
    for causal in (False, True):
        o1, lse = attend(q, k, v1, 1.1, causal)
        o2, _ = attend(q, k, v2, 1.1, causal)
        o12, _ = attend(q, k, v1 - 2.5 * v2, 1.1, causal)
        if not np.allclose(o12, o1 - 2.5 * o2, atol=1e-13):
            return False
        s = 1.1 * (q @ k.T)
        for i in range(14):
            vis = np.arange(i + 1) if causal else np.arange(14)
            smax = s[i, vis].max()
            if not (smax - 1e-13 <= lse[i] <= smax + math.log(len(vis)) + 1e-13):
                return False
            if (np.any(o1[i] < v1[vis].min(axis=0) - 1e-13)
                    or np.any(o1[i] > v1[vis].max(axis=0) + 1e-13)):
                return False
    return True


def pin_blockwise_recurrence(attend):
    """The online (running max / running sum) recurrence the kernel follows,
    written independently, equals the one-piece definition."""
    for n in (1, 2, 5, 16, 37):
        q, k, v = _rand((n, 7), 30 + n), _rand((n, 7), 31 + n), _rand((n, 3), 32 + n)
        for causal in (False, True):
            o, lse = attend(q, k, v, 0.9, causal)
            for blk in (1, 2, 3, 5, 7, n):
                ob, lseb = blockwise_head(q, k, v, 0.9, causal, blk)
                if np.abs(ob - o).max() > 1e-12 or np.abs(lseb - lse).max() > 1e-12:
                    return False
    return True


def pin_torch_library(attend):
    """Special case reducing to library routines: torch fp64 softmax, matmul,
    logsumexp and scaled_dot_product_attention on the CPU."""
    for causal in (False, True):
        q, k, v = _rand((33, 16), 40), _rand((33, 16), 41), _rand((33, 8), 42)
        o, lse = attend(q, k, v, 0.25, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        s = 0.25 * (tq @ tk.T)
        if causal:
            s = s.masked_fill(torch.ones(33, 33, dtype=torch.bool).triu(1), float("-inf"))
        o_t = torch.softmax(s, dim=-1) @ tv
        lse_t = torch.logsumexp(s, dim=-1)
        sdpa = torch.nn.functional.scaled_dot_product_attention(
            tq[None], tk[None], tv[None], is_causal=causal, scale=0.25)[0]
        if not (np.allclose(o, o_t.numpy(), atol=1e-12)
                and np.allclose(lse, lse_t.numpy(), atol=1e-12)
                and np.allclose(o, sdpa.numpy(), atol=1e-12)):
            return False
    return True


PINS = [pin_golden, pin_rows_are_distributions, pin_uniform_when_scores_vanish,
        pin_constant_values, pin_causal_first_row, pin_permutations,
        pin_key_shift, pin_linearity_and_bounds, pin_blockwise_recurrence,
        pin_torch_library]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    assert pin(attend_head)


# ----------------------------------------------------- oracle's own plumbing --

def test_batched_wrapper_matches_heads():
    q, k, v = _rand((2, 3, 9, 4), 50), _rand((2, 3, 9, 4), 51), _rand((2, 3, 9, 4), 52)
    for causal in (False, True):
        o, lse = attention_ref(q, k, v, 0.5, causal)
        assert o.shape == (2, 3, 9, 4) and lse.shape == (2, 3, 9)
        for b in range(2):
            for h in range(3):
                oh, lh = attend_head(q[b, h], k[b, h], v[b, h], 0.5, causal)
                assert np.array_equal(o[b, h], oh) and np.array_equal(lse[b, h], lh)


def test_golden_through_batched_wrapper():
    for c in GOLDEN_CASES:
        o, lse = attention_ref(c["Q"][None, None], c["K"][None, None],
                               c["V"][None, None], c["scale"], c["causal"])
        assert np.allclose(o[0, 0], c["O"], atol=1e-13)
        assert np.allclose(lse[0, 0], c["lse"], atol=1e-13)


def test_row_sample_positions_match_full():
    """Sampling query rows with their positions gives the full result's rows
    (how full-size parity checks sample outputs)."""
    q, k, v = _rand((40, 6), 60), _rand((40, 6), 61), _rand((40, 6), 62)
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        o, lse = attend_head(q, k, v, 0.3, causal)
        os_, ls = attend_head(q[rows], k, v, 0.3, causal, q_pos=rows)
        assert np.allclose(os_, o[rows], atol=1e-14)
        assert np.allclose(ls, lse[rows], atol=1e-14)


def test_chunking_does_not_change_result():
    q, k, v = _rand((25, 6), 70), _rand((25, 6), 71), _rand((25, 6), 72)
    for causal in (False, True):
        o, lse = attend_head(q, k, v, 0.3, causal)
        for chunk in (1, 4, 7):
            o2, l2 = attend_head(q, k, v, 0.3, causal, chunk=chunk)
            assert np.allclose(o2, o, atol=1e-14) and np.allclose(l2, lse, atol=1e-14)


def test_shape_errors():
    with pytest.raises(ValueError):
        attend_head(np.zeros((2, 3)), np.zeros((2, 4)), np.zeros((2, 4)), 1.0, False)
    with pytest.raises(ValueError):
        attention_ref(np.zeros((2, 3)), np.zeros((2, 3)), np.zeros((2, 3)), 1.0, False)


# --------------------------------------------- planted mistakes must be caught --

def _mutant(kind):
    """A copy of the oracle's computation with one plausible mistake planted."""
    def attend(q, k, v, scale, causal, q_pos=None, return_weights=False, chunk=1024):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        n_q, n_k = q.shape[0], k.shape[0]
        offset = 0 if kind == "top_left_alignment" else n_k - n_q
        pos = np.arange(n_q) + offset if q_pos is None else np.asarray(q_pos)
        if kind == "transposed_scores":
            if n_q != n_k:
                s = scale * (q @ k.T)
            else:
                s = scale * (k @ q.T)
        elif kind == "scale_dropped":
            s = q @ k.T
        elif kind == "scale_squared":
            s = scale * scale * (q @ k.T)
        else:
            s = scale * (q @ k.T)
        if causal:
            j = np.arange(n_k)[None, :]
            i = pos[:, None]
            hidden = {"causal_flipped": j < i, "causal_off_by_one": j >= i}.get(kind, j > i)
            s = np.where(hidden, -np.inf, s)
        m = s.max(axis=1, keepdims=True)
        empty = np.isneginf(m[:, 0])
        if kind != "empty_rows_nan":
            m[empty] = 0.0
        if kind == "no_max_subtraction":
            w = np.exp(s)
            m = np.zeros_like(m)
        elif kind == "softmax_over_queries":
            w = np.exp(s - s.max(axis=0, keepdims=True))
        else:
            w = np.exp(s - m)
        axis = 0 if kind == "softmax_over_queries" else 1
        l = w.sum(axis=axis, keepdims=True)
        if kind != "empty_rows_nan" and axis == 1:
            l[empty] = 1.0
        o = w @ v if kind == "not_normalised" else (w / l) @ v
        if kind == "values_rows_reversed":
            o = (w / l) @ v[::-1]
        lse_l = l[:, 0] if axis == 1 else l[0, :]
        if kind == "lse_base2":
            lse = m[:, 0] / math.log(2) + np.log2(lse_l)
        elif kind == "lse_without_max":
            lse = np.log(lse_l)
        elif kind == "lse_of_unscaled":
            lse = m[:, 0] / scale + np.log(lse_l) if scale != 0 else m[:, 0] + np.log(lse_l)
        else:
            lse = m[:, 0] + np.log(lse_l)
        if kind != "empty_rows_nan" and axis == 1:
            lse = np.where(empty, -np.inf, lse)
        if return_weights:
            return o, lse, w / l
        return o, lse
    return attend


MUTANTS = ["transposed_scores", "scale_dropped", "scale_squared", "causal_flipped",
           "causal_off_by_one", "no_max_subtraction", "softmax_over_queries",
           "not_normalised", "values_rows_reversed", "lse_base2", "lse_without_max",
           "lse_of_unscaled", "top_left_alignment", "empty_rows_nan"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    mutant = _mutant(kind)
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                ok = pin(mutant)
            except Exception:
                ok = False
            if not ok:
                caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {kind!r}"


def test_unmutated_copy_passes_every_pin():
    """The mutant scaffold itself, with no mistake planted, passes every pin, so
    a caught mutant is caught for its planted mistake alone."""
    clean = _mutant("none")
    for pin in PINS:
        assert pin(clean), pin.__name__
