"""Pins of the oracle's attention gradients (CPU only).

Every pin checks the gradient function against something other than its own
formula: hand-derived exact gradients, central finite differences of the
forward oracle, torch autograd, and identities that follow from the forward
definition (softmax rows are shift-invariant and sum to one). Each planted
mistake below must fail at least one pin.
"""

import functools
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attend_head, attend_head_grad, attention_grad_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_gradients.txt")


def _entry(tok):
    tok = tok.strip()
    if "*ln(" in tok:
        coef, arg = tok.split("*ln(")
        return float(Fraction(coef)) * math.log(float(Fraction(arg.rstrip(")"))))
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
        case = {"name": fields["name"], "scale": float(Fraction(fields["scale"])),
                "causal": bool(int(fields["causal"]))}
        for key in ("Q", "K", "V", "dO", "dQ", "dK", "dV"):
            case[key] = _matrix(fields[key])
        cases.append(case)
    return cases


GOLDEN_GRADS = load_golden()


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _visible(m, n, causal):
    """[m, n] boolean: key j visible to query i (ends of both axes aligned)."""
    pos = np.arange(m) + (n - m)
    return (np.arange(n)[None, :] <= pos[:, None]) if causal else np.ones((m, n), bool)


# Shapes used by the pins: square, more keys than queries, and more queries
# than keys (causal: the first rows see no key).
SHAPES = [(6, 6), (5, 9), (9, 4)]


def _safe(pin):
    def wrapped(grad):
        try:
            return bool(pin(grad))
        except (ValueError, IndexError, FloatingPointError):
            return False
    wrapped.__name__ = pin.__name__
    return wrapped


# -------------------------------------------------------------------- pins --
# Each pin takes a function with attend_head_grad's signature and returns True
# when it behaves as the forward definition and calculus require.

@_safe
def pin_golden(grad):
    for c in GOLDEN_GRADS:
        dq, dk, dv = grad(c["Q"], c["K"], c["V"], c["dO"], c["scale"], c["causal"])
        for got, want in ((dq, c["dQ"]), (dk, c["dK"]), (dv, c["dV"])):
            if got.shape != want.shape or not np.allclose(got, want, rtol=0, atol=1e-13):
                return False
    return True


def _loss(q, k, v, do, scale, causal):
    o, _ = attend_head(q, k, v, scale, causal)
    return float((o * do).sum())


@_safe
def pin_finite_differences(grad):
    """Central differences of L = sum(dO * O) through the forward oracle."""
    h = 1e-6
    for (m, n), causal, seed in ((SHAPES[0], False, 11), (SHAPES[1], True, 12),
                                 (SHAPES[2], True, 13), (SHAPES[2], False, 14)):
        d = 3
        q, k, v, do = (_rand((m, d), seed), _rand((n, d), seed + 1), _rand((n, d), seed + 2),
                       _rand((m, d), seed + 3))
        scale = 0.7
        got = grad(q, k, v, do, scale, causal)
        for idx, x in enumerate((q, k, v)):
            fd = np.zeros_like(x)
            for pos in np.ndindex(x.shape):
                keep = x[pos]
                x[pos] = keep + h
                up = _loss(q, k, v, do, scale, causal)
                x[pos] = keep - h
                down = _loss(q, k, v, do, scale, causal)
                x[pos] = keep
                fd[pos] = (up - down) / (2 * h)
            if got[idx].shape != fd.shape or not np.allclose(got[idx], fd, rtol=0, atol=1e-7):
                return False
    return True


@_safe
def pin_torch_autograd(grad):
    """torch's softmax and matmul backward in fp64 on the CPU (no empty rows)."""
    for (m, n), causal, seed in (((7, 7), False, 21), ((7, 7), True, 22), ((4, 10), True, 23)):
        d = 5
        q, k, v, do = (_rand((m, d), seed), _rand((n, d), seed + 1), _rand((n, d), seed + 2),
                       _rand((m, d), seed + 3))
        scale = 0.4
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = scale * tq @ tk.T
        if causal:
            s = s.masked_fill(~torch.tensor(_visible(m, n, True)), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        o.backward(torch.tensor(do))
        got = grad(q, k, v, do, scale, causal)
        for g, t in zip(got, (tq, tk, tv)):
            if not np.allclose(g, t.grad.numpy(), rtol=0, atol=1e-12):
                return False
    return True


@_safe
def pin_key_shift_invariance(grad):
    """Adding one vector u to every key adds scale*q_i.u to every visible score
    of row i, which the softmax ignores: so sum_j dK_j = 0."""
    for (m, n) in SHAPES:
        for causal in (False, True):
            q, k, v, do = (_rand((m, 4), 31), _rand((n, 4), 32), _rand((n, 4), 33),
                           _rand((m, 4), 34))
            _, dk, _ = grad(q, k, v, do, 0.8, causal)
            if not np.allclose(dk.sum(axis=0), 0.0, atol=1e-12):
                return False
    return True


@_safe
def pin_value_sums(grad):
    """Adding one vector u to every value adds u to every row that sees a key:
    so sum_j dV_j = sum of dO over rows that see at least one key."""
    for (m, n) in SHAPES:
        for causal in (False, True):
            q, k, v, do = (_rand((m, 4), 41), _rand((n, 4), 42), _rand((n, 4), 43),
                           _rand((m, 4), 44))
            _, _, dv = grad(q, k, v, do, 0.8, causal)
            seen = _visible(m, n, causal).any(axis=1)
            if not np.allclose(dv.sum(axis=0), do[seen].sum(axis=0), atol=1e-12):
                return False
    return True


@_safe
def pin_constant_values(grad):
    """Every value row equal to c makes O = c whatever Q and K are: dQ = dK = 0."""
    for (m, n) in SHAPES:
        for causal in (False, True):
            q, k, do = _rand((m, 4), 51), _rand((n, 4), 52), _rand((m, 4), 53)
            v = np.tile(_rand((1, 4), 54), (n, 1))
            dq, dk, _ = grad(q, k, v, do, 1.3, causal)
            if not (np.allclose(dq, 0.0, atol=1e-12) and np.allclose(dk, 0.0, atol=1e-12)):
                return False
    return True


@_safe
def pin_scale_identity(grad):
    """The scores depend on Q and K only through scale * Q K^T, so scaling Q by
    t and K by 1/t changes nothing: sum_i q_i.dQ_i = sum_j k_j.dK_j."""
    for (m, n) in SHAPES:
        for causal in (False, True):
            q, k, v, do = (_rand((m, 4), 61), _rand((n, 4), 62), _rand((n, 4), 63),
                           _rand((m, 4), 64))
            dq, dk, _ = grad(q, k, v, do, 0.9, causal)
            if not np.isclose((q * dq).sum(), (k * dk).sum(), rtol=0, atol=1e-12):
                return False
    return True


@_safe
def pin_uniform_weights_at_scale_zero(grad):
    """scale = 0: every visible key has weight 1/|J_i|, so dQ = dK = 0 and
    dV_j = sum over rows i that see j of dO_i / |J_i|."""
    for (m, n) in SHAPES:
        for causal in (False, True):
            q, k, v, do = (_rand((m, 4), 71), _rand((n, 4), 72), _rand((n, 4), 73),
                           _rand((m, 4), 74))
            dq, dk, dv = grad(q, k, v, do, 0.0, causal)
            vis = _visible(m, n, causal).astype(np.float64)
            cnt = vis.sum(axis=1, keepdims=True)
            w = np.divide(vis, cnt, out=np.zeros_like(vis), where=cnt > 0)
            if not (np.allclose(dq, 0, atol=1e-14) and np.allclose(dk, 0, atol=1e-14)
                    and np.allclose(dv, w.T @ do, atol=1e-13)):
                return False
    return True


@_safe
def pin_linear_in_upstream(grad):
    """The gradient of sum(dO * O) is linear in dO."""
    q, k, v = _rand((6, 4), 81), _rand((9, 4), 82), _rand((9, 4), 83)
    a, b = _rand((6, 4), 84), _rand((6, 4), 85)
    for causal in (False, True):
        ga = grad(q, k, v, a, 0.6, causal)
        gb = grad(q, k, v, b, 0.6, causal)
        gab = grad(q, k, v, a - 2.5 * b, 0.6, causal)
        for x, y, z in zip(ga, gb, gab):
            if not np.allclose(z, x - 2.5 * y, atol=1e-12):
                return False
    return True


@_safe
def pin_rows_without_keys_drop_out(grad):
    """Rows that see no key (causal, more queries than keys) have o = 0 for any
    input: their dQ is 0 and removing them leaves dK and dV unchanged."""
    m, n = 9, 4  # rows 0..4 see no key
    q, k, v, do = _rand((m, 4), 91), _rand((n, 4), 92), _rand((n, 4), 93), _rand((m, 4), 94)
    dq, dk, dv = grad(q, k, v, do, 1.1, True)
    dq2, dk2, dv2 = grad(q[5:], k, v, do[5:], 1.1, True)
    return (np.all(dq[:5] == 0) and np.allclose(dq[5:], dq2, atol=1e-13)
            and np.allclose(dk, dk2, atol=1e-13) and np.allclose(dv, dv2, atol=1e-13))


PINS = [pin_golden, pin_finite_differences, pin_torch_autograd, pin_key_shift_invariance,
        pin_value_sums, pin_constant_values, pin_scale_identity,
        pin_uniform_weights_at_scale_zero, pin_linear_in_upstream,
        pin_rows_without_keys_drop_out]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_grad_meets_pin(pin):
    assert pin(attend_head_grad)


@pytest.mark.parametrize("chunk", [1, 2, 3])
def test_chunked_oracle_grad_meets_every_pin(chunk):
    """The pins again with the query rows taken a few at a time, so that every
    pin shape (up to 9 rows) spans several chunks and a ragged last one: a
    chunk that drops its share of dk or dv, or writes dq rows in the wrong
    place, fails them."""
    grad = functools.partial(attend_head_grad, chunk=chunk)
    failed = [p.__name__ for p in PINS if not p(grad)]
    assert not failed, failed


def _dropped_chunk_share(q, k, v, do, scale, causal, q_pos=None):
    """A chunked gradient with one slip: dk and dv keep only the last chunk's
    share (assigned instead of added)."""
    q, k, v, do = (np.asarray(t, np.float64) for t in (q, k, v, do))
    m, n = q.shape[0], k.shape[0]
    pos = np.arange(m) + (n - m) if q_pos is None else np.asarray(q_pos)
    dq = np.empty_like(q)
    dk = dv = None
    for r0 in range(0, m, 2):
        rows = np.arange(r0, min(r0 + 2, m))
        dq[rows], dk, dv = attend_head_grad(q[rows], k, v, do[rows], scale, causal,
                                            q_pos=pos[rows])
    return dq, dk, dv


def test_dropped_chunk_share_fails_a_pin():
    assert [p.__name__ for p in PINS if not p(_dropped_chunk_share)]


@pytest.mark.parametrize("m,n", [(25, 25), (25, 40), (40, 25), (1, 30)])
def test_chunk_size_does_not_change_gradients(m, n):
    q, k, v, do = _rand((m, 6), 100), _rand((n, 6), 101), _rand((n, 6), 102), _rand((m, 6), 103)
    for causal in (False, True):
        ref = attend_head_grad(q, k, v, do, 0.45, causal)
        for chunk in (1, 4, 7, m):
            got = attend_head_grad(q, k, v, do, 0.45, causal, chunk=chunk)
            for g, r in zip(got, ref):
                assert g.shape == r.shape and np.allclose(g, r, rtol=0, atol=1e-13)


def test_row_sample_gradients_sum_to_the_full_key_side():
    """Because L sums over rows, dk and dv of a row subset (with its
    positions) summed over a partition of the rows equal the full result; this
    is how full-size parity builds the key-side gradients of long heads."""
    m = n = 37
    q, k, v, do = _rand((m, 5), 110), _rand((n, 5), 111), _rand((n, 5), 112), _rand((m, 5), 113)
    for causal in (False, True):
        dq, dk, dv = attend_head_grad(q, k, v, do, 0.6, causal)
        sk, sv = np.zeros_like(dk), np.zeros_like(dv)
        for rows in (np.arange(0, 10), np.arange(10, 31), np.arange(31, 37)):
            rq, rk, rv = attend_head_grad(q[rows], k, v, do[rows], 0.6, causal, q_pos=rows)
            assert np.allclose(rq, dq[rows], atol=1e-13)
            sk += rk
            sv += rv
        assert np.allclose(sk, dk, atol=1e-13) and np.allclose(sv, dv, atol=1e-13)


# ------------------------------------------------------------ planted mistakes --
# Each mutant is the oracle's chain rule with one plausible slip.

def _weights(q, k, scale, causal):
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    _, _, p = attend_head(q, k, np.zeros((k.shape[0], 1)), scale, causal, return_weights=True)
    return p


def _mutant(kind):
    def grad(q, k, v, do, scale, causal, q_pos=None):
        q, k, v, do = (np.asarray(t, np.float64) for t in (q, k, v, do))
        p = _weights(q, k, scale, False if kind == "unmasked" else causal)
        dv = p @ do if kind == "dv_untransposed" else p.T @ do
        dp = do @ v.T
        if kind == "no_row_term":
            ds = p * dp
        elif kind == "row_term_over_queries":
            ds = p * (dp - (p * dp).sum(axis=0, keepdims=True))
        elif kind == "sign_flipped":
            ds = p * ((p * dp).sum(axis=1, keepdims=True) - dp)
        elif kind == "row_term_without_weights":
            ds = p * (dp - dp.sum(axis=1, keepdims=True))
        else:
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if kind == "dk_without_scale":
            dk = ds.T @ q
        if kind == "dq_scale_squared":
            dq = scale * dq
        if kind == "dq_from_values":
            dq = scale * (ds @ v)
        if kind == "dk_from_upstream":
            dk = scale * (ds.T @ do)
        if kind == "dk_dq_swapped":
            dq, dk = scale * (ds.T @ q), scale * (ds @ k)
        return dq, dk, dv
    return grad


MUTANTS = ["no_row_term", "row_term_over_queries", "sign_flipped", "row_term_without_weights",
           "unmasked", "dk_without_scale", "dq_scale_squared", "dq_from_values",
           "dk_from_upstream", "dv_untransposed", "dk_dq_swapped"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_fails_a_pin(kind):
    wrong = _mutant(kind)
    failed = [p.__name__ for p in PINS if not p(wrong)]
    assert failed, f"mutant {kind} passes every pin"


def test_mutant_harness_reproduces_the_oracle():
    """The mutant template without a slip is the oracle (so the mutants differ
    from it only by their slip)."""
    clean = _mutant("none")
    assert all(p(clean) for p in PINS)


# ------------------------------------------------- the stored-output form --

@pytest.mark.parametrize("m,n", [(25, 25), (25, 40), (40, 25), (1, 2), (9, 1)])
def test_stored_output_form_equals_the_definition(m, n):
    """Given the exact output o (from attend_head), the row term rowsum(do * o)
    equals rowsum(P * dP) because o = P v, so the gradients agree with the
    plain form; small chunks check that o is sliced with its rows, and causal
    Nq > Nk includes rows that see no key (o = 0, no contribution)."""
    q, k, v, do = _rand((m, 6), 120), _rand((n, 6), 121), _rand((n, 6), 122), _rand((m, 6), 123)
    for causal in (False, True):
        o, _ = attend_head(q, k, v, 0.7, causal)
        ref = attend_head_grad(q, k, v, do, 0.7, causal)
        for chunk in (1, 4, 1024):
            got = attend_head_grad(q, k, v, do, 0.7, causal, chunk=chunk, o=o)
            for g, r in zip(got, ref):
                assert np.allclose(g, r, rtol=0, atol=1e-12)


def test_stored_output_moves_only_the_softmax_term():
    """dv = P^T do does not involve the output at all, and a rounded output
    moves dq and dk by an amount that vanishes with the rounding."""
    q, k, v, do = _rand((12, 5), 130), _rand((9, 5), 131), _rand((9, 5), 132), _rand((12, 5), 133)
    o, _ = attend_head(q, k, v, 0.5, True)
    ref = attend_head_grad(q, k, v, do, 0.5, True)
    rounded = np.round(o * 256) / 256
    got = attend_head_grad(q, k, v, do, 0.5, True, o=rounded)
    assert np.array_equal(got[2], ref[2])
    assert not np.allclose(got[0], ref[0], rtol=0, atol=1e-12)
    for g, r in zip(got[:2], ref[:2]):
        assert np.abs(g - r).max() <= 1e-2 * np.abs(r).max()
    with pytest.raises(ValueError):
        attend_head_grad(q, k, v, do, 0.5, True, o=o[:, :4])


# ------------------------------------------------------------------ plumbing --

def test_batched_equals_per_head():
    rng = np.random.default_rng(5)
    q, do = rng.standard_normal((2, 3, 7, 4)), rng.standard_normal((2, 3, 7, 4))
    k, v = rng.standard_normal((2, 3, 11, 4)), rng.standard_normal((2, 3, 11, 4))
    for causal in (False, True):
        dq, dk, dv = attention_grad_ref(q, k, v, do, 0.5, causal)
        for b in range(2):
            for h in range(3):
                r = attend_head_grad(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, causal)
                assert np.array_equal(dq[b, h], r[0]) and np.array_equal(dk[b, h], r[1])
                assert np.array_equal(dv[b, h], r[2])


def test_without_keys():
    dq, dk, dv = attend_head_grad(np.ones((3, 4)), np.zeros((0, 4)), np.zeros((0, 4)),
                                  np.ones((3, 4)), 0.5, False)
    assert dq.shape == (3, 4) and np.all(dq == 0) and dk.shape == (0, 4) and dv.shape == (0, 4)


def test_shape_errors():
    with pytest.raises(ValueError):
        attend_head_grad(np.ones((3, 4)), np.ones((5, 4)), np.ones((5, 4)), np.ones((3, 5)),
                         0.5, False)
