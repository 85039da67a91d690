"""Parity of the HIP attention forward against the fp64 oracle (GPU only).

The bar, for bf16 inputs with fp32 accumulation: max |O - O_ref| <= 2e-2 and
max |lse - lse_ref| <= 1e-3, element by element, on the same seeded inputs.
Every call goes through the C ABI (the ctypes binding). Each GPU step prints
the case it runs first, so a failing run names it.
"""

import math

import numpy as np
import pytest
import torch

import tiled_attention_forward_02_amd as mi
from oracle import attend_head, attention_ref
from tiled_attention_forward_02_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    mi.load_library()


def run_gpu(inp, scale=None, causal=None, stream=None):
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    o, lse = mi.attn_fwd(q, k, v, scale=inp["scale"] if scale is None else scale,
                         causal=inp["causal"] if causal is None else causal,
                         stream=stream)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def as64(t):
    return t.to(torch.float64).numpy()


def check(o, lse, o_ref, lse_ref, what):
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    eo = float(np.abs(o - o_ref).max()) if o.size else 0.0
    el = float(np.abs(lse - lse_ref).max()) if lse.size else 0.0
    print(f"  {what}: max|dO|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= O_TOL, f"{what}: max |O - O_ref| = {eo}"
    assert el <= LSE_TOL, f"{what}: max |lse - lse_ref| = {el}"


# ---------------------------------------------- the five metric workloads --

@pytest.mark.parametrize("idx", [1, 2, 3])
def test_workload_full(idx):
    """Small workloads: every output element against the oracle."""
    w = WORKLOADS[idx - 1]
    announce(f"workload {w.name} full compare")
    inp = make_inputs(w)
    o, lse = run_gpu(inp)
    o_ref, lse_ref = attention_ref(as64(inp["q"]), as64(inp["k"]), as64(inp["v"]),
                                   inp["scale"], w.causal)
    check(o, lse, o_ref, lse_ref, w.name)


@pytest.mark.parametrize("idx", [4, 5])
def test_workload_every_element(idx):
    """Full-size workloads in the benchmark's launch (B=16, H=16, N=4096, d=128
    and the causal B=1, H=32, N=16384, d=128): every output element of every
    head against the oracle, the heads spread over host processes."""
    import multiprocessing as mp
    import os

    from tests.oracle_pool import head_errors, limit_blas_threads

    w = WORKLOADS[idx - 1]
    announce(f"workload {w.name} every element")
    inp = make_inputs(w)
    o, lse = run_gpu(inp)
    q, k, v = (inp[n].float().numpy() for n in ("q", "k", "v"))
    jobs = ((f"({b},{h})", q[b, h], k[b, h], v[b, h], o[b, h], lse[b, h], inp["scale"],
             w.causal) for b in range(w.B) for h in range(w.H))
    workers = min(16, os.cpu_count() or 1)
    worst_o = worst_l = 0.0
    done = 0
    with mp.get_context("spawn").Pool(workers, initializer=limit_blas_threads) as pool:
        for tag, eo, el, finite in pool.imap_unordered(head_errors, jobs):
            assert finite, f"{w.name} head {tag}: non-finite output"
            assert eo <= O_TOL, f"{w.name} head {tag}: max |O - O_ref| = {eo}"
            assert el <= LSE_TOL, f"{w.name} head {tag}: max |lse - lse_ref| = {el}"
            worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
            done += 1
            if done % 16 == 0 or done == w.B * w.H:
                print(f"  {done}/{w.B * w.H} heads: max|dO|={worst_o:.3e} "
                      f"max|dlse|={worst_l:.3e}", flush=True)
    assert done == w.B * w.H


# ------------------------------------------- ragged and small shapes --

RAGGED = [(1, 1, 1), (1, 2, 17), (2, 3, 100), (1, 2, 127), (1, 1, 129), (2, 2, 300),
          (1, 3, 513), (1, 1, 1000), (3, 5, 64), (1, 1, 256)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", RAGGED)
def test_ragged(B, H, N, d, causal):
    """Any N: partial query tiles, partial key tiles, N below one tile."""
    announce(f"ragged B={B} H={H} N={N} d={d} causal={causal}")
    w = WORKLOADS[1]
    inp = make_inputs(w, B=B, H=H, N=N, d=d, seed=1000 + N + d)
    o, lse = run_gpu(inp, causal=causal)
    o_ref, lse_ref = attention_ref(as64(inp["q"]), as64(inp["k"]), as64(inp["v"]),
                                   inp["scale"], causal)
    check(o, lse, o_ref, lse_ref, f"N={N} d={d} causal={causal}")


# ------------------------------------------------ closed forms on the GPU --

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(d, causal):
    announce(f"Q=0 d={d} causal={causal}")
    inp = make_inputs(WORKLOADS[1], B=1, H=2, N=333, d=d, seed=7)
    inp["q"] = torch.zeros_like(inp["q"])
    o, lse = run_gpu(inp, causal=causal)
    v = as64(inp["v"])
    n = np.arange(1, 334)
    if causal:
        o_ref = np.cumsum(v, axis=2) / n[None, None, :, None]
        lse_ref = np.broadcast_to(np.log(n), lse.shape)
    else:
        o_ref = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        lse_ref = np.full(lse.shape, math.log(333))
    check(o, lse, o_ref, lse_ref, "Q=0")


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale(causal):
    announce(f"scale=0 causal={causal}")
    inp = make_inputs(WORKLOADS[1], B=1, H=2, N=200, d=64, seed=8)
    o, lse = run_gpu(inp, scale=0.0, causal=causal)
    o_ref, lse_ref = attention_ref(as64(inp["q"]), as64(inp["k"]), as64(inp["v"]),
                                   0.0, causal)
    check(o, lse, o_ref, lse_ref, "scale=0")


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values(causal):
    announce(f"constant V causal={causal}")
    inp = make_inputs(WORKLOADS[1], B=2, H=2, N=190, d=128, seed=9)
    inp["v"] = torch.full_like(inp["v"], 0.375)
    o, _ = run_gpu(inp, causal=causal)
    assert np.abs(o - 0.375).max() <= O_TOL


@pytest.mark.parametrize("scale", [-0.125, 0.9, -2.0, 5.0])
@pytest.mark.parametrize("causal", [False, True])
def test_other_scales(scale, causal):
    """Negative scales and peaky softmax (large scale) follow the definition."""
    announce(f"scale={scale} causal={causal}")
    inp = make_inputs(WORKLOADS[1], B=1, H=2, N=257, d=64, seed=10)
    o, lse = run_gpu(inp, scale=scale, causal=causal)
    o_ref, lse_ref = attention_ref(as64(inp["q"]), as64(inp["k"]), as64(inp["v"]),
                                   np.float32(scale), causal)
    check(o, lse, o_ref, lse_ref, f"scale={scale}")


def max_key_length(d):
    """Largest Nk the library accepts at head dim d: one head's key tensor plus
    one 128-row tile of slack must stay below 2^31 bytes (its buffer offsets
    are 32-bit), as include/mi_attn.h states for ATTN_ERR_SHAPE."""
    return (2**31 - 1 - 128 * d * 2) // (d * 2)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_longest_key_axis(d):
    """The longest key axis one head may have (K and V 2 GiB each), checked by
    closed forms, since the oracle cannot hold these tensors: needles at keys
    spread over the whole axis, its last row included, and Q = 0.

    Query i (i < Nq <= d) is 32 e_i and its needle key is 32 e_i; every other
    key is 0, so query i scores s = 1024 * scale on its needle and 0 on every
    other key. Then o_i = v_needle (the other weights are below 2^-130) and
    lse_i = s + ln(1 + (Nk - 1) e^-s). With Q = 0 every weight is 1:
    o_i = mean of V, lse_i = ln Nk."""
    Nk = max_key_length(d)
    Nq = min(64, d)
    announce(f"longest key axis: d={d} Nq={Nq} Nk={Nk}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(41 + d)
    v = torch.randn((1, 1, Nk, d), generator=g, device=dev, dtype=torch.float32)
    v = (v + 1.0).to(torch.bfloat16)
    k = torch.zeros((1, 1, Nk, d), device=dev, dtype=torch.bfloat16)
    q = torch.zeros((1, 1, Nq, d), device=dev, dtype=torch.bfloat16)
    half = Nq // 2
    # the second half of the needles sits in the last tile, up to row Nk - 1
    pos = [j * (Nk // half) + 7 * j for j in range(half)] + [Nk - 1 - j for j in range(Nq - half)]
    for i, pj in enumerate(pos):
        q[0, 0, i, i] = 32.0
        k[0, 0, pj, i] = 32.0
    scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    o, lse = mi.attn_fwd_cross(q, k, v, scale=scale, causal=False)
    torch.cuda.synchronize()
    s = 1024.0 * scale
    lse_ref = np.full(Nq, s + math.log1p((Nk - 1) * math.exp(-s)))
    o_ref = v[0, 0, pos].double().cpu().numpy()
    check(o[0, 0].float().cpu().numpy(), lse[0, 0].cpu().numpy(), o_ref, lse_ref,
          f"needles, d={d}")
    o0, lse0 = mi.attn_fwd_cross(torch.zeros_like(q), k, v, scale=scale, causal=False)
    torch.cuda.synchronize()
    mean = v[0, 0].mean(dim=0, dtype=torch.float64).cpu().numpy()
    check(o0[0, 0].float().cpu().numpy(), lse0[0, 0].cpu().numpy(),
          np.broadcast_to(mean, (Nq, d)), np.full(Nq, math.log(Nk)), f"Q = 0, d={d}")
    del v, k


def test_large_shift_of_keys():
    """A big common shift of all keys leaves O unchanged (needs the running
    maximum; scores reach about 2e2)."""
    announce("key shift")
    inp = make_inputs(WORKLOADS[3], B=1, H=1, N=300, d=128, seed=11)
    inp["k"] = (inp["k"].float() + 16.0).to(torch.bfloat16)
    inp["q"] = (inp["q"].float() + 1.0).to(torch.bfloat16)
    o, lse = run_gpu(inp)
    o_ref, lse_ref = attention_ref(as64(inp["q"]), as64(inp["k"]), as64(inp["v"]),
                                   inp["scale"], False)
    check(o, lse, o_ref, lse_ref, "key shift")


# ------------------------------------------------------- runtime behaviour --

def test_deterministic():
    announce("determinism")
    inp = make_inputs(WORKLOADS[2], B=2, H=4, N=700, d=64, seed=12)
    o1, l1 = run_gpu(inp)
    o2, l2 = run_gpu(inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_non_default_stream_and_preallocated_outputs():
    announce("side stream")
    inp = make_inputs(WORKLOADS[3], B=1, H=2, N=400, d=128, seed=13)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=dev)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        mi.attn_fwd(q, k, v, scale=inp["scale"], causal=True, out=out, lse=lse)
    s.synchronize()
    o_ref, lse_ref = attention_ref(as64(inp["q"]), as64(inp["k"]), as64(inp["v"]),
                                   inp["scale"], True)
    check(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "side stream")


def test_empty_batch_is_a_no_op():
    announce("empty")
    dev = torch.device("cuda:0")
    q = torch.zeros(0, 4, 128, 64, dtype=torch.bfloat16, device=dev)
    o, lse = mi.attn_fwd(q, q, q)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (0, 4, 128)


def test_rejections_leave_outputs_untouched():
    announce("rejection")
    dev = torch.device("cuda:0")
    q = torch.randn(1, 1, 64, 64, device=dev).to(torch.bfloat16)
    out = torch.full_like(q, 7.0)
    lse = torch.full((1, 1, 64), 7.0, device=dev)
    with pytest.raises(mi.AttnError):
        mi.attn_fwd(q, q, q, scale=float("nan"), out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out == 7).all()) and bool((lse == 7).all())


# ---------------------------------------------- queries and keys of two lengths --

def run_cross(q, k, v, scale, causal):
    dev = torch.device("cuda:0")
    o, lse = mi.attn_fwd_cross(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def check_with_empty_rows(o, lse, o_ref, lse_ref, what):
    """Like check(), but rows that see no key must be exactly o = 0, lse = -inf."""
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    assert np.all(o[empty] == 0.0), f"{what}: empty rows must be zero"
    check(o[~empty], lse[~empty], o_ref[~empty], lse_ref[~empty], what)


CROSS = [(1, 1), (3, 2), (2, 3), (100, 37), (37, 100), (129, 1000), (1000, 129),
         (256, 64), (64, 256), (200, 1)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", CROSS)
def test_cross_lengths(Nq, Nk, d, causal):
    """Nq queries against Nk keys, causal aligned at the ends of both axes."""
    announce(f"cross Nq={Nq} Nk={Nk} d={d} causal={causal}")
    qi = make_inputs(WORKLOADS[1], B=2, H=2, N=Nq, d=d, seed=2000 + Nq)
    ki = make_inputs(WORKLOADS[1], B=2, H=2, N=Nk, d=d, seed=3000 + Nk)
    o, lse = run_cross(qi["q"], ki["k"], ki["v"], qi["scale"], causal)
    o_ref, lse_ref = attention_ref(as64(qi["q"]), as64(ki["k"]), as64(ki["v"]),
                                   qi["scale"], causal)
    check_with_empty_rows(o, lse, o_ref, lse_ref, f"cross {Nq}x{Nk}")


def test_cross_without_keys():
    announce("cross Nk=0")
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 70, 64).to(torch.bfloat16).to(dev)
    k = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    o, lse = mi.attn_fwd_cross(q, k, k, causal=False)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_cross_equals_self_attention_when_lengths_match():
    announce("cross == self")
    inp = make_inputs(WORKLOADS[3], B=1, H=2, N=300, d=128, seed=14)
    dev = torch.device("cuda:0")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    for causal in (False, True):
        o1, l1 = mi.attn_fwd(q, k, v, scale=inp["scale"], causal=causal)
        o2, l2 = mi.attn_fwd_cross(q, k, v, scale=inp["scale"], causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_hand_examples_on_gpu():
    """The hand-derived examples, zero-padded to d=64 (scores unchanged, the
    padded output columns are 0), against the oracle on the same bf16 values."""
    from tests.test_oracle import GOLDEN_CASES
    for c in GOLDEN_CASES:
        announce(f"golden {c['name']}")
        def pad(a):
            t = torch.zeros(1, 1, a.shape[0], 64, dtype=torch.float64)
            t[0, 0, :, :a.shape[1]] = torch.from_numpy(a)
            return t.to(torch.bfloat16)
        q, k, v = pad(c["Q"]), pad(c["K"]), pad(c["V"])
        scale = float(np.float32(c["scale"]))
        o, lse = run_cross(q, k, v, scale, c["causal"])
        o_ref, lse_ref = attention_ref(as64(q), as64(k), as64(v), scale, c["causal"])
        check_with_empty_rows(o, lse, o_ref, lse_ref, c["name"])
        # and the exact values, within the bf16 rounding of the inputs
        nd = c["O"].shape[1]
        fin = np.isfinite(c["lse"])
        assert np.allclose(o[0, 0, :, :nd], c["O"], atol=0.05)
        assert np.allclose(lse[0, 0][fin], c["lse"][fin], atol=0.05)


# ------------------------------------------- float16 and head dims 32, 256 --

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


def run_ex(q, k, v, scale, causal):
    dev = torch.device("cuda:0")
    o, lse = mi.attn_fwd_ex(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == q.dtype
    return o.float().cpu().numpy(), lse.cpu().numpy()


EX_SELF = [(1, 1, 1), (1, 2, 17), (2, 3, 100), (1, 1, 129), (2, 2, 300), (1, 3, 513),
           (1, 1, 1000)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", EX_SELF)
def test_ex_self(B, H, N, d, causal, dt):
    """Every head dim in both element types, Nq == Nk, ragged N."""
    announce(f"ex self B={B} H={H} N={N} d={d} causal={causal} {dt}")
    inp = make_inputs(WORKLOADS[1], B=B, H=H, N=N, d=d, seed=4000 + N + d, dtype=DTYPES[dt])
    o, lse = run_ex(inp["q"], inp["k"], inp["v"], inp["scale"], causal)
    o_ref, lse_ref = attention_ref(as64(inp["q"]), as64(inp["k"]), as64(inp["v"]),
                                   inp["scale"], causal)
    check(o, lse, o_ref, lse_ref, f"N={N} d={d} causal={causal} {dt}")


EX_CROSS = [(1, 1), (3, 2), (100, 37), (37, 100), (129, 1000), (1000, 129), (200, 1)]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", EX_CROSS)
def test_ex_cross(Nq, Nk, d, causal, dt):
    announce(f"ex cross Nq={Nq} Nk={Nk} d={d} causal={causal} {dt}")
    qi = make_inputs(WORKLOADS[1], B=2, H=2, N=Nq, d=d, seed=5000 + Nq, dtype=DTYPES[dt])
    ki = make_inputs(WORKLOADS[1], B=2, H=2, N=Nk, d=d, seed=6000 + Nk, dtype=DTYPES[dt])
    o, lse = run_ex(qi["q"], ki["k"], ki["v"], qi["scale"], causal)
    o_ref, lse_ref = attention_ref(as64(qi["q"]), as64(ki["k"]), as64(ki["v"]),
                                   qi["scale"], causal)
    check_with_empty_rows(o, lse, o_ref, lse_ref, f"cross {Nq}x{Nk} d={d} {dt}")


@pytest.mark.parametrize("d", [32, 96, 256])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_ex_without_keys(d, dt):
    announce(f"ex Nk=0 d={d} {dt}")
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 70, d).to(DTYPES[dt]).to(dev)
    k = torch.zeros(1, 2, 0, d, dtype=DTYPES[dt], device=dev)
    o, lse = mi.attn_fwd_ex(q, k, k, causal=True)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_ex_bf16_is_attn_fwd_cross():
    """The bf16 path of attn_fwd_ex is the kernel attn_fwd_cross runs."""
    announce("ex bf16 == cross")
    qi = make_inputs(WORKLOADS[3], B=1, H=2, N=300, d=128, seed=15)
    ki = make_inputs(WORKLOADS[3], B=1, H=2, N=170, d=128, seed=16)
    dev = torch.device("cuda:0")
    q, k, v = qi["q"].to(dev), ki["k"].to(dev), ki["v"].to(dev)
    for causal in (False, True):
        o1, l1 = mi.attn_fwd_cross(q, k, v, causal=causal)
        o2, l2 = mi.attn_fwd_ex(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("d", [32, 96, 256])
def test_ex_zero_query_gives_mean_of_visible_values(d, dt):
    """q = 0: every visible key has weight 1/count, so O is a running mean of
    V and lse = ln(count), at any size."""
    announce(f"ex zero query d={d} {dt}")
    N = 777
    dev = torch.device("cuda:0")
    g = torch.Generator("cpu").manual_seed(d)
    v = torch.randn(1, 2, N, d, generator=g).to(DTYPES[dt])
    k = torch.randn(1, 2, N, d, generator=g).to(DTYPES[dt])
    q = torch.zeros(1, 2, N, d, dtype=DTYPES[dt])
    o, lse = run_ex(q, k, v, 0.3, True)
    cnt = np.arange(1, N + 1, dtype=np.float64)
    mean = np.cumsum(as64(v), axis=2) / cnt[None, None, :, None]
    check(o, lse, mean, np.broadcast_to(np.log(cnt), lse.shape), f"zero query d={d} {dt}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("d,N,causal", [(32, 16384, True), (96, 16384, True),
                                        (256, 8192, False), (256, 8192, True)])
def test_ex_long_sampled(d, N, causal, dt):
    """Long sequences at the other head dims: 48 sampled rows per head (the first,
    the last, and rows around tile edges) against the oracle row by row."""
    announce(f"ex long d={d} N={N} causal={causal} {dt}")
    inp = make_inputs(WORKLOADS[4], B=1, H=4, N=N, d=d, seed=7000 + d, dtype=DTYPES[dt])
    o, lse = run_ex(inp["q"], inp["k"], inp["v"], inp["scale"], causal)
    rng = np.random.default_rng(d + N)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N - 129, N - 1],
                                     rng.integers(0, N, 42)]))
    q64, k64, v64 = as64(inp["q"]), as64(inp["k"]), as64(inp["v"])
    for h in range(4):
        o_ref, lse_ref = attend_head(q64[0, h, rows], k64[0, h], v64[0, h], inp["scale"],
                                     causal, q_pos=rows)
        check(o[0, h, rows], lse[0, h, rows], o_ref, lse_ref, f"head {h}")


# d = 128 picks its workgroup shape from the grid size: 512 query rows a
# workgroup (two blocks of 32 a wave, eight waves) when the grid still gives
# each CU two workgroups' worth, else 256 (two blocks, four waves), else 128
# (one block, four waves). d = 96 takes the 512-row shape (the ping-pong
# kernel) when the grid gives every CU two workgroups, else 128 rows. Each
# case below lands on one shape, with ragged lengths and (causal) Nq != Nk,
# checked on sampled rows of a few heads. d = 256 takes eight one-block waves
# on grids of two full rounds of one workgroup per CU, d = 32 on grids of two
# full rounds of two per CU, else four.
SHAPES = [
    # (d, B, H, Nq, Nk, causal, rows per workgroup, element type)
    (128, 8, 16, 4000, 4000, False, 512, "bf16"),
    (128, 8, 16, 4000, 4000, True, 512, "bf16"),
    (128, 8, 16, 3000, 4100, True, 512, "bf16"),
    (128, 8, 16, 4000, 4000, True, 512, "f16"),
    (128, 2, 16, 4000, 4000, False, 256, "bf16"),
    (128, 2, 16, 4000, 4000, True, 256, "bf16"),
    (128, 2, 16, 3900, 1500, True, 256, "bf16"),
    (128, 1, 16, 4000, 4000, True, 128, "bf16"),
    (64, 4, 16, 4100, 4100, False, 512, "bf16"),
    (64, 4, 16, 4100, 4100, True, 512, "f16"),
    (64, 5, 16, 4096, 6000, True, 512, "bf16"),
    (64, 4, 16, 4000, 4000, True, 128, "bf16"),
    (96, 4, 16, 4000, 4000, False, 512, "bf16"),
    (96, 4, 16, 4000, 4000, True, 512, "bf16"),
    (96, 6, 16, 3000, 4100, True, 512, "bf16"),
    (96, 4, 16, 4000, 4000, False, 512, "f16"),
    (96, 2, 16, 4000, 4000, True, 128, "bf16"),
    (256, 2, 16, 4000, 4000, False, 256, "bf16"),
    (256, 3, 16, 3000, 4100, True, 256, "f16"),
    (256, 1, 16, 4000, 4000, True, 128, "bf16"),
    (32, 4, 16, 4000, 4000, True, 256, "bf16"),
    (32, 6, 16, 3000, 4100, False, 256, "f16"),
    (32, 2, 16, 4000, 4000, False, 128, "bf16"),
    # the ping-pong shapes with causal Nk < Nq: the first Nq - Nk rows see no
    # key (o = 0, lse = -inf), whole waves and workgroups among them
    (128, 8, 16, 4000, 1500, True, 512, "bf16"),
    (96, 8, 16, 4000, 1500, True, 512, "f16"),
    (64, 4, 16, 6000, 4100, True, 512, "bf16"),
    (256, 16, 16, 600, 300, True, 256, "bf16"),
]


@pytest.mark.parametrize("d,B,H,Nq,Nk,causal,rows,dt", SHAPES)
def test_workgroup_shapes(d, B, H, Nq, Nk, causal, rows, dt):
    announce(f"shapes d={d} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} rows={rows} {dt}")
    assert mi.attn_fwd_launch_shape(B, H, Nq, d, causal)["block_m"] == rows
    qi = make_inputs(WORKLOADS[3], B=B, H=H, N=Nq, d=d, seed=8100 + Nq + B + d,
                     dtype=DTYPES[dt])
    ki = qi if Nk == Nq else make_inputs(WORKLOADS[3], B=B, H=H, N=Nk, d=d,
                                         seed=8200 + Nk + d, dtype=DTYPES[dt])
    dev = torch.device("cuda:0")
    o, lse = mi.attn_fwd_ex(qi["q"].to(dev), ki["k"].to(dev), ki["v"].to(dev),
                            scale=qi["scale"], causal=causal)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(Nq + Nk + B)
    # the first and last rows, rows on both sides of workgroup and wave-block
    # edges, and random ones
    edges = [0, 31, 32, 63, 64, rows - 1, rows, 2 * rows - 1, Nq - rows, Nq - 33, Nq - 1]
    sample = np.unique(np.clip(np.concatenate([edges, rng.integers(0, Nq, 30)]), 0, Nq - 1))
    pos = sample + (Nk - Nq)
    for b, h in ((0, 0), (B // 2, H // 3), (B - 1, H - 1)):
        o_ref, lse_ref = attend_head(as64(qi["q"][b, h, sample]), as64(ki["k"][b, h]),
                                     as64(ki["v"][b, h]), qi["scale"], causal, q_pos=pos)
        check_with_empty_rows(o[b, h, sample], lse[b, h, sample], o_ref, lse_ref,
                              f"head ({b},{h})")


@pytest.mark.parametrize("d,rows", [(128, 512), (256, 256), (96, 512), (64, 512)])
@pytest.mark.parametrize("times", [-1.0, 0.0, 2.0])
@pytest.mark.parametrize("causal", [False, True])
def test_scales_on_the_eight_wave_shapes(d, rows, times, causal):
    """The big-grid workgroup shapes (eight waves, and two query blocks a wave
    at d = 64 and 128) with the scale negated, zero and doubled (times
    1/sqrt(d)): many short heads (N = 600; at d = 64, whose 512-row shape
    needs rows of 4096 or more, B=4 H=16 N=4096) make the grid big; every
    element of 14 heads spread over the batch against the oracle. (Much larger scales make the
    softmax nearly one-hot on rows that see few keys, |O| reaches 4 and more,
    and bf16's half-ulp there, 0.0156, with the weights' rounding can pass
    the 2e-2 bar on any kernel shape: 0.0207 and 0.0213 were measured at 8.8
    and 3.4 times 1/sqrt(d).)"""
    scale = times * float(torch.tensor(d ** -0.5, dtype=torch.float32))
    B, H, N = {256: (16, 16, 600), 64: (4, 16, 4096)}.get(d, (32, 16, 600))
    announce(f"eight-wave scales d={d} scale={scale} causal={causal}")
    assert mi.attn_fwd_launch_shape(B, H, N, d, causal)["block_m"] == rows
    inp = make_inputs(WORKLOADS[3], B=B, H=H, N=N, d=d, seed=9000 + d)
    o, lse = run_gpu(inp, scale=scale, causal=causal)
    for head in range(0, B * H, (B * H) // 13):
        b, h = divmod(head, H)
        o_ref, lse_ref = attend_head(as64(inp["q"][b, h]), as64(inp["k"][b, h]),
                                     as64(inp["v"][b, h]), np.float32(scale), causal)
        check(o[b, h], lse[b, h], o_ref, lse_ref, f"d={d} scale={scale} head ({b},{h})")


# --------------------------------------- the rounding bound at large scales --

def half_ulp(x, bits):
    """Half a unit in the last place of |x| in a binary format with `bits`
    significant bits (bf16: 8, fp16: 11), normal range; 0 at 0."""
    m, e = np.frexp(np.abs(x))  # |x| = m 2^e, m in [0.5, 1)
    return np.where(m > 0, np.ldexp(1.0, e - 1 - bits), 0.0)


# (d, times 1/sqrt(d), causal, every head or every 8th): the first two are
# where max |O - O_ref| was measured above 2e-2.
LARGE_SCALES = [(96, 8.8, False, True), (128, -3.4, True, True), (96, 8.8, True, False),
                (128, 8.8, False, False), (128, 3.4, False, False), (64, 8.8, True, False),
                (64, -3.4, False, False), (32, 8.8, True, False), (256, 8.8, False, False),
                (256, -3.4, True, False)]


@pytest.mark.parametrize("d,times,causal,all_heads", LARGE_SCALES)
def test_large_scale_rounding_bound(d, times, causal, all_heads):
    """With scales several times 1/sqrt(d) the softmax is nearly one-hot on
    many rows and |O| takes the size of single V entries, so the bf16
    roundings alone can pass 2e-2. What the arithmetic does bound, element by
    element: the weights are rounded to bf16 before P*V (relative error
    <= 2^-8 each, normalised by the sum of the unrounded fp32 weights), so
    the numerator is off by at most 2^-8 * A_ic with A_ic = sum_j w_ij |v_jc|
    (the attention output of |V|, from the oracle); O is then rounded to bf16
    (half an ulp of a value within that distance of O_ref). Scores, exp2,
    the fp32 sums and the division add far less than the 1e-4 * A_ic allowed
    on top. lse keeps its 1e-3 bar. Big grids, so the eight-wave (and at
    d = 128 two-block) workgroup shapes run."""
    base = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    scale = float(np.float32(times * base))
    B, H, N = (16, 16, 600) if d == 256 else (32, 16, 600)
    announce(f"large scale d={d} scale={scale} causal={causal} all_heads={all_heads}")
    inp = make_inputs(WORKLOADS[3], B=B, H=H, N=N, d=d, seed=9500 + d)
    o, lse = run_gpu(inp, scale=scale, causal=causal)
    heads = range(B * H) if all_heads else range(0, B * H, 8)
    worst_err = worst_ratio = worst_l = 0.0
    for head in heads:
        b, h = divmod(head, H)
        q, k, v = (as64(inp[n][b, h]) for n in ("q", "k", "v"))
        o_ref, lse_ref = attend_head(q, k, v, np.float32(scale), causal)
        a_abs, _ = attend_head(q, k, np.abs(v), np.float32(scale), causal)
        slack = 2.0 ** -8 + 1e-4
        bound = slack * a_abs + half_ulp(np.abs(o_ref) + slack * a_abs, 8) + 1e-6
        err = np.abs(o[b, h] - o_ref)
        assert np.all(np.isfinite(o[b, h])), f"head ({b},{h}): non-finite output"
        bad = err > bound
        assert not bad.any(), (f"head ({b},{h}): {int(bad.sum())} elements past the bound, "
                               f"e.g. err {err[bad][0]} bound {bound[bad][0]}")
        el = float(np.abs(lse[b, h] - lse_ref).max())
        assert el <= LSE_TOL, f"head ({b},{h}): max |lse - lse_ref| = {el}"
        worst_err = max(worst_err, float(err.max()))
        worst_ratio = max(worst_ratio, float((err / bound).max()))
        worst_l = max(worst_l, el)
    print(f"  max|dO|={worst_err:.3e} (largest share of the bound {worst_ratio:.3f}) "
          f"max|dlse|={worst_l:.3e}", flush=True)


# ------------------------------------------------- seeded random shapes --

def _random_shape_cases(n=40, seed=20261203, cap=1 << 25):
    """Shapes drawn at random with a fixed seed, across every head dim, both
    element types, with and without the mask, self and cross lengths (half
    log-uniform from 1, half from 2000 to 6000). Sizes go up to
    B*H*max(Nq, Nk)*d = cap (half the cases at the cap), so that about half
    land on the big-grid workgroup shapes and the rest on the small ones."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 64, 96, 128, 128, 256]))
        dt = "bf16" if rng.random() < 0.6 else "f16"
        causal = bool(rng.random() < 0.5)
        length = lambda: int(np.exp(rng.uniform(0.0, np.log(6000.0))) if rng.random() < 0.5
                             else rng.integers(2000, 6001))
        nq = length()
        nk = nq if rng.random() < 0.6 else length()
        bh_max = max(1, cap // (max(nq, nk) * d))
        bh = bh_max if rng.random() < 0.5 else int(np.exp(rng.uniform(0.0, np.log(bh_max))))
        H = max(h for h in (1, 2, 4, 8, 16) if h <= bh)
        B = max(1, bh // H)
        cases.append((d, B, H, nq, nk, causal, dt))
    return cases


@pytest.mark.parametrize("d,B,H,Nq,Nk,causal,dt", _random_shape_cases())
def test_random_shapes(d, B, H, Nq, Nk, causal, dt):
    rows_per_wg = mi.attn_fwd_launch_shape(B, H, Nq, d, causal)["block_m"]
    announce(f"random shape d={d} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} {dt} "
             f"rows/workgroup={rows_per_wg}")
    seed = 12000 + d + Nq + 7 * Nk + B
    qi = make_inputs(WORKLOADS[3], B=B, H=H, N=Nq, d=d, seed=seed, dtype=DTYPES[dt])
    ki = qi if Nk == Nq else make_inputs(WORKLOADS[3], B=B, H=H, N=Nk, d=d, seed=seed + 1,
                                         dtype=DTYPES[dt])
    dev = torch.device("cuda:0")
    o, lse = mi.attn_fwd_ex(qi["q"].to(dev), ki["k"].to(dev), ki["v"].to(dev),
                            scale=qi["scale"], causal=causal)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(seed)
    edges = [0, 31, 32, rows_per_wg - 1, rows_per_wg, Nq - 33, Nq - 1]
    sample = np.unique(np.clip(np.concatenate([edges, rng.integers(0, Nq, 20)]), 0, Nq - 1))
    pos = sample + (Nk - Nq)
    for b, h in ((0, 0), (B - 1, H - 1)):
        o_ref, lse_ref = attend_head(as64(qi["q"][b, h, sample]), as64(ki["k"][b, h]),
                                     as64(ki["v"][b, h]), qi["scale"], causal, q_pos=pos)
        check_with_empty_rows(o[b, h, sample], lse[b, h, sample], o_ref, lse_ref,
                              f"head ({b},{h})")
