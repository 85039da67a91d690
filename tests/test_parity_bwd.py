"""Parity of the HIP attention backward against the fp64 oracle (GPU only).

Each case runs the HIP forward (attn_fwd_ex) for o and lse, then attn_bwd,
and compares dq, dk, dv with the oracle's gradients of the same rounded
inputs. The bar, per gradient tensor X (bf16 or fp16 products, fp32
accumulation; P, dS and the outputs rounded to the element type, each about
2^-8 relative):

    max |X - X_ref|  <= 2e-2 * max |X_ref| + 1e-5
    ||X - X_ref||_F  <= 1e-2 * ||X_ref||_F + 1e-5 * sqrt(size)

The 1e-5 floor covers gradients that vanish exactly (one visible key gives
dS = P (dP - D) = 0, while the kernel's dP and D round differently in fp32).

delta (the row sums of dO * O, fp32) is checked against the same sums of the
GPU's own o, to 1e-5 relative. Every call goes through the C ABI (the ctypes
binding); each GPU step prints its case first.
"""

import numpy as np
import pytest
import torch

import tiled_attention_forward_02_amd as mi
from oracle import attend_head, attend_head_grad, attention_grad_ref
from tiled_attention_forward_02_amd.workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

MAX_TOL = 2e-2
FRO_TOL = 1e-2
ATOL = 1e-5
DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    mi.load_library()


def as64(t):
    return t.to(torch.float64).numpy()


def upstream(shape, seed, dtype):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def run(q, k, v, do, scale, causal):
    """GPU forward then backward; returns numpy dq, dk, dv, delta, o."""
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = mi.attn_fwd_ex(q, k, v, scale=scale, causal=causal)
    delta = torch.empty(lse.shape, dtype=torch.float32, device=dev)
    dq, dk, dv = mi.attn_bwd(q, k, v, o, lse, do, scale=scale, causal=causal, delta=delta)
    torch.cuda.synchronize()
    out = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    return out + [delta.cpu().numpy(), o.to(torch.float64).cpu().numpy()]


def check_grad(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    if ref.size == 0:
        return
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    fro = float(np.linalg.norm(got - ref))
    fro_ref = float(np.linalg.norm(ref))
    print(f"  {what}: max|err|={err:.3e} (max|ref|={scale:.3e}) fro={fro / max(fro_ref, 1e-300):.3e}",
          flush=True)
    assert err <= MAX_TOL * scale + ATOL, f"{what}: max error {err} vs max|ref| {scale}"
    assert fro <= FRO_TOL * fro_ref + ATOL * np.sqrt(ref.size), \
        f"{what}: Frobenius error {fro} vs {fro_ref}"


def check_all(q, k, v, do, scale, causal, what):
    dq, dk, dv, delta, o = run(q, k, v, do, scale, causal)
    rq, rk, rv = attention_grad_ref(as64(q), as64(k), as64(v), as64(do), scale, causal)
    check_grad(dq, rq, f"{what} dq")
    check_grad(dk, rk, f"{what} dk")
    check_grad(dv, rv, f"{what} dv")
    ref_delta = (as64(do) * o).sum(-1)
    assert np.allclose(delta, ref_delta, rtol=1e-5, atol=1e-5 * max(1.0, np.abs(ref_delta).max()))


# ------------------------------------------------------------ ragged shapes --

RAGGED = [(1, 1, 1), (1, 2, 17), (2, 3, 100), (1, 1, 129), (2, 2, 300), (1, 3, 513)]


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", RAGGED)
def test_bwd_ragged(B, H, N, d, causal):
    announce(f"bwd ragged B={B} H={H} N={N} d={d} causal={causal}")
    inp = make_inputs(WORKLOADS[1], B=B, H=H, N=N, d=d, seed=8000 + N + d)
    do = upstream(inp["q"].shape, 9000 + N + d, torch.bfloat16)
    check_all(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal, f"N={N} d={d}")


CROSS = [(3, 2), (2, 3), (100, 37), (37, 100), (129, 1000), (1000, 129), (200, 1), (1, 200)]


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", CROSS)
def test_bwd_cross(Nq, Nk, d, causal):
    """Nq queries against Nk keys; causal rows that see no key get no gradient."""
    announce(f"bwd cross Nq={Nq} Nk={Nk} d={d} causal={causal}")
    qi = make_inputs(WORKLOADS[1], B=2, H=2, N=Nq, d=d, seed=10000 + Nq)
    ki = make_inputs(WORKLOADS[1], B=2, H=2, N=Nk, d=d, seed=11000 + Nk)
    do = upstream(qi["q"].shape, 12000 + Nq + Nk, torch.bfloat16)
    check_all(qi["q"], ki["k"], ki["v"], do, qi["scale"], causal, f"cross {Nq}x{Nk}")


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [100, 300])
def test_bwd_fp16(N, d, causal):
    announce(f"bwd fp16 N={N} d={d} causal={causal}")
    inp = make_inputs(WORKLOADS[1], B=2, H=2, N=N, d=d, seed=13000 + N + d,
                      dtype=torch.float16)
    do = upstream(inp["q"].shape, 14000 + N, torch.float16)
    check_all(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal, f"fp16 N={N} d={d}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.9])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_other_scales(scale, causal):
    announce(f"bwd scale={scale} causal={causal}")
    inp = make_inputs(WORKLOADS[1], B=1, H=2, N=200, d=64, seed=15)
    do = upstream(inp["q"].shape, 16, torch.bfloat16)
    dq, dk, dv, _, _ = run(inp["q"], inp["k"], inp["v"], do, scale, causal)
    rq, rk, rv = attention_grad_ref(as64(inp["q"]), as64(inp["k"]), as64(inp["v"]), as64(do),
                                    scale, causal)
    if scale == 0.0:
        # uniform weights: dq = dk = 0 exactly
        assert np.all(dq == 0) and np.all(dk == 0)
    else:
        check_grad(dq, rq, "dq")
        check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


# --------------------------------------------------------------- edge cases --

@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_bwd_longest_key_axis(d):
    """Gradients on the longest key axis one head may have (K, V, dK, dV
    2 GiB each), checked by closed forms, since the oracle cannot hold these
    tensors. Query i (i < Nq <= d) is 32 e_i and its needle key 32 e_i, every
    other key 0: its weights are 1 on the needle and below 2^-130 elsewhere,
    so o_i = v_needle, and with D_i = dO_i . o_i every dS vanishes. Then
    dq = 0, dk = 0, and dv is dO_i on needle i's row and 0 on every other
    row. The outputs start as NaN, so a row left unwritten fails."""
    longest = (2**31 - 1 - 128 * d * 2) // (d * 2)
    Nq = min(64, d)
    announce(f"bwd longest key axis: d={d} Nq={Nq} Nk={longest}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(61 + d)
    v = torch.randn((1, 1, longest, d), generator=g, device=dev,
                    dtype=torch.float32).to(torch.bfloat16)
    do = torch.randn((1, 1, Nq, d), generator=g, device=dev,
                     dtype=torch.float32).to(torch.bfloat16)
    k = torch.zeros((1, 1, longest, d), device=dev, dtype=torch.bfloat16)
    q = torch.zeros((1, 1, Nq, d), device=dev, dtype=torch.bfloat16)
    half = Nq // 2
    pos = [j * (longest // half) + 7 * j for j in range(half)] + \
          [longest - 1 - j for j in range(Nq - half)]
    for i, pj in enumerate(pos):
        q[0, 0, i, i] = 32.0
        k[0, 0, pj, i] = 32.0
    scale = float(torch.tensor(d ** -0.5, dtype=torch.float32))
    o, lse = mi.attn_fwd_ex(q, k, v, scale=scale, causal=False)
    nan = float("nan")
    dq = torch.full_like(q, nan)
    dk = torch.full_like(k, nan)
    dv = torch.full_like(v, nan)
    mi.attn_bwd(q, k, v, o, lse, do, scale=scale, causal=False, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    dv_ref = torch.zeros_like(dv)
    dv_ref[0, 0, pos] = do[0, 0]
    errs = {"dq": float(dq.float().abs().max()),
            "dk": float(dk.float().abs().max()),
            "dv": float((dv.float() - dv_ref.float()).abs().max())}
    print(f"  max errors {errs}", flush=True)
    del k, dk, dv_ref
    assert all(np.isfinite(x) for x in errs.values()), errs
    assert errs["dq"] <= 1e-3 and errs["dk"] <= 1e-3, errs
    assert errs["dv"] <= MAX_TOL * float(do.float().abs().max()), errs


def test_bwd_one_side_empty():
    announce("bwd Nq=0 and Nk=0")
    dev = torch.device("cuda:0")
    k = torch.randn(1, 2, 50, 64).to(torch.bfloat16).to(dev)
    q0 = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    lse0 = torch.zeros(1, 2, 0, dtype=torch.float32, device=dev)
    dq, dk, dv = mi.attn_bwd(q0, k, k, q0, lse0, q0, causal=False)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and bool((dk == 0).all()) and bool((dv == 0).all())
    q = torch.randn(1, 2, 40, 64).to(torch.bfloat16).to(dev)
    k0 = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=dev)
    o, lse = mi.attn_fwd_ex(q, k0, k0, causal=True)
    do = torch.randn(1, 2, 40, 64).to(torch.bfloat16).to(dev)
    dq, dk, dv = mi.attn_bwd(q, k0, k0, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert bool((dq == 0).all()) and dk.numel() == 0 and dv.numel() == 0


EIGHT_WAVE = [(2100, 2100, False), (2100, 2200, False),
              (2100, 2100, True), (2100, 2300, True), (2300, 2100, True)]


@pytest.mark.parametrize("Nq,Nk,causal", EIGHT_WAVE)
def test_bwd_eight_wave_workgroups(Nq, Nk, causal):
    """d = 128, B*H = 64 heads of at least 2048 rows and keys
    (B*H*ceil(Nq/256) >= 512): the dQ side runs eight-wave workgroups of 256
    rows, the last one ragged, with or without the mask; without it the key
    side does too. With the mask and Nk < Nq the first Nq - Nk rows see no key
    (their dq is zero), and a workgroup's waves can stop at different keys.
    Two heads against the oracle, and four heads bit-identical to a call on
    just those heads, whose small grid runs four-wave workgroups: each row's
    dq and each key's dk, dv take the same tiles in the same order either
    way. The two-head calls get the big call's o and lse."""
    announce(f"bwd eight-wave workgroups Nq={Nq} Nk={Nk} d=128 causal={causal}")
    dev = torch.device("cuda:0")
    qi = make_inputs(WORKLOADS[1], B=4, H=16, N=Nq, d=128, seed=23000 + Nq)
    ki = make_inputs(WORKLOADS[1], B=4, H=16, N=Nk, d=128, seed=24000 + Nk)
    do = upstream(qi["q"].shape, 25000 + Nk, torch.bfloat16)
    scale = qi["scale"]
    q, k, v, dog = qi["q"].to(dev), ki["k"].to(dev), ki["v"].to(dev), do.to(dev)
    o, lse = mi.attn_fwd_ex(q, k, v, scale=scale, causal=causal)
    big = mi.attn_bwd(q, k, v, o, lse, dog, scale=scale, causal=causal)
    torch.cuda.synchronize()
    for b, hs in ((0, slice(0, 2)), (3, slice(14, 16))):
        part = mi.attn_bwd(*(t[b:b + 1, hs].contiguous() for t in (q, k, v, o, lse, dog)),
                           scale=scale, causal=causal)
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), big, part):
            assert torch.equal(x[b:b + 1, hs], y), f"batch {b} heads {hs}: {name} differs"
    q64, k64, v64, do64 = (as64(t) for t in (qi["q"], ki["k"], ki["v"], do))
    dq, dk, dv = (t.float().cpu().numpy() for t in big)
    if causal and Nk < Nq:
        assert not dq[:, :, :Nq - Nk].any(), "rows that see no key have a nonzero dq"
    for b, h in ((0, 0), (3, 15)):
        rq, rk, rv = attend_head_grad(q64[b, h], k64[b, h], v64[b, h], do64[b, h], scale, causal)
        check_grad(dq[b, h], rq, f"({b},{h}) dq")
        check_grad(dk[b, h], rk, f"({b},{h}) dk")
        check_grad(dv[b, h], rv, f"({b},{h}) dv")


def test_bwd_deterministic():
    announce("bwd deterministic")
    dev = torch.device("cuda:0")
    inp = make_inputs(WORKLOADS[1], B=2, H=4, N=700, d=128, seed=17)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    do = upstream(q.shape, 18, torch.bfloat16).to(dev)
    o, lse = mi.attn_fwd_ex(q, k, v, causal=True)
    a = mi.attn_bwd(q, k, v, o, lse, do, causal=True)
    b = mi.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bwd_non_default_stream_and_given_outputs():
    announce("bwd side stream")
    dev = torch.device("cuda:0")
    inp = make_inputs(WORKLOADS[1], B=1, H=2, N=300, d=64, seed=19)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    do = upstream(q.shape, 20, torch.bfloat16).to(dev)
    o, lse = mi.attn_fwd_ex(q, k, v, causal=False)
    ref = mi.attn_bwd(q, k, v, o, lse, do, causal=False)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    outs = [torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)]
    with torch.cuda.stream(s):
        mi.attn_bwd(q, k, v, o, lse, do, causal=False, dq=outs[0], dk=outs[1], dv=outs[2],
                    stream=s)
    s.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(ref, outs))


# ------------------------------------------------- the metric's workloads --

@pytest.mark.parametrize("idx,heads", [(1, None), (2, None), (3, ((0, 0), (7, 15)))])
def test_bwd_workloads(idx, heads):
    """Full size on the GPU; every element of the listed heads (all heads when
    None) against the oracle."""
    w = WORKLOADS[idx - 1]
    announce(f"bwd workload {w.name}")
    inp = make_inputs(w)
    do = upstream(inp["q"].shape, 20000 + idx, torch.bfloat16)
    dq, dk, dv, delta, o = run(inp["q"], inp["k"], inp["v"], do, inp["scale"], w.causal)
    q64, k64, v64, do64 = (as64(t) for t in (inp["q"], inp["k"], inp["v"], do))
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in heads:
        rq, rk, rv = attend_head_grad(q64[b, h], k64[b, h], v64[b, h], do64[b, h],
                                      inp["scale"], w.causal)
        check_grad(dq[b, h], rq, f"({b},{h}) dq")
        check_grad(dk[b, h], rk, f"({b},{h}) dk")
        check_grad(dv[b, h], rv, f"({b},{h}) dv")


def test_bwd_workload_every_element():
    """B=16, H=16, N=4096, d=128 at full size: every gradient element of every
    head against the oracle, the heads spread over host processes."""
    import multiprocessing as mp
    import os

    from tests.oracle_pool import head_grad_errors, limit_blas_threads

    w = WORKLOADS[3]
    announce(f"bwd workload {w.name} every element")
    inp = make_inputs(w)
    do = upstream(inp["q"].shape, 20004, torch.bfloat16)
    dq, dk, dv, _, _ = run(inp["q"], inp["k"], inp["v"], do, inp["scale"], w.causal)
    q, k, v, d_o = (t.float().numpy() for t in (inp["q"], inp["k"], inp["v"], do))
    jobs = ((f"({b},{h})", q[b, h], k[b, h], v[b, h], d_o[b, h], dq[b, h], dk[b, h], dv[b, h],
             inp["scale"], w.causal) for b in range(w.B) for h in range(w.H))
    worst = [0.0, 0.0, 0.0]
    done = 0
    with mp.get_context("spawn").Pool(min(16, os.cpu_count() or 1),
                                      initializer=limit_blas_threads) as pool:
        for tag, res in pool.imap_unordered(head_grad_errors, jobs):
            for i, (name, (err, ref, fro, fro_ref, finite)) in enumerate(zip(("dq", "dk", "dv"),
                                                                              res)):
                assert finite, f"head {tag} {name}: non-finite gradient"
                assert err <= MAX_TOL * ref + ATOL, f"head {tag} {name}: {err} vs {ref}"
                assert fro <= FRO_TOL * fro_ref + ATOL * np.sqrt(w.N * w.d), \
                    f"head {tag} {name}: Frobenius {fro} vs {fro_ref}"
                worst[i] = max(worst[i], err / ref if ref else 0.0)
            done += 1
            if done % 32 == 0 or done == w.B * w.H:
                print(f"  {done}/{w.B * w.H} heads: max err / max|ref| dq {worst[0]:.2e} "
                      f"dk {worst[1]:.2e} dv {worst[2]:.2e}", flush=True)
    assert done == w.B * w.H


def test_bwd_long_causal():
    """The long causal workload (B=1, H=32, N=16384, d=128) at full size: every
    gradient element of four heads against the oracle (whose gradient takes
    the query rows in chunks, so a head fits in host memory; the heads run in
    parallel host processes), dq on sampled rows of three more, and for every
    head the identities that hold at any size: sum_j dk_j = 0 and
    sum_j dv_j = sum_i do_i."""
    import multiprocessing as mp

    from tests.oracle_pool import head_grad_errors, limit_blas_threads

    w = WORKLOADS[4]
    announce(f"bwd workload {w.name}")
    inp = make_inputs(w)
    do = upstream(inp["q"].shape, 20005, torch.bfloat16)
    dq, dk, dv, _, _ = run(inp["q"], inp["k"], inp["v"], do, inp["scale"], True)
    q, k, v, d_o = (t.float().numpy() for t in (inp["q"], inp["k"], inp["v"], do))
    full = (0, 13, 22, 31)
    jobs = [(f"head {h}", q[0, h], k[0, h], v[0, h], d_o[0, h], dq[0, h], dk[0, h], dv[0, h],
             inp["scale"], True) for h in full]
    done = 0
    with mp.get_context("spawn").Pool(len(full), initializer=limit_blas_threads,
                                      initargs=(4,)) as pool:
        for tag, res in pool.imap_unordered(head_grad_errors, jobs):
            for name, (err, ref, fro, fro_ref, finite) in zip(("dq", "dk", "dv"), res):
                print(f"  {tag} {name}: max|err|={err:.3e} (max|ref|={ref:.3e}) "
                      f"fro={fro / max(fro_ref, 1e-300):.3e}", flush=True)
                assert finite, f"{tag} {name}: non-finite gradient"
                assert err <= MAX_TOL * ref + ATOL, f"{tag} {name}: {err} vs {ref}"
                assert fro <= FRO_TOL * fro_ref + ATOL * np.sqrt(w.N * w.d), \
                    f"{tag} {name}: Frobenius {fro} vs {fro_ref}"
            done += 1
    assert done == len(full)
    q64, k64, v64, do64 = (as64(t) for t in (inp["q"], inp["k"], inp["v"], do))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 127, 128, w.N - 1], rng.integers(0, w.N, 25)]))
    for h in (5, 17, 26):
        rq, _, _ = attend_head_grad(q64[0, h, rows], k64[0, h], v64[0, h], do64[0, h, rows],
                                    inp["scale"], True, q_pos=rows)
        check_grad(dq[0, h, rows], rq, f"head {h} dq rows")
    # Each identity is compared with the size of the terms it sums.
    dk64, dv64 = dk.astype(np.float64), dv.astype(np.float64)
    assert np.abs(dk64.sum(axis=2)).max() <= 1e-2 * np.abs(dk64).sum(axis=2).max()
    gap = np.abs(dv64.sum(axis=2) - do64.sum(axis=2)).max()
    assert gap <= 1e-2 * max(np.abs(dv64).sum(axis=2).max(), np.abs(do64).sum(axis=2).max())


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_bwd_long_other_head_dims(d):
    """N = 4096 at every head dim the backward takes, with and without the
    causal mask: two heads' every gradient element against the oracle, at
    full size on the GPU (B=2, H=4)."""
    announce(f"bwd long d={d}")
    w = WORKLOADS[3]
    inp = make_inputs(w, B=2, H=4, N=4096, d=d, seed=21000 + d)
    do = upstream(inp["q"].shape, 22000 + d, torch.bfloat16)
    for causal in (False, True):
        dq, dk, dv, _, _ = run(inp["q"], inp["k"], inp["v"], do, inp["scale"], causal)
        q64, k64, v64, do64 = (as64(t) for t in (inp["q"], inp["k"], inp["v"], do))
        for b, h in ((0, 0), (1, 3)):
            rq, rk, rv = attend_head_grad(q64[b, h], k64[b, h], v64[b, h], do64[b, h],
                                          inp["scale"], causal)
            check_grad(dq[b, h], rq, f"({b},{h}) causal={causal} dq")
            check_grad(dk[b, h], rk, f"({b},{h}) causal={causal} dk")
            check_grad(dv[b, h], rv, f"({b},{h}) causal={causal} dv")


# ------------------------------------------------------- random shapes --

def _random_bwd_cases(n=24, seed=20261204, cap=1 << 25):
    """Shapes drawn at random with a fixed seed, across every head dim, both
    element types, with and without the mask, self and cross lengths (half
    log-uniform from 1, half from 2048 to 4500). Sizes go up to
    B*H*max(Nq, Nk)*d = cap (half the cases at the cap), so that some d = 128
    cases land on the eight-wave shapes (B*H*ceil(N/256) >= 512 with both
    lengths at least 2048) and the rest on four-wave workgroups."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 96, 128, 128, 256]))
        dt = "bf16" if rng.random() < 0.6 else "f16"
        causal = bool(rng.random() < 0.5)
        length = lambda: int(np.exp(rng.uniform(0.0, np.log(4500.0))) if rng.random() < 0.5
                             else rng.integers(2048, 4501))
        nq = length()
        nk = nq if rng.random() < 0.6 else length()
        bh_max = max(1, cap // (max(nq, nk) * d))
        bh = bh_max if rng.random() < 0.5 else int(np.exp(rng.uniform(0.0, np.log(bh_max))))
        H = max(h for h in (1, 2, 4, 8, 16) if h <= bh)
        B = max(1, bh // H)
        cases.append((d, B, H, nq, nk, causal, dt))
    return cases


@pytest.mark.parametrize("d,B,H,Nq,Nk,causal,dt", _random_bwd_cases())
def test_bwd_random_shapes(d, B, H, Nq, Nk, causal, dt):
    """Every gradient element of two heads against the oracle, with the same
    inputs on both sides. The backward is handed o and lse; for the two heads
    it checks, those are the oracle's own (o rounded to the element type, lse
    to fp32), and the oracle forms the softmax row term from that same o, as
    the kernels do (heads are independent, so the other heads may keep the
    GPU forward's outputs). Fed the GPU forward's rounded o instead, a row
    whose weights sit mostly on one of few keys moves dq by scale * dD * (P K)
    with dD = do . (o - o_exact): 2.2% of max |dq| on one such head (d = 256,
    Nq = 1, Nk = 2), past the bar, which counts the backward's own roundings
    only."""
    announce(f"bwd random shape d={d} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} {dt}")
    seed = 26000 + d + Nq + 7 * Nk + B
    qi = make_inputs(WORKLOADS[3], B=B, H=H, N=Nq, d=d, seed=seed, dtype=DTYPES[dt])
    ki = qi if Nk == Nq else make_inputs(WORKLOADS[3], B=B, H=H, N=Nk, d=d, seed=seed + 1,
                                         dtype=DTYPES[dt])
    do = upstream(qi["q"].shape, seed + 2, DTYPES[dt])
    scale = qi["scale"]
    dev = torch.device("cuda:0")
    q, k, v, dog = qi["q"].to(dev), ki["k"].to(dev), ki["v"].to(dev), do.to(dev)
    o, lse = mi.attn_fwd_ex(q, k, v, scale=scale, causal=causal)
    heads = sorted({(0, 0), (B - 1, H - 1)})
    fed = {}
    for b, h in heads:
        o_ref, lse_ref = attend_head(as64(qi["q"][b, h]), as64(ki["k"][b, h]),
                                     as64(ki["v"][b, h]), scale, causal)
        o_in = torch.from_numpy(o_ref).to(DTYPES[dt])
        o[b, h].copy_(o_in.to(dev))
        lse[b, h].copy_(torch.from_numpy(lse_ref).to(torch.float32).to(dev))
        fed[(b, h)] = o_in.to(torch.float64).numpy()
    delta = torch.empty(lse.shape, dtype=torch.float32, device=dev)
    grads = mi.attn_bwd(q, k, v, o, lse, dog, scale=scale, causal=causal, delta=delta)
    torch.cuda.synchronize()
    dq, dk, dv = (t.float().cpu().numpy() for t in grads)
    delta = delta.cpu().numpy()
    for b, h in heads:
        rq, rk, rv = attend_head_grad(as64(qi["q"][b, h]), as64(ki["k"][b, h]),
                                      as64(ki["v"][b, h]), as64(do[b, h]), scale, causal,
                                      o=fed[(b, h)])
        check_grad(dq[b, h], rq, f"({b},{h}) dq")
        check_grad(dk[b, h], rk, f"({b},{h}) dk")
        check_grad(dv[b, h], rv, f"({b},{h}) dv")
        ref_delta = (as64(do[b, h]) * fed[(b, h)]).sum(-1)
        assert np.allclose(delta[b, h], ref_delta, rtol=1e-5,
                           atol=1e-5 * max(1.0, np.abs(ref_delta).max()))
