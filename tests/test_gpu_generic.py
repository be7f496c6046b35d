"""GPU parity of the generic kernels: chunk sizes 16, 32 and 128, d_k != d_v
and fp32 at d = 128 (every size the tuned chunk-64 kernels leave out)
against the fp64 oracle, to the tuned path's bars (per (sequence, head)
slice, max|gpu - ref| / max|ref|: 1e-4 for fp32 inputs, 2e-2 for bf16).
The oracle is the token-by-token recurrence, so these cases also show that
the output does not depend on the chunk size.  The full-size workloads at
chunk 128 are in test_gpu_parity.py, beside their chunk-64 runs."""
import sys
import time

import numpy as np
import pytest

import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print("[gpu-generic] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch, torch.device("cuda:0")


def _run(torch, dev, inp, chunk, varlen=None, profile=False):
    import gated_delta_rule_30_amd as kda
    s = inp.spec
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    q, k, v, beta, g = (torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(tdt)
                        for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    S0 = torch.from_numpy(inp.S0).to(dev) if inp.S0 is not None else None
    use_cu = s.varlen if varlen is None else varlen
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev) if use_cu else None
    if profile:
        o, ST, ms = kda.chunk_fwd_profile(q, k, v, beta, g, S0=S0, cu_seqlens=cu, n_seqs=s.n_seqs, chunk=chunk)
    else:
        o, ST = kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu, n_seqs=s.n_seqs, chunk=chunk)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ST.cpu().numpy()


def _check(inp, o, ST, what):
    s = inp.spec
    tol = TOL[s.dtype]
    t0 = time.time()
    o_ref, S_ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.g, inp.S0, inp.cu_seqlens)
    eo = oracle.parity_error(o, o_ref, inp.cu_seqlens)
    es = oracle.parity_error(ST, S_ref)
    _say("%s: o err %.3e  S_T err %.3e  (tol %.0e, oracle %.1fs)" % (what, eo, es, tol, time.time() - t0))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    assert eo <= tol, "o parity %.3e > %.0e" % (eo, tol)
    assert es <= tol, "S_T parity %.3e > %.0e" % (es, tol)


def _spec(name, dtype, lengths, H, dk, dv, seed, s0=0.3, varlen=True):
    return ki.Spec(name, dtype, tuple(lengths), H, dk, dv, s0_std=s0, varlen=varlen, seed=seed)


# Ragged packed batches: an empty sequence, a one-token sequence, lengths
# that cut through 16-token sub-tiles and chunks of every size.
LENGTHS = (100, 37, 0, 130, 1, 64)
SWEEP = [(C, dt, dk, dv) for C in (16, 32, 64, 128) for dt in ("f32", "bf16")
         for dk, dv in ((64, 64), (128, 128), (64, 128), (128, 64))]


@pytest.mark.parametrize("C,dtype,dk,dv", SWEEP, ids=["C%d-%s-dk%d-dv%d" % c for c in SWEEP])
def test_sizes_sweep(torch_dev, C, dtype, dk, dv):
    """Every supported (chunk, dtype, d_k, d_v) on one ragged packed batch
    with S0: the generic kernels, or the tuned ones where they apply."""
    torch, dev = torch_dev
    inp = ki.generate_numpy(_spec("sweep", dtype, LENGTHS, 2, dk, dv, seed=C + dk + 3 * dv))
    _say("sweep C=%d %s dk=%d dv=%d lengths %s" % (C, dtype, dk, dv, LENGTHS))
    o, ST = _run(torch, dev, inp, C)
    _check(inp, o, ST, "C=%d %s dk=%d dv=%d" % (C, dtype, dk, dv))


EDGE = [(C, dt, sp) for C in (16, 128) for dt in ("f32", "bf16")
        for sp in ("g_min", "alpha_one", "beta_zero", "beta_one")]


@pytest.mark.parametrize("C,dtype,special", EDGE, ids=["C%d-%s-%s" % e for e in EDGE])
def test_special_values(torch_dev, C, dtype, special):
    """The degenerate inputs: log alpha = -5 everywhere (over a 128-token
    chunk the decay ratios reach e^-635, far below fp32's range: the terms
    underflow to zero, as they should), alpha = 1 (no decay), beta = 0 (no
    write: per-channel gated linear attention with an unchanged state) and
    beta = 1."""
    torch, dev = torch_dev
    inp = ki.generate_numpy(_spec("special", dtype, (300, 45), 2, 128, 64, seed=7))
    if special == "g_min":
        inp.g[:] = -5.0
    elif special == "alpha_one":
        inp.g[:] = 0.0
    elif special == "beta_zero":
        inp.beta[:] = 0.0
    elif special == "beta_one":
        inp.beta[:] = 1.0
    _say("special C=%d %s %s" % (C, dtype, special))
    o, ST = _run(torch, dev, inp, C)
    _check(inp, o, ST, "C=%d %s %s" % (C, dtype, special))


@pytest.mark.parametrize("C", [16, 32, 128])
def test_equal_lengths_without_cu_seqlens(torch_dev, C):
    """Three sequences of 200 tokens passed as equal lengths (cu_seqlens
    NULL): the chunks (ending in a partial one) are derived from the index."""
    torch, dev = torch_dev
    inp = ki.generate_numpy(_spec("equal", "bf16", (200, 200, 200), 3, 128, 128, seed=C, varlen=False))
    _say("equal lengths 3 x 200 C=%d, cu_seqlens NULL" % C)
    o, ST = _run(torch, dev, inp, C)
    _check(inp, o, ST, "equal lengths C=%d" % C)


def test_many_sequences(torch_dev):
    """1500 sequences of 0..40 tokens at chunk 32 (two 1024-sequence batches
    of the chunk table, empty sequences at the batch edge)."""
    torch, dev = torch_dev
    lengths = [int(x) for x in np.random.default_rng(3).integers(0, 41, size=1500)]
    lengths[1023] = 0
    lengths[1024] = 40
    inp = ki.generate_numpy(_spec("many", "bf16", lengths, 2, 64, 128, seed=2))
    _say("many sequences: N=%d T=%d C=32" % (len(lengths), sum(lengths)))
    o, ST = _run(torch, dev, inp, 32)
    _check(inp, o, ST, "many sequences C=32")


def test_no_tokens(torch_dev):
    """total_tokens = 0 at chunk 128: S_T is S0."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    q = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device=dev)
    v = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device=dev)
    beta = torch.zeros((0, 2), dtype=torch.bfloat16, device=dev)
    S0 = torch.randn((3, 2, 128, 64), device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    o, ST = kda.chunk_fwd(q, q, v, beta, q, S0=S0, cu_seqlens=cu, chunk=128)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 64) and torch.equal(ST, S0)


@pytest.mark.parametrize("dtype,C", [("f32", 128), ("bf16", 128), ("f32", 16)])
def test_configs_small_at_other_chunks(torch_dev, dtype, C):
    """The two small workloads at other chunk sizes: fp32 B=1 H=2 T=256 d=64,
    and bf16 B=4 H=16 T=4096 d=128, compared in full."""
    torch, dev = torch_dev
    spec = ki.headline_configs()[0 if dtype == "f32" else 1]
    inp = ki.generate_numpy(spec)
    _say("%s at chunk %d" % (spec.name, C))
    o, ST = _run(torch, dev, inp, C)
    _check(inp, o, ST, "%s chunk %d" % (spec.name, C))


def test_profile_entry_and_determinism(torch_dev):
    """The measurement entry point runs the same generic kernels (bit for bit
    the plain call's result), and two calls agree bit for bit."""
    torch, dev = torch_dev
    inp = ki.generate_numpy(_spec("det", "bf16", (500, 77), 2, 128, 64, seed=5))
    o1, S1 = _run(torch, dev, inp, 128)
    o2, S2 = _run(torch, dev, inp, 128)
    o3, S3 = _run(torch, dev, inp, 128, profile=True)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    assert np.array_equal(o1, o3) and np.array_equal(S1, S3)


RANDOM_CASES = 16


@pytest.mark.parametrize("case", range(RANDOM_CASES))
def test_random_cases(torch_dev, case):
    """Seeded random (chunk, dtype, d_k, d_v, heads, lengths, S0) draws, the
    lengths taken around the sub-tile and chunk edges (0, 1, 15..17, 31..33,
    63..65, 127..129, and longer), each against the oracle."""
    torch, dev = torch_dev
    rng = np.random.default_rng(1000 + case)
    C = int(rng.choice([16, 32, 64, 128]))
    dtype = str(rng.choice(["f32", "bf16"]))
    dk, dv = (int(x) for x in rng.choice([64, 128], size=2))
    edges = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 257]
    lengths = [int(x) for x in rng.choice(edges, size=int(rng.integers(1, 6)))]
    if sum(lengths) == 0:
        lengths[0] = 33
    H = int(rng.integers(1, 4))
    s0 = float(rng.choice([0.0, 0.3]))
    inp = ki.generate_numpy(_spec("random", dtype, lengths, H, dk, dv, seed=2000 + case, s0=s0))
    what = "case %d: C=%d %s dk=%d dv=%d H=%d lengths %s S0 %.1f" % (case, C, dtype, dk, dv, H, lengths, s0)
    _say(what)
    o, ST = _run(torch, dev, inp, C)
    _check(inp, o, ST, what)
