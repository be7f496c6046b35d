"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (per (sequence, head) slice, max|gpu - ref| / max|ref|): 1e-4 for fp32
inputs, 2e-2 for bf16 inputs with fp32 state, for both o and S_T.  Small
workloads are compared element by element in full; the full-size workloads
are compared on whole sampled heads / sequences (every output the oracle
computes for them), with the kernel launched exactly as the benchmark
launches it.
"""
import sys
import time

import numpy as np
import pytest

import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print("[gpu-parity] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch, torch.device("cuda:0")


def _to_dev(torch, dev, x, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(tdt)


def _run_numpy_inputs(torch, dev, inp, with_S0=True, varlen=None):
    import gated_delta_rule_30_amd as kda
    s = inp.spec
    q, k, v, beta, g = (_to_dev(torch, dev, a, s.dtype) for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    S0 = torch.from_numpy(inp.S0).to(dev) if (inp.S0 is not None and with_S0) else None
    use_cu = s.varlen if varlen is None else varlen
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev) if use_cu else None
    o, ST = kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu, n_seqs=s.n_seqs)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ST.cpu().numpy()


def _check(inp, o, ST, tol=None, what=""):
    s = inp.spec
    tol = TOL[s.dtype] if tol is None else tol
    t0 = time.time()
    o_ref, S_ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.g, inp.S0, inp.cu_seqlens)
    eo = oracle.parity_error(o, o_ref, inp.cu_seqlens)
    es = oracle.parity_error(ST, S_ref)
    _say("%s: o err %.3e  S_T err %.3e  (tol %.0e, oracle %.1fs)" % (what or s.name, eo, es, tol, time.time() - t0))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    assert eo <= tol, "o parity %.3e > %.0e" % (eo, tol)
    assert es <= tol, "S_T parity %.3e > %.0e" % (es, tol)


def test_config0_fp32(torch_dev):
    torch, dev = torch_dev
    inp = ki.generate_numpy(ki.headline_configs()[0])
    _say("config 0 fp32 B=1 H=2 T=256 d=64")
    o, ST = _run_numpy_inputs(torch, dev, inp)
    _check(inp, o, ST)


def test_config1_bf16(torch_dev):
    torch, dev = torch_dev
    inp = ki.generate_numpy(ki.headline_configs()[1])
    _say("config 1 bf16 B=4 H=16 T=4096 d=128")
    o, ST = _run_numpy_inputs(torch, dev, inp)
    _check(inp, o, ST)


EDGE = [
    ("f32", [1], 1, 64, None),
    ("f32", [15], 2, 64, None),
    ("f32", [17], 2, 64, None),
    ("f32", [100, 37, 64, 65, 1], 2, 64, None),
    ("f32", [130, 0, 77], 2, 64, None),
    ("bf16", [1], 2, 128, None),
    ("bf16", [15], 2, 128, None),
    ("bf16", [130], 3, 128, None),
    ("bf16", [100, 37, 0, 64, 200], 3, 128, None),
    ("bf16", [333], 2, 64, None),
    ("bf16", [300], 2, 128, "alpha_one"),
    ("bf16", [300], 2, 128, "g_min"),
    ("bf16", [300], 2, 128, "beta_zero"),
    ("bf16", [40], 2, 128, "beta_zero"),
    ("f32", [40], 2, 64, "beta_zero"),
    ("bf16", [300], 2, 128, "beta_one"),
    ("f32", [200], 2, 64, "g_min"),
    ("f32", [200], 2, 64, "beta_one"),
]


@pytest.mark.parametrize("dtype,lengths,H,d,special", EDGE,
                         ids=["%s-%s-H%d-d%d-%s" % (e[0], "_".join(map(str, e[1])), e[2], e[3], e[4]) for e in EDGE])
def test_edge_cases(torch_dev, dtype, lengths, H, d, special):
    torch, dev = torch_dev
    spec = ki.custom("edge", dtype, lengths, H, d, s0_std=0.3, varlen=len(lengths) > 1, seed=len(lengths) + H)
    inp = ki.generate_numpy(spec)
    if special == "alpha_one":
        inp.g[:] = 0.0
    elif special == "g_min":
        inp.g[:] = -5.0
    elif special == "beta_zero":
        inp.beta[:] = 0.0
    elif special == "beta_one":
        inp.beta[:] = 1.0
    _say("edge %s %s H=%d d=%d %s" % (dtype, lengths, H, d, special))
    o, ST = _run_numpy_inputs(torch, dev, inp)
    _check(inp, o, ST, what="edge %s %s %s" % (dtype, lengths, special))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_equal_ragged_lengths_without_cu_seqlens(torch_dev, dtype, d):
    """Three sequences of 100 tokens passed as equal lengths (cu_seqlens NULL):
    each sequence's chunks (64 + 36 tokens) are derived from the index."""
    torch, dev = torch_dev
    spec = ki.custom("equal ragged", dtype, [100, 100, 100], 2, d, s0_std=0.3, varlen=False, seed=9)
    inp = ki.generate_numpy(spec)
    _say("equal ragged lengths 3 x 100 %s d=%d, cu_seqlens NULL" % (dtype, d))
    o, ST = _run_numpy_inputs(torch, dev, inp)
    _check(inp, o, ST, what="equal ragged %s" % dtype)


def test_many_sequences(torch_dev):
    """2100 sequences (three 1024-sequence batches of the chunk table), lengths
    0..70 with empty ones, so chunk records straddle batch boundaries."""
    torch, dev = torch_dev
    import numpy as np
    lengths = [int(x) for x in np.random.default_rng(11).integers(0, 71, size=2100)]
    lengths[0] = 0
    lengths[1023] = 0
    lengths[1024] = 70
    spec = ki.custom("many", "bf16", lengths, 2, 64, s0_std=0.3, varlen=True, seed=5)
    inp = ki.generate_numpy(spec)
    _say("many sequences: N=%d T=%d H=2 d=64" % (len(lengths), sum(lengths)))
    o, ST = _run_numpy_inputs(torch, dev, inp)
    _check(inp, o, ST, what="many sequences")


def test_s0_null_equals_zeros(torch_dev):
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    inp = ki.generate_numpy(ki.custom("z", "bf16", [190, 70], 2, 128, varlen=True))
    q, k, v, beta, g = (_to_dev(torch, dev, a, "bf16") for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    o1, S1 = kda.chunk_fwd(q, k, v, beta, g, S0=None, cu_seqlens=cu)
    o2, S2 = kda.chunk_fwd(q, k, v, beta, g, S0=torch.zeros(2, 2, 128, 128, device=dev), cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_deterministic(torch_dev):
    torch, dev = torch_dev
    inp = ki.generate_numpy(ki.custom("det", "bf16", [4096, 1000, 3000], 8, 128, s0_std=0.02, varlen=True))
    o1, S1 = _run_numpy_inputs(torch, dev, inp)
    o2, S2 = _run_numpy_inputs(torch, dev, inp)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def _sample_check(torch, inp, o_dev, ST_dev, heads, seqs, what):
    """Oracle on whole sequences `seqs` for heads `heads` (inputs copied back
    from the device as the exact values the kernels read)."""
    cu = inp.cu_seqlens
    lo_w, hi_w = inp.window
    worst_o = worst_s = 0.0
    for n in seqs:
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda t: t[a:b][:, heads].float().cpu().numpy()
        q, k, v, g = sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g)
        beta = inp.beta[a:b][:, heads].float().cpu().numpy()
        S0 = None if inp.S0 is None else inp.S0[n:n + 1][:, heads].cpu().numpy()
        wlo, whi = max(a, lo_w) - a, min(b, hi_w) - a
        t0 = time.time()
        o_ref, S_ref = oracle.forward(q, k, v, beta, g, S0, None, out_range=(wlo, whi))
        o_gpu = o_dev[a + wlo:a + whi][:, heads].float().cpu().numpy()
        S_gpu = ST_dev[n:n + 1][:, heads].cpu().numpy()
        eo = oracle.parity_error(o_gpu, o_ref) if whi > wlo else 0.0
        es = oracle.parity_error(S_gpu, S_ref)
        _say("%s seq %d (len %d, window %d) heads %s: o %.3e S_T %.3e (oracle %.1fs)"
             % (what, n, b - a, whi - wlo, heads, eo, es, time.time() - t0))
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    assert worst_o <= TOL["bf16"] and worst_s <= TOL["bf16"], (worst_o, worst_s)


def _run_torch_inputs(torch, inp):
    import gated_delta_rule_30_amd as kda
    s = inp.spec
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(inp.q.device) if s.varlen else None
    o, ST = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.beta, inp.g, S0=inp.S0, cu_seqlens=cu, n_seqs=s.n_seqs)
    torch.cuda.synchronize()
    return o, ST


def test_config2_headline_sampled(torch_dev):
    torch, dev = torch_dev
    spec = ki.headline_configs()[2]
    _say("config 2 generate (torch, on device)")
    inp = ki.generate_torch(spec, dev)
    o, ST = _run_torch_inputs(torch, inp)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(ST).all())
    _sample_check(torch, inp, o, ST, heads=[0, 13, 31], seqs=[0], what="config 2")
    del inp, o, ST
    torch.cuda.empty_cache()


def test_config3_varlen_sampled(torch_dev):
    torch, dev = torch_dev
    spec = ki.headline_configs()[3]
    _say("config 3 generate (torch, on device), T_total=%d" % spec.total_tokens)
    inp = ki.generate_torch(spec, dev)
    o, ST = _run_torch_inputs(torch, inp)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(ST).all())
    L = np.array(spec.lengths)
    rng = np.random.default_rng(3)
    seqs = sorted({int(L.argmin()), int(L.argmax()), *[int(x) for x in rng.choice(len(L), 2, replace=False)]})
    _sample_check(torch, inp, o, ST, heads=[5, 30], seqs=seqs, what="config 3")
    del inp, o, ST
    torch.cuda.empty_cache()


def test_config4_1m_sampled(torch_dev):
    torch, dev = torch_dev
    spec = ki.headline_configs()[4]
    _say("config 4 generate (torch, on device)")
    inp = ki.generate_torch(spec, dev)
    o, ST = _run_torch_inputs(torch, inp)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(ST).all())
    _say("config 4 window %s" % (inp.window,))
    _sample_check(torch, inp, o, ST, heads=[0, 9], seqs=[0], what="config 4")
    del inp, o, ST
    torch.cuda.empty_cache()
