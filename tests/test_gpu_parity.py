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


@pytest.mark.parametrize("d", [128, 64])
def test_wide_slabs_match_narrow(torch_dev, d):
    """A batch whose 16-column recurrence chains outnumber the CUs runs the
    32-column workgroups; three of its sequences on their own run the
    16-column ones.  Each column's arithmetic is the same in both, so o and
    S_T of those sequences must agree bit for bit; the whole batch is also
    held to the oracle.  Lengths include empty, single-token, sub-tile and
    chunk-boundary sequences."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    lengths = [int(x) for x in np.random.default_rng(23).integers(0, 301, size=40)]
    lengths[:10] = [130, 0, 65, 1, 15, 16, 63, 64, 17, 300]
    H = 4
    spec = ki.custom("wide", "bf16", lengths, H, d, s0_std=0.3, varlen=True, seed=8)
    inp = ki.generate_numpy(spec)
    _say("wide slabs: N=%d H=%d d=%d (batch), sequences 0..2 alone" % (len(lengths), H, d))
    q, k, v, beta, g = (_to_dev(torch, dev, a, "bf16") for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    S0 = torch.from_numpy(inp.S0).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    o_all, S_all = kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu)
    n3 = int(inp.cu_seqlens[3])
    o_3, S_3 = kda.chunk_fwd(q[:n3].contiguous(), k[:n3].contiguous(), v[:n3].contiguous(), beta[:n3].contiguous(),
                             g[:n3].contiguous(), S0=S0[:3].contiguous(), cu_seqlens=cu[:4].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o_all[:n3], o_3), "o differs between 32- and 16-column workgroups"
    assert torch.equal(S_all[:3], S_3), "S_T differs between 32- and 16-column workgroups"
    _check(inp, o_all.float().cpu().numpy(), S_all.cpu().numpy(), what="wide slabs d=%d" % d)


def test_wide_slabs_paced_long_sequence(torch_dev):
    """32-column workgroups (40 sequences x 4 heads: more 16-column chains
    than CUs) with one sequence of 140,000 tokens (2188 chunks), whose
    workgroups run the pacing wave: every (sequence, head) slice against the
    oracle."""
    torch, dev = torch_dev
    lengths = [int(x) for x in np.random.default_rng(29).integers(0, 400, size=40)]
    lengths[7] = 140000
    spec = ki.custom("wide paced", "bf16", lengths, 4, 128, s0_std=0.3, varlen=True, seed=12)
    inp = ki.generate_numpy(spec)
    _say("wide slabs with a paced sequence: N=%d T=%d H=4 d=128" % (len(lengths), sum(lengths)))
    o, ST = _run_numpy_inputs(torch, dev, inp)
    _check(inp, o, ST, what="wide slabs, paced long sequence")


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


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("f32", 64, 64), ("bf16", 64, 32)])
def test_without_final_state(torch_dev, dtype, d, chunk):
    """S_T omitted (NULL through the C ABI): o is the same, bit for bit, as
    with S_T requested (tuned kernels, and the generic ones at chunk 32)."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    inp = ki.generate_numpy(ki.custom("nost", dtype, [300, 45, 0, 129], 2, d, s0_std=0.3, varlen=True, seed=4))
    q, k, v, beta, g = (_to_dev(torch, dev, a, dtype) for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    S0 = torch.from_numpy(inp.S0).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    o1, S1 = kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu, chunk=chunk)
    o2, S2 = kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu, chunk=chunk, output_final_state=False)
    torch.cuda.synchronize()
    assert S2 is None and torch.equal(o1, o2)


def test_deterministic(torch_dev):
    torch, dev = torch_dev
    inp = ki.generate_numpy(ki.custom("det", "bf16", [4096, 1000, 3000], 8, 128, s0_std=0.02, varlen=True))
    o1, S1 = _run_numpy_inputs(torch, dev, inp)
    o2, S2 = _run_numpy_inputs(torch, dev, inp)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def _slice_errors(x, ref):
    """max|x - ref| / max(max|ref|, 1e-30) per head of one sequence's slice
    [T, H, ...]; non-finite values give inf."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    H = x.shape[1]
    xf = np.moveaxis(x, 1, 0).reshape(H, -1)
    rf = np.moveaxis(ref, 1, 0).reshape(H, -1)
    num = np.max(np.abs(xf - rf), axis=1) if xf.shape[1] else np.zeros(H)
    den = np.maximum(np.max(np.abs(rf), axis=1) if rf.shape[1] else np.zeros(H), 1e-30)
    err = num / den
    err[~np.all(np.isfinite(xf), axis=1)] = np.inf
    return err


def _full_check(torch, inp, o_dev, ST_dev, what, seq_groups, head_groups, extra=()):
    """Every (sequence, head) slice of o (within the workload's output
    window) and of S_T against the oracle, run group by group on the exact
    values the kernels read (copied back from the device).  `extra` holds
    more (label, o, S_T) results of the same inputs (other chunk sizes),
    checked against the same oracle output.  Prints the worst slice of each
    and the slices whose element offsets pass 2^31; returns the first run's
    worst errors and that slice count."""
    cu = inp.cu_seqlens
    lo_w, hi_w = inp.window
    H, d = inp.q.shape[1], inp.q.shape[2]
    runs = [(what, o_dev, ST_dev)] + list(extra)
    worst = {name: {"o": (0.0, None), "S_T": (0.0, None)} for name, _, _ in runs}
    big_slices = 0
    for seqs in seq_groups:
        a, b = int(cu[seqs[0]]), int(cu[seqs[-1] + 1])
        wlo, whi = max(a, lo_w), min(b, hi_w)
        for heads in head_groups:
            hs = slice(heads[0], heads[-1] + 1)
            host = lambda t: t[a:b, hs].float().cpu().numpy()
            q, k, v, g, beta = host(inp.q), host(inp.k), host(inp.v), host(inp.g), host(inp.beta)
            S0 = None if inp.S0 is None else inp.S0[seqs[0]:seqs[-1] + 1, hs].cpu().numpy()
            lcu = cu[seqs[0]:seqs[-1] + 2] - a
            t0 = time.time()
            o_ref, S_ref = oracle.forward(q, k, v, beta, g, S0, lcu,
                                          out_range=(max(wlo - a, 0), max(whi - a, 0)))
            t_or = time.time() - t0
            for name, o_d, ST_d in runs:
                w = worst[name]
                o_gpu = o_d[max(wlo, a):max(whi, a), hs].float().cpu().numpy()
                S_gpu = ST_d[seqs[0]:seqs[-1] + 1, hs].cpu().numpy()
                assert o_gpu.shape == o_ref.shape and S_gpu.shape == S_ref.shape, (o_gpu.shape, o_ref.shape)
                g_o = g_s = 0.0
                for i, n in enumerate(seqs):
                    sa, sb = int(cu[n]), int(cu[n + 1])
                    oa, ob = max(sa, wlo), min(sb, whi)
                    if ob > oa:
                        e = _slice_errors(o_gpu[oa - wlo:ob - wlo], o_ref[oa - wlo:ob - wlo])
                        h = int(np.argmax(e))
                        g_o = max(g_o, float(e[h]))
                        if e[h] > w["o"][0] or w["o"][1] is None:
                            w["o"] = (float(e[h]), (n, heads[0] + h))
                    es = _slice_errors(S_gpu[i:i + 1].transpose(1, 0, 2, 3), S_ref[i:i + 1].transpose(1, 0, 2, 3))
                    h = int(np.argmax(es))
                    g_s = max(g_s, float(es[h]))
                    if es[h] > w["S_T"][0] or w["S_T"][1] is None:
                        w["S_T"] = (float(es[h]), (n, heads[0] + h))
                    if name == what and (int(cu[n + 1]) * H * d) > 2 ** 31:
                        big_slices += len(heads)
                _say("%s seqs %d..%d (tokens %d..%d) heads %d..%d: o %.3e S_T %.3e (oracle %.1fs)"
                     % (name, seqs[0], seqs[-1], a, b, heads[0], heads[-1], g_o, g_s, t_or))
    for name, _, _ in runs:
        w = worst[name]
        _say("%s worst slice: o %.3e at (seq, head) %s; S_T %.3e at %s"
             % (name, w["o"][0], w["o"][1], w["S_T"][0], w["S_T"][1]))
    _say("%s: %d slices reach element offsets past 2^31" % (what, big_slices))
    for name, _, _ in runs:
        w = worst[name]
        assert w["o"][0] <= TOL["bf16"] and w["S_T"][0] <= TOL["bf16"], (name, w)
    return worst[what], big_slices


def _run_torch_inputs(torch, inp, chunk=64):
    import gated_delta_rule_30_amd as kda
    s = inp.spec
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(inp.q.device) if s.varlen else None
    o, ST = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.beta, inp.g, S0=inp.S0, cu_seqlens=cu, n_seqs=s.n_seqs,
                          chunk=chunk)
    torch.cuda.synchronize()
    return o, ST


@pytest.mark.timeout(900)
def test_config2_headline_full(torch_dev):
    """B=1, H=32, T=65536, d=128, S0 ~ 0.02 N(0,1), launched as the
    benchmark launches it: all 32 heads of o and S_T against the oracle; the
    same at chunks 16, 32 and 128 (the generic kernels: 4096, 2048 and 512
    chunk steps) against the same oracle run."""
    torch, dev = torch_dev
    spec = ki.headline_configs()[2]
    _say("config 2 generate (torch, on device)")
    inp = ki.generate_torch(spec, dev)
    o, ST = _run_torch_inputs(torch, inp)
    extra = [("config 2 chunk %d" % c,) + _run_torch_inputs(torch, inp, chunk=c) for c in (16, 32, 128)]
    _full_check(torch, inp, o, ST, "config 2", [[0]], [list(range(0, 16)), list(range(16, 32))], extra=extra)
    del inp, o, ST, extra
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_config3_varlen_full(torch_dev):
    """64 packed sequences (L ~ U[512, 16384], 550,809 tokens), H=32, d=128,
    25 % of channels at g = -5: every (sequence, head) slice of o and S_T,
    at chunk 64 and at chunks 16, 32 and 128.  Sequences 60-63 sit at
    element offsets past 2^31 (from token 524,288)."""
    torch, dev = torch_dev
    spec = ki.headline_configs()[3]
    _say("config 3 generate (torch, on device), T_total=%d" % spec.total_tokens)
    inp = ki.generate_torch(spec, dev)
    o, ST = _run_torch_inputs(torch, inp)
    extra = [("config 3 chunk %d" % c,) + _run_torch_inputs(torch, inp, chunk=c) for c in (16, 32, 128)]
    groups = [list(range(i, min(i + 8, spec.n_seqs))) for i in range(0, spec.n_seqs, 8)]
    _, big = _full_check(torch, inp, o, ST, "config 3", groups, [list(range(32))], extra=extra)
    assert big >= 4 * 32, "the slices past 2^31 element offsets must be among those compared"
    del inp, o, ST, extra
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_config4_1m_full(torch_dev):
    """B=1, H=16, T=1,048,576, d=128, S0 ~ 0.02 N(0,1): all 16 heads, o on
    the seeded 8192-token window and S_T (the oracle runs all 1M tokens), at
    chunk 64 and at chunks 32 and 128 (32,768 and 8192 chunk steps)."""
    torch, dev = torch_dev
    spec = ki.headline_configs()[4]
    _say("config 4 generate (torch, on device)")
    inp = ki.generate_torch(spec, dev)
    o, ST = _run_torch_inputs(torch, inp)
    extra = [("config 4 chunk %d" % c,) + _run_torch_inputs(torch, inp, chunk=c) for c in (32, 128)]
    _say("config 4 window %s" % (inp.window,))
    _full_check(torch, inp, o, ST, "config 4", [[0]], [list(range(h, h + 4)) for h in range(0, 16, 4)],
                extra=extra)
    del inp, o, ST, extra
    torch.cuda.empty_cache()


@pytest.mark.parametrize("lengths,H,d,s0", [((135000, 135000), 2, 128, 0.02), ((140000,), 3, 64, 0.0)],
                         ids=["2seq-d128-S0", "1seq-d64-zeroS0"])
def test_pipelined_forward(torch_dev, lengths, H, d, s0):
    """Equal-length sequences of more than 2048 chunks whose recurrence fills
    at most half of the CUs take the pipelined path (k_prep of the next token
    block on a side stream while the recurrence works on this one, state
    handed between blocks in fp32; with 4 sequence-heads, the first case, on
    a 256-CU device the recurrence holds XCDs 0..3 and k_prep XCDs 4..7; the
    second, 3 sequence-heads, shares them): every (sequence, head) slice
    against the oracle, and bit for bit equal to the same kernels run one
    after another (the measurement entry point does not pipeline)."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    spec = ki.custom("pipe", "bf16", list(lengths), H, d, s0_std=s0, varlen=False, seed=21)
    inp = ki.generate_torch(spec, dev)
    N = spec.n_seqs
    _say("pipelined forward: %s H=%d d=%d" % (lengths, H, d))
    o, ST = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.beta, inp.g, S0=inp.S0, n_seqs=N)
    o2, ST2, _ = kda.chunk_fwd_profile(inp.q, inp.k, inp.v, inp.beta, inp.g, S0=inp.S0, n_seqs=N)
    o3, _ = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.beta, inp.g, S0=inp.S0, n_seqs=N, output_final_state=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ST, ST2), "pipelined and sequential launches differ"
    assert torch.equal(o, o3), "the pipelined forward without S_T differs"
    del o2, ST2, o3
    _full_check(torch, inp, o, ST, "pipelined", [[n] for n in range(N)], [list(range(H))])
