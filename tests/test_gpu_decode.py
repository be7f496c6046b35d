"""GPU parity of the decode entry point (kda_recurrent_fwd) and the input
validator (kda_validate_inputs), through the C ABI.

Decode advances each sequence's state token by token; the fp64 oracle's
forward over the same tokens from the same initial states is the reference
(the recurrence is the definition of both).  Bar as for the chunked pass:
per (sequence, head) slice max|gpu - ref| / max|ref| <= 1e-4 (fp32 inputs)
or 2e-2 (bf16 inputs, fp32 state), for o and the final states.
"""
import sys

import numpy as np
import pytest

import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print("[gpu-decode] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd  # noqa: F401
    return torch, torch.device("cuda:0")


def _dev(torch, dev, x, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(tdt)


DECODE = [
    ("f32", 3, 1, 2, 64, 0.3),
    ("f32", 2, 5, 2, 64, 0.3),
    ("f32", 2, 3, 3, 128, 0.0),
    ("bf16", 4, 1, 4, 128, 0.3),
    ("bf16", 3, 3, 4, 128, 0.3),
    ("bf16", 5, 2, 2, 64, 0.0),
    ("bf16", 1, 16, 2, 128, 0.02),
]


@pytest.mark.parametrize("dtype,N,n,H,d,s0", DECODE,
                         ids=["%s-N%d-n%d-H%d-d%d-s%g" % c for c in DECODE])
def test_decode_matches_oracle(torch_dev, dtype, N, n, H, d, s0):
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    spec = ki.custom("dec", dtype, [n] * N, H, d, s0_std=s0, varlen=True, seed=N * 7 + n)
    inp = ki.generate_numpy(spec)
    _say("decode %s N=%d n=%d H=%d d=%d S0 std %g" % (dtype, N, n, H, d, s0))
    q, k, v, beta, g = (_dev(torch, dev, a, dtype) for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    S_in = torch.from_numpy(inp.S0).to(dev) if inp.S0 is not None else None
    o, S_out = kda.recurrent_fwd(q, k, v, beta, g, S_in=S_in, n_seqs=N)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.g, inp.S0, inp.cu_seqlens)
    eo = oracle.parity_error(o.float().cpu().numpy(), o_ref, inp.cu_seqlens)
    es = oracle.parity_error(S_out.cpu().numpy(), S_ref)
    _say("  o err %.3e  S err %.3e (tol %.0e)" % (eo, es, TOL[dtype]))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_in_place_and_chained(torch_dev):
    """In place (S_out is S_in) gives the same as separate buffers, and two
    calls of 3 then 5 tokens equal one call of 8 (the state hand-off)."""
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    N, H, d = 3, 2, 128
    spec = ki.custom("chain", "bf16", [8] * N, H, d, s0_std=0.3, varlen=True, seed=3)
    inp = ki.generate_numpy(spec)
    t = {name: _dev(torch, dev, getattr(inp, name), "bf16") for name in ("q", "k", "v", "beta", "g")}
    S0 = torch.from_numpy(inp.S0).to(dev)
    o8, S8 = kda.recurrent_fwd(t["q"], t["k"], t["v"], t["beta"], t["g"], S_in=S0, n_seqs=N)
    # split per sequence into tokens [0,3) and [3,8)
    def part(x, a, b):
        return x.reshape(N, 8, *x.shape[1:])[:, a:b].reshape(-1, *x.shape[1:]).contiguous()
    S = S0.clone()
    oa, _ = kda.recurrent_fwd(*(part(t[n_], 0, 3) for n_ in ("q", "k", "v", "beta", "g")), S_in=S, S_out=S,
                              n_seqs=N)
    ob, _ = kda.recurrent_fwd(*(part(t[n_], 3, 8) for n_ in ("q", "k", "v", "beta", "g")), S_in=S, S_out=S,
                              n_seqs=N)
    torch.cuda.synchronize()
    o_split = torch.cat([oa.reshape(N, 3, H, d), ob.reshape(N, 5, H, d)], dim=1).reshape(-1, H, d)
    assert torch.equal(S, S8)
    assert torch.equal(o_split, o8)


def test_decode_agrees_with_chunked(torch_dev):
    """The same tokens through kda_chunk_fwd and kda_recurrent_fwd agree to the
    parity bar (both are checked against the oracle elsewhere)."""
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    N, n, H, d = 2, 40, 2, 128
    spec = ki.custom("agree", "bf16", [n] * N, H, d, s0_std=0.3, varlen=True, seed=4)
    inp = ki.generate_numpy(spec)
    t = [_dev(torch, dev, getattr(inp, name), "bf16") for name in ("q", "k", "v", "beta", "g")]
    S0 = torch.from_numpy(inp.S0).to(dev)
    o1, S1 = kda.recurrent_fwd(*t, S_in=S0, n_seqs=N)
    o2, S2 = kda.chunk_fwd(*t, S0=S0, n_seqs=N)
    torch.cuda.synchronize()
    cu = inp.cu_seqlens
    e_o = oracle.parity_error(o1.float().cpu().numpy(), o2.float().cpu().numpy().astype(np.float64), cu)
    e_s = oracle.parity_error(S1.cpu().numpy(), S2.cpu().numpy().astype(np.float64))
    _say("decode vs chunked: o %.3e  S %.3e" % (e_o, e_s))
    assert e_o <= 2e-2 and e_s <= 2e-2


def test_validate_inputs_counts(torch_dev):
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    spec = ki.custom("val", "bf16", [100, 37, 64], 3, 64, varlen=True, seed=2)
    inp = ki.generate_numpy(spec)
    g = _dev(torch, dev, inp.g, "bf16")
    beta = _dev(torch, dev, inp.beta, "bf16")
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    assert kda.validate_inputs(beta, g, cu) == {"log_alpha": 0, "beta": 0, "cu_seqlens": 0}
    g[0, 0, 0] = -6.0
    g[5, 1, 3] = 0.5
    g[7, 2, 1] = float("nan")
    g[9, 0, 9] = -5.0           # in range (the bound itself)
    beta[2, 1] = 1.5
    beta[3, 0] = -0.25
    beta[4, 2] = float("inf")
    beta[6, 1] = 1.0            # in range
    bad_cu = torch.tensor([0, 120, 100, 200], dtype=torch.int32, device=dev)   # decreasing, wrong end
    assert kda.validate_inputs(beta, g, bad_cu) == {"log_alpha": 3, "beta": 3, "cu_seqlens": 2}
    assert kda.validate_inputs(beta, g, None, n_seqs=1) == {"log_alpha": 3, "beta": 3, "cu_seqlens": 0}


COMMIT = [("bf16", 128, (0, 1, 4, 2, 9, -3)), ("f32", 64, (3, 0, 4, 1))]


@pytest.mark.parametrize("dtype,d,accept", COMMIT, ids=["bf16-d128", "f32-d64"])
def test_commit_matches_prefix_oracle(torch_dev, dtype, d, accept):
    """kda_recurrent_commit over n = 4 cached draft slots per sequence takes
    each sequence's first n_accept tokens (clamped to [0, n]: 9 -> 4,
    -3 -> 0): states and the taken rows of o match the oracle run over just
    those prefixes; the other o rows keep their NaN fill."""
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    N, n, H = len(accept), 4, 2
    spec = ki.custom("commit", dtype, [n] * N, H, d, s0_std=0.3, varlen=True, seed=11)
    inp = ki.generate_numpy(spec)
    _say("commit %s d=%d accept %s" % (dtype, d, accept))
    t = [_dev(torch, dev, getattr(inp, name), dtype) for name in ("q", "k", "v", "beta", "g")]
    S_in = torch.from_numpy(inp.S0).to(dev)
    acc = torch.tensor(accept, dtype=torch.int32, device=dev)
    o = torch.full((N * n, H, d), float("nan"), dtype=t[0].dtype, device=dev)
    _, S_out = kda.recurrent_fwd(*t, S_in=S_in, n_seqs=N, o=o, n_accept=acc)
    torch.cuda.synchronize()
    taken = [min(max(a, 0), n) for a in accept]
    rows = np.concatenate([np.arange(i * n, i * n + a) for i, a in enumerate(taken)]).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(taken)])
    sub = [np.ascontiguousarray(getattr(inp, name)[rows]) for name in ("q", "k", "v", "beta", "g")]
    o_ref, S_ref = oracle.forward(*sub, inp.S0, cu)
    og = o.float().cpu().numpy()
    eo = oracle.parity_error(og[rows], o_ref, cu)
    es = oracle.parity_error(S_out.cpu().numpy(), S_ref)
    skipped = np.setdiff1d(np.arange(N * n), rows)
    _say("  o err %.3e  S err %.3e (tol %.0e); %d skipped rows" % (eo, es, TOL[dtype], skipped.size))
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    assert np.isnan(og[skipped]).all()
    for i, a in enumerate(taken):
        if a == 0:
            assert torch.equal(S_out[i], S_in[i])


def test_speculative_verify_then_commit(torch_dev):
    """The serving flow: verify a draft of 5 tokens from the kept state into a
    scratch state, then commit each sequence's accepted prefix in place with
    no output.  The committed state equals, bit for bit, what
    kda_recurrent_fwd reaches over just the accepted tokens, and the draft's
    outputs for accepted tokens are the committed run's outputs."""
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    N, n, H, d = 4, 5, 3, 128
    accept = (5, 2, 0, 3)
    spec = ki.custom("spec", "bf16", [n] * N, H, d, s0_std=0.3, varlen=True, seed=12)
    inp = ki.generate_numpy(spec)
    t = [_dev(torch, dev, getattr(inp, name), "bf16") for name in ("q", "k", "v", "beta", "g")]
    S = torch.from_numpy(inp.S0).to(dev)
    S_keep = S.clone()
    o_draft, S_draft = kda.recurrent_fwd(*t, S_in=S, n_seqs=N)
    acc = torch.tensor(accept, dtype=torch.int32, device=dev)
    o_none, S_after = kda.recurrent_fwd(*t, S_in=S, S_out=S, n_seqs=N, n_accept=acc, want_o=False)
    torch.cuda.synchronize()
    assert o_none is None and S_after is S
    assert torch.equal(S[2], S_keep[2])              # nothing accepted: the kept state
    for i, a in enumerate(accept):
        if a == 0:
            continue
        sl = [x.reshape(N, n, *x.shape[1:])[i, :a].clone() for x in t]   # fresh, aligned buffers
        o_i, S_i = kda.recurrent_fwd(*sl, S_in=S_keep[i:i + 1].clone(), n_seqs=1)
        torch.cuda.synchronize()
        assert torch.equal(S[i], S_i[0]), "sequence %d" % i
        assert torch.equal(o_draft.reshape(N, n, H, d)[i, :a], o_i)
        if a == n:
            assert torch.equal(S[i], S_draft[i])
