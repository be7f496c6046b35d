"""GPU parity of sequence-parallel state passing on one GPU: segment
transitions (kda_chunk_transition), state composition (kda_compose_states),
and the whole scheme (sequence_parallel_fwd) against the single-pass fp64
oracle.  Bars: bf16 inputs 2e-2 (per (sequence, head) slice, max|err| /
max|ref|), fp32 composition 1e-5."""
import sys

import numpy as np
import pytest

import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu


def _say(msg):
    print("[gpu-seqpar] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd  # noqa: F401
    return torch, torch.device("cuda:0")


def _bf(torch, dev, x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)


# With the workloads' decay (mean log-decay -2.5) a transition over more than
# a few tokens is ~exp(-2.5 T) and compares as zero; `weak` rescales the
# log-decay into (-0.025, 0) so the products of (I - beta k k^T) stay O(1).
# 40 sequences x 4 heads: more 16-column chains than CUs, so the transition
# runs on 32-column workgroups
MANY = [int(x) for x in np.random.default_rng(31).integers(0, 200, size=40)]


@pytest.mark.parametrize("lengths,H,d,weak", [([300], 2, 128, True), ([150, 77, 0, 64, 200], 3, 64, True),
                                              ([1, 65], 2, 128, False), ([300], 2, 128, False),
                                              (MANY, 4, 128, True), (MANY, 4, 64, True)],
                         ids=["one-seq-d128-weak", "varlen-d64-weak", "tiny-d128", "one-seq-d128",
                              "many-d128-weak", "many-d64-weak"])
def test_transition_matches_oracle(torch_dev, lengths, H, d, weak):
    """P = prod (I - beta k k^T) Diag(alpha): the oracle's recurrence with
    v = 0 from S0 = I gives it exactly (its S_T)."""
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    spec = ki.custom("tr", "bf16", lengths, H, d, varlen=True, seed=len(lengths) + d)
    inp = ki.generate_numpy(spec)
    if weak:
        inp.g[:] = ki.round_bf16(inp.g * 0.005)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    P = kda.chunk_transition(_bf(torch, dev, inp.k), _bf(torch, dev, inp.beta), _bf(torch, dev, inp.g),
                             cu_seqlens=cu)
    torch.cuda.synchronize()
    N = len(lengths)
    eye = np.broadcast_to(np.eye(d), (N, H, d, d)).copy()
    _, P_ref = oracle.forward(inp.k, inp.k, np.zeros_like(inp.v), inp.beta, inp.g, eye, inp.cu_seqlens)
    err = oracle.parity_error(P.cpu().numpy(), P_ref)
    _say("transition %s H=%d d=%d weak=%s: err %.3e (max|P| %.2e)" % (lengths, H, d, weak, err, np.abs(P_ref).max()))
    assert err <= 2e-2
    for n, L in enumerate(lengths):
        if L == 0:
            assert np.array_equal(P[n].cpu().numpy(), eye[n])   # empty sequence: identity


def test_compose_states_matches_definition(torch_dev):
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    rng = np.random.default_rng(5)
    for G, H, d in ((5, 3, 128), (1, 2, 64), (7, 1, 64)):
        P = (rng.standard_normal((G, H, d, d)) / np.sqrt(d)).astype(np.float32)
        Z = rng.standard_normal((G, H, d, d)).astype(np.float32)
        S0 = rng.standard_normal((H, d, d)).astype(np.float32)
        S = kda.compose_states(torch.from_numpy(P).to(dev), torch.from_numpy(Z).to(dev), torch.from_numpy(S0).to(dev))
        torch.cuda.synchronize()
        ref = [S0.astype(np.float64)]
        for g in range(G):
            ref.append(P[g].astype(np.float64) @ ref[-1] + Z[g])
        ref = np.stack(ref)
        err = np.max(np.abs(S.cpu().numpy() - ref)) / np.max(np.abs(ref))
        _say("compose G=%d H=%d d=%d: err %.3e" % (G, H, d, err))
        assert err <= 1e-5


@pytest.mark.parametrize("T,H,d,G,weak", [(1000, 2, 128, 4, False), (777, 3, 64, 5, False), (4096, 2, 128, 8, False),
                                          (1000, 2, 128, 4, True), (777, 3, 64, 5, True)])
def test_sequence_parallel_matches_single_pass_oracle(torch_dev, T, H, d, G, weak):
    import gated_delta_rule_30_amd as kda
    torch, dev = torch_dev
    spec = ki.custom("sp", "bf16", [T], H, d, s0_std=0.3, varlen=False, seed=T + G)
    inp = ki.generate_numpy(spec)
    if weak:   # incoming states carry across segments
        inp.g[:] = ki.round_bf16(inp.g * 0.005)
    t = [_bf(torch, dev, getattr(inp, name)) for name in ("q", "k", "v", "beta", "g")]
    S0 = torch.from_numpy(inp.S0).to(dev)
    o, ST = kda.sequence_parallel_fwd(*t, S0=S0, n_segments=G)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.g, inp.S0, inp.cu_seqlens)
    eo = oracle.parity_error(o.float().cpu().numpy(), o_ref, inp.cu_seqlens)
    es = oracle.parity_error(ST.cpu().numpy(), S_ref)
    _say("sequence-parallel T=%d H=%d d=%d G=%d weak=%s: o %.3e  S_T %.3e" % (T, H, d, G, weak, eo, es))
    assert eo <= 2e-2 and es <= 2e-2
