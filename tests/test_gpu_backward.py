"""GPU parity of the backward pass (kda_chunk_bwd) against the fp64 oracle's
gradients of the token-by-token recurrence (oracle.backward).

Bar: 2e-2 for bf16 inputs, per (sequence, head) slice max|gpu - ref| /
max|ref|, for dq, dk, dv, dbeta, dlog_alpha and dS0 -- the forward's bf16 bar.
The backward keeps bf16 operands for every matrix product and bf16 copies of
the per-chunk states; at d_k = d_v = 64 and 128 its worst slice error is
below 1e-2 in an fp64 model of exactly those roundings.
"""
import sys
import time

import numpy as np
import pytest

import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2
KEYS = ("dq", "dk", "dv", "dbeta", "dg", "dS0")


def _say(msg):
    print("[gpu-bwd] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd  # noqa: F401  (fails loudly if the library is missing)
    return torch, torch.device("cuda:0")


def _bf(torch, dev, x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch.bfloat16)


def _gpu_bwd(torch, dev, inp, dO, dS_T, varlen):
    import gated_delta_rule_30_amd as kda
    s = inp.spec
    q, k, v, beta, g, dOd = (_bf(torch, dev, a) for a in (inp.q, inp.k, inp.v, inp.beta, inp.g, dO))
    S0 = torch.from_numpy(inp.S0).to(dev) if inp.S0 is not None else None
    dST = torch.from_numpy(dS_T).to(dev) if dS_T is not None else None
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev) if varlen else None
    out = kda.chunk_bwd(q, k, v, beta, g, dOd, S0=S0, dS_T=dST, cu_seqlens=cu, n_seqs=s.n_seqs)
    torch.cuda.synchronize()
    return {key: val.float().cpu().numpy() for key, val in out.items()}


def _errors(inp, got, ref):
    cu = inp.cu_seqlens
    e = {}
    for key in ("dq", "dk", "dv", "dg"):
        e[key] = oracle.parity_error(got[key], ref[key], cu)
    e["dbeta"] = oracle.parity_error(got["dbeta"][:, :, None], ref["dbeta"][:, :, None], cu)
    e["dS0"] = oracle.parity_error(got["dS0"], ref["dS0"])
    return e


CASES = [
    # lengths, H, d, s0_std, pin_frac, varlen, with_dS_T, weak
    ((100, 37, 1, 64, 200), 2, 64, 0.02, 0.0, True, True, False),
    ((300,), 2, 128, 0.02, 0.25, True, True, False),
    ((256, 256), 3, 128, 0.0, 0.0, False, False, False),
    ((130, 77, 0, 200), 2, 64, 0.02, 0.0, True, True, True),
    ((1000,), 1, 128, 0.02, 0.25, True, True, True),
    ((100, 100, 100), 2, 64, 0.02, 0.0, False, True, False),
]


@pytest.mark.parametrize("lengths,H,d,s0,pin,varlen,with_dst,weak", CASES,
                         ids=["varlen-d64", "one-seq-d128-pinned", "equal-d128-no-state", "varlen-d64-weak",
                              "long-d128-weak", "equal-ragged-d64"])
def test_backward_matches_oracle(torch_dev, lengths, H, d, s0, pin, varlen, with_dst, weak):
    torch, dev = torch_dev
    spec = ki.Spec("bwd", "bf16", tuple(lengths), H, d, d, s0_std=s0, pin_frac=pin, varlen=varlen, seed=7)
    inp = ki.generate_numpy(spec)
    if weak:   # slow decay: gradients carry across many chunks
        inp.g[:] = ki.round_bf16(inp.g * 0.005)
    dO, dS_T = ki.generate_grads_numpy(spec, with_dS_T=with_dst)
    _say("case %s H=%d d=%d weak=%s" % (lengths, H, d, weak))
    got = _gpu_bwd(torch, dev, inp, dO, dS_T, varlen)
    t0 = time.time()
    ref = oracle.backward(inp.q, inp.k, inp.v, inp.beta, inp.g, dO, inp.S0, dS_T, inp.cu_seqlens)
    e = _errors(inp, got, ref)
    _say("  " + " ".join("%s=%.2e" % (key, e[key]) for key in KEYS) + "  (oracle %.1fs)" % (time.time() - t0))
    for key in KEYS:
        assert np.all(np.isfinite(got[key])), key
        assert e[key] <= TOL, "%s parity %.3e > %.0e" % (key, e[key], TOL)


def test_backward_empty_input(torch_dev):
    """No tokens: every token gradient is empty and dS0 = dS_T."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    H, d = 2, 64
    z = torch.zeros((0, H, d), dtype=torch.bfloat16, device=dev)
    zb = torch.zeros((0, H), dtype=torch.bfloat16, device=dev)
    dST = torch.randn((3, H, d, d), device=dev)
    cu = torch.zeros(4, dtype=torch.int32, device=dev)
    out = kda.chunk_bwd(z, z, z, zb, z, z, dS_T=dST, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert out["dq"].shape == (0, H, d)
    assert torch.equal(out["dS0"], dST)


def test_backward_config1_sampled(torch_dev):
    """The batched bf16 workload (B=4, H=16, T=4096, d=128), one backward
    launch over all of it; two (sequence, head) slices checked in full."""
    torch, dev = torch_dev
    spec = ki.headline_configs()[1]
    inp = ki.generate_numpy(spec)
    dO, dS_T = ki.generate_grads_numpy(spec)
    _say("config 1 backward: B=4 H=16 T=4096 d=128")
    got = _gpu_bwd(torch, dev, inp, dO, dS_T, False)
    L = spec.lengths[0]
    for n, h in ((0, 0), (3, 11)):
        sl = slice(n * L, (n + 1) * L)
        S0n = None if inp.S0 is None else inp.S0[n:n + 1, h:h + 1]
        ref = oracle.backward(inp.q[sl, h:h + 1], inp.k[sl, h:h + 1], inp.v[sl, h:h + 1], inp.beta[sl, h:h + 1],
                              inp.g[sl, h:h + 1], dO[sl, h:h + 1], S0n, dS_T[n:n + 1, h:h + 1])
        e = {key: oracle.parity_error(got[key][sl, h:h + 1], ref[key]) for key in ("dq", "dk", "dv", "dg")}
        e["dbeta"] = oracle.parity_error(got["dbeta"][sl, h:h + 1, None], ref["dbeta"][:, :, None])
        e["dS0"] = oracle.parity_error(got["dS0"][n:n + 1, h:h + 1], ref["dS0"])
        _say("  seq %d head %d: " % (n, h) + " ".join("%s=%.2e" % (key, e[key]) for key in KEYS))
        for key in KEYS:
            assert e[key] <= TOL, "%s parity %.3e > %.0e (seq %d head %d)" % (key, e[key], TOL, n, h)


def test_backward_headline_sampled(torch_dev):
    """The headline workload (B=1, H=32, T=65536, d=128, S0 ~ 0.02 N(0,1)) in
    one backward launch over all heads, with dO and dS_T drawn as the
    benchmark draws them; head 5 checked in full against the oracle."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    spec = ki.headline_configs()[2]
    inp = ki.generate_torch(spec, dev)
    T, H, d, N = spec.total_tokens, spec.n_heads, spec.d_k, spec.n_seqs
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed + 1000003)
    dO = torch.randn((T, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    dST = torch.randn((N, H, d, d), generator=gen, device=dev, dtype=torch.float32)
    _say("headline backward: B=1 H=32 T=65536 d=128")
    out = kda.chunk_bwd(inp.q, inp.k, inp.v, inp.beta, inp.g, dO, S0=inp.S0, dS_T=dST, n_seqs=N)
    torch.cuda.synchronize()
    h = 5
    host = lambda x: x[:, h:h + 1].float().cpu().numpy()
    t0 = time.time()
    ref = oracle.backward(host(inp.q), host(inp.k), host(inp.v), host(inp.beta), host(inp.g), host(dO),
                          inp.S0[:, h:h + 1].cpu().numpy(), dST[:, h:h + 1].cpu().numpy())
    e = {key: oracle.parity_error(host(out[key]), ref[key]) for key in ("dq", "dk", "dv", "dg")}
    e["dbeta"] = oracle.parity_error(host(out["dbeta"])[:, :, None], ref["dbeta"][:, :, None])
    e["dS0"] = oracle.parity_error(out["dS0"][:, h:h + 1].cpu().numpy(), ref["dS0"])
    _say("  head %d: " % h + " ".join("%s=%.2e" % (key, e[key]) for key in KEYS) +
         "  (oracle %.1fs)" % (time.time() - t0))
    for key in KEYS:
        assert e[key] <= TOL, "%s parity %.3e > %.0e" % (key, e[key], TOL)


@pytest.mark.parametrize("lengths,H,d,varlen", [((100, 37, 1, 64, 200), 2, 64, True), ((4096,) * 2, 4, 128, False)],
                         ids=["varlen-d64", "equal-d128"])
def test_training_pair_matches_recompute(torch_dev, lengths, H, d, varlen):
    """kda_chunk_fwd_train + kda_chunk_bwd_ctx give kda_chunk_fwd's o and S_T
    and kda_chunk_bwd's gradients bit for bit (same kernels, same inputs)."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    spec = ki.Spec("pair", "bf16", tuple(lengths), H, d, d, s0_std=0.02, varlen=varlen, seed=3)
    inp = ki.generate_numpy(spec)
    dO, dS_T = ki.generate_grads_numpy(spec)
    q, k, v, beta, g, dOd = (_bf(torch, dev, a) for a in (inp.q, inp.k, inp.v, inp.beta, inp.g, dO))
    S0 = torch.from_numpy(inp.S0).to(dev)
    dST = torch.from_numpy(dS_T).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev) if varlen else None
    N = spec.n_seqs
    o_ref, ST_ref = kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu, n_seqs=N)
    ref = kda.chunk_bwd(q, k, v, beta, g, dOd, S0=S0, dS_T=dST, cu_seqlens=cu, n_seqs=N)
    o, ST, ctx = kda.chunk_fwd_train(q, k, v, beta, g, S0=S0, cu_seqlens=cu, n_seqs=N)
    got = kda.chunk_bwd(q, k, v, beta, g, dOd, dS_T=dST, cu_seqlens=cu, n_seqs=N, context=ctx)
    torch.cuda.synchronize()
    _say("training pair %s H=%d d=%d" % (lengths, H, d))
    assert torch.equal(o, o_ref) and torch.equal(ST, ST_ref)
    for key in KEYS:
        assert torch.equal(got[key], ref[key]), key


def test_backward_config3_sampled(torch_dev):
    """The ragged packed batch (64 sequences, L ~ U[512, 16384], H=32, d=128,
    25 % of channels at g = -5) in one backward launch; the shortest and the
    longest sequence checked in full on two heads each."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    spec = ki.headline_configs()[3]
    inp = ki.generate_torch(spec, dev)
    T, H, d, N = spec.total_tokens, spec.n_heads, spec.d_k, spec.n_seqs
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed + 1000003)
    dO = torch.randn((T, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    dST = torch.randn((N, H, d, d), generator=gen, device=dev, dtype=torch.float32)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    _say("config 3 backward: N=64 varlen, H=32, d=128, pinned channels")
    out = kda.chunk_bwd(inp.q, inp.k, inp.v, inp.beta, inp.g, dO, S0=None, dS_T=dST, cu_seqlens=cu)
    torch.cuda.synchronize()
    lens = np.diff(inp.cu_seqlens)
    for n in (int(np.argmin(lens)), int(np.argmax(lens))):
        a, b = int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
        for h in (3, 30):
            host = lambda x: x[a:b, h:h + 1].float().cpu().numpy()
            ref = oracle.backward(host(inp.q), host(inp.k), host(inp.v), host(inp.beta), host(inp.g), host(dO),
                                  None, dST[n:n + 1, h:h + 1].cpu().numpy())
            e = {key: oracle.parity_error(host(out[key]), ref[key]) for key in ("dq", "dk", "dv", "dg")}
            e["dbeta"] = oracle.parity_error(host(out["dbeta"])[:, :, None], ref["dbeta"][:, :, None])
            e["dS0"] = oracle.parity_error(out["dS0"][n:n + 1, h:h + 1].cpu().numpy(), ref["dS0"])
            _say("  seq %d (len %d) head %d: " % (n, b - a, h) + " ".join("%s=%.2e" % (key, e[key]) for key in KEYS))
            for key in KEYS:
                assert e[key] <= TOL, "%s parity %.3e > %.0e (seq %d head %d)" % (key, e[key], TOL, n, h)


def test_long_sequence_paced_sampled(torch_dev):
    """One 131,072-token sequence: 2048 chunks, so the recurrence's slab
    workgroups pace each other (in the forward, the checkpointing forward and
    the state-gradient pass).  H=4, d=64, S0 ~ 0.02 N(0,1); the forward and
    the backward run over all heads, head 2 is checked in full against the
    oracle (o and S_T, and every gradient)."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    spec = ki.custom("paced", "bf16", [131072], 4, 64, s0_std=0.02, varlen=False, seed=9)
    inp = ki.generate_torch(spec, dev)
    T, H, d, N = spec.total_tokens, spec.n_heads, spec.d_k, spec.n_seqs
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.seed + 77)
    dO = torch.randn((T, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    dST = torch.randn((N, H, d, d), generator=gen, device=dev, dtype=torch.float32)
    _say("paced long sequence: T=131072 H=4 d=64")
    o, S_T = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.beta, inp.g, S0=inp.S0, n_seqs=N)
    out = kda.chunk_bwd(inp.q, inp.k, inp.v, inp.beta, inp.g, dO, S0=inp.S0, dS_T=dST, n_seqs=N)
    torch.cuda.synchronize()
    h = 2
    host = lambda x: x[:, h:h + 1].float().cpu().numpy()
    S0h = inp.S0[:, h:h + 1].cpu().numpy()
    t0 = time.time()
    o_ref, S_ref = oracle.forward(host(inp.q), host(inp.k), host(inp.v), host(inp.beta), host(inp.g), S0h)
    ref = oracle.backward(host(inp.q), host(inp.k), host(inp.v), host(inp.beta), host(inp.g), host(dO), S0h,
                          dST[:, h:h + 1].cpu().numpy())
    e = {"o": oracle.parity_error(host(o), o_ref), "S_T": oracle.parity_error(S_T[:, h:h + 1].cpu().numpy(), S_ref)}
    e.update({key: oracle.parity_error(host(out[key]), ref[key]) for key in ("dq", "dk", "dv", "dg")})
    e["dbeta"] = oracle.parity_error(host(out["dbeta"])[:, :, None], ref["dbeta"][:, :, None])
    e["dS0"] = oracle.parity_error(out["dS0"][:, h:h + 1].cpu().numpy(), ref["dS0"])
    _say("  head %d: " % h + " ".join("%s=%.2e" % kv for kv in e.items()) + "  (oracle %.1fs)" % (time.time() - t0))
    for key, err in e.items():
        assert err <= TOL, "%s parity %.3e > %.0e" % (key, err, TOL)
