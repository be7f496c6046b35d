"""Prefix-cache checkpoints (kda_chunk_fwd_ckpt): the state after every
`every`-th chunk of each sequence, against the fp64 oracle run on that
prefix; o and S_T unchanged from kda_chunk_fwd; the checkpoints packed in
sequence order and no slot past the last one written."""
import sys

import numpy as np
import pytest

import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2   # bf16 bar, per (sequence, head) slice


def _say(msg):
    print("[gpu-ckpt] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd  # noqa: F401
    return torch, torch.device("cuda:0")


@pytest.mark.parametrize("lengths,H,d,every,varlen", [
    ((700, 64, 1100, 0, 513), 2, 128, 2, True),
    ((700, 64, 1100, 0, 513), 2, 64, 8, True),
    ((600, 600), 3, 128, 3, False),
    ((64, 63, 65, 1, 200, 128), 2, 64, 1, True),
], ids=["varlen-d128-every2", "varlen-d64-every8", "equal-d128-every3", "varlen-d64-every1"])
def test_checkpoints_match_prefix_oracle(torch_dev, lengths, H, d, every, varlen):
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    spec = ki.custom("ckpt", "bf16", list(lengths), H, d, s0_std=0.3, varlen=varlen, seed=13)
    inp = ki.generate_numpy(spec)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    q, k, v, beta, g = (t(a) for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    S0 = torch.from_numpy(inp.S0).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev) if varlen else None
    N = len(lengths)
    nbytes = kda.ckpt_size(spec.total_tokens, N, H, d, d, every)
    S_ckpt = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=dev).view(-1, H, d, d)
    o, ST, _ = kda.chunk_fwd_ckpt(q, k, v, beta, g, every, S_ckpt=S_ckpt, S0=S0, cu_seqlens=cu, n_seqs=N)
    o_ref, ST_ref = kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu, n_seqs=N)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ST, ST_ref)
    ck = S_ckpt.cpu().numpy()
    slots = kda.ckpt_slots(lengths, every)
    written = set()
    worst = 0.0
    for n, lst in enumerate(slots):
        s0 = int(inp.cu_seqlens[n])
        for tokens, slot in lst:
            written.add(slot)
            sl = slice(s0, s0 + tokens)
            _, S_ref = oracle.forward(inp.q[sl], inp.k[sl], inp.v[sl], inp.beta[sl], inp.g[sl],
                                      inp.S0[n:n + 1], np.array([0, tokens], np.int64))
            for h in range(H):
                ref = S_ref[0, h]
                e = float(np.max(np.abs(ck[slot, h] - ref)) / max(np.max(np.abs(ref)), 1e-30))
                worst = max(worst, e)
    _say("%s H=%d d=%d every=%d: %d checkpoints, worst %.2e" % (lengths, H, d, every, len(written), worst))
    assert written, "no checkpoint in this case"
    assert worst <= TOL
    assert written == set(range(len(written))), "checkpoints are not packed from slot 0"
    assert len(written) <= ck.shape[0]
    assert np.all(np.isnan(ck[len(written):])), "a slot past the last checkpoint was written"
