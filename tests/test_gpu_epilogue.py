"""GPU parity of the output epilogue (kda_output_gate) against the fp64
oracle (oracle/epilogue.py): y = RMSNorm(o) * w * sigmoid(gate) per row.

Bar: the forward's, 1e-4 for fp32 and 2e-2 for bf16, as max|gpu - ref| /
max|ref| per head slice; in practice bf16 sits at its output rounding."""
import sys

import numpy as np
import pytest

import kda_inputs as ki
from oracle import epilogue

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print("[gpu-epilogue] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd  # noqa: F401
    return torch, torch.device("cuda:0")


def _err(y, ref):
    num = np.max(np.abs(y - ref), axis=(0, 2))
    den = np.maximum(np.max(np.abs(ref), axis=(0, 2)), 1e-30)
    return float(np.max(num / den))


@pytest.mark.parametrize("dtype,T,H,d,with_w,eps,inplace", [
    ("bf16", 1000, 3, 128, True, 1e-6, False), ("bf16", 77, 2, 64, False, 1e-5, True),
    ("f32", 513, 2, 64, True, 1e-6, False), ("f32", 300, 4, 128, False, 0.0, True),
    ("bf16", 1, 1, 128, True, 1e-6, False),
    # 1,120,016 rows: more than one pass of the grid-stride loop (16384 workgroups x 64 rows), ragged tail
    ("bf16", 70001, 16, 64, True, 1e-6, False)])
def test_output_gate_matches_oracle(torch_dev, dtype, T, H, d, with_w, eps, inplace):
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    rng = np.random.default_rng(T + d)
    rnd = ki.round_bf16 if dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    o = rnd(rng.standard_normal((T, H, d)).astype(np.float32) * rng.uniform(0.01, 3.0, (T, H, 1)).astype(np.float32))
    z = rnd(2.0 * rng.standard_normal((T, H, d)).astype(np.float32))
    w = rng.uniform(0.5, 1.5, d).astype(np.float32) if with_w else None
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    od = torch.from_numpy(o).to(dev).to(tdt)
    zd = torch.from_numpy(z).to(dev).to(tdt)
    wd = torch.from_numpy(w).to(dev) if w is not None else None
    y = kda.output_gate(od, zd, wd, eps=eps, out=od if inplace else None)
    torch.cuda.synchronize()
    ref = epilogue.output_gate(o, z, w, eps)
    e = _err(y.float().cpu().numpy(), ref)
    _say("%s T=%d H=%d d=%d weight=%s eps=%g inplace=%s: err %.2e" % (dtype, T, H, d, with_w, eps, inplace, e))
    assert e <= TOL[dtype]


def test_output_gate_on_headline_forward_output(torch_dev):
    """The epilogue applied to the forward's o at the headline shape (H=32,
    T=65536, d=128, bf16), one launch over all rows; 4096 seeded rows checked."""
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    spec = ki.headline_configs()[2]
    inp = ki.generate_torch(spec, dev)
    o, _ = kda.chunk_fwd(inp.q, inp.k, inp.v, inp.beta, inp.g, S0=inp.S0, output_final_state=False)
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    z = torch.randn(o.shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    w = torch.rand((o.shape[-1],), generator=gen, device=dev, dtype=torch.float32) + 0.5
    y = kda.output_gate(o, z, w, eps=1e-6)
    torch.cuda.synchronize()
    rows = np.random.default_rng(5).choice(o.shape[0] * o.shape[1], 4096, replace=False)
    flat = lambda t: t.reshape(-1, t.shape[-1])[torch.from_numpy(rows).to(dev)].float().cpu().numpy()
    ref = epilogue.output_gate(flat(o), flat(z), w.cpu().numpy(), 1e-6)
    e = float(np.max(np.abs(flat(y) - ref)) / np.max(np.abs(ref)))
    _say("headline rows: err %.2e" % e)
    assert e <= TOL["bf16"]
