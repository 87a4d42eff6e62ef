"""GPU parity of the restore and permute variants: moe_combine_rows on bf16,
fp16 and fp32 rows, with and without routing weights (score applied before
the experts) and with a shared expert's rows merged, and moe_permute_weighted;
against oracle.combine.combine_rows / oracle.permute.permute_weighted, all
bit-exact (both sides do the same fp32 operations and one rounding)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from workloads import MoEConfig
from oracle import combine as ocombine, layout as olayout, permute as opermute, route as oroute
from gpu_util import DEV, bits, f64, from_bits, i32

pytestmark = pytest.mark.gpu
moe = pytest.importorskip("combine_top_router_amd")

SHAPES = {
    "tiny": (workloads.get("tiny"), 1),
    "ragged": (MoEConfig(name="ragged_var", num_tokens=3000, hidden=392, num_experts=16,
                         top_k=4, inter=128, ep_size=4, local_rank=2, align=128), 2),
    "deepseek_share": (workloads.get("deepseek_v3_ep8_share"), 0),
}
DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _routing(name):
    cfg, share = SHAPES[name]
    _, logits = workloads.gen.routing_inputs(cfg, "balanced", 0, device="cpu")
    idx = oroute.select(logits.numpy(), cfg.top_k)
    w = oroute.weights(logits.numpy(), idx).astype(np.float32)
    L = olayout.layout(idx, cfg.num_experts, cfg.ep_size, share, cfg.align)
    return cfg, w, L


def _values(t: torch.Tensor) -> np.ndarray:
    return f64(t) if t.dtype == torch.bfloat16 else t.detach().cpu().double().numpy()


def _same_bits(a: torch.Tensor, b: np.ndarray, dtype):
    """a (device rows) equals the float64 values b rounded to dtype, bit for bit."""
    want = torch.from_numpy(np.ascontiguousarray(b)).to(dtype)
    got = a.cpu()
    assert torch.equal(got.view(torch.int16 if dtype != torch.float32 else torch.int32),
                       want.view(torch.int16 if dtype != torch.float32 else torch.int32))


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("dt", list(DTYPES))
@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("with_shared", [False, True])
def test_combine_rows(name, dt, weighted, with_shared):
    print("CASE combine_rows", name, dt, weighted, with_shared, flush=True)
    cfg, w, L = _routing(name)
    dtype = DTYPES[dt]
    rows = max(int(L["offsets"][-1]), 1)
    y = workloads.gen.random_rows(cfg, rows, dtype, 0)
    shared = workloads.gen.random_rows(cfg, cfg.num_tokens, dtype, 1) if with_shared else None
    out = moe.ops.combine_rows(y.to(DEV), i32(L["dst_row"]),
                               torch.from_numpy(w).to(DEV) if weighted else None,
                               shared.to(DEV) if with_shared else None)
    torch.cuda.synchronize()
    want = ocombine.combine_rows(_values(y), L["dst_row"], w if weighted else None,
                                 _values(shared) if with_shared else None, row_dtype=dt)
    _same_bits(out, want, dtype)


@pytest.mark.parametrize("name", list(SHAPES))
def test_permute_weighted(name):
    print("CASE permute_weighted", name, flush=True)
    cfg, w, L = _routing(name)
    share = SHAPES[name][1]
    x = workloads.gen.random_rows(cfg, cfg.num_tokens, torch.bfloat16, 2)
    m_cap = cfg.m_cap(share)
    xp = from_bits(np.full((m_cap, cfg.hidden), 0x7FC1, dtype=np.uint16))
    moe.ops.permute_weighted(x.to(DEV), i32(L["dst_row"]), torch.from_numpy(w).to(DEV), m_cap,
                             out=xp)
    torch.cuda.synchronize()
    want, written = opermute.permute_weighted(f64(x), L["dst_row"], w, m_cap)
    got = bits(xp)
    r = np.nonzero(written)[0]
    np.testing.assert_array_equal(got[r], bits(torch.from_numpy(want[r].astype(np.float32))
                                               .to(torch.bfloat16)))
    assert (got[~written] == 0x7FC1).all()
