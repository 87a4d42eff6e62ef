"""The seeded input generators that both the HIP path and the oracle are fed
from: reproducible, per-tensor seeds, and the value recipe and routing
distributions they document (CPU only)."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads
from workloads import MoEConfig, gen

CFG = MoEConfig(name="gen_check", num_tokens=2048, hidden=512, num_experts=256, top_k=8,
                inter=256, ep_size=8, local_rank=0, align=128,
                dists=("balanced", "mild", "severe", "zipf"))


def test_same_seed_same_inputs_other_seed_other_inputs():
    x0, l0 = gen.routing_inputs(CFG, "mild", 0)
    x1, l1 = gen.routing_inputs(CFG, "mild", 0)
    assert torch.equal(x0.view(torch.int16), x1.view(torch.int16)) and torch.equal(l0, l1)
    x2, l2 = gen.routing_inputs(CFG, "mild", 1)
    assert not torch.equal(x0.view(torch.int16), x2.view(torch.int16))
    assert not torch.equal(l0, l2)


def test_an_experts_weights_do_not_depend_on_its_neighbours():
    one = gen.expert_weights(CFG, [37], 0)
    many = gen.expert_weights(CFG, [5, 37, 200], 0)
    for a, b in zip(one, many):
        assert torch.equal(a[0].view(torch.int16), b[1].view(torch.int16))


def test_value_recipe():
    x, logits = gen.routing_inputs(CFG, "balanced", 0)
    xf = x.float()
    assert abs(xf.mean().item()) < 0.01 and abs(xf.std().item() - 1.0) < 0.01
    # logits = x Wr with Wr ~ N(0, 1/H): unit variance per logit
    assert abs(logits.std().item() - 1.0) < 0.03
    w1, w3, w2 = gen.expert_weights(CFG, range(8), 0)
    H, I = CFG.hidden, CFG.inter
    assert tuple(w1.shape) == (8, H, I) and tuple(w2.shape) == (8, I, H)
    for w, std in ((w1, 1 / math.sqrt(H)), (w3, 1 / math.sqrt(H)), (w2, 1 / math.sqrt(I))):
        assert abs(w.float().std().item() / std - 1.0) < 0.01
    assert not torch.equal(w1.view(torch.int16), w3.view(torch.int16))


def test_routing_distributions():
    E = CFG.num_experts
    assert not gen.routing_bias(CFG, "balanced").any()
    severe = gen.routing_bias(CFG, "severe").numpy()
    assert (severe == 3.0).sum() == 16 and ((severe == 0) | (severe == 3.0)).all()
    mild = gen.routing_bias(CFG, "mild").numpy().astype(np.float64)
    assert 0.35 < mild.var() < 0.65  # one N(0, 0.5) draw per expert, 256 experts
    zipf = np.sort(gen.routing_bias(CFG, "zipf").numpy().astype(np.float64))[::-1]
    np.testing.assert_allclose(zipf, -1.2 * np.log1p(np.arange(E)), rtol=0, atol=1e-6)
    with pytest.raises(ValueError):
        gen.routing_bias(CFG, "uniform")


def test_severe_routing_concentrates_on_the_hot_experts():
    # with +3 on 16 of 256 experts, most top-8 picks land on those 16
    _, logits = gen.routing_inputs(CFG, "severe", 0)
    hot = np.nonzero(gen.routing_bias(CFG, "severe").numpy() > 0)[0]
    top = torch.topk(logits, CFG.top_k, dim=1).indices.numpy()
    share = np.isin(top, hot).mean()
    assert share > 0.8, share


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_every_workload_has_its_distributions(name):
    cfg = workloads.get(name)
    for dist in cfg.dists:
        assert gen.routing_bias(cfg, dist).shape == (cfg.num_experts,)
