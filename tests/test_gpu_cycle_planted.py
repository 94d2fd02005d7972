"""The planted-acceptance variant of the cycle (a measurement harness for
tokens/s at the acceptance lengths the pages report; random weights alone
give tau ~ 1): accepted-prefix lengths k are planted into the target rows
between the head and the verification, which must then return tau = k + 1
under greedy and rejection-sampling verification, emit the drafted tokens
as the accepted prefix, and leave the target rows as they were.

Cases: the reduced bf16 drafter (3 ragged sequences), greedy with fp32
target rows and rejection sampling (Gumbel-max drafting) with bf16 target
rows; planted k of 0 (nothing accepted), gamma (bonus) and in between, then
k drawn by the harness at alpha = 0.86 over several cycles.
"""

import numpy as np
import pytest
import torch

from block_diffusion_speculative_kv_amd.cycle import Cycle
from synth import configs
from tests.helpers import device, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("verify,head,tdt", [("greedy", "argmax", "f32"),
                                             ("rs", "gumbel", "bf16")])
def test_planted_prefixes(verify, head, tdt):
    cfg = configs.small_bf16(verify=verify, lm_mode=head, target_dtype=tdt)
    cyc = Cycle(cfg, device=device(), n_new=4)
    assert cyc.can_plant()
    g, bs = cyc.gamma, cfg["bs"]
    pristine = cyc.target.clone()
    plans = [np.array([0, 7, g]), np.array([g, 0, 1]), np.array([g - 1, 3, 0])]
    plans += [cyc.plant_draw(10 + i, 0.86) for i in range(4)]
    for c, k in enumerate(plans):
        cyc.step(cycle=c, plant_k=k)
        torch.cuda.synchronize()
        tau = to_np(cyc.tau)
        assert np.array_equal(tau, k + 1), f"cycle {c}: tau {tau}, planted {k}"
        ids = to_np(cyc.ids).reshape(bs, g)
        toks = to_np(cyc.out_tokens)
        for b in range(bs):
            assert np.array_equal(toks[b, :k[b]], ids[b, :k[b]]), f"cycle {c} seq {b}"
        assert torch.equal(cyc.target, pristine), f"cycle {c}: target rows not restored"
