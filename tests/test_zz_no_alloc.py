"""GPU test of the allocation-free verification entry point
(spec_verify_tree_static): its results equal spec_verify_tree's on the same
trees and logits, through the C ABI, for greedy and stochastic verification,
on two calls in a row (the second with a smaller batch, tree and vocabulary,
so stale scratch from the first call would show)."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce, tree_to_device
from speculative_decoding_aux_amd import spec as S
from synth import configs, gen

pytestmark = pytest.mark.gpu


def _inputs(cfg, B, seed, mode):
    tree = gen.random_tree(cfg, seed, batch=B)
    logits = gen.plant_target_logits(dict(cfg, batch=B), tree, seed)
    if mode:
        # raise the drafted children so that stochastic acceptance happens
        for b in range(B):
            for c in range(1, int(tree["num_nodes"][b]) + 1):
                logits[b, tree["parent"][b, c], tree["tokens"][b, c]] += 12.0
    u = gen.make_accept_u(cfg, seed, batch=B) if mode else None
    return tree, logits, u


@pytest.mark.parametrize("mode", [0, 1])
def test_static_verify_equals_verify(mode):
    shapes = [  # (config, B, vocab): the second call is smaller in every way
        ("qwen8b_tree", 32, 151936),
        ("qwen4b_tree", 3, 50000),
    ]
    for i, (name, B, V) in enumerate(shapes):
        announce(f"static verify mode={mode} call {i}: {name} B={B} V={V}")
        cfg = configs.get(name, batch=B, vocab=V, draft_vocab=min(V, 32000))
        seed = configs.SEEDS[name] + 900 + i
        tree, logits, u = _inputs(cfg, B, seed, mode)
        ctx = S.SpecContext(cfg, max_batch=B)
        tr = tree_to_device(tree, ctx)
        lg = torch.from_numpy(logits).to(DEV)
        ut = torch.from_numpy(u).to(DEV) if u is not None else None
        pseed = gen.philox_seed(seed)
        want = S.spec_verify_tree(ctx, tr, lg, mode, 1.0, ut, pseed)
        got = S.spec_verify_tree_static(tr, lg, mode, cfg["total_tokens"], cfg["depth"], cfg["top_k"], 1.0, ut,
                                        pseed)
        torch.cuda.synchronize()
        for g, w in zip(got, want):
            np.testing.assert_array_equal(g.cpu().numpy(), w.cpu().numpy())
        assert want[1].cpu().numpy().max() > 0  # some drafts were accepted
        ctx.close()


def test_static_verify_rejects_oversized_shapes():
    # 40000 sequences of 64 nodes need far more than the fixed scratch: the
    # call is refused on the host, before any launch
    tr = S.Tree(40000, 64, DEV)
    lg = torch.zeros(40000, 64, 8, device=DEV)
    with pytest.raises(S.SpecError, match="scratch bytes"):
        S.spec_verify_tree_static(tr, lg, 0, 63, 7, 8)
