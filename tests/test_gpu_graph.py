"""A whole speculation step (tree build, verification, KV compaction)
captured in a HIP graph and replayed: every replay must reproduce the eager
step bit for bit.  Between replays the caches are restored and the outputs
cleared by eager work on the same stream, with host synchronisation, so each
replay starts from the same state as the eager step.  Cases: a bf16 tree with
stochastic verification, a bf16 chain over a vocabulary-wide LM head (the
one-launch chain tail), and an EAGLE-3.1 tree (its normed recurrent output is
a device-to-device copy inside the graph)."""

import numpy as np
import pytest
import torch

from gpu_helpers import DEV, announce
from speculative_decoding_aux_amd import spec as S
from speculative_decoding_aux_amd.tensors import to_device, upload_kv, upload_weights
from synth import configs, gen

pytestmark = pytest.mark.gpu

SMALL = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512, vocab=2048,
             draft_vocab=2048, top_k=3, depth=3, total_tokens=8, dtype="bf16", batch=3, ctx=40)

CASES = {
    "tree_stochastic": (dict(SMALL), 1),
    "chain_bigvocab": (dict(SMALL, vocab=70000, draft_vocab=70000, top_k=1, depth=4, total_tokens=4), 0),
    "tree_eagle31": (dict(SMALL, fc_norm=1, norm_output=1), 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_the_eager_step(name):
    over, mode = CASES[name]
    announce(f"graph replay {name}")
    cfg = configs.get("tiny_chain", **over)
    B, D = cfg["batch"], cfg["depth"]
    seed = 950 + len(name)
    W = gen.make_weights(cfg, seed)
    inp = gen.make_step_inputs(cfg, seed)
    ctx = S.SpecContext(cfg, max_batch=B)
    w = upload_weights(cfg, W)
    draft = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
    k0, v0 = draft.k.clone(), draft.v.clone()
    aux = to_device(inp["aux"], cfg["dtype"])
    tok = torch.from_numpy(inp["in_tokens"]).to(DEV)
    cl = torch.from_numpy(inp["ctx_len"]).to(DEV)
    base = (cl + cfg["n_new"] - 1).to(torch.int32)
    tree = S.Tree(B, cfg["total_tokens"] + 1, DEV)
    # target logits and uniforms planted on the eager step's own tree
    S.spec_build_tree(ctx, w, draft, aux, tok, cl, tree=tree)
    torch.cuda.synchronize()
    logits = torch.from_numpy(gen.plant_target_logits(cfg, tree.numpy(), seed)).to(DEV)
    u = torch.from_numpy(gen.make_accept_u(cfg, seed, batch=B)).to(DEV) if mode else None
    pseed = gen.philox_seed(seed)
    out = (torch.empty(B, D + 1, dtype=torch.int32, device=DEV), torch.empty(B, dtype=torch.int32, device=DEV),
           torch.empty(B, D, dtype=torch.int32, device=DEV))

    def reset():
        draft.k.copy_(k0)
        draft.v.copy_(v0)
        for t in out:
            t.fill_(-7)

    def step():
        S.spec_build_tree(ctx, w, draft, aux, tok, cl, tree=tree)
        S.spec_verify_tree(ctx, tree, logits, mode, 1.0, u, pseed, out=out)
        S.spec_compact_kv(ctx, draft, base, out[2], out[1])

    def snapshot():
        torch.cuda.synchronize()
        t = tree.numpy()
        return ({f: np.array(t[f]) for f in ("tokens", "parent", "depth", "position", "score")},
                [o.cpu().numpy() for o in out], draft.k.cpu().clone(), draft.v.cpu().clone())

    reset()
    step()
    want = snapshot()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        reset()
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for f in want[0]:
            np.testing.assert_array_equal(got[0][f], want[0][f], err_msg=f"replay {rep} tree {f}")
        for a, b in zip(got[1], want[1]):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep} verification")
        assert torch.equal(got[2], want[2]) and torch.equal(got[3], want[3]), f"replay {rep} KV"
    assert want[1][1].max() >= 0
