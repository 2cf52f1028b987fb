"""Pins of the oracle's draft pass (CPU only): an independent torch float64
formulation built from library routines, and closed-form special cases."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import draft as od
from oracle import numerics as on
from synth import configs, gen


def _cfg(dtype, **kw):
    base = dict(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, intermediate=96, vocab=512,
                draft_vocab=512, top_k=2, depth=3, total_tokens=4, dtype=dtype, batch=2, ctx=12)
    base.update(kw)
    return configs.get("tiny_chain", **base)


# ------------------------------------------------------------ numerics
def test_bf16_rounding_known_patterns():
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -1 - 2**-8, 3.4e38], np.float64)
    got = on.to_storage(x, "bf16")
    want = [1.0, 1.0, 1 + 2**-6, 1 + 2**-7, -1.0, np.inf]
    assert got.tolist() == want
    t = torch.tensor(np.random.default_rng(0).normal(size=1000).astype(np.float32))
    np.testing.assert_array_equal(on.to_storage(t.numpy(), "bf16"), t.to(torch.bfloat16).float().numpy())


def test_rope_identities():
    rng = np.random.default_rng(1)
    x = rng.normal(size=(5, 64))
    np.testing.assert_allclose(on.rope(x, np.zeros(5), 10000.0), x, atol=0)
    y = on.rope(x, np.full(5, 37.0), 10000.0)
    # each (i, i + hd/2) pair keeps its length
    np.testing.assert_allclose(x[:, :32] ** 2 + x[:, 32:] ** 2, y[:, :32] ** 2 + y[:, 32:] ** 2, rtol=1e-12)
    # rotations compose
    np.testing.assert_allclose(on.rope(on.rope(x, np.full(5, 5.0), 500.0), np.full(5, 9.0), 500.0),
                               on.rope(x, np.full(5, 14.0), 500.0), atol=1e-12)


def test_rmsnorm_of_constant_vector():
    x = np.full((2, 16), 3.0)
    np.testing.assert_allclose(on.rmsnorm(x, np.ones(16), 0.0), np.ones((2, 16)))
    np.testing.assert_allclose(on.rmsnorm(-x, np.full(16, 2.0), 0.0), -2 * np.ones((2, 16)))


# ----------------------------------------------------- attention cases
def test_attention_special_cases():
    rng = np.random.default_rng(2)
    kc = rng.normal(size=(2, 10, 16))
    vc = rng.normal(size=(2, 10, 16))
    q = rng.normal(size=(4, 16))
    out = od.attention_row(q, kc, vc, np.array([6]), 2)
    np.testing.assert_allclose(out[:2], np.tile(vc[0, 6], (2, 1)))
    np.testing.assert_allclose(out[2:], np.tile(vc[1, 6], (2, 1)))
    out = od.attention_row(np.zeros((4, 16)), kc, vc, np.array([1, 3, 4]), 2)
    np.testing.assert_allclose(out[0], vc[0, [1, 3, 4]].mean(0), atol=1e-12)
    assert not od.attention_row(q, kc, vc, np.array([], np.int64), 2).any()


def test_window_visibility():
    cfg = _cfg("f32", sliding_window=1)
    assert od.visible_slots(cfg, 50, 48, [48, 60, 61]).tolist() == [61]
    cfg = _cfg("f32", sliding_window=4)
    # query at 50; chain slots 48, 60, 61 hold positions 48, 49, 50
    assert od.visible_slots(cfg, 50, 48, [48, 60, 61, -1]).tolist() == [47, 48, 60, 61]
    cfg = _cfg("f32", sliding_window=0)
    assert od.visible_slots(cfg, 50, 3, [48, 60, 61]).tolist() == [0, 1, 2, 48, 60, 61]


# --------------------------------------- P6: independent torch formulation
def _torch_pass(cfg, W, kc, vc, mode, hidden, tokens, seq, pos, slot, vis_fn):
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    if cfg["dtype"] == "bf16":
        rnd = lambda x: x.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    else:
        rnd = lambda x: x.to(torch.float32).to(torch.float64)
    H, nq, nkv, hd, I = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "intermediate"))
    eps = cfg["rms_eps"]
    x = t(hidden)
    g = rnd(x @ t(W["fc"]).T) if mode == 0 else rnd(x)
    e = t(W["embed"])[torch.tensor(tokens)]
    c = torch.cat([rnd(F.rms_norm(e, (H,), t(W["input_norm"]), eps)),
                   rnd(F.rms_norm(g, (H,), t(W["hidden_norm"]), eps))], dim=1)
    qkv = rnd(c @ t(W["wqkv"]).T)
    M = x.shape[0]
    q = qkv[:, : nq * hd].reshape(M, nq, hd)
    k = qkv[:, nq * hd:(nq + nkv) * hd].reshape(M, nkv, hd)
    v = qkv[:, (nq + nkv) * hd:].reshape(M, nkv, hd)

    def rot(z, p):  # complex-number form of the rotation
        half = hd // 2
        ang = torch.tensor(p, dtype=torch.float64)[:, None, None] * \
            torch.tensor(cfg["rope_base"], dtype=torch.float64) ** (-torch.arange(half, dtype=torch.float64) * 2 / hd)
        zc = torch.complex(z[..., :half], z[..., half:]) * torch.polar(torch.ones_like(ang), ang)
        return torch.cat([zc.real, zc.imag], dim=-1)

    q, k = rnd(rot(q, pos)), rnd(rot(k, pos))
    K, Vc = t(kc), t(vc)
    for r in range(M):
        K[seq[r], :, slot[r]] = k[r]
        Vc[seq[r], :, slot[r]] = v[r]
    o = torch.zeros(M, nq * hd, dtype=torch.float64)
    group = nq // nkv
    for r in range(M):
        mask = torch.tensor(vis_fn(r), dtype=torch.bool)[None, None, None, :]
        kk = K[seq[r]].repeat_interleave(group, dim=0)[None]
        vv = Vc[seq[r]].repeat_interleave(group, dim=0)[None]
        o[r] = rnd(F.scaled_dot_product_attention(q[r][None, :, None, :], kk, vv, attn_mask=mask)).reshape(-1)
    h1 = rnd(g + o @ t(W["wo"]).T)
    m = rnd(F.rms_norm(h1, (H,), t(W["post_attn_norm"]), eps))
    gu = m @ t(W["w_gate_up"]).T
    s = rnd(F.silu(gu[:, :I]) * gu[:, I:])
    h_out = rnd(h1 + s @ t(W["w_down"]).T)
    n = rnd(F.rms_norm(h_out, (H,), t(W["final_norm"]), eps))
    return h_out.numpy(), (n @ t(W["lm_head"]).T).numpy(), K.numpy(), Vc.numpy()


@pytest.mark.parametrize("dtype,window", [("f32", 0), ("bf16", 0), ("bf16", 6)])
def test_draft_pass_matches_torch_formulation(dtype, window):
    cfg = _cfg(dtype, sliding_window=window)
    W = gen.make_weights(cfg, 21)
    inp = gen.make_step_inputs(cfg, 21, ctx_len=[12, 9])
    ctx = inp["ctx_len"]
    S = cfg["kv_capacity"]
    # slot -> position: context and root slots hold their own index; the two
    # beam rows of the second pass share position ctx+1
    posmap = [dict((s, s) for s in range(S)) for _ in range(2)]

    def vis(seq_r, pq, extra):
        def f(r):
            b = seq_r[r]
            ok = np.zeros(S, bool)
            for s in range(S):
                p = posmap[b][s]
                inwin = window == 0 or pq[r] - window < p <= pq[r]
                ok[s] = inwin and (s < ctx[b] or s in extra[r])
            return ok
        return f

    kc_o, vc_o = inp["k_cache"].copy(), inp["v_cache"].copy()
    kc_t, vc_t = inp["k_cache"].copy(), inp["v_cache"].copy()
    # pass 1: one root row per sequence, initial mode
    seq = [0, 1]
    pos = [int(ctx[0]), int(ctx[1])]
    anc = [[pos[0]], [pos[1]]]
    o1 = od.draft_pass(cfg, W, kc_o, vc_o, 0, inp["aux"][:, 0], inp["in_tokens"][:, 0], seq, pos, pos, ctx, anc)
    h_t, z_t, kc_t, vc_t = _torch_pass(cfg, W, kc_t, vc_t, 0, inp["aux"][:, 0], inp["in_tokens"][:, 0],
                                        seq, pos, pos, vis(seq, pos, [set(a) for a in anc]))
    tol = dict(atol=1e-5, rtol=1e-5) if dtype == "f32" else dict(atol=2e-2, rtol=0)
    np.testing.assert_allclose(o1["logits"], z_t, **tol)
    np.testing.assert_allclose(o1["h_out"], h_t, **tol)
    # pass 2: two beam rows per sequence, recurrent mode, slots root+1, root+2
    seq2 = [0, 0, 1, 1]
    pos2 = [pos[0] + 1] * 2 + [pos[1] + 1] * 2
    slot2 = [pos[0] + 1, pos[0] + 2, pos[1] + 1, pos[1] + 2]
    for b, s in zip(seq2, slot2):
        posmap[b][s] = pos[b] + 1
    anc2 = [[pos[0], slot2[0]], [pos[0], slot2[1]], [pos[1], slot2[2]], [pos[1], slot2[3]]]
    hid = o1["h_out"][[0, 0, 1, 1]]
    toks = [3, 4, 5, 6]
    o2 = od.draft_pass(cfg, W, kc_o, vc_o, 1, hid, toks, seq2, pos2, slot2, ctx, anc2)
    h2, z2, kc_t, vc_t = _torch_pass(cfg, W, kc_t, vc_t, 1, hid, toks, seq2, pos2, slot2,
                                      vis(seq2, pos2, [set(a) for a in anc2]))
    np.testing.assert_allclose(o2["logits"], z2, **tol)
    np.testing.assert_allclose(kc_o, kc_t, **tol)


def test_wide_window_equals_full_attention():
    cfg0 = _cfg("bf16", sliding_window=0)
    cfgw = _cfg("bf16", sliding_window=64)
    W = gen.make_weights(cfg0, 22)
    inp = gen.make_step_inputs(cfg0, 22)
    args = (0, inp["aux"][:, 0], inp["in_tokens"][:, 0], [0, 1], [12, 12], [12, 12], inp["ctx_len"], [[12], [12]])
    a = od.draft_pass(cfg0, W, inp["k_cache"].copy(), inp["v_cache"].copy(), *args)
    b = od.draft_pass(cfgw, W, inp["k_cache"].copy(), inp["v_cache"].copy(), *args)
    np.testing.assert_array_equal(a["logits"], b["logits"])


# ------------------------------------------------ EAGLE-3.1 normalisation flags
def test_fc_norm_makes_the_pass_invariant_to_the_fc_scale():
    """With fc_norm the layer input is RMSNorm(FC(a)): scaling the FC weights
    by 8 (exact in bf16) leaves the pass unchanged (eps = 0); without it the
    scale changes the logits."""
    for flag in (1, 0):
        cfg = _cfg("bf16", fc_norm=flag, rms_eps=0.0)
        W = gen.make_weights(cfg, 23)
        inp = gen.make_step_inputs(cfg, 23)
        W8 = dict(W, fc=W["fc"] * np.float32(8.0))
        args = (0, inp["aux"][:, 0], inp["in_tokens"][:, 0], [0, 1], [12, 12], [12, 12], inp["ctx_len"],
                [[12], [12]])
        a = od.draft_pass(cfg, W, inp["k_cache"].copy(), inp["v_cache"].copy(), *args)
        b = od.draft_pass(cfg, W8, inp["k_cache"].copy(), inp["v_cache"].copy(), *args)
        if flag:
            np.testing.assert_allclose(a["logits"], b["logits"], rtol=0, atol=1e-6)
            np.testing.assert_array_equal(a["h_out"], b["h_out"])
        else:
            assert np.abs(a["logits"] - b["logits"]).max() > 1e-2


def test_norm_output_returns_the_normed_row():
    """With norm_output the recurrent output is the final-normed row: it
    equals the LM head's input and has unit RMS (gain 1), while the logits do
    not change."""
    cfg0 = _cfg("f32")
    cfg1 = _cfg("f32", norm_output=1)
    W = gen.make_weights(cfg0, 24)
    inp = gen.make_step_inputs(cfg0, 24)
    args = (0, inp["aux"][:, 0], inp["in_tokens"][:, 0], [0, 1], [12, 12], [12, 12], inp["ctx_len"],
            [[12], [12]])
    a = od.draft_pass(cfg0, W, inp["k_cache"].copy(), inp["v_cache"].copy(), *args)
    b = od.draft_pass(cfg1, W, inp["k_cache"].copy(), inp["v_cache"].copy(), *args)
    np.testing.assert_array_equal(a["logits"], b["logits"])
    np.testing.assert_array_equal(b["h_out"], b["normed"])
    np.testing.assert_allclose(np.sqrt((b["h_out"].astype(np.float64) ** 2).mean(axis=1)), 1.0, rtol=1e-5)
    assert not np.allclose(a["h_out"], b["h_out"])
