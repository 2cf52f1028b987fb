"""Benchmark of one speculation step (draft tree + verify + KV compaction).

A step is spec_build_tree + spec_verify_tree + spec_compact_kv for the whole
batch, on inputs already resident in HBM.  Default workload: the
Qwen3-8B-shaped tree (batch 32, context 2048, top_k 8 / depth 7 / 63 draft
tokens, stochastic verification at T = 1 against target logits made of the
oracle's draft logits of every node plus N(0, 1) noise), on synthetic seeded
inputs.  The oracle leg (cpu_baseline) runs first: it times whole oracle
steps on the host cores and prepares those target logits, which both legs
then verify.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                    [--graph] [--no-cpu-baseline] [--n-new N] [--paged BS]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "speculation steps/sec (draft tree + verify) at 1 GPU; HBM GB/s & MFMA util vs peak"
HBM_PEAK_GBS = 8000.0
# Kernel timing (events carried in the dispatch packets) runs on every
# PROF_EVERY-th timed step: it still costs the stream a few microseconds per
# timed launch, so the other steps run untimed.
PROF_EVERY = 5
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen8b_tree")
    ap.add_argument("--graph", action="store_true", help="replay the step as one captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the attainable-peak probes run after the timed steps")
    ap.add_argument("--cpu-steps", type=int, default=3)
    ap.add_argument("--flat-sampling", type=int, default=0, metavar="B",
                    help="instead of the step, time rejection sampling of a flat batch of B "
                         "variable-length chains with per-request temperature/top-k/top-p "
                         "(the workload's vocabulary and draft length)")
    ap.add_argument("--target-forward", type=int, default=0, metavar="L",
                    help="instead of the step, time the target's verification forward over the "
                         "workload's trees with L synthetic layers of the workload's shapes")
    ap.add_argument("--paged", type=int, default=0, metavar="BS",
                    help="keep the draft KV cache in a paged pool of BS-slot blocks (shuffled)")
    ap.add_argument("--n-new", type=int, default=0, metavar="N",
                    help="new aux rows per sequence on the root pass (default: the workload's, 1); "
                         "a sensitivity run, e.g. depth + 1 after a fully accepted chain")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (counter calibration)")
    return ap.parse_args()


def lm_head_bytes(cfg, M):
    """Algorithmic bytes of one LM-head launch over M rows: the weight stream
    and the normed rows in; out, the float32 logits, or - when the vocab
    top-k is fused into the launch (bf16 weight streaming at M <= 64,
    unsplit: Vd >= 65536, or column strips filling the grid) - one (top-k
    list, max, sum) record per row and column strip; beyond 64 rows (tiled
    head) one (max, sum exp) record per row and 128-column strip (the logits
    it also writes are a round trip the method does not need and are not
    counted).  EAGLE-4: the low-rank score GEMM, scores out."""
    H = cfg["hidden"]
    if cfg["cand_rank"]:
        r, V = cfg["cand_rank"], cfg["vocab"]
        return V * r * 2 + M * r * 2 + M * V * 4
    Vd, k = cfg["draft_vocab"], cfg["top_k"]
    if cfg["dtype"] == "bf16" and M > 64 and k <= 8:
        return Vd * H * 2 + M * H * 2 + M * -(-Vd // 128) * 8
    cw1 = M <= 16 and Vd >= 65536
    cols = 64 if cw1 else 128
    strips = -(-Vd // cols)
    unsplit = Vd >= 65536 or strips * -(-M // 64) >= (1024 if cw1 else 2048)
    fused = cfg["dtype"] == "bf16" and k <= 8 and M <= 64 and unsplit
    out = M * strips * (8 * (1 if k == 1 else 8) + 16) if fused else M * Vd * 4
    return Vd * H * 2 + M * H * 2 + out


def measured_traffic(workload, kernel="lm_head"):
    """HBM bytes per launch of the roofline kernel from the committed counter
    profile (FETCH_SIZE and WRITE_SIZE scaled by a copy of known size), or
    None when the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for src in rec["kernel_sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["kernel_source_sha256"] else None


def kernel_figures(cfg, rows, lm, lmt, att, ver, alen=None):
    """Per-label launch figures of the sampled steps: average launch time,
    algorithmic bytes (and, for the LM head, GEMM flops) per launch, achieved
    rates and their fractions of the published peaks.  LM head: the launches
    up to 64 rows (root pass, chains) and the tiled launches of the beam
    passes apart; attention: the visible context K and V of every (sequence,
    kv head) once per pass (the window at most); verify: the target-logit rows
    of the nodes the acceptance walks reach, once (alen: accepted lengths)."""
    es = 2 if cfg["dtype"] == "bf16" else 4
    B, nkv, hd = cfg["batch"], cfg["n_kv_heads"], cfg["head_dim"]
    ctx = min(cfg["ctx"], cfg["sliding_window"]) if cfg["sliding_window"] else cfg["ctx"]
    out = {}

    def rate(name, nl, ms, byts, flops=None):
        if nl <= 0:
            return
        us = ms / nl * 1e3
        e = {"avg_launch_us": round(us, 2), "launches": nl, "algorithmic_bytes_per_launch": int(byts),
             "achieved_gbs": round(byts / (us * 1e-6) / 1e9, 1)}
        e["frac"] = round(e["achieved_gbs"] / HBM_PEAK_GBS, 4)
        if flops:
            e["flops_per_launch"] = int(flops)
            e["mfma_tflops"] = round(flops / (us * 1e-6) / 1e12, 1)
            e["mfma_frac"] = round(e["mfma_tflops"] / BF16_PEAK_TFLOPS, 4)
        out[name] = e

    if cfg["dtype"] == "bf16" and not cfg["cand_rank"]:
        small = [m for m in rows if m <= 64]
        big = [m for m in rows if m > 64]
        for name, rs, (nl, ms) in (("lm_head", small, lm), ("lm_head_tiled", big, lmt)):
            if rs:
                byts = sum(lm_head_bytes(cfg, m) for m in rs) / len(rs)
                flops = sum(2.0 * m * cfg["draft_vocab"] * cfg["hidden"] for m in rs) / len(rs)
                rate(name, nl, ms, byts, flops)
    rate("attention", att[0], att[1], B * nkv * ctx * hd * 2 * es)
    # verify: the target-logit rows the walks need, (accepted + 1) per sequence
    vrows = int(np.sum(alen + 1)) if alen is not None else B * (cfg["total_tokens"] + 1)
    rate("verify", ver[0], ver[1], vrows * cfg["vocab"] * 4)
    if "verify" in out:
        out["verify"]["rows_needed"] = vrows
    return out


def pass_rows(cfg):
    B, k, D, n_new = cfg["batch"], cfg["top_k"], cfg["depth"], cfg["n_new"]
    return [B * n_new] + [B * k] * (D - 1)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return os.cpu_count()


def _oracle_step(cfg, W, inp, seed, make_logits, sl=slice(None)):
    """One whole step of the oracle over the sequences ``sl``: tree build,
    verification, compaction (of a 1-layer target-shaped cache).  The target
    logits come from ``make_logits(tree, sub_cfg, record, caches)`` between
    the build and the verification; that preparation is not timed.  Returns
    (seconds, accepted lengths, logits)."""
    from oracle import compact as oc
    from oracle import tree as ot
    from oracle import verify as ov
    from synth import gen

    B = len(range(*sl.indices(cfg["batch"])))
    c = dict(cfg, batch=B)
    kc, vc = inp["k_cache"][sl].copy(), inp["v_cache"][sl].copy()
    ctx_len = inp["ctx_len"][sl]
    rec = []
    t0 = time.perf_counter()
    tree = ot.build_tree(c, W, kc, vc, inp["aux"][sl], inp["in_tokens"][sl], ctx_len, record=rec)
    t1 = time.perf_counter()
    logits = make_logits(tree, c, rec, (kc, vc), sl)
    del rec
    t2 = time.perf_counter()
    if cfg["verify"] == "greedy":
        out, alen, nodes = ov.verify_greedy(tree, logits, cfg["depth"])
    else:
        u = gen.make_accept_u(cfg, seed)[sl]
        out, alen, nodes = ov.verify_stochastic(tree, logits, cfg["depth"], cfg["temperature"], u,
                                                gen.philox_seed(seed))
    base = ctx_len + cfg["n_new"] - 1
    tk = np.zeros((1, B, cfg["n_kv_heads"], cfg["kv_capacity"], cfg["head_dim"]), np.float32)
    oc.compact_kv(tk, tk.copy(), base, nodes, alen)
    t3 = time.perf_counter()
    return (t1 - t0) + (t3 - t2), alen, logits


def oracle_leg(cfg, W, inp, seed, steps):
    """The oracle, as it stands, timed on the host cores, on whole steps of
    the same workload (same weights and inputs).  For the workload whose
    target logits are the draft's own logits plus N(0, 1) noise, the first
    step's tree gives those logits (the draft logits of every node, with one
    extra pass for the nodes it never expanded; not timed) and every step,
    and the GPU leg, verifies them.  Returns (cpu_baseline, target logits of
    the whole batch or None)."""
    from oracle import tree as ot
    from synth import gen

    threads = _blas_threads()
    noisy = cfg["target_logits"] == "draft_plus_noise"
    held = {}

    def make_logits(tree, c, rec, caches, sl):
        if not noisy:
            return gen.plant_target_logits(c, tree, seed)
        if "tl" not in held:
            t0 = time.perf_counter()
            dl = ot.node_draft_logits(c, W, caches[0], caches[1], inp["ctx_len"][sl], tree, rec)
            held["tl"] = gen.add_noise_logits(dl, seed)
            print(f"[bench] oracle draft logits of every node: {time.perf_counter() - t0:.1f} s",
                  file=sys.stderr, flush=True)
        return held["tl"][sl]

    times = []
    for s in range(steps):
        sec, _, _ = _oracle_step(cfg, W, inp, seed, make_logits)
        times.append(sec)
        print(f"[bench] oracle step {s + 1}/{steps}: {sec:.2f} s", file=sys.stderr, flush=True)
    med = float(np.median(times))
    B = cfg["batch"]
    res = {"value": round(1.0 / med, 5), "unit": "steps/s", "cores": int(threads),
           "host_cpus": os.cpu_count(), "kind": "oracle",
           "sample": f"{steps} whole steps of the same workload (batch {B}); median {med:.3f} s per step "
                     f"(all: {', '.join(f'{t:.2f}' for t in times)} s); numpy with {threads} BLAS threads; "
                     f"compaction on a 1-layer cache; target-logit preparation not timed"}
    # the same step on one thread, over a bounded sample of the sequences
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return res, held.get("tl")
    bs = max(1, B // 8)
    with threadpool_limits(limits=1):
        sec1 = _oracle_step(cfg, W, inp, seed, make_logits, sl=slice(0, bs))[0]
    res["value_1thread"] = round(1.0 / (sec1 * B / bs), 5)
    res["sample_1thread"] = (f"1 whole step over {bs} of the {B} sequences on 1 thread: {sec1:.2f} s, "
                             f"scaled by {B}/{bs} to the batch")
    print(f"[bench] oracle on 1 thread, {bs} sequences: {sec1:.2f} s", file=sys.stderr, flush=True)
    return res, held.get("tl")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported in this build "
              "(the step is data-parallel over sequences and would shard by batch)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "launches": 3}))
        return

    if args.flat_sampling:
        bench_flat_sampling(args)
        return
    if args.target_forward:
        bench_target_forward(args)
        return

    from speculative_decoding_aux_amd import spec as S
    from speculative_decoding_aux_amd import _lib as L
    from speculative_decoding_aux_amd.tensors import to_device, upload_kv, upload_weights
    from synth import configs, gen

    cfg = configs.get(args.config, **({"n_new": args.n_new} if args.n_new else {}))
    seed = configs.SEEDS[args.config]
    B = cfg["batch"]
    print(f"[bench] generating inputs for {args.config}", file=sys.stderr, flush=True)
    W = gen.make_weights(cfg, seed)
    inp = gen.make_step_inputs(cfg, seed)
    cpu_res, tl_oracle = None, None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu_res, tl_oracle = oracle_leg(cfg, W, inp, seed, args.cpu_steps)
    dev = "cuda"
    w = upload_weights(cfg, W)
    draft_kv = upload_kv(cfg, inp["k_cache"], inp["v_cache"])
    if args.paged:
        draft_kv = paged_copy(draft_kv, args.paged, seed)
    aux = to_device(inp["aux"], cfg["dtype"])
    in_tok = torch.from_numpy(inp["in_tokens"]).to(dev)
    ctx_len = torch.from_numpy(inp["ctx_len"]).to(dev)
    # target-shaped KV for compaction: target_layers x [B, nkv, ctx + N + 1 (+pad), hd]
    t_slots = cfg["ctx"] + cfg["n_new"] + cfg["total_tokens"] + 8
    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(seed)
    tshape = (cfg["target_layers"], B, cfg["n_kv_heads"], t_slots, cfg["head_dim"])
    target_kv = S.KVCache(torch.randn(tshape, generator=g, device=dev).to(tdt),
                          torch.randn(tshape, generator=g, device=dev).to(tdt))
    tree_base = (ctx_len + cfg["n_new"] - 1).to(torch.int32)
    ctx = S.SpecContext(cfg, max_batch=B, max_new=cfg["n_new"])
    tree = S.Tree(B, cfg["total_tokens"] + 1, dev)
    D = cfg["depth"]
    vout = (torch.empty(B, D + 1, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev),
            torch.empty(B, D, dtype=torch.int32, device=dev))
    # target logits planted on this run's own tree (one untimed draft pass)
    S.spec_build_tree(ctx, w, draft_kv, aux, in_tok, ctx_len, tree=tree)
    torch.cuda.synchronize()
    tnp = tree.numpy()
    if cfg["target_logits"] == "planted":
        tl, tl_kind = gen.plant_target_logits(cfg, tnp, seed), "planted"
    elif tl_oracle is not None:  # the oracle's draft logits of every node + N(0, 1), as the oracle leg
        tl, tl_kind = tl_oracle, "oracle_draft_logits_plus_noise"
    else:  # oracle leg skipped: random logits of the draft's scale + N(0, 1)
        base = gen.random_logits(seed, "bench_draft_like", (B, cfg["total_tokens"] + 1, cfg["vocab"]), std=1.28)
        tl, tl_kind = gen.add_noise_logits(base, seed), "random_plus_noise"
    target_logits = torch.from_numpy(tl).to(dev)
    mode = 0 if cfg["verify"] == "greedy" else 1
    accept_u = torch.from_numpy(gen.make_accept_u(cfg, seed)).to(dev) if mode else None
    pseed = gen.philox_seed(seed)

    def step():
        S.spec_build_tree(ctx, w, draft_kv, aux, in_tok, ctx_len, tree=tree)
        S.spec_verify_tree(ctx, tree, target_logits, mode, cfg["temperature"], accept_u, pseed, out=vout)
        S.spec_compact_kv(ctx, target_kv, tree_base, vout[2], vout[1])

    stream = torch.cuda.current_stream()
    graph = None
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    run = graph.replay if graph is not None else step

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    if graph is None:  # the kernel timing of every PROF_EVERY-th timed step
        ctx.profile(True)
        ctx.profile(False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        sample = graph is None and i % PROF_EVERY == 0
        if sample:
            ctx.profile(True, reset=False)
        run()
        if sample:
            ctx.profile(False)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    roof = None
    if graph is None:
        n, ms = ctx.profile_read(L.SPEC_PROF_LM_HEAD)
        nt, mst = ctx.profile_read(L.SPEC_PROF_LM_HEAD_TILED)
        na, msa = ctx.profile_read(L.SPEC_PROF_ATTENTION)
        nv, msv = ctx.profile_read(L.SPEC_PROF_VERIFY)
        ctx.profile(False)
        rows = pass_rows(cfg)
        kern = kernel_figures(cfg, rows, (n, ms), (nt, mst), (na, msa), (nv, msv),
                              vout[1].cpu().numpy())
        # the roofline kernel: the LM head launch that takes the most time per
        # step (the tiled beam-pass head of tree workloads beyond 64 rows)
        tiled = "lm_head_tiled" in kern and nt * mst >= n * ms
        if tiled:
            big = [m for m in rows if m > 64]
            byts = sum(lm_head_bytes(cfg, m) for m in big) / len(big)
            nl, avg_ms = nt, mst / max(nt, 1)
            kname = "tiled beam-pass LM head (gemm_dma_kernel<128,256,64,512,3,REC,PERSIST>)"
        else:
            small = [m for m in rows if m <= 64] or rows
            byts = sum(lm_head_bytes(cfg, m) for m in small) / len(small)
            nl, avg_ms = n, ms / max(n, 1)
            kname = ("LM head (gemm_lmhead_topk_kernel / gemm_bf16_stream<*,1,*>)" if cfg["dtype"] == "bf16"
                     else "gemm_f32_rows")
        achieved = byts / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if args.n_new else measured_traffic(args.config, "lm_head_tiled" if tiled else "lm_head"),
                "kernel": kname, "avg_launch_us": round(avg_ms * 1e3, 2), "launches": nl,
                "timed_every_nth_step": PROF_EVERY, "algorithmic_bytes_per_launch": int(byts)}
        if tiled:
            e = kern["lm_head_tiled"]
            M = rows[-1]
            roof.update(mfma_tflops=e["mfma_tflops"], mfma_frac=e["mfma_frac"],
                        arithmetic_intensity=round(e["flops_per_launch"] / byts, 1),
                        attainable_mfma_frac=round(min(1.0, HBM_PEAK_GBS * 1e9 * e["flops_per_launch"] / byts
                                                       / (BF16_PEAK_TFLOPS * 1e12)), 4),
                        rows=M)
        print(f"[bench] lm_head {n} launches avg {ms / max(n, 1) * 1e3:.1f} us; tiled lm_head {nt} launches avg "
              f"{mst / max(nt, 1) * 1e3:.1f} us; attention avg {msa / max(na, 1) * 1e3:.1f} us; verify avg "
              f"{msv / max(nv, 1) * 1e3:.1f} us", file=sys.stderr, flush=True)
    res = {
        "metric": METRIC,
        "value": round(1000.0 / ms_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.config, "batch": B, "ctx": cfg["ctx"], "top_k": cfg["top_k"],
                   "depth": cfg["depth"], "total_tokens": cfg["total_tokens"], "verify": cfg["verify"],
                   "n_new": cfg["n_new"], "graph": bool(graph is not None), "paged_block": args.paged or None,
                   "wall_s": round(wall, 3)},
        "roofline": roof,
    }
    # acceptance of the last timed step on the synthetic target logits: mean
    # accepted drafts per sequence and mean emitted tokens (accepted + the
    # correction or bonus token)
    alen = vout[1].cpu().numpy()
    res["acceptance"] = {"mean_accepted": round(float(alen.mean()), 4),
                         "mean_emitted": round(float(alen.mean()) + 1.0, 4), "sequences": int(B),
                         "target_logits": tl_kind}
    if cfg["cand_rank"]:
        res["candidate_recall"] = candidate_recall(cfg, ctx, w, draft_kv, aux, inp)
    if roof is not None:
        res["kernels"] = kern
        if not args.no_peaks:
            from speculative_decoding_aux_amd import peaks as PK

            print("[bench] measuring attainable peaks (read/copy stream, MFMA loop)", file=sys.stderr, flush=True)
            pk = PK.measure()
            res["peaks_measured"] = pk
            roof["measured_peak"] = pk["hbm_read_gbs"]
            roof["frac_of_measured"] = round(roof["achieved"] / pk["hbm_read_gbs"], 4)
            for v in kern.values():
                if "achieved_gbs" in v:
                    v["frac_of_measured"] = round(v["achieved_gbs"] / pk["hbm_read_gbs"], 4)
                if "mfma_tflops" in v:
                    v["mfma_frac_of_measured"] = round(v["mfma_tflops"] / pk["mfma_bf16_tflops"], 4)
    if cpu_res is not None:
        res["cpu_baseline"] = cpu_res
    print(json.dumps(res), flush=True)


def paged_copy(kv, bs, seed):
    """The same caches as a pool of bs-slot blocks in a shuffled order (plus
    spare blocks) with a block table: [layers, blocks, n_kv, bs, hd]."""
    import torch

    from speculative_decoding_aux_amd import spec as S

    Lr, B, nkv, Sl, hd = kv.k.shape
    mb = -(-Sl // bs)
    nb = B * mb + 8
    g = torch.Generator().manual_seed(seed)
    table = torch.randperm(nb, generator=g)[: B * mb].reshape(B, mb).to(torch.int32)
    pools = []
    for a in (kv.k, kv.v):
        pad = torch.zeros(Lr, B, nkv, mb * bs, hd, dtype=a.dtype, device=a.device)
        pad[:, :, :, :Sl] = a
        pool = torch.zeros(Lr, nb, nkv, bs, hd, dtype=a.dtype, device=a.device)
        blocks = pad.reshape(Lr, B, nkv, mb, bs, hd).permute(0, 1, 3, 2, 4, 5).reshape(Lr, B * mb, nkv, bs, hd)
        pool[:, table.reshape(-1).long().to(a.device)] = blocks
        pools.append(pool.contiguous())
    return S.PagedKVCache(pools[0], pools[1], table.to(kv.k.device).contiguous())


def candidate_recall(cfg, ctx4, w, draft_kv, aux, inp):
    """EAGLE-4 candidate recall on the root pass: the share of the full LM
    head's top-k (an EAGLE-3 head over the same lm_head, the same rows and
    inputs) that the low-rank head's retrieved candidates contain; at 1 and
    at top_k, averaged over the sequences.  Both passes run in the library;
    they write the root rows' K/V into a copy of the draft cache."""
    import torch

    from speculative_decoding_aux_amd import spec as S

    B, k = cfg["batch"], cfg["top_k"]
    cfg3 = dict(cfg, cand_rank=0, num_candidates=0)
    ctx3 = S.SpecContext(cfg3, max_batch=B, max_new=cfg["n_new"])
    kv = S.KVCache(draft_kv.k.clone(), draft_kv.v.clone())
    pos = inp["ctx_len"].astype(np.int32)
    toks = inp["in_tokens"][:, 0]
    anc = pos[:, None]
    g4 = S.spec_draft_step(ctx4, w, kv, B, 1, 0, aux[:, 0].contiguous(), toks, pos, pos, inp["ctx_len"], anc,
                           k, want_candidates=True)
    g3 = S.spec_draft_step(ctx3, w, kv, B, 1, 0, aux[:, 0].contiguous(), toks, pos, pos, inp["ctx_len"], anc,
                           k)
    torch.cuda.synchronize()
    full = g3["ids"].cpu().numpy()
    cands = g4["cand_ids"].cpu().numpy()
    at1 = np.mean([full[r, 0] in set(cands[r].tolist()) for r in range(B)])
    atk = np.mean([len(set(full[r].tolist()) & set(cands[r].tolist())) / k for r in range(B)])
    del kv
    ctx3.close()
    return {"at_1": round(float(at1), 4), f"at_{k}": round(float(atk), 4), "rows": int(B),
            "candidates": int(cfg["num_candidates"]), "note": "random synthetic factors: recall near K/V"}


def bench_flat_sampling(args):
    """Rejection sampling of one flat batch per call (spec_rejection_sample):
    B requests with 0..K drafts each over the workload's target vocabulary,
    mixed greedy / random requests with per-request temperature, top-k and
    top-p (synth.gen.flat_batch).  Algorithmic bytes: every logits row (each
    draft row and each bonus row) read once."""
    import torch

    from oracle import sampling as osm
    from speculative_decoding_aux_amd import spec as S
    from speculative_decoding_aux_amd import _lib as L
    from synth import configs, gen

    cfg0 = configs.get(args.config)
    B, K, V = args.flat_sampling, cfg0["total_tokens"], cfg0["vocab"]
    cfg = configs.get(args.config, batch=B)
    seed = configs.SEEDS[args.config] + 500
    d = gen.flat_batch(seed, B, K, V)
    nd = d["num_draft_tokens"]
    T = int(nd.sum())
    ctx = S.SpecContext(cfg, max_batch=B, max_new=cfg["n_new"])
    dev = "cuda"
    meta = S.spec_decode_metadata(ctx, d["cu_num_scheduled_tokens"], nd, T)
    cu, _, tgt, bonus = meta
    lg = torch.from_numpy(d["logits"]).to(dev)
    drafts = torch.from_numpy(d["draft_token_ids"]).to(dev)
    temp = torch.from_numpy(d["temperature"]).to(dev)
    tk = torch.from_numpy(d["top_k"]).to(dev)
    tp = torch.from_numpy(d["top_p"]).to(dev)
    u = torch.from_numpy(d["uniform"]).to(dev)
    out = (torch.empty(B, K + 1, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))

    def call():
        S.spec_rejection_sample(ctx, cu, drafts, lg, tgt, bonus, temp, tk, tp, u, d["seed"], K, out=out)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} flat-sampling calls (B={B}, rows={T + B}, V={V})",
          file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ctx.profile(True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    n, ms = ctx.profile_read(L.SPEC_PROF_VERIFY)
    ctx.profile(False)
    ms_call = e0.elapsed_time(e1) / args.steps
    avg_ms = ms / max(n, 1)
    byts = (T + B) * V * 4
    achieved = byts / (avg_ms * 1e-3) / 1e9
    res = {"metric": "flat-batch rejection sampling calls/sec at 1 GPU", "value": round(1000.0 / ms_call, 2),
           "unit": "calls/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms_call, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"flat_sampling_{args.config}", "requests": B, "max_spec_len": K,
                      "drafts": T, "logits_rows": T + B, "vocab": V,
                      "greedy_requests": int((d["temperature"] == 0).sum())},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "sample_row_kernel + sample_gumbel_kernel + sample_emit_kernel",
                        "avg_launch_us": round(avg_ms * 1e3, 2), "launches": n,
                        "algorithmic_bytes_per_launch": byts}}
    if not args.no_cpu_baseline:
        wall = []
        for _ in range(max(1, args.cpu_steps)):
            t0 = time.perf_counter()
            m = osm.spec_decode_metadata(d["cu_num_scheduled_tokens"], nd)
            osm.rejection_sample(m[0], d["draft_token_ids"], d["logits"], m[2], m[3], d["temperature"],
                                 d["top_k"], d["top_p"], d["uniform"], d["seed"], K)
            wall.append(time.perf_counter() - t0)
        med = float(np.median(wall))
        res["cpu_baseline"] = {"value": round(1.0 / med, 3), "unit": "calls/s", "cores": 1, "kind": "oracle",
                               "sample": f"{len(wall)} whole calls of the same batch; median {med:.3f} s"}
    print(json.dumps(res), flush=True)


def bench_target_forward(args):
    """spec_target_forward over the workload's tree shape (chain trees of K
    drafts for chain workloads, random trees otherwise) with L synthetic
    target layers of the workload's dimensions.  Algorithmic bytes per
    forward: every layer's weights and the final LM head once, the context
    K/V of every layer once per sequence, the logits written once."""
    import torch

    from speculative_decoding_aux_amd import spec as S
    from speculative_decoding_aux_amd import _lib as L
    from speculative_decoding_aux_amd.tensors import to_device, upload_target_weights
    from synth import configs, gen

    # the target has the workload's dimensions and its full vocabulary head
    cfg = configs.get(args.config, cand_rank=0, num_candidates=0, sliding_window=0)
    cfg["draft_vocab"] = cfg["vocab"]
    Lr, B, N, dt = args.target_forward, cfg["batch"], cfg["total_tokens"], cfg["dtype"]
    n1 = N + 1
    seed = configs.SEEDS[args.config] + 600
    H, I, V = cfg["hidden"], cfg["intermediate"], cfg["vocab"]
    nkv, hd = cfg["n_kv_heads"], cfg["head_dim"]
    print(f"[bench] generating a {Lr}-layer target for {args.config}", file=sys.stderr, flush=True)
    W = gen.make_target_weights(cfg, seed, Lr)
    ctx_len = np.full(B, cfg["ctx"], np.int64)
    slots = cfg["kv_capacity"]
    if cfg["top_k"] == 1:
        tree = gen.chain_tree(B, N, V, ctx_len, seed)
    else:
        tree = gen.with_positions(gen.random_tree(cfg, seed, batch=B), ctx_len)
    dev = "cuda"
    tw = upload_target_weights(cfg, W)
    del W
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    g = torch.Generator(device=dev).manual_seed(seed)
    shape = (Lr, B, nkv, slots, hd)
    kv = S.KVCache(torch.randn(shape, generator=g, device=dev).to(tdt),
                   torch.randn(shape, generator=g, device=dev).to(tdt))
    ctx = S.SpecContext(cfg, max_batch=B, max_new=n1)
    tr = S.Tree(B, n1, dev)
    for f in ("tokens", "parent", "depth", "position", "num_nodes"):
        getattr(tr, f).copy_(torch.from_numpy(np.ascontiguousarray(tree[f], dtype=np.int32)))
    tr.anc_mask.copy_(torch.from_numpy(np.ascontiguousarray(tree["anc_mask"]).view(np.int64)))
    cl = torch.from_numpy(ctx_len.astype(np.int32)).to(dev)
    for _ in range(args.warmup):
        S.spec_target_forward(ctx, tw, kv, tr, cl)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} target forwards ({Lr} layers, {B * n1} rows)", file=sys.stderr,
          flush=True)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ctx.profile(True)
    e0.record(stream)
    for _ in range(args.steps):
        S.spec_target_forward(ctx, tw, kv, tr, cl)
    e1.record(stream)
    torch.cuda.synchronize()
    nl, msl = ctx.profile_read(L.SPEC_PROF_LM_HEAD)
    na, msa = ctx.profile_read(L.SPEC_PROF_ATTENTION)
    ctx.profile(False)
    ms = e0.elapsed_time(e1) / args.steps
    es = 2 if dt == "bf16" else 4
    qkvN = (cfg["n_q_heads"] + 2 * nkv) * hd
    layer_w = (qkvN * H + H * cfg["n_q_heads"] * hd + 2 * I * H + H * I) * es
    kv_bytes = Lr * B * nkv * cfg["ctx"] * hd * es * 2
    byts = Lr * layer_w + V * H * es + kv_bytes + B * n1 * V * 4
    achieved = byts / (ms * 1e-3) / 1e9
    M = B * n1
    flops = 2.0 * M * (Lr * (qkvN * H + H * cfg["n_q_heads"] * hd + 2 * I * H + H * I) + V * H)
    res = {"metric": "target verification forwards/sec at 1 GPU", "value": round(1000.0 / ms, 2),
           "unit": "forwards/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": dt, "data": "synthetic",
           "config": {"workload": f"target_forward_{args.config}", "layers": Lr, "batch": B, "tree_rows": M,
                      "ctx": cfg["ctx"]},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "whole forward (weights, context K/V, logits)",
                        "algorithmic_bytes_per_launch": int(byts),
                        "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
           "kernels": {"lm_head": {"avg_launch_us": round(msl / max(nl, 1) * 1e3, 2), "launches": nl},
                       "attention": {"avg_launch_us": round(msa / max(na, 1) * 1e3, 2), "launches": na}}}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
