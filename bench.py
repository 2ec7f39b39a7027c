"""Benchmark of the streaming pyramid's hot path on one MI355X.

One step is one pyramid round at 512x512 on the device: the 16 reference-bank
spatial self-attention layers of the SD1.5 denoiser (16 frames, 8 heads,
frame tokens + reference + m anchors as keys, fp16), the fused per-window DDIM
step over the 16x4x64x64 fp32 latents pile with the leaving window's x0, and
the 512-d motion-bank min-L2 check.  Inputs are seeded synthetic tensors
already resident in HBM; every launch goes through the C ABI (libpl.so).

Prints ONE JSON line on stdout.  Everything else goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --layer d00 [--steps K] [--warmup W]    (one attention layer alone)

The ``cpu_baseline`` leg times the fp64 CPU oracle on a bounded sample of the
same workload (a few (frame, head) pairs of the first 64^2 layer); it is a
reported baseline, not the target.
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Published MI355X figures: fp16 dense MFMA 2.5 PFLOP/s, HBM3E 8 TB/s.
PEAK_FP16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
FRAMES_OUT_PER_ROUND = 4      # one window of 4 frames leaves per round
SEED = 4                      # seed of the full-round workload


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--m", type=int, default=None, help="anchors per round (default: one seeded draw)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the DDIM bandwidth sweep")
    ap.add_argument("--copy-calib", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--layer", default=None,
                    help="profiling mode: launch only this attention layer (d00, d10, m, ...) "
                         "--warmup + --steps times and print its timing as the JSON line")
    return ap.parse_args()


def attention_flops(F, L, C, lk):
    """Algorithmic FLOPs of one layer: QK^T and PV, 2 flops per MAC each."""
    return 4 * F * L * lk * C


def attention_bytes(F, L, C, m):
    """Compulsory HBM bytes of one layer: Q, K_self, V_self, O plus the shared bank, fp16."""
    return (4 * F * L * C + 2 * (1 + m) * L * C) * 2


def traffic_record(kernel_key):
    """Measured HBM bytes per launch for a kernel, from the committed counter summary.

    The summary names the kernel source hash it was taken on; when the
    source has changed since, the figure no longer applies and None is
    returned.
    """
    path = os.path.join(ROOT, "profiles", "refbank_attn_full_round_m3_hbm_traffic.md")
    src = os.path.join(ROOT, "streaming_diffusion_portrait_amd", "csrc", "attn.hip")
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    with open(src, "rb") as fh:
        h = hashlib.sha256(fh.read()).hexdigest()[:16]
    for line in open(path, encoding="utf-8"):
        # | key | source sha256[:16] | bytes per launch | ...
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 3 and cells[0] == kernel_key and cells[1] == h:
            try:
                return float(cells[2])
            except ValueError:
                return None
    return None


def one_layer(args, B, todev, m, F, H):
    """Launch one attention layer of the round alone (for counter and trace runs)."""
    import torch

    names = [n for n, _, _ in inputs_layers()]
    if args.layer not in names:
        log(f"unknown layer {args.layer}; one of {' '.join(names)}")
        sys.exit(2)
    from streaming_diffusion_portrait_amd import inputs
    li = names.index(args.layer)
    _, L, C = inputs.SD15_LAYERS[li]
    lay = inputs.attention_layer(1000 * SEED + li, F, L, C, m)
    q = todev(lay["q"])
    segs = [(todev(lay["k_self"]), todev(lay["v_self"]))]
    segs += [(todev(k), todev(v)) for k, v in zip(lay["bank_k"], lay["bank_v"])]
    out = torch.empty_like(q)
    call = B.PreparedAttn(q, segs, H, out)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / max(args.steps, 1) * 1e3
    fl = attention_flops(F, L, C, L * (2 + m))
    tf = fl / (us * 1e-6) / 1e12
    print(json.dumps({"layer": args.layer, "L": L, "C": C, "d": C // H, "m": m, "launches": args.steps,
                      "us_per_launch": round(us, 2), "tflops": round(tf, 1),
                      "pct_fp16_peak": round(100 * tf / PEAK_FP16_TFLOPS, 2)}), flush=True)


def build_round(B, inputs, todev, m, F, H, dev, keep_host=True):
    """One round's device state at anchor count m: fresh seeded tensors for the
    16 attention layers (prepared calls), the 16x4x64x64 pile, the motion bank."""
    import torch

    layers = []
    for li, (name, L, C) in enumerate(inputs.SD15_LAYERS):
        lay = inputs.attention_layer(1000 * SEED + li, F, L, C, m)
        q = todev(lay["q"])
        segs = [(todev(lay["k_self"]), todev(lay["v_self"]))]
        segs += [(todev(k), todev(v)) for k, v in zip(lay["bank_k"], lay["bank_v"])]
        out = torch.empty_like(q)
        lk = L * (2 + m)
        layers.append(dict(name=name, L=L, C=C, d=C // H, lk=lk, q=q, segs=segs, out=out,
                           call=B.PreparedAttn(q, segs, H, out), host=lay if (li == 0 and keep_host) else None,
                           flops=attention_flops(F, L, C, lk), bytes=attention_bytes(F, L, C, m)))
    x_t_np, eps_np = inputs.ddim_pile(SEED, (16, 4, 64, 64))
    R = dict(layers=layers, m=m, x_t=todev(x_t_np), eps=todev(eps_np))
    R["x_prev"] = torch.empty_like(R["x_t"])
    R["x0"] = torch.empty((4, 4, 64, 64), dtype=torch.float32, device=dev)
    bank_np, q_np, _ = inputs.motion_bank(SEED, 1 + m, 512, nq=1)
    R["mb"], R["mq"] = todev(bank_np), todev(q_np)
    R["md"] = (torch.empty(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.int32, device=dev),
               torch.empty(1, dtype=torch.uint8, device=dev))
    R["pile"] = B.Pile(4, 333)
    R["next_window"] = 4  # ids 0..2 prefilled, 3 enters with the first round
    return R


def eager_round(B, R, events=None):
    """The round as separate library calls from the host: the 16 attention layers,
    the rolling DDIM step (which also draws the next window's noise into the
    leaving window's slot) with the host pile state machine, the drift check."""
    for li, lay in enumerate(R["layers"]):
        if events is not None:
            events[li][0].record()
        lay["call"]()
        if events is not None:
            events[li][1].record()
    _, t_slot, emit = R["pile"].begin_round()
    B.pyramid_ddim_step(R["x_t"], R["eps"], t_slot, x_prev=R["x_prev"], x0_out=R["x0"], emit_window=emit,
                        roll=(SEED, R["next_window"]))
    R["next_window"] += 1
    R["pile"].end_round()
    B.motion_bank_min_l2(R["mq"], R["mb"], 17.0, out=R["md"])


def time_eager_rounds(R, warmup, K):
    """K eager rounds bracketed by synchronisations, HIP events around every
    attention launch.  Returns (ms per round, per-layer ms)."""
    import numpy as np
    import torch

    from streaming_diffusion_portrait_amd import binding as B
    for _ in range(warmup):
        eager_round(B, R)
    torch.cuda.synchronize()
    nl = len(R["layers"])
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(nl)]
           for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(K):
        eager_round(B, R, evs[k])
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t_start) / K
    per_layer = [float(np.mean([evs[k][li][0].elapsed_time(evs[k][li][1]) for k in range(K)])) for li in range(nl)]
    return ms, per_layer


def time_graph_rounds(B, R, warmup, K):
    """The round with its pile state on the device, captured once as a graph and
    replayed K times (one host call per round).  Also returns the host time to
    issue one round: the graph replay against the eager sequence of calls."""
    import torch

    dpile = B.DevicePile(4, 333)
    xg = R["x_t"].clone()  # the graph's own pile, rolled in place
    x0g = torch.empty_like(R["x0"])

    def dev_round(stream):
        for lay in R["layers"]:
            lay["call"](stream)
        dpile.step(xg, R["eps"], xg, x0g, SEED, stream=stream)
        B.motion_bank_min_l2(R["mq"], R["mb"], 17.0, out=R["md"], stream=stream)

    dev_round(torch.cuda.current_stream())  # every kernel has run once before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        dev_round(torch.cuda.current_stream())
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(K):
        g.replay()
    host_graph = (time.perf_counter() - t_start) / K
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t_start) / K
    # host cost of issuing the eager round (its launches queue behind each other)
    n = 5
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(n):
        eager_round(B, R)
    host_eager = (time.perf_counter() - t_start) / n
    torch.cuda.synchronize()
    del g
    return dict(ms_per_step=ms, host_us_graph=1e6 * host_graph, host_us_eager=1e6 * host_eager,
                launches_per_round=len(R["layers"]) + 3)


def inputs_layers():
    from streaming_diffusion_portrait_amd import inputs
    return inputs.SD15_LAYERS


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("this benchmark runs on exactly one GPU: the streaming round's work is one GPU's share "
            "(frame sharding across GPUs is a design note only); run with --gpus 1")
        sys.exit(2)

    import numpy as np
    import torch

    from streaming_diffusion_portrait_amd import binding as B, inputs

    if not torch.cuda.is_available():
        log("no GPU visible: bench.py needs an MI355X")
        sys.exit(1)
    B.load()  # raises if libpl.so is missing: there is no other path
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs {props.multi_processor_count}")

    m = inputs.round_m(SEED) if args.m is None else int(args.m)
    F, H = 16, 8
    todev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    if args.layer is not None:
        one_layer(args, B, todev, m, F, H)
        return

    # ---- the round at the seeded m: inputs, eager timed region, captured graph ---------------
    t0 = time.perf_counter()
    R = build_round(B, inputs, todev, m, F, H, dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f}s (m={m})")
    K = args.steps
    ms_per_step, per_layer_ms = time_eager_rounds(R, args.warmup, K)
    graph = time_graph_rounds(B, R, args.warmup, K)
    layers = R["layers"]
    round_flops = sum(l["flops"] for l in layers)
    attn_ms = sum(per_layer_ms)
    tflops_round = round_flops / (ms_per_step * 1e-3) / 1e12
    frames_per_s = FRAMES_OUT_PER_ROUND / (ms_per_step * 1e-3)
    log(f"  round m={m}: eager {ms_per_step:.3f} ms, graph {graph['ms_per_step']:.3f} ms; host issue per round: "
        f"eager {graph['host_us_eager']:.0f} us, graph {graph['host_us_graph']:.0f} us")

    # dominant kernel: the d=40 (64^2 level) attention launches, 87% of the round's FLOPs at m=0
    dom = [li for li, l in enumerate(layers) if l["d"] == 40]
    dom_ms = float(np.mean([per_layer_ms[li] for li in dom]))
    dom_flops = layers[dom[0]]["flops"]
    dom_tflops = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic = traffic_record(f"attn_d40_L4096_m{m}")

    layer_report = [dict(layer=l["name"], L=l["L"], C=l["C"], d=l["d"], keys=l["lk"],
                         us=round(1e3 * per_layer_ms[li], 2),
                         tflops=round(l["flops"] / (per_layer_ms[li] * 1e-3) / 1e12, 1),
                         pct_fp16_peak=round(100 * l["flops"] / (per_layer_ms[li] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 1))
                    for li, l in enumerate(layers)]
    for r in layer_report:
        log(f"  {r['layer']:>4} L={r['L']:5d} d={r['d']:3d} keys={r['keys']:5d}  {r['us']:9.2f} us  "
            f"{r['tflops']:7.1f} TFLOP/s  {r['pct_fp16_peak']:5.1f}%")
    x_t, eps, x_prev, x0 = R["x_t"], R["eps"], R["x_prev"], R["x0"]
    mb, mq, md = R["mb"], R["mq"], R["md"]
    n_bank = 1 + m

    # ---- the round at every anchor count m = 0..3 (fresh seeded tensors per m) ----------------
    sweep_m = []
    for mm in range(4):
        if mm == m:
            sm = dict(ms=ms_per_step, per_layer=per_layer_ms, graph_ms=graph["ms_per_step"], flops=round_flops)
        else:
            Rm = build_round(B, inputs, todev, mm, F, H, dev, keep_host=False)
            mms, mpl = time_eager_rounds(Rm, args.warmup, K)
            gm = time_graph_rounds(B, Rm, args.warmup, K)
            sm = dict(ms=mms, per_layer=mpl, graph_ms=gm["ms_per_step"], flops=sum(l["flops"] for l in Rm["layers"]))
            del Rm, gm
            torch.cuda.synchronize()
        d40 = float(np.mean([sm["per_layer"][li] for li in dom]))
        rec = dict(m=mm, keys_64x64=4096 * (2 + mm), round_attn_tflop=round(sm["flops"] / 1e12, 4),
                   ms_per_round=round(sm["ms"], 4), graph_ms_per_round=round(sm["graph_ms"], 4),
                   tflops=round(sm["flops"] / (sm["ms"] * 1e-3) / 1e12, 1),
                   pct_fp16_peak=round(100 * sm["flops"] / (sm["ms"] * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 2),
                   frames_per_s=round(FRAMES_OUT_PER_ROUND / (sm["ms"] * 1e-3), 1),
                   d40_us_per_launch=round(1e3 * d40, 1),
                   d40_pct_fp16_peak=round(100 * (4 * 16 * 4096 * 4096 * (2 + mm) * 320) / (d40 * 1e-3) / 1e12
                                           / PEAK_FP16_TFLOPS, 2))
        sweep_m.append(rec)
        log(f"  m={mm}: round {rec['ms_per_round']:.3f} ms (graph {rec['graph_ms_per_round']:.3f}), "
            f"{rec['tflops']:.0f} TFLOP/s = {rec['pct_fp16_peak']:.1f}%, {rec['frames_per_s']:.0f} frames/s, "
            f"d=40 {rec['d40_us_per_launch']:.0f} us ({rec['d40_pct_fp16_peak']:.1f}%)")

    # ---- DDIM and motion at the round's shapes (separately timed, same kernels) ---------------
    def time_it(fn, n=200):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3  # us per call (includes launch gaps)

    t_slot = [0, 333, 666, 999]
    ddim_us = time_it(lambda: B.pyramid_ddim_step(x_t, eps, t_slot, x_prev=x_prev, x0_out=x0, emit_window=0))
    roll_us = time_it(lambda: B.pyramid_ddim_step(x_t, eps, t_slot, x_prev=x_prev, x0_out=x0, emit_window=0,
                                                  roll=(SEED, 9)))
    # expression cross-attention (32 tokens per frame, same boundary call, short-context
    # kernel) at each level: HBM-bound, so bytes = Q + O + K/V
    short_ctx = []
    for L, C in ((4096, 320), (1024, 640), (256, 1280), (64, 1280)):
        g = torch.Generator(device=dev).manual_seed(L)
        sq = torch.randn(F, L, C, device=dev, generator=g).half()
        sk = torch.randn(F, 32, C, device=dev, generator=g).half()
        sv = torch.randn(F, 32, C, device=dev, generator=g).half()
        so = torch.empty_like(sq)
        scall = B.PreparedAttn(sq, [(sk, sv)], H, so)
        s_us = time_it(scall, n=50)
        s_bytes = (2 * F * L * C + 2 * F * 32 * C) * 2
        short_ctx.append(dict(L=L, C=C, keys=32, us=round(s_us, 2), bytes=s_bytes,
                              GBps=round(s_bytes / (s_us * 1e-6) / 1e9, 1),
                              frac_hbm_peak=round(s_bytes / (s_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)))
        del sq, sk, sv, so, scall
    log("  expression cross-attention (32 keys/frame): " +
        ", ".join(f"L={r['L']} {r['us']:.1f} us {r['GBps']:.0f} GB/s" for r in short_ctx))
    # the key-axis split: one frame of the 16^2 and 8^2 levels against the 4x bank (the
    # round's own launches fill the CUs and do not split), split and single pass
    key_split = []
    for L in (256, 64):
        g = torch.Generator(device=dev).manual_seed(11 * L)
        kq = torch.randn(1, L, 1280, device=dev, generator=g).half()
        ksegs = [(torch.randn(1, L, 1280, device=dev, generator=g).half(),
                  torch.randn(1, L, 1280, device=dev, generator=g).half())]
        ksegs += [(torch.randn(L, 1280, device=dev, generator=g).half(),
                   torch.randn(L, 1280, device=dev, generator=g).half()) for _ in range(4)]
        ko = torch.empty_like(kq)
        rec = dict(L=L, C=1280, frames=1, keys=5 * L)
        for mode, ws in (("split", None), ("single_pass", False)):
            kcall = B.PreparedAttn(kq, ksegs, H, ko, workspace=ws)
            rec[f"{mode}_us"] = round(time_it(kcall, n=100), 2)
            if mode == "split":
                rec["workspace_bytes"] = kcall.workspace_bytes
            del kcall
        key_split.append(rec)
        del kq, ksegs, ko
    log("  key split (one frame, 4x bank): " +
        ", ".join(f"L={r['L']} split {r['split_us']:.1f} us / single {r['single_pass_us']:.1f} us" for r in key_split))
    # block-causal attention over chunked sequences (pl_refbank_attn_chunked): the 64^2
    # level's 4096 tokens per frame as 4 chunks of 1024, each row seeing its own chunk,
    # the earlier ones (all, or only the previous one) and the reference; FLOPs count
    # only the keys a row sees
    chunked = []
    g = torch.Generator(device=dev).manual_seed(4096 + 17)
    cq = torch.randn(F, 4096, 320, device=dev, generator=g).half()
    ck = torch.randn(F, 4096, 320, device=dev, generator=g).half()
    cv = torch.randn(F, 4096, 320, device=dev, generator=g).half()
    cbk = torch.randn(4096, 320, device=dev, generator=g).half()
    cbv = torch.randn(4096, 320, device=dev, generator=g).half()
    co = torch.empty_like(cq)
    for hist in (-1, 1):
        nch, cl = 4, 1024
        keys = [cl * (c + 1 - (max(0, c - hist) if hist >= 0 else 0)) + 4096 for c in range(nch)]
        c_flops = sum(4 * F * cl * k * 320 for k in keys)
        c_us = time_it(lambda: B.chunked_attn(cq, (ck, cv), [(cbk, cbv)], H, cl, hist, out=co), n=20)
        chunked.append(dict(L=4096, C=320, chunk_len=cl, chunks=nch, max_history=hist, bank=4096, launches=nch,
                            us=round(c_us, 2), tflops=round(c_flops / (c_us * 1e-6) / 1e12, 1),
                            pct_fp16_peak=round(100 * c_flops / (c_us * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 2)))
    del cq, ck, cv, cbk, cbv, co
    log("  block-causal chunks (64^2, 4 x 1024 + reference): " +
        ", ".join(f"history {r['max_history']}: {r['us']:.0f} us {r['tflops']:.0f} TFLOP/s" for r in chunked))
    # the projections either side of the attention: fused q/k/v ([3C, C]) and the
    # output projection ([C, C] + bias) over the 16 frames of each level
    projections = []
    for L, C in ((4096, 320), (1024, 640), (256, 1280), (64, 1280)):
        g = torch.Generator(device=dev).manual_seed(7 * L)
        px = torch.randn(F * L, C, device=dev, generator=g).half()
        for pname, N, with_bias in (("qkv", 3 * C, False), ("out", C, True)):
            pw = (torch.randn(N, C, device=dev, generator=g) / C ** 0.5).half()
            pb = torch.randn(N, device=dev, generator=g) if with_bias else None
            py = torch.empty(F * L, N, device=dev, dtype=torch.float16)
            p_us = time_it(lambda: B.linear(px, pw, pb, out=py), n=50)
            p_fl = 2 * F * L * N * C
            p_by = (F * L * C + N * C + F * L * N) * 2
            projections.append(dict(name=pname, L=L, C=C, N=N, us=round(p_us, 2),
                                    tflops=round(p_fl / (p_us * 1e-6) / 1e12, 1),
                                    GBps=round(p_by / (p_us * 1e-6) / 1e9, 1),
                                    frac_hbm_peak=round(p_by / (p_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)))
            del pw, py
        del px
    log("  projections: " + ", ".join(f"{r['name']} L={r['L']} {r['us']:.1f} us" for r in projections))
    prefill_ref = torch.randn(4 * 4 * 64 * 64, device=dev)
    prefill_out = torch.empty((3, prefill_ref.numel()), device=dev)
    prefill_us = time_it(lambda: B.pile_prefill(prefill_ref, 3, SEED, out=prefill_out))
    motion_us = time_it(lambda: B.motion_bank_min_l2(mq, mb, 17.0, out=md))

    # ---- DDIM bandwidth sweep: rotating working sets well beyond the 256 MB cache ------------
    sweep = None
    if not args.no_sweep:
        per_window = 16 * 1024 * 1024  # elements; 4 windows -> 256 MiB per tensor
        sets = []
        for s in range(2):
            a = torch.randn(4 * per_window, device=dev)
            e = torch.randn(4 * per_window, device=dev)
            sets.append((a, e, torch.empty_like(a), torch.empty(per_window, device=dev)))
        sweep_bytes = 4 * per_window * 12 + per_window * 4
        ts = [999, 666, 333, 0]
        for s in sets:
            B.pyramid_ddim_step(s[0], s[1], ts, x_prev=s[2], x0_out=s[3], emit_window=3)
        torch.cuda.synchronize()
        reps = 20
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for r in range(reps):
            s = sets[r % 2]
            B.pyramid_ddim_step(s[0], s[1], ts, x_prev=s[2], x0_out=s[3], emit_window=3)
        b.record()
        torch.cuda.synchronize()
        sw_us = a.elapsed_time(b) / reps * 1e3
        gbs = sweep_bytes / (sw_us * 1e-6) / 1e9
        sweep = dict(bytes_per_call=sweep_bytes, working_set_bytes=2 * (4 * per_window * 12 + per_window * 4),
                     us=round(sw_us, 1), GBps=round(gbs, 1), frac_hbm_peak=round(gbs / PEAK_HBM_GBS, 3))
        del sets
        log(f"  DDIM sweep: {sweep_bytes / 2**20:.0f} MiB per call, {sw_us:.1f} us, {gbs:.0f} GB/s "
            f"({100 * gbs / PEAK_HBM_GBS:.1f}% of 8 TB/s)")

    if args.copy_calib:
        # a plain elementwise copy kernel over exactly 1 GiB (reads 1 GiB, writes 1 GiB):
        # the yardstick that scales the FETCH_SIZE / WRITE_SIZE counters into bytes
        src = torch.empty(2**28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- CPU baseline: the oracle on a bounded sample -------------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers[0], F, H, m)

    dom_l = layers[dom[0]]
    result = {
        "metric": "ref-bank attn TFLOP/s (% fp16 MFMA peak) + pyramid-step frames/s on 1 MI355X",
        "value": round(tflops_round, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (f"full pyramid round at 512x512: 16 SD1.5 reference-bank attention layers "
                         f"(16 frames, 8 heads, keys = own tokens + reference + {m} anchors), fused DDIM on "
                         f"a 16x4x64x64 fp32 pile at t=999/666/333/0, motion-bank min-L2 512-d vs {n_bank} entries"),
            "frames": F, "windows": 4, "heads": H, "m": m, "layers": len(layers), "resolution": 512,
        },
        "pct_fp16_peak": round(100 * tflops_round / PEAK_FP16_TFLOPS, 2),
        "frames_per_s": round(frames_per_s, 1),
        "attn_ms_per_round": round(attn_ms, 4),
        "round_attn_tflop": round(round_flops / 1e12, 4),
        "roofline": {
            "bound": "mfma",
            "kernel": f"refbank_attn d=40 (64^2 level: F=16, L=4096, C=320, keys={dom_l['lk']})",
            "achieved": round(dom_tflops, 2),
            "peak": PEAK_FP16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dom_tflops / PEAK_FP16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": dom_flops,
            "algorithmic_bytes_per_launch": dom_l["bytes"],
            "avg_launch_us": round(1e3 * dom_ms, 2),
        },
        "graph": {"ms_per_step": round(graph["ms_per_step"], 4),
                  "frames_per_s": round(FRAMES_OUT_PER_ROUND / (graph["ms_per_step"] * 1e-3), 1),
                  "host_us_per_round_graph": round(graph["host_us_graph"], 1),
                  "host_us_per_round_eager": round(graph["host_us_eager"], 1),
                  "launches_per_round": graph["launches_per_round"],
                  "note": "the same round with the pile state on the device, captured once and replayed: "
                          "one host call per round"},
        "m_sweep": sweep_m,
        "ddim": {"us_at_round_shape": round(ddim_us, 2), "bytes_at_round_shape": 3407872,
                 "us_with_roll_at_round_shape": round(roll_us, 2), "sweep": sweep},
        "pile_prefill_us": round(prefill_us, 2),
        "expression_cross_attention": short_ctx,
        "key_split_one_frame": key_split,
        "block_causal_chunks": chunked,
        "projections": projections,
        "motion_us": round(motion_us, 2),
        "layers": layer_report,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(lay0, F, H, m):
    """Time the fp64 oracle on a sample of the first 64^2 layer and compare it with the GPU output.

    A thread pool runs (frame, head) pairs side by side with one BLAS thread per
    worker; workers = the host cores this process may use, capped by
    OMP_NUM_THREADS (the CPU share a GPU job is given).  One pair is timed first
    to size the sample (about 4 s per pass), then the same pairs run three
    times; the median pass is reported.
    """
    import concurrent.futures

    import numpy as np

    import oracle

    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity))))
    host = lay0["host"]
    segs = [(host["k_self"], host["v_self"], False)]
    segs += [(k, v, True) for k, v in zip(host["bank_k"], host["bank_v"])]
    got = lay0["out"].cpu().numpy()
    L, C = lay0["L"], lay0["C"]
    d = C // H
    lk = lay0["lk"]
    chunk = 1024  # query rows per oracle call: bounds each worker's score matrix to 1024 x keys fp64

    def one_pair(idx):
        f, h = divmod(int(idx), H)
        err = 0.0
        for r0 in range(0, L, chunk):
            rows = np.arange(r0, min(L, r0 + chunk))
            ref = oracle.refbank_attention(host["q"], segs, H, frames=[f], head_list=[h], rows=rows)[(f, h)]
            err = max(err, float(np.abs(got[f][rows, h * d:(h + 1) * d].astype(np.float64) - ref).max()))
        return err

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl ships with the image
        threadpool_limits = None
    order = np.random.default_rng(0).permutation(F * H)
    passes, err_max = [], 0.0
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx is not None:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        err_max = one_pair(order[0])
        t_pair = time.perf_counter() - t0
        n_pairs = int(min(F * H, max(workers, round(workers * 4.0 / max(t_pair, 1e-3)))))
        sample = order[:n_pairs]
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            for _ in range(3):
                t0 = time.perf_counter()
                errs = list(ex.map(one_pair, sample))
                passes.append(time.perf_counter() - t0)
                err_max = max([err_max] + errs)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    sec = float(np.median(passes))
    flops = 4 * L * lk * d * n_pairs
    log(f"  cpu oracle: {n_pairs} (frame, head) pairs per pass on {workers} workers (1 BLAS thread each, "
        f"{affinity} cores in the affinity mask), passes {', '.join(f'{p:.1f}' for p in passes)} s, "
        f"max|gpu - oracle| {err_max:.2e}")
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "sample": (f"{n_pairs} of {F * H} (frame, head) pairs of the first 64^2 layer (L={L}, d={d}, "
                       f"keys={lk}), fp64 NumPy oracle in a {workers}-thread pool with one BLAS thread each, "
                       f"median of 3 passes ({', '.join(f'{p:.1f}' for p in passes)} s)"),
            "seconds": round(sec, 2), "affinity_cores": affinity, "max_abs_err_gpu_vs_oracle": err_max}


if __name__ == "__main__":
    main()
