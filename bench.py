"""Benchmark of the GIFT FP8 gradient round trip on one MI355X.

Workload: one Llama-style block at hidden 1024 -- q, k, v, o (1024 x 1024),
gate and up (2816 x 1024), down (1024 x 2816) fp32 weight gradients, 8192
bf16 activation tokens per distinct input (attention in, o in, MLP in,
down in) with a power-law spectrum of exponent 1.5; rank-32 factors; all 7
matrices whitened; per-tensor E4M3.

One step = the per-step path of GIFT over the block: the grouped
whiten + quantize of the 7 gradients and the grouped dequantize + un-whiten,
with the factor refresh of the 4 inputs run inside the timed loop every 50
steps (the paper's refresh interval), so it is amortized exactly as in
training.  Each step takes the next gradient set from a ring of resident
sets whose footprint is several times the 256 MB Infinity Cache, so every
step reads its gradients from HBM.  Inputs are resident in HBM before the
timed region.  One JSON line on stdout.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10]
"""

import argparse
import hashlib
import json
import os
import sys
import time

METRIC = ("GB/s of fp32 gradient through whiten→FP8→unwhiten (% HBM peak); "
          "rel. error vs Euclid")
HBM_PEAK_GBS = 8000.0
VALU_F32_PEAK_TFLOPS = 78.6     # 256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz (no packed fp32)
MFMA_BF16_PEAK_TFLOPS = 2500.0
REFRESH_EVERY = 50
HERE = os.path.dirname(os.path.abspath(__file__))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--ring", type=int, default=4, help="resident gradient sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--quiet", action="store_true")
    return p.parse_args()


def log(args, msg):
    if not args.quiet:
        print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for name in ("roundtrip.hip", "device.hpp", "refresh.hip"):
        with open(os.path.join(HERE, "fac_whitening_gift_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, src_hash, elems):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel sources; else None."""
    path = os.path.join(HERE, "profiles", "traffic_%s.json" % kernel)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != src_hash or t.get("elements") != elems:
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the GIFT path here has no inter-GPU part "
              "(the collective is out of scope); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import fac_whitening_gift_amd as fg

    fg.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.llama_block(hidden=1024, mlp=2816, tokens=8192, exponent=1.5)
    elems = w.gradient_elements
    grad_bytes = 4 * elems
    log(args, "workload %s: %d layers, %.1f M gradient elements" %
        (w.name, len(w.layers), elems / 1e6))

    # ---- resident inputs ---------------------------------------------------
    inputs, factors = {}, {}
    for k, spec in enumerate(w.inputs):
        inputs[spec.name] = synth.draw_input(spec, seed=1000 + k, device=dev, as_bf16=True)
        factors[spec.name] = fg.Factor(spec.d_in, device=dev)
    ring = []
    for r in range(args.ring):
        layers = []
        for i, l in enumerate(w.layers):
            inp = inputs[l.input]
            G = synth.draw_gradient(l.d_out, inp["Q"], inp["ev"], seed=5000 + 100 * r + i,
                                    device=dev)
            layers.append(fg.Layer(G, factor=factors[l.input]))
        ring.append(layers)
    items = [dict(X=inputs[spec.name]["X"], factor=factors[spec.name], seed=0)
             for spec in w.inputs]
    ws_ref = torch.empty(fg.gift_refresh_group_workspace_bytes(items), dtype=torch.uint8,
                         device=dev)
    nb_w = max(fg.gift_group_workspace_bytes(0, ring[0], fg.SCALE_TENSOR), 256)
    ws_w = torch.empty(nb_w, dtype=torch.uint8, device=dev)
    nb_e = max(fg.gift_group_workspace_bytes(2, ring[0], fg.SCALE_TENSOR), 256)
    ws_e = torch.empty(nb_e, dtype=torch.uint8, device=dev)
    nb_d = max(fg.gift_group_workspace_bytes(1, ring[0], fg.SCALE_TENSOR), 256)
    ws_d = torch.empty(nb_d, dtype=torch.uint8, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)

    def refresh_all(seed):
        for k, it in enumerate(items):
            it["seed"] = seed + k
        fg.gift_refresh_factors(items, ws=ws_ref)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    refresh_all(1)
    torch.cuda.synchronize()

    def step(s, timed):
        layers = ring[s % len(ring)]
        if s % REFRESH_EVERY == 0:
            refresh_all(7 * s + 1)
        if timed:
            e0, e1, e2 = ev(), ev(), ev()
            e0.record()
            fg.gift_whiten_quantize(layers, flags=flags, ws=ws_w)
            e1.record()
            fg.gift_dequant_unwhiten(layers, ws=ws_d)
            e2.record()
            return e0, e1, e2
        fg.gift_whiten_quantize(layers, flags=flags, ws=ws_w)
        fg.gift_dequant_unwhiten(layers, ws=ws_d)
        return None

    for s in range(args.warmup):
        step(s + 1, False)          # warm-up steps never hit the refresh slot
    torch.cuda.synchronize()
    log(args, "timing %d steps" % args.steps)
    marks = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        marks.append(step(s, True))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    t_wq = np.array([a.elapsed_time(b) for a, b, c in marks]) * 1e-3
    t_du = np.array([b.elapsed_time(c) for a, b, c in marks]) * 1e-3
    value = grad_bytes * args.steps / elapsed / 1e9
    ms_per_step = elapsed / args.steps * 1e3

    # ---- refresh on its own ------------------------------------------------
    r0, r1 = ev(), ev()
    r0.record()
    for _ in range(3):
        refresh_all(11)
    r1.record()
    torch.cuda.synchronize()
    refresh_ms = r0.elapsed_time(r1) / 3
    syrk_flops = sum(2.0 * s.tokens * s.d_in * s.d_in for s in w.inputs)

    # ---- Euclidean baseline and 1x128 variant (same ring) -------------------
    def timed_loop(fn, n):
        es = []
        for s in range(n):
            a, b = ev(), ev()
            a.record()
            fn(ring[s % len(ring)])
            b.record()
            es.append((a, b))
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in es]) * 1e-3

    t_eu = timed_loop(lambda L: fg.gift_euclid_fp8_roundtrip(L, ws=ws_e), 20)
    ring_b = [[fg.Layer(L.G, factor=L.factor, block128=True) for L in layers] for layers in ring]
    nb_b = max(fg.gift_group_workspace_bytes(0, ring_b[0], fg.SCALE_BLOCK128),
               fg.gift_group_workspace_bytes(1, ring_b[0], fg.SCALE_BLOCK128), 256)
    ws_b = torch.empty(nb_b, dtype=torch.uint8, device=dev)
    t_b = []
    for s in range(20):
        a, b = ev(), ev()
        a.record()
        fg.gift_whiten_quantize(ring_b[s % len(ring_b)], scaling=fg.SCALE_BLOCK128, ws=ws_b)
        fg.gift_dequant_unwhiten(ring_b[s % len(ring_b)], scaling=fg.SCALE_BLOCK128, ws=ws_b)
        b.record()
        t_b.append((a, b))
    torch.cuda.synchronize()
    t_b = np.array([a.elapsed_time(b) for a, b in t_b]) * 1e-3

    # ---- quality: relative error vs Euclidean FP8 ---------------------------
    layers = ring[0]
    fg.gift_whiten_quantize(layers, ws=ws_w)
    fg.gift_dequant_unwhiten(layers, ws=ws_d)
    err_g = fg.gift_roundtrip_error(layers).cpu().numpy()
    eu_layers = [fg.Layer(L.G) for L in layers]
    fg.gift_euclid_fp8_roundtrip(eu_layers, ws=ws_e)
    err_e = fg.gift_roundtrip_error(eu_layers).cpu().numpy()
    m1_g = float(np.sqrt(err_g[:, 0].sum() / err_g[:, 1].sum()))
    m1_e = float(np.sqrt(err_e[:, 0].sum() / err_e[:, 1].sum()))
    # K-FAC-metric error: ||(G^-G) S|| / ||G S||, S = (A + lambda_floor I)^-1/2 from
    # the exact covariance (measurement only; fp64 torch on the device)
    num_g = num_e = den = 0.0
    S_cache = {}
    for L, E, l in zip(layers, eu_layers, w.layers):
        if l.input not in S_cache:
            X = inputs[l.input]["X"].double()
            A = X.T @ X / X.shape[0]
            lam = 1e-3 * torch.trace(A) / A.shape[0]
            ev_, V = torch.linalg.eigh(A)
            S_cache[l.input] = (V * (ev_.clamp_min(0) + lam).rsqrt()) @ V.T
        S = S_cache[l.input]
        G = L.G.double()
        num_g += float(torch.linalg.norm((L.G_hat.double() - G) @ S) ** 2)
        num_e += float(torch.linalg.norm((E.G_hat.double() - G) @ S) ** 2)
        den += float(torch.linalg.norm(G @ S) ** 2)
    m2_g, m2_e = float(np.sqrt(num_g / den)), float(np.sqrt(num_e / den))

    # ---- roofline of the dominant launch -------------------------------------
    src = kernel_source_hash()
    wq, du = float(np.mean(t_wq)), float(np.mean(t_du))
    if du >= wq:
        kname, t_k, alg_bytes, alg_flops = "dequant_unwhiten", du, 5.0 * elems, 128.0 * elems
    else:
        kname, t_k, alg_bytes, alg_flops = "whiten_quantize", wq, 5.0 * elems, 192.0 * elems
    gbs = alg_bytes / t_k / 1e9
    tfl = alg_flops / t_k / 1e12
    traffic = load_traffic(kname, src, elems)
    if tfl / VALU_F32_PEAK_TFLOPS > gbs / HBM_PEAK_GBS:
        roof = {"bound": "alu", "achieved": round(tfl, 3), "peak": VALU_F32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tfl / VALU_F32_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic
    roof["kernel"] = kname
    roof["hbm_achieved_gbs"] = round(gbs, 1)
    roof["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    roof["launch_ms"] = round(t_k * 1e3, 4)
    roof["source_hash"] = src

    # ---- CPU baseline: the oracle on the host ------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, w, args)

    rt = wq + du
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: q,k,v,o 1024x1024, gate/up 2816x1024, down 1024x2816 fp32 "
                               "gradients; 8192 bf16 tokens per input, spectrum i^-1.5; rank 32; "
                               "per-tensor E4M3; refresh every %d steps; ring of %d gradient "
                               "sets" % (w.name, REFRESH_EVERY, args.ring),
                   "layers": len(w.layers), "gradient_elements": elems},
        "hbm_frac_of_value": round(value / HBM_PEAK_GBS, 4),
        "roundtrip_only_gbps": round(grad_bytes / rt / 1e9, 2),
        "whiten_quantize_ms": round(wq * 1e3, 4), "dequant_unwhiten_ms": round(du * 1e3, 4),
        "layers_per_s": round(len(w.layers) / rt, 1),
        "refresh_ms_4_inputs": round(refresh_ms, 3),
        "refresh_syrk_mfma_frac_lower_bound": round(syrk_flops / (refresh_ms * 1e-3) / 1e12 /
                                                     MFMA_BF16_PEAK_TFLOPS, 4),
        "euclid_roundtrip_gbps": round(grad_bytes / float(np.mean(t_eu)) / 1e9, 2),
        "block128_roundtrip_gbps": round(grad_bytes / float(np.mean(t_b)) / 1e9, 2),
        "quality": {"m1_gift": round(m1_g, 5), "m1_euclid": round(m1_e, 5),
                    "m1_ratio": round(m1_g / m1_e, 4), "m2_gift": round(m2_g, 5),
                    "m2_euclid": round(m2_e, 5), "m2_ratio": round(m2_g / m2_e, 4),
                    "damping": "floor+tail"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(layers, w, args):
    """The oracle (fp64 numpy, as it stands) on the host: the same round trip
    (whiten, E4M3, dequantize, un-whiten) on the block's gradients, repeated
    until about cpu_seconds of work; GB/s of fp32 gradient."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import gift as og

    log(args, "cpu baseline (oracle)")
    host = []
    for L in layers:
        c = L.factor.coef.cpu().numpy().astype(np.float64)
        f = og.factor_from_parts(L.factor.U.cpu().numpy(), L.factor.theta.cpu().numpy(),
                                 c[2], c[3], c[4], c[5])
        host.append((L.G.cpu().numpy(), f))
    done_bytes, t0 = 0, time.perf_counter()
    passes = 0
    while True:
        for G, f in host:
            og.gift_roundtrip(G, f)
            done_bytes += G.nbytes
        passes += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    el = time.perf_counter() - t0
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "%d pass(es) over the block's 7 gradients (%.1f MB fp32), %.1f s, "
                      "BLAS threads %d, host CPUs %d" % (passes, sum(G.nbytes for G, _ in host)
                                                         / 1e6, el, threads,
                                                         len(os.sched_getaffinity(0)))}


if __name__ == "__main__":
    main()
