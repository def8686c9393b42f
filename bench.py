"""Throughput of the theta-bundle projection on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload large60] [--tokens M] [--bands G]

One step is one pass of the hot path over a synthetic Gemma-shaped layer
stack: for every layer, the band of the layer (tb_band_index) and then the
seven projections q, k, v, o, gate, up, down (tb_linear_forward), each reading
its band's W0 and the layer's s, U, V from HBM.  All inputs are resident on
the device before timing starts.

Workloads (synthetic, seeded; value distributions of the measured stacks):
  large60        60 layers, hidden 5376, MLP 21504, rank 256, G=6 (default)
  banded26       26 layers, hidden 1152, MLP 6912, rank 128, G=4
  passthrough26  26 layers, G=26, rank 0, s=1
Token counts <= 64 report GB/s of algorithmic bytes (HBM-bound); larger
token counts report TFLOP/s of algorithmic flops (matrix-core-bound).

Prints one JSON line.  The roofline object covers the dominant kernel; the
cpu_baseline object times the float64 oracle on a bounded host sample.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "theta-bundle projection TFLOP/s (prefill M) and GB/s (decode M), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
DECODE_MAX_TOKENS = 64

# Projections of a layer that read the same input, grouped into one call.
GROUPS = [["q_proj", "k_proj", "v_proj"], ["o_proj"], ["gate_proj", "up_proj"], ["down_proj"]]

WORKLOADS = {
    "large60": dict(layers=60, shapes="SHAPES_60", rank=256, bands=6, tokens=16, seed=4),
    "banded26": dict(layers=26, shapes="SHAPES_26", rank=128, bands=4, tokens=4, seed=3),
    "passthrough26": dict(layers=26, shapes="SHAPES_26", rank=0, bands=26, tokens=8, seed=2),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large60", choices=sorted(WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--bands", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-group", action="store_true",
                    help="one tb_linear_forward call per projection instead of grouping q/k/v and gate/up")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget of the oracle timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device copies of a known size (scales the HBM byte counters)")
    return ap.parse_args()


COPY_BYTES = 512 << 20


def copy_calibration():
    """Plain 512 MiB device-to-device copies: what the FETCH_SIZE / WRITE_SIZE counters read for them
    against the bytes actually moved gives the scale applied to the projection kernel's counters."""
    import torch
    torch.cuda.set_device(0)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "copies": 4}), flush=True)


def call_bytes(M, O, I, R, e=2):
    return e * (O * I + R * (O + I) + O + M * (I + O))


def call_flops(M, O, I, R):
    return 2 * M * (O * I + R * (O + I))


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_factored_linear_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel, workload_tag):
    """HBM bytes per launch from the committed counter summary, if it is current."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        rec = data.get(workload_tag)
        if rec and rec.get("kernel_source_digest") == kernel_source_digest() and rec.get("kernel") == kernel:
            return rec.get("bytes_per_launch")
    except Exception:
        return None
    return None


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is not sharded across GPUs",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rank_factored_linear_amd import binding as tb
    from rank_factored_linear_amd import inputs as gen

    wl = dict(WORKLOADS[args.workload])
    if args.tokens is not None:
        wl["tokens"] = args.tokens
    if args.bands is not None:
        wl["bands"] = args.bands
    L, R, G, M = wl["layers"], wl["rank"], wl["bands"], wl["tokens"]
    shapes = getattr(gen, wl["shapes"])
    passthrough = args.workload == "passthrough26"
    torch.cuda.set_device(0)
    dev = "cuda"
    t_setup = time.time()

    # ---- resident inputs ---------------------------------------------------
    band_of = []
    for l in range(L):
        b = ctypes.c_int32()
        st = tb.lib.tb_band_index(L, G, l, ctypes.byref(b))
        assert st == 0
        band_of.append(b.value)
    W0 = {}
    for b in range(G):
        for fam in gen.FAMILIES:
            W0[(b, fam)] = gen.device_w0(torch, wl["seed"], fam, shapes, b)
    bundles, xs = {}, {}
    for l in range(L):
        for fam in gen.FAMILIES:
            if passthrough:
                O = shapes[fam][0]
                bundles[(l, fam)] = {"s": torch.ones(O, dtype=torch.bfloat16, device=dev), "U": None, "V": None}
            else:
                bundles[(l, fam)] = gen.device_bundle(torch, wl["seed"], fam, shapes, l, band_of[l], R, with_w0=False)
            xs[(l, fam)] = gen.device_activations(torch, wl["seed"], fam, shapes, l, M)
    ys = {fam: torch.empty((M, shapes[fam][0]), dtype=torch.bfloat16, device=dev) for fam in gen.FAMILIES}
    # Projections that take the same layer input go in one grouped call.
    groups = [[f] for f in gen.FAMILIES] if args.no_group else GROUPS
    ws_need = []
    for grp in groups:
        dims = (tb.Projection * len(grp))(*[tb.Projection(None, None, None, None, None, None, *shapes[f], R)
                                            for f in grp])
        nb = ctypes.c_size_t(0)
        assert tb.lib.tb_linear_forward_group_workspace_size(len(grp), dims, M, tb.TB_BF16, ctypes.byref(nb)) == 0
        ws_need.append(nb.value)
    ws = tb.workspace_for(max(ws_need))
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    # Prepared argument tuples: the timed loop only crosses the C ABI.
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    fwd = tb.lib.tb_linear_forward
    fwd_group = tb.lib.tb_linear_forward_group
    calls = []   # (layer, families, function, argument tuple)
    for l in range(L):
        for grp in groups:
            members = []
            for fam in grp:
                bd = bundles[(l, fam)]
                members.append((xs[(l, fam)], bd["s"], W0[(band_of[l], fam)], bd["U"] if R else None,
                                bd["V"] if R else None, ys[fam]))
            if len(grp) == 1:
                x, s_, w0, u, v, y = members[0]
                O, I = shapes[grp[0]]
                argv = (x.data_ptr(), s_.data_ptr(), w0.data_ptr(), u.data_ptr() if R else None,
                        v.data_ptr() if R else None, y.data_ptr(), M, O, I, R, tb.TB_BF16, ws.data_ptr(), ws.numel(),
                        stream)
                calls.append((l, grp, fwd, argv))
            else:
                arr = tb.projection_array(members)
                calls.append((l, grp, fwd_group, (len(grp), arr, M, tb.TB_BF16, ws.data_ptr(), ws.numel(), stream)))
    band_idx = tb.lib.tb_band_index
    bout = ctypes.c_int32()
    per_layer = len(groups)

    def step(events=None):
        n = 0
        for l in range(L):
            band_idx(L, G, l, ctypes.byref(bout))          # band select (host)
            for _ in range(per_layer):
                if events is not None:
                    events[n].record()
                fn, argv = calls[n][2], calls[n][3]
                st = fn(*argv)
                if st:
                    raise RuntimeError(tb.lib.tb_last_error().decode())
                n += 1
        if events is not None:
            events[n].record()

    def grp_bytes(grp):
        return sum(call_bytes(M, *shapes[f], R) for f in grp)

    def grp_flops(grp):
        return sum(call_flops(M, *shapes[f], R) for f in grp)

    step_bytes = sum(grp_bytes(c[1]) for c in calls)
    step_flops = sum(grp_flops(c[1]) for c in calls)
    decode = M <= DECODE_MAX_TOKENS

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region --------------------------------------------------------
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    if tb.workspace_error_word() != 0:
        raise RuntimeError("a bounded wait in the projection kernel timed out")

    # ---- per-launch durations of the projection kernel (same steps again) ----
    per_call_ms = np.zeros(len(calls))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
    for _ in range(args.steps):
        step(ev)
        torch.cuda.synchronize()
        per_call_ms += np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(len(calls))])
    per_call_ms /= args.steps
    launch_bytes = np.array([grp_bytes(c[1]) for c in calls], dtype=np.float64)
    launch_flops = np.array([grp_flops(c[1]) for c in calls], dtype=np.float64)

    if decode:
        unit = "GB/s"
        value = step_bytes / (ms * 1e-3) / 1e9
        achieved = launch_bytes.sum() / (per_call_ms.sum() * 1e-3) / 1e9
        kernel = "decode_kernel<bf16,%d,*>" % (1 if M <= 16 else (2 if M <= 32 else 4))
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
        per_launch = float(launch_bytes.mean())
    else:
        unit = "TFLOP/s"
        value = step_flops / (ms * 1e-3) / 1e12
        achieved = launch_flops.sum() / (per_call_ms.sum() * 1e-3) / 1e12
        kernel = "big::gemm_kernel (with xv::xv_kernel in the same call)"
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
        per_launch = float(launch_flops.mean())
    roof["kernel"] = kernel
    roof["calls_per_step"] = len(calls)
    roof["avg_launch_us"] = round(float(per_call_ms.mean()) * 1e3, 2)
    roof["algorithmic_per_launch"] = round(per_launch, 1)
    tag = f"{args.workload}_M{M}_G{G}"
    traffic = counter_traffic(kernel, tag)
    roof["traffic"] = traffic

    # ---- CPU baseline: the float64 oracle on a bounded sample ------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, wl, shapes, calls, bundles, W0, xs, band_of, passthrough, decode)

    line = {
        "metric": METRIC,
        "value": round(value, 2 if decode else 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {L}-layer stack, 7 projections per layer, rank {R}, "
                               f"G={G} bands, {M} tokens",
                   "layers": L, "projections_per_step": L * len(gen.FAMILIES),
                   "grouping": "+".join(",".join(f.split("_")[0] for f in g) for g in groups),
                   "rank": R, "bands": G, "tokens": M,
                   "hidden": shapes["q_proj"][1], "mlp": shapes["gate_proj"][0],
                   "step_bytes": step_bytes, "step_flops": step_flops, "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(f"# setup {t_setup:.1f}s  step {ms:.3f} ms  per-launch sum {per_call_ms.sum():.3f} ms", file=sys.stderr)
    print(json.dumps(line), flush=True)


def cpu_baseline(args, wl, shapes, calls, bundles, W0, xs, band_of, passthrough, decode):
    """Time the float64 oracle on the first layer's projections of the same stack."""
    import numpy as np
    import torch

    import oracle

    try:
        import threadpoolctl
        threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    M, R = wl["tokens"], wl["rank"]
    Mc = M if decode else min(M, 256)       # prefill: a token slice keeps it bounded
    done_bytes, done_flops, secs, used = 0, 0, 0.0, []
    for l, fam in ((c[0], f) for c in calls for f in c[1]):
        if secs > args.cpu_seconds:
            break
        O, I = shapes[fam]
        bd = bundles[(l, fam)]
        host = dict(x=bits(xs[(l, fam)][:Mc]), s=bits(bd["s"]), W0=bits(W0[(band_of[l], fam)]))
        if R:
            host["U"], host["V"] = bits(bd["U"]), bits(bd["V"])
        t = time.perf_counter()
        dec = {k: oracle.bf16_bits_to_f64(v) for k, v in host.items()}
        U = dec.get("U", np.zeros((O, 0)))
        V = dec.get("V", np.zeros((I, 0)))
        oracle.forward(dec["x"], dec["s"], dec["W0"], U, V)
        secs += time.perf_counter() - t
        done_bytes += call_bytes(Mc, O, I, R)
        done_flops += call_flops(Mc, O, I, R)
        used.append(f"{l}:{fam}")
    if decode:
        val, unit = done_bytes / secs / 1e9, "GB/s"
    else:
        val, unit = done_flops / secs / 1e12, "TFLOP/s"
    return {"value": round(val, 4), "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{len(used)} projections of the same stack ({used[0]} .. {used[-1]}), {Mc} tokens, "
                      f"float64 NumPy incl. bf16 decoding, {secs:.1f} s"}


if __name__ == "__main__":
    main()
