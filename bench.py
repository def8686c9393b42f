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
  reconstruct60  the 60-layer stack's 420 (layer, projection) weights rebuilt
                 as diag(s) W0 + U V^T in fp32 (tb_reconstruct_weight) and
                 compared with the originals a W0_band + N(0, 2e-3) by the
                 relative Frobenius error (tb_rel_frobenius_error); --rank 0
                 for the rank-0 bundle; --fused measures the same errors
                 without writing the rebuilt weight (tb_reconstruction_error),
                 --bands/--rank give one point of a (G, rank) sweep
Token counts <= 64 report GB/s of algorithmic bytes (HBM-bound); larger
token counts report TFLOP/s of algorithmic flops (matrix-core-bound).

Beside the K-step figure the line carries the per-step spread, the same stack
replayed from a captured graph, and the GPU clock and power sampled while the
graph replays for about a second more.  Stacks whose distinct inputs are smaller than twice the 256 MB
Infinity Cache are timed over a rotating pool of replicas of at least 1 GiB,
so that every step reads cold data (the figure reported); the stack-order
figure from one replica is reported beside it.

Prints one JSON line.  The roofline object covers the dominant kernel; the
cpu_baseline object times the float64 oracle on a bounded host sample.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "theta-bundle projection TFLOP/s (prefill M) and GB/s (decode M), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores
DECODE_MAX_TOKENS = 64
CACHE_BYTES = 256 << 20        # MI355X Infinity Cache
COLD_POOL_BYTES = 1 << 30

# Projections of a layer that read the same input, grouped into one call.
GROUPS = [["q_proj", "k_proj", "v_proj"], ["o_proj"], ["gate_proj", "up_proj"], ["down_proj"]]

WORKLOADS = {
    "large60": dict(layers=60, shapes="SHAPES_60", rank=256, bands=6, tokens=16, seed=4, prefill=4096),
    "banded26": dict(layers=26, shapes="SHAPES_26", rank=128, bands=4, tokens=4, seed=3, prefill=2048),
    "passthrough26": dict(layers=26, shapes="SHAPES_26", rank=0, bands=26, tokens=8, seed=2, prefill=0),
    "reconstruct60": dict(layers=60, shapes="SHAPES_60", rank=256, bands=6, tokens=0, seed=5),
    "decompose26": dict(layers=26, shapes="SHAPES_26", rank=128, bands=4, tokens=0, seed=6),
    "decompose60": dict(layers=60, shapes="SHAPES_60", rank=256, bands=6, tokens=0, seed=7),
    "tiny4": dict(layers=4, rank=16, bands=2, tokens=8, seed=1),
}
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large60", choices=sorted(WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--bands", type=int, default=None)
    ap.add_argument("--rank", type=int, default=None, help="rank of the bundles (reconstruct60 only)")
    ap.add_argument("--fused", action="store_true",
                    help="reconstruct60: measure the error without writing the rebuilt weight (tb_reconstruction_error)")
    ap.add_argument("--materialised", action="store_true",
                    help="forward stacks: rebuild every layer's weight once in bf16 (outside the timed region) and "
                         "time the dense projections of the materialise-once mode (tb_dense_forward semantics)")
    ap.add_argument("--power-iters", type=int, default=2, help="decompose*: power iterations of the randomized SVD")
    ap.add_argument("--als-iters", type=int, default=0,
                    help="decompose*: also time this many rounds of alternating least squares on the shared blocks")
    ap.add_argument("--tie-families", choices=["all", "attn"], default="all",
                    help="forward stacks: 'attn' shares W0 for the attention families only and keeps the MLP "
                         "projections as dense weights (rank 0, no scale, tb_dense_forward semantics)")
    ap.add_argument("--replicas", type=int, default=None,
                    help="rotating pool of input replicas (default: enough for >= 1 GiB when the stack is small)")
    ap.add_argument("--no-graph", action="store_true", help="skip the captured-graph leg")
    ap.add_argument("--prefill-tokens", type=int, default=None,
                    help="token count of the prefill object beside a decode line (default: the workload's, "
                         "4096 for large60, 2048 for banded26; 0: none)")
    ap.add_argument("--prefill-steps", type=int, default=5)
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


# ---- algorithmic work -------------------------------------------------------------


def call_bytes(M, O, I, R, e=2):
    """Forward: W0, U, V and s once, x in and y out."""
    return e * (O * I + R * (O + I) + O + M * (I + O))


def dense_call_bytes(M, O, I, e=2):
    """Materialise-once forward: the whole weight once, x in and y out."""
    return e * (O * I + M * (I + O))


def call_flops(M, O, I, R):
    return 2 * M * (O * I + R * (O + I))


def reconstruct_bytes(O, I, R, e_in=2, e_out=4):
    """Reconstruct: s, W0, U and V in, the rebuilt weight out."""
    return e_in * (O * I + R * (O + I) + O) + e_out * O * I


def frobenius_bytes(O, I, e=4):
    """Error: both matrices read once."""
    return 2 * e * O * I


def reconstruct_kernel_names(R):
    """The kernels that rebuild a bf16 bundle of rank R into fp32, and that measure its error without rebuilding.
    The persistent kernel takes k-tiles of 32 per tile, 2, 4 or 8 of them (its error variant at least 4)."""
    k32 = (R + 31) // 32
    kt = 2 if k32 <= 2 else 4 if k32 <= 4 else 8
    rec = ("reconstruct_rank0_kernel" if R == 0 else
           f"rp::reconstruct_persistent_kernel<float, false, {kt}>" if R <= 256 and R % 8 == 0 else
           "mm::reconstruct_mfma_kernel" if R % 8 == 0 else "reconstruct_lowrank_kernel")
    fused = ("rerr_rank0_kernel" if R == 0 else
             f"rp::reconstruct_persistent_kernel<float, true, {max(kt, 4)}>" if R <= 256 and R % 8 == 0 else
             "rerr_t128_kernel" if R % 8 == 0 else "rerr_t64_kernel")
    return rec, fused


def fused_error_bytes(O, I, R, e_in=2, e_orig=4):
    """Error without the rebuilt weight: s, W0, U, V and the original read once."""
    return e_in * (O * I + R * (O + I) + O) + e_orig * O * I


# ---- counters committed under profiles/ ---------------------------------------------


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


def profile_durations(tag):
    """Average duration per call of the dominant kernel(s) in the committed rocprofv3 kernel trace of the same
    bench command, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "kernel_durations.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(tag)
        if rec and rec.get("kernel_source_digest") == kernel_source_digest():
            return {"file": rec["file"], "avg_call_us": rec["avg_call_us"], "kernel": rec["kernel"]}
    except Exception:
        return None
    return None


# ---- timing helpers -----------------------------------------------------------------


def timed_steps(torch, run_step, steps):
    """K steps between two events on the launch stream (the figure reported), with an event at every step
    boundary in between for the spread."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for k in range(steps):
        run_step(k)
        ev[k + 1].record()
    torch.cuda.synchronize()
    per = [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
    return ev[0].elapsed_time(ev[-1]) / steps, per


def spread(per_step_ms):
    s = sorted(per_step_ms)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    return {"median_ms": round(med, 4), "min_ms": round(s[0], 4), "max_ms": round(s[-1], 4), "trials": n}


class ClockSampler:
    """GPU shader clock (MHz) and socket power sampled every 50 ms from a side thread (amdsmi through torch),
    around untimed graph replays."""

    def __init__(self, torch):
        self.torch, self.clk, self.pwr, self.err = torch, [], [], None
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            try:
                self.clk.append(float(self.torch.cuda.clock_rate(0)))
                self.pwr.append(float(self.torch.cuda.power_draw(0)))
            except Exception as e:        # amdsmi missing or not permitted: no figure
                self.err = f"{type(e).__name__}: {e}"[:120]
                return
            self._stop.wait(0.05)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=5)

    def summary(self):
        if not self.clk:
            return {"available": False, "reason": self.err or "no samples"}
        c, p = sorted(self.clk), sorted(self.pwr)
        return {"available": True, "samples": len(c), "gfx_clock_mhz_median": c[len(c) // 2],
                "gfx_clock_mhz_min": c[0], "gfx_clock_mhz_max": c[-1],
                "power_median": p[len(p) // 2], "power_max": p[-1], "power_unit": "as torch.cuda.power_draw"}


def graph_leg(torch, make_step, steps, outputs):
    """Capture one step into a graph and replay it.  Each checked replay's outputs must equal the eager step's
    bit for bit (the kernels are deterministic); an eager step runs before each checked replay."""
    side = torch.cuda.Stream()
    step_on_side = make_step(side.cuda_stream)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_on_side()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step_on_side()
    torch.cuda.synchronize()
    eager_step = make_step(torch.cuda.current_stream().cuda_stream)
    for _ in range(2):
        eager_step()
        torch.cuda.synchronize()
        want = [o.clone() for o in outputs]
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(want, outputs):
            if not torch.equal(a.view(torch.uint8), b.view(torch.uint8)):
                raise RuntimeError("a replay of the captured step differs from the eager step")
    for _ in range(2):
        g.replay()
    ms, per = timed_steps(torch, lambda k: g.replay(), steps)
    # Clock and power while the same replays run for about a second (outside the timed region).
    with ClockSampler(torch) as clk:
        t_end, n = time.time() + 1.0, 0
        while time.time() < t_end or n < steps:
            g.replay()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    return ms, per, clk.summary()


def _bits(torch, np, t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _blas_threads():
    try:
        import threadpoolctl
        return max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        return len(os.sched_getaffinity(0))


def _host_info():
    """CPU model and BLAS library of the host that times the oracle."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        import threadpoolctl
        libs = [f"{p.get('internal_api')} {p.get('version')}" for p in threadpoolctl.threadpool_info()
                if p.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas, "affinity_cpus": len(os.sched_getaffinity(0))}


# ---- forward stacks -----------------------------------------------------------------


def bench_forward(args, torch, np, tb, gen):
    wl = dict(WORKLOADS[args.workload])
    if args.tokens is not None:
        wl["tokens"] = args.tokens
    if args.bands is not None:
        wl["bands"] = args.bands
    L, R, G, M = wl["layers"], wl["rank"], wl["bands"], wl["tokens"]
    shapes = getattr(gen, wl["shapes"])
    passthrough = args.workload == "passthrough26"
    dev = "cuda"
    t_setup = time.time()

    # ---- resident weights ----------------------------------------------------
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
    bundles = {}
    for l in range(L):
        for fam in gen.FAMILIES:
            if passthrough:
                O = shapes[fam][0]
                bundles[(l, fam)] = {"s": torch.ones(O, dtype=torch.bfloat16, device=dev), "U": None, "V": None}
            else:
                bundles[(l, fam)] = gen.device_bundle(torch, wl["seed"], fam, shapes, l, band_of[l], R, with_w0=False)

    # Materialise-once mode (every family) and tie_families="attn" (the MLP
    # families): W = diag(s) W0 + U V^T per layer, rebuilt once in bf16; each
    # such call is a dense projection (no scale, rank 0).
    dense_fams = set(gen.FAMILIES) if args.materialised else (
        set(tb.MLP_FAMILIES) if args.tie_families == "attn" else set())
    dense = None
    if dense_fams:
        dense = {}
        for l in range(L):
            for fam in sorted(dense_fams):
                bd = bundles[(l, fam)]
                dense[(l, fam)] = tb.reconstruct_weight(bd["s"], W0[(band_of[l], fam)], bd["U"] if R else None,
                                                        bd["V"] if R else None, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()

    def nbytes(t):
        return 0 if t is None else t.numel() * t.element_size()

    distinct = (sum(nbytes(t) for t in (dense or {}).values()) +
                sum(nbytes(t) for k, t in W0.items() if k[1] not in dense_fams) +
                sum(nbytes(v) for k, bd in bundles.items() if k[1] not in dense_fams for v in bd.values()))
    replicas = args.replicas
    if replicas is None:
        replicas = 1 if distinct >= 2 * CACHE_BYTES else math.ceil(COLD_POOL_BYTES / distinct)
    # Replica r > 0 holds copies of every weight tensor at addresses of its own; x is shared.
    pools = [(W0, bundles, dense)]
    for _ in range(1, replicas):
        pools.append(({k: t.clone() for k, t in W0.items() if k[1] not in dense_fams},
                      {k: {n: (None if t is None else t.clone()) for n, t in bd.items()}
                       for k, bd in bundles.items() if k[1] not in dense_fams},
                      None if dense is None else {k: t.clone() for k, t in dense.items()}))
    # Projections that take the same layer input go in one grouped call.
    groups = [[f] for f in gen.FAMILIES] if args.no_group else GROUPS
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    fwd = tb.lib.tb_linear_forward
    fwd_group = tb.lib.tb_linear_forward_group
    band_idx = tb.lib.tb_band_index
    bout = ctypes.c_int32()
    per_layer = len(groups)

    def time_stack(M, steps, warmup, with_graph, with_cpu, cpu_seconds):
        """One leg: K steps of the whole stack at M tokens over the resident weights (one JSON object)."""
        t0 = time.time()
        xs = {(l, fam): gen.device_activations(torch, wl["seed"], fam, shapes, l, M)
              for l in range(L) for fam in gen.FAMILIES}
        ys = {fam: torch.empty((M, shapes[fam][0]), dtype=torch.bfloat16, device=dev) for fam in gen.FAMILIES}
        ws_need = []
        for grp in groups:
            dims = (tb.Projection * len(grp))(*[tb.Projection(None, None, None, None, None, None, *shapes[f],
                                                              0 if f in dense_fams else R) for f in grp])
            nb = ctypes.c_size_t(0)
            assert tb.lib.tb_linear_forward_group_workspace_size(len(grp), dims, M, tb.TB_BF16, ctypes.byref(nb)) == 0
            ws_need.append(nb.value)
        ws = tb.workspace_for(max(ws_need))

        def build_calls(stream_handle, pool):
            """Prepared argument tuples: the timed loop only crosses the C ABI."""
            W0p, bundlesp, densep = pool
            stream = ctypes.c_void_p(stream_handle)
            calls = []   # (layer, families, function, argument tuple)
            for l in range(L):
                for grp in groups:
                    members = []
                    for fam in grp:
                        if fam in dense_fams:
                            members.append((xs[(l, fam)], None, densep[(l, fam)], None, None, ys[fam]))
                        else:
                            bd = bundlesp[(l, fam)]
                            members.append((xs[(l, fam)], bd["s"], W0p[(band_of[l], fam)], bd["U"] if R else None,
                                            bd["V"] if R else None, ys[fam]))
                    if len(grp) == 1:
                        x, s_, w0, u, v, y = members[0]
                        O, I = shapes[grp[0]]
                        Rc = 0 if grp[0] in dense_fams else R
                        argv = (x.data_ptr(), None if s_ is None else s_.data_ptr(), w0.data_ptr(),
                                u.data_ptr() if Rc else None, v.data_ptr() if Rc else None, y.data_ptr(), M, O, I,
                                Rc, tb.TB_BF16, ws.data_ptr(), ws.numel(), stream)
                        calls.append((l, grp, fwd, argv))
                    else:
                        arr = tb.projection_array(members)   # the tuple keeps the array alive
                        calls.append((l, grp, fwd_group, (len(grp), arr, M, tb.TB_BF16, ws.data_ptr(), ws.numel(),
                                                          stream)))
            return calls

        def run(calls):
            n = 0
            for l in range(L):
                band_idx(L, G, l, ctypes.byref(bout))          # band select (host)
                for _ in range(per_layer):
                    fn, argv = calls[n][2], calls[n][3]
                    st = fn(*argv)
                    if st:
                        raise RuntimeError(tb.lib.tb_last_error().decode())
                    n += 1

        main_stream = torch.cuda.current_stream().cuda_stream
        pool_calls = [build_calls(main_stream, p) for p in pools]
        calls = pool_calls[0]

        def grp_bytes(grp):
            return sum(dense_call_bytes(M, *shapes[f]) if f in dense_fams else call_bytes(M, *shapes[f], R)
                       for f in grp)

        def grp_flops(grp):
            return sum(call_flops(M, *shapes[f], 0 if f in dense_fams else R) for f in grp)

        step_bytes = sum(grp_bytes(c[1]) for c in calls)
        step_flops = sum(grp_flops(c[1]) for c in calls)
        decode = M <= DECODE_MAX_TOKENS

        def rate(ms):
            return step_bytes / (ms * 1e-3) / 1e9 if decode else step_flops / (ms * 1e-3) / 1e12

        for k in range(warmup):
            run(pool_calls[k % replicas])
        torch.cuda.synchronize()
        t_prep = time.time() - t0

        # ---- timed region: K steps, rotating over the pool (one replica: plain stack order) ----
        ms, per_step = timed_steps(torch, lambda k: run(pool_calls[k % replicas]), steps)
        if tb.workspace_error_word() != 0:
            raise RuntimeError("a bounded wait in the projection kernel timed out")
        effective = None
        if replicas > 1:      # the stack from one replica: the cache-assisted stack-order figure
            ms_eff, per_eff = timed_steps(torch, lambda k: run(calls), steps)
            effective = {"value": round(rate(ms_eff), 3), "ms_per_step": round(ms_eff, 4), **spread(per_eff)}

        # ---- the same step replayed from a captured graph ----------------------------
        graph = None
        if with_graph:
            def make_step(handle):
                c = build_calls(handle, pools[0])
                return lambda: run(c)
            g_ms, g_per, clocks = graph_leg(torch, make_step, steps, list(ys.values()))
            graph = {"value": round(rate(g_ms), 3), "ms_per_step": round(g_ms, 4), **spread(g_per),
                     "pool": "replica 0", "gpu": clocks}
            if tb.workspace_error_word() != 0:
                raise RuntimeError("a bounded wait in the projection kernel timed out")

        # ---- roofline of the dominant kernel ---------------------------------------
        # The timed region holds nothing but the launches of the projection calls
        # (decode: one decode_kernel launch per call; prefill: x . V then the GEMM per
        # call), so its duration over the launch count is the average duration per
        # call, gaps between launches included (an upper bound; the committed
        # rocprofv3 kernel trace of the same command gives the kernel time alone).
        per_call_us = ms * 1e3 / len(calls)
        launch_bytes = float(np.mean([grp_bytes(c[1]) for c in calls]))
        launch_flops = float(np.mean([grp_flops(c[1]) for c in calls]))
        nt = 1 if M <= 16 else (2 if M <= 32 else 4)
        tag = f"{args.workload}_M{M}_G{G}" + ("" if R == wl["rank"] else f"_R{R}")
        if decode:
            kernel = f"decode_kernel<bf16,{nt},*>"
            achieved = launch_bytes / (per_call_us * 1e-6) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "kernel": kernel, "launches_per_call": 1}
            per_launch = launch_bytes
        else:
            kernel = "big::gemm_kernel" if R == 0 or dense_fams == set(gen.FAMILIES) else \
                "xv::xv_kernel + big::gemm_kernel"
            achieved = launch_flops / (per_call_us * 1e-6) / 1e12
            roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "kernel": kernel,
                    "launches_per_call": 1 if "+" not in kernel else 2}
            per_launch = launch_flops
        roof["calls_per_step"] = len(calls)
        roof["avg_call_us"] = round(per_call_us, 2)
        roof["algorithmic_per_call"] = round(per_launch, 1)
        roof["traffic"] = counter_traffic(kernel, tag) if replicas == 1 and dense is None else None
        prof = profile_durations(tag)
        if prof is not None:
            roof["profile"] = {**prof, "frac_from_profile": round(
                (launch_bytes / (prof["avg_call_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS) if decode else
                (launch_flops / (prof["avg_call_us"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS), 4)}

        cpu = None
        if with_cpu and dense is None:
            cpu = cpu_baseline_forward(cpu_seconds, wl, shapes, calls, bundles, W0, xs, band_of, decode, M, R)

        out = {
            "value": round(rate(ms), 2 if decode else 3),
            "unit": "GB/s" if decode else "TFLOP/s",
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": round(ms, 4),
            "tokens": M,
            "step_bytes": step_bytes,
            "step_flops": step_flops,
            "trials": spread(per_step),
            "effective_one_replica": effective,
            "graph": graph,
            "roofline": roof,
            "cpu_baseline": cpu,
        }
        print(f"# M={M}: inputs and warm-up {t_prep:.1f}s  step {ms:.3f} ms  {out['value']} {out['unit']}",
              file=sys.stderr, flush=True)
        del xs, ys, pool_calls, calls
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return out

    leg = time_stack(M, args.steps, args.warmup, not args.no_graph, not args.no_cpu_baseline, args.cpu_seconds)
    prefill = None
    pm = wl.get("prefill", 0) if args.prefill_tokens is None else args.prefill_tokens
    if pm and M <= DECODE_MAX_TOKENS:
        prefill = time_stack(pm, args.prefill_steps, 2, False, not args.no_cpu_baseline, args.cpu_seconds / 2)
        prefill["config"] = f"{args.workload}: the same resident stack at {pm} tokens (matrix-core-bound)"

    line = {
        "metric": METRIC,
        "value": leg["value"],
        "unit": leg["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": leg["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {L}-layer stack, 7 projections per layer, rank {R}, "
                               f"G={G} bands, {M} tokens"
                               + (", materialised once (dense bf16 weights)" if args.materialised else
                                  ", tie_families=attn (MLP dense)" if dense_fams else ""),
                   "materialised": args.materialised, "tie_families": args.tie_families,
                   "layers": L, "projections_per_step": L * len(gen.FAMILIES),
                   "grouping": "+".join(",".join(f.split("_")[0] for f in g) for g in groups),
                   "rank": R, "bands": G, "tokens": M,
                   "hidden": shapes["q_proj"][1], "mlp": shapes["gate_proj"][0],
                   "step_bytes": leg["step_bytes"], "step_flops": leg["step_flops"], "distinct_input_bytes": distinct,
                   "replicas": replicas, "parallelism": "single-gpu"},
        "trials": leg["trials"],
        "effective_one_replica": leg["effective_one_replica"],
        "graph": leg["graph"],
        "roofline": leg["roofline"],
        "cpu_baseline": leg["cpu_baseline"],
        "prefill": prefill,
    }
    print(f"# setup {t_setup:.1f}s  step {leg['ms_per_step']:.3f} ms", file=sys.stderr)
    print(json.dumps(line), flush=True)


def cpu_baseline_forward(cpu_seconds, wl, shapes, calls, bundles, W0, xs, band_of, decode, M, R):
    """Time the float64 oracle on the first projections of the same stack (prefill: a 256-token slice of each,
    whose flops scale linearly to the whole token count)."""
    import numpy as np
    import torch

    import oracle

    Mc = M if decode else min(M, 256)       # prefill: a token slice keeps it bounded
    done_bytes, done_flops, secs, used = 0, 0, 0.0, []
    for l, fam in ((c[0], f) for c in calls for f in c[1]):
        if secs > cpu_seconds:
            break
        O, I = shapes[fam]
        bd = bundles[(l, fam)]
        host = dict(x=_bits(torch, np, xs[(l, fam)][:Mc]), s=_bits(torch, np, bd["s"]),
                    W0=_bits(torch, np, W0[(band_of[l], fam)]))
        if R:
            host["U"], host["V"] = _bits(torch, np, bd["U"]), _bits(torch, np, bd["V"])
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
    step_units = sum(call_bytes(M, *shapes[f], R) if decode else call_flops(M, *shapes[f], R)
                     for c in calls for f in c[1])
    return {"value": round(val, 4), "unit": unit, "cores": int(_blas_threads()), "kind": "oracle",
            "sample": f"{len(used)} projections of the same stack ({used[0]} .. {used[-1]}), {Mc} tokens, "
                      f"float64 NumPy incl. bf16 decoding, {secs:.1f} s",
            "extrapolated_step_s": round(step_units / (val * (1e9 if decode else 1e12)), 2), **_host_info()}


# ---- reconstruction and error stack -------------------------------------------------------


def bench_reconstruct(args, torch, np, tb, gen):
    wl = dict(WORKLOADS["reconstruct60"])
    if args.bands is not None:
        wl["bands"] = args.bands
    if args.rank is not None:
        wl["rank"] = args.rank
    L, R, G = wl["layers"], wl["rank"], wl["bands"]
    shapes = getattr(gen, wl["shapes"])
    seed = wl["seed"]
    nfam = len(gen.FAMILIES)
    t_setup = time.time()
    band_of = []
    for l in range(L):
        b = ctypes.c_int32()
        assert tb.lib.tb_band_index(L, G, l, ctypes.byref(b)) == 0
        band_of.append(b.value)
    W0 = {(b, fam): gen.device_w0(torch, seed, fam, shapes, b) for b in range(G) for fam in gen.FAMILIES}
    bundles, originals = {}, {}
    for l in range(L):
        for fam in gen.FAMILIES:
            bd = gen.device_bundle(torch, seed, fam, shapes, l, band_of[l], R, with_w0=False)
            if R == 0:
                bd["U"] = bd["V"] = None
            bundles[(l, fam)] = bd
            originals[(l, fam)] = gen.device_original(torch, W0[(band_of[l], fam)], seed, fam, l)
    rebuilt = {} if args.fused else {fam: torch.empty(shapes[fam], dtype=torch.float32, device="cuda")
                                     for fam in gen.FAMILIES}
    errors = torch.zeros(L * nfam, dtype=torch.float64, device="cuda")
    fws = torch.zeros(tb.FROBENIUS_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    rec = tb.lib.tb_reconstruct_weight
    frob = tb.lib.tb_rel_frobenius_error
    rerr = tb.lib.tb_reconstruction_error
    fused = args.fused

    def build_calls(stream_handle):
        stream = ctypes.c_void_p(stream_handle)
        calls = []   # (kind, family, function, argument tuple)
        for l in range(L):
            for j, fam in enumerate(gen.FAMILIES):
                O, I = shapes[fam]
                bd = bundles[(l, fam)]
                if fused:
                    calls.append(("fused", fam, rerr,
                                  (bd["s"].data_ptr(), W0[(band_of[l], fam)].data_ptr(),
                                   bd["U"].data_ptr() if R else None, bd["V"].data_ptr() if R else None,
                                   originals[(l, fam)].data_ptr(), O, I, R, tb.TB_BF16, tb.TB_F32,
                                   errors.data_ptr() + 8 * (l * nfam + j), fws.data_ptr(), fws.numel(), stream)))
                    continue
                w = rebuilt[fam]
                calls.append(("reconstruct", fam, rec,
                              (bd["s"].data_ptr(), W0[(band_of[l], fam)].data_ptr(),
                               bd["U"].data_ptr() if R else None, bd["V"].data_ptr() if R else None, w.data_ptr(),
                               O, I, R, tb.TB_BF16, tb.TB_F32, stream)))
                calls.append(("frobenius", fam, frob,
                              (originals[(l, fam)].data_ptr(), w.data_ptr(), O, I, tb.TB_F32,
                               errors.data_ptr() + 8 * (l * nfam + j), fws.data_ptr(), fws.numel(), stream)))
        return calls

    band_idx = tb.lib.tb_band_index
    bout = ctypes.c_int32()
    per_layer = (1 if fused else 2) * nfam

    def run(calls, events=None):
        n = 0
        for l in range(L):
            band_idx(L, G, l, ctypes.byref(bout))          # band select (host)
            for _ in range(per_layer):
                if events is not None:
                    events[n].record()
                st = calls[n][2](*calls[n][3])
                if st:
                    raise RuntimeError(tb.lib.tb_last_error().decode())
                n += 1
        if events is not None:
            events[n].record()

    calls = build_calls(torch.cuda.current_stream().cuda_stream)
    nbytes = np.array([reconstruct_bytes(*shapes[c[1]], R) if c[0] == "reconstruct" else
                       fused_error_bytes(*shapes[c[1]], R) if c[0] == "fused" else
                       frobenius_bytes(*shapes[c[1]]) for c in calls], dtype=np.float64)
    step_bytes = float(nbytes.sum())
    step_flops = sum(2 * shapes[c[1]][0] * shapes[c[1]][1] * R for c in calls if c[0] in ("reconstruct", "fused"))

    for _ in range(args.warmup):
        run(calls)
    torch.cuda.synchronize()
    ms, per_step = timed_steps(torch, lambda k: run(calls), args.steps)
    err_host = errors.cpu().numpy()

    per_call_ms = np.zeros(len(calls))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
    for _ in range(args.steps):
        run(calls, ev)
        torch.cuda.synchronize()
        per_call_ms += np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(len(calls))])
    per_call_ms /= args.steps

    graph = None
    if not args.no_graph:
        def make_step(handle):
            c = build_calls(handle)
            return lambda: run(c)
        g_ms, g_per, clocks = graph_leg(torch, make_step, args.steps,
                                        [errors] + ([] if fused else list(rebuilt.values())))
        graph = {"value": round(step_bytes / (g_ms * 1e-3) / 1e9, 2), "ms_per_step": round(g_ms, 4),
                 **spread(g_per), "gpu": clocks}

    kernels = {}
    rec_kernel, fused_kernel = reconstruct_kernel_names(R)
    kinds = (("fused", fused_kernel),) if fused else (("reconstruct", rec_kernel), ("frobenius", "frob_kernel"))
    for kind, name in kinds:
        sel = np.array([c[0] == kind for c in calls])
        t = float(per_call_ms[sel].sum())
        gbs = float(nbytes[sel].sum()) / (t * 1e-3) / 1e9
        kernels[kind] = {"kernel": name, "ms_per_step": round(t, 4), "achieved": round(gbs, 1),
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_per_launch": round(float(nbytes[sel].mean()), 1)}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    roof = {"bound": "hbm", "achieved": kernels[dom]["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": kernels[dom]["frac"], "kernel": kernels[dom]["kernel"], "calls_per_step": L * nfam,
            "avg_launch_us": round(kernels[dom]["ms_per_step"] * 1e3 / (L * nfam), 2),
            "algorithmic_per_launch": kernels[dom]["algorithmic_per_launch"],
            "traffic": counter_traffic(kernels[dom]["kernel"], f"reconstruct60_R{R}_G{G}{'_fused' if fused else ''}"),
            "kernels": kernels}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_reconstruct(args, shapes, bundles, W0, originals, band_of, L, R, gen, fused)

    line = {
        "metric": METRIC,
        "value": round(step_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->f32",
        "data": "synthetic",
        "config": {"workload": f"reconstruct60: {L}-layer stack, 7 projections per layer, rank {R}, G={G} bands, "
                               + ("error against the originals without writing the rebuilt weight" if fused else
                                  "rebuilt in fp32 and compared with the originals"),
                   "fused": fused,
                   "layers": L, "rank": R, "bands": G, "pairs_per_step": L * nfam,
                   "step_bytes": step_bytes, "step_flops": step_flops, "parallelism": "single-gpu",
                   "mean_rel_error": float(err_host.mean()), "max_rel_error": float(err_host.max())},
        "trials": spread(per_step),
        "graph": graph,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(f"# setup {t_setup:.1f}s  step {ms:.3f} ms  per-launch sum {per_call_ms.sum():.3f} ms", file=sys.stderr)
    print(json.dumps(line), flush=True)


def cpu_baseline_reconstruct(args, shapes, bundles, W0, originals, band_of, L, R, gen, fused=False):
    """Time the float64 oracle's reconstruct + error on the first (layer, projection) pairs of the stack."""
    import numpy as np
    import torch

    import oracle

    done_bytes, secs, used = 0, 0.0, []
    for l, fam in ((l, f) for l in range(L) for f in gen.FAMILIES):
        if secs > args.cpu_seconds:
            break
        O, I = shapes[fam]
        bd = bundles[(l, fam)]
        s_bits, w0_bits = _bits(torch, np, bd["s"]), _bits(torch, np, W0[(band_of[l], fam)])
        u_bits = _bits(torch, np, bd["U"]) if R else None
        v_bits = _bits(torch, np, bd["V"]) if R else None
        orig = originals[(l, fam)].cpu().numpy()
        t = time.perf_counter()
        s, w0 = oracle.bf16_bits_to_f64(s_bits), oracle.bf16_bits_to_f64(w0_bits)
        U = oracle.bf16_bits_to_f64(u_bits) if R else np.zeros((O, 0))
        V = oracle.bf16_bits_to_f64(v_bits) if R else np.zeros((I, 0))
        oracle.relative_frobenius_error(orig, oracle.reconstruct_weight(s, w0, U, V))
        secs += time.perf_counter() - t
        done_bytes += fused_error_bytes(O, I, R) if fused else reconstruct_bytes(O, I, R) + frobenius_bytes(O, I)
        used.append(f"{l}:{fam}")
    rate = done_bytes / secs
    step = L * sum(fused_error_bytes(o, i, R) if fused else reconstruct_bytes(o, i, R) + frobenius_bytes(o, i)
                   for o, i in shapes.values())
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": int(_blas_threads()),
            "kind": "oracle",
            "sample": f"{len(used)} (layer, projection) pairs of the same stack ({used[0]} .. {used[-1]}): "
                      f"float64 NumPy reconstruct incl. bf16 decoding, then the error, {secs:.1f} s",
            "extrapolated_step_s": round(step / rate, 1), **_host_info()}


def bench_decompose(args, torch, np, tb, gen):
    """The analytic decomposition of a whole stack on the GPU: every family's band means, row scales and
    randomized low-rank factors (tb_shared_block, tb_row_scale, tb_lowrank_factors through decompose())."""
    wl = dict(WORKLOADS[args.workload])
    if args.bands is not None:
        wl["bands"] = args.bands
    if args.rank is not None:
        wl["rank"] = args.rank
    L, R, G, seed = wl["layers"], wl["rank"], wl["bands"], wl["seed"]
    shapes = getattr(gen, wl["shapes"])
    t_setup = time.time()
    band_of = [tb.band_index(L, G, l) for l in range(L)]
    # Originals: a_l * W0_band + N(0, 2e-3) in bf16 (the reconstruction workload's recipe).
    originals = {}
    for fam in gen.FAMILIES:
        blocks = {b: gen.device_w0(torch, seed, fam, shapes, b) for b in set(band_of)}
        originals[fam] = [gen.device_original(torch, blocks[band_of[l]], seed, fam, l).to(torch.bfloat16)
                          for l in range(L)]
        del blocks
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup
    orig_bytes = sum(t.numel() * t.element_size() for ts in originals.values() for t in ts)
    ks = {fam: min(R + 16, *shapes[fam]) for fam in gen.FAMILIES}
    q = args.power_iters
    gemm_flops = L * sum(2 * (2 + 2 * q) * shapes[f][0] * shapes[f][1] * ks[f] +
                         2 * (shapes[f][0] + shapes[f][1]) * ks[f] * R for f in gen.FAMILIES)

    def step(keep=False):
        out = {}
        for fam in gen.FAMILIES:
            out[fam] = tb.decompose(originals[fam], G, R, power_iters=q, seed=seed)
            if not keep:
                out[fam] = None
        return out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, per_step = timed_steps(torch, lambda k: step(), args.steps)
    # Quality of the last decomposition (the (G, rank) sweep's figure for this synthetic stack).
    bundles = step(keep=True)
    errs = []
    for fam in gen.FAMILIES:
        b = bundles[fam]
        for l in range(L):
            e = tb.reconstruction_error(originals[fam][l], b["s"][l], b["W0"][b["band"][l]], b["U"][l], b["V"][l])
            errs.append(float(e.item()))
    del bundles
    als = None
    if args.als_iters > 0:
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        refined = {fam: tb.als_decompose(originals[fam], G, R, args.als_iters, power_iters=q, seed=seed)
                   for fam in gen.FAMILIES}
        ev[1].record()
        torch.cuda.synchronize()
        als_errs = [float(tb.reconstruction_error(originals[fam][l], b["s"][l], b["W0"][b["band"][l]], b["U"][l],
                                                  b["V"][l]).item())
                    for fam, b in refined.items() for l in range(L)]
        als = {"iters": args.als_iters, "ms_incl_decomposition": round(ev[0].elapsed_time(ev[1]), 1),
               "mean_rel_error": float(np.mean(als_errs))}
        del refined
    value = orig_bytes / (ms * 1e-3) / 1e9
    achieved = gemm_flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "analytic decomposition of a stack (band means, row scales, randomized low-rank factors)",
        "value": round(value, 2),
        "unit": "GB/s of original bf16 weights",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32 (f64 solvers)",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {L}-layer stack, 7 families, G={G}, rank {R}, "
                               f"k = rank + 16, {q} power iterations, each band's layers batched",
                   "layers": L, "bands": G, "rank": R, "power_iters": q,
                   "matrices": L * len(gen.FAMILIES), "original_bytes": orig_bytes,
                   "matrices_per_s": round(L * len(gen.FAMILIES) / (ms * 1e-3), 2),
                   "mean_rel_error": float(np.mean(errs)), "als": als, "parallelism": "single-gpu"},
        "trials": spread(per_step),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / FP32_PEAK_TFLOPS, 4), "traffic": None,
                     "note": "fp32 GEMM work of the randomized SVDs over the whole step; the fp64 "
                             "single-workgroup solvers (Jacobi, Cholesky) take most of the rest"},
        "cpu_baseline": None,
    }
    print(f"# setup {t_setup:.1f}s  step {ms:.1f} ms", file=sys.stderr)
    print(json.dumps(line), flush=True)


def bench_tiny(args, torch, np, tb, gen):
    """The tiny fp32 stack: 4 layers, G = 2, one 512 -> 256 projection per layer, rank 16, 8 tokens.  Its
    bundle comes from the GPU decomposition of the workload's weights (setup, untimed); a step is the four
    layers' band select and tb_linear_forward (fp32).  Bound by launch latency, not by HBM: the figure is
    reported with its time per call."""
    wl = dict(WORKLOADS["tiny4"])
    L, R, G = wl["layers"], wl["rank"], wl["bands"]
    M = wl["tokens"] if args.tokens is None else args.tokens
    weights, x_host = gen.tiny_stack(wl["seed"])
    O, I = weights[0].shape
    dev = "cuda"
    t_setup = time.time()
    wd = [torch.from_numpy(w.astype(np.float32)).to(dev) for w in weights]
    bun = tb.decompose(wd, G, R, seed=wl["seed"])
    xs = np.resize(x_host, (M, I)) if M != x_host.shape[0] else x_host
    x = torch.from_numpy(xs.astype(np.float32)).to(dev)
    y = torch.empty((M, O), dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t(0)
    assert tb.lib.tb_linear_forward_workspace_size(M, O, I, R, tb.TB_F32, ctypes.byref(nb)) == 0
    ws = tb.workspace_for(nb.value)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup
    fwd, band_idx, bout = tb.lib.tb_linear_forward, tb.lib.tb_band_index, ctypes.c_int32()

    def build_calls(handle):
        stream = ctypes.c_void_p(handle)
        return [(x.data_ptr(), bun["s"][l].data_ptr(), bun["W0"][bun["band"][l]].data_ptr(), bun["U"][l].data_ptr(),
                 bun["V"][l].data_ptr(), y.data_ptr(), M, O, I, R, tb.TB_F32, ws.data_ptr(), ws.numel(), stream)
                for l in range(L)]

    def make_step(handle):
        calls = build_calls(handle)

        def run():
            for l in range(L):
                band_idx(L, G, l, ctypes.byref(bout))
                if fwd(*calls[l]):
                    raise RuntimeError(tb.lib.tb_last_error().decode())
        return run

    step = make_step(torch.cuda.current_stream().cuda_stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, per_step = timed_steps(torch, lambda k: step(), args.steps)
    if tb.workspace_error_word() != 0:
        raise RuntimeError("a bounded wait in the projection kernel timed out")
    graph = None
    if not args.no_graph:
        g_ms, g_per, clocks = graph_leg(torch, make_step, args.steps, [y])
        graph = {"ms_per_step": round(g_ms, 5), **spread(g_per), "gpu": clocks,
                 "value": round(L * call_bytes(M, O, I, R, e=4) / (g_ms * 1e-3) / 1e9, 3)}
    step_bytes = L * call_bytes(M, O, I, R, e=4)
    value = step_bytes / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        host = [{k: bun[k][l].cpu().numpy().astype(np.float64) for k in ("s", "U", "V")} for l in range(L)]
        w0h = [t.cpu().numpy().astype(np.float64) for t in bun["W0"]]
        x64 = xs.astype(np.float64)
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 2.0):
            for l in range(L):
                oracle.forward(x64, host[l]["s"], w0h[bun["band"][l]], host[l]["U"], host[l]["V"])
            n += 1
        secs = time.perf_counter() - t0
        cpu = {"value": round(n * step_bytes / secs / 1e9, 4), "unit": "GB/s", "cores": int(_blas_threads()),
               "kind": "oracle", "sample": f"the whole 4-layer step, {n} times, float64 NumPy, {secs:.1f} s",
               "ms_per_step": round(secs / n * 1e3, 4), **_host_info()}
    line = {
        "metric": "theta-bundle projection TFLOP/s (prefill M) and GB/s (decode M), % of roofline",
        "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"tiny4: 4 layers, G={G}, one {I}->{O} projection per layer, rank {R}, {M} tokens, "
                               "fp32, bundle from the GPU decomposition",
                   "layers": L, "bands": G, "rank": R, "tokens": M, "step_bytes": step_bytes,
                   "us_per_call": round(ms * 1e3 / L, 2), "parallelism": "single-gpu"},
        "trials": spread(per_step),
        "graph": graph,
        "roofline": {"bound": "hbm", "achieved": round(value, 3), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(value / 8000.0, 5), "traffic": None,
                     "kernel": "decode_kernel<float,1,*>", "launches_per_call": 1, "calls_per_step": L,
                     "note": "0.6 MB per call: launch latency bounds it, not HBM"},
        "cpu_baseline": cpu,
    }
    prof = profile_durations(f"tiny4_M{M}_G{G}")
    if prof is not None:
        per_call = call_bytes(M, O, I, R, e=4)
        line["roofline"]["profile"] = {**prof, "frac_from_profile": round(
            per_call / (prof["avg_call_us"] * 1e-6) / 1e9 / 8000.0, 5)}
    print(f"# setup {t_setup:.1f}s  step {ms:.4f} ms", file=sys.stderr)
    print(json.dumps(line), flush=True)


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

    torch.cuda.set_device(0)
    if args.workload == "reconstruct60":
        bench_reconstruct(args, torch, np, tb, gen)
    elif args.workload.startswith("decompose"):
        bench_decompose(args, torch, np, tb, gen)
    elif args.workload == "tiny4":
        bench_tiny(args, torch, np, tb, gen)
    else:
        bench_forward(args, torch, np, tb, gen)


if __name__ == "__main__":
    main()
