#!/usr/bin/env python3
"""Throughput of the local MoE forward (route -> dispatch -> SwiGLU experts -> combine) on one
MI355X, through the C ABI of librudnn_moe.so.

One step = one ``rudnn_moe_forward`` over one batch of the Mixtral-shaped layer (T=4096 tokens,
H=4096, I=14336, E=8, top_k=2, renormalised, bf16), all inputs resident in HBM.  Prints one
JSON line with tokens/s, the roofline of the dominant kernel (the gate/up expert GEMM, timed
with HIP events on its launch stream during the timed steps), a per-kernel breakdown, the HBM
rates of route / dispatch / combine on the routing+dispatch workload (T=65536, E=128, k=8,
H=2048, bf16, identity experts), the forward of the decode-shaped, skewed and tiny layers
(`forward_other`, not part of `value`), the fused gate projection + routing on the same token
shapes, and the CPU oracle timed on a bounded sample of the same layer.  HBM-bound stages start from a
cold cache: 512 MiB are read (not written) before each timed launch, so that the caches hold
neither the inputs nor dirty lines whose write-back would land in the timed kernel.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s (1 GPU); expert-GEMM MFMA %; route/dispatch/combine GB/s"
HBM_PEAK_GBS = 8000.0                     # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}  # dense; fp32 = vector FMA peak
DTYPE_BYTES = {"bf16": 2, "f16": 2, "f32": 4}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["mixture_experts_layer_23_amd/csrc/experts.hip", "mixture_experts_layer_23_amd/csrc/device.hpp",
                  "mixture_experts_layer_23_amd/csrc/internal.hpp"]



def _cpu_model() -> str:
    """The host CPU's model name as /proc/cpuinfo gives it (empty when unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""

def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Hip:
    """HIP events through the runtime torch already loaded (same soname as the library's)."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so.7")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.L.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        self.L.hipEventSynchronize(b)
        v = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(v), a, b) == 0
        return float(v.value)

    def ms_if_recorded(self, a, b):
        """Elapsed time, or None when the pair was never recorded (its kernel did not launch)."""
        self.L.hipEventSynchronize(b)
        v = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(v), a, b) != 0:
            self.L.hipGetLastError()  # the failed query must not leave an error for the next HIP call
            return None
        return float(v.value)


class ProfilerRegion:
    """roctx marks around the timed steps: a range named ``bench timed steps`` (under
    ``rocprofv3 --marker-trace`` the kernels that run inside it are exactly the timed launches)
    and resume/pause for ``--selected-regions``.  Outside rocprofv3 these calls do nothing."""

    NAME = b"bench timed steps"

    def __init__(self):
        try:
            self.L = ctypes.CDLL("librocprofiler-sdk-roctx.so.1")
            self.L.roctxProfilerResume.argtypes = [ctypes.c_uint64]
            self.L.roctxProfilerPause.argtypes = [ctypes.c_uint64]
            self.L.roctxRangePushA.argtypes = [ctypes.c_char_p]
        except (OSError, AttributeError):
            self.L = None

    def resume(self):
        if self.L is not None:
            self.L.roctxProfilerResume(0)
            self.L.roctxRangePushA(self.NAME)

    def pause(self):
        if self.L is not None:
            self.L.roctxRangePop()
            self.L.roctxProfilerPause(0)


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed PMC summary, if taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    ent = d.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_sha256") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target CPU time of the oracle baseline sample (sized from 8- and 64-token probes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-stages", action="store_true")
    ap.add_argument("--no-sigmoid", action="store_true",
                    help="skip the group-limited sigmoid routing measurements")
    ap.add_argument("--no-projection", action="store_true",
                    help="skip the fused gate projection + routing measurements")
    ap.add_argument("--no-training", action="store_true",
                    help="skip the first-order training (backward chain) measurements")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the forward of the decode-shaped, skewed and tiny layers")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (scale for FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library is a single-GPU local MoE forward with no "
              "multi-GPU path, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixture_experts_layer_23_amd import moe
    from mixture_experts_layer_23_amd.inputs import WORKLOADS, make_experts, make_logits, make_tokens

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = Hip()
    stream = torch.cuda.current_stream(dev).cuda_stream
    flush_buf, flush_sink = None, None

    def flush():
        """Evict the caches by reading 512 MiB (2x the 256 MB Infinity Cache); no dirty lines."""
        nonlocal flush_buf, flush_sink
        if flush_buf is None:
            flush_buf = torch.ones(64 << 20, dtype=torch.int64, device=dev)
            flush_sink = torch.zeros((), dtype=torch.int64, device=dev)
        torch.sum(flush_buf, dim=0, out=flush_sink)

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    moe.lib()

    # ---------------- the Mixtral-shaped layer ----------------
    w = WORKLOADS["mixtral"]
    renorm = w.renormalize[0]
    log("generating", w.name)
    logits_cpu, _ = make_logits(w)
    logits = logits_cpu.to(dev)
    x = make_tokens(w, dev)
    gate, up, down = make_experts(w, dev)
    ex = moe.SwiGluExperts(gate, up, down)
    out = torch.empty_like(x)
    ws = torch.empty(moe.forward_workspace_size(ex, w.T, w.top_k, logits.dtype), dtype=torch.uint8, device=dev)

    def step():
        ex.forward(x, logits, w.top_k, renorm, out=out, workspace=ws)

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps back to back; HIP events around every gate/up GEMM launch and around
    # its split-K reduce (the epilogue of the K-split tail tiles), when that launches
    K = args.steps
    gu_ev = [(hip.event(), hip.event()) for _ in range(K)]
    gur_ev = [(hip.event(), hip.event()) for _ in range(K)]
    t_start, t_stop = hip.event(), hip.event()
    region = ProfilerRegion()
    torch.cuda.synchronize()
    region.resume()
    wall0 = time.perf_counter()
    hip.record(t_start, stream)
    for i in range(K):
        moe.time_next_launch("experts_gate_up", *gu_ev[i])
        moe.time_next_launch("experts_gate_up_reduce", *gur_ev[i])
        step()
        moe.time_next_launch("experts_gate_up_reduce", None, None)  # clear it if it did not launch
    hip.record(t_stop, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    region.pause()
    ms_total = hip.ms(t_start, t_stop)
    ms_per_step = ms_total / K
    tokens_per_s = w.T / (ms_per_step / 1e3)
    gu_main_ms = float(np.mean([hip.ms(a, b) for a, b in gu_ev]))
    gur = [hip.ms_if_recorded(a, b) for a, b in gur_ev]
    gu_reduce_ms = float(np.mean([v for v in gur if v is not None])) if any(v is not None for v in gur) else 0.0
    gu_ms = gu_main_ms + gu_reduce_ms
    log(f"{K} steps: {ms_per_step:.3f} ms/step (host wall {wall / K * 1e3:.3f} ms), gate/up {gu_ms:.3f} ms")

    T, H, I, E, k = w.T, w.H, w.I, w.E, w.top_k
    s = 2
    gu_flops = 4.0 * T * k * H * I
    dn_flops = 2.0 * T * k * H * I
    gu_tflops = gu_flops / (gu_ms / 1e3) / 1e12

    # per-kernel breakdown (separate pass, every kernel timed)
    # what the softmax forward with ready logits launches
    fwd_kernels = ["route", "dispatch_count", "dispatch_scan", "dispatch_copy", "experts_plan",
                   "experts_gate_up", "experts_down", "combine", "experts_gate_up_reduce", "experts_down_reduce"]
    stage_ev = {kn: [(hip.event(), hip.event()) for _ in range(max(3, K // 4))] for kn in fwd_kernels}
    for i in range(max(3, K // 4)):
        for kn in fwd_kernels:
            moe.time_next_launch(kn, *stage_ev[kn][i])
        step()
        for kn in fwd_kernels:  # a kernel this layer does not launch leaves its pair unrecorded
            moe.time_next_launch(kn, None, None)
    torch.cuda.synchronize()

    def mean_recorded(pairs):
        v = [hip.ms_if_recorded(a, b) for a, b in pairs]
        v = [x for x in v if x is not None]
        return float(np.mean(v)) if v else 0.0

    stage_ms = {kn: mean_recorded(v) for kn, v in stage_ev.items()}
    dispatch_bytes = T * k * 4 * 2 + T * H * s + T * k * H * s + T * k * 4 + 4 * (E + 1)
    stages = {
        "route": {"us": stage_ms["route"] * 1e3, "bytes": T * E * s + T * k * (4 + s)},
        "dispatch": {"us": sum(stage_ms[f"dispatch_{p}"] for p in ("count", "scan", "copy")) * 1e3,
                     "bytes": dispatch_bytes},
        "experts_gate_up": {"us": stage_ms["experts_gate_up"] * 1e3, "flops": gu_flops},
        "experts_down": {"us": stage_ms["experts_down"] * 1e3, "flops": dn_flops},
        "experts_plan": {"us": stage_ms["experts_plan"] * 1e3},
        "experts_split_reduce": {"us": (stage_ms["experts_gate_up_reduce"] + stage_ms["experts_down_reduce"]) * 1e3},
        "combine": {"us": stage_ms["combine"] * 1e3, "bytes": T * k * H * s + T * k * (s + 4) + T * H * s},
    }
    for v in stages.values():
        if "bytes" in v:
            v["GBps"] = v["bytes"] / (v["us"] / 1e6) / 1e9
            v["hbm_frac"] = v["GBps"] / HBM_PEAK_GBS
        if "flops" in v:
            v["TFLOPps"] = v["flops"] / (v["us"] / 1e6) / 1e12
            v["mfma_frac"] = v["TFLOPps"] / MFMA_PEAK_TFLOPS[w.dtype]
    experts_us = sum(stages[n]["us"] for n in ("experts_gate_up", "experts_down", "experts_plan", "experts_split_reduce"))
    stages["experts_total"] = {"us": experts_us, "TFLOPps": (gu_flops + dn_flops) / (experts_us / 1e6) / 1e12}
    stages["experts_total"]["mfma_frac"] = stages["experts_total"]["TFLOPps"] / MFMA_PEAK_TFLOPS[w.dtype]

    # ---------------- CPU oracle on a bounded sample of the same layer ----------------
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle
        g_c, u_c, d_c = gate.cpu(), up.cpu(), down.cpu()
        x_c = x.cpu()
        # two probes give a fixed cost (weight rows decoded once per block) and a cost per token
        times = {}
        for probe in (8, 64):
            t0 = time.perf_counter()
            oracle.forward(x_c[:probe], logits_cpu[:probe], k, renorm, g_c, u_c, d_c)
            times[probe] = time.perf_counter() - t0
        per_token = max((times[64] - times[8]) / 56, 1e-6)
        fixed = max(times[8] - 8 * per_token, 0.0)
        n = int(min(T, max(64, (args.cpu_seconds - fixed) / per_token)))
        log(f"cpu baseline: {n} tokens through the oracle (probes: {per_token * 1e3:.2f} ms/token + {fixed:.2f} s)")
        t0 = time.perf_counter()
        oracle.forward(x_c[:n], logits_cpu[:n], k, renorm, g_c, u_c, d_c)
        dt = time.perf_counter() - t0
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "cpu_model": _cpu_model(),
               "sample": f"first {n} of the {T} tokens of the Mixtral-shaped layer, whole forward "
                         f"(route, dispatch, SwiGLU experts, combine) in the fp64 oracle; {dt:.1f} s"}
        del g_c, u_c, d_c, x_c

    # ---------------- HBM-bound stages on the routing+dispatch workload ----------------
    hbm = None
    if not args.no_hbm_stages:
        del ws, out
        torch.cuda.empty_cache()
        w2 = WORKLOADS["route_dispatch"]
        log("generating", w2.name)
        lg2_cpu, _ = make_logits(w2)
        lg2 = lg2_cpu.to(dev)
        x2 = make_tokens(w2, dev)
        T2, E2, k2, H2 = w2.T, w2.E, w2.top_k, w2.H
        idx2 = torch.empty(T2, k2, dtype=torch.int32, device=dev)
        wt2 = torch.empty(T2, k2, dtype=lg2.dtype, device=dev)
        d2 = moe.Dispatched(torch.empty(T2 * k2, H2, dtype=x2.dtype, device=dev),
                            torch.empty(E2 + 1, dtype=torch.int32, device=dev),
                            torch.empty(T2, k2, dtype=torch.int32, device=dev))
        dws = torch.empty(max(moe.lib().rudnn_moe_dispatch_workspace_size(T2, k2, E2), 1), dtype=torch.uint8,
                          device=dev)
        o2 = torch.empty_like(x2)
        reps = 5
        ev = {n_: [(hip.event(), hip.event()) for _ in range(reps)] for n_ in ("route", "dispatch", "combine")}
        for i in range(reps + 1):
            rec = i > 0
            for name, fn in (("route", lambda: moe.lib().rudnn_moe_route(
                                 lg2.data_ptr(), 2, T2, E2, moe.RoutingOptions(k2, 1), idx2.data_ptr(), wt2.data_ptr(),
                                 stream)),
                             ("dispatch", lambda: moe.dispatch(idx2, x2, E2, out=d2, workspace=dws)),
                             ("combine", lambda: moe.combine(d2.dispatched, d2.token_map, wt2, out=o2))):
                flush()
                if rec:
                    hip.record(ev[name][i - 1][0], stream)
                rc = fn()
                if isinstance(rc, int):
                    assert rc == 0, rc
                if rec:
                    hip.record(ev[name][i - 1][1], stream)
        torch.cuda.synchronize()
        pk = T2 * k2
        hbm_bytes = {"route": T2 * E2 * s + pk * (4 + s),
                     "dispatch": pk * 4 * 2 + T2 * H2 * s + pk * H2 * s + pk * 4 + 4 * (E2 + 1),
                     "combine": pk * H2 * s + pk * (s + 4) + T2 * H2 * s}
        hbm = {"workload": "routing+dispatch T=65536 E=128 k=8 H=2048 bf16, identity experts, caches evicted by a "
                           "512 MiB read before each launch"}
        for name in ("route", "dispatch", "combine"):
            us = float(np.median([hip.ms(a, b) for a, b in ev[name]])) * 1e3
            gbs = hbm_bytes[name] / (us / 1e6) / 1e9
            hbm[name] = {"us": us, "bytes": hbm_bytes[name], "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}

        # The whole routing+dispatch pass in its fused form: rudnn_moe_route_dispatch (routing with
        # the per-chunk dispatch step, the scan, the copy with the map), then combine; caches
        # evicted once before each pass.  Per-kernel times from a separate pass.
        rd_kernels = ("route", "dispatch_scan", "dispatch_copy", "combine")
        pass_ev = [(hip.event(), hip.event()) for _ in range(reps)]
        kev = {n_: [(hip.event(), hip.event()) for _ in range(reps)] for n_ in rd_kernels}

        def rd_pass():
            moe.route_dispatch(lg2, k2, True, x2, out=d2, workspace=dws)
            moe.combine(d2.dispatched, d2.token_map, wt2, out=o2)

        for i in range(reps + 1):
            flush()
            if i > 0:
                hip.record(pass_ev[i - 1][0], stream)
            rd_pass()
            if i > 0:
                hip.record(pass_ev[i - 1][1], stream)
        for i in range(reps):
            flush()
            for kn in rd_kernels:
                moe.time_next_launch(kn, *kev[kn][i])
            rd_pass()
        torch.cuda.synchronize()
        pass_us = float(np.median([hip.ms(a, b) for a, b in pass_ev])) * 1e3
        k_us = {kn: float(np.median([hip.ms(a, b) for a, b in v])) * 1e3 for kn, v in kev.items()}
        roof_us = (hbm_bytes["route"] + hbm_bytes["dispatch"] + hbm_bytes["combine"]) / (HBM_PEAK_GBS * 1e3)
        hbm["fused_pass"] = {
            "calls": "rudnn_moe_route_dispatch + rudnn_moe_combine, renormalize",
            "us": pass_us, "tokens_per_s": T2 / (pass_us / 1e6),
            "roofline_tokens_per_s": T2 / (roof_us / 1e6), "roofline_frac": roof_us / pass_us,
            "kernels_us": k_us,
            "route_and_scan_us": k_us["route"] + k_us["dispatch_scan"],
        }

    # ---------------- group-limited sigmoid routing (section 10) ----------------
    sig = None
    if not args.no_sigmoid:
        if not args.no_hbm_stages:
            del x2, d2, o2, dws, lg2, idx2, wt2
        torch.cuda.empty_cache()
        from mixture_experts_layer_23_amd.inputs import make_sigmoid_logits
        ws_ = WORKLOADS["sigmoid_route"]
        log("generating", ws_.name)
        lg3_cpu, b3_cpu, _ = make_sigmoid_logits(ws_)
        lg3, b3 = lg3_cpu.to(dev), b3_cpu.to(dev)
        sg = ws_.sigmoid
        o3 = moe.GroupRoutingOptions(ws_.top_k, sg.groups, sg.selected_groups, int(sg.group_top_two),
                                     int(sg.renormalize), sg.scale)
        T3, E3, k3 = ws_.T, ws_.E, ws_.top_k
        idx3 = torch.empty(T3, k3, dtype=torch.int32, device=dev)
        wt3 = torch.empty(T3, k3, dtype=lg3.dtype, device=dev)
        reps = 5
        ev3 = [(hip.event(), hip.event()) for _ in range(reps)]
        for i in range(reps + 1):
            flush()
            if i:
                hip.record(ev3[i - 1][0], stream)
            rc = moe.lib().rudnn_moe_route_sigmoid_grouped(lg3.data_ptr(), 2, T3, E3, b3.data_ptr(), o3,
                                                           idx3.data_ptr(), wt3.data_ptr(), stream)
            assert rc == 0, rc
            if i:
                hip.record(ev3[i - 1][1], stream)
        torch.cuda.synchronize()
        us3 = float(np.median([hip.ms(a, b) for a, b in ev3])) * 1e3
        b3_bytes = T3 * E3 * 2 + E3 * 4 + T3 * k3 * (4 + 2)
        sig = {"route": {"workload": f"T={T3} E={E3} groups={sg.groups} selected={sg.selected_groups} top-two "
                                     f"k={k3} bf16 logits + FP32 bias, caches evicted",
                         "us": us3, "bytes": b3_bytes, "GBps": b3_bytes / (us3 / 1e6) / 1e9,
                         "hbm_frac": b3_bytes / (us3 / 1e6) / 1e9 / HBM_PEAK_GBS}}
        del lg3, b3, idx3, wt3
        # the decode-shaped layer routed this way (256 experts, weights streamed from HBM)
        wd = WORKLOADS["sigmoid_decode"]
        log("generating", wd.name)
        lgd_cpu, bd_cpu, _ = make_sigmoid_logits(wd)
        lgd, bd = lgd_cpu.to(dev), bd_cpu.to(dev)
        xd = make_tokens(wd, dev)
        gd, ud, dd = make_experts(wd, dev)
        exd = moe.SwiGluExperts(gd, ud, dd)
        sgd = wd.sigmoid
        od = moe.GroupRoutingOptions(wd.top_k, sgd.groups, sgd.selected_groups, int(sgd.group_top_two),
                                     int(sgd.renormalize), sgd.scale)
        outd = torch.empty_like(xd)
        wsd = torch.empty(moe.forward_workspace_size(exd, wd.T, wd.top_k, lgd.dtype), dtype=torch.uint8, device=dev)
        for _ in range(3):
            exd.forward_sigmoid_grouped(xd, lgd, bd, od, out=outd, workspace=wsd)
        torch.cuda.synchronize()
        nd = 20
        a_, b_ = hip.event(), hip.event()
        hip.record(a_, stream)
        for _ in range(nd):
            exd.forward_sigmoid_grouped(xd, lgd, bd, od, out=outd, workspace=wsd)
        hip.record(b_, stream)
        msd = hip.ms(a_, b_) / nd
        active = int(torch.unique(moe.route_sigmoid_grouped(lgd, bd, od)[0]).numel())
        wbytes = active * 3 * wd.H * wd.I * 2
        sig["decode_forward"] = {"workload": f"T={wd.T} H={wd.H} I={wd.I} E={wd.E} k={wd.top_k} bf16, "
                                             f"{active} active experts",
                                 "ms": msd, "tokens_per_s": wd.T / (msd / 1e3),
                                 "weight_GBps": wbytes / (msd / 1e3) / 1e9,
                                 "hbm_frac": wbytes / (msd / 1e3) / 1e9 / HBM_PEAK_GBS}
        del gd, ud, dd, exd, wsd

    # ---------------- the forward on the other layers of the workload set ----------------
    other = None
    if not args.no_other:
        torch.cuda.empty_cache()
        other = measure_other_forwards(moe, hip, stream, dev)

    # ---------------- gate projection fused with routing ----------------
    proj = None
    if not args.no_projection:
        torch.cuda.empty_cache()
        proj = measure_projection(args, moe, hip, stream, flush, dev, ex, w, out_shape=(w.T, w.H))

    # ---------------- first-order training: the backward chain ----------------
    train = None
    if not args.no_training:
        torch.cuda.empty_cache()
        train = measure_training(moe, hip, stream, flush, dev, ex, w, logits, x)

    traffic = traffic_for("experts_gate_up", "mixtral")
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; random-init expert weights N(0,1)/sqrt(fan_in))",
        "config": {"workload": "Mixtral-shaped MoE layer", "T": T, "H": H, "I": I, "E": E, "top_k": k,
                   "renormalize": renorm, "token_dtype": w.dtype, "logits_dtype": w.logits_dtype},
        "roofline": {"bound": "mfma", "kernel": "experts_gate_up", "achieved": gu_tflops,
                     "peak": MFMA_PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                     "frac": gu_tflops / MFMA_PEAK_TFLOPS[w.dtype], "traffic": traffic,
                     "algorithmic_per_launch": gu_flops, "avg_launch_ms": gu_ms,
                     "avg_launch_ms_parts": {"experts_gate_up": gu_main_ms, "experts_gate_up_reduce": gu_reduce_ms}},
        "cpu_baseline": cpu,
        "stages": stages,
        "hbm_stages": hbm,
        "forward_other": other,
        "sigmoid_routing": sig,
        "projection": proj,
        "training": train,
    }
    print(json.dumps(result), flush=True)


FORWARD_KERNELS = ("route", "dispatch_count", "dispatch_scan", "dispatch_copy", "experts_plan", "experts_gate_up",
                   "experts_gate_up_reduce", "experts_down", "experts_down_reduce", "combine")


def kernel_breakdown(moe, hip, fn, reps=5, kernels=FORWARD_KERNELS):
    """Mean µs of each kernel ``fn`` launches (HIP events on its launch stream through the
    library's timing hook), over ``reps`` calls; kernels that never launched are left out."""
    import numpy as np
    import torch

    ev = {kn: [(hip.event(), hip.event()) for _ in range(reps)] for kn in kernels}
    for i in range(reps):
        for kn in kernels:
            moe.time_next_launch(kn, *ev[kn][i])
        fn()
        for kn in kernels:  # a kernel this call does not launch leaves its pair unrecorded
            moe.time_next_launch(kn, None, None)
    torch.cuda.synchronize()
    out = {}
    for kn, pairs in ev.items():
        v = [hip.ms_if_recorded(a, b) for a, b in pairs]
        v = [x for x in v if x is not None]
        if v:
            out[kn] = float(np.mean(v)) * 1e3
    return out


def measure_other_forwards(moe, hip, stream, dev, steps=20):
    """rudnn_moe_forward on the decode-shaped, skewed and tiny layers (inputs resident in HBM,
    back-to-back steps): ms per forward, tokens/s, and the expert weights streamed per second
    (active experts' 3*H*I elements) or the expert GEMMs' flops per second."""
    import numpy as np
    import torch

    from mixture_experts_layer_23_amd.inputs import WORKLOADS, make_experts, make_logits, make_tokens

    res = {}
    for name in ("decode", "skewed", "tiny"):
        w = WORKLOADS[name]
        log("forward", name)
        lg_cpu, _ = make_logits(w)
        lg = lg_cpu.to(dev)
        x = make_tokens(w, dev)
        g, u, d = make_experts(w, dev)
        ex = moe.SwiGluExperts(g, u, d)
        out = torch.empty_like(x)
        ws = torch.empty(moe.forward_workspace_size(ex, w.T, w.top_k, lg.dtype), dtype=torch.uint8, device=dev)
        renorm = w.renormalize[0]
        for _ in range(3):
            ex.forward(x, lg, w.top_k, renorm, out=out, workspace=ws)
        torch.cuda.synchronize()
        a, b = hip.event(), hip.event()
        hip.record(a, stream)
        for _ in range(steps):
            ex.forward(x, lg, w.top_k, renorm, out=out, workspace=ws)
        hip.record(b, stream)
        torch.cuda.synchronize()
        ms = hip.ms(a, b) / steps
        s = DTYPE_BYTES[w.dtype]
        active = int(np.count_nonzero(np.bincount(moe.route(lg, w.top_k, renorm)[0].cpu().numpy().ravel(),
                                                  minlength=w.E)))
        wbytes = active * 3 * w.H * w.I * s
        flops = 6.0 * w.T * w.top_k * w.H * w.I
        ent = {"workload": f"T={w.T} H={w.H} I={w.I} E={w.E} k={w.top_k} {w.dtype}, {active} active experts",
               "ms": ms, "tokens_per_s": w.T / (ms / 1e3),
               "expert_weight_GBps": wbytes / (ms / 1e3) / 1e9, "hbm_frac": wbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
               "expert_TFLOPps": flops / (ms / 1e3) / 1e12}
        if w.dtype != "f32":  # the FP32 layer runs on the vector FMAs, not the matrix cores
            ent["mfma_frac"] = ent["expert_TFLOPps"] / MFMA_PEAK_TFLOPS[w.dtype]
        ent["kernels_us"] = kernel_breakdown(
            moe, hip, lambda: ex.forward(x, lg, w.top_k, renorm, out=out, workspace=ws))
        res[name] = ent
        del lg, x, g, u, d, ex, out, ws
        torch.cuda.empty_cache()
    return res


def measure_projection(args, moe, hip, stream, flush, dev, ex, wmix, out_shape):
    """The fused gate projection + routing (rudnn_moe_route_projected): kernel time on the
    routing+dispatch token shape (T=65536, H=2048, E=128, k=8) and on 65536 tokens of the 256-expert
    shape (H=7168), caches evicted before each launch; and, on the Mixtral-shaped layer and the
    decode shape, the whole call back to back next to the forward that takes ready logits."""
    import numpy as np
    import torch
    from mixture_experts_layer_23_amd.inputs import WORKLOADS, make_logits, make_projection_inputs

    def cold_kernel(x, router, T, H, E, k, reps=5):
        idx = torch.empty(T, k, dtype=torch.int32, device=dev)
        wt = torch.empty(T, k, dtype=x.dtype, device=dev)
        need = moe.route_projected_workspace_size(T, H, E, x.dtype)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        ev = [(hip.event(), hip.event()) for _ in range(reps)]
        for i in range(reps + 1):
            flush()
            if i:
                moe.time_next_launch("route_projected", *ev[i - 1])
            rc = moe.lib().rudnn_moe_route_projected(x.data_ptr(), 2, router.data_ptr(), T, H, E,
                                                     moe.RoutingOptions(k, 1), None, idx.data_ptr(), wt.data_ptr(),
                                                     ws.data_ptr(), ws.numel(), stream)
            assert rc == 0, rc
        torch.cuda.synchronize()
        us = float(np.median([hip.ms(a, b) for a, b in ev])) * 1e3
        byts = T * H * 2 + E * H * 2 + T * k * (4 + 2)
        flops = 2.0 * T * H * E
        return {"workload": f"T={T} H={H} E={E} k={k} bf16, caches evicted", "kernel_us": us, "bytes": byts,
                "GBps": byts / (us / 1e6) / 1e9, "hbm_frac": byts / (us / 1e6) / 1e9 / HBM_PEAK_GBS,
                "TFLOPps": flops / (us / 1e6) / 1e12, "mfma_frac": flops / (us / 1e6) / 1e12 / MFMA_PEAK_TFLOPS["bf16"]}

    res = {}
    for name, E, k in (("route_dispatch", None, None), ("sigmoid_route", None, None)):
        wl = WORKLOADS[name]
        log("generating projection inputs", name)
        x, router, _ = make_projection_inputs(wl, dev)
        res[name] = cold_kernel(x, router, wl.T, wl.H, wl.E, wl.top_k)
        del x, router
        torch.cuda.empty_cache()

    def back_to_back(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = hip.event(), hip.event()
        hip.record(a, stream)
        for _ in range(n):
            fn()
        hip.record(b, stream)
        return hip.ms(a, b) / n

    # Mixtral-shaped layer: forward from hidden states vs forward with ready logits
    log("projection: Mixtral-shaped layer")
    x, router, _ = make_projection_inputs(wmix, dev)
    lg = make_logits(wmix)[0].to(dev)
    out = torch.empty_like(x)
    wsf = torch.empty(moe.forward_workspace_size(ex, wmix.T, wmix.top_k, lg.dtype), dtype=torch.uint8, device=dev)
    wsp = torch.empty(moe.forward_projected_workspace_size(ex, wmix.T, wmix.top_k), dtype=torch.uint8, device=dev)
    ms_fwd = back_to_back(lambda: ex.forward(x, lg, wmix.top_k, True, out=out, workspace=wsf))
    ms_proj = back_to_back(lambda: ex.forward_projected(x, router, wmix.top_k, True, out=out, workspace=wsp))
    kev = [(hip.event(), hip.event()) for _ in range(5)]
    rev = [(hip.event(), hip.event()) for _ in range(5)]
    for i in range(5):
        moe.time_next_launch("route_projected", *kev[i])
        moe.time_next_launch("route_projected_reduce", *rev[i])
        ex.forward_projected(x, router, wmix.top_k, True, out=out, workspace=wsp)
    torch.cuda.synchronize()
    res["mixtral_layer"] = {
        "workload": f"T={wmix.T} H={wmix.H} I={wmix.I} E={wmix.E} k={wmix.top_k} bf16, router [E, H]",
        "forward_ms": ms_fwd, "forward_projected_ms": ms_proj,
        "forward_projected_tokens_per_s": wmix.T / (ms_proj / 1e3),
        "route_projected_kernel_us": float(np.median([hip.ms(a, b) for a, b in kev])) * 1e3,
        "route_projected_reduce_us": float(np.median([hip.ms(a, b) for a, b in rev])) * 1e3}
    del x, router, lg, out, wsf, wsp
    torch.cuda.empty_cache()

    # decode shape: the H split over blocks + the reduce kernel, whole call back to back
    wd = WORKLOADS["decode"]
    x, router, _ = make_projection_inputs(wd, dev)
    idx = torch.empty(wd.T, wd.top_k, dtype=torch.int32, device=dev)
    wt = torch.empty(wd.T, wd.top_k, dtype=x.dtype, device=dev)
    ws = torch.empty(max(moe.route_projected_workspace_size(wd.T, wd.H, wd.E, x.dtype), 256), dtype=torch.uint8,
                     device=dev)

    def dec():
        rc = moe.lib().rudnn_moe_route_projected(x.data_ptr(), 2, router.data_ptr(), wd.T, wd.H, wd.E,
                                                 moe.RoutingOptions(wd.top_k, 1), None, idx.data_ptr(), wt.data_ptr(),
                                                 ws.data_ptr(), ws.numel(), stream)
        assert rc == 0, rc
    ms_dec = back_to_back(dec, 50)
    res["decode"] = {"workload": f"T={wd.T} H={wd.H} E={wd.E} k={wd.top_k} bf16 (H split over blocks)",
                     "call_us": ms_dec * 1e3, "router_GBps": wd.E * wd.H * 2 / (ms_dec / 1e3) / 1e9}
    return res


def measure_training(moe, hip, stream, flush, dev, ex, w, logits, x):
    """The first-order training step of section 12 on the Mixtral-shaped layer: the experts
    forward that keeps its FP32 pre-activations as the cache (next to the plain forward), then the
    backward chain combine_backward -> experts backward from that cache -> dispatch_backward ->
    selected_router_backward, timed back to back per step with every kernel's time (and the same
    chain recomputing gate/up instead of reading a cache); combine/dispatch backward on the
    routing+dispatch workload with the caches evicted."""
    import numpy as np
    import torch
    from mixture_experts_layer_23_amd.inputs import WORKLOADS, make_logits, make_tokens

    idx, wt = moe.route(logits, w.top_k, True)
    d = moe.dispatch(idx, x, w.E)
    rows = d.dispatched.shape[0]
    fws = torch.empty(moe.experts_workspace_size(ex, rows), dtype=torch.uint8, device=dev)
    y = torch.empty_like(d.dispatched)
    pre = torch.empty(rows, 2 * w.I, dtype=torch.float32, device=dev)
    g = torch.Generator(device=dev).manual_seed(1)
    dout = (torch.randn(w.T, w.H, generator=g, device=dev) * 0.05).bfloat16()
    ws = torch.empty(moe.experts_backward_workspace_size(ex, rows), dtype=torch.uint8, device=dev)
    dexp = torch.zeros_like(y)

    def timed(fn, names, reps=5):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        per = {n: [] for n in names}
        tot = []
        for _ in range(reps):
            ev = {n: (hip.event(), hip.event()) for n in names}
            for n in names:
                moe.time_next_launch(n, *ev[n])
            a, b = hip.event(), hip.event()
            hip.record(a, stream)
            fn()
            hip.record(b, stream)
            torch.cuda.synchronize()
            for n in names:
                per[n].append(hip.ms(*ev[n]))
            tot.append(hip.ms(a, b))
        return {n: float(np.median(v)) * 1e3 for n, v in per.items()}, float(np.median(tot))

    fwd_names = ["experts_plan", "experts_gate_up", "experts_gate_up_reduce", "experts_down", "experts_down_reduce"]
    us_plain, ms_plain = timed(lambda: moe.experts_forward(ex, d.dispatched, d.expert_offsets, out=y, workspace=fws),
                               fwd_names)
    us_train, ms_train = timed(lambda: moe.experts_forward_training(ex, d.dispatched, d.expert_offsets, out=y,
                                                                    cache=pre, workspace=fws), fwd_names)

    def chain(cache):
        _, dw = moe.combine_backward(y, d.token_map, wt, dout, grad_expert_output=dexp)
        dx, _, _, _ = moe.experts_backward(ex, d.dispatched, d.expert_offsets, dexp, cache=cache, workspace=ws)
        moe.dispatch_backward(dx, d.token_map)
        moe.selected_router_backward(logits, idx, dw, "softmax", True, 1.0)

    names = ["combine_backward", "experts_backward_dh", "experts_backward_dx", "experts_backward_dw",
             "dispatch_backward", "selected_router"]
    us, ms = timed(lambda: chain(pre), names)
    us_rc, ms_rc = timed(lambda: chain(None), names + ["experts_backward_gu"])
    H, I = w.H, w.I
    fl = {"experts_backward_dh": 2.0 * rows * H * I, "experts_backward_dx": 4.0 * rows * H * I,
          "experts_backward_dw": 2.0 * rows * H * I}
    kern = {n: {"us": us[n]} for n in names}
    for n, f in fl.items():
        kern[n]["TFLOPps"] = f / (us[n] / 1e6) / 1e12
        kern[n]["mfma_frac"] = kern[n]["TFLOPps"] / MFMA_PEAK_TFLOPS["bf16"]
    kern["experts_backward_dw"]["note"] = "the last of three launches (ddown); dgate and dup have the same shape"
    gu_us = us_rc["experts_backward_gu"]
    res = {"mixtral_layer": {
        "workload": f"T={w.T} H={H} I={I} E={w.E} k={w.top_k} bf16, softmax router renormalised",
        "experts_forward_ms": ms_plain, "experts_forward_training_ms": ms_train,
        "gate_up_us": {"forward": us_plain["experts_gate_up"], "forward_training": us_train["experts_gate_up"]},
        "cache_bytes": rows * 2 * I * 4,
        "backward_chain_ms": ms, "backward_tokens_per_s": w.T / (ms / 1e3),
        "experts_backward_TFLOPps": 12.0 * rows * H * I / (ms / 1e3) / 1e12,
        "training_step_ms": ms_train + ms,
        "backward_chain_recompute_ms": ms_rc,
        "recomputed_gate_up": {"us": gu_us, "TFLOPps": 4.0 * rows * H * I / (gu_us / 1e6) / 1e12},
        "note": "backward from the forward's FP32 pre-activation cache; experts backward algorithmic flops "
                "12 rows H I; training_step_ms = experts forward with cache + backward chain (routing, dispatch "
                "and combine forward not included)",
        "kernels": kern}}
    del d, y, ws, dexp, dout, pre, fws
    torch.cuda.empty_cache()

    # combine / dispatch backward on the routing+dispatch workload, caches evicted
    w2 = WORKLOADS["route_dispatch"]
    lg2 = make_logits(w2)[0].to(dev)
    x2 = make_tokens(w2, dev)
    idx2, wt2 = moe.route(lg2, w2.top_k, True)
    d2 = moe.dispatch(idx2, x2, w2.E)
    dout2 = torch.randn(w2.T, w2.H, generator=g, device=dev).bfloat16()
    dexp2 = torch.empty_like(d2.dispatched)
    din2 = torch.empty_like(x2)
    reps = 5
    ev = {n: [(hip.event(), hip.event()) for _ in range(reps)] for n in ("combine_backward", "dispatch_backward")}
    for i in range(reps + 1):
        flush()
        if i:
            moe.time_next_launch("combine_backward", *ev["combine_backward"][i - 1])
        moe.combine_backward(d2.dispatched, d2.token_map, wt2, dout2, grad_expert_output=dexp2)
        flush()
        if i:
            moe.time_next_launch("dispatch_backward", *ev["dispatch_backward"][i - 1])
        moe.dispatch_backward(dexp2, d2.token_map, out=din2)
    torch.cuda.synchronize()
    T2, k2, H2 = w2.T, w2.top_k, w2.H
    nbytes = {"combine_backward": 2 * T2 * k2 * H2 * 2 + T2 * H2 * 2 + T2 * k2 * (4 + 2 + 4),
              "dispatch_backward": T2 * k2 * H2 * 2 + T2 * H2 * 2 + T2 * k2 * 4}
    hb = {"workload": "routing+dispatch T=65536 H=2048 k=8 bf16, caches evicted"}
    for n in nbytes:
        u = float(np.median([hip.ms(a, b) for a, b in ev[n]])) * 1e3
        gbs = nbytes[n] / (u / 1e6) / 1e9
        hb[n] = {"us": u, "bytes": nbytes[n], "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    res["hbm_stages"] = hb
    return res


if __name__ == "__main__":
    main()
