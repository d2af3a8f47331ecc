#!/usr/bin/env python
"""Throughput of the sparse-convolution hot path on one MI355X.

One step runs every stage of the path once on one batch of synthetic input.
It starts with the LiDAR-like scene: 2 samples x 60k voxels on a 41 x 1600 x
1408 grid, fp16, 64 channels.  The stages are, in order:

    kmap_subm       submanifold kernel map k=3 (table build + probe + pair lists + order)
    fwd_subm        SubMConv3d k=3 forward 64 -> 64
    fwd_k1          k=1 layer 64 -> 64 on that output
    dinput_subm     dinput of the k=3 layer
    dfilter_subm    dfilter of the k=3 layer
    kmap_strided    strided kernel map k=3 s=2 p=1 (output sites, maps, pairs)
    fwd_strided     SparseConv3d forward 64 -> 128
    dinput_strided  its dinput
    dfilter_strided its dfilter

Both kernel maps depend on the coordinates only, so the step builds each on
a stream of its own (default priority), while the main stream finishes the
previous step: the SubM map first (its layer is next on the main stream), the
strided map after it, beside the SubM layer; each layer waits for its map.  The maps are marked
as used by the main stream, so their memory is not reused early.  Running the
SubM dinput and dfilter side by side as well was slower (each fills the GPU).

``--workload shells`` runs the same stages on the mesh-shell sets: 4 x 128^3,
bf16, 128 channels, with k=1 128 -> 128.  The strided layer there is 128 -> 128.

value = effective TFLOP/s of the whole step: 2 * pairs * Cin * Cout summed
over the convolution stages (pairs counted from the kernel map, k=1 counts N
pairs), divided by the step time.  The kernel-map rate is reported as voxels/s
(N over the kmap_subm time).  The K timed steps run bare; a second pass of K
steps times every stage with HIP events on the stream it runs on (the event
records cost host time, so that pass is not the timed one) and reports each
stage's median.  With the two streams overlapping, a stage's time includes
what it shares the GPU with.  The roofline is given for the single-kernel
stage with the longest kernel: each such kernel is also launched back to back
between two HIP events, behind a few ms of queued fills so that no host time
between launches counts (the step's stage timings include host gaps, e.g. after
the strided kernel map's one synchronisation), and that average is its launch
duration.  Its HBM traffic comes from the rocprofv3 counter runs recorded in
profiles/traffic.json, and only while the kernel source is the one measured.

``--kmap-sweep`` replaces the step by the kernel-map rate on the shell sets at
4, 8, 16 and 32 samples (one JSON line each), to show the maps as the scene grows
past the sizes where launch latency dominates.

``extras`` times the layers beyond the step the same way, one launch each on
this step's maps: fwd_inverse is the upsampling layer back from the strided
layer (its channels reversed); fwd_subm_add_relu_fused is the k=3 layer as a
residual block relu(conv(x) + x) in one kernel, and ..._unfused the same
through the plain forward plus torch's add and relu (three launches, timed
together); maxpool_fwd / maxpool_bwd pool x over the strided layer's map
(3^3, stride 2); subm_step_graph replays the SubM half of the step (kernel map,
forward, k=1, dinput, dfilter) as one captured HIP graph, subm_step_eager makes
the same calls one by one; point_to_voxel voxelises a 200k-point synthetic sweep
(one call, its host synchronisation included).  They are not part of ``value``.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
SINGLE_KERNEL_STAGES = ("fwd_subm", "fwd_k1", "dinput_subm", "fwd_strided", "dinput_strided")
KERNEL_REPS = 20         # back-to-back launches per single-kernel stage for its duration
BUSY_FILLS = 3           # 1 GiB fills queued ahead of them (~0.5 ms of GPU time)
CPU_MIN_S = 10.0         # the oracle repeats whole steps for at least this long (within --cpu-budget)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=("lidar", "shells"), default="lidar")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="seconds of oracle work to time at most")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--no-extras", action="store_true", help="skip timing the layers beyond the step")
    ap.add_argument("--kmap-sweep", action="store_true",
                    help="instead of the step: kernel-map rate on the shell sets at 4..32 samples (one line each)")
    return ap.parse_args()


# ---------------------------------------------------------------- inputs

def make_inputs(kind: str):
    import numpy as np
    import torch
    import workloads as W

    if kind == "lidar":
        w = W.workload("subm_k3_f16_lidar120k", with_grad=True)
        ws = W.workload("strided_k3s2_f16_lidar120k")
        return dict(name="lidar_2x60k_41x1600x1408_f16_c64", coords=w.coords, batch=w.batch, shape=w.shape,
                    dtype=w.dtype, feats=w.feats, w3=w.weight, w1=w.extra["weight_k1"], grad=w.grad,
                    ws=ws.weight, grad_rng=ws.extra["grad_rng"])
    w = W.workload("subm_k3_k1_bf16_shells128")
    g = W.rng(6, "grad")
    c = w.cin
    grad = W.grad_for(g, w.n, c, w.dtype)
    wstr = (torch.from_numpy(W.rng(6, "weight").standard_normal((27, c, c), dtype=np.float32)
                             / np.sqrt(27 * c)).to(w.dtype))
    return dict(name="shells_4x128^3_bf16_c128", coords=w.coords, batch=w.batch, shape=w.shape, dtype=w.dtype,
                feats=w.feats, w3=w.weight, w1=w.extra["weight_k1"], grad=grad, ws=wstr, grad_rng=W.rng(6, "bias"))


# ---------------------------------------------------------------- GPU step

class Step:
    """Holds device inputs and runs the stages of one step through the library."""

    def __init__(self, inp, dev):
        import torch
        import sparse_convolution_hash_amd as spc
        import workloads as W

        self.spc, self.torch = spc, torch
        self.inp = inp
        t = lambda a: (torch.from_numpy(a) if not isinstance(a, torch.Tensor) else a).contiguous().to(dev)
        self.coords, self.x, self.w3, self.w1, self.g = (t(inp[k]) for k in ("coords", "feats", "w3", "w1", "grad"))
        self.ws = t(inp["ws"])
        self.n = self.coords.shape[0]
        self.dev = dev
        # strided output size and its upstream gradient, drawn once
        km = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, 2, 1, 1, subm=False, orders=True)
        self.m = km["n_out"]
        self.gs = t(W.grad_for(inp["grad_rng"], self.m, self.ws.shape[2], inp["dtype"]))
        ks = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3)
        self.P = int(ks["pair_ptr"][-1].item())
        self.Ps = int(km["pair_ptr"][-1].item())
        self.names = ("kmap_subm", "fwd_subm", "fwd_k1", "dinput_subm", "dfilter_subm",
                      "kmap_strided", "fwd_strided", "dinput_strided", "dfilter_strided")
        self.ev = None
        self.side = None             # the kernel maps' streams (created on first use)
        self.km, self.ks = None, km  # maps held for kernel_ms (the SubM one is built on first use)

    def kernel_ms(self, stage: str, reps: int = KERNEL_REPS) -> float:
        """Average duration of one single-kernel stage launched `reps` times back to
        back between two HIP events (the queue never drains, so no host gap counts)."""
        spc, inp = self.spc, self.inp
        if self.km is None:
            self.km = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, orders=True)
        km, ks = self.km, self.ks
        y = self.x if self.w1.shape[1] == self.x.shape[1] else None
        make = {  # stage -> a function that makes its launch
            "fwd_subm": lambda: self.conv_only(self.x, self.w3, km["nbr"], self.n, True, km["order"]),
            "fwd_k1": lambda: self.conv_only(y, self.w1, None, self.n, False, None),
            "dinput_subm": lambda: lambda: spc.conv_bwd_input(self.g, self.w3, km["nbr"], True, self.n, km["order"]),
            "fwd_strided": lambda: self.conv_only(self.x, self.ws, ks["nbr"], ks["n_out"], False, ks["order"]),
            "dinput_strided": lambda: lambda: spc.conv_bwd_input(self.gs, self.ws, ks["nbr_in"], False, self.n,
                                                                 ks["order_in"]),
        }[stage]
        return self.time_launch(make(), reps)

    def conv_only(self, x, w, map_, n_rows, subm, order):
        """A forward stage's convolution kernel alone.  Where the library hands
        the kernel pre-transposed weights (a second, small kernel per call, which
        the step itself runs every time), they are transposed once here, so
        that the timed launches are the convolution's."""
        spc = self.spc
        if not spc.binding._pretranspose(x.dtype, w.shape[1], None):
            if map_ is None:
                return lambda: spc.subm_conv_fwd(x, w, None, None)
            if subm:
                return lambda: spc.subm_conv_fwd(x, w, None, map_, order)
            return lambda: spc.sparse_conv_fwd(x, w, None, map_, n_rows, order)
        wt = spc.transpose_weight(w)
        return lambda: spc.conv_fwd_wt(x, wt, None, map_, n_rows, subm, order)

    def run(self, events=None):
        """One step.  Each kernel map depends on the coordinates only, so each
        is built on a stream of its own (default priority) while the main
        stream finishes the previous step; the main stream waits for a map
        (a persistent event) before its layer.  Each stage's events are
        recorded on the stream it runs on."""
        spc, inp, torch = self.spc, self.inp, self.torch
        E = events or {}
        if self.side is None:  # the streams and the events that join them, made once
            self.side = (torch.cuda.current_stream(), torch.cuda.Stream(), torch.cuda.Stream(),
                         torch.cuda.Event(), torch.cuda.Event())
        main, side_s, side_k, done_s, done_k = self.side

        def mark(name, i):
            if name in E:
                E[name][i].record()

        def used_on_main(maps):
            # the main stream reads these maps: their memory is not reused before it is done
            for t in maps.values():
                if isinstance(t, torch.Tensor):
                    t.record_stream(main)

        torch.cuda.set_stream(side_s)
        mark("kmap_subm", 0)
        km = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, orders=True)
        mark("kmap_subm", 1)
        done_s.record(side_s)
        torch.cuda.set_stream(side_k)
        side_k.wait_event(done_s)   # the SubM map first: its layer is the next on the main stream
        mark("kmap_strided", 0)
        ks = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, 2, 1, 1, subm=False, out_cap=self.m,
                            orders=True)
        mark("kmap_strided", 1)
        done_k.record(side_k)
        torch.cuda.set_stream(main)
        used_on_main(km)
        used_on_main(ks)
        main.wait_event(done_s)
        mark("fwd_subm", 0)
        y = spc.subm_conv_fwd(self.x, self.w3, None, km["nbr"], km["order"])
        mark("fwd_subm", 1)
        mark("fwd_k1", 0)
        spc.subm_conv_fwd(y, self.w1, None, None)
        mark("fwd_k1", 1)
        mark("dinput_subm", 0)
        spc.conv_bwd_input(self.g, self.w3, km["nbr"], True, self.n, km["order"])
        mark("dinput_subm", 1)
        mark("dfilter_subm", 0)
        spc.conv_bwd_filter(self.x, self.g, 27, km["pair_ptr"], km["pair_in"], km["pair_out"])
        mark("dfilter_subm", 1)
        main.wait_event(done_k)
        mark("fwd_strided", 0)
        spc.sparse_conv_fwd(self.x, self.ws, None, ks["nbr"], ks["n_out"], ks["order"])
        mark("fwd_strided", 1)
        mark("dinput_strided", 0)
        spc.conv_bwd_input(self.gs, self.ws, ks["nbr_in"], False, self.n, ks["order_in"])
        mark("dinput_strided", 1)
        mark("dfilter_strided", 0)
        spc.conv_bwd_filter(self.x, self.gs, 27, ks["pair_ptr"], ks["pair_in"], ks["pair_out"])
        mark("dfilter_strided", 1)

    def extras(self):
        """The widened layers, each one launch timed like a single-kernel stage:
        name -> (launch, effective FLOP, algorithmic HBM bytes).  They reuse this
        step's maps and synthetic tensors of the right shapes (the strided
        layer's upstream gradient serves as the coarse features)."""
        import workloads as W
        spc, torch = self.spc, self.torch
        ks = self.ks
        n, m, Ps, K = self.n, self.m, self.Ps, 27
        cin, cs = self.ws.shape[1], self.ws.shape[2]
        s = self.x.element_size()
        if not hasattr(self, "w_inv"):
            self.w_inv = self.ws.transpose(1, 2).contiguous()  # [K, cs, cin]: upsampling back to cin channels
            self.pool_y, self.pool_a = spc.sparse_maxpool_fwd(self.x, ks["nbr"], m)
            self.pool_g = self.gs[:, :cin].contiguous()  # an upstream gradient of the pooled shape
            self.pts = torch.from_numpy(W.lidar_points(W.rng(236))).to(self.dev)
        vc = W.LIDAR_VOXEL
        if self.km is None:
            self.km = spc.build_kmap(self.coords, self.inp["batch"], self.inp["shape"], 3, orders=True)
        km, P, c1 = self.km, self.P, self.w3.shape[2]

        def unfused():  # the same layer as three launches: conv, then torch's add and relu
            y = spc.subm_conv_fwd(self.x, self.w3, None, km["nbr"], km["order"])
            y.add_(self.x).relu_()

        sub_bytes = n * cin * s + K * n * 4 + K * cin * c1 * s + n * c1 * s
        inp = self.inp

        def subm_step():  # the SubM half of the step: kernel map, forward, k=1, dinput, dfilter
            kmap = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, orders=True)
            y = spc.subm_conv_fwd(self.x, self.w3, None, kmap["nbr"], kmap["order"])
            spc.subm_conv_fwd(y, self.w1, None, None)
            spc.conv_bwd_input(self.g, self.w3, kmap["nbr"], True, n, kmap["order"])
            spc.conv_bwd_filter(self.x, self.g, K, kmap["pair_ptr"], kmap["pair_in"], kmap["pair_out"])

        if not hasattr(self, "graph"):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):  # warm the allocator on the capture stream
                subm_step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            self.graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.graph):
                subm_step()
        f, b = self.work()
        st_f = sum(f[k] for k in ("fwd_subm", "fwd_k1", "dinput_subm", "dfilter_subm"))
        st_b = sum(b[k] for k in ("kmap_subm", "fwd_subm", "fwd_k1", "dinput_subm", "dfilter_subm"))
        return {
            "fwd_inverse": (lambda: spc.sparse_inverse_conv_fwd(self.gs, self.w_inv, None, ks["nbr_in"], n,
                                                                ks["order_in"]),
                            2 * Ps * cs * cin, m * cs * s + K * n * 4 + K * cs * cin * s + n * cin * s),
            # relu(conv(x) + x): the residual read is one more [n, c1] pass
            "fwd_subm_add_relu_fused": (lambda: spc.conv_fwd_fused(self.x, self.w3, None, km["nbr"], n, km["order"],
                                                                   residual=self.x, relu=True),
                                        2 * P * cin * c1, sub_bytes + n * c1 * s),
            "fwd_subm_add_relu_unfused": (unfused, 2 * P * cin * c1, sub_bytes + n * c1 * s),
            # 3^3 stride-2 max pooling of x on the strided layer's map; the bytes
            # count the map, each input and output row once, and the winner bytes
            "maxpool_fwd": (lambda: spc.sparse_maxpool_fwd(self.x, ks["nbr"], m, out=self.pool_y, argk=self.pool_a),
                            0, m * K * 4 + n * cin * s + m * cin * s + m * cin),
            "maxpool_bwd": (lambda: spc.sparse_maxpool_bwd(self.pool_g, self.pool_a, ks["nbr_in"], n),
                            0, n * K * 4 + m * cin * s + m * cin + n * cin * s),
            # a 200k-point synthetic sweep into 0.1 x 0.1 x 0.2 m voxels (one call,
            # including its one host synchronisation); bytes: the points read, the
            # voxel block, coordinates, counts and point ids written
            # the SubM half of the step replayed as one captured HIP graph, and the
            # same calls made one by one
            "subm_step_graph": (self.graph.replay, st_f, st_b),
            "subm_step_eager": (subm_step, st_f, st_b),
            "point_to_voxel": (lambda: spc.point_to_voxel(self.pts, vc["vsize_xyz"], vc["range_xyz"],
                                                          vc["max_voxels"], vc["max_points"], True, with_id=True),
                               0, self.pts.numel() * 4 + vc["max_voxels"] * (vc["max_points"] * self.pts.shape[1] * 4
                                                                            + 16) + self.pts.shape[0] * 4),
        }

    def time_launch(self, launch, reps: int = KERNEL_REPS) -> float:
        """Average duration of one launch repeated back to back between two events.
        Some GPU work is queued first (fills, then one untimed launch that brings
        the caches back), so the host has enqueued every timed launch before the
        first one starts and the host's per-call cost is not timed."""
        torch = self.torch
        launch()
        torch.cuda.synchronize()
        if not hasattr(self, "busy"):
            self.busy = torch.empty(1 << 30, dtype=torch.uint8, device=self.dev)
        for _ in range(BUSY_FILLS):
            self.busy.fill_(1)
        launch()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            launch()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # effective FLOP and algorithmic HBM bytes per stage (one launch / call)
    def work(self):
        n, m, P, Ps = self.n, self.m, self.P, self.Ps
        cin, c1 = self.w3.shape[1], self.w3.shape[2]
        cs = self.ws.shape[2]
        s = self.x.element_size()
        K = 27
        f = {
            "fwd_subm": 2 * P * cin * c1, "fwd_k1": 2 * n * c1 * self.w1.shape[2],
            "dinput_subm": 2 * P * cin * c1, "dfilter_subm": 2 * P * cin * c1,
            "fwd_strided": 2 * Ps * cin * cs, "dinput_strided": 2 * Ps * cin * cs,
            "dfilter_strided": 2 * Ps * cin * cs,
        }
        b = {
            "kmap_subm": n * (16 + 4 * K) + 8 * P + 4 * (K + 1) + 4 * n,
            "fwd_subm": n * cin * s + K * n * 4 + K * cin * c1 * s + n * c1 * s,
            "fwd_k1": n * c1 * s + c1 * self.w1.shape[2] * s + n * self.w1.shape[2] * s,
            "dinput_subm": n * c1 * s + K * n * 4 + K * cin * c1 * s + n * cin * s,
            "dfilter_subm": n * cin * s + n * c1 * s + 8 * P + 4 * (K + 1) + K * cin * c1 * 4,
            "kmap_strided": n * 16 + m * 16 + 4 * K * (m + n) + 8 * Ps + 4 * (K + 1) + 4 * (m + n),
            "fwd_strided": n * cin * s + K * m * 4 + K * cin * cs * s + m * cs * s,
            "dinput_strided": m * cs * s + K * n * 4 + K * cin * cs * s + n * cin * s,
            "dfilter_strided": n * cin * s + m * cs * s + 8 * Ps + 4 * (K + 1) + K * cin * cs * 4,
        }
        return f, b


# ---------------------------------------------------------------- CPU oracle

def cpu_baseline(inp, step_flops_fn, budget):
    """Times the oracle on the same step, stage by stage, until the budget is spent."""
    import numpy as np
    import threadpoolctl
    from oracle import conv as OC
    from oracle import kmap as OK
    import workloads as W

    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    c, sh, b = inp["coords"], inp["shape"], inp["batch"]
    done, spent, flops = [], 0.0, 0.0
    state = {}

    def st_kmap_subm():
        state["nbr"] = OK.subm_kmap(c, sh, 3)
        state["P"] = int((state["nbr"] >= 0).sum())

    def st_fwd():
        state["y"] = OC.conv_fwd(inp["feats"], inp["w3"], None, state["nbr"])

    def st_k1():
        OC.conv_fwd(state["y"], inp["w1"], None, np.arange(c.shape[0])[None])

    def st_din():
        OC.conv_bwd_input(inp["grad"], inp["w3"], state["nbr"], c.shape[0])

    def st_dw():
        OC.conv_bwd_filter(inp["feats"], inp["grad"], state["nbr"])

    def st_kmap_str():
        state["s"] = OK.strided_kmap(c, b, sh, 3, 2, 1, 1)
        state["Ps"] = int((state["s"]["nbr_out"] >= 0).sum())
        state["gs"] = W.grad_for(inp["grad_rng"], state["s"]["out_coords"].shape[0], inp["ws"].shape[2],
                                 inp["dtype"])

    def st_fwd_s():
        OC.conv_fwd(inp["feats"], inp["ws"], None, state["s"]["nbr_out"])

    def st_din_s():
        OC.conv_bwd_input(state["gs"], inp["ws"], state["s"]["nbr_out"], c.shape[0])

    def st_dw_s():
        OC.conv_bwd_filter(inp["feats"], state["gs"], state["s"]["nbr_out"])

    stages = [("kmap_subm", st_kmap_subm), ("fwd_subm", st_fwd), ("fwd_k1", st_k1), ("dinput_subm", st_din),
              ("dfilter_subm", st_dw), ("kmap_strided", st_kmap_str), ("fwd_strided", st_fwd_s),
              ("dinput_strided", st_din_s), ("dfilter_strided", st_dw_s)]
    times = {}
    steps = 0
    # whole steps, repeated until CPU_MIN_S have passed; a step that would not
    # fit the budget is cut after the stage that crosses it
    while spent < min(CPU_MIN_S, budget):
        for name, fn in stages:
            if spent > budget:
                break
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
            times[name] = times.get(name, 0.0) + dt
            spent += dt
            if steps == 0:
                done.append(name)
            flops += step_flops_fn(name, state)
        else:
            steps += 1
            continue
        break
    per = max(steps, 1)
    return {"value": flops / spent / 1e12 if spent > 0 else None, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{steps} whole step(s)" if steps else f"first {len(done)} of {len(stages)} stages")
                      + f" ({', '.join(done)}), {spent:.1f} s, numpy fp64 on {threads} BLAS threads",
            "stage_s": {k: round(v / per, 3) for k, v in times.items()},
            "kmap_voxels_per_s": c.shape[0] * per / times["kmap_subm"] if "kmap_subm" in times else None}


# ---------------------------------------------------------------- HBM traffic

def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of a stage's kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by the copy calibration recorded with
    them), or None if there are none or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f)[workload][stage]
        with open(os.path.join(ROOT, entry["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != entry["source_sha256"]:
                return None
        return entry["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


# ---------------------------------------------------------------- main

def kmap_sweep(batches=(4, 8, 16, 32), reps=10):
    """Kernel-map rate as the scene grows: the 128^3 shell sets (3 k=3 SubM map
    with pairs and order; the k3 s2 p1 strided map with pairs and both orders),
    one JSON line per batch size; medians of `reps` calls timed with HIP events."""
    import torch
    import sparse_convolution_hash_amd as spc
    import workloads as W

    K = 27
    for B in batches:
        c = torch.from_numpy(W.mesh_shells(W.rng(3), batch=B)).cuda()
        n = c.shape[0]
        shape = (128, 128, 128)
        m0 = spc.build_kmap(c, B, shape, 3, 2, 1, 1, subm=False, pairs=False)["n_out"]
        calls = {  # (the strided call gets the exact capacity, as in the step)
            "subm": lambda: spc.build_kmap(c, B, shape, 3, orders=True),
            "strided": lambda: spc.build_kmap(c, B, shape, 3, 2, 1, 1, subm=False, out_cap=m0, orders=True),
        }
        line = {"kmap_sweep": {"samples": B, "n_voxels": n}}
        for name, call in calls.items():
            r = call()
            torch.cuda.synchronize()
            P = int(r["pair_ptr"][-1].item())
            m = r["n_out"]
            ms = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                call()
                b.record()
                torch.cuda.synchronize()
                ms.append(a.elapsed_time(b))
            t = sorted(ms)[reps // 2] * 1e-3
            # algorithmic bytes: coordinates in, maps and pair lists out, orders out
            by = (n * (16 + 4 * K) + 8 * P + 4 * (K + 1) + 4 * n if name == "subm" else
                  16 * n + 16 * m + 4 * K * (m + n) + 8 * P + 4 * (K + 1) + 4 * (m + n))
            line["kmap_sweep"][name] = {"ms": round(t * 1e3, 4), "voxels_per_s": round(n / t, 1),
                                        "n_out": m, "pairs": P, "alg_GB/s": round(by / t / 1e9, 1),
                                        "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
        print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the per-sample sharding is described in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.kmap_sweep:
        kmap_sweep()
        return
    dev = torch.device("cuda:0")
    inp = make_inputs(args.workload)
    step = Step(inp, dev)
    flops, bytes_ = step.work()
    total_flop = sum(flops.values())

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # the timed steps, as a caller runs them (no per-stage instrumentation)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # then the same number of steps with HIP events around every stage, for the
    # per-stage breakdown (the event records cost host time, so this pass is
    # not the timed one)
    events = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)] for k in step.names}
    stage_ms = {k: 0.0 for k in step.names}
    for i in range(args.steps):
        step.run({k: events[k][i] for k in step.names})
    torch.cuda.synchronize()
    for k in step.names:
        stage_ms[k] = sorted(a.elapsed_time(b) for a, b in events[k])[args.steps // 2]   # median

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bb = torch.empty_like(a)
        bb.copy_(a)
        torch.cuda.synchronize()

    dtype = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}[inp["dtype"]]
    stages = {}
    for k in step.names:
        t = stage_ms[k] * 1e-3
        stages[k] = {"ms": round(stage_ms[k], 4),
                     "TFLOP/s": round(flops[k] / t / 1e12, 2) if k in flops and t > 0 else None,
                     "alg_GB/s": round(bytes_[k] / t / 1e9, 1) if t > 0 else None}
    kernel_ms = {k: step.kernel_ms(k) for k in SINGLE_KERNEL_STAGES}
    dom = max(SINGLE_KERNEL_STAGES, key=lambda k: kernel_ms[k])
    t_dom = kernel_ms[dom] * 1e-3
    ai = flops[dom] / bytes_[dom]
    ridge = MFMA_PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(bytes_[dom] / t_dom / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(flops[dom] / t_dom / 1e12, 2),
                "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(args.workload, dom)
    roof["kernel"] = f"k_conv ({dom})"
    roof["algorithmic_bytes_per_launch"] = bytes_[dom]
    roof["flop_per_launch"] = flops[dom]
    roof["avg_launch_ms"] = round(kernel_ms[dom], 4)
    roof["kernel_ms"] = {k: round(v, 4) for k, v in kernel_ms.items()}

    extras = {}
    for name, (launch, fl, by) in ({} if args.no_extras else step.extras()).items():
        ms = step.time_launch(launch)
        t = ms * 1e-3
        bound = "hbm" if fl / by < ridge else "mfma"
        ach = by / t / 1e9 if bound == "hbm" else fl / t / 1e12
        peak = HBM_PEAK_GBS if bound == "hbm" else MFMA_PEAK_TFLOPS[dtype]
        extras[name] = {"kernel_ms": round(ms, 4), "TFLOP/s": round(fl / t / 1e12, 2) if fl else None,
                        "alg_GB/s": round(by / t / 1e9, 1), "bound": bound, "frac": round(ach / peak, 4)}

    kmap_vps = step.n / (stage_ms["kmap_subm"] * 1e-3)
    out = {
        "metric": "effective TFLOP/s of SubMConv3d fwd (occupied pairs) + kmap voxels/s, 1 MI355X",
        "value": round(total_flop / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": inp["name"], "n_voxels": step.n, "pairs_subm_k3": step.P,
                   "n_out_strided": step.m, "pairs_strided": step.Ps,
                   "channels": [int(step.w3.shape[1]), int(step.w3.shape[2]), int(step.ws.shape[2])]},
        "subm_fwd_TFLOP/s": stages["fwd_subm"]["TFLOP/s"],
        "kmap_voxels_per_s": round(kmap_vps, 1),
        "stages": stages,
        "roofline": roof,
        "extras": extras,
    }
    if not args.no_cpu_baseline:
        def stage_flops(name, state):
            cin, c1, cs = inp["w3"].shape[1], inp["w3"].shape[2], inp["ws"].shape[2]
            n = inp["coords"].shape[0]
            return {"fwd_subm": 2 * state.get("P", 0) * cin * c1, "fwd_k1": 2 * n * c1 * inp["w1"].shape[2],
                    "dinput_subm": 2 * state.get("P", 0) * cin * c1, "dfilter_subm": 2 * state.get("P", 0) * cin * c1,
                    "fwd_strided": 2 * state.get("Ps", 0) * cin * cs,
                    "dinput_strided": 2 * state.get("Ps", 0) * cin * cs,
                    "dfilter_strided": 2 * state.get("Ps", 0) * cin * cs}.get(name, 0)
        out["cpu_baseline"] = cpu_baseline(inp, stage_flops, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
