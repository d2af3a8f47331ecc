#!/usr/bin/env python
"""Throughput of the sparse-convolution hot path on one MI355X.

The headline workload is the mesh-shell sets: 4 samples of 8 one-voxel sphere
shells on 128^3 (N = 266,426), bf16, 128 channels.  One step runs every stage
of the path once on that batch:

    kmap_subm       submanifold kernel map k=3 (hash build + probe + pair lists + order)
    fwd_subm        SubMConv3d k=3 forward 128 -> 128
    fwd_k1          k=1 layer 128 -> 128 on that output
    dinput_subm     dinput of the k=3 layer
    dfilter_subm    dfilter of the k=3 layer
    kmap_strided    strided kernel map k=3 s=2 p=1 (output sites, maps, pairs, both orders)
    fwd_strided     SparseConv3d forward 128 -> 128
    dinput_strided  its dinput
    dfilter_strided its dfilter

value = effective TFLOP/s of the SubMConv3d k=3 forward: 2 * P * Cin * Cout
(P = occupied pairs, counted from the kernel map) over the forward's duration,
the mean of HIP events recorded around it (on its stream) in each of the K
timed steps.  kmap_voxels_per_s = N over the mean duration of the SubM kernel
map (hash table, pair lists, processing order) called 20 times alone between
HIP events; in the step it overlaps the convolutions on a side stream, and
that time is kmap_subm_ms_in_step.  ms_per_step is the wall time of the K
timed steps.
The forward uses weights transposed once at set-up (a layer keeps its weights
in the layout its kernel reads), so the timed forward is one kernel, which is
also the roofline's kernel: its algorithmic FLOP over that mean duration
against the bf16 MFMA peak, and its HBM traffic from the committed rocprofv3
counter runs (profiles/traffic.json, only while the kernel source is the one
measured).

Both kernel maps depend on the coordinates only, so each is built on a stream
of its own (default priority) while the main stream finishes the previous
step; each layer waits for its map.  On the shell sets the strided map starts
after the SubM forward has been issued, so the timed forward runs alone; on
the LiDAR scene, whose step is bound by host time, it starts right after the
SubM map.  A second, untimed pass of K
steps records HIP events around every stage for the per-stage breakdown.

Sections of the same JSON line (``--sections`` picks them):
    lidar_step      the same step on the LiDAR scene (2 x 60k voxels on 41 x
                    1600 x 1408, fp16, 64 -> 64; strided 64 -> 128), timed the
                    same way, with its own roofline (the strided forward, HBM)
    train96         the training step of SubMConv3d k=3, bf16, 96 -> 96 on the
                    shell sets: forward + dinput + dfilter, 3 * 2 * P * 96^2
                    FLOP per step; forward and forward-plus-backward separately
    uniform32_f32   SubMConv3d k=3 fp32 16 -> 16 on 2,000 sites of 32^3: kernel
                    map + forward + backward (latency-bound)
    kmap_tables     each kernel map with the hash and with the index grid
    extras          the layers beyond the path, on the LiDAR step's maps
``--kmap-sweep`` prints kernel-map rates as the scene grows instead.
``cpu_baseline`` times the oracle on the headline metric: the SubM kernel map
and forward on a bounded sample of the same workload, at 1 thread, at most 24
threads and on every core this process may use.
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
# every stage timed back to back: the single-kernel ones, and dfilter, one call of two kernels (the split-K
# partial products over pair segments, k_dfilter, then their fixed-order sum, k_reduce_segs)
CALL_STAGES = SINGLE_KERNEL_STAGES + ("dfilter_subm", "dfilter_strided")
STAGE_KERNELS = {s: "k_conv" for s in SINGLE_KERNEL_STAGES}
STAGE_KERNELS.update(dfilter_subm="k_dfilter + k_reduce_segs", dfilter_strided="k_dfilter + k_reduce_segs")
KERNEL_REPS = 20         # back-to-back launches per single-kernel stage for its duration
BUSY_FILLS = 3           # 1 GiB fills queued ahead of them (~0.5 ms of GPU time)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
SECTIONS = ("lidar_step", "train96", "uniform32_f32", "kmap_tables", "extras", "step_graph")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=("shells", "lidar"), default="shells",
                    help="headline workload (shells: the 128^3 mesh-shell sets, bf16, 128 channels)")
    ap.add_argument("--sections", default=",".join(SECTIONS),
                    help=f"comma-separated sections to add (of {', '.join(SECTIONS)}; 'none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="seconds of oracle work to time at most")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--kmap-sweep", action="store_true",
                    help="instead of the step: kernel-map rates as the scene grows (one line per size)")
    ap.add_argument("--calibration", action="store_true",
                    help="instead of the step: measured MFMA rates (both bf16 shapes, 1-8 waves per SIMD) "
                         "and a streaming-copy HBM rate")
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


def dtype_name(dt) -> str:
    import torch
    return {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}[dt]


def event_pair():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def mean(v):
    return sum(v) / len(v)


# ---------------------------------------------------------------- GPU step

class Step:
    """Holds device inputs and runs the stages of one step through the library."""

    names = ("kmap_subm", "fwd_subm", "fwd_k1", "dinput_subm", "dfilter_subm",
             "kmap_strided", "fwd_strided", "dinput_strided", "dfilter_strided")

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
        # weights in the layout the forward kernels read, made once (a layer
        # keeps them so); dinput reads W as it is
        self.pre = spc.binding._pretranspose(self.x.dtype, self.w3.shape[1], None)
        self.w3t = spc.transpose_weight(self.w3) if self.pre else None
        self.w1t = spc.transpose_weight(self.w1) if self.pre else None
        self.wst = spc.transpose_weight(self.ws) if self.pre else None
        # counts for the FLOP and byte figures, and the strided layer's upstream gradient
        km = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, 2, 1, 1, subm=False, orders=True)
        self.m = km["n_out"]
        self.gs = t(W.grad_for(inp["grad_rng"], self.m, self.ws.shape[2], inp["dtype"]))
        ks = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3)
        self.P = int(ks["pair_ptr"][-1].item())
        self.Ps = int(km["pair_ptr"][-1].item())
        self.side = None             # the kernel maps' streams (created on first use)
        # the strided map after the SubM forward (the forward then runs alone),
        # or right after the SubM map, beside the SubM layer (the host-bound
        # LiDAR step gets its count earlier)
        self.strided_after_fwd = inp["name"].startswith("shells")
        self.km, self.ks = None, km  # maps held for kernel_ms (the SubM one is built on first use)
        # the strided layer of the captured step runs over capacity-sized buffers
        # (the map's geometric bound): its upstream gradient padded with zeros
        self.cap = spc.strided_out_bound(self.n, inp["batch"], inp["shape"], 3, 2, 1, 1)
        self.gs_cap = torch.zeros((self.cap, self.gs.shape[1]), dtype=self.gs.dtype, device=dev)
        self.gs_cap[:self.m] = self.gs

    def fwd(self, x, w, wt, map_, n_rows, subm, order):
        spc = self.spc
        if wt is None:
            if map_ is None:
                return spc.subm_conv_fwd(x, w, None, None)
            if subm:
                return spc.subm_conv_fwd(x, w, None, map_, order)
            return spc.sparse_conv_fwd(x, w, None, map_, n_rows, order)
        return spc.conv_fwd_wt(x, wt, None, map_, n_rows, subm, order)

    def kernel_ms(self, stage: str, reps: int = KERNEL_REPS) -> float:
        """Average duration of one stage's call launched `reps` times back to back
        between two HIP events (the queue never drains, so no host gap counts)."""
        spc, inp = self.spc, self.inp
        if self.km is None:
            self.km = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, orders=True)
        km, ks = self.km, self.ks
        y = self.x if self.w1.shape[1] == self.x.shape[1] else None
        make = {  # stage -> its launch
            "fwd_subm": lambda: self.fwd(self.x, self.w3, self.w3t, km["nbr"], self.n, True, km["order"]),
            "fwd_k1": lambda: self.fwd(y, self.w1, self.w1t, None, self.n, False, None),
            "dinput_subm": lambda: spc.conv_bwd_input(self.g, self.w3, km["nbr"], True, self.n, km["order"]),
            "fwd_strided": lambda: self.fwd(self.x, self.ws, self.wst, ks["nbr"], ks["n_out"], False, ks["order"]),
            "dinput_strided": lambda: spc.conv_bwd_input(self.gs, self.ws, ks["nbr_in"], False, self.n,
                                                         ks["order_in"]),
            "dfilter_subm": lambda: spc.conv_bwd_filter(self.x, self.g, 27, km["pair_ptr"], km["pair_in"],
                                                        km["pair_out"]),
            "dfilter_strided": lambda: spc.conv_bwd_filter(self.x, self.gs, 27, ks["pair_ptr"], ks["pair_in"],
                                                           ks["pair_out"]),
        }[stage]
        return time_launch(self, make, reps)

    def run(self, events=None, timed=None):
        """One step.  Each kernel map depends on the coordinates only, so each
        is built on a stream of its own (default priority) while the main
        stream finishes the previous step; the main stream waits for a map
        (a persistent event) before its layer, and the strided map starts
        after the SubM forward is issued, or after the SubM map
        (strided_after_fwd).  `events` (stage -> pair) records
        every stage; `timed` (stage -> list) gets event pairs around the
        SubM map and forward only."""
        spc, inp, torch = self.spc, self.inp, self.torch
        E = dict(events or {})
        if timed is not None:
            for k in ("kmap_subm", "fwd_subm"):
                E[k] = event_pair()
                timed[k].append(E[k])
        if self.side is None:  # the streams and the events that join them, made once
            self.side = (torch.cuda.current_stream(), torch.cuda.Stream(), torch.cuda.Stream(),
                         torch.cuda.Event(), torch.cuda.Event(), torch.cuda.Event())
        main, side_s, side_k, done_s, done_k, fwd_issued = self.side

        def mark(name, i):
            if name in E:
                E[name][i].record()

        def used_on_main(maps):
            # the main stream reads these maps: their memory is not reused before it is done
            for t in maps.values():
                if isinstance(t, torch.Tensor):
                    t.record_stream(main)

        def strided_map(after):
            torch.cuda.set_stream(side_k)
            side_k.wait_event(after)
            mark("kmap_strided", 0)
            ks = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, 2, 1, 1, subm=False, orders=True)
            mark("kmap_strided", 1)
            done_k.record(side_k)
            torch.cuda.set_stream(main)
            used_on_main(ks)
            return ks

        torch.cuda.set_stream(side_s)
        mark("kmap_subm", 0)
        km = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, orders=True)
        mark("kmap_subm", 1)
        done_s.record(side_s)
        if not self.strided_after_fwd:
            ks = strided_map(done_s)
        torch.cuda.set_stream(main)
        used_on_main(km)
        main.wait_event(done_s)
        mark("fwd_subm", 0)
        y = self.fwd(self.x, self.w3, self.w3t, km["nbr"], self.n, True, km["order"])
        mark("fwd_subm", 1)
        if self.strided_after_fwd:
            fwd_issued.record(main)
            ks = strided_map(fwd_issued)
        mark("fwd_k1", 0)
        self.fwd(y, self.w1, self.w1t, None, self.n, False, None)
        mark("fwd_k1", 1)
        mark("dinput_subm", 0)
        spc.conv_bwd_input(self.g, self.w3, km["nbr"], True, self.n, km["order"])
        mark("dinput_subm", 1)
        mark("dfilter_subm", 0)
        spc.conv_bwd_filter(self.x, self.g, 27, km["pair_ptr"], km["pair_in"], km["pair_out"])
        mark("dfilter_subm", 1)
        main.wait_event(done_k)
        mark("fwd_strided", 0)
        self.fwd(self.x, self.ws, self.wst, ks["nbr"], ks["n_out"], False, ks["order"])
        mark("fwd_strided", 1)
        mark("dinput_strided", 0)
        spc.conv_bwd_input(self.gs, self.ws, ks["nbr_in"], False, self.n, ks["order_in"])
        mark("dinput_strided", 1)
        mark("dfilter_strided", 0)
        spc.conv_bwd_filter(self.x, self.gs, 27, ks["pair_ptr"], ks["pair_in"], ks["pair_out"])
        mark("dfilter_strided", 1)

    def run_captured(self):
        """The step as one HIP graph captures it: the strided map leaves its
        count M on the device (spc_build_kmap_async) and the strided layer is
        sized by the map's capacity (spc_conv_fwd_dev_rows; dinput and dfilter
        read only the first M rows of the capacity-sized gradient).  The maps
        run on streams forked from the current one and joined back, as in
        run(), so a captured graph keeps them beside the convolutions."""
        spc, inp, torch = self.spc, self.inp, self.torch
        if getattr(self, "cap_side", None) is None:
            self.cap_side = (torch.cuda.Stream(), torch.cuda.Stream())
        side_s, side_k = self.cap_side
        main = torch.cuda.current_stream()
        keep = []  # every intermediate stays referenced until the step is issued
        capturing = torch.cuda.is_current_stream_capturing()

        def used_on_main(maps):
            # made on a side stream, read on main: outside a capture the memory
            # must not be reused before main is done (a graph holds its own)
            if not capturing:
                for v in maps.values():
                    if isinstance(v, torch.Tensor):
                        v.record_stream(main)

        def strided_map(after):
            side_k.wait_event(after)
            with torch.cuda.stream(side_k):
                ks = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, 2, 1, 1, subm=False, orders=True,
                                    out_cap=self.cap, device_count=True)
            done = torch.cuda.Event()
            done.record(side_k)
            used_on_main(ks)
            keep.append(ks)
            return ks, done

        start = torch.cuda.Event()
        start.record(main)
        side_s.wait_event(start)
        with torch.cuda.stream(side_s):
            km = spc.build_kmap(self.coords, inp["batch"], inp["shape"], 3, orders=True)
        done_s = torch.cuda.Event()
        done_s.record(side_s)
        used_on_main(km)
        keep.append(km)
        if not self.strided_after_fwd:
            ks, done_k = strided_map(done_s)
        main.wait_event(done_s)
        y = self.fwd(self.x, self.w3, self.w3t, km["nbr"], self.n, True, km["order"])
        if self.strided_after_fwd:
            issued = torch.cuda.Event()
            issued.record(main)
            ks, done_k = strided_map(issued)
        keep.append(y)
        keep.append(self.fwd(y, self.w1, self.w1t, None, self.n, False, None))
        keep.append(spc.conv_bwd_input(self.g, self.w3, km["nbr"], True, self.n, km["order"]))
        keep.append(spc.conv_bwd_filter(self.x, self.g, 27, km["pair_ptr"], km["pair_in"], km["pair_out"]))
        main.wait_event(done_k)
        if self.pre:
            keep.append(spc.conv_fwd_dev_rows(self.x, self.wst, None, ks["nbr"], ks["n_out_dev"], self.cap,
                                              ks["order"], weight_t=True))
        else:
            keep.append(spc.conv_fwd_dev_rows(self.x, self.ws, None, ks["nbr"], ks["n_out_dev"], self.cap,
                                              ks["order"]))
        keep.append(spc.conv_bwd_input(self.gs_cap, self.ws, ks["nbr_in"], False, self.n, ks["order_in"]))
        keep.append(spc.conv_bwd_filter(self.x, self.gs_cap, 27, ks["pair_ptr"], ks["pair_in"], ks["pair_out"]))
        return keep

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
            # the SubM half of the step replayed as one captured HIP graph, and the
            # same calls made one by one
            "subm_step_graph": (self.graph.replay, st_f, st_b),
            "subm_step_eager": (subm_step, st_f, st_b),
            # a 200k-point synthetic sweep into 0.1 x 0.1 x 0.2 m voxels (one call,
            # including its one host synchronisation); bytes: the points read, the
            # voxel block, coordinates, counts and point ids written
            "point_to_voxel": (lambda: spc.point_to_voxel(self.pts, vc["vsize_xyz"], vc["range_xyz"],
                                                          vc["max_voxels"], vc["max_points"], True, with_id=True),
                               0, self.pts.numel() * 4 + vc["max_voxels"] * (vc["max_points"] * self.pts.shape[1] * 4
                                                                            + 16) + self.pts.shape[0] * 4),
        }


def time_launch(holder, launch, reps: int = KERNEL_REPS) -> float:
    """Average duration of one launch repeated back to back between two events.
    Some GPU work is queued first (fills, then one untimed launch that brings
    the caches back), so the host has enqueued every timed launch before the
    first one starts and the host's per-call cost is not timed."""
    import torch
    launch()
    torch.cuda.synchronize()
    if not hasattr(holder, "busy"):
        holder.busy = torch.empty(1 << 30, dtype=torch.uint8, device=holder.dev)
    for _ in range(BUSY_FILLS):
        holder.busy.fill_(1)
    launch()
    a, b = event_pair()
    a.record()
    for _ in range(reps):
        launch()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


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


def stage_rooflines(r: dict, dtype: str, workload: str) -> dict:
    """A roofline entry for every stage timed back to back (kernel_ms)."""
    return {k: roofline(STAGE_KERNELS[k], k, r["flops"][k], r["bytes"][k], ms, dtype, workload)
            for k, ms in r["kernel_ms"].items()}


def roofline(kernel: str, stage: str, flop: float, nbytes: float, ms: float, dtype: str, workload: str) -> dict:
    """Roofline entry of one kernel: bound by MFMA when its arithmetic intensity
    is above the ridge, else by HBM; achieved = algorithmic FLOP (or bytes) per
    launch over the average launch duration `ms`."""
    t = ms * 1e-3
    ridge = MFMA_PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flop / nbytes < ridge:
        r = {"bound": "hbm", "achieved": round(nbytes / t / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": round(flop / t / 1e12, 2), "peak": MFMA_PEAK_TFLOPS[dtype],
             "unit": "TFLOP/s"}
    r["frac"] = round(r["achieved"] / r["peak"], 4)
    r["traffic"] = measured_traffic(workload, stage)
    r["kernel"] = f"{kernel} ({stage})"
    r["algorithmic_bytes_per_launch"] = int(nbytes)
    r["flop_per_launch"] = int(flop)
    r["avg_launch_ms"] = round(ms, 4)
    return r


# ---------------------------------------------------------------- step runs

def run_step(inp, dev, steps, warmup, kernel_stages=True):
    """Warmup, the K timed steps (events around the SubM map and forward only),
    then an instrumented pass of K steps for the per-stage medians."""
    import torch
    step = Step(inp, dev)
    flops, bytes_ = step.work()
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    timed = {"kmap_subm": [], "fwd_subm": []}
    t0 = time.perf_counter()
    for _ in range(steps):
        step.run(timed=timed)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dur = {k: [a.elapsed_time(b) for a, b in v] for k, v in timed.items()}

    events = {k: [event_pair() for _ in range(steps)] for k in step.names}
    for i in range(steps):
        step.run({k: events[k][i] for k in step.names})
    torch.cuda.synchronize()
    stage_ms = {k: sorted(a.elapsed_time(b) for a, b in events[k])[steps // 2] for k in step.names}
    stages = {}
    for k in step.names:
        t = stage_ms[k] * 1e-3
        stages[k] = {"ms": round(stage_ms[k], 4),
                     "TFLOP/s": round(flops[k] / t / 1e12, 2) if k in flops and t > 0 else None,
                     "alg_GB/s": round(bytes_[k] / t / 1e9, 1) if t > 0 else None}
    kernel_ms = {k: step.kernel_ms(k) for k in CALL_STAGES} if kernel_stages else {}
    return step, dict(wall=wall, dur=dur, stages=stages, kernel_ms=kernel_ms, flops=flops, bytes=bytes_)


def graph_step(step, steps, warmup) -> dict:
    """The whole step captured as one HIP graph (Step.run_captured, kernel
    maps on forked streams) and replayed K times between two HIP events,
    against the same launches made eagerly."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the allocator on the capture stream
        for _ in range(max(warmup, 1)):
            step.run_captured()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        held = step.run_captured()  # noqa: F841 (the graph's buffers)
    out = {}
    for name, call in (("graph", graph.replay), ("eager", step.run_captured)):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        a, b = event_pair()
        t0 = time.perf_counter()
        a.record()
        for _ in range(steps):
            call()
        b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        out[f"{name}_ms_per_step"] = round(a.elapsed_time(b) / steps, 4)
        out[f"{name}_host_ms_per_step"] = round(wall * 1e3 / steps, 4)
    return out


def step_summary(inp, step, r, steps, dtype):
    fwd_ms = mean(r["dur"]["fwd_subm"])
    kmap_ms = mean(r["dur"]["kmap_subm"])
    return {
        "workload": inp["name"], "ms_per_step": round(r["wall"] * 1e3 / steps, 4),
        "subm_fwd_TFLOP/s": round(r["flops"]["fwd_subm"] / (fwd_ms * 1e-3) / 1e12, 2),
        "subm_fwd_ms": round(fwd_ms, 4),
        "kmap_voxels_per_s": round(step.n / (kmap_ms * 1e-3), 1), "kmap_subm_ms": round(kmap_ms, 4),
        "n_voxels": step.n, "pairs_subm_k3": step.P, "n_out_strided": step.m, "pairs_strided": step.Ps,
        "channels": [int(step.w3.shape[1]), int(step.w3.shape[2]), int(step.ws.shape[2])], "dtype": dtype,
        "stages": r["stages"], "kernel_ms": {k: round(v, 4) for k, v in r["kernel_ms"].items()},
    }


# ---------------------------------------------------------------- sections

def section_lidar(dev, steps, warmup):
    """The LiDAR scene's step (configs 2 and 4), with the roofline of its
    longest single kernel."""
    inp = make_inputs("lidar")
    step, r = run_step(inp, dev, steps, warmup)
    out = step_summary(inp, step, r, steps, dtype_name(inp["dtype"]))
    dom = max(SINGLE_KERNEL_STAGES, key=lambda k: r["kernel_ms"][k])
    out["roofline"] = roofline("k_conv", dom, r["flops"][dom], r["bytes"][dom], r["kernel_ms"][dom],
                               dtype_name(inp["dtype"]), "lidar")
    out["rooflines"] = stage_rooflines(r, dtype_name(inp["dtype"]), "lidar")
    out["step_graph"] = graph_step(step, steps, warmup)
    return step, out


def section_train96(dev, steps, warmup):
    """SubMConv3d k=3, bf16, 96 -> 96 on the shell sets: forward + dinput +
    dfilter per step (the kernel map built once: the sites do not change
    during training), with forward and forward-plus-backward timed apart."""
    import torch
    import sparse_convolution_hash_amd as spc
    import workloads as W
    w = W.workload("train_subm_k3_bf16_shells96")
    c = torch.from_numpy(w.coords).to(dev)
    x, wt, g = (t.to(dev) for t in (w.feats, w.weight, w.grad))
    km = spc.build_kmap(c, w.batch, w.shape, 3, orders=True)
    P = int(km["pair_ptr"][-1].item())
    K = 27

    def one(ev=None):
        if ev:
            ev[0].record()
        spc.subm_conv_fwd(x, wt, None, km["nbr"], km["order"])   # the weights change every step: no cached transpose
        if ev:
            ev[1].record()
        spc.conv_bwd_input(g, wt, km["nbr"], True, w.n, km["order"])
        spc.conv_bwd_filter(x, g, K, km["pair_ptr"], km["pair_in"], km["pair_out"])
        if ev:
            ev[2].record()

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    t0 = time.perf_counter()
    for e in evs:
        one(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = mean([a.elapsed_time(b) for a, b, _ in evs])
    full = mean([a.elapsed_time(cc) for a, _, cc in evs])
    flop1 = 2 * P * 96 * 96
    return {"workload": "train_shells_4x128^3_bf16_c96", "n_voxels": w.n, "pairs": P, "dtype": "bf16",
            "ms_per_step": round(wall * 1e3 / steps, 4), "fwd_ms": round(fwd, 4), "fwd_bwd_ms": round(full, 4),
            "TFLOP/s": round(3 * flop1 / (full * 1e-3) / 1e12, 2),
            "fwd_TFLOP/s": round(flop1 / (fwd * 1e-3) / 1e12, 2),
            "mfma_frac": round(3 * flop1 / (full * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4)}


def section_uniform32(dev, steps, warmup):
    """SubMConv3d k=3 fp32 16 -> 16 on 2,000 sites of 32^3 with bias: kernel map,
    forward, dinput and dfilter per step (latency-bound at this size)."""
    import torch
    import sparse_convolution_hash_amd as spc
    import workloads as W
    w = W.workload("subm_k3_f32_uniform32", with_grad=True)
    c = torch.from_numpy(w.coords).to(dev)
    x, wt, b, g = (t.to(dev) for t in (w.feats, w.weight, w.bias, w.grad))

    def one(ev=None):
        if ev:
            ev[0].record()
        km = spc.build_kmap(c, w.batch, w.shape, 3, orders=True)
        spc.subm_conv_fwd(x, wt, b, km["nbr"], km["order"])
        if ev:
            ev[1].record()
        spc.conv_bwd_input(g, wt, km["nbr"], True, w.n, km["order"])
        spc.conv_bwd_filter(x, g, 27, km["pair_ptr"], km["pair_in"], km["pair_out"], want_dbias=True)
        if ev:
            ev[2].record()
        return km

    P = int(one()["pair_ptr"][-1].item())
    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    t0 = time.perf_counter()
    for e in evs:
        one(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = mean([a.elapsed_time(bb) for a, bb, _ in evs])
    full = mean([a.elapsed_time(cc) for a, _, cc in evs])
    return {"workload": "uniform_2000_of_32^3_f32_c16", "n_voxels": w.n, "pairs": P, "dtype": "f32",
            "ms_per_step": round(wall * 1e3 / steps, 4), "kmap_fwd_ms": round(fwd, 4),
            "kmap_fwd_bwd_ms": round(full, 4),
            "fwd_TFLOP/s_incl_kmap": round(2 * P * 16 * 16 / (fwd * 1e-3) / 1e12, 4)}


def kmap_time(call, reps):
    """Mean duration of a kernel-map call between HIP events (host time before
    the first launch counts, as a caller sees it)."""
    import torch
    call()
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = event_pair()
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    return mean(ms)


def kmap_bytes(kind, n, m, P, K=27):
    """Algorithmic bytes of a kernel map: coordinates in, maps, pair lists and orders out."""
    if kind == "subm":
        return n * (16 + 4 * K) + 8 * P + 4 * (K + 1) + 4 * n
    return 16 * n + 16 * m + 4 * K * (m + n) + 8 * P + 4 * (K + 1) + 4 * (m + n)


def section_kmap_tables(dev, reps=20):
    """The SubM maps of the LiDAR scene and the shell sets and the LiDAR strided
    map, each with the hash table and with the index grid (pairs and orders)."""
    import torch
    import sparse_convolution_hash_amd as spc
    import workloads as W
    out = {}
    for wname, kinds in (("subm_k3_f16_lidar120k", ("subm", "strided")), ("subm_k3_k1_bf16_shells128", ("subm",))):
        w = W.workload(wname)
        c = torch.from_numpy(w.coords).to(dev)
        for kind in kinds:
            for table in ("hash", "grid"):
                if kind == "subm":
                    call = lambda t=table: spc.build_kmap(c, w.batch, w.shape, 3, orders=True, table=t)
                else:
                    call = lambda t=table: spc.build_kmap(c, w.batch, w.shape, 3, 2, 1, 1, subm=False, orders=True,
                                                          table=t)
                r = call()
                P, m = int(r["pair_ptr"][-1].item()), r["n_out"]
                ms = kmap_time(call, reps)
                by = kmap_bytes(kind, w.n, m, P)
                out[f"{wname.split('_')[-1]}_{kind}_{table}"] = {
                    "ms": round(ms, 4), "voxels_per_s": round(w.n / (ms * 1e-3), 1),
                    "alg_GB/s": round(by / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "n_out": m, "pairs": P}
    return out


def section_extras(step, dtype):
    extras = {}
    ridge = MFMA_PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    for name, (launch, fl, by) in step.extras().items():
        ms = time_launch(step, launch)
        t = ms * 1e-3
        bound = "hbm" if fl / by < ridge else "mfma"
        ach = by / t / 1e9 if bound == "hbm" else fl / t / 1e12
        peak = HBM_PEAK_GBS if bound == "hbm" else MFMA_PEAK_TFLOPS[dtype]
        extras[name] = {"kernel_ms": round(ms, 4), "TFLOP/s": round(fl / t / 1e12, 2) if fl else None,
                        "alg_GB/s": round(by / t / 1e9, 1), "bound": bound, "frac": round(ach / peak, 4)}
    return extras


# ---------------------------------------------------------------- CPU oracle

def cpu_baseline(inp, budget):
    """The oracle on the headline metric: the SubM kernel map of the whole
    workload, then the forward sum over a bounded sample of its output rows
    (FLOP counted from that sample's pairs), at 1 thread, at min(24, cores)
    threads and on every core this process may use."""
    import numpy as np
    import threadpoolctl
    from oracle import conv as OC
    from oracle import kmap as OK

    cores = len(os.sched_getaffinity(0))
    c, sh = inp["coords"], inp["shape"]
    t0 = time.perf_counter()
    nbr = OK.subm_kmap(c, sh, 3)
    t_kmap = time.perf_counter() - t0
    cin, cout = inp["w3"].shape[1], inp["w3"].shape[2]
    feats, w3 = inp["feats"], inp["w3"]
    n = c.shape[0]
    points = sorted({1, min(24, cores), cores})
    per_point = max(1.0, (budget - t_kmap) / len(points))
    res, sample_rows = {}, None
    for th in points:
        with threadpoolctl.threadpool_limits(th):
            rows = 4096 if sample_rows is None else sample_rows
            while True:   # grow the row sample until one forward takes a fair share of the budget
                sub = nbr[:, :rows]
                t0 = time.perf_counter()
                OC.conv_fwd(feats, w3, None, sub)
                dt = time.perf_counter() - t0
                if dt > per_point / 3 or rows >= n or sample_rows is not None:
                    break
                rows = min(n, rows * 4)
            sample_rows = rows
            pairs = int((sub >= 0).sum())
            res[th] = {"TFLOP/s": 2 * pairs * cin * cout / dt / 1e12, "s": dt}
    top = res[cores]
    return {"value": round(top["TFLOP/s"], 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"SubM k=3 forward (numpy fp64) over the first {sample_rows} of {n} output rows "
                      f"({top['s']:.1f} s on {cores} threads), after the oracle's SubM kernel map of all {n} rows",
            "threads": {str(k): round(v["TFLOP/s"], 6) for k, v in res.items()},
            "kmap_voxels_per_s": round(n / t_kmap, 1), "kmap_s": round(t_kmap, 3)}


# ---------------------------------------------------------------- main

def kmap_sweep(reps=10):
    """Kernel-map rate as the scene grows: the 128^3 shell sets at 4..32
    samples and the LiDAR scene at 2..32 samples (k=3 SubM map with pairs and
    order; k3 s2 p1 strided map with pairs and both orders; each with the hash
    and the index grid where the grid fits), one JSON line per size."""
    import torch
    import sparse_convolution_hash_amd as spc
    import workloads as W

    cases = [("shells", B, lambda B=B: W.mesh_shells(W.rng(3), batch=B), (128, 128, 128)) for B in (4, 8, 16, 32)]
    cases += [("lidar", B, lambda B=B: W.lidar_scene(W.rng(20 + B), batch=B), (41, 1600, 1408)) for B in (2, 8, 32)]
    for scene, B, gen, shape in cases:
        c = torch.from_numpy(gen()).cuda()
        n = c.shape[0]
        cells = B * shape[0] * shape[1] * shape[2]
        line = {"kmap_sweep": {"scene": scene, "samples": B, "n_voxels": n}}
        for table in ("hash", "grid"):
            if table == "grid" and cells * 4.125 > 16e9:
                continue
            calls = {
                "subm": lambda t=table: spc.build_kmap(c, B, shape, 3, orders=True, table=t),
                "strided": lambda t=table: spc.build_kmap(c, B, shape, 3, 2, 1, 1, subm=False, orders=True, table=t),
            }
            for name, call in calls.items():
                r = call()
                torch.cuda.synchronize()
                P, m = int(r["pair_ptr"][-1].item()), r["n_out"]
                t = kmap_time(call, reps) * 1e-3
                by = kmap_bytes(name, n, m, P)
                line["kmap_sweep"][f"{name}_{table}"] = {
                    "ms": round(t * 1e3, 4), "voxels_per_s": round(n / t, 1), "n_out": m, "pairs": P,
                    "alg_GB/s": round(by / t / 1e9, 1), "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
                del r
        print(json.dumps(line), flush=True)
        del c
        torch.cuda.empty_cache()


def calibration(iters=4000):
    """Measured rates of this part for reading the roofline: the bf16 MFMA
    shapes' FLOP rate on register operands (spc_calibrate_mfma) at 1, 2, 4 and
    8 waves per SIMD, and a 4 GiB device-to-device copy (read + write bytes over
    time).  One JSON line."""
    import torch
    import sparse_convolution_hash_amd as spc
    dev = torch.device("cuda:0")
    sink = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    out = {"calibration": {"mfma_bf16_TFLOP/s": {}, "published_peak": {"bf16_TFLOP/s": MFMA_PEAK_TFLOPS["bf16"],
                                                                       "hbm_GB/s": HBM_PEAK_GBS}}}
    for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
        for blocks in (256, 512, 1024, 2048):
            spc.calibrate_mfma(shape, blocks, iters, sink)
            torch.cuda.synchronize()
            a, b = event_pair()
            a.record()
            flop = spc.calibrate_mfma(shape, blocks, iters, sink)
            b.record()
            torch.cuda.synchronize()
            tf = flop / (a.elapsed_time(b) * 1e-3) / 1e12
            out["calibration"]["mfma_bf16_TFLOP/s"][f"{name}_{blocks * 4 // 1024}waves_per_simd"] = round(tf, 1)
    x = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    a, b = event_pair()
    a.record()
    for _ in range(5):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    out["calibration"]["copy_GB/s"] = round(5 * 2 * x.numel() / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    print(json.dumps(out), flush=True)


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
    if args.calibration:
        calibration()
        return
    sections = [] if args.sections in ("", "none") else [s for s in args.sections.split(",")]
    bad = [s for s in sections if s not in SECTIONS]
    if bad:
        sys.exit(f"unknown sections {bad}; known: {SECTIONS}")
    dev = torch.device("cuda:0")
    inp = make_inputs(args.workload)
    dtype = dtype_name(inp["dtype"])
    step, r = run_step(inp, dev, args.steps, args.warmup)
    head = step_summary(inp, step, r, args.steps, dtype)
    fwd_ms = head["subm_fwd_ms"]

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bb = torch.empty_like(a)
        bb.copy_(a)
        torch.cuda.synchronize()

    # the kernel-map rate from the SubM map alone (in the step it shares the GPU with the convolutions)
    kmap_alone_ms = kmap_time(lambda: step.spc.build_kmap(step.coords, inp["batch"], inp["shape"], 3, orders=True), 20)
    roof = roofline("k_conv", "fwd_subm", r["flops"]["fwd_subm"], r["bytes"]["fwd_subm"], fwd_ms, dtype,
                    args.workload)
    roof["kernel_ms_back_to_back"] = round(r["kernel_ms"]["fwd_subm"], 4)
    out = {
        "metric": "effective TFLOP/s of SubMConv3d fwd (occupied pairs) + kmap voxels/s, 1 MI355X",
        "value": head["subm_fwd_TFLOP/s"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": inp["name"], "n_voxels": step.n, "pairs_subm_k3": step.P,
                   "n_out_strided": step.m, "pairs_strided": step.Ps,
                   "channels": head["channels"], "kmap_table": "hash"},
        "kmap_voxels_per_s": round(step.n / (kmap_alone_ms * 1e-3), 1),
        "kmap_subm_ms": round(kmap_alone_ms, 4),
        "subm_fwd_ms": fwd_ms,
        "kmap_subm_ms_in_step": head["kmap_subm_ms"],
        "stages": head["stages"],
        "kernel_ms": head["kernel_ms"],
        "roofline": roof,
        "rooflines": stage_rooflines(r, dtype, args.workload),
    }
    lidar_step = None
    if "lidar_step" in sections or "extras" in sections:
        lidar_step, lid = section_lidar(dev, args.steps, args.warmup)
        if "lidar_step" in sections:
            out["lidar_step"] = lid
    if "train96" in sections:
        out["train96"] = section_train96(dev, args.steps, args.warmup)
    if "uniform32_f32" in sections:
        out["uniform32_f32"] = section_uniform32(dev, args.steps, args.warmup)
    if "kmap_tables" in sections:
        out["kmap_tables"] = section_kmap_tables(dev)
    if "step_graph" in sections:
        out["step_graph"] = graph_step(step, args.steps, args.warmup)
    if "extras" in sections:
        out["extras"] = section_extras(lidar_step, dtype_name(lidar_step.x.dtype))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
