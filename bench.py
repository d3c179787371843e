#!/usr/bin/env python3
"""Throughput of the gated N-D FFT convolution on one MI355X.

One step = one ``hyenand_fftconv_fwd`` over the whole synthetic batch (gate,
forward transforms, product with the precomputed kernel spectrum, inverse
transforms, crop, store), inputs resident in HBM.  Default workload: the 256x256
image, B=8, C=64, fp32 I/O.  With ``--pass bwd`` a step is one
``hyenand_fftconv_bwd`` (dx, dalpha, dbeta and dK for a synthetic output
gradient).  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload NAME] [--pass fwd|bwd]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Gvoxel·channels/s of gated N-D FFT conv fwd; % of HBM roofline (1 GPU)"
METRIC_CIRC = "Gvoxel·channels/s of gated N-D FFT conv fwd, circular mode; % of HBM roofline (1 GPU)"
METRIC_PS = "Gvoxel·channels/s of gated N-D FFT conv fwd, one kernel per (b, c); % of HBM roofline (1 GPU)"
METRIC_GEN = ("Gvoxel·channels/s of gated N-D FFT conv fwd with input-dependent kernels generated in the step; "
              "% of HBM roofline (1 GPU)")
METRIC_BWD = "Gvoxel·channels/s of gated N-D FFT conv bwd (dx, dalpha, dbeta, dK); % of HBM roofline (1 GPU)"
METRIC_BWD_PS = ("Gvoxel·channels/s of gated N-D FFT conv bwd (dx, dalpha, dbeta, dK), one kernel per (b, c); "
                 "% of HBM roofline (1 GPU)")
METRIC_BWD_CIRC = ("Gvoxel·channels/s of gated N-D FFT conv bwd (dx, dalpha, dbeta, dK), circular mode; "
                   "% of HBM roofline (1 GPU)")
UNIT = "Gvoxel·channels/s"
HBM_PEAK = 8.0e12            # bytes/s, MI355X HBM3E
# MI355X's published fp32 vector peak (157.3 TFLOP/s: 256 CUs x 2.4 GHz x 256
# flop per CU per clock, counting FMA as two flops and packed-FP32 issue).  This
# build compiles with packed FP32 disabled, so its own ceiling is half of that;
# the roofline is still priced against the published figure.
ALU_PEAK = 157.3e12
SETTLE_S = 0.3               # untimed calls before the warmup steps (GPU clock ramp)
DEFAULT_WORKLOAD = "2d_256x256_b8_c64_f32"
# The second workload with a throughput target (the 128^3 volume), measured by
# the default invocation as well.
SECOND_WORKLOAD = "3d_128x128x128_b1_c32_f32"


def _geom(dims, circ=False):
    """Grid, padded transform lengths (N = 2n, or N = n in circular mode) and
    per-pair / per-channel sizes in complex values."""
    d = len(dims)
    no, nm, ni = (1, 1, dims[0]) if d == 1 else ((dims[0], 1, dims[1]) if d == 2 else tuple(dims))
    f = 1 if circ else 2
    No, Nm, Ni = (f * no if d >= 2 else 1), (f * nm if d == 3 else 1), f * ni
    S = Ni // 2
    return dict(no=no, nm=nm, ni=ni, No=No, Nm=Nm, Ni=Ni, S=S, vox=no * nm * ni, wsp=no * Nm * S if d >= 2 else 0,
                ksz=No * Nm * S + No * Nm, kmain=No * Nm * S,
                kl=no * nm * ni if circ else (2 * no - 1) * (2 * nm - 1) * (2 * ni - 1),
                prune=0 if circ else 1)


def _long_row_len(N):
    """Row length N2 of the long 1-D path's N1 x N2 factorisation of N = 2n."""
    return min(N // 4, 2048) if N <= (1 << 22) else (4096 if N <= (1 << 24) else 8192)


def _fft_flops(N, lines, prune):
    """Nominal flops of `lines` complex length-N transforms: 5 N log2 N, less
    2N for each pruned half (zero half input, or half output unused)."""
    return lines * (5.0 * N * math.log2(N) - 2.0 * N * prune)


def pass_model(name, dims, B_chunk_pairs, nch, es, circ=False):
    """(algorithmic bytes, nominal flops) of one launch of pass `name` over a
    chunk of `B_chunk_pairs` (b,c) pairs covering `nch` channels (circular
    mode: transforms of length n, nothing pruned)."""
    g = _geom(dims, circ)
    P = B_chunk_pairs
    rows = g["no"] * g["nm"]
    pr = g["prune"]
    if name == "row_fwd":
        by = P * g["vox"] * es + P * rows * g["S"] * 8
        fl = _fft_flops(g["Ni"], P * rows / 2, pr) + P * rows * g["S"] * 2 * 2 + P * g["vox"] * 5
    elif name == "row_inv":
        by = P * rows * g["S"] * 8 + P * g["vox"] * es
        fl = _fft_flops(g["Ni"], P * rows / 2, pr) + P * rows * g["S"] * 4
    elif name == "col_mid_fwd" or name == "col_mid_inv":
        by = P * (rows * g["S"] + g["no"] * g["Nm"] * g["S"]) * 8
        fl = _fft_flops(g["Nm"], P * g["no"] * g["S"], pr)
    elif name == "col_out":
        by = 2 * P * g["wsp"] * 8 + nch * g["ksz"] * 8
        lines = P * g["Nm"] * g["S"]
        fl = 2 * _fft_flops(g["No"], lines, pr) + lines * g["No"] * 6
    elif name == "fused2d":
        # x read, y written, K_hat read once per pair (L2 serves the batch after
        # the first); row and column transforms as in the multi-pass passes
        by = 2 * P * g["vox"] * es + nch * g["ksz"] * 8
        rows = g["no"]
        lines = P * g["S"]
        fl = (2 * _fft_flops(g["Ni"], P * rows / 2, pr) + 2 * _fft_flops(g["No"], lines, pr)
              + lines * g["No"] * 6 + P * rows * g["S"] * 8 + P * g["vox"] * 5)
    elif name == "conv1d":
        by = 2 * P * g["vox"] * es + nch * g["ksz"] * 8
        fl = 2 * _fft_flops(g["Ni"], P / 2, pr) + P * g["S"] * (6 + 4) + P * g["vox"] * 5
    # ---- backward passes (dK wanted)
    elif name in ("row_fwd_dy", "row_fwd_u"):
        by = P * g["vox"] * es + P * rows * g["S"] * 8
        fl = _fft_flops(g["Ni"], P * rows / 2, pr) + P * rows * g["S"] * 2 * 2 + (P * g["vox"] * 5 if name == "row_fwd_u" else 0)
    elif name in ("col_mid_fwd_dy", "col_mid_fwd_u"):
        return pass_model("col_mid_fwd", dims, P, nch, es, circ)
    elif name == "col_out_bwd":
        # dy planes read and written, u planes read, K_hat read, kernel-gradient planes written
        by = 3 * P * g["wsp"] * 8 + nch * g["ksz"] * 8 + nch * g["kmain"] * 8
        lines = P * g["Nm"] * g["S"]
        fl = 3 * _fft_flops(g["No"], lines, pr) + lines * g["No"] * (6 + 8) + _fft_flops(g["No"], nch * g["Nm"] * g["S"], 0)
    elif name == "row_inv_bwd":
        by = P * rows * g["S"] * 8 + 2 * P * g["vox"] * es + P * max(rows // 2, 1) * 8
        fl = _fft_flops(g["Ni"], P * rows / 2, pr) + P * rows * g["S"] * 4 + P * g["vox"] * 14
    elif name == "gate_reduce":
        by = P * max(rows // 2, 1) * 8
        fl = P * max(rows // 2, 1) * 2
    elif name == "mid_inv_dk":
        by = 2 * nch * g["kmain"] * 8
        fl = _fft_flops(g["Nm"], nch * g["No"] * g["S"], 0)
    elif name == "dk_row":
        by = (nch * g["kmain"] * 8 if len(dims) > 1 else P * g["S"] * 8) + nch * g["kl"] * 4
        fl = _fft_flops(g["Ni"], nch * g["No"] * g["Nm"] / 2, 0) + nch * g["No"] * g["Nm"] * g["S"] * 4
    elif name == "conv1d_bwd":
        by = 3 * P * g["vox"] * es + nch * g["ksz"] * 8 + P * 8
        fl = 2 * _fft_flops(g["Ni"], P / 2, pr) + P * g["S"] * (6 + 4) + P * g["vox"] * 14
    # ---- long 1-D (four-step: N = 2n = N1 x N2, complex arithmetic)
    elif name == "lng_col_fwd":
        N = 2 * g["ni"]
        N2 = _long_row_len(N)
        by = P * g["vox"] * es + P * N * 8
        fl = P * N2 * (5.0 * (N // N2) * math.log2(N // N2) - 2.0 * (N // N2)) + P * N * 6 + P * g["vox"] * 5
    elif name == "lng_row":
        N = 2 * g["ni"]
        N2 = _long_row_len(N)
        by = 2 * P * N * 8 + nch * N * 8
        fl = 2 * P * (N // N2) * 5.0 * N2 * math.log2(N2) + P * N * 6
    elif name == "lng_col_inv":
        N = 2 * g["ni"]
        N2 = _long_row_len(N)
        by = P * N * 8 + P * g["vox"] * es
        fl = P * N2 * (5.0 * (N // N2) * math.log2(N // N2) - 2.0 * (N // N2)) + P * N * 6
    elif name in ("lng_col_fwd_dy", "lng_col_fwd_u"):
        by, fl = pass_model("lng_col_fwd", dims, P, nch, es, circ)
        if name == "lng_col_fwd_dy":
            fl -= P * g["vox"] * 5  # no gate
    elif name == "lng_row_du":
        return pass_model("lng_row", dims, P, nch, es, circ)
    elif name == "lng_row_dk":
        # dy and u rows read, the channel's kernel-gradient rows written; with
        # 4096-point rows (N > 2^22) also the spectrum read and the du rows written
        N = 2 * g["ni"]
        N2 = _long_row_len(N)
        by = 2 * P * N * 8 + nch * N * 8
        fl = (2 * P + nch) * (N // N2) * 5.0 * N2 * math.log2(N2) + P * N * 8
        if N2 >= 4096:
            by += P * N * 8 + nch * N * 8
            fl += P * (N // N2) * 5.0 * N2 * math.log2(N2) + P * N * 6
    elif name == "lng_col_inv_bwd":
        by, fl = pass_model("lng_col_inv", dims, P, nch, es, circ)
        by += P * g["vox"] * es  # x read again for the gate derivative
        fl += P * g["vox"] * 14
    elif name == "lng_col_dk":
        N = 2 * g["ni"]
        N2 = _long_row_len(N)
        by = nch * N * 8 + nch * (2 * g["ni"] - 1) * 4
        fl = nch * N2 * 5.0 * (N // N2) * math.log2(N // N2) + nch * N * 6
    elif name == "corr1d":
        by = 2 * P * g["vox"] * es + P * g["S"] * 8
        fl = _fft_flops(g["Ni"], P, pr) + P * g["S"] * 10 + P * g["vox"] * 5
    else:
        raise KeyError(name)
    return by, fl


KERNEL_LABEL = {"row_fwd": "k_row_fwd", "row_inv": "k_row_inv", "col_out": "k_col_out", "col_mid_fwd": "k_col_mid",
                "col_mid_inv": "k_col_mid", "conv1d": "k_conv1d", "row_fwd_dy": "k_row_fwd", "row_fwd_u": "k_row_fwd",
                "col_mid_fwd_dy": "k_col_mid", "col_mid_fwd_u": "k_col_mid", "col_out_bwd": "k_col_out_bwd",
                "row_inv_bwd": "k_row_inv", "gate_reduce": "k_gate_reduce", "mid_inv_dk": "k_plane_mid_inv",
                "dk_row": "k_dk_row", "conv1d_bwd": "k_conv1d", "corr1d": "k_corr1d", "lng_col_fwd": "k_lng_col_fwd",
                "lng_row": "k_lng_prod", "lng_col_inv": "k_lng_col_inv", "lng_col_fwd_dy": "k_lng_col_fwd",
                "lng_col_fwd_u": "k_lng_col_fwd", "lng_row_dk": "k_lng_prod_dk", "lng_row_du": "k_lng_prod",
                "lng_col_inv_bwd": "k_lng_col_inv", "lng_col_dk": "k_lng_col_dk", "fused2d": "k_fused2d"}


# The sources of the zero-padded forward's kernels and of its planning (the
# traffic record stays valid while none of them changes).
FWD_SOURCES = ("api.cpp", "conv_bodies.h", "fft_core.h", "fused2d.h", "k_fused2d_bf16.hip", "k_fused2d_f32.hip",
               "k_fwd.hip", "k_spec.hip", "kernels_dev.h", "launch.h", "plan.h")


def _src_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dimensional_fft_long_amd", "csrc")
    for f in FWD_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def write_traffic_record(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mb, workload, out_json):
    """The HBM traffic record that `roofline.traffic` reads: FETCH_SIZE and
    WRITE_SIZE per dispatch (KiB, from two rocprofv3 --pmc runs of the bench
    on `workload`), each scaled by what the same counter reads for a
    device-to-device copy of copy_mb MiB (two more runs of --copy-probe-mb),
    averaged per kernel."""
    import csv
    import re
    import statistics

    import dimensional_fft_long_amd as H
    import synth
    import torch

    def per_kernel(path):
        out = {}
        for r in csv.DictReader(open(path)):
            m = re.search(r"::(k_\w+)<", r["Kernel_Name"]) or re.search(r"(copyBuffer)", r["Kernel_Name"])
            if m:
                out.setdefault(m.group(1), []).append(float(r["Counter_Value"]))
        return {k: statistics.mean(v) for k, v in out.items()}

    n = copy_mb << 20
    f_scale = n / (per_kernel(copy_fetch_csv)["copyBuffer"] * 1024)
    w_scale = n / (per_kernel(copy_write_csv)["copyBuffer"] * 1024)
    fe, wr = per_kernel(fetch_csv), per_kernel(write_csv)
    wl = {w.name: w for w in synth.WORKLOADS}[workload]
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    per_ch = H.workspace_bytes(wl.B, wl.C, wl.dims, dt, minimum=True)
    nch = wl.C
    if per_ch:
        nch = min(wl.C, H.workspace_bytes(wl.B, wl.C, wl.dims, dt) // per_ch)
        nch = -(-wl.C // -(-wl.C // nch))
    kernels = {}
    for k in sorted(set(fe) & set(wr)):
        rd, wt = fe[k] * 1024 * f_scale, wr[k] * 1024 * w_scale
        kernels[k] = {"fetch_kib": fe[k], "write_kib": wr[k], "read_bytes": rd, "write_bytes": wt,
                      "traffic_bytes_per_launch": rd + wt}
    rec = {"source_hash": _src_hash(), "workload": workload, "chunk_channels": nch, "copy_probe_bytes": n,
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": kernels}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def _traffic_from_profile(kernel_name, workload, chunk_channels):
    """HBM bytes per launch of `kernel_name` from a committed rocprofv3 PMC
    record (profiles/pmc_traffic*.json, one per workload: FETCH_SIZE and
    WRITE_SIZE scaled by what they read for a copy of known size), if it was
    taken on the current kernel sources and the same workload; else None."""
    import glob

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "pmc_traffic*.json"))):
        try:
            rec = json.load(open(path))
        except ValueError:
            continue
        if (rec.get("source_hash") == _src_hash() and rec.get("workload") == workload
                and rec.get("chunk_channels") == chunk_channels):
            return rec.get("kernels", {}).get(kernel_name, {}).get("traffic_bytes_per_launch")
    return None


def cpu_baseline(wl, circ=False, max_seconds=20.0):
    """The fp64 oracle (O2 FFT route, as written; its circular route in
    circular mode) on a bounded sample of the same workload: consecutive (b,c)
    pairs until about `max_seconds` pass."""
    import numpy as np

    import oracle
    import synth

    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype).float().numpy()
    K = (synth.circular_kernel(wl.dims, p) if circ else synth.kernel_channels(wl.dims, p)).numpy()
    route = oracle.fftconv_circ if circ else oracle.fftconv
    done = 0
    t_total = 0.0
    batch = 1
    while t_total < max_seconds and done < wl.B * wl.C:
        pairs = np.arange(done, min(done + batch, wl.B * wl.C))
        t0 = time.perf_counter()
        route(x, p.alpha, p.beta, K, pairs=pairs)
        t_total += time.perf_counter() - t0
        done += len(pairs)
        batch = min(batch * 2, 64)
    vox = done * wl.voxels
    return {"value": vox / t_total / 1e9, "unit": UNIT, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} of {wl.B * wl.C} (b,c) pairs of {wl.name}, fp64 O2 (radix-2 FFT) route"
                      f"{', circular' if circ else ''}, "
                      f"{t_total:.1f} s"}


def cpu_baseline_bwd(wl, circ=False, max_seconds=20.0):
    """The fp64 oracle's backward (O2 FFT route, as written; its circular
    route in circular mode) on a bounded sample of the same workload: whole
    channels (every batch entry) until about `max_seconds` pass."""
    import oracle
    import synth

    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype).float().numpy()
    dy = synth.draw_dy(wl.dims, wl.B, wl.C, wl.dtype, wl.seed).float().numpy()
    done = 0
    t_total = 0.0
    while t_total < max_seconds and done < wl.C:
        c = done
        if circ:
            K = synth.circular_kernel(wl.dims, p).numpy()[c:c + 1]
        else:
            K = synth.kernel_channels(wl.dims, p, channels=[c]).numpy()
        t0 = time.perf_counter()
        (oracle.bwd_fft_circ if circ else oracle.bwd_fft)(x[:, c:c + 1], p.alpha[c:c + 1], p.beta[c:c + 1], K,
                                                          dy[:, c:c + 1])
        t_total += time.perf_counter() - t0
        done += 1
    vox = done * wl.B * wl.voxels
    return {"value": vox / t_total / 1e9, "unit": UNIT, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} of {wl.C} channels (all {wl.B} batch entries each) of {wl.name}, fp64 O2 backward "
                      f"(radix-2 FFT) route{', circular' if circ else ''}, {t_total:.1f} s"}


def _alg_bytes(name, wl, nch_pairs, nch, es, circ=False, ps=False):
    """Algorithmic bytes of one launch of pass `name`: the method's own
    traffic only (x read, K_hat read, y written, and in the backward dy read,
    dx and dK written), never the workspace that the passes hand each other."""
    g = _geom(wl.dims, circ)
    P = nch_pairs
    kbytes = nch * (2 * wl.dims[0] if (wl.d == 1 and wl.dims[0] > 1024) else g["ksz"]) * 8
    xb = P * g["vox"] * es
    table = {"row_fwd": xb, "row_inv": xb, "col_out": kbytes, "conv1d": 2 * xb + kbytes,
             "col_mid_fwd": 0, "col_mid_inv": 0, "lng_col_fwd": xb, "lng_row": kbytes, "lng_col_inv": xb,
             "plane_fwd": xb, "plane_inv": xb, "fused2d": 2 * xb + kbytes,
             "row_fwd_dy": xb, "row_fwd_u": xb, "col_mid_fwd_dy": 0, "col_mid_fwd_u": 0,
             "col_out_bwd": kbytes, "row_inv_bwd": 2 * xb, "gate_reduce": 0, "mid_inv_dk": 0,
             "dk_row": nch * g["kl"] * 4, "conv1d_bwd": 3 * xb + kbytes, "corr1d": 2 * xb,
             "lng_col_fwd_dy": xb, "lng_col_fwd_u": xb, "lng_row_dk": 0, "lng_row_du": kbytes,
             "lng_col_inv_bwd": 2 * xb, "lng_col_dk": nch * g["kl"] * 4}
    return table[name]


def run_workload(H, wl, which="fwd", boundary="padded", kernel="shared", steps=50, warmup=10, settle_s=SETTLE_S,
                 ws_mb=None, with_cpu=True):
    """Time one workload; returns the fields of its JSON line."""
    import numpy as np
    import torch

    import synth

    circ = boundary == "circular"
    gen_mode = kernel == "generated"
    ps = kernel == "per-sample" or gen_mode
    dev = torch.device("cuda:0")
    es = 2 if wl.dtype == "bf16" else 4

    # Inputs of record: seeded parameters and x on the host, kernel evaluated on the device.
    p = synth.draw_params(wl.dims, wl.C, wl.seed)
    x = synth.draw_x(p.rng, wl.B, wl.C, wl.dims, wl.dtype).to(dev)
    K = synth.circular_kernel(wl.dims, p, device=dev) if circ else synth.kernel_channels(wl.dims, p, device=dev)
    if ps:
        # One kernel per (b, c): the channel's kernel scaled and shifted by a
        # seeded per-sample factor (a stand-in for the FiLM modulation).
        rng_ps = np.random.Generator(np.random.PCG64([wl.seed, 3]))
        gsc = torch.from_numpy(rng_ps.uniform(0.5, 1.5, (wl.B, wl.C)).astype(np.float32)).to(dev)
        gsh = torch.from_numpy(rng_ps.uniform(-0.1, 0.1, (wl.B, wl.C)).astype(np.float32)).to(dev)
        shape = (wl.B, wl.C) + (1,) * len(wl.dims)
        K = (K.unsqueeze(0) * gsc.reshape(shape) + gsh.reshape(shape)).contiguous()
    al = torch.from_numpy(p.alpha).to(dev)
    be = torch.from_numpy(p.beta).to(dev)
    if gen_mode:
        # Input-dependent kernels generated from x on the GPU at every step
        # (registers -> control -> FiLM SIREN -> window, into the spectra).
        gen = {k: (torch.from_numpy(v).to(dev) if isinstance(v, np.ndarray) else v)
               for k, v in synth.draw_generator(wl.dims, wl.C, wl.seed).items()}
        kh_gen = torch.empty(H.spectrum_bytes(wl.B * wl.C, wl.dims) // 8, dtype=torch.complex64,
                             device=dev).view(wl.B * wl.C, -1)
        gws = torch.empty(H.generated_workspace_bytes(wl.B, wl.C, wl.dims, x.dtype), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def spectrum():
        if gen_mode:
            return H.generate_kernel_spectrum(x, gen, out=kh_gen)
        return H.kernel_spectrum_circ(K) if circ else (H.kernel_spectrum_per_sample(K) if ps else H.kernel_spectrum(K))

    kh = spectrum()  # the first call also loads the spectrum kernels' code
    torch.cuda.synchronize()
    s0.record()
    kh = spectrum()
    s1.record()
    torch.cuda.synchronize()
    spectrum_ms = s0.elapsed_time(s1)
    del K
    bwd = which == "bwd"
    if bwd:
        dy = synth.draw_dy(wl.dims, wl.B, wl.C, wl.dtype, wl.seed).to(dev)
        kshape = ((wl.B,) if ps else ()) + (wl.C,) + (tuple(wl.dims) if circ else tuple(2 * n - 1 for n in wl.dims))
        outs = (torch.empty_like(x), torch.empty(wl.C, device=dev), torch.empty(wl.C, device=dev),
                torch.empty(kshape, device=dev))
        B_ws = 1 if ps else wl.B  # the per-sample backward runs the batch entries one at a time
        ws_bytes = H.bwd_workspace_bytes(B_ws, wl.C, wl.dims, x.dtype, circular=circ)
        if ws_mb is not None:
            ws_bytes = max(H.bwd_workspace_bytes(B_ws, wl.C, wl.dims, x.dtype, minimum=True, circular=circ),
                           int(ws_mb * 2**20))
    elif circ:
        y = torch.empty_like(x)
        ws_bytes = H.circ_workspace_bytes(wl.B, wl.C, wl.dims, x.dtype)
        if ws_mb is not None:
            ws_bytes = max(H.circ_workspace_bytes(wl.B, wl.C, wl.dims, x.dtype, minimum=True), int(ws_mb * 2**20))
    else:
        y = torch.empty_like(x)
        ws_bytes = H.workspace_bytes(wl.B, wl.C, wl.dims, x.dtype)
        if ws_mb is not None:
            ws_bytes = max(H.workspace_bytes(wl.B, wl.C, wl.dims, x.dtype, minimum=True), int(ws_mb * 2**20))
    ws = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device=dev)

    def call():
        if bwd:
            f = H.fftconv_bwd_circ if circ else (H.fftconv_bwd_per_sample if ps else H.fftconv_bwd)
            f(x, al, be, kh, dy, *outs, workspace=ws)
        elif circ:
            H.fftconv_fwd_circ(x, al, be, kh, y=y, workspace=ws)
        elif gen_mode:
            H.fftconv_fwd_generated(x, al, be, gen, K_hat=kh_gen, y=y, workspace=gws)
        elif ps:
            H.fftconv_fwd_per_sample(x, al, be, kh, y=y, workspace=ws)
        else:
            H.fftconv_fwd(x, al, be, kh, y=y, workspace=ws)

    def traced(events):
        if bwd:
            return H.fftconv_bwd_traced(x, al, be, kh, dy, outs, ws, events, circular=circ, per_sample=ps)
        if circ:
            return H.fftconv_fwd_circ_traced(x, al, be, kh, y, ws, events)
        if ps:
            return H.fftconv_fwd_per_sample_traced(x, al, be, kh, y, ws, events)
        return H.fftconv_fwd_traced(x, al, be, kh, y, ws, events)

    # Launch count per step, then one event slot before each launch and one at the end.
    probe = [torch.cuda.Event(enable_timing=True) for _ in range(1)]
    n_launch = traced(probe)
    torch.cuda.synchronize()
    # Clock settle (untimed): the GPU needs tens of milliseconds of load to
    # reach its steady clock (256^2: the first ~20 ms of calls run ~10% slower),
    # so calls repeat for at least settle_s before the W warmup steps.
    t0 = time.perf_counter()
    settle_calls = 0
    while time.perf_counter() - t0 < settle_s:
        for _ in range(8):
            call()
        settle_calls += 8
        torch.cuda.synchronize()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` plain calls, bracketed by synchronisations.
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(steps):
        call()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / steps

    gen_compare = None
    if gen_mode:
        # The same step as two calls (generator for every pair, then the
        # forward), the forward alone and the generator alone, for comparison.
        def timed(fn):
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a0.record()
            for _ in range(steps):
                fn()
            a1.record()
            torch.cuda.synchronize()
            return a0.elapsed_time(a1) / steps

        def sequential():
            H.generate_kernel_spectrum(x, gen, out=kh_gen)
            H.fftconv_fwd_per_sample(x, al, be, kh_gen, y=y, workspace=ws)

        gen_compare = {"sequential_ms_per_step": timed(sequential),
                       "forward_alone_ms_per_step": timed(lambda: H.fftconv_fwd_per_sample(x, al, be, kh_gen, y=y,
                                                                                            workspace=ws)),
                       "generator_alone_ms": timed(lambda: H.generate_kernel_spectrum(x, gen, out=kh_gen))}

    # Per-kernel durations: the same `steps` calls again through the traced
    # entry point, which records HIP events on the launch stream between kernels.
    # The traced calls are enqueued behind `steps` plain calls, with no host
    # synchronisation between: the GPU stays loaded (at its steady clock; an
    # idle gap before them, or a spin kernel, measured 10-15% slower kernels)
    # while the host submits them.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_launch + 1)] for _ in range(steps)]
    for _ in range(steps):
        call()
    for k in range(steps):
        traced(evs[k])
    torch.cuda.synchronize()
    # The interval between two events around a kernel also holds the
    # processing of one event marker; measured here as the interval between
    # two markers with nothing in between, then taken off each kernel's.
    mk = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    st = torch.cuda.current_stream()
    for _ in range(steps):
        call()
    for k in range(steps):
        mk[2 * k].record(st)
        mk[2 * k + 1].record(st)
    torch.cuda.synchronize()
    marker_ms = sorted(mk[2 * k].elapsed_time(mk[2 * k + 1]) for k in range(steps))[steps // 2]

    # Cold-cache steps (secondary figure): a 1 GiB buffer is rewritten before
    # each call, evicting the 256 MB Infinity Cache and the L2s, so every input
    # comes from HBM.  Percentiles over `steps` single calls.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for k in range(steps):
        flush.fill_(float(k))
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(st)
        call()
        c1.record(st)
        cold.append((c0, c1))
    torch.cuda.synchronize()
    cold_ms = sorted(c0.elapsed_time(c1) for c0, c1 in cold)
    del flush

    g = _geom(wl.dims, circ)
    long1d = wl.d == 1 and wl.dims[0] > 1024
    if bwd:
        per_ch = H.bwd_workspace_bytes(B_ws, wl.C, wl.dims, x.dtype, minimum=True, circular=circ)
        nch = min(wl.C, ws_bytes // per_ch)
        nch = -(-wl.C // -(-wl.C // nch))  # balanced chunks, as the library splits them
        # x, dy and dx once, K_hat once, dK once (alpha, beta, dalpha, dbeta negligible)
        nk = wl.C * (wl.B if ps else 1)
        bytes_min = 3 * wl.B * wl.C * wl.voxels * es + nk * g["ksz"] * 8 + nk * g["kl"] * 4
        names = H.BWD_PASS_NAMES[(("long4096" if 2 * wl.dims[0] > (1 << 22) else "long") if long1d else wl.d, True)]
        if long1d:
            bytes_min = 3 * wl.B * wl.C * wl.voxels * es + wl.C * 2 * wl.dims[0] * 8 + wl.C * g["kl"] * 4
    else:
        per_ch = (H.circ_workspace_bytes if circ else H.workspace_bytes)(wl.B, wl.C, wl.dims, x.dtype, minimum=True)
        if per_ch > 0:
            nch = min(wl.C, ws_bytes // per_ch)
            nch = -(-wl.C // -(-wl.C // nch))  # balanced chunks, as the library splits them
        else:
            nch = wl.C
        ksz = 2 * wl.dims[0] if long1d else g["ksz"]
        bytes_min = 2 * wl.B * wl.C * wl.voxels * es + wl.C * ksz * 8 * (wl.B if ps else 1)
        names = ("lng_col_fwd", "lng_row", "lng_col_inv") if long1d else H.pass_names(wl.dims, circ)
    per_pass = {nm: [] for nm in names}
    step_ms = []
    for k in range(steps):
        e = evs[k]
        step_ms.append(e[0].elapsed_time(e[-1]))
        for j in range(n_launch):
            per_pass[names[j % len(names)]].append(e[j].elapsed_time(e[j + 1]) - marker_ms)
    dominant = max(per_pass, key=lambda nm: sum(per_pass[nm]))
    dom_s = sum(per_pass[dominant]) / len(per_pass[dominant]) / 1e3
    if bwd and ps:  # one batch entry per launch, its own spectra
        P_l, nk_l = nch, nch
    else:
        P_l, nk_l = nch * wl.B, nch * (wl.B if ps else 1)
    moved, fl = pass_model(dominant, wl.dims, P_l, nk_l, es, circ)
    alg = _alg_bytes(dominant, wl, P_l, nk_l, es, circ, ps)
    kernel_label = KERNEL_LABEL[dominant]
    hbm = {"bound": "hbm", "achieved": alg / dom_s / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    alu = {"bound": "alu", "achieved": fl / dom_s / 1e12, "peak": ALU_PEAK / 1e12, "unit": "TFLOP/s"}
    for r in (hbm, alu):
        r["frac"] = r["achieved"] / r["peak"]
    roof = hbm if hbm["frac"] >= alu["frac"] else alu
    traffic = None if (circ or ps) else _traffic_from_profile(kernel_label, wl.name, nch)
    roof.update({"traffic": traffic, "kernel": kernel_label, "avg_us": dom_s * 1e6,
                 "traffic_over_algorithmic": (traffic / alg) if (traffic and alg) else None,
                 "design_bytes_per_launch": moved})
    roof["other_bound"] = {k: v for k, v in (alu if roof is hbm else hbm).items()}

    voxch = wl.B * wl.C * wl.voxels
    out = {
        "value": voxch / (ms_per_step / 1e3) / 1e9,
        "ms_per_step": ms_per_step,
        "config": {"workload": wl.name, "pass": which, "boundary": boundary, "kernel": kernel,
                   "grid": list(wl.dims), "padded": [n if circ else 2 * n for n in wl.dims], "B": wl.B,
                   "C": wl.C, "io_dtype": "bf16" if wl.dtype == "bf16" else "fp32",
                   "launches_per_step": n_launch, "workspace_mib": ws_bytes / 2**20, "chunk_channels": nch},
        "hbm_roofline_frac_of_metric": bytes_min / (ms_per_step / 1e3) / HBM_PEAK,
        "bytes_min": bytes_min,
        "traced_step_ms_median": sorted(step_ms)[len(step_ms) // 2],
        "traced_step_ms_p10_p90": [sorted(step_ms)[len(step_ms) // 10], sorted(step_ms)[(9 * len(step_ms)) // 10]],
        "cold_cache_ms_per_step": {"median": cold_ms[len(cold_ms) // 2], "p10": cold_ms[len(cold_ms) // 10],
                                   "p90": cold_ms[(9 * len(cold_ms)) // 10]},
        "per_kernel_us": {nm: 1e3 * sum(v) / len(v) for nm, v in per_pass.items()},
        "event_marker_us": 1e3 * marker_ms,
        "settle_calls": settle_calls,
        "spectrum_ms": spectrum_ms,
        "roofline": roof,
    }
    if gen_compare:
        out["generated"] = gen_compare
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline_bwd(wl, circ) if bwd else cpu_baseline(wl, circ)
    return out


def copy_bandwidth(mib=1024, reps=10):
    """Device-to-device copy bandwidth (read + write bytes per second) on this
    GPU, as context for the HBM figures (the roofline peak stays 8 TB/s)."""
    import torch

    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    return 2 * (mib << 20) * reps / (a.elapsed_time(b) / 1e3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward with the kernel gradient")
    ap.add_argument("--boundary", choices=("padded", "circular"), default="padded",
                    help="zero-padded non-circular convolution (default) or the circular mode")
    ap.add_argument("--kernel", choices=("shared", "per-sample", "generated"), default="shared",
                    help="one kernel per channel (default), one per (b, c) (input-dependent kernels, "
                         "zero-padded mode only), or one per (b, c) generated from x on the GPU inside every "
                         "step (registers, FiLM SIREN, Gaussian window; the step then includes the generator)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", default=None,
                    help="comma-separated further workloads measured the same way and reported under "
                         f"'also' (default for the default invocation: {SECOND_WORKLOAD}; 'none' for none)")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of untimed calls before the warmup (0 for profiler runs)")
    ap.add_argument("--ws-mb", type=float, default=None,
                    help="workspace size in MiB (default: the library's recommendation)")
    ap.add_argument("--copy-probe-mb", type=int, default=None,
                    help="only run 5 device-to-device copies of this many MiB (a kernel of known HBM "
                         "traffic, to scale the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--traffic-record", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "OUT_JSON"),
                    help="write the HBM traffic record of --workload from rocprofv3 counter_collection CSVs "
                         "(the bench's FETCH_SIZE and WRITE_SIZE runs and the --copy-probe-mb runs, "
                         "copy size --copy-probe-mb, default 256) and exit (no GPU work)")
    args = ap.parse_args()
    if args.traffic_record:
        fc, wc, cfc, cwc, out_json = args.traffic_record
        rec = write_traffic_record(fc, wc, cfc, cwc, args.copy_probe_mb or 256, args.workload, out_json)
        print(json.dumps({k: v for k, v in rec.items() if k != "kernels"}))
        return 0
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "channel with no communication, but no multi-GPU run is part of it.", file=sys.stderr)
        return 2

    import torch

    if args.copy_probe_mb is not None:
        n = args.copy_probe_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "copies": 5}))
        return 0

    import dimensional_fft_long_amd as H
    import synth

    if args.boundary == "circular" and args.kernel != "shared":
        print("bench.py: per-sample kernels are built for the zero-padded mode only", file=sys.stderr)
        return 2
    if args.which == "bwd" and args.kernel == "generated":
        print("bench.py: the generated-kernel step is timed for the forward only", file=sys.stderr)
        return 2
    torch.cuda.set_device(torch.device("cuda:0"))
    by_name = {w.name: w for w in synth.WORKLOADS}
    wl = by_name[args.workload]
    main_run = run_workload(H, wl, args.which, args.boundary, args.kernel, args.steps, args.warmup, args.settle_s,
                            args.ws_mb, with_cpu=not args.no_cpu_baseline)
    circ, ps, bwd = args.boundary == "circular", args.kernel != "shared", args.which == "bwd"
    out = {
        "metric": ((METRIC_BWD_CIRC if circ else (METRIC_BWD_PS if ps else METRIC_BWD)) if bwd
                   else (METRIC_CIRC if circ else (METRIC_GEN if args.kernel == "generated"
                                                   else (METRIC_PS if ps else METRIC)))),
        "value": main_run.pop("value"),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_run.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type of every transform, product and gate (bf16
        # workloads read and write bf16: config.io_dtype)
        "dtype": "f32",
        "data": "synthetic",
    }
    out.update(main_run)
    also = args.also
    if also is None:
        default_call = (args.workload == DEFAULT_WORKLOAD and not circ and not ps and not bwd)
        also = SECOND_WORKLOAD if default_call else "none"
    extra = {}
    for name in [a for a in also.split(",") if a and a != "none"]:
        r = run_workload(H, by_name[name], args.which, args.boundary, args.kernel, args.steps, args.warmup,
                         args.settle_s, None, with_cpu=False)
        extra[name] = {k: r[k] for k in ("value", "ms_per_step", "hbm_roofline_frac_of_metric", "bytes_min",
                                         "cold_cache_ms_per_step", "per_kernel_us", "roofline", "config")}
    if extra:
        out["also"] = extra
    out["copy_bandwidth_GBps"] = copy_bandwidth()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
