"""Benchmark: quantize GB/s (algorithmic bytes in + out) on one MI355X.

One step = one pass of the whole quantizer path over full-size synthetic
inputs already resident in HBM (an MoE layer's worth of quantization work):
  act   MXFP8 row+col of a 2048x2048 BF16 activation
  wgt   MXFP8 row+col of an 8192x2048 BF16 weight
  tok   per-token NVFP4 of 8192x2048 Student-t(3)*0.5 activations, + BF16 dequant
  exp   NVFP4 export of 128 experts (gate/up 768x2048 under one scale per pair,
        down 2048x768 under its own), + BF16 dequant of all three
  grp   grouped MXFP8 row+col and per-token NVFP4 of 262,144 expert-sorted rows
        x 2048 (32,768 tokens routed top-8 of 128), + BF16 dequant of both
Algorithmic bytes count each input read once and each output written once.
Each leg is bracketed by HIP events on the stream the library launches on.

Prints one JSON line.  Extra fields: per-leg GB/s and % of the 8 TB/s HBM
peak ("legs"); per-config timings ("configs": 50 back-to-back launches per
sample over rotating buffer sets larger than the MALL, median and minimum per
launch, for C2a/C2b in four data modes, C3 quantize and dequant, C4 and C5);
the roofline of the dominant kernel; and the CPU oracle timed on the host
cores (all cores over a whole step, one thread over 1/16 of it).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "quantize GB/s (bytes in+out) and % of MI355X HBM peak, MXFP8 row+col & NVFP4"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


CSRC = os.path.join(ROOT, "nvfp4_block_scaled_amax_amd", "csrc")
COMMON_SOURCES = ["mxq_device.h", "mxq_dequant.h", "mxq_launch.h", "mxq_runtime.cpp", "../build.py"]
KERNEL_SOURCES = {
    "mxfp8_tile_kernel": ["mxq_mxfp8.hip"],
    "grouped_prefix_kernel": ["mxq_mxfp8.hip"],
    "nvfp4_token_kernel": ["mxq_nvfp4.hip"],
    "nvfp4_token_split_kernel": ["mxq_nvfp4.hip"],
    "nvfp4_scoped_kernel": ["mxq_nvfp4.hip"],
    "dequant_mxfp8_kernel": ["mxq_dequant.hip"],
    "dequant_nvfp4_kernel": ["mxq_dequant.hip"],
    "mxfp8_gemm_kernel": ["mxq_gemm.hip"],
    "mxfp8_grouped_gemm_kernel": ["mxq_gemm.hip"],
    "mxfp8_grouped_wgrad_kernel": ["mxq_gemm.hip"],
    "mxfp8_grouped_colt_kernel": ["mxq_mxfp8.hip"],
    "mxfp8_colt_staged_kernel": ["mxq_mxfp8.hip"],
    "nvfp4_gemm_kernel": ["mxq_gemm.hip"],
    "nvfp4_grouped_gemm_kernel": ["mxq_gemm.hip"],
    "mxfp8_row_qdq_kernel": ["mxq_mxfp8.hip"],
    "nvfp4_token_qdq_kernel": ["mxq_nvfp4.hip"],
}


def code_text(src: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed to one
    space: what the compiler sees, so that an edit of comments alone (which
    leaves the code object unchanged) keeps a kernel's digest.  String and
    character literals are kept whole."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def csrc_digest(files=None) -> str:
    """Digest of the sources a kernel is built from (all of csrc/ by default):
    the code text of the C/C++ files (code_text) and build.py as it is."""
    if files is None:
        files = sorted(os.listdir(CSRC)) + ["../build.py"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            raw = fh.read()
        body = raw if f.endswith(".py") else code_text(raw.decode()).encode()
        h.update(f.encode() + body)
    return h.hexdigest()[:16]


def kernel_digest(kernel: str) -> str:
    base = kernel.split("<")[0]
    return csrc_digest(KERNEL_SOURCES[base] + COMMON_SOURCES)


class Leg:
    def __init__(self, name, launch, bytes_in, bytes_out, elems, kernels, desc):
        self.name, self.launch = name, launch
        self.bytes_in, self.bytes_out, self.elems = bytes_in, bytes_out, elems
        self.kernels, self.desc = kernels, desc
        self.times_ms = []

    @property
    def bytes(self):
        return self.bytes_in + self.bytes_out


def build_legs(torch, mxq, api, W, log, want=lambda group: True):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    u8 = torch.uint8
    legs = []
    E = mxq

    def empty(shape, dt=u8):
        return torch.empty(shape, dtype=dt, device="cuda")

    # act / wgt: MXFP8 row+col
    for name, rows, cols, gen in (("act", 2048, 2048, W.config2_activation),
                                  ("wgt", 8192, 2048, W.config2_weight)):
        if not want(name):
            continue
        x_np = gen("random")
        x = dev(x_np)
        rc, rs, cc, cs = empty((rows, cols)), empty((rows, cols // 32)), empty((rows, cols)), \
            empty((rows // 32, cols))
        n = rows * cols
        legs.append(Leg(f"mxfp8_rowcol_{name}",
                        (lambda x=x, rows=rows, cols=cols, rc=rc, rs=rs, cc=cc, cs=cs:
                         E.mxq_mxfp8_quantize_rowcol(x, rows, cols, rc, rs, cc, cs)),
                        2 * n, 2 * n + 2 * n // 32, n, ["mxfp8_tile_kernel<true, true, false, 4, false>"],
                        f"MXFP8 row+col {rows}x{cols}"))
    log("act/wgt ready")

    if want("tok"):
        build_tok(torch, E, W, legs, dev, empty)
        log("tok ready")
    if want("exp"):
        build_exp(torch, E, W, legs, dev, empty)
        log("exp ready")
    if want("grp"):
        build_grp(torch, E, W, legs, dev, empty)
        log("grp ready")
    if want("dsp"):
        build_dsp(torch, E, W, legs, dev, empty)
        log("dsp ready")
    if want("qdq"):
        build_qdq(torch, E, W, legs, dev, empty)
        log("qdq ready")
    if want("gemm"):
        build_gemm(torch, E, W, legs, dev, empty)
        log("gemm ready")
    return legs


def build_tok(torch, E, W, legs, dev, empty):
    """Per-token NVFP4 of 8192x2048 Student-t activations, + dequant."""
    rows, cols = 8192, 2048
    x = dev(W.config3())
    n = rows * cols
    codes, bs, ts = empty((rows, cols // 2)), empty((rows, cols // 16)), \
        empty((rows,), torch.float32)
    y = empty((rows, cols), torch.bfloat16)
    q_out = n // 2 + n // 16 + 4 * rows
    legs.append(Leg("nvfp4_tok", lambda: E.mxq_nvfp4_quantize_per_token(x, rows, cols, codes, bs, ts),
                    2 * n, q_out, n, ["nvfp4_token_split_kernel<1, true>"], "NVFP4 per-token 8192x2048"))
    legs.append(Leg("nvfp4_tok_dequant",
                    lambda: E.mxq_dequantize_bf16(E.MXQ_FMT_NVFP4, codes, bs, ts, 1, rows, cols, y),
                    q_out, 2 * n, n, ["dequant_nvfp4_kernel"], "NVFP4 -> BF16 8192x2048"))


def build_exp(torch, E, W, legs, dev, empty):
    """NVFP4 export of 128 experts (gate/up pairs + down), + dequant."""
    gate, up, down = W.config4()
    g, u, dn = dev(gate), dev(up), dev(down)
    NE, I, H = 128, 768, 2048
    # Each scope's largest magnitude as BF16 bits (an integer max), for the
    # export variant that takes the scope amax from the caller.
    amax_pair = np.maximum((gate.reshape(NE, -1) & 0x7FFF).max(1),
                           (up.reshape(NE, -1) & 0x7FFF).max(1)).astype(np.uint16)
    amax_down = (down.reshape(NE, -1) & 0x7FFF).max(1).astype(np.uint16)
    ap, ad = dev(amax_pair), dev(amax_down)
    del gate, up, down
    ng = NE * I * H
    gc, gb, uc, ub = empty((NE, I, H // 2)), empty((NE, I, H // 16)), empty((NE, I, H // 2)), \
        empty((NE, I, H // 16))
    dc, db = empty((NE, H, I // 2)), empty((NE, H, I // 16))
    sp, sd = empty((NE,), torch.float32), empty((NE,), torch.float32)
    yg, yu, yd = empty((NE * I, H), torch.bfloat16), empty((NE * I, H), torch.bfloat16), \
        empty((NE * H, I), torch.bfloat16)
    pair_out = 2 * (ng // 2 + ng // 16) + 4 * NE
    down_out = ng // 2 + ng // 16 + 4 * NE
    legs.append(Leg("nvfp4_export_gateup",
                    lambda: E.mxq_nvfp4_quantize_gateup_pair(g, u, NE, I, H, gc, gb, uc, ub, sp),
                    2 * 2 * ng, pair_out, 2 * ng,
                    ["scope_amax_kernel", "scope_finalize_kernel", "nvfp4_scoped_kernel"],
                    "NVFP4 gate/up export 128x2x768x2048, shared scale per pair"))
    legs.append(Leg("nvfp4_export_down",
                    lambda: E.mxq_nvfp4_quantize_gateup_pair(dn, None, NE, H, I, dc, db, None, None, sd),
                    2 * ng, down_out, ng,
                    ["scope_amax_kernel", "scope_finalize_kernel", "nvfp4_scoped_kernel"],
                    "NVFP4 down export 128x2048x768"))

    _SHARED["exp_amax_legs"] = [
        Leg("nvfp4_export_gateup_amax",
            lambda: E.mxq_nvfp4_quantize_gateup_pair_amax(g, u, ap, NE, I, H, gc, gb, uc, ub, sp),
            2 * 2 * ng + 2 * NE, pair_out, 2 * ng, ["scope_scale_from_amax_kernel",
                                                    "nvfp4_scoped_kernel"],
            "NVFP4 gate/up export 128x2x768x2048, scope amax supplied (one read)"),
        Leg("nvfp4_export_down_amax",
            lambda: E.mxq_nvfp4_quantize_gateup_pair_amax(dn, None, ad, NE, H, I, dc, db, None,
                                                          None, sd),
            2 * ng + 2 * NE, down_out, ng, ["scope_scale_from_amax_kernel", "nvfp4_scoped_kernel"],
            "NVFP4 down export 128x2048x768, scope amax supplied (one read)")]

    def exp_dequant():
        E.mxq_dequantize_bf16(E.MXQ_FMT_NVFP4, gc, gb, sp, I, NE * I, H, yg)
        E.mxq_dequantize_bf16(E.MXQ_FMT_NVFP4, uc, ub, sp, I, NE * I, H, yu)
        E.mxq_dequantize_bf16(E.MXQ_FMT_NVFP4, dc, db, sd, H, NE * H, I, yd)
    legs.append(Leg("nvfp4_export_dequant", exp_dequant, pair_out + down_out, 2 * 3 * ng, 3 * ng,
                    ["dequant_nvfp4_kernel"], "NVFP4 -> BF16 of gate, up, down"))


_SHARED = {}     # inputs one leg group lends another (generated once)


def build_grp(torch, E, W, legs, dev, empty):
    """Grouped MXFP8 row+col and NVFP4 over 262144 expert-sorted rows, + dequant."""
    u8 = torch.uint8
    xg_np, off_np = W.config5()
    R, K = xg_np.shape
    G = off_np.size - 1
    xg = dev(xg_np)
    del xg_np
    _SHARED["grouped_x"] = xg
    off = torch.from_numpy(off_np).cuda()
    n = R * K
    g8 = {"row_codes": empty((R, K)), "row_scales": empty((R, K // 32)),
          "col_codes": empty((R, K)), "col_scales": empty((R // 32 + G, K)),
          "col_scale_offsets": empty((G + 1,), torch.int64)}
    g4 = {"codes": empty((R, K // 2)), "block_scales": empty((R, K // 16)),
          "token_scales": empty((R,), torch.float32)}
    col_scale_rows = int(sum((int(off_np[e + 1]) - int(off_np[e]) + 31) // 32 for e in range(G)))
    mx_out = 2 * n + n // 32 + col_scale_rows * K + 8 * (G + 1)
    nv_out = n // 2 + n // 16 + 4 * R
    legs.append(Leg("grouped_mxfp8_rowcol",
                    lambda: E.mxq_grouped_quantize(E.MXQ_FMT_MXFP8_ROWCOL, xg, R, K, off, G, g8),
                    2 * n + 8 * (G + 1), mx_out, n, ["mxfp8_tile_kernel<true, true, true, 8, false, true>"],
                    f"grouped MXFP8 row+col {R}x{K}, {G} segments"))
    legs.append(Leg("grouped_nvfp4",
                    lambda: E.mxq_grouped_quantize(E.MXQ_FMT_NVFP4, xg, R, K, off, G, g4),
                    2 * n + 8 * (G + 1), nv_out, n, ["nvfp4_token_kernel<2, true, false>"],
                    f"grouped per-token NVFP4 {R}x{K}"))
    y8, y4 = empty((R, K), torch.bfloat16), empty((R, K), torch.bfloat16)
    legs.append(Leg("grouped_dequant_mxfp8",
                    lambda: E.mxq_dequantize_bf16(E.MXQ_FMT_MXFP8_ROW, g8["row_codes"],
                                                  g8["row_scales"], None, 0, R, K, y8),
                    n + n // 32, 2 * n, n, ["dequant_mxfp8_kernel<false>"], "MXFP8 rowwise -> BF16"))
    legs.append(Leg("grouped_dequant_nvfp4",
                    lambda: E.mxq_dequantize_bf16(E.MXQ_FMT_NVFP4, g4["codes"], g4["block_scales"],
                                                  g4["token_scales"], 1, R, K, y4),
                    nv_out, 2 * n, n, ["dequant_nvfp4_kernel"], "NVFP4 -> BF16"))


CPU_SAMPLE_DIV = 1          # all host cores: one whole step
CPU_SINGLE_DIV = 16         # one thread: 1/16 of every leg


def oracle_step(W, D):
    """Inputs for the oracle over 1/D of every leg (generated here, outside any
    timed region) and a function that runs the oracle on them and returns the
    algorithmic bytes it processed."""
    import oracle
    if not os.path.exists(oracle._LIB):
        oracle.build()
    wgt = W.config2_weight("random")[:8192 // D]
    act = W.config2_activation("random")[:2048 // D]
    tok = W.config3()[:8192 // D]
    gate, up, down = W.config4(max(1, 128 // D))
    xg = W.student_t_activations(262144 // D, 2048, 5)

    def run():
        total = 0
        for x in (wgt, act):
            oracle.mxfp8_rowwise(x)
            oracle.mxfp8_colwise(x)
            total += x.size * 4 + x.size // 16
        c, b, s = oracle.nvfp4_per_token(tok)
        oracle.dequant_nvfp4(c, b, s, 1)
        total += 2 * (2 * tok.size + tok.size // 2 + tok.size // 16 + 4 * tok.shape[0])
        gc, gb, uc, ub, sp = oracle.nvfp4_gateup_pair(gate, up)
        dc, db, _, _, sd = oracle.nvfp4_gateup_pair(down, None)
        oracle.dequant_nvfp4(gc.reshape(-1, 1024), gb.reshape(-1, 128), sp, 768)
        oracle.dequant_nvfp4(uc.reshape(-1, 1024), ub.reshape(-1, 128), sp, 768)
        oracle.dequant_nvfp4(dc.reshape(-1, 384), db.reshape(-1, 48), sd, 2048)
        ng = gate.size
        total += 2 * (3 * 2 * ng + 3 * (ng // 2 + ng // 16))
        rc, rs = oracle.mxfp8_rowwise(xg)
        oracle.mxfp8_colwise(xg)
        c, b, s = oracle.nvfp4_per_token(xg)
        oracle.dequant_mxfp8_rowwise(rc, rs)
        oracle.dequant_nvfp4(c, b, s, 1)
        n = xg.size
        total += (2 * n + 2 * n + n // 16) + (2 * n + n // 2 + n // 16) + \
            (n + n // 32 + 2 * n) + (n // 2 + n // 16 + 2 * n)
        return total

    return run


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, log):
    """The oracle (as it stands) timed on the host cores: all cores over one
    whole step of the workload, and one thread over 1/16 of every leg."""
    import oracle
    run = oracle_step(W, CPU_SAMPLE_DIV)
    cores = oracle.max_threads()
    t0 = time.perf_counter()
    nbytes = run()
    dt = time.perf_counter() - t0
    log(f"cpu baseline ({cores} threads): {nbytes / 1e9:.3f} GB in {dt:.1f} s")
    del run
    run1 = oracle_step(W, CPU_SINGLE_DIV)
    oracle.set_threads(1)
    t1 = time.perf_counter()
    nbytes1 = run1()
    dt1 = time.perf_counter() - t1
    oracle.set_threads(cores)
    log(f"cpu baseline (1 thread): {nbytes1 / 1e9:.3f} GB in {dt1:.1f} s")
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"one whole step (every leg at full size: 8192x2048 weight, 2048x2048 "
                       "activation, 8192 tokens, 128 experts, 262144 grouped rows as one "
                       "segment); input generation excluded"),
            "seconds": round(dt, 2), "bytes": nbytes,
            "single_thread": {"value": round(nbytes1 / dt1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"1/{CPU_SINGLE_DIV} of every leg's rows",
                              "seconds": round(dt1, 2), "bytes": nbytes1},
            "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}


CFG_LAUNCHES, CFG_WARMUP, CFG_SAMPLES = 50, 10, 5
ROTATE_BYTES = 1 << 30      # buffer sets rotated per config: > the 256 MB MALL


def time_launches(torch, launches, n_launch, warmup, samples):
    """Mean time per launch (ms) of n_launch back-to-back launches cycling
    through `launches`, for each of `samples` samples (after warmup launches)."""
    stream = torch.cuda.current_stream()
    for k in range(warmup):
        launches[k % len(launches)]()
    out = []
    for _ in range(samples):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k in range(n_launch):
            launches[k % len(launches)]()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / n_launch)
    return out


def time_graph(torch, launches, n_launch, samples):
    """Per-launch time (ms) of n_launch launches cycling through `launches`,
    captured once in a HIP graph and replayed `samples` times: the device's
    rate without the host's per-call cost (argument checks, Python), which
    bounds back-to-back eager launches of kernels of a few us."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        for k in range(n_launch):
            launches[k % len(launches)]()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(samples):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / n_launch)
    del g
    return out


STREAMS = 4


def time_streams(torch, launches, n_launch, warmup, samples, n_streams=STREAMS):
    """Per-call time (ms) of n_launch calls cycling through `launches` (each a
    distinct buffer set), issued round-robin on n_streams streams of default
    priority and captured once in a HIP graph, so that one call's ramp and
    drain can overlap another's: the sustained device rate of independent
    calls, without the host's per-call cost.  (Issued eagerly, the stream
    switch per call costs the host more than these kernels take.)  The side
    streams fork from the capture stream and join it at the end."""
    streams = [torch.cuda.Stream() for _ in range(n_streams)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        cap = torch.cuda.current_stream()
        for st in streams:
            st.wait_stream(cap)
        for k in range(n_launch):
            with torch.cuda.stream(streams[k % n_streams]):
                launches[k % len(launches)]()
        for st in streams:
            cap.wait_stream(st)
    for _ in range(max(1, warmup // n_launch)):
        g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(samples):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / n_launch)
    del g
    return out


_FLOORS = {}


def copy_floor(torch, E, rbytes, wbytes, sets, graph, n_launch=CFG_LAUNCHES, warmup=CFG_WARMUP,
               streams=False):
    """The copy floor of a workload: mxq_copy_floor (a kernel that only reads
    rbytes and writes wbytes, no arithmetic) timed with the workload's own
    protocol and buffer rotation.  Returns (eager ms list, graph ms list or
    None[, concurrent-streams ms list when streams]); cached per byte counts."""
    key = (rbytes, wbytes, sets, graph, n_launch, streams)
    if key in _FLOORS:
        return _FLOORS[key]
    r16, w16 = -(-rbytes // 16) * 16, -(-wbytes // 16) * 16
    bufs = [(torch.empty(r16, dtype=torch.uint8, device="cuda"),
             torch.empty(w16, dtype=torch.uint8, device="cuda")) for _ in range(sets)]
    launches = [(lambda b=b: E.mxq_copy_floor(b[0], r16, b[1], w16)) for b in bufs]
    ms = time_launches(torch, launches, n_launch, warmup, CFG_SAMPLES)
    gms = time_graph(torch, launches, n_launch, CFG_SAMPLES) if graph else None
    sms = time_streams(torch, launches, n_launch, warmup, CFG_SAMPLES) if streams else None
    del bufs, launches
    torch.cuda.empty_cache()
    _FLOORS[key] = (ms, gms, sms) if streams else (ms, gms)
    return _FLOORS[key]


def cfg_record(name, desc, ms_list, nbytes, elems, sets, kernels, graph_ms=None, floor=None,
               rw=None, streams_ms=None):
    """One config's record.  floor: (eager, graph) ms lists of the copy floor of
    the same read and write bytes: "vs_copy_floor" is the floor's time over the
    kernel's (1.0 = as fast as a plain copy of those bytes)."""
    med, mn = float(np.median(ms_list)), float(np.min(ms_list))
    gbs = nbytes / (med * 1e-3) / 1e9
    rec = {"desc": desc, "kernels": kernels, "ms_median": round(med, 5),
           "ms_min": round(mn, 5), "bytes": nbytes, "GB_s": round(gbs, 1),
           "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
           "elements_per_s": round(elems / (med * 1e-3), 1), "buffer_sets": sets}
    if rw is not None:
        rec.update({"bytes_in": rw[0], "bytes_out": rw[1]})
    if floor is not None:
        fmed = float(np.median(floor[0]))
        fgbs = nbytes / (fmed * 1e-3) / 1e9
        rec.update({"copy_floor_ms": round(fmed, 5), "copy_floor_GB_s": round(fgbs, 1),
                    "copy_floor_pct_hbm_peak": round(100 * fgbs / HBM_PEAK_GBS, 2),
                    "vs_copy_floor": round(fmed / med, 4)})
    if graph_ms is not None:
        gmed = float(np.median(graph_ms))
        ggbs = nbytes / (gmed * 1e-3) / 1e9
        rec.update({"graph_ms_median": round(gmed, 5), "graph_GB_s": round(ggbs, 1),
                    "graph_pct_hbm_peak": round(100 * ggbs / HBM_PEAK_GBS, 2)})
        if floor is not None and floor[1] is not None:
            fg = float(np.median(floor[1]))
            rec.update({"graph_copy_floor_ms": round(fg, 5),
                        "graph_vs_copy_floor": round(fg / gmed, 4)})
    if streams_ms is not None:
        smed = float(np.median(streams_ms))
        sgbs = nbytes / (smed * 1e-3) / 1e9
        rec.update({f"graph_streams{STREAMS}_ms_median": round(smed, 5),
                    f"graph_streams{STREAMS}_GB_s": round(sgbs, 1),
                    f"graph_streams{STREAMS}_pct_hbm_peak": round(100 * sgbs / HBM_PEAK_GBS, 2)})
        if floor is not None and len(floor) > 2 and floor[2] is not None:
            fs = float(np.median(floor[2]))
            rec.update({f"graph_streams{STREAMS}_copy_floor_ms": round(fs, 5),
                        f"graph_streams{STREAMS}_vs_copy_floor": round(fs / smed, 4)})
    return name, rec


def config_timings(torch, E, W, legs, log, only=None):
    """The per-config protocol: hipEvents around 50 back-to-back launches per
    sample (5 samples after 10 warm-up launches), median and minimum per launch.
    Configs under 256 MB rotate distinct buffer sets totalling over 1 GiB, so
    every launch reads inputs that are not in the MALL; C5 is over 1 GiB
    itself.  C2b and C3 (and C5) are the shapes the 70% bar applies to.  Each
    config is timed beside the copy floor of its read and write bytes.
    only: a set of config names to time (all when None)."""
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    empty = lambda shape, dt=torch.uint8: torch.empty(shape, dtype=dt, device="cuda")
    res = {}
    sel = (lambda name: True) if only is None else (lambda name: name in only)

    def mxfp8_cfg(name, rows, cols, x_np, transposed=False):
        """transposed: the columnwise copy in the transposed layout
        (mxq_mxfp8_quantize_rowcol_t), the same bytes permuted."""
        if not sel(name):
            return
        n = rows * cols
        nbytes = 2 * n + 2 * n + 2 * (n // 32)
        sets = -(-ROTATE_BYTES // nbytes)
        x0 = dev(x_np)
        ccs = ((cols, rows), (cols, rows // 32)) if transposed else ((rows, cols), (rows // 32, cols))
        bufs = [(x0 if k == 0 else x0.clone(), empty((rows, cols)), empty((rows, cols // 32)),
                 empty(ccs[0]), empty(ccs[1])) for k in range(sets)]
        fn = E.mxq_mxfp8_quantize_rowcol_t if transposed else E.mxq_mxfp8_quantize_rowcol
        launches = [(lambda b=b: fn(b[0], rows, cols, b[1], b[2], b[3], b[4])) for b in bufs]
        ms = time_launches(torch, launches, CFG_LAUNCHES, CFG_WARMUP, CFG_SAMPLES)
        gms = time_graph(torch, launches, CFG_LAUNCHES, CFG_SAMPLES)
        sms = time_streams(torch, launches, CFG_LAUNCHES, CFG_WARMUP, CFG_SAMPLES)
        del bufs, launches, x0
        torch.cuda.empty_cache()
        rw = (2 * n, 2 * n + 2 * (n // 32))
        fl = copy_floor(torch, E, *rw, sets, True, streams=True)
        desc = f"MXFP8 row+col {rows}x{cols}" + (", columnwise copy transposed" if transposed
                                                  else "")
        k, v = cfg_record(name, desc, ms, nbytes, n, sets,
                          ["mxfp8_colt_staged_kernel" if transposed else "mxfp8_tile_kernel"],
                          gms, fl, rw, sms)
        res[k] = v

    for mode in W.MXFP8_MODES:
        mxfp8_cfg(f"C2a_{mode}", 2048, 2048, W.config2_activation(mode))
        mxfp8_cfg(f"C2b_{mode}", 8192, 2048, W.config2_weight(mode))
    mxfp8_cfg("C2b_rowcol_t", 8192, 2048, W.config2_weight("random"), transposed=True)
    log("C2 timed")

    rows, cols = 8192, 2048
    n = rows * cols
    q_out = n // 2 + n // 16 + 4 * rows
    q_bytes = 2 * n + q_out
    d_bytes = q_out + 2 * n
    if sel("C3_nvfp4") or sel("C3_dequant"):
        sets = -(-ROTATE_BYTES // q_bytes)
        x0 = dev(W.config3())
        bufs = [(x0 if k == 0 else x0.clone(), empty((rows, cols // 2)),
                 empty((rows, cols // 16)), empty((rows,), torch.float32),
                 empty((rows, cols), torch.bfloat16)) for k in range(sets)]
        q = [(lambda b=b: E.mxq_nvfp4_quantize_per_token(b[0], rows, cols, b[1], b[2], b[3]))
             for b in bufs]
        ms = time_launches(torch, q, CFG_LAUNCHES, CFG_WARMUP, CFG_SAMPLES)
        gms = time_graph(torch, q, CFG_LAUNCHES, CFG_SAMPLES)
        sms = time_streams(torch, q, CFG_LAUNCHES, CFG_WARMUP, CFG_SAMPLES)
        d = [(lambda b=b: E.mxq_dequantize_bf16(E.MXQ_FMT_NVFP4, b[1], b[2], b[3], 1, rows,
                                                 cols, b[4])) for b in bufs]
        dms = time_launches(torch, d, CFG_LAUNCHES, CFG_WARMUP, CFG_SAMPLES)
        dgms = time_graph(torch, d, CFG_LAUNCHES, CFG_SAMPLES)
        dsms = time_streams(torch, d, CFG_LAUNCHES, CFG_WARMUP, CFG_SAMPLES)
        del bufs, q, d, x0
        torch.cuda.empty_cache()
        if sel("C3_nvfp4"):
            fl = copy_floor(torch, E, 2 * n, q_out, sets, True, streams=True)
            k, v = cfg_record("C3_nvfp4", f"NVFP4 per-token {rows}x{cols}", ms, q_bytes, n, sets,
                              ["nvfp4_token_split_kernel"], gms, fl, (2 * n, q_out), sms)
            res[k] = v
        if sel("C3_dequant"):
            fl = copy_floor(torch, E, q_out, 2 * n, sets, True, streams=True)
            k, v = cfg_record("C3_dequant", f"NVFP4 -> BF16 {rows}x{cols}", dms, d_bytes, n,
                              sets, ["dequant_nvfp4_kernel"], dgms, fl, (q_out, 2 * n), dsms)
            res[k] = v
        log("C3 timed")

    by_name = {l.name: l for l in legs}
    for leg, cfg in (("grouped_mxfp8_rowcol", "C5_mxfp8"), ("grouped_nvfp4", "C5_nvfp4"),
                     ("grouped_dequant_mxfp8", "C5_dequant_mxfp8"),
                     ("grouped_dequant_nvfp4", "C5_dequant_nvfp4"),
                     ("nvfp4_export_gateup", "C4_gateup"), ("nvfp4_export_down", "C4_down")):
        if leg in by_name and sel(cfg):
            l = by_name[leg]
            # A dequant config decodes what its quantize leg wrote: run that
            # leg once first (with --config-only it may not have run).
            src = {"grouped_dequant_mxfp8": "grouped_mxfp8_rowcol",
                   "grouped_dequant_nvfp4": "grouped_nvfp4"}.get(leg)
            if src in by_name:
                by_name[src].launch()
                torch.cuda.synchronize()
            ms = time_launches(torch, [l.launch], 10, 2, CFG_SAMPLES)
            fl = copy_floor(torch, E, l.bytes_in, l.bytes_out, 1, False, 10, 2)
            k, v = cfg_record(cfg, l.desc, ms, l.bytes, l.elems, 1, l.kernels, None, fl,
                              (l.bytes_in, l.bytes_out))
            res[k] = v
    for l, cfg in zip(_SHARED.get("exp_amax_legs", []), ("C4_gateup_amax", "C4_down_amax")):
        if sel(cfg):
            ms = time_launches(torch, [l.launch], 10, 2, CFG_SAMPLES)
            fl = copy_floor(torch, E, l.bytes_in, l.bytes_out, 1, False, 10, 2)
            k, v = cfg_record(cfg, l.desc, ms, l.bytes, l.elems, 1, l.kernels, None, fl,
                              (l.bytes_in, l.bytes_out))
            res[k] = v
    log("C4/C5 timed")

    if "grouped_mxfp8_rowcol" in by_name and only is None:
        res.update(dispatch_timings(torch, E, W, dev, empty))
        log("C5 dispatch timed")
        res.update(qdq_timings(torch, E, W, dev, empty))
        log("quantize + dequant timed")
        res.update(gemm_timings(torch, E, W, dev, empty))
        log("GEMM timed")
        res.update(wgrad_timings(torch, E, W, dev, empty))
        log("weight gradient timed")
    elif only is not None:
        if any(c.startswith("G_") and "wgrad" not in c for c in only):
            res.update({k: v for k, v in gemm_timings(torch, E, W, dev, empty).items()
                        if k in only})
            log("GEMM timed")
        if any("wgrad" in c or c in ("C5_colt_mxfp8", "C5_rowcolt_mxfp8") for c in only):
            res.update(wgrad_timings(torch, E, W, dev, empty, only))
            log("weight gradient timed")
        if any("_qdq_" in c for c in only):
            res.update({k: v for k, v in qdq_timings(torch, E, W, dev, empty).items()
                        if k in only})
            log("quantize + dequant timed")
    return res


def build_qdq(torch, E, W, legs, dev, empty):
    """Quantize + BF16 dequant in one pass over the grouped rows (262144 x
    2048, Student-t): rowwise MXFP8 and per-token NVFP4.  Each is the
    alternative to a quantize leg followed by its dequant leg."""
    xg = _SHARED.get("grouped_x")
    if xg is None:
        xg = dev(W.student_t_activations(262144, 2048, 5))
    R, K = xg.shape
    n = R * K
    y = empty((R, K), torch.bfloat16)
    rc, rs = empty((R, K)), empty((R, K // 32))
    c4, b4, t4 = empty((R, K // 2)), empty((R, K // 16)), empty((R,), torch.float32)
    legs.append(Leg("qdq_mxfp8_rowwise",
                    lambda: E.mxq_quantize_dequant_bf16(E.MXQ_FMT_MXFP8_ROW, xg, R, K, rc, rs, None,
                                                        y),
                    2 * n, n + n // 32 + 2 * n, n, ["mxfp8_row_qdq_kernel<true, 8>"],
                    f"MXFP8 rowwise quantize + BF16 dequant, one pass, {R}x{K}"))
    legs.append(Leg("qdq_nvfp4",
                    lambda: E.mxq_quantize_dequant_bf16(E.MXQ_FMT_NVFP4, xg, R, K, c4, b4, t4, y),
                    2 * n, n // 2 + n // 16 + 4 * R + 2 * n, n,
                    ["nvfp4_token_qdq_kernel<2, true>"],
                    f"per-token NVFP4 quantize + BF16 dequant, one pass, {R}x{K}"))


def qdq_small_timings(torch, E, W, dev, empty):
    """One-pass quantize + dequant on the 8192 x 2048 shapes (weight, random
    mode; Student-t activations), rotating buffer sets over 1 GiB."""
    res = {}
    rows, cols = 8192, 2048
    n = rows * cols
    for name, fmt, x_np, out_b in (
            ("C2b_qdq_mxfp8", E.MXQ_FMT_MXFP8_ROW, W.config2_weight("random"),
             n + n // 32 + 2 * n),
            ("C3_qdq_nvfp4", E.MXQ_FMT_NVFP4, W.config3(), n // 2 + n // 16 + 4 * rows + 2 * n)):
        nbytes = 2 * n + out_b
        sets = -(-ROTATE_BYTES // nbytes)
        x0 = dev(x_np)
        if fmt == E.MXQ_FMT_NVFP4:
            bufs = [(x0 if k == 0 else x0.clone(), empty((rows, cols // 2)),
                     empty((rows, cols // 16)), empty((rows,), torch.float32),
                     empty((rows, cols), torch.bfloat16)) for k in range(sets)]
        else:
            bufs = [(x0 if k == 0 else x0.clone(), empty((rows, cols)), empty((rows, cols // 32)),
                     None, empty((rows, cols), torch.bfloat16)) for k in range(sets)]
        launches = [(lambda b=b, fmt=fmt: E.mxq_quantize_dequant_bf16(fmt, b[0], rows, cols, b[1],
                                                                      b[2], b[3], b[4]))
                    for b in bufs]
        ms = time_launches(torch, launches, CFG_LAUNCHES, CFG_WARMUP, CFG_SAMPLES)
        gms = time_graph(torch, launches, CFG_LAUNCHES, CFG_SAMPLES)
        del bufs, launches, x0
        torch.cuda.empty_cache()
        fl = copy_floor(torch, E, 2 * n, out_b, sets, True)
        kern = "mxfp8_row_qdq_kernel" if fmt == E.MXQ_FMT_MXFP8_ROW else "nvfp4_token_split_kernel"
        k, v = cfg_record(name, f"quantize + BF16 dequant, one pass, {rows}x{cols}", ms, nbytes,
                          n, sets, [kern], gms, fl, (2 * n, out_b))
        res[k] = v
    return res


def build_gemm(torch, E, W, legs, dev, empty):
    """The dense-layer GEMMs (2048 x 8192 x 2048, BF16 result) as legs, for
    kernel statistics; bytes are the operands read and the result written,
    elems the multiply-adds.  Timed with their matrix roofline in the configs."""
    M, N, K = 2048, 8192, 2048
    x, w = dev(W.config2_activation("random")), dev(W.config2_weight("random"))
    ac, as_, bc, bs_ = empty((M, K)), empty((M, K // 32)), empty((N, K)), empty((N, K // 32))
    E.mxq_mxfp8_quantize_rowcol(x, M, K, ac, as_, None, None)
    E.mxq_mxfp8_quantize_rowcol(w, N, K, bc, bs_, None, None)
    c = empty((M, N), torch.bfloat16)
    legs.append(Leg("gemm_mxfp8", lambda: E.mxq_mxfp8_gemm(ac, as_, bc, bs_, M, N, K,
                                                           E.MXQ_OUT_BF16, c),
                    (M + N) * K * (1 + 1 / 32), 2 * M * N, M * N * K, ["mxfp8_gemm_kernel<true>"],
                    f"MXFP8 GEMM {M}x{N}x{K}, BF16 out"))
    na, nb, ns = empty((M, K // 2)), empty((M, K // 16)), empty((M,), torch.float32)
    wa, wb, ws = empty((N, K // 2)), empty((N, K // 16)), empty((1,), torch.float32)
    E.mxq_nvfp4_quantize_per_token(x, M, K, na, nb, ns)
    E.mxq_nvfp4_quantize_gateup_pair(w, None, 1, N, K, wa, wb, None, None, ws)
    c4 = empty((M, N), torch.bfloat16)
    legs.append(Leg("gemm_nvfp4", lambda: E.mxq_nvfp4_gemm(na, nb, ns, 1, wa, wb, ws, N, M, N, K,
                                                           E.MXQ_OUT_BF16, c4),
                    (M + N) * K * (0.5 + 1 / 16) + 4 * M + 4, 2 * M * N, M * N * K,
                    ["nvfp4_gemm_kernel<true>"], f"NVFP4 GEMM {M}x{N}x{K}, BF16 out"))


MFMA_FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8 matrix peak
MFMA_F16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 (and bf16) matrix peak


def gemm_timings(torch, E, W, dev, empty):
    """Block-scaled MXFP8 GEMM of the dense layer: the 2048 x 2048 activation
    times the 8192 x 2048 weight (rowwise MXFP8 copies made by the library's
    quantizer), BF16 result; timed like the other configs and priced against
    the fp8 matrix-instruction peak."""
    res = {}
    for name, (M, N, K) in (("G_mxfp8_gemm_2048x8192x2048", (2048, 8192, 2048)),
                            ("G_mxfp8_gemm_8192x8192x2048", (8192, 8192, 2048))):
        x = dev(W.student_t_activations(M, K, 81) if M != 2048 else W.config2_activation("random"))
        w = dev(W.config2_weight("random") if N == 8192 and K == 2048 else
                W.mode_random(N, K, 82))
        ac, as_ = empty((M, K)), empty((M, K // 32))
        bc, bs_ = empty((N, K)), empty((N, K // 32))
        E.mxq_mxfp8_quantize_rowcol(x, M, K, ac, as_, None, None)
        E.mxq_mxfp8_quantize_rowcol(w, N, K, bc, bs_, None, None)
        c = empty((M, N), torch.bfloat16)
        fn = lambda: E.mxq_mxfp8_gemm(ac, as_, bc, bs_, M, N, K, E.MXQ_OUT_BF16, c)
        ms = time_launches(torch, [fn], 10, 2, CFG_SAMPLES)
        med = float(np.median(ms))
        flops = 2.0 * M * N * K
        tf = flops / (med * 1e-3) / 1e12
        res[name] = {"desc": f"MXFP8 GEMM C[{M}][{N}] = A[{M}][{K}] B[{N}][{K}]^T, BF16 out",
                     "kernels": ["mxfp8_gemm_kernel<true>"], "ms_median": round(med, 5),
                     "ms_min": round(float(np.min(ms)), 5), "flops": flops,
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                  "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tf / MFMA_FP8_PEAK_TFLOPS, 4)}}
        del x, w, ac, as_, bc, bs_, c
        torch.cuda.empty_cache()
    # Grouped (MoE expert layer): config 5's expert-sorted rows (262144 x 2048,
    # 128 segments of the top-8 routing of 32768 tokens) times each expert's
    # 768 x 2048 weight.  Inputs are seeded torch normals generated on the
    # device (generating 2^29 Student-t values on the host would take longer
    # than the timing), quantized by the library.
    for name, (R, N, K, G) in (("G_mxfp8_grouped_gemm_262144x768x2048", (262144, 768, 2048, 128)),):
        _, offsets = W.routing(W.N_TOKENS, G, W.TOP_K, 6)
        gen = torch.Generator(device="cuda").manual_seed(93)
        x = (torch.randn((R, K), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
        w = (torch.randn((G * N, K), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
        ac, as_ = empty((R, K)), empty((R, K // 32))
        bc, bs_ = empty((G * N, K)), empty((G * N, K // 32))
        E.mxq_mxfp8_quantize_rowcol(x, R, K, ac, as_, None, None)
        E.mxq_mxfp8_quantize_rowcol(w, G * N, K, bc, bs_, None, None)
        off = torch.from_numpy(offsets).cuda()
        c = empty((R, N), torch.bfloat16)
        fn = lambda: E.mxq_mxfp8_grouped_gemm(ac, as_, bc, bs_, off, G, R, N, K, E.MXQ_OUT_BF16, c)
        ms = time_launches(torch, [fn], 10, 2, CFG_SAMPLES)
        med = float(np.median(ms))
        flops = 2.0 * R * N * K
        tf = flops / (med * 1e-3) / 1e12
        res[name] = {"desc": f"grouped MXFP8 GEMM: {R} expert-sorted rows x {G} experts' "
                             f"[{N}][{K}] weights (config 5 routing), BF16 out",
                     "kernels": ["mxfp8_grouped_gemm_kernel<true>"], "ms_median": round(med, 5),
                     "ms_min": round(float(np.min(ms)), 5), "flops": flops,
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                  "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tf / MFMA_FP8_PEAK_TFLOPS, 4)}}
        del x, w, ac, as_, bc, bs_, off, c
        torch.cuda.empty_cache()
    # The same expert layer on per-token NVFP4 rows and NVFP4 expert weights
    # (one scope scale each, as the export writes them); BF16 matrix
    # instructions, so priced against the BF16 peak.
    for name, (R, N, K, G) in (("G_nvfp4_grouped_gemm_262144x768x2048", (262144, 768, 2048, 128)),):
        _, offsets = W.routing(W.N_TOKENS, G, W.TOP_K, 6)
        gen = torch.Generator(device="cuda").manual_seed(97)
        x = (torch.randn((R, K), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
        w = (torch.randn((G, N, K), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
        ac, ab, as_ = empty((R, K // 2)), empty((R, K // 16)), empty((R,), torch.float32)
        bc, bb, bs_ = empty((G, N, K // 2)), empty((G, N, K // 16)), empty((G,), torch.float32)
        E.mxq_nvfp4_quantize_per_token(x, R, K, ac, ab, as_)
        E.mxq_nvfp4_quantize_gateup_pair(w, None, G, N, K, bc, bb, None, None, bs_)
        off = torch.from_numpy(offsets).cuda()
        c = empty((R, N), torch.bfloat16)
        fn = lambda: E.mxq_nvfp4_grouped_gemm(ac, ab, as_, bc, bb, bs_, off, G, R, N, K,
                                              E.MXQ_OUT_BF16, c)
        ms = time_launches(torch, [fn], 10, 2, CFG_SAMPLES)
        med = float(np.median(ms))
        flops = 2.0 * R * N * K
        tf = flops / (med * 1e-3) / 1e12
        res[name] = {"desc": f"grouped NVFP4 GEMM: {R} per-token NVFP4 rows x {G} experts' "
                             f"[{N}][{K}] NVFP4 weights (config 5 routing), BF16 out",
                     "kernels": ["nvfp4_grouped_gemm_kernel<true>"], "ms_median": round(med, 5),
                     "ms_min": round(float(np.min(ms)), 5), "flops": flops,
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                  "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}}
        del x, w, ac, ab, as_, bc, bb, bs_, off, c
        torch.cuda.empty_cache()
    # NVFP4: per-token activations times a weight with one scope scale; the
    # matrix instructions are BF16 (the per-16 E4M3 block scales rule out the
    # fp4 ones), so the peak is the BF16 one.
    for name, (M, N, K) in (("G_nvfp4_gemm_2048x8192x2048", (2048, 8192, 2048)),):
        x = dev(W.student_t_activations(M, K, 83))
        w = dev(W.bf16_bits(np.random.default_rng(84).normal(0, 0.02, (N, K))))
        ac, ab, as_ = empty((M, K // 2)), empty((M, K // 16)), empty((M,), torch.float32)
        bc, bb, bs_ = empty((N, K // 2)), empty((N, K // 16)), empty((1,), torch.float32)
        E.mxq_nvfp4_quantize_per_token(x, M, K, ac, ab, as_)
        E.mxq_nvfp4_quantize_gateup_pair(w, None, 1, N, K, bc, bb, None, None, bs_)
        c = empty((M, N), torch.bfloat16)
        fn = lambda: E.mxq_nvfp4_gemm(ac, ab, as_, 1, bc, bb, bs_, N, M, N, K, E.MXQ_OUT_BF16, c)
        ms = time_launches(torch, [fn], 10, 2, CFG_SAMPLES)
        med = float(np.median(ms))
        flops = 2.0 * M * N * K
        tf = flops / (med * 1e-3) / 1e12
        res[name] = {"desc": f"NVFP4 GEMM C[{M}][{N}] = A[{M}][{K}] B[{N}][{K}]^T, per-token and "
                             "per-tensor FP32 scales, BF16 out",
                     "kernels": ["nvfp4_gemm_kernel<true>"], "ms_median": round(med, 5),
                     "ms_min": round(float(np.min(ms)), 5), "flops": flops,
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                  "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}}
        del x, w, ac, ab, as_, bc, bb, bs_, c
        torch.cuda.empty_cache()
    return res


def qdq_timings(torch, E, W, dev, empty):
    legs = []
    build_qdq(torch, E, W, legs, dev, empty)
    res = {}
    for l, cfg in zip(legs, ("C5_qdq_mxfp8", "C5_qdq_nvfp4")):
        ms = time_launches(torch, [l.launch], 10, 2, CFG_SAMPLES)
        fl = copy_floor(torch, E, l.bytes_in, l.bytes_out, 1, False, 10, 2)
        k, v = cfg_record(cfg, l.desc, ms, l.bytes, l.elems, 1, l.kernels, None, fl,
                          (l.bytes_in, l.bytes_out))
        res[k] = v
    del legs
    torch.cuda.empty_cache()
    res.update(qdq_small_timings(torch, E, W, dev, empty))
    return res


def build_dsp(torch, E, W, legs, dev, empty):
    """The grouped workload quantized straight from its 32768 unpermuted tokens
    (top-8 of 128 experts): MXFP8 row+col and per-token NVFP4, plus torch's own
    row gather, the pass the fused call saves.  The algorithmic bytes read each
    token once."""
    tok_np, rt_np, tr_np, off_np = W.config5_dispatch()
    T, K = tok_np.shape
    R, G, top_k = rt_np.size, off_np.size - 1, tr_np.shape[1]
    tok = dev(tok_np)
    del tok_np
    rt, tr, off = (torch.from_numpy(a).cuda() for a in (rt_np, tr_np, off_np))
    n = R * K
    col_scale_rows = int(sum((int(off_np[e + 1]) - int(off_np[e]) + 31) // 32 for e in range(G)))
    g8 = {"row_codes": empty((R, K)), "row_scales": empty((R, K // 32)),
          "col_codes": empty((R, K)), "col_scales": empty((R // 32 + G, K)),
          "col_scale_offsets": empty((G + 1,), torch.int64)}
    g4 = {"codes": empty((R, K // 2)), "block_scales": empty((R, K // 16)),
          "token_scales": empty((R,), torch.float32)}
    legs.append(Leg("dispatch_mxfp8_rowcol",
                    lambda: E.mxq_grouped_quantize_dispatch(E.MXQ_FMT_MXFP8_ROWCOL, tok, T, K, 0,
                                                            None, rt, R, off, G, g8),
                    2 * T * K + 8 * R + 8 * (G + 1),
                    2 * n + n // 32 + col_scale_rows * K + 8 * (G + 1), n,
                    ["grouped_prefix_kernel", "mxfp8_tile_kernel<true, true, true, 8, true, false>"],
                    f"dispatch + grouped MXFP8 row+col, {T} tokens -> {R}x{K}, {G} segments"))
    legs.append(Leg("dispatch_nvfp4",
                    lambda: E.mxq_grouped_quantize_dispatch(E.MXQ_FMT_NVFP4, tok, T, K, top_k, tr,
                                                            None, R, None, 0, g4),
                    2 * T * K + 8 * T * top_k, n // 2 + n // 16 + 4 * R, n,
                    ["nvfp4_token_kernel<2, true, true>"],
                    f"dispatch + per-token NVFP4, {T} tokens -> {R}x{K} (top-{top_k})"))
    xg = empty((R, K), torch.bfloat16)
    tb = tok.view(torch.bfloat16)
    legs.append(Leg("gather_torch", lambda: torch.index_select(tb, 0, rt, out=xg),
                    2 * T * K + 8 * R, 2 * n, n, ["index_select"],
                    f"torch.index_select of {R} rows of {T}x{K} BF16 (the copy a fused "
                    "dispatch avoids)"))


def wgrad_timings(torch, E, W, dev, empty, only=None):
    """The expert layer's weight-gradient pair at config 5's routing: the
    grouped transposed columnwise copies of X [262144][2048] (timed, with its
    copy floor: a quantize config; also with the rowwise copy from the same
    read, the two copies dY needs) and of dY [262144][768], then
    dW_e [768][2048] = dY_e^T X_e for all 128 experts (timed, priced against
    the fp8 matrix peak).  Inputs are seeded torch normals on the device."""
    sel = (lambda n: True) if only is None else (lambda n: n in only)
    res = {}
    R, K, M, G = 262144, 2048, 768, 128
    _, offsets = W.routing(W.N_TOKENS, G, W.TOP_K, 6)
    off = torch.from_numpy(offsets).cuda()
    gen = torch.Generator(device="cuda").manual_seed(98)
    x = (torch.randn((R, K), generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    dy = (torch.randn((R, M), generator=gen, device="cuda") * 0.01).to(torch.bfloat16)
    pitch = -(-R // 128) * 128 + 128 * G                 # grouped_colt_pitch
    gx = (empty((K, pitch)), empty((K, pitch // 32)), empty((G + 1,), torch.int64))
    gd = (empty((M, pitch)), empty((M, pitch // 32)), empty((G + 1,), torch.int64))
    if sel("C5_colt_mxfp8"):
        fn = lambda: E.mxq_mxfp8_grouped_colwise_t(x, R, K, off, G, gx[0], gx[1], gx[2])
        ms = time_launches(torch, [fn], 10, 2, CFG_SAMPLES)
        # Algorithmic bytes: X once, every padded code and scale column written.
        rb, wb = 2 * R * K + 8 * (G + 1), 0
        fn()
        torch.cuda.synchronize()
        blocks = int(gx[2][-1].item())
        wb = K * 32 * blocks + K * blocks + 8 * (G + 1)
        fl = copy_floor(torch, E, rb, wb, 1, False, 10, 2)
        k, v = cfg_record("C5_colt_mxfp8", f"grouped MXFP8 columnwise, transposed and padded to "
                          f"128 rows per segment, {R}x{K}, {G} segments", ms, rb + wb, R * K, 1,
                          ["mxfp8_grouped_colt_kernel<8, false, true>"], None,
                          fl, (rb, wb))
        res[k] = v
    if sel("C5_rowcolt_mxfp8"):
        rc, rs = empty((R, K)), empty((R, K // 32))
        fn = lambda: E.mxq_mxfp8_grouped_quantize_rowcol_t(x, R, K, off, G, rc, rs, gx[0], gx[1],
                                                           gx[2])
        ms = time_launches(torch, [fn], 10, 2, CFG_SAMPLES)
        fn()
        torch.cuda.synchronize()
        blocks = int(gx[2][-1].item())
        rb = 2 * R * K + 8 * (G + 1)
        wb = R * K + R * K // 32 + K * 32 * blocks + K * blocks + 8 * (G + 1)
        fl = copy_floor(torch, E, rb, wb, 1, False, 10, 2)
        k, v = cfg_record("C5_rowcolt_mxfp8", f"grouped MXFP8 rowwise copy plus the columnwise "
                          f"copy transposed and padded, one read, {R}x{K}, {G} segments", ms,
                          rb + wb, R * K, 1,
                          ["mxfp8_grouped_colt_kernel<8, true, true>"], None,
                          fl, (rb, wb))
        res[k] = v
        del rc, rs
    name = f"G_mxfp8_grouped_wgrad_{M}x{K}_over_{R}"
    if sel(name):
        E.mxq_mxfp8_grouped_colwise_t(x, R, K, off, G, gx[0], gx[1], gx[2])
        E.mxq_mxfp8_grouped_colwise_t(dy, R, M, off, G, gd[0], gd[1], gd[2])
        c = empty((G, M, K), torch.bfloat16)
        fn = lambda: E.mxq_mxfp8_grouped_wgrad(gd[0], gd[1], gx[0], gx[1], gd[2], G, M, K, pitch,
                                               E.MXQ_OUT_BF16, c)
        ms = time_launches(torch, [fn], 10, 2, CFG_SAMPLES)
        med = float(np.median(ms))
        flops = 2.0 * R * M * K
        tf = flops / (med * 1e-3) / 1e12
        res[name] = {"desc": f"grouped MXFP8 weight gradient: dW_e[{M}][{K}] = dY_e^T X_e over "
                             f"each of {G} segments of {R} rows (config 5 routing), BF16 out",
                     "kernels": ["mxfp8_grouped_wgrad_kernel<true>"], "ms_median": round(med, 5),
                     "ms_min": round(float(np.min(ms)), 5), "flops": flops,
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                  "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tf / MFMA_FP8_PEAK_TFLOPS, 4)}}
        del c
    del x, dy, gx, gd, off
    torch.cuda.empty_cache()
    return res


def dispatch_timings(torch, E, W, dev, empty):
    legs = []
    build_dsp(torch, E, W, legs, dev, empty)
    res = {}
    for l, cfg in zip(legs, ("C5_dispatch_mxfp8", "C5_dispatch_nvfp4", "C5_gather_torch")):
        ms = time_launches(torch, [l.launch], 10, 2, CFG_SAMPLES)
        fl = copy_floor(torch, E, l.bytes_in, l.bytes_out, 1, False, 10, 2)
        k, v = cfg_record(cfg, l.desc, ms, l.bytes, l.elems, 1, l.kernels, None, fl,
                          (l.bytes_in, l.bytes_out))
        res[k] = v
    return res


# ---------------------------------------------------------------------------
# rocprofv3 summaries (CPU only): the HBM traffic of each kernel from two
# counter runs, and the kernel statistics of a kernel-trace run.
# ---------------------------------------------------------------------------

PMC_CMD = ("rocprofv3 --pmc {counter} -d OUT/pmc_{tag} -o {tag} --output-format csv -- "
           "python3 bench.py --groups grp,dsp,qdq --steps 2 --warmup 1 --no-cpu-baseline "
           "--no-configs --copy-calibration-mib 1024")
STATS_CMD = ("rocprofv3 --kernel-trace --stats -d OUT/prof_bench -o bench --output-format "
             "csv -- python3 bench.py --groups act,wgt,tok,exp,grp,dsp,qdq,gemm --steps 5 "
             "--warmup 2 --no-cpu-baseline --no-configs")
GEMM_CONFIGS = ("G_mxfp8_gemm_2048x8192x2048,G_mxfp8_gemm_8192x8192x2048,"
                "G_nvfp4_gemm_2048x8192x2048,G_mxfp8_grouped_gemm_262144x768x2048,"
                "G_nvfp4_grouped_gemm_262144x768x2048,G_mxfp8_grouped_wgrad_768x2048_over_262144")
GEMM_STATS_CMD = ("rocprofv3 --kernel-trace --stats -d OUT/gemm_stats -o gemm --output-format "
                  "csv -- python3 bench.py --config-only " + GEMM_CONFIGS)


def kernel_short_name(name: str) -> str:
    """'void mxq::k<a, b>(args)' -> 'k<a, b>' (the names the legs use)."""
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            name = name[:i]
            break
    return name[5:] if name.startswith("mxq::") else name


def pmc_per_dispatch(path: str):
    """{raw kernel name: [counter value summed per dispatch, ...]} of a
    rocprofv3 counter-collection CSV holding one counter."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            d = r.get("Dispatch_Id") or r.get("Correlation_Id")
            k = per.setdefault(r["Kernel_Name"], {})
            k[d] = k.get(d, 0.0) + float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def summarize_pmc(fetch_csv: str, write_csv: str, bench_log: str, out_json: str, out_txt: str):
    """HBM bytes per launch of every single-kernel leg of one bench run under
    the two counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each
    counter scaled by what it reads for the plain copy of the same run."""
    line = [ln for ln in open(bench_log) if ln.startswith("{")][-1]
    run = json.loads(line)
    fetch, write = pmc_per_dispatch(fetch_csv), pmc_per_dispatch(write_csv)
    mean = lambda v: sum(v) / len(v)
    copy_bytes = run["copy_calibration"]["bytes"] // 2          # read once, written once
    copy_f = [mean(v) for k, v in fetch.items() if "bitwise_not" in k]
    copy_w = [mean(v) for k, v in write.items() if "bitwise_not" in k]
    f_scale = copy_bytes / (copy_f[0] * 1024)
    w_scale = copy_bytes / (copy_w[0] * 1024)
    short_f = {kernel_short_name(k): v for k, v in fetch.items()}
    short_w = {kernel_short_name(k): v for k, v in write.items()}
    kernels = {}
    rows = []
    for leg, info in run["legs"].items():
        kern = info["kernels"][-1]
        if kern not in short_f or kern not in short_w:
            continue
        users = [l for l, i in run["legs"].items() if i["kernels"][-1] == kern]
        if len(users) != 1:
            continue                    # one kernel for several legs: sizes differ
        fk, wk = mean(short_f[kern]), mean(short_w[kern])
        hbm = int(round(fk * 1024 * f_scale + wk * 1024 * w_scale))
        kernels[kern] = {"leg": leg, "source_digest": kernel_digest(kern), "fetch_kib": fk,
                         "write_kib": wk, "hbm_bytes_per_launch": hbm,
                         "algorithmic_bytes": info["bytes"], "launches": len(short_f[kern])}
        rows.append((kern, leg, fk, wk, hbm, info["bytes"]))
    doc = {"calibration": {"copy_bytes": copy_bytes, "fetch_kib": copy_f[0],
                           "write_kib": copy_w[0], "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": kernels}
    with open(out_json, "w") as f:
        json.dump(doc, f, indent=1)
    out = ["HBM traffic per launch from rocprofv3 TCC counters (FETCH_SIZE and WRITE_SIZE, KiB per",
           "dispatch, averaged over the launches of each kernel), each scaled by what the same counter",
           f"reads for a plain copy kernel (int32 bitwise not of {copy_bytes} bytes: reads and writes",
           "each byte once).", "",
           "Commands (run from the repository root on one MI355X, ROCm 7.2, TMPDIR=/tmp; OUT is the",
           "directory the CSVs go to):",
           "  " + PMC_CMD.format(counter="FETCH_SIZE", tag="fetch"),
           "  " + PMC_CMD.format(counter="WRITE_SIZE", tag="write"),
           "Summary: python3 bench.py --summarize-pmc <fetch csv> <write csv> <log of the fetch run>",
           "",
           f"copy calibration: FETCH_SIZE {copy_f[0]:.0f} KiB for {copy_bytes} bytes read -> "
           f"scale {f_scale:.4f};",
           f"                  WRITE_SIZE {copy_w[0]:.0f} KiB for {copy_bytes} bytes written -> "
           f"scale {w_scale:.4f}", "",
           f"{'kernel':<46} {'leg':<26} {'FETCH KiB':>10} {'WRITE KiB':>10} {'HBM bytes':>14} "
           f"{'algorithmic':>14} {'ratio':>6}"]
    for kern, leg, fk, wk, hbm, alg in rows:
        out.append(f"{kern:<46} {leg:<26} {fk:>10.0f} {wk:>10.0f} {hbm:>14} {alg:>14} "
                   f"{hbm / alg:>6.3f}")
    with open(out_txt, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


SHAPE_VALU = ("SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_BUSY_CYCLES SQ_WAVE_CYCLES "
              "SQ_INSTS_VALU_CVT SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR GRBM_GUI_ACTIVE")
SHAPE_BENCH = "python3 bench.py --config-only {configs} --copy-calibration-mib 1024"
SHAPE_CMDS = (
    ("stats", "rocprofv3 --kernel-trace --stats -d OUT/{tag}_stats -o s --output-format csv -- "),
    ("fetch", "rocprofv3 --pmc FETCH_SIZE -d OUT/{tag}_fetch -o f --output-format csv -- "),
    ("write", "rocprofv3 --pmc WRITE_SIZE -d OUT/{tag}_write -o w --output-format csv -- "),
    ("valu", "rocprofv3 --pmc " + SHAPE_VALU + " -d OUT/{tag}_valu -o v --output-format csv -- "))


def pmc_counters(path: str):
    """{(raw kernel name, grid size): {counter: [value summed per dispatch, ...]}}."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            d = r.get("Dispatch_Id") or r.get("Correlation_Id")
            key = (r["Kernel_Name"], int(r["Grid_Size"]))
            c = per.setdefault(key, {}).setdefault(r["Counter_Name"], {})
            c[d] = c.get(d, 0.0) + float(r["Counter_Value"])
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per.items()}


def trace_durations(path: str):
    """{(raw kernel name, grid size): [duration in us, ...]} of a kernel trace."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) *
                   int(r["Grid_Size_Z"]))
            per.setdefault(key, []).append((int(r["End_Timestamp"]) -
                                            int(r["Start_Timestamp"])) / 1e3)
    return per


def floor_grid(rbytes: int, wbytes: int):
    """(variant, grid size in work-items) of mxq_copy_floor over those bytes."""
    r16, w16 = -(-rbytes // 16), -(-wbytes // 16)
    return ("true" if r16 >= w16 else "false"), -(-w16 // 256) * 256


def summarize_shape(tag: str, configs: str, trace_csv: str, fetch_csv: str, write_csv: str,
                    valu_csv: str, bench_json: str, out_txt: str):
    """One shape's profile from four rocprofv3 runs of bench.py --config-only:
    device durations from the kernel trace, HBM bytes per launch (FETCH_SIZE
    and WRITE_SIZE, KiB per dispatch, scaled by what each counter reads for
    the 1 GiB calibration copy of the same run) against algorithmic bytes, the
    copy floor of each config's bytes, and VALU counters per wavefront.
    Dispatches are grouped by kernel and grid size."""
    run = json.loads([ln for ln in open(bench_json) if ln.startswith("{")][-1])
    cfgs = run["configs"]
    copy_bytes = run["copy_calibration"]["bytes"] // 2
    mean = lambda v: sum(v) / len(v)
    med = lambda v: sorted(v)[len(v) // 2]
    fetch, write, valu = pmc_counters(fetch_csv), pmc_counters(write_csv), pmc_counters(valu_csv)
    dur = trace_durations(trace_csv)
    cal = lambda d, c: [mean(v[c]) for k, v in d.items() if "bitwise_not" in k[0]][0]
    f_scale = copy_bytes / (cal(fetch, "FETCH_SIZE") * 1024)
    w_scale = copy_bytes / (cal(write, "WRITE_SIZE") * 1024)
    # Which config each (kernel, grid) group belongs to.
    owner = {}
    for key in dur:
        short = kernel_short_name(key[0])
        base = short.split("<")[0]
        if base == "copy_floor_kernel":
            var = "true" if "<true>" in short else "false"
            names = [n for n, c in cfgs.items() if "copy_floor_ms" in c and
                     floor_grid(c["bytes_in"], c["bytes_out"]) == (var, key[1])]
            owner[key] = ("floor", names)
        elif "mxq::" in key[0]:
            # A config naming the kernel with its template arguments owns that
            # instance alone; otherwise any instance of the kernel.
            names = [n for n, c in cfgs.items() if short in c["kernels"]]
            if not names:
                names = [n for n, c in cfgs.items() if any(k.split("<")[0] == base
                                                           for k in c["kernels"])]
            owner[key] = ("kernel", names)
    cmds = ["  " + pre.format(tag=tag) + SHAPE_BENCH.format(configs=configs)
            for _, pre in SHAPE_CMDS]
    what = ", ".join(f"{n} ({c['desc']})" for n, c in cfgs.items())
    out = [f"{tag}: rocprofv3 profile of {what}.",
           "", "Commands (repository root, one MI355X, ROCm 7.2, TMPDIR=/tmp; OUT is where the "
           "CSVs go):", *cmds,
           f"Summary: python3 bench.py --summarize-shape {tag} {configs} <stats "
           "kernel_trace.csv> <fetch counter_collection.csv> <write ...> <valu ...> "
           "<stdout of the stats run>", "",
           f"Calibration (int32 bitwise not of {copy_bytes} bytes, read once and written once): "
           f"FETCH_SIZE x {f_scale:.4f}, WRITE_SIZE x {w_scale:.4f} -> bytes.",
           "Durations are device times from the kernel trace (the bench's own event timings in",
           "the traced run include the tracer's per-dispatch overhead and are not used).", "",
           f"{'kernel':<50} {'grid':>9} {'calls':>5} {'avg us':>8} {'HBM read':>12} "
           f"{'HBM write':>12}  config"]
    rows = []
    for key, ts in sorted(dur.items(), key=lambda t: -sum(t[1])):
        if key not in owner:
            continue
        short = kernel_short_name(key[0])
        fk = mean(fetch[key]["FETCH_SIZE"]) * 1024 * f_scale if key in fetch else float("nan")
        wk = mean(write[key]["WRITE_SIZE"]) * 1024 * w_scale if key in write else float("nan")
        kind, names = owner[key]
        label = ("copy floor of " if kind == "floor" else "") + ", ".join(names)
        out.append(f"{short[:50]:<50} {key[1]:>9} {len(ts):>5} {mean(ts):>8.2f} {fk:>12.0f} "
                   f"{wk:>12.0f}  {label}")
        rows.append((key, short, kind, names, mean(ts), fk, wk))
    out += ["", "Per config (kernels owned by that config alone; algorithmic bytes count each "
            "input read once and each output written once):", "",
            f"{'config':<18} {'kernel us':>9} {'% of 8TB/s':>10} {'HBM bytes':>12} "
            f"{'algorithmic':>12} {'ratio':>6} {'floor us':>9} {'floor/kernel':>12}"]
    notes = set()
    for n, c in cfgs.items():
        mine = [r for r in rows if r[2] == "kernel" and r[3] == [n]]
        fl = [r for r in rows if r[2] == "floor" and n in r[3]]
        if mine:
            t = sum(r[4] for r in mine)
            hbm = sum(r[5] + r[6] for r in mine)
            hbm_s, ratio_s = f"{hbm:>12.0f}", f"{hbm / c['bytes']:>6.3f}"
        else:       # kernels shared with other configs of the run: the bench's timing
            t = 1e3 * c["ms_median"]
            hbm_s, ratio_s = f"{'-':>12}", f"{'-':>6}"
            notes.add("b")
        # A floor grid serves every config of the same read and write bytes;
        # configs of equal write bytes but other read bytes share its grid
        # without sharing its time.
        if len(fl) == 1 and len({(cfgs[m]["bytes_in"], cfgs[m]["bytes_out"])
                                 for m in fl[0][3]}) == 1:
            ft, mark = fl[0][4], " "
        else:
            ft, mark = 1e3 * c.get("copy_floor_ms", float("nan")), "*"
            notes.add("f")
        out.append(f"{n:<18} {t:>9.2f}{'b' if not mine else ' '} "
                   f"{100 * c['bytes'] / (t * 1e-6) / 8e12:>9.2f} {hbm_s} {c['bytes']:>12} "
                   f"{ratio_s} {ft:>8.2f}{mark} {ft / t:>12.3f}")
    if "b" in notes:
        out.append("b: the config's kernels also run for other configs of this run; its time is "
                   "the bench's median per call (tracer overhead included).")
    if "f" in notes:
        out.append("*: the copy floor's grid is shared with a config of other read bytes; the "
                   "floor time is the bench's median for this config's bytes (tracer overhead "
                   "included).")
    out += ["", "VALU counters (medians over dispatches); per wave: instructions, conversion",
            "instructions, VALU issue quad-cycles; 'VALU share' = SQ_ACTIVE_INST_VALU /",
            "SQ_WAVE_CYCLES, the fraction of the waves' resident time spent issuing VALU:", "",
            f"{'kernel':<50} {'grid':>9} {'waves':>7} {'VALU/w':>7} {'cvt/w':>6} {'qcyc/w':>7} "
            f"{'VALU share':>10}"]
    for key, short, *_ in rows:
        if key not in valu:
            continue
        c = {k: med(v) for k, v in valu[key].items()}
        w = c["SQ_WAVES"]
        out.append(f"{short[:50]:<50} {key[1]:>9} {w:>7.0f} {c['SQ_INSTS_VALU'] / w:>7.1f} "
                   f"{c['SQ_INSTS_VALU_CVT'] / w:>6.1f} {c['SQ_ACTIVE_INST_VALU'] / w:>7.1f} "
                   f"{c['SQ_ACTIVE_INST_VALU'] / c['SQ_WAVE_CYCLES']:>10.3f}")
    with open(out_txt, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_stats(trace_csv: str, out_txt: str, title: str, cmd: str = STATS_CMD,
                    flag: str = "--summarize-stats"):
    """Per (kernel, grid size) statistics of a rocprofv3 kernel trace as a text
    table: launches of one kernel on different shapes stay apart."""
    dur = trace_durations(trace_csv)
    total = sum(sum(v) for v in dur.values())
    rows = []
    for (name, grid), ts in dur.items():
        short = (kernel_short_name(name) if "mxq::" in name else
                 name.replace("(anonymous namespace)", "{anon}").split("(")[0]
                 .replace("void ", ""))
        rows.append((short, grid, len(ts), sum(ts) / len(ts), min(ts), max(ts),
                     100.0 * sum(ts) / total))
    rows.sort(key=lambda t: -t[6])
    out = [title, "", "Command (run from the repository root on one MI355X, ROCm 7.2; OUT is the "
           "directory the CSVs go to):",
           "  " + cmd, f"Summary: python3 bench.py {flag} <kernel_trace.csv>", "",
           "Device durations from the kernel trace, per kernel and grid size (work-items).", "",
           f"{'kernel':<60} {'grid':>10} {'calls':>6} {'avg us':>10} {'min us':>10} "
           f"{'max us':>10} {'share':>6}"]
    for name, grid, calls, avg, mn, mx, pct in rows:
        out.append(f"{name[:60]:<60} {grid:>10} {calls:>6} {avg:>10.2f} {mn:>10.2f} "
                   f"{mx:>10.2f} {pct:>5.1f}%")
    with open(out_txt, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config timings (50 back-to-back launches over "
                         "rotating buffer sets)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--groups", default="act,wgt,tok,exp,grp",
                    help="comma list of leg groups to run (for profiling single kernels); "
                         "'dsp' adds the fused-dispatch legs, 'qdq' the one-pass quantize + "
                         "dequant legs, 'gemm' the dense-layer GEMMs; the first two replace legs "
                         "of the default step (the separate gather; quantize followed by "
                         "dequant) and the GEMMs consume its outputs, so none is part of it")
    ap.add_argument("--config-only", default=None,
                    help="comma list of config names (C2a_<mode>, C2b_<mode>, C2b_rowcol_t, C3_nvfp4, "
                         "C3_dequant, C4_gateup, C4_down, C4_gateup_amax, C4_down_amax, C5_mxfp8, C5_nvfp4, C5_dequant_mxfp8, "
                         "C5_dequant_nvfp4, C5_colt_mxfp8, C5_rowcolt_mxfp8, C5_qdq_<fmt>, C2b_qdq_mxfp8, "
                         "C3_qdq_nvfp4, G_<gemm>): time "
                         "only these, each beside its copy floor, and "
                         "print them as one JSON line (no step, no CPU baseline); for "
                         "profiling one shape per run")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also time a plain elementwise copy of this many MiB (int32 bitwise "
                         "not, reads and writes each byte once), reported apart from the step, "
                         "to scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "BENCH_LOG"),
                    help="(no GPU) write profiles/traffic.json and its text table from the "
                         "counter CSVs of the FETCH_SIZE and WRITE_SIZE runs and the bench output "
                         "of the first")
    ap.add_argument("--summarize-shape", nargs=7,
                    metavar=("TAG", "CONFIGS", "STATS_CSV", "FETCH_CSV", "WRITE_CSV", "VALU_CSV",
                             "BENCH_JSON"),
                    help="(no GPU) write profiles/TAG_profile.txt from the four rocprofv3 runs of "
                         "bench.py --config-only CONFIGS --copy-calibration-mib 1024")
    ap.add_argument("--summarize-gemm-stats", metavar="KERNEL_TRACE_CSV",
                    help="(no GPU) write profiles/gemm_kernels_stats.txt from rocprofv3's "
                         "kernel trace of the GEMM configs")
    ap.add_argument("--summarize-stats", metavar="KERNEL_TRACE_CSV",
                    help="(no GPU) write profiles/step_all_kernels_stats.txt from rocprofv3's "
                         "kernel trace")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, TRAFFIC_FILE,
                      os.path.join(ROOT, "profiles", "grouped_262144x2048_hbm_traffic.txt"))
        return
    if args.summarize_shape:
        tag = args.summarize_shape[0]
        summarize_shape(*args.summarize_shape,
                        os.path.join(ROOT, "profiles", f"{tag}_profile.txt"))
        return
    if args.summarize_gemm_stats:
        summarize_stats(args.summarize_gemm_stats,
                        os.path.join(ROOT, "profiles", "gemm_kernels_stats.txt"),
                        "rocprofv3 kernel statistics of the GEMM configs (each: 2 warm-up "
                        "launches, then 5 samples of 10 back-to-back launches): dense MXFP8 2048x8192x2048 "
                        "and 8192x8192x2048, dense NVFP4 2048x8192x2048, the grouped MXFP8 and "
                        "NVFP4 expert layers over config 5's 262144 rows (128 experts, 768x2048 "
                        "weights) and the grouped MXFP8 weight gradient (dW_e 768x2048).",
                        GEMM_STATS_CMD, "--summarize-gemm-stats")
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats,
                        os.path.join(ROOT, "profiles", "step_all_kernels_stats.txt"),
                        "rocprofv3 kernel statistics of bench.py: every leg of the step (MXFP8 "
                        "row+col 2048x2048 and 8192x2048, per-token NVFP4 8192x2048, NVFP4 export "
                        "of 128 experts, grouped MXFP8/NVFP4 262144x2048 and their dequant) plus "
                        "the fused-dispatch legs (32768 tokens top-8 of 128), the one-pass "
                        "quantize + dequant legs (262144x2048) and the dense-layer GEMMs "
                        "(2048x8192x2048).")
        return

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the quantizers shard by rows with no exchange, "
              "and runs on several GPUs are not supported (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_block_scaled_amax_amd as mxq
    from nvfp4_block_scaled_amax_amd import api
    from nvfp4_block_scaled_amax_amd import workloads as W

    mxq.lib()
    torch.cuda.set_device(0)
    if args.config_only:
        only = set(args.config_only.split(","))
        need = set()
        if only & {"C4_gateup", "C4_down", "C4_gateup_amax", "C4_down_amax"}:
            need.add("exp")
        if any(c.startswith("C5_") for c in only):
            need.add("grp")
        legs = build_legs(torch, mxq, api, W, log,
                          want=lambda g: g in need and g not in ("act", "wgt"))
        res = config_timings(torch, mxq, W, legs, log, only=only)
        calib = None
        if args.copy_calibration_mib > 0:
            nbytes = args.copy_calibration_mib << 20
            src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32,
                                device="cuda")
            dst = torch.empty_like(src)
            ms = time_launches(torch, [lambda: torch.bitwise_not(src, out=dst)], 5, 2, 1)
            calib = {"bytes": 2 * nbytes, "ms": round(float(np.median(ms)), 5)}  # in + out
            del src, dst
        print(json.dumps({"configs": res, "copy_calibration": calib,
                          "csrc_digest": csrc_digest()}), flush=True)
        return
    t_gen = time.perf_counter()
    groups = set(args.groups.split(","))
    legs = build_legs(torch, mxq, api, W, log, want=lambda g: g in groups)
    calib = None
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        calib = Leg("copy_calibration", lambda: torch.bitwise_not(src, out=dst), nbytes, nbytes,
                    nbytes // 4, ["elementwise_kernel"], f"int32 bitwise not of {nbytes} bytes")
    log(f"inputs generated and resident in {time.perf_counter() - t_gen:.1f} s")

    stream = torch.cuda.current_stream()

    def step(timed):
        for leg in legs:
            if timed:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                leg.launch()
                b.record(stream)
                leg._ev.append((a, b))
            else:
                leg.launch()

    for leg in legs:
        leg._ev = []
    for _ in range(args.warmup):
        step(False)
    if calib is not None:
        calib._ev = []
        for _ in range(args.warmup):
            calib.launch()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(True)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if calib is not None:
        for _ in range(args.steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            calib.launch()
            b.record(stream)
            calib._ev.append((a, b))
        torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall:.2f} s)")

    total_bytes = sum(l.bytes for l in legs)
    total_elems = sum(l.elems for l in legs)
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    def info(l):
        ts = [a.elapsed_time(b) for a, b in l._ev]
        ms = float(np.mean(ts))
        gbs = l.bytes / (ms * 1e-3) / 1e9
        return {"desc": l.desc, "kernels": l.kernels, "ms": round(ms, 5),
                "ms_min": round(float(np.min(ts)), 5), "bytes": l.bytes, "GB_s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                "elements_per_s": round(l.elems / (ms * 1e-3), 1)}

    leg_info = {l.name: info(l) for l in legs}
    # The dominant kernel: the longest leg that is one launch of one kernel
    # (with up to 256 segments the grouped kernels form their segment prefix
    # themselves; above that a ~4 us prefix launch precedes them).
    # The export legs (four kernels, two reads of the weights) and the
    # three-launch export dequant are reported per leg but are not one launch.
    single = [l for l in legs if l.name not in ("nvfp4_export_gateup", "nvfp4_export_down",
                                                "nvfp4_export_dequant", "gather_torch",
                                                "gemm_mxfp8", "gemm_nvfp4")]
    dom = max(single or legs, key=lambda l: leg_info[l.name]["ms"])
    dom_ms = leg_info[dom.name]["ms"]
    achieved = dom.bytes / (dom_ms * 1e-3) / 1e9
    # HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated
    # against a plain copy; null once the kernel's sources have changed.
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f).get("kernels", {}).get(dom.kernels[-1])
        if tr and tr.get("source_digest") == kernel_digest(dom.kernels[-1]) \
                and tr.get("leg") == dom.name:
            traffic = tr.get("hbm_bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom.kernels[-1], "leg": dom.name, "leg_kernels": dom.kernels,
                "algorithmic_bytes": dom.bytes, "ms_per_launch": dom_ms}

    configs = None
    if not args.no_configs and "grp" in groups:
        configs = config_timings(torch, mxq, W, legs, log)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W, log)
        cpu["gpu_over_cpu"] = round(value / cpu["value"], 1)
        cpu["gpu_over_cpu_single_thread"] = round(value / cpu["single_thread"]["value"], 1)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->mxfp8|nvfp4",
        "data": "synthetic",
        "config": {"workload": "moe-layer quantize step: MXFP8 row+col 2048x2048 + 8192x2048, "
                               "per-token NVFP4 8192x2048 + dequant, NVFP4 export of 128 "
                               "experts (gate/up pairs + down) + dequant, grouped MXFP8 row+col "
                               "+ NVFP4 over 262144x2048 top-8/128 + dequant",
                   "groups": sorted(groups), "bytes_per_step": total_bytes,
                   "elements_per_step": total_elems},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "elements_per_s": round(total_elems / (ms_per_step * 1e-3), 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "legs": leg_info,
        "configs": configs,
        "copy_calibration": info(calib) if calib is not None else None,
        "csrc_digest": csrc_digest(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
