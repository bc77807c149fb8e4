"""Benchmark of the gated delta rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--legs prefill,prefill_b4,decode,gdp,long_packed,gates,boundary,
                            conv_norm,backward]

Nine legs, each timed over exactly K steps bracketed by torch.cuda.synchronize():
  prefill: packed varlen gated delta rule, 8 sequences of U{1..8192} tokens
           (~32.8K tokens), 16 q/k heads shared by 32 v heads, K = V = 128, bf16
           q/k/v, fp32 g/beta, fp32 slot-cache states, chunk 64.  Its tokens/s is
           the headline `value`.
  prefill_b4: the batched gated delta rule, B=4, T=4096, H=16, K = V = 128, bf16
           q/k/v, fp32 g/beta, a random N(0, 0.1) initial state and the final
           state written, chunk 64; tokens/s with its HBM and matrix-core
           fractions.
  decode:  one token for each of 128 requests (16 padding) over a
           [256, 32, 128, 128] fp32 slot cache; reported as state GB/s.  The
           256 MB last-level cache is flushed (1 GiB read) before every launch,
           outside the timed launch.
  gdp:     gated delta product, 2 Householder sub-steps, B=1, T=65536, H=32,
           K = V = 128, bf16, chunk 128 tokens; tokens/s.
  long_packed: one packed request of 65 536 tokens over a slot cache (cu_seqlens,
           H = 32, K = V = 128, bf16): the segment slots planned on the device,
           against the single pass; tokens/s.
  gates:   the prefill and decode workloads again with g and beta given as raw
           projections and formed inside the kernels (A_log, dt_bias); kernel
           times and their ratio to the legs above.
  boundary: the prefill again, also writing boundary states every 1024 and every
           64 tokens (prefix caching); kernel times and bytes written.
  conv_norm: the short causal conv over the workload's V/K/Q projection (prefill
           and a 128-request decode step) and the gated RMS norm of its output;
           kernel times and achieved bandwidth.
  backward: the chunked backward (gradients of q, k, v, g, beta and the initial
           state) at B=4, T=4096, H=16, D=128, bf16 inputs, and of the gated delta
           product (n_h = 2) at B=1, T=16384, H=32; one call = the forward
           recompute plus the backward kernels; tokens/s, the fraction of the
           bf16 matrix-core peak its dense contractions reach (their products of
           bf16 inputs run on the fp16 matrix cores) and the HBM rate of its
           algorithmic bytes; the roofline object is the one of the two whose
           algorithmic time at peak is longer (HBM at these shapes).
Kernel durations come from HIP events on the launch stream: one pair around the K
back-to-back launches (a pair around each launch where a cache flush precedes it).  The
roofline object is for the headline prefill kernel: algorithmic HBM bytes per
launch (inputs read once, outputs and states written once) over the mean launch
time, against 8 TB/s.  The CPU baseline is the fp64 oracle on a bounded sample
of the prefill workload, on all host cores.
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

METRIC = "prefill tokens/s (H=32,K=V=128) + decode state GB/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2516.6   # dense fp16/bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs",
                    default="prefill,prefill_b4,decode,gdp,long_packed,gates,boundary,conv_norm,"
                            "backward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32,
                    help="value heads of the prefill workload the CPU oracle runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU oracle repeats its sample until this much time has passed")
    ap.add_argument("--profile-run", action="store_true",
                    help="a short run for hardware-counter profiling: 3 prefill and 3 decode "
                         "launches plus a device copy of known size (counter calibration)")
    ap.add_argument("--summarize-db", metavar="DB",
                    help="print a text summary of a rocprofv3 results database and exit")
    ap.add_argument("--mfma-from", metavar="DB",
                    help="matrix-core flops and utilisation per kernel from a counter pass")
    ap.add_argument("--lds-from", metavar="DB",
                    help="print LDS bank-conflict counters per kernel from a rocprofv3 database")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="derive HBM bytes per launch from a FETCH_SIZE and a WRITE_SIZE "
                         "profile of --profile-run, write profiles/traffic.json and exit")
    return ap.parse_args()


PROFILES = os.path.join(ROOT, "profiles")
COPY_PROBE_BYTES = 1 << 30     # the calibration copy reads and writes 1 GiB each


def kernel_source_hash(name, text=None):
    """sha256 of a kernel source file's code (comments and whitespace removed): ties
    stored counter data to the code measured, not to its commentary."""
    import hashlib
    import re
    if text is None:
        path = os.path.join(ROOT, "gated_delta_rule_71_amd", "csrc", name)
        with open(path, encoding="utf-8") as f:
            text = f.read()
    code = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = re.sub(r"\s+", "", code)
    return hashlib.sha256(code.encode("utf-8")).hexdigest()[:16]


def stored_traffic(kernel, source):
    """Counter-measured HBM bytes per launch for `kernel`, if taken on this source."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(kernel)
    if not rec or rec.get("source_sha") != kernel_source_hash(source):
        return None
    return rec.get("bytes_per_launch")


def summarize_db(db):
    """Kernel durations and hardware counters per kernel from a rocprofv3 database."""
    import sqlite3
    con = sqlite3.connect(db)
    tabs = {r[0] for r in con.execute("select name from sqlite_master")}
    if "top_kernels" in tabs and con.execute("select count(*) from top_kernels").fetchone()[0]:
        print("kernel durations (us): name | calls | total | average | percent")
        for name, calls, tot, avg, pct in con.execute(
                "select name, total_calls, total_duration, average, percentage "
                "from top_kernels order by total_duration desc"):
            print(f"  {name[:110]} | {calls} | {tot:.0f} | {avg:.1f} | {pct:.2f}")
    if "kernels" in tabs and con.execute("select count(*) from kernels").fetchone()[0]:
        # the same kernel on different workloads differs in its grid
        print("by launch grid (us): name | grid (threads) | calls | average")
        for name, gx, gy, calls, avg in con.execute(
                "select name, grid_x, grid_y, count(*), avg(end - start) / 1000.0 from kernels "
                "group by name, grid_x, grid_y order by sum(end - start) desc"):
            print(f"  {name[:100]} | {gx}x{gy} | {calls} | {avg:.1f}")
    if "pmc_events" in tabs and con.execute("select count(*) from pmc_events").fetchone()[0]:
        print("counters per dispatch (summed over instances): dispatch | kernel | counter | value")
        rows = con.execute(
            "select dispatch_id, name, counter_name, sum(counter_value) from pmc_events "
            "group by dispatch_id, counter_name order by dispatch_id").fetchall()
        for d, name, cn, val in rows:
            print(f"  {d} | {name[:90]} | {cn} | {val:.6g}")


def traffic_from(fetch_db, write_db):
    """HBM bytes per launch of the prefill and decode kernels from two counter profiles.

    Each counter is scaled by what it reads for the calibration copy of
    COPY_PROBE_BYTES (the largest device copy in the profile), so the result is
    in bytes whatever unit or coverage the counter has on this part.
    """
    import sqlite3

    def per_kernel(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute(
            "select dispatch_id, name, sum(counter_value) from pmc_events where counter_name = ? "
            "group by dispatch_id", (counter,)).fetchall()
        copy = max(v for _, n, v in rows if "copyBuffer" in n)
        scale = COPY_PROBE_BYTES / copy
        out = {}
        for key, pat in (("prefill_varlen", "prefill64_kernel"), ("decode", "decode_kernel")):
            vals = [v for _, n, v in rows if pat in n]
            out[key] = (float(np.mean(vals)) * scale, len(vals))
        return out, scale

    fetch, fs = per_kernel(fetch_db, "FETCH_SIZE")
    write, ws = per_kernel(write_db, "WRITE_SIZE")
    data = {}
    for key, src in (("prefill_varlen", "prefill64.hip"), ("decode", "decode.hip")):
        data[key] = {"source_sha": kernel_source_hash(src),
                     "fetch_bytes": fetch[key][0], "write_bytes": write[key][0],
                     "bytes_per_launch": fetch[key][0] + write[key][0],
                     "launches": fetch[key][1]}
    data["calibration"] = {"copy_bytes": COPY_PROBE_BYTES, "fetch_scale": fs, "write_scale": ws,
                           "note": "counter value x scale = bytes; scale from the copy probe"}
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(data, indent=1))


def mfma_from(db):
    """Matrix-core work per kernel from one counter pass (SQ_INSTS_VALU_MFMA_MOPS_F16,
    SQ_INSTS_VALU_MFMA_MOPS_F32, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE): flops =
    MOPS x 512 (the counters count multiply or add operations / 512), achieved
    TFLOP/s over the dispatch's traced duration, and the utilisation
    sum(MFMA busy cycles) / (max(GUI active cycles) x 1024 SIMDs)."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute(
        "select dispatch_id, name, counter_name, sum(counter_value), max(counter_value) "
        "from pmc_events group by dispatch_id, counter_name").fetchall()
    per = {}
    for d, name, cn, total, peak in rows:
        per.setdefault(d, {"name": name})[cn] = peak if cn == "GRBM_GUI_ACTIVE" else total
    dur = {}
    tabs = {r[0] for r in con.execute("select name from sqlite_master")}
    if "kernels" in tabs:
        for d, t0, t1 in con.execute("select dispatch_id, start, end from kernels"):
            dur[d] = (t1 - t0) * 1e-9
    print("dispatch | kernel | MFMA flops (f16, f32) | duration us | TFLOP/s | MFMA busy %")
    for d in sorted(per):
        r = per[d]
        f16 = r.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) * 512
        f32 = r.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) * 512
        if f16 + f32 == 0:
            continue
        busy, active = r.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), r.get("GRBM_GUI_ACTIVE", 0.0)
        util = 100.0 * busy / (active * 1024) if active else float("nan")
        t = dur.get(d)
        tf = (f16 + f32) / t / 1e12 if t else float("nan")
        print(f"  {d} | {r['name'][:70]} | {f16:.4g}, {f32:.4g} | "
              f"{t * 1e6 if t else float('nan'):.1f} | {tf:.1f} | {util:.1f}")


def lds_from(db):
    """LDS bank conflicts per kernel from one counter pass (SQ_LDS_BANK_CONFLICT,
    SQ_LDS_IDX_ACTIVE, SQ_INSTS_LDS, GRBM_GUI_ACTIVE), dispatches of one kernel
    summed: conflict cycles / LDS-active cycles, and per-dispatch means."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute(
        "select dispatch_id, name, counter_name, sum(counter_value), max(counter_value) "
        "from pmc_events group by dispatch_id, counter_name").fetchall()
    per = {}
    for d, name, cn, total, peak in rows:
        per.setdefault(d, {"name": name})[cn] = peak if cn == "GRBM_GUI_ACTIVE" else total
    agg = {}
    for r in per.values():
        a = agg.setdefault(r["name"][:90], [0, 0.0, 0.0, 0.0, 0.0])
        a[0] += 1
        for i, cn in enumerate(("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS",
                                "GRBM_GUI_ACTIVE"), 1):
            a[i] += r.get(cn, 0.0)
    print("kernel | dispatches | conflict / LDS-active | LDS-active per dispatch | "
          "LDS instructions per dispatch | GUI-active per dispatch")
    for name, (n, conf, act, insts, gui) in sorted(agg.items(), key=lambda x: -x[1][2]):
        if act:
            print(f"  {name} | {n} | {conf / act:.3f} | {act / n:.3g} | {insts / n:.3g} | "
                  f"{gui / n:.3g}")


def up(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def nbytes(*arrays):
    return int(sum(a.nbytes for a in arrays if a is not None))


def time_launches(launch, steps, warmup, before=None):
    """Run `launch` warmup + steps times; returns (wall ms/step, mean event ms/launch)."""
    import torch
    for _ in range(warmup):
        if before:
            before()
        launch()
    torch.cuda.synchronize()
    evs = []
    stream = torch.cuda.current_stream()
    wall = 0.0
    if before is None:
        # one event pair around the K back-to-back launches: an event between launches
        # would add its own marker packet (and cache release) to every launch's time
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(steps):
            launch()
        end.record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        evs = [start.elapsed_time(end) / steps]
    else:
        # per-launch preparation (cache flush) stays outside the timed launches
        for i in range(steps):
            before()
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record(stream)
            launch()
            e.record(stream)
            torch.cuda.synchronize()
            evs.append(s.elapsed_time(e))
        wall = float(np.mean(evs))
    return wall, float(np.mean(evs))


def prefill_bytes(wl, out_bytes_per_elem=2):
    """Algorithmic HBM bytes of one prefill: inputs once, output once, states in and out."""
    B, T, Hk, Hv, K, V = wl.shape
    N = wl.num_seqs
    tokens = B * T
    io = nbytes(wl.q, wl.k, wl.v, wl.g, wl.beta) + tokens * Hv * V * out_bytes_per_elem
    states = 2 * N * Hv * K * V * 4
    return io + states


def prefill_flops_per_token(wl, chunk_tokens):
    """Dense-tile flops per token of the chunked form with chunks of C tokens.

    The delta rule: per q/k head the chunk's K K^T and Q K^T (2 C K each), per value
    head W = T diag(beta e^G) K and U = T diag(beta) V (2 C K + 2 C V), the
    intra-chunk P D (2 C V) and the state products K H, Q H and K^T D (2 K V each).
    The product with n_h sub-steps per token runs the same steps on n_h C rows per
    chunk, with queries on one row per token."""
    B, T, Hk, Hv, K, V = wl.shape
    n_h = wl.num_householder
    C = chunk_tokens
    if n_h == 1:
        return Hk * 4 * C * K + Hv * (2 * C * K + 4 * C * V + 6 * K * V)
    return Hv * ((4 * n_h + 2) * K * V + 2 * n_h * n_h * C * (2 * K + V) + 2 * n_h * C * (K + V))


def run_prefill_leg(wl, steps, warmup, boundary_interval=None, segments=True):
    import torch
    import gated_delta_rule_71_amd as gdr
    d = {n: up(getattr(wl, n)) for n in ("q", "k", "v", "g", "beta")}
    cu = up(wl.cu_seqlens)
    idx = up(wl.state_indices)
    h0 = up(wl.initial_state)
    out = torch.empty((wl.q.shape[0], wl.q.shape[1], wl.v.shape[-2], wl.v.shape[-1]),
                      dtype=torch.bfloat16, device="cuda")
    fs = torch.empty_like(h0) if idx is None else h0
    gate = dict(A_log=up(wl.A_log), dt_bias=up(wl.dt_bias))   # None unless raw gates
    if boundary_interval:
        lens = np.diff(wl.cu_seqlens) if wl.cu_seqlens is not None else [wl.q.shape[1]] * \
            wl.q.shape[0]
        E = gdr.boundary_count(lens, boundary_interval)
        gate.update(boundary_states=torch.empty((E,) + tuple(h0.shape[1:]), dtype=torch.float32,
                                                device="cuda"),
                    boundary_interval=boundary_interval)
    # one checked call through the Python binding, then the same C call with the
    # argument struct built once, so the timed launches carry no Python marshalling
    gdr.chunk_gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"],
                               chunk_size=wl.chunk_size, initial_state=h0,
                               output_final_state=True, cu_seqlens=cu, state_indices=idx,
                               out=out, final_state=fs, segments=segments, **gate)
    args = gdr.prefill_args(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=wl.chunk_size,
                            initial_state=h0, final_state=fs, cu_seqlens=cu,
                            state_indices=idx, out=out, **gate)
    lib = gdr.library()
    # long batched rows run in segments when given the workspace
    need = int(lib.gdr_prefill_workspace_bytes(args))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if segments and need else None
    if ws is not None:
        args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.gdr_chunk_gated_delta_rule(args, stream)
        assert rc == 0, rc

    wall, kern = time_launches(launch, steps, warmup)
    return wall, kern


def run_decode_leg(wl3, steps, warmup):
    import torch
    import gated_delta_rule_71_amd as gdr
    d = [up(x) for x in (wl3.q, wl3.k, wl3.v, wl3.g, wl3.beta)]
    cache = up(wl3.cache)
    idx = up(wl3.batch_indices)
    gate = dict(A_log=up(wl3.A_log), dt_bias=up(wl3.dt_bias))   # None unless raw gates
    out = torch.empty((wl3.q.shape[0], wl3.v.shape[1], wl3.v.shape[2]),
                      dtype=torch.bfloat16, device="cuda")
    # 1 GiB read before each launch evicts the 256 MB last-level cache without
    # leaving dirty lines to be written back during the timed launch
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    gdr.ssm_decode(*d, cache, batch_indices=idx, out=out, **gate)
    dargs = gdr.decode_args(*d, cache, batch_indices=idx, out=out, **gate)
    lib = gdr.library()
    stream = torch.cuda.current_stream().cuda_stream

    def launch_dec():
        rc = lib.gdr_ssm_decode(dargs, stream)
        assert rc == 0, rc

    wall, kern = time_launches(launch_dec, steps, warmup, before=lambda: flush.sum())
    del cache, flush
    return wall, kern


def run_conv_norm_leg(wl2, steps, warmup):
    """The conv over the packed V/K/Q projection of the prefill workload (C = 2 Hk K
    + Hv V channels, W = 4, SiLU, slot-indexed conv state), the cached conv decode
    of 128 requests, and the gated RMS norm of the prefill output; kernel times and
    bytes (read + written once) against the HBM peak."""
    import torch
    import gated_delta_rule_71_amd as gdr
    rng = np.random.default_rng(9)
    T = wl2.tokens
    Hk, K = wl2.q.shape[2], wl2.q.shape[3]
    Hv, V = wl2.v.shape[-2], wl2.v.shape[-1]
    C, Wd = 2 * Hk * K + Hv * V, 4
    N = wl2.num_seqs
    x = torch.randn((T, C), device="cuda", dtype=torch.bfloat16)
    w = torch.randn((C, Wd), device="cuda") * 0.5
    b = torch.randn(C, device="cuda") * 0.1
    cu = up(wl2.cu_seqlens)
    state = torch.zeros((2 * N, C, Wd - 1), device="cuda")
    idx = torch.from_numpy(rng.permutation(2 * N)[:N].astype(np.int32)).cuda()
    y = torch.empty_like(x)
    lib = gdr.library()
    stream = torch.cuda.current_stream().cuda_stream
    a = gdr.conv_prefill_args(x, w, b, cu, conv_state=state, state_indices=idx, out=y)
    assert lib.gdr_causal_conv1d_prefill(a, stream) == 0
    _, kc = time_launches(lambda: lib.gdr_causal_conv1d_prefill(a, stream), steps, warmup)
    conv_bytes = 2 * x.numel() * 2
    n = 128
    xd = torch.randn((n, 1, C), device="cuda", dtype=torch.bfloat16)
    sd = torch.zeros((256, C, Wd - 1), device="cuda")
    bi = torch.from_numpy(rng.permutation(256)[:n].astype(np.int32)).cuda()
    yd = torch.empty_like(xd)
    ad = gdr.conv_decode_args(xd, w, b, sd, batch_indices=bi, out=yd)
    assert lib.gdr_causal_conv1d_decode(ad, stream) == 0
    _, kd = time_launches(lambda: lib.gdr_causal_conv1d_decode(ad, stream), steps, warmup)
    dec_bytes = 2 * xd.numel() * 2 + 2 * n * C * (Wd - 1) * 4
    o = torch.randn((T, Hv, V), device="cuda", dtype=torch.bfloat16)
    z = torch.randn((T, Hv, V), device="cuda", dtype=torch.bfloat16)
    wn = torch.ones(Hv * V, device="cuda")
    yn = torch.empty_like(o)
    gdr.gated_rmsnorm(o, z, wn, out=yn)

    def norm_launch():
        gdr.gated_rmsnorm(o, z, wn, out=yn)

    _, kn = time_launches(norm_launch, steps, warmup)
    norm_bytes = 3 * o.numel() * 2
    gbs = lambda byt, ms: byt / (ms * 1e-3) / 1e9
    # reference: a plain device copy of the conv's input (the same bytes read and
    # written once), what a stream of this size reaches on this part
    xc = torch.empty_like(x)
    _, kcp = time_launches(lambda: xc.copy_(x), steps, warmup)
    copy_gbs = gbs(conv_bytes, kcp)
    return {
        "copy_reference": {"kernel_ms": kcp, "bytes": conv_bytes, "achieved_gbs": copy_gbs,
                           "hbm_frac": copy_gbs / HBM_PEAK_GBS,
                           "note": "torch device copy of the conv input (read + write once)"},
        "conv_prefill": {"kernel_ms": kc, "channels": C, "tokens": T, "bytes": conv_bytes,
                         "achieved_gbs": gbs(conv_bytes, kc),
                         "hbm_frac": gbs(conv_bytes, kc) / HBM_PEAK_GBS,
                         "vs_copy": gbs(conv_bytes, kc) / copy_gbs,
                         "note": "two launches: outputs, then the conv-state update"},
        "conv_decode": {"kernel_ms": kd, "requests": n, "bytes": dec_bytes,
                        "achieved_gbs": gbs(dec_bytes, kd)},
        "gated_rmsnorm": {"kernel_ms": kn, "rows": T * Hv, "group": V, "bytes": norm_bytes,
                          "achieved_gbs": gbs(norm_bytes, kn),
                          "hbm_frac": gbs(norm_bytes, kn) / HBM_PEAK_GBS,
                          "vs_copy": gbs(norm_bytes, kn) / copy_gbs},
    }


def backward_flops_per_token(Hv, D, C=64, n_h=1):
    """Dense-tile flops per token of the backward kernels (forward recompute excluded):
    per 64-row chunk and value head, eleven C x C x D products (K K^T, Q K^T, T R;
    P^T dO, T^T dD; dR D^T, dO D^T, dPs K, dAs K, dAs^T K, dPs^T Q) and seven C x D x D
    ones (K H0; K dH, Q^T dO, K^T dR; dO H0^T, dR H0^T, D dH^T), 2 flops per
    multiply-add; n_h rows per token."""
    return n_h * Hv * (22 * C * D + 14 * D * D)


def run_backward_leg(steps, warmup, *, name="bwd_bf16_B4_T4096_H16_D128", B=4, T=4096, H=16,
                     n_h=1):
    import torch
    import gated_delta_rule_71_amd as gdr
    from gated_delta_rule_71_amd import workloads as W
    bw = W.backward_workload(name, 1, Hk=H, Hv=H, D=128, dtype=W.BF16, B=B, T=T, decay="config",
                             num_householder=n_h)
    f = bw.fwd
    d = {n: up(getattr(f, n)) for n in ("q", "k", "v", "g", "beta")}
    do, dht, h0 = up(bw.do), up(bw.dht), up(f.initial_state)
    gdr.chunk_gated_delta_rule_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], do, dht=dht,
                                        initial_state=h0)
    B, T, Hk, D = f.q.shape
    Hv = f.v.shape[-2]
    outs = [torch.empty(s, dtype=torch.float32, device="cuda")
            for s in ((B, T, Hk, D), f.k.shape, f.v.shape, (B, T, Hv), f.beta.shape,
                      (B, Hv, D, D))]
    a = gdr.backward_args(d["q"], d["k"], d["v"], d["g"], d["beta"], do, dq=outs[0],
                          dk=outs[1], dv=outs[2], dg=outs[3], dbeta=outs[4], dh0=outs[5],
                          dht=dht, initial_state=h0)
    lib = gdr.library()
    ws = torch.empty(int(lib.gdr_backward_workspace_bytes(a)), dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.gdr_chunk_gated_delta_rule_backward(a, stream)
        assert rc == 0, rc

    wall, kern = time_launches(launch, steps, warmup)
    tokens = B * T
    F = backward_flops_per_token(Hv, D, n_h=n_h)
    tf = F * tokens / (kern * 1e-3) / 1e12
    # algorithmic bytes: bf16 q, k, v, dO and fp32 g, beta read once, fp32 gradients
    # written once, the initial state and dH_T read and dH0 written once
    rows = tokens * n_h
    alg = (2 * (tokens * Hk * D + rows * Hk * D + rows * Hv * D + tokens * Hv * D)
           + 4 * (tokens * Hv + rows * Hv)
           + 4 * (tokens * Hk * D + rows * Hk * D + rows * Hv * D + tokens * Hv + rows * Hv)
           + 4 * 3 * B * Hv * D * D)
    gbs = alg / (kern * 1e-3) / 1e9
    mfma = {"achieved": tf, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / MFMA_PEAK_TFLOPS,
            "note": "products of bf16 inputs on the fp16 matrix cores, other operands as "
                    "fp16 hi/lo pairs (the extra instructions not counted)"}
    hbm = {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
           "algorithmic_bytes": alg,
           "note": "the per-chunk states and matrices of the workspace come on top of these "
                   "bytes"}
    # the roofline's bound: the larger of the two algorithmic times at peak
    hbm_bound = alg / (HBM_PEAK_GBS * 1e9) >= F * tokens / (MFMA_PEAK_TFLOPS * 1e12)
    roof = dict(hbm if hbm_bound else mfma, bound="hbm" if hbm_bound else "mfma")
    roof["note"] += "; the call time includes the forward recompute"
    return {"workload": bw.fwd.name, "tokens": tokens, "call_ms": kern, "wall_ms": wall,
            "value": tokens / (kern * 1e-3), "unit": "tokens/s",
            "workspace_bytes": ws.numel(),
            "flops_per_token": F, "achieved_tflops": tf,
            "roofline": roof, "mfma": mfma, "hbm": hbm}


def profile_run():
    """3 prefill launches, 3 decode launches (cache flushed before each) and a copy probe."""
    import torch
    from __graft_entry__ import _ensure_built
    _ensure_built()
    import gated_delta_rule_71_amd as gdr
    from gated_delta_rule_71_amd import workloads as W
    wl2 = W.config2()
    run_prefill_leg(wl2, 3, 0)
    wl3 = W.config3()
    d = [up(x) for x in (wl3.q, wl3.k, wl3.v, wl3.g, wl3.beta)]
    cache, idx = up(wl3.cache), up(wl3.batch_indices)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    for _ in range(3):
        flush.sum()
        gdr.ssm_decode(*d, cache, batch_indices=idx)
    src = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    dst.copy_(src)
    torch.cuda.synchronize()
    print("profile run done", file=sys.stderr)


def main():
    args = parse()
    if args.summarize_db:
        summarize_db(args.summarize_db)
        return
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.mfma_from:
        mfma_from(args.mfma_from)
        return
    if args.lds_from:
        lds_from(args.lds_from)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    from __graft_entry__ import _ensure_built
    _ensure_built()
    import gated_delta_rule_71_amd as gdr
    from gated_delta_rule_71_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.profile_run:
        profile_run()
        return
    legs = set(args.legs.split(","))
    res = {}
    t_start = time.perf_counter()

    # ---- headline: packed varlen prefill, Hv = 32 ----------------------------------
    wl2 = W.config2()
    tokens2 = wl2.tokens
    print(f"[bench] prefill workload {wl2.name}: {tokens2} tokens, lengths "
          f"{wl2.meta['lengths']}", file=sys.stderr, flush=True)
    if "prefill" in legs:
        wall, kern = run_prefill_leg(wl2, args.steps, args.warmup)
        byt = prefill_bytes(wl2)
        F = prefill_flops_per_token(wl2, wl2.chunk_size)
        res["prefill"] = dict(wall_ms=wall, kernel_ms=kern, tokens=tokens2, bytes=byt,
                              flops=F * tokens2, flops_per_token=F)
        print(f"[bench] prefill: {wall:.3f} ms/step, kernel {kern:.3f} ms", file=sys.stderr,
              flush=True)

    # ---- batched prefill, B = 4, T = 4096, H = 16 --------------------------------------
    if "prefill_b4" in legs:
        wl1 = W.config1()
        wall, kern = run_prefill_leg(wl1, args.steps, args.warmup)
        byt = prefill_bytes(wl1)
        F = prefill_flops_per_token(wl1, wl1.chunk_size)
        res["prefill_b4"] = dict(wall_ms=wall, kernel_ms=kern, tokens=wl1.tokens, bytes=byt,
                                 flops=F * wl1.tokens, flops_per_token=F, workload=wl1.name)
        print(f"[bench] prefill B4 T4096 H16: kernel {kern:.3f} ms", file=sys.stderr,
              flush=True)
        del wl1

    # ---- decode ------------------------------------------------------------------------
    if "decode" in legs:
        wl3 = W.config3()
        wall, kern = run_decode_leg(wl3, args.steps, args.warmup)
        n_real = int((wl3.batch_indices >= 0).sum())
        Hv, K, V = wl3.cache.shape[1:]
        state_bytes = 2 * n_real * Hv * K * V * 4
        res["decode"] = dict(wall_ms=wall, kernel_ms=kern, state_bytes=state_bytes,
                             workload=wl3.name, n_real=n_real)
        print(f"[bench] decode: kernel {kern:.4f} ms", file=sys.stderr, flush=True)

    # ---- gated delta product, long context ----------------------------------------------
    if "gdp" in legs:
        wl4 = W.config4()
        wall, kern = run_prefill_leg(wl4, max(2, args.steps // 4), min(args.warmup, 2))
        _, kern1 = run_prefill_leg(wl4, 2, 1, segments=False)
        byt = prefill_bytes(wl4)
        F = prefill_flops_per_token(wl4, wl4.chunk_size)
        res["gdp"] = dict(wall_ms=wall, kernel_ms=kern, tokens=wl4.tokens, bytes=byt,
                          flops=F * wl4.tokens, flops_per_token=F, workload=wl4.name,
                          single_pass_ms=kern1)
        print(f"[bench] gdp: kernel {kern:.3f} ms", file=sys.stderr, flush=True)
        del wl4

    # ---- one long packed request (segments planned on the device) ----------------------
    if "long_packed" in legs:
        wl5 = W.long_packed()
        wall, kern = run_prefill_leg(wl5, max(2, args.steps // 4), min(args.warmup, 2))
        _, kern1 = run_prefill_leg(wl5, 2, 1, segments=False)
        res["long_packed"] = dict(wall_ms=wall, kernel_ms=kern, tokens=wl5.tokens,
                                  workload=wl5.name, single_pass_ms=kern1)
        print(f"[bench] long_packed: kernel {kern:.3f} ms (single pass {kern1:.3f} ms)",
              file=sys.stderr, flush=True)
        del wl5

    # ---- gates formed in the kernels from raw projections (same workloads) --------------
    if "gates" in legs:
        gw2 = W.with_raw_gates(wl2, 2)
        _, kp = run_prefill_leg(gw2, args.steps, args.warmup)
        gw3 = W.with_raw_gates(W.config3(), 3)
        _, kd = run_decode_leg(gw3, args.steps, args.warmup)
        res["gates"] = {"prefill_kernel_ms": kp, "decode_kernel_ms": kd,
                        "note": "packed prefill and decode workloads with g, beta formed in "
                                "the kernels from raw projections (A_log, dt_bias)"}
        if "prefill" in res:
            res["gates"]["prefill_vs_formed"] = kp / res["prefill"]["kernel_ms"]
        if "decode" in res:
            res["gates"]["decode_vs_formed"] = kd / res["decode"]["kernel_ms"]
        print(f"[bench] fused gates: prefill {kp:.3f} ms, decode {kd:.4f} ms", file=sys.stderr,
              flush=True)
        del gw2, gw3

    # ---- short causal conv and gated RMS norm around the recurrence -------------------
    if "conv_norm" in legs:
        res["conv_norm"] = run_conv_norm_leg(wl2, args.steps, args.warmup)
        print(f"[bench] conv/norm: {res['conv_norm']}", file=sys.stderr, flush=True)

    # ---- boundary states (prefix caching) on the packed prefill ------------------------
    if "boundary" in legs:
        res["boundary"] = {"note": "packed prefill also writing each sequence's state every "
                                   "`interval` tokens; bytes = entries x Hv x K x V x 4"}
        for iv in (1024, 64):
            _, kb = run_prefill_leg(wl2, args.steps, args.warmup, boundary_interval=iv)
            E = sum(int(L) // iv for L in np.diff(wl2.cu_seqlens))
            nbytes_b = E * int(np.prod(wl2.initial_state.shape[1:])) * 4
            entry = {"kernel_ms": kb, "entries": E, "bytes": nbytes_b}
            if "prefill" in res:
                entry["vs_without"] = kb / res["prefill"]["kernel_ms"]
            res["boundary"][f"interval_{iv}"] = entry
            print(f"[bench] boundary states every {iv}: {kb:.3f} ms ({E} entries)",
                  file=sys.stderr, flush=True)

    # ---- chunked backward at the batched training shape ------------------------------
    if "backward" in legs:
        res["backward"] = run_backward_leg(max(2, args.steps // 4), min(args.warmup, 2))
        print(f"[bench] backward: {res['backward']['call_ms']:.3f} ms per call",
              file=sys.stderr, flush=True)
        res["backward"]["gated_delta_product"] = run_backward_leg(
            2, 1, name="bwd_gdp2_bf16_B1_T16384_H32_D128", B=1, T=16384, H=32, n_h=2)
        print(f"[bench] backward (product): "
              f"{res['backward']['gated_delta_product']['call_ms']:.3f} ms per call",
              file=sys.stderr, flush=True)

    # ---- CPU baseline: the oracle on a bounded sample of the prefill workload ------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from gated_delta_rule_71_amd.workloads import as_f64
        Hv = wl2.v.shape[-2]
        Hk = wl2.q.shape[-2]
        nh = min(args.cpu_heads, Hv)
        heads = list(range(0, nh))
        kh = sorted(set(h * Hk // Hv for h in heads))
        sel_k = {hk: i for i, hk in enumerate(kh)}
        q = as_f64(wl2.q[:, :, kh])
        k = as_f64(wl2.k[:, :, kh])
        v = as_f64(wl2.v[:, :, heads])
        g = wl2.g[:, :, heads].astype(np.float64)
        beta = wl2.beta[:, :, heads].astype(np.float64)
        cache = as_f64(wl2.initial_state[:, heads]).copy()
        # grouping is preserved: the selected v heads map onto the selected k heads
        assert all(sel_k[h * Hk // Hv] == h * len(kh) // nh for h in heads)
        threads = oracle.threads_used(0)
        reps, dt = 0, 0.0
        while reps == 0 or dt < args.cpu_seconds:
            state = cache.copy()
            t0 = time.perf_counter()
            oracle.prefill(q, k, v, g, beta, cu_seqlens=wl2.cu_seqlens, initial_state=state,
                           state_indices=wl2.state_indices, final_state_out=state,
                           threads=threads)
            dt += time.perf_counter() - t0
            reps += 1
        cpu = dict(value=reps * tokens2 * nh / Hv / dt, unit="tokens/s", cores=threads,
                   kind="oracle",
                   sample=f"{wl2.name}: all {tokens2} tokens of the 8 sequences, {nh} of "
                          f"{Hv} value heads, {reps} passes ({dt:.1f} s)"
                          + ("" if nh == Hv else ", scaled to all heads"))
        print(f"[bench] cpu oracle: {dt:.1f} s on {threads} threads", file=sys.stderr,
              flush=True)

    # ---- report -----------------------------------------------------------------------
    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16/f32", "data": "synthetic"}
    if "prefill" in res:
        p = res["prefill"]
        tps = p["tokens"] / (p["wall_ms"] * 1e-3)
        achieved = p["bytes"] / (p["kernel_ms"] * 1e-3) / 1e9
        line.update(value=tps, unit="tokens/s", ms_per_step=p["wall_ms"])
        line["config"] = {
            "workload": wl2.name, "tokens": p["tokens"], "seq_lens": wl2.meta["lengths"],
            "num_qk_heads": int(wl2.q.shape[2]), "num_v_heads": int(wl2.v.shape[-2]),
            "head_k": 128, "head_v": 128, "chunk_size": wl2.chunk_size, "qkv": "bf16",
            "state": "fp32 slot cache", "parallelism": "single GPU"}
        line["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                            "traffic": stored_traffic("prefill_varlen", "prefill64.hip"),
                            "kernel": "prefill64_kernel", "bytes_per_launch": p["bytes"],
                            "kernel_ms": p["kernel_ms"]}
        tf = p["flops"] / (p["kernel_ms"] * 1e-3) / 1e12
        line["mfma"] = {"flops_per_token": p["flops_per_token"], "achieved_tflops": tf,
                        "peak_tflops": MFMA_PEAK_TFLOPS, "frac": tf / MFMA_PEAK_TFLOPS}
    if "decode" in res:
        dd = res["decode"]
        gbs = dd["state_bytes"] / (dd["kernel_ms"] * 1e-3) / 1e9
        line["decode"] = {"workload": dd["workload"], "value": gbs, "unit": "GB/s",
                          "kernel_ms": dd["kernel_ms"], "state_bytes": dd["state_bytes"],
                          "real_requests": dd["n_real"],
                          "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                       "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                       "traffic": stored_traffic("decode", "decode.hip")}}
        if "prefill" not in res:
            line.update(value=gbs, unit="GB/s", ms_per_step=dd["wall_ms"])
    if "prefill_b4" in res:
        pb = res["prefill_b4"]
        gbs = pb["bytes"] / (pb["kernel_ms"] * 1e-3) / 1e9
        tf = pb["flops"] / (pb["kernel_ms"] * 1e-3) / 1e12
        line["prefill_b4"] = {
            "workload": pb["workload"], "value": pb["tokens"] / (pb["wall_ms"] * 1e-3),
            "unit": "tokens/s", "kernel_ms": pb["kernel_ms"], "tokens": pb["tokens"],
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": pb["bytes"]},
            "mfma": {"flops_per_token": pb["flops_per_token"], "achieved_tflops": tf,
                     "peak_tflops": MFMA_PEAK_TFLOPS, "frac": tf / MFMA_PEAK_TFLOPS}}
    if "gdp" in res:
        gg = res["gdp"]
        tps = gg["tokens"] / (gg["wall_ms"] * 1e-3)
        gbs = gg["bytes"] / (gg["kernel_ms"] * 1e-3) / 1e9
        tf = gg["flops"] / (gg["kernel_ms"] * 1e-3) / 1e12
        # the product's arithmetic intensity (~444 flop/B) is past the ridge (~315):
        # its roofline is the matrix cores'
        line["gdp"] = {"workload": gg["workload"], "value": tps, "unit": "tokens/s",
                       "kernel_ms": gg["kernel_ms"], "single_pass_ms": gg["single_pass_ms"],
                       "note": "in 8 segments of 8192 tokens: three chunked passes and a "
                               "state combine; single_pass_ms is the one-pass kernel",
                       "roofline": {"bound": "mfma", "achieved": tf,
                                    "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                    "frac": tf / MFMA_PEAK_TFLOPS,
                                    "flops_per_token": gg["flops_per_token"]},
                       "hbm": {"achieved_gbs": gbs, "frac": gbs / HBM_PEAK_GBS}}
    if "long_packed" in res:
        lp = res["long_packed"]
        line["long_packed"] = {"workload": lp["workload"],
                               "value": lp["tokens"] / (lp["wall_ms"] * 1e-3),
                               "unit": "tokens/s", "kernel_ms": lp["kernel_ms"],
                               "single_pass_ms": lp["single_pass_ms"],
                               "note": "8 segment slots planned on the device: three "
                                       "chunked passes and a state combine"}
    if "gates" in res:
        line["fused_gates"] = res["gates"]
    if "boundary" in res:
        line["boundary_states"] = res["boundary"]
    if "conv_norm" in res:
        line["conv_norm"] = res["conv_norm"]
    if "backward" in res:
        line["backward"] = res["backward"]
    if cpu is not None:
        line["cpu_baseline"] = cpu
    line["bench_wall_s"] = time.perf_counter() - t_start
    print(json.dumps(line))


if __name__ == "__main__":
    main()
