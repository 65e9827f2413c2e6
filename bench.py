"""Throughput of causal softmax attention fwd + bwd on one MI355X.

One step = one forward and one backward pass (upstream gradient dO = O, the
loss sum(o^2)/2) over the bfloat16 workload of 8 x 32 heads x 4096 tokens,
D = 64, inputs resident in HBM before the timed region.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--no-secondary] [--steps-before-only] [--copy-calibration]

value: algorithmic TFLOP/s of the whole step.  Algorithmic work counts only the
N(N+1)/2 pairs (i, j <= i) of each head: 4 D flops per pair in the forward
(Q K^T and P V) and 10 D in the backward (Q K^T recomputed, dO V^T, P^T dO,
dS^T Q, dS K), 14 D = 896 flops per pair in all.

roofline: the kernel with the largest share of the step (picked in the warm-up
steps), timed live in the timed steps with HIP events on the library's stream
(the timer hook of the C ABI; only that kernel carries events there), against the
bf16 dense MFMA peak of MI355X (2516.6 TFLOP/s).  traffic: HBM bytes per
launch from rocprofv3's L2-to-memory request counters by size class
(32 RDREQ_32B + 64 RDREQ_64B + 128 RDREQ_128B read, 32 (WRREQ - WRREQ_64B)
+ 64 WRREQ_64B written) recorded in profiles/traffic.json, reported only
while the kernel's source is unchanged since they were taken.

cpu_baseline: the float64 oracle (test infrastructure, never tuned) on a
bounded sample of whole heads of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK = 2516.6       # TFLOP/s, MI355X dense bf16 MFMA
F32_PEAK = 157.3         # TFLOP/s, MI355X fp32 MFMA
HBM_PEAK = 8000.0        # GB/s
D = 64
METRIC = "causal attn fwd+bwd TFLOP/s at N=4096 D=64 bf16; % of MFMA peak"

# Algorithmic flops per pair (i, j <= i) credited to each timed kernel: the
# method's five backward products are S, dP = dO V^T, dV = P^T dO, dK = dS^T Q
# and dQ = dS K (10 D), the forward's two S and P V (4 D).  The dK/dV pass
# forms the first four; the dQ pass is credited with dQ alone (2 D): its own
# recomputation of S and dP is work the method does not need.  The credits sum
# to the 14 D of the headline.
KERNEL_FLOPS_PER_PAIR = {"fwd": 4 * D, "bwd_dkdv": 8 * D, "bwd_dq": 2 * D, "bwd_pre": 0}
COPY_BYTES = 256 << 20   # the plain device copy used to calibrate HBM byte counters


def pairs(heads: int, n: int) -> int:
    return heads * n * (n + 1) // 2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "causal_softmax_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(slot: str):
    """HBM bytes per launch of `slot` from profiles/traffic.json: the
    kernel's L2-to-memory read and write requests, each weighted by its size
    class (a plain 256 MiB copy checks the sums).  None unless the kernel's
    sources still hash as they did when the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(slot)
    if not rec:
        return None
    if rec.get("source_sha") != source_sha(rec["sources"]):
        return None
    return rec["bytes_per_launch"]


def make_inputs(name):
    import numpy as np
    import torch

    import causal_softmax_attention_amd.inputs as inp
    a = inp.workload(name)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}[a.dtype]

    def dev(x):
        if a.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        return torch.from_numpy(x).to("cuda:0")
    return a, [dev(getattr(a, x)) for x in "qkv"], dt


def time_attention(q, k, v, steps, warmup, with_bwd=True, per_kernel=True, mask="causal",
                   window=0, fused=False, seg=None, only=None):
    """Run `steps` timed steps; returns (mean ms per step, wall ms per step,
    {slot: mean ms}, outputs, sorted per-step ms).
    The causal predicate goes through attn_causal_fwd / _bwd, others through
    attn_fwd / attn_bwd, segment ids (seg) through attn_fwd_seg / _bwd_seg;
    fused: attn_fwd_train (forward + loss + the backward's per-row values) and
    attn_bwd_from_fwd."""
    import torch

    import causal_softmax_attention_amd as csa
    B, H, N, _ = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32 if q.dtype != torch.float64 else torch.float64,
                      device=q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    code = {torch.bfloat16: csa.ATTN_BF16, torch.float32: csa.ATTN_F32,
            torch.float64: csa.ATTN_F64}[q.dtype]
    ws = torch.empty(max(16, csa.attn_causal_bwd_workspace_bytes(code, B, H, N, D)),
                     dtype=torch.uint8, device=q.device)

    loss = torch.empty(1, dtype=torch.float64, device=q.device)

    def step():
        if seg is not None:
            csa.attn_fwd_seg(q, k, v, seg, 0.125, mask, window, o=o, lse=lse)
            if with_bwd:
                csa.attn_bwd_seg(q, k, v, o, o, lse, seg, 0.125, mask, window, dq=dq, dk=dk,
                                 dv=dv, workspace=ws)
        elif fused:
            csa.attn_fwd_train(q, k, v, 0.125, mask, window, o=o, lse=lse, workspace=ws, loss=loss)
            csa.attn_bwd_from_fwd(q, k, v, o, lse, ws, 0.125, mask, window, dq=dq, dk=dk, dv=dv)
        elif mask == "causal":
            csa.attn_causal_fwd(q, k, v, 0.125, o=o, lse=lse)
            if with_bwd:
                csa.attn_causal_bwd(q, k, v, o, o, lse, 0.125, dq=dq, dk=dk, dv=dv, workspace=ws)
        else:
            csa.attn_fwd(q, k, v, 0.125, mask, window, o=o, lse=lse)
            if with_bwd:
                csa.attn_bwd(q, k, v, o, o, lse, 0.125, mask, window, dq=dq, dk=dk, dv=dv,
                             workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    slots = [csa.TIMER_FWD] + ([csa.TIMER_BWD_DKDV, csa.TIMER_BWD_DQ] if fused else
                               [csa.TIMER_BWD_PRE, csa.TIMER_BWD_DKDV, csa.TIMER_BWD_DQ]
                               if with_bwd else [])
    if only is not None:  # time only these kernels (fewer events in the stream)
        slots = [s_ for s_ in slots if s_ in only]
    events = []
    if per_kernel:
        for _ in range(steps):
            ev = {}
            for s in slots:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(); b.record()            # materialise the HIP events
                ev[s] = (a, b)
            events.append(ev)
        torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        if per_kernel:
            for s in slots:
                csa.attn_set_kernel_timer(s, *events[i][s])
        marks[i].record()
        step()
    marks[steps].record()
    stop.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    for s in slots:
        csa.attn_set_kernel_timer(s, None, None)
    ms = start.elapsed_time(stop) / steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    per = {}
    if per_kernel:
        for s in slots:
            per[csa.TIMER_NAMES[s]] = sum(e[s][0].elapsed_time(e[s][1]) for e in events) / steps
    return ms, wall, per, (o, lse), per_step


def time_alternating(q, k, v, variants, rounds, steps):
    """Time several step variants (name -> time_attention keywords) in
    alternating rounds of `steps` steps each, so that clock and temperature
    drift reach every variant alike.  Returns {name: (median ms over rounds,
    per-kernel ms of the last round)}."""
    import statistics
    got = {name: [] for name in variants}
    per_last = {}
    for _ in range(rounds):
        for name, kw in variants.items():
            ms, _, per, _, _ = time_attention(q, k, v, steps, 1, **kw)
            got[name].append(ms)
            per_last[name] = per
    return {name: (statistics.median(v_), per_last[name]) for name, v_ in got.items()}


def _blas_vendor() -> str:
    import numpy as np
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:  # noqa: BLE001
        return "unknown"


def cpu_baseline(a, budget_s=10.0):
    """The oracle (as it stands) on whole heads of the workload until ~budget_s
    of wall time: its [B, H, N, D] wrappers with their thread pool over heads,
    one worker per core of this process's CPU share, one BLAS thread each."""
    import numpy as np

    import causal_softmax_attention_amd.inputs as inp
    import oracle
    cores = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    if share and share.isdigit() and int(share) > 0:
        cores = min(cores, int(share))
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except Exception:  # noqa: BLE001
        limit = contextlib.nullcontext()
    B, H, N = a.q.shape[:3]
    flat = [(b, h) for b in range(B) for h in range(H)]
    done, t0 = 0, time.perf_counter()
    with limit:
        while done < len(flat):
            batch = flat[done:done + cores]
            def f64(name):
                x = getattr(a, name)
                sel = np.stack([x[b, h] for b, h in batch])[None]
                return inp.bf16_bits_to_f32(sel).astype(np.float64)
            q, k, v = f64("q"), f64("k"), f64("v")
            oracle.forward(q, k, v, 0.125, workers=cores)
            oracle.backward(q, k, v, None, 0.125, workers=cores)
            done += len(batch)
            if time.perf_counter() - t0 >= budget_s:
                break
    el = time.perf_counter() - t0
    flops = 14 * D * pairs(done, N)
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {B * H} heads (N={N}), float64 fwd + bwd, {el:.1f} s wall; "
                      f"a pool of {cores} threads over heads (os.sched_getaffinity within the "
                      f"process's OMP_NUM_THREADS share), 1 BLAS thread each",
            "blas": _blas_vendor()}


class SclkSampler:
    """Samples the GPU's graphics clock (MHz) from a background thread while
    the timed region runs, through the amdsmi Python module: the current GFX
    clock (amdsmi_get_clock_info) and, where the GPU metrics table has them,
    the per-XCD current gfx clocks.  The first raw reading is kept, so the
    record shows which fields the clock came from."""

    def __init__(self, period_s=0.002):
        import threading
        self.samples, self.xcd_samples, self.error, self.raw = [], [], None, {}
        self._stop = threading.Event()
        self._period = period_s
        self._ok = False
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            c = amdsmi.amdsmi_get_clock_info(self._h, amdsmi.AmdSmiClkType.GFX)
            self.raw["clock_info_gfx"] = {k: c[k] for k in c}
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(self._h)
                self.raw["gpu_metrics"] = {k: m[k] for k in m
                                           if "gfxclk" in k or "clk" in k.lower()}
            except Exception as e:  # noqa: BLE001
                self.raw["gpu_metrics"] = str(e)
            self._ok = True
        except Exception as e:  # noqa: BLE001
            self.error = f"amdsmi: {e}"
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        am, h = self._amdsmi, self._h
        while not self._stop.is_set():
            try:
                c = am.amdsmi_get_clock_info(h, am.AmdSmiClkType.GFX)
                self.samples.append(float(c["clk"]))
                m = am.amdsmi_get_gpu_metrics_info(h)
                xs = m.get("current_gfxclks")
                if isinstance(xs, (list, tuple)):
                    xs = [x for x in xs if isinstance(x, (int, float)) and 0 < x < 10000]
                    if xs:
                        self.xcd_samples.append(sum(xs) / len(xs))
            except Exception as e:  # noqa: BLE001
                self.error = str(e)
                return
            self._stop.wait(self._period)

    def __enter__(self):
        if self._ok:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        # The driver refreshes these readings only every few hundred ms, so the
        # first readings of a window can still show the idle clock from
        # before the load: statistics are taken from the first reading that
        # differs from the window's first one (all readings if none does).
        def stats(v):
            if not v:
                return None
            first_change = next((i for i, x in enumerate(v) if x != v[0]), 0)
            w = sorted(v[first_change:])
            return {"median": w[len(w) // 2], "min": w[0], "max": w[-1], "samples": len(w),
                    "stale_leading_samples": first_change, "leading_value": v[0]}
        return {"gfx_clock_info_mhz": stats(self.samples),
                "gpu_metrics_current_gfxclks_mean_mhz": stats(self.xcd_samples),
                "raw_first_reading": self.raw, "error": self.error}


def secondary(steps):
    """Other workloads: fp32 forward, long-sequence bf16 fwd+bwd, other join
    predicates, fp64 latency, the NW control, and the steps before the path."""
    import numpy as np
    import torch

    import causal_softmax_attention_amd as csa
    import causal_softmax_attention_amd.inputs as inp
    out = {}
    a, (q, k, v), _ = make_inputs("fp32_2k")
    ms, _, per, _, _ = time_attention(q, k, v, steps, 2, with_bwd=False)
    fl = 4 * D * pairs(64, 2048)
    out["fp32_2k_fwd"] = {"ms": ms, "TFLOP/s": fl / ms / 1e9,
                          "frac_of_fp32_mfma_peak": fl / ms / 1e9 / F32_PEAK}
    del q, k, v
    a, (q, k, v), _ = make_inputs("bf16_32k")
    ms, _, per, _, _ = time_attention(q, k, v, max(2, steps // 4), 1)
    fl = 14 * D * pairs(16, 32768)
    out["bf16_32k_fwd_bwd"] = {"ms": ms, "TFLOP/s": fl / ms / 1e9,
                               "frac_of_bf16_peak": fl / ms / 1e9 / BF16_PEAK,
                               "kernels_ms": per}
    del q, k, v
    # the same step with the loss fused into the forward (attn_fwd_train +
    # attn_bwd_from_fwd): the backward's per-row pass is folded away.  Timed in
    # alternating rounds with the unfused step, so both see the same clock.
    a, (q, k, v), _ = make_inputs("bf16_4k")
    alt = time_alternating(q, k, v, {"unfused": {}, "fused": {"fused": True}}, 6,
                           max(3, steps // 2))
    ms, per = alt["fused"]
    fl = 14 * D * pairs(256, 4096)
    out["bf16_4k_train_step_fused_loss"] = {"ms": ms, "TFLOP/s": fl / ms / 1e9,
                                            "frac_of_bf16_peak": fl / ms / 1e9 / BF16_PEAK,
                                            "unfused_ms_same_rounds": alt["unfused"][0],
                                            "fused_over_unfused": ms / alt["unfused"][0],
                                            "timing": "medians over 6 alternating rounds",
                                            "kernels_ms": per}
    del q, k, v
    # the other join predicates on the same 8 x 32 x 4096 bf16 inputs; flops
    # count each predicate's own pairs (N^2 per head for the full one)
    a, (q, k, v), _ = make_inputs("bf16_4k")
    B_, H_, N_ = q.shape[:3]
    for mask, window, key in (("full", 0, "bf16_4k_full_fwd_bwd"),
                              ("window", 512, "bf16_4k_window512_fwd_bwd")):
        ms, _, per, _, _ = time_attention(q, k, v, max(2, steps // 2), 1, mask=mask, window=window)
        npairs = B_ * H_ * (N_ * N_ if mask == "full" else
                            sum(min(i + 1, window) for i in range(N_)))
        fl = 14 * D * npairs
        out[key] = {"ms": ms, "TFLOP/s": fl / ms / 1e9, "frac_of_bf16_peak": fl / ms / 1e9 / BF16_PEAK,
                    "pairs": npairs, "kernels_ms": per}
    # segment ids on the same inputs (causal): packed documents of mean 512
    # tokens, and two interleaved ids per row (every tile masked); flops count
    # the pairs that exist
    for kind, key in (("packed", "bf16_4k_segments_packed512_fwd_bwd"),
                      ("interleaved", "bf16_4k_segments_interleaved2_fwd_bwd")):
        seg = inp.segment_ids(45, B_, N_, kind, mean_len=512, n_ids=2)
        i = np.arange(N_)
        npairs = H_ * int(sum(((sg[None, :] == sg[:, None]) & (i[None, :] <= i[:, None])).sum()
                              for sg in seg))
        sd = torch.from_numpy(seg).to(q.device)
        ms, _, per, _, _ = time_attention(q, k, v, max(2, steps // 2), 1, seg=sd)
        fl = 14 * D * npairs
        out[key] = {"ms": ms, "TFLOP/s": fl / ms / 1e9, "frac_of_bf16_peak": fl / ms / 1e9 / BF16_PEAK,
                    "pairs": npairs, "kernels_ms": per}
    del q, k, v
    a, (q, k, v), _ = make_inputs("fp64_256")
    ms, _, per, _, _ = time_attention(q, k, v, steps, 2)
    out["fp64_256_fwd_bwd"] = {"us": ms * 1e3, "kernels_us": {k_: v_ * 1e3 for k_, v_ in per.items()}}
    nw = inp.nw_inputs()
    cols = [torch.from_numpy(x).to("cuda:0") for x in (nw.tx, nw.ty, nw.sx, nw.sy, nw.sv)]
    res = torch.empty_like(cols[0])
    for _ in range(2):
        csa.nw_gauss_average(*cols, 0.25, out=res)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        csa.nw_gauss_average(*cols, 0.25, out=res)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    # ALU bound: a wave64 VALU op holds its SIMD 4 cycles (16 lanes/clock) and
    # v_exp_f32 8 (transcendentals at half rate, issued like any VALU op); 7 ops
    # and 1 exp per pair make 36 cycles per 64 pairs: 256 CUs x 4 SIMDs x 64 x
    # 2.4 GHz / 36
    nw_bound = 256 * 4 * 64 * 2.4e9 / (7 * 4 + 8) / 1e9
    out["nw_64k"] = {"ms": ms, "Gpairs/s": 65536.0 ** 2 / ms / 1e6,
                     "alu_bound_Gpairs/s": nw_bound,
                     "frac_of_alu_bound": 65536.0 ** 2 / ms / 1e6 / nw_bound}
    del cols, res
    out.update(steps_before_the_path(steps))
    return out


def _mean_ms(call, steps, warmup=2):
    """Mean wall time of one call on the current stream, HIP events around `steps` calls."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        call()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def steps_before_the_path(steps):
    """The fused Q/K/V projection producing the bf16_4k inputs, and the long-table
    adapter on a 2^25-row bf16 table (16 heads of 32768 tokens)."""
    import numpy as np
    import torch

    import causal_softmax_attention_amd as csa
    import causal_softmax_attention_amd.inputs as inp
    dev = "cuda:0"
    bits = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    out = {}
    _, B_, N_, Dm_, H_, _ = inp.PROJECTION_WORKLOADS["proj_4k"]
    pa = inp.projection_workload("proj_4k")
    xw = [bits(getattr(pa, n)) for n in ("x", "wq", "wk", "wv")]
    qkv = [torch.empty((B_, H_, N_, D), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    ms = _mean_ms(lambda: csa.attn_qkv_project(*xw, H_, *qkv), steps)
    fl = 3 * 2 * B_ * N_ * Dm_ * H_ * D
    out["qkv_project_4k"] = {"ms": ms, "TFLOP/s": fl / ms / 1e9,
                             "frac_of_bf16_peak": fl / ms / 1e9 / BF16_PEAK,
                             "shape": f"x [{B_}, {N_}, {Dm_}] -> q, k, v [{B_}, {H_}, {N_}, 64]"}
    del xw, qkv, pa
    seed, T_, D2, _ = inp.TABLE_WORKLOADS["table_16x32k"]
    m, perm = inp.table_matrix(seed, T_, D2, "bf16")
    md = bits(m)
    t, d, x = csa.attn_matrix_to_table(md)
    p = torch.from_numpy(perm).to(dev)
    ts, ds, xs = t[p], d[p], x[p]
    del p
    mat = torch.empty_like(md)
    ws = torch.empty(csa.attn_table_workspace_bytes(csa.ATTN_BF16, T_, D2), dtype=torch.uint8,
                     device=dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    ms = _mean_ms(lambda: csa.attn_table_to_matrix(ts, ds, xs, T_, D2, m=mat, workspace=ws,
                                                   status=st, check=False), steps)
    cells = T_ * D2
    algo = cells * (8 + 8 + 2) + cells * 2          # read t, d, x; write the matrix
    out["table_to_matrix_16x32k"] = {"ms": ms, "Mrows/s": cells / ms / 1e3,
                                     "GB/s": algo / ms / 1e6,
                                     "frac_of_hbm": algo / ms / 1e6 / HBM_PEAK,
                                     "algorithmic_bytes": algo,
                                     "status": int(st.item())}
    # the same rows in (t, d) order, as the forward's ORDER BY t, d returns them
    ms = _mean_ms(lambda: csa.attn_table_to_matrix(t, d, x, T_, D2, m=mat, workspace=ws,
                                                   status=st, check=False), steps)
    out["table_to_matrix_16x32k_ordered"] = {"ms": ms, "GB/s": algo / ms / 1e6,
                                             "frac_of_hbm": algo / ms / 1e6 / HBM_PEAK,
                                             "status": int(st.item())}
    ms = _mean_ms(lambda: csa.attn_matrix_to_table(md, t=t, d=d, x=x), steps)
    algo = cells * 2 + cells * (8 + 8 + 2)          # read the matrix; write t, d, x
    out["matrix_to_table_16x32k"] = {"ms": ms, "GB/s": algo / ms / 1e6,
                                     "frac_of_hbm": algo / ms / 1e6 / HBM_PEAK,
                                     "algorithmic_bytes": algo}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--steps-before-only", action="store_true",
                    help="time only the Q/K/V projection and the long-table adapter (one JSON "
                         "line of those); for profiling their kernels")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock-sampling steps after the timed ones (no amdsmi thread; "
                         "for rocprofv3 counter runs, which need only the kernels' dispatches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy (3x), the known-size check "
                         "of the byte counts derived from rocprofv3 request counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this library has no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import causal_softmax_attention_amd as csa
    if not os.path.exists(csa.LIB_PATH):
        from causal_softmax_attention_amd import _build
        _build.build()
    csa.lib()
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.steps_before_only:
        print(json.dumps({"steps_before_the_path": steps_before_the_path(args.steps)}))
        return
    log("generating bf16_4k inputs")
    a, (q, k, v), _ = make_inputs("bf16_4k")
    B, H, N = q.shape[:3]
    log(f"timing {args.steps} steps after {args.warmup} warmup")
    algo = KERNEL_FLOPS_PER_PAIR
    # The warm-up steps carry a HIP event pair around every kernel and pick
    # the one with the largest share; the timed steps then carry events around
    # that kernel only (the roofline's live figure).  Events around all four
    # kernels cost about 1.3 % of the step, one pair about nothing.
    dom = "bwd_dkdv"
    if args.warmup > 0:
        warm_per = time_attention(q, k, v, args.warmup, 0)[2]
        dom = max((s for s in warm_per if algo.get(s)), key=lambda s: warm_per[s])
    slot = {name: s_ for s_, name in csa.TIMER_NAMES.items()}[dom]
    ms, wall, per, _, per_step = time_attention(q, k, v, args.steps, 0, only=[slot])
    # the GPU's clock readings refresh more slowly than the ~55 ms timed region,
    # so the clock is sampled over about 2.5 s of the same step right after it,
    # with every kernel timed (the per-kernel breakdown of the record)
    if args.no_clock:
        sclk = {"skipped": "--no-clock"}
        sus_per = per
    else:
        sustain = max(50, int(2500.0 / ms))
        log(f"sampling the graphics clock over {sustain} more steps")
        with SclkSampler(period_s=0.01) as clk:
            sus_ms, _, sus_per, _, _ = time_attention(q, k, v, sustain, 0)
        sclk = clk.summary()
        sclk["window"] = (f"{sustain} steps of the same fwd+bwd ({sustain * sus_ms / 1e3:.2f} s) "
                          "run right after the timed steps, every kernel timed")
        sclk["ms_per_step_over_window"] = round(sus_ms, 4)
    flops = 14 * D * pairs(B * H, N)
    value = flops / ms / 1e9
    kflops = algo[dom] * pairs(B * H, N)
    achieved = kflops / per[dom] / 1e9
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK,
            "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK, 4),
            "traffic": traffic_for(dom), "kernel_ms": round(per[dom], 4),
            "algorithmic_flops_per_launch": kflops}
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v; no dataset)",
        "config": {"workload": "bf16_4k: causal attention fwd+bwd, B=8 H=32 N=4096 D=64, "
                               "scale 1/8, dO = O", "global_batch": B, "heads": H, "seq_len": N,
                   "head_dim": D, "parallelism": "none (1 GPU)"},
        "frac_of_bf16_mfma_peak": round(value / BF16_PEAK, 4),
        "wall_ms_per_step": round(wall, 4),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 4),
        "ms_per_step_min": round(per_step[0], 4),
        "TFLOP/s_at_median": round(flops / per_step[len(per_step) // 2] / 1e9, 2),
        "sclk_mhz": sclk,
        "kernels_ms": {k_: round(v_, 4) for k_, v_ in sus_per.items()},
        "kernels_ms_window": "the clock-sampling steps after the timed ones (roofline.kernel_ms "
                             "is the timed steps' own)",
        "roofline": roof,
    }
    del q, k, v
    torch.cuda.empty_cache()
    if not args.no_secondary:
        log("secondary workloads")
        rec["secondary"] = secondary(max(3, args.steps // 2))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        rec["cpu_baseline"] = cpu_baseline(a, args.cpu_budget)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
