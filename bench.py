"""Benchmark of the jagged flash-attention hot path on one MI355X.

One step = jfa_fwd + jfa_bwd over one synthetic batch already resident in
HBM.  Default workload: prod_bcast (broadcast Q [4, 256, 128], B = 1024
sequences with lengths U[64, 2048], bf16, non-causal).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload prod_bcast]

Useful FLOPs count visible (query, key) pairs only, no padding: 4*d per pair
and head in the forward (two GEMMs), 10*d in the backward (five GEMMs).  The
same convention reproduces the FMHA guide's printed TFLOPS
("cuTile Kernels -- FMHA Implementation", "Performance Results").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_FLOP_PER_CLK_PER_CU = 4096   # dense bf16
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E
PEAK_SCLK_GHZ = 2.4               # MI355X peak engine clock
PROFILE_DIR = os.path.join(ROOT, "profiles")


# ------------------------------------------------------------ counting ----
def visible_pairs(lengths, Lq: int, causal: bool, broadcast_q: bool, window: int = 0) -> int:
    """Number of (query, key) pairs the mask leaves visible, per head
    (window W > 0 with causal: query i sees keys i - W < j <= i)."""
    L = np.asarray(lengths, dtype=np.int64)
    if causal and window > 0:
        if broadcast_q:
            i = np.arange(Lq, dtype=np.int64)[:, None]
            hi = np.minimum(i, L[None, :] - 1)
            lo = np.maximum(i - window + 1, 0)
            return int(np.maximum(hi - lo + 1, 0).sum())
        short = np.minimum(L, window)
        return int((short * (short + 1) // 2 + (L - short) * window).sum())
    if broadcast_q:
        if not causal:
            return int(Lq * L.sum())
        # query i sees min(i + 1, L) keys
        i = np.arange(Lq, dtype=np.int64)[:, None]
        return int(np.minimum(i + 1, L[None, :]).sum())
    if causal:
        return int((L * (L + 1) // 2).sum())
    return int((L * L).sum())


def useful_flops(lengths, H: int, d: int, Lq: int, causal: bool, broadcast_q: bool, window: int = 0):
    n = visible_pairs(lengths, Lq, causal, broadcast_q, window)
    return 4 * d * H * n, 10 * d * H * n


def dq_split(B: int, H: int, Lq: int, P: int):
    """Broadcast dQ work split of the library: (query blocks of 256 rows,
    sequence chunks)."""
    n_qb = -(-Lq // 256)
    nc = max(1, min(P // (H * n_qb), B, 256))
    return n_qb, nc


def algorithmic_bytes(kernel: str, lengths, H: int, d: int, Lq: int, broadcast_q: bool, P: int,
                      H_kv: int = 0) -> int:
    """Bytes a kernel must move between HBM and the chip for one launch:
    every input element read once and every output element written once.
    With H_kv < H key / value heads the dK/dV kernel writes one fp32 slice
    per query head, which group_sum_kernel adds per group."""
    T = int(np.asarray(lengths).sum())
    B = len(lengths)
    H_kv = H_kv or H
    kv = T * H_kv * d * 2                 # one bf16 [T, H_kv, d] tensor
    rows = B * H * Lq if broadcast_q else T * H
    row_bf16 = rows * d * 2               # out / dout, bf16
    q_bytes = H * Lq * d * 2 if broadcast_q else T * H * d * 2
    if kernel == "fwd_kernel":
        return 2 * kv + q_bytes + row_bf16 + rows * 4
    if kernel == "delta_kernel":
        # O, dO, lse in; delta, lse*log2(e) and the two 16-byte row terms out
        return 2 * row_bf16 + 3 * rows * 4 + 2 * rows * 16
    if kernel == "dkdv_kernel":
        # K, V, Q, dO, the two 16-byte row terms in; dK, dV (fp32) out
        return 2 * kv + q_bytes + row_bf16 + 2 * rows * 16 + 2 * T * H * d * 4
    if kernel == "dq_kernel":
        # K, V, Q, dO, lse, delta in; dQ (self) or the fp32 partials (broadcast) out
        b = 2 * kv + q_bytes + row_bf16 + 2 * rows * 4
        if broadcast_q:
            n_qb, nc = dq_split(B, H, Lq, P)
            return b + H * n_qb * nc * 256 * d * 4
        return b + T * H * d * 4
    if kernel == "group_sum_kernel":
        return 2 * T * H * d * 4 + 2 * T * H_kv * d * 4
    if kernel == "dq_reduce":
        n_qb, nc = dq_split(B, H, Lq, P)
        return H * n_qb * nc * 256 * d * 4 + H * Lq * d * 4
    return 0


def kernel_flops(kernel: str, fwd_flops: int, bwd_flops: int, broadcast_q: bool) -> int:
    """Useful (unpadded) flops of one launch.  dK/dV: S, dP, dV, dK (4 of
    the 5 backward products); dQ: the dQ product plus S and dP recomputed."""
    if kernel == "fwd_kernel":
        return fwd_flops
    if kernel == "dkdv_kernel":
        return bwd_flops * 8 // 10
    if kernel == "dq_kernel":
        return bwd_flops * 2 // 10 + fwd_flops
    return 0


# ---------------------------------------------------------- traffic -------
def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "jagged_flashattention_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != kernel_source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# Kernel symbols behind each of the library's timing labels.
LABEL_SYMBOLS = {
    "fwd_kernel": ("fwd_kernel", "fwd_kernel_dma"),
    "delta_kernel": ("delta_kernel",),
    "delta_exact_kernel": ("delta_exact_kernel",),
    "dkdv_kernel": ("dkdv_kernel", "dkdv_pair_kernel"),
    "dq_kernel": ("dq_kernel", "dq_bcast_kernel"),
    "dq_reduce": ("dq_reduce",),
    "group_sum_kernel": ("group_sum_kernel",),
    "fwd_mx_kernel": ("fwd_mx_kernel",),
    "delta_mx_kernel": ("delta_mx_kernel",),
    "dkdv_mx_kernel": ("dkdv_mx_kernel",),
    "dq_mx_kernel": ("dq_mx_kernel",),
}
# Counter passes of the counters summary (rocprofv3 collects each pass in a
# run of its own; at most 8 SQ and 2 GRBM counters per pass).
COUNTER_PASSES = (
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
    "SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
    "SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SALU "
    "SQ_INSTS_VMEM SQ_WAVES GRBM_GUI_ACTIVE",
)
N_XCD = 8          # MI355X: GRBM_GUI_ACTIVE is summed over the 8 XCDs
SIMD_PER_CU = 4
MFMA_CYCLES = 32   # v_mfma_f32_32x32x16_bf16 on one SIMD


def kernel_base(name: str) -> str:
    """Bare function name of a rocprofv3 kernel name ("void ns::f<...>(...)" -> "f")."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("(anonymous namespace)", "")
    depth, out = 0, []
    for ch in n:  # drop template arguments and the parameter list
        if ch in "<(":
            if depth == 0 and ch == "(":
                break
            depth += 1
        elif ch in ">)":
            depth -= 1
        elif depth == 0:
            out.append(ch)
    return "".join(out).split("::")[-1].strip()


def label_of(name: str):
    base = kernel_base(name)
    for label, syms in LABEL_SYMBOLS.items():
        if base in syms:
            return label
    return None


def counter_rows(paths):
    """{label: {counter: [value per dispatch]}} and the plain copy's values."""
    import csv
    out, copy = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            name, ctr, val = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name:
                copy.setdefault(ctr, []).append(val)
                continue
            lab = label_of(name)
            if lab:
                out.setdefault(lab, {}).setdefault(ctr, []).append(val)
    return out, copy


def summarize_pmc(fetch_csv: str, write_csv: str, workload: str, copy_bytes: int, mxfp8: bool = False):
    """Write profiles/traffic_<kernel>_<workload>.txt for every timed kernel
    from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch).
    Each counter is scaled by bytes-moved / counter-reading of the plain
    device copy of copy_bytes that bench.py --copy-calibration-mib runs in
    the same process."""
    fetch, fcopy = counter_rows([fetch_csv])
    write, wcopy = counter_rows([write_csv])
    copy_fetch = sum(fcopy["FETCH_SIZE"]) * 1024.0
    copy_write = sum(wcopy["WRITE_SIZE"]) * 1024.0
    f_scale = copy_bytes / copy_fetch
    w_scale = copy_bytes / copy_write
    paths = []
    for label in sorted(set(fetch) & set(write)):
        fv = [v * 1024.0 for v in fetch[label].get("FETCH_SIZE", [])]
        wv = [v * 1024.0 for v in write[label].get("WRITE_SIZE", [])]
        if not fv or not wv:
            continue
        kf, kw = sum(fv) / len(fv), sum(wv) / len(wv)
        path = os.path.join(PROFILE_DIR, f"traffic_{label}_{workload}{'_mxfp8' if mxfp8 else ''}.txt")
        mode = " --mxfp8" if mxfp8 else ""
        with open(path, "w") as f:
            f.write(f"# HBM traffic of {label} ({', '.join(LABEL_SYMBOLS[label])}) on {workload}, "
                    "from rocprofv3 FETCH_SIZE and WRITE_SIZE\n")
            f.write("# commands (MI355X; one counter per run):\n")
            for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                f.write(f"#   cd /tmp && rocprofv3 --pmc {ctr} --output-format csv -d $REPO/gpurun_out/pmc_{ctr} "
                        f"-o pmc -- python -u $REPO/bench.py --workload {workload}{mode} --steps 2 --warmup 1 "
                        f"--no-cpu-baseline --copy-calibration-mib {copy_bytes >> 20}\n")
            f.write(f"#   python bench.py --summarize-pmc <fetch csv> <write csv> --workload {workload}{mode}\n")
            f.write(f"# calibration: plain copy of {copy_bytes} bytes read {copy_fetch:.0f} FETCH bytes and "
                    f"{copy_write:.0f} WRITE bytes\n")
            f.write(f"fetch_scale: {f_scale:.4f}\n")
            f.write(f"write_scale: {w_scale:.4f}\n")
            f.write(f"dispatches: {len(fv)} / {len(wv)}\n")
            f.write(f"fetch_bytes_per_launch_raw: {kf:.0f}\n")
            f.write(f"write_bytes_per_launch_raw: {kw:.0f}\n")
            f.write(f"hbm_bytes_per_launch: {kf * f_scale + kw * w_scale:.0f}\n")
            f.write(f"source_digest: {kernel_source_digest()}\n")
        paths.append(path)
    return paths


def summarize_stats(stats_csv: str, bench_json: str, workload: str, mxfp8: bool = False) -> str:
    """Write profiles/kernels_<workload>.md from a rocprofv3 --kernel-trace
    --stats run of bench.py and the JSON line of a plain bench.py run."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    b = json.load(open(bench_json))
    c = b["config"]
    mode = " --mxfp8" if mxfp8 else ""
    path = os.path.join(PROFILE_DIR, f"kernels_{workload}{'_mxfp8' if mxfp8 else ''}.md")
    lines = [f"# rocprofv3 kernel statistics, {workload}{' MXFP8 step' if mxfp8 else ''} (B={c['B']}, H={c['H']}, "
             f"H_kv={c['H_kv']}, d={c['d']}, Lq={c['Lq']}, causal={c['causal']}, broadcast_q={c['broadcast_q']})", "",
             "Commands (MI355X, one GPU; `$REPO` is the repository root):", "", "```",
             "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             f"-d $REPO/gpurun_out/stats_{workload} -o stats -- python -u $REPO/bench.py --workload {workload}{mode} "
             "--steps 10 --warmup 2 --no-cpu-baseline",
             f"python bench.py --workload {workload}{mode} --no-cpu-baseline > bench.json",
             f"python bench.py --summarize-stats <stats_kernel_stats.csv> bench.json --workload {workload}{mode}",
             "```", "", "| kernel | calls | avg (us) | total (ms) | % |", "|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"].replace("|", "/")
        if len(n) > 90:
            n = n[:90] + "..."
        lines.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.1f} |")
    lines += ["", f"HIP-event timing inside the bench run (`bench.py{mode} --steps {b['steps']} "
                  f"--warmup {b['warmup']}`):", ""]
    r = b["roofline"]
    if mxfp8:
        for k, v in b["kernels"].items():
            lines.append(f"- {k}: {v['launches']} launches, avg {v['avg_ms']} ms, {v['gbs']} GB/s algorithmic"
                         + (f", {v['tflops']} useful TFLOP/s ({v['pct_of_fp8_peak'] * 100:.1f}% of the dense FP8 "
                            "peak)" if "tflops" in v else ""))
        lines += ["", f"Step: {b['value']} useful TFLOP/s, {b['ms_per_step']} ms; forward {b['fwd']['ms']} ms "
                      f"({b['fwd']['tflops']} TFLOP/s), backward {b['bwd']['ms']} ms ({b['bwd']['tflops']} TFLOP/s).",
                  f"Dominant kernel {r['kernel']}: {r['achieved']} {r['unit']} of {r['peak']} "
                  f"({r['frac'] * 100:.1f}%), traffic {r['traffic']}.", ""]
    else:
        for k, v in b["kernels"].items():
            lines.append(f"- {k}: {v['launches']} launches, avg {v['avg_ms']} ms"
                         + (f", {v['gbs']} GB/s algorithmic" if "gbs" in v else ""))
        lines += ["", f"Step: {b['value']} useful TFLOP/s ({b['pct_of_peak'] * 100:.1f}% of "
                      f"{b['device']['bf16_peak_tflops']} TFLOP/s), {b['ms_per_step']} ms; forward {b['fwd']['ms']} "
                      f"ms ({b['fwd']['tflops']} TFLOP/s), backward {b['bwd']['ms']} ms ({b['bwd']['tflops']} TFLOP/s).",
                  f"Dominant kernel {r['kernel']}: {r['achieved']} {r['unit']} of {r['peak']} "
                  f"({r['frac'] * 100:.1f}%), traffic {r['traffic']}.", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def summarize_counters(csvs, workload: str, cus: int = 256, mxfp8: bool = False) -> str:
    """Write profiles/counters_<workload>.md from the COUNTER_PASSES runs:
    per kernel, the mean of each counter over its dispatches and the ratios
    read from them."""
    rows, _ = counter_rows(csvs)
    mode = " --mxfp8" if mxfp8 else ""
    path = os.path.join(PROFILE_DIR, f"counters_{workload}{'_mxfp8' if mxfp8 else ''}.md")
    simds = cus * SIMD_PER_CU
    lines = [f"# Hardware counters per kernel, {workload}{' MXFP8 step' if mxfp8 else ''} (MI355X)", "",
             "Commands (one rocprofv3 run per counter pass; `$REPO` is the repository root):", "", "```"]
    for i, ps in enumerate(COUNTER_PASSES):
        lines.append(f"cd /tmp && timeout -s KILL 120 rocprofv3 --pmc {ps} --output-format csv "
                     f"-d $REPO/gpurun_out/ctr_p{i} -o pmc -- python -u $REPO/bench.py --workload {workload}{mode} "
                     "--steps 2 --warmup 1 --no-cpu-baseline")
    lines += [f"python bench.py --summarize-counters <the {len(COUNTER_PASSES)} counter_collection.csv files> "
              f"--workload {workload}{mode}", "```", "",
              "Ratios:",
              f"- MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCD} x {simds} SIMDs); "
              f"GRBM_GUI_ACTIVE counts every XCD's cycles. In the bf16 kernels SQ_VALU_MFMA_BUSY_CYCLES = "
              f"{MFMA_CYCLES} x SQ_INSTS_MFMA, one 32x32x16 bf16 product per 32 cycles of a SIMD.",
              "- LDS conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles the LDS stalls on "
              "bank conflicts, of the cycles it is busy with indexed access).",
              "- LDS cycles per instruction = SQ_LDS_IDX_ACTIVE / SQ_INSTS_LDS.",
              "- VALU / MFMA co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES.",
              "- wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave cycles spent in s_waitcnt).", ""]
    order = [k for k in ("fwd_kernel", "fwd_mx_kernel", "delta_kernel", "delta_mx_kernel", "dkdv_kernel",
                         "dkdv_mx_kernel", "dq_kernel", "dq_mx_kernel", "dq_reduce", "delta_exact_kernel",
                         "group_sum_kernel") if k in rows]
    ratio_hdr = "| kernel | MFMA busy | LDS conflict share | LDS cycles / instr | VALU-MFMA co-issue | wait share | VALU / MFMA instr |"
    lines += [ratio_hdr, "|" + "---|" * 7]

    def mean(lab, c):
        v = rows[lab].get(c)
        return sum(v) / len(v) if v else None

    def ratio(a, b, scale=1.0):
        return f"{a / b * scale:.3f}" if a is not None and b else "n/a"

    for lab in order:
        gui = mean(lab, "GRBM_GUI_ACTIVE")
        busy = mean(lab, "SQ_VALU_MFMA_BUSY_CYCLES")
        lines.append(f"| {lab} | {ratio(busy, gui / N_XCD * simds if gui else None)} | "
                     f"{ratio(mean(lab, 'SQ_LDS_BANK_CONFLICT'), mean(lab, 'SQ_LDS_IDX_ACTIVE'))} | "
                     f"{ratio(mean(lab, 'SQ_LDS_IDX_ACTIVE'), mean(lab, 'SQ_INSTS_LDS'))} | "
                     f"{ratio(mean(lab, 'SQ_VALU_MFMA_COEXEC_CYCLES'), busy)} | "
                     f"{ratio(mean(lab, 'SQ_WAIT_INST_ANY'), mean(lab, 'SQ_WAVE_CYCLES'))} | "
                     f"{ratio(mean(lab, 'SQ_INSTS_VALU'), mean(lab, 'SQ_INSTS_MFMA'))} |")
    ctrs = sorted({c for lab in order for c in rows[lab]})
    lines += ["", "Mean per dispatch:", "", "| counter | " + " | ".join(order) + " |", "|" + "---|" * (len(order) + 1)]
    for c in ctrs:
        vals = []
        for lab in order:
            m = mean(lab, c)
            vals.append(f"{m:.4g}" if m is not None else "")
        lines.append(f"| {c} | " + " | ".join(vals) + " |")
    lines += ["", f"source_digest: {kernel_source_digest()}", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


# ------------------------------------------------------- cpu baseline ----
def _oracle_item(args):
    """One (sequence, head) of the fp64 oracle: forward, then backward."""
    qb, kb, vb, dob, scale, causal, window = args
    from oracle import jfa_oracle as jo
    jo.sequence_forward(qb, kb, vb, scale, causal, window)
    jo.sequence_backward(qb, kb, vb, dob, scale, causal, window)
    return 0


def cpu_baseline(t, w, scale, seconds: float):
    """The fp64 oracle, as it stands, on the host cores: a process pool (one
    BLAS thread per worker, one worker per core this process may run on)
    over the (sequence, head) items of the same workload, in sequence order,
    until `seconds` of wall time are spent (or the whole workload is done)."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    off = t["offsets"].cpu().numpy()
    G = w.H // w.kv_heads
    q = t["q"].float().cpu().numpy()
    keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in keep:
        os.environ[k] = "1"
    try:
        pool = mp.get_context("spawn").Pool(cores)
    finally:
        for k, v in keep.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    with pool:
        pool.map(_oracle_item, [(np.zeros((1, 1)), np.zeros((1, 1)), np.zeros((1, 1)), np.zeros((1, 1)),
                                 1.0, False, 0)] * cores)  # workers started before the clock
        pending, done, flops = [], 0, 0
        t0 = time.perf_counter()
        b = 0
        while b < w.B and time.perf_counter() - t0 < seconds:
            # one sequence's heads per submission round, at most 2 * cores in flight
            s0, s1 = int(off[b]), int(off[b + 1])
            kb = t["k"][s0:s1].float().cpu().numpy()
            vb = t["v"][s0:s1].float().cpu().numpy()
            dob = (t["dout"][b] if w.broadcast_q else t["dout"][s0:s1]).float().cpu().numpy()
            for h in range(w.H):
                qb = q[h] if w.broadcast_q else q[s0:s1, h]
                d_h = dob[h] if w.broadcast_q else dob[:, h]
                pending.append(pool.apply_async(_oracle_item, ((qb, kb[:, h // G], vb[:, h // G], d_h, scale,
                                                                w.causal, w.window),)))
            f, bw = useful_flops([s1 - s0], w.H, w.d, w.Lq, w.causal, w.broadcast_q, w.window)
            flops += f + bw
            b += 1
            while len(pending) > 2 * cores:
                pending.pop(0).get()
        for p in pending:
            p.get()
        el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle forward+backward of the first {b} of {w.B} sequences "
                      f"({w.H} heads each; one process per core, one BLAS thread each) of the same "
                      f"workload, {el:.1f} s",
            "seconds": round(el, 2), "sequences": b}


# ---------------------------------------------------------------- MXFP8 ----
FP8_MFMA_FLOP_PER_CLK_PER_CU = 8192  # dense E4M3 (twice bf16)


def mx_algorithmic_bytes(kernel: str, lengths, H: int, H_kv: int, d: int, Lq: int, broadcast_q: bool,
                         P: int = 256) -> int:
    """Bytes an MXFP8 kernel must move per launch: every input encoding it
    reads once (E4M3 codes, 1 byte per element, with their E8M0 scales, one
    byte per 32 elements) and every output written once."""
    T = int(np.asarray(lengths).sum())
    B = len(lengths)
    t_pad = max(64, -(-T // 64) * 64)
    enc = d + d // 32                              # one row-wise or transposed encoding, per row
    kv_rows = T * H_kv * enc                       # K or V, row-wise
    kv_t = H_kv * d * t_pad + H_kv * (t_pad // 32) * d   # K^T or V^T
    q_rows = H * Lq if broadcast_q else T * H
    rows = B * H * Lq if broadcast_q else T * H
    if kernel == "fwd_mx_kernel":                 # Q, K, V^T in; O (bf16), lse out
        return kv_rows + kv_t + q_rows * enc + rows * (2 * d + 4)
    if kernel == "delta_mx_kernel":               # O, dO, lse in; delta, lse * log2(e) out
        return rows * (2 * d + enc + 4) + rows * 8
    if kernel == "dkdv_mx_kernel":                # K, V, Q and Q^T, dO and dO^T, lse, delta in; dK, dV (fp32) out
        return 2 * kv_rows + 2 * q_rows * enc + 2 * rows * enc + rows * 8 + 2 * T * H_kv * d * 4
    if kernel == "dq_mx_kernel":                  # K, V, K^T, Q, dO, lse, delta in; dQ or the partials out
        b = 2 * kv_rows + kv_t + q_rows * enc + rows * (enc + 8)
        if broadcast_q:
            n_qb, nc = dq_split(B, H, Lq, P)
            return b + H * n_qb * nc * 256 * d * 4
        return b + T * H * d * 4
    if kernel == "dq_reduce":
        n_qb, nc = dq_split(B, H, Lq, P)
        return H * n_qb * nc * 256 * d * 4 + H * Lq * d * 4
    return 0


MX_KERNELS = ("fwd_mx_kernel", "delta_mx_kernel", "dkdv_mx_kernel", "dq_mx_kernel", "dq_reduce")


def bench_mxfp8(args) -> int:
    """The MXFP8 step (forward, then backward) on a workload's shapes, from
    random E4M3 / E8M0 codes in every encoding: K timed steps by the host
    clock, then an instrumented run of K steps for each kernel's own time.
    Prints one JSON line of its own."""
    import torch
    import workloads as wl
    import jagged_flashattention_fwd_amd as jfa

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    peak8 = cus * FP8_MFMA_FLOP_PER_CLK_PER_CU * PEAK_SCLK_GHZ * 1e9 / 1e12
    w = wl.workload(args.workload)
    if w.d != 128 or w.window:
        print(f"--mxfp8 needs d = 128 and no window ({w.name})", file=sys.stderr)
        return 2
    t = wl.make_mx_bwd_workload(w, device=dev)
    lengths, T = t["lengths"], t["total_len"]
    H, H_kv, d, Lq, B = w.H, w.kv_heads, w.d, w.Lq, w.B
    bq, causal = w.broadcast_q, w.causal
    if bq:
        out = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
        dq = torch.empty((H, Lq, d), dtype=torch.float32, device=dev)
    else:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        dq = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    dk = torch.empty((T, H_kv, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws_f = jfa.workspace(T, B, H, Lq, d, causal, bq, 0, dev, H_kv=H_kv)
    ws_b = jfa.workspace(T, B, H, Lq, d, causal, bq, 1, dev, H_kv=H_kv)

    def fwd():
        jfa.jfa_fwd_mxfp8(t["q8"], t["q_scale"], t["k8"], t["k_scale"], t["vt8"], t["vt_scale"], t["offsets"],
                          B, H, H_kv, Lq, d, w.scale, causal, bq, out, lse, T, ws_f)

    def bwd():
        jfa.jfa_bwd_mxfp8(t, t["offsets"], B, H, H_kv, Lq, d, w.scale, causal, bq, out, lse, dq, dk, dv, T, ws_b)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # instrumented run: the forward's and the backward's calls, and each kernel
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    jfa.jfa_timing_enable(16 * args.steps + 16)
    jfa.jfa_timing_reset()
    for e in ev:
        e[0].record(s)
        fwd()
        e[1].record(s)
        bwd()
        e[2].record(s)
    torch.cuda.synchronize()
    kt = jfa.kernel_times()
    jfa.jfa_timing_enable(0)
    f_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    b_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    fl, bfl = useful_flops(lengths, H, d, Lq, causal, bq, 0)
    kflops = {"fwd_mx_kernel": fl, "dkdv_mx_kernel": bfl * 8 // 10, "dq_mx_kernel": bfl * 2 // 10 + fl}
    kernels = {}
    for name in MX_KERNELS:
        n, kms = kt.get(name, (0, 0.0))
        if not n:
            continue
        nbytes = mx_algorithmic_bytes(name, lengths, H, H_kv, d, Lq, bq, cus)
        e = {"launches": n, "avg_ms": round(kms / n, 4), "gbs": round(nbytes / (kms / n * 1e-3) / 1e9, 1),
             "algorithmic_bytes": nbytes}
        if name in kflops:
            tf = kflops[name] / (kms / n * 1e-3) / 1e12
            e["tflops"] = round(tf, 1)
            e["pct_of_fp8_peak"] = round(tf / peak8, 4)
        kernels[name] = e
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    kd = kernels[dom]
    t_hbm = kd["algorithmic_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = kflops.get(dom, 0) / (peak8 * 1e12)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": kd["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kd["gbs"] / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": kd["tflops"], "peak": round(peak8, 1), "unit": "TFLOP/s",
                "frac": round(kd["tflops"] / peak8, 4)}
    roof.update({"kernel": dom, "traffic": measured_traffic(dom, w.name + "_mxfp8"),
                 "algorithmic_bytes": kd["algorithmic_bytes"], "useful_flops": kflops.get(dom, 0)})
    tot = fl + bfl
    res = {
        "metric": "useful TFLOP/s, MXFP8 step: forward + backward (E4M3 operands, E8M0 block scales)",
        "value": round(tot / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e4m3", "data": "synthetic (random E4M3 / E8M0 codes, every encoding)",
        "config": {"workload": w.name, "B": B, "H": H, "H_kv": H_kv, "d": d, "Lq": Lq, "causal": causal,
                   "broadcast_q": bq, "total_len": T, "accumulate": "fp32", "out": "bf16", "grads": "fp32"},
        "timing": "value and ms_per_step: host clock over the K timed steps; fwd / bwd and kernels: hipEvents "
                  "on the launch stream over a second, instrumented run of K steps",
        "fwd": {"ms": round(f_ms, 4), "tflops": round(fl / (f_ms * 1e-3) / 1e12, 1),
                "pct_of_fp8_peak": round(fl / (f_ms * 1e-3) / 1e12 / peak8, 4)},
        "bwd": {"ms": round(b_ms, 4), "tflops": round(bfl / (b_ms * 1e-3) / 1e12, 1),
                "pct_of_fp8_peak": round(bfl / (b_ms * 1e-3) / 1e12 / peak8, 4)},
        "kernels": kernels,
        "roofline": roof,
        "device": {"cus": cus, "fp8_peak_tflops": round(peak8, 1), "hbm_peak_gbs": HBM_PEAK_GBS},
    }
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n * 4
    print(json.dumps(res), flush=True)
    return 0


# ---------------------------------------------------------------- main ----
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prod_bcast")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the timed region, run one plain device copy of this many MiB "
                         "(reference kernel for scaling hardware byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summaries under profiles/ from two counter runs and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="write profiles/counters_<workload>.md from the counter-pass runs and exit")
    ap.add_argument("--mxfp8", action="store_true",
                    help="measure the MXFP8 step (forward + backward) on the workload's shapes instead "
                         "(its own JSON line)")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "BENCH_JSON"),
                    help="write profiles/kernels_<workload>.md from a --kernel-trace --stats run and exit")
    args = ap.parse_args(argv)
    if args.summarize_stats:
        print(summarize_stats(args.summarize_stats[0], args.summarize_stats[1], args.workload, args.mxfp8))
        return 0
    if args.summarize_pmc:
        for p in summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                               (args.copy_calibration_mib or 1024) << 20, args.mxfp8):
            print(p)
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, args.workload, mxfp8=args.mxfp8))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on a single MI355X).", file=sys.stderr)
        return 2
    if args.mxfp8:
        return bench_mxfp8(args)

    import torch
    import workloads as wl
    import jagged_flashattention_fwd_amd as jfa

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    clock_ghz = PEAK_SCLK_GHZ  # published peak engine clock; the reported current clock varies
    peak_tflops = cus * MFMA_FLOP_PER_CLK_PER_CU * clock_ghz * 1e9 / 1e12

    w = wl.workload(args.workload)
    seed = wl.WORKLOADS.index(w)
    t = wl.make_workload(w, seed=seed, device=dev)
    lengths = t["lengths"]
    T = t["total_len"]
    scale = w.scale
    H, d, Lq, B = w.H, w.d, w.Lq, w.B
    H_kv, window = w.kv_heads, w.window
    bq, causal = w.broadcast_q, w.causal
    q, k, v, off, dout = t["q"], t["k"], t["v"], t["offsets"], t["dout"]

    if bq:
        out = torch.empty((B, H, Lq, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=dev)
    else:
        out = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty((T, H_kv, d), dtype=torch.float32, device=dev)
    dv = torch.empty((T, H_kv, d), dtype=torch.float32, device=dev)
    ws_f = jfa.workspace(T, B, H, Lq, d, causal, bq, 0, dev, H_kv=H_kv)
    ws_b = jfa.workspace(T, B, H, Lq, d, causal, bq, 1, dev, H_kv=H_kv)
    _, P = jfa.jfa_schedule_params(1, causal, bq, d)

    def fwd():
        jfa.jfa_fwd_ex(q, k, v, off, B, H, H_kv, Lq, d, scale, causal, window, bq, out, lse, T, ws_f)

    def bwd():
        jfa.jfa_bwd_ex(q, k, v, off, B, H, H_kv, Lq, d, scale, causal, window, bq, out, lse, dout, dq, dk, dv,
                       T, ws_b)

    def step():
        fwd()
        bwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps bracketed by synchronisations, nothing else
    # enqueued.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # Instrumented pass, the same K steps again: forward / backward events on
    # the launch stream, and the library's own per-kernel events around every
    # launch.
    jfa.jfa_timing_enable(16 * args.steps + 16)
    jfa.jfa_timing_reset()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    ktimes = jfa.kernel_times()
    jfa.jfa_timing_enable(0)

    fwd_ms = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
    bwd_ms = float(np.median([b.elapsed_time(c) for _, b, c in ev]))
    fwd_fl, bwd_fl = useful_flops(lengths, H, d, Lq, causal, bq, window)
    value = (fwd_fl + bwd_fl) / (ms_step * 1e-3) / 1e12
    fwd_tf = fwd_fl / (fwd_ms * 1e-3) / 1e12
    bwd_tf = bwd_fl / (bwd_ms * 1e-3) / 1e12

    # Dominant kernel: largest device time per step.
    per_kernel = {}
    for name, (n, ms) in ktimes.items():
        if n:
            per_kernel[name] = {"launches": n, "avg_ms": ms / n,
                                "ms_per_step": ms / args.steps}
    dom = max(per_kernel, key=lambda n: per_kernel[n]["ms_per_step"])
    avg_s = per_kernel[dom]["avg_ms"] * 1e-3
    nbytes = algorithmic_bytes(dom, lengths, H, d, Lq, bq, P, H_kv)
    kfl = kernel_flops(dom, fwd_fl, bwd_fl, bq)
    gbs = nbytes / avg_s / 1e9
    tfl = kfl / avg_s / 1e12 if kfl else 0.0
    # bound: whichever of HBM time and MFMA time at peak is larger
    hbm_bound = nbytes / (HBM_PEAK_GBS * 1e9) >= kfl / (peak_tflops * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tfl, 1), "peak": round(peak_tflops, 1),
                "unit": "TFLOP/s", "frac": round(tfl / peak_tflops, 4)}
    roof["traffic"] = measured_traffic(dom, w.name)
    roof.update({"kernel": dom, "avg_launch_ms": round(per_kernel[dom]["avg_ms"], 4),
                 "algorithmic_bytes": nbytes, "kernel_useful_flops": kfl,
                 "kernel_tflops": round(tfl, 1), "kernel_gbs": round(gbs, 1)})
    for name, rec in per_kernel.items():
        b = algorithmic_bytes(name, lengths, H, d, Lq, bq, P, H_kv)
        rec["avg_ms"] = round(rec["avg_ms"], 4)
        rec["ms_per_step"] = round(rec["ms_per_step"], 4)
        if b:
            rec["gbs"] = round(b / (rec["avg_ms"] * 1e-3) / 1e9, 1)

    res = {
        "metric": "useful TFLOP/s fwd & bwd (no padding) + % of MI355X bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "H_kv": H_kv, "window": window, "d": d, "Lq": Lq,
                   "lengths": list(w.lengths), "causal": causal, "broadcast_q": bq,
                   "total_len": T, "seed": seed, "accumulate": "fp32", "grad_dtype": "fp32"},
        "pct_of_peak": round(value / peak_tflops, 4),
        "timing": "value and ms_per_step: host clock over the K timed steps alone; fwd, bwd and kernels: "
                  "hipEvents on the launch stream over a second, instrumented run of K steps",
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_tf, 1),
                "pct_of_peak": round(fwd_tf / peak_tflops, 4), "useful_flops": fwd_fl},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_tf, 1),
                "pct_of_peak": round(bwd_tf / peak_tflops, 4), "useful_flops": bwd_fl},
        "device": {"name": props.name, "cus": cus, "clock_ghz": clock_ghz,
                   "bf16_peak_tflops": round(peak_tflops, 1)},
        "kernels": per_kernel,
        "roofline": roof,
    }
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n * 4
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(t, w, scale, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
