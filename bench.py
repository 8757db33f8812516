"""Benchmark of the chunked LM-head forward+backward on one MI355X.

Default workload: SFT head, bf16 inputs with fp32 accumulation, T = 9000
tokens, D = 2560, V = 151936, chunk C = 1024 (Qwen3-4B-shaped head; seeded
synthetic inputs).  One step = one full call of the library's SFT entry point
(label scan, every chunk's logits GEMM + LSE, dlogits, dH and dW GEMMs, loss
reduce) with inputs already resident in HBM.  ``--tiled-logits`` times the
library's tiled logits operands instead: the per-call copy of W into tiles is
then inside the timed step, the results are bitwise those of the plain path,
and the workspace grows by V x D bf16 (``workspace_bytes`` in the output).

Other workloads (``--workload``): ``grpo_8x12288_bf16`` times the GRPO entry
point, ``ppo_8x12288_bf16`` the off-policy clipped-surrogate entry point at
the same shapes, ``dpo_4pairs_16384_bf16`` both DPO passes (8TVD flops),
``long_sft_32768_bf16`` the SFT entry point at T = 32768, D = 5120 (``--chunk``
sweeps C), ``tiny_sft_f32`` the fp32 path.

Prints one JSON line.  `value` and `ms_per_step` come from K steps with no
per-launch events.  The same K steps then run again with the library's
HIP-event timer (an event pair on the call's stream around every launch):
`kernels` holds that pass's per-kernel times (`kernels_pass_ms_per_step` its
step time) and `roofline` covers the kernel with the largest share of it.
`cpu_baseline` times the fp64 CPU oracle on a bounded slice of the same
workload.  `epilogue_hbm` is the backward row pass (softmax - onehot over
the chunk logits, in place) against HBM and against torch's in-place
elementwise rate over a buffer of the same shape.  `mfma_probe` is the sustained rate of a loop of nothing but the
GEMMs' MFMA instruction (the achievable peak beside the data-sheet one, and
the step's fraction of it); `yardstick` times torch's own bf16 GEMMs
(hipBLASLt) on one chunk's three shapes beside the library's kernels.
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

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sft_9k_bf16")
    ap.add_argument("--chunk", type=int, default=0, help="override the workload's chunk size")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-rows", type=int, default=6000, help="tokens in the oracle's timed slice")
    ap.add_argument("--tiled-logits", action=argparse.BooleanOptionalAction, default=False,
                    help="logits GEMM from tiled copies of W and H (bf16; V*D bf16 more workspace, bitwise "
                         "the same results; off by default, as in the library)")
    ap.add_argument("--dpo-row-pass", action="store_true",
                    help="DPO pass 2 through the row pass instead of the logits epilogue's direct gradient")
    ap.add_argument("--compact", action="store_true",
                    help="masked-row compaction: run the chunk loop over valid rows only (reported separately; "
                         "flops counted over the valid rows)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-yardstick", action="store_true",
                    help="skip the sustained-MFMA probe and the torch GEMMs of the chunk's shapes")
    ap.add_argument("--no-clocks", action="store_true",
                    help="do not run rocm-smi for the GPU clocks (for runs under rocprofv3 --pmc)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one device-to-device copy of MIB MiB (reference for HBM byte counters)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="no GPU work: summarise rocprofv3 CSV output found under each DIR (kernel stats, "
                         "counter means per kernel kind and, for a kernel trace, each kernel kind's fraction "
                         "of its roof at the --workload / --chunk shapes) as markdown")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: from a FETCH_SIZE and a WRITE_SIZE rocprofv3 pass of a run with "
                         "--copy-calibration MIB, write profiles/<workload>_traffic.json for these kernel sources")
    return ap.parse_args()


# kernel kinds by the rocprofv3 kernel name (the names bench.py's event timing uses)
def kernel_kind(name):
    for pat, kind in (("copyBuffer", "copy"), ("native::reduce_kernel", "read_only"), ("EpiLogits", "logits_lse"),
                      ("EpiStore", "dh_gemm"),
                      ("EpiAccum", "dw_gemm"), ("rows_kernel", "rows_lse_dlogits"),
                      ("splitk_reduce", "dh_splitk_reduce"), ("tile32", "tile"), ("scan_labels", "scan_labels"),
                      ("gemm_f32", "gemm_f32")):
        if pat in name:
            return kind
    return None


def _csv_rows(d, suffix):
    import csv
    import glob
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def counter_dispatches(d):
    """{(kind, counter, dispatch id): value summed over the counter's instances}."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        kind = kernel_kind(r["Kernel_Name"])
        if kind is None:
            continue
        key = (kind, r["Counter_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return per


def counter_means(d):
    """{kind: {counter: (mean per dispatch, dispatches)}} from the counter CSVs under d."""
    acc = {}
    for (kind, ctr, _), v in counter_dispatches(d).items():
        s, n = acc.setdefault(kind, {}).get(ctr, (0.0, 0))
        acc[kind][ctr] = (s + v, n + 1)
    return {k: {c: (s / n, n) for c, (s, n) in cs.items()} for k, cs in acc.items()}


def trace_roofline(d, wl):
    """{kind: figures} from the kernel trace under d: launches, mean launch
    time, and the launch's algorithmic work at the shapes of workload wl
    (rows per launch = T over the call's chunks, as in the timed step) over
    that time, against the roof that can bind it: the GEMMs against the
    dense MFMA peak of the inputs' type, the dW launch and the backward row
    pass also against HBM (the row pass's bytes are those of a backward
    pass, so DPO, whose first pass has none, gets no HBM figure)."""
    acc = {}
    for r in _csv_rows(d, "kernel_stats.csv"):
        k = kernel_kind(r["Name"])
        if k is None or k in ("copy", "read_only"):
            continue
        n = int(r["Calls"])
        tot, cnt = acc.get(k, (0.0, 0))
        acc[k] = (tot + float(r["AverageNs"]) * n, cnt + n)
    n_chunks = -(-wl.T // wl.C)
    rows = wl.T / n_chunks
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    out = {}
    for k, (tot, n) in acc.items():
        avg_s = tot / n / 1e9
        e = {"launches": n, "avg_us": avg_s * 1e6}
        f = gemm_flops_per_launch(k, rows, wl)
        if f:
            e["tflops"] = f / avg_s / 1e12
            e["frac_mfma"] = e["tflops"] / peak
        b = None
        if k == "dw_gemm":
            b = dw_bytes_per_launch(rows, n_chunks, wl)
        elif k == "rows_lse_dlogits" and wl.kind != "dpo":
            b = rows_bytes_per_launch(rows, wl)
        if b:
            e["bytes"] = b
            e["gbs"] = b / avg_s / 1e9
            e["frac_hbm"] = e["gbs"] / PEAK_HBM_GBS
        out[k] = e
    return out


def summarize(dirs, wl=None):
    for d in dirs:
        stats = _csv_rows(d, "kernel_stats.csv")
        if stats:
            print(f"\n{d}: kernel stats\n\n| kernel | calls | avg us | min us | max us | % of GPU time |\n|---|---|---|---|---|---|")
            for r in stats:
                print(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                      f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
            if wl is not None:
                print(f"\n{d}: each kind against its roof ({wl.name}, C={wl.C})\n")
                print(roofline_markdown(trace_roofline(d, wl)))
        means = counter_means(d)
        if means:
            ctrs = sorted({c for cs in means.values() for c in cs})
            print(f"\n{d}: counter means per dispatch\n\n| kind | dispatches | " + " | ".join(ctrs) + " |")
            print("|---|---|" + "---|" * len(ctrs))
            for k, cs in sorted(means.items()):
                n = max(v[1] for v in cs.values())
                print(f"| {k} | {n} | " + " | ".join(f"{cs[c][0]:.4g}" if c in cs else "" for c in ctrs) + " |")


def roofline_markdown(rl):
    peak_note = "MFMA peak"
    rows = ["| kernel kind | launches | avg us | TFLOP/s | of the " + peak_note + " | algorithmic GB/launch | GB/s | of 8 TB/s |",
            "|---|---|---|---|---|---|---|---|"]
    for k, e in sorted(rl.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["launches"]):
        def cell(key, fmt):
            return format(e[key], fmt) if key in e else ""
        rows.append(f"| {k} | {e['launches']} | {e['avg_us']:.1f} | {cell('tflops', '.1f')} | "
                    f"{cell('frac_mfma', '.3f')} | {format(e['bytes'] / 1e9, '.3f') if 'bytes' in e else ''} | "
                    f"{cell('gbs', '.0f')} | {cell('frac_hbm', '.3f')} |")
    return "\n".join(rows)


def write_traffic(workload, fetch_dir, write_dir, copy_mib):
    """HBM-side bytes per launch and kernel kind: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled so that the calibration copy of
    copy_mib MiB reads and writes exactly its size."""
    f, w = counter_means(fetch_dir), counter_means(write_dir)
    copy_bytes = copy_mib << 20

    def largest(d, ctr, kind):  # the calibration kernels; the workload makes small copies too
        vals = [v for (k, c, _), v in counter_dispatches(d).items() if k == kind and c == ctr]
        return max(vals) if vals else None
    fs = copy_bytes / (largest(fetch_dir, "FETCH_SIZE", "copy") * 1024)
    ws = copy_bytes / (largest(write_dir, "WRITE_SIZE", "copy") * 1024)
    ro = largest(fetch_dir, "FETCH_SIZE", "read_only")
    fs_ro = copy_bytes / (ro * 1024) if ro else None
    per = {}
    for k in sorted(set(f) & set(w)):
        if k in ("copy", "read_only") or "FETCH_SIZE" not in f[k] or "WRITE_SIZE" not in w[k]:
            continue
        per[k] = {"fetch_bytes": f[k]["FETCH_SIZE"][0] * 1024 * fs, "write_bytes": w[k]["WRITE_SIZE"][0] * 1024 * ws,
                  "fetch_kib_raw": f[k]["FETCH_SIZE"][0], "write_kib_raw": w[k]["WRITE_SIZE"][0],
                  "dispatches": f[k]["FETCH_SIZE"][1]}
    rec = {"workload": workload, "source_sha256": kernel_source_sha256(),
           "calibration": {"copy_bytes": copy_bytes, "fetch_scale": fs, "write_scale": ws,
                           "fetch_scale_read_only": fs_ro}, "per_launch": per}
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(f"calibration: FETCH_SIZE x {fs:.4f} (copy), x {fs_ro if fs_ro else float('nan'):.4f} (read-only "
          f"reduction), WRITE_SIZE x {ws:.4f}; wrote {path}")
    print("| kernel | dispatches | FETCH_SIZE KiB raw | WRITE_SIZE KiB raw | fetched GB/launch (scaled) | "
          "written GB/launch (scaled) |\n|---|---|---|---|---|---|")
    for k, v in per.items():
        print(f"| {k} | {v['dispatches']} | {v['fetch_kib_raw']:.0f} | {v['write_kib_raw']:.0f} | "
              f"{v['fetch_bytes'] / 1e9:.3f} | {v['write_bytes'] / 1e9:.3f} |")


def kernel_source_sha256():
    """Hash of the HIP sources; HBM counters recorded for other sources are stale."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "loss_head_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic(workload, kernel):
    """HBM-side bytes per launch of `kernel` (rocprofv3 FETCH_SIZE + WRITE_SIZE,
    scaled by a copy of known size; profiles/<workload>_traffic.json), or None
    when absent or recorded for different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_sha256() or kernel not in rec.get("per_launch", {}):
        return None
    k = rec["per_launch"][kernel]
    return k["fetch_bytes"] + k["write_bytes"]


def gemm_flops_per_launch(kind, rows, wl):
    # each of the three GEMMs of a chunk does 2 * rows * V * D flops
    return 2.0 * rows * wl.V * wl.D if kind in ("logits_lse", "dh_gemm", "dw_gemm") else 0.0


def dw_bytes_per_launch(rows, n_launch, wl):
    """Algorithmic HBM bytes of one dW launch, averaged over the call's
    launches: G (rows x V, 2 or 4 B) and H_c read, dW (V x D fp32) written,
    and the old dW read on every launch but the first (no accumulate)."""
    b = 2 if wl.dtype == "bf16" else 4
    vd4 = 4.0 * wl.V * wl.D
    return rows * wl.V * b + rows * wl.D * b + vd4 + vd4 * (n_launch - 1) / max(1, n_launch)


def mfma_probe(dev, reps=3):
    """Sustained dense bf16 rate of the library's pure-MFMA probe (the GEMMs'
    instruction on fixed register operands), best of `reps` timed launches."""
    import ctypes

    import torch

    from loss_head_amd import _capi

    lib = _capi.load()
    blocks, iters = 4096, 6000
    st = torch.cuda.current_stream(dev)
    out = {}
    for changing, key in ((0, "same_operands_tflops"), (1, "changing_operands_tflops")):
        flops, best = ctypes.c_double(), 0.0
        for r in range(reps + 1):  # the first launch is a warmup
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rc = lib.streambp_head_mfma_probe(blocks, iters, changing, ctypes.byref(flops),
                                              ctypes.c_void_p(st.cuda_stream))
            e1.record(st)
            e1.synchronize()
            if rc != 0:
                raise RuntimeError(f"streambp_head_mfma_probe: status {rc}")
            if r:
                best = max(best, flops.value / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        out[key] = round(best, 1)
    out["what"] = (f"loops of v_mfma_f32_32x32x16_bf16 on register operands ({blocks} blocks of 4 waves x 8 "
                   "chains, no memory traffic): the same operand pair in every instruction, and pseudo-random "
                   "pairs that change per instruction as in a GEMM")
    return out


def torch_yardstick(H, W, labels, C, dev, reps=5):
    """torch's bf16 GEMMs (hipBLASLt) on one chunk's three shapes with the
    workload's own data: Z = H_c W^T, dH = G W, dW = G^T H_c, bf16 outputs,
    no epilogue.  G is the chunk's w (softmax - onehot), as the row pass forms it."""
    import torch

    Hc = H[:C].contiguous()
    y = labels[:C].long()
    with torch.no_grad():
        Z = torch.nn.functional.linear(Hc, W)
        n = max(1, int((labels >= 0).sum().item()))
        P = torch.softmax(Z.float(), dim=1)
        ok = y >= 0
        P[ok, y[ok]] -= 1.0
        P[~ok] = 0.0
        G = (P / n).to(torch.bfloat16)
        del P
        Gt = G.t().contiguous()
    shapes = {"logits_lse": lambda: torch.nn.functional.linear(Hc, W),
              "dh_gemm": lambda: torch.matmul(G, W),
              "dw_gemm": lambda: torch.matmul(Gt, Hc)}
    flops = 2.0 * C * W.shape[0] * W.shape[1]
    out = {}
    st = torch.cuda.current_stream(dev)
    for name, fn in shapes.items():
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        e1.synchronize()
        out[name] = round(flops / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e12, 1)
    del Z, G, Gt
    torch.cuda.empty_cache()
    return out


def torch_inplace_hbm(rows, V, dev, reps=10):
    """torch's in-place elementwise rate over a rows x V bf16 buffer (the row
    pass's chunk logits): one read and one write of every element, GB/s."""
    import torch

    buf = torch.ones(rows * V, dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream(dev)
    for _ in range(3):
        buf.mul_(1.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        buf.mul_(1.0)
    e1.record(st)
    e1.synchronize()
    gbs = 2.0 * buf.numel() * 2 / (e0.elapsed_time(e1) * 1e-3 / reps) / 1e9
    del buf
    torch.cuda.empty_cache()
    return round(gbs, 1)


def environment(dev, clocks=True):
    """Software and device the numbers were taken on, and the GPU clocks that
    rocm-smi reports at the end of the run (None where a tool is missing, or
    with clocks=False: under a counter-collecting profiler the GPU is set up
    before the program starts, and rocm-smi, a script, is not started then)."""
    import subprocess

    import torch

    p = torch.cuda.get_device_properties(dev)
    env = {"torch": torch.__version__, "hip": torch.version.hip, "device": p.name,
           "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
           "hbm_gib": round(p.total_memory / 2**30, 1), "clocks": None}
    if not clocks:
        return env
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        card = next(iter(json.loads(out.stdout).values()))
        env["clocks"] = {k.rstrip(":").strip(): v.strip("()") for k, v in card.items()
                         if "clock speed" in k.lower()}
    except Exception:  # no rocm-smi, or output it cannot parse: the clocks stay unknown
        pass
    return env


def rows_bytes_per_launch(rows, wl):
    """Algorithmic HBM bytes of one backward row pass (softmax - onehot in
    place over the chunk logits): Z read and G written (rows x V), the LSE
    partials (rows x ceil(V/256) x 8 B), the rows of H and W_y its fp32
    label logit reads (2 x rows x D), and the per-token arrays (labels, weight,
    log-prob, fp64 loss term; PPO adds two log-probs)."""
    b = 2 if wl.dtype == "bf16" else 4
    per_token = 20 + (8 if wl.kind == "ppo" else 0)
    return rows * (2.0 * wl.V * b + -(-wl.V // 256) * 8 + 2.0 * wl.D * b + per_token)


def main():
    args = parse()
    if args.summarize:
        wl = None
        if "--workload" in sys.argv or "--chunk" in sys.argv:
            from workloads import gen
            wl = gen.ALL[args.workload]
            if args.chunk:
                wl = wl.with_(C=args.chunk)
        summarize(args.summarize, wl)
        return
    if args.write_traffic:
        write_traffic(args.workload, *args.write_traffic, args.copy_calibration or 1024)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the head's data-parallel split across GPUs is described in the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    from loss_head_amd import Head
    from workloads import gen

    wl = gen.ALL[args.workload]
    if args.chunk:
        wl = wl.with_(C=args.chunk)
    print(f"[bench] generating {wl.name} T={wl.T} D={wl.D} V={wl.V} C={wl.C}", file=sys.stderr, flush=True)
    inp = gen.make_inputs(wl, args.seed)
    dev = torch.device("cuda", 0)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    if wl.dtype == "bf16":
        H = torch.from_numpy(inp.H.view(np.int16)).view(torch.bfloat16).to(dev)
        W = torch.from_numpy(inp.W.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        H, W = torch.from_numpy(inp.H).to(dev), torch.from_numpy(inp.W).to(dev)
    y = torch.from_numpy(inp.labels.astype(np.int32)).to(dev)
    off = torch.from_numpy(inp.offsets.astype(np.int32)).to(dev)
    adv = None if inp.adv is None else torch.from_numpy(inp.adv).to(dev)
    ref = None if inp.ref_logp is None else torch.from_numpy(inp.ref_logp).to(dev)
    lp_old = None if inp.logp_old is None else torch.from_numpy(inp.logp_old).to(dev)
    lp_ref = None if inp.logp_ref is None else torch.from_numpy(inp.logp_ref).to(dev)
    tiled = bool(args.tiled_logits) and wl.dtype == "bf16"
    head = Head(wl.D, wl.V, wl.C, wl.dtype, compact=args.compact, tiled_logits=tiled)
    dH = torch.empty((wl.T, wl.D), dtype=torch.float32, device=dev)
    dW = torch.empty((wl.V, wl.D), dtype=torch.float32, device=dev)
    head.workspace(wl.T, wl.n_seq)
    torch.cuda.synchronize()

    if args.copy_calibration:
        # HBM byte counters' references: a device copy (reads and writes n
        # bytes) and a read-only reduction over n bytes (reads n, writes 4)
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        total = src.view(torch.float32).sum()
        torch.cuda.synchronize()
        del src, dst, total

    if wl.kind == "sft":
        def step():
            head.sft(H, W, y, dH=dH, dW=dW, check=False)
    elif wl.kind == "grpo":
        def step():
            head.grpo(H, W, y, off, adv, dH=dH, dW=dW, check=False)
    elif wl.kind == "ppo":
        def step():
            head.ppo(H, W, y, off, adv, lp_old, lp_ref, 0.2, wl.beta, dH=dH, dW=dW, check=False)
    else:  # dpo: both passes (sequence log-prob sums, then the backward)
        def step():
            head.dpo(H, W, y, off, ref, wl.beta, dH=dH, dW=dW, check=False, fuse=not args.dpo_row_pass)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    status = int(head.status.item())
    mem0 = torch.cuda.memory_allocated(dev)

    # the headline: K steps with no per-launch events on the stream
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    # the per-kernel breakdown: the same K steps again, each launch bracketed
    # by a pair of HIP events on the call's stream (the library's timer)
    ktimes, ms_events = {}, None
    if not args.no_kernel_timing:
        print(f"[bench] per-kernel event timing, {args.steps} steps", file=sys.stderr, flush=True)
        head.set_timing(True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms_events = (time.perf_counter() - t1) * 1e3 / args.steps
        ktimes = head.kernel_times()
        head.set_timing(False)
    tok_s = wl.T / (ms / 1e3)
    # executed GEMM flops: 2TVD each for logits, dH and dW; DPO adds the
    # forward-only first pass
    n_valid = int(((inp.labels >= 0) & (inp.labels < wl.V)).sum())
    rows_run = n_valid if args.compact else wl.T
    flops = (8.0 if wl.kind == "dpo" else 6.0) * rows_run * wl.V * wl.D
    tflops = flops / (ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS

    # roofline of the kernel with the largest total time in the timed region
    roofline, epilogue = None, None
    kernels = {}
    if ktimes:
        n_full, tail = divmod(rows_run, wl.C)
        live_chunks = n_full + (1 if tail else 0)
        rows_per_launch = rows_run / max(1, live_chunks)
        # with compaction the chunks past the valid rows launch and exit at
        # once: per-launch averages count the live launches only
        live_frac = live_chunks / max(1, -(-wl.T // wl.C))
        for k, (tot, n) in ktimes.items():
            if n:
                n_eff = max(1.0, n * live_frac) if args.compact else n
                kernels[k] = {"ms_total": round(tot, 4), "launches": n, "avg_us": round(tot / n_eff * 1e3, 2)}
        dom = max((k for k in kernels if k in ("logits_lse", "dh_gemm", "dw_gemm")),
                  key=lambda k: kernels[k]["ms_total"])
        avg_s = kernels[dom]["avg_us"] / 1e6
        traffic = recorded_traffic(wl.name, dom)
        flops_l = gemm_flops_per_launch(dom, rows_per_launch, wl)
        bytes_l = dw_bytes_per_launch(rows_per_launch, live_chunks, wl) if dom == "dw_gemm" else None
        # the binding roof: HBM when the launch's flops per algorithmic byte
        # fall below the ridge point (the dW read-modify-write at small C)
        if bytes_l is not None and flops_l / bytes_l < peak * 1e12 / (PEAK_HBM_GBS * 1e9):
            ach = bytes_l / avg_s / 1e9
            roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes_per_launch": round(bytes_l), "intensity_flop_per_byte":
                        round(flops_l / bytes_l, 1), "mfma_tflops": round(flops_l / avg_s / 1e12, 1)}
        else:
            ach = flops_l / avg_s / 1e12
            roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": peak,
                        "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
        roofline.update({"traffic": None if traffic is None else round(traffic / 1e9, 3),
                         "traffic_unit": "GB/launch", "avg_launch_us": round(avg_s * 1e6, 1)})
        for k in kernels:
            f = gemm_flops_per_launch(k, rows_per_launch, wl)
            if f:
                t = f / (kernels[k]["avg_us"] / 1e6) / 1e12
                kernels[k]["tflops"] = round(t, 1)
                kernels[k]["frac_peak"] = round(t / peak, 4)
        # the HBM-bound epilogue: the row pass's bytes against HBM
        if wl.kind in ("sft", "grpo", "ppo") and "rows_lse_dlogits" in kernels:
            b_l = rows_bytes_per_launch(rows_per_launch, wl)
            t_s = kernels["rows_lse_dlogits"]["avg_us"] / 1e6
            tr = recorded_traffic(wl.name, "rows_lse_dlogits")
            epilogue = {"kernel": "rows_lse_dlogits", "bound": "hbm", "achieved": round(b_l / t_s / 1e9, 1),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(b_l / t_s / 1e9 / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes_per_launch": round(b_l),
                        "traffic": None if tr is None else round(tr / 1e9, 3), "traffic_unit": "GB/launch",
                        "avg_launch_us": round(t_s * 1e6, 1)}

    probe, yard = None, None
    if not args.no_yardstick and wl.dtype == "bf16":
        print("[bench] sustained-MFMA probe and torch GEMM yardstick", file=sys.stderr, flush=True)
        probe = mfma_probe(dev)
        probe["step_frac_of_changing"] = round(tflops / probe["changing_operands_tflops"], 4)
        ours = {k: v["tflops"] for k, v in kernels.items() if "tflops" in v}
        torch_t = torch_yardstick(H, W, y, min(wl.C, wl.T), dev)
        yard = {"what": "torch bf16 GEMMs (hipBLASLt) of one chunk's three shapes on the workload's data, bf16 "
                        "outputs, no epilogue; ours with their epilogues (LSE partials and bf16 Z store; split-K "
                        "slabs; dW's fp32 read-modify-write), from the event-timed pass",
                "torch_tflops": torch_t, "ours_tflops": ours,
                "ours_over_torch": {k: round(ours[k] / torch_t[k], 3) for k in torch_t if k in ours}}
        if epilogue is not None:
            # the achievable rate of the row pass's access pattern beside the data-sheet one
            ref = torch_inplace_hbm(min(wl.C, wl.T), wl.V, dev)
            epilogue["torch_inplace_gbs"] = ref
            epilogue["frac_of_torch_inplace"] = round(epilogue["achieved"] / ref, 4)

    cpu = None
    if not args.no_cpu_baseline and wl.kind == "sft":
        cpu = cpu_baseline(inp, wl, args.cpu_rows)

    out = {
        "metric": ("LM-head fwd+bwd tokens/s and % bf16 MFMA peak (T=9k, D=2560, V=151936)"
                   if wl.name == "sft_9k_bf16" and not args.compact else f"LM-head fwd+bwd tokens/s ({wl.kind}, "
                   f"T={wl.T}, D={wl.D}, V={wl.V}{', masked rows skipped' if args.compact else ''})"),
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "D": wl.D, "V": wl.V, "chunk": wl.C,
                   "objective": wl.kind, "n_seq": wl.n_seq, "masked": int((inp.labels == -100).sum()),
                   "row_compaction": bool(args.compact), "tiled_logits": tiled,
                   **({"dpo_pass2": "row_pass" if args.dpo_row_pass else "fused"} if wl.kind == "dpo" else {})},
        "tflops": round(tflops, 1),
        "frac_bf16_peak": round(tflops / peak, 4),
        "roofline": roofline,
        "epilogue_hbm": epilogue,
        "mfma_probe": probe,
        "yardstick": yard,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "kernels_pass_ms_per_step": None if ms_events is None else round(ms_events, 4),
        "device_status": status,
        "environment": environment(dev, clocks=not args.no_clocks),
        "workspace_bytes": head.workspace_bytes(wl.T, 1),
        "device_mem_allocated_bytes": mem0,
    }
    print(json.dumps(out), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(inp, wl, rows):
    """The fp64 oracle, as it stands, on a slice of `rows` valid tokens of the
    same workload (full forward + backward including the V x D dW)."""
    from oracle import streambp_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 0) for i in threadpool_info()), default=os.cpu_count())
    except Exception:
        cores = os.cpu_count()
    valid = np.nonzero(inp.labels != -100)[0]
    lo = int(valid[0]) if valid.size else 0
    sl = slice(lo, min(wl.T, lo + rows))
    n = sl.stop - sl.start
    print(f"[bench] cpu oracle on rows {sl.start}..{sl.stop}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    O.sft(inp.H[sl], inp.W, inp.labels[sl])
    t = time.perf_counter() - t0
    return {"value": round(n / t, 2), "unit": "tokens/s", "cores": int(cores), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"rows {sl.start}-{sl.stop - 1} of {wl.name} ({n} valid tokens), fp64 numpy, "
                      f"full V x D head forward+backward; {t:.1f} s"}


if __name__ == "__main__":
    main()
