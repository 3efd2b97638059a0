"""Benchmark of the multi-LoRA shrink/expand hot path on one MI355X.

A step is one pass of the whole path over one batch: slot metadata
(lora_prepare_meta), then shrink and expand (lora_apply).  The K steps are
captured once into a HIP graph and the timed region is one replay of it,
bracketed by HIP events on the launch stream: a serving loop launches these
calls the same way, and an eager Python loop would time the host's issue rate
instead (reported separately).  Per-call averages come from graphs holding only
that call.  Inputs are resident in HBM before the timed region starts, and a
1 GiB copy runs right before every timed replay, so no timed step finds its
data in the 256 MB last-level cache (MALL) or the L2s, whatever K is; enough
copies of the inputs are rotated that consecutive steps of one replay do not
either.

Default workload: prefill (SGMV form) on a fused gate/up shape, 4096 -> 2 x
14336, rank 64, 8 slots, 16 requests of 128..2048 tokens (17 705 tokens), bf16.
The decode workloads (q_proj 4096 -> 4096 at rank 16, 256 tokens; down_proj
14336 -> 4096 at rank 64, 4096 tokens over 128 slots) are measured in the same
run and reported under "extra", each with its own roofline.

One JSON line on stdout:  value = tokens per second of the whole step (all T
tokens of the batch, including those without an adapter), plus the roofline
of the dominant call (algorithmic bytes / measured average duration against
the 8 TB/s HBM peak, with the bf16 matrix-core rate from counters beside it),
a measured device copy rate, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA shrink+expand tokens/s; % HBM peak (decode) / % bf16 MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3,
                    help="workload 1..8 (3 = prefill gate/up, the headline; 2, 5 = decode; 7, 8 = MoE experts' LoRA)")
    ap.add_argument("--extra", default="2,4,5,6,7,8",
                    help="comma-separated workloads also measured and reported under 'extra' ('' for none)")
    ap.add_argument("--mode", default="auto", choices=["auto", "bgmv", "sgmv"])
    ap.add_argument("--slot-ranks", action="store_true",
                    help="pass each slot's own rank (the kernels then skip the zero-padded ranks)")
    ap.add_argument("--a-rank-rows", action="store_true",
                    help="hand A over rank-major ([S][r][d_in], the pages' A layout), so that with --slot-ranks "
                         "the ranks past a slot's own are whole rows that are never fetched")
    ap.add_argument("--b-out-rows", action="store_true",
                    help="hand B over output-major ([S][w][r], the pages' stacked B layout); lora_apply then runs "
                         "the tile shrink and the matrix-core expand")
    ap.add_argument("--rotate-mb", type=float, default=640.0,
                    help="total size of the rotated input copies (beats the 256 MB MALL)")
    ap.add_argument("--flush-mb", type=float, default=1024.0,
                    help="size of the copy run before every timed replay (evicts the MALL and the L2s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: every host core)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run under rocprofv3 --pmc: a plain copy of known size, then --steps eager steps")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of --pmc-pass (FETCH_SIZE, WRITE_SIZE) into the "
                         "traffic summary under profiles/")
    ap.add_argument("--summarize-mfma", metavar="MFMA_DIR",
                    help="turn a rocprofv3 --pmc run of --pmc-pass (SQ_INSTS_VALU_MFMA_MOPS_BF16 MfmaUtil) "
                         "into the matrix-core summary under profiles/")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_JSON"),
                    help="turn a rocprofv3 --kernel-trace --stats run of this bench (and its JSON line) into "
                         "the trace summary under profiles/")
    ap.add_argument("--phase-budget", metavar="OUT_MD",
                    help="build the library with the split kernel's phase clock (-DLORA_PHASE_CLOCK) into a "
                         "temporary directory, run --steps cold steps of the workload on it and write the "
                         "per-phase latency budget of the one-slice split kernel to OUT_MD")
    ap.add_argument("--tile-phase-budget", metavar="OUT_MD",
                    help="the same measurement build, for the tile shrink and the tile expand of the workload: "
                         "their items' timing per workgroup, written to OUT_MD")
    return ap.parse_args()


PMC_COPY_ELEMS = 64 << 20   # bf16 elements of the calibration copy (128 MiB read, 128 MiB written)
PROFILES = os.path.join(ROOT, "profiles")


def rel(path):
    """A path as given on the command line, relative to the repository root
    when it lies inside it (for the commands recorded in profiles/)."""
    a = os.path.abspath(path)
    return os.path.relpath(a, ROOT) if a.startswith(ROOT + os.sep) else path


KERNEL_SOURCES = {   # the sources each measured kernel is built from
    "bgmv_split": ["lora_bgmv_split.hip"],
    "bgmv_fused_kernel": ["lora_bgmv.hip"],
    "shrink+expand": ["lora_shrink.hip", "lora_expand.hip"],
    "shrink+u_planes+expand_rows": ["lora_shrink.hip", "lora_expand.hip"],
}


def source_digest(kernel_key):
    """Hash of the code of one kernel (its file, the shared device headers,
    the C header), comments and blank lines left out: a traffic figure is only
    reported while the code it was measured on is unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "segmented_gather_rank_amd", "csrc")
    files = [os.path.join(csrc, f) for f in KERNEL_SOURCES[kernel_key] + ["lora_common.h", "lora_host.h"]]
    files += [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))]
    for f in files:
        text = re.sub(r"/\*.*?\*/", "", open(f, encoding="utf-8").read(), flags=re.S)
        code = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
        h.update(os.path.basename(f).encode())
        h.update("\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()[:16]


class MoeFlat:
    """An MoE step seen as the plain batch the kernels run: one row per
    (token, choice) pair whose slot is its (slot, local expert) key, factors
    stacked [S * E_local][...].  Used for the byte accounting and kernel
    choice; the keys themselves are computed on the device by the library."""

    def __init__(self, c):
        import numpy as np
        self.moe = c
        e = c.topk_ids.reshape(-1).astype(np.int64)
        tok = np.repeat(np.arange(c.T), c.topk)
        slot = c.token_slot[tok]
        le = c.expert_map[e] if c.expert_map is not None else e
        self.token_slot = np.where((slot >= 0) & (le >= 0), slot * c.num_local_experts + le, -1).astype(np.int32)
        self.T = c.rows
        self.num_slots = c.num_slots * c.num_local_experts
        self.n_slices, self.d_in, self.r_max, self.widths = c.n_slices, c.d_in, c.r_max, c.widths
        self.dtype, self.name, self.scale, self.offsets = c.dtype, c.name, c.scale, c.offsets
        self.ranks = np.repeat(np.asarray(c.ranks, np.int32), c.num_local_experts)
        # x rows the step must read: tokens with a keyed pair (gate/up), or keyed pairs (down)
        keyed = self.token_slot >= 0
        self.x_rows = int(keyed.sum()) if c.x_per_pair else int(np.unique(tok[keyed]).shape[0])


def dominant_kernel(c, mode, b_out_rows=False):
    """Name (substring) of the kernel that lora_apply runs on this workload."""
    if b_out_rows:   # output-major B: the tile kernels only
        return "shrink+expand"
    sw = sum(c.widths)
    e = 4 if c.dtype == "f32" else 2
    w_tok = (c.n_slices * c.d_in + sw) * c.r_max * e
    enabled = os.environ.get("LORA_DISABLE_FUSED_BGMV", "0") in ("", "0")
    decode = mode != "sgmv" and (mode == "bgmv" or c.T <= 16 * c.num_slots)
    if enabled and decode and split_takes(c):
        return "bgmv_split"
    if enabled and decode and sw // 8 <= 1024 and c.d_in * e <= 32768 and w_tok <= (1 << 20):
        return "bgmv_fused_kernel"
    if rows_takes(c, mode):
        return "shrink+u_planes+expand_rows"
    return "shrink+expand"


def rows_takes(c, mode):
    """Whether the call's expand runs on the long-segment kernel: bf16, AUTO or
    SGMV, at least 64 tokens per possible segment, and y and the rank rows
    within its 32-bit buffer offsets (LORA_EXPAND_ROWS=0/1 forces it)."""
    force = os.environ.get("LORA_EXPAND_ROWS", "")
    if c.dtype != "bf16" or mode == "bgmv":
        return False
    if force:
        ok = int(force) > 0
    else:
        ok = c.T >= 64 * (c.num_slots + 1)
    ldy = getattr(c, "ldy", None) or max(o + w for o, w in zip(c.offsets, c.widths))
    y_end = max(o + w for o, w in zip(c.offsets, c.widths))
    y_bytes = ((c.T - 1) * ldy + y_end) * 2
    return ok and y_bytes + 4096 < 0x7FFFFFF0 and c.n_slices * c.T * c.r_max * 2 < (1 << 30)


def split_takes(c):
    """Whether a decode-shaped call runs the split kernel (each work tile spread
    over several workgroups): bf16, and some member count of at most 16 gives
    every member an A chunk and a B share that fit its LDS.  Up to four slices
    run side by side (one slice per workgroup: A chunk <= 512 rows, 1024 at
    rank <= 16; the widest slice sets the B share); more slices share each
    workgroup (every slice's A chunk, <= 512 rows)."""
    if c.dtype != "bf16" or os.environ.get("LORA_DISABLE_SPLIT_BGMV", "0") not in ("", "0"):
        return False
    rp = max(16, c.r_max)
    if c.T * c.n_slices * rp > (1 << 17):
        return False
    side = c.n_slices <= 4
    if not side and (1 << (c.n_slices - 1).bit_length()) * (rp // 16) > 8:
        return False
    blocks = [(w + 15) // 16 for w in c.widths]
    nbt = max(blocks) if side else sum(blocks)
    a_slices = 1 if side else c.n_slices
    kc_max = 1024 if side and c.r_max <= 16 else 512
    g = 1
    while g <= 16:
        kc = max(128, 1 << max(0, (-(-c.d_in // g) - 1).bit_length()))
        bpm = -(-nbt // g)
        if kc <= kc_max and a_slices * kc * (rp // 8) <= 2048 and bpm <= 32 and bpm * 2 * rp <= 2048:
            return True
        g *= 2
    return False


def kernel_keys(kernel_key):
    """Substrings of the kernel names that make up one lora_apply launch."""
    return kernel_key.split("+")


def variant(args):
    """(file-name suffix, command-line flags) of the weight options of a run."""
    flags = [f for f, on in (("--slot-ranks", args.slot_ranks), ("--a-rank-rows", args.a_rank_rows),
                             ("--b-out-rows", args.b_out_rows)) if on]
    return "".join("_" + f[2:].replace("-", "_") for f in flags), "".join(" " + f for f in flags)


def traffic_file(c, args):
    return os.path.join(PROFILES, f"traffic_{c.name}{variant(args)[0]}.md")


def read_traffic(c, kernel_key, args):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is missing or was taken on other kernel sources."""
    try:
        text = open(traffic_file(c, args)).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if line.startswith("- ") and ": " in line)
    if fields.get("- kernel sources") != source_digest(kernel_key):
        return None
    return int(fields["- traffic bytes per launch"])


def summarize_pmc(c, k, fetch_dir, write_dir, kernel_key, args):
    """FETCH_SIZE / WRITE_SIZE per dispatch (KiB) of the dominant kernel, scaled
    by what the same counters read for the calibration copy."""
    import csv
    import glob

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert f, f"no counter_collection.csv under {d}"
        vals = {}
        for r in csv.DictReader(open(f[0])):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        copy = [v for k, v in vals.items() if "neg" in k.lower()]
        kern = [v for k, v in vals.items() if any(key in k for key in kernel_keys(kernel_key))]
        assert copy and kern, (counter, list(vals))
        copy_kib = sum(copy[0]) / len(copy[0])
        # one apply = one dispatch of each of its kernels: sum their per-dispatch means
        kern_kib = sum(sum(v) / len(v) for v in kern)
        out[counter] = (kern_kib, copy_kib, min(len(v) for v in kern))
    nbytes = PMC_COPY_ELEMS * 2
    f_r = nbytes / (out["FETCH_SIZE"][1] * 1024)
    f_w = nbytes / (out["WRITE_SIZE"][1] * 1024)
    traffic = out["FETCH_SIZE"][0] * 1024 * f_r + out["WRITE_SIZE"][0] * 1024 * f_w
    alg = algorithmic(c, args.slot_ranks)
    alg_b = alg["shrink_bytes"] + alg["expand_bytes"]
    sfx, fl = variant(args)
    lines = [
        f"# HBM traffic of `{kernel_key}` on workload {c.name}{fl}",
        "",
        "Two rocprofv3 counter runs of `bench.py --pmc-pass` (a bf16 negation of "
        f"{PMC_COPY_ELEMS} elements as the plain copy of known size, then the workload's steps):",
        "",
        "```",
        "export TMPDIR=/tmp",
        f"rocprofv3 --pmc FETCH_SIZE -d {rel(fetch_dir)} -o p --output-format csv -- python bench.py --config {k} --pmc-pass --steps 200{fl}",
        f"rocprofv3 --pmc WRITE_SIZE -d {rel(write_dir)} -o p --output-format csv -- python bench.py --config {k} --pmc-pass --steps 200{fl}",
        f"python bench.py --config {k} --summarize-pmc {rel(fetch_dir)} {rel(write_dir)}{fl}",
        "```",
        "",
        f"| Counter | `{kernel_key}` KiB/dispatch | copy KiB/dispatch | copy bytes | scale |",
        "|---|---|---|---|---|",
        f"| FETCH_SIZE | {out['FETCH_SIZE'][0]:.1f} (n={out['FETCH_SIZE'][2]}) | {out['FETCH_SIZE'][1]:.1f} | {nbytes} | {f_r:.4f} |",
        f"| WRITE_SIZE | {out['WRITE_SIZE'][0]:.1f} (n={out['WRITE_SIZE'][2]}) | {out['WRITE_SIZE'][1]:.1f} | {nbytes} | {f_w:.4f} |",
        "",
        f"Scaled traffic {traffic / 1e6:.3f} MB per launch against {alg_b / 1e6:.3f} MB algorithmic "
        f"({traffic / alg_b:.3f}x)" + ("" if not args.slot_ranks else
                                       f"; the same workload without per-slot ranks moves "
                                       f"{sum(algorithmic(c)[q] for q in ('shrink_bytes', 'expand_bytes')) / 1e6:.3f} MB "
                                       f"algorithmic") + ".",
        "",
        f"- kernel sources: {source_digest(kernel_key)}",
        f"- traffic bytes per launch: {int(round(traffic))}",
        "",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    open(traffic_file(c, args), "w").write("\n".join(lines))
    print("\n".join(lines))


def algorithmic(c, ranked=False):
    """Bytes and flops the method must move/compute for one batch (per kernel).

    A and B slot blocks of every distinct slot used are read once; x rows of
    tokens with an adapter are read once (for an MoE step, the distinct x rows
    its keyed pairs use); the y windows of those tokens are
    read and written once (add into y).  Metadata and the fp32 rank-r buffer
    are overheads and are not counted.  r is the padded r_max the kernels read,
    or, with per-slot ranks, each slot's own rank rounded up to 8.
    """
    import numpy as np
    ts = c.token_slot
    lora = ts >= 0
    used = np.unique(ts[lora])
    U = int(used.shape[0])
    TL = int(lora.sum())
    e = 4 if c.dtype == "f32" else 2
    sw = sum(c.widths)
    if ranked:
        r_slot = np.minimum(c.r_max, (np.asarray(c.ranks, np.int64) + 7) // 8 * 8)
        r_sum = int(r_slot[used].sum())                 # ranks over the distinct slots
        r_tok = int(r_slot[ts[lora]].sum())             # ranks over the LoRA tokens
    else:
        r_sum, r_tok = U * c.r_max, TL * c.r_max
    x_rows = getattr(c, "x_rows", TL)
    shrink_bytes = r_sum * c.n_slices * c.d_in * e + x_rows * c.d_in * e
    expand_bytes = r_sum * sw * e + TL * sw * e * 2
    shrink_flops = 2 * r_tok * c.n_slices * c.d_in
    expand_flops = 2 * r_tok * sw
    return dict(U=U, T_lora=TL, shrink_bytes=shrink_bytes, expand_bytes=expand_bytes,
                shrink_flops=shrink_flops, expand_flops=expand_flops)


def _counter_means(d, counter):
    """Per-kernel lists of one counter's per-dispatch values from a rocprofv3
    --pmc run (csv output) under directory d."""
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert f, f"no counter_collection.csv under {d}"
    vals = {}
    for r in csv.DictReader(open(f[0])):
        if r["Counter_Name"] == counter:
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def mfma_file(c):
    return os.path.join(PROFILES, f"mfma_{c.name}.md")


def summarize_mfma(c, k, d, kernel_key):
    """bf16 matrix-core operations per launch of the dominant call (the sum over
    its kernels of SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per dispatch) and the
    derived MfmaUtil (matrix-core busy cycles over all SIMDs and the busy time)."""
    mops = _counter_means(d, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    util = _counter_means(d, "MfmaUtil")
    keys = kernel_keys(kernel_key)
    rows, flops = [], 0.0
    for name, v in sorted(mops.items()):
        if not any(key in name for key in keys):
            continue
        f = 512.0 * sum(v) / len(v)
        u = util.get(name, [float("nan")])
        flops += f
        rows.append(f"| `{name[:90]}` | {len(v)} | {f / 1e9:.3f} | {sum(u) / len(u):.2f} |")
    assert rows, list(mops)
    alg = algorithmic(c)
    alg_f = alg["shrink_flops"] + alg["expand_flops"]
    lines = [
        f"# bf16 matrix-core work of `{kernel_key}` on workload {c.name}",
        "",
        "One rocprofv3 counter run of `bench.py --pmc-pass` (the workload's steps, eager):",
        "",
        "```",
        "export TMPDIR=/tmp",
        f"rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 MfmaUtil -d {rel(d)} -o p --output-format csv -- "
        f"python bench.py --config {k} --pmc-pass --steps 20",
        f"python bench.py --config {k} --summarize-mfma {rel(d)}",
        "```",
        "",
        "| Kernel | dispatches | bf16 MFMA GFLOP per dispatch (MOPS x 512) | MfmaUtil % |",
        "|---|---|---|---|",
        *rows,
        "",
        f"Per launch {flops / 1e9:.3f} GFLOP issued on the matrix cores against {alg_f / 1e9:.3f} GFLOP algorithmic "
        f"({flops / alg_f:.2f}x; above 1 where a kernel multiplies the rank-r rows as bf16 high and low parts, or "
        "pads a short tile to a whole 16-token block).",
        "The bench divides the issued figure by its own measured duration of the call.",
        "",
        f"- kernel sources: {source_digest(kernel_key)}",
        f"- mfma flops per launch: {int(round(flops))}",
        "",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    open(mfma_file(c), "w").write("\n".join(lines))
    print("\n".join(lines))


def read_mfma(c, kernel_key):
    """Matrix-core flops per launch from the committed counter summary, or None
    when it is missing or was taken on other kernel sources."""
    try:
        text = open(mfma_file(c)).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if line.startswith("- ") and ": " in line)
    if fields.get("- kernel sources") != source_digest(kernel_key):
        return None
    return int(fields["- mfma flops per launch"])


def summarize_trace(c, k, d, bench_json, kernel_key, args):
    """rocprofv3 --kernel-trace --stats summary of a bench run (the stats csv)
    next to the bench's own figures for the dominant call."""
    import csv
    import glob
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    assert f, f"no kernel_stats.csv under {d}"
    rows = list(csv.DictReader(open(f[0])))
    b = json.loads(open(bench_json).read().strip().splitlines()[-1])
    sfx, fl = variant(args)
    lines = [f"# Kernel trace: {c.name}{fl}", "", "Command (repository root, one MI355X):", "", "```",
             "export TMPDIR=/tmp",
             f"rocprofv3 --kernel-trace --stats -d {rel(d)} -o t --output-format csv -- "
             f"python bench.py --config {k} --extra '' --no-cpu-baseline{fl} > {rel(bench_json)}",
             f"python bench.py --config {k} --summarize-trace {rel(d)} {rel(bench_json)}{fl}",
             "```", "",
             "Kernel statistics (durations in ns; the step graph is replayed twice and each per-call graph "
             f"{CALL_REPLAYS + 1} times, plus eager warm-up and reference steps and the flush copies):", "",
             "| Kernel | Calls | Average ns | Min ns | Max ns | Share |", "|---|---|---|---|---|---|"]
    apply_ns = 0.0
    for r in rows:
        name = r["Name"]
        avg = float(r["AverageNs"])
        lines.append(f"| `{name[:100]}` | {r['Calls']} | {avg:.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r['Percentage']):.2f} % |")
        if any(key in name for key in kernel_keys(kernel_key)):
            apply_ns += avg
    alg = algorithmic(c, args.slot_ranks)
    ab = alg["shrink_bytes"] + alg["expand_bytes"]
    bus = b["roofline"]["kernel_avg_us"]
    lines += ["",
              f"Trace average of the dominant call `{kernel_key}` (sum of its kernels' averages): "
              f"{apply_ns / 1e3:.3f} us, {ab / (apply_ns * 1e-9) / 1e9:.1f} GB/s = "
              f"{ab / (apply_ns * 1e-9) / 1e9 / HBM_PEAK_GBS:.4f} of 8 TB/s "
              f"({ab} algorithmic bytes per launch).",
              f"The same run's bench line (HIP events around a flushed graph of the calls): {bus:.3f} us, "
              f"frac {b['roofline']['frac']:.4f} ({100 * (bus * 1e3 - apply_ns) / apply_ns:+.1f} % from the trace; "
              "the tracer adds its own time between graph nodes, which the events count and the per-kernel "
              "durations do not).", ""]
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"trace_{c.name}{sfx}.md")
    open(out, "w").write("\n".join(lines))
    print("\n".join(lines))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(c, seconds, threads):
    """The oracle as it stands (plain C, fp64) on a bounded sample of the same
    workload: whole batches, metadata plus every token's delta, until `seconds`
    have passed.  The oracle's calls run on `threads` host threads at once,
    each on its own chunk of rows (the C calls release the interpreter lock);
    the oracle itself is unchanged.  An MoE step is counted in tokens: a token
    is done when all its top-k pairs are."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle
    moe = getattr(c, "moe", None)
    T = c.T if moe is None else moe.T
    rows_per_call = max(1, min(T, 16 if moe is None else 4))
    deadline = [None]

    def rows_of(r0):
        return np.arange(r0, min(T, r0 + rows_per_call))

    def work(r0):
        if time.perf_counter() > deadline[0]:
            return 0
        rows = rows_of(r0)
        if moe is None:
            oracle.lora_rows(c.x, c.token_slot, c.num_slots, c.A, c.B, c.offsets, c.scale, c.y0, rows=rows)
        else:
            pairs = (rows[:, None] * moe.topk + np.arange(moe.topk)).reshape(-1)
            oracle.moe_rows(moe.x, moe.topk_ids, moe.token_slot, moe.num_slots, moe.num_experts,
                            moe.num_local_experts, moe.A, moe.B, moe.offsets, moe.scale, moe.y0,
                            expert_map=moe.expert_map, x_per_pair=moe.x_per_pair, rows=pairs)
        return rows.shape[0]

    oracle.load()
    done = 0
    t0 = time.perf_counter()
    deadline[0] = t0 + seconds
    with ThreadPoolExecutor(threads) as pool:
        while time.perf_counter() < deadline[0]:
            if moe is None:
                oracle.prepare_meta(c.token_slot, c.num_slots)
            else:
                oracle.prepare_meta(oracle.moe_keys(moe.topk_ids, moe.token_slot, moe.num_slots, moe.num_experts,
                                                    moe.num_local_experts, moe.expert_map), c.num_slots)
            done += sum(pool.map(work, range(0, T, rows_per_call)))
    dt = time.perf_counter() - t0
    return dict(value=round(done / dt, 2), unit="tokens/s", cores=threads, kind="oracle", cpu_model=cpu_model(),
                sample=f"{done} tokens of workload '{c.name}' (metadata + fp64 delta of every token, batches of "
                       f"{T}, {rows_per_call} rows per oracle call) in {dt:.1f} s on {threads} host threads")


def load_case(k):
    import workloads as W
    c = W.config(k)
    moe = None
    if isinstance(c, W.MoeCase):
        moe, c = c, MoeFlat(c)
    return c, moe


class Flush:
    """A copy of flush_mb MiB (half read, half written) run before a timed
    region, so that no input of the timed steps is left in the MALL or an L2."""

    def __init__(self, torch, dev, mb):
        n = max(1, int(mb * 2 ** 20 / 2))
        self.src = torch.ones(n // 2, dtype=torch.uint8, device=dev)
        self.dst = torch.empty_like(self.src)

    def __call__(self):
        self.dst.copy_(self.src)


def copy_rate_gbs(torch, dev):
    """Device copy rate: a 1 GiB copy, best of 5, timed with HIP events
    (2 GiB moved per copy)."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    best = float("inf")
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    return 2 * n / (best * 1e-3) / 1e9


CALL_REPLAYS = 5   # timed replays of each per-call graph (their median is reported)


def measure(c, moe, args, L, torch, dev, flush, K, warmup):
    """Graph-timed step, metadata and apply of one workload; returns the
    figures of its JSON line (roofline of lora_apply included)."""
    import numpy as np

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    alg = algorithmic(c, args.slot_ranks)
    if moe is None:
        A_host = [np.transpose(a, (0, 2, 1)) for a in c.A] if args.a_rank_rows else c.A
        B_host = [np.transpose(b, (0, 2, 1)) for b in c.B] if args.b_out_rows else c.B
        base = dict(ts=torch.from_numpy(c.token_slot).to(dev), x=to_dev(c.x),
                    A=[to_dev(a) for a in A_host], B=[to_dev(b) for b in B_host], y=to_dev(c.y0))
    else:
        SE = c.num_slots
        base = dict(ts=torch.from_numpy(moe.token_slot).to(dev), x=to_dev(moe.x),
                    A=[to_dev(a).view(SE, *a.shape[2:]) for a in moe.A],
                    B=[to_dev(np.transpose(b, (0, 1, 3, 2)) if args.b_out_rows else b).view(
                        SE, *(b.shape[:1:-1] if args.b_out_rows else b.shape[2:])) for b in moe.B],
                    y=to_dev(moe.y0),
                    topk=torch.from_numpy(moe.topk_ids).to(dev),
                    emap=None if moe.expert_map is None else torch.from_numpy(moe.expert_map).to(dev))
    set_bytes = sum(t.numel() * t.element_size()
                    for t in [base["ts"], base["x"], base["y"], *base["A"], *base["B"]])
    nrot = max(1, min(64, int(np.ceil(args.rotate_mb * 2 ** 20 / set_bytes))))
    sets = [base] + [{k: (None if v is None else [a.clone() for a in v] if isinstance(v, list) else v.clone())
                      for k, v in base.items()} for _ in range(nrot - 1)]
    dtype = base["x"].dtype
    r = c.r_max
    ap_need = L.lora_apply_workspace_bytes(c.T, c.num_slots, c.d_in, c.n_slices, r, dtype, args.mode)
    mws_bytes = (L.lora_meta_workspace_bytes(c.T, c.num_slots) if moe is None else
                 L.lora_moe_meta_workspace_bytes(moe.T, moe.topk, moe.num_slots, moe.num_local_experts))
    for s in sets:
        s["mws"] = torch.empty(mws_bytes, dtype=torch.uint8, device=dev)
        s["aws"] = L.apply_workspace(ap_need, dev)

    metas = [None] * nrot
    ranks = torch.from_numpy(np.asarray(c.ranks, np.int32)).to(dev) if args.slot_ranks else None

    def meta_call(i):
        s = sets[i % nrot]
        if moe is None:
            metas[i % nrot] = L.lora_prepare_meta(s["ts"], c.num_slots, workspace=s["mws"])
        else:
            m = L.lora_prepare_moe_meta(s["topk"], s["ts"], moe.num_slots, moe.num_experts,
                                        moe.num_local_experts, s["emap"], workspace=s["mws"])
            metas[i % nrot] = m.with_x_row_div(1) if moe.x_per_pair else m

    def apply_call(i):
        s = sets[i % nrot]
        L.lora_apply(metas[i % nrot], s["x"], s["A"], s["B"], c.offsets, s["y"], scale=c.scale,
                     add=True, mode=args.mode, workspace=s["aws"], slot_rank=ranks, a_rank_rows=args.a_rank_rows,
                     b_out_rows=args.b_out_rows)

    def step(i):
        meta_call(i)
        apply_call(i)

    # eager warm-up (also builds every set's metadata once)
    for i in range(max(warmup, nrot)):
        step(i)
    torch.cuda.synchronize()

    def capture(fn, n):
        """HIP graph of n calls of fn, as a serving loop would launch them."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        return g

    def time_graph(g):
        g.replay()                       # first replay (uploads the graph)
        flush()                          # nothing the timed replay reads stays cached
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    g_step = capture(step, K)
    g_meta = capture(meta_call, K)
    g_apply = capture(apply_call, K)
    t_host0 = time.perf_counter()
    total_ms = time_graph(g_step)           # the timed region: exactly K steps
    t_host = time.perf_counter() - t_host0
    # per-call figures: the median of CALL_REPLAYS replays, each after a flush
    meta_us = 1e3 * float(np.median([time_graph(g_meta) for _ in range(CALL_REPLAYS)])) / K
    apply_us = 1e3 * float(np.median([time_graph(g_apply) for _ in range(CALL_REPLAYS)])) / K
    del g_step, g_meta, g_apply

    # the same steps issued eagerly from Python, for reference (host-issue bound)
    flush()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_ms_per_step = e0.elapsed_time(e1) / K
    # the split decode kernel's rendezvous counters, summed over the sets'
    # workspaces: waits that gave up, and flags met from another XCD (both
    # mean a member computed a peer's partials itself)
    n_apply = max(warmup, nrot) + 2 + 4 * K + K
    rdv = {"apply_calls": n_apply, "waits_gave_up": 0, "flags_from_other_xcd": 0}
    for s in sets:
        cnt = L.apply_workspace_counters(s["aws"])
        rdv["waits_gave_up"] += cnt["gave_up"]
        rdv["flags_from_other_xcd"] += cnt["other_xcd"]
    del sets, metas
    torch.cuda.empty_cache()

    ms_per_step = total_ms / K
    tokens = c.T if moe is None else moe.T       # an MoE step's tokens (each with top-k pairs)
    key = dominant_kernel(c, args.mode, args.b_out_rows)
    d_bytes = alg["shrink_bytes"] + alg["expand_bytes"]
    d_flops = alg["shrink_flops"] + alg["expand_flops"]
    achieved = d_bytes / (apply_us * 1e-6) / 1e9
    mf = None if args.slot_ranks or args.a_rank_rows or args.b_out_rows else read_mfma(c, key)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(c, key, args),
                "traffic_unit": "bytes per launch", "kernel": "lora_apply (" + key + ")",
                "kernel_avg_us": round(apply_us, 3), "algorithmic_bytes_per_launch": int(d_bytes),
                "mfma_bf16": {"algorithmic_tflops": round(d_flops / (apply_us * 1e-6) / 1e12, 2),
                              "algorithmic_frac": round(d_flops / (apply_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                              "issued_tflops": None if mf is None else round(mf / (apply_us * 1e-6) / 1e12, 2),
                              "issued_frac": None if mf is None else round(
                                  mf / (apply_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                              "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                              "issued_from": "rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per launch (profiles/)"}}
    config = {"workload": c.name, "tokens": tokens,
              **({} if moe is None else {"topk": moe.topk, "pairs": c.T, "experts": moe.num_experts,
                                         "local_experts": moe.num_local_experts,
                                         "adapter_slots": moe.num_slots}),
              "tokens_with_adapter" if moe is None else "keyed_pairs": alg["T_lora"],
              "distinct_slots" if moe is None else "distinct_keys": alg["U"],
              "slots": c.num_slots, "d_in": c.d_in,
              "slice_widths": c.widths, "r_max": r, "mode": args.mode,
              "slot_ranks": bool(args.slot_ranks), "a_rank_rows": bool(args.a_rank_rows),
              "b_out_rows": bool(args.b_out_rows),
              "rotated_input_sets": nrot, "flush_mb_before_timed_replay": args.flush_mb,
              "parallelism": "single GPU"}
    return {
        "value": round(tokens * K / (total_ms / 1e3), 1), "ms_per_step": round(ms_per_step, 5),
        "dtype": "bf16" if c.dtype == "bf16" else "f32", "config": config, "roofline": roofline,
        "calls_us": {"lora_prepare_meta": round(meta_us, 3), "lora_apply": round(apply_us, 3),
                     "lora_prepare_meta_per_layer_of_32": round(meta_us / 32, 3),
                     "timed_as": f"a HIP graph of K calls of one kind, the median of {CALL_REPLAYS} replays, "
                                 "each after a flushing copy"},
        "step": {"algorithmic_bytes": int(d_bytes),
                 "hbm_frac": round(d_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_bf16_frac": round(d_flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
                 "timed_as": "one HIP graph of the K steps, replayed once after a flushing copy",
                 "host_wall_s": round(t_host, 4), "eager_ms_per_step": round(eager_ms_per_step, 5)},
        **({"split_rendezvous": rdv} if key.startswith("bgmv_split") else {}),
    }


PHASES = ["launch spread (start - first start)", "tile header (1 - 0)", "A chunk in LDS (2 - 1)",
          "rest of batch, shrink, partials stored, B staged (3 - 2)",
          "rendezvous: the members' first-block partials polled in (4 - 3)",
          "sum of the first block's u (5 - 4)", "expand, y stores acknowledged (6 - 5)",
          "workgroup total (6 - 0)", "end (6 - first start)"]


def phase_budget(c, args, out_md):
    """Per-phase latency of the one-slice split kernel, from its own clock.

    The measurement build records, per workgroup, the 100 MHz real-time counter
    at the kernel's phase boundaries (csrc/lora_bgmv_split.hip, LORA_PHASE_CLOCK).
    Each of --steps steps is one flushing copy, the metadata and lora_apply,
    as in the timed graph; the records of the workgroups that had work are
    read back after each step."""
    import importlib.util
    import tempfile

    import numpy as np

    spec = importlib.util.spec_from_file_location(
        "_lora_hip_build", os.path.join(ROOT, "segmented_gather_rank_amd", "build.py"))
    hb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(hb)
    tmp = tempfile.mkdtemp(prefix="lora_phase_")
    lib = hb.build(out=os.path.join(tmp, "liblora_mi355x_phase.so"), extra=["-DLORA_PHASE_CLOCK"])
    os.environ["LORA_MI355X_LIB"] = lib
    import ctypes

    import torch

    import segmented_gather_rank_amd as L
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    words = 10
    clk = torch.zeros(words * 8192, dtype=torch.int64, device=dev)
    L._cdll.lora_debug_phase_clock.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L._cdll.lora_debug_phase_clock(ctypes.c_void_p(clk.data_ptr()), clk.numel())
    ts, x, y = torch.from_numpy(c.token_slot).to(dev), to_dev(c.x), to_dev(c.y0)
    A, B = [to_dev(a) for a in c.A], [to_dev(b) for b in c.B]
    ws = L.apply_workspace(L.lora_apply_workspace_bytes(c.T, c.num_slots, c.d_in, c.n_slices, c.r_max,
                                                        x.dtype, args.mode), dev)
    mws = torch.empty(L.lora_meta_workspace_bytes(c.T, c.num_slots), dtype=torch.uint8, device=dev)
    flush = Flush(torch, dev, args.flush_mb)
    rows, spans_ev = [], []
    xcc_total = xcc_match = 0
    for it in range(args.warmup + args.steps):
        flush()
        clk.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m = L.lora_prepare_meta(ts, c.num_slots, workspace=mws)
        e0.record()
        L.lora_apply(m, x, A, B, c.offsets, y, scale=c.scale, add=True, mode=args.mode, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        if it < args.warmup:
            continue
        r = clk.cpu().numpy().reshape(-1, words)
        # the record's index is the workgroup's flat index (blockIdx.y * gridDim.x + blockIdx.x);
        # every slice's row of the grid is a multiple of 8 wide, so blockIdx.x mod 8 = index mod 8
        live_idx = np.nonzero(r[:, 0] != 0)[0]
        xcc_total += live_idx.shape[0]
        xcc_match += int(np.sum(r[live_idx, 9] == live_idx % 8))
        r = r[r[:, 0] != 0]
        if r.shape[0] == 0:
            raise SystemExit("the split kernel did not run (no phase records): not a split-kernel workload")
        t = r[:, :7].astype(np.float64) * 10.0 / 1000.0   # 100 MHz ticks -> us
        first = t[:, 0].min()
        rows.append(np.stack([t[:, 0] - first, t[:, 1] - t[:, 0], t[:, 2] - t[:, 1], t[:, 3] - t[:, 2],
                              t[:, 4] - t[:, 3], t[:, 5] - t[:, 4], t[:, 6] - t[:, 5], t[:, 6] - t[:, 0],
                              t[:, 6] - first], axis=1))
        spans_ev.append(e0.elapsed_time(e1) * 1e3)
    allr = np.concatenate(rows)
    ends = np.array([rr[:, 8].max() for rr in rows])
    crit = np.stack([rr[int(np.argmax(rr[:, 8]))] for rr in rows])   # the last workgroup of each step
    lines = [f"# Phase budget of the one-slice split kernel: {c.name}", "",
             "Command (repository root, one MI355X):", "", "```",
             f"python bench.py --config {args.config} --steps {args.steps} --warmup {args.warmup} "
             f"--phase-budget {out_md}", "```", "",
             "The library is rebuilt with `-DLORA_PHASE_CLOCK`: each workgroup of the kernel writes the 100 MHz "
             "real-time counter at its phase boundaries (10 ns resolution). Each step is a 1 GiB flushing copy, "
             "`lora_prepare_meta`, then `lora_apply`, as in the timed graph. "
             f"{args.steps} steps, {allr.shape[0] // len(rows)} workgroups with work per step.", "",
             "| Phase (us) | median | p90 | max | last workgroup (median) |", "|---|---|---|---|---|"]
    for i, name in enumerate(PHASES):
        col = allr[:, i]
        lines.append(f"| {name} | {np.median(col):.2f} | {np.percentile(col, 90):.2f} | {col.max():.2f} | "
                     f"{np.median(crit[:, i]):.2f} |")
    lines += ["", f"First start to last end, median over steps: {np.median(ends):.2f} us "
              f"(p90 {np.percentile(ends, 90):.2f}). HIP events around the lora_apply launch of the same steps: "
              f"median {np.median(spans_ev):.2f} us (these add the launch and the gap before the first "
              f"workgroup starts).", "",
              f"XCD placement: the hardware register XCC_ID equals blockIdx mod 8 in {xcc_match} of {xcc_total} "
              f"workgroup records (the split kernel assumes it for a tile's members, and computes a peer's "
              f"partials itself when a peer's tags name another XCD)."]
    os.makedirs(os.path.dirname(os.path.abspath(out_md)), exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def tile_phase_budget(c, moe, args, out_md):
    """Timing of the tile shrink's items and of the tile expand's phases, from
    their own clocks in the measurement build (LORA_PHASE_CLOCK; the kernel
    that records is chosen with LORA_PHASE_KERNEL).  Each of --steps steps is
    one flushing copy, the metadata and lora_apply, as in the timed graph,
    once with the shrink recording and once with the expand recording."""
    import ctypes
    import importlib.util
    import tempfile

    import numpy as np

    if moe is not None:
        raise SystemExit("--tile-phase-budget takes a plain (non-MoE) workload")
    spec = importlib.util.spec_from_file_location(
        "_lora_hip_build", os.path.join(ROOT, "segmented_gather_rank_amd", "build.py"))
    hb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(hb)
    tmp = tempfile.mkdtemp(prefix="lora_phase_")
    os.environ["LORA_MI355X_LIB"] = hb.build(out=os.path.join(tmp, "liblora_mi355x_phase.so"),
                                             extra=["-DLORA_PHASE_CLOCK"])
    import torch

    import segmented_gather_rank_amd as L
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    words = 16   # 64-bit words per workgroup record (kTilePhaseWords)
    clk = torch.zeros(words * 8192, dtype=torch.int64, device=dev)
    L._cdll.lora_debug_phase_clock.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L._cdll.lora_debug_phase_clock(ctypes.c_void_p(clk.data_ptr()), clk.numel())
    ts, x, y = torch.from_numpy(c.token_slot).to(dev), to_dev(c.x), to_dev(c.y0)
    A, B = [to_dev(a) for a in c.A], [to_dev(b) for b in c.B]
    ws = L.apply_workspace(L.lora_apply_workspace_bytes(c.T, c.num_slots, c.d_in, c.n_slices, c.r_max,
                                                        x.dtype, args.mode), dev)
    mws = torch.empty(L.lora_meta_workspace_bytes(c.T, c.num_slots), dtype=torch.uint8, device=dev)
    flush = Flush(torch, dev, args.flush_mb)

    def records(kernel):
        os.environ["LORA_PHASE_KERNEL"] = kernel
        out = []
        for it in range(args.warmup + args.steps):
            flush()
            clk.zero_()
            m = L.lora_prepare_meta(ts, c.num_slots, workspace=mws)
            L.lora_apply(m, x, A, B, c.offsets, y, scale=c.scale, add=True, mode=args.mode, workspace=ws)
            torch.cuda.synchronize()
            if it >= args.warmup:
                r = clk.cpu().numpy().reshape(-1, words).astype(np.float64)
                r = r[(r[:, 0] != 0) & (r[:, 15] != 0)]
                if r.shape[0]:
                    out.append(r)
        os.environ.pop("LORA_PHASE_KERNEL")
        return out

    q = lambda a: f"{np.median(a):.1f} | {np.percentile(a, 90):.1f} | {a.max():.1f}"
    lines = [f"# Tile shrink and tile expand timing: {c.name}", "",
             "Command (repository root, one MI355X):", "", "```",
             f"python bench.py --config {args.config} --steps {args.steps} --warmup {args.warmup} "
             f"--tile-phase-budget {out_md}", "```", "",
             "The library is rebuilt with `-DLORA_PHASE_CLOCK`: the chosen kernel's workgroups write the 100 MHz "
             "real-time counter at their phase boundaries (10 ns resolution). Each step is a 1 GiB flushing copy, "
             "`lora_prepare_meta`, then `lora_apply`; the shrink records in one set of steps, the expand in "
             f"another ({args.steps} each). Times in us from the kernel's first workgroup start; "
             "median | p90 | max over workgroups and steps.", ""]
    # the shrink: items per workgroup and each item's duration
    sh = records("shrink")
    if not sh:
        raise SystemExit("the tile shrink did not run: not a tile-path workload")
    durs, ends, nits, first_d, later_d = [], [], [], [], []
    for r in sh:
        t0 = r[:, 0].min()
        for w in r:
            n = int(w[13])
            nits.append(n)
            ends.append((w[15] - t0) / 100.0)
            for j in range(min(n, 6)):
                d = (w[2 + 2 * j] - w[1 + 2 * j]) / 100.0
                durs.append(d)
                (first_d if j == 0 else later_d).append(d)
    nits, ends = np.array(nits), np.array(ends)
    lines += ["## Tile shrink (`shrink_mma_kernel`)", "",
              f"{sh[0].shape[0]} workgroups; items per workgroup: " +
              ", ".join(f"{int(k)}: {int(v // len(sh))}" for k, v in zip(*np.unique(nits, return_counts=True))) +
              ".", "", "| | median | p90 | max |", "|---|---|---|---|",
              f"| item duration | {q(np.array(durs))} |",
              f"| first item of a workgroup | {q(np.array(first_d))} |"]
    if later_d:
        lines.append(f"| later items | {q(np.array(later_d))} |")
    for n in sorted(set(nits.tolist())):
        lines.append(f"| end, workgroups of {n} item(s) | {q(ends[nits == n])} |")
    spans = [(r[:, 15].max() - r[:, 0].min()) / 100.0 for r in sh]
    busy = [np.sum(r[:, 15] - r[:, 0]) / (r.shape[0] * (r[:, 15].max() - r[:, 0].min())) for r in sh]
    lines += ["", f"Kernel span (first start to last end), median over steps: {np.median(spans):.1f} us; "
              f"workgroups busy {np.median(busy):.2f} of it.", ""]
    # the expand: phases of each workgroup's first item, by the tile's rows
    ex = records("expand")
    if not ex:
        lines += ["The expand of this workload is the long-segment kernel, which does not record."]
    rows_all, hdr, pro, step, end = [], [], [], [], []
    for r in ex:
        t0 = r[:, 0].min()
        for w in r:
            ns, rw = int(w[13]) & 255, (int(w[13]) >> 8) & 255
            k = min(ns, 10)
            rows_all.append(rw)
            hdr.append((w[1] - w[0]) / 100.0)
            pro.append((w[2] - w[1]) / 100.0)
            step.append(np.mean(np.diff(w[2:3 + k])) / 100.0 if k else 0.0)
            end.append((w[15] - t0) / 100.0)
    rows_all, hdr, pro, step, end = map(np.array, (rows_all, hdr, pro, step, end))
    lines += [] if not ex else ["## Tile expand (`expand_mma_kernel`), each workgroup's first item", "",
              f"{ex[0].shape[0]} workgroups per step.", "",
              "| Tile rows | workgroups | header in | prologue | one step | end |", "|---|---|---|---|---|---|"]
    for lo, hi in ((1, 16), (17, 32), (33, 48), (49, 64)):
        mask = (rows_all >= lo) & (rows_all <= hi)
        if mask.any():
            lines.append(f"| {lo}-{hi} | {int(mask.sum() // len(ex))} | {np.median(hdr[mask]):.2f} | "
                         f"{np.median(pro[mask]):.2f} | {np.median(step[mask]):.2f} | {np.median(end[mask]):.1f} |")
    if ex:
        spans = [(r[:, 15].max() - r[:, 0].min()) / 100.0 for r in ex]
        lines += ["", "Medians in us: header in = the tile header's arrival after the workgroup's start; prologue = "
                  "B's first step staged and the tile's rank rows gathered; one step = a step of 128 or more "
                  "columns; end = from the kernel's first start.", "",
                  f"Kernel span (first start to last end), median over steps: {np.median(spans):.1f} us."]
    os.makedirs(os.path.dirname(os.path.abspath(out_md)), exist_ok=True)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU (the path has no multi-GPU stage); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    c, moe = load_case(args.config)
    if args.summarize_pmc:
        summarize_pmc(c, args.config, *args.summarize_pmc, kernel_key=dominant_kernel(c, args.mode, args.b_out_rows),
                      args=args)
        return
    if args.summarize_mfma:
        summarize_mfma(c, args.config, args.summarize_mfma, dominant_kernel(c, args.mode, args.b_out_rows))
        return
    if args.summarize_trace:
        summarize_trace(c, args.config, *args.summarize_trace, dominant_kernel(c, args.mode, args.b_out_rows), args)
        return
    if args.phase_budget:
        phase_budget(c, args, args.phase_budget)
        return
    if args.tile_phase_budget:
        tile_phase_budget(c, moe, args, args.tile_phase_budget)
        return

    import torch

    import segmented_gather_rank_amd as L

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K = args.steps

    if args.pmc_pass:
        import numpy as np

        def to_dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)
        # the calibration copy (reads and writes PMC_COPY_ELEMS bf16 values),
        # then K eager steps; rocprofv3 --pmc collects the counters per dispatch
        src = torch.ones(PMC_COPY_ELEMS, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        src = moe if moe is not None else c
        ts = torch.from_numpy(src.token_slot).to(dev)
        x, y = to_dev(src.x), to_dev(src.y0)
        SE = c.num_slots
        A = [to_dev(a).view(SE, *a.shape[2:]) if moe is not None else
             to_dev(np.transpose(a, (0, 2, 1)) if args.a_rank_rows else a) for a in src.A]
        B = [to_dev(np.transpose(b, (0, 1, 3, 2)) if args.b_out_rows else b).view(
                 SE, *(b.shape[:1:-1] if args.b_out_rows else b.shape[2:])) if moe is not None else
             to_dev(np.transpose(b, (0, 2, 1)) if args.b_out_rows else b) for b in src.B]
        ranks = torch.from_numpy(np.asarray(c.ranks, np.int32)).to(dev) if args.slot_ranks else None
        ws = L.apply_workspace(L.lora_apply_workspace_bytes(c.T, c.num_slots, c.d_in, c.n_slices, c.r_max,
                                                            x.dtype, args.mode), dev)
        for i in range(K):
            if moe is None:
                m = L.lora_prepare_meta(ts, c.num_slots)
            else:
                m = L.lora_prepare_moe_meta(torch.from_numpy(moe.topk_ids).to(dev), ts, moe.num_slots,
                                            moe.num_experts, moe.num_local_experts,
                                            None if moe.expert_map is None else
                                            torch.from_numpy(moe.expert_map).to(dev))
                m = m.with_x_row_div(1) if moe.x_per_pair else m
            L.lora_apply(m, x, A, B, c.offsets, y, scale=c.scale, add=True, mode=args.mode, workspace=ws,
                         slot_rank=ranks, a_rank_rows=args.a_rank_rows, b_out_rows=args.b_out_rows)
        torch.cuda.synchronize()
        print(f"pmc pass done: {K} steps of {c.name}", flush=True)
        return

    flush = Flush(torch, dev, args.flush_mb)
    print(f"bench: workload {c.name}, {K} steps", file=sys.stderr, flush=True)
    head = measure(c, moe, args, L, torch, dev, flush, K, args.warmup)
    extra = {}
    for k in [int(v) for v in args.extra.split(",") if v.strip()]:
        if k == args.config:
            continue
        ck, mk = load_case(k)
        print(f"bench: extra workload {ck.name}", file=sys.stderr, flush=True)
        e = measure(ck, mk, args, L, torch, dev, flush, K, args.warmup)
        extra[ck.name] = {kk: e[kk] for kk in ("value", "ms_per_step", "roofline", "calls_us", "split_rendezvous")
                          if kk in e}
        extra[ck.name]["unit"] = "tokens/s"
        if not args.no_cpu_baseline and k in (1, 2):
            # the small workloads' oracle also on one thread (a few seconds)
            extra[ck.name]["cpu_baseline_one_thread"] = cpu_baseline(ck, 3.0, 1)
        del ck, mk
    del flush
    torch.cuda.empty_cache()
    copy_gbs = copy_rate_gbs(torch, dev)

    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic",
        "config": head["config"], "roofline": head["roofline"], "calls_us": head["calls_us"], "step": head["step"],
        **({"split_rendezvous": head["split_rendezvous"]} if "split_rendezvous" in head else {}),
        "hbm_copy_gbs": {"measured": round(copy_gbs, 1), "peak": HBM_PEAK_GBS,
                         "frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                         "how": "torch copy_ of 1 GiB (2 GiB moved), best of 6, HIP events"},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c, args.cpu_seconds, args.cpu_threads or host_threads())
        if args.config in (1, 2):
            out["cpu_baseline_one_thread"] = cpu_baseline(c, 3.0, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
