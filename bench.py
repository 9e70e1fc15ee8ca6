"""Benchmark: paged-attention decode KV GB/s (% of HBM peak) and seq-tokens/s
on one MI355X.

One step = one decode step through L attention layers: for every layer, the
step's new K/V rows are scatter-written into that layer's paged pool and one
batched attention runs over it, both through paged_attention_append_forward
(equal to kv_append_scatter followed by paged_attention_forward; decode batches
take the new tokens inside the attention launches).
Layers are distinct pool copies sharing one set of block tables, so a step
touches more memory than the 256 MB last-level cache holds and the reported
bandwidth is HBM bandwidth. Block allocation (kv_pool_alloc) happens once per
batch on the host and is timed separately.

Prints one JSON line. --gpus above 1 is refused: the library runs on one GPU
(the path would shard by KV heads or sequences; no collective is built).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "paged-attn decode KV GB/s (% of HBM peak) + seq-tokens/s, 1 GPU"
MIN_FOOTPRINT = 1 << 30        # bytes of pool touched per step


def row_bytes(w):
    """Bytes one token's K (or V) row of one KV head occupies in the pool:
    head_dim elements, or for 8- and 4-bit pools head_dim codes (one or half
    a byte each) and a float32 scale."""
    return {"bf16": 2 * w.head_dim, "f32": 4 * w.head_dim, "fp8": w.head_dim + 4,
            "fp4": w.head_dim // 2 + 4}[w.dtype]


def elem_bytes(w):
    """Bytes of one element of the queries and the new K/V rows."""
    return 4 if w.dtype == "f32" else 2


def unique_kv_bytes(w, tables):
    """K+V bytes of the visible tokens of every distinct physical block, once."""
    seen = {}
    for s, seq in enumerate(w.seqs):
        nb = -(-seq.ctx // 16)
        for j in range(nb):
            b = int(tables[s, j])
            seen[b] = max(seen.get(b, 0), min(16, seq.ctx - 16 * j))
    tokens = sum(seen.values())
    return tokens * w.num_kv_heads * row_bytes(w) * 2


def visible_kv_bytes(w, window):
    """K+V bytes of the keys some row of each sequence sees under a sliding
    window (the workloads given a window share no block inside it)."""
    tokens = sum(seq.ctx - max(0, seq.ctx - seq.q_len - window + 1) for seq in w.seqs)
    return tokens * w.num_kv_heads * row_bytes(w) * 2


def parse_workload(name):
    """A synthetic workload name with optional suffixes: "_tree" (each
    sequence's window is a seeded random draft tree, attended through
    paged_attention_masked_forward) and "_swa<W>" (a sliding window of W
    keys, the blocks below every row's window freed first)."""
    tree, window, base = False, 0, name
    if "_swa" in base:
        base, w = base.rsplit("_swa", 1)
        window = int(w)
    if base.endswith("_tree"):
        base, tree = base[:-5], True
    return base, tree, window


def tree_mask_words(w, seed=1234):
    """Ancestor masks of one random tree per window (parent of row r drawn
    from -1 .. r - 1), bit r set for the row itself."""
    rng = np.random.default_rng(seed)
    words = []
    for seq in w.seqs:
        masks = []
        for r in range(seq.q_len):
            p = int(rng.integers(-1, r)) if r else -1
            masks.append((1 << r) | (masks[p] if p >= 0 else 0))
        words += masks
    return np.array(words, dtype=np.uint32)


def visible_keys(w, window=0, tree_words=None):
    """Keys attended per layer, summed over query rows: row r of a sequence
    sits at p = ctx - q_len + r and sees keys 0..p, or the last `window` of
    them, or (a draft tree) every key before the window plus its ancestors."""
    total, i = 0, 0
    for seq in w.seqs:
        base = seq.ctx - seq.q_len
        for r in range(seq.q_len):
            p = base + r
            if tree_words is not None:
                total += base + bin(int(tree_words[i]) & ((1 << (r + 1)) - 1)).count("1")
            elif window:
                total += min(p + 1, window)
            else:
                total += p + 1
            i += 1
    return total


def logical_kv_bytes(w):
    return sum(seq.ctx for seq in w.seqs) * w.num_kv_heads * row_bytes(w) * 2


def host_cpu_model():
    """The host CPU's model name (the "model name" field of /proc/cpuinfo,
    which lscpu also reports), or None where the file has none."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, kv_bytes, rows, seconds, tree_mask=None, window=0):
    """The oracle, as it stands, on the host cores: its own allocation and
    scatter build the pools once; each timed call is gather + fp64 attention
    over the whole batch of one layer."""
    import oracle
    a = oracle.Allocator(w.num_blocks, w.block_size, w.free_order)
    if w.dtype == "fp8":
        kp, vp = oracle.fp8_empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim)
        put = oracle.fp8_scatter
    elif w.dtype == "fp4":
        kp, vp = oracle.fp4_empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim)
        put = oracle.fp4_scatter
    else:
        kp, vp = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype)
        put = oracle.scatter
    tables = []
    for s, seq in enumerate(w.seqs):
        row, _, _, slots = a.alloc(s, seq.tokens, w.max_blocks_per_seq)
        put(kp, vp, seq.k, seq.v, slots)
        tables.append(row)
    tables = np.array(tables, dtype=np.int32)
    threads = oracle.default_threads()
    cpu_model = host_cpu_model()
    times = []
    want = None
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or len(times) < 2:
        t1 = time.perf_counter()
        out = oracle.paged_attention(w.q, kp, vp, tables, w.context_lens, w.qsl, w.num_q_heads,
                                     w.num_kv_heads, w.scale, w.sinks, w.dtype, threads, tree_mask=tree_mask,
                                     window=window)
        times.append(time.perf_counter() - t1)
        if want is None:
            want = out
        if len(times) >= 500:
            break
    med = float(np.median(times))
    return {"value": round(kv_bytes / med / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"{len(times)} calls over one layer's batch ({rows} rows, {kv_bytes / 1e6:.1f} MB of "
                      f"K/V), median {med * 1e3:.2f} ms per call (gather + fp64 attention); "
                      f"seq-tokens/s {rows / med:.1f}"}, want


# max-abs tolerance against the fp64 oracle, per pool format (8- and 4-bit
# pools against the oracle's attention over its own dequantized codes)
TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8": 2e-3, "fp4": 2e-3}


def rows_alone_equal(pk, torch, st, w, rows):
    """Bitwise: each listed query row, submitted by itself as one decode row
    over the keys up to its position through the same block table, against
    the same row in the batch output held in st.out."""
    batch = st.out.contiguous().view(torch.int32).cpu().numpy()
    dev = st.q.device
    for i in rows:
        s = int(np.searchsorted(w.qsl, i, side="right") - 1)
        seq = w.seqs[s]
        p = seq.ctx - seq.q_len + (i - int(w.qsl[s]))
        one = pk.paged_attention_forward(
            st.q[i:i + 1].contiguous(), st.k_pools[0], st.v_pools[0], st.tables[s:s + 1].contiguous(),
            torch.tensor([p + 1], dtype=torch.int32, device=dev), torch.tensor([0, 1], dtype=torch.int32, device=dev),
            1, p + 1, w.scale, sinks=st.sinks)
        if not np.array_equal(one.contiguous().view(torch.int32).cpu().numpy()[0], batch[i]):
            return False
    return True


def copy_calibrate(nbytes, reps):
    """A plain device-to-device copy of nbytes, reps times: its HBM counters
    per dispatch (read nbytes, write nbytes) scale the attention kernels'."""
    import torch
    n = (nbytes // 16) * 16
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0").view(torch.int32)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)
    return 0


# ---------------------------------------------------------------------------
# rocprofv3 summaries: kernel durations and HBM traffic per attention launch.
# ---------------------------------------------------------------------------
ATTN_SOURCE = os.path.join(ROOT, "paged_kv_attention_block_amd", "csrc", "attention.hip")
PRODUCER_SOURCE = os.path.join(ROOT, "paged_kv_attention_block_amd", "csrc", "producer.hip")
ATTN_KERNELS = ("attn_parallel", "attn_fold", "attn_sequential", "attn_f32")
PRODUCER_KERNEL = "qknorm_rope_scatter_kernel"


def source_digest(path=ATTN_SOURCE):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name):
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "").replace("pkv::", "").strip()


def _appending(kernel):
    """True for attn_parallel instances with the appending path: template
    arguments <head_dim, tiles, prefetch, append, tile format, masked>."""
    if not kernel.startswith("attn_parallel<"):
        return False
    args = [a.strip() for a in kernel[kernel.index("<") + 1:kernel.rindex(">")].split(",")]
    return len(args) >= 4 and args[3] == "true"


def _counter_means(d, counter):
    """Mean of `counter` per dispatch, per kernel, in the counter's unit."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def summarize_profile(d, workload, commands, producer=False):
    """Write profiles/attention_<workload>.md from a directory holding the
    rocprofv3 outputs: stats/ (--kernel-trace --stats), fetch/ and write/
    (--pmc FETCH_SIZE, --pmc WRITE_SIZE over the bench), copy_fetch/ and
    copy_write/ (the same counters over --copy-calibrate)."""
    stats = _csv_rows(os.path.join(d, "stats"), "kernel_stats.csv")
    copy = json.load(open(os.path.join(d, "copy.json")))
    cbytes = copy["copy_bytes"]
    cf = _counter_means(os.path.join(d, "copy_fetch"), "FETCH_SIZE")
    cw = _counter_means(os.path.join(d, "copy_write"), "WRITE_SIZE")
    ckey = max(cf, key=lambda k: cf[k][0])
    f_scale = cbytes / (cf[ckey][0] * 1024.0)       # true bytes per counted byte
    w_scale = cbytes / (cw[max(cw, key=lambda k: cw[k][0])][0] * 1024.0)
    fetch = _counter_means(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = _counter_means(os.path.join(d, "write"), "WRITE_SIZE")
    src = PRODUCER_SOURCE if producer else ATTN_SOURCE
    title = "Producer kernel (kv_qknorm_rope_scatter)" if producer else "Attention kernels"
    lines = [f"# {title}, workload {workload}", "",
             f"Source digest (sha256/16 of {os.path.basename(src)}): `{source_digest(src)}`", "",
             "Commands (run from the repository root):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "## Kernel durations (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:8]:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    lines += ["", "## HBM traffic per dispatch (rocprofv3 --pmc, one counter per run)", "",
              f"Copy calibration: a {cbytes} B device copy (`{ckey}`) reads FETCH_SIZE "
              f"{cf[ckey][0]:.0f} KiB and WRITE_SIZE {cw[max(cw, key=lambda k: cw[k][0])][0]:.0f} KiB per "
              f"dispatch; scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write) turn counted KiB into bytes.",
              "", "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled fetch MB | scaled write MB |",
              "|---|---|---|---|---|---|"]
    traffic = 0.0
    for k in sorted(set(fetch) | set(write)):
        if producer:
            if PRODUCER_KERNEL not in k:
                continue
            fk, fn = fetch.get(k, (0.0, 0))
            wk, _ = write.get(k, (0.0, 0))
            fb, wb = fk * 1024 * f_scale, wk * 1024 * w_scale
            traffic += fb + wb
            lines.append(f"| {k} | {fn} | {fk:.0f} | {wk:.0f} | {fb / 1e6:.2f} | {wb / 1e6:.2f} |")
            continue
        if not k.startswith(ATTN_KERNELS) and "scatter" not in k:
            continue
        fk, fn = fetch.get(k, (0.0, 0))
        wk, _ = write.get(k, (0.0, 0))
        fb, wb = fk * 1024 * f_scale, wk * 1024 * w_scale
        # the attention call as paged_attention_forward issues it: split
        # kernels without the appending path (its last template argument)
        if k.startswith(ATTN_KERNELS) and not _appending(k):
            traffic += fb + wb
        lines.append(f"| {k} | {fn} | {fk:.0f} | {wk:.0f} | {fb / 1e6:.2f} | {wb / 1e6:.2f} |")
    if producer:
        lines += ["", "Traffic of one kv_qknorm_rope_scatter launch.", "",
                  f"traffic_bytes_per_producer_call: {traffic:.0f}", ""]
    else:
        lines += ["", "Traffic of one paged_attention_forward call (the bench's attention-only timing): the split",
                  "kernels without the appending path, the fold, the prefill shape.", "",
                  f"traffic_bytes_per_attention_call: {traffic:.0f}", ""]
    out = os.path.join(ROOT, "profiles", f"{'producer' if producer else 'attention'}_{workload}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(out)
    return 0


MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU",
                 "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES", "SQ_WAVES", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4                # MI355X: 256 compute units of 4 SIMDs
XCDS = 8


def summarize_mfma(d, workload, commands):
    """Write profiles/mfma_<workload>.md from one rocprofv3 --pmc run over the
    bench with MFMA_COUNTERS. MFMA utilisation follows rocprofv3's own
    MfmaUtil: summed SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE of the
    busiest die x SIMDs); the counter as collected sums the eight dies, so
    its per-die maximum is taken as that sum / 8. A 16x16x32 bf16 MFMA is
    16384 FLOP."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        k = _short(r["Kernel_Name"])
        if not k.startswith(ATTN_KERNELS):
            continue
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = [f"# MFMA and VALU counters, workload {workload}", "",
             f"Source digest (sha256/16 of {os.path.basename(ATTN_SOURCE)}): `{source_digest()}`", "",
             "Command (run from the repository root):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "Per dispatch, averaged over the run's dispatches of each kernel. MFMA utilisation:",
              "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs), as rocprofv3's MfmaUtil;",
              "MFMA TFLOP/s: SQ_INSTS_MFMA x 16384 FLOP over the dispatch's GRBM_GUI_ACTIVE / 8 cycles at 2.4 GHz.",
              "", "| kernel | dispatches | SQ_INSTS_MFMA | SQ_VALU_MFMA_BUSY_CYCLES | GRBM_GUI_ACTIVE | SQ_INSTS_VALU "
              "| VALU per MFMA | MFMA util % | issued MFMA TFLOP/s |", "|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(acc):
        m = {c: sum(v) / len(v) for c, v in acc[k].items()}
        if not all(c in m for c in MFMA_COUNTERS):
            continue
        n = len(acc[k]["SQ_INSTS_MFMA"])
        die_cycles = m["GRBM_GUI_ACTIVE"] / XCDS
        util = 100.0 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (die_cycles * SIMDS) if die_cycles else 0.0
        tflops = m["SQ_INSTS_MFMA"] * 16384 / (die_cycles / 2.4e9) / 1e12 if die_cycles else 0.0
        vpm = f"{m['SQ_INSTS_VALU'] / m['SQ_INSTS_MFMA']:.1f}" if m["SQ_INSTS_MFMA"] else "—"
        lines.append(f"| {k} | {n} | {m['SQ_INSTS_MFMA']:.0f} | {m['SQ_VALU_MFMA_BUSY_CYCLES']:.0f} | "
                     f"{m['GRBM_GUI_ACTIVE']:.0f} | {m['SQ_INSTS_VALU']:.0f} | {vpm} | {util:.1f} | {tflops:.0f} |")
    out = os.path.join(ROOT, "profiles", f"mfma_{workload}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)
    return 0


def committed_traffic(workload, producer=False):
    """HBM bytes per call from the committed summary, or None when there is
    none or the kernels changed since it was taken."""
    kind, src = ("producer", PRODUCER_SOURCE) if producer else ("attention", ATTN_SOURCE)
    p = os.path.join(ROOT, "profiles", f"{kind}_{workload}.md")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    if f"`{source_digest(src)}`" not in txt:
        return None
    for line in txt.splitlines():
        if line.startswith(f"traffic_bytes_per_{kind}_call:"):
            return float(line.split(":")[1])
    return None


def producer_bench(args, torch, synth, pk):
    """kv_qknorm_rope_scatter over the step tokens of a bf16 workload (every
    row of every sequence: its Q, K and V heads), Qwen3-like settings (norm
    weights, NeoX RoPE over the whole head, theta 1e6). Enough copies of the
    inputs and pools that one timed step misses the last-level cache."""
    w = synth.by_name(args.workload)
    if w.dtype != "bf16":
        print("bench.py: the producer step writes bf16 pools", file=sys.stderr)
        return 2
    n, Hq, Hkv, D = w.total_rows, w.num_q_heads, w.num_kv_heads, w.head_dim
    alg = 2 * n * (Hq + 2 * Hkv) * D * 2 + 8 * n        # rows read and written, positions and slots
    copies = args.layers or max(1, math.ceil(MIN_FOOTPRINT / alg))
    g = torch.Generator(device="cuda").manual_seed(7)
    mk = lambda *s: torch.randn(s, generator=g, device="cuda").to(torch.bfloat16)
    nb = -(-n // 16) + 1
    sets = []
    pos = torch.from_numpy(np.concatenate([np.arange(s.ctx - s.q_len, s.ctx) for s in w.seqs]).astype(np.int32)).cuda()
    slots = torch.arange(n, dtype=torch.int32, device="cuda") + 16    # whole blocks where the rows allow
    for _ in range(copies):
        kp, vp = pk.empty_pools(nb + 1, Hkv, D, torch.bfloat16, "cuda")
        sets.append((mk(n, Hq, D), mk(n, Hkv, D), mk(n, Hkv, D), torch.empty(n, Hq, D, dtype=torch.bfloat16,
                                                                            device="cuda"), kp, vp))
    qw, kw = mk(D), mk(D)

    def step():
        for q, k, v, qo, kp, vp in sets:
            pk.kv_qknorm_rope_scatter(q, k, v, pos, slots, kp, vp, q_norm_weight=qw, k_norm_weight=kw, eps=1e-6,
                                      rope_theta=1e6, rotary_dim=D, q_out=qo)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    us_call = ms * 1e3 / copies
    gbs = alg / (us_call * 1e-6) / 1e9
    print(json.dumps({
        "metric": "kv_qknorm_rope_scatter GB/s (QK-norm + NeoX RoPE + paged scatter), 1 GPU", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic (seeded N(0,1) rows)",
        "config": {"workload": args.workload, "tokens": n, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                   "copies_per_step": copies},
        "call_us": round(us_call, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": committed_traffic(args.workload, producer=True),
                     "kernel": "qknorm_rope_scatter_kernel", "alg_bytes_per_launch": alg},
    }), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--loops", type=int, default=5, help="timed loops of --steps steps; the median is reported")
    # the largest decode workload is the default: 32 sequences of 1024-8192
    # keys, 64 q / 8 KV heads, D 64, with sinks (226 MB of K/V per layer)
    ap.add_argument("--workload", default="sink_decode")
    ap.add_argument("--layers", type=int, default=0, help="pool copies per step (0: reach 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle sample budget (0: skip)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (for counter calibration) and exit")
    ap.add_argument("--summarize", metavar="DIR", help="only write the profile summary from rocprofv3 output")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="only write the MFMA/VALU counter summary from one rocprofv3 --pmc run")
    ap.add_argument("--commands", nargs="*", default=[], help="commands recorded in the summary")
    ap.add_argument("--no-prefix", action="store_true",
                    help="do not pass the batch's shared prompt prefix (from its block tables) to the attention calls")
    ap.add_argument("--producer", action="store_true",
                    help="time kv_qknorm_rope_scatter on the workload's step tokens instead of the attention step")
    args = ap.parse_args(argv)

    if args.summarize:
        return summarize_profile(args.summarize, args.workload, args.commands, producer=args.producer)
    if args.summarize_mfma:
        return summarize_mfma(args.summarize_mfma, args.workload, args.commands)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU only; multi-GPU runs are not supported "
              "(--gpus must be 1).", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibrate:
        return copy_calibrate(args.copy_calibrate, max(1, args.steps))

    import synth
    import paged_kv_attention_block_amd as pk
    from paged_kv_attention_block_amd.staging import prefix_hint, stage

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.producer:
        return producer_bench(args, torch, synth, pk)
    base, tree, window = parse_workload(args.workload)
    w = synth.by_name(base)
    w.name = args.workload
    elt = elem_bytes(w)
    if tree and max(seq.q_len for seq in w.seqs) > 32:
        print("bench.py: tree windows take at most 32 rows per sequence", file=sys.stderr)
        return 2

    # host block allocation for the batch, timed on its own
    t0 = time.perf_counter()
    pool = pk.kv_pool_create(w.num_blocks, 16, w.free_order)
    for s, seq in enumerate(w.seqs):
        pk.kv_pool_alloc(pool, s, seq.tokens, w.max_blocks_per_seq)
    alloc_us = (time.perf_counter() - t0) * 1e6
    del pool

    pool_bytes = w.num_blocks * w.num_kv_heads * 16 * row_bytes(w) * 2
    # enough pool copies that one step touches more than the last-level cache
    # holds; a sliding window touches only its keys, so its copies are counted
    # from those (at most 40 GiB of pools)
    touched = visible_kv_bytes(w, window) if window else pool_bytes
    layers = args.layers or max(1, min(math.ceil(MIN_FOOTPRINT / touched), (40 << 30) // pool_bytes))
    st = stage(w, device=dev, copies=layers, poison=False)
    kv_bytes = unique_kv_bytes(w, st.tables_np) if not window else visible_kv_bytes(w, window)
    tables = st.tables
    if window:
        # blocks below every row's window go back to the pool
        for s, seq in enumerate(w.seqs):
            pk.kv_pool_drop_prefix(st.pool, s, max(0, seq.ctx - seq.q_len - window + 1))
        rows_np = np.stack([pk.kv_pool_alloc(st.pool, s, [], st.max_blocks)[0] for s in range(len(w.seqs))])
        tables = torch.from_numpy(rows_np.astype(np.int32)).to(dev)
    tmask = torch.from_numpy(tree_mask_words(w).view(np.int32)).to(dev) if tree else None
    masked = tree or window > 0
    # a prompt prefix the batch's sequences hold in the same physical blocks,
    # as the host tables show it: the attention calls read it once per group
    pre_seqs, pre_tokens = (0, 0) if (masked or args.no_prefix) else prefix_hint(st.tables_np)
    use_prefix = pre_seqs >= 2
    rows = w.total_rows
    q_bytes = rows * w.num_q_heads * w.head_dim * elt
    out_bytes = rows * w.num_q_heads * w.head_dim * 4
    n_step_tok = int(st.step_slots_np.size)
    scatter_bytes = n_step_tok * w.num_kv_heads * (w.head_dim * elt + row_bytes(w)) * 2
    stream = torch.cuda.current_stream()

    def attend(l):
        if masked:
            pk.paged_attention_masked_forward(st.q, st.k_pools[l], st.v_pools[l], tables, st.context_lens, st.qsl,
                                              st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks,
                                              tree_mask=tmask, sliding_window=window, out=st.out,
                                              workspace=st.workspace)
        elif use_prefix:
            pk.paged_attention_prefix_forward(st.q, st.k_pools[l], st.v_pools[l], tables, st.context_lens, st.qsl,
                                              st.max_q_len, st.max_context_len, w.scale, pre_seqs, pre_tokens,
                                              sinks=st.sinks, out=st.out, workspace=st.workspace)
        else:
            pk.paged_attention_forward(st.q, st.k_pools[l], st.v_pools[l], tables, st.context_lens, st.qsl,
                                       st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks, out=st.out,
                                       workspace=st.workspace)

    def layer_call(l):
        if masked or use_prefix:
            # masked and prefix calls take no appended rows: scatter, then attend
            pk.kv_append_scatter(st.k_step, st.v_step, st.step_slots, st.k_pools[l], st.v_pools[l])
            attend(l)
        else:
            pk.paged_attention_append_forward(st.q, st.k_step, st.v_step, st.step_slots, st.k_pools[l],
                                              st.v_pools[l], tables, st.context_lens, st.qsl, st.max_q_len,
                                              st.max_context_len, w.scale, sinks=st.sinks, out=st.out,
                                              workspace=st.workspace)

    def step():
        for l in range(layers):
            layer_call(l)

    def attention_only():
        for l in range(layers):
            attend(l)

    # Both loops are captured once into HIP graphs and replayed, as a serving
    # loop replays its decode step: host launch cost stays out of the timing.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(1, args.warmup)):
            step()
            attention_only()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        step()
    g_att = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_att):
        attention_only()
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def timed(graph, n):
        """Milliseconds per replay of `graph` over n back-to-back replays,
        events recorded on the launch stream; the median of --loops loops."""
        per = []
        for _ in range(max(1, args.loops)):
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / n)
        return float(np.median(per)), per

    ms_per_step, step_loops = timed(g_step, args.steps)

    # attention launches alone, back to back: average duration per call
    att_graph_ms, _ = timed(g_att, args.steps)
    att_ms = att_graph_ms / layers

    # the step's scatter-write alone (kv_append_scatter of every new row into
    # one layer's pools), timed the same way
    g_sc = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_sc):
        for l in range(layers):
            pk.kv_append_scatter(st.k_step, st.v_step, st.step_slots, st.k_pools[l], st.v_pools[l])
    g_sc.replay()
    scatter_ms = timed(g_sc, args.steps)[0] / layers

    # the same step launched eagerly (host launch cost included), for reference
    e0.record(stream)
    step()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1)

    value = kv_bytes * layers / (ms_per_step * 1e-3) / 1e9
    att_alg_bytes = kv_bytes + q_bytes + out_bytes
    achieved = att_alg_bytes / (att_ms * 1e-3) / 1e9

    # Checks on the same inputs, outside the timed regions, with the oracle
    # leg (runs that skip it, such as the profiler's, launch nothing more):
    # the batch output of the last call against the oracle's, and, without
    # tree masks or a window, the first and last rows computed alone, bit
    # for bit.
    cpu = parity = None
    if args.cpu_seconds > 0:
        got = st.out.cpu().numpy()
        cpu, want = cpu_baseline(w, kv_bytes, rows, args.cpu_seconds, tree_mask_words(w) if tree else None, window)
        err = float(np.max(np.abs(got.astype(np.float64) - want))) if got.size else 0.0
        parity = {"max_abs_err": err, "tol": TOL[w.dtype], "ok": bool(np.all(np.isfinite(got)) and err <= TOL[w.dtype])}
        if not masked and rows:
            parity["rows_alone_bitwise"] = rows_alone_equal(pk, torch, st, w, sorted({0, rows - 1}))

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "loops": max(1, args.loops),
        "ms_per_step_loops": [round(x, 4) for x in step_loops],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded block placement)",
        "config": {
            "workload": w.name, "seqs": len(w.seqs), "context_lens": [int(s.ctx) for s in w.seqs],
            "rows_per_layer": rows, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": 16, "layers_per_step": layers,
            "tree_windows": tree, "sliding_window": window,
            "shared_prefix": {"seqs": pre_seqs, "tokens": pre_tokens} if use_prefix else None,
            "kv_bytes_per_layer": kv_bytes, "logical_kv_bytes_per_layer": logical_kv_bytes(w),
        },
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "seq_tokens_per_s": round(rows / (ms_per_step * 1e-3), 1),
        "ctx_tokens_per_s": round(visible_keys(w, window, tree_mask_words(w) if tree else None)
                                  / (ms_per_step * 1e-3), 1),
        "attention_call_us": round(att_ms * 1e3, 3),
        "scatter_call_us": round(scatter_ms * 1e3, 3),
        "scatter_tokens": n_step_tok,
        "scatter_gbs": round(scatter_bytes / (scatter_ms * 1e-3) / 1e9, 2) if scatter_ms > 0 else None,
        "eager_ms_per_step": round(eager_ms, 4),
        "layer_us": round(ms_per_step * 1e3 / layers, 3),
        "host_alloc_us_per_batch": round(alloc_us, 1),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(w.name),
            "kernel": "paged_attention_forward (split + fold launches)",
            "alg_bytes_per_launch": att_alg_bytes,
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)
    if parity and (not parity.get("ok", True) or not parity.get("rows_alone_bitwise", True)):
        print(f"bench.py: output check failed: {parity}", file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
