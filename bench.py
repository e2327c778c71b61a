#!/usr/bin/env python3
"""Benchmark: one DiT block forward (attention half) at the full 58,758-token pack.

A step is one dit_block_forward over the full-shape workload: AdaLN ->
fused QKV -> 3D RoPE -> packed attention -> to_out.0 + gated residual, bf16
with float32 accumulation, inputs resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` is the block's algorithmic TFLOP/s; the
attention kernel (85% of the block's FLOPs) is the dominant kernel for the
roofline entry, timed with HIP events recorded by the library around each
stage on the stream the kernels run on.  ``ffn_half`` times the block's
feed-forward half (d_ff = 4 d_model) on its own; it is not part of ``value``.
``denoise_step`` times the denoising step around the block (one streaming
pass over the packed latent state), at the workload's size and on a 16-pack
batch large enough to stream from HBM; ``nft_loss`` does the same for the
DiffusionNFT loss and its gradient (one sample per request); ``fp8`` times the
block's four projections in FP8 (e4m3 codes, per-row scales) against the
e4m3 MFMA peak, the row quantization and the FP8-output AdaLN against HBM,
the two halves of the block with FP8 projections (``block_fp8``,
``ffn_fp8``, ms per call), the FP8 attention (operand preparation and the
attention, against the e4m3 peak) and the attention half with the attention
in FP8 too (``block_fp8_attn``).  ``backward`` times the attention backward, the
whole backward pass of the attention half and that of the feed-forward half
(each recomputes its forward).
``cpu_baseline`` times the float64 oracle on a bounded row sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DiT-block ms + attention TFLOP/s at 58,758 tokens; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6       # 256 CUs x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0        # dense e4m3 MFMA, twice the bf16 rate
ATTN_KERNEL = "attn_bf16_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_full_hbm_traffic.md")
KERNEL_SOURCES = ("joint_audio_video_amd/csrc/attn.hip", "joint_audio_video_amd/csrc/common.h")


def kernel_source_hash() -> str:
    """sha256 over the attention kernel's sources: the traffic figure is only valid for it."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per attention launch from the committed counter summary, or None when
    that summary was taken on different kernel sources (or does not exist)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _short_kernel(name: str) -> str:
    short = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", short)


def summarize_profile(kind: str, out_dir: str) -> int:
    """Print a markdown summary of rocprofv3 CSV output (committed under profiles/).

    Kernels are grouped by name and grid size, so launches of one kernel at
    different sizes (and the calibration copy) are reported apart."""
    if kind == "stats":
        per = {}
        files = glob.glob(os.path.join(out_dir, "**", "*kernel_trace.csv"), recursive=True)
        dbs = glob.glob(os.path.join(out_dir, "**", "*results.db"), recursive=True)
        if files:
            for r in csv.DictReader(open(files[0])):
                name = r["Kernel_Name"]
                if "dit::" not in name and "copyBuffer" not in name:
                    continue
                key = (_short_kernel(name), int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)
                       * int(r.get("Grid_Size_Y", 1) or 1) * int(r.get("Grid_Size_Z", 1) or 1))
                dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
                per.setdefault(key, []).append(dur)
        elif dbs:
            # rocprofv3's default output: a rocpd SQLite database with a kernels view
            import sqlite3
            con = sqlite3.connect(dbs[0])
            for name, gx, gy, gz, start, end in con.execute(
                    "select name, grid_x, grid_y, grid_z, start, end from kernels"):
                if "dit::" not in name and "copyBuffer" not in name:
                    continue
                key = (_short_kernel(name), int(gx) * int(gy) * int(gz))
                per.setdefault(key, []).append((int(end) - int(start)) / 1e6)
            con.close()
        else:
            print(f"no kernel_trace.csv or results.db under {out_dir}", file=sys.stderr)
            return 1
        total = sum(sum(v) for v in per.values())
        print("| kernel | grid (work-items) | calls | avg ms | min ms | max ms | total % |")
        print("|---|---|---|---|---|---|---|")
        for (k, grid), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            print(f"| {k[:60]} | {grid} | {len(v)} | {sum(v) / len(v):.4f} | {min(v):.4f} | "
                  f"{max(v):.4f} | {100 * sum(v) / total:.2f} |")
        return 0
    files = glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        print(f"no counter_collection.csv under {out_dir}", file=sys.stderr)
        return 1
    per = {}
    for r in csv.DictReader(open(files[0])):
        name = r["Kernel_Name"]
        if "dit::" not in name and "copyBuffer" not in name:
            continue
        key = f"{_short_kernel(name)} [grid {r['Grid_Size']}]"
        per.setdefault((key, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    print("| kernel | counter | dispatches | mean per dispatch |")
    print("|---|---|---|---|")
    for (k, c), vals in sorted(per.items()):
        if "copyBuffer" in k and max(vals) < 1024:
            continue   # small runtime copies
        print(f"| {k[:72]} | {c} | {len(vals)} | {sum(vals) / len(vals):.6g} |")
    return 0


def block_flops(n_tokens, d, cu, causal=False):
    """Algorithmic FLOPs: attention 4*D*(visible q,k pairs); QKV 6*N*D^2; out 2*N*D^2."""
    pairs = 0
    for a, b in zip(cu, cu[1:]):
        L = b - a
        pairs += L * (L + 1) // 2 if causal else L * L
    attn = 4.0 * d * pairs
    qkv = 6.0 * n_tokens * d * d
    out = 2.0 * n_tokens * d * d
    return attn, qkv, out


def elementwise_bytes(n_tokens, d, elt=2):
    """adaln: read x + write y (+ modality); rope: read+write q and k (+ positions)."""
    adaln = n_tokens * (2 * d * elt + 1)
    rope = n_tokens * (4 * d * elt + 12)
    return adaln, rope


DENOISE_CHANNELS = 96        # 24 latent channels x the 1x2x2 patch of a video token


def denoise_anchors(mod, pos):
    """Anchor rows of the synthetic recipe: the first video frame (t = 0) and the first
    8 audio tokens of each channel."""
    return (((mod == 0) & (pos[:, 0] == 0)) | ((mod == 1) & (pos[:, 0] < 8))).astype(np.uint8)


def denoise_bytes(mod, anchor, channels, v_elt=2):
    """Algorithmic bytes of one denoise_step with an X0 output: every row reads its id;
    latent rows read their anchor flag; free latent rows read z and v and write z and
    X0; anchor rows read their anchor value and write z and X0; text rows nothing more."""
    lat = mod != 2
    pin = lat & (anchor != 0)
    free = lat & ~pin
    c = channels
    return int(mod.size + lat.sum() + free.sum() * (4 * c + v_elt * c + 8 * c)
               + pin.sum() * 12 * c)


def nft_loss_mask(mod, pos, cu, t_last):
    """Loss-bearing rows of the synthetic recipe: video and audio rows except the first
    and last video frame of each request (condition frames of a first/last-frame task)."""
    keep = np.zeros(mod.size, dtype=np.uint8)
    for (a, b), tl in zip(zip(cu, cu[1:]), t_last):
        m, p = mod[a:b], pos[a:b]
        cond = (m == 0) & ((p[:, 0] == 0) | (p[:, 0] == tl))
        keep[a:b] = ((m != 2) & ~cond).astype(np.uint8)
    return keep


def nft_bytes(keep, channels, v_elt=2):
    """Algorithmic bytes of one nft_loss with a gradient: every row reads its mask byte
    and writes its gradient row; loss-bearing rows also read v_theta, v_old (v_elt each)
    and the float32 target."""
    c = channels
    return int(keep.size * (1 + 4 * c) + int((keep != 0).sum()) * (2 * v_elt * c + 4 * c))


def _cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _attn_head_task(task):
    """One (segment, head) of the oracle's attention for the sampled query rows,
    in a worker process with one BLAS thread.  The segment's keys and values are
    seeded N(0, 1) bf16 values generated here (they cost the same arithmetic as
    the block's own and need no transfer)."""
    import oracle
    import synth
    seg_len, rows_rel, q_rows, seed = task
    k = synth.normal_array((seg_len, q_rows.shape[1]), seed=seed, dtype="bf16")
    v = synth.normal_array((seg_len, q_rows.shape[1]), seed=seed + 1, dtype="bf16")
    q = np.zeros((seg_len, q_rows.shape[1]))
    q[rows_rel] = q_rows
    t0 = time.perf_counter()
    o = oracle.attention(q, k, v, [0, seg_len], 1, q_rows.shape[1], rows=rows_rel)
    return time.perf_counter() - t0, o


def cpu_baseline(wl, inp, lay, rows_n: int, workers: int):
    """Oracle (float64 NumPy) on a bounded sample of the block: `rows_n` random
    query rows through AdaLN, the fused QKV projection (all 3 D columns) and the
    3D RoPE with BLAS on every core; their attention against all keys of their
    segment as a process pool over (segment, head), one BLAS thread per worker;
    then to_out.0 with the gated residual.  Keys and values are synthetic (see
    _attn_head_task).  The rate is the sample's algorithmic FLOPs over its wall
    time; the full block's oracle time is that rate applied to the block's FLOPs
    (extrapolated, not run)."""
    import multiprocessing as mp

    import oracle
    n, d, H, Dh = wl.n_tokens, wl.d_model, wl.n_heads, wl.head_dim
    rows = np.sort(np.random.Generator(np.random.PCG64(7)).choice(n, size=rows_n, replace=False))
    cu = [int(c) for c in lay["cu_seqlens"]]
    # one BLAS thread in the workers: set before they start (spawned: they
    # import NumPy afresh and read these)
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                             "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    ctx = mp.get_context("spawn")
    pool = ctx.Pool(workers)
    for k, v in saved.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v
    try:
        # warm the workers (each imports NumPy and the oracle); a worker that cannot
        # start makes the pool respawn it forever, so every wait has a limit
        pool.map_async(_attn_head_task,
                       [(64, np.arange(1), np.zeros((1, Dh)), 1)] * workers).get(timeout=300)
        t0 = time.perf_counter()
        y = oracle.adaln_modulate(inp.x, lay["modality"], inp.table, wl.eps, rows=rows)
        qkv = oracle.qkv_project(y, inp.w_qkv)
        pos = np.asarray(lay["pos"])[rows]
        q_rot = oracle.rope3d(qkv[:, :d], pos, H, Dh, wl.sections, wl.theta)
        _ = oracle.rope3d(qkv[:, d:2 * d], pos, H, Dh, wl.sections, wl.theta)
        t_rows = time.perf_counter() - t0
        tasks, where = [], []
        for si, (a, b) in enumerate(zip(cu, cu[1:])):
            sel = np.nonzero((rows >= a) & (rows < b))[0]
            if sel.size == 0:
                continue
            for h in range(H):
                tasks.append((b - a, rows[sel] - a,
                              q_rot[sel, h * Dh:(h + 1) * Dh], 1000 + 2 * (si * H + h)))
                where.append((sel, h))
        t1 = time.perf_counter()
        res = pool.map_async(_attn_head_task, tasks, chunksize=1).get(timeout=900)
        t_attn = time.perf_counter() - t1
        o = np.zeros((rows.size, d))
        for (sel, h), (_, oh) in zip(where, res):
            o[sel, h * Dh:(h + 1) * Dh] = oh
        t2 = time.perf_counter()
        _ = oracle.out_proj_gated(o, inp.w_o, inp.x, lay["modality"], inp.table, rows=rows)
        t_out = time.perf_counter() - t2
    finally:
        pool.terminate()
        pool.join()
    dt = t_rows + t_attn + t_out
    flops = 0.0
    for a, b in zip(cu, cu[1:]):
        cnt = int(((rows >= a) & (rows < b)).sum())
        flops += cnt * (4.0 * d * (b - a) + 8.0 * d * d)
    rate = flops / dt
    a_f, q_f, o_f = block_flops(n, d, cu)
    return dict(value=rate / 1e12, unit="TFLOP/s", cores=len(os.sched_getaffinity(0)),
                kind="oracle",
                sample=(f"{rows_n} random query rows of the {n:,}-token block: AdaLN, fused QKV "
                        f"and RoPE with BLAS on every core ({t_rows:.1f} s), their attention "
                        f"against all {n:,} keys (synthetic seeded k, v) as {len(tasks)} "
                        f"(segment, head) tasks on {workers} one-thread processes "
                        f"({t_attn:.1f} s wall, {sum(r[0] for r in res):.1f} s in tasks), "
                        f"to_out.0 + gated residual ({t_out:.1f} s); float64 NumPy"),
                cpu_model=_cpu_model(), workers=workers,
                oracle_block_ms_extrapolated=round((a_f + q_f + o_f) / rate * 1e3, 1),
                seconds=dt)


CONFIG_RUNS = (("tiny_f32", "tiny", False), ("small", "small", False), ("medium", "medium", False),
               ("varlen_bidirectional", "varlen", False), ("varlen_causal", "varlen", True))


def _timed(torch, fn, reps, stream, batches=3):
    """ms per call: one untimed call, then the median over `batches` timed batches
    of `reps` calls (a single batch also catches the clock's ramp after a change
    of kernel)."""
    fn()
    per = []
    for _ in range(batches):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / reps)
    return sorted(per)[len(per) // 2]


def measure_workload(jav, torch, name, causal, stream, reps=10):
    """dit_block_forward on one workload (seeded inputs resident in HBM): block ms
    and the in-block stage ms from the library's events, the attention's and the
    projections' TFLOP/s, and the standalone AdaLN and RoPE kernels' GB/s on the
    workload's shapes (the block rotates q and k inside its QKV stage)."""
    import synth
    wl = synth.WORKLOADS[name]
    n, d, H, Dh = wl.n_tokens, wl.d_model, wl.n_heads, wl.head_dim
    inp = synth.block_inputs(wl)
    lay = jav.pack_layout([r.grid for r in wl.requests])
    bf = wl.dtype == "bf16"
    tdt = torch.bfloat16 if bf else torch.float32

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(tdt).cuda()

    x, w_qkv, w_o = t(inp.x), t(inp.w_qkv), t(inp.w_o)
    table = torch.from_numpy(inp.table).cuda()
    mod = torch.from_numpy(lay["modality"]).cuda()
    pos = torch.from_numpy(lay["pos"]).cuda()
    cu = torch.from_numpy(lay["cu_seqlens"]).cuda()
    desc = jav.block_desc(jav.DIT_BF16 if bf else jav.DIT_F32, d, H, Dh, wl.sections, wl.theta,
                          wl.eps, causal=causal)
    ws = torch.empty(jav.block_workspace_bytes(desc, n), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)

    def blk():
        jav.block_forward(desc, x, mod, pos, cu, lay["max_seqlen"], table, w_qkv, w_o, out=out,
                          workspace=ws, stream=stream)

    blk()
    torch.cuda.synchronize()
    jav.profile_enable(reps)
    block_ms = _timed(torch, blk, reps, stream)
    st_sum, calls = jav.profile_read()
    jav.profile_enable(0)
    st = {k: v / max(calls, 1) for k, v in zip(jav.STAGES, st_sum)}
    y = torch.empty_like(x)
    qk = torch.zeros((2, n, d), dtype=tdt, device="cuda")
    iso_adaln = _timed(torch, lambda: jav.adaln_modulate(x, mod, table, wl.eps, out=y,
                                                         stream=stream), 20, stream)
    iso_rope = _timed(torch, lambda: jav.rope3d_apply(qk[0], qk[1], pos, H, Dh, wl.sections,
                                                      wl.theta, stream=stream), 20, stream)
    a_f, q_f, o_f = block_flops(n, d, lay["cu_seqlens"].tolist(), causal)
    ab, rb = elementwise_bytes(n, d, 2 if bf else 4)
    rec = {
        "n_tokens": n, "d_model": d, "n_heads": H, "dtype": wl.dtype,
        "segments": int(cu.numel() - 1), "causal": causal,
        "block_ms": round(block_ms, 4),
        "block_tflops": round((a_f + q_f + o_f) / (block_ms * 1e-3) / 1e12, 2),
        "stage_ms": {k: round(v, 4) for k, v in st.items()},
        "attention_ms": round(st["attn"], 4),
        "attention_tflops": round(a_f / (st["attn"] * 1e-3) / 1e12, 2),
        "qkv_rope_tflops": round(q_f / (st["qkv"] * 1e-3) / 1e12, 2),
        "out_proj_tflops": round(o_f / (st["out"] * 1e-3) / 1e12, 2),
        "adaln_isolated_gbs": round(ab / (iso_adaln * 1e-3) / 1e9, 1),
        "rope_isolated_gbs": round(rb / (iso_rope * 1e-3) / 1e9, 1),
    }
    if bf:
        rec["attention_frac_of_bf16_peak"] = round(a_f / (st["attn"] * 1e-3) / 1e12
                                                   / PEAK_BF16_TFLOPS, 4)
        rec["block_frac_of_bf16_peak"] = round((a_f + q_f + o_f) / (block_ms * 1e-3) / 1e12
                                               / PEAK_BF16_TFLOPS, 4)
        rec["adaln_isolated_frac_of_hbm"] = round(ab / (iso_adaln * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        rec["rope_isolated_frac_of_hbm"] = round(rb / (iso_rope * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    del x, w_qkv, w_o, ws, out, y, qk
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="full", choices=["small", "medium", "full", "varlen"])
    ap.add_argument("--causal", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ffn", action="store_true",
                    help="skip timing the feed-forward half (d_ff = 4 d_model)")
    ap.add_argument("--no-denoise", action="store_true",
                    help="skip timing the denoising step around the block")
    ap.add_argument("--no-nft", action="store_true",
                    help="skip timing the DiffusionNFT loss")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip timing the FP8 projections")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward pass of the attention half")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the block on the other workloads (tiny float32, small, medium, "
                         "the 4-request pack bidirectional and causal)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-profile", nargs=2, metavar=("KIND", "DIR"),
                    help="print a summary of rocprofv3 CSV output: KIND is stats or pmc")
    args = ap.parse_args()
    if args.summarize_profile:
        return summarize_profile(*args.summarize_profile)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the block is measured on one MI355X).", file=sys.stderr)
        return 2

    import torch

    import joint_audio_video_amd as jav
    import synth

    wl = synth.WORKLOADS[args.workload]
    n, d, H, Dh = wl.n_tokens, wl.d_model, wl.n_heads, wl.head_dim
    print(f"# bench: workload={wl.name} N={n} D={d} H={H} steps={args.steps} "
          f"warmup={args.warmup}", file=sys.stderr, flush=True)
    inp = synth.block_inputs(wl)
    lay = jav.pack_layout([r.grid for r in wl.requests])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev)

    x, w_qkv, w_o = bf(inp.x), bf(inp.w_qkv), bf(inp.w_o)
    table = torch.from_numpy(inp.table).to(dev)
    mod = torch.from_numpy(lay["modality"]).to(dev)
    pos = torch.from_numpy(lay["pos"]).to(dev)
    cu = torch.from_numpy(lay["cu_seqlens"]).to(dev)
    ms_len = lay["max_seqlen"]
    desc = jav.block_desc(jav.DIT_BF16, d, H, Dh, wl.sections, wl.theta, wl.eps,
                          causal=args.causal)
    out = torch.empty_like(x)
    ws = torch.empty(jav.block_workspace_bytes(desc, n), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        jav.block_forward(desc, x, mod, pos, cu, ms_len, table, w_qkv, w_o, out=out,
                          workspace=ws, stream=stream)

    if args.copy_mib > 0:
        # a plain copy of known size, so HBM counters can be scaled to bytes
        n_el = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n_el, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    jav.profile_enable(args.steps)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    stage_sum, ncalls = jav.profile_read()
    jav.profile_enable(0)
    ms_step = total_ms / args.steps
    stage_ms = {s: v / max(ncalls, 1) for s, v in zip(jav.STAGES, stage_sum)}
    print(f"# timed {args.steps} steps: {ms_step:.3f} ms/step; stages {stage_ms}",
          file=sys.stderr, flush=True)

    # Each stage again on its own (fresh buffers, same inputs), so its rate can be
    # read apart from its neighbours in the block (the block's stage times include
    # the event brackets and the power state the previous kernel left behind):
    # the median of three timed batches.
    print("# isolated stages ...", file=sys.stderr, flush=True)
    # q, k, v as three [N][D] planes, the layout dit_block_forward's workspace uses
    y = torch.empty_like(x)
    qkv = torch.empty((n, 3 * d), dtype=torch.bfloat16, device=dev)
    planes = torch.empty((3, n, d), dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(x)
    jav.adaln_modulate(x, mod, table, wl.eps, out=y, stream=stream)
    jav.qkv_project(y, w_qkv, out=qkv, stream=stream)
    for i in range(3):
        planes[i].copy_(qkv[:, i * d:(i + 1) * d])
    q_v, k_v, v_v = planes[0], planes[1], planes[2]
    spare = torch.empty_like(x)
    iso_ops = {
        "adaln": (20, lambda: jav.adaln_modulate(x, mod, table, wl.eps, out=y, stream=stream)),
        "qkv": (5, lambda: jav.qkv_project(y, w_qkv, out=qkv, stream=stream)),
        "rope": (20, lambda: jav.rope3d_apply(q_v, k_v, pos, H, Dh, wl.sections, wl.theta,
                                              stream=stream)),
        # the block's form: rotated q into a spare plane, rotated k over q's plane
        "rope_to": (20, lambda: jav.rope3d_apply_to(q_v, k_v, spare, q_v, pos, H, Dh,
                                                    wl.sections, wl.theta, stream=stream)),
        "attn": (3, lambda: jav.attn_packed(q_v, k_v, v_v, cu, ms_len, H, Dh,
                                            causal=args.causal, out=o, stream=stream)),
        "out": (5, lambda: jav.out_proj_gated(o, w_o, x, mod, table, out=out, stream=stream)),
    }
    iso_ms = {}
    for name, (reps, fn) in iso_ops.items():
        iso_ms[name] = _timed(torch, fn, reps, stream)
    del y, qkv, planes, spare, o, q_v, k_v, v_v
    print(f"# isolated: {iso_ms}", file=sys.stderr, flush=True)

    # The feed-forward half of the same block (d_ff = 4 d_model), timed on its own:
    # the whole half, then each of its GEMMs.
    ffn_rec = None
    if not args.no_ffn:
        print("# feed-forward half ...", file=sys.stderr, flush=True)
        fi = synth.ffn_inputs(wl)
        F = wl.d_ff
        w1, w2 = bf(fi.w1), bf(fi.w2)
        table2 = torch.from_numpy(fi.table).to(dev)
        fdesc = jav.ffn_desc(jav.DIT_BF16, d, F, wl.eps)
        fws = torch.empty(jav.ffn_workspace_bytes(fdesc, n), dtype=torch.uint8, device=dev)
        y2 = torch.empty_like(x)
        h2 = torch.empty((n, F), dtype=torch.bfloat16, device=dev)
        jav.adaln_modulate(x, mod, table2, wl.eps, out=y2, stream=stream)
        ffn_ops = {
            "ffn": (5, lambda: jav.ffn_forward(fdesc, x, mod, table2, w1, w2, out=out,
                                               workspace=fws, stream=stream)),
            "ffn_up": (5, lambda: jav.ffn_up_gelu(y2, w1, out=h2, stream=stream)),
            "ffn_down": (5, lambda: jav.ffn_down_gated(h2, w2, x, mod, table2, out=out,
                                                       stream=stream)),
        }
        for name, (reps, fn) in ffn_ops.items():
            fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            iso_ms[name] = e0.elapsed_time(e1) / reps
        gemm_f = 2.0 * n * d * F
        ffn_rec = {
            "d_ff": F,
            "ffn_ms": round(iso_ms["ffn"], 4),
            "ffn_tflops": round(2 * gemm_f / (iso_ms["ffn"] * 1e-3) / 1e12, 2),
            "ffn_frac_of_bf16_peak": round(2 * gemm_f / (iso_ms["ffn"] * 1e-3) / 1e12
                                           / PEAK_BF16_TFLOPS, 4),
            "up_gelu_tflops": round(gemm_f / (iso_ms["ffn_up"] * 1e-3) / 1e12, 2),
            "down_gated_tflops": round(gemm_f / (iso_ms["ffn_down"] * 1e-3) / 1e12, 2),
        }
        del fws, y2, h2, w1, w2
        print(f"# ffn: {ffn_rec}", file=sys.stderr, flush=True)

    # The denoising step around the block: one streaming pass over the packed latent
    # state (float32 z, bf16 velocity, float32 X0), at the workload's size (79 MB, held
    # in the Infinity Cache between launches) and on 16 packs (1.27 GB from HBM).
    den_rec = None
    if not args.no_denoise:
        print("# denoise step ...", file=sys.stderr, flush=True)
        C = DENOISE_CHANNELS
        sig = (0.62, 0.6, 0.5, 0.47)
        mod_h = np.asarray(lay["modality"])
        an_h = denoise_anchors(mod_h, np.asarray(lay["pos"]))
        den_rec = {"channels": C, "sigmas": list(sig), "anchor_rows": int(an_h.sum())}
        for label, packs, reps in (("pack", 1, 50), ("16_packs", 16, 20)):
            di = synth.denoise_inputs(wl, C, n_rows=n * packs)
            m_h, a_h = np.tile(mod_h, packs), np.tile(an_h, packs)
            z_d = torch.from_numpy(di.z).to(dev)
            v_d = bf(di.v)
            av_d = torch.from_numpy(di.anchor_vals).to(dev)
            x0_d = torch.empty_like(z_d)
            m_d, a_d = torch.from_numpy(m_h).to(dev), torch.from_numpy(a_h).to(dev)
            fn = (lambda z_d=z_d, v_d=v_d, m_d=m_d, x0_d=x0_d, a_d=a_d, av_d=av_d:
                  jav.denoise_step(z_d, v_d, m_d, sig, x0=x0_d, anchor=a_d, anchor_vals=av_d,
                                   stream=stream))
            fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t_ms = e0.elapsed_time(e1) / reps
            b = denoise_bytes(m_h, a_h, C)
            den_rec[label] = {"rows": int(m_h.size), "us": round(t_ms * 1e3, 2), "bytes": b,
                              "gbs": round(b / (t_ms * 1e-3) / 1e9, 1),
                              "frac_of_hbm": round(b / (t_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            del z_d, v_d, av_d, x0_d, m_d, a_d, di
        print(f"# denoise: {den_rec}", file=sys.stderr, flush=True)

    # The DiffusionNFT loss and its gradient over the same latent rows, one sample per
    # request, at the pack's size and on 16 packs.
    nft_rec = None
    if not args.no_nft:
        print("# nft loss ...", file=sys.stderr, flush=True)
        C = DENOISE_CHANNELS
        mod_h, pos_h = np.asarray(lay["modality"]), np.asarray(lay["pos"])
        cu_h = lay["cu_seqlens"].tolist()
        keep_h = nft_loss_mask(mod_h, pos_h, cu_h, [r.t - 1 for r in wl.requests])
        nft_rec = {"channels": C, "beta": 0.5, "kept_rows": int(keep_h.sum())}
        for label, packs, reps in (("pack", 1, 50), ("16_packs", 16, 20)):
            S = (len(cu_h) - 1) * packs
            ni = synth.nft_inputs(wl, S, C, n_rows=n * packs)
            k_h = np.tile(keep_h, packs)
            cu_p = np.concatenate([[0]] + [np.asarray(cu_h[1:]) + i * n for i in range(packs)])
            vt_d, vo_d = bf(ni.v_theta), bf(ni.v_old)
            tg_d = torch.from_numpy(ni.v_target).to(dev)
            g_d = torch.empty_like(tg_d)
            out_d = torch.empty((S, 3), dtype=torch.float32, device=dev)
            k_d = torch.from_numpy(k_h).to(dev)
            cu_d = torch.from_numpy(cu_p.astype(np.int32)).to(dev)
            r_d = torch.from_numpy(ni.reward).to(dev)
            max_rows = int(np.max(np.diff(cu_p)))
            nws = torch.empty(jav.nft_workspace_bytes(S, max_rows), dtype=torch.uint8, device=dev)
            fn = (lambda vt_d=vt_d, vo_d=vo_d, tg_d=tg_d, cu_d=cu_d, max_rows=max_rows, r_d=r_d,
                  k_d=k_d, g_d=g_d, out_d=out_d, nws=nws:
                  jav.nft_loss(vt_d, vo_d, tg_d, cu_d, max_rows, r_d, 0.5, loss_mask=k_d,
                               grad=g_d, loss_out=out_d, workspace=nws, stream=stream))
            fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t_ms = e0.elapsed_time(e1) / reps
            b = nft_bytes(k_h, C)
            nft_rec[label] = {"rows": int(k_h.size), "samples": S, "us": round(t_ms * 1e3, 2),
                              "bytes": b, "gbs": round(b / (t_ms * 1e-3) / 1e9, 1),
                              "frac_of_hbm": round(b / (t_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            del vt_d, vo_d, tg_d, g_d, out_d, k_d, cu_d, r_d, nws, ni
        print(f"# nft: {nft_rec}", file=sys.stderr, flush=True)

    # The block's projections in FP8: activations and weights quantized per row on the
    # GPU, then the four products (QKV into planes, to_out.0 gated, ff.net.0.proj with
    # GELU, ff.net.2 gated) timed on their own.
    fp8_rec = None
    if not args.no_fp8:
        print("# fp8 projections ...", file=sys.stderr, flush=True)
        F = wl.d_ff
        fi = synth.ffn_inputs(wl)
        wq, wqs = jav.quantize_rows_fp8(w_qkv)
        wo, wos = jav.quantize_rows_fp8(w_o)
        w1 = bf(fi.w1)
        w1q, w1s = jav.quantize_rows_fp8(w1)
        del w1
        w2 = bf(fi.w2)
        w2q, w2s = jav.quantize_rows_fp8(w2)
        del w2
        xq = torch.empty((n, d), dtype=torch.uint8, device=dev)
        xs = torch.empty(n, dtype=torch.float32, device=dev)
        hq = torch.empty((n, F), dtype=torch.uint8, device=dev)
        hs = torch.empty(n, dtype=torch.float32, device=dev)
        jav.quantize_rows_fp8(x, codes=xq, scales=xs, stream=stream)
        hq.random_(0, 120)                 # finite codes, magnitudes up to 240
        hs.fill_(1.0 / 64)
        qkv8 = torch.empty((n, 3 * d), dtype=torch.bfloat16, device=dev)
        h8 = torch.empty((n, F), dtype=torch.bfloat16, device=dev)
        out8 = torch.empty_like(x)
        table8 = torch.from_numpy(fi.table).to(dev)
        ws_b8 = torch.empty(jav.block_fp8_attn_workspace_bytes(desc, n, cu.numel() - 1),
                            dtype=torch.uint8, device=dev)
        ws_a8 = torch.empty(jav.attn_fp8_workspace_bytes(n, cu.numel() - 1, H), dtype=torch.uint8,
                            device=dev)
        o8 = torch.empty_like(x)
        fdesc8 = jav.ffn_desc(jav.DIT_BF16, d, F, wl.eps)
        ws_f8 = torch.empty(jav.ffn_fp8_workspace_bytes(fdesc8, n), dtype=torch.uint8,
                            device=dev)
        ops8 = {
            "quant_x": (20, lambda: jav.quantize_rows_fp8(x, codes=xq, scales=xs, stream=stream)),
            "adaln_fp8": (20, lambda: jav.adaln_modulate_fp8(x, mod, table, wl.eps, codes=xq,
                                                             scales=xs, stream=stream)),
            "block_fp8": (3, lambda: jav.block_forward_fp8(desc, x, mod, pos, cu, ms_len, table,
                                                           wq, wqs, wo, wos, out=out8,
                                                           workspace=ws_b8, stream=stream)),
            "ffn_fp8": (3, lambda: jav.ffn_forward_fp8(fdesc8, x, mod, table8, w1q, w1s, w2q,
                                                       w2s, out=out8, workspace=ws_f8,
                                                       stream=stream)),
            "qkv": (5, lambda: jav.linear_fp8(xq, xs, wq, wqs, out=qkv8, stream=stream)),
            "out": (5, lambda: jav.linear_fp8(xq, xs, wo, wos, epilogue="gated", x=x,
                                              modality=mod, table=table, out=out8,
                                              stream=stream)),
            "ffn_up": (5, lambda: jav.linear_fp8(xq, xs, w1q, w1s, epilogue="gelu", out=h8,
                                                 stream=stream)),
            "ffn_down": (5, lambda: jav.linear_fp8(hq, hs, w2q, w2s, epilogue="gated", x=x,
                                                   modality=mod, table=table, out=out8,
                                                   stream=stream)),
            # FP8 attention on the QKV product above (q, k, v: strided column blocks)
            "attn_fp8_prepare": (5, lambda: jav.attn_fp8_prepare(
                qkv8[:, :d], qkv8[:, d:2 * d], qkv8[:, 2 * d:], cu, ms_len, H, Dh,
                workspace=ws_a8, stream=stream)),
            "attn_fp8": (3, lambda: jav.attn_packed_fp8(ws_a8, cu, ms_len, n, H, Dh,
                                                        causal=args.causal, out=o8,
                                                        stream=stream)),
            "block_fp8_attn": (3, lambda: jav.block_forward_fp8(
                desc, x, mod, pos, cu, ms_len, table, wq, wqs, wo, wos, out=out8,
                workspace=ws_b8, stream=stream, fp8_attention=True)),
        }
        t8 = {}
        for name, (reps, fn) in ops8.items():
            fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t8[name] = e0.elapsed_time(e1) / reps
        fl = {"qkv": 6.0 * n * d * d, "out": 2.0 * n * d * d, "ffn_up": 2.0 * n * d * F,
              "ffn_down": 2.0 * n * d * F}
        fp8_rec = {"format": "e4m3, per-row float32 scales", "ms": {k: round(v, 4) for k, v in t8.items()}}
        for k, f in fl.items():
            tf = f / (t8[k] * 1e-3) / 1e12
            fp8_rec[f"{k}_tflops"] = round(tf, 1)
            fp8_rec[f"{k}_frac_of_fp8_peak"] = round(tf / PEAK_FP8_TFLOPS, 4)
        af8 = block_flops(n, d, lay["cu_seqlens"].tolist(), args.causal)[0]
        fp8_rec["attn_fp8_tflops"] = round(af8 / (t8["attn_fp8"] * 1e-3) / 1e12, 1)
        fp8_rec["attn_fp8_frac_of_fp8_peak"] = round(af8 / (t8["attn_fp8"] * 1e-3) / 1e12
                                                     / PEAK_FP8_TFLOPS, 4)
        qb = n * (d * 2 + d + 4)
        fp8_rec["quant_x_gbs"] = round(qb / (t8["quant_x"] * 1e-3) / 1e9, 1)
        fp8_rec["quant_x_frac_of_hbm"] = round(qb / (t8["quant_x"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        # AdaLN with FP8 output: reads x (bf16), writes codes and scales
        fp8_rec["adaln_fp8_gbs"] = round(qb / (t8["adaln_fp8"] * 1e-3) / 1e9, 1)
        fp8_rec["adaln_fp8_frac_of_hbm"] = round(qb / (t8["adaln_fp8"] * 1e-3) / 1e9
                                                 / PEAK_HBM_GBS, 4)
        del wq, wo, w1q, w2q, xq, hq, qkv8, h8, out8, ws_b8, ws_f8, table8, ws_a8, o8
        print(f"# fp8: {fp8_rec}", file=sys.stderr, flush=True)

    # The backward pass of the attention half: the attention backward on its own
    # (given q', k', v, o, lse and dout) and the whole dit_block_backward (which
    # recomputes the forward).  Algorithmic FLOPs: attention backward = 2.5 x the
    # forward's (five products of the same size, S recomputed); the block
    # backward = its forward again + z + attention backward + four GEMMs (do,
    # dW_o, dy, dW_qkv).
    bwd_rec = None
    if not args.no_backward:
        print("# backward ...", file=sys.stderr, flush=True)
        dout = bf(synth.normal_array((n, d), seed=wl.seed + 4000, dtype="bf16"))
        q_r = bf(synth.normal_array((n, d), seed=wl.seed + 4001, dtype="bf16"))
        k_r = bf(synth.normal_array((n, d), seed=wl.seed + 4002, dtype="bf16"))
        v_r = bf(synth.normal_array((n, d), seed=wl.seed + 4003, dtype="bf16"))
        o_r, lse_r = jav.attn_packed_lse(q_r, k_r, v_r, cu, ms_len, H, Dh, causal=args.causal)
        dq_r, dk_r, dv_r = (torch.empty_like(q_r) for _ in range(3))
        aws = torch.empty(jav.attn_backward_workspace_bytes(n, H), dtype=torch.uint8, device=dev)
        bws = torch.empty(jav.block_backward_workspace_bytes(desc, n), dtype=torch.uint8,
                          device=dev)
        dx_b = torch.empty_like(x)
        ops_b = {
            "attn_bwd": (3, lambda: jav.attn_packed_backward(
                q_r, k_r, v_r, o_r, dout, lse_r, cu, ms_len, H, Dh, causal=args.causal, dq=dq_r,
                dk=dk_r, dv=dv_r, workspace=aws, stream=stream)),
            "block_bwd": (2, lambda: jav.block_backward(
                desc, x, dout, mod, pos, cu, ms_len, table, w_qkv, w_o, dx=dx_b, workspace=bws,
                stream=stream)),
        }
        tb = {}
        for name, (reps, fn) in ops_b.items():
            fn()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            tb[name] = e0.elapsed_time(e1) / reps
        # the feed-forward half's backward (d_ff = 4 d_model)
        fi_b = synth.ffn_inputs(wl)
        fdesc_b = jav.ffn_desc(jav.DIT_BF16, d, wl.d_ff, wl.eps)
        fws_b = torch.empty(jav.ffn_backward_workspace_bytes(fdesc_b, n), dtype=torch.uint8,
                            device=dev)
        w1_b, w2_b = bf(fi_b.w1), bf(fi_b.w2)
        t2_b = torch.from_numpy(fi_b.table).to(dev)
        fn_f = (lambda: jav.ffn_backward(fdesc_b, x, dout, mod, t2_b, w1_b, w2_b, dx=dx_b,
                                         workspace=fws_b, stream=stream))
        fn_f()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(2):
            fn_f()
        e1.record(stream)
        torch.cuda.synchronize()
        tb["ffn_bwd"] = e0.elapsed_time(e1) / 2
        del fws_b, w1_b, w2_b, t2_b
        a_f, q_f, o_f = block_flops(n, d, lay["cu_seqlens"].tolist(), args.causal)
        attn_bwd_f = 2.5 * a_f
        blk_bwd_f = (a_f + q_f + o_f) + o_f + attn_bwd_f + 2 * o_f + 2 * q_f
        bwd_rec = {
            "attention_backward_ms": round(tb["attn_bwd"], 3),
            "attention_backward_tflops": round(attn_bwd_f / (tb["attn_bwd"] * 1e-3) / 1e12, 1),
            "attention_backward_frac_of_bf16_peak": round(
                attn_bwd_f / (tb["attn_bwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "block_backward_ms": round(tb["block_bwd"], 3),
            "block_backward_tflops": round(blk_bwd_f / (tb["block_bwd"] * 1e-3) / 1e12, 1),
            "block_backward_frac_of_bf16_peak": round(
                blk_bwd_f / (tb["block_bwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            # forward again (a, z) + dh, dW2, dy, dW1: six products of 2 N D d_ff
            "ffn_backward_ms": round(tb["ffn_bwd"], 3),
            "ffn_backward_tflops": round(12.0 * n * d * wl.d_ff / (tb["ffn_bwd"] * 1e-3) / 1e12,
                                         1),
        }
        del dout, q_r, k_r, v_r, o_r, lse_r, dq_r, dk_r, dv_r, aws, bws, dx_b
        print(f"# backward: {bwd_rec}", file=sys.stderr, flush=True)

    cfg_rec = None
    if not args.no_configs:
        print("# other workloads ...", file=sys.stderr, flush=True)
        cfg_rec = {}
        for label, name, causal in CONFIG_RUNS:
            cfg_rec[label] = measure_workload(jav, torch, name, causal, stream)
            print(f"# {label}: {cfg_rec[label]}", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()

    cu_list = lay["cu_seqlens"].tolist()
    attn_f, qkv_f, out_f = block_flops(n, d, cu_list, args.causal)
    blk_f = attn_f + qkv_f + out_f
    adaln_b, rope_b = elementwise_bytes(n, d)
    attn_tflops = attn_f / (stage_ms["attn"] * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(blk_f / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, N(0,0.1) AdaLN table)",
        "config": {
            "workload": (f"{wl.name}: one DiT block, {n:,} packed tokens "
                         + " + ".join(f"[video {r.t}x{r.h}x{r.w} + audio 2x{r.audio_per_ch} "
                                      f"+ text {r.text_len}]" for r in wl.requests)
                         + f", d_model {d}, {H} heads x {Dh}, "
                         + ("causal" if args.causal else "bidirectional") + " attention"),
            "n_tokens": n, "d_model": d, "n_heads": H, "head_dim": Dh,
            "segments": len(cu_list) - 1, "causal": bool(args.causal),
        },
        "block_ms": round(ms_step, 4),
        "block_frac_of_bf16_peak": round(blk_f / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "attention_ms": round(stage_ms["attn"], 4),
        "attention_tflops": round(attn_tflops, 2),
        "attention_frac_of_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        # the qkv stage is the rotation table's kernel plus the QKV GEMM, which
        # rotates q and k in its epilogue: RoPE has no stage of its own in the block
        "qkv_tflops": round(qkv_f / (stage_ms["qkv"] * 1e-3) / 1e12, 2),
        "rope_in_qkv_epilogue": True,
        "out_proj_tflops": round(out_f / (stage_ms["out"] * 1e-3) / 1e12, 2),
        "adaln_gbs": round(adaln_b / (stage_ms["adaln"] * 1e-3) / 1e9, 1),
        "adaln_frac_of_hbm": round(adaln_b / (stage_ms["adaln"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "isolated_ms": {k: round(v, 4) for k, v in iso_ms.items()},
        "isolated": {
            "attention_tflops": round(attn_f / (iso_ms["attn"] * 1e-3) / 1e12, 2),
            "qkv_tflops": round(qkv_f / (iso_ms["qkv"] * 1e-3) / 1e12, 2),
            "out_proj_tflops": round(out_f / (iso_ms["out"] * 1e-3) / 1e12, 2),
            "adaln_gbs": round(adaln_b / (iso_ms["adaln"] * 1e-3) / 1e9, 1),
            "adaln_frac_of_hbm": round(adaln_b / (iso_ms["adaln"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "rope_gbs": round(rope_b / (iso_ms["rope"] * 1e-3) / 1e9, 1),
            "rope_frac_of_hbm": round(rope_b / (iso_ms["rope"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "rope_to_gbs": round(rope_b / (iso_ms["rope_to"] * 1e-3) / 1e9, 1),
            "rope_to_frac_of_hbm": round(rope_b / (iso_ms["rope_to"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                         4),
        },
        "roofline": {
            "kernel": "attn_bf16_kernel",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_traffic() if (wl.name == "full" and not args.causal) else None,
        },
    }
    if cfg_rec is not None:
        rec["workloads"] = cfg_rec
    if ffn_rec is not None:
        rec["ffn_half"] = ffn_rec
    if den_rec is not None:
        rec["denoise_step"] = den_rec
    if nft_rec is not None:
        rec["nft_loss"] = nft_rec
    if fp8_rec is not None:
        rec["fp8_projections"] = fp8_rec
    if bwd_rec is not None:
        rec["backward"] = bwd_rec
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        import oracle
        # the whole block in the oracle on the two small workloads (no sample)
        whole = {}
        for label, name in (("tiny_f32", "tiny"), ("small", "small")):
            wl_c = synth.WORKLOADS[name]
            inp_c = synth.block_inputs(wl_c)
            lay_c = oracle.pack_layout([r.grid for r in wl_c.requests])
            t0 = time.perf_counter()
            oracle.block_forward(inp_c.x, lay_c["modality"], lay_c["pos"], lay_c["cu_seqlens"],
                                 inp_c.table, inp_c.w_qkv, inp_c.w_o, n_heads=wl_c.n_heads,
                                 head_dim=wl_c.head_dim, sections=wl_c.sections,
                                 theta=wl_c.theta, eps=wl_c.eps)
            whole[label] = round((time.perf_counter() - t0) * 1e3, 1)
        print(f"# oracle whole-block ms: {whole}", file=sys.stderr, flush=True)
        olay = oracle.pack_layout([r.grid for r in wl.requests])
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        cb = cpu_baseline(wl, inp, olay, args.cpu_rows, workers)
        cb.pop("seconds")
        cb["value"] = round(cb["value"], 6)
        cb["gpu_block_ms"] = rec["block_ms"]
        cb["oracle_whole_block_ms"] = whole
        rec["cpu_baseline"] = cb
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
