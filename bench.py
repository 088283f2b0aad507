"""Benchmark of the sliding-window / global attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one bf16 SWA (W=128) + sink prefill of 32768 tokens (B=1, 64
query heads, 8 KV heads, head_dim 128, causal).  `value` is that prefill's
throughput in algorithmic TFLOP/s (4*D FLOP per (query head, key) pair inside
the window; masked or skipped tile work is not counted), over K timed steps
with inputs resident in HBM.  The same run also times the q_len=4 MTP verify
on 64 requests (global-layer cache with contexts U[4096, 65536] and a
128-slot SWA ring) and reports its HBM GB/s from algorithmic bytes (every
K/V row the windows need read once, plus Q, the new rows and O), and the
same for a plain q_len=1 decode step on the same shapes.  Further sections
(context for the same run, not the headline): the 48-layer self-speculative
MTP step (verify of 39 SWA and 9 global layers, greedy acceptance over a
152064-token vocabulary, append, advance) against the q_len=1 decode step;
the partial rotary embedding, standalone and fused into the SWA prefill;
the SWA 32K training forward (saved log-sum-exp) and backward; and the 256K
long-context block (chunked SWA prefill of 262144 tokens on 5 layers, then
a B=1 global q_len=4 verify against the 262144-token cache).

Prints ONE JSON line.  Inputs are seeded synthetic N(0,1) tensors rounded to
bf16 (random numbers, no dataset).  --gpus above 1 is refused: this build
runs on one GPU.

Before the W warmup steps of each workload the step is repeated, untimed, for
--settle-seconds (default 0.5 s): MI355X raises its clocks only under
sustained load, and a sub-millisecond step timed right after an idle period
measures the ramp rather than the kernel (about 20% slower for the 32K SWA
prefill).  The timed region is exactly K steps, as always.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
PROFILE_DIR = os.path.join(ROOT, "profiles")
_CSRC = os.path.join(ROOT, "hybrid_sliding_window_swa_amd", "csrc")
# sources a kernel's HBM traffic depends on (counters are void once these change)
PREFILL_KERNEL_SRC = [os.path.join(_CSRC, f) for f in ("prefill_bf16.hip", "common.hpp", "launch.hpp")]
VERIFY_KERNEL_SRC = [os.path.join(_CSRC, f) for f in ("verify_bf16.hip", "common.hpp", "launch.hpp")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true", help="time the SWA prefill only")
    ap.add_argument("--only", choices=["prefill", "ga", "verify", "mtp", "rope", "backward", "stack"], default=None,
                    help="run one workload only (for profiler runs); prints its own JSON line")
    ap.add_argument("--settle-seconds", type=float, default=0.5,
                    help="untimed repetition of each step before its warmup, so the clocks are at "
                         "their sustained level (0 disables)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (HBM counter calibration) and exit")
    ap.add_argument("--torch-copy-ceiling", action="store_true",
                    help="time torch's device copy_ of 4 GiB (a second copy ceiling beside swa_peaks), "
                         "print one swa_peaks-style JSON line and exit")
    return ap.parse_args()


def swa_pairs(S: int, W: int, q_offset: int = 0) -> int:
    """(query, key) pairs inside the causal window, per head."""
    if W <= 0:
        return sum(q_offset + r + 1 for r in range(S))
    tot = 0
    for r in range(S):
        i = q_offset + r
        tot += min(i + 1, W)
    return tot


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(name: str, src: str):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a copy-kernel calibration), kept under profiles/.
    Returns None if absent or taken on a different kernel source."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != source_hash(src):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma_busy(section: str):
    """Matrix-core busy fraction of one prefill kernel from the committed
    rocprofv3 counter summary (profiles/prefill_bf16_mfma_counters.txt,
    section "[prefill]" or "[ga]"), or None when absent or taken on other
    kernel sources."""
    path = os.path.join(PROFILE_DIR, "prefill_bf16_mfma_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    start = text.find(f"[{section}]")
    if start < 0:
        return None
    end = text.find("\n[", start + 1)
    block = text[start:end if end > 0 else len(text)]
    busy, src = None, None
    for line in block.splitlines():
        if line.startswith("derived: matrix-core busy fraction"):
            busy = line.split()[-1]
        elif line.startswith("kernel_source_sha256_16:"):
            src = line.split()[-1]
    if busy is None or src != source_hash(PREFILL_KERNEL_SRC):
        return None
    try:
        return float(busy)
    except ValueError:
        return None


def time_launches(fn, steps, stream, before=None):
    """Average duration (ms) of fn() over `steps` launches, measured with HIP
    events recorded on the stream the kernels run on."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        if before is not None:
            before()
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps


def read_peaks():
    """Ceilings measured on this GPU by swa_peaks (profiles/mi355x_peaks.txt),
    or None when the file is absent."""
    path = os.path.join(PROFILE_DIR, "mi355x_peaks.txt")
    if not os.path.exists(path):
        return None
    out = {}
    for line in open(path):
        if line.startswith("{"):
            d = json.loads(line)
            if d["measure"] == "hbm_read":
                out["hbm_read_GBs"] = d["GB/s"]
            elif d["measure"].startswith("hbm_copy"):
                if d["measure"] == "hbm_copy_head_groups":
                    # the sliding-window prefill's own access pattern as a
                    # copy: 2 KiB head-group segments of 16 KiB token rows
                    out["hbm_copy_head_groups_GBs"] = d["GB/s"]
                # the fastest copy: the library's copy kernels (contiguous or
                # grid-stride ranges, head-group segments) and torch's copy_
                if d["GB/s"] > out.get("hbm_copy_GBs", 0.0):
                    out["hbm_copy_GBs"] = d["GB/s"]
                    out["hbm_copy_by"] = d["measure"]
            elif d["measure"] == "mfma_bf16_32x32x16_random_operands":
                # operands switching every instruction, as attention's do:
                # the rate at the clock the chip's power limit then allows
                out["mfma_bf16_random_operands_TFLOPs"] = d["TFLOP/s"]
            elif d["measure"].startswith("mfma_bf16"):
                out["mfma_bf16_TFLOPs"] = d["TFLOP/s"]
            elif d["measure"] == "hbm_read_head_rows":
                # the global-cache verify's own access pattern: one KV head's
                # 256-byte rows per workgroup
                out["hbm_read_head_rows_GBs"] = d["GB/s"]
            elif d["measure"] == "hbm_read_cold_small":
                out["hbm_read_cold_small_us"] = d["us_median"]
                out["hbm_read_cold_small_bytes"] = d["bytes"]
    out["source"] = "profiles/mi355x_peaks.txt (swa_peaks)"
    return out


def settle(fn, seconds):
    """Repeat fn() untimed for `seconds` of wall time so that the GPU clocks
    reach their sustained-load level before anything is timed."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def run_prefill(args, swa, torch, dev, stream, cfg):
    """Time the SWA 32K prefill: wall clock over K steps + per-launch events."""
    from swa_inputs import prefill_inputs
    q, k, v, sinks = prefill_inputs(cfg, device=dev)
    o = torch.empty_like(q)
    flop = 4.0 * cfg.D * swa_pairs(cfg.S, cfg.window) * cfg.Hq * cfg.B
    p_bytes = 2 * cfg.B * (2 * cfg.S * cfg.Hq * cfg.D + 2 * cfg.keys * cfg.Hkv * cfg.D)

    def prefill():
        swa.swa_attn_prefill(q, k, v, sinks, cfg.window, cfg.q_offset, cfg.scale, out=o)

    settle(prefill, args.settle_seconds)
    for _ in range(args.warmup):
        prefill()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        prefill()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_kernel = time_launches(prefill, max(args.steps, 5), stream)
    ach_gbs = p_bytes / (ms_kernel * 1e-3) / 1e9
    res = {
        "ms_per_step": wall * 1e3 / args.steps,
        "value": flop / (wall / args.steps) / 1e12,
        "config": {
            "workload": "swa_32k_prefill",
            "batch": cfg.B, "seq_len": cfg.S, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
            "head_dim": cfg.D, "window": cfg.window, "causal": True, "sinks": "per-head N(0,1)",
            "inputs": "seeded N(0,1) rounded to bf16", "algorithmic_flop_per_step": flop,
            "algorithmic_bytes_per_step": p_bytes,
        },
        "roofline": {
            "kernel": "prefill_swa_strip_kernel",
            "bound": "hbm",
            "achieved": round(ach_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ach_gbs / HBM_PEAK_GBS, 4),
            "traffic": read_traffic("prefill_bf16_swa32k_hbm_counters.txt", PREFILL_KERNEL_SRC),
            "kernel_ms": round(ms_kernel, 5),
            "mfma_tflops": round(flop / (ms_kernel * 1e-3) / 1e12, 2),
            "mfma_frac_of_bf16_peak": round(flop / (ms_kernel * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "matrix_core_busy_by_counters": read_mfma_busy("prefill"),
            "roofline_tflops": round(min(MFMA_BF16_PEAK_TFLOPS, flop / p_bytes * HBM_PEAK_GBS / 1e3), 1),
        },
    }
    return res, (q, k, v, sinks)


def run_ga(args, swa, torch, dev, stream):
    """Time the global-attention 32K prefill (per-launch events)."""
    from swa_inputs import PREFILL_CONFIGS, prefill_inputs
    gcfg = PREFILL_CONFIGS["ga_32k"]
    gq, gk, gv, gs = prefill_inputs(gcfg, device=dev)
    go = torch.empty_like(gq)
    gflop = 4.0 * gcfg.D * swa_pairs(gcfg.S, gcfg.window) * gcfg.Hq * gcfg.B

    def ga_prefill():
        swa.swa_attn_prefill(gq, gk, gv, gs, gcfg.window, gcfg.q_offset, gcfg.scale, out=go)

    settle(ga_prefill, args.settle_seconds)
    for _ in range(max(1, args.warmup)):
        ga_prefill()
    gms = time_launches(ga_prefill, max(3, min(args.steps, 10)), stream)
    del gq, gk, gv, go
    torch.cuda.empty_cache()
    return {
        "workload": "ga_32k_prefill", "window": "global", "seq_len": gcfg.S,
        "algorithmic_flop": gflop, "ms": round(gms, 4),
        "TFLOP/s": round(gflop / (gms * 1e-3) / 1e12, 2),
        "frac_of_bf16_mfma_peak": round(gflop / (gms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        # rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over the active cycles of the
        # 1024 SIMDs (profiles/prefill_bf16_mfma_counters.txt); the chip runs
        # this kernel below the 2.4 GHz the datasheet peak assumes
        "matrix_core_busy_by_counters": read_mfma_busy("ga"),
    }


def run_verify(args, swa, torch, dev, stream, names=("verify_ga_b64", "verify_swa_b64")):
    """Time the q_len=4 verify (or, with the decode names, the q_len=1 decode)
    on the global-layer cache and the SWA ring."""
    from swa_inputs import VERIFY_CONFIGS, verify_inputs
    vres = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for name in names:
        vc = VERIFY_CONFIGS[name]
        inp = verify_inputs(vc, device=dev)
        cl = inp["cache_len"].to(torch.int32).to(dev)
        L = inp["cache_len"].to(torch.int64)
        need = swa.swa_attn_verify_workspace_bytes(vc.B, vc.T, vc.Hq, vc.Hkv, vc.D, vc.slots,
                                                   vc.ring, vc.window)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        ov = torch.empty_like(inp["q"])
        # rows the windows need: history positions max(0, L-W+1) .. L-1 (global: 0 .. L-1)
        if vc.window > 0:
            hist_rows = int(torch.clamp(L, max=vc.window - 1).sum())
        else:
            hist_rows = int(L.sum())
        row_b = vc.Hkv * vc.D * 2
        vbytes = (2 * hist_rows * row_b                      # K and V history
                  + 2 * vc.B * vc.T * row_b                  # new K and V rows
                  + 2 * vc.B * vc.T * vc.Hq * vc.D * 2)      # Q in, O out

        def verify():
            swa.swa_attn_verify(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"],
                                inp["v_cache"], cl, inp["sinks"], vc.window, vc.ring, vc.scale,
                                workspace=ws, out=ov)

        settle(verify, args.settle_seconds)
        for _ in range(args.warmup):
            verify()
        # small working sets would sit in the 256 MB Infinity Cache: flush it first
        before = (lambda: flush.zero_()) if vbytes < (1 << 30) else None
        ms = time_launches(verify, max(args.steps, 5), stream, before)
        vres[name] = {
            "workload": name, "batch": vc.B, "q_len": vc.T, "cache": "ring" if vc.ring else "linear",
            "slots": vc.slots, "window": vc.window, "context_lengths": [vc.len_lo, vc.len_hi],
            "algorithmic_bytes": vbytes, "ms": round(ms, 5),
            "GB/s": round(vbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(vbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        # small working sets: the floor is one cold read of the same bytes in
        # one launch (swa_peaks' hbm_read_cold_small), not the streaming rate
        pk = read_peaks() or {}
        if pk.get("hbm_read_cold_small_bytes") == vbytes:
            vres[name]["cold_read_floor_ms"] = round(pk["hbm_read_cold_small_us"] * 1e-3, 5)
            vres[name]["frac_of_cold_read_floor"] = round(pk["hbm_read_cold_small_us"] * 1e-3 / ms, 4)
        del inp, ws, ov
        torch.cuda.empty_cache()
    ga = vres[names[0]]
    if names[0].startswith("decode"):
        return {"metric": "q_len=1 decode HBM GB/s", "value": ga["GB/s"], "unit": "GB/s", "workloads": vres}
    return {
        "metric": "q_len=4 verify-decode HBM GB/s",
        "value": ga["GB/s"], "unit": "GB/s", "workloads": vres,
        "roofline": {
            "kernel": "verify_bf16_kernel + verify_combine_kernel", "bound": "hbm",
            "achieved": ga["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": ga["frac_of_hbm_peak"],
            "traffic": read_traffic("verify_bf16_ga_b64_hbm_counters.txt", VERIFY_KERNEL_SRC),
        },
    }


def run_stack_256k(args, swa, torch, dev, stream):
    """The 256K long-context block: the chunked SWA prefill of a 262144-token
    sequence (8 chunks of 32768 queries over the whole K/V) on each of 5
    sliding-window layers, then the q_len=4 verify of one global layer
    against the full 262144-token cache (B = 1, so the split-KV partitioning
    is the only parallelism).  Every layer reuses the same synthetic tensors:
    the work per layer is identical."""
    from swa_inputs import PREFILL_CONFIGS, VERIFY_CONFIGS, prefill_inputs, verify_inputs
    cfg = PREFILL_CONFIGS["swa_256k"]
    q, k, v, sinks = prefill_inputs(cfg, device=dev)
    o = torch.empty_like(q)
    chunk = cfg.chunk

    def swa_layer():
        for c0 in range(0, cfg.S, chunk):
            swa.swa_attn_prefill(q[:, c0:c0 + chunk], k, v, sinks, cfg.window, c0, cfg.scale,
                                 out=o[:, c0:c0 + chunk])

    vc = VERIFY_CONFIGS["verify_ga_256k"]
    inp = verify_inputs(vc, device=dev)
    cl = inp["cache_len"].to(torch.int32).to(dev)
    need = swa.swa_attn_verify_workspace_bytes(vc.B, vc.T, vc.Hq, vc.Hkv, vc.D, vc.slots, vc.ring, vc.window)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ov = torch.empty_like(inp["q"])
    row_b = vc.Hkv * vc.D * 2
    L = int(inp["cache_len"].to(torch.int64).sum())
    vbytes = 2 * L * row_b + 2 * vc.B * vc.T * row_b + 2 * vc.B * vc.T * vc.Hq * vc.D * 2

    def verify():
        swa.swa_attn_verify(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], cl,
                            inp["sinks"], vc.window, vc.ring, vc.scale, workspace=ws, out=ov)

    def block():
        for _ in range(5):
            swa_layer()
        verify()

    settle(block, args.settle_seconds)
    for _ in range(max(1, args.warmup)):
        block()
    n = max(3, min(args.steps, 10))
    layer_ms = time_launches(swa_layer, n, stream)
    verify_ms = time_launches(verify, n, stream)
    block_ms = time_launches(block, n, stream)
    flop = 4.0 * cfg.D * swa_pairs(cfg.S, cfg.window) * cfg.Hq * cfg.B
    del q, k, v, o, inp, ws, ov
    torch.cuda.empty_cache()
    return {
        "workload": "stack_256k: 5 SWA layers (chunked prefill, 8 x 32768 of 262144 tokens) + 1 global "
                    "q_len=4 verify at L=262144, B=1",
        "ms_swa_layer": round(layer_ms, 4),
        "swa_TFLOP/s": round(flop / (layer_ms * 1e-3) / 1e12, 2),
        "ms_global_verify": round(verify_ms, 4),
        "verify_algorithmic_bytes": vbytes,
        "verify_GB/s": round(vbytes / (verify_ms * 1e-3) / 1e9, 1),
        "ms_block": round(block_ms, 4),
    }


# The model's 48 layers: 39 sliding-window and 9 global (technical-report
# digest, "Model Architecture" hyper-parameters).  Which layers are global is
# not given; the order does not change the step time.
N_SWA_LAYERS, N_GA_LAYERS = 39, 9


def run_mtp(args, swa, torch, dev, stream):
    """One self-speculative decode step of the attention path for 64 requests:
    the q_len=4 verify of all 48 layers (9 global layers on linear caches with
    contexts U[4096, 65536], 39 SWA layers on 128-slot rings), greedy
    acceptance on bf16 logits over a 152064-token vocabulary, the append of
    the accepted rows to all 48 caches, and the length advance.  Compared with
    the plain q_len=1 decode step (same layers, argmax, append of one row)."""
    import dataclasses
    from swa_inputs import ACCEPT_CONFIGS, VERIFY_CONFIGS, accept_inputs, derive_seed, normal, verify_inputs

    acfg = ACCEPT_CONFIGS["accept_b64"]
    gcfg = VERIFY_CONFIGS["verify_ga_b64"]
    scfg = VERIFY_CONFIGS["verify_swa_b64"]
    B, T, V = gcfg.B, gcfg.T, acfg.vocab
    assert acfg.B == B and acfg.T == T and scfg.B == B and scfg.T == T
    # room for the appended rows behind the longest context
    gcfg = dataclasses.replace(gcfg, slots=gcfg.len_hi + 4 * T)
    ga_in = verify_inputs(gcfg, device=dev)
    sw_in = verify_inputs(scfg, device=dev)
    assert torch.equal(ga_in["cache_len"], sw_in["cache_len"])
    cl0 = ga_in["cache_len"].to(torch.int32).to(dev)
    L = ga_in["cache_len"].to(torch.int64)
    cl = cl0.clone()
    layers = []
    for li in range(N_SWA_LAYERS + N_GA_LAYERS):
        is_ga = li == 0 or li % 6 == 5     # 9 global layers among 48
        cfg, src = (gcfg, ga_in) if is_ga else (scfg, sw_in)
        first = not any(l["cfg"] is cfg for l in layers)
        kc = src["k_cache"] if first else src["k_cache"].clone()
        vc = src["v_cache"] if first else src["v_cache"].clone()
        shp_q, shp_kv = (B, T, cfg.Hq, cfg.D), (B, T, cfg.Hkv, cfg.D)
        q = normal(shp_q, derive_seed("mtp_bench", li, "q"), dev, torch.bfloat16)
        kn = normal(shp_kv, derive_seed("mtp_bench", li, "k"), dev, torch.bfloat16)
        vn = normal(shp_kv, derive_seed("mtp_bench", li, "v"), dev, torch.bfloat16)
        layers.append(dict(cfg=cfg, k=kc, v=vc, q=q, kn=kn, vn=vn, o=torch.empty_like(q),
                           q1=q[:, :1].contiguous(), kn1=kn[:, :1].contiguous(),
                           vn1=vn[:, :1].contiguous(), o1=torch.empty_like(q[:, :1]),
                           sinks=src["sinks"]))
    assert sum(l["cfg"] is gcfg for l in layers) == N_GA_LAYERS
    ws_need = max(swa.swa_attn_verify_workspace_bytes(B, t, gcfg.Hq, gcfg.Hkv, gcfg.D, gcfg.slots,
                                                      False, 0) for t in (1, T))
    ws = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=dev)
    n_sets = 4
    sets = [accept_inputs(acfg, device=dev, step=i) for i in range(n_sets)]
    sets1 = [(lg[:, :1].contiguous(), None) for lg, _ in sets]
    aws = torch.empty(max(swa.swa_mtp_accept_workspace_bytes(B, T, V), 1), dtype=torch.uint8, device=dev)
    tgt = torch.empty((B, T), dtype=torch.int32, device=dev)
    tgt1 = torch.empty((B, 1), dtype=torch.int32, device=dev)
    na = torch.empty((B,), dtype=torch.int32, device=dev)
    mean_tokens = 0.0
    for lg, dr in sets:
        swa.swa_mtp_greedy_accept(lg, dr, workspace=aws, target=tgt, n_append=na)
        mean_tokens += float(na.sum()) / B / n_sets
    it = [0]

    def verify_all(decode=False):
        for l in layers:
            c = l["cfg"]
            if decode:
                swa.swa_attn_verify(l["q1"], l["kn1"], l["vn1"], l["k"], l["v"], cl, l["sinks"], c.window,
                                    c.ring, c.scale, workspace=ws, out=l["o1"])
            else:
                swa.swa_attn_verify(l["q"], l["kn"], l["vn"], l["k"], l["v"], cl, l["sinks"], c.window,
                                    c.ring, c.scale, workspace=ws, out=l["o"])

    def accept(decode=False):
        lg, dr = (sets1 if decode else sets)[it[0] % n_sets]
        it[0] += 1
        swa.swa_mtp_greedy_accept(lg, dr, workspace=aws, target=tgt1 if decode else tgt, n_append=na)

    def commit(decode=False):
        for l in layers:
            swa.kv_ring_append(l["k"], l["v"], l["kn1"] if decode else l["kn"],
                               l["vn1"] if decode else l["vn"], cl, na, l["cfg"].ring)
        swa.swa_cache_advance(cl, na)

    def mtp_step():
        verify_all()
        accept()
        commit()

    def decode_step():
        verify_all(True)
        accept(True)
        commit(True)

    filler = next(l for l in layers if l["cfg"] is gcfg)

    def before():
        # restore the committed lengths, then queue two global-layer verifies
        # (about 3 ms of GPU work) so that the host has enqueued all of the
        # timed launches before the GPU reaches them: the timed region then
        # holds GPU time only, not the host's launch latency
        cl.copy_(cl0)
        for _ in range(2):
            swa.swa_attn_verify(filler["q"], filler["kn"], filler["vn"], filler["k"], filler["v"], cl,
                                filler["sinks"], 0, False, gcfg.scale, workspace=ws, out=filler["o"])

    def timed(fn):
        def once():
            cl.copy_(cl0)
            fn()
        settle(once, args.settle_seconds)
        for _ in range(args.warmup):
            once()
        return time_launches(fn, max(args.steps, 5), stream, before)

    mtp_ms = timed(mtp_step)
    dec_ms = timed(decode_step)
    ver_ms = timed(verify_all)
    acc_ms = timed(accept)
    com_ms = timed(commit)
    logit_bytes = B * T * V * 2
    per_tok = mtp_ms / mean_tokens
    del layers, ga_in, sw_in, ws, sets, sets1
    torch.cuda.empty_cache()
    return {
        "workload": "mtp_step_b64: 39 SWA ring layers + 9 global linear layers, q_len=4, vocab 152064",
        "metric": "attention-path tokens/s of self-speculative decoding (verify + accept + append)",
        "value": round(B * mean_tokens / (mtp_ms * 1e-3), 1), "unit": "tokens/s",
        "batch": B, "q_len": T, "layers": {"swa": N_SWA_LAYERS, "global": N_GA_LAYERS},
        "context_lengths": [gcfg.len_lo, gcfg.len_hi], "vocab": V,
        "per_draft_agreement": acfg.p_accept, "mean_tokens_per_step": round(mean_tokens, 4),
        "ms_per_step": round(mtp_ms, 4), "ms_verify_48_layers": round(ver_ms, 4),
        "ms_accept": round(acc_ms, 4), "ms_append_48_layers_and_advance": round(com_ms, 4),
        "attention_ms_per_token": round(per_tok, 4),
        "decode_ms_per_step": round(dec_ms, 4),
        "decode_tokens_per_s": round(B / (dec_ms * 1e-3), 1),
        "speedup_vs_decode": round(dec_ms / per_tok, 3),
        "accept_logits_bytes": logit_bytes,
        "accept_GB/s": round(logit_bytes / (acc_ms * 1e-3) / 1e9, 1),
    }


def run_rope(args, swa, torch, dev, stream, cfg, prefill_ms):
    """Partial rotary embedding (rot = 42 of 128 dims) around the 32768-token
    sliding-window prefill: the standalone in-place kernel on q and k (its HBM
    rate), and the prefill that rotates q as it stages it after one
    standalone pass over k (its cost over the plain prefill)."""
    from swa_inputs import prefill_inputs
    q, k, v, sinks = prefill_inputs(cfg, device=dev)
    rot = swa.rope_dims(cfg.D)
    base = 10000.0
    o = torch.empty_like(q)

    def rope_qk():
        swa.swa_rope_apply(q, rot, base)
        swa.swa_rope_apply(k, rot, base)

    def rope_k_fused_prefill():
        swa.swa_rope_apply(k, rot, base)
        swa.swa_attn_prefill_rope(q, k, v, sinks, cfg.window, rot, base, 0, cfg.scale, out=o)

    def fused_prefill():
        swa.swa_attn_prefill_rope(q, k, v, sinks, cfg.window, rot, base, 0, cfg.scale, out=o)

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    res = {}
    for name, fn in (("standalone_q_and_k", rope_qk), ("k_then_fused_prefill", rope_k_fused_prefill),
                     ("fused_prefill_only", fused_prefill)):
        settle(fn, args.settle_seconds)
        for _ in range(args.warmup):
            fn()
        res[name] = time_launches(fn, max(args.steps, 5), stream, lambda: flush.zero_())
    rows = cfg.B * cfg.keys * (cfg.Hq + cfg.Hkv)
    nbytes = rows * rot * 2 * 2           # rotated bf16 elements, read and written
    ms = res["standalone_q_and_k"]
    del q, k, v, o, flush
    torch.cuda.empty_cache()
    return {
        "workload": "rope_swa_32k: q [1,32768,64,128] and k [1,32768,8,128] bf16, rot 42, base 1e4",
        "rot_dim": rot,
        "standalone": {"algorithmic_bytes": nbytes, "ms": round(ms, 5),
                       "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                       "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "fraction_of_swa_prefill_time": round(ms / prefill_ms, 4)},
        "fused": {"ms_rope_k_plus_prefill_rotating_q": round(res["k_then_fused_prefill"], 5),
                  "ms_prefill_rotating_q": round(res["fused_prefill_only"], 5),
                  "ms_plain_prefill": round(prefill_ms, 5),
                  "overhead_vs_plain_prefill": round(res["k_then_fused_prefill"] / prefill_ms - 1.0, 4)},
    }


def run_backward(args, swa, torch, dev, stream, cfg):
    """One training step of the attention on the 32768-token sliding-window
    workload: the forward that saves the log-sum-exp, and the backward (dq,
    dk, dv, dsink).  Algorithmic FLOP per (query head, in-window key) pair:
    4*D forward (QK^T, PV) and 10*D backward (QK^T recomputed, dO V^T, P^T dO,
    dS^T Q, dS K)."""
    from swa_inputs import derive_seed, normal, prefill_inputs
    q, k, v, sinks = prefill_inputs(cfg, device=dev)
    dout = normal(q.shape, derive_seed(cfg.seed, "dout"), dev, torch.bfloat16)
    pairs = swa_pairs(cfg.S, cfg.window, cfg.q_offset) * cfg.B * cfg.Hq
    o, lse = swa.swa_attn_prefill_lse(q, k, v, sinks, cfg.window, cfg.q_offset, cfg.scale)
    ws = torch.empty(swa.swa_attn_backward_workspace_bytes(cfg.B, cfg.S, cfg.Hq), dtype=torch.uint8, device=dev)

    def fwd():
        swa.swa_attn_prefill_lse(q, k, v, sinks, cfg.window, cfg.q_offset, cfg.scale)

    def bwd():
        swa.swa_attn_backward(q, k, v, sinks, o, lse, dout, cfg.window, cfg.q_offset, cfg.scale, workspace=ws)

    res = {}
    for name, fn in (("forward_lse", fwd), ("backward", bwd)):
        settle(fn, args.settle_seconds)
        for _ in range(args.warmup):
            fn()
        res[name] = time_launches(fn, max(args.steps, 5), stream)
    ms_f, ms_b = res["forward_lse"], res["backward"]
    # HBM bytes the backward must move at least: q, o, dO read, dq written
    # (B*S*Hq*D each), k, v read and dk, dv written (B*Sk*Hkv*D each), the
    # lse read, all bf16 except lse (fp32)
    bytes_b = (4 * cfg.B * cfg.S * cfg.Hq * cfg.D + 4 * cfg.B * cfg.keys * cfg.Hkv * cfg.D) * 2 + cfg.B * cfg.S * cfg.Hq * 4
    del q, k, v, o, lse, dout, ws
    torch.cuda.empty_cache()
    return {
        "workload": "swa_32k training step: B1 S32768 Hq64 Hkv8 D128 W128 bf16 with sinks",
        "ms_forward_lse": round(ms_f, 5), "ms_backward": round(ms_b, 5),
        "forward_TFLOP/s": round(4.0 * cfg.D * pairs / (ms_f * 1e-3) / 1e12, 1),
        "backward_TFLOP/s": round(10.0 * cfg.D * pairs / (ms_b * 1e-3) / 1e12, 1),
        "backward_min_bytes": bytes_b,
        "backward_GB/s_of_min_bytes": round(bytes_b / (ms_b * 1e-3) / 1e9, 1),
        "step_ms": round(ms_f + ms_b, 5),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note, not part of this build).", file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_sliding_window_swa_amd as swa
    from swa_inputs import PREFILL_CONFIGS

    swa.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))
        return

    if args.torch_copy_ceiling:
        n = 4 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        settle(lambda: dst.copy_(src), 0.5)
        ms = time_launches(lambda: dst.copy_(src), 10, stream)
        print(json.dumps({"measure": "hbm_copy_torch", "bytes_read_plus_written": 2 * n, "ms": round(ms, 4),
                          "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    if args.only == "ga":
        print(json.dumps({"ga_prefill": run_ga(args, swa, torch, dev, stream)}), flush=True)
        return
    if args.only == "verify":
        print(json.dumps({"verify": run_verify(args, swa, torch, dev, stream)}), flush=True)
        return
    if args.only == "mtp":
        print(json.dumps({"mtp_step": run_mtp(args, swa, torch, dev, stream)}), flush=True)
        return
    if args.only == "stack":
        print(json.dumps({"stack_256k": run_stack_256k(args, swa, torch, dev, stream)}), flush=True)
        return
    if args.only == "backward":
        print(json.dumps({"backward": run_backward(args, swa, torch, dev, stream, PREFILL_CONFIGS["swa_32k"])}),
              flush=True)
        return
    if args.only == "rope":
        print(json.dumps({"rope": run_rope(args, swa, torch, dev, stream, PREFILL_CONFIGS["swa_32k"], 0.28)}),
              flush=True)
        return

    cfg = PREFILL_CONFIGS["swa_32k"]
    pres, tensors = run_prefill(args, swa, torch, dev, stream, cfg)
    result = {
        "metric": "SWA(W=128)+sink attn: prefill TFLOP/s; q_len=4 verify-decode HBM GB/s",
        "value": round(pres["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": args.settle_seconds,
        "ms_per_step": round(pres["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": pres["config"],
        "roofline": pres["roofline"],
    }
    if args.only is None and not args.no_verify:
        result["ga_prefill"] = run_ga(args, swa, torch, dev, stream)
        result["verify"] = run_verify(args, swa, torch, dev, stream)
        result["decode"] = run_verify(args, swa, torch, dev, stream, ("decode_ga_b64", "decode_swa_b64"))
        result["mtp_step"] = run_mtp(args, swa, torch, dev, stream)
        result["rope"] = run_rope(args, swa, torch, dev, stream, cfg, pres["roofline"]["kernel_ms"])
        result["backward"] = run_backward(args, swa, torch, dev, stream, cfg)
        result["stack_256k"] = run_stack_256k(args, swa, torch, dev, stream)
    peaks = read_peaks()
    if peaks is not None:
        # fractions of the ceilings measured on this GPU: the SWA prefill moves
        # as many bytes out as in (copy-like), the verify reads, the global
        # prefill is a contraction
        result["measured_ceilings"] = peaks
        result["roofline"]["frac_of_measured_copy"] = round(
            result["roofline"]["achieved"] / peaks["hbm_copy_GBs"], 4)
        if "hbm_copy_head_groups_GBs" in peaks:
            result["roofline"]["frac_of_measured_head_group_copy"] = round(
                result["roofline"]["achieved"] / peaks["hbm_copy_head_groups_GBs"], 4)
        if "verify" in result:
            v = result["verify"]["roofline"]
            v["frac_of_measured_read"] = round(v["achieved"] / peaks["hbm_read_GBs"], 4)
            if "hbm_read_head_rows_GBs" in peaks:
                v["frac_of_measured_head_rows_read"] = round(v["achieved"] / peaks["hbm_read_head_rows_GBs"], 4)
        if "ga_prefill" in result:
            gp = result["ga_prefill"]
            gp["frac_of_measured_mfma"] = round(gp["TFLOP/s"] / peaks["mfma_bf16_TFLOPs"], 4)
            if "mfma_bf16_random_operands_TFLOPs" in peaks:
                gp["frac_of_measured_mfma_random_operands"] = round(
                    gp["TFLOP/s"] / peaks["mfma_bf16_random_operands_TFLOPs"], 4)
    if args.only is None and not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, *tensors, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(cfg, q, k, v, sinks, target_s):
    """Time the CPU oracle on a bounded sample of rows of the same workload
    and convert to algorithmic TFLOP/s."""
    import torch
    import oracle
    from swa_inputs import sample_rows

    threads = oracle.num_threads()
    kk = k[0].float().cpu()
    vv = v[0].float().cpu()
    s = sinks.cpu()

    def run(n):
        rows = sample_rows(cfg.S, n, 777 + n, ())
        qr = q[0].index_select(0, rows.to(q.device)).cpu()
        t0 = time.perf_counter()
        oracle.prefill_rows(qr, rows, kk, vv, s, cfg.window, cfg.q_offset, cfg.scale)
        dt = time.perf_counter() - t0
        pairs = sum(min(int(r) + cfg.q_offset + 1, cfg.window) for r in rows) * cfg.Hq
        return dt, pairs, len(rows)

    dt, pairs, n = run(256)
    scale = max(1.0, target_s / max(dt, 1e-3))
    n2 = min(cfg.S, int(256 * scale))
    dt, pairs, n = run(n2)
    flop = 4.0 * cfg.D * pairs
    return {
        "value": round(flop / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n} of {cfg.S} query rows x {cfg.Hq} heads of the swa_32k prefill "
                  f"(fp64 C oracle, OpenMP), {dt:.1f} s",
        "seconds": round(dt, 2),
        "rows_per_s": round(n * cfg.Hq / dt, 1),
        "cpu_model": cpu_model(),
    }


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
