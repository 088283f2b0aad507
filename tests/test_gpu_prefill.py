"""GPU parity of swa_attn_prefill against the CPU oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, F32_TOL, assert_close, device, rel_l2, swa
from swa_inputs import PREFILL_CONFIGS, PrefillConfig, derive_seed, normal, prefill_inputs, sample_rows

pytestmark = pytest.mark.gpu


def _run(cfg: PrefillConfig, sinks_mode="normal", q_offset=None):
    dev = device()
    m = swa()
    q, k, v, sinks = prefill_inputs(cfg)
    if sinks_mode == "none":
        sinks = None
    elif sinks_mode == "-inf":
        sinks = torch.full_like(sinks, float("-inf"))
    elif sinks_mode == "large":
        sinks = sinks * 6.0
    off = cfg.q_offset if q_offset is None else q_offset
    o = m.swa_attn_prefill(q.to(dev), k.to(dev), v.to(dev), None if sinks is None else sinks.to(dev),
                           cfg.window, off, cfg.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, sinks, cfg.window, off, cfg.scale)
    return o, ref


def _cfg(name, B, S, Hq, Hkv, D, W, dtype, Sk=None, seed=None):
    return PrefillConfig(name, B, S, Hq, Hkv, D, W, dtype, seed=seed or derive_seed(name) % 100000, Sk=Sk)


F32_CASES = [
    PREFILL_CONFIGS["tiny_f32"],                          # the tiny fp32 workload
    _cfg("f32_d128_g2", 2, 200, 4, 2, 128, 50, "f32"),
    _cfg("f32_global", 1, 150, 8, 2, 64, 0, "f32"),
    _cfg("f32_prefix", 1, 77, 6, 3, 64, 32, "f32", Sk=140),
    _cfg("f32_w1", 1, 40, 2, 1, 64, 1, "f32"),
]


@pytest.mark.parametrize("cfg", F32_CASES, ids=lambda c: c.name)
def test_prefill_f32(cfg):
    o, ref = _run(cfg)
    assert_close(o, ref, F32_TOL, cfg.name)


BF16_CASES = [
    _cfg("swa_ragged", 1, 300, 16, 2, 128, 128, "bf16"),
    _cfg("swa_heads64", 2, 513, 64, 8, 128, 128, "bf16"),
    _cfg("w1", 1, 200, 8, 1, 128, 1, "bf16"),
    _cfg("w127", 1, 400, 8, 1, 128, 127, "bf16"),
    _cfg("w129", 1, 400, 8, 1, 128, 129, "bf16"),
    _cfg("w512", 1, 900, 8, 1, 128, 512, "bf16"),
    _cfg("global", 1, 700, 8, 1, 128, 0, "bf16"),
    _cfg("global_g8", 1, 333, 64, 8, 128, 0, "bf16"),
    _cfg("g1", 1, 260, 4, 4, 128, 128, "bf16"),
    _cfg("g2", 1, 260, 8, 4, 128, 128, "bf16"),
    _cfg("g4", 1, 260, 8, 2, 128, 128, "bf16"),
    _cfg("g16", 1, 130, 32, 2, 128, 128, "bf16"),
    _cfg("g32", 1, 100, 32, 1, 128, 64, "bf16"),
    _cfg("d64", 2, 300, 16, 2, 64, 128, "bf16"),
    _cfg("d64_global", 1, 257, 8, 1, 64, 0, "bf16"),
    _cfg("prefix", 1, 190, 16, 2, 128, 128, "bf16", Sk=450),
    _cfg("prefix_global", 1, 61, 16, 2, 128, 0, "bf16", Sk=300),
    # the no-window kernel at every group size (waves of one workgroup whose
    # queries end in different key tiles fold the later tiles fully masked)
    _cfg("global_g1", 1, 300, 4, 4, 128, 0, "bf16"),
    _cfg("global_g2_d64", 1, 170, 8, 4, 64, 0, "bf16"),
    _cfg("global_g4", 1, 300, 8, 2, 128, 0, "bf16"),
    _cfg("global_g16", 1, 130, 32, 2, 128, 0, "bf16"),
    _cfg("global_g32", 2, 70, 32, 1, 128, 0, "bf16"),
    _cfg("prefix_global_g4", 1, 77, 8, 2, 128, 0, "bf16", Sk=301),
    _cfg("one_row", 1, 1, 8, 1, 128, 128, "bf16"),
    _cfg("one_row_offset", 1, 1, 8, 1, 128, 128, "bf16", Sk=1000),
    _cfg("short", 3, 17, 8, 1, 128, 4, "bf16"),
]


@pytest.mark.parametrize("cfg", BF16_CASES, ids=lambda c: c.name)
def test_prefill_bf16(cfg):
    o, ref = _run(cfg)
    assert_close(o, ref, BF16_TOL, cfg.name)
    assert rel_l2(o, ref) < 1e-2


@pytest.mark.parametrize("mode", ["none", "-inf", "large"])
def test_prefill_bf16_sink_modes(mode):
    cfg = _cfg("sinks_" + mode, 1, 260, 16, 2, 128, 128, "bf16")
    o, ref = _run(cfg, sinks_mode=mode)
    assert_close(o, ref, BF16_TOL, cfg.name)


def test_prefill_chunked_equals_oracle():
    """Chunked prefill (queries [c0, c0 + C) over the full K/V with q_offset = c0)."""
    dev = device()
    m = swa()
    cfg = _cfg("chunks", 1, 640, 16, 2, 128, 128, "bf16")
    q, k, v, sinks = prefill_inputs(cfg)
    ref = oracle.prefill(q, k, v, sinks, cfg.window, 0, cfg.scale)
    kd, vd, sd = k.to(dev), v.to(dev), sinks.to(dev)
    for c0 in range(0, 640, 160):
        o = m.swa_attn_prefill(q[:, c0:c0 + 160].contiguous().to(dev), kd, vd, sd, cfg.window, c0)
        torch.cuda.synchronize()
        assert_close(o, ref[:, c0:c0 + 160], BF16_TOL, f"chunk {c0}")


@pytest.mark.parametrize("D,S", [(64, 300), (64, 301), (128, 301)])
def test_prefill_repeated_calls_stable(D, S):
    """Many calls of the sliding-window kernel against one oracle result.

    Guards the output path of the strip kernel: a 16-byte store whose data
    registers are rewritten too early corrupts a few lanes only now and then,
    so one call is not enough to see it.  S = 301 leaves a partial wave."""
    dev = device()
    m = swa()
    cfg = _cfg(f"repeat_d{D}_s{S}", 2, S, 16, 2, D, 128, "bf16")
    q, k, v, sinks = prefill_inputs(cfg)
    ref = oracle.prefill(q, k, v, sinks, cfg.window, 0, cfg.scale)
    qd, kd, vd, sd = q.to(dev), k.to(dev), v.to(dev), sinks.to(dev)
    for rep in range(60):
        out = torch.full_like(qd, float("nan"))
        m.swa_attn_prefill(qd, kd, vd, sd, cfg.window, 0, cfg.scale, out=out)
        torch.cuda.synchronize()
        assert_close(out, ref, BF16_TOL, f"{cfg.name} call {rep}")


def test_prefill_deterministic():
    dev = device()
    m = swa()
    cfg = _cfg("determinism", 1, 500, 64, 8, 128, 0, "bf16")
    q, k, v, s = [t.to(dev) for t in prefill_inputs(cfg)]
    o1 = m.swa_attn_prefill(q, k, v, s, cfg.window)
    o2 = m.swa_attn_prefill(q, k, v, s, cfg.window)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_prefill_out_of_window_keys_unread():
    """Keys that can never enter any window of the launched queries are not
    read: poisoning them with NaN leaves the output finite and correct."""
    dev = device()
    m = swa()
    cfg = _cfg("poison", 1, 100, 8, 1, 128, 128, "bf16", Sk=600)
    q, k, v, s = prefill_inputs(cfg)
    ref = oracle.prefill(q, k, v, s, 128, 500, cfg.scale)
    # queries sit at 500..599, so keys < 373 are outside every window; the
    # kernel reads whole 32-key tiles, so poison up to the tile below 373
    k[:, :352] = float("nan")
    v[:, :352] = float("nan")
    o = m.swa_attn_prefill(q.to(dev), k.to(dev), v.to(dev), s.to(dev), 128, 500)
    torch.cuda.synchronize()
    assert_close(o, ref, BF16_TOL, "poisoned prefix")


# ---------------------------------------------------------------- full sizes

def _full_size(cfg: PrefillConfig, n_rows: int, forced):
    """Run the whole workload on the GPU (chunked if the config says so) and
    check sampled rows against the oracle."""
    dev = device()
    m = swa()
    print(f"[full-size] {cfg.name}: generating inputs on {dev}", flush=True)
    q, k, v, sinks = prefill_inputs(cfg, device=dev)
    o = torch.empty_like(q)
    chunk = cfg.chunk or cfg.S
    for c0 in range(0, cfg.S, chunk):
        m.swa_attn_prefill(q[:, c0:c0 + chunk], k, v, sinks, cfg.window, cfg.q_offset + c0,
                           cfg.scale, out=o[:, c0:c0 + chunk])
    torch.cuda.synchronize()
    rows = sample_rows(cfg.S, n_rows, cfg.seed, forced)
    rows_d = rows.to(dev)
    q_rows = q[0].index_select(0, rows_d).cpu()
    got = o[0].index_select(0, rows_d).cpu()
    assert torch.isfinite(got.float()).all()
    print(f"[full-size] {cfg.name}: oracle on {len(rows)} rows x {cfg.Hq} heads", flush=True)
    if cfg.window > 0:
        # only the keys the sampled rows can see
        lo = max(0, int(rows.min()) + cfg.q_offset - cfg.window + 1)
        hi = int(rows.max()) + cfg.q_offset + 1
        kk, vv = k[0, lo:hi].cpu(), v[0, lo:hi].cpu()
        ref = oracle.prefill_rows(q_rows, rows, kk, vv, sinks.cpu(), cfg.window, cfg.q_offset,
                                  cfg.scale, k_base=lo)
    else:
        hi = int(rows.max()) + cfg.q_offset + 1
        ref = oracle.prefill_rows(q_rows, rows, k[0, :hi].cpu(), v[0, :hi].cpu(), sinks.cpu(),
                                  cfg.window, cfg.q_offset, cfg.scale)
    assert_close(got, ref, BF16_TOL, cfg.name)
    for h in range(cfg.Hq):
        assert rel_l2(got[:, h], ref[:, h]) < 1e-2, f"head {h} relative L2 too large"


def test_full_size_swa_32k():
    S = 32768
    _full_size(PREFILL_CONFIGS["swa_32k"], 2048, (0, 1, 31, 32, 127, 128, 129, S - 2, S - 1))


def test_full_size_global_32k():
    S = 32768
    _full_size(PREFILL_CONFIGS["ga_32k"], 256, (0, 1, 127, 128, 129, S - 1))


def test_full_size_swa_256k_chunked():
    cfg = PREFILL_CONFIGS["swa_256k"]
    forced = []
    for c0 in range(0, cfg.S, cfg.chunk):
        forced += [c0 + d for d in (0, 1, 126, 127, 128)]
        forced += [c0 - 1]
    _full_size(cfg, 1024, forced + [cfg.S - 1])
