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
    # the strip kernel with block starts off the 32-key tile grid (q_offset
    # % 32 != 0): windows of 96 or less still fit its 6-tile ring
    _cfg("strip_w96_g8_offset170", 1, 200, 64, 8, 128, 96, "bf16", Sk=370),
    _cfg("strip_w96_g4_offset177", 1, 200, 16, 4, 128, 96, "bf16", Sk=377),
    _cfg("strip_w64_d64_offset13", 2, 150, 16, 2, 64, 64, "bf16", Sk=163),
    _cfg("strip_w33_g8_offset1", 1, 97, 16, 2, 128, 33, "bf16", Sk=98),
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


@pytest.mark.parametrize("W,G,with_sink", [(128, 8, False), (128, 8, True), (96, 4, False), (512, 8, False),
                                           (0, 8, False), (0, 8, True), (0, 2, False)])
def test_prefill_bf16_large_scores(W, G, with_sink):
    """Queries scaled by 8 (exact in bf16): scores far above the running
    shift keep arriving, so the kernels' rescale path (raising the shift,
    rescaling the accumulator, recomputing the tile's weights) runs often,
    also while no sink has fixed the shift yet.  Output and saved LSE
    against the oracle."""
    dev = device()
    m = swa()
    cfg = _cfg(f"large_scores_w{W}_g{G}_{int(with_sink)}", 1, 300, 16, 16 // G, 128, W, "bf16", Sk=332)
    q, k, v, sinks = prefill_inputs(cfg)
    q = q * 8
    sinks = sinks if with_sink else None
    sd = None if sinks is None else sinks.to(dev)
    o = m.swa_attn_prefill(q.to(dev), k.to(dev), v.to(dev), sd, W, cfg.q_offset, cfg.scale)
    o2, lse = m.swa_attn_prefill_lse(q.to(dev), k.to(dev), v.to(dev), sd, W, cfg.q_offset, cfg.scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, sinks, W, cfg.q_offset, cfg.scale, want_lse=True)
    assert_close(o, ref["o"], BF16_TOL, cfg.name)
    assert_close(o2, ref["o"], BF16_TOL, cfg.name + " (lse variant)")
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() <= 2 * 2.0 ** -9


# The strip kernel's continuous skewed pipeline (query lengths a multiple of
# the 32-token block, no rotary mode): strips of several blocks (B * Hkv
# workgroups share the CUs, so each strip gets n_tb * B * Hkv / CUs blocks),
# unaligned offsets, D 64, G 4, W = 1 (one tile per block), a prefix.
SKEW_CASES = [
    # name, B, S, Hq, Hkv, D, W, Sk, q_offset
    ("skew_w128_g8", 8, 1024, 64, 8, 128, 128, None, 0),
    ("skew_w96_g4_unaligned", 4, 512, 32, 8, 128, 96, 682, 170),
    ("skew_w64_d64_g8", 8, 512, 64, 8, 64, 64, None, 0),
    ("skew_w1_g8", 8, 512, 64, 8, 128, 1, None, 0),
    ("skew_w32_d64_g4_offset", 4, 1024, 32, 8, 64, 32, 1088, 64),
    ("skew_w128_prefix", 2, 640, 64, 8, 128, 128, 1000, 352),
    ("skew_one_block_strips", 1, 96, 16, 2, 128, 128, None, 0),
]


@pytest.mark.parametrize("case", SKEW_CASES, ids=[c[0] for c in SKEW_CASES])
def test_prefill_skewed_strips(case):
    """Every row and head against the oracle; the log-sum-exp variant gives
    the same output bit for bit and its LSE within the bound of the
    training-forward tests."""
    name, B, S, Hq, Hkv, D, W, Sk, off = case
    dev = device()
    m = swa()
    cfg = _cfg(name, B, S, Hq, Hkv, D, W, "bf16", Sk=Sk)
    q, k, v, sinks = prefill_inputs(cfg)
    ref = oracle.prefill(q, k, v, sinks, W, off, cfg.scale, want_lse=True)
    qd, kd, vd, sd = q.to(dev), k.to(dev), v.to(dev), sinks.to(dev)
    o = m.swa_attn_prefill(qd, kd, vd, sd, W, off, cfg.scale)
    o2, lse = m.swa_attn_prefill_lse(qd, kd, vd, sd, W, off, cfg.scale)
    torch.cuda.synchronize()
    assert_close(o, ref["o"], BF16_TOL, name)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), f"{name}: LSE variant output differs"
    err = np.abs(lse.cpu().numpy() - ref["lse"]).max()
    assert err <= 2 * 2.0 ** -9, f"{name}: LSE error {err:.3e}"


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


POISON_CASES = [
    # name, B, Sq, q_offset, Sk, Hq, Hkv, D, window, dtype
    ("strip_w128", 2, 100, 512, 700, 64, 8, 128, 128, "bf16"),       # keys used 385..611
    ("strip_w96_unaligned", 1, 200, 250, 520, 64, 8, 128, 96, "bf16"),
    ("skew_strip_w96_unaligned", 1, 192, 250, 520, 64, 8, 128, 96, "bf16"),
    ("strip_w64_g4_d64", 1, 90, 310, 460, 16, 4, 64, 64, "bf16"),
    ("generic_w128_unaligned", 1, 100, 600, 760, 16, 2, 128, 128, "bf16"),
    ("generic_w512", 1, 200, 700, 1000, 8, 1, 128, 512, "bf16"),
    ("generic_g2_w64", 1, 50, 370, 470, 8, 4, 128, 64, "bf16"),
    ("global_top_tail", 1, 77, 423, 560, 16, 2, 128, 0, "bf16"),
    ("global_g8_top_tail", 1, 33, 267, 340, 64, 8, 64, 0, "bf16"),
    ("f32_w128", 1, 100, 600, 760, 8, 2, 64, 128, "f32"),
]


@pytest.mark.parametrize("case", POISON_CASES, ids=[c[0] for c in POISON_CASES])
def test_prefill_unused_key_rows_may_hold_nan(case):
    """Rows of k and v that no query of the call can see (below the first
    query's window, at or past the last query) may hold NaN: a chunked
    prefill over a partly filled cache.  The poisoned rows share 32-key tiles
    with used ones."""
    name, B, Sq, off, Sk, Hq, Hkv, D, W, dtype = case
    dev = device()
    m = swa()
    cfg = _cfg(name, B, Sq, Hq, Hkv, D, W, dtype, Sk=Sk)
    q, k, v, s = prefill_inputs(cfg)
    ref = oracle.prefill(q, k, v, s, W, off, cfg.scale)
    lo = max(0, off - W + 1) if W > 0 else 0
    hi = off + Sq
    assert hi < Sk and hi % 32 != 0 and (W <= 0 or lo % 32 != 0), "poison must share tiles with used rows"
    kp, vp = k.clone(), v.clone()
    for t in (kp, vp):
        t[:, :lo] = float("nan")
        t[:, hi:] = float("nan")
    o = m.swa_attn_prefill(q.to(dev), kp.to(dev), vp.to(dev), s.to(dev), W, off, cfg.scale)
    torch.cuda.synchronize()
    assert_close(o, ref, BF16_TOL if dtype == "bf16" else F32_TOL, name)
    if dtype == "bf16":
        o2, _ = m.swa_attn_prefill_lse(q.to(dev), kp.to(dev), vp.to(dev), s.to(dev), W, off, cfg.scale)
        torch.cuda.synchronize()
        if W > 0:
            assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
        else:
            assert_close(o2, ref, BF16_TOL, name + " (lse variant)")


# ---------------------------------------------------------------- full sizes

def _full_size(cfg: PrefillConfig, n_rows, forced=()):
    """Run the whole workload on the GPU (chunked if the config says so) and
    check it against the oracle: every row when n_rows is None (in slabs of
    4096 rows), else n_rows sampled rows plus the forced ones."""
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
    if n_rows is None:
        slabs = [torch.arange(r0, min(r0 + 4096, cfg.S)) for r0 in range(0, cfg.S, 4096)]
    else:
        slabs = [sample_rows(cfg.S, n_rows, cfg.seed, forced)]
    print(f"[full-size] {cfg.name}: oracle on {sum(len(r) for r in slabs)} rows x {cfg.Hq} heads", flush=True)
    sinks_c = sinks.cpu()
    sq_err = sq_ref = None
    for rows in slabs:
        rows_d = rows.to(dev)
        q_rows = q[0].index_select(0, rows_d).cpu()
        got = o[0].index_select(0, rows_d).cpu()
        assert torch.isfinite(got.float()).all()
        # only the keys the rows can see
        lo = max(0, int(rows.min()) + cfg.q_offset - cfg.window + 1) if cfg.window > 0 else 0
        hi = int(rows.max()) + cfg.q_offset + 1
        ref = oracle.prefill_rows(q_rows, rows, k[0, lo:hi].cpu(), v[0, lo:hi].cpu(), sinks_c, cfg.window,
                                  cfg.q_offset, cfg.scale, k_base=lo)
        assert_close(got, ref, BF16_TOL, f"{cfg.name} rows {int(rows.min())}..{int(rows.max())}")
        d = (got.double().numpy() - ref) ** 2
        e = (d.sum(axis=(0, 2)), (ref ** 2).sum(axis=(0, 2)))
        sq_err = e[0] if sq_err is None else sq_err + e[0]
        sq_ref = e[1] if sq_ref is None else sq_ref + e[1]
    rel = np.sqrt(sq_err / sq_ref)
    print(f"[full-size] {cfg.name}: worst per-head relative L2 {rel.max():.3e}", flush=True)
    assert (rel < 1e-2).all(), f"heads {np.nonzero(rel >= 1e-2)[0].tolist()} relative L2 too large"


def test_full_size_swa_32k():
    """Every row of the 32K sliding-window prefill (32768 rows x 64 heads)."""
    _full_size(PREFILL_CONFIGS["swa_32k"], None)


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
