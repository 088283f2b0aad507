"""GPU parity of the partial rotary embedding against the oracle, alone and
composed with prefill and verify (rotated queries and keys, caches holding
rotated keys)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, F32_TOL, assert_close, device, swa
from swa_inputs import (PrefillConfig, VerifyConfig, derive_seed, normal, prefill_inputs,
                        ring_from_history, verify_inputs)

pytestmark = pytest.mark.gpu

ROPE_CASES = [
    # name, B, S, H, D, rot, base, dtype, pos0, pos_offset
    ("q_ga_256k_positions", 2, 300, 64, 128, 42, 640000.0, "bf16", [0, 262100], 5),
    ("k_swa", 3, 257, 8, 128, 42, 10000.0, "bf16", None, 0),
    ("f32_d64", 2, 100, 4, 64, 20, 5e6, "f32", [7, 100000], 0),
    ("full_rotation", 1, 65, 8, 128, 128, 10000.0, "bf16", [3], 0),
    ("one_pair", 2, 33, 8, 64, 2, 10000.0, "bf16", None, 11),
    ("odd_heads", 2, 77, 3, 64, 20, 10000.0, "bf16", [1, 2], 0),
    ("one_head_many_positions", 1, 1000, 1, 256, 256, 5e6, "f32", None, 262144),
    ("d256_bf16", 2, 40, 5, 256, 84, 640000.0, "bf16", [9, 0], 0),
]


def _check_rope(got, x, ref, rot, dtype, name):
    g = got.float().cpu().numpy()
    xf = x.float().numpy()
    # dimensions past rot are untouched, bit for bit
    assert np.array_equal(got.cpu()[..., rot:].view(torch.int16 if dtype == "bf16" else torch.int32),
                          x[..., rot:].view(torch.int16 if dtype == "bf16" else torch.int32)), name
    err = np.abs(g[..., :rot] - ref[..., :rot])
    if dtype == "bf16":
        # correctly rounded to bf16: half an ulp of the reference's binade
        # (bf16 keeps 8 significant bits), plus fp32 arithmetic noise
        _, e = np.frexp(ref[..., :rot])
        bound = np.ldexp(1.0, e - 9) * 1.001 + 1e-6 * (np.abs(ref[..., :rot]) + 1.0)
    else:
        bound = 1e-6 * (np.abs(xf[..., :rot]).max(axis=-1, keepdims=True) + 1.0)
    assert (err <= bound).all(), f"{name}: max excess {(err - bound).max():.3e}"


@pytest.mark.parametrize("case", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_rope_matches_oracle(case):
    name, B, S, H, D, rot, base, dtype, pos0, off = case
    dev = device()
    m = swa()
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = normal((B, S, H, D), derive_seed("rope", name), dtype=dt)
    xg = x.to(dev)
    p0 = None if pos0 is None else torch.tensor(pos0, dtype=torch.int32, device=dev)
    m.swa_rope_apply(xg, rot, base, p0, off)
    torch.cuda.synchronize()
    pos = (np.zeros(B, np.int64) if pos0 is None else np.array(pos0))[:, None] + off + np.arange(S)[None, :]
    ref = oracle.rope(x, pos, rot, base)
    _check_rope(xg, x, ref, rot, dtype, name)


@pytest.mark.parametrize("window,q_offset", [(128, 0), (0, 0), (128, 200), (0, 200)])
def test_rope_then_prefill(window, q_offset):
    dev = device()
    m = swa()
    S, Sk = 300, 300 + q_offset
    cfg = PrefillConfig("rope_prefill", 1, S, 16, 2, 128, window, "bf16", seed=31, Sk=Sk)
    q, k, v, sinks = prefill_inputs(cfg)
    rot, base = 42, 10000.0 if window > 0 else 640000.0
    qg, kg = q.to(dev), k.to(dev)
    m.swa_rope_apply(qg, rot, base, None, q_offset)
    m.swa_rope_apply(kg, rot, base, None, 0)
    o = m.swa_attn_prefill(qg, kg, v.to(dev), sinks.to(dev), window, q_offset, cfg.scale)
    torch.cuda.synchronize()
    q_ref = oracle.rope(q, q_offset + np.arange(S)[None, :], rot, base)
    k_ref = oracle.rope(k, np.arange(Sk)[None, :], rot, base)
    ref = oracle.prefill(q_ref, k_ref, v, sinks, window, q_offset, cfg.scale)
    assert_close(o, ref, BF16_TOL, f"rope prefill W={window} off={q_offset}")


@pytest.mark.parametrize("ring", [True, False])
def test_rope_then_verify(ring):
    """Keys are rotated once (history at its positions, new rows at
    cache_len + t) and the cache holds rotated keys; queries are rotated at
    cache_len + t."""
    dev = device()
    m = swa()
    W = 128 if ring else 0
    slots = 128 if ring else 1200
    cfg = VerifyConfig("rope_verify", 6, 4, 64, 8, 128, W, ring, slots, 0, 0, "bf16", seed=33)
    lens = [0, 1, 127, 128, 129, 1100]
    inp = verify_inputs(cfg, cache_len=lens, build_cache=False)
    rot, base = 42, 10000.0 if ring else 5e6
    L = inp["cache_len"]
    L_dev = L.to(torch.int32).to(dev)
    base_dev = inp["hist_base"].to(torch.int32).to(dev)
    kh = inp["k_hist"].to(dev)
    m.swa_rope_apply(kh, rot, base, base_dev, 0)
    kc = ring_from_history(kh, inp["hist_base"], L, slots) if ring else kh
    vc = ring_from_history(inp["v_hist"].to(dev), inp["hist_base"], L, slots) if ring else inp["v_hist"].to(dev)
    qg, kn = inp["q"].to(dev), inp["k_new"].to(dev)
    m.swa_rope_apply(qg, rot, base, L_dev, 0)
    m.swa_rope_apply(kn, rot, base, L_dev, 0)
    o = m.swa_attn_verify(qg, kn, inp["v_new"].to(dev), kc.contiguous(), vc.contiguous(), L_dev,
                          inp["sinks"].to(dev), W, ring, cfg.scale)
    torch.cuda.synchronize()
    T = cfg.T
    newpos = L.numpy()[:, None] + np.arange(T)[None, :]
    histpos = inp["hist_base"].numpy()[:, None] + np.arange(inp["k_hist"].shape[1])[None, :]
    q_ref = oracle.rope(inp["q"], newpos, rot, base)
    kn_ref = oracle.rope(inp["k_new"], newpos, rot, base)
    kh_ref = oracle.rope(inp["k_hist"], histpos, rot, base)
    ref = oracle.verify(q_ref, kn_ref, inp["v_new"], kh_ref, inp["v_hist"], inp["hist_base"], L,
                        inp["sinks"], W, cfg.scale)
    assert_close(o, ref, BF16_TOL, f"rope verify ring={ring}")


FUSED_CASES = [
    # name, B, S, Sk, Hq, Hkv, D, window, rot
    ("w128_g8_d128", 1, 300, 300, 16, 2, 128, 128, 42),
    ("w128_g8_chunk", 2, 200, 520, 16, 2, 128, 128, 42),
    ("w128_g4_d128", 1, 257, 257, 16, 4, 128, 128, 42),
    ("w64_g8_d64", 2, 190, 190, 16, 2, 64, 64, 20),
    ("w128_g4_d64_rot32", 1, 161, 193, 8, 2, 64, 128, 32),
    ("w1_g8", 1, 70, 70, 8, 1, 128, 1, 42),
    ("model_heads", 1, 600, 600, 64, 8, 128, 128, 42),
    # block starts off the 32-key tile grid (q_offset % 32 != 0)
    ("w96_g8_offset170", 1, 200, 370, 64, 8, 128, 96, 42),
    ("w96_g4_d64_offset21", 1, 150, 171, 16, 4, 64, 96, 20),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_prefill_rope_fused_matches_oracle(case):
    """Queries rotated while they are staged (q itself untouched) match the
    oracle's attention over rotated queries and keys."""
    name, B, S, Sk, Hq, Hkv, D, W, rot = case
    dev = device()
    m = swa()
    cfg = PrefillConfig(name, B, S, Hq, Hkv, D, W, "bf16", seed=derive_seed("fused", name) % 100000, Sk=Sk)
    q, k, v, sinks = prefill_inputs(cfg)
    base = 10000.0
    qg, kg = q.to(dev), k.to(dev)
    m.swa_rope_apply(kg, rot, base, None, 0)
    o = m.swa_attn_prefill_rope(qg, kg, v.to(dev), sinks.to(dev), W, rot, base, cfg.q_offset, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(qg.cpu().view(torch.int16), q.view(torch.int16)), "q was modified"
    q_ref = oracle.rope(q, cfg.q_offset + np.arange(S)[None, :], rot, base)
    k_ref = oracle.rope(k, np.arange(Sk)[None, :], rot, base)
    ref = oracle.prefill(q_ref, k_ref, v, sinks, W, cfg.q_offset, cfg.scale)
    assert_close(o, ref, BF16_TOL, name)


def test_prefill_rope_zero_rot_is_prefill():
    dev = device()
    m = swa()
    cfg = PrefillConfig("rot0", 1, 200, 16, 2, 128, 128, "bf16", seed=5)
    q, k, v, sinks = (t.to(dev) for t in prefill_inputs(cfg))
    a = m.swa_attn_prefill(q, k, v, sinks, 128)
    b = m.swa_attn_prefill_rope(q, k, v, sinks, 128, 0, 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefill_rope_unsupported_configs_raise():
    dev = device()
    m = swa()
    q = torch.zeros((1, 64, 16, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device=dev)
    for window, rot in ((0, 42), (128, 66), (1024, 42)):
        with pytest.raises(m.SwaError):
            m.swa_attn_prefill_rope(q, k, k, None, window, rot, 10000.0)
    # a chunk whose first query is not 32-aligned: the window needs 7 key tiles
    k2 = torch.zeros((1, 64 + 333, 2, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(m.SwaError):
        m.swa_attn_prefill_rope(q, k2, k2, None, 128, 42, 10000.0, q_offset=333)


def test_full_size_rope_32k():
    """The bench's RoPE workload: every rotated element of q [1,32768,64,128]
    and k [1,32768,8,128] against the oracle, at positions 229376 .. 262143
    (the 256K stack's last chunk) for q and 0 .. 32767 for k."""
    from swa_inputs import PREFILL_CONFIGS
    dev = device()
    m = swa()
    cfg = PREFILL_CONFIGS["swa_32k"]
    q, k, _, _ = prefill_inputs(cfg, device=dev)
    rot, base = m.rope_dims(cfg.D), 640000.0
    for name, x, off in (("q", q, 229376), ("k", k, 0)):
        x0 = x.cpu()
        m.swa_rope_apply(x, rot, base, None, off)
        torch.cuda.synchronize()
        pos = off + np.arange(cfg.S)[None, :]
        ref = oracle.rope(x0[..., :rot].contiguous(), pos, rot, base)
        got = x.cpu()
        _check_rope(got[..., :rot].contiguous(), x0[..., :rot].contiguous(), ref, rot, "bf16", f"full {name}")
        assert torch.equal(got[..., rot:].view(torch.int16), x0[..., rot:].view(torch.int16))


def test_full_size_prefill_rope_32k():
    """The fused SWA prefill at 32K (queries rotated as staged, keys rotated
    once) on sampled rows against the oracle."""
    from swa_inputs import PREFILL_CONFIGS, sample_rows
    dev = device()
    m = swa()
    cfg = PREFILL_CONFIGS["swa_32k"]
    q, k, v, sinks = prefill_inputs(cfg, device=dev)
    rot, base = m.rope_dims(cfg.D), 10000.0
    k_rot = k.clone()
    m.swa_rope_apply(k_rot, rot, base)
    o = m.swa_attn_prefill_rope(q, k_rot, v, sinks, cfg.window, rot, base, 0, cfg.scale)
    torch.cuda.synchronize()
    S = cfg.S
    rows = sample_rows(S, 512, cfg.seed + 1, (0, 1, 31, 32, 127, 128, 129, S - 1))
    rows_d = rows.to(dev)
    got = o[0].index_select(0, rows_d).cpu()
    q_rows = oracle.rope(q[0].index_select(0, rows_d).cpu()[None], rows.numpy()[None, :], rot, base)[0]
    lo = max(0, int(rows.min()) - cfg.window + 1)
    hi = int(rows.max()) + 1
    kk = oracle.rope(k[0, lo:hi].cpu()[None], np.arange(lo, hi)[None, :], rot, base)[0]
    ref = oracle.prefill_rows(q_rows, rows, kk, v[0, lo:hi].cpu(), sinks.cpu(), cfg.window, 0, cfg.scale,
                              k_base=lo)
    assert_close(got, ref, BF16_TOL, "full prefill_rope")
