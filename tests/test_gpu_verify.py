"""GPU parity of swa_attn_verify and kv_ring_append against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, F32_TOL, assert_close, device, rel_l2, swa
from swa_inputs import VERIFY_CONFIGS, VerifyConfig, derive_seed, verify_inputs

pytestmark = pytest.mark.gpu


def _vcfg(name, B, T, Hq, Hkv, D, W, ring, slots, lo, hi, dtype="bf16"):
    return VerifyConfig(name, B, T, Hq, Hkv, D, W, ring, slots, lo, hi, dtype,
                        seed=derive_seed(name) % 100000)


def _run(cfg, cache_len=None, sinks_mode="normal"):
    dev = device()
    m = swa()
    inp = verify_inputs(cfg, cache_len=cache_len)
    sinks = inp["sinks"] if sinks_mode == "normal" else None
    o = m.swa_attn_verify(inp["q"].to(dev), inp["k_new"].to(dev), inp["v_new"].to(dev),
                          inp["k_cache"].to(dev), inp["v_cache"].to(dev),
                          inp["cache_len"].to(torch.int32).to(dev),
                          None if sinks is None else sinks.to(dev), cfg.window, cfg.ring,
                          cfg.scale)
    torch.cuda.synchronize()
    ref = oracle.verify(inp["q"], inp["k_new"], inp["v_new"], inp["k_hist"], inp["v_hist"],
                        inp["hist_base"], inp["cache_len"], sinks, cfg.window, cfg.scale)
    return o, ref, inp


EDGE_LENS = [0, 1, 2, 31, 32, 33, 127, 128, 129, 1000]

CASES = [
    # ring-buffer sliding-window caches
    (_vcfg("ring_w128_t4", 10, 4, 64, 8, 128, 128, True, 128, 0, 0), EDGE_LENS),
    (_vcfg("ring_w128_t1", 10, 1, 64, 8, 128, 128, True, 128, 0, 0), EDGE_LENS),
    (_vcfg("ring_w128_t3", 10, 3, 16, 2, 128, 128, True, 128, 0, 0), EDGE_LENS),
    (_vcfg("ring_slots160", 10, 4, 64, 8, 128, 128, True, 160, 0, 0), EDGE_LENS),
    (_vcfg("ring_w64", 10, 4, 64, 8, 128, 64, True, 128, 0, 0), EDGE_LENS),
    (_vcfg("ring_w2", 10, 4, 64, 8, 128, 2, True, 2, 0, 0), EDGE_LENS),
    (_vcfg("ring_d64", 10, 4, 16, 2, 64, 128, True, 128, 0, 0), EDGE_LENS),
    (_vcfg("ring_t8_g8", 10, 8, 64, 8, 128, 128, True, 128, 0, 0), EDGE_LENS),
    # q_len 16: at D = 128 the tile of new rows is then an ordinary last tile
    # (more new rows than the wave that computes it first can hold), at
    # D = 64 it is still computed first
    (_vcfg("ring_t16_g4", 10, 16, 16, 4, 128, 128, True, 128, 0, 0), EDGE_LENS),
    (_vcfg("ring_t16_g4_d64", 10, 16, 16, 4, 64, 128, True, 128, 0, 0), EDGE_LENS),
    # the wider window the pages compare W = 128 against, on a 512-slot ring
    (_vcfg("ring_w512", 10, 4, 64, 8, 128, 512, True, 512, 0, 0),
     [0, 1, 127, 128, 129, 511, 512, 513, 1000, 5000]),
    # linear global caches (several splits + combine)
    (_vcfg("linear_global_t4", 10, 4, 64, 8, 128, 0, False, 1100, 0, 0), EDGE_LENS),
    (_vcfg("linear_global_t1", 10, 1, 16, 2, 128, 0, False, 1100, 0, 0), EDGE_LENS),
    (_vcfg("linear_global_t8", 10, 8, 64, 8, 128, 0, False, 1100, 0, 0), EDGE_LENS),
    (_vcfg("linear_global_d64", 10, 4, 16, 2, 64, 0, False, 1100, 0, 0), EDGE_LENS),
    (_vcfg("linear_global_t16_g2", 10, 16, 8, 4, 128, 0, False, 1100, 0, 0), EDGE_LENS),
    # a sliding window over a linear cache
    (_vcfg("linear_w128", 10, 4, 64, 8, 128, 128, False, 1100, 0, 0), EDGE_LENS),
    (_vcfg("linear_long", 3, 4, 64, 8, 128, 0, False, 20000, 0, 0), [19999, 7777, 12345]),
]


@pytest.mark.parametrize("cfg,lens", CASES, ids=[c[0].name for c in CASES])
def test_verify_bf16(cfg, lens):
    o, ref, _ = _run(cfg, cache_len=lens)
    assert_close(o, ref, BF16_TOL, cfg.name)
    assert rel_l2(o, ref) < 1e-2


@pytest.mark.parametrize("ring", [True, False])
def test_verify_no_sink(ring):
    cfg = _vcfg("nosink", 10, 4, 64, 8, 128, 128 if ring else 0, ring, 128 if ring else 1100, 0, 0)
    o, ref, _ = _run(cfg, cache_len=EDGE_LENS, sinks_mode="none")
    assert_close(o, ref, BF16_TOL, cfg.name)


F32_CASES = [
    (_vcfg("f32_ring", 10, 4, 16, 2, 128, 128, True, 128, 0, 0, "f32"), EDGE_LENS),
    (_vcfg("f32_linear", 10, 4, 16, 2, 64, 0, False, 1100, 0, 0, "f32"), EDGE_LENS),
    (_vcfg("f32_linear_w", 10, 3, 8, 8, 128, 50, False, 1100, 0, 0, "f32"), EDGE_LENS),
]


@pytest.mark.parametrize("cfg,lens", F32_CASES, ids=[c[0].name for c in F32_CASES])
def test_verify_f32(cfg, lens):
    o, ref, _ = _run(cfg, cache_len=lens)
    assert_close(o, ref, F32_TOL, cfg.name)


def test_verify_deterministic():
    dev = device()
    m = swa()
    cfg = _vcfg("det", 4, 4, 64, 8, 128, 0, False, 9000, 0, 0)
    inp = verify_inputs(cfg, cache_len=[8999, 4000, 17, 6000])
    args = [inp[n].to(dev) for n in ("q", "k_new", "v_new", "k_cache", "v_cache")]
    cl = inp["cache_len"].to(torch.int32).to(dev)
    o1 = m.swa_attn_verify(*args, cl, inp["sinks"].to(dev), 0, False)
    o2 = m.swa_attn_verify(*args, cl, inp["sinks"].to(dev), 0, False)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("ring,dtype", [(True, "bf16"), (False, "bf16"), (True, "f32"), (False, "f32")])
def test_append_matches_oracle(ring, dtype):
    dev = device()
    m = swa()
    slots = 128 if ring else 1200
    cfg = _vcfg("append", 8, 4, 64, 8, 128, 128 if ring else 0, ring, slots, 0, 0, dtype)
    lens = [0, 1, 126, 127, 128, 129, 1000, 1196] if ring else [0, 1, 126, 127, 128, 129, 1000, 1196]
    inp = verify_inputs(cfg, cache_len=lens)
    n_app = torch.tensor([4, 0, 3, 1, 2, 4, 3, 4], dtype=torch.int32)
    kc, vc = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    m.kv_ring_append(kc, vc, inp["k_new"].to(dev), inp["v_new"].to(dev),
                     inp["cache_len"].to(torch.int32).to(dev), n_app.to(dev), ring)
    torch.cuda.synchronize()
    iv = torch.int16 if dtype == "bf16" else torch.int32
    k_ref = inp["k_cache"].view(iv).numpy().copy()
    v_ref = inp["v_cache"].view(iv).numpy().copy()
    oracle.ring_append(k_ref, v_ref, inp["k_new"].view(iv).numpy(), inp["v_new"].view(iv).numpy(),
                       inp["cache_len"], n_app, ring)
    assert np.array_equal(kc.cpu().view(iv).numpy(), k_ref)
    assert np.array_equal(vc.cpu().view(iv).numpy(), v_ref)


@pytest.mark.parametrize("ring", [True, False])
def test_verify_equals_successive_decodes(ring):
    """A q_len=4 verify equals four q_len=1 decodes with an append after each
    (both on the GPU, both checked against the oracle's verify)."""
    dev = device()
    m = swa()
    W = 128 if ring else 0
    slots = 128 if ring else 1200
    cfg = _vcfg("succ", 6, 4, 64, 8, 128, W, ring, slots, 0, 0)
    lens = [0, 1, 127, 128, 129, 1100]
    inp = verify_inputs(cfg, cache_len=lens)
    ref = oracle.verify(inp["q"], inp["k_new"], inp["v_new"], inp["k_hist"], inp["v_hist"],
                        inp["hist_base"], inp["cache_len"], inp["sinks"], W, cfg.scale)
    q, kn, vn = inp["q"].to(dev), inp["k_new"].to(dev), inp["v_new"].to(dev)
    kc, vc = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    sinks = inp["sinks"].to(dev)
    cl = inp["cache_len"].to(torch.int32).to(dev)
    full = m.swa_attn_verify(q, kn, vn, kc, vc, cl, sinks, W, ring)
    one = torch.ones(cfg.B, dtype=torch.int32, device=dev)
    outs = []
    for t in range(4):
        kt, vt = kn[:, t:t + 1].contiguous(), vn[:, t:t + 1].contiguous()
        outs.append(m.swa_attn_verify(q[:, t:t + 1].contiguous(), kt, vt, kc, vc, cl, sinks, W, ring))
        m.kv_ring_append(kc, vc, kt, vt, cl, one, ring)
        cl = cl + 1
    torch.cuda.synchronize()
    step = torch.cat(outs, dim=1)
    assert_close(full, ref, BF16_TOL, "q_len=4 verify")
    assert_close(step, ref, BF16_TOL, "successive decodes")
    assert (full.float() - step.float()).abs().max().item() < 2e-2


def test_ring_equals_linear():
    """The same requests on a ring cache and on a linear cache give the same
    output for a window that fits the ring."""
    dev = device()
    m = swa()
    lens = [0, 5, 127, 128, 129, 700]
    lin = _vcfg("rl", 6, 4, 64, 8, 128, 128, False, 800, 0, 0)
    inp = verify_inputs(lin, cache_len=lens)
    from swa_inputs import ring_from_history
    ring_k = ring_from_history(inp["k_hist"], inp["hist_base"], inp["cache_len"], 128)
    ring_v = ring_from_history(inp["v_hist"], inp["hist_base"], inp["cache_len"], 128)
    args = [inp[n].to(dev) for n in ("q", "k_new", "v_new")]
    cl = inp["cache_len"].to(torch.int32).to(dev)
    s = inp["sinks"].to(dev)
    o_lin = m.swa_attn_verify(*args, inp["k_cache"].to(dev), inp["v_cache"].to(dev), cl, s, 128, False)
    o_ring = m.swa_attn_verify(*args, ring_k.to(dev), ring_v.to(dev), cl, s, 128, True)
    torch.cuda.synchronize()
    assert (o_lin.float() - o_ring.float()).abs().max().item() < 2e-2


# ---------------------------------------------------------------- full sizes

def _full_verify(cfg: VerifyConfig, check_b):
    dev = device()
    m = swa()
    print(f"[full-size] {cfg.name}: generating inputs on {dev}", flush=True)
    inp = verify_inputs(cfg, device=dev)
    cl = inp["cache_len"].to(torch.int32).to(dev)
    o = m.swa_attn_verify(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], cl,
                          inp["sinks"], cfg.window, cfg.ring, cfg.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    L = inp["cache_len"]
    print(f"[full-size] {cfg.name}: oracle on {len(check_b)} requests", flush=True)
    for b in check_b:
        Lb = int(L[b])
        base = int(inp["hist_base"][b])
        n = Lb - base
        ref = oracle.verify(inp["q"][b:b + 1].cpu(), inp["k_new"][b:b + 1].cpu(),
                            inp["v_new"][b:b + 1].cpu(), inp["k_hist"][b:b + 1, :n].cpu(),
                            inp["v_hist"][b:b + 1, :n].cpu(), inp["hist_base"][b:b + 1],
                            L[b:b + 1], inp["sinks"].cpu(), cfg.window, cfg.scale)
        assert_close(o[b:b + 1], ref, BF16_TOL, f"{cfg.name} request {b} (L={Lb})")
        assert rel_l2(o[b:b + 1], ref) < 1e-2, f"{cfg.name} request {b}: relative L2"


def test_full_size_verify_ga_b64():
    """Every request of the 64-request q_len = 4 verify on the global cache."""
    cfg = VERIFY_CONFIGS["verify_ga_b64"]
    _full_verify(cfg, range(cfg.B))


def test_full_size_verify_swa_b64():
    cfg = VERIFY_CONFIGS["verify_swa_b64"]
    _full_verify(cfg, range(cfg.B))


def test_full_size_decode_ga_b64():
    """Every request of the q_len = 1 decode over the 64-request global cache
    (the verify entry point)."""
    cfg = VERIFY_CONFIGS["decode_ga_b64"]
    _full_verify(cfg, range(cfg.B))


def test_full_size_decode_swa_b64():
    cfg = VERIFY_CONFIGS["decode_swa_b64"]
    _full_verify(cfg, range(cfg.B))


def test_full_size_verify_ga_256k():
    cfg = VERIFY_CONFIGS["verify_ga_256k"]
    _full_verify(cfg, [0])


def test_verify_many_requests_split():
    """More requests than the longest-first split order serves (B > 256):
    the split workgroups then take the plain grid order.  A few requests are
    long enough for two 16384-row splits plus the combine; the rest are short
    or empty.  Every request is checked."""
    cfg = _vcfg("many_requests", 300, 4, 16, 2, 64, 0, False, 16500, 0, 0)
    g = torch.Generator()
    g.manual_seed(derive_seed("many_requests", "lens"))
    lens = torch.randint(0, 700, (cfg.B,), generator=g)
    lens[torch.tensor([0, 7, 150, 299])] = torch.tensor([16500, 16385, 16384, 16499])
    lens[torch.tensor([1, 2])] = 0
    dev = device()
    m = swa()
    assert m.swa_attn_verify_workspace_bytes(cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D, cfg.slots, False, 0) > 0
    inp = verify_inputs(cfg, device=dev, cache_len=lens)
    cl = inp["cache_len"].to(torch.int32).to(dev)
    o = m.swa_attn_verify(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], cl,
                          inp["sinks"], cfg.window, cfg.ring, cfg.scale)
    torch.cuda.synchronize()
    L = inp["cache_len"]
    # the short requests in one oracle call over their 700-row histories, the
    # long ones one at a time
    short = torch.nonzero(L < 700).flatten()
    groups = [(short, 700)] + [(torch.tensor([b]), int(L[b])) for b in torch.nonzero(L >= 700).flatten()]
    for idx, hlen in groups:
        idx_d = idx.to(dev)
        sel = lambda t: t.index_select(0, idx_d).cpu()
        ref = oracle.verify(sel(inp["q"]), sel(inp["k_new"]), sel(inp["v_new"]), sel(inp["k_hist"][:, :hlen]),
                            sel(inp["v_hist"][:, :hlen]), inp["hist_base"][idx], L[idx], inp["sinks"].cpu(),
                            cfg.window, cfg.scale)
        got = o.index_select(0, idx_d)
        assert_close(got, ref, BF16_TOL, f"{cfg.name} requests {idx.tolist()[:4]}...")
        assert rel_l2(got, ref) < 1e-2
