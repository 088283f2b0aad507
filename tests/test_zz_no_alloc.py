"""GPU check of swa_attn_verify_noalloc (split partials in the library's
fixed per-GPU scratch) against swa_attn_verify (caller workspace): two calls
in a row, the second on a smaller input, each bit-identical to the existing
entry point and within tolerance of the oracle."""
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, assert_close, device, swa
from swa_inputs import VerifyConfig, derive_seed, verify_inputs

pytestmark = pytest.mark.gpu


def _case(name, B, slots, lens):
    cfg = VerifyConfig(name, B, 4, 64, 8, 128, 0, False, slots, 0, 0, "bf16", seed=derive_seed(name) % 100000)
    return cfg, lens


CASES = [
    # 16 requests over 20000-slot global caches: two 16384-row splits for the
    # long ones (partials + combine), 1.4 MB of scratch
    _case("noalloc_first", 16, 20000, [20000, 19999, 16385, 16384, 16383, 5000, 1, 0,
                                       12000, 17000, 333, 18000, 4096, 129, 20000, 7]),
    # then fewer requests and shorter caches: the scratch still holds the
    # first call's partials, which must not leak into this one
    _case("noalloc_second", 5, 17000, [17000, 16390, 3, 900, 16999]),
]


def _run_both(m, dev, cfg, lens):
    inp = verify_inputs(cfg, device=dev, cache_len=lens)
    assert m.swa_attn_verify_workspace_bytes(cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D, cfg.slots, False, 0) > 0
    cl = inp["cache_len"].to(torch.int32).to(dev)
    args = (inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], cl, inp["sinks"])
    ref_out = torch.full_like(inp["q"], float("nan"))
    m.swa_attn_verify(*args, cfg.window, cfg.ring, cfg.scale, out=ref_out)
    out = torch.full_like(inp["q"], float("nan"))
    m.swa_attn_verify_noalloc(*args, cfg.window, cfg.ring, cfg.scale, out=out)
    torch.cuda.synchronize()
    return inp, ref_out, out


def test_verify_noalloc_matches_verify_twice():
    dev = device()
    m = swa()
    for cfg, lens in CASES:
        print(f"[noalloc] {cfg.name}: B={cfg.B} slots={cfg.slots}", flush=True)
        inp, ref_out, out = _run_both(m, dev, cfg, lens)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"{cfg.name}: differs from swa_attn_verify"
        L = inp["cache_len"]
        hmax = int(L.max())
        ref = oracle.verify(inp["q"].cpu(), inp["k_new"].cpu(), inp["v_new"].cpu(), inp["k_hist"][:, :hmax].cpu(),
                            inp["v_hist"][:, :hmax].cpu(), inp["hist_base"], L, inp["sinks"].cpu(), cfg.window,
                            cfg.scale)
        assert_close(out, ref, BF16_TOL, cfg.name)


def test_verify_noalloc_ring_without_scratch():
    """A ring verify needs no partials: the entry point runs the direct kernel."""
    dev = device()
    m = swa()
    cfg = VerifyConfig("noalloc_ring", 6, 4, 64, 8, 128, 128, True, 128, 0, 0, "bf16", seed=71)
    inp = verify_inputs(cfg, device=dev, cache_len=[0, 1, 127, 128, 129, 5000])
    cl = inp["cache_len"].to(torch.int32).to(dev)
    args = (inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], cl, inp["sinks"])
    a = m.swa_attn_verify(*args, cfg.window, cfg.ring, cfg.scale)
    b = m.swa_attn_verify_noalloc(*args, cfg.window, cfg.ring, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
