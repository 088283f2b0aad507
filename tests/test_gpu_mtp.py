"""GPU parity of the MTP step after a verify pass: greedy draft acceptance
(bit-exact against the oracle), the committed-length advance, and a
multi-step self-speculative loop (verify on a sliding-window ring layer and a
global linear layer, accept, append, advance) checked against the oracle at
every step."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, assert_close, device, swa
from swa_inputs import (ACCEPT_CONFIGS, AcceptConfig, VerifyConfig, accept_inputs, derive_seed,
                        normal, tied_logits, torch_dtype, verify_inputs)

pytestmark = pytest.mark.gpu


def _draft_like(logits: torch.Tensor, seed: int, p: float = 0.8) -> torch.Tensor:
    """Drafts that agree with the first maximal index (numpy's argmax) with
    probability p per position, else a random token."""
    B, T, V = logits.shape
    first = np.argmax(logits.float().numpy(), axis=-1)[:, :T - 1]
    rng = np.random.default_rng(seed)
    rand = rng.integers(0, V, size=(B, T - 1))
    return torch.from_numpy(np.where(rng.random((B, T - 1)) < p, first, rand).astype(np.int32))


def _accept_case(B, T, V, kind, dtype, seed):
    if kind == "planted":
        cfg = AcceptConfig("case", B, T, V, 0.83, dtype, seed)
        return accept_inputs(cfg)
    lg = tied_logits(B, T, V, seed, dtype=torch_dtype(dtype))
    return lg, _draft_like(lg, seed)


ACCEPT_CASES = [
    # name, B, T, vocab, logits kind, dtype, element offset of the logits pointer
    ("b64_full_vocab_bf16", 64, 4, 152064, "planted", "bf16", 0),
    ("b64_full_vocab_f32", 64, 4, 152064, "planted", "f32", 0),
    ("ties_full_vocab_bf16", 8, 4, 152064, "tied", "bf16", 0),
    ("ties_small_vocab_f32", 16, 4, 1000, "tied", "f32", 0),
    ("q_len1", 5, 1, 777, "tied", "bf16", 0),
    ("ragged_vocab_bf16", 7, 3, 4099, "planted", "bf16", 0),
    ("ragged_vocab_ties_f32", 7, 3, 4099, "tied", "f32", 0),
    ("vocab3", 9, 4, 3, "tied", "f32", 0),
    ("one_request_q16", 1, 16, 152064, "tied", "bf16", 0),
    ("many_rows", 4096, 4, 64, "tied", "bf16", 0),
    ("unaligned_pointer_bf16", 8, 4, 8192, "planted", "bf16", 1),
    ("unaligned_pointer_f32", 8, 4, 8192, "tied", "f32", 3),
]


@pytest.mark.parametrize("case", ACCEPT_CASES, ids=[c[0] for c in ACCEPT_CASES])
def test_accept_matches_oracle(case):
    name, B, T, V, kind, dtype, offset = case
    dev = device()
    m = swa()
    logits, draft = _accept_case(B, T, V, kind, dtype, derive_seed("accept", name) % 100000)
    n = logits.numel()
    buf = torch.empty(n + 8, dtype=logits.dtype, device=dev)
    lg_dev = buf[offset:offset + n].view(B, T, V)
    lg_dev.copy_(logits.to(dev))
    target, n_append = m.swa_mtp_greedy_accept(lg_dev, draft.to(dev) if T > 1 else None)
    torch.cuda.synchronize()
    ref_t, ref_n = oracle.greedy_accept(logits, draft if T > 1 else np.zeros((B, 0), np.int32))
    assert np.array_equal(target.cpu().numpy(), ref_t), name
    assert np.array_equal(n_append.cpu().numpy(), ref_n), name


def test_accept_planted_acceptance_law():
    """The benchmark's inputs: every acceptance length occurs and the mean is
    near 1 + p + p^2 + p^3 (= 3.09 for p = 0.83)."""
    dev = device()
    m = swa()
    cfg = ACCEPT_CONFIGS["accept_b64"]
    counts = []
    for step in range(4):
        lg, dr = accept_inputs(cfg, step=step)
        _, na = m.swa_mtp_greedy_accept(lg.to(dev), dr.to(dev))
        counts += na.cpu().tolist()
    assert set(counts) == {1, 2, 3, 4}
    assert abs(np.mean(counts) - 3.09) < 0.25


def test_accept_nan_never_selected():
    """NaN entries are skipped; a row of only NaN gives index 0 (no oracle:
    the oracle's contract excludes NaN logits)."""
    dev = device()
    m = swa()
    B, T, V = 3, 2, 5000
    lg = tied_logits(B, T, V, 77, dtype=torch.float32)
    lg[0, 0, 0] = float("nan")
    lg[0, 0, 4321] = 9.0
    lg[0, 1, ::2] = float("nan")
    lg[1, :, :] = float("nan")
    lg[2, 1, 1234] = float("nan")
    dr = torch.zeros((B, T - 1), dtype=torch.int32)
    target, n_append = m.swa_mtp_greedy_accept(lg.to(dev), dr.to(dev))
    torch.cuda.synchronize()
    t = target.cpu().numpy()
    x = lg.numpy()
    assert t[0, 0] == 4321
    assert t[0, 1] == np.nanargmax(x[0, 1])
    assert t[1].tolist() == [0, 0]
    assert t[2].tolist() == [np.argmax(x[2, 0]), np.nanargmax(x[2, 1])]
    assert n_append.cpu().tolist()[1] == 2   # index 0 equals the zero draft


def test_cache_advance():
    dev = device()
    m = swa()
    g = torch.Generator()
    g.manual_seed(5)
    for B in (1, 64, 300):
        cl = torch.randint(0, 1 << 20, (B,), generator=g, dtype=torch.int32)
        na = torch.randint(1, 5, (B,), generator=g, dtype=torch.int32)
        cl_dev = cl.to(dev)
        m.swa_cache_advance(cl_dev, na.to(dev))
        torch.cuda.synchronize()
        assert torch.equal(cl_dev.cpu(), cl + na)


def _vcfg(name, B, T, W, ring, slots):
    return VerifyConfig(name, B, T, 64, 8, 128, W, ring, slots, 0, 0, "bf16",
                        seed=derive_seed(name) % 100000)


class _OracleLayer:
    """The oracle's copy of one layer: the cache in the GPU layout (int16
    bits of bf16) and the logical history the oracle's verify reads."""

    def __init__(self, inp, ring, cap):
        self.ring = ring
        self.cache_k = inp["k_cache"].view(torch.int16).numpy().copy()
        self.cache_v = inp["v_cache"].view(torch.int16).numpy().copy()
        B, H, Hkv, D = inp["k_hist"].shape
        self.base = inp["hist_base"].clone()
        self.hist_k = torch.full((B, cap, Hkv, D), float("nan"), dtype=torch.bfloat16)
        self.hist_v = torch.full((B, cap, Hkv, D), float("nan"), dtype=torch.bfloat16)
        self.hist_k[:, :H] = inp["k_hist"]
        self.hist_v[:, :H] = inp["v_hist"]

    def verify(self, q, k_new, v_new, sinks, cache_len, window):
        return oracle.verify(q, k_new, v_new, self.hist_k, self.hist_v, self.base, cache_len, sinks,
                             window, 1.0 / np.sqrt(q.shape[-1]))

    def append(self, k_new, v_new, cache_len, n_append):
        kn = k_new.view(torch.int16).numpy()
        vn = v_new.view(torch.int16).numpy()
        oracle.ring_append(self.cache_k, self.cache_v, kn, vn, cache_len, n_append, self.ring)
        hk = self.hist_k.view(torch.int16).numpy()
        hv = self.hist_v.view(torch.int16).numpy()
        oracle.ring_append(hk, hv, kn, vn, cache_len - self.base, n_append, False)


def test_mtp_steps_match_oracle():
    """Six self-speculative steps over an SWA ring layer (W = 128, 128 slots)
    and a global linear layer sharing the committed lengths: each step's
    attention, acceptance, caches and lengths match the oracle's."""
    dev = device()
    m = swa()
    B, T, steps = 8, 4, 6
    lens0 = [0, 1, 126, 127, 128, 129, 700, 1500]
    lin_slots = max(lens0) + T * steps + 8
    layers = {"swa": _vcfg("mtp_swa", B, T, 128, True, 128),
              "ga": _vcfg("mtp_ga", B, T, 0, False, lin_slots)}
    acc_cfg = AcceptConfig("mtp_accept", B, T, 32000, 0.83, "bf16", seed=21)
    gpu, ref = {}, {}
    for name, cfg in layers.items():
        inp = verify_inputs(cfg, cache_len=lens0)
        cap = (cfg.slots if cfg.ring else lin_slots) + T * steps
        ref[name] = _OracleLayer(inp, cfg.ring, cap)
        gpu[name] = dict(k=inp["k_cache"].to(dev), v=inp["v_cache"].to(dev), sinks=inp["sinks"])
    cache_len = torch.tensor(lens0, dtype=torch.int64)
    cache_len_dev = cache_len.to(torch.int32).to(dev)
    seen = set()
    for step in range(steps):
        for name, cfg in layers.items():
            sh_q, sh_kv = (B, T, cfg.Hq, cfg.D), (B, T, cfg.Hkv, cfg.D)
            q = normal(sh_q, derive_seed("mtp", step, name, "q"), dtype=torch.bfloat16)
            kn = normal(sh_kv, derive_seed("mtp", step, name, "k"), dtype=torch.bfloat16)
            vn = normal(sh_kv, derive_seed("mtp", step, name, "v"), dtype=torch.bfloat16)
            g = gpu[name]
            g["k_new"], g["v_new"] = kn, vn
            o = m.swa_attn_verify(q.to(dev), kn.to(dev), vn.to(dev), g["k"], g["v"], cache_len_dev,
                                  g["sinks"].to(dev), cfg.window, cfg.ring, cfg.scale)
            torch.cuda.synchronize()
            o_ref = ref[name].verify(q, kn, vn, g["sinks"], cache_len, cfg.window)
            assert_close(o, o_ref, BF16_TOL, f"step {step} {name}")
        logits, draft = accept_inputs(acc_cfg, step=step)
        target, n_append = m.swa_mtp_greedy_accept(logits.to(dev), draft.to(dev))
        t_ref, n_ref = oracle.greedy_accept(logits, draft)
        torch.cuda.synchronize()
        assert np.array_equal(target.cpu().numpy(), t_ref), f"step {step}"
        assert np.array_equal(n_append.cpu().numpy(), n_ref), f"step {step}"
        seen.update(n_ref.tolist())
        for name, cfg in layers.items():
            g = gpu[name]
            m.kv_ring_append(g["k"], g["v"], g["k_new"].to(dev), g["v_new"].to(dev), cache_len_dev,
                             n_append, cfg.ring)
            ref[name].append(g["k_new"], g["v_new"], cache_len, n_ref.astype(np.int64))
        m.swa_cache_advance(cache_len_dev, n_append)
        cache_len = cache_len + torch.from_numpy(n_ref.astype(np.int64))
        torch.cuda.synchronize()
        assert torch.equal(cache_len_dev.cpu().to(torch.int64), cache_len), f"step {step}"
        for name in layers:
            assert np.array_equal(gpu[name]["k"].cpu().view(torch.int16).numpy(), ref[name].cache_k)
            assert np.array_equal(gpu[name]["v"].cpu().view(torch.int16).numpy(), ref[name].cache_v)
    assert len(seen) >= 3   # the steps exercise several acceptance lengths
