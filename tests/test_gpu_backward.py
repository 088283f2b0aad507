"""GPU parity of the training forward (saved log-sum-exp) and the backward
(dq, dk, dv, dsink) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import BF16_TOL, assert_close, device, rel_l2, swa
from swa_inputs import PrefillConfig, derive_seed, normal, prefill_inputs

pytestmark = pytest.mark.gpu

# Gradient tolerance.  The kernels see bf16 inputs exactly (the oracle gets
# the same values), accumulate in fp32, and round P and dS to bf16 (relative
# 2^-9) before the matrix cores, as the forward rounds P; dq/dk/dv are
# rounded to bf16 (2^-9).  The largest elementwise errors come from the row
# term D_i = <dO_i, O_i>, formed (as in any backward that keeps only the
# forward's output) from the bf16-rounded O: its error, up to 2^-9 of
# sum_d |dO_id O_id|, enters dS_ij = P_ij (dP_ij - D_i) unreduced where dP_ij
# and D_i nearly cancel (a query whose weight sits on few keys, e.g. W = 1).
# Each element is judged against the gradient's scale:
# |gpu - ref| <= GRAD_TOL * (|ref| + rms(ref)), plus, at W = 1 where the
# cancellation is exact, the derived D-term bound of _d_term_bounds.  Over
# every case below and the full 32K workload the largest err / (|ref| + rms)
# measured on the MI355X outside W = 1 is 3.6e-2 (dq at 32K); GRAD_TOL keeps
# a 1.2x margin above it.
# The relative L2 error per tensor is held to the bf16 rtol of 1e-2
# (measured at most 6.6e-3).
GRAD_TOL = 4.5e-2
GRAD_L2 = 1e-2
# The saved LSE: the forward sums its attention weights after rounding each
# to bf16 (relative error <= 2^-9, the same rounding that enters P V), and
# the sum instruction may add one more rounding at that level, so
# |lse - lse_ref| <= 2 * 2^-9 (natural-log units; measured up to 3.4e-3).
LSE_TOL = 2 * 2.0 ** -9

CASES = [
    # name, B, S, Sk, Hq, Hkv, D, window, sinks
    ("swa_g8", 1, 300, 300, 16, 2, 128, 128, True),
    ("global_g8", 1, 200, 200, 16, 2, 128, 0, True),
    ("swa_g4_d64", 2, 150, 150, 16, 4, 64, 64, True),
    ("chunk_offset", 1, 130, 300, 16, 2, 128, 128, True),
    ("no_sink", 1, 190, 190, 8, 1, 128, 128, False),
    ("g1_w1", 1, 70, 70, 4, 4, 64, 1, True),
    ("model_heads", 1, 256, 256, 64, 8, 128, 128, True),
    ("global_chunk_g2", 2, 77, 120, 8, 4, 128, 0, True),
    # the LSE-saving global kernel at D 64
    ("global_d64_g4", 1, 150, 150, 8, 2, 64, 0, True),
    # the other instantiations of the strip dQ kernel (G 4 with D 128, G 8
    # with D 64) and a window that is not a multiple of the tile
    ("swa_g4_d128", 1, 200, 200, 16, 4, 128, 128, True),
    ("swa_g8_d64_w96", 1, 160, 160, 16, 2, 64, 96, True),
    # the fused sliding-window kernel (D 128, G 4 or 8, q_offset a multiple
    # of 32 / G) over several strips per (b, g): key tiles two strips share
    # (partials added by the fix-up kernel), ragged last blocks, an offset
    # chunk, two requests, W = 1 and a window that is not a multiple of 32
    ("strips_g8", 1, 1100, 1100, 16, 2, 128, 128, True),
    ("strips_many_g8", 1, 2600, 2600, 8, 1, 128, 128, True),
    ("strips_g4_w100", 1, 1500, 1500, 16, 4, 128, 100, True),
    ("strips_chunk_g8", 1, 1202, 1402, 16, 2, 128, 128, True),
    ("strips_b2_nosink", 2, 1100, 1100, 8, 1, 128, 128, False),
    ("strips_w1_g8", 1, 1030, 1030, 8, 1, 128, 1, True),
    # the fused kernel on a single (ragged) query block, with and without an
    # offset: one strip of one block, fewer than five live key tiles
    ("tiny_g8", 1, 3, 3, 16, 2, 128, 128, True),
    ("tiny_g4_offset", 1, 5, 21, 8, 2, 128, 64, True),
]


def _check_grad(got, ref, name, extra=None):
    """|got - ref| <= GRAD_TOL * (|ref| + rms(ref)) + extra elementwise, and
    the relative L2 error below GRAD_L2 (extra: a derived error term, see
    _d_term_bounds)."""
    g = got.detach().float().cpu().numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(g).all(), f"{name}: non-finite"
    rms = float(np.sqrt((r ** 2).mean())) if r.size else 0.0
    err = np.abs(g - r)
    bound = GRAD_TOL * (np.abs(r) + rms)
    if extra is not None:
        bound = bound + extra
    worst = float((err - bound).max()) if r.size else 0.0
    l2 = rel_l2(got, r) if rms > 0 else 0.0
    need = float((err / (np.abs(r) + rms)).max()) if rms > 0 else 0.0
    print(f"{name}: max abs err {err.max():.3e} rms(ref) {rms:.3e} rel L2 {l2:.3e} "
          f"max err/(|ref|+rms) {need:.3e}" + ("" if extra is None else " (+ D term)"), flush=True)
    assert worst <= 0, f"{name}: max excess {worst:.3e}"
    assert l2 < GRAD_L2, f"{name}: relative L2 {l2:.3e}"


def _d_term_bounds(q, k, v, dout, sinks, cfg):
    """Error terms of the gradients that come from the row term D_i = <dO_i, O_i>
    at W = 1, where it cancels against dP_ii.  The kernels form D_i from the
    forward's bf16 output; with one key per row that output is the exact one
    within 2^-8 elementwise (the weight rounded once to bf16 before P V and
    the normaliser built from the same rounded weight, then O rounded to
    bf16), so |D_i - D_i(exact)| <= e_i = 2^-8 sum_d |dO_id O_id|, and through
    dS_ij = P_ij (dP_ij - D_i):
      |err dq_i| <= scale e_i sum_j P_ij |k_j|,
      |err dk_j| <= scale sum_i P_ij e_i |q_i|,  and dv does not use D
    (dsink sums these errors over many rows with random signs and stays within
    GRAD_TOL without a term of its own).  Returns the (dq, dk) terms from the
    oracle's weights, or Nones."""
    if cfg.window != 1:
        return None, None
    ref = oracle.prefill(q, k, v, sinks, cfg.window, cfg.q_offset, cfg.scale, want_lse=True, want_weights=True)
    P = np.asarray(ref["weights"], dtype=np.float64)              # [B, Sq, Hq, Sk]
    e = 2.0 ** -8 * np.abs(dout.double().numpy() * ref["o"]).sum(-1)  # [B, Sq, Hq]
    G = cfg.Hq // cfg.Hkv
    ka = np.repeat(np.abs(k.double().numpy()), G, axis=2)         # [B, Sk, Hq, D]
    qa = np.abs(q.double().numpy())
    x_dq = cfg.scale * e[..., None] * np.einsum("bihj,bjhd->bihd", P, ka)
    x_dk = cfg.scale * np.einsum("bihj,bih,bihd->bjhd", P, e, qa)
    x_dk = x_dk.reshape(x_dk.shape[0], x_dk.shape[1], cfg.Hkv, G, -1).sum(3)
    return x_dq, x_dk


def _inputs(case):
    name, B, S, Sk, Hq, Hkv, D, W, with_sink = case
    cfg = PrefillConfig(name, B, S, Hq, Hkv, D, W, "bf16", seed=derive_seed("bwd", name) % 100000, Sk=Sk)
    q, k, v, sinks = prefill_inputs(cfg)
    dout = normal(q.shape, derive_seed("bwd", name, "dout"), dtype=torch.bfloat16)
    return cfg, q, k, v, (sinks if with_sink else None), dout


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_lse_matches_oracle(case):
    dev = device()
    m = swa()
    cfg, q, k, v, sinks, _ = _inputs(case)
    sd = None if sinks is None else sinks.to(dev)
    o, lse = m.swa_attn_prefill_lse(q.to(dev), k.to(dev), v.to(dev), sd, cfg.window, cfg.q_offset, cfg.scale)
    o_plain = m.swa_attn_prefill(q.to(dev), k.to(dev), v.to(dev), sd, cfg.window, cfg.q_offset, cfg.scale)
    torch.cuda.synchronize()
    if cfg.window > 0:
        assert torch.equal(o.view(torch.int16), o_plain.view(torch.int16))
    else:
        # without a window the plain prefill sums the weights before their
        # rounding (at most 2^-9 apart relatively); a sum near the
        # lazy-rescale threshold can also move a rescale, and with it the
        # rounding of later weights, so the two agree to the bf16 tolerance
        assert_close(o, o_plain.float().cpu().numpy().astype(np.float64), BF16_TOL,
                     case[0] + " (training vs plain)")
    ref = oracle.prefill(q, k, v, sinks, cfg.window, cfg.q_offset, cfg.scale, want_lse=True)
    assert_close(o, ref["o"], BF16_TOL, case[0])
    err = np.abs(lse.cpu().numpy() - ref["lse"]).max()
    assert err <= LSE_TOL, f"{case[0]}: lse max abs err {err:.3e}"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    dev = device()
    m = swa()
    cfg, q, k, v, sinks, dout = _inputs(case)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    sd = None if sinks is None else sinks.to(dev)
    o, lse = m.swa_attn_prefill_lse(qd, kd, vd, sd, cfg.window, cfg.q_offset, cfg.scale)
    dq, dk, dv, dsink = m.swa_attn_backward(qd, kd, vd, sd, o, lse, dout.to(dev), cfg.window, cfg.q_offset,
                                            cfg.scale)
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.prefill_backward(q, k, v, dout, sinks, cfg.window, cfg.q_offset, cfg.scale)
    x_dq, x_dk = _d_term_bounds(q, k, v, dout, sinks, cfg)
    _check_grad(dq, rq, case[0] + " dq", x_dq)
    _check_grad(dk, rk, case[0] + " dk", x_dk)
    _check_grad(dv, rv, case[0] + " dv")
    if sinks is not None:
        _check_grad(dsink, rs, case[0] + " dsink")


def test_backward_dsink_deterministic_and_unseen_keys_zero():
    """Two backward calls give bit-identical gradients (fixed summation
    order), and keys that no query can see get exactly zero gradients."""
    dev = device()
    m = swa()
    case = ("unseen", 1, 64, 400, 16, 2, 128, 128, True)   # queries at 336..399
    cfg, q, k, v, sinks, dout = _inputs(case)
    args = [t.to(dev) for t in (q, k, v)]
    o, lse = m.swa_attn_prefill_lse(*args, sinks.to(dev), cfg.window, cfg.q_offset, cfg.scale)
    a = m.swa_attn_backward(*args, sinks.to(dev), o, lse, dout.to(dev), cfg.window, cfg.q_offset, cfg.scale)
    b = m.swa_attn_backward(*args, sinks.to(dev), o, lse, dout.to(dev), cfg.window, cfg.q_offset, cfg.scale)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
    first_seen = cfg.q_offset - cfg.window + 1            # 209
    assert not a[1][:, :first_seen].float().abs().sum().item()
    assert not a[2][:, :first_seen].float().abs().sum().item()
    assert a[1][:, first_seen:].float().abs().sum().item() > 0


def test_full_size_backward_swa_32k():
    """The bench's training workload (SWA 32K, 64 query heads, 8 KV heads,
    D 128, sinks): every element of dq, dk, dv and dsink against the oracle."""
    from swa_inputs import PREFILL_CONFIGS
    dev = device()
    m = swa()
    cfg = PREFILL_CONFIGS["swa_32k"]
    print(f"[full-size] {cfg.name} backward: inputs", flush=True)
    q, k, v, sinks = prefill_inputs(cfg, device=dev)
    dout = normal(q.shape, derive_seed(cfg.seed, "dout"), dev, torch.bfloat16)
    o, lse = m.swa_attn_prefill_lse(q, k, v, sinks, cfg.window, cfg.q_offset, cfg.scale)
    dq, dk, dv, dsink = m.swa_attn_backward(q, k, v, sinks, o, lse, dout, cfg.window, cfg.q_offset, cfg.scale)
    torch.cuda.synchronize()
    print(f"[full-size] {cfg.name} backward: oracle", flush=True)
    rq, rk, rv, rs = oracle.prefill_backward(q, k, v, dout, sinks, cfg.window, cfg.q_offset, cfg.scale)
    _check_grad(dq, rq, "full dq")
    _check_grad(dk, rk, "full dk")
    _check_grad(dv, rv, "full dv")
    _check_grad(dsink, rs, "full dsink")
