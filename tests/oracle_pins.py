"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function raises AssertionError on failure.  They are run
directly by ``test_oracle_pins.py`` and again, against deliberately broken
copies of the oracle, by ``test_oracle_mutants.py`` (which expects every
broken copy to fail at least one pin).

What pins what:
  * torch scaled_dot_product_attention (fp64, CPU) with a band mask and one
    extra key/value column of zeros whose additive bias is the sink logit:
    the whole formula (scores, scale, masking, sink in the denominator, value
    sum, GQA grouping via repeat_interleave).
  * sink = None / -inf against SDPA with the band mask only; W >= S and W <= 0
    against SDPA with is_causal=True.
  * closed forms: W=1 gives sigmoid(s_ii - sink) * V_i; Q=0 with one-hot
    values gives the exact window membership and the 1/(n + e^sink) weights.
  * invariants: weights + sink mass = 1; O_sink = sigmoid(LSE - sink) O_nosink.
  * verify == successive single-token decodes == the last rows of a prefill;
    chunked prefill == unchunked; sampled rows == full prefill.
  * ring append: every slot checked against the stated placement rule.
  * greedy draft acceptance: the release blog's verify diagram (accept,
    accept, reject, discard gives three rows to append), a match after the
    first rejection that must not count, ties resolved to the lowest index,
    T=1 and all-accepted edge cases, and numpy's argmax (first occurrence of
    the maximum) plus a brute-force prefix count on random integer logits.
  * partial rotary embedding: one-hot inputs at known angles (cos / sin of
    pos * base^(-2i/rot) by hand), position 0 as the identity, R(a) R(b) =
    R(a + b), preserved pair norms with untouched tail dimensions, and the
    relative-position property <R(p+c) q, R(p'+c) k> = <R(p) q, R(p') k>.
  * backward: central finite differences of the forward oracle's loss
    sum(dO * O) on inputs on the bf16 grid (so the +-2^-10 steps are exact in
    fp32), torch fp64 autograd through the SDPA-with-sink-column reference,
    and dsink_h = -sum_i p_sink,i <dO_i, O_i> from the forward's sink mass.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from swa_inputs import normal, derive_seed

TOL = 1e-12


def _rand(shape, *key):
    return normal(shape, derive_seed("pins", *key)).double()


def _sdpa_reference(q, k, v, sinks, window, q_offset, scale):
    """torch SDPA (fp64) of q [B,Sq,Hq,D] over k/v [B,Sk,Hkv,D] with a band
    mask built from positions and, if sinks is given, one extra zero key/value
    whose additive bias is the sink logit."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qt = q.double().permute(0, 2, 1, 3)                                   # [B,Hq,Sq,D]
    kt = k.double().repeat_interleave(G, dim=2).permute(0, 2, 1, 3)       # [B,Hq,Sk,D]
    vt = v.double().repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    i = torch.arange(Sq).view(-1, 1) + q_offset
    j = torch.arange(Sk).view(1, -1)
    allowed = j <= i
    if window > 0:
        allowed &= j > i - window
    bias = torch.zeros(Sq, Sk, dtype=torch.float64).masked_fill(~allowed, float("-inf"))
    bias = bias.view(1, 1, Sq, Sk).expand(B, Hq, Sq, Sk)
    if sinks is not None:
        zk = torch.zeros(B, Hq, 1, D, dtype=torch.float64)
        kt = torch.cat([kt, zk], dim=2)
        vt = torch.cat([vt, zk], dim=2)
        sb = sinks.double().view(1, Hq, 1, 1).expand(B, Hq, Sq, 1)
        bias = torch.cat([bias, sb], dim=3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                                         attn_mask=bias, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


PREFILL_CASES = [
    # B, Sq, Sk, Hq, Hkv, D, window, q_offset
    (1, 24, 24, 2, 1, 8, 5, 0),
    (2, 17, 23, 4, 2, 16, 4, 6),
    (1, 33, 33, 3, 3, 8, 1, 0),
    (1, 20, 20, 4, 1, 8, 0, 0),
    (2, 9, 40, 2, 2, 4, 128, 31),
    (1, 40, 40, 8, 2, 16, 7, 0),
]


def pin_sdpa_with_sink_column():
    for n, (B, Sq, Sk, Hq, Hkv, D, W, off) in enumerate(PREFILL_CASES):
        q = _rand((B, Sq, Hq, D), "q", n)
        k = _rand((B, Sk, Hkv, D), "k", n)
        v = _rand((B, Sk, Hkv, D), "v", n)
        sinks = _rand((Hq,), "s", n)
        scale = 1.0 / math.sqrt(D) * (1.0 + 0.25 * n)
        got = oracle.prefill(q, k, v, sinks, W, off, scale)
        ref = _sdpa_reference(q, k, v, sinks, W, off, scale)
        err = np.abs(got - ref).max()
        assert err < TOL, f"case {n}: oracle vs SDPA+sink column max err {err}"


def pin_no_sink_is_band_softmax():
    for n, (B, Sq, Sk, Hq, Hkv, D, W, off) in enumerate(PREFILL_CASES):
        q = _rand((B, Sq, Hq, D), "q", n)
        k = _rand((B, Sk, Hkv, D), "k", n)
        v = _rand((B, Sk, Hkv, D), "v", n)
        ref = _sdpa_reference(q, k, v, None, W, off, 1.0 / math.sqrt(D))
        for sinks in (None, torch.full((Hq,), float("-inf"))):
            got = oracle.prefill(q, k, v, sinks, W, off, 1.0 / math.sqrt(D))
            err = np.abs(got - ref).max()
            assert err < TOL, f"case {n}: no-sink oracle vs band SDPA max err {err}"


def pin_wide_window_is_causal():
    B, S, Hq, Hkv, D = 2, 30, 4, 2, 8
    q, k, v = _rand((B, S, Hq, D), "cq"), _rand((B, S, Hkv, D), "ck"), _rand((B, S, Hkv, D), "cv")
    qt = q.permute(0, 2, 1, 3)
    kt = k.repeat_interleave(2, dim=2).permute(0, 2, 1, 3).contiguous()
    vt = v.repeat_interleave(2, dim=2).permute(0, 2, 1, 3).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ref = ref.permute(0, 2, 1, 3).numpy()
    for W in (0, -1, S, S + 7):
        got = oracle.prefill(q, k, v, None, W, 0)
        err = np.abs(got - ref).max()
        assert err < TOL, f"W={W}: oracle vs causal SDPA max err {err}"


def pin_window_one_closed_form():
    B, S, Hq, Hkv, D = 1, 19, 4, 2, 8
    q, k, v = _rand((B, S, Hq, D), "1q"), _rand((B, S, Hkv, D), "1k"), _rand((B, S, Hkv, D), "1v")
    sinks = _rand((Hq,), "1s")
    scale = 0.3
    got = oracle.prefill(q, k, v, sinks, 1, 0, scale)
    kk = k.repeat_interleave(2, dim=2)
    vv = v.repeat_interleave(2, dim=2)
    s_ii = scale * (q * kk).sum(-1)                                   # [B,S,Hq]
    ref = torch.sigmoid(s_ii - sinks.view(1, 1, -1)).unsqueeze(-1) * vv
    err = np.abs(got - ref.numpy()).max()
    assert err < TOL, f"W=1 closed form max err {err}"


def pin_zero_query_window_membership():
    """Q = 0 makes every score 0, so each key in J(i) gets weight 1/(n + e^sink)
    with n = |J(i)|; one-hot values V[j] = e_{j mod D} reveal exactly which
    positions are in J(i)."""
    for (S, W, off, D) in ((40, 5, 3, 16), (21, 0, 0, 32), (12, 1, 0, 4), (50, 9, 11, 16)):
        Sk = S + off
        Hq = Hkv = 1
        q = torch.zeros(1, S, Hq, D, dtype=torch.float64)
        k = _rand((1, Sk, Hkv, D), "0k", S, W)
        v = torch.zeros(1, Sk, Hkv, D, dtype=torch.float64)
        for j in range(Sk):
            v[0, j, 0, j % D] = 1.0
        sink = 0.7
        got = oracle.prefill(q, k, v, torch.tensor([sink], dtype=torch.float64), W, off, 0.5)
        for r in range(S):
            i = r + off
            members = [j for j in range(Sk) if j <= i and (W <= 0 or j > i - W)]
            expect = np.zeros(D)
            for j in members:
                expect[j % D] += 1.0
            expect /= len(members) + math.exp(sink)
            err = np.abs(got[0, r, 0] - expect).max()
            assert err < TOL, f"S={S} W={W} off={off} row {r}: window membership err {err}"


def pin_weights_and_sink_mass_sum_to_one():
    B, S, Hq, Hkv, D, W = 2, 26, 4, 1, 8, 6
    q, k, v = _rand((B, S, Hq, D), "wq"), _rand((B, S, Hkv, D), "wk"), _rand((B, S, Hkv, D), "wv")
    sinks = _rand((Hq,), "ws") * 2
    out = oracle.prefill(q, k, v, sinks, W, 0, 0.4, want_psink=True, want_weights=True)
    w, ps = out["weights"], out["psink"]
    total = w.sum(-1) + ps
    assert np.abs(total - 1).max() < TOL, "weights + sink mass != 1"
    i = np.arange(S).reshape(-1, 1)
    j = np.arange(S).reshape(1, -1)
    outside = (j > i) | (j <= i - W)
    for r in range(S):
        for c in range(S):
            if outside[r, c]:
                assert np.all(w[:, r, :, c] == 0.0), "weight outside the window"
                continue
            assert np.all(w[:, r, :, c] > 0.0), "zero weight inside the window"
    # O = weights @ V
    vv = v.repeat_interleave(4, dim=2).numpy()
    o_w = np.einsum("bshj,bjhd->bshd", w, vv)
    assert np.abs(o_w - out["o"]).max() < TOL


def pin_lse_sigmoid_identity():
    """With LSE of the keys alone, O_sink = sigmoid(LSE - sink) * O_nosink."""
    B, S, Hq, Hkv, D, W = 1, 31, 2, 1, 16, 10
    q, k, v = _rand((B, S, Hq, D), "lq"), _rand((B, S, Hkv, D), "lk"), _rand((B, S, Hkv, D), "lv")
    sinks = _rand((Hq,), "ls")
    plain = oracle.prefill(q, k, v, None, W, 0, want_lse=True)
    with_sink = oracle.prefill(q, k, v, sinks, W, 0)
    sig = 1.0 / (1.0 + np.exp(-(plain["lse"] - sinks.numpy().reshape(1, 1, -1))))
    err = np.abs(with_sink - sig[..., None] * plain["o"]).max()
    assert err < TOL, f"sigmoid(LSE - sink) identity err {err}"


def pin_gqa_equals_repeated_heads():
    B, S, Hq, Hkv, D, W = 2, 18, 8, 2, 8, 5
    q, k, v = _rand((B, S, Hq, D), "gq"), _rand((B, S, Hkv, D), "gk"), _rand((B, S, Hkv, D), "gv")
    sinks = _rand((Hq,), "gs")
    got = oracle.prefill(q, k, v, sinks, W, 0)
    ref = oracle.prefill(q, k.repeat_interleave(4, dim=2), v.repeat_interleave(4, dim=2), sinks, W, 0)
    assert np.abs(got - ref).max() == 0.0, "GQA grouping differs from repeat_interleave"
    # and the grouping is contiguous: head h uses KV head h // (Hq/Hkv)
    k2 = k.clone()
    k2[:, :, 1] += 1.0  # perturb KV head 1 only: heads 4..7 must change, 0..3 must not
    got2 = oracle.prefill(q, k2, v, sinks, W, 0)
    assert np.abs(got2[:, :, :4] - got[:, :, :4]).max() == 0.0
    assert np.abs(got2[:, :, 4:] - got[:, :, 4:]).min() > 0.0


def _verify_case(n, B=3, T=4, Hq=4, Hkv=2, D=8, W=6, Lmax=20):
    g = torch.Generator().manual_seed(derive_seed("pins-verify", n))
    L = torch.randint(0, Lmax + 1, (B,), generator=g)
    L[0] = Lmax
    q = _rand((B, T, Hq, D), "vq", n)
    kn, vn = _rand((B, T, Hkv, D), "vkn", n), _rand((B, T, Hkv, D), "vvn", n)
    kh, vh = _rand((B, Lmax, Hkv, D), "vkh", n), _rand((B, Lmax, Hkv, D), "vvh", n)
    sinks = _rand((Hq,), "vs", n)
    return L, q, kn, vn, kh, vh, sinks


def pin_verify_equals_prefill_rows():
    for n, W in enumerate((6, 0, 1, 3, 100)):
        L, q, kn, vn, kh, vh, sinks = _verify_case(n, W=W)
        B, T = q.shape[:2]
        got = oracle.verify(q, kn, vn, kh, vh, torch.zeros(B, dtype=torch.long), L, sinks, W)
        for b in range(B):
            Lb = int(L[b])
            kfull = torch.cat([kh[b:b + 1, :Lb], kn[b:b + 1]], dim=1)
            vfull = torch.cat([vh[b:b + 1, :Lb], vn[b:b + 1]], dim=1)
            ref = oracle.prefill(q[b:b + 1], kfull, vfull, sinks, W, Lb)
            err = np.abs(got[b] - ref[0]).max()
            assert err < TOL, f"W={W} b={b}: verify vs prefill rows err {err}"


def pin_verify_equals_successive_decodes():
    for n, W in enumerate((6, 0, 2)):
        L, q, kn, vn, kh, vh, sinks = _verify_case(10 + n, W=W)
        B, T = q.shape[:2]
        zero = torch.zeros(B, dtype=torch.long)
        got = oracle.verify(q, kn, vn, kh, vh, zero, L, sinks, W)
        Hlen = kh.shape[1] + T
        khist = torch.full((B, Hlen) + kh.shape[2:], float("nan"), dtype=torch.float64)
        vhist = khist.clone()
        for b in range(B):
            khist[b, :int(L[b])] = kh[b, :int(L[b])]
            vhist[b, :int(L[b])] = vh[b, :int(L[b])]
        for t in range(T):
            Lt = L + t
            one = oracle.verify(q[:, t:t + 1], kn[:, t:t + 1], vn[:, t:t + 1], khist, vhist,
                                zero, Lt, sinks, W)
            err = np.abs(one[:, 0] - got[:, t]).max()
            assert err < TOL, f"W={W} t={t}: verify vs successive decode err {err}"
            for b in range(B):  # commit token t, then decode the next one
                khist[b, int(Lt[b])] = kn[b, t]
                vhist[b, int(Lt[b])] = vn[b, t]


def pin_chunked_prefill_equals_unchunked():
    B, S, Hq, Hkv, D = 1, 64, 4, 2, 8
    q, k, v = _rand((B, S, Hq, D), "kq"), _rand((B, S, Hkv, D), "kk"), _rand((B, S, Hkv, D), "kv")
    sinks = _rand((Hq,), "ks")
    for W in (7, 0):
        full = oracle.prefill(q, k, v, sinks, W, 0)
        for c0 in range(0, S, 16):
            part = oracle.prefill(q[:, c0:c0 + 16], k[:, :c0 + 16], v[:, :c0 + 16], sinks, W, c0)
            assert np.abs(part - full[:, c0:c0 + 16]).max() < TOL
        rows = torch.tensor([0, 1, 6, 7, 8, 33, 63])
        got = oracle.prefill_rows(q[0, rows], rows, k[0], v[0], sinks, W, 0)
        assert np.abs(got - full[0, rows.numpy()]).max() < TOL
        # a key slice that starts later than position 0 (only for a finite window)
        if W > 0:
            rows = torch.tensor([40, 41, 63])
            got = oracle.prefill_rows(q[0, rows], rows, k[0, 30:], v[0, 30:], sinks, W, 0, k_base=30)
            assert np.abs(got - full[0, rows.numpy()]).max() < TOL


def pin_ring_append_placement():
    B, T, Hkv, D = 5, 4, 2, 3
    for ring, slots in ((True, 8), (False, 24)):
        rng = np.random.default_rng(7)
        kc = rng.standard_normal((B, slots, Hkv, D)).astype(np.float32)
        vc = rng.standard_normal((B, slots, Hkv, D)).astype(np.float32)
        kn = rng.standard_normal((B, T, Hkv, D)).astype(np.float32)
        vn = rng.standard_normal((B, T, Hkv, D)).astype(np.float32)
        L = np.array([0, 3, 7, 17, 20]) if ring else np.array([0, 3, 7, 17, 20])
        na = np.array([4, 0, 3, 1, 4])
        k0, v0 = kc.copy(), vc.copy()
        oracle.ring_append(kc, vc, kn, vn, L, na, ring)
        for b in range(B):
            written = {}
            for t in range(na[b]):
                p = L[b] + t
                written[(p % slots) if ring else p] = t
            for s in range(slots):
                if s in written:
                    assert np.array_equal(kc[b, s], kn[b, written[s]])
                    assert np.array_equal(vc[b, s], vn[b, written[s]])
                else:
                    assert np.array_equal(kc[b, s], k0[b, s]) and np.array_equal(vc[b, s], v0[b, s])


def _onehot_logits(tokens, V, base=-3.0, peak=5.0):
    """logits [B,T,V] whose row (b,t) peaks at tokens[b][t]."""
    B, T = len(tokens), len(tokens[0])
    lg = np.full((B, T, V), base, dtype=np.float32)
    for b in range(B):
        for t in range(T):
            lg[b, t, tokens[b][t]] = peak
    return lg


def pin_accept_blog_example():
    # verify diagram: token i and drafts i+1..i+3 go in; the model's outputs
    # for i+1 and i+2 match the drafts (accepted), the one for i+3 does not
    # (rejected: it becomes the corrected token) and the one for i+4 is
    # discarded.  Rows i, i+1, i+2 join the cache.
    V = 11
    target = [[4, 9, 2, 7]]
    draft = np.array([[4, 9, 5]], dtype=np.int32)
    tg, na = oracle.greedy_accept(_onehot_logits(target, V), draft)
    assert tg.tolist() == target and na.tolist() == [3]


def pin_accept_stops_at_first_rejection():
    V = 7
    target = [[1, 2, 3, 4], [1, 2, 3, 4], [1, 2, 3, 4]]
    draft = np.array([[0, 2, 3],      # first draft wrong: later matches discarded
                      [1, 0, 3],      # second wrong
                      [1, 2, 3]],     # all three accepted
                     dtype=np.int32)
    tg, na = oracle.greedy_accept(_onehot_logits(target, V), draft)
    assert tg.tolist() == target and na.tolist() == [1, 2, 4]


def pin_accept_ties_and_edges():
    V = 9
    lg = np.zeros((3, 2, V), dtype=np.float32)
    lg[0, 0, [2, 5]] = 1.0           # tie between 2 and 5 -> 2
    lg[0, 1, [8, 3]] = 2.0           # tie between 3 and 8 -> 3
    lg[1, :, :] = -np.inf            # every entry equal -> 0
    lg[2, 0, V - 1] = 0.5            # maximum at the last index
    lg[2, 1, :] = -1.0
    draft = np.array([[2], [1], [V - 1]], dtype=np.int32)
    tg, na = oracle.greedy_accept(lg, draft)
    assert tg.tolist() == [[2, 3], [0, 0], [V - 1, 0]]
    assert na.tolist() == [2, 1, 2]
    # q_len = 1 (plain decode): nothing to accept, one row appended
    tg1, na1 = oracle.greedy_accept(lg[:, :1], np.zeros((3, 0), dtype=np.int32))
    assert tg1.tolist() == [[2], [0], [V - 1]] and na1.tolist() == [1, 1, 1]


def pin_accept_vs_numpy_argmax():
    rng = np.random.default_rng(11)
    B, T, V = 40, 4, 37
    # small integer logits: many exact ties
    lg = rng.integers(-3, 4, size=(B, T, V)).astype(np.float32)
    ref_t = np.argmax(lg, axis=-1)   # numpy returns the first maximal index
    # drafts agree with the reference target with probability 3/4 each
    draft = np.where(rng.random((B, T - 1)) < 0.75, ref_t[:, :T - 1],
                     rng.integers(0, V, size=(B, T - 1))).astype(np.int32)
    tg, na = oracle.greedy_accept(lg, draft)
    assert np.array_equal(tg, ref_t)
    for b in range(B):
        n = 0
        while n < T - 1 and draft[b, n] == ref_t[b, n]:
            n += 1
        assert na[b] == n + 1
    assert len(set(na.tolist())) == T   # every acceptance length occurs


def pin_rope_closed_form():
    # D = 8, rot = 4, base 100: pairs (0, 2) and (1, 3) turn by p and p / 10
    p = 3
    eye = np.eye(8).reshape(8, 1, 8)
    out = oracle.rope(eye, np.full(8, p), 4, 100.0)[:, 0, :]
    a0, a1 = 3.0, 3.0 * 100.0 ** (-2.0 / 4.0)
    exp = np.eye(8)
    exp[0, [0, 2]] = [math.cos(a0), math.sin(a0)]
    exp[2, [0, 2]] = [-math.sin(a0), math.cos(a0)]
    exp[1, [1, 3]] = [math.cos(a1), math.sin(a1)]
    exp[3, [1, 3]] = [-math.sin(a1), math.cos(a1)]
    assert np.abs(out - exp).max() < TOL
    assert oracle.rope_dims(128) == 42 and oracle.rope_dims(64) == 20 and oracle.rope_dims(192) == 64


def pin_rope_identity_composition_norm():
    x = _rand((5, 3, 128), "rope")
    rot, base = 42, 640000.0
    assert np.array_equal(oracle.rope(x, np.zeros(5), rot, base), x.numpy())
    p1 = np.array([1, 17, 4096, 65535, 262147])
    p2 = np.array([5, 0, 123, 1, 99])
    twice = oracle.rope(oracle.rope(x, p1, rot, base), p2, rot, base)
    once = oracle.rope(x, p1 + p2, rot, base)
    assert np.abs(twice - once).max() < 1e-9
    y = oracle.rope(x, p1, rot, base)
    xn = x.numpy()
    assert np.array_equal(y[..., rot:], xn[..., rot:])
    h = rot // 2
    n_in = xn[..., :h] ** 2 + xn[..., h:rot] ** 2
    n_out = y[..., :h] ** 2 + y[..., h:rot] ** 2
    assert np.abs(n_in - n_out).max() < 1e-12
    assert oracle.rope(x, p1, 0, base).tolist() == xn.tolist()


def pin_rope_relative_position():
    q = _rand((1, 1, 64), "rope_q")
    k = _rand((1, 1, 64), "rope_k")
    rot, base = 20, 10000.0
    ref = None
    for c in (0, 7, 1000, 250000):
        qq = oracle.rope(q, [100 + c], rot, base)[0, 0]
        kk = oracle.rope(k, [37 + c], rot, base)[0, 0]
        dot = float(qq @ kk)
        ref = dot if ref is None else ref
        assert abs(dot - ref) < 1e-9


BWD_CASES = [
    # B, Sq, Sk, Hq, Hkv, D, window, q_offset
    (1, 7, 7, 2, 1, 4, 3, 0),
    (2, 5, 9, 4, 2, 4, 0, 4),
    (1, 6, 6, 2, 2, 3, 1, 0),
]


def _bwd_inputs(n, B, Sq, Sk, Hq, Hkv, D):
    r = lambda shape, tag: _rand(shape, "bwd", tag, n).to(torch.bfloat16).double()
    return (r((B, Sq, Hq, D), "q"), r((B, Sk, Hkv, D), "k"), r((B, Sk, Hkv, D), "v"),
            r((B, Sq, Hq, D), "do"), _rand((Hq,), "bwd", "s", n))


def pin_backward_finite_differences():
    eps = 2.0 ** -10
    rng = np.random.default_rng(3)
    for n, (B, Sq, Sk, Hq, Hkv, D, W, off) in enumerate(BWD_CASES):
        q, k, v, do, sinks = _bwd_inputs(n, B, Sq, Sk, Hq, Hkv, D)
        scale = 0.7
        grads = oracle.prefill_backward(q, k, v, do, sinks, W, off, scale)
        dn = do.numpy()

        def loss(qq, kk, vv, ss):
            return float((oracle.prefill(qq, kk, vv, ss, W, off, scale) * dn).sum())

        for which, (x, g) in enumerate(zip((q, k, v), grads[:3])):
            flat = x.reshape(-1)
            for idx in rng.choice(flat.numel(), size=min(10, flat.numel()), replace=False):
                args = [q, k, v]
                hi, lo = flat.clone(), flat.clone()
                hi[idx] += eps
                lo[idx] -= eps
                args[which] = hi.view(x.shape)
                f_hi = loss(*args, sinks)
                args[which] = lo.view(x.shape)
                f_lo = loss(*args, sinks)
                fd = (f_hi - f_lo) / (2 * eps)
                assert abs(fd - g.reshape(-1)[idx]) < 2e-5, (n, which, int(idx), fd, g.reshape(-1)[idx])
        for h in range(Hq):
            e = torch.zeros(Hq, dtype=torch.float64)
            e[h] = 1e-4
            fd = (loss(q, k, v, sinks + e) - loss(q, k, v, sinks - e)) / 2e-4
            assert abs(fd - grads[3][h]) < 1e-6, (n, h, fd, grads[3][h])


def pin_backward_vs_torch_autograd():
    for n, (B, Sq, Sk, Hq, Hkv, D, W, off) in enumerate(BWD_CASES + [(2, 17, 23, 4, 2, 16, 4, 6)]):
        q, k, v, do, sinks = _bwd_inputs(n + 10, B, Sq, Sk, Hq, Hkv, D)
        scale = 1.0 / math.sqrt(D)
        got = oracle.prefill_backward(q, k, v, do, sinks, W, off, scale)
        ts = [t.clone().requires_grad_(True) for t in (q, k, v, sinks)]
        G = Hq // Hkv
        qt = ts[0].permute(0, 2, 1, 3)
        kt = ts[1].repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
        vt = ts[2].repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
        i = torch.arange(Sq).view(-1, 1) + off
        j = torch.arange(Sk).view(1, -1)
        allowed = j <= i
        if W > 0:
            allowed &= j > i - W
        bias = torch.zeros(Sq, Sk, dtype=torch.float64).masked_fill(~allowed, float("-inf"))
        bias = bias.view(1, 1, Sq, Sk).expand(B, Hq, Sq, Sk)
        zk = torch.zeros(B, Hq, 1, D, dtype=torch.float64)
        kt = torch.cat([kt, zk], dim=2)
        vt = torch.cat([vt, zk], dim=2)
        bias = torch.cat([bias, ts[3].view(1, Hq, 1, 1).expand(B, Hq, Sq, 1)], dim=3)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                                             attn_mask=bias, scale=scale)
        (o.permute(0, 2, 1, 3) * do).sum().backward()
        for name, a, t in zip(("dq", "dk", "dv", "dsink"), got, ts):
            err = np.abs(a - t.grad.numpy()).max()
            assert err < 1e-10, (n, name, err)


def pin_backward_sink_identity():
    B, Sq, Sk, Hq, Hkv, D, W, off = 2, 12, 12, 4, 2, 8, 5, 0
    q, k, v, do, sinks = _bwd_inputs(99, B, Sq, Sk, Hq, Hkv, D)
    fwd = oracle.prefill(q, k, v, sinks, W, off, 0.5, want_psink=True)
    delta = (fwd["o"] * do.numpy()).sum(-1)                       # [B, Sq, Hq]
    ref = -(fwd["psink"] * delta).sum(axis=(0, 1))
    got = oracle.prefill_backward(q, k, v, do, sinks, W, off, 0.5)[3]
    assert np.abs(got - ref).max() < 1e-12
    # no sink: no sink gradient, and the other gradients equal those of -inf
    a = oracle.prefill_backward(q, k, v, do, None, W, off, 0.5)
    b = oracle.prefill_backward(q, k, v, do, torch.full((Hq,), float("-inf")), W, off, 0.5)
    assert not a[3].any()
    for x, y in zip(a[:3], b[:3]):
        assert np.abs(x - y).max() < 1e-12


ALL_PINS = [
    pin_sdpa_with_sink_column,
    pin_no_sink_is_band_softmax,
    pin_wide_window_is_causal,
    pin_window_one_closed_form,
    pin_zero_query_window_membership,
    pin_weights_and_sink_mass_sum_to_one,
    pin_lse_sigmoid_identity,
    pin_gqa_equals_repeated_heads,
    pin_verify_equals_prefill_rows,
    pin_verify_equals_successive_decodes,
    pin_chunked_prefill_equals_unchunked,
    pin_ring_append_placement,
    pin_accept_blog_example,
    pin_accept_stops_at_first_rejection,
    pin_accept_ties_and_edges,
    pin_accept_vs_numpy_argmax,
    pin_rope_closed_form,
    pin_rope_identity_composition_norm,
    pin_rope_relative_position,
    pin_backward_finite_differences,
    pin_backward_vs_torch_autograd,
    pin_backward_sink_identity,
]
