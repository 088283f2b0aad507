"""Seeded synthetic inputs for sliding-window / global attention with sinks.

This module is the only code shared by the CPU oracle tests, the GPU parity
tests and the benchmark.  It holds none of the attention arithmetic: it draws
seeded N(0,1) tensors, rounds them to the storage dtype, draws request context
lengths, and lays a logical per-request KV history out in the two cache
layouts the verify step reads (a ring of ``slots`` rows where position ``p``
lives in slot ``p % slots``, or a linear cache where it lives in slot ``p``).
Slots that hold no committed position are filled with NaN so that any read of
them shows up in the output.

Workload shapes follow the hybrid-attention model the pages describe: window
W=128 (MiMo-V2-Flash technical-report digest, section "Model Architecture";
release blog, section on efficiency), 64 query heads (model card config
extract), 8 KV heads and head_dim 128 (assumed; the pages do not give them).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

__all__ = [
    "PrefillConfig", "VerifyConfig", "PREFILL_CONFIGS", "VERIFY_CONFIGS",
    "derive_seed", "normal", "prefill_inputs", "verify_inputs",
    "ring_from_history", "linear_from_history", "sample_rows", "torch_dtype",
    "AcceptConfig", "ACCEPT_CONFIGS", "accept_inputs", "tied_logits",
]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def derive_seed(*keys) -> int:
    """A 62-bit seed from any tuple of ints/strings (stable across runs)."""
    h = hashlib.sha256(repr(keys).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 62) - 1)


def normal(shape, seed: int, device="cpu", dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """i.i.d. N(0,1) drawn in fp32 from a seeded generator, then rounded
    (round-to-nearest-even) to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    S: int            # query rows per request
    Hq: int
    Hkv: int
    D: int
    window: int       # <= 0 means global (W = infinity)
    dtype: str        # "f32" or "bf16"
    seed: int
    Sk: Optional[int] = None   # key rows (defaults to S); q_offset = Sk - S
    chunk: Optional[int] = None  # chunked prefill: queries split into chunks of this size

    @property
    def keys(self) -> int:
        return self.S if self.Sk is None else self.Sk

    @property
    def q_offset(self) -> int:
        return self.keys - self.S

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)


@dataclasses.dataclass(frozen=True)
class VerifyConfig:
    name: str
    B: int
    T: int            # query length per request (1 committed + drafts)
    Hq: int
    Hkv: int
    D: int
    window: int       # <= 0 means global
    ring: bool        # True: ring of `slots` rows; False: linear cache
    slots: int
    len_lo: int       # context length drawn uniformly in [len_lo, len_hi]
    len_hi: int
    dtype: str
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)


PREFILL_CONFIGS = {
    # tiny fp32 SWA + sink prefill
    "tiny_f32": PrefillConfig("tiny_f32", 1, 512, 4, 1, 64, 128, "f32", seed=1),
    # SWA layer prefill, 32K tokens
    "swa_32k": PrefillConfig("swa_32k", 1, 32768, 64, 8, 128, 128, "bf16", seed=2),
    # global-attention layer prefill, 32K tokens
    "ga_32k": PrefillConfig("ga_32k", 1, 32768, 64, 8, 128, 0, "bf16", seed=3),
    # one SWA layer of the 256K stack: 8 chunks of 32768 queries over all keys
    "swa_256k": PrefillConfig("swa_256k", 1, 262144, 64, 8, 128, 128, "bf16", seed=5, chunk=32768),
}

VERIFY_CONFIGS = {
    # q_len=4 MTP verify, 64 requests, global-layer cache, contexts U[4096, 65536]
    "verify_ga_b64": VerifyConfig("verify_ga_b64", 64, 4, 64, 8, 128, 0, False, 65536,
                                  4096, 65536, "bf16", seed=4),
    # the same requests on an SWA layer: 128-slot ring buffer, W=128
    "verify_swa_b64": VerifyConfig("verify_swa_b64", 64, 4, 64, 8, 128, 128, True, 128,
                                   4096, 65536, "bf16", seed=4),
    # global-layer verify of the 256K stack: one request, 262144 committed tokens
    "verify_ga_256k": VerifyConfig("verify_ga_256k", 1, 4, 64, 8, 128, 0, False, 262144 + 4,
                                   262144, 262144, "bf16", seed=5),
    # plain single-token decode (q_len=1, also the MTP draft layers' step) on the
    # same 64-request shapes: global-layer cache and 128-slot SWA ring
    "decode_ga_b64": VerifyConfig("decode_ga_b64", 64, 1, 64, 8, 128, 0, False, 65536,
                                  4096, 65536, "bf16", seed=6),
    "decode_swa_b64": VerifyConfig("decode_swa_b64", 64, 1, 64, 8, 128, 128, True, 128,
                                   4096, 65536, "bf16", seed=6),
}


def prefill_inputs(cfg: PrefillConfig, device="cpu", dtype: Optional[torch.dtype] = None):
    """q [B,S,Hq,D], k,v [B,Sk,Hkv,D] in the config dtype; sinks [Hq] fp32."""
    dt = torch_dtype(cfg.dtype) if dtype is None else dtype
    q = normal((cfg.B, cfg.S, cfg.Hq, cfg.D), derive_seed(cfg.seed, "q"), device, dt)
    k = normal((cfg.B, cfg.keys, cfg.Hkv, cfg.D), derive_seed(cfg.seed, "k"), device, dt)
    v = normal((cfg.B, cfg.keys, cfg.Hkv, cfg.D), derive_seed(cfg.seed, "v"), device, dt)
    sinks = normal((cfg.Hq,), derive_seed(cfg.seed, "sinks"), device, torch.float32)
    return q, k, v, sinks


def draw_lengths(B: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """Per-request committed context lengths, uniform integers in [lo, hi]."""
    g = torch.Generator()
    g.manual_seed(derive_seed(seed, "cache_len"))
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64)


def ring_from_history(hist: torch.Tensor, hist_base, cache_len, slots: int) -> torch.Tensor:
    """Lay a logical history out as a ring cache [B, slots, Hkv, D].

    ``hist[b, r]`` holds position ``hist_base[b] + r``.  Every committed
    position p in [max(0, L_b - slots), L_b) goes to slot ``p % slots``;
    slots that hold no position are NaN."""
    B, _, Hkv, D = hist.shape
    ring = torch.full((B, slots, Hkv, D), float("nan"), dtype=hist.dtype, device=hist.device)
    for b in range(B):
        L = int(cache_len[b])
        p0 = max(0, L - slots)
        if L <= p0:
            continue
        base = int(hist_base[b])
        assert p0 >= base, "history does not reach back far enough for this ring"
        pos = torch.arange(p0, L, device=hist.device)
        ring[b, pos % slots] = hist[b, pos - base]
    return ring


def linear_from_history(hist: torch.Tensor, cache_len, slots: int) -> torch.Tensor:
    """Linear cache [B, slots, Hkv, D] with history position p in slot p; slots
    at or beyond L_b are NaN.  ``hist`` must start at position 0."""
    B, H, Hkv, D = hist.shape
    out = torch.full((B, slots, Hkv, D), float("nan"), dtype=hist.dtype, device=hist.device)
    for b in range(B):
        L = int(cache_len[b])
        out[b, :L] = hist[b, :L]
    return out


def verify_inputs(cfg: VerifyConfig, device="cpu", dtype: Optional[torch.dtype] = None,
                  build_cache: bool = True, cache_len=None):
    """Inputs of one verify call.

    Returns a dict with cache_len [B] (int64, host), q [B,T,Hq,D], k_new/v_new
    [B,T,Hkv,D], the logical history k_hist/v_hist [B,Hlen,Hkv,D] with
    hist_base [B] (history row r is position hist_base[b] + r), sinks [Hq], and
    (if build_cache) the cache k_cache/v_cache [B, slots, Hkv, D] in the
    config's layout.

    A ring config only draws the last ``slots`` positions of each history (the
    older ones can never be inside its window); a linear config draws the whole
    history.  Linear histories are drawn per request with a per-request seed so
    a request's values do not depend on the batch size.
    """
    dt = torch_dtype(cfg.dtype) if dtype is None else dtype
    if cache_len is None:
        cache_len = draw_lengths(cfg.B, cfg.len_lo, cfg.len_hi, cfg.seed)
    cache_len = torch.as_tensor(cache_len, dtype=torch.int64).cpu()
    B, T, Hq, Hkv, D = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.D
    layer = "swa" if cfg.ring else "ga"
    q = normal((B, T, Hq, D), derive_seed(cfg.seed, layer, "q"), device, dt)
    k_new = normal((B, T, Hkv, D), derive_seed(cfg.seed, layer, "k_new"), device, dt)
    v_new = normal((B, T, Hkv, D), derive_seed(cfg.seed, layer, "v_new"), device, dt)
    sinks = normal((Hq,), derive_seed(cfg.seed, layer, "sinks"), device, torch.float32)
    if cfg.ring:
        hlen = cfg.slots
        hist_base = torch.clamp(cache_len - cfg.slots, min=0)
    else:
        hlen = cfg.slots
        hist_base = torch.zeros(B, dtype=torch.int64)
        assert int(cache_len.max()) <= cfg.slots, "linear cache too small for the context"
    k_hist = torch.empty((B, hlen, Hkv, D), dtype=dt, device=device)
    v_hist = torch.empty((B, hlen, Hkv, D), dtype=dt, device=device)
    for b in range(B):
        n = int(min(hlen, int(cache_len[b]) - int(hist_base[b])))
        k_hist[b, :n] = normal((n, Hkv, D), derive_seed(cfg.seed, layer, "k_hist", b), device, dt)
        v_hist[b, :n] = normal((n, Hkv, D), derive_seed(cfg.seed, layer, "v_hist", b), device, dt)
        k_hist[b, n:] = float("nan")
        v_hist[b, n:] = float("nan")
    out = dict(cache_len=cache_len, q=q, k_new=k_new, v_new=v_new, k_hist=k_hist,
               v_hist=v_hist, hist_base=hist_base, sinks=sinks)
    if build_cache:
        if cfg.ring:
            out["k_cache"] = ring_from_history(k_hist, hist_base, cache_len, cfg.slots)
            out["v_cache"] = ring_from_history(v_hist, hist_base, cache_len, cfg.slots)
        else:
            # the history tensor already is the linear cache (NaN beyond L_b)
            out["k_cache"] = k_hist
            out["v_cache"] = v_hist
    return out


def sample_rows(S: int, n: int, seed: int, forced=()) -> torch.Tensor:
    """Sorted distinct query rows: ``n`` drawn uniformly without replacement
    plus the ``forced`` rows that lie in [0, S)."""
    g = torch.Generator()
    g.manual_seed(derive_seed(seed, "rows", S, n))
    n = min(n, S)
    pick = torch.randperm(S, generator=g)[:n]
    forced = torch.tensor([r for r in forced if 0 <= r < S], dtype=torch.int64)
    return torch.unique(torch.cat([pick, forced]))


@dataclasses.dataclass(frozen=True)
class AcceptConfig:
    name: str
    B: int
    T: int            # verified positions per request (1 committed + T-1 drafts)
    vocab: int
    p_accept: float   # probability that a draft equals the planted top token
    dtype: str        # logits dtype
    seed: int


ACCEPT_CONFIGS = {
    # 64 requests, 3 drafts; per-draft agreement 0.83 gives a mean of
    # 1 + p + p^2 + p^3 = 3.09 tokens per step, inside the reported 2.8-3.6.
    # The vocabulary size is not on the pages; 152064 is assumed.
    "accept_b64": AcceptConfig("accept_b64", 64, 4, 152064, 0.83, "bf16", seed=8),
}


def accept_inputs(cfg: AcceptConfig, device="cpu", step: int = 0):
    """Synthetic verify logits [B,T,vocab] and drafts [B,T-1] int32.

    Logits are N(0,1) with one planted entry of +8 per row (at a uniformly
    drawn token), far above every other draw.  Draft t equals the planted
    token of row t with probability ``p_accept`` and otherwise is another
    uniformly drawn token, so the acceptance length follows the geometric
    prefix law of independent per-draft agreement."""
    dt = torch_dtype(cfg.dtype)
    B, T, V = cfg.B, cfg.T, cfg.vocab
    logits = normal((B, T, V), derive_seed(cfg.seed, step, "logits"), device, torch.float32)
    g = torch.Generator()
    g.manual_seed(derive_seed(cfg.seed, step, "tokens"))
    top = torch.randint(0, V, (B, T), generator=g)
    agree = torch.rand((B, max(T - 1, 0)), generator=g) < cfg.p_accept
    other = (top[:, :T - 1] + 1 + torch.randint(0, max(V - 1, 1), (B, max(T - 1, 0)), generator=g)) % V
    draft = torch.where(agree, top[:, :T - 1], other).to(torch.int32)
    logits = logits.view(B * T, V)
    logits[torch.arange(B * T, device=logits.device), top.reshape(-1).to(logits.device)] = 8.0
    logits = logits.view(B, T, V).to(dt)
    return logits, draft.to(device)


def tied_logits(B: int, T: int, V: int, seed: int, lo: int = -2, hi: int = 2,
                device="cpu", dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Integer-valued logits in [lo, hi]: every row has many equal maxima."""
    g = torch.Generator()
    g.manual_seed(derive_seed(seed, "tied", B, T, V))
    x = torch.randint(lo, hi + 1, (B, T, V), generator=g).to(torch.float32)
    return x.to(device=device, dtype=dtype)
