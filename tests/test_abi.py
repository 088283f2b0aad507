"""CPU checks of the C ABI: the library loads, exports exactly the declared
entry points, and rejects bad host-visible arguments before launching
anything (these calls return before any HIP call, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import hybrid_sliding_window_swa_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa_attn.h")
OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4
BF16, F32 = 1, 0


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(swa.library_path()):
        from hybrid_sliding_window_swa_amd import build
        build.build()
    return swa.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return set(re.findall(r"^SWA_API\s+(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, re.M))


def test_header_declares_entry_points():
    assert declared_symbols() == set(swa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    # and nothing else with external linkage in the text section
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", swa.library_path()],
                         capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == declared_symbols()


def test_status_strings(lib):
    for code in range(6):
        assert lib.swa_status_string(code)


def _prefill(lib, q=1, k=1, v=1, o=1, B=1, Sq=8, Sk=8, Hq=8, Hkv=1, D=128, W=128, off=0, dt=BF16,
             scale=0.1):
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.swa_attn_prefill(P(q), P(k), P(v), None, P(o), B, Sq, Sk, Hq, Hkv, D, W, off, scale, dt, None)


def test_prefill_validation(lib):
    assert _prefill(lib, q=0) == NULL
    assert _prefill(lib, o=0) == NULL
    assert _prefill(lib, Hq=6, Hkv=4) == SHAPE
    assert _prefill(lib, D=96) == UNSUP
    assert _prefill(lib, D=256) == UNSUP
    assert _prefill(lib, off=1) == SHAPE            # q_offset + Sq > Sk
    assert _prefill(lib, off=-1) == SHAPE
    assert _prefill(lib, Sq=-1) == SHAPE
    assert _prefill(lib, dt=7) == UNSUP
    assert _prefill(lib, Hq=64, Hkv=1) == UNSUP     # bf16 needs 32 % G == 0
    assert _prefill(lib, Hq=12, Hkv=4) == UNSUP     # G = 3
    assert _prefill(lib, Hq=256, Hkv=1, dt=F32) == UNSUP
    assert _prefill(lib, scale=0.0) == UNSUP
    assert _prefill(lib, scale=-0.1) == UNSUP
    assert _prefill(lib, scale=float("nan")) == UNSUP
    assert _prefill(lib, scale=float("inf")) == UNSUP
    # empty work is a no-op even with NULL pointers
    assert _prefill(lib, q=0, k=0, v=0, o=0, B=0) == OK
    assert _prefill(lib, q=0, k=0, v=0, o=0, Sq=0) == OK


def _verify(lib, ptr=1, B=2, T=4, Hq=64, Hkv=8, D=128, slots=128, ring=1, W=128, dt=BF16,
            ws=None, ws_bytes=0, scale=0.1):
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.swa_attn_verify(P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), None, P(ptr),
                               B, T, Hq, Hkv, D, slots, ring, W, scale, dt, P(ws), ws_bytes, None)


def test_verify_validation(lib):
    assert _verify(lib, ptr=0) == NULL
    assert _verify(lib, T=0) == SHAPE
    assert _verify(lib, T=17) == SHAPE
    assert _verify(lib, slots=127) == SHAPE          # ring shorter than the window
    assert _verify(lib, W=0) == SHAPE                # ring needs a finite window
    assert _verify(lib, ring=2) == SHAPE
    assert _verify(lib, Hq=63) == SHAPE
    assert _verify(lib, D=32) == UNSUP
    assert _verify(lib, T=9) == UNSUP                # bf16: G * q_len <= 64
    assert _verify(lib, dt=3) == UNSUP
    assert _verify(lib, scale=0.0) == UNSUP
    assert _verify(lib, scale=float("nan")) == UNSUP
    # linear global cache with many rows needs a workspace
    assert _verify(lib, ring=0, W=0, slots=65536, ws=None) == WS
    need = lib.swa_attn_verify_workspace_bytes(2, 4, 64, 8, 128, 65536, 0, 0, BF16)
    assert need > 0
    assert _verify(lib, ring=0, W=0, slots=65536, ws=256, ws_bytes=need - 1) == WS
    assert _verify(lib, ring=0, W=0, slots=65536, ws=257, ws_bytes=need) == WS  # misaligned
    assert _verify(lib, B=0, ptr=0) == OK


def _verify_noalloc(lib, ptr=1, B=2, T=4, Hq=64, Hkv=8, D=128, slots=128, ring=1, W=128, dt=BF16,
                    scale=0.1):
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.swa_attn_verify_noalloc(P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), None, P(ptr),
                                       B, T, Hq, Hkv, D, slots, ring, W, scale, dt, None)


def test_verify_noalloc_validation(lib):
    """The allocation-free verify rejects what swa_attn_verify rejects, and
    sizes whose split partials exceed its fixed scratch, before any HIP call."""
    assert _verify_noalloc(lib, ptr=0) == NULL
    assert _verify_noalloc(lib, T=17) == SHAPE
    assert _verify_noalloc(lib, slots=127) == SHAPE
    assert _verify_noalloc(lib, D=32) == UNSUP
    assert _verify_noalloc(lib, scale=float("nan")) == UNSUP
    assert _verify_noalloc(lib, B=0, ptr=0) == OK
    limit = 64 << 20
    # 128 requests over 65536-slot global caches: 68 MB of partials > 64 MiB
    assert lib.swa_attn_verify_workspace_bytes(128, 4, 64, 8, 128, 65536, 0, 0, BF16) > limit
    assert _verify_noalloc(lib, B=128, ring=0, W=0, slots=65536) == WS
    assert lib.swa_attn_verify_workspace_bytes(64, 4, 64, 8, 128, 65536, 0, 0, BF16) <= limit


def test_workspace_sizes(lib):
    ws = lambda *a: lib.swa_attn_verify_workspace_bytes(*a)
    # ring of 128 slots: one split, the kernel writes O directly
    assert ws(64, 4, 64, 8, 128, 128, 1, 128, BF16) == 0
    # fp32 path needs none
    assert ws(64, 4, 64, 8, 128, 65536, 0, 0, F32) == 0
    # invalid arguments -> 0
    assert ws(64, 4, 64, 8, 100, 65536, 0, 0, BF16) == 0
    # global cache of 65536 rows: splits of <= 16384 rows, (D + 2) floats per row and split
    b = ws(64, 4, 64, 8, 128, 65536, 0, 0, BF16)
    assert b == 64 * 8 * 4 * 32 * 130 * 4
    # one request of 262148 rows: the 8 KV heads paired (4 items per split), so
    # splits of 4096 rows for about 256 workgroups: 65 splits
    assert ws(1, 4, 64, 8, 128, 262148, 0, 0, BF16) == 1 * 8 * 65 * 32 * 130 * 4
    # with an odd number of KV heads there are no pairs: 7 items, splits of 8192 rows
    assert ws(1, 4, 56, 7, 128, 262148, 0, 0, BF16) == 1 * 7 * 33 * 32 * 130 * 4


def _append(lib, ptr=1, B=2, T=4, Hkv=8, D=128, slots=128, ring=1, dt=BF16):
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.kv_ring_append(P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), P(ptr), B, T, Hkv, D,
                              slots, ring, dt, None)


def test_append_validation(lib):
    assert _append(lib, ptr=0) == NULL
    assert _append(lib, slots=0) == SHAPE
    assert _append(lib, T=0) == SHAPE
    assert _append(lib, ring=5) == SHAPE
    assert _append(lib, Hkv=1, D=3) == UNSUP        # row not a multiple of 16 bytes
    assert _append(lib, B=0, ptr=0) == OK


def _accept(lib, ptr=1, draft=1, B=64, T=4, V=152064, dt=BF16, ws=256, ws_bytes=1 << 30):
    P = lambda x: ctypes.c_void_p(x) if x else None
    return lib.swa_mtp_greedy_accept(P(ptr), P(draft), P(ptr), P(ptr), B, T, V, dt, P(ws), ws_bytes, None)


def test_accept_validation(lib):
    assert _accept(lib, ptr=0) == NULL
    assert _accept(lib, draft=0) == NULL             # drafts are needed when q_len > 1
    assert _accept(lib, T=0) == SHAPE
    assert _accept(lib, T=17) == SHAPE
    assert _accept(lib, V=0) == SHAPE
    assert _accept(lib, V=1 << 31) == SHAPE          # indices are int32
    assert _accept(lib, B=16384, T=4) == SHAPE       # B * q_len > 65535
    assert _accept(lib, dt=9) == UNSUP
    assert _accept(lib, ws=0) == WS
    need = lib.swa_mtp_accept_workspace_bytes(64, 4, 152064)
    assert need > 0
    assert _accept(lib, ws_bytes=need - 1) == WS
    assert _accept(lib, ws=258, ws_bytes=need) == WS  # not 4-byte aligned
    assert _accept(lib, B=0, ptr=0, draft=0, ws=0, ws_bytes=0) == OK


def test_accept_workspace_sizes(lib):
    ws = lib.swa_mtp_accept_workspace_bytes
    # every row is split into chunks of a multiple of 1024 logits, about 2048
    # workgroups per launch; 8 bytes (max, index) per row and chunk
    assert ws(64, 4, 152064) == 64 * 4 * 8 * 8        # 8 chunks of 19456
    assert ws(1, 1, 152064) == 149 * 8                # 149 chunks of 1024
    assert ws(1, 1, 5) == 8                           # one short chunk
    assert ws(0, 4, 100) == 0 and ws(2, 0, 100) == 0 and ws(2, 4, 0) == 0


def test_advance_validation(lib):
    P = lambda x: ctypes.c_void_p(x) if x else None
    assert lib.swa_cache_advance(P(0), P(1), 4, None) == NULL
    assert lib.swa_cache_advance(P(1), P(1), -1, None) == SHAPE
    assert lib.swa_cache_advance(P(0), P(0), 0, None) == OK


def _rope(lib, x=256, B=2, S=8, H=8, D=128, rot=42, off=0, base=10000.0, dt=BF16):
    P = lambda v: ctypes.c_void_p(v) if v else None
    return lib.swa_rope_apply(P(x), None, off, B, S, H, D, rot, base, dt, None)


def test_rope_validation(lib):
    assert _rope(lib, x=0) == NULL
    assert _rope(lib, x=264) == UNSUP            # not 16-byte aligned
    assert _rope(lib, rot=43) == SHAPE           # odd
    assert _rope(lib, rot=130) == SHAPE          # beyond D
    assert _rope(lib, D=100) == SHAPE            # D % 8 != 0
    assert _rope(lib, D=264, rot=42) == SHAPE    # D > 256
    assert _rope(lib, off=-1) == SHAPE
    assert _rope(lib, H=0) == SHAPE
    assert _rope(lib, base=0.0) == UNSUP
    assert _rope(lib, base=float("nan")) == UNSUP
    assert _rope(lib, dt=5) == UNSUP
    assert _rope(lib, x=0, B=0) == OK and _rope(lib, x=0, S=0) == OK and _rope(lib, x=0, rot=0) == OK


def test_rope_dims_rule():
    assert swa.rope_dims(128) == 42 and swa.rope_dims(64) == 20 and swa.rope_dims(192) == 64


def test_prefill_rope_validation(lib):
    P = lambda v: ctypes.c_void_p(v) if v else None
    f = lambda rot=42, W=128, Hq=16, Hkv=2, D=128, dt=BF16, base=10000.0, ptr=256: lib.swa_attn_prefill_rope(
        P(ptr), P(ptr), P(ptr), None, P(ptr), 1, 64, 64, Hq, Hkv, D, W, 0, 0.1, rot, base, dt, None)
    assert f(rot=41) == SHAPE
    assert f(rot=130) == SHAPE
    assert f(base=-1.0) == UNSUP
    assert f(ptr=0) == NULL
    # host-visible unsupported configurations return before any launch
    assert f(rot=66) == UNSUP          # beyond D / 2
    assert f(W=0) == UNSUP             # global attention: not the strip kernel
    assert f(Hq=32, Hkv=2) == UNSUP    # G = 16
    assert f(dt=F32) == UNSUP


def test_backward_validation(lib):
    P = lambda v: ctypes.c_void_p(v) if v else None
    need = lib.swa_attn_backward_workspace_bytes(1, 64, 16)
    assert need > 0 and lib.swa_attn_backward_workspace_bytes(1, 64, 0) == 0

    def f(ptr=256, ws=256, ws_bytes=need, dt=BF16, Hq=16, Hkv=2, D=128, lse=256):
        return lib.swa_attn_backward(P(ptr), P(ptr), P(ptr), None, P(ptr), P(lse), P(ptr), P(ptr), P(ptr), P(ptr),
                                     None, 1, 64, 64, Hq, Hkv, D, 128, 0, 0.1, dt, P(ws), ws_bytes, None)
    assert f(dt=F32) == UNSUP
    assert f(lse=0) == NULL
    assert f(ws=0) == WS
    assert f(ws_bytes=need - 1) == WS
    assert f(ws=512 + 16) == WS                # not 256-byte aligned
    assert f(D=96) == UNSUP
    assert f(Hq=64, Hkv=1) == UNSUP            # 32 % G != 0
    assert lib.swa_attn_prefill_lse(P(256), P(256), P(256), None, P(256), None, 1, 8, 8, 16, 2, 128, 128, 0, 0.1,
                                    BF16, None) == NULL
    assert lib.swa_attn_prefill_lse(P(256), P(256), P(256), None, P(256), P(256), 1, 8, 8, 16, 2, 128, 128, 0, 0.1,
                                    F32, None) == UNSUP
