"""The C-ABI library without a GPU: exports, config and argument validation.

Validation runs before any HIP call, so every rejection below is checked on
the CPU; nothing here launches a kernel or touches device memory.
"""

import ctypes
import math
import os
import re
import subprocess

import pytest

from sparse_weight_memory_amd import _lib
from workloads import CONFIGS

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "fwpkm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fwpkm_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(fwpkm_lib):
    decl = declared_functions()
    assert set(decl) == set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fwpkm_\w+)", out))
    for name in decl:
        assert name in exported, name
        assert hasattr(fwpkm_lib, name)


def test_no_torch_types_in_the_header():
    text = open(HEADER).read()
    assert "torch" not in text.replace("torch tensors", "")
    assert 'extern "C"' in text


def cfg(**kw):
    base = dict(sqrt_slots=32, dim_qk=64, dim_v=64, topk=4, chunk_size=64,
                num_heads=1, max_batch=2, eps=1e-3, score_mode=_lib.SCORE_IDW)
    base.update(kw)
    return _lib.CConfig(**base)


def create(lib, c):
    h = ctypes.c_void_p()
    rc = lib.fwpkm_create(ctypes.byref(c), ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(sqrt_slots=0), _lib.ERR_INVALID_ARG),
    (dict(dim_qk=63), _lib.ERR_INVALID_ARG),
    (dict(dim_qk=0), _lib.ERR_INVALID_ARG),
    (dict(dim_v=0), _lib.ERR_INVALID_ARG),
    (dict(topk=0), _lib.ERR_INVALID_ARG),
    (dict(topk=33, sqrt_slots=32), _lib.ERR_INVALID_ARG),     # k > n
    (dict(chunk_size=0), _lib.ERR_INVALID_ARG),
    (dict(num_heads=0), _lib.ERR_INVALID_ARG),
    (dict(max_batch=0), _lib.ERR_INVALID_ARG),
    (dict(eps=0.0), _lib.ERR_INVALID_ARG),
    (dict(eps=float("nan")), _lib.ERR_INVALID_ARG),
    (dict(score_mode=7), _lib.ERR_INVALID_ARG),
    (dict(addr_weight=float("nan")), _lib.ERR_INVALID_ARG),
    (dict(addr_weight=float("inf")), _lib.ERR_INVALID_ARG),
    (dict(sqrt_slots=5000, topk=4), _lib.ERR_UNSUPPORTED),
    (dict(dim_qk=66), _lib.ERR_UNSUPPORTED),                  # d_h = 33
    (dict(dim_v=66), _lib.ERR_UNSUPPORTED),
    (dict(topk=33, sqrt_slots=64), _lib.ERR_UNSUPPORTED),
    (dict(chunk_size=2048), _lib.ERR_UNSUPPORTED),
    (dict(chunk_size=1024, topk=16), _lib.ERR_UNSUPPORTED),   # C*k > 8192
])
def test_create_rejects_bad_configs(fwpkm_lib, kw, code):
    rc, h = create(fwpkm_lib, cfg(**kw))
    assert rc == code
    assert h.value is None
    assert fwpkm_lib.fwpkm_last_error().decode() != ""
    assert fwpkm_lib.fwpkm_workspace_bytes(ctypes.byref(cfg(**kw))) == 0


@pytest.mark.parametrize("idx", sorted(CONFIGS))
def test_create_accepts_every_workload(fwpkm_lib, idx):
    w = CONFIGS[idx]
    c = cfg(sqrt_slots=w.sqrt_slots, dim_qk=w.dim_qk, dim_v=w.dim_v, topk=w.topk,
            chunk_size=w.chunk, num_heads=w.heads, max_batch=w.batch)
    rc, h = create(fwpkm_lib, c)
    assert rc == _lib.OK, fwpkm_lib.fwpkm_last_error()
    ws = fwpkm_lib.fwpkm_workspace_bytes(ctypes.byref(c))
    assert 0 < ws < 512 * 2 ** 20
    fwpkm_lib.fwpkm_destroy(h)
    fwpkm_lib.fwpkm_destroy(None)                         # NULL-safe


# ----------------------------------------------------------- forward checks
# Fake, never-dereferenced device addresses laid out far apart.
Q, Y, R = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000
PK1, PK2, PV = 0x40_0000_0000, 0x50_0000_0000, 0x60_0000_0000
NK1, NK2, NV = 0x70_0000_0000, 0x80_0000_0000, 0x90_0000_0000
SK = 32 * 32        # H*n*d_h elements
SV = 1024 * 64      # H*N*d_v elements


def state(k1, k2, v, sk=SK, sv=SV):
    return _lib.CState(k1, k2, v, sk, sv)


@pytest.fixture
def handle(fwpkm_lib):
    rc, h = create(fwpkm_lib, cfg())
    assert rc == _lib.OK
    yield h
    fwpkm_lib.fwpkm_destroy(h)


def fwd(lib, h, q=Q, y=Y, batch=2, tokens=64, lr=1.0, past=None, nxt=None, r=R, slots=None, w=None):
    past = past if past is not None else state(PK1, PK2, PV)
    nxt = nxt if nxt is not None else state(PK1, PK2, PV)
    return lib.fwpkm_forward_chunk(h, q, y, batch, tokens, lr, ctypes.byref(past), ctypes.byref(nxt),
                                   r, slots, w, None)


def test_forward_argument_errors(fwpkm_lib, handle):
    L = fwpkm_lib
    E = _lib.ERR_INVALID_ARG
    assert fwd(L, None) == E
    assert fwd(L, handle, q=None) == E
    assert fwd(L, handle, r=None) == E
    assert fwd(L, handle, batch=0) == E
    assert fwd(L, handle, batch=3) == E
    assert fwd(L, handle, tokens=0) == E
    assert fwd(L, handle, tokens=65) == E
    assert fwd(L, handle, lr=math.nan) == E
    assert fwd(L, handle, lr=math.inf) == E
    assert fwd(L, handle, past=state(PK1, None, PV)) == E
    assert fwd(L, handle, past=state(PK1, PK2, PV, sk=SK - 1)) == E
    # in place on a table shared by two sequences
    assert fwd(L, handle, past=state(PK1, PK2, PV, 0, 0), nxt=state(PK1, PK2, PV, 0, 0)) == E
    # a shared past may be expanded into per-sequence tables: that passes
    # validation and only then needs the device
    assert "stride" in L.fwpkm_last_error().decode()


def test_forward_alias_errors(fwpkm_lib, handle):
    L = fwpkm_lib
    A = _lib.ERR_ALIAS
    # next overlapping past without being the same tables
    assert fwd(L, handle, nxt=state(PK1 + 4, NK2, NV)) == A
    assert fwd(L, handle, nxt=state(NK1, NK2, PV + 4 * SV)) == A          # second sequence of past V
    # next tables overlapping each other
    assert fwd(L, handle, nxt=state(NK1, NK1 + 8, NV)) == A
    # retrieved overlapping an input or the state
    assert fwd(L, handle, r=Q + 16) == A
    assert fwd(L, handle, r=PV + 1024) == A
    # optional outputs overlapping each other or an input
    assert fwd(L, handle, slots=R + 64) == A
    assert fwd(L, handle, slots=0xA0_0000_0000, w=0xA0_0000_0010) == A
    assert fwd(L, handle, w=Y) == A
    # next state overlapping the queries
    assert fwd(L, handle, nxt=state(Q, NK2, NV)) == A


def test_valid_call_without_gpu_reports_hip_error(fwpkm_lib, handle):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = fwd(fwpkm_lib, handle, past=state(PK1, PK2, PV, 0, 0), nxt=state(NK1, NK2, NV))
    assert rc == _lib.ERR_HIP
    assert "hipGetDevice" in fwpkm_lib.fwpkm_last_error().decode()


# --------------------------------------------------- token-weighted entry
TW = 0xB0_0000_0000   # [batch, tokens, H] fp32 weights (fake address)


def fwd_w(lib, h, tw=TW, r=R, nxt=None, batch=2, tokens=64, lr=1.0):
    past = state(PK1, PK2, PV)
    nxt = nxt if nxt is not None else state(PK1, PK2, PV)
    return lib.fwpkm_forward_chunk_weighted(h, Q, Y, tw, batch, tokens, lr, ctypes.byref(past),
                                            ctypes.byref(nxt), r, None, None, None)


def test_weighted_entry_checks_like_the_plain_one(fwpkm_lib, handle):
    L = fwpkm_lib
    assert fwd_w(L, None) == _lib.ERR_INVALID_ARG
    assert fwd_w(L, handle, batch=3) == _lib.ERR_INVALID_ARG
    assert fwd_w(L, handle, lr=math.nan) == _lib.ERR_INVALID_ARG
    # the weights are an input: outputs and the next state must not overlap them
    # (2 sequences x 64 tokens x 1 head = 128 floats)
    assert fwd_w(L, handle, r=TW + 4 * 100) == _lib.ERR_ALIAS
    assert fwd_w(L, handle, nxt=state(NK1, NK2, TW)) == _lib.ERR_ALIAS
    # just past the weights' end is fine (fails later, for want of a device)
    import torch
    if not torch.cuda.is_available():
        assert fwd_w(L, handle, r=TW + 4 * 2 * 64) == _lib.ERR_HIP
        assert fwd_w(L, handle, tw=None) == _lib.ERR_HIP      # NULL = all weights 1


def test_addressing_workspace_only_when_enabled(fwpkm_lib):
    """The [units, 2, tokens, n] score buffer and the key gradients are
    allocated only with a non-zero addressing weight."""
    off = fwpkm_lib.fwpkm_workspace_bytes(ctypes.byref(cfg()))
    on = fwpkm_lib.fwpkm_workspace_bytes(ctypes.byref(cfg(addr_weight=0.1)))
    units, tokens, n, half = 2, 64, 32, 32
    assert on - off >= 4 * units * 2 * (tokens * n + n * half)


# ------------------------------------------------------- sequence entry
# cfg(): n 32, d_qk 64, d_v 64, k 4, chunk 64, one head, max_batch 2: D = 64
X, WIN, WG, BG = 0xC0_0000_0000, 0xC8_0000_0000, 0xD0_0000_0000, 0xD8_0000_0000
OUT, WS = 0xE0_0000_0000, 0xF0_0000_0000


def seq_ws(lib, batch=2, seq=100, **kw):
    return lib.fwpkm_sequence_workspace_bytes(ctypes.byref(cfg(**kw)), batch, seq)


def fwd_s(lib, h, x=X, out=OUT, ws=WS, ws_bytes=None, batch=2, seq=100, lr=1.0, nxt=None,
          slots=None, w=None, b_gate=BG):
    past = state(PK1, PK2, PV)
    nxt = nxt if nxt is not None else state(PK1, PK2, PV)
    ws_bytes = seq_ws(lib, batch if 1 <= batch <= 2 else 2, max(seq, 1)) if ws_bytes is None else ws_bytes
    return lib.fwpkm_forward_sequence(h, x, WIN, WG, b_gate, batch, seq, lr, ctypes.byref(past),
                                      ctypes.byref(nxt), out, slots, w, ws, ws_bytes, None)


def test_sequence_workspace_bytes(fwpkm_lib):
    L = fwpkm_lib
    # queries and targets of every token, plus the last chunk's weights
    need = seq_ws(L, 2, 100)
    assert need >= 4 * 2 * 100 * (64 + 64) + 4 * 2 * 64
    assert seq_ws(L, 2, 200) > need
    assert seq_ws(L, 0, 100) == 0 and seq_ws(L, 2, 0) == 0
    assert L.fwpkm_sequence_workspace_bytes(ctypes.byref(cfg(sqrt_slots=0)), 2, 10) == 0


def test_sequence_argument_errors(fwpkm_lib, handle):
    L = fwpkm_lib
    E = _lib.ERR_INVALID_ARG
    assert fwd_s(L, None) == E
    assert fwd_s(L, handle, x=None) == E
    assert fwd_s(L, handle, out=None) == E
    assert fwd_s(L, handle, ws=None) == E
    assert fwd_s(L, handle, batch=3) == E
    assert fwd_s(L, handle, seq=0) == E
    assert fwd_s(L, handle, lr=math.nan) == E
    assert fwd_s(L, handle, ws_bytes=seq_ws(L) - 1) == E
    assert "workspace" in L.fwpkm_last_error().decode()


def test_sequence_alias_errors(fwpkm_lib, handle):
    L = fwpkm_lib
    A = _lib.ERR_ALIAS
    assert fwd_s(L, handle, out=X + 4 * 64) == A                  # out over x
    assert fwd_s(L, handle, out=WIN + 4) == A                     # out over the projection
    assert fwd_s(L, handle, ws=X + 4 * 8) == A                    # workspace over x
    assert fwd_s(L, handle, ws=PV + 4 * 1024) == A                # workspace over the state
    assert fwd_s(L, handle, out=WS + 4 * 64) == A                 # out over the workspace
    assert fwd_s(L, handle, nxt=state(NK1, NK2, X)) == A          # next state over x
    assert fwd_s(L, handle, slots=BG) == A                        # selections over the gate bias
    # everything apart: passes validation, then needs the device
    import torch
    if not torch.cuda.is_available():
        assert fwd_s(L, handle) == _lib.ERR_HIP
        assert fwd_s(L, handle, b_gate=None) == _lib.ERR_HIP


def test_library_leaves_no_kernel_symbol_undefined():
    """Every kernel the launchers reference is defined in the library (a shared
    object links with undefined symbols and would only fail when loaded)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    assert "fwpkm" not in out, out


def test_checked_build_exports_the_same_abi():
    """libfwpkm_checked.so (device checks compiled in) declares itself and
    exports every symbol of the header; the product library reports 0."""
    from sparse_weight_memory_amd import build as B
    if not os.path.exists(_lib.CHECKED_LIB_PATH):
        B.build(checked=True)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.CHECKED_LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fwpkm_\w+)", out))
    assert set(declared_functions()) <= exported
    code = ("import ctypes, sys; lib = ctypes.CDLL(sys.argv[1]); "
            "lib.fwpkm_checked_build.restype = ctypes.c_int32; print(lib.fwpkm_checked_build())")
    for path, want in ((_lib.CHECKED_LIB_PATH, "1"), (_lib.LIB_PATH, "0")):
        r = subprocess.run(["python3", "-c", code, path], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        assert r.stdout.strip().splitlines()[-1] == want
