"""Python binding of the FwPKM chunk step (argument marshalling only).

    mem = Memory(Config(sqrt_slots=256, dim_qk=512, dim_v=512, topk=8,
                        chunk_size=256, max_batch=2))
    retrieved, next_state = mem.forward_chunk(queries, targets, lr, past_state)

mirrors the chained ``mem(tokens, past_memories=...) -> (retrieved,
next_memories)`` usage on the PyPI page "fast-weight-product-key-memory",
with queries and targets passed in directly.  Every step of the computation
runs in the HIP library; torch provides device memory and the stream.
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import NamedTuple, Optional

import torch

from . import _lib


class FwPKMError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"fwpkm error {code}: {message}")
        self.code = code


@dataclasses.dataclass(frozen=True)
class Config:
    sqrt_slots: int
    dim_qk: int
    dim_v: int
    topk: int
    chunk_size: int
    num_heads: int = 1
    max_batch: int = 1
    eps: float = 1e-3
    score_mode: str = "idw"      # "idw" or "dot"
    addr_weight: float = 0.0     # lambda of the marginal-entropy addressing loss (0: off)

    @property
    def num_slots(self) -> int:
        return self.sqrt_slots * self.sqrt_slots

    @property
    def half(self) -> int:
        return self.dim_qk // 2

    def to_c(self) -> _lib.CConfig:
        mode = {"idw": _lib.SCORE_IDW, "dot": _lib.SCORE_DOT}.get(self.score_mode, -1)
        return _lib.CConfig(self.sqrt_slots, self.dim_qk, self.dim_v, self.topk,
                            self.chunk_size, self.num_heads, self.max_batch,
                            float(self.eps), mode, float(self.addr_weight))


class State(NamedTuple):
    """Fast weights on the GPU, fp32 contiguous.

    Per-sequence tables: k1, k2 [B, H, n, d_h], v [B, H, N, d_v].
    Shared tables (one set for the whole batch; past state only):
    k1, k2 [H, n, d_h], v [H, N, d_v].
    """
    k1: torch.Tensor
    k2: torch.Tensor
    v: torch.Tensor

    def clone(self) -> "State":
        return State(self.k1.clone(), self.k2.clone(), self.v.clone())


def _check_tensor(name, t, dtype=torch.float32):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def state_strides(shapes, cfg: Config, batch: int):
    """Element strides between sequences of a state whose tables have the
    given shapes (k1, k2, v), after checking that they hold what a call with
    `batch` sequences reads and writes:

      per-sequence  k1, k2 [B', H, n, d_h], v [B', H, N, d_v] with B' >= batch
                    (the same B' in all three) -> one sequence's tables apart;
      shared        k1, k2 [H, n, d_h], v [H, N, d_v] -> stride 0.

    Raises ValueError otherwise: the C library cannot see allocation sizes,
    so this is what keeps it inside the caller's tensors."""
    H, n, dh, N, dv = cfg.num_heads, cfg.sqrt_slots, cfg.half, cfg.num_slots, cfg.dim_v
    k1, k2, v = (tuple(int(d) for d in s) for s in shapes)
    if len(k1) == 3:
        if k1 != (H, n, dh) or k2 != (H, n, dh) or v != (H, N, dv):
            raise ValueError(f"shared state tables must be k1, k2 [{H}, {n}, {dh}] and "
                             f"v [{H}, {N}, {dv}]; got {k1}, {k2}, {v}")
        return 0, 0
    if len(k1) != 4 or k1[1:] != (H, n, dh) or k2[1:] != (H, n, dh) or len(v) != 4 or v[1:] != (H, N, dv):
        raise ValueError(f"per-sequence state tables must be k1, k2 [B, {H}, {n}, {dh}] and "
                         f"v [B, {H}, {N}, {dv}]; got {k1}, {k2}, {v}")
    if not (k1[0] == k2[0] == v[0]):
        raise ValueError(f"state tables hold different numbers of sequences: {k1[0]}, {k2[0]}, {v[0]}")
    if k1[0] < batch:
        raise ValueError(f"state tables hold {k1[0]} sequence(s), the call carries {batch}")
    return H * n * dh, H * N * dv


def _c_state(s: State, cfg: Config, batch: int) -> _lib.CState:
    for name, t in (("k1", s.k1), ("k2", s.k2), ("v", s.v)):
        _check_tensor(f"state.{name}", t)
    stride_k, stride_v = state_strides((s.k1.shape, s.k2.shape, s.v.shape), cfg, batch)
    return _lib.CState(s.k1.data_ptr(), s.k2.data_ptr(), s.v.data_ptr(), stride_k, stride_v)


def check_rows(name: str, shape, batch: int, rows: int, heads: int, width: int) -> None:
    """`name` must be [batch, rows, heads, width] (or [batch, rows, width]
    when heads == 1): a caller-supplied output the library writes in full."""
    shape = tuple(int(d) for d in shape)
    ok = shape == (batch, rows, heads, width) or (heads == 1 and shape == (batch, rows, width))
    if not ok:
        raise ValueError(f"{name} must be [{batch}, {rows}, {heads}, {width}], got {list(shape)}")


def empty_state(cfg: Config, batch: int, device="cuda") -> State:
    n, dh, N, dv, H = cfg.sqrt_slots, cfg.half, cfg.num_slots, cfg.dim_v, cfg.num_heads
    return State(torch.empty((batch, H, n, dh), device=device),
                 torch.empty((batch, H, n, dh), device=device),
                 torch.empty((batch, H, N, dv), device=device))


class Memory:
    """One handle of the C ABI: a configuration plus its device workspace."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self._lib = _lib.load()
        self._c_cfg = cfg.to_c()
        h = ctypes.c_void_p()
        rc = self._lib.fwpkm_create(ctypes.byref(self._c_cfg), ctypes.byref(h))
        if rc != _lib.OK:
            raise FwPKMError(rc, _lib.last_error())
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._lib.fwpkm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def profile(self, enable: bool = True) -> None:
        """Start (clearing totals) or stop per-kernel event timing."""
        rc = self._lib.fwpkm_profile_enable(self._h, 1 if enable else 0)
        if rc != _lib.OK:
            raise FwPKMError(rc, _lib.last_error())

    def profile_read(self) -> dict:
        """{kernel name: (total ms, launches)} of the timed launches so far."""
        ms = (ctypes.c_double * _lib.NUM_TIMED)()
        cnt = (ctypes.c_int64 * _lib.NUM_TIMED)()
        rc = self._lib.fwpkm_profile_read(self._h, ms, cnt)
        if rc != _lib.OK:
            raise FwPKMError(rc, _lib.last_error())
        return {self._lib.fwpkm_kernel_name(i).decode(): (ms[i], int(cnt[i]))
                for i in range(_lib.NUM_TIMED)}

    @property
    def workspace_bytes(self) -> int:
        return int(self._lib.fwpkm_workspace_bytes(ctypes.byref(self._c_cfg)))

    def forward_chunk(self, queries: torch.Tensor, targets: torch.Tensor, lr: float,
                      past: State, next: Optional[State] = None,
                      return_selection: bool = False, retrieved: Optional[torch.Tensor] = None,
                      token_weights: Optional[torch.Tensor] = None, noalloc: bool = False):
        """One chunk: (retrieved [B, T, H, d_v], next state) from past state.

        queries [B, T, H, d_qk] (or [B, T, d_qk] when H == 1), targets likewise
        with d_v.  next=None allocates per-sequence tables and fills them
        (functional update); next=past updates in place.  token_weights
        [B, T, H] (or [B, T] when H == 1) scales each token's loss; a weight
        of 0 reads without writing (fwpkm_forward_chunk_weighted).
        noalloc=True calls fwpkm_forward_chunk_noalloc, which works in the
        library's fixed device workspace and allocates nothing; to allocate
        nothing in this method either, pass next and retrieved and leave
        return_selection False.  It takes no token weights.
        """
        cfg = self.cfg
        _check_tensor("queries", queries)
        _check_tensor("targets", targets)
        B, T = queries.shape[0], queries.shape[1]
        if queries.numel() != B * T * cfg.num_heads * cfg.dim_qk:
            raise ValueError("queries must be [B, T, H, d_qk]")
        if targets.numel() != B * T * cfg.num_heads * cfg.dim_v or targets.shape[:2] != queries.shape[:2]:
            raise ValueError("targets must be [B, T, H, d_v]")
        if next is None:
            next = empty_state(cfg, B, queries.device)
        c_past = _c_state(past, cfg, B)
        c_next = _c_state(next, cfg, B)
        if retrieved is None:
            retrieved = torch.empty((B, T, cfg.num_heads, cfg.dim_v), device=queries.device)
        else:
            _check_tensor("retrieved", retrieved)
            check_rows("retrieved", retrieved.shape, B, T, cfg.num_heads, cfg.dim_v)
        slots = weights = None
        if return_selection:
            slots = torch.empty((B, T, cfg.num_heads, cfg.topk), device=queries.device, dtype=torch.int32)
            weights = torch.empty((B, T, cfg.num_heads, cfg.topk), device=queries.device)
        stream = torch.cuda.current_stream(queries.device).cuda_stream
        sel_ptrs = (slots.data_ptr() if slots is not None else None,
                    weights.data_ptr() if weights is not None else None)
        if noalloc:
            if token_weights is not None:
                raise ValueError("fwpkm_forward_chunk_noalloc takes no token weights")
            rc = self._lib.fwpkm_forward_chunk_noalloc(
                self._h, queries.data_ptr(), targets.data_ptr(), B, T, float(lr),
                ctypes.byref(c_past), ctypes.byref(c_next), retrieved.data_ptr(),
                *sel_ptrs, stream)
        elif token_weights is None:
            rc = self._lib.fwpkm_forward_chunk(
                self._h, queries.data_ptr(), targets.data_ptr(), B, T, float(lr),
                ctypes.byref(c_past), ctypes.byref(c_next), retrieved.data_ptr(),
                *sel_ptrs, stream)
        else:
            _check_tensor("token_weights", token_weights)
            if token_weights.numel() != B * T * cfg.num_heads or token_weights.shape[:2] != queries.shape[:2]:
                raise ValueError("token_weights must be [B, T, H]")
            rc = self._lib.fwpkm_forward_chunk_weighted(
                self._h, queries.data_ptr(), targets.data_ptr(), token_weights.data_ptr(),
                B, T, float(lr), ctypes.byref(c_past), ctypes.byref(c_next),
                retrieved.data_ptr(), *sel_ptrs, stream)
        if rc != _lib.OK:
            raise FwPKMError(rc, _lib.last_error())
        if return_selection:
            return retrieved, next, slots, weights
        return retrieved, next

    def sequence_workspace_bytes(self, batch: int, seq: int) -> int:
        n = int(self._lib.fwpkm_sequence_workspace_bytes(ctypes.byref(self._c_cfg), int(batch), int(seq)))
        if n == 0:
            raise FwPKMError(_lib.ERR_INVALID_ARG, _lib.last_error())
        return n

    def forward_sequence(self, x: torch.Tensor, w_in: torch.Tensor, w_gate: torch.Tensor,
                         b_gate: Optional[torch.Tensor], lr: float, past: State,
                         next: Optional[State] = None, out: Optional[torch.Tensor] = None,
                         return_selection: bool = False,
                         workspace: Optional[torch.Tensor] = None):
        """Whole sequences: (out [B, S, D], next state), D = H * d_v.

        x [B, S, D]; w_in [H*d_qk + H*d_v, D] (query rows of every head, then
        value rows); w_gate [H, D]; b_gate [H] or None.  Each token's target
        is the next token's value; the last token reads without writing; the
        sequence runs through the chunk step chunk_size tokens at a time and
        out = g * read + (1 - g) * x per head with g = sigmoid(w_gate x + b)
        (fwpkm_forward_sequence).  workspace: a device byte tensor of at least
        sequence_workspace_bytes(B, S) bytes, or None to allocate one.
        """
        cfg = self.cfg
        H = cfg.num_heads
        D = H * cfg.dim_v
        _check_tensor("x", x)
        _check_tensor("w_in", w_in)
        _check_tensor("w_gate", w_gate)
        if x.dim() != 3 or x.shape[2] != D:
            raise ValueError(f"x must be [B, S, {D}]")
        B, S = x.shape[0], x.shape[1]
        if tuple(w_in.shape) != (H * (cfg.dim_qk + cfg.dim_v), D):
            raise ValueError(f"w_in must be [{H * (cfg.dim_qk + cfg.dim_v)}, {D}]")
        if tuple(w_gate.shape) != (H, D):
            raise ValueError(f"w_gate must be [{H}, {D}]")
        if b_gate is not None:
            _check_tensor("b_gate", b_gate)
            if b_gate.numel() != H:
                raise ValueError(f"b_gate must have {H} entries")
        if next is None:
            next = empty_state(cfg, B, x.device)
        c_past = _c_state(past, cfg, B)
        c_next = _c_state(next, cfg, B)
        if out is None:
            out = torch.empty((B, S, D), device=x.device)
        else:
            _check_tensor("out", out)
            if tuple(out.shape) != (B, S, D):
                raise ValueError(f"out must be [{B}, {S}, {D}]")
        need = self.sequence_workspace_bytes(B, S)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        elif workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous device tensor of >= {need} bytes")
        slots = weights = None
        if return_selection:
            slots = torch.empty((B, S, H, cfg.topk), device=x.device, dtype=torch.int32)
            weights = torch.empty((B, S, H, cfg.topk), device=x.device)
        stream = torch.cuda.current_stream(x.device).cuda_stream
        rc = self._lib.fwpkm_forward_sequence(
            self._h, x.data_ptr(), w_in.data_ptr(), w_gate.data_ptr(),
            b_gate.data_ptr() if b_gate is not None else None, B, S, float(lr),
            ctypes.byref(c_past), ctypes.byref(c_next), out.data_ptr(),
            slots.data_ptr() if slots is not None else None,
            weights.data_ptr() if weights is not None else None,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
        if rc != _lib.OK:
            raise FwPKMError(rc, _lib.last_error())
        if return_selection:
            return out, next, slots, weights
        return out, next
