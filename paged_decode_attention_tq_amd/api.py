"""Python entry points over the C ABI (same names as include/tq.h).

PyTorch supplies device memory and the current HIP stream; every step of
the write, the readback and the decode runs in the HIP kernels of ``libtq.so``.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import TQError, check

__all__ = [
    "TQError",
    "row_bytes",
    "codebook",
    "rht_signs",
    "Context",
    "write_kv",
    "write_kv_pair",
    "prod_row_bytes",
    "write_kv_prod",
    "prod_scores_workspace_bytes",
    "prod_scores",
    "decompress_kv",
    "decode_workspace_bytes",
    "decode_kernel",
    "paged_decode",
    "hybrid_workspace_bytes",
    "paged_decode_hybrid",
    "prefill_workspace_bytes",
    "paged_prefill",
    "paged_decode_noalloc",
    "paged_decode_append",
]

_DTYPES = {torch.float32: _lib.TQ_F32, torch.float16: _lib.TQ_F16, torch.bfloat16: _lib.TQ_BF16}


def row_bytes(head_dim: int, bits: int) -> int:
    return int(_lib.lib().tq_row_bytes(head_dim, bits))


def codebook(head_dim: int, bits: int):
    """(centroids[2^b], boundaries[2^b - 1]) as float32 numpy arrays (host solver)."""
    n = 1 << bits
    c = np.zeros(n, np.float32)
    t = np.zeros(n - 1, np.float32)
    check(_lib.lib().tq_codebook(head_dim, bits, c.ctypes.data, t.ctypes.data), "tq_codebook")
    return c, t


def rht_signs(seed: int, head_dim: int) -> np.ndarray:
    s = np.zeros(head_dim, np.int8)
    check(_lib.lib().tq_rht_signs(seed, head_dim, s.ctypes.data), "tq_rht_signs")
    return s


class Context:
    """Rotation signs and codebooks for one head_dim and seed (host memory only)."""

    def __init__(self, head_dim: int = 128, seed: int = 42):
        self.head_dim = int(head_dim)
        self.seed = int(seed)
        h = ctypes.c_void_p()
        check(_lib.lib().tq_ctx_create(self.head_dim, self.seed, ctypes.byref(h)), "tq_ctx_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _lib.lib().tq_ctx_destroy(h)
            except Exception:
                pass
            self._h = None


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def write_kv(ctx: Context, raw: torch.Tensor, pages: torch.Tensor, slots: torch.Tensor, bits: int,
             err_count: torch.Tensor | None = None, check_slots: bool = True) -> int:
    """Encode ``raw[N, Hkv, d]`` into ``pages[NB, BS, Hkv, RB]`` at ``slots[N]``.

    Negative slots are skipped.  Out-of-range slots are skipped and counted;
    with ``check_slots`` the call synchronises and raises ``TQError`` if any
    were found.  Returns the number of out-of-range slots when checked.
    """
    _need(raw.is_cuda and pages.is_cuda and slots.is_cuda, "tensors must be on the GPU")
    _need(raw.dim() == 3 and raw.shape[2] == ctx.head_dim and raw.is_contiguous(), "raw must be [N, Hkv, d]")
    _need(pages.dtype == torch.uint8 and pages.dim() == 4 and pages.is_contiguous(), "pages must be uint8 4-D")
    NB, BS, Hkv, RB = pages.shape
    _need(raw.shape[1] == Hkv, "num_kv_heads mismatch")
    _need(RB == row_bytes(ctx.head_dim, bits), "pages row_bytes does not match bits")
    _need(slots.dtype == torch.int64 and slots.shape == (raw.shape[0],) and slots.is_contiguous(),
          "slots must be int64 [N]")
    _need(raw.dtype in _DTYPES, "raw dtype must be fp32/fp16/bf16")
    own = err_count is None and check_slots
    if own:
        err_count = torch.zeros(1, dtype=torch.int32, device=raw.device)
    st = _lib.lib().tq_write_kv(
        ctx.handle, raw.data_ptr(), _DTYPES[raw.dtype], raw.shape[0], Hkv, pages.data_ptr(), NB, BS,
        slots.data_ptr(), bits, err_count.data_ptr() if err_count is not None else None, _stream(raw))
    check(st, "tq_write_kv")
    if check_slots:
        n_bad = int(err_count.item())
        if n_bad:
            raise TQError(f"tq_write_kv: {n_bad} slot(s) outside the allocated pages")
        return n_bad
    return 0


def write_kv_pair(ctx: Context, raw_k: torch.Tensor, raw_v: torch.Tensor, k_pages: torch.Tensor,
                  v_pages: torch.Tensor, slots: torch.Tensor, k_bits: int, v_bits: int,
                  err_count: torch.Tensor | None = None, check_slots: bool = True) -> int:
    """``write_kv`` for K and for V of the same tokens, in one launch."""
    _need(raw_k.is_cuda and raw_v.is_cuda and k_pages.is_cuda and v_pages.is_cuda and slots.is_cuda,
          "tensors must be on the GPU")
    _need(raw_k.shape == raw_v.shape and raw_k.dtype == raw_v.dtype, "raw_k / raw_v shape or dtype mismatch")
    _need(raw_k.dim() == 3 and raw_k.shape[2] == ctx.head_dim and raw_k.is_contiguous() and raw_v.is_contiguous(),
          "raw must be [N, Hkv, d]")
    for name, pg, bits in (("k_pages", k_pages, k_bits), ("v_pages", v_pages, v_bits)):
        _need(pg.dtype == torch.uint8 and pg.dim() == 4 and pg.is_contiguous(), f"{name} must be uint8 4-D")
        _need(pg.shape[3] == row_bytes(ctx.head_dim, bits), f"{name} row_bytes does not match bits")
    NB, BS, Hkv, _ = k_pages.shape
    _need(tuple(v_pages.shape[:3]) == (NB, BS, Hkv), "k_pages / v_pages geometry mismatch")
    _need(raw_k.shape[1] == Hkv, "num_kv_heads mismatch")
    _need(slots.dtype == torch.int64 and slots.shape == (raw_k.shape[0],) and slots.is_contiguous(),
          "slots must be int64 [N]")
    _need(raw_k.dtype in _DTYPES, "raw dtype must be fp32/fp16/bf16")
    own = err_count is None and check_slots
    if own:
        err_count = torch.zeros(1, dtype=torch.int32, device=raw_k.device)
    st = _lib.lib().tq_write_kv_pair(
        ctx.handle, raw_k.data_ptr(), raw_v.data_ptr(), _DTYPES[raw_k.dtype], raw_k.shape[0], Hkv,
        k_pages.data_ptr(), k_bits, v_pages.data_ptr(), v_bits, NB, BS, slots.data_ptr(),
        err_count.data_ptr() if err_count is not None else None, _stream(raw_k))
    check(st, "tq_write_kv_pair")
    if check_slots:
        n_bad = int(err_count.item())
        if n_bad:
            raise TQError(f"tq_write_kv_pair: {n_bad} slot(s) outside the allocated pages")
        return n_bad
    return 0


def prod_row_bytes(head_dim: int, bits: int) -> int:
    return int(_lib.lib().tq_prod_row_bytes(head_dim, bits))


def write_kv_prod(ctx: Context, raw: torch.Tensor, pages: torch.Tensor, slots: torch.Tensor, bits: int,
                  sketch: torch.Tensor, err_count: torch.Tensor | None = None, check_slots: bool = True) -> int:
    """Encode ``raw[N, Hkv, d]`` into prod key rows of ``pages[NB, BS, Hkv, RB]`` at
    ``slots[N]`` with the sketch matrix ``sketch`` (fp32 ``[d, d]``).  Slot rules as ``write_kv``."""
    _need(raw.is_cuda and pages.is_cuda and slots.is_cuda and sketch.is_cuda, "tensors must be on the GPU")
    _need(raw.dim() == 3 and raw.shape[2] == ctx.head_dim and raw.is_contiguous(), "raw must be [N, Hkv, d]")
    _need(pages.dtype == torch.uint8 and pages.dim() == 4 and pages.is_contiguous(), "pages must be uint8 4-D")
    NB, BS, Hkv, RB = pages.shape
    _need(raw.shape[1] == Hkv, "num_kv_heads mismatch")
    _need(RB == prod_row_bytes(ctx.head_dim, bits), "pages row_bytes does not match bits")
    _need(slots.dtype == torch.int64 and slots.shape == (raw.shape[0],) and slots.is_contiguous(),
          "slots must be int64 [N]")
    _need(raw.dtype in _DTYPES, "raw dtype must be fp32/fp16/bf16")
    _need(sketch.dtype == torch.float32 and sketch.shape == (ctx.head_dim, ctx.head_dim) and sketch.is_contiguous(),
          "sketch must be fp32 [d, d]")
    own = err_count is None and check_slots
    if own:
        err_count = torch.zeros(1, dtype=torch.int32, device=raw.device)
    st = _lib.lib().tq_write_kv_prod(
        ctx.handle, raw.data_ptr(), _DTYPES[raw.dtype], raw.shape[0], Hkv, pages.data_ptr(), NB, BS,
        slots.data_ptr(), bits, sketch.data_ptr(), err_count.data_ptr() if err_count is not None else None,
        _stream(raw))
    check(st, "tq_write_kv_prod")
    if check_slots:
        n_bad = int(err_count.item())
        if n_bad:
            raise TQError(f"tq_write_kv_prod: {n_bad} slot(s) outside the allocated pages")
        return n_bad
    return 0


def prod_scores_workspace_bytes(batch: int, num_q_heads: int) -> int:
    """Bytes of device workspace ``prod_scores`` needs (rotated queries and their sketches)."""
    return int(_lib.lib().tq_prod_scores_workspace_bytes(batch, num_q_heads))


def prod_scores(ctx: Context, q: torch.Tensor, pages: torch.Tensor, block_table: torch.Tensor,
                seq_lens: torch.Tensor, bits: int, sketch: torch.Tensor, max_seq_len: int | None = None,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Estimated ``<q[b, h], k_t>`` over prod key pages -> fp32 ``[B, Hq, max_seq_len]``."""
    _need(q.is_cuda and q.dim() == 3 and q.shape[2] == ctx.head_dim and q.is_contiguous(), "q must be [B, Hq, d]")
    _need(q.dtype in _DTYPES, "q dtype must be fp32/fp16/bf16")
    B, Hq, d = q.shape
    _need(pages.dtype == torch.uint8 and pages.dim() == 4 and pages.is_contiguous(), "pages must be uint8 4-D")
    NB, BS, Hkv, RB = pages.shape
    _need(RB == prod_row_bytes(d, bits), "pages row_bytes does not match bits")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B
          and block_table.is_contiguous(), "block_table must be int32 [B, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    _need(sketch.dtype == torch.float32 and sketch.shape == (d, d) and sketch.is_contiguous(),
          "sketch must be fp32 [d, d]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty((B, Hq, max_seq_len), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.shape == (B, Hq, max_seq_len) and out.is_contiguous(),
          "out must be fp32 [B, Hq, max_seq_len]")
    need = prod_scores_workspace_bytes(B, Hq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = _lib.lib().tq_prod_scores(
        ctx.handle, q.data_ptr(), _DTYPES[q.dtype], B, Hq, Hkv, pages.data_ptr(), bits, NB, BS,
        block_table.data_ptr(), block_table.shape[1], seq_lens.data_ptr(), max_seq_len, sketch.data_ptr(),
        out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    check(st, "tq_prod_scores")
    return out


def decompress_kv(ctx: Context, pages: torch.Tensor, slots: torch.Tensor, bits: int,
                  out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.float32,
                  err_count: torch.Tensor | None = None, check_slots: bool = True) -> torch.Tensor:
    """Dense rows ``[N, Hkv, d]`` read back from ``pages[NB, BS, Hkv, RB]`` at ``slots[N]``.

    Negative slots give zero rows.  Out-of-range slots give zero rows and are
    counted; with ``check_slots`` the call synchronises and raises
    ``TQError`` if any were found.
    """
    _need(pages.is_cuda and slots.is_cuda, "tensors must be on the GPU")
    _need(pages.dtype == torch.uint8 and pages.dim() == 4 and pages.is_contiguous(), "pages must be uint8 4-D")
    NB, BS, Hkv, RB = pages.shape
    _need(RB == row_bytes(ctx.head_dim, bits), "pages row_bytes does not match bits")
    _need(slots.dtype == torch.int64 and slots.dim() == 1 and slots.is_contiguous(), "slots must be int64 [N]")
    N = slots.shape[0]
    if out is None:
        out = torch.empty((N, Hkv, ctx.head_dim), dtype=out_dtype, device=pages.device)
    _need(out.dtype in _DTYPES and out.shape == (N, Hkv, ctx.head_dim) and out.is_contiguous(),
          "out must be fp32/fp16/bf16 [N, Hkv, d]")
    own = err_count is None and check_slots
    if own:
        err_count = torch.zeros(1, dtype=torch.int32, device=pages.device)
    st = _lib.lib().tq_decompress_kv(
        ctx.handle, pages.data_ptr(), NB, BS, Hkv, bits, slots.data_ptr(), N, out.data_ptr(), _DTYPES[out.dtype],
        err_count.data_ptr() if err_count is not None else None, _stream(pages))
    check(st, "tq_decompress_kv")
    if check_slots:
        n_bad = int(err_count.item())
        if n_bad:
            raise TQError(f"tq_decompress_kv: {n_bad} slot(s) outside the allocated pages")
    return out


def decode_workspace_bytes(ctx: Context, batch, num_q_heads, num_kv_heads, max_seq_len, block_size=16) -> int:
    return int(_lib.lib().tq_decode_workspace_bytes(ctx.handle, batch, num_q_heads, num_kv_heads,
                                                    max_seq_len, block_size))


def decode_kernel(batch, num_q_heads, num_kv_heads, max_seq_len, k_bits, v_bits) -> str | None:
    """'wave', 'wave1' (the wave kernel as one workgroup, no merge kernel) or 'staged': the decode
    kernel these sizes run on the current device (None: unsupported)."""
    name = _lib.lib().tq_decode_kernel(batch, num_q_heads, num_kv_heads, max_seq_len, k_bits, v_bits)
    return name.decode() if name else None


def paged_decode(ctx: Context, q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                 block_table: torch.Tensor, seq_lens: torch.Tensor, k_bits: int, v_bits: int,
                 max_seq_len: int | None = None, scale: float | None = None,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Single-query paged decode -> fp32 ``[B, Hq, d]``.

    ``max_seq_len`` defaults to ``seq_lens.max()`` (a device-to-host sync).
    """
    _need(q.is_cuda and q.dim() == 3 and q.shape[2] == ctx.head_dim and q.is_contiguous(), "q must be [B, Hq, d]")
    _need(q.dtype in _DTYPES, "q dtype must be fp32/fp16/bf16")
    B, Hq, d = q.shape
    for name, pg, bits in (("k_pages", k_pages, k_bits), ("v_pages", v_pages, v_bits)):
        _need(pg.dtype == torch.uint8 and pg.dim() == 4 and pg.is_contiguous(), f"{name} must be uint8 4-D")
        _need(pg.shape[3] == row_bytes(d, bits), f"{name} row_bytes does not match bits")
    NB, BS, Hkv, _ = k_pages.shape
    _need(tuple(v_pages.shape[:3]) == (NB, BS, Hkv), "k_pages / v_pages geometry mismatch")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B
          and block_table.is_contiguous(), "block_table must be int32 [B, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.shape == (B, Hq, d) and out.is_contiguous(), "out must be fp32 [B, Hq, d]")
    need = decode_workspace_bytes(ctx, B, Hq, Hkv, max_seq_len, BS)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = _lib.lib().tq_paged_decode(
        ctx.handle, q.data_ptr(), _DTYPES[q.dtype], B, Hq, Hkv, k_pages.data_ptr(), k_bits,
        v_pages.data_ptr(), v_bits, NB, BS, block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), max_seq_len, float(scale) if scale else 0.0, out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    check(st, "tq_paged_decode")
    return out


def paged_decode_append(ctx: Context, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                        seq_lens: torch.Tensor, k_bits: int, v_bits: int, max_seq_len: int | None = None,
                        scale: float | None = None, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, err_count: torch.Tensor | None = None,
                        check_pages: bool = True) -> torch.Tensor:
    """One decode step in one call: the new rows ``k_new``/``v_new`` ``[B, Hkv, d]``
    are written at each sequence's last token (position ``seq_lens[b] - 1``)
    and the decode attends over every token -> fp32 ``[B, Hq, d]``.

    Equal bit for bit to ``write_kv_pair`` at those slots followed by
    ``paged_decode``.  A sequence whose last page has a block id outside the
    pages is counted in ``err_count`` and its rows are not written; with
    ``check_pages`` the call synchronises and raises ``TQError`` if any were.
    """
    _need(q.is_cuda and q.dim() == 3 and q.shape[2] == ctx.head_dim and q.is_contiguous(), "q must be [B, Hq, d]")
    _need(q.dtype in _DTYPES, "q dtype must be fp32/fp16/bf16")
    B, Hq, d = q.shape
    for name, pg, bits in (("k_pages", k_pages, k_bits), ("v_pages", v_pages, v_bits)):
        _need(pg.dtype == torch.uint8 and pg.dim() == 4 and pg.is_contiguous(), f"{name} must be uint8 4-D")
        _need(pg.shape[3] == row_bytes(d, bits), f"{name} row_bytes does not match bits")
    NB, BS, Hkv, _ = k_pages.shape
    _need(tuple(v_pages.shape[:3]) == (NB, BS, Hkv), "k_pages / v_pages geometry mismatch")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t.is_cuda and t.shape == (B, Hkv, d) and t.is_contiguous(), f"{name} must be [B, Hkv, d]")
    _need(k_new.dtype == v_new.dtype and k_new.dtype in _DTYPES, "k_new / v_new must share an fp32/fp16/bf16 dtype")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B
          and block_table.is_contiguous(), "block_table must be int32 [B, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.shape == (B, Hq, d) and out.is_contiguous(), "out must be fp32 [B, Hq, d]")
    need = decode_workspace_bytes(ctx, B, Hq, Hkv, max_seq_len, BS)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    own = err_count is None and check_pages
    if own:
        err_count = torch.zeros(1, dtype=torch.int32, device=q.device)
    st = _lib.lib().tq_paged_decode_append(
        ctx.handle, q.data_ptr(), _DTYPES[q.dtype], B, Hq, Hkv, k_new.data_ptr(), v_new.data_ptr(),
        _DTYPES[k_new.dtype], k_pages.data_ptr(), k_bits, v_pages.data_ptr(), v_bits, NB, BS,
        block_table.data_ptr(), block_table.shape[1], seq_lens.data_ptr(), max_seq_len,
        float(scale) if scale else 0.0, out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), err_count.data_ptr() if err_count is not None else None,
        _stream(q))
    check(st, "tq_paged_decode_append")
    if check_pages:
        n_bad = int(err_count.item())
        if n_bad:
            raise TQError(f"tq_paged_decode_append: {n_bad} sequence(s) whose last page is outside the pages")
    return out


def hybrid_workspace_bytes(ctx: Context, batch, num_q_heads, num_kv_heads, max_seq_len, block_size=16) -> int:
    return int(_lib.lib().tq_hybrid_workspace_bytes(ctx.handle, batch, num_q_heads, num_kv_heads,
                                                    max_seq_len, block_size))


def paged_decode_hybrid(ctx: Context, q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                        block_table: torch.Tensor, seq_lens: torch.Tensor, recent_k: torch.Tensor,
                        recent_v: torch.Tensor, recent_lens: torch.Tensor, k_bits: int, v_bits: int,
                        max_seq_len: int | None = None, scale: float | None = None,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode over packed history plus the exact recent window -> fp32 ``[B, Hq, d]``.

    ``recent_k`` / ``recent_v``: ``[B, cap, Hkv, d]`` fp32/fp16/bf16;
    ``recent_lens``: int32 ``[B]`` (rows used per sequence).
    """
    _need(q.is_cuda and q.dim() == 3 and q.shape[2] == ctx.head_dim and q.is_contiguous(), "q must be [B, Hq, d]")
    _need(q.dtype in _DTYPES, "q dtype must be fp32/fp16/bf16")
    B, Hq, d = q.shape
    for name, pg, bits in (("k_pages", k_pages, k_bits), ("v_pages", v_pages, v_bits)):
        _need(pg.dtype == torch.uint8 and pg.dim() == 4 and pg.is_contiguous(), f"{name} must be uint8 4-D")
        _need(pg.shape[3] == row_bytes(d, bits), f"{name} row_bytes does not match bits")
    NB, BS, Hkv, _ = k_pages.shape
    _need(tuple(v_pages.shape[:3]) == (NB, BS, Hkv), "k_pages / v_pages geometry mismatch")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B
          and block_table.is_contiguous(), "block_table must be int32 [B, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    _need(recent_k.is_cuda and recent_v.is_cuda and recent_lens.is_cuda, "tensors must be on the GPU")
    _need(recent_k.dim() == 4 and recent_k.shape[0] == B and tuple(recent_k.shape[2:]) == (Hkv, d)
          and recent_k.is_contiguous(), "recent_k must be [B, cap, Hkv, d]")
    _need(recent_v.shape == recent_k.shape and recent_v.dtype == recent_k.dtype and recent_v.is_contiguous(),
          "recent_v must match recent_k")
    _need(recent_k.dtype in _DTYPES, "recent dtype must be fp32/fp16/bf16")
    _need(recent_lens.dtype == torch.int32 and recent_lens.shape == (B,), "recent_lens must be int32 [B]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.shape == (B, Hq, d) and out.is_contiguous(), "out must be fp32 [B, Hq, d]")
    need = hybrid_workspace_bytes(ctx, B, Hq, Hkv, max_seq_len, BS)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = _lib.lib().tq_paged_decode_hybrid(
        ctx.handle, q.data_ptr(), _DTYPES[q.dtype], B, Hq, Hkv, k_pages.data_ptr(), k_bits,
        v_pages.data_ptr(), v_bits, NB, BS, block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), max_seq_len, recent_k.data_ptr(), recent_v.data_ptr(), _DTYPES[recent_k.dtype],
        recent_k.shape[1], recent_lens.data_ptr(), float(scale) if scale else 0.0, out.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    check(st, "tq_paged_decode_hybrid")
    return out


def prefill_workspace_bytes(ctx: Context, batch, q_len, num_q_heads, num_kv_heads, max_seq_len,
                            block_size=16) -> int:
    return int(_lib.lib().tq_prefill_workspace_bytes(ctx.handle, batch, q_len, num_q_heads, num_kv_heads,
                                                     max_seq_len, block_size))


def paged_prefill(ctx: Context, q: torch.Tensor, q_lens: torch.Tensor, k_pages: torch.Tensor,
                  v_pages: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, k_bits: int,
                  v_bits: int, max_seq_len: int | None = None, scale: float | None = None,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Multi-query attention, causal within each sequence's last ``q_lens[b]``
    tokens -> fp32 ``[B, Lq, Hq, d]`` (rows past ``q_lens[b]`` are zeros).

    ``q``: ``[B, Lq, Hq, d]`` fp32/fp16/bf16; ``q_lens``: int32 ``[B]``.
    """
    _need(q.is_cuda and q.dim() == 4 and q.shape[3] == ctx.head_dim and q.is_contiguous(),
          "q must be [B, Lq, Hq, d]")
    _need(q.dtype in _DTYPES, "q dtype must be fp32/fp16/bf16")
    B, Lq, Hq, d = q.shape
    for name, pg, bits in (("k_pages", k_pages, k_bits), ("v_pages", v_pages, v_bits)):
        _need(pg.dtype == torch.uint8 and pg.dim() == 4 and pg.is_contiguous(), f"{name} must be uint8 4-D")
        _need(pg.shape[3] == row_bytes(d, bits), f"{name} row_bytes does not match bits")
    NB, BS, Hkv, _ = k_pages.shape
    _need(tuple(v_pages.shape[:3]) == (NB, BS, Hkv), "k_pages / v_pages geometry mismatch")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B
          and block_table.is_contiguous(), "block_table must be int32 [B, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    _need(q_lens.is_cuda and q_lens.dtype == torch.int32 and q_lens.shape == (B,), "q_lens must be int32 [B]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty((B, Lq, Hq, d), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.shape == (B, Lq, Hq, d) and out.is_contiguous(),
          "out must be fp32 [B, Lq, Hq, d]")
    need = prefill_workspace_bytes(ctx, B, Lq, Hq, Hkv, max_seq_len, BS)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = _lib.lib().tq_paged_prefill(
        ctx.handle, q.data_ptr(), _DTYPES[q.dtype], B, Lq, q_lens.data_ptr(), Hq, Hkv, k_pages.data_ptr(), k_bits,
        v_pages.data_ptr(), v_bits, NB, BS, block_table.data_ptr(), block_table.shape[1], seq_lens.data_ptr(),
        max_seq_len, float(scale) if scale else 0.0, out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(q))
    check(st, "tq_paged_prefill")
    return out


def paged_decode_noalloc(ctx: Context, q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                         block_table: torch.Tensor, seq_lens: torch.Tensor, k_bits: int, v_bits: int,
                         max_seq_len: int | None = None, scale: float | None = None,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """``paged_decode`` without a workspace: the library's static scratch holds
    the split partials (nothing is allocated when ``out`` is given)."""
    _need(q.is_cuda and q.dim() == 3 and q.shape[2] == ctx.head_dim and q.is_contiguous(), "q must be [B, Hq, d]")
    _need(q.dtype in _DTYPES, "q dtype must be fp32/fp16/bf16")
    B, Hq, d = q.shape
    for name, pg, bits in (("k_pages", k_pages, k_bits), ("v_pages", v_pages, v_bits)):
        _need(pg.dtype == torch.uint8 and pg.dim() == 4 and pg.is_contiguous(), f"{name} must be uint8 4-D")
        _need(pg.shape[3] == row_bytes(d, bits), f"{name} row_bytes does not match bits")
    NB, BS, Hkv, _ = k_pages.shape
    _need(tuple(v_pages.shape[:3]) == (NB, BS, Hkv), "k_pages / v_pages geometry mismatch")
    _need(block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.shape[0] == B
          and block_table.is_contiguous(), "block_table must be int32 [B, max_blocks]")
    _need(seq_lens.dtype == torch.int32 and seq_lens.shape == (B,), "seq_lens must be int32 [B]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _need(out.dtype == torch.float32 and out.shape == (B, Hq, d) and out.is_contiguous(), "out must be fp32 [B, Hq, d]")
    st = _lib.lib().tq_paged_decode_noalloc(
        ctx.handle, q.data_ptr(), _DTYPES[q.dtype], B, Hq, Hkv, k_pages.data_ptr(), k_bits,
        v_pages.data_ptr(), v_bits, NB, BS, block_table.data_ptr(), block_table.shape[1],
        seq_lens.data_ptr(), max_seq_len, float(scale) if scale else 0.0, out.data_ptr(), _stream(q))
    check(st, "tq_paged_decode_noalloc")
    return out
