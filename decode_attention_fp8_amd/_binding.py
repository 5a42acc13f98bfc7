"""ctypes marshalling for libpkv.so (the C ABI declared in include/pkv.h).

Every function here only converts torch tensors to device pointers, reads
torch's current HIP stream, calls the library and raises on a bad status.
No step of the computation runs in Python: without the built library the
import fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EHIP = 0, -1, -2, -3
PKV_KV_E4M3, PKV_KV_BF16 = 1, 2

EXPORTS = ("pkv_scales_from_amax", "pkv_append", "pkv_verify", "pkv_verify_append",
           "pkv_decode_attn",
           "pkv_combine", "pkv_step_decode", "pkv_step_combine", "pkv_step_launches",
           "pkv_decode_attn_drafts", "pkv_requantize_pages", "pkv_int4_linear",
           "pkv_int4_linear_workspace", "pkv_fill_u32", "pkv_read_u32",
           "pkv_decode_attn_static",
           "pkv_suggest_split", "pkv_strerror", "pkv_version")


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({pkv_strerror(status)})")
        self.status = status


class PkvCacheStruct(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("dtype", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("page_tags", ctypes.c_void_p),
                ("k_row_scale", ctypes.c_void_p), ("v_row_scale", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python decode_attention_fp8_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    CP = ctypes.POINTER(PkvCacheStruct)
    sig = {
        "pkv_scales_from_amax": (I32, [P, I64, I32, I32, I32, P, P]),
        "pkv_append": (I32, [CP, P, P, P, P, P, I64, P]),
        "pkv_verify": (I32, [CP, P, P, P, I32, I32, P, P]),
        "pkv_verify_append": (I32, [CP, P, P, P, I32, I32, P, P, P, P, P]),
        "pkv_decode_attn": (I32, [CP, P, I32, P, P, I32, I32, I32, P, F, I32, I32, P, P, P]),
        "pkv_combine": (I32, [P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, P]),
        "pkv_step_decode": (I32, [CP, P, I32, P, P, P, P, P, I32, I32, I32, F, I32, I32, P, P, P,
                                  P, P]),
        "pkv_step_combine": (I32, [CP, I32, P, P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, P,
                                   P, P]),
        "pkv_step_launches": (I32, [CP, I32, I32]),
        "pkv_decode_attn_drafts": (I32, [CP, P, I32, I32, P, P, I32, I32, I32, P, F, I32, I32, P,
                                         P, P]),
        "pkv_requantize_pages": (I32, [CP, CP, P, P, P, P, I32, P]),
        "pkv_int4_linear": (I32, [P, P, P, I32, I32, I32, P, P, P]),
        "pkv_int4_linear_workspace": (I64, [I32, I32, I32]),
        "pkv_fill_u32": (I32, [P, I64, ctypes.c_uint32, P]),
        "pkv_read_u32": (I32, [P, I64, P, P]),
        "pkv_decode_attn_static": (I32, [CP, P, I32, P, P, I32, I32, I32, P, F, I32, P, P, P]),
        "pkv_suggest_split": (I32, [CP, I32, I32, I64, I32]),
        "pkv_strerror": (ctypes.c_char_p, [I32]),
        "pkv_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def pkv_strerror(status: int) -> str:
    return _lib.pkv_strerror(int(status)).decode()


def pkv_version() -> int:
    return int(_lib.pkv_version())


def pkv_suggest_split(cache: Cache, num_q_heads: int, batch: int, total_tokens: int,
                      max_seq_len: int) -> int:
    # only the geometry is read; v_pool's NULL-ness marks the latent layout
    cs = PkvCacheStruct(None, None if cache.v_pool is None else 1, cache.dtype, cache.num_pages,
                        cache.page_size, cache.num_kv_heads, cache.head_dim_k, cache.head_dim_v,
                        None, None, None)
    r = int(_lib.pkv_suggest_split(ctypes.byref(cs), num_q_heads, batch, int(total_tokens),
                                   max_seq_len))
    if r < 0:
        raise PkvError("pkv_suggest_split", r)
    return r


def _check(fn: str, status: int) -> None:
    if status != PKV_OK:
        raise PkvError(fn, status)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libpkv takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libpkv takes contiguous tensors")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


@dataclass
class Cache:
    """A paged cache held in torch device tensors.

    k_pool: uint8 (e4m3 codes) or bfloat16, [num_pages, Hkv, P, Dk]
    v_pool: same dtype, [num_pages, Hkv, P, Dv]; None = latent layout
            (V is the first ``latent_dim_v`` values of each K row)
    k_scale, v_scale: float32 [Hkv] (e4m3 only)
    page_tags: int32 or uint32 [num_pages]
    k_row_scale, v_row_scale: float32 [num_pages, Hkv, P], scales set at
            append, one per row (e4m3 with separate pools); None = the
            static per-head scales
    """
    k_pool: torch.Tensor
    v_pool: torch.Tensor | None = None
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None
    page_tags: torch.Tensor | None = None
    latent_dim_v: int | None = None
    k_row_scale: torch.Tensor | None = None
    v_row_scale: torch.Tensor | None = None

    @property
    def dtype(self) -> int:
        return PKV_KV_E4M3 if self.k_pool.dtype == torch.uint8 else PKV_KV_BF16

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def page_size(self) -> int:
        return int(self.k_pool.shape[2])

    @property
    def head_dim_k(self) -> int:
        return int(self.k_pool.shape[3])

    @property
    def head_dim_v(self) -> int:
        return int(self.v_pool.shape[3]) if self.v_pool is not None else int(self.latent_dim_v)

    def struct(self) -> PkvCacheStruct:
        if self.k_pool.dtype not in (torch.uint8, torch.bfloat16):
            raise ValueError("pool dtype must be uint8 (e4m3) or bfloat16")
        if self.v_pool is not None and self.v_pool.dtype != self.k_pool.dtype:
            raise ValueError("K and V pools differ in dtype")
        if self.v_pool is None and self.latent_dim_v is None:
            raise ValueError("latent layout needs latent_dim_v")
        for t in (self.k_scale, self.v_scale, self.k_row_scale, self.v_row_scale):
            if t is not None and t.dtype != torch.float32:
                raise ValueError("scales are float32")
        for t in (self.k_row_scale, self.v_row_scale):
            if t is not None and tuple(t.shape) != (self.num_pages, self.num_kv_heads,
                                                    self.page_size):
                raise ValueError("row scales are [num_pages, num_kv_heads, page_size]")
        if self.page_tags is not None and self.page_tags.element_size() != 4:
            raise ValueError("page tags are 32-bit")
        return PkvCacheStruct(_ptr(self.k_pool), _ptr(self.v_pool), self.dtype, self.num_pages,
                              self.page_size, self.num_kv_heads, self.head_dim_k,
                              self.head_dim_v, _ptr(self.k_scale), _ptr(self.v_scale),
                              _ptr(self.page_tags), _ptr(self.k_row_scale),
                              _ptr(self.v_row_scale))


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def pkv_scales_from_amax(x: torch.Tensor, per_head: bool, scale_out: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """x: bf16 [n_rows, H, D] -> float32 [H] scales (written into scale_out)."""
    _need(x, torch.bfloat16, "x")
    n, H, D = x.shape
    if scale_out is None:
        scale_out = torch.empty(H, dtype=torch.float32, device=x.device)
    _check("pkv_scales_from_amax", _lib.pkv_scales_from_amax(
        _ptr(x), n, H, D, 1 if per_head else 0, _ptr(scale_out), _stream(stream)))
    return scale_out


def pkv_append(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor | None,
               slot: torch.Tensor, token_req: torch.Tensor | None = None,
               abort_flags: torch.Tensor | None = None, stream=None) -> None:
    _need(k_new, torch.bfloat16, "k_new")
    if v_new is not None:
        _need(v_new, torch.bfloat16, "v_new")
    _need(slot, torch.int32, "slot")
    cs = cache.struct()
    _check("pkv_append", _lib.pkv_append(
        ctypes.byref(cs), _ptr(k_new), _ptr(v_new), _ptr(slot), _ptr(token_req),
        _ptr(abort_flags), int(slot.numel()), _stream(stream)))


def pkv_decode_attn_drafts(cache: Cache, q: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, max_seq_len: int,
                           abort_flags: torch.Tensor | None, sm_scale: float, split_tokens: int,
                           o_part: torch.Tensor, lse_part: torch.Tensor, stream=None) -> None:
    """q: bf16 [B, q_len, Hq, Dk] (a token and its drafts per request);
    o_part [B, q_len*Hq, max_splits, Dv], lse_part [B, q_len*Hq, max_splits]."""
    _need(q, torch.bfloat16, "q")
    B, T, Hq, _ = q.shape
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    if o_part.shape[1] != T * Hq or lse_part.shape[1] != T * Hq:
        raise ValueError("o_part / lse_part need q_len * num_q_heads rows per request")
    cs = cache.struct()
    _check("pkv_decode_attn_drafts", _lib.pkv_decode_attn_drafts(
        ctypes.byref(cs), _ptr(q), Hq, T, _ptr(block_table), _ptr(seq_lens), B,
        int(block_table.shape[1]), int(max_seq_len), _ptr(abort_flags), float(sm_scale),
        int(split_tokens), int(o_part.shape[2]), _ptr(o_part), _ptr(lse_part), _stream(stream)))


def pkv_int4_linear(x: torch.Tensor, w: torch.Tensor, scales: torch.Tensor, y: torch.Tensor,
                    workspace: torch.Tensor | None = None, stream=None) -> None:
    """y bf16 [B, n] = x bf16 [B, k] times the INT4 weights w uint8 [n, k/2]
    with bf16 group scales [k/128, n]; workspace: a uint8 device tensor of at
    least pkv_int4_linear_workspace(B, n, k) bytes, or None."""
    _need(x, torch.bfloat16, "x")
    _need(scales, torch.bfloat16, "scales")
    _need(y, torch.bfloat16, "y")
    if w.dtype != torch.uint8 or not w.is_contiguous():
        raise ValueError("w: contiguous uint8 [n, k/2]")
    B, k = x.shape
    n = w.shape[0]
    if w.shape[1] * 2 != k or tuple(scales.shape) != (k // 128, n) or tuple(y.shape) != (B, n):
        raise ValueError("pkv_int4_linear: shapes x [B, k], w [n, k/2], scales [k/128, n], y [B, n]")
    ws = None
    if workspace is not None:
        need = pkv_int4_linear_workspace(B, n, k)
        if workspace.device != x.device or workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace: at least {need} bytes on {x.device}")
        ws = _ptr(workspace)
    _check("pkv_int4_linear", _lib.pkv_int4_linear(_ptr(x), _ptr(w), _ptr(scales), B, n, k,
                                                   _ptr(y), ws, _stream(stream)))


def pkv_int4_linear_workspace(batch: int, n: int, k: int) -> int:
    """Bytes of workspace pkv_int4_linear wants (0: none)."""
    r = int(_lib.pkv_int4_linear_workspace(batch, n, k))
    if r < 0:
        _check("pkv_int4_linear_workspace", r)
    return r


def int4_workspace(max_batch: int, n: int, k: int, device) -> torch.Tensor | None:
    """A workspace for pkv_int4_linear calls of up to max_batch tokens on an
    n x k layer (None if they need none); reusable across calls and shapes
    that fit it."""
    need = max(pkv_int4_linear_workspace(b, n, k) for b in range(1, max_batch + 1))
    return torch.zeros((need,), dtype=torch.uint8, device=device) if need else None


def pkv_requantize_pages(src: Cache, dst: Cache, src_pages: torch.Tensor, dst_pages: torch.Tensor,
                         new_tags: torch.Tensor | None = None, stream=None) -> None:
    """Re-encode BF16 pages of src into e4m3 pages of dst; with new_tags, the
    destination pages' tags in dst.page_tags become new_tags."""
    _need(src_pages, torch.int32, "src_pages")
    _need(dst_pages, torch.int32, "dst_pages")
    if src_pages.numel() != dst_pages.numel():
        raise ValueError("src_pages and dst_pages differ in length")
    if new_tags is not None:
        if new_tags.numel() != src_pages.numel() or new_tags.element_size() != 4:
            raise ValueError("new_tags: one 32-bit tag per page pair")
        if dst.page_tags is None:
            raise ValueError("new_tags needs dst.page_tags")
    ss, ds = src.struct(), dst.struct()
    _check("pkv_requantize_pages", _lib.pkv_requantize_pages(
        ctypes.byref(ss), ctypes.byref(ds), _ptr(src_pages), _ptr(dst_pages), _ptr(new_tags),
        _ptr(dst.page_tags) if new_tags is not None else None, int(src_pages.numel()),
        _stream(stream)))


def pkv_verify(cache: Cache, block_table: torch.Tensor, expected_tags: torch.Tensor,
               seq_lens: torch.Tensor, abort_out: torch.Tensor, stream=None) -> None:
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(abort_out, torch.uint8, "abort_out")
    if expected_tags.element_size() != 4:
        raise ValueError("expected_tags are 32-bit")
    B, max_pages = block_table.shape
    cs = cache.struct()
    _check("pkv_verify", _lib.pkv_verify(
        ctypes.byref(cs), _ptr(block_table), _ptr(expected_tags), _ptr(seq_lens), B, max_pages,
        _ptr(abort_out), _stream(stream)))


def pkv_verify_append(cache: Cache, block_table: torch.Tensor, expected_tags: torch.Tensor,
                      seq_lens: torch.Tensor, abort_out: torch.Tensor, k_new: torch.Tensor,
                      v_new: torch.Tensor | None, slot: torch.Tensor, stream=None) -> None:
    """The tag check and the append of one new token per request (k_new[b]
    of request b, at slot[b]) in one launch; an aborted request writes
    nothing."""
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(abort_out, torch.uint8, "abort_out")
    _need(slot, torch.int32, "slot")
    _need(k_new, torch.bfloat16, "k_new")
    if v_new is not None:
        _need(v_new, torch.bfloat16, "v_new")
    if expected_tags.element_size() != 4:
        raise ValueError("expected_tags are 32-bit")
    B, max_pages = block_table.shape
    if k_new.shape[0] != B or slot.numel() != B:
        raise ValueError("one new token per request")
    cs = cache.struct()
    _check("pkv_verify_append", _lib.pkv_verify_append(
        ctypes.byref(cs), _ptr(block_table), _ptr(expected_tags), _ptr(seq_lens), B, max_pages,
        _ptr(abort_out), _ptr(k_new), _ptr(v_new), _ptr(slot), _stream(stream)))


def pkv_decode_attn(cache: Cache, q: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, max_seq_len: int, abort_flags: torch.Tensor | None,
                    sm_scale: float, split_tokens: int, o_part: torch.Tensor,
                    lse_part: torch.Tensor, stream=None) -> None:
    """q bf16 [B, Hq, Dk]; o_part f32 [B, Hq, max_splits, Dv]; lse_part f32 [B, Hq, max_splits]."""
    _need(q, torch.bfloat16, "q")
    _need(o_part, torch.float32, "o_part")
    _need(lse_part, torch.float32, "lse_part")
    B, Hq, _ = q.shape
    max_splits = int(lse_part.shape[2])
    cs = cache.struct()
    _check("pkv_decode_attn", _lib.pkv_decode_attn(
        ctypes.byref(cs), _ptr(q), Hq, _ptr(block_table), _ptr(seq_lens), B,
        int(block_table.shape[1]), int(max_seq_len), _ptr(abort_flags), float(sm_scale),
        int(split_tokens), max_splits, _ptr(o_part), _ptr(lse_part), _stream(stream)))


def pkv_combine(o_part: torch.Tensor, lse_part: torch.Tensor, seq_lens: torch.Tensor,
                split_tokens: int, max_seq_len: int, abort_flags: torch.Tensor | None,
                out: torch.Tensor, lse_out: torch.Tensor | None = None, stream=None) -> None:
    """out bf16 [B, Hq, Dv]; lse_out f32 [B, Hq] or None."""
    _need(out, torch.bfloat16, "out")
    B, Hq, max_splits, Dv = o_part.shape
    _check("pkv_combine", _lib.pkv_combine(
        _ptr(o_part), _ptr(lse_part), _ptr(seq_lens), B, Hq, Dv, int(split_tokens), max_splits,
        int(max_seq_len), _ptr(abort_flags), _ptr(out), _ptr(lse_out), _stream(stream)))


def pkv_step_decode(cache: Cache, q: torch.Tensor, k_new: torch.Tensor,
                    v_new: torch.Tensor | None, block_table: torch.Tensor,
                    expected_tags: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                    sm_scale: float, split_tokens: int, o_part: torch.Tensor,
                    lse_part: torch.Tensor, unit_flags: torch.Tensor, abort_out: torch.Tensor,
                    stream=None) -> None:
    """First launch of a step in two: the decode with each split's tag check
    (none when expected_tags is None) and each request's new token (k_new[b],
    v_new[b] at position seq_lens[b] - 1) read from its values. unit_flags
    uint8 [B, max_splits]."""
    _need(q, torch.bfloat16, "q")
    _need(k_new, torch.bfloat16, "k_new")
    if v_new is not None:
        _need(v_new, torch.bfloat16, "v_new")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    _need(o_part, torch.float32, "o_part")
    _need(lse_part, torch.float32, "lse_part")
    _need(unit_flags, torch.uint8, "unit_flags")
    _need(abort_out, torch.uint8, "abort_out")
    if expected_tags is not None and expected_tags.element_size() != 4:
        raise ValueError("expected_tags are 32-bit")
    B, Hq, _ = q.shape
    max_splits = int(lse_part.shape[2])
    if k_new.shape[0] != B or tuple(unit_flags.shape) != (B, max_splits):
        raise ValueError("one new token per request; unit_flags [B, max_splits]")
    cs = cache.struct()
    _check("pkv_step_decode", _lib.pkv_step_decode(
        ctypes.byref(cs), _ptr(q), Hq, _ptr(k_new), _ptr(v_new), _ptr(block_table),
        _ptr(expected_tags), _ptr(seq_lens), B, int(block_table.shape[1]), int(max_seq_len),
        float(sm_scale), int(split_tokens), max_splits, _ptr(o_part), _ptr(lse_part),
        _ptr(unit_flags), _ptr(abort_out), _stream(stream)))


def pkv_step_combine(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor | None,
                     block_table: torch.Tensor, expected_tags: torch.Tensor,
                     seq_lens: torch.Tensor, max_seq_len: int, split_tokens: int,
                     o_part: torch.Tensor, lse_part: torch.Tensor, unit_flags: torch.Tensor,
                     abort_out: torch.Tensor, out: torch.Tensor,
                     lse_out: torch.Tensor | None = None, stream=None) -> None:
    """Second launch of a step in two (after pkv_step_decode with the same
    arguments): the abort flags, the append of each standing request's new
    token, the merge into out bf16 [B, Hq, Dv] and lse_out f32 [B, Hq]."""
    _need(out, torch.bfloat16, "out")
    _need(unit_flags, torch.uint8, "unit_flags")
    _need(abort_out, torch.uint8, "abort_out")
    if expected_tags is not None and expected_tags.element_size() != 4:
        raise ValueError("expected_tags are 32-bit")
    B, Hq, max_splits, _ = o_part.shape
    cs = cache.struct()
    _check("pkv_step_combine", _lib.pkv_step_combine(
        ctypes.byref(cs), Hq, _ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(expected_tags),
        _ptr(seq_lens), B, int(block_table.shape[1]), int(max_seq_len), int(split_tokens),
        max_splits, _ptr(o_part), _ptr(lse_part), _ptr(unit_flags), _ptr(abort_out), _ptr(out),
        _ptr(lse_out), _stream(stream)))


def pkv_step_launches(cache: Cache, num_q_heads: int, split_tokens: int) -> int:
    """2 if this shape's step runs in two launches, 3 if in three."""
    # only the geometry is read (as for pkv_suggest_split)
    rows = 1 if cache.k_row_scale is not None else None
    cs = PkvCacheStruct(1, None if cache.v_pool is None else 1, cache.dtype, cache.num_pages,
                        cache.page_size, cache.num_kv_heads, cache.head_dim_k, cache.head_dim_v,
                        None, None, None, rows, rows)
    n = _lib.pkv_step_launches(ctypes.byref(cs), int(num_q_heads), int(split_tokens))
    _check("pkv_step_launches", min(n, 0))
    return n


def pkv_fill_u32(dst: torch.Tensor, value: int, stream=None) -> None:
    """Write `value` to every 32-bit word of a contiguous device tensor (a
    measurement helper: evicts the last-level cache between timed steps)."""
    if not dst.is_contiguous() or dst.numel() * dst.element_size() % 4:
        raise ValueError("dst must be contiguous whole 32-bit words")
    _check("pkv_fill_u32", _lib.pkv_fill_u32(
        _ptr(dst), dst.numel() * dst.element_size() // 4, int(value) & 0xFFFFFFFF,
        _stream(stream)))



def pkv_read_u32(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every whole 16-byte word of a contiguous device tensor, XORing
    into sink (one int32 on the device): with pkv_fill_u32, the last-level
    cache flush of the measurement."""
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    _check("pkv_read_u32", _lib.pkv_read_u32(
        _ptr(src), src.numel() * src.element_size() // 4, _ptr(sink), _stream(stream)))

STATIC_SCRATCH_BYTES = 64 << 20  # PKV_STATIC_SCRATCH_BYTES of include/pkv.h


def pkv_decode_attn_static(cache: Cache, q: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, max_seq_len: int,
                           abort_flags: torch.Tensor | None, sm_scale: float, split_tokens: int,
                           out: torch.Tensor, lse_out: torch.Tensor | None = None,
                           stream=None) -> None:
    """Decode and combine with the partials in the library's own device array
    (no caller buffers, nothing allocated): q bf16 [B, Hq, Dk] -> out bf16
    [B, Hq, Dv], lse_out f32 [B, Hq] or None."""
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    B, Hq, _ = q.shape
    cs = cache.struct()
    _check("pkv_decode_attn_static", _lib.pkv_decode_attn_static(
        ctypes.byref(cs), _ptr(q), Hq, _ptr(block_table), _ptr(seq_lens), B,
        int(block_table.shape[1]), int(max_seq_len), _ptr(abort_flags), float(sm_scale),
        int(split_tokens), _ptr(out), _ptr(lse_out), _stream(stream)))
