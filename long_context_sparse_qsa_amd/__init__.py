"""Python binding of libqsa.so, the MI355X (gfx950) QSA layer-path library.

Argument marshalling only: every step of the path runs in the HIP kernels of
libqsa.so, called through its C ABI (include/qsa.h) with ``ctypes``.
PyTorch supplies device memory and the current HIP stream; no torch type
crosses the ABI.  Importing this package fails loudly if the library has
not been built (``python -m long_context_sparse_qsa_amd.build``); there is no
other code path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first: libqsa.so then binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_OK = 0
QSA_ERR_ARG = -1
QSA_ERR_UNSUPPORTED = -2
QSA_ERR_WORKSPACE = -3
QSA_ERR_LAUNCH = -4
QSA_ERR_DEVICE = -5
QSA_F32 = 0
QSA_BF16 = 1
QSA_KV_SAME = 0
QSA_KV_FP8_E4M3 = 1
QSA_KV_Q8_0 = 2
INDEX_DIM = 128
INDEX_HEADS = 4
BLOCK_TOKENS = 4
MAX_K_BLOCKS = 1024
MAX_SEGMENTS = 16

EXPORTED = (
    "qsa_append_pool", "qsa_score_blocks", "qsa_select_topk", "qsa_gathered_attn",
    "qsa_append_score", "qsa_quantize_kv_fp8", "qsa_score_select", "qsa_score_select_workspace_bytes",
    "qsa_select_workspace_bytes", "qsa_attn_workspace_bytes", "qsa_attn_plan", "qsa_gathered_attn_noalloc",
    "qsa_quantize_kv_q8_0",
    "qsa_device_check", "qsa_last_error", "qsa_version",
)

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_qsa_amd.build` "
        "(hipcc, gfx950). The QSA path has no fallback.")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


class QsaKvSegments(ctypes.Structure):
    """ctypes mirror of ``qsa_kv_segments`` (include/qsa.h)."""

    _fields_ = [
        ("n_seq", _I32), ("n_seg_total", _I32), ("max_seg_per_seq", _I32), ("kv_format", _I32),
        ("seq_seg_begin", _P), ("seg_start", _P), ("seg_len", _P), ("seg_cap", _P),
        ("k_seg", _P), ("v_seg", _P), ("k_scale_seg", _P), ("v_scale_seg", _P),
    ]


_lib.qsa_append_pool.argtypes = [_P, _I32, _I32, _P, _P, _P, _P, _I32, _I64, _P]
_lib.qsa_score_blocks.argtypes = [_P, _I32, _I32, _P, _P, _P, _I32, _I64, _I64, _P, _I64, _P, _SZ, _P]
_lib.qsa_select_topk.argtypes = [_P, _I64, _I32, _P, _I64, _I32, _P, _P, _P, _SZ, _I32, _P]
_lib.qsa_gathered_attn.argtypes = [_P, _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P,
                                   ctypes.POINTER(QsaKvSegments), _P, _P, _I32, _P, _P, _P, _SZ, _P]
_lib.qsa_gathered_attn_noalloc.argtypes = [_P, _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P,
                                           ctypes.POINTER(QsaKvSegments), _P, _P, _I32, _P, _P, _P]
_lib.qsa_append_score.argtypes = [_P, _I32, _P, _P, _P, _I64, _P, _I32, _I32, _P, _I64, _P, _I64, _P, _SZ, _P]
_lib.qsa_quantize_kv_fp8.argtypes = [_P, _I32, _I32, _I32, _I64, _P, _P, _I64, _P]
_lib.qsa_quantize_kv_q8_0.argtypes = [_P, _I32, _I32, _I32, _I64, _P, _P, _I64, _P]
_lib.qsa_score_select.argtypes = [_P, _I32, _P, _P, _I64, _I32, _P, _P, _P, _SZ, _P]
_lib.qsa_score_select_workspace_bytes.argtypes = [_I32, _I64, _I32]
_lib.qsa_score_select_workspace_bytes.restype = _SZ
_lib.qsa_select_workspace_bytes.argtypes = [_I32, _I64, _I32]
_lib.qsa_select_workspace_bytes.restype = _SZ
_lib.qsa_attn_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
_lib.qsa_attn_workspace_bytes.restype = _SZ
_lib.qsa_attn_plan.argtypes = [_I32, _I32, _I32, _I32, ctypes.POINTER(_I32)]
_lib.qsa_device_check.argtypes = []
_lib.qsa_last_error.restype = ctypes.c_char_p
_lib.qsa_version.restype = ctypes.c_char_p
for _f in ("qsa_append_pool", "qsa_score_blocks", "qsa_select_topk", "qsa_gathered_attn",
           "qsa_append_score", "qsa_quantize_kv_fp8", "qsa_score_select", "qsa_attn_plan", "qsa_device_check",
           "qsa_gathered_attn_noalloc", "qsa_quantize_kv_q8_0"):
    getattr(_lib, _f).restype = ctypes.c_int


class QsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"QSA status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != QSA_OK:
        raise QsaError(status, _lib.qsa_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return QSA_BF16
    if t.dtype == torch.float32:
        return QSA_F32
    raise TypeError(f"QSA tensors are bfloat16 or float32, got {t.dtype}")


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def version() -> str:
    return _lib.qsa_version().decode()


def qsa_device_check() -> None:
    """Raise unless the current device is gfx950."""
    _check(_lib.qsa_device_check())


def qsa_select_workspace_bytes(max_m: int, nb_max: int, k_blocks: int) -> int:
    return int(_lib.qsa_select_workspace_bytes(max_m, nb_max, k_blocks))


def qsa_attn_workspace_bytes(max_m: int, hq: int, head_dim: int, k_blocks: int) -> int:
    return int(_lib.qsa_attn_workspace_bytes(max_m, hq, head_dim, k_blocks))


def qsa_attn_plan(m: int, hkv: int, k_blocks: int, dtype=torch.bfloat16) -> dict:
    """The split plan ``qsa_gathered_attn`` uses for ``m`` rows (host only)."""
    out = (_I32 * 4)()
    code = QSA_BF16 if dtype == torch.bfloat16 else QSA_F32
    _check(_lib.qsa_attn_plan(int(m), int(hkv), int(k_blocks), code, out))
    return {"waves": out[0], "tile_tokens": out[1], "tiles_per_split": out[2], "splits": out[3]}


def qsa_append_pool(new_idx: torch.Tensor, pos: torch.Tensor, idx_cache: torch.Tensor,
                    pooled: torch.Tensor, seq: torch.Tensor | None = None, stream=None) -> None:
    """Write ``new_idx`` [T,128] at positions ``pos`` (int64 [T]) of
    ``idx_cache`` [n_seq,cap,128] (or [cap,128]) and pool completed blocks
    into ``pooled`` [n_seq,cap/4,128] float32."""
    cache = idx_cache if idx_cache.dim() == 3 else idx_cache.unsqueeze(0)
    _need(new_idx.is_contiguous() and cache.is_contiguous() and pooled.is_contiguous(), "tensors must be contiguous")
    _need(pos.dtype == torch.int64 and (seq is None or seq.dtype == torch.int32), "pos int64, seq int32")
    _need(new_idx.dtype == cache.dtype and pooled.dtype == torch.float32, "dtype mismatch")
    _need(new_idx.shape[-1] == INDEX_DIM and cache.shape[-1] == INDEX_DIM, "index width must be 128")
    n_seq, cap = cache.shape[0], cache.shape[1]
    _need(pooled.numel() == n_seq * (cap // BLOCK_TOKENS) * INDEX_DIM, "pooled shape mismatch")
    _need(pos.numel() == new_idx.shape[0] and (seq is None or seq.numel() == new_idx.shape[0]), "pos/seq length")
    _check(_lib.qsa_append_pool(_ptr(new_idx), _dtype_code(new_idx), new_idx.shape[0], _ptr(pos),
                                _ptr(seq), _ptr(cache), _ptr(pooled), n_seq, cap, _stream(stream)))


def qsa_score_blocks(idx_q: torch.Tensor, row_pos: torch.Tensor, pooled: torch.Tensor,
                     scores: torch.Tensor, nb_max: int, row_seq: torch.Tensor | None = None,
                     sel_workspace: torch.Tensor | None = None, stream=None) -> None:
    """``scores`` [M, ld] float32 <- block scores of the rows ``idx_q`` [M,4,128].
    With ``sel_workspace`` the pass also prepares ``qsa_select_topk(prepared=True)``."""
    pl = pooled if pooled.dim() == 3 else pooled.unsqueeze(0)
    _need(idx_q.is_contiguous() and pl.is_contiguous() and scores.is_contiguous(), "tensors must be contiguous")
    _need(row_pos.dtype == torch.int64 and (row_seq is None or row_seq.dtype == torch.int32), "row_pos int64, row_seq int32")
    m = idx_q.shape[0]
    _need(idx_q.shape[1:] == (INDEX_HEADS, INDEX_DIM), "idx_q must be [M,4,128]")
    _need(scores.dim() == 2 and scores.shape[0] >= m and scores.dtype == torch.float32, "scores [M, ld] float32")
    _check(_lib.qsa_score_blocks(_ptr(idx_q), _dtype_code(idx_q), m, _ptr(row_pos), _ptr(row_seq),
                                 _ptr(pl), pl.shape[0], pl.shape[1] * BLOCK_TOKENS, int(nb_max),
                                 _ptr(scores), scores.shape[1], _ptr(sel_workspace), _nbytes(sel_workspace),
                                 _stream(stream)))


def qsa_select_topk(scores: torch.Tensor, row_pos: torch.Tensor, nb_max: int, k_blocks: int,
                    sel: torch.Tensor, n_sel: torch.Tensor, workspace: torch.Tensor | None = None,
                    prepared: bool = False, stream=None) -> None:
    """``sel`` [M,k] int32 (ascending, -1 padded), ``n_sel`` [M] int32.
    ``workspace``: zero-filled once; ``prepared``: the scoring call built its
    histograms (``qsa_score_blocks(..., sel_workspace=workspace)``)."""
    m = row_pos.numel()
    _need(sel.dtype == torch.int32 and n_sel.dtype == torch.int32 and sel.is_contiguous(), "sel/n_sel int32")
    _need(sel.shape[0] >= m and sel.shape[1] == k_blocks, "sel must be [M, k_blocks]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.qsa_select_topk(_ptr(scores), scores.shape[1], m, _ptr(row_pos), int(nb_max),
                                int(k_blocks), _ptr(sel), _ptr(n_sel), _ptr(workspace), ws_bytes,
                                1 if prepared else 0, _stream(stream)))


class KvSegments:
    """Device segment table of a batch of sequences for ``qsa_gathered_attn``.

    ``segments[s]`` is a list of (start, length, K, V) for sequence s, with
    K/V tensors [hkv, cap, head_dim] (cap >= length) in the query dtype, or
    (start, length, K, V, K_scale, V_scale) for quantized K/V: fp8 as uint8
    E4M3 codes [hkv, cap, head_dim] with float16 scales [hkv, cap] (see
    ``qsa_quantize_kv_fp8``), Q8_0 as int8 codes [hkv, cap, head_dim] with
    float16 scales [hkv, cap, head_dim / 32] (see ``qsa_quantize_kv_q8_0``).
    The tensors must stay alive (and in place) while the table is used; the
    table keeps references.
    """

    def __init__(self, segments: list, device=None):
        dev = device or segments[0][0][2].device
        self._keep = []
        begin, starts, lens, caps, kp, vp, ksp, vsp = [0], [], [], [], [], [], [], []
        quant = len(segments[0][0]) == 6
        q8 = quant and segments[0][0][2].dtype == torch.int8
        fp8 = quant and not q8
        for segs in segments:
            for seg in segs:
                _need(len(seg) == (6 if quant else 4), "all segments quantized or none")
                st, ln, k, v = seg[:4]
                assert k.is_contiguous() and v.is_contiguous() and k.shape == v.shape
                starts.append(int(st))
                lens.append(int(ln))
                caps.append(int(k.shape[1]))
                kp.append(k.data_ptr())
                vp.append(v.data_ptr())
                self._keep += [k, v]
                if quant:
                    ks, vs = seg[4], seg[5]
                    want = torch.int8 if q8 else torch.uint8
                    _need(k.dtype == want and ks.dtype == torch.float16 and vs.dtype == torch.float16,
                          "quantized segments: uint8 (fp8) or int8 (Q8_0) codes, float16 scales")
                    sshape = (k.shape[0], k.shape[1], k.shape[2] // 32) if q8 else k.shape[:2]
                    _need(ks.is_contiguous() and vs.is_contiguous() and ks.shape == sshape == vs.shape,
                          "scale shape [hkv, cap] (fp8) or [hkv, cap, head_dim / 32] (Q8_0)")
                    ksp.append(ks.data_ptr())
                    vsp.append(vs.data_ptr())
                    self._keep += [ks, vs]
            begin.append(len(starts))
        self.fp8 = fp8
        self.q8 = q8
        self.max_seg = max(len(s) for s in segments)
        self.seq_seg_begin = torch.tensor(begin, dtype=torch.int32, device=dev)
        self.seg_start = torch.tensor(starts, dtype=torch.int64, device=dev)
        self.seg_len = torch.tensor(lens, dtype=torch.int64, device=dev)
        self.seg_cap = torch.tensor(caps, dtype=torch.int64, device=dev)
        self.k_ptrs = torch.tensor(kp, dtype=torch.int64, device=dev)
        self.v_ptrs = torch.tensor(vp, dtype=torch.int64, device=dev)
        self.ks_ptrs = torch.tensor(ksp, dtype=torch.int64, device=dev) if quant else None
        self.vs_ptrs = torch.tensor(vsp, dtype=torch.int64, device=dev) if quant else None
        fmt = QSA_KV_Q8_0 if q8 else QSA_KV_FP8_E4M3 if fp8 else QSA_KV_SAME
        self.struct = QsaKvSegments(
            len(segments), len(starts), self.max_seg, fmt,
            self.seq_seg_begin.data_ptr(), self.seg_start.data_ptr(), self.seg_len.data_ptr(),
            self.seg_cap.data_ptr(), self.k_ptrs.data_ptr(), self.v_ptrs.data_ptr(),
            self.ks_ptrs.data_ptr() if quant else None, self.vs_ptrs.data_ptr() if quant else None)

    @classmethod
    def single(cls, k: torch.Tensor, v: torch.Tensor, length: int | None = None,
               k_scale: torch.Tensor | None = None, v_scale: torch.Tensor | None = None):
        """One sequence held in one [hkv, cap, D] buffer (fp8 / Q8_0: with its scales)."""
        n = k.shape[1] if length is None else length
        if k_scale is not None:
            return cls([[(0, n, k, v, k_scale, v_scale)]])
        return cls([[(0, n, k, v)]])


def qsa_append_score(new_idx: torch.Tensor, new_pos: torch.Tensor, idx_cache: torch.Tensor, pooled: torch.Tensor,
                     idx_q: torch.Tensor, row_pos: torch.Tensor, scores: torch.Tensor, nb_max: int,
                     sel_workspace: torch.Tensor | None = None, stream=None) -> None:
    """``qsa_append_pool`` of ``new_idx`` at ``new_pos`` into one sequence's
    ``idx_cache`` [cap,128] / ``pooled`` [cap/4,128], then ``qsa_score_blocks``
    of the rows ``idx_q`` over it: one launch where possible."""
    cache = idx_cache[0] if idx_cache.dim() == 3 else idx_cache
    pl = pooled[0] if pooled.dim() == 3 else pooled
    _need(new_idx.is_contiguous() and cache.is_contiguous() and pl.is_contiguous() and idx_q.is_contiguous()
          and scores.is_contiguous(), "tensors must be contiguous")
    _need(new_idx.dtype == cache.dtype == idx_q.dtype and pl.dtype == torch.float32, "dtype mismatch")
    _need(new_pos.dtype == torch.int64 and row_pos.dtype == torch.int64, "positions int64")
    cap = cache.shape[0]
    _need(pl.shape[0] == cap // BLOCK_TOKENS, "pooled shape mismatch")
    _check(_lib.qsa_append_score(_ptr(new_idx), new_idx.shape[0], _ptr(new_pos), _ptr(cache), _ptr(pl), cap,
                                 _ptr(idx_q), _dtype_code(idx_q), idx_q.shape[0], _ptr(row_pos), int(nb_max),
                                 _ptr(scores), scores.shape[1], _ptr(sel_workspace), _nbytes(sel_workspace),
                                 _stream(stream)))


def qsa_score_select_workspace_bytes(max_m: int, nb_max: int, k_blocks: int) -> int:
    return int(_lib.qsa_score_select_workspace_bytes(int(max_m), int(nb_max), int(k_blocks)))


def qsa_score_select(idx_q: torch.Tensor, row_pos: torch.Tensor, pooled: torch.Tensor, nb_max: int,
                     k_blocks: int, sel: torch.Tensor, n_sel: torch.Tensor, workspace: torch.Tensor,
                     stream=None) -> None:
    """``sel`` [M,k] / ``n_sel`` [M] <- top-k blocks of the bf16 rows ``idx_q``
    [M,4,128] over ``pooled`` ([cap/4,128] or [1,cap/4,128]) without writing
    the score matrix."""
    _need(idx_q.dtype == torch.bfloat16 and idx_q.is_contiguous(), "idx_q: contiguous bf16 [M,4,128]")
    _need(pooled.dtype == torch.float32 and pooled.is_contiguous(), "pooled: contiguous float32")
    _need(row_pos.dtype == torch.int64 and sel.dtype == torch.int32 and n_sel.dtype == torch.int32, "dtypes")
    m = idx_q.shape[0]
    _need(sel.shape[0] >= m and sel.shape[1] == k_blocks and sel.is_contiguous(), "sel [M, k_blocks]")
    _check(_lib.qsa_score_select(_ptr(idx_q), m, _ptr(row_pos), _ptr(pooled), int(nb_max), int(k_blocks),
                                 _ptr(sel), _ptr(n_sel), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def qsa_quantize_kv_fp8(src: torch.Tensor, dst: torch.Tensor, dst_scale: torch.Tensor, t0: int = 0,
                        stream=None) -> None:
    """E4M3 codes and f16 scales of ``src`` [n_head, T, D] bf16 written to rows
    t0 .. t0+T-1 of ``dst`` uint8 [n_head, cap, D] and ``dst_scale`` float16
    [n_head, cap]."""
    _need(src.dtype == torch.bfloat16 and dst.dtype == torch.uint8 and dst_scale.dtype == torch.float16,
          "src bf16, dst uint8, dst_scale float16")
    _need(src.is_contiguous() and dst.is_contiguous() and dst_scale.is_contiguous(), "tensors must be contiguous")
    h, t, d = src.shape
    _need(dst.dim() == 3 and dst.shape[0] == h and dst.shape[2] == d and dst_scale.shape == dst.shape[:2],
          "dst [n_head, cap, D], dst_scale [n_head, cap]")
    cap = dst.shape[1]
    _need(0 <= t0 and t0 + t <= cap, "rows t0..t0+T-1 must lie inside the cache")
    _check(_lib.qsa_quantize_kv_fp8(_ptr(src), h, t, d, t, dst.data_ptr() + t0 * d,
                                    dst_scale.data_ptr() + 2 * t0, cap, _stream(stream)))


def qsa_quantize_kv_q8_0(src: torch.Tensor, dst: torch.Tensor, dst_scale: torch.Tensor, t0: int = 0,
                         stream=None) -> None:
    """Q8_0 int8 codes and f16 scales (one per 32 values) of ``src`` [n_head,
    T, D] bf16 written to rows t0 .. t0+T-1 of ``dst`` int8 [n_head, cap, D]
    and ``dst_scale`` float16 [n_head, cap, D / 32]."""
    _need(src.dtype == torch.bfloat16 and dst.dtype == torch.int8 and dst_scale.dtype == torch.float16,
          "src bf16, dst int8, dst_scale float16")
    _need(src.is_contiguous() and dst.is_contiguous() and dst_scale.is_contiguous(), "tensors must be contiguous")
    h, t, d = src.shape
    _need(dst.dim() == 3 and dst.shape[0] == h and dst.shape[2] == d and
          dst_scale.shape == (h, dst.shape[1], d // 32), "dst [n_head, cap, D], dst_scale [n_head, cap, D / 32]")
    cap = dst.shape[1]
    _need(0 <= t0 and t0 + t <= cap, "rows t0..t0+T-1 must lie inside the cache")
    _check(_lib.qsa_quantize_kv_q8_0(_ptr(src), h, t, d, t, dst.data_ptr() + t0 * d,
                                     dst_scale.data_ptr() + 2 * t0 * (d // 32), cap, _stream(stream)))


def qsa_gathered_attn(q: torch.Tensor, row_pos: torch.Tensor, kv: KvSegments, sel: torch.Tensor,
                      n_sel: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, hkv: int,
                      scale: float | None = None, row_seq: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None) -> None:
    """``out`` [M,hq,D] (q dtype) and ``lse`` [M,hq] float32 <- attention of the
    rows ``q`` [M,hq,D] over their kept blocks plus tails."""
    m, hq, d = q.shape
    _need(q.is_contiguous() and out.is_contiguous() and lse.is_contiguous(), "tensors must be contiguous")
    _need(out.dtype == q.dtype and out.shape == q.shape and lse.dtype == torch.float32, "out/lse")
    _need(sel.shape[0] >= m and n_sel.numel() >= m, "sel/n_sel rows")
    scale = 1.0 / (d ** 0.5) if scale is None else float(scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.qsa_gathered_attn(_ptr(q), _dtype_code(q), m, hq, int(hkv), d, scale, _ptr(row_pos),
                                  _ptr(row_seq), ctypes.byref(kv.struct), _ptr(sel), _ptr(n_sel),
                                  sel.shape[1], _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                  _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20  # the static scratch of qsa_gathered_attn_noalloc, per device


def qsa_gathered_attn_noalloc(q: torch.Tensor, row_pos: torch.Tensor, kv: KvSegments, sel: torch.Tensor,
                              n_sel: torch.Tensor, out: torch.Tensor, lse: torch.Tensor, hkv: int,
                              scale: float | None = None, row_seq: torch.Tensor | None = None,
                              stream=None) -> None:
    """``qsa_gathered_attn`` with its split partials in the library's static
    device scratch: no workspace argument, nothing allocated.  Calls that
    overlap in time on one device race."""
    m, hq, d = q.shape
    _need(q.is_contiguous() and out.is_contiguous() and lse.is_contiguous(), "tensors must be contiguous")
    _need(out.dtype == q.dtype and out.shape == q.shape and lse.dtype == torch.float32, "out/lse")
    _need(sel.shape[0] >= m and n_sel.numel() >= m, "sel/n_sel rows")
    scale = 1.0 / (d ** 0.5) if scale is None else float(scale)
    _check(_lib.qsa_gathered_attn_noalloc(_ptr(q), _dtype_code(q), m, hq, int(hkv), d, scale, _ptr(row_pos),
                                          _ptr(row_seq), ctypes.byref(kv.struct), _ptr(sel), _ptr(n_sel),
                                          sel.shape[1], _ptr(out), _ptr(lse), _stream(stream)))
