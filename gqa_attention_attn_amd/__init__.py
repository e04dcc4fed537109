"""Python binding of the gfx950 grouped-query fused attention library.

The functions named ``gqa_attn_*`` mirror the C ABI in ``include/gqa_attn.h``
one to one (raw device pointers as ints, descriptor structs).  ``decode`` and
``prefill`` are conveniences that fill a descriptor from torch tensors and call
the same entry points; they only marshal arguments - every step of the
computation runs in the HIP kernels of ``libgqa_attn.so``.  There is no CPU or
PyTorch fallback: if the library is missing every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_attn.so")

# status codes and dtypes (must equal include/gqa_attn.h; checked by a CPU test)
GQA_OK = 0
GQA_ERR_NULL = 1
GQA_ERR_SHAPE = 2
GQA_ERR_UNSUPPORTED = 3
GQA_ERR_ALIGN = 4
GQA_ERR_WORKSPACE = 5
GQA_ERR_HIP = 6
GQA_ERR_SCRATCH = 7
GQA_F32 = 0
GQA_BF16 = 1
GQA_ATTN_HEAD_DIM = 128
GQA_ATTN_MAX_GROUP = 16
GQA_ATTN_VERSION = 3
GQA_ATTN_STATIC_SCRATCH_BYTES = 16 << 20

EXPORTS = (
    "gqa_attn_status_string",
    "gqa_attn_version",
    "gqa_attn_decode_plan",
    "gqa_attn_decode_workspace_size",
    "gqa_attn_decode",
    "gqa_attn_decode_partition",
    "gqa_attn_decode_merge",
    "gqa_attn_decode_static",
    "gqa_attn_decode_paged",
    "gqa_attn_prefill_workspace_size",
    "gqa_attn_prefill",
    "gqa_attn_prefill_keys",
    "gqa_attn_prefill_attend",
    "gqa_attn_prefill_chunk",
    "gqa_attn_prefill_chunk_paged",
)


class GqaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gqa_attn_status_string(status)} (status {status})")


class GqaDecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("kv_split_tokens", ctypes.c_int32),
        ("q_stride_b", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("k_stride_b", ctypes.c_int64), ("k_stride_h", ctypes.c_int64), ("k_stride_s", ctypes.c_int64),
        ("v_stride_b", ctypes.c_int64), ("v_stride_h", ctypes.c_int64), ("v_stride_s", ctypes.c_int64),
        ("out_stride_b", ctypes.c_int64), ("out_stride_h", ctypes.c_int64),
        ("eps", ctypes.c_float), ("scale", ctypes.c_float), ("write_new_k", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
    ]


class GqaPrefillDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("q_stride_b", ctypes.c_int64), ("q_stride_h", ctypes.c_int64), ("q_stride_s", ctypes.c_int64),
        ("k_stride_b", ctypes.c_int64), ("k_stride_h", ctypes.c_int64), ("k_stride_s", ctypes.c_int64),
        ("v_stride_b", ctypes.c_int64), ("v_stride_h", ctypes.c_int64), ("v_stride_s", ctypes.c_int64),
        ("out_stride_b", ctypes.c_int64), ("out_stride_h", ctypes.c_int64), ("out_stride_s", ctypes.c_int64),
        ("eps", ctypes.c_float), ("scale", ctypes.c_float), ("max_chunk", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("write_k_cache", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgqa_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (python -m gqa_attention_attn_amd.build); "
                               "there is no fallback implementation")
        # The library needs the HIP runtime by its soname (libamdhip64.so.7),
        # as does the copy torch ships.  Loaded after torch, the library binds
        # to torch's runtime, so torch's device memory and streams are valid
        # for it; loaded first, it would bring in the system runtime and torch
        # a second one, and the library's launches would fail.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p, szp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_size_t)
        L.gqa_attn_status_string.argtypes = [ctypes.c_int]
        L.gqa_attn_status_string.restype = ctypes.c_char_p
        L.gqa_attn_version.argtypes = []
        L.gqa_attn_version.restype = ctypes.c_int32
        L.gqa_attn_decode_plan.argtypes = [ctypes.POINTER(GqaDecodeDesc), i32p, i32p]
        L.gqa_attn_decode_plan.restype = ctypes.c_int
        L.gqa_attn_decode_workspace_size.argtypes = [ctypes.POINTER(GqaDecodeDesc), szp]
        L.gqa_attn_decode_workspace_size.restype = ctypes.c_int
        L.gqa_attn_decode.argtypes = [ctypes.POINTER(GqaDecodeDesc), vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp,
                                      vp, ctypes.c_size_t, vp]
        L.gqa_attn_decode.restype = ctypes.c_int
        L.gqa_attn_decode_partition.argtypes = L.gqa_attn_decode.argtypes
        L.gqa_attn_decode_partition.restype = ctypes.c_int
        L.gqa_attn_decode_merge.argtypes = [ctypes.POINTER(GqaDecodeDesc), vp, vp, vp, ctypes.c_size_t, vp]
        L.gqa_attn_decode_merge.restype = ctypes.c_int
        L.gqa_attn_decode_static.argtypes = [ctypes.POINTER(GqaDecodeDesc), vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.c_float, vp, vp]
        L.gqa_attn_decode_static.restype = ctypes.c_int
        L.gqa_attn_decode_paged.argtypes = [ctypes.POINTER(GqaDecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                            ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
        L.gqa_attn_decode_paged.restype = ctypes.c_int
        L.gqa_attn_prefill_workspace_size.argtypes = [ctypes.POINTER(GqaPrefillDesc), szp]
        L.gqa_attn_prefill_workspace_size.restype = ctypes.c_int
        L.gqa_attn_prefill.argtypes = [ctypes.POINTER(GqaPrefillDesc), vp, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                       vp, vp, ctypes.c_size_t, vp]
        L.gqa_attn_prefill.restype = ctypes.c_int
        for name in ("gqa_attn_prefill_keys", "gqa_attn_prefill_attend"):
            getattr(L, name).argtypes = L.gqa_attn_prefill.argtypes
            getattr(L, name).restype = ctypes.c_int
        L.gqa_attn_prefill_chunk.argtypes = [ctypes.POINTER(GqaPrefillDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
        L.gqa_attn_prefill_chunk.restype = ctypes.c_int
        L.gqa_attn_prefill_chunk_paged.argtypes = [ctypes.POINTER(GqaPrefillDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                                   vp, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
        L.gqa_attn_prefill_chunk_paged.restype = ctypes.c_int
        _lib = L
    return _lib


def use_library(path: str) -> None:
    """Take the entry points from another build of the same sources (the
    timeline build, libgqa_attn_timeline.so) instead of libgqa_attn.so; call
    it before the first call into the library."""
    global LIB_PATH, _lib
    if _lib is not None and os.path.abspath(path) != os.path.abspath(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is already loaded")
    LIB_PATH = os.path.abspath(path)


# ----------------------------------------------------------------- raw C ABI mirrors

def gqa_attn_status_string(status: int) -> str:
    return lib().gqa_attn_status_string(int(status)).decode()


def gqa_attn_version() -> int:
    return int(lib().gqa_attn_version())


def gqa_attn_decode_plan(desc: Optional[GqaDecodeDesc]) -> Tuple[int, int, int]:
    """Returns (status, split_tokens, num_splits)."""
    t, n = ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib().gqa_attn_decode_plan(ctypes.byref(desc) if desc is not None else None, ctypes.byref(t), ctypes.byref(n))
    return int(st), int(t.value), int(n.value)


def gqa_attn_decode_workspace_size(desc: Optional[GqaDecodeDesc]) -> Tuple[int, int]:
    """Returns (status, bytes)."""
    b = ctypes.c_size_t(0)
    st = lib().gqa_attn_decode_workspace_size(ctypes.byref(desc) if desc is not None else None, ctypes.byref(b))
    return int(st), int(b.value)


def gqa_attn_decode(desc, q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out,
                    workspace, workspace_bytes, stream) -> int:
    """Raw entry point: pointers are ints (0 = NULL); returns the status."""
    return int(lib().gqa_attn_decode(ctypes.byref(desc) if desc is not None else None, q, k_cache, v_cache, seq_lens,
                                     positions, q_norm_w, k_norm_w, float(rope_theta), out, workspace,
                                     int(workspace_bytes), stream))


def gqa_attn_decode_partition(desc, q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w, rope_theta,
                              out, workspace, workspace_bytes, stream) -> int:
    return int(lib().gqa_attn_decode_partition(ctypes.byref(desc) if desc is not None else None, q, k_cache,
                                               v_cache, seq_lens, positions, q_norm_w, k_norm_w, float(rope_theta),
                                               out, workspace, int(workspace_bytes), stream))


def gqa_attn_decode_merge(desc, seq_lens, out, workspace, workspace_bytes, stream) -> int:
    return int(lib().gqa_attn_decode_merge(ctypes.byref(desc) if desc is not None else None, seq_lens, out,
                                           workspace, int(workspace_bytes), stream))


def gqa_attn_decode_static(desc, q, k_cache, v_cache, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out,
                           stream) -> int:
    """gqa_attn_decode with the partials in the library's static device array (no workspace)."""
    return int(lib().gqa_attn_decode_static(ctypes.byref(desc) if desc is not None else None, q, k_cache, v_cache,
                                            seq_lens, positions, q_norm_w, k_norm_w, float(rope_theta), out,
                                            stream))


def gqa_attn_decode_paged(desc, q, k_pages, v_pages, block_table, seq_lens, positions, q_norm_w, k_norm_w,
                          rope_theta, out, workspace, workspace_bytes, stream) -> int:
    return int(lib().gqa_attn_decode_paged(ctypes.byref(desc) if desc is not None else None, q, k_pages, v_pages,
                                           block_table, seq_lens, positions, q_norm_w, k_norm_w, float(rope_theta),
                                           out, workspace, int(workspace_bytes), stream))


def gqa_attn_prefill_workspace_size(desc: Optional[GqaPrefillDesc]) -> Tuple[int, int]:
    """Returns (status, bytes)."""
    b = ctypes.c_size_t(0)
    st = lib().gqa_attn_prefill_workspace_size(ctypes.byref(desc) if desc is not None else None, ctypes.byref(b))
    return int(st), int(b.value)


def gqa_attn_prefill(desc, q, k, v, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out, workspace,
                     workspace_bytes, stream) -> int:
    return int(lib().gqa_attn_prefill(ctypes.byref(desc) if desc is not None else None, q, k, v, seq_lens, positions,
                                      q_norm_w, k_norm_w, float(rope_theta), out, workspace, int(workspace_bytes),
                                      stream))


def gqa_attn_prefill_keys(desc, q, k, v, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out, workspace,
                          workspace_bytes, stream) -> int:
    return int(lib().gqa_attn_prefill_keys(ctypes.byref(desc) if desc is not None else None, q, k, v, seq_lens,
                                           positions, q_norm_w, k_norm_w, float(rope_theta), out, workspace,
                                           int(workspace_bytes), stream))


def gqa_attn_prefill_attend(desc, q, k, v, seq_lens, positions, q_norm_w, k_norm_w, rope_theta, out, workspace,
                            workspace_bytes, stream) -> int:
    return int(lib().gqa_attn_prefill_attend(ctypes.byref(desc) if desc is not None else None, q, k, v, seq_lens,
                                             positions, q_norm_w, k_norm_w, float(rope_theta), out, workspace,
                                             int(workspace_bytes), stream))


def gqa_attn_prefill_chunk(desc, q, k_cache, v_cache, past_lens, chunk_lens, positions, q_norm_w, k_norm_w,
                           rope_theta, out, workspace, workspace_bytes, stream) -> int:
    return int(lib().gqa_attn_prefill_chunk(ctypes.byref(desc) if desc is not None else None, q, k_cache, v_cache,
                                            past_lens, chunk_lens, positions, q_norm_w, k_norm_w, float(rope_theta),
                                            out, workspace, int(workspace_bytes), stream))


def gqa_attn_prefill_chunk_paged(desc, q, k_pages, v_pages, block_table, past_lens, chunk_lens, positions,
                                 q_norm_w, k_norm_w, rope_theta, out, workspace, workspace_bytes, stream) -> int:
    return int(lib().gqa_attn_prefill_chunk_paged(ctypes.byref(desc) if desc is not None else None, q, k_pages,
                                                  v_pages, block_table, past_lens, chunk_lens, positions, q_norm_w,
                                                  k_norm_w, float(rope_theta), out, workspace, int(workspace_bytes),
                                                  stream))


# ----------------------------------------------------------------- torch conveniences

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    if t.dtype == torch.float32:
        return GQA_F32
    raise GqaError(GQA_ERR_UNSUPPORTED, f"dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def decode_desc(q, k_cache, v_cache, out, kv_split_tokens: int = 0, eps: float = 1e-6,
                scale: float = 0.0, write_new_k: bool = False) -> GqaDecodeDesc:
    """Descriptor for q [B, Hq, 128], caches [B, Hkv, S, 128], out [B, Hq, 128]."""
    B, Hq, d = q.shape
    _, Hkv, S, _ = k_cache.shape
    return GqaDecodeDesc(
        batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_seq=S, in_dtype=_dtype_code(q),
        out_dtype=_dtype_code(out), kv_split_tokens=int(kv_split_tokens),
        q_stride_b=q.stride(0), q_stride_h=q.stride(1),
        k_stride_b=k_cache.stride(0), k_stride_h=k_cache.stride(1), k_stride_s=k_cache.stride(2),
        v_stride_b=v_cache.stride(0), v_stride_h=v_cache.stride(1), v_stride_s=v_cache.stride(2),
        out_stride_b=out.stride(0), out_stride_h=out.stride(1), eps=float(eps), scale=float(scale),
        write_new_k=1 if write_new_k else 0)


def prefill_desc(q, k, v, out, causal: bool = True, eps: float = 1e-6, scale: float = 0.0,
                 write_k_cache: bool = False) -> GqaPrefillDesc:
    """Descriptor for q [B, Hq, S, 128], k/v [B, Hkv, S, 128], out [B, Hq, S, 128]."""
    B, Hq, S, d = q.shape
    Hkv = k.shape[1]
    return GqaPrefillDesc(
        batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_seq=S, in_dtype=_dtype_code(q),
        out_dtype=_dtype_code(out), causal=1 if causal else 0,
        q_stride_b=q.stride(0), q_stride_h=q.stride(1), q_stride_s=q.stride(2),
        k_stride_b=k.stride(0), k_stride_h=k.stride(1), k_stride_s=k.stride(2),
        v_stride_b=v.stride(0), v_stride_h=v.stride(1), v_stride_s=v.stride(2),
        out_stride_b=out.stride(0), out_stride_h=out.stride(1), out_stride_s=out.stride(2),
        eps=float(eps), scale=float(scale), write_k_cache=1 if write_k_cache else 0)


def prefill_chunk_desc(q, k_cache, v_cache, out, causal: bool = True, eps: float = 1e-6,
                       scale: float = 0.0, write_k_cache: bool = False) -> GqaPrefillDesc:
    """Descriptor for a chunk: q / out [B, Hq, T_max, 128], caches [B, Hkv, S, 128]."""
    B, Hq, T, d = q.shape
    _, Hkv, S, _ = k_cache.shape
    return GqaPrefillDesc(
        batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_seq=S, in_dtype=_dtype_code(q),
        out_dtype=_dtype_code(out), causal=1 if causal else 0,
        q_stride_b=q.stride(0), q_stride_h=q.stride(1), q_stride_s=q.stride(2),
        k_stride_b=k_cache.stride(0), k_stride_h=k_cache.stride(1), k_stride_s=k_cache.stride(2),
        v_stride_b=v_cache.stride(0), v_stride_h=v_cache.stride(1), v_stride_s=v_cache.stride(2),
        out_stride_b=out.stride(0), out_stride_h=out.stride(1), out_stride_s=out.stride(2),
        eps=float(eps), scale=float(scale), max_chunk=T, write_k_cache=1 if write_k_cache else 0)


def _stream_ptr(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def decode_workspace(desc: GqaDecodeDesc, device) -> "object":
    """Allocate (with torch) a workspace of the size the library asks for, or None."""
    import torch
    st, nbytes = gqa_attn_decode_workspace_size(desc)
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_decode_workspace_size")
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def decode(q, k_cache, v_cache, seq_lens, positions, q_norm_w=None, k_norm_w=None, rope_theta: float = 0.0,
           out=None, workspace=None, kv_split_tokens: int = 0, eps: float = 1e-6, scale: float = 0.0,
           out_dtype=None, stream=None, write_new_k: bool = False):
    """gqa_attn_decode on torch tensors (device memory); returns out.  With
    write_new_k, k_cache[b, :, seq_lens[b]-1] receives its post-prologue row."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    desc = decode_desc(q, k_cache, v_cache, out, kv_split_tokens, eps, scale, write_new_k)
    if workspace is None:
        workspace = decode_workspace(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = gqa_attn_decode(desc, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(positions),
                         _ptr(q_norm_w), _ptr(k_norm_w), rope_theta, _ptr(out), _ptr(workspace), ws_bytes,
                         _stream_ptr(stream))
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_decode")
    return out


def prefill_workspace(desc: GqaPrefillDesc, device) -> "object":
    """Allocate (with torch) the optional prefill workspace."""
    import torch
    st, nbytes = gqa_attn_prefill_workspace_size(desc)
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill_workspace_size")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def prefill(q, k, v, seq_lens, positions, q_norm_w=None, k_norm_w=None, rope_theta: float = 0.0, out=None,
            causal: bool = True, eps: float = 1e-6, scale: float = 0.0, out_dtype=None, workspace="auto",
            stream=None, write_k_cache: bool = False):
    """gqa_attn_prefill on torch tensors (device memory); returns out.
    workspace: "auto" allocates one (two-phase path), None selects the
    single-kernel path, or a uint8 device tensor.  With write_k_cache, k
    receives the post-prologue keys (bf16)."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    desc = prefill_desc(q, k, v, out, causal, eps, scale, write_k_cache)
    if isinstance(workspace, str):
        workspace = prefill_workspace(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = gqa_attn_prefill(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(positions), _ptr(q_norm_w),
                          _ptr(k_norm_w), rope_theta, _ptr(out), _ptr(workspace), ws_bytes, _stream_ptr(stream))
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill")
    return out


def prefill_chunk(q, k_cache, v_cache, past_lens, chunk_lens, positions, q_norm_w=None, k_norm_w=None,
                  rope_theta: float = 0.0, out=None, causal: bool = True, eps: float = 1e-6, scale: float = 0.0,
                  out_dtype=None, workspace=None, stream=None, write_k_cache: bool = False):
    """gqa_attn_prefill_chunk on torch tensors (device memory); returns out.
    workspace: a uint8 device tensor, or None to allocate one.  With
    write_k_cache, the chunk's key rows receive their post-prologue values."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    desc = prefill_chunk_desc(q, k_cache, v_cache, out, causal, eps, scale, write_k_cache)
    if workspace is None:
        workspace = prefill_workspace(desc, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = gqa_attn_prefill_chunk(desc, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(past_lens), _ptr(chunk_lens),
                                _ptr(positions), _ptr(q_norm_w), _ptr(k_norm_w), rope_theta, _ptr(out),
                                _ptr(workspace), ws_bytes, _stream_ptr(stream))
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill_chunk")
    return out


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, positions, q_norm_w=None, k_norm_w=None,
                 rope_theta: float = 0.0, out=None, workspace=None, kv_split_tokens: int = 0, eps: float = 1e-6,
                 scale: float = 0.0, out_dtype=None, stream=None, write_new_k: bool = False):
    """gqa_attn_decode_paged on torch tensors: k_pages / v_pages [num_pages, Hkv, bs, 128],
    block_table [B, max_blocks] int32 (max_seq = max_blocks * bs); returns out."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    B, Hq, d = q.shape
    _, Hkv, bs, _ = k_pages.shape
    max_seq = block_table.shape[1] * bs
    desc = GqaDecodeDesc(
        batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_seq=max_seq, in_dtype=_dtype_code(q),
        out_dtype=_dtype_code(out), kv_split_tokens=int(kv_split_tokens),
        q_stride_b=q.stride(0), q_stride_h=q.stride(1),
        k_stride_b=k_pages.stride(0), k_stride_h=k_pages.stride(1), k_stride_s=k_pages.stride(2),
        v_stride_b=v_pages.stride(0), v_stride_h=v_pages.stride(1), v_stride_s=v_pages.stride(2),
        out_stride_b=out.stride(0), out_stride_h=out.stride(1), eps=float(eps), scale=float(scale),
        write_new_k=1 if write_new_k else 0, block_size=bs)
    if workspace is None:
        workspace = decode_workspace(desc, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = gqa_attn_decode_paged(desc, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens),
                               _ptr(positions), _ptr(q_norm_w), _ptr(k_norm_w), rope_theta, _ptr(out),
                               _ptr(workspace), ws_bytes, _stream_ptr(stream))
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_decode_paged")
    return out


def prefill_chunk_paged(q, k_pages, v_pages, block_table, past_lens, chunk_lens, positions, q_norm_w=None,
                        k_norm_w=None, rope_theta: float = 0.0, out=None, causal: bool = True, eps: float = 1e-6,
                        scale: float = 0.0, out_dtype=None, workspace=None, stream=None,
                        write_k_cache: bool = False):
    """gqa_attn_prefill_chunk_paged on torch tensors: k_pages / v_pages [num_pages, Hkv, bs, 128],
    block_table [B, max_blocks] int32 (cache capacity max_blocks * bs); returns out."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    B, Hq, T, d = q.shape
    _, Hkv, bs, _ = k_pages.shape
    desc = GqaPrefillDesc(
        batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_seq=block_table.shape[1] * bs,
        in_dtype=_dtype_code(q), out_dtype=_dtype_code(out), causal=1 if causal else 0,
        q_stride_b=q.stride(0), q_stride_h=q.stride(1), q_stride_s=q.stride(2),
        k_stride_b=k_pages.stride(0), k_stride_h=k_pages.stride(1), k_stride_s=k_pages.stride(2),
        v_stride_b=v_pages.stride(0), v_stride_h=v_pages.stride(1), v_stride_s=v_pages.stride(2),
        out_stride_b=out.stride(0), out_stride_h=out.stride(1), out_stride_s=out.stride(2),
        eps=float(eps), scale=float(scale), max_chunk=T, block_size=bs, write_k_cache=1 if write_k_cache else 0)
    if workspace is None:
        workspace = prefill_workspace(desc, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = gqa_attn_prefill_chunk_paged(desc, _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                      _ptr(past_lens), _ptr(chunk_lens), _ptr(positions), _ptr(q_norm_w),
                                      _ptr(k_norm_w), rope_theta, _ptr(out), _ptr(workspace), ws_bytes,
                                      _stream_ptr(stream))
    if st != GQA_OK:
        raise GqaError(st, "gqa_attn_prefill_chunk_paged")
    return out
