"""Thin Python binding of libpkv (include/pkv.h), one function per entry point.

Argument marshalling only: torch tensors are checked for device, dtype and
layout, their pointers and the current HIP stream are passed to the C ABI,
and a non-zero return raises PkvError with the library's message.  Every
step of the computation runs in the library's kernels; there is no fallback:
if libpkv.so is missing, lib() raises.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_OK = 0
ERRORS = {
    -1: "PKV_ERR_INVALID_ARG", -2: "PKV_ERR_AUTO_SIZE_REFUSED", -3: "PKV_ERR_GEOMETRY",
    -4: "PKV_ERR_WORKSPACE", -5: "PKV_ERR_PAGE_TABLE", -6: "PKV_ERR_LAUNCH", -7: "PKV_ERR_DEVICE",
    -8: "PKV_ERR_LEASE", -9: "PKV_ERR_BUSY", -10: "PKV_ERR_QUARANTINED",
}
KERNELS = {"default": 0, "valu": 1, "mfma": 2}

# every symbol include/pkv.h declares
ABI_VERSION = 5      # PKV_ABI_VERSION of the include/pkv.h this binding follows

EXPORTS = [
    "pkv_last_error", "pkv_abi_version", "pkv_page_bytes", "pkv_pool_create", "pkv_pool_info",
    "pkv_pool_destroy", "pkv_page_table_validate", "pkv_page_table_write",
    "pkv_decode_workspace_bytes", "pkv_decode_attention", "pkv_merge_partials",
    "pkv_append_kv", "pkv_stager_create", "pkv_lease_begin", "pkv_lease_seal",
    "pkv_stager_retire", "pkv_stager_info", "pkv_stager_fail", "pkv_stager_destroy",
    "pkv_admit_create", "pkv_admit_add", "pkv_admit_set_target", "pkv_admit_remove",
    "pkv_admit_step", "pkv_admit_get_counts", "pkv_admit_events", "pkv_admit_destroy",
    "pkv_compact_page_bytes", "pkv_compact_pool_create", "pkv_pool_format",
    "pkv_compact_convert", "pkv_compact_crc", "pkv_plan_tiles", "pkv_decode_attention_rows",
    "pkv_decode_attention_merged", "pkv_decode_attention_runs",
    "pkv_decode_attention_merged_noalloc",
    "pkv_page_table_write_async",
    "pkv_live_create", "pkv_live_add", "pkv_live_set_target", "pkv_live_remove",
    "pkv_live_admission", "pkv_live_step_begin", "pkv_live_layer", "pkv_live_destroy",
    "pkv_live_attach_compact", "pkv_live_publish", "pkv_live_retract",
]


class PkvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code
        self.name = ERRORS.get(code, str(code))


class Geom(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_tokens", ctypes.c_int32)]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("split_tokens", ctypes.c_int32),
                ("slot_offset", ctypes.c_int32)]


class DecodeRun(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("dev_table", ctypes.c_void_p),
                ("pt_stride", ctypes.c_int32), ("dev_ctx_lens", ctypes.c_void_p),
                ("token_count", ctypes.c_int32), ("tile_tokens", ctypes.c_int32),
                ("slot_offset", ctypes.c_int32)]


class AdmitCounts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "steps", "reuse_own", "take_free", "reclaim_borrowed", "reclaim_above_target",
        "reclaim_idle", "shrink_own", "refused", "free_pages")]


class AdmitEvent(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int64), ("kind", ctypes.c_int32), ("context", ctypes.c_int32),
                ("victim", ctypes.c_int32), ("page", ctypes.c_int32), ("logical", ctypes.c_int32)]


ADMIT_KINDS = {1: "reuse_own", 2: "take_free", 3: "reclaim_borrowed", 4: "reclaim_above_target",
               5: "reclaim_idle", 6: "shrink_own", 7: "refused"}
ADMIT_STATUS = {0: "full", 1: "partial", 2: "refused"}


class Lease(ctypes.Structure):
    _fields_ = [("generation", ctypes.c_uint64), ("layer", ctypes.c_int32),
                ("window_begin", ctypes.c_int32), ("buffer", ctypes.c_int32),
                ("staging_layer", ctypes.c_int32), ("dev_table", ctypes.c_void_p),
                ("pt_stride", ctypes.c_int32)]


_lib = None
P = ctypes.c_void_p
I32 = ctypes.c_int32
U64 = ctypes.c_uint64
I32P = ctypes.POINTER(ctypes.c_int32)


def lib():
    """Load libpkv.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_10_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        L.pkv_last_error.restype = ctypes.c_char_p
        L.pkv_last_error.argtypes = []
        L.pkv_abi_version.restype = I32
        L.pkv_abi_version.argtypes = []
        L.pkv_page_bytes.argtypes = [ctypes.POINTER(Geom), ctypes.POINTER(U64)]
        L.pkv_pool_create.argtypes = [ctypes.POINTER(Geom), P, U64, ctypes.POINTER(P)]
        L.pkv_pool_info.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(U64),
                                    ctypes.POINTER(P)]
        L.pkv_pool_destroy.argtypes = [P]
        L.pkv_compact_page_bytes.argtypes = [ctypes.POINTER(Geom), ctypes.POINTER(U64)]
        L.pkv_compact_pool_create.argtypes = [ctypes.POINTER(Geom), P, U64, ctypes.POINTER(P)]
        L.pkv_pool_format.argtypes = [P, I32P]
        L.pkv_compact_convert.argtypes = [P, P, P, P, I32, P, P]
        L.pkv_compact_crc.argtypes = [P, P, I32, P, P]
        L.pkv_page_table_validate.argtypes = [P, I32P, I32P, I32, I32]
        L.pkv_page_table_write.argtypes = [P, I32P, I32P, I32, I32, P, P, P]
        L.pkv_page_table_write_async.argtypes = [P, P, P, I32, I32, P, P, P, P]
        L.pkv_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32,
                                                 ctypes.POINTER(DecodeOpts), ctypes.POINTER(U64)]
        L.pkv_decode_attention.argtypes = [P, I32, P, P, I32, P, I32, I32, I32, I32, I32,
                                           ctypes.c_float, P, P, I32, P, U64,
                                           ctypes.POINTER(DecodeOpts), P]
        L.pkv_merge_partials.argtypes = [P, P, I32, I32, I32, P, P, P]
        L.pkv_decode_attention_merged.argtypes = [P, I32, P, P, I32, P, I32, I32, I32, I32,
                                                  ctypes.c_float, P, P, I32, P, P, P, U64,
                                                  ctypes.POINTER(DecodeOpts), P]
        L.pkv_decode_attention_merged_noalloc.argtypes = [P, I32, P, P, I32, P, I32, I32, I32,
                                                          I32, ctypes.c_float, P, P, I32, P, P,
                                                          ctypes.POINTER(DecodeOpts), P]
        L.pkv_plan_tiles.argtypes = [I32P, I32, I32, I32, I32, I32P, I32P]
        L.pkv_decode_attention_runs.argtypes = [I32, P, I32, I32, ctypes.POINTER(DecodeRun), I32,
                                                ctypes.c_float, P, P, I32, P]
        L.pkv_decode_attention_rows.argtypes = [P, I32, P, P, I32, P, I32, I32, P, I32, I32,
                                                ctypes.c_float, P, P, I32,
                                                ctypes.POINTER(DecodeOpts), P]
        L.pkv_append_kv.argtypes = [P, I32, P, I32, P, I32, P, P, P]
        L.pkv_stager_create.argtypes = [P, P, U64, I32, I32, I32, I32, P, P, P, P,
                                        ctypes.POINTER(P)]
        L.pkv_lease_begin.argtypes = [P, I32, I32P, I32, I32P, I32, I32, ctypes.POINTER(Lease)]
        L.pkv_lease_seal.argtypes = [P, ctypes.POINTER(Lease), I32]
        L.pkv_stager_retire.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.pkv_stager_info.argtypes = [P, ctypes.POINTER(U64), ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(I32), ctypes.POINTER(I32)]
        L.pkv_stager_destroy.argtypes = [P]
        L.pkv_stager_fail.argtypes = [P]
        I64P = ctypes.POINTER(ctypes.c_int64)
        L.pkv_admit_create.argtypes = [ctypes.c_int64, I32, ctypes.POINTER(P)]
        L.pkv_admit_add.argtypes = [P, I32, I32, I32]
        L.pkv_admit_set_target.argtypes = [P, I32, I32, I32]
        L.pkv_admit_remove.argtypes = [P, I32]
        L.pkv_admit_step.argtypes = [P, I32, I32P, I64P, I32P, I32, I32P]
        L.pkv_admit_get_counts.argtypes = [P, ctypes.POINTER(AdmitCounts)]
        L.pkv_admit_events.argtypes = [P, ctypes.POINTER(AdmitEvent), I32, ctypes.POINTER(I32)]
        L.pkv_admit_destroy.argtypes = [P]
        L.pkv_live_create.argtypes = [P, P, P, U64, I32, I32, P, P, P, P, ctypes.POINTER(P)]
        L.pkv_live_add.argtypes = [P, I32, I32, I32]
        L.pkv_live_set_target.argtypes = [P, I32, I32, I32]
        L.pkv_live_remove.argtypes = [P, I32]
        L.pkv_live_admission.argtypes = [P, ctypes.POINTER(P)]
        L.pkv_live_step_begin.argtypes = [P, I32, I32P, I64P, I32P, I32, I32P,
                                          ctypes.POINTER(LiveInfo)]
        L.pkv_live_layer.argtypes = [P, I32, P, P, P, I32, I32, ctypes.c_float, P, P, I32, P, P,
                                     P, U64, ctypes.POINTER(DecodeOpts)]
        L.pkv_live_destroy.argtypes = [P]
        L.pkv_live_attach_compact.argtypes = [P, P, P, U64, I32, P]
        L.pkv_live_publish.argtypes = [P, I32P, I32]
        L.pkv_live_retract.argtypes = [P, I32P, I32]
        for name in EXPORTS[2:]:
            getattr(L, name).restype = ctypes.c_int
        got = L.pkv_abi_version()
        if got != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {got}, this binding is written for "
                               f"{ABI_VERSION}: rebuild the library")
        _lib = L
    return _lib


def _check(rc):
    if rc != PKV_OK:
        raise PkvError(rc, lib().pkv_last_error().decode())


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, dtype=None, name="tensor", need_cuda=True):
    if t is None:
        return None
    if need_cuda and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, need {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _i32_array(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(I32P)


def _opts(kernel, split_tokens, slot_offset=0):
    if kernel in (0, 0.0, None):
        k = 0
    else:
        k = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    return DecodeOpts(k, int(split_tokens or 0), int(slot_offset or 0))


def abi_version():
    return lib().pkv_abi_version()


def page_bytes(num_layers, num_kv_heads, head_dim=256, page_tokens=64):
    out = U64()
    _check(lib().pkv_page_bytes(ctypes.byref(Geom(num_layers, num_kv_heads, head_dim, page_tokens)),
                                ctypes.byref(out)))
    return out.value


class Pool:
    """A page pool over a caller-owned arena (any device tensor; its bytes are
    the arena).  `arena_bytes` defaults to the tensor's size; 0 is refused.
    compact=True makes a pool of compact (E4M3) pages."""

    def __init__(self, arena, num_layers, num_kv_heads, head_dim=256, page_tokens=64,
                 arena_bytes=None, compact=False):
        self.arena = arena                     # keeps the memory alive
        self.geom = Geom(num_layers, num_kv_heads, head_dim, page_tokens)
        nbytes = arena.numel() * arena.element_size() if arena_bytes is None else int(arena_bytes)
        h = P()
        ptr = arena.data_ptr()
        create = lib().pkv_compact_pool_create if compact else lib().pkv_pool_create
        _check(create(ctypes.byref(self.geom), ptr, nbytes, ctypes.byref(h)))
        self.compact = compact
        self.handle = h
        n = ctypes.c_int64()
        pb = U64()
        _check(lib().pkv_pool_info(h, ctypes.byref(n), ctypes.byref(pb), None))
        self.num_pages = n.value
        self.page_bytes = pb.value
        self.num_layers = num_layers
        self.num_kv_heads = num_kv_heads

    def close(self):
        if getattr(self, "handle", None):
            lib().pkv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def page_table_validate(pool, table, ctx_lens):
    """Host-only check of an int32 [batch, pt_stride] table and [batch] lengths."""
    t, tp = _i32_array(table)
    c, cp = _i32_array(ctx_lens)
    if t.ndim != 2 or c.shape != (t.shape[0],):
        raise ValueError("table must be [batch, pt_stride] and ctx_lens [batch]")
    _check(lib().pkv_page_table_validate(pool.handle, tp, cp, t.shape[0], t.shape[1]))


def page_table_write(pool, table, ctx_lens, dev_table, dev_ctx_lens, stream=None):
    """Validate host arrays, then copy them into int32 device tensors."""
    import torch
    t, tp = _i32_array(table)
    c, cp = _i32_array(ctx_lens)
    if t.ndim != 2 or c.shape != (t.shape[0],):
        raise ValueError("table must be [batch, pt_stride] and ctx_lens [batch]")
    if dev_table.numel() < t.size or dev_ctx_lens.numel() < c.size:
        raise ValueError("device table / ctx_lens tensors are too small")
    _check(lib().pkv_page_table_write(pool.handle, tp, cp, t.shape[0], t.shape[1],
                                      _ptr(dev_table, torch.int32, "dev_table"),
                                      _ptr(dev_ctx_lens, torch.int32, "dev_ctx_lens"),
                                      _stream(stream)))


def page_table_write_async(pool, host_table, host_ctx_lens, dev_table, dev_ctx_lens,
                           stream=None, done_event=None):
    """Validate pinned host tensors (int32 [batch, pt_stride] and [batch])
    and queue their copy into the device tensors on `stream` without
    waiting; records done_event (a torch.cuda.Event) after the copy.  The
    host tensors must stay unchanged until done_event completes."""
    import torch
    if not (host_table.is_pinned() and host_ctx_lens.is_pinned()):
        raise ValueError("host_table and host_ctx_lens must be pinned host tensors")
    if host_table.dtype != torch.int32 or host_ctx_lens.dtype != torch.int32:
        raise ValueError("host_table and host_ctx_lens must be int32")
    if host_table.dim() != 2 or not host_table.is_contiguous() or \
            tuple(host_ctx_lens.shape) != (host_table.shape[0],):
        raise ValueError("host_table must be a contiguous [batch, pt_stride], ctx_lens [batch]")
    if dev_table.numel() < host_table.numel() or dev_ctx_lens.numel() < host_ctx_lens.numel():
        raise ValueError("device table / ctx_lens tensors are too small")
    ev = None
    if done_event is not None:
        if done_event.cuda_event == 0:          # torch creates the event on its first record
            done_event.record(torch.cuda.current_stream() if stream is None else stream)
        ev = done_event.cuda_event
    _check(lib().pkv_page_table_write_async(
        pool.handle, host_table.data_ptr(), host_ctx_lens.data_ptr(), host_table.shape[0],
        host_table.shape[1], _ptr(dev_table, torch.int32, "dev_table"),
        _ptr(dev_ctx_lens, torch.int32, "dev_ctx_lens"), _stream(stream), ev))


def decode_workspace_bytes(batch, num_q_heads, token_count, tile_tokens, head_dim=256,
                           kernel=0, split_tokens=0):
    out = U64()
    o = _opts(kernel, split_tokens)
    _check(lib().pkv_decode_workspace_bytes(batch, num_q_heads, head_dim, token_count,
                                            tile_tokens, ctypes.byref(o), ctypes.byref(out)))
    return out.value


def decode_attention(pool, layer, q, dev_table, dev_ctx_lens, token_begin, token_count,
                     tile_tokens, scale, part_out, part_lse, workspace=None, kernel=0,
                     split_tokens=0, stream=None, slot_offset=0):
    """Tile partials of one layer for tokens [token_begin, token_begin + token_count).

    q: bf16 [B, Hq, D]; dev_table: int32 [B, pt_stride] (entry i = logical page
    token_begin/64 + i); part_out: fp32 [B, Hq, num_slots, D]; part_lse: fp32
    [B, Hq, num_slots]."""
    import torch
    B, Hq, D = q.shape
    if part_out.dim() != 4 or part_out.shape[:2] != (B, Hq) or part_out.shape[3] != D:
        raise ValueError("part_out must be [B, Hq, num_slots, D]")
    num_slots = part_out.shape[2]
    if tuple(part_lse.shape) != (B, Hq, num_slots):
        raise ValueError("part_lse must be [B, Hq, num_slots]")
    if dev_table.dim() != 2 or dev_table.shape[0] != B:
        raise ValueError("dev_table must be [B, pt_stride]")
    if dev_table.stride(1) != 1:
        raise ValueError("dev_table rows must be contiguous")
    o = _opts(kernel, split_tokens, slot_offset)
    ws_ptr = _ptr(workspace, None, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pkv_decode_attention(
        pool.handle, int(layer), _ptr(q, torch.bfloat16, "q"),
        dev_table.data_ptr(), int(dev_table.stride(0)),
        _ptr(dev_ctx_lens, torch.int32, "dev_ctx_lens"), B, Hq,
        int(token_begin), int(token_count), int(tile_tokens), float(scale),
        _ptr(part_out, torch.float32, "part_out"), _ptr(part_lse, torch.float32, "part_lse"),
        num_slots, ws_ptr, ws_bytes, ctypes.byref(o), _stream(stream)))


def decode_attention_merged(pool, layer, q, dev_table, dev_ctx_lens, token_count, tile_tokens,
                            scale, part_out, part_lse, out, lse, workspace=None, kernel=0,
                            split_tokens=0, stream=None):
    """Tile partials of the whole history and their merge in one call:
    part_out / part_lse as decode_attention (token_begin 0, every slot), out
    [B, Hq, D] and lse [B, Hq] as merge_partials over them."""
    import torch
    B, Hq, D = q.shape
    if part_out.dim() != 4 or part_out.shape[:2] != (B, Hq) or part_out.shape[3] != D:
        raise ValueError("part_out must be [B, Hq, num_slots, D]")
    num_slots = part_out.shape[2]
    if tuple(part_lse.shape) != (B, Hq, num_slots):
        raise ValueError("part_lse must be [B, Hq, num_slots]")
    if tuple(out.shape) != (B, Hq, D) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out must be [B, Hq, D] and lse [B, Hq]")
    if dev_table.dim() != 2 or dev_table.shape[0] != B or dev_table.stride(1) != 1:
        raise ValueError("dev_table must be [B, pt_stride] with contiguous rows")
    o = _opts(kernel, split_tokens, 0)
    ws_ptr = _ptr(workspace, None, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pkv_decode_attention_merged(
        pool.handle, int(layer), _ptr(q, torch.bfloat16, "q"),
        dev_table.data_ptr(), int(dev_table.stride(0)),
        _ptr(dev_ctx_lens, torch.int32, "dev_ctx_lens"), B, Hq, int(token_count),
        int(tile_tokens), float(scale), _ptr(part_out, torch.float32, "part_out"),
        _ptr(part_lse, torch.float32, "part_lse"), num_slots, _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), ws_ptr, ws_bytes, ctypes.byref(o), _stream(stream)))


def decode_attention_merged_noalloc(pool, layer, q, dev_table, dev_ctx_lens, token_count,
                                    tile_tokens, scale, part_out, part_lse, out, lse, kernel=0,
                                    split_tokens=0, stream=None):
    """decode_attention_merged with the library's static device scratch in
    place of a workspace (pkv_decode_attention_merged_noalloc)."""
    import torch
    B, Hq, D = q.shape
    if part_out.dim() != 4 or part_out.shape[:2] != (B, Hq) or part_out.shape[3] != D:
        raise ValueError("part_out must be [B, Hq, num_slots, D]")
    num_slots = part_out.shape[2]
    if tuple(part_lse.shape) != (B, Hq, num_slots):
        raise ValueError("part_lse must be [B, Hq, num_slots]")
    if tuple(out.shape) != (B, Hq, D) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out must be [B, Hq, D] and lse [B, Hq]")
    if dev_table.dim() != 2 or dev_table.shape[0] != B or dev_table.stride(1) != 1:
        raise ValueError("dev_table must be [B, pt_stride] with contiguous rows")
    o = _opts(kernel, split_tokens, 0)
    _check(lib().pkv_decode_attention_merged_noalloc(
        pool.handle, int(layer), _ptr(q, torch.bfloat16, "q"),
        dev_table.data_ptr(), int(dev_table.stride(0)),
        _ptr(dev_ctx_lens, torch.int32, "dev_ctx_lens"), B, Hq, int(token_count),
        int(tile_tokens), float(scale), _ptr(part_out, torch.float32, "part_out"),
        _ptr(part_lse, torch.float32, "part_lse"), num_slots, _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse"), ctypes.byref(o), _stream(stream)))


STATIC_SCRATCH_BYTES = 16 << 20     # PKV_STATIC_SCRATCH_BYTES


def decode_attention_runs(layer, q, runs, scale, part_out, part_lse, stream=None):
    """Runs decoded in one launch.  runs: a list of (pool, dev_table,
    dev_ctx_lens, token_count, tile_tokens, slot_offset); part_out [B, Hq,
    num_slots, D], part_lse [B, Hq, num_slots]."""
    import torch
    B, Hq, D = q.shape
    if part_out.dim() != 4 or part_out.shape[:2] != (B, Hq) or part_out.shape[3] != D:
        raise ValueError("part_out must be [B, Hq, num_slots, D]")
    num_slots = part_out.shape[2]
    if tuple(part_lse.shape) != (B, Hq, num_slots):
        raise ValueError("part_lse must be [B, Hq, num_slots]")
    arr = (DecodeRun * max(1, len(runs)))()
    for k, (pool, table, ctx, count, tile, off) in enumerate(runs):
        if table.dim() != 2 or table.shape[0] != B or table.stride(1) != 1:
            raise ValueError("each run's table must be [B, pt_stride] with contiguous rows")
        arr[k] = DecodeRun(pool.handle, table.data_ptr(), int(table.stride(0)),
                           _ptr(ctx, torch.int32, "dev_ctx_lens"), int(count), int(tile), int(off))
    _check(lib().pkv_decode_attention_runs(
        int(layer), _ptr(q, torch.bfloat16, "q"), B, Hq, arr, len(runs), float(scale),
        _ptr(part_out, torch.float32, "part_out"), _ptr(part_lse, torch.float32, "part_lse"),
        num_slots, _stream(stream)))


def plan_tiles(ctx_lens, num_kv_heads, work_groups=256, max_tile_tokens=16384):
    """Per-request tile lengths for a batch (host): (int32 [B] tile tokens,
    max tiles per request)."""
    import numpy as np
    c = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    tiles = np.zeros(c.size, dtype=np.int32)
    mx = ctypes.c_int32(0)
    _check(lib().pkv_plan_tiles(c.ctypes.data_as(I32P), int(c.size), int(num_kv_heads),
                                int(work_groups), int(max_tile_tokens),
                                tiles.ctypes.data_as(I32P), ctypes.byref(mx)))
    return tiles, mx.value


def decode_attention_rows(pool, layer, q, dev_table, dev_ctx_lens, dev_row_tiles, max_row_tile,
                          max_tiles, scale, part_out, part_lse, kernel=0, stream=None,
                          slot_offset=0):
    """Partials of tiles of each request's own length (dev_row_tiles: int32
    [B] on the device, from plan_tiles); slots slot_offset .. +max_tiles-1."""
    import torch
    B, Hq, D = q.shape
    if part_out.dim() != 4 or part_out.shape[:2] != (B, Hq) or part_out.shape[3] != D:
        raise ValueError("part_out must be [B, Hq, num_slots, D]")
    num_slots = part_out.shape[2]
    if tuple(part_lse.shape) != (B, Hq, num_slots):
        raise ValueError("part_lse must be [B, Hq, num_slots]")
    if dev_table.dim() != 2 or dev_table.shape[0] != B or dev_table.stride(1) != 1:
        raise ValueError("dev_table must be [B, pt_stride] with contiguous rows")
    if tuple(dev_row_tiles.shape) != (B,):
        raise ValueError("dev_row_tiles must be [B]")
    o = _opts(kernel, 0, slot_offset)
    _check(lib().pkv_decode_attention_rows(
        pool.handle, int(layer), _ptr(q, torch.bfloat16, "q"),
        dev_table.data_ptr(), int(dev_table.stride(0)),
        _ptr(dev_ctx_lens, torch.int32, "dev_ctx_lens"), B, Hq,
        _ptr(dev_row_tiles, torch.int32, "dev_row_tiles"), int(max_row_tile), int(max_tiles),
        float(scale), _ptr(part_out, torch.float32, "part_out"),
        _ptr(part_lse, torch.float32, "part_lse"), num_slots, ctypes.byref(o), _stream(stream)))


def merge_partials(part_out, part_lse, out, lse, stream=None):
    """FP32 LSE merge of every slot of each row: part_out [..., S, D] -> out [..., D]."""
    import torch
    D = part_out.shape[-1]
    S = part_out.shape[-2]
    rows = part_out.numel() // (S * D)
    if part_lse.numel() != rows * S or out.numel() != rows * D or lse.numel() != rows:
        raise ValueError("part_lse / out / lse shapes do not match part_out")
    _check(lib().pkv_merge_partials(
        _ptr(part_out, torch.float32, "part_out"), _ptr(part_lse, torch.float32, "part_lse"),
        rows, S, D, _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse"),
        _stream(stream)))


def append_kv(pool, layer, dev_table, dev_positions, k_new, v_new, stream=None):
    """Write token dev_positions[b] of request b (rows k_new[b], v_new[b]:
    bf16 [B, Hkv, 256]) into its page of `layer`."""
    import torch
    B = k_new.shape[0]
    if tuple(k_new.shape) != (B, pool.num_kv_heads, 256) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new and v_new must be [B, num_kv_heads, 256]")
    if dev_table.dim() != 2 or dev_table.shape[0] != B or dev_table.stride(1) != 1:
        raise ValueError("dev_table must be [B, pt_stride] with contiguous rows")
    if dev_positions.numel() != B:
        raise ValueError("dev_positions must have B entries")
    _check(lib().pkv_append_kv(pool.handle, int(layer), dev_table.data_ptr(),
                               int(dev_table.stride(0)),
                               _ptr(dev_positions, torch.int32, "dev_positions"), B,
                               _ptr(k_new, torch.bfloat16, "k_new"),
                               _ptr(v_new, torch.bfloat16, "v_new"), _stream(stream)))


class Stager:
    """Staged tiles under a lease (pkv_stager_*): history in pinned host
    memory `host_arena` (a pinned tensor in pool layout with `host_layers`
    layers), staging buffers in layer 0 of `staging_pool`."""

    def __init__(self, staging_pool, host_arena, host_layers, max_batch, window_tokens,
                 num_buffers, copy_stream, compute_stream, writeback_stream):
        import torch
        if not host_arena.is_pinned():
            raise ValueError("host_arena must be pinned host memory")
        self.pool = staging_pool
        self.host_arena = host_arena
        self.max_batch = max_batch
        self.window_pages = window_tokens // 64
        self.num_buffers = num_buffers
        self.streams = (copy_stream, compute_stream, writeback_stream)
        self.dev_tables = torch.empty((num_buffers, max_batch, self.window_pages),
                                      dtype=torch.int32, device="cuda")
        h = P()
        _check(lib().pkv_stager_create(
            staging_pool.handle, host_arena.data_ptr(),
            host_arena.numel() * host_arena.element_size(), host_layers, max_batch,
            window_tokens, num_buffers, self.dev_tables.data_ptr(), _stream(copy_stream),
            _stream(compute_stream), _stream(writeback_stream), ctypes.byref(h)))
        self.handle = h

    def begin(self, layer, host_table, host_ctx_lens, window_begin):
        """Queue the window's copy; returns the Lease."""
        t, tp = _i32_array(host_table)
        c, cp = _i32_array(host_ctx_lens)
        lease = Lease()
        _check(lib().pkv_lease_begin(self.handle, int(layer), tp, t.shape[1], cp, t.shape[0],
                                     int(window_begin), ctypes.byref(lease)))
        lease.batch = t.shape[0]
        return lease

    def table(self, lease):
        """The lease's staging page table as a device tensor [batch, pt_stride]."""
        return self.dev_tables[lease.buffer, :lease.batch]

    def seal(self, lease, write_back_tail=False):
        _check(lib().pkv_lease_seal(self.handle, ctypes.byref(lease), int(bool(write_back_tail))))

    def retire(self):
        n = ctypes.c_int64()
        _check(lib().pkv_stager_retire(self.handle, ctypes.byref(n)))
        return n.value

    def info(self):
        g, u, o, q = U64(), ctypes.c_int64(), I32(), I32()
        _check(lib().pkv_stager_info(self.handle, ctypes.byref(g), ctypes.byref(u),
                                     ctypes.byref(o), ctypes.byref(q)))
        return dict(generation=g.value, unretired=u.value, open=bool(o.value),
                    quarantined=bool(q.value))

    def fail(self):
        _check(lib().pkv_stager_fail(self.handle))

    def destroy(self):
        if getattr(self, "handle", None):
            _check(lib().pkv_stager_destroy(self.handle))
            self.handle = None


class Admission:
    """Host-side device page admission (pkv_admit_*)."""

    def __init__(self, num_pages, page_tokens=64, _borrowed=None):
        if _borrowed is not None:          # a planner owned by a live pool: never destroyed here
            self.handle, self.num_pages, self._owned = _borrowed, num_pages, False
            return
        h = P()
        _check(lib().pkv_admit_create(int(num_pages), int(page_tokens), ctypes.byref(h)))
        self.handle = h
        self.num_pages = num_pages
        self._owned = True

    def add(self, ctx, target, burst=0):
        _check(lib().pkv_admit_add(self.handle, ctx, target, burst))

    def set_target(self, ctx, target, burst=0):
        _check(lib().pkv_admit_set_target(self.handle, ctx, target, burst))

    def remove(self, ctx):
        _check(lib().pkv_admit_remove(self.handle, ctx))

    def step(self, ctx_ids, lengths, pt_stride):
        """Returns (table int32 [n, pt_stride], status list of 'full' /
        'partial' / 'refused')."""
        import numpy as np
        ids, idp = _i32_array(ctx_ids)
        ln = np.ascontiguousarray(lengths, dtype=np.int64)
        n = len(ids)
        table = np.empty((max(n, 1), pt_stride), dtype=np.int32)
        status = np.empty(max(n, 1), dtype=np.int32)
        _check(lib().pkv_admit_step(self.handle, n, idp,
                                    ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    table.ctypes.data_as(I32P), pt_stride,
                                    status.ctypes.data_as(I32P)))
        return table[:n], [ADMIT_STATUS[int(x)] for x in status[:n]]

    def counts(self):
        c = AdmitCounts()
        _check(lib().pkv_admit_get_counts(self.handle, ctypes.byref(c)))
        return {n: getattr(c, n) for n, _ in AdmitCounts._fields_}

    def events(self):
        out = []
        buf = (AdmitEvent * 256)()
        while True:
            n = I32()
            _check(lib().pkv_admit_events(self.handle, buf, 256, ctypes.byref(n)))
            out += [dict(step=e.step, kind=ADMIT_KINDS[e.kind], context=e.context,
                         victim=e.victim, page=e.page, logical=e.logical) for e in buf[:n.value]]
            if n.value < 256:
                return out

    def close(self):
        if getattr(self, "handle", None) and getattr(self, "_owned", True):
            lib().pkv_admit_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LiveInfo(ctypes.Structure):
    _fields_ = [("copied_in_pages", ctypes.c_int64), ("staged_pages", ctypes.c_int64),
                ("refused", ctypes.c_int32), ("resident_pages", ctypes.c_int32),
                ("compact_staged_pages", ctypes.c_int64)]


class Live:
    """The live pool (pkv_live_*): histories in the pinned host tensor
    `host_arena` (pool layout, the pool's layers), device pages of `pool`
    admitted per step, the rest staged into `stage_pool` (its layers are the
    staging buffers), one decode over a composed table per layer."""

    def __init__(self, pool, stage_pool, host_arena, max_batch, pt_stride, copy_stream,
                 compute_stream, writeback_stream):
        import torch
        if not host_arena.is_pinned():
            raise ValueError("host_arena must be pinned host memory")
        self.pool, self.stage_pool, self.host_arena = pool, stage_pool, host_arena
        self.max_batch, self.pt_stride = max_batch, pt_stride
        self.streams = (copy_stream, compute_stream, writeback_stream)
        self.dev_state = torch.full((max_batch * (pt_stride + 2),), -1, dtype=torch.int32,
                                    device="cuda")
        h = P()
        _check(lib().pkv_live_create(pool.handle, stage_pool.handle, host_arena.data_ptr(),
                                     host_arena.numel() * host_arena.element_size(), max_batch,
                                     pt_stride, self.dev_state.data_ptr(), _stream(copy_stream),
                                     _stream(compute_stream), _stream(writeback_stream),
                                     ctypes.byref(h)))
        self.handle = h
        a = P()
        _check(lib().pkv_live_admission(self.handle, ctypes.byref(a)))
        self.admission = Admission(pool.num_pages, _borrowed=a)

    def add(self, ctx, target, burst=0):
        _check(lib().pkv_live_add(self.handle, ctx, target, burst))

    def set_target(self, ctx, target, burst=0):
        _check(lib().pkv_live_set_target(self.handle, ctx, target, burst))

    def remove(self, ctx):
        _check(lib().pkv_live_remove(self.handle, ctx))

    def begin(self, ctx_ids, lengths, host_rows):
        """Open a step: lengths include the new token; host_rows int32
        [n, stride] host pages.  Returns (status list, info dict)."""
        import numpy as np
        ids, idp = _i32_array(ctx_ids)
        ln = np.ascontiguousarray(lengths, dtype=np.int64)
        hr, hp = _i32_array(host_rows)
        n = len(ids)
        if hr.shape[0] != n:
            raise ValueError("host_rows must have one row per context")
        status = np.empty(max(n, 1), dtype=np.int32)
        info = LiveInfo()
        _check(lib().pkv_live_step_begin(self.handle, n, idp,
                                         ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), hp,
                                         hr.shape[1], status.ctypes.data_as(I32P),
                                         ctypes.byref(info)))
        return ([ADMIT_STATUS[int(x)] for x in status[:n]],
                {k: getattr(info, k) for k, _ in LiveInfo._fields_})

    def layer(self, layer, q, k_new, v_new, tile_tokens, scale, part_out, part_lse, out, lse,
              workspace=None, split_tokens=0):
        import torch
        n, Hq, D = q.shape
        num_slots = part_out.shape[2]
        if tuple(part_out.shape) != (n, Hq, num_slots, D) or tuple(part_lse.shape) != (n, Hq, num_slots):
            raise ValueError("part_out must be [n, Hq, num_slots, D] and part_lse [n, Hq, num_slots]")
        if tuple(out.shape) != (n, Hq, D) or tuple(lse.shape) != (n, Hq):
            raise ValueError("out must be [n, Hq, D] and lse [n, Hq]")
        if k_new.shape[0] != n or v_new.shape != k_new.shape:
            raise ValueError("k_new and v_new must be [n, Hkv, D]")
        o = _opts(0, split_tokens, 0)
        ws_ptr = _ptr(workspace, None, "workspace") if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        _check(lib().pkv_live_layer(self.handle, int(layer), _ptr(q, torch.bfloat16, "q"),
                                    _ptr(k_new, torch.bfloat16, "k_new"),
                                    _ptr(v_new, torch.bfloat16, "v_new"), Hq, int(tile_tokens),
                                    float(scale), _ptr(part_out, torch.float32, "part_out"),
                                    _ptr(part_lse, torch.float32, "part_lse"), num_slots,
                                    _ptr(out, torch.float32, "out"),
                                    _ptr(lse, torch.float32, "lse"), ws_ptr, ws_bytes,
                                    ctypes.byref(o)))

    def attach_compact(self, cstage_pool, compact_host, compact_tile_tokens):
        """Compact older pages: `compact_host` (pinned) holds every host
        page's compact copy in the layout of a compact pool of the host's
        pages; `cstage_pool` (E4M3) stages them, its layers the buffers."""
        import torch
        if not compact_host.is_pinned():
            raise ValueError("compact_host must be pinned host memory")
        dev_cstate = torch.full((self.max_batch * (self.pt_stride + 1),), -1,
                                dtype=torch.int32, device="cuda")
        _check(lib().pkv_live_attach_compact(self.handle, cstage_pool.handle,
                                             compact_host.data_ptr(),
                                             compact_host.numel() * compact_host.element_size(),
                                             int(compact_tile_tokens), dev_cstate.data_ptr()))
        # the runtime now addresses these: keep them alive with it
        self.cstage_pool, self.compact_host, self.dev_cstate = cstage_pool, compact_host, dev_cstate
        self.compact_tile_tokens = int(compact_tile_tokens)

    def publish(self, host_pages):
        a, p = _i32_array(host_pages)
        _check(lib().pkv_live_publish(self.handle, p, len(a)))

    def retract(self, host_pages):
        a, p = _i32_array(host_pages)
        _check(lib().pkv_live_retract(self.handle, p, len(a)))

    def compact_table(self, n):
        """The open step's compact-run table and lengths (device)."""
        t = self.dev_cstate[:self.max_batch * self.pt_stride].view(self.max_batch, self.pt_stride)
        lens = self.dev_cstate[self.max_batch * self.pt_stride:]
        return t[:n], lens[:n]

    def table(self, n):
        """The open step's composed table, lengths and positions (device)."""
        t = self.dev_state[:self.max_batch * self.pt_stride].view(self.max_batch, self.pt_stride)
        lens = self.dev_state[self.max_batch * self.pt_stride:][:self.max_batch]
        return t[:n], lens[:n]

    def destroy(self):
        if getattr(self, "handle", None):
            _check(lib().pkv_live_destroy(self.handle))
            self.handle = None


def pool_format(pool):
    f = I32()
    _check(lib().pkv_pool_format(pool.handle, ctypes.byref(f)))
    return {0: "bf16", 1: "e4m3"}[f.value]


def compact_page_bytes(num_layers, num_kv_heads, head_dim=256, page_tokens=64):
    g = Geom(num_layers, num_kv_heads, head_dim, page_tokens)
    out = U64()
    _check(lib().pkv_compact_page_bytes(ctypes.byref(g), ctypes.byref(out)))
    return out.value


def compact_convert(exact, compact, src_pages, dst_pages, crc, stream=None):
    """Convert exact pages src_pages[i] into compact pages dst_pages[i] and
    write each compact page's CRC-32 into crc[i].  src_pages, dst_pages:
    device int32 [n]; crc: device int32 [n] (the CRC's 32 bits)."""
    import torch
    n = src_pages.numel()
    if dst_pages.numel() != n or crc.numel() != n:
        raise ValueError("src_pages, dst_pages and crc must have the same length")
    _check(lib().pkv_compact_convert(
        exact.handle, compact.handle, _ptr(src_pages, torch.int32, "src_pages"),
        _ptr(dst_pages, torch.int32, "dst_pages"), n, _ptr(crc, torch.int32, "crc"),
        _stream(stream)))


def compact_crc(compact, pages, crc, stream=None):
    """CRC-32 of compact pages already written: crc[i] for pages[i]."""
    import torch
    n = pages.numel()
    if crc.numel() != n:
        raise ValueError("pages and crc must have the same length")
    _check(lib().pkv_compact_crc(compact.handle, _ptr(pages, torch.int32, "pages"), n,
                                 _ptr(crc, torch.int32, "crc"), _stream(stream)))
