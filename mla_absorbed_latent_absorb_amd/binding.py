"""Thin Python binding of libmla_absorb.so (the C ABI in include/mla_absorb.h).

Argument marshalling only: each function checks the torch tensors it is given
(device, dtype, shape, contiguity), passes their data pointers and the current
HIP stream to the C function of the same name, and raises MlaError with the
library's message on a non-zero status.  Every step of the decode runs in the
library's HIP kernels; there is no fallback path.  PyTorch provides device
memory and streams only.
"""

import ctypes
import os

import torch

from . import build as _build

MLA_DTYPE_BF16 = 0
MLA_DTYPE_FP8_E4M3 = 1

_STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_MISSING_DIM", 3: "MLA_ERR_UNSUPPORTED",
           4: "MLA_ERR_BAD_LENGTH", 5: "MLA_ERR_BUFFER", 6: "MLA_ERR_ALIGN", 7: "MLA_ERR_HIP"}

EXPORTED = ["mla_last_error", "mla_version", "mla_kv_cache_bytes", "mla_decode_kv_read_bytes",
            "mla_absorb_q", "mla_decode_latent", "mla_combine_splits", "mla_expand_v",
            "mla_recommended_splits", "mla_cache_append", "mla_decode_step_fused", "mla_naive_workspace_bytes",
            "mla_naive_decode", "mla_prefill_latent", "mla_combine_expand_v", "mla_decode_latent_noalloc",
            "mla_plan_decode_splits", "mla_decode_latent_planned", "mla_combine_splits_planned",
            "mla_combine_expand_v_planned"]


class MlaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class MlaDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("kv_lora_rank", ctypes.c_int32), ("qk_rope_head_dim", ctypes.c_int32),
                ("qk_nope_head_dim", ctypes.c_int32), ("v_head_dim", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class MlaCache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("kv", ctypes.c_void_p), ("pe", ctypes.c_void_p),
                ("kv_stride", ctypes.c_int64), ("pe_stride", ctypes.c_int64),
                ("token_scale", ctypes.c_void_p), ("seq_stride", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32)]


_lib = None


def library_path():
    return _build.LIB_PATH


def load():
    """Load libmla_absorb.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m mla_absorbed_latent_absorb_amd.build "
                           "or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    st = ctypes.c_int
    D = ctypes.POINTER(MlaDims)
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_version.restype = ctypes.c_char_p
    lib.mla_version.argtypes = []
    lib.mla_kv_cache_bytes.restype = st
    lib.mla_kv_cache_bytes.argtypes = [D, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_decode_kv_read_bytes.restype = st
    lib.mla_decode_kv_read_bytes.argtypes = [D, ctypes.c_int32, P, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_absorb_q.restype = st
    lib.mla_absorb_q.argtypes = [D, P, P, P, P]
    lib.mla_decode_latent.restype = st
    lib.mla_decode_latent.argtypes = [D, ctypes.POINTER(MlaCache), P, P, P, ctypes.c_int32, ctypes.c_int32,
                                      P, P, P, P, P]
    lib.mla_decode_latent_noalloc.restype = st
    lib.mla_decode_latent_noalloc.argtypes = [D, ctypes.POINTER(MlaCache), P, P, P, ctypes.c_int32, ctypes.c_int32,
                                              P, P, P]
    lib.mla_plan_decode_splits.restype = st
    lib.mla_plan_decode_splits.argtypes = [D, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P]
    lib.mla_decode_latent_planned.restype = st
    lib.mla_decode_latent_planned.argtypes = [D, ctypes.POINTER(MlaCache), P, P, P, ctypes.c_int32, P,
                                              ctypes.c_int32, P, P, P]
    lib.mla_combine_splits_planned.restype = st
    lib.mla_combine_splits_planned.argtypes = [D, P, P, P, ctypes.c_int32, P, P, P]
    lib.mla_combine_expand_v_planned.restype = st
    lib.mla_combine_expand_v_planned.argtypes = [D, P, P, P, ctypes.c_int32, P, P, P, P, P]
    lib.mla_combine_splits.restype = st
    lib.mla_combine_splits.argtypes = [D, P, P, ctypes.c_int32, P, P, P]
    lib.mla_combine_expand_v.restype = st
    lib.mla_combine_expand_v.argtypes = [D, P, P, ctypes.c_int32, P, P, P, P, P]
    lib.mla_expand_v.restype = st
    lib.mla_expand_v.argtypes = [D, P, P, P, P]
    lib.mla_cache_append.restype = st
    lib.mla_cache_append.argtypes = [D, ctypes.POINTER(MlaCache), P, ctypes.c_int64, P, ctypes.c_int32,
                                     ctypes.c_float, P]
    lib.mla_decode_step_fused.restype = st
    lib.mla_decode_step_fused.argtypes = [D, ctypes.POINTER(MlaCache), P, P, P, P, P, ctypes.c_int32, P, P, P, P]
    lib.mla_naive_workspace_bytes.restype = st
    lib.mla_naive_workspace_bytes.argtypes = [D, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_naive_decode.restype = st
    lib.mla_naive_decode.argtypes = [D, ctypes.POINTER(MlaCache), P, P, P, P, P, ctypes.c_int32, P, ctypes.c_size_t,
                                     P, P]
    lib.mla_prefill_latent.restype = st
    lib.mla_prefill_latent.argtypes = [D, ctypes.POINTER(MlaCache), P, P, P, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, P, P, P, P, P]
    lib.mla_recommended_splits.restype = ctypes.c_int32
    lib.mla_recommended_splits.argtypes = [D, ctypes.c_int32, ctypes.c_int32]
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise MlaError(status, load().mla_last_error().decode())


def dims(batch, num_heads, softmax_scale, kv_lora_rank=512, qk_rope_head_dim=64, qk_nope_head_dim=128,
         v_head_dim=128):
    return MlaDims(batch, num_heads, kv_lora_rank, qk_rope_head_dim, qk_nope_head_dim, v_head_dim,
                   softmax_scale)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _expect(t, name, dtype, shape, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def mla_version():
    return load().mla_version().decode()


def mla_last_error():
    return load().mla_last_error().decode()


def mla_kv_cache_bytes(d, dtype=MLA_DTYPE_BF16):
    out = ctypes.c_size_t(0)
    _check(load().mla_kv_cache_bytes(ctypes.byref(d), dtype, ctypes.byref(out)))
    return out.value


def mla_decode_kv_read_bytes(d, host_seq_lens, dtype=MLA_DTYPE_BF16):
    lens = (ctypes.c_int32 * len(host_seq_lens))(*[int(x) for x in host_seq_lens])
    out = ctypes.c_size_t(0)
    _check(load().mla_decode_kv_read_bytes(ctypes.byref(d), dtype, ctypes.cast(lens, ctypes.c_void_p),
                                           ctypes.byref(out)))
    return out.value


def mla_recommended_splits(d, max_seq_len, num_cus):
    return int(load().mla_recommended_splits(ctypes.byref(d), int(max_seq_len), int(num_cus)))


def mla_absorb_q(d, q_nope, w_uk, q_lat=None, stream=None):
    """q_lat[b,h,:] = q_nope[b,h,:] . W_UK[h] (bf16 in, fp32 accumulate, bf16 out)."""
    B, H = d.batch, d.num_heads
    _expect(q_nope, "q_nope", torch.bfloat16, (B, H, d.qk_nope_head_dim))
    _expect(w_uk, "w_uk", torch.bfloat16, (H, d.qk_nope_head_dim, d.kv_lora_rank), q_nope.device)
    if q_lat is None:
        q_lat = torch.empty((B, H, d.kv_lora_rank), dtype=torch.bfloat16, device=q_nope.device)
    _expect(q_lat, "q_lat", torch.bfloat16, (B, H, d.kv_lora_rank), q_nope.device)
    _check(load().mla_absorb_q(ctypes.byref(d), _ptr(q_nope), _ptr(w_uk), _ptr(q_lat), _stream(stream)))
    return q_lat


def make_cache(kv_rows, pe_rows, seq_stride=0, block_table=None, block_size=0, token_scale=None):
    """Describe a latent cache given [num_slots, 512] / [num_slots, 64] row views."""
    if kv_rows.dtype == torch.bfloat16:
        dt = MLA_DTYPE_BF16
    elif kv_rows.dtype == torch.uint8:
        dt = MLA_DTYPE_FP8_E4M3
    else:
        raise TypeError(f"cache rows must be bfloat16 or uint8 (E4M3 codes), got {kv_rows.dtype}")
    if pe_rows.dtype != kv_rows.dtype:
        raise TypeError("kv and pe rows must share a dtype")
    for name, t in (("kv_rows", kv_rows), ("pe_rows", pe_rows)):
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be a 2-D view with unit element stride")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    mb = 0
    if block_table is not None:
        _expect(block_table, "block_table", torch.int32, None, kv_rows.device)
        mb = block_table.shape[1]
    if token_scale is not None:
        _expect(token_scale, "token_scale", torch.float32, None, kv_rows.device)
    c = MlaCache(dt, kv_rows.data_ptr(), pe_rows.data_ptr(), kv_rows.stride(0), pe_rows.stride(0),
                 None if token_scale is None else token_scale.data_ptr(), int(seq_stride),
                 None if block_table is None else block_table.data_ptr(), int(block_size), int(mb))
    c._keep = (kv_rows, pe_rows, block_table, token_scale)
    return c


def mla_decode_latent(d, cache, q_lat, q_pe, seq_lens, max_seq_len, num_splits=1, o_part=None, lse_part=None,
                      o_lat=None, lse=None, stream=None):
    """Latent attention of one decode step.  num_splits == 1 returns (o_lat, lse);
    num_splits > 1 returns the split partials (o_part, lse_part)."""
    B, H = d.batch, d.num_heads
    dev = q_lat.device
    _expect(q_lat, "q_lat", torch.bfloat16, (B, H, d.kv_lora_rank))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, H, d.qk_rope_head_dim), dev)
    _expect(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if num_splits == 1:
        if o_lat is None:
            o_lat = torch.empty((B, H, d.kv_lora_rank), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        _expect(o_lat, "o_lat", torch.bfloat16, (B, H, d.kv_lora_rank), dev)
        _expect(lse, "lse", torch.float32, (B, H), dev)
    else:
        if o_part is None:
            o_part = torch.empty((B, num_splits, H, d.kv_lora_rank), dtype=torch.bfloat16, device=dev)
        if lse_part is None:
            lse_part = torch.empty((B, num_splits, H), dtype=torch.float32, device=dev)
        _expect(o_part, "o_part", torch.bfloat16, (B, num_splits, H, d.kv_lora_rank), dev)
        _expect(lse_part, "lse_part", torch.float32, (B, num_splits, H), dev)
    _check(load().mla_decode_latent(ctypes.byref(d), ctypes.byref(cache), _ptr(q_lat), _ptr(q_pe), _ptr(seq_lens),
                                    int(max_seq_len), int(num_splits),
                                    _ptr(o_part) if num_splits > 1 else None,
                                    _ptr(lse_part) if num_splits > 1 else None,
                                    _ptr(o_lat) if num_splits == 1 else None,
                                    _ptr(lse) if num_splits == 1 else None, _stream(stream)))
    return (o_lat, lse) if num_splits == 1 else (o_part, lse_part)


def mla_decode_latent_noalloc(d, cache, q_lat, q_pe, seq_lens, max_seq_len, num_splits, o_lat, lse, stream=None):
    """Split-KV latent attention and merge with the partials in the library's
    device scratch: writes o_lat [B, H, 512] bf16 and lse [B, H] fp32, which
    the caller provides (nothing is allocated here or in the library)."""
    B, H = d.batch, d.num_heads
    dev = q_lat.device
    _expect(q_lat, "q_lat", torch.bfloat16, (B, H, d.kv_lora_rank))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, H, d.qk_rope_head_dim), dev)
    _expect(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _expect(o_lat, "o_lat", torch.bfloat16, (B, H, d.kv_lora_rank), dev)
    _expect(lse, "lse", torch.float32, (B, H), dev)
    _check(load().mla_decode_latent_noalloc(ctypes.byref(d), ctypes.byref(cache), _ptr(q_lat), _ptr(q_pe),
                                            _ptr(seq_lens), int(max_seq_len), int(num_splits), _ptr(o_lat), _ptr(lse),
                                            _stream(stream)))
    return o_lat, lse


class SplitPlan:
    """A length-aware split plan (mla_plan_decode_splits) on the host and its
    device copy: items [n, 4] (sequence, first tile, tile count, partial row)
    in launch order and seq_first [B + 1] int32."""

    def __init__(self, items, seq_first, device):
        self.items_host, self.seq_first_host = items, seq_first
        self.num_items = int(items.shape[0])
        self.items = items.to(device)
        self.seq_first = seq_first.to(device)


def mla_plan_decode_splits(d, host_seq_lens, max_seq_len, num_cus, device=None):
    """Plan on the host from host lengths; with `device`, also copy it there."""
    B = d.batch
    lens = torch.as_tensor([int(v) for v in host_seq_lens], dtype=torch.int32)
    if lens.numel() != B:
        raise ValueError(f"host_seq_lens must have {B} entries")
    cap = B + 12 * int(num_cus)  # enough for every budget the planner compares
    items = torch.empty((cap, 4), dtype=torch.int32)
    first = torch.empty((B + 1,), dtype=torch.int32)
    n = ctypes.c_int32(0)
    _check(load().mla_plan_decode_splits(ctypes.byref(d), ctypes.c_void_p(lens.data_ptr()), int(max_seq_len),
                                         int(num_cus), cap, ctypes.c_void_p(items.data_ptr()),
                                         ctypes.c_void_p(first.data_ptr()), ctypes.byref(n)))
    items = items[:n.value].clone()
    if device is None:
        return items, first
    return SplitPlan(items, first, device)


def mla_decode_latent_planned(d, cache, q_lat, q_pe, seq_lens, max_seq_len, plan, o_part=None, lse_part=None,
                              stream=None):
    """Latent attention over the items of a SplitPlan -> partials
    (o_part [n, H, 512] bf16, lse_part [n, H] fp32)."""
    B, H, n = d.batch, d.num_heads, plan.num_items
    dev = q_lat.device
    _expect(q_lat, "q_lat", torch.bfloat16, (B, H, d.kv_lora_rank))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, H, d.qk_rope_head_dim), dev)
    _expect(seq_lens, "seq_lens", torch.int32, (B,), dev)
    _expect(plan.items, "plan.items", torch.int32, (n, 4), dev)
    if o_part is None:
        o_part = torch.empty((n, H, d.kv_lora_rank), dtype=torch.bfloat16, device=dev)
    if lse_part is None:
        lse_part = torch.empty((n, H), dtype=torch.float32, device=dev)
    _expect(o_part, "o_part", torch.bfloat16, (n, H, d.kv_lora_rank), dev)
    _expect(lse_part, "lse_part", torch.float32, (n, H), dev)
    _check(load().mla_decode_latent_planned(ctypes.byref(d), ctypes.byref(cache), _ptr(q_lat), _ptr(q_pe),
                                            _ptr(seq_lens), int(max_seq_len), _ptr(plan.items), n, _ptr(o_part),
                                            _ptr(lse_part), _stream(stream)))
    return o_part, lse_part


def mla_combine_splits_planned(d, o_part, lse_part, plan, o_lat=None, lse=None, stream=None):
    """Merge planned partials per sequence -> (o_lat bf16, lse fp32)."""
    B, H, n = d.batch, d.num_heads, plan.num_items
    dev = o_part.device
    _expect(o_part, "o_part", torch.bfloat16, (n, H, d.kv_lora_rank))
    _expect(lse_part, "lse_part", torch.float32, (n, H), dev)
    _expect(plan.seq_first, "plan.seq_first", torch.int32, (B + 1,), dev)
    if o_lat is None:
        o_lat = torch.empty((B, H, d.kv_lora_rank), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _expect(o_lat, "o_lat", torch.bfloat16, (B, H, d.kv_lora_rank), dev)
    _expect(lse, "lse", torch.float32, (B, H), dev)
    _check(load().mla_combine_splits_planned(ctypes.byref(d), _ptr(o_part), _ptr(lse_part), _ptr(plan.seq_first), n,
                                             _ptr(o_lat), _ptr(lse), _stream(stream)))
    return o_lat, lse


def mla_combine_expand_v_planned(d, o_part, lse_part, plan, w_uv, out=None, o_lat=None, lse=None, stream=None):
    """Planned merge + value absorption in one launch -> out (bf16 [B, H, 128])."""
    B, H, n = d.batch, d.num_heads, plan.num_items
    dev = o_part.device
    _expect(o_part, "o_part", torch.bfloat16, (n, H, d.kv_lora_rank))
    _expect(lse_part, "lse_part", torch.float32, (n, H), dev)
    _expect(plan.seq_first, "plan.seq_first", torch.int32, (B + 1,), dev)
    _expect(w_uv, "w_uv", torch.bfloat16, (H, d.v_head_dim, d.kv_lora_rank), dev)
    if out is None:
        out = torch.empty((B, H, d.v_head_dim), dtype=torch.bfloat16, device=dev)
    _expect(out, "out", torch.bfloat16, (B, H, d.v_head_dim), dev)
    if o_lat is not None:
        _expect(o_lat, "o_lat", torch.bfloat16, (B, H, d.kv_lora_rank), dev)
    if lse is not None:
        _expect(lse, "lse", torch.float32, (B, H), dev)
    _check(load().mla_combine_expand_v_planned(ctypes.byref(d), _ptr(o_part), _ptr(lse_part), _ptr(plan.seq_first),
                                               n, _ptr(w_uv), _ptr(out), _ptr(o_lat) if o_lat is not None else None,
                                               _ptr(lse) if lse is not None else None, _stream(stream)))
    return out


def mla_prefill_latent(d, cache, q_lat, q_pe, q_start, max_seq_len, num_splits=1, o_part=None, lse_part=None,
                       o_lat=None, lse=None, stream=None):
    """Causal latent attention of a prefill chunk: q_lat [B, L, H, 512],
    q_pe [B, L, H, 64], q_start [B] int32.  num_splits == 1 returns
    (o_lat [B, L, H, 512], lse [B, L, H]); num_splits > 1 returns the partials
    (o_part [B*L, P, H, 512], lse_part [B*L, P, H])."""
    B, H = d.batch, d.num_heads
    dev = q_lat.device
    if q_lat.dim() != 4:
        raise ValueError("q_lat must be [B, L, H, 512]")
    L = q_lat.shape[1]
    _expect(q_lat, "q_lat", torch.bfloat16, (B, L, H, d.kv_lora_rank))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, L, H, d.qk_rope_head_dim), dev)
    _expect(q_start, "q_start", torch.int32, (B,), dev)
    if num_splits == 1:
        if o_lat is None:
            o_lat = torch.empty((B, L, H, d.kv_lora_rank), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, L, H), dtype=torch.float32, device=dev)
        _expect(o_lat, "o_lat", torch.bfloat16, (B, L, H, d.kv_lora_rank), dev)
        _expect(lse, "lse", torch.float32, (B, L, H), dev)
    else:
        if o_part is None:
            o_part = torch.empty((B * L, num_splits, H, d.kv_lora_rank), dtype=torch.bfloat16, device=dev)
        if lse_part is None:
            lse_part = torch.empty((B * L, num_splits, H), dtype=torch.float32, device=dev)
        _expect(o_part, "o_part", torch.bfloat16, (B * L, num_splits, H, d.kv_lora_rank), dev)
        _expect(lse_part, "lse_part", torch.float32, (B * L, num_splits, H), dev)
    _check(load().mla_prefill_latent(ctypes.byref(d), ctypes.byref(cache), _ptr(q_lat), _ptr(q_pe), _ptr(q_start),
                                     int(L), int(max_seq_len), int(num_splits),
                                     _ptr(o_part) if num_splits > 1 else None,
                                     _ptr(lse_part) if num_splits > 1 else None,
                                     _ptr(o_lat) if num_splits == 1 else None,
                                     _ptr(lse) if num_splits == 1 else None, _stream(stream)))
    return (o_lat, lse) if num_splits == 1 else (o_part, lse_part)


def mla_combine_splits(d, o_part, lse_part, o_lat=None, lse=None, stream=None):
    """Log-sum-exp merge of split partials -> (o_lat bf16, lse fp32)."""
    B, H = d.batch, d.num_heads
    P = o_part.shape[1]
    dev = o_part.device
    _expect(o_part, "o_part", torch.bfloat16, (B, P, H, d.kv_lora_rank))
    _expect(lse_part, "lse_part", torch.float32, (B, P, H), dev)
    if o_lat is None:
        o_lat = torch.empty((B, H, d.kv_lora_rank), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    _expect(o_lat, "o_lat", torch.bfloat16, (B, H, d.kv_lora_rank), dev)
    _expect(lse, "lse", torch.float32, (B, H), dev)
    _check(load().mla_combine_splits(ctypes.byref(d), _ptr(o_part), _ptr(lse_part), int(P), _ptr(o_lat), _ptr(lse),
                                     _stream(stream)))
    return o_lat, lse


def mla_expand_v(d, o_lat, w_uv, out=None, stream=None):
    """out[b,h,:] = W_UV[h] . o_lat[b,h,:] (bf16 in, fp32 accumulate, bf16 out)."""
    B, H = d.batch, d.num_heads
    _expect(o_lat, "o_lat", torch.bfloat16, (B, H, d.kv_lora_rank))
    _expect(w_uv, "w_uv", torch.bfloat16, (H, d.v_head_dim, d.kv_lora_rank), o_lat.device)
    if out is None:
        out = torch.empty((B, H, d.v_head_dim), dtype=torch.bfloat16, device=o_lat.device)
    _expect(out, "out", torch.bfloat16, (B, H, d.v_head_dim), o_lat.device)
    _check(load().mla_expand_v(ctypes.byref(d), _ptr(o_lat), _ptr(w_uv), _ptr(out), _stream(stream)))
    return out


def mla_combine_expand_v(d, o_part, lse_part, w_uv, out=None, o_lat=None, lse=None, stream=None):
    """Split merge + value absorption in one launch -> out (bf16 [B, H, 128]).
    o_lat / lse are written when given (else not at all)."""
    B, H = d.batch, d.num_heads
    P = o_part.shape[1]
    dev = o_part.device
    _expect(o_part, "o_part", torch.bfloat16, (B, P, H, d.kv_lora_rank))
    _expect(lse_part, "lse_part", torch.float32, (B, P, H), dev)
    _expect(w_uv, "w_uv", torch.bfloat16, (H, d.v_head_dim, d.kv_lora_rank), dev)
    if out is None:
        out = torch.empty((B, H, d.v_head_dim), dtype=torch.bfloat16, device=dev)
    _expect(out, "out", torch.bfloat16, (B, H, d.v_head_dim), dev)
    if o_lat is not None:
        _expect(o_lat, "o_lat", torch.bfloat16, (B, H, d.kv_lora_rank), dev)
    if lse is not None:
        _expect(lse, "lse", torch.float32, (B, H), dev)
    _check(load().mla_combine_expand_v(ctypes.byref(d), _ptr(o_part), _ptr(lse_part), int(P), _ptr(w_uv), _ptr(out),
                                       _ptr(o_lat) if o_lat is not None else None,
                                       _ptr(lse) if lse is not None else None, _stream(stream)))
    return out


def mla_decode_step_fused(d, cache, q_nope, q_pe, w_uk, w_uv, seq_lens, max_seq_len, out=None, o_lat=None,
                          lse=None, want_latent=False, stream=None):
    """The three decode stages in one launch (short contexts).  Returns out,
    or (out, o_lat, lse) with want_latent=True."""
    B, H = d.batch, d.num_heads
    dev = q_nope.device
    _expect(q_nope, "q_nope", torch.bfloat16, (B, H, d.qk_nope_head_dim))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, H, d.qk_rope_head_dim), dev)
    _expect(w_uk, "w_uk", torch.bfloat16, (H, d.qk_nope_head_dim, d.kv_lora_rank), dev)
    _expect(w_uv, "w_uv", torch.bfloat16, (H, d.v_head_dim, d.kv_lora_rank), dev)
    _expect(seq_lens, "seq_lens", torch.int32, (B,), dev)
    if out is None:
        out = torch.empty((B, H, d.v_head_dim), dtype=torch.bfloat16, device=dev)
    _expect(out, "out", torch.bfloat16, (B, H, d.v_head_dim), dev)
    if want_latent:
        if o_lat is None:
            o_lat = torch.empty((B, H, d.kv_lora_rank), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if o_lat is not None:
        _expect(o_lat, "o_lat", torch.bfloat16, (B, H, d.kv_lora_rank), dev)
    if lse is not None:
        _expect(lse, "lse", torch.float32, (B, H), dev)
    _check(load().mla_decode_step_fused(ctypes.byref(d), ctypes.byref(cache), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk),
                                        _ptr(w_uv), _ptr(seq_lens), int(max_seq_len), _ptr(out), _ptr(o_lat),
                                        _ptr(lse), _stream(stream)))
    return (out, o_lat, lse) if want_latent else out


def mla_naive_workspace_bytes(d, max_seq_len):
    out = ctypes.c_size_t(0)
    _check(load().mla_naive_workspace_bytes(ctypes.byref(d), int(max_seq_len), ctypes.byref(out)))
    return out.value


def mla_naive_decode(d, cache, q_nope, q_pe, w_uk, w_uv, seq_lens, max_seq_len, workspace=None, out=None,
                     stream=None):
    """Expand-every-step decode (baseline).  workspace: a uint8 device tensor of
    at least mla_naive_workspace_bytes bytes (allocated here if None)."""
    B, H = d.batch, d.num_heads
    dev = q_nope.device
    _expect(q_nope, "q_nope", torch.bfloat16, (B, H, d.qk_nope_head_dim))
    _expect(q_pe, "q_pe", torch.bfloat16, (B, H, d.qk_rope_head_dim), dev)
    _expect(w_uk, "w_uk", torch.bfloat16, (H, d.qk_nope_head_dim, d.kv_lora_rank), dev)
    _expect(w_uv, "w_uv", torch.bfloat16, (H, d.v_head_dim, d.kv_lora_rank), dev)
    _expect(seq_lens, "seq_lens", torch.int32, (B,), dev)
    need = mla_naive_workspace_bytes(d, max_seq_len)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    if out is None:
        out = torch.empty((B, H, d.v_head_dim), dtype=torch.bfloat16, device=dev)
    _expect(out, "out", torch.bfloat16, (B, H, d.v_head_dim), dev)
    _check(load().mla_naive_decode(ctypes.byref(d), ctypes.byref(cache), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk),
                                   _ptr(w_uv), _ptr(seq_lens), int(max_seq_len), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))
    return out


def mla_cache_append(d, cache, kv_in, positions, rope_base=10000.0, stream=None):
    """Write kv_in [B, n, >= 576] bf16 (latent row + unrotated RoPE key per
    token) into the cache at positions[b] + j; the cache's buffers are
    written in place.  Rows may be a view with any row stride (multiple of 8
    elements) as long as element and token strides nest."""
    B = d.batch
    if not isinstance(kv_in, torch.Tensor) or kv_in.dtype != torch.bfloat16:
        raise TypeError("kv_in must be a bfloat16 torch.Tensor")
    if kv_in.dim() != 3 or kv_in.shape[0] != B or kv_in.shape[2] < d.kv_lora_rank + d.qk_rope_head_dim:
        raise ValueError(f"kv_in must have shape ({B}, n, >= {d.kv_lora_rank + d.qk_rope_head_dim}), "
                         f"got {tuple(kv_in.shape)}")
    n = kv_in.shape[1]
    row = kv_in.stride(1)
    if kv_in.stride(2) != 1 or (B > 1 and n > 0 and kv_in.stride(0) != n * row):
        raise ValueError("kv_in rows must have unit element stride and sequences must follow each other")
    if not kv_in.is_cuda:
        raise ValueError("kv_in must be a device tensor")
    _expect(positions, "positions", torch.int32, (B,), kv_in.device)
    _check(load().mla_cache_append(ctypes.byref(d), ctypes.byref(cache), _ptr(kv_in), int(row), _ptr(positions),
                                   int(n), float(rope_base), _stream(stream)))


class DecodeStep:
    """One absorbed decode step with preallocated buffers (so a timed or
    captured step allocates nothing): mla_absorb_q, mla_decode_latent, then
    mla_expand_v (one split) or mla_combine_expand_v (split-KV).  With
    keep_latent the merged o_lat and lse are written too (the step's output is
    `out` either way)."""

    def __init__(self, d, cache, seq_lens, max_seq_len, num_splits, device, keep_latent=True):
        B, H = d.batch, d.num_heads
        self.keep_latent = bool(keep_latent)
        self.d, self.cache, self.seq_lens = d, cache, seq_lens
        self.max_seq_len, self.num_splits = int(max_seq_len), int(num_splits)
        bf, f32 = torch.bfloat16, torch.float32
        self.q_lat = torch.empty((B, H, d.kv_lora_rank), dtype=bf, device=device)
        self.o_lat = torch.empty((B, H, d.kv_lora_rank), dtype=bf, device=device)
        self.lse = torch.empty((B, H), dtype=f32, device=device)
        self.out = torch.empty((B, H, d.v_head_dim), dtype=bf, device=device)
        if self.num_splits > 1:
            self.o_part = torch.empty((B, self.num_splits, H, d.kv_lora_rank), dtype=bf, device=device)
            self.lse_part = torch.empty((B, self.num_splits, H), dtype=f32, device=device)
        else:
            self.o_part = self.lse_part = None

    def attend(self, q_pe, stream=None):
        """Latent attention (+ combine) given self.q_lat."""
        if self.num_splits > 1:
            mla_decode_latent(self.d, self.cache, self.q_lat, q_pe, self.seq_lens, self.max_seq_len,
                              self.num_splits, o_part=self.o_part, lse_part=self.lse_part, stream=stream)
            mla_combine_splits(self.d, self.o_part, self.lse_part, o_lat=self.o_lat, lse=self.lse, stream=stream)
        else:
            mla_decode_latent(self.d, self.cache, self.q_lat, q_pe, self.seq_lens, self.max_seq_len, 1,
                              o_lat=self.o_lat, lse=self.lse, stream=stream)

    def decode(self, q_pe, stream=None):
        """mla_decode_latent alone: partials (split-KV) or o_lat / lse."""
        if self.num_splits > 1:
            mla_decode_latent(self.d, self.cache, self.q_lat, q_pe, self.seq_lens, self.max_seq_len,
                              self.num_splits, o_part=self.o_part, lse_part=self.lse_part, stream=stream)
        else:
            mla_decode_latent(self.d, self.cache, self.q_lat, q_pe, self.seq_lens, self.max_seq_len, 1,
                              o_lat=self.o_lat, lse=self.lse, stream=stream)

    def finish(self, w_uv, stream=None):
        """What follows mla_decode_latent: the merge (if split) and W_UV."""
        if self.num_splits > 1:
            keep = self.keep_latent
            mla_combine_expand_v(self.d, self.o_part, self.lse_part, w_uv, out=self.out,
                                 o_lat=self.o_lat if keep else None, lse=self.lse if keep else None,
                                 stream=stream)
        else:
            mla_expand_v(self.d, self.o_lat, w_uv, out=self.out, stream=stream)

    def __call__(self, q_nope, q_pe, w_uk, w_uv, stream=None):
        mla_absorb_q(self.d, q_nope, w_uk, q_lat=self.q_lat, stream=stream)
        self.decode(q_pe, stream=stream)
        self.finish(w_uv, stream=stream)
        return self.out


class PlannedDecodeStep:
    """One absorbed decode step over a length-aware split plan, with
    preallocated buffers: mla_absorb_q, mla_decode_latent_planned, then
    mla_combine_expand_v_planned.  Same interface as DecodeStep."""

    def __init__(self, d, cache, seq_lens, max_seq_len, plan, device, keep_latent=True):
        B, H = d.batch, d.num_heads
        self.keep_latent = bool(keep_latent)
        self.d, self.cache, self.seq_lens, self.plan = d, cache, seq_lens, plan
        self.max_seq_len = int(max_seq_len)
        self.num_splits = plan.num_items
        bf, f32 = torch.bfloat16, torch.float32
        self.q_lat = torch.empty((B, H, d.kv_lora_rank), dtype=bf, device=device)
        self.o_lat = torch.empty((B, H, d.kv_lora_rank), dtype=bf, device=device)
        self.lse = torch.empty((B, H), dtype=f32, device=device)
        self.out = torch.empty((B, H, d.v_head_dim), dtype=bf, device=device)
        self.o_part = torch.empty((plan.num_items, H, d.kv_lora_rank), dtype=bf, device=device)
        self.lse_part = torch.empty((plan.num_items, H), dtype=f32, device=device)

    def decode(self, q_pe, stream=None):
        mla_decode_latent_planned(self.d, self.cache, self.q_lat, q_pe, self.seq_lens, self.max_seq_len, self.plan,
                                  o_part=self.o_part, lse_part=self.lse_part, stream=stream)

    def finish(self, w_uv, stream=None):
        keep = self.keep_latent
        mla_combine_expand_v_planned(self.d, self.o_part, self.lse_part, self.plan, w_uv, out=self.out,
                                     o_lat=self.o_lat if keep else None, lse=self.lse if keep else None,
                                     stream=stream)

    def __call__(self, q_nope, q_pe, w_uk, w_uv, stream=None):
        mla_absorb_q(self.d, q_nope, w_uk, q_lat=self.q_lat, stream=stream)
        self.decode(q_pe, stream=stream)
        self.finish(w_uv, stream=stream)
        return self.out
