"""Python binding of libpda.so: paged grouped-query decode attention on MI355X.

Argument marshalling only.  Every function has the name and the argument
order of the C entry point it calls (``include/pda.h``); every step of the
computation runs in the library's gfx950 kernels.  Device buffers are passed
as torch tensors (or raw integer addresses); torch provides device memory and
streams and nothing else.  A status other than PDA_OK raises ``PdaError`` (a
RuntimeError carrying the status code and the library's detail text).  If the
compiled library is missing the import fails with RuntimeError; there is no
fallback of any kind, as for the AstrAI page's wrappers ("CUDA Kernels",
section "Python Wrappers", which raise when their .so is absent).
"""
from __future__ import annotations

import ctypes
import os

# torch ships its own copy of the HIP runtime (loaded by file name, under the
# same SONAME as the system's).  Loading torch first makes libpda.so bind to
# that very runtime instance, so the device memory and streams torch hands out
# are valid inside the library; loaded the other way round the process would
# hold two HIP runtimes and the library would see no device.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpda.so")

if not os.path.exists(LIB_PATH):
    raise RuntimeError(
        f"{LIB_PATH} is missing: build it with `python paged_gqa_decode_pda_amd/build.py` "
        "(or __graft_entry__.build()); there is no fallback path")

_lib = ctypes.CDLL(LIB_PATH)

PDA_OK = 0
STATUS_NAMES = ["PDA_OK", "PDA_ERR_NULL", "PDA_ERR_DIMS", "PDA_ERR_GQA", "PDA_ERR_HEAD_DIM",
                "PDA_ERR_MAX_SEQS", "PDA_ERR_ALIGN", "PDA_ERR_WORKSPACE", "PDA_ERR_HIP"]
for _i, _n in enumerate(STATUS_NAMES):
    globals()[_n] = _i

EXPORTED = ["pda_dims_validate", "pda_state_bytes", "pda_state_offsets", "pda_blocks_per_split",
            "pda_workspace_bytes", "pda_paged_strides", "pda_scratch_pool_strides",
            "pda_scratch_pool_v_offset", "pda_create", "pda_destroy", "pda_begin_step",
            "pda_step_tile", "pda_finalize", "pda_decode", "pda_decode_noalloc", "pda_decode_masked",
            "pda_prefill_workspace_bytes", "pda_prefill", "pda_rope", "pda_rope_append_kv",
            "pda_debug_time_attention",
            "pda_status_string", "pda_last_error"]


class pda_dims(ctypes.Structure):
    _fields_ = [("max_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("tile_capacity", ctypes.c_int32)]


class pda_strides(ctypes.Structure):
    _fields_ = [("blk", ctypes.c_int64), ("tok", ctypes.c_int64), ("kvh", ctypes.c_int64)]

    def astuple(self):
        return (self.blk, self.tok, self.kvh)


class PdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {detail}")


_P = ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_PD = ctypes.POINTER(pda_dims)


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("pda_dims_validate", ctypes.c_int, _PD)
_sig("pda_state_bytes", _sz, _PD)
_sig("pda_state_offsets", ctypes.c_int, _PD, ctypes.POINTER(_sz))
_sig("pda_blocks_per_split", _i32, _PD, _i32)
_sig("pda_workspace_bytes", _sz, _PD, _i32)
_sig("pda_paged_strides", pda_strides, _PD)
_sig("pda_scratch_pool_strides", pda_strides, _PD)
_sig("pda_scratch_pool_v_offset", _i64, _PD)
_sig("pda_create", ctypes.c_int, _PD, _P, _P, _sz, _i32, ctypes.POINTER(_P))
_sig("pda_destroy", None, _P)
_sig("pda_begin_step", ctypes.c_int, _P, _i32, _P)
_sig("pda_step_tile", ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _i32, _i32, pda_strides, _P)
_sig("pda_finalize", ctypes.c_int, _P, _P, _i32, _P)
_sig("pda_decode", ctypes.c_int, _PD, _P, _P, _P, _P, _P, _P, _i32, _i32, pda_strides, _P, _sz,
     _P, _i32, _P)
_sig("pda_decode_noalloc", ctypes.c_int, _PD, _P, _P, _P, _P, _P, _P, _i32, _i32, pda_strides, _P,
     _i32, _P)
_sig("pda_decode_masked", ctypes.c_int, _PD, _P, _P, _P, _P, _P, _P, _i32, _i32, pda_strides, _P,
     _i64, _P, _sz, _P, _i32, _P)
_sig("pda_prefill_workspace_bytes", _sz, _PD, _i32, _i32)
_sig("pda_prefill", ctypes.c_int, _PD, _i32, _P, _P, _P, _P, _P, _P, _i32, _i32, pda_strides, _i32,
     _P, _i64, _i64, _P, _sz, _P, _i32, _i32, _P)
_sig("pda_rope", ctypes.c_int, _P, _P, _i64, _i32, _i32, _P, _P, _i32, _P, _P)
_sig("pda_rope_append_kv", ctypes.c_int, _PD, _P, _P, _i64, _P, _P, _P, _P, _i32, _P, _P, _P,
     pda_strides, _P)
_sig("pda_debug_time_attention", ctypes.c_int, _P, _P)
_sig("pda_status_string", ctypes.c_char_p, ctypes.c_int)
_sig("pda_last_error", ctypes.c_char_p)


def _dims(d) -> pda_dims:
    if isinstance(d, pda_dims):
        return d
    if isinstance(d, dict):
        return pda_dims(**d)
    return pda_dims(*d)


def _strides(s) -> pda_strides:
    if isinstance(s, pda_strides):
        return s
    return pda_strides(*[int(x) for x in s])


def _addr(x):
    """Device address of a tensor (its data_ptr) or an integer address; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _nbytes(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        raise TypeError("pass the byte count explicitly with an integer address")
    return x.numel() * x.element_size()


def _stream(s):
    """hipStream_t handle: None -> torch's current stream on the current device."""
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int):
    if status != PDA_OK:
        raise PdaError(status, _lib.pda_last_error().decode())


def pda_status_string(status: int) -> str:
    return _lib.pda_status_string(status).decode()


def pda_last_error() -> str:
    return _lib.pda_last_error().decode()


def pda_dims_validate(dims) -> None:
    d = _dims(dims)
    _check(_lib.pda_dims_validate(ctypes.byref(d)))


def pda_state_bytes(dims) -> int:
    d = _dims(dims)
    return _lib.pda_state_bytes(ctypes.byref(d))


def pda_state_offsets(dims):
    d = _dims(dims)
    off = (_sz * 3)()
    _check(_lib.pda_state_offsets(ctypes.byref(d), off))
    return tuple(off)


def pda_blocks_per_split(dims, blocks_per_split: int = 0) -> int:
    d = _dims(dims)
    return _lib.pda_blocks_per_split(ctypes.byref(d), blocks_per_split)


def pda_workspace_bytes(dims, blocks_per_split: int = 0) -> int:
    d = _dims(dims)
    return _lib.pda_workspace_bytes(ctypes.byref(d), blocks_per_split)


def pda_paged_strides(dims):
    d = _dims(dims)
    return _lib.pda_paged_strides(ctypes.byref(d)).astuple()


def pda_scratch_pool_strides(dims):
    d = _dims(dims)
    return _lib.pda_scratch_pool_strides(ctypes.byref(d)).astuple()


def pda_scratch_pool_v_offset(dims) -> int:
    d = _dims(dims)
    return _lib.pda_scratch_pool_v_offset(ctypes.byref(d))


def pda_create(dims, state, workspace, blocks_per_split: int = 0, workspace_bytes=None) -> int:
    """Returns the plan handle (an integer host address)."""
    d = _dims(dims)
    out = _P()
    nb = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    _check(_lib.pda_create(ctypes.byref(d), _addr(state), _addr(workspace), nb, blocks_per_split,
                           ctypes.byref(out)))
    return out.value


def pda_destroy(plan) -> None:
    _lib.pda_destroy(plan)


def pda_begin_step(plan, num_seqs: int, stream=None) -> None:
    _check(_lib.pda_begin_step(plan, num_seqs, _stream(stream)))


def pda_step_tile(plan, q, k_pool, v_pool, tile_blocks, tile_block_counts, last_block_valid,
                  last_block_valid_default: int, num_seqs: int, strides, stream=None) -> None:
    _check(_lib.pda_step_tile(plan, _addr(q), _addr(k_pool), _addr(v_pool), _addr(tile_blocks),
                              _addr(tile_block_counts), _addr(last_block_valid),
                              last_block_valid_default, num_seqs, _strides(strides),
                              _stream(stream)))


def pda_finalize(plan, out, num_seqs: int, stream=None) -> None:
    _check(_lib.pda_finalize(plan, _addr(out), num_seqs, _stream(stream)))


def pda_debug_time_attention(before, after) -> None:
    """Arms the next attention launch on this thread to record two events
    around its attention kernel.  Events are torch.cuda.Event objects that
    have been recorded once (so that they exist), raw hipEvent_t integers, or
    None, None to disarm."""
    def handle(e):
        if e is None or isinstance(e, int):
            return e
        return e.cuda_event
    _check(_lib.pda_debug_time_attention(handle(before), handle(after)))


def pda_decode(dims, q, k_pool, v_pool, block_tables, block_counts, last_block_valid,
               last_block_valid_default: int, num_seqs: int, strides, workspace, out,
               blocks_per_split: int = 0, stream=None, workspace_bytes=None) -> None:
    d = _dims(dims)
    nb = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    _check(_lib.pda_decode(ctypes.byref(d), _addr(q), _addr(k_pool), _addr(v_pool),
                           _addr(block_tables), _addr(block_counts), _addr(last_block_valid),
                           last_block_valid_default, num_seqs, _strides(strides), _addr(workspace),
                           nb, _addr(out), blocks_per_split, _stream(stream)))


# Bytes of the library's built-in scratch for pda_decode_noalloc (per GPU).
PDA_NOALLOC_SCRATCH_BYTES = 64 << 20


def pda_decode_noalloc(dims, q, k_pool, v_pool, block_tables, block_counts, last_block_valid,
                       last_block_valid_default: int, num_seqs: int, strides, out,
                       blocks_per_split: int = 0, stream=None) -> None:
    """pda_decode with the library's built-in scratch instead of a workspace:
    allocates nothing (for callers that cannot allocate device memory)."""
    d = _dims(dims)
    _check(_lib.pda_decode_noalloc(ctypes.byref(d), _addr(q), _addr(k_pool), _addr(v_pool),
                                   _addr(block_tables), _addr(block_counts),
                                   _addr(last_block_valid), last_block_valid_default, num_seqs,
                                   _strides(strides), _addr(out), blocks_per_split,
                                   _stream(stream)))


def pda_decode_masked(dims, q, k_pool, v_pool, block_tables, block_counts, last_block_valid,
                      last_block_valid_default: int, num_seqs: int, strides, kv_mask,
                      mask_stride: int, workspace, out, blocks_per_split: int = 0, stream=None,
                      workspace_bytes=None) -> None:
    d = _dims(dims)
    nb = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    _check(_lib.pda_decode_masked(ctypes.byref(d), _addr(q), _addr(k_pool), _addr(v_pool),
                                  _addr(block_tables), _addr(block_counts),
                                  _addr(last_block_valid), last_block_valid_default, num_seqs,
                                  _strides(strides), _addr(kv_mask), int(mask_stride),
                                  _addr(workspace), nb, _addr(out), blocks_per_split,
                                  _stream(stream)))


def pda_prefill_workspace_bytes(dims, q_len: int, blocks_per_split: int = 0) -> int:
    d = _dims(dims)
    return _lib.pda_prefill_workspace_bytes(ctypes.byref(d), q_len, blocks_per_split)


def pda_prefill(dims, q_len: int, q, k_pool, v_pool, block_tables, block_counts, last_block_valid,
                last_block_valid_default: int, num_seqs: int, strides, causal: bool, kv_mask,
                mask_seq_stride: int, mask_q_stride: int, workspace, out,
                blocks_per_split: int = 0, rows_per_wave: int = 0, stream=None,
                workspace_bytes=None) -> None:
    d = _dims(dims)
    nb = _nbytes(workspace) if workspace_bytes is None else int(workspace_bytes)
    _check(_lib.pda_prefill(ctypes.byref(d), int(q_len), _addr(q), _addr(k_pool), _addr(v_pool),
                            _addr(block_tables), _addr(block_counts), _addr(last_block_valid),
                            last_block_valid_default, num_seqs, _strides(strides),
                            1 if causal else 0, _addr(kv_mask), int(mask_seq_stride),
                            int(mask_q_stride), _addr(workspace), nb, _addr(out),
                            blocks_per_split, rows_per_wave, _stream(stream)))


def pda_rope(x, out, num_tokens: int, num_heads: int, head_dim: int, cos_table, sin_table,
             max_positions: int, positions, stream=None) -> None:
    _check(_lib.pda_rope(_addr(x), _addr(out), int(num_tokens), num_heads, head_dim,
                         _addr(cos_table), _addr(sin_table), int(max_positions), _addr(positions),
                         _stream(stream)))


def pda_rope_append_kv(dims, k_new, v_new, num_tokens: int, token_seq, positions, cos_table,
                       sin_table, max_positions: int, block_tables, k_pool, v_pool, strides,
                       stream=None) -> None:
    d = _dims(dims)
    _check(_lib.pda_rope_append_kv(ctypes.byref(d), _addr(k_new), _addr(v_new), int(num_tokens),
                                   _addr(token_seq), _addr(positions), _addr(cos_table),
                                   _addr(sin_table), int(max_positions), _addr(block_tables),
                                   _addr(k_pool), _addr(v_pool), _strides(strides),
                                   _stream(stream)))


def apply_rotary_emb(x, freqs_cis, positions, out=None, stream=None):
    """Rotary embedding in the pages' calling convention: x [batch, seq_len,
    n_heads, head_dim] bf16 (blhd), freqs_cis = (cos, sin) fp32 tables
    [max_positions, head_dim / 2], positions int32 [batch, seq_len] (each
    token's position).  Returns out (a new tensor unless given; out=x rotates
    in place).  Argument marshalling only; the rotation runs in the library."""
    import torch
    cos_t, sin_t = freqs_cis
    if x.dim() != 4 or x.dtype != torch.bfloat16 or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("x must be a contiguous bfloat16 device tensor [batch, seq_len, n_heads, head_dim]")
    B, L, H, D = x.shape
    for t in (cos_t, sin_t):
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] * 2 != D or t.device.type != "cuda":
            raise ValueError("cos and sin must be float32 device tensors [max_positions, head_dim / 2]")
    pos = positions.to(device=x.device, dtype=torch.int32).contiguous()
    if pos.numel() != B * L:
        raise ValueError("positions must hold one entry per token")
    own = []
    if out is None:
        out = torch.empty_like(x)
        own.append(out)
    ct, st = cos_t.contiguous(), sin_t.contiguous()
    _use_on_stream(stream, [pos, ct, st] + own)
    pda_rope(x, out, B * L, H, D, ct, st, cos_t.shape[0], pos, stream)
    return out


def _use_on_stream(stream, temporaries):
    """Ordering for a wrapper that computes temporaries with torch ops (on
    torch's current stream) and launches on another stream: that stream
    first waits for the work enqueued so far on the current one, and every
    temporary is marked as used on it, so torch's caching allocator does not
    hand its memory out again before that stream is done with it.  A raw
    integer stream handle carries no such information: the caller orders it."""
    import torch
    if stream is None or isinstance(stream, int):
        return
    cur = torch.cuda.current_stream(stream.device)
    if stream == cur:
        return
    stream.wait_stream(cur)
    for t in temporaries:
        if t is not None:
            t.record_stream(stream)


def _paged_args(q, k_cache, v_cache, block_table, seq_lens):
    """Checks of the pages' wrapper convention and the C-ABI arguments derived
    from it: (dims, strides, block_table, counts, last_valid)."""
    import torch
    B, _, Hq, D = q.shape
    nblk, bs, Hkv, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache must both be [num_blocks, block_size, n_kv_heads, head_dim]")
    for t in (q, k_cache, v_cache):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("q, k_cache and v_cache must be contiguous bfloat16 tensors")
        if t.device.type != "cuda":
            raise ValueError("q, k_cache and v_cache must be device tensors")
    if block_table.device.type != "cuda":
        raise ValueError("block_table must be a device tensor")
    block_table = block_table.to(torch.int32).contiguous()
    cap = block_table.shape[1]
    lens = seq_lens.to(device=block_table.device, dtype=torch.int32)
    counts = ((lens + (bs - 1)) // bs).to(torch.int32).contiguous()
    lastv = torch.where(counts > 0, lens - (counts - 1) * bs, torch.zeros_like(lens)).to(torch.int32).contiguous()
    dims = pda_dims(B, Hq, Hkv, D, bs, cap)
    return dims, pda_paged_strides(dims), block_table, counts, lastv


def attn_paged_prefill(q, k_cache, v_cache, block_table, seq_lens, is_causal: bool = True,
                       mask=None, out=None, workspace=None, blocks_per_split: int = 0,
                       rows_per_wave: int = 0, stream=None):
    """Prefill attention in the pages' wrapper convention: q [batch, q_len,
    n_heads, head_dim] bf16 (blhd), the chunk's keys already in k_cache /
    v_cache [num_blocks, block_size, n_kv_heads, head_dim] as the newest q_len
    of seq_lens[b] tokens; is_causal as the pages' switch; mask optional bool
    [batch, kv_len] or [batch, q_len, kv_len] (True = keep).  Returns out
    [batch, q_len, n_heads, head_dim] bf16.  Argument derivation and
    allocation only; the attention runs in the library's kernels."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [batch, q_len, n_heads, head_dim]")
    B, Q, Hq, D = q.shape
    if mask is not None and seq_lens.device.type == "cpu" and seq_lens.numel() and \
            int(seq_lens.max()) > mask.shape[-1]:
        raise ValueError("mask rows are shorter than the longest sequence")
    dims, strides, block_table, counts, lastv = _paged_args(q, k_cache, v_cache, block_table, seq_lens)
    bs = dims.block_size
    own = []
    if out is None:
        out = torch.empty((B, Q, Hq, D), dtype=torch.bfloat16, device=q.device)
        own.append(out)
    if workspace is None:
        nb = pda_prefill_workspace_bytes(dims, Q, blocks_per_split)
        workspace = torch.empty(max(1, (nb + 3) // 4), dtype=torch.float32, device=q.device)
        own.append(workspace)
    m, ss, qs = None, 0, 0
    if mask is not None:
        m = mask.to(device=q.device, dtype=torch.uint8).contiguous()
        if m.dim() == 2 and m.shape[0] == B:
            ss, qs = m.shape[1], 0
        elif m.dim() == 3 and m.shape[0] == B and m.shape[1] == Q:
            ss, qs = m.shape[1] * m.shape[2], m.shape[2]
        else:
            raise ValueError("mask must be [batch, kv_len] or [batch, q_len, kv_len]")
    _use_on_stream(stream, [block_table, counts, lastv, m] + own)
    pda_prefill(dims, Q, q, k_cache, v_cache, block_table, counts, lastv, bs, B, strides,
                is_causal, m, ss, qs, workspace, out, blocks_per_split, rows_per_wave, stream)
    return out


def attn_paged_decode(q, k_cache, v_cache, block_table, seq_lens, mask=None, out=None,
                      workspace=None, blocks_per_split: int = 0, stream=None):
    """Decode attention in the calling convention of the pages' paged decode
    wrapper: q [batch, 1, n_heads, head_dim] bf16 (blhd, one query token),
    k_cache / v_cache [num_blocks, block_size, n_kv_heads, head_dim] bf16
    (block_size 1 = token-granular tables), block_table int32 [batch,
    max_blocks], seq_lens int32 [batch] tokens per sequence, mask optional
    bool [batch, >= max(seq_lens)] (True = keep).  Scale 1/sqrt(head_dim).
    Returns out [batch, 1, n_heads, head_dim] bf16.  Everything runs in the
    library's kernels; this function only derives the C-ABI arguments (page
    counts and last-page valid slots from seq_lens) and allocates the output
    and workspace when they are not given."""
    import torch
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be [batch, 1, n_heads, head_dim]")
    B, _, Hq, D = q.shape
    if mask is not None and seq_lens.device.type == "cpu" and seq_lens.numel() and \
            int(seq_lens.max()) > mask.shape[-1]:
        raise ValueError("mask rows are shorter than the longest sequence")
    dims, strides, block_table, counts, lastv = _paged_args(q, k_cache, v_cache, block_table, seq_lens)
    bs = dims.block_size
    own = []
    if out is None:
        out = torch.empty((B, 1, Hq, D), dtype=torch.bfloat16, device=q.device)
        own.append(out)
    if workspace is None:   # needs no clearing
        workspace = torch.empty(max(1, pda_workspace_bytes(dims, blocks_per_split) // 4),
                                dtype=torch.float32, device=q.device)
        own.append(workspace)
    m = None
    if mask is not None:
        m = mask.to(device=q.device, dtype=torch.uint8).contiguous()
        if m.dim() != 2 or m.shape[0] != B:
            raise ValueError("mask must be [batch, kv_len]")
    _use_on_stream(stream, [block_table, counts, lastv, m] + own)
    if m is None:
        pda_decode(dims, q, k_cache, v_cache, block_table, counts, lastv, bs, B, strides,
                   workspace, out, blocks_per_split, stream)
    else:
        pda_decode_masked(dims, q, k_cache, v_cache, block_table, counts, lastv, bs, B, strides,
                          m, m.shape[1], workspace, out, blocks_per_split, stream)
    return out
