"""Host-side checks of the C-ABI library: it loads, exports every declared
symbol, and validates arguments before enqueuing anything (CPU only; no
call here reaches a kernel)."""
import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import paged_gqa_decode_pda_amd as pda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pda.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(pda_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(pda.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", pda.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", dyn, re.M), f"{n} not a defined text symbol"
    assert sorted(pda.EXPORTED) == names


def test_header_compiles_as_c():
    src = f'#include "{HEADER}"\nint main(void){{pda_dims d={{1,1,1,8,1,1}};return (int)pda_dims_validate(&d);}}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", "-"],
                       input=src, text=True, capture_output=True)
    assert r.returncode == 0, r.stderr


def dims(**kw):
    base = dict(max_seqs=4, num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                tile_capacity=32)
    base.update(kw)
    return pda.pda_dims(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), pda.PDA_OK),
    (dict(num_q_heads=6, num_kv_heads=4), pda.PDA_ERR_GQA),
    (dict(head_dim=264), pda.PDA_ERR_HEAD_DIM),
    (dict(head_dim=60), pda.PDA_ERR_HEAD_DIM),
    (dict(head_dim=256), pda.PDA_OK),
    (dict(head_dim=8), pda.PDA_OK),
    (dict(max_seqs=0), pda.PDA_ERR_DIMS),
    (dict(num_kv_heads=0), pda.PDA_ERR_DIMS),
    (dict(block_size=0), pda.PDA_ERR_DIMS),
    (dict(tile_capacity=0), pda.PDA_ERR_DIMS),
    (dict(tile_capacity=1 << 21, block_size=16), pda.PDA_ERR_DIMS),
    (dict(block_size=1), pda.PDA_OK),
    (dict(num_q_heads=64, num_kv_heads=2), pda.PDA_OK),
])
def test_dims_validate(kw, status):
    if status == pda.PDA_OK:
        pda.pda_dims_validate(dims(**kw))
    else:
        with pytest.raises(pda.PdaError) as e:
            pda.pda_dims_validate(dims(**kw))
        assert e.value.status == status
        assert pda.pda_last_error()


def test_page_constants_golden():
    g = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    with pytest.raises(pda.PdaError):
        pda.pda_dims_validate(dims(head_dim=g["max_head_dim"]["value"] + 8))
    pda.pda_dims_validate(dims(head_dim=g["max_head_dim"]["value"]))


def test_strides_golden():
    g = json.load(open(os.path.join(GOLDEN, "strides.json")))
    for c in g["cases"]:
        d = pda.pda_dims(1, c["num_kv_heads"], c["num_kv_heads"], c["head_dim"], c["block_size"], 1)
        if c["layout"] == "paged":
            assert list(pda.pda_paged_strides(d)) == c["strides"]
        else:
            assert list(pda.pda_scratch_pool_strides(d)) == c["strides"]
            assert pda.pda_scratch_pool_v_offset(d) == c["v_offset"]


def test_state_and_workspace_sizes():
    d = dims()
    rows = 4 * 8
    assert pda.pda_state_bytes(d) == rows * 4 * (2 + 64)
    assert pda.pda_state_offsets(d) == (0, rows * 4, 2 * rows * 4)
    for bps in (1, 3, 32, 100):
        eff = min(bps, 32)
        assert pda.pda_blocks_per_split(d, bps) == eff
        # 256 bytes of control words, the arrival counters, then the
        # partials: one slot per split of a sequence of up to ceil(32 / bps)
        # splits; (m, l) pairs padded to 16 bytes
        slots = -(-32 // eff)
        ml = -(-(rows * slots * 2 * 4) // 16) * 16
        arrive = 4 * 2 * 8    # one 64-bit arrival counter per (sequence, kv head)
        assert pda.pda_workspace_bytes(d, bps) == 256 + arrive + ml + rows * slots * 64 * 4
    auto = pda.pda_blocks_per_split(d, 0)
    assert 1 <= auto <= 32
    assert pda.pda_workspace_bytes(d, 0) >= pda.pda_workspace_bytes(d, auto)
    big = dims(tile_capacity=4096)
    assert pda.pda_blocks_per_split(big, 0) >= 4096 // 256
    # the library's split: about 256 tokens, 352 above head dim 128 (at most 256 splits)
    for D, bs, want in ((128, 16, 16), (64, 8, 32), (256, 16, 22), (256, 32, 11), (200, 16, 22)):
        assert pda.pda_blocks_per_split(dims(head_dim=D, block_size=bs, tile_capacity=512), 0) == want
    assert pda.pda_state_bytes(dims(num_q_heads=6, num_kv_heads=4)) == 0


@pytest.mark.parametrize("max_seqs,hq,hkv,bps", [(1, 9, 3, 1), (3, 5, 5, 3), (1, 1, 1, 7), (7, 3, 1, 2)])
def test_regions_start_16_byte_aligned(max_seqs, hq, hkv, bps):
    """The state's o rows and the workspace's o partials start on 16-byte
    boundaries whatever the row counts (odd q-head counts included): the
    kernels write them 16 bytes at a time."""
    d = dims(max_seqs=max_seqs, num_q_heads=hq, num_kv_heads=hkv, tile_capacity=9)
    rows = max_seqs * hq
    offs = pda.pda_state_offsets(d)
    assert all(o % 16 == 0 for o in offs)
    assert offs[1] >= rows * 4 and offs[2] >= offs[1] + rows * 4
    assert pda.pda_state_bytes(d) == offs[2] + rows * 64 * 4
    slots = -(-9 // bps)
    ml = rows * slots * 2 * 4
    arrive = -(-(max_seqs * hkv * 8) // 16) * 16    # G <= 16: one head chunk per kv head
    assert pda.pda_workspace_bytes(d, bps) == 256 + arrive + (-(-ml // 16) * 16) + rows * slots * 64 * 4


FAKE = 1 << 20          # a 16-byte aligned host-side address that is never dereferenced


def test_decode_validation_before_enqueue():
    d = dims()
    st = (16 * 2 * 64, 2 * 64, 64)
    args = dict(dims=d, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_tables=FAKE, block_counts=FAKE,
                last_block_valid=None, last_block_valid_default=16, num_seqs=4, strides=st,
                workspace=FAKE, out=FAKE, blocks_per_split=0, stream=0,
                workspace_bytes=pda.pda_workspace_bytes(d))
    cases = [
        (dict(q=None), pda.PDA_ERR_NULL),
        (dict(block_counts=None), pda.PDA_ERR_NULL),
        (dict(out=None), pda.PDA_ERR_NULL),
        (dict(q=FAKE + 2), pda.PDA_ERR_ALIGN),
        (dict(k_pool=FAKE + 8), pda.PDA_ERR_ALIGN),
        (dict(block_tables=FAKE + 2), pda.PDA_ERR_ALIGN),
        (dict(out=FAKE + 4), pda.PDA_ERR_ALIGN),
        (dict(strides=(st[0], st[1] + 4, st[2])), pda.PDA_ERR_ALIGN),
        (dict(strides=(-st[0], st[1], st[2])), pda.PDA_ERR_ALIGN),
        (dict(strides=(st[0], 1 << 30, st[2])), pda.PDA_ERR_DIMS),
        (dict(strides=(1 << 32, st[1], st[2])), pda.PDA_ERR_DIMS),
        (dict(strides=((1 << 63) - 8, st[1], st[2])), pda.PDA_ERR_DIMS),
        (dict(strides=(st[0], (1 << 63) - 8, st[2])), pda.PDA_ERR_DIMS),
        (dict(num_seqs=5), pda.PDA_ERR_MAX_SEQS),
        (dict(num_seqs=-1), pda.PDA_ERR_MAX_SEQS),
        (dict(workspace_bytes=16), pda.PDA_ERR_WORKSPACE),
        (dict(workspace=None, workspace_bytes=0), pda.PDA_ERR_WORKSPACE),
        (dict(blocks_per_split=-1), pda.PDA_ERR_DIMS),
        (dict(dims=dims(num_q_heads=6, num_kv_heads=4)), pda.PDA_ERR_GQA),
    ]
    for change, status in cases:
        with pytest.raises(pda.PdaError) as e:
            pda.pda_decode(**{**args, **change})
        assert e.value.status == status, (change, e.value)
    # num_seqs == 0 is a valid no-op that enqueues nothing
    pda.pda_decode(**{**args, "num_seqs": 0})


def test_plan_validation_before_enqueue():
    d = dims()
    ws = pda.pda_workspace_bytes(d)
    with pytest.raises(pda.PdaError) as e:
        pda.pda_create(d, None, FAKE, 0, workspace_bytes=ws)
    assert e.value.status == pda.PDA_ERR_NULL
    with pytest.raises(pda.PdaError) as e:
        pda.pda_create(d, FAKE, FAKE, 0, workspace_bytes=ws - 4)
    assert e.value.status == pda.PDA_ERR_WORKSPACE
    with pytest.raises(pda.PdaError) as e:
        pda.pda_create(d, FAKE + 4, FAKE, 0, workspace_bytes=ws)
    assert e.value.status == pda.PDA_ERR_ALIGN
    plan = pda.pda_create(d, FAKE, FAKE, 0, workspace_bytes=ws)
    try:
        with pytest.raises(pda.PdaError) as e:
            pda.pda_begin_step(plan, 5, stream=0)
        assert e.value.status == pda.PDA_ERR_MAX_SEQS
        st = (16 * 2 * 64, 2 * 64, 64)
        with pytest.raises(pda.PdaError) as e:
            pda.pda_step_tile(plan, FAKE, FAKE, None, FAKE, FAKE, None, 16, 4, st, stream=0)
        assert e.value.status == pda.PDA_ERR_NULL
        with pytest.raises(pda.PdaError) as e:
            pda.pda_step_tile(plan, FAKE, FAKE, FAKE, FAKE, FAKE, None, 16, 9, st, stream=0)
        assert e.value.status == pda.PDA_ERR_MAX_SEQS
        with pytest.raises(pda.PdaError) as e:
            pda.pda_finalize(plan, None, 4, stream=0)
        assert e.value.status == pda.PDA_ERR_NULL
        with pytest.raises(pda.PdaError) as e:
            pda.pda_finalize(plan, FAKE, 5, stream=0)
        assert e.value.status == pda.PDA_ERR_MAX_SEQS
        pda.pda_begin_step(plan, 0, stream=0)
        pda.pda_finalize(plan, FAKE, 0, stream=0)
    finally:
        pda.pda_destroy(plan)


def test_status_strings():
    for i, n in enumerate(pda.STATUS_NAMES):
        assert pda.pda_status_string(i) == n


def test_missing_library_raises(tmp_path):
    """Importing the binding without its library fails loudly; nothing falls back."""
    import shutil
    import sys
    pkg = tmp_path / "paged_gqa_decode_pda_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "paged_gqa_decode_pda_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import paged_gqa_decode_pda_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "RuntimeError" in r.stderr and "missing" in r.stderr


def test_small_blocks_per_split_accepted_on_host():
    """A tiny explicit split size with a long page list passes host checks
    (the work queue has no grid-dimension limit); here it stops at the
    workspace check."""
    d = dims(tile_capacity=1 << 17, block_size=1)
    st = (1 * 2 * 64, 2 * 64, 64)
    with pytest.raises(pda.PdaError) as e:
        pda.pda_decode(d, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4, st, FAKE, FAKE, 1, stream=0,
                       workspace_bytes=16)
    assert e.value.status == pda.PDA_ERR_WORKSPACE


def test_debug_time_attention_arming():
    """The timing hook takes both events or neither; arming and disarming
    touch no device."""
    with pytest.raises(pda.PdaError) as e:
        pda.pda_debug_time_attention(FAKE, None)
    assert e.value.status == pda.PDA_ERR_NULL
    with pytest.raises(pda.PdaError):
        pda.pda_debug_time_attention(None, FAKE)
    pda.pda_debug_time_attention(FAKE, FAKE + 64)
    pda.pda_debug_time_attention(None, None)


def test_decode_masked_validation_before_enqueue():
    """pda_decode_masked rejects a NULL mask and a non-positive row stride
    before anything is enqueued (addresses are never dereferenced)."""
    d = dims()
    common = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, block_tables=FAKE, block_counts=FAKE,
                  last_block_valid=FAKE, last_block_valid_default=16, num_seqs=2,
                  strides=pda.pda_paged_strides(d), workspace=FAKE, out=FAKE,
                  workspace_bytes=pda.pda_workspace_bytes(d), stream=0)
    with pytest.raises(pda.PdaError) as e:
        pda.pda_decode_masked(d, **common, kv_mask=None, mask_stride=64)
    assert e.value.status == pda.PDA_ERR_NULL
    for stride in (0, -5):
        with pytest.raises(pda.PdaError) as e:
            pda.pda_decode_masked(d, **common, kv_mask=FAKE, mask_stride=stride)
        assert e.value.status == pda.PDA_ERR_DIMS
    with pytest.raises(pda.PdaError) as e:   # the ordinary checks still apply
        pda.pda_decode_masked(d, **{**common, "num_seqs": 99}, kv_mask=FAKE, mask_stride=64)
    assert e.value.status == pda.PDA_ERR_MAX_SEQS


def test_attn_paged_decode_rejects_host_tensors():
    """The blhd convenience wrapper refuses host tensors and wrong shapes
    before any library call."""
    import torch
    q = torch.zeros(2, 1, 4, 64, dtype=torch.bfloat16)
    kc = torch.zeros(8, 1, 2, 64, dtype=torch.bfloat16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    lens = torch.tensor([3, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        pda.attn_paged_decode(q, kc, kc, bt, lens)
    with pytest.raises(ValueError):
        pda.attn_paged_decode(q[:, 0], kc, kc, bt, lens)


def test_prefill_workspace_sizes():
    """Split partials of max_seqs * q_len * Hq rows, ceil(cap / bps) slots each,
    (head_dim + 2) floats per slot plus 16 bytes of alignment padding; none
    when one split covers the page list."""
    d = dims()   # 4 seqs, 8 q heads, head_dim 64, block_size 16, capacity 32
    for q_len in (1, 7):
        rows = 4 * q_len * 8
        for bps in (1, 3, 16):
            slots = -(-32 // bps)
            assert pda.pda_prefill_workspace_bytes(d, q_len, bps) == rows * slots * 66 * 4 + 16
        assert pda.pda_prefill_workspace_bytes(d, q_len, 32) == 0
        assert pda.pda_prefill_workspace_bytes(d, q_len, 99) == 0
        # the library's choice never splits below 256 tokens (16 pages here)
        assert pda.pda_prefill_workspace_bytes(d, q_len, 0) == rows * 2 * 66 * 4 + 16
    assert pda.pda_prefill_workspace_bytes(d, 0, 0) == 0
    assert pda.pda_prefill_workspace_bytes(dims(num_q_heads=6, num_kv_heads=4), 4, 0) == 0


def test_prefill_validation_before_enqueue():
    """pda_prefill checks every argument before anything is enqueued
    (addresses are never dereferenced)."""
    d = dims()
    st = (16 * 2 * 64, 2 * 64, 64)
    args = dict(dims=d, q_len=5, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_tables=FAKE,
                block_counts=FAKE, last_block_valid=None, last_block_valid_default=16,
                num_seqs=4, strides=st, causal=True, kv_mask=None, mask_seq_stride=0,
                mask_q_stride=0, workspace=FAKE, out=FAKE, blocks_per_split=0,
                rows_per_wave=0, stream=0, workspace_bytes=pda.pda_prefill_workspace_bytes(d, 5))
    cases = [
        (dict(q=None), pda.PDA_ERR_NULL),
        (dict(out=None), pda.PDA_ERR_NULL),
        (dict(block_tables=None), pda.PDA_ERR_NULL),
        (dict(q=FAKE + 2), pda.PDA_ERR_ALIGN),
        (dict(out=FAKE + 8), pda.PDA_ERR_ALIGN),
        (dict(workspace=FAKE + 4), pda.PDA_ERR_ALIGN),
        (dict(strides=(st[0], st[1] + 4, st[2])), pda.PDA_ERR_ALIGN),
        (dict(q_len=0), pda.PDA_ERR_DIMS),
        (dict(q_len=1 << 23), pda.PDA_ERR_DIMS),
        (dict(rows_per_wave=48), pda.PDA_ERR_DIMS),
        (dict(blocks_per_split=-2), pda.PDA_ERR_DIMS),
        (dict(kv_mask=FAKE, mask_seq_stride=-1), pda.PDA_ERR_DIMS),
        (dict(kv_mask=FAKE, mask_q_stride=-3), pda.PDA_ERR_DIMS),
        (dict(num_seqs=5), pda.PDA_ERR_MAX_SEQS),
        (dict(workspace_bytes=16), pda.PDA_ERR_WORKSPACE),
        (dict(workspace=None, workspace_bytes=0), pda.PDA_ERR_WORKSPACE),
        (dict(dims=dims(num_q_heads=6, num_kv_heads=4)), pda.PDA_ERR_GQA),
        (dict(dims=dims(head_dim=260)), pda.PDA_ERR_HEAD_DIM),
    ]
    for change, status in cases:
        with pytest.raises(pda.PdaError) as e:
            pda.pda_prefill(**{**args, **change})
        assert e.value.status == status, (change, e.value)
    pda.pda_prefill(**{**args, "num_seqs": 0})


def test_attn_paged_prefill_rejects_host_tensors():
    import torch
    q = torch.zeros(2, 3, 4, 64, dtype=torch.bfloat16)
    kc = torch.zeros(8, 1, 2, 64, dtype=torch.bfloat16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    lens = torch.tensor([3, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        pda.attn_paged_prefill(q, kc, kc, bt, lens)
    with pytest.raises(ValueError):
        pda.attn_paged_prefill(q[:, 0], kc, kc, bt, lens)


def test_rope_validation_before_enqueue():
    """pda_rope and pda_rope_append_kv check their arguments before anything
    is enqueued (addresses are never dereferenced)."""
    args = dict(x=FAKE, out=FAKE, num_tokens=4, num_heads=2, head_dim=64, cos_table=FAKE,
                sin_table=FAKE, max_positions=128, positions=FAKE, stream=0)
    cases = [
        (dict(x=None), pda.PDA_ERR_NULL), (dict(out=None), pda.PDA_ERR_NULL),
        (dict(cos_table=None), pda.PDA_ERR_NULL), (dict(positions=None), pda.PDA_ERR_NULL),
        (dict(head_dim=60), pda.PDA_ERR_HEAD_DIM), (dict(head_dim=264), pda.PDA_ERR_HEAD_DIM),
        (dict(num_heads=0), pda.PDA_ERR_DIMS), (dict(num_tokens=-1), pda.PDA_ERR_DIMS),
        (dict(max_positions=0), pda.PDA_ERR_DIMS),
        (dict(x=FAKE + 8), pda.PDA_ERR_ALIGN), (dict(sin_table=FAKE + 4), pda.PDA_ERR_ALIGN),
        (dict(positions=FAKE + 2), pda.PDA_ERR_ALIGN),
    ]
    for change, status in cases:
        with pytest.raises(pda.PdaError) as e:
            pda.pda_rope(**{**args, **change})
        assert e.value.status == status, (change, e.value)
    pda.pda_rope(**{**args, "num_tokens": 0})
    d = dims()
    app = dict(dims=d, k_new=FAKE, v_new=FAKE, num_tokens=3, token_seq=FAKE, positions=FAKE,
               cos_table=FAKE, sin_table=FAKE, max_positions=64, block_tables=FAKE, k_pool=FAKE,
               v_pool=FAKE, strides=pda.pda_paged_strides(d), stream=0)
    cases = [
        (dict(v_new=None), pda.PDA_ERR_NULL), (dict(block_tables=None), pda.PDA_ERR_NULL),
        (dict(k_pool=None), pda.PDA_ERR_NULL), (dict(token_seq=None), pda.PDA_ERR_NULL),
        (dict(v_pool=FAKE + 2), pda.PDA_ERR_ALIGN), (dict(token_seq=FAKE + 1), pda.PDA_ERR_ALIGN),
        (dict(strides=(8, 4, 8)), pda.PDA_ERR_ALIGN),
        (dict(dims=dims(num_q_heads=6, num_kv_heads=4)), pda.PDA_ERR_GQA),
        (dict(num_tokens=-2), pda.PDA_ERR_DIMS),
    ]
    for change, status in cases:
        with pytest.raises(pda.PdaError) as e:
            pda.pda_rope_append_kv(**{**app, **change})
        assert e.value.status == status, (change, e.value)
    pda.pda_rope_append_kv(**{**app, "num_tokens": 0})


def test_decode_noalloc_validation_before_enqueue():
    d = dims()
    st = (16 * 2 * 64, 2 * 64, 64)
    args = dict(dims=d, q=FAKE, k_pool=FAKE, v_pool=FAKE, block_tables=FAKE, block_counts=FAKE,
                last_block_valid=None, last_block_valid_default=16, num_seqs=4, strides=st,
                out=FAKE, blocks_per_split=0, stream=0)
    cases = [
        (dict(q=None), pda.PDA_ERR_NULL),
        (dict(out=None), pda.PDA_ERR_NULL),
        (dict(out=FAKE + 4), pda.PDA_ERR_ALIGN),
        (dict(num_seqs=5), pda.PDA_ERR_MAX_SEQS),
        (dict(blocks_per_split=-1), pda.PDA_ERR_DIMS),
        (dict(dims=dims(num_q_heads=6, num_kv_heads=4)), pda.PDA_ERR_GQA),
    ]
    for change, status in cases:
        with pytest.raises(pda.PdaError) as e:
            pda.pda_decode_noalloc(**{**args, **change})
        assert e.value.status == status, (change, e.value)
    # sizes whose partials exceed the built-in scratch are refused with the limit named
    big = dims(max_seqs=4096, tile_capacity=4096)
    need = pda.pda_workspace_bytes(big, 0)
    assert need > pda.PDA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(pda.PdaError) as e:
        pda.pda_decode_noalloc(**{**args, "dims": big})
    assert e.value.status == pda.PDA_ERR_WORKSPACE
    assert str(pda.PDA_NOALLOC_SCRATCH_BYTES) in str(e.value)
    # a larger split fits; num_seqs == 0 is a no-op that needs no device
    assert pda.pda_workspace_bytes(big, 4096) <= pda.PDA_NOALLOC_SCRATCH_BYTES
    pda.pda_decode_noalloc(**{**args, "dims": big, "blocks_per_split": 4096, "num_seqs": 0})
    pda.pda_decode_noalloc(**{**args, "num_seqs": 0})


def test_noalloc_scratch_constant_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define PDA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pda.PDA_NOALLOC_SCRATCH_BYTES
