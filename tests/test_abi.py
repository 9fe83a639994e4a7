"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")

ops = pytest.importorskip("paged_kv_cache_289_amd.ops",
                          reason="libpagedattn.so not built (python -m paged_kv_cache_289_amd.build)")

FAKE = ctypes.c_void_p(0x10000)    # never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(paged_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert names, "no declarations found"
    for n in names:
        assert hasattr(ops.LIB, n), f"{n} missing from {ops.LIB_PATH}"
    assert sorted(ops.SIGNATURES) == names


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert ops.status_string(st)
    assert ops.status_string(-99) == "unknown status"


def _decode(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tbl=FAKE, lens=FAKE, S=4, H=32, Hk=8, D=128, B=16,
             NB=100, mbs=64, maxctx=1024, scale=0.088, dt=ops.PA_BF16, odt=ops.PA_BF16, part=0,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return ops.LIB.paged_attn_decode(a["out"], a["q"], a["k"], a["v"], a["tbl"], a["lens"], a["S"],
                                     a["H"], a["Hk"], a["D"], a["B"], a["NB"], a["mbs"],
                                     a["maxctx"], a["scale"], a["dt"], a["odt"], a["part"],
                                     a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), ops.PA_ERR_NULL),
    (dict(out=None), ops.PA_ERR_NULL),
    (dict(tbl=None), ops.PA_ERR_NULL),
    (dict(lens=None), ops.PA_ERR_NULL),
    (dict(S=-1), ops.PA_ERR_SHAPE),
    (dict(H=30, Hk=8), ops.PA_ERR_SHAPE),
    (dict(H=0), ops.PA_ERR_SHAPE),
    (dict(maxctx=64 * 16 + 1), ops.PA_ERR_SHAPE),
    (dict(maxctx=-5), ops.PA_ERR_SHAPE),
    (dict(part=24), ops.PA_ERR_SHAPE),
    (dict(scale=float("inf")), ops.PA_ERR_SHAPE),
    (dict(scale=float("nan")), ops.PA_ERR_SHAPE),
    (dict(D=96), ops.PA_ERR_UNSUPPORTED),
    (dict(B=12), ops.PA_ERR_UNSUPPORTED),
    (dict(dt=7), ops.PA_ERR_UNSUPPORTED),
    (dict(odt=ops.PA_F16), ops.PA_ERR_UNSUPPORTED),
    (dict(H=34, Hk=2), ops.PA_ERR_UNSUPPORTED),
    (dict(q=ctypes.c_void_p(0x10008)), ops.PA_ERR_UNSUPPORTED),
    (dict(ws=None, part=256), ops.PA_ERR_WORKSPACE),
    (dict(wsb=100, part=256), ops.PA_ERR_WORKSPACE),
])
def test_decode_rejects_bad_arguments_on_host(kw, code):
    assert _decode(**kw) == code


@pytest.mark.parametrize("kw", [dict(dt=3), dict(dt=3, D=64, B=8), dict(dt=3, H=64, Hk=4),
                                dict(dt=3, odt=ops.PA_F32)])
def test_plain_decode_rejects_8bit_caches(kw):
    # 8-bit E4M3 caches (code 3) are served by paged_attn_decode_fp8kv only, which
    # also rejects the shapes the 8-bit kernels cannot take
    assert ops.PA_FP8_E4M3 == 3
    assert _decode(**kw) == ops.PA_ERR_UNSUPPORTED


def test_binding_rejects_cache_dtype_other_than_the_query():
    import torch
    q = torch.zeros((2, 8, 128), dtype=torch.bfloat16)
    codes = torch.zeros((4, 2, 16, 128), dtype=torch.uint8)
    tbl = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.ones((2,), dtype=torch.int32)
    qoff = torch.tensor([0, 1, 2], dtype=torch.int32)
    with pytest.raises(ops.PagedAttnError) as e:
        ops.decode(q, codes, codes, tbl, lens, 0.1, 16)
    assert e.value.status == ops.PA_ERR_UNSUPPORTED
    with pytest.raises(ops.PagedAttnError):
        ops.multiq(q, codes.view(torch.float16), codes.view(torch.float16), tbl, lens, qoff, 0.1,
                   16, 1)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), ops.PA_ERR_NULL),
    (dict(S=-1), ops.PA_ERR_SHAPE),
    (dict(D=96), ops.PA_ERR_UNSUPPORTED),
    (dict(dt=3), ops.PA_ERR_UNSUPPORTED),
    (dict(H=30, Hk=8), ops.PA_ERR_SHAPE),
    (dict(q=ctypes.c_void_p(0x10008)), ops.PA_ERR_UNSUPPORTED),
    (dict(S=0, q=None, out=None), ops.PA_OK),
])
def test_noalloc_decode_rejects_bad_arguments_on_host(kw, code):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tbl=FAKE, lens=FAKE, S=4, H=32, Hk=8, D=128, B=16,
             NB=100, mbs=64, maxctx=1024, scale=0.088, dt=ops.PA_BF16, odt=ops.PA_BF16, part=0,
             stream=None)
    a.update(kw)
    assert ops.LIB.paged_attn_decode_noalloc(
        a["out"], a["q"], a["k"], a["v"], a["tbl"], a["lens"], a["S"], a["H"], a["Hk"], a["D"],
        a["B"], a["NB"], a["mbs"], a["maxctx"], a["scale"], a["dt"], a["odt"], a["part"],
        a["stream"]) == code


def test_decode_with_no_sequences_is_a_no_op():
    assert _decode(S=0, q=None, out=None) == ops.PA_OK


def test_multiq_rejects_bad_arguments_on_host():
    L = ops.LIB
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 5, 32, 8, 128, 16, 100, 64, 1024,
            0.08, 1, ops.PA_BF16, ops.PA_BF16, 0, FAKE, 1 << 30, None]
    def call(i, v):
        a = list(base)
        a[i] = v
        return L.paged_attn_multiq(*a)
    assert call(6, None) == ops.PA_ERR_NULL          # q_offsets
    assert call(8, -1) == ops.PA_ERR_SHAPE           # total_q
    assert call(9, 4) == ops.PA_ERR_SHAPE            # max_q_len * S < total_q
    assert call(12, 80) == ops.PA_ERR_UNSUPPORTED    # head_dim
    a = list(base)
    a[21], a[23] = 256, 8                              # 256-token partitions, 8-byte workspace
    assert L.paged_attn_multiq(*a) == ops.PA_ERR_WORKSPACE


def test_gather_and_check_reject_bad_arguments_on_host():
    L = ops.LIB
    g = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 16, 100, 16, ops.PA_BF16, None]
    a = list(g); a[2] = None
    assert L.paged_kv_gather(*a) == ops.PA_ERR_NULL
    a = list(g); a[13] = 9
    assert L.paged_kv_gather(*a) == ops.PA_ERR_UNSUPPORTED
    a = list(g); a[7] = -3
    assert L.paged_kv_gather(*a) == ops.PA_ERR_SHAPE
    assert L.paged_attn_check_inputs(FAKE, FAKE, 2, 16, 100, 16, 256, None, None) == \
        ops.PA_ERR_NULL
    assert L.paged_attn_check_inputs(FAKE, FAKE, 2, 0, 100, 16, 256, FAKE, None) == \
        ops.PA_ERR_SHAPE


def test_hbm_read_rejects_unknown_patterns_on_host():
    L = ops.LIB
    assert L.paged_hbm_read(FAKE, 4096, FAKE, 0, 3, None) == ops.PA_ERR_SHAPE
    assert L.paged_hbm_read(FAKE, 4096, FAKE, 0, -1, None) == ops.PA_ERR_SHAPE
    assert L.paged_hbm_read(FAKE, 4096, FAKE, -1, 0, None) == ops.PA_ERR_SHAPE
    assert L.paged_hbm_read(FAKE, 4095, FAKE, 0, 2, None) == ops.PA_ERR_UNSUPPORTED
    assert L.paged_hbm_read(None, 4096, FAKE, 0, 2, None) == ops.PA_ERR_NULL


def test_workspace_size_formula():
    # Decode, 64 sequences x 8 KV heads (G = 4), head_dim 128, contexts up to 4096 in
    # 16-token blocks, 256-token pieces: each (sequence, KV head) is at most 256 block
    # items plus its 4 fixed-cost items, 64*8*260 = 133120 items in pieces of 16 ->
    # 8320 waves; the plan (2 + 65 int32, on 256 bytes), then fp32 (max, sum) and
    # outputs for (64*8 + 8320) slots x 4 heads, each region on a 256-byte boundary.
    seg = 4
    n = ops.workspace_size(64, 64, 1, 32, 8, 128, 16, 4096, 256)
    slots = 64 * 8 + (64 * 8 * (256 + seg) + 15) // 16
    assert n == 512 + slots * 4 * 2 * 4 + slots * 4 * 128 * 4
    assert (slots * 4 * 2 * 4) % 256 == 0
    # default pieces: the launch never exceeds 8192 waves
    slots = 64 * 8 + 8192
    assert ops.workspace_size(64, 64, 1, 32, 8, 128, 16, 4096, 0) == \
        512 + slots * 4 * 2 * 4 + slots * 4 * 128 * 4
    # multi-token rows whose contexts fit one partition need no workspace with an
    # explicit partition size
    assert ops.workspace_size(2, 10, 5, 32, 8, 128, 16, 256, 256) == 0
    # ... while the library's own split (5 tokens x G 4 = 20 rows: one row tile per
    # KV head) holds a 32-row piece per (sequence, KV head, row tile) unit and per
    # wave: 2*8 = 16 units of 256/32 + 4 items each (the sizing takes the larger
    # fixed cost, an 8-bit cache's) = 192 waves at most; the plan (2 + 3 int32, on
    # 256 bytes), then fp32 (max, sum) and 128 outputs per row
    rows = (16 + 192) * 32
    assert ops.workspace_size(2, 10, 5, 32, 8, 128, 16, 256, 0) == \
        256 + rows * 2 * 4 + rows * 128 * 4
    # the waves stop at 4096 (64 sequences of up to 8192 keys)
    rows = (64 * 8 + 4096) * 32
    assert ops.workspace_size(64, 320, 5, 32, 8, 128, 16, 8192, 0) == \
        512 + rows * 2 * 4 + rows * 128 * 4
    assert ops.workspace_size(64, 64, 1, 32, 8, 128, 16, 4096, 24) == 0     # rejected
    assert ops.default_partition(64, 32, 8, 16, 4096, 1) % 16 == 0
    assert ops.default_partition(1, 32, 8, 16, 4608, 512) % 32 == 0


def test_multiq_split_choice():
    """Which multi-token calls take the balanced split: bf16/f16, head_dim 128, the
    library's own work split, 2 or more query tokens and at most three 32-row tiles
    of rows per KV head."""
    bf, f16, f32 = ops.PA_BF16, ops.PA_F16, ops.PA_F32
    assert ops.multiq_uses_split(64, 5, 32, 8, 128, bf)            # 20 rows per KV head
    assert ops.multiq_uses_split(64, 5, 32, 8, 128, f16)
    assert ops.multiq_uses_split(4, 24, 32, 8, 128, bf)            # 96 rows: three tiles
    assert not ops.multiq_uses_split(4, 25, 32, 8, 128, bf)        # 100 rows: row groups
    assert not ops.multiq_uses_split(64, 5, 32, 8, 128, f32)       # vector-ALU path
    assert not ops.multiq_uses_split(64, 5, 32, 8, 64, bf)         # head_dim 64
    assert not ops.multiq_uses_split(64, 5, 32, 8, 128, bf, 256)   # explicit partitions
    assert not ops.multiq_uses_split(64, 1, 32, 8, 128, bf)        # one token per sequence
    assert not ops.multiq_uses_split(8193, 2, 32, 8, 128, bf)      # past 8192 sequences
    assert not ops.multiq_uses_split(2048, 5, 32, 16, 128, bf)     # past 16384 units
    assert ops.multiq_uses_split(2048, 5, 32, 8, 128, bf)          # 16384 units


def _shared(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tbl=FAKE, lens=FAKE, S=4, H=32, Hk=8, D=128, B=16,
             NB=100, mbs=64, maxctx=1024, P=8, scale=0.088, dt=ops.PA_BF16, odt=ops.PA_BF16,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return ops.LIB.paged_attn_decode_shared_prefix(
        a["out"], a["q"], a["k"], a["v"], a["tbl"], a["lens"], a["S"], a["H"], a["Hk"], a["D"],
        a["B"], a["NB"], a["mbs"], a["maxctx"], a["P"], a["scale"], a["dt"], a["odt"], a["ws"],
        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(P=-1), ops.PA_ERR_SHAPE),
    (dict(P=65), ops.PA_ERR_SHAPE),
    (dict(P=8, maxctx=100), ops.PA_ERR_SHAPE),
    (dict(q=None), ops.PA_ERR_NULL),
    (dict(wsb=16), ops.PA_ERR_WORKSPACE),
    (dict(ws=None), ops.PA_ERR_WORKSPACE),
    (dict(H=30), ops.PA_ERR_SHAPE),
    (dict(S=0), ops.PA_OK),
])
def test_shared_prefix_rejects_bad_arguments(kw, code):
    assert _shared(**kw) == code


def test_shared_prefix_workspace_size():
    full = ops.shared_prefix_workspace_size(256, 32, 8, 128, 16, 6144, 128)
    assert full > ops.workspace_size(256, 256, 1, 32, 8, 128, 16, 6144)
    assert ops.shared_prefix_workspace_size(256, 32, 8, 128, 16, 6144, 0) == \
        ops.workspace_size(256, 256, 1, 32, 8, 128, 16, 6144)
    assert ops.shared_prefix_workspace_size(4, 32, 8, 128, 16, 100, 8) == 0   # prefix > context
