"""The C-ABI library: it loads, exports every symbol include/pa.h declares, and its host
argument checks return the documented status codes before any HIP call (no GPU needed:
only invalid calls are made, and they return before touching the device)."""
import ctypes
import os
import re

import pytest

from pagedattention_block_table_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libpa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(pa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_signatures():
    names = declared_functions()
    assert names == sorted(_lib.SIGNATURES), names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    assert _lib.pa_status_str(0) == "ok"
    assert "workspace" in _lib.pa_status_str(-3)
    assert _lib.pa_status_str(12345) == "unknown status"
    assert _lib.pa_version() >= 100


def test_workspace_bytes_formula():
    # per (sequence, head, partition): max, sum and head_dim partial outputs, fp32
    assert _lib.pa_partitioned_workspace_bytes(8, 32, 128, 32768, 512) == 8 * 32 * 64 * 130 * 4
    assert _lib.pa_partitioned_workspace_bytes(2, 4, 64, 1000, 0) == 2 * 4 * 2 * 66 * 4
    assert _lib.pa_partitioned_workspace_bytes(2, 4, 64, 0, 0) == 2 * 4 * 1 * 66 * 4
    assert _lib.pa_partitioned_workspace_bytes(0, 4, 64, 10, 0) == 0
    assert _lib.pa_partitioned_workspace_bytes(1, 4, 64, -1, 0) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


def good_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, S=4, MB=7, NB=32, H=4, Hkv=4, D=64, BS=16,
             scale=0.125, io=_lib.PA_F32, kv=_lib.PA_F32, ks=1.0, vs=1.0)
    a.update(over)
    return [a[k] for k in ("q", "k", "v", "bt", "cl", "S", "MB", "NB", "H", "Hkv", "D", "BS",
                           "scale", "io", "kv", "ks", "vs")]


BAD = [
    (dict(q=0), _lib.PA_ERR_INVALID),
    (dict(bt=0), _lib.PA_ERR_INVALID),
    (dict(cl=0), _lib.PA_ERR_INVALID),
    (dict(S=0), _lib.PA_ERR_INVALID),
    (dict(NB=-1), _lib.PA_ERR_INVALID),
    (dict(io=3), _lib.PA_ERR_INVALID),
    (dict(io=7), _lib.PA_ERR_INVALID),
    (dict(kv=9), _lib.PA_ERR_INVALID),
    (dict(H=6, Hkv=4), _lib.PA_ERR_INVALID),
    (dict(scale=0.0), _lib.PA_ERR_INVALID),
    (dict(scale=float("nan")), _lib.PA_ERR_INVALID),
    (dict(kv=_lib.PA_FP8_E4M3, ks=0.0), _lib.PA_ERR_INVALID),
    (dict(kv=_lib.PA_FP8_E4M3, vs=float("inf")), _lib.PA_ERR_INVALID),
    (dict(q=FAKE + 2), _lib.PA_ERR_INVALID),
    (dict(k=FAKE + 8), _lib.PA_ERR_INVALID),
    (dict(kv=_lib.PA_F16), _lib.PA_ERR_UNSUPPORTED),
    (dict(D=96), _lib.PA_ERR_UNSUPPORTED),
    (dict(BS=48), _lib.PA_ERR_UNSUPPORTED),
    (dict(BS=1024), _lib.PA_ERR_UNSUPPORTED),
    (dict(H=48, Hkv=3), _lib.PA_ERR_UNSUPPORTED),
    (dict(io=_lib.PA_F16, kv=_lib.PA_FP8_E4M3, D=64, BS=8), _lib.PA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("over,code", BAD, ids=[str(b[0]) for b in BAD])
def test_decode_rejects(over, code):
    L = _lib.lib()
    assert L.pa_decode(*good_args(**over), FAKE, None) == code
    assert L.pa_decode(*good_args(**over), 0, None) == _lib.PA_ERR_INVALID  # null out first


@pytest.mark.parametrize("over,code", BAD[:6], ids=[str(b[0]) for b in BAD[:6]])
def test_partitioned_rejects(over, code):
    L = _lib.lib()
    assert L.pa_decode_partitioned(*good_args(**over), 100, 64, FAKE, 1 << 20, FAKE, None) == code


def test_partitioned_workspace_and_partition_checks():
    L = _lib.lib()
    a = good_args()
    # partition not a multiple of block_size
    assert L.pa_decode_partitioned(*a, 100, 24, FAKE, 1 << 20, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_decode_partitioned(*a, 100, -16, FAKE, 1 << 20, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_decode_partitioned(*a, -5, 64, FAKE, 1 << 20, FAKE, None) == _lib.PA_ERR_INVALID
    need = _lib.pa_partitioned_workspace_bytes(4, 4, 64, 100, 32)
    assert L.pa_decode_partitioned(*a, 100, 32, FAKE, need - 4, FAKE, None) == _lib.PA_ERR_WORKSPACE
    assert L.pa_decode_partitioned(*a, 100, 32, 0, need, FAKE, None) == _lib.PA_ERR_WORKSPACE
    assert L.pa_decode_partitioned(*a, 100, 32, FAKE + 4, need, FAKE, None) == _lib.PA_ERR_INVALID


def test_debug_trace_requires_buffers():
    L = _lib.lib()
    a = good_args()
    assert L.pa_debug_trace(*a, 100, 0, 0, None, 0, FAKE, 0, FAKE, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_trace(*a, 100, 0, 0, None, 0, FAKE, FAKE, FAKE, 0, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_trace(*a, 0, 0, 0, None, 0, FAKE, FAKE, FAKE, FAKE, None) == _lib.PA_ERR_INVALID
    # a partition size and a workgroup count at once, or negative values
    assert L.pa_debug_trace(*a, 100, 16, 8, FAKE, 1 << 20, FAKE, FAKE, FAKE, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_trace(*a, 100, 0, -1, FAKE, 1 << 20, FAKE, FAKE, FAKE, FAKE, None) == _lib.PA_ERR_INVALID


@pytest.mark.parametrize("over,code", BAD[:15], ids=[str(b[0]) for b in BAD[:15]])
def test_balanced_rejects(over, code):
    L = _lib.lib()
    assert L.pa_decode_balanced(*good_args(**over), 64, FAKE, 1 << 20, FAKE, None) == code


def test_balanced_workspace_checks():
    L = _lib.lib()
    # a shape the balanced kernel takes: f16, 8 query heads over 2 KV heads, head_dim 128
    a = good_args(io=_lib.PA_F16, kv=_lib.PA_F16, H=8, Hkv=2, D=128)
    need = _lib.pa_balanced_workspace_bytes(4, 8, 2, 128, 64)
    assert L.pa_decode_balanced(*a, 64, FAKE, need - 16, FAKE, None) == _lib.PA_ERR_WORKSPACE
    assert L.pa_decode_balanced(*a, 64, 0, need, FAKE, None) == _lib.PA_ERR_WORKSPACE
    assert L.pa_decode_balanced(*a, 64, FAKE + 4, need, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_decode_balanced(*a, -2, FAKE, need, FAKE, None) == _lib.PA_ERR_INVALID


@pytest.mark.parametrize("over,code", BAD, ids=[str(b[0]) for b in BAD])
def test_ordered_rejects(over, code):
    # argument errors are reported before anything (the ordering launch included) is enqueued
    L = _lib.lib()
    assert L.pa_decode_ordered(*good_args(**over), FAKE, 1 << 20, FAKE, None) == code


def test_ordered_needs_no_workspace():
    # the longest-first decode derives its order inside the launch: no workspace, and the
    # host checks still reject bad arguments before any HIP call
    L = _lib.lib()
    assert _lib.pa_ordered_workspace_bytes(4) == 0
    assert _lib.pa_ordered_workspace_bytes(100) == 0
    assert L.pa_decode_ordered(*good_args(q=0), None, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_decode_ordered(*good_args(H=6, Hkv=4), None, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_decode_ordered(*good_args(D=96), None, 0, FAKE, None) == _lib.PA_ERR_UNSUPPORTED


@pytest.mark.parametrize("over,code", BAD, ids=[str(b[0]) for b in BAD])
def test_grouped_rejects(over, code):
    L = _lib.lib()
    assert L.pa_decode_grouped(*good_args(**over), 4, FAKE, 1 << 20, FAKE, None) == code


def test_grouped_workspace_checks():
    L = _lib.lib()
    # a shape the grouped kernel takes: bf16, 8 query heads over 2 KV heads, head_dim 128
    a = good_args(io=_lib.PA_BF16, kv=_lib.PA_BF16, H=8, Hkv=2, D=128)
    need = _lib.pa_grouped_workspace_bytes(4, 8, 2, 128, 3)
    assert need == 4 * 8 * 3 * 130 * 4
    assert L.pa_decode_grouped(*a, 3, FAKE, need - 4, FAKE, None) == _lib.PA_ERR_WORKSPACE
    assert L.pa_decode_grouped(*a, 3, None, need, FAKE, None) == _lib.PA_ERR_WORKSPACE
    assert L.pa_decode_grouped(*a, 3, FAKE + 4, need, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_decode_grouped(*a, -1, FAKE, need, FAKE, None) == _lib.PA_ERR_INVALID


def test_grouped_workspace_formula():
    # fp32 (max, exp-sum, head_dim partial outputs) per (sequence, query head, split);
    # none for one split or for group sizes the grouped kernel does not take
    assert _lib.pa_grouped_workspace_bytes(64, 32, 8, 128, 4) == 64 * 32 * 4 * 130 * 4
    assert _lib.pa_grouped_workspace_bytes(64, 32, 8, 128, 1) == 0
    assert _lib.pa_grouped_workspace_bytes(64, 32, 32, 128, 4) == 0
    assert _lib.pa_grouped_workspace_bytes(64, 48, 8, 128, 4) == 0
    assert _lib.pa_grouped_workspace_bytes(0, 32, 8, 128, 4) == 0
    assert _lib.pa_grouped_workspace_bytes(64, 32, 8, 128, -1) == 0


def test_grouped_debug_trace_checks():
    L = _lib.lib()
    a = good_args(io=_lib.PA_BF16, kv=_lib.PA_BF16, H=8, Hkv=2, D=128)
    # no block-read counters
    assert L.pa_debug_trace_grouped(*a, 100, 1, None, 0, FAKE, FAKE, FAKE, FAKE, None, None) == \
        _lib.PA_ERR_INVALID
    # a shape the grouped kernel does not take
    b = good_args(io=_lib.PA_F32, kv=_lib.PA_F32, H=8, Hkv=2, D=128)
    assert L.pa_debug_trace_grouped(*b, 100, 1, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == \
        _lib.PA_ERR_UNSUPPORTED
    assert L.pa_debug_trace_grouped(*good_args(q=0), 100, 1, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == \
        _lib.PA_ERR_INVALID


def test_balanced_workspace_formula():
    # counters: one int32 per (KV head, sequence), padded to 256 bytes; then per workgroup
    # two slots of G maxima, G sums and G x head_dim partial outputs, fp32
    assert _lib.pa_balanced_workspace_bytes(64, 32, 8, 128, 512) == 2048 + 512 * 2 * 4 * 130 * 4
    assert _lib.pa_balanced_workspace_bytes(3, 4, 4, 64, 10) == 256 + 10 * 2 * 1 * 66 * 4
    assert _lib.pa_balanced_workspace_bytes(0, 4, 4, 64, 10) == 0
    assert _lib.pa_balanced_workspace_bytes(2, 6, 4, 64, 10) == 0
    assert _lib.pa_balanced_workspace_bytes(2, 4, 4, 64, -1) == 0


def test_small_entry_points_reject():
    L = _lib.lib()
    assert L.pa_check_tables(0, FAKE, 4, 7, 32, 16, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_check_tables(FAKE, FAKE, 0, 7, 32, 16, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_fp8_to_f32(FAKE, FAKE, 0, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_fp8_to_f32(0, FAKE, 16, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_fp8_to_16bit(FAKE, FAKE, 0, _lib.PA_F16, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_fp8_to_16bit(0, FAKE, 16, _lib.PA_BF16, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_fp8_to_16bit(FAKE, FAKE, 16, _lib.PA_F32, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_fp8_to_16bit(FAKE, FAKE, 16, _lib.PA_FP8_E4M3, None) == _lib.PA_ERR_INVALID
    # streaming-read probe: bytes a positive multiple of 4096 * unroll, unroll 4 / 8 / 16
    assert L.pa_debug_stream_read(0, 4096 * 4, 4, 0, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_stream_read(FAKE, 4096 * 4, 4, 0, 0, 0, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_stream_read(FAKE, 0, 4, 0, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_stream_read(FAKE, 4096 * 4 + 16, 4, 0, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_stream_read(FAKE, 4096 * 8, 6, 0, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_stream_read(FAKE + 8, 4096 * 8, 8, 0, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_stream_read(FAKE, 4096 * 8, 8, -1, 0, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_debug_stream_read(FAKE, 4096 * 8, 8, 0, 2, FAKE, None) == _lib.PA_ERR_INVALID


def test_noalloc_refuses_requests_beyond_its_scratch():
    """The allocation-free decode checks the partition-state size against its static scratch
    on the host, before any HIP call."""
    L = _lib.lib()
    a = good_args(S=8, H=32, Hkv=32, D=128, BS=32, MB=1024, NB=8192, io=_lib.PA_F16, kv=_lib.PA_F16)
    assert _lib.pa_partitioned_workspace_bytes(8, 32, 128, 65536, 512) > _lib.PA_NOALLOC_SCRATCH_BYTES
    assert L.pa_decode_partitioned_noalloc(*a, 65536, 512, FAKE, None) == _lib.PA_ERR_SCRATCH
    assert L.pa_decode_partitioned_noalloc(*a, 65536, 0, FAKE, None) == _lib.PA_ERR_SCRATCH
    assert L.pa_decode_partitioned_noalloc(*a, 32768, 48, FAKE, None) == _lib.PA_ERR_INVALID  # P % BS
    assert L.pa_decode_partitioned_noalloc(*a, -1, 512, FAKE, None) == _lib.PA_ERR_INVALID
    assert L.pa_decode_partitioned_noalloc(*a, 32768, -512, FAKE, None) == _lib.PA_ERR_INVALID
    bad = good_args(q=0)
    assert L.pa_decode_partitioned_noalloc(*bad, 100, 16, FAKE, None) == _lib.PA_ERR_INVALID
    assert "scratch" in _lib.pa_status_str(_lib.PA_ERR_SCRATCH)


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 64)
    pool = torch.zeros(2, 4, 16, 64)
    bt = torch.zeros(1, 1, dtype=torch.int32)
    cl = torch.ones(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.pa_decode(q, pool, pool, bt, cl)


def test_append_rejects():
    L = _lib.lib()
    good = dict(kn=FAKE, vn=FAKE, seq=FAKE, pos=FAKE, T=4, bt=FAKE, S=2, MB=3, kp=FAKE, vp=FAKE, NB=8,
                Hkv=2, D=128, BS=16, src=_lib.PA_F16, kv=_lib.PA_F16, ks=1.0, vs=1.0)

    def call(**over):
        a = dict(good)
        a.update(over)
        return L.pa_append_kv(a["kn"], a["vn"], a["seq"], a["pos"], a["T"], a["bt"], a["S"], a["MB"],
                              a["kp"], a["vp"], a["NB"], a["Hkv"], a["D"], a["BS"], a["src"], a["kv"],
                              a["ks"], a["vs"], None)

    assert call(kn=0) == _lib.PA_ERR_INVALID
    assert call(bt=0) == _lib.PA_ERR_INVALID
    assert call(T=-1) == _lib.PA_ERR_INVALID
    assert call(S=0) == _lib.PA_ERR_INVALID
    assert call(src=_lib.PA_FP8_E4M3) == _lib.PA_ERR_INVALID      # new rows come in an io dtype
    assert call(kv=7) == _lib.PA_ERR_INVALID
    assert call(kv=_lib.PA_BF16) == _lib.PA_ERR_UNSUPPORTED       # only copy or fp8 quantise
    assert call(kv=_lib.PA_FP8_E4M3, ks=0.0) == _lib.PA_ERR_INVALID
    assert call(kv=_lib.PA_FP8_E4M3, vs=float("nan")) == _lib.PA_ERR_INVALID
    assert call(kp=FAKE + 4) == _lib.PA_ERR_INVALID
    assert call(D=96) == _lib.PA_ERR_UNSUPPORTED
    assert call(D=512) == _lib.PA_ERR_UNSUPPORTED
    assert call(BS=48) == _lib.PA_ERR_UNSUPPORTED
    assert call(BS=1024) == _lib.PA_ERR_UNSUPPORTED
    assert call(T=0) == _lib.PA_OK                                 # nothing to write, nothing enqueued


def test_copy_blocks_rejects():
    L = _lib.lib()
    good = dict(kp=FAKE, vp=FAKE, pairs=FAKE, n=3, NB=8, Hkv=2, D=128, BS=16, kv=_lib.PA_F16)

    def call(**over):
        a = dict(good)
        a.update(over)
        return L.pa_copy_blocks(a["kp"], a["vp"], a["pairs"], a["n"], a["NB"], a["Hkv"], a["D"], a["BS"],
                                a["kv"], None)

    assert call(kp=0) == _lib.PA_ERR_INVALID
    assert call(pairs=0) == _lib.PA_ERR_INVALID
    assert call(n=-1) == _lib.PA_ERR_INVALID
    assert call(NB=0) == _lib.PA_ERR_INVALID
    assert call(kv=9) == _lib.PA_ERR_INVALID
    assert call(vp=FAKE + 8) == _lib.PA_ERR_INVALID
    assert call(Hkv=1, D=3, BS=1, kv=_lib.PA_FP8_E4M3) == _lib.PA_ERR_UNSUPPORTED  # 3-byte blocks
    assert call(n=0, pairs=0) == _lib.PA_OK                        # nothing to copy, nothing enqueued


def test_extend_rejects():
    L = _lib.lib()
    good = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, qsl=FAKE, S=2, MB=4, NB=8, MQ=5, H=8, Hkv=2,
                D=128, BS=16, scale=0.1, io=_lib.PA_F16, kv=_lib.PA_F16, ks=1.0, vs=1.0, out=FAKE)

    def call(**over):
        a = dict(good)
        a.update(over)
        return L.pa_extend(a["q"], a["k"], a["v"], a["bt"], a["cl"], a["qsl"], a["S"], a["MB"], a["NB"],
                           a["MQ"], a["H"], a["Hkv"], a["D"], a["BS"], a["scale"], a["io"], a["kv"],
                           a["ks"], a["vs"], a["out"], None)

    assert call(qsl=0) == _lib.PA_ERR_INVALID
    assert call(out=0) == _lib.PA_ERR_INVALID
    assert call(MQ=-1) == _lib.PA_ERR_INVALID
    assert call(H=6, Hkv=4) == _lib.PA_ERR_INVALID
    assert call(scale=float("inf")) == _lib.PA_ERR_INVALID
    assert call(kv=_lib.PA_FP8_E4M3, ks=-1.0) == _lib.PA_ERR_INVALID
    assert call(q=FAKE + 4) == _lib.PA_ERR_INVALID
    assert call(io=_lib.PA_F32, kv=_lib.PA_F32) == _lib.PA_ERR_UNSUPPORTED   # 16-bit queries only
    assert call(kv=_lib.PA_BF16) == _lib.PA_ERR_UNSUPPORTED
    assert call(D=96) == _lib.PA_ERR_UNSUPPORTED
    assert call(BS=24) == _lib.PA_ERR_UNSUPPORTED
    assert call(BS=1024) == _lib.PA_ERR_UNSUPPORTED
    assert call(H=32, Hkv=2) == _lib.PA_ERR_UNSUPPORTED                      # group of 16
    assert call(MQ=0) == _lib.PA_OK                                          # nothing enqueued
