"""The C ABI on the host: the library loads, exports every function that
include/kda.h declares, and rejects bad descriptors before touching the GPU.
No GPU is needed: every call here fails validation (or only sizes the
workspace), so nothing is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_present() -> bool:
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The pointer checks below pass made-up device addresses that validation must
# reject.  They run where no GPU is visible, so a validation bug can never turn
# into a launch with those addresses.
no_gpu_only = pytest.mark.skipif(_gpu_present(), reason="fake-pointer checks run without a GPU")


@pytest.fixture(scope="module")
def abi():
    from gated_delta_rule_55_amd import _abi

    if not os.path.exists(_abi.LIB_PATH):
        pytest.skip("libkda.so not built")
    return _abi


def declared_functions():
    text = "".join(open(os.path.join(ROOT, "include", h)).read() for h in ("kda.h", "kda_conv.h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(kda_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(abi):
    names = declared_functions()
    assert "kda_chunk_prefill" in names and "kda_recurrent_decode" in names
    assert "kda_causal_conv1d_fwd" in names and "kda_causal_conv1d_update" in names
    lib = ctypes.CDLL(abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_version_and_strings(abi):
    L = abi.lib()
    assert L.kda_abi_version() == abi.KDA_ABI_VERSION
    for st in range(0, -11, -1):
        assert abi.status_string(st) != "unknown status"
    assert abi.status_string(-99) == "unknown status"


def test_struct_sizes_match_header(abi, tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include <stdio.h>\n#include "kda_conv.h"\n'
                   'int main(void){printf("%zu %zu %zu", sizeof(kda_prefill_desc),'
                   ' sizeof(kda_decode_desc), sizeof(kda_conv_desc));return 0;}\n')
    exe = tmp_path / "sz"
    os.system(f"gcc -I{ROOT}/include {src} -o {exe}")
    out = os.popen(str(exe)).read().split()
    assert [int(x) for x in out] == [ctypes.sizeof(abi.PrefillDesc), ctypes.sizeof(abi.DecodeDesc),
                                     ctypes.sizeof(abi.ConvDesc)]


def _valid_prefill(abi, **over):
    kw = dict(dtype=abi.KDA_DTYPE_BF16, n_seqs=1, n_heads=2, dk=128, dv=128, chunk=64,
              t_total=100, q=0x100000, k=0x200000, v=0x300000, g=0x400000, beta=0x500000,
              o=0x600000)
    kw.update(over)
    return abi.prefill_desc(**kw)


@pytest.mark.parametrize("over,status", [
    (dict(dtype=0), -3), (dict(dtype=3), -3), (dict(n_seqs=0), -2), (dict(n_heads=0), -2),
    (dict(t_total=-1), -2), (dict(dk=96, dv=96), -4), (dict(dk=128, dv=64), -4),
    (dict(chunk=48), -4), (dict(dtype=1, chunk=64), -4),
    # grid and item counts past 32 bits: 20M sequences x 32 heads x 8 column
    # blocks of the scan; 134M chunks of 16 tokens x 65535 heads
    (dict(n_seqs=20_000_000, n_heads=32), -2),
    (dict(t_total=(1 << 31) - 100, chunk=16, n_heads=65535), -2),
])
def test_workspace_query_validation(abi, over, status):
    d = _valid_prefill(abi, **over)
    st = ctypes.c_int(0)
    n = abi.lib().kda_chunk_prefill_workspace_bytes(ctypes.byref(d), ctypes.byref(st))
    assert st.value == status and n == 0


def test_workspace_two_pass_layout(abi):
    """The two-pass workspace is the chunk table plus one block of chunk-local
    results (80.5 KiB at d = 128, C = 64) per (chunk, head)."""
    block = 82432
    small = abi.workspace_bytes(_valid_prefill(abi, t_total=64, n_heads=1))
    big = abi.workspace_bytes(_valid_prefill(abi, t_total=64 * 1001, n_heads=1))
    # t_total / C + 1 chunk bound: 2 chunks -> 1002 chunks, one head
    assert big - small >= 1000 * block and big - small < 1000 * block + 64 * 1024
    assert small < 4 * block + 64 * 1024


def test_workspace_query_sizes(abi):
    d = _valid_prefill(abi)
    n = abi.workspace_bytes(d)
    assert n > 0 and n % 256 == 0
    d2 = _valid_prefill(abi, t_total=1000)
    assert abi.workspace_bytes(d2) >= n
    d3 = _valid_prefill(abi, struct_size=8)
    st = ctypes.c_int(0)
    abi.lib().kda_chunk_prefill_workspace_bytes(ctypes.byref(d3), ctypes.byref(st))
    assert st.value == abi.KDA_ERR_VERSION


@no_gpu_only
@pytest.mark.parametrize("over,status", [
    (dict(q=None), -1), (dict(o=None), -1), (dict(n_seqs=2), -1),   # cu_seqlens NULL, N > 1
    (dict(q=0x100008), -5), (dict(g=0x400002), -5),
    (dict(v=0x300008), -5), (dict(g=0x400004), -5), (dict(h0=0x700008), -5),  # vector reads
    (dict(o=0x100000 + 64), -9),                                      # o overlaps q
    (dict(h0=0x700000, ht=0x700000 + 16), -9),                        # ht partly overlaps h0
])
def test_prefill_rejects_bad_pointers(abi, over, status):
    d = _valid_prefill(abi, **over)
    assert abi.chunk_prefill_raw(d, 0x10000000, 1 << 30, 0) == status


@no_gpu_only
@pytest.mark.parametrize("gate,g,status", [
    ((5, 0x800000, 0x900000, 0xa00000), 0x400000, -4),        # unknown mode
    ((1, None, 0x900000, 0xa00000), None, -1),                 # KIMI without x
    ((1, 0x800000, None, 0xa00000), None, -1),                 # KIMI without a_log
    ((1, 0x800001, 0x900000, 0xa00000), None, -5),             # x misaligned (bf16)
    ((1, 0x800000, 0x900002, 0xa00000), None, -5),             # a_log misaligned
    ((1, 0x600000 + 64, 0x900000, 0xa00000), None, -9),        # x overlaps o
    ((0, None, None, None), None, -1),                         # GIVEN without g
])
def test_prefill_gate_validation(abi, gate, g, status):
    d = _valid_prefill(abi, gate=gate, g=g)
    assert abi.chunk_prefill_raw(d, 0x10000000, 1 << 30, 0) == status


@no_gpu_only
def test_prefill_gate_kimi_needs_no_g(abi):
    """With the gate computed in the kernels, g may be NULL: every pointer check
    passes and the call stops at the (too small) workspace."""
    d = _valid_prefill(abi, gate=(1, 0x800000, 0x900000, 0xa00000), g=None)
    assert abi.chunk_prefill_raw(d, 0x10000000, 16, 0) == abi.KDA_ERR_WORKSPACE


@no_gpu_only
def test_decode_gate_validation(abi):
    kw = dict(dtype=abi.KDA_DTYPE_BF16, n_seqs=2, n_heads=2, dk=64, dv=64, state=0x100000,
              q=0x900000, k=0xa00000, v=0xb00000, g=None, beta=0xd00000, o=0xe00000)
    d = abi.decode_desc(**kw, gate=(1, None, 0x700000, 0x780000))
    assert abi.recurrent_decode_raw(d, 0) == abi.KDA_ERR_NULL
    d = abi.decode_desc(**kw, gate=(3, 0x600000, 0x700000, 0x780000))
    assert abi.recurrent_decode_raw(d, 0) == abi.KDA_ERR_UNSUPPORTED
    d = abi.decode_desc(**kw, gate=(1, 0xe00000, 0x700000, 0x780000))  # x is o
    assert abi.recurrent_decode_raw(d, 0) == abi.KDA_ERR_ALIAS


@no_gpu_only
def test_state_pool_and_recurrent_validation(abi):
    # a slot table needs a pool size; indices are 4-byte aligned
    d = _valid_prefill(abi, state_indices=0xb00000, n_slots=0)
    assert abi.chunk_prefill_raw(d, 0x10000000, 1 << 30, 0) == abi.KDA_ERR_SHAPE
    d = _valid_prefill(abi, state_indices=0xb00002, n_slots=4)
    assert abi.chunk_prefill_raw(d, 0x10000000, 1 << 30, 0) == abi.KDA_ERR_ALIGN
    # the recurrent prefill ignores chunk and plan but checks everything else
    d = _valid_prefill(abi, chunk=48, plan=abi.KDA_PLAN_FUSED, q=0x100008)
    assert abi.chunk_prefill_raw(d, 0x10000000, 1 << 30, 0) == abi.KDA_ERR_UNSUPPORTED
    assert abi.recurrent_prefill_raw(d, 0) == abi.KDA_ERR_ALIGN
    d = _valid_prefill(abi, o=0x100000 + 64)
    assert abi.recurrent_prefill_raw(d, 0) == abi.KDA_ERR_ALIAS
    kw = dict(dtype=abi.KDA_DTYPE_BF16, n_seqs=2, n_heads=2, dk=64, dv=64, state=0x100000,
              q=0x900000, k=0xa00000, v=0xb00000, g=0xc00000, beta=0xd00000, o=0xe00000)
    assert abi.recurrent_decode_raw(abi.decode_desc(**kw, state_indices=0xf00000, n_slots=0),
                                    0) == abi.KDA_ERR_SHAPE
    # with a pool of 40 slots the state spans 40 x 2 x 64 x 64 x 4 bytes: o inside it
    assert abi.recurrent_decode_raw(abi.decode_desc(**dict(kw, o=0x100000 + 2 * 2 * 64 * 64 * 4 + 64),
                                                    state_indices=0xf00000, n_slots=40),
                                    0) == abi.KDA_ERR_ALIAS


@no_gpu_only
def test_fused_plan_value_is_refused(abi):
    """The reserved fused-plan value is refused on the host, before any launch."""
    d = _valid_prefill(abi, plan=abi.KDA_PLAN_FUSED)
    st = ctypes.c_int(0)
    abi.lib().kda_chunk_prefill_workspace_bytes(ctypes.byref(d), ctypes.byref(st))
    assert st.value == abi.KDA_ERR_UNSUPPORTED
    assert abi.chunk_prefill_raw(d, 0x10000000, 1 << 30, 0) == abi.KDA_ERR_UNSUPPORTED


@no_gpu_only
def test_prefill_rejects_small_or_missing_workspace(abi):
    d = _valid_prefill(abi)
    need = abi.workspace_bytes(d)
    assert abi.chunk_prefill_raw(d, 0, need, 0) == abi.KDA_ERR_WORKSPACE
    assert abi.chunk_prefill_raw(d, 0x10000000, need - 1, 0) == abi.KDA_ERR_WORKSPACE
    assert abi.chunk_prefill_raw(d, 0x10000000 + 16, need, 0) == abi.KDA_ERR_ALIGN
    assert abi.chunk_prefill_raw(d, 0x100000 - 256, need, 0) == abi.KDA_ERR_ALIAS


@no_gpu_only
@pytest.mark.parametrize("over,status", [
    (dict(struct_size=4), -8), (dict(dtype=9), -3), (dict(n_heads=0), -2), (dict(n_seqs=-1), -2),
    (dict(dk=64, dv=128), -4), (dict(state=None), -1), (dict(state=0x100008), -5),
    (dict(q=0x900008), -5), (dict(g=0xc00004), -5),
    (dict(o=0x100000), -9),
])
def test_decode_validation(abi, over, status):
    kw = dict(dtype=abi.KDA_DTYPE_BF16, n_seqs=2, n_heads=2, dk=64, dv=64, state=0x100000,
              q=0x900000, k=0xa00000, v=0xb00000, g=0xc00000, beta=0xd00000, o=0xe00000)
    kw.update(over)
    d = abi.decode_desc(**kw)
    if "struct_size" in over:
        d.struct_size = over["struct_size"]
    assert abi.recurrent_decode_raw(d, 0) == status


@no_gpu_only
def test_null_descriptors(abi):
    L = abi.lib()
    assert L.kda_chunk_prefill(None, None, 0, None) == abi.KDA_ERR_NULL
    assert L.kda_recurrent_decode(None, None) == abi.KDA_ERR_NULL
    assert L.kda_workspace_status(None, None) == abi.KDA_ERR_NULL


@no_gpu_only
def test_decode_zero_batch_is_noop(abi):
    d = abi.decode_desc(dtype=abi.KDA_DTYPE_F32, n_seqs=0, n_heads=1, dk=32, dv=32)
    assert abi.recurrent_decode_raw(d, 0) == abi.KDA_OK


def _valid_conv(abi, **over):
    kw = dict(dtype=abi.KDA_DTYPE_BF16, n_seqs=2, dim=256, width=4, activation=1, t_total=100,
              x=0x100000, weight=0x200000, bias=0x300000, cu_seqlens=0x400000,
              state_in=0x500000, state_out=0x500000, n_out=1, y=[0x600000, None, None],
              y_width=[256, 0, 0])
    kw.update(over)
    return abi.conv_desc(**kw)


@no_gpu_only
@pytest.mark.parametrize("over,status", [
    (dict(struct_size=4), -8), (dict(dtype=0), -3), (dict(width=5), -4), (dict(width=1), -4),
    (dict(activation=2), -4), (dict(dim=260, y_width=[260, 0, 0]), -2), (dict(n_seqs=0), -2),
    (dict(t_total=-1), -2), (dict(n_out=4), -2), (dict(n_out=2, y_width=[128, 64, 0]), -2),
    (dict(n_out=2, y_width=[128, 132, 0], y=[0x600000, 0x700000, None]), -2),
    (dict(weight=None), -1), (dict(x=None), -1), (dict(cu_seqlens=None), -1),
    (dict(n_out=2, y_width=[128, 128, 0]), -1),                         # y[1] missing
    (dict(x=0x100008), -5), (dict(bias=0x300004), -5), (dict(state_out=0x500008), -5),
    (dict(y=[0x100000 + 4096, None, None]), -9),                        # y overlaps x
    (dict(state_out=0x500000 + 512), -9),                               # partly over state_in
    (dict(state_out=0x100000 + 1024, state_in=None), -9),               # state_out over x
    (dict(state_indices=0x800000, n_slots=0), -2),
])
def test_conv_fwd_validation(abi, over, status):
    d = _valid_conv(abi, **over)
    if "struct_size" in over:
        d.struct_size = over["struct_size"]
    assert abi.conv_fwd_raw(d, 0) == status


@no_gpu_only
def test_conv_update_validation(abi):
    d = _valid_conv(abi, n_seqs=0, x=None, y=[None, None, None])
    assert abi.conv_update_raw(d, 0) == abi.KDA_OK              # nothing to do
    d = _valid_conv(abi, cu_seqlens=None, x=0x100000 + 8)
    assert abi.conv_update_raw(d, 0) == abi.KDA_ERR_ALIGN
    d = _valid_conv(abi, cu_seqlens=None, y=[0x500000, None, None])
    assert abi.conv_update_raw(d, 0) == abi.KDA_ERR_ALIAS       # y over the state
    L = abi.lib()
    assert L.kda_causal_conv1d_fwd(None, None) == abi.KDA_ERR_NULL
    assert L.kda_causal_conv1d_update(None, None) == abi.KDA_ERR_NULL


def test_product_path_fails_loudly_without_library(monkeypatch):
    from gated_delta_rule_55_amd import _abi

    monkeypatch.setattr(_abi, "_LIB", None)
    monkeypatch.setattr(_abi, "LIB_PATH", "/nonexistent/libkda.so")
    with pytest.raises(RuntimeError, match="missing"):
        _abi.lib()


@no_gpu_only
def test_state_dtype_validation(abi):
    """The state dtype is fp32 (0 or KDA_DTYPE_F32) or bf16 with bf16 inputs;
    byte ranges of bf16 states are half as long."""
    F32, BF16 = abi.KDA_DTYPE_F32, abi.KDA_DTYPE_BF16
    ws = (0x10000000, 1 << 30, 0)
    assert abi.chunk_prefill_raw(_valid_prefill(abi, state_dtype=7), *ws) == abi.KDA_ERR_DTYPE
    d = _valid_prefill(abi, dtype=F32, state_dtype=BF16)
    assert abi.chunk_prefill_raw(d, *ws) == abi.KDA_ERR_UNSUPPORTED
    assert abi.recurrent_prefill_raw(d, 0) == abi.KDA_ERR_UNSUPPORTED
    # 1 x 2 x 128 x 128 states: 64 KiB in bf16, 128 KiB in fp32
    h0 = 0x700000
    d = _valid_prefill(abi, h0=h0, ht=h0 + 65536, state_dtype=F32)
    assert abi.chunk_prefill_raw(d, *ws) == abi.KDA_ERR_ALIAS
    d = _valid_prefill(abi, h0=h0, ht=h0 + 65536, state_dtype=BF16)
    assert abi.chunk_prefill_raw(d, *ws) == abi.KDA_ERR_HIP      # checks pass; no device
    kw = dict(dtype=BF16, n_seqs=2, n_heads=2, dk=64, dv=64, state=0x100000, q=0x900000,
              k=0xa00000, v=0xb00000, g=0xc00000, beta=0xd00000, o=0xe00000)
    assert abi.recurrent_decode_raw(abi.decode_desc(**kw, state_dtype=5), 0) == abi.KDA_ERR_DTYPE
    assert abi.recurrent_decode_raw(abi.decode_desc(**dict(kw, dtype=F32), state_dtype=BF16),
                                    0) == abi.KDA_ERR_UNSUPPORTED
    # a pool of 40 bf16 slots spans 40 x 2 x 64 x 64 x 2 bytes: o just past it
    o = 0x100000 + 40 * 2 * 64 * 64 * 2 + 64
    pool = dict(state_indices=0xf00000, n_slots=40)
    assert abi.recurrent_decode_raw(abi.decode_desc(**dict(kw, o=o), **pool, state_dtype=F32),
                                    0) == abi.KDA_ERR_ALIAS
    assert abi.recurrent_decode_raw(abi.decode_desc(**dict(kw, o=o), **pool, state_dtype=BF16),
                                    0) == abi.KDA_ERR_HIP


@no_gpu_only
def test_noalloc_rejects_oversize_before_launch(abi):
    """The no-allocation entry point refuses a call whose workspace would not
    fit its static buffer (64 MiB), on the host; 1,536 tokens at 32 heads fit,
    1,600 do not."""
    L = abi.lib()
    far = dict(q=0x10000000, k=0x20000000, v=0x30000000, g=0x40000000, beta=0x50000000,
               o=0x60000000)  # made-up addresses far enough apart not to alias
    big = _valid_prefill(abi, t_total=1600, n_heads=32, **far)
    assert abi.workspace_bytes(big) > abi.KDA_NOALLOC_WORKSPACE_BYTES
    assert L.kda_chunk_prefill_noalloc(ctypes.byref(big), None) == abi.KDA_ERR_WORKSPACE
    ok = _valid_prefill(abi, t_total=1536, n_heads=32, **far)
    assert abi.workspace_bytes(ok) <= abi.KDA_NOALLOC_WORKSPACE_BYTES
    bad = _valid_prefill(abi, t_total=1536, n_heads=32, dtype=7, **far)
    assert L.kda_chunk_prefill_noalloc(ctypes.byref(bad), None) == abi.KDA_ERR_DTYPE
