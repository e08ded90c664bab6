"""C-ABI checks that run without a GPU.

libfa.so must load, export every function include/fa.h declares, and reject
bad arguments on the host before any HIP call (so the error paths can be
exercised here with dummy, never-dereferenced pointers).
"""

import ctypes
import os
import re

import pytest

from io_aware_exact_24_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, INVALID, UNSUPPORTED = binding.FA_OK, binding.FA_ERR_INVALID_ARG, binding.FA_ERR_UNSUPPORTED
P = 0x10000  # a 16-byte-aligned dummy address; validation fails before it is used


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libfa.so is not built (python -m io_aware_exact_24_amd.build)")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings(lib):
    assert binding.fa_status_string(OK) == "ok"
    assert binding.fa_status_string(INVALID) == "invalid argument"
    assert binding.fa_status_string(UNSUPPORTED) == "unsupported configuration"
    assert binding.fa_status_string(binding.FA_ERR_HIP) == "HIP launch error"
    assert binding.fa_status_string(binding.FA_ERR_TOO_LARGE) == \
        "sizes exceed the fixed scratch of this entry point"
    assert binding.fa_status_string(42) == "unknown status"


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=64, dtype=binding.FA_BF16,
        scale=0.125, causal=0, key_lens=None, p=0.0, seed=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, dtype, scale, causal, key_lens, p, seed, None)


def bwd(lib, ptrs=None, B=1, H=1, N=128, d=64, dtype=binding.FA_BF16, scale=0.125, causal=0,
        key_lens=None, p=0.0, seed=0, ws=P, ws_bytes=None):
    ptrs = ptrs or [P] * 9
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d, dtype)
    return lib.fa_bwd(*ptrs, B, H, N, d, dtype, scale, causal, key_lens, p, seed, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(lse=None), INVALID),
    (dict(k=P + 8), INVALID), (dict(v=P + 4), INVALID), (dict(key_lens=P + 2), INVALID),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(N=0), INVALID),
    (dict(B=1 << 16, H=1 << 16, N=1), INVALID),            # B*H*N overflows int32 rows
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(p=1.0), INVALID), (dict(p=-0.1), INVALID), (dict(p=float("nan")), INVALID),
    (dict(dtype=7), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(d=16), UNSUPPORTED), (dict(d=512), UNSUPPORTED),
    (dict(d=0), INVALID), (dict(dtype=binding.FA_F32, p=0.1), UNSUPPORTED),
])
def test_forward_rejects(lib, kw, expect):
    assert fwd(lib, **kw) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(B=0), INVALID), (dict(scale=float("nan")), INVALID), (dict(p=1.0), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(dtype=binding.FA_F32, p=0.1), UNSUPPORTED),
    (dict(ws=None), INVALID), (dict(ws=P + 4), INVALID), (dict(ws_bytes=0), INVALID),
])
def test_backward_rejects(lib, kw, expect):
    assert bwd(lib, **kw) == expect


@pytest.mark.parametrize("idx", range(9))
def test_backward_rejects_null_tensor(lib, idx):
    ptrs = [P] * 9
    ptrs[idx] = None
    assert bwd(lib, ptrs=ptrs) == INVALID


@pytest.mark.parametrize("N,d", [(1 << 24, 128), (1 << 25, 64)])
def test_per_head_byte_range_beyond_32_bits_is_unsupported(lib, N, d):
    # one (b, h) slice of N * d bf16 elements reaches 2^32 bytes: the kernels'
    # 32-bit buffer offsets could not address it, so every entry point refuses
    # before any HIP call (the dummy pointers are never touched)
    assert fwd(lib, N=N, d=d) == UNSUPPORTED
    assert fwd(lib, N=N - 1, d=d, dtype=binding.FA_F32) == UNSUPPORTED  # fp32: 4 bytes each
    assert split(lib, N=N, d=d, ws_bytes=1 << 62) == UNSUPPORTED
    assert bwd(lib, N=N, d=d, ws_bytes=1 << 62) == UNSUPPORTED
    assert set(stage_calls(lib, N=N, d=d, ws_bytes=1 << 62).values()) == {UNSUPPORTED}
    assert lib.fa_bwd_workspace_size(1, 1, N, d, binding.FA_BF16) == 0
    assert lib.fa_fwd_split_workspace_size(1, 1, N, d, binding.FA_BF16, 2) == 0


def test_backward_rejects_short_workspace(lib):
    need = lib.fa_bwd_workspace_size(2, 3, 100, 128, binding.FA_BF16)
    assert bwd(lib, B=2, H=3, N=100, d=128, ws_bytes=need - 1) == INVALID


def test_workspace_size_is_linear_in_n():
    # fp32 D and fp32 LSE*log2(e) per row, each padded to 256 bytes: O(B*H*N),
    # never O(N^2).
    ws = binding.fa_bwd_workspace_size
    assert ws(1, 1, 128, 64) == 2 * 512
    assert ws(1, 1, 100, 64) == 2 * 512
    assert ws(4, 32, 4096, 128) == 2 * 4 * 32 * 4096 * 4
    assert ws(1, 8, 65536, 64) == 2 * 8 * 65536 * 4
    assert ws(1, 1, 65536, 64) < 65536 * 65536 // 16
    assert ws(1, 1, 128, 48) == 0
    # the same two row arrays for every supported type and head size
    for d in (32, 96, 256):
        assert ws(3, 2, 100, d, binding.FA_F32) == ws(3, 2, 100, 64) == ws(3, 2, 100, d, binding.FA_F16)
    assert ws(0, 1, 128, 64) == 0


def stage_calls(lib, B=1, H=1, N=128, d=64, dtype=binding.FA_BF16, scale=0.125, p=0.0, ws=P,
                ws_bytes=None, null=None):
    """The backward stages with placeholder pointers; `null` names one
    tensor argument to pass as NULL."""
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d, dtype)

    def t(name):
        return None if name == null else P

    return {
        "preprocess": lib.fa_bwd_preprocess(t("o"), t("dout"), t("lse"), B, H, N, d, dtype, ws,
                                            ws_bytes, None),
        "dkdv": lib.fa_bwd_dkdv(t("q"), t("k"), t("v"), t("dout"), t("dk"), t("dv"), B, H, N, d,
                                dtype, scale, 0, None, p, 0, ws, ws_bytes, None),
        "dq": lib.fa_bwd_dq(t("q"), t("k"), t("v"), t("o"), t("dout"), t("lse"), t("dq"), B, H, N,
                            d, dtype, scale, 0, None, p, 0, ws, ws_bytes, None),
    }


@pytest.mark.parametrize("kw,expect", [
    (dict(B=0), INVALID), (dict(N=-3), INVALID), (dict(d=48), UNSUPPORTED),
    (dict(d=512), UNSUPPORTED), (dict(dtype=9), INVALID),
    (dict(ws=None), INVALID), (dict(ws=P + 4), INVALID), (dict(ws_bytes=0), INVALID),
])
def test_backward_stages_reject(lib, kw, expect):
    assert set(stage_calls(lib, **kw).values()) == {expect}


@pytest.mark.parametrize("kw", [dict(scale=float("nan")), dict(scale=0.0), dict(p=1.0)])
def test_backward_compute_stages_check_scale_and_dropout(lib, kw):
    got = stage_calls(lib, **kw)
    assert got["dkdv"] == INVALID and got["dq"] == INVALID


@pytest.mark.parametrize("name,stage", [
    ("o", "preprocess"), ("dout", "preprocess"), ("lse", "preprocess"),
    ("q", "dkdv"), ("k", "dkdv"), ("v", "dkdv"), ("dout", "dkdv"), ("dk", "dkdv"), ("dv", "dkdv"),
    ("q", "dq"), ("k", "dq"), ("v", "dq"), ("o", "dq"), ("dout", "dq"), ("lse", "dq"), ("dq", "dq"),
])
def test_backward_stages_reject_null(lib, name, stage):
    assert stage_calls(lib, null=name)[stage] == INVALID


def split(lib, B=1, H=1, N=128, d=64, dtype=binding.FA_BF16, splits=2, ws=P, ws_bytes=None,
          p=0.0, q=P):
    if ws_bytes is None:
        ws_bytes = lib.fa_fwd_split_workspace_size(B, H, N, d, dtype, splits)
    return lib.fa_fwd_split(q, P, P, P, P, B, H, N, d, dtype, 0.125, 1, None, p, 0, splits, ws,
                            ws_bytes, None)


def test_split_workspace_size():
    ws = binding.fa_fwd_split_workspace_size
    # fp32 partial O per split (padded to 256 B) then fp32 partial LSE per split
    assert ws(2, 3, 100, 64, 4) == 4 * 2 * 3 * 100 * 64 * 4 + ((4 * 2 * 3 * 100 * 4 + 255) // 256) * 256
    assert ws(1, 8, 4096, 128, 1) == 8 * 4096 * 128 * 4 + 8 * 4096 * 4
    assert ws(1, 1, 128, 96, 2) == 0  # the split forward is for the MFMA head sizes only
    assert ws(1, 1, 128, 64, 0) == 0
    assert ws(1, 1, 128, 64, binding.FA_MAX_SPLITS + 1) == 0
    assert ws(1, 1, 128, 64, 2, binding.FA_F32) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(splits=0), INVALID), (dict(splits=binding.FA_MAX_SPLITS + 1), INVALID),
    (dict(dtype=binding.FA_F32), UNSUPPORTED), (dict(d=96, ws_bytes=1 << 30), UNSUPPORTED),
    (dict(d=256, ws_bytes=1 << 30), UNSUPPORTED),
    (dict(ws=None), INVALID), (dict(ws=P + 8), INVALID), (dict(ws_bytes=16), INVALID),
    (dict(q=None), INVALID), (dict(p=1.0), INVALID), (dict(N=0), INVALID),
])
def test_split_rejects(lib, kw, expect):
    assert split(lib, **kw) == expect


def bsplit(lib, B=1, H=1, N=128, d=64, dtype=binding.FA_BF16, splits=2, ws=P, ws_bytes=None,
           p=0.0, q=P, dq=P):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_split_workspace_size(B, H, N, d, dtype, splits)
    return lib.fa_bwd_split(q, P, P, P, P, P, dq, P, P, B, H, N, d, dtype, 0.125, 1, None, p, 0,
                            splits, ws, ws_bytes, None)


def test_backward_split_workspace_size():
    ws = binding.fa_bwd_split_workspace_size
    base = binding.fa_bwd_workspace_size
    # fa_bwd's two row arrays, then fp32 partial dQ, dK and dV per split, each
    # padded to 256 bytes
    part = ((3 * 2 * 3 * 100 * 64 * 4 + 255) // 256) * 256
    assert ws(2, 3, 100, 64, 3) == base(2, 3, 100, 64) + 3 * part
    assert ws(1, 8, 4096, 128, 2) == 2 * 8 * 4096 * 4 + 3 * 2 * 8 * 4096 * 128 * 4
    assert ws(1, 1, 128, 96, 2) == 0  # MFMA head sizes only
    assert ws(1, 1, 128, 64, 0) == 0
    assert ws(1, 1, 128, 64, binding.FA_MAX_SPLITS + 1) == 0
    assert ws(1, 1, 128, 64, 2, binding.FA_F32) == 0
    assert ws(1, 1, 1 << 24, 128, 2) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(splits=0), INVALID), (dict(splits=binding.FA_MAX_SPLITS + 1), INVALID),
    (dict(dtype=binding.FA_F32, ws_bytes=1 << 30), UNSUPPORTED),
    (dict(d=96, ws_bytes=1 << 30), UNSUPPORTED), (dict(d=256, ws_bytes=1 << 30), UNSUPPORTED),
    (dict(d=48, ws_bytes=1 << 30), UNSUPPORTED), (dict(N=1 << 24, d=128, ws_bytes=1 << 62), UNSUPPORTED),
    (dict(ws=None), INVALID), (dict(ws=P + 8), INVALID), (dict(ws_bytes=16), INVALID),
    (dict(q=None), INVALID), (dict(dq=None), INVALID), (dict(p=1.0), INVALID), (dict(N=0), INVALID),
    (dict(dtype=7), INVALID),
])
def test_backward_split_rejects(lib, kw, expect):
    assert bsplit(lib, **kw) == expect


def test_backward_split_rejects_workspace_one_byte_short(lib):
    need = lib.fa_bwd_split_workspace_size(2, 3, 100, 128, binding.FA_BF16, 4)
    assert bsplit(lib, B=2, H=3, N=100, d=128, splits=4, ws_bytes=need - 1) == INVALID


def noalloc(lib, ptrs=None, B=1, H=1, N=128, d=64, dtype=binding.FA_BF16, scale=0.125, p=0.0):
    ptrs = ptrs or [P] * 9
    return lib.fa_bwd_noalloc(*ptrs, B, H, N, d, dtype, scale, 0, None, p, 0, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=0), INVALID), (dict(scale=float("nan")), INVALID), (dict(p=1.0), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(dtype=binding.FA_F32, p=0.1), UNSUPPORTED),
    (dict(N=1 << 24, d=128), UNSUPPORTED),
    # one query row past the fixed scratch (2 x 4 bytes per row): refused on the
    # host before any HIP call
    (dict(B=1, H=1, N=(1 << 22) + 1), binding.FA_ERR_TOO_LARGE),
    (dict(B=4, H=32, N=32768 + 64), binding.FA_ERR_TOO_LARGE),
])
def test_noalloc_rejects(lib, kw, expect):
    assert noalloc(lib, **kw) == expect


@pytest.mark.parametrize("idx", range(9))
def test_noalloc_rejects_null_tensor(lib, idx):
    ptrs = [P] * 9
    ptrs[idx] = None
    assert noalloc(lib, ptrs=ptrs) == INVALID


def test_noalloc_limit_is_the_workspace_of_4m_rows(lib):
    # the largest accepted size fills the scratch exactly
    assert lib.fa_bwd_workspace_size(1, 1, 1 << 22, 64, binding.FA_BF16) == \
        binding.FA_NOALLOC_SCRATCH_BYTES
    assert lib.fa_bwd_workspace_size(1, 1, (1 << 22) + 1, 64, binding.FA_BF16) > \
        binding.FA_NOALLOC_SCRATCH_BYTES


# ---- fa_fwd_strided / fa_bwd_strided: the fa_strides rules of include/fa.h
#
# No call here may pass every check: it would launch kernels on the dummy
# pointers.  Strides that are accepted are shown with a later check failing
# instead (fp32 with dropout, UNSUPPORTED only once the strides have passed).


def contig(H, N, d):
    return (H * N * d, N * d, d)


def strides_arr(rows):
    arr = (binding.FaStrides * len(rows))()
    for a, (b, h, n) in zip(arr, rows):
        a.batch, a.head, a.row = b, h, n
    return arr


def fwd_s(lib, rows, B=2, H=2, N=128, d=64, dtype=binding.FA_BF16, p=0.0):
    return lib.fa_fwd_strided(*([P] * 5), strides_arr(rows), B, H, N, d, dtype, 0.125, 0, None, p, 0,
                              None)


def fwd_s_accepts(lib, rows, **kw):
    """The strides pass (fp32 + dropout is then the first check to fail)."""
    return fwd_s(lib, rows, dtype=binding.FA_F32, p=0.1, **kw) == UNSUPPORTED


def bwd_s(lib, rows, B=2, H=2, N=128, d=64, dtype=binding.FA_BF16, p=0.0):
    ws_bytes = lib.fa_bwd_workspace_size(B, H, N, d, binding.FA_BF16)
    return lib.fa_bwd_strided(*([P] * 9), strides_arr(rows), B, H, N, d, dtype, 0.125, 0, None, p,
                              0, P, ws_bytes, None)


def bwd_s_accepts(lib, rows):
    """The strides pass (fp32 with dropout is then the first check to fail)."""
    return bwd_s(lib, rows, dtype=binding.FA_F32, p=0.1) == UNSUPPORTED


@pytest.mark.parametrize("which", range(4))
@pytest.mark.parametrize("bad,expect", [
    ((0, 0, 32), INVALID),                 # row < d
    ((-64, 64, 64), INVALID),              # negative batch stride
    ((2 * 128 * 64, 128 * 64, 68), INVALID),  # row not a multiple of 8 bf16 elements
    ((2 * 128 * 64 + 4, 128 * 64, 64), INVALID),  # batch not 16-byte aligned
    ((2 * 128 * 64, 128 * 64, 1 << 23), UNSUPPORTED),  # (N + 256) rows span > 2^32 bytes
])
def test_strided_forward_rejects_bad_strides(lib, which, bad, expect):
    rows = [contig(2, 128, 64)] * 4
    assert fwd_s_accepts(lib, rows)
    rows[which] = bad
    assert fwd_s(lib, rows) == expect


def test_strided_output_rows_must_not_overlap(lib):
    good = contig(2, 128, 64)
    # o with head stride 0: two heads would write the same rows
    assert fwd_s(lib, [good] * 3 + [(2 * 128 * 64, 0, 64)]) == INVALID
    # o rows 64 apart but heads only 64 * 100 apart: head 1 overlaps rows 100.. of head 0
    assert fwd_s(lib, [good] * 3 + [(2 * 128 * 64, 64 * 100, 64)]) == INVALID
    # [B, N, H, d] memory (rows H * d apart, heads d apart) is a valid output,
    # and so are rows with gaps between them
    bnhd = (128 * 2 * 64, 64, 2 * 64)
    assert fwd_s_accepts(lib, [good] * 3 + [bnhd])
    assert fwd_s_accepts(lib, [good] * 3 + [(2 * 128 * 72, 128 * 72, 72)])
    # an input may repeat rows (head stride 0): only outputs must be one-to-one
    assert fwd_s_accepts(lib, [good, (2 * 128 * 64, 0, 64), good, good])


@pytest.mark.parametrize("which,expect", [(0, INVALID), (4, INVALID), (5, INVALID), (7, INVALID)])
def test_strided_backward_rejects_bad_strides(lib, which, expect):
    rows = [contig(2, 128, 64)] * 8
    assert bwd_s_accepts(lib, rows)
    rows[which] = (0, 0, 32)
    assert bwd_s(lib, rows) == expect


def test_strided_backward_outputs_must_not_overlap(lib):
    rows = [contig(2, 128, 64)] * 8
    rows[6] = (0, 128 * 64, 64)  # dk: both batch entries on the same rows
    assert bwd_s(lib, rows) == INVALID
    rows[6] = contig(2, 128, 64)
    rows[1] = (0, 128 * 64, 64)  # k: an input may be shared across the batch
    assert bwd_s_accepts(lib, rows)


def test_fp16_is_a_16_bit_type_everywhere(lib):
    f16 = binding.FA_F16
    assert fwd(lib, dtype=f16, d=48) == UNSUPPORTED   # recognised, d still checked
    assert fwd(lib, dtype=f16, p=1.0) == INVALID
    assert fwd(lib, dtype=3) == INVALID
    assert lib.fa_bwd_workspace_size(1, 1, 128, 64, f16) == \
        lib.fa_bwd_workspace_size(1, 1, 128, 64, binding.FA_BF16)
    assert lib.fa_fwd_split_workspace_size(1, 1, 128, 64, f16, 2) == \
        lib.fa_fwd_split_workspace_size(1, 1, 128, 64, binding.FA_BF16, 2)
    assert bwd(lib, dtype=f16, d=48) == UNSUPPORTED
    # fp16 rows of 16 bytes: strides in units of 8 elements, like bf16
    rows = [contig(2, 128, 64)] * 4
    rows[0] = (2 * 128 * 64, 128 * 64, 68)
    assert fwd_s(lib, rows, dtype=f16) == INVALID
    # fp32 rows: units of 4 elements
    assert fwd_s_accepts(lib, rows)


# ---- fa_fwd_varlen / fa_bwd_varlen: packed sequences (host offsets)


def cu_arr(vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def fwd_v(lib, cu, H=2, d=64, dtype=binding.FA_BF16, p=0.0, strides=None, ptrs=None):
    ptrs = ptrs or [P] * 5
    n = len(cu) - 1 if cu is not None else 1
    return lib.fa_fwd_varlen(*ptrs, strides, cu_arr(cu) if cu is not None else None, n, H, d, dtype,
                             0.125, 0, p, 0, None)


def test_varlen_rejects_bad_offsets(lib):
    assert fwd_v(lib, None) == INVALID                 # no offsets
    assert lib.fa_fwd_varlen(*([P] * 5), None, cu_arr([0]), 0, 2, 64, binding.FA_BF16, 0.125, 0,
                             0.0, 0, None) == INVALID  # no sequence
    assert fwd_v(lib, [3, 10]) == INVALID              # must start at 0
    assert fwd_v(lib, [0, 10, 5]) == INVALID           # must not decrease
    assert fwd_v(lib, [0, 10], d=48) == UNSUPPORTED
    assert fwd_v(lib, [0, 10], dtype=7) == INVALID
    assert fwd_v(lib, [0, 10], ptrs=[P, P, P, P + 8, P]) == INVALID  # o misaligned
    # LSE needs 4-byte alignment only (sequence blocks start at H * offset);
    # accepted here, then fp32 + dropout is the first check to fail
    assert fwd_v(lib, [0, 3, 10], ptrs=[P, P, P, P, P + 4], dtype=binding.FA_F32, p=0.1) == UNSUPPORTED
    assert fwd_v(lib, [0, 3, 10], ptrs=[P, P, P, P, P + 2]) == INVALID


def test_varlen_strides_are_checked_over_all_tokens(lib):
    T, H, d = 40, 2, 64
    packed = (0, d, H * d)
    good = strides_arr([packed] * 4)
    assert fwd_v(lib, [0, 15, 40], strides=good, dtype=binding.FA_F32, p=0.1) == UNSUPPORTED
    # o rows 64 apart with 2 heads: heads overlap the next token's rows
    bad = strides_arr([packed] * 3 + [(0, d, d)])
    assert fwd_v(lib, [0, 15, 40], strides=bad) == INVALID
    # only empty sequences: no token, nothing to check against, nothing launched
    assert fwd_v(lib, [0, 0, 0], strides=bad) == OK


def test_varlen_backward_workspace_and_rejects(lib):
    ws = lib.fa_bwd_varlen_workspace_size
    # the per-row terms of the longest sequence, reused by the others
    assert ws(cu_arr([0, 100, 130, 380]), 3, 2, 64, binding.FA_BF16) == \
        lib.fa_bwd_workspace_size(1, 2, 250, 64, binding.FA_BF16)
    assert ws(cu_arr([0, 0]), 1, 2, 64, binding.FA_BF16) == 0
    assert ws(cu_arr([2, 5]), 1, 2, 64, binding.FA_BF16) == 0
    need = ws(cu_arr([0, 100, 130]), 2, 2, 64, binding.FA_BF16)
    call = lambda cu, dt=binding.FA_BF16, wsb=need, p=0.0: lib.fa_bwd_varlen(
        *([P] * 9), None, cu_arr(cu), len(cu) - 1, 2, 64, dt, 0.125, 0, p, 0, P, wsb, None)
    assert call([0, 100, 130], wsb=need - 1) == INVALID
    assert call([0, 100, 90]) == INVALID
    assert call([0, 100, 130], dt=binding.FA_F32, p=0.1) == UNSUPPORTED


# ---- fa_fwd_varlen_device / fa_bwd_varlen_device: packed sequences (device offsets)


def fwd_vd(lib, n=2, max_len=64, total=100, H=2, d=64, dtype=binding.FA_BF16, p=0.0, strides=None,
           ptrs=None, cu=P, scale=0.125):
    ptrs = ptrs or [P] * 5
    return lib.fa_fwd_varlen_device(*ptrs, strides, cu, n, max_len, total, H, d, dtype, scale, 0, p,
                                    0, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(cu=None), INVALID), (dict(cu=P + 2), INVALID), (dict(n=0), INVALID),
    (dict(max_len=-1), INVALID), (dict(total=-1), INVALID), (dict(H=0), INVALID),
    (dict(dtype=7), INVALID), (dict(scale=0.0), INVALID), (dict(p=1.0), INVALID),
    (dict(d=48), UNSUPPORTED),
    # one launch needs the MFMA kernels: 16-bit, d <= 128
    (dict(dtype=binding.FA_F32), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(ptrs=[P, P, P, P + 8, P]), INVALID), (dict(ptrs=[P, P, P, P, P + 2]), INVALID),
    # o rows 64 apart with 2 heads: heads overlap the next token's rows
    (dict(strides=strides_arr([(0, 64, 128)] * 3 + [(0, 64, 64)])), INVALID),
])
def test_varlen_device_rejects(lib, kw, expect):
    assert fwd_vd(lib, **kw) == expect


def test_varlen_device_empty_is_a_no_op(lib):
    # no row at all: nothing to compute and nothing launched
    assert fwd_vd(lib, max_len=0) == OK
    assert fwd_vd(lib, total=0) == OK


def test_varlen_device_backward_workspace_and_rejects(lib):
    ws = lib.fa_bwd_varlen_device_workspace_size
    # D and LSE * log2(e) of every token and head, each padded to 256 bytes
    assert ws(1000, 3, 64, binding.FA_BF16) == 2 * ((1000 * 3 * 4 + 255) // 256) * 256
    assert ws(-1, 3, 64, binding.FA_BF16) == 0
    assert ws(10, 3, 48, binding.FA_BF16) == 0
    need = ws(100, 2, 64, binding.FA_BF16)

    def call(wsb=need, dt=binding.FA_BF16, d=64, cu=P, n=2, ptrs=None):
        ptrs = ptrs or [P] * 9
        return lib.fa_bwd_varlen_device(*ptrs, None, cu, n, 64, 100, 2, d, dt, 0.125, 0, 0.0, 0, P,
                                        wsb, None)
    assert call(wsb=need - 1) == INVALID
    assert call(cu=None) == INVALID
    assert call(n=0) == INVALID
    assert call(dt=binding.FA_F32) == UNSUPPORTED
    assert call(d=256, wsb=1 << 30) == UNSUPPORTED
    assert call(ptrs=[P] * 6 + [None] + [P] * 2) == INVALID
