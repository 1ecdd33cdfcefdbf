"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/sherry.h declares, answers the size queries, and rejects every bad
argument before any launch.

Every rejected call here has exactly one invalid argument, and each check
returns before anything is enqueued, so no kernel ever sees the fake (but
aligned) device addresses used below.
"""

import os
import re

import pytest

from conftest import ROOT

S = pytest.importorskip("ternary_weight_quantization_sparse_amd")
L = S._lib

FAKE = 0x10000          # aligned, never dereferenced (the call fails validation first)
FAKE2 = 0x20000
MIS = 0x10008           # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    return L.load()


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "sherry.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sherry_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_symbols()
    assert len(declared) == 16
    assert set(declared) == set(L.SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.sherry_abi_version() == 2
    for code in range(11):
        assert lib.sherry_status_string(code).decode().startswith("SHERRY_")
    assert b"unknown" in lib.sherry_status_string(99)


def test_size_queries(lib):
    assert lib.sherry_packed_bytes(256, 512) == 256 * 512 * 5 // 32
    assert lib.sherry_packed_bytes(8192, 8192) == 10485760
    assert lib.sherry_packed_bytes(2048, 100) == 0
    assert lib.sherry_num_scales(8192, 8192, L.PER_GROUP, 128) == 524288
    assert lib.sherry_num_scales(8192, 8192, L.PER_CHANNEL, 128) == 8192
    assert lib.sherry_num_scales(8192, 8192, L.PER_TENSOR, 128) == 1
    assert lib.sherry_num_scales(8, 130, L.PER_GROUP, 128) == -1
    # quantize workspace, rows of up to 512 superblocks: none for per_group and
    # per_channel (the scales are finished in the pack kernel); per_tensor keeps
    # one partial per 8-row group when K/128 is a power of two (else every
    # superblock sum), plus two level buffers of ceil(partials / 4096)
    assert lib.sherry_workspace_bytes(L.OP_QUANTIZE_PACK, 64, 512, L.PER_GROUP, 128, 1, 1) == 0
    assert lib.sherry_workspace_bytes(L.OP_QUANTIZE_PACK, 64, 512, L.PER_GROUP, 256, 1, 1) == 0
    assert lib.sherry_workspace_bytes(L.OP_QUANTIZE_PACK, 64, 512, L.PER_CHANNEL, 128, 1, 1) == 0
    assert lib.sherry_workspace_bytes(L.OP_QUANTIZE_PACK, 64, 512, L.PER_TENSOR, 128, 1, 1) == (8 + 2) * 4
    assert lib.sherry_workspace_bytes(L.OP_QUANTIZE_PACK, 64, 384, L.PER_TENSOR, 128, 1, 1) == (64 * 3 + 2) * 4
    # longer rows: superblock sums, N*K/128 of them
    assert lib.sherry_workspace_bytes(L.OP_QUANTIZE_PACK, 8, 128 * 600, L.PER_CHANNEL, 128, 1, 1) == 8 * 600 * 4
    assert lib.sherry_workspace_bytes(L.OP_QUANTIZE_PACK, 8, 128 * 600, L.PER_GROUP, 128, 1, 1) == 0
    assert lib.sherry_workspace_bytes(L.OP_UNPACK, 64, 512, L.PER_TENSOR, 128, 1, 1) == 0
    assert lib.sherry_workspace_bytes(L.OP_GEMV, 64, 512, L.PER_GROUP, 128, 17, 1) == (1 << 64) - 1
    assert lib.sherry_workspace_bytes(9, 64, 512, L.PER_GROUP, 128, 1, 1) == (1 << 64) - 1


def qp(lib, n=64, k=512, gran=L.PER_GROUP, g=128, w=FAKE, wd=L.F32, packed=FAKE, alpha=FAKE2,
       ws=None, wsb=0):
    return lib.sherry_quantize_pack(n, k, gran, g, w, wd, packed, alpha, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), L.ERR_SHAPE), (dict(k=0), L.ERR_SHAPE), (dict(k=514), L.ERR_SHAPE),
    (dict(n=-3), L.ERR_SHAPE), (dict(gran=3), L.ERR_GRANULARITY), (dict(gran=-1), L.ERR_GRANULARITY),
    (dict(g=0), L.ERR_GROUP), (dict(g=-128), L.ERR_GROUP), (dict(g=96), L.ERR_GROUP),
    (dict(k=520, g=130), L.ERR_GROUP),
    (dict(k=520, gran=L.PER_TENSOR), L.ERR_UNSUPPORTED), (dict(g=64), L.ERR_UNSUPPORTED),
    (dict(wd=L.I8), L.ERR_DTYPE), (dict(wd=7), L.ERR_DTYPE),
    (dict(w=None), L.ERR_NULL), (dict(packed=None), L.ERR_NULL), (dict(alpha=None), L.ERR_NULL),
    (dict(w=MIS), L.ERR_ALIGN), (dict(packed=MIS), L.ERR_ALIGN), (dict(alpha=MIS), L.ERR_ALIGN),
    (dict(gran=L.PER_TENSOR), L.ERR_WORKSPACE), (dict(gran=L.PER_TENSOR, ws=FAKE, wsb=4), L.ERR_WORKSPACE),
    (dict(k=128 * 600, gran=L.PER_CHANNEL, ws=FAKE, wsb=4), L.ERR_WORKSPACE),
    (dict(k=128 * 600, g=256), L.ERR_WORKSPACE),
])
def test_quantize_pack_rejects(lib, kw, code):
    assert qp(lib, **kw) == code


def up(lib, n=64, k=512, gran=L.PER_GROUP, g=128, packed=FAKE, alpha=FAKE2, out=FAKE, od=L.F32):
    return lib.sherry_unpack(n, k, gran, g, packed, alpha, out, od, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=6), L.ERR_SHAPE), (dict(gran=5), L.ERR_GRANULARITY), (dict(g=100), L.ERR_GROUP),
    (dict(od=9), L.ERR_DTYPE), (dict(packed=None), L.ERR_NULL), (dict(out=None), L.ERR_NULL),
    (dict(alpha=None), L.ERR_NULL), (dict(out=MIS), L.ERR_ALIGN), (dict(k=132, gran=L.PER_TENSOR), L.ERR_UNSUPPORTED),
])
def test_unpack_rejects(lib, kw, code):
    assert up(lib, **kw) == code


def gv(lib, n=64, k=512, gran=L.PER_GROUP, g=128, packed=FAKE, alpha=FAKE2, x=FAKE, b=1, y=FAKE2,
       yd=L.BF16, count=1, ps=0, as_=0, ys=0, ws=None, wsb=0):
    return lib.sherry_gemv(n, k, gran, g, packed, alpha, x, b, y, yd, count, ps, as_, ys, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), L.ERR_SHAPE), (dict(gran=7), L.ERR_GRANULARITY), (dict(g=0), L.ERR_GROUP),
    (dict(yd=L.I8), L.ERR_DTYPE), (dict(x=None), L.ERR_NULL), (dict(alpha=None), L.ERR_NULL),
    (dict(y=None), L.ERR_NULL), (dict(packed=None), L.ERR_NULL), (dict(x=MIS), L.ERR_ALIGN),
    (dict(b=0), L.ERR_BATCH), (dict(b=17), L.ERR_BATCH), (dict(count=0), L.ERR_BATCH),
    (dict(count=2, ps=100, as_=256, ys=64), L.ERR_BATCH),
    (dict(count=2, ps=64 * 512 * 5 // 32, as_=255, ys=64), L.ERR_BATCH),
    (dict(count=2, ps=64 * 512 * 5 // 32, as_=256, ys=63), L.ERR_BATCH),
    (dict(count=2, ps=64 * 512 * 5 // 32 + 8, as_=256, ys=64), L.ERR_ALIGN),
    (dict(count=2, ps=64 * 512 * 5 // 32, as_=258, ys=64), L.ERR_ALIGN),
    (dict(k=520, gran=L.PER_TENSOR), L.ERR_UNSUPPORTED),
])
def test_gemv_rejects(lib, kw, code):
    assert gv(lib, **kw) == code


def test_gemv_workspace_rejected_when_needed(lib):
    # a batch-1 call splits K inside its workgroups (no workspace); at batch 4
    # a 64x512 single call is split across workgroups, which needs one
    assert lib.sherry_workspace_bytes(L.OP_GEMV, 64, 512, L.PER_GROUP, 128, 1, 1) == 0
    need = lib.sherry_workspace_bytes(L.OP_GEMV, 64, 512, L.PER_GROUP, 128, 4, 1)
    assert need > 0
    assert gv(lib, b=4) == L.ERR_WORKSPACE
    assert gv(lib, b=4, ws=FAKE, wsb=need - 4) == L.ERR_WORKSPACE


@pytest.mark.parametrize("n,k,count,split", [
    (3072, 3072, 28, 6),   # 3B q / o over 28 layers: 6 splits of one 4-superblock window
    (1024, 3072, 28, 6),   # 3B k / v: 6, not 8 splits of 3 superblocks
    (8192, 3072, 28, 2),   # 3B gate / up: 2 splits of 12 superblocks
    (3072, 8192, 28, 4),   # 3B down: 4 splits of 16 superblocks
    (2048, 8192, 1, 16),   # a K = 8192 single call: 16 splits, not 64 of one superblock
    (2048, 2048, 1366, 1),  # the 1B headline launches: no split
])
def test_gemv_batch1_split_sizes(lib, n, k, count, split):
    """Batch 1 splits K across workgroups by the largest divisor of the groups
    that keeps the launch within ~2048 workgroups and leaves each split whole
    4-superblock windows; the workspace holds count * split * N fp32
    partials."""
    need = lib.sherry_workspace_bytes(L.OP_GEMV, n, k, L.PER_GROUP, 128, 1, count)
    assert need == (count * split * n * 4 if split > 1 else 0)


def gm(lib, n=64, k=512, gran=L.PER_GROUP, g=128, packed=FAKE, alpha=FAKE2, x=FAKE, m=32, y=FAKE2):
    return lib.sherry_gemm(n, k, gran, g, packed, alpha, x, m, y, None, 0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=2), L.ERR_SHAPE), (dict(gran=9), L.ERR_GRANULARITY), (dict(g=1000), L.ERR_GROUP),
    (dict(x=None), L.ERR_NULL), (dict(y=None), L.ERR_NULL), (dict(y=MIS), L.ERR_ALIGN),
    (dict(m=0), L.ERR_BATCH), (dict(m=-5), L.ERR_BATCH), (dict(k=516, gran=L.PER_TENSOR), L.ERR_UNSUPPORTED),
    (dict(n=8, k=(1 << 21) + 128, gran=L.PER_TENSOR, m=1), L.ERR_UNSUPPORTED),
])
def test_gemm_rejects(lib, kw, code):
    assert gm(lib, **kw) == code


def test_grid_limits_are_unsupported(lib):
    assert lib.sherry_quantize_pack(65535 * 64 + 1, 128, L.PER_TENSOR, 128, FAKE, L.F32, FAKE2, FAKE, None, 0,
                                    None) == L.ERR_UNSUPPORTED
    assert lib.sherry_quantize_pack(1, 128 * 65536, L.PER_TENSOR, 128, FAKE, L.F32, FAKE2, FAKE, None, 0,
                                    None) == L.ERR_UNSUPPORTED


def test_gemm_workspace_rejected_when_needed(lib):
    # 128 rows against a 512x2048 weight give 8 output tiles: the plan splits
    # K, which needs a workspace
    need = lib.sherry_workspace_bytes(L.OP_GEMM, 512, 2048, L.PER_GROUP, 128, 128, 1)
    assert need > 0 and need % (512 * 128 * 4) == 0
    assert gm(lib, n=512, k=2048, m=128) == L.ERR_WORKSPACE
    assert lib.sherry_gemm(512, 2048, L.PER_GROUP, 128, FAKE, FAKE2, FAKE, 128, FAKE2, FAKE, need - 4,
                           None) == L.ERR_WORKSPACE
    assert lib.sherry_gemm(512, 2048, L.PER_GROUP, 128, FAKE, FAKE2, FAKE, 128, FAKE2, MIS, need,
                           None) == L.ERR_ALIGN


def fq(lib, n=64, k=512, gran=L.PER_GROUP, g=128, w=FAKE, wdt=L.F32, out=FAKE2, odt=L.BF16, alpha=FAKE,
       ws=None, wsb=0):
    return lib.sherry_fake_quant(n, k, gran, g, w, wdt, out, odt, alpha, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=2), L.ERR_SHAPE), (dict(gran=9), L.ERR_GRANULARITY), (dict(g=1000), L.ERR_GROUP),
    (dict(wdt=L.I8), L.ERR_DTYPE), (dict(odt=L.I8), L.ERR_DTYPE), (dict(odt=7), L.ERR_DTYPE),
    (dict(w=None), L.ERR_NULL), (dict(out=None), L.ERR_NULL), (dict(alpha=None), L.ERR_NULL),
    (dict(out=MIS), L.ERR_ALIGN), (dict(k=516, gran=L.PER_TENSOR), L.ERR_UNSUPPORTED),
    (dict(gran=L.PER_TENSOR), L.ERR_WORKSPACE), (dict(k=128 * 200, gran=L.PER_CHANNEL), L.ERR_WORKSPACE),
    (dict(k=128 * 200, g=256), L.ERR_WORKSPACE),
])
def test_fake_quant_rejects(lib, kw, code):
    assert fq(lib, **kw) == code


def test_fake_quant_workspace_sizes(lib):
    # one kernel, no workspace: per_group 128 at any K; per_channel and
    # per_group G > 128 with K up to 16384 (128 superblocks).  The rest pack
    # into the workspace first, then unpack.
    for gran, g in ((L.PER_GROUP, 128), (L.PER_CHANNEL, 128), (L.PER_GROUP, 256)):
        assert lib.sherry_workspace_bytes(L.OP_FAKE_QUANT, 64, 512, gran, g, 1, 1) == 0
        assert lib.sherry_workspace_bytes(L.OP_FAKE_QUANT, 64, 16384, gran, g, 1, 1) == 0
    assert lib.sherry_workspace_bytes(L.OP_FAKE_QUANT, 64, 128 * 200, L.PER_GROUP, 128, 1, 1) == 0
    for gran, k in ((L.PER_TENSOR, 512), (L.PER_CHANNEL, 128 * 129), (L.PER_GROUP, 128 * 200)):
        need = lib.sherry_workspace_bytes(L.OP_FAKE_QUANT, 64, k, gran, 128 if gran != L.PER_GROUP else 256, 1, 1)
        assert need >= 64 * k * 5 // 32  # the packed planes
    need = lib.sherry_workspace_bytes(L.OP_FAKE_QUANT, 64, 512, L.PER_TENSOR, 128, 1, 1)
    assert fq(lib, gran=L.PER_TENSOR, ws=FAKE, wsb=need - 4) == L.ERR_WORKSPACE


def ar(lib, n=64, k=512, gran=L.PER_GROUP, g=128, packed=FAKE, alpha=FAKE2, w=FAKE, lam=0.5, x=FAKE2, m=32,
       y=FAKE, ws=None, wsb=0):
    return lib.sherry_arenas_gemm(n, k, gran, g, packed, alpha, w, lam, x, m, y, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=2), L.ERR_SHAPE), (dict(gran=9), L.ERR_GRANULARITY), (dict(g=1000), L.ERR_GROUP),
    (dict(w=None), L.ERR_NULL), (dict(x=None), L.ERR_NULL), (dict(w=MIS), L.ERR_ALIGN),
    (dict(m=0), L.ERR_BATCH), (dict(k=516, gran=L.PER_TENSOR), L.ERR_UNSUPPORTED),
    (dict(n=1 << 18, k=8192, gran=L.PER_TENSOR), L.ERR_UNSUPPORTED),
    (dict(n=512, k=2048, m=128), L.ERR_WORKSPACE),
])
def test_arenas_gemm_rejects(lib, kw, code):
    assert ar(lib, **kw) == code


def test_compare_bytes_and_rejections(lib):
    assert lib.sherry_compare_bytes(L.CMP_2BIT, 3, 256) == 3 * 256 // 4
    assert lib.sherry_compare_bytes(L.CMP_TL2, 3, 256) == 3 * 2 * 40   # K padded to 384
    assert lib.sherry_compare_bytes(L.CMP_TL2, 3, 384) == 3 * 2 * 40
    assert lib.sherry_compare_bytes(2, 3, 256) == 0 and lib.sherry_compare_bytes(0, 3, 100) == 0
    assert lib.sherry_compare_repack(5, 64, 512, FAKE, FAKE2, None) == L.ERR_DTYPE
    assert lib.sherry_compare_repack(0, 64, 516, FAKE, FAKE2, None) == L.ERR_UNSUPPORTED
    assert lib.sherry_compare_repack(0, 64, 512, None, FAKE2, None) == L.ERR_NULL
    assert lib.sherry_compare_repack(1, 64, 512, FAKE, MIS, None) == L.ERR_ALIGN
    g = lib.sherry_compare_gemv
    assert g(3, 64, 512, FAKE, FAKE2, FAKE, FAKE2, 1, 0, 0, 0, None) == L.ERR_DTYPE
    assert g(0, 64, 512, FAKE, None, FAKE, FAKE2, 1, 0, 0, 0, None) == L.ERR_NULL
    assert g(0, 64, 512, FAKE, FAKE2, FAKE, FAKE2, 0, 0, 0, 0, None) == L.ERR_BATCH
    assert g(0, 64, 512, FAKE, FAKE2, FAKE, FAKE2, 2, 64 * 512 // 4 - 16, 64, 64, None) == L.ERR_BATCH
    assert g(1, 64, 512, FAKE, FAKE2, FAKE, FAKE2, 2, 64 * 3 * 40 + 8, 64, 64, None) == L.ERR_ALIGN


def test_fused_packing_refuses_per_tensor():
    torch = pytest.importorskip("torch")
    w = torch.zeros((4, 128))
    with pytest.raises(ValueError):
        S.quantize_pack_fused([w, w], "per_tensor")
    with pytest.raises(ValueError):
        S.quantize_pack_fused([w, torch.zeros((4, 256))], "per_group")


def test_binding_raises_value_error():
    with pytest.raises(ValueError):
        L.check(L.ERR_SHAPE)
    with pytest.raises(NotImplementedError):
        L.check(L.ERR_UNSUPPORTED)
    with pytest.raises(S.SherryError):
        L.check(L.ERR_HIP)
    L.check(L.OK)


def test_arenas_lambda_matches_oracle(lib):
    """The library's cosine schedule against the oracle's, whose values are
    pinned in tests/test_oracle_matmul.py (lambda0 at t = 0, lambda0 (1/2 +
    sqrt(2)/4) at T/4, lambda0 / 2 at T/2, 0 at and after T); the binding
    returns the library's value."""
    import math
    import oracle as O
    lam0, T = 0.75, 1000
    assert lib.sherry_arenas_lambda(0, T, lam0) == lam0
    assert abs(lib.sherry_arenas_lambda(T // 4, T, lam0) - lam0 * (0.5 + math.sqrt(2.0) / 4)) < 1e-15
    assert abs(lib.sherry_arenas_lambda(T // 2, T, lam0) - lam0 / 2) < 1e-15
    assert lib.sherry_arenas_lambda(T, T, lam0) == 0.0
    assert lib.sherry_arenas_lambda(T + 5, T, lam0) == 0.0
    assert lib.sherry_arenas_lambda(3, 0, lam0) == 0.0
    for t in range(0, T + 7, 13):
        assert lib.sherry_arenas_lambda(t, T, lam0) == O.arenas_lambda(t, T, lam0), t
        assert S.arenas_lambda(t, T, lam0) == O.arenas_lambda(t, T, lam0), t
    assert lib.sherry_arenas_lambda(300, 1000, -2.5) == O.arenas_lambda(300, 1000, -2.5)


def test_binding_rejects_host_tensors():
    """The binding refuses tensors that are not on the GPU before calling
    the library: the kernels would dereference a host address."""
    torch = pytest.importorskip("torch")
    w = torch.zeros((64, 256))
    with pytest.raises(ValueError, match="CUDA"):
        S.quantize_pack(w)
    with pytest.raises(ValueError, match="CUDA"):
        S.fake_quant(w)
    pw = S.PackedWeight(torch.zeros(64 * 256 * 5 // 32, dtype=torch.uint8), torch.zeros(128), 64, 256)
    x = torch.zeros((1, 256), dtype=torch.bfloat16)
    for call in (lambda: S.gemv(pw, x), lambda: S.gemm(pw, x), lambda: S.unpack(pw),
                 lambda: S.arenas_gemm(pw, w, 0.5, x), lambda: S.compare_repack(pw, 0),
                 lambda: S.gemv_batched(pw.packed, pw.alpha, 64, 256, x, 1, 0, 0),
                 lambda: S.compare_gemv(0, pw.packed, pw.alpha, 64, 256, x)):
        with pytest.raises(ValueError):
            call()


def test_quantize_noalloc_rejects_before_any_launch(lib):
    """The allocation-free quantize checks its arguments like
    sherry_quantize_pack, and refuses a weight whose workspace exceeds the
    static buffer (8 MiB) before touching the device."""
    f = lib.sherry_quantize_pack_noalloc
    assert f(64, 514, L.PER_GROUP, 128, FAKE, L.F32, FAKE2, FAKE, None) == L.ERR_SHAPE
    assert f(64, 512, L.PER_GROUP, 128, FAKE, L.I8, FAKE2, FAKE, None) == L.ERR_DTYPE
    assert f(64, 512, L.PER_GROUP, 128, None, L.F32, FAKE2, FAKE, None) == L.ERR_NULL
    assert f(64, 512, L.PER_GROUP, 128, MIS, L.F32, FAKE2, FAKE, None) == L.ERR_ALIGN
    # 8192 x 131072 (1024 superblocks a row): 8 Mi superblock sums = 32 MiB
    need = lib.sherry_workspace_bytes(L.OP_QUANTIZE_PACK, 8192, 131072, L.PER_TENSOR, 128, 1, 1)
    assert need > L.QUANTIZE_SCRATCH_BYTES
    assert f(8192, 131072, L.PER_TENSOR, 128, FAKE, L.BF16, FAKE2, FAKE, None) == L.ERR_WORKSPACE
    assert f(8192, 131072, L.PER_CHANNEL, 128, FAKE, L.BF16, FAKE2, FAKE, None) == L.ERR_WORKSPACE
    # 8192 x 49152 per_tensor (384 superblocks, not a power of two): 12 MiB of sums
    assert f(8192, 49152, L.PER_TENSOR, 128, FAKE, L.BF16, FAKE2, FAKE, None) == L.ERR_WORKSPACE
