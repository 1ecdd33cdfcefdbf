"""The allocation-free quantize entry point (sherry_quantize_pack_noalloc),
called through the C ABI, against sherry_quantize_pack: packed bytes and
scales bit for bit, on two calls in a row (the second on a smaller weight, so
it reuses the static workspace the first one filled).  The cases that use the
static workspace: per_tensor (one partial per 8 rows when K/128 is a power of
two, else every superblock sum) and rows longer than 512 superblocks
(superblock sums for per_channel and per_group G > 128); and cases that need
none (per_group 128, per_channel and per_group 256 on shorter rows)."""

import ctypes

import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("ternary_weight_quantization_sparse_amd")
L = S._lib

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    S.load()


def _noalloc(w, gran, g=128):
    lib = L.load()
    n, k = w.shape
    packed = torch.full((S.packed_bytes(n, k),), 0xA5, dtype=torch.uint8, device=DEV)
    alpha = torch.full((S.num_scales(n, k, gran, g),), -1.0, dtype=torch.float32, device=DEV)
    code = L.BF16 if w.dtype == torch.bfloat16 else L.F32
    st = lib.sherry_quantize_pack_noalloc(n, k, L.GRANULARITY[gran], g, w.data_ptr(), code, packed.data_ptr(),
                                          alpha.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == L.OK, L.status_string(st)
    return packed, alpha


def _same(pw, packed, alpha, what):
    torch.cuda.synchronize()
    assert torch.equal(pw.packed, packed), f"{what}: packed bytes differ"
    assert torch.equal(pw.alpha.view(torch.int32), alpha.view(torch.int32)), f"{what}: scales differ"


POW2 = [(2048, 8192, 5100), (300, 1024, 5101)]      # K/128 a power of two
OTHER = [(1000, 3072, 5103), (300, 1152, 5104)]     # K/128 = 24, 9
LONG = [(64, 128 * 600, 5105), (8, 128 * 520, 5106)]  # rows past 512 superblocks


@pytest.mark.parametrize("gran,g,shapes", [
    ("per_tensor", 128, POW2), ("per_tensor", 128, OTHER), ("per_channel", 128, LONG),
    ("per_group", 256, LONG), ("per_channel", 128, POW2), ("per_group", 256, POW2),
    ("per_group", 128, POW2), ("per_group", 128, LONG)],
    ids=["tensor-pow2", "tensor-other", "channel-long", "group256-long", "channel-pow2", "group256-pow2",
         "group128-pow2", "group128-long"])
def test_noalloc_matches_quantize_pack_two_calls(gran, g, shapes):
    # second call smaller
    for n, k, seed in shapes:
        bits, _ = WL.latent_weight_outliers_bf16(n, k, seed)
        w = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
        print(f"[noalloc] {n}x{k} {gran} G={g}", flush=True)
        packed, alpha = _noalloc(w, gran, g)
        _same(S.quantize_pack(w, gran, g), packed, alpha, f"{n}x{k} {gran}")


def test_noalloc_fp32_and_binding():
    """fp32 weights, and the binding's wrapper over the same entry point."""
    w = torch.from_numpy(WL.latent_weight(640, 2048, 5102)).to(DEV)
    for gran in ("per_tensor", "per_channel"):
        packed, alpha = _noalloc(w, gran)
        _same(S.quantize_pack(w, gran), packed, alpha, f"fp32 {gran}")
        p2 = torch.empty_like(packed)
        a2 = torch.empty_like(alpha)
        pw = S.quantize_pack_noalloc(w, p2, a2, gran)
        _same(pw, packed, alpha, f"binding {gran}")
