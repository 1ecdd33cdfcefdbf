"""GPU parity over a seeded sweep of configurations, through the C ABI.

Each case draws its shape, granularity, group size, batch, copy count and
output dtype from a fixed seed, so the list is the same on every run; the
sizes stay small enough for the oracle to finish each case in well under a
second, and cover ragged row counts (off every rows-per-workgroup and
panel step), K from one superblock up to 24, groups of 1-4 superblocks,
batches 1..16 (the batch-1 table kernel and the MFMA kernel), split and
unsplit launches.  Bar as in the other parity tests: codes and scales
bit-exact, products within 1e-3 * sum_k |x_k * alpha(n, k)| of the oracle's
fp64 product (+ half a bf16 ulp for bf16 outputs).
"""

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("ternary_weight_quantization_sparse_amd")

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    S.load()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_np(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_close(y, y_ref, bound, what):
    err = np.abs(np.asarray(y, dtype=np.float64) - y_ref)
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= bound), f"{what}: max err/bound {ratio[worst]:.3g} at {worst}"


def _granularity(g):
    gran = ("per_group", "per_group", "per_channel", "per_tensor")[int(g.integers(0, 4))]
    return gran


def _cases(seed, count, draw):
    g = np.random.default_rng(seed)
    return [draw(g, i) for i in range(count)]


def _draw_gemv(g, i):
    gran = _granularity(g)
    r = int(g.choice([1, 2, 3, 4])) if gran == "per_group" else 1
    nsb = r * int(g.integers(1, max(2, 24 // r + 1)))
    n = int(g.integers(1, 1500))
    batch = int(g.choice([1, 1, 2, 3, 4, 5, 8, 13, 16]))
    count = int(g.choice([1, 1, 1, 2, 3]))
    y_dtype = ("float32", "bfloat16")[int(g.integers(0, 2))]
    return (n, 128 * nsb, gran, 128 * r, batch, count, y_dtype, 9000 + i)


def _draw_gemm(g, i):
    gran = _granularity(g)
    r = int(g.choice([1, 2])) if gran == "per_group" else 1
    nsb = r * int(g.integers(1, max(2, 16 // r + 1)))
    n = int(g.integers(1, 700))
    m = int(g.integers(1, 600))
    return (n, 128 * nsb, m, gran, 128 * r, 9500 + i)


GEMV_CASES = _cases(20261, 40, _draw_gemv)
GEMM_CASES = _cases(20262, 24, _draw_gemm)


def _packed(n, k, gran, gs, seed, dtype):
    """Latent weight (fp32, or its bf16 rounding), packed on the GPU; codes
    and scales checked bit-exact against the oracle."""
    w = WL.latent_weight(n, k, seed)
    if dtype == "bf16":
        bits = WL.f32_to_bf16_bits(w)
        w = WL.bf16_bits_to_f32(bits)
        pw = S.quantize_pack(dev_bf16(bits), gran, gs)
    else:
        pw = S.quantize_pack(dev_f32(w), gran, gs)
    ref_p, ref_a = O.quantize_pack(w, gran, gs)
    assert np.array_equal(to_np(pw.packed), ref_p)
    got_a = to_np(pw.alpha)
    assert np.array_equal(got_a.view(np.uint32), np.ascontiguousarray(ref_a, dtype=np.float32).reshape(-1).view(np.uint32))
    return w, pw, np.asarray(ref_a)


@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: "n%d-k%d-%s%d-B%d-c%d-%s" % c[:7])
def test_gemv_sweep(case):
    n, k, gran, gs, batch, count, y_dtype, seed = case
    print(f"[sweep gemv] n={n} k={k} {gran} G={gs} B={batch} count={count} {y_dtype}", flush=True)
    mats = [_packed(n, k, gran, gs, seed + 31 * c, "bf16" if c % 2 else "f32") for c in range(count)]
    xb, xv = WL.activations_bf16(batch, k, seed + 7)
    if count == 1:
        w, pw, a = mats[0]
        ys = [to_np(S.gemv(pw, dev_bf16(xb), y_dtype))]
    else:
        nbytes, nsc = S.packed_bytes(n, k), S.num_scales(n, k, gran, gs)
        # strides keep the 16-byte alignment the ABI asks for, with padding
        ps, as_ = (nbytes + 256 + 255) // 256 * 256, (nsc + 64 + 63) // 64 * 64
        packed_all = torch.zeros(count * ps, dtype=torch.uint8, device=DEV)
        alpha_all = torch.zeros(count * as_, dtype=torch.float32, device=DEV)
        for c, (_, pw, _) in enumerate(mats):
            packed_all[c * ps:c * ps + nbytes] = pw.packed
            alpha_all[c * as_:c * as_ + nsc] = pw.alpha
        ydt = torch.float32 if y_dtype == "float32" else torch.bfloat16
        y_stride = (batch * n + 8 + 7) // 8 * 8
        y = torch.zeros((count, y_stride), dtype=ydt, device=DEV)
        S.gemv_batched(packed_all, alpha_all, n, k, dev_bf16(xb), count, ps, as_, gran, gs,
                       y_dtype=y_dtype, y=y, y_stride=y_stride)
        yv = to_np(y)
        ys = [yv[c, :batch * n].reshape(batch, n) for c in range(count)]
    for c, (w, _, a) in enumerate(mats):
        yc = ys[c]
        if y_dtype == "bfloat16":
            yc = O.bf16_bits_to_f32(yc)
        wq = O.dequant(O.ternary(w), a, gran, gs)
        y_ref = O.gemv(xv, wq)
        bound = O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, gran, gs),
                                  y_ref if y_dtype == "bfloat16" else None)
        check_close(yc.reshape(batch, n), y_ref, bound, f"gemv copy {c}")


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "n%d-k%d-m%d-%s%d" % c[:5])
def test_gemm_sweep(case):
    n, k, m, gran, gs, seed = case
    print(f"[sweep gemm] n={n} k={k} M={m} {gran} G={gs}", flush=True)
    w, pw, a = _packed(n, k, gran, gs, seed, "f32")
    xb, xv = WL.activations_bf16(m, k, seed + 3)
    y = O.bf16_bits_to_f32(to_np(S.gemm(pw, dev_bf16(xb))))
    wq = O.dequant(O.ternary(w), a, gran, gs)
    y_ref = O.gemm(xv, wq)
    bound = O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, gran, gs), y_ref)
    check_close(y, y_ref, bound, "gemm")
    # the unpacked weight of the same case, bit-exact
    assert np.array_equal(to_np(S.unpack(pw, "int8")), O.ternary(w))
    got = to_np(S.unpack(pw, "float32"))
    assert np.array_equal(got.view(np.uint32), wq.astype(np.float32).view(np.uint32))
