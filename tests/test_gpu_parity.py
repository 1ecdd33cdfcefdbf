"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: packed bytes, codes and scales bit-exact; unpacked T / T*alpha /
bf16(T*alpha) bit-exact; GEMV and GEMM outputs within
1e-3 * sum_k |x_k * alpha(n, k)| of the oracle's fp64 product, per element.
Inputs are the seeded synthetic workloads (LLaMA-3.2-1B/3B-shaped linears,
N(0, 0.02) weights, N(0, 1) bf16 activations; the 8192x8192 bf16 quantize
workload with 1% outliers x10).
"""

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
S = pytest.importorskip("ternary_weight_quantization_sparse_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    S.load()


DEV = "cuda:0"


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_np(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_quantize(w_dev, w_vals, gran, g=128):
    n, k = w_vals.shape
    print(f"[quantize] {n}x{k} {gran} G={g} {w_dev.dtype}", flush=True)
    pw = S.quantize_pack(w_dev, gran, g)
    ref_p, ref_a = O.quantize_pack(w_vals, gran, g)
    got_p, got_a = to_np(pw.packed), to_np(pw.alpha)
    ref_a = np.ascontiguousarray(ref_a).reshape(-1)
    assert got_p.size == ref_p.size and got_a.size == ref_a.size
    bad = np.flatnonzero(got_p != ref_p)
    assert bad.size == 0, f"{bad.size} packed bytes differ, first at {bad[:5]}"
    bad_a = np.flatnonzero(got_a.view(np.uint32) != ref_a.view(np.uint32))
    assert bad_a.size == 0, f"{bad_a.size} scales differ, first {bad_a[:5]}"
    return pw, ref_a


def check_close(y, y_ref, bound, what):
    err = np.abs(np.asarray(y, dtype=np.float64) - y_ref)
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= bound), f"{what}: max err/bound {ratio[worst]:.3g} at {worst}"
    return float(ratio.max())


# ------------------------------------------------------------------ quantize
@pytest.mark.parametrize("gran,g", [("per_group", 128), ("per_group", 256), ("per_group", 512),
                                    ("per_channel", 128), ("per_tensor", 128)])
def test_quantize_single_layer(gran, g):
    w = WL.latent_weight(256, 512, WL.SEED_SMALL_W)
    check_quantize(dev_f32(w), w, gran, g)


@pytest.mark.parametrize("n,k", [(1, 128), (63, 384), (65, 640), (100, 256), (3, 1152)])
@pytest.mark.parametrize("gran", ["per_group", "per_channel", "per_tensor"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_ragged(n, k, gran, dtype):
    w = WL.latent_weight(n, k, 7 + n + k)
    if dtype == "bf16":
        bits = WL.f32_to_bf16_bits(w)
        check_quantize(dev_bf16(bits), WL.bf16_bits_to_f32(bits), gran)
    else:
        check_quantize(dev_f32(w), w, gran)


@pytest.mark.parametrize("gran,g", [("per_group", 384), ("per_group", 1152)])
def test_quantize_group_not_power_of_two(gran, g):
    w = WL.latent_weight(70, 1152, 31)
    check_quantize(dev_f32(w), w, gran, g)


@pytest.mark.parametrize("g", [256, 384, 512, 1536])
def test_quantize_bf16_groups_of_several_superblocks(g):
    """bf16 weights, groups of 2, 3, 4 and 12 superblocks (the group tree runs
    over each group's superblock sums after the chunk walk), ragged rows."""
    bits, vals = WL.latent_weight_outliers_bf16(37, 1536, 33)
    check_quantize(dev_bf16(bits), vals, "per_group", g)


@pytest.mark.parametrize("gran", ["per_group", "per_channel", "per_tensor"])
def test_quantize_ties_zeros_signed_zero(gran):
    g = np.random.default_rng(12)
    w = (g.integers(-2, 3, size=(96, 512)) * 0.25).astype(np.float32)
    w[5] = 0.0                      # all-zero row
    w[7, ::3] = -0.0                # negative zeros
    w[9, :128] = 0.5                # constant magnitude (all ties)
    w[9, 128:256] = -0.5
    check_quantize(dev_f32(w), w, gran)
    bits = WL.f32_to_bf16_bits(w)
    check_quantize(dev_bf16(bits), WL.bf16_bits_to_f32(bits), gran)


@pytest.mark.parametrize("gran", ["per_group", "per_channel", "per_tensor"])
@pytest.mark.parametrize("k", [1024, 128 * 40])
def test_quantize_bf16_special_patterns(gran, k):
    """bf16 blocks built from signed zeros, subnormals, the smallest normal,
    +-1 and its neighbour and large finite values: every ordered block of 4
    over six of them (ties of equal magnitude and opposite sign, zeros kept
    beside a zero), then random blocks over the whole set.  The kernel
    compares bf16 magnitudes as integers; the oracle compares the values."""
    enum = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3F80, 0xBF80], np.uint16)
    extra = np.array([0x007F, 0x807F, 0x0080, 0x8080, 0x3F81, 0xBF81, 0x7000, 0xF000, 0x0100], np.uint16)
    pool = np.concatenate([enum, extra])
    n = 64
    g = np.random.default_rng(31 + k)
    bits = pool[g.integers(0, pool.size, size=n * k)]
    combos = np.stack(np.meshgrid(*([np.arange(enum.size)] * 4), indexing="ij"), -1).reshape(-1, 4)
    bits[:combos.size] = enum[combos].reshape(-1)
    bits = bits.reshape(n, k)
    vals = WL.bf16_bits_to_f32(bits)
    check_quantize(dev_bf16(bits), vals, gran)
    check_quantize(dev_f32(vals), vals, gran)


@pytest.mark.parametrize("gran", ["per_group", "per_channel", "per_tensor"])
def test_quantize_8192_bf16_outliers(gran):
    bits, vals = WL.latent_weight_outliers_bf16(8192, 8192, 5000)
    check_quantize(dev_bf16(bits), vals, gran)


def test_quantize_deterministic():
    bits, _ = WL.latent_weight_outliers_bf16(1024, 2048, 77)
    wd = dev_bf16(bits)
    for gran in ("per_group", "per_tensor"):
        a = S.quantize_pack(wd, gran)
        b = S.quantize_pack(wd, gran)
        assert torch.equal(a.packed, b.packed) and torch.equal(a.alpha, b.alpha)


# ------------------------------------------------------------------ unpack
@pytest.mark.parametrize("gran,g,n,k", [(gr, g, n, k) for gr, g in [("per_group", 128), ("per_group", 256),
                                                                      ("per_channel", 128), ("per_tensor", 128)]
                                          for n, k in [(256, 512), (37, 384)] if k % g == 0])
def test_unpack(gran, g, n, k):
    w = WL.latent_weight(n, k, 3 + n)
    pw, ref_a = check_quantize(dev_f32(w), w, gran, g)
    t_ref = O.ternary(w)
    assert np.array_equal(to_np(S.unpack(pw, "int8")), t_ref)
    wq = O.dequant(t_ref, ref_a, gran, g).astype(np.float32)   # exact: T in {-1,0,1}
    got = to_np(S.unpack(pw, "float32"))
    assert np.array_equal(got.view(np.uint32), wq.view(np.uint32))
    got_b = to_np(S.unpack(pw, "bfloat16"))
    assert np.array_equal(got_b, O.round_to_bf16_bits(wq))


@pytest.mark.parametrize("gran", ["per_group", "per_tensor"])
@pytest.mark.parametrize("n,k", [(1, 128), (9, 640), (33, 1152), (96, 512)])
def test_unpack_edges(gran, n, k):
    """Row counts off every rows-per-workgroup step (32, 16, 8), an odd number
    of superblock columns, and all-zero rows / groups: their kept weights are
    -1 with alpha 0, so T*alpha is -0.0 there."""
    g = np.random.default_rng(n * 7 + k)
    w = (g.integers(-2, 3, size=(n, k)) * 0.25).astype(np.float32)
    w[0, :128] = 0.0
    if n > 5:
        w[5] = 0.0
    pw, ref_a = check_quantize(dev_f32(w), w, gran)
    t_ref = O.ternary(w)
    assert np.array_equal(to_np(S.unpack(pw, "int8")), t_ref)
    wq = O.dequant(t_ref, ref_a, gran, 128).astype(np.float32)
    assert np.array_equal(to_np(S.unpack(pw, "float32")).view(np.uint32), wq.view(np.uint32))
    assert np.array_equal(to_np(S.unpack(pw, "bfloat16")), O.round_to_bf16_bits(wq))


def test_unpack_8192_bf16_outliers():
    bits, vals = WL.latent_weight_outliers_bf16(8192, 8192, 5000)
    pw = S.quantize_pack(dev_bf16(bits), "per_group", 128)
    t_ref = O.ternary(vals)
    assert np.array_equal(to_np(S.unpack(pw, "int8")), t_ref)
    rows = np.random.default_rng(3).choice(8192, 48, replace=False)
    ref_a = O.alpha(vals[rows], "per_group", 128)
    wq = O.dequant(t_ref[rows], ref_a, "per_group", 128).astype(np.float32)
    assert np.array_equal(to_np(S.unpack(pw, "float32"))[rows].view(np.uint32), wq.view(np.uint32))
    assert np.array_equal(to_np(S.unpack(pw, "bfloat16"))[rows], O.round_to_bf16_bits(wq))


# ------------------------------------------------------------------ gemv
def gemv_case(n, k, wseed, xbits, xvals, gran="per_group", g=128, y_dtype="float32"):
    w = WL.latent_weight(n, k, wseed)
    pw = S.quantize_pack(dev_f32(w), gran, g)
    a = O.alpha(w, gran, g)
    wq = O.dequant(O.ternary(w), a, gran, g)
    y = S.gemv(pw, dev_bf16(xbits), y_dtype)
    yv = to_np(y)
    if y_dtype == "bfloat16":
        yv = O.bf16_bits_to_f32(yv)
    y_ref = O.gemv(xvals, wq)
    bound = O.tolerance_bound(xvals, O.alpha_per_weight(a, n, k, gran, g),
                              y_ref if y_dtype == "bfloat16" else None)
    return check_close(yv, y_ref, bound, f"gemv {n}x{k} {gran} B={xbits.shape[0]}")


@pytest.mark.parametrize("y_dtype", ["float32", "bfloat16"])
def test_gemv_single_layer(y_dtype):
    xb, xv = WL.activations_bf16(1, 512, WL.SEED_SMALL_X)
    print("[gemv] 256x512 B=1", flush=True)
    gemv_case(256, 512, WL.SEED_SMALL_W, xb, xv, y_dtype=y_dtype)


@pytest.mark.parametrize("i", range(7))
def test_gemv_llama1b_layer(i):
    name, n, k = WL.LLAMA_1B[i]
    xb, xv = WL.activations_bf16(1, k, 200)
    print(f"[gemv] 1B {name} {n}x{k}", flush=True)
    gemv_case(n, k, WL.layer_1b_weight_seed(i), xb, xv, y_dtype="bfloat16")


@pytest.mark.parametrize("gran,g", [("per_channel", 128), ("per_tensor", 128), ("per_group", 256),
                                    ("per_group", 384)])
@pytest.mark.parametrize("batch", [1, 3, 16])
def test_gemv_granularities(gran, g, batch):
    xb, xv = WL.activations_bf16(batch, 1536, 41)
    gemv_case(300, 1536, 40, xb, xv, gran, g)


@pytest.mark.parametrize("n,k", [(1, 128), (17, 256), (64, 2048), (257, 640), (4100, 128)])
@pytest.mark.parametrize("batch", [1, 2, 5])
def test_gemv_ragged_and_split(n, k, batch):
    xb, xv = WL.activations_bf16(batch, k, 50 + n)
    gemv_case(n, k, 60 + k, xb, xv)


@pytest.mark.parametrize("batch", [1, 4, 16])
@pytest.mark.parametrize("i", [0, 1, 3, 4, 6])
def test_gemv_llama3b_batches(i, batch):
    name, n, k = WL.LLAMA_3B[i]
    xb, xv = WL.activations_bf16(batch, k, 2000 + batch)
    print(f"[gemv] 3B {name} {n}x{k} B={batch}", flush=True)
    gemv_case(n, k, WL.layer_3b_weight_seed(0, i), xb, xv, y_dtype="bfloat16")


@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_one_hot_exact(batch):
    n, k = 192, 384
    w = WL.latent_weight(n, k, 99)
    pw = S.quantize_pack(dev_f32(w), "per_group", 128)
    a = O.alpha(w, "per_group", 128).reshape(k // 128, n)
    t = O.ternary(w)
    cols = [0, 131, 383, 200][:batch] if batch > 1 else [131]
    xv = np.zeros((batch, k), dtype=np.float32)
    for b, c in enumerate(cols):
        xv[b, c] = 1.0
    y = to_np(S.gemv(pw, dev_bf16(WL.f32_to_bf16_bits(xv)), "float32"))
    for b, c in enumerate(cols):
        expect = (t[:, c].astype(np.float32) * a[c // 128]).astype(np.float32)
        assert np.array_equal(y[b], expect)


def test_gemv_zero_input():
    w = WL.latent_weight(128, 256, 5)
    pw = S.quantize_pack(dev_f32(w))
    for b in (1, 8):
        y = S.gemv(pw, torch.zeros((b, 256), dtype=torch.bfloat16, device=DEV), "float32")
        assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_count_strided(batch):
    """One launch over 3 different matrices with padded strides; the padding
    of y is left untouched."""
    n, k, count = 320, 1024, 3
    nbytes = S.packed_bytes(n, k)
    nsc = S.num_scales(n, k)
    ps, as_, ys = nbytes + 48, nsc + 12, batch * n + 16
    packed_all = torch.zeros(count * ps, dtype=torch.uint8, device=DEV)
    alpha_all = torch.zeros(count * as_, dtype=torch.float32, device=DEV)
    ws, refs = [], []
    for c in range(count):
        w = WL.latent_weight(n, k, 500 + c)
        pw = S.quantize_pack(dev_f32(w))
        packed_all[c * ps:c * ps + nbytes] = pw.packed
        alpha_all[c * as_:c * as_ + nsc] = pw.alpha
        ws.append(w)
        refs.append(O.alpha(w, "per_group", 128))
    xb, xv = WL.activations_bf16(batch, k, 600)
    y = torch.full((count, ys), 7.0, dtype=torch.float32, device=DEV)
    S.gemv_batched(packed_all, alpha_all, n, k, dev_bf16(xb), count, ps, as_, y_dtype="float32",
                   y=y, y_stride=ys)
    yv = to_np(y)
    for c in range(count):
        wq = O.dequant(O.ternary(ws[c]), refs[c], "per_group", 128)
        bound = O.tolerance_bound(xv, O.alpha_per_weight(refs[c], n, k, "per_group", 128))
        check_close(yv[c, :batch * n].reshape(batch, n), O.gemv(xv, wq), bound, f"copy {c}")
        assert np.all(yv[c, batch * n:] == 7.0)


def test_gemv_bench_launch_configuration():
    """The launch the benchmark times: the 1B q projection streamed over >= 1
    GiB of copies in one call; copy 0 against the oracle, every copy equal."""
    import bench
    name, n, k = WL.LLAMA_1B[0]
    w = WL.latent_weight(n, k, WL.layer_1b_weight_seed(0))
    pw = S.quantize_pack(dev_f32(w))
    rep = bench.Replicated(pw, bench.copies_for(n, k, "per_group", 128))
    xb, xv = WL.activations_bf16(1, k, 200)
    print(f"[gemv] bench launch q x {rep.count} copies", flush=True)
    y = rep.gemv(dev_bf16(xb))
    yv = to_np(y)
    a = O.alpha(w, "per_group", 128)
    wq = O.dequant(O.ternary(w), a, "per_group", 128)
    y_ref = O.gemv(xv, wq)
    bound = O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, "per_group", 128), y_ref)
    check_close(O.bf16_bits_to_f32(yv[0, :n]).reshape(1, n), y_ref, bound, "copy 0")
    assert np.all(yv[:, :n] == yv[0:1, :n])


# ------------------------------------------------------------------ gemm
def gemm_case(n, k, m, wseed, xseed, gran="per_group", g=128, rows=None):
    w = WL.latent_weight(n, k, wseed)
    pw = S.quantize_pack(dev_f32(w), gran, g)
    a = O.alpha(w, gran, g)
    xb, xv = WL.activations_bf16(m, k, xseed)
    y = O.bf16_bits_to_f32(to_np(S.gemm(pw, dev_bf16(xb))))
    wq = O.dequant(O.ternary(w), a, gran, g)
    if rows is not None:
        xv, y = xv[rows], y[rows]
    y_ref = O.gemm(xv, wq)
    bound = O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, gran, g), y_ref)
    return check_close(y, y_ref, bound, f"gemm {n}x{k} M={m} {gran}")


@pytest.mark.parametrize("i", range(7))
def test_gemm_llama1b_m512(i):
    name, n, k = WL.LLAMA_1B[i]
    print(f"[gemm] 1B {name} {n}x{k} M=512", flush=True)
    gemm_case(n, k, 512, WL.layer_1b_weight_seed(i), 812)


@pytest.mark.parametrize("i", range(7))
def test_gemm_llama1b_m2048_sampled(i):
    name, n, k = WL.LLAMA_1B[i]
    rows = np.random.default_rng(i).choice(2048, size=96, replace=False)
    print(f"[gemm] 1B {name} {n}x{k} M=2048 (96 sampled rows)", flush=True)
    gemm_case(n, k, 2048, WL.layer_1b_weight_seed(i), 2348, rows=rows)


@pytest.mark.parametrize("n,k,m", [(100, 256, 77), (1, 128, 1), (130, 384, 129), (64, 128, 300)])
@pytest.mark.parametrize("gran,g", [("per_group", 128), ("per_channel", 128), ("per_tensor", 128)])
def test_gemm_ragged(n, k, m, gran, g):
    gemm_case(n, k, m, 900 + n, 5000 + m, gran, g)


@pytest.mark.parametrize("gran,g,k", [("per_group", 128, 256), ("per_group", 256, 512),
                                       ("per_channel", 128, 256), ("per_tensor", 128, 384)])
def test_gemm_wide_tiles_ragged(gran, g, k):
    """Launches with >= 512 tiles of 64 x 256 take the 256-row weight tiles:
    N = 4000 leaves a partial last weight tile (160 rows), M = 2000 a partial
    last activation tile (16 rows); every output is checked."""
    n, m = 4000, 2000
    print(f"[gemm] wide tiles {n}x{k} M={m} {gran} G={g}", flush=True)
    gemm_case(n, k, m, 3100 + k, 3200 + g, gran, g)


@pytest.mark.parametrize("gran", ["per_group", "per_channel", "per_tensor"])
def test_gemm_correlated_inputs(gran):
    """Activation rows drawn from the weight's own stream (x = w / 0.02 for
    the first rows), so |y| approaches sum|x*alpha| on the diagonal: the
    case where the bf16 output rounding dominates the bound."""
    gemm_case(130, 384, 129, 1030, 1030, gran, 128)


@pytest.mark.parametrize("n,k,m", [(512, 2048, 128), (300, 1024, 70), (2048, 8192, 64)])
@pytest.mark.parametrize("gran", ["per_group", "per_channel", "per_tensor"])
def test_gemm_split_k(n, k, m, gran):
    """Few output tiles: the plan splits K into fp32 partials summed by a
    second kernel; the result is checked and must repeat bit for bit."""
    from ternary_weight_quantization_sparse_amd import _lib as L
    need = L.load().sherry_workspace_bytes(L.OP_GEMM, n, k, L.GRANULARITY[gran], 128, m, 1)
    assert need > 0, "expected a split-K plan for this shape"
    print(f"[gemm] split-K {n}x{k} M={m} {gran}", flush=True)
    gemm_case(n, k, m, 960 + n, 961 + m, gran, 128)
    w = WL.latent_weight(n, k, 960 + n)
    pw = S.quantize_pack(dev_f32(w), gran, 128)
    xb, _ = WL.activations_bf16(m, k, 961 + m)
    x = dev_bf16(xb)
    y1 = to_np(S.gemm(pw, x))
    y2 = to_np(S.gemm(pw, x))
    assert np.array_equal(y1, y2)


def test_gemm_rows_past_one_launch():
    """X larger than 2^31 bytes: the host runs the rows in several launches
    (32-bit buffer offsets).  Rows on both sides of each launch boundary and
    the last rows are checked against the oracle."""
    n, k, m = 64, 8192, 140000
    print(f"[gemm] {n}x{k} M={m} (two launches)", flush=True)
    w = WL.latent_weight(n, k, 970)
    pw = S.quantize_pack(dev_f32(w))
    gen = torch.Generator(device="cuda").manual_seed(971)
    x = torch.randn((m, k), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = S.gemm(pw, x)
    chunk = ((2 ** 31 // (2 * k) - 128) // 128) * 128
    rows = np.array(sorted({0, 1, chunk - 2, chunk - 1, chunk, chunk + 1, m - 2, m - 1}))
    xr = x[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    yr = y[torch.from_numpy(rows).cuda()].float().cpu().numpy()
    del x, y
    a = O.alpha(w, "per_group", 128)
    wq = O.dequant(O.ternary(w), a, "per_group", 128)
    y_ref = O.gemm(xr, wq)
    bound = O.tolerance_bound(xr, O.alpha_per_weight(a, n, k, "per_group", 128), y_ref)
    check_close(yr, y_ref, bound, f"gemm {n}x{k} M={m}")


def test_gemm_group_256():
    gemm_case(256, 1024, 192, 950, 951, "per_group", 256)


def test_gemm_one_hot_exact():
    n, k = 160, 256
    w = WL.latent_weight(n, k, 17)
    pw = S.quantize_pack(dev_f32(w))
    a = O.alpha(w, "per_group", 128).reshape(k // 128, n)
    t = O.ternary(w)
    xv = np.zeros((3, k), dtype=np.float32)
    cols = [0, 129, 255]
    for r, c in enumerate(cols):
        xv[r, c] = 1.0
    y = to_np(S.gemm(pw, dev_bf16(WL.f32_to_bf16_bits(xv))))
    for r, c in enumerate(cols):
        expect = O.round_to_bf16_bits((t[:, c].astype(np.float32) * a[c // 128]).astype(np.float32))
        assert np.array_equal(y[r], expect)


@pytest.mark.parametrize("n,nsb", [(5, 65), (3, 600), (2, 1030), (9, 64), (7, 1)])
def test_quantize_per_channel_reduction_paths(n, nsb):
    """Rows of 65, 600 and 1030 superblocks exercise the lane-blocked wave
    reductions and the sequential fallback."""
    w = WL.latent_weight(n, 128 * nsb, 70 + nsb)
    check_quantize(dev_f32(w), w, "per_channel")


@pytest.mark.parametrize("n,k", [(1000, 128 * 9), (4096, 128), (33, 128 * 131), (70000, 128),
                                 (40, 128 * 64)])
def test_quantize_per_tensor_multi_level(n, k):
    """More than 4096 superblock sums (or, for power-of-two rows, more than
    4096 16-row partials): the tree runs over two or three levels."""
    w = WL.latent_weight(n, k, 90 + n)
    check_quantize(dev_f32(w), w, "per_tensor")


@pytest.mark.parametrize("gran,g", [("per_group", 128), ("per_group", 256), ("per_channel", 128),
                                    ("per_tensor", 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_rows_past_512_superblocks(gran, g, dtype):
    """Rows longer than 512 superblocks take the superblock-tile kernel."""
    w = WL.latent_weight(5, 128 * 600, 61)
    if dtype == "bf16":
        bits = WL.f32_to_bf16_bits(w)
        check_quantize(dev_bf16(bits), WL.bf16_bits_to_f32(bits), gran, g)
    else:
        check_quantize(dev_f32(w), w, gran, g)


# ------------------------------------------------------------------ fake quant
@pytest.mark.parametrize("n,k,gran,g", [(n, k, gr, g) for n, k in [(256, 512), (130, 384), (1, 128), (19, 1536),
                                                                     (9, 128 * 130)]
                                          for gr, g in [("per_group", 128), ("per_group", 256), ("per_group", 384),
                                                        ("per_channel", 128), ("per_tensor", 128)]
                                          if k % g == 0])
@pytest.mark.parametrize("odt", ["float32", "bfloat16"])
@pytest.mark.parametrize("wdt", ["f32", "bf16"])
def test_fake_quant_matches_oracle(n, k, gran, g, odt, wdt):
    """Dense T * alpha and the scales, bit for bit: fp32 exactly, bf16 as the
    nearest-even rounding of the fp32 product.  Covers the three kernels:
    per_group 128 fused, per_channel / per_group G > 128 fused in the
    row-group kernel (K up to 128 superblocks), and quantize + unpack (per
    tensor; rows of 130 superblocks)."""
    w = WL.latent_weight(n, k, 40 + n)
    if wdt == "bf16":
        bits = WL.f32_to_bf16_bits(w)
        w, wd = WL.bf16_bits_to_f32(bits), dev_bf16(bits)
    else:
        wd = dev_f32(w)
    out, a = S.fake_quant(wd, gran, g, out_dtype=getattr(torch, odt))
    ref, ref_a = O.fake_quant(w, gran, g)
    assert np.array_equal(to_np(a).view(np.uint32), ref_a.reshape(-1).view(np.uint32))
    ref32 = ref.astype(np.float32)
    if odt == "float32":
        assert np.array_equal(to_np(out).view(np.uint32), ref32.view(np.uint32))
    else:
        assert np.array_equal(to_np(out), O.round_to_bf16_bits(ref32))


@pytest.mark.parametrize("gran", ["per_group", "per_channel"])
def test_fake_quant_bf16_outliers_8192(gran):
    """The 8192x8192 bf16 weight with 1% outliers x10, bf16 out (per_group
    128: the fused quantize kernel; per_channel: the row-group kernel's dense
    phase); ties at the block minimum occur here."""
    wb, wv = WL.latent_weight_outliers_bf16(8192, 8192, 5000)
    print(f"[fake-quant] 8192x8192 bf16 outliers {gran}", flush=True)
    out, a = S.fake_quant(dev_bf16(wb), gran, 128)
    ref, ref_a = O.fake_quant(wv, gran, 128)
    assert np.array_equal(to_np(a).view(np.uint32), ref_a.reshape(-1).view(np.uint32))
    assert np.array_equal(to_np(out), O.round_to_bf16_bits(ref.astype(np.float32)))


def test_fake_quant_ste_gradient_passes_through():
    w = dev_f32(WL.latent_weight(64, 256, 44)).requires_grad_(True)
    gy = torch.randn((64, 256), device=DEV, generator=torch.Generator(device=DEV).manual_seed(45))
    y = S.fake_quant_ste(w, "per_group", 128)
    ref, _ = O.fake_quant(w.detach().cpu().numpy(), "per_group", 128)
    assert np.array_equal(to_np(y.detach()).view(np.uint32), ref.astype(np.float32).view(np.uint32))
    (y * gy).sum().backward()
    assert torch.equal(w.grad, gy)


# ------------------------------------------------------------------ fused members

@pytest.mark.parametrize("gran", ["per_group", "per_channel"])
@pytest.mark.parametrize("model,batch", [("1b", 1), ("3b", 1), ("3b", 4)])
def test_fused_qkv_pack_and_gemv(gran, model, batch):
    """q/k/v of a 1B or 3B layer packed as one weight (3072 x 2048 or
    5120 x 3072): every member has the codes and scales of packing it alone,
    and one GEMV launch gives each member's product within tolerance."""
    if model == "1b":
        members = WL.LLAMA_1B[:3]
        ws = [WL.latent_weight(n, k, WL.layer_1b_weight_seed(i)) for i, (_, n, k) in enumerate(members)]
    else:
        members = WL.LLAMA_3B[:3]
        ws = [WL.latent_weight(n, k, WL.layer_3b_weight_seed(0, i)) for i, (_, n, k) in enumerate(members)]
    fw = S.quantize_pack_fused([dev_f32(w) for w in ws], gran, 128)
    k = members[0][2]
    t_all = to_np(S.unpack(fw.pw, "int8"))
    a_all = to_np(fw.pw.alpha)
    a_all = a_all.reshape(k // 128, -1) if gran == "per_group" else a_all.reshape(1, -1)
    xb, xv = WL.activations_bf16(batch, k, 200 + batch)
    print(f"[gemv] fused q/k/v {model} {gran} batch {batch}", flush=True)
    ys = [O.bf16_bits_to_f32(to_np(y)) for y in S.gemv_fused(fw, dev_bf16(xb))]
    r0 = 0
    for w, (name, n, _), y in zip(ws, members, ys):
        t_ref = O.ternary(w)
        a_ref = O.alpha(w, gran, 128)
        a_ref = a_ref.reshape(k // 128, n) if gran == "per_group" else a_ref.reshape(1, n)
        assert np.array_equal(t_all[r0:r0 + n], t_ref), name
        assert np.array_equal(a_all[:, r0:r0 + n].view(np.uint32), a_ref.view(np.uint32)), name
        y_ref = O.gemv(xv, O.dequant(t_ref, a_ref, gran, 128))
        check_close(y, y_ref, O.tolerance_bound(xv, O.alpha_per_weight(a_ref, n, k, gran, 128), y_ref),
                    f"fused {name}")
        r0 += n


@pytest.mark.parametrize("gran", ["per_group", "per_channel"])
def test_fused_qkv_gemm(gran):
    """The prefill GEMM over q/k/v of a 1B layer packed as one 3072 x 2048
    weight (one launch of 64 x 128 tiles, no K split, where k and v alone
    split K): each member's slice within tolerance of the oracle product."""
    members = WL.LLAMA_1B[:3]
    ws = [WL.latent_weight(n, k, WL.layer_1b_weight_seed(i)) for i, (_, n, k) in enumerate(members)]
    fw = S.quantize_pack_fused([dev_f32(w) for w in ws], gran, 128)
    k = members[0][2]
    m = 200
    xb, xv = WL.activations_bf16(m, k, 207)
    print(f"[gemm] fused q/k/v 1b {gran} M={m}", flush=True)
    ys = [O.bf16_bits_to_f32(to_np(y)) for y in S.gemm_fused(fw, dev_bf16(xb))]
    for w, (name, n, _), y in zip(ws, members, ys):
        a_ref = O.alpha(w, gran, 128)
        a_ref = a_ref.reshape(k // 128, n) if gran == "per_group" else a_ref.reshape(1, n)
        y_ref = O.gemm(xv, O.dequant(O.ternary(w), a_ref, gran, 128))
        check_close(y, y_ref, O.tolerance_bound(xv, O.alpha_per_weight(a_ref, n, k, gran, 128), y_ref),
                    f"fused gemm {name}")


@pytest.mark.parametrize("gran", ["per_group", "per_channel"])
@pytest.mark.parametrize("members,m", [("qkv", 512), ("qkv", 2048), ("gateup", 512), ("gateup", 2048)])
def test_fused_gemm_llama1b_bench_sizes(members, m, gran):
    """The fused-weight prefill GEMM at the sizes the benchmark times: q/k/v
    (3072 x 2048) and gate/up (16384 x 2048) of the 1B layer as one weight
    each, at M = 512 (every output of q/k/v; 128 sampled rows of gate/up) and
    M = 2048 (128 sampled rows); each member's slice against the oracle."""
    idx = (0, 1, 2) if members == "qkv" else (4, 5)
    mem = [WL.LLAMA_1B[i] for i in idx]
    ws = [WL.latent_weight(n, k, WL.layer_1b_weight_seed(i)) for i, (_, n, k) in zip(idx, mem)]
    fw = S.quantize_pack_fused([dev_f32(w) for w in ws], gran, 128)
    k = mem[0][2]
    xb, xv = WL.activations_bf16(m, k, 300 + m)
    print(f"[gemm] fused {members} 1b {gran} M={m}", flush=True)
    ys = [O.bf16_bits_to_f32(to_np(y.contiguous())) for y in S.gemm_fused(fw, dev_bf16(xb))]
    rows = None
    if m > 512 or members == "gateup":
        rows = np.random.default_rng(m + len(idx)).choice(m, size=128, replace=False)
    for w, (name, n, _), y in zip(ws, mem, ys):
        a_ref = O.alpha(w, gran, 128)
        a_ref = a_ref.reshape(k // 128, n) if gran == "per_group" else a_ref.reshape(1, n)
        xr, yr = (xv, y) if rows is None else (xv[rows], y[rows])
        y_ref = O.gemm(xr, O.dequant(O.ternary(w), a_ref, gran, 128))
        check_close(yr, y_ref, O.tolerance_bound(xr, O.alpha_per_weight(a_ref, n, k, gran, 128), y_ref),
                    f"fused gemm {members}/{name} M={m}")


# ------------------------------------------------------------------ binding safety
def test_binding_rejects_mismatched_operands():
    """Wrong K, wrong output dtype or size, a non-contiguous output and
    host-side activations are refused with ValueError before any launch."""
    w = WL.latent_weight(128, 256, 11)
    pw = S.quantize_pack(dev_f32(w))
    x_bad_k = torch.zeros((2, 384), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((2, 256), dtype=torch.bfloat16, device=DEV)
    for call in (lambda: S.gemv(pw, x_bad_k), lambda: S.gemm(pw, x_bad_k),
                 lambda: S.gemv(pw, x.float()), lambda: S.gemv(pw, x.cpu()),
                 lambda: S.gemv(pw, x, "float32", out=torch.empty((2, 128), dtype=torch.bfloat16, device=DEV)),
                 lambda: S.gemv(pw, x, "float32", out=torch.empty((2, 100), dtype=torch.float32, device=DEV)),
                 lambda: S.gemm(pw, x, out=torch.empty((128, 2), dtype=torch.bfloat16, device=DEV).t()),
                 lambda: S.gemm(pw, x, out=torch.empty((2, 128), dtype=torch.float32, device=DEV)),
                 lambda: S.arenas_gemm(pw, dev_f32(w), 0.5, x_bad_k),
                 lambda: S.gemv_batched(pw.packed, pw.alpha, 128, 256, x, 2, pw.packed.numel(), 256),
                 lambda: S.gemv_batched(pw.packed, pw.alpha, 128, 512, x, 1, 0, 0),
                 lambda: S.unpack(S.PackedWeight(pw.packed[:100], pw.alpha, 128, 256))):
        with pytest.raises(ValueError):
            call()
    torch.cuda.synchronize()


def test_split_k_on_a_side_stream():
    """Split-K GEMV (batch 1: inside the workgroups; batch 4: across them,
    with a workspace) and GEMM launched on a non-default stream: the binding
    allocates their workspaces on that stream, so the caching allocator
    cannot hand the memory to other work while the kernels run.  Other work
    queued on the default stream meanwhile must not disturb the results."""
    n, k = 512, 2048
    w = WL.latent_weight(n, k, 1500)
    pw = S.quantize_pack(dev_f32(w))
    a = O.alpha(w, "per_group", 128)
    wq = O.dequant(O.ternary(w), a, "per_group", 128)
    for m, kind in ((1, "gemv"), (4, "gemv"), (128, "gemm")):
        # (batch 1 splits K inside its workgroups: no workspace)
        assert (S.workspace_bytes(2 if kind == "gemv" else 3, n, k, "per_group", 128, m, 1) > 0) == (m > 1)
        xb, xv = WL.activations_bf16(m, k, 1501 + m)
        x = dev_bf16(xb)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        outs = []
        for rep in range(3):
            with torch.cuda.stream(side):
                y = S.gemv(pw, x, "float32", stream=side) if kind == "gemv" else S.gemm(pw, x, stream=side)
            outs.append(y)
            junk = torch.full((1 << 22,), float(rep), device=DEV)   # default-stream traffic
            junk.mul_(3.0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        y_ref = O.gemv(xv, wq)
        bound = O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, "per_group", 128),
                                  y_ref if kind == "gemm" else None)
        for y in outs:
            yv = to_np(y)
            if kind == "gemm":
                yv = O.bf16_bits_to_f32(yv)
            check_close(yv, y_ref, bound, f"{kind} on a side stream, M={m}")


# ------------------------------------------------------------------ GEMV splits at scale
@pytest.mark.parametrize("gran", ["per_channel", "per_tensor", "per_group"])
def test_gemv_3b_gate_batch16_all_granularities(gran):
    """8192 x 3072 at batch 16 (131072 outputs, K split over workgroups):
    every output of every granularity against the oracle."""
    n, k = 8192, 3072
    xb, xv = WL.activations_bf16(16, k, 2016)
    print(f"[gemv] 8192x3072 B=16 {gran}", flush=True)
    gemv_case(n, k, WL.layer_3b_weight_seed(0, 4), xb, xv, gran, 128, y_dtype="bfloat16")


@pytest.mark.parametrize("batch,n", [(16, 1024), (3, 2731)])
@pytest.mark.parametrize("gran", ["per_group", "per_channel"])
def test_gemv_batched_many_copies_split(batch, n, gran):
    """count = 8 matrices in one launch with K split and batch * N * count
    above 2^16 outputs; (3, 2731) makes batch * N odd.  Every copy against
    the oracle."""
    k, count = 3072, 8
    nbytes, nsc = S.packed_bytes(n, k), S.num_scales(n, k, gran, 128)
    ps, as_, ys = (nbytes + 255) // 256 * 256, (nsc + 63) // 64 * 64, (batch * n + 7) // 8 * 8 + 8
    packed_all = torch.zeros(count * ps, dtype=torch.uint8, device=DEV)
    alpha_all = torch.zeros(count * as_, dtype=torch.float32, device=DEV)
    wl, refs = [], []
    for c in range(count):
        w = WL.latent_weight(n, k, 1700 + c)
        pw = S.quantize_pack(dev_f32(w), gran)
        packed_all[c * ps:c * ps + nbytes] = pw.packed
        alpha_all[c * as_:c * as_ + nsc] = pw.alpha
        wl.append(w)
        refs.append(O.alpha(w, gran, 128))
    xb, xv = WL.activations_bf16(batch, k, 1710 + batch)
    print(f"[gemv] batched count={count} {n}x{k} B={batch} {gran}", flush=True)
    y = torch.full((count, ys), -3.0, dtype=torch.float32, device=DEV)
    S.gemv_batched(packed_all, alpha_all, n, k, dev_bf16(xb), count, ps, as_, gran, 128, y_dtype="float32",
                   y=y, y_stride=ys)
    yv = to_np(y)
    for c in range(count):
        wq = O.dequant(O.ternary(wl[c]), refs[c], gran, 128)
        bound = O.tolerance_bound(xv, O.alpha_per_weight(refs[c], n, k, gran, 128))
        check_close(yv[c, :batch * n].reshape(batch, n), O.gemv(xv, wq), bound, f"copy {c}")
        assert np.all(yv[c, batch * n:] == -3.0)


def test_gemv_3b_stack_bench_inputs():
    """The 3B-stack weights exactly as the benchmark draws them (torch's
    seeded Philox generator on the GPU) and the launch it times (one batched
    GEMV over the 28 layers' copies, bench.Replicated), for the q and down
    shapes at batch 1 and 4: layers 0 and 27 are copied back, quantized by
    the oracle, and their products checked against the oracle's."""
    import bench
    for i in (0, 6):
        name, n, k = WL.LLAMA_3B[i]
        wl, rep = {}, None
        for layer in range(WL.LLAMA_3B_LAYERS):
            wd = WL.latent_weight_device(n, k, WL.layer_3b_weight_seed(layer, i), DEV)
            pw = S.quantize_pack(wd, "per_group", 128)
            if rep is None:
                rep = bench.Replicated(pw, WL.LLAMA_3B_LAYERS, batch=4)
            else:
                rep.packed_all[layer, :rep.nbytes] = pw.packed
                rep.alpha_all[layer, :rep.nsc] = pw.alpha
            if layer in (0, WL.LLAMA_3B_LAYERS - 1):
                wl[layer] = wd.cpu().numpy()
            del wd, pw
        for batch in (1, 4):
            rep.batch = batch
            wsb = S.workspace_bytes(2, n, k, "per_group", 128, batch, WL.LLAMA_3B_LAYERS)
            rep.ws = torch.empty(wsb, dtype=torch.uint8, device=DEV) if wsb else None
            xb, xv = WL.activations_bf16(batch, k, 2000 + batch)
            print(f"[gemv] 3B bench launch {name} x {WL.LLAMA_3B_LAYERS} layers B={batch}", flush=True)
            y = to_np(rep.gemv(dev_bf16(xb)))
            for layer, w in wl.items():
                a = O.alpha(w, "per_group", 128)
                y_ref = O.gemv(xv, O.dequant(O.ternary(w), a, "per_group", 128))
                got = O.bf16_bits_to_f32(y[layer, :batch * n]).reshape(batch, n)
                check_close(got, y_ref, O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, "per_group", 128), y_ref),
                            f"3B {name} layer {layer} B={batch}")
        del rep
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ Arenas
@pytest.mark.parametrize("n,k,m", [(256, 512, 64), (130, 384, 129), (512, 2048, 128), (2048, 2048, 512),
                                   (1000, 1024, 600), (770, 1024, 650)])
@pytest.mark.parametrize("gran", ["per_group", "per_channel", "per_tensor"])
def test_arenas_gemm_matches_oracle(n, k, m, gran):
    """Y = X (T alpha)^T + lambda X W^T with W the bf16 latent weight, lambda
    from the cosine schedule; several of these shapes split K.  The last two
    have 10 x 8 and 11 x 7 tiles: a short last band of 2 or 3 m-tiles in the
    banded tile order, with and without the per-XCD ranges (77 tiles)."""
    w = WL.latent_weight(n, k, 980 + n)
    wb = WL.f32_to_bf16_bits(w)
    pw = S.quantize_pack(dev_f32(w), gran, 128)
    a = O.alpha(w, gran, 128)
    lam = S.arenas_lambda(300, 1000, 0.5)
    assert lam == O.arenas_lambda(300, 1000, 0.5)
    xb, xv = WL.activations_bf16(m, k, 981 + m)
    print(f"[arenas] {n}x{k} M={m} {gran} lambda={lam:.4f}", flush=True)
    y = O.bf16_bits_to_f32(to_np(S.arenas_gemm(pw, dev_bf16(wb), lam, dev_bf16(xb))))
    wv = WL.bf16_bits_to_f32(wb)
    y_ref = O.arenas_forward(xv, O.dequant(O.ternary(w), a, gran, 128), wv, lam)
    mag = O.alpha_per_weight(a, n, k, gran, 128) + np.abs(np.float32(lam) * wv)
    check_close(y, y_ref, O.tolerance_bound(xv, mag, y_ref), f"arenas {n}x{k} M={m} {gran}")


@pytest.mark.parametrize("i,m", [(4, 2048), (6, 512)])
def test_arenas_gemm_llama1b_sampled(i, m):
    """Full 1B shapes as bench.py launches them, per_group, the schedule's
    lambda: gate at M = 2048 (32 x 64 tiles, four bands of 8 m-tiles) and
    down at M = 512 (K split in 4); 96 sampled output rows against the
    oracle."""
    name, n, k = WL.LLAMA_1B[i]
    w = WL.latent_weight(n, k, WL.layer_1b_weight_seed(i))
    wb = WL.f32_to_bf16_bits(w)
    pw = S.quantize_pack(dev_f32(w), "per_group", 128)
    lam = S.arenas_lambda(300, 1000, 0.5)
    lam_ref = O.arenas_lambda(300, 1000, 0.5)
    assert lam == lam_ref
    xb, xv = WL.activations_bf16(m, k, 1300 + m)
    rows = np.random.default_rng(1400 + i).choice(m, size=96, replace=False)
    print(f"[arenas] 1B {name} {n}x{k} M={m} (96 sampled rows)", flush=True)
    y = O.bf16_bits_to_f32(to_np(S.arenas_gemm(pw, dev_bf16(wb), lam, dev_bf16(xb))))[rows]
    a = O.alpha(w, "per_group", 128)
    wv = WL.bf16_bits_to_f32(wb)
    xr = xv[rows]
    y_ref = O.arenas_forward(xr, O.dequant(O.ternary(w), a, "per_group", 128), wv, lam_ref)
    mag = O.alpha_per_weight(a, n, k, "per_group", 128) + np.abs(np.float32(lam_ref) * wv)
    check_close(y, y_ref, O.tolerance_bound(xr, mag, y_ref), f"arenas 1B {name} M={m}")


def test_arenas_gemm_rows_past_one_launch():
    """The Arenas forward with X larger than 2^31 bytes: the host runs the
    rows in several launches, each over the whole latent weight.  Rows on
    both sides of the launch boundary and the last rows against the oracle."""
    n, k, m = 64, 8192, 140000
    print(f"[arenas] {n}x{k} M={m} (two launches)", flush=True)
    w = WL.latent_weight(n, k, 972)
    wb = WL.f32_to_bf16_bits(w)
    pw = S.quantize_pack(dev_f32(w))
    lam = 0.3
    gen = torch.Generator(device="cuda").manual_seed(973)
    x = torch.randn((m, k), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = S.arenas_gemm(pw, dev_bf16(wb), lam, x)
    chunk = ((2 ** 31 // (2 * k) - 128) // 128) * 128
    rows = np.array(sorted({0, 1, chunk - 2, chunk - 1, chunk, chunk + 1, m - 2, m - 1}))
    xr = x[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    yr = O.bf16_bits_to_f32(to_np(y[torch.from_numpy(rows).cuda()]))
    del x, y
    a = O.alpha(w, "per_group", 128)
    wv = WL.bf16_bits_to_f32(wb)
    lam32 = float(np.float32(lam))
    y_ref = O.arenas_forward(xr, O.dequant(O.ternary(w), a, "per_group", 128), wv, lam32)
    mag = O.alpha_per_weight(a, n, k, "per_group", 128) + np.abs(np.float32(lam32) * wv)
    check_close(yr, y_ref, O.tolerance_bound(xr, mag, y_ref), f"arenas {n}x{k} M={m}")


@pytest.mark.parametrize("lam", [1e-20, 0.003, 3.0, -0.7, 1e25])
def test_arenas_gemm_lambda_range(lam):
    """per_group runs one of two kernels: for 2^-60 <= |lambda| <= 2^60 the
    dense product accumulates with the group sums scaled by alpha / lambda,
    times lambda at the end (a negative lambda included); outside that range
    (here 1e-20 and 1e25) three separate accumulator sets.  Both against the
    oracle."""
    n, k, m = 384, 1024, 96
    w = WL.latent_weight(n, k, 995)
    wb = WL.f32_to_bf16_bits(w)
    pw = S.quantize_pack(dev_f32(w), "per_group", 128)
    a = O.alpha(w, "per_group", 128)
    xb, xv = WL.activations_bf16(m, k, 996)
    print(f"[arenas] lambda={lam}", flush=True)
    y = O.bf16_bits_to_f32(to_np(S.arenas_gemm(pw, dev_bf16(wb), lam, dev_bf16(xb))))
    wv = WL.bf16_bits_to_f32(wb)
    lam32 = float(np.float32(lam))
    y_ref = O.arenas_forward(xv, O.dequant(O.ternary(w), a, "per_group", 128), wv, lam32)
    mag = O.alpha_per_weight(a, n, k, "per_group", 128) + np.abs(np.float32(lam32) * wv)
    check_close(y, y_ref, O.tolerance_bound(xv, mag, y_ref), f"arenas lambda={lam}")


def test_arenas_gemm_lambda_zero_is_the_sherry_product():
    n, k, m = 300, 1024, 70
    w = WL.latent_weight(n, k, 990)
    pw = S.quantize_pack(dev_f32(w))
    xb, _ = WL.activations_bf16(m, k, 991)
    x = dev_bf16(xb)
    y0 = O.bf16_bits_to_f32(to_np(S.arenas_gemm(pw, dev_f32(w), 0.0, x)))
    y1 = O.bf16_bits_to_f32(to_np(S.gemm(pw, x)))
    assert np.array_equal(y0, y1)


# ------------------------------------------------------------------ comparison packings
@pytest.mark.parametrize("n,k", [(256, 512), (130, 384), (300, 2048), (2048, 8192)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_compare_repack_and_gemv(n, k, fmt):
    """Padded 2-bit / three-in-five packings of the Sherry ternary matrix:
    bytes equal the oracle's encoding, and the per-channel GEMV over them is
    within tolerance of the oracle product."""
    w = WL.latent_weight(n, k, 1200 + n)
    pw = S.quantize_pack(dev_f32(w), "per_channel")
    planes = S.compare_repack(pw, fmt)
    t = O.ternary(w)
    if n * k <= 300 * 2048:
        ref = O.encode_2bit(t) if fmt == 0 else O.encode_tl2(t)
        assert np.array_equal(to_np(planes), ref)
    else:
        # large shape: the records of sampled rows, each encoded on its own
        got = to_np(planes)
        assert got.size == O.compare_bytes(fmt, n, k)
        rec = 32 if fmt == 0 else 40
        nsb = O.k_padded(fmt, k) // (128 if fmt == 0 else 192)
        for r in (0, 7, n // 2, n - 1):
            one = O.encode_2bit(t[r:r + 1]) if fmt == 0 else O.encode_tl2(t[r:r + 1])
            for g in range(nsb):
                assert np.array_equal(got[(g * n + r) * rec:(g * n + r + 1) * rec], one[g * rec:(g + 1) * rec]), (r, g)
    a = O.alpha(w, "per_channel", 128)
    xb, xv = WL.activations_bf16(1, k, 1201)
    print(f"[compare] fmt {fmt} {n}x{k}", flush=True)
    y = O.bf16_bits_to_f32(to_np(S.compare_gemv(fmt, planes, pw.alpha, n, k, dev_bf16(xb))))
    wq = O.dequant(t, a, "per_channel", 128)
    y_ref = O.gemv(xv, wq)
    check_close(y, y_ref, O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, "per_channel", 128), y_ref),
                f"compare fmt {fmt} {n}x{k}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_compare_gemv_count_strides(fmt):
    n, k, count = 300, 1024, 3
    ws = [WL.latent_weight(n, k, 1300 + c) for c in range(count)]
    pws = [S.quantize_pack(dev_f32(w), "per_channel") for w in ws]
    planes = [S.compare_repack(pw, fmt) for pw in pws]
    nb = planes[0].numel()
    ps = (nb + 255) // 256 * 256
    allp = torch.zeros((count, ps), dtype=torch.uint8, device=DEV)
    alla = torch.zeros((count, 304), dtype=torch.float32, device=DEV)
    for c in range(count):
        allp[c, :nb] = planes[c]
        alla[c, :n] = pws[c].alpha
    xb, xv = WL.activations_bf16(1, k, 1310)
    y = torch.empty((count, 304), dtype=torch.bfloat16, device=DEV)
    S.compare_gemv(fmt, allp, alla, n, k, dev_bf16(xb), count, ps, 304, y, 304)
    yv = O.bf16_bits_to_f32(to_np(y))
    for c in range(count):
        a = O.alpha(ws[c], "per_channel", 128)
        y_ref = O.gemv(xv, O.dequant(O.ternary(ws[c]), a, "per_channel", 128))
        check_close(yv[c:c + 1, :n], y_ref,
                    O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, "per_channel", 128), y_ref), f"copy {c}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_compare_gemv_many_copies(fmt):
    """A launch large enough for the 2-bit kernel's 512-row workgroups (2100
    copies of a 1000 x 384 matrix, the last workgroup of each copy ragged):
    the first and last copies against the oracle, every copy equal to the
    first."""
    n, k, count = 1000, 384, 2100
    w = WL.latent_weight(n, k, 1400)
    pw = S.quantize_pack(dev_f32(w), "per_channel")
    planes = S.compare_repack(pw, fmt)
    nb = planes.numel()
    ps = (nb + 255) // 256 * 256
    as_ = 1024
    allp = torch.empty((count, ps), dtype=torch.uint8, device=DEV)
    allp[:, :nb] = planes
    alla = torch.empty((count, as_), dtype=torch.float32, device=DEV)
    alla[:, :n] = pw.alpha
    xb, xv = WL.activations_bf16(1, k, 1410)
    y = torch.empty((count, as_), dtype=torch.bfloat16, device=DEV)
    print(f"[compare] fmt {fmt} {n}x{k} x {count} copies", flush=True)
    S.compare_gemv(fmt, allp, alla, n, k, dev_bf16(xb), count, ps, as_, y, as_)
    yv = to_np(y)[:, :n]
    assert np.array_equal(yv, np.broadcast_to(yv[0], yv.shape))
    a = O.alpha(w, "per_channel", 128)
    y_ref = O.gemv(xv, O.dequant(O.ternary(w), a, "per_channel", 128))
    bound = O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, "per_channel", 128), y_ref)
    for c in (0, count - 1):
        check_close(O.bf16_bits_to_f32(yv[c:c + 1]), y_ref, bound, f"copy {c}")


@pytest.mark.parametrize("gran", ["per_group", "per_channel"])
def test_gemv_512_row_panels_ragged(gran):
    """Batch 1 over 1100 copies of a 1000 x 384 matrix: enough workgroups for
    the 512-row panels, the second panel of each copy ragged (488 rows);
    the first and last copies against the oracle, every copy equal."""
    n, k, count = 1000, 384, 1100
    w = WL.latent_weight(n, k, 1500)
    pw = S.quantize_pack(dev_f32(w), gran)
    nb, nsc = S.packed_bytes(n, k), S.num_scales(n, k, gran, 128)
    ps, as_ = (nb + 255) // 256 * 256, (nsc + 63) // 64 * 64
    allp = torch.empty((count, ps), dtype=torch.uint8, device=DEV)
    allp[:, :nb] = pw.packed
    alla = torch.empty((count, as_), dtype=torch.float32, device=DEV)
    alla[:, :nsc] = pw.alpha
    xb, xv = WL.activations_bf16(1, k, 1510)
    ys = 1024
    y = torch.empty((count, ys), dtype=torch.float32, device=DEV)
    print(f"[gemv] {n}x{k} {gran} x {count} copies", flush=True)
    S.gemv_batched(allp, alla, n, k, dev_bf16(xb), count, ps, as_, gran, 128, y_dtype="float32", y=y,
                   y_stride=ys)
    yv = to_np(y)[:, :n]
    assert np.array_equal(yv, np.broadcast_to(yv[0], yv.shape))
    a = O.alpha(w, gran, 128)
    y_ref = O.gemv(xv, O.dequant(O.ternary(w), a, gran, 128))
    bound = O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, gran, 128))
    for c in (0, count - 1):
        check_close(yv[c:c + 1], y_ref, bound, f"copy {c}")


@pytest.mark.parametrize("n,k,gran,g,count,y_dtype", [
    (1000, 8192, "per_group", 128, 1, "bfloat16"),   # 16 splits of one 4-superblock window
    (1000, 8192, "per_group", 256, 1, "float32"),    # the same with 2-superblock groups
    (700, 8192, "per_channel", 128, 1, "float32"),
    (700, 8192, "per_tensor", 128, 1, "bfloat16"),
    (1024, 3072, "per_group", 128, 3, "float32"),    # 6 splits of one window
    (300, 512, "per_group", 128, 1100, "float32"),   # no split, K of one 4-superblock window
    (300, 256, "per_channel", 128, 2100, "bfloat16"),  # no split, a 2-superblock window
    (300, 128, "per_tensor", 128, 4200, "float32"),  # no split, a 1-superblock window
    (1000, 512, "per_group", 128, 1100, "bfloat16"),  # the same on 512-row workgroups (ragged last panel)
    (1000, 256, "per_tensor", 128, 2100, "float32"),
])
def test_gemv_one_window_launches(n, k, gran, g, count, y_dtype):
    """Batch-1 launches whose workgroups each cover exactly one table window
    (a K split into single windows, or K of one window): the records and the
    table's activations are loaded together before the table build.  Codes
    and scales bit-exact, products of the first and last copies against the
    oracle, every copy equal."""
    w = WL.latent_weight(n, k, 1600 + n)
    pw = S.quantize_pack(dev_f32(w), gran, g)
    ref_p, ref_a = O.quantize_pack(w, gran, g)
    assert np.array_equal(to_np(pw.packed), ref_p)
    assert np.array_equal(to_np(pw.alpha).view(np.uint32),
                          np.ascontiguousarray(ref_a, dtype=np.float32).reshape(-1).view(np.uint32))
    xb, xv = WL.activations_bf16(1, k, 1610 + n)
    print(f"[gemv one window] {n}x{k} {gran} G={g} x {count} {y_dtype}", flush=True)
    if count == 1:
        yv = to_np(S.gemv(pw, dev_bf16(xb), y_dtype)).reshape(1, n)
    else:
        nb, nsc = S.packed_bytes(n, k), S.num_scales(n, k, gran, g)
        ps, as_ = (nb + 255) // 256 * 256, (nsc + 63) // 64 * 64
        allp = torch.empty((count, ps), dtype=torch.uint8, device=DEV)
        allp[:, :nb] = pw.packed
        alla = torch.empty((count, as_), dtype=torch.float32, device=DEV)
        alla[:, :nsc] = pw.alpha
        ys = (n + 7) // 8 * 8
        ydt = torch.float32 if y_dtype == "float32" else torch.bfloat16
        y = torch.empty((count, ys), dtype=ydt, device=DEV)
        S.gemv_batched(allp, alla, n, k, dev_bf16(xb), count, ps, as_, gran, g, y_dtype=y_dtype, y=y, y_stride=ys)
        yv = to_np(y)[:, :n]
        assert np.array_equal(yv, np.broadcast_to(yv[0], yv.shape))
    if y_dtype == "bfloat16":
        yv = O.bf16_bits_to_f32(yv)
    a = np.asarray(ref_a)
    y_ref = O.gemv(xv, O.dequant(O.ternary(w), a, gran, g))
    bound = O.tolerance_bound(xv, O.alpha_per_weight(a, n, k, gran, g), y_ref if y_dtype == "bfloat16" else None)
    for c in sorted({0, count - 1}):
        check_close(yv[c:c + 1], y_ref, bound, f"copy {c}")
