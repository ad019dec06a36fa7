"""GPU parity: the HIP path against the CPU oracle, byte for byte.

Tolerance is zero: E4M3 bytes, fp32 scale bits and E8M0 bytes must be
identical. Every configuration is compared whole, at its full size and in
the launch configuration the benchmark uses; for the large ones the oracle
runs on independent slices of the same input bytes in a thread pool
(tests/oracle_pool.py: column slices for dim0, row slices for dim1 and MX).
Every output buffer carries guard bands that must stay untouched.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import Guarded, assert_same_bytes, to_dev
from oracle_pool import check_dim0_whole, check_dim1_whole, check_mx_whole

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


# ----------------------------------------------------------------- runners


def gpu_dim0(x, off, pow2=False):
    M, K = x.shape
    G = len(off)
    gq, gs = Guarded((M, K), torch.uint8), Guarded((G, K), torch.float32)
    mgs.mgs_quant_groups_dim0(to_dev(x), to_dev(off), pow2, q=gq.view, scales=gs.view)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    return gq.numpy(), gs.numpy()


def gpu_dim1(x, off, pow2=False):
    M, K = x.shape
    G = len(off)
    gq, gs = Guarded((M, K), torch.uint8), Guarded((M, G), torch.float32)
    mgs.mgs_quant_groups_dim1(to_dev(x), to_dev(off), pow2, q=gq.view, scales=gs.view)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    return gq.numpy(), gs.numpy()


def gpu_mx(x, mode):
    M, K = x.shape
    gq, gs = Guarded((M, K), torch.uint8), Guarded((M, K // 32), torch.uint8)
    mgs.mgs_mx_quant_dim0(to_dev(x), mode, q=gq.view, scales=gs.view)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    return gq.numpy(), gs.numpy()


def check_dim0(x, off, pow2=False, what="dim0"):
    q, s = gpu_dim0(x, off, pow2)
    rq, rs = oracle.quant_groups_dim0(x, off, pow2)
    assert_same_bytes(s, rs, what + " scales")
    assert_same_bytes(q, rq, what + " q")


def check_dim1(x, off, pow2=False, what="dim1"):
    q, s = gpu_dim1(x, off, pow2)
    rq, rs = oracle.quant_groups_dim1(x, off, pow2)
    assert_same_bytes(s, rs, what + " scales")
    assert_same_bytes(q, rq, what + " q")


def check_mx(x, mode, what="mx"):
    q, s = gpu_mx(x, mode)
    rq, rs = oracle.mx_quant_dim0(x, mode)
    assert_same_bytes(s, rs, what + " scales")
    assert_same_bytes(q, rq, what + " q")


# ------------------------------------------------------- the cast, all fp32


def test_cast_e4m3_every_binary32():
    """The library's cast against the oracle encoder on all 2^32 patterns
    (NaN patterns excluded: outside the contract)."""
    chunk = 1 << 26
    inp = torch.empty(chunk, dtype=torch.int32, device="cuda")
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    sub = chunk // 16
    with cf.ThreadPoolExecutor(16) as pool:
        for c in range(1 << 32 >> 26):
            first = c * chunk
            pat = torch.arange(first, first + chunk, dtype=torch.int64, device="cuda")
            inp.copy_(torch.where(pat >= (1 << 31), pat - (1 << 32), pat).to(torch.int32))
            mgs.mgs_cast_e4m3(inp.view(torch.float32), out=out)
            got = out.cpu().numpy()
            want = np.concatenate(list(pool.map(lambda i: oracle.e4m3_encode_f32_bits(first + i * sub, sub),
                                                range(16))))
            bits = np.arange(first, first + chunk, dtype=np.uint64).astype(np.uint32)
            nan = ((bits & 0x7F800000) == 0x7F800000) & ((bits & 0x7FFFFF) != 0)
            bad = np.nonzero((got != want) & ~nan)[0]
            assert bad.size == 0, ["%08x: got %02x want %02x" % (bits[i], got[i], want[i]) for i in bad[:8]]


# ---------------------------------------------------------------- dim0


def test_dim0_c1():
    w = wl.c1_dim0_small()
    check_dim0(w.x, w.offsets, w.pow2, w.name)


def test_dim0_c2_pow2_empty_and_zero_groups():
    w = wl.c2_dim0_pow2()
    sizes = wl.sizes_from_offsets(w.offsets)
    assert (sizes == 0).any()
    check_dim0(w.x, w.offsets, w.pow2, w.name)


def test_dim0_c3_dirichlet_whole():
    w = wl.c3_dim0_large()
    assert wl.sizes_from_offsets(w.offsets).max() > 896      # exercises chunked groups
    q, s = gpu_dim0(w.x, w.offsets, w.pow2)
    check_dim0_whole(w.x, w.offsets, w.pow2, q, s, w.name)


def test_dim0_c6_target_whole(token_major):
    w = wl.c6_dim0_target(64, token_major)
    q, s = gpu_dim0(w.x, w.offsets, w.pow2)
    check_dim0_whole(w.x, w.offsets, w.pow2, q, s, w.name)


# ---------------------------------------------------------------- dim1


@pytest.mark.parametrize("G", [1, 16, 64])
def test_dim1_c4_whole(token_major, G):
    w = wl.c4_dim1(G, token_major)
    q, s = gpu_dim1(w.x, w.offsets)
    check_dim1_whole(w.x, w.offsets, False, q, s, w.name)


# ------------------------------------------------------------------ MX


@pytest.mark.parametrize("mode", [mgs.MGS_MX_FLOOR, mgs.MGS_MX_RCEIL])
def test_mx_c5_whole(c5, mode):
    q, s = gpu_mx(c5.x, mode)
    check_mx_whole(c5.x, mode, q, s, "mx mode %d" % mode)


# --------------------------------------------------------------- edges


def edge_values(rng, shape):
    """randn mixed with exact zeros, -0.0, bf16 subnormals, tiny and huge
    magnitudes and outliers."""
    x = wl.randn_bf16(rng, shape, 0.02, 0.003, 8.0)
    n = x.size
    flat = x.reshape(-1)
    pick = rng.choice(n, size=max(1, n // 20), replace=False)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80,
                         0x7F7F, 0xFF7F, 0x0400, 0x1000], dtype=np.uint16)
    flat[pick] = specials[rng.integers(0, len(specials), len(pick))]
    return x


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("M", [37, 300000])
def test_dim1_no_columns_writes_scales(M, pow2):
    # every group of every row is empty: all M * G scales get the amax = 0
    # value (300000 rows: more scales than one pass of the fill's grid)
    x = np.zeros((M, 0), np.uint16)
    off = np.zeros(4, np.int32)
    q, s = gpu_dim1(x, off, pow2)
    _, rs = oracle.quant_groups_dim1(x, off, pow2)
    assert_same_bytes(s, rs, "dim1 K=0 scales")


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("M,K,sizes", [
    (1, 8, [1]),
    (40, 200, [0, 17, 0, 23, 0]),                # ragged strip (K % 128 != 0), empty groups
    (512, 256, [512]),                           # exactly one chunk
    (513, 136, [513]),                           # just taller than one chunk
    (1500, 128, [0, 1024, 3, 473]),              # tall group next to tiny ones
    (2000, 384, [700, 0, 0, 1300]),              # two- and three-chunk teams around empty groups
    (96, 64, [32, 32, 32]),
    (12000, 136, [0, 11000, 1000]),              # a group cut into chunks (maxima through the workspace)
    (7000, 512, [5121, 1279, 600]),              # chunked groups next to one just under the threshold
    (6000, 64, [5120, 880]),                     # chunked, with 64-column rows
    (2600, 264, [1280, 1281, 39]),               # two chunked groups and a short one
    (1300, 264, [576, 577, 147]),                # 128-column strips with a ragged last slab
    (1300, 264, [640, 641, 19]),                 # either side of a 128-column tile's register rows
    (2000, 264, [896, 897, 207]),                # either side of dim0's chunking threshold
])
def test_dim0_edges(M, K, sizes, pow2):
    rng = np.random.default_rng(M * 7 + K)
    x = edge_values(rng, (M, K))
    off = np.cumsum(sizes).astype(np.int32)
    assert off[-1] == M
    # a group of all zeros where there is one with rows
    nz = [i for i, s in enumerate(sizes) if s > 0]
    if len(nz) > 1:
        g = nz[-1]
        x[off[g] - sizes[g]:off[g]] = 0
    check_dim0(x, off, pow2, "dim0 edge %s" % (sizes,))


def test_dim0_no_rows_writes_scales():
    x = np.zeros((0, 64), np.uint16)
    off = np.zeros(3, np.int32)
    q, s = gpu_dim0(x, off)
    _, rs = oracle.quant_groups_dim0(x, off)
    assert_same_bytes(s, rs, "dim0 M=0 scales")


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("M,K,sizes", [
    (3, 16, [16]),
    (5, 160, [0, 16, 0, 144, 0]),
    (4, 2080 * 8, None),                         # a c4 row with 64 groups
    (2, 16384, [16] * 1024),                     # the group limit, every group one vector pair
    (3, 40960, [0, 20480, 20480]),               # rows longer than one register pass
    (7, 1024, [1024]),
])
def test_dim1_edges(M, K, sizes, pow2):
    rng = np.random.default_rng(M * 13 + K)
    x = edge_values(rng, (M, K))
    off = wl.target_offsets(64) if sizes is None else np.cumsum(sizes).astype(np.int32)
    assert off[-1] == K
    check_dim1(x, off, pow2, "dim1 edge")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (17, 5120), (2, 4096 + 32)])
def test_mx_edges(M, K, mode):
    rng = np.random.default_rng(M + K)
    x = edge_values(rng, (M, K))
    x[0, :32] = 0
    if K >= 64:
        x[0, 32:64] = rng.integers(0, 0x80, 32).astype(np.uint16)   # subnormal-only block
    check_mx(x, mode, "mx edge")


def test_every_finite_bf16_through_dim1():
    """Each finite bf16 value x goes through the kernel's cast with a scale
    fixed by an anchor in the same (row, group): row r = [x_r, anchor_r, 0...]."""
    b = np.arange(0x10000, dtype=np.uint32)
    finite = (b & 0x7F80) != 0x7F80
    xs = b[finite].astype(np.uint16)
    mags = xs & 0x7FFF
    for variant in range(3):
        if variant == 0:
            anchor = mags.copy()
        elif variant == 1:      # next power of two (exponent + 1, mantissa 0)
            anchor = (((mags >> 7) + 1) << 7).astype(np.uint16)
        else:                   # 1.75 x that power
            anchor = ((((mags >> 7) + 1) << 7) | 0x60).astype(np.uint16)
        anchor = np.where(mags == 0, 0x3F80, anchor)
        ok = (anchor & 0x7F80) != 0x7F80
        rows = np.zeros((int(ok.sum()), 16), np.uint16)
        rows[:, 0] = xs[ok]
        rows[:, 1] = anchor[ok]
        check_dim1(rows, np.array([16], np.int32), False, "bf16 sweep %d" % variant)


def bf16_sweep_columns(variant):
    """(16, N) bf16 with column j = [x_j, anchor_j, 0, ...] over every finite
    bf16 x_j (N padded to a multiple of 8 with zero columns), and how many of
    its products fl32(x * s) exceed 448 in magnitude (those the grouped
    kernels' cast reaches without a clamp)."""
    b = np.arange(0x10000, dtype=np.uint32)
    xs = b[(b & 0x7F80) != 0x7F80].astype(np.uint16)
    mags = xs & 0x7FFF
    if variant == 0:
        anchor = mags.copy()
    elif variant == 1:
        anchor = (((mags >> 7) + 1) << 7).astype(np.uint16)
    else:
        anchor = ((((mags >> 7) + 1) << 7) | 0x60).astype(np.uint16)
    anchor = np.where(mags == 0, 0x3F80, anchor)
    ok = (anchor & 0x7F80) != 0x7F80
    n = int(ok.sum())
    N = (n + 7) // 8 * 8
    x = np.zeros((16, N), np.uint16)
    x[0, :n] = xs[ok]
    x[1, :n] = anchor[ok]
    f32 = lambda u: (u.astype(np.uint32) << 16).view(np.float32)
    s = np.float32(448.0) / np.maximum(f32(anchor[ok]), np.float32(1e-12))
    above = int(np.count_nonzero(np.abs(f32(xs[ok]) * s) > np.float32(448.0)))
    return x, above


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_every_finite_bf16_through_dim0(variant):
    """The dim0 kernel's cast on every finite bf16 value, with the scale of its
    column fixed by an anchor; the anchor = |x| sweep reaches binary32
    products just above 448, which must give 0x7E / 0xFE."""
    x, above = bf16_sweep_columns(variant)
    if variant == 0:
        assert above > 1000
    off = np.array([16], np.int32)
    for pow2 in (False, True):
        check_dim0(x, off, pow2, "dim0 bf16 sweep %d pow2=%s" % (variant, pow2))


def test_every_finite_bf16_through_dim0_t():
    x, above = bf16_sweep_columns(0)
    assert above > 1000
    off = np.array([16], np.int32)
    M, K = x.shape
    gq, gs = Guarded((K, M), torch.uint8), Guarded((K, 1), torch.float32)
    mgs.mgs_quant_groups_dim0_t(to_dev(x), to_dev(off), False, q_t=gq.view, scales_t=gs.view)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    rq, rs = oracle.quant_groups_dim0_t(x, off, False)
    assert_same_bytes(gs.numpy(), rs, "dim0_t bf16 sweep scales_t")
    assert_same_bytes(gq.numpy(), rq, "dim0_t bf16 sweep q_t")


# ------------------------------------------------- identities, determinism


def test_transpose_identity_on_gpu():
    rng = np.random.default_rng(99)
    T = wl.randn_bf16(rng, (1040, 2048), 0.02, 0.001, 8.0)
    off = wl.uniform_group_offsets(rng, 1040, 9)
    q0, s0 = gpu_dim0(T, off)
    q1, s1 = gpu_dim1(np.ascontiguousarray(T.T), off)
    assert_same_bytes(q1, q0.T.copy(), "dim1(T^T) vs dim0(T)^T q")
    assert_same_bytes(s1, s0.T.copy(), "dim1(T^T) vs dim0(T)^T scales")


def test_repeat_runs_are_bit_identical():
    rng = np.random.default_rng(8)
    x = wl.randn_bf16(rng, (8192, 1024), 1.0)
    xt, ot = to_dev(x), to_dev(np.array([100, 3000, 3000, 8192], np.int32))
    a = [mgs.mgs_quant_groups_dim0(xt, ot) for _ in range(2)]
    b = [mgs.mgs_quant_groups_dim1(xt, to_dev(np.array([512, 1024], np.int32))) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(a[0][0], a[1][0]) and torch.equal(a[0][1], a[1][1])
    assert torch.equal(b[0][0], b[1][0]) and torch.equal(b[0][1], b[1][1])


def test_bad_offsets_stay_in_bounds():
    """Unsorted and out-of-range offsets give unspecified values but must
    not write outside the outputs."""
    rng = np.random.default_rng(3)
    x = wl.randn_bf16(rng, (300, 256), 1.0)
    for off in ([400, 10, -5, 300], [-1, -1, 7], [1 << 30, 5]):
        o = np.array(off, np.int32)
        gpu_dim0(x, o)
        gpu_dim1(x, o)


def test_validate_flag():
    """MGS_FLAG_VALIDATE: good offsets give the oracle's bytes; malformed
    ones are rejected with MGS_ERR_INVALID_ARG before any launch."""
    rng = np.random.default_rng(11)
    x = wl.randn_bf16(rng, (200, 64), 1.0)
    xt = to_dev(x)
    good = np.array([48, 48, 200], np.int32)
    q, s = mgs.mgs_quant_groups_dim0(xt, to_dev(good), validate=True)
    rq, rs = oracle.quant_groups_dim0(x, good)
    assert_same_bytes(q.cpu().numpy(), rq, "dim0 q (validated)")
    assert_same_bytes(s.cpu().numpy(), rs, "dim0 scales (validated)")
    good1 = np.array([16, 16, 64], np.int32)
    q1, s1 = mgs.mgs_quant_groups_dim1(xt, to_dev(good1), validate=True)
    rq1, rs1 = oracle.quant_groups_dim1(x, good1)
    assert_same_bytes(q1.cpu().numpy(), rq1, "dim1 q (validated)")
    assert_same_bytes(s1.cpu().numpy(), rs1, "dim1 scales (validated)")
    bad_dim0 = ([100, 50, 200], [100, 300], [100, 150], [-1, 200])
    for off in bad_dim0:
        with pytest.raises(mgs.MgsError) as e:
            mgs.mgs_quant_groups_dim0(xt, to_dev(np.array(off, np.int32)), validate=True)
        assert e.value.status == mgs.MGS_ERR_INVALID_ARG, off
    for off in ([8, 64], [32, 16, 64], [16, 48], [16, 80]):
        with pytest.raises(mgs.MgsError) as e:
            mgs.mgs_quant_groups_dim1(xt, to_dev(np.array(off, np.int32)), validate=True)
        assert e.value.status == mgs.MGS_ERR_INVALID_ARG, off


# ------------------------------------------------ outliers at group edges


@pytest.mark.parametrize("pow2", [False, True])
def test_outliers_at_group_edges(pow2):
    """The largest magnitude of every group sits in its first or last row
    (dim0, dim0_t) or column (dim1), with small values elsewhere. A group
    boundary off by one would put an outlier into the neighbouring group's
    amax and change that group's scales."""
    rng = np.random.default_rng(4242)
    # dim0 / dim0_t: 16-aligned boundaries (dim0_t's requirement), groups of
    # 16 rows to tall chunked ones, and empty groups
    sizes = np.array([16, 0, 48, 1024, 16, 0, 2048, 32, 112, 3200], np.int64)
    off = np.cumsum(sizes).astype(np.int32)
    M, K = int(off[-1]), 264
    x = wl.randn_bf16(rng, (M, K), 0.02)
    start = 0
    for g, n in enumerate(sizes):
        if n:
            edge = start if g % 2 == 0 else start + n - 1
            big = wl.f32_to_bf16_bits(np.float32(rng.choice([-1.0, 1.0]) * (8.0 + g)))
            x[edge, :] = big
        start += n
    check_dim0(x, off, pow2, "dim0 edge outliers")
    q_t, s_t = mgs.mgs_quant_groups_dim0_t(to_dev(x), to_dev(off), pow2)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_groups_dim0_t(x, off, pow2)
    assert_same_bytes(s_t.cpu().numpy(), rs, "dim0_t edge outliers scales")
    assert_same_bytes(q_t.cpu().numpy(), rq, "dim0_t edge outliers q")
    # dim1: the same along the columns of 40 rows
    xs = wl.randn_bf16(rng, (40, M), 0.02)
    start = 0
    for g, n in enumerate(sizes):
        if n:
            edge = start if g % 2 == 0 else start + n - 1
            xs[:, edge] = wl.f32_to_bf16_bits(np.float32(-(8.0 + g)))
        start += n
    check_dim1(xs, off, pow2, "dim1 edge outliers")
