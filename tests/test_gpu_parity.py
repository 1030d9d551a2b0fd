"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: packed bytes, scales, codes and status bits bit-exact; matmul outputs
within |y - y_ref| <= 1e-3 * sum_k |x_k w_hat_k| per element (y_ref fp64);
one-hot activations bit-exact.
"""
import itertools

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import (assert_within_bound, check_quantize_exact, gpu_matmul,
                               gpu_quantize, gpu_unpack, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,G", [(512, 64), (320, 64), (512, 128)])
def test_small_matrix_quantize_unpack_exact(K, G):
    w = inputs.small_matrix(K=K)
    say("small matrix W[256,%d] G=%d seed 0: quantize_pack, unpack" % (K, G))
    p, s = check_quantize_exact(w, G, "W[256,%d] G=%d" % (K, G))
    codes_gpu, st = gpu_unpack(p, 256, K, G)
    codes_ref, st_ref = oracle.unpack(p, 256, K, G)
    assert st == st_ref == 0
    assert np.array_equal(codes_gpu, codes_ref)


@pytest.mark.parametrize("K,G", [(512, 64), (320, 64), (512, 128)])
@pytest.mark.parametrize("kind,M", [("gemv", 1), ("gemv", 8), ("gemv", 3), ("gemv", 10),
                                    ("gemv", 16), ("gemm", 1), ("gemm", 8), ("gemm", 128),
                                    ("gemm", 513)])
def test_small_matrix_matmul(K, G, kind, M):
    w = inputs.small_matrix(K=K)
    p, s, _ = oracle.quantize_pack(w, G)
    x = inputs.activation(1 if M == 1 else 2, M, K)
    say("%s M=%d W[256,%d] G=%d" % (kind, M, K, G))
    y, st = gpu_matmul(kind, x, p, s, 256, K, G)
    y_ref, bound, _ = oracle.matmul(x, p, s, 256, K, G)
    assert st == 0
    assert_within_bound(y, y_ref, bound, "%s M=%d K=%d G=%d" % (kind, M, K, G))


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
@pytest.mark.parametrize("G", [64, 128])
def test_one_hot_activations_exact(kind, G):
    """x = e_k gives y[n] = c[n,k] * s[n,k/G] exactly: pins K indexing, digit
    order within a byte and the group -> scale mapping bit for bit."""
    N, K = 250, 1024
    w = inputs.normal_bf16(31, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    codes, _ = oracle.unpack(p, N, K, G)
    ks = [0, 1, 2, 3, 4, 5, 6, 63, 64, 65, 127, 128, 500, 1023, 640, 641, 642, 643, 644, 645]
    ks = ks[:16]
    x = np.zeros((len(ks), K), np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80
    say("one-hot %s G=%d N=%d K=%d" % (kind, G, N, K))
    y, _ = gpu_matmul(kind, x, p, s, N, K, G)
    sf = s.view(np.float16).astype(np.float32)
    for i, k in enumerate(ks):
        want = codes[:, k].astype(np.float32) * sf[:, k // G]
        assert np.array_equal(y[i], want), (kind, k)


def test_ones_times_single_group_exact():
    """x = ones, W nonzero in one group: y = s * sum(c) exactly."""
    N, K, G = 64, 512, 128
    w = np.zeros((N, K), np.uint16)
    w[:, 256:384] = inputs.normal_bf16(32, (N, 128), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    codes, _ = oracle.unpack(p, N, K, G)
    x = np.full((2, K), 0x3F80, np.uint16)
    for kind in ("gemv", "gemm"):
        y, _ = gpu_matmul(kind, x, p, s, N, K, G)
        want = codes[:, 256:384].sum(1).astype(np.float32) * s[:, 2].view(np.float16).astype(np.float32)
        assert np.array_equal(y[0], want) and np.array_equal(y[1], want)


def _random_finite_bf16(rng, n, emin, emax):
    sign = rng.integers(0, 2, n).astype(np.uint16) << 15
    e = rng.integers(emin, emax + 1, n).astype(np.uint16) << 7
    m = rng.integers(0, 128, n).astype(np.uint16)
    return sign | e | m


def _bf16(v):
    return int(inputs.f32_to_bf16_bits(np.array([v], np.float32))[0])


@pytest.mark.parametrize("G", [64, 128])
def test_quantize_stress_groups_exact(G):
    """Groups built to break a windowed or floating-point sum: exponents over
    ~140 binades, bf16 subnormals, fp16 midpoints with and without a 2^-100
    excess, overflow and non-finite groups."""
    rng = np.random.default_rng(33)
    rows = [
        _random_finite_bf16(rng, 64 * G, 0, 140).reshape(64, G),
        _random_finite_bf16(rng, 64 * G, 90, 120).reshape(64, G),
        _random_finite_bf16(rng, 64 * G, 0, 10).reshape(64, G),
        _random_finite_bf16(rng, 64 * G, 126, 145).reshape(64, G),
    ]
    special = np.zeros((8, G), np.uint16)
    # exact fp16 midpoint (ties to even) and the same plus 2^-100 (rounds up)
    # sum = G * (1 + 2^-11): mean on the midpoint of 0x3C00 / 0x3C01
    half = G // 2
    special[0, :half] = _bf16(2.0)
    special[0, half] = _bf16(G * 2.0 ** -11)
    special[1] = special[0]
    special[1, half + 1] = _bf16(2.0 ** -100)
    special[2, :] = _bf16(7e4)               # overflow
    special[3, :] = _bf16(2.0 ** -30)        # underflow to 0
    special[4, :] = inputs.normal_bf16(34, (G,), 0.02)
    special[4, 3] = 0x7FC1                   # NaN
    special[5, :] = _bf16(1.0)
    special[5, 7] = 0xFF80                   # -inf
    special[6, :] = _bf16(2.0 ** -133 * 5)   # smallest subnormals
    special[7, :] = _bf16(65504.0 / 2)
    w = np.concatenate(rows + [special])
    say("quantize stress G=%d rows=%d" % (G, w.shape[0]))
    check_quantize_exact(w, G, "stress G=%d" % G)


def test_unpack_flags_invalid_and_padding():
    N, K, G = 16, 256, 64
    w = inputs.normal_bf16(35, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    bad = p.copy()
    bad[3, 5] = 250
    codes, st = gpu_unpack(bad, N, K, G)
    codes_ref, st_ref = oracle.unpack(bad, N, K, G)
    assert st == st_ref == 4 and np.array_equal(codes, codes_ref)
    pad = p.copy()
    pad[7, 12] = pad[7, 12] + 81 if pad[7, 12] < 162 else pad[7, 12] - 81
    codes, st = gpu_unpack(pad, N, K, G)
    codes_ref, st_ref = oracle.unpack(pad, N, K, G)
    assert st == st_ref == 8 and np.array_equal(codes, codes_ref)
    for kind in ("gemv", "gemm"):
        x = inputs.activation(36, 2, K)
        _, st = gpu_matmul(kind, x, bad, s, N, K, G)
        assert st & 4


def test_quantize_deterministic_and_repeatable():
    w = inputs.normal_bf16(37, (1000, 3584), 0.02)
    a = gpu_quantize(w, 128)
    b = gpu_quantize(w, 128)
    assert all(np.array_equal(u, v) for u, v in zip(a[:2], b[:2])) and a[2] == b[2]


@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (1, 128, 128), (7, 192, 64), (3, 384, 128)])
def test_degenerate_shapes(N, K, G):
    w = inputs.normal_bf16(38, (N, K), 0.02)
    p, s = check_quantize_exact(w, G, "N=%d K=%d G=%d" % (N, K, G))
    codes, st = gpu_unpack(p, N, K, G)
    assert np.array_equal(codes, oracle.unpack(p, N, K, G)[0])
    for kind, M in itertools.product(("gemv", "gemm"), (1, 5)):
        x = inputs.activation(39, M, K)
        y, st = gpu_matmul(kind, x, p, s, N, K, G)
        y_ref, bound, _ = oracle.matmul(x, p, s, N, K, G)
        assert_within_bound(y, y_ref, bound, "%s N=%d K=%d G=%d M=%d" % (kind, N, K, G, M))


@pytest.mark.parametrize("N,K,G,count", [(256, 512, 64, 5), (250, 1024, 128, 3), (96, 320, 64, 70),
                                         (100, 3584, 128, 2), (40, 14336, 128, 2), (33, 4096, 64, 4)])
def test_gemv_batched_matches_oracle(N, K, G, count):
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16, dev_f16bits, dev_u8
    ws = [inputs.normal_bf16(300 + i, (N, K), 0.02) for i in range(count)]
    xs = [inputs.activation(400 + i, 1, K) for i in range(count)]
    refs = [oracle.quantize_pack(w, G) for w in ws]
    say("gemv_batched N=%d K=%d G=%d count=%d" % (N, K, G, count))
    st = tq.new_status()
    ys = tq.gemv_batched([dev_bf16(x) for x in xs], [dev_u8(p) for p, _, _ in refs],
                         [dev_f16bits(s) for _, s, _ in refs], N, K, G, status=st)
    import torch
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i in range(count):
        p, s, _ = refs[i]
        y_ref, bound, _ = oracle.matmul(xs[i], p, s, N, K, G)
        assert_within_bound(ys[i].cpu().numpy(), y_ref, bound, "batched item %d" % i)
    # an invalid byte in one problem is reported
    bad = refs[count - 1][0].copy()
    bad[0, 0] = 247
    st = tq.new_status()
    tq.gemv_batched([dev_bf16(xs[0])], [dev_u8(bad)], [dev_f16bits(refs[count - 1][1])], N, K, G,
                    status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 4


@pytest.mark.parametrize("M,count", [(2, 1), (5, 2)])
def test_skinny_matmul_blocks_with_several_chunks(M, count):
    """The skinny matmul (2 <= M <= 16) on tall matrices: 2500 tiles of 16 or
    32 rows leave more chunks than the 256 persistent blocks, so blocks walk
    two chunks; every output is checked, over one and two problems."""
    import torch
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16, dev_f16bits, dev_u8
    N, K, G = 40000, 512, 128
    ws = [inputs.normal_bf16(500 + i, (N, K), 0.02) for i in range(count)]
    refs = [oracle.quantize_pack(w, G) for w in ws]
    xs = [inputs.activation(510 + i, M, K) for i in range(count)]
    say("skinny matmul M=%d N=%d K=%d count=%d" % (M, N, K, count))
    st = tq.new_status()
    ys = tq.gemv_batched([dev_bf16(x) for x in xs], [dev_u8(p) for p, _, _ in refs],
                         [dev_f16bits(s) for _, s, _ in refs], N, K, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i in range(count):
        p, s, _ = refs[i]
        y_ref, bound, _ = oracle.matmul(xs[i], p, s, N, K, G)
        assert_within_bound(ys[i].cpu().numpy(), y_ref, bound, "skinny M=%d problem %d" % (M, i))


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("offset", [0, 1, 2, 3])
def test_gemm_ragged_unaligned_packed_and_invalid_bytes(G, offset):
    """tq_gemm over partial tiles (M=300, N=200 leave ragged 256-row and
    128-row tiles), packed bytes at every alignment (the ABI allows any), and
    an invalid byte at the first and at the very last byte of the buffer."""
    import torch
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16, dev_f16bits
    M, N, K = 300, 200, 640
    w = inputs.normal_bf16(60 + G, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    x = inputs.activation(61, M, K)
    y_ref, bound, _ = oracle.matmul(x, p, s, N, K, G)
    flat = p.reshape(-1)
    buf = torch.zeros(flat.size + 8, dtype=torch.uint8, device="cuda")
    pd = buf[offset:offset + flat.size]
    xd, sd = dev_bf16(x), dev_f16bits(s)
    say("gemm ragged M=%d N=%d K=%d G=%d packed offset %d" % (M, N, K, G, offset))
    pd.copy_(torch.from_numpy(flat))
    st = tq.new_status()
    y = tq.gemm(xd, pd, sd, N, K, G, status=st).cpu().numpy()
    assert int(st.item()) == 0
    assert_within_bound(y, y_ref, bound, "gemm ragged G=%d offset %d" % (G, offset))
    for pos in (0, flat.size - 1):
        bad = flat.copy()
        bad[pos] = 243 + pos % 13
        pd.copy_(torch.from_numpy(bad))
        st = tq.new_status()
        tq.gemm(xd, pd, sd, N, K, G, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) & 4, "invalid byte at %d not flagged" % pos


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("N", [200, 201, 202, 203])
def test_gemv_ragged_buffer_ends_and_invalid_bytes(G, N):
    """tq_gemv at M = 1, 5 and 16 over ragged row tiles, with N chosen so the
    packed buffer (N * 130 bytes) ends at every offset modulo 4: the last
    dword loads of the last row run past the end of the buffer.  An invalid
    byte at the first and at the very last byte of the buffer is flagged."""
    import torch
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16, dev_f16bits, dev_u8
    K = 640
    w = inputs.normal_bf16(70 + G + N, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    flat = p.reshape(-1)
    sd = dev_f16bits(s)
    for M in (1, 5, 16):
        x = inputs.activation(71 + M, M, K)
        y_ref, bound, _ = oracle.matmul(x, p, s, N, K, G)
        xd = dev_bf16(x)
        say("gemv ragged M=%d N=%d K=%d G=%d" % (M, N, K, G))
        st = tq.new_status()
        y = tq.gemv(xd, dev_u8(p), sd, N, K, G, status=st).cpu().numpy()
        assert int(st.item()) == 0
        assert_within_bound(y, y_ref, bound, "gemv ragged M=%d N=%d G=%d" % (M, N, G))
        for pos in (0, flat.size - 1):
            bad = flat.copy()
            bad[pos] = 243 + pos % 13
            st = tq.new_status()
            tq.gemv(xd, dev_u8(bad.reshape(p.shape)), sd, N, K, G, status=st)
            torch.cuda.synchronize()
            assert int(st.item()) & 4, "invalid byte at %d not flagged (M=%d)" % (pos, M)


# Row lengths K that take every block shape of the one-row kernel: 16-, 32-
# and 64-lane rows summed inside a wave, 48-lane rows that cross waves, and
# 80- to 256-lane rows summed through LDS; activations staged with two
# blocks per CU or, from K = 6848, one; batch steps in whole dwords or not (K = 9280 and 13376
# give odd byte offsets from one batch to the next).
@pytest.mark.parametrize("K,G", [(1088, 64), (2048, 128), (2560, 64), (3072, 128), (4160, 64),
                                 (6144, 128), (6784, 64), (6848, 64), (7168, 64), (8192, 128),
                                 (9280, 64), (13376, 64), (16384, 128)])
def test_gemv_row_shapes(K, G):
    """tq_gemv at M = 1 over K values covering each row shape, N = 37 (a
    ragged last batch of rows); an invalid byte in the middle of the buffer
    is flagged."""
    import torch
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16, dev_f16bits, dev_u8
    N = 37
    w = inputs.normal_bf16(90 + K // 64, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack(w, G)
    x = inputs.activation(91, 1, K)
    y_ref, bound, _ = oracle.matmul(x, p, s, N, K, G)
    say("gemv row shape M=1 N=%d K=%d G=%d" % (N, K, G))
    xd, sd = dev_bf16(x), dev_f16bits(s)
    st = tq.new_status()
    y = tq.gemv(xd, dev_u8(p), sd, N, K, G, status=st).cpu().numpy()
    assert int(st.item()) == 0
    assert_within_bound(y, y_ref, bound, "gemv M=1 N=%d K=%d G=%d" % (N, K, G))
    bad = p.reshape(-1).copy()
    bad[bad.size // 2 + 3] = 250
    st = tq.new_status()
    tq.gemv(xd, dev_u8(bad.reshape(p.shape)), sd, N, K, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 4


@pytest.mark.parametrize("G", [64, 128])
def test_gemv_grouped_mixed_shapes(G):
    """tq_gemv_grouped over mixed shapes -- several kernel configurations
    (among them rows long enough to run one block per CU), one shape the
    M = 1 kernel does not take (K = 8320: 130 chunks), ragged N --
    and more problems than one launch holds for the commonest configuration:
    bit-identical to one tq_gemv per problem, every output within the
    oracle's bound; an invalid byte in one problem is flagged."""
    import torch
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16, dev_f16bits, dev_u8
    base = [(96, 1024), (40, 3584), (37, 640), (5, 8320), (64, 2048)]
    shapes = [base[i % len(base)] if i < 10 else (32 + i % 7, 1024) for i in range(140)]
    # rows of 6784 (two blocks a CU) and 6848 and 14336 (one block a CU, x
    # staged): three more configurations in the same call
    shapes += [(23, 6784), (19, 6848), (11, 14336)]
    shapes = [(n, k) for n, k in shapes if k % G == 0]
    ws = [inputs.normal_bf16(900 + i, (n, k), 0.02) for i, (n, k) in enumerate(shapes)]
    xs = [inputs.activation(1000 + i, 1, k) for i, (n, k) in enumerate(shapes)]
    refs = [oracle.quantize_pack(w, G) for w in ws]
    xd = [dev_bf16(x) for x in xs]
    pdv = [dev_u8(p) for p, _, _ in refs]
    sdv = [dev_f16bits(s) for _, s, _ in refs]
    Ns = [n for n, _ in shapes]
    Ks = [k for _, k in shapes]
    say("gemv_grouped G=%d count=%d" % (G, len(shapes)))
    st = tq.new_status()
    ys = tq.gemv_grouped(xd, pdv, sdv, Ns, Ks, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, (n, k) in enumerate(shapes):
        y1 = tq.gemv(xd[i], pdv[i], sdv[i], n, k, G)
        assert torch.equal(ys[i], y1), "grouped item %d (N=%d K=%d) differs" % (i, n, k)
        p, s, _ = refs[i]
        y_ref, bound, _ = oracle.matmul(xs[i], p, s, n, k, G)
        assert_within_bound(ys[i].cpu().numpy(), y_ref, bound, "grouped item %d" % i)
    bad = refs[1][0].reshape(-1).copy()
    bad[bad.size // 3] = 247
    pdv[1] = dev_u8(bad.reshape(refs[1][0].shape))
    st = tq.new_status()
    tq.gemv_grouped(xd, pdv, sdv, Ns, Ks, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 4


def test_gemm_wide_tiles_ragged_unaligned_and_invalid_bytes():
    """tq_gemm_batched at G = 128 with enough 256 x 128 tiles to take the
    wide-tile kernel (48 problems of M=300, N=200: ragged tiles in both M and
    N), the packed bytes of each problem at offset i % 4 (any alignment is
    allowed), every output within the bound of the oracle; then an invalid
    byte at the last byte of one problem's buffer is flagged."""
    import torch
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16, dev_f16bits
    M, N, K, G, count = 300, 200, 640, 128, 48
    ws = [inputs.normal_bf16(700 + i, (N, K), 0.02) for i in range(count)]
    xs = [inputs.activation(800 + i % 4, M, K) for i in range(count)]
    refs = [oracle.quantize_pack(w, G) for w in ws]
    flat_size = refs[0][0].size
    bufs = [torch.zeros(flat_size + 8, dtype=torch.uint8, device="cuda") for _ in range(count)]
    pdv = []
    for i, (p, _, _) in enumerate(refs):
        pd = bufs[i][i % 4:i % 4 + flat_size]
        pd.copy_(torch.from_numpy(p.reshape(-1)))
        pdv.append(pd)
    xd = [dev_bf16(x) for x in xs]
    sdv = [dev_f16bits(s) for _, s, _ in refs]
    say("gemm wide tiles M=%d N=%d K=%d G=%d count=%d" % (M, N, K, G, count))
    st = tq.new_status()
    ys = tq.gemm_batched(xd, pdv, sdv, N, K, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i in range(count):
        p, s, _ = refs[i]
        y_ref, bound, _ = oracle.matmul(xs[i], p, s, N, K, G)
        assert_within_bound(ys[i].cpu().numpy(), y_ref, bound, "wide item %d" % i)
    bad = refs[5][0].reshape(-1).copy()
    bad[-1] = 249
    pdv[5].copy_(torch.from_numpy(bad))
    st = tq.new_status()
    tq.gemm_batched(xd, pdv, sdv, N, K, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 4


@pytest.mark.parametrize("M,N,K,G,count", [(512, 3584, 1024, 128, 3), (100, 200, 640, 64, 5),
                                           (300, 96, 320, 64, 70)])
def test_gemm_batched_matches_single_calls_and_oracle(M, N, K, G, count):
    """tq_gemm_batched: bit-identical to one tq_gemm per problem (count=70
    takes two launches), and every output within the bound of the oracle."""
    import torch
    import ternary_weight_only_amd as tq
    from tests.gpu_helpers import dev_bf16, dev_f16bits, dev_u8
    ws = [inputs.normal_bf16(500 + i, (N, K), 0.02) for i in range(count)]
    xs = [inputs.activation(600 + i, M, K) for i in range(count)]
    refs = [oracle.quantize_pack(w, G) for w in ws]
    xd = [dev_bf16(x) for x in xs]
    pdv = [dev_u8(p) for p, _, _ in refs]
    sdv = [dev_f16bits(s) for _, s, _ in refs]
    say("gemm_batched M=%d N=%d K=%d G=%d count=%d" % (M, N, K, G, count))
    st = tq.new_status()
    ys = tq.gemm_batched(xd, pdv, sdv, N, K, G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i in range(count):
        y1 = tq.gemm(xd[i], pdv[i], sdv[i], N, K, G)
        assert torch.equal(ys[i], y1), "batched item %d differs from the single call" % i
        p, s, _ = refs[i]
        y_ref, bound, _ = oracle.matmul(xs[i], p, s, N, K, G)
        assert_within_bound(ys[i].cpu().numpy(), y_ref, bound, "batched item %d" % i)
