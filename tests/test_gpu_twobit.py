"""GPU parity of the 2-bit ternary format (tq_quantize_pack2, tq_unpack2,
tq_gemv2, tq_gemv2_batched) against the CPU oracle.

Format: codes c in {-1, 0, +1} stored as fields c + 1 in two bits, four a
byte, first weight lowest (Avenue README, size note on 2-bit packing;
"Autoregressive Language Model on the 6502 Processor": ternary parameters
packed four a byte); the scale and the codes are those of the base-3 format.
Bars: packing and unpacking bit-exact with the status bits; the GEMV within
1e-3 * sum_k |x_k w_hat_k| of the oracle's fp64 result (tiny-llm "Week 2
Day 3: Quantize the Model", "Mathematical Formulation")."""
import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import assert_within_bound, dev_bf16, dev_f16bits, dev_u8, host_u16, say
from tests.test_gpu_parity import _bf16, _random_finite_bf16

pytestmark = pytest.mark.gpu


def gpu_pack2(w_bits, G):
    import torch
    import ternary_weight_only_amd as tq
    st = tq.new_status()
    p, s = tq.quantize_pack2(dev_bf16(w_bits), G, status=st)
    torch.cuda.synchronize()
    return p.cpu().numpy(), host_u16(s), int(st.item())


def gpu_unpack2(packed, N, K, G):
    import torch
    import ternary_weight_only_amd as tq
    st = tq.new_status()
    c = tq.unpack2(dev_u8(packed), N, K, G, status=st)
    torch.cuda.synchronize()
    return c.cpu().numpy(), int(st.item())


def gpu_gemv2(x_bits, packed, scales, N, K, G):
    import torch
    import ternary_weight_only_amd as tq
    st = tq.new_status()
    y = tq.gemv2(dev_bf16(x_bits), dev_u8(packed), dev_f16bits(scales), N, K, G, status=st)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(st.item())


def check_pack2_exact(w, G, what):
    p, s, st = gpu_pack2(w, G)
    p_ref, s_ref, st_ref = oracle.quantize_pack2(w, G)
    assert np.array_equal(s, s_ref), "%s: scales differ at %s" % (
        what, np.argwhere(s != s_ref)[:5].tolist())
    assert np.array_equal(p, p_ref), "%s: packed differ at %s" % (
        what, np.argwhere(p != p_ref)[:5].tolist())
    assert st == st_ref, "%s: status %d vs %d" % (what, st, st_ref)
    return p_ref, s_ref


@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (1, 128, 128), (7, 192, 64), (3, 384, 128),
                                   (250, 1024, 128), (33, 3584, 128), (129, 4096, 64)])
def test_quantize_pack2_exact(N, K, G):
    w = inputs.normal_bf16(300 + N, (N, K), 0.02)
    say("quantize_pack2 W[%d,%d] G=%d" % (N, K, G))
    check_pack2_exact(w, G, "W[%d,%d] G=%d" % (N, K, G))


@pytest.mark.parametrize("G", [64, 128])
def test_quantize_pack2_stress_groups_exact(G):
    """The scale's hard cases (wide exponent spread, subnormals, fp16 ties
    with and without a tiny excess, overflow, NaN and Inf groups) give the
    same scales, fields and flags as the oracle."""
    rng = np.random.default_rng(301)
    rows = [_random_finite_bf16(rng, 32 * G, 0, 140).reshape(32, G),
            _random_finite_bf16(rng, 32 * G, 126, 145).reshape(32, G)]
    special = np.zeros((7, G), np.uint16)
    half = G // 2
    special[0, :half] = _bf16(2.0)
    special[0, half] = _bf16(G * 2.0 ** -11)
    special[1] = special[0]
    special[1, half + 1] = _bf16(2.0 ** -100)
    special[2, :] = _bf16(7e4)
    special[3, :] = inputs.normal_bf16(302, (G,), 0.02)
    special[3, 3] = 0x7FC1
    special[4, :] = _bf16(1.0)
    special[4, 7] = 0xFF80
    special[5, :] = _bf16(2.0 ** -133 * 5)
    special[6, :] = _bf16(65504.0 / 2)
    w = np.concatenate(rows + [special])
    say("quantize_pack2 stress G=%d" % G)
    p, s = check_pack2_exact(w, G, "stress G=%d" % G)
    # flagged groups hold code 0 everywhere: every field is 1
    n0 = w.shape[0] - special.shape[0]
    assert all((p[n0 + r] == 0x55).all() for r in (2, 3, 4))


@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (5, 128, 128), (37, 320, 64), (300, 1024, 128)])
def test_unpack2_every_byte_value(N, K, G):
    """Random bytes over 0..255, fields of 3 included: codes and the invalid
    flag exactly as the oracle's (a field of 3 reads as 0)."""
    rng = np.random.default_rng(310 + N)
    p = rng.integers(0, 256, size=(N, K // 4)).astype(np.uint8)
    say("unpack2 random bytes W[%d,%d] G=%d" % (N, K, G))
    c, st = gpu_unpack2(p, N, K, G)
    c_ref, st_ref = oracle.unpack2(p, N, K, G)
    assert np.array_equal(c, c_ref), np.argwhere(c != c_ref)[:5].tolist()
    assert st == st_ref == 4


def test_unpack2_valid_and_last_field():
    N, K, G = 9, 256, 64
    w = inputs.normal_bf16(320, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack2(w, G)
    c, st = gpu_unpack2(p, N, K, G)
    c_ref, _ = oracle.unpack2(p, N, K, G)
    assert st == 0 and np.array_equal(c, c_ref)
    bad = p.copy()
    bad.reshape(-1)[-1] |= 0xC0                  # the last weight's field becomes 3
    c, st = gpu_unpack2(bad, N, K, G)
    c_ref, st_ref = oracle.unpack2(bad, N, K, G)
    assert st == st_ref == 4 and np.array_equal(c, c_ref) and c[-1, -1] == 0


@pytest.mark.parametrize("N,K,G", [(1, 64, 64), (3, 128, 128), (17, 640, 64), (250, 1024, 128),
                                   (1025, 1088, 64), (100, 2048, 128), (300, 2112, 64),
                                   (64, 4096, 128), (3584, 1024, 128), (1024, 3584, 128),
                                   (70001, 256, 64)])
def test_gemv2_parity(N, K, G):
    """Row counts that leave ragged ring rounds and partial row steps, every
    lanes-per-row width (K/64 up to 16, 32 and 64), and grids capped at 512
    blocks (N = 70001)."""
    w = inputs.normal_bf16(330 + N, (N, K), 0.02)
    x = inputs.activation(331 + K, 1, K)
    p, s, _ = oracle.quantize_pack2(w, G)
    say("gemv2 W[%d,%d] G=%d" % (N, K, G))
    y, st = gpu_gemv2(x, p, s, N, K, G)
    y_ref, bound, st_ref = oracle.matmul2(x, p, s, N, K, G)
    assert st == st_ref == 0
    assert_within_bound(y, y_ref, bound, "gemv2 W[%d,%d] G=%d" % (N, K, G))


@pytest.mark.parametrize("G", [64, 128])
def test_gemv2_one_hot_exact(G):
    """x = e_k picks one column: y[n] = c[n,k] * s[n, k/G] exactly."""
    N, K = 200, 1024
    w = inputs.normal_bf16(340, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack2(w, G)
    c, _ = oracle.unpack2(p, N, K, G)
    sf = s.view(np.float16).astype(np.float64)
    for k in (0, 63, 64, G - 1, G + 5, K - 1):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = _bf16(1.0)
        y, st = gpu_gemv2(x, p, s, N, K, G)
        assert st == 0
        assert np.array_equal(y[0].astype(np.float64), c[:, k] * sf[:, k // G]), k


@pytest.mark.parametrize("G", [64, 128])
def test_gemv2_invalid_fields_flagged_and_read_as_zero(G):
    N, K = 130, 512
    w = inputs.normal_bf16(350, (N, K), 0.02)
    x = inputs.activation(351, 1, K)
    p, s, _ = oracle.quantize_pack2(w, G)
    bad = p.copy()
    bad[0, 0] |= 0x03                            # first field of the matrix
    bad[77, 40] |= 0x30
    bad.reshape(-1)[-1] |= 0xC0                  # last field of the matrix
    y, st = gpu_gemv2(x, bad, s, N, K, G)
    y_ref, bound, st_ref = oracle.matmul2(x, bad, s, N, K, G)
    assert st == st_ref == 4
    assert_within_bound(y, y_ref, bound, "invalid fields G=%d" % G)


def test_gemv2_nonfinite_activation_sets_no_flag():
    N, K, G = 64, 256, 64
    w = inputs.normal_bf16(360, (N, K), 0.02)
    p, s, _ = oracle.quantize_pack2(w, G)
    x = inputs.activation(361, 1, K)
    x[0, 5] = 0x7F80                             # +inf
    y, st = gpu_gemv2(x, p, s, N, K, G)
    assert st == 0


def test_gemv2_batched_matches_single_bitwise_at_stack_shapes():
    """The decode stack's shapes through one batched call per shape, each
    result bit-identical to the single call and within the bound of the
    oracle (every matrix checked)."""
    import torch
    import ternary_weight_only_amd as tq
    for N, K, count in ((3584, 1024, 6), (1024, 3584, 3)):
        G = 128
        ws = [inputs.normal_bf16(370 + i + K, (N, K), 0.02) for i in range(count)]
        xs = [inputs.activation(380 + i + K, 1, K) for i in range(count)]
        packs = [oracle.quantize_pack2(w, G)[:2] for w in ws]
        say("gemv2_batched %d x W[%d,%d]" % (count, N, K))
        st = tq.new_status()
        ys = tq.gemv2_batched([dev_bf16(x) for x in xs], [dev_u8(p) for p, _ in packs],
                              [dev_f16bits(s) for _, s in packs], N, K, G, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        for i in range(count):
            y1, _ = gpu_gemv2(xs[i], packs[i][0], packs[i][1], N, K, G)
            yb = ys[i].cpu().numpy()
            assert np.array_equal(yb.view(np.uint32), y1.view(np.uint32)), i
            y_ref, bound, _ = oracle.matmul2(xs[i], packs[i][0], packs[i][1], N, K, G)
            assert_within_bound(yb, y_ref, bound, "batched %d" % i)


def test_gemv2_repeatable():
    N, K, G = 3584, 1024, 128
    w = inputs.normal_bf16(390, (N, K), 0.02)
    x = inputs.activation(391, 1, K)
    p, s, _ = oracle.quantize_pack2(w, G)
    y1, _ = gpu_gemv2(x, p, s, N, K, G)
    y2, _ = gpu_gemv2(x, p, s, N, K, G)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_gemv2_agrees_with_base3_gemv_on_same_weights():
    """Same scales and codes in both formats: the two GEMVs agree within the
    sum of their bounds."""
    N, K, G = 1000, 1024, 128
    w = inputs.normal_bf16(395, (N, K), 0.02)
    x = inputs.activation(396, 1, K)
    p2, s2, _ = oracle.quantize_pack2(w, G)
    p3, s3, _ = oracle.quantize_pack(w, G)
    assert np.array_equal(s2, s3)
    from tests.gpu_helpers import gpu_matmul
    y2, _ = gpu_gemv2(x, p2, s2, N, K, G)
    y3, _ = gpu_matmul("gemv", x, p3, s3, N, K, G)
    _, bound, _ = oracle.matmul2(x, p2, s2, N, K, G)
    assert (np.abs(y2.astype(np.float64) - y3.astype(np.float64)) <= 2e-3 * bound).all()


def test_gemv2_grouped_mixed_shapes_bitwise_equal_to_single():
    """One grouped launch over problems of different shapes (the decode
    stack's two, a ragged one, every lanes-per-row width, a single row): each
    result bit-identical to tq_gemv2 on its own and within the oracle's
    bound."""
    import torch
    import ternary_weight_only_amd as tq
    G = 128
    shapes = [(3584, 1024)] * 5 + [(1024, 3584)] * 3 + [(1, 128), (777, 2048), (64, 4096),
                                                        (300, 1152)]
    probs = []
    for i, (N, K) in enumerate(shapes):
        w = inputs.normal_bf16(500 + i, (N, K), 0.02)
        p, s, _ = oracle.quantize_pack2(w, G)
        probs.append((inputs.activation(520 + i, 1, K), p, s))
    say("gemv2_grouped %d problems" % len(shapes))
    st = tq.new_status()
    ys = tq.gemv2_grouped([dev_bf16(x) for x, _, _ in probs], [dev_u8(p) for _, p, _ in probs],
                          [dev_f16bits(s) for _, _, s in probs], [N for N, _ in shapes],
                          [K for _, K in shapes], G, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for i, ((N, K), (x, p, s)) in enumerate(zip(shapes, probs)):
        yg = ys[i].cpu().numpy()
        y1, _ = gpu_gemv2(x, p, s, N, K, G)
        assert np.array_equal(yg.view(np.uint32), y1.view(np.uint32)), i
        if i in (0, 5, 8, 9, 10, 11):
            y_ref, bound, _ = oracle.matmul2(x, p, s, N, K, G)
            assert_within_bound(yg, y_ref, bound, "grouped %d" % i)


@pytest.mark.parametrize("G", [64, 128])
def test_quantize_pack2_batched_exact(G):
    """Batched 2-bit packing: every matrix bit-exact with the oracle (scales,
    fields, flags), including a matrix with a non-finite group."""
    import torch
    import ternary_weight_only_amd as tq
    N, K, count = 97, 1024, 5
    ws = [inputs.normal_bf16(700 + i + G, (N, K), 0.02) for i in range(count)]
    ws[3] = ws[3].copy()
    ws[3][10, 5] = 0x7FC1                          # NaN: its group is flagged
    say("quantize_pack2_batched %d x W[%d,%d] G=%d" % (count, N, K, G))
    st = tq.new_status()
    out = tq.quantize_pack2_batched([dev_bf16(w) for w in ws], G, status=st)
    torch.cuda.synchronize()
    flags = 0
    for i, (p, s) in enumerate(out):
        p_ref, s_ref, st_ref = oracle.quantize_pack2(ws[i], G)
        assert np.array_equal(p.cpu().numpy(), p_ref), i
        assert np.array_equal(host_u16(s), s_ref), i
        flags |= st_ref
    assert int(st.item()) == flags == 1
