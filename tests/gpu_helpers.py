"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its C ABI, and compare with the CPU oracle."""
import sys

import numpy as np
import torch

import oracle
import ternary_weight_only_amd as tq


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def dev_f16bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.float16)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_quantize(w_bits: np.ndarray, G: int):
    w = dev_bf16(w_bits)
    st = tq.new_status()
    packed, scales = tq.quantize_pack(w, G, status=st)
    torch.cuda.synchronize()
    return packed.cpu().numpy(), host_u16(scales), int(st.item())


def gpu_unpack(packed: np.ndarray, N: int, K: int, G: int):
    st = tq.new_status()
    codes = tq.unpack(dev_u8(packed), N, K, G, status=st)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), int(st.item())


def gpu_matmul(kind: str, x_bits, packed, scales, N, K, G):
    st = tq.new_status()
    fn = tq.gemv if kind == "gemv" else tq.gemm
    y = fn(dev_bf16(x_bits), dev_u8(packed), dev_f16bits(scales), N, K, G, status=st)
    torch.cuda.synchronize()
    return y.cpu().numpy(), int(st.item())


def assert_within_bound(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str):
    """|y_gpu - y_ref| <= 1e-3 * sum_k |x_k w_hat_k| per element (y_ref in fp64)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = 1e-3 * bound
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outside 1e-3*bound; first at %s: gpu=%r ref=%r bound=%r"
                             % (what, int(bad.sum()), bad.size, tuple(i), float(y_gpu[tuple(i)]),
                                float(y_ref[tuple(i)]), float(bound[tuple(i)])))
    assert np.isfinite(y_gpu).all(), what


def check_quantize_exact(w_bits: np.ndarray, G: int, what: str):
    p_gpu, s_gpu, st_gpu = gpu_quantize(w_bits, G)
    p_ref, s_ref, st_ref = oracle.quantize_pack(w_bits, G)
    assert np.array_equal(s_gpu, s_ref), "%s: scales differ at %s" % (
        what, np.argwhere(s_gpu != s_ref)[:5].tolist())
    assert np.array_equal(p_gpu, p_ref), "%s: packed differ at %s" % (
        what, np.argwhere(p_gpu != p_ref)[:5].tolist())
    assert st_gpu == st_ref, "%s: status %d vs %d" % (what, st_gpu, st_ref)
    return p_ref, s_ref
