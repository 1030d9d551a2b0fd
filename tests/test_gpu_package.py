"""File replay of the ternary weight package through the device: quantize
on the GPU, write, read back, decode to bf16 on the GPU, serialize the
checkpoint (precisit "pack-unpack-run" README, screen.py description: the
decoder takes only the package, verifies hashes, hands the weights back as
bf16 and checks every tensor after serialization; test_codec.py
description: file replay, and a changed valid code byte must change the
reconstruction).  Every decoded tensor is compared with the oracle's
decode of the oracle's packing, bit for bit."""
import json

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from tests.gpu_helpers import dev_bf16, host_u16, say

pytestmark = pytest.mark.gpu

SHAPES = {"layers.0.mlp.gate_proj.weight": (3584, 1024), "layers.0.mlp.up_proj.weight": (3584, 1024),
          "layers.0.mlp.down_proj.weight": (1024, 3584), "layers.1.mlp.gate_proj.weight": (200, 640)}


def _weights():
    return {n: inputs.normal_bf16(300 + i, s, 0.02) for i, (n, s) in enumerate(SHAPES.items())}


@pytest.mark.parametrize("G", [64, 128])
def test_replay_write_read_decode(tmp_path, G):
    import torch
    from ternary_weight_only_amd import package
    w = _weights()
    emb = inputs.normal_bf16(399, (64, 32), 1.0)
    say("package replay G=%d" % G)
    pkg = package.from_device({n: dev_bf16(a) for n, a in w.items()}, G,
                              unchanged={"embed_tokens.weight": dev_bf16(emb)},
                              assets={"config.json": b'{"layers": 2}'})
    package.write_package(str(tmp_path), pkg)
    dec1 = package.decode(package.read_package(str(tmp_path)))
    dec2 = package.decode(package.read_package(str(tmp_path)))
    for n, a in w.items():
        N, K = SHAPES[n]
        p, s, st = oracle.quantize_pack(a, G)
        assert st == 0
        ref, _ = oracle.dequantize(p, s, N, K, G)
        got = host_u16(dec1[n])
        assert np.array_equal(got, ref), n
        assert np.array_equal(host_u16(dec2[n]), got), n
    assert np.array_equal(host_u16(dec1["embed_tokens.weight"]), emb)
    sha = package.save_checkpoint(dec1, str(tmp_path / "decoded.safetensors"))
    assert sha == package.save_checkpoint(dec2, str(tmp_path / "decoded2.safetensors"))
    torch.cuda.synchronize()


def test_changed_code_byte_changes_reconstruction(tmp_path):
    """A package rewritten with one valid code byte changed (new hashes)
    decodes differently, exactly at that byte's five weights where their
    codes differ, and equal to the oracle's decode of the changed bytes."""
    from ternary_weight_only_amd import package
    n = "layers.1.mlp.gate_proj.weight"
    N, K = SHAPES[n]
    G = 64
    a = _weights()[n]
    pkg = package.from_device({n: dev_bf16(a)}, G)
    package.write_package(str(tmp_path / "a"), pkg)
    base = host_u16(package.decode(package.read_package(str(tmp_path / "a")))[n])
    t = pkg.tensors[n]
    row, b = 17, 5                      # byte 5 of group 0: weights 25..29 of row 17
    codes = t.codes.copy()
    codes[row, b] = (int(codes[row, b]) + 1) % 243
    pkg2 = package.Package(G=G, tensors={n: package.TernaryTensor(codes, t.scales, t.shape)})
    package.write_package(str(tmp_path / "b"), pkg2)
    say("package changed byte")
    got = host_u16(package.decode(package.read_package(str(tmp_path / "b")))[n])
    ref, st = oracle.dequantize(codes, t.scales.view(np.uint16), N, K, G)
    assert st == 0 and np.array_equal(got, ref)
    diff = np.argwhere(got != base)
    assert len(diff) >= 1
    assert all(r == row and 25 <= c < 30 for r, c in diff)


def test_decode_refuses_invalid_bytes_and_tampering(tmp_path):
    from ternary_weight_only_amd import package
    n = "layers.1.mlp.gate_proj.weight"
    G = 128
    pkg = package.from_device({n: dev_bf16(_weights()[n])}, G)
    t = pkg.tensors[n]
    codes = t.codes.copy()
    codes[3, 7] = 249                   # an invalid byte, consistently hashed
    package.write_package(str(tmp_path), package.Package(
        G=G, tensors={n: package.TernaryTensor(codes, t.scales, t.shape)}))
    with pytest.raises(package.PackageError, match="device status 4"):
        package.decode(package.read_package(str(tmp_path)))
    # a valid package whose bytes change after writing is refused before decoding
    package.write_package(str(tmp_path), pkg)
    man = json.loads((tmp_path / "manifest.json").read_text())
    f = tmp_path / man["tensors"][n]["file"]
    raw = bytearray(f.read_bytes())
    raw[-40] ^= 0x10
    f.write_bytes(bytes(raw))
    with pytest.raises(package.PackageError, match="sha256"):
        package.read_package(str(tmp_path))
