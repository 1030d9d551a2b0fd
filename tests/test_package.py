"""The ternary weight package on the host: write, read back, verify hashes,
refuse tampered or foreign files (precisit "pack-unpack-run" README,
screen.py description: per-tensor NPZ files of codes and fp16 scales, a
decoder that takes only the package and checks its hashes; test_codec.py
description: file replay)."""
import json
import os

import numpy as np
import pytest

import oracle
from ternary_weight_only_amd import inputs
from ternary_weight_only_amd.package import (FORMAT, Package, PackageError, TernaryTensor,
                                             read_package, write_package)


def _pkg(G=64):
    pkg = Package(G=G)
    for i, (N, K) in enumerate([(48, 256), (16, 512), (48, 256)]):
        w = inputs.normal_bf16(200 + i, (N, K), 0.02)
        p, s, st = oracle.quantize_pack(w, G)
        assert st == 0
        pkg.tensors["layers.%d.mlp.weight" % i] = TernaryTensor(p, s.view(np.float16), (N, K))
    pkg.unchanged["embed.weight"] = (inputs.normal_bf16(210, (10, 8), 1.0), "bfloat16")
    pkg.unchanged["norm.weight"] = (np.arange(8, dtype=np.float32), "float32")
    pkg.assets["config.json"] = b'{"hidden_size": 256}'
    pkg.assets["tokenizer.json"] = bytes(range(256))
    return pkg


def test_write_read_round_trip(tmp_path):
    pkg = _pkg()
    man = write_package(str(tmp_path), pkg)
    assert man["format"] == FORMAT and man["G"] == 64
    back = read_package(str(tmp_path))
    assert back.G == 64 and set(back.tensors) == set(pkg.tensors)
    for name, t in pkg.tensors.items():
        b = back.tensors[name]
        assert b.shape == t.shape
        assert np.array_equal(b.codes, t.codes)
        assert np.array_equal(b.scales.view(np.uint16), t.scales.view(np.uint16))
    for name, (a, dt) in pkg.unchanged.items():
        assert back.unchanged[name][1] == dt and np.array_equal(back.unchanged[name][0], a)
    assert back.assets == pkg.assets


def test_rewrite_gives_identical_files(tmp_path):
    """Writing the same package twice gives the same bytes and hashes."""
    a, b = tmp_path / "a", tmp_path / "b"
    ma = write_package(str(a), _pkg())
    mb = write_package(str(b), _pkg())
    assert ma == mb
    for f in os.listdir(a):
        assert (a / f).read_bytes() == (b / f).read_bytes(), f


def test_a_flipped_byte_in_any_file_is_refused(tmp_path):
    write_package(str(tmp_path), _pkg())
    for f in sorted(os.listdir(tmp_path)):
        if f == "manifest.json":
            continue
        raw = bytearray((tmp_path / f).read_bytes())
        pos = len(raw) // 2
        raw[pos] ^= 1
        (tmp_path / f).write_bytes(bytes(raw))
        with pytest.raises(PackageError, match="sha256"):
            read_package(str(tmp_path))
        raw[pos] ^= 1
        (tmp_path / f).write_bytes(bytes(raw))
        read_package(str(tmp_path))  # restored: accepted again


def test_manifest_and_file_errors(tmp_path):
    write_package(str(tmp_path), _pkg())
    man_path = tmp_path / "manifest.json"
    man = json.loads(man_path.read_text())

    def with_manifest(m, match):
        man_path.write_text(json.dumps(m))
        with pytest.raises(PackageError, match=match):
            read_package(str(tmp_path))
        man_path.write_text(json.dumps(man))

    name = sorted(man["tensors"])[0]
    m = json.loads(json.dumps(man)); m["format"] = "something else"
    with_manifest(m, "package")
    m = json.loads(json.dumps(man)); m["tensors"][name]["file"] = "../t00000.npz"
    with_manifest(m, "bad file name")
    m = json.loads(json.dumps(man)); m["tensors"][name]["file"] = "missing.npz"
    with_manifest(m, "missing.npz")
    m = json.loads(json.dumps(man)); m["tensors"][name]["shape"] = [48, 320]
    with_manifest(m, "codes")
    m = json.loads(json.dumps(man)); m["G"] = 128
    with_manifest(m, "groups|codes|scales")  # 4 x 13 bytes == 2 x 26: only the scales differ
    m = json.loads(json.dumps(man)); m["tensors"][name]["codes_sha256"] = "0" * 64
    with_manifest(m, "array hashes")
    man_path.write_text("{not json")
    with pytest.raises(PackageError, match="manifest"):
        read_package(str(tmp_path))


def test_foreign_npz_contents_are_refused_without_unpickling(tmp_path):
    """A file holding an object array (pickled data), an extra array or the
    wrong dtype is refused even when its hash matches; nothing is unpickled."""
    import hashlib
    write_package(str(tmp_path), _pkg())
    man_path = tmp_path / "manifest.json"
    man = json.loads(man_path.read_text())
    name = sorted(man["tensors"])[0]
    entry = man["tensors"][name]
    good = np.load(tmp_path / entry["file"])
    codes, scales = good["codes"], good["scales"]
    cases = [
        ({"codes": np.array([{"x": 1}], dtype=object), "scales": scales}, "plain NPZ"),
        ({"codes": codes, "scales": scales, "extra": codes}, "holds arrays"),
        ({"codes": codes.astype(np.int16), "scales": scales}, "codes"),
        ({"codes": codes, "scales": scales.view(np.uint16)}, "scales"),
    ]
    for arrays, match in cases:
        f = tmp_path / entry["file"]
        with open(f, "wb") as fh:
            np.savez(fh, **arrays)
        entry["sha256"] = hashlib.sha256(f.read_bytes()).hexdigest()
        man_path.write_text(json.dumps(man))
        with pytest.raises(PackageError, match=match):
            read_package(str(tmp_path))


def test_writer_refuses_inconsistent_tensors(tmp_path):
    pkg = _pkg()
    name = sorted(pkg.tensors)[0]
    t = pkg.tensors[name]
    pkg.tensors[name] = TernaryTensor(t.codes[:, :-1], t.scales, t.shape)
    with pytest.raises(PackageError, match="codes"):
        write_package(str(tmp_path), pkg)
    pkg.tensors[name] = TernaryTensor(t.codes, t.scales, (48, 250))
    with pytest.raises(PackageError, match="groups"):
        write_package(str(tmp_path), pkg)
