"""Ternary weight package: write, verify, decode to bf16.

Follows the package and decoder described for precisit "pack-unpack-run"
(README, screen.py description): one NPZ file per selected tensor holding
its packed codes and fp16 group scales, the unchanged tensors and the
tokenizer/configuration assets beside them, and a decoder that takes only
the package, checks its hashes, hands the selected weights back as bf16 and
checks every tensor again after the checkpoint is serialized.

Layout of a package directory:

    manifest.json            format, G, and per entry its file and hashes
    t00000.npz ...           a ternary tensor: "codes" uint8 [N, K/G*ceil(G/5)]
                             (the packed bytes of include/tq.h) and "scales"
                             float16 [N, K/G]
    u00000.npz ...           an unchanged tensor: "data" (bf16 kept as its
                             uint16 bit patterns, "dtype" in the manifest)
    a00000.bin ...           an asset, byte for byte

Every file is recorded with the sha256 of its bytes, and every array with
the sha256 of its contents; reading checks both and refuses anything else
(missing or extra arrays, other dtypes or shapes, object arrays -- NPZ files
are opened with allow_pickle=False, so nothing in a file is executed).

Quantizing and decoding run in libtq.so (tq_quantize_pack,
tq_dequantize_batched); this module moves bytes between files and device
tensors and checks them.
"""
from __future__ import annotations

import hashlib
import json
import os
from dataclasses import dataclass, field

import numpy as np

FORMAT = "tq-ternary-base3/1"
MANIFEST = "manifest.json"


class PackageError(RuntimeError):
    pass


@dataclass
class TernaryTensor:
    """Packed codes (uint8 [N, K/G*ceil(G/5)]) and fp16 scales ([N, K/G])."""
    codes: np.ndarray
    scales: np.ndarray
    shape: tuple


@dataclass
class Package:
    G: int
    tensors: dict = field(default_factory=dict)      # name -> TernaryTensor
    unchanged: dict = field(default_factory=dict)    # name -> (np.ndarray, dtype name)
    assets: dict = field(default_factory=dict)       # name -> bytes


def _sha(b: bytes) -> str:
    return hashlib.sha256(b).hexdigest()


def _arr_sha(a: np.ndarray) -> str:
    return _sha(np.ascontiguousarray(a).tobytes())


def _row_bytes(K: int, G: int) -> int:
    return (K // G) * ((G + 4) // 5)


def _check_ternary(name, codes, scales, shape, G):
    if G not in (64, 128):
        raise PackageError("%s: G=%r not supported" % (name, G))
    if len(shape) != 2:
        raise PackageError("%s: shape %r is not 2-D" % (name, shape))
    N, K = int(shape[0]), int(shape[1])
    if N < 1 or K < 1 or K % G:
        raise PackageError("%s: shape %r does not split into groups of %d" % (name, shape, G))
    if codes.dtype != np.uint8 or codes.shape != (N, _row_bytes(K, G)):
        raise PackageError("%s: codes %s %r, expected uint8 %r"
                           % (name, codes.dtype, codes.shape, (N, _row_bytes(K, G))))
    if scales.dtype != np.float16 or scales.shape != (N, K // G):
        raise PackageError("%s: scales %s %r, expected float16 %r"
                           % (name, scales.dtype, scales.shape, (N, K // G)))


def _write_npz(path: str, arrays: dict) -> bytes:
    tmp = path + ".tmp"
    with open(tmp, "wb") as f:
        np.savez(f, **arrays)
    os.replace(tmp, path)
    with open(path, "rb") as f:
        return f.read()


def write_package(path: str, pkg: Package) -> dict:
    """Write `pkg` into the directory `path` (created if missing; files of
    the same names are replaced).  Returns the manifest."""
    os.makedirs(path, exist_ok=True)
    man = {"format": FORMAT, "G": int(pkg.G), "tensors": {}, "unchanged": {}, "assets": {}}
    for i, (name, t) in enumerate(sorted(pkg.tensors.items())):
        codes = np.ascontiguousarray(t.codes)
        scales = np.ascontiguousarray(t.scales)
        if scales.dtype == np.uint16:
            scales = scales.view(np.float16)
        _check_ternary(name, codes, scales, t.shape, pkg.G)
        fname = "t%05d.npz" % i
        raw = _write_npz(os.path.join(path, fname), {"codes": codes, "scales": scales})
        man["tensors"][name] = {"file": fname, "shape": [int(s) for s in t.shape],
                                "sha256": _sha(raw), "codes_sha256": _arr_sha(codes),
                                "scales_sha256": _arr_sha(scales)}
    for i, (name, (a, dtype)) in enumerate(sorted(pkg.unchanged.items())):
        a = np.ascontiguousarray(a)
        fname = "u%05d.npz" % i
        raw = _write_npz(os.path.join(path, fname), {"data": a})
        man["unchanged"][name] = {"file": fname, "dtype": dtype, "shape": list(a.shape),
                                  "sha256": _sha(raw), "data_sha256": _arr_sha(a)}
    for i, (name, data) in enumerate(sorted(pkg.assets.items())):
        fname = "a%05d.bin" % i
        with open(os.path.join(path, fname), "wb") as f:
            f.write(bytes(data))
        man["assets"][name] = {"file": fname, "sha256": _sha(bytes(data))}
    tmp = os.path.join(path, MANIFEST + ".tmp")
    with open(tmp, "w") as f:
        json.dump(man, f, indent=1, sort_keys=True)
    os.replace(tmp, os.path.join(path, MANIFEST))
    return man


def _read_verified(path: str, entry: dict) -> bytes:
    fname = entry.get("file")
    if not isinstance(fname, str) or os.path.basename(fname) != fname or not fname:
        raise PackageError("bad file name %r in the manifest" % (fname,))
    fp = os.path.join(path, fname)
    try:
        with open(fp, "rb") as f:
            raw = f.read()
    except OSError as e:
        raise PackageError("%s: %s" % (fname, e)) from None
    if _sha(raw) != entry.get("sha256"):
        raise PackageError("%s: sha256 does not match the manifest" % fname)
    return raw


def _load_npz(raw: bytes, fname: str, keys: set) -> dict:
    import io
    try:
        with np.load(io.BytesIO(raw), allow_pickle=False) as z:
            if set(z.files) != keys:
                raise PackageError("%s holds arrays %s, expected %s"
                                   % (fname, sorted(z.files), sorted(keys)))
            return {k: z[k] for k in keys}
    except PackageError:
        raise
    except Exception as e:  # a broken or object-holding file
        raise PackageError("%s: not a plain NPZ of numeric arrays (%s)" % (fname, e)) from None


def read_package(path: str) -> Package:
    """Read and verify a package: the manifest's format, every file's sha256,
    every array's dtype, shape and sha256.  Raises PackageError on any
    mismatch."""
    try:
        with open(os.path.join(path, MANIFEST)) as f:
            man = json.load(f)
    except (OSError, ValueError) as e:
        raise PackageError("manifest: %s" % e) from None
    if not isinstance(man, dict) or man.get("format") != FORMAT:
        raise PackageError("not a %s package" % FORMAT)
    G = man.get("G")
    pkg = Package(G=G)
    for name, e in man.get("tensors", {}).items():
        raw = _read_verified(path, e)
        arrs = _load_npz(raw, e["file"], {"codes", "scales"})
        shape = tuple(e.get("shape", ()))
        _check_ternary(name, arrs["codes"], arrs["scales"], shape, G)
        if _arr_sha(arrs["codes"]) != e.get("codes_sha256") or \
                _arr_sha(arrs["scales"]) != e.get("scales_sha256"):
            raise PackageError("%s: array hashes do not match the manifest" % name)
        pkg.tensors[name] = TernaryTensor(arrs["codes"], arrs["scales"], shape)
    for name, e in man.get("unchanged", {}).items():
        raw = _read_verified(path, e)
        a = _load_npz(raw, e["file"], {"data"})["data"]
        if list(a.shape) != list(e.get("shape", [])) or _arr_sha(a) != e.get("data_sha256"):
            raise PackageError("%s: unchanged tensor does not match the manifest" % name)
        pkg.unchanged[name] = (a, e.get("dtype", str(a.dtype)))
    for name, e in man.get("assets", {}).items():
        pkg.assets[name] = _read_verified(path, e)
    return pkg


# ---------------------------------------------------------------------------
# device side: quantize into a package, decode a package
# ---------------------------------------------------------------------------

def _torch_dtype(name: str):
    import torch
    return {"bfloat16": torch.bfloat16, "float16": torch.float16, "float32": torch.float32,
            "int64": torch.int64, "int32": torch.int32, "uint8": torch.uint8}[name]


def from_device(weights: dict, G: int, unchanged: dict | None = None,
                assets: dict | None = None) -> Package:
    """Quantize device bf16 matrices with tq_quantize_pack into a Package.

    weights: name -> bf16 [N,K] device tensor; unchanged: name -> any tensor
    kept as is (bf16 stored as its bit patterns); assets: name -> bytes.
    Raises PackageError if the device reports a non-finite weight or a scale
    overflow."""
    import torch
    from . import binding as tq
    pkg = Package(G=G, assets=dict(assets or {}))
    st = tq.new_status(next(iter(weights.values())).device if weights else None)
    dev = {}
    for name, w in weights.items():
        dev[name] = (tq.quantize_pack(w, G, status=st), tuple(w.shape))
    if weights:
        torch.cuda.synchronize()
        if tq.check(st):
            raise PackageError("quantize_pack reported device status %d" % tq.check(st))
    for name, ((p, s), shape) in dev.items():
        N, K = shape
        pkg.tensors[name] = TernaryTensor(p.cpu().numpy().reshape(N, -1),
                                          s.cpu().numpy().reshape(N, -1), shape)
    for name, t in (unchanged or {}).items():
        t = t.detach().contiguous().cpu()
        dtype = str(t.dtype).replace("torch.", "")
        a = t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
        pkg.unchanged[name] = (a.copy(), dtype)
    return pkg


def decode(pkg: Package, device="cuda") -> dict:
    """Decode every ternary tensor to bf16 on the device (one
    tq_dequantize_batched call per shape) and move the unchanged tensors
    there.  Raises PackageError if the device flags an invalid byte, a
    non-zero padding trit or a non-finite scale."""
    import torch
    from . import binding as tq
    out = {}
    st = tq.new_status(device)
    by_shape = {}
    for name, t in pkg.tensors.items():
        by_shape.setdefault(tuple(t.shape), []).append(name)
    for (N, K), names in by_shape.items():
        pk = [torch.from_numpy(np.ascontiguousarray(pkg.tensors[n].codes)).to(device)
              for n in names]
        sc = [torch.from_numpy(np.ascontiguousarray(pkg.tensors[n].scales)).to(device)
              for n in names]
        for n, w in zip(names, tq.dequantize_batched(pk, sc, N, K, pkg.G, status=st)):
            out[n] = w
    torch.cuda.synchronize()
    if tq.check(st):
        raise PackageError("decode reported device status %d" % tq.check(st))
    for name, (a, dtype) in pkg.unchanged.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dtype == "bfloat16":
            t = t.view(torch.int16).view(torch.bfloat16)
        elif str(t.dtype).replace("torch.", "") != dtype:
            raise PackageError("%s: stored as %s, recorded as %s" % (name, t.dtype, dtype))
        out[name] = t.to(device)
    return out


def save_checkpoint(tensors: dict, path: str) -> str:
    """Serialize tensors to a safetensors file, read it back and compare
    every tensor bit for bit.  Returns the file's sha256."""
    import torch
    from safetensors.torch import load_file, save_file
    host = {k: v.detach().contiguous().cpu() for k, v in tensors.items()}
    save_file(host, path)
    back = load_file(path)
    if set(back) != set(host):
        raise PackageError("checkpoint holds %d tensors, expected %d" % (len(back), len(host)))
    for k, v in host.items():
        b = back[k]
        if b.dtype != v.dtype or b.shape != v.shape or not torch.equal(
                b.reshape(-1).view(torch.uint8), v.reshape(-1).view(torch.uint8)):
            raise PackageError("checkpoint tensor %s differs after serialization" % k)
    with open(path, "rb") as f:
        return _sha(f.read())
