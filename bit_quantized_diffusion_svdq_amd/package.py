"""Packaged SVDQ layers: one quantised layer's arrays plus the metadata that
says how to read them, in a safetensors file.

The donmalab.com page (section on quantising a model yourself) lists the
tool chain as inspect, quantize, package, validate; the remio.ai page
(section on how Diffusers support changes the loading path) says a
quantised checkpoint carries, per module, the scheme, precision, group size
and low-rank correction, and (section on what to watch after the Lite
release) that malformed configurations should fail with clear errors. This
module is the package step for one layer and the loader's checks:

* ``save_layer`` writes the layer's arrays (in the library's layouts) and
  a metadata record: format name and version, the library version whose
  layouts the arrays use, K, N, rank, group, number format, the layout of
  every array, and optional provenance (alpha, seed, anything else given).
* ``load_layer`` reads the file with safetensors' loader (no code runs from
  the file), checks the record with the library's own rules
  (svdq_validate_desc, svdq_layer_sizes_of), checks every array's dtype and
  byte size against them, and returns an ``SvdqLinear`` on the requested
  device. Any mismatch raises ``ValueError`` naming the field.

Marshalling only: no arithmetic of the method happens here.
"""
from __future__ import annotations

import json
import os

import torch

from . import _lib
from .block import SvdqLinear

FORMAT_NAME = "svdq-layer"
FORMAT_VERSION = 1

# dtype and layout of every array, by number format
_SPECS = {
    "int4": {
        "qw": (torch.uint8, "codes [N][K/2]: format v2, 16 sign-magnitude codes per 64-bit word as "
                            "FP6 E2M3 fields with the zero exponent bits folded out"),
        "sw": (torch.float16, "scales [ceil(K/256)][N][4] fp16: format v3, quad-major"),
    },
    "mxfp4": {
        "qw": (torch.uint8, "codes [N][K/2]: E2M1 nibbles, element 2i in bits 0-3 of byte i"),
        "sw": (torch.uint8, "E8M0 exponents [ceil(K/256)][N][8]: even blocks of a quad in bytes 0-3"),
    },
}
_COMMON = {
    "inv_lambda": (torch.float32, "smoothing reciprocals fp32 [K]"),
    "l1t": (torch.bfloat16, "down-projection L1 (K x rank) in the format v4 tile layout"),
    "l2t": (torch.bfloat16, "up-projection transposed, bf16 [N][rank]"),
    "bias": (torch.bfloat16, "bias bf16 [N]"),
}
_SIZE_KEY = {"qw": "qw", "sw": "sw", "l1t": "l1t", "l2t": "l2t", "inv_lambda": "inv_lambda", "bias": "bias"}


def _library_version() -> int:
    return int(_lib.load_library().svdq_version())


def _specs(fmt: str) -> dict:
    if fmt not in _SPECS:
        raise ValueError(f"unknown number format {fmt!r} (expected 'int4' or 'mxfp4')")
    return {**_SPECS[fmt], **_COMMON}


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def save_layer(path: str, layer: SvdqLinear, **provenance) -> dict:
    """Write ``layer`` to ``path`` (safetensors). ``provenance`` (for example
    alpha=0.5, seed=0) is stored as JSON in the metadata. Returns the
    metadata record."""
    from safetensors.torch import save_file

    desc = _lib.layer_desc(layer.K, layer.N, layer.rank, 64, layer.fmt)
    sizes = _lib.layer_sizes(desc)          # raises on a malformed layer
    specs = _specs(layer.fmt)
    arrays = {"qw": layer.qw, "sw": layer.sw, "inv_lambda": layer.inv_lambda}
    if layer.rank:
        arrays.update(l1t=layer.l1t, l2t=layer.l2t)
    if layer.bias is not None:
        arrays["bias"] = layer.bias
    tensors = {}
    for name, t in arrays.items():
        dtype, _ = specs[name]
        if t is None or t.dtype != dtype or _nbytes(t) != sizes[_SIZE_KEY[name]]:
            raise ValueError(f"{name}: expected {dtype} with {sizes[_SIZE_KEY[name]]} bytes, got "
                             f"{None if t is None else (t.dtype, _nbytes(t))}")
        tensors[name] = t.detach().to("cpu").contiguous()
    meta = {
        "format": FORMAT_NAME, "format_version": str(FORMAT_VERSION),
        "library_version": str(_library_version()),
        "K": str(layer.K), "N": str(layer.N), "rank": str(layer.rank), "group": "64", "fmt": layer.fmt,
        "layouts": json.dumps({n: specs[n][1] for n in tensors}),
        "provenance": json.dumps(provenance, sort_keys=True),
    }
    save_file(tensors, path, metadata=meta)
    return meta


def read_metadata(path: str) -> dict:
    """The metadata record of a packaged layer (no arrays are read)."""
    from safetensors import safe_open

    if not os.path.isfile(path):
        raise ValueError(f"{path}: no such file")
    try:
        with safe_open(path, framework="pt") as f:
            return dict(f.metadata() or {})
    except Exception as e:  # noqa: BLE001 - any parse failure is a malformed file
        raise ValueError(f"{path}: not a safetensors file ({e})") from e


def _int_field(meta: dict, key: str) -> int:
    if key not in meta:
        raise ValueError(f"metadata field {key!r} is missing")
    try:
        return int(meta[key])
    except ValueError:
        raise ValueError(f"metadata field {key!r} is not an integer: {meta[key]!r}") from None


def load_layer(path: str, device="cuda") -> SvdqLinear:
    """Read a packaged layer, check it, and return it on ``device``."""
    from safetensors.torch import load_file

    meta = read_metadata(path)
    if meta.get("format") != FORMAT_NAME:
        raise ValueError(f"{path}: format {meta.get('format')!r} is not {FORMAT_NAME!r}")
    if _int_field(meta, "format_version") != FORMAT_VERSION:
        raise ValueError(f"{path}: format version {meta['format_version']} is not {FORMAT_VERSION}")
    lib_v = _int_field(meta, "library_version")
    if lib_v // 100 != _library_version() // 100:
        raise ValueError(f"{path}: arrays use the layouts of library version {lib_v}, this library "
                         f"reads format {_library_version() // 100}")
    K, N, rank, group = (_int_field(meta, k) for k in ("K", "N", "rank", "group"))
    fmt = meta.get("fmt")
    specs = _specs(fmt)
    desc = _lib.layer_desc(K, N, rank, group, fmt)
    status = _lib.svdq_validate_desc(desc)
    if status != 0:
        detail = _lib.load_library().svdq_last_error().decode()
        raise ValueError(f"{path}: malformed layer record ({_lib.STATUS_NAMES.get(status, status)}: {detail})")
    sizes = _lib.layer_sizes(desc)
    tensors = load_file(path, device="cpu")
    need = ["qw", "sw", "inv_lambda"] + (["l1t", "l2t"] if rank else [])
    for name in need:
        if name not in tensors:
            raise ValueError(f"{path}: array {name!r} is missing")
    for name, t in tensors.items():
        if name not in specs:
            raise ValueError(f"{path}: unexpected array {name!r}")
        dtype, _ = specs[name]
        if t.dtype != dtype:
            raise ValueError(f"{path}: {name} has dtype {t.dtype}, expected {dtype}")
        if _nbytes(t) != sizes[_SIZE_KEY[name]]:
            raise ValueError(f"{path}: {name} has {_nbytes(t)} bytes, the record (K {K}, N {N}, rank {rank}, "
                             f"{fmt}) needs {sizes[_SIZE_KEY[name]]}")
    if tuple(tensors["qw"].shape) != (N, K // 2):
        raise ValueError(f"{path}: qw has shape {tuple(tensors['qw'].shape)}, expected {(N, K // 2)}")
    dev = torch.device(device)
    t = {k: v.to(dev) for k, v in tensors.items()}
    return SvdqLinear(t["inv_lambda"], t.get("l1t"), t.get("l2t"), t["qw"], t["sw"], t.get("bias"), rank, fmt)


# ---------------------------------------------------------------- AWQ W4A16 layers

AWQ_FORMAT_NAME = "awq-w4a16-layer"
_AWQ_SPECS = {
    "qwt": (torch.uint8, "unsigned 4-bit codes in the GEMV tile layout [N/16][K/128][16][64 B]"),
    "scale_t": (torch.float16, "scales [N/16][K/64][16] fp16"),
    "zero_t": (torch.float16, "zero points (integers 0..15) [N/16][K/64][16] fp16"),
    "inv_s": (torch.float32, "reciprocal activation-aware channel scales fp32 [K]"),
    "bias": (torch.bfloat16, "bias bf16 [N]"),
}


def _awq_sizes(K: int, N: int) -> dict:
    if K < 128 or K % 128 or N < 16 or N % 16:
        raise ValueError(f"AWQ layer needs K a positive multiple of 128 and N of 16, got K {K}, N {N}")
    return {"qwt": N * K // 2, "scale_t": N * (K // 64) * 2, "zero_t": N * (K // 64) * 2, "inv_s": K * 4,
            "bias": N * 2}


def save_awq_layer(path: str, layer: dict, bias=None, **provenance) -> dict:
    """Write an AWQ W4A16 layer (the dict quantize_awq returns: qwt, scale_t,
    zero_t, inv_s (or None), K, N; plus an optional bf16 bias) with its
    metadata record. Returns the record."""
    from safetensors.torch import save_file

    K, N = int(layer["K"]), int(layer["N"])
    sizes = _awq_sizes(K, N)
    arrays = {"qwt": layer["qwt"], "scale_t": layer["scale_t"], "zero_t": layer["zero_t"]}
    if layer.get("inv_s") is not None:
        arrays["inv_s"] = layer["inv_s"]
    if bias is not None:
        arrays["bias"] = bias
    tensors = {}
    for name, t in arrays.items():
        dtype, _ = _AWQ_SPECS[name]
        if t.dtype != dtype or _nbytes(t) != sizes[name]:
            raise ValueError(f"{name}: expected {dtype} with {sizes[name]} bytes, got {(t.dtype, _nbytes(t))}")
        tensors[name] = t.detach().to("cpu").contiguous().reshape(-1)
    meta = {
        "format": AWQ_FORMAT_NAME, "format_version": str(FORMAT_VERSION),
        "library_version": str(_library_version()), "K": str(K), "N": str(N), "group": "64",
        "layouts": json.dumps({n: _AWQ_SPECS[n][1] for n in tensors}),
        "provenance": json.dumps(provenance, sort_keys=True),
    }
    save_file(tensors, path, metadata=meta)
    return meta


def load_awq_layer(path: str, device="cuda") -> dict:
    """Read a packaged AWQ W4A16 layer, check it, and return the dict the GEMV
    takes (qwt, scale_t, zero_t, inv_s or None, bias or None, K, N) on
    ``device``."""
    from safetensors.torch import load_file

    meta = read_metadata(path)
    if meta.get("format") != AWQ_FORMAT_NAME:
        raise ValueError(f"{path}: format {meta.get('format')!r} is not {AWQ_FORMAT_NAME!r}")
    if _int_field(meta, "format_version") != FORMAT_VERSION:
        raise ValueError(f"{path}: format version {meta['format_version']} is not {FORMAT_VERSION}")
    lib_v = _int_field(meta, "library_version")
    if lib_v // 100 != _library_version() // 100:
        raise ValueError(f"{path}: arrays use the layouts of library version {lib_v}, this library "
                         f"reads format {_library_version() // 100}")
    if _int_field(meta, "group") != 64:
        raise ValueError(f"{path}: group {meta['group']} is not 64")
    K, N = _int_field(meta, "K"), _int_field(meta, "N")
    try:
        sizes = _awq_sizes(K, N)
    except ValueError as e:
        raise ValueError(f"{path}: malformed layer record ({e})") from None
    tensors = load_file(path, device="cpu")
    for name in ("qwt", "scale_t", "zero_t"):
        if name not in tensors:
            raise ValueError(f"{path}: array {name!r} is missing")
    for name, t in tensors.items():
        if name not in _AWQ_SPECS:
            raise ValueError(f"{path}: unexpected array {name!r}")
        dtype, _ = _AWQ_SPECS[name]
        if t.dtype != dtype:
            raise ValueError(f"{path}: {name} has dtype {t.dtype}, expected {dtype}")
        if _nbytes(t) != sizes[name]:
            raise ValueError(f"{path}: {name} has {_nbytes(t)} bytes, the record (K {K}, N {N}) needs {sizes[name]}")
    dev = torch.device(device)
    out = {k: v.to(dev) for k, v in tensors.items()}
    out.setdefault("inv_s", None)
    out.setdefault("bias", None)
    out.update(K=K, N=N)
    return out
