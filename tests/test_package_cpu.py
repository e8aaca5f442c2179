"""Packaged layers (save_layer / load_layer for SVDQ layers, save_awq_layer /
load_awq_layer for AWQ W4A16 layers) on the host: round trips in both SVDQ
number formats and for AWQ, the metadata record, and every malformed-file
error the loaders document. No GPU: arrays stay on the CPU and the library is used
only for its host-side checks (svdq_validate_desc, svdq_layer_sizes_of)."""
import json

import pytest
import torch
from safetensors.torch import load_file, save_file

import bit_quantized_diffusion_svdq_amd as svdq
from bit_quantized_diffusion_svdq_amd import SvdqLinear, load_layer, read_metadata, save_layer


def make_layer(K=512, N=192, rank=32, fmt="int4", bias=True, seed=0):
    g = torch.Generator().manual_seed(seed)
    G4 = (K // 64 + 3) // 4
    qw = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8)
    if fmt == "int4":
        sw = torch.rand((G4, N, 4), generator=g).to(torch.float16)
    else:
        sw = torch.randint(110, 130, (G4, N, 8), generator=g, dtype=torch.uint8)
    inv = torch.rand(K, generator=g) + 0.5
    l1t = torch.randn(K * rank, generator=g).to(torch.bfloat16) if rank else None
    l2t = torch.randn((N, rank), generator=g).to(torch.bfloat16) if rank else None
    b = torch.randn(N, generator=g).to(torch.bfloat16) if bias else None
    return SvdqLinear(inv, l1t, l2t, qw, sw, b, rank, fmt)


def same(a, b):
    return (a is None and b is None) or (a is not None and b is not None and a.dtype == b.dtype
                                         and torch.equal(a.view(torch.uint8), b.view(torch.uint8)))


@pytest.mark.parametrize("fmt,rank,bias", [("int4", 32, True), ("mxfp4", 0, False), ("int4", 0, True),
                                           ("mxfp4", 16, True)])
def test_round_trip(tmp_path, fmt, rank, bias):
    layer = make_layer(rank=rank, fmt=fmt, bias=bias)
    p = str(tmp_path / "layer.safetensors")
    meta = save_layer(p, layer, alpha=0.5, seed=7)
    back = load_layer(p, device="cpu")
    assert (back.K, back.N, back.rank, back.fmt) == (layer.K, layer.N, layer.rank, layer.fmt)
    for name in ("inv_lambda", "l1t", "l2t", "qw", "sw", "bias"):
        assert same(getattr(back, name), getattr(layer, name)), name
    m = read_metadata(p)
    assert m == meta
    assert m["format"] == "svdq-layer" and m["fmt"] == fmt and int(m["K"]) == 512 and int(m["N"]) == 192
    assert int(m["library_version"]) == svdq.load_library().svdq_version()
    assert json.loads(m["provenance"]) == {"alpha": 0.5, "seed": 7}
    assert set(json.loads(m["layouts"])) == {"qw", "sw", "inv_lambda"} | ({"l1t", "l2t"} if rank else set()) \
        | ({"bias"} if bias else set())


def test_save_rejects_a_malformed_layer(tmp_path):
    layer = make_layer()
    layer.sw = layer.sw[:, :-8]                     # too few scale rows
    with pytest.raises(ValueError, match="sw"):
        save_layer(str(tmp_path / "x.safetensors"), layer)
    layer = make_layer(fmt="int4")
    layer.sw = layer.sw.view(torch.uint8)           # wrong dtype for INT4 scales
    with pytest.raises(ValueError, match="sw"):
        save_layer(str(tmp_path / "x.safetensors"), layer)


def rewrite(tmp_path, src, tensors=None, meta=None):
    t = load_file(src)
    m = read_metadata(src)
    if tensors:
        tensors(t)
    if meta:
        meta(m)
    p = str(tmp_path / "bad.safetensors")
    save_file(t, p, metadata=m)
    return p


@pytest.mark.parametrize("case,match", [
    ("format", "format"), ("format_version", "format version"), ("library_version", "library version"),
    ("K_not_integer", "not an integer"), ("K_missing", "missing"), ("K_ragged", "malformed layer record"),
    ("group", "malformed layer record"), ("fmt", "unknown number format"), ("rank", "malformed layer record"),
    ("K_mismatch", "bytes"), ("missing_l1t", "missing"), ("dtype", "dtype"), ("extra", "unexpected"),
    ("qw_shape", "shape"),
])
def test_load_rejects(tmp_path, case, match):
    good = str(tmp_path / "good.safetensors")
    save_layer(good, make_layer())
    edits = {
        "format": dict(meta=lambda m: m.update(format="other")),
        "format_version": dict(meta=lambda m: m.update(format_version="2")),
        "library_version": dict(meta=lambda m: m.update(library_version="302")),
        "K_not_integer": dict(meta=lambda m: m.update(K="512.0")),
        "K_missing": dict(meta=lambda m: m.pop("K")),
        "K_ragged": dict(meta=lambda m: m.update(K="520")),
        "group": dict(meta=lambda m: m.update(group="128")),
        "fmt": dict(meta=lambda m: m.update(fmt="nf4")),
        "rank": dict(meta=lambda m: m.update(rank="24")),
        "K_mismatch": dict(meta=lambda m: m.update(K="1024")),
        "missing_l1t": dict(tensors=lambda t: t.pop("l1t")),
        "dtype": dict(tensors=lambda t: t.update(inv_lambda=t["inv_lambda"].to(torch.float64)[: t["inv_lambda"].numel() // 2])),
        "extra": dict(tensors=lambda t: t.update(l3=torch.zeros(4))),
        "qw_shape": dict(tensors=lambda t: t.update(qw=t["qw"].reshape(-1, 128))),
    }
    p = rewrite(tmp_path, good, **edits[case])
    with pytest.raises(ValueError, match=match):
        load_layer(p, device="cpu")


def test_load_rejects_files_that_are_not_packaged_layers(tmp_path):
    with pytest.raises(ValueError, match="no such file"):
        load_layer(str(tmp_path / "absent.safetensors"), device="cpu")
    junk = tmp_path / "junk.safetensors"
    junk.write_bytes(b"\x10\x00\x00\x00\x00\x00\x00\x00not json at all!")
    with pytest.raises(ValueError, match="not a safetensors file"):
        load_layer(str(junk), device="cpu")


# ---------------------------------------------------------------- AWQ W4A16 layers

def make_awq(K=256, N=48, scaled=True, seed=1):
    g = torch.Generator().manual_seed(seed)
    return dict(qwt=torch.randint(0, 256, (N * K // 2,), generator=g, dtype=torch.uint8),
                scale_t=torch.rand(N * K // 64, generator=g).to(torch.float16),
                zero_t=torch.randint(0, 16, (N * K // 64,), generator=g).to(torch.float16),
                inv_s=(torch.rand(K, generator=g) + 0.5) if scaled else None, K=K, N=N)


@pytest.mark.parametrize("scaled,bias", [(True, True), (False, False)])
def test_awq_round_trip(tmp_path, scaled, bias):
    layer = make_awq(scaled=scaled)
    b = torch.randn(48).to(torch.bfloat16) if bias else None
    p = str(tmp_path / "awq.safetensors")
    meta = svdq.save_awq_layer(p, layer, bias=b, seed=3)
    back = svdq.load_awq_layer(p, device="cpu")
    assert (back["K"], back["N"]) == (256, 48)
    for name in ("qwt", "scale_t", "zero_t", "inv_s"):
        assert same(back[name], layer[name]), name
    assert same(back["bias"], b)
    assert read_metadata(p) == meta and meta["format"] == "awq-w4a16-layer"


@pytest.mark.parametrize("case,match", [
    ("format", "format"), ("N_ragged", "malformed layer record"), ("K_mismatch", "bytes"),
    ("missing", "missing"), ("dtype", "dtype"), ("group", "group"),
])
def test_awq_load_rejects(tmp_path, case, match):
    good = str(tmp_path / "good.safetensors")
    svdq.save_awq_layer(good, make_awq())
    edits = {
        "format": dict(meta=lambda m: m.update(format="svdq-layer")),
        "N_ragged": dict(meta=lambda m: m.update(N="40")),
        "K_mismatch": dict(meta=lambda m: m.update(K="512")),
        "missing": dict(tensors=lambda t: t.pop("zero_t")),
        "dtype": dict(tensors=lambda t: t.update(scale_t=t["scale_t"].view(torch.bfloat16))),
        "group": dict(meta=lambda m: m.update(group="128")),
    }
    p = rewrite(tmp_path, good, **edits[case])
    with pytest.raises(ValueError, match=match):
        svdq.load_awq_layer(p, device="cpu")


def test_layer_kinds_are_not_interchangeable(tmp_path):
    a = str(tmp_path / "awq.safetensors")
    s = str(tmp_path / "svdq.safetensors")
    svdq.save_awq_layer(a, make_awq())
    save_layer(s, make_layer())
    with pytest.raises(ValueError, match="format"):
        load_layer(a, device="cpu")
    with pytest.raises(ValueError, match="format"):
        svdq.load_awq_layer(s, device="cpu")
