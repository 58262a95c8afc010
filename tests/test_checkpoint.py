"""The mmap-loaded safetensors checkpoint (host side): the file is a valid
safetensors file that a third-party reader decodes to the same bf16 values,
each block's tensors follow the oracle's parameter table back to back, and
malformed files are rejected before anything is loaded."""
import json
import struct

import numpy as np
import pytest

import synth
from oracle import layout as OL
from layerwise_weight_streaming_dit_amd import checkpoint as C


def _tiny(tmp_path, blocks=None):
    wl = synth.workload("tiny")
    shapes = list(wl.blocks) if blocks is None else [wl.blocks[b] for b in blocks]
    W = [synth.block_weights(wl.wid, b, OL.block_numel(s)) for b, s in enumerate(shapes)]
    path = str(tmp_path / "tiny.safetensors")
    size = C.write(path, shapes, lambda b: W[b])
    return path, shapes, W, size


def test_round_trip_bitwise(tmp_path):
    path, shapes, W, size = _tiny(tmp_path)
    import os
    assert os.path.getsize(path) == size
    for b in range(len(shapes)):
        assert np.array_equal(C.read_block(path, shapes, b), W[b])


def test_header_follows_the_oracle_parameter_table(tmp_path):
    path, shapes, W, _ = _tiny(tmp_path)
    start, header = C.read_header(path)
    assert start % 8 == 0
    ranges = []
    for b, s in enumerate(shapes):
        for p in OL.param_table(s):
            t = header[f"blocks.{b}.{p.name}"]
            assert t["dtype"] == "BF16"
            assert tuple(t["shape"]) == tuple(p.shape)
            ranges.append(tuple(t["data_offsets"]))
    # dense: the tensors tile the data section with no holes, in layout order
    assert ranges[0][0] == 0
    for (a0, a1), (b0, b1) in zip(ranges, ranges[1:]):
        assert a1 == b0
    assert ranges[-1][1] == 2 * sum(OL.block_numel(s) for s in shapes)


def test_third_party_reader_decodes_the_same_values(tmp_path):
    torch = pytest.importorskip("torch")
    safetensors = pytest.importorskip("safetensors")
    path, shapes, W, _ = _tiny(tmp_path)
    with safetensors.safe_open(path, framework="pt") as f:
        for b, s in enumerate(shapes):
            for p in OL.param_table(s):
                t = f.get_tensor(f"blocks.{b}.{p.name}")
                assert t.dtype == torch.bfloat16 and tuple(t.shape) == tuple(p.shape)
                got = t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)
                want = W[b][p.offset: p.offset + int(np.prod(p.shape))]
                assert np.array_equal(got, want), (b, p.name)


def _rewrite_header(path, mutate):
    start, header = C.read_header(path)
    with open(path, "rb") as f:
        data = f.read()[start:]
    mutate(header)
    raw = json.dumps(header).encode()
    raw += b" " * (-len(raw) % 8)
    with open(path, "wb") as f:
        f.write(struct.pack("<Q", len(raw)) + raw + data)


@pytest.mark.parametrize("mutate,msg", [
    (lambda h: h.pop("blocks.1.W1"), "missing tensor"),
    (lambda h: h["blocks.0.Wo"].update(dtype="F16"), "dtype"),
    (lambda h: h["blocks.2.bo"].update(shape=[3]), "shape"),
    (lambda h: h.update({"blocks.9.Wqkv": h["blocks.0.Wqkv"]}), "not in the block layout"),
    (lambda h: h["__metadata__"].update(format="other"), "metadata format"),
    (lambda h: h["blocks.0.Wo"].update(data_offsets=[h["blocks.0.Wo"]["data_offsets"][0] + 2,
                                                     h["blocks.0.Wo"]["data_offsets"][1] + 2]), "after the previous"),
])
def test_malformed_files_rejected(tmp_path, mutate, msg):
    path, shapes, W, _ = _tiny(tmp_path)
    _rewrite_header(path, mutate)
    with pytest.raises(ValueError, match=msg):
        C.plan(path, shapes)


def test_truncated_file_rejected(tmp_path):
    path, shapes, W, size = _tiny(tmp_path)
    with open(path, "r+b") as f:
        f.truncate(size - 2)
    with pytest.raises(ValueError, match="file has"):
        C.plan(path, shapes)


def test_wrong_block_count_rejected(tmp_path):
    path, shapes, W, _ = _tiny(tmp_path, blocks=[0, 1])
    with pytest.raises(ValueError):
        C.plan(path, shapes + [shapes[0]])
    with pytest.raises(ValueError, match="not in the block layout"):
        C.plan(path, shapes[:1])


def test_host_memory_reports_rss_and_pss():
    """The resident-memory figures the checkpoint test reports: RSS and its
    parts from /proc/self/status, PSS and its parts from smaps_rollup; a new
    anonymous 64 MiB region, once touched, shows up in both anonymous sums."""
    m0 = C.host_memory()
    for k in ("VmRSS", "RssAnon", "RssFile"):
        assert m0[k] > 0
    if "Pss" not in m0:
        pytest.skip("no /proc/self/smaps_rollup on this kernel")
    assert 0 < m0["Pss"] <= m0["VmRSS"]
    buf = np.ones(64 << 20, dtype=np.uint8)
    m1 = C.host_memory()
    assert m1["RssAnon"] - m0["RssAnon"] >= (60 << 20)
    assert m1["Pss_Anon"] - m0["Pss_Anon"] >= (60 << 20)
    del buf
