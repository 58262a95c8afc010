"""Checkpoints of a streamed model as safetensors files, loaded through mmap.

The release page's technique 1 (meta-device initialisation + mmap loading)
keeps the host from holding the model twice: the checkpoint is memory-mapped
instead of read into process memory, and the only anonymous host copy of the
weights is the pinned shards that ``dlo_load_shards`` builds (technique 2).

File format: safetensors -- an 8-byte little-endian header length N, N bytes
of JSON header (padded with spaces to a multiple of 8), then the data.  Every
tensor is named ``blocks.{b}.{param}`` with dtype ``BF16`` and the parameter
shape of the block layout (``block_layout``); the tensors of a block are
stored back to back in layout order, so a block's flat weight is one
contiguous byte range of the file and reaches ``dlo_load_shards`` as a view
of the mapping, without a copy.  Any safetensors reader can open the file.

Host-side marshalling only: no step of the forward runs here.
"""
from __future__ import annotations

import json
import mmap
import os
import struct
from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np

from ._lib import block_layout

FORMAT = "dlo-blocks"


def _tensor_name(b: int, param: str) -> str:
    return f"blocks.{b}.{param}"


def write(path: str, shapes: Sequence, block_fn: Callable[[int], np.ndarray]) -> int:
    """Write the flat bf16 weights ``block_fn(b)`` (uint16 bit patterns, numel_b
    elements each) of every block to ``path``.  Blocks are produced and written
    one at a time.  Returns the file size in bytes."""
    header: Dict[str, dict] = {"__metadata__": {"format": FORMAT, "num_blocks": str(len(shapes))}}
    layouts = [block_layout(s, 1) for s in shapes]
    off = 0
    for b, (numel, _, params) in enumerate(layouts):
        for name, p_off, shape in params:
            n = int(np.prod(shape))
            header[_tensor_name(b, name)] = {"dtype": "BF16", "shape": list(shape),
                                             "data_offsets": [off + 2 * p_off, off + 2 * (p_off + n)]}
        off += 2 * numel
    raw = json.dumps(header, separators=(",", ":")).encode()
    raw += b" " * (-len(raw) % 8)
    with open(path, "wb") as f:
        f.write(struct.pack("<Q", len(raw)))
        f.write(raw)
        for b, (numel, _, _) in enumerate(layouts):
            flat = np.ascontiguousarray(block_fn(b), dtype=np.uint16)
            if flat.size != numel:
                raise ValueError(f"block {b}: {flat.size} elements, layout has {numel}")
            f.write(flat.tobytes())
    return 8 + len(raw) + off


def read_header(path: str) -> Tuple[int, dict]:
    """(data start offset, header dict) of a safetensors file."""
    with open(path, "rb") as f:
        head = f.read(8)
        if len(head) != 8:
            raise ValueError("not a safetensors file: shorter than 8 bytes")
        (n,) = struct.unpack("<Q", head)
        size = os.fstat(f.fileno()).st_size
        if n > size - 8:
            raise ValueError(f"header length {n} beyond the file ({size} bytes)")
        return 8 + n, json.loads(f.read(n))


def plan(path: str, shapes: Sequence) -> List[Tuple[int, int]]:
    """Validate the file against the block shapes and return, per block, the
    (byte offset in the file, numel) of its flat weight.  Raises ValueError on
    a missing, extra, misnamed, mistyped, misshaped or non-contiguous tensor,
    or a file too short for its data."""
    start, header = read_header(path)
    size = os.path.getsize(path)
    meta = header.get("__metadata__", {})
    tensors = {k: v for k, v in header.items() if k != "__metadata__"}
    if meta.get("format") != FORMAT:
        raise ValueError(f"metadata format {meta.get('format')!r}, expected {FORMAT!r}")
    out = []
    seen = 0
    for b, s in enumerate(shapes):
        numel, _, params = block_layout(s, 1)
        first = None
        cursor = None
        for name, p_off, shape in params:
            key = _tensor_name(b, name)
            t = tensors.get(key)
            if t is None:
                raise ValueError(f"missing tensor {key}")
            seen += 1
            if t.get("dtype") != "BF16":
                raise ValueError(f"{key}: dtype {t.get('dtype')}, expected BF16")
            if tuple(t.get("shape", ())) != tuple(shape):
                raise ValueError(f"{key}: shape {t.get('shape')}, expected {list(shape)}")
            lo, hi = t["data_offsets"]
            n = int(np.prod(shape))
            if hi - lo != 2 * n:
                raise ValueError(f"{key}: {hi - lo} bytes for {n} elements")
            if first is None:
                first = lo
            elif lo != cursor:
                raise ValueError(f"{key}: not stored right after the previous parameter of block {b}")
            if lo - first != 2 * p_off:
                raise ValueError(f"{key}: at byte {lo - first} of the block, layout offset {2 * p_off}")
            cursor = hi
        if start + cursor > size:
            raise ValueError(f"block {b}: data ends at {start + cursor}, file has {size} bytes")
        if (start + first) % 2:
            raise ValueError(f"block {b}: data not 2-byte aligned")
        out.append((start + first, numel))
    if seen != len(tensors):
        extra = sorted(set(tensors) - {_tensor_name(b, p[0]) for b, s in enumerate(shapes)
                                       for p in block_layout(s, 1)[2]})
        raise ValueError(f"tensors not in the block layout: {extra[:5]}")
    return out


def load(ctx, path: str) -> Dict[str, int]:
    """Shard and pin every block of ``ctx`` (a StreamedDiT) straight from the
    memory-mapped file.  The mapping is closed before returning."""
    ranges = plan(path, ctx.shapes)
    with open(path, "rb") as f:
        mm = mmap.mmap(f.fileno(), 0, access=mmap.ACCESS_READ)
    buf = np.frombuffer(mm, dtype=np.uint8)
    try:
        for b, (off, numel) in enumerate(ranges):
            ctx.load_shards(b, buf[off: off + 2 * numel].view(np.uint16))
    finally:
        buf = None  # drop the exported view before closing the mapping
        mm.close()
    return {"blocks": len(ranges), "bytes": sum(2 * n for _, n in ranges)}


def read_block(path: str, shapes: Sequence, b: int) -> np.ndarray:
    """Copy of block b's flat weight (uint16 bit patterns) from the file."""
    off, numel = plan(path, shapes)[b]
    with open(path, "rb") as f:
        f.seek(off)
        return np.frombuffer(f.read(2 * numel), dtype=np.uint16).copy()


def host_memory() -> Dict[str, int]:
    """This process's resident memory in bytes (Linux /proc): RSS, its
    anonymous and file-backed parts and the peak RSS, and the proportional
    set size (PSS: each shared page divided among the processes mapping it,
    so a checkpoint's page cache mapped by several processes is counted
    once overall) with its anonymous and file-backed parts, where the kernel
    provides smaps_rollup."""
    out = {}
    with open("/proc/self/status") as f:
        for line in f:
            k, _, v = line.partition(":")
            if k in ("VmRSS", "RssAnon", "RssFile", "RssShmem", "VmHWM"):
                out[k] = int(v.split()[0]) * 1024
    try:
        with open("/proc/self/smaps_rollup") as f:
            for line in f:
                k, _, v = line.partition(":")
                if k in ("Pss", "Pss_Anon", "Pss_File"):
                    out[k] = int(v.split()[0]) * 1024
    except OSError:
        pass
    return out


def reset_peak_rss() -> bool:
    """Reset VmHWM to the current RSS (Linux clear_refs); False if refused."""
    try:
        with open("/proc/self/clear_refs", "w") as f:
            f.write("5")
        return True
    except OSError:
        return False
