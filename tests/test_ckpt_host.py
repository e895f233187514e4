"""Checkpoint file format on the host: headers written here by hand from the
documented layout must be accepted, and every malformed one rejected, before
any device access."""
import struct

import numpy as np
import pytest

import oracle
import zero_sharded_mixed_grads_amd as z


def write_shard(path, psi, nd, rank, step, master=None, m=None, v=None, magic=b"ZEROCKPT",
                version=1, extra=b"", flags=0):
    b, e = oracle.partition(psi, nd, rank)
    n = e - b
    rng = np.random.default_rng(rank)
    arrs = [a if a is not None else rng.standard_normal(n).astype(np.float32)
            for a in (master, m, v)]
    hdr = struct.pack("<8sIIIIQQQQQ", magic, version, nd, rank, 0, psi, b, e, step, flags)
    assert len(hdr) == 64
    with open(path, "wb") as f:
        f.write(hdr)
        for a in arrs:
            f.write(np.ascontiguousarray(a, np.float32).tobytes())
        f.write(extra)
    return arrs


def _status(fn, *a):
    try:
        fn(*a)
    except z.ZeroError as e:
        return e.status
    return z.ZERO_OK


def test_header_roundtrip(tmp_path):
    p = str(tmp_path / "r1.zck")
    write_shard(p, 1_000_003, 3, 1, 42)
    h = z.zero_ckpt_read_header(p)
    b, e = oracle.partition(1_000_003, 3, 1)
    assert (h.magic, h.version, h.nd, h.rank, h.psi, h.begin, h.end, h.step) == \
        (b"ZEROCKPT", 1, 3, 1, 1_000_003, b, e, 42)


def test_header_rejections(tmp_path):
    p = str(tmp_path / "x.zck")
    write_shard(p, 1000, 3, 1, 1, magic=b"NOTACKPT")
    assert _status(z.zero_ckpt_read_header, p) == z.ZERO_EINVAL
    write_shard(p, 1000, 3, 1, 1, version=2)
    assert _status(z.zero_ckpt_read_header, p) == z.ZERO_EINVAL
    write_shard(p, 1000, 3, 1, 1, extra=b"\0")  # size does not match the range
    assert _status(z.zero_ckpt_read_header, p) == z.ZERO_EIO
    with open(p, "wb") as f:
        f.write(b"short")
    assert _status(z.zero_ckpt_read_header, p) == z.ZERO_EIO
    assert _status(z.zero_ckpt_read_header, str(tmp_path / "missing")) == z.ZERO_EIO
    # a range that is not the partition of (psi, nd, rank)
    hdr = struct.pack("<8sIIIIQQQQQ", b"ZEROCKPT", 1, 3, 1, 0, 1000, 300, 600, 1, 0)
    with open(p, "wb") as f:
        f.write(hdr + bytes(12 * 300))
    assert _status(z.zero_ckpt_read_header, p) == z.ZERO_EINVAL


def test_load_rejects_incomplete_or_mixed_sets(tmp_path):
    psi = 10_007
    paths = [str(tmp_path / f"r{r}.zck") for r in range(4)]
    for r, p in enumerate(paths):
        write_shard(p, psi, 4, r, 5)
    fake = 0x7F0000000000
    args = (psi, 2, 0, fake, fake + (1 << 20), fake + (2 << 20), fake + (3 << 20), 0)
    assert _status(z.zero_ckpt_load, paths[:3], *args) == z.ZERO_EINVAL        # a rank missing
    assert _status(z.zero_ckpt_load, paths + [paths[0]], *args) == z.ZERO_EINVAL  # overlap
    assert _status(z.zero_ckpt_load, paths, psi + 1, *args[1:]) == z.ZERO_EINVAL  # other psi
    write_shard(paths[2], psi, 4, 2, 6)                                        # other save
    assert _status(z.zero_ckpt_load, paths, *args) == z.ZERO_EINVAL
    assert _status(z.zero_ckpt_load, [], *args) == z.ZERO_EINVAL
    assert _status(z.zero_ckpt_load, paths, psi, 0, 0, *args[3:]) == z.ZERO_EINVAL  # nd = 0


def test_loss_scale_record_flag(tmp_path):
    """Flags bit 0 announces a 32-byte loss-scale record after the arrays: the
    file size must include it, and unknown flag bits are rejected."""
    rec = struct.pack("<ddQQ", 1024.0, 1 / 1024.0, 3, 1)
    p = str(tmp_path / "s.zck")
    write_shard(p, 10_000, 2, 0, 7, flags=1, extra=rec)
    h = z.zero_ckpt_read_header(p)
    assert h.flags == 1 and h.step == 7
    write_shard(p, 10_000, 2, 0, 7, flags=1)  # record missing
    assert _status(z.zero_ckpt_read_header, p) == z.ZERO_EIO
    write_shard(p, 10_000, 2, 0, 7, flags=0, extra=rec)  # record not announced
    assert _status(z.zero_ckpt_read_header, p) == z.ZERO_EIO
    write_shard(p, 10_000, 2, 0, 7, flags=2, extra=rec)
    assert _status(z.zero_ckpt_read_header, p) == z.ZERO_EINVAL
