"""Host logic of the expert store (no GPU): one container file of fixed-stride
blobs, each fetched with one positioned read at an offset computed from
(layer, id) (linlog.top article, core design 2, fixed-stride reads; Swiftlet
README translation, "How it works").  The layout checked here is the one
include/moe_layer.h states: a 4096-byte header, then blob (layer, id) at
4096 + (layer * n_experts + id) * stride."""

import struct

import numpy as np
import pytest

import int4_quantized_expert_amd as M
import synth

GEO = synth.PRESETS["tiny"]
L = 3


def _blobs(seed=5):
    out = []
    for l in range(L):
        pool, _ = synth.make_pool(GEO, seed, l)
        out.append(pool.reshape(GEO.n_experts, GEO.blob_stride))
    return out


def _make(path, blobs):
    st = M.ExpertStore.create(str(path), L, GEO.n_experts, GEO.blob_stride, GEO.blob_bytes(GEO.inter))
    for l in range(L):
        for e in range(GEO.n_experts):
            st.write(l, e, blobs[l][e])
    st.close()


def test_store_round_trip_and_file_layout(tmp_path):
    blobs = _blobs()
    path = tmp_path / "s.store"
    _make(path, blobs)
    raw = path.read_bytes()
    stride = GEO.blob_stride
    assert len(raw) == 4096 + L * GEO.n_experts * stride
    magic, nl, ne, st, bb = struct.unpack_from("<8siiqq", raw, 0)
    assert (magic, nl, ne, st, bb) == (b"MOEBLOB1", L, GEO.n_experts, stride, GEO.blob_bytes(GEO.inter))
    assert raw[struct.calcsize("<8siiqq"):4096] == bytes(4096 - struct.calcsize("<8siiqq"))
    s = M.ExpertStore(str(path))
    assert (s.n_layers, s.n_experts, s.stride) == (L, GEO.n_experts, stride)
    buf = np.empty(stride, dtype=np.uint8)
    for l in range(L):
        for e in (0, 7, GEO.n_experts - 1):
            off = 4096 + (l * GEO.n_experts + e) * stride
            assert raw[off:off + stride] == blobs[l][e].tobytes()
            s.read(l, e, buf)
            assert np.array_equal(buf, blobs[l][e])
    s.close()


def test_store_direct_reads_match(tmp_path):
    blobs = _blobs(6)
    path = tmp_path / "d.store"
    _make(path, blobs)
    try:
        s = M.ExpertStore(str(path), direct=True)
    except M.MoeError as err:
        if "Invalid argument" in str(err) or "not supported" in str(err).lower():
            pytest.skip(f"this file system refuses O_DIRECT: {err}")
        raise
    stride = GEO.blob_stride
    # the store reads through its own aligned buffer: any destination works
    big = np.zeros(stride + 4096, dtype=np.uint8)
    a = (-big.ctypes.data) % 4096
    for off in (a, a + 16):
        dst = big[off:off + stride]
        s.read(2, 3, dst)
        assert np.array_equal(dst, blobs[2][3])
    s.close()


def test_store_rejects_bad_files_and_arguments(tmp_path):
    stride = GEO.blob_stride
    with pytest.raises(M.MoeError):
        M.ExpertStore(str(tmp_path / "missing.store"))
    with pytest.raises(M.MoeError):          # stride not a multiple of 4096
        M.ExpertStore.create(str(tmp_path / "a.store"), 1, 4, 4096 + 256, 100)
    with pytest.raises(M.MoeError):          # blob larger than its stride
        M.ExpertStore.create(str(tmp_path / "b.store"), 1, 4, 4096, 4097)
    bad = tmp_path / "bad.store"
    bad.write_bytes(b"NOTASTORE" + bytes(8192))
    with pytest.raises(M.MoeError):
        M.ExpertStore(str(bad))
    # a store whose file ends before its last blob
    path = tmp_path / "short.store"
    _make(path, _blobs())
    with open(path, "r+b") as fh:
        fh.truncate(4096 + (L * GEO.n_experts - 1) * stride)
    with pytest.raises(M.MoeError, match="shorter"):
        M.ExpertStore(str(path))
    # reads outside the store and writes to a read-only store
    path2 = tmp_path / "ok.store"
    _make(path2, _blobs())
    s = M.ExpertStore(str(path2))
    buf = np.empty(stride, dtype=np.uint8)
    for l, e in ((L, 0), (0, GEO.n_experts), (-1, 0)):
        with pytest.raises(M.MoeError):
            s.read(l, e, buf)
    with pytest.raises(M.MoeError, match="read-only"):
        s.write(0, 0, buf)
    s.close()


def test_fresh_store_reads_zeros_until_written(tmp_path):
    stride = GEO.blob_stride
    s = M.ExpertStore.create(str(tmp_path / "z.store"), 2, 4, stride, GEO.blob_bytes(GEO.inter))
    one = np.full(stride, 7, dtype=np.uint8)
    s.write(1, 2, one)
    buf = np.empty(stride, dtype=np.uint8)
    s.read(1, 1, buf)
    assert not buf.any()
    s.read(1, 2, buf)
    assert np.array_equal(buf, one)
    s.close()


def test_cache_from_store_rejects_bad_arguments_before_any_device_call(tmp_path):
    path = tmp_path / "c.store"
    _make(path, _blobs())
    s = M.ExpertStore(str(path))
    L_ = M.lib()
    fake = 1 << 20          # never dereferenced: validation fails first
    assert not L_.moe_cache_create_from_store(8, None, s._h, fake, 4)        # no pool
    assert not L_.moe_cache_create_from_store(8, fake, None, fake, 4)        # no store
    assert not L_.moe_cache_create_from_store(8, fake, s._h, None, 4)        # no staging
    assert not L_.moe_cache_create_from_store(8, fake, s._h, fake, 0)        # no staging buffers
    assert not L_.moe_cache_create_from_store(8, fake, s._h, fake, 65)       # too many
    assert "staging" in L_.moe_cache_last_error().decode()
    s.close()
