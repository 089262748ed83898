"""Host-side checks of the quantized load cache ("Model-agnostic LLM inference", section
"The quantized load cache"): the library's SHA-256 against hashlib, and the validity gate
(magic + dims + source digest + exact length, plus the payload hash) on cache files this
test writes itself from the format documented in include/qd.h.  No GPU."""
import hashlib
import os
import struct

import numpy as np
import pytest

import int8_weight_only_amd as qd
from workloads import SHAPES


@pytest.mark.parametrize("n", [0, 1, 3, 55, 56, 57, 63, 64, 65, 119, 120, 1000, 100003])
def test_sha256_matches_hashlib(n):
    data = np.random.default_rng(n).integers(0, 256, n, dtype=np.uint8).tobytes()
    assert qd.sha256(data) == hashlib.sha256(data).digest()


def _payload_bytes(s):
    d, L, H, KV, D, I, V = s.hidden, s.n_layers, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.vocab
    nqkv = H * D + 2 * KV * D
    per_layer = (nqkv * d + 4 * nqkv + d * H * D + 4 * d + 2 * I * d + 8 * I + d * I + 4 * d
                 + 4 * d + 4 * d + 4 * D + 4 * D)
    return V * d + 4 * V + 4 * d + L * per_layer


def _payload_digest(payload, chunk=16 << 20):
    """The documented payload digest: SHA-256 of the concatenated SHA-256 digests of the
    payload's consecutive 16 MiB chunks."""
    sums = b"".join(hashlib.sha256(payload[i:i + chunk]).digest()
                    for i in range(0, len(payload), chunk))
    return hashlib.sha256(sums).digest()


def _write(path, s, digest, payload, **over):
    f = dict(magic=b"QDI8WCV1", version=2, header_bytes=128, payload_bytes=len(payload),
             dims=[s.hidden, s.n_layers, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate,
                   s.vocab, struct.unpack("<I", struct.pack("<f", s.rms_eps))[0],
                   struct.unpack("<I", struct.pack("<f", s.rope_theta))[0]],
             src=digest, sha=_payload_digest(payload))
    f.update(over)
    hdr = (f["magic"] + struct.pack("<IIQ", f["version"], f["header_bytes"], f["payload_bytes"])
           + struct.pack("<9I", *f["dims"]) + f["src"] + f["sha"] + b"\0" * 4)
    assert len(hdr) == 128
    with open(path, "wb") as fh:
        fh.write(hdr + payload)


@pytest.fixture
def cache(tmp_path):
    s = SHAPES["tiny"]
    digest = hashlib.sha256(b"manifest of the tiny checkpoint").digest()
    payload = np.random.default_rng(0).integers(0, 256, _payload_bytes(s), dtype=np.uint8).tobytes()
    return s, digest, payload, str(tmp_path / "weights_i8.cache")


def test_gate_accepts_a_well_formed_cache(cache):
    s, digest, payload, path = cache
    _write(path, s, digest, payload)
    qd.check_cache(s, path, digest)


def test_payload_digest_over_several_chunks(tmp_path):
    """A payload of several 16 MiB chunks (a tiny decoder with a 150,000-token vocabulary:
    19.8 MB) passes with the two-level digest and fails if one byte of its second chunk
    changes."""
    import dataclasses
    s = dataclasses.replace(SHAPES["tiny"], vocab=150000)
    digest = hashlib.sha256(b"manifest").digest()
    n = _payload_bytes(s)
    assert n > 16 << 20
    payload = np.random.default_rng(1).integers(0, 256, n, dtype=np.uint8).tobytes()
    path = str(tmp_path / "big.cache")
    _write(path, s, digest, payload)
    qd.check_cache(s, path, digest)
    bad = bytearray(payload)
    bad[(16 << 20) + 5] ^= 1
    _write(path, s, digest, bytes(bad), sha=_payload_digest(payload))
    with pytest.raises(qd.QdError) as e:
        qd.check_cache(s, path, digest)
    assert e.value.code == "cache_miss" and "digest" in str(e.value)


@pytest.mark.parametrize("change,needle", [
    (dict(magic=b"QDI8WCV0"), "magic"),
    (dict(version=1), "format version"),
    (dict(dims=None), "vocab differs"),
    (dict(src=None), "source checkpoint digest"),
    (dict(payload_bytes=None), "payload length"),
    (dict(sha=b"\0" * 32), "payload digest"),
])
def test_gate_names_each_mismatch(cache, change, needle):
    s, digest, payload, path = cache
    if "dims" in change:
        d = [s.hidden, s.n_layers, s.n_heads, s.n_kv_heads, s.head_dim, s.intermediate, s.vocab + 1,
             struct.unpack("<I", struct.pack("<f", s.rms_eps))[0],
             struct.unpack("<I", struct.pack("<f", s.rope_theta))[0]]
        change = dict(dims=d)
    if "src" in change:
        change = dict(src=hashlib.sha256(b"another checkpoint").digest())
    if "payload_bytes" in change:
        change = dict(payload_bytes=len(payload) - 1)
    _write(path, s, digest, payload, **change)
    with pytest.raises(qd.QdError) as e:
        qd.check_cache(s, path, digest)
    assert e.value.code == "cache_miss" and needle in str(e.value), str(e.value)


@pytest.mark.parametrize("edit", ["truncate", "append", "flip"])
def test_gate_refuses_damaged_files(cache, edit):
    s, digest, payload, path = cache
    _write(path, s, digest, payload)
    raw = bytearray(open(path, "rb").read())
    if edit == "truncate":
        raw = raw[:-1]
    elif edit == "append":
        raw += b"\0"
    else:
        raw[128 + len(payload) // 2] ^= 1
    open(path, "wb").write(bytes(raw))
    with pytest.raises(qd.QdError) as e:
        qd.check_cache(s, path, digest)
    assert e.value.code == "cache_miss"


def test_gate_reports_a_missing_file(tmp_path):
    with pytest.raises(qd.QdError) as e:
        qd.check_cache(SHAPES["tiny"], str(tmp_path / "absent.cache"), b"\0" * 32)
    assert e.value.code == "cache_miss"


def test_packed_size_matches_the_pages_cache_sizes():
    # 0.598 GB and 1.724 GB in the section's table
    assert round(_payload_bytes(SHAPES["qwen3-0.6b"]) / 1e9, 3) == 0.598
    assert round(_payload_bytes(SHAPES["qwen3-1.7b"]) / 1e9, 3) == 1.724
