"""The C-ABI library loads, exports what include/lfm3.h declares, and refuses bad configs and bad
blobs on the host before touching a device (TensorFold #1491: names, shapes, dtypes and byte ranges
are checked before any kernel runs). CPU only: no call here reaches a GPU."""
import ctypes
import struct

import numpy as np
import pytest

from attention_decoder_amd import lfm3, synth


def test_library_exports_every_declared_symbol():
    lib = lfm3.load_library()
    names = lfm3.header_symbols()
    assert "lfm3_create" in names and "lfm3_decode_batch" in names
    for n in names:
        assert hasattr(lib, n), n


def test_config_struct_layout_matches_header():
    # 21 int32 + float = 88 bytes, two doubles, 64 layer bytes, then ffn_format
    assert ctypes.sizeof(lfm3.Config) == 88 + 16 + 64 + 4 + 4   # + tail padding to the doubles' alignment
    assert lfm3.Config.rope_theta_full.offset == 88
    assert lfm3.Config.ffn_format.offset == 88 + 16 + 64


def test_query_sizes_full_geometry():
    cfg = synth.full_config(bits=4, group=64, max_slots=1, max_ctx=4096, max_chunk=2048)
    blob_bytes, ws = lfm3.lfm3_query_sizes(lfm3.config_from_dict(cfg))
    # the blob holds exactly the MLX 4-bit data bytes plus table and alignment padding
    assert 973_008_384 < blob_bytes < 973_008_384 + 1_000_000
    assert ws > 0


@pytest.mark.parametrize("field,value,frag", [
    ("bits", 5, "unsupported affine bits 5"),
    ("group", 128, "unsupported affine group 128"),
    ("head_dim", 64, "head_dim 64"),
    ("n_kv_heads", 8, "4 query heads per KV head"),
    ("page_tokens", 512, "page_tokens 512"),
    ("conv_taps", 9, "conv_taps 9"),
])
def test_config_refusals_are_named(field, value, frag):
    cfg = synth.full_config()
    cfg[field] = value
    with pytest.raises(lfm3.LFM3Error) as ei:
        lfm3.lfm3_query_sizes(lfm3.config_from_dict(cfg))
    assert ei.value.status == 2
    assert frag in ei.value.message


@pytest.fixture(scope="module")
def small_blob():
    cfg = synth.slice3_config()
    return cfg, synth.cached_blob(cfg, seed=0)


def test_validate_accepts_seeded_blob(small_blob):
    cfg, blob = small_blob
    st, msg = lfm3.lfm3_validate_blob(lfm3.config_from_dict(cfg), blob)
    assert st == 0, msg
    blob_bytes, _ = lfm3.lfm3_query_sizes(lfm3.config_from_dict(cfg))
    assert blob_bytes == len(blob)


def _corrupt_entry(blob, name, field_off, fmt, value):
    magic, ver, n, tab, dat, total = struct.unpack_from("<8sIIQQQ", blob, 0)
    b = bytearray(blob)
    for i in range(n):
        nm = bytes(b[tab + 128 * i: tab + 128 * i + 80]).rstrip(b"\0").decode()
        if nm == name:
            struct.pack_into(fmt, b, tab + 128 * i + field_off, value)
            return bytes(b)
    raise KeyError(name)


def test_validate_refusals(small_blob):
    cfg, blob = small_blob
    c = lfm3.config_from_dict(cfg)
    bad_magic = b"XXXXXXXX" + blob[8:]
    assert lfm3.lfm3_validate_blob(c, bad_magic)[0] == 3
    st, msg = lfm3.lfm3_validate_blob(c, blob[:-256])
    assert st == 3 and "size" in msg
    st, msg = lfm3.lfm3_validate_blob(c, _corrupt_entry(blob, "layers.0.conv.kernel", 92, "<I", 3))
    assert st == 3 and "layers.0.conv.kernel" in msg
    st, msg = lfm3.lfm3_validate_blob(c, _corrupt_entry(blob, "layers.1.attn.qkvg_proj.q", 80, "<I", 1))
    assert st == 3 and "dtype" in msg
    st, msg = lfm3.lfm3_validate_blob(c, _corrupt_entry(blob, "embedding_norm", 0, "<14s", b"embedding_nope"))
    assert st == 3 and "lacks tensor embedding_norm" in msg
    st, msg = lfm3.lfm3_validate_blob(c, _corrupt_entry(blob, "layers.2.ffn.w2.scales", 104, "<Q", len(blob) - 16))
    assert st == 3 and "past the blob end" in msg
    # a config that disagrees with the blob (8-bit codes) is refused by shape
    cfg8 = dict(cfg, bits=8)
    st, msg = lfm3.lfm3_validate_blob(lfm3.config_from_dict(cfg8), blob)
    assert st == 3


def test_binding_has_no_fallback(tmp_path, monkeypatch):
    monkeypatch.setattr(lfm3, "_lib", None)
    with pytest.raises(OSError):
        lfm3.load_library(str(tmp_path / "missing.so"))


@pytest.mark.parametrize("ffn_format", [1, 2])
def test_nvfp4_and_fp8_layouts_admitted(ffn_format):
    """The NVFP4 export's layout (FFN in fp4 with e4m3 block scales and fp32 tensor / input scales,
    everything else bf16) and the block-FP8 FFN: the host admission accepts the seeded blobs of
    the three-layer slice and names a missing scale."""
    cfg = synth.make_config(layer_types=[0, 2, 1], bits=16, group=0, embed_bits=16, embed_group=0,
                            ffn_format=ffn_format, max_slots=1, max_ctx=128, max_chunk=64)
    cfg["vocab"] = 256
    blob = synth.cached_blob(cfg, seed=0)
    c = lfm3.config_from_dict(cfg)
    assert lfm3.lfm3_query_sizes(c)[0] == len(blob)
    st, msg = lfm3.lfm3_validate_blob(c, blob)
    assert st == 0, msg
    name = "layers.0.ffn.w2.block_scales"
    st, msg = lfm3.lfm3_validate_blob(c, _corrupt_entry(blob, name, 0, "<20s", b"layers.0.ffn.w2.nope"))
    assert st == 3 and "block_scales" in msg


def test_ffn_format_refused_by_name():
    cfg = synth.full_config()
    cfg["ffn_format"] = 3
    with pytest.raises(lfm3.LFM3Error) as ei:
        lfm3.lfm3_query_sizes(lfm3.config_from_dict(cfg))
    assert ei.value.status == 2 and "ffn_format 3" in ei.value.message
