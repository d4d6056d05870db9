"""Structural pins of the oracle's layer composition (CPU only).

The sandwich-norm order of every layer ("LFM3-1.7B port", comparison table, the row for the norms:
operator_norm -> mixer -> post_operator_norm -> + residual -> ffn_norm -> SwiGLU FFN ->
post_ffn_norm -> + residual; RMSNorm eps 1e-5) fixes exact consequences that do not depend on any
other implementation. Each is checked on the seeded three-layer slice (conv, sliding, full) by
editing stored tensors of the blob:

- zeroing a layer's operator_norm weight zeroes the mixer's input, so the mixer adds nothing: the
  output equals that of zeroing its post_operator_norm weight, bit for bit (likewise ffn_norm and
  post_ffn_norm for the FFN);
- with eps set to 0 every RMSNorm is exactly invariant to a power-of-2 scale of its input (the
  scale passes exactly through squares, mean, sqrt and division), so:
  - scaling a mixer's or FFN's output projection by 2 (scales and biases, exact in bf16) leaves
    the output bit for bit unchanged, because the post-norm removes the scale;
  - scaling a conv layer's operator_norm weight by 2 scales u, hence B, C and x, the kept state by
    4 and the mixer's output by 8 before the post-norm: unchanged bit for bit; the same scale on
    ffn_norm moves the output (silu is not homogeneous);
  - zeroing the gate rows of qkvg makes every head's gate sigmoid(0) = 1/2, one common factor
    before o_proj that the post-norm removes: the output equals the no-gate control's bit for bit;
- zeroing the conv layer's C rows of in_proj zeroes C * y, so the conv mixer adds nothing;
- zeroing embedding_norm zeroes the final rows and the logits.

A composition mistake -- dropping post_operator_norm, applying it after the residual add, or using
ffn_norm where operator_norm belongs -- breaks at least one of these.
"""
import zlib

import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Blob, Oracle


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def edit(blob: bytes, name: str, fn, rows=None) -> bytes:
    """A copy of the blob with bf16 tensor `name` replaced by fn(values) (rows: a row slice of a 2-D
    tensor)."""
    b = Blob(blob)
    dt, shape, off, nb = b.entries[name]
    assert dt == 1
    vals = b.bf16(name).astype(np.float32)
    new = vals.copy()
    if rows is None:
        new = fn(new)
    else:
        new[rows] = fn(new[rows])
    bits = synth.f32_to_bf16_bits(new.astype(np.float32))
    out = bytearray(blob)
    out[off:off + nb] = bits.tobytes()
    return bytes(out)


def zero(v):
    return np.zeros_like(v)


def times2(v):
    return v * 2


@pytest.fixture(scope="module")
def rows40():
    return synth.bf16_bits_to_f32(synth.hidden_rows(11, 40)).astype(np.float64)


_DEQ = {}


def run(cfg, blob, rows, controls=()):
    """The oracle's final rows; dequantised linears are reused across edited blobs when their
    stored bytes are unchanged (setup only)."""
    orc = Oracle(cfg, blob, controls=controls)
    for name in {k.rsplit(".", 1)[0] for k in orc.blob.entries if k.endswith(".q")}:
        key = (name, zlib.crc32(b"".join(orc.blob.raw(name + sfx)[2].tobytes() for sfx in (".q", ".scales", ".biases"))))
        if key not in _DEQ:
            _DEQ[key] = orc._lin(name)
        orc._w[name] = _DEQ[key]
    return orc.forward(orc.new_slot(), hidden=rows, capture=True)["final"]


def eps0(cfg):
    return dict(cfg, norm_eps=0.0)


@pytest.fixture(scope="module")
def base(slice3, rows40):
    cfg, blob = slice3
    return run(cfg, blob, rows40)


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_zero_operator_norm_equals_zero_post_operator_norm(slice3, rows40, base, layer):
    cfg, blob = slice3
    a = run(cfg, edit(blob, f"layers.{layer}.operator_norm", zero), rows40)
    b = run(cfg, edit(blob, f"layers.{layer}.post_operator_norm", zero), rows40)
    assert np.array_equal(a, b), layer
    assert _rel(a, base) > 1e-3


@pytest.mark.parametrize("layer", [0, 1, 2])
def test_zero_ffn_norm_equals_zero_post_ffn_norm(slice3, rows40, base, layer):
    cfg, blob = slice3
    a = run(cfg, edit(blob, f"layers.{layer}.ffn_norm", zero), rows40)
    b = run(cfg, edit(blob, f"layers.{layer}.post_ffn_norm", zero), rows40)
    assert np.array_equal(a, b), layer
    assert _rel(a, base) > 1e-3


@pytest.mark.parametrize("name", ["layers.0.conv.out_proj", "layers.1.attn.o_proj", "layers.2.attn.o_proj",
                                  "layers.0.ffn.w2", "layers.2.ffn.w2"])
def test_output_projection_scale_is_removed_by_the_post_norm(slice3, rows40, name):
    cfg, blob = slice3
    b2 = edit(edit(blob, name + ".scales", times2), name + ".biases", times2)
    assert np.array_equal(run(eps0(cfg), b2, rows40), run(eps0(cfg), blob, rows40)), name


def test_operator_norm_scale_on_a_conv_layer_is_removed_and_ffn_norm_scale_is_not(slice3, rows40):
    cfg, blob = slice3
    ref = run(eps0(cfg), blob, rows40)
    assert np.array_equal(run(eps0(cfg), edit(blob, "layers.0.operator_norm", times2), rows40), ref)
    assert _rel(run(eps0(cfg), edit(blob, "layers.0.ffn_norm", times2), rows40), ref) > 1e-2


def test_zero_conv_gate_rows_remove_the_conv_mixer(slice3, rows40):
    cfg, blob = slice3
    H = cfg["hidden"]
    c_rows = slice(H, 2 * H)
    bz = edit(edit(blob, "layers.0.conv.in_proj.scales", zero, c_rows), "layers.0.conv.in_proj.biases", zero, c_rows)
    a = run(cfg, bz, rows40)
    b = run(cfg, edit(blob, "layers.0.post_operator_norm", zero), rows40)
    assert np.array_equal(a, b)


def test_zero_gate_rows_equal_the_no_gate_control(slice3, rows40, base):
    cfg, blob = slice3
    d = cfg["head_dim"]
    g0 = (cfg["n_q_heads"] + 2 * cfg["n_kv_heads"]) * d
    g_rows = slice(g0, g0 + cfg["n_q_heads"])
    bz = blob
    for layer in (1, 2):
        name = f"layers.{layer}.attn.qkvg_proj"
        bz = edit(edit(bz, name + ".scales", zero, g_rows), name + ".biases", zero, g_rows)
    assert np.array_equal(run(eps0(cfg), bz, rows40), run(eps0(cfg), blob, rows40, controls=("no_gate",)))
    assert _rel(run(cfg, bz, rows40), base) > 1e-3


def test_zero_embedding_norm_zeroes_logits():
    cfg = synth.make_config(layer_types=[0, 2, 1], max_slots=1, max_ctx=128, max_chunk=64)
    cfg["vocab"] = 256
    blob = synth.build_blob(cfg, seed=3)
    toks = synth.prompt_tokens(4, 12, vocab=256)
    orc = Oracle(cfg, edit(blob, "embedding_norm", zero))
    out = orc.forward(orc.new_slot(), tokens=toks, logits="all")
    assert np.all(out["final"] == 0.0) and np.all(out["logits"] == 0.0)
    ref = Oracle(cfg, blob).forward(Oracle(cfg, blob).new_slot(), tokens=toks, logits="all")
    assert np.abs(ref["logits"]).max() > 1e-2
