"""Pins of the float64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it checks. None of them retypes the oracle's formula: they use hand
packed bits, closed forms, invariants, brute force on tiny inputs, library routines for special
cases, and the header totals printed by the pages.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from attention_decoder_amd import synth
from oracle import ref

# ----------------------------------------------------------------------------------------------
# dequantisation ("TensorFold #1491", Checkpoint handling: MLX affine groups)
# ----------------------------------------------------------------------------------------------


def _pack_by_hand(codes_row, bits):
    """Bitstream by integer arithmetic: code k occupies bits [k*bits, (k+1)*bits), LSB first."""
    acc = 0
    for k, c in enumerate(codes_row):
        acc |= int(c) << (k * bits)
    nbytes = len(codes_row) * bits // 8
    return np.frombuffer(acc.to_bytes(nbytes, "little"), dtype=np.uint8)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_unpack_matches_hand_packed_bits(bits):
    rng = np.random.default_rng(bits)
    k = 128
    codes = rng.integers(0, 2 ** bits, size=(3, k))
    packed = np.stack([_pack_by_hand(r, bits) for r in codes])
    assert np.array_equal(ref.unpack_codes(packed, bits, k), codes)
    # the input generator's packer writes the same bitstream
    assert np.array_equal(synth.pack_codes(codes.astype(np.uint8), bits), packed)


def test_dequant_hand_values():
    # one row, two groups of 4: codes 0..7, scale/bias chosen as exact binary fractions
    codes = np.arange(8)[None, :]
    s = np.array([[0.5, 0.25]])
    b = np.array([[-1.0, 2.0]])
    w = ref.dequant(codes, s, b, 4)
    assert w.tolist() == [[-1.0, -0.5, 0.0, 0.5, 3.0, 3.25, 3.5, 3.75]]


def test_dequant_is_exact_in_fp32(slice3):
    """q*scale+bias of every stored weight is exactly representable in fp32 (the GPU's type)."""
    cfg, blob = slice3
    b = ref.Blob(blob)
    for name in ["layers.0.conv.in_proj", "layers.1.attn.qkvg_proj", "layers.2.ffn.w2"]:
        w = ref.load_linear(b, name, cfg["bits"], cfg["group"], row_chunk=512)
        assert np.array_equal(w.astype(np.float32).astype(np.float64), w)
        # and codes span the full 4-bit range
        _, shp, qb = b.raw(name + ".q")
        q = ref.unpack_codes(qb.reshape(shp)[:64], cfg["bits"], shp[1] * 2)
        assert q.min() == 0 and q.max() == 15


# ----------------------------------------------------------------------------------------------
# geometry: the header totals ("TensorFold PR #1508", NVFP4 admission commit)
# ----------------------------------------------------------------------------------------------


def _geometry():
    H, F, V, D, HQ, HKV = 2048, 7680, 128000, 128, 16, 4
    n_conv, n_attn = 13, 11
    conv_lin = [(3 * H, H), (H, H)]
    attn_lin = [(HQ * D, H), (HKV * D, H), (HKV * D, H), (HQ, H), (H, HQ * D)]
    ffn_lin = [(F, H), (F, H), (H, F)]
    extras_bf16 = n_conv * H * 7 + 24 * 4 * H + n_attn * 2 * D + H
    return H, V, n_conv, n_attn, conv_lin, attn_lin, ffn_lin, extras_bf16


def _golden_totals():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "header_totals.json")) as f:
        return json.load(f)


def test_mlx_q4_header_totals():
    """594 tensors / 973,008,384 B for the MLX 4-bit export follow from the geometry."""
    want = _golden_totals()["mlx_q4_g64"]
    H, V, n_conv, n_attn, conv_lin, attn_lin, ffn_lin, extras = _geometry()
    lins = n_conv * conv_lin + n_attn * attn_lin + 24 * ffn_lin + [(V, H)]
    qbytes = sum(n * k // 2 + 2 * 2 * n * (k // 64) for n, k in lins)
    assert qbytes + 2 * extras == want["bytes"]
    n_tensors = n_conv * (3 * 2 + 1 + 4 + 9) + n_attn * (3 * 5 + 2 + 4 + 9) + 3 + 1
    assert n_tensors == want["tensors"]


def test_nvfp4_header_totals():
    """502 tensors / 1,829,689,408 B for the NVFP4 export (FFN fp4 g16 + e4m3 scales)."""
    want = _golden_totals()["nvfp4"]
    H, V, n_conv, n_attn, conv_lin, attn_lin, ffn_lin, extras = _geometry()
    ffn = 24 * ffn_lin
    fp4 = sum(n * k // 2 + n * k // 16 + 4 + 4 for n, k in ffn)
    bf16 = 2 * sum(n * k for n, k in n_conv * conv_lin + n_attn * attn_lin + [(V, H)])
    assert fp4 + bf16 + 2 * extras == want["bytes"]
    assert 72 * 4 + n_conv * 7 + n_attn * 11 + 2 == want["tensors"]


def test_blob_plan_matches_header_total():
    """Our fused blob stores exactly the MLX 4-bit data bytes (fusing moves no byte)."""
    cfg = synth.full_config(bits=4, group=64)
    total = 0
    for name, kind, shape, bits, group in synth.tensor_plan(cfg):
        if kind == "lin":
            n, k = shape
            total += n * k * bits // 8 + 2 * 2 * n * (k // group)
        else:
            total += 2 * int(np.prod(shape))
    assert total == 973_008_384
    types = synth.default_layer_types()
    assert types.count(0) == 13 and types.count(1) == 6 and types.count(2) == 5


def test_slice_blob_entries(slice3):
    cfg, blob = slice3
    b = ref.Blob(blob)
    assert b.entries["layers.1.attn.qkvg_proj.q"][1] == (3088, 1024)
    assert b.entries["layers.0.conv.kernel"][1] == (2048, 7)
    assert "embedding.q" not in b.entries and "embedding_norm" in b.entries


# ----------------------------------------------------------------------------------------------
# RMSNorm, gate, SwiGLU ("LFM3-1.7B port", comparison table)
# ----------------------------------------------------------------------------------------------


def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0]])                 # mean square 12.5
    y = ref.rmsnorm(x, np.ones(2), 0.0)
    assert np.allclose(y, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=0, atol=1e-15)
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 2048)) * 7
    out = ref.rmsnorm(z, np.ones(2048), 1e-5)
    rms = np.sqrt((out ** 2).mean(axis=1))
    ms = (z ** 2).mean(axis=1)
    assert np.allclose(rms, np.sqrt(ms / (ms + 1e-5)), rtol=1e-13)
    # scale invariance up to eps, and weight multiplies per channel
    w = rng.standard_normal(2048)
    assert np.allclose(ref.rmsnorm(z * 1e3, w, 0.0), ref.rmsnorm(z, w, 0.0), rtol=1e-12)
    assert np.allclose(ref.sigmoid(np.zeros(3)), 0.5)
    assert ref.silu(np.array([0.0]))[0] == 0.0
    assert abs(ref.silu(np.array([50.0]))[0] - 50.0) < 1e-15


# ----------------------------------------------------------------------------------------------
# RoPE ("LFM3-1.7B port", "partial_rotary_factor" section and table row 3)
# ----------------------------------------------------------------------------------------------


def _pair_angles(theta, pairs, p):
    """Recover each pair's rotation angle by rotating unit vectors e_i (i < 64)."""
    d = 128
    out = []
    for i in range(64):
        x = np.zeros((1, 1, d))
        x[0, 0, i] = 1.0
        y = ref.rope_apply(x, ref.rope_angles(np.array([p]), theta, pairs, d))[0, 0]
        # e_i rotates inside the (i, i+64) plane only
        rest = np.delete(y, [i, i + 64])
        assert np.all(rest == 0.0)
        out.append(math.atan2(y[i + 64], y[i]))
    return np.array(out)


def test_rope_full_layers_partial():
    a = _pair_angles(1e6, 32, 1)
    # the page: first 32 entries theta^(-2i/128), the last 32 are zero
    assert abs(a[0] - 1.0) < 1e-15
    assert abs(a[1] - 1e6 ** (-1 / 64)) < 1e-14         # exponent over 128, not over 64
    assert np.all(a[32:] == 0.0)
    ratios = a[1:32] / a[:31]
    assert np.allclose(ratios, ratios[0], rtol=1e-12)
    # dims 32..63 and 96..127 pass through at any position
    x = np.random.default_rng(1).standard_normal((6, 4, 128))
    pos = np.array([0, 1, 7, 255, 256, 32767])
    y = ref.rope_apply(x, ref.rope_angles(pos, 1e6, 32, 128))
    assert np.array_equal(y[..., 32:64], x[..., 32:64])
    assert np.array_equal(y[..., 96:], x[..., 96:])
    assert not np.allclose(y[1:, :, :32], x[1:, :, :32])


def test_rope_sliding_layers_full():
    a = _pair_angles(1e4, 64, 1)
    assert abs(a[0] - 1.0) < 1e-15
    assert abs(a[63] - 1e4 ** (-126 / 128)) < 1e-15
    assert np.all(a != 0.0)


@pytest.mark.parametrize("theta,pairs", [(1e6, 32), (1e4, 64)])
def test_rope_invariants(theta, pairs):
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 128))
    k = rng.standard_normal((1, 2, 128))
    # identity at p = 0
    assert np.array_equal(ref.rope_apply(q, ref.rope_angles(np.array([0]), theta, pairs, 128)), q)
    # each (i, i+64) pair's norm is preserved at any position
    for p in [1, 7, 255, 256, 32767]:
        y = ref.rope_apply(q, ref.rope_angles(np.array([p]), theta, pairs, 128))
        n0 = q[..., :64] ** 2 + q[..., 64:] ** 2
        n1 = y[..., :64] ** 2 + y[..., 64:] ** 2
        assert np.allclose(n0, n1, rtol=1e-12)

    # q(p) . k(p') depends only on p - p'
    def dot(p, pp):
        qa = ref.rope_apply(q, ref.rope_angles(np.array([p]), theta, pairs, 128))
        ka = ref.rope_apply(k, ref.rope_angles(np.array([pp]), theta, pairs, 128))
        return (qa * ka).sum(axis=-1)
    assert np.allclose(dot(10, 3), dot(1007, 1000), rtol=1e-9, atol=1e-12)
    assert np.allclose(dot(300, 44), dot(256, 0), rtol=1e-9, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# short conv and its state ("LFM3-1.7B port", table row 1 and "--pad-tail")
# ----------------------------------------------------------------------------------------------


def test_conv_matches_direct_convolution():
    rng = np.random.default_rng(3)
    c, t = 5, 40
    z = rng.standard_normal((t, c))
    ker = rng.standard_normal((c, 7))
    state = np.zeros((6, c))
    ys = []
    for r in range(t):
        y, state = ref.conv_step(state, z[r], ker)
        ys.append(y)
    ys = np.array(ys)
    for ch in range(c):
        # library 1-D convolution of the zero-padded sequence; K[:, 6] meets the current row
        full = np.convolve(z[:, ch], ker[ch, ::-1], mode="full")[:t]
        assert np.allclose(ys[:, ch], full, rtol=1e-12, atol=1e-13)
    # the state is the last 6 z rows
    assert np.array_equal(state, z[-6:])


@pytest.mark.parametrize("n", [1, 5, 6, 7])
def test_conv_state_partial_chunk_rule(n):
    """After a chunk of n real rows, the state is columns [n, n+6) of [state | z]."""
    rng = np.random.default_rng(4 + n)
    c = 3
    state0 = rng.standard_normal((6, c))
    z = rng.standard_normal((n, c))
    ker = rng.standard_normal((c, 7))
    st = state0
    for r in range(n):
        _, st = ref.conv_step(st, z[r], ker)
    cat = np.concatenate([state0, z], axis=0)
    assert np.array_equal(st, cat[n:n + 6])


# ----------------------------------------------------------------------------------------------
# attention: GQA and the sliding window ("LFM3-1.7B port", window section; PR #1508)
# ----------------------------------------------------------------------------------------------


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(5)
    t, d = 20, 128
    q = rng.standard_normal((t, 16, d))
    k = rng.standard_normal((t, 4, d))
    v = rng.standard_normal((t, 4, d))
    pos = np.arange(t)
    out = ref.attention_rows(q, k, v, pos, None)
    for h in range(16):
        kv = h // 4
        for p in range(t):
            s = q[p, h] @ k[: p + 1, kv].T / math.sqrt(d)
            ref_o = sp_softmax(s) @ v[: p + 1, kv]
            assert np.allclose(out[p, h], ref_o, rtol=1e-12, atol=1e-13)


def _brute_sliding(q, k, v, p, window):
    """Per-key loop with the page's rule: key j visible iff 0 <= p - j < window."""
    d = q.shape[-1]
    num = np.zeros(d)
    den = 0.0
    scores = {}
    for j in range(k.shape[0]):
        if 0 <= p - j < window:
            scores[j] = float(q @ k[j]) / math.sqrt(d)
    mx = max(scores.values())
    for j, s in scores.items():
        e = math.exp(s - mx)
        num += e * v[j]
        den += e
    return num / den, sorted(scores)


def test_sliding_window_seams():
    rng = np.random.default_rng(6)
    t = 600
    q = rng.standard_normal((t, 4, 128))
    k = rng.standard_normal((t, 1, 128))
    v = rng.standard_normal((t, 1, 128))
    pos = np.arange(t)
    out = ref.attention_rows(q, k, v, pos, 256)
    for p in [0, 1, 255, 256, 257, 511, 599]:
        for h in range(4):
            o, keys = _brute_sliding(q[p, h], k[:, 0], v[:, 0], p, 256)
            assert np.allclose(out[p, h], o, rtol=1e-12, atol=1e-13)
        if p == 255:
            assert keys == list(range(0, 256))
        if p == 256:
            assert keys[0] == 1 and len(keys) == 256
        if p == 257:
            assert keys[0] == 2
    # perturbing key 0 leaves p = 256 unchanged and moves p = 255
    k2 = k.copy()
    v2 = v.copy()
    k2[0] += 3.0
    v2[0] += 3.0
    out2 = ref.attention_rows(q, k2, v2, pos, 256)
    assert np.array_equal(out2[256:], out[256:])
    assert not np.allclose(out2[255], out[255])


def test_window_beyond_context_equals_causal():
    rng = np.random.default_rng(7)
    t = 200
    q = rng.standard_normal((t, 4, 128))
    k = rng.standard_normal((t, 1, 128))
    v = rng.standard_normal((t, 1, 128))
    pos = np.arange(t)
    assert np.array_equal(ref.attention_rows(q, k, v, pos, 256), ref.attention_rows(q, k, v, pos, None))


# ----------------------------------------------------------------------------------------------
# greedy argmax convention ("TensorFold PR #1508": ties to the lower id, NaN ranked as -inf)
# ----------------------------------------------------------------------------------------------


def test_argmax_ties_and_nan():
    x = np.array([[1.0, 3.0, 3.0, np.nan], [np.nan, np.nan, -5.0, -5.0]])
    assert ref.greedy_argmax(x).tolist() == [1, 2]


def test_f16_round_properties():
    # exact on fp16 values, ties to even, 11 significant bits
    assert ref.f16_round(np.array([1.0 + 2 ** -10]))[0] == 1.0 + 2 ** -10
    assert ref.f16_round(np.array([1.0 + 2 ** -11]))[0] == 1.0            # tie -> even
    assert ref.f16_round(np.array([1.0 + 3 * 2 ** -11]))[0] == 1.0 + 2 ** -9  # tie -> even (up)
    assert ref.f16_round(np.array([2049.0]))[0] == 2048.0


def test_bf16_round_matches_storage_rounding():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(10000).astype(np.float32)
    via_bits = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(ref.bf16_round(x.astype(np.float64)), via_bits)


# ----------------------------------------------------------------------------------------------
# NVFP4 and block-FP8 weights ("TensorFold PR #1508": the FFN as e2m1 codes in groups of 16 with
# e4m3 block scales and an fp32 tensor scale; block-FP8 linears)
# ----------------------------------------------------------------------------------------------


def test_e4m3_matches_torch_float8_for_every_byte():
    """The oracle's E4M3 decoder against torch's float8_e4m3fn, an independent implementation."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ref.e4m3_values(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert ref.e4m3_values(np.array([0x7E]))[0] == 448.0          # the largest finite value
    assert ref.e4m3_values(np.array([0x01]))[0] == 2.0 ** -9      # the smallest subnormal


def test_e2m1_through_e4m3():
    """E2M1 (exponent bias 1) embeds in E4M3 (bias 7): a normal code (s, e, m) is the E4M3 byte with
    exponent e + 6 and mantissa m << 2; the subnormal 0.5 is exponent 6, mantissa 0. torch's E4M3
    decoder then gives every E2M1 value; they are the 8 magnitudes 0 .. 6 and their negatives."""
    import torch
    codes = np.arange(16)
    s, e, m = codes >> 3, (codes >> 1) & 3, codes & 1
    byte = np.where(e > 0, (s << 7) | ((e + 6) << 3) | (m << 2),
                    np.where(m == 1, (s << 7) | (6 << 3), s << 7)).astype(np.uint8)
    want = torch.from_numpy(byte).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ref.e2m1_values(codes), want)
    assert sorted(set(np.abs(want))) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_nvfp4_dequant_hand_packed():
    """Two rows of 32 codes: element 2i in a byte's low nibble, one e4m3 scale per 16 k, the
    tensor scale on everything."""
    packed = np.zeros((2, 16), dtype=np.uint8)
    packed[0, 0] = 0x2A          # k0: code 0xA = -1.0, k1: code 0x2 = +1.0
    packed[0, 7] = 0xF1          # k14: 0x1 = 0.5, k15: 0xF = -6.0
    packed[0, 8] = 0x07          # k16: 0x7 = 6.0 (next group), k17: 0
    packed[1, 15] = 0x5B         # k30: 0xB = -1.5, k31: 0x5 = 3.0
    scales = np.array([[0x38, 0x40], [0x30, 0x48]], dtype=np.uint8)   # 1.0, 2.0 / 0.5, 4.0
    w = ref.dequant_nvfp4(packed, scales, 0.25)
    want = np.zeros((2, 32))
    want[0, [0, 1, 14, 15]] = np.array([-1.0, 1.0, 0.5, -6.0]) * 1.0 * 0.25
    want[0, 16] = 6.0 * 2.0 * 0.25
    want[1, [30, 31]] = np.array([-1.5, 3.0]) * 4.0 * 0.25
    assert np.array_equal(w, want)


def test_fp8_block_dequant_boundaries():
    """One scale per 128 x 128 block: the scales change exactly at row 128 and at column 128."""
    codes = np.full((130, 260), 0x38, dtype=np.uint8)        # every code 1.0
    sc = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    w = ref.dequant_fp8_block(codes, sc)
    assert w[127, 127] == 1.0 and w[127, 128] == 2.0 and w[128, 127] == 4.0 and w[129, 259] == 6.0
    assert w[0, 256] == 3.0
