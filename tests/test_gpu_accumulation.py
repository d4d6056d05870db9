"""Accumulation witnesses for every linear path (TensorFold issue #1491, "Validation": stress cases
that tell fp32 accumulation from reduced precision).

Every weight of the edited linear is exactly 1 or 1 + d and every input is 1, so row n's product
is y_n = K + c_n d, with c_n the row's count of (1 + d) weights:
- MLX affine rows: codes in {0, 1}, scale 2^-10 and bias 1 in every group (d = 2^-10);
- bf16 rows: values 1 and 1 + 2^-7 (d = 2^-7, the smallest step above 1 in bf16);
- NVFP4 rows: e2m1 codes 1.0 and 1.5, e4m3 block scale 1.0, tensor scale 1.0 (d = 0.5).
Each such weight is exact in its storage, in the decode GEMV's exact form and in an fp16 operand,
every product with 1 is exact, and every partial sum of any order is a multiple of d below 2^14,
exact in fp32: an fp32 accumulator returns y_n bit for bit. fp16 and bf16 accumulators cannot
(their unit at 2048 is 2 and 16; tests/test_accumulation_witness.py shows on the CPU that they miss
y_n by at least two units of d in sequential and pairwise order). The tests require the exact value from
the decode GEMV (1-8 rows), the prefill GEMM (its fp16 copy and its in-loop dequantisation) and the
decode MFMA GEMM (3-64 rows) on real layer shapes (K = 2048 and 7680).
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Blob

pytestmark = pytest.mark.gpu


def _bf16_bits(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _put(out, b, name, arr):
    dt, shape, off, nb = b.entries[name]
    raw = np.ascontiguousarray(arr).tobytes()
    assert len(raw) == nb, (name, len(raw), nb)
    out[off:off + nb] = raw


def witness_affine(cfg, blob, names, seed):
    """A copy of the blob whose affine linears `names` hold the 1 / 1 + 2^-10 rows; returns the blob
    and, per name, (K, d, counts)."""
    b = Blob(blob)
    out = bytearray(blob)
    rng = np.random.default_rng(seed)
    meta = {}
    bits, group = cfg["bits"], cfg["group"]
    for name in names:
        shape = b.entries[name + ".q"][1]
        n, k = shape[0], shape[1] * 8 // bits
        q = (rng.random((n, k)) < 0.3).astype(np.uint8)
        _put(out, b, name + ".q", synth.pack_codes(q, bits))
        _put(out, b, name + ".scales", np.full((n, k // group), _bf16_bits(2.0 ** -10), dtype=np.uint16))
        _put(out, b, name + ".biases", np.full((n, k // group), _bf16_bits(1.0), dtype=np.uint16))
        meta[name] = (k, 2.0 ** -10, q.sum(axis=1))
    return bytes(out), meta


def witness_formats(blob, bf16_names, nvfp4_names, seed):
    b = Blob(blob)
    out = bytearray(blob)
    rng = np.random.default_rng(seed)
    meta = {}
    for name in bf16_names:
        n, k = b.entries[name + ".weight"][1]
        sel = rng.random((n, k)) < 0.3
        w = np.where(sel, 1.0 + 2.0 ** -7, 1.0).astype(np.float32)
        _put(out, b, name + ".weight", _bf16_bits(w))
        meta[name] = (k, 2.0 ** -7, sel.sum(axis=1))
    for name in nvfp4_names:
        n, kh = b.entries[name + ".fp4"][1]
        k = 2 * kh
        sel = rng.random((n, k)) < 0.3
        codes = np.where(sel, 3, 2).astype(np.uint8)          # e2m1: 0b0010 = 1.0, 0b0011 = 1.5
        _put(out, b, name + ".fp4", (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
        _put(out, b, name + ".block_scales", np.full((n, k // 16), 0x38, dtype=np.uint8))   # e4m3 1.0
        _put(out, b, name + ".tensor_scale", np.array([1.0], dtype=np.float32))
        meta[name] = (k, 0.5, sel.sum(axis=1))
    return bytes(out), meta


def _expected(k, d, counts):
    return (np.float64(k) + counts.astype(np.float64) * d).astype(np.float32)


def _run_paths(eng, torch, meta, paths):
    for name, (k, d, counts) in meta.items():
        want = _expected(k, d, counts)
        for path, rows_list in paths:
            for rows in rows_list:
                x = torch.ones((rows, k), dtype=torch.float16, device="cuda")
                y = eng.linear(name, x, path)
                torch.cuda.synchronize()
                got = y.cpu().numpy()
                assert got.dtype == np.float32
                bad = np.argwhere(got != want[None, :])
                assert bad.size == 0, (name, path, rows, bad[:4].tolist(),
                                       [float(got[r, c]) - float(want[c]) for r, c in bad[:4]])
        print(f"{name}: exact on paths {[p for p, _ in paths]}", flush=True)


AFFINE_NAMES = ["layers.0.conv.in_proj", "layers.1.attn.qkvg_proj", "layers.2.attn.o_proj", "layers.2.ffn.w2"]


@pytest.mark.parametrize("bits", [4, 6])
def test_affine_paths_accumulate_exactly(bits):
    import torch
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.slice3_config(bits=bits, group=64, max_slots=1, max_chunk=512)
    blob, meta = witness_affine(cfg, synth.cached_blob(cfg, seed=0), AFFINE_NAMES, seed=bits)
    eng = Engine(cfg, blob)
    try:
        # GEMV (1-8 rows), prefill GEMM (fp16 copy at 6 bits, in-loop at 4), in-loop GEMM, decode MFMA
        _run_paths(eng, torch, meta, [(0, (1, 2, 5)), (1, (1, 77, 300)), (6, (7,)), (4, (3, 8, 40))])
    finally:
        eng.close()


def test_bf16_and_nvfp4_paths_accumulate_exactly():
    import torch
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.make_config(layer_types=[0, 2, 1], bits=16, group=0, embed_bits=16, embed_group=0,
                            ffn_format=synth.FFN_NVFP4, max_slots=8, max_ctx=1024, max_chunk=512)
    cfg["vocab"] = 1024
    blob, meta = witness_formats(synth.cached_blob(cfg, seed=0), ["layers.2.attn.o_proj", "layers.0.conv.in_proj"],
                                 ["layers.2.ffn.w2"], seed=11)
    eng = Engine(cfg, blob)
    try:
        _run_paths(eng, torch, meta, [(0, (1, 2)), (1, (1, 130)), (4, (3, 8))])
    finally:
        eng.close()
