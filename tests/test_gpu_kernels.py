"""Kernel-level GPU parity: the decode dequant-GEMV and the prefill dequant MFMA GEMM on
real layer shapes of the seeded three-layer slice, against the float64 oracle's dequantised
weights times the same fp16 rows (MLX affine: w = q * scale + bias per group of 64)."""
import numpy as np
import pytest

from oracle import ref

pytestmark = pytest.mark.gpu

SHAPES = ["layers.0.conv.in_proj", "layers.1.attn.qkvg_proj", "layers.2.ffn.w13", "layers.2.ffn.w2",
          "layers.2.attn.o_proj"]


@pytest.fixture(scope="module")
def eng(slice3):
    from attention_decoder_amd.lfm3 import Engine
    cfg, blob = slice3
    e = Engine(dict(cfg, max_slots=8, max_chunk=2048), blob)
    yield e
    e.close()


@pytest.fixture(scope="module")
def weights(slice3):
    cfg, blob = slice3
    b = ref.Blob(blob)
    return {n: ref.load_linear(b, n, cfg["bits"], cfg["group"]) for n in SHAPES}


def _x(torch, rows, k, seed):
    x = np.random.default_rng(seed).standard_normal((rows, k)).astype(np.float16)
    return x, torch.from_numpy(x).cuda()


@pytest.mark.parametrize("name", SHAPES)
def test_gemv_matches_float64(eng, weights, name):
    import torch
    w = weights[name]
    for rows in (1, 3, 8):
        x, xd = _x(torch, rows, w.shape[1], rows)
        y = eng.linear(name, xd, 0).cpu().numpy().astype(np.float64)
        want = x.astype(np.float64) @ w.T
        err = np.abs(y - want).max() / np.abs(want).max()
        # exact weights and fp16 inputs; the 1024 + q operand form costs ~2^10/q of the fp32
        # accumulation precision (about 3e-5 relative), still far below fp16 input rounding
        assert err < 1e-4, (name, rows, err)


@pytest.mark.parametrize("bits,group", [(8, 64), (6, 64), (4, 32)])
def test_gemv_other_schemes(bits, group):
    """The decode GEMV (exact weights) at 8-bit, 6-bit and 4-bit g32 on the slice's shapes, at 1, 2 and
    5 rows, against the float64 product with the exactly dequantised weights."""
    import torch
    from attention_decoder_amd import synth
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.slice3_config(bits=bits, group=group, max_slots=1, max_chunk=64)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    b = ref.Blob(blob)
    try:
        for name in SHAPES:
            w = ref.load_linear(b, name, bits, group)
            for rows in (1, 2, 5):
                x, xd = _x(torch, rows, w.shape[1], 100 + bits + group + rows)
                y = eng.linear(name, xd, 0).float().cpu().numpy().astype(np.float64)
                want = x.astype(np.float64) @ w.T
                err = np.abs(y - want).max() / np.abs(want).max()
                assert err < 1e-4, (bits, group, name, rows, err)
    finally:
        eng.close()


@pytest.mark.parametrize("name", SHAPES)
def test_gemm_matches_float64(eng, weights, name):
    import torch
    w = weights[name]
    for rows in (1, 77, 300):
        x, xd = _x(torch, rows, w.shape[1], 10 + rows)
        y = eng.linear(name, xd, 1).cpu().numpy().astype(np.float64)
        want_exact = x.astype(np.float64) @ w.T
        want_f16w = x.astype(np.float64) @ ref.f16_round(w).T      # the GEMM's stated rounding point
        assert np.abs(y - want_f16w).max() / np.abs(want_f16w).max() < 2e-5, (name, rows)
        rel = np.linalg.norm(y - want_exact) / np.linalg.norm(want_exact)
        assert rel < 1e-3, (name, rows, rel)


@pytest.mark.parametrize("name,path", [("layers.2.ffn.w13", 1), ("layers.2.ffn.w13", 3), ("layers.0.conv.in_proj", 1)])
def test_gemm_prefill_chunk_sampled_rows(eng, weights, name, path):
    """At a full prefill chunk (1800 rows: 128- or 64-row tiles with a ragged last row tile) every
    sampled output row matches the float64 product with the fp16-rounded weights."""
    import torch
    w = weights[name]
    rows = 1800
    x, xd = _x(torch, rows, w.shape[1], 7)
    y = eng.linear(name, xd, path).float().cpu().numpy().astype(np.float64)
    pick = np.r_[0:8, 250:262, 1790:1800, np.random.default_rng(3).integers(0, rows, 24)]
    xs = x[pick].astype(np.float64)
    if path == 1:
        want = xs @ ref.f16_round(w).T
        assert np.abs(y[pick] - want).max() / np.abs(want).max() < 2e-5, name
    else:
        F = w.shape[0] // 2
        ab = xs @ ref.f16_round(w).T
        g, u = ab[:, :F], ab[:, F:]
        want = g / (1 + np.exp(-g)) * u
        assert np.abs(y[pick] - want).max() / np.abs(want).max() < 2e-3, name


@pytest.mark.parametrize("name,path", [(n, 0) for n in SHAPES] + [("layers.2.ffn.w13", 2)])
def test_gemv_rows_independent_of_batch(eng, weights, name, path):
    """A row's GEMV result does not depend on the other rows of the batch or its position."""
    import torch
    x, xd = _x(torch, 8, weights[name].shape[1], 99)
    solo = [eng.linear(name, xd[i:i + 1].contiguous(), path) for i in range(8)]
    for rows in (2, 3, 4, 8):
        y = eng.linear(name, xd[:rows].contiguous(), path)
        for i in range(rows):
            d = (y[i].float() - solo[i][0].float()).abs().max().item()
            assert d == 0.0, (rows, i, d)


def test_swiglu_epilogues(eng, weights):
    """silu(gate) * up of the fused [w1 | w3] weight, GEMV and GEMM, against float64."""
    import torch
    w = weights["layers.2.ffn.w13"]
    F = w.shape[0] // 2
    for path, rows in ((2, 4), (3, 96)):
        x, xd = _x(torch, rows, w.shape[1], 7 + path)
        y = eng.linear("layers.2.ffn.w13", xd, path).float().cpu().numpy().astype(np.float64)
        ab = x.astype(np.float64) @ w.T
        want = ab[:, :F] / (1 + np.exp(-ab[:, :F])) * ab[:, F:]
        rel = np.linalg.norm(y - want) / np.linalg.norm(want)
        assert rel < 2e-3, (path, rel)


@pytest.mark.parametrize("bits,group", [(8, 64), (6, 64), (4, 32)])
def test_gemm_other_schemes(bits, group):
    """The prefill GEMM (re-tiled weights) at 8-bit, 6-bit and 4-bit g32 on the slice's shapes, at a
    ragged row count: the float64 product with the fp16-rounded dequantised weights (SwiGLU for
    w13)."""
    import torch
    from attention_decoder_amd import synth
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.slice3_config(bits=bits, group=group, max_slots=1, max_chunk=512)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    b = ref.Blob(blob)
    try:
        for name, path in [("layers.0.conv.in_proj", 1), ("layers.0.ffn.w2", 1), ("layers.2.attn.qkvg_proj", 1),
                           ("layers.1.ffn.w13", 3)]:
            w = ref.load_linear(b, name, bits, group)
            x, xd = _x(torch, 300, w.shape[1], bits + group)
            y = eng.linear(name, xd, path).float().cpu().numpy().astype(np.float64)
            ab = x.astype(np.float64) @ ref.f16_round(w).T
            if path == 3:
                F = w.shape[0] // 2
                want = ab[:, :F] / (1 + np.exp(-ab[:, :F])) * ab[:, F:]
                tol = 2e-3
            else:
                want, tol = ab, 2e-5
            err = np.abs(y - want).max() / np.abs(want).max()
            print(f"{bits}-bit g{group} {name}: max rel err {err:.2e}")
            assert err < tol, (bits, group, name, err)
            if path == 1:
                # at 6 bits the GEMM reads the fp16 operand copy: it holds exactly the weights the
                # K loop would dequantise (path 6), so the outputs are bitwise equal
                y6 = eng.linear(name, xd, 6).float().cpu().numpy().astype(np.float64)
                assert np.array_equal(y, y6), (bits, group, name)
    finally:
        eng.close()


@pytest.mark.parametrize("name", SHAPES)
def test_decode_mfma_matches_float64(eng, weights, name):
    """The decode MFMA GEMM (3+ rows) at 3, 8, 32 and 64 rows: the float64 product with the
    fp16-rounded weights (SwiGLU for w13), and each row independent of the rows beside it."""
    import torch
    w = weights[name]
    wf = ref.f16_round(w)
    swiglu = name.endswith("w13")
    x64, xd64 = _x(torch, 64, w.shape[1], 64)
    for rows in (3, 8, 32, 64):
        y = eng.linear(name, xd64[:rows].contiguous(), 5 if swiglu else 4).float().cpu().numpy().astype(np.float64)
        ab = x64[:rows].astype(np.float64) @ wf.T
        if swiglu:
            F = w.shape[0] // 2
            want, tol = ab[:, :F] / (1 + np.exp(-ab[:, :F])) * ab[:, F:], 2e-3
        else:
            want, tol = ab, 2e-5
        err = np.abs(y - want).max() / np.abs(want).max()
        assert err < tol, (name, rows, err)
        if rows == 64:
            y3 = eng.linear(name, xd64[61:64].contiguous(), 5 if swiglu else 4).float().cpu().numpy()
            assert np.array_equal(y3, y[61:64].astype(np.float32)), name
