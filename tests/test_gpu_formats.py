"""The NVFP4 and block-FP8 FFN formats and stored-bf16 linears ("TensorFold PR #1508": the NVFP4
export keeps the FFN as e2m1 codes in groups of 16 with e4m3 block scales and an fp32 tensor
scale, and the mixers, embedding and tied head in bf16; its block-FP8 counterpart) on the GPU
against the float64 oracle.

Kernel level, on a three-layer slice with a small tied head (vocab 1024):
- dequantisation bit-exact: the device's fp32 value of every weight equals the oracle's exact value
  rounded to fp32 (exact for bf16; one rounding of the scaled code for NVFP4 and block-FP8), and its
  fp16 value that value rounded to fp16;
- the decode GEMV (exact weights) against the float64 product, within 1e-4 relative;
- the prefill GEMM and the decode MFMA GEMM against the float64 product with the fp16-rounded
  weights (their stated rounding point), within 2e-5 relative (SwiGLU: 2e-3).
Model level: the full 24-layer geometry in the NVFP4 export's layout, a 300-token prompt and
greedy steps teacher-forced against the oracle, and one batch-8 decode step; the block-FP8 FFN on
the slice, per-layer residuals against the oracle.
"""
import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import Blob, Oracle, f16_round, load_weight

from gpu_full_common import REL_L2, compare_logits, dev_tokens, gpu_greedy, oracle_teacher_forced, rel_l2

pytestmark = pytest.mark.gpu

LINEARS = ["layers.0.conv.in_proj", "layers.1.attn.qkvg_proj", "layers.2.attn.o_proj", "layers.0.ffn.w13",
           "layers.2.ffn.w2"]


def _slice_cfg(ffn_format):
    cfg = synth.make_config(layer_types=[0, 2, 1], bits=16, group=0, embed_bits=16, embed_group=0,
                            ffn_format=ffn_format, max_slots=8, max_ctx=1024, max_chunk=512)
    cfg["vocab"] = 1024
    return cfg


@pytest.fixture(scope="module", params=[1, 2], ids=["nvfp4", "fp8_block"])
def fmt_engine(request):
    from attention_decoder_amd.lfm3 import Engine
    cfg = _slice_cfg(request.param)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    orc = Oracle(cfg, blob)
    print(f"ffn_format {request.param} slice engine ready", flush=True)
    yield cfg, blob, eng, orc
    eng.close()


def _w(orc, name):
    fmt, b, g = orc.fmt_of(name)
    return load_weight(orc.blob, name, fmt, b, g)


def _x(torch, rows, k, seed):
    x = np.random.default_rng(seed).standard_normal((rows, k)).astype(np.float16)
    return x, torch.from_numpy(x).cuda()


def test_dequant_bit_exact(fmt_engine):
    cfg, blob, eng, orc = fmt_engine
    for name in LINEARS + ["embedding"]:
        w = _w(orc, name)
        rows = min(w.shape[0], 300)
        f32, f16 = eng.dequant_rows(name, 0, rows)
        want32 = w[:rows].astype(np.float32)
        assert np.array_equal(f32.cpu().numpy(), want32), name
        assert np.array_equal(f16.cpu().numpy(), want32.astype(np.float16)), name


def test_gemv_exact_weights(fmt_engine):
    import torch
    cfg, blob, eng, orc = fmt_engine
    for name in LINEARS:
        w = _w(orc, name)
        for rows in (1, 2, 5):
            x, xd = _x(torch, rows, w.shape[1], rows)
            y = eng.linear(name, xd, 0).cpu().numpy().astype(np.float64)
            want = x.astype(np.float64) @ w.T
            err = np.abs(y - want).max() / np.abs(want).max()
            assert err < 1e-4, (name, rows, err)
    w = _w(orc, "layers.0.ffn.w13")
    F = w.shape[0] // 2
    x, xd = _x(torch, 3, w.shape[1], 9)
    y = eng.linear("layers.0.ffn.w13", xd, 2).float().cpu().numpy().astype(np.float64)
    ab = x.astype(np.float64) @ w.T
    want = ab[:, :F] / (1 + np.exp(-ab[:, :F])) * ab[:, F:]
    assert np.linalg.norm(y - want) / np.linalg.norm(want) < 2e-3


@pytest.mark.parametrize("path", [1, 4])
def test_mfma_paths_fp16_weights(fmt_engine, path):
    import torch
    cfg, blob, eng, orc = fmt_engine
    for name in LINEARS:
        w = _w(orc, name)
        wf = f16_round(w.astype(np.float32).astype(np.float64))
        swiglu = name.endswith("w13")
        for rows in ((3, 8, 32) if path == 4 else (1, 77, 300)):
            x, xd = _x(torch, rows, w.shape[1], 40 + rows)
            p = (5 if path == 4 else 3) if swiglu else path
            y = eng.linear(name, xd, p).float().cpu().numpy().astype(np.float64)
            ab = x.astype(np.float64) @ wf.T
            if swiglu:
                F = w.shape[0] // 2
                want, tol = ab[:, :F] / (1 + np.exp(-ab[:, :F])) * ab[:, F:], 2e-3
            else:
                want, tol = ab, 2e-5
            err = np.abs(y - want).max() / np.abs(want).max()
            assert err < tol, (name, path, rows, err)


def test_slice_layers_against_oracle(fmt_engine):
    """64 prompt tokens then 8 decode steps through the whole slice: every layer's residual within
    the rel-L2 bar and the last rows' logits within the logit bar."""
    import torch
    cfg, blob, eng, orc = fmt_engine
    toks = synth.prompt_tokens(13, 72, vocab=1024)
    L, H = cfg["n_layers"], cfg["hidden"]
    cap = torch.zeros((L, 64, H), dtype=torch.float32, device="cuda")
    eng.reset(0)
    eng.capture(cap, 64)
    eng.prefill(0, tokens=dev_tokens(torch, toks[:64]), logits=False, argmax=False)
    eng.capture(None, 0)
    lg = []
    for t in toks[64:]:
        o = eng.decode([0], tokens=dev_tokens(torch, [t]), logits=True, argmax=True)
        lg.append(o["logits"][0].cpu().numpy().astype(np.float64))
    torch.cuda.synchronize()
    st = orc.new_slot()
    out = orc.forward(st, tokens=toks[:64], logits=None, capture=True)
    rels = [rel_l2(cap[i].cpu().numpy().astype(np.float64), out["layers"][i]) for i in range(L)]
    print("per-layer rel-L2:", rels)
    assert max(rels) <= REL_L2
    want = np.stack([orc.forward(st, tokens=[t], logits="last")["logits"][0] for t in toks[64:]])
    d = np.abs(np.stack(lg) - want).max()
    print(f"decode logits max|d| {d:.3e}")
    assert d <= 2e-2


def test_slice_batch8_decode_against_oracle(fmt_engine):
    """Eight slots decoded in one step (the decode MFMA GEMM from the fp16 copies: the conv
    in_proj with its input pair, the split output projections, SwiGLU and the head): each row's
    logits against the oracle's decode of that slot alone."""
    import torch
    cfg, blob, eng, orc = fmt_engine
    prompts = [synth.prompt_tokens(70 + i, 10 + 7 * i, vocab=1024) for i in range(8)]
    for i in range(8):
        eng.reset(i)
        eng.prefill(i, tokens=dev_tokens(torch, prompts[i]), logits=False, argmax=False)
    step = [int(t) for t in synth.prompt_tokens(80, 8, vocab=1024)]
    o = eng.decode(list(range(8)), tokens=dev_tokens(torch, step), logits=True, argmax=True)
    got = o["logits"].cpu().numpy().astype(np.float64)
    for i in range(8):
        st = orc.new_slot()
        orc.forward(st, tokens=prompts[i], logits=None)
        want = orc.forward(st, tokens=[step[i]], logits="last")["logits"][0]
        d = np.abs(got[i] - want).max()
        assert d <= 2e-2, (i, d)


def test_nvfp4_full_geometry():
    """The NVFP4 export's layout at the full geometry: a 300-token prompt and 4 greedy steps at
    batch 1, then one batch-8 step, against the oracle."""
    import torch
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.nvfp4_config(max_slots=8, max_ctx=1024, max_chunk=2048)
    blob = synth.cached_blob(cfg, seed=0)
    eng = Engine(cfg, blob)
    try:
        prompt = synth.prompt_tokens(41, 300)
        fed, ids, lg = gpu_greedy(eng, torch, 0, prompt, 4)
        prompts = [synth.prompt_tokens(50 + i, 20 + 30 * i) for i in range(8)]
        for i in range(8):
            eng.reset(i)
            eng.prefill(i, tokens=dev_tokens(torch, prompts[i]), logits=False, argmax=False)
        step = [int(t) for t in synth.prompt_tokens(60, 8)]
        o8 = eng.decode(list(range(8)), tokens=dev_tokens(torch, step), logits=True, argmax=True)
        l8 = o8["logits"].cpu().numpy().astype(np.float64)
        a8 = [int(v) for v in o8["argmax"].cpu().numpy()]
        print("GPU done", flush=True)
    finally:
        eng.close()
    orc = Oracle(cfg, blob)
    orc.preload(16)
    try:
        ref = oracle_teacher_forced(orc, prompt, fed)
        compare_logits(lg, ids, ref, "NVFP4 layout, 300-token prompt + 4 greedy")
        for i in (0, 7):
            want = oracle_teacher_forced(orc, np.concatenate([prompts[i], [step[i]]]), [])
            compare_logits(l8[i:i + 1], [a8[i]], want, f"NVFP4 layout, batch-8 decode, stream {i}")
    finally:
        orc.drop_cache()
