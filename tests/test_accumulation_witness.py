"""The accumulation witness of tests/test_gpu_accumulation.py is sharp (CPU only).

Rows whose terms are all 1 or 1 + d (d = 2^-10, 2^-7 or 0.5), K = 2048 or 7680 of them, sum to
K + c d, a multiple of d below 2^14 that fp32 holds exactly in any order. Summed with an fp16 or a
bf16 accumulator (each partial sum rounded to that format), in sequential or pairwise order, the
result misses K + c d by at least two units of d -- so a kernel that returns K + c d bit for bit
does not accumulate in those formats (TensorFold issue #1491, "Validation": stress cases that tell
fp32 accumulation from reduced precision).
"""
import numpy as np

from attention_decoder_amd import synth


def test_reduced_precision_accumulators_miss_the_witness():
    """The witness is sharp: fp16 or bf16 accumulation of one row's terms, sequential or pairwise,
    misses K + c d by at least two units of d (CPU, numpy)."""
    rng = np.random.default_rng(5)

    def bf16(v):
        return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32)))

    def pairwise(t, rnd):
        t = [rnd(v) for v in t]
        while len(t) > 1:
            t = [rnd(t[i] + t[i + 1]) if i + 1 < len(t) else t[i] for i in range(0, len(t), 2)]
        return float(t[0])

    def sequential(t, rnd):
        s = rnd(0.0)
        for v in t:
            s = rnd(s + v)
        return float(s)

    def f16(v):
        return np.float16(v)

    def bf(v):
        return float(bf16(v).reshape(-1)[0])

    errs = []
    for k, d in ((2048, 2.0 ** -10), (7680, 2.0 ** -10), (2048, 2.0 ** -7), (7680, 0.5)):
        sel = rng.random(k) < 0.3
        terms = np.where(sel, 1.0 + d, 1.0)
        exact = k + sel.sum() * d
        assert float(np.float32(np.sum(terms.astype(np.float32)))) == exact      # fp32 holds it
        for acc in (sequential, pairwise):
            for rnd in (f16, bf):
                err = abs(acc(terms, rnd) - exact)
                errs.append((k, d, acc.__name__, rnd.__name__, err))
    for k, d, how, fmt, err in errs:
        assert err >= 2 * d, (k, d, how, fmt, err)
