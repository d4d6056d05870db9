"""lfm3_attention_noalloc -- decode attention with its split partials in the library's own static
device array, for callers that cannot allocate -- against lfm3_attention (the same kernels with the
partials in the context's workspace): bitwise equal outputs on two calls in a row, the second
smaller, for a full layer (shuffled pages, multi-split rows) and a sliding layer; oversize and
incomplete calls are refused before anything is enqueued."""
import numpy as np
import pytest

from attention_decoder_amd import synth

import test_gpu_attention as A

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nctx():
    import torch
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.slice3_config(max_slots=8, max_ctx=8192 + 64, max_chunk=256, n_pages=1)
    eng = Engine(cfg, synth.cached_blob(cfg, seed=0))
    yield torch, cfg, eng
    eng.close()


def _run(torch, eng, case, kc, vc, noalloc):
    from attention_decoder_amd.lfm3 import lfm3_attention
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kd, vd = t(kc.view(np.int16)), t(vc.view(np.int16))
    out = torch.empty((case.n, A.HQ * A.D), dtype=torch.float16, device="cuda")
    print(f"noalloc={noalloc} sliding={case.sliding} rows={case.n} pos={case.pos}", flush=True)
    lfm3_attention(eng.ctx, sliding=case.sliding, decode=1, slots=case.slots, pos=case.pos, qkvg=t(case.qkvg),
                   q_norm=t(case.qn.view(np.int16)), k_norm=t(case.kn.view(np.int16)), k_cache=kd, v_cache=vd,
                   out=out, page_table=None if case.pt is None else t(case.pt), max_pages=case.max_pages,
                   n_pool_pages=case.n_pool, n_slots=max(case.slots) + 1, ring_rows=case.ring, noalloc=noalloc)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), kd.cpu().numpy(), vd.cpu().numpy()


@pytest.mark.parametrize("sliding", [0, 1])
def test_noalloc_equals_workspace_entry_point(nctx, sliding):
    torch, cfg, eng = nctx
    rng = np.random.default_rng(77 + sliding)
    for lengths in ([4097, 8192, 1, 300, 4095, 65, 5000, 2], [700, 3]):   # the second call is smaller
        case, hist = A._decode_case(rng, cfg, sliding, lengths)
        own = {b: lengths[b] - 1 for b in range(len(lengths))}
        kc, vc = A._lay_out_cache(rng, case, hist, own)
        got = _run(torch, eng, case, kc, vc, True)
        want = _run(torch, eng, case, kc, vc, False)
        for g, w in zip(got, want):
            assert np.array_equal(g, w), lengths


def test_noalloc_refusals(nctx):
    torch, cfg, eng = nctx
    from attention_decoder_amd.lfm3 import LFM3Error
    rng = np.random.default_rng(5)
    case, hist = A._decode_case(rng, cfg, 0, [40] * 9)
    kc, vc = A._lay_out_cache(rng, case, hist, {b: 39 for b in range(9)})
    with pytest.raises(LFM3Error) as ei:
        _run(torch, eng, case, kc, vc, True)
    assert ei.value.status == 5
    from attention_decoder_amd import lfm3
    import ctypes
    io = lfm3.AttnIO(0, 1, 1, (ctypes.c_int32 * 1)(0), (ctypes.c_int32 * 1)(3))
    st = lfm3.load_library().lfm3_attention_noalloc(eng.ctx, ctypes.byref(io), None)
    assert st == 1
