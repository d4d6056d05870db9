"""Kernel-level parity of the attention core (q/k norm + RoPE + KV store, attention, head gate) at
the served shapes, through the lfm3_attention hook of the C ABI, against the float64 oracle's
``attention_core``.

What is run (the shapes the benchmark and the pages use):
- decode on a full layer at T = 4095, 4097, 8192 and 32768 visible keys (the one-tile and the
  64-split regimes of the split-K kernel and their seam), alone and in batches of 8 and 32 rows of
  mixed lengths;
- decode on a sliding layer across the window seams 255 / 256 / 257 and far past the ring's wrap;
- prefill passes on both layer kinds: 256 rows with no history, 64 rows after 3,000 keys and 100
  after 500 (the served shapes of "TensorFold PR #1508", prefill-attention gate), and a 2048-row
  chunk after 6,144 keys (the 8k prefill's last chunk), the sliding one across the ring's wrap;
  on a full layer, the 2048-row chunk after 30,720 keys (the last pass of a 32768-token prompt).

Full layers read their keys through a shuffled page table (slots' pages interleaved at random in the
pool). Every cache row that holds no visible key -- unused pages, the tail of a slot's last page,
stale ring rows, the rows' own positions before the call writes them -- is filled with NaN and
+-inf ("planted NaN/inf"), so a kernel that reads outside its keys, or multiplies a masked
probability by such a value, fails. Some history keys are "needles" aligned with a chosen query
head, so the softmax is peaked at known positions (the first key, split and page boundaries, the
window's edge, the last key) rather than flat.

The bar is a float64 bound on the kernel's own roundings, per output element: the queries (and the
pass's own keys) rounded to fp16 perturb each score by at most 2^-11 * sum_i |q_i k_i| / sqrt(128)
(twice that for an own key); a score error e_j moves the output by sum_j p_j e_j |v_j - o| (first
order); the probabilities fed to P V in fp16 and the own values stored fp16 add 2^-10 sum_j p_j |v_j|;
the fp16 output adds 2^-11 |o|. The test takes twice the first-order terms and requires
|gpu - float64| <= bound at every element. A planted control -- the oracle reading the values of the
neighbouring 8 dims -- must exceed the same bound many times over, which shows the check can fail.
"""
import zlib

import numpy as np
import pytest

from attention_decoder_amd import synth
from oracle import attention_core, rmsnorm, rope_angles, rope_apply, sigmoid

pytestmark = pytest.mark.gpu

HQ, HKV, D, PG = 16, 4, 128, 16
WIDTH = (HQ + 2 * HKV) * D + HQ
F16_PLANT = np.array([0x7E00, 0x7C00, 0xFC00], dtype=np.uint16)   # NaN, +inf, -inf
RING = 256 + 2048


@pytest.fixture(scope="module")
def actx():
    import torch
    from attention_decoder_amd.lfm3 import Engine
    cfg = synth.slice3_config(max_slots=32, max_ctx=32768 + 64, max_chunk=2048, n_pages=1)
    eng = Engine(cfg, synth.cached_blob(cfg, seed=0))
    print("attention hook context ready", flush=True)
    yield torch, cfg, eng
    eng.close()


def _planted(shape, rng):
    return F16_PLANT[rng.integers(0, 3, size=shape, dtype=np.uint8)]


def _f16(x):
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _val(u16):
    return u16.view(np.float16).astype(np.float64)


class Case:
    """Host arrays of one hook call and, per query group, the oracle's history."""

    def __init__(self, rng, sliding, decode, slots, pos, n_rows):
        self.sliding, self.decode = sliding, decode
        self.slots, self.pos, self.n = list(slots), list(pos), n_rows
        self.qkvg = rng.standard_normal((n_rows, WIDTH), dtype=np.float32)
        self.qn = synth.f32_to_bf16_bits(1 + 0.02 * rng.standard_normal(D).astype(np.float32))
        self.kn = synth.f32_to_bf16_bits(1 + 0.02 * rng.standard_normal(D).astype(np.float32))
        self.theta, self.pairs = (1.0e4, 64) if sliding else (1.0e6, 32)
        self.window = 256 if sliding else None
        self.pt, self.max_pages, self.n_pool, self.ring = None, 0, 0, 0

    def row_pos(self):
        """Absolute position of every query row."""
        return np.array(self.pos if self.decode else [self.pos[0] + r for r in range(self.n)])

    def exact_q(self):
        q = self.qkvg[:, :HQ * D].reshape(self.n, HQ, D).astype(np.float64)
        q = rmsnorm(q, synth.bf16_bits_to_f32(self.qn).astype(np.float64), 1e-5)
        return rope_apply(q, rope_angles(self.row_pos(), self.theta, self.pairs, D))


def _history(rng, case, q, groups):
    """groups: list of (slot, first own position, [query rows]). Returns {slot: (K, V)} float16 bit
    arrays [h, HKV, D] for positions 0 .. h-1, with needles aligned to the group's query heads."""
    hist = {}
    for slot, h, rows in groups:
        K = rng.standard_normal((h, HKV, D), dtype=np.float32)
        V = rng.standard_normal((h, HKV, D), dtype=np.float32)
        if h > 0:
            for i in range(8):
                r = rows[(i * 7) % len(rows)]
                p = case.row_pos()[r]
                lo = max(0, p - 255) if case.sliding else 0
                hi = min(h - 1, p - 1)
                if hi < lo:
                    continue
                cands = [lo, hi, lo + 1, (lo + hi) // 2, min(hi, lo + 511), min(hi, lo + 512), min(hi, lo + 16),
                         int(rng.integers(lo, hi + 1))]
                n = min(max(cands[i], lo), hi)
                beta = 0.9 if i % 2 == 0 else 0.6
                for g in range(HKV):
                    qh = q[r, 4 * g + i % 4]
                    K[n, g] = (beta * qh / np.linalg.norm(qh) * np.sqrt(D)).astype(np.float32)
        hist[slot] = (_f16(K), _f16(V))
    return hist


def _lay_out_cache(rng, case, hist, own):
    """Place the histories in a shuffled paged pool or in per-slot rings; everything else planted.
    own: {slot: last own position} (the call writes positions from the history's end to it)."""
    n_slots = max(case.slots) + 1
    if case.sliding:
        case.ring = RING
        kc = _planted((n_slots, HKV, RING, D), rng)
        vc = _planted((n_slots, HKV, RING, D), rng)
        for slot, (K, V) in hist.items():
            h = K.shape[0]
            lo = max(0, h - 255)
            p = np.arange(lo, h)
            kc[slot][:, p % RING, :] = K[lo:h].transpose(1, 0, 2)
            vc[slot][:, p % RING, :] = V[lo:h].transpose(1, 0, 2)
        return kc, vc
    need = {s: own[s] // PG + 1 for s in own}
    total = sum(need.values()) + 5
    perm = rng.permutation(total)
    case.max_pages = max(need.values()) + 3
    case.n_pool = total
    pt = np.full((n_slots, case.max_pages), perm[-1], dtype=np.int32)   # unused entries: a planted page
    off = 0
    for s in sorted(need):
        pt[s, :need[s]] = perm[off:off + need[s]]
        off += need[s]
    case.pt = pt
    kc = _planted((total, HKV, PG, D), rng)
    vc = _planted((total, HKV, PG, D), rng)
    for slot, (K, V) in hist.items():
        h = K.shape[0]
        if h == 0:
            continue
        p = np.arange(h)
        kc[pt[slot, p // PG], :, p % PG, :] = K
        vc[pt[slot, p // PG], :, p % PG, :] = V
    return kc, vc


def _run_gpu(torch, eng, case, kc, vc):
    from attention_decoder_amd.lfm3 import lfm3_attention
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kd, vd = t(kc.view(np.int16)), t(vc.view(np.int16))
    out = torch.empty((case.n, HQ * D), dtype=torch.float16, device=dev)
    pt = t(case.pt) if case.pt is not None else None
    print(f"attention hook: sliding={case.sliding} decode={case.decode} rows={case.n} pos={case.pos[:8]}", flush=True)
    lfm3_attention(eng.ctx, sliding=case.sliding, decode=case.decode, slots=case.slots, pos=case.pos,
                   qkvg=t(case.qkvg), q_norm=t(case.qn.view(np.int16)), k_norm=t(case.kn.view(np.int16)),
                   k_cache=kd, v_cache=vd, out=out, page_table=pt, max_pages=case.max_pages,
                   n_pool_pages=case.n_pool, n_slots=max(case.slots) + 1, ring_rows=case.ring)
    torch.cuda.synchronize()
    return (out.cpu().numpy().astype(np.float64), kd.cpu().numpy().view(np.uint16),
            vd.cpu().numpy().view(np.uint16))


def f16_bound(q, kc, vc, pos, window, new0, gate):
    """The per-element bound described in the module docstring. q [M, HQ, D] exact queries; kc, vc
    [T, HKV, D] float64 keys / values of positions 0 .. T-1 (keys >= new0 are the pass's own);
    gate [M, HQ] = sigmoid(g)."""
    m, t = q.shape[0], kc.shape[0]
    j = np.arange(t)
    own = np.where(j >= new0, 2.0, 1.0)
    out = np.empty((m, HQ, D))
    for r0 in range(0, m, 64):
        qq, pp = q[r0:r0 + 64], pos[r0:r0 + 64]
        vis = j[None, :] <= pp[:, None]
        if window:
            vis &= (pp[:, None] - j[None, :]) < window
        for g in range(HKV):
            qh = qq[:, 4 * g:4 * g + 4].transpose(1, 0, 2)             # [4, m, D]
            K, V = kc[:, g, :], vc[:, g, :]
            s = np.where(vis[None], np.matmul(qh, K.T) / np.sqrt(D), -np.inf)
            e = np.exp(s - s.max(axis=2, keepdims=True))
            p = e / e.sum(axis=2, keepdims=True)
            o = np.matmul(p, V)
            eps = 2.0 ** -11 * np.matmul(np.abs(qh), np.abs(K).T) / np.sqrt(D) * own[None, None, :] + 2.0 ** -24
            w = p * eps
            first = np.matmul(w, np.abs(V)) + np.abs(o) * w.sum(axis=2, keepdims=True)
            pv = np.matmul(p, np.abs(V))
            gg = gate[r0:r0 + 64, 4 * g:4 * g + 4].T[:, :, None]
            b = gg * 2.0 * (first + 2.0 ** -10 * pv) + 2.0 ** -11 * np.abs(gg * o) + 1e-6
            out[r0:r0 + 64, 4 * g:4 * g + 4] = b.transpose(1, 0, 2)
    return out.reshape(m, HQ * D)


def _oracle_group(cfg, case, rows, K, V, shift=0):
    """The oracle's gated output, the bound, and the cache after the append, for query rows `rows`
    of one slot whose history is K, V (fp16 bits [h, HKV, D])."""
    pos = case.row_pos()[rows]
    h = K.shape[0]
    Kh, Vh = _val(K), _val(V)
    if case.sliding:                       # keys outside every row's window are never visible
        lo = max(0, int(pos.min()) - 255)
        Kh[:lo] = 0.0
        Vh[:lo] = 0.0
    qkvg = case.qkvg[rows].astype(np.float64)
    if shift:                              # planted control: every value read from dims d + shift
        Vh = np.roll(Vh, shift, axis=2)
        v0 = (HQ + HKV) * D
        vv = qkvg[:, v0:v0 + HKV * D].reshape(-1, HKV, D)
        qkvg[:, v0:v0 + HKV * D] = np.roll(vv, shift, axis=2).reshape(-1, HKV * D)
    qn = synth.bf16_bits_to_f32(case.qn).astype(np.float64)
    kn = synth.bf16_bits_to_f32(case.kn).astype(np.float64)
    o, kc, vc = attention_core(qkvg, qn, kn, Kh, Vh, pos, cfg, case.theta, case.pairs, case.window)
    if shift:
        return o, None, kc, vc
    q = case.exact_q()[rows]
    gate = sigmoid(qkvg[:, (HQ + 2 * HKV) * D:])
    return o, f16_bound(q, kc, vc, pos, case.window, h, gate), kc, vc


def _check(torch, eng, cfg, case, hist, label):
    rng = np.random.default_rng(zlib.crc32(label.encode()))
    own = {s: (case.pos[b] if case.decode else case.pos[0] + case.n - 1) for b, s in enumerate(case.slots)}
    kc, vc = _lay_out_cache(rng, case, hist, own)
    got, kc_after, vc_after = _run_gpu(torch, eng, case, kc, vc)
    assert np.isfinite(got).all(), label
    groups = ([(s, [b]) for b, s in enumerate(case.slots)] if case.decode
              else [(case.slots[0], list(range(case.n)))])
    worst, worst_ctl, worst_abs = 0.0, np.inf, 0.0
    for slot, rows in groups:
        K, V = hist[slot]
        want, bound, kcat, vcat = _oracle_group(cfg, case, rows, K, V)
        err = np.abs(got[rows] - want)
        ratio = err / bound
        worst = max(worst, float(ratio.max()))
        worst_abs = max(worst_abs, float(err.max()))
        assert ratio.max() <= 1.0, (label, slot, float(ratio.max()), np.unravel_index(ratio.argmax(), ratio.shape))
        ctl, _, _, _ = _oracle_group(cfg, case, rows, K, V, shift=8)
        worst_ctl = min(worst_ctl, float((np.abs(got[rows] - ctl) / bound).max()))
        # the rows' own keys and values were written into the cache: keys within fp16 rounding of
        # the oracle's normed and rotated keys, values bitwise fp16(v)
        h = K.shape[0]
        for r_i, r in enumerate(rows):
            p = case.row_pos()[r]
            if case.sliding:
                kw, vw = kc_after[slot][:, p % case.ring, :], vc_after[slot][:, p % case.ring, :]
            else:
                kw = kc_after[case.pt[slot, p // PG], :, p % PG, :]
                vw = vc_after[case.pt[slot, p // PG], :, p % PG, :]
            kref = kcat[h + r_i]
            # one fp16 rounding (2^-11 relative) of an fp32 value that carries a few fp32 ulps of
            # the norm and the rotation, relative to the norm of the rotated pair (i, i + 64): a
            # rotated element can be small by cancellation while its pair is not
            pair = np.sqrt(kref[:, :D // 2] ** 2 + kref[:, D // 2:] ** 2)
            pair = np.concatenate([pair, pair], axis=1)
            assert np.all(np.abs(_val(kw) - kref) <= 2.0 ** -11 * np.abs(kref) + 2.0 ** -20 * pair + 2.0 ** -24), (label, r)
            vraw = case.qkvg[r, (HQ + HKV) * D:(HQ + 2 * HKV) * D].reshape(HKV, D)
            assert np.array_equal(vw, _f16(vraw)), (label, r)
    print(f"{label}: max |gpu - float64| {worst_abs:.3e}, max ratio to the bound {worst:.3f}; "
          f"V-from-the-neighbouring-8-dims control: min over groups of its max ratio {worst_ctl:.1f}")
    assert worst_ctl > 10.0, (label, worst_ctl)


def _decode_case(rng, cfg, sliding, lengths):
    """One decode launch: row b is slot b at position lengths[b] - 1 (lengths = visible keys)."""
    n = len(lengths)
    case = Case(rng, sliding, 1, range(n), [t - 1 for t in lengths], n)
    q = case.exact_q()
    hist = _history(rng, case, q, [(b, lengths[b] - 1, [b]) for b in range(n)])
    return case, hist


@pytest.mark.parametrize("T", [4095, 4097, 8192, 32768])
def test_decode_full_long_context(actx, T):
    torch, cfg, eng = actx
    rng = np.random.default_rng(T)
    case, hist = _decode_case(rng, cfg, 0, [T])
    _check(torch, eng, cfg, case, hist, f"decode full T={T}")


def test_decode_full_batch8(actx):
    torch, cfg, eng = actx
    rng = np.random.default_rng(8)
    case, hist = _decode_case(rng, cfg, 0, [4095, 4097, 8192, 32768, 1, 64, 65, 20000])
    _check(torch, eng, cfg, case, hist, "decode full B=8")


def test_decode_full_batch32(actx):
    torch, cfg, eng = actx
    rng = np.random.default_rng(32)
    lengths = [4095, 4097, 8192, 32768] + [int(t) for t in rng.integers(1, 32769, size=28)]
    case, hist = _decode_case(rng, cfg, 0, lengths)
    _check(torch, eng, cfg, case, hist, "decode full B=32")


def test_decode_sliding_window_seams(actx):
    torch, cfg, eng = actx
    rng = np.random.default_rng(256)
    case, hist = _decode_case(rng, cfg, 1, [1, 2, 255, 256, 257, 258, 3001, 5000])
    _check(torch, eng, cfg, case, hist, "decode sliding B=8")


PREFILL_SHAPES = [(0, 256), (3000, 64), (500, 100), (6144, 2048)]


@pytest.mark.parametrize("sliding", [0, 1])
@pytest.mark.parametrize("hist_len,rows", PREFILL_SHAPES)
def test_prefill_pass(actx, sliding, hist_len, rows):
    torch, cfg, eng = actx
    rng = np.random.default_rng(1000 * hist_len + rows + sliding)
    case = Case(rng, sliding, 0, [3], [hist_len], rows)
    q = case.exact_q()
    hist = _history(rng, case, q, [(3, hist_len, list(range(rows)))])
    _check(torch, eng, cfg, case, hist, f"prefill {'sliding' if sliding else 'full'} {rows} rows after {hist_len}")


def test_prefill_pass_32k_last_chunk(actx):
    """The last 2048-row pass of a 32768-token prompt on a full layer (2048 rows after 30,720
    keys), the prompt length of the 4-bit g32 / 8-bit head workload. The oracle's dense scores for
    it take about 9 GB of host memory and a minute."""
    torch, cfg, eng = actx
    hist_len, rows = 30720, 2048
    rng = np.random.default_rng(1000 * hist_len + rows)
    case = Case(rng, 0, 0, [3], [hist_len], rows)
    q = case.exact_q()
    hist = _history(rng, case, q, [(3, hist_len, list(range(rows)))])
    _check(torch, eng, cfg, case, hist, f"prefill full {rows} rows after {hist_len}")


def test_hook_refuses_bad_arguments(actx):
    """Host-side checks: nothing is enqueued for a page outside the pool, a ring too small for the
    pass, or a position past the RoPE tables."""
    import torch
    from attention_decoder_amd.lfm3 import LFM3Error, lfm3_attention
    _, cfg, eng = actx
    rng = np.random.default_rng(5)
    case = Case(rng, 0, 1, [0], [40], 1)
    dev = "cuda"
    z = lambda *s: torch.zeros(s, dtype=torch.int16, device=dev)
    qkvg = torch.from_numpy(case.qkvg).to(dev)
    pt = torch.tensor([[0, 1, 7]], dtype=torch.int32, device=dev)
    out = torch.empty((1, HQ * D), dtype=torch.float16, device=dev)
    kw = dict(qkvg=qkvg, q_norm=z(D), k_norm=z(D), out=out)
    with pytest.raises(LFM3Error) as ei:
        lfm3_attention(eng.ctx, sliding=0, decode=1, slots=[0], pos=[40], k_cache=z(4, HKV, PG, D),
                       v_cache=z(4, HKV, PG, D), page_table=pt, max_pages=3, n_pool_pages=4, n_slots=1, **kw)
    assert ei.value.status == 1 and "n_pool_pages" in ei.value.message
    with pytest.raises(LFM3Error):
        lfm3_attention(eng.ctx, sliding=1, decode=0, slots=[0], pos=[0], k_cache=z(1, HKV, 300, D),
                       v_cache=z(1, HKV, 300, D), ring_rows=300, n_slots=1,
                       **dict(kw, qkvg=torch.zeros((64, WIDTH), device=dev),
                              out=torch.empty((64, HQ * D), dtype=torch.float16, device=dev)))
    with pytest.raises(LFM3Error):
        lfm3_attention(eng.ctx, sliding=1, decode=1, slots=[0], pos=[cfg["max_ctx"]], k_cache=z(1, HKV, 300, D),
                       v_cache=z(1, HKV, 300, D), ring_rows=300, n_slots=1, **kw)
