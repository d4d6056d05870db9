"""Float64 reference of the LFM3-1.7B hybrid decoder (test infrastructure only; see package doc).

What each function follows, and what pins it (tests in tests/test_oracle_*.py):

- ``unpack_codes`` / ``dequant``: MLX affine weights, w = q * scale + bias per group along the
  input dim ("TensorFold #1491", Checkpoint handling: affine groups of 64, the VL 4-bit export at
  groups of 32 with an 8-bit embedding). Pinned by exact equality on hand-built codes and by the
  byte totals of the checkpoint header ("TensorFold PR #1508", NVFP4 admission commit: 594 tensors
  / 973,008,384 B at MLX 4-bit, 502 / 1,829,689,408 B at NVFP4) reproduced from the geometry.
- ``rmsnorm``: x / sqrt(mean(x^2) + eps) * w, eps 1e-5 ("LFM3-1.7B port", comparison table,
  "Unchanged" line). Pinned by closed-form special cases.
- ``rope_angles`` / ``rope_apply``: inv_freq over the whole head_dim, first n_pairs entries
  theta^(-2i/head_dim) and the rest 0, duplicated and applied with rotate_half, so pairs (i, i+64)
  rotate ("LFM3-1.7B port", "partial_rotary_factor" section). Full layers theta 1e6 and 32 pairs,
  sliding layers theta 1e4 and all 64 pairs (comparison table row 3). Pinned by a per-pair
  2x2-rotation check, norm preservation, relative-position invariance, identity at p = 0 and the
  pass-through dims.
- ``conv_step``: depthwise causal short conv over [state | B*x], the state being the last 6
  columns of B*x ("LFM3-1.7B port", table row 1; "--pad-tail": the new state is columns [n, n+6)
  of [state | Bx]). Pinned by a brute-force direct convolution of the whole sequence.
- ``attention_rows``: softmax(q k / sqrt(d)) v over visible keys; GQA with 4 query heads per KV
  head ("TensorFold PR #1508", prefill-attention commit); sliding visibility is
  0 <= query pos - key pos < 256 ("LFM3-1.7B port", "window_size, with no mask input"). Pinned by
  per-key brute force at the seams 255/256/257 and by the repeated-KV MHA reduction.
- Gate: o_h * sigmoid(g_h), g from the mixer's normed input, in fp32 on the pages (table row 4 and
  the fp32-gate paragraph). Sandwich norms and the SwiGLU FFN: table row 5 and "Unchanged".
- ``Oracle``: the whole forward, rows in position order; prefill is the same per-row math as
  one-row decode. Pinned by prefill == decode at every cut point and by the model-level negative
  controls (drop the gate, rotate every dim, remove the window, drop the conv state) that the
  pages ran. Whole-model logits against the real checkpoint: parity unpinned (no checkpoint).
"""
from __future__ import annotations

import struct
from dataclasses import dataclass, field

import numpy as np

LT_CONV, LT_FULL, LT_SLIDING = 0, 1, 2

# ----------------------------------------------------------------------------------------------
# blob reader (independent of the writer and of the C++ reader)
# ----------------------------------------------------------------------------------------------


class Blob:
    """Reads this library's weight blob: 64-byte header, 128-byte entries, aligned tensor data."""

    def __init__(self, data: bytes):
        self.data = memoryview(data)
        magic, ver, n, tab, dat, total = struct.unpack_from("<8sIIQQQ", data, 0)
        if magic != b"LFM3BLB1" or ver != 1:
            raise ValueError("not an LFM3 blob")
        if total != len(data):
            raise ValueError("blob size mismatch")
        self.entries = {}
        for i in range(n):
            raw = struct.unpack_from("<80sII4IQQ", data, tab + 128 * i)
            name = raw[0].rstrip(b"\0").decode()
            dt, nd = raw[1], raw[2]
            shape = tuple(raw[3:3 + nd])
            off, nb = raw[7], raw[8]
            self.entries[name] = (dt, shape, off, nb)

    def raw(self, name):
        dt, shape, off, nb = self.entries[name]
        return dt, shape, np.frombuffer(self.data[off:off + nb], dtype=np.uint8)

    def f32(self, name) -> np.ndarray:
        """An fp32 tensor as float64 values."""
        dt, shape, b = self.raw(name)
        assert dt == 2
        return b.view(np.float32).astype(np.float64).reshape(shape)

    def bf16(self, name) -> np.ndarray:
        """A bf16 tensor as exact float64 values."""
        dt, shape, b = self.raw(name)
        assert dt == 1
        bits = b.view(np.uint16).astype(np.uint64) << np.uint64(16)
        return bits.astype(np.uint32).view(np.float32).astype(np.float64).reshape(shape)


def unpack_codes(packed: np.ndarray, bits: int, k: int) -> np.ndarray:
    """Packed bytes [N, k*bits/8] -> integer codes [N, k]: a little-endian, low-bit-first bitstream."""
    n = packed.shape[0]
    bitstream = np.unpackbits(packed.reshape(n, -1), axis=1, bitorder="little")
    bitstream = bitstream[:, : k * bits].reshape(n, k, bits).astype(np.int64)
    weights = (1 << np.arange(bits, dtype=np.int64))
    return (bitstream * weights).sum(axis=2)


def dequant(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray, group: int) -> np.ndarray:
    """w[n, k] = q[n, k] * scale[n, k // group] + bias[n, k // group], exactly, in float64."""
    n, k = codes.shape
    s = np.repeat(scales, group, axis=1)
    b = np.repeat(biases, group, axis=1)
    return codes.astype(np.float64) * s + b


def e2m1_values(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (0..15) -> float64: bit 3 sign, bits 2..1 exponent with bias 1, bit 0
    mantissa; exponent 0 is subnormal (0 or 0.5). The element format of NVFP4 ("TensorFold PR
    #1508": the FFN's e2m1 codes)."""
    c = np.asarray(codes).astype(np.int64)
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3 (the finite variant) bytes -> float64: bit 7 sign, bits 6..3 exponent with bias 7,
    bits 2..0 mantissa; exponent 0 is subnormal (m * 2^-9); 0x7F and 0xFF are NaN. NVFP4's block
    scales ("TensorFold PR #1508": e4m3 block scales) and block-FP8 weights are in it."""
    c = np.asarray(codes).astype(np.int64)
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


def dequant_nvfp4(packed: np.ndarray, block_scales: np.ndarray, tensor_scale: float) -> np.ndarray:
    """NVFP4 weight [N, K] from packed e2m1 codes [N, K/2] (two a byte, element 2i in the low
    nibble), e4m3 scales [N, K/16] (one per 16 consecutive k) and the fp32 tensor scale:
    w = e2m1(code) * e4m3(scale) * tensor_scale, exactly in float64 ("TensorFold PR #1508": e2m1
    codes in groups of 16 with e4m3 block scales and an fp32 tensor scale)."""
    n = packed.shape[0]
    codes = np.empty((n, packed.shape[1] * 2), dtype=np.int64)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    sc = np.repeat(e4m3_values(block_scales), 16, axis=1)
    return e2m1_values(codes) * sc * float(tensor_scale)


def dequant_fp8_block(codes: np.ndarray, block_scales: np.ndarray, block: int = 128) -> np.ndarray:
    """Block-FP8 weight [N, K]: e4m3 codes times one fp32 scale per block x block tile of the
    weight (scales [ceil(N/block), ceil(K/block)]), exactly in float64."""
    n, k = codes.shape
    sc = np.repeat(np.repeat(block_scales, block, axis=0)[:n], block, axis=1)[:, :k]
    return e4m3_values(codes) * sc


def load_weight(blob: Blob, name: str, fmt: str, bits: int = 0, group: int = 0) -> np.ndarray:
    """Float64 weight [N, K] of linear `name` in storage format `fmt`: "affine" (MLX codes with bf16
    scale and bias), "bf16" (stored bf16 values), "nvfp4" or "fp8b" (block-FP8, 128 x 128)."""
    if fmt == "affine":
        return load_linear(blob, name, bits, group)
    if fmt == "bf16":
        return blob.bf16(name + ".weight")
    if fmt == "nvfp4":
        _, shape, q = blob.raw(name + ".fp4")
        _, sshape, sb = blob.raw(name + ".block_scales")
        ts = float(blob.f32(name + ".tensor_scale")[0])
        return dequant_nvfp4(q.reshape(shape), sb.reshape(sshape), ts)
    if fmt == "fp8b":
        _, shape, q = blob.raw(name + ".fp8")
        return dequant_fp8_block(q.reshape(shape), blob.f32(name + ".block_scales"))
    raise ValueError(f"unknown weight format {fmt}")


def load_linear(blob: Blob, name: str, bits: int, group: int, row_chunk: int = 8192) -> np.ndarray:
    """Dequantized float64 weight [N, K] of a quantized linear stored in the blob."""
    _, qshape, qb = blob.raw(name + ".q")
    n, kbytes = qshape
    k = kbytes * 8 // bits
    s = blob.bf16(name + ".scales")
    b = blob.bf16(name + ".biases")
    assert s.shape == (n, k // group) and b.shape == (n, k // group)
    q = qb.reshape(n, kbytes)
    out = np.empty((n, k), dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        out[r0:r1] = dequant(unpack_codes(q[r0:r1], bits, k), s[r0:r1], b[r0:r1], group)
    return out


# ----------------------------------------------------------------------------------------------
# elementwise definitions
# ----------------------------------------------------------------------------------------------


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of float64 data."""
    f = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(f)                      # f = m * 2^e, 0.5 <= |m| < 1
    scaled = np.ldexp(m, 8)                 # 8 significant bits
    r = np.round(scaled)                    # numpy rounds half to even
    return np.ldexp(r, e - 8)


def f16_round(x: np.ndarray) -> np.ndarray:
    """Nearest IEEE fp16 value (ties to even, with fp16 range); used only by the storage diagnostic."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def silu(a):
    return a / (1.0 + np.exp(-a))


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def rope_angles(pos: np.ndarray, theta: float, n_pairs: int, head_dim: int) -> np.ndarray:
    """Angles [M, head_dim/2]: pos * inv_freq, inv_freq_i = theta^(-2i/head_dim) for i < n_pairs, else 0."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv = np.where(i < n_pairs, float(theta) ** (-2.0 * i / head_dim), 0.0)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope_apply(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """x [M, heads, D] rotated with cat(freqs, freqs) and rotate_half: pairs (i, i + D/2)."""
    half = x.shape[-1] // 2
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def conv_step(state: np.ndarray, z: np.ndarray, kernel: np.ndarray):
    """One causal depthwise step. state [taps-1, C] oldest first, z [C], kernel [C, taps].

    window = [state | z]; y = sum_j kernel[:, j] * window[j]; new state = window[1:].
    """
    window = np.concatenate([state, z[None, :]], axis=0)
    y = np.einsum("jc,cj->c", window, kernel)
    return y, window[1:]


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, qpos: np.ndarray,
                   window: int | None) -> np.ndarray:
    """q [M, Hq, D] at absolute positions qpos; k, v [T, Hkv, D] at positions 0..T-1.

    Key j is visible to a query at p iff j <= p, and (sliding) p - j < window.
    Query head h reads KV head h // (Hq // Hkv).
    """
    m, hq, d = q.shape
    t, hkv, _ = k.shape
    rep = hq // hkv
    kk = np.repeat(k, rep, axis=1)          # [T, Hq, D]
    vv = np.repeat(v, rep, axis=1)
    # scores[h, m, t] = q[m, h, :] . k[t, h, :] / sqrt(D), as one batched matmul over heads
    scores = np.matmul(q.transpose(1, 0, 2), kk.transpose(1, 2, 0)) / np.sqrt(d)
    j = np.arange(t)[None, :]
    p = np.asarray(qpos)[:, None]
    vis = j <= p
    if window is not None:
        vis &= (p - j) < window
    scores = np.where(vis[None], scores, -np.inf)
    mx = scores.max(axis=2, keepdims=True)
    e = np.exp(scores - mx)
    e = np.where(vis[None], e, 0.0)
    pr = e / e.sum(axis=2, keepdims=True)
    # o[m, h, :] = sum_t pr[h, m, t] v[t, h, :]
    return np.matmul(pr, vv.transpose(1, 0, 2)).transpose(1, 0, 2)


def greedy_argmax(logits: np.ndarray) -> np.ndarray:
    """Argmax over the last axis; ties go to the lower id and NaN ranks as -inf."""
    x = np.where(np.isnan(logits), -np.inf, logits)
    return np.argmax(x, axis=-1)          # numpy returns the first maximum


def top2_margin(logits: np.ndarray) -> np.ndarray:
    x = np.sort(np.where(np.isnan(logits), -np.inf, logits), axis=-1)
    return x[..., -1] - x[..., -2]


def attention_core(qkvg, q_norm, k_norm, k_hist, v_hist, pos, cfg, theta, n_pairs, window, gate=True,
                   rnd=lambda x: x):
    """The attention mixer from its qkvg linear output to the gated head outputs, for rows at
    absolute positions ``pos`` appended after the cached keys / values ``k_hist``, ``v_hist``
    [T0, Hkv, D] of positions 0 .. T0-1 ("LFM3-1.7B port", comparison table rows 2-4: per-head q/k
    RMSNorm, RoPE, GQA attention, sigmoid output gate in fp32; "window_size" section for the sliding
    mask). qkvg [M, Hq*D + 2*Hkv*D + Hq] splits into q | k | v | g. Norm first, then RoPE.

    Returns (o [M, Hq*D] gated, K [T0+M, Hkv, D], V [T0+M, Hkv, D]) -- the cache after the append.
    ``rnd`` is the storage-point rounding of the diagnostic mode (identity by default).
    """
    hq, hkv, d, eps = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["norm_eps"]
    m = qkvg.shape[0]
    q = qkvg[:, : hq * d].reshape(m, hq, d)
    k = qkvg[:, hq * d: hq * d + hkv * d].reshape(m, hkv, d)
    v = qkvg[:, hq * d + hkv * d: hq * d + 2 * hkv * d].reshape(m, hkv, d)
    g = qkvg[:, hq * d + 2 * hkv * d: hq * d + 2 * hkv * d + hq]
    q = rmsnorm(q, q_norm, eps)
    k = rmsnorm(k, k_norm, eps)
    ang = rope_angles(pos, theta, n_pairs, d)
    q = rnd(rope_apply(q, ang))
    k = rnd(rope_apply(k, ang))
    kc = np.concatenate([k_hist, k], axis=0)
    vc = np.concatenate([v_hist, rnd(v)], axis=0)
    o = np.empty((m, hq, d))
    for r0 in range(0, m, 256):
        r1 = min(m, r0 + 256)
        o[r0:r1] = attention_rows(q[r0:r1], kc, vc, pos[r0:r1], window)
    if gate:
        o = o * sigmoid(g)[:, :, None]
    return o.reshape(m, hq * d), kc, vc


# ----------------------------------------------------------------------------------------------
# whole model
# ----------------------------------------------------------------------------------------------


@dataclass
class SlotState:
    length: int = 0
    conv: dict = field(default_factory=dict)     # layer -> [taps-1, C]
    k: dict = field(default_factory=dict)        # layer -> [T, Hkv, D]
    v: dict = field(default_factory=dict)

    def copy(self):
        return SlotState(self.length, {a: b.copy() for a, b in self.conv.items()},
                         {a: b.copy() for a, b in self.k.items()}, {a: b.copy() for a, b in self.v.items()})


class Oracle:
    """The decoder in float64. ``controls`` plants model-level mistakes for negative tests:
    'no_gate', 'rotate_all' (full layers rotate every pair), 'no_window', 'no_conv_state'."""

    def __init__(self, cfg: dict, blob: bytes, controls: tuple = (), storage_points=False):
        self.cfg = cfg
        self.blob = Blob(blob)
        self.controls = set(controls)
        # storage diagnostic: False (plain float64, the parity reference), "bf16" or "fp16" (round
        # every storage point to that format), "fp16_pair" (fp16, with the operator-norm output
        # carried as an fp16 pair); True means "fp16_pair"
        if storage_points is True:
            storage_points = "fp16_pair"
        if storage_points not in (False, None, "bf16", "fp16", "fp16_pair"):
            raise ValueError(f"unknown storage_points {storage_points!r}")
        self.storage = storage_points or None
        self._w = {}

    # weights -------------------------------------------------------------------------------
    def fmt_of(self, name: str):
        """(format, bits, group) of linear `name` under the config: the embedding follows
        embed_bits / embed_group, the FFN (w13, w2) ffn_format, the mixers bits / group; 16 bits
        means stored bf16 ("TensorFold PR #1508": the NVFP4 export keeps the mixers, embedding and
        tied head in bf16 and only the FFN in fp4)."""
        c = self.cfg
        if name == "embedding":
            return ("bf16", 16, 0) if c["embed_bits"] == 16 else ("affine", c["embed_bits"], c["embed_group"])
        ff = c.get("ffn_format", 0)
        if ".ffn." in name and ff:
            return ({1: "nvfp4", 2: "fp8b"}[ff], 0, 0)
        return ("bf16", 16, 0) if c["bits"] == 16 else ("affine", c["bits"], c["group"])

    def _lin(self, name, bits=None, group=None):
        if name not in self._w:
            fmt, b, g = self.fmt_of(name)
            self._w[name] = load_weight(self.blob, name, fmt, b, g)
        return self._w[name]

    def embedding(self):
        return self._lin("embedding")

    def drop_cache(self):
        self._w.clear()

    def preload(self, threads: int = 8):
        """Dequantize every linear up front (setup only; the same loader per tensor)."""
        from concurrent.futures import ThreadPoolExecutor
        suffixes = (".q", ".weight", ".fp4", ".fp8")
        names = sorted({k.rsplit(".", 1)[0] for k in self.blob.entries if k.endswith(suffixes)})
        if not self.cfg["has_embedding"]:
            names = [n for n in names if n != "embedding"]
        todo = [n for n in names if n not in self._w]

        def one(n):
            fmt, b, g = self.fmt_of(n)
            return load_weight(self.blob, n, fmt, b, g)
        with ThreadPoolExecutor(threads) as ex:
            for n, w in zip(todo, ex.map(one, todo)):
                self._w[n] = w

    def new_slot(self) -> SlotState:
        c = self.cfg
        st = SlotState()
        for i, lt in enumerate(c["layer_type"]):
            if lt == LT_CONV:
                st.conv[i] = np.zeros((c["conv_taps"] - 1, c["hidden"]))
            else:
                st.k[i] = np.zeros((0, c["n_kv_heads"], c["head_dim"]))
                st.v[i] = np.zeros((0, c["n_kv_heads"], c["head_dim"]))
        return st

    def _r(self, x):
        """Storage diagnostic mode (off by default; parity is judged against plain float64): round
        where the GPU stores a 16-bit value -- the matmul inputs (the ffn-norm rows, the conv's z
        and C*y, the gated attention output, the SwiGLU product), the cached k and v, and the conv
        state -- to bf16 or fp16. Linear outputs and the residual stream stay wide."""
        if self.storage is None:
            return x
        return bf16_round(x) if self.storage == "bf16" else f16_round(x)

    def _r2(self, x):
        """Storage diagnostic for the conv layers' operator-norm output, which feeds in_proj: one
        rounding, or in "fp16_pair" mode the high part plus its rounded remainder."""
        if self.storage != "fp16_pair":
            return self._r(x)
        hi = f16_round(x)
        return hi + f16_round(x - hi)

    # layers ---------------------------------------------------------------------------------
    def _conv_mixer(self, i, st, u):
        c = self.cfg
        H = c["hidden"]
        bcx = u @ self._lin(f"layers.{i}.conv.in_proj").T
        b, cg, x = bcx[:, :H], bcx[:, H:2 * H], bcx[:, 2 * H:]
        z = self._r(b * x)
        ker = self.blob.bf16(f"layers.{i}.conv.kernel")
        ys = np.empty_like(z)
        state = st.conv[i]
        for t in range(z.shape[0]):
            ys[t], state = conv_step(state, z[t], ker)
        if "no_conv_state" not in self.controls:   # control: the state is not written back
            st.conv[i] = self._r(state)
        o = self._r(cg * ys)
        return o @ self._lin(f"layers.{i}.conv.out_proj").T

    def _attn_mixer(self, i, st, u, pos, lt):
        c = self.cfg
        qkvg = u @ self._lin(f"layers.{i}.attn.qkvg_proj").T
        if lt == LT_FULL:
            theta, pairs = c["rope_theta_full"], c["rope_pairs_full"]
            if "rotate_all" in self.controls:
                pairs = c["head_dim"] // 2
        else:
            theta, pairs = c["rope_theta_sliding"], c["rope_pairs_sliding"]
        win = c["window"] if (lt == LT_SLIDING and "no_window" not in self.controls) else None
        o, k, v = attention_core(qkvg, self.blob.bf16(f"layers.{i}.attn.q_norm"),
                                 self.blob.bf16(f"layers.{i}.attn.k_norm"), st.k[i], st.v[i], pos, c,
                                 theta, pairs, win, gate="no_gate" not in self.controls, rnd=self._r)
        st.k[i], st.v[i] = k, v
        return self._r(o) @ self._lin(f"layers.{i}.attn.o_proj").T

    def _ffn(self, i, h):
        c = self.cfg
        F = c["ffn"]
        u = self._r(rmsnorm(h, self.blob.bf16(f"layers.{i}.ffn_norm"), c["norm_eps"]))
        ab = u @ self._lin(f"layers.{i}.ffn.w13").T
        s = self._r(silu(ab[:, :F]) * ab[:, F:])
        return s @ self._lin(f"layers.{i}.ffn.w2").T

    # forward --------------------------------------------------------------------------------
    def forward(self, st: SlotState, tokens=None, hidden=None, logits: str = "last",
                capture: bool = False):
        """Append rows to the slot. tokens [M] int or hidden [M, H] float64 (exactly one).

        Returns dict: 'layers' (list of residuals after each layer, if capture), 'final'
        (embedding_norm output [M, H]), 'logits' ([1, V] for 'last', [M, V] for 'all', or None).
        """
        c = self.cfg
        eps = c["norm_eps"]
        if tokens is not None:
            tokens = np.asarray(tokens, dtype=np.int64)
            h = self.embedding()[tokens]
        else:
            h = np.asarray(hidden, dtype=np.float64)
        m = h.shape[0]
        pos = np.arange(st.length, st.length + m)
        layers = []
        for i, lt in enumerate(c["layer_type"]):
            u = rmsnorm(h, self.blob.bf16(f"layers.{i}.operator_norm"), eps)
            u = self._r2(u) if lt == LT_CONV else self._r(u)
            if lt == LT_CONV:
                mo = self._conv_mixer(i, st, u)
            else:
                mo = self._attn_mixer(i, st, u, pos, lt)
            h = h + rmsnorm(mo, self.blob.bf16(f"layers.{i}.post_operator_norm"), eps)
            f = self._ffn(i, h)
            h = h + rmsnorm(f, self.blob.bf16(f"layers.{i}.post_ffn_norm"), eps)
            if capture:
                layers.append(h.copy())
        st.length += m
        final = rmsnorm(h, self.blob.bf16("embedding_norm"), eps)
        out = {"layers": layers, "final": final, "logits": None}
        if logits and c["has_embedding"]:
            rows = final[-1:] if logits == "last" else final
            out["logits"] = rows @ self.embedding().T
        return out
