"""Seeded synthetic inputs for the LFM3-1.7B hybrid decoder: configs, weights, blob, prompts.

This module is shared by the oracle-side tests and the GPU-side harness. It holds no step of the
forward pass: it draws random numbers, turns them into MLX-style affine codes (the input format),
packs them, and writes the weight blob. The forward pass itself lives in the HIP library (product)
and, independently, in ``oracle/`` (test infrastructure).

Sources (the pages this build follows):
- "LFM3-1.7B port" knowledge note, LFM2.5 -> LFM3 comparison table: 24 layers, width 2048, FFN 7680,
  16 q / 4 kv heads of 128, 13 conv + 11 attention (6 full + 5 sliding, window 256), conv kernel 7,
  partial RoPE on the full layers (theta 1e6) and full RoPE on the sliding ones (theta 1e4),
  sandwich RMSNorm eps 1e-5, vocab 128000 tied.
- TensorFold issue "Add native Metal support for LFM3-1.7B ...", "Checkpoint handling": MLX affine
  4/6/8-bit in groups of 64; the VL 4-bit export uses groups of 32 with an 8-bit embedding.

Blob layout (this library's own format; both readers are written independently):
  bytes 0..8    magic b"LFM3BLB1"
  u32 version (=1), u32 n_tensors, u64 table_offset (=64), u64 data_offset, u64 total_bytes, 24 B pad
  n_tensors x 128-byte entries at table_offset:
     char name[80], u32 dtype, u32 ndim, u32 shape[4], u64 offset, u64 nbytes, 8 B pad
  tensor data at 256-byte-aligned offsets.
dtype codes: 0 = packed unsigned codes (u8 bytes), 1 = bf16, 2 = f32, 3 = i32.
Quantized linear "<name>" of shape [N, K] is three tensors:
  <name>.q       u8   [N, K*bits/8]   codes little-endian, low bits first (a plain bitstream per row)
  <name>.scales  bf16 [N, K/group]
  <name>.biases  bf16 [N, K/group]
"""
from __future__ import annotations

import hashlib
import json
import os
import struct
from concurrent.futures import ThreadPoolExecutor

import numpy as np

MAGIC = b"LFM3BLB1"
VERSION = 1
ENTRY_BYTES = 128
TABLE_OFFSET = 64
DT_CODES, DT_BF16, DT_F32, DT_I32 = 0, 1, 2, 3
LT_CONV, LT_FULL, LT_SLIDING = 0, 1, 2

# ----------------------------------------------------------------------------------------------
# configs
# ----------------------------------------------------------------------------------------------


def default_layer_types(n_layers: int = 24) -> list[int]:
    """Interleaving for the seeded 24-layer geometry (the pages print only "interleaved").

    Layer i is attention iff i is odd and i <= 21; the attention layers alternate sliding, full,
    sliding, ... and layer 21 is full. That gives 13 conv, 5 sliding and 6 full layers.
    """
    assert n_layers == 24
    out = []
    for i in range(n_layers):
        if i % 2 == 1 and i <= 21:
            out.append(LT_FULL if (i == 21 or (i // 2) % 2 == 1) else LT_SLIDING)
        else:
            out.append(LT_CONV)
    return out


FFN_AS_LINEARS, FFN_NVFP4, FFN_FP8B = 0, 1, 2


def make_config(*, layer_types, bits=4, group=64, embed_bits=None, embed_group=None,
                has_embedding=1, max_slots=1, max_ctx=4096, max_chunk=2048, n_pages=None,
                page_tokens=16, ffn_format=FFN_AS_LINEARS):
    """A complete config dict. Every field the library takes is explicit here. bits = 16 stores
    the mixers' linears (and, with embed_bits = 16, the embedding / head) as bf16; ffn_format
    stores w13 and w2 as NVFP4 or block-FP8 instead of the mixers' format."""
    if embed_bits is None:
        embed_bits = bits
    if embed_group is None:
        embed_group = group
    if n_pages is None:
        n_pages = max_slots * ((max_ctx + page_tokens - 1) // page_tokens)
    return dict(
        n_layers=len(layer_types), hidden=2048, ffn=7680, n_q_heads=16, n_kv_heads=4, head_dim=128,
        vocab=128000, conv_taps=7, window=256, layer_type=list(layer_types),
        rope_theta_full=1.0e6, rope_theta_sliding=1.0e4, rope_pairs_full=32, rope_pairs_sliding=64,
        norm_eps=1e-5, bits=bits, group=group, embed_bits=embed_bits, embed_group=embed_group,
        has_embedding=has_embedding, max_slots=max_slots, max_ctx=max_ctx, page_tokens=page_tokens,
        max_chunk=max_chunk, n_pages=n_pages, ffn_format=ffn_format,
    )


def slice3_config(**kw):
    """Three-layer slice at real width: conv, sliding attention, full attention; no embedding/head."""
    kw.setdefault("max_ctx", 1024)
    kw.setdefault("max_chunk", 512)
    return make_config(layer_types=[LT_CONV, LT_SLIDING, LT_FULL], has_embedding=0, **kw)


def full_config(bits=4, group=64, **kw):
    """The full 24-layer LFM3-1.7B geometry."""
    return make_config(layer_types=default_layer_types(24), bits=bits, group=group, **kw)


def nvfp4_config(**kw):
    """The layout of the NVFP4 export ("TensorFold PR #1508"): FFN w1 | w3 and w2 in NVFP4, every
    mixer projection, the embedding and the tied head in bf16."""
    kw.setdefault("embed_bits", 16)
    kw.setdefault("embed_group", 0)
    return full_config(bits=16, group=0, ffn_format=FFN_NVFP4, **kw)


# ----------------------------------------------------------------------------------------------
# tensor inventory (shared naming; each reader validates it on its own)
# ----------------------------------------------------------------------------------------------


def linear_shapes(cfg, lt):
    """(name-suffix, N, K) of the quantized linears of one layer of type lt."""
    H, F = cfg["hidden"], cfg["ffn"]
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    kvd = cfg["n_kv_heads"] * cfg["head_dim"]
    out = []
    if lt == LT_CONV:
        out += [("conv.in_proj", 3 * H, H), ("conv.out_proj", H, H)]
    else:
        out += [("attn.qkvg_proj", qd + 2 * kvd + cfg["n_q_heads"], H), ("attn.o_proj", H, qd)]
    out += [("ffn.w13", 2 * F, H), ("ffn.w2", H, F)]
    return out


def linear_kind(cfg, name):
    """Storage of linear `name`: "lin" (MLX affine), "bf16lin", "nvfp4" or "fp8b"."""
    if name == "embedding":
        return "bf16lin" if cfg["embed_bits"] == 16 else "lin"
    ff = cfg.get("ffn_format", FFN_AS_LINEARS)
    if ".ffn." in name and ff:
        return {FFN_NVFP4: "nvfp4", FFN_FP8B: "fp8b"}[ff]
    return "bf16lin" if cfg["bits"] == 16 else "lin"


def tensor_plan(cfg):
    """Ordered list of (name, kind, shape, bits, group); kind in {"lin", "bf16lin", "nvfp4",
    "fp8b", "bf16"}.

    For linears the shape is the logical [N, K]. The blob stores "lin" as .q/.scales/.biases,
    "bf16lin" as .weight (bf16), "nvfp4" as .fp4 (codes [N, K/2]), .block_scales (e4m3 bytes
    [N, K/16]), .tensor_scale and .input_scale (fp32 [1]), "fp8b" as .fp8 (e4m3 bytes [N, K]) and
    .block_scales (fp32 [ceil(N/128), ceil(K/128)]).
    """
    H, D = cfg["hidden"], cfg["head_dim"]
    plan = []
    if cfg["has_embedding"]:
        plan.append(("embedding", linear_kind(cfg, "embedding"), (cfg["vocab"], H), cfg["embed_bits"], cfg["embed_group"]))
    for i, lt in enumerate(cfg["layer_type"]):
        p = f"layers.{i}."
        for nm in ("operator_norm", "post_operator_norm", "ffn_norm", "post_ffn_norm"):
            plan.append((p + nm, "bf16", (H,), 0, 0))
        if lt == LT_CONV:
            plan.append((p + "conv.kernel", "bf16", (H, cfg["conv_taps"]), 0, 0))
        else:
            plan.append((p + "attn.q_norm", "bf16", (D,), 0, 0))
            plan.append((p + "attn.k_norm", "bf16", (D,), 0, 0))
        for nm, n, k in linear_shapes(cfg, lt):
            plan.append((p + nm, linear_kind(cfg, p + nm), (n, k), cfg["bits"], cfg["group"]))
    plan.append(("embedding_norm", "bf16", (H,), 0, 0))
    return plan


# ----------------------------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (uint16). Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------------------------
# MLX-style affine quantizer + bit packing (input generation, not part of the forward pass)
# ----------------------------------------------------------------------------------------------


def quantize_affine(w: np.ndarray, bits: int, group: int):
    """w [N, K] float32 -> (codes uint8 [N, K], scales bf16 bits [N, K/g], biases bf16 bits).

    Per group: bias = bf16(min), scale = bf16((max - min) / (2^bits - 1)),
    code = clip(round((w - bias) / scale), 0, 2^bits - 1).
    """
    n, k = w.shape
    g = w.reshape(n, k // group, group)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    levels = float(2 ** bits - 1)
    scale_b = f32_to_bf16_bits((mx - mn) / levels)
    bias_b = f32_to_bf16_bits(mn)
    s = bf16_bits_to_f32(scale_b)
    b = bf16_bits_to_f32(bias_b)
    s_safe = np.where(s == 0, 1.0, s).astype(np.float32)
    q = np.rint((g - b[:, :, None]) / s_safe[:, :, None])
    q = np.clip(q, 0, levels).astype(np.uint8).reshape(n, k)
    return q, scale_b, bias_b


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """codes [N, K] (each < 2^bits) -> bytes [N, K*bits/8], a little-endian bitstream per row."""
    n, k = q.shape
    q = q.astype(np.uint32)
    if bits == 8:
        return q.astype(np.uint8)
    if bits == 4:
        q2 = q.reshape(n, k // 2, 2)
        return (q2[:, :, 0] | (q2[:, :, 1] << 4)).astype(np.uint8)
    if bits == 6:
        q4 = q.reshape(n, k // 4, 4)
        word = q4[:, :, 0] | (q4[:, :, 1] << 6) | (q4[:, :, 2] << 12) | (q4[:, :, 3] << 18)
        out = np.empty((n, k // 4, 3), dtype=np.uint8)
        out[:, :, 0] = word & 0xFF
        out[:, :, 1] = (word >> 8) & 0xFF
        out[:, :, 2] = (word >> 16) & 0xFF
        return out.reshape(n, k // 4 * 3)
    raise ValueError(f"unsupported bits {bits}")


# ----------------------------------------------------------------------------------------------
# weight generation and the blob
# ----------------------------------------------------------------------------------------------


def _rng(seed: int, idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, idx])))


_E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 bytes, round to nearest (torch's float8_e4m3fn conversion), clamped to 448."""
    import torch
    t = torch.from_numpy(np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_decode(b: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def quantize_nvfp4(w: np.ndarray):
    """w [N, K] float32 -> (packed e2m1 [N, K/2], e4m3 scale bytes [N, K/16], tensor scale, input
    scale). Tensor scale = amax / (6 * 448); a group's scale = e4m3(group amax / (6 * tensor
    scale)); a code is the nearest e2m1 value of w / (scale * tensor scale)."""
    n, k = w.shape
    ts = np.float32(max(float(np.abs(w).max()), 1e-30) / (6.0 * 448.0))
    g = w.reshape(n, k // 16, 16)
    sb = _e4m3_bits(np.abs(g).max(axis=2) / (np.float32(6.0) * ts))
    eff = _e4m3_decode(sb).astype(np.float32) * ts
    r = g / np.where(eff == 0, np.float32(1.0), eff)[:, :, None]
    mag = np.abs(r)
    idx = np.abs(mag[..., None] - _E2M1_MAGS).argmin(axis=-1)
    codes = (idx + np.where(r < 0, 8, 0)).astype(np.uint8).reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb, ts, np.float32(1.0)


def quantize_fp8_block(w: np.ndarray, block: int = 128):
    """w [N, K] float32 -> (e4m3 bytes [N, K], fp32 scales [ceil(N/128), ceil(K/128)]): per block
    scale = amax / 448, code = e4m3(w / scale)."""
    n, k = w.shape
    nb, kb = -(-n // block), -(-k // block)
    sc = np.zeros((nb, kb), dtype=np.float32)
    for i in range(nb):
        for j in range(kb):
            a = float(np.abs(w[i * block:(i + 1) * block, j * block:(j + 1) * block]).max())
            sc[i, j] = a / 448.0 if a > 0 else 1.0
    full = np.repeat(np.repeat(sc, block, axis=0)[:n], block, axis=1)[:, :k]
    return _e4m3_bits(w / full), sc


def _gen_tensor(args):
    idx, (name, kind, shape, bits, group), seed = args
    rng = _rng(seed, idx)
    if kind in ("lin", "bf16lin", "nvfp4", "fp8b"):
        n, k = shape
        w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
        if kind == "bf16lin":
            return [(name + ".weight", DT_BF16, f32_to_bf16_bits(w))]
        if kind == "nvfp4":
            packed, sb, ts, ins = quantize_nvfp4(w)
            return [(name + ".fp4", DT_CODES, packed), (name + ".block_scales", DT_CODES, sb),
                    (name + ".tensor_scale", DT_F32, np.array([ts], dtype=np.float32)),
                    (name + ".input_scale", DT_F32, np.array([ins], dtype=np.float32))]
        if kind == "fp8b":
            codes, sc = quantize_fp8_block(w)
            return [(name + ".fp8", DT_CODES, codes), (name + ".block_scales", DT_F32, sc)]
        q, s, b = quantize_affine(w, bits, group)
        return [(name + ".q", DT_CODES, pack_codes(q, bits)), (name + ".scales", DT_BF16, s),
                (name + ".biases", DT_BF16, b)]
    if name.endswith("conv.kernel"):
        w = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    else:  # norm weights 1 + N(0, 0.02)
        w = np.float32(1.0) + rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    return [(name, DT_BF16, f32_to_bf16_bits(w))]


def build_blob(cfg, seed: int = 0, threads: int | None = None) -> bytes:
    """Seeded weights -> packed blob bytes. Deterministic in (cfg geometry, seed)."""
    plan = tensor_plan(cfg)
    threads = threads or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(_gen_tensor, [(i, p, seed) for i, p in enumerate(plan)]))
    tensors = [t for part in parts for t in part]
    n = len(tensors)
    data_offset = TABLE_OFFSET + n * ENTRY_BYTES
    data_offset = (data_offset + 4095) // 4096 * 4096
    entries = []
    off = data_offset
    for name, dt, arr in tensors:
        nb = arr.nbytes
        entries.append((name, dt, arr.shape, off, nb))
        off = (off + nb + 255) // 256 * 256
    total = off
    buf = bytearray(total)
    struct.pack_into("<8sIIQQQ", buf, 0, MAGIC, VERSION, n, TABLE_OFFSET, data_offset, total)
    for i, (name, dt, shape, o, nb) in enumerate(entries):
        nm = name.encode()
        assert len(nm) < 80
        shp = list(shape) + [0] * (4 - len(shape))
        struct.pack_into("<80sII4IQQ", buf, TABLE_OFFSET + i * ENTRY_BYTES, nm, dt, len(shape), *shp, o, nb)
    mv = memoryview(buf)
    for (name, dt, arr), (_, _, _, o, nb) in zip(tensors, entries):
        mv[o:o + nb] = np.ascontiguousarray(arr).view(np.uint8).reshape(-1).tobytes()
    return bytes(buf)


def geometry_key(cfg) -> str:
    keys = ["n_layers", "hidden", "ffn", "n_q_heads", "n_kv_heads", "head_dim", "vocab", "conv_taps",
            "layer_type", "bits", "group", "embed_bits", "embed_group", "has_embedding"]
    d = {k: cfg[k] for k in keys}
    if cfg.get("ffn_format", FFN_AS_LINEARS):
        d["ffn_format"] = cfg["ffn_format"]
    return hashlib.sha1(json.dumps(d, sort_keys=True).encode()).hexdigest()[:16]


def cached_blob(cfg, seed: int = 0, cache_dir: str | None = None) -> bytes:
    """build_blob with an on-disk cache keyed by geometry and seed (blobs are ~1-2 GB)."""
    cache_dir = cache_dir or os.environ.get("LFM3_BLOB_CACHE", "/tmp/lfm3_blobs")
    os.makedirs(cache_dir, exist_ok=True)
    path = os.path.join(cache_dir, f"{geometry_key(cfg)}_s{seed}.bin")
    if os.path.exists(path):
        with open(path, "rb") as f:
            return f.read()
    blob = build_blob(cfg, seed)
    tmp = path + f".tmp{os.getpid()}"
    with open(tmp, "wb") as f:
        f.write(blob)
    os.replace(tmp, path)
    return blob


# ----------------------------------------------------------------------------------------------
# seeded inputs
# ----------------------------------------------------------------------------------------------


def prompt_tokens(seed: int, n: int, vocab: int = 128000) -> np.ndarray:
    """Token ids uniform in [0, vocab)."""
    return _rng(seed, 1_000_001).integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def hidden_rows(seed: int, n: int, hidden: int = 2048) -> np.ndarray:
    """Input hidden rows N(0, 1) as bf16 bit patterns [n, hidden] (the no-embedding slice)."""
    x = _rng(seed, 1_000_002).standard_normal((n, hidden), dtype=np.float32)
    return f32_to_bf16_bits(x)


def stream_prompt_lengths(seed: int, n_streams: int, lo: int = 300, hi: int = 2960) -> np.ndarray:
    """Per-stream prompt lengths uniform in [lo, hi]."""
    return _rng(seed, 1_000_003).integers(lo, hi + 1, size=n_streams).astype(np.int32)


def stream_prompts(seed: int, lengths) -> list[np.ndarray]:
    """Independent token prompts, one per stream, ids uniform in [0, 128000)."""
    return [_rng(seed, 2_000_000 + i).integers(0, 128000, size=int(n)).astype(np.int32)
            for i, n in enumerate(lengths)]
