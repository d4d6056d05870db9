"""ctypes binding of liblfm3.so (include/lfm3.h): argument marshalling only.

Every step of the forward pass runs in the HIP library; PyTorch provides device memory and the
stream. There is no fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LFM3_LIBRARY", os.path.join(HERE, "liblfm3.so"))
HEADER = os.path.join(os.path.dirname(HERE), "include", "lfm3.h")

STATUS = {0: "LFM3_OK", 1: "LFM3_ERR_ARG", 2: "LFM3_ERR_CONFIG", 3: "LFM3_ERR_BLOB", 4: "LFM3_ERR_SLOT",
          5: "LFM3_ERR_CAPACITY", 6: "LFM3_ERR_DEVICE"}
MAX_LAYERS = 64
MAX_BATCH = 64


class LFM3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "ffn", "n_q_heads", "n_kv_heads", "head_dim", "vocab", "conv_taps", "window",
        "rope_pairs_full", "rope_pairs_sliding", "bits", "group", "embed_bits", "embed_group", "has_embedding",
        "max_slots", "max_ctx", "page_tokens", "max_chunk", "n_pages")] + [
        ("norm_eps", ctypes.c_float), ("rope_theta_full", ctypes.c_double), ("rope_theta_sliding", ctypes.c_double),
        ("layer_type", ctypes.c_uint8 * MAX_LAYERS), ("ffn_format", ctypes.c_int32)]


def config_from_dict(d: dict) -> Config:
    c = Config()
    for name, _ in Config._fields_:
        if name == "layer_type":
            lt = (ctypes.c_uint8 * MAX_LAYERS)(*([int(v) for v in d["layer_type"]] + [0] * (MAX_LAYERS - len(d["layer_type"]))))
            c.layer_type = lt
        elif name == "ffn_format":
            c.ffn_format = int(d.get("ffn_format", 0))
        else:
            setattr(c, name, d[name])
    return c


class AttnIO(ctypes.Structure):
    """lfm3_attn_io: the attention-core hook's buffers (include/lfm3.h)."""
    _fields_ = [("sliding", ctypes.c_int32), ("decode", ctypes.c_int32), ("n_rows", ctypes.c_int32),
                ("slots_host", ctypes.POINTER(ctypes.c_int32)), ("pos_host", ctypes.POINTER(ctypes.c_int32)),
                ("qkvg_dev", ctypes.c_void_p), ("ld", ctypes.c_int32),
                ("q_norm_dev", ctypes.c_void_p), ("k_norm_dev", ctypes.c_void_p),
                ("k_cache_dev", ctypes.c_void_p), ("v_cache_dev", ctypes.c_void_p),
                ("page_table_dev", ctypes.c_void_p),
                ("max_pages", ctypes.c_int32), ("n_pool_pages", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("ring_rows", ctypes.c_int32), ("out_dev", ctypes.c_void_p)]


_lib = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblfm3.so (raises if it is not built: there is no other implementation)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run __graft_entry__.build() (hipcc --offload-arch=gfx950)")
    # torch first: it brings its own HIP runtime, and the library must bind to that one. Loaded
    # first, the library pulls in the system runtime and torch then loads a second one, whose
    # device memory and streams the first cannot use (lfm3_create reports no HIP device).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    sig = {
        "lfm3_query_sizes": (_i32, [P(Config), P(_sz), P(_sz)]),
        "lfm3_validate_blob": (_i32, [P(Config), _vp, _sz, ctypes.c_char_p, _sz]),
        "lfm3_create": (_i32, [P(Config), _vp, _sz, _vp, _sz, _vp, P(_vp)]),
        "lfm3_destroy": (None, [_vp]),
        "lfm3_prefill": (_i32, [_vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp]),
        "lfm3_decode_batch": (_i32, [_vp, _i32, P(_i32), _vp, _vp, _vp, _vp, _vp]),
        "lfm3_reset_slot": (_i32, [_vp, _i32]),
        "lfm3_synchronize": (_i32, [_vp]),
        "lfm3_state_bytes": (_i32, [_vp, _i32, P(_sz)]),
        "lfm3_verify": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp]),
        "lfm3_commit": (_i32, [_vp, _i32, _i32]),
        "lfm3_save_state": (_i32, [_vp, _i32, _vp, _sz, P(_i32)]),
        "lfm3_load_state": (_i32, [_vp, _i32, _vp, _sz, _i32]),
        "lfm3_slot_length": (_i32, [_vp, _i32]),
        "lfm3_free_pages": (_i32, [_vp]),
        "lfm3_last_error": (ctypes.c_char_p, [_vp]),
        "lfm3_capture_layers": (_i32, [_vp, _vp, _i32]),
        "lfm3_dequant_rows": (_i32, [_vp, ctypes.c_char_p, _i32, _i32, _vp, _vp]),
        "lfm3_linear": (_i32, [_vp, ctypes.c_char_p, _i32, _vp, _i32, _vp]),
        "lfm3_attention": (_i32, [_vp, P(AttnIO)]),
        "lfm3_attention_noalloc": (_i32, [_vp, P(AttnIO), P(_i32)]),
        "lfm3_profile": (_i32, [_vp, _i32]),
        "lfm3_profile_read": (_i32, [_vp, _i32, P(ctypes.c_double), P(ctypes.c_int64), P(ctypes.c_double),
                                     P(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_symbols(path: str = HEADER) -> list[str]:
    """Names of the functions include/lfm3.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"\b(lfm3_[a-z_]+)\s*\(", text)))


def _check(st: int, ctx=None):
    if st != 0:
        msg = load_library().lfm3_last_error(ctx).decode(errors="replace")
        raise LFM3Error(st, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---- the C calls under their own names -----------------------------------------------------------

def lfm3_query_sizes(cfg: Config):
    b, w = _sz(), _sz()
    _check(load_library().lfm3_query_sizes(ctypes.byref(cfg), ctypes.byref(b), ctypes.byref(w)))
    return b.value, w.value


def lfm3_validate_blob(cfg: Config, blob: bytes) -> tuple[int, str]:
    buf = ctypes.create_string_buffer(512)
    st = load_library().lfm3_validate_blob(ctypes.byref(cfg), ctypes.c_char_p(blob), len(blob), buf, 512)
    return st, buf.value.decode(errors="replace")


def lfm3_create(cfg: Config, blob_dev, blob_bytes: int, ws_dev, ws_bytes: int, stream_handle: int):
    ctx = ctypes.c_void_p()
    _check(load_library().lfm3_create(ctypes.byref(cfg), _ptr(blob_dev), blob_bytes, _ptr(ws_dev), ws_bytes,
                                      ctypes.c_void_p(stream_handle), ctypes.byref(ctx)))
    return ctx


def lfm3_prefill(ctx, slot, tokens, hidden, n_rows, logits_last, argmax_last, hidden_out):
    _check(load_library().lfm3_prefill(ctx, slot, _ptr(tokens), _ptr(hidden), n_rows, _ptr(logits_last),
                                       _ptr(argmax_last), _ptr(hidden_out)), ctx)


def lfm3_decode_batch(ctx, slots, tokens, hidden, logits, argmax, hidden_out):
    arr = (ctypes.c_int32 * len(slots))(*[int(s) for s in slots])
    _check(load_library().lfm3_decode_batch(ctx, len(slots), arr, _ptr(tokens), _ptr(hidden), _ptr(logits),
                                            _ptr(argmax), _ptr(hidden_out)), ctx)


def lfm3_reset_slot(ctx, slot):
    _check(load_library().lfm3_reset_slot(ctx, slot), ctx)


def lfm3_synchronize(ctx):
    _check(load_library().lfm3_synchronize(ctx), ctx)


def lfm3_verify(ctx, slot, tokens, n_rows, logits, argmax):
    _check(load_library().lfm3_verify(ctx, slot, _ptr(tokens), n_rows, _ptr(logits), _ptr(argmax)), ctx)


def lfm3_commit(ctx, slot, n_accept):
    _check(load_library().lfm3_commit(ctx, slot, n_accept), ctx)


def lfm3_state_bytes(ctx, length) -> int:
    b = _sz()
    _check(load_library().lfm3_state_bytes(ctx, length, ctypes.byref(b)), ctx)
    return b.value


def lfm3_save_state(ctx, slot, buf) -> int:
    n = _i32()
    _check(load_library().lfm3_save_state(ctx, slot, _ptr(buf), buf.numel() * buf.element_size(), ctypes.byref(n)),
           ctx)
    return n.value


def lfm3_load_state(ctx, slot, buf, length):
    _check(load_library().lfm3_load_state(ctx, slot, _ptr(buf), buf.numel() * buf.element_size(), length), ctx)


def lfm3_slot_length(ctx, slot) -> int:
    return load_library().lfm3_slot_length(ctx, slot)


def lfm3_free_pages(ctx) -> int:
    return load_library().lfm3_free_pages(ctx)


def lfm3_capture_layers(ctx, buf, max_rows):
    _check(load_library().lfm3_capture_layers(ctx, _ptr(buf), max_rows), ctx)


def lfm3_dequant_rows(ctx, name: str, row0: int, n_rows: int, out_f32, out_f16):
    _check(load_library().lfm3_dequant_rows(ctx, name.encode(), row0, n_rows, _ptr(out_f32), _ptr(out_f16)), ctx)


def lfm3_destroy(ctx):
    load_library().lfm3_destroy(ctx)


def lfm3_linear(ctx, name: str, path: int, x, rows: int, y):
    _check(load_library().lfm3_linear(ctx, name.encode(), path, _ptr(x), rows, _ptr(y)), ctx)


def lfm3_attention(ctx, *, sliding, decode, slots, pos, qkvg, q_norm, k_norm, k_cache, v_cache, out,
                   page_table=None, max_pages=0, n_pool_pages=0, n_slots=1, ring_rows=0, noalloc=False):
    """The attention-core hook: torch device tensors in, marshalled into lfm3_attn_io (noalloc:
    through lfm3_attention_noalloc, with a host copy of the page table)."""
    n = int(qkvg.shape[0])
    sl = (ctypes.c_int32 * len(slots))(*[int(v) for v in slots])
    ps = (ctypes.c_int32 * len(pos))(*[int(v) for v in pos])
    io = AttnIO(int(sliding), int(decode), n, sl, ps, qkvg.data_ptr(), int(qkvg.stride(0)), q_norm.data_ptr(),
                k_norm.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                None if page_table is None else page_table.data_ptr(), int(max_pages), int(n_pool_pages),
                int(n_slots), int(ring_rows), out.data_ptr())
    if noalloc:
        pth = None
        if page_table is not None:
            flat = [int(v) for v in page_table.cpu().reshape(-1).tolist()]
            pth = (ctypes.c_int32 * len(flat))(*flat)
        _check(load_library().lfm3_attention_noalloc(ctx, ctypes.byref(io), pth), ctx)
    else:
        _check(load_library().lfm3_attention(ctx, ctypes.byref(io)), ctx)


PROF_KINDS = {"gemv": 0, "gemm": 1, "attn_decode": 2, "attn_prefill": 3, "conv": 4, "norm": 5, "other": 6}


def lfm3_profile(ctx, enable: bool):
    _check(load_library().lfm3_profile(ctx, 1 if enable else 0), ctx)


def lfm3_profile_read(ctx, kind: int):
    ms, n, by, fl = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
    _check(load_library().lfm3_profile_read(ctx, kind, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(by),
                                            ctypes.byref(fl)), ctx)
    return {"ms": ms.value, "launches": n.value, "bytes": by.value, "flops": fl.value}


# ---- a small owner of the device regions -----------------------------------------------------------

class Engine:
    """Holds the device blob and workspace (torch tensors) and a context on one stream."""

    def __init__(self, cfg: dict, blob: bytes, device: str = "cuda:0", stream=None):
        import numpy as np
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.c = config_from_dict(cfg)
        blob_bytes, ws_bytes = lfm3_query_sizes(self.c)
        if blob_bytes != len(blob):
            raise LFM3Error(3, f"blob is {len(blob)} B, config implies {blob_bytes} B")
        self.stream = stream or torch.cuda.current_stream(self.device)
        self.blob = torch.from_numpy(np.frombuffer(blob, dtype=np.uint8).copy()).to(self.device)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        self.ws_bytes = ws_bytes
        torch.cuda.synchronize(self.device)
        self.ctx = lfm3_create(self.c, self.blob, len(blob), self.ws, ws_bytes, self.stream.cuda_stream)

    def close(self):
        if self.ctx:
            self.torch.cuda.synchronize(self.device)
            lfm3_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _empty(self, shape, dtype):
        return self.torch.empty(shape, dtype=dtype, device=self.device)

    def prefill(self, slot, tokens=None, hidden=None, logits=True, argmax=True, hidden_out=False):
        t = self.torch
        n = int(tokens.shape[0] if tokens is not None else hidden.shape[0])
        out = {}
        has_head = bool(self.cfg["has_embedding"])
        out["logits"] = self._empty((self.cfg["vocab"],), t.float32) if (logits and has_head) else None
        out["argmax"] = self._empty((1,), t.int32) if (argmax and has_head) else None
        out["hidden"] = self._empty((n, self.cfg["hidden"]), t.float32) if hidden_out else None
        lfm3_prefill(self.ctx, slot, tokens, hidden, n, out["logits"], out["argmax"], out["hidden"])
        return out

    def decode(self, slots, tokens=None, hidden=None, logits=True, argmax=True, hidden_out=False, out=None):
        t = self.torch
        n = len(slots)
        has_head = bool(self.cfg["has_embedding"])
        if out is None:
            out = {}
            out["logits"] = self._empty((n, self.cfg["vocab"]), t.float32) if (logits and has_head) else None
            out["argmax"] = self._empty((n,), t.int32) if (argmax and has_head) else None
            out["hidden"] = self._empty((n, self.cfg["hidden"]), t.float32) if hidden_out else None
        lfm3_decode_batch(self.ctx, slots, tokens, hidden, out.get("logits"), out.get("argmax"), out.get("hidden"))
        return out

    def reset(self, slot):
        lfm3_reset_slot(self.ctx, slot)

    def synchronize(self):
        lfm3_synchronize(self.ctx)

    def verify(self, slot, tokens):
        """A verify window of len(tokens) rows on `slot`: (logits [n, vocab], argmax [n])."""
        n = int(tokens.shape[0])
        lg = self._empty((n, self.cfg["vocab"]), self.torch.float32)
        am = self._empty((n,), self.torch.int32)
        lfm3_verify(self.ctx, slot, tokens, n, lg, am)
        return lg, am

    def commit(self, slot, n_accept):
        lfm3_commit(self.ctx, slot, n_accept)

    def save_state(self, slot, buf=None):
        """Kept state of `slot` into buf (a new uint8 device tensor if None): (buf, length)."""
        n = self.length(slot)
        if buf is None:
            buf = self.torch.empty(lfm3_state_bytes(self.ctx, n), dtype=self.torch.uint8, device=self.device)
        return buf, lfm3_save_state(self.ctx, slot, buf)

    def load_state(self, slot, buf, length):
        lfm3_load_state(self.ctx, slot, buf, length)

    def length(self, slot):
        return lfm3_slot_length(self.ctx, slot)

    def free_pages(self):
        return lfm3_free_pages(self.ctx)

    def capture(self, buf, max_rows):
        lfm3_capture_layers(self.ctx, buf, max_rows)

    def linear(self, name, x_f16, path):
        """y fp32 [rows, N] = x (torch fp16 [rows, K]) through the GEMV (path 0), the prefill GEMM
        (path 1; path 6 dequantises the codes in the K loop instead of reading the fp16 copy) or the
        decode MFMA GEMM (path 4); paths 2, 3, 5: the same with the SwiGLU epilogue
        (fp16 [rows, N/2])."""
        n = None
        from .synth import tensor_plan
        for nm, kind, shape, bits, group in tensor_plan(self.cfg):
            if nm == name:
                n = shape[0]
        if n is None:
            raise LFM3Error(1, f"no quantized linear named {name}")
        if path in (2, 3, 5):
            y = self._empty((x_f16.shape[0], n // 2), self.torch.float16)
        else:
            y = self._empty((x_f16.shape[0], n), self.torch.float32)
        lfm3_linear(self.ctx, name, path, x_f16, x_f16.shape[0], y)
        return y

    def profile(self, enable: bool):
        lfm3_profile(self.ctx, enable)

    def profile_read(self):
        return {k: lfm3_profile_read(self.ctx, v) for k, v in PROF_KINDS.items()}

    def dequant_rows(self, name, row0, n, f32=True, f16=True):
        t = self.torch
        k = None
        # K from the blob-side shape is not needed: the library knows it; ask via a probe size
        from .synth import tensor_plan
        for nm, kind, shape, bits, group in tensor_plan(self.cfg):
            if nm == name:
                k = shape[1]
        if k is None:
            raise LFM3Error(1, f"no quantized linear named {name}")
        of = self._empty((n, k), t.float32) if f32 else None
        ob = self._empty((n, k), t.float16) if f16 else None
        lfm3_dequant_rows(self.ctx, name, row0, n, of, ob)
        return of, ob


def bf16_to_f32(t):
    """int16 tensor of bf16 bit patterns -> float32 tensor (same device)."""
    import torch
    return (t.to(torch.int32) << 16).view(torch.float32)


def f32_to_bf16_bits(t):
    """float32 tensor -> int16 bf16 bit patterns (round to nearest even)."""
    import torch
    return t.to(torch.bfloat16).view(torch.int16)
