"""Python binding of libqdec (ctypes): argument marshalling only.

Every step of the forward pass runs in the HIP kernels of libqdec.so; this
module checks arguments, turns torch tensors into device pointers on the
current HIP stream, and maps status codes to exceptions.  Conventions follow
tessl `python/README.md`, "Handle ownership, closing and errors": a handle is
freed exactly once (idempotent ``close()``), copies and pickling are refused,
the handle is used from the thread that made it, status 1 raises ``QdecError``,
status 2 ``QdecPanic``, and a poisoned handle ``QdecPoisoned``.

``QDEC_LIB`` overrides the library path.  There is no fallback: without the
built library every call raises.
"""
import ctypes
import os
import threading

__all__ = ["Model", "QdecError", "QdecPanic", "QdecPoisoned", "lib", "config_struct",
           "debug_sample", "sample_noalloc", "debug_matmul", "gguf_config", "archdef_builtin", "T_F32", "T_Q4_0", "T_Q8_0", "ALL_LOGITS", "TOKENS_ON_DEVICE"]

T_F32, T_Q4_0, T_Q8_0 = 0, 2, 8
ALL_LOGITS, TOKENS_ON_DEVICE = 1, 2
_ACTS = {"silu": 0, "gelu_tanh": 1}
_I32 = (-(2 ** 31), 2 ** 31 - 1)
_U64 = (0, 2 ** 64 - 1)


class QdecError(RuntimeError):
    """Status 1: the library refused the call; nothing was enqueued."""


class QdecPanic(QdecError):
    """Status 2: an internal error caught at the library boundary."""


class QdecPoisoned(QdecError):
    """The handle latched after a GPU failure; free it and load again."""


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_layer", "hidden", "n_head", "n_head_kv", "head_dim", "ffn", "vocab")] + \
               [(n, ctypes.c_float) for n in ("rms_eps", "rope_theta", "rope_theta_local")] + \
               [(n, ctypes.c_int32) for n in ("window", "window_period", "qk_norm", "sandwich_norm", "act",
                                              "qkv_bias")]


class _Tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("type", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("host_data", ctypes.c_void_p), ("n_bytes", ctypes.c_int64)]


class _KStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("bytes", ctypes.c_double), ("flops", ctypes.c_double)]


_lib = None
_lib_lock = threading.Lock()


def lib_path():
    return os.environ.get("QDEC_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqdec.so")


def lib():
    """The loaded libqdec.so (raises if it has not been built)."""
    global _lib
    with _lib_lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise QdecError(f"libqdec.so not found at {path}: build it first "
                                "(python -m decoder_gguf_quantized_amd.build)")
            L = ctypes.CDLL(path)
            P, I32, I64, U32, U64, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                        ctypes.c_uint64, ctypes.c_float)
            sig = {
                "qdec_abi_version": (I32, []),
                "qdec_last_error": (ctypes.c_char_p, []),
                "qdec_load_weights": (ctypes.c_int, [ctypes.POINTER(_Config), ctypes.POINTER(_Tensor), I32, I32, I32, P,
                                                     ctypes.POINTER(P)]),
                "qdec_prefill": (ctypes.c_int, [P, I32, P, I32, P, P, U32, P]),
                "qdec_decode_step": (ctypes.c_int, [P, P, I32, P, P, F, F, U64, U64, U32, P]),
                "qdec_kv_reset": (ctypes.c_int, [P, I32]),
                "qdec_kv_truncate": (ctypes.c_int, [P, I32, I32]),
                "qdec_kv_write": (ctypes.c_int, [P, I32, I32, P, P, I32, P]),
                "qdec_kv_len": (ctypes.c_int, [P, I32, ctypes.POINTER(I32)]),
                "qdec_poisoned": (ctypes.c_int, [P]),
                "qdec_set_prefill_precision": (ctypes.c_int, [P, I32]),
                "qdec_free": (ctypes.c_int, [P]),
                "qdec_debug_dequant": (ctypes.c_int, [P, ctypes.c_char_p, P, P]),
                "qdec_debug_embed": (ctypes.c_int, [P, P, I32, P, P]),
                "qdec_debug_sample": (ctypes.c_int, [P, I32, I32, F, F, U64, U64, P, P]),
                "qdec_debug_matmul": (ctypes.c_int, [I32, I64, I64, P, I64, P, I32, P, I32, P]),
                "qdec_kernel_timing": (ctypes.c_int, [P, I32, ctypes.POINTER(_KStat), I32, ctypes.POINTER(I32)]),
                "qdec_gguf_config": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_char_p, ctypes.POINTER(_Config)]),
                "qdec_load_gguf": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_char_p, I32, I32, P, ctypes.POINTER(P)]),
                "qdec_archdef_builtin": (ctypes.c_char_p, [ctypes.c_char_p]),
                "qdec_decode_batch": (ctypes.c_int, [P, P, P, I32, P, P, F, F, U64, U64, U32, P]),
                "qdec_kv_paged": (ctypes.c_int, [P, I32, I32, P]),
                "qdec_kv_pages": (ctypes.c_int, [P, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32)]),
                "qdec_kv_ring": (ctypes.c_int, [P, I32, P]),
                "qdec_kv_ring_positions": (ctypes.c_int, [P, I32, ctypes.POINTER(I32)]),
                "qdec_decode_chunks": (ctypes.c_int, [P, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
                "qdec_debug_inject_fault": (ctypes.c_int, [P, I32]),
                "qdec_sample_noalloc": (ctypes.c_int, [P, I32, I32, F, F, U64, U64, P, P]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
        return _lib


def _last_error():
    msg = lib().qdec_last_error()
    return msg.decode() if msg else ""


def _int(name, v, lo_hi=_I32):
    if isinstance(v, bool) or not isinstance(v, int):
        try:
            import numpy as np
            if isinstance(v, np.integer):
                v = int(v)
            else:
                raise TypeError
        except (ImportError, TypeError):
            raise QdecError(f"{name} must be an integer, got {type(v).__name__}") from None
    if not lo_hi[0] <= v <= lo_hi[1]:
        raise QdecError(f"{name} = {v} outside [{lo_hi[0]}, {lo_hi[1]}]")
    return v


def _dev_ptr(name, t, dtype, min_numel):
    import torch
    if not isinstance(t, torch.Tensor):
        raise QdecError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise QdecError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise QdecError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise QdecError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise QdecError(f"{name} holds {t.numel()} elements, needs {min_numel}")
    end = (t.storage_offset() + t.numel()) * t.element_size()
    if end > t.untyped_storage().nbytes():
        raise QdecError(f"{name} view runs past its storage")
    return t.data_ptr()


def _stream():
    """The current HIP stream of torch, or the null stream when no GPU is
    visible (host-only runs against a stand-in library: QDEC_LIB)."""
    import torch
    if not torch.cuda.is_available():
        return None
    return torch.cuda.current_stream().cuda_stream


def config_struct(cfg):
    """qdec_config from a shape dict (the keys of synth.configs entries)."""
    c = _Config()
    for k in ("n_layer", "hidden", "n_head", "n_head_kv", "head_dim", "ffn", "vocab", "window", "window_period"):
        setattr(c, k, _int(k, int(cfg[k])))
    c.rms_eps = float(cfg["rms_eps"])
    c.rope_theta = float(cfg["rope_theta"])
    c.rope_theta_local = float(cfg.get("rope_theta_local", cfg["rope_theta"]))
    c.qk_norm = 1 if cfg["qk_norm"] else 0
    c.sandwich_norm = 1 if cfg["sandwich_norm"] else 0
    c.qkv_bias = 1 if cfg.get("qkv_bias") else 0
    act = cfg["act"]
    c.act = _ACTS[act] if isinstance(act, str) else int(act)
    return c


def _config_dict(c):
    d = {k: int(getattr(c, k)) for k in ("n_layer", "hidden", "n_head", "n_head_kv", "head_dim", "ffn", "vocab",
                                         "window", "window_period")}
    d.update(rms_eps=float(c.rms_eps), rope_theta=float(c.rope_theta), rope_theta_local=float(c.rope_theta_local),
             qk_norm=bool(c.qk_norm), sandwich_norm=bool(c.sandwich_norm), qkv_bias=bool(c.qkv_bias),
             act={v: k for k, v in _ACTS.items()}.get(int(c.act), int(c.act)))
    return d


def _path_arg(name, v):
    if isinstance(v, os.PathLike):
        v = os.fspath(v)
    if not isinstance(v, str):
        raise QdecError(f"{name} must be a path string")
    return v.encode()


def gguf_config(path, archdef=None):
    """The model shape a GGUF file and an architecture definition give (no GPU
    work): a dict with the keys of ``config_struct``.  ``archdef`` is the
    definition's text, or None for the library's built-in one for the file's
    architecture."""
    c = _Config()
    ad = None if archdef is None else str(archdef).encode()
    rc = lib().qdec_gguf_config(_path_arg("path", path), ad, ctypes.byref(c))
    if rc != 0:
        raise QdecError(_last_error())
    return _config_dict(c)


def archdef_builtin(arch):
    """Text of the library's built-in definition of ``arch``, or None."""
    t = lib().qdec_archdef_builtin(str(arch).encode())
    return t.decode() if t else None


class Model:
    """One loaded model (a libqdec handle).  ``tensors`` maps GGUF names to
    records with ``type``, ``rows``, ``cols`` and ``data`` (raw bytes as a
    uint8 numpy array)."""

    def __init__(self, cfg, tensors, max_seqs=1, max_ctx=4096):
        import numpy as np
        self._h = None
        self._thread = threading.get_ident()
        self.cfg = dict(cfg)
        self.vocab = int(cfg["vocab"])
        self.max_seqs = _int("max_seqs", max_seqs)
        self.max_ctx = _int("max_ctx", max_ctx)
        recs = list(tensors.values()) if isinstance(tensors, dict) else list(tensors)
        arr = (_Tensor * len(recs))()
        keep = []
        for i, t in enumerate(recs):
            data = np.ascontiguousarray(np.asarray(t.data, dtype=np.uint8))
            keep.append(data)
            name = t.name.encode()
            keep.append(name)
            arr[i] = _Tensor(name, _int("type", int(t.type)), _int("rows", int(t.rows), (0, 2 ** 62)),
                             _int("cols", int(t.cols), (0, 2 ** 62)), data.ctypes.data, data.nbytes)
        h = ctypes.c_void_p()
        rc = lib().qdec_load_weights(ctypes.byref(config_struct(cfg)), arr, len(recs), self.max_seqs, self.max_ctx,
                                     _stream(), ctypes.byref(h))
        del keep
        if rc == 1:
            raise QdecError(_last_error())
        if rc != 0:
            raise QdecPanic(_last_error())
        self._h = h

    @classmethod
    def from_gguf(cls, path, archdef=None, max_seqs=1, max_ctx=4096):
        """Load a GGUF file; the block layout comes from ``archdef`` (text) or the
        library's built-in definition for the file's architecture."""
        cfg = gguf_config(path, archdef)
        m = cls.__new__(cls)
        m._h = None
        m._thread = threading.get_ident()
        m.cfg = cfg
        m.vocab = cfg["vocab"]
        m.max_seqs = _int("max_seqs", max_seqs)
        m.max_ctx = _int("max_ctx", max_ctx)
        h = ctypes.c_void_p()
        ad = None if archdef is None else str(archdef).encode()
        rc = lib().qdec_load_gguf(_path_arg("path", path), ad, m.max_seqs, m.max_ctx, _stream(), ctypes.byref(h))
        if rc == 1:
            raise QdecError(_last_error())
        if rc != 0:
            raise QdecPanic(_last_error())
        m._h = h
        return m

    # ------------------------------------------------------------ ownership
    def __copy__(self):
        raise TypeError("a qdec Model owns a library handle and cannot be copied")

    def __deepcopy__(self, memo):
        raise TypeError("a qdec Model owns a library handle and cannot be copied")

    def __reduce__(self):
        raise TypeError("a qdec Model cannot be pickled")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            if self._h is not None and threading.get_ident() == self._thread:
                lib().qdec_free(self._h)
                self._h = None
        except Exception:
            pass

    @property
    def closed(self):
        return self._h is None

    def close(self):
        """Free the handle (idempotent)."""
        if self._h is None:
            return
        if threading.get_ident() != self._thread:
            self._h = None
            raise QdecError("close() from another thread: the handle is leaked, not freed")
        h, self._h = self._h, None
        rc = lib().qdec_free(h)
        if rc != 0:
            raise QdecPanic(_last_error())

    def _handle(self):
        if self._h is None:
            raise QdecError("model is closed")
        if threading.get_ident() != self._thread:
            raise QdecError("a model is used from the thread that created it")
        return self._h

    def _check(self, rc):
        if rc == 0:
            return
        msg = _last_error()
        if lib().qdec_poisoned(self._h) == 1:
            h, self._h = self._h, None
            lib().qdec_free(h)
            raise QdecPoisoned(msg)
        if rc == 1:
            raise QdecError(msg)
        raise QdecPanic(msg)

    # ------------------------------------------------------------ forward
    def prefill(self, seq, tokens, logits, token_out=None, all_logits=False):
        """Append host token ids to sequence ``seq``; logits f32 on the GPU
        ([vocab], or [n][vocab] with all_logits)."""
        import numpy as np
        import torch
        h = self._handle()
        toks = np.ascontiguousarray(np.asarray(tokens.cpu() if isinstance(tokens, torch.Tensor) else tokens,
                                               dtype=np.int64))
        if toks.ndim != 1:
            raise QdecError("tokens must be 1-D")
        if toks.size and (toks.min() < _I32[0] or toks.max() > _I32[1]):
            raise QdecError("token ids must fit int32")
        toks = toks.astype(np.int32)
        n = toks.size
        lp = _dev_ptr("logits", logits, torch.float32, (n if all_logits else 1) * self.vocab)
        tp = _dev_ptr("token_out", token_out, torch.int32, 1) if token_out is not None else None
        rc = lib().qdec_prefill(h, _int("seq", seq), toks.ctypes.data, _int("n_tokens", n), lp, tp,
                                ALL_LOGITS if all_logits else 0, _stream())
        self._check(rc)

    def decode_step(self, tokens, logits, token_out, temperature=0.0, seed=0, step=0, top_p=1.0):
        """One token for each of sequences 0..B-1.  ``tokens``: host ids, or an
        int32 GPU tensor (e.g. the previous ``token_out``).  ``top_p`` < 1 with
        ``temperature`` > 0 samples from the nucleus."""
        self._decode(None, tokens, logits, token_out, temperature, seed, step, top_p)

    def decode_batch(self, seqs, tokens, logits, token_out, temperature=0.0, seed=0, step=0, top_p=1.0):
        """One token for each sequence slot in ``seqs`` (distinct host ints): row
        r of ``tokens`` / ``logits`` / ``token_out`` serves sequence seqs[r]."""
        import numpy as np
        sq = np.ascontiguousarray(np.asarray([_int("seq", int(x)) for x in seqs], dtype=np.int32))
        self._decode(sq, tokens, logits, token_out, temperature, seed, step, top_p)

    def _decode(self, seqs, tokens, logits, token_out, temperature, seed, step, top_p):
        import numpy as np
        import torch
        h = self._handle()
        if isinstance(tokens, torch.Tensor) and tokens.device.type == "cuda":
            n = tokens.numel()
            tp_in = _dev_ptr("tokens", tokens, torch.int32, n)
            flags = TOKENS_ON_DEVICE
            keep = None
        else:
            keep = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
            if keep.size and (keep.min() < _I32[0] or keep.max() > _I32[1]):
                raise QdecError("token ids must fit int32")
            keep = keep.astype(np.int32).reshape(-1)
            n = keep.size
            tp_in = keep.ctypes.data
            flags = 0
        lp = _dev_ptr("logits", logits, torch.float32, n * self.vocab)
        op = _dev_ptr("token_out", token_out, torch.int32, n)
        args = (lp, op, float(temperature), float(top_p), _int("seed", seed, _U64), _int("step", step, _U64), flags,
                _stream())
        if seqs is None:
            rc = lib().qdec_decode_step(h, tp_in, _int("n_seqs", n), *args)
        else:
            if seqs.size != n:
                raise QdecError(f"{seqs.size} sequence slots for {n} tokens")
            rc = lib().qdec_decode_batch(h, seqs.ctypes.data, tp_in, _int("n", n), *args)
        self._check(rc)

    def kv_paged(self, page_size, n_pages):
        """Switch to a paged KV cache: a pool of ``n_pages`` pages of
        ``page_size`` positions shared by all sequences (every sequence empty)."""
        self._check(lib().qdec_kv_paged(self._handle(), _int("page_size", page_size), _int("n_pages", n_pages),
                                        _stream()))

    def kv_ring(self, enable):
        """Sliding-window layers keep a ring of their last positions (True, the
        state after load) or every position (False); every sequence empty."""
        self._check(lib().qdec_kv_ring(self._handle(), 1 if enable else 0, _stream()))

    def kv_ring_positions(self, layer):
        """Positions of ``layer``'s ring, 0 when it keeps max_ctx positions."""
        out = ctypes.c_int32()
        self._check(lib().qdec_kv_ring_positions(self._handle(), _int("layer", layer), ctypes.byref(out)))
        return out.value

    def kv_pages(self):
        """(page_size, n_pages, n_free); page_size 0 = contiguous cache."""
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._check(lib().qdec_kv_pages(self._handle(), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
        return a.value, b.value, c.value

    def set_prefill_precision(self, precision):
        """Operand precision of later prefill projections: "f32" (default),
        "bf16x3" (exact three-term bf16 split of the activations) or "bf16"."""
        self._check(lib().qdec_set_prefill_precision(self._handle(), _precision(precision)))

    def kv_reset(self, seq=-1):
        self._check(lib().qdec_kv_reset(self._handle(), _int("seq", seq)))

    def kv_truncate(self, seq, n):
        """Roll sequence ``seq`` back to its first ``n`` positions."""
        self._check(lib().qdec_kv_truncate(self._handle(), _int("seq", seq), _int("n", n)))

    def kv_write(self, seq, layer, k, v):
        """Install preset post-RoPE K, V (f32 GPU tensors [n_kv][n_pos][head_dim])."""
        import torch
        h = self._handle()
        if k.shape != v.shape or k.dim() != 3:
            raise QdecError("k and v must both be [n_kv][n_pos][head_dim]")
        n_pos = k.shape[1]
        kp = _dev_ptr("k", k, torch.float32, k.numel())
        vp = _dev_ptr("v", v, torch.float32, v.numel())
        self._check(lib().qdec_kv_write(h, _int("seq", seq), _int("layer", layer), kp, vp, _int("n_pos", n_pos),
                                        _stream()))

    def decode_chunks(self):
        """(positions per decode-attention chunk, chunks per sequence and KV head)."""
        a, b = ctypes.c_int32(), ctypes.c_int32()
        self._check(lib().qdec_decode_chunks(self._handle(), ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def debug_inject_fault(self, armed=True):
        """Arm (or disarm) a synthetic HIP error on the next kernel launch of a
        call: that call then fails with status 2 and poisons the handle."""
        self._check(lib().qdec_debug_inject_fault(self._handle(), 1 if armed else 0))

    def kv_len(self, seq):
        out = ctypes.c_int32()
        self._check(lib().qdec_kv_len(self._handle(), _int("seq", seq), ctypes.byref(out)))
        return out.value

    @property
    def poisoned(self):
        return self._h is not None and lib().qdec_poisoned(self._h) == 1

    # ------------------------------------------------------------ tests and measurement
    def debug_dequant(self, name, out):
        import torch
        self._check(lib().qdec_debug_dequant(self._handle(), name.encode(), _dev_ptr("out", out, torch.float32, 1),
                                             _stream()))

    def debug_embed(self, tokens, out):
        import torch
        n = tokens.numel()
        self._check(lib().qdec_debug_embed(self._handle(), _dev_ptr("tokens", tokens, torch.int32, n), _int("n", n),
                                           _dev_ptr("out", out, torch.float32, n * int(self.cfg["hidden"])),
                                           _stream()))

    def kernel_timing(self, enable):
        """Start (True) or stop (False) per-kernel event timing; stopping returns
        {class: {launches, ms, bytes, flops}}."""
        h = self._handle()
        if enable:
            self._check(lib().qdec_kernel_timing(h, 1, None, 0, None))
            return None
        buf = (_KStat * 64)()
        n = ctypes.c_int32()
        self._check(lib().qdec_kernel_timing(h, 0, buf, 64, ctypes.byref(n)))
        return {buf[i].name.decode(): dict(launches=buf[i].launches, ms=buf[i].total_ms, bytes=buf[i].bytes,
                                           flops=buf[i].flops) for i in range(n.value)}


def debug_sample(logits, temperature, seed, step, out, top_p=1.0):
    """Row-wise token choice with the decode step's rule; logits [rows][vocab]."""
    import torch
    rows, vocab = logits.shape
    rc = lib().qdec_debug_sample(_dev_ptr("logits", logits, torch.float32, rows * vocab), _int("rows", rows),
                                 _int("vocab", vocab), float(temperature), float(top_p), _int("seed", seed, _U64),
                                 _int("step", step, _U64), _dev_ptr("out", out, torch.int32, rows), _stream())
    if rc:
        raise (QdecError if rc == 1 else QdecPanic)(_last_error())


def sample_noalloc(logits, temperature, seed, step, out, top_p=1.0):
    """debug_sample's rule through the allocation-free entry point (partials in
    the library's fixed device scratch; rows <= 64, vocab <= 2^20; no host
    wait)."""
    import torch
    rows, vocab = logits.shape
    rc = lib().qdec_sample_noalloc(_dev_ptr("logits", logits, torch.float32, rows * vocab), _int("rows", rows),
                                   _int("vocab", vocab), float(temperature), float(top_p), _int("seed", seed, _U64),
                                   _int("step", step, _U64), _dev_ptr("out", out, torch.int32, rows), _stream())
    if rc:
        raise (QdecError if rc == 1 else QdecPanic)(_last_error())


PREFILL_PRECISIONS = {"f32": 0, "bf16x3": 1, "bf16": 2}


def _precision(name):
    if name not in PREFILL_PRECISIONS:
        raise QdecError(f"prefill precision must be one of {sorted(PREFILL_PRECISIONS)}, got {name!r}")
    return PREFILL_PRECISIONS[name]


def debug_matmul(ttype, rows, cols, raw, x, y, precision="f32"):
    """y[r] = W x[r] with the forward pass's projection kernels (GEMV for <= 16
    rows, MFMA GEMM above, operands in ``precision``); W given as GGUF bytes."""
    import numpy as np
    import torch
    raw = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8))
    n = x.shape[0]
    kp = ((cols + 31) // 32) * 32
    rc = lib().qdec_debug_matmul(_int("type", ttype), rows, cols, raw.ctypes.data, raw.nbytes,
                                 _dev_ptr("x", x, torch.float32, n * kp), _int("n_x", n),
                                 _dev_ptr("y", y, torch.float32, n * rows), _precision(precision), _stream())
    if rc:
        raise (QdecError if rc == 1 else QdecPanic)(_last_error())
