"""ctypes binding of libzimg_dit.so (include/zimg_dit.h, include/zimg_ops.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  Device buffers are torch CUDA tensors (PyTorch provides device
memory and streams); host arrays are numpy.  The library must have been
built (``python -m diffusion_transformer_image_amd.build``); loading fails
loudly otherwise -- there is no fallback path.
"""

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzimg_dit.so")

ZIMG_OK = 0
ZIMG_EINVAL = -1
ZIMG_EWEIGHT = -2
ZIMG_EUNSUPPORTED = -3
ZIMG_ENOMEM = -4
ZIMG_EHIP = -5
ZIMG_ESTATE = -6
ZIMG_ENONFINITE = -7
ZIMG_F32 = 0
ZIMG_BF16 = 1
EPI_BF16 = 0
EPI_F32_BIAS = 1
EPI_SWIGLU = 2

_CODES = {ZIMG_EINVAL: "EINVAL", ZIMG_EWEIGHT: "EWEIGHT", ZIMG_EUNSUPPORTED: "EUNSUPPORTED",
          ZIMG_ENOMEM: "ENOMEM", ZIMG_EHIP: "EHIP", ZIMG_ESTATE: "ESTATE",
          ZIMG_ENONFINITE: "ENONFINITE"}


class ZimgError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"zimg error {_CODES.get(code, code)}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("n_layers", ctypes.c_int32), ("n_noise_refiner", ctypes.c_int32),
        ("n_context_refiner", ctypes.c_int32), ("in_channels", ctypes.c_int32),
        ("patch", ctypes.c_int32), ("cap_feat_dim", ctypes.c_int32), ("adaln_dim", ctypes.c_int32),
        ("t_mid", ctypes.c_int32), ("rope_axes", ctypes.c_int32 * 3), ("rope_theta", ctypes.c_float),
        ("t_scale", ctypes.c_float), ("max_period", ctypes.c_float), ("norm_eps", ctypes.c_float),
        ("final_eps", ctypes.c_float), ("max_batch", ctypes.c_int32),
        ("max_image_tokens", ctypes.c_int32), ("max_caption_tokens", ctypes.c_int32),
        ("batch_invariant", ctypes.c_int32), ("linear_int8", ctypes.c_int32), ("token_pad", ctypes.c_int32),
        ("check_finite", ctypes.c_int32),
    ]

    def as_dict(self):
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["rope_axes"] = tuple(self.rope_axes)
        return d


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class Tensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("shape", ctypes.c_int64 * 4)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_I32P = ctypes.POINTER(ctypes.c_int32)
_F32P = ctypes.POINTER(ctypes.c_float)

# name -> (restype, argtypes); the exported C ABI
SIGNATURES = {
    "zimg_last_error": (ctypes.c_char_p, []),
    "zimg_dit_default_config": (None, [ctypes.POINTER(Config)]),
    "zimg_dit_check_config": (_I32, [ctypes.POINTER(Config)]),
    "zimg_dit_manifest_size": (_I32, [ctypes.POINTER(Config), _I32P]),
    "zimg_dit_manifest_entry": (_I32, [ctypes.POINTER(Config), _I32, ctypes.POINTER(ctypes.c_char_p), _I32P,
                                       ctypes.POINTER(ctypes.c_int64)]),
    "zimg_dit_create": (_I32, [ctypes.POINTER(Config), ctypes.POINTER(Tensor), _I32, _P, ctypes.POINTER(_P)]),
    "zimg_dit_alloc": (_I32, [ctypes.POINTER(Config), _P, ctypes.POINTER(_P)]),
    "zimg_dit_set_weight": (_I32, [_P, ctypes.POINTER(Tensor)]),
    "zimg_dit_finalize": (_I32, [_P]),
    "zimg_dit_forward": (_I32, [_P, _P, _I32, _I32, _I32, _P, _I32, _I32P, _F32P, _P, _P]),
    "zimg_dit_destroy": (None, [_P]),
    "zimg_safetensors_check": (_I32, [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_char_p), _I32, _I32P]),
    "zimg_dit_load_safetensors": (_I32, [_P, ctypes.POINTER(ctypes.c_char_p), _I32]),
    "zimg_dit_create_from_safetensors": (_I32, [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_char_p), _I32, _P,
                                                ctypes.POINTER(_P)]),
    "zimg_dit_manifest_digest": (_I32, [ctypes.POINTER(Config), ctypes.c_char_p]),
    "zimg_dit_last_error": (ctypes.c_char_p, [_P]),
    "zimg_dit_set_capture": (_I32, [_P, _P, ctypes.c_size_t]),
    "zimg_position_ids": (_I32, [_I32, _I32, _I32, _I32P, _I32P]),
    "zimg_rope_tables": (_I32, [ctypes.POINTER(Config), _I32P, _I64, _F32P, _F32P]),
    "zimg_row_layout": (_I32, [_I32, _I32, _I32P, _I32P, _I32P, _I32P]),
    "zimg_row_layout_varsize": (_I32, [_I32, _I32P, _I32P, _I32P, _I32P, _I32P]),
    "zimg_dit_forward_varsize": (_I32, [_P, _P, _I32, _I32P, _I32P, _P, _I32, _I32P, _F32P, _P, _P]),
    "zimg_dit_run_blocks": (_I32, [_P, _P, _I32, _I32, _I32, _I32P, _F32P, _I32, _I32, _P]),
    "zimg_gemm_bf16": (_I32, [_P, _I64, _P, _I64, _P, _I64, _I32, _I32, _I32, _I32, _P, _P]),
    "zimg_gemm_i8": (_I32, [_P, _I64, _P, _P, _I64, _P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P]),
    "zimg_quantize_rows": (_I32, [_P, _I32, _I64, _P, _I64, _P, _I32, _I32, _I32, _P]),
    "zimg_euler_step": (_I32, [_P, _P, ctypes.c_float, _I64, _P]),
    "zimg_flowmatch_schedule": (_I32, [_I32, ctypes.c_double, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)]),
    "zimg_cfg_euler_step": (_I32, [_P, _P, _P, ctypes.c_float, ctypes.c_float, _I64, _P]),
    "zimg_dit_profile": (_I32, [_P, _I32]),
    "zimg_dit_profile_read": (_I32, [_P, ctypes.POINTER(KernelStat), _I32, _I32P]),
    "zimg_dit_attention_plan": (_I32, [_P, _I32, _I32P]),
    "zimg_attention_workspace_size": (_I32, [_I32, _I32, _I32P, _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "zimg_attention": (_I32, [_P, _P, _I64, _P, _I32, _I32, _I32P, _P, ctypes.c_size_t, _P]),
    "zimg_attention_noalloc": (_I32, [_P, _P, _I64, _P, _I32, _I32, _I32P, _P]),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m diffusion_transformer_image_amd.build` (there is no fallback)")
        # One HIP runtime per process: PyTorch ships its own libamdhip64 (same
        # soname as the one the library is linked against).  Loaded first, it
        # is the one the library's dependency resolves to; loaded second, a
        # second runtime would come up beside the library's and, on some
        # hosts, find no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc, handle=None):
    if rc != ZIMG_OK:
        msg = lib().zimg_last_error().decode()
        if not msg and handle:
            msg = lib().zimg_dit_last_error(handle).decode()
        raise ZimgError(rc, msg)


def config(**overrides):
    c = Config()
    lib().zimg_dit_default_config(ctypes.byref(c))
    for k, v in overrides.items():
        if k == "rope_axes":
            c.rope_axes = (ctypes.c_int32 * 3)(*v)
        elif k in dict(Config._fields_):
            setattr(c, k, v)
        else:
            raise KeyError(f"unknown config field {k}")
    return c


def check_config(cfg):
    _check(lib().zimg_dit_check_config(ctypes.byref(cfg)))


def manifest(cfg):
    """[(name, shape)] the engine expects, in canonical order."""
    n = ctypes.c_int32()
    _check(lib().zimg_dit_manifest_size(ctypes.byref(cfg), ctypes.byref(n)))
    out = []
    for i in range(n.value):
        name = ctypes.c_char_p()
        nd = ctypes.c_int32()
        shp = (ctypes.c_int64 * 4)()
        _check(lib().zimg_dit_manifest_entry(ctypes.byref(cfg), i, ctypes.byref(name), ctypes.byref(nd), shp))
        out.append((name.value.decode(), tuple(shp[:nd.value])))
    return out


def _paths(paths):
    if isinstance(paths, (str, bytes, os.PathLike)):
        paths = [paths]
    enc = [os.fsencode(p) for p in paths]
    return (ctypes.c_char_p * len(enc))(*enc), len(enc)


def safetensors_check(cfg, paths):
    """Validate safetensors files against the config's weight table
    (zimg_safetensors_check); returns the tensor count."""
    arr, n = _paths(paths)
    cnt = ctypes.c_int32()
    _check(lib().zimg_safetensors_check(ctypes.byref(cfg), arr, n, ctypes.byref(cnt)))
    return cnt.value


def manifest_digest(cfg):
    """SHA-256 of the sorted weight names (zimg_dit_manifest_digest)."""
    buf = ctypes.create_string_buffer(65)
    _check(lib().zimg_dit_manifest_digest(ctypes.byref(cfg), buf))
    return buf.value.decode()


def _tensor(name, arr):
    """Tensor descriptor for a host numpy array (float32 or uint16 bf16 bits)."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.float32:
        dt = ZIMG_F32
    elif a.dtype == np.uint16:
        dt = ZIMG_BF16
    else:
        raise TypeError(f"{name}: weights must be float32 or uint16 bf16 bits, got {a.dtype}")
    t = Tensor()
    t.name = name.encode()
    t.data = a.ctypes.data
    t.dtype = dt
    t.ndim = a.ndim
    for i, s in enumerate(a.shape):
        t.shape[i] = s
    return t, a


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _want(t, name, dtypes, ndim=None, contiguous=False):
    """Refuse, before any native call, a tensor the entry point cannot read:
    not a CUDA tensor, another dtype or rank, or rows that are not unit-stride
    (or, with ``contiguous``, not one dense block)."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: a torch CUDA tensor is required")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} is not one of {tuple(str(d) for d in dtypes)}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: a {ndim}-d tensor is required, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: a contiguous tensor is required")
    if t.dim() >= 1 and t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name}: rows must be unit-stride")


def _f32():
    import torch
    return (torch.float32,)


def _per_sample(caption_lens, t, B):
    """Host arrays of one caption length and one model time per sample; the
    library reads exactly B of each, so shorter (or longer) sequences are
    refused here."""
    lens = np.ascontiguousarray(caption_lens, dtype=np.int32).reshape(-1)
    tt = np.ascontiguousarray(t, dtype=np.float32).reshape(-1)
    if lens.size != B:
        raise ValueError(f"caption_lens: {B} lengths required (one per sample), got {lens.size}")
    if tt.size != B:
        raise ValueError(f"t: {B} model times required (one per sample), got {tt.size}")
    return lens, tt


def _check_captions(caption_feats, lens, cap_dim):
    """Packed caption rows: cap_feat_dim wide and at least as many rows as
    the lengths add up to (the library reads exactly that many)."""
    need = int(np.clip(lens.astype(np.int64), 0, None).sum())
    if caption_feats.shape[1] != cap_dim or caption_feats.shape[0] < need:
        raise ValueError(f"caption_feats must be [>= {need}, {cap_dim}] (the captions packed back to back), "
                         f"got {list(caption_feats.shape)}")


def _f32_bf16():
    import torch
    return (torch.float32, torch.bfloat16)


class DiT:
    """Handle of one engine instance (device weights + workspace)."""

    def __init__(self, cfg, weights, stream=None):
        """``weights``: iterable of (name, numpy array) or a mapping.  The
        set-up work runs on ``stream`` (default: torch's current stream)."""
        self.cfg = cfg
        self._h = ctypes.c_void_p()
        _check(lib().zimg_dit_alloc(ctypes.byref(cfg), _stream(stream), ctypes.byref(self._h)))
        try:
            items = weights.items() if hasattr(weights, "items") else weights
            for name, arr in items:
                t, keep = _tensor(name, arr)
                _check(lib().zimg_dit_set_weight(self._h, ctypes.byref(t)), self._h)
                del keep
            _check(lib().zimg_dit_finalize(self._h), self._h)
        except Exception:
            self.close()
            raise
        self._capture = None

    @classmethod
    def from_safetensors(cls, cfg, paths, stream=None):
        """An engine whose weights come from safetensors files
        (zimg_dit_create_from_safetensors)."""
        self = cls.__new__(cls)
        self.cfg = cfg
        self._h = ctypes.c_void_p()
        self._capture = None
        arr, n = _paths(paths)
        _check(lib().zimg_dit_create_from_safetensors(ctypes.byref(cfg), arr, n, _stream(stream), ctypes.byref(self._h)))
        return self

    def close(self):
        if self._h:
            lib().zimg_dit_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def n_blocks(self):
        c = self.cfg
        return c.n_layers + c.n_noise_refiner + c.n_context_refiner

    def forward(self, latent, caption_feats, caption_lens, t, out, stream=None):
        """latent, caption_feats, out: torch CUDA tensors (fp32 latent/out,
        fp32 or bf16 packed captions); caption_lens, t: host sequences."""
        import torch
        _want(latent, "latent", _f32(), 4, contiguous=True)
        _want(out, "out", _f32(), 4, contiguous=True)
        _want(caption_feats, "caption_feats", _f32_bf16(), 2, contiguous=True)
        if out.shape != latent.shape:
            raise ValueError("out must have the latent's shape")
        B, C, Hl, Wl = latent.shape
        if C != self.cfg.in_channels:
            raise ValueError(f"latent: {self.cfg.in_channels} channels required, got {C}")
        lens, tt = _per_sample(caption_lens, t, B)
        _check_captions(caption_feats, lens, self.cfg.cap_feat_dim)
        cap_dt = ZIMG_BF16 if caption_feats.dtype == torch.bfloat16 else ZIMG_F32
        _check(lib().zimg_dit_forward(self._h, _ptr(latent), B, Hl, Wl, _ptr(caption_feats), cap_dt,
                                      lens.ctypes.data_as(_I32P), tt.ctypes.data_as(_F32P), _ptr(out),
                                      _stream(stream)), self._h)
        return out

    def forward_varsize(self, latents, caption_feats, caption_lens, t, outs, stream=None):
        """latents, outs: sequences of torch CUDA fp32 tensors [C, Hl_b, Wl_b]
        (samples may differ in size); caption_feats packed as for forward."""
        import torch
        B = len(latents)
        if len(outs) != B:
            raise ValueError("one output per latent")
        hl = np.ascontiguousarray([x.shape[-2] for x in latents], dtype=np.int32)
        wl = np.ascontiguousarray([x.shape[-1] for x in latents], dtype=np.int32)
        for x, o in zip(latents, outs):
            _want(x, "latents", _f32(), contiguous=True)
            _want(o, "outs", _f32(), contiguous=True)
            shp = tuple(x.shape)
            if len(shp) == 4 and shp[0] == 1:
                shp = shp[1:]
            if len(shp) != 3 or shp[0] != self.cfg.in_channels:
                raise ValueError(f"latents: [{self.cfg.in_channels}, Hl, Wl] per sample required, got {list(x.shape)}")
            if o.numel() != x.numel() or tuple(o.shape[-3:]) != tuple(x.shape[-3:]):
                raise ValueError("latents and outs: contiguous fp32 tensors of matching shapes")
        _want(caption_feats, "caption_feats", _f32_bf16(), 2, contiguous=True)
        lens, tt = _per_sample(caption_lens, t, B)
        _check_captions(caption_feats, lens, self.cfg.cap_feat_dim)
        lp = (ctypes.c_void_p * B)(*[x.data_ptr() for x in latents])
        op = (ctypes.c_void_p * B)(*[o.data_ptr() for o in outs])
        cap_dt = ZIMG_BF16 if caption_feats.dtype == torch.bfloat16 else ZIMG_F32
        _check(lib().zimg_dit_forward_varsize(self._h, lp, B, hl.ctypes.data_as(_I32P), wl.ctypes.data_as(_I32P),
                                              _ptr(caption_feats), cap_dt, lens.ctypes.data_as(_I32P),
                                              tt.ctypes.data_as(_F32P), op, _stream(stream)), self._h)
        return outs

    def run_blocks(self, x, B, Hl, Wl, caption_lens, t, first, n, stream=None):
        """Blocks [first, first + n) in place on the fp32 residual x (torch
        CUDA, [S_total, hidden] in the engine's row layout)."""
        _want(x, "x", _f32(), contiguous=True)
        lens, tt = _per_sample(caption_lens, t, B)
        p = self.cfg.patch
        if Hl % p or Wl % p or Hl <= 0 or Wl <= 0:
            raise ValueError(f"Hl and Wl must be positive multiples of {p}, got {Hl} x {Wl}")
        _, _, S = row_layout(B, (Hl // p) * (Wl // p), lens)
        if x.numel() != S * self.cfg.hidden:
            raise ValueError(f"x: {S} x {self.cfg.hidden} values required (the row layout of this batch), "
                             f"got {x.numel()}")
        _check(lib().zimg_dit_run_blocks(self._h, _ptr(x), B, Hl, Wl, lens.ctypes.data_as(_I32P),
                                         tt.ctypes.data_as(_F32P), first, n, _stream(stream)), self._h)
        return x

    def profile(self, enable):
        """Start (reset) or stop per-kernel-class event timing."""
        _check(lib().zimg_dit_profile(self._h, 1 if enable else 0), self._h)

    def profile_read(self):
        """{class name: (launches, total_ms)} accumulated since profile(True)."""
        stats = (KernelStat * 32)()
        n = ctypes.c_int32()
        _check(lib().zimg_dit_profile_read(self._h, stats, 32, ctypes.byref(n)), self._h)
        return {stats[i].name.decode(): (stats[i].launches, stats[i].total_ms) for i in range(min(n.value, 32))}

    def attention_plan(self, stage):
        """(pairs, pairs computed whole, chunks per split pair) of a stage at
        the geometry of the last forward / run_blocks call."""
        out = (ctypes.c_int32 * 3)()
        _check(lib().zimg_dit_attention_plan(self._h, stage, out), self._h)
        return tuple(out)

    def set_capture(self, buf):
        """buf: torch CUDA fp32 tensor or None."""
        self._capture = buf
        if buf is None:
            _check(lib().zimg_dit_set_capture(self._h, None, 0), self._h)
        else:
            _check(lib().zimg_dit_set_capture(self._h, _ptr(buf), buf.numel() * 4), self._h)


def row_layout(B, n_image_tokens, caption_lens):
    lens = np.ascontiguousarray(caption_lens, dtype=np.int32)
    img = np.zeros(B, np.int32)
    cap = np.zeros(B, np.int32)
    S = ctypes.c_int32()
    _check(lib().zimg_row_layout(B, n_image_tokens, lens.ctypes.data_as(_I32P), img.ctypes.data_as(_I32P),
                                 cap.ctypes.data_as(_I32P), ctypes.byref(S)))
    return img, cap, S.value


def row_layout_varsize(n_image_tokens, caption_lens):
    n = np.ascontiguousarray(n_image_tokens, dtype=np.int32)
    lens = np.ascontiguousarray(caption_lens, dtype=np.int32)
    B = len(n)
    img = np.zeros(B, np.int32)
    cap = np.zeros(B, np.int32)
    S = ctypes.c_int32()
    _check(lib().zimg_row_layout_varsize(B, n.ctypes.data_as(_I32P), lens.ctypes.data_as(_I32P),
                                         img.ctypes.data_as(_I32P), cap.ctypes.data_as(_I32P), ctypes.byref(S)))
    return img, cap, S.value


def position_ids(L, Hp, Wp):
    cap = np.zeros((L, 3), np.int32)
    img = np.zeros((Hp * Wp, 3), np.int32)
    _check(lib().zimg_position_ids(L, Hp, Wp, cap.ctypes.data_as(_I32P), img.ctypes.data_as(_I32P)))
    return cap, img


def rope_tables(cfg, ids):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    S = ids.shape[0]
    cs = np.zeros((S, 64), np.float32)
    sn = np.zeros((S, 64), np.float32)
    _check(lib().zimg_rope_tables(ctypes.byref(cfg), ids.ctypes.data_as(_I32P), S, cs.ctypes.data_as(_F32P),
                                  sn.ctypes.data_as(_F32P)))
    return cs, sn


def _gemm_out_checks(A, W, C, epilogue, bias):
    import torch
    if A.shape[1] != W.shape[1]:
        raise ValueError(f"A and W disagree on K: {tuple(A.shape)} vs {tuple(W.shape)}")
    out_dt = (torch.float32,) if epilogue == EPI_F32_BIAS else (torch.bfloat16,)
    _want(C, "C", out_dt, 2)
    n_out = W.shape[0] // 2 if epilogue == EPI_SWIGLU else W.shape[0]
    if C.shape[0] != A.shape[0] or C.shape[1] != n_out:
        raise ValueError(f"C must be [{A.shape[0]}, {n_out}], got {tuple(C.shape)}")
    if bias is not None:
        _want(bias, "bias", _f32(), 1, contiguous=True)
        if bias.numel() != W.shape[0]:
            raise ValueError("bias: one value per output column")


def gemm_bf16(A, W, C, epilogue=EPI_BF16, bias=None, stream=None):
    """C = epilogue(A W^T) on torch CUDA tensors (A, W bf16; C bf16 or fp32)."""
    import torch
    _want(A, "A", (torch.bfloat16,), 2)
    _want(W, "W", (torch.bfloat16,), 2)
    _gemm_out_checks(A, W, C, epilogue, bias)
    M, K = A.shape
    N = W.shape[0]
    _check(lib().zimg_gemm_bf16(_ptr(A), A.stride(0), _ptr(W), W.stride(0), _ptr(C), C.stride(0), M, N, K,
                                epilogue, _ptr(bias) if bias is not None else None, _stream(stream)))
    return C


def gemm_i8(A, sa, W, sw, C, epilogue=EPI_BF16, bias=None, stream=None):
    """C = epilogue((A W^T) * sa[:, None] * sw[None, :]) on torch CUDA tensors
    (A, W int8 codes; sa, sw fp32 row scales; C bf16 or fp32)."""
    import torch
    _want(A, "A", (torch.int8,), 2)
    _want(W, "W", (torch.int8,), 2)
    _want(sa, "sa", _f32(), 1, contiguous=True)
    _want(sw, "sw", _f32(), 1, contiguous=True)
    if sa.numel() != A.shape[0] or sw.numel() != W.shape[0]:
        raise ValueError("sa and sw: one scale per row of A and of W")
    _gemm_out_checks(A, W, C, epilogue, bias)
    M, K = A.shape
    N = W.shape[0]
    _check(lib().zimg_gemm_i8(_ptr(A), A.stride(0), _ptr(sa), _ptr(W), W.stride(0), _ptr(sw), _ptr(C), C.stride(0),
                              M, N, K, epilogue, _ptr(bias) if bias is not None else None, _stream(stream)))
    return C


def quantize_rows(x, q, scale, rotate_block=0, stream=None):
    """Per-row int8 codes q and scales of x (torch CUDA fp32 or bf16 rows),
    after a 128-point Walsh-Hadamard rotation when rotate_block is 128."""
    import torch
    if isinstance(x, torch.Tensor) and x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"quantize_rows takes fp32 or bf16 rows, got {x.dtype}")
    _want(x, "x", _f32_bf16(), 2)
    _want(q, "q", (torch.int8,), 2)
    _want(scale, "scale", _f32(), 1, contiguous=True)
    rows, K = x.shape
    if tuple(q.shape) != (rows, K) or scale.numel() != rows:
        raise ValueError("q must have x's shape and scale one value per row")
    dt = ZIMG_BF16 if x.dtype == torch.bfloat16 else ZIMG_F32
    _check(lib().zimg_quantize_rows(_ptr(x), dt, x.stride(0), _ptr(q), q.stride(0), _ptr(scale), rows, K,
                                    rotate_block, _stream(stream)))
    return q, scale


def cfg_euler_step(x, out_cond, out_uncond, guidance, dt, stream=None):
    """x += dt * -(out_cond + guidance * (out_cond - out_uncond)) (torch CUDA fp32)."""
    for name, v in (("x", x), ("out_cond", out_cond), ("out_uncond", out_uncond)):
        _want(v, name, _f32(), contiguous=True)
        if v.numel() != x.numel():
            raise ValueError(f"{name}: {x.numel()} elements required")
    _check(lib().zimg_cfg_euler_step(_ptr(x), _ptr(out_cond), _ptr(out_uncond), float(guidance), float(dt),
                                     x.numel(), _stream(stream)))
    return x


def _attention_args(qkv, vT, out, H, segments):
    import torch
    _want(qkv, "qkv", (torch.bfloat16,), 2, contiguous=True)
    _want(vT, "vT", (torch.bfloat16,), 2, contiguous=True)
    _want(out, "out", (torch.bfloat16,), 2, contiguous=True)
    D = int(H) * 128
    seg = np.ascontiguousarray(segments, dtype=np.int32).reshape(-1, 4)
    if qkv.shape[1] != 3 * D or vT.shape[0] != D or out.shape[1] != D:
        raise ValueError(f"qkv must be [rows, {3 * D}], vT [{D}, S_pad] and out [rows, {D}]")
    ends = np.maximum(seg[:, 0] + seg[:, 1], seg[:, 2] + seg[:, 3]) if len(seg) else np.zeros(0)
    if len(seg) and (int(ends.max()) > qkv.shape[0] or int(ends.max()) > out.shape[0]):
        raise ValueError("a segment reaches past the rows of qkv or out")
    return seg, vT.shape[1]


def attention_workspace_size(H, segments, S_pad):
    seg = np.ascontiguousarray(segments, dtype=np.int32).reshape(-1, 4)
    n = ctypes.c_size_t()
    _check(lib().zimg_attention_workspace_size(int(H), len(seg), seg.ctypes.data_as(_I32P), int(S_pad),
                                               ctypes.byref(n)))
    return n.value


def attention(qkv, vT, out, H, segments, workspace=None, stream=None):
    """The block's attention on torch CUDA buffers in the engine's layout
    (zimg_attention): qkv bf16 [rows, 3 H 128], vT bf16 [H 128, S_pad],
    out bf16 [rows, H 128]; segments [B][4] = (start, rows, start, rows).
    ``workspace``: a uint8 CUDA tensor (default: one of the size
    zimg_attention_workspace_size gives, allocated here)."""
    import torch
    seg, S_pad = _attention_args(qkv, vT, out, H, segments)
    if workspace is None:
        n = attention_workspace_size(H, seg, S_pad)
        workspace = torch.empty(n + 256, dtype=torch.uint8, device=qkv.device)
        off = (-workspace.data_ptr()) % 256
        workspace = workspace[off:off + n]
    _want(workspace, "workspace", (torch.uint8,), 1, contiguous=True)
    _check(lib().zimg_attention(_ptr(qkv), _ptr(vT), S_pad, _ptr(out), int(H), len(seg), seg.ctypes.data_as(_I32P),
                                _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def attention_noalloc(qkv, vT, out, H, segments, stream=None):
    """zimg_attention_noalloc: the attention op with the library's static
    device scratch (no workspace, nothing allocated)."""
    seg, S_pad = _attention_args(qkv, vT, out, H, segments)
    _check(lib().zimg_attention_noalloc(_ptr(qkv), _ptr(vT), S_pad, _ptr(out), int(H), len(seg),
                                        seg.ctypes.data_as(_I32P), _stream(stream)))
    return out


def flowmatch_schedule(n_steps, shift):
    """(sigma' [n_steps + 1] ending at 0, model times t [n_steps]) as float64
    numpy arrays, computed by the library (zimg_flowmatch_schedule)."""
    sig = np.zeros(max(int(n_steps), 0) + 1, np.float64)
    t = np.zeros(max(int(n_steps), 1), np.float64)  # (the library refuses n_steps < 1)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(lib().zimg_flowmatch_schedule(int(n_steps), float(shift), sig.ctypes.data_as(dp), t.ctypes.data_as(dp)))
    return sig, t


def euler_step(x, model_out, dt, stream=None):
    """x += dt * -model_out (torch CUDA fp32)."""
    for name, v in (("x", x), ("model_out", model_out)):
        _want(v, name, _f32(), contiguous=True)
        if v.numel() != x.numel():
            raise ValueError(f"{name}: {x.numel()} elements required")
    _check(lib().zimg_euler_step(_ptr(x), _ptr(model_out), float(dt), x.numel(), _stream(stream)))
    return x
