"""Python binding of libsr: streaming chunk-causal attention over a paged KV cache (gfx950).

Thin ctypes layer over the C ABI declared in include/sr.h: the functions below carry the
C names and only marshal arguments (tensor pointers, the current HIP stream, status
codes -> exceptions).  All work runs in the library's HIP kernels; there is no fallback.
PyTorch provides device memory and streams.  Importing the package does not need a GPU;
calling into the library does need the built libsr.so (build() or
`python -m chunk_causal_attention_amd.build`).
"""
import ctypes
import os

__all__ = [
    "SrError", "sr_kvcache_config", "sr_segment", "load", "build", "config_for",
    "sr_kvcache_required_bytes", "sr_kvcache_init", "sr_kvcache_append_chunk", "sr_kvcache_evict",
    "sr_chunk_attention", "sr_kvcache_gather", "sr_kvcache_ring", "sr_kvcache_destroy",
    "sr_attention_workspace_bytes", "sr_kvcache_set_workspace", "workspace_for",
    "sr_ring_create", "sr_ring_append", "sr_ring_evict", "sr_ring_segments", "sr_ring_destroy",
    "sr_status_string", "sr_last_error", "KVCache", "SR_BF16", "SR_F32", "SR_MX", "window_layout", "PAGE_TOKENS", "MAX_WINDOW",
    "MAX_VISIBLE_PAGES",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsr.so")

SR_OK, SR_E_INVALID, SR_E_STATE, SR_E_NOMEM, SR_E_DEVICE, SR_E_UNSUPPORTED = range(6)
SR_BF16, SR_F32, SR_MX = 0, 1, 2   # SR_MX: MXFP6 keys, FP8 values; bf16 inputs and outputs
PAGE_TOKENS = 128         # SR_PAGE_TOKENS
MAX_WINDOW = 14           # SR_MAX_WINDOW
MAX_VISIBLE_PAGES = 1024  # SR_MAX_VISIBLE_PAGES


class SrError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")


_STATUS_NAMES = {0: "SR_OK", 1: "SR_E_INVALID", 2: "SR_E_STATE", 3: "SR_E_NOMEM", 4: "SR_E_DEVICE",
                 5: "SR_E_UNSUPPORTED"}


class sr_kvcache_config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("persistent_tokens", ctypes.c_int32), ("num_banks", ctypes.c_int32),
                ("chunk_capacity", ctypes.c_int32), ("window_chunks", ctypes.c_int32),
                ("causal_block", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class sr_segment(ctypes.Structure):
    _fields_ = [("chunk_id", ctypes.c_int64), ("kind", ctypes.c_int32), ("slot", ctypes.c_int32),
                ("page", ctypes.c_int32), ("length", ctypes.c_int32)]


MAX_LAYOUT_WINDOWS = 64


class sr_window_layout(ctypes.Structure):
    _fields_ = [("num_windows", ctypes.c_int32), ("frames_per_chunk", ctypes.c_int32), ("window_pages", ctypes.c_int32),
                ("window_tokens", ctypes.c_int32 * MAX_LAYOUT_WINDOWS)]


def window_layout(window_tokens, frames_per_chunk, window_pages):
    """sr_window_layout of windows holding window_tokens[w] tokens per latent frame."""
    wt = list(window_tokens)
    if len(wt) > MAX_LAYOUT_WINDOWS:
        raise ValueError(f"at most {MAX_LAYOUT_WINDOWS} windows")
    arr = (ctypes.c_int32 * MAX_LAYOUT_WINDOWS)(*(wt + [0] * (MAX_LAYOUT_WINDOWS - len(wt))))
    return sr_window_layout(len(wt), frames_per_chunk, window_pages, arr)


class sr_qk_prep(ctypes.Structure):
    _fields_ = [("rope_sections", ctypes.c_int32 * 3), ("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float)]


def qk_prep(sections, base=10000.0, eps=1e-6):
    """sr_qk_prep for rotation-pair sections (t, y, x), frequency base and RMSNorm epsilon."""
    return sr_qk_prep((ctypes.c_int32 * 3)(*sections), float(base), float(eps))


_lib = None


def build():
    from .build import build as _b
    return _b()


def load():
    """The loaded library.  torch is imported first so libsr binds to torch's HIP runtime."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (HIP runtime shared with torch)
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m chunk_causal_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    cfgp = ctypes.POINTER(sr_kvcache_config)
    sig = {
        "sr_kvcache_required_bytes": [cfgp, ctypes.POINTER(SZ)],
        "sr_kvcache_init": [cfgp, P, SZ, P, P, P, ctypes.POINTER(P)],
        "sr_kvcache_append_chunk": [P, I64, P, P, I32, P],
        "sr_kvcache_evict": [P, ctypes.POINTER(I64)],
        "sr_chunk_attention": [P, I32, P, P, P, F32, P],
        "sr_window_attention": [P, I32, P, I32, P, P, F32, P],
        "sr_prefix_attention": [P, I32, P, P, P, F32, P],
        "sr_kvcache_update_chunk": [P, I64, P, P, I32, P],
        "sr_kvcache_append_qkv": [P, I64, P, P, I32, P, P, ctypes.POINTER(sr_qk_prep), P, P],
        "sr_kvcache_gather": [P, I32, P, P, I32, ctypes.POINTER(I32), P],
        "sr_kvcache_destroy": [P],
        "sr_attention_workspace_bytes": [cfgp, I32, ctypes.POINTER(SZ)],
        "sr_kvcache_set_workspace": [P, P, SZ, P],
        "sr_ring_create": [cfgp, ctypes.POINTER(P)],
        "sr_ring_append": [P, I64, I32, ctypes.POINTER(I32), ctypes.POINTER(I64)],
        "sr_ring_evict": [P, ctypes.POINTER(I64)],
        "sr_ring_update": [P, I64, I32, ctypes.POINTER(I32)],
        "sr_ring_segments": [P, I32, ctypes.POINTER(sr_segment), I32, ctypes.POINTER(I32)],
        "sr_ring_destroy": [P],
        "sr_kvcache_set_window_layout": [P, ctypes.POINTER(sr_window_layout)],
        "sr_window_layout_check": [cfgp, ctypes.POINTER(sr_window_layout)],
        "sr_kvcache_set_bank": [P, I32, P, P, P],
        "sr_kvcache_append_windows": [P, I64, P, P, P],
        "sr_windows_attention": [P, I32, P, P, P, F32, P],
        "sr_global_attention": [P, I32, P, I32, P, P, F32, P],
        "sr_probe_mfma_bf16": [P, I32, I32, P],
        "sr_probe_lds_read": [P, I64, P, P],
        "sr_global_attention_static": [P, I32, P, I32, P, P, F32, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.sr_kvcache_ring.argtypes = [P]
    L.sr_kvcache_ring.restype = P
    L.sr_status_string.argtypes = [ctypes.c_int]
    L.sr_status_string.restype = ctypes.c_char_p
    L.sr_last_error.argtypes = []
    L.sr_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status):
    if status != SR_OK:
        raise SrError(status, load().sr_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def config_for(num_heads, head_dim, persistent_tokens, chunk_capacity, window_chunks, causal_block=None,
               num_banks=1, dtype=SR_BF16):
    return sr_kvcache_config(num_heads, head_dim, persistent_tokens, num_banks, chunk_capacity, window_chunks,
                             chunk_capacity if causal_block is None else causal_block, dtype)


def sr_status_string(status):
    return load().sr_status_string(status).decode()


def sr_last_error():
    return load().sr_last_error().decode()


def sr_kvcache_required_bytes(cfg):
    n = ctypes.c_size_t()
    _check(load().sr_kvcache_required_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def sr_kvcache_init(cfg, pool, persistent_k=None, persistent_v=None, stream=None):
    h = ctypes.c_void_p()
    _check(load().sr_kvcache_init(ctypes.byref(cfg), _ptr(pool), pool.numel() * pool.element_size(),
                                  _ptr(persistent_k), _ptr(persistent_v), _stream(stream), ctypes.byref(h)))
    return h


def sr_kvcache_append_chunk(h, chunk_id, k, v, n_tokens=None, stream=None):
    n = k.shape[0] if n_tokens is None else n_tokens
    _check(load().sr_kvcache_append_chunk(h, chunk_id, _ptr(k), _ptr(v), n, _stream(stream)))


def sr_kvcache_append_qkv(h, chunk_id, qkv, positions, q_gain, k_gain, prep, q_out, n_tokens=None, stream=None):
    n = qkv.shape[0] if n_tokens is None else n_tokens
    _check(load().sr_kvcache_append_qkv(h, chunk_id, _ptr(qkv), _ptr(positions), n, _ptr(q_gain), _ptr(k_gain),
                                        ctypes.byref(prep), _ptr(q_out), _stream(stream)))


def sr_kvcache_evict(h):
    e = ctypes.c_int64(-1)
    _check(load().sr_kvcache_evict(h, ctypes.byref(e)))
    return e.value


def sr_chunk_attention(h, bank, q, out, lse=None, softmax_scale=None, stream=None):
    if softmax_scale is None:
        softmax_scale = q.shape[-1] ** -0.5
    _check(load().sr_chunk_attention(h, bank, _ptr(q), _ptr(out), _ptr(lse), float(softmax_scale),
                                     _stream(stream)))


def sr_window_attention(h, bank, q, out, lse=None, softmax_scale=None, stream=None):
    if softmax_scale is None:
        softmax_scale = q.shape[-1] ** -0.5
    _check(load().sr_window_attention(h, bank, _ptr(q), q.shape[0], _ptr(out), _ptr(lse), float(softmax_scale),
                                      _stream(stream)))


def sr_prefix_attention(h, bank, q, out, lse=None, softmax_scale=None, stream=None):
    if softmax_scale is None:
        softmax_scale = q.shape[-1] ** -0.5
    _check(load().sr_prefix_attention(h, bank, _ptr(q), _ptr(out), _ptr(lse), float(softmax_scale),
                                      _stream(stream)))


def sr_kvcache_update_chunk(h, chunk_id, k, v, n_tokens=None, stream=None):
    n = k.shape[0] if n_tokens is None else n_tokens
    _check(load().sr_kvcache_update_chunk(h, chunk_id, _ptr(k), _ptr(v), n, _stream(stream)))


def sr_kvcache_set_window_layout(h, layout):
    _check(load().sr_kvcache_set_window_layout(h, ctypes.byref(layout)))


def sr_probe_mfma_bf16(out, workgroups, iters, stream=None):
    """Dense bf16 MFMA probe: out a device float tensor of >= workgroups * 512 elements."""
    if out.numel() < workgroups * 512:
        raise ValueError("out holds fewer than workgroups * 512 floats")
    _check(load().sr_probe_mfma_bf16(_ptr(out), workgroups, iters, _stream(stream)))


def sr_probe_lds_read(src, out, stream=None):
    """Global-to-LDS read probe over the bytes of device tensor src (a multiple of 64 KiB); out a
    device float tensor of >= src bytes / 256 elements."""
    nbytes = src.numel() * src.element_size()
    if out.numel() < nbytes // 256:
        raise ValueError("out holds fewer than bytes / 256 floats")
    _check(load().sr_probe_lds_read(_ptr(src), nbytes, _ptr(out), _stream(stream)))


def sr_window_layout_check(cfg, layout):
    _check(load().sr_window_layout_check(ctypes.byref(cfg), ctypes.byref(layout)))


def sr_kvcache_set_bank(h, bank, k, v, stream=None):
    _check(load().sr_kvcache_set_bank(h, bank, _ptr(k), _ptr(v), _stream(stream)))


def sr_kvcache_append_windows(h, chunk_id, k, v, stream=None):
    _check(load().sr_kvcache_append_windows(h, chunk_id, _ptr(k), _ptr(v), _stream(stream)))


def sr_windows_attention(h, bank, q, out, lse=None, softmax_scale=None, stream=None):
    scale = softmax_scale if softmax_scale is not None else 1.0 / (q.shape[-1] ** 0.5)
    _check(load().sr_windows_attention(h, bank, _ptr(q), _ptr(out), _ptr(lse), scale, _stream(stream)))


def sr_global_attention(h, bank, q, out, lse=None, softmax_scale=None, stream=None):
    scale = softmax_scale if softmax_scale is not None else 1.0 / (q.shape[-1] ** 0.5)
    _check(load().sr_global_attention(h, bank, _ptr(q), q.shape[0], _ptr(out), _ptr(lse), scale, _stream(stream)))


def sr_global_attention_static(h, bank, q, out, lse=None, softmax_scale=None, stream=None):
    scale = softmax_scale if softmax_scale is not None else 1.0 / (q.shape[-1] ** 0.5)
    _check(load().sr_global_attention_static(h, bank, _ptr(q), q.shape[0], _ptr(out), _ptr(lse), scale,
                                             _stream(stream)))


def sr_kvcache_gather(h, bank, k_out, v_out, stream=None):
    n = ctypes.c_int32()
    _check(load().sr_kvcache_gather(h, bank, _ptr(k_out), _ptr(v_out), k_out.shape[0], ctypes.byref(n),
                                    _stream(stream)))
    return n.value


def sr_attention_workspace_bytes(cfg, num_workgroups=0):
    n = ctypes.c_size_t()
    _check(load().sr_attention_workspace_bytes(ctypes.byref(cfg), num_workgroups, ctypes.byref(n)))
    return n.value


def sr_kvcache_set_workspace(h, ws, stream=None):
    """Attach device tensor `ws` (uint8, 256-byte aligned) as the attention workspace; None detaches."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().sr_kvcache_set_workspace(h, _ptr(ws), nbytes, _stream(stream)))


def workspace_for(*cfgs, device="cuda"):
    """A workspace tensor large enough for caches of every config in `cfgs` (shareable by
    caches whose attention calls are ordered on one stream)."""
    import torch
    n = max(sr_attention_workspace_bytes(c) for c in cfgs)
    return torch.empty(n, dtype=torch.uint8, device=device)


def sr_kvcache_ring(h):
    return ctypes.c_void_p(load().sr_kvcache_ring(h))


def sr_kvcache_destroy(h):
    _check(load().sr_kvcache_destroy(h))


def sr_ring_create(cfg):
    r = ctypes.c_void_p()
    _check(load().sr_ring_create(ctypes.byref(cfg), ctypes.byref(r)))
    return r


def sr_ring_append(r, chunk_id, n_tokens):
    slot, com = ctypes.c_int32(), ctypes.c_int64()
    _check(load().sr_ring_append(r, chunk_id, n_tokens, ctypes.byref(slot), ctypes.byref(com)))
    return slot.value, com.value


def sr_ring_evict(r):
    e = ctypes.c_int64()
    _check(load().sr_ring_evict(r, ctypes.byref(e)))
    return e.value


def sr_ring_update(r, chunk_id, n_tokens):
    slot = ctypes.c_int32()
    _check(load().sr_ring_update(r, chunk_id, n_tokens, ctypes.byref(slot)))
    return slot.value


def sr_ring_segments(r, bank, max_segments=MAX_WINDOW + 2):
    arr = (sr_segment * max_segments)()
    n = ctypes.c_int32()
    _check(load().sr_ring_segments(r, bank, arr, max_segments, ctypes.byref(n)))
    return [(s.chunk_id, s.kind, s.slot, s.page, s.length) for s in arr[:n.value]]


def sr_ring_destroy(r):
    _check(load().sr_ring_destroy(r))


class KVCache:
    """Owns a pool tensor and a cache handle; methods call the C ABI on the current stream.

    workspace: "own" (default) allocates and attaches a workspace for this cache, so the
    attention call splits its key tiles evenly over the device; a uint8 device tensor
    (e.g. from workspace_for) attaches a shared one; None runs without a workspace.
    """

    def __init__(self, cfg, persistent_k=None, persistent_v=None, device="cuda", stream=None, workspace="own"):
        import torch
        self.cfg = cfg
        self.h = None
        self.dtype = torch.float32 if cfg.dtype == SR_F32 else torch.bfloat16   # of inputs and outputs
        self.bytes = sr_kvcache_required_bytes(cfg)
        self.pool = torch.empty(self.bytes, dtype=torch.uint8, device=device)
        for t in (persistent_k, persistent_v):
            if t is not None:
                self._check_tensor(t, (cfg.num_banks, cfg.persistent_tokens, cfg.num_heads, cfg.head_dim))
        self.h = sr_kvcache_init(cfg, self.pool, persistent_k, persistent_v, stream)
        self.workspace = None
        if isinstance(workspace, str):
            if workspace != "own":
                raise ValueError('workspace must be "own", None or a device tensor')
            workspace = workspace_for(cfg, device=device)
        self.set_workspace(workspace, stream)

    def set_workspace(self, workspace, stream=None):
        sr_kvcache_set_workspace(self.h, workspace, stream)
        self.workspace = workspace

    def _check_tensor(self, t, shape=None):
        if t.dtype != self.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"expected a contiguous {self.dtype} device tensor, got {t.dtype} {t.device}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"expected shape {tuple(shape)}, got {tuple(t.shape)}")

    def append(self, chunk_id, k, v, stream=None):
        self._check_tensor(k, (k.shape[0], self.cfg.num_heads, self.cfg.head_dim))
        self._check_tensor(v, k.shape)
        sr_kvcache_append_chunk(self.h, chunk_id, k, v, k.shape[0], stream)

    def update(self, chunk_id, k, v, stream=None):
        """Rewrite, in place, a chunk in the window (history or current)."""
        self._check_tensor(k, (k.shape[0], self.cfg.num_heads, self.cfg.head_dim))
        self._check_tensor(v, k.shape)
        sr_kvcache_update_chunk(self.h, chunk_id, k, v, k.shape[0], stream)

    def append_qkv(self, chunk_id, qkv, positions, q_gain, k_gain, prep, q_out=None, stream=None):
        """Fused append after the qkv projection: qkv [n][3][H][D], positions int32 [n][3],
        gains fp32 [D]; writes the prepared K and V to the chunk's slot and returns the
        prepared queries [n][H][D]."""
        import torch
        H, D = self.cfg.num_heads, self.cfg.head_dim
        self._check_tensor(qkv, (qkv.shape[0], 3, H, D))
        n = qkv.shape[0]
        if positions.dtype != torch.int32 or tuple(positions.shape) != (n, 3) or not positions.is_contiguous():
            raise ValueError("positions must be a contiguous int32 [n][3] device tensor")
        for g in (q_gain, k_gain):
            if g.dtype != torch.float32 or tuple(g.shape) != (D,) or not g.is_contiguous():
                raise ValueError("gains must be contiguous float32 [D] device tensors")
        if q_out is None:
            q_out = torch.empty((n, H, D), dtype=self.dtype, device=qkv.device)
        self._check_tensor(q_out, (n, H, D))
        sr_kvcache_append_qkv(self.h, chunk_id, qkv, positions, q_gain, k_gain, prep, q_out, n, stream)
        return q_out

    def evict(self):
        return sr_kvcache_evict(self.h)

    def segments(self, bank=0):
        return sr_ring_segments(sr_kvcache_ring(self.h), bank)

    def attention(self, bank, q, out=None, lse=None, softmax_scale=None, stream=None):
        import torch
        self._check_tensor(q, (q.shape[0], self.cfg.num_heads, self.cfg.head_dim))
        if out is None:
            out = torch.empty_like(q)
        self._check_tensor(out, q.shape)
        if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (self.cfg.num_heads, q.shape[0])):
            raise ValueError("lse must be float32 [H][n]")
        sr_chunk_attention(self.h, bank, q, out, lse, softmax_scale, stream)
        return out

    def _out_lse(self, q, out, lse):
        import torch
        self._check_tensor(q, (q.shape[0], self.cfg.num_heads, self.cfg.head_dim))
        if out is None:
            out = torch.empty_like(q)
        self._check_tensor(out, q.shape)
        if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (self.cfg.num_heads, q.shape[0])):
            raise ValueError("lse must be float32 [H][n]")
        return out

    def window_attention(self, bank, q, out=None, lse=None, softmax_scale=None, stream=None):
        """Moving rows q (history oldest first, then current) over the whole window."""
        out = self._out_lse(q, out, lse)
        sr_window_attention(self.h, bank, q, out, lse, softmax_scale, stream)
        return out

    def prefix_attention(self, bank, q, out=None, lse=None, softmax_scale=None, stream=None):
        """Prefix rows q [P][H][D] of bank `bank` over that bank only."""
        out = self._out_lse(q, out, lse)
        sr_prefix_attention(self.h, bank, q, out, lse, softmax_scale, stream)
        return out

    def set_window_layout(self, window_tokens, frames_per_chunk, window_pages):
        """Window layout of a decoder cache (once, before the first append)."""
        sr_kvcache_set_window_layout(self.h, window_layout(window_tokens, frames_per_chunk, window_pages))
        self.layout = (list(window_tokens), frames_per_chunk, window_pages)
        self.window_rows = frames_per_chunk * sum(window_tokens)

    def _packed_rows(self):
        """Rows of a chunk packed window by window (the library reads exactly that many)."""
        rows = getattr(self, "window_rows", None)
        if rows is None:
            raise SrError(2, "no window layout: set one first")
        return rows

    def set_bank(self, bank, k, v, stream=None):
        """Rewrite the persistent tokens of `bank` ([P][H][D])."""
        shape = (self.cfg.persistent_tokens, self.cfg.num_heads, self.cfg.head_dim)
        self._check_tensor(k, shape)
        self._check_tensor(v, shape)
        sr_kvcache_set_bank(self.h, bank, k, v, stream)

    def append_windows(self, chunk_id, k, v, stream=None):
        """Append a chunk packed window by window ([T][H][D])."""
        self._check_tensor(k, (self._packed_rows(), self.cfg.num_heads, self.cfg.head_dim))
        self._check_tensor(v, k.shape)
        sr_kvcache_append_windows(self.h, chunk_id, k, v, stream)

    def windows_attention(self, bank, q, out=None, lse=None, softmax_scale=None, stream=None):
        """Every window's rows of the current chunk (packed [T][H][D]) over the bank and the window's keys."""
        self._check_tensor(q, (self._packed_rows(), self.cfg.num_heads, self.cfg.head_dim))
        out = self._out_lse(q, out, lse)
        sr_windows_attention(self.h, bank, q, out, lse, softmax_scale, stream)
        return out

    def global_attention(self, bank, q, out=None, lse=None, softmax_scale=None, stream=None):
        """Global-token queries [G][H][D] over the bank and every frame token of the current chunk."""
        out = self._out_lse(q, out, lse)
        sr_global_attention(self.h, bank, q, out, lse, softmax_scale, stream)
        return out

    def global_attention_static(self, bank, q, out=None, lse=None, softmax_scale=None, stream=None):
        """global_attention with its records in the library's static scratch (allocates nothing)."""
        out = self._out_lse(q, out, lse)
        sr_global_attention_static(self.h, bank, q, out, lse, softmax_scale, stream)
        return out

    def gather(self, bank=0, max_tokens=None, stream=None):
        import torch
        if max_tokens is None:
            max_tokens = sum(s[4] for s in self.segments(bank))
        shape = (max_tokens, self.cfg.num_heads, self.cfg.head_dim)
        k = torch.empty(shape, dtype=self.dtype, device=self.pool.device)
        v = torch.empty(shape, dtype=self.dtype, device=self.pool.device)
        n = sr_kvcache_gather(self.h, bank, k, v, stream)
        return k[:n], v[:n]

    def close(self):
        if self.h is not None:
            sr_kvcache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
