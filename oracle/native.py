"""ctypes wrapper of the plain C++17 fp64 oracle (oracle/cpp/attention_oracle.cpp).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the smoke check and
the benchmark's CPU-baseline leg may load it.  The C++ file shares no code with the HIP
library and none with the numpy oracle; the functions here only marshal arguments and keep
the numpy oracle's signatures, so that the same pins run against both:

  masked_attention(q, k, v, visible, scale, return_probs=False)   the definition
  StreamingCache(pk, pv, window, capacity=None)                    the cache model
  chunk_attention(cache, bank, q, scale, causal_block, dtype, heads=None, rows=None, threads=0)
  full_sequence_attention(prefix_k, prefix_v, chunks_k, chunks_v, q, window, causal_block,
                          scale, dtype)                            the dense route, no cache

What each computes, with citations of the pages, is stated in the C++ file's header.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "cpp", "attention_oracle.cpp")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
# Built on this machine and run on others: a fixed x86-64 level (x86-64-v4: AVX-512 F/BW/CD/DQ/VL),
# not -march=native; the loader checks the running CPU for it.
CXXFLAGS = ["-O3", "-std=c++17", "-march=x86-64-v4", "-fopenmp-simd", "-fPIC", "-shared", "-pthread"]
_REQUIRED_CPU_FLAGS = ("avx2", "fma", "avx512f", "avx512bw", "avx512cd", "avx512dq", "avx512vl")
_lib = None


def build(force=False):
    """Compiles the C++ oracle in-tree with g++ (when missing or older than its source)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++"] + CXXFLAGS + [SOURCE, "-o", tmp])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def cpu_model():
    """The host CPU's model name and logical CPU count, from /proc/cpuinfo."""
    model, n = "unknown", 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name") and model == "unknown":
                    model = line.split(":", 1)[1].strip()
                if line.startswith("processor"):
                    n += 1
    except OSError:
        pass
    return model, n


def _check_cpu():
    try:
        with open("/proc/cpuinfo") as f:
            flags = next((l.split(":", 1)[1].split() for l in f if l.startswith("flags")), [])
    except OSError:
        return
    missing = [x for x in _REQUIRED_CPU_FLAGS if x not in flags]
    if missing:
        raise RuntimeError("the C++ oracle is built for x86-64-v4; this CPU lacks " + ", ".join(missing))


def _bind(path):
    L = ctypes.CDLL(path)
    P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    sig = {
        "orc_hardware_threads": ([], I),
        "orc_attention": ([I, I, I, I, P, P, P, P, D, P, P, P], I),
        "orc_cache_create": ([I, I, I, I, I, I, I, P, P, ctypes.POINTER(P)], I),
        "orc_cache_destroy": ([P], None),
        "orc_cache_append": ([P, I64, P, P, I], I),
        "orc_cache_update": ([P, I64, P, P, I], I),
        "orc_cache_evict": ([P, ctypes.POINTER(I64)], I),
        "orc_cache_set_bank": ([P, I, P, P], I),
        "orc_cache_visible_ids": ([P, ctypes.POINTER(I64), I], I),
        "orc_cache_sequence_len": ([P, I, ctypes.POINTER(I), ctypes.POINTER(I)], I),
        "orc_cache_gather": ([P, I, P, P], I),
        "orc_chunk_attention": ([P, I, P, I, D, I, P, I, P, I, I, P, P], I),
        "orc_full_sequence_attention": ([I, I, I, I, P, P, I, P, P, P, P, I, I, D, I, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def load(path=None):
    """The loaded oracle library (built first if needed); `path` loads another build of it."""
    global _lib
    if path is not None:
        _check_cpu()
        return _bind(path)
    if _lib is None:
        _check_cpu()
        _lib = _bind(build())
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _storage(a):
    """(contiguous array, dtype code): bf16 bit patterns (uint16) -> 0, float32 -> 1."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, 0
    if a.dtype == np.float32:
        return a, 1
    raise TypeError("storage values are bf16 bit patterns (uint16) or float32, not %s" % a.dtype)


class CacheStateError(Exception):
    """An append/update/evict that the state machine rejects (state unchanged)."""


def masked_attention(q, k, v, visible, scale, return_probs=False, lib=None):
    """q [Nq, D], k [Nk, D], v [Nk, Dv], visible bool [Nq, Nk] -> (o, lse[, probs]) fp64."""
    L = lib or load()
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    vis = np.ascontiguousarray(visible, dtype=np.uint8)
    nq, d = q.shape
    nk, dv = v.shape
    o = np.zeros((nq, dv))
    lse = np.zeros(nq)
    probs = np.zeros((nq, nk)) if return_probs else None
    st = L.orc_attention(nq, nk, d, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(vis), float(scale), _ptr(o), _ptr(lse),
                         _ptr(probs) if return_probs else None)
    if st:
        raise ValueError("a query row sees no key")
    return (o, lse, probs) if return_probs else (o, lse)


class StreamingCache:
    """The C++ cache model behind the numpy StreamingCache's interface."""

    def __init__(self, persistent_k, persistent_v, window, capacity=None, lib=None):
        self._L = lib or load()
        pk, self.dtype_code = _storage(persistent_k)
        pv, dv = _storage(persistent_v)
        if pk.shape != pv.shape or dv != self.dtype_code or pk.ndim != 4:
            raise ValueError("persistent K/V: [banks][P][H][D] of one storage type")
        banks, P, H, D = pk.shape
        self.H, self.D, self.P, self._banks = H, D, P, banks
        self.window = window
        h = ctypes.c_void_p()
        if self._L.orc_cache_create(banks, P, H, D, self.dtype_code, window, capacity or 0, _ptr(pk), _ptr(pv),
                                    ctypes.byref(h)):
            raise ValueError("bad cache geometry")
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None):
            self._L.orc_cache_destroy(self._h)
            self._h = None

    @property
    def banks(self):
        return self._banks

    def _chunk(self, k, v):
        k, dk = _storage(k)
        v, dv = _storage(v)
        if k.shape != v.shape or k.ndim != 3 or dk != self.dtype_code or dv != self.dtype_code or \
                k.shape[1:] != (self.H, self.D):
            raise CacheStateError("bad chunk shape or storage type")
        return k, v

    def append(self, chunk_id, k, v):
        k, v = self._chunk(k, v)
        if self._L.orc_cache_append(self._h, int(chunk_id), _ptr(k), _ptr(v), k.shape[0]):
            raise CacheStateError("append rejected")

    def update(self, chunk_id, k, v):
        k, v = self._chunk(k, v)
        if self._L.orc_cache_update(self._h, int(chunk_id), _ptr(k), _ptr(v), k.shape[0]):
            raise CacheStateError("chunk %d is not in the window" % chunk_id)

    def evict(self):
        e = ctypes.c_int64()
        if self._L.orc_cache_evict(self._h, ctypes.byref(e)):
            raise CacheStateError("nothing to evict")
        return e.value

    def set_bank(self, bank, k, v):
        k, _ = _storage(k)
        v, _ = _storage(v)
        if k.shape != (self.P, self.H, self.D) or v.shape != k.shape:
            raise CacheStateError("a bank keeps its shape")
        if self._L.orc_cache_set_bank(self._h, bank, _ptr(k), _ptr(v)):
            raise CacheStateError("bank out of range")

    def prefix_len(self, bank):
        return self.P

    def visible_ids(self):
        ids = (ctypes.c_int64 * (self.window + 2))()
        n = self._L.orc_cache_visible_ids(self._h, ids, self.window + 2)
        return [int(ids[i]) for i in range(n)]

    def sequence(self, bank):
        """(k [N][H][D], v [N][H][D], n_fixed) in storage values, exactly as stored."""
        n, nf = ctypes.c_int(), ctypes.c_int()
        if self._L.orc_cache_sequence_len(self._h, bank, ctypes.byref(n), ctypes.byref(nf)):
            raise CacheStateError("no current chunk or bank out of range")
        dt = np.uint16 if self.dtype_code == 0 else np.float32
        k = np.zeros((n.value, self.H, self.D), dt)
        v = np.zeros_like(k)
        self._L.orc_cache_gather(self._h, bank, _ptr(k), _ptr(v))
        return k, v, nf.value


def chunk_attention(cache, bank, q, scale, causal_block, dtype, heads=None, rows=None, threads=0):
    """q [n][H][D] storage values of the current chunk -> (o [len(rows)][len(heads)][D],
    lse [len(heads)][len(rows)]) fp64; `threads` <= 0 uses every hardware thread."""
    q, code = _storage(q)
    if code != cache.dtype_code or {"bf16": 0, "f32": 1}[dtype] != code:
        raise TypeError("queries, cache and dtype disagree")
    heads = np.arange(cache.H, dtype=np.int32) if heads is None else np.ascontiguousarray(heads, dtype=np.int32)
    rows = np.arange(q.shape[0], dtype=np.int32) if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    o = np.zeros((len(rows), len(heads), cache.D))
    lse = np.zeros((len(heads), len(rows)))
    st = cache._L.orc_chunk_attention(cache._h, bank, _ptr(q), q.shape[0], float(scale), int(causal_block),
                                      _ptr(heads), len(heads), _ptr(rows), len(rows), int(threads), _ptr(o), _ptr(lse))
    if st == 1:
        raise ValueError("bad chunk call (queries must be the current chunk's tokens)")
    if st == 2:
        raise ValueError("a query row sees no key")
    return o, lse


def full_sequence_attention(prefix_k, prefix_v, chunks_k, chunks_v, q, window, causal_block, scale, dtype,
                            threads=0, lib=None):
    """The last chunk's queries over [prefix; every chunk so far] with the window mask, no cache."""
    L = lib or load()
    pk, code = _storage(prefix_k)
    pv, _ = _storage(prefix_v)
    q, _ = _storage(q)
    if {"bf16": 0, "f32": 1}[dtype] != code:
        raise TypeError("storage type and dtype disagree")
    lens = np.array([c.shape[0] for c in chunks_k], dtype=np.int32)
    ck = np.ascontiguousarray(np.concatenate(list(chunks_k), axis=0))
    cv = np.ascontiguousarray(np.concatenate(list(chunks_v), axis=0))
    P, H, D = pk.shape
    n = q.shape[0]
    o = np.zeros((n, H, D))
    lse = np.zeros((H, n))
    st = L.orc_full_sequence_attention(P, H, D, code, _ptr(pk), _ptr(pv), len(lens), _ptr(lens), _ptr(ck), _ptr(cv),
                                       _ptr(q), int(window), int(causal_block), float(scale), int(threads), _ptr(o),
                                       _ptr(lse))
    if st:
        raise ValueError("bad full-sequence call")
    return o, lse
