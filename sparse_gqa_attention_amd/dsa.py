"""ctypes binding of libdsa.so (include/dsa.h): argument marshalling only.

Each function has the name of the C entry point it wraps and takes torch
tensors that live on the GPU.  Shapes, dtypes and pointers are read from the
tensors and handed to the C ABI unchanged; every step of the computation runs
in the HIP kernels of libdsa.so.  There is no fallback: if the library is not
built, importing this module raises.
"""
import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_F32, DSA_F16, DSA_BF16, DSA_I8 = 0, 1, 2, 3
_DTYPE_CODE = {torch.float32: DSA_F32, torch.float16: DSA_F16,
               torch.bfloat16: DSA_BF16, torch.int8: DSA_I8}
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARGUMENT", 2: "DSA_ERR_UNSUPPORTED",
          3: "DSA_ERR_MISALIGNED", 4: "DSA_ERR_WORKSPACE_TOO_SMALL", 5: "DSA_ERR_HIP"}

EXPORTS = ("dsa_abi_version", "dsa_last_error", "dsa_indexer_score",
           "dsa_topk_workspace_bytes", "dsa_topk", "dsa_attention_workspace_bytes",
           "dsa_attention_decode", "dsa_attention_prefill", "dsa_attention_decode_noalloc",
           "dsa_describe_plan", "dsa_cache_append", "dsa_rmsnorm_rope", "dsa_rmsnorm_rope_multi")
DSA_PLAN_INDEXER, DSA_PLAN_TOPK, DSA_PLAN_ATTENTION_DECODE, DSA_PLAN_ATTENTION_PREFILL = 0, 1, 2, 3


class DsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class AttentionArgs(ctypes.Structure):
    """Mirror of dsa_attention_args."""
    _fields_ = [("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("indices", ctypes.c_void_p), ("k", ctypes.c_int32),
                ("kv_len", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H_q", ctypes.c_int32),
                ("H_kv", ctypes.c_int32), ("D", ctypes.c_int32), ("L_cap", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int32),
                ("aux_k", ctypes.c_void_p), ("aux_v", ctypes.c_void_p),
                ("aux_dtype", ctypes.c_int32), ("aux_len", ctypes.c_int32)]


class CacheAppendArgs(ctypes.Structure):
    """Mirror of dsa_cache_append_args."""
    _fields_ = [("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p), ("new_dtype", ctypes.c_int32),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("kv_dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("key_state_new", ctypes.c_void_p), ("key_state", ctypes.c_void_p),
                ("idx_dtype", ctypes.c_int32),
                ("kv_len", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("D", ctypes.c_int32), ("D_idx", ctypes.c_int32), ("L_cap", ctypes.c_int32)]


class RopeArgs(ctypes.Structure):
    """Mirror of dsa_rmsnorm_rope_args."""
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32),
                ("gamma", ctypes.c_void_p),
                ("cos_cache", ctypes.c_void_p), ("sin_cache", ctypes.c_void_p),
                ("kv_len", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("max_pos", ctypes.c_int32),
                ("eps", ctypes.c_float), ("interleaved", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("out_dtype", ctypes.c_int32)]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.dsa_abi_version.restype = i32
    lib.dsa_abi_version.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_indexer_score.restype = i32
    lib.dsa_indexer_score.argtypes = [vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.dsa_topk_workspace_bytes.restype = sz
    lib.dsa_topk_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.dsa_topk.restype = i32
    lib.dsa_topk.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, sz, vp]
    lib.dsa_attention_workspace_bytes.restype = sz
    lib.dsa_attention_workspace_bytes.argtypes = [ctypes.POINTER(AttentionArgs), i32]
    for name in ("dsa_attention_decode", "dsa_attention_prefill"):
        f = getattr(lib, name)
        f.restype = i32
        f.argtypes = [ctypes.POINTER(AttentionArgs), vp, sz, vp]
    lib.dsa_attention_decode_noalloc.restype = i32
    lib.dsa_attention_decode_noalloc.argtypes = [ctypes.POINTER(AttentionArgs), vp]
    lib.dsa_describe_plan.restype = sz
    lib.dsa_describe_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32,
                                      ctypes.POINTER(AttentionArgs), ctypes.c_char_p, sz]
    lib.dsa_rmsnorm_rope.restype = i32
    lib.dsa_rmsnorm_rope.argtypes = [ctypes.POINTER(RopeArgs), vp]
    lib.dsa_rmsnorm_rope_multi.restype = i32
    lib.dsa_rmsnorm_rope_multi.argtypes = [ctypes.POINTER(RopeArgs), i32, vp]
    lib.dsa_cache_append.restype = i32
    lib.dsa_cache_append.argtypes = [ctypes.POINTER(CacheAppendArgs), vp]
    return lib


LIB = _load()


def _check(status):
    if status != 0:
        raise DsaError(status, LIB.dsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _gpu(t, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    return t


def dsa_abi_version():
    return LIB.dsa_abi_version()


def dsa_last_error():
    return LIB.dsa_last_error().decode()


# ------------------------------------------------------------------ indexer
def dsa_indexer_score(q_idx, w_idx, key_state, kv_len, scores, max_kv_len=None, stream=None):
    """scores[b,s,j] = sum_h w_idx[b,s,h] * (q_idx[b,s,h,:] . key_state[b,j,:])."""
    B, S, H, Di = q_idx.shape
    L = key_state.shape[1]
    for t, n in ((q_idx, "q_idx"), (w_idx, "w_idx"), (key_state, "key_state"),
                 (kv_len, "kv_len"), (scores, "scores")):
        _gpu(t, n)
    _check(LIB.dsa_indexer_score(_ptr(q_idx), _ptr(w_idx), _ptr(key_state),
                                 _DTYPE_CODE[q_idx.dtype], _ptr(kv_len), B, S, H, Di, L,
                                 L if max_kv_len is None else max_kv_len, _ptr(scores),
                                 _stream(stream)))
    return scores


# ------------------------------------------------------------------ top-k
def dsa_topk_workspace_bytes(B, S, L_cap, k):
    return LIB.dsa_topk_workspace_bytes(B, S, L_cap, k)


def dsa_topk(scores, kv_len, k, indices, workspace=None, max_kv_len=None, stream=None):
    """indices[b,s,:] = ascending top-k of scores[b,s,:pos+1], ties to the lower index."""
    B, S, L = scores.shape
    _gpu(scores, "scores"), _gpu(kv_len, "kv_len"), _gpu(indices, "indices")
    need = LIB.dsa_topk_workspace_bytes(B, S, L, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.dsa_topk(_ptr(scores), _ptr(kv_len), B, S, L,
                        L if max_kv_len is None else max_kv_len, k, _ptr(indices),
                        _ptr(workspace), nbytes, _stream(stream)))
    return indices


# ------------------------------------------------------------------ attention
def attention_args(q, k_cache, v_cache, indices, kv_len, out, k_scale=None, v_scale=None,
                   softmax_scale=0.0, max_kv_len=None, aux_k=None, aux_v=None):
    B, S, H_q, D = q.shape
    L, H_kv = k_cache.shape[1], k_cache.shape[2]
    a = AttentionArgs()
    a.q, a.q_dtype = q.data_ptr(), _DTYPE_CODE[q.dtype]
    a.k_cache, a.v_cache, a.kv_dtype = k_cache.data_ptr(), v_cache.data_ptr(), _DTYPE_CODE[k_cache.dtype]
    a.k_scale = None if k_scale is None else k_scale.data_ptr()
    a.v_scale = None if v_scale is None else v_scale.data_ptr()
    a.indices, a.k = indices.data_ptr(), indices.shape[-1]
    a.kv_len = kv_len.data_ptr()
    a.B, a.S, a.H_q, a.H_kv, a.D, a.L_cap = B, S, H_q, H_kv, D, L
    a.max_kv_len = L if max_kv_len is None else max_kv_len
    a.softmax_scale = float(softmax_scale)
    a.out, a.out_dtype = out.data_ptr(), _DTYPE_CODE[out.dtype]
    if aux_k is not None:
        a.aux_k, a.aux_v = aux_k.data_ptr(), aux_v.data_ptr()
        a.aux_dtype, a.aux_len = _DTYPE_CODE[aux_k.dtype], aux_k.shape[1]
    return a


def dsa_attention_workspace_bytes(args, is_decode):
    return LIB.dsa_attention_workspace_bytes(ctypes.byref(args), int(is_decode))


def _attention(fn, is_decode, q, k_cache, v_cache, indices, kv_len, out, k_scale, v_scale,
               softmax_scale, workspace, max_kv_len, stream, aux_k=None, aux_v=None):
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (indices, "indices"),
                 (kv_len, "kv_len"), (out, "out")):
        _gpu(t, n)
    if aux_k is not None:
        _gpu(aux_k, "aux_k"), _gpu(aux_v, "aux_v")
    a = attention_args(q, k_cache, v_cache, indices, kv_len, out, k_scale, v_scale,
                       softmax_scale, max_kv_len, aux_k, aux_v)
    need = LIB.dsa_attention_workspace_bytes(ctypes.byref(a), int(is_decode))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(ctypes.byref(a), _ptr(workspace), nbytes, _stream(stream)))
    return out


def dsa_attention_decode(q, k_cache, v_cache, indices, kv_len, out, k_scale=None, v_scale=None,
                         softmax_scale=0.0, workspace=None, max_kv_len=None, stream=None,
                         aux_k=None, aux_v=None):
    """Split-K sparse GQA attention (decode form); see include/dsa.h."""
    return _attention(LIB.dsa_attention_decode, True, q, k_cache, v_cache, indices, kv_len, out,
                      k_scale, v_scale, softmax_scale, workspace, max_kv_len, stream, aux_k, aux_v)


def dsa_attention_prefill(q, k_cache, v_cache, indices, kv_len, out, k_scale=None, v_scale=None,
                          softmax_scale=0.0, workspace=None, max_kv_len=None, stream=None,
                          aux_k=None, aux_v=None):
    """One workgroup per (row, KV head) sparse GQA attention (prefill form)."""
    return _attention(LIB.dsa_attention_prefill, False, q, k_cache, v_cache, indices, kv_len,
                      out, k_scale, v_scale, softmax_scale, workspace, max_kv_len, stream,
                      aux_k, aux_v)


def dsa_attention_decode_noalloc(q, k_cache, v_cache, indices, kv_len, out, k_scale=None,
                                 v_scale=None, softmax_scale=0.0, max_kv_len=None, stream=None,
                                 aux_k=None, aux_v=None):
    """Decode form with the library's built-in scratch instead of a workspace; see include/dsa.h."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (indices, "indices"),
                 (kv_len, "kv_len"), (out, "out")):
        _gpu(t, n)
    if aux_k is not None:
        _gpu(aux_k, "aux_k"), _gpu(aux_v, "aux_v")
    a = attention_args(q, k_cache, v_cache, indices, kv_len, out, k_scale, v_scale,
                       softmax_scale, max_kv_len, aux_k, aux_v)
    _check(LIB.dsa_attention_decode_noalloc(ctypes.byref(a), _stream(stream)))
    return out


# ------------------------------------------------------------------ launch plans
def dsa_describe_plan(op, B=0, S=0, L_cap=0, max_kv_len=None, k=0, D_idx=0, attention=None):
    """The "key=value" description of the launches `op` would make (no device work)."""
    mx = L_cap if max_kv_len is None else max_kv_len
    ap = None if attention is None else ctypes.byref(attention)
    n = LIB.dsa_describe_plan(op, B, S, L_cap, mx, k, D_idx, ap, None, 0)
    if n == 0:
        raise DsaError(1, LIB.dsa_last_error().decode())
    buf = ctypes.create_string_buffer(n + 1)
    LIB.dsa_describe_plan(op, B, S, L_cap, mx, k, D_idx, ap, buf, n + 1)
    return buf.value.decode()


def plan_fields(text):
    """The description as a dict of its key=value words."""
    return dict(w.split("=", 1) for w in text.split())


# ------------------------------------------------------------------ cache append
def cache_append_args(k_new, v_new, k_cache, v_cache, kv_len, k_scale=None, v_scale=None,
                      key_state_new=None, key_state=None):
    B, S, H_kv, D = k_new.shape
    a = CacheAppendArgs()
    a.k_new, a.v_new, a.new_dtype = k_new.data_ptr(), v_new.data_ptr(), _DTYPE_CODE[k_new.dtype]
    a.k_cache, a.v_cache, a.kv_dtype = k_cache.data_ptr(), v_cache.data_ptr(), _DTYPE_CODE[k_cache.dtype]
    a.k_scale = None if k_scale is None else k_scale.data_ptr()
    a.v_scale = None if v_scale is None else v_scale.data_ptr()
    if key_state is not None:
        a.key_state_new, a.key_state = key_state_new.data_ptr(), key_state.data_ptr()
        a.idx_dtype, a.D_idx = _DTYPE_CODE[key_state.dtype], key_state.shape[-1]
    a.kv_len = kv_len.data_ptr()
    a.B, a.S, a.H_kv, a.D, a.L_cap = B, S, H_kv, D, k_cache.shape[1]
    return a


def dsa_cache_append(k_new, v_new, k_cache, v_cache, kv_len, k_scale=None, v_scale=None,
                     key_state_new=None, key_state=None, stream=None):
    """Write the S new tokens at kv_len[b] - S + s (INT8 caches: quantised); see include/dsa.h."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (kv_len, "kv_len")):
        _gpu(t, n)
    a = cache_append_args(k_new, v_new, k_cache, v_cache, kv_len, k_scale, v_scale,
                          key_state_new, key_state)
    _check(LIB.dsa_cache_append(ctypes.byref(a), _stream(stream)))


# ------------------------------------------------------------------ RMSNorm + rotary
def rope_args(x, gamma, cos_cache, sin_cache, kv_len, out, eps=1e-6, interleaved=False):
    B, S, H, D = x.shape
    a = RopeArgs()
    a.x, a.x_dtype = x.data_ptr(), _DTYPE_CODE[x.dtype]
    a.gamma, a.cos_cache, a.sin_cache = gamma.data_ptr(), cos_cache.data_ptr(), sin_cache.data_ptr()
    a.kv_len = kv_len.data_ptr()
    a.B, a.S, a.H, a.D, a.max_pos = B, S, H, D, cos_cache.shape[0]
    a.eps, a.interleaved = float(eps), int(bool(interleaved))
    a.out, a.out_dtype = out.data_ptr(), _DTYPE_CODE[out.dtype]
    return a


def dsa_rmsnorm_rope(x, gamma, cos_cache, sin_cache, kv_len, out, eps=1e-6, interleaved=False,
                     stream=None):
    """out = rotary(RMSNorm(x) * gamma) at position kv_len[b] - S + s, in FP32; see include/dsa.h."""
    for t, n in ((x, "x"), (gamma, "gamma"), (cos_cache, "cos_cache"), (sin_cache, "sin_cache"),
                 (kv_len, "kv_len"), (out, "out")):
        _gpu(t, n)
    a = rope_args(x, gamma, cos_cache, sin_cache, kv_len, out, eps, interleaved)
    _check(LIB.dsa_rmsnorm_rope(ctypes.byref(a), _stream(stream)))
    return out


def dsa_rmsnorm_rope_multi(jobs, stream=None):
    """Several dsa_rmsnorm_rope jobs in one launch; jobs: sequence of dicts with the keys
    x, gamma, cos_cache, sin_cache, kv_len, out and optionally eps, interleaved.
    Returns the list of outputs; see include/dsa.h."""
    jobs = list(jobs)
    arr = (RopeArgs * max(1, len(jobs)))()
    for i, j in enumerate(jobs):
        for n in ("x", "gamma", "cos_cache", "sin_cache", "kv_len", "out"):
            _gpu(j[n], f"jobs[{i}].{n}")
        arr[i] = rope_args(j["x"], j["gamma"], j["cos_cache"], j["sin_cache"], j["kv_len"],
                           j["out"], j.get("eps", 1e-6), j.get("interleaved", False))
    _check(LIB.dsa_rmsnorm_rope_multi(arr, len(jobs), _stream(stream)))
    return [j["out"] for j in jobs]
