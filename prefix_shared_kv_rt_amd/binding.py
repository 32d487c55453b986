"""ctypes binding of libradixrt.so.  Argument marshalling only: every call
goes straight to the C entry point of the same name in include/radixrt.h.

Host arrays are numpy int32/int64 arrays; device buffers are torch tensors
(passed as raw pointers together with the current HIP stream).
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libradixrt.so")
# Checking builds: RADIXRT_LIB names another build of the library to load;
# with RADIXRT_HOST_ONLY=1 it may hold only the host half (tree, pool, batch
# helpers), and the device entry points are left unbound (calling one fails).
if os.environ.get("RADIXRT_LIB"):
    LIB_PATH = os.environ["RADIXRT_LIB"]
_HOST_ONLY = os.environ.get("RADIXRT_HOST_ONLY") == "1"

RT_OK, RT_ERR_INVALID, RT_ERR_OOM, RT_ERR_LOCKED, RT_ERR_HIP = 0, -1, -2, -3, -4
RT_F32, RT_BF16 = 0, 1

EXPORTS = [
    "rt_last_error", "rt_abi_version",
    "rt_pool_create", "rt_pool_destroy", "rt_pool_alloc", "rt_pool_free", "rt_pool_available",
    "rt_pool_capacity", "rt_pool_free_list", "rt_pool_create_paged", "rt_pool_page_size", "rt_alloc_positions",
    "rt_tree_create", "rt_tree_destroy", "rt_match_prefix", "rt_insert", "rt_lock", "rt_unlock",
    "rt_evict_lru_leaves", "rt_alloc_with_evict", "rt_evictable_size", "rt_protected_size",
    "rt_tree_num_nodes", "rt_tree_dump", "rt_admit_batch", "rt_decode_slots_batch", "rt_finish_batch",
    "kv_store", "req_to_token_scatter", "decode_append", "kv_store_fp8", "radix_decode_attention_fp8kv",
    "radix_extend_attention_fp8kv", "decode_append_fp8", "kv_store_extend", "kv_store_extend_fp8",
    "radix_mixed_attention", "radix_mixed_attention_fp8kv",
    "radix_decode_shared_workspace_bytes", "radix_decode_attention_shared", "radix_decode_attention_shared_fp8kv",
    "radix_extend_attention", "radix_decode_workspace_bytes", "radix_decode_attention",
    "rt_copy_from_host", "rt_copy_from_host_2d", "rt_copy_from_host_check",
    "radix_decode_attention_noalloc",
    "radix_decode_attention_append", "radix_decode_attention_append_fp8kv",
    "radix_decode_attention_shared_append", "radix_decode_attention_shared_append_fp8kv",
]


class RadixRTError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"radixrt error {code}: {msg}")
        self.code = code


class OOMError(RadixRTError):
    pass


_lib = None

# Every pointer argument is declared void*: host arrays go in as their raw
# address (numpy's .ctypes.data), which costs a fraction of building a typed
# ctypes pointer per argument and per call.
_vp = ctypes.c_void_p
_i32p = _vp
_i64p = _vp


def lib():
    """The loaded library.  Fails loudly if it has not been built: there is
    no fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m prefix_shared_kv_rt_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "rt_last_error": (ctypes.c_char_p, []),
            "rt_abi_version": (ctypes.c_int, []),
            "rt_pool_create": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(_vp)]),
            "rt_pool_create_paged": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_vp)]),
            "rt_pool_page_size": (ctypes.c_int32, [_vp]),
            "rt_alloc_positions": (ctypes.c_int, [_vp, ctypes.c_int32, _i32p, _i32p, _i32p, _i32p, ctypes.c_int64,
                                                  ctypes.c_int32, _i32p, ctypes.c_int64, _i32p]),
            "rt_pool_destroy": (None, [_vp]),
            "rt_pool_alloc": (ctypes.c_int, [_vp, ctypes.c_int32, _i32p]),
            "rt_pool_free": (ctypes.c_int, [_vp, _i32p, ctypes.c_int32]),
            "rt_pool_available": (ctypes.c_int32, [_vp]),
            "rt_pool_capacity": (ctypes.c_int32, [_vp]),
            "rt_pool_free_list": (ctypes.c_int, [_vp, _i32p, ctypes.c_int32, _i32p]),
            "rt_tree_create": (ctypes.c_int, [_vp, ctypes.POINTER(_vp)]),
            "rt_tree_destroy": (None, [_vp]),
            "rt_match_prefix": (ctypes.c_int, [_vp, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32, _i32p, _i64p]),
            "rt_insert": (ctypes.c_int, [_vp, _i32p, _i32p, ctypes.c_int32, _i32p]),
            "rt_lock": (ctypes.c_int, [_vp, ctypes.c_int64]),
            "rt_unlock": (ctypes.c_int, [_vp, ctypes.c_int64]),
            "rt_evict_lru_leaves": (ctypes.c_int, [_vp, ctypes.c_int32, _i32p, _i32p, ctypes.c_int32]),
            "rt_alloc_with_evict": (ctypes.c_int, [_vp, ctypes.c_int32, _i32p, _i32p]),
            "rt_evictable_size": (ctypes.c_int64, [_vp]),
            "rt_protected_size": (ctypes.c_int64, [_vp]),
            "rt_tree_num_nodes": (ctypes.c_int64, [_vp]),
            "rt_tree_dump": (ctypes.c_int, [_vp, ctypes.c_char_p, ctypes.c_int64, _i64p]),
            "rt_admit_batch": (ctypes.c_int, [_vp, _i32p, _i64p, ctypes.c_int32, _i32p, ctypes.c_int64,
                                              ctypes.c_int32, _i32p, _i32p, _i32p, _i64p, _i32p, ctypes.c_int64,
                                              _i64p]),
            "rt_decode_slots_batch": (ctypes.c_int, [_vp, ctypes.c_int32, _i32p, _i32p, _i32p, ctypes.c_int64,
                                                     ctypes.c_int32, _i32p]),
            "rt_finish_batch": (ctypes.c_int, [_vp, _i32p, _i64p, ctypes.c_int32, _i32p, ctypes.c_int64,
                                               ctypes.c_int32, _i32p, _i32p, _i64p, _i64p]),
            "kv_store": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int, _vp]),
            "req_to_token_scatter": (ctypes.c_int, [_vp, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_int32, _vp]),
            "kv_store_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_float, ctypes.c_float, _vp]),
            "radix_decode_attention_fp8kv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp,
                                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                                            ctypes.c_float, ctypes.c_float, _vp, ctypes.c_int64,
                                                            _vp]),
            "radix_extend_attention_fp8kv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                                            _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                                            ctypes.c_float, ctypes.c_float, _vp]),
            "decode_append": (ctypes.c_int, [_vp, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int, _vp]),
            "decode_append_fp8": (ctypes.c_int, [_vp, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                                 _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                                 _vp]),
            "kv_store_extend": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int, _vp]),
            "kv_store_extend_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.c_float, ctypes.c_float, _vp]),
            "radix_mixed_attention": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                                     ctypes.c_int, _vp]),
            "radix_mixed_attention_fp8kv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                                           _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                           ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                                           ctypes.c_float, _vp]),
            "radix_decode_shared_workspace_bytes": (ctypes.c_int64, [ctypes.c_int32] * 8),
            "radix_decode_attention_shared": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                                             _vp] + [ctypes.c_int32] * 8 + [ctypes.c_float, _vp,
                                                                                             ctypes.c_int64, _vp]),
            "radix_decode_attention_shared_fp8kv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp,
                                                                   _vp, _vp] + [ctypes.c_int32] * 8 +
                                                    [ctypes.c_float] * 3 + [_vp, ctypes.c_int64, _vp]),
            "rt_copy_from_host": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, _vp]),
            "rt_copy_from_host_2d": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int64,
                                                    ctypes.c_int64, _vp]),
            "radix_extend_attention": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int,
                                                      _vp]),
            "radix_decode_workspace_bytes": (ctypes.c_int64, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                              ctypes.c_int32, ctypes.c_int32]),
            "radix_decode_attention": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int,
                                                      _vp, ctypes.c_int64, _vp]),
            "rt_copy_from_host_check": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.c_int64]),
            "radix_decode_attention_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp,
                                                              _vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                                              ctypes.c_int, _vp]),
            "radix_decode_attention_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp] +
                                              [ctypes.c_int32] * 5 + [ctypes.c_float, _vp, _vp, _vp, _vp,
                                                                      ctypes.c_int64, _vp]),
            "radix_decode_attention_append_fp8kv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp,
                                                                   _vp] + [ctypes.c_int32] * 5 +
                                                    [ctypes.c_float] * 3 + [_vp, _vp, _vp, _vp, ctypes.c_int64,
                                                                            _vp]),
            "radix_decode_attention_shared_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp,
                                                                    _vp, _vp, _vp] + [ctypes.c_int32] * 8 +
                                                     [ctypes.c_float, _vp, _vp, _vp, _vp, ctypes.c_int64, _vp]),
            "radix_decode_attention_shared_append_fp8kv": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                                                          _vp, _vp, _vp, _vp] +
                                                           [ctypes.c_int32] * 8 + [ctypes.c_float] * 3 +
                                                           [_vp, _vp, _vp, _vp, ctypes.c_int64, _vp]),
        }
        for name, (res, args) in sig.items():
            if _HOST_ONLY and not hasattr(L, name):
                continue
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != RT_OK:
        msg = lib().rt_last_error().decode()
        if rc == RT_ERR_OOM:
            raise OOMError(rc, msg)
        raise RadixRTError(rc, msg)
    return rc


_addressof, _c_char = ctypes.addressof, ctypes.c_char


def _p32(a):
    """Address of a host array's data.  The buffer-protocol route costs about
    a third of ``a.ctypes.data``; read-only and empty arrays take the latter."""
    if a is None:
        return None
    try:
        return _addressof(_c_char.from_buffer(a))
    except (TypeError, ValueError, BufferError):
        return a.ctypes.data


_p64 = _p32


def _i32(x):
    return np.ascontiguousarray(x, dtype=np.int32)


# ------------------------------------------------------------------ host --
def rt_pool_create(num_slots, page_size=1):
    h = _vp()
    if page_size == 1:
        _check(lib().rt_pool_create(int(num_slots), ctypes.byref(h)))
    else:
        _check(lib().rt_pool_create_paged(int(num_slots), int(page_size), ctypes.byref(h)))
    return h


def rt_pool_page_size(pool):
    return int(lib().rt_pool_page_size(pool))


def rt_pool_destroy(pool):
    lib().rt_pool_destroy(pool)


def rt_pool_alloc(pool, n):
    out = np.empty(max(int(n), 0), dtype=np.int32)
    _check(lib().rt_pool_alloc(pool, int(n), _p32(out)))
    return out


def rt_pool_free(pool, slots):
    s = _i32(slots)
    _check(lib().rt_pool_free(pool, _p32(s), int(s.size)))


def rt_pool_available(pool):
    return int(lib().rt_pool_available(pool))


def rt_pool_capacity(pool):
    return int(lib().rt_pool_capacity(pool))


def rt_pool_free_list(pool):
    n = rt_pool_available(pool)
    out = np.empty(n, dtype=np.int32)
    got = ctypes.c_int32()
    _check(lib().rt_pool_free_list(pool, _p32(out), n, ctypes.byref(got)))
    return out[:got.value]


def rt_tree_create(pool):
    h = _vp()
    _check(lib().rt_tree_create(pool, ctypes.byref(h)))
    return h


def rt_tree_destroy(tree):
    lib().rt_tree_destroy(tree)


def rt_match_prefix(tree, tokens):
    t = _i32(tokens)
    out = np.empty(max(t.size, 1), dtype=np.int32)
    n = ctypes.c_int32()
    node = ctypes.c_int64()
    _check(lib().rt_match_prefix(tree, _p32(t), int(t.size), _p32(out), int(out.size), ctypes.byref(n),
                                 ctypes.byref(node)))
    return out[:n.value].copy(), int(node.value)


def rt_insert(tree, tokens, slots):
    t, s = _i32(tokens), _i32(slots)
    if t.size != s.size:
        raise ValueError("tokens and slots differ in length")
    present = ctypes.c_int32()
    _check(lib().rt_insert(tree, _p32(t), _p32(s), int(t.size), ctypes.byref(present)))
    return int(present.value)


def rt_lock(tree, node):
    _check(lib().rt_lock(tree, int(node)))


def rt_unlock(tree, node):
    _check(lib().rt_unlock(tree, int(node)))


def rt_evict_lru_leaves(tree, num_tokens, freed_cap=None):
    """Returns (tokens evicted, freed slots in order)."""
    cap = int(freed_cap) if freed_cap is not None else int(rt_evictable_size(tree))
    out = np.empty(max(cap, 1), dtype=np.int32)
    ev = ctypes.c_int32()
    _check(lib().rt_evict_lru_leaves(tree, int(num_tokens), ctypes.byref(ev), _p32(out), cap))
    return int(ev.value), out[:min(ev.value, cap)].copy()


def rt_alloc_with_evict(tree, n):
    """Returns (slots, tokens evicted)."""
    out = np.empty(max(int(n), 1), dtype=np.int32)
    ev = ctypes.c_int32()
    _check(lib().rt_alloc_with_evict(tree, int(n), _p32(out), ctypes.byref(ev)))
    return out[:int(n)].copy(), int(ev.value)


def _host_table(req_to_token):
    """(stride, rows) of a host slot table: a C-contiguous 2-D int32 array,
    which the library writes in place (so it must not be a converted copy)."""
    if not (isinstance(req_to_token, np.ndarray) and req_to_token.dtype == np.int32 and req_to_token.ndim == 2
            and req_to_token.flags.c_contiguous):
        raise ValueError("req_to_token must be a C-contiguous 2-D int32 numpy array")
    return req_to_token.shape[1], req_to_token.shape[0]


def rt_alloc_positions(tree, rows, first_positions, counts, req_to_token):
    """Slots of runs of positions by the page rule, written into the host
    slot-table rows; returns (slots concatenated in run order, tokens
    evicted)."""
    rows, first, cnt = _i32(rows), _i32(first_positions), _i32(counts)
    stride, num_rows = _host_table(req_to_token)
    total = int(cnt.sum()) if cnt.size else 0
    out = np.empty(max(total, 1), dtype=np.int32)
    ev = ctypes.c_int32()
    _check(lib().rt_alloc_positions(tree, rows.size, _p32(rows), _p32(first), _p32(cnt), _p32(req_to_token),
                                    stride, num_rows, _p32(out), out.size, ctypes.byref(ev)))
    return out[:total].copy(), int(ev.value)


def rt_evictable_size(tree):
    return int(lib().rt_evictable_size(tree))


def rt_protected_size(tree):
    return int(lib().rt_protected_size(tree))


def rt_tree_num_nodes(tree):
    return int(lib().rt_tree_num_nodes(tree))


def rt_tree_dump(tree):
    need = ctypes.c_int64()
    lib().rt_tree_dump(tree, None, 0, ctypes.byref(need))
    buf = ctypes.create_string_buffer(need.value + 1)
    _check(lib().rt_tree_dump(tree, buf, need.value + 1, ctypes.byref(need)))
    return buf.raw[:need.value].decode()


_loc_scratch = np.empty(1, dtype=np.int32)


def rt_admit_batch(tree, tokens, token_offsets, req_to_token, rows):
    """tokens: int32 concat; token_offsets: int64 [n+1]; req_to_token: int32
    [R, stride] host array (written in place).  Returns (prefix_lens,
    extend_lens, nodes, out_cache_loc)."""
    global _loc_scratch
    t = _i32(tokens)
    off = np.ascontiguousarray(token_offsets, dtype=np.int64)
    rows = _i32(rows)
    n = rows.size
    stride, num_rows = _host_table(req_to_token)
    pl = np.empty(n, dtype=np.int32)
    el = np.empty(n, dtype=np.int32)
    nodes = np.empty(n, dtype=np.int64)
    cap = int(off[-1] - off[0]) if n else 0
    if _loc_scratch.size < max(cap, 1):   # reused between calls: only the new slots are copied out
        _loc_scratch = np.empty(max(cap, 1), dtype=np.int32)
    loc = _loc_scratch
    nnew = ctypes.c_int64()
    _check(lib().rt_admit_batch(tree, _p32(t), _p64(off), n, _p32(req_to_token), stride, num_rows, _p32(rows),
                                _p32(pl), _p32(el), _p64(nodes), _p32(loc), cap, ctypes.byref(nnew)))
    return pl, el, nodes, loc[:nnew.value].copy()


def rt_decode_slots_batch(tree, rows, positions, req_to_token):
    rows, pos = _i32(rows), _i32(positions)
    stride, num_rows = _host_table(req_to_token)
    out = np.empty(max(rows.size, 1), dtype=np.int32)
    _check(lib().rt_decode_slots_batch(tree, rows.size, _p32(rows), _p32(pos), _p32(req_to_token), stride, num_rows,
                                       _p32(out)))
    return out[:rows.size].copy()


def rt_finish_batch(tree, tokens, token_offsets, req_to_token, rows, prefix_lens, nodes):
    t = _i32(tokens)
    off = np.ascontiguousarray(token_offsets, dtype=np.int64)
    rows, pl = _i32(rows), _i32(prefix_lens)
    nodes = np.ascontiguousarray(nodes, dtype=np.int64)
    stride, num_rows = _host_table(req_to_token)
    freed = ctypes.c_int64()
    _check(lib().rt_finish_batch(tree, _p32(t), _p64(off), rows.size, _p32(req_to_token), stride, num_rows,
                                 _p32(rows), _p32(pl), _p64(nodes), ctypes.byref(freed)))
    return int(freed.value)


# ---------------------------------------------------------------- device --
def _dptr(t):
    # a plain int: ctypes turns it into the void* argument directly
    return t.data_ptr() if t is not None else None


_torch = None
_dtype_codes = None


def _torch_mod():
    global _torch, _dtype_codes
    if _torch is None:
        import torch
        _torch = torch
        _dtype_codes = {torch.bfloat16: RT_BF16, torch.float32: RT_F32}
    return _torch


def _stream(stream):
    if stream is None:
        stream = _torch_mod().cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t):
    if _dtype_codes is None:
        _torch_mod()
    code = _dtype_codes.get(t.dtype)
    if code is None:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return code


def kv_store(k_pool, v_pool, k_new, v_new, out_cache_loc, stream=None):
    n, hkv, d = k_new.shape
    _check(lib().kv_store(_dptr(k_pool), _dptr(v_pool), _dptr(k_new), _dptr(v_new), _dptr(out_cache_loc), n, hkv,
                          d, _dtype_code(k_new), _stream(stream)))


def kv_store_extend(k_pool, v_pool, k_new, v_new, req_to_token, req_pool_indices, prefix_lens, extend_lens,
                    qo_indptr, max_extend_len, stream=None):
    _, hkv, d = k_new.shape
    _check(lib().kv_store_extend(_dptr(k_pool), _dptr(v_pool), _dptr(k_new), _dptr(v_new), _dptr(req_to_token),
                                 req_to_token.shape[1], _dptr(req_pool_indices), _dptr(prefix_lens),
                                 _dptr(extend_lens), _dptr(qo_indptr), prefix_lens.shape[0], int(max_extend_len),
                                 hkv, d, _dtype_code(k_new), _stream(stream)))


def kv_store_extend_fp8(k_pool, v_pool, k_new, v_new, req_to_token, req_pool_indices, prefix_lens, extend_lens,
                        qo_indptr, max_extend_len, k_scale=1.0, v_scale=1.0, stream=None):
    """kv_store_extend into FP8 pools (uint8 codes); k_new, v_new bf16."""
    _, hkv, d = k_new.shape
    _check(lib().kv_store_extend_fp8(_dptr(k_pool), _dptr(v_pool), _dptr(k_new), _dptr(v_new), _dptr(req_to_token),
                                     req_to_token.shape[1], _dptr(req_pool_indices), _dptr(prefix_lens),
                                     _dptr(extend_lens), _dptr(qo_indptr), prefix_lens.shape[0],
                                     int(max_extend_len), hkv, d, float(k_scale), float(v_scale), _stream(stream)))


def rt_copy_from_host(dst, src, stream=None):
    """Copy the pinned host tensor src into the device tensor dst (at least as
    many bytes) with a kernel on `stream`; pageable memory is refused."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("rt_copy_from_host: destination smaller than source")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("rt_copy_from_host: tensors must be contiguous")
    _check(lib().rt_copy_from_host(_dptr(dst), _dptr(src), n, _stream(stream)))


def rt_copy_from_host_2d(dst, src, stream=None):
    """Copy the 2-D pinned host view src (contiguous rows, any row stride)
    into the device view dst of the same shape and dtype."""
    if src.dim() != 2 or dst.shape != src.shape or dst.dtype != src.dtype or src.stride(1) != 1 or dst.stride(1) != 1:
        raise ValueError("rt_copy_from_host_2d: needs 2-D views of one shape and dtype with contiguous rows")
    es = src.element_size()
    _check(lib().rt_copy_from_host_2d(_dptr(dst), dst.stride(0) * es, _dptr(src), src.stride(0) * es,
                                      src.shape[1] * es, src.shape[0], _stream(stream)))


def rt_copy_from_host_check(dst, src, dst_pitch=None, src_pitch=None, width=None, height=1):
    """The host-side checks of a copy from host tensor src to device tensor
    dst, launching nothing (raises RadixRTError when refused).  Defaults:
    one row of src's bytes."""
    nbytes = src.numel() * src.element_size()
    width = nbytes if width is None else int(width)
    _check(lib().rt_copy_from_host_check(_dptr(dst), int(width if dst_pitch is None else dst_pitch), _dptr(src),
                                         int(width if src_pitch is None else src_pitch), width, int(height)))


def req_to_token_scatter(req_to_token, rows, positions, slots, stream=None):
    _check(lib().req_to_token_scatter(_dptr(req_to_token), req_to_token.shape[1], _dptr(rows), _dptr(positions),
                                      _dptr(slots), rows.shape[0], _stream(stream)))


def kv_store_fp8(k_pool, v_pool, k_new, v_new, out_cache_loc, k_scale=1.0, v_scale=1.0, stream=None):
    """k_pool, v_pool: uint8 (FP8 E4M3 codes); k_new, v_new: bf16."""
    n, hkv, d = k_new.shape
    _check(lib().kv_store_fp8(_dptr(k_pool), _dptr(v_pool), _dptr(k_new), _dptr(v_new), _dptr(out_cache_loc), n, hkv,
                              d, float(k_scale), float(v_scale), _stream(stream)))


def radix_decode_attention_fp8kv(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, max_kv_len,
                                 sm_scale, workspace, k_scale=1.0, v_scale=1.0, stream=None):
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention_fp8kv(_dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token),
                                              req_to_token.shape[1], _dptr(req_pool_indices), _dptr(prefix_lens),
                                              batch, int(max_kv_len), hq, hkv, d, float(sm_scale), float(k_scale),
                                              float(v_scale), _dptr(workspace), workspace.numel() * workspace.element_size(),
                                              _stream(stream)))


def radix_extend_attention_fp8kv(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, extend_lens,
                                 qo_indptr, max_extend_len, sm_scale, k_scale=1.0, v_scale=1.0, stream=None):
    batch = prefix_lens.shape[0]
    _, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_extend_attention_fp8kv(_dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token),
                                              req_to_token.shape[1], _dptr(req_pool_indices), _dptr(prefix_lens),
                                              _dptr(extend_lens), _dptr(qo_indptr), batch, int(max_extend_len), hq, hkv,
                                              d, float(sm_scale), float(k_scale), float(v_scale), _stream(stream)))


def decode_append(req_to_token, rows, positions, slots, k_pool, v_pool, k_new, v_new, stream=None):
    n, hkv, d = k_new.shape
    _check(lib().decode_append(_dptr(req_to_token), req_to_token.shape[1], _dptr(rows), _dptr(positions),
                               _dptr(slots), n, _dptr(k_pool), _dptr(v_pool), _dptr(k_new), _dptr(v_new), hkv, d,
                               _dtype_code(k_new), _stream(stream)))


def decode_append_fp8(req_to_token, rows, positions, slots, k_pool, v_pool, k_new, v_new, k_scale=1.0, v_scale=1.0,
                      stream=None):
    """decode_append into FP8 pools (uint8 codes); k_new, v_new bf16."""
    n, hkv, d = k_new.shape
    _check(lib().decode_append_fp8(_dptr(req_to_token), req_to_token.shape[1], _dptr(rows), _dptr(positions),
                                   _dptr(slots), n, _dptr(k_pool), _dptr(v_pool), _dptr(k_new), _dptr(v_new), hkv, d,
                                   float(k_scale), float(v_scale), _stream(stream)))


def radix_extend_attention(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, extend_lens,
                           qo_indptr, max_extend_len, sm_scale, stream=None):
    _, hq, d = q.shape
    hkv = k_pool.shape[1]
    batch = prefix_lens.shape[0]
    _check(lib().radix_extend_attention(_dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token),
                                        req_to_token.shape[1], _dptr(req_pool_indices), _dptr(prefix_lens),
                                        _dptr(extend_lens), _dptr(qo_indptr), batch, int(max_extend_len), hq, hkv, d,
                                        float(sm_scale), _dtype_code(q), _stream(stream)))


def radix_mixed_attention(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, extend_lens,
                          qo_indptr, num_extend, max_extend_len, max_tail_len, sm_scale, stream=None):
    _, hq, d = q.shape
    hkv = k_pool.shape[1]
    batch = prefix_lens.shape[0]
    _check(lib().radix_mixed_attention(_dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token),
                                       req_to_token.shape[1], _dptr(req_pool_indices), _dptr(prefix_lens),
                                       _dptr(extend_lens), _dptr(qo_indptr), batch, int(num_extend),
                                       int(max_extend_len), int(max_tail_len), hq, hkv, d, float(sm_scale),
                                       _dtype_code(q), _stream(stream)))


def radix_mixed_attention_fp8kv(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, extend_lens,
                                qo_indptr, num_extend, max_extend_len, max_tail_len, sm_scale, k_scale=1.0,
                                v_scale=1.0, stream=None):
    _, hq, d = q.shape
    hkv = k_pool.shape[1]
    batch = prefix_lens.shape[0]
    _check(lib().radix_mixed_attention_fp8kv(_dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token),
                                             req_to_token.shape[1], _dptr(req_pool_indices), _dptr(prefix_lens),
                                             _dptr(extend_lens), _dptr(qo_indptr), batch, int(num_extend),
                                             int(max_extend_len), int(max_tail_len), hq, hkv, d, float(sm_scale),
                                             float(k_scale), float(v_scale), _stream(stream)))


def radix_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, max_kv_len):
    return int(lib().radix_decode_workspace_bytes(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim),
                                                  int(max_kv_len)))


def radix_decode_attention(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, max_kv_len, sm_scale,
                           workspace, extend_lens=None, stream=None):
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention(_dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token),
                                        req_to_token.shape[1], _dptr(req_pool_indices), _dptr(prefix_lens),
                                        _dptr(extend_lens), batch, int(max_kv_len), hq, hkv, d, float(sm_scale),
                                        _dtype_code(q), _dptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(stream)))


# RT_NOALLOC_MAX_WORKSPACE_BYTES of include/radixrt.h
NOALLOC_MAX_WORKSPACE_BYTES = 32 << 20


def radix_decode_attention_noalloc(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, max_kv_len,
                                   sm_scale, extend_lens=None, stream=None):
    """radix_decode_attention with the split-K workspace in the library's own
    device array (no allocation)."""
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention_noalloc(_dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool),
                                                _dptr(req_to_token), req_to_token.shape[1], _dptr(req_pool_indices),
                                                _dptr(prefix_lens), _dptr(extend_lens), batch, int(max_kv_len), hq,
                                                hkv, d, float(sm_scale), _dtype_code(q), _stream(stream)))


def radix_decode_shared_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, n_groups, max_group_size,
                                        max_shared_len, max_private_len):
    return int(lib().radix_decode_shared_workspace_bytes(int(batch), int(num_q_heads), int(num_kv_heads),
                                                         int(head_dim), int(n_groups), int(max_group_size),
                                                         int(max_shared_len), int(max_private_len)))


def radix_decode_attention_shared(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, shared_lens,
                                  group_start, max_group_size, max_shared_len, max_private_len, sm_scale, workspace,
                                  stream=None):
    """Decode with shared prefixes read once per group; group_start is a
    device int32 tensor of n_groups + 1 entries."""
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention_shared(
        _dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token), req_to_token.shape[1],
        _dptr(req_pool_indices), _dptr(prefix_lens), _dptr(shared_lens), _dptr(group_start), batch,
        group_start.shape[0] - 1, int(max_group_size), int(max_shared_len), int(max_private_len), hq, hkv, d,
        float(sm_scale), _dptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def radix_decode_attention_shared_fp8kv(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens,
                                        shared_lens, group_start, max_group_size, max_shared_len, max_private_len,
                                        sm_scale, workspace, k_scale=1.0, v_scale=1.0, stream=None):
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention_shared_fp8kv(
        _dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token), req_to_token.shape[1],
        _dptr(req_pool_indices), _dptr(prefix_lens), _dptr(shared_lens), _dptr(group_start), batch,
        group_start.shape[0] - 1, int(max_group_size), int(max_shared_len), int(max_private_len), hq, hkv, d,
        float(sm_scale), float(k_scale), float(v_scale), _dptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def radix_decode_attention_append(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens, max_kv_len,
                                  sm_scale, k_new, v_new, new_slots, workspace, stream=None):
    """decode_append of (req_pool_indices, prefix_lens, new_slots, k_new,
    v_new) and radix_decode_attention in the decode's launches (bf16)."""
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention_append(
        _dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token), req_to_token.shape[1],
        _dptr(req_pool_indices), _dptr(prefix_lens), batch, int(max_kv_len), hq, hkv, d, float(sm_scale),
        _dptr(k_new), _dptr(v_new), _dptr(new_slots), _dptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def radix_decode_attention_append_fp8kv(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens,
                                        max_kv_len, sm_scale, k_new, v_new, new_slots, workspace, k_scale=1.0,
                                        v_scale=1.0, stream=None):
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention_append_fp8kv(
        _dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token), req_to_token.shape[1],
        _dptr(req_pool_indices), _dptr(prefix_lens), batch, int(max_kv_len), hq, hkv, d, float(sm_scale),
        float(k_scale), float(v_scale), _dptr(k_new), _dptr(v_new), _dptr(new_slots), _dptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def radix_decode_attention_shared_append(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens,
                                         shared_lens, group_start, max_group_size, max_shared_len, max_private_len,
                                         sm_scale, k_new, v_new, new_slots, workspace, stream=None):
    """decode_append and radix_decode_attention_shared in the decode's launches (bf16)."""
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention_shared_append(
        _dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token), req_to_token.shape[1],
        _dptr(req_pool_indices), _dptr(prefix_lens), _dptr(shared_lens), _dptr(group_start), batch,
        group_start.shape[0] - 1, int(max_group_size), int(max_shared_len), int(max_private_len), hq, hkv, d,
        float(sm_scale), _dptr(k_new), _dptr(v_new), _dptr(new_slots), _dptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def radix_decode_attention_shared_append_fp8kv(q, o, k_pool, v_pool, req_to_token, req_pool_indices, prefix_lens,
                                               shared_lens, group_start, max_group_size, max_shared_len,
                                               max_private_len, sm_scale, k_new, v_new, new_slots, workspace,
                                               k_scale=1.0, v_scale=1.0, stream=None):
    batch, hq, d = q.shape
    hkv = k_pool.shape[1]
    _check(lib().radix_decode_attention_shared_append_fp8kv(
        _dptr(q), _dptr(o), _dptr(k_pool), _dptr(v_pool), _dptr(req_to_token), req_to_token.shape[1],
        _dptr(req_pool_indices), _dptr(prefix_lens), _dptr(shared_lens), _dptr(group_start), batch,
        group_start.shape[0] - 1, int(max_group_size), int(max_shared_len), int(max_private_len), hq, hkv, d,
        float(sm_scale), float(k_scale), float(v_scale), _dptr(k_new), _dptr(v_new), _dptr(new_slots),
        _dptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
