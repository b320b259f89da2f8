"""Python binding of libmvk.so, the MI355X paged KV-cache attention library.

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels. There
is no fallback: if libmvk.so is missing, the first call fails with instructions.

    reshape_and_cache(key, value, k_cache, v_cache, slot_mapping)
    paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale,
                           max_context_len=None, out=None, partition_tokens=0,
                           workspace=None, new_key=None, new_value=None,
                           slot_mapping=None)
    paged_attention_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens,
                                   scale, max_context_len, out, partition_tokens=0,
                                   new_key=None, new_value=None, slot_mapping=None)
    workspace_size(...), workspace_bytes(...), scratch_limit()
    plan_size(...), make_plan(block_tables, context_lens, num_q_heads, head_dim,
                              max_context_len, slot_mapping=None, plan=None)
    paged_attention_decode_planned(q, k_cache, v_cache, plan, scale, max_context_len,
                                   out=None, new_key=None, new_value=None)
    paged_attention_multi_query(q, k_cache, v_cache, block_tables, context_lens,
                                query_start, scale, max_query_len=None,
                                max_context_len=None, out=None, partition_tokens=0,
                                workspace=None)
    prefill_attention(q, key, value, cu_seqlens, scale, max_seqlen=None,
                      k_cache=None, v_cache=None, slot_mapping=None, out=None)
    BlockManager(num_blocks, prefix_cache=True)   # host-side block tables and slots

The loader relies on torch having loaded its HIP runtime first: the library's
dependency on libamdhip64.so.7 then resolves to that same runtime, so the
stream handles torch hands over are valid inside the library.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmvk.so")

ABI_VERSION = 8
MVK_OK = 0
MVK_ERR_INVALID_ARGUMENT = 1
MVK_ERR_UNSUPPORTED = 2
MVK_ERR_WORKSPACE_TOO_SMALL = 3
MVK_ERR_HIP = 4
MVK_ERR_OUT_OF_BLOCKS = 5
MVK_ERR_SCRATCH_LIMIT = 6
MVK_F16 = 0
MVK_BF16 = 1

_DTYPE = {torch.float16: MVK_F16, torch.bfloat16: MVK_BF16}

# (name, restype, argtypes) of every symbol declared in include/mvk.h
_c_int, _c_float, _c_size, _ptr = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "mvk_abi_version": (_c_int, []),
    "mvk_status_string": (ctypes.c_char_p, [_c_int]),
    "mvk_reshape_and_cache": (_c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int,
                                       _c_int, _c_int, _ptr]),
    "mvk_paged_attention_workspace_size": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                                    ctypes.POINTER(_c_size),
                                                    ctypes.POINTER(_c_int)]),
    "mvk_paged_attention_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "mvk_paged_attention_decode": (_c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                            _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_int, _c_float, _c_int, _c_int, _ptr,
                                            _c_size, _ptr]),
    "mvk_paged_attention_decode_noalloc": (_c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                                    _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                                                    _c_int, _c_int, _c_int, _c_float, _c_int,
                                                    _c_int, _ptr]),
    "mvk_paged_attention_scratch_limit": (_c_size, []),
    "mvk_paged_attention_plan_size": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int,
                                               ctypes.POINTER(_c_size)]),
    "mvk_paged_attention_plan": (_c_int, [_ptr, _c_size, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _ptr]),
    "mvk_paged_attention_decode_planned": (_c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                                    _c_size, _c_int, _c_int, _c_int, _c_int,
                                                    _c_int, _c_int, _c_int, _c_float, _c_int,
                                                    _ptr]),
    "mvk_stream_read_probe": (_c_int, [_ptr, _c_size, _ptr, _c_int, _ptr]),
    "mvk_check_indices": (_c_int, [_ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _ptr, _c_int, _c_int,
                                   _ptr]),
    "mvk_paged_attention_multi_query_workspace_size": (
        _c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                 ctypes.POINTER(_c_size), ctypes.POINTER(_c_int)]),
    "mvk_prefill_attention": (
        _c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int,
                 _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _ptr]),
    "mvk_paged_attention_multi_query": (
        _c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _c_int, _c_int, _c_int, _c_int, _c_int,
                 _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _ptr, _c_size,
                 _ptr]),
    "mvk_paged_attention_multi_query_planned": (
        _c_int, [_ptr, _ptr, _ptr, _ptr, _ptr, _c_size, _ptr, _c_int, _c_int, _c_int, _c_int,
                 _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _ptr]),
    "mvk_bm_create": (_ptr, [_c_int, _c_int, _c_int]),
    "mvk_bm_destroy": (None, [_ptr]),
    "mvk_bm_num_free": (_c_int, [_ptr]),
    "mvk_bm_can_admit": (_c_int, [_ptr, _ptr, _c_int, ctypes.POINTER(_c_int)]),
    "mvk_bm_admit": (_c_int, [_ptr, ctypes.c_int64, _ptr, _c_int, ctypes.POINTER(_c_int)]),
    "mvk_bm_append": (_c_int, [_ptr, ctypes.c_int64, _c_int, ctypes.POINTER(_c_int)]),
    "mvk_bm_rollback": (_c_int, [_ptr, ctypes.c_int64, _c_int]),
    "mvk_bm_release": (_c_int, [_ptr, ctypes.c_int64]),
    "mvk_bm_seq_info": (_c_int, [_ptr, ctypes.c_int64, ctypes.POINTER(_c_int),
                                 ctypes.POINTER(_c_int)]),
    "mvk_bm_block_table": (_c_int, [_ptr, ctypes.c_int64, _ptr, _c_int]),
    "mvk_bm_slots": (_c_int, [_ptr, ctypes.c_int64, _c_int, _c_int, _ptr]),
    "mvk_bm_block_ref": (_c_int, [_ptr, _c_int]),
}


class MvkError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {status_string(status)} (status {status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m paged_kv_cache_206_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use, so that the build module can be
    imported before anything is built)."""
    global _LIB
    if _LIB is None:
        loaded = load_library()
        if loaded.mvk_abi_version() != ABI_VERSION:
            raise ImportError(f"libmvk ABI version {loaded.mvk_abi_version()} != {ABI_VERSION}")
        _LIB = loaded
    return _LIB


def status_string(status: int) -> str:
    return lib().mvk_status_string(status).decode()


def abi_version() -> int:
    return lib().mvk_abi_version()


def _check(func: str, status: int) -> None:
    if status != MVK_OK:
        raise MvkError(func, status)


def _stream(*tensors) -> int:
    """The current stream of the tensors' device; every tensor given (None
    skipped) must be on that one device."""
    dev = tensors[0].device
    for t in tensors[1:]:
        if t is not None and t.device != dev:
            raise ValueError(f"all tensors must be on {dev}; found one on {t.device}")
    return torch.cuda.current_stream(dev).cuda_stream


def _require(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float16 or bfloat16") from None


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Write new K/V rows ([T, Hkv, D]) into pools ([NB, 16, Hkv, D]) at
    flat slots `slot_mapping` (int32 [T]; negative = skip). Asynchronous on the
    current stream."""
    for t, n in ((key, "key"), (value, "value")):
        _require(t, n, ndim=3)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _require(t, n, dtype=key.dtype, ndim=4)
    _require(value, "value", dtype=key.dtype)
    _require(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    T, hkv, d = key.shape
    nb, bs, hkv2, d2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or (hkv2, d2) != (hkv, d) \
            or slot_mapping.shape[0] != T:
        raise ValueError("inconsistent shapes")
    st = lib().mvk_reshape_and_cache(key.data_ptr(), value.data_ptr(), k_cache.data_ptr(),
                                    v_cache.data_ptr(), slot_mapping.data_ptr(), T, hkv, d, bs,
                                    nb, _dtype_code(key),
                                    _stream(key, value, k_cache, v_cache, slot_mapping))
    _check("mvk_reshape_and_cache", st)


def workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   max_context_len: int, partition_tokens: int = 0):
    """(workspace bytes, partition length) the decode call will use."""
    nbytes = ctypes.c_size_t(0)
    chosen = ctypes.c_int32(0)
    st = lib().mvk_paged_attention_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 max_context_len, partition_tokens,
                                                 ctypes.byref(nbytes), ctypes.byref(chosen))
    _check("mvk_paged_attention_workspace_size", st)
    return nbytes.value, chosen.value


def workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_context_len: int) -> int:
    """Workspace bytes that suffice for the decode call at these sizes with the
    library's partition choice, for any number of KV heads (an upper bound;
    workspace_size() gives the exact figure). Raises on invalid sizes."""
    n = lib().mvk_paged_attention_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len)
    if n == ctypes.c_size_t(-1).value:
        raise MvkError("mvk_paged_attention_workspace_bytes", MVK_ERR_INVALID_ARGUMENT)
    return n


def scratch_limit() -> int:
    """Bytes of the static per-GPU scratch of paged_attention_decode_noalloc."""
    return lib().mvk_paged_attention_scratch_limit()


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, out,
                 new_key, new_value, slot_mapping):
    """Checks shared by the two decode entry points; returns the pieces of the
    C call that do not depend on the workspace."""
    _require(q, "q", ndim=3)
    _require(k_cache, "k_cache", dtype=q.dtype, ndim=4)
    _require(v_cache, "v_cache", dtype=q.dtype, ndim=4)
    _require(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    S, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d or block_tables.shape[0] != S \
            or context_lens.shape[0] != S:
        raise ValueError("inconsistent shapes")
    fused = (new_key, new_value, slot_mapping)
    if any(t is not None for t in fused):
        if any(t is None for t in fused):
            raise ValueError("new_key, new_value and slot_mapping go together")
        _require(new_key, "new_key", dtype=q.dtype, ndim=3)
        _require(new_value, "new_value", dtype=q.dtype, ndim=3)
        _require(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
        if new_key.shape != (S, hkv, d) or new_value.shape != new_key.shape \
                or slot_mapping.shape[0] != S:
            raise ValueError("fused cache write: new rows must be [num_seqs, Hkv, D]")
        nk, nv, sm = new_key.data_ptr(), new_value.data_ptr(), slot_mapping.data_ptr()
    else:
        nk = nv = sm = None
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if S else 0
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", dtype=q.dtype)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    return S, hq, hkv, d, nb, bs, nk, nv, sm, max_context_len, out


def paged_attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                           max_context_len: int | None = None, out: torch.Tensor | None = None,
                           partition_tokens: int = 0, workspace: torch.Tensor | None = None,
                           new_key: torch.Tensor | None = None,
                           new_value: torch.Tensor | None = None,
                           slot_mapping: torch.Tensor | None = None) -> torch.Tensor:
    """One batched decode step: out[s, j] = softmax(scale * q[s, j] K_s^T) V_s
    over the context_lens[s] tokens reached through block_tables[s].

    With new_key / new_value ([S, Hkv, D]) and slot_mapping (int32 [S]) the
    step's cache write is fused in: row s is stored at slot_mapping[s] and
    sequence s attends over it.

    `max_context_len` must bound context_lens; when omitted it is read from the
    device (a synchronising copy). `workspace` (uint8, on the device, at least
    workspace_size() bytes) must be zero-filled before its first use; calls
    leave it ready for the next call. It is allocated through torch when
    needed and not given."""
    S, hq, hkv, d, nb, bs, nk, nv, sm, max_context_len, out = _decode_args(
        q, k_cache, v_cache, block_tables, context_lens, max_context_len, out, new_key,
        new_value, slot_mapping)
    need, _ = workspace_size(S, hq, hkv, d, max_context_len, partition_tokens)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:   # zero-filled, as a workspace must be before its first use
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        _require(workspace, "workspace", dtype=torch.uint8)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib().mvk_paged_attention_decode(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
                                          v_cache.data_ptr(), block_tables.data_ptr(),
                                          context_lens.data_ptr(), nk, nv, sm, S, hq, hkv, d, bs,
                                          nb, block_tables.shape[1], max_context_len,
                                          float(scale), _dtype_code(q), partition_tokens, ws_ptr,
                                          ws_bytes,
                                          _stream(q, out, k_cache, v_cache, block_tables,
                                                  context_lens, new_key, new_value, slot_mapping,
                                                  workspace))
    _check("mvk_paged_attention_decode", st)
    return out


def paged_attention_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                                   v_cache: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: float,
                                   max_context_len: int, out: torch.Tensor,
                                   partition_tokens: int = 0,
                                   new_key: torch.Tensor | None = None,
                                   new_value: torch.Tensor | None = None,
                                   slot_mapping: torch.Tensor | None = None) -> torch.Tensor:
    """paged_attention_decode without a workspace: the library keeps split
    partitions' partial states in its static per-GPU scratch
    (scratch_limit() bytes; larger needs raise MvkError with
    MVK_ERR_SCRATCH_LIMIT). `max_context_len` and `out` are required, so that
    the call neither synchronises nor allocates. Calls that may overlap on one
    GPU race on the shared scratch."""
    if max_context_len is None or out is None:
        raise ValueError("paged_attention_decode_noalloc needs max_context_len and out")
    S, hq, hkv, d, nb, bs, nk, nv, sm, max_context_len, out = _decode_args(
        q, k_cache, v_cache, block_tables, context_lens, max_context_len, out, new_key,
        new_value, slot_mapping)
    st = lib().mvk_paged_attention_decode_noalloc(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), nk, nv, sm, S, hq, hkv, d, bs, nb,
        block_tables.shape[1], max_context_len, float(scale), _dtype_code(q), partition_tokens,
        _stream(q, out, k_cache, v_cache, block_tables, context_lens, new_key, new_value,
                slot_mapping))
    _check("mvk_paged_attention_decode_noalloc", st)
    return out


def plan_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
              max_context_len: int):
    """Bytes of a decode plan for these sizes, or None when the planned path
    does not cover them (paged_attention_decode covers every batch)."""
    nbytes = ctypes.c_size_t(0)
    st = lib().mvk_paged_attention_plan_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             max_context_len, ctypes.byref(nbytes))
    if st == MVK_ERR_UNSUPPORTED:
        return None
    _check("mvk_paged_attention_plan_size", st)
    return nbytes.value


def make_plan(block_tables: torch.Tensor, context_lens: torch.Tensor, num_q_heads: int,
              num_kv_heads: int, head_dim: int, max_context_len: int,
              slot_mapping: torch.Tensor | None = None,
              plan: torch.Tensor | None = None) -> torch.Tensor:
    """Build a decode step's plan on the device (asynchronous on the current
    stream) from its block tables, context lengths and, for fused cache
    writes, its new-token slots; returns the plan (uint8 device tensor, a
    snapshot of those arrays) for paged_attention_decode_planned."""
    _require(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    S = context_lens.shape[0]
    if block_tables.shape[0] != S:
        raise ValueError("inconsistent shapes")
    if slot_mapping is not None:
        _require(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
        if slot_mapping.shape[0] != S:
            raise ValueError("slot_mapping must have one slot per sequence")
    need = plan_size(S, num_q_heads, num_kv_heads, head_dim, max_context_len)
    if need is None:
        raise MvkError("mvk_paged_attention_plan_size", MVK_ERR_UNSUPPORTED)
    if plan is None:
        plan = torch.empty(max(need, 16), dtype=torch.uint8, device=context_lens.device)
    _require(plan, "plan", dtype=torch.uint8)
    st = lib().mvk_paged_attention_plan(
        plan.data_ptr(), plan.numel(), block_tables.data_ptr(), context_lens.data_ptr(),
        None if slot_mapping is None else slot_mapping.data_ptr(), S, num_q_heads, num_kv_heads,
        head_dim, block_tables.shape[1], max_context_len,
        _stream(context_lens, block_tables, slot_mapping, plan))
    _check("mvk_paged_attention_plan", st)
    return plan


def paged_attention_decode_planned(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                   plan: torch.Tensor, scale: float, max_context_len: int,
                                   out: torch.Tensor | None = None,
                                   new_key: torch.Tensor | None = None,
                                   new_value: torch.Tensor | None = None) -> torch.Tensor:
    """One layer's decode step through a plan (make_plan): the result of
    paged_attention_decode for the arrays the plan was built from; with
    new_key / new_value the cache write is fused in at the plan's slots.
    `max_context_len` must be the plan's."""
    _require(q, "q", ndim=3)
    _require(k_cache, "k_cache", dtype=q.dtype, ndim=4)
    _require(v_cache, "v_cache", dtype=q.dtype, ndim=4)
    _require(plan, "plan", dtype=torch.uint8)
    S, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d:
        raise ValueError("inconsistent shapes")
    if (new_key is None) != (new_value is None):
        raise ValueError("new_key and new_value go together")
    if new_key is not None:
        _require(new_key, "new_key", dtype=q.dtype, ndim=3)
        _require(new_value, "new_value", dtype=q.dtype, ndim=3)
        if new_key.shape != (S, hkv, d) or new_value.shape != new_key.shape:
            raise ValueError("fused cache write: new rows must be [num_seqs, Hkv, D]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", dtype=q.dtype)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    st = lib().mvk_paged_attention_decode_planned(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if new_key is None else new_key.data_ptr(),
        None if new_value is None else new_value.data_ptr(), plan.data_ptr(), plan.numel(), S, hq,
        hkv, d, bs, nb, max_context_len, float(scale), _dtype_code(q),
        _stream(q, out, k_cache, v_cache, plan, new_key, new_value))
    _check("mvk_paged_attention_decode_planned", st)
    return out


def stream_read_probe(src: torch.Tensor, sink: torch.Tensor, nbytes: int | None = None) -> None:
    """Measurement aid: read `nbytes` (default: all) bytes of `src` with the
    attention kernels' streaming loads; `sink` (int32, one per workgroup)
    receives one word per workgroup. Asynchronous on the current stream."""
    _require(src, "src")
    _require(sink, "sink", dtype=torch.int32, ndim=1)
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    st = lib().mvk_stream_read_probe(src.data_ptr(), n, sink.data_ptr(), sink.numel(),
                                     _stream(src, sink))
    _check("mvk_stream_read_probe", st)


def check_indices(block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                  num_blocks: int, slot_mapping: torch.Tensor | None = None) -> dict:
    """Debug check of a step's index arrays on the device (the attention and
    cache-write calls never validate index contents): the number of context
    lengths outside [0, max_context_len], of block ids a call would read
    outside [0, num_blocks), and of slots past the pool (negative slots mean
    no write). Synchronises the current stream to read the counts."""
    _require(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    if block_tables.shape[0] != context_lens.shape[0]:
        raise ValueError("inconsistent shapes")
    if slot_mapping is not None:
        _require(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    counts = torch.empty(3, dtype=torch.int64, device=context_lens.device)
    st = lib().mvk_check_indices(
        counts.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), context_lens.shape[0],
        block_tables.shape[1], max_context_len,
        None if slot_mapping is None else slot_mapping.data_ptr(),
        0 if slot_mapping is None else slot_mapping.shape[0], num_blocks,
        _stream(counts, block_tables, context_lens, slot_mapping))
    _check("mvk_check_indices", st)
    c = counts.tolist()
    return {"context_lens": c[0], "block_ids": c[1], "slots": c[2]}


def multi_query_workspace_size(num_seqs: int, num_query_tokens: int, max_query_len: int,
                               num_q_heads: int, num_kv_heads: int, head_dim: int,
                               max_context_len: int, partition_tokens: int = 0):
    """(workspace bytes, partition length) the multi-query call will use."""
    nbytes = ctypes.c_size_t(0)
    chosen = ctypes.c_int32(0)
    st = lib().mvk_paged_attention_multi_query_workspace_size(
        num_seqs, num_query_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim,
        max_context_len, partition_tokens, ctypes.byref(nbytes), ctypes.byref(chosen))
    _check("mvk_paged_attention_multi_query_workspace_size", st)
    return nbytes.value, chosen.value


def paged_attention_multi_query(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_tables: torch.Tensor, context_lens: torch.Tensor,
                                query_start: torch.Tensor, scale: float,
                                max_query_len: int | None = None,
                                max_context_len: int | None = None,
                                out: torch.Tensor | None = None, partition_tokens: int = 0,
                                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Several new tokens per sequence, causal among them: sequence s owns
    query rows query_start[s] .. query_start[s+1]-1 of q ([T, Hq, D]), the
    last n_s of its context_lens[s] cached tokens; row query_start[s] + i
    attends over positions 0 .. context_lens[s] - n_s + i.

    `max_query_len` / `max_context_len` must bound n_s / context_lens; when
    omitted they are read from the device (a synchronising copy). The
    workspace (uint8, on the device, at least multi_query_workspace_size()
    bytes) needs no clearing; it is allocated through torch when needed and
    not given."""
    _require(q, "q", ndim=3)
    _require(k_cache, "k_cache", dtype=q.dtype, ndim=4)
    _require(v_cache, "v_cache", dtype=q.dtype, ndim=4)
    _require(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _require(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _require(query_start, "query_start", dtype=torch.int32, ndim=1)
    T, hq, d = q.shape
    S = context_lens.shape[0]
    nb, bs, hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d or block_tables.shape[0] != S \
            or query_start.shape[0] != S + 1:
        raise ValueError("inconsistent shapes")
    if max_query_len is None:
        max_query_len = max(int((query_start[1:] - query_start[:-1]).max().item()), 1) if S else 1
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if S else 0
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", dtype=q.dtype)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    need, _ = multi_query_workspace_size(S, T, max_query_len, hq, hkv, d, max_context_len,
                                         partition_tokens)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _require(workspace, "workspace", dtype=torch.uint8)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    st = lib().mvk_paged_attention_multi_query(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(), S, T,
        max_query_len, hq, hkv, d, bs, nb, block_tables.shape[1], max_context_len, float(scale),
        _dtype_code(q), partition_tokens, ws_ptr, ws_bytes,
        _stream(q, out, k_cache, v_cache, block_tables, context_lens, query_start, workspace))
    _check("mvk_paged_attention_multi_query", st)
    return out


def paged_attention_multi_query_planned(q: torch.Tensor, k_cache: torch.Tensor,
                                        v_cache: torch.Tensor, plan: torch.Tensor,
                                        query_start: torch.Tensor, num_seqs: int, scale: float,
                                        max_query_len: int, max_context_len: int,
                                        out: torch.Tensor | None = None) -> torch.Tensor:
    """paged_attention_multi_query through a plan (make_plan of the same block
    tables and context lengths, without slot_mapping): `num_seqs`,
    `max_context_len` and the heads must be the plan's; `max_query_len`
    bounds the new tokens per sequence."""
    _require(q, "q", ndim=3)
    _require(k_cache, "k_cache", dtype=q.dtype, ndim=4)
    _require(v_cache, "v_cache", dtype=q.dtype, ndim=4)
    _require(plan, "plan", dtype=torch.uint8)
    _require(query_start, "query_start", dtype=torch.int32, ndim=1)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d or query_start.shape[0] != num_seqs + 1:
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", dtype=q.dtype)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    st = lib().mvk_paged_attention_multi_query_planned(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), plan.data_ptr(),
        plan.numel(), query_start.data_ptr(), num_seqs, T, max_query_len, hq, hkv, d, bs, nb,
        max_context_len, float(scale), _dtype_code(q),
        _stream(q, out, k_cache, v_cache, plan, query_start))
    _check("mvk_paged_attention_multi_query_planned", st)
    return out


def prefill_attention(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                      cu_seqlens: torch.Tensor, scale: float, max_seqlen: int | None = None,
                      k_cache: torch.Tensor | None = None, v_cache: torch.Tensor | None = None,
                      slot_mapping: torch.Tensor | None = None,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal self-attention of packed new prompts (prompt s owns rows
    cu_seqlens[s] .. cu_seqlens[s+1]-1 of q [T, Hq, D] and key/value
    [T, Hkv, D]); with k_cache / v_cache / slot_mapping the rows of key/value
    are also stored into the pools at their slots. `max_seqlen` bounds the
    prompt lengths; when omitted it is read from the device (a synchronising
    copy)."""
    _require(q, "q", ndim=3)
    _require(key, "key", dtype=q.dtype, ndim=3)
    _require(value, "value", dtype=q.dtype, ndim=3)
    _require(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1)
    T, hq, d = q.shape
    S = cu_seqlens.shape[0] - 1
    if key.shape != value.shape or key.shape[0] != T or key.shape[2] != d or S < 0:
        raise ValueError("inconsistent shapes")
    hkv = key.shape[1]
    write = (k_cache, v_cache, slot_mapping)
    if any(t is not None for t in write):
        if any(t is None for t in write):
            raise ValueError("k_cache, v_cache and slot_mapping go together")
        _require(k_cache, "k_cache", dtype=q.dtype, ndim=4)
        _require(v_cache, "v_cache", dtype=q.dtype, ndim=4)
        _require(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
        nb, bs, hkv2, d2 = k_cache.shape
        if v_cache.shape != k_cache.shape or (hkv2, d2) != (hkv, d) or slot_mapping.shape[0] != T:
            raise ValueError("inconsistent cache shapes")
        kc, vc, sm = k_cache.data_ptr(), v_cache.data_ptr(), slot_mapping.data_ptr()
    else:
        nb, bs, kc, vc, sm = 0, 16, None, None, None
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if S else 0
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", dtype=q.dtype)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    st = lib().mvk_prefill_attention(out.data_ptr(), q.data_ptr(), key.data_ptr(),
                                     value.data_ptr(), kc, vc, sm, cu_seqlens.data_ptr(), S, T,
                                     max_seqlen, hq, hkv, d, bs, nb, float(scale), _dtype_code(q),
                                     _stream(q, out, key, value, cu_seqlens, k_cache, v_cache,
                                             slot_mapping))
    _check("mvk_prefill_attention", st)
    return out



def _int32_array(values) -> ctypes.Array:
    vals = [int(v) for v in values]
    return (ctypes.c_int32 * max(len(vals), 1))(*vals)


class BlockManager:
    """Host-side owner of the KV pools' 16-token blocks (libmvk's block manager):
    per-sequence block tables and slot mappings, prefix sharing of full blocks,
    release with least-recently-released reuse, and rollback of rejected draft
    tokens. Out of blocks raises MvkError with status MVK_ERR_OUT_OF_BLOCKS and
    changes nothing."""

    BLOCK = 16

    def __init__(self, num_blocks: int, prefix_cache: bool = True):
        self._lib = lib()
        self._h = self._lib.mvk_bm_create(num_blocks, self.BLOCK, 1 if prefix_cache else 0)
        if not self._h:
            raise ValueError(f"cannot create a block manager of {num_blocks} blocks")
        self.num_blocks = num_blocks

    def close(self) -> None:
        if self._h:
            self._lib.mvk_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def num_free(self) -> int:
        return self._lib.mvk_bm_num_free(self._h)

    def can_admit(self, token_ids) -> tuple[bool, int]:
        """(whether the prompt fits now, how many of its leading tokens are cached)."""
        ids = _int32_array(token_ids)
        cached = ctypes.c_int32(0)
        st = self._lib.mvk_bm_can_admit(self._h, ids, len(token_ids), ctypes.byref(cached))
        if st not in (MVK_OK, MVK_ERR_OUT_OF_BLOCKS):
            raise MvkError("mvk_bm_can_admit", st)
        return st == MVK_OK, cached.value

    def admit(self, seq_id: int, token_ids) -> int:
        """Admit a prompt; returns the number of leading tokens already cached."""
        ids = _int32_array(token_ids)
        cached = ctypes.c_int32(0)
        _check("mvk_bm_admit", self._lib.mvk_bm_admit(self._h, seq_id, ids, len(token_ids),
                                                      ctypes.byref(cached)))
        return cached.value

    def append(self, seq_id: int, token_id: int) -> int:
        """Append one token; returns its slot."""
        slot = ctypes.c_int32(0)
        _check("mvk_bm_append", self._lib.mvk_bm_append(self._h, seq_id, token_id,
                                                        ctypes.byref(slot)))
        return slot.value

    def rollback(self, seq_id: int, num_tokens: int) -> None:
        _check("mvk_bm_rollback", self._lib.mvk_bm_rollback(self._h, seq_id, num_tokens))

    def release(self, seq_id: int) -> None:
        _check("mvk_bm_release", self._lib.mvk_bm_release(self._h, seq_id))

    def seq_info(self, seq_id: int) -> tuple[int, int]:
        """(tokens, blocks) the sequence holds."""
        n, b = ctypes.c_int32(0), ctypes.c_int32(0)
        _check("mvk_bm_seq_info", self._lib.mvk_bm_seq_info(self._h, seq_id, ctypes.byref(n),
                                                            ctypes.byref(b)))
        return n.value, b.value

    def block_table(self, seq_id: int, max_blocks: int) -> list[int]:
        table = (ctypes.c_int32 * max(max_blocks, 1))()
        _check("mvk_bm_block_table",
               self._lib.mvk_bm_block_table(self._h, seq_id, table, max_blocks))
        return list(table[:max_blocks])

    def slots(self, seq_id: int, first_token: int, count: int) -> list[int]:
        out = (ctypes.c_int32 * max(count, 1))()
        _check("mvk_bm_slots", self._lib.mvk_bm_slots(self._h, seq_id, first_token, count, out))
        return list(out[:count])

    def block_ref(self, block: int) -> int:
        return self._lib.mvk_bm_block_ref(self._h, block)
