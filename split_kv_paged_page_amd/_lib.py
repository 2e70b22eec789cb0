"""ctypes binding of libsplitkv (include/attn_decode.h).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  Device buffers are passed as raw pointers (torch tensors are
accepted and their ``data_ptr()`` is used); streams as hipStream_t handles
(``torch.cuda.Stream.cuda_stream``).  The library must have been built
(``python -m split_kv_paged_page_amd.build``); loading fails loudly otherwise.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SPLITKV_LIB names another build of the same library (the CPU tests load the
# host-sanitized build this way); by default the in-tree libsplitkv.so.
LIB_PATH = os.environ.get("SPLITKV_LIB") or os.path.join(HERE, "libsplitkv.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EWORKSPACE, ATTN_EHIP = range(5)
ATTN_F32, ATTN_BF16 = 0, 1
ATTN_PLAN_POLICY_P2 = 1
ATTN_PLAN_NO_XCD_REMAP = 2
ATTN_PLAN_FUSED_MERGE = 4
ATTN_PLAN_PRIVATE_PAGES = 8
ATTN_PLAN_SHARED_PASS = 16
ATTN_VARIANT_VALU, ATTN_VARIANT_MFMA = 1, 2

EXPORTED = ["attn_decode_plan", "attn_decode_plan_lens", "attn_decode_run", "attn_decode_partials", "attn_decode_merge",
            "attn_decode_workspace_layout", "attn_decode_workspace_init", "attn_decode_split_range",
            "attn_decode_run_noalloc", "attn_decode_plan_prefix", "attn_decode_run_prefix", "attn_decode_last_error"]
NOALLOC_SCRATCH_BYTES = 64 << 20   # ATTN_NOALLOC_SCRATCH_BYTES
MAX_SPLIT_TABLE = 64               # ATTN_MAX_SPLIT_TABLE
SHARED_PASS_MIN_ROWS = 128         # ATTN_SHARED_PASS_MIN_ROWS

_STATUS = {ATTN_OK: "ATTN_OK", ATTN_EINVAL: "ATTN_EINVAL", ATTN_EUNSUPPORTED: "ATTN_EUNSUPPORTED",
           ATTN_EWORKSPACE: "ATTN_EWORKSPACE", ATTN_EHIP: "ATTN_EHIP"}


class AttnDecodeError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{_STATUS.get(status, status)}: {text}")
        self.status = status


class AttnDecodeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "num_q_heads", "num_kv_heads", "head_dim_qk", "head_dim_v", "page_size",
        "max_pages_per_req", "dtype", "causal", "v_aliases_k", "reserved")] + \
        [(n, ctypes.c_int64) for n in (
            "num_pages", "k_stride_page", "k_stride_head", "k_stride_tok",
            "v_stride_page", "v_stride_head", "v_stride_tok")]


class AttnDecodePlan(ctypes.Structure):
    _fields_ = [("desc", AttnDecodeDesc)] + [(n, ctypes.c_int32) for n in (
        "max_context_len", "num_splits", "max_splits", "split_align", "variant", "rows_per_wg",
        "head_tiles", "stage1_waves", "xcd_remap", "flags", "split_chunk", "live_splits")] + \
        [("workspace_bytes", ctypes.c_int64), ("key", ctypes.c_uint64),
         ("split_start", ctypes.c_int32 * (MAX_SPLIT_TABLE + 1))]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f not in ("desc", "split_start")}
        d["split_start"] = list(self.split_start)
        d["desc"] = {f: getattr(self.desc, f) for f, _ in AttnDecodeDesc._fields_}
        return d


class AttnDecodePrefixPlan(ctypes.Structure):
    _fields_ = [("shared", AttnDecodePlan), ("own", AttnDecodePlan)] + [(n, ctypes.c_int32) for n in (
        "prefix_group", "prefix_len", "num_splits", "reserved")] + \
        [("workspace_bytes", ctypes.c_int64), ("key", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f not in ("shared", "own")}
        d["shared"] = self.shared.as_dict()
        d["own"] = self.own.as_dict()
        return d


_lib = None


def one_hip_runtime() -> None:
    """Import torch, when installed, before a HIP library of this package is
    opened.  torch ships its own libamdhip64.so and asks for it by the name
    libamdhip64.so, while the libraries here are linked against the soname
    libamdhip64.so.7: opened first, a library here would map the system HIP
    runtime and torch would then map its own, leaving two runtimes in the
    process, and a kernel launched through one on memory the other allocated
    fails.  With torch loaded first, its runtime carries the soname the
    libraries ask for and the process keeps one runtime."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        one_hip_runtime()
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m split_kv_paged_page_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.attn_decode_plan.argtypes = [P(AttnDecodeDesc), i32, i32, i32, P(AttnDecodePlan)]
        L.attn_decode_plan_lens.argtypes = [P(AttnDecodeDesc), P(i32), i32, i32, P(AttnDecodePlan)]
        L.attn_decode_run.argtypes = [P(AttnDecodePlan), vp, vp, vp, vp, vp, f32, i32, vp, vp, vp, i64, vp]
        L.attn_decode_partials.argtypes = [P(AttnDecodePlan), vp, vp, vp, vp, vp, f32, i32, vp, i64, vp]
        L.attn_decode_merge.argtypes = [P(AttnDecodePlan), i32, vp, i64, vp, vp, vp]
        L.attn_decode_workspace_layout.argtypes = [P(AttnDecodePlan), i32, P(i64), P(i64), P(i64)]
        L.attn_decode_workspace_init.argtypes = [P(AttnDecodePlan), vp, i64, vp]
        L.attn_decode_split_range.argtypes = [P(AttnDecodePlan), i32, i32, i32, P(i32), P(i32)]
        L.attn_decode_run_noalloc.argtypes = [P(AttnDecodePlan), vp, vp, vp, vp, vp, f32, i32, vp, vp, vp]
        L.attn_decode_plan_prefix.argtypes = [P(AttnDecodeDesc), i32, i32, i32, i32, P(AttnDecodePrefixPlan)]
        L.attn_decode_run_prefix.argtypes = [P(AttnDecodePrefixPlan), vp, vp, vp, vp, vp, f32, vp, vp, vp, i64, vp]
        L.attn_decode_last_error.argtypes = []
        L.attn_decode_last_error.restype = ctypes.c_char_p
        for n in EXPORTED[:-1]:
            getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != ATTN_OK:
        raise AttnDecodeError(status, lib().attn_decode_last_error().decode())


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(*, batch, q_len, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, page_size,
              max_pages_per_req, dtype, causal, v_aliases_k, num_pages, k_strides, v_strides) -> AttnDecodeDesc:
    d = AttnDecodeDesc()
    d.batch, d.q_len, d.num_q_heads, d.num_kv_heads = batch, q_len, num_q_heads, num_kv_heads
    d.head_dim_qk, d.head_dim_v, d.page_size, d.max_pages_per_req = head_dim_qk, head_dim_v, page_size, \
        max_pages_per_req
    d.dtype, d.causal, d.v_aliases_k, d.reserved = dtype, int(causal), int(v_aliases_k), 0
    d.num_pages = num_pages
    d.k_stride_page, d.k_stride_head, d.k_stride_tok = k_strides
    d.v_stride_page, d.v_stride_head, d.v_stride_tok = v_strides
    return d


def attn_decode_plan(desc: AttnDecodeDesc, max_context_len: int, num_splits: int = 0,
                     flags: int = 0) -> AttnDecodePlan:
    p = AttnDecodePlan()
    _check(lib().attn_decode_plan(ctypes.byref(desc), max_context_len, num_splits, flags, ctypes.byref(p)))
    return p


def attn_decode_plan_lens(desc: AttnDecodeDesc, host_context_lens, num_splits: int = 0,
                          flags: int = 0) -> AttnDecodePlan:
    """Plan with the batch's context lengths known on the host (a sequence of
    ints); the policy may then fix one split length for every request."""
    lens = [int(x) for x in host_context_lens]
    if len(lens) != desc.batch:
        raise ValueError(f"{len(lens)} context lengths for a batch of {desc.batch}")
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens)
    p = AttnDecodePlan()
    _check(lib().attn_decode_plan_lens(ctypes.byref(desc), arr, num_splits, flags, ctypes.byref(p)))
    return p


def attn_decode_plan_prefix(desc: AttnDecodeDesc, max_context_len: int, prefix_group: int, prefix_len: int,
                            flags: int = 0) -> AttnDecodePrefixPlan:
    """Plan for batches whose groups of prefix_group consecutive requests share
    their first prefix_len keys (the same page ids).  Where the shared pass
    would not pay (the rule in include/attn_decode.h) the result is the
    default plan (prefix_len 0) unless flags hold ATTN_PLAN_SHARED_PASS."""
    p = AttnDecodePrefixPlan()
    _check(lib().attn_decode_plan_prefix(ctypes.byref(desc), max_context_len, prefix_group, prefix_len, flags,
                                         ctypes.byref(p)))
    return p


def attn_decode_run_prefix(plan, q, k_cache, v_cache, page_table, context_lens, scale, out, lse, workspace,
                           workspace_bytes=None, stream=None):
    wb = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
    _check(lib().attn_decode_run_prefix(ctypes.byref(plan), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(page_table), _ptr(context_lens), float(scale), _ptr(out), _ptr(lse),
                                        _ptr(workspace), wb, _stream(stream)))


def attn_decode_run(plan, q, k_cache, v_cache, page_table, context_lens, scale, num_splits, out,
                    lse, workspace, workspace_bytes=None, stream=None):
    wb = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
    _check(lib().attn_decode_run(ctypes.byref(plan), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(page_table), _ptr(context_lens), float(scale), int(num_splits),
                                 _ptr(out), _ptr(lse), _ptr(workspace), wb, _stream(stream)))


def attn_decode_run_noalloc(plan, q, k_cache, v_cache, page_table, context_lens, scale, num_splits, out,
                            lse, stream=None):
    """attn_decode_run with the workspace in the library's static device
    scratch (NOALLOC_SCRATCH_BYTES per GPU): nothing is allocated.  Calls
    that overlap in time on one GPU race on that scratch."""
    _check(lib().attn_decode_run_noalloc(ctypes.byref(plan), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(page_table), _ptr(context_lens), float(scale), int(num_splits),
                                         _ptr(out), _ptr(lse), _stream(stream)))


def attn_decode_partials(plan, q, k_cache, v_cache, page_table, context_lens, scale, num_splits,
                         workspace, workspace_bytes=None, stream=None):
    wb = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
    _check(lib().attn_decode_partials(ctypes.byref(plan), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(page_table), _ptr(context_lens), float(scale), int(num_splits),
                                      _ptr(workspace), wb, _stream(stream)))


def attn_decode_merge(plan, num_splits, workspace, out, lse, workspace_bytes=None, stream=None):
    wb = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
    _check(lib().attn_decode_merge(ctypes.byref(plan), int(num_splits), _ptr(workspace), wb, _ptr(out),
                                   _ptr(lse), _stream(stream)))


def attn_decode_workspace_layout(plan, num_splits: int = 0) -> tuple:
    o, l_, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().attn_decode_workspace_layout(ctypes.byref(plan), num_splits, ctypes.byref(o),
                                              ctypes.byref(l_), ctypes.byref(b)))
    return o.value, l_.value, b.value


def attn_decode_workspace_init(plan, workspace, workspace_bytes=None, stream=None):
    """Zero the in-kernel merge's counters of a workspace (a no-op for plans
    without ATTN_PLAN_FUSED_MERGE); once per workspace before its first run."""
    wb = workspace_bytes if workspace_bytes is not None else _nbytes(workspace)
    _check(lib().attn_decode_workspace_init(ctypes.byref(plan), _ptr(workspace), wb, _stream(stream)))


def attn_decode_split_range(plan, context_len: int, num_splits: int, split: int) -> tuple:
    b, e = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().attn_decode_split_range(ctypes.byref(plan), context_len, num_splits, split,
                                         ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def attn_decode_last_error() -> str:
    return lib().attn_decode_last_error().decode()


def _nbytes(t) -> int:
    if t is None:
        return 0
    return t.numel() * t.element_size()
