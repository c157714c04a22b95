"""MI355X-native paged GQA target-verify attention.

A thin Python binding over the C ABI of ``libva.so`` (include/va.h).  It only
marshals arguments: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.

    plan = Plan(num_seqs=16, num_q_heads=16, num_kv_heads=1, max_seqlen_q=4,
                max_seqlen_k=32768, max_blocks_per_seq=2048, num_blocks=32768,
                total_q=64, kv_dtype="fp8")
    out = plan.run(q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k,
                   softmax_scale=256 ** -0.5, k_descale=kd, v_descale=vd)

The library is loaded from this package directory.  If it is not built, the
first use raises ``RuntimeError``; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libva.so")

VA_OK, VA_ERR_INVALID_ARG, VA_ERR_UNSUPPORTED, VA_ERR_WORKSPACE, VA_ERR_HIP, VA_ERR_DEVICE_DATA = range(6)
VA_DT_BF16, VA_DT_FP8_E4M3FN = 1, 2
VA_STAGE_ALL, VA_STAGE_SPLIT_KV, VA_STAGE_MERGE = 0, 1, 2
VA_LAYOUT_PAGED, VA_LAYOUT_PREFIX_EXTEND = 0, 1
# va_validate result bits
VA_BAD_CU_SEQLENS_Q, VA_BAD_Q_LEN, VA_BAD_SEQUSED_K, VA_BAD_Q_GT_K, VA_BAD_PAGE = 1, 2, 4, 8, 16

EXPORTED = ("va_plan", "va_plan_workspace_bytes", "va_plan_grid", "va_run", "va_run_ex",
            "va_plan_destroy", "va_plan_kernel", "va_status_str", "va_fp8_to_bf16", "va_stream_pages", "va_spec_block_table",
            "va_validate", "va_run_prefix_extend", "va_run_timed", "va_set_stamp_buffer",
            "va_run_noalloc")

_lib = None


class VaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class _Problem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64), ("total_q", ctypes.c_int64),
        ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("num_cus", ctypes.c_int32), ("force_grid", ctypes.c_int32),
        ("window_left", ctypes.c_int32), ("softcap", ctypes.c_float),
        ("layout", ctypes.c_int32), ("v_head_dim", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
    ]


def library(path: str = LIB_PATH):
    """Load libva.so (once) and declare the C ABI."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m paged_gqa_attention_va_amd._build` "
                           "or __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.va_plan.restype = ctypes.c_int
    lib.va_plan.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(P)]
    lib.va_plan_workspace_bytes.restype = ctypes.c_int
    lib.va_plan_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.va_plan_grid.restype = ctypes.c_int
    lib.va_plan_grid.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.va_plan_kernel.restype = ctypes.c_int
    lib.va_plan_kernel.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    run_args = [P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, ctypes.c_size_t, P]
    lib.va_run.restype = ctypes.c_int
    lib.va_run.argtypes = run_args
    lib.va_run_ex.restype = ctypes.c_int
    lib.va_run_ex.argtypes = [P, ctypes.c_int32] + run_args[1:10] + [P] + run_args[10:]
    lib.va_plan_destroy.restype = None
    lib.va_plan_destroy.argtypes = [P]
    lib.va_status_str.restype = ctypes.c_char_p
    lib.va_status_str.argtypes = [ctypes.c_int]
    lib.va_spec_block_table.restype = ctypes.c_int
    lib.va_spec_block_table.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P]
    lib.va_run_prefix_extend.restype = ctypes.c_int
    lib.va_run_prefix_extend.argtypes = [P, ctypes.c_int32, P, P, P, P, P, ctypes.c_int64, P, P, P,
                                         ctypes.c_float, P, P, P, P, P, ctypes.c_size_t, P]
    lib.va_validate.restype = ctypes.c_int
    lib.va_validate.argtypes = [P, P, P, P, P, P]
    lib.va_fp8_to_bf16.restype = ctypes.c_int
    lib.va_fp8_to_bf16.argtypes = [P, P, ctypes.c_int64, P]
    lib.va_stream_pages.restype = ctypes.c_int
    lib.va_stream_pages.argtypes = [P, ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P]
    lib.va_run_timed.restype = ctypes.c_int
    lib.va_run_timed.argtypes = run_args[:10] + [P] + run_args[10:] + [P, P]
    lib.va_set_stamp_buffer.restype = ctypes.c_int
    lib.va_set_stamp_buffer.argtypes = [P, ctypes.c_size_t]
    lib.va_run_noalloc.restype = ctypes.c_int
    lib.va_run_noalloc.argtypes = run_args[:10] + [P, P, P]
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    try:
        return library().va_status_str(int(status)).decode()
    except RuntimeError:
        return "unknown"


def _check(status: int, where: str) -> None:
    if status != VA_OK:
        raise VaError(status, where)


def _same_device(device, *tensors) -> None:
    """Every tensor must live on ``device``: the kernels are launched there and
    dereference the pointers as that device's memory."""
    for t in tensors:
        if t is not None and t.device != device:
            raise ValueError(f"all tensors must be on {device}, got one on {t.device}")


def _dtype_code(name: str) -> int:
    if name in ("fp8", "fp8_e4m3fn", "float8_e4m3fn"):
        return VA_DT_FP8_E4M3FN
    if name in ("bf16", "bfloat16"):
        return VA_DT_BF16
    raise ValueError(f"unsupported dtype {name!r}")


class Plan:
    """A host-side plan for one problem shape (wraps va_plan / va_plan_destroy)."""

    def __init__(self, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                 max_seqlen_q: int, max_seqlen_k: int, max_blocks_per_seq: int,
                 num_blocks: int, total_q: int, kv_dtype: str = "fp8",
                 num_cus: int = 0, force_grid: int = 0, head_dim: int = 256,
                 window_left: int = -1, softcap: float = 0.0,
                 page_size: int = 16, q_dtype: str = "bf16", layout: str = "paged",
                 v_head_dim: int = 0, kernel: int = 0):
        self._lib = library()
        if layout not in ("paged", "prefix_extend"):
            raise ValueError(f"unknown layout {layout!r}")
        pr = _Problem(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
                      max_seqlen_q, max_seqlen_k, max_blocks_per_seq, num_blocks, total_q,
                      _dtype_code(q_dtype), _dtype_code(kv_dtype), num_cus, force_grid,
                      int(window_left), float(softcap),
                      VA_LAYOUT_PAGED if layout == "paged" else VA_LAYOUT_PREFIX_EXTEND, int(v_head_dim),
                      int(kernel))
        self.problem = pr
        self.v_head_dim = int(v_head_dim) or int(head_dim)
        self.kv_dtype = kv_dtype
        self.layout = layout
        h = ctypes.c_void_p()
        _check(self._lib.va_plan(ctypes.byref(pr), ctypes.byref(h)), "va_plan")
        self._h = h
        n = ctypes.c_size_t()
        _check(self._lib.va_plan_workspace_bytes(h, ctypes.byref(n)), "va_plan_workspace_bytes")
        self.workspace_bytes = int(n.value)
        g = ctypes.c_int32()
        _check(self._lib.va_plan_grid(h, ctypes.byref(g)), "va_plan_grid")
        self.grid = int(g.value)
        kk = ctypes.c_int32()
        _check(self._lib.va_plan_kernel(h, ctypes.byref(kk)), "va_plan_kernel")
        self.kernel = int(kk.value)        # FP8 paged GQA: 1 one wave per SIMD, 2 two row groups

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.va_plan_destroy(h)
            self._h = None

    @classmethod
    def for_problem(cls, p, **kw) -> "Plan":
        """Plan for a ``va_inputs.Problem``-like object (duck typed)."""
        return cls(num_seqs=p.num_seqs, num_q_heads=p.num_q_heads, num_kv_heads=p.num_kv_heads,
                   max_seqlen_q=max(1, p.max_seqlen_q), max_seqlen_k=p.max_seqlen_k,
                   max_blocks_per_seq=int(p.block_table.shape[1]), num_blocks=p.num_blocks,
                   total_q=p.total_q, kv_dtype=p.kv_dtype, head_dim=getattr(p, "head_dim", 256),
                   v_head_dim=getattr(p, "v_head_dim", None) or 0,
                   window_left=getattr(p, "window_left", -1), softcap=getattr(p, "softcap", 0.0), **kw)

    @classmethod
    def for_prefix_extend(cls, p, **kw) -> "Plan":
        """Plan for a ``va_inputs.PrefixExtendProblem``-like object (duck typed)."""
        return cls(num_seqs=p.num_seqs, num_q_heads=p.num_q_heads, num_kv_heads=p.num_kv_heads,
                   max_seqlen_q=max(1, p.max_seqlen_q), max_seqlen_k=p.max_seqlen_k,
                   max_blocks_per_seq=1, num_blocks=p.num_rows, page_size=1,
                   total_q=p.total_q, kv_dtype=p.kv_dtype, layout="prefix_extend",
                   window_left=getattr(p, "window_left", -1), softcap=getattr(p, "softcap", 0.0), **kw)

    def run_prefix_extend(self, q, k_buffer, v_buffer, kv_indptr, kv_indices, k_extend, v_extend,
                          cu_seqlens_q, softmax_scale: float, k_descale=None, v_descale=None,
                          out=None, workspace=None, stream=None, stage: int = VA_STAGE_ALL,
                          sinks=None):
        """Enqueue the attention of a prefix + extend call (va_run_prefix_extend).
        k_buffer / v_buffer: [rows, Hkv, 256]; k_extend / v_extend: [total_q, Hkv, 256]."""
        import torch
        pr = self.problem
        if self.layout != "prefix_extend":
            raise ValueError("run_prefix_extend needs a plan with layout='prefix_extend'")
        kv_ok = (torch.uint8, torch.float8_e4m3fn) if self.kv_dtype == "fp8" else (torch.bfloat16,)
        if q.dtype != torch.bfloat16 or tuple(q.shape) != (pr.total_q, pr.num_q_heads, pr.head_dim):
            raise ValueError(f"q must be bf16 [{pr.total_q}, {pr.num_q_heads}, {pr.head_dim}]")
        rows = pr.num_blocks * pr.page_size
        for name, t, shape in (("k_buffer", k_buffer, (rows, pr.num_kv_heads, pr.head_dim)),
                               ("v_buffer", v_buffer, (rows, pr.num_kv_heads, pr.head_dim)),
                               ("k_extend", k_extend, (pr.total_q, pr.num_kv_heads, pr.head_dim)),
                               ("v_extend", v_extend, (pr.total_q, pr.num_kv_heads, pr.head_dim))):
            if t.dtype not in kv_ok or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be {self.kv_dtype} {shape}, got {t.dtype} {tuple(t.shape)}")
        if kv_indptr.dtype != torch.int32 or tuple(kv_indptr.shape) != (pr.num_seqs + 1,):
            raise ValueError("kv_indptr must be int32 [num_seqs + 1]")
        if kv_indices.dtype != torch.int32 or kv_indices.dim() != 1:
            raise ValueError("kv_indices must be a 1-D int32 tensor")
        if cu_seqlens_q.dtype != torch.int32 or tuple(cu_seqlens_q.shape) != (pr.num_seqs + 1,):
            raise ValueError("cu_seqlens_q must be int32 [num_seqs + 1]")
        for name, t in (("k_descale", k_descale), ("v_descale", v_descale)):
            if t is not None and (t.dtype != torch.float32 or t.numel() < 1):
                raise ValueError(f"{name} must be a float32 device tensor with one element")
        if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != pr.num_q_heads):
            raise ValueError("sinks must be a float32 device tensor with num_q_heads elements")
        for t in (q, k_buffer, v_buffer, kv_indptr, kv_indices, k_extend, v_extend, cu_seqlens_q,
                  k_descale, v_descale, sinks):
            if t is not None and (not t.is_cuda or not t.is_contiguous()):
                raise ValueError("all tensors must be contiguous device tensors")
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.workspace(q.device)
        if out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous():
            raise ValueError("out must be a contiguous bf16 tensor shaped like q")
        _same_device(q.device, k_buffer, v_buffer, kv_indptr, kv_indices, k_extend, v_extend, cu_seqlens_q,
                     k_descale, v_descale, sinks, out, workspace)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        n_idx = kv_indices.numel()
        st = self._lib.va_run_prefix_extend(
            self._h, int(stage), ptr(q), ptr(k_buffer), ptr(v_buffer), ptr(kv_indptr),
            ptr(kv_indices) if n_idx else None, n_idx, ptr(k_extend), ptr(v_extend), ptr(cu_seqlens_q),
            ctypes.c_float(softmax_scale), ptr(k_descale), ptr(v_descale), ptr(sinks), ptr(out),
            ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
            ctypes.c_void_p(sptr))
        _check(st, "va_run_prefix_extend")
        return out

    def workspace(self, device=None):
        import torch
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device or "cuda")

    def run(self, q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, softmax_scale: float,
            k_descale=None, v_descale=None, out=None, workspace=None, stream=None,
            stage: int = VA_STAGE_ALL, sinks=None):
        """Enqueue the attention on ``stream`` (default: torch's current stream).
        sinks: optional float32 device tensor [Hq] of sink logits."""
        import torch
        self._check_tensors(q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k,
                            k_descale, v_descale)
        if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != self.problem.num_q_heads
                                  or not sinks.is_cuda or not sinks.is_contiguous()):
            raise ValueError("sinks must be a contiguous float32 device tensor with num_q_heads elements")
        oshape = (q.shape[0], q.shape[1], self.v_head_dim)
        if out is None:
            out = torch.empty(oshape, dtype=torch.bfloat16, device=q.device)
        if workspace is None:
            workspace = self.workspace(q.device)
        if out.dtype != torch.bfloat16 or tuple(out.shape) != oshape or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous bf16 tensor of shape {oshape}")
        if workspace.numel() * workspace.element_size() < self.workspace_bytes:
            raise ValueError("workspace smaller than plan.workspace_bytes")
        _same_device(q.device, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, k_descale, v_descale,
                     sinks, out, workspace)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        st = self._lib.va_run_ex(
            self._h, int(stage), ptr(q), ptr(k_pool), ptr(v_pool), ptr(block_table),
            ptr(cu_seqlens_q), ptr(seqused_k), ctypes.c_float(softmax_scale),
            ptr(k_descale), ptr(v_descale), ptr(sinks), ptr(out), ptr(workspace),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()),
            ctypes.c_void_p(sptr))
        _check(st, "va_run")
        return out

    def run_timed(self, q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, softmax_scale: float,
                  k_descale, v_descale, out, workspace, stream, main_start: int, main_stop: int, sinks=None):
        """Enqueue one whole call (va_run_timed) whose main-kernel dispatch records
        the two hipEvent_t handles main_start / main_stop (ints)."""
        self._check_tensors(q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, k_descale, v_descale)
        _same_device(q.device, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, k_descale, v_descale,
                     sinks, out, workspace)
        sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        st = self._lib.va_run_timed(
            self._h, ptr(q), ptr(k_pool), ptr(v_pool), ptr(block_table), ptr(cu_seqlens_q), ptr(seqused_k),
            ctypes.c_float(softmax_scale), ptr(k_descale), ptr(v_descale), ptr(sinks), ptr(out), ptr(workspace),
            ctypes.c_size_t(workspace.numel() * workspace.element_size()), ctypes.c_void_p(sptr),
            ctypes.c_void_p(main_start), ctypes.c_void_p(main_stop))
        _check(st, "va_run_timed")
        return out

    def run_noalloc(self, q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, softmax_scale: float,
                    k_descale=None, v_descale=None, out=None, stream=None, sinks=None):
        """Enqueue the attention through va_run_noalloc (the library's own scratch
        instead of a workspace; calls on one device must not overlap)."""
        import torch
        self._check_tensors(q, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, k_descale, v_descale)
        oshape = (q.shape[0], q.shape[1], self.v_head_dim)
        if out is None:
            out = torch.empty(oshape, dtype=torch.bfloat16, device=q.device)
        if out.dtype != torch.bfloat16 or tuple(out.shape) != oshape or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous bf16 tensor of shape {oshape}")
        if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != self.problem.num_q_heads
                                  or not sinks.is_cuda or not sinks.is_contiguous()):
            raise ValueError("sinks must be a contiguous float32 device tensor with num_q_heads elements")
        _same_device(q.device, k_pool, v_pool, block_table, cu_seqlens_q, seqused_k, k_descale, v_descale,
                     sinks, out)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        st = self._lib.va_run_noalloc(
            self._h, ptr(q), ptr(k_pool), ptr(v_pool), ptr(block_table), ptr(cu_seqlens_q), ptr(seqused_k),
            ctypes.c_float(softmax_scale), ptr(k_descale), ptr(v_descale), ptr(sinks), ptr(out),
            ctypes.c_void_p(sptr))
        _check(st, "va_run_noalloc")
        return out

    def validate(self, block_table, cu_seqlens_q, seqused_k, result=None, stream=None):
        """Enqueue va_validate; returns the int32 device tensor [bits, first bad
        sequence] (read it after the stream has reached it)."""
        import torch
        pr = self.problem
        meta = ((block_table, (pr.num_seqs, pr.max_blocks_per_seq)), (cu_seqlens_q, (pr.num_seqs + 1,)),
                (seqused_k, (pr.num_seqs,)))
        for t, shape in meta:
            if t.dtype != torch.int32 or tuple(t.shape) != shape or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"metadata must be contiguous int32 device tensors shaped {shape}")
        if result is None:
            result = torch.empty(2, dtype=torch.int32, device=block_table.device)
        if result.dtype != torch.int32 or result.numel() < 2 or not result.is_contiguous():
            raise ValueError("result must be a contiguous int32 tensor with 2 elements")
        _same_device(block_table.device, cu_seqlens_q, seqused_k, result)
        if stream is None:
            stream = torch.cuda.current_stream(block_table.device)
        sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        _check(self._lib.va_validate(self._h, ctypes.c_void_p(block_table.data_ptr()),
                                     ctypes.c_void_p(cu_seqlens_q.data_ptr()),
                                     ctypes.c_void_p(seqused_k.data_ptr()),
                                     ctypes.c_void_p(result.data_ptr()), ctypes.c_void_p(sptr)),
               "va_validate")
        return result

    def _check_tensors(self, q, k_pool, v_pool, block_table, cu, seqused, kd, vd):
        import torch
        pr = self.problem
        if q.dtype != torch.bfloat16 or q.dim() != 3 or tuple(q.shape) != (pr.total_q, pr.num_q_heads, pr.head_dim):
            raise ValueError(f"q must be bf16 [{pr.total_q}, {pr.num_q_heads}, {pr.head_dim}], got {q.dtype} {tuple(q.shape)}")
        kv_ok = (torch.uint8, torch.float8_e4m3fn) if self.kv_dtype == "fp8" else (torch.bfloat16,)
        shape = (pr.num_blocks, pr.page_size, pr.num_kv_heads, pr.head_dim)
        for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
            if t.dtype not in kv_ok or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be {self.kv_dtype} {shape}, got {t.dtype} {tuple(t.shape)}")
        if tuple(block_table.shape) != (pr.num_seqs, pr.max_blocks_per_seq) or block_table.dtype != torch.int32:
            raise ValueError("block_table must be int32 [num_seqs, max_blocks_per_seq]")
        if tuple(cu.shape) != (pr.num_seqs + 1,) or cu.dtype != torch.int32:
            raise ValueError("cu_seqlens_q must be int32 [num_seqs + 1]")
        if tuple(seqused.shape) != (pr.num_seqs,) or seqused.dtype != torch.int32:
            raise ValueError("seqused_k must be int32 [num_seqs]")
        for name, t in (("k_descale", kd), ("v_descale", vd)):
            if t is not None and (t.dtype != torch.float32 or t.numel() < 1):
                raise ValueError(f"{name} must be a float32 device tensor with one element")
        for t in (q, k_pool, v_pool, block_table, cu, seqused, kd, vd):
            if t is not None and (not t.is_cuda or not t.is_contiguous()):
                raise ValueError("all tensors must be contiguous device tensors")


def fp8_to_bf16(codes, stream=None):
    """Device fp8 e4m3fn -> bf16 with the kernels' own in-register conversion."""
    import torch
    lib = library()
    codes = codes.contiguous().view(torch.uint8)
    out = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device)
    if stream is None:
        stream = torch.cuda.current_stream(codes.device)
    _check(lib.va_fp8_to_bf16(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                              codes.numel(), ctypes.c_void_p(stream.cuda_stream)), "va_fp8_to_bf16")
    return out


def stream_pages(pool, pages, depth: int = 10, grid: int = 256, sums=None, stream=None):
    """Diagnostic streaming ceiling (va_stream_pages): copy the 4 KiB pages
    pool[4096 * pages[i]] into LDS as the FP8 kernel's ring does and nothing
    else.  pool: a device uint8 tensor, pages: a device int32 tensor.  Returns
    the per-wave sums of each page's first 32-bit word, modulo 2^32 (an int32
    tensor of grid * 4 holding the uint32 bits)."""
    import torch
    lib = library()
    if pool.dtype != torch.uint8 or not pool.is_cuda or not pool.is_contiguous():
        raise ValueError("pool must be a contiguous device uint8 tensor")
    if pages.dtype != torch.int32 or not pages.is_cuda or not pages.is_contiguous():
        raise ValueError("pages must be a contiguous device int32 tensor")
    if sums is None:
        sums = torch.zeros(grid * 4, dtype=torch.int32, device=pool.device)
    if stream is None:
        stream = torch.cuda.current_stream(pool.device)
    _check(lib.va_stream_pages(ctypes.c_void_p(pool.data_ptr()), pool.numel(), ctypes.c_void_p(pages.data_ptr()),
                               pages.numel(), depth, grid, ctypes.c_void_p(sums.data_ptr()),
                               ctypes.c_void_p(stream.cuda_stream)), "va_stream_pages")
    return sums


def set_stamp_buffer(buf, lib=None) -> None:
    """Point a VA_STAMPS build of the library at a device buffer (a uint8 or
    int64 tensor) for phase timestamps; None turns recording off."""
    lib = lib or library()
    if buf is None:
        _check(lib.va_set_stamp_buffer(None, 0), "va_set_stamp_buffer")
    else:
        _check(lib.va_set_stamp_buffer(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size()),
               "va_set_stamp_buffer")


def build(verbose: bool = False) -> str:
    """Compile libva.so in-tree (hipcc, gfx950)."""
    from . import _build as _b
    global _lib
    _lib = None
    return _b.build(verbose=verbose)


def spec_block_table(kv_indptr, kv_indices, max_blocks_per_seq: int, page_size: int = 16,
                     stream=None):
    """Device block table and seqused_k of a draft-extend call from its spec
    metadata (kv_indptr [B+1], kv_indices: int32 device tensors)."""
    import torch
    lib = library()
    B = kv_indptr.numel() - 1
    for t in (kv_indptr, kv_indices):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("kv_indptr and kv_indices must be contiguous int32 device tensors")
    _same_device(kv_indptr.device, kv_indices)
    bt = torch.empty((B, max_blocks_per_seq), dtype=torch.int32, device=kv_indptr.device)
    sk = torch.empty((B,), dtype=torch.int32, device=kv_indptr.device)
    if stream is None:
        stream = torch.cuda.current_stream(kv_indptr.device)
    idx = kv_indices if kv_indices.numel() else torch.zeros(1, dtype=torch.int32, device=kv_indptr.device)
    _check(lib.va_spec_block_table(ctypes.c_void_p(kv_indptr.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                                   B, page_size, max_blocks_per_seq, ctypes.c_void_p(bt.data_ptr()),
                                   ctypes.c_void_p(sk.data_ptr()), ctypes.c_void_p(stream.cuda_stream)),
           "va_spec_block_table")
    return bt, sk
