"""Dynamic block-sparse attention from block means, on AMD MI355X (gfx950).

Thin Python binding of libsparse_attn.so (declared in include/sparse_attn.h): argument
marshalling only. Every step of the path runs in the library's HIP kernels; torch only
provides device memory and the current stream. There is no CPU fallback: without the
built library every call raises.

    plan = plan(q, k, block_q=128, block_k=64, keep=0.1)        # int32 [B,H,nQ,n_keep]
    out  = forward(q, k, v, plan, block_q=128, block_k=64, mode="int8fp8")

q, k, v are CUDA tensors of logical shape [B, H, L, 128] (any strides with the last
dimension contiguous, e.g. a [B, L, H, D] tensor viewed through .transpose(1, 2)).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SA_MODE_BF16", "SA_MODE_INT8_FP8", "attend", "debug_qk_tile", "debug_qk_tile_fp8", "forward", "forward_layout",
    "forward_workspace_bytes", "lib", "n_keep", "num_blocks", "plan", "plan_prepare",
    "plan_prologue_workspace_bytes", "plan_workspace_bytes", "plan_noalloc", "plan_noalloc_max_bytes",
    "pool", "prepare", "select", "library_path", "ulysses_pack_head", "ulysses_pack_seq",
    "ulysses_payload_bytes", "ulysses_unpack_head", "ulysses_unpack_seq", "nvfp4_quantize", "nvfp4_gemm",
]

SA_MODE_BF16 = 0
SA_MODE_INT8_FP8 = 1
SA_MODE_FP8 = 2
SA_DTYPE_FP32 = 0
SA_DTYPE_BF16 = 1
_MODES = {"bf16": SA_MODE_BF16, "int8fp8": SA_MODE_INT8_FP8, "fp8": SA_MODE_FP8}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse_attn.so")


class SaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("L", ctypes.c_int64),
                ("D", ctypes.c_int64), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_l", ctypes.c_int64)]


class SaForwardLayout(ctypes.Structure):
    _fields_ = [("nQ", ctypes.c_int64), ("nK", ctypes.c_int64), ("q_off", ctypes.c_size_t),
                ("k_off", ctypes.c_size_t), ("v_off", ctypes.c_size_t), ("sq_off", ctypes.c_size_t),
                ("sk_off", ctypes.c_size_t), ("sv_off", ctypes.c_size_t), ("total", ctypes.c_size_t)]


class SaQkPrologue(ctypes.Structure):
    _fields_ = [("q_gain", ctypes.c_void_p), ("k_gain", ctypes.c_void_p), ("eps", ctypes.c_double),
                ("grid_t", ctypes.c_int64), ("grid_h", ctypes.c_int64), ("grid_w", ctypes.c_int64),
                ("theta", ctypes.c_double)]


_lib = None
_P = ctypes.POINTER


def lib():
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is not built; run `python -m dynamic_block_sparse_mean_amd.build`")
    L = ctypes.CDLL(library_path)
    i64, i32, vp, sz, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_double
    T = _P(SaTensor)
    sig = {
        "sa_status_string": (ctypes.c_char_p, [i32]),
        "sa_last_error": (ctypes.c_char_p, []),
        "sa_num_blocks": (i64, [i64, i64]),
        "sa_plan_n_keep": (i64, [i64, dbl]),
        "sa_plan_workspace_bytes": (i32, [i64, i64, i64, i64, i32, i32, _P(sz)]),
        "sa_forward_workspace_bytes": (i32, [i64, i64, i64, i64, i32, i32, i32, _P(sz)]),
        "sa_forward_workspace_layout": (i32, [i64, i64, i64, i64, i32, i32, i32, _P(SaForwardLayout)]),
        "sparse_attn_plan": (i32, [T, T, i32, i32, dbl, vp, i64, vp, sz, vp]),
        "sparse_attn_forward": (i32, [T, T, T, vp, i32, i32, i64, i32, ctypes.c_float, T, vp, sz, vp]),
        "sparse_attn_plan_prepare": (i32, [T, T, T, i32, i32, dbl, i32, vp, i64, vp, sz, vp, sz, vp]),
        "sa_plan_prologue_workspace_bytes": (i32, [i64, i64, i64, i64, i32, i32, i64, i64, i64, _P(sz)]),
        "sparse_attn_plan_prepare_prologue": (i32, [T, T, T, i32, i32, dbl, i32, _P(SaQkPrologue), vp, i64,
                                                    vp, sz, vp, sz, vp]),
        "sparse_attn_pool": (i32, [T, i32, vp, vp]),
        "sparse_attn_select": (i32, [vp, vp, i64, i64, i64, i64, i64, i64, vp, vp, sz, vp]),
        "sparse_attn_prepare": (i32, [T, T, T, i32, i32, i32, vp, sz, vp]),
        "sparse_attn_attend": (i32, [T, vp, i32, i32, i64, i32, ctypes.c_float, T, vp, sz, vp]),
        "sparse_attn_debug_qk_tile": (i32, [vp, sz, i64, i64, i64, i64, i32, i32, vp, i64, i64, i64,
                                            i64, i64, vp, vp]),
        "sparse_attn_debug_qk_tile_fp8": (i32, [vp, sz, i64, i64, i64, i64, i32, i32, vp, i64, i64, i64,
                                                i64, i64, vp, vp]),
        "sa_plan_noalloc_max_bytes": (sz, []),
        "sparse_attn_plan_noalloc": (i32, [T, T, i32, i32, dbl, vp, i64, vp]),
        "sa_nvfp4_quantize_workspace_bytes": (i32, [i64, i64, _P(sz)]),
        "sa_nvfp4_quantize": (i32, [vp, i64, i64, i64, vp, vp, vp, vp, sz, vp]),
        "sa_nvfp4_gemm": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp]),
        "sa_ulysses_payload_bytes": (i32, [i64, i64, i64, i64, i32, i32, _P(sz), _P(sz)]),
        "sa_ulysses_pack_seq": (i32, [T, i32, i64, i32, i32, i32, i32, vp, sz, vp]),
        "sa_ulysses_unpack_head": (i32, [vp, sz, i32, T, i32, vp]),
        "sa_ulysses_pack_head": (i32, [T, i32, i32, vp, sz, vp]),
        "sa_ulysses_unpack_seq": (i32, [vp, sz, i64, i32, i32, i32, i32, T, i32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise RuntimeError(f"{what}: {L.sa_status_string(status).decode()}: {L.sa_last_error().decode()}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _desc(x: torch.Tensor, name: str) -> SaTensor:
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if x.dim() != 4:
        raise ValueError(f"{name} must have 4 dims [B, H, L, D], got {tuple(x.shape)}")
    if x.dtype == torch.bfloat16:
        dt = SA_DTYPE_BF16
    elif x.dtype == torch.float32:
        dt = SA_DTYPE_FP32
    else:
        raise ValueError(f"{name}: dtype {x.dtype} not supported (bf16 or fp32)")
    if x.stride(3) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    B, H, L, D = x.shape
    sb, sh, sl, _ = x.stride()
    return SaTensor(x.data_ptr(), dt, 0, B, H, L, D, sb, sh, sl)


def _mode(mode) -> int:
    if isinstance(mode, str):
        if mode not in _MODES:
            raise ValueError(f"mode must be one of {list(_MODES)}")
        return _MODES[mode]
    return int(mode)


# ---- sizes --------------------------------------------------------------------------
def num_blocks(L: int, block: int) -> int:
    return int(lib().sa_num_blocks(L, block))


def n_keep(nK: int, keep: float) -> int:
    n = int(lib().sa_plan_n_keep(nK, float(keep)))
    if n < 0:
        raise ValueError(f"keep={keep} not in (0, 1] or nK={nK} < 1")
    return n


def plan_workspace_bytes(B, H, L, D, block_q, block_k) -> int:
    out = ctypes.c_size_t()
    _check(lib().sa_plan_workspace_bytes(B, H, L, D, block_q, block_k, ctypes.byref(out)),
           "sa_plan_workspace_bytes")
    return out.value


def forward_workspace_bytes(B, H, L, D, block_q, block_k, mode="int8fp8") -> int:
    out = ctypes.c_size_t()
    _check(lib().sa_forward_workspace_bytes(B, H, L, D, block_q, block_k, _mode(mode), ctypes.byref(out)),
           "sa_forward_workspace_bytes")
    return out.value


def forward_layout(B, H, L, D, block_q, block_k, mode="int8fp8") -> dict:
    lay = SaForwardLayout()
    _check(lib().sa_forward_workspace_layout(B, H, L, D, block_q, block_k, _mode(mode), ctypes.byref(lay)),
           "sa_forward_workspace_layout")
    return {f: getattr(lay, f) for f, _ in SaForwardLayout._fields_}


def _check_plan(p, B, H, nQ, nk=None, device=None, name="plan_idx"):
    if not (isinstance(p, torch.Tensor) and p.is_cuda and p.dtype == torch.int32 and p.is_contiguous()
            and p.dim() == 4 and tuple(p.shape[:3]) == (B, H, nQ)
            and (nk is None or p.shape[3] == nk) and (device is None or p.device == device)):
        want = nk if nk is not None else "n_keep"
        raise ValueError(f"{name} must be a contiguous int32 tensor [{B}, {H}, {nQ}, {want}] on "
                         f"{device if device is not None else 'the inputs device'}")


def _workspace(nbytes, device, given):
    if given is not None:
        if not (isinstance(given, torch.Tensor) and given.is_cuda and given.device == device
                and given.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous CUDA tensor on {device}")
        if given.numel() * given.element_size() < nbytes:
            raise ValueError(f"workspace has {given.numel() * given.element_size()} bytes, needs {nbytes}")
        return given
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


# ---- the method ------------------------------------------------------------------------
def plan(q, k, block_q=128, block_k=64, keep=0.1, out=None, workspace=None):
    """Per query block, the ascending indices of the kept key blocks: int32 [B, H, nQ, n_keep]."""
    dq, dk = _desc(q, "q"), _desc(k, "k")
    B, H, L, D = q.shape
    nQ, nK = num_blocks(L, block_q), num_blocks(L, block_k)
    nk = n_keep(nK, keep)
    if out is None:
        out = torch.empty((B, H, nQ, nk), dtype=torch.int32, device=q.device)
    _check_plan(out, B, H, nQ, nk, q.device, "out")
    ws = _workspace(plan_workspace_bytes(B, H, L, D, block_q, block_k), q.device, workspace)
    _check(lib().sparse_attn_plan(ctypes.byref(dq), ctypes.byref(dk), block_q, block_k, float(keep),
                                  out.data_ptr(), nk, ws.data_ptr(), ws.numel() * ws.element_size(),
                                  _stream()), "sparse_attn_plan")
    return out


def plan_noalloc_max_bytes() -> int:
    """Scratch limit of plan_noalloc (bytes of sa_plan_workspace_bytes it accepts)."""
    return lib().sa_plan_noalloc_max_bytes()


def plan_noalloc(q, k, block_q, block_k, keep, out):
    """`plan` into a caller-given `out` with no allocation at all: the library's own fixed
    device scratch stands in for the workspace (see sparse_attn_plan_noalloc)."""
    dq, dk = _desc(q, "q"), _desc(k, "k")
    B, H, L, D = q.shape
    nQ, nK = num_blocks(L, block_q), num_blocks(L, block_k)
    nk = n_keep(nK, keep)
    _check_plan(out, B, H, nQ, nk, q.device, "out")
    _check(lib().sparse_attn_plan_noalloc(ctypes.byref(dq), ctypes.byref(dk), block_q, block_k, float(keep),
                                          out.data_ptr(), nk, _stream()), "sparse_attn_plan_noalloc")
    return out


def plan_prologue_workspace_bytes(B, H, L, D, block_q, block_k, grid) -> int:
    out = ctypes.c_size_t()
    _check(lib().sa_plan_prologue_workspace_bytes(B, H, L, D, block_q, block_k, *grid, ctypes.byref(out)),
           "sa_plan_prologue_workspace_bytes")
    return out.value


def _gain(g, H, D, name):
    if not (isinstance(g, torch.Tensor) and g.is_cuda and g.dtype == torch.float32 and g.is_contiguous()
            and tuple(g.shape) == (H, D)):
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor [{H}, {D}]")
    return g


def plan_prepare(q, k, v, block_q=128, block_k=64, keep=0.1, mode="int8fp8", out=None,
                 plan_workspace=None, workspace=None, prologue=None):
    """`plan` and `prepare` with one pass over the inputs; returns (plan_idx, forward workspace).

    prologue: None, or a dict with q_gain and k_gain (float32 [H, D] CUDA tensors), eps, grid
    (T, Hg, Wg) and theta (default 10000): Q and K then go through RMSNorm and 3-D RoPE first,
    in the same pass. In bf16 mode the workspace then holds the normalized, rotated Q (bf16),
    which `attend` reads instead of its q argument."""
    B, H, L, D = q.shape
    m = _mode(mode)
    nQ, nK = num_blocks(L, block_q), num_blocks(L, block_k)
    nk = n_keep(nK, keep)
    if out is None:
        out = torch.empty((B, H, nQ, nk), dtype=torch.int32, device=q.device)
    _check_plan(out, B, H, nQ, nk, q.device, "out")
    if prologue is None:
        pbytes = plan_workspace_bytes(B, H, L, D, block_q, block_k)
    else:
        pbytes = plan_prologue_workspace_bytes(B, H, L, D, block_q, block_k, tuple(prologue["grid"]))
    pws = _workspace(pbytes, q.device, plan_workspace)
    fws = _workspace(forward_workspace_bytes(B, H, L, D, block_q, block_k, m), q.device, workspace)
    dq, dk, dv = _desc(q, "q"), _desc(k, "k"), _desc(v, "v")
    common = (block_q, block_k, float(keep), m)
    tail = (out.data_ptr(), nk, pws.data_ptr(), pws.numel() * pws.element_size(), fws.data_ptr(),
            fws.numel() * fws.element_size(), _stream())
    if prologue is None:
        _check(lib().sparse_attn_plan_prepare(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), *common,
                                              *tail), "sparse_attn_plan_prepare")
    else:
        gq = _gain(prologue["q_gain"], H, D, "q_gain")
        gk = _gain(prologue["k_gain"], H, D, "k_gain")
        T_, Hg, Wg = prologue["grid"]
        pro = SaQkPrologue(gq.data_ptr(), gk.data_ptr(), float(prologue["eps"]), T_, Hg, Wg,
                           float(prologue.get("theta", 10000.0)))
        _check(lib().sparse_attn_plan_prepare_prologue(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                                                       *common, ctypes.byref(pro), *tail),
               "sparse_attn_plan_prepare_prologue")
    return out, fws


def forward(q, k, v, plan_idx, block_q=128, block_k=64, mode="int8fp8", sm_scale=None, out=None,
            workspace=None):
    """Block-sparse attention over `plan_idx`; returns bf16 [B, H, L, D]."""
    B, H, L, D = q.shape
    m = _mode(mode)
    if out is None:
        out = torch.empty((B, H, L, D), dtype=torch.bfloat16, device=q.device)
    ws = _workspace(forward_workspace_bytes(B, H, L, D, block_q, block_k, m), q.device, workspace)
    _check_plan(plan_idx, B, H, num_blocks(L, block_q))
    dq, dk, dv, do = _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), _desc(out, "out")
    _check(lib().sparse_attn_forward(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                                     plan_idx.data_ptr(), block_q, block_k, plan_idx.shape[-1], m,
                                     float(sm_scale or 0.0), ctypes.byref(do), ws.data_ptr(),
                                     ws.numel() * ws.element_size(), _stream()), "sparse_attn_forward")
    return out


# ---- stage calls -------------------------------------------------------------------------
def pool(x, block):
    """fp64 block means [B, H, n, D] of x over blocks of `block` tokens."""
    d = _desc(x, "x")
    B, H, L, D = x.shape
    means = torch.empty((B, H, num_blocks(L, block), D), dtype=torch.float64, device=x.device)
    _check(lib().sparse_attn_pool(ctypes.byref(d), block, means.data_ptr(), _stream()), "sparse_attn_pool")
    return means


def select(q_means, k_means, n_keep_, out=None, workspace=None):
    """Top-n_keep key blocks per query block from fp64 means (as `pool` returns them)."""
    for name, m in (("q_means", q_means), ("k_means", k_means)):
        if not (isinstance(m, torch.Tensor) and m.is_cuda and m.dtype == torch.float64 and m.dim() == 4):
            raise ValueError(f"{name} must be a float64 CUDA tensor [B, H, n, D]")
    B, H, nQ, D = q_means.shape
    nK = k_means.shape[2]
    if (k_means.shape[0], k_means.shape[1], k_means.shape[3]) != (B, H, D) or k_means.device != q_means.device:
        raise ValueError(f"k_means must be [{B}, {H}, nK, {D}] on {q_means.device}, got "
                         f"{tuple(k_means.shape)} on {k_means.device}")
    q_means, k_means = q_means.contiguous(), k_means.contiguous()
    if out is None:
        out = torch.empty((B, H, nQ, n_keep_), dtype=torch.int32, device=q_means.device)
    _check_plan(out, B, H, nQ, n_keep_, q_means.device, "out")
    ws = _workspace(B * H * nQ * nK * 8, q_means.device, workspace)
    _check(lib().sparse_attn_select(q_means.data_ptr(), k_means.data_ptr(), B, H, nQ, nK, D, n_keep_,
                                    out.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                    _stream()), "sparse_attn_select")
    return out


def prepare(q, k, v, block_q=128, block_k=64, mode="int8fp8", workspace=None):
    """Run the prepare stage; returns the forward workspace (uint8 tensor)."""
    B, H, L, D = q.shape
    m = _mode(mode)
    ws = _workspace(forward_workspace_bytes(B, H, L, D, block_q, block_k, m), q.device, workspace)
    dq, dk, dv = _desc(q, "q"), _desc(k, "k"), _desc(v, "v")
    _check(lib().sparse_attn_prepare(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), block_q,
                                     block_k, m, ws.data_ptr(), ws.numel() * ws.element_size(),
                                     _stream()), "sparse_attn_prepare")
    return ws


def attend(q, plan_idx, workspace, block_q=128, block_k=64, mode="int8fp8", sm_scale=None, out=None):
    """Run the attend stage on a workspace written by `prepare`."""
    B, H, L, D = q.shape
    _check_plan(plan_idx, B, H, num_blocks(L, block_q))
    if out is None:
        out = torch.empty((B, H, L, D), dtype=torch.bfloat16, device=q.device)
    dq, do = _desc(q, "q"), _desc(out, "out")
    _check(lib().sparse_attn_attend(ctypes.byref(dq), plan_idx.data_ptr(), block_q, block_k,
                                    plan_idx.shape[-1], _mode(mode), float(sm_scale or 0.0),
                                    ctypes.byref(do), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream()),
           "sparse_attn_attend")
    return out


def debug_qk_tile(workspace, shape, block_q, block_k, plan_idx, b, h, i, t):
    """int32 [block_q, block_k] tile S = Q^_i K^_j^T (j = plan_idx[b, h, i, t]) from the INT8 path."""
    B, H, L, D = shape
    out = torch.empty((block_q, block_k), dtype=torch.int32, device=workspace.device)
    _check(lib().sparse_attn_debug_qk_tile(workspace.data_ptr(), workspace.numel(), B, H, L, D, block_q,
                                           block_k, plan_idx.data_ptr(), plan_idx.shape[-1], b, h, i, t,
                                           out.data_ptr(), _stream()), "sparse_attn_debug_qk_tile")
    return out


def debug_qk_tile_fp8(workspace, shape, block_q, block_k, plan_idx, b, h, i, t):
    """fp32 [block_q, block_k] scores (s_q Q^_i)(s_k K^_j)^T from an all-FP8 workspace, through
    the scaled FP8 MFMA path of that mode (j = plan_idx[b, h, i, t])."""
    B, H, L, D = shape
    out = torch.empty((block_q, block_k), dtype=torch.float32, device=workspace.device)
    _check(lib().sparse_attn_debug_qk_tile_fp8(workspace.data_ptr(), workspace.numel(), B, H, L, D, block_q,
                                               block_k, plan_idx.data_ptr(), plan_idx.shape[-1], b, h, i, t,
                                               out.data_ptr(), _stream()), "sparse_attn_debug_qk_tile_fp8")
    return out


# ---- Light-Ulysses FP8 exchange payload -------------------------------------------------------
def _descs(tensors, name):
    tensors = list(tensors)
    if not 1 <= len(tensors) <= 3:
        raise ValueError(f"{name}: 1 to 3 tensors, got {len(tensors)}")
    arr = (SaTensor * len(tensors))(*[_desc(t, f"{name}[{i}]") for i, t in enumerate(tensors)])
    return arr, len(tensors)


def ulysses_payload_bytes(B, head_count, L, peers, n_tensors, D=128):
    """(bytes of one chunk, bytes of the whole payload of `peers` chunks)."""
    chunk, total = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().sa_ulysses_payload_bytes(B, head_count, L, D, peers, n_tensors, ctypes.byref(chunk),
                                          ctypes.byref(total)), "sa_ulysses_payload_bytes")
    return chunk.value, total.value


def _payload(nbytes, device, given):
    if given is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if given.dtype != torch.uint8 or not given.is_contiguous() or given.numel() < nbytes:
        raise ValueError(f"payload must be a contiguous uint8 tensor of at least {nbytes} bytes")
    return given


def ulysses_pack_seq(tensors, L, peers, rank, head_begin=0, head_count=None, payload=None):
    """Pack this peer's token shard of each tensor ([B, H, L_r, D] bf16) for the sequence-to-head
    all-to-all: returns the uint8 payload of `peers` equal chunks (chunk c goes to peer c)."""
    arr, n = _descs(tensors, "tensors")
    B, H = arr[0].B, arr[0].H
    hc = H // peers - head_begin if head_count is None else head_count
    _, total = ulysses_payload_bytes(B, hc, L, peers, n)
    payload = _payload(total, tensors[0].device, payload)
    _check(lib().sa_ulysses_pack_seq(arr, n, L, peers, rank, head_begin, hc, payload.data_ptr(),
                                     payload.numel(), _stream()), "sa_ulysses_pack_seq")
    return payload


def ulysses_unpack_head(payload, peers, outs):
    """Unpack a received payload (chunk c from the peer of token shard c) into the head-side
    tensors `outs` ([B, head_count, L, D] bf16, written in place); returns outs."""
    arr, n = _descs(outs, "outs")
    if payload.dtype != torch.uint8 or not payload.is_contiguous():
        raise ValueError("payload must be a contiguous uint8 tensor")
    _check(lib().sa_ulysses_unpack_head(payload.data_ptr(), payload.numel(), peers, arr, n, _stream()),
           "sa_ulysses_unpack_head")
    return outs


def ulysses_pack_head(tensors, peers, payload=None):
    """Pack head-side tensors ([B, head_count, L, D] bf16) for the head-to-sequence all-to-all:
    chunk c holds the tokens of shard c."""
    arr, n = _descs(tensors, "tensors")
    _, total = ulysses_payload_bytes(arr[0].B, arr[0].H, arr[0].L, peers, n)
    payload = _payload(total, tensors[0].device, payload)
    _check(lib().sa_ulysses_pack_head(arr, n, peers, payload.data_ptr(), payload.numel(), _stream()),
           "sa_ulysses_pack_head")
    return payload


def ulysses_unpack_seq(payload, L, peers, rank, outs, head_begin=0, head_count=None):
    """Unpack a received payload (chunk c from the peer of head group c) into this peer's token
    shard `outs` ([B, H, L_r, D] bf16); heads c*(H/P) + [head_begin, head_begin + head_count)
    are written. Returns outs."""
    arr, n = _descs(outs, "outs")
    if payload.dtype != torch.uint8 or not payload.is_contiguous():
        raise ValueError("payload must be a contiguous uint8 tensor")
    hc = arr[0].H // peers - head_begin if head_count is None else head_count
    _check(lib().sa_ulysses_unpack_seq(payload.data_ptr(), payload.numel(), L, peers, rank, head_begin, hc,
                                       arr, n, _stream()), "sa_ulysses_unpack_seq")
    return outs


# ---- NVFP4 block-scaled GEMM --------------------------------------------------------------------
def nvfp4_quantize(x, out=None, workspace=None):
    """Quantize a bf16 CUDA matrix x [rows, K] (last dim contiguous) to NVFP4: returns
    (codes uint8 [rows, K/2], scales uint8 [rows, K/16] E4M3 bits, tensor scale float32 [1])."""
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2
            and x.stride(1) == 1):
        raise ValueError("x must be a bf16 CUDA matrix with a contiguous last dimension")
    R, K = x.shape
    if out is None:
        out = (torch.empty((R, K // 2), dtype=torch.uint8, device=x.device),
               torch.empty((R, K // 16), dtype=torch.uint8, device=x.device),
               torch.empty(1, dtype=torch.float32, device=x.device))
    codes, scales, S = out
    nbytes = ctypes.c_size_t()
    _check(lib().sa_nvfp4_quantize_workspace_bytes(R, K, ctypes.byref(nbytes)), "sa_nvfp4_quantize_workspace_bytes")
    ws = _workspace(nbytes.value, x.device, workspace)
    _check(lib().sa_nvfp4_quantize(x.data_ptr(), R, K, x.stride(0), codes.data_ptr(), scales.data_ptr(),
                                   S.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream()),
           "sa_nvfp4_quantize")
    return codes, scales, S


def nvfp4_gemm(a, w, bias=None, out=None):
    """a, w: (codes, scales, tensor scale) as nvfp4_quantize returns them, for activations [M, K]
    and weights [N, K]; bias: bf16 [N] or None. Returns bf16 [M, N]."""
    (ac, asc, aS), (wc, wsc, wS) = a, w
    M, N, K = ac.shape[0], wc.shape[0], ac.shape[1] * 2
    if wc.shape[1] * 2 != K:
        raise ValueError("a and w have different K")
    for t in (ac, asc, wc, wsc, aS, wS):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("NVFP4 operands must be contiguous CUDA tensors")
    if bias is not None and not (bias.is_cuda and bias.dtype == torch.bfloat16 and bias.is_contiguous()
                                 and bias.numel() == N):
        raise ValueError(f"bias must be a contiguous bf16 CUDA tensor of {N} values")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=ac.device)
    _check(lib().sa_nvfp4_gemm(ac.data_ptr(), asc.data_ptr(), aS.data_ptr(), wc.data_ptr(), wsc.data_ptr(),
                               wS.data_ptr(), bias.data_ptr() if bias is not None else None, out.data_ptr(),
                               M, N, K, out.stride(0), _stream()), "sa_nvfp4_gemm")
    return out
