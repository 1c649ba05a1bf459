"""ctypes binding of libsmlp.so: argument marshalling only.

torch supplies device memory (tensors) and the current HIP stream; every step of
the computation runs in the library's HIP kernels.  The library must be built
(``python -m moe_shared_expert_amd.build``); if it is missing, loading fails with
an error -- there is no fallback implementation.

torch is imported before the library is loaded so that the library binds to the
HIP runtime torch already loaded (one runtime per process).
"""
from __future__ import annotations

import ctypes
import os

import torch

SMLP_BF16, SMLP_FP32, SMLP_BF16_HILO, SMLP_FP16 = 0, 1, 2, 3
PATH_NAMES = {0: "none", 1: "fp32", 2: "small_m", 3: "large_m"}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmlp.so")
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_int = ctypes.c_int


class SmlpError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class _Plan(ctypes.Structure):
    _fields_ = [("path", _int), ("h_dtype", _int), ("h_offset", _sz), ("workspace_bytes", _sz),
                ("gate_up_ksplit", _int), ("down_ksplit", _int), ("gate_up_blocks", _int),
                ("down_blocks", _int), ("kernels", _int)]


EXPORTS = {
    "shared_mlp_status_string": (ctypes.c_char_p, [_int]),
    "shared_mlp_last_error": (ctypes.c_char_p, []),
    "shared_mlp_plan": (_int, [_i64, _i64, _i64, _int, _int, ctypes.POINTER(_Plan)]),
    "shared_mlp_workspace_bytes": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(_sz)]),
    "shared_mlp_forward": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _sz, _vp]),
    "shared_mlp_forward_noalloc": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _vp]),
    "shared_mlp_gate_up_act": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _sz, _vp]),
    "shared_mlp_down": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _vp, _sz, _vp]),
    "shared_mlp_set_large_m_threshold": (_i64, [_i64]),
    "shared_mlp_shard_eligible": (_int, [_int, _int, _int, _int, _i64, _i64]),
    "shared_mlp_slice_rank": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _int, _int, _int, _vp]),
    "shared_mlp_rms_rescale": (_int, [_vp, _vp, _i64, _i64, _vp]),
    "shared_mlp_forward_rank": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _vp, _sz, _vp]),
    # declared in include/smlp_latent.h
    "shared_mlp_linear_plan": (_int, [_i64, _i64, _i64, ctypes.POINTER(_Plan)]),
    "shared_mlp_linear_workspace_bytes": (_int, [_i64, _i64, _i64, ctypes.POINTER(_sz)]),
    "shared_mlp_linear": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp, _sz, _vp]),
    "shared_mlp_restore_logical": (_int, [_vp, _vp, _i64, _i64, ctypes.POINTER(_i64), _int, _int, _int,
                                          _vp]),
}


class LayoutModel(ctypes.Structure):
    _fields_ = [("tp", _int), ("hidden", _i64), ("partial_elem_bytes", _int), ("alpha_us", ctypes.c_double),
                ("link_gbps", ctypes.c_double), ("links", _int),
                ("n_rep", _int), ("rep_m", ctypes.POINTER(ctypes.c_double)), ("rep_us", ctypes.POINTER(ctypes.c_double)),
                ("n_shard", _int), ("shard_m", ctypes.POINTER(ctypes.c_double)),
                ("shard_us", ctypes.POINTER(ctypes.c_double))]


_dp = ctypes.POINTER(ctypes.c_double)
# declared in include/smlp_layout.h
LAYOUT_EXPORTS = {
    "shared_mlp_layout_times": (_int, [ctypes.POINTER(LayoutModel), _i64, _dp, _dp]),
    "shared_mlp_choose_layout": (_int, [ctypes.POINTER(LayoutModel), _i64, ctypes.POINTER(_int)]),
    "shared_mlp_layout_crossover": (_int, [ctypes.POINTER(LayoutModel), _i64, ctypes.POINTER(_i64)]),
}
# declared in include/smlp_ceilings.h
CEILING_EXPORTS = {
    "shared_mlp_ceiling_empty": (_int, [_int, _vp]),
    "shared_mlp_ceiling_read": (_int, [_vp, _sz, _int, _sz, _int, _vp, _vp]),
    "shared_mlp_ceiling_mfma": (_int, [_int, _int, _vp, _vp, _vp, _vp]),
    "shared_mlp_ceiling_lds": (_int, [_int, _int, _vp, _vp, _vp]),
    "shared_mlp_ceiling_two_phase": (_int, [_vp, _sz, _int, _sz, _int, _vp, _vp, _vp]),
}
# declared in include/smlp_tuning.h
TUNING_EXPORTS = {
    "shared_mlp_tune_skinny": (_int, [_int, _int, _int, _int, _int, _int]),
    "shared_mlp_tune_gemm": (_int, [_int, _int, _int, _int, _int, _int, _int]),
    "shared_mlp_tune_h_planes": (_int, [_int]),
    "shared_mlp_tune_h_format": (_int, [_int]),
    "shared_mlp_tune_layer_fusion": (_int, [_int, _int]),
    "shared_mlp_tune_weight_convert": (_i64, [_i64]),
    "shared_mlp_tune_token_split": (_int, [_int]),
}


def lib():
    """Load libsmlp.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m moe_shared_expert_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in {**EXPORTS, **TUNING_EXPORTS, **LAYOUT_EXPORTS, **CEILING_EXPORTS}.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        L = lib()
        raise SmlpError(status, L.shared_mlp_status_string(status).decode(),
                        L.shared_mlp_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SMLP_BF16
    if t.dtype == torch.float32:
        return SMLP_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def shared_mlp_plan(M: int, H: int, I: int, dtype: int = SMLP_BF16, partial_fp32: bool = False) -> dict:
    p = _Plan()
    _check(lib().shared_mlp_plan(M, H, I, dtype, int(bool(partial_fp32)), ctypes.byref(p)))
    d = {k: getattr(p, k) for k, _ in _Plan._fields_}
    d["path_name"] = PATH_NAMES.get(d["path"], "?")
    return d


def shared_mlp_workspace_bytes(M: int, H: int, I: int, dtype: int = SMLP_BF16) -> int:
    b = _sz()
    _check(lib().shared_mlp_workspace_bytes(M, H, I, dtype, ctypes.byref(b)))
    return b.value


def _shapes(x, w_gate_up, w_down, out):
    M, H = x.shape
    two_i, H2 = w_gate_up.shape
    if H2 != H or two_i % 2:
        raise ValueError(f"w_gate_up {tuple(w_gate_up.shape)} does not match x {tuple(x.shape)}")
    I = two_i // 2
    if w_down is not None and tuple(w_down.shape) != (H, I):
        raise ValueError(f"w_down {tuple(w_down.shape)} != ({H}, {I})")
    if out is not None and tuple(out.shape) != (M, H):
        raise ValueError(f"out {tuple(out.shape)} != ({M}, {H})")
    return M, H, I


def _out_dtype(x_dtype, partial_fp32):
    """The output element type the library writes: fp32 for a partial or fp32 inputs, else bf16."""
    return torch.float32 if (partial_fp32 or x_dtype == torch.float32) else torch.bfloat16


def _check_types(x, weights, out, partial_fp32):
    """The library cannot see buffer sizes, so element types are checked here: every
    weight has x's dtype and out has the dtype the kernels write (a mismatch would make
    them read or write past the end of a buffer)."""
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"x dtype {x.dtype} is neither bfloat16 nor float32")
    for name, w in weights:
        if w is not None and w.dtype != x.dtype:
            raise TypeError(f"{name} dtype {w.dtype} differs from x dtype {x.dtype}")
    if out is not None:
        want = _out_dtype(x.dtype, partial_fp32)
        if out.dtype != want:
            raise TypeError(f"out dtype {out.dtype}: the kernels write {want} here "
                            f"(partial_fp32={bool(partial_fp32)}, x {x.dtype})")
    for name, t in (("x", x), *weights, ("out", out)):
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")


def _ws_bytes(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _workspace(workspace, M, H, I, dtype, device):
    need = shared_mlp_workspace_bytes(M, H, I, dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def shared_mlp_forward(x, w_gate_up, w_down, out, partial_fp32=False, workspace=None, stream=None):
    """out = down(SiLU(x Wg^T) * (x Wu^T)); out is bf16, or fp32 for partial_fp32 / fp32 inputs."""
    M, H, I = _shapes(x, w_gate_up, w_down, out)
    _check_types(x, (("w_gate_up", w_gate_up), ("w_down", w_down)), out, partial_fp32)
    dt = _dtype_code(x)
    workspace = _workspace(workspace, M, H, I, dt, x.device)
    _check(lib().shared_mlp_forward(_ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(out), M, H, I, dt,
                                    int(bool(partial_fp32)), _ptr(workspace), _ws_bytes(workspace),
                                    _stream(stream, x.device)))
    return out


def shared_mlp_forward_noalloc(x, w_gate_up, w_down, out, partial_fp32=False, stream=None):
    """shared_mlp_forward on the library's static per-GPU scratch array: no workspace and
    no allocation (calls that overlap on one GPU race; see include/smlp.h)."""
    M, H, I = _shapes(x, w_gate_up, w_down, out)
    _check_types(x, (("w_gate_up", w_gate_up), ("w_down", w_down)), out, partial_fp32)
    dt = _dtype_code(x)
    _check(lib().shared_mlp_forward_noalloc(_ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(out), M, H, I, dt,
                                            int(bool(partial_fp32)), _stream(stream, x.device)))
    return out


def shared_mlp_gate_up_act(x, w_gate_up, workspace, partial_fp32=False, stream=None):
    M, H, I = _shapes(x, w_gate_up, None, None)
    _check_types(x, (("w_gate_up", w_gate_up),), None, partial_fp32)
    dt = _dtype_code(x)
    _check(lib().shared_mlp_gate_up_act(_ptr(x), _ptr(w_gate_up), M, H, I, dt, int(bool(partial_fp32)),
                                        _ptr(workspace), _ws_bytes(workspace), _stream(stream, x.device)))


def shared_mlp_down(w_down, out, workspace, partial_fp32=False, stream=None):
    H, I = w_down.shape
    if out.dim() != 2 or out.shape[1] != H:
        raise ValueError(f"out {tuple(out.shape)} must be [M, {H}] for w_down {tuple(w_down.shape)}")
    M = out.shape[0]
    dt = _dtype_code(w_down)
    want = _out_dtype(w_down.dtype, partial_fp32)
    if out.dtype != want:
        raise TypeError(f"out dtype {out.dtype}: the down kernels write {want} here")
    if out.device != w_down.device:
        raise ValueError(f"out is on {out.device}, w_down on {w_down.device}")
    _check(lib().shared_mlp_down(_ptr(w_down), _ptr(out), M, H, I, dt, int(bool(partial_fp32)),
                                 _ptr(workspace), _ws_bytes(workspace), _stream(stream, w_down.device)))


def read_h(workspace, M: int, I: int, H: int, dtype: int = SMLP_BF16, partial_fp32=False):
    """The intermediate h [M, I] held in a workspace (after shared_mlp_gate_up_act), as
    stored (fp32 or bf16) or, for two bf16 planes, their fp32 sum."""
    p = shared_mlp_plan(M, H, I, dtype, partial_fp32)
    o = p["h_offset"]
    if p["h_dtype"] == SMLP_FP32:
        return workspace[o:o + 4 * M * I].view(torch.float32).view(M, I)
    if p["h_dtype"] == SMLP_BF16_HILO:
        planes = workspace[o:o + 4 * M * I].view(torch.bfloat16).view(2, M, I)
        return planes[0].float() + planes[1].float()
    if p["h_dtype"] == SMLP_FP16:
        return workspace[o:o + 2 * M * I].view(torch.float16).view(M, I)
    return workspace[o:o + 2 * M * I].view(torch.bfloat16).view(M, I)


def shared_mlp_tune_skinny(stage: int, kind: int = 0, nb: int = 0, waves: int = 0, u: int = 0,
                           ksplit: int = 0):
    """Pin small-M planner parameters (0 = automatic); see include/smlp_tuning.h."""
    _check(lib().shared_mlp_tune_skinny(stage, kind, nb, waves, u, ksplit))


def shared_mlp_tune_gemm(stage: int, bm: int = 0, bn: int = 0, wm: int = 0, wn: int = 0, ns: int = 0,
                         ksplit: int = 0):
    """Pin large-M tile parameters (0 = automatic); see include/smlp_tuning.h."""
    _check(lib().shared_mlp_tune_gemm(stage, bm, bn, wm, wn, ns, ksplit))


def shared_mlp_tune_h_planes(planes: int = 0):
    """Planes of h on the small-M path (0 = automatic); see include/smlp_tuning.h."""
    _check(lib().shared_mlp_tune_h_planes(planes))


def shared_mlp_tune_token_split(mode: int = 0):
    """Token-split gate_up on the tiled path (0 auto, 1 always, 2 never); see include/smlp_tuning.h."""
    _check(lib().shared_mlp_tune_token_split(mode))


def shared_mlp_tune_weight_convert(min_m: int) -> int:
    """Token count from which the fp16-h down stage converts w_down once; returns the previous value."""
    prev = lib().shared_mlp_tune_weight_convert(int(min_m))
    if prev < 0:
        _check(8)
    return prev


def shared_mlp_tune_layer_fusion(mode: int = 0, poll_limit: int = 0):
    _check(lib().shared_mlp_tune_layer_fusion(mode, poll_limit))


def shared_mlp_tune_h_format(fmt: int = 0):
    """Format of h on the large-M path (0 = automatic); see include/smlp_tuning.h."""
    _check(lib().shared_mlp_tune_h_format(fmt))


def forward(x, w_gate_up, w_down, partial_fp32=False, workspace=None, stream=None):
    """Allocating convenience wrapper around shared_mlp_forward."""
    odt = torch.float32 if (partial_fp32 or x.dtype == torch.float32) else torch.bfloat16
    out = torch.empty(x.shape[0], x.shape[1], dtype=odt, device=x.device)
    return shared_mlp_forward(x, w_gate_up, w_down, out, partial_fp32, workspace, stream)


def shared_mlp_set_large_m_threshold(threshold: int) -> int:
    prev = lib().shared_mlp_set_large_m_threshold(threshold)
    if prev < 0:
        _check(8)
    return prev


def shared_mlp_shard_eligible(flag_on, use_sequence_parallel, caller_eligible, tp, H, I) -> bool:
    return bool(lib().shared_mlp_shard_eligible(int(bool(flag_on)), int(bool(use_sequence_parallel)),
                                                int(bool(caller_eligible)), int(tp), int(H), int(I)))


def shared_mlp_slice_rank(w_gate_up, w_down, w_gate_up_r, w_down_r, tp: int, rank: int, stream=None):
    two_i, H = w_gate_up.shape
    I = two_i // 2
    dt = _dtype_code(w_gate_up)
    if tuple(w_down.shape) != (H, I):
        raise ValueError(f"w_down {tuple(w_down.shape)} != ({H}, {I})")
    if tp >= 1 and I % tp == 0:
        s = I // tp
        if tuple(w_gate_up_r.shape) != (2 * s, H) or tuple(w_down_r.shape) != (H, s):
            raise ValueError(f"slice destinations {tuple(w_gate_up_r.shape)}, {tuple(w_down_r.shape)} must be "
                             f"({2 * s}, {H}) and ({H}, {s})")
    for name, t in (("w_down", w_down), ("w_gate_up_r", w_gate_up_r), ("w_down_r", w_down_r)):
        if t.dtype != w_gate_up.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from w_gate_up dtype {w_gate_up.dtype}")
    _check(lib().shared_mlp_slice_rank(_ptr(w_gate_up), _ptr(w_down), _ptr(w_gate_up_r), _ptr(w_down_r),
                                       H, I, tp, rank, dt, _stream(stream, w_gate_up.device)))


def shared_mlp_rms_rescale(inp, out, stream=None):
    M, H = inp.shape
    if inp.dtype != torch.float32 or out.dtype != torch.bfloat16 or tuple(out.shape) != (M, H):
        raise ValueError("rescale takes fp32 [M, H] in and bf16 [M, H] out")
    _check(lib().shared_mlp_rms_rescale(_ptr(inp), _ptr(out), M, H, _stream(stream, inp.device)))


def shared_mlp_linear_plan(M: int, K: int, N: int) -> dict:
    p = _Plan()
    _check(lib().shared_mlp_linear_plan(M, K, N, ctypes.byref(p)))
    d = {k: getattr(p, k) for k, _ in _Plan._fields_}
    d["path_name"] = PATH_NAMES.get(d["path"], "?")
    return d


def shared_mlp_linear_workspace_bytes(M: int, K: int, N: int) -> int:
    b = _sz()
    _check(lib().shared_mlp_linear_workspace_bytes(M, K, N, ctypes.byref(b)))
    return b.value


def shared_mlp_linear(x, w, y, workspace=None, stream=None):
    """y = x w^T (bf16 x [M, K], w [N, K]; y bf16 or fp32 [M, N]).  y may be a column
    block of a wider row-major tensor (unit column stride), e.g. a rank's slot of a
    gathered buffer; its row stride is passed as ldy."""
    M, K = x.shape
    N, K2 = w.shape
    if K2 != K or tuple(y.shape) != (M, N):
        raise ValueError(f"shapes x {tuple(x.shape)}, w {tuple(w.shape)}, y {tuple(y.shape)} do not match")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16 or y.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("the projection takes bf16 x and w, and a bf16 or fp32 y")
    if not y.is_cuda or (N > 1 and y.stride(1) != 1):
        raise ValueError("y must be a GPU tensor with unit column stride")
    ldy = y.stride(0) if M > 1 else N
    need = shared_mlp_linear_workspace_bytes(M, K, N)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib().shared_mlp_linear(_ptr(x), _ptr(w), y.data_ptr(), M, K, N, ldy, int(y.dtype == torch.float32),
                                   _ptr(workspace) if workspace is not None else None,
                                   _ws_bytes(workspace),
                                   _stream(stream, x.device)))
    return y


def shared_mlp_restore_logical(gathered, out, sizes, tp: int, stream=None):
    """Rank-major gathered [M, sum(sizes)] -> logical out (same shape and dtype)."""
    M, N = gathered.shape
    if tuple(out.shape) != (M, N) or out.dtype != gathered.dtype:
        raise ValueError("out must match gathered in shape and dtype")
    eb = gathered.element_size()
    arr = (_i64 * max(len(sizes), 1))(*[int(v) for v in sizes])
    _check(lib().shared_mlp_restore_logical(_ptr(gathered), _ptr(out), M, N, arr, len(sizes), int(tp), eb,
                                            _stream(stream, gathered.device)))
    return out


def layout_model(tp, hidden, rep_curve, shard_curve, alpha_us, link_gbps, links=7, partial_elem_bytes=4):
    """Build an smlp_layout_model; the returned object keeps the curve arrays alive."""
    def arr(v):
        return (ctypes.c_double * len(v))(*[float(a) for a in v])
    keep = [arr(rep_curve[0]), arr(rep_curve[1]), arr(shard_curve[0]), arr(shard_curve[1])]
    m = LayoutModel(int(tp), int(hidden), int(partial_elem_bytes), float(alpha_us), float(link_gbps), int(links),
                    len(rep_curve[0]), ctypes.cast(keep[0], _dp), ctypes.cast(keep[1], _dp),
                    len(shard_curve[0]), ctypes.cast(keep[2], _dp), ctypes.cast(keep[3], _dp))
    m._keep = keep
    return m


def shared_mlp_layout_times(model, T: int):
    r, s = ctypes.c_double(), ctypes.c_double()
    _check(lib().shared_mlp_layout_times(ctypes.byref(model), int(T), ctypes.byref(r), ctypes.byref(s)))
    return r.value, s.value


def shared_mlp_choose_layout(model, T: int) -> bool:
    v = _int()
    _check(lib().shared_mlp_choose_layout(ctypes.byref(model), int(T), ctypes.byref(v)))
    return bool(v.value)


def shared_mlp_layout_crossover(model, T_max: int) -> int:
    v = _i64()
    _check(lib().shared_mlp_layout_crossover(ctypes.byref(model), int(T_max), ctypes.byref(v)))
    return v.value


def shared_mlp_forward_rank(x, w_gate_up, w_down, out, tp: int, rank: int, workspace=None, stream=None):
    """Rank `rank`'s fp32 partial computed in place from the full weights (no shard copy)."""
    M, H, I = _shapes(x, w_gate_up, w_down, out)
    _check_types(x, (("w_gate_up", w_gate_up), ("w_down", w_down)), out, True)
    dt = _dtype_code(x)
    if workspace is None:
        need = shared_mlp_workspace_bytes(M, H, I // tp if tp > 0 and I % tp == 0 else I, dt)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check(lib().shared_mlp_forward_rank(_ptr(x), _ptr(w_gate_up), _ptr(w_down), _ptr(out), M, H, I, int(tp),
                                         int(rank), dt, _ptr(workspace), _ws_bytes(workspace),
                                         _stream(stream, x.device)))
    return out


# Measurement kernels (include/smlp_ceilings.h): launch them, time them on the caller's side.

def ceiling_empty(blocks: int = 256, stream=None):
    _check(lib().shared_mlp_ceiling_empty(int(blocks), _stream(stream, torch.device("cuda"))))


def ceiling_read(src, blocks: int, bytes_per_block: int, shared: bool, sink, stream=None):
    """Streaming read of src (a uint8/any GPU tensor) by `blocks` workgroups; see the header."""
    _check(lib().shared_mlp_ceiling_read(_ptr(src), src.numel() * src.element_size(), int(blocks),
                                         int(bytes_per_block), int(bool(shared)), _ptr(sink),
                                         _stream(stream, src.device)))


def ceiling_mfma(blocks: int, iters: int, sink, cycles, ticks, stream=None):
    if sink.dtype != torch.float32 or cycles.dtype != torch.int64 or ticks.dtype != torch.int64:
        raise TypeError("sink is fp32, cycles and ticks int64")
    if min(sink.numel(), cycles.numel(), ticks.numel()) < blocks:
        raise ValueError("sink, cycles and ticks need one element per block")
    _check(lib().shared_mlp_ceiling_mfma(int(blocks), int(iters), _ptr(sink), _ptr(cycles), _ptr(ticks),
                                         _stream(stream, sink.device)))


def ceiling_lds(blocks: int, iters: int, sink, cycles, stream=None):
    if sink.dtype != torch.float32 or cycles.dtype != torch.int64:
        raise TypeError("sink is fp32, cycles int64")
    if sink.numel() < blocks * 512 or cycles.numel() < blocks:
        raise ValueError("sink needs 512 fp32 and cycles one int64 per block")
    _check(lib().shared_mlp_ceiling_lds(int(blocks), int(iters), _ptr(sink), _ptr(cycles),
                                        _stream(stream, sink.device)))


CEILING_BAR_WORDS = 1280  # SMLP_CEILING_BAR_WORDS


def ceiling_two_phase(src, blocks: int, bytes_per_block: int, barrier: int, bar_state, sink, stream=None):
    """barrier: 0 none, 1 one counter, 2 two-level (see include/smlp_ceilings.h)."""
    if bar_state.dtype != torch.int32 or bar_state.numel() < CEILING_BAR_WORDS:
        raise TypeError(f"bar_state is {CEILING_BAR_WORDS} int32")
    if sink.dtype != torch.float32 or sink.numel() < blocks:
        raise ValueError("sink needs one fp32 per block")
    _check(lib().shared_mlp_ceiling_two_phase(_ptr(src), src.numel() * src.element_size(), int(blocks),
                                              int(bytes_per_block), int(barrier), _ptr(bar_state),
                                              _ptr(sink), _stream(stream, src.device)))
