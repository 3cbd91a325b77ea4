"""ctypes binding of libmoe_mi355x.so (argument marshalling only).

Each function checks dtypes, devices and contiguity of the torch tensors it
is given, passes raw device pointers, sizes and the current HIP stream to
the C ABI in include/moe.h, and raises MoeError on a non-zero status.  All
computation happens in the library's kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

STATUS = {0: "ok", -1: "null pointer", -2: "unsupported shape", -3: "misaligned pointer or dimension",
          -4: "workspace too small", -5: "device is not gfx950", -6: "HIP runtime error",
          -7: "weights not declared in the tiled layout"}

WEIGHTS_PLAIN, WEIGHTS_TILED = 0, 1   # moe_shape.weight_layout


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")
        self.status = status


class MoeShape(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("expert_begin", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("swiglu_limit", ctypes.c_float), ("exact_silu", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32)]


class PlanView(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("scalars", "counts", "offsets", "slot", "row_token", "row_topk",
                                               "block_expert", "slack", "pull_order")] + \
               [("capacity_rows", ctypes.c_int64)]


class ForwardView(ctypes.Structure):
    _fields_ = [("h_q", ctypes.c_void_p), ("h_sf", ctypes.c_void_p), ("yslot", ctypes.c_void_p),
                ("plan", ctypes.c_void_p), ("capacity_rows", ctypes.c_int64), ("sync_status", ctypes.c_void_p)]


_lib = None

EXPORTS = ["moe_capacity_rows", "moe_suggest_block_m", "moe_gemm_launches", "moe_plan_workspace_bytes", "moe_plan", "moe_plan_view_get",
           "moe_forward_workspace_bytes", "moe_forward", "moe_linear1", "moe_linear2", "moe_combine",
           "moe_expert_ffn", "moe_prepare_weights", "moe_forward_noalloc",
           "moe_forward_view_get", "moe_device_supported", "moe_status_str"]


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with python -m moe_expert_ffn_plan_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, VP, SZ = ctypes.POINTER, ctypes.c_void_p, ctypes.c_size_t
        S = P(MoeShape)
        L.moe_capacity_rows.argtypes = [S, P(ctypes.c_int64)]
        L.moe_suggest_block_m.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int32)]
        L.moe_gemm_launches.argtypes = [S, P(ctypes.c_int32), P(ctypes.c_int32)]
        L.moe_plan_workspace_bytes.argtypes = [S, P(SZ)]
        L.moe_forward_workspace_bytes.argtypes = [S, P(SZ)]
        L.moe_plan.argtypes = [S, VP, VP, SZ, VP]
        L.moe_plan_view_get.argtypes = [S, VP, P(PlanView)]
        L.moe_forward.argtypes = [S, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_forward_noalloc.argtypes = [S, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP]
        L.moe_prepare_weights.argtypes = [S, ctypes.c_int, VP, VP, VP, VP, VP]
        L.moe_linear1.argtypes = [S, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_linear2.argtypes = [S, VP, VP, VP, VP, SZ, VP]
        L.moe_combine.argtypes = [S, VP, VP, SZ, VP, VP]
        L.moe_expert_ffn.argtypes = [S, VP, VP, VP, VP, VP, VP, VP, VP, VP, SZ, VP]
        L.moe_forward_view_get.argtypes = [S, VP, P(ForwardView)]
        L.moe_device_supported.argtypes = [ctypes.c_int]
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        for f in EXPORTS:
            if f != "moe_status_str":
                getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def make_shape(num_tokens, hidden, intermediate, num_experts, topk, block_m, expert_begin=0, swiglu_limit=0.0,
               exact_silu=False, weight_layout=WEIGHTS_TILED) -> MoeShape:
    """A moe_shape.  weight_layout states the layout of the weights the call is given: the Python side
    always passes the tiled weights prepare_weights returns, hence the default."""
    return MoeShape(num_tokens, hidden, intermediate, num_experts, expert_begin, topk, block_m, float(swiglu_limit),
                    int(bool(exact_silu)), int(weight_layout))


def shape_of(workload, num_tokens=None, expert_begin=0, swiglu_limit=0.0, exact_silu=False,
             weight_layout=WEIGHTS_TILED) -> MoeShape:
    w = workload
    return make_shape(w.num_tokens if num_tokens is None else num_tokens, w.hidden, w.intermediate,
                      w.num_experts, w.topk, w.block_m, expert_begin, swiglu_limit, exact_silu, weight_layout)


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status)


def _ptr(t, dtype, name, device=None, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def capacity_rows(shape: MoeShape) -> int:
    v = ctypes.c_int64()
    _check("moe_capacity_rows", lib().moe_capacity_rows(ctypes.byref(shape), ctypes.byref(v)))
    return v.value


def suggest_block_m(num_tokens: int, topk: int, num_experts: int) -> int:
    """moe_suggest_block_m: routing block rows for num_tokens tokens routed top-k over num_experts experts."""
    v = ctypes.c_int32()
    _check("moe_suggest_block_m", lib().moe_suggest_block_m(num_tokens, topk, num_experts, ctypes.byref(v)))
    return v.value


def gemm_launches(shape: MoeShape) -> tuple[int, int]:
    """moe_gemm_launches: (GEMM launches of moe_expert_ffn, GEMM launches of moe_forward), 1 or 2 each."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check("moe_gemm_launches", lib().moe_gemm_launches(ctypes.byref(shape), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def plan_workspace_bytes(shape: MoeShape) -> int:
    v = ctypes.c_size_t()
    _check("moe_plan_workspace_bytes", lib().moe_plan_workspace_bytes(ctypes.byref(shape), ctypes.byref(v)))
    return v.value


def forward_workspace_bytes(shape: MoeShape) -> int:
    v = ctypes.c_size_t()
    _check("moe_forward_workspace_bytes", lib().moe_forward_workspace_bytes(ctypes.byref(shape), ctypes.byref(v)))
    return v.value


def device_supported(device: int = 0) -> bool:
    return lib().moe_device_supported(device) == 0


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


class Bound:
    """One library call with its arguments checked and marshalled once: calling it with a stream (None:
    torch's current one) enqueues the call and raises on an error status.  It keeps the shape and the
    tensors it points at alive.  For loops that issue the same calls many times (the benchmark)."""
    __slots__ = ("fn", "name", "args", "keep")

    def __init__(self, fn, name, args, keep):
        self.fn, self.name, self.args, self.keep = fn, name, tuple(args), keep

    def __call__(self, stream=None) -> None:
        _check(self.name, self.fn(*self.args, _stream(stream)))


def _call(name, shape, args, keep, stream, bind):
    fn = getattr(lib(), name)
    args = [ctypes.byref(shape)] + list(args)
    if bind:
        return Bound(fn, name, args, (shape, keep))
    _check(name, fn(*args, _stream(stream)))
    return None


def plan(shape: MoeShape, topk_idx: torch.Tensor, plan_ws: torch.Tensor, stream=None, bind=False):
    """moe_plan; bind=True: return the call as a Bound instead of enqueueing it."""
    dev = plan_ws.device
    args = [_ptr(topk_idx, torch.int64, "topk_idx", dev, shape.num_tokens * shape.topk),
            _ptr(plan_ws, torch.uint8, "plan_ws"), plan_ws.numel()]
    return _call("moe_plan", shape, args, (topk_idx, plan_ws), stream, bind)


def forward(shape: MoeShape, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y, ws, plan_ws=None,
            stream=None, bind=False):
    """moe_forward (plan_ws None: the plan is built inside ws); bind=True: return the call as a Bound."""
    T, H, I, E, k = shape.num_tokens, shape.hidden, shape.intermediate, shape.num_experts, shape.topk
    dev = ws.device
    u8, args = torch.uint8, []
    args.append(_ptr(x, u8, "x", dev, T * H))
    args.append(_ptr(x_sf, u8, "x_sf", dev, T * H // 32))
    args.append(_ptr(topk_idx, torch.int64, "topk_idx", dev, T * k))
    args.append(_ptr(topk_w, torch.float32, "topk_w", dev, T * k))
    args.append(_ptr(w1, u8, "w1", dev, E * 2 * I * H // 2))
    args.append(_ptr(w1_sf, u8, "w1_sf", dev, E * 2 * I * H // 32))
    args.append(_ptr(w2, u8, "w2", dev, E * H * I // 2))
    args.append(_ptr(w2_sf, u8, "w2_sf", dev, E * H * I // 32))
    yv = y.view(torch.int16) if y.dtype == torch.bfloat16 else y
    args.append(_ptr(yv, torch.int16, "y", dev, T * H))
    args.append(_ptr(plan_ws, u8, "plan_ws", dev))
    args += [_ptr(ws, u8, "ws"), ws.numel()]
    return _call("moe_forward", shape, args, (x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y, ws, plan_ws),
                 stream, bind)


NOALLOC_WORKSPACE_BYTES = 32 << 20   # MOE_NOALLOC_WORKSPACE_BYTES


def forward_noalloc(shape: MoeShape, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, y, stream=None) -> None:
    """moe_forward_noalloc: moe_forward (routing included) with the library's own device workspace."""
    T, H, I, E, k = shape.num_tokens, shape.hidden, shape.intermediate, shape.num_experts, shape.topk
    dev = y.device
    u8, args = torch.uint8, []
    args.append(_ptr(x, u8, "x", dev, T * H))
    args.append(_ptr(x_sf, u8, "x_sf", dev, T * H // 32))
    args.append(_ptr(topk_idx, torch.int64, "topk_idx", dev, T * k))
    args.append(_ptr(topk_w, torch.float32, "topk_w", dev, T * k))
    args.append(_ptr(w1, u8, "w1", dev, E * 2 * I * H // 2))
    args.append(_ptr(w1_sf, u8, "w1_sf", dev, E * 2 * I * H // 32))
    args.append(_ptr(w2, u8, "w2", dev, E * H * I // 2))
    args.append(_ptr(w2_sf, u8, "w2_sf", dev, E * H * I // 32))
    yv = y.view(torch.int16) if y.dtype == torch.bfloat16 else y
    args.append(_ptr(yv, torch.int16, "y", dev, T * H))
    _check("moe_forward_noalloc", lib().moe_forward_noalloc(ctypes.byref(shape), *args, _stream(stream)))


def prepare_weights(shape: MoeShape, which: int, w, w_sf, stream=None):
    """Tiled copies (new tensors) of one plain weight tensor and its scales (which = 1: W1, 2: W2)."""
    H, I, E = shape.hidden, shape.intermediate, shape.num_experts
    N, K = (2 * I, H) if which == 1 else (H, I)
    dev = w.device
    _ptr(w, torch.uint8, "w", dev, E * N * K // 2)
    _ptr(w_sf, torch.uint8, "w_sf", dev, E * N * K // 32)
    wt = torch.empty(E * N * K // 2, dtype=torch.uint8, device=dev)
    st_ = torch.empty(E * N * K // 32, dtype=torch.uint8, device=dev)
    st = lib().moe_prepare_weights(ctypes.byref(shape), which, _ptr(w, torch.uint8, "w"), _ptr(w_sf, torch.uint8, "w_sf"),
                                   _ptr(wt, torch.uint8, "w_tiled"), _ptr(st_, torch.uint8, "w_sf_tiled"), _stream(stream))
    _check("moe_prepare_weights", st)
    return wt, st_


def prepare_all(shape: MoeShape, d: dict, stream=None) -> dict:
    """Tiled W1/W2 (keys w1, w1_sf, w2, w2_sf) from a dict holding the plain ones."""
    w1, w1_sf = prepare_weights(shape, 1, d["w1"], d["w1_sf"], stream)
    w2, w2_sf = prepare_weights(shape, 2, d["w2"], d["w2_sf"], stream)
    return {"w1": w1, "w1_sf": w1_sf, "w2": w2, "w2_sf": w2_sf}


def untile_row_scales(tiled: torch.Tensor, cap: int, k: int, block_m: int) -> torch.Tensor:
    """[cap/bm][k/128][bm][4] per-row-block scales -> plain [cap, k/32] (for tests and inspection)."""
    return tiled.view(cap // block_m, k // 128, block_m, 4).permute(0, 2, 1, 3).reshape(cap, k // 32)


def linear1(shape: MoeShape, x, x_sf, topk_w, w1, w1_sf, plan_ws, ws, stream=None, bind=False):
    T, H, I, E, k = shape.num_tokens, shape.hidden, shape.intermediate, shape.num_experts, shape.topk
    dev, u8 = ws.device, torch.uint8
    args = [_ptr(x, u8, "x", dev, T * H), _ptr(x_sf, u8, "x_sf", dev, T * H // 32),
            _ptr(topk_w, torch.float32, "topk_w", dev, T * k),
            _ptr(w1, u8, "w1", dev, E * 2 * I * H // 2), _ptr(w1_sf, u8, "w1_sf", dev, E * 2 * I * H // 32),
            _ptr(plan_ws, u8, "plan_ws", dev), _ptr(ws, u8, "ws"), ws.numel()]
    return _call("moe_linear1", shape, args, (x, x_sf, topk_w, w1, w1_sf, plan_ws, ws), stream, bind)


def linear2(shape: MoeShape, w2, w2_sf, plan_ws, ws, stream=None, bind=False):
    H, I, E = shape.hidden, shape.intermediate, shape.num_experts
    dev, u8 = ws.device, torch.uint8
    args = [_ptr(w2, u8, "w2", dev, E * H * I // 2), _ptr(w2_sf, u8, "w2_sf", dev, E * H * I // 32),
            _ptr(plan_ws, u8, "plan_ws", dev), _ptr(ws, u8, "ws"), ws.numel()]
    return _call("moe_linear2", shape, args, (w2, w2_sf, plan_ws, ws), stream, bind)


def expert_ffn(shape: MoeShape, x, x_sf, topk_w, w1, w1_sf, w2, w2_sf, plan_ws, ws, stream=None, bind=False):
    T, H, I, E, k = shape.num_tokens, shape.hidden, shape.intermediate, shape.num_experts, shape.topk
    dev, u8 = ws.device, torch.uint8
    args = [_ptr(x, u8, "x", dev, T * H), _ptr(x_sf, u8, "x_sf", dev, T * H // 32),
            _ptr(topk_w, torch.float32, "topk_w", dev, T * k),
            _ptr(w1, u8, "w1", dev, E * 2 * I * H // 2), _ptr(w1_sf, u8, "w1_sf", dev, E * 2 * I * H // 32),
            _ptr(w2, u8, "w2", dev, E * H * I // 2), _ptr(w2_sf, u8, "w2_sf", dev, E * H * I // 32),
            _ptr(plan_ws, u8, "plan_ws", dev), _ptr(ws, u8, "ws"), ws.numel()]
    return _call("moe_expert_ffn", shape, args, (x, x_sf, topk_w, w1, w1_sf, w2, w2_sf, plan_ws, ws), stream, bind)


def expert_ffn_is_fused(shape: MoeShape) -> bool:
    """Whether moe_expert_ffn runs as one persistent launch for this shape."""
    return gemm_launches(shape)[0] == 1


def forward_uses_expert_ffn(shape: MoeShape) -> bool:
    """Whether moe_forward runs the GEMMs as one moe_expert_ffn launch (else moe_linear1 + moe_linear2)."""
    return gemm_launches(shape)[1] == 1


def combine(shape: MoeShape, plan_ws, ws, y, stream=None, bind=False):
    dev = ws.device
    yv = y.view(torch.int16) if y.dtype == torch.bfloat16 else y
    args = [_ptr(plan_ws, torch.uint8, "plan_ws", dev), _ptr(ws, torch.uint8, "ws"), ws.numel(),
            _ptr(yv, torch.int16, "y", dev, shape.num_tokens * shape.hidden)]
    return _call("moe_combine", shape, args, (plan_ws, ws, y), stream, bind)


def _slice(base: torch.Tensor, ptr: int, dtype, n: int) -> torch.Tensor:
    off = ptr - base.data_ptr()
    item = torch.empty(0, dtype=dtype).element_size()
    assert off % item == 0 and off >= 0
    return base[off:off + n * item].view(dtype)


def plan_view(shape: MoeShape, plan_ws: torch.Tensor) -> dict:
    v = PlanView()
    _check("moe_plan_view_get", lib().moe_plan_view_get(ctypes.byref(shape), ctypes.c_void_p(plan_ws.data_ptr()),
                                                        ctypes.byref(v)))
    cap, T, k, E = v.capacity_rows, shape.num_tokens, shape.topk, shape.num_experts
    i32 = torch.int32
    return {"scalars": _slice(plan_ws, v.scalars, i32, 4), "counts": _slice(plan_ws, v.counts, i32, E),
            "offsets": _slice(plan_ws, v.offsets, i32, E + 1), "slot": _slice(plan_ws, v.slot, i32, T * k),
            "row_token": _slice(plan_ws, v.row_token, i32, cap), "row_topk": _slice(plan_ws, v.row_topk, i32, cap),
            "block_expert": _slice(plan_ws, v.block_expert, i32, cap // shape.block_m),
            "slack": _slice(plan_ws, v.slack, i32, cap // shape.block_m),
            "pull_order": _slice(plan_ws, v.pull_order, i32, T), "capacity_rows": cap}


def forward_view(shape: MoeShape, ws: torch.Tensor) -> dict:
    v = ForwardView()
    _check("moe_forward_view_get", lib().moe_forward_view_get(ctypes.byref(shape), ctypes.c_void_p(ws.data_ptr()),
                                                              ctypes.byref(v)))
    cap, H, I = v.capacity_rows, shape.hidden, shape.intermediate
    plan_off = v.plan - ws.data_ptr()
    return {"h_q": _slice(ws, v.h_q, torch.uint8, cap * I).view(cap, I),
            "h_sf": untile_row_scales(_slice(ws, v.h_sf, torch.uint8, cap * I // 32), cap, I, shape.block_m),
            "yslot": _slice(ws, v.yslot, torch.int16, cap * H).view(cap, H),
            "plan_ws": ws[plan_off:], "capacity_rows": cap,
            "sync_status": _slice(ws, v.sync_status, torch.int32, 1)}
