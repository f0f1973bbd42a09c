"""ctypes binding of libq4moe.so (the HIP library); argument marshalling only.

Every function here checks tensor devices, dtypes, shapes and contiguity, allocates
outputs with PyTorch (device memory is PyTorch's job) and calls the C entry point of
the same name on the current HIP stream.  All computation happens in the library's
kernels; there is no fallback: if the library is missing, importing this module
raises.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("Q4MOE_LIB") or os.path.join(_HERE, "libq4moe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python int4_group_quantized_g128_amd/build.py, or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

# status codes and enums (mirror include/q4moe.h)
Q4_OK, Q4_ERR_NULL, Q4_ERR_SHAPE, Q4_ERR_ALIGN, Q4_ERR_DTYPE = 0, 1, 2, 3, 4
Q4_ERR_WORKSPACE, Q4_ERR_UNSUPPORTED, Q4_ERR_HIP = 5, 6, 7
Q4_F32, Q4_F16, Q4_BF16 = 0, 1, 2
Q4_W4A16, Q4_W4A8, Q4_W8A8 = 0, 1, 2
Q4_REPACK_PLAIN, Q4_REPACK_GATE_UP = 0, 1
Q4_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
Q4_QFLAG_NONFINITE, Q4_QFLAG_SCALE_OVERFLOW = 1, 2

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_int = ctypes.c_int


class Q4MoELayer(ctypes.Structure):
    """Mirror of q4_moe_layer_t."""
    _fields_ = [
        ("num_experts", _i32), ("hidden", _i32), ("inter", _i32), ("top_k", _i32),
        ("asymmetric", _i32), ("shared_inter", _i32),
        ("gate_up", _vp), ("down", _vp), ("shared_gate_up", _vp), ("shared_down", _vp),
        ("weight_bits", _i32),
        ("expert_bits", _vp), ("gate_up_offsets", _vp), ("down_offsets", _vp),
        ("expert_groups", _vp),
    ]


class Q4LoraLayer(ctypes.Structure):
    """Mirror of q4_lora_layer_t."""
    _fields_ = [
        ("num_experts", _i32), ("hidden", _i32), ("inter", _i32), ("top_k", _i32),
        ("rank", _i32), ("asymmetric", _i32),
        ("base_gate_up", _vp), ("base_down", _vp), ("a_gate_up", _vp), ("b_gate", _vp),
        ("b_up", _vp), ("a_down", _vp), ("b_down", _vp),
    ]


class Q4FfnViews(ctypes.Structure):
    """Mirror of q4_ffn_views_t."""
    _fields_ = [
        ("counts", _vp), ("offsets", _vp), ("perm", _vp), ("inv", _vp), ("h", _vp),
        ("h_is_f32", _i32), ("slots_per_token", _i32), ("positions", _i64),
        ("y", _vp), ("q_x", _vp), ("s_x", _vp), ("q_h", _vp), ("s_h", _vp),
        ("y_slices", _i32), ("y_slice_groups", _i32), ("y_slice_stride", _i64),
    ]


class Q4FfnPlan(ctypes.Structure):
    """Mirror of q4_ffn_plan_t."""
    _fields_ = [("kernel", _i32), ("tile_rows", _i32), ("down_ksplit", _i32), ("prefill_addr_limited", _i32),
                ("rows_in_token_order", _i32), ("combine_in_down", _i32), ("slot_tiles", _i32),
                ("workspace_bytes", _i64)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_sig("q4_status_string", ctypes.c_char_p, [_int])
_sig("q4_last_error", ctypes.c_char_p, [])
_sig("q4_version", ctypes.c_char_p, [])
_sig("quantize_int4_g128", _int, [_vp, _int, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp])
_sig("q4_device_bytes", _sz, [_i64, _i64, _int])
_sig("q4_repack_device", _int, [_vp, _vp, _vp, _i64, _i64, _int, _int, _vp, _sz, _vp])
_sig("quantize_int4_grouped", _int, [_vp, _int, _i64, _i64, _i32, _int, _vp, _vp, _vp, _vp, _vp])
_sig("q4_device_bytes_grouped", _sz, [_i64, _i64, _int, _i32])
_sig("q4_repack_device_grouped", _int, [_vp, _vp, _vp, _i64, _i64, _int, _i32, _int, _vp, _sz, _vp])
_sig("quantize_int8_g128", _int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp])
_sig("q8_device_bytes", _sz, [_i64, _i64])
_sig("quantize_int2_g128", _int, [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp])
_sig("q2_device_bytes", _sz, [_i64, _i64])
_sig("q2_repack_device", _int, [_vp, _vp, _i64, _i64, _int, _vp, _sz, _vp])
_sig("int2_w2a8_group_acc", _int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp])
_sig("moe_expert_bits_apex", _int, [ctypes.POINTER(_i64), _i32, ctypes.c_double, ctypes.c_double, _int,
                                    ctypes.POINTER(_i32)])
_sig("q8_repack_device", _int, [_vp, _vp, _i64, _i64, _int, _vp, _sz, _vp])
_sig("int8_w8a8_group_acc", _int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp])
_sig("moe_route_workspace_bytes", _sz, [_i64, _i64, _i32])
_sig("moe_route_topk", _int, [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp])
_sig("moe_permute", _int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp])
_sig("act_quant_int8", _int, [_vp, _int, _i64, _i64, _vp, _vp, _vp])
_sig("moe_int4_ffn_workspace_bytes", _sz, [ctypes.POINTER(Q4MoELayer), _i64, _int])
_sig("moe_int4_ffn_forward", _int, [ctypes.POINTER(Q4MoELayer), _vp, _i64, _vp, _vp, _int, _vp, _vp, _sz, _vp])
_sig("moe_int4_ffn_debug", _int, [ctypes.POINTER(Q4MoELayer), _vp, _i64, _vp, _vp, _int, _vp, _vp, _sz,
                                  ctypes.POINTER(Q4FfnViews), _vp])
_sig("moe_lora_ffn_workspace_bytes", _sz, [ctypes.POINTER(Q4LoraLayer), _i64])
_sig("moe_lora_ffn_forward", _int, [ctypes.POINTER(Q4LoraLayer), _vp, _i64, _vp, _vp, _vp, _vp, _sz, _vp])
_sig("int4_linear_forward", _int, [_vp, _int, _i64, _i64, _vp, _i64, _int, _vp, _vp])
_sig("int4_w4a8_group_acc", _int, [_vp, _i64, _i64, _vp, _i64, _int, _vp, _vp])

_sig("moe_int4_ffn_forward_noalloc", _int, [ctypes.POINTER(Q4MoELayer), _vp, _i64, _vp, _vp, _int, _vp, _vp])
_sig("moe_int4_ffn_plan", _int, [ctypes.POINTER(Q4MoELayer), _i64, _int, ctypes.POINTER(Q4FfnPlan)])
_sig("moe_expert_bits_by_hotness", _int, [ctypes.POINTER(_i64), _i32, ctypes.c_double, _int, ctypes.POINTER(_i32)])
_sig("moe_expert_groups_by_hotness", _int, [ctypes.POINTER(_i64), _i32, ctypes.c_double, ctypes.c_double, _int,
                                            ctypes.POINTER(_i32)])
_sig("q4_set_stage_events", _int, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _int])

raw = _lib  # the C entry points, for tests of the ABI itself

STAGES = ("permute", "x_quant", "gate_up", "h_quant", "down", "combine")


class Q4Error(RuntimeError):
    def __init__(self, name, code):
        msg = _lib.q4_last_error().decode()
        super().__init__(f"{name}: {_lib.q4_status_string(code).decode()} ({code}): {msg}")
        self.code = code


def _check(name, code):
    if code != Q4_OK:
        raise Q4Error(name, code)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t


_DT = {torch.float32: Q4_F32, torch.float16: Q4_F16, torch.bfloat16: Q4_BF16}


def version():
    return _lib.q4_version().decode()


def set_stage_events(begin, end):
    """Per-stage HIP event markers for moe_int4_ffn_forward on this thread: ``begin``
    and ``end`` are lists of torch.cuda.Event (enable_timing=True), one per stage
    (STAGES order); None disables."""
    if begin is None:
        _check("q4_set_stage_events", _lib.q4_set_stage_events(None, None, 0))
        return
    arr = ctypes.c_void_p * len(STAGES)
    b = arr(*[ctypes.c_void_p(e.cuda_event) for e in begin])
    e_ = arr(*[ctypes.c_void_p(e.cuda_event) for e in end])
    _check("q4_set_stage_events", _lib.q4_set_stage_events(b, e_, len(STAGES)))


# ------------------------------------------------------------------ A1 / A2
def quantize_int8_g128(w, flags=None):
    """INT8 g128 quantisation (the W8A8 weight format) of w [n, k] -> (q int8 [n, k],
    scales int16 [n, k/128] (binary16 bits))."""
    _need(w, (torch.float32, torch.float16, torch.bfloat16), "w", 2)
    n, k = w.shape
    q = torch.empty((n, k), dtype=torch.int8, device=w.device)
    scales = torch.empty((n, max(k // 128, 1)), dtype=torch.int16, device=w.device)
    _check("quantize_int8_g128", _lib.quantize_int8_g128(
        _ptr(w), _DT[w.dtype], n, k, _ptr(q), _ptr(scales), _ptr(flags), _stream()))
    return q, scales


def q8_device_bytes(n, k):
    return int(_lib.q8_device_bytes(n, k))


def q8_repack_device(q, scales, n, k, gate_up=False, out=None):
    """INT8 codes + scales -> device tiles (uint8 tensor of q8_device_bytes(n, k))."""
    nbytes = q8_device_bytes(n, k)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check("q8_repack_device", _lib.q8_repack_device(
        _ptr(q), _ptr(scales), n, k, Q4_REPACK_GATE_UP if gate_up else Q4_REPACK_PLAIN, _ptr(out), out.numel(),
        _stream()))
    return out


def quantize_int2_g128(w, flags=None):
    """2-bit g128 quantisation on the GPU: (packed uint8 [n, k/4], scale bits int16 [n, k/128])."""
    _need(w, (torch.float32, torch.float16, torch.bfloat16), "w", 2)
    n, k = w.shape
    packed = torch.empty((n, k // 4), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // 128), dtype=torch.int16, device=w.device)
    _check("quantize_int2_g128", _lib.quantize_int2_g128(_ptr(w), _DT[w.dtype], n, k, _ptr(packed), _ptr(scales),
                                                         _ptr(flags), _stream()))
    return packed, scales


def q2_device_bytes(n, k):
    return int(_lib.q2_device_bytes(n, k))


def q2_repack_device(packed, scales, n, k, gate_up=False, out=None):
    nbytes = q2_device_bytes(n, k)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=packed.device)
    _check("q2_repack_device", _lib.q2_repack_device(_ptr(packed), _ptr(scales), n, k,
                                                     Q4_REPACK_GATE_UP if gate_up else Q4_REPACK_PLAIN,
                                                     _ptr(out), out.numel(), _stream()))
    return out


def quantize_int4_g128(w, asymmetric=False, flags=None):
    """Canonical INT4 g128 quantisation of w [n, k] -> (packed u8 [n, k/2],
    scales int16 [n, k/128] (binary16 bits), zeros u8 [n, ceil(G/2)] or None)."""
    _need(w, (torch.float32, torch.float16, torch.bfloat16), "w", 2)
    n, k = w.shape
    g = k // 128
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, max(g, 1)), dtype=torch.int16, device=w.device)
    zeros = torch.empty((n, (g + 1) // 2), dtype=torch.uint8, device=w.device) if asymmetric else None
    _check("quantize_int4_g128", _lib.quantize_int4_g128(
        _ptr(w), _DT[w.dtype], n, k, int(bool(asymmetric)), _ptr(packed), _ptr(scales), _ptr(zeros),
        _ptr(flags), _stream()))
    return packed, scales, zeros


def q4_device_bytes(n, k, asymmetric=False):
    return int(_lib.q4_device_bytes(n, k, int(bool(asymmetric))))


def quantize_int4_grouped(w, group, asymmetric=False, flags=None):
    """INT4 quantisation of w [n, k] with groups of `group` (32, 64, 128, 256) along k ->
    (packed u8 [n, k/2], scales int16 [n, k/group] (binary16 bits), zeros u8 or None)."""
    _need(w, (torch.float32, torch.float16, torch.bfloat16), "w", 2)
    n, k = w.shape
    g = max(k // group, 1)
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, g), dtype=torch.int16, device=w.device)
    zeros = torch.empty((n, (g + 1) // 2), dtype=torch.uint8, device=w.device) if asymmetric else None
    _check("quantize_int4_grouped", _lib.quantize_int4_grouped(
        _ptr(w), _DT[w.dtype], n, k, group, int(bool(asymmetric)), _ptr(packed), _ptr(scales), _ptr(zeros),
        _ptr(flags), _stream()))
    return packed, scales, zeros


def q4_device_bytes_grouped(n, k, asymmetric=False, group=128):
    return int(_lib.q4_device_bytes_grouped(n, k, int(bool(asymmetric)), group))


def q4_repack_device_grouped(packed, scales, zeros, n, k, group, asymmetric=False, gate_up=False, out=None):
    """Canonical bytes (groups of `group`) -> device tile layout with SG scale entries per tile."""
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.int16, "scales")
    if zeros is not None:
        _need(zeros, torch.uint8, "zeros")
    nbytes = q4_device_bytes_grouped(n, k, asymmetric, group)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=packed.device)
    _check("q4_repack_device_grouped", _lib.q4_repack_device_grouped(
        _ptr(packed), _ptr(scales), _ptr(zeros), n, k, int(bool(asymmetric)), group,
        Q4_REPACK_GATE_UP if gate_up else Q4_REPACK_PLAIN, _ptr(out), out.numel(), _stream()))
    return out


def q4_repack_device(packed, scales, zeros, n, k, asymmetric=False, gate_up=False, out=None):
    """Canonical bytes -> device tile layout (u8 tensor of q4_device_bytes bytes)."""
    _need(packed, torch.uint8, "packed")
    _need(scales, torch.int16, "scales")
    if zeros is not None:
        _need(zeros, torch.uint8, "zeros")
    nbytes = q4_device_bytes(n, k, asymmetric)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=packed.device)
    _check("q4_repack_device", _lib.q4_repack_device(
        _ptr(packed), _ptr(scales), _ptr(zeros), n, k, int(bool(asymmetric)),
        Q4_REPACK_GATE_UP if gate_up else Q4_REPACK_PLAIN, _ptr(out), out.numel(), _stream()))
    return out


# ------------------------------------------------------------------ A3..A6
def moe_route_topk(x, w_router, bias, k):
    """-> (logits fp32 [t, e], ids int32 [t, k], weights fp32 [t, k])."""
    _need(x, torch.bfloat16, "x", 2)
    _need(w_router, torch.float32, "w_router", 2)
    if bias is not None:
        _need(bias, torch.float32, "bias", 1)
    t, h = x.shape
    e = w_router.shape[0]
    logits = torch.empty((t, e), dtype=torch.float32, device=x.device)
    ids = torch.empty((t, k), dtype=torch.int32, device=x.device)
    w = torch.empty((t, k), dtype=torch.float32, device=x.device)
    ws_bytes = int(_lib.moe_route_workspace_bytes(t, h, e))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _check("moe_route_topk", _lib.moe_route_topk(
        _ptr(x), _ptr(w_router), _ptr(bias), t, h, e, k, _ptr(logits), _ptr(ids), _ptr(w),
        _ptr(ws), ws_bytes, _stream()))
    return logits, ids, w


def moe_permute(ids, num_experts):
    """-> (counts [e], offsets [e + 1], perm [t k], inv [t k]) int32."""
    _need(ids, torch.int32, "ids", 2)
    t, k = ids.shape
    dev = ids.device
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(t * k, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(t * k, 1), dtype=torch.int32, device=dev)
    _check("moe_permute", _lib.moe_permute(
        _ptr(ids), t, k, num_experts, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _stream()))
    return counts, offsets, perm[: t * k], inv[: t * k]


def act_quant_int8(x):
    """Per-row INT8 quantisation of x [rows, cols] (bf16 or fp32) -> (q int8, s fp32 [rows])."""
    _need(x, (torch.bfloat16, torch.float32), "x", 2)
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    s = torch.empty(max(rows, 1), dtype=torch.float32, device=x.device)
    _check("act_quant_int8", _lib.act_quant_int8(
        _ptr(x), Q4_F32 if x.dtype == torch.float32 else Q4_BF16, rows, cols, _ptr(q), _ptr(s), _stream()))
    return q, s[:rows]


# ------------------------------------------------------------------ layer + forward
def _hotness(name, counts, shared, *fracs):
    counts = [int(c) for c in counts]
    e = len(counts)
    out = (_i32 * (e + (1 if shared else 0)))()
    _check(name, getattr(_lib, name)((_i64 * e)(*counts), e, *fracs, int(bool(shared)), out))
    return list(out)


def expert_bits_by_hotness(counts, frac8=0.05, shared=False):
    """Per-expert weight widths (4 or 8) from routing hit counts; the rule is the C
    library's moe_expert_bits_by_hotness (host arrays, no device work)."""
    return _hotness("moe_expert_bits_by_hotness", counts, shared, float(frac8))


def expert_bits_apex(counts, frac8=0.0, cold_share=0.25, shared=False):
    """Per-expert widths (2, 4 or 8) from routing hit counts; the rule is the C library's
    moe_expert_bits_apex (host arrays, no device work)."""
    return _hotness("moe_expert_bits_apex", counts, shared, float(frac8), float(cold_share))


def expert_groups_by_hotness(counts, hot_frac=0.05, cold_share=0.1, shared=False):
    """Per-expert group sizes (32, 64 or 256) from routing hit counts; the rule is the C
    library's moe_expert_groups_by_hotness (host arrays, no device work)."""
    return _hotness("moe_expert_groups_by_hotness", counts, shared, float(hot_frac), float(cold_share))


def moe_int4_ffn_plan(layer, t, mode):
    """Launch plan of moe_int4_ffn_forward for (layer, t, mode): a dict with kernel
    ("decode" / "prefill"), tile_rows, down_ksplit, prefill_addr_limited, workspace_bytes.
    ``layer`` is a MoELayer or a Q4MoELayer descriptor."""
    desc = layer.desc if hasattr(layer, "desc") else layer
    p = Q4FfnPlan()
    _check("moe_int4_ffn_plan", _lib.moe_int4_ffn_plan(ctypes.byref(desc), t, mode, ctypes.byref(p)))
    return {"kernel": "prefill" if p.kernel == 1 else "decode", "tile_rows": p.tile_rows,
            "down_ksplit": p.down_ksplit, "prefill_addr_limited": bool(p.prefill_addr_limited),
            "rows_in_token_order": bool(p.rows_in_token_order), "combine_in_down": bool(p.combine_in_down),
            "slot_tiles": bool(p.slot_tiles), "workspace_bytes": int(p.workspace_bytes)}


class MoELayer:
    """Device-resident MoE layer (experts in the device tile layouts).

    weight_bits 4 (INT4 g128, symmetric or asymmetric) or 8 (INT8 g128, symmetric) for
    every expert; or expert_bits, one width (4 or 8) per expert plus one for the shared
    expert, for a mixed symmetric layer run in W4A8 (INT8 activations everywhere)."""

    def __init__(self, num_experts, hidden, inter, top_k, asymmetric=False, shared=False, device="cuda",
                 weight_bits=4, expert_bits=None, expert_groups=None):
        self.num_experts, self.hidden, self.inter, self.top_k = num_experts, hidden, inter, top_k
        self.asymmetric = bool(asymmetric)
        self.shared = bool(shared)
        if weight_bits not in (4, 8) or (weight_bits == 8 and asymmetric):
            raise ValueError("weight_bits must be 4, or 8 with symmetric weights")
        self.mixed = expert_bits is not None or expert_groups is not None
        nexp = num_experts + int(self.shared)
        if expert_groups is not None:
            groups = [int(g) for g in expert_groups]
            if len(groups) != nexp or any(g not in (32, 64, 128, 256) for g in groups):
                raise ValueError("expert_groups needs one group size (32, 64, 128, 256) per expert (and shared)")
            if asymmetric:
                raise ValueError("layers with per-expert group sizes are symmetric")
        else:
            groups = [128] * nexp
        self.groups = groups
        if expert_bits is not None:
            bits = [int(b) for b in expert_bits]
            if len(bits) != num_experts + int(self.shared) or any(b not in (2, 4, 8) for b in bits):
                raise ValueError("expert_bits needs one width, 2, 4 or 8, per expert (and the shared expert)")
            if asymmetric:
                raise ValueError("mixed layers are symmetric")
        else:
            bits = [weight_bits] * nexp
        if any(b != 4 and g != 128 for b, g in zip(bits, groups)):
            raise ValueError("2- and 8-bit experts use groups of 128")
        self.bits = bits
        self.weight_bits = 0 if self.mixed else weight_bits

        def sizes(b, g):
            if b == 8:
                return q8_device_bytes(2 * inter, hidden), q8_device_bytes(hidden, inter)
            if b == 2:
                return q2_device_bytes(2 * inter, hidden), q2_device_bytes(hidden, inter)
            return (q4_device_bytes_grouped(2 * inter, hidden, asymmetric, g),
                    q4_device_bytes_grouped(hidden, inter, asymmetric, g))

        sz = [sizes(b, g) for b, g in zip(bits, groups)]
        if any(a == 0 or b == 0 for a, b in sz):
            raise ValueError("hidden and inter must be multiples of 128")
        self.gu_offs, self.dn_offs = [0], [0]
        for a, b in sz[:num_experts]:
            self.gu_offs.append(self.gu_offs[-1] + a)
            self.dn_offs.append(self.dn_offs[-1] + b)
        self.gu_bytes, self.dn_bytes = sz[0]   # uniform layers: bytes of one expert
        self.gate_up = torch.empty(self.gu_offs[-1], dtype=torch.uint8, device=device)
        self.down = torch.empty(self.dn_offs[-1], dtype=torch.uint8, device=device)
        self.shared_gate_up = torch.empty(sz[-1][0], dtype=torch.uint8, device=device) if shared else None
        self.shared_down = torch.empty(sz[-1][1], dtype=torch.uint8, device=device) if shared else None
        if self.mixed:
            self.bits_dev = torch.tensor(bits, dtype=torch.uint8, device=device) if expert_bits is not None else None
            self.groups_dev = (torch.tensor([g // 32 for g in groups], dtype=torch.uint8, device=device)
                               if expert_groups is not None else None)
            self.gu_offs_dev = torch.tensor(self.gu_offs[:-1], dtype=torch.int64, device=device)
            self.dn_offs_dev = torch.tensor(self.dn_offs[:-1], dtype=torch.int64, device=device)
        self.desc = Q4MoELayer(num_experts, hidden, inter, top_k, int(self.asymmetric),
                               inter if shared else 0, self.gate_up.data_ptr(), self.down.data_ptr(),
                               self.shared_gate_up.data_ptr() if shared else None,
                               self.shared_down.data_ptr() if shared else None, self.weight_bits,
                               self.bits_dev.data_ptr() if self.mixed and self.bits_dev is not None else None,
                               self.gu_offs_dev.data_ptr() if self.mixed else None,
                               self.dn_offs_dev.data_ptr() if self.mixed else None,
                               self.groups_dev.data_ptr() if self.mixed and self.groups_dev is not None else None)

    def weight_bytes(self):
        """Device bytes of all expert weights."""
        return self.gate_up.numel() + self.down.numel() + (
            self.shared_gate_up.numel() + self.shared_down.numel() if self.shared else 0)

    def set_expert(self, e, gate, up, down):
        """Quantise (on the GPU) and place expert e; e == num_experts is the shared expert."""
        I, H = self.inter, self.hidden
        for name, t, shape in (("gate", gate, (I, H)), ("up", up, (I, H)), ("down", down, (H, I))):
            _need(t, (torch.float32, torch.float16, torch.bfloat16), name, 2)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must be {shape}, got {tuple(t.shape)}")
        if e == self.num_experts:
            if not self.shared:
                raise ValueError("layer has no shared expert")
            gu_out, dn_out = self.shared_gate_up, self.shared_down
        else:
            gu_out = self.gate_up[self.gu_offs[e]:self.gu_offs[e + 1]]
            dn_out = self.down[self.dn_offs[e]:self.dn_offs[e + 1]]
        if self.bits[e] == 8:
            q, s = quantize_int8_g128(torch.cat([gate, up], dim=0).contiguous())
            q8_repack_device(q, s, 2 * I, H, gate_up=True, out=gu_out)
            q, s = quantize_int8_g128(down.contiguous())
            q8_repack_device(q, s, H, I, gate_up=False, out=dn_out)
            return
        if self.bits[e] == 2:
            q, s = quantize_int2_g128(torch.cat([gate, up], dim=0).contiguous())
            q2_repack_device(q, s, 2 * I, H, gate_up=True, out=gu_out)
            q, s = quantize_int2_g128(down.contiguous())
            q2_repack_device(q, s, H, I, gate_up=False, out=dn_out)
            return
        if self.groups[e] != 128:
            grp = self.groups[e]
            pg, sg_, _ = quantize_int4_grouped(gate.contiguous(), grp)
            pu, su, _ = quantize_int4_grouped(up.contiguous(), grp)
            q4_repack_device_grouped(torch.cat([pg, pu], 0), torch.cat([sg_, su], 0), None, 2 * I, H, grp,
                                     gate_up=True, out=gu_out)
            dp, ds, _ = quantize_int4_grouped(down.contiguous(), grp)
            q4_repack_device_grouped(dp, ds, None, H, I, grp, out=dn_out)
            return
        g = H // 128
        dev = gate.device
        packed = torch.empty((2 * I, H // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((2 * I, g), dtype=torch.int16, device=dev)
        zeros = torch.empty((2 * I, (g + 1) // 2), dtype=torch.uint8, device=dev) if self.asymmetric else None
        for half, w in ((0, gate), (1, up)):
            sl = slice(half * I, (half + 1) * I)
            _check("quantize_int4_g128", _lib.quantize_int4_g128(
                _ptr(w), _DT[w.dtype], I, H, int(self.asymmetric), _ptr(packed[sl]), _ptr(scales[sl]),
                _ptr(zeros[sl]) if zeros is not None else ctypes.c_void_p(0), ctypes.c_void_p(0), _stream()))
        q4_repack_device(packed, scales, zeros, 2 * I, H, self.asymmetric, gate_up=True, out=gu_out)
        dp, ds, dz = quantize_int4_g128(down, self.asymmetric)
        q4_repack_device(dp, ds, dz, H, I, self.asymmetric, gate_up=False, out=dn_out)

    def workspace_bytes(self, t, mode):
        return int(_lib.moe_int4_ffn_workspace_bytes(ctypes.byref(self.desc), t, mode))


def moe_int4_ffn_forward(layer, x, ids, weights, mode=Q4_W4A16, out=None, workspace=None):
    """out [t, H] bf16 = sum_j w[t, j] FFN_{ids[t, j]}(x[t]) (+ shared)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(ids, torch.int32, "ids", 2)
    _need(weights, torch.float32, "weights", 2)
    t = x.shape[0]
    if x.shape[1] != layer.hidden or tuple(ids.shape) != (t, layer.top_k) or tuple(weights.shape) != (t, layer.top_k):
        raise ValueError("shape mismatch between x, ids, weights and the layer")
    if out is None:
        out = torch.empty_like(x)
    nbytes = layer.workspace_bytes(t, mode)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check("moe_int4_ffn_forward", _lib.moe_int4_ffn_forward(
        ctypes.byref(layer.desc), _ptr(x), t, _ptr(ids), _ptr(weights), mode, _ptr(out),
        _ptr(workspace), workspace.numel(), _stream()))
    return out


def moe_int4_ffn_forward_noalloc(layer, x, ids, weights, mode=Q4_W4A16, out=None):
    """moe_int4_ffn_forward with the library's own fixed device scratch as workspace
    (moe_int4_ffn_forward_noalloc): no workspace argument, no device allocation in the
    call; batches whose workspace exceeds the scratch size raise Q4Error."""
    _need(x, torch.bfloat16, "x", 2)
    _need(ids, torch.int32, "ids", 2)
    _need(weights, torch.float32, "weights", 2)
    t = x.shape[0]
    if x.shape[1] != layer.hidden or tuple(ids.shape) != (t, layer.top_k) or tuple(weights.shape) != (t, layer.top_k):
        raise ValueError("shape mismatch between x, ids, weights and the layer")
    if out is None:
        out = torch.empty_like(x)
    _need(out, torch.bfloat16, "out", 2)
    _check("moe_int4_ffn_forward_noalloc", _lib.moe_int4_ffn_forward_noalloc(
        ctypes.byref(layer.desc), _ptr(x), t, _ptr(ids), _ptr(weights), mode, _ptr(out), _stream()))
    return out


def moe_int4_ffn_debug(layer, x, ids, weights, mode=Q4_W4A16):
    """moe_int4_ffn_forward plus its intermediates: returns (out, views) where views
    maps counts, offsets, perm, inv, h, y (and q_x, s_x, q_h, s_h in W4A8) to tensors
    that are views into the call's workspace (shapes as in q4_ffn_views_t)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(ids, torch.int32, "ids", 2)
    _need(weights, torch.float32, "weights", 2)
    t = x.shape[0]
    if x.shape[1] != layer.hidden or tuple(ids.shape) != (t, layer.top_k) or tuple(weights.shape) != (t, layer.top_k):
        raise ValueError("shape mismatch between x, ids, weights and the layer")
    out = torch.empty_like(x)
    ws = torch.empty(max(layer.workspace_bytes(t, mode), 1), dtype=torch.uint8, device=x.device)
    v = Q4FfnViews()
    _check("moe_int4_ffn_debug", _lib.moe_int4_ffn_debug(
        ctypes.byref(layer.desc), _ptr(x), t, _ptr(ids), _ptr(weights), mode, _ptr(out),
        _ptr(ws), ws.numel(), ctypes.byref(v), _stream()))
    base = ws.data_ptr()
    P, S, E = int(v.positions), int(v.slots_per_token), layer.num_experts + (1 if layer.shared else 0)
    H, I = layer.hidden, layer.inter

    def view(ptr, dtype, shape):
        if not ptr:
            return None
        n = 1
        for d in shape:
            n *= d
        off = ptr - base
        esz = torch.empty((), dtype=dtype).element_size()
        return ws[off:off + n * esz].view(dtype).view(shape)

    views = {
        "slots_per_token": S,
        "counts": view(v.counts, torch.int32, (E,)),
        "offsets": view(v.offsets, torch.int32, (E + 1,)),
        "perm": view(v.perm, torch.int32, (P,)),
        "inv": view(v.inv, torch.int32, (P,)),
        "h": view(v.h, torch.float32 if v.h_is_f32 else torch.bfloat16, (P, I)),
        "y_slices": int(v.y_slices),
        "y_slice_groups": int(v.y_slice_groups),
        # [y_slices][P][H]: partial sums over consecutive K ranges (one slice: whole rows)
        "y": view(v.y, torch.float32, (int(v.y_slices), P, H)),
        "q_x": view(v.q_x, torch.int8, (t, H)),
        "s_x": view(v.s_x, torch.float32, (t,)),
        "q_h": view(v.q_h, torch.int8, (P, I)),
        "s_h": view(v.s_h, torch.float32, (P,)),
        "workspace": ws,
    }
    return out, views


class LoRALayer:
    """LoRA-mode MoE layer: one frozen INT4 g128 dense SwiGLU FFN (device layout) and
    rank-r bf16 adapters per expert, stacked as q4_lora_layer_t describes."""

    def __init__(self, num_experts, hidden, inter, top_k, rank, asymmetric=False, device="cuda"):
        self.num_experts, self.hidden, self.inter, self.top_k, self.rank = num_experts, hidden, inter, top_k, rank
        self.asymmetric = bool(asymmetric)
        E, H, I, r = num_experts, hidden, inter, rank
        self.gu_bytes = q4_device_bytes(2 * I, H, asymmetric)
        self.dn_bytes = q4_device_bytes(H, I, asymmetric)
        if self.gu_bytes == 0 or self.dn_bytes == 0:
            raise ValueError("hidden and inter must be multiples of 128")
        self.base_gate_up = torch.empty(self.gu_bytes, dtype=torch.uint8, device=device)
        self.base_down = torch.empty(self.dn_bytes, dtype=torch.uint8, device=device)
        bf = dict(dtype=torch.bfloat16, device=device)
        self.a_gate_up = torch.zeros((E, 2 * r, H), **bf)
        self.b_gate = torch.zeros((E, I, r), **bf)
        self.b_up = torch.zeros((E, I, r), **bf)
        self.a_down = torch.zeros((E, r, I), **bf)
        self.b_down = torch.zeros((E, H, r), **bf)
        self.desc = Q4LoraLayer(E, H, I, top_k, r, int(self.asymmetric), self.base_gate_up.data_ptr(),
                                self.base_down.data_ptr(), self.a_gate_up.data_ptr(), self.b_gate.data_ptr(),
                                self.b_up.data_ptr(), self.a_down.data_ptr(), self.b_down.data_ptr())

    def set_base(self, gate, up, down):
        """Quantise (on the GPU) and place the frozen dense FFN."""
        I, H = self.inter, self.hidden
        gu = torch.cat([gate, up], dim=0).contiguous()
        p, s, z = quantize_int4_g128(gu, self.asymmetric)
        q4_repack_device(p, s, z, 2 * I, H, self.asymmetric, gate_up=False, out=self.base_gate_up)
        p, s, z = quantize_int4_g128(down.contiguous(), self.asymmetric)
        q4_repack_device(p, s, z, H, I, self.asymmetric, gate_up=False, out=self.base_down)

    def set_adapters(self, e, ad):
        """ad: {"A_gate", "B_gate", "A_up", "B_up", "A_down", "B_down"} tensors (bf16 values)."""
        r = self.rank
        self.a_gate_up[e, :r] = ad["A_gate"]
        self.a_gate_up[e, r:] = ad["A_up"]
        self.b_gate[e] = ad["B_gate"]
        self.b_up[e] = ad["B_up"]
        self.a_down[e] = ad["A_down"]
        self.b_down[e] = ad["B_down"]

    def weight_bytes(self):
        ad = sum(t.numel() * 2 for t in (self.a_gate_up, self.b_gate, self.b_up, self.a_down, self.b_down))
        return self.gu_bytes + self.dn_bytes + ad

    def workspace_bytes(self, t):
        return int(_lib.moe_lora_ffn_workspace_bytes(ctypes.byref(self.desc), t))


def moe_lora_ffn_forward(layer, x, ids, weights, out=None, workspace=None):
    """out [t, H] bf16 = sum_j w[t, j] FFN_{ids[t, j]}(x[t]) for LoRA-mode experts."""
    _need(x, torch.bfloat16, "x", 2)
    _need(ids, torch.int32, "ids", 2)
    _need(weights, torch.float32, "weights", 2)
    t = x.shape[0]
    if x.shape[1] != layer.hidden or tuple(ids.shape) != (t, layer.top_k) or tuple(weights.shape) != (t, layer.top_k):
        raise ValueError("shape mismatch between x, ids, weights and the layer")
    if out is None:
        out = torch.empty_like(x)
    nbytes = layer.workspace_bytes(t)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check("moe_lora_ffn_forward", _lib.moe_lora_ffn_forward(
        ctypes.byref(layer.desc), _ptr(x), t, _ptr(ids), _ptr(weights), _ptr(out), _ptr(workspace),
        workspace.numel(), _stream()))
    return out


def int4_linear_forward(x, w_dev, n, asymmetric=False):
    """y [t, n] fp32 = x W_hat^T for x [t, k] fp16/bf16 and a PLAIN device-layout weight."""
    _need(x, (torch.float16, torch.bfloat16), "x", 2)
    _need(w_dev, torch.uint8, "w_dev")
    t, k = x.shape
    y = torch.empty((t, n), dtype=torch.float32, device=x.device)
    _check("int4_linear_forward", _lib.int4_linear_forward(
        _ptr(x), _DT[x.dtype], t, k, _ptr(w_dev), n, int(bool(asymmetric)), _ptr(y), _stream()))
    return y


def int8_w8a8_group_acc(q, w_dev, n):
    """INT32 group accumulators acc [rows, n, k/128] of int8 codes q [rows, k] with
    8-bit weights (q8_repack_device output)."""
    _need(q, torch.int8, "q", 2)
    _need(w_dev, torch.uint8, "w_dev")
    rows, k = q.shape
    acc = torch.empty((rows, n, k // 128), dtype=torch.int32, device=q.device)
    _check("int8_w8a8_group_acc", _lib.int8_w8a8_group_acc(
        _ptr(q), rows, k, _ptr(w_dev), n, _ptr(acc), _stream()))
    return acc


def int2_w2a8_group_acc(q, w_dev, n):
    """INT32 group accumulators acc [rows, n, k/128] of int8 codes q [rows, k] with a
    2-bit device-layout weight."""
    _need(q, torch.int8, "q", 2)
    _need(w_dev, torch.uint8, "w_dev")
    rows, k = q.shape
    acc = torch.empty((rows, n, k // 128), dtype=torch.int32, device=q.device)
    _check("int2_w2a8_group_acc", _lib.int2_w2a8_group_acc(_ptr(q), rows, k, _ptr(w_dev), n, _ptr(acc), _stream()))
    return acc


def int4_w4a8_group_acc(q, w_dev, n, asymmetric=False):
    """INT32 group accumulators acc [rows, n, k/128] of int8 codes q [rows, k]."""
    _need(q, torch.int8, "q", 2)
    _need(w_dev, torch.uint8, "w_dev")
    rows, k = q.shape
    acc = torch.empty((rows, n, k // 128), dtype=torch.int32, device=q.device)
    _check("int4_w4a8_group_acc", _lib.int4_w4a8_group_acc(
        _ptr(q), rows, k, _ptr(w_dev), n, int(bool(asymmetric)), _ptr(acc), _stream()))
    return acc
