"""Thin Python binding of libqmoe.so (the C ABI in include/qmoe.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers are handed to the library, and torch allocates the
output and workspace buffers. Every step of the MoE path runs in the library's HIP
kernels; there is no Python or CPU fallback. If the library is missing the first
call raises.
"""
import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "qmoe.h")

SCHEDULE_AUTO, SCHEDULE_DECODE, SCHEDULE_PREFILL = 0, 1, 2
FORMAT_W4A16, FORMAT_FP8, FORMAT_MXFP4, FORMAT_NVFP4 = 0, 1, 2, 3
STATUS = {0: "QMOE_OK", 1: "QMOE_ERR_INVALID_ARG", 2: "QMOE_ERR_UNSUPPORTED",
          3: "QMOE_ERR_WORKSPACE", 4: "QMOE_ERR_HIP"}

_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZP = ctypes.POINTER(ctypes.c_size_t)


class QMoEError(RuntimeError):
    def __init__(self, func, status, message):
        self.status = status
        super().__init__(f"{func}: {STATUS.get(status, status)}: {message}")


def load():
    """Load libqmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    lib.qmoe_abi_version.restype = _I32
    lib.qmoe_status_string.argtypes = [_I32]
    lib.qmoe_status_string.restype = ctypes.c_char_p
    lib.qmoe_last_error.restype = ctypes.c_char_p
    lib.moe_align.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P]
    lib.moe_align.restype = _I32
    lib.moe_topk_softmax.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P]
    lib.moe_topk_softmax.restype = _I32
    lib.moe_w4a16_forward.argtypes = [_P] * 7 + [_I32] * 6 + [_P, _P, _SZP, _P]
    lib.moe_w4a16_forward.restype = _I32
    lib.moe_w4a16_forward_noalloc.argtypes = [_P] * 7 + [_I32] * 6 + [_P, _P]
    lib.moe_w4a16_forward_noalloc.restype = _I32
    lib.moe_mxfp4_forward.argtypes = [_P] * 7 + [_I32] * 6 + [_P, _P, _SZP, _P]
    lib.moe_mxfp4_forward.restype = _I32
    lib.moe_nvfp4_forward.argtypes = [_P] * 9 + [_I32] * 6 + [_P, _P, _SZP, _P]
    lib.moe_nvfp4_forward.restype = _I32
    for name in ("moe_w4a16_grouped_contiguous", "moe_w4a16_grouped_masked"):
        fn = getattr(lib, name)
        fn.argtypes = [_P] * 6 + [_I32] * 6 + [_P, _P, _SZP, _P]
        fn.restype = _I32
    lib.moe_fp8_block_forward.argtypes = [_P] * 8 + [_I32] * 6 + [_P, _P, _SZP, _P]
    lib.moe_fp8_block_forward.restype = _I32
    lib.qmoe_fp8_quantize_blocks.argtypes = [_P, _I64, _I64, _I32, _I32, _P, _P, _P]
    lib.qmoe_fp8_quantize_blocks.restype = _I32
    lib.qmoe_fp8_quantize_blocks_bf16.argtypes = [_P, _I64, _I64, _I32, _I32, _P, _P, _P]
    lib.qmoe_fp8_quantize_blocks_bf16.restype = _I32
    lib.qmoe_plan.argtypes = [_I32] * 7 + [ctypes.POINTER(_I32), ctypes.POINTER(_I32), _SZP]
    lib.qmoe_plan.restype = _I32
    lib.qmoe_workspace_regions.argtypes = [_I32] * 7 + [ctypes.POINTER(_I64)] * 2
    lib.qmoe_workspace_regions.restype = _I32
    lib.qmoe_set_tuning.argtypes = [_I32] * 4
    lib.qmoe_set_tuning.restype = _I32
    _lib = lib
    return lib


def declared_functions():
    """Names of the functions include/qmoe.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def _check(func, status):
    if status != 0:
        msg = load().qmoe_last_error().decode(errors="replace")
        raise QMoEError(func, status, msg)


def _stream_ptr(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtypes, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_F8 = (torch.uint8, torch.float8_e4m3fn)


def plan(fmt, T, H, I, E, k, schedule=SCHEDULE_AUTO):
    """(chosen schedule, align block_m, workspace bytes) of a forward; host only."""
    chosen, bm, ws = _I32(0), _I32(0), ctypes.c_size_t(0)
    _check("qmoe_plan", load().qmoe_plan(fmt, T, H, I, E, k, schedule, ctypes.byref(chosen),
                                         ctypes.byref(bm), ctypes.byref(ws)))
    return chosen.value, bm.value, ws.value


REGIONS = ("sorted_ids", "expert_ids", "num_tokens_padded", "expert_offsets", "tile_offsets",
           "xs", "h", "h32", "hq", "hs", "out32", "y")


def workspace_regions(fmt, T, H, I, E, k, schedule=SCHEDULE_AUTO):
    """{region name: (byte offset, bytes)} of a forward's workspace, for the regions the
    plan has (qmoe_workspace_regions); host only."""
    n = len(REGIONS)
    offs, sizes = (_I64 * n)(), (_I64 * n)()
    _check("qmoe_workspace_regions",
           load().qmoe_workspace_regions(fmt, T, H, I, E, k, schedule, offs, sizes))
    return {name: (offs[i], sizes[i]) for i, name in enumerate(REGIONS) if offs[i] >= 0}


def set_tuning(tile_rows=0, rows_per_pass=0, kslices=0, tile_grid=0):
    """Process-wide schedule overrides of the 4-bit formats (qmoe_set_tuning); 0 keeps the
    library's choice. Set before planning; set_tuning() restores the defaults. Host only."""
    _check("qmoe_set_tuning", load().qmoe_set_tuning(tile_rows, rows_per_pass, kslices, tile_grid))


def moe_topk_softmax(logits, k, renormalize=True, expert_map=None, stream=None):
    """Router: (topk_ids int32 [T,k], topk_weights fp32 [T,k]) from fp32 logits [T,E].

    expert_map: optional int32 [E] GPU tensor of local ids (-1: expert held elsewhere).
    """
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    lp = _dev(logits, "logits", (torch.float32,))
    mp = None if expert_map is None else _dev(expert_map, "expert_map", (torch.int32,), (E,))
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    wts = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check("moe_topk_softmax",
           load().moe_topk_softmax(lp, T, E, k, 1 if renormalize else 0, mp, ids.data_ptr(),
                                   wts.data_ptr(), _stream_ptr(stream)))
    return ids, wts


def moe_align(topk_ids, E, block_m, stream=None):
    """Returns (sorted_ids [L], expert_ids [NB], num_tokens_padded [1], expert_offsets [E+1])."""
    T, k = topk_ids.shape
    ids = _dev(topk_ids, "topk_ids", (torch.int32,))
    P = T * k
    L = P + E * (block_m - 1)
    NB = (L + block_m - 1) // block_m
    dev = topk_ids.device
    sorted_ids = torch.empty(L, dtype=torch.int32, device=dev)
    expert_ids = torch.empty(NB, dtype=torch.int32, device=dev)
    ntp = torch.empty(1, dtype=torch.int32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    _check("moe_align", load().moe_align(ids, T, k, E, block_m, sorted_ids.data_ptr(),
                                         expert_ids.data_ptr(), ntp.data_ptr(), offs.data_ptr(),
                                         _stream_ptr(stream)))
    return sorted_ids, expert_ids, ntp, offs


def _workspace(fmt, T, H, I, E, k, schedule, workspace, device):
    need = plan(fmt, T, H, I, E, k, schedule)[2]
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def _four_bit_forward(name, fmt, sdtypes, x, w13, s13, w2, s2, topk_ids, topk_weights,
                      schedule, out, workspace, stream):
    T, H = x.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    k = topk_ids.shape[1]
    args = [_dev(x, "x", _BF16, (T, H)),
            _dev(w13, "w13", _U8, (E, 2 * I, H // 2)), _dev(s13, "s13", sdtypes, (E, 2 * I, H // 32)),
            _dev(w2, "w2", _U8, (E, H, I // 2)), _dev(s2, "s2", sdtypes, (E, H, I // 32)),
            _dev(topk_ids, "topk_ids", (torch.int32,), (T, k)),
            _dev(topk_weights, "topk_weights", (torch.float32,), (T, k))]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    optr = _dev(out, "out", _BF16, (T, H))
    workspace = _workspace(fmt, T, H, I, E, k, schedule, workspace, x.device)
    wptr = _dev(workspace, "workspace", (torch.uint8,))
    size = ctypes.c_size_t(workspace.numel())
    _check(name, getattr(load(), name)(*args, T, H, I, E, k, schedule, optr, wptr,
                                       ctypes.byref(size), _stream_ptr(stream)))
    return out


def moe_w4a16_forward(x, w13, s13, w2, s2, topk_ids, topk_weights, schedule=SCHEDULE_AUTO,
                      out=None, workspace=None, stream=None):
    return _four_bit_forward("moe_w4a16_forward", FORMAT_W4A16, _BF16, x, w13, s13, w2, s2,
                             topk_ids, topk_weights, schedule, out, workspace, stream)


def moe_w4a16_forward_noalloc(x, w13, s13, w2, s2, topk_ids, topk_weights,
                              schedule=SCHEDULE_AUTO, out=None, stream=None):
    """moe_w4a16_forward on the library's static per-GPU scratch instead of a workspace
    (nothing is allocated by the library; `out` may be given so that nothing is allocated
    here either). Shapes whose plan needs more than the scratch holds raise QMoEError."""
    T, H = x.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    k = topk_ids.shape[1]
    args = [_dev(x, "x", _BF16, (T, H)),
            _dev(w13, "w13", _U8, (E, 2 * I, H // 2)), _dev(s13, "s13", _BF16, (E, 2 * I, H // 32)),
            _dev(w2, "w2", _U8, (E, H, I // 2)), _dev(s2, "s2", _BF16, (E, H, I // 32)),
            _dev(topk_ids, "topk_ids", (torch.int32,), (T, k)),
            _dev(topk_weights, "topk_weights", (torch.float32,), (T, k))]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    optr = _dev(out, "out", _BF16, (T, H))
    _check("moe_w4a16_forward_noalloc",
           load().moe_w4a16_forward_noalloc(*args, T, H, I, E, k, schedule, optr,
                                            _stream_ptr(stream)))
    return out


def moe_mxfp4_forward(x, w13, s13, w2, s2, topk_ids, topk_weights, schedule=SCHEDULE_AUTO,
                      out=None, workspace=None, stream=None):
    """MXFP4 weights (E2M1 codes packed two per byte, E8M0 scales uint8 [.., K/32])."""
    return _four_bit_forward("moe_mxfp4_forward", FORMAT_MXFP4, _U8 + (torch.float8_e8m0fnu,),
                             x, w13, s13, w2, s2, topk_ids, topk_weights, schedule, out,
                             workspace, stream)

def moe_nvfp4_forward(x, w13, s13, g13, w2, s2, g2, topk_ids, topk_weights,
                      schedule=SCHEDULE_AUTO, out=None, workspace=None, stream=None):
    """NVFP4 weights: E2M1 codes packed two per byte, E4M3 scales uint8 [.., K/16], fp32
    scales per expert g13 [E] and g2 [E]."""
    T, H = x.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    k = topk_ids.shape[1]
    s8 = _U8 + (torch.float8_e4m3fn,)
    args = [_dev(x, "x", _BF16, (T, H)),
            _dev(w13, "w13", _U8, (E, 2 * I, H // 2)), _dev(s13, "s13", s8, (E, 2 * I, H // 16)),
            _dev(g13, "g13", (torch.float32,), (E,)),
            _dev(w2, "w2", _U8, (E, H, I // 2)), _dev(s2, "s2", s8, (E, H, I // 16)),
            _dev(g2, "g2", (torch.float32,), (E,)),
            _dev(topk_ids, "topk_ids", (torch.int32,), (T, k)),
            _dev(topk_weights, "topk_weights", (torch.float32,), (T, k))]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    optr = _dev(out, "out", _BF16, (T, H))
    workspace = _workspace(FORMAT_NVFP4, T, H, I, E, k, schedule, workspace, x.device)
    wptr = _dev(workspace, "workspace", (torch.uint8,))
    size = ctypes.c_size_t(workspace.numel())
    _check("moe_nvfp4_forward",
           load().moe_nvfp4_forward(*args, T, H, I, E, k, schedule, optr, wptr, ctypes.byref(size),
                                    _stream_ptr(stream)))
    return out


def _grouped(name, a2, w13, s13, w2, s2, route, M, rows, expected_m, schedule, out, workspace,
             stream):
    H = a2.shape[1]
    E, twoI, _ = w13.shape
    I = twoI // 2
    args = [_dev(a2, "a", _BF16, (rows, H)),
            _dev(w13, "w13", _U8, (E, 2 * I, H // 2)), _dev(s13, "s13", _BF16, (E, 2 * I, H // 32)),
            _dev(w2, "w2", _U8, (E, H, I // 2)), _dev(s2, "s2", _BF16, (E, H, I // 32)), route]
    if out is None:
        out = torch.empty((rows, H), dtype=torch.bfloat16, device=a2.device)
    optr = _dev(out, "out", _BF16, (rows, H))
    fn = getattr(load(), name)
    tail = (M, H, I, E, expected_m, schedule, optr)
    if workspace is None:
        need = ctypes.c_size_t(0)
        _check(name, fn(*args, *tail, None, ctypes.byref(need), _stream_ptr(stream)))
        workspace = torch.empty(max(need.value, 256), dtype=torch.uint8, device=a2.device)
    wptr = _dev(workspace, "workspace", (torch.uint8,))
    size = ctypes.c_size_t(workspace.numel())
    _check(name, fn(*args, *tail, wptr, ctypes.byref(size), _stream_ptr(stream)))
    return out

def grouped_workspace_bytes(masked, M, H, I, E, expected_m=0, schedule=SCHEDULE_AUTO):
    """Workspace bytes of a grouped forward (M = rows, or max_m when masked); host only."""
    name = "moe_w4a16_grouped_masked" if masked else "moe_w4a16_grouped_contiguous"
    need = ctypes.c_size_t(0)
    _check(name, getattr(load(), name)(*([None] * 6), M, H, I, E, expected_m, schedule, None, None,
                                       ctypes.byref(need), None))
    return need.value


def moe_w4a16_grouped_contiguous(a, w13, s13, w2, s2, m_indices, expected_m=0,
                                 schedule=SCHEDULE_AUTO, out=None, workspace=None, stream=None):
    """W4A16 expert FFN on rows grouped by expert: a [M, H] bf16, m_indices int32 [M] (the
    row's expert, -1 on padding rows). Returns [M, H] bf16, zero on padding rows."""
    M = a.shape[0]
    route = _dev(m_indices, "m_indices", (torch.int32,), (M,))
    return _grouped("moe_w4a16_grouped_contiguous", a, w13, s13, w2, s2, route, M, M, expected_m,
                    schedule, out, workspace, stream)


def moe_w4a16_grouped_masked(a, w13, s13, w2, s2, masked_m, expected_m=0,
                             schedule=SCHEDULE_AUTO, out=None, workspace=None, stream=None):
    """W4A16 expert FFN on a fixed row budget per expert: a [E, max_m, H] bf16, masked_m
    int32 [E] valid rows per expert (on the GPU). Returns [E * max_m, H] bf16, zero past
    each expert's count."""
    if a.dim() != 3:
        raise ValueError("a must be [E, max_m, H]")
    E, max_m, H = a.shape
    route = _dev(masked_m, "masked_m", (torch.int32,), (E,))
    if w13.shape[0] != E:
        raise ValueError(f"a holds {E} experts, w13 {w13.shape[0]}")
    return _grouped("moe_w4a16_grouped_masked", a.view(E * max_m, H), w13, s13, w2, s2, route,
                    max_m, E * max_m, expected_m, schedule, out, workspace, stream)


def moe_fp8_block_forward(a_q, a_scale, w13, s13, w2, s2, topk_ids, topk_weights,
                          schedule=SCHEDULE_AUTO, out=None, workspace=None, stream=None):
    T, H = a_q.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    k = topk_ids.shape[1]
    args = [_dev(a_q, "a_q", _F8, (T, H)), _dev(a_scale, "a_scale", (torch.float32,), (T, H // 128)),
            _dev(w13, "w13", _F8, (E, 2 * I, H)),
            _dev(s13, "s13", (torch.float32,), (E, 2 * I // 128, H // 128)),
            _dev(w2, "w2", _F8, (E, H, I)),
            _dev(s2, "s2", (torch.float32,), (E, H // 128, I // 128)),
            _dev(topk_ids, "topk_ids", (torch.int32,), (T, k)),
            _dev(topk_weights, "topk_weights", (torch.float32,), (T, k))]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=a_q.device)
    optr = _dev(out, "out", _BF16, (T, H))
    workspace = _workspace(FORMAT_FP8, T, H, I, E, k, schedule, workspace, a_q.device)
    wptr = _dev(workspace, "workspace", (torch.uint8,))
    size = ctypes.c_size_t(workspace.numel())
    _check("moe_fp8_block_forward",
           load().moe_fp8_block_forward(*args, T, H, I, E, k, schedule, optr, wptr,
                                        ctypes.byref(size), _stream_ptr(stream)))
    return out


def fp8_quantize_blocks(v, br, bc, stream=None):
    """Block E4M3 quantizer on a 2-D fp32 or bf16 GPU tensor: returns (codes uint8, scales
    fp32). bf16 values are widened exactly, so they quantize like their fp32 values."""
    R, C = v.shape
    bf16 = v.dtype in _BF16
    vptr = _dev(v, "v", _BF16 if bf16 else (torch.float32,))
    q = torch.empty((R, C), dtype=torch.uint8, device=v.device)
    s = torch.empty(((R + br - 1) // br, (C + bc - 1) // bc), dtype=torch.float32, device=v.device)
    name = "qmoe_fp8_quantize_blocks_bf16" if bf16 else "qmoe_fp8_quantize_blocks"
    _check(name, getattr(load(), name)(vptr, R, C, br, bc, q.data_ptr(), s.data_ptr(),
                                       _stream_ptr(stream)))
    return q, s
