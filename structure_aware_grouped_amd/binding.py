"""ctypes binding of librs_hip.so: the C-ABI calls under the same names.

Argument marshalling only (torch tensors -> device pointers and sizes, spec
lists -> C structs, the current HIP stream); every step of the layout
transform runs in the library. torch is imported before the library is
opened so that the library binds to the HIP runtime torch already loaded.
If the library is missing, load() raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import json
import os
from typing import List, NamedTuple, Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librs_hip.so")

RS_OK, RS_EINVAL, RS_EPLAN, RS_EALIGN, RS_EDTYPE, RS_ENOMEM, RS_EHIP, RS_ERANGE = 0, -1, -2, -3, -4, -5, -6, -7
STATUS_NAMES = {0: "RS_OK", -1: "RS_EINVAL", -2: "RS_EPLAN", -3: "RS_EALIGN", -4: "RS_EDTYPE",
                -5: "RS_ENOMEM", -6: "RS_EHIP", -7: "RS_ERANGE"}
KINDS = {"ELEM": 0, "ROWS": 1, "TILE": 2, "FLAT": 3, "WHOLE": 4, "TILEMAJOR": 5}
ORDER_KINDS = {0: "default", 1: "by_block_size", 2: "by_shape"}
RS_F32, RS_BF16, RS_E4M3, RS_I8, RS_U8 = 0, 1, 2, 3, 4
CODE_FORMATS = {"e4m3": RS_E4M3, "i8": RS_I8, "u8": RS_U8}
EXPORTS = ("rs_plan_build", "rs_plan_load", "rs_plan_info", "rs_plan_free", "rs_unpack_gathered",
           "rs_pack_scatter", "rs_block_quant", "rs_block_dequant", "rs_unpack_dequant", "rs_adam8_step",
           "rs_last_error", "rs_block_quant_noalloc")


class RsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class AdamHParamsC(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("step", ctypes.c_int64)]


class TensorSpecC(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("kind", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("p0", ctypes.c_int64), ("p1", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with structure_aware_grouped_amd.build "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    PI64 = ctypes.POINTER(ctypes.c_int64)
    PI32 = ctypes.POINTER(ctypes.c_int32)
    lib.rs_plan_build.argtypes = [ctypes.POINTER(TensorSpecC), I64, I64, I64, I32, PI64, PI64, PI64, PI32]
    lib.rs_plan_load.argtypes = [ctypes.POINTER(TensorSpecC), I64, I64, I64, PI64, I64, I32,
                                 ctypes.POINTER(P)]
    lib.rs_plan_info.argtypes = [P, PI64, PI64, PI64]
    lib.rs_plan_free.argtypes = [P]
    lib.rs_plan_free.restype = None
    lib.rs_unpack_gathered.argtypes = [P, P, I32, ctypes.POINTER(P), P]
    lib.rs_pack_scatter.argtypes = [P, ctypes.POINTER(P), I32, P, P, I32, I32, F, P]
    lib.rs_block_quant.argtypes = [P, P, I32, P, I32, P, P]
    lib.rs_block_dequant.argtypes = [P, P, I32, P, P, P]
    lib.rs_unpack_dequant.argtypes = [P, P, I32, P, ctypes.POINTER(P), I32, P]
    lib.rs_adam8_step.argtypes = [P, P, P, P, P, P, P, ctypes.POINTER(AdamHParamsC), P]
    lib.rs_block_quant_noalloc.argtypes = [ctypes.POINTER(TensorSpecC), I64, I64, I64, PI64, I64, P, I32, P, I32,
                                           P, I64, P]
    lib.rs_last_error.argtypes = []
    lib.rs_last_error.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("rs_plan_free", "rs_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != RS_OK:
        raise RsError(status, load().rs_last_error().decode())


def specs_array(specs) -> ctypes.Array:
    arr = (TensorSpecC * len(specs))()
    for i, s in enumerate(specs):
        arr[i].rows, arr[i].cols = int(s.rows), int(s.cols)
        arr[i].kind = KINDS[s.kind] if isinstance(s.kind, str) else int(s.kind)
        arr[i].reserved = 0
        arr[i].p0, arr[i].p1 = int(getattr(s, "p0", 0)), int(getattr(s, "p1", 0))
    return arr


def _i64(values) -> ctypes.Array:
    return (ctypes.c_int64 * len(values))(*[int(v) for v in values])


def _ptrs(tensors) -> ctypes.Array:
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _copy_code(t: torch.Tensor) -> int:
    """Unpack copies bits: only the element size matters (4, 2 or 1 bytes)."""
    code = {4: RS_F32, 2: RS_BF16, 1: RS_U8}.get(t.element_size())
    if code is None:
        raise TypeError(f"unsupported element size {t.element_size()}")
    return code


# ---------------------------------------------------------------- planner

def rs_plan_build(specs, V: int, align: int = 16, policy: str = "best"):
    """(S, starts, order, order_name) from the host planner. policy: "best" (the three orders),
    or one order: "default", "by_block_size", "by_shape"."""
    lib = load()
    n = len(specs)
    S = ctypes.c_int64()
    starts = (ctypes.c_int64 * n)()
    order = (ctypes.c_int64 * n)()
    kind = ctypes.c_int32()
    pol = {"best": 0, "default": 1, "by_block_size": 2, "by_shape": 3}[policy]
    _check(lib.rs_plan_build(specs_array(specs), n, int(V), int(align), pol, ctypes.byref(S),
                             starts, order, ctypes.byref(kind)))
    return S.value, list(starts), list(order), ORDER_KINDS[kind.value]


# ---------------------------------------------------------------- plans as data

PLAN_FORMAT = "rs-plan/1"


class PlanSpec(NamedTuple):
    """One tensor of a plan read back from JSON (the fields rs_plan_load reads)."""
    name: str
    rows: int
    cols: int
    kind: str
    p0: int = 0
    p1: int = 0

    @property
    def numel(self) -> int:
        return self.rows * self.cols


def plan_to_json(specs, V: int, S: int, starts: Sequence[int], R_mat: Optional[int] = None) -> str:
    """A plan as JSON. A plan is pure data: the tensors (shape and atomic block),
    V, S, the starts and the materialised ranks. rs_plan_load validates it again
    and rebuilds the same device work lists from it, so a saved plan resumes a
    group without planning again."""
    kinds = {v: k for k, v in KINDS.items()}
    out = []
    for i, sp in enumerate(specs):
        kind = sp.kind if isinstance(sp.kind, str) else kinds[int(sp.kind)]
        out.append({"name": str(getattr(sp, "name", f"t{i}")), "rows": int(sp.rows), "cols": int(sp.cols),
                    "kind": kind, "p0": int(getattr(sp, "p0", 0)), "p1": int(getattr(sp, "p1", 0))})
    return json.dumps({"format": PLAN_FORMAT, "V": int(V), "S": int(S), "R_mat": int(V if R_mat is None else R_mat),
                       "starts": [int(x) for x in starts], "tensors": out})


def plan_from_json(text: str):
    """(specs, V, S, starts, R_mat) from plan_to_json's output; checks the format
    and the field types only (validation is rs_plan_load's)."""
    d = json.loads(text)
    if d.get("format") != PLAN_FORMAT:
        raise ValueError(f"not an {PLAN_FORMAT} plan: format {d.get('format')!r}")
    specs = []
    for t in d["tensors"]:
        if t["kind"] not in KINDS:
            raise ValueError(f"unknown block kind {t['kind']!r}")
        specs.append(PlanSpec(str(t["name"]), int(t["rows"]), int(t["cols"]), t["kind"], int(t["p0"]), int(t["p1"])))
    starts = [int(x) for x in d["starts"]]
    if len(starts) != len(specs):
        raise ValueError(f"{len(starts)} starts for {len(specs)} tensors")
    return specs, int(d["V"]), int(d["S"]), starts, int(d["R_mat"])


class Plan:
    """A loaded plan (device work lists); freed with close() or when collected."""

    def __init__(self, handle, specs, V, S, starts, R_mat, device):
        self._h = handle
        self.specs, self.V, self.S, self.starts = list(specs), V, S, list(starts)
        self.R_mat, self.device = R_mat, device
        r, q, pad = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(load().rs_plan_info(handle, ctypes.byref(r), ctypes.byref(q), ctypes.byref(pad)))
        self.R_used, self.n_qblocks, self.padding = r.value, q.value, pad.value
        self.numels = [int(s.rows) * int(s.cols) for s in specs]

    def to_json(self) -> str:
        return plan_to_json(self.specs, self.V, self.S, self.starts, self.R_mat)

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("plan already freed")
        return self._h

    def close(self):
        if self._h is not None:
            load().rs_plan_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rs_plan_load(specs, V: int, S: int, starts: Sequence[int], R_mat: Optional[int] = None,
                 device: int = 0) -> Plan:
    lib = load()
    n = len(specs)
    if R_mat is None:
        R_mat = V
    h = ctypes.c_void_p()
    _check(lib.rs_plan_load(specs_array(specs), n, int(V), int(S), _i64(starts), int(R_mat),
                            int(device), ctypes.byref(h)))
    return Plan(h, specs, int(V), int(S), starts, int(R_mat), int(device))


# ---------------------------------------------------------------- transforms

def _count_check(plan: Plan, items, what: str):
    """The C calls read exactly one pointer per tensor of the plan."""
    if len(items) != len(plan.numels):
        raise ValueError(f"{what}: {len(items)} entries for a plan of {len(plan.numels)} tensors")


def _scales_check(plan: Plan, scales: torch.Tensor):
    """The kernels read n_qblocks fp32 scales: a tensor of another dtype with that many
    entries would be read past its end."""
    if scales.dtype != torch.float32 or scales.numel() < plan.n_qblocks:
        raise ValueError("scales: fp32 with n_qblocks entries")


def _dev_check(plan: Plan, *tensors):
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda" or t.device.index != plan.device:
            raise ValueError(f"tensor on {t.device}, plan on cuda:{plan.device}")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def rs_unpack_gathered(plan: Plan, gathered: torch.Tensor, dsts: List[torch.Tensor]):
    """dst_i <- gathered[s_i : s_i + n_i] for every tensor (same dtype)."""
    _count_check(plan, dsts, "dsts")
    _dev_check(plan, gathered, *dsts)
    if gathered.numel() < plan.R_mat * plan.S:
        raise ValueError("gathered buffer shorter than R_mat * S")
    for d, n in zip(dsts, plan.numels):
        if d.numel() != n or d.dtype != gathered.dtype:
            raise ValueError("destination size or dtype does not match its tensor")
    _check(load().rs_unpack_gathered(plan.handle, gathered.data_ptr(), _copy_code(gathered),
                                     _ptrs(dsts), _stream(plan.device)))


def rs_pack_scatter(plan: Plan, srcs: List[torch.Tensor], packed: torch.Tensor,
                    prev: Optional[torch.Tensor] = None, scale: Optional[float] = None):
    """packed <- [prev +] src * sigma on tensors, +0.0 on padding; sigma = fl32(1/V) unless given.
    packed is fp32, or bf16 (each fp32 result rounded once to nearest even); prev is fp32."""
    _count_check(plan, srcs, "srcs")
    if srcs[0].dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("sources are fp32 or bf16")
    _dev_check(plan, packed, prev, *srcs)
    if packed.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("packed is fp32 or bf16")
    if prev is not None and prev.dtype != torch.float32:
        raise ValueError("prev is fp32")
    if packed.numel() < plan.R_mat * plan.S or (prev is not None and prev.numel() < plan.R_mat * plan.S):
        raise ValueError("packed / prev shorter than R_mat * S")
    dt = srcs[0].dtype
    for s, n in zip(srcs, plan.numels):
        if s.numel() != n or s.dtype != dt:
            raise ValueError("source size or dtype does not match its tensor")
    mode, val = (0, 0.0) if scale is None else (1, float(scale))
    _check(load().rs_pack_scatter(plan.handle, _ptrs(srcs), RS_F32 if dt == torch.float32 else RS_BF16,
                                  prev.data_ptr() if prev is not None else None, packed.data_ptr(),
                                  RS_F32 if packed.dtype == torch.float32 else RS_BF16,
                                  mode, ctypes.c_float(val), _stream(plan.device)))


def rs_block_quant(plan: Plan, src: torch.Tensor, q: torch.Tensor, fmt: str, scales: torch.Tensor):
    """Per-block absmax codes (fmt "e4m3" | "i8" | "u8") of the flat buffer, plus fp32 scales."""
    _scales_check(plan, scales)
    _dev_check(plan, src, q, scales)
    if src.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("src is fp32 or bf16")
    if src.numel() < plan.R_mat * plan.S or q.numel() * q.element_size() < plan.R_mat * plan.S:
        raise ValueError("src / q shorter than R_mat * S")
    _check(load().rs_block_quant(plan.handle, src.data_ptr(),
                                 RS_F32 if src.dtype == torch.float32 else RS_BF16, q.data_ptr(),
                                 CODE_FORMATS[fmt], scales.data_ptr(), _stream(plan.device)))


def rs_block_dequant(plan: Plan, q: torch.Tensor, fmt: str, scales: torch.Tensor, out: torch.Tensor):
    """out <- code value * block scale inside blocks, +0.0 elsewhere."""
    _scales_check(plan, scales)
    _dev_check(plan, q, scales, out)
    if out.dtype != torch.float32 or out.numel() < plan.R_mat * plan.S:
        raise ValueError("out: fp32 with R_mat * S entries")
    if q.numel() * q.element_size() < plan.R_mat * plan.S or scales.numel() < plan.n_qblocks:
        raise ValueError("q / scales too short")
    _check(load().rs_block_dequant(plan.handle, q.data_ptr(), CODE_FORMATS[fmt], scales.data_ptr(),
                                   out.data_ptr(), _stream(plan.device)))


def rs_unpack_dequant(plan: Plan, q: torch.Tensor, fmt: str, scales: torch.Tensor,
                      dsts: List[Optional[torch.Tensor]]):
    """dst_i <- fl32(code value * block scale) (rounded to bf16 for bf16 tensors) for every
    quantised tensor; entries for other tensors may be None."""
    _scales_check(plan, scales)
    _count_check(plan, dsts, "dsts")
    _dev_check(plan, q, scales, *[d for d in dsts if d is not None])
    if q.numel() * q.element_size() < plan.R_mat * plan.S or scales.numel() < plan.n_qblocks:
        raise ValueError("q / scales too short")
    dt = None
    for d, n, sp in zip(dsts, plan.numels, plan.specs):
        if d is None:
            continue
        if d.numel() != n or d.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("destination size or dtype does not match its tensor")
        if dt is not None and d.dtype != dt:
            raise ValueError("destinations share one dtype")
        dt = d.dtype
    ptrs = (ctypes.c_void_p * len(dsts))(*[d.data_ptr() if d is not None else None for d in dsts])
    _check(load().rs_unpack_dequant(plan.handle, q.data_ptr(), CODE_FORMATS[fmt], scales.data_ptr(), ptrs,
                                    RS_BF16 if dt == torch.bfloat16 else RS_F32, _stream(plan.device)))


def rs_adam8_step(plan: Plan, param: torch.Tensor, grad: torch.Tensor, q_m: torch.Tensor,
                  s_m: torch.Tensor, q_v: torch.Tensor, s_v: torch.Tensor, lr: float, beta1: float,
                  beta2: float, eps: float, weight_decay: float, step: int):
    """One AdamW step on every quantisation block, in place: param (fp32 flat), int8 m codes and
    scales, uint8 v codes and scales; grad is the packed fp32 gradient."""
    _dev_check(plan, param, grad, q_m, s_m, q_v, s_v)
    total = plan.R_mat * plan.S
    for t, dt in ((param, torch.float32), (grad, torch.float32), (s_m, torch.float32), (s_v, torch.float32)):
        if t.dtype != dt:
            raise ValueError("param, grad and scales are fp32")
    if param.numel() < total or grad.numel() < total or q_m.numel() < total or q_v.numel() < total:
        raise ValueError("buffers shorter than R_mat * S")
    if s_m.numel() < plan.n_qblocks or s_v.numel() < plan.n_qblocks:
        raise ValueError("scales shorter than n_qblocks")
    hp = AdamHParamsC(lr, beta1, beta2, eps, weight_decay, 0, int(step))
    _check(load().rs_adam8_step(plan.handle, param.data_ptr(), grad.data_ptr(), q_m.data_ptr(), s_m.data_ptr(),
                                q_v.data_ptr(), s_v.data_ptr(), ctypes.byref(hp), _stream(plan.device)))


def rs_block_quant_noalloc(specs, V: int, S: int, starts: Sequence[int], R_mat: int, src: torch.Tensor,
                           q: torch.Tensor, fmt: str, scales: torch.Tensor):
    """rs_block_quant without a loaded plan and without any allocation on the device: the
    plan is passed as data and its work list goes into the library's static device memory
    (calls that overlap on one GPU race; calls in order on one stream do not)."""
    if src.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("src is fp32 or bf16")
    if scales.dtype != torch.float32:
        raise ValueError("scales: fp32")
    for t in (src, q, scales):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("src, q and scales are contiguous device tensors")
    if src.numel() < R_mat * S or q.numel() * q.element_size() < R_mat * S:
        raise ValueError("src / q shorter than R_mat * S")
    _check(load().rs_block_quant_noalloc(specs_array(specs), len(specs), int(V), int(S), _i64(starts), int(R_mat),
                                         src.data_ptr(), RS_F32 if src.dtype == torch.float32 else RS_BF16,
                                         q.data_ptr(), CODE_FORMATS[fmt], scales.data_ptr(), scales.numel(),
                                         _stream(src.device)))
