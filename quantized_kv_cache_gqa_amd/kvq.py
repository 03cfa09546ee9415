"""ctypes binding of libkvq.so (argument marshalling only).

Every step of the path runs in the library's HIP kernels; this module turns
torch tensors into the plain pointers and sizes of include/kvq.h and allocates
output buffers with torch.  It raises if the built library is missing: there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")
# the same kernels with kvq_test_set_team_hooks (tests only)
TEST_LIB_PATH = os.path.join(_PKG, "libkvq_test.so")

FMT = {"bf16": 0, "fp8": 1, "int8": 2, "fp32": 3, "int8g32": 5}
INT8_GROUP = 32                # channels per scale of "int8g32"
HEAD_DIM = 128
N_BANDS = 16
INT8_BLOCK = 256
STATUS = {0: "ok", 1: "null", 2: "shape", 3: "format", 4: "align", 5: "unsupported",
          6: "workspace", 7: "launch"}
# plan flags (kvq_attn_args.plan_flags) and device status bits
PLAN_NO_TEAM = 0x01
PLAN_VECTOR_ALU = 0x02
PLAN_GROUP8_SEPARATE = 0x04
PLAN_FINALIZE_IN_PLACE = 0x08
PLAN_LAUNCH_PER_REGION = 0x10
DEVSTATUS_TEAM_WAIT = 0x1


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: kvq status {status} ({STATUS.get(status, '?')})")
        self.status = status


c_void_p = ctypes.c_void_p
c_int32 = ctypes.c_int32


class Region(ctypes.Structure):
    _fields_ = [("k_format", c_int32), ("v_format", c_int32), ("k", c_void_p), ("v", c_void_p),
                ("k_scale", c_void_p), ("v_scale", c_void_p), ("witness", c_void_p),
                ("k_exact", c_void_p), ("k_exact_format", c_int32), ("length", c_int32),
                ("lengths", c_void_p), ("page_table", c_void_p), ("page_size", c_int32),
                ("max_pages", c_int32), ("seed", ctypes.c_uint64), ("layer", c_int32),
                ("stream_id", c_int32), ("stream_ids", c_void_p), ("v_witness", c_void_p),
                ("outlier_pairs", c_void_p), ("k_outliers", c_void_p), ("n_outlier_pairs", c_int32)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("num_q_heads", c_int32), ("num_kv_heads", c_int32),
                ("head_dim", c_int32), ("sm_scale", ctypes.c_float), ("split_tokens", c_int32),
                ("plan_flags", ctypes.c_uint32), ("status", c_void_p),
                ("q", c_void_p), ("prefix", Region), ("suffix", Region), ("out", c_void_p)]


class MeterOut(ctypes.Structure):
    _fields_ = [("tv", c_void_p), ("bound_raw", c_void_p), ("meter", c_void_p), ("log_a", c_void_p),
                ("log_a_b", c_void_p), ("bound_b_raw", c_void_p), ("meter_b", c_void_p),
                ("delta_b", ctypes.c_double), ("value_err", c_void_p), ("v_norm_max", c_void_p),
                ("out_bound", c_void_p), ("log_a_minus", c_void_p), ("bound_two_sided", c_void_p),
                ("meter_two_sided", c_void_p), ("block_mass", c_void_p), ("block_excess", c_void_p),
                ("block_excess_b", c_void_p), ("block_order", c_void_p), ("bound_tanh", c_void_p)]


class QuantArgs(ctypes.Structure):
    _fields_ = [("k_format", c_int32), ("v_format", c_int32), ("in_format", c_int32),
                ("k_in", c_void_p), ("v_in", c_void_p), ("n_seq", c_int32),
                ("num_kv_heads", c_int32), ("head_dim", c_int32), ("capacity", c_int32),
                ("tok_begin", c_int32), ("tok_end", c_int32), ("k_out", c_void_p),
                ("v_out", c_void_p), ("k_scale_out", c_void_p), ("v_scale_out", c_void_p),
                ("witness_out", c_void_p), ("seed", ctypes.c_uint64), ("layer", c_int32),
                ("stream_id", c_int32), ("stream_ids", c_void_p), ("v_witness_out", c_void_p),
                ("outlier_pairs", c_void_p), ("k_outliers_out", c_void_p), ("n_outlier_pairs", c_int32)]


_libs = {}                      # loaded libraries by absolute path

SYMBOLS = ["kvq_abi_version", "kvq_status_string", "kvq_quantize", "kvq_workspace_bytes",
           "kvq_decode_plan", "kvq_workspace_init", "kvq_decode_attn", "kvq_meter",
           "kvq_decode_attn_noalloc"]
SCRATCH_BYTES = 96 << 20       # KVQ_SCRATCH_BYTES: the static scratch of kvq_decode_attn_noalloc
ABI_VERSION = 11


class PlanInfo(ctypes.Structure):
    _fields_ = [("team", c_int32), ("n_teams", c_int32), ("rounds", c_int32), ("grid", c_int32),
                ("chunk", c_int32), ("chunks", c_int32), ("launches", c_int32), ("reserved", c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (after torch, so both share torch's HIP runtime)."""
    path = os.path.abspath(path)
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{os.path.basename(path)} not built at {path}; run quantized_kv_cache_gqa_amd.build")
    lib = ctypes.CDLL(path)
    lib.kvq_abi_version.restype = ctypes.c_int
    if lib.kvq_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path}: ABI version {lib.kvq_abi_version()}, this binding is {ABI_VERSION}")
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_quantize.restype = ctypes.c_int
    lib.kvq_quantize.argtypes = [ctypes.POINTER(QuantArgs), c_void_p]
    lib.kvq_workspace_bytes.restype = ctypes.c_size_t
    lib.kvq_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(MeterOut)]
    lib.kvq_decode_plan.restype = ctypes.c_int
    lib.kvq_decode_plan.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(MeterOut), ctypes.c_int,
                                    ctypes.POINTER(PlanInfo)]
    lib.kvq_workspace_init.restype = ctypes.c_int
    lib.kvq_workspace_init.argtypes = [c_void_p, ctypes.c_size_t, c_void_p]
    for name in ("kvq_decode_attn", "kvq_meter"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(MeterOut), c_void_p,
                      ctypes.c_size_t, c_void_p]
    lib.kvq_decode_attn_noalloc.restype = ctypes.c_int
    lib.kvq_decode_attn_noalloc.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(MeterOut), c_void_p]
    if hasattr(lib, "kvq_test_set_team_hooks"):
        lib.kvq_test_set_team_hooks.restype = None
        lib.kvq_test_set_team_hooks.argtypes = [ctypes.c_uint, ctypes.c_int]
    _libs[path] = lib
    return lib


def load_test() -> ctypes.CDLL:
    """The test build (same kernels, plus kvq_test_set_team_hooks)."""
    return load(TEST_LIB_PATH)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("kvq: tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("kvq: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(status: int, what: str) -> None:
    if status != 0:
        raise KvqError(status, what)


# ------------------------------------------------------------------ write path

@dataclass
class Stored:
    """Stored codes, scales and witness of one region (prefix: n_seq = 1, squeezed)."""
    fmt_k: str
    fmt_v: str
    k: torch.Tensor
    v: Optional[torch.Tensor]
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    witness: Optional[torch.Tensor]
    v_witness: Optional[torch.Tensor] = None   # fp16 [.., capacity, 2]: rho, ||v||
    k_outliers: Optional[torch.Tensor] = None  # bf16 bits [.., capacity, 2 m]: the bypassed key values
    outlier_pairs: Optional[torch.Tensor] = None   # int32 [h_kv, m]: fixed outlier RoPE pairs

    @property
    def n_outlier_pairs(self) -> int:
        return 0 if self.outlier_pairs is None else int(self.outlier_pairs.shape[1])


def alloc_stored(n_seq: int, h_kv: int, capacity: int, fmt_k: str, fmt_v: Optional[str],
                 witness: bool, device, value_witness: bool = False,
                 outlier_pairs: Optional[torch.Tensor] = None) -> Stored:
    """outlier_pairs: int32 [h_kv, m] fixed outlier RoPE pairs of "int8g32" keys
    (kept exactly, left out of the group maximum), or None."""
    def codes(fmt):
        dt = {"bf16": torch.bfloat16, "fp8": torch.uint8, "int8": torch.int8, "int8g32": torch.int8}[fmt]
        return torch.zeros((n_seq, h_kv, capacity, HEAD_DIM), dtype=dt, device=device)

    def scale(fmt):
        if fmt == "fp8":
            return torch.zeros((n_seq, h_kv, capacity), dtype=torch.float32, device=device)
        if fmt == "int8":
            nb = (capacity + INT8_BLOCK - 1) // INT8_BLOCK
            return torch.zeros((n_seq, h_kv, nb, HEAD_DIM), dtype=torch.float16, device=device)
        if fmt == "int8g32":                    # per (token, 32-channel group)
            return torch.zeros((n_seq, h_kv, capacity, HEAD_DIM // INT8_GROUP), dtype=torch.float16,
                               device=device)
        return None

    return Stored(fmt_k, fmt_v or "bf16", codes(fmt_k), codes(fmt_v) if fmt_v else None,
                  scale(fmt_k), scale(fmt_v) if fmt_v else None,
                  torch.zeros((n_seq, h_kv, capacity, N_BANDS), dtype=torch.float16, device=device)
                  if witness else None,
                  torch.zeros((n_seq, h_kv, capacity, 2), dtype=torch.float16, device=device)
                  if value_witness and fmt_v else None,
                  torch.zeros((n_seq, h_kv, capacity, 2 * outlier_pairs.shape[1]), dtype=torch.int16,
                              device=device) if outlier_pairs is not None else None,
                  outlier_pairs)


def quantize_into(st: Stored, k_in: torch.Tensor, v_in: Optional[torch.Tensor], *, tok_begin: int = 0,
                  tok_end: Optional[int] = None, seed: int = 0, layer: int = 0, stream_id: int = 0,
                  stream_ids: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvq_quantize: k_in / v_in are [n_seq, h_kv, capacity, 128] bf16 or fp32."""
    lib = load()
    n_seq, h_kv, cap, d = k_in.shape
    in_fmt = {torch.bfloat16: FMT["bf16"], torch.float32: FMT["fp32"]}[k_in.dtype]
    if v_in is not None and v_in.dtype != k_in.dtype:
        raise ValueError("k_in and v_in must share a dtype")
    a = QuantArgs(k_format=FMT[st.fmt_k], v_format=FMT[st.fmt_v], in_format=in_fmt,
                  k_in=_ptr(k_in), v_in=_ptr(v_in), n_seq=n_seq, num_kv_heads=h_kv, head_dim=d,
                  capacity=cap, tok_begin=tok_begin, tok_end=cap if tok_end is None else tok_end,
                  k_out=_ptr(st.k), v_out=_ptr(st.v) if v_in is not None else None,
                  k_scale_out=_ptr(st.k_scale),
                  v_scale_out=_ptr(st.v_scale) if v_in is not None else None,
                  witness_out=_ptr(st.witness), seed=seed, layer=layer, stream_id=stream_id,
                  stream_ids=_ptr(stream_ids),
                  v_witness_out=_ptr(st.v_witness) if v_in is not None else None,
                  outlier_pairs=_ptr(st.outlier_pairs), k_outliers_out=_ptr(st.k_outliers),
                  n_outlier_pairs=st.n_outlier_pairs)
    _check(lib.kvq_quantize(ctypes.byref(a), _stream(stream)), "kvq_quantize")


# ------------------------------------------------------------------ read path

@dataclass
class RegionView:
    """One KV region as the decode call sees it (torch tensors, all on the GPU)."""
    stored: Stored
    length: int                              # prefix tokens / suffix capacity
    k_exact: Optional[torch.Tensor] = None   # bf16 or fp32, same layout as the codes
    lengths: Optional[torch.Tensor] = None   # int32 [batch]
    page_table: Optional[torch.Tensor] = None
    page_size: int = 0
    seed: int = 0
    layer: int = 0
    stream_id: int = 0
    stream_ids: Optional[torch.Tensor] = None
    use_witness: bool = True

    def to_c(self, need_v: bool = True) -> Region:
        st = self.stored
        exf = 0
        if self.k_exact is not None:
            exf = {torch.bfloat16: FMT["bf16"], torch.float32: FMT["fp32"]}[self.k_exact.dtype]
        return Region(k_format=FMT[st.fmt_k], v_format=FMT[st.fmt_v], k=_ptr(st.k),
                      v=_ptr(st.v) if need_v else None, k_scale=_ptr(st.k_scale),
                      v_scale=_ptr(st.v_scale) if need_v else None,
                      witness=_ptr(st.witness) if self.use_witness else None,
                      k_exact=_ptr(self.k_exact), k_exact_format=exf, length=self.length,
                      lengths=_ptr(self.lengths), page_table=_ptr(self.page_table),
                      page_size=self.page_size,
                      max_pages=self.page_table.shape[1] if self.page_table is not None else 0,
                      seed=self.seed, layer=self.layer, stream_id=self.stream_id,
                      stream_ids=_ptr(self.stream_ids), v_witness=_ptr(st.v_witness),
                      outlier_pairs=_ptr(st.outlier_pairs), k_outliers=_ptr(st.k_outliers),
                      n_outlier_pairs=st.n_outlier_pairs)


def _attn_args(q, prefix: Optional[RegionView], suffix: Optional[RegionView], out, sm_scale,
               split_tokens, num_kv_heads, need_v=True, plan_flags: int = 0, status=None) -> AttnArgs:
    batch, hq, d = q.shape
    return AttnArgs(batch=batch, num_q_heads=hq, num_kv_heads=num_kv_heads, head_dim=d,
                    sm_scale=sm_scale, split_tokens=split_tokens, plan_flags=plan_flags,
                    status=status if isinstance(status, int) else _ptr(status), q=_ptr(q),
                    prefix=prefix.to_c(need_v) if prefix else Region(),
                    suffix=suffix.to_c(need_v) if suffix else Region(), out=_ptr(out))


def workspace_bytes(args: AttnArgs, meter: MeterOut) -> int:
    return int(load().kvq_workspace_bytes(ctypes.byref(args), ctypes.byref(meter)))


class Workspace:
    """Device scratch for kvq_decode_attn / kvq_meter (grown on demand), with
    the status word the calls that use it report to (int32 [4], word 0)."""

    def __init__(self, device):
        self.device = device
        self.buf: Optional[torch.Tensor] = None
        self.status = torch.zeros(4, dtype=torch.int32, device=device)

    def read_status(self) -> int:
        """The status bits reported so far (synchronizes with the device)."""
        return int(self.status[0].item())

    def get(self, nbytes: int, stream=None) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            _check(load().kvq_workspace_init(self.buf.data_ptr(), self.buf.numel(), _stream(stream)),
                   "kvq_workspace_init")
        return self.buf


METER_KEYS = ("tv", "bound_raw", "meter", "log_a")
TIER_B_KEYS = ("log_a_b", "bound_b_raw", "meter_b")
VALUE_KEYS = ("value_err", "v_norm_max", "out_bound")
TWO_SIDED_KEYS = ("log_a_minus", "bound_two_sided", "meter_two_sided", "bound_tanh")
REPORT_KEYS = ("block_mass", "block_excess", "block_order")
INT8_BLOCK_TOKENS = 256


def n_report_blocks(prefix: Optional["RegionView"], suffix: Optional["RegionView"]) -> int:
    """Blocks of the risk report: 256-token blocks per region, prefix first."""
    return sum(-(-r.length // INT8_BLOCK_TOKENS) for r in (prefix, suffix) if r is not None)


def _meter_keys(meter, tier_b_delta, value_bound, two_sided, report):
    if not meter:
        return ()
    keys = METER_KEYS
    keys += TIER_B_KEYS if tier_b_delta is not None else ()
    keys += VALUE_KEYS if value_bound else ()
    keys += TWO_SIDED_KEYS if two_sided else ()
    keys += REPORT_KEYS + (("block_excess_b",) if tier_b_delta is not None else ()) if report else ()
    return keys


def plan(q: torch.Tensor, num_kv_heads: int, prefix: Optional[RegionView],
         suffix: Optional[RegionView], *, sm_scale: float, split_tokens: int = 0,
         meter: bool = True, meter_only: bool = False, tier_b_delta: Optional[float] = None,
         value_bound: bool = False, two_sided: bool = False, report: bool = False,
         plan_flags: int = 0, with_status: bool = True) -> dict:
    """kvq_decode_plan for the arguments decode_attn would pass (host only;
    the output, meter and status pointers only need to be non-NULL and
    aligned)."""
    dummy = _ptr(q) if meter else None
    keys = _meter_keys(meter, tier_b_delta, value_bound, two_sided, report)
    m = MeterOut(**{k: dummy for k in keys}, delta_b=tier_b_delta or 0.0)
    args = _attn_args(q, prefix, suffix, None if meter_only else q, sm_scale, split_tokens,
                      num_kv_heads, need_v=not meter_only, plan_flags=plan_flags,
                      status=_ptr(q) if with_status else None)
    info = PlanInfo()
    _check(load().kvq_decode_plan(ctypes.byref(args), ctypes.byref(m), int(meter_only), ctypes.byref(info)),
           "kvq_decode_plan")
    return {name: int(getattr(info, name)) for name, _ in PlanInfo._fields_}


def decode_attn(q: torch.Tensor, num_kv_heads: int, prefix: Optional[RegionView],
                suffix: Optional[RegionView], *, sm_scale: float, split_tokens: int = 0,
                meter: bool = True, workspace: Optional[Workspace] = None, out=None,
                meter_bufs=None, stream=None, meter_only: bool = False,
                tier_b_delta: Optional[float] = None, value_bound: bool = False,
                two_sided: bool = False, report: bool = False, plan_flags: int = 0,
                status: Optional[torch.Tensor] = None, lib: Optional[ctypes.CDLL] = None):
    """kvq_decode_attn (or kvq_meter when meter_only).  Returns (out, dict of
    meter tensors); tier_b_delta adds the Tier B outputs with that failure
    probability, value_bound the value term and the joint output bound,
    two_sided the two-sided form of the meter, report the per-block risk
    report ([batch, num_q_heads, n_blocks] arrays).  The call reports to
    `status` (int32 device tensor), else to the workspace's status word.
    plan_flags: KVQ_PLAN_* bits.  lib: another build of the library (tests)."""
    lib = lib or load()
    batch, hq, d = q.shape
    if out is None and not meter_only:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    if meter_bufs is None:
        nb = n_report_blocks(prefix, suffix)
        meter_bufs = {}
        for k in _meter_keys(meter, tier_b_delta, value_bound, two_sided, report):
            if k.startswith("block_"):
                meter_bufs[k] = torch.empty((batch, hq, nb), device=q.device,
                                            dtype=torch.int32 if k == "block_order" else torch.float32)
            else:
                meter_bufs[k] = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    m = MeterOut(**{k: _ptr(v) for k, v in meter_bufs.items()}, delta_b=tier_b_delta or 0.0)
    workspace = workspace or Workspace(q.device)
    if status is None:
        status = workspace.status
    args = _attn_args(q, prefix, suffix, None if meter_only else out, sm_scale, split_tokens,
                      num_kv_heads, need_v=not meter_only, plan_flags=plan_flags, status=status)
    nbytes = int(lib.kvq_workspace_bytes(ctypes.byref(args), ctypes.byref(m)))
    if nbytes == 0:
        raise KvqError(2, "kvq_workspace_bytes (invalid arguments)")
    ws = workspace.get(nbytes, stream)
    fn = lib.kvq_meter if meter_only else lib.kvq_decode_attn
    _check(fn(ctypes.byref(args), ctypes.byref(m), ws.data_ptr(), ws.numel(), _stream(stream)),
           "kvq_meter" if meter_only else "kvq_decode_attn")
    return out, meter_bufs


def decode_attn_noalloc(q: torch.Tensor, num_kv_heads: int, prefix: Optional[RegionView],
                        suffix: Optional[RegionView], *, sm_scale: float, out: torch.Tensor,
                        meter_bufs: dict, status: torch.Tensor, split_tokens: int = 0,
                        plan_flags: int = 0, tier_b_delta: Optional[float] = None, stream=None) -> None:
    """kvq_decode_attn_noalloc: the decode call on the library's static scratch.
    The caller brings every output buffer and the status word (this function
    allocates nothing either); raises KvqError(6) when the plan needs more than
    SCRATCH_BYTES."""
    lib = load()
    m = MeterOut(**{k: _ptr(v) for k, v in meter_bufs.items()}, delta_b=tier_b_delta or 0.0)
    args = _attn_args(q, prefix, suffix, out, sm_scale, split_tokens, num_kv_heads,
                      plan_flags=plan_flags, status=status)
    _check(lib.kvq_decode_attn_noalloc(ctypes.byref(args), ctypes.byref(m), _stream(stream)),
           "kvq_decode_attn_noalloc")
