"""ctypes binding of libmoe_ternary.so (argument marshalling only).

Every step of the block runs in the library's HIP kernels; this module only
turns numpy arrays and torch device tensors into the pointers and sizes the C
ABI takes (include/moe_ternary.h), and raises MoeError on a non-zero status.
PyTorch provides device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

PQ2_0 = 142
PTQ1_0 = 143

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ternary.so")

_ERRORS = {
    -1: "MOE_E_ARG", -2: "MOE_E_FORMAT", -3: "MOE_E_SHAPE", -4: "MOE_E_CODE",
    -5: "MOE_E_NONFINITE", -6: "MOE_E_SPACE", -7: "MOE_E_DEVICE",
}

EXPORTS = [
    "moe_block_bytes", "moe_packed_bytes", "moe_pack", "moe_unpack", "moe_unpack_device",
    "moe_quantize_device", "moe_ple_gather_q4_0", "moe_ternary_forward_q", "moe_draft_head_workspace_bytes",
    "moe_draft_head", "moe_lowrank_workspace_bytes", "moe_lowrank_apply",
    "moe_workspace_bytes_factored", "moe_ternary_forward_factored",
    "moe_tile_container", "moe_untile_container", "moe_workspace_bytes", "moe_ternary_forward", "moe_route_workspace_bytes", "moe_route",
    "moe_route_workspace_bytes_factored", "moe_route_factored", "moe_ternary_forward_noalloc",
    "moe_set_stage_events", "moe_last_error",
]
N_STAGES = 5
STAGES = ["xproj", "routing", "gate_up", "down", "combine"]


class MoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_ERRORS.get(code, code)}: {message}")
        self.code = code
        self.name = _ERRORS.get(code, str(code))


class ExpertBanksC(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("banks", ctypes.c_void_p), ("banks_bytes", ctypes.c_int64),
        ("offsets", ctypes.c_void_p), ("formats", ctypes.c_void_p),
        ("offsets_host", ctypes.c_void_p), ("formats_host", ctypes.c_void_p),
        ("layout", ctypes.c_int32),
    ]


BANKS_ROW_MAJOR, BANKS_TILE_MAJOR = 1, 2


_lib = None


def lib():
    """Load the library; fails loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: run `python -m ternary_quantized_moe_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        sig = {
            "moe_block_bytes": (i64, [i32]),
            "moe_packed_bytes": (i64, [i32, i64]),
            "moe_pack": (i32, [i32, vp, vp, i64, vp, i64]),
            "moe_unpack": (i32, [i32, vp, i64, vp, vp, i64]),
            "moe_unpack_device": (i32, [i32, vp, i64, vp, vp, vp]),
            "moe_quantize_device": (i32, [i32, i32, vp, i64, vp, vp, vp]),
            "moe_ple_gather_q4_0": (i32, [vp, i64, i32, vp, i64, vp, vp]),
            "moe_ternary_forward_q": (i32, [vp, i64, vp, vp, ctypes.POINTER(ExpertBanksC), vp, vp, i32,
                                            i32, vp, vp, i64, vp]),
            "moe_draft_head_workspace_bytes": (i64, [i64, i32, i32]),
            "moe_draft_head": (i32, [vp, vp, i64, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp]),
            "moe_lowrank_workspace_bytes": (i64, [i64, i32, i32]),
            "moe_lowrank_apply": (i32, [vp, vp, i64, i32, vp, vp, vp, vp, i32, vp, vp, i64, vp]),
            "moe_workspace_bytes_factored": (i64, [ctypes.POINTER(ExpertBanksC), i64, i32, i32, i32]),
            "moe_ternary_forward_factored": (i32, [vp, i64, vp, vp, vp, i32, ctypes.POINTER(ExpertBanksC), vp, vp,
                                                   i32, i32, vp, vp, i64, vp]),
            "moe_tile_container": (i32, [i32, vp, i64, i64, vp, i64]),
            "moe_untile_container": (i32, [i32, vp, i64, i64, vp, i64]),
            "moe_workspace_bytes": (i64, [ctypes.POINTER(ExpertBanksC), i64, i32, i32]),
            "moe_ternary_forward": (i32, [vp, i64, vp, vp, ctypes.POINTER(ExpertBanksC), vp, vp, i32,
                                          i32, vp, vp, i64, vp]),
            "moe_route_workspace_bytes": (i64, [i64, i32, i32, i32]),
            "moe_route": (i32, [vp, i64, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp]),
            "moe_route_workspace_bytes_factored": (i64, [i64, i32, i32, i32, i32]),
            "moe_route_factored": (i32, [vp, i64, i32, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64,
                                         vp]),
            "moe_ternary_forward_noalloc": (i32, [vp, i64, vp, vp, ctypes.POINTER(ExpertBanksC), vp, vp, i32, i32,
                                                  vp, vp]),
            "moe_set_stage_events": (i32, [ctypes.POINTER(ctypes.c_void_p), i32]),
            "moe_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise MoeError(rc, lib().moe_last_error().decode())


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _dev_ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    """The HIP stream handle: the given torch stream's, else torch's current
    stream on the current device (read through torch's C binding where it has
    one, which costs less per call than building a Stream object)."""
    import torch
    if stream is not None:
        return stream.cuda_stream
    try:
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
    except AttributeError:
        return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------ host codec
def block_bytes(fmt: int) -> int:
    return lib().moe_block_bytes(fmt)


def packed_bytes(fmt: int, n_weights: int) -> int:
    return lib().moe_packed_bytes(fmt, n_weights)


def pack(fmt: int, trits: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    trits = np.ascontiguousarray(trits, dtype=np.int8).reshape(-1)
    scale_bits = np.ascontiguousarray(scale_bits, dtype=np.uint16).reshape(-1)
    n = trits.size
    nbytes = lib().moe_packed_bytes(fmt, n)
    if nbytes < 0:
        # let the library produce the error message
        _check(lib().moe_pack(fmt, _np_ptr(trits), _np_ptr(scale_bits), n, None, 0))
    if scale_bits.size != n // 128:
        raise MoeError(-1, f"need {n // 128} scales, got {scale_bits.size}")
    out = np.empty(nbytes, dtype=np.uint8)
    _check(lib().moe_pack(fmt, _np_ptr(trits), _np_ptr(scale_bits), n, _np_ptr(out), nbytes))
    return out


def unpack(fmt: int, data: np.ndarray, n_weights: int):
    data = np.ascontiguousarray(data, dtype=np.uint8).reshape(-1)
    trits = np.empty(n_weights, dtype=np.int8)
    scales = np.empty(max(n_weights // 128, 1), dtype=np.uint16)
    _check(lib().moe_unpack(fmt, _np_ptr(data), data.size, _np_ptr(trits), _np_ptr(scales), n_weights))
    return trits, scales[: n_weights // 128]


def tile_container(fmt: int, data: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Row-major container -> the tile-major block order the expert kernels read."""
    data = np.ascontiguousarray(data, dtype=np.uint8).reshape(-1)
    out = np.empty(data.size, dtype=np.uint8)
    _check(lib().moe_tile_container(fmt, _np_ptr(data), rows, cols, _np_ptr(out), out.size))
    return out


def untile_container(fmt: int, data: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Inverse of tile_container."""
    data = np.ascontiguousarray(data, dtype=np.uint8).reshape(-1)
    out = np.empty(data.size, dtype=np.uint8)
    _check(lib().moe_untile_container(fmt, _np_ptr(data), rows, cols, _np_ptr(out), out.size))
    return out


# ------------------------------------------------------------------ device
def unpack_device(fmt: int, d_src, n_weights: int, stream=None):
    import torch
    trits = torch.empty(n_weights, dtype=torch.int8, device=d_src.device)
    scales = torch.empty(max(n_weights // 128, 1), dtype=torch.int16, device=d_src.device)
    _check(lib().moe_unpack_device(fmt, _dev_ptr(d_src), n_weights, _dev_ptr(trits), _dev_ptr(scales),
                                   _stream(stream)))
    return trits, scales[: n_weights // 128]


QUANT_ABSMEAN = 0
QUANT_LLOYD = 1


def quantize_device(fmt: int, method: int, d_w, out=None, rounds=None, stream=None):
    """bfloat16 weights (a contiguous device tensor, size a multiple of 128;
    bf16 or int16 bit patterns) -> container bytes (uint8 device tensor).
    rounds: None, or a uint8 device tensor of n/128 entries that receives the
    Lloyd rounds per group."""
    import torch
    n = d_w.numel()
    nbytes = lib().moe_packed_bytes(fmt, n)
    if nbytes < 0:
        _check(lib().moe_quantize_device(fmt, method, None, n, None, None, _stream(stream)))
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=d_w.device)
    elif out.numel() < nbytes:
        raise MoeError(-6, f"out holds {out.numel()} bytes, {nbytes} needed")
    if rounds is not None and rounds.numel() < n // 128:
        raise MoeError(-6, f"rounds holds {rounds.numel()} entries, {n // 128} needed")
    _check(lib().moe_quantize_device(fmt, method, _dev_ptr(d_w), n, _dev_ptr(out), _dev_ptr(rounds),
                                     _stream(stream)))
    return out[:nbytes]


def ple_gather(d_table, n_rows: int, row_len: int, d_idx, out=None, stream=None):
    """Rows d_idx (int64 device tensor) of a Q4_0 table (uint8 device tensor of
    n_rows rows of row_len values) -> fp32 device tensor [len(d_idx), row_len]."""
    import torch
    n = d_idx.numel()
    if out is None:
        out = torch.empty((n, row_len), dtype=torch.float32, device=d_idx.device)
    elif out.numel() < n * row_len:
        raise MoeError(-6, f"out holds {out.numel()} values, {n * row_len} needed")
    _check(lib().moe_ple_gather_q4_0(_dev_ptr(d_table), n_rows, row_len, _dev_ptr(d_idx), n, _dev_ptr(out),
                                     _stream(stream)))
    return out


class ExpertBanks:
    """One layer's expert containers in device memory plus the host copies the
    library validates against.  `data` is the concatenation of every bank's
    [gate | up | down] containers, each in the tile-major block order of
    tile_container (layers.build_banks writes that order); bank e starts at
    offsets[e]."""

    def __init__(self, data: np.ndarray, offsets: np.ndarray, formats: np.ndarray, d_model: int,
                 d_ff: int, n_experts: int, n_shared: int, device="cuda"):
        import torch
        self.d_model, self.d_ff, self.n_experts, self.n_shared = d_model, d_ff, n_experts, n_shared
        self.offsets_host = np.ascontiguousarray(offsets, dtype=np.int64)
        self.formats_host = np.ascontiguousarray(formats, dtype=np.uint8)
        self.data = torch.from_numpy(np.ascontiguousarray(data, dtype=np.uint8)).to(device)
        self.offsets = torch.from_numpy(self.offsets_host).to(device)
        self.formats = torch.from_numpy(self.formats_host).to(device)
        self.nbytes = int(data.size)
        self._c = ExpertBanksC(d_model, d_ff, n_experts, n_shared, self.data.data_ptr(), self.nbytes,
                               self.offsets.data_ptr(), self.formats.data_ptr(),
                               self.offsets_host.ctypes.data, self.formats_host.ctypes.data, BANKS_TILE_MAJOR)

    @classmethod
    def from_tensors(cls, data_dev, offsets_host, formats_host, d_model, d_ff, n_experts, n_shared):
        """Wrap a device byte tensor that already holds the containers."""
        import torch
        self = cls.__new__(cls)
        self.d_model, self.d_ff, self.n_experts, self.n_shared = d_model, d_ff, n_experts, n_shared
        self.offsets_host = np.ascontiguousarray(offsets_host, dtype=np.int64)
        self.formats_host = np.ascontiguousarray(formats_host, dtype=np.uint8)
        self.data = data_dev
        self.offsets = torch.from_numpy(self.offsets_host).to(data_dev.device)
        self.formats = torch.from_numpy(self.formats_host).to(data_dev.device)
        self.nbytes = int(data_dev.numel())
        self._c = ExpertBanksC(d_model, d_ff, n_experts, n_shared, data_dev.data_ptr(), self.nbytes,
                               self.offsets.data_ptr(), self.formats.data_ptr(),
                               self.offsets_host.ctypes.data, self.formats_host.ctypes.data, BANKS_TILE_MAJOR)
        return self

    @property
    def c(self):
        return ctypes.byref(self._c)


def workspace_bytes(banks: ExpertBanks, n_tokens: int, top_k: int, corr_rank: int) -> int:
    return lib().moe_workspace_bytes(banks.c, n_tokens, top_k, corr_rank)


def alloc_workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256) + 256, dtype=torch.uint8, device=device)


def _aligned(ws):
    p = ws.data_ptr()
    off = (-p) % 256
    return p + off, ws.numel() - off


def forward(x, router, router_delta, banks: ExpertBanks, corr_a, corr_b, top_k: int, y=None,
            workspace=None, stream=None):
    """x: bf16 [T, d] (torch.bfloat16 or int16 bits) on the GPU; returns y (same dtype as x)."""
    import torch
    T = x.shape[0]
    r = 0 if corr_a is None else corr_a.shape[0]
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        need = workspace_bytes(banks, T, top_k, r)
        if need < 0:
            raise MoeError(-1, "invalid arguments for the workspace size")
        workspace = alloc_workspace(need, x.device)
    wp, wn = _aligned(workspace)
    _check(lib().moe_ternary_forward(_dev_ptr(x), T, _dev_ptr(router), _dev_ptr(router_delta), banks.c,
                                     _dev_ptr(corr_a), _dev_ptr(corr_b), r, top_k, _dev_ptr(y), wp, wn,
                                     _stream(stream)))
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_noalloc(x, router, router_delta, banks: ExpertBanks, corr_a, corr_b, top_k: int, y, stream=None):
    """forward() with the library's own scratch as workspace (nothing is
    allocated, by the library or here: the caller passes y).  Calls that overlap
    on one GPU share that scratch and race."""
    T = x.shape[0]
    r = 0 if corr_a is None else corr_a.shape[0]
    _check(lib().moe_ternary_forward_noalloc(_dev_ptr(x), T, _dev_ptr(router), _dev_ptr(router_delta), banks.c,
                                             _dev_ptr(corr_a), _dev_ptr(corr_b), r, top_k, _dev_ptr(y),
                                             _stream(stream)))
    return y


def forward_q(x, router, router_delta_q, banks: ExpertBanks, corr_a_q, corr_b_q, corr_rank: int, top_k: int,
              y=None, workspace=None, stream=None):
    """forward() with the router delta and the correction given as ternary PQ2_0
    containers (uint8 device tensors in moe_pack's row-major order, or None)."""
    import torch
    T = x.shape[0]
    r = 0 if corr_a_q is None else corr_rank
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        need = workspace_bytes(banks, T, top_k, r)
        if need < 0:
            raise MoeError(-1, "invalid arguments for the workspace size")
        workspace = alloc_workspace(need, x.device)
    wp, wn = _aligned(workspace)
    _check(lib().moe_ternary_forward_q(_dev_ptr(x), T, _dev_ptr(router), _dev_ptr(router_delta_q), banks.c,
                                       _dev_ptr(corr_a_q), _dev_ptr(corr_b_q), r, top_k, _dev_ptr(y), wp, wn,
                                       _stream(stream)))
    return y


def forward_factored(x, router, delta_u, delta_v, banks: ExpertBanks, corr_a, corr_b, top_k: int, y=None,
                     workspace=None, stream=None):
    """forward() with the router delta as fp16 factors U [E, rd] and V [rd, d]."""
    import torch
    T = x.shape[0]
    rd = delta_u.shape[1]
    r = 0 if corr_a is None else corr_a.shape[0]
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        need = lib().moe_workspace_bytes_factored(banks.c, T, top_k, r, rd)
        if need < 0:
            raise MoeError(-1, "invalid arguments for the workspace size")
        workspace = alloc_workspace(need, x.device)
    wp, wn = _aligned(workspace)
    _check(lib().moe_ternary_forward_factored(_dev_ptr(x), T, _dev_ptr(router), _dev_ptr(delta_u), _dev_ptr(delta_v),
                                              rd, banks.c, _dev_ptr(corr_a), _dev_ptr(corr_b), r, top_k,
                                              _dev_ptr(y), wp, wn, _stream(stream)))
    return y


def draft_head(hidden, emb, w1, b1, w2, b2, y=None, workspace=None, stream=None):
    """The k=1 draft head: bf16 hidden and emb [T, h] (bf16 or int16 bits),
    fp16 w1 [m, 2h], w2 [h, m], optional fp16 biases -> y [T, h]."""
    T, h = hidden.shape
    m = w1.shape[0]
    if y is None:
        import torch
        y = torch.empty_like(hidden)
    if workspace is None:
        need = lib().moe_draft_head_workspace_bytes(T, h, m)
        if need < 0:
            raise MoeError(-3, f"invalid draft head shape T={T} h={h} m={m}")
        workspace = alloc_workspace(need, hidden.device)
    wp, wn = _aligned(workspace)
    _check(lib().moe_draft_head(_dev_ptr(hidden), _dev_ptr(emb), T, h, m, _dev_ptr(w1), _dev_ptr(b1), _dev_ptr(w2),
                                _dev_ptr(b2), _dev_ptr(y), wp, wn, _stream(stream)))
    return y


def lowrank_apply(x, y_in, a, b, rank: int, a_q=None, b_q=None, y=None, workspace=None, stream=None):
    """y = y_in + B (A x): x, y_in bf16 [T, d] (y_in may be None, y may be y_in);
    A fp16 [r, d] or a_q its PQ2_0 container, B fp16 [d, r] or b_q."""
    import torch
    T, d = x.shape
    if y is None:
        y = torch.empty_like(x)
    if workspace is None:
        need = lib().moe_lowrank_workspace_bytes(T, d, rank)
        if need < 0:
            raise MoeError(-3, f"invalid low-rank shape T={T} d={d} r={rank}")
        workspace = alloc_workspace(need, x.device)
    wp, wn = _aligned(workspace)
    _check(lib().moe_lowrank_apply(_dev_ptr(x), _dev_ptr(y_in), T, d, _dev_ptr(a), _dev_ptr(a_q), _dev_ptr(b),
                                   _dev_ptr(b_q), rank, _dev_ptr(y), wp, wn, _stream(stream)))
    return y


def _route_outputs(T, n_experts, top_k, dev):
    import torch
    return dict(
        logits=torch.empty((T, n_experts), dtype=torch.float32, device=dev),
        idx=torch.empty((T, top_k), dtype=torch.int32, device=dev),
        w=torch.empty((T, top_k), dtype=torch.float32, device=dev),
        counts=torch.empty(n_experts, dtype=torch.int32, device=dev),
        offsets=torch.empty(n_experts + 1, dtype=torch.int32, device=dev),
        perm=torch.empty(max(T * top_k, 1), dtype=torch.int32, device=dev),
    )


def route_factored(x, router, delta_u, delta_v, n_experts: int, top_k: int, workspace=None, stream=None):
    """Routing half of forward_factored (router delta as fp16 factors U [E, rd],
    V [rd, d]); returns the same dict as route()."""
    T, d = x.shape
    rd = delta_u.shape[1]
    out = _route_outputs(T, n_experts, top_k, x.device)
    if workspace is None:
        need = lib().moe_route_workspace_bytes_factored(T, d, n_experts, top_k, rd)
        if need < 0:
            raise MoeError(-1, "invalid arguments for the routing workspace size")
        workspace = alloc_workspace(need, x.device)
    wp, wn = _aligned(workspace)
    _check(lib().moe_route_factored(_dev_ptr(x), T, d, n_experts, _dev_ptr(router), _dev_ptr(delta_u),
                                    _dev_ptr(delta_v), rd, top_k, _dev_ptr(out["logits"]), _dev_ptr(out["idx"]),
                                    _dev_ptr(out["w"]), _dev_ptr(out["counts"]), _dev_ptr(out["offsets"]),
                                    _dev_ptr(out["perm"]), wp, wn, _stream(stream)))
    out["perm"] = out["perm"][: T * top_k]
    return out


def route(x, router, router_delta, n_experts: int, top_k: int, workspace=None, stream=None):
    """Routing half of the block; returns dict of device tensors
    (logits, idx, w, counts, offsets, perm)."""
    import torch
    T, d = x.shape
    dev = x.device
    out = dict(
        logits=torch.empty((T, n_experts), dtype=torch.float32, device=dev),
        idx=torch.empty((T, top_k), dtype=torch.int32, device=dev),
        w=torch.empty((T, top_k), dtype=torch.float32, device=dev),
        counts=torch.empty(n_experts, dtype=torch.int32, device=dev),
        offsets=torch.empty(n_experts + 1, dtype=torch.int32, device=dev),
        perm=torch.empty(max(T * top_k, 1), dtype=torch.int32, device=dev),
    )
    if workspace is None:
        need = lib().moe_route_workspace_bytes(T, d, n_experts, top_k)
        if need < 0:
            raise MoeError(-1, "invalid arguments for the routing workspace size")
        workspace = alloc_workspace(need, dev)
    wp, wn = _aligned(workspace)
    _check(lib().moe_route(_dev_ptr(x), T, d, n_experts, _dev_ptr(router), _dev_ptr(router_delta), top_k,
                           _dev_ptr(out["logits"]), _dev_ptr(out["idx"]), _dev_ptr(out["w"]),
                           _dev_ptr(out["counts"]), _dev_ptr(out["offsets"]), _dev_ptr(out["perm"]),
                           wp, wn, _stream(stream)))
    out["perm"] = out["perm"][: T * top_k]
    return out


class StageTimer:
    """Per-stage device time of forward calls, from the library's stage events.

    Create once, then `with timer.step():` around each forward call; events are
    recorded on the call's stream.  `ms()` synchronises and returns the mean
    duration per stage over the recorded steps."""

    def __init__(self, n_steps: int, stages=None):
        """stages: indices of the stages to time (default: all); the others
        record nothing, which keeps the timed stream free of extra markers."""
        import torch
        self.stages = list(range(N_STAGES)) if stages is None else list(stages)
        self._ev = [[torch.cuda.Event(enable_timing=True) if (i // 2) in self.stages else None
                     for i in range(2 * N_STAGES)] for _ in range(n_steps)]
        for evs in self._ev:          # torch creates the HIP event on first record
            for e in evs:
                if e is not None:
                    e.record()
        torch.cuda.synchronize()
        self._arr = [(ctypes.c_void_p * (2 * N_STAGES))(*[e.cuda_event if e is not None else None for e in evs])
                     for evs in self._ev]
        self._i = 0

    def step(self):
        timer = self

        class _Ctx:
            def __enter__(self_inner):
                _check(lib().moe_set_stage_events(timer._arr[timer._i], 2 * N_STAGES))

            def __exit__(self_inner, *exc):
                _check(lib().moe_set_stage_events(None, 0))
                timer._i += 1
        return _Ctx()

    def ms(self):
        import torch
        torch.cuda.synchronize()
        out = np.full(N_STAGES, np.nan)
        for s in self.stages:
            out[s] = sum(evs[2 * s].elapsed_time(evs[2 * s + 1]) for evs in self._ev[: self._i])
        return out / max(self._i, 1)
