"""ctypes front end of the CPU oracle (``moe_oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It converts host
torch tensors to pointers and calls the plain fp64 C++ loops; it does no
arithmetic of its own beyond allocating outputs.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

ODT = {torch.float32: 0, torch.bfloat16: 1, torch.float64: 2}
SCORE = {"softmax": 0, "sigmoid": 1}

_P = ctypes.c_void_p
_I = ctypes.c_int
_LL = ctypes.c_longlong


def lib():
    global _LIB
    if _LIB is None:
        # ORACLE_LIBRARY: an alternative build of moe_oracle.cpp (the mutation
        # test points the pins at deliberately broken copies).
        path = os.environ.get("ORACLE_LIBRARY") or _build.library_path()
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        sig = {
            "oracle_num_threads": (_I, []),
            "oracle_set_threads": (None, [_I]),
            "oracle_router_logits": (None, [_I, _I, _I, _I, _P, _P, _P, _P]),
            "oracle_topk": (None, [_I, _I, _I, _I, _P, _I, _I, _P, _P]),
            "oracle_route": (None, [_I, _I, _I, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P]),
            "oracle_dispatch": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _LL]),
            "oracle_expert_mlp": (None, [_I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P]),
            "oracle_combine_tokens": (None, [_I, _P, _I, _I, _I, _I, _P, _P, _I, _P, _I, _P, _P]),
            "oracle_combine": (None, [_I, _I, _I, _I, _P, _P, _I, _P, _I, _P, _P]),
            "oracle_forward": (_I, [_I] * 11 + [_P] * 13),
            "oracle_split_point": (_I, [_I, _I]),
            "oracle_forward_split": (None, [_I] * 11 + [_P] * 9 + [_I, _P]),
            "oracle_forward_split_at": (None, [_I] * 11 + [_P] * 9 + [_I, _P]),
            "oracle_dbo_split": (_I, [_I] * 6),
            "oracle_round_bf16": (None, [_LL, _P, _P]),
            "oracle_e4m3_encode": (ctypes.c_uint8, [ctypes.c_double]),
            "oracle_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "oracle_mxfp8_quantize": (None, [_I, _I, _I, _P, _LL, _P, _P]),
            "oracle_mxfp8_dequantize": (None, [_I, _I, _P, _P, _P]),
            "oracle_forward_mxfp8": (_I, [_I] * 11 + [_P] * 9 + [_I] + [_P] * 4),
            "oracle_expert_mlp_mxfp8": (None, [_I] * 5 + [_P] * 5 + [_I, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.device.type == "cpu" and t.is_contiguous(), "oracle takes contiguous host tensors"
    return ctypes.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    return ODT[t.dtype]


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def router_logits(x, w_router, bias=None) -> torch.Tensor:
    T, d = x.shape
    E = w_router.shape[0]
    assert w_router.dtype == x.dtype
    z = torch.empty(T, E, dtype=torch.float64)
    lib().oracle_router_logits(T, d, E, _dt(x), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(z))
    return z


def topk(logits, K: int, score: str, renorm: bool):
    T, E = logits.shape
    ids = torch.empty(T, K, dtype=torch.int32)
    w = torch.empty(T, K, dtype=torch.float64)
    lib().oracle_topk(T, E, K, _dt(logits), _ptr(logits), SCORE[score], int(renorm),
                      _ptr(ids), _ptr(w))
    return ids, w


def route(x, w_router, bias, K: int, score: str, renorm: bool):
    T, d = x.shape
    E = w_router.shape[0]
    ids = torch.empty(T, K, dtype=torch.int32)
    w = torch.empty(T, K, dtype=torch.float64)
    z = torch.empty(T, E, dtype=torch.float64)
    lib().oracle_route(T, d, E, K, _dt(x), _ptr(x), _ptr(w_router), _ptr(bias), SCORE[score],
                       int(renorm), _ptr(ids), _ptr(w), _ptr(z))
    return ids, w, z


def dispatch(ids, E: int, e_begin: int, e_end: int, x=None):
    """Returns dict(counts, offsets, src_index, row_of, n_invalid, n_rows[, x_sorted])."""
    T, K = ids.shape
    ids = ids.to(torch.int32).contiguous()
    counts = torch.empty(E, dtype=torch.int32)
    offsets = torch.empty(e_end - e_begin + 1, dtype=torch.int32)
    src = torch.full((T * K,), -1, dtype=torch.int32)
    row_of = torch.empty(T * K, dtype=torch.int32)
    bad = torch.zeros(1, dtype=torch.int32)
    xs = None
    rb = 0
    if x is not None:
        xs = torch.zeros(T * K, x.shape[1], dtype=x.dtype)
        rb = x.shape[1] * x.element_size()
    n = lib().oracle_dispatch(T, E, K, e_begin, e_end, _ptr(ids), _ptr(counts), _ptr(offsets),
                              _ptr(src), _ptr(row_of), _ptr(bad), _ptr(x), _ptr(xs), rb)
    out = dict(counts=counts, offsets=offsets, src_index=src[:n].clone(), row_of=row_of,
               n_invalid=int(bad.item()), n_rows=int(n))
    if xs is not None:
        out["x_sorted"] = xs[:n].clone()
    return out


def expert_mlp(x_rows, row_expert, w_gate, w_up, w_down) -> torch.Tensor:
    """y [n, d] fp64 for rows x_rows [n, d]; row r uses expert row_expert[r]."""
    n, d = x_rows.shape
    I = w_gate.shape[1]
    y = torch.empty(n, d, dtype=torch.float64)
    if n == 0:
        return y
    re = row_expert.to(torch.int32).contiguous()
    assert w_gate.dtype == w_up.dtype == w_down.dtype
    lib().oracle_expert_mlp(n, d, I, _dt(x_rows), _ptr(x_rows.contiguous()), _ptr(re),
                            _dt(w_gate), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y))
    return y


def combine(y_sorted, row_of, weights, T: int, K: int, y_shared=None,
            tokens: Optional[Sequence[int]] = None) -> torch.Tensor:
    d = y_sorted.shape[1]
    n_sh = 0 if y_shared is None else y_shared.shape[0]
    if y_shared is not None:
        assert y_shared.dtype == y_sorted.dtype
    row_of = row_of.to(torch.int32).contiguous()
    weights = weights.contiguous()
    if tokens is None:
        out = torch.empty(T, d, dtype=torch.float64)
        lib().oracle_combine(T, d, K, _dt(y_sorted), _ptr(y_sorted), _ptr(row_of),
                             _dt(weights), _ptr(weights), n_sh, _ptr(y_shared), _ptr(out))
        return out
    tok = torch.as_tensor(list(tokens), dtype=torch.int32)
    out = torch.empty(len(tok), d, dtype=torch.float64)
    lib().oracle_combine_tokens(len(tok), _ptr(tok), T, d, K, _dt(y_sorted), _ptr(y_sorted),
                                _ptr(row_of), _dt(weights), _ptr(weights), n_sh,
                                _ptr(y_shared), _ptr(out))
    return out


def forward(cfg, inp: dict, x=None):
    """Whole layer, fp64 out [T,d], ids [T,K], weights [T,K] fp64, counts [E]."""
    x = inp["x"] if x is None else x
    T, d = x.shape
    K, E = cfg.top_k, cfg.num_experts
    out = torch.empty(T, d, dtype=torch.float64)
    ids = torch.empty(T, K, dtype=torch.int32)
    w = torch.empty(T, K, dtype=torch.float64)
    counts = torch.empty(E, dtype=torch.int32)
    lib().oracle_forward(T, d, E, K, cfg.intermediate, cfg.expert_begin, cfg.expert_end,
                         cfg.num_shared, SCORE[cfg.score], int(cfg.renormalize), _dt(x),
                         _ptr(x), _ptr(inp["w_router"]), _ptr(inp["bias"]), _ptr(inp["w_gate"]),
                         _ptr(inp["w_up"]), _ptr(inp["w_down"]), _ptr(inp.get("ws_gate")),
                         _ptr(inp.get("ws_up")), _ptr(inp.get("ws_down")), _ptr(out), _ptr(ids),
                         _ptr(w), _ptr(counts))
    return out, ids, w, counts


def expert_mlp_mxfp8(x_rows, row_expert, w_gate, w_up, w_down, down: bool = False):
    """y [n, d] fp64 of the block-scaled expert MLP on rows x_rows [n, d]
    (row r uses expert row_expert[r] of the stacks)."""
    n, d = x_rows.shape
    n_exp, I = w_gate.shape[0], w_gate.shape[1]
    y = torch.empty(n, d, dtype=torch.float64)
    if n == 0:
        return y
    assert x_rows.dtype == w_gate.dtype == w_up.dtype == w_down.dtype
    lib().oracle_expert_mlp_mxfp8(n, d, I, n_exp, _dt(x_rows), _ptr(x_rows.contiguous()),
                                  _ptr(row_expert.to(torch.int32).contiguous()),
                                  _ptr(w_gate.contiguous()), _ptr(w_up.contiguous()),
                                  _ptr(w_down.contiguous()), int(down), _ptr(y))
    return y


def forward_mxfp8(cfg, inp: dict, down: bool = False):
    """Whole layer with the MX-FP8 payload: the dispatched rows (and, for the
    shared experts, the tokens) and the gate / up weights decoded from their
    MX-FP8 encodings (with down=True also h and the down weights); returns
    like forward."""
    x = inp["x"]
    T, d = x.shape
    K, E = cfg.top_k, cfg.num_experts
    assert d % 32 == 0
    out = torch.empty(T, d, dtype=torch.float64)
    ids = torch.empty(T, K, dtype=torch.int32)
    w = torch.empty(T, K, dtype=torch.float64)
    counts = torch.empty(E, dtype=torch.int32)
    S = cfg.num_shared
    sh = lambda k: _ptr(inp.get(k)) if S > 0 else None
    lib().oracle_forward_mxfp8(T, d, E, K, cfg.intermediate, cfg.expert_begin, cfg.expert_end, S,
                               SCORE[cfg.score], int(cfg.renormalize), _dt(x), _ptr(x),
                               _ptr(inp["w_router"]), _ptr(inp["bias"]), _ptr(inp["w_gate"]),
                               _ptr(inp["w_up"]), _ptr(inp["w_down"]), sh("ws_gate"),
                               sh("ws_up"), sh("ws_down"), int(down), _ptr(out), _ptr(ids),
                               _ptr(w), _ptr(counts))
    return out, ids, w, counts


def split_point(T: int, pad: int = 256) -> int:
    return int(lib().oracle_split_point(T, pad))


def dbo_split(T: int, has_prefill: bool, decode_threshold: int, prefill_threshold: int,
              query_len: int = 1, pad: int = 256) -> int:
    return int(lib().oracle_dbo_split(T, int(has_prefill), decode_threshold, prefill_threshold,
                                      query_len, pad))


def forward_split_at(cfg, inp: dict, split: int) -> torch.Tensor:
    x = inp["x"]
    T, d = x.shape
    out = torch.empty(T, d, dtype=torch.float64)
    lib().oracle_forward_split_at(T, d, cfg.num_experts, cfg.top_k, cfg.intermediate,
                                  cfg.expert_begin, cfg.expert_end, cfg.num_shared,
                                  SCORE[cfg.score], int(cfg.renormalize), _dt(x), _ptr(x),
                                  _ptr(inp["w_router"]), _ptr(inp["bias"]), _ptr(inp["w_gate"]),
                                  _ptr(inp["w_up"]), _ptr(inp["w_down"]),
                                  _ptr(inp.get("ws_gate")), _ptr(inp.get("ws_up")),
                                  _ptr(inp.get("ws_down")), int(split), _ptr(out))
    return out


def forward_split(cfg, inp: dict, pad: int = 256) -> torch.Tensor:
    x = inp["x"]
    T, d = x.shape
    out = torch.empty(T, d, dtype=torch.float64)
    lib().oracle_forward_split(T, d, cfg.num_experts, cfg.top_k, cfg.intermediate,
                               cfg.expert_begin, cfg.expert_end, cfg.num_shared,
                               SCORE[cfg.score], int(cfg.renormalize), _dt(x), _ptr(x),
                               _ptr(inp["w_router"]), _ptr(inp["bias"]), _ptr(inp["w_gate"]),
                               _ptr(inp["w_up"]), _ptr(inp["w_down"]), _ptr(inp.get("ws_gate")),
                               _ptr(inp.get("ws_up")), _ptr(inp.get("ws_down")), pad, _ptr(out))
    return out


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(int(code)))


def mxfp8_quantize(x: torch.Tensor):
    """Rows of x (bf16 / fp32 / fp64) -> (E4M3 codes [rows, cols] uint8,
    scale bytes [rows, cols/32] uint8)."""
    x = x.contiguous()
    rows, cols = x.shape
    assert cols % 32 == 0
    codes = torch.empty(rows, cols, dtype=torch.uint8)
    scales = torch.empty(rows, cols // 32, dtype=torch.uint8)
    lib().oracle_mxfp8_quantize(rows, cols, _dt(x), _ptr(x), cols, _ptr(codes), _ptr(scales))
    return codes, scales


def mxfp8_dequantize(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    codes, scales = codes.contiguous(), scales.contiguous()
    rows, cols = codes.shape
    out = torch.empty(rows, cols, dtype=torch.float64)
    lib().oracle_mxfp8_dequantize(rows, cols, _ptr(codes), _ptr(scales), _ptr(out))
    return out


def round_bf16(v: torch.Tensor) -> torch.Tensor:
    """fp64 -> bf16, round to nearest even, directly (no fp32 step)."""
    v = v.to(torch.float64).contiguous()
    out = torch.empty(v.shape, dtype=torch.int16)
    lib().oracle_round_bf16(v.numel(), _ptr(v), _ptr(out))
    return out.view(torch.bfloat16)
