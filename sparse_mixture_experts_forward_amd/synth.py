"""Seeded synthetic inputs for the MoE layer, reproducible bit for bit on CPU and GPU.

This module holds no arithmetic of the layer itself: it only draws numbers.  Both the
HIP path (through torch tensors on the GPU) and the CPU oracle (through numpy arrays)
take their inputs from here, so the two can be compared on identical data.  The
largest weight sets (17 GB for the decode workload) are drawn on the GPU; the oracle
redraws only the experts it needs, on the CPU, and gets the same bits.

Generator (counter based, same definition in numpy and in torch):
  * hash      lowbias32 (from Chris Wellons' hash-prospector):
                x ^= x >> 16; x *= 0x7feb352d; x ^= x >> 15; x *= 0x846ca68b; x ^= x >> 16
              over uint32, multiplication modulo 2**32;
  * stream    key = chain of lowbias32 over (seed, workload id, tensor id, expert id);
  * element i of a tensor uses the four words  h_r = lowbias32(i ^ lowbias32(key + r)),
              r = 0..3;
  * normal    the eight 16-bit halves of h_0..h_3 are summed (Irwin-Hall of 8 discrete
              uniforms, bell-shaped, support +-4.9 sigma); D = 2*S - 8*65535 is an exact
              integer, and the value is float32(D) * float32(std / (2 sigma_S)), one IEEE
              multiplication, so CPU and GPU round it identically;
  * uniform   U(-a, a): float32(2*(h_0 >> 9) - (2**23 - 1)) * float32(a / 2**23);
  * bf16      round-to-nearest-even of the float32 value.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .configs import MoEConfig

MASK32 = 0xFFFFFFFF
_M1 = 0x7FEB352D
_M2 = 0x846CA68B

# tensor ids of the streams
T_X, T_ROUTER, T_LOGIT_BIAS, T_W1, T_W3, T_W2, T_B1, T_B2, T_SW1, T_SW3, T_SW2 = range(1, 12)

_SIGMA8 = math.sqrt(8.0 * (65536.0 ** 2 - 1.0) / 12.0)


def _h32(x: int) -> int:
    x &= MASK32
    x ^= x >> 16
    x = (x * _M1) & MASK32
    x ^= x >> 15
    x = (x * _M2) & MASK32
    x ^= x >> 16
    return x


def stream_key(seed: int, cfg_id: int, tensor_id: int, index: int = 0) -> int:
    k = _h32(seed + 0x9E3779B9)
    k = _h32(k ^ cfg_id)
    k = _h32(k ^ tensor_id)
    k = _h32(k ^ index)
    return k


def _normal_scale(std: float) -> np.float32:
    return np.float32(std / (2.0 * _SIGMA8))


# ---------------------------------------------------------------- numpy (CPU) side
def _np_h32(x: np.ndarray) -> np.ndarray:
    x = x ^ (x >> np.uint32(16))
    x = x * np.uint32(_M1)
    x = x ^ (x >> np.uint32(15))
    x = x * np.uint32(_M2)
    x = x ^ (x >> np.uint32(16))
    return x


def normal_np(key: int, n: int, std: float, start: int = 0) -> np.ndarray:
    """Elements start .. start+n-1 of the normal stream `key`, float32."""
    i = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)
    s = np.zeros(n, dtype=np.int64)
    for r in range(4):
        h = _np_h32(i ^ np.uint32(_h32(key + r)))
        s += (h & np.uint32(0xFFFF)).astype(np.int64) + (h >> np.uint32(16)).astype(np.int64)
    d = 2 * s - 8 * 65535
    return d.astype(np.float32) * _normal_scale(std)


def uniform_np(key: int, n: int, half_width: float) -> np.ndarray:
    i = np.arange(n, dtype=np.uint32)
    h = _np_h32(i ^ np.uint32(_h32(key)))
    d = 2 * (h >> np.uint32(9)).astype(np.int64) - (2 ** 23 - 1)
    return d.astype(np.float32) * np.float32(half_width / 2.0 ** 23)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- torch side
def _t_mul32(x, c: int):
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & MASK32


def _t_h32(x):
    x = x ^ (x >> 16)
    x = _t_mul32(x, _M1)
    x = x ^ (x >> 15)
    x = _t_mul32(x, _M2)
    x = x ^ (x >> 16)
    return x


def normal_torch(key: int, n: int, std: float, device, start: int = 0, chunk: int = 1 << 25):
    """Same values as normal_np, computed with torch int64 ops on `device`."""
    import torch

    out = torch.empty(n, dtype=torch.float32, device=device)
    scale = torch.tensor(float(_normal_scale(std)), dtype=torch.float32, device=device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        i = torch.arange(start + c0, start + c1, dtype=torch.int64, device=device) & MASK32
        s = torch.zeros(c1 - c0, dtype=torch.int64, device=device)
        for r in range(4):
            h = _t_h32(i ^ _h32(key + r))
            s += (h & 0xFFFF) + (h >> 16)
        d = 2 * s - 8 * 65535
        out[c0:c1] = d.to(torch.float32) * scale
    return out


def uniform_torch(key: int, n: int, half_width: float, device):
    import torch

    i = torch.arange(n, dtype=torch.int64, device=device)
    h = _t_h32(i ^ _h32(key))
    d = 2 * (h >> 9) - (2 ** 23 - 1)
    scale = torch.tensor(float(np.float32(half_width / 2.0 ** 23)), dtype=torch.float32,
                         device=device)
    return d.to(torch.float32) * scale


# ---------------------------------------------------------------- workload tensors
def _std(fan_in: int) -> float:
    return 1.0 / math.sqrt(fan_in)


def logit_bias_np(cfg: MoEConfig, seed: int = 0) -> Optional[np.ndarray]:
    if cfg.logit_bias == "none":
        return None
    if cfg.logit_bias == "skew4":
        b = np.zeros(cfg.n_experts, dtype=np.float32)
        b[:4] = 2.0
        return b
    if cfg.logit_bias == "uniform0.1":
        return uniform_np(stream_key(seed, cfg.cfg_id, T_LOGIT_BIAS), cfg.n_experts, 0.1)
    if cfg.logit_bias == "skew0":  # +4.0 on expert 0: nearly every token picks it
        b = np.zeros(cfg.n_experts, dtype=np.float32)
        b[0] = 4.0
        return b
    raise ValueError(cfg.logit_bias)


def _maybe_bf16_np(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


class HostInputs:
    """Numpy view of a workload's inputs.  Expert weights are drawn on demand, one
    expert at a time (bf16 as uint16 bit patterns, f32 as float32)."""

    def __init__(self, cfg: MoEConfig, seed: int = 0):
        self.cfg, self.seed = cfg, seed
        c = cfg
        x = normal_np(stream_key(seed, c.cfg_id, T_X), c.n_tokens * c.d_model, 1.0)
        self.x = _maybe_bf16_np(x, c.dtype).reshape(c.n_tokens, c.d_model)
        self.w_router = normal_np(stream_key(seed, c.cfg_id, T_ROUTER),
                                  c.d_model * c.n_experts, _std(c.d_model)
                                  ).reshape(c.d_model, c.n_experts)
        self.logit_bias = logit_bias_np(c, seed)

    def _mat(self, tid: int, e: int, rows: int, cols: int, fan_in: int) -> np.ndarray:
        a = normal_np(stream_key(self.seed, self.cfg.cfg_id, tid, e), rows * cols, _std(fan_in))
        return _maybe_bf16_np(a, self.cfg.dtype).reshape(rows, cols)

    def expert(self, e: int, shared: bool = False) -> dict:
        c = self.cfg
        t1, t3, t2 = (T_SW1, T_SW3, T_SW2) if shared else (T_W1, T_W3, T_W2)
        w = {"w1": self._mat(t1, e, c.d_ff, c.d_model, c.d_model),
             "w2": self._mat(t2, e, c.d_model, c.d_ff, c.d_ff)}
        if c.act == "swiglu":
            w["w3"] = self._mat(t3, e, c.d_ff, c.d_model, c.d_model)
        if c.expert_bias and not shared:
            w["b1"] = self._mat(T_B1, e, 1, c.d_ff, c.d_model).reshape(-1)
            w["b2"] = self._mat(T_B2, e, 1, c.d_model, c.d_ff).reshape(-1)
        return w


class DeviceInputs:
    """Torch tensors of a workload's inputs on `device` (bf16 tensors for bf16
    workloads), drawn with the same generator as HostInputs."""

    def __init__(self, cfg: MoEConfig, device, seed: int = 0):
        import torch

        self.cfg, self.seed, self.device = cfg, seed, device
        c = cfg
        tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        self.tdtype = tdt
        self.x = normal_torch(stream_key(seed, c.cfg_id, T_X), c.n_tokens * c.d_model, 1.0,
                              device).to(tdt).reshape(c.n_tokens, c.d_model)
        self.w_router = normal_torch(stream_key(seed, c.cfg_id, T_ROUTER),
                                     c.d_model * c.n_experts, _std(c.d_model), device
                                     ).reshape(c.d_model, c.n_experts)
        lb = logit_bias_np(c, seed)
        self.logit_bias = None if lb is None else torch.from_numpy(lb).to(device)

        def stack(tid, n_e, rows, cols, fan_in):
            t = torch.empty((n_e, rows, cols), dtype=tdt, device=device)
            for e in range(n_e):
                t[e] = normal_torch(stream_key(seed, c.cfg_id, tid, e), rows * cols,
                                    _std(fan_in), device).to(tdt).reshape(rows, cols)
            return t

        E, S = c.n_experts, c.n_shared
        self.w1 = stack(T_W1, E, c.d_ff, c.d_model, c.d_model)
        self.w2 = stack(T_W2, E, c.d_model, c.d_ff, c.d_ff)
        self.w3 = stack(T_W3, E, c.d_ff, c.d_model, c.d_model) if c.act == "swiglu" else None
        if c.expert_bias:
            self.b1 = stack(T_B1, E, 1, c.d_ff, c.d_model).reshape(E, c.d_ff)
            self.b2 = stack(T_B2, E, 1, c.d_model, c.d_ff).reshape(E, c.d_model)
        else:
            self.b1 = self.b2 = None
        if S > 0:
            self.sw1 = stack(T_SW1, S, c.d_ff, c.d_model, c.d_model)
            self.sw2 = stack(T_SW2, S, c.d_model, c.d_ff, c.d_ff)
            self.sw3 = stack(T_SW3, S, c.d_ff, c.d_model, c.d_model) if c.act == "swiglu" else None
        else:
            self.sw1 = self.sw2 = self.sw3 = None


def torch_bf16_from_bits(bits: np.ndarray, device):
    """Upload uint16 bf16 patterns as a torch.bfloat16 tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bits_from_torch_bf16(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(__import__("torch").int16).numpy().view(np.uint16)
