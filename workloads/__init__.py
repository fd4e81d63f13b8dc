"""Seeded synthetic inputs for the selective-scan workloads, and the error metric.

This module is shared by the oracle side and the HIP side of every test and
benchmark.  It holds input recipes only (shapes, distributions, seeds) and the
comparison metric; none of the scan's arithmetic lives here.

Recipe (the five workloads; every tensor is synthetic, no dataset or weights):
  * x, z, B, C, raw delta ~ N(0, 1);
  * delta_bias[d] = softplus^-1(u) = log(expm1(u)), u log-uniform on [1e-3, 1e-1],
    so softplus(raw + bias) starts around u;
  * A[d, n] = -(n + 1) (the S4D-real diagonal of the Mamba block, page
    youngju.dev section 3.4: A = -exp(A_log), A_log = log(1..N));
  * D = 1, or D ~ N(1, 0.1) where noted; h0 = 0, or ~ N(0, 0.1) for decode;
  * bf16 tensors are fp32 draws rounded to nearest-even by torch.
Seeds: numpy PCG64 seeded from SeedSequence([20261203, workload_index, *extra]),
one spawned stream per tensor in the fixed order x, delta, B, C, z, u, D, h0.
Inputs of several GiB per tensor (make_large_inputs) are drawn by torch's CPU
generator, seeded from the same SeedSequence, in blocks of tokens.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

ROOT_SEED = 20261203


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: torch.dtype
    gate: bool
    d_noise: bool          # D ~ N(1, 0.1) instead of ones
    final_state: bool      # the workload asks for hT
    chunks: int = 1        # run as `chunks` calls passing the state along
    steps: int = 0         # decode: number of successive L=1 steps (0 = not decode)
    h0_std: float = 0.0    # decode: initial state ~ N(0, h0_std)

    @property
    def elems(self) -> int:
        """B*L*D*N scan elements of the whole workload."""
        L = self.steps if self.steps else self.seqlen
        return self.batch * L * self.dim * self.dstate

    def describe(self) -> str:
        return (f"{self.name}: B={self.batch} L={self.seqlen} D={self.dim} N={self.dstate} "
                f"{str(self.dtype).replace('torch.', '')} gate={self.gate}"
                + (f" chunks={self.chunks}" if self.chunks > 1 else "")
                + (f" steps={self.steps}" if self.steps else ""))


WORKLOADS = [
    Workload(0, "tiny_fp32_B1_L256_D64_N16", 1, 256, 64, 16, torch.float32,
             gate=False, d_noise=False, final_state=True),
    Workload(1, "mamba130m_B8_L2048_D1536_N16", 8, 2048, 1536, 16, torch.bfloat16,
             gate=True, d_noise=False, final_state=True),
    Workload(2, "mamba1p4b_B4_L8192_D4096_N16", 4, 8192, 4096, 16, torch.bfloat16,
             gate=True, d_noise=True, final_state=True),
    Workload(3, "longctx_B1_L262144_D1536_N16", 1, 262144, 1536, 16, torch.bfloat16,
             gate=True, d_noise=False, final_state=True, chunks=32),
    Workload(4, "decode_B256_D5120_N16_x128", 256, 1, 5120, 16, torch.bfloat16,
             gate=True, d_noise=True, final_state=True, steps=128, h0_std=0.1),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def _streams(index: int, extra=()):
    ss = np.random.SeedSequence([ROOT_SEED, int(index), *[int(e) for e in extra]])
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(8)]


def _cast(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)


def make_params(w: Workload, dim: int | None = None, dstate: int | None = None, *,
                seed_extra=()):
    """Per-channel parameters: A (D,N), D (D), delta_bias (D), all fp32."""
    dim = dim or w.dim
    N = dstate or w.dstate
    g = _streams(w.index, seed_extra)
    u = np.exp(g[5].uniform(math.log(1e-3), math.log(1e-1), size=dim))
    bias = np.log(np.expm1(u))
    A = -np.tile(np.arange(1, N + 1, dtype=np.float64), (dim, 1))
    Dsk = g[6].normal(1.0, 0.1, size=dim) if w.d_noise else np.ones(dim)
    return {
        "A": torch.from_numpy(A.astype(np.float32)),
        "D": torch.from_numpy(Dsk.astype(np.float32)),
        "delta_bias": torch.from_numpy(bias.astype(np.float32)),
    }


def make_inputs(w: Workload, *, batch: int | None = None, seqlen: int | None = None,
                dim: int | None = None, dstate: int | None = None, seed_extra=()):
    """Seeded CPU tensors for one call of the workload (optionally resized).

    Returns a dict with x, delta, B, C, z (or None), A, D, delta_bias, h0 (or None).
    """
    bsz = batch or w.batch
    L = seqlen or (1 if w.steps else w.seqlen)
    dim = dim or w.dim
    N = dstate or w.dstate
    g = _streams(w.index, seed_extra)
    f32 = np.float32
    x = g[0].standard_normal((bsz, L, dim), dtype=f32)
    delta = g[1].standard_normal((bsz, L, dim), dtype=f32)
    Bm = g[2].standard_normal((bsz, L, N), dtype=f32)
    Cm = g[3].standard_normal((bsz, L, N), dtype=f32)
    z = g[4].standard_normal((bsz, L, dim), dtype=f32) if w.gate else None
    h0 = None
    if w.h0_std > 0:
        h0 = torch.from_numpy((g[7].standard_normal((bsz, dim, N)) * w.h0_std).astype(f32))
    out = {
        "x": _cast(x, w.dtype), "delta": _cast(delta, w.dtype),
        "B": _cast(Bm, w.dtype), "C": _cast(Cm, w.dtype),
        "z": _cast(z, w.dtype) if z is not None else None,
        "h0": h0,
    }
    out.update(make_params(w, dim, N, seed_extra=seed_extra))
    return out


def make_large_inputs(w: Workload, *, batch: int, seqlen: int, dim: int, seed_extra=(), rows_per_draw=8192):
    """Seeded inputs too large for make_inputs' numpy fp32 intermediates (rows
    of several GiB): the same distributions, drawn rows_per_draw tokens at a time
    by torch's CPU generator (seeded from the workload's SeedSequence, one
    generator per tensor) straight into tensors of the workload's dtype.
    x, delta, z ~ N(0, 1) (z only for gated workloads), B, C ~ N(0, 1), no h0;
    A, D, delta_bias from make_params."""
    N = w.dstate
    ss = np.random.SeedSequence([ROOT_SEED, int(w.index), *[int(e) for e in seed_extra], 1])
    seeds = [int(c.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1)) for c in ss.spawn(5)]
    gens = [torch.Generator().manual_seed(sd) for sd in seeds]

    def draw(i, shape):
        return torch.randn(shape, generator=gens[i], dtype=torch.float32).to(w.dtype)

    out = {"x": torch.empty((batch, seqlen, dim), dtype=w.dtype),
           "delta": torch.empty((batch, seqlen, dim), dtype=w.dtype),
           "z": torch.empty((batch, seqlen, dim), dtype=w.dtype) if w.gate else None,
           "B": draw(2, (batch, seqlen, N)), "C": draw(3, (batch, seqlen, N)), "h0": None}
    for key, i in (("x", 0), ("delta", 1), ("z", 4)):
        if out[key] is None:
            continue
        for b in range(batch):
            for t0 in range(0, seqlen, rows_per_draw):
                rows = min(rows_per_draw, seqlen - t0)
                out[key][b, t0:t0 + rows] = draw(i, (rows, dim))
    out.update(make_params(w, dim, N, seed_extra=seed_extra))
    return out


def make_large_cotangents(w: Workload, *, batch: int, seqlen: int, dim: int, seed_extra=(), rows_per_draw=8192):
    """make_cotangents' recipe (dy, dhT ~ N(0, 1)) for inputs of several GiB, drawn
    like make_large_inputs by torch's CPU generator in blocks of tokens."""
    ss = np.random.SeedSequence([ROOT_SEED, int(w.index), 2000, *[int(e) for e in seed_extra], 1])
    gens = [torch.Generator().manual_seed(int(c.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1)))
            for c in ss.spawn(2)]
    dy = torch.empty((batch, seqlen, dim), dtype=w.dtype)
    for b in range(batch):
        for t0 in range(0, seqlen, rows_per_draw):
            rows = min(rows_per_draw, seqlen - t0)
            dy[b, t0:t0 + rows] = torch.randn((rows, dim), generator=gens[0], dtype=torch.float32).to(w.dtype)
    return {"dy": dy, "dhT": torch.randn((batch, dim, w.dstate), generator=gens[1], dtype=torch.float32)}


def make_decode_step(w: Workload, step: int, *, batch: int | None = None, dim: int | None = None):
    """Fresh per-step tensors (x, delta, B, C, z) of a decode workload, L = 1."""
    bsz = batch or w.batch
    dim = dim or w.dim
    N = w.dstate
    g = _streams(w.index, (1000 + int(step),))
    f32 = np.float32
    return {
        "x": _cast(g[0].standard_normal((bsz, 1, dim), dtype=f32), w.dtype),
        "delta": _cast(g[1].standard_normal((bsz, 1, dim), dtype=f32), w.dtype),
        "B": _cast(g[2].standard_normal((bsz, 1, N), dtype=f32), w.dtype),
        "C": _cast(g[3].standard_normal((bsz, 1, N), dtype=f32), w.dtype),
        "z": _cast(g[4].standard_normal((bsz, 1, dim), dtype=f32), w.dtype) if w.gate else None,
    }


def make_cotangents(w: Workload, *, batch: int | None = None, seqlen: int | None = None,
                    dim: int | None = None, dstate: int | None = None, seed_extra=()):
    """Seeded upstream gradients for a backward call: dy (B, L, D) in the
    workload's dtype and dhT (B, D, N) fp32, both N(0, 1)."""
    bsz = batch or w.batch
    L = seqlen if seqlen is not None else (1 if w.steps else w.seqlen)
    dim = dim or w.dim
    N = dstate or w.dstate
    g = _streams(w.index, (2000, *seed_extra))
    f32 = np.float32
    return {
        "dy": _cast(g[0].standard_normal((bsz, L, dim), dtype=f32), w.dtype),
        "dhT": torch.from_numpy(g[1].standard_normal((bsz, dim, N), dtype=f32)),
    }


def make_conv_params(w: Workload, dim: int | None = None, width: int = 4, seed_extra=()):
    """Taps (D, W) and bias (D) of the conv1d prologue, fp32, drawn like PyTorch's
    Conv1d initialisation for a depthwise layer: uniform on +-1/sqrt(W)."""
    dim = dim or w.dim
    g = _streams(w.index, (3000, *seed_extra))
    bound = 1.0 / math.sqrt(width)
    return {
        "weight": torch.from_numpy(g[0].uniform(-bound, bound, size=(dim, width)).astype(np.float32)),
        "bias": torch.from_numpy(g[1].uniform(-bound, bound, size=dim).astype(np.float32)),
    }


@dataclasses.dataclass(frozen=True)
class SsdWorkload:
    """A Mamba-2 state-space dual layer: x (B, L, H, P), B/C (B, L, G, N)."""
    index: int
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int

    @property
    def elems(self) -> int:
        """B*L*H*P*N state updates of the whole workload."""
        return self.batch * self.seqlen * self.nheads * self.headdim * self.dstate

    def describe(self) -> str:
        return (f"{self.name}: B={self.batch} L={self.seqlen} H={self.nheads} P={self.headdim} "
                f"G={self.ngroups} N={self.dstate} bf16")


# The page's Mamba-2 layer (d_model 2048, expand 2, headdim 64, d_state 128:
# 64 heads, one B/C group) at the token count of the 1.4B-shaped scan layer,
# and a small case for element-wise parity.
SSD_WORKLOADS = [
    SsdWorkload(100, "ssd_small_B2_L200_H4_P64_G2_N64", 2, 200, 4, 64, 2, 64),
    SsdWorkload(101, "mamba2_B4_L8192_H64_P64_N128", 4, 8192, 64, 64, 1, 128),
    # one long sequence: 64 (b, h) pairs for 256 compute units, the time-split case
    SsdWorkload(102, "mamba2_longctx_B1_L32768_H64_P64_N128", 1, 32768, 64, 64, 1, 128),
]
SSD_BY_NAME = {w.name: w for w in SSD_WORKLOADS}


def make_ssd_inputs(w: SsdWorkload, *, batch=None, seqlen=None, nheads=None, ngroups=None, dstate=None,
                    with_h0=False, seed_extra=()):
    """Seeded CPU tensors of one SSD call: x, dt, B, C bf16 ~ N(0, 1); A[h] = -U(1, 16)
    (the Mamba-2 initialisation A = -exp(A_log), A_log = log U(1, 16)); dt_bias the
    inverse softplus of log-uniform [1e-3, 1e-1] steps; D = 1; h0 ~ N(0, 0.1) or None."""
    bsz = batch or w.batch
    L = seqlen if seqlen is not None else w.seqlen
    H = nheads or w.nheads
    G = ngroups or w.ngroups
    N = dstate or w.dstate
    P = w.headdim
    g = _streams(w.index, seed_extra)
    f32 = np.float32
    bf = torch.bfloat16
    u = np.exp(g[5].uniform(math.log(1e-3), math.log(1e-1), size=H))
    return {
        "x": _cast(g[0].standard_normal((bsz, L, H, P), dtype=f32), bf),
        "dt": _cast(g[1].standard_normal((bsz, L, H), dtype=f32), bf),
        "A": torch.from_numpy(-g[4].uniform(1.0, 16.0, size=H).astype(f32)),
        "B": _cast(g[2].standard_normal((bsz, L, G, N), dtype=f32), bf),
        "C": _cast(g[3].standard_normal((bsz, L, G, N), dtype=f32), bf),
        "D": torch.ones(H, dtype=torch.float32),
        "dt_bias": torch.from_numpy(np.log(np.expm1(u)).astype(f32)),
        "h0": torch.from_numpy((g[6].standard_normal((bsz, H, P, N)) * 0.1).astype(f32)) if with_h0 else None,
    }


@dataclasses.dataclass(frozen=True)
class GlaWorkload:
    """A gated-linear-attention / mLSTM layer: v (B, L, H, P), q/k (B, L, G, N),
    per-token forget and input gates (gated) or none (plain linear attention),
    optionally the elu + 1 feature map on q and k."""
    index: int
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    gated: bool
    feature_map: bool

    @property
    def elems(self) -> int:
        """B*L*H*P*N state updates of the whole workload."""
        return self.batch * self.seqlen * self.nheads * self.headdim * self.dstate

    def describe(self) -> str:
        kind = "gated (forget/input gates)" if self.gated else "ungated linear attention"
        fm = ", elu+1 feature map" if self.feature_map else ""
        return (f"{self.name}: B={self.batch} L={self.seqlen} H={self.nheads} P={self.headdim} "
                f"G={self.ngroups} N={self.dstate} bf16, {kind}{fm}")


# An mLSTM-style gated layer at the token count and head layout of the Mamba-2
# workload (64 heads, values of 64, keys/queries of 128 shared by one group), the
# same with plain linear attention and the elu + 1 feature map, and small cases.
GLA_WORKLOADS = [
    GlaWorkload(110, "gla_small_B2_L200_H4_P64_G2_N64", 2, 200, 4, 64, 2, 64, True, False),
    GlaWorkload(111, "mlstm_B4_L8192_H64_P64_N128", 4, 8192, 64, 64, 1, 128, True, False),
    GlaWorkload(112, "linattn_elu_B4_L8192_H64_P64_N128", 4, 8192, 64, 64, 1, 128, False, True),
    GlaWorkload(113, "mlstm_longctx_B1_L32768_H64_P64_N128", 1, 32768, 64, 64, 1, 128, True, False),
]
GLA_BY_NAME = {w.name: w for w in GLA_WORKLOADS}


def make_gla_inputs(w: GlaWorkload, *, batch=None, seqlen=None, nheads=None, ngroups=None, dstate=None,
                    gated=None, with_h0=False, seed_extra=()):
    """Seeded CPU tensors of one call: q, v bf16 ~ N(0, 1); k bf16 ~ N(0, 1/N) (keys
    scaled by N^-1/2); gated: log_f = log sigmoid(u), u ~ N(3, 1) (forget gates
    near 0.95) and in_gate = sigmoid(N(0, 1)), both fp32, else None; h0 fp32
    ~ N(0, 0.1) or None."""
    bsz = batch or w.batch
    L = seqlen if seqlen is not None else w.seqlen
    H = nheads or w.nheads
    G = ngroups or w.ngroups
    N = dstate or w.dstate
    P = w.headdim
    gated = w.gated if gated is None else gated
    g = _streams(w.index, seed_extra)
    f32 = np.float32
    bf = torch.bfloat16
    sig = lambda a: 1.0 / (1.0 + np.exp(-a))
    return {
        "q": _cast(g[0].standard_normal((bsz, L, G, N), dtype=f32), bf),
        "k": _cast(g[1].standard_normal((bsz, L, G, N), dtype=f32) / math.sqrt(N), bf),
        "v": _cast(g[2].standard_normal((bsz, L, H, P), dtype=f32), bf),
        "log_f": torch.from_numpy(np.log(sig(g[3].normal(3.0, 1.0, (bsz, L, H)))).astype(f32)) if gated else None,
        "in_gate": torch.from_numpy(sig(g[4].standard_normal((bsz, L, H))).astype(f32)) if gated else None,
        "h0": torch.from_numpy((g[5].standard_normal((bsz, H, P, N)) * 0.1).astype(f32)) if with_h0 else None,
    }


def tolerance(dtype: torch.dtype) -> float:
    """Max floored relative error allowed: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs."""
    return 1e-4 if dtype == torch.float32 else 2e-2


def rel_err(got, ref) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)): relative error floored at the RMS of the
    reference so that entries near zero do not blow it up."""
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    if r.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms if rms > 0 else 1e-300)
    e = np.abs(g - r) / den
    if not np.all(np.isfinite(g)):
        return math.inf
    return float(np.max(e))
