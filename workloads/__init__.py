"""Seeded synthetic inputs for the KDA state-update path.

This module only draws inputs: random tensors with the distributions, shapes,
slot layouts and length mixes of the five workloads below. It contains none of
the method's arithmetic (no decay, no normalisation of keys at use, no
recurrence), so both sides of a parity test (the FP64 oracle and the GPU
library) can take their inputs from it.

Distributions (sigma is the standard deviation):

* state ~ N(0, 0.1), every slot including the null slot and unused slots;
* keys: x ~ N(0, 1)^128 scaled to unit L2 norm per (token, head) in FP32, then
  rounded to BF16; q = BF16(N(0, 1) * 128^-0.5); v, raw_g, raw_beta = BF16(N(0, 1));
* A_log ~ N(0, 0.5), dt_bias ~ N(0, 0.1) (FP32), lower bound -5, null slot 0;
* records: corrections ~ N(0, 0.5) FP32; key/gate = unit keys as above, then
  raw gates BF16(N(0, 1));
* for the key-normalisation edge cases, keys rescaled per vector to a norm
  drawn from KEY_NORMS (0, 1e-4, 1e-2, 1, 30).

BF16 rounding is round-to-nearest-even (torch's FP32 -> BF16 conversion).
Everything is drawn from ``torch.Generator`` objects seeded per workload; the
big state pools can be drawn directly on a GPU device (a device generator,
seeded the same way) so that multi-GiB pools do not pass through the host.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

K = 128
V = 128
LOWER_BOUND = -5.0
NULL_SLOT = 0


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(gen: torch.Generator, shape, std=1.0, device="cpu") -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32, device=device) * std


def unit_keys(gen: torch.Generator, shape) -> torch.Tensor:
    """N(0,1) vectors over the last axis scaled to unit norm in FP32 (a draw
    recipe: the keys' distribution is uniform on the sphere)."""
    x = normal(gen, shape)
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


def bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def bits(x: torch.Tensor) -> np.ndarray:
    """A BF16 tensor's bit patterns as a uint16 numpy array (host copy)."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Window:
    """One verify window of T tokens for B requests and H heads:
    q, k, raw_g [B*T, H, K], v [B*T, H, V], raw_beta [B*T, H], all BF16."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    raw_g: torch.Tensor
    raw_beta: torch.Tensor

    def to(self, device):
        return Window(*(t.to(device) for t in (self.q, self.k, self.v, self.raw_g, self.raw_beta)))


def draw_window(gen, B: int, T: int, H: int) -> Window:
    n = B * T
    k = bf16(unit_keys(gen, (n, H, K)))
    q = bf16(normal(gen, (n, H, K)) * (K ** -0.5))
    v = bf16(normal(gen, (n, H, V)))
    raw_g = bf16(normal(gen, (n, H, K)))
    raw_beta = bf16(normal(gen, (n, H)))
    return Window(q, k, v, raw_g, raw_beta)


@dataclass
class ConvInputs:
    """Inputs of the convolution prologue for B requests of T tokens and H heads:

    * x [B*T, pitch] BF16: a packed projection row per token whose columns
      [0, 3HK) are the q | k | v pre-activations (HK = H*128 channels each); the
      rest of the row holds the projection's other outputs and is drawn too;
    * weight [3, 4, HK] BF16 (part, tap, channel), tap 3 meeting the current
      token; bias [3*HK] BF16;
    * window pool [slots, 3*HK, W] BF16, W = RQ + 2 values per channel.
    """
    x: torch.Tensor
    weight: torch.Tensor
    bias: torch.Tensor
    window: torch.Tensor

    @property
    def pitch(self) -> int:
        return self.x.shape[1]


def draw_conv_inputs(gen, B: int, T: int, H: int, RQ: int, slots: int) -> ConvInputs:
    """x = BF16(N(0, 1)); weight = BF16(N(0, 0.5)); bias = BF16(N(0, 0.1));
    every window value = BF16(N(0, 1)). pitch = 4HK + 128 + H rounded up to a
    multiple of 8 (16-byte rows)."""
    hk = H * K
    pitch = (4 * hk + 128 + H + 7) // 8 * 8
    x = bf16(normal(gen, (B * T, pitch)))
    weight = bf16(normal(gen, (3, 4, hk), 0.5))
    bias = bf16(normal(gen, (3 * hk,), 0.1))
    window = bf16(normal(gen, (slots, 3 * hk, RQ + 2)))
    return ConvInputs(x, weight, bias, window)


def draw_gate_factors(gen, N: int, H: int, exact: bool = True, rank: int = 128):
    """Factors of the low-rank gate projection raw_g = F_A F_B^T: F_A [N, rank]
    and F_B [H*128, rank], BF16.

    exact (default): values on a grid, F_A = m * 2^-6 and F_B = m' * 2^-7 with
    m, m' = round(N(0, 24)) clipped to [-127, 127]. Every product and every
    partial sum of a row is then an integer multiple of 2^-13 below 2^21 * 2^-13,
    so an FP32 accumulation is exact in any order and raw_g's BF16 rounding is
    the same decision on every implementation; raw_g ~ N(0, 0.8).
    Otherwise F_A = BF16(N(0, 1)), F_B = BF16(N(0, 1) / sqrt(rank))."""
    if exact:
        ma = torch.clamp(torch.round(normal(gen, (N, rank), 24.0)), -127, 127)
        mb = torch.clamp(torch.round(normal(gen, (H * K, rank), 24.0)), -127, 127)
        return bf16(ma * 2.0 ** -6), bf16(mb * 2.0 ** -7)
    return bf16(normal(gen, (N, rank))), bf16(normal(gen, (H * K, rank), rank ** -0.5))


def draw_gate_params(gen, L: int, H: int):
    a_log = normal(gen, (L, H), 0.5)
    dt_bias = normal(gen, (L, H, K), 0.1)
    return a_log, dt_bias


def draw_records(gen, rows: int, H: int, RQ: int):
    corr = normal(gen, (rows, H, RQ, V), 0.5)
    keys = bf16(unit_keys(gen, (rows, H, RQ, K)))
    gates = bf16(normal(gen, (rows, H, RQ, K)))
    kg = torch.cat([keys, gates], dim=-1).contiguous()
    return corr, kg


# Key norms for the normalisation edge: the all-zero key, norms whose squares
# (1e-8, 1e-4) are below or near the 1e-6 added inside the root, the unit
# norm of the workloads, and a large one.
KEY_NORMS = (0.0, 1e-4, 1e-2, 1.0, 30.0)


def rescale_keys(gen, keys: torch.Tensor, norms=KEY_NORMS) -> torch.Tensor:
    """BF16 keys (last axis K, unit norm) rescaled per vector to a norm drawn
    uniformly from ``norms`` (0 gives the all-zero key), rounded to BF16 again."""
    idx = torch.randint(0, len(norms), keys.shape[:-1], generator=gen)
    scale = torch.tensor(norms, dtype=torch.float32)[idx]
    return bf16(keys.float() * scale[..., None])


def rescale_record_keys(gen, kg: torch.Tensor, norms=KEY_NORMS) -> torch.Tensor:
    """Key/gate records [..., 2K] with their key halves rescaled as rescale_keys."""
    out = kg.clone()
    out[..., :K] = rescale_keys(gen, kg[..., :K], norms)
    return out


def draw_state(seed: int, n_elems: int, dtype, device="cpu", chunk=1 << 26) -> torch.Tensor:
    """A flat pool of N(0, 0.1) values in ``dtype`` drawn in chunks on ``device``
    (a generator of that device, seeded with ``seed``)."""
    g = _gen(seed, device)
    out = torch.empty(n_elems, dtype=dtype, device=device)
    for start in range(0, n_elems, chunk):
        stop = min(n_elems, start + chunk)
        out[start:stop] = (torch.randn(stop - start, generator=g, device=device) * 0.1).to(dtype)
    return out


def uniform_int(gen, lo: int, hi: int, n: int) -> torch.Tensor:
    """n integers uniform on [lo, hi] (inclusive), int32."""
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int32)


def permutation(gen, n: int) -> torch.Tensor:
    return torch.randperm(n, generator=gen).to(torch.int32)


@dataclass
class Workload:
    name: str
    layers: int
    heads: int
    batch: int
    tokens: int            # q: verify window, or the commit window Q
    record_tokens: int     # RQ: tokens a record holds
    slots: int
    state_bf16: bool
    seed: int
    arrays: Dict[str, torch.Tensor] = field(default_factory=dict)
    windows: Dict[str, Window] = field(default_factory=dict)
    # Per-layer slot strides (elements), for the multi-layer commit.
    slot_strides: List[int] = field(default_factory=list)
    lower_bound: float = LOWER_BOUND
    null_slot: int = NULL_SLOT
    notes: str = ""

    @property
    def page_elems(self) -> int:
        return self.heads * V * K


def config0(seed: int = 0) -> Workload:
    """Tiny: L=1, H=4, B=2, q=4, FP32 state [4 slots, 4, 128, 128]; requests on
    slots {1, 2} (source = destination), slot 3 a spare that must stay
    unchanged, record rows {0, 1}. Sequence: verify the window, then commit
    lens {0, 3}."""
    g = _gen(seed)
    H, B, T, S = 4, 2, 4, 4
    w = Workload("tiny", 1, H, B, T, T, S, False, seed)
    a_log, dt_bias = draw_gate_params(g, 1, H)
    state = normal(g, (S * H * V * K,), 0.1)
    win = draw_window(g, B, T, H)
    w.arrays.update(
        state=state, a_log=a_log, dt_bias=dt_bias,
        state_indices=torch.tensor([1, 2], dtype=torch.int32),
        record_rows=torch.tensor([0, 1], dtype=torch.int32),
        commit_lens=torch.tensor([0, 3], dtype=torch.int32),
        corr=torch.zeros((B, H, T, V), dtype=torch.float32),
        kg=torch.zeros((B, H, T, 2 * K), dtype=torch.bfloat16),
    )
    w.windows["new"] = win
    w.slot_strides = [H * V * K]
    return w


def config1(seed: int = 1, device="cpu") -> Workload:
    """Commit only: L=1, H=32, B=64, window 4, BF16 state [256 slots]; rows 0-55
    live with disjoint sources and destinations from a permutation of 1..255,
    rows 56-63 padded (source = destination = null); lens uniform 0..4."""
    g = _gen(seed)
    H, B, Q, S = 32, 64, 4, 256
    w = Workload("commit", 1, H, B, Q, Q, S, True, seed)
    a_log, dt_bias = draw_gate_params(g, 1, H)
    perm = permutation(g, S - 1) + 1
    live = 56
    src = torch.zeros(B, dtype=torch.int32)
    dst = torch.zeros(B, dtype=torch.int32)
    src[:live] = perm[:live]
    dst[:live] = perm[live:2 * live]
    corr, kg = draw_records(g, B, H, Q)
    lens = uniform_int(g, 0, Q, B)
    w.arrays.update(a_log=a_log, dt_bias=dt_bias, sources=src, destinations=dst,
                    commit_lens=lens, corr=corr, kg=kg)
    w.arrays["state"] = draw_state(seed * 1000 + 7, S * H * V * K, torch.bfloat16, device)
    w.slot_strides = [H * V * K]
    return w


def config2(seed: int = 2, device="cpu") -> Workload:
    """Fused replay+verify: L=1, H=32, B=128, q=4, FP32 state [256 slots];
    request slots are the first 128 of a permutation of 1..255, record rows a
    permutation of 0..127, pending uniform 0..4. The records come from a
    verify of a prior window (drawn here, with seed + 100) run by the caller."""
    g = _gen(seed)
    H, B, T, S = 32, 128, 4, 256
    w = Workload("fused", 1, H, B, T, T, S, False, seed)
    a_log, dt_bias = draw_gate_params(g, 1, H)
    slots = (permutation(g, S - 1) + 1)[:B].contiguous()
    rows = permutation(g, B)
    pending = uniform_int(g, 0, T, B)
    w.windows["new"] = draw_window(g, B, T, H)
    w.windows["prior"] = draw_window(_gen(seed + 100), B, T, H)
    w.arrays.update(a_log=a_log, dt_bias=dt_bias, state_indices=slots, record_rows=rows,
                    pending=pending,
                    corr=torch.zeros((B, H, T, V), dtype=torch.float32),
                    kg=torch.zeros((B, H, T, 2 * K), dtype=torch.bfloat16))
    w.arrays["state"] = draw_state(seed * 1000 + 7, S * H * V * K, torch.float32, device)
    return w


def config3(seed: int = 3, device="cpu", layers: int = 8) -> Workload:
    """Prefix-cache align commit: L=8 per-layer BF16 pools of 641 slots (null,
    256 sources, 256 destinations, 128 boundaries, all disjoint); slot stride
    32*128*128 elements on even layers and 64 elements more on odd layers;
    B=256, window 8, lens uniform 1..8; 128 requests with n >= 2 get a boundary
    slot and m uniform on 1..n-1, the rest boundary 0 and m 0."""
    g = _gen(seed)
    H, B, Q, S = 32, 256, 8, 641
    w = Workload("align_commit", layers, H, B, Q, Q, S, True, seed)
    a_log, dt_bias = draw_gate_params(g, layers, H)
    perm = permutation(g, S - 1) + 1
    src, dst, bnd_pool = perm[:B], perm[B:2 * B], perm[2 * B:2 * B + 128]
    lens = uniform_int(g, 1, Q, B)
    eligible = torch.nonzero(lens >= 2).flatten()
    pick = eligible[torch.randperm(eligible.numel(), generator=g)[:128]]
    bnd = torch.zeros(B, dtype=torch.int32)
    blen = torch.zeros(B, dtype=torch.int32)
    for i, b in enumerate(pick.tolist()):
        bnd[b] = bnd_pool[i]
        n = int(lens[b])
        blen[b] = int(torch.randint(1, n, (1,), generator=g))
    page = H * V * K
    strides = [page if l % 2 == 0 else page + 64 for l in range(layers)]
    corrs, kgs = [], []
    for l in range(layers):
        c, k = draw_records(g, B, H, Q)
        corrs.append(c)
        kgs.append(k)
    w.arrays.update(a_log=a_log, dt_bias=dt_bias, sources=src.contiguous(),
                    destinations=dst.contiguous(), commit_lens=lens, boundaries=bnd,
                    boundary_lens=blen)
    for l in range(layers):
        w.arrays[f"corr{l}"] = corrs[l]
        w.arrays[f"kg{l}"] = kgs[l]
        w.arrays[f"state{l}"] = draw_state(seed * 1000 + 7 + l, S * strides[l],
                                           torch.bfloat16, device)
    w.slot_strides = strides
    return w


def config4(seed: int = 4, device="cpu") -> Workload:
    """Large decode batch: L=1, H=64, B=512, q=8, FP32 state [512 slots] (2 GiB).
    Rows 0-12 have the null slot, rows 13-25 record row -1 (together about 5%
    no-ops); the other requests have distinct slots from 1..511; record rows a
    permutation of 0..511; pending uniform 0..8; the records come from a verify
    of a prior window run by the caller. After the fused step, accepted counts
    uniform 0..8 feed the defer step, then the flush plan and the in-place
    FP32 commit."""
    g = _gen(seed)
    H, B, T, S = 64, 512, 8, 512
    w = Workload("large_decode", 1, H, B, T, T, S, False, seed)
    a_log, dt_bias = draw_gate_params(g, 1, H)
    slots = (permutation(g, S - 1) + 1)[:B - 13]
    state_indices = torch.zeros(B, dtype=torch.int32)
    state_indices[13:] = slots
    rows = permutation(g, B)
    rows[13:26] = -1
    pending = uniform_int(g, 0, T, B)
    accepted = uniform_int(g, 0, T, B)
    w.windows["new"] = draw_window(g, B, T, H)
    w.windows["prior"] = draw_window(_gen(seed + 100), B, T, H)
    w.arrays.update(a_log=a_log, dt_bias=dt_bias, state_indices=state_indices,
                    record_rows=rows, pending=pending, accepted=accepted,
                    corr=torch.zeros((B, H, T, V), dtype=torch.float32),
                    kg=torch.zeros((B, H, T, 2 * K), dtype=torch.bfloat16))
    w.arrays["state"] = draw_state(seed * 1000 + 7, S * H * V * K, torch.float32, device)
    return w


def draw_output_stage(gen, B: int, T: int, H: int):
    """Inputs of the gated RMSNorm output stage: gate = BF16(N(0,1)) per output
    element, weight 1 + N(0, 0.1) per value channel (shared by the heads),
    eps 1e-5."""
    gate = bf16(normal(gen, (B * T, H * V)))
    weight = 1.0 + normal(gen, (V,), 0.1)
    return gate, weight, 1e-5


CONFIGS = {0: config0, 1: config1, 2: config2, 3: config3, 4: config4}


def small_fused_case(seed: int, H: int, B: int, T: int, RQ: int, slots: int,
                     null_rows=(), no_record_rows=(), pending_max: Optional[int] = None):
    """A small randomized fused/verify case: distinct slots from 1..slots-1,
    record rows a permutation, pending uniform 0..pending_max (default RQ),
    optional null-slot and no-record rows; random prior records."""
    g = _gen(seed)
    a_log, dt_bias = draw_gate_params(g, 1, H)
    perm = permutation(g, slots - 1) + 1
    assert B <= slots - 1
    si = perm[:B].clone()
    for b in null_rows:
        si[b] = 0
    rows = permutation(g, B)
    for b in no_record_rows:
        rows[b] = -1
    pm = RQ if pending_max is None else pending_max
    pending = uniform_int(g, 0, pm, B)
    corr, kg = draw_records(g, B, H, RQ)
    state = normal(g, (slots * H * V * K,), 0.1)
    win = draw_window(g, B, T, H)
    return dict(a_log=a_log, dt_bias=dt_bias, state_indices=si, record_rows=rows,
                pending=pending, corr=corr, kg=kg, state=state, window=win)
