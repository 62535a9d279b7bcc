"""Seeded synthetic workloads for the KDA speculative verify/commit path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the CPU oracle's tests and the GPU tests/benchmark
take their inputs from here, so both sides see the same bits.

Workloads (K = V = 128 throughout, scale = 1/sqrt(128)):

  tiny      B=4 rows, H=4, T=4 (window Q=4); q,k,v,g_raw,beta_raw ~N(0,1) in bf16;
            A_log = log U[1,16] per head; g_bias = 0; unbounded gate;
            checkpoints ~N(0,0.02) in slots 1..4 of a 5-slot pool;
            num_accepted ~U{0..4}.
  decode    B=64, H=32, T=4 (Q=4); activations ~N(0,1); g_bias ~N(0,0.1);
            A_log = log U[1,16]; unbounded gate; 256-slot pool, rows in slots
            1..64; checkpoints = the state after 64 random prefill tokens from a
            zero state (the prefill tokens are drawn here; running them through
            the recurrence is left to the caller); num_accepted ~Binomial(4,0.7).
  deep      B=256, H=32, T=8 (Q=8); checkpoints ~N(0,0.02); 1024-slot pool,
            rows in a random sample of slots 1..1023; num_accepted ~U{0..8}.
  decode_bounded
            the decode batch with the bounded gate, lower_bound=-5 (the same
            draws as decode; the prefill that makes the checkpoints runs with
            this gate too).
  ragged    B=128, H=32, T_i ~U{1..8} packed by cu_seqlens (Q=8); g_raw ~N(0,2),
            other activations ~N(0,1); bounded gate, lower_bound=-5; 256-slot
            pool; each row skipped w.p. 0.1 (slot 0 and -1 alternating);
            num_accepted ~U{0..T_i}.
  deferred  B=512, H=32, T=4 (Q=4), 8 layers each with its own 513-slot pool
            and parameters; record_rows a fixed permutation of 0..511; per step
            fresh activations per layer, num_accepted ~U{0..4} and a 20% eager
            mask per request (shared by the layers).

Every draw comes from ``numpy.random.default_rng([seed, *keys])`` with
seed = 1000 + config number and a fixed key per component, so any component
(one layer's pool, one step's activations) can be drawn on its own.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
CONFIG_NAMES = ("tiny", "decode", "deep", "ragged", "deferred")
_SEEDS = {name: 1000 + i + 1 for i, name in enumerate(CONFIG_NAMES)}

# Component keys of the random substreams.
_META, _ACT, _POOL, _PARAM, _PREFILL, _STEP = 1, 2, 3, 4, 5, 6


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.default_rng([seed, *keys])


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    return bf16_from_f32(rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


@dataclass
class Tokens:
    """A packed ragged batch of raw activations (bf16 bit patterns).

    ``qkv`` is one [tokens, 3*H*K] projection output; q, k and v are its
    three [tokens, H, K] column blocks (token stride 3*H*K), as a merged
    q|k|v projection produces them. g is dense [tokens, H, K]; beta [tokens, H].
    """
    qkv: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    H: int
    K: int = HEAD_DIM

    @property
    def num_tokens(self) -> int:
        return self.qkv.shape[0]

    def _block(self, j: int) -> np.ndarray:
        hk = self.H * self.K
        return self.qkv[:, j * hk:(j + 1) * hk].reshape(-1, self.H, self.K)

    @property
    def q(self):
        return self._block(0)

    @property
    def k(self):
        return self._block(1)

    @property
    def v(self):
        return self._block(2)


def _draw_tokens(rng, ntok: int, H: int, g_sigma: float = 1.0) -> Tokens:
    K = HEAD_DIM
    qkv = _normal_bf16(rng, (ntok, 3 * H * K))
    g = _normal_bf16(rng, (ntok, H, K), g_sigma)
    beta = _normal_bf16(rng, (ntok, H))
    return Tokens(qkv=qkv, g=g, beta=beta, H=H)


def _draw_params(rng, H: int, g_bias_sigma: float):
    a_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    if g_bias_sigma > 0:
        g_bias = (rng.standard_normal(H * HEAD_DIM) * g_bias_sigma).astype(np.float32)
    else:
        g_bias = np.zeros(H * HEAD_DIM, np.float32)
    return a_log, g_bias


def checkpoint_slot(seed: int, layer: int, slot: int, H: int, sigma: float = 0.02) -> np.ndarray:
    """One slot's synthetic fp32 checkpoint [H, V, K] ~N(0, sigma)."""
    rng = _rng(seed, _POOL, layer, slot)
    return rng.standard_normal((H, HEAD_DIM, HEAD_DIM), dtype=np.float32) * np.float32(sigma)


@dataclass
class Batch:
    """One layer call's worth of inputs for verify + commit."""
    name: str
    seed: int
    H: int
    Q: int
    scale: float
    lower_bound: float | None
    a_log: np.ndarray          # float32 [H]
    g_bias: np.ndarray         # float32 [H*K]
    cu_seqlens: np.ndarray     # int32 [N+1]
    state_indices: np.ndarray  # int32 [N]; <= 0: skipped row
    num_slots: int
    tokens: Tokens
    num_accepted: np.ndarray   # int32 [N]
    init: str                  # "normal": slots ~N(0,0.02); "prefill": see prefill
    prefill: Tokens | None = None          # 64 tokens per row (init == "prefill")
    prefill_cu: np.ndarray | None = None   # int32 [N+1] for the prefill tokens
    K: int = HEAD_DIM

    @property
    def num_rows(self) -> int:
        return len(self.state_indices)

    def seq_lens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)

    def valid_rows(self) -> np.ndarray:
        return (self.state_indices > 0) & (self.seq_lens() > 0)

    def initial_pool(self) -> np.ndarray:
        """fp32 pool [slots, H, V, K]. For init == "normal" the used slots hold
        N(0, 0.02) draws; unused slots (and all slots for "prefill") are 0."""
        pool = np.zeros((self.num_slots, self.H, self.K, self.K), np.float32)
        if self.init == "normal":
            for s in self.state_indices:
                if s > 0:
                    pool[s] = checkpoint_slot(self.seed, 0, int(s), self.H)
        return pool


# Variants of a workload: (base workload, lower_bound override).
_VARIANTS = {"decode_bounded": ("decode", -5.0)}
SINGLE_CALL = ("tiny", "decode", "decode_bounded", "deep", "ragged")


def make_batch(name: str, B: int | None = None, H: int | None = None) -> Batch:
    """Draw one of the single-call workloads. B and H may be reduced for quick
    runs; every other part of the recipe stays the same."""
    if name in _VARIANTS:
        base, lb = _VARIANTS[name]
        batch = make_batch(base, B, H)
        batch.name = name
        batch.lower_bound = lb
        return batch
    seed = _SEEDS[name]
    meta = _rng(seed, _META)
    if name == "tiny":
        B, H = B or 4, H or 4
        T, Q, num_slots = np.full(B, 4), 4, B + 1
        slots = np.arange(1, B + 1, dtype=np.int32)
        a_log, g_bias = _draw_params(_rng(seed, _PARAM), H, 0.0)
        num_acc = meta.integers(0, 5, size=B)
        lb, init, g_sigma = None, "normal", 1.0
    elif name == "decode":
        B, H = B or 64, H or 32
        T, Q, num_slots = np.full(B, 4), 4, 256
        slots = np.arange(1, B + 1, dtype=np.int32)
        a_log, g_bias = _draw_params(_rng(seed, _PARAM), H, 0.1)
        num_acc = meta.binomial(4, 0.7, size=B)
        lb, init, g_sigma = None, "prefill", 1.0
    elif name == "deep":
        B, H = B or 256, H or 32
        T, Q, num_slots = np.full(B, 8), 8, 1024
        slots = (meta.permutation(num_slots - 1)[:B] + 1).astype(np.int32)
        a_log, g_bias = _draw_params(_rng(seed, _PARAM), H, 0.1)
        num_acc = meta.integers(0, 9, size=B)
        lb, init, g_sigma = None, "normal", 1.0
    elif name == "ragged":
        B, H = B or 128, H or 32
        Q, num_slots = 8, 256
        T = meta.integers(1, 9, size=B)
        slots = (meta.permutation(num_slots - 1)[:B] + 1).astype(np.int32)
        skip = meta.random(B) < 0.1
        nskip = int(skip.sum())
        slots[skip] = np.where(np.arange(nskip) % 2 == 0, 0, -1)
        a_log, g_bias = _draw_params(_rng(seed, _PARAM), H, 0.1)
        num_acc = np.array([meta.integers(0, t + 1) for t in T])
        lb, init, g_sigma = -5.0, "normal", 2.0
    else:
        raise ValueError(f"unknown single-call workload {name!r}")
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(T)
    tokens = _draw_tokens(_rng(seed, _ACT), int(cu[-1]), H, g_sigma)
    batch = Batch(name=name, seed=seed, H=H, Q=Q, scale=HEAD_DIM ** -0.5, lower_bound=lb,
                  a_log=a_log, g_bias=g_bias, cu_seqlens=cu, state_indices=slots.astype(np.int32),
                  num_slots=num_slots, tokens=tokens, num_accepted=num_acc.astype(np.int32),
                  init=init)
    if init == "prefill":
        P = 64
        batch.prefill = _draw_tokens(_rng(seed, _PREFILL), B * P, H)
        batch.prefill_cu = (np.arange(B + 1) * P).astype(np.int32)
    return batch


@dataclass
class LayerParams:
    a_log: np.ndarray
    g_bias: np.ndarray


@dataclass
class DeferredRun:
    """The multi-layer, multi-step deferred-commit workload."""
    seed: int
    B: int
    H: int
    T: int
    Q: int
    layers: int
    steps: int
    num_slots: int
    scale: float
    lower_bound: float | None
    state_indices: np.ndarray   # int32 [B]
    record_rows: np.ndarray     # int32 [B], a permutation of 0..B-1
    cu_seqlens: np.ndarray      # int32 [B+1]
    params: list = field(default_factory=list)   # LayerParams per layer
    K: int = HEAD_DIM

    def num_accepted(self, step: int) -> np.ndarray:
        return _rng(self.seed, _STEP, step, 0).integers(0, self.T + 1, size=self.B).astype(np.int32)

    def eager(self, step: int) -> np.ndarray:
        return (_rng(self.seed, _STEP, step, 1).random(self.B) < 0.2).astype(np.uint8)

    def tokens(self, layer: int, step: int) -> Tokens:
        return _draw_tokens(_rng(self.seed, _ACT, layer, step), self.B * self.T, self.H)

    def slot_state(self, layer: int, slot: int) -> np.ndarray:
        return checkpoint_slot(self.seed, layer, slot, self.H)

    def initial_pool(self, layer: int) -> np.ndarray:
        pool = np.zeros((self.num_slots, self.H, self.K, self.K), np.float32)
        for s in self.state_indices:
            pool[s] = self.slot_state(layer, int(s))
        return pool


def make_deferred(B: int | None = None, H: int | None = None, layers: int | None = None,
                  steps: int = 4) -> DeferredRun:
    seed = _SEEDS["deferred"]
    B, H, layers = B or 512, H or 32, layers or 8
    T = Q = 4
    meta = _rng(seed, _META)
    num_slots = B + 1
    slots = (meta.permutation(B) + 1).astype(np.int32)
    record_rows = meta.permutation(B).astype(np.int32)
    params = []
    for layer in range(layers):
        a_log, g_bias = _draw_params(_rng(seed, _PARAM, layer), H, 0.1)
        params.append(LayerParams(a_log, g_bias))
    cu = (np.arange(B + 1) * T).astype(np.int32)
    return DeferredRun(seed=seed, B=B, H=H, T=T, Q=Q, layers=layers, steps=steps,
                       num_slots=num_slots, scale=HEAD_DIM ** -0.5, lower_bound=None,
                       state_indices=slots, record_rows=record_rows, cu_seqlens=cu,
                       params=params)
