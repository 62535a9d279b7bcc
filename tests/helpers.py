"""Shared test utilities: moving seeded workloads to the GPU, running the
oracle on them, and the parity criteria.

Parity criteria (fp32 state, bf16 outputs):
  state  per (slot, head): ||S_gpu - S_ref||_F <= 1e-5 * ||S_ref||_F
  o      the stated gate: |o_gpu - o_ref| <= ulp_bf16(o_ref) + 1e-3, o_ref the
         oracle's bf16 value; and a tight check on every comparison:
         |o_gpu - o_ref| <= ulp_bf16(o_ref) + 1e-5. The outputs of these
         workloads are small (median |o| about 1e-3), where the gate's
         absolute term alone would pass a zero output; an fp32 computation
         of o that differs from the fp64 one only by rounding lands on the
         oracle's bf16 value or a neighbour, which the tight check allows.
  records, untouched memory: bitwise
"""

from __future__ import annotations

import numpy as np

from oracle import kda_ref as ref

S_RTOL = 1e-5
O_ATOL = 1e-3          # the stated output tolerance (the gate)
O_ATOL_TIGHT = 1e-5    # the tight check applied alongside it


def bf16_val(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(bits: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at each value: 2^(exponent - 7); the smallest
    subnormal spacing 2^-133 for the subnormal range and zero."""
    b = np.asarray(bits, np.uint16)
    e = ((b >> 7) & 0xFF).astype(np.int64)
    return np.ldexp(1.0, np.maximum(e, 1) - 127 - 7)


def o_stats(o_gpu_bits: np.ndarray, o_ref_bits: np.ndarray, mask=None) -> dict:
    """Distance of the GPU outputs from the oracle's in bf16 steps: the
    largest |difference| / ulp_bf16(reference), the share that is
    bit-identical and the number compared."""
    g, r = bf16_val(o_gpu_bits), bf16_val(o_ref_bits)
    ulp = ulp_bf16(o_ref_bits)
    d = np.abs(g - r) / ulp
    same = np.asarray(o_gpu_bits, np.uint16) == np.asarray(o_ref_bits, np.uint16)
    if mask is not None:
        m = np.broadcast_to(mask, d.shape)
        d, same = d[m], same[m]
    n = int(d.size)
    return {"n": n, "max_ulp": float(d.max()) if n else 0.0,
            "bit_exact": float(same.mean()) if n else 1.0}


def check_o(o_gpu_bits: np.ndarray, o_ref_bits: np.ndarray, mask=None, what="o",
            quiet: bool = False) -> dict:
    """Both output checks (the gate and the tight one); prints and returns
    the ulp statistics."""
    g, r = bf16_val(o_gpu_bits), bf16_val(o_ref_bits)
    ulp = ulp_bf16(o_ref_bits)
    err = np.abs(g - r)
    for atol, kind in ((O_ATOL, "tolerance"), (O_ATOL_TIGHT, "tight check")):
        bad = err > ulp + atol
        if mask is not None:
            bad &= mask
        if bad.any():
            idx = np.argwhere(bad)[:5]
            raise AssertionError(f"{what}: {int(bad.sum())} elements outside the {kind} "
                                 f"(1 ulp + {atol:g}), e.g. at {idx.tolist()}: gpu "
                                 f"{g[tuple(idx[0])]} ref {r[tuple(idx[0])]}")
    st = o_stats(o_gpu_bits, o_ref_bits, mask)
    if not quiet:
        print(f"  {what}: {st['n']} outputs, max {st['max_ulp']:.2f} ulp, "
              f"{100 * st['bit_exact']:.2f}% bit-exact", flush=True)
    return st


def check_state(S_gpu: np.ndarray, S_ref: np.ndarray, what="state") -> float:
    """S_* [..., V, K] fp32; per-head relative Frobenius error over the last two axes."""
    d = S_gpu.astype(np.float64) - S_ref.astype(np.float64)
    num = np.sqrt(np.sum(d * d, axis=(-1, -2)))
    den = np.sqrt(np.sum(S_ref.astype(np.float64) ** 2, axis=(-1, -2)))
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= S_RTOL, f"{what}: relative Frobenius error {worst:.3e} > {S_RTOL}"
    return worst


def oracle_layer(batch) -> ref.Layer:
    return ref.Layer(batch.a_log, batch.g_bias, batch.scale, batch.lower_bound)


def oracle_records(rows: int, H: int, Q: int, fill: int = 0) -> ref.Records:
    return ref.Records.empty(rows, H, Q, 128, fill=fill)


def oracle_prefill_pool(batch) -> np.ndarray:
    """The batch's fp32 checkpoint pool; for the prefill recipe the state
    after the prefill tokens from zero, by the oracle's recurrence."""
    pool = batch.initial_pool()
    if batch.init == "prefill":
        p = batch.prefill
        o = np.zeros((p.num_tokens, batch.H, 128), np.uint16)
        ref.kda_recurrent(oracle_layer(batch), p.q, p.k, p.v, p.g, p.beta, batch.prefill_cu,
                          pool, batch.state_indices, o)
    return pool


# ------------------------------------------------------------ GPU side ----

def to_dev(x: np.ndarray, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def bf16_dev(bits: np.ndarray, device="cuda:0"):
    import torch
    return to_dev(np.ascontiguousarray(bits).view(np.int16), device).view(torch.bfloat16)


def bits_host(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class DevTokens:
    """A workloads.Tokens on the GPU: q/k/v are column blocks of one qkv."""

    def __init__(self, tokens, device="cuda:0"):
        n, H, K = tokens.num_tokens, tokens.H, tokens.K
        self.qkv = bf16_dev(tokens.qkv, device)
        hk = H * K
        self.q = self.qkv[:, 0:hk].view(n, H, K)
        self.k = self.qkv[:, hk:2 * hk].view(n, H, K)
        self.v = self.qkv[:, 2 * hk:3 * hk].view(n, H, K)
        self.g = bf16_dev(tokens.g, device)
        self.beta = bf16_dev(tokens.beta, device)

    def args(self):
        return self.q, self.k, self.v, self.g, self.beta


def dev_layer(batch, device="cuda:0"):
    import linear_attention_speculative_kda_amd as kda
    return kda.Layer(a_log=to_dev(batch.a_log, device), g_bias=to_dev(batch.g_bias, device),
                     scale=batch.scale, lower_bound=batch.lower_bound)


def dev_records(rows: int, H: int, Q: int, fill: int = 0, device="cuda:0"):
    import torch
    import linear_attention_speculative_kda_amd as kda
    rec = kda.allocate_records(rows, H, Q, device)
    for t in (rec.k, rec.v, rec.g, rec.beta):
        t.view(torch.int16).fill_(np.int16(np.uint16(fill).view(np.int16)))
    return rec


def records_host(rec) -> ref.Records:
    return ref.Records(k=bits_host(rec.k), v=bits_host(rec.v), g=bits_host(rec.g),
                       beta=bits_host(rec.beta))
