"""Seeded synthetic inputs for the slot-KV decode-attention step.

This module only draws random inputs and parameter tables; it performs none of
the step's arithmetic.  It is the one piece that both the HIP path (through the
tests and the benchmark) and the CPU oracle consume.

Every workload follows one recipe (numpy ``Generator(PCG64(seed))``):

  1. ``slots``      -- a random permutation of ``range(n_slots)`` cut to B;
  2. ``positions``  -- per the workload's length mix;
  3. per layer, in order: q [B, n_heads*D], k_new [B, kv_dim], v_new [B, kv_dim]
     ~ N(0, 1); q_norm_w, k_norm_w [D] ~ 1 + N(0, 0.1); sinks [n_heads] ~ N(0, 1)
     when the workload has sinks.

The RoPE table is ``inv_freq[i] = float32(theta ** (-2 i / D))`` computed in
float64 -- the table that the model uploads once at init (ZINC "Forward Cuda",
init section), handed to both sides as data.  ``scale`` is float32(1/sqrt(D))
and ``eps`` is 1e-6.

History K/V (the slot contents for positions 0..pos-1) is N(0, 1).  Small
workloads draw it here with numpy (``history_host``); the large ones are filled
on the device from a seeded ``torch.Generator`` by the caller, and the oracle
reads back the rows it checks before the step runs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np


@dataclasses.dataclass
class LayerParams:
    n_heads: int
    n_kv_heads: int
    head_dim: int
    q_norm_w: np.ndarray  # [D] f32
    k_norm_w: np.ndarray  # [D] f32
    inv_freq: np.ndarray  # [D/2] f32
    sinks: Optional[np.ndarray]  # [n_heads] f32 or None
    eps: float
    scale: float
    flags: int = 0  # convention flags: 1 V-norm, 2 interleaved RoPE, 4 (1 + w) norm weights

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim


@dataclasses.dataclass
class LayerInputs:
    q: np.ndarray      # [B, n_heads*D] f32
    k_new: np.ndarray  # [B, kv_dim] f32
    v_new: np.ndarray  # [B, kv_dim] f32


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    n_slots: int
    slot_ctx: int
    layers: List[LayerParams]
    positions: np.ndarray  # [B] u32
    slots: np.ndarray      # [B] u32
    inputs: List[LayerInputs]
    theta: float

    @property
    def B(self) -> int:
        return int(self.positions.shape[0])

    @property
    def kv_dims(self) -> List[int]:
        return [L.kv_dim for L in self.layers]

    def kv_bytes(self, layer: Optional[int] = None) -> int:
        """Algorithmic KV bytes of one step: sum_b (pos_b + 1) * kv_dim * 4 for
        K and again for V, for one layer or (layer=None) for every layer."""
        keys = int(self.positions.astype(np.int64).sum()) + self.B
        layers = self.layers if layer is None else [self.layers[layer]]
        return sum(keys * L.kv_dim * 4 * 2 for L in layers)


def rope_inv_freq(theta: float, head_dim: int) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return (theta ** (-2.0 * i / head_dim)).astype(np.float32)


def make_layer(rng, n_heads, n_kv_heads, head_dim, theta, with_sinks, eps=1e-6):
    return LayerParams(
        n_heads=n_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
        q_norm_w=(1.0 + 0.1 * rng.standard_normal(head_dim)).astype(np.float32),
        k_norm_w=(1.0 + 0.1 * rng.standard_normal(head_dim)).astype(np.float32),
        inv_freq=rope_inv_freq(theta, head_dim),
        sinks=(rng.standard_normal(n_heads).astype(np.float32) if with_sinks else None),
        eps=eps, scale=float(np.float32(1.0 / math.sqrt(head_dim))))


def _layer_inputs(rng, B, n_heads, n_kv_heads, head_dim) -> LayerInputs:
    return LayerInputs(
        q=rng.standard_normal((B, n_heads * head_dim), dtype=np.float32),
        k_new=rng.standard_normal((B, n_kv_heads * head_dim), dtype=np.float32),
        v_new=rng.standard_normal((B, n_kv_heads * head_dim), dtype=np.float32))


def _build(name, seed, n_slots, slot_ctx, B, shapes, theta, sinks, pos_fn):
    rng = np.random.Generator(np.random.PCG64(seed))
    slots = rng.permutation(n_slots)[:B].astype(np.uint32)
    positions = np.asarray(pos_fn(rng, B, slot_ctx), dtype=np.uint32)
    layers, inputs = [], []
    for (H, Hkv, D) in shapes:
        # draw the per-layer inputs first, then the parameter tables
        li = _layer_inputs(rng, B, H, Hkv, D)
        L = make_layer(rng, H, Hkv, D, theta, sinks)
        layers.append(L)
        inputs.append(li)
    return Workload(name=name, seed=seed, n_slots=n_slots, slot_ctx=slot_ctx,
                    layers=layers, positions=positions, slots=slots,
                    inputs=inputs, theta=theta)


def tiny() -> Workload:
    """1 layer, 4 heads / 2 kv heads / D=64, 4 slots x 128, B=4, pos U{0..127},
    theta 1e4, no sinks."""
    return _build("tiny", 1, 4, 128, 4, [(4, 2, 64)], 1e4, False,
                  lambda r, B, C: r.integers(0, C, size=B))


def mid() -> Workload:
    """1 layer, 32 heads / 8 kv heads / D=128 (GQA 4:1), 64 slots x 4096,
    B=64 (one row per slot), pos U{1..4095}, theta 1e6."""
    return _build("mid", 2, 64, 4096, 64, [(32, 8, 128)], 1e6, False,
                  lambda r, B, C: r.integers(1, C, size=B))


def _log_uniform(r, B, C):
    p = np.floor(np.exp(r.random(B) * math.log(C))).astype(np.int64)
    return np.clip(p, 1, C - 1)


def long_ctx() -> Workload:
    """1 layer, 16 heads / 8 kv heads / D=256, 16 slots x 32768, B=16,
    pos log-uniform in [1, 32767], theta 1e6."""
    return _build("long", 3, 16, 32768, 16, [(16, 8, 256)], 1e6, False, _log_uniform)


def _many_positions(r, B, C):
    p = r.integers(1, C, size=B)
    fresh = r.choice(B, size=int(round(0.1 * B)), replace=False)
    p[fresh] = 0
    return p


def many_short() -> Workload:
    """1 layer, 32 heads / 4 kv heads / D=128, 256 slots x 2048, B=256; 10% of
    rows at pos 0 (freshly admitted reused slots), the rest U{1..2047};
    theta 1e6."""
    return _build("many", 4, 256, 2048, 256, [(32, 4, 128)], 1e6, False, _many_positions)


def layer_stack() -> Workload:
    """8 layers alternating kv_dim 1024 (8 x 128) and 2048 (8 x 256), 32 heads,
    per-head sinks ~ N(0,1), 128 slots x 8192, B=128, pos U{1..8191}, theta 1e6."""
    shapes = [(32, 8, 128) if (l % 2 == 0) else (32, 8, 256) for l in range(8)]
    return _build("layer_stack", 5, 128, 8192, 128, shapes, 1e6, True,
                  lambda r, B, C: r.integers(1, C, size=B))


WORKLOADS = {"tiny": tiny, "mid": mid, "long": long_ctx, "many": many_short,
             "layer_stack": layer_stack}


def history_host(w: Workload, layer: int, seed_offset: int = 0):
    """Full slot history for one layer as host arrays [n_slots, slot_ctx,
    kv_dim] f32 ~ N(0,1) (small workloads only)."""
    L = w.layers[layer]
    rng = np.random.Generator(np.random.PCG64(1000 * w.seed + 17 * layer + seed_offset))
    shape = (w.n_slots, w.slot_ctx, L.kv_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return k, v


def device_history_seed(w: Workload, layer: int, which: int) -> int:
    """Seed of the torch generator that fills K (which=0) or V (which=1) of one
    layer on the device."""
    return 1_000_003 * w.seed + 7919 * layer + which


def poison_outside(cache: np.ndarray, positions, slots, value) -> None:
    """Fill every cell that no batch row may read -- positions > pos_b of each
    batch slot and every slot outside the batch -- with ``value``."""
    n_slots, slot_ctx, _ = cache.shape
    used = np.zeros(n_slots, bool)
    for p, s in zip(positions, slots):
        cache[s, int(p) + 1:, :] = value
        used[s] = True
    cache[~used] = value


# ---------------------------------------------------------------- slot prefill
@dataclasses.dataclass
class PrefillWorkload:
    """T tokens of one sequence written into slot ``slot`` at positions
    pos0 .. pos0+T-1 (the history 0..pos0-1 is already in the slot)."""
    name: str
    seed: int
    n_slots: int
    slot_ctx: int
    slot: int
    pos0: int
    layer: LayerParams
    inputs: LayerInputs  # q [T, n_heads*D], k_new / v_new [T, kv_dim]
    theta: float

    @property
    def T(self) -> int:
        return int(self.inputs.q.shape[0])

    def attn_flops(self) -> int:
        """Multiply-adds of the attention counted as 2 flops each: token t
        scores pos0+t+1 keys and sums as many value rows, per query head."""
        L = self.layer
        keys = self.T * self.pos0 + self.T * (self.T + 1) // 2
        return 2 * 2 * keys * L.n_heads * L.head_dim


def _build_prefill(name, seed, n_slots, slot_ctx, pos0, T, shape, theta, sinks):
    """Recipe: slot = a uniform draw from range(n_slots); then q [T, H*D],
    k_new / v_new [T, kv_dim] ~ N(0, 1); then the layer's tables as above."""
    rng = np.random.Generator(np.random.PCG64(seed))
    slot = int(rng.integers(0, n_slots))
    H, Hkv, D = shape
    li = _layer_inputs(rng, T, H, Hkv, D)
    L = make_layer(rng, H, Hkv, D, theta, sinks)
    return PrefillWorkload(name=name, seed=seed, n_slots=n_slots, slot_ctx=slot_ctx, slot=slot,
                           pos0=pos0, layer=L, inputs=li, theta=theta)


def prefill_tiny() -> PrefillWorkload:
    """4 heads / 2 kv heads / D=64, 4 slots x 128; 37 tokens after 21 of history."""
    return _build_prefill("prefill_tiny", 11, 4, 128, 21, 37, (4, 2, 64), 1e4, False)


def prefill_prompt() -> PrefillWorkload:
    """A 2048-token prompt from position 0 into one slot of a 64-slot x 4096
    cache; 32 heads / 8 kv heads / D=128 (the decode workload's layer shape)."""
    return _build_prefill("prefill_prompt", 12, 64, 4096, 0, 2048, (32, 8, 128), 1e6, False)


def prefill_chunk() -> PrefillWorkload:
    """A 512-token chunk appended after 3072 positions of history, same shapes."""
    return _build_prefill("prefill_chunk", 13, 64, 4096, 3072, 512, (32, 8, 128), 1e6, False)


PREFILL_WORKLOADS = {"prefill_tiny": prefill_tiny, "prefill_prompt": prefill_prompt,
                     "prefill_chunk": prefill_chunk}


# ---------------------------------------------------------------- multi-row verify
@dataclasses.dataclass
class VerifyWorkload:
    """ks[i] consecutive rows for each sequence i, at positions pos0[i] ..
    of slot slots[i] (rows sequence-major in ``inputs``)."""
    name: str
    seed: int
    n_slots: int
    slot_ctx: int
    slots: np.ndarray  # [n_seq] u32
    pos0: np.ndarray   # [n_seq] u32
    ks: np.ndarray     # [n_seq] u32
    layer: LayerParams
    inputs: LayerInputs  # [sum ks] rows
    theta: float

    @property
    def rows(self) -> int:
        return int(self.ks.astype(np.int64).sum())

    def kv_bytes(self) -> int:
        """K and V bytes of the keys the rows attend over, each key once per
        sequence: sum_i (pos0_i + ks_i) * kv_dim * 4 * 2."""
        keys = int((self.pos0.astype(np.int64) + self.ks).sum())
        return keys * self.layer.kv_dim * 4 * 2


def _build_verify(name, seed, n_slots, slot_ctx, n_seq, k, shape, theta, sinks):
    """Recipe: slots = a permutation of range(n_slots) cut to n_seq; pos0 ~
    U{1 .. slot_ctx - k}; every sequence has k rows; then q / k_new / v_new
    [n_seq*k, ...] ~ N(0, 1) and the layer's tables as above."""
    rng = np.random.Generator(np.random.PCG64(seed))
    slots = rng.permutation(n_slots)[:n_seq].astype(np.uint32)
    pos0 = rng.integers(1, slot_ctx - k + 1, size=n_seq).astype(np.uint32)
    ks = np.full(n_seq, k, np.uint32)
    H, Hkv, D = shape
    li = _layer_inputs(rng, n_seq * k, H, Hkv, D)
    L = make_layer(rng, H, Hkv, D, theta, sinks)
    return VerifyWorkload(name=name, seed=seed, n_slots=n_slots, slot_ctx=slot_ctx, slots=slots,
                          pos0=pos0, ks=ks, layer=L, inputs=li, theta=theta)


def verify_mid() -> VerifyWorkload:
    """4 rows (a draft to verify) for each of 64 sequences, one per slot of a
    64-slot x 4096 cache, at pos0 U{1..4092}; the decode workload's layer
    shape (32 heads / 8 kv heads / D=128)."""
    return _build_verify("verify_mid", 14, 64, 4096, 64, 4, (32, 8, 128), 1e6, False)


VERIFY_WORKLOADS = {"verify_mid": verify_mid}


# ---------------------------------------------------------------- per-slot SSM state
@dataclasses.dataclass
class StateWorkload:
    """Reset on admit of ``slots`` in a slot state of ``n_slots`` slots whose
    ssm layers each hold a conv ring of conv_state_len floats and a recurrent
    state of ssm_state_len floats per slot (no attention layers: their KV
    needs no reset).  The state's contents before the reset are seeded
    N(0, 1) (``state_seed`` drives torch generators on the device)."""
    name: str
    seed: int
    n_slots: int
    conv_state_len: list
    ssm_state_len: list
    slots: np.ndarray  # [n_reset] u32

    @property
    def state_seed(self) -> int:
        return 1000 + self.seed

    def bytes_per_slot(self) -> int:
        return 4 * (sum(self.conv_state_len) + sum(self.ssm_state_len))

    def write_bytes(self) -> int:
        """Bytes a reset writes: every listed slot's conv ring and recurrent
        state in every ssm layer, once per listed slot."""
        return len(self.slots) * self.bytes_per_slot()


def _build_state(name, seed, n_slots, conv_lens, ssm_lens, n_reset):
    """Recipe: slots = a permutation of range(n_slots) cut to n_reset."""
    rng = np.random.Generator(np.random.PCG64(seed))
    slots = rng.permutation(n_slots)[:n_reset].astype(np.uint32)
    return StateWorkload(name=name, seed=seed, n_slots=n_slots, conv_state_len=list(conv_lens),
                         ssm_state_len=list(ssm_lens), slots=slots)


def state_tiny() -> StateWorkload:
    """Ragged sizes (not multiples of 4 floats; one state spanning several
    16 KiB tiles) over few slots."""
    return _build_state("state_tiny", 16, 6, [27, 8, 3], [4099, 10000, 7], 3)


def state_admit() -> StateWorkload:
    """8 admits into 64 slots of a 36-ssm-layer hybrid whose layers keep a
    3-step conv ring over 8192 channels (24576 floats) and a 32-head
    128 x 128 recurrent state (524288 floats) per slot: 2.2 MB per layer and
    slot, 633 MB written per call.  The sizes are chosen here as typical of a
    gated linear-attention layer; the pages give none."""
    return _build_state("state_admit", 15, 64, [3 * 8192] * 36, [32 * 128 * 128] * 36, 8)


STATE_WORKLOADS = {"state_tiny": state_tiny, "state_admit": state_admit}
