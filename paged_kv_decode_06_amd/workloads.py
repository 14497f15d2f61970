"""Seeded synthetic workloads for paged decode attention.

This module only draws inputs: sequence lengths, a shuffled pool of physical
blocks, block tables, slot mappings and N(0,1) tensors.  It holds none of the
attention or append arithmetic, and both the HIP path and the fp64 oracle read
the same tensors it produces.

The one place where a value is derived rather than drawn is the pre-filled fp8
cache: its codes are made by torch's own ``float8_e4m3fn`` cast (a library
routine) of the N(0,1) source divided by a per-(block, kv head) scale
amax/448 over the tokens already in that block.  Those bytes are an input to
both sides; neither side's encoder is involved.  The pre-filled int8 cache is
drawn outright: codes uniform in [-127, 127] and per-(block, kv head) scales
uniform in [0.01, 0.02] (values within +-2.54, spread about like N(0,1) data).

Recipes (lengths from ``numpy.random.default_rng(seed)``, tensors from a
``torch.Generator`` seeded ``1000 + seed`` on the target device):

  tiny          B=4  Hq=8  Hkv=2 D=64  BS=16, lengths {1, 17, 33, 100}, 64 blocks
  llama3_8b     B=64 Hq=32 Hkv=8 D=128 BS=16, lengths uniform in [512, 4096]
  long_context  B=4  Hq=32 Hkv=8 D=128 BS=16, lengths 131072
  mixed_70b     B=256 Hq=64 Hkv=8 D=128 BS=16, lengths lognormal(median 1500,
                sigma 1) rounded and clipped to [1, 16384], then 13 (5%) set to 1
  fp8           B=128 Hq=32 Hkv=8 D=128 BS=32, lengths uniform in [1024, 16384],
                then 32 sequences (25%) moved so that the appended token opens a
                new block; e4m3fn K/V with fp32 scales per (block, kv head)
  int8          the fp8 recipe with int8 K/V codes (seed 5)
  llama3_8b_verify4
                the llama3_8b recipe (seed 1) with 4 query tokens per sequence
                (a speculative-decoding verify step: the 4 new tokens are
                appended, then each attends causally, bottom-right aligned)
  long_context_window
                the long_context recipe (seed 2) attending a sliding window of
                the last 8192 tokens plus 16 sink tokens
  mixed_70b_verify4
                the mixed_70b recipe (seed 3) with min(4, L) query tokens per
                sequence (G = 8: 32 query columns per kv head)

Every sequence's history holds L-q_len tokens before the step (q_len = 1
unless a recipe says otherwise); the step appends tokens L-q_len .. L-1
(slot = block_tables[b][t//BS]*BS + t%BS for position t) and then attends
over L tokens.  The pool has ceil(1.1 * pages needed) blocks (64 for tiny),
handed out in (sequence, logical page) order from a random permutation, so
about 10% of the blocks are free.  Unused block-table entries are -1.  With
``poison=True`` every cache byte outside the pre-filled history (free blocks,
the tail of each last block, the slot about to be appended) holds NaN, and so
do the scales of blocks with no pre-filled token.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np
import torch

BF16_NAN_BITS = 0x7FC0
E4M3FN_NAN_CODE = 0x7F
E4M3FN_MAX = 448.0


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    kv_dtype: str  # "bf16", "fp8" or "int8"
    max_len: int   # largest length the recipe can produce (sets max_blocks_per_seq)
    description: str = ""
    q_len: int = 1     # query tokens per sequence
    window: int = 0    # sliding window (0: the whole history)
    sinks: int = 0     # tokens kept visible at the start when a window is set
    lengths_from: str = ""   # draw lengths with another recipe's rule


CONFIGS = {
    "tiny": Config("tiny", 0, 4, 8, 2, 64, 16, "bf16", 100,
                   "B4 Hq8 Hkv2 D64 BS16, lengths {1,17,33,100}, pool of 64 blocks"),
    "llama3_8b": Config("llama3_8b", 1, 64, 32, 8, 128, 16, "bf16", 4096,
                        "Llama-3-8B-shaped layer: B64 Hq32 Hkv8 D128 BS16, L~U[512,4096]"),
    "long_context": Config("long_context", 2, 4, 32, 8, 128, 16, "bf16", 131072,
                           "long context: B4 Hq32 Hkv8 D128 BS16, L=131072"),
    "mixed_70b": Config("mixed_70b", 3, 256, 64, 8, 128, 16, "bf16", 16384,
                        "70B-shaped mixed batch: B256 Hq64 Hkv8 D128 BS16, lognormal L"),
    "fp8": Config("fp8", 4, 128, 32, 8, 128, 32, "fp8", 16384,
                  "fp8 e4m3fn KV: B128 Hq32 Hkv8 D128 BS32, L~U[1024,16384]"),
    "int8": Config("int8", 5, 128, 32, 8, 128, 32, "int8", 16384,
                   "int8 KV: B128 Hq32 Hkv8 D128 BS32, L~U[1024,16384]", lengths_from="fp8"),
    "llama3_8b_verify4": Config("llama3_8b_verify4", 1, 64, 32, 8, 128, 16, "bf16", 4096,
                                "speculative verify: llama3_8b shapes, 4 query tokens per "
                                "sequence, bottom-right causal", q_len=4,
                                lengths_from="llama3_8b"),
    "mixed_70b_verify4": Config("mixed_70b_verify4", 3, 256, 64, 8, 128, 16, "bf16", 16384,
                                "speculative verify on the 70B-shaped mix: 4 query tokens per "
                                "sequence (fewer where the history is shorter), bottom-right "
                                "causal; G = 8, so 32 query columns per kv head", q_len=4,
                                lengths_from="mixed_70b"),
    "long_context_window": Config("long_context_window", 2, 4, 32, 8, 128, 16, "bf16", 131072,
                                  "long context, sliding window 8192 + 16 sink tokens",
                                  window=8192, sinks=16, lengths_from="long_context"),
}
CONFIG_ORDER = ["tiny", "llama3_8b", "long_context", "mixed_70b", "fp8", "int8",
                "llama3_8b_verify4", "long_context_window", "mixed_70b_verify4"]


def draw_lengths(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    """Context lengths (including the tokens appended this step) for a config."""
    rule = cfg.lengths_from or cfg.name
    if rule == "tiny":
        L = np.array([1, 17, 33, 100], dtype=np.int64)
    elif rule == "llama3_8b":
        L = rng.integers(512, 4096, cfg.B, endpoint=True)
    elif rule == "long_context":
        L = np.full(cfg.B, 131072, dtype=np.int64)
    elif rule == "mixed_70b":
        x = rng.lognormal(mean=math.log(1500.0), sigma=1.0, size=cfg.B)
        L = np.clip(np.rint(x), 1, 16384).astype(np.int64)
        ones = rng.choice(cfg.B, size=int(round(0.05 * cfg.B)), replace=False)
        L[ones] = 1
    elif rule == "fp8":
        L = rng.integers(1024, 16384, cfg.B, endpoint=True)
        cross = rng.choice(cfg.B, size=cfg.B // 4, replace=False)
        is_cross = np.zeros(cfg.B, dtype=bool)
        is_cross[cross] = True
        # the appended token sits at position L-1; it opens a block when
        # (L-1) % BS == 0
        L[is_cross] = cfg.BS * ((L[is_cross] - 1) // cfg.BS) + 1
        lands_on_zero = (~is_cross) & ((L - 1) % cfg.BS == 0)
        L[lands_on_zero] += 1
    else:
        raise KeyError(cfg.name)
    return L.astype(np.int64)


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    NB: int
    MBS: int
    kv_dtype: str
    scale: float
    lengths: np.ndarray            # host copy of context_lens (int64)
    block_tables_np: np.ndarray    # host copy (int32) [B, MBS]
    slot_mapping_np: np.ndarray    # host copy (int32) [B]
    context_lens: torch.Tensor     # int32 [B]
    block_tables: torch.Tensor     # int32 [B, MBS]
    slot_mapping: torch.Tensor     # int32 [B]
    q: torch.Tensor                # bf16 [B, Hq, D]
    k_new: torch.Tensor            # bf16 [B, Hkv, D]
    v_new: torch.Tensor            # bf16 [B, Hkv, D]
    k_cache: torch.Tensor          # bf16 or uint8 [NB, BS, Hkv, D]
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor] = None  # fp32 [NB, Hkv] (fp8 and int8)
    v_scale: Optional[torch.Tensor] = None
    q_lens: Optional[np.ndarray] = None      # query tokens per sequence (None: all 1)
    q_start_np: Optional[np.ndarray] = None  # int32 [B + 1] cumulative query counts
    q_start: Optional[torch.Tensor] = None
    window: int = 0
    sinks: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


def _bf16_randn(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def build_workload(name: str, B: int, Hq: int, Hkv: int, D: int, BS: int,
                   lengths: Sequence[int], kv_dtype: str = "bf16", seed: int = 0,
                   NB: Optional[int] = None, MBS: Optional[int] = None,
                   scale: Optional[float] = None, device="cpu", poison: bool = False,
                   rng: Optional[np.random.Generator] = None,
                   q_lens: Optional[Sequence[int]] = None, window: int = 0,
                   sinks: int = 0) -> Workload:
    """Draw one workload with the given shapes and context lengths.  q, k_new,
    v_new and slot_mapping have one row per query token (sum of q_lens, one
    per sequence by default); q_start holds the cumulative counts."""
    if rng is None:
        rng = np.random.default_rng(seed)
    L = np.asarray(lengths, dtype=np.int64)
    assert L.shape == (B,)
    assert (L >= 1).all(), "every sequence holds at least the appended token"
    pages = (L + BS - 1) // BS
    needed = int(pages.sum())
    if MBS is None:
        MBS = int(pages.max())
    assert int(pages.max()) <= MBS
    if NB is None:
        NB = int(math.ceil(1.10 * needed))
    assert NB >= needed
    perm = rng.permutation(NB)[:needed].astype(np.int32)
    bt = np.full((B, MBS), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        n = int(pages[b])
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    ql = np.ones(B, dtype=np.int64) if q_lens is None else np.asarray(q_lens, dtype=np.int64)
    assert ql.shape == (B,) and (ql >= 1).all() and (ql <= L).all()
    q_start = np.zeros(B + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(ql)
    TQ = int(q_start[-1])
    seq_of = np.repeat(np.arange(B), ql)                   # sequence of each query token
    tpos = np.concatenate([np.arange(L[b] - ql[b], L[b]) for b in range(B)]).astype(np.int64)
    slots = (bt[seq_of, tpos // BS].astype(np.int64) * BS + tpos % BS).astype(np.int32)

    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(1000 + seed)
    q = _bf16_randn((TQ, Hq, D), gen, device)
    k_new = _bf16_randn((TQ, Hkv, D), gen, device)
    v_new = _bf16_randn((TQ, Hkv, D), gen, device)

    # which (block, in-block slot) pairs hold a pre-filled token (positions < L-q_len)
    filled = np.zeros((NB, BS), dtype=bool)
    for b in range(B):
        n_tok = int(L[b]) - int(ql[b])
        full, rem = divmod(n_tok, BS)
        if full:
            filled[bt[b, :full]] = True
        if rem:
            filled[bt[b, full], :rem] = True
    filled_t = torch.from_numpy(filled).to(device)

    k_scale = v_scale = None
    if kv_dtype == "bf16":
        k_cache = _bf16_randn((NB, BS, Hkv, D), gen, device)
        v_cache = _bf16_randn((NB, BS, Hkv, D), gen, device)
        if poison:
            nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device=device)
            hole = ~filled_t[:, :, None, None]
            k_cache = torch.where(hole, nan, k_cache)
            v_cache = torch.where(hole, nan, v_cache)
    elif kv_dtype == "fp8":
        caches, scales = [], []
        for _ in range(2):
            src = torch.randn((NB, BS, Hkv, D), generator=gen, device=device,
                              dtype=torch.float32).to(torch.bfloat16).float()
            src = src * filled_t[:, :, None, None]
            amax = src.abs().amax(dim=(1, 3))              # [NB, Hkv]
            sc = amax / E4M3FN_MAX
            empty = amax == 0
            sc = torch.where(empty, torch.full_like(sc, float("nan") if poison else 1.0), sc)
            y = src / torch.where(empty, torch.ones_like(sc), sc)[:, None, :, None]
            codes = y.clamp(-E4M3FN_MAX, E4M3FN_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
            if poison:
                codes = torch.where(~filled_t[:, :, None, None],
                                    torch.tensor(E4M3FN_NAN_CODE, dtype=torch.uint8, device=device),
                                    codes)
            caches.append(codes.contiguous())
            scales.append(sc.contiguous())
            del src, y
        k_cache, v_cache = caches
        k_scale, v_scale = scales
    elif kv_dtype == "int8":
        caches, scales = [], []
        used = torch.from_numpy(filled.any(axis=1)).to(device)   # blocks with a pre-filled token
        for _ in range(2):
            codes = torch.randint(-127, 128, (NB, BS, Hkv, D), generator=gen, device=device,
                                  dtype=torch.int8)
            hole = ~filled_t[:, :, None, None]
            codes = torch.where(hole, torch.tensor(-128 if poison else 0, dtype=torch.int8,
                                                   device=device), codes)
            sc = 0.01 + 0.01 * torch.rand((NB, Hkv), generator=gen, device=device,
                                          dtype=torch.float32)
            sc = torch.where(used[:, None], sc,
                             torch.full_like(sc, float("nan") if poison else 1.0))
            caches.append(codes.contiguous())
            scales.append(sc.contiguous())
        k_cache, v_cache = caches
        k_scale, v_scale = scales
    else:
        raise ValueError(kv_dtype)

    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Workload(
        name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, BS=BS, NB=NB, MBS=MBS, kv_dtype=kv_dtype,
        scale=float(scale), lengths=L, block_tables_np=bt, slot_mapping_np=slots,
        context_lens=torch.from_numpy(L.astype(np.int32)).to(device),
        block_tables=torch.from_numpy(bt).to(device),
        slot_mapping=torch.from_numpy(slots).to(device),
        q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
        k_scale=k_scale, v_scale=v_scale, q_lens=ql, q_start_np=q_start,
        q_start=torch.from_numpy(q_start).to(device), window=int(window), sinks=int(sinks))


def make_config_workload(name: str, device="cpu", poison: bool = False) -> Workload:
    """The named synthetic configuration, seeded by its index."""
    cfg = CONFIGS[name]
    rng = np.random.default_rng(cfg.seed)
    L = draw_lengths(cfg, rng)
    MBS = (cfg.max_len + cfg.BS - 1) // cfg.BS
    NB = 64 if cfg.name == "tiny" else None
    return build_workload(cfg.name, cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.BS, L,
                          kv_dtype=cfg.kv_dtype, seed=cfg.seed, NB=NB, MBS=MBS,
                          device=device, poison=poison, rng=rng,
                          q_lens=np.minimum(cfg.q_len, L), window=cfg.window, sinks=cfg.sinks)


# ---- host views for the oracle ---------------------------------------------

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a bf16 tensor, as a numpy uint16 array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def cache_host(t: torch.Tensor) -> np.ndarray:
    """Host copy of a cache in the oracle's raw form (uint16 bf16 bits, uint8
    e4m3fn codes or int8 codes)."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    assert t.dtype in (torch.uint8, torch.int8)
    return t.detach().contiguous().cpu().numpy()
