"""Seeded synthetic workloads for paged decode attention.

Shared by the tests, the benchmark and the smoke check: it draws inputs only
(lengths, page tables, slot mappings, Q/K/V values, poison) and holds none of
the method's arithmetic.  Values are drawn in float32 with torch's seeded
generator on the requested device, then cast (round to nearest even) to the
storage dtype; lengths, block placement and table padding come from a seeded
numpy generator.

The five workloads mirror the shapes the pages talk about (16-token blocks,
decode over every cached token, GQA head groups, long contexts, FP8 cache with
shared prefixes); sizes and distributions are fixed here:

* tiny      B=4, Hq=Hkv=4, D=64, f16, lengths {1,17,33,50}, 64-block pool.
* llama7b   B=32, Hq=Hkv=32, D=128, f16, lengths uniform in [1, 2048].
* gqa70b    B=64, Hq=64, Hkv=8, D=128, bf16, lengths round(1024*e^Z), Z~N(0,1),
            clipped to [16, 4096].
* longctx   B=8, Hq=Hkv=32, D=128, f16, lengths uniform in [32768, 131072],
            512-token partitions, values N(0, std 0.5).
* fp8beams  16 prompts x 4 beams (B=64), Hq=32, Hkv=8, D=128, Q bf16, FP8 E4M3
            cache with per-token scales; each beam's table holds its prompt's
            1024-token prefix blocks (shared by the 4 beams) then 256 private
            tokens.
* llama7b_b256  the llama7b shape with B=256 sequences.

Conventions (all workloads):

* ``context_lens[b]`` counts the token appended in this step: before the step
  the cache holds tokens 0..L_b-2 and the new token goes to position L_b-1.
* Pools hold num_blocks = ceil(1.1 * blocks in use) physical blocks (64 for
  tiny), handed out in a seeded random order.
* Every slot that holds no token yet (free blocks, slots past the end of a
  sequence, the new token's slot) is filled with NaN bit patterns, and table
  entries past a sequence's last block point at NaN-filled free blocks when
  any exist, so that any read of them shows up in the output.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

from .blocks import BLOCK_SIZE, BlockPool, blocks_for, slot_of

NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F}
TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str
    cache_dtype: str
    lengths: str                 # "fixed", "uniform", "lognormal", "beams"
    len_args: tuple
    value_std: float = 1.0
    partition_size: int = 0      # 0 = library's choice
    pool_blocks: int = 0         # 0 = ceil(1.1 * blocks in use)
    seed: int = 0
    beams: int = 1               # >1: shared-prefix beam groups
    prefix_len: int = 0

    @property
    def src_dtype(self):
        """dtype of freshly produced K/V (the append's input)."""
        return self.q_dtype if self.cache_dtype == "fp8_e4m3" else self.cache_dtype

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)


CONFIGS = {
    "tiny": DecodeConfig("tiny", 4, 4, 4, 64, "f16", "f16", "fixed", (1, 17, 33, 50),
                         pool_blocks=64, seed=1001),
    "llama7b": DecodeConfig("llama7b", 32, 32, 32, 128, "f16", "f16", "uniform", (1, 2048),
                            seed=1002),
    "gqa70b": DecodeConfig("gqa70b", 64, 64, 8, 128, "bf16", "bf16", "lognormal", (1024.0, 1.0, 16, 4096),
                           seed=1003),
    "longctx": DecodeConfig("longctx", 8, 32, 32, 128, "f16", "f16", "uniform", (32768, 131072),
                            value_std=0.5, partition_size=512, seed=1004),
    "fp8beams": DecodeConfig("fp8beams", 64, 32, 8, 128, "bf16", "fp8_e4m3", "beams", (1280,),
                             seed=1005, beams=4, prefix_len=1024),
    # the LLaMA-7B shape at a serving-size batch (the balanced split over more than 64 sequences)
    "llama7b_b256": DecodeConfig("llama7b_b256", 256, 32, 32, 128, "f16", "f16", "uniform", (1, 2048),
                                 seed=1006),
}


def sample_lengths(cfg, rng):
    B = cfg.num_seqs
    if cfg.lengths == "fixed":
        lens = np.array(cfg.len_args, dtype=np.int64)
        assert lens.size == B
    elif cfg.lengths == "uniform":
        lo, hi = cfg.len_args
        lens = rng.integers(lo, hi + 1, size=B)
    elif cfg.lengths == "lognormal":
        median, sigma, lo, hi = cfg.len_args
        lens = np.clip(np.round(median * np.exp(sigma * rng.standard_normal(B))), lo, hi)
    elif cfg.lengths == "beams":
        lens = np.full(B, cfg.len_args[0])
    else:
        raise ValueError(cfg.lengths)
    return lens.astype(np.int32)


@dataclass
class Workload:
    cfg: DecodeConfig
    query: torch.Tensor          # [B, Hq, D] q dtype
    key_cache: torch.Tensor      # [nb, 16, Hkv, D] cache dtype (uint8 codes for FP8)
    value_cache: torch.Tensor
    k_scale: torch.Tensor        # [nb, 16] float32 (FP8 cache only, else None)
    v_scale: torch.Tensor
    block_tables: torch.Tensor   # [B, max_blocks] int32
    context_lens: torch.Tensor   # [B] int32
    slot_mapping: torch.Tensor   # [B] int64: slot of each sequence's new token
    key_new: torch.Tensor        # [B, Hkv, D] src dtype
    value_new: torch.Tensor
    # FP8 cache only: K/V of every cached token (before this step) and their slots,
    # to be written into the empty pool by the quantising append.
    fill_key: torch.Tensor = None
    fill_value: torch.Tensor = None
    fill_slots: torch.Tensor = None
    lens_np: np.ndarray = field(default=None)
    tables_np: np.ndarray = field(default=None)
    num_blocks: int = 0
    used_blocks: int = 0

    @property
    def max_context_len(self):
        return int(self.lens_np.max()) if self.lens_np.size else 0

    def tensors(self):
        return {k: v for k, v in self.__dict__.items() if isinstance(v, torch.Tensor)}


def _randn(shape, std, dtype, gen, device, chunk_rows=1 << 20):
    """float32 N(0, std) draws cast to ``dtype``, produced in row chunks."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1] = x.to(dtype)
    return out


def _rows_per_chunk(row_elems, budget_elems=1 << 28):
    return max(1, budget_elems // max(1, row_elems))


def build_tables(cfg, lens, rng):
    """Page tables for all sequences: (tables int32 [B, max_blocks], num_blocks, used, pool)."""
    B = cfg.num_seqs
    if cfg.beams > 1:
        prompts = B // cfg.beams
        per_beam_private = blocks_for(int(lens[0])) - cfg.prefix_len // BLOCK_SIZE
        used = prompts * (cfg.prefix_len // BLOCK_SIZE) + B * per_beam_private
    else:
        used = int(sum(blocks_for(int(n)) for n in lens))
    nb = cfg.pool_blocks or int(math.ceil(1.1 * used))
    pool = BlockPool(rng.permutation(nb))
    rows = []
    if cfg.beams > 1:
        assert cfg.prefix_len % BLOCK_SIZE == 0
        for p in range(B // cfg.beams):
            prefix = pool.allocate_tokens(cfg.prefix_len)
            for beam in range(cfg.beams):
                shared = pool.share(prefix) if beam else list(prefix)
                private = pool.allocate_tokens(int(lens[p * cfg.beams + beam]) - cfg.prefix_len)
                rows.append(shared + private)
    else:
        for n in lens:
            rows.append(pool.allocate_tokens(int(n)))
    max_blocks = max(1, max(len(r) for r in rows))
    free = np.array(pool.free_ids(), dtype=np.int64)
    tables = np.zeros((B, max_blocks), dtype=np.int32)
    for b, r in enumerate(rows):
        tables[b, :len(r)] = r
        pad = max_blocks - len(r)
        if pad:
            tables[b, len(r):] = rng.choice(free, size=pad) if free.size else 0
    return tables, nb, used, pool


def _poison_mask(cfg, lens, tables, nb):
    """bool [nb, 16]: True for every slot that holds no cached token before this step."""
    holds = np.zeros((nb, BLOCK_SIZE), dtype=bool)
    for b, n in enumerate(lens):
        n_cached = int(n) - 1
        for j in range(blocks_for(n_cached)):
            cnt = min(BLOCK_SIZE, n_cached - j * BLOCK_SIZE)
            holds[tables[b, j], :cnt] = True
    return ~holds


def make_workload(name_or_cfg, device="cpu", seed=None, **overrides):
    """Build one workload on ``device`` (a config name or a DecodeConfig)."""
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if overrides:
        cfg = DecodeConfig(**{**cfg.__dict__, **overrides})
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    lens = sample_lengths(cfg, rng)
    tables, nb, used, _ = build_tables(cfg, lens, rng)
    B, Hq, Hkv, D = cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    qdt, cdt, sdt = TORCH_DTYPE[cfg.q_dtype], TORCH_DTYPE[cfg.cache_dtype], TORCH_DTYPE[cfg.src_dtype]

    query = _randn((B, Hq, D), cfg.value_std, qdt, gen, device)
    key_new = _randn((B, Hkv, D), cfg.value_std, sdt, gen, device)
    value_new = _randn((B, Hkv, D), cfg.value_std, sdt, gen, device)
    slots = np.array([slot_of(tables[b], int(lens[b]) - 1) if lens[b] > 0 else -1 for b in range(B)],
                     dtype=np.int64)
    poison = torch.from_numpy(_poison_mask(cfg, lens, tables, nb)).to(device)

    k_scale = v_scale = fill_key = fill_value = fill_slots = None
    if cfg.cache_dtype == "fp8_e4m3":
        key_cache = torch.full((nb, BLOCK_SIZE, Hkv, D), NAN_BITS["fp8_e4m3"], dtype=torch.uint8, device=device)
        value_cache = torch.full_like(key_cache, NAN_BITS["fp8_e4m3"])
        k_scale = torch.full((nb, BLOCK_SIZE), float("nan"), dtype=torch.float32, device=device)
        v_scale = torch.full_like(k_scale, float("nan"))
        # Every cached token once: shared prefix blocks are listed by their first holder only.
        seen = set()
        fill = []
        for b in range(B):
            for t in range(int(lens[b]) - 1):
                s = slot_of(tables[b], t)
                if s not in seen:
                    seen.add(s)
                    fill.append(s)
        fill_slots = torch.tensor(fill, dtype=torch.int64, device=device)
        fill_key = _randn((len(fill), Hkv, D), cfg.value_std, sdt, gen, device)
        fill_value = _randn((len(fill), Hkv, D), cfg.value_std, sdt, gen, device)
    else:
        rows = _rows_per_chunk(BLOCK_SIZE * Hkv * D)
        key_cache = _randn((nb, BLOCK_SIZE, Hkv, D), cfg.value_std, cdt, gen, device, rows)
        value_cache = _randn((nb, BLOCK_SIZE, Hkv, D), cfg.value_std, cdt, gen, device, rows)
        nan = NAN_BITS[cfg.cache_dtype]
        nan = nan - 0x10000 if nan >= 0x8000 else nan
        for cache in (key_cache, value_cache):
            bits = cache.view(torch.int16)
            bits.masked_fill_(poison[:, :, None, None].expand_as(bits), nan)

    return Workload(
        cfg=cfg, query=query, key_cache=key_cache, value_cache=value_cache,
        k_scale=k_scale, v_scale=v_scale,
        block_tables=torch.from_numpy(tables).to(device),
        context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        slot_mapping=torch.from_numpy(slots).to(device),
        key_new=key_new, value_new=value_new,
        fill_key=fill_key, fill_value=fill_value, fill_slots=fill_slots,
        lens_np=lens, tables_np=tables, num_blocks=nb, used_blocks=used,
    )


def bits_np(t):
    """Host numpy view of a tensor's bit patterns (uint16 for 16-bit types, uint8 for codes)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    return t.numpy()
