"""Seeded synthetic workloads with the shapes of the pages' decode settings.

Recipe (all values from torch generators seeded per workload):
* q and bfloat16 cache rows: N(0, 1) in float32, rounded to bfloat16;
* paged caches: 64-token pages drawn from a shuffled pool (``randperm``), so
  consecutive logical pages of a request sit at random physical places; table
  slots past a request's last page are 0 and never read;
* DSA top-k: per query token, ``topk`` distinct logical tokens of the request,
  encoded as page_block*64 + offset through the request's block table; each
  slot is set to -1 with probability ``invalid_frac``;
* peaked top-k rows: slot 0 holds the query's own (newest) token r and
  q[b, 0, h] = 0.25 * k_r for every head (exact in bfloat16);
* FP8 cache: per token, N(0, 1) latent values quantised per 1x128 tile with
  scale = amax / 448 and float8_e4m3fn codes (torch's round-to-nearest cast
  after clamping to +-448); RoPE values N(0, 1) rounded to bfloat16; record =
  [512 codes | 4 float32 scales | 64 bfloat16], little-endian.

Large tensors are drawn on ``device`` with a generator for that device, so the
values depend on the device the workload is built for; index structures are
always drawn on the CPU.
"""

from dataclasses import dataclass, field
from typing import Optional
import math

import torch

D_QK = 576
D_V = 512
BLOCK = 64
FP8_RECORD = 656

CONFIG_NAMES = {
    1: 'tiny dense b=2 s_q=1 h_q=16 L={200,256} fp32 out',
    2: 'DeepSeek-V3 dense b=64 s_q=1 h_q=128 L=4096',
    3: 'var-len spec decode b=128 s_q=2 causal h_q=128 L~U[1,8192]',
    4: 'sparse top-k b=64 s_q=1 h_q=128 topk=2048 pool 32768/seq 5% invalid',
    5: 'FP8 cache b=32 s_q=1 h_q=128 L=16384',
}


@dataclass
class Workload:
    name: str
    batch: int
    s_q: int
    h_q: int
    causal: bool
    topk: int                       # 0 = dense
    kv_format: str                  # 'bf16' | 'fp8'
    out_dtype: str                  # 'bf16' | 'fp32'
    softmax_scale: float
    q: torch.Tensor                 # bf16 [B, S, H, 576]
    kv: torch.Tensor                # bf16 [NB, 64, 1, 576] or uint8 [NB, 64, 1, 656]
    block_table: torch.Tensor       # int32 [B, max_blocks]
    cache_seqlens: torch.Tensor     # int32 [B]
    indices: Optional[torch.Tensor] = None   # int32 [B, S, topk]
    meta: dict = field(default_factory=dict)
    topk_length: Optional[torch.Tensor] = None   # int32 [B, S] or None (all topk entries)
    attn_sink: Optional[torch.Tensor] = None     # float32 [H] or None

    @property
    def num_blocks(self):
        return int(self.kv.shape[0])

    @property
    def max_blocks_per_seq(self):
        return int(self.block_table.shape[1])

    def to(self, device):
        kw = {}
        for k in ('q', 'kv', 'block_table', 'cache_seqlens', 'indices', 'topk_length', 'attn_sink'):
            v = getattr(self, k)
            kw[k] = None if v is None else v.to(device)
        return Workload(self.name, self.batch, self.s_q, self.h_q, self.causal, self.topk,
                        self.kv_format, self.out_dtype, self.softmax_scale, meta=dict(self.meta), **kw)


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn_bf16(shape, g, device, chunk_rows=4096):
    """N(0,1) float32 rounded to bfloat16, drawn in chunks along dim 0."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    n0 = shape[0]
    for s in range(0, n0, chunk_rows):
        e = min(n0, s + chunk_rows)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device).to(torch.bfloat16)
    return out


def _paged_table(seqlens, max_blocks, g_cpu, pool_blocks=None):
    """Shuffled pool of pages; returns (num_blocks, table int32 [B, max_blocks])."""
    need = [max(1, math.ceil(int(L) / BLOCK)) if int(L) > 0 else 0 for L in seqlens]
    total = sum(need)
    nb = total if pool_blocks is None else int(pool_blocks)
    assert nb >= total
    perm = torch.randperm(nb, generator=g_cpu)
    table = torch.zeros((len(seqlens), max_blocks), dtype=torch.int32)
    o = 0
    for b, k in enumerate(need):
        assert k <= max_blocks
        table[b, :k] = perm[o:o + k].to(torch.int32)
        o += k
    return nb, table


def make_dense(batch, s_q, h_q, seqlens, *, causal=False, seed=0, device='cpu', out_dtype='bf16',
               max_blocks=None, pool_blocks=None, softmax_scale=None, name='dense'):
    g_cpu = _gen('cpu', seed)
    seqlens = [int(x) for x in seqlens]
    assert len(seqlens) == batch
    if max_blocks is None:
        max_blocks = max(1, max(math.ceil(L / BLOCK) for L in seqlens))
    nb, table = _paged_table(seqlens, max_blocks, g_cpu, pool_blocks)
    g = _gen(device, seed + 7919)
    q = _randn_bf16((batch, s_q, h_q, D_QK), g, device, chunk_rows=64)
    kv = _randn_bf16((max(nb, 1), BLOCK, 1, D_QK), g, device, chunk_rows=1024)
    return Workload(name, batch, s_q, h_q, causal, 0, 'bf16', out_dtype,
                    softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D_QK),
                    q, kv, table.to(device), torch.tensor(seqlens, dtype=torch.int32, device=device))


def encode_fp8_records(x, rope_bf16):
    """x float32 [n, 512], rope bf16 [n, 64] -> uint8 records [n, 656]."""
    n = x.shape[0]
    tiles = x.view(n, 4, 128)
    amax = tiles.abs().amax(dim=2)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.float32)
    codes = (tiles / scale[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(n, 512)
    rec = torch.empty((n, FP8_RECORD), dtype=torch.uint8, device=x.device)
    rec[:, :512] = codes.view(torch.uint8)
    rec[:, 512:528] = scale.contiguous().view(torch.uint8).view(n, 16)
    rec[:, 528:] = rope_bf16.contiguous().view(torch.uint8).view(n, 128)
    return rec


def make_fp8_dense(batch, s_q, h_q, seqlens, *, causal=False, seed=0, device='cpu', out_dtype='bf16',
                   max_blocks=None, pool_blocks=None, softmax_scale=None, name='fp8'):
    g_cpu = _gen('cpu', seed)
    seqlens = [int(x) for x in seqlens]
    if max_blocks is None:
        max_blocks = max(1, max(math.ceil(L / BLOCK) for L in seqlens))
    nb, table = _paged_table(seqlens, max_blocks, g_cpu, pool_blocks)
    g = _gen(device, seed + 7919)
    q = _randn_bf16((batch, s_q, h_q, D_QK), g, device, chunk_rows=64)
    nb = max(nb, 1)
    kv = torch.empty((nb, BLOCK, 1, FP8_RECORD), dtype=torch.uint8, device=device)
    step = 256
    for s in range(0, nb, step):
        e = min(nb, s + step)
        n = (e - s) * BLOCK
        x = torch.randn((n, D_QK), generator=g, device=device)
        rec = encode_fp8_records(x[:, :512].contiguous(), x[:, 512:].to(torch.bfloat16))
        kv[s:e] = rec.view(e - s, BLOCK, 1, FP8_RECORD)
    return Workload(name, batch, s_q, h_q, causal, 0, 'fp8', out_dtype,
                    softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D_QK),
                    q, kv, table.to(device), torch.tensor(seqlens, dtype=torch.int32, device=device))


def make_sparse(batch, s_q, h_q, *, pool_tokens_per_seq, topk, invalid_frac=0.05, seed=0, device='cpu',
                out_dtype='bf16', peaked=False, order='asis', softmax_scale=None, kv_format='bf16',
                name='sparse'):
    """DSA-style top-k decode inputs.  ``order``: 'asis' | 'self_last' | 'perm'."""
    g_cpu = _gen('cpu', seed)
    blocks_per_seq = math.ceil(pool_tokens_per_seq / BLOCK)
    seqlens = [pool_tokens_per_seq] * batch
    nb, table = _paged_table(seqlens, blocks_per_seq, g_cpu)
    n_tok = pool_tokens_per_seq
    assert topk <= n_tok
    idx = torch.empty((batch, s_q, topk), dtype=torch.int64)
    for b in range(batch):
        for i in range(s_q):
            if peaked:
                self_tok = n_tok - s_q + i
                rest = torch.randperm(n_tok - 1, generator=g_cpu)[:topk - 1]
                rest = torch.where(rest >= self_tok, rest + 1, rest)
                sel = torch.cat([torch.tensor([self_tok]), rest])
            else:
                sel = torch.randperm(n_tok, generator=g_cpu)[:topk]
            phys = table[b].to(torch.int64)[sel // BLOCK] * BLOCK + sel % BLOCK
            drop = torch.rand(topk, generator=g_cpu) < invalid_frac
            if peaked:
                drop[0] = False
            phys = torch.where(drop, torch.full_like(phys, -1), phys)
            if order == 'self_last':
                phys = torch.roll(phys, -1)
            elif order == 'perm':
                phys = phys[torch.randperm(topk, generator=g_cpu)]
            idx[b, i] = phys
    g = _gen(device, seed + 7919)
    if kv_format == 'bf16':
        kv = _randn_bf16((nb, BLOCK, 1, D_QK), g, device, chunk_rows=1024)
    else:
        kv = torch.empty((nb, BLOCK, 1, FP8_RECORD), dtype=torch.uint8, device=device)
        for s in range(0, nb, 256):
            e = min(nb, s + 256)
            x = torch.randn(((e - s) * BLOCK, D_QK), generator=g, device=device)
            kv[s:e] = encode_fp8_records(x[:, :512].contiguous(),
                                         x[:, 512:].to(torch.bfloat16)).view(e - s, BLOCK, 1, FP8_RECORD)
    q = _randn_bf16((batch, s_q, h_q, D_QK), g, device, chunk_rows=64)
    indices = idx.to(torch.int32).to(device)
    if peaked:
        assert kv_format == 'bf16'
        flat = kv.view(-1, D_QK)
        for b in range(batch):
            for i in range(s_q):
                self_tok = n_tok - s_q + i
                r = int(table[b, self_tok // BLOCK]) * BLOCK + self_tok % BLOCK
                q[b, i, :, :] = (flat[r].to(torch.float32) * 0.25).to(torch.bfloat16)[None, :]
    return Workload(name, batch, s_q, h_q, False, topk, kv_format, out_dtype,
                    softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D_QK),
                    q, kv, table.to(device), torch.tensor(seqlens, dtype=torch.int32, device=device),
                    indices=indices, meta={'peaked': peaked, 'order': order})


V41_RECORD = 528
FP4_RECORD = 288


def encode_v41_records(x):
    """float32 [n, 512] -> uint8 [n, 528]: per group of 32 values the smallest power of two 2^(e-127) with
    amax / 2^(e-127) <= 448 (e = 127 for an all-zero group), the codes float8_e4m3fn(x / 2^(e-127)) (torch's
    round-to-nearest cast after clamping to +-448), then the 16 exponent bytes e."""
    n = x.shape[0]
    g = x.view(n, 16, 32)
    amax = g.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax / 448.0)), torch.zeros_like(amax)) + 127
    e = e.clamp(0, 254)
    scale = torch.pow(2.0, e - 127)
    # the log2 above can land one short: move up until every value fits
    e = torch.where(amax / scale > 448.0, e + 1, e)
    scale = torch.pow(2.0, e - 127)
    codes = (g / scale[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, 512)
    return torch.cat([codes, e.to(torch.uint8)], dim=1)


def make_v41_sparse(batch, s_q, h_q, *, pool_tokens_per_seq, topk, invalid_frac=0.0, seed=0, device='cpu',
                    name='v41_sparse'):
    """Top-k decode inputs over the 528-byte records of the 512-wide head (RoPE dims quantised too): q is
    [batch, s_q, h_q, 512]; cache values N(0, 1) encoded by ``encode_v41_records``; indices as for
    ``make_sparse``."""
    w = make_sparse(batch, s_q, h_q, pool_tokens_per_seq=pool_tokens_per_seq, topk=topk, invalid_frac=invalid_frac,
                    seed=seed, device=device, name=name)
    nb = w.num_blocks
    g = _gen(device, seed + 104729)
    kv = torch.empty((nb, BLOCK, 1, V41_RECORD), dtype=torch.uint8, device=device)
    for s in range(0, nb, 256):
        e = min(nb, s + 256)
        x = torch.randn(((e - s) * BLOCK, 512), generator=g, device=device)
        kv[s:e] = encode_v41_records(x).view(e - s, BLOCK, 1, V41_RECORD)
    w.kv = kv
    w.kv_format = 'fp8_528'
    w.q = _randn_bf16((batch, s_q, h_q, 512), g, device, chunk_rows=64)
    w.softmax_scale = 1.0 / math.sqrt(512)
    return w


E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)   # codes 0..7 (bit 3 is the sign)


def encode_fp4_records(x):
    """float32 [n, 512] -> uint8 [n, 288]: per group of 16 values the scale float8_e4m3fn(amax / 6) (torch's
    round-to-nearest cast; 1 for an all-zero group), each value x / scale rounded to the nearest e2m1
    magnitude (ties to the smaller code) with its sign, two codes per byte with the even index in the low
    nibble, then the 32 scale bytes."""
    n = x.shape[0]
    g = x.view(n, 32, 16)
    amax = g.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 6.0, torch.ones_like(amax)).to(torch.float8_e4m3fn)
    s = scale.to(torch.float32)
    s = torch.where(s > 0, s, torch.ones_like(s))
    y = (g / s[..., None]).reshape(n, 512)
    mags = torch.tensor(E2M1_MAGNITUDES, device=x.device)
    code = (y.abs()[..., None] - mags).abs().argmin(dim=-1)          # first minimum: ties to the smaller code
    code = code + 8 * ((y < 0) & (code > 0)).to(code.dtype)
    code = code.to(torch.uint8)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return torch.cat([packed, scale.view(torch.uint8)], dim=1)


def make_fp4_sparse(batch, s_q, h_q, *, pool_tokens_per_seq, topk, invalid_frac=0.0, seed=0, device='cpu',
                    name='fp4_sparse'):
    """Top-k decode inputs over the 288-byte FP4 records of the 512-wide head: q is [batch, s_q, h_q, 512];
    cache values N(0, 1) encoded by ``encode_fp4_records``; indices as for ``make_sparse``."""
    w = make_sparse(batch, s_q, h_q, pool_tokens_per_seq=pool_tokens_per_seq, topk=topk, invalid_frac=invalid_frac,
                    seed=seed, device=device, name=name)
    nb = w.num_blocks
    g = _gen(device, seed + 130363)
    kv = torch.empty((nb, BLOCK, 1, FP4_RECORD), dtype=torch.uint8, device=device)
    for s in range(0, nb, 256):
        e = min(nb, s + 256)
        x = torch.randn(((e - s) * BLOCK, 512), generator=g, device=device)
        kv[s:e] = encode_fp4_records(x).view(e - s, BLOCK, 1, FP4_RECORD)
    w.kv = kv
    w.kv_format = 'fp4_288'
    w.q = _randn_bf16((batch, s_q, h_q, 512), g, device, chunk_rows=64)
    w.softmax_scale = 1.0 / math.sqrt(512)
    return w


def make_fp8_sparse(topk, device='cpu', seed=None, batch=128, s_q=2, h_q=128):
    """The FP8 sparse decode shape the pages quote for the H800 kernel: 128
    requests, 2 query tokens each, 128 heads, top-k 2048 or 32768 over a
    656-byte record cache.  Every slot is valid; each request holds
    max(32768, 2 topk) cached tokens to choose from."""
    seed = 2000 + topk if seed is None else seed
    pool = max(32768, 2 * topk)
    return make_sparse(batch, s_q, h_q, pool_tokens_per_seq=pool, topk=topk, invalid_frac=0.0, seed=seed,
                       device=device, kv_format='fp8', name=f'fp8_sparse_b{batch}_s{s_q}_topk{topk}')


@dataclass
class PrefillWorkload:
    """Sparse prefill inputs: a flat, unpaged cache of s_kv rows."""
    name: str
    s_q: int
    h_q: int
    topk: int
    kv_format: str                  # 'bf16' | 'fp8'
    softmax_scale: float
    q: torch.Tensor                 # bf16 [s_q, h_q, 576]
    kv: torch.Tensor                # bf16 [s_kv, 1, 576] or uint8 [s_kv, 1, 656]
    indices: torch.Tensor           # int32 [s_q, 1, topk]
    topk_length: Optional[torch.Tensor] = None   # int32 [s_q]
    attn_sink: Optional[torch.Tensor] = None     # float32 [h_q]

    @property
    def s_kv(self):
        return int(self.kv.shape[0])


def make_sparse_prefill(s_q, s_kv, h_q, topk, *, invalid_frac=0.0, seed=0, device='cpu', kv_format='bf16',
                        name='sparse_prefill'):
    """Query row s picks ``topk`` distinct rows of the first min(s_kv, s_kv - s_q + 1 + s) cache rows (the
    rows a causal prefill chunk at the end of the sequence can see), each entry -1 with probability
    ``invalid_frac``; q and cache values as for decode."""
    g_cpu = _gen('cpu', seed)
    idx = torch.empty((s_q, 1, topk), dtype=torch.int64)
    for s in range(s_q):
        vis = min(s_kv, s_kv - s_q + 1 + s)
        assert vis >= topk
        idx[s, 0] = torch.randperm(vis, generator=g_cpu)[:topk]
    drop = torch.rand((s_q, 1, topk), generator=g_cpu) < invalid_frac
    idx = torch.where(drop, torch.full_like(idx, -1), idx)
    g = _gen(device, seed + 7919)
    if kv_format == 'bf16':
        kv = _randn_bf16((s_kv, 1, D_QK), g, device, chunk_rows=4096)
    else:
        x = torch.randn((s_kv, D_QK), generator=g, device=device)
        kv = encode_fp8_records(x[:, :512].contiguous(), x[:, 512:].to(torch.bfloat16)).view(s_kv, 1, FP8_RECORD)
    q = _randn_bf16((s_q, h_q, D_QK), g, device, chunk_rows=64)
    return PrefillWorkload(name, s_q, h_q, topk, kv_format, 1.0 / math.sqrt(D_QK), q, kv,
                           idx.to(torch.int32).to(device))


def make_config(i, device='cpu', seed=None, **kw):
    """The five workloads, with seed 1000 + i unless given."""
    seed = 1000 + i if seed is None else seed
    if i == 1:
        return make_dense(2, 1, 16, [200, 256], seed=seed, device=device, out_dtype='fp32',
                          max_blocks=4, pool_blocks=8, name='config1', **kw)
    if i == 2:
        return make_dense(64, 1, 128, [4096] * 64, seed=seed, device=device, max_blocks=64,
                          pool_blocks=4096, name='config2', **kw)
    if i == 3:
        g = _gen('cpu', seed + 17)
        lens = torch.randint(1, 8193, (128,), generator=g).tolist()
        return make_dense(128, 2, 128, lens, causal=True, seed=seed, device=device, max_blocks=128,
                          name='config3', **kw)
    if i == 4:
        return make_sparse(64, 1, 128, pool_tokens_per_seq=32768, topk=2048, invalid_frac=0.05,
                           seed=seed, device=device, name='config4', **kw)
    if i == 5:
        return make_fp8_dense(32, 1, 128, [16384] * 32, seed=seed, device=device, max_blocks=256,
                              pool_blocks=8192, name='config5', **kw)
    raise ValueError(i)
