"""Decompress transformer blocks just before use, or fuse the decode into
each projection.

GeekNews, "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan LLM
menjadi 70% ukurannya", sections "Dekompresi yang disesuaikan untuk inferensi
GPU" and "Dekompresi per transformer block": weights stay compressed in HBM,
each block is decompressed into a scratch buffer right before its forward
pass and discarded after it.  BlockDecoder does that on the caller's stream,
or, with overlap=True, decodes block i + 1 on a side stream into the other of
two scratch buffers while the caller computes with block i.
"""

from __future__ import annotations

from typing import Dict, Iterator, List, Optional, Sequence, Tuple, Union

from .df11 import DF11Block, DF11BlockBatch

Block = Union[DF11Block, DF11BlockBatch]


class BlockDecoder:
    """Iterate over compressed blocks, yielding (index, {name: bf16 weight})
    with every weight already decoded in the caller's stream order.

    By default each block is decoded on the caller's stream right before it
    is yielded.  With overlap=True, block i + 1 is decoded on a side stream
    while the caller enqueues block i's work; an event recorded on the
    caller's stream when it asks for the next block marks block i's scratch
    buffer free again.  Either way the weights of block i are valid until the
    caller asks for block i + 2 (two scratch buffers alternate), so the caller
    must finish enqueuing block i's work before advancing.

    Overlap rarely pays on one GPU: the decoder's persistent grid fills every
    CU and is bound by HBM, and so are the caller's GEMMs at small batch.
    decode_workgroups caps the workgroups of an overlapped decode (0: fill the
    GPU) so the caller's kernels find room beside it.
    """

    def __init__(self, blocks: Sequence[Block], device="cuda", overlap: bool = False, decode_workgroups: int = 0):
        import torch
        self.blocks = list(blocks)
        self.device = torch.device(device)
        self.overlap = overlap
        self.decode_workgroups = decode_workgroups
        n = max((b.n_elements for b in self.blocks), default=0)
        self._scratch = [torch.empty(max(n, 1), dtype=torch.bfloat16, device=self.device) for _ in range(2)]
        # Default priority: streams of different priorities are avoided.
        self._side = torch.cuda.Stream(self.device) if overlap else None

    def __len__(self) -> int:
        return len(self.blocks)

    def _decode(self, i: int, stream, cap: int = 0) -> Dict:
        b = self.blocks[i]
        if cap:
            b.set_max_workgroups(cap)
        try:
            return b.decompress(scratch=self._scratch[i % 2], stream=stream)
        finally:
            if cap:
                b.set_max_workgroups(0)

    def __iter__(self) -> Iterator[Tuple[int, Dict]]:
        import torch
        if not self.blocks:
            return
        main = torch.cuda.current_stream(self.device)
        if not self.overlap:
            for i in range(len(self.blocks)):
                yield i, self._decode(i, main)
            return
        side = self._side
        free = [None, None]      # event: the caller has finished with scratch[k]
        ready = [None] * len(self.blocks)

        def launch(i: int):
            side.wait_stream(main) if free[i % 2] is None else side.wait_event(free[i % 2])
            views = self._decode(i, side, self.decode_workgroups)
            ev = torch.cuda.Event()
            ev.record(side)
            ready[i] = ev
            return views

        pending = launch(0)
        for i in range(len(self.blocks)):
            views = pending
            main.wait_event(ready[i])
            if i + 1 < len(self.blocks):
                pending = launch(i + 1)
            yield i, views
            # the caller has enqueued block i's work on `main`
            ev = torch.cuda.Event()
            ev.record(main)
            free[i % 2] = ev


def block_forward(x, w: Dict, eps: float = 1e-5):
    """A synthetic Llama-style block forward on BF16 weights (no attention
    mixing, which needs no weights): RMS-normed projections q, k, v and o
    with a residual, then the gated MLP (gate, up, down) with a residual.
    Used to show the decompressed weights in use; shapes follow the weights."""
    import torch
    import torch.nn.functional as F

    def rms(h):
        return h * torch.rsqrt(h.float().pow(2).mean(-1, keepdim=True) + eps).to(h.dtype)

    h = rms(x)
    q = F.linear(h, w["q_proj"])
    k = F.linear(h, w["k_proj"])
    v = F.linear(h, w["v_proj"])
    rep = q.shape[-1] // k.shape[-1]
    a = q + (k * v).repeat_interleave(rep, dim=-1)
    x = x + F.linear(a, w["o_proj"])
    h = rms(x)
    x = x + F.linear(F.silu(F.linear(h, w["gate_proj"])) * F.linear(h, w["up_proj"]), w["down_proj"])
    return x


# Token counts up to which the fused products beat decoding the block first
# and calling torch's GEMM (Llama-3-8B block, measured): the matrix-core
# product sweeps the stream once per 64 tokens, the row-order product takes
# up to 8 tokens.
FUSED_MAX_TOKENS_TILES = 64
FUSED_MAX_TOKENS_ROWS = 8


def fused_block_forward(x, blk: DF11BlockBatch, eps: float = 1e-5, scratch=None):
    """block_forward with each projection's decode fused into its product:
    blk holds one DF11 stream per weight, and no weight is ever decompressed
    to HBM.  Weights in MFMA tile order (compress_block(..., layout=
    "mfma_tiles")) go through the matrix-core product (df11_matmul_batch:
    q, k and v in one launch, o, gate and up in one, down), for any token
    count; weights in row order through the row-order product
    (df11_linear_batch / df11_linear), for 1..8 tokens.  The products
    accumulate in float32 and are rounded to x's dtype, like the resident
    path's outputs, but in another order, so the last bits can differ from
    block_forward's.  Above FUSED_MAX_TOKENS_TILES (tile order) or
    FUSED_MAX_TOKENS_ROWS (row order) tokens the block is decoded (into
    scratch, if given) and block_forward runs on it: there the GEMM's reuse
    of W across tokens outweighs the decode."""
    import torch
    import torch.nn.functional as F
    from .df11 import linear_batch, matmul_batch

    w = {nm: t for (nm, _, _), t in zip(blk.views, blk.tensors)}
    tiled = all(t.tile_cols for t in blk.tensors)
    if x.shape[0] > (FUSED_MAX_TOKENS_TILES if tiled else FUSED_MAX_TOKENS_ROWS):
        return block_forward(x, blk.decompress(scratch=scratch), eps)

    def products(names_, xin, outs):
        ts = [w[nm] for nm in names_]
        if tiled:
            matmul_batch(ts, [xin] * len(ts), outs=outs, accumulate=True)
        elif len(ts) == 1:
            ts[0].linear(xin, out=outs[0], accumulate=True)
        else:
            linear_batch(ts, xin, outs=outs, accumulate=True)

    def rms(h):
        return h * torch.rsqrt(h.float().pow(2).mean(-1, keepdim=True) + eps).to(h.dtype)

    # The seven products accumulate into views of one buffer, zeroed by one
    # fill, rather than each zeroing its own output (df11_linear_acc).
    names = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")
    tokens = x.shape[0]
    sizes = [tokens * w[nm].shape[0] for nm in names]
    buf = torch.zeros(sum(sizes), dtype=torch.float32, device=x.device)
    y = {nm: part.view(tokens, w[nm].shape[0]) for nm, part in zip(names, torch.split(buf, sizes))}

    h = rms(x).contiguous()
    products(("q_proj", "k_proj", "v_proj"), h, [y["q_proj"], y["k_proj"], y["v_proj"]])
    q, k, v = (y[nm].to(x.dtype) for nm in ("q_proj", "k_proj", "v_proj"))
    rep = q.shape[-1] // k.shape[-1]
    a = q + (k * v).repeat_interleave(rep, dim=-1)
    products(("o_proj",), a.contiguous(), [y["o_proj"]])
    x = x + y["o_proj"].to(x.dtype)
    h = rms(x).contiguous()
    products(("gate_proj", "up_proj"), h, [y["gate_proj"], y["up_proj"]])
    g, u = (y[nm].to(x.dtype) for nm in ("gate_proj", "up_proj"))
    products(("down_proj",), (F.silu(g) * u).contiguous(), [y["down_proj"]])
    x = x + y["down_proj"].to(x.dtype)
    return x


def fused_model_forward(x, blocks: Sequence[DF11BlockBatch]):
    """fused_block_forward over every block in order."""
    for blk in blocks:
        x = fused_block_forward(x, blk)
    return x


class CapturedForward:
    """A forward captured once into a HIP graph and replayed.

    At a few tokens a forward is many small launches (per block: the
    products, or decodes and products, plus norms, activations and residual
    adds); a graph replay issues all of them at once.  forward(x) must run on
    the current stream and keep its shapes: this wrapper runs it `warmup`
    times on a side stream (so that launch-time queries, torch's allocations
    and the decode tables' caches are settled), then captures one call into a
    graph that reads a static copy of x and writes a static output.
    __call__(x) copies x in, replays, and returns that output, which the next
    call overwrites.  Every DF11 kernel launches without memsets or host
    synchronisation and leaves its work counters zero, so replays are
    independent.  The forward's own buffers (weights, BlockDecoder scratch)
    must stay alive as long as this object."""

    def __init__(self, forward, example_x, warmup: int = 2):
        import torch
        self._forward = forward
        self.x = example_x.clone()
        side = torch.cuda.Stream(self.x.device)
        side.wait_stream(torch.cuda.current_stream(self.x.device))
        with torch.cuda.stream(side):
            for _ in range(warmup):
                forward(self.x)
        torch.cuda.current_stream(self.x.device).wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.y = forward(self.x)

    def __call__(self, x):
        if x.shape != self.x.shape or x.dtype != self.x.dtype:
            raise ValueError("a captured forward takes inputs of the captured shape and dtype")
        self.x.copy_(x)
        self.graph.replay()
        return self.y


def model_forward(x, blocks: Union[BlockDecoder, List[Dict]]):
    """Run block_forward over every block in order, taking the weights from a
    BlockDecoder (compressed) or from a list of dicts (resident BF16)."""
    items = iter(blocks) if isinstance(blocks, BlockDecoder) else enumerate(blocks)
    for _, w in items:
        x = block_forward(x, w)
    return x
