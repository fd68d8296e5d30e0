"""GPU parity of the matrix-core product (df11_matmul) and of decompressing
a weight stored in MFMA tile order, through the C ABI.

The product's reference is the oracle's float64 y = x W^T on the original
row-major W (oracle.linear); the bound is the float32 summation bound
gamma_n = 1.01 * in_features * 2^-24 * sum |x w| per output (every BF16 x
BF16 product is exact in float32; in_features additions in float32 in some
order).  Decompression must give back W's bits exactly.

Method: GeekNews, "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan
LLM menjadi 70% ukurannya", sections "Dekompresi yang disesuaikan untuk
inferensi GPU" and "Opini Hacker News" (a GEMM that decompresses each tile).
"""

import sys

import numpy as np
import pytest

import oracle
from entropy_decoding_df11_amd import df11, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    return torch


def _note(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _u16(t):
    import torch
    return t.detach().reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)


def _weights(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return workloads.f32_to_bf16_bits(rng.standard_normal(n) * 0.02)
    if kind == "student_t":
        return workloads.f32_to_bf16_bits(rng.standard_t(5, n) * 0.015)
    if kind == "stress_tuned":  # codes of up to ~29 bits through the LUT hierarchy
        return workloads.gen_stress(seed=seed, n=n)
    if kind == "zeros":
        return np.zeros(n, np.uint16)
    if kind == "integers":  # small integers: every sum exact, so y must equal the oracle exactly
        return workloads.f32_to_bf16_bits(rng.integers(-8, 9, n).astype(np.float64))
    raise ValueError(kind)


def _tokens(t, c, seed, integers=False):
    rng = np.random.default_rng(seed)
    x = rng.integers(-4, 5, t * c).astype(np.float64) if integers else rng.standard_normal(t * c) * 0.5
    return workloads.f32_to_bf16_bits(x).reshape(t, c)


def _bound(xb, w, rows, cols):
    xa = np.abs(oracle.bf16_to_f64(xb).reshape(-1, cols))
    wa = np.abs(oracle.bf16_to_f64(w).reshape(rows, cols))
    return 1.01 * cols * 2.0 ** -24 * (xa @ wa.T)


def _device_x(torch, xb):
    return torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)).to("cuda").view(torch.bfloat16)


# (64, 32) and (64, 96) have an odd number of k-steps per panel and take
# the chunk-by-chunk stores; the others go back in whole lines (pair-rounds).
# "zeros" (1-bit codes) gives groups of 2048 chunks, more pair-rounds than
# the sign/mantissa registers prefetch.
@pytest.mark.parametrize("rows,cols", [(64, 32), (64, 96), (128, 1024), (192, 4096), (64, 14336), (1024, 4096)])
@pytest.mark.parametrize("kind", ["normal", "stress_tuned", "zeros"])
def test_tiled_decompress_is_row_major(torch_cuda, rows, cols, kind):
    torch = torch_cuda
    _note(f"tiled decompress {kind} {rows}x{cols}")
    w = _weights(kind, rows * cols, rows + cols)
    t = df11.compress(w, shape=(rows, cols), layout="mfma_tiles")
    out = torch.full((rows, cols), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    t.decompress(out=out)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(out), w)


def test_tiled_decompress_batch_mixed_and_full_block(torch_cuda):
    """Batched decompression of tile-ordered streams: a batch mixing an odd
    k-step count (chunk-by-chunk stores for the whole launch) with even ones,
    then the full-size per-weight block in MFMA tile order (whole-line
    stores), each weight bit-exact in row-major order."""
    torch = torch_cuda
    _note("tiled decompress: mixed batch")
    shapes = [(128, 1024), (64, 96), (192, 4096)]
    ws = [_weights("normal", r * c, r + c) for r, c in shapes]
    ts = [df11.compress(w, shape=s, layout="mfma_tiles") for w, s in zip(ws, shapes)]
    outs = [torch.full(s, 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16) for s in shapes]
    df11.decompress_batch(ts, outs)
    df11.decompress_batch([ts[0], ts[2]], [outs[0], outs[2]])  # (every stream paired)
    torch.cuda.synchronize()
    for w, o in zip(ws, outs):
        assert np.array_equal(_u16(o), w)
    _note("tiled decompress: full-size per-weight block")
    flat, views = workloads.gen_block()
    blk = df11.compress_block([(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views],
                              codebook="per_weight", layout="mfma_tiles")
    scratch = torch.full((blk.n_elements,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    blk.decompress(scratch=scratch)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(scratch), flat)


@pytest.mark.parametrize("bits,gpw", [(10, 2), (12, 2), (11, 1), (11, 4)])
def test_tiled_decompress_table_widths_and_group_counts(torch_cuda, bits, gpw):
    """The whole-line decompression at every decode-table width and every
    number of groups per workgroup, bit-exact."""
    torch = torch_cuda
    _note(f"tiled decompress bits={bits} gpw={gpw}")
    r, c = 1024, 4096
    w = _weights("student_t", r * c, 95)
    t = df11.compress(w, shape=(r, c), layout="mfma_tiles", decode_table_bits=bits)
    t.set_groups_per_workgroup(gpw)
    out = torch.full((r, c), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    t.decompress(out=out)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(out), w)


def test_tiled_streams_with_the_derived_decode_table(torch_cuda):
    """Tile-ordered streams launched with the page's arrays alone (the
    first-level table derived in LDS, whose space precedes the whole-line
    stage): decompression, single and batched, bit-exact; the matrix-core
    product at one and twenty tokens within the float32 bound."""
    torch = torch_cuda
    shapes = [(1024, 4096), (64, 96), (192, 128)]
    ws = [_weights("stress_tuned" if i == 0 else "normal", r * c, 90 + i) for i, (r, c) in enumerate(shapes)]
    ts = [df11.compress(w, shape=s, layout="mfma_tiles") for w, s in zip(ws, shapes)]
    for t in ts:
        t.use_decode_table(False)
    _note("tiled, derived table: decompress")
    for w, t, s in zip(ws, ts, shapes):
        out = torch.full(s, 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        t.decompress(out=out)
        torch.cuda.synchronize()
        assert np.array_equal(_u16(out), w), s
    _note("tiled, derived table: batched decompress")
    outs = [torch.full(s, 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16) for s in shapes]
    df11.decompress_batch([ts[0], ts[2]], [outs[0], outs[2]])
    torch.cuda.synchronize()
    assert np.array_equal(_u16(outs[0]), ws[0]) and np.array_equal(_u16(outs[2]), ws[2])
    for n_tokens in (1, 20):
        _note(f"tiled, derived table: matmul tokens={n_tokens}")
        r, c = shapes[0]
        xb = _tokens(n_tokens, c, 91 + n_tokens)
        y = ts[0].matmul(_device_x(torch, xb))
        torch.cuda.synchronize()
        err = np.abs(y.cpu().numpy().astype(np.float64) - oracle.linear(oracle.encode(ws[0]), xb, r))
        assert np.all(err <= _bound(xb, ws[0], r, c)), float(err.max())


MATMUL_CASES = [  # (weights, rows, cols)
    ("normal", 64, 32),          # one panel of one k-step: groups span many panels
    ("normal", 128, 1024),       # groups across panel edges
    ("student_t", 192, 4096),
    ("stress_tuned", 64, 14336),  # one long panel; codes through the LUT hierarchy
    ("zeros", 128, 512),          # one exponent: y is exactly zero
]


@pytest.mark.parametrize("n_tokens", [1, 3, 16, 17, 33, 64, 65, 130])
@pytest.mark.parametrize("kind,rows,cols", MATMUL_CASES)
def test_matmul_matches_oracle(torch_cuda, kind, rows, cols, n_tokens):
    torch = torch_cuda
    _note(f"matmul {kind} {rows}x{cols} tokens={n_tokens}")
    w = _weights(kind, rows * cols, 7 + rows)
    xb = _tokens(n_tokens, cols, n_tokens + cols)
    t = df11.compress(w, shape=(rows, cols), layout="mfma_tiles")
    ref = oracle.linear(oracle.encode(w), xb, rows)
    bound = _bound(xb, w, rows, cols)
    x = _device_x(torch, xb)
    for _ in range(2):  # y is overwritten on every call
        y = t.matmul(x)
        torch.cuda.synchronize()
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= bound), (float(err.max()), float((err - bound).max()))


def test_matmul_exact_on_integers_and_accumulate(torch_cuda):
    """Small integer weights and tokens: every partial sum is an integer below
    2^24, so y equals the oracle exactly whatever the summation order; the
    accumulating entry point adds to what y holds."""
    torch = torch_cuda
    rows, cols, n_tokens = 256, 2048, 40
    w = _weights("integers", rows * cols, 1)
    xb = _tokens(n_tokens, cols, 2, integers=True)
    t = df11.compress(w, shape=(rows, cols), layout="mfma_tiles")
    ref = oracle.linear(oracle.encode(w), xb, rows)
    x = _device_x(torch, xb)
    y = t.matmul(x)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)
    t.matmul(x, out=y, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), 2 * ref)


def test_matmul_one_hot_tokens_return_columns(torch_cuda):
    """Token t one-hot at column c gives y[t] = W[:, c] exactly (a transposed
    or misplaced operand fails)."""
    torch = torch_cuda
    rows, cols = 192, 1024
    w = _weights("normal", rows * cols, 5)
    cs = np.random.default_rng(9).choice(cols, 37, replace=False)
    xb = np.zeros((cs.size, cols), np.uint16)
    xb[np.arange(cs.size), cs] = 0x3F80  # 1.0
    t = df11.compress(w, shape=(rows, cols), layout="mfma_tiles")
    y = t.matmul(_device_x(torch, xb))
    torch.cuda.synchronize()
    wf = oracle.bf16_to_f64(w).reshape(rows, cols)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), wf[:, cs].T)


@pytest.mark.parametrize("name", ["gate_proj", "down_proj"])
@pytest.mark.parametrize("n_tokens", [16, 256, 4096])
def test_matmul_full_size_block_matrix(torch_cuda, name, n_tokens):
    """The Llama-3-8B block's gate_proj (14336 x 4096) and down_proj (4096 x
    14336) at full size: every output row against the oracle for a sample of
    the tokens (all of them up to 16)."""
    torch = torch_cuda
    flat, views = workloads.gen_block()
    (off, (rows, cols)), = [(o, shp) for nm, o, shp in views if nm == name]
    w = np.ascontiguousarray(flat[off:off + rows * cols])
    del flat
    _note(f"matmul full size {name} {rows}x{cols} tokens={n_tokens}")
    xb = _tokens(n_tokens, cols, n_tokens)
    t = df11.compress(w, shape=(rows, cols), layout="mfma_tiles")
    y = t.matmul(_device_x(torch, xb))
    torch.cuda.synchronize()
    sample = np.arange(n_tokens) if n_tokens <= 16 else np.sort(
        np.random.default_rng(n_tokens).choice(n_tokens, 24, replace=False))
    ref = oracle.linear(oracle.encode(w), xb[sample], rows)
    bound = _bound(xb[sample], w, rows, cols)
    got = y.cpu().numpy()[sample].astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= bound), (float(err.max()), float((err - bound).max()))
    assert np.all(np.isfinite(y.cpu().numpy()))


@pytest.mark.parametrize("n_tokens", [1, 16, 40])
def test_matmul_batch_matches_oracle(torch_cuda, n_tokens):
    """Several products in one launch (df11_matmul_batch): shapes of a
    block's projections scaled down, two of them sharing one x, an empty
    weight skipped; then accumulating into the outputs."""
    torch = torch_cuda
    _note(f"matmul batch tokens={n_tokens}")
    shapes = [(256, 1024), (64, 1024), (64, 1024), (0, 1024), (512, 2048), (128, 4096)]
    ws, ts, xs, refs, bounds = [], [], [], [], []
    x_by_cols = {}
    for i, (r, c) in enumerate(shapes):
        w = _weights("student_t" if i % 2 else "normal", r * c, 40 + i)
        if c not in x_by_cols:
            x_by_cols[c] = _tokens(n_tokens, c, c + n_tokens)
        xb = x_by_cols[c]
        ws.append(w)
        ts.append(df11.compress(w, shape=(r, c), layout="mfma_tiles"))
        xs.append(_device_x(torch, xb))
        refs.append(oracle.linear(oracle.encode(w), xb, r) if r else np.zeros((n_tokens, 0)))
        bounds.append(_bound(xb, w, r, c) if r else np.zeros((n_tokens, 0)))
    xs[2] = xs[1]  # the same x for two weights
    ys = df11.matmul_batch(ts, xs)
    torch.cuda.synchronize()
    for y, ref, bound in zip(ys, refs, bounds):
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= bound), (float(err.max()), float((err - bound).max()))
    df11.matmul_batch(ts, xs, outs=ys, accumulate=True)
    torch.cuda.synchronize()
    for y, ref, bound in zip(ys, refs, bounds):
        err = np.abs(y.cpu().numpy().astype(np.float64) - 2 * ref)
        assert np.all(err <= 2 * bound), (float(err.max()), float((err - 2 * bound).max()))


@pytest.fixture(scope="module")
def full_block(torch_cuda):
    """The Llama-3-8B block's seven matrices: original bits, shape, the
    tile-ordered DF11 stream on the GPU and the oracle's encoding."""
    flat, views = workloads.gen_block()
    items = []
    for nm, off, (r, c) in views:
        w = np.ascontiguousarray(flat[off:off + r * c])
        items.append((nm, w, r, c, df11.compress(w, shape=(r, c), layout="mfma_tiles"), oracle.encode(w)))
    del flat
    return items


@pytest.mark.parametrize("n_tokens", [1, 17, 40])
def test_matmul_batch_of_one_matches_oracle(torch_cuda, n_tokens):
    """A batch holding one product (alone, or beside an empty weight) takes
    the one-stream kernel; its output, then accumulated once more, against
    the oracle."""
    torch = torch_cuda
    _note(f"matmul batch of one, tokens={n_tokens}")
    r, c = 1024, 4096
    w = _weights("normal", r * c, 77)
    t = df11.compress(w, shape=(r, c), layout="mfma_tiles")
    empty = df11.compress(np.zeros(0, np.uint16), shape=(0, 1024), layout="mfma_tiles")
    xb = _tokens(n_tokens, c, 78)
    x = _device_x(torch, xb)
    ref = oracle.linear(oracle.encode(w), xb, r)
    bound = _bound(xb, w, r, c)
    for tensors, xs in (([t], [x]), ([empty, t], [_device_x(torch, _tokens(n_tokens, 1024, 79)), x])):
        ys = df11.matmul_batch(tensors, xs)
        y = ys[-1]
        torch.cuda.synchronize()
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= bound), (float(err.max()), float((err - bound).max()))
        df11.matmul_batch(tensors, xs, outs=ys, accumulate=True)
        torch.cuda.synchronize()
        err = np.abs(y.cpu().numpy().astype(np.float64) - 2 * ref)
        assert np.all(err <= 2 * bound), (float(err.max()), float((err - 2 * bound).max()))


@pytest.mark.parametrize("n_tokens", [1, 2, 8, 16])
def test_matmul_batch_full_block(torch_cuda, full_block, n_tokens):
    """The whole block's seven products in one launch, every output against
    the oracle.  Up to 8 tokens each stream sweeps fixed ranges over most of
    its super-groups and deals the rest out with its work counters; at 16
    only fixed ranges run.  Launched twice in a row (the second time
    accumulating), the counters must be zero after each launch."""
    torch = torch_cuda
    _note(f"matmul batch: full block, {n_tokens} tokens")
    ts = [it[4] for it in full_block]
    xbs = [_tokens(n_tokens, c, r + n_tokens) for _, _, r, c, _, _ in full_block]
    xs = [_device_x(torch, xb) for xb in xbs]
    refs = [oracle.linear(enc, xb, r) for (_, _, r, _, _, enc), xb in zip(full_block, xbs)]
    bounds = [_bound(xb, w, r, c) for (_, w, r, c, _, _), xb in zip(full_block, xbs)]
    ys = df11.matmul_batch(ts, xs)
    torch.cuda.synchronize()
    for t in ts:
        assert not t._schedule.cpu().numpy().any()
    for y, ref, bound in zip(ys, refs, bounds):
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= bound), (float(err.max()), float((err - bound).max()))
    df11.matmul_batch(ts, xs, outs=ys, accumulate=True)
    torch.cuda.synchronize()
    for t in ts:
        assert not t._schedule.cpu().numpy().any()
    for y, ref, bound in zip(ys, refs, bounds):
        err = np.abs(y.cpu().numpy().astype(np.float64) - 2 * ref)
        assert np.all(err <= 2 * bound), (float(err.max()), float((err - 2 * bound).max()))


def test_matmul_batch_same_tensor_twice(torch_cuda, full_block):
    """One tensor named twice in a batch at one token: the two entries share
    work counters, so the launch sweeps fixed ranges only; both outputs must
    match the oracle and the counters stay zero."""
    torch = torch_cuda
    _note("matmul batch: gate_proj twice, 1 token")
    nm, w, r, c, t, enc = next(it for it in full_block if it[0] == "gate_proj")
    xb = _tokens(1, c, 7)
    x = _device_x(torch, xb)
    ys = df11.matmul_batch([t, t], [x, x])
    torch.cuda.synchronize()
    ref, bound = oracle.linear(enc, xb, r), _bound(xb, w, r, c)
    for y in ys:
        err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
        assert np.all(err <= bound)
    assert not t._schedule.cpu().numpy().any()


@pytest.mark.parametrize("cap", [270, 97])
def test_matmul_batch_full_block_capped_grid(torch_cuda, full_block, cap):
    """The block's seven products at one token on a capped grid (cap
    workgroups shared by the seven streams: 2 to 72 each, one work counter
    each, long fixed ranges): the fixed ranges and the dealt rest still
    cover every super-group once, and the counters are left zero."""
    torch = torch_cuda
    _note(f"matmul batch: full block, 1 token, {cap} workgroups")
    ts = [it[4] for it in full_block]
    xbs = [_tokens(1, c, r + 3) for _, _, r, c, _, _ in full_block]
    xs = [_device_x(torch, xb) for xb in xbs]
    try:
        for t in ts:
            t.set_max_workgroups(cap)
        ys = df11.matmul_batch(ts, xs)
        torch.cuda.synchronize()
    finally:
        for t in ts:
            t.set_max_workgroups(0)
    for t in ts:
        assert not t._schedule.cpu().numpy().any()
    for y, (_, w, r, c, _, enc), xb in zip(ys, full_block, xbs):
        err = np.abs(y.cpu().numpy().astype(np.float64) - oracle.linear(enc, xb, r))
        assert np.all(err <= _bound(xb, w, r, c))
