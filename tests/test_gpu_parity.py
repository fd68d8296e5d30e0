"""GPU parity: the gfx950 decoder through the C ABI against the original BF16
bits (the exact result, "identik bit demi bit") and against the oracle.

Method: GeekNews, "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan
LLM menjadi 70% ukurannya", sections "Kernel GPU 2 tahap dan metadata bantu"
and "Dekompresi per transformer block".
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


def _to_u16(t):
    import torch
    return t.detach().reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)


def _gpu_decode(torch, w, bits=12, shape=None, fill=0x5A5A):
    t = df11.compress(w, shape=shape or (w.size,), decode_table_bits=bits)
    out = torch.full(t.shape, fill, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    t.decompress(out=out)
    torch.cuda.synchronize()
    return _to_u16(out), t


def _fib(n):
    f = [1, 1]
    while len(f) < n:
        f.append(f[-1] + f[-2])
    return f[:n]


def _case(kind, size, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return workloads.f32_to_bf16_bits(rng.standard_normal(size) * 0.02)
    if kind == "student_t":
        return workloads.f32_to_bf16_bits(rng.standard_t(5, size) * 0.015)
    if kind == "uniform_bits":  # flat: uniform sign/mantissa, exponents uniform over 60 values
        e = rng.integers(90, 150, size)
        return workloads.f32_to_bf16_bits(np.ldexp(1.0 + rng.integers(0, 128, size) / 128.0, e - 127)
                                          * rng.choice([-1.0, 1.0], size))
    if kind == "zeros":
        return np.zeros(size, np.uint16)
    if kind == "fib_chain":  # codes up to 29 bits, 4 LUT levels
        p = np.array(_fib(30)[::-1], np.float64)
        e = rng.choice(np.arange(90, 120), size, p=p / p.sum())
        return workloads.f32_to_bf16_bits(np.ldexp(1.0 + rng.integers(0, 128, size) / 128.0, e - 127)
                                          * rng.choice([-1.0, 1.0], size))
    if kind == "stress_tuned":  # a 1-bit code and 28+ bit codes
        return workloads.gen_stress(seed=seed, n=size)
    if kind == "stress_literal":  # 8 LUTs
        return workloads.gen_stress(seed=seed, n=size, kind="literal")
    raise ValueError(kind)


SMALL_CASES = [(k, n) for k in ("normal", "student_t", "uniform_bits", "zeros", "fib_chain", "stress_tuned",
                                "stress_literal")
               for n in (1, 2, 7, 64, 1000, 6403, 12345, 100003, (1 << 20) + 17)]


@pytest.mark.parametrize("kind,size", SMALL_CASES)
def test_small_cases_bitexact(torch_cuda, kind, size):
    w = _case(kind, size, seed=size % 97)
    _note(f"small kind={kind} size={size}")
    s = oracle.encode(w)
    ref = oracle.decode_treewalk(s)
    assert np.array_equal(ref, w)
    got, t = _gpu_decode(torch_cuda, w)
    assert np.array_equal(got, w), f"first mismatch at {int(np.argmax(got != w))}"


def _random_stream(rng):
    """A seeded random BF16 stream: a random length, and exponents from a
    random mix (a Gaussian of random scale, random-rate outliers and tiny
    values, or a random Zipf law over a random set of exponents), so that
    code lengths, LUT depths and the codes at group edges vary widely."""
    n = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(5000, 400_000)),
                        int(rng.integers(400_000, 3_000_000))]))
    if rng.random() < 0.5:
        v = rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 1)
        for scale in (1.0, 1e-6):
            k = rng.random(n) < 10.0 ** rng.uniform(-5, -2)
            v[k] = rng.standard_normal(int(k.sum())) * scale
        return workloads.f32_to_bf16_bits(v)
    used = rng.choice(np.arange(1, 240), size=int(rng.integers(2, 60)), replace=False)
    p = 1.0 / np.arange(1, used.size + 1) ** rng.uniform(0.5, 2.5)
    e = rng.choice(used, n, p=p / p.sum())
    return workloads.f32_to_bf16_bits(np.ldexp(1.0 + rng.integers(0, 128, n) / 128.0, e - 127)
                                      * rng.choice([-1.0, 1.0], n))


def test_random_streams_bit_exact(torch_cuda):
    """100 seeded random streams (lengths 1..3M, random exponent laws)
    decoded bit for bit by the Huffman decoder and by the rANS decoder."""
    torch = torch_cuda
    rng = np.random.default_rng(2024)
    for i in range(100):
        w = _random_stream(rng)
        _note(f"random stream {i} n={w.size}")
        got, _ = _gpu_decode(torch, w, bits=11)
        assert np.array_equal(got, w), (i, w.size, int(np.argmax(got != w)))
        r = df11.rans_compress(w, shape=(w.size,))
        out = torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        r.decompress(out=out)
        torch.cuda.synchronize()
        assert np.array_equal(_to_u16(out), w), ("rans", i, w.size)


def test_random_shapes_linear(torch_cuda):
    """The fused product on 24 seeded random shapes (in_features a multiple
    of 8 from 512 up, 1..8 tokens) within the float32 bound of the oracle."""
    torch = torch_cuda
    rng = np.random.default_rng(77)
    for i in range(24):
        in_f = 8 * int(rng.integers(64, 1200))
        out_f = int(rng.integers(1, max(2, 600_000 // in_f)))
        T = int(rng.integers(1, 9))
        w = workloads.f32_to_bf16_bits(rng.standard_normal(out_f * in_f) * 0.02)
        _note(f"random linear {i} {out_f}x{in_f} T={T}")
        t = df11.compress(w, shape=(out_f, in_f))
        _check_linear(torch, t, w, _tokens(T, in_f, 100 + i), out_f, in_f, calls=1)


@pytest.mark.parametrize("bits", [10, 11, 12])
@pytest.mark.parametrize("kind", ["normal", "fib_chain", "stress_tuned", "uniform_bits"])
def test_decode_table_widths_agree(torch_cuda, bits, kind):
    w = _case(kind, 300001, seed=bits)
    _note(f"widths kind={kind} bits={bits}")
    got, _ = _gpu_decode(torch_cuda, w, bits=bits)
    assert np.array_equal(got, w)


@pytest.mark.parametrize("name", ["single_1024x1024", "proj_4096x4096_outliers", "mlp_14336x4096_t5"])
def test_workload_parity(torch_cuda, workload, name):
    w = workload(name)
    _note(f"workload {name} n={w.size}")
    got, t = _gpu_decode(torch_cuda, w)
    assert np.array_equal(got, w)
    if w.size <= (1 << 24):
        s = oracle.encode(w)
        assert np.array_equal(oracle.decode_treewalk(s), got)


def test_block_workload_full_size(torch_cuda):
    """The Llama-3-8B-shaped block as one stream with a shared codebook,
    decoded in one launch into one scratch buffer; sampled groups checked
    against the oracle's own encode and tree-walk decode."""
    torch = torch_cuda
    flat, views = workloads.gen_block()
    _note(f"block n={flat.size}")
    blk = df11.compress_block([(name, flat[off:off + r * c].reshape(r, c)) for name, off, (r, c) in views])
    scratch = torch.empty(flat.size + 1000, dtype=torch.bfloat16, device="cuda")
    out = blk.decompress(scratch=scratch)
    torch.cuda.synchronize()
    got = _to_u16(scratch[: flat.size])
    assert np.array_equal(got, flat)
    for name, off, (r, c) in views:
        assert tuple(out[name].shape) == (r, c)
        assert out[name].data_ptr() == scratch.data_ptr() + 2 * off
    s = oracle.encode(flat)
    rng = np.random.default_rng(7)
    ref = np.zeros_like(flat)
    for g in sorted(set(rng.integers(0, s["n_groups"], 200).tolist()) | {0, s["n_groups"] - 1}):
        oracle.decode_groups(s, g, g + 1, ref)
        lo, hi = int(s["out_pos"][g]), int(s["out_pos"][g + 1])
        assert np.array_equal(ref[lo:hi], got[lo:hi]), g


def test_stress_workload_full_size(torch_cuda):
    w = workloads.gen_stress()
    _note(f"stress n={w.size}")
    got, t = _gpu_decode(torch_cuda, w)
    assert np.array_equal(got, w)
    assert t.header.max_len >= 28


def test_empty_and_repeat_and_side_stream(torch_cuda):
    torch = torch_cuda
    t = df11.compress(np.zeros(0, np.uint16), shape=(0,))
    out = t.decompress()
    assert out.numel() == 0
    w = _case("normal", 77777, 3)
    t = df11.compress(w, shape=(w.size,))
    side = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(side):
        for _ in range(3):
            outs.append(t.decompress(stream=side))
    side.synchronize()
    for o in outs:
        assert np.array_equal(_to_u16(o), w)


@pytest.mark.parametrize("dynamic", [True, False])
def test_schedule_repeat_launches_and_counter_reset(torch_cuda, dynamic):
    """Dynamic load balancing hands super-groups out from device counters;
    every launch must leave them zero, and back-to-back launches must all be
    bit-exact.  The stream (64M weights with ~6-bit exponent codes, ~23K
    groups) is long enough for the dynamic schedule at two groups per
    workgroup; one group per workgroup, four, the static schedule and capped
    grids (with every count of work counters, and below one workgroup per
    CU) must give the same bytes."""
    torch = torch_cuda
    w = _case("uniform_bits", 64 << 20, 11)
    _note(f"schedule dynamic={dynamic}")
    t = df11.compress(w, shape=(w.size,), decode_table_bits=11)
    assert t.header.n_groups >= 2 * 12 * 768
    t.set_dynamic_schedule(dynamic)
    for gpw in (2, 1, 4):
        t.set_groups_per_workgroup(gpw)
        outs = []
        for _ in range(3):
            out = torch.full(t.shape, 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            outs.append(t.decompress(out=out))
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(_to_u16(o), w), gpw
        assert not t._schedule.cpu().numpy().any()
        del outs
    t.set_groups_per_workgroup(2)
    # (672, 576, 480 and 270 workgroups take 7, 6, 5 and 3 work counters,
    # which do not divide the 8 XCDs; 100 takes 2, 7 and 1 one)
    for cap in (672, 576, 480, 270, 100, 7, 1):
        t.set_max_workgroups(cap)
        out = torch.full(t.shape, 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        t.decompress(out=out)
        torch.cuda.synchronize()
        assert np.array_equal(_to_u16(out), w), cap
        assert not t._schedule.cpu().numpy().any()
    t.set_max_workgroups(0)


@pytest.mark.parametrize("bits", [0, 10, 11, 12])
@pytest.mark.parametrize("kind", ["normal", "fib_chain", "stress_tuned", "stress_literal", "uniform_bits", "zeros"])
def test_derived_decode_table(torch_cuda, kind, bits):
    """A stream given with the page's arrays alone (no decode table): every
    workgroup derives the first-level table in LDS from the LUTs and
    CodeLengths (bits 0: the default width)."""
    torch = torch_cuda
    w = _case(kind, 300001, 5 + bits)
    _note(f"derived table {kind} bits={bits}")
    t = df11.compress(w, shape=(w.size,), decode_table_bits=bits or 11)
    t.use_decode_table(False)
    t.device_stream().decode_table_bits = bits
    out = torch.full(t.shape, 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    t.decompress(out=out)
    torch.cuda.synchronize()
    assert np.array_equal(_to_u16(out), w)


def test_derived_decode_table_full_block_batch_and_linear(torch_cuda):
    """The derived table on the full-size block, in a batched launch and in
    the fused product."""
    torch = torch_cuda
    flat, views = workloads.gen_block()
    _note("derived table: full block")
    blk = df11.compress_block([(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views])
    blk.tensor.use_decode_table(False)
    scratch = torch.empty(blk.n_elements, dtype=torch.bfloat16, device="cuda")
    blk.decompress(scratch=scratch)
    torch.cuda.synchronize()
    assert np.array_equal(_to_u16(scratch), flat)
    del blk, scratch
    _note("derived table: batch of three")
    ws = [_case(k, n, 9) for k, n in (("normal", 100003), ("fib_chain", 7), ("stress_tuned", 654321))]
    ts = [df11.compress(w, shape=(w.size,)) for w in ws]
    for t in ts[:2]:
        t.use_decode_table(False)
    outs = [torch.empty(w.size, dtype=torch.bfloat16, device="cuda") for w in ws]
    df11.decompress_batch(ts, outs)
    torch.cuda.synchronize()
    for w, o in zip(ws, outs):
        assert np.array_equal(_to_u16(o), w)
    _note("derived table: fused product")
    wm = _case("stress_tuned", 256 * 1024, 3)
    t = df11.compress(wm, shape=(256, 1024))
    t.use_decode_table(False)
    _check_linear(torch, t, wm, _tokens(3, 1024, 4), 256, 1024)


def test_launches_on_two_streams_are_serialised(torch_cuda):
    """Launches of one tensor share its work counters, so the binding orders
    a launch after the tensor's previous one when that went to another
    stream.  Alternating two streams with no synchronisation of the caller's
    own must leave every output bit-exact and the counters zero."""
    torch = torch_cuda
    w = _case("uniform_bits", 64 << 20, 12)
    _note("two streams, one tensor")
    t = df11.compress(w, shape=(w.size,), decode_table_bits=11)
    assert t.header.n_groups >= 2 * 12 * 768  # long enough for the dynamic schedule
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full(t.shape, 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16) for _ in range(4)]
    torch.cuda.synchronize()  # the fills ran on the default stream
    for i, o in enumerate(outs):
        t.decompress(out=o, stream=streams[i % 2])
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(_to_u16(o), w)
    assert not t._schedule.cpu().numpy().any()


@pytest.mark.parametrize("bits", [10, 11, 12])
def test_timed_entry_point_matches(torch_cuda, bits):
    """df11_decompress_timed decodes the same bytes and records the kernel's
    own start and end in the caller's events."""
    torch = torch_cuda
    w = _case("normal", 1_500_003, bits)
    _note(f"timed bits={bits}")
    t = df11.compress(w, shape=(w.size,), decode_table_bits=bits)
    out = torch.full(t.shape, 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t.decompress(out=out, events=ev)
    torch.cuda.synchronize()
    assert np.array_equal(_to_u16(out), w)
    assert ev[0].elapsed_time(ev[1]) > 0


def test_batch_of_independent_streams(torch_cuda):
    """One launch decodes streams with different codebooks, sizes (empty and
    single-element ones included) and code-length profiles."""
    torch = torch_cuda
    cases = [("normal", 77_777, 1), ("fib_chain", 300_001, 2), ("uniform_bits", 1_000_003, 3), ("normal", 1, 4),
             ("stress_tuned", 2_000_000, 5), ("student_t", 0, 6), ("stress_literal", 123_457, 7)]
    _note("batch of independent streams")
    ws = [_case(k, n, seed) if n else np.zeros(0, np.uint16) for k, n, seed in cases]
    ts = [df11.compress(w, shape=(w.size,), decode_table_bits=11) for w in ws]
    outs = [torch.full((max(w.size, 1),), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)[: w.size]
            for w in ws]
    df11.decompress_batch(ts, outs)
    torch.cuda.synchronize()
    for (kind, n, _), w, o in zip(cases, ws, outs):
        assert np.array_equal(_to_u16(o), w), kind


def test_block_with_per_weight_codebooks(torch_cuda):
    """The Llama-3-8B-shaped block with a codebook per weight, decoded by one
    batched launch into one scratch buffer; then the same block with the
    dynamic schedule off."""
    torch = torch_cuda
    flat, views = workloads.gen_block()
    _note(f"block per-weight codebooks n={flat.size}")
    blk = df11.compress_block([(name, flat[off:off + r * c].reshape(r, c)) for name, off, (r, c) in views],
                              codebook="per_weight")
    assert len(blk.tensors) == len(views)
    scratch = torch.empty(blk.n_elements, dtype=torch.bfloat16, device="cuda")
    for dynamic in (True, False):
        for t in blk.tensors:
            t.set_dynamic_schedule(dynamic)
        scratch.view(torch.int16).fill_(0x5A5A)
        out = blk.decompress(scratch=scratch)
        torch.cuda.synchronize()
        for name, off, (r, c) in views:
            assert np.array_equal(_to_u16(out[name]), flat[off:off + r * c]), (name, dynamic)
        for t in blk.tensors:
            assert not t._schedule.cpu().numpy().any()
    # The timed batch entry point decodes the same bytes and records the
    # batched kernel's own start and end.
    scratch.view(torch.int16).fill_(0x5A5A)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    out = blk.decompress(scratch=scratch, events=ev)
    torch.cuda.synchronize()
    for name, off, (r, c) in views:
        assert np.array_equal(_to_u16(out[name]), flat[off:off + r * c]), name
    assert ev[0].elapsed_time(ev[1]) > 0


def test_lm_head_single_stream_full_size(torch_cuda):
    """An LM-head / embedding-sized matrix (128256x4096, 525M weights) as one
    stream, decoded unbatched; the original bits are the exact result."""
    w = workloads.gen_lm_head()
    _note(f"lm head n={w.size}")
    got, t = _gpu_decode(torch_cuda, w, bits=11)
    assert np.array_equal(got, w)
    assert t.header.n_elements == 128256 * 4096


SMALL_BLOCK = [("q_proj", (1024, 1024)), ("k_proj", (256, 1024)), ("v_proj", (256, 1024)),
               ("o_proj", (1024, 1024)), ("gate_proj", (3584, 1024)), ("up_proj", (3584, 1024)),
               ("down_proj", (1024, 3584))]


@pytest.mark.parametrize("overlap,cap", [(False, 0), (True, 0), (True, 24)])
@pytest.mark.parametrize("codebook", ["shared", "per_weight"])
def test_block_decoder_forward_matches_resident_weights(torch_cuda, overlap, cap, codebook):
    """A synthetic 6-block forward whose weights are decompressed block by
    block (in line, or block i + 1 on a side stream while block i computes,
    with the decode's grid capped or not) gives the same bits as the forward
    on the original BF16 weights."""
    torch = torch_cuda
    from entropy_decoding_df11_amd import runtime
    _note(f"block decoder overlap={overlap} cap={cap} codebook={codebook}")
    blocks, resident = [], []
    for b in range(6):
        flat, views = workloads.gen_block(seed=100 + b, shapes=SMALL_BLOCK)
        parts = [(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views]
        blocks.append(df11.compress_block(parts, codebook=codebook))
        resident.append({nm: torch.from_numpy(a.astype(np.int16)).to("cuda").view(torch.bfloat16)
                         for nm, a in parts})
    x = workloads.f32_to_bf16_bits(np.random.default_rng(9).standard_normal(64 * 1024) * 0.5).reshape(64, 1024)
    x = torch.from_numpy(x.astype(np.int16)).to("cuda").view(torch.bfloat16)
    ref = runtime.model_forward(x, resident)
    pf = runtime.BlockDecoder(blocks, overlap=overlap, decode_workgroups=cap)
    for _ in range(2):  # the scratch buffers are reused across passes
        got = runtime.model_forward(x, pf)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


# ---------------------------------------------------------------------------
# Decode fused into the matrix product (df11_linear): y = x W^T
# ---------------------------------------------------------------------------

def _linear_bound(x_bits, w_bits, out_f, in_f):
    """Largest allowed |y_gpu - y_oracle| per output.  Every BF16 x BF16
    product is exact in float32, and the kernel adds the in_f products of
    an output in float32 in some order (lane, wave, LDS and global atomic
    sums).  With u = 2^-24 the error of any such order is at most
    gamma_n * sum |x w| with n = in_f additions, and gamma_n = n u / (1 - n u)
    < 1.01 n u for n u < 0.01."""
    xa = np.abs(oracle.bf16_to_f64(x_bits).reshape(-1, in_f))
    wa = np.abs(oracle.bf16_to_f64(w_bits).reshape(out_f, in_f))
    return 1.01 * in_f * 2.0 ** -24 * (xa @ wa.T)


def _tokens(n_tokens, in_f, seed):
    x = np.random.default_rng(seed).standard_normal(n_tokens * in_f) * 0.5
    return workloads.f32_to_bf16_bits(x).reshape(n_tokens, in_f)


def _check_linear(torch, t, w, x, out_f, in_f, calls=2):
    ref = oracle.linear(oracle.encode(w), x, out_f)
    bound = _linear_bound(x, w, out_f, in_f)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    for _ in range(calls):  # y is overwritten on every call
        y = t.linear(xd)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        assert got.shape == ref.shape
        err = np.abs(got - ref)
        assert np.all(err <= bound), (float(err.max()), float((err - bound).max()))


LINEAR_CASES = [  # (weights, out_features, in_features)
    ("normal", 300, 1024),        # ~50 groups; rows inside groups and across their edges
    ("student_t", 77, 4104),      # rows not a multiple of 512 long
    ("normal", 1000, 512),        # the shortest rows: several rows per group
    ("stress_tuned", 40, 14336),  # codes through the LUT hierarchy; rows longer than a group
    ("fib_chain", 129, 2048),     # 4 LUT levels
    ("zeros", 64, 1024),          # one exponent: y is exactly zero
]


@pytest.mark.parametrize("kind,out_f,in_f", LINEAR_CASES)
@pytest.mark.parametrize("n_tokens", [1, 2, 5, 8])
def test_linear_matches_oracle(torch_cuda, kind, out_f, in_f, n_tokens):
    torch = torch_cuda
    _note(f"linear {kind} {out_f}x{in_f} tokens={n_tokens}")
    w = _case(kind, out_f * in_f, 21)
    x = _tokens(n_tokens, in_f, n_tokens)
    t = df11.compress(w, shape=(out_f, in_f))
    _check_linear(torch, t, w, x, out_f, in_f)


@pytest.mark.parametrize("bits", [10, 12])
def test_linear_table_widths(torch_cuda, bits):
    torch = torch_cuda
    _note(f"linear bits={bits}")
    w = _case("student_t", 300 * 1024, 5)
    t = df11.compress(w, shape=(300, 1024), decode_table_bits=bits)
    _check_linear(torch, t, w, _tokens(4, 1024, 7), 300, 1024)


def test_linear_capped_grid_and_dynamic_schedule(torch_cuda):
    """With a grid of 3 or 7 workgroups the stream (~160 groups) runs on the
    dynamic schedule; the result must not change and the counters must be
    left at zero."""
    torch = torch_cuda
    w = _case("normal", 1000 * 1024, 8)
    t = df11.compress(w, shape=(1000, 1024))
    x = _tokens(3, 1024, 9)
    for cap in (3, 7):
        _note(f"linear cap={cap}")
        t.set_max_workgroups(cap)
        _check_linear(torch, t, w, x, 1000, 1024, calls=1)
        assert not t._schedule.cpu().numpy().any()
    t.set_max_workgroups(0)


def test_linear_argument_errors(torch_cuda):
    torch = torch_cuda
    w = _case("normal", 64 * 1024, 1)
    t = df11.compress(w, shape=(64, 1024))
    x = torch.zeros((9, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib_error()):
        t.linear(x)  # more tokens than the fused kernel takes
    with pytest.raises(ValueError):
        t.linear(torch.zeros((2, 1000), dtype=torch.bfloat16, device="cuda"))


def test_linear_accumulate(torch_cuda):
    """df11_linear_acc and df11_linear_batch_acc add x W^T to what the output
    holds: starting from a known y0, two calls give y0 + 2 x W^T within twice
    the float32 bound; without an output the binding refuses."""
    torch = torch_cuda
    in_f = 1024
    shapes = [(300, in_f), (77, in_f)]
    ws = [_case("normal", r * c, 60 + i) for i, (r, c) in enumerate(shapes)]
    ts = [df11.compress(w, shape=s) for w, s in zip(ws, shapes)]
    x = _tokens(3, in_f, 61)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    refs = [oracle.linear(oracle.encode(w), x, r) for w, (r, _) in zip(ws, shapes)]
    bounds = [_linear_bound(x, w, r, c) for w, (r, c) in zip(ws, shapes)]
    y0s = [np.random.default_rng(i).standard_normal((3, r)).astype(np.float32) for i, (r, _) in enumerate(shapes)]

    def bound(y0, b):
        # 2 in_f + 1 float32 additions in any order: gamma_{2n+1} (|y0| + 2 sum |x w|),
        # where b = 1.01 in_f u sum |x w| is the one-call bound
        sum_abs = b / (1.01 * in_f * 2.0 ** -24)
        return 1.01 * (2 * in_f + 1) * 2.0 ** -24 * (np.abs(y0.astype(np.float64)) + 2 * sum_abs)

    # one matrix
    y = torch.from_numpy(y0s[0].copy()).to("cuda")
    for _ in range(2):
        ts[0].linear(xd, out=y, accumulate=True)
    torch.cuda.synchronize()
    err = np.abs(y.cpu().numpy().astype(np.float64) - (y0s[0] + 2 * refs[0]))
    assert np.all(err <= bound(y0s[0], bounds[0]))
    # a batch
    ys = [torch.from_numpy(v.copy()).to("cuda") for v in y0s]
    for _ in range(2):
        df11.linear_batch(ts, xd, outs=ys, accumulate=True)
    torch.cuda.synchronize()
    for got, y0, ref, b in zip(ys, y0s, refs, bounds):
        err = np.abs(got.cpu().numpy().astype(np.float64) - (y0 + 2 * ref))
        assert np.all(err <= bound(y0, b))
    with pytest.raises(ValueError):
        ts[0].linear(xd, accumulate=True)
    with pytest.raises(ValueError):
        df11.linear_batch(ts, xd, accumulate=True)


def test_same_stream_twice_in_one_batch(torch_cuda):
    """A batch that holds one tensor twice: both entries would use the same
    work counters, so the second runs the static schedule.  The grid is capped
    so that the first entry takes the dynamic schedule; both outputs must be
    exact (decode) or within the float32 bound (product), on two calls in a
    row, and the counters must be zero afterwards."""
    torch = torch_cuda
    out_f, in_f = 1024, 4096
    w = _case("normal", out_f * in_f, 17)
    t = df11.compress(w, shape=(out_f, in_f))
    t.set_max_workgroups(32)
    _note("same stream twice in one batch")
    x = _tokens(2, in_f, 9)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    ref = oracle.linear(oracle.encode(w), x, out_f)
    bound = _linear_bound(x, w, out_f, in_f)
    for _ in range(2):
        outs = [torch.full((w.size,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
                for _ in range(2)]
        df11.decompress_batch([t, t], outs)
        ys = df11.linear_batch([t, t], xd)
        torch.cuda.synchronize()
        for o in outs:
            assert np.array_equal(_to_u16(o), w)
        for y in ys:
            assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - ref) <= bound)
        assert not t._schedule.cpu().numpy().any()
    t.set_max_workgroups(0)


def test_outputs_on_another_device_are_rejected(torch_cuda):
    """Every entry point refuses an output (or x, or scratch) that is not on
    the weights' device before anything is launched."""
    torch = torch_cuda
    w = _case("normal", 64 * 1024, 1)
    t = df11.compress(w, shape=(64, 1024))
    x = torch.zeros((1, 1024), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        t.decompress(out=torch.empty((64, 1024), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        t.linear(x, out=torch.empty((1, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        t.linear(x.cpu())
    with pytest.raises(ValueError):
        df11.linear_batch([t, t], x, outs=[torch.empty((1, 64), dtype=torch.float32, device="cuda"),
                                           torch.empty((1, 64), dtype=torch.float32)])
    with pytest.raises(ValueError):
        df11.decompress_batch([t], [torch.empty(64 * 1024, dtype=torch.bfloat16)])
    r = df11.rans_compress(w, shape=(64, 1024))
    with pytest.raises(ValueError):
        r.decompress(out=torch.empty((64, 1024), dtype=torch.bfloat16))
    # Nothing was launched: a normal call still decodes exactly.
    assert np.array_equal(t.decompress().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1), w)


def _lib_error():
    from entropy_decoding_df11_amd import _lib
    return _lib.Df11Error


@pytest.mark.parametrize("name", ["gate_proj", "down_proj"])
def test_linear_full_size_block_matrix(torch_cuda, name):
    """Llama-3-8B-shaped gate_proj (14336 x 4096) and down_proj (4096 x
    14336), each its own stream, at 4 tokens: every output against the
    oracle."""
    torch = torch_cuda
    shapes = dict(workloads.LLAMA3_8B_BLOCK)
    out_f, in_f = shapes[name]
    flat, views = workloads.gen_block(seed=3)
    off = {nm: o for nm, o, _ in views}[name]
    w = np.ascontiguousarray(flat[off:off + out_f * in_f])
    del flat
    _note(f"linear full size {name} {out_f}x{in_f}")
    t = df11.compress(w, shape=(out_f, in_f))
    _check_linear(torch, t, w, _tokens(4, in_f, 11), out_f, in_f, calls=1)


# ---------------------------------------------------------------------------
# rANS exponent coder (df11_rans_decompress): bit-exact against the
# original weights, whose rANS stream the library encoder writes byte for
# byte as the oracle does (CPU tests)
# ---------------------------------------------------------------------------

RANS_SIZES = [1, 63, 64, 65, 511, 512, 513, 4097, 32767, 32768, 32769, 100_003, (1 << 20) + 17]


@pytest.mark.parametrize("kind", ["normal", "student_t", "uniform_bits", "zeros", "fib_chain", "stress_tuned",
                                  "stress_literal"])
def test_rans_decode_bit_exact(torch_cuda, kind):
    torch = torch_cuda
    for n in RANS_SIZES:
        _note(f"rans {kind} n={n}")
        w = _case(kind, n, 17)
        t = df11.rans_compress(w, shape=(n,))
        out = torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        t.decompress(out=out)
        torch.cuda.synchronize()
        assert np.array_equal(_to_u16(out), w), n


def test_rans_empty_stream(torch_cuda):
    torch = torch_cuda
    t = df11.rans_compress(np.zeros(0, np.uint16), shape=(0,))
    out = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    t.decompress(out=out)
    torch.cuda.synchronize()


def test_rans_full_size_block_repeat_and_timed(torch_cuda):
    """The Llama-3-8B-shaped block (218M weights) as one rANS stream:
    bit-exact on back-to-back launches and through the timed entry point."""
    torch = torch_cuda
    flat, _ = workloads.gen_block()
    _note("rans full-size block")
    t = df11.rans_compress(flat, shape=(flat.size,))
    out = torch.full((flat.size,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    for _ in range(2):
        t.decompress(out=out)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t.decompress(out=out, events=ev)
    torch.cuda.synchronize()
    assert np.array_equal(_to_u16(out), flat)
    assert ev[0].elapsed_time(ev[1]) > 0


# Segment counts at which the launch picks each workgroup shape on a 256-CU
# MI355X (14, 8, 10, 11, 12 and 13 waves); on another GPU they still check
# whatever shapes it picks.
RANS_SHAPE_SEGMENTS = [1, 9, 2049, 2561, 2817, 3073]


def test_rans_every_launch_shape(torch_cuda):
    """Streams sized to select every workgroup shape of the rANS decoder,
    each with a ragged last segment: bit-exact."""
    torch = torch_cuda
    seg = 64 * 512
    base = _case("normal", 1 << 22, 23)
    for n_seg in RANS_SHAPE_SEGMENTS:
        n = (n_seg - 1) * seg + 1000
        w = np.resize(base, n)
        _note(f"rans shape, {n_seg} segments")
        t = df11.rans_compress(w, shape=(n,))
        assert t.header.n_segments == n_seg
        out = torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        t.decompress(out=out)
        torch.cuda.synchronize()
        assert np.array_equal(_to_u16(out), w)
        del t, out


@pytest.mark.parametrize("n_tokens", [1, 3, 8])
def test_linear_batch_matches_oracle(torch_cuda, n_tokens):
    """q, k and v shaped matrices (different row counts, each its own
    stream) multiplying one x in one launch, each output within the float32
    bound of the oracle; an empty matrix in the batch is skipped."""
    torch = torch_cuda
    _note(f"linear batch tokens={n_tokens}")
    in_f = 1024
    shapes = [(300, in_f), (77, in_f), (128, in_f), (0, in_f)]
    ws = [_case("normal" if i % 2 == 0 else "student_t", r * c, 40 + i) for i, (r, c) in enumerate(shapes)]
    ts = [df11.compress(w, shape=s) for w, s in zip(ws, shapes)]
    x = _tokens(n_tokens, in_f, 5)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    for _ in range(2):
        ys = df11.linear_batch(ts, xd)
        torch.cuda.synchronize()
        for w, (r, c), y in zip(ws, shapes, ys):
            if r == 0:
                assert y.numel() == 0
                continue
            ref = oracle.linear(oracle.encode(w), x, r)
            err = np.abs(y.cpu().numpy().astype(np.float64) - ref)
            assert np.all(err <= _linear_bound(x, w, r, c))


def test_linear_batch_full_size_qkv(torch_cuda):
    """The Llama-3-8B q, k and v projections (4096, 1024 and 1024 rows of
    4096) in one launch at one token, against the oracle."""
    torch = torch_cuda
    flat, views = workloads.gen_block(seed=3)
    ws, shapes = [], []
    for nm, o, (r, c) in views[:3]:
        ws.append(np.ascontiguousarray(flat[o:o + r * c]))
        shapes.append((r, c))
    del flat
    _note("linear batch full-size qkv")
    ts = [df11.compress(w, shape=s) for w, s in zip(ws, shapes)]
    x = _tokens(1, 4096, 12)
    ys = df11.linear_batch(ts, torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16))
    torch.cuda.synchronize()
    for w, (r, c), y in zip(ws, shapes, ys):
        ref = oracle.linear(oracle.encode(w), x, r)
        assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - ref) <= _linear_bound(x, w, r, c))


@pytest.mark.parametrize("n_tokens,layout", [(1, "rows"), (4, "rows"), (8, "rows"), (1, "mfma_tiles"),
                                             (16, "mfma_tiles"), (64, "mfma_tiles"), (100, "mfma_tiles"),
                                             (20, "rows")])
def test_fused_block_forward_close_to_resident(torch_cuda, n_tokens, layout):
    """A block forward whose projections decode inside their products gives
    what the forward on the original BF16 weights gives, up to the order of
    the float32 sums (outputs rounded to bf16 either way): within 2% of the
    output's largest magnitude after one block."""
    torch = torch_cuda
    from entropy_decoding_df11_amd import runtime
    _note(f"fused block forward tokens={n_tokens} layout={layout}")
    flat, views = workloads.gen_block(seed=7, shapes=SMALL_BLOCK)
    parts = [(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views]
    blk = df11.compress_block(parts, codebook="per_weight", layout=layout)
    resident = {nm: torch.from_numpy(a.astype(np.int16)).to("cuda").view(torch.bfloat16) for nm, a in parts}
    x = workloads.f32_to_bf16_bits(np.random.default_rng(n_tokens).standard_normal(n_tokens * 1024) * 0.5)
    x = torch.from_numpy(x.astype(np.int16).reshape(n_tokens, 1024)).to("cuda").view(torch.bfloat16)
    ref = runtime.block_forward(x, resident).float()
    got = runtime.fused_block_forward(x, blk).float()
    torch.cuda.synchronize()
    assert got.shape == ref.shape
    assert float((got - ref).abs().max()) <= 0.02 * float(ref.abs().max())
    limit = runtime.FUSED_MAX_TOKENS_TILES if layout == "mfma_tiles" else runtime.FUSED_MAX_TOKENS_ROWS
    if n_tokens > limit:  # decoded first, then the resident path's own GEMMs: the same bits
        assert torch.equal(got, ref)


@pytest.mark.parametrize("path", ["resident", "inline", "fused", "fused_tiles"])
def test_captured_forward_replays_match_eager(torch_cuda, path):
    """A 3-block forward captured into a HIP graph (runtime.CapturedForward)
    and replayed on five inputs, with eager forwards and synchronisations
    between the replays: every replay gives the eager resident-weight
    forward's output, bit for bit on the resident and in-line decode paths,
    and within 5% of the output's largest magnitude on the fused path (its
    float32 sums run in another order)."""
    torch = torch_cuda
    from entropy_decoding_df11_amd import runtime
    _note(f"captured forward path={path}")
    resident, shared, per_weight = [], [], []
    for b in range(3):
        flat, views = workloads.gen_block(seed=200 + b, shapes=SMALL_BLOCK)
        parts = [(nm, flat[o:o + r * c].reshape(r, c)) for nm, o, (r, c) in views]
        resident.append({nm: torch.from_numpy(a.astype(np.int16)).to("cuda").view(torch.bfloat16)
                         for nm, a in parts})
        if path == "inline":
            shared.append(df11.compress_block(parts, codebook="shared"))
        if path.startswith("fused"):
            per_weight.append(df11.compress_block(parts, codebook="per_weight",
                                                  layout="mfma_tiles" if path == "fused_tiles" else "rows"))
    xs = []
    for i in range(5):
        xb = workloads.f32_to_bf16_bits(np.random.default_rng(30 + i).standard_normal(4 * 1024) * 0.5)
        xs.append(torch.from_numpy(xb.astype(np.int16).reshape(4, 1024)).to("cuda").view(torch.bfloat16))
    refs = [runtime.model_forward(x, resident).clone() for x in xs]
    if path == "resident":
        fwd = lambda x: runtime.model_forward(x, resident)  # noqa: E731
    elif path == "inline":
        decoder = runtime.BlockDecoder(shared)
        fwd = lambda x: runtime.model_forward(x, decoder)  # noqa: E731
    else:
        fwd = lambda x: runtime.fused_model_forward(x, per_weight)  # noqa: E731
    g = runtime.CapturedForward(fwd, xs[0])
    for i, x in enumerate(xs):
        got = g(x).clone()
        torch.cuda.synchronize()
        if path.startswith("fused"):
            err = float((got.float() - refs[i].float()).abs().max())
            assert err <= 0.05 * float(refs[i].float().abs().max()), (i, err)
        else:
            assert torch.equal(got.view(torch.int16), refs[i].view(torch.int16)), i
        fwd(xs[(i + 2) % len(xs)])  # eager work between replays
        torch.cuda.synchronize()


def test_linear_lm_head_full_size(torch_cuda):
    """The LM-head-sized matrix (128256 x 4096, 525M weights, one stream) at
    two tokens: long enough for the dynamic schedule, and every one of the
    256,512 outputs against the oracle."""
    torch = torch_cuda
    w = workloads.gen_lm_head()
    out_f, in_f = workloads.LM_HEAD_SHAPE
    _note("linear lm head full size")
    t = df11.compress(w, shape=(out_f, in_f))
    assert t.header.n_groups >= 2 * 12 * 768  # many rounds per workgroup: the dynamic schedule runs
    x = _tokens(2, in_f, 13)
    xd = torch.from_numpy(x.view(np.int16)).to("cuda").view(torch.bfloat16)
    y = t.linear(xd)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    del t, y
    ref = oracle.linear(oracle.encode(w), x, out_f)
    assert np.all(np.abs(got - ref) <= _linear_bound(x, w, out_f, in_f))
    assert not np.array_equal(got[0], got[1])


@pytest.mark.timeout(600)
def test_largest_stream(torch_cuda):
    """The largest stream the library takes, DF11_MAX_ELEMENTS = 2^32 - 2^16
    weights (the block workload's weights repeated; 8.6 GB of BF16): output
    indices up to the 32-bit limit decode to the original bits."""
    torch = torch_cuda
    from entropy_decoding_df11_amd import _lib
    n = _lib.MAX_ELEMENTS
    w = np.resize(workloads.gen_block(seed=3)[0], n)
    _note(f"largest stream n={n}")
    t = df11.compress(w, shape=(n,), decode_table_bits=11)
    assert t.header.n_elements == n
    ref = torch.from_numpy(w.view(np.int16)).to("cuda")
    tail = w[-100003:].copy()
    del w
    out = torch.full((n,), 0x5A5A, dtype=torch.int16, device="cuda")
    t.decompress(out=out.view(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert np.array_equal(out[-100003:].cpu().numpy().view(np.uint16), tail)
