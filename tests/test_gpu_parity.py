"""GPU parity: the HIP library (through its C ABI) against the f64 oracle on the
same seeded inputs.  Tolerances (relative L1, f64 accumulation): outputs 1e-5
for f32 inputs, 2e-2 for bf16/fp16 outputs; fp32 states 1e-4; padded rows
exact zeros; untouched slots and input buffers byte-identical."""
import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import linear_attention_recurrence_gdn_amd as gdn
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# gate
# ---------------------------------------------------------------------------
def test_gate_branch_fixture(dev):
    announce("gate: page fixture + configured alphas")
    n = 48
    rng = np.random.default_rng(11)
    alpha = np.where(np.arange(n) % 3 == 0, 22.0 + 6.0 * (np.arange(n) % 17),
                     rng.normal(0, 3.0, n)).astype(np.float32)[None, :]
    dt = rng.normal(0, 0.5, n).astype(np.float32)
    a = (-(np.abs(rng.normal(0, 1, n)) + 0.1)).astype(np.float32)
    want = oracle.gate(alpha, W.F32, dt, a)
    got = gdn.gate(torch.from_numpy(alpha).to(dev), torch.from_numpy(dt).to(dev),
                   torch.from_numpy(a).to(dev)).cpu().numpy()
    assert np.all(np.isfinite(got))
    assert H.rel_l1(got, want) <= 1e-6
    assert np.all(np.exp(got.astype(np.float64)) < 1.0)


@pytest.mark.parametrize("alpha_dt", [W.F32, W.BF16, W.F16])
def test_gate_configured_inputs(dev, alpha_dt):
    announce(f"gate: decode-B256 alphas, alpha dtype {alpha_dt}")
    case = W.decode_b256()
    alpha = W.encode(case.alpha, alpha_dt)
    want = oracle.gate(alpha, alpha_dt, case.dt_bias, case.ssm_a)
    # strided alpha: place the [B, hv] block inside wider rows
    wide = np.zeros((case.batch, case.hv + 8), dtype=alpha.dtype)
    wide[:, 3:3 + case.hv] = alpha
    dwide = H.to_dev(wide, alpha_dt, dev)
    got = gdn.gate(dwide[:, 3:3 + case.hv], torch.from_numpy(case.dt_bias).to(dev),
                   torch.from_numpy(case.ssm_a).to(dev)).cpu().numpy()
    assert H.rel_l1(got, want) <= 1e-6
    assert np.all(np.isfinite(got)) and np.all(got < 0)


# ---------------------------------------------------------------------------
# decode: the pages' hand cases
# ---------------------------------------------------------------------------
def test_decode_hand_single_step(dev):
    announce("decode: hand single step (page table)")
    d = json.load(open(os.path.join(GOLD, "decode_single_step.json")))
    # The gate is fused in decode: choose alpha, dt_bias, ssm_a so that
    # g = softplus(25) * ssm_a = 25 * ssm_a = ln(0.5) (branch side: exact).
    ssm_a = np.array([math.log(0.5) / 25.0], np.float32)
    g = 25.0 * float(ssm_a[0])
    for dt in (W.F32, W.BF16):
        case = W.DecodeCase(
            name="hand", batch=1, hk=1, hv=1, dk=16, dv=2, in_dtype=dt, out_dtype=dt,
            q=W.View(W.encode(np.pad(np.array([d["q"]], float), ((0, 0), (0, 14))), dt), 0, 16, dt),
            k=W.View(W.encode(np.pad(np.array([d["k"]], float), ((0, 0), (0, 14))), dt), 0, 16, dt),
            v=W.View(W.encode(np.array([d["v"]], float), dt), 0, 2, dt),
            alpha=np.array([[25.0]], np.float32), dt_bias=np.zeros(1, np.float32), ssm_a=ssm_a,
            beta=np.array([[d["beta"]]], np.float32),
            pool=np.pad(np.array(d["S0"], np.float32), ((0, 0), (0, 14)))[None, None].copy(),
            idx=np.zeros(1, np.int32), scale=d["scale"], l2norm=False)
        res = H.run_decode(case, dev)
        tol = 1e-6 if dt == W.F32 else 0.01
        # decay = exp(25 * ssm_a) differs from 0.5 by f32 rounding of ssm_a only
        assert abs(math.exp(g) - 0.5) < 1e-7
        np.testing.assert_allclose(res.out[0, 0], d["out"], rtol=tol)
        st = res.pool[0, 0, :, :2].cpu().numpy()
        np.testing.assert_allclose(st, d["S"], rtol=1e-6)
        want_out, want_state = oracle.decode_case(case)
        H.check_decode(case, res, want_out, want_state)


# ---------------------------------------------------------------------------
# decode: shape / dtype / layout matrix at small sizes
# ---------------------------------------------------------------------------
DECODE_CASES = [
    # (batch, hk, hv, dk, dv, in, out, slots, packed_pad, null_rows)
    (3, 1, 1, 16, 16, W.F32, W.F32, 4, None, ()),
    (5, 2, 6, 16, 16, W.F32, W.F32, 8, None, (1,)),
    (4, 2, 4, 32, 40, W.BF16, W.BF16, 6, None, ()),
    (4, 1, 3, 64, 64, W.F16, W.F32, 5, None, (0, 3)),
    (7, 2, 6, 128, 128, W.BF16, W.BF16, 11, None, (2,)),
    (6, 2, 4, 128, 72, W.F16, W.F16, 9, 64, (5,)),
    (5, 3, 9, 128, 130, W.BF16, W.F32, 7, 256, ()),
    (3, 1, 2, 256, 128, W.BF16, W.BF16, 4, None, ()),
    (9, 4, 8, 128, 128, W.F32, W.F32, 12, 32, (0,)),
    # GQA 8 with 256 state rows per head
    (4, 1, 8, 128, 256, W.BF16, W.BF16, 6, None, (1,)),
]


@pytest.mark.parametrize("spec", DECODE_CASES, ids=lambda s: "B{}-hk{}-hv{}-dk{}-dv{}-{}-{}".format(
    s[0], s[1], s[2], s[3], s[4], W.DTYPE_NAMES[s[5]], W.DTYPE_NAMES[s[6]]))
def test_decode_matrix(dev, spec):
    B, hk, hv, dk, dv, ind, outd, slots, pad, nulls = spec
    announce(f"decode matrix {spec}")
    case = W.make_decode_case("m", 1000 + B * dk + dv, batch=B, hk=hk, hv=hv, dk=dk, dv=dv,
                              in_dtype=ind, out_dtype=outd, slots=slots, packed_pad=pad,
                              null_rows=nulls, large_every_third=True)
    res = H.run_decode(case, dev)
    want_out, want_state = oracle.decode_case(case)
    H.check_decode(case, res, want_out, want_state)


def test_decode_without_l2norm(dev):
    announce("decode without q/k norm")
    case = W.make_decode_case("nonorm", 77, batch=4, hk=2, hv=4, dk=128, dv=128,
                              in_dtype=W.F32, out_dtype=W.F32, slots=4)
    # unnormalised keys make the step contractive only for small k: scale them down
    case.k.buf[:] *= np.float32(0.05)
    case.l2norm = False
    res = H.run_decode(case, dev)
    want_out, want_state = oracle.decode_case(case)
    H.check_decode(case, res, want_out, want_state)


def test_decode_beta0_g0_leaves_state_bit_exact(dev):
    announce("decode: beta=0, g=0 invariant")
    case = W.make_decode_case("inv", 5, batch=4, hk=2, hv=4, dk=128, dv=128, in_dtype=W.BF16,
                              out_dtype=W.F32, slots=6)
    case.beta[:] = 0.0
    case.ssm_a[:] = -0.0   # g = softplus(.) * -0 = -0, decay = 1
    res = H.run_decode(case, dev)
    live = case.idx
    assert torch.equal(res.pool[live].view(torch.int32), res.pool0[live].view(torch.int32))
    want_out, want_state = oracle.decode_case(case)
    H.check_decode(case, res, want_out, want_state, out_tolerance=1e-5)


GUARD = 256          # guard bytes on each side of a buffer
GUARD_BYTE = 0xA5


def guarded(nbytes: int, dev):
    """A device byte buffer with GUARD bytes of 0xA5 on each side of
    `nbytes` usable bytes; returns (whole buffer, usable view)."""
    buf = torch.full((nbytes + 2 * GUARD,), GUARD_BYTE, dtype=torch.uint8, device=dev)
    return buf, buf[GUARD:GUARD + nbytes]


def guards_intact(buf: torch.Tensor) -> bool:
    return bool((buf[:GUARD] == GUARD_BYTE).all()) and bool((buf[-GUARD:] == GUARD_BYTE).all())


def test_decode_graph_replay(dev):
    """vllm.cpp "CUDA gdn packed decode capture replays preserve padding state
    and canaries": the pool and the output sit between 256-byte 0xA5 guard
    bands; each replay equals the eager call, the guards and the padded row's
    slot are untouched."""
    announce("decode: HIP graph capture and replay, guard bands around out and the pool")
    case = W.make_decode_case("graph", 21, batch=6, hk=2, hv=4, dk=128, dv=128,
                              in_dtype=W.BF16, out_dtype=W.BF16, slots=8, null_rows=(4,))
    dbufs, q, k, v = H.upload_views(case, dev, case.batch)
    t = lambda a: torch.from_numpy(a).to(dev)
    alpha, dt_bias, ssm_a, beta, idx = (t(case.alpha), t(case.dt_bias), t(case.ssm_a),
                                        t(case.beta), t(case.idx))
    pool0 = t(case.pool)
    # eager reference: two consecutive steps
    pe = pool0.clone()
    oe1 = gdn.decode(q, k, v, alpha, dt_bias, ssm_a, beta, pe, idx, scale=case.scale).clone()
    oe2 = gdn.decode(q, k, v, alpha, dt_bias, ssm_a, beta, pe, idx, scale=case.scale).clone()
    pool_buf, pool_bytes = guarded(pool0.numel() * 4, dev)
    pg = pool_bytes.view(torch.float32).view(pool0.shape)
    pg.copy_(pool0)
    out_buf, out_bytes = guarded(case.batch * case.hv * case.dv * 2, dev)
    out = out_bytes.view(torch.bfloat16).view(case.batch, case.hv, case.dv)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        gdn.decode(q, k, v, alpha, dt_bias, ssm_a, beta, pg, idx, scale=case.scale, out=out)
    torch.cuda.synchronize()
    assert torch.equal(pg.view(torch.int32), pool0.view(torch.int32)), "capture must not run"
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), oe1.view(torch.int16))
    assert guards_intact(out_buf) and guards_intact(pool_buf), "replay 1 wrote a guard band"
    o1 = out.clone()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), oe2.view(torch.int16))
    assert torch.equal(pg.view(torch.int32), pe.view(torch.int32))
    assert not torch.equal(o1, out)
    assert guards_intact(out_buf) and guards_intact(pool_buf), "replay 2 wrote a guard band"
    untouched = sorted(set(range(case.num_slots)) - set(int(i) for i in case.idx if i >= 0))
    ut = torch.tensor(untouched, device=dev)
    assert H.bytes_equal(pg[ut], pool0[ut]), "a slot no live row names changed"
    assert torch.equal(out[4], torch.zeros_like(out[4])), "the padded row must be zeros"


# ---------------------------------------------------------------------------
# decode at the configured sizes
# ---------------------------------------------------------------------------
def test_decode_b256_full(dev):
    announce("decode B=256 Hk16 Hv32 D128 bf16, 1024-slot pool: all rows vs oracle")
    case = W.decode_b256()
    res = H.run_decode(case, dev)
    want_out, want_state = oracle.decode_case(case)
    H.check_decode(case, res, want_out, want_state, verbose=True)


def test_decode_packed_b1024_all_rows(dev):
    announce("decode B=1024 packed fp16 stride+256, 4096-slot pool: every row vs the oracle")
    case = W.decode_packed_b1024()
    res = H.run_decode(case, dev)
    # the oracle streams over row batches so its f64 states stay bounded
    for r0 in range(0, case.batch, 128):
        rows = np.arange(r0, min(r0 + 128, case.batch))
        want_out, want_state = oracle.decode_case(case, rows=rows)
        H.check_decode(case, res, want_out, want_state, rows=rows,
                       check_untouched=(r0 == 0), verbose=(r0 == 0))
        del want_out, want_state
    # the NaN padding columns were never read
    assert np.isfinite(res.out).all()


def test_tiny_prefill_then_four_decode_steps(dev):
    announce("tiny f32: T=64 prefill then 4 decode steps on the resulting state")
    pre, steps = W.tiny_prefill_then_decode()
    for sequential in (True, False):
        res = H.run_prefill(pre, dev, sequential=sequential)
        want_out, want_state = oracle.prefill_case(pre)
        H.check_prefill(pre, res, want_out, want_state)
        pool = res.pool
        pool_np = want_state.astype(np.float32)  # oracle chain continues from its own state
        for st in steps:
            st.pool = pool_np
            r = H.run_decode(st, dev, pool=pool)
            o, s = oracle.decode_case(st)
            # the GPU state entering this step differs from the oracle's by f32
            # rounding only; compare against the oracle chain
            H.check_decode(st, r, o, s)
            pool = r.pool
            pool_np = s.astype(np.float32)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------
PREFILL_CASES = [
    # (lengths, hk, hv, dk, dv, in, out, has_init)
    ([64], 2, 2, 16, 16, W.F32, W.F32, [1]),
    ([1, 0, 63, 64, 65, 130], 2, 6, 128, 128, W.BF16, W.BF16, [1, 1, 0, 1, 0, 1]),
    ([200, 3], 1, 3, 128, 128, W.F16, W.F16, [1, 1]),
    ([17, 140], 2, 4, 64, 48, W.F16, W.F32, [0, 1]),
    ([33, 5, 96], 1, 2, 32, 32, W.BF16, W.BF16, [1, 0, 1]),
    ([70], 1, 1, 256, 128, W.BF16, W.BF16, [1]),
    # chunk-boundary lengths, GQA 3, two 32-row state tiles
    ([1, 63, 64, 65, 127, 128, 129], 2, 6, 128, 64, W.BF16, W.BF16, [1, 0, 1, 1, 0, 1, 1]),
    ([300, 17], 1, 2, 128, 96, W.F16, W.F16, [1, 0]),
    ([190], 2, 4, 128, 128, W.BF16, W.F32, [1]),
]


@pytest.mark.parametrize("sequential", [True, False], ids=["sequential", "default"])
@pytest.mark.parametrize("spec", PREFILL_CASES, ids=lambda s: "L{}-hk{}-hv{}-dk{}-dv{}-{}".format(
    "_".join(map(str, s[0])), s[1], s[2], s[3], s[4], W.DTYPE_NAMES[s[5]]))
def test_prefill_matrix(dev, spec, sequential):
    lengths, hk, hv, dk, dv, ind, outd, hi = spec
    announce(f"prefill matrix {spec} sequential={sequential}")
    case = W.make_prefill_case("pm", 2000 + sum(lengths) + dk, lengths=lengths, hk=hk, hv=hv,
                               dk=dk, dv=dv, in_dtype=ind, out_dtype=outd,
                               slots=len(lengths) + 2, has_init=hi)
    res = H.run_prefill(case, dev, sequential=sequential)
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, res, want_out, want_state)


def test_prefill_t1_equals_decode(dev):
    announce("prefill T=1 equals decode")
    dcase = W.make_decode_case("t1", 31, batch=1, hk=2, hv=4, dk=128, dv=128, in_dtype=W.F32,
                               out_dtype=W.F32, slots=1)
    r_dec = H.run_decode(dcase, dev)
    pcase = W.PrefillCase(name="t1p", total_tokens=1, num_seqs=1, hk=2, hv=4, dk=128, dv=128,
                          in_dtype=W.F32, out_dtype=W.F32, q=dcase.q, k=dcase.k, v=dcase.v,
                          alpha=dcase.alpha, dt_bias=dcase.dt_bias, ssm_a=dcase.ssm_a,
                          beta=dcase.beta, cu_seqlens=np.array([0, 1], np.int32),
                          pool=dcase.pool, idx=dcase.idx, has_init=np.ones(1, np.int8),
                          scale=dcase.scale)
    r_pre = H.run_prefill(pcase, dev, sequential=True)
    np.testing.assert_allclose(r_pre.out, r_dec.out, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(r_pre.pool.cpu().numpy(), r_dec.pool.cpu().numpy(), rtol=2e-6,
                               atol=1e-7)


def test_prefill_t4096_all_heads(dev):
    announce("prefill T=4096 Hk16 Hv32 D128 bf16, zero init (NaN slot): every head vs the oracle")
    case = W.prefill_t4096()
    res = H.run_prefill(case, dev)
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, res, want_out, want_state, verbose=True)


def test_prefill_varlen_gqa3_all_heads(dev):
    announce("prefill varlen 8 seqs T=32768 Hk8 Hv24 GQA3 fp16: every head vs the oracle")
    case = W.prefill_varlen_gqa3()
    res = H.run_prefill(case, dev)
    want_out, want_state = oracle.prefill_case(case)
    print(f"  lengths {case.meta['lengths']}", flush=True)
    H.check_prefill(case, res, want_out, want_state, verbose=True)


def test_prefill_skewed_batch_split_schedule(dev):
    """One 8192-token sequence beside seven of 2048 (GQA 3, fp16): the longest
    sequence bounds the call, so the chunked path walks it as soon as its own
    records exist while the others' records and walks run beside it on the
    caller's second stream (gdn_prefill_varlen_aux).  The split rank is read
    back from the metadata the call leaves in the workspace (int32 words
    cs[n+1], order[n], ocs[n+1], then the split rank)."""
    announce("prefill skewed batch [8192, 7 x 2048] Hk8 Hv24 fp16: split schedule, every head")
    lengths = [8192] + [2048] * 7
    case = W.make_prefill_case("skew", 4242, lengths=lengths, hk=8, hv=24, dk=128, dv=128,
                               in_dtype=W.F16, out_dtype=W.F16, slots=12,
                               has_init=[1, 0, 1, 1, 0, 1, 1, 1])
    T, N = case.total_tokens, case.num_seqs
    _, q, k, v = H.upload_views(case, dev, T)
    t = lambda a: torch.from_numpy(a).to(dev)
    g = gdn.gate(t(case.alpha), t(case.dt_bias), t(case.ssm_a))
    pool = t(case.pool)
    pool0 = pool.clone()
    ws_n = gdn.prefill_workspace_size(T, N, case.hk, case.hv, case.dk, case.dv, torch.float16)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    aux = torch.cuda.Stream()
    out = gdn.prefill_varlen(q, k, v, g, t(case.beta), pool, t(case.cu_seqlens),
                             scale=case.scale, state_idx=t(case.idx),
                             has_initial_state=t(case.has_init), workspace=ws, aux_stream=aux)
    torch.cuda.synchronize()
    words = ws[:4 * (3 * N + 5)].view(torch.int32).cpu().numpy()
    split_rank, split_seqs, segments = (int(x) for x in words[3 * N + 2:3 * N + 5])
    assert list(words[N + 1:2 * N + 1][:1]) == [0]      # the 8192-token sequence ranks first
    assert split_rank >= 1, f"split rank {split_rank}"
    want_out, want_state = oracle.prefill_case(case)
    res = H.PrefillResult(H.out_to_f64(out), pool, pool0, True)
    print(f"  split rank {split_rank}, {split_seqs} sequence(s) in {segments} segments",
          flush=True)
    H.check_prefill(case, res, want_out, want_state, verbose=True)


def test_prefill_skewed_batch_in_a_captured_graph(dev):
    """The same skewed batch captured into a graph (the library keeps the whole
    call on the captured stream then): every replay, from a restored pool,
    gives the eager call's outputs and final states."""
    announce("prefill skewed batch captured into a graph: replays equal the eager call")
    lengths = [1500] + [300] * 5
    case = W.make_prefill_case("skewg", 4343, lengths=lengths, hk=2, hv=6, dk=128, dv=64,
                               in_dtype=W.BF16, out_dtype=W.BF16, slots=8,
                               has_init=[1, 1, 0, 1, 1, 1])
    T, N = case.total_tokens, case.num_seqs
    _, q, k, v = H.upload_views(case, dev, T)
    t = lambda a: torch.from_numpy(a).to(dev)
    g = gdn.gate(t(case.alpha), t(case.dt_bias), t(case.ssm_a))
    beta, cu, idx, hi = t(case.beta), t(case.cu_seqlens), t(case.idx), t(case.has_init)
    pool0 = t(case.pool)
    ws = torch.empty(gdn.prefill_workspace_size(T, N, case.hk, case.hv, case.dk, case.dv,
                                                torch.bfloat16), dtype=torch.uint8, device=dev)
    out = torch.empty((T, case.hv, case.dv), dtype=torch.bfloat16, device=dev)
    pool = pool0.clone()

    def call():
        gdn.prefill_varlen(q, k, v, g, beta, pool, cu, scale=case.scale, state_idx=idx,
                           has_initial_state=hi, out=out, workspace=ws,
                           stream=torch.cuda.current_stream())

    call()
    torch.cuda.synchronize()
    want_out, want_pool = out.clone(), pool.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        pool.copy_(pool0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        pool.copy_(pool0)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_out), f"replay {rep}: outputs differ"
        assert H.bytes_equal(pool, want_pool), f"replay {rep}: states differ"
    want_o, want_s = oracle.prefill_case(case)
    H.check_prefill(case, H.PrefillResult(H.out_to_f64(want_out), want_pool, pool0, True),
                    want_o, want_s)


@pytest.mark.parametrize("nseq", [256, 257, 300, 1100], ids=["n256", "n257", "n300", "n1100"])
def test_prefill_many_short_sequences(dev, nseq):
    """Hundreds of short sequences (zero-length ones among them), in one
    stream order: up to 256 sequences the prep launch forms the metadata in
    its workgroup 0 and its other workgroups index themselves from
    cu_seqlens, above that the metadata has a launch of its own and spans
    several 256-wide scans, and beyond 1024 sequences the walk keeps index
    order instead of ranking by length."""
    announce(f"prefill {nseq} short sequences (0..20 tokens), GQA 2, bf16")
    rng = np.random.default_rng(nseq)
    lengths = [int(x) for x in rng.integers(0, 21, size=nseq)]
    case = W.make_prefill_case("many", 5000 + nseq, lengths=lengths, hk=1, hv=2, dk=128, dv=32,
                               in_dtype=W.BF16, out_dtype=W.BF16, slots=nseq + 3,
                               has_init=[int(x) for x in rng.integers(0, 2, size=nseq)])
    res = H.run_prefill(case, dev)
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, res, want_out, want_state)


# GQA groups wider than the prep's four v-heads at once (ratios 5, 8 and 9:
# the gate factors of a second and third group are formed mid-unit), exactly
# one group (4), and the narrowest and widest state rows the chunked walk
# takes (Dv = 16: three of its four waves past Dv; Dv = 256: four 64-row
# workgroups per v-head)
WIDE_CASES = [
    # (lengths, hk, hv, dv, in, out, has_init)
    ([130, 64, 1, 300], 1, 5, 128, W.BF16, W.BF16, [1, 0, 1, 1]),
    ([200, 0, 65], 1, 8, 64, W.F16, W.F16, [1, 1, 0]),
    ([129, 40], 2, 18, 32, W.BF16, W.F32, [0, 1]),
    ([257, 3], 1, 4, 256, W.F16, W.F16, [1, 1]),
    ([190, 64, 7], 2, 2, 16, W.BF16, W.BF16, [1, 0, 1]),
]


@pytest.mark.parametrize("aux", [False, True], ids=["one_stream", "split"])
@pytest.mark.parametrize("spec", WIDE_CASES, ids=lambda s: "L{}-hk{}-hv{}-dv{}".format(
    "_".join(map(str, s[0])), s[1], s[2], s[3]))
def test_prefill_wide_gqa_and_state_rows(dev, spec, aux):
    lengths, hk, hv, dv, ind, outd, hi = spec
    announce(f"prefill wide GQA / state rows {spec} aux={aux}")
    case = W.make_prefill_case("wide", 7100 + hv * 31 + dv, lengths=lengths, hk=hk, hv=hv,
                               dk=128, dv=dv, in_dtype=ind, out_dtype=outd,
                               slots=len(lengths) + 2, has_init=hi)
    res = H.run_prefill(case, dev, aux=aux)
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, res, want_out, want_state)


@pytest.mark.parametrize("ind", [W.BF16, W.F16], ids=["bf16", "f16"])
def test_prefill_chunked_matches_sequential(dev, ind):
    announce(f"prefill: chunked MFMA path vs token-sequential path ({W.DTYPE_NAMES[ind]})")
    case = W.make_prefill_case("cvs", 4321, lengths=[257, 64, 1, 130], hk=2, hv=4, dk=128,
                               dv=128, in_dtype=ind, out_dtype=ind, slots=6)
    rs = H.run_prefill(case, dev, sequential=True)
    rc = H.run_prefill(case, dev, sequential=False)
    # vllm.cpp's chunked-vs-sequential case: elementwise with the dtype combo,
    # and the max / mean absolute differences (AbsoluteDiffStats)
    H.check_units(rc.out, rs.out, 2, H.OUT_TOL_HALF, "chunked vs sequential output")
    H.check_close(rc.out, rs.out, *H.CLOSE_HALF, "chunked vs sequential output")
    idx = torch.from_numpy(case.idx.astype(np.int64)).to(dev)
    st_c, st_s = rc.pool[idx].cpu().numpy(), rs.pool[idx].cpu().numpy()
    H.check_units(st_c, st_s, 2, H.STATE_TOL, "chunked vs sequential state")
    H.check_close(st_c, st_s, *H.CLOSE_HALF_F32, "chunked vs sequential state")
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, rc, want_out, want_state)
    H.check_prefill(case, rs, want_out, want_state)
    om, oa = H.diff_stats(rc.out, rs.out)
    sm, sa = H.diff_stats(st_c, st_s)
    print(f"  chunked vs sequential: out max {om:.2e} mean {oa:.2e}; "
          f"state max {sm:.2e} mean {sa:.2e}", flush=True)


@pytest.mark.parametrize("sequential", [True, False], ids=["sequential", "default"])
def test_prefill_trailing_empty_sequence(dev, sequential):
    """A zero-length sequence at the end of cu_seqlens (its first token index
    equals total_tokens) reads no token row: its state passes through, or is
    zeroed without an initial state."""
    announce(f"prefill: trailing zero-length sequences sequential={sequential}")
    case = W.make_prefill_case("tail0", 6061, lengths=[70, 5, 0, 0], hk=2, hv=4, dk=128,
                               dv=128, in_dtype=W.BF16, out_dtype=W.BF16, slots=6,
                               has_init=[1, 1, 1, 0])
    res = H.run_prefill(case, dev, sequential=sequential)
    want_out, want_state = oracle.prefill_case(case)
    H.check_prefill(case, res, want_out, want_state)
    # the pass-through slot keeps its exact bytes; the zeroed one is exact zeros
    s2, s3 = int(case.idx[2]), int(case.idx[3])
    assert H.bytes_equal(res.pool[s2], res.pool0[s2])
    assert bool((res.pool[s3] == 0).all())


def test_prefill_no_tokens(dev):
    """total_tokens = 0 with two sequences (has_init 1 and 0) and no token
    buffers at all: the first state passes through bit for bit, the second is
    zeroed; nothing else is touched."""
    announce("prefill: two sequences, zero tokens, null token pointers")
    t = lambda a: torch.from_numpy(a).to(dev)
    hk, hv, dk, dv, slots = 2, 4, 128, 128, 5
    rng = np.random.default_rng(6062)
    pool0 = t(rng.normal(0, 0.05, size=(slots, hv, dv, dk)).astype(np.float32))
    pool = pool0.clone()
    lib = gdn.load_library()
    cu = t(np.zeros(3, np.int32))
    idx = t(np.array([3, 1], np.int32))
    hi = t(np.array([1, 0], np.int8))
    rc = lib.gdn_prefill_varlen(None, gdn.GDN_BF16, None, None, None, gdn.GDN_BF16,
                                hk * dk, hk * dk, hv * dv, None, hv, None, hv,
                                pool.data_ptr(), slots, idx.data_ptr(), hi.data_ptr(),
                                cu.data_ptr(), 2, 0, hk, hv, dk, dv, 0.0883883, 1e-6, 1,
                                None, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.gdn_last_error()
    torch.cuda.synchronize()
    assert H.bytes_equal(pool[3], pool0[3])
    assert bool((pool[1] == 0).all())
    for sl in (0, 2, 4):
        assert H.bytes_equal(pool[sl], pool0[sl])


def test_prefill_on_a_side_stream_then_reallocate(dev):
    """A call on a stream other than the current one allocates its output and
    workspace on that stream, so memory freed and reused right after the call
    on the current stream cannot overwrite them while the kernels run."""
    announce("prefill on a side stream, then reallocate on the current stream")
    case = W.make_prefill_case("side", 6063, lengths=[900, 300, 17], hk=2, hv=6, dk=128,
                               dv=128, in_dtype=W.BF16, out_dtype=W.BF16, slots=5)
    _, q, k, v = H.upload_views(case, dev, case.total_tokens)
    t = lambda a: torch.from_numpy(a).to(dev)
    g = gdn.gate(t(case.alpha), t(case.dt_bias), t(case.ssm_a))
    beta, cu, idx = t(case.beta), t(case.cu_seqlens), t(case.idx)
    pool = t(case.pool)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    out = gdn.prefill_varlen(q, k, v, g, beta, pool, cu, scale=case.scale, state_idx=idx,
                             stream=side)
    # allocations on the current stream right after the call, written at once
    junk = [torch.full((1 << 22,), 7, dtype=torch.uint8, device=dev) for _ in range(32)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    want_out, want_state = oracle.prefill_case(case)
    res = H.PrefillResult(H.out_to_f64(out), pool, None, True)
    H.check_prefill(case, res, want_out, want_state)


def test_prefill_split_on_side_streams_then_reallocate(dev):
    """The same with the split schedule: the call and its second stream are
    both side streams, and the output and workspace are the binding's own;
    memory allocated and filled on the current stream right after the call
    must not land on them while either stream's kernels run."""
    announce("prefill split on two side streams, then reallocate on the current stream")
    case = W.make_prefill_case("side2", 6065, lengths=[2100, 900, 300, 17], hk=2, hv=6, dk=128,
                               dv=128, in_dtype=W.F16, out_dtype=W.F16, slots=6)
    _, q, k, v = H.upload_views(case, dev, case.total_tokens)
    t = lambda a: torch.from_numpy(a).to(dev)
    g = gdn.gate(t(case.alpha), t(case.dt_bias), t(case.ssm_a))
    beta, cu, idx = t(case.beta), t(case.cu_seqlens), t(case.idx)
    pool = t(case.pool)
    side, aux = torch.cuda.Stream(), torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    out = gdn.prefill_varlen(q, k, v, g, beta, pool, cu, scale=case.scale, state_idx=idx,
                             stream=side, aux_stream=aux)
    junk = [torch.full((1 << 22,), 9, dtype=torch.uint8, device=dev) for _ in range(32)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    want_out, want_state = oracle.prefill_case(case)
    res = H.PrefillResult(H.out_to_f64(out), pool, None, True)
    H.check_prefill(case, res, want_out, want_state)


def test_prefill_calls_on_two_streams_run_concurrently(dev):
    """Two prefill calls on two streams, each with its own second stream for
    the split schedule, enqueued back to back with no synchronisation between
    them: outputs and final states byte-equal to the same calls run one after
    the other (the library shares no stream, event or lock between calls)."""
    announce("prefill: two calls on two streams concurrently vs one after the other")
    cases = [W.make_prefill_case("c2a", 6071, lengths=[3000, 200, 700, 50], hk=2, hv=6, dk=128,
                                 dv=128, in_dtype=W.BF16, out_dtype=W.BF16, slots=6),
             W.make_prefill_case("c2b", 6072, lengths=[90, 2500, 1300], hk=1, hv=3, dk=128,
                                 dv=128, in_dtype=W.F16, out_dtype=W.F16, slots=5)]
    t = lambda a: torch.from_numpy(a).to(dev)
    inputs = []
    for case in cases:
        _, q, k, v = H.upload_views(case, dev, case.total_tokens)
        g = gdn.gate(t(case.alpha), t(case.dt_bias), t(case.ssm_a))
        ws = torch.empty(gdn.prefill_workspace_size(case.total_tokens, case.num_seqs, case.hk,
                                                    case.hv, case.dk, case.dv,
                                                    H.TORCH_OF[case.in_dtype]),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((case.total_tokens, case.hv, case.dv),
                          dtype=H.TORCH_OF[case.out_dtype], device=dev)
        inputs.append((case, q, k, v, g, t(case.beta), t(case.cu_seqlens), t(case.idx),
                       t(case.pool), ws, out))
    torch.cuda.synchronize()

    def call(inp, pool, stream, aux):
        case, q, k, v, g, beta, cu, idx, _, ws, out = inp
        gdn.prefill_varlen(q, k, v, g, beta, pool, cu, scale=case.scale, state_idx=idx,
                           out=out, workspace=ws, stream=stream, aux_stream=aux)

    # one after the other on the current stream (each with a second stream)
    seq = []
    for inp in inputs:
        pool = inp[8].clone()
        call(inp, pool, torch.cuda.current_stream(), torch.cuda.Stream())
        torch.cuda.synchronize()
        seq.append((inp[10].clone(), pool))
    # concurrently
    streams = [torch.cuda.Stream() for _ in range(4)]
    pools = [inp[8].clone() for inp in inputs]
    for inp in inputs:
        inp[10].zero_()
    torch.cuda.synchronize()
    for i, inp in enumerate(inputs):
        streams[2 * i].wait_stream(torch.cuda.current_stream())
        call(inp, pools[i], streams[2 * i], streams[2 * i + 1])
    torch.cuda.synchronize()
    for i, inp in enumerate(inputs):
        assert H.bytes_equal(inp[10], seq[i][0]), f"call {i}: outputs differ"
        assert H.bytes_equal(pools[i], seq[i][1]), f"call {i}: states differ"
    for i, inp in enumerate(inputs):
        want_out, want_state = oracle.prefill_case(inp[0])
        H.check_prefill(inp[0], H.PrefillResult(H.out_to_f64(seq[i][0]), seq[i][1], None, True),
                        want_out, want_state)
