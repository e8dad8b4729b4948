"""GPU parity of the grouped GEMMs and of finalize against the oracle, each on
its own, at sizes that span several tiles with ragged tails, for every tile
shape the library picks (the shape follows the mean rows per local expert:
>= 512, >= 128, >= 16, below), including segments that end inside each of
the 32-row fragments of the 128-row weight-streaming tile and segments longer
than one m-tile.

Bar: relative Frobenius error <= 1e-2 for bf16 outputs against the float64
oracle (the GPU accumulates in fp32 and rounds once to bf16: expected ~3e-3).
Rows the kernels must not touch are checked untouched, and NaN planted in
rows they must not read must not reach the outputs."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_scan_amd as moe
import oracle
import synth
from synth import configs

from gpu_util import dev, dev_bf16, host_bf16_bits, host_f64, need_gpu, rel_fro, segments_of

pytestmark = pytest.mark.gpu

TOL = 1e-2
NAN_BITS = 0x7FC0


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


GEMM_CASES = [
    # name, counts per local expert, H, I
    ("thin_tiles", [0, 1, 5, 33, 2, 0, 17, 40], 256, 192),
    ("wide_tiles", [70, 0, 130, 55], 384, 320),
    ("wide_ragged_fragments", [0, 3, 129, 31, 64, 97], 256, 192),
    ("mid_tiles", [300, 1, 420], 256, 448),
    ("big_tiles", [700, 613], 512, 384),
    ("one_expert_many_rows", [1100], 256, 256),
    # few rows and a long reduction: the k-range splits into pieces (fp32
    # partial slices in the workspace, then a fixed-order sum)
    ("split_decode", [1, 0, 2, 1, 0, 3], 1024, 512),
    ("split_wide", [20, 30, 0, 16], 1024, 512),
    # decode-like segments of 0-9 rows with a reduction of 10 k-steps
    ("decode_ragged", [9, 0, 1, 5, 4], 640, 320),
    # under 16 rows per expert on average (128 rows over 16 experts): the
    # whole-k decode kernel, with five 32-k steps in flight per wave (GEMM1,
    # k = 2048) and with one (GEMM2, k = 256; k = 768 below)
    ("decode_kernel", [1, 0, 2, 1, 0, 3, 0, 0, 1, 0, 0, 0, 4, 0, 0, 2], 2048, 256),
    # an expert past 16 rows takes two passes
    ("decode_kernel_two_passes", [0, 20, 1, 0, 0, 0, 0, 0, 3, 0, 0, 0, 0, 0, 0, 0], 2048, 512),
    ("decode_kernel_short_k", [2, 1, 0, 0, 0, 5, 0, 0, 0, 0, 1, 0, 0, 0, 0, 1], 768, 768),
]


def _setup(counts, H, I, seed):
    E_l = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R_l = int(offsets[-1])
    R_pad = ((R_l + 127) // 128) * 128
    a = synth.normal_bf16(seed, 0, (R_pad, H))
    a[R_l:] = NAN_BITS  # never read
    w1 = synth.normal_bf16(seed, 2, (E_l, 2 * I, H), std=1 / np.sqrt(H))
    w2 = synth.normal_bf16(seed, 3, (E_l, H, I), std=1 / np.sqrt(I))
    return E_l, offsets, R_l, R_pad, a, w1, w2


@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_grouped_gemm1_act(case):
    name, counts, H, I = case
    E_l, offsets, R_l, R_pad, a, w1, w2 = _setup(counts, H, I, seed=sum(counts))
    h = torch.full((R_pad, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm1_act(dev_bf16(a), dev(offsets), moe.Weights(dev_bf16(w1)), I, h=h)
    torch.cuda.synchronize()
    eor = segments_of(offsets, R_l)
    ref = oracle.hidden_rows(a[:R_l], oracle.Weights(w1), eor, I)
    assert rel_fro(host_f64(h, slice(None, R_l)), ref) < TOL
    assert np.all(host_bf16_bits(h)[R_l:] == NAN_BITS)


@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_grouped_gemm2(case):
    name, counts, H, I = case
    E_l, offsets, R_l, R_pad, a, w1, w2 = _setup(counts, H, I, seed=sum(counts) + 1)
    hb = synth.normal_bf16(sum(counts), 7, (R_pad, I))
    hb[R_l:] = NAN_BITS
    y = torch.full((R_pad, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm2(dev_bf16(hb), dev(offsets), moe.Weights(dev_bf16(w2)), H, y=y)
    torch.cuda.synchronize()
    eor = segments_of(offsets, R_l)
    ref = oracle.out_rows(hb[:R_l], oracle.Weights(w2), eor, H)
    assert rel_fro(host_f64(y, slice(None, R_l)), ref) < TOL
    assert np.all(host_bf16_bits(y)[R_l:] == NAN_BITS)


@pytest.mark.parametrize("split", [True, False], ids=["split_ok", "no_split"])
@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_grouped_gemms_mxfp4_weights(case, split):
    """MXFP4 weights (e2m1 + E8M0 per 32 along K): both GEMMs against the
    oracle's decode of the same packed bytes (without a scratch the
    weight-streaming shapes take the eight-wave tile)."""
    name, counts, H, I = case
    E_l, offsets, R_l, R_pad, a, w1, w2 = _setup(counts, H, I, seed=sum(counts) + 2)
    q1, s1 = synth.mxfp4_quantize(w1)
    q2, s2 = synth.mxfp4_quantize(w2)
    W1 = moe.Weights(dev(q1), dev(s1))
    W2 = moe.Weights(dev(q2), dev(s2))
    h = torch.full((R_pad, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm1_act(dev_bf16(a), dev(offsets), W1, I, h=h, split=split)
    hb = synth.normal_bf16(sum(counts), 8, (R_pad, I))
    y = moe.moe_grouped_gemm2(dev_bf16(hb), dev(offsets), W2, H, split=split)
    torch.cuda.synchronize()
    eor = segments_of(offsets, R_l)
    ref_h = oracle.hidden_rows(a[:R_l], oracle.Weights(q1, s1), eor, I)
    ref_y = oracle.out_rows(hb[:R_l], oracle.Weights(q2, s2), eor, H)
    assert rel_fro(host_f64(h, slice(None, R_l)), ref_h) < TOL
    assert np.all(host_bf16_bits(h)[R_l:] == NAN_BITS)
    assert rel_fro(host_f64(y, slice(None, R_l)), ref_y) < TOL


@pytest.mark.parametrize("case", [c for c in GEMM_CASES if c[0].startswith("split")],
                         ids=lambda c: c[0])
def test_split_reduction_matches_unsplit(case):
    """The split path (pieces summed in order) and the unsplit path agree to
    rounding, and the split path gives the same bits on every run."""
    name, counts, H, I = case
    E_l, offsets, R_l, R_pad, a, w1, w2 = _setup(counts, H, I, seed=sum(counts) + 3)
    assert moe.moe_grouped_gemm_workspace_size(R_pad, I, True) > 0
    ad, od, W1 = dev_bf16(a), dev(offsets), moe.Weights(dev_bf16(w1))
    h_split = [host_bf16_bits(moe.moe_grouped_gemm1_act(ad, od, W1, I))[:R_l] for _ in range(2)]
    h_plain = moe.moe_grouped_gemm1_act(ad, od, W1, I, split=False)
    torch.cuda.synchronize()
    assert np.array_equal(h_split[0], h_split[1])
    ref = oracle.hidden_rows(a[:R_l], oracle.Weights(w1), segments_of(offsets, R_l), I)
    assert rel_fro(synth.bf16_bits_to_f32(h_split[0]).astype(np.float64), ref) < TOL
    assert rel_fro(host_f64(h_plain, slice(None, R_l)), ref) < TOL


def test_gemm_deterministic():
    E_l, offsets, R_l, R_pad, a, w1, w2 = _setup([300, 1, 420], 256, 448, seed=99)
    outs = []
    for _ in range(2):
        h = moe.moe_grouped_gemm1_act(dev_bf16(a), dev(offsets), moe.Weights(dev_bf16(w1)), 448)
        outs.append(host_bf16_bits(h)[:R_l])
    assert np.array_equal(outs[0], outs[1])


FIN_CASES = [
    # name, T, E, E_l (None: all local), k, H, weights dtype, shared
    ("tiny_f32", 16, 8, None, 2, 128, torch.float32, False),
    ("deepseek_shared_f32", 64, 256, None, 8, 7168, torch.float32, True),
    ("ep_rank_bf16", 64, 256, 32, 8, 7168, torch.bfloat16, False),
    ("ep_rank_single_token", 1, 256, 32, 8, 7168, torch.bfloat16, False),
    ("mixtral_f32", 512, 8, None, 2, 4096, torch.float32, False),
]


@pytest.mark.parametrize("case", FIN_CASES, ids=[c[0] for c in FIN_CASES])
def test_finalize(case):
    name, T, E, E_l, k, H, wdt, with_shared = case
    seed = T + H
    logits = synth.normal_f32(seed, 1, (T, E))
    ids, w = oracle.route(logits, k, 1, True, 2.5)
    emap = None
    if E_l is not None:
        emap = configs.expert_map(configs.EP_DECODE)
    m, off, _ = oracle.permute(ids, E, E_l or E, emap)
    R_l = int(off[-1])
    R_pad = configs.permuted_rows(T, k)
    y = synth.normal_bf16(seed, 2, (R_pad, H))
    y[R_l:] = NAN_BITS
    shared = synth.normal_bf16(seed, 5, (T, H)) if with_shared else None
    w_dev = dev(w.astype(np.float32))
    if wdt == torch.bfloat16:
        w_dev = w_dev.to(torch.bfloat16)
    w_used = host_f64(w_dev)  # the oracle gets the weights the kernel reads
    out = moe.moe_finalize(dev_bf16(y), w_dev, dev(m), 1.0,
                           None if shared is None else dev_bf16(shared))
    torch.cuda.synchronize()
    ref = oracle.finalize(y, w_used, m, 1.0, shared)
    got = host_f64(out)
    assert np.all(np.isfinite(got))
    assert rel_fro(got, ref) < TOL
    # tokens with no local route get exactly 0 (or exactly their shared row)
    none = np.all(m < 0, axis=1)
    if none.any():
        want = synth.bf16_bits_to_f32(shared[none]) if with_shared else 0.0
        assert np.all(got[none] == want)


def test_finalize_in_place_over_shared_and_rsf():
    T, k, H = 32, 2, 256
    logits = synth.normal_f32(5, 1, (T, 8))
    ids, w = oracle.route(logits, k, 0, True, 1.0)
    m, off, _ = oracle.permute(ids, 8, 8)
    y = synth.normal_bf16(5, 2, (configs.permuted_rows(T, k), H))
    shared = synth.normal_bf16(5, 5, (T, H))
    s_dev = dev_bf16(shared)
    w_dev = dev(w.astype(np.float32))
    out = moe.moe_finalize(dev_bf16(y), w_dev, dev(m), 0.5, s_dev, out=s_dev)
    torch.cuda.synchronize()
    ref = oracle.finalize(y, host_f64(w_dev), m, 0.5, shared)
    assert out.data_ptr() == s_dev.data_ptr()
    assert rel_fro(host_f64(out), ref) < TOL


def test_finalize_reads_only_y_rows():
    # y_perm holds R rows of a larger buffer whose rows past R are NaN bits;
    # map entries naming those rows count as -1 (nothing read), and an out
    # placed right after y's R rows is accepted although T * k > R (the
    # batched experts format's shape: E_l * max_tokens rows below T * k)
    T, k, H, R = 40, 4, 256, 96
    logits = synth.normal_f32(17, 1, (T, 8))
    _, w = oracle.route(logits, k, 0, True, 1.0)
    rng = np.random.default_rng(17)
    m = rng.integers(-1, R + 32, size=(T, k)).astype(np.int32)   # some entries >= R
    assert (m >= R).any() and T * k > R
    buf = torch.empty((R + 32 + T) * H, dtype=torch.bfloat16, device="cuda")
    y = synth.normal_bf16(17, 2, (R, H))
    bits = np.full((R + 32, H), NAN_BITS, dtype=np.uint16)
    bits[:R] = y
    buf[:(R + 32) * H].copy_(dev_bf16(bits).view(-1))
    y_dev = buf[:R * H].view(R, H)
    out = buf[R * H:(R + T) * H].view(T, H)        # overlaps the NaN rows, not y
    w_dev = dev(w.astype(np.float32))
    m_dev = dev(m)
    moe.moe_finalize(y_dev, w_dev, m_dev, 1.0, None, out=out)
    torch.cuda.synchronize()
    m_ref = np.where(m < R, m, -1).astype(np.int32)
    ref = oracle.finalize(y, host_f64(w_dev), m_ref, 1.0, None)
    got = host_f64(out)
    assert np.all(np.isfinite(got)) and rel_fro(got, ref) < TOL
    # the fused tail the same way
    res = synth.normal_bf16(17, 6, (T, H))
    gamma = synth.normal_bf16(17, 7, (H,), mean=1.0, std=0.2)
    res_dev = dev_bf16(res)
    out2 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_finalize_add_rmsnorm(y_dev, w_dev, m_dev, res_dev, dev_bf16(gamma), 1e-6, 1.0,
                                 None, out=out2)
    torch.cuda.synchronize()
    ref_res, ref_out = oracle.finalize_add_rmsnorm(y, host_f64(w_dev), m_ref, res, gamma, 1e-6,
                                                   1.0, None)
    assert rel_fro(host_f64(res_dev), ref_res) < TOL
    assert np.all(np.isfinite(host_f64(out2))) and rel_fro(host_f64(out2), ref_out) < TOL


@pytest.mark.parametrize("mxfp4", [False, True], ids=["bf16", "mxfp4"])
def test_tail_round_split(mxfp4):
    """Whole-k tiles (128x256, >= 512 rows per expert) whose count leaves a
    last round of 32 tiles on a 256-CU part: those tiles are cut along k,
    summed from fp32 slabs by the reduce kernel (the scratch header records
    the split).  Both GEMMs against the oracle, bit-identical on a rerun,
    the same values without the scratch (no split) within rounding."""
    counts = [2304, 2250]        # 18 m-tiles each: 36 x 8 n-tiles = 288 tiles
    E_l = len(counts)
    H, I = (1024, 1024) if mxfp4 else (256, 1024)     # GEMM1: K = H; GEMM2: K = I, N = H
    H2 = 2048                                         # GEMM2's output width: 8 n-tiles
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R_l = int(offsets[-1])
    R_pad = ((R_l + 127) // 128) * 128
    a = synth.normal_bf16(61, 0, (R_pad, H))
    hb = synth.normal_bf16(61, 7, (R_pad, I))
    w1 = synth.normal_bf16(61, 2, (E_l, 2 * I, H), std=1 / np.sqrt(H))
    w2 = synth.normal_bf16(61, 3, (E_l, H2, I), std=1 / np.sqrt(I))
    if mxfp4:
        q1, s1 = synth.mxfp4_quantize(w1)
        q2, s2 = synth.mxfp4_quantize(w2)
        W1, W2 = moe.Weights(dev(q1), dev(s1)), moe.Weights(dev(q2), dev(s2))
        O1, O2 = oracle.Weights(q1, s1), oracle.Weights(q2, s2)
    else:
        W1, W2 = moe.Weights(dev_bf16(w1)), moe.Weights(dev_bf16(w2))
        O1, O2 = oracle.Weights(w1), oracle.Weights(w2)
    off = dev(offsets)
    ws = torch.empty(moe.moe_grouped_gemm_workspace_size(R_pad, H2, False), dtype=torch.uint8,
                     device="cuda")
    ad, hd = dev_bf16(a), dev_bf16(hb)
    h = moe.moe_grouped_gemm1_act(ad, off, W1, I, workspace=ws)
    y = moe.moe_grouped_gemm2(hd, off, W2, H2, workspace=ws)
    hdr = ws[:8].view(torch.int32).cpu().numpy()   # GEMM2's header (the last call)
    y2 = moe.moe_grouped_gemm2(hd, off, W2, H2, workspace=ws)
    y_plain = moe.moe_grouped_gemm2(hd, off, W2, H2, split=False)
    torch.cuda.synchronize()
    props = torch.cuda.get_device_properties(0)
    if props.multi_processor_count == 256:
        assert hdr[0] == 32 and hdr[1] >= 2, hdr
    assert np.array_equal(host_bf16_bits(y)[:R_l], host_bf16_bits(y2)[:R_l])  # rows past R_l unwritten
    eor = segments_of(offsets, R_l)
    ref_h = oracle.hidden_rows(a[:R_l], O1, eor, I)
    ref_y = oracle.out_rows(hb[:R_l], O2, eor, H2)
    assert rel_fro(host_f64(h, slice(None, R_l)), ref_h) < TOL
    assert rel_fro(host_f64(y, slice(None, R_l)), ref_y) < TOL
    assert rel_fro(host_f64(y, slice(None, R_l)), host_f64(y_plain, slice(None, R_l))) < 1e-3


@pytest.mark.parametrize("tail", [8, 40, 64])
@pytest.mark.parametrize("gated", [False, True], ids=["gemm2", "gemm1"])
def test_tail_split_tiles_against_unsplit(tail, gated):
    """Tail splits of several sizes on both GEMMs: shapes whose 128x256 tile
    count is one full round of the persistent grid (one workgroup per CU) plus
    `tail` tiles.  Every element outside the tail tiles the scratch header
    records is bit-identical to the call without scratch (no split); the tail
    tiles agree within fp32 summation-order rounding; sampled rows match the
    oracle."""
    G = torch.cuda.get_device_properties(0).multi_processor_count
    n_tiles = 8
    m_total = (G + tail) // n_tiles
    if m_total * n_tiles != G + tail:
        pytest.skip("tail not a multiple of the n-tiles on this part")
    E_l = 3
    m_e = [m_total // E_l + (1 if e < m_total % E_l else 0) for e in range(E_l)]
    counts = [128 * (m - 1) + 1 + (37 * e) % 127 for e, m in enumerate(m_e)]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R_l = int(offsets[-1])
    R_pad = ((R_l + 127) // 128) * 128
    K = 512
    N_out = 128 * n_tiles if gated else 256 * n_tiles
    a = synth.normal_bf16(90 + tail, 0, (R_pad, K))
    w = synth.normal_bf16(90 + tail, 2, (E_l, 2 * N_out if gated else N_out, K),
                          std=1 / np.sqrt(K))
    W = moe.Weights(dev_bf16(w))
    off, ad = dev(offsets), dev_bf16(a)
    ws = torch.empty(moe.moe_grouped_gemm_workspace_size(R_pad, N_out, gated), dtype=torch.uint8,
                     device="cuda")
    if gated:
        c = moe.moe_grouped_gemm1_act(ad, off, W, N_out, workspace=ws)
        c_plain = moe.moe_grouped_gemm1_act(ad, off, W, N_out, split=False)
    else:
        c = moe.moe_grouped_gemm2(ad, off, W, N_out, workspace=ws)
        c_plain = moe.moe_grouped_gemm2(ad, off, W, N_out, split=False)
    torch.cuda.synchronize()
    hdr = ws[:1024].view(torch.int32).cpu().numpy()
    assert hdr[0] == tail and hdr[1] >= 2, hdr[:2]
    got, ref = host_bf16_bits(c)[:R_l], host_bf16_bits(c_plain)[:R_l]
    in_tail = np.zeros((R_l, N_out), dtype=bool)
    out_n = 128 if gated else 256
    for i in range(tail):
        row0, rows, n0 = hdr[2 + 3 * i: 5 + 3 * i]
        assert 1 <= rows <= 128 and row0 + rows <= R_l and n0 % out_n == 0
        assert not in_tail[row0:row0 + rows, n0:n0 + out_n].any()   # tail tiles are disjoint
        in_tail[row0:row0 + rows, n0:n0 + out_n] = True
    assert np.array_equal(got[~in_tail], ref[~in_tail])
    assert rel_fro(host_f64(c, slice(None, R_l))[in_tail], host_f64(c_plain, slice(None, R_l))[in_tail]) < 1e-3
    rows = np.unique(np.concatenate([np.nonzero(in_tail.any(axis=1))[0][::97], [0, R_l - 1]]))
    eor = segments_of(offsets, R_l)[rows]
    if gated:
        o = oracle.hidden_rows(a[rows], oracle.Weights(w), eor, N_out)
    else:
        o = oracle.out_rows(a[rows], oracle.Weights(w), eor, N_out)
    assert rel_fro(host_f64(c, rows), o) < TOL
