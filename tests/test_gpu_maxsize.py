"""Parity at the largest sizes the library accepts.

* GEMMs at kpad = 2^24, the longest contraction the calls take (a 128-row
  operand panel of 4-bit codes is then 2^30 bytes, inside the 32-bit buffer
  offsets), dense (FPROP and split-K WGRAD) and K-grouped (WGRAD over three
  token groups and an empty one, padded to exactly 2^24), on random codes and
  scales: sampled outputs against the oracle's FP64 GEMM within
  1e-5 * sum_k |a_k||b_k| (the GEMMs of paperlayer.ai summary section 2
  "Random Hadamard transforms").  Once with random signs and once with every
  product positive, where a single FP32 running sum over 2^20 blocks drifts
  by about 1e-3 of the result: the kernels flush their FP32 sums to the
  output every 65536 K-elements, which holds the error near 1e-7.  bf16
  outputs of contractions several chunks long (dense, K-grouped and
  M-grouped) against the oracle within the bar plus half a bf16 ulp.
* Column-wise (transposing) quantization of rows 2^26 elements long, the
  largest row stride the call takes (16 rows then span 2^31 bytes): sampled
  output rows against the oracle bit for bit (RTNE and SR), and the
  dual-axis kernel's two outputs equal to the single-axis calls' whole
  outputs.
* 1024 expert groups, the largest group count the grouped calls take
  (quantizations and GEMMs), most of them empty or shorter than a block."""
import numpy as np
import pytest
import torch

from oracle import ufp4_oracle as O
from uniform_grid_fp4_amd import ufp4 as U
from uniform_grid_fp4_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 1e-5
KMAX = 1 << 24
LDMAX = 1 << 26
MASK = 0x3C5A


def random_operand(rows, kpad, seed, positive):
    """Codes with every nibble drawn uniformly (sign bits cleared when
    `positive`), scales 2^u with u uniform in [-6, 6)."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    codes = torch.randint(0, 256, (rows, kpad // 2), dtype=torch.uint8, device=DEV, generator=g)
    if positive:
        codes &= 0x77
    u = torch.empty((rows, kpad // 16), dtype=torch.float32, device=DEV).uniform_(-6.0, 6.0,
                                                                                  generator=g)
    scales = torch.exp2(u)
    return U.Quantized(codes, scales, rows, kpad, kpad, U.GRID_UNIFORM, 1, MASK)


def host_rows(q, rows, k0=0, k1=None):
    k1 = q.kpad if k1 is None else k1
    return (q.codes[rows, k0 // 2:k1 // 2].cpu().numpy(),
            q.scales[rows, k0 // 16:k1 // 16].cpu().numpy())


def check(got, C, bound, what):
    err = np.abs(got.astype(np.float64) - C)
    lim = TOL * bound
    assert (err <= lim).all(), f"{what}: worst err / bound = {(err / bound).max():.3g}"


@pytest.mark.parametrize("positive", [False, True])
def test_dense_gemm_at_the_largest_kpad(positive):
    M, N = 160, 136
    print(f"[maxsize] dense kpad=2^24 M={M} N={N} positive={positive}", flush=True)
    a = random_operand(M, KMAX, 101, positive)
    b = random_operand(N, KMAX, 102, positive)
    fprop = U.ufp4_gemm_fprop(a, b)
    need = U.ufp4_workspace_size(U.WGRAD, M, N, KMAX)
    assert need > 0
    ws = torch.empty(need // 4, dtype=torch.float32, device=DEV)
    split = U.ufp4_gemm_wgrad(a, b, workspace=ws)
    torch.cuda.synchronize()
    rows, cols = [0, 97, M - 1], [0, 64, N - 1]
    ca, sa = host_rows(a, rows)
    cb, sb = host_rows(b, cols)
    C, bound = O.gemm_tn(ca, sa, cb, sb)
    for name, out in (("fprop", fprop), ("split-K wgrad", split)):
        got = out.cpu().numpy()[np.ix_(rows, cols)]
        check(got, C, bound, name)


def test_grouped_wgrad_at_the_largest_kpad():
    """Token groups of 5000003, 0, 6999997 and 4777191 rows: padded to 16
    each they fill kpad = 2^24 exactly; every product positive."""
    M, N = 144, 130
    counts = [5000003, 0, 6999997, 4777191]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    poff = O.padded_offsets(off)
    assert poff[-1] == KMAX
    print(f"[maxsize] grouped wgrad kpad=2^24 groups={counts}", flush=True)
    a = random_operand(M, KMAX, 103, True)
    b = random_operand(N, KMAX, 104, True)
    dw = U.ufp4_grouped_gemm(U.WGRAD, torch.as_tensor(off, device=DEV), a, b)
    torch.cuda.synchronize()
    assert (dw[1] == 0).all()
    rows, cols = [0, 77, M - 1], [0, 3, N - 1]
    for e, c in enumerate(counts):
        if c == 0:
            continue
        k0, k1 = int(poff[e]), int(poff[e + 1])
        ca, sa = host_rows(a, rows, k0, k1)
        cb, sb = host_rows(b, cols, k0, k1)
        C, bound = O.gemm_tn(ca, sa, cb, sb)
        check(dw[e].cpu().numpy()[np.ix_(rows, cols)], C, bound, f"group {e}")


def oracle_cols(bits, cols, rnd, seed, sid):
    """The oracle's column-wise quantization of the sampled input columns:
    output rows `cols` (their SR indices too)."""
    xb = O.to_blocked_rows(O.bf16_bits_to_f32(bits), O.AXIS_ROWS)
    nib, s = O.quantize_blocked(xb, True, MASK, O.GRID_UNIFORM, rnd, seed, sid, row_ids=cols)
    return O.pack_nibbles(nib), s


@pytest.mark.parametrize("n_cols", [LDMAX, LDMAX - 1])
def test_column_quantize_at_the_largest_row_length(n_cols):
    """17 rows (a full block of 16 and a ragged one) of a row stride 2^26:
    n_cols = 2^26 takes the 8-byte vector loads, 2^26 - 1 the 2-byte ones."""
    print(f"[maxsize] column-wise quantization ld=2^26 n_cols={n_cols}", flush=True)
    full = W.bf16(W.normal((17, LDMAX), 1.0, 105, DEV))
    x = full[:, :n_cols]
    cols = np.array([0, 1, 2, 3, 1000003, (1 << 25) + 17, n_cols - 4, n_cols - 3, n_cols - 2,
                     n_cols - 1], dtype=np.int64)
    bits = W.bits_numpy(x[:, torch.as_tensor(cols, device=DEV)])
    seed = 909
    for rnd in (U.ROUND_RTNE, U.ROUND_SR):
        cq = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_ROWS, True, MASK, U.GRID_UNIFORM, rnd, seed, 1)
        torch.cuda.synchronize()
        codes, scales = oracle_cols(bits, cols, rnd, seed, 1)
        assert np.array_equal(cq.codes[cols].cpu().numpy(), codes), rnd
        assert np.array_equal(cq.scales[cols].cpu().numpy().view(np.uint32),
                              scales.view(np.uint32)), rnd
        rq = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_COLS, True, 0x0F0F, U.GRID_UNIFORM, rnd, seed, 0)
        dr, dc = U.ufp4_rht_quantize_dual(x, (True, 0x0F0F, 0), (True, MASK, 1), rnd=rnd,
                                          seed=seed)
        torch.cuda.synchronize()
        assert torch.equal(dc.codes, cq.codes) and torch.equal(dc.scales, cq.scales), rnd
        assert torch.equal(dr.codes, rq.codes) and torch.equal(dr.scales, rq.scales), rnd
        del cq, rq, dr, dc


def check_bf16(out, C, bound, what):
    """bf16 output: the FP32 result within the bar, then rounded to bf16
    (at most half a bf16 ulp, <= 2^-8 of the value)."""
    o = out.float().cpu().numpy().astype(np.float64)
    lim = TOL * bound + 2.0 ** -8 * (np.abs(C) + TOL * bound)
    err = np.abs(o - C)
    assert (err <= lim).all(), f"{what}: worst err / limit = {(err / lim).max():.3g}"


def test_bf16_outputs_across_chunks():
    """bf16 outputs of contractions several chunks long (the output holds the
    bf16 part of the running result between chunks, the tile the residual):
    a dense GEMM over 2^18 + 48 K-elements and a K-grouped WGRAD with groups
    of 200003, 0 and 70001 tokens, every product positive; all outputs
    against the oracle, and within one bf16 ulp of the FP32 output's
    rounding."""
    M, N, K = 96, 80, (1 << 18) + 48
    print(f"[maxsize] bf16 outputs over {K} K-elements", flush=True)
    a = random_operand(M, K, 111, True)
    b = random_operand(N, K, 112, True)
    bf = U.ufp4_gemm_out(U.WGRAD, a, b, dtype=torch.bfloat16)
    f32 = U.ufp4_gemm_out(U.WGRAD, a, b, dtype=torch.float32)
    torch.cuda.synchronize()
    C, bound = O.gemm_tn(a.codes.cpu().numpy(), a.scales.cpu().numpy(), b.codes.cpu().numpy(),
                         b.scales.cpu().numpy())
    check(f32.cpu().numpy(), C, bound, "dense f32")
    check_bf16(bf, C, bound, "dense bf16")
    near = f32.to(torch.bfloat16).float()
    assert ((bf.float() - near).abs() <= 2.0 ** -7 * near.abs()).all()

    counts = [200003, 0, 70001]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    poff = O.padded_offsets(off)
    kp = int(poff[-1])
    ga = random_operand(M, kp, 113, True)
    gb = random_operand(N, kp, 114, True)
    offd = torch.as_tensor(off, device=DEV)
    gbf = U.ufp4_grouped_gemm_out(U.WGRAD, offd, ga, gb, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert (gbf[1] == 0).all()
    for e, c in enumerate(counts):
        if c == 0:
            continue
        k0, k1 = int(poff[e]), int(poff[e + 1])
        C, bound = O.gemm_tn(ga.codes[:, k0 // 2:k1 // 2].cpu().numpy(),
                             ga.scales[:, k0 // 16:k1 // 16].cpu().numpy(),
                             gb.codes[:, k0 // 2:k1 // 2].cpu().numpy(),
                             gb.scales[:, k0 // 16:k1 // 16].cpu().numpy())
        check_bf16(gbf[e], C, bound, f"grouped bf16 group {e}")


def gemm_bound_check(got, C, bound, what):
    err = np.abs(got.astype(np.float64) - C)
    bad = err > TOL * bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outside"


def test_grouped_at_the_largest_group_count():
    """1024 expert groups, the calls' limit (the GEMMs' and quantizers' group
    tables; above 256 groups the K-grouped WGRAD takes its groups in index
    order instead of heaviest first): counts 0..6 with every fifth group
    empty, so most groups are shorter than a 16-row block.  Grouped
    quantizations (single-axis, stacked and dual-axis) bit-exact against the
    oracle, and FPROP, DGRAD and WGRAD on them element by element."""
    E, H, F = 1024, 48, 32
    counts = np.random.default_rng(7).integers(0, 7, size=E)
    counts[::5] = 0
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T = int(off[-1])
    print(f"[maxsize] {E} groups, {T} rows", flush=True)
    offd = torch.as_tensor(off, device=DEV)
    x = W.bf16(W.normal((T, H), 1.0, 120, DEV))
    w = W.bf16(W.normal((E * F, H), 0.02, 121, DEV))
    dy = W.bf16(W.normal((T, F), 1e-4, 122, DEV))
    m1, m2, m3, seed = 0x1F2E, 0x3D4C, 0x5B6A, 55
    xb, wb, gb = W.bits_numpy(x), W.bits_numpy(w), W.bits_numpy(dy)
    host = lambda t: t.cpu().numpy()

    def same(q, ref, what):
        codes, scales, _ = ref
        assert np.array_equal(host(q.codes), codes), what
        assert np.array_equal(host(q.scales).view(np.uint32), scales.view(np.uint32)), what

    xq = U.ufp4_rht_quantize(x, U.BLOCKS_ALONG_COLS, True, m1)
    wq = U.ufp4_rht_quantize(w, U.BLOCKS_ALONG_COLS, True, m1)
    wtq = U.ufp4_rht_quantize(w, U.BLOCKS_ALONG_ROWS_STACKED, True, m2, n_groups=E)
    dyq = U.ufp4_rht_quantize(dy, U.BLOCKS_ALONG_COLS, True, m2, rnd=U.ROUND_SR, seed=seed)
    dq, dtq = U.ufp4_rht_quantize_dual(dy, (True, m2, 0), (True, m3, 1), rnd=U.ROUND_SR,
                                       seed=seed, group_offsets=offd)
    _, xtq = U.ufp4_rht_quantize_dual(x, (True, m1, 0), (True, m3, 0), group_offsets=offd)
    torch.cuda.synchronize()
    assert torch.equal(dq.codes, dyq.codes) and torch.equal(dq.scales, dyq.scales)
    kp = dtq.kpad
    same(wtq, O.quantize(wb, O.AXIS_ROWS_STACKED, True, m2, O.GRID_UNIFORM, 0, n_stack=E),
         "stacked W^T")
    same(dtq, O.quantize(gb, O.AXIS_ROWS, True, m3, O.GRID_UNIFORM, 1, seed, 1, group_offsets=off,
                         kpad=kp), "grouped dY^T")
    same(xtq, O.quantize(xb, O.AXIS_ROWS, True, m3, O.GRID_UNIFORM, 0, group_offsets=off,
                         kpad=kp), "grouped X^T")

    y = U.ufp4_grouped_gemm(U.FPROP, offd, xq, wq)
    dx = U.ufp4_grouped_gemm(U.DGRAD, offd, dyq, wtq)
    dw = U.ufp4_grouped_gemm(U.WGRAD, offd, dtq, xtq)
    torch.cuda.synchronize()
    C, bnd = O.grouped_gemm(0, off, host(xq.codes), host(xq.scales), host(wq.codes),
                            host(wq.scales), F)
    gemm_bound_check(host(y), C, bnd, "fprop")
    C, bnd = O.grouped_gemm(1, off, host(dyq.codes), host(dyq.scales), host(wtq.codes),
                            host(wtq.scales), H)
    gemm_bound_check(host(dx), C, bnd, "dgrad")
    C, bnd = O.grouped_gemm(2, off, host(dtq.codes), host(dtq.scales), host(xtq.codes),
                            host(xtq.scales), 0)
    gemm_bound_check(host(dw), C, bnd, "wgrad")
    assert (host(dw)[counts == 0] == 0).all()


def test_m_grouped_gemm_across_chunks():
    """Grouped FPROP (groups along M) over 2^17 + 16 K-elements, two chunks
    and a remainder, every product positive: FP32 and bf16 outputs against
    the oracle."""
    counts = [70, 0, 200, 33]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    T, E, N, K = int(off[-1]), len(counts), 72, (1 << 17) + 16
    print(f"[maxsize] M-grouped FPROP over {K} K-elements", flush=True)
    a = random_operand(T, K, 131, True)
    b = random_operand(E * N, K, 132, True)
    offd = torch.as_tensor(off, device=DEV)
    f32 = U.ufp4_grouped_gemm(U.FPROP, offd, a, b)
    bf = U.ufp4_grouped_gemm_out(U.FPROP, offd, a, b, torch.bfloat16)
    torch.cuda.synchronize()
    C, bound = O.grouped_gemm(0, off, a.codes.cpu().numpy(), a.scales.cpu().numpy(),
                              b.codes.cpu().numpy(), b.scales.cpu().numpy(), N)
    check(f32.cpu().numpy(), C, bound, "M-grouped f32")
    check_bf16(bf, C, bound, "M-grouped bf16")
