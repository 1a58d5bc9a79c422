"""Op-level parity of the HIP library against the oracle on seeded inputs:
bit-exact for quantised codes, scales, routing and permutation, SiLU-requant
and combine; the float32 summation bound for the grouped GEMM.  Shapes cover
several tiles, ragged tails, empty groups and the degenerate cases."""
import numpy as np
import pytest
import torch

from _helpers import (F32, bf16_tensor, check_gemm, dev, exact_gemm_rows, log, oracle_nvfp4, to_np)
from block_scaled_fp4_03_amd import ops
from oracle import formats, fp8, moe, quant

pytestmark = pytest.mark.gpu


def _x(rows, cols, seed, outliers=True, scale=1.0):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * scale).astype(np.float32)
    if outliers and x.size >= 1000:
        pos = rng.choice(x.size, x.size // 1000, replace=False)
        x.reshape(-1)[pos] *= 20
    if rows > 1 and cols >= 32:
        x[0, :16] = 0.0
        x[1, 16:32] *= np.float32(1e-7)
    return formats.bf16_round(x)


# --- quantise ---------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,dtype", [(1, 16, "bf16"), (7, 48, "f32"), (33, 256, "bf16"),
                                             (300, 7168, "bf16"), (64, 3072, "f32")])
def test_quantize_bit_exact(rows, cols, dtype):
    log("quantize", rows, cols, dtype)
    x = _x(rows, cols, rows + cols)
    gs = quant.global_scale(quant.amax(x))
    c_ref, s_ref = quant.quantize(x, gs)
    xt = bf16_tensor(x, dev()) if dtype == "bf16" else torch.from_numpy(x).to(dev())
    gst = torch.tensor([gs], dtype=torch.float32, device=dev())
    c, s = ops.quantize(xt, gst)
    assert np.array_equal(to_np(c), c_ref)
    assert np.array_equal(to_np(s), s_ref)
    # with the f16 form: same codes, and dq = e2m1 * e4m3 exactly
    c2, s2, dq = ops.quantize(xt, gst, dq=True)
    assert np.array_equal(to_np(c2), c_ref) and np.array_equal(to_np(s2), s_ref)
    assert np.array_equal(to_np(dq).astype(np.float64), quant.dequantize_blocks(c_ref, s_ref))


def test_quantize_saturation_and_tiny_gs():
    log("quantize saturation")
    x = _x(16, 128, 3)
    for gs in [F32(0.00025141), F32(1e-6), F32(7.5), F32(1e-30)]:
        c_ref, s_ref = quant.quantize(x, gs)
        c, s = ops.quantize(bf16_tensor(x, dev()), torch.tensor([gs], device=dev()))
        assert np.array_equal(to_np(c), c_ref) and np.array_equal(to_np(s), s_ref), gs


def test_quantize_rounding_ties_and_signs():
    """Every E2M1 rounding midpoint, both signs, signed zeros and values just
    either side of a midpoint, in blocks whose reciprocal is exactly 1 (gs = 1,
    block maximum 6), so each value reaches the encoder unchanged."""
    log("quantize ties")
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    vals = []
    for m in mids:
        vals += [m, -m, float(np.nextafter(F32(m), F32(0))), float(np.nextafter(F32(m), F32(8)))]
    vals += [0.0, -0.0, 6.0, -6.0]
    vals = np.array(vals, dtype=np.float32)
    blocks = []
    for b0 in range(0, len(vals), 15):
        chunk = vals[b0:b0 + 15]
        blk = np.zeros(16, dtype=np.float32)
        blk[0] = 6.0                        # the block maximum: scale 1
        blk[1:1 + len(chunk)] = chunk
        blocks.append(blk)
    x = np.stack(blocks).reshape(1, -1).repeat(3, axis=0)
    x[1] *= -1.0
    gs = F32(1.0)
    c_ref, s_ref = quant.quantize(x, gs)
    assert (s_ref == 0x38).all()           # E4M3 1.0 everywhere
    c, s = ops.quantize(torch.from_numpy(x).to(dev()), torch.tensor([gs], device=dev()))
    assert np.array_equal(to_np(s), s_ref)
    assert np.array_equal(to_np(c), c_ref)


def test_quantize_reciprocal_overflow():
    """A subnormal global scale: blocks whose 1/(sf*gs) overflows to inf take
    the comparison encoder (zeros stay zero), the rest the packed conversion."""
    log("quantize reciprocal overflow")
    x = _x(8, 64, 9).astype(np.float32)
    x[2, :16] = 0.0
    x[2, 1], x[2, 2], x[2, 3] = F32(5e-39), F32(-1e-39), F32(-0.0)
    x[3, 16:32] *= F32(1e-38)
    for gs in [F32(1e-40), F32(3e-39)]:
        c_ref, s_ref = quant.quantize(x, gs)
        c, s = ops.quantize(torch.from_numpy(x).to(dev()), torch.tensor([gs], device=dev()))
        assert np.array_equal(to_np(c), c_ref) and np.array_equal(to_np(s), s_ref), gs


def test_quantize_row_pitch_and_empty():
    log("quantize pitch")
    x = _x(9, 96, 4)
    big = np.zeros((9, 128), dtype=np.float32)
    big[:, :96] = x
    gs = quant.global_scale(quant.amax(x))
    t = bf16_tensor(big, dev())[:, :96]
    c, s = ops.quantize(t, torch.tensor([gs], device=dev()))
    c_ref, s_ref = quant.quantize(x, gs)
    assert np.array_equal(to_np(c), c_ref) and np.array_equal(to_np(s), s_ref)
    c0, s0 = ops.quantize(torch.empty(0, 64, dtype=torch.bfloat16, device=dev()), torch.ones(1, device=dev()))
    assert c0.shape == (0, 32)


def test_global_scale_bit_exact():
    log("global_scale")
    x = _x(48, 7168, 5)
    t = torch.from_numpy(x).to(dev())
    g = to_np(ops.global_scale(t.reshape(1, -1)))
    assert g[0] == quant.global_scale(quant.amax(x))
    rows = to_np(ops.global_scale(t))            # a 2-D tensor: one scale per row
    assert all(rows[i] == quant.global_scale(quant.amax(x[i])) for i in range(x.shape[0]))
    g2 = to_np(ops.global_scale(t.reshape(4, -1)))
    for b in range(4):
        assert g2[b] == quant.global_scale(quant.amax(x.reshape(4, -1)[b]))
    gb = to_np(ops.global_scale(bf16_tensor(x, dev()).reshape(-1)))
    assert gb[0] == g[0]
    z = to_np(ops.global_scale(torch.zeros(2, 64, device=dev())))
    assert (z == 1.0).all()


# --- routing and permutation --------------------------------------------------

def _route_case(T, E, k, seed, zipf=0.0, ties=False):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if zipf:
        rank = rng.permutation(E) + 1.0
        lg = (lg + (-zipf * np.log(rank)).astype(np.float32)).astype(np.float32)
    if ties:
        lg = np.round(lg * 2).astype(np.float32) / 2
        lg[::3] = 0.0
        lg[1::5, ::2] = -0.0
    return lg


@pytest.mark.parametrize("T,E,k,zipf,ties", [(16, 8, 2, 0, False), (256, 384, 6, 0, False),
                                             (8192, 384, 6, 1.1, False), (100, 384, 6, 0, True),
                                             (5, 1, 1, 0, False), (3, 16, 16, 0, True),
                                             (77, 1024, 16, 0, False), (1, 64, 6, 0, True),
                                             (3001, 384, 7, 1.1, False), (4096, 1024, 8, 0.5, True)])
def test_route_permute_bit_exact(T, E, k, zipf, ties):
    # R = T * k entries: up to 4096 in one block, else in blocks of 4096 (the
    # last one ragged) with a table of first positions between the passes
    log("route", T, E, k, zipf, ties)
    lg = _route_case(T, E, k, T * 7 + E, zipf, ties)
    ids_r, w_r = moe.route_topk(lg, k)
    off_r, srt_r, inv_r = moe.permute(ids_r, E)
    ids, w, off, srt, inv = ops.route_permute(torch.from_numpy(lg).to(dev()), k)
    assert np.array_equal(to_np(ids), ids_r)
    assert np.array_equal(to_np(w).view(np.uint32), w_r.view(np.uint32))
    assert np.array_equal(to_np(off), off_r)
    assert np.array_equal(to_np(srt), srt_r)
    assert np.array_equal(to_np(inv), inv_r)


@pytest.mark.parametrize("T,E,k,ns,ties", [(16, 8, 2, 1, False), (256, 384, 6, 1, False), (100, 384, 6, 2, True),
                                           (5, 1, 1, 1, False), (3, 16, 15, 1, True), (1, 1022, 6, 2, False),
                                           (8192, 384, 6, 1, False)])
def test_route_permute_shared_bit_exact(T, E, k, ns, ties):
    # the shared experts folded in: routed slots as without them, then slots
    # k.. with ids E.. and weight 1; the permutation over E + ns groups
    log("route shared", T, E, k, ns, ties)
    lg = _route_case(T, E, k, T * 11 + E, 0.0, ties)
    ids_r, w_r = moe.append_shared(*moe.route_topk(lg, k), E, ns)
    off_r, srt_r, inv_r = moe.permute(ids_r, E + ns)
    ids, w, off, srt, inv = ops.route_permute(torch.from_numpy(lg).to(dev()), k, n_shared=ns)
    assert np.array_equal(to_np(ids), ids_r)
    assert np.array_equal(to_np(w).view(np.uint32), w_r.view(np.uint32))
    assert np.array_equal(to_np(off), off_r)
    assert np.array_equal(to_np(srt), srt_r)
    assert np.array_equal(to_np(inv), inv_r)
    _, _, off0, _, _ = ops.route_permute(torch.empty(0, E, device=dev()), k, n_shared=ns)
    assert off0.shape == (E + ns + 1,) and (to_np(off0) == 0).all()


def test_route_permute_empty_batch():
    ids, w, off, srt, inv = ops.route_permute(torch.empty(0, 8, device=dev()), 2)
    assert (to_np(off) == 0).all()


# --- grouped GEMM ---------------------------------------------------------------

def _gemm_case(counts, N, K, n_seg, seed, gather=False, out_bf16=False, a_extra=3):
    log("gemm", counts if len(counts) < 12 else (len(counts), sum(counts)), N, K, n_seg, gather, out_bf16)
    rng = np.random.default_rng(seed)
    G = len(counts)
    M = int(sum(counts))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a_rows = M + a_extra if gather else M
    ac, as_, ags = oracle_nvfp4(_x(max(a_rows, 1), K, seed, outliers=True))
    ac, as_ = ac[:a_rows], as_[:a_rows]
    row_index = rng.integers(0, a_rows, M).astype(np.int32) if gather else None
    S = len(n_seg) - 1
    wc = np.empty((G, N, K // 2), np.uint8)
    ws = np.empty((G, N, K // 16), np.uint8)
    wgs = np.empty((G, S), np.float32)
    for g in range(G):
        wf = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        for s in range(S):
            r0, r1 = n_seg[s], n_seg[s + 1]
            c, sc, gg = oracle_nvfp4(wf[r0:r1])
            wc[g, r0:r1], ws[g, r0:r1], wgs[g, s] = c, sc, gg
    d = dev()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    args = (T(ac), T(as_), torch.tensor([ags], device=d), T(wc), T(ws), T(wgs), n_seg, T(off), M)
    kw = dict(a_row_index=T(row_index) if gather else None, out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    out = ops.grouped_gemm(*args, **kw)
    got = to_np(out)
    outs = [("rows", got)]
    if K % 256 == 0:
        # the tiled weight layout (which may route many-row groups to another
        # kernel) is checked against the same bound
        tiled = ops.prepare_weights(T(wc), T(ws))
        outs.append(("tiled", to_np(ops.grouped_gemm(*args, w_tiled=tiled, **kw))))
        if ops.gemm_workspace_size(G, M, N, K, True) > 0:
            # the same without a split-K workspace: the one-pass kernels
            outs.append(("tiled, one pass", to_np(ops.grouped_gemm(*args, w_tiled=tiled, workspace=False, **kw))))
        if ops.gemm_reads_dq(G, M, K, a_rows, True):
            # A also in f16 form (from the oracle's dequantisation): the
            # many-row kernel copies it instead of decoding the codes.  Rows in
            # full 256-row tiles see the same products in the same order as
            # without it, so they are identical; the rest (the last tile of
            # each group) is checked against the bound below
            a_dq = T(quant.dequantize_blocks(ac, as_).astype(np.float16))
            o_dq = to_np(ops.grouped_gemm(*args, w_tiled=tiled, a_dq=a_dq, **kw))
            if ops.gemm_workspace_size(G, M, N, K, True) == 0:
                # (a split K adds the same products in another order: then
                # only the bound below applies)
                for g in range(G):
                    full = (off[g + 1] - off[g]) // 256 * 256
                    assert np.array_equal(o_dq[off[g]:off[g] + full], outs[-1][1][off[g]:off[g] + full]), g
            else:
                # split K is deterministic, and without the workspace the
                # one-pass kernel gives the same rows within the bound
                assert np.array_equal(o_dq, to_np(ops.grouped_gemm(*args, w_tiled=tiled, a_dq=a_dq, **kw)))
                outs.append(("tiled+dq, one pass", to_np(ops.grouped_gemm(*args, w_tiled=tiled, a_dq=a_dq,
                                                                          workspace=False, **kw))))
            outs.append(("tiled+dq", o_dq))
    # oracle (the definition) and the float64 pieces for the error bound
    ref_o = moe.grouped_gemm(ac, as_, ags, wc, ws, wgs, n_seg, off, a_row_index=row_index,
                             out_dtype="bf16" if out_bf16 else "f32")
    A_idx = row_index if gather else np.arange(M)
    worst = 0.0
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r1 == r0:
            continue
        ex, ab = exact_gemm_rows(ac[A_idx[r0:r1]], as_[A_idx[r0:r1]], wc[g], ws[g])
        alpha = np.empty(N)
        for s in range(S):
            alpha[n_seg[s]:n_seg[s + 1]] = float(F32(F32(ags) * wgs[g, s]))
        for name, o in outs:
            worst = max(worst, check_gemm(o[r0:r1], ex, ab, alpha[None, :], K, out_bf16, "%s group %d" % (name, g)))
            # and against the oracle's own rounded output
            assert np.allclose(o[r0:r1], ref_o[r0:r1], rtol=2 ** -7 if out_bf16 else 1e-4,
                               atol=np.abs(ref_o[r0:r1]).max() * 1e-4 + 1e-30)
    log("  max err / rms = %.3g (%s)" % (worst, ", ".join(n for n, _ in outs)))
    return got


def test_gemm_one_group_plain():
    _gemm_case([64], 128, 256, [0, 128], 1)


def test_gemm_decode_shaped_many_groups_with_empty():
    rng = np.random.default_rng(2)
    counts = rng.integers(0, 12, 40).tolist()
    counts[3] = 0
    counts[-1] = 0
    _gemm_case(counts, 320, 1024, [0, 160, 320], 2, gather=True)


def test_gemm_rows_over_16_per_group_and_ragged_n():
    _gemm_case([17, 1, 33, 0, 5], 200, 512, [0, 100, 200], 3, gather=True, out_bf16=True)


def test_gemm_streaming_runs_of_column_tiles():
    # few rows per group and 2K/256 divisible by 3: the streaming kernel takes
    # runs of column tiles per workgroup; a ragged last tile and last run, a
    # group of two 32-row slots, an empty group, a segment boundary inside a
    # column block
    rng = np.random.default_rng(41)
    counts = rng.integers(0, 12, 24).tolist()
    counts[2] = 0
    counts[5] = 40
    _gemm_case(counts, 1320, 768, [0, 500, 1320], 41, gather=True, out_bf16=True)
    _gemm_case(counts[:10], 1064, 1536, [0, 1064], 42)


def test_gemm_k_tails():
    for K in (32, 96, 160, 288, 320, 544, 576):
        _gemm_case([5, 9], 72, K, [0, 72], 4 + K)


def test_gemm_tile_kernel_shapes():
    # enough rows per group for the tiled kernels; ragged M and N tails
    _gemm_case([300, 130, 0, 77], 200, 256, [0, 64, 200], 5, gather=True)
    _gemm_case([513], 384, 512, [0, 384], 6, out_bf16=True)


def test_gemm_big_tiles_with_remainders():
    # full 256-row tiles plus left-over rows of 1..255 in several groups,
    # column tiles with a partial last one, two segments
    _gemm_case([456, 3, 256, 0, 611, 70], 520, 512, [0, 260, 520], 12, gather=True)
    _gemm_case([1024, 255, 257], 256, 768, [0, 256], 13, out_bf16=True)


def test_gemm_tiles_from_16_or_32_rows_per_group():
    # 16..64 rows per group on average: the matrix-core tiles from 32 rows
    # per group (16 where K <= 4096), each group's rows as 32/64/128-row
    # tiles; with an empty group, a group of two slots, partial column tiles
    assert ops.gemm_reads_dq(7, 336, 512, 336, True)
    assert ops.gemm_reads_dq(16, 16 * 17, 4096, 16 * 17, True)
    assert not ops.gemm_reads_dq(16, 16 * 17, 4352, 16 * 17, True)
    _gemm_case([40, 55, 0, 47, 63, 41, 90], 320, 512, [0, 160, 320], 31, gather=True)
    _gemm_case([17] * 15 + [30], 320, 4096, [0, 320], 35, gather=True, out_bf16=True)
    # below 256 rows in all: the streaming kernel
    assert not ops.gemm_reads_dq(5, 224, 768, 224, True)
    _gemm_case([65, 44, 50, 64, 1], 200, 768, [0, 200], 32, gather=True, out_bf16=True)


def test_gemm_big_tiles_every_last_tile_height():
    # group sizes whose last tile takes each form: with A in f16 form a
    # 32-, 64- or 128-row tile past the full 128-row tiles; without it (the
    # 256-row kernel) the streaming kernel takes the left-over rows 1, 31,
    # 32, 33, 64, 65, 128, 129, 255
    _gemm_case([257, 287, 288, 289, 320, 321, 384, 385, 511, 256], 96, 256, [0, 40, 96], 14, gather=True)
    _gemm_case([257, 288, 289, 320, 321, 384, 385], 64, 4608, [0, 64], 17, gather=True)


def test_gemm_big_tiles_last_tile_heights_at_model_depths():
    # the last-tile forms at the depths of the MoE layer's two GEMMs (K = 7168
    # for gate_up, 3072 for down): left-over rows past the full 128-row tiles
    # as a 32-, 64- or 128-row tile
    _gemm_case([257, 300, 320, 321, 384, 385, 511, 64], 64, 7168, [0, 32, 64], 33, gather=True)
    _gemm_case([260, 289, 330, 400, 449, 600, 33], 96, 3072, [0, 96], 34, gather=True, out_bf16=True)


def test_gemm_left_over_rows_beyond_one_round_of_the_persistent_grid():
    # 400 groups of 257..320 rows at N = 1024.  Without A's f16 form each
    # group's 1..64 rows past its 256-row tile go to the persistent streaming
    # kernel, about 600 32-row slots x 4 column tiles = 2400 tiles for its
    # 768 workgroups, so every workgroup runs several rounds; with it they
    # are 32- and 64-row tiles of the 128-row launch.  Codes and scales are
    # random bytes (any NVFP4 operand is valid input).
    log("gemm left-over rounds")
    rng = np.random.default_rng(40)
    G, N, K = 400, 1024, 256
    counts = rng.integers(257, 321, G)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    as_ = rng.integers(0x28, 0x49, (M, K // 16), dtype=np.uint8)
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    ws = rng.integers(0x20, 0x41, (G, N, K // 16), dtype=np.uint8)
    wgs = rng.uniform(0.5, 2.0, (G, 1)).astype(np.float32)
    ags = F32(1.0 / 64)
    slots = int(((counts - 256 + 31) // 32).sum())
    assert slots * (N // 256) > 3 * 768
    d = dev()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    assert ops.gemm_reads_dq(G, M, K, M, True)
    tiled = ops.prepare_weights(T(wc), T(ws))
    a_dq = T(quant.dequantize_blocks(ac, as_).astype(np.float16))
    for dq in (None, a_dq):
        out = to_np(ops.grouped_gemm(T(ac), T(as_), torch.tensor([ags], device=d), T(wc), T(ws), T(wgs), [0, N],
                                     T(off), M, w_tiled=tiled, a_dq=dq))
        worst = 0.0
        for g in range(G):
            r0, r1 = int(off[g]), int(off[g + 1])
            # every left-over row, and 8 rows of the group's first 256 rows
            rows = np.concatenate([np.arange(r0 + 256, r1), r0 + rng.choice(256, 8, replace=False)])
            ex, ab = exact_gemm_rows(ac[rows], as_[rows], wc[g], ws[g])
            worst = max(worst, check_gemm(out[rows], ex, ab, float(F32(ags * wgs[g, 0])), K, False, "group %d" % g))
        log("  %s: %d left-over slots x %d column tiles; max err / rms = %.3g" % (
            "f16 A" if dq is not None else "codes A", slots, N // 256, worst))


def test_gemm_big_tiles_split_k_one_group():
    # one group with few 128-row tiles: K is split over them (f16 A, 8
    # ranges), every row, the last partial slot (50 or 12 rows) included,
    # from the split tiles and the reduction
    assert ops.gemm_workspace_size(1, 562, 512, 2048, True) > 0
    _gemm_case([562], 512, 2048, [0, 300, 512], 18)
    _gemm_case([652], 512, 2048, [0, 512], 19, gather=True, out_bf16=True)


def test_gemm_split_k_one_small_group():
    # few workgroups: the tiled path splits K (4 ranges here) and reduces in
    # order; checked against the bound in both output dtypes, without the
    # workspace too, and for determinism
    _gemm_case([100], 320, 2048, [0, 160, 320], 15, gather=False)
    _gemm_case([61, 40], 256, 2048, [0, 256], 16, gather=True, out_bf16=True)
    # the reduction's four-column lanes: a segment boundary inside one
    # lane's columns; N % 4 != 0 (one column per lane)
    _gemm_case([100], 320, 2048, [0, 162, 320], 36, gather=False)
    _gemm_case([70], 322, 2048, [0, 322], 37, gather=False, out_bf16=True)
    d = dev()
    rng = np.random.default_rng(17)
    ac, as_, ags = oracle_nvfp4(_x(100, 2048, 17))
    wf = (rng.standard_normal((320, 2048)) * 0.02).astype(np.float32)
    wc, ws, wg = oracle_nvfp4(wf)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    tiled = ops.prepare_weights(T(wc[None]), T(ws[None]))
    args = (T(ac), T(as_), torch.tensor([ags], dtype=torch.float32, device=d), T(wc[None]), T(ws[None]),
            torch.tensor([[wg]], dtype=torch.float32, device=d),
            [0, 320], torch.tensor([0, 100], dtype=torch.int32, device=d), 100)
    assert ops.gemm_workspace_size(1, 100, 320, 2048, True) > 0
    a1 = to_np(ops.grouped_gemm(*args, w_tiled=tiled))
    a2 = to_np(ops.grouped_gemm(*args, w_tiled=tiled))
    a3 = to_np(ops.grouped_gemm(*args, w_tiled=tiled, workspace=False))
    assert np.array_equal(a1, a2)                       # deterministic
    for dt in (torch.float32, torch.bfloat16):
        # rows of 322 elements: the reduction stores column by column, with
        # the same values as into whole rows
        wide = torch.full((100, 322), 7.0, dtype=dt, device=d)
        ops.grouped_gemm(*args, w_tiled=tiled, out=wide[:, :320])
        whole = ops.grouped_gemm(*args, w_tiled=tiled, out_dtype=dt)
        assert torch.equal(wide[:, :320], whole) and bool((wide[:, 320:] == 7.0).all())
    ex, ab = exact_gemm_rows(ac, as_, wc, ws)
    for o in (a1, a3):
        check_gemm(o, ex, ab, float(F32(F32(ags) * wg)), 2048, False, "split-K")


def _mlp_case(counts, H, I, seed, gather=True):
    """nvfp4_moe_expert_mlp (one persistent launch) against the two launches
    it replaces and the oracle: h bit-identical to the fused first GEMM and
    to the oracle's SiLU-requant of the unfused first GEMM's float32 output;
    y bit-identical to the second grouped GEMM (same streaming tiles) and
    within the float32 summation bound of the exact contraction of h."""
    log("expert mlp", counts if len(counts) < 12 else (len(counts), sum(counts)), H, I, gather)
    rng = np.random.default_rng(seed)
    G = len(counts)
    R = int(sum(counts))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = max(R // 3, 1) if gather else R
    xc, xs, xg = oracle_nvfp4(_x(T, H, seed))
    sorted_ids = rng.integers(0, T, R).astype(np.int32) if gather else None
    w1c = np.empty((G, 2 * I, H // 2), np.uint8)
    w1s = np.empty((G, 2 * I, H // 16), np.uint8)
    w1g = np.empty((G, 2), np.float32)
    w2c = np.empty((G, H, I // 2), np.uint8)
    w2s = np.empty((G, H, I // 16), np.uint8)
    w2g = np.empty((G, 1), np.float32)
    for g in range(G):
        wf = (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32)
        for sg in range(2):
            c, sc, gg = oracle_nvfp4(wf[sg * I:(sg + 1) * I])
            w1c[g, sg * I:(sg + 1) * I], w1s[g, sg * I:(sg + 1) * I], w1g[g, sg] = c, sc, gg
        w2c[g], w2s[g], w2g[g, 0] = oracle_nvfp4((rng.standard_normal((H, I)) * 0.02).astype(np.float32))
    d = dev()
    Td = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    x_gs = torch.tensor([xg], device=d)
    gs_h = torch.tensor([0.004], dtype=torch.float32, device=d)
    t1 = ops.prepare_weights(Td(w1c), Td(w1s))
    t2 = ops.prepare_weights(Td(w2c), Td(w2s))
    sid = Td(sorted_ids) if gather else None
    offs = Td(off)
    hc, hs, y = ops.moe_expert_mlp(Td(xc), Td(xs), x_gs, sid, offs, t1, Td(w1g), t2, Td(w2g), R, H, I, gs_h)
    # the two launches it replaces
    hc2, hs2 = ops.grouped_gemm_silu_requant(Td(xc), Td(xs), x_gs, t1, Td(w1g), offs, R, I, H, gs_h,
                                             a_row_index=sid)
    y2 = ops.grouped_gemm(hc2, hs2, gs_h, Td(w2c), Td(w2s), Td(w2g), [0, H], offs, R, w_tiled=t2,
                          out_dtype=torch.bfloat16, workspace=False)
    gu = to_np(ops.grouped_gemm(Td(xc), Td(xs), x_gs, Td(w1c), Td(w1s), Td(w1g), [0, I, 2 * I], offs, R,
                                a_row_index=sid, w_tiled=t1, workspace=False))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(hc), to_np(hc2)) and np.array_equal(to_np(hs), to_np(hs2))
    hc_o, hs_o = moe.silu_mul_requant(gu, F32(0.004))
    assert np.array_equal(to_np(hc), hc_o) and np.array_equal(to_np(hs), hs_o)
    yn = to_np(y)
    assert np.array_equal(yn.view(np.uint32), to_np(y2).view(np.uint32))
    hcn, hsn = to_np(hc), to_np(hs)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r1 > r0:
            ex, ab = exact_gemm_rows(hcn[r0:r1], hsn[r0:r1], w2c[g], w2s[g])
            check_gemm(yn[r0:r1], ex, ab, float(F32(F32(0.004) * w2g[g, 0])), I, True, "expert mlp group %d" % g)


def test_moe_expert_mlp_one_launch_matches_two():
    # decode-like: few rows per group, empty groups, gathered rows
    rng = np.random.default_rng(50)
    counts = rng.integers(0, 9, 48).tolist()
    counts[0] = 0
    counts[-1] = 0
    _mlp_case(counts, 512, 256, 51)
    # groups of several 32-row slots (slot tiles that are not the whole group)
    _mlp_case([70, 0, 33, 5, 100], 256, 512, 52)
    # one group, rows not gathered
    _mlp_case([40], 768, 256, 53, gather=False)


def test_moe_expert_mlp_many_tiles_in_the_queue():
    # 300 groups: about 9k tiles through the device queue for 768 workgroups
    rng = np.random.default_rng(54)
    _mlp_case(rng.integers(0, 7, 300).tolist(), 256, 256, 55)


def test_moe_expert_mlp_bounded_wait_gives_up_and_finishes():
    # failure handling forced from the host: with one poll allowed, second-GEMM
    # tiles that start before their slot's h is complete give up at once; the
    # launch must still finish (no hang), the timeout is recorded in the
    # status word, and a normal call afterwards is correct again
    import os
    rng = np.random.default_rng(56)
    counts = rng.integers(1, 9, 200).tolist()
    R, H, I = int(sum(counts)), 512, 256
    d = dev()
    G = len(counts)
    xc = torch.randint(0, 256, (R, H // 2), dtype=torch.uint8, device=d)
    xs = torch.full((R, H // 16), 0x38, dtype=torch.uint8, device=d)
    w1 = ops.prepare_weights(torch.randint(0, 256, (G, 2 * I, H // 2), dtype=torch.uint8, device=d),
                             torch.full((G, 2 * I, H // 16), 0x30, dtype=torch.uint8, device=d))
    w2 = ops.prepare_weights(torch.randint(0, 256, (G, H, I // 2), dtype=torch.uint8, device=d),
                             torch.full((G, H, I // 16), 0x30, dtype=torch.uint8, device=d))
    g1 = torch.full((G, 2), 0.01, device=d)
    g2 = torch.full((G, 1), 0.01, device=d)
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(d)
    one = torch.ones(1, device=d)
    ws = torch.zeros(ops._lib.load().nvfp4_moe_expert_mlp_workspace_size(G, R), dtype=torch.uint8, device=d)
    args = (xc, xs, one, None, off, w1, g1, w2, g2, R, H, I, one)
    os.environ["NVFP4MOE_SPIN_LIMIT"] = "1"
    try:
        ops.moe_expert_mlp(*args, workspace=ws)
        torch.cuda.synchronize()
    finally:
        del os.environ["NVFP4MOE_SPIN_LIMIT"]
    status = int(ws[4:8].view(torch.int32).item())
    log("  status after the one-poll launch: %d" % status)
    assert status in (0, 1)
    hc, hs, y = ops.moe_expert_mlp(*args, workspace=ws)
    hc2, hs2 = ops.grouped_gemm_silu_requant(xc, xs, one, w1, g1, off, R, I, H, one)
    torch.cuda.synchronize()
    assert int(ws[4:8].view(torch.int32).item()) == 0
    assert torch.equal(hc, hc2) and torch.equal(hs, hs2)


def test_gemm_four_segments_and_bf16():
    _gemm_case([70, 70], 256, 128, [0, 32, 100, 160, 256], 7, out_bf16=True)


def test_gemm_empty_m():
    d = dev()
    z = torch.zeros(0, 32, dtype=torch.uint8, device=d)
    out = ops.grouped_gemm(z, torch.zeros(0, 4, dtype=torch.uint8, device=d), torch.ones(1, device=d),
                           torch.zeros(1, 16, 32, dtype=torch.uint8, device=d),
                           torch.zeros(1, 16, 4, dtype=torch.uint8, device=d), torch.ones(1, 1, device=d),
                           [0, 16], torch.zeros(2, dtype=torch.int32, device=d), 0)
    assert out.shape == (0, 16)


def test_prepare_weights_is_the_documented_permutation():
    log("prepare layout")
    rng = np.random.default_rng(11)
    G, N, K = 2, 37, 512
    wc = rng.integers(0, 256, (G, N, K // 2), dtype=np.uint8)
    ws = rng.integers(0, 127, (G, N, K // 16), dtype=np.uint8)
    out = to_np(ops.prepare_weights(torch.from_numpy(wc).to(dev()), torch.from_numpy(ws).to(dev())))
    NB, KS = (N + 31) // 32, K // 256
    assert out.size == G * NB * KS * 4608
    t = out.reshape(G, NB, KS, 4608)
    for g in range(G):
        for nb in range(NB):
            for ks in range(KS):
                for h in range(2):
                    for l in range(64):
                        c, kh = l % 32, l // 32
                        row = nb * 32 + c
                        c0 = t[g, nb, ks, 2048 * h + 16 * l:2048 * h + 16 * l + 16]
                        c1 = t[g, nb, ks, 2048 * h + 1024 + 16 * l:2048 * h + 1024 + 16 * l + 16]
                        sc = t[g, nb, ks, 4096 + 256 * h + 4 * l:4096 + 256 * h + 4 * l + 4]
                        if row < N:
                            base = ks * 128 + 64 * h + 32 * kh
                            assert np.array_equal(c0, wc[g, row, base:base + 16])
                            assert np.array_equal(c1, wc[g, row, base + 16:base + 32])
                            sb = ks * 16 + 8 * h + 4 * kh
                            assert np.array_equal(sc, ws[g, row, sb:sb + 4])
                        else:
                            assert not c0.any() and not c1.any() and not sc.any()


def test_gemm_deterministic():
    a = _gemm_case([9, 40, 3], 256, 512, [0, 256], 8, gather=True)
    b = _gemm_case([9, 40, 3], 256, 512, [0, 256], 8, gather=True)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# --- fused first GEMM + SiLU-requant ----------------------------------------------

def _fused_case(counts, I, K, seed, gather=True, use_dq=False, split=None, extra_rows=0):
    """nvfp4_grouped_gemm_silu_requant against the unfused pair (grouped
    GEMM to float32, then silu_mul_requant): codes, scales and the f16 copy
    must be identical.  Both GEMMs get the split-K workspace the library
    asks for, or none with split=False; split=True asserts that K is split.
    extra_rows: M exceeds the last group offset by that many rows, which
    every call must leave untouched."""
    log("fused gemm+silu", counts if len(counts) < 12 else (len(counts), sum(counts)), I, K, gather, use_dq, split,
        extra_rows)
    rng = np.random.default_rng(seed)
    G, M = len(counts), int(sum(counts)) + extra_rows
    Mg = int(sum(counts))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a_rows = M + 5 if gather else M
    ac, as_, ags = oracle_nvfp4(_x(a_rows, K, seed, outliers=True))
    row_index = rng.integers(0, a_rows, M).astype(np.int32) if gather else None
    N = 2 * I
    wc = np.empty((G, N, K // 2), np.uint8)
    ws = np.empty((G, N, K // 16), np.uint8)
    wgs = np.empty((G, 2), np.float32)
    for g in range(G):
        wf = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        for sg in range(2):
            c, sc, gg = oracle_nvfp4(wf[sg * I:(sg + 1) * I])
            wc[g, sg * I:(sg + 1) * I], ws[g, sg * I:(sg + 1) * I], wgs[g, sg] = c, sc, gg
    d = dev()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    tiled = ops.prepare_weights(T(wc), T(ws))
    a_dq = T(quant.dequantize_blocks(ac, as_).astype(np.float16)) if use_dq else None
    ri = T(row_index) if gather else None
    args = (T(ac), T(as_), torch.tensor([ags], device=d))
    if split is True:
        assert ops.gemm_workspace_size(G, M, N, K, True) > 0
    wsp = False if split is False else None
    gu = ops.grouped_gemm(*args, T(wc), T(ws), T(wgs), [0, I, N], T(off), M, a_row_index=ri, w_tiled=tiled,
                          a_dq=a_dq, workspace=wsp)
    gs_h = ops.silu_mul_global_scale(gu[:Mg])
    hc, hs, hdq = ops.silu_mul_requant(gu[:Mg].contiguous(), gs_h, dq=True)
    # sentinels: rows outside every group stay untouched
    fc = torch.full((M, I // 2), 0xA5, dtype=torch.uint8, device=d)
    fs = torch.full((M, I // 16), 0x5A, dtype=torch.uint8, device=d)
    fq = torch.full((M, I), 0x3C00, dtype=torch.int16, device=d).view(torch.float16)
    fc, fs, fdq = ops.grouped_gemm_silu_requant(*args, tiled, T(wgs), T(off), M, I, K, gs_h, a_row_index=ri,
                                                a_dq=a_dq, dq=fq, codes=fc, scales=fs, workspace=wsp)
    assert np.array_equal(to_np(fc)[:Mg], to_np(hc)), "codes"
    assert np.array_equal(to_np(fs)[:Mg], to_np(hs)), "scales"
    assert np.array_equal(to_np(fdq).view(np.uint16)[:Mg], to_np(hdq).view(np.uint16)), "f16 copy"
    assert (to_np(fc)[Mg:] == 0xA5).all() and (to_np(fs)[Mg:] == 0x5A).all(), "rows outside every group"
    assert (to_np(fdq).view(np.uint16)[Mg:] == 0x3C00).all(), "f16 copy of rows outside every group"
    fc2, fs2 = ops.grouped_gemm_silu_requant(*args, tiled, T(wgs), T(off), M, I, K, gs_h, a_row_index=ri,
                                             a_dq=a_dq, workspace=wsp)
    assert np.array_equal(to_np(fc2)[:Mg], to_np(hc)) and np.array_equal(to_np(fs2)[:Mg], to_np(hs))


def test_fused_silu_requant_decode_shaped():
    rng = np.random.default_rng(21)
    counts = rng.integers(0, 12, 40).tolist()
    counts[5] = 0
    _fused_case(counts, 160, 512, 21)


def test_fused_silu_requant_big_tiles():
    # many rows per group: with A's f16 form 128-row tiles and last tiles of
    # 32, 64 and 128 rows; without it the fused GEMM streams in 32-row slots
    counts = [456, 3, 256, 0, 611, 70, 385]
    _fused_case(counts, 256, 512, 22, use_dq=True)
    _fused_case(counts, 256, 512, 23, use_dq=False)


def test_fused_silu_requant_32_to_128_row_groups():
    # 16..64 rows per group on average: without A's f16 form the fused GEMM
    # streams in 32-row slots; with it, each group is one 32-, 64- or
    # 128-row matrix-core tile (or two)
    _fused_case([40, 55, 0, 47, 63, 41, 90], 160, 512, 26)
    _fused_case([40, 55, 0, 47, 63, 41, 90], 160, 512, 27, use_dq=True)


def test_fused_silu_requant_one_group_no_gather():
    _fused_case([300], 96, 768, 24, gather=False, use_dq=True, split=True)
    _fused_case([300], 96, 768, 24, gather=False, use_dq=True, split=False)
    _fused_case([17], 128, 256, 25, gather=False)


def test_fused_silu_requant_split_k():
    # few workgroups for the chip: K is split into ranges and the fused
    # reduction re-quantises the sums.  One group of 128 and 100 rows (the
    # shared expert's form) over short ranges (2 k-steps), 3-step ranges on
    # the streaming kernel, and 128-row matrix-core tiles with A's f16 form
    _fused_case([128], 128, 4096, 30, gather=False, split=True)
    _fused_case([100], 128, 9216, 31, gather=False, split=True)
    _fused_case([128], 256, 2048, 32, gather=False, use_dq=True, split=True)
    _fused_case([100], 64, 2048, 33, gather=False, use_dq=True, split=True)
    # rows past the last group offset (left untouched by the partial GEMM,
    # the reduction and the f16 copy)
    _fused_case([100], 128, 4096, 36, gather=False, split=True, extra_rows=20)
    _fused_case([100], 128, 2048, 37, gather=False, use_dq=True, split=True, extra_rows=20)
    # several groups (an empty one, a ragged last row block) with gathered A
    _fused_case([5, 0, 40, 19], 96, 4096, 34, split=True)
    _fused_case([5, 0, 40, 19], 96, 4096, 35, use_dq=True, split=True)
    _fused_case([5, 0, 40, 19], 96, 4096, 35, use_dq=True, split=False)


def _silu_f32_case(counts, I, K, seed, gather=True, use_dq=False, extra_rows=0):
    """nvfp4_grouped_gemm_silu_f32 against the unfused GEMM (float32 gate_up):
    h must equal silu_mul_requant's float32 SiLU(gate)*up of that gate_up
    (the oracle's silu_mul, bit for bit), the maximum of the partial maxima
    must be max |h|, and quantising h with the resulting global scale must
    give silu_mul_requant's codes, scales and f16 copy.  Rows past the last
    group offset stay untouched."""
    log("gemm+silu f32", counts if len(counts) < 12 else (len(counts), sum(counts)), I, K, gather, use_dq,
        extra_rows)
    rng = np.random.default_rng(seed)
    G, Mg = len(counts), int(sum(counts))
    M = Mg + extra_rows
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a_rows = M + 5 if gather else M
    ac, as_, ags = oracle_nvfp4(_x(a_rows, K, seed, outliers=True))
    row_index = rng.integers(0, a_rows, M).astype(np.int32) if gather else None
    N = 2 * I
    wc = np.empty((G, N, K // 2), np.uint8)
    ws = np.empty((G, N, K // 16), np.uint8)
    wgs = np.empty((G, 2), np.float32)
    for g in range(G):
        wf = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        for sg in range(2):
            c, sc, gg = oracle_nvfp4(wf[sg * I:(sg + 1) * I])
            wc[g, sg * I:(sg + 1) * I], ws[g, sg * I:(sg + 1) * I], wgs[g, sg] = c, sc, gg
    d = dev()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    tiled = ops.prepare_weights(T(wc), T(ws))
    a_dq = T(quant.dequantize_blocks(ac, as_).astype(np.float16)) if use_dq else None
    ri = T(row_index) if gather else None
    args = (T(ac), T(as_), torch.tensor([ags], device=d))
    assert ops.gemm_workspace_size(G, M, N, K, True) == 0      # no split K in this mode
    gu = ops.grouped_gemm(*args, T(wc), T(ws), T(wgs), [0, I, N], T(off), M, a_row_index=ri, w_tiled=tiled,
                          a_dq=a_dq)
    h0 = torch.full((M, I), -7.0, dtype=torch.float32, device=d)
    h, part = ops.grouped_gemm_silu_f32(*args, tiled, T(wgs), T(off), M, I, K, a_row_index=ri, a_dq=a_dq, h=h0)
    g_gu = to_np(gu)[:Mg]
    h_np = to_np(h)
    assert np.array_equal(h_np[:Mg].view(np.uint32), moe.silu_mul(g_gu).view(np.uint32)), "h"
    assert (h_np[Mg:] == -7.0).all(), "rows outside every group"
    assert to_np(part).max() == np.abs(h_np[:Mg]).max(), "partial maxima"
    gs_f = ops.global_scale(part.view(1, -1))
    gs_u = ops.silu_mul_global_scale(gu[:Mg])
    assert to_np(gs_f)[0] == to_np(gs_u)[0], "gs_h"
    hc, hs, hdq = ops.quantize(h[:Mg], gs_f, dq=True)
    rc, rs, rdq = ops.silu_mul_requant(gu[:Mg].contiguous(), gs_u, dq=True)
    assert np.array_equal(to_np(hc), to_np(rc)) and np.array_equal(to_np(hs), to_np(rs)), "codes"
    assert np.array_equal(to_np(hdq).view(np.uint16), to_np(rdq).view(np.uint16)), "f16 copy"


def test_silu_f32_streaming_and_tiles():
    # decode-shaped groups on the weight-streaming kernel; many-row groups on
    # the 128-row tiles with A's f16 form (last tiles of 32, 64 and 128 rows);
    # and the same groups streamed without it
    rng = np.random.default_rng(51)
    counts = rng.integers(0, 12, 40).tolist()
    counts[3] = 0
    _silu_f32_case(counts, 160, 512, 51)
    big = [456, 3, 256, 0, 611, 70, 385]
    _silu_f32_case(big, 256, 512, 52, use_dq=True, extra_rows=9)
    _silu_f32_case(big, 256, 512, 53, extra_rows=9)
    _silu_f32_case([300, 17], 96, 768, 54, gather=False, use_dq=True)


# --- SiLU-requant and combine ---------------------------------------------------

@pytest.mark.parametrize("M,I,dtype", [(1, 16, "f32"), (37, 128, "f32"), (200, 3072, "f32"), (64, 512, "bf16")])
def test_silu_mul_requant_bit_exact(M, I, dtype):
    log("silu", M, I, dtype)
    rng = np.random.default_rng(M + I)
    gu = (rng.standard_normal((M, 2 * I)) * 3).astype(np.float32)
    gu[0, :4] = [0.0, 30.0, -95.0, 89.5]
    if dtype == "bf16":
        gu = formats.bf16_round(gu)
    h = moe.silu_mul(gu)
    gs = quant.global_scale(quant.amax(h) * F32(0.8))
    c_ref, s_ref = quant.quantize(h, gs)
    t = torch.from_numpy(gu).to(dev())
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    c, s = ops.silu_mul_requant(t, torch.tensor([gs], device=dev()))
    assert np.array_equal(to_np(c), c_ref)
    assert np.array_equal(to_np(s), s_ref)
    c2, s2, dq = ops.silu_mul_requant(t, torch.tensor([gs], device=dev()), dq=True)
    assert np.array_equal(to_np(c2), c_ref) and np.array_equal(to_np(s2), s_ref)
    assert np.array_equal(to_np(dq).astype(np.float64), quant.dequantize_blocks(c_ref, s_ref))
    g = to_np(ops.silu_mul_global_scale(t))
    assert g[0] == quant.global_scale(quant.amax(h))


# (the last case has more tokens than the grid's y extent: the
# one-dimensional launch)
@pytest.mark.parametrize("T,k,H,dtype", [(16, 2, 256, "bf16"), (256, 6, 7168, "bf16"), (9, 1, 24, "f32"),
                                         (33, 16, 64, "f32"), (40, 7, 512, "bf16"), (12, 8, 64, "f32"),
                                         (21, 11, 128, "bf16"), (70001, 2, 16, "bf16")])
def test_combine_bit_exact(T, k, H, dtype):
    log("combine", T, k, H, dtype)
    rng = np.random.default_rng(T * k)
    y = formats.bf16_round(rng.standard_normal((T * k, H)).astype(np.float32))
    if dtype == "f32":
        y = rng.standard_normal((T * k, H)).astype(np.float32)
    inv = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    ref = moe.combine(y, inv, w)
    yt = torch.from_numpy(y).to(dev())
    if dtype == "bf16":
        yt = yt.to(torch.bfloat16)
    out = ops.combine(yt, torch.from_numpy(inv).to(dev()), torch.from_numpy(w).to(dev()))
    assert np.array_equal(to_np(out).view(np.uint32), ref.view(np.uint32))
    # with a residual (added after the slots, before the one bf16 rounding)
    r = formats.bf16_round((rng.standard_normal((T, H)) * 2).astype(np.float32))
    ref_r = moe.combine(y, inv, w, residual=r)
    out_r = ops.combine(yt, torch.from_numpy(inv).to(dev()), torch.from_numpy(w).to(dev()),
                        residual=bf16_tensor(r, dev()))
    assert np.array_equal(to_np(out_r).view(np.uint32), ref_r.view(np.uint32))
    assert not np.array_equal(ref_r, ref)


# --- FP8 weight-only projection (wo_a) ------------------------------------------

@pytest.mark.parametrize("N,K", [(128, 128), (200, 384), (300, 1024)])
def test_fp8_quantize_weight_bit_exact(N, K):
    log("fp8 quantize", N, K)
    rng = np.random.default_rng(N + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[:, :128][:min(N, 128)] *= 300.0          # one block with another range
    if N > 128 and K > 128:
        w[128:, 128:256] = 0.0                 # an all-zero block
    w[1, 2] = -0.0
    c_ref, s_ref = fp8.quantize_weight(w)
    c, s = ops.fp8_quantize_weight(torch.from_numpy(w).to(dev()))
    assert np.array_equal(to_np(c), c_ref)
    assert np.array_equal(to_np(s), s_ref)


@pytest.mark.parametrize("M,N,K,out_bf16", [(1, 128, 128, False), (200, 300, 512, False), (64, 128, 1024, True),
                                             (257, 140, 384, True)])
def test_fp8_weight_gemm_within_bound(M, N, K, out_bf16):
    log("fp8 gemm", M, N, K, out_bf16)
    rng = np.random.default_rng(M * 7 + N + K)
    x = formats.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[:, K // 2:] *= 50.0                      # blocks with different scales
    codes, scales = fp8.quantize_weight(w)
    d = dev()
    out = ops.fp8_weight_gemm(bf16_tensor(x, d), torch.from_numpy(codes).to(d), torch.from_numpy(scales).to(d),
                              out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    W = fp8.dequantize_weight(codes, scales)
    exact = x.astype(np.float64) @ W.T
    absum = np.abs(x.astype(np.float64)) @ np.abs(W).T
    check_gemm(to_np(out), exact, absum, 1.0, K, out_bf16, "fp8")
    ref = fp8.weight_gemm(x, codes, scales, "bf16" if out_bf16 else "f32")
    assert np.allclose(to_np(out), ref, rtol=2 ** -7 if out_bf16 else 1e-4, atol=np.abs(ref).max() * 1e-4)
