"""Pins of the CPU oracle to facts the pages and the mathematics fix.

None of these re-types an oracle formula: each compares the oracle with a
closed form, a textbook or library routine (complex multiplication, torch's
scaled_dot_product_attention, torch's bfloat16 conversion), an invariant, or
brute force on tiny inputs, so that a dropped term, a wrong sign, a wrong index
or a transposed operand in the oracle fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O


# ------------------------------------------------------------------- RoPE


def test_inv_freq_closed_form():
    # theta ** (-2i/D) = 10 ** (-i) when theta = 10 ** (D/2): D = 8 with 1e4,
    # D = 12 with 1e6.
    for d, theta in ((8, 1e4), (12, 1e6)):
        f = O.rope_inv_freq(d, theta)
        assert f.dtype == np.float32
        expect = np.array([10.0 ** (-i) for i in range(d // 2)]).astype(np.float32)
        np.testing.assert_array_equal(f, expect)
    f = O.rope_inv_freq(128, 1e6)
    assert f[0] == 1.0 and f.shape == (64,)
    assert np.all(np.diff(f) < 0)


def test_rope_is_complex_rotation_of_interleaved_pairs(rng):
    # Pair (x[2i], x[2i+1]) rotates like the complex number x[2i] + 1j*x[2i+1]
    # multiplied by exp(1j * angle_i): the interleaved convention, counter-clockwise.
    d, theta = 16, 1e4
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 100, 4095])
    ang = O.rope_angles(pos, O.rope_inv_freq(d, theta)).astype(np.float64)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * ang)
    y = O.apply_rope(x, pos, theta)
    np.testing.assert_allclose(y[:, 0::2], z.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y[:, 1::2], z.imag, rtol=0, atol=1e-13)


def test_rope_worked_rotation():
    # head_dim 2: inv_freq = 1, so position p rotates by p radians:
    # (1, 0) -> (cos p, sin p) and (0, 1) -> (-sin p, cos p).
    p = 3
    y = O.apply_rope(np.array([[1.0, 0.0], [0.0, 1.0]]), np.array([p, p]), 1e4)
    np.testing.assert_allclose(y, [[math.cos(3), math.sin(3)], [-math.sin(3), math.cos(3)]], atol=1e-15)


def test_rope_identity_norm_and_pair_locality(rng):
    d, theta = 64, 1e6
    x = rng.standard_normal((4, d))
    np.testing.assert_array_equal(O.apply_rope(x, np.zeros(4, dtype=int), theta), x)
    pos = np.array([5, 123, 9999, 131087])
    y = O.apply_rope(x, pos, theta)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    for i in (0, 5, 31):
        xp = x.copy()
        xp[:, 2 * i] += 1.0
        changed = np.any(O.apply_rope(xp, pos, theta) != y, axis=0)
        assert set(np.nonzero(changed)[0]) == {2 * i, 2 * i + 1}


def test_rope_angle_is_one_float32_product(rng):
    # The angle is the float32 product rope_tables forms (modeling_flashmap.py:
    # positions.float() * inv_freq): torch's own float32 multiply of the
    # positions and the inverse frequencies gives the same bits, at every
    # position up to the long request's last draft slot (131072 + 16).  The
    # rotation uses exactly that angle: at positions past 2^17 a rotation by the
    # exact float64 angle pos * theta^(-2i/D) differs from it by far more than
    # float64 rounding, so an oracle that formed the angle in float64 fails here.
    d, theta = 128, 1e6
    inv = O.rope_inv_freq(d, theta)
    pos = np.arange(0, 131072 + 17)
    want = torch.arange(0, 131072 + 17).float()[:, None] * torch.from_numpy(inv)[None, :]
    got = O.rope_angles(pos, inv)
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got.view(np.uint32), want.numpy().view(np.uint32))

    far = np.array([131072, 131075, 131087, 131088])
    x = rng.standard_normal((len(far), d))
    ang32 = (torch.from_numpy(far).float()[:, None] * torch.from_numpy(inv)[None, :]).double().numpy()
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * ang32)
    y = O.apply_rope(x, far, theta)
    np.testing.assert_allclose(y[:, 0::2], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[:, 1::2], z.imag, rtol=0, atol=1e-12)
    ang64 = far[:, None].astype(np.float64) * np.array([theta ** (-2.0 * i / d) for i in range(d // 2)])[None, :]
    z64 = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * ang64)
    assert np.max(np.abs(y[:, 0::2] - z64.real)) > 1e-4, "the angle must carry float32 rounding"


def test_rope_relative_position(rng):
    # <R_m q, R_n k> depends only on m - n (up to the float32 rounding of angles).
    d, theta = 64, 1e6
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    for m, n in ((10, 3), (1000, 1500), (40, 40)):
        base = O.apply_rope(q[None], [m], theta)[0] @ O.apply_rope(k[None], [n], theta)[0]
        for shift in (1, 17, 1000):
            got = O.apply_rope(q[None], [m + shift], theta)[0] @ O.apply_rope(k[None], [n + shift], theta)[0]
            assert abs(got - base) <= 2e-3 * np.linalg.norm(q) * np.linalg.norm(k)


# ---------------------------------------------------------------- RMSNorm


def test_rms_norm_closed_forms(rng):
    eps = 1e-6
    x = rng.standard_normal((6, 128)) * rng.uniform(0.01, 10, (6, 1))
    ms = np.mean(x * x, axis=1)
    y = O.rms_norm(x, np.ones(128), eps)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)
    # (3, 4): mean square 12.5
    np.testing.assert_allclose(O.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0), [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    # scale invariance (eps = 0) and channel-wise weight
    np.testing.assert_allclose(O.rms_norm(7.5 * x, np.ones(128), 0.0), O.rms_norm(x, np.ones(128), 0.0), rtol=1e-12)
    w = rng.uniform(0.5, 1.5, 128)
    np.testing.assert_allclose(O.rms_norm(x, w, eps), O.rms_norm(x, np.ones(128), eps) * w, rtol=1e-14)


# ------------------------------------------------------------ bf16 storage


def test_round_to_bfloat16_matches_torch(rng):
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-8, 8, 20000))).astype(np.float32)
    # exact ties: bf16 grid midpoints (low 16 bits = 0x8000) with both parities
    bits = rng.integers(0x3000, 0x4800, 2000).astype(np.uint32) << 16 | 0x8000
    ties = bits.view(np.float32)
    for v in (x32, ties, -ties):
        ours = O.round_to_bfloat16(v.astype(np.float64))
        ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
        np.testing.assert_array_equal(ours, ref)
    assert O.round_to_bfloat16(np.array([0.0]))[0] == 0.0


# -------------------------------------------------------------- attention


def test_round_to_e4m3_matches_torch_and_saturates(rng):
    # torch's float8_e4m3fn conversion is nearest-even on the same grid; it maps
    # magnitudes past 464 to NaN, where the pool saturates to 448 instead.
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0)])
    x = np.concatenate([x[np.abs(x) <= 464.0], [0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6,
                                                  448.0, 464.0, -464.0, 1.0625, 1.1875, -0.99]])
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_e4m3(x), ref)
    np.testing.assert_array_equal(O.round_to_e4m3(np.array([470.0, -600.0, 1e9])), [448.0, -448.0, 448.0])
    # all 256 codes: 253 distinct finite values (0x7F / 0xFF are NaN, +0 and -0 coincide), each a
    # fixed point; a midpoint between neighbours goes to the code whose mantissa is even
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    grid = np.unique(codes[np.isfinite(codes)])
    assert len(grid) == 253 and grid[0] == -448.0 and grid[-1] == 448.0
    np.testing.assert_array_equal(O.round_to_e4m3(grid), grid)
    pos = grid[grid >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    even = np.where(np.arange(len(mids)) % 2 == 0, pos[:-1], pos[1:])  # code index parity = mantissa parity
    np.testing.assert_array_equal(O.round_to_e4m3(mids), even)


def test_quantize_query_e4m3_scale_and_error(rng):
    q = rng.standard_normal((16, 128)) * 3.0
    q8, s = O.quantize_query_e4m3(q)
    assert np.max(np.abs(q8)) == 448.0                  # the largest magnitude lands on 448 exactly
    assert s == np.max(np.abs(q)) / 448.0
    big = np.abs(q) >= 2.0 ** -6 * s                    # normal range: relative error <= 2^-4
    assert np.all(np.abs(q8 * s - q)[big] <= 2.0 ** -4 * np.abs(q)[big] + 1e-15)
    np.testing.assert_array_equal(O.quantize_query_e4m3(np.zeros((4, 8)))[0], 0.0)


def test_attention_matches_sdpa(rng):
    for n, t, d in ((16, 1, 64), (16, 37, 128), (3, 500, 64)):
        q, k, v = rng.standard_normal((n, d)), rng.standard_normal((t, d)), rng.standard_normal((t, d))
        scale = d ** -0.5
        ref = F.scaled_dot_product_attention(*(torch.from_numpy(a)[None, None] for a in (q, k, v)), scale=scale)[0, 0]
        np.testing.assert_allclose(O.attention(q, k, v, scale), ref.numpy(), rtol=1e-12, atol=1e-13)


def test_attention_special_cases(rng):
    d = 64
    q = rng.standard_normal((16, d))
    v = rng.standard_normal((9, d))
    k = rng.standard_normal((9, d))
    np.testing.assert_array_equal(O.attention(q, k[:1], v[:1], 0.125), np.repeat(v[:1], 16, 0))
    same = np.repeat(k[:1], 9, 0)
    np.testing.assert_allclose(O.attention(q, same, v, 0.125), np.repeat(v.mean(0, keepdims=True), 16, 0), atol=1e-14)
    np.testing.assert_allclose(O.attention(q, k, v, 0.0), np.repeat(v.mean(0, keepdims=True), 16, 0), atol=1e-14)
    peaky = k.copy()
    peaky[4] = q[0] * 100.0
    out = O.attention(q[:1], peaky, v, 1.0)
    np.testing.assert_allclose(out[0], v[4], atol=1e-12)
    assert np.all(O.attention(q, k[:0], v[:0], 0.125) == 0)


# ---------------------------------------------------------- paged context


def _place_dense(dense_k, dense_v, ctx, page_table, ps, n_pages, H, D):
    """Test-side placement: logical position t of request b -> page
    page_table[b][t // ps], slot t % ps (written independently of the oracle)."""
    pk = np.zeros((n_pages, ps, H, D))
    pv = np.zeros((n_pages, ps, H, D))
    for b, n in enumerate(ctx):
        for t in range(n):
            pk[page_table[b][t // ps], t % ps] = dense_k[b][t]
            pv[page_table[b][t // ps], t % ps] = dense_v[b][t]
    return pk, pv


def _paged_case(rng, ctx, nq, H=2, D=64, ps=16):
    bs = len(ctx)
    pages_per = [-(-c // ps) for c in ctx]
    n_pages = sum(pages_per) + 3
    perm = rng.permutation(n_pages)
    width = max(max(pages_per), 1)
    pt = np.zeros((bs, width), dtype=np.int64)
    at = 0
    for b, n in enumerate(pages_per):
        pt[b, :n] = perm[at:at + n]
        at += n
    dense_k = [rng.standard_normal((c, H, D)) for c in ctx]
    dense_v = [rng.standard_normal((c, H, D)) for c in ctx]
    pk, pv = _place_dense(dense_k, dense_v, ctx, pt, ps, n_pages, H, D)
    cu = np.concatenate([[0], np.cumsum(nq)])
    q = rng.standard_normal((cu[-1], H, D))
    w = 1.0 + 0.1 * rng.standard_normal(D)
    return dict(ctx=ctx, pt=pt, pk=pk, pv=pv, dense_k=dense_k, dense_v=dense_v, cu=cu, q=q, w=w, ps=ps, H=H, D=D)


def test_paged_cross_attention_equals_dense(rng):
    # The draft step (modeling_flashmap.py ``draft``): anchor = cache length,
    # context = positions 0..anchor, query slot k at anchor + 1 + k.
    c = _paged_case(rng, ctx=[64, 1, 37, 0, 200], nq=[16, 16, 3, 16, 5])
    theta, eps, scale = 1e6, 1e-6, c["D"] ** -0.5
    out = O.paged_cross_attention(c["q"], c["w"], c["pk"], c["pv"], c["pt"], c["ctx"], c["cu"],
                                  c["ps"], scale, theta, eps)
    for b, n in enumerate(c["ctx"]):
        r0, r1 = c["cu"][b], c["cu"][b + 1]
        anchor = n - 1
        pos = anchor + 1 + np.arange(r1 - r0)
        for h in range(c["H"]):
            qh = O.apply_rope(O.rms_norm(c["q"][r0:r1, h], c["w"], eps), pos, theta)
            if n == 0:
                np.testing.assert_array_equal(out[r0:r1, h], 0.0)
                continue
            kt = torch.from_numpy(c["dense_k"][b][:, h])
            vt = torch.from_numpy(c["dense_v"][b][:, h])
            ref = F.scaled_dot_product_attention(torch.from_numpy(qh)[None], kt[None], vt[None], scale=scale)[0]
            np.testing.assert_allclose(out[r0:r1, h], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_paged_cross_attention_e4m3_query_against_torch_fp8(rng):
    # fp8 pool (sglang model ``_paged_cross_attention_fp8``): e4m3 keys/values,
    # query scaled by amax/448 over the request's rows and the head's channels,
    # cast to e4m3, then descaled in the scores.  The cast here is torch's.
    c = _paged_case(rng, ctx=[40, 1, 0, 130], nq=[32, 16, 16, 7])
    pk, pv = O.round_to_e4m3(c["pk"] * 4.0), O.round_to_e4m3(c["pv"] * 4.0)
    theta, eps, scale = 1e6, 1e-6, c["D"] ** -0.5
    args = (c["pt"], c["ctx"], c["cu"], c["ps"], scale, theta, eps)
    out = O.paged_cross_attention(c["q"], c["w"], pk, pv, *args, kv_e4m3=True)
    plain = O.paged_cross_attention(c["q"], c["w"], pk, pv, *args)
    per_row_gap = 0.0
    for b, n in enumerate(c["ctx"]):
        r0, r1 = c["cu"][b], c["cu"][b + 1]
        pos = n + np.arange(r1 - r0) % 16
        for h in range(c["H"]):
            if n == 0:
                np.testing.assert_array_equal(out[r0:r1, h], 0.0)
                continue
            qh = torch.from_numpy(O.apply_rope(O.rms_norm(c["q"][r0:r1, h], c["w"], eps), pos, theta))
            qs = qh.abs().max() / 448.0
            q8 = (qh / qs).to(torch.float8_e4m3fn).to(torch.float64) * qs
            dk = torch.from_numpy(O.round_to_e4m3(c["dense_k"][b][:, h] * 4.0))
            dv = torch.from_numpy(O.round_to_e4m3(c["dense_v"][b][:, h] * 4.0))
            ref = F.scaled_dot_product_attention(q8[None], dk[None], dv[None], scale=scale)[0]
            np.testing.assert_allclose(out[r0:r1, h], ref.numpy(), rtol=1e-11, atol=1e-12)
            # quantizing each row on its own scale gives other values
            q8r = (qh / (qh.abs().amax(1, keepdim=True) / 448.0)).to(torch.float8_e4m3fn).to(torch.float64) \
                * (qh.abs().amax(1, keepdim=True) / 448.0)
            alt = F.scaled_dot_product_attention(q8r[None], dk[None], dv[None], scale=scale)[0]
            per_row_gap = max(per_row_gap, float(np.abs(alt.numpy() - out[r0:r1, h]).max()))
            # within the quantization bound of the unquantized query: |dq| <= 2^-4 |q| + 2^-10 qs
            # per channel, |d score| <= M, and every output moves by at most (e^{2M} - 1) max|v|
            dq = (2.0 ** -4) * qh.abs() + (2.0 ** -10) * qs
            M = scale * float((dq @ dk.abs().T).max())
            bound = (np.exp(2 * M) - 1) * float(dv.abs().max())
            assert np.abs(out[r0:r1, h] - plain[r0:r1, h]).max() <= bound
    assert per_row_gap > 1e-6
    assert np.nanmax(np.abs(out - plain)) > 1e-6


def test_fp8_static_and_tensor_scales(rng):
    # vLLM's fp8 cache: static per-tensor q scale, per-tensor k/v descales.
    c = _paged_case(rng, ctx=[70], nq=[16], H=1)
    pk, pv = O.round_to_e4m3(c["pk"] * 4.0), O.round_to_e4m3(c["pv"] * 4.0)
    theta, eps, scale = 1e6, 1e-6, c["D"] ** -0.5
    args = (c["pt"], c["ctx"], c["cu"], c["ps"], scale, theta, eps)
    dyn = O.paged_cross_attention(c["q"], c["w"], pk, pv, *args, kv_e4m3=True)
    # one (request, head): the static scale equal to its amax / 448 is the dynamic case
    qh = O.apply_rope(O.rms_norm(c["q"][:, 0], c["w"], eps), 70 + np.arange(16), theta)
    stat = O.paged_cross_attention(c["q"], c["w"], pk, pv, *args, kv_e4m3=True, q_scale=np.abs(qh).max() / 448.0)
    np.testing.assert_array_equal(stat, dyn)
    # the output is linear in the value descale
    v2 = O.paged_cross_attention(c["q"], c["w"], pk, pv, *args, kv_e4m3=True, v_scale=2.5)
    np.testing.assert_allclose(v2, 2.5 * dyn, rtol=1e-12, atol=1e-14)
    # a key descale multiplies the logits: k_scale = s with softmax scale / s is the same attention
    k2 = O.paged_cross_attention(c["q"], c["w"], pk, pv, c["pt"], c["ctx"], c["cu"], c["ps"], scale / 2.0, theta,
                                 eps, kv_e4m3=True, k_scale=2.0)
    np.testing.assert_allclose(k2, dyn, rtol=1e-12, atol=1e-13)
    # a static scale quantizes q^ / s with torch's cast, no per-row or per-request amax
    s_fix = 0.01
    q8 = (torch.from_numpy(qh) / s_fix).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64) * s_fix
    t8 = lambda x: torch.from_numpy(x * 4.0).to(torch.float8_e4m3fn).to(torch.float64)  # noqa: E731
    dk = t8(c["dense_k"][0][:, 0]) * 1.5      # logical context, cast by torch
    dv = t8(c["dense_v"][0][:, 0]) * 0.5
    ref = F.scaled_dot_product_attention(q8[None], dk[None], dv[None], scale=scale)[0]
    got = O.paged_cross_attention(c["q"], c["w"], pk, pv, *args, kv_e4m3=True, q_scale=s_fix, k_scale=1.5,
                                  v_scale=0.5)
    np.testing.assert_allclose(got[:, 0], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_scatter_divides_by_the_layer_scales(rng):
    keys = rng.standard_normal((3, 2, 1, 8)) * 3
    values = rng.standard_normal((3, 2, 1, 8)) * 3
    pk = [np.zeros((2, 4, 1, 8)) for _ in range(2)]
    pv = [np.zeros((2, 4, 1, 8)) for _ in range(2)]
    O.scatter_into_pool(pk, pv, np.array([5, -1, 0]), keys, values, 4, "e4m3", kv_scales=[[1.0, 1.0], [0.5, 4.0]])
    t = lambda x: torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()  # noqa: E731
    np.testing.assert_array_equal(pk[0][1, 1], t(keys[0, 0]))
    np.testing.assert_array_equal(pk[1][1, 1], t(keys[0, 1] / 0.5))
    np.testing.assert_array_equal(pv[1][0, 0], t(values[2, 1] / 4.0))
    assert not pk[0][0, 1].any() and not pv[1][0, 2].any()


def test_paged_cross_attention_page_permutation_invariant(rng):
    c = _paged_case(rng, ctx=[100, 33, 16], nq=[16, 16, 16])
    args = (c["cu"], c["ps"], 0.125, 1e6, 1e-6)
    base = O.paged_cross_attention(c["q"], c["w"], c["pk"], c["pv"], c["pt"], c["ctx"], *args)
    relabel = rng.permutation(c["pk"].shape[0])          # new id of each old page
    pk2 = np.empty_like(c["pk"])
    pv2 = np.empty_like(c["pv"])
    pk2[relabel] = c["pk"]
    pv2[relabel] = c["pv"]
    pt2 = relabel[c["pt"]]
    moved = O.paged_cross_attention(c["q"], c["w"], pk2, pv2, pt2, c["ctx"], *args)
    np.testing.assert_array_equal(moved, base)


def test_candidate_blocks_read_one_context(rng):
    # Tree drafting (sglang/model.py ``forward``): a request's n candidate
    # blocks sit side by side on the query axis, candidate-major, and share its
    # context; candidate c's slot j sits at the same position as slot j of a
    # single block.  So a request with 3 blocks of 16 rows (the last ragged)
    # must equal three one-block requests over the same pages, row for row,
    # and against brute-force dense attention; identical candidates give
    # identical rows.
    ctx = [70, 16, 0]
    c = _paged_case(rng, ctx=ctx, nq=[40, 32, 20])
    theta, eps, scale = 1e6, 1e-6, c["D"] ** -0.5
    joint = O.paged_cross_attention(c["q"], c["w"], c["pk"], c["pv"], c["pt"], c["ctx"], c["cu"], c["ps"], scale,
                                    theta, eps)
    # the same rows split into one-block requests that repeat their request's pages
    split_ctx, split_pt, split_cu = [], [], [0]
    for b, n in enumerate(ctx):
        rows = c["cu"][b + 1] - c["cu"][b]
        for c0 in range(0, rows, 16):
            split_ctx.append(n)
            split_pt.append(c["pt"][b])
            split_cu.append(split_cu[-1] + min(16, rows - c0))
    split = O.paged_cross_attention(c["q"], c["w"], c["pk"], c["pv"], np.array(split_pt), split_ctx,
                                    np.array(split_cu), c["ps"], scale, theta, eps)
    # (equal up to the matrix products' rounding order over different row counts)
    np.testing.assert_allclose(joint, split, rtol=1e-12, atol=1e-14)
    for b, n in enumerate(ctx):
        r0, r1 = c["cu"][b], c["cu"][b + 1]
        pos = n + np.arange(r1 - r0) % 16
        for h in range(c["H"]):
            qh = O.apply_rope(O.rms_norm(c["q"][r0:r1, h], c["w"], eps), pos, theta)
            if n == 0:
                np.testing.assert_array_equal(joint[r0:r1, h], 0.0)
                continue
            kt = torch.from_numpy(c["dense_k"][b][:, h])
            vt = torch.from_numpy(c["dense_v"][b][:, h])
            ref = F.scaled_dot_product_attention(torch.from_numpy(qh)[None], kt[None], vt[None], scale=scale)[0]
            np.testing.assert_allclose(joint[r0:r1, h], ref.numpy(), rtol=1e-11, atol=1e-12)
    q2 = c["q"].copy()
    q2[16:32] = q2[0:16]                 # request 0: candidate 1 repeats candidate 0
    twin = O.paged_cross_attention(q2, c["w"], c["pk"], c["pv"], c["pt"], c["ctx"], c["cu"], c["ps"], scale,
                                   theta, eps)
    np.testing.assert_allclose(twin[16:32], twin[0:16], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------- self-attention


def test_block_self_attention_matches_sdpa_and_k1(rng):
    nb, K, H, D = 3, 16, 2, 64
    qkv = rng.standard_normal((nb, K, 3, H, D))
    wq, wk = 1 + 0.1 * rng.standard_normal(D), 1 + 0.1 * rng.standard_normal(D)
    ctx = np.array([5, 1000, 0])
    theta, eps, scale = 1e6, 1e-6, D ** -0.5
    out = O.block_self_attention(qkv, wq, wk, ctx, scale, theta, eps)
    for b in range(nb):
        pos = ctx[b] + np.arange(K)
        for h in range(H):
            q = O.apply_rope(O.rms_norm(qkv[b, :, 0, h], wq, eps), pos, theta)
            k = O.apply_rope(O.rms_norm(qkv[b, :, 1, h], wk, eps), pos, theta)
            ref = F.scaled_dot_product_attention(*(torch.from_numpy(a)[None] for a in (q, k, qkv[b, :, 2, h])), scale=scale)[0]
            np.testing.assert_allclose(out[b, :, h], ref.numpy(), rtol=1e-11, atol=1e-12)
    one = O.block_self_attention(qkv[:, :1], wq, wk, ctx, scale, theta, eps)
    np.testing.assert_allclose(one[:, 0], qkv[:, 0, 2], rtol=0, atol=1e-15)


def test_block_self_attention_shift_invariant(rng):
    # q and k of a block rotate at the same positions, so shifting the block's
    # base position changes no score (RoPE's relative property).
    qkv = rng.standard_normal((1, 16, 3, 2, 64))
    w = np.ones(64)
    a = O.block_self_attention(qkv, w, w, [40], 0.125, 1e6, 1e-6)
    b = O.block_self_attention(qkv, w, w, [1040], 0.125, 1e6, 1e-6)
    np.testing.assert_allclose(a, b, atol=2e-3)


# ------------------------------------------------------------------ write


def test_projection_concatenates_layers(rng):
    # load_weights: the all-layer weight is cat over layers of [k_proj_l; v_proj_l].
    L, H, D, din = 3, 2, 8, 24
    wk = [rng.standard_normal((H * D, din)) for _ in range(L)]
    wv = [rng.standard_normal((H * D, din)) for _ in range(L)]
    w_kv = np.concatenate([m for l in range(L) for m in (wk[l], wv[l])])
    x = rng.standard_normal((5, din))
    y = O.project_context_rows(x, w_kv, L, H, D)
    for l in range(L):
        np.testing.assert_allclose(y[:, l, 0].reshape(5, -1), x @ wk[l].T, rtol=1e-13)
        np.testing.assert_allclose(y[:, l, 1].reshape(5, -1), x @ wv[l].T, rtol=1e-13)
    # brute-force dot products on a tiny case
    for r in range(5):
        for col in (0, 7, H * D * 2 * L - 1):
            l, rest = divmod(col, 2 * H * D)
            kv, rest = divmod(rest, H * D)
            h, d = divmod(rest, D)
            assert abs(y[r, l, kv, h, d] - sum(x[r, i] * w_kv[col, i] for i in range(din))) < 1e-12


def _write_case(rng, L=2, H=2, D=16, ps=4):
    bs, window = 3, 5
    commit = np.array([2, 5, 1])
    anchor = np.array([9, 17, 4])                 # anchor positions p_b
    # window column j of request b sits at p_b - c_b + j; the anchor row at p_b
    row_req = np.concatenate([np.repeat(np.arange(bs), window), np.arange(bs)])
    row_pos = np.concatenate([anchor[b] - commit[b] + np.arange(window) for b in range(bs)] + [anchor])
    width = -(-(anchor.max() + window + 1) // ps)
    n_pages = bs * width
    pt = rng.permutation(n_pages).reshape(bs, width)
    din = 2 * H * D
    x = rng.standard_normal((len(row_pos), din))
    return dict(L=L, H=H, D=D, ps=ps, bs=bs, window=window, commit=commit, anchor=anchor,
                row_req=row_req, row_pos=row_pos, pt=pt, n_pages=n_pages, x=x)


def test_context_input_rows_against_torch_and_selector(rng):
    # fc then hidden_norm (the sglang model's _write_context)
    n, aux, dt, dim = 7, 3, 16, 12
    x = rng.standard_normal((n, aux * dt))
    w = rng.standard_normal((dim, aux * dt)) * 0.3
    g = 1.0 + 0.1 * rng.standard_normal(dim)
    got = O.context_input_rows(x, w, g, 1e-6)
    ref = F.rms_norm(F.linear(torch.from_numpy(x), torch.from_numpy(w)), (dim,), torch.from_numpy(g), 1e-6)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)
    # fc selecting the second aux block: the norm of that block alone
    sel = np.zeros((dt, aux * dt))
    sel[:, dt:2 * dt] = np.eye(dt)
    np.testing.assert_allclose(O.context_input_rows(x, sel, np.ones(dt), 0.0),
                               x[:, dt:2 * dt] / np.sqrt(np.mean(x[:, dt:2 * dt] ** 2, axis=1, keepdims=True)),
                               rtol=1e-13, atol=0)


def test_anchor_input_rows_against_torch_and_closed_forms(rng):
    vocab, dt, dim = 50, 16, 12
    emb = rng.standard_normal((vocab, dt))
    w = rng.standard_normal((dim, dt)) * 0.3
    b = rng.standard_normal(dim)
    g = 1.0 + 0.1 * rng.standard_normal(dim)
    ids = np.array([3, 49, 0, 3])
    got = O.anchor_input_rows(ids, emb, w, b, g, 1e-6)
    e = F.embedding(torch.from_numpy(ids), torch.from_numpy(emb))
    ref = F.rms_norm(F.linear(e, torch.from_numpy(w), torch.from_numpy(b)), (dim,), torch.from_numpy(g), 1e-6)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(got[0], got[3])                  # repeated token, identical row
    # a zero projection leaves rms_norm(bias) in every row
    z = O.anchor_input_rows(ids, emb, np.zeros((dim, dt)), b, np.ones(dim), 0.0)
    np.testing.assert_allclose(z, np.tile(b / np.sqrt(np.mean(b ** 2)), (4, 1)), rtol=1e-13, atol=0)


def test_write_identity_weight_passthrough_and_commit_rule(rng):
    c = _write_case(rng, L=1)
    H, D = c["H"], c["D"]
    w_kv = np.eye(2 * H * D)                     # x = concat(k, v) passes through
    knw = 1 + 0.1 * rng.standard_normal((1, D))
    slots, keys, values = O.write_context_kv(c["x"], w_kv, knw, c["row_req"], c["row_pos"], c["pt"], c["ps"],
                                             1, H, D, 1e-6, 1e6, commit_lens=c["commit"], window=c["window"])
    for r in range(len(c["row_pos"])):
        if r < c["bs"] * c["window"]:
            b, j = divmod(r, c["window"])
            live = j < c["commit"][b]
        else:
            b, live = r - c["bs"] * c["window"], True
        if not live:
            assert slots[r] == -1
            continue
        pos = c["row_pos"][r]
        # brute-force slot: enumerate the request's pages in logical order
        logical = [(page, off) for page in c["pt"][b] for off in range(c["ps"])]
        page, off = logical[pos]
        assert slots[r] == page * c["ps"] + off
        k = c["x"][r, : H * D].reshape(H, D)
        v = c["x"][r, H * D:].reshape(H, D)
        np.testing.assert_array_equal(values[r, 0], v)
        np.testing.assert_allclose(keys[r, 0], O.apply_rope(O.rms_norm(k, knw[0], 1e-6), np.full(H, pos), 1e6), rtol=1e-14)
    # anchors always live, uncommitted columns never
    assert np.all(slots[c["bs"] * c["window"]:] >= 0)
    assert (slots >= 0).sum() == c["commit"].sum() + c["bs"]


def test_scatter_touches_only_written_slots(rng):
    c = _write_case(rng)
    L, H, D, ps = c["L"], c["H"], c["D"], c["ps"]
    w_kv = rng.standard_normal((L * 2 * H * D, c["x"].shape[1])) * 0.2
    slots, keys, values = O.write_context_kv(c["x"], w_kv, np.ones((L, D)), c["row_req"], c["row_pos"], c["pt"], ps,
                                             L, H, D, 1e-6, 1e6, commit_lens=c["commit"], window=c["window"])
    sentinel = -12345.0
    pk = [np.full((c["n_pages"], ps, H, D), sentinel) for _ in range(L)]
    pv = [np.full((c["n_pages"], ps, H, D), sentinel) for _ in range(L)]
    O.scatter_into_pool(pk, pv, slots, keys, values, ps, "bf16")
    for l in range(L):
        changed = np.nonzero(np.any(pk[l] != sentinel, axis=(2, 3)).reshape(-1))[0]
        assert set(changed) == set(int(s) for s in slots if s >= 0)
        for r in np.nonzero(slots >= 0)[0]:
            page, off = divmod(int(slots[r]), ps)
            np.testing.assert_array_equal(pk[l][page, off], O.round_to_bfloat16(keys[r, l]))
            np.testing.assert_array_equal(pv[l][page, off], O.round_to_bfloat16(values[r, l]))
    with pytest.raises(ValueError):
        dup = slots.copy()
        dup[np.nonzero(slots >= 0)[0][:2]] = slots[slots >= 0][0]
        O.scatter_into_pool(pk, pv, dup, keys, values, ps, "bf16")


def test_written_context_is_read_back_by_paged_attention(rng):
    # Write a whole context 0..p (committed rows + the anchor at p), then the
    # paged attention over ctx_len = p + 1 equals dense attention over the rows
    # just written: ties the write's slot rule to the read's.
    L, H, D, ps = 1, 2, 16, 4
    p = 13
    pt = rng.permutation(6)[None, :]
    x = rng.standard_normal((p + 1, 2 * H * D))
    w_kv = rng.standard_normal((2 * H * D, 2 * H * D)) * 0.3
    slots, keys, values = O.write_context_kv(x, w_kv, np.ones((1, D)), np.zeros(p + 1, int), np.arange(p + 1),
                                             pt, ps, L, H, D, 1e-6, 1e6)
    pk = [np.zeros((6, ps, H, D))]
    pv = [np.zeros((6, ps, H, D))]
    O.scatter_into_pool(pk, pv, slots, keys, values, ps, "f32")
    q = rng.standard_normal((16, H, D))
    out = O.paged_cross_attention(q, np.ones(D), pk[0], pv[0], pt, [p + 1], [0, 16], ps, 0.25, 1e6, 1e-6)
    for h in range(H):
        qh = O.apply_rope(O.rms_norm(q[:, h], np.ones(D), 1e-6), p + 1 + np.arange(16), 1e6)
        kk = O.round_to_storage(keys[:, 0, h], "f32")
        vv = O.round_to_storage(values[:, 0, h], "f32")
        np.testing.assert_allclose(out[:, h], O.attention(qh, kk, vv, 0.25), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------- the DiT layer


def test_layer_norm_and_gelu_against_torch(rng):
    x = rng.standard_normal((5, 64)) * 3 + 1.5
    np.testing.assert_allclose(O.layer_norm(x, 1e-6), F.layer_norm(torch.from_numpy(x), (64,), eps=1e-6).numpy(),
                               rtol=1e-12, atol=1e-13)
    y = O.layer_norm(x, 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-12)
    g = rng.standard_normal(1000) * 4
    np.testing.assert_allclose(O.gelu(g), F.gelu(torch.from_numpy(g)).numpy(), rtol=1e-12, atol=1e-15)
    # closed forms: Phi(0) = 1/2, Phi(1) = (1 + erf(1/sqrt 2)) / 2 = 0.841344746068543
    np.testing.assert_allclose(O.gelu(np.array([0.0, 1.0, -1.0])), [0.0, 0.841344746068543, -0.158655253931457],
                               rtol=1e-14, atol=1e-15)


def _dit_case(rng, M=6, dim=16, inter=40):
    w = {"qkv": rng.standard_normal((3 * dim, dim)) * 0.3, "o_self": rng.standard_normal((dim, dim)) * 0.3,
         "q": rng.standard_normal((dim, dim)) * 0.3, "o_cross": rng.standard_normal((dim, dim)) * 0.3,
         "fc1": rng.standard_normal((inter, dim)) * 0.3, "b1": rng.standard_normal(inter) * 0.1,
         "fc2": rng.standard_normal((dim, inter)) * 0.3, "b2": rng.standard_normal(dim) * 0.1}
    mod = {k: (1.0 + 0.2 * rng.standard_normal(dim)) if k.endswith("scale") else 0.3 * rng.standard_normal(dim)
           for k in ("s_scale", "s_shift", "s_gate", "c_scale", "c_shift", "c_gate", "m_scale", "m_shift", "m_gate")}
    h = rng.standard_normal((M, dim)) * 2
    return h, mod, w


def test_dit_layer_against_a_torch_composition(rng):
    h, mod, w = _dit_case(rng)
    ctx = rng.standard_normal((9, 16))
    sa = lambda qkv: np.tanh(qkv[:, :16] + qkv[:, 32:])       # stand-ins: any fixed maps  # noqa: E731
    ca = lambda q: q @ ctx.T @ ctx / 9.0                        # noqa: E731
    got = O.dit_layer(h, mod, w, sa, ca, 1e-6)
    t = {k: torch.from_numpy(np.asarray(v)) for k, v in {**w, **mod}.items()}
    x = torch.from_numpy(h)
    ln = lambda v, a, b: F.layer_norm(v, (16,), eps=1e-6) * t[a] + t[b]  # noqa: E731
    x = x + t["s_gate"] * F.linear(torch.from_numpy(sa(F.linear(ln(x, "s_scale", "s_shift"), t["qkv"]).numpy())),
                                   t["o_self"])
    x = x + t["c_gate"] * F.linear(torch.from_numpy(ca(F.linear(ln(x, "c_scale", "c_shift"), t["q"]).numpy())),
                                   t["o_cross"])
    x = x + t["m_gate"] * F.linear(F.gelu(F.linear(ln(x, "m_scale", "m_shift"), t["fc1"], t["b1"])), t["fc2"], t["b2"])
    np.testing.assert_allclose(got, x.numpy(), rtol=1e-11, atol=1e-12)


def test_dit_layer_gates_and_zero_branches(rng):
    h, mod, w = _dit_case(rng)
    sa = lambda qkv: qkv[:, :16] * 2.0                          # noqa: E731
    ca = lambda q: q - 1.0                                      # noqa: E731
    closed = dict(mod, s_gate=np.zeros(16), c_gate=np.zeros(16), m_gate=np.zeros(16))
    np.testing.assert_array_equal(O.dit_layer(h, closed, w, sa, ca, 1e-6), h)   # every gate shut: identity
    # only the MLP open, with fc2 = 0: the residual gains m_gate * b2 exactly
    only = dict(closed, m_gate=mod["m_gate"])
    got = O.dit_layer(h, only, dict(w, fc2=np.zeros_like(w["fc2"])), sa, ca, 1e-6)
    np.testing.assert_allclose(got, h + mod["m_gate"] * w["b2"], rtol=1e-15, atol=1e-15)
