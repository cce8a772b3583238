"""Parity at the full workload sizes, in the launch configuration the
benchmark times (same entry points, shapes, dtypes and strides), on sampled
rows that the oracle computes one by one.

For every linear of a workload:

* packed weights: every row's codes and scale against the oracle's pack;
* packed activation: sampled rows (first/last rows, rows at 256-row tile
  edges, the rows holding the largest outliers, a seeded random set);
* int32 accumulator (same launch shape, int32 output): bit-exact on the
  sampled rows against the exact integer product of the GPU's own codes;
* the bf16 output launch: on the sampled rows, within one bf16 ulp of the
  rounding of the fp64 epilogue of that accumulator, and within the 2e-3
  relative Frobenius gate of the oracle's own end-to-end Y.

Layers after a harness op (GELU, the gated product) are checked on the GPU's
own intermediate copied to the host, so each layer's parity is isolated.
Routed layers (K % G != 0) are checked against fp64 X W^T + b.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.convrot_oracle as O
import w8a8_int8_linear_amd as cr
import workloads as W
from tests import parity as R
from tests.gpu_util import sample_rows, to_dev, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

EPI_ULP_FRAC = 1e-3   # share of bf16 outputs allowed one ulp off the fp64 epilogue


def say(msg):
    print(msg, flush=True)


def bf16_ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two arrays of bf16 values held in fp32."""
    def ordered(x):
        u = np.ascontiguousarray(x, dtype=np.float32).view(np.int32) >> 16
        mag = (u & 0x7FFF).astype(np.int64)
        return np.where(u < 0, -mag, mag)
    return np.abs(ordered(a) - ordered(b))


def rows_to_check(X: np.ndarray, seed: int) -> np.ndarray:
    M = X.shape[0]
    rows = set(sample_rows(M, seed, n_random=48, edge=24).tolist())
    rows.update(np.argsort(np.max(np.abs(X), axis=1))[-8:].tolist())
    return np.array(sorted(rows), dtype=np.int64)


def check_weight_pack(name, W_np, pw, G, kind, signs):
    q_ref, s_ref, xr = O.pack(W_np, G, kind, signs)
    rep = R.compare_codes(to_np(pw.q), q_ref, O.code_values(xr, s_ref))
    srel = R.scale_rel_diff(to_np(pw.scale), s_ref)
    say(f"  weight {name} {W_np.shape}: {rep}; scale rel {srel:.2e}")
    assert rep.ok(), f"{name}: {rep}"
    assert srel <= R.SCALE_RTOL
    return q_ref, s_ref


def check_act_pack(name, X_rows, pa, S, G, kind, signs):
    q_ref, s_ref, xr = O.pack(X_rows, G, kind, signs)
    rep = R.compare_codes(to_np(pa.q[S]), q_ref, O.code_values(xr, s_ref))
    srel = R.scale_rel_diff(to_np(pa.scale[S]), s_ref)
    say(f"  act {name} rows {len(S)}: {rep}; scale rel {srel:.2e}")
    assert rep.ok(), f"{name}: {rep}"
    assert srel <= R.SCALE_RTOL
    return q_ref, s_ref


def check_linear(name, pa, pw, b_np, S, qx_ref, sx_ref, qw_ref, sw_ref, y_dev):
    """y_dev is the bf16 output of the timed launch shape."""
    St = torch.from_numpy(S).to(pa.q.device)
    A = cr.linear(pa, pw, out_dtype=torch.int32)
    A_s = to_np(A.index_select(0, St)).astype(np.int64)
    del A
    qx_g = to_np(pa.q.index_select(0, St))
    qw_g = to_np(pw.q)
    exact = O.int_gemm(qx_g, qw_g)
    assert np.array_equal(A_s, exact), f"{name}: accumulator differs on sampled rows"
    y_s = to_np(y_dev.index_select(0, St))
    sx_g = to_np(pa.scale.index_select(0, St))
    sw_g = to_np(pw.scale)
    epi = O.bf16_round(O.epilogue64(exact, sx_g, sw_g, b_np).astype(np.float32))
    ulp = bf16_ulp_dist(y_s, epi)
    frac1 = float(np.count_nonzero(ulp)) / ulp.size
    y_ref = O.bf16_round(O.epilogue64(O.int_gemm(qx_ref, qw_ref), sx_ref, sw_ref, b_np).astype(np.float32))
    err = R.rel_fro(y_s, y_ref)
    say(f"  linear {name}: A exact on {len(S)} rows x {qw_g.shape[0]}; epilogue max ulp {int(ulp.max())}, "
        f"{frac1:.2e} off by one; Y rel Frobenius {err:.3e}")
    assert ulp.max() <= 1 and frac1 <= EPI_ULP_FRAC
    assert err <= R.Y_RTOL


def check_routed(name, X_rows, W_np, b_np, y_rows):
    ref = O.bf16_round(O.linear_unquantized64(X_rows, W_np, b_np).astype(np.float32))
    err = R.rel_fro(y_rows, ref)
    say(f"  routed {name}: bf16 linear rel Frobenius {err:.3e}")
    assert err <= R.Y_RTOL


def dev_weight(lin):
    return to_dev(lin.W, torch.bfloat16 if lin.wdtype == "bf16" else torch.float32)


def test_dit_attn_proj_full(cuda):
    """X bf16 [4096, 3072] (8 outlier channels), QKV [9216, 3072] and a second
    [3072, 3072] sharing one packed activation, G=256, bf16 output."""
    wl = W.config2()
    G = wl.G
    X = wl.X
    xd = to_dev(X, torch.bfloat16)
    pa = cr.pack_act(xd, G)
    S = rows_to_check(X, 2)
    qx_ref, sx_ref = check_act_pack("X", X[S], pa, S, G, "regular", None)
    packs, refs = [], []
    for lin in wl.linears:
        pw = cr.pack_weight(dev_weight(lin), G)
        qw_ref, sw_ref = check_weight_pack(lin.name, lin.W, pw, G, "regular", None)
        y = cr.linear(pa, pw, to_dev(lin.b, torch.float32))
        check_linear(lin.name, pa, pw, lin.b, S, qx_ref, sx_ref, qw_ref, sw_ref, y)
        packs.append(pw)
        refs.append((qw_ref, sw_ref))
    # The benchmark runs both linears as one launch over the concatenated
    # packed weight ([12288, 3072], 256 x 256 tiles); each output is a column
    # slice of that launch.
    Wc = np.concatenate([lin.W for lin in wl.linears])
    bc = np.concatenate([lin.b for lin in wl.linears])
    pwc = cr.pack_weight(to_dev(Wc, torch.bfloat16), G)
    assert torch.equal(pwc.q, torch.cat([p.q for p in packs]))
    assert torch.equal(pwc.scale, torch.cat([p.scale for p in packs]))
    del packs
    y = cr.linear(pa, pwc, to_dev(bc, torch.float32))
    check_linear("qkv+second", pa, pwc, bc, S, qx_ref, sx_ref, np.concatenate([r[0] for r in refs]),
                 np.concatenate([r[1] for r in refs]), y)


@pytest.mark.parametrize("r", [32, 128])
def test_dit_attn_proj_lora_full(cuda, r):
    """The LoRA workloads' correction at full size, as the benchmark runs it:
    X [4096, 3072], rank r on the QKV's 9216 columns, added in place into the
    QKV's column view of the one launch over both linears (row pitch 12288).
    T is checked on sampled rows within one bf16 ulp plus the fp32 summation
    bound of the oracle's; Y on
    those rows against bf16(Y0 + scale T B^T) from the GPU's own T, and the
    other linear's columns must stay untouched."""
    wl = W.config2()
    G, X = wl.G, wl.X
    qkv = wl.linears[0]
    K, N = qkv.W.shape[1], qkv.W.shape[0]
    A, B = W.lora_adapter(K, N, r)
    xd = to_dev(X, torch.bfloat16)
    Wc = np.concatenate([lin.W for lin in wl.linears])
    bc = np.concatenate([lin.b for lin in wl.linears])
    y = cr.linear(cr.pack_act(xd, G), cr.pack_weight(to_dev(Wc, torch.bfloat16), G), to_dev(bc, torch.float32))
    y0 = y.clone()
    ws = torch.empty((cr.lora_workspace_bytes(X.shape[0], K, r) + 1) // 2, dtype=torch.bfloat16, device=cuda)
    cr.lora_add(xd, to_dev(A, torch.bfloat16), to_dev(B, torch.bfloat16), 0.5, y[:, :N], workspace=ws)
    S = rows_to_check(X, 5)
    St = torch.from_numpy(S).to(cuda)
    T = to_np(ws[:X.shape[0] * r].view(X.shape[0], r).index_select(0, St))
    T_ref = O.lora_intermediate(X[S], A)
    # T is an fp32 sum of K products in an unspecified order, rounded to bf16:
    # one bf16 ulp plus the worst-case fp32 summation error K 2^-24 sum|x a|
    # (the outlier channels make some sums cancel far below their terms).
    mag = np.abs(X[S].astype(np.float64)) @ np.abs(A.astype(np.float64)).T
    bound = np.abs(T_ref) * 2.0 ** -7 + K * 2.0 ** -24 * mag + 1e-30
    d = np.abs(T.astype(np.float64) - T_ref)
    say(f"  lora r={r}: T max |d| / bound {float(np.max(d / bound)):.3f}, "
        f"{np.count_nonzero(d > np.abs(T_ref) * 2.0 ** -7)} of {d.size} beyond one bf16 ulp")
    assert np.all(d <= bound)
    got = to_np(y.index_select(0, St))
    base = to_np(y0.index_select(0, St))
    want = O.bf16_round((base[:, :N].astype(np.float64) + 0.5 * (T.astype(np.float64) @ B.astype(np.float64).T))
                        .astype(np.float32))
    ulp = bf16_ulp_dist(got[:, :N], want)
    err = R.rel_fro(got[:, :N], O.bf16_round((base[:, :N].astype(np.float64) + O.lora_delta64(X[S], A, B, 0.5))
                                              .astype(np.float32)))
    say(f"  lora r={r}: {len(S)} rows; Y max ulp {int(ulp.max())}, "
        f"{np.count_nonzero(ulp) / ulp.size:.2e} off; rel Frobenius vs oracle delta {err:.3e}")
    assert ulp.max() <= 1 and np.count_nonzero(ulp) / ulp.size <= EPI_ULP_FRAC
    assert err <= 2e-3
    assert torch.equal(y[:, N:], y0[:, N:])


def test_dit_mlp_full(cuda):
    """X bf16 [8192, 3072] with a Student-t tail -> up [12288, 3072] -> GELU
    (torch) -> pack of the [8192, 12288] intermediate -> down [3072, 12288]."""
    wl = W.config3()
    G = wl.G
    up, down = wl.linears
    X = wl.X
    pa = cr.pack_act(to_dev(X, torch.bfloat16), G)
    S = rows_to_check(X, 3)
    qx_ref, sx_ref = check_act_pack("X", X[S], pa, S, G, "regular", None)
    pw_up = cr.pack_weight(dev_weight(up), G)
    qw_ref, sw_ref = check_weight_pack("up", up.W, pw_up, G, "regular", None)
    y_up = cr.linear(pa, pw_up, to_dev(up.b, torch.float32))
    check_linear("up", pa, pw_up, up.b, S, qx_ref, sx_ref, qw_ref, sw_ref, y_up)
    # The same layer with GELU fused into its epilogue (the launch the MLP
    # benchmark times), against GELU of the oracle's Y.
    St0 = torch.from_numpy(S).to(cuda)
    g_fused = to_np(cr.linear_act(pa, pw_up, to_dev(up.b, torch.float32), cr.GELU_ERF).index_select(0, St0))
    ref = O.bf16_round(R.gelu64(O.epilogue64(O.int_gemm(qx_ref, qw_ref), sx_ref, sw_ref, up.b), "gelu_erf")
                       .astype(np.float32))
    err = R.rel_fro(g_fused, ref)
    say(f"  fused up+GELU: Y rel Frobenius {err:.3e}")
    assert err <= R.Y_RTOL
    # Producer fusion of the down layer's pack, as the benchmark's
    # --producer-fusion step runs it: the same Y, group maxima of its
    # rotation, and a pack from those maxima equal to the pack of Y.
    g_full = cr.linear_act(pa, pw_up, to_dev(up.b, torch.float32), cr.GELU_ERF)
    g_f2, pm = cr.linear_act_rowmax(pa, pw_up, G, to_dev(up.b, torch.float32), cr.GELU_ERF)
    assert torch.equal(g_f2, g_full)
    del g_full
    pm_rows = to_np(pm.index_select(0, St0))
    pm_ref = O.group_absmax(O.rotate(to_np(g_f2.index_select(0, St0)), G), G)
    row = np.max(pm_ref, axis=1, keepdims=True)
    assert np.all(np.abs(pm_rows - pm_ref) <= R.ROT_RTOL * row)
    p_f2 = cr.pack_act_rowmax(g_f2, pm, G)
    p_un = cr.pack_act(g_f2, G)
    assert torch.equal(p_f2.q, p_un.q) and torch.equal(p_f2.scale, p_un.scale)
    say(f"  producer fusion: group maxima on {len(S)} rows within {R.ROT_RTOL} of the oracle, pack from them "
        f"equal to the pack of Y")
    del g_f2, pm, p_f2, p_un
    h = torch.nn.functional.gelu(y_up)
    del y_up
    St = torch.from_numpy(S).to(cuda)
    h_rows = to_np(h.index_select(0, St))
    pa2 = cr.pack_act(h, G)
    qh_ref, sh_ref = check_act_pack("gelu(up)", h_rows, pa2, S, G, "regular", None)
    pw_dn = cr.pack_weight(dev_weight(down), G)
    qw_ref, sw_ref = check_weight_pack("down", down.W, pw_dn, G, "regular", None)
    y = cr.linear(pa2, pw_dn, to_dev(down.b, torch.float32))
    check_linear("down", pa2, pw_dn, down.b, S, qh_ref, sh_ref, qw_ref, sw_ref, y)


def test_large_m_full(cuda):
    """X bf16 [32700, 6144] with 0.1% outliers x100 against QKV [18432, 6144]
    (ragged last row tile), plus the routed K=2688 layer on the bf16 linear."""
    wl = W.config4(with_routed=True)
    G = wl.G
    X = wl.X
    lin = wl.linears[0]
    S = rows_to_check(X, 4)
    pa = cr.pack_act(to_dev(X, torch.bfloat16), G)
    qx_ref, sx_ref = check_act_pack("X", X[S], pa, S, G, "regular", None)
    pw = cr.pack_weight(dev_weight(lin), G)
    qw_ref, sw_ref = check_weight_pack(lin.name, lin.W, pw, G, "regular", None)
    y = cr.linear(pa, pw, to_dev(lin.b, torch.float32))
    check_linear(lin.name, pa, pw, lin.b, S, qx_ref, sx_ref, qw_ref, sw_ref, y)
    del y, pa, pw
    r = wl.extra["routed"]
    X2 = wl.extra["X_routed"]
    assert O.routes_to_fallback(X2.shape[1], G)
    y2 = cr.linear_bf16(to_dev(X2, torch.bfloat16), to_dev(r.W, torch.bfloat16), to_dev(r.b, torch.float32))
    check_routed(r.name, X2[S], r.W, r.b, to_np(y2.index_select(0, torch.from_numpy(S).to(cuda))))


DECODE = [(m, g, k) for m in (1, 4, 16) for g, k in ((16, "regular"), (64, "regular"), (128, "randomized"),
                                                      (1024, "regular"))]


@pytest.mark.parametrize("M,G,kind", DECODE)
def test_decode_ffn_full(cuda, M, G, kind):
    """Gated FFN decode: X bf16 [M, 1152] (2 outlier channels x40); gate and up
    [6912, 1152] share one pack; h = gelu_tanh(gate) * up (torch) feeds down
    [1152, 6912].  G=1024 divides neither width: every layer is routed."""
    wl = W.config5(M=M, G=G, kind=kind)
    gate, up, down = wl.linears
    X = wl.X
    S = np.arange(M)
    F = torch.nn.functional
    if O.routes_to_fallback(X.shape[1], G):
        xd = to_dev(X, torch.bfloat16)
        yg, yu = (cr.linear_bf16(xd, to_dev(l.W, torch.bfloat16), to_dev(l.b, torch.float32)) for l in (gate, up))
        check_routed("gate", X, gate.W, gate.b, to_np(yg))
        check_routed("up", X, up.W, up.b, to_np(yu))
        h = F.gelu(yg, approximate="tanh") * yu
        y = cr.linear_bf16(h, to_dev(down.W, torch.bfloat16), to_dev(down.b, torch.float32))
        check_routed("down", to_np(h), down.W, down.b, to_np(y))
        return
    sg = wl.signs
    sd = wl.extra["signs_down"]
    sgd = to_dev(sg, torch.int8) if sg is not None else None
    sdd = to_dev(sd, torch.int8) if sd is not None else None
    pa = cr.pack_act(to_dev(X, torch.bfloat16), G, kind, sgd)
    qx_ref, sx_ref = check_act_pack("X", X, pa, S, G, kind, sg)
    outs = {}
    for lin in (gate, up):
        pw = cr.pack_weight(dev_weight(lin), G, kind, sgd)
        qw_ref, sw_ref = check_weight_pack(lin.name, lin.W, pw, G, kind, sg)
        outs[lin.name] = cr.linear(pa, pw, to_dev(lin.b, torch.float32))
        check_linear(lin.name, pa, pw, lin.b, S, qx_ref, sx_ref, qw_ref, sw_ref, outs[lin.name])
    # The gated launch (both weights in one pass, the product in the
    # epilogue) against gelu_tanh(gate) * up of the oracle.
    pw_g, pw_u = (cr.pack_weight(dev_weight(l), G, kind, sgd) for l in (gate, up))
    fused = to_np(cr.linear_gated(pa, pw_g, pw_u, to_dev(gate.b, torch.float32), to_dev(up.b, torch.float32),
                                  cr.GELU_TANH))
    qg_ref, sg_ref, _ = O.pack(gate.W, G, kind, sg)
    qu_ref, su_ref, _ = O.pack(up.W, G, kind, sg)
    ref = O.bf16_round((R.gelu64(O.epilogue64(O.int_gemm(qx_ref, qg_ref), sx_ref, sg_ref, gate.b), "gelu_tanh")
                        * O.epilogue64(O.int_gemm(qx_ref, qu_ref), sx_ref, su_ref, up.b)).astype(np.float32))
    err = R.rel_fro(fused, ref)
    say(f"  gated gate/up: Y rel Frobenius {err:.3e}")
    assert err <= R.Y_RTOL
    h = F.gelu(outs["gate"], approximate="tanh") * outs["up"]
    pa2 = cr.pack_act(h, G, kind, sdd)
    qh_ref, sh_ref = check_act_pack("h", to_np(h), pa2, S, G, kind, sd)
    pw = cr.pack_weight(dev_weight(down), G, kind, sdd)
    qw_ref, sw_ref = check_weight_pack("down", down.W, pw, G, kind, sd)
    y = cr.linear(pa2, pw, to_dev(down.b, torch.float32))
    check_linear("down", pa2, pw, down.b, S, qh_ref, sh_ref, qw_ref, sw_ref, y)
