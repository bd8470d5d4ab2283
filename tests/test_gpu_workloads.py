"""GPU parity at the workloads' full sizes, through the batched calls in the
launch configuration bench.py times (one batched projection sampling per
update; per microbatch one rgc_project_batch and one rgc_accumulate_batch
over the block; one rgc_apply_batch).

Inputs are drawn on the GPU from torch's seeded generator and copied to the
host for the oracle (inputs flow to the oracle, never results). Every output
is compared in full: P (bit-exact; QR under the margin rule), C after the
last microbatch (relative Frobenius), the updated W (the update bar of the
parity tests) and the norms. The workloads:

  * the Qwen3-1.7B-shaped block, r = 64 QR, 8 x 4096 tokens (the bench step);
  * the same block, r = 256 with a fixed Rademacher P, 16 x 4096 tokens;
  * a square 4096 x 4096 layer, r = 64 QR, Student-t activations, 32 x 4096
    tokens, 10 chained updates with a new projection seed each (the GPU
    chain against the oracle's own chain);
  * one layer of the Qwen3-8B-shaped set, r = 128 QR, 8 x 4096 tokens.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import rgc, synth
from parity_tools import assert_update_close, qr_margin_mismatches, rel_frobenius

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits

BLOCK_1P7B = [("q", 2048, 2048, "attn_in"), ("k", 1024, 2048, "attn_in"), ("v", 1024, 2048, "attn_in"),
              ("o", 2048, 2048, "attn_out"), ("gate", 6144, 2048, "mlp_in"), ("up", 6144, 2048, "mlp_in"),
              ("down", 2048, 6144, "mlp_act")]
ACTS_1P7B = {"attn_in": 2048, "attn_out": 2048, "mlp_in": 2048, "mlp_act": 6144}
LAYER_8B = [("q", 4096, 4096, "attn_in"), ("k", 1024, 4096, "attn_in"), ("v", 1024, 4096, "attn_in"),
            ("o", 4096, 4096, "attn_out"), ("gate", 12288, 4096, "mlp_in"), ("up", 12288, 4096, "mlp_in"),
            ("down", 4096, 12288, "mlp_act")]
ACTS_8B = {"attn_in": 4096, "attn_out": 4096, "mlp_in": 4096, "mlp_act": 12288}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


def _inputs(dev, mats, acts, tokens, seed0, x_dist="normal"):
    """X per activation (shared by the matrices that read it), D and W per
    matrix: X ~ N(0,1) (or Student-t(4) at unit variance), D ~ N(0, 1e-3^2),
    W ~ N(0, 0.02^2), bf16, drawn on the GPU."""
    X = {}
    for i, (name, width) in enumerate(acts.items()):
        if x_dist == "student_t":
            X[name] = synth.student_t_bf16((tokens, width), 4.0, seed=seed0 + 10 * i, device=dev)
        else:
            X[name] = synth.normal_bf16((tokens, width), 1.0, seed=seed0 + 10 * i, device=dev)
    D = [synth.normal_bf16((tokens, d), 1e-3, seed=seed0 + 100 + m, device=dev) for m, (_, d, _, _) in enumerate(mats)]
    W = [synth.normal_bf16((d, k), 0.02, seed=seed0 + 200 + m, device=dev) for m, (_, d, k, _) in enumerate(mats)]
    return X, D, W


def _gpu_update(dev, mats, X, D, W, kind, r, mb, p_seeds, sr_seeds, tau, P=None):
    """One update of the block through the batched entry points; W is updated
    in place. Returns P, C, stats."""
    tokens = D[0].shape[0]
    if P is None:
        P = [torch.empty((k, r), dtype=torch.bfloat16, device=dev) for _, _, k, _ in mats]
        rgc.rgc_sample_projections(kind, p_seeds, P)
    C = [torch.zeros((d, r), dtype=torch.float32, device=dev) for _, d, _, _ in mats]
    XP = [torch.empty((mb, r), dtype=torch.bfloat16, device=dev) for _ in mats]
    for i in range(tokens // mb):
        rgc.rgc_project_batch([X[src][i * mb:(i + 1) * mb] for _, _, _, src in mats], P, outs=XP)
        rgc.rgc_accumulate_batch([D[m][i * mb:(i + 1) * mb] for m in range(len(mats))], XP, C)
    stats = [torch.zeros(4, device=dev) for _ in mats]
    rgc.rgc_apply_batch(W, C, P, tau, sr_seeds, stats=stats)
    torch.cuda.synchronize()
    return P, C, stats


def _oracle_update(mats, xb, db, wb, kind, r, mb, p_seeds, sr_seeds, tau, pb=None):
    """The same update on the oracle, from host copies of the inputs (bits)."""
    tokens = db[0].shape[0]
    if pb is None:
        pb = [orc.sample_projection(kind, s, k, r) for s, (_, _, k, _) in zip(p_seeds, mats)]
    out = []
    for m, (_, d, k, src) in enumerate(mats):
        c = np.zeros((d, r), np.float32)
        for i in range(tokens // mb):
            xp = orc.project(xb[src][i * mb:(i + 1) * mb], pb[m])
            c = orc.accumulate(c, db[m][i * mb:(i + 1) * mb], xp)
        w_new, st = orc.apply_update(wb[m], c, pb[m], tau, sr_seeds[m])
        out.append((c, w_new, st))
    return pb, out


def _check_update(mats, kind, p_seeds, P, C, stats, W, pb, ref, what):
    for m, (name, d, k, _) in enumerate(mats):
        got_p = bits(P[m])
        if kind == "qr":
            assert qr_margin_mismatches(got_p, p_seeds[m], k, got_p.shape[1]) <= 2, f"{what} {name}: P"
        else:
            assert np.array_equal(got_p, pb[m]), f"{what} {name}: P"
        c_ref, w_ref, st_ref = ref[m]
        err = rel_frobenius(C[m].cpu().numpy(), c_ref)
        # 2e-3 is the bar; XP elements that round to the other bf16 neighbour
        # (allowed at 1e-3) carry into C at a few 1e-5
        assert err < 2e-3 and err < 1e-4, f"{what} {name}: C rel err {err:.2e}"
        st = stats[m].cpu().numpy()
        assert st[3] == 0 and st_ref[3] == 0
        np.testing.assert_allclose(st[:3], st_ref[:3], rtol=1e-5, err_msg=f"{what} {name}: stats")
        abs_terms = np.abs(c_ref.astype(np.float64)) @ np.abs(orc.bf16_to_f64(pb[m])).T
        assert_update_close(bits(W[m]), w_ref, st_ref[2], abs_terms, what=f"{what} {name}: W")


def _block_case(dev, mats, acts, kind, r, tokens, mb, seed0, tau=1e-3):
    X, D, W = _inputs(dev, mats, acts, tokens, seed0)
    xb = {n: bits(x) for n, x in X.items()}
    db = [bits(d) for d in D]
    wb = [bits(w) for w in W]
    p_seeds = [(seed0 << 32) | (m << 8) for m in range(len(mats))]
    sr_seeds = [(seed0 << 32) | (m << 8) | 1 for m in range(len(mats))]
    P, C, stats = _gpu_update(dev, mats, X, D, W, kind, r, mb, p_seeds, sr_seeds, tau)
    pb, ref = _oracle_update(mats, xb, db, wb, kind, r, mb, p_seeds, sr_seeds, tau)
    _check_update(mats, kind, p_seeds, P, C, stats, W, pb, ref, f"{kind} r={r}")


def test_qwen3_1p7b_block_r64_qr_step(dev):
    """The bench step: 7 projections, r = 64 QR, 32768 tokens in 8 x 4096."""
    _block_case(dev, BLOCK_1P7B, ACTS_1P7B, "qr", 64, 32768, 4096, seed0=2)


def test_qwen3_1p7b_block_r256_rademacher_step(dev):
    """Same block at r = 256 with a fixed Rademacher P, 65536 tokens in 16 x 4096."""
    _block_case(dev, BLOCK_1P7B, ACTS_1P7B, "rademacher", 256, 65536, 4096, seed0=3)


def test_qwen3_8b_layer_r128_qr_step(dev):
    """One layer of the Qwen3-8B-shaped set, r = 128 QR, 32768 tokens in 8 x 4096."""
    _block_case(dev, LAYER_8B, ACTS_8B, "qr", 128, 32768, 4096, seed0=5)


def test_square_layer_ten_chained_updates(dev):
    """d = k = 4096, r = 64 QR, Student-t(4) activations, 131072 tokens in
    32 x 4096, 10 updates with a new projection seed each; X and D fixed, W
    evolving. The GPU chain is compared with the oracle's own chain after every
    update."""
    mats = [("w", 4096, 4096, "x")]
    tau, r, mb, tokens = 1e-3, 64, 4096, 131072
    X, D, W = _inputs(dev, mats, {"x": 4096}, tokens, seed0=4, x_dist="student_t")
    xb = {"x": bits(X["x"])}
    db = [bits(D[0])]
    w_ref = bits(W[0])
    w_got = w_ref
    for u in range(10):
        p_seeds, sr_seeds = [(4 << 32) | (u << 8)], [(4 << 32) | (u << 8) | 1]
        P, C, stats = _gpu_update(dev, mats, X, D, W, "qr", r, mb, p_seeds, sr_seeds, tau)
        w_ref_prev, w_got_prev = w_ref, w_got
        pb, ref = _oracle_update(mats, xb, db, [w_ref], "qr", r, mb, p_seeds, sr_seeds, tau)
        c_ref, w_ref, st_ref = ref[0]
        assert qr_margin_mismatches(bits(P[0]), p_seeds[0], 4096, r) <= 2
        err = rel_frobenius(C[0].cpu().numpy(), c_ref)
        assert err < 2e-3 and err < 1e-4, f"update {u}: C rel err {err:.2e}"
        np.testing.assert_allclose(stats[0].cpu().numpy()[:3], st_ref[:3], rtol=1e-5)
        # a difference in the previous w moves the stochastically rounded
        # result by about the same amount (same random bits), so earlier
        # differences persist without growing while each update may add a few
        abs_terms = np.abs(c_ref.astype(np.float64)) @ np.abs(orc.bf16_to_f64(pb[0])).T
        w_got = bits(W[0])
        assert_update_close(w_got, w_ref, st_ref[2], abs_terms, max_mismatch_frac=1e-4 * (u + 1),
                            what=f"update {u}: W", prev_got_bits=w_got_prev, prev_ref_bits=w_ref_prev)
