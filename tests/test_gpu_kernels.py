"""Kernel-level parity of the HIP path against the CPU oracle (GPU only)."""
import math
import sys

import numpy as np
import pytest

import oracle as O
from oracle.gpt import _Num
from tests.gpu_util import rel_err, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():   # collected on CPU hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import gpt_pretraining_step_amd as G  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def rnd_in(shape, seed, scale=1.0, bf16=True):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * scale
    return O.round_bf16(x) if bf16 else x


def tdtype(dt):
    return torch.bfloat16 if dt == G.BF16 else torch.float32


# ------------------------------------------------------------------ GEMM
GEMM_SHAPES = [(130, 70, 50), (256, 256, 64), (300, 200, 96), (512, 384, 256),
               (1000, 257, 160)]


def _gemm_ref(op, A, B):
    A64, B64 = A.astype(np.float64), B.astype(np.float64)
    if op == G.GEMM_NT:
        return A64 @ B64.T
    if op == G.GEMM_NN:
        return A64 @ B64
    return A64.T @ B64


@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("op", [G.GEMM_NT, G.GEMM_NN, G.GEMM_TN])
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm_store_and_f32(dt, op, shape):
    M, N, K = shape
    say("gemm", dt, op, shape)
    bf = dt == G.BF16
    Ash = (M, K) if op != G.GEMM_TN else (K, M)
    Bsh = (N, K) if op == G.GEMM_NT else (K, N)
    A, B = rnd_in(Ash, 1, bf16=bf), rnd_in(Bsh, 2, bf16=bf)
    ref = _gemm_ref(op, A, B)
    tA, tB = dev(A, tdtype(dt)), dev(B, tdtype(dt))
    lda, ldb = Ash[1], Bsh[1]
    C = torch.zeros(M, N, dtype=tdtype(dt), device=DEV)
    G.k_gemm(op, M, N, K, tA, lda, tB, ldb, C, N, G.EPI_STORE, None, dt)
    C32 = torch.full((M, N), 0.5, dtype=torch.float32, device=DEV)
    G.k_gemm(op, M, N, K, tA, lda, tB, ldb, C32, N, G.EPI_F32_ACC, None, dt)
    torch.cuda.synchronize()
    tol = 8e-3 if bf else 1e-5
    assert rel_err(to_np(C), ref) < tol
    assert rel_err(to_np(C32), ref + 0.5) < 1e-5
    if bf and op == G.GEMM_TN:
        # the same products with split-K scratch: partial tiles summed in order
        sb = G.k_gemm_scratch_bytes(M, N, K)
        scr = torch.empty(max(sb, 16), dtype=torch.uint8, device=DEV)
        S32 = torch.full((M, N), 0.5, dtype=torch.float32, device=DEV)
        G.k_gemm(op, M, N, K, tA, lda, tB, ldb, S32, N, G.EPI_F32_ACC, None, dt, scratch=scr)
        S0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
        G.k_gemm(op, M, N, K, tA, lda, tB, ldb, S0, N, G.EPI_F32, None, dt, scratch=scr)
        torch.cuda.synchronize()
        assert rel_err(to_np(S32), ref + 0.5) < 1e-5
        assert rel_err(to_np(S0), ref) < 1e-5


@pytest.mark.parametrize("op", [G.GEMM_NT, G.GEMM_NN, G.GEMM_TN])
@pytest.mark.parametrize("M,N,K", [(4096, 8192, 128), (4136, 8192, 192)])
def test_gemm_large_tiles(op, M, N, K):
    """Products big enough for the 256x256 double-buffered kernel (ragged M)."""
    say("gemm large", op, M, N, K)
    Ash = (M, K) if op != G.GEMM_TN else (K, M)
    Bsh = (N, K) if op == G.GEMM_NT else (K, N)
    A, B = rnd_in(Ash, 21), rnd_in(Bsh, 22)
    tA, tB = dev(A, torch.bfloat16), dev(B, torch.bfloat16)
    C = torch.empty(M, N, dtype=torch.float32, device=DEV)
    G.k_gemm(op, M, N, K, tA, Ash[1], tB, Bsh[1], C, N, G.EPI_F32, None, G.BF16)
    R = dev(rnd_in((M, N), 23), torch.bfloat16)
    R0 = R.clone()
    G.k_gemm(op, M, N, K, tA, Ash[1], tB, Bsh[1], R, N, G.EPI_RESADD, None, G.BF16)
    torch.cuda.synchronize()
    ref = torch.from_numpy(_gemm_ref(op, A, B)).to(DEV)
    assert rel_err(to_np(C), to_np(ref)) < 1e-5
    assert rel_err(to_np(R), to_np(R0.double() + ref)) < 2e-2


@pytest.mark.parametrize("M,N,K", [(256, 512, 4096), (384, 128, 8192), (64, 96, 1024),
                                   (512, 512, 8192), (520, 776, 8192)])
def test_gemm_tn_split_k(M, N, K):
    """Weight-gradient shapes: few output tiles, long reduction."""
    A, B = rnd_in((K, M), 13), rnd_in((K, N), 14)
    ref = A.astype(np.float64).T @ B.astype(np.float64)
    sb = G.k_gemm_scratch_bytes(M, N, K)
    assert sb > 0
    scr = torch.empty(sb, dtype=torch.uint8, device=DEV)
    C32 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    tA, tB = dev(A, torch.bfloat16), dev(B, torch.bfloat16)
    G.k_gemm(G.GEMM_TN, M, N, K, tA, M, tB, N, C32, N, G.EPI_F32, None, G.BF16, scratch=scr)
    first = C32.clone()
    G.k_gemm(G.GEMM_TN, M, N, K, tA, M, tB, N, C32, N, G.EPI_F32, None, G.BF16, scratch=scr)
    torch.cuda.synchronize()
    assert rel_err(to_np(C32), ref) < 1e-5
    assert torch.equal(first, C32)            # fixed-order reduction: bitwise repeatable


@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("shape", [(200, 130, 64), (512, 256, 128)])
def test_gemm_epilogues(dt, shape):
    M, N, K = shape
    bf = dt == G.BF16
    num = _Num("bf16emu" if bf else "fp32")
    A, B = rnd_in((M, K), 3, bf16=bf), rnd_in((N, K), 4, bf16=bf)
    acc = (A.astype(np.float64) @ B.astype(np.float64).T).astype(np.float32)
    R = rnd_in((M, N), 5, bf16=bf)
    U = rnd_in((M, N), 6, bf16=bf)
    tA, tB = dev(A, tdtype(dt)), dev(B, tdtype(dt))
    # residual add
    C = dev(R, tdtype(dt))
    G.k_gemm(G.GEMM_NT, M, N, K, tA, K, tB, K, C, N, G.EPI_RESADD, None, dt)
    # relu^2 (a = relu(u)^2 with u rounded first)
    Ca = torch.zeros(M, N, dtype=tdtype(dt), device=DEV)
    G.k_gemm(G.GEMM_NT, M, N, K, tA, K, tB, K, Ca, N, G.EPI_RELU2, None, dt)
    # relu^2 backward from the stored a: du = acc * 2 sqrt(a)
    Cd = torch.zeros(M, N, dtype=tdtype(dt), device=DEV)
    Ua = num.rnd(np.maximum(U, 0) ** 2)
    tUa = dev(Ua, tdtype(dt))
    G.k_gemm(G.GEMM_NT, M, N, K, tA, K, tB, K, Cd, N, G.EPI_DRELU2, tUa, dt)
    torch.cuda.synchronize()
    tol = 2e-2 if bf else 1e-5
    assert rel_err(to_np(C), num.rnd(R + acc)) < tol
    u = num.rnd(acc)
    assert rel_err(to_np(Ca), num.rnd(np.maximum(u, 0) ** 2)) < tol
    assert rel_err(to_np(Cd), num.rnd(acc * 2 * np.sqrt(Ua))) < tol
    # sqrt of the stored a is relu(u) to within half a rounding step
    assert rel_err(np.sqrt(Ua), np.maximum(U, 0)) < (4e-3 if bf else 1e-6)


@pytest.mark.parametrize("op", [G.GEMM_NT, G.GEMM_NN, G.GEMM_TN])
def test_gemm_direct_to_lds_epilogues(op):
    """A product large enough for the direct-to-LDS kernel (>= 2^31 multiply-
    adds, K % 64 == 0), ragged in M and N, through every epilogue."""
    M, N, K = 1288, 1032, 2048
    say("gemm dma", op, M, N, K)
    num = _Num("bf16emu")
    Ash = (M, K) if op != G.GEMM_TN else (K, M)
    Bsh = (N, K) if op == G.GEMM_NT else (K, N)
    A, B = rnd_in(Ash, 31), rnd_in(Bsh, 32)
    acc = _gemm_ref(op, A, B)
    R, U = rnd_in((M, N), 33, 4.0), rnd_in((M, N), 34)
    tA, tB = dev(A, torch.bfloat16), dev(B, torch.bfloat16)
    lda, ldb = Ash[1], Bsh[1]
    bf = torch.bfloat16

    def run(epi, C, aux=None):
        G.k_gemm(op, M, N, K, tA, lda, tB, ldb, C, N, epi, aux, G.BF16)
        return C

    Cs = run(G.EPI_STORE, torch.zeros(M, N, dtype=bf, device=DEV))
    Cf = run(G.EPI_F32, torch.zeros(M, N, dtype=torch.float32, device=DEV))
    Ca = run(G.EPI_F32_ACC, torch.full((M, N), 0.25, dtype=torch.float32, device=DEV))
    Cr = run(G.EPI_RESADD, dev(R, bf))
    Ca2 = run(G.EPI_RELU2, torch.zeros(M, N, dtype=bf, device=DEV))
    Ua = num.rnd(np.maximum(U, 0) ** 2)
    Cd = run(G.EPI_DRELU2, torch.zeros(M, N, dtype=bf, device=DEV), dev(Ua, bf))
    torch.cuda.synchronize()
    acc32 = acc.astype(np.float32)
    assert rel_err(to_np(Cf), acc) < 1e-5
    assert rel_err(to_np(Ca), acc + 0.25) < 1e-5
    assert rel_err(to_np(Cs), acc) < 8e-3
    assert rel_err(to_np(Cr), num.rnd(R + acc32)) < 2e-2
    u = num.rnd(acc32)
    assert rel_err(to_np(Ca2), num.rnd(np.maximum(u, 0) ** 2)) < 2e-2
    assert rel_err(to_np(Cd), num.rnd(acc32 * 2 * np.sqrt(Ua))) < 2e-2


# --------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("D", [16, 100, 256, 768, 1536])
def test_rmsnorm(dt, D):
    rows = 77
    bf = dt == G.BF16
    num = _Num("bf16emu" if bf else "fp32")
    x = rnd_in((rows, D), 7, 3.0, bf)
    dy = rnd_in((rows, D), 8, 1.0, bf)
    dres = rnd_in((rows, D), 9, 1.0, bf)
    y_ref, r_ref = O.rmsnorm(x, 1e-5, num)
    tx = dev(x, tdtype(dt))
    ty = torch.empty_like(tx)
    tr = torch.empty(rows, dtype=torch.float32, device=DEV)
    G.k_rmsnorm_fwd(tx, ty, tr, rows, D, 1e-5, dt)
    tdx = dev(dres, tdtype(dt))
    G.k_rmsnorm_bwd(dev(dy, tdtype(dt)), ty, tr, tdx, tdx, rows, D, dt)
    torch.cuda.synchronize()
    tol = 1e-2 if bf else 1e-5
    assert rel_err(to_np(ty), y_ref) < tol
    assert rel_err(to_np(tr), r_ref) < 1e-5
    dx_ref = num.rnd(dres + O.rmsnorm_bwd(dy, y_ref, r_ref, num))
    assert rel_err(to_np(tdx), dx_ref) < (2e-2 if bf else 1e-5)


# ------------------------------------------------- rotary + QK-norm
@pytest.mark.parametrize("dt,hd", [(G.F32, 4), (G.BF16, 64), (G.BF16, 128), (G.F32, 128)])
def test_rope_qknorm(dt, hd):
    B, T, H, Hkv = 2, 50, 4, 2
    bf = dt == G.BF16
    num = _Num("bf16emu" if bf else "fp32")
    ld = (H + 2 * Hkv) * hd
    qkv = rnd_in((B, T, ld), 10, 1.0, bf)
    cs = torch.empty(T * hd, dtype=torch.float32, device=DEV)
    G.k_rope_table(cs, T, hd, 10000.0)
    tq = dev(qkv, tdtype(dt)).reshape(B * T, ld)
    rq = torch.empty(B * T * H, dtype=torch.float32, device=DEV)
    rk = torch.empty(B * T * Hkv, dtype=torch.float32, device=DEV)
    G.k_rope_qknorm_fwd(tq, rq, rk, cs, B, T, H, Hkv, hd, 1e-5, dt)
    cos, sin = O.rope_tables(T, hd, 10000.0)
    q = qkv[..., :H * hd].reshape(B, T, H, hd)
    k = qkv[..., H * hd:(H + Hkv) * hd].reshape(B, T, Hkv, hd)
    qn, rq_ref = O.rmsnorm(O.rope(q, cos, sin, num), 1e-5, num)
    kn, rk_ref = O.rmsnorm(O.rope(k, cos, sin, num), 1e-5, num)
    dqkv = rnd_in((B, T, ld), 11, 1.0, bf)
    td = dev(dqkv, tdtype(dt)).reshape(B * T, ld)
    G.k_rope_qknorm_bwd(td, tq, rq, rk, cs, B, T, H, Hkv, hd, dt)
    torch.cuda.synchronize()
    got = to_np(tq).reshape(B, T, ld)
    tol = 1e-2 if bf else 1e-5
    assert rel_err(got[..., :H * hd], qn.reshape(B, T, -1)) < tol
    assert rel_err(got[..., H * hd:(H + Hkv) * hd], kn.reshape(B, T, -1)) < tol
    np.testing.assert_array_equal(got[..., (H + Hkv) * hd:], qkv[..., (H + Hkv) * hd:])
    assert rel_err(to_np(rq), rq_ref.reshape(-1)) < 1e-5
    assert rel_err(to_np(rk), rk_ref.reshape(-1)) < 1e-5
    gq = dqkv[..., :H * hd].reshape(B, T, H, hd)
    gk = dqkv[..., H * hd:(H + Hkv) * hd].reshape(B, T, Hkv, hd)
    yq = to_np(tq).reshape(B, T, ld)[..., :H * hd].reshape(B, T, H, hd)
    yk = to_np(tq).reshape(B, T, ld)[..., H * hd:(H + Hkv) * hd].reshape(B, T, Hkv, hd)
    rq_g = to_np(rq).reshape(B, T, H)
    rk_g = to_np(rk).reshape(B, T, Hkv)
    dq_ref = num.rnd(O.rope_bwd(O.rmsnorm_bwd(gq, yq, rq_g, num), cos, sin, num))
    dk_ref = num.rnd(O.rope_bwd(O.rmsnorm_bwd(gk, yk, rk_g, num), cos, sin, num))
    gd = to_np(td).reshape(B, T, ld)
    tolb = 2e-2 if bf else 1e-5
    assert rel_err(gd[..., :H * hd], dq_ref.reshape(B, T, -1)) < tolb
    assert rel_err(gd[..., H * hd:(H + Hkv) * hd], dk_ref.reshape(B, T, -1)) < tolb


# -------------------------------------------------------------- attention
ATTN_CASES = [
    # dt, B, T, H, Hkv, hd, W
    (G.F32, 2, 16, 4, 2, 4, 16),
    (G.F32, 2, 37, 4, 2, 4, 5),
    (G.F32, 1, 40, 2, 1, 32, 0),
    (G.BF16, 2, 130, 2, 1, 64, 31),
    (G.BF16, 2, 128, 2, 2, 128, 128),
    (G.BF16, 1, 300, 6, 2, 128, 64),
    (G.BF16, 2, 257, 2, 2, 128, 127),
    (G.BF16, 1, 512, 4, 4, 128, 100),
]


def _attn_inputs(B, T, H, Hkv, hd, bf, seed=12):
    num = _Num("bf16emu" if bf else "fp32")
    q = rnd_in((B, T, H, hd), seed, 1.0, bf)
    k = rnd_in((B, T, Hkv, hd), seed + 1, 1.0, bf)
    v = rnd_in((B, T, Hkv, hd), seed + 2, 1.0, bf)
    # q and k unit-RMS per head, as after QK-norm
    q = O.rmsnorm(q, 1e-5, num)[0]
    k = O.rmsnorm(k, 1e-5, num)[0]
    qkv = np.concatenate([q.reshape(B, T, -1), k.reshape(B, T, -1), v.reshape(B, T, -1)], -1)
    return q, k, v, qkv


@pytest.mark.parametrize("bounded", [False, True])
@pytest.mark.parametrize("case", ATTN_CASES)
def test_attention_fwd_bwd(case, bounded):
    """bounded: the forward is told that |q . k| / sqrt(hd) <= 1.01 sqrt(hd),
    which holds for these unit-RMS rows (the step's QK-normed q and k)."""
    dt, B, T, H, Hkv, hd, W = case
    say("attn", case, "bounded" if bounded else "")
    bf = dt == G.BF16
    num = _Num("bf16emu" if bf else "fp32")
    q, k, v, qkv = _attn_inputs(B, T, H, Hkv, hd, bf)
    o_ref, lse_ref = O.attention(q, k, v, W, num)
    do = rnd_in((B, T, H, hd), 20, 1.0, bf)
    dq_ref, dk_ref, dv_ref = O.attention_bwd(q, k, v, o_ref, lse_ref, do, W, num)
    tqkv = dev(qkv, tdtype(dt)).reshape(B * T, -1)
    to = torch.empty(B * T, H * hd, dtype=tdtype(dt), device=DEV)
    tl = torch.empty(B * H * T, dtype=torch.float32, device=DEV)
    G.k_attn_fwd(tqkv, to, tl, B, T, H, Hkv, hd, W, dt,
                 score_bound=1.01 * np.sqrt(hd) if bounded else 0.0)
    # the backward consumes the kernel's own o and lse, as in the step
    tdq = torch.zeros_like(tqkv)
    scr = torch.empty(max(16, G.k_attn_bwd_scratch_bytes(B, T, H, hd)), dtype=torch.uint8,
                      device=DEV)
    G.k_attn_bwd(tqkv, to, tl, dev(do, tdtype(dt)).reshape(B * T, -1), tdq, scr, B, T, H, Hkv,
                 hd, W, dt)
    torch.cuda.synchronize()
    tol = 2e-2 if bf else 1e-4
    assert rel_err(to_np(to).reshape(B, T, H, hd), o_ref) < tol
    assert rel_err(to_np(tl).reshape(B, H, T), lse_ref) < 1e-5
    g = to_np(tdq).reshape(B, T, -1)
    if W == 0:
        # each query sees only itself: P = 1, dS = dP - Delta = 0, so dq and
        # dk are exactly zero and the oracle's values are rounding noise
        assert np.abs(g[..., :(H + Hkv) * hd]).max() < 1e-5
        assert np.abs(dq_ref).max() < 1e-5 and np.abs(dk_ref).max() < 1e-5
    else:
        assert rel_err(g[..., :H * hd], dq_ref.reshape(B, T, -1)) < tol
        assert rel_err(g[..., H * hd:(H + Hkv) * hd], dk_ref.reshape(B, T, -1)) < tol
    assert rel_err(g[..., (H + Hkv) * hd:], dv_ref.reshape(B, T, -1)) < tol


@pytest.mark.parametrize("bounded", [False, True])
@pytest.mark.parametrize("W", [0, 1, 31, 32, 64, 127, 128])
@pytest.mark.parametrize("hd", [128, 32])
def test_attention_mask_exact_one_hot_values(W, hd, bounded):
    """With v_j = e_j the output row i is the probability row P_i itself, so
    its zero pattern must equal the window predicate exactly."""
    T = hd
    B, H, Hkv = 1, 2, 1
    dt = G.BF16
    q, k, _, _ = _attn_inputs(B, T, H, Hkv, hd, True, seed=30)
    q = q * 0.25                                  # keep every visible p far from 0
    v = np.zeros((B, T, Hkv, hd), np.float32)
    v[0, np.arange(T), 0, np.arange(T)] = 1.0
    qkv = np.concatenate([O.round_bf16(q).reshape(B, T, -1), k.reshape(B, T, -1),
                          v.reshape(B, T, -1)], -1)
    tqkv = dev(qkv, torch.bfloat16).reshape(B * T, -1)
    to = torch.empty(B * T, H * hd, dtype=torch.bfloat16, device=DEV)
    tl = torch.empty(B * H * T, dtype=torch.float32, device=DEV)
    G.k_attn_fwd(tqkv, to, tl, B, T, H, Hkv, hd, W, dt,
                 score_bound=1.01 * np.sqrt(hd) if bounded else 0.0)
    torch.cuda.synchronize()
    o = to_np(to).reshape(T, H, hd)
    mask = O.visible_mask(T, W)
    for h in range(H):
        np.testing.assert_array_equal(o[:, h, :] != 0.0, mask)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_attention_bounded_extreme_scores(sign):
    """Every key equal to +-q (one shared unit-RMS vector): every score is
    +-sqrt(hd), the two ends of the bound.  Attention is then uniform over
    the visible keys, so o_i is the mean of the visible v_j and
    lse_i = ln(count) +- sqrt(hd), whatever the fixed offset."""
    B, T, H, Hkv, hd, W = 1, 200, 2, 1, 128, 70
    rng = np.random.default_rng(7)
    x = rng.standard_normal(hd).astype(np.float32)
    x = O.round_bf16(x / np.sqrt(np.mean(x.astype(np.float64) ** 2)))
    q = np.broadcast_to(x, (B, T, H, hd)).astype(np.float32)
    k = np.broadcast_to(sign * x, (B, T, Hkv, hd)).astype(np.float32)
    v = O.round_bf16(rng.standard_normal((B, T, Hkv, hd)).astype(np.float32))
    qkv = np.concatenate([q.reshape(B, T, -1), k.reshape(B, T, -1), v.reshape(B, T, -1)], -1)
    tqkv = dev(qkv, torch.bfloat16).reshape(B * T, -1)
    to = torch.empty(B * T, H * hd, dtype=torch.bfloat16, device=DEV)
    tl = torch.empty(B * H * T, dtype=torch.float32, device=DEV)
    G.k_attn_fwd(tqkv, to, tl, B, T, H, Hkv, hd, W, G.BF16, score_bound=1.01 * np.sqrt(hd))
    torch.cuda.synchronize()
    s = float(np.dot(x.astype(np.float64), sign * x.astype(np.float64))) / np.sqrt(hd)
    lo = np.maximum(np.arange(T) - W, 0)
    cnt = np.arange(T) - lo + 1
    csum = np.concatenate([np.zeros((1, hd)), np.cumsum(v[0, :, 0].astype(np.float64), 0)])
    mean = (csum[np.arange(T) + 1] - csum[lo]) / cnt[:, None]
    o = to_np(to).reshape(T, H, hd)
    for h in range(H):
        assert rel_err(o[:, h], mean) < 1e-2
    np.testing.assert_allclose(to_np(tl).reshape(H, T), np.broadcast_to(np.log(cnt) + s, (H, T)),
                               rtol=0, atol=1e-4)


# ----------------------------------------------------------- cross-entropy
# ------------------------------------------------ token / value embedding
def _tokens(B, T, V, seed, spread):
    """Rows of T+1 ids; ids drawn from the first `spread` entries so most
    repeat, and every id >= spread is absent from the batch."""
    return np.random.default_rng(seed).integers(0, spread, (B, T + 1)).astype(np.int32)


@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("D,sorted_path", [(96, True), (96, False), (30, False)])
def test_token_embedding(dt, D, sorted_path):
    B, T, V = 3, 70, 300
    say("embed", dt, D, sorted_path)
    bf = dt == G.BF16
    tok = _tokens(B, T, V, 60, 40)
    inp = tok[:, :T]
    wte = rnd_in((V, D), 61, bf16=bf)
    dx = rnd_in((B * T, D), 62, bf16=bf)
    ttok = dev(tok, torch.int32)
    x = torch.empty(B * T, D, dtype=tdtype(dt), device=DEV)
    G.k_embed_fwd(ttok, B, T, dev(wte, tdtype(dt)), V, D, x, dt)
    scr = (torch.empty(G.k_embed_bwd_scratch_bytes(B, T, V, D), dtype=torch.uint8, device=DEV)
           if sorted_path else None)
    tdx = dev(dx, tdtype(dt))
    dW = torch.full((V, D), 7.0, dtype=torch.float32, device=DEV)   # overwritten
    G.k_embed_bwd(ttok, B, T, tdx, V, D, dW, 0, scr, dt)
    first = dW.clone()
    G.k_embed_bwd(ttok, B, T, tdx, V, D, dW, 1, scr, dt)            # += the same
    torch.cuda.synchronize()
    # the lookup copies rows exactly
    np.testing.assert_array_equal(to_np(x).reshape(B, T, D), wte[inp])
    ref = O.embedding_bwd(dx.astype(np.float64), inp, V)
    assert rel_err(to_np(first), ref) < 1e-6
    assert rel_err(to_np(dW), 2 * ref) < 1e-6
    assert np.all(to_np(first)[40:] == 0.0)          # absent ids: exact zeros
    if sorted_path:                                   # fixed summation order
        G.k_embed_bwd(ttok, B, T, tdx, V, D, dW, 0, scr, dt)
        torch.cuda.synchronize()
        assert torch.equal(first, dW)


@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("C,hd", [(32, 16), (7, 32), (64, 128)])
def test_value_embedding(dt, C, hd):
    B, T, V, D, H, Hkv = 2, 50, 60, 64, 2, 2
    say("ve", dt, C, hd)
    bf = dt == G.BF16
    num = _Num("bf16emu" if bf else "fp32")
    tok = _tokens(B, T, V, 70, 25)
    inp = tok[:, :T]
    ld = (H + 2 * Hkv) * hd
    voff = (H + Hkv) * hd
    h = rnd_in((B, T, D), 71, bf16=bf)
    wg = rnd_in((Hkv, C), 72, 0.3, bf16=bf)
    E = rnd_in((V, Hkv * hd), 73, bf16=bf)
    qkv = rnd_in((B * T, ld), 74, bf16=bf)
    v = qkv[:, voff:].reshape(B, T, Hkv, hd)
    v_ref, g_ref, e = O.value_embedding(v, h, wg, E, inp, C, num)
    ttok = dev(tok, torch.int32)
    th, twg, tE = dev(h, tdtype(dt)).reshape(B * T, D), dev(wg, tdtype(dt)), dev(E, tdtype(dt))
    tqkv = dev(qkv, tdtype(dt))
    g = torch.empty(B * T, Hkv, dtype=torch.float32, device=DEV)
    G.k_ve_fwd(ttok, B, T, th, D, twg, C, tE, tqkv, ld, voff, g, Hkv, hd, dt)
    # backward from a random dv (in the v slot of a dqkv buffer)
    dqkv = rnd_in((B * T, ld), 75, bf16=bf)
    dv = dqkv[:, voff:].reshape(B, T, Hkv, hd)
    dzg, dwg_ref, dE_ref, _ = O.value_embedding_bwd(dv.astype(np.float64), g_ref.astype(np.float64),
                                                    e.astype(np.float64), h.astype(np.float64),
                                                    wg.astype(np.float64), inp, V)
    vez = torch.empty(B * T, Hkv, dtype=torch.float32, device=DEV)
    dE = torch.empty(V, Hkv * hd, dtype=torch.float32, device=DEV)
    dwg = torch.empty(Hkv, C, dtype=torch.float32, device=DEV)
    scr = torch.empty(G.k_ve_bwd_scratch_bytes(B, T, V, Hkv, hd, C), dtype=torch.uint8,
                      device=DEV)
    G.k_ve_bwd(ttok, B, T, dev(dqkv, tdtype(dt)), ld, voff, tE, g, th, D, C, V, Hkv, hd, vez, dE,
               dwg, 0, scr, dt)
    torch.cuda.synchronize()
    out = to_np(tqkv)
    tol = 2e-2 if bf else 1e-5
    assert rel_err(out[:, voff:].reshape(B, T, Hkv, hd), v_ref) < tol
    np.testing.assert_array_equal(out[:, :voff], qkv[:, :voff])      # q, k untouched
    assert rel_err(to_np(g).reshape(B, T, Hkv), g_ref) < 1e-5
    assert rel_err(to_np(vez).reshape(B, T, Hkv), dzg) < 1e-5
    assert rel_err(to_np(dE), dE_ref) < 1e-5
    assert rel_err(to_np(dwg), dwg_ref) < 1e-5


@pytest.mark.parametrize("rows,D,V,scale", [(300, 128, 1024, 1.0), (513, 64, 32768, 0.3),
                                            (37, 256, 512, 4.0)])
def test_fused_lm_head_cross_entropy(rows, D, V, scale):
    """The step's fused lm_head + CE path against the oracle's CE on the
    exact logits of the same bf16 inputs: ragged row tiles, targets on tile
    edges, and (scale 4) logits spread over +-100, where exp(logit - tile
    max) falls far below fp16's range for most columns."""
    say("lm_ce", rows, D, V, scale)
    rng = np.random.default_rng(50 + rows)
    h = O.round_bf16(rng.standard_normal((rows, D)).astype(np.float32))
    w = O.round_bf16((rng.standard_normal((V, D)) * scale / np.sqrt(D) * 8).astype(np.float32))
    tgt = rng.integers(0, V, rows).astype(np.int32)
    edges = [0, 255, 256, V - 1, V - 256, 511 % V]
    tgt[:len(edges)] = edges
    z = (h.astype(np.float64) @ w.astype(np.float64).T)
    num = _Num("bf16emu")
    ell_ref, lse_ref, dz_ref = O.cross_entropy(z, tgt, num)
    ell = torch.empty(rows, dtype=torch.float32, device=DEV)
    lse = torch.empty(rows, dtype=torch.float32, device=DEV)
    dz = torch.empty(rows, V, dtype=torch.bfloat16, device=DEV)
    scr = torch.empty(G.k_lm_ce_scratch_bytes(rows, V), dtype=torch.uint8, device=DEV)
    G.k_lm_ce(dev(h, torch.bfloat16), dev(w, torch.bfloat16), dev(tgt, torch.int32), rows, D, V,
              ell, lse, dz, 1.0 / rows, scr)
    torch.cuda.synchronize()
    # fp32 accumulation of the logits: lse and the loss to ~1e-6 relative
    assert np.abs(to_np(lse) - lse_ref).max() < 1e-5 * max(1.0, np.abs(lse_ref).max())
    assert np.abs(to_np(ell) - ell_ref).max() < 1e-5 * max(1.0, np.abs(lse_ref).max())
    assert rel_err(to_np(dz), num.rnd(dz_ref)) < 1e-2


@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("V", [27, 1000, 32768])
def test_cross_entropy(dt, V):
    rows = 37
    rng = np.random.default_rng(40)
    z = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    tgt = rng.integers(0, V, rows).astype(np.int32)
    num = _Num("bf16emu" if dt == G.BF16 else "fp32")
    ell_ref, lse_ref, dz_ref = O.cross_entropy(z, tgt, num)
    tz = dev(z, torch.float32)
    ell = torch.empty(rows, dtype=torch.float32, device=DEV)
    lse = torch.empty(rows, dtype=torch.float32, device=DEV)
    dz = torch.empty(rows, V, dtype=tdtype(dt), device=DEV)
    G.k_ce(tz, dev(tgt, torch.int32), rows, V, ell, lse, dz, 1.0 / rows, dt)
    torch.cuda.synchronize()
    assert rel_err(to_np(ell), ell_ref) < 1e-5
    assert rel_err(to_np(lse), lse_ref) < 1e-6
    assert rel_err(to_np(dz), num.rnd(dz_ref)) < (1e-2 if dt == G.BF16 else 1e-5)


# ------------------------------------------------------ KV-cache decode
# B, Tq, Tmax, H, Hkv, window, cache lengths
DECODE_CASES = [
    (3, 1, 300, 6, 6, 300, [300, 1, 157]),
    (2, 4, 1000, 8, 2, 100, [1000, 517]),
    (1, 1, 64, 2, 1, 64, [64]),
    (4, 3, 2048, 12, 2, 1023, [2048, 2000, 5, 0]),
    (2, 2, 700, 4, 4, 5000, [9000, -4]),
    (5, 1, 4096, 6, 2, 4096, [4096, 4000, 3333, 64, 65]),
    (2, 16, 513, 2, 1, 40, [513, 200]),
]


def decode_inputs(B, Tq, Tmax, H, Hkv, lens, seed=40, nan_tail=True):
    """q and cached k unit-RMS per head (rows after QK-norm), v N(0, 1), all
    bf16; cache rows at or past a sequence's length hold NaN, which must never
    reach the output."""
    num = _Num("bf16emu")
    q = O.rmsnorm(rnd_in((B, Tq, H, 128), seed), 1e-5, num)[0]
    kc = O.rmsnorm(rnd_in((B, Tmax, Hkv, 128), seed + 1), 1e-5, num)[0]
    vc = rnd_in((B, Tmax, Hkv, 128), seed + 2)
    if nan_tail:
        for b, L in enumerate(lens):
            L = min(max(L, 0), Tmax)
            kc[b, L:] = np.nan
            vc[b, L:] = np.nan
    return q, kc, vc


def run_decode(q, kc, vc, lens, W, bounded, scr=None):
    B, Tq, H, _ = q.shape
    Tmax, Hkv = kc.shape[1], kc.shape[2]
    tq, tk, tv = (dev(a, torch.bfloat16) for a in (q, kc, vc))
    tlen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    to = torch.empty(B, Tq, H, 128, dtype=torch.bfloat16, device=DEV)
    tl = torch.empty(B, H, Tq, dtype=torch.float32, device=DEV)
    nb = G.k_attn_decode_scratch_bytes(B, Tq, H, Hkv, Tmax, W)
    if scr is None:
        scr = torch.zeros(max(nb, 16), dtype=torch.uint8, device=DEV)
    assert scr.numel() >= nb
    G.k_attn_decode(tq, tk, tv, tlen, to, tl, B, Tq, Tmax, H, Hkv, 128, W,
                    1.01 * math.sqrt(128) if bounded else 0.0, scr, G.BF16)
    torch.cuda.synchronize()
    return to_np(to), to_np(tl), nb


@pytest.mark.parametrize("bounded", [False, True])
@pytest.mark.parametrize("case", DECODE_CASES)
def test_attention_decode(case, bounded):
    """Decode attention of the newest Tq tokens over per-sequence cache
    lengths (ragged, empty, shorter than Tq, clamped) against the oracle;
    split-key chunks and their merge included (scratch > 0)."""
    B, Tq, Tmax, H, Hkv, W, lens = case
    say("decode", case, "bounded" if bounded else "")
    q, kc, vc = decode_inputs(B, Tq, Tmax, H, Hkv, lens)
    o_ref, lse_ref = O.decode_attention(q, kc, vc, np.array(lens), W, _Num("bf16emu"))
    o, lse, nb = run_decode(q, kc, vc, lens, W, bounded)
    say("  scratch bytes", nb)
    assert np.isfinite(o).all()
    assert rel_err(o, o_ref) < 2e-2
    dead = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), dead)
    assert np.all(o.transpose(0, 2, 1, 3)[dead] == 0.0)
    if (~dead).any():
        assert rel_err(lse[~dead], lse_ref[~dead]) < 1e-5


def test_attention_decode_one_hot_values_and_determinism():
    """v_j = e_(j mod 128) turns each output row into sums of probabilities
    over keys j = c (mod 128): with a window below 128 every visible key has
    its own column, so the zero pattern of the output must equal the window
    predicate exactly.  Two calls give identical bits."""
    B, Tq, Tmax, H, Hkv, W = 2, 3, 900, 4, 2, 100
    lens = [900, 333]
    q, kc, _ = decode_inputs(B, Tq, Tmax, H, Hkv, lens, seed=50, nan_tail=False)
    vc = np.zeros((B, Tmax, Hkv, 128), np.float32)
    vc[:, np.arange(Tmax), :, np.arange(Tmax) % 128] = 1.0
    o, lse, _ = run_decode(q, kc, vc, lens, W, False)
    for b, L in enumerate(lens):
        for t in range(Tq):
            p = L - Tq + t
            vis = np.zeros(128, bool)
            for j in range(max(0, p - W), p + 1):
                vis[j % 128] = True
            for h in range(H):
                assert np.array_equal(o[b, t, h] > 0, vis), (b, t, h)
    o2, lse2, _ = run_decode(q, kc, vc, lens, W, False)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_attention_decode_scratch_reuse():
    """One zero-filled scratch buffer serves consecutive calls of different
    shapes and chunk counts (each call leaves its arrival counters at zero):
    every call equals the same call on a fresh buffer."""
    cases = [DECODE_CASES[5], DECODE_CASES[1], DECODE_CASES[0], DECODE_CASES[5],
             DECODE_CASES[3]]
    shared = torch.zeros(1 << 24, dtype=torch.uint8, device=DEV)
    for B, Tq, Tmax, H, Hkv, W, lens in cases:
        say("decode reuse", B, Tq, Tmax, H, Hkv, W)
        q, kc, vc = decode_inputs(B, Tq, Tmax, H, Hkv, lens, seed=60)
        fresh = run_decode(q, kc, vc, lens, W, True)
        again = run_decode(q, kc, vc, lens, W, True, scr=shared)
        assert np.array_equal(fresh[0], again[0]) and np.array_equal(fresh[1], again[1])


# ------------------------------------------------------ FP8 (tensor-wise)
FP8_FMT = {G.FP8_E4M3: "e4m3", G.FP8_E5M2: "e5m2"}


def _fp8_input(rows, cols, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    if spread:   # magnitudes over many binades: exercises subnormals and the top
        x *= np.exp2(rng.integers(-12, 4, (rows, cols))).astype(np.float32)
    return x


def run_fp8_cast(x, dt, fmt, want_q=True, want_t=False):
    rows, cols = x.shape
    tx = dev(x, tdtype(dt))
    q = torch.empty(rows, cols, dtype=torch.uint8, device=DEV) if want_q else None
    qt = torch.empty(cols, rows, dtype=torch.uint8, device=DEV) if want_t else None
    sc = torch.empty(4, dtype=torch.float32, device=DEV)
    scr = torch.empty(G.k_fp8_cast_scratch_bytes(), dtype=torch.uint8, device=DEV)
    G.k_fp8_cast(tx, rows, cols, dt, fmt, q, qt, sc, scr)
    torch.cuda.synchronize()
    return (q.cpu().numpy() if want_q else None, qt.cpu().numpy() if want_t else None,
            sc.cpu().numpy())


@pytest.mark.parametrize("fmt", [G.FP8_E4M3, G.FP8_E5M2])
@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("shape,trans", [((64, 64), True), ((130, 48), False), ((144, 80), True),
                                         ((1008, 768), True), ((1000, 768), False), ((16, 3072), True)])
def test_fp8_cast(shape, trans, dt, fmt):
    """Codes bit-exact against the oracle's cast (same fp32 scale, same fp32
    product, nearest-even rounding); the transposed copy is the transpose;
    s and 1/s exact."""
    from oracle import fp8
    say("fp8 cast", shape, trans, dt, fmt)
    x = _fp8_input(*shape, seed=70 + shape[0])
    if dt == G.BF16:
        x = O.round_bf16(x)
    codes, _, s, inv = fp8.quantize(x, FP8_FMT[fmt])
    q, qt, sc = run_fp8_cast(x, dt, fmt, True, trans)
    assert sc[0] == s and sc[1] == inv
    np.testing.assert_array_equal(q, codes)
    if trans:
        np.testing.assert_array_equal(qt, codes.T)


def test_fp8_cast_zero_and_saturation():
    """An all-zero tensor casts to zero codes with s = 448 / 1e-12; a tensor
    whose amax times s lands above 448 in fp32 keeps its largest element at
    the format's maximum (code 0x7E), never NaN."""
    from oracle import fp8
    z = np.zeros((32, 32), np.float32)
    q, qt, sc = run_fp8_cast(z, G.F32, G.FP8_E4M3, True, True)
    assert np.all(q == 0) and np.all(qt == 0)
    assert sc[0] == np.float32(np.float32(448) / np.float32(1e-12))
    x = _fp8_input(32, 32, 5, spread=False) * 0.1
    x[3, 3] = np.float32(12.5159)
    q, _, _ = run_fp8_cast(x, G.F32, G.FP8_E4M3)
    assert q[3, 3] == 0x7E
    np.testing.assert_array_equal(q, fp8.quantize(x, "e4m3")[0])


def fp8_mm_bound(va, ia, vb, ib):
    """Elementwise error bound of an fp32-output FP8 product: the matrix
    cores form each 128-long block dot product of 8-bit values with about 16
    significant bits before adding it to the fp32 accumulator (measured:
    |error| / sum |a b| <= 2e-5 for one block, falling with K as blocks
    add), so the bound is 2^-13 sum_k |a_k b_k| (1/sa) (1/sb)."""
    mag = np.abs(np.asarray(va, np.float64)) @ np.abs(np.asarray(vb, np.float64)).T
    return 2.0 ** -13 * mag * np.float64(ia) * np.float64(ib)


def _gemm_fp8_case(M, N, K, fa, fb, seed):
    from oracle import fp8
    ca, va, _, ia = fp8.quantize(_fp8_input(M, K, seed, spread=False), FP8_FMT[fa])
    cb, vb, _, ib = fp8.quantize(_fp8_input(N, K, seed + 1, spread=False), FP8_FMT[fb])
    return ca, va, ia, cb, vb, ib


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (300, 200, 384), (512, 768, 768),
                                   (1000, 260, 256), (64, 3072, 1024)])
def test_gemm_fp8(M, N, K, fa, fb):
    """The FP8 product on the oracle's own codes and inverse scales: bf16
    output normwise within 1e-2 of the fp64 product (one bf16 step, 2^-7 of
    an element, when the accumulation error moves a value across a rounding
    boundary), fp32 output (+= onto a random C) elementwise within the
    matrix cores' FP8 accumulation bound."""
    from oracle import fp8
    say("gemm fp8", M, N, K, fa, fb)
    ca, va, ia, cb, vb, ib = _gemm_fp8_case(M, N, K, fa, fb, seed=M + N)
    ref = fp8.scaled_mm(va, ia, vb, ib)
    tA, tB = dev(ca, torch.uint8), dev(cb, torch.uint8)
    tia = torch.tensor([ia], dtype=torch.float32, device=DEV)
    tib = torch.tensor([ib], dtype=torch.float32, device=DEV)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    G.k_gemm_fp8(M, N, K, tA, K, fa, tB, K, fb, tia, tib, out, N, G.EPI_STORE)
    c0 = np.random.default_rng(3).standard_normal((M, N)).astype(np.float32)
    acc = dev(c0, torch.float32)
    G.k_gemm_fp8(M, N, K, tA, K, fa, tB, K, fb, tia, tib, acc, N, G.EPI_F32_ACC)
    torch.cuda.synchronize()
    assert rel_err(to_np(out), ref) < 1e-2
    err = np.abs(to_np(acc) - (ref + c0))
    assert np.all(err <= fp8_mm_bound(va, ia, vb, ib) + 1e-6 * np.abs(ref + c0))


def test_gemm_fp8_split_k_and_strides():
    """fp32 output with the K split over scratch partials (fixed-order sum),
    and operands with leading dimensions above K."""
    from oracle import fp8
    M, N, K, lda, ldb = 256, 192, 8192, 8192 + 64, 8192 + 128
    ca, va, ia, cb, vb, ib = _gemm_fp8_case(M, N, K, 0, 1, seed=11)
    A = np.zeros((M, lda), np.uint8)
    A[:, :K] = ca
    B = np.full((N, ldb), 0x7F, np.uint8)     # NaN codes past K must never be read
    B[:, :K] = cb
    tA, tB = dev(A, torch.uint8), dev(B, torch.uint8)
    tia = torch.tensor([ia], dtype=torch.float32, device=DEV)
    tib = torch.tensor([ib], dtype=torch.float32, device=DEV)
    nb = G.k_gemm_fp8_scratch_bytes(M, N, K)
    assert nb > 0
    scr = torch.empty(nb, dtype=torch.uint8, device=DEV)
    out = torch.empty(M, N, dtype=torch.float32, device=DEV)
    G.k_gemm_fp8(M, N, K, tA, lda, 0, tB, ldb, 1, tia, tib, out, N, G.EPI_F32, scr)
    torch.cuda.synchronize()
    ref = fp8.scaled_mm(va, ia, vb, ib)
    err = np.abs(to_np(out) - ref)
    assert np.all(err <= fp8_mm_bound(va, ia, vb, ib) + 1e-6 * np.abs(ref))


def test_fp8_linear_forward_and_backward_chain():
    """Float8Linear end to end on the GPU (cast kernels feeding the product)
    against the oracle: y = x W^T (e4m3 x e4m3), dX = dY W (e5m2 dY against
    the transposed e4m3 weight copy) and dW = dY^T X (transposed copies of
    both), at a d12 MLP shape."""
    from oracle import fp8
    M, K, N = 2048, 768, 3072           # tokens, in, out
    x = O.round_bf16(_fp8_input(M, K, 1, spread=False))
    w = O.round_bf16(_fp8_input(N, K, 2, spread=False) * 0.02)
    dy = O.round_bf16(_fp8_input(M, N, 3, spread=False) * 1e-3)
    tx, tw, tdy = dev(x, torch.bfloat16), dev(w, torch.bfloat16), dev(dy, torch.bfloat16)
    scr = torch.empty(G.k_fp8_cast_scratch_bytes(), dtype=torch.uint8, device=DEV)

    def cast(t, rows, cols, fmt):
        q = torch.empty(rows, cols, dtype=torch.uint8, device=DEV)
        qt = torch.empty(cols, rows, dtype=torch.uint8, device=DEV)
        sc = torch.empty(2, dtype=torch.float32, device=DEV)
        G.k_fp8_cast(t, rows, cols, G.BF16, fmt, q, qt, sc, scr)
        return q, qt, sc

    qx, qxt, sx = cast(tx, M, K, G.FP8_E4M3)
    qw, qwt, sw = cast(tw, N, K, G.FP8_E4M3)
    qd, qdt, sd = cast(tdy, M, N, G.FP8_E5M2)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    G.k_gemm_fp8(M, N, K, qx, K, 0, qw, K, 0, sx[1:], sw[1:], y, N, G.EPI_STORE)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    G.k_gemm_fp8(M, K, N, qd, N, 1, qwt, N, 0, sd[1:], sw[1:], dx, K, G.EPI_STORE)
    dw = torch.empty(N, K, dtype=torch.float32, device=DEV)
    G.k_gemm_fp8(N, K, M, qdt, M, 1, qxt, M, 0, sd[1:], sx[1:], dw, K, G.EPI_F32)
    torch.cuda.synchronize()
    _, vx, _, ix = fp8.quantize(x, "e4m3")
    _, vw, _, iw = fp8.quantize(w, "e4m3")
    _, vd, _, idy = fp8.quantize(dy, "e5m2")
    assert rel_err(to_np(y), fp8.fp8_linear(x, w)) < 1e-2
    assert rel_err(to_np(dx), fp8.scaled_mm(vd, idy, vw.T, iw)) < 1e-2
    dw_ref = fp8.scaled_mm(vd.T, idy, vx.T, ix)
    assert np.all(np.abs(to_np(dw) - dw_ref) <= fp8_mm_bound(vd.T, idy, vx.T, ix)
                  + 1e-6 * np.abs(dw_ref))
    # and FP8 stays close to the bf16 product it stands in for
    assert rel_err(to_np(y), x.astype(np.float64) @ w.astype(np.float64).T) < 0.1


# ------------------------------------------------------ Muon Newton-Schulz
NS_PAGE = [(8.156, -22.483, 15.879), (4.043, -2.809, 0.500)]
NS_CLASSIC = (3.4445, -4.7750, 2.0315)


@pytest.mark.parametrize("dt", [G.F32, G.BF16])
@pytest.mark.parametrize("m,n,steps,batch", [(64, 32, 2, 1), (32, 96, 2, 3), (768, 768, 5, 2),
                                             (2304, 768, 5, 1), (768, 3072, 5, 2),
                                             (136, 72, 0, 2), (72, 136, 1, 1),
                                             (2304, 768, 5, 12), (768, 3072, 5, 12)])
def test_polar_express(m, n, steps, batch, dt):
    """The orthogonalized updates of a batch of matrices against the
    oracle's bf16 Gram-matrix form and against the exact result (the SVD
    definition), each matrix on its own.  The batches of 12 d12 matrices
    run the polynomial products on the direct-to-LDS kernel, whose grid
    numbers (matrix, tile) pairs per XCD.  Tuples: the
    page's two, or the classic quintic tuple five times (a convergent
    schedule: the page's two tuples expect the three elided ones after
    them)."""
    from oracle import muon
    say("polar express", m, n, steps, batch, dt)
    coeffs = NS_PAGE[:steps] if steps <= 2 else [NS_CLASSIC] * steps
    g = np.random.default_rng(m * 7 + n).standard_normal((batch, m, n)).astype(np.float32)
    g[-1] *= 40.0                       # matrices of different norms share the launches
    if dt == G.BF16:
        g = O.round_bf16(g)
    tg = dev(g, tdtype(dt))
    x = torch.empty(batch, m, n, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(G.k_polar_express_ws_bytes(m, n, batch), dtype=torch.uint8, device=DEV)
    G.k_polar_express(tg, m, n, dt, coeffs, muon.NS_EPS, x, ws, batch=batch)
    torch.cuda.synchronize()
    for i in range(batch):
        got = to_np(x[i])
        ref_b = muon.polar_express(g[i], coeffs, bf16=True)
        ref = muon.polar_express(g[i], coeffs)
        say("  err vs bf16 oracle", rel_err(got, ref_b), "vs exact", rel_err(got, ref))
        # against the exact iteration: the 2e-2 bar of bf16 results; against
        # the bf16 emulation, whose own roundings are independent of the
        # kernels', the sum of both deviations
        assert rel_err(got, ref) < 2e-2
        assert rel_err(got, ref_b) < 3e-2
        if steps == 0:   # the normalised start only: one bf16 rounding
            assert rel_err(got, ref) < 4e-3


# ------------------------------------------------------ optimizer step
@pytest.mark.parametrize("n", [4096, 1_000_004])
def test_optimizer_elementwise(n):
    """Muon momentum (Nesterov and plain), the Muon parameter step and AdamW
    against the oracle over three steps (fp32 arithmetic against fp64:
    1e-5 relative), bf16 copies equal to the rounded fp32 weights."""
    from oracle import muon
    say("optim", n)
    rng = np.random.default_rng(n % 97)
    w0 = rng.standard_normal(n).astype(np.float32)
    grads = [rng.standard_normal(n).astype(np.float32) for _ in range(3)]
    xs = [O.round_bf16(rng.standard_normal(n).astype(np.float32) * 0.02) for _ in range(3)]
    tw = dev(w0, torch.float32)
    tw16 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    tmom = torch.zeros(n, dtype=torch.float32, device=DEV)
    tu = torch.empty(n, dtype=torch.float32, device=DEV)
    tu16 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    aw, am, av = dev(w0, torch.float32), torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    w, mom = w0.astype(np.float64), np.zeros(n)
    a_w, a_m, a_v = w0.astype(np.float64), np.zeros(n), np.zeros(n)
    hp = dict(lr=3e-3, beta1=0.8, beta2=0.95, eps=1e-10, wd=0.01)
    for k in range(3):
        tg = dev(grads[k], torch.float32)
        G.k_muon_momentum(tg, tmom, tu, n, 0.95, True, G.F32)
        mom, u = muon.muon_momentum(grads[k], mom, 0.95)
        torch.cuda.synchronize()
        assert rel_err(to_np(tu), u) < 1e-6
        # the plain form on a copy of the updated momentum M gives beta M +
        # (1 - beta) G: the Nesterov value above, here rounded to bf16
        G.k_muon_momentum(tg, tmom.clone(), tu16, n, 0.95, False, G.BF16)
        G.k_muon_update(tw, dev(xs[k], torch.bfloat16), n, 0.02, 0.1, tw16)
        w = muon.muon_update(w, xs[k], 0.02, 0.1)
        G.k_adamw(aw, tg, am, av, n, k + 1, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                  hp["wd"])
        a_w, a_m, a_v = muon.adamw(a_w, grads[k], a_m, a_v, k + 1, **hp)
        torch.cuda.synchronize()
        assert rel_err(to_np(tu16), O.round_bf16(u.astype(np.float32))) < 8e-3
        assert rel_err(to_np(tw), w) < 1e-5
        np.testing.assert_array_equal(to_np(tw16), O.round_bf16(tw.cpu().numpy()))
        assert rel_err(to_np(aw), a_w) < 1e-5
        assert rel_err(to_np(am), a_m) < 1e-5 and rel_err(to_np(av), a_v) < 1e-5
        assert rel_err(to_np(tmom), mom) < 1e-6


@pytest.mark.parametrize("rows,cols", [(768, 768), (3072, 768), (40, 3072), (5, 8)])
def test_normuon_update(rows, cols):
    """NorMuon's step on one matrix, three steps from a zero second moment,
    against the oracle (fp32 kernels against fp64: 1e-5 relative on the
    weights' change and on the state); rows of very different scales so
    the per-row normalisation matters; the bf16 copy is the rounded
    master."""
    from oracle import muon
    say("normuon", rows, cols)
    rng = np.random.default_rng(rows + cols)
    # weights small enough that their fp32 rounding stays well under the
    # bar relative to the step's change
    w0 = (0.01 * rng.standard_normal((rows, cols))).astype(np.float32)
    tw = dev(w0, torch.float32)
    tw16 = torch.empty(rows * cols, dtype=torch.bfloat16, device=DEV)
    tv = torch.zeros(rows, dtype=torch.float32, device=DEV)
    scr = torch.empty(G.k_normuon_scratch_bytes(rows), dtype=torch.uint8, device=DEV)
    w, v = w0.astype(np.float64), np.zeros(rows)
    for k in range(3):
        x = O.round_bf16((rng.standard_normal((rows, cols)) *
                          np.geomspace(0.05, 2.0, rows)[:, None] * 0.03).astype(np.float32))
        G.k_normuon_update(tw, dev(x, torch.bfloat16), tv, rows, cols, 0.9, 0.02, 0.1, scr,
                           w_bf16=tw16)
        xs, v = muon.normuon(x, v, 0.9)
        w = muon.muon_update(w, xs, 0.02, 0.1)
        torch.cuda.synchronize()
        got = to_np(tw).reshape(rows, cols)
        assert rel_err(got - w0, w - w0) < 1e-5
        assert rel_err(to_np(tv), v) < 1e-5
        np.testing.assert_array_equal(to_np(tw16), O.round_bf16(tw.cpu().numpy()).reshape(-1))


# ------------------------------------------------------ model extras
@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("lams", [(0.9, 0.3), (1.0, -0.45)])   # mixing; backout
def test_resid_mix(lams, dt):
    """Residual mixing y = lr x + l0 x0 (and backout as lr = 1, l0 = -lambda)
    with its backward (dx, dx0 accumulated onto a running value, the two
    scalar gradients) against the oracle."""
    from oracle import extras as X
    say("resid mix", lams, dt)
    bf = dt == G.BF16
    N, D = 4096 + 16, 768
    x, x0, dy, acc0 = (rnd_in((N, D), 90 + i, 1.0, bf) for i in range(4))
    lam = np.array(lams, np.float32)
    if bf:
        lam = O.round_bf16(lam)
    lr, l0 = float(lam[0]), float(lam[1])
    tl = dev(lam, tdtype(dt))
    tx, tx0, tdy = dev(x, tdtype(dt)), dev(x0, tdtype(dt)), dev(dy, tdtype(dt))
    y = torch.empty_like(tx)
    G.k_resid_mix_fwd(tx, tx0, y, N * D, tl, dt)
    dx = torch.empty_like(tx)
    dx0 = dev(acc0, tdtype(dt))
    dl = torch.empty(2, dtype=torch.float32, device=DEV)
    scr = torch.empty(G.lib().gpt_k_resid_mix_bwd_scratch_bytes(), dtype=torch.uint8, device=DEV)
    G.k_resid_mix_bwd(tdy, tx, tx0, dx, dx0, True, N * D, tl, dl, scr, dt)
    torch.cuda.synchronize()
    tol = 1e-2 if bf else 1e-6
    assert rel_err(to_np(y), X.resid_mix(x, x0, lr, l0)) < tol
    rdx, rdx0, rlr, rl0 = X.resid_mix_bwd(dy, x, x0, lr, l0)
    assert rel_err(to_np(dx), rdx) < tol
    assert rel_err(to_np(dx0), rdx0 + acc0) < tol
    np.testing.assert_allclose(to_np(dl), [rlr, rl0], rtol=1e-4)


@pytest.mark.parametrize("dt", [G.BF16, G.F32])
@pytest.mark.parametrize("B,T,D", [(2, 64, 768), (3, 5, 24), (1, 1, 256)])
def test_smear(B, T, D, dt):
    """Smear forward (y, the saved gates) and backward (dx, dw, dlambda)
    against the oracle; a row of one token is never mixed."""
    from oracle import extras as X
    say("smear", B, T, D, dt)
    bf = dt == G.BF16
    N = B * T
    x, dy = rnd_in((N, D), 95, 1.0, bf), rnd_in((N, D), 96, 1.0, bf)
    w = rnd_in((24,), 97, 0.3, bf)
    lam = np.array([0.7], np.float32)
    if bf:
        lam = O.round_bf16(lam)
    lv = float(lam[0])
    tx, tdy = dev(x, tdtype(dt)), dev(dy, tdtype(dt))
    tw, tl = dev(w, tdtype(dt)), dev(lam, tdtype(dt))
    y = torch.empty_like(tx)
    gate = torch.empty(N, dtype=torch.float32, device=DEV)
    G.k_smear_fwd(tx, B, T, D, tw, tl, y, gate, dt)
    dx = torch.empty_like(tx)
    dwl = torch.empty(25, dtype=torch.float32, device=DEV)
    scr = torch.empty(G.lib().gpt_k_smear_bwd_scratch_bytes(), dtype=torch.uint8, device=DEV)
    G.k_smear_bwd(tdy, tx, B, T, D, tw, tl, gate, dx, dwl, scr, dt)
    torch.cuda.synchronize()
    ry, rg = X.smear(x, w, lv, T)
    rdx, rdw, rdl = X.smear_bwd(dy, x, w, lv, T)
    tol = 1e-2 if bf else 1e-5
    assert rel_err(to_np(y), ry) < tol
    np.testing.assert_allclose(to_np(gate), rg, rtol=1e-5, atol=1e-6)
    assert rel_err(to_np(dx), rdx) < tol
    got = to_np(dwl)
    if T > 1:
        assert rel_err(got[:24], rdw) < 1e-4
        assert got[24] == pytest.approx(rdl, rel=1e-4)
    else:
        assert np.all(got == 0.0)


# ------------------------------------------------------ whole optimizer step
@pytest.mark.parametrize("which,normuon", [("small_bf16", False), ("tiny", False),
                                           ("small_bf16_extras", False), ("small_bf16", True),
                                           ("tiny", True)])
def test_optim_step(which, normuon):
    """gpt_optim_step over every tensor of a model, two steps, against the
    oracle's Muon (momentum, exact Newton-Schulz, NorMuon's per-row
    rescaling when on, lr max(1, rows/cols)^0.5 step) and AdamW per tensor:
    Muon tensors' changes within 2e-2 normwise (the kernels' bf16
    iteration), AdamW tensors to 1e-5; the bf16 copy is the rounded
    master."""
    from oracle import muon
    from tests.gpu_util import small_bf16, tiny_plus
    import gptinputs as gi
    cfgd = {"small_bf16": small_bf16, "tiny": tiny_plus,
            "small_bf16_extras": lambda: small_bf16(resid_lambdas=1, smear=1,
                                                    backout_layer=1)}[which]()
    say("optim step", which, "normuon", normuon)
    cfg = G.make_config(cfgd)
    n = O.param_count(cfgd)
    rng = np.random.default_rng(21)
    w0 = (rng.standard_normal(n) * 0.05).astype(np.float32)
    grads = [rng.standard_normal(n).astype(np.float32) * 1e-2 for _ in range(2)]
    coeffs = [NS_CLASSIC] * 5
    hpd = dict(muon_lr=0.02, muon_momentum=0.9, muon_wd=0.01, adam_lr_embed=0.05,
               adam_lr_head=0.004, adam_lr_gate=0.01, beta1=0.8, beta2=0.95, eps=1e-10,
               adam_wd=0.001)
    hp = G.make_optim_hparams(coeffs, normuon=normuon, normuon_beta2=0.9, **hpd)
    master = dev(w0, torch.float32)
    bf = cfgd["dtype"] == G.BF16
    params = torch.empty(n, dtype=torch.bfloat16, device=DEV) if bf else None
    s1, s2 = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    ws = torch.empty(G.optim_ws_bytes(cfg), dtype=torch.uint8, device=DEV)
    for k in range(2):
        G.optim_step(cfg, hp, k + 1, master, params, dev(grads[k], torch.float32), s1, s2, ws)
    torch.cuda.synchronize()
    got = to_np(master)
    # oracle, tensor by tensor
    off = 0
    ref = w0.astype(np.float64).copy()
    for name, shape in O.param_layout(cfgd):
        size = int(np.prod(shape))
        sl = slice(off, off + size)
        base = name.split(".")[-1]
        w = w0[sl].astype(np.float64).reshape(shape)
        if base in ("wqkv", "wo", "wfc", "wproj"):
            mom, vrow = np.zeros(shape), np.zeros(shape[0])
            lr = hpd["muon_lr"] * max(1.0, shape[0] / shape[1]) ** 0.5
            for k in range(2):
                mom, u = muon.muon_momentum(grads[k][sl].reshape(shape), mom, 0.9)
                x = muon.polar_express(u, coeffs)
                if normuon:
                    x, vrow = muon.normuon(x, vrow, 0.9)
                w = muon.muon_update(w, x, lr, hpd["muon_wd"])
            d_ref, d_got = w - w0[sl].reshape(shape), got[sl].reshape(shape) - w0[sl].reshape(shape)
            # NorMuon rescales each row by the bf16 iterate's own row
            # statistics, which carry the iteration's error once more: the
            # bar of the orthogonalization against its bf16 emulation
            assert rel_err(d_got, d_ref) < (3e-2 if normuon else 2e-2), name
        else:
            lr = {"wte": hpd["adam_lr_embed"], "ve": hpd["adam_lr_embed"],
                  "wlm": hpd["adam_lr_head"], "wg": hpd["adam_lr_gate"],
                  "extras": hpd["adam_lr_gate"]}[base]
            m = v = np.zeros(shape)
            for k in range(2):
                w, m, v = muon.adamw(w, grads[k][sl].reshape(shape), m, v, k + 1, lr,
                                     hpd["beta1"], hpd["beta2"], hpd["eps"], hpd["adam_wd"])
            assert rel_err(got[sl], w.reshape(-1)) < 1e-5, name
        off += size
    assert off == n
    if bf:
        np.testing.assert_array_equal(to_np(params), O.round_bf16(got.astype(np.float32)))


@pytest.mark.parametrize("normuon", [False, True])
def test_optim_step_streams_bitwise(normuon):
    """The Muon groups on the library's side streams (the default for bf16)
    leave masters, bf16 copies and both states bit for bit as on one
    stream: each group's kernels and inputs are the same, only the overlap
    differs.  Three steps, so the second and third read the states the
    concurrent groups wrote."""
    from tests.gpu_util import small_bf16
    cfgd = small_bf16(resid_lambdas=1, smear=1, backout_layer=1)
    say("optim streams", "normuon", normuon)
    n = O.param_count(cfgd)
    rng = np.random.default_rng(23)
    w0 = (rng.standard_normal(n) * 0.05).astype(np.float32)
    grads = [dev(rng.standard_normal(n).astype(np.float32) * 1e-2, torch.float32)
             for _ in range(3)]
    hp = G.make_optim_hparams([NS_CLASSIC] * 5, normuon=normuon, normuon_beta2=0.9)
    out = []
    for one in (0, 1):
        cfg = G.make_config(dict(cfgd, one_stream=one))
        master = dev(w0, torch.float32)
        params = torch.empty(n, dtype=torch.bfloat16, device=DEV)
        s1, s2 = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
        ws = torch.empty(G.optim_ws_bytes(cfg), dtype=torch.uint8, device=DEV)
        for k in range(3):
            G.optim_step(cfg, hp, k + 1, master, params, grads[k], s1, s2, ws)
        torch.cuda.synchronize()
        out.append([to_np(t) for t in (master, params.float(), s1, s2)])
    for a, b in zip(*out):
        np.testing.assert_array_equal(a, b)
