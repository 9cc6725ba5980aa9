"""Pins for the oracle of the KV append with RoPE (``oracle.append``).

Each test checks the oracle against something other than itself: correctly
rounded casts of numpy (float64 -> float16) and torch (float32 -> bfloat16 /
float8_e4m3fn), tie cases the formats' definitions fix, the defining
properties of a rotary embedding (position 0 is the identity, rotations keep
lengths, scores depend only on the distance between positions), the complex-
number form of the same rotation, and brute-force bookkeeping of which cache
slots an append writes. The functions are looked up at call time so
``test_oracle_mutants.py`` can swap them.
"""

import math

import numpy as np
import pytest
import torch

import oracle.append as AP
from oracle.fp8 import e4m3_value
from workloads import make_workload
from workloads.synth import to_paged


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ rounding


def test_round_to_f16_matches_numpy_float64_cast():
    r = _rng(1)
    x = np.concatenate([r.standard_normal(4000) * 10.0 ** r.integers(-9, 5, 4000),
                        r.standard_normal(200) * 1e-6, [0.0, -0.0, 65504.0, 65519.0, 65520.0, -7e5]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    got = AP.round_to_format(x, "f16")
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_round_to_bf16_and_e4m3_match_torch_float32_casts():
    r = _rng(2)
    x32 = (r.standard_normal(5000) * 10.0 ** r.integers(-12, 3, 5000)).astype(np.float32)
    t = torch.from_numpy(x32)
    assert np.array_equal(AP.round_to_format(x32.astype(np.float64), "bf16"),
                          t.to(torch.bfloat16).to(torch.float64).numpy())
    # torch's E4M3 cast turns values that round past 448 into NaN; compare in range
    small = x32[np.abs(x32) < 464]
    ts = torch.from_numpy(small)
    assert np.array_equal(AP.round_to_format(small.astype(np.float64), "e4m3", saturate=True),
                          ts.to(torch.float8_e4m3fn).to(torch.float64).numpy())


def test_rounding_ties_and_saturation_closed_forms():
    f = AP.round_to_format
    # ties go to the even mantissa
    assert f(1 + 2 ** -11, "f16") == 1.0 and f(1 + 3 * 2 ** -11, "f16") == 1 + 2 ** -9
    assert f(2 ** -25, "f16") == 0.0 and f(3 * 2 ** -25, "f16") == 2 ** -23          # subnormal ties
    assert f(1 + 2 ** -8, "bf16") == 1.0 and f(1 + 3 * 2 ** -8, "bf16") == 1 + 2 ** -6
    assert f(2 ** -10, "e4m3") == 0.0 and f(3 * 2 ** -10, "e4m3") == 2 ** -8
    assert f(1 + 2 ** -4, "e4m3") == 1.0 and f(1 + 3 * 2 ** -4, "e4m3") == 1.25
    # overflow
    assert f(65520.0, "f16") == math.inf and f(-70000.0, "f16") == -math.inf
    assert f(500.0, "e4m3", saturate=True) == 448.0 and f(-1e9, "e4m3", saturate=True) == -448.0
    assert f(460.0, "e4m3", saturate=True) == 448.0


def test_e4m3_code_inverts_the_decoder():
    for c in range(256):
        v = e4m3_value(c)
        if not math.isnan(v):
            assert AP.e4m3_code(v) == c


# ---------------------------------------------------------------------- RoPE


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_rope_position_zero_is_identity_and_rotations_keep_lengths(style):
    r = _rng(3)
    x = r.standard_normal((5, 64))
    assert np.array_equal(AP.rope_rotate(x, 0, 10000.0, style), x)
    y = AP.rope_rotate(x, 12345, 10000.0, style)
    a, b = AP.rope_pairs(64, style)
    assert np.allclose(x[:, a] ** 2 + x[:, b] ** 2, y[:, a] ** 2 + y[:, b] ** 2, rtol=1e-13)


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_rope_scores_depend_only_on_the_distance(style):
    """<R(m) q, R(n) k> = <R(m - n) q, k>: the property rotary embeddings are built for."""
    r = _rng(4)
    q, k = r.standard_normal(128), r.standard_normal(128)
    for m, n in [(5, 3), (1000, 17), (131071, 131000), (40, 90)]:
        lhs = AP.rope_rotate(q, m, 500000.0, style) @ AP.rope_rotate(k, n, 500000.0, style)
        rhs = AP.rope_rotate(q, m - n, 500000.0, style) @ k
        assert abs(lhs - rhs) < 1e-9 * np.linalg.norm(q) * np.linalg.norm(k)


def test_rope_interleaved_is_complex_multiplication_and_half_is_a_permutation():
    """Pairs as complex numbers x_2i + i x_2i+1 multiplied by exp(i pos base^(-2i/d));
    the half pairing is the same rotation with dimensions (i, i + d/2) gathered."""
    r = _rng(5)
    d, pos, base = 128, 7777, 10000.0
    x = r.standard_normal(d)
    z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * pos * base ** (-np.arange(d // 2) * 2.0 / d))
    y = AP.rope_rotate(x, pos, base, "interleaved")
    assert np.allclose(y[0::2], z.real, rtol=0, atol=1e-12) and np.allclose(y[1::2], z.imag, rtol=0, atol=1e-12)
    perm = np.empty(d, dtype=int)
    perm[0::2], perm[1::2] = np.arange(d // 2), np.arange(d // 2) + d // 2
    yh = AP.rope_rotate(x[np.argsort(perm)], pos, base, "half")     # half layout of the same pairs
    assert np.allclose(yh[perm], y, rtol=0, atol=1e-12)
    # the first pair turns by exactly pos radians, the last by pos * base^(-(d-2)/d)
    ang = AP.rope_angles(pos, d, base)
    assert ang[0] == pos and abs(ang[-1] - pos * base ** (-(d - 2) / d)) < 1e-12 * pos


# -------------------------------------------------------------------- append


def _paged(dtype=torch.float16, lens=(17, 32, 5), hq=4, hkv=2, d=64, seed=9):
    wl = make_workload(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seq_lens=list(lens),
                       dtype=dtype, seed=seed)
    return to_paged(wl, 16, spare_pages=3)


@pytest.mark.parametrize("n", [1, 3])
def test_append_writes_only_the_new_tokens_slots(n):
    """New token j of sequence b lands at position L_b - n + j: the block-table
    entry (L_b - n + j) // 16, slot (L_b - n + j) % 16. Nothing else changes."""
    wl = _paged()
    B, hkv, d = wl.batch, wl.num_kv_heads, wl.head_dim
    g = torch.Generator().manual_seed(3)
    kn = torch.randn(B, n, hkv, d, generator=g).to(torch.float16)
    vn = torch.randn(B, n, hkv, d, generator=g).to(torch.float16)
    kc, vc, _ = AP.append_kv(wl.k, wl.v, wl.block_table, wl.seq_lens, kn, vn, rope_style=None)
    expect = set()
    for b, L in enumerate(wl.lens):
        for j in range(n):
            pos = L - n + j
            expect.add((int(wl.block_table[b, pos // 16]), pos % 16))
            assert torch.equal(vc[int(wl.block_table[b, pos // 16]), pos % 16], vn[b, j])
            assert torch.equal(kc[int(wl.block_table[b, pos // 16]), pos % 16], kn[b, j])
    changed = set()
    for p in range(wl.k.shape[0]):
        for s in range(16):
            same = torch.equal(kc[p, s].view(torch.int16), wl.k[p, s].view(torch.int16)) and \
                torch.equal(vc[p, s].view(torch.int16), wl.v[p, s].view(torch.int16))
            if not same:
                changed.add((p, s))
    assert changed <= expect and len(expect) == B * n


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float8_e4m3fn])
def test_append_rotates_keys_and_queries_and_rounds_once(dtype):
    """Keys and queries at their positions, rotated (checked against the
    complex form) and rounded once to the storage format (checked against
    numpy / torch casts of the exact rotation)."""
    wl = _paged(torch.bfloat16 if dtype == torch.bfloat16 else torch.float16)
    B, hkv, hq, d, n = wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim, 2
    g = torch.Generator().manual_seed(4)
    qdt = wl.dtype
    kn = torch.randn(B, n, hkv, d, generator=g).to(qdt)
    vn = torch.randn(B, n, hkv, d, generator=g).to(qdt)
    q = torch.randn(B, n, hq, d, generator=g).to(qdt)
    kc0, vc0 = wl.k, wl.v
    ks = vs = None
    if dtype == torch.float8_e4m3fn:
        kc0, vc0 = wl.k.to(dtype), wl.v.to(dtype)
        ks, vs = torch.tensor([0.01, 0.02]), torch.tensor([0.004, 0.5])
    kc, vc, qr = AP.append_kv(kc0, vc0, wl.block_table, wl.seq_lens, kn, vn, q, rope_style="half",
                              rope_base=10000.0, k_scale=ks, v_scale=vs)
    base = 10000.0
    for b, L in enumerate(wl.lens):
        for j in range(n):
            pos = L - n + j
            page, slot = int(wl.block_table[b, pos // 16]), pos % 16
            ang = pos * base ** (-np.arange(d // 2) * 2.0 / d)
            rot = np.exp(1j * ang)

            def rotate(x):
                x = x.double().numpy()
                z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * rot
                return np.concatenate([z.real, z.imag], axis=-1)

            kx = rotate(kn[b, j])
            qx = rotate(q[b, j])
            if dtype == torch.float8_e4m3fn:
                kx32 = kx / ks.double().numpy()[:, None]
                ok = np.abs(kx32) < 448
                ref = torch.from_numpy(kx32.astype(np.float32)).to(dtype).to(torch.float64).numpy()
                got = kc[page, slot].to(torch.float64).numpy()
                # torch rounds a float32 rounding of the value; only where that cannot matter
                close = np.abs(got - kx32) <= np.abs(ref - kx32) + 1e-12
                assert close[ok].all()
            else:
                ref = torch.from_numpy(kx).to(dtype) if dtype == torch.float16 else None
                got = kc[page, slot].double().numpy()
                if dtype == torch.float16:
                    assert np.array_equal(got, kx.astype(np.float16).astype(np.float64))
                else:
                    assert np.max(np.abs(got - kx) / np.maximum(np.abs(kx), 1e-30)) <= 2 ** -8
            assert np.allclose(qr[b, j].double().numpy(), qx, rtol=2 ** -7, atol=1e-6)
    assert qr.dtype == q.dtype


def test_append_rejects_a_short_sequence():
    wl = _paged(lens=(1, 20))
    kn = torch.zeros(2, 2, 2, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        AP.append_kv(wl.k, wl.v, wl.block_table, wl.seq_lens, kn, kn)
