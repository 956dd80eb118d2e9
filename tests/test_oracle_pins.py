"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a worked example printed on a source page
(tests/golden), a closed form, an invariant, a library routine that computes a special case, or
brute force over a tiny input.  Sources cited by key:
  [KUNLUN] "Gemma 4 模型架构解析" (vLLM-Kunlun Gemma 4 adaptation guide)
  [MNN]    "MNN 支持 Gemma4 全系列：PLE、KV共享与多模态"
  [INFLM]  "Feat/add gemma3 model" (InfiniLM pull request 581)
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, FP32
from layout import logical_k, page_rows, put_k_rows, unit_elems

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BS = 16


# ------------------------------------------------------------------ helpers (test-side) ---

def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """torch's own fp32 -> bf16 conversion (round to nearest even), as bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_paged(K, V, seed, spare=3):
    """Scatter contiguous per-sequence K[b] [Hkv,L_b,D] / V[b] into the documented page layout.

    Written independently of the oracle with numpy fancy indexing: K pages in the 16-byte unit
    layout (tests/layout.py, fp32 units of 4), V pages [blk][g][d][off].  Returns (k_cache,
    v_cache, block_table) as float32 arrays."""
    rng = np.random.default_rng(seed)
    Hkv, _, D = K[0].shape
    need = [-(-k.shape[1] // BS) for k in K]
    nb = sum(need) + spare
    perm = rng.permutation(nb)
    bt = np.zeros((len(K), max(need)), np.int32)
    kc = np.full((nb, Hkv, BS, D), np.nan, np.float32)
    vc = np.full((nb, Hkv, D, BS), np.nan, np.float32)
    pos = 0
    for b, (k, v) in enumerate(zip(K, V)):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        bt[b, need[b]:] = perm[-1]
        pos += need[b]
        L = k.shape[1]
        j = np.arange(L)
        blk = bt[b, j // BS]
        off = j % BS
        for g in range(Hkv):
            put_k_rows(kc, blk, g, j, k[g], unit_elems("fp32"))
            vc[blk, g, :, off] = v[g]
    return kc, vc, bt


def visible(past, n, W, L):
    """[INFLM] Gemma-3 §3, by brute force.  Query i of a chunk of n new tokens appended after
    `past` cached ones sees key j when j is not later than its own position (the causal limit
    aligned to the end of the L keys: j < L - n + i + 1) and, on a sliding layer, when its
    distance past + i - j is below W.  W = 0: no band."""
    m = np.zeros((n, L), bool)
    for i in range(n):
        for j in range(L):
            causal_ok = j < (L - n + i + 1)
            band_ok = (W == 0) or not (past + i - j >= W)
            m[i, j] = causal_ok and band_ok
    return m


def run_attn(kc, vc, bt, q, cu, cl, Hkv, window=0, scale=1.0, cap=0.0, k_eq_v=0, rows=None):
    Hq, D = q.shape[1], q.shape[2]
    return oracle.attention(FP32, Hq, Hkv, D, window, scale, cap, k_eq_v,
                            np.ascontiguousarray(q, np.float32), cu, kc, vc, bt, cl, rows=rows)


# ------------------------------------------------------------------ number format ---------

def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, 1e-40, -1e-42])]).astype(np.float32)
    ours = np.array([oracle.double_to_bf16(float(v)) for v in x], np.uint16)
    np.testing.assert_array_equal(ours, bf16_bits_from_f32(x))


@pytest.mark.parametrize("x,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),                 # tie between 1 and 1+2^-7: even (1.0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie between 1+2^-7 and 1+2^-6: even
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie: up (a float32 detour ties)
    (1.0 + 2.0 ** -8 - 2.0 ** -30, 0x3F80),    # just below the tie: down
    (2.0 ** -140, 0x0000),                     # below half the smallest subnormal
    (3 * 2.0 ** -134, 0x0002),                 # 1.5 subnormal quanta: tie to even (2)
    (2.0 ** 128 - 2.0 ** 118, 0x7F80),         # rounds past the largest finite: +inf
    (-(2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100), 0xFF7F),  # just below the overflow tie: largest
    (2.0 ** 128 - 2.0 ** 119, 0x7F80),         # the overflow tie itself: +inf
])
def test_bf16_rounding_ties_and_edges(x, bits):
    assert oracle.double_to_bf16(x) == bits


def test_bf16_nan_and_roundtrip():
    assert math.isnan(oracle.bf16_to_double(oracle.double_to_bf16(float("nan"))))
    for h in (0x3F80, 0xC2C8, 0x0001, 0x7F7F, 0x8000):
        assert oracle.double_to_bf16(oracle.bf16_to_double(h)) == h


# ------------------------------------------------------------------ paging ----------------

def test_slot_worked_example_from_the_page():
    """[KUNLUN] §6.3 prints: block_size 64, position 130 -> block_table[row][2], offset 2."""
    ex = json.load(open(os.path.join(GOLDEN, "slot_example.json")))
    bt = np.array([ex["table_row"]], np.int32)
    s, blk, off = oracle.slot(bt, 0, ex["token_position"], ex["block_size"])
    assert blk == ex["table_row"][ex["expected_table_column"]] == ex["expected_block_id"]
    assert off == ex["expected_offset"]
    assert s == ex["expected_slot"] == blk * ex["block_size"] + off


def test_slots_of_a_sequence_are_a_bijection_onto_its_pages():
    rng = np.random.default_rng(1)
    bt = rng.permutation(40).astype(np.int32).reshape(2, 20)
    for row in range(2):
        slots = [oracle.slot(bt, row, p, 16)[0] for p in range(20 * 16)]
        expect = sorted(int(b) * 16 + o for b in bt[row] for o in range(16))
        assert sorted(slots) == expect


def test_ring_slot_worked_example():
    """A ring row of 5 entries: logical page p sits in entry p mod 5, so position t and
    t + 80 share a slot.  Expected values worked by hand from slot = id * 16 + t % 16."""
    bt = np.array([[7, 3, 9, 1, 4]], np.int32)
    for pos, blk_id, off in ((0, 7, 0), (79, 4, 15), (83, 7, 3), (115, 9, 3), (1000, 9, 8)):
        s, blk, o = oracle.slot(bt, 0, pos, 16, page_ring=True)
        assert (blk, o, s) == (blk_id, off, blk_id * 16 + off), pos
    # any 5 consecutive pages occupy 5 distinct entries; the plain table reads column p
    for p0 in range(0, 40):
        assert sorted(oracle.slot(bt, 0, 16 * p, 16, True)[1] for p in range(p0, p0 + 5)) == \
            sorted(bt[0].tolist())
    assert oracle.slot(bt, 0, 70, 16)[1] == 4


def _serve_chunks(ring, W, lens, chunk, rng, Hq=4, Hkv=2, D=16):
    """Write every sequence chunk by chunk (oracle write) and attend each chunk right after its
    write (oracle attention), once through a plain table and once through a ring table of
    `ring` entries per sequence.  Returns the two lists of chunk outputs."""
    B = len(lens)
    pages = [-(-L // BS) for L in lens]
    plain_bt = np.arange(sum(pages) + 0, dtype=np.int32)
    bt_full = np.zeros((B, max(pages)), np.int32)
    at = 0
    for b in range(B):
        bt_full[b, :pages[b]] = plain_bt[at:at + pages[b]]
        at += pages[b]
    bt_ring = rng.permutation(B * ring).astype(np.int32).reshape(B, ring)
    caches = {}
    for name, bt, nb in (("full", bt_full, sum(pages)), ("ring", bt_ring, B * ring)):
        caches[name] = (np.full((nb, Hkv, BS, D), np.nan, np.float32),
                        np.full((nb, Hkv, D, BS), np.nan, np.float32), bt)
    outs = {"full": [], "ring": []}
    done = np.zeros(B, np.int64)
    while (done < lens).any():
        n = np.minimum(np.asarray(lens) - done, chunk).astype(np.int32)
        cl = (done + n).astype(np.int32)
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        T = int(cu[-1])
        k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        q = rng.standard_normal((T, Hq, D)).astype(np.float32)
        for name in ("full", "ring"):
            kc, vc, bt = caches[name]
            oracle.kv_cache_write(FP32, Hq, Hkv, D, 1e4, 1e-6, 0, None, k, v, None, None, None,
                                  cu, cl, bt, kc, vc, page_ring=(name == "ring"))
            outs[name].append(oracle.attention(FP32, Hq, Hkv, D, W, 1.0, 0.0, 0, q, cu, kc, vc,
                                               bt, cl, page_ring=(name == "ring")))
        done += n
    return outs["full"], outs["ring"]


def test_ring_table_serves_the_window_exactly_like_a_plain_table():
    """[INFLM] Gemma-3 §3 / follow-up 2: a sliding layer's chunk needs only keys from its first
    query's window start on.  A ring of floor((n + W - 2) / 16) + 3 pages (the bound the
    library enforces for prefill chunks of n) keeps all of them through every chunk's write,
    so each chunk's attention equals the plain table's bit for bit; a ring of ceil(W / 16)
    pages does not."""
    rng = np.random.default_rng(60)
    W, chunk, lens = 37, 20, [300, 45, 145]
    ring = (chunk + W - 2) // BS + 3
    full, ring_out = _serve_chunks(ring, W, lens, chunk, rng)
    assert len(full) == 15
    for a, b in zip(full, ring_out):
        np.testing.assert_array_equal(a, b)
    full, small = _serve_chunks(-(-W // BS), W, lens, chunk, np.random.default_rng(60))
    assert any(not np.array_equal(a, b) for a, b in zip(full, small))


# ------------------------------------------------------------------ RMSNorm ---------------

def test_rms_norm_matches_torch_library_routine():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(256) * 3.0
    w = (1 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    ours = oracle.rms_norm(x, w, 1e-6)
    lib = torch.nn.functional.rms_norm(torch.from_numpy(x), (256,),
                                       torch.from_numpy(w.astype(np.float64)), eps=1e-6).numpy()
    np.testing.assert_allclose(ours, lib, rtol=1e-13, atol=0)


def test_rms_norm_closed_forms():
    x = np.array([3.0, 4.0])
    # unit weights, eps 0: x / sqrt((9 + 16) / 2)
    np.testing.assert_allclose(oracle.rms_norm(x, np.ones(2, np.float32), 0.0),
                               x / math.sqrt(12.5), rtol=1e-15)
    rng = np.random.default_rng(3)
    y = rng.standard_normal(512)
    ms = float(np.mean(y * y))
    out = oracle.rms_norm(y, np.ones(512, np.float32), 1e-6)
    assert abs(np.mean(out * out) - ms / (ms + 1e-6)) < 1e-12
    # scale invariance with eps = 0, identity without a weight
    np.testing.assert_allclose(oracle.rms_norm(7.5 * y, np.ones(512, np.float32), 0.0),
                               oracle.rms_norm(y, np.ones(512, np.float32), 0.0), rtol=1e-13)
    np.testing.assert_array_equal(oracle.rms_norm(y, None, 1e-6), y)


# ------------------------------------------------------------------ RoPE ------------------

def test_rope_listing_inverse_frequencies():
    """[KUNLUN] 挑战 5: pair k turns at the inverse frequency base^(-2k / head_size), one pair
    per rotated angle (all D/2 of them under full rotation).  Read each pair's frequency back
    from the oracle by rotating the unit vector e_k by one position."""
    for D, theta in ((256, 1e4), (512, 1e6), (8, 10.0)):
        listing = 1.0 / (theta ** (np.arange(0, D, 2, dtype=np.float64) / D))
        for k in range(D // 2):
            e = np.zeros(D)
            e[k] = 1.0
            y = oracle.rope(e, 1.0, theta)
            ang = math.atan2(y[k + D // 2], y[k])
            assert abs(ang - listing[k]) < 1e-12, (D, k)
            # the rest of the vector is untouched
            rest = np.delete(y, [k, k + D // 2])
            assert not rest.any()


def test_rope_invariants():
    rng = np.random.default_rng(4)
    D, theta = 256, 1e4
    x, z = rng.standard_normal(D), rng.standard_normal(D)
    np.testing.assert_array_equal(oracle.rope(x, 0.0, theta), x)          # t = 0: identity
    np.testing.assert_array_equal(oracle.rope(x, 123.0, 0.0), x)          # no RoPE
    for t in (1.0, 77.0, 36043.0):
        assert abs(np.linalg.norm(oracle.rope(x, t, theta)) - np.linalg.norm(x)) < 1e-12
    # the score depends only on the distance between positions
    a = oracle.rope(x, 900.0, theta) @ oracle.rope(z, 13.0, theta)
    b = oracle.rope(x, 1887.0, theta) @ oracle.rope(z, 1000.0, theta)
    assert abs(a - b) < 1e-9
    # composition
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, 40.0, theta), 2.0, theta),
                               oracle.rope(x, 42.0, theta), atol=1e-12)


def test_rope_equals_complex_rotation_of_half_pairs():
    """Rotate-half RoPE is the complex product z_k * exp(i t w_k) with z_k = x_k + i x_{k+D/2}."""
    rng = np.random.default_rng(5)
    D, theta, t = 512, 1e6, 31337.0
    x = rng.standard_normal(D)
    w = np.array([theta ** (-2.0 * k / D) for k in range(D // 2)])
    zc = (x[:D // 2] + 1j * x[D // 2:]) * np.exp(1j * t * w)
    np.testing.assert_allclose(oracle.rope(x, t, theta), np.concatenate([zc.real, zc.imag]),
                               atol=1e-11)


@pytest.mark.parametrize("D,theta,n,f", [(512, 1e6, 64, 1.0), (256, 1e4, 0, 1.0),
                                         (128, 1e4, 0, 8.0), (8, 10.0, 1, 1.0)])
def test_rope_rows_rotates_each_row_at_its_own_position(D, theta, n, f):
    """The batched rotation (every row x[i] at its own position t[i]) against the complex form
    z_k * exp(i (t_i / f) w_k), w_k = theta^(-2k/D) for k < n (all pairs when n = 0) and 0
    above, built here from the page's frequency list; and row by row equal to the single-vector
    rotation.  Positions are mixed (0, small, large, repeated, descending) so a wrong row or
    position stride fails."""
    rng = np.random.default_rng(D + n)
    t = np.array([0.0, 1.0, 36043.0, 5.0, 5.0, 4099.0, 2.0, 17.0, 1000.0, 31337.0])
    x = rng.standard_normal((len(t), D))
    nr = n if n else D // 2
    w = np.concatenate([1.0 / theta ** (np.arange(0, 2 * nr, 2, dtype=np.float64) / D),
                        np.zeros(D // 2 - nr)])
    y = oracle.rope_rows(x, t, theta, n, f)
    for i in range(len(t)):
        zc = (x[i, :D // 2] + 1j * x[i, D // 2:]) * np.exp(1j * (t[i] / f) * w)
        np.testing.assert_allclose(y[i], np.concatenate([zc.real, zc.imag]), rtol=0,
                                   atol=1e-11 * max(1.0, t[i] / f * w.max()))
        np.testing.assert_array_equal(y[i], oracle.rope(x[i], t[i], theta, n, f))
    # rows travel with their positions
    perm = rng.permutation(len(t))
    np.testing.assert_array_equal(oracle.rope_rows(x[perm], t[perm], theta, n, f), y[perm])
    # the input is not modified and a single row works
    np.testing.assert_array_equal(oracle.rope_rows(x[3:4], t[3:4], theta, n, f), y[3:4])


def _pair_angles(D, theta, angles=0, pos_scale=1.0, t=1.0):
    """Angle each pair (k, k + D/2) turns by, read back by rotating the unit vectors e_k."""
    out = np.empty(D // 2)
    for k in range(D // 2):
        e = np.zeros(D)
        e[k] = 1.0
        y = oracle.rope(e, t, theta, angles, pos_scale)
        out[k] = math.atan2(y[k + D // 2], y[k])
        assert not np.delete(y, [k, k + D // 2]).any()
    return out


@pytest.mark.parametrize("D,theta,n", [(512, 1e6, 64), (256, 1e4, 32), (8, 10.0, 1)])
def test_proportional_rope_listing_frequencies(D, theta, n):
    """[KUNLUN] 挑战 5: with n rotated angles the exponent still divides by the head size (not
    by 2n), and the D/2 - n remaining pairs get frequency 0 (identity).  Built here as the
    page's list: base^(-(0, 2, .., 2n-2) / head_size) followed by zeros."""
    listing = np.concatenate([1.0 / theta ** (np.arange(0, 2 * n, 2, dtype=np.float64) / D),
                              np.zeros(D // 2 - n)])
    np.testing.assert_allclose(_pair_angles(D, theta, n), listing, rtol=0, atol=1e-12)
    # the plausible slip of normalising by the rotated width instead would differ
    wrong = 1.0 / theta ** (np.arange(0, 2 * n, 2, dtype=np.float64) / (2 * n))
    if n > 1:
        assert np.abs(_pair_angles(D, theta, n)[:n] - wrong).max() > 1e-3


def test_proportional_rope_special_cases():
    rng = np.random.default_rng(41)
    D, theta = 256, 1e4
    x = rng.standard_normal(D)
    full = oracle.rope(x, 777.0, theta)
    np.testing.assert_array_equal(oracle.rope(x, 777.0, theta, D // 2), full)  # n = D/2: full
    np.testing.assert_array_equal(oracle.rope(x, 777.0, theta, 0), full)       # 0 means all
    y = oracle.rope(x, 777.0, theta, 16)
    keep = np.r_[16:D // 2, D // 2 + 16:D]
    np.testing.assert_array_equal(y[keep], x[keep])          # unrotated dims pass through
    rot = np.r_[0:16, D // 2:D // 2 + 16]
    np.testing.assert_array_equal(y[rot], full[rot])         # rotated dims as under full RoPE


def test_linear_rope_scaling_divides_the_position():
    """[INFLM] follow-up list: linear scaling divides the position by the factor, so position
    f*m under factor f turns exactly like position m unscaled, and every pair's angle at one
    position is the unscaled frequency over f."""
    rng = np.random.default_rng(42)
    D, theta, f = 512, 1e6, 8.0
    x = rng.standard_normal(D)
    for m in (0, 1, 5, 4099):
        np.testing.assert_allclose(oracle.rope(x, f * m, theta, 0, f),
                                   oracle.rope(x, float(m), theta), rtol=0, atol=1e-12)
    listing = 1.0 / theta ** (np.arange(0, D, 2, dtype=np.float64) / D)
    np.testing.assert_allclose(_pair_angles(D, theta, 0, f), listing / f, rtol=0, atol=1e-15)
    # scaled rotations stay relative: the score depends on the distance only
    z = rng.standard_normal(D)
    a = oracle.rope(x, 900.0, theta, 0, f) @ oracle.rope(z, 13.0, theta, 0, f)
    b = oracle.rope(x, 1887.0, theta, 0, f) @ oracle.rope(z, 1000.0, theta, 0, f)
    assert abs(a - b) < 1e-9


# ------------------------------------------------------------------ write path ------------

def test_plain_scatter_is_bit_exact_both_dtypes():
    rng = np.random.default_rng(6)
    Hq, Hkv, D = 2, 2, 8
    cl = np.array([21, 5, 33], np.int32)
    n = np.array([21, 3, 17], np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(cu[-1])
    nb = sum(-(-int(L) // BS) for L in cl) + 4
    bt = rng.permutation(nb)[:3 * 3].reshape(3, 3).astype(np.int32)
    for dt in (FP32, BF16):
        k32 = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        v32 = rng.standard_normal((T, Hkv, D)).astype(np.float32)
        k = bf16_bits_from_f32(k32) if dt == BF16 else k32
        v = bf16_bits_from_f32(v32) if dt == BF16 else v32
        et = np.uint16 if dt == BF16 else np.float32
        kc = np.zeros((nb, Hkv, BS, D), et)
        vc = np.zeros((nb, Hkv, D, BS), et)
        oracle.kv_cache_write(dt, Hq, Hkv, D, 0.0, 1e-6, 0, None, k, v, None, None, None, cu, cl,
                              bt, kc, vc)
        for b in range(3):
            past = cl[b] - n[b]
            for i in range(n[b]):
                t = past + i
                blk, off = bt[b, t // BS], t % BS
                for g in range(Hkv):
                    rows = page_rows(kc[blk, g].reshape(-1), D, unit_elems(
                        "bf16" if dt == BF16 else "fp32"), (t // BS) % 2)
                    np.testing.assert_array_equal(rows[off], k[cu[b] + i, g])
                np.testing.assert_array_equal(vc[blk, :, :, off], v[cu[b] + i])


def test_write_norm_then_rope_on_q_k_not_v():
    """[KUNLUN] §4.3 forward of a layer with its own cache: k_norm, then RoPE on q and k,
    then v_norm; [MNN] §6.1: q, k and v each have an RMSNorm."""
    rng = np.random.default_rng(7)
    Hq, Hkv, D, theta, eps = 4, 2, 16, 1e4, 1e-6
    cl, n = np.array([40], np.int32), np.array([7], np.int32)
    cu = np.array([0, 7], np.int32)
    bt = np.array([[5, 0, 3]], np.int32)
    q = rng.standard_normal((7, Hq, D)).astype(np.float32)
    k = rng.standard_normal((7, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((7, Hkv, D)).astype(np.float32)
    ws = [(1 + 0.1 * rng.standard_normal(D)).astype(np.float32) for _ in range(3)]
    kc = np.zeros((6, Hkv, BS, D), np.float32)
    vc = np.zeros((6, Hkv, D, BS), np.float32)
    q_out = q.copy()
    oracle.kv_cache_write(FP32, Hq, Hkv, D, theta, eps, 0, q_out, k, v, *ws, cu, cl, bt, kc, vc)

    def norm(x, w):  # torch's library routine
        return torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (D,),
                                            torch.from_numpy(w.astype(np.float64)), eps).numpy()

    def rot(x, t):   # complex formulation
        w = theta ** (-2.0 * np.arange(D // 2) / D)
        z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * t * w)
        return np.concatenate([z.real, z.imag], -1)

    for i in range(7):
        t = 33 + i
        blk, off = bt[0, t // BS], t % BS
        np.testing.assert_allclose(q_out[i], rot(norm(q[i], ws[0]), t), rtol=2e-7, atol=2e-7)
        krow = np.stack([page_rows(kc[blk, g].reshape(-1), D, unit_elems("fp32"),
                                   (t // BS) % 2)[off] for g in range(Hkv)])
        np.testing.assert_allclose(krow, rot(norm(k[i], ws[1]), t), rtol=2e-7, atol=2e-7)
        np.testing.assert_allclose(vc[blk, :, :, off], norm(v[i], ws[2]), rtol=2e-7, atol=2e-7)


def test_write_positions_follow_context_lens():
    """Token i of sequence b sits at absolute position context_lens[b] - n_b + i: with no norm,
    RoPE turns e_0 into (cos t, sin t) on the first pair (frequency 1)."""
    D, Hkv = 8, 1
    cl, n = np.array([50, 3], np.int32), np.array([4, 3], np.int32)
    cu = np.array([0, 4, 7], np.int32)
    bt = np.array([[0, 1, 2, 3], [4, 5, 5, 5]], np.int32)
    k = np.zeros((7, Hkv, D), np.float32)
    k[:, :, 0] = 1.0
    v = np.zeros_like(k)
    kc = np.zeros((6, Hkv, BS, D), np.float32)
    vc = np.zeros((6, Hkv, D, BS), np.float32)
    oracle.kv_cache_write(FP32, 1, Hkv, D, 1e4, 1e-6, 0, None, k, v, None, None, None, cu, cl,
                          bt, kc, vc)
    for b, poss in ((0, range(46, 50)), (1, range(0, 3))):
        for t in poss:
            row = page_rows(kc[bt[b, t // BS], 0].reshape(-1), D, unit_elems("fp32"),
                            (t // BS) % 2)[t % BS]
            assert abs(row[0] - math.cos(t)) < 1e-7 and abs(row[D // 2] - math.sin(t)) < 1e-7


def test_write_proportional_scaled_rope_and_q_only_layer():
    """Write with n rotated angles and a linear factor f ([KUNLUN] 挑战 5, [INFLM] follow-up
    list), checked against torch's RMSNorm and the complex rotation with the page's frequency
    list; then the same q through a layer that shares the cache ([KUNLUN] §4.3): k = v = None
    normalises and rotates q identically and leaves both caches bit-for-bit unchanged."""
    rng = np.random.default_rng(43)
    Hq, Hkv, D, theta, eps, n, f = 4, 2, 16, 1e6, 1e-6, 2, 8.0
    cl, cu = np.array([75], np.int32), np.array([0, 6], np.int32)
    bt = np.array([[5, 0, 3, 1, 2]], np.int32)
    q = rng.standard_normal((6, Hq, D)).astype(np.float32)
    k = rng.standard_normal((6, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((6, Hkv, D)).astype(np.float32)
    ws = [(1 + 0.1 * rng.standard_normal(D)).astype(np.float32) for _ in range(3)]
    kc = np.zeros((6, Hkv, BS, D), np.float32)
    vc = np.zeros((6, Hkv, D, BS), np.float32)
    q_out = q.copy()
    oracle.kv_cache_write(FP32, Hq, Hkv, D, theta, eps, 0, q_out, k, v, *ws, cu, cl, bt, kc, vc,
                          rope_angles=n, rope_scale=f)
    inv = np.concatenate([1.0 / theta ** (np.arange(0, 2 * n, 2, dtype=np.float64) / D),
                          np.zeros(D // 2 - n)])

    def norm(x, w):
        return torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (D,),
                                            torch.from_numpy(w.astype(np.float64)), eps).numpy()

    def rot(x, t):
        z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * (t / f) * inv)
        return np.concatenate([z.real, z.imag], -1)

    for i in range(6):
        t = 69 + i
        blk, off = bt[0, t // BS], t % BS
        np.testing.assert_allclose(q_out[i], rot(norm(q[i], ws[0]), t), rtol=2e-7, atol=2e-7)
        krow = np.stack([page_rows(kc[blk, g].reshape(-1), D, unit_elems("fp32"),
                                   (t // BS) % 2)[off] for g in range(Hkv)])
        np.testing.assert_allclose(krow, rot(norm(k[i], ws[1]), t), rtol=2e-7, atol=2e-7)

    kc0, vc0 = kc.copy(), vc.copy()
    q_shared = q.copy()
    oracle.kv_cache_write(FP32, Hq, Hkv, D, theta, eps, 0, q_shared, None, None, ws[0], None,
                          None, cu, cl, bt, kc, vc, rope_angles=n, rope_scale=f)
    np.testing.assert_array_equal(q_shared, q_out)
    np.testing.assert_array_equal(kc, kc0)
    np.testing.assert_array_equal(vc, vc0)


# ------------------------------------------------------------------ attention -------------

def _rand_case(rng, B=2, Hq=4, Hkv=2, D=16, lens=(37, 20), news=(9, 20)):
    K = [rng.standard_normal((Hkv, L, D)) for L in lens]
    V = [rng.standard_normal((Hkv, L, D)) for L in lens]
    kc, vc, bt = make_paged([k.astype(np.float32) for k in K], [v.astype(np.float32) for v in V],
                            seed=int(rng.integers(1 << 30)))
    n = np.array(news, np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), Hq, D)).astype(np.float32)
    return K, V, kc, vc, bt, q, cu, np.array(lens, np.int32), n


@pytest.mark.parametrize("W", [0, 1, 5, 16, 100])
def test_attention_matches_torch_sdpa_with_brute_force_mask(W):
    """No softcap: the oracle equals torch's scaled_dot_product_attention in float64 on the
    gathered K/V, with the mask enumerated from the page's rule and K/V heads repeated G times
    (GQA as repeat_kv)."""
    rng = np.random.default_rng(10 + W)
    K, V, kc, vc, bt, q, cu, cl, n = _rand_case(rng)
    Hq, D, Hkv = q.shape[1], q.shape[2], 2
    out = run_attn(kc, vc, bt, q, cu, cl, Hkv, window=W, scale=0.3)
    for b in range(len(cl)):
        L, nb, past = int(cl[b]), int(n[b]), int(cl[b] - n[b])
        qb = torch.from_numpy(q[cu[b]:cu[b + 1]].astype(np.float64)).permute(1, 0, 2)  # [Hq,n,D]
        kb = torch.from_numpy(K[b].astype(np.float32).astype(np.float64))
        vb = torch.from_numpy(V[b].astype(np.float32).astype(np.float64))
        kb = kb.repeat_interleave(Hq // Hkv, dim=0)
        vb = vb.repeat_interleave(Hq // Hkv, dim=0)
        mask = torch.from_numpy(visible(past, nb, W, L))
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask,
                                                               scale=0.3)
        np.testing.assert_allclose(out[cu[b]:cu[b + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("past,nnew,W", [(5, 6, 4), (0, 9, 3), (12, 4, 1), (3, 8, 0),
                                         (17, 15, 16), (16, 1, 16)])
def test_one_hot_probes_reproduce_the_brute_force_mask(past, nnew, W):
    """Plant one key whose score beats all others by 200 (exp(-200) ~ 1e-87): each query's
    output equals that key's value exactly when the key is visible to it."""
    L, D = past + nnew, 16
    for jstar in range(L):
        K = np.zeros((1, L, D))
        K[0, jstar, 0] = 200.0
        V = np.zeros((1, L, D))
        V[0, :, 1] = np.arange(L) + 1.0
        V[0, jstar, 1] = -1000.0
        kc, vc, bt = make_paged([K.astype(np.float32)], [V.astype(np.float32)], seed=jstar)
        q = np.zeros((nnew, 1, D), np.float32)
        q[:, 0, 0] = 1.0
        out = run_attn(kc, vc, bt, q, np.array([0, nnew], np.int32),
                       np.array([L], np.int32), 1, window=W)
        got = np.abs(out[:, 0, 1] + 1000.0) < 1e-6
        np.testing.assert_array_equal(got, visible(past, nnew, W, L)[:, jstar])


def test_equal_scores_give_the_mean_of_visible_values():
    rng = np.random.default_rng(11)
    K, V, kc, vc, bt, q, cu, cl, n = _rand_case(rng)
    q[:] = 0.0
    for W in (0, 7):
        out = run_attn(kc, vc, bt, q, cu, cl, 2, window=W, cap=50.0)
        for b in range(2):
            past = cl[b] - n[b]
            for i in range(n[b]):
                t = past + i
                lo = max(0, t - W + 1) if W else 0
                for h in range(4):
                    mean = V[b][h // 2, lo:t + 1].astype(np.float32).astype(np.float64).mean(0)
                    np.testing.assert_allclose(out[cu[b] + i, h], mean, rtol=1e-12, atol=1e-14)


def test_window_one_returns_own_value_and_wide_window_equals_global():
    rng = np.random.default_rng(12)
    K, V, kc, vc, bt, q, cu, cl, n = _rand_case(rng)
    out1 = run_attn(kc, vc, bt, q, cu, cl, 2, window=1, cap=10.0)
    for b in range(2):
        past = cl[b] - n[b]
        for i in range(n[b]):
            for h in range(4):
                np.testing.assert_array_equal(out1[cu[b] + i, h],
                                              V[b][h // 2, past + i].astype(np.float32))
    np.testing.assert_array_equal(run_attn(kc, vc, bt, q, cu, cl, 2, window=int(cl.max())),
                                  run_attn(kc, vc, bt, q, cu, cl, 2, window=0))


def test_softcap_two_key_closed_form_and_bound():
    """[INFLM] Gemma-2 §1: scores are capped as cap*tanh(s/cap) after scaling and before the
    softmax.  Two keys: out = v1 + sigmoid(c2 - c1) (v2 - v1) with c = cap*tanh(scale*s/cap)."""
    D = 16
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    for s1, s2, cap, scale in ((3.0, 90.0, 50.0, 1.0), (-40.0, 40.0, 5.0, 0.5), (1.0, 2.0, 50.0, 0.0625)):
        K = np.zeros((1, 2, D))
        K[0, 0, 0], K[0, 1, 0] = s1, s2
        V = np.random.default_rng(13).standard_normal((1, 2, D))
        kc, vc, bt = make_paged([K.astype(np.float32)], [V.astype(np.float32)], seed=1)
        out = run_attn(kc, vc, bt, q, np.array([0, 1], np.int32), np.array([2], np.int32), 1,
                       scale=scale, cap=cap)[0, 0]
        c1, c2 = cap * math.tanh(scale * s1 / cap), cap * math.tanh(scale * s2 / cap)
        v = V.astype(np.float32).astype(np.float64)[0]
        expect = v[0] + (v[1] - v[0]) / (1.0 + math.exp(-(c2 - c1)))
        np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-13)
        # capped scores differ by less than 2*cap, so neither weight drops below 1/(1+e^(2cap))
        w2 = (out[1] - v[0, 1]) / (v[1, 1] - v[0, 1])
        assert 1.0 / (1.0 + math.exp(2 * cap)) <= w2 <= 1.0 - 1.0 / (1.0 + math.exp(2 * cap))


def test_softcap_large_cap_tends_to_uncapped():
    rng = np.random.default_rng(14)
    K, V, kc, vc, bt, q, cu, cl, n = _rand_case(rng)
    a = run_attn(kc, vc, bt, q, cu, cl, 2, window=6, cap=1e7)
    b = run_attn(kc, vc, bt, q, cu, cl, 2, window=6, cap=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-10)
    c = run_attn(kc, vc, bt, q, cu, cl, 2, window=6, cap=3.0)
    assert np.abs(c - b).max() > 1e-3   # a small cap does change the result


def test_k_eq_v_equals_separate_cache_holding_the_same_tensor():
    rng = np.random.default_rng(15)
    K, V, kc, vc, bt, q, cu, cl, n = _rand_case(rng)
    # the same tensor in the V page layout: K's logical rows, transposed per page
    vc_from_k = np.ascontiguousarray(np.swapaxes(logical_k(kc, bt, cl, unit_elems("fp32")), 2, 3))
    a = run_attn(kc, None, bt, q, cu, cl, 2, window=9, k_eq_v=1)
    b = run_attn(kc, vc_from_k, bt, q, cu, cl, 2, window=9, k_eq_v=0)
    np.testing.assert_array_equal(a, b)


def test_paging_is_invisible_shuffled_equals_contiguous():
    rng = np.random.default_rng(16)
    K, V, kc, vc, bt, q, cu, cl, n = _rand_case(rng)
    ident_kc, ident_vc = np.empty_like(kc), np.empty_like(vc)
    bt2 = np.zeros_like(bt)
    nxt = 0
    for b in range(bt.shape[0]):
        for p in range(-(-int(cl[b]) // BS)):
            ident_kc[nxt], ident_vc[nxt] = kc[bt[b, p]], vc[bt[b, p]]
            bt2[b, p] = nxt
            nxt += 1
    a = run_attn(kc, vc, bt, q, cu, cl, 2, window=5, cap=30.0)
    c = run_attn(ident_kc, ident_vc, bt2, q, cu, cl, 2, window=5, cap=30.0)
    np.testing.assert_array_equal(a, c)


def test_decode_is_last_row_of_prefill_and_chunked_equals_one_shot():
    rng = np.random.default_rng(17)
    K, V, kc, vc, bt, q, cu, cl, n = _rand_case(rng, lens=(40, 33), news=(40, 33))
    full = run_attn(kc, vc, bt, q, cu, cl, 2, window=11, cap=20.0)
    # decode at L: the last new token of each sequence
    qd = np.ascontiguousarray(q[cu[1:] - 1])
    dec = oracle.attn_decode(FP32, 4, 2, 16, 11, 1.0, 20.0, 0, qd, kc, vc, bt, cl)
    np.testing.assert_array_equal(dec, full[cu[1:] - 1])
    # chunked: the last 12 / 5 tokens as a chunk appended to the rest
    m = np.array([12, 5], np.int32)
    cu2 = np.concatenate([[0], np.cumsum(m)]).astype(np.int32)
    rows = np.concatenate([np.arange(cu[b + 1] - m[b], cu[b + 1]) for b in range(2)])
    part = run_attn(kc, vc, bt, np.ascontiguousarray(q[rows]), cu2, cl, 2, window=11, cap=20.0)
    np.testing.assert_array_equal(part, full[rows])


def test_row_subset_computes_only_listed_rows():
    rng = np.random.default_rng(18)
    K, V, kc, vc, bt, q, cu, cl, n = _rand_case(rng)
    full = run_attn(kc, vc, bt, q, cu, cl, 2, window=3)
    rows = np.array([0, 8, 9, 28], np.int32)
    sub = run_attn(kc, vc, bt, q, cu, cl, 2, window=3, rows=rows)
    np.testing.assert_array_equal(sub[rows], full[rows])
    assert np.isnan(np.delete(sub, rows, axis=0)).all()
