"""CPU: the MFMA operand layouts the prefill kernels assume, emulated lane by
lane in numpy, compute the matrices the kernels intend.  The per-lane layout
of the two gfx950 instructions (v_mfma_f32_16x16x16_bf16 and
v_mfma_f32_16x16x32_bf16), as AMD's CDNA matrix-instruction documentation
gives it, with lane = 16 lq + ln:
  A operand: lane holds A[ln][K block of lq]     (4 or 8 consecutive K)
  B operand: lane holds B[K block of lq][ln]
  result C : lane holds C[4 lq + i][ln], i = 0..3
On these layouts the tests check the kernels' layout arithmetic: chained
16 x 16 products with no data movement (prod), the copy of a row-loaded tile
into the C layout by an identity or a 0/1 selector, the channel order of the
state tiles (chan), and the hi + lo split of U in the state update."""
import numpy as np

RNG = np.random.default_rng(5)
LANES = [(l >> 4, l & 15) for l in range(64)]   # (lq, ln)


def mfma(A_lanes, B_lanes, C_lanes=None):
    """D = A B (+ C) from per-lane operands: A_lanes[l] and B_lanes[l] hold
    KB = K / 4 values each (K = 16 or 32); returns per-lane results [64, 4]."""
    kb = A_lanes.shape[1]
    A = np.zeros((16, 4 * kb))
    B = np.zeros((4 * kb, 16))
    for l, (lq, ln) in enumerate(LANES):
        A[ln, kb * lq:kb * lq + kb] = A_lanes[l]
        B[kb * lq:kb * lq + kb, ln] = B_lanes[l]
    D = A @ B
    out = np.array([[D[4 * lq + i, ln] for i in range(4)] for lq, ln in LANES])
    return out if C_lanes is None else out + C_lanes


def c_layout(X):
    """Per-lane C-layout registers of a 16 x 16 matrix."""
    return np.array([[X[4 * lq + i, ln] for i in range(4)] for lq, ln in LANES])


def from_c(lanes):
    X = np.zeros((16, 16))
    for l, (lq, ln) in enumerate(LANES):
        for i in range(4):
            X[4 * lq + i, ln] = lanes[l, i]
    return X


def test_prod_chains_without_moves():
    """prod(XT, Y) = mma16(C(X^T), C(Y)) is C(X Y): the result of one product
    is directly an operand of the next (the Neumann chain of stage B1)."""
    X, Y, Z = (RNG.standard_normal((16, 16)) for _ in range(3))
    XY = mfma(c_layout(X.T), c_layout(Y))       # prod(C(M), C(N)) = C(M^T N)
    assert np.allclose(from_c(XY), X @ Y)
    # (X Y) Z needs C((X Y)^T) as A: prod(C(Y), C(X^T)) = C(Y^T X^T), as stage B1
    # forms L^2 and (L^2)^T side by side
    XYT = mfma(c_layout(Y), c_layout(X.T))
    assert np.allclose(from_c(XYT), (X @ Y).T)
    assert np.allclose(from_c(mfma(XYT, c_layout(Z))), X @ Y @ Z)


def test_identity_and_selector_copies():
    """A row-loaded 16 x 16 bf16 tile (lane: row ln, columns 4 lq .. +3) times the
    identity B operand (lane value e = 1 iff 4 lq + e == ln) is the tile's C
    layout; with K = 32, a 0/1 selector picks columns 16 h .. +15 of a row-loaded
    32-column block (lane: row ln, columns 8 lq .. +7)."""
    V = RNG.standard_normal((16, 16))
    rows = np.array([V[ln, 4 * lq:4 * lq + 4] for lq, ln in LANES])
    eye = np.array([[1.0 if 4 * lq + e == ln else 0.0 for e in range(4)] for lq, ln in LANES])
    assert np.array_equal(from_c(mfma(rows, eye)), V)
    W = RNG.standard_normal((16, 32))
    rows32 = np.array([W[ln, 8 * lq:8 * lq + 8] for lq, ln in LANES])
    for h in range(2):
        sel = np.array([[1.0 if (lq == 2 * h + (ln >> 3) and e == (ln & 7)) else 0.0 for e in range(8)]
                        for lq, ln in LANES])
        assert np.array_equal(from_c(mfma(rows32, sel)), W[:, 16 * h:16 * h + 16])


def chan(m, lq, i):
    return 32 * (m >> 1) + 8 * lq + 4 * (m & 1) + i


def test_state_channel_order():
    """State tile m holds channels chan(m, lq, i) in row 4 lq + i; then the 8 K
    values of lane quarter lq in K block s (tiles 2 s, 2 s + 1, packed as
    [tile 2 s | tile 2 s + 1]) are the consecutive channels 32 s + 8 lq .. +7:
    W' = w S over K = d_k is a sum of NKB 16x16x32 products whose A operand is a
    plain 16-byte load of a token's w row."""
    dk, cols = 128, 16
    S = RNG.standard_normal((dk, cols))         # d_k x 16 columns of the state
    w = RNG.standard_normal((16, dk))           # 16 tokens x d_k
    tiles = [np.array([[S[chan(m, lq, i), ln] for i in range(4)] for lq, ln in LANES]) for m in range(dk // 16)]
    acc = np.zeros((64, 4))
    for s in range(dk // 32):
        A = np.array([w[ln, 32 * s + 8 * lq:32 * s + 8 * lq + 8] for lq, ln in LANES])
        Bop = np.concatenate([tiles[2 * s], tiles[2 * s + 1]], axis=1)
        acc = mfma(A, Bop, acc)
    assert np.allclose(from_c(acc), w @ S)
    # the channels of lane quarter lq in block s are exactly those 8 consecutive ones
    for s in range(dk // 32):
        for lq in range(4):
            got = [chan(2 * s, lq, i) for i in range(4)] + [chan(2 * s + 1, lq, i) for i in range(4)]
            assert got == list(range(32 * s + 8 * lq, 32 * s + 8 * lq + 8))


def bf16(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def test_hilo_state_update():
    """S += k^r^T U with U as [hi | lo] bf16 and k^r repeated in both halves:
    one 16x16x32 product whose error is that of U to ~2^-16, not 2^-9."""
    U = RNG.standard_normal((16, 16))             # tokens x columns
    kr = bf16(RNG.standard_normal((16, 16)))      # tokens x 16 channels (bf16 operand)
    hi = bf16(U)
    lo = bf16(U - hi)
    # A: lane (lq, ln) = channel ln, K = [tokens 4 lq .. +3 (hi) | the same tokens (lo)]
    A = np.array([np.concatenate([kr[4 * lq:4 * lq + 4, ln], kr[4 * lq:4 * lq + 4, ln]]) for lq, ln in LANES])
    Bop = np.array([np.concatenate([hi[4 * lq:4 * lq + 4, ln], lo[4 * lq:4 * lq + 4, ln]]) for lq, ln in LANES])
    # the emulation's K order is [8 lq .. 8 lq + 7]; both operands use the same order, so the sum is unchanged
    got = from_c(mfma(A, Bop))
    want = kr.T @ U
    err_hilo = np.max(np.abs(got - want)) / np.max(np.abs(want))
    err_single = np.max(np.abs(kr.T @ hi - want)) / np.max(np.abs(want))
    assert err_hilo < 2.0 ** -14 < err_single
