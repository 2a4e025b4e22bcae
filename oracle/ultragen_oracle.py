"""fp64 CPU oracle for UltraGen's composite-masked hierarchical local attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it, and
it shares no code, header or table with the library.

Sources (cited by page title and section):
  [KD1] "UltraGen: Efficient Ultra-High-Resolution Image Generation with
        Hierarchical Local Attention", papernotes.org notes, 关键设计 1
        (window-first local window attention): non-overlapping l x l windows,
        l = 16, tokens regrouped window by window, adjacent-window interaction.
  [KD2] same page, 关键设计 2 (scale-aligned low-resolution guidance): the LR
        latent with rho = H/h, the coordinate map (m, n) -> (rho*m, rho*n), and
        the attention-mask description (text <-> itself and HR; HR -> own and
        adjacent windows, text and LR anchors; LR -> all LR).
  [KD3] same page, 关键设计 3: the joint sequence [C_T; X; X_lr] and the joint
        attention softmax(Q K^T (masked) / sqrt(d)) V.
  [GS-B] "UltraGen ..." summary on gist.science (paper 2510.16325), section
        2.B (Attention Masking): windows attend to themselves and adjacent
        windows and to the scaled global guidance tokens; LR tokens attend
        globally to each other.
  [KD3-FT] papernotes.org notes, 关键设计 3 and the 损失函数 / 训练策略
        section: the LR branch is fine-tuned (LoRA on its Q, K, V
        projections) by gradient descent on the flow-matching loss, so the
        loss is differentiated through the joint attention.
  [KD4] same page, 关键设计 4 (guidance-weighted warm start): the LR latent is
        upsampled by interpolation and sharpened into a reference, and the HR
        start latent is alpha * X_T + (1 - alpha) * reference, alpha = t/T;
        [GS] section 2.C repeats it (upsampled, sharpened, added at an
        intermediate timestep).

Everything is computed in float64, in RASTER order (text rows, then HR rows
r*W + c, then LR rows m*w + n), and every mask decision is taken from 2D
coordinates, never from a permutation.  Readings of points the pages leave
open (R1-R12, each taken as the plainest reading the rest of the pages supports):
  R1 windows and tokens inside a window are both ordered row-major;
  R2 ragged grids use a ceil partition with partial edge windows and a compact
     permutation (no padding);
  R3 LR grid defaults to ceil(H/rho) x ceil(W/rho); LR position = (rho*m, rho*n);
  R4 text tokens sit at position (0, 0), i.e. are not rotated;
  R5 axial RoPE: first half of the head dims rotated by the row position, second
     half by the column position, adjacent pairs (x[2k], x[2k+1]), frequency
     omega_k = theta^(-2k/(D/2)), k = 0 .. D/4-1;
  R6 the mask is additive -inf (masked keys excluded), scale 1/sqrt(D), one
     softmax over the union of allowed keys;
  R7 "adjacent" = Chebyshev window distance <= radius (radius 1 = 3x3 windows);
  R8 HR queries see ALL LR tokens; LR queries see LR and text; text queries see
     text and HR, not LR.
  R8' (variant, lr_mode = 1) [KD2] says HR tokens attend to the
     *corresponding* LR anchors: an LR token corresponds to the window that
     contains its scaled position (rho*m, rho*n); an HR query sees the LR
     tokens of the windows within its neighbourhood radius, exactly like its
     HR keys.  An LR token whose scaled position lies beyond the window grid
     (only possible when the LR grid is given larger than ceil(H/rho) x
     ceil(W/rho)) is inside no window, so it corresponds to none and no HR
     query sees it; LR queries still see it.
  R11 backward [KD3-FT]: the pages only say the attention is trained, so the
     backward is the exact derivative of the forward above (RoPE, composite
     mask, softmax, PV) with respect to the raster Q, K, V, given dO; the
     log-sum-exp saved by the forward is the natural log of the softmax
     denominator of the scaled logits q.k/sqrt(D).
  R12 warm start [KD4]: the pages name the steps but not the operators.
     Interpolation is bilinear on the HR grid with LR sample (m, n) at HR
     position (rho*m, rho*n) (the coordinate map of [KD2]); HR rows/columns
     past the last sample take its value.  Sharpening is unsharp masking,
     Y = U + s * (U - B*U), B the 3x3 binomial blur ([1 2 1]/4 both ways) with
     edges replicated, strength s a parameter (0 = none).  The noising at
     time t is the blend itself: alpha * X_T + (1 - alpha) * Y with alpha =
     t/T is the rectified-flow noising of Y at t, and the formula for the
     reference carries no noise term of its own.  X_T (Gaussian) is an input.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

TEXT, HR, LR = 0, 1, 2


@dataclass(frozen=True)
class Geometry:
    """Token grid geometry of one attention layer ([KD1], [KD2], [KD3])."""
    hr_h: int
    hr_w: int
    lr_h: int
    lr_w: int
    n_text: int
    window: int
    radius: int
    rho: int
    lr_mode: int = 0   # 0: HR sees all LR (R8); 1: corresponding LR only (R8')

    @property
    def n_hr(self):
        return self.hr_h * self.hr_w

    @property
    def n_lr(self):
        return self.lr_h * self.lr_w

    @property
    def seq_len(self):
        return self.n_text + self.n_hr + self.n_lr

    @property
    def grid(self):
        """Windows per column / row of the HR grid: ceil partition (R2)."""
        return (-(-self.hr_h // self.window), -(-self.hr_w // self.window))


def geometry(hr_h, hr_w, n_text, window=16, radius=1, rho=4, lr_h=None, lr_w=None, lr_mode=0) -> Geometry:
    """LR grid defaults to ceil(H/rho) x ceil(W/rho), since rho = H/h ([KD2], R3);
    an explicit 0 means no LR tokens."""
    if lr_h is None:
        lr_h = -(-hr_h // rho)
    if lr_w is None:
        lr_w = -(-hr_w // rho)
    return Geometry(hr_h, hr_w, lr_h, lr_w, n_text, window, radius, rho, lr_mode)


def geometry_of(w) -> Geometry:
    """Geometry of a workloads.Workload (duck-typed)."""
    return geometry(w.hr_h, w.hr_w, w.n_text, w.window, w.radius, w.rho, w.lr_h, w.lr_w,
                    getattr(w, "lr_mode", 0))


def token_coords(g: Geometry):
    """Per raster row: kind, RoPE position (row, col) and HR window (wy, wx).

    HR token r*W + c sits at (r, c) in window (r // l, c // l) [KD1]; LR token
    m*w + n sits at (rho*m, rho*n) [KD2], in the window containing that
    position (R8'); text sits at (0, 0) (R4) and has window -1.
    """
    L = g.seq_len
    kind = np.empty(L, np.int64)
    pr = np.zeros(L, np.int64)
    pc = np.zeros(L, np.int64)
    wy = np.full(L, -1, np.int64)
    wx = np.full(L, -1, np.int64)
    T, N = g.n_text, g.n_hr
    kind[:T] = TEXT
    kind[T:T + N] = HR
    kind[T + N:] = LR
    r, c = np.divmod(np.arange(N), g.hr_w)
    pr[T:T + N], pc[T:T + N] = r, c
    wy[T:T + N], wx[T:T + N] = r // g.window, c // g.window
    if g.n_lr:
        m, n = np.divmod(np.arange(g.n_lr), g.lr_w)
        pr[T + N:], pc[T + N:] = g.rho * m, g.rho * n
        wy[T + N:], wx[T + N:] = g.rho * m // g.window, g.rho * n // g.window
    return kind, pr, pc, wy, wx


# --------------------------------------------------------------------------
# Window-first order and window adjacency, derived from coordinates
# --------------------------------------------------------------------------

def window_first_perm(hr_h: int, hr_w: int, window: int) -> np.ndarray:
    """perm[j] = raster index of the j-th HR token in window-first order.

    [KD1]: the token sequence is regrouped window by window so that each
    window is one contiguous block.  Sort key (R1): window row, window column,
    row inside the window, column inside the window.
    """
    r, c = np.divmod(np.arange(hr_h * hr_w), hr_w)
    keys = (c % window, r % window, c // window, r // window)  # lexsort: last key is primary
    return np.lexsort(keys).astype(np.int64)


def window_offsets(hr_h: int, hr_w: int, window: int) -> np.ndarray:
    """Start of each window (row-major window order) in window-first order."""
    gy, gx = -(-hr_h // window), -(-hr_w // window)
    sizes = []
    for a in range(gy):
        for b in range(gx):
            hy = min(window, hr_h - a * window)
            hx = min(window, hr_w - b * window)
            sizes.append(hy * hx)
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


def lr_window_first_perm(g: Geometry) -> np.ndarray:
    """LR tokens grouped by the window containing their scaled position
    (R8'), windows row-major, tokens row-major inside; LR tokens whose
    position falls outside the HR window grid come last, in raster order."""
    gy, gx = g.grid
    m, n = np.divmod(np.arange(g.n_lr), g.lr_w)
    a, b = g.rho * m // g.window, g.rho * n // g.window
    outside = ((a >= gy) | (b >= gx)).astype(np.int64)
    win = np.where(outside == 1, 0, a * gx + b)
    return np.lexsort((n, m, win, outside)).astype(np.int64)


def lr_window_offsets(g: Geometry) -> np.ndarray:
    """Start of each window's LR tokens in the LR window-first order; the
    last entry is where the out-of-grid tail starts (then n_lr follows)."""
    gy, gx = g.grid
    m, n = np.divmod(np.arange(g.n_lr), g.lr_w)
    a, b = g.rho * m // g.window, g.rho * n // g.window
    inside = (a < gy) & (b < gx)
    counts = np.bincount((a * gx + b)[inside], minlength=gy * gx)
    return np.concatenate([[0], np.cumsum(counts), [g.n_lr]]).astype(np.int64)


def neighbour_windows(hr_h: int, hr_w: int, window: int, radius: int):
    """For each window (row-major), the windows within Chebyshev distance
    `radius` (its own included), ascending by window index ([KD1] adjacent
    windows, [GS-B], R7).  Returns (flat list, offsets)."""
    gy, gx = -(-hr_h // window), -(-hr_w // window)
    flat, off = [], [0]
    for a in range(gy):
        for b in range(gx):
            for a2 in range(gy):
                for b2 in range(gx):
                    if max(abs(a - a2), abs(b - b2)) <= radius:
                        flat.append(a2 * gx + b2)
            off.append(len(flat))
    return np.asarray(flat, np.int64), np.asarray(off, np.int64)


# --------------------------------------------------------------------------
# 2D axial RoPE ([KD1] RoPE range, [KD2] scaled LR positions; R4, R5)
# --------------------------------------------------------------------------

def rope_rotate(x: np.ndarray, pos_r: np.ndarray, pos_c: np.ndarray, theta: float) -> np.ndarray:
    """Rotate rows of x [n, D] (float64) at positions (pos_r, pos_c).

    Dims [0, D/2) carry the row position, dims [D/2, D) the column position.
    Inside each half, pair (2k, 2k+1) turns by angle pos * theta^(-2k/(D/2)):
    (a, b) -> (a cos - b sin, a sin + b cos).
    """
    n, D = x.shape
    assert D % 4 == 0
    half = D // 2
    k = np.arange(D // 4, dtype=np.float64)
    omega = theta ** (-2.0 * k / half)
    out = np.array(x, dtype=np.float64, copy=True)
    for base, pos in ((0, pos_r), (half, pos_c)):
        ang = np.asarray(pos, np.float64)[:, None] * omega[None, :]
        cs, sn = np.cos(ang), np.sin(ang)
        a = x[:, base + 0:base + half:2]
        b = x[:, base + 1:base + half:2]
        out[:, base + 0:base + half:2] = a * cs - b * sn
        out[:, base + 1:base + half:2] = a * sn + b * cs
    return out


# --------------------------------------------------------------------------
# The composite mask ([KD2], [GS-B], [KD3]; R6-R8)
# --------------------------------------------------------------------------

def _in_window_grid(g: Geometry, wy, wx) -> np.ndarray:
    """Whether a token's window (wy, wx) is one of the gy x gx grid windows
    (R8': an LR anchor beyond the grid belongs to no window)."""
    gy, gx = g.grid
    return (wy >= 0) & (wy < gy) & (wx >= 0) & (wx < gx)


def allowed_keys_of(g: Geometry, coords, i: int) -> np.ndarray:
    """Raster indices of the keys query row i may attend to."""
    kind, _, _, wy, wx = coords
    if kind[i] == TEXT:
        ok = (kind == TEXT) | (kind == HR)
    elif kind[i] == LR:
        ok = (kind == LR) | (kind == TEXT)
    else:
        near = np.maximum(np.abs(wy - wy[i]), np.abs(wx - wx[i])) <= g.radius
        lr_ok = (kind == LR) & (near & _in_window_grid(g, wy, wx) if g.lr_mode == 1 else True)
        ok = (kind == TEXT) | lr_ok | (near & (kind == HR))
    return np.nonzero(ok)[0]


def allowed_dense(g: Geometry) -> np.ndarray:
    """Explicit L x L boolean mask (small grids only)."""
    kind, _, _, wy, wx = token_coords(g)
    qt, kt = kind[:, None], kind[None, :]
    near = np.maximum(np.abs(wy[:, None] - wy[None, :]), np.abs(wx[:, None] - wx[None, :])) <= g.radius
    hr_near = near & (qt == HR) & (kt == HR)
    text_q = (qt == TEXT) & ((kt == TEXT) | (kt == HR))
    lr_q = (qt == LR) & ((kt == LR) | (kt == TEXT))
    hr_lr = (qt == HR) & (kt == LR)
    if g.lr_mode == 1:
        hr_lr = hr_lr & near & _in_window_grid(g, wy, wx)[None, :]
    hr_q = (qt == HR) & (kt == TEXT)
    return text_q | lr_q | hr_q | hr_lr | hr_near


def pair_count(g: Geometry) -> int:
    """Exact number of allowed (query, key) pairs per head, counted from
    coordinates one query group at a time."""
    T, N, Nl = g.n_text, g.n_hr, g.n_lr
    total = T * (T + N) + Nl * (Nl + T)
    off = window_offsets(g.hr_h, g.hr_w, g.window)
    size = np.diff(off)
    lr_size = np.diff(lr_window_offsets(g))[:-1] if Nl else np.zeros(size.size, np.int64)
    gy, gx = g.grid
    for a in range(gy):
        for b in range(gx):
            seen = 0
            lr_seen = 0
            for a2 in range(max(0, a - g.radius), min(gy, a + g.radius + 1)):
                for b2 in range(max(0, b - g.radius), min(gx, b + g.radius + 1)):
                    seen += int(size[a2 * gx + b2])
                    lr_seen += int(lr_size[a2 * gx + b2])
            lr_keys = lr_seen if g.lr_mode == 1 else Nl
            total += int(size[a * gx + b]) * (T + lr_keys + seen)
    return total


# --------------------------------------------------------------------------
# Attention ([KD3]: softmax(Q K^T / sqrt(d), masked) V over [C_T; X; X_lr])
# --------------------------------------------------------------------------

def _softmax_rows(s: np.ndarray) -> np.ndarray:
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def attention_dense(q, k, v, allowed):
    """Mode (i): one head, explicit boolean mask; masked logits are -inf."""
    D = q.shape[1]
    s = (q @ k.T) / math.sqrt(D)
    s = np.where(allowed, s, -np.inf)
    return _softmax_rows(s) @ v


def _rows_attention(qr, kr, v, rows, keys):
    D = qr.shape[1]
    s = (qr[rows] @ kr[keys].T) / math.sqrt(D)
    return _softmax_rows(s) @ v[keys]


def attention_grouped(g: Geometry, qr, kr, v):
    """Mode (ii): one head; query rows grouped by the key set they share
    (text rows, LR rows, HR rows of one window); key indices gathered from
    coordinates.  qr, kr are already rotated."""
    coords = token_coords(g)
    kind, _, _, wy, wx = coords
    out = np.empty_like(v, dtype=np.float64)
    T, N = g.n_text, g.n_hr
    groups = []
    if T:
        groups.append(np.arange(T))
    if g.n_lr:
        groups.append(np.arange(T + N, g.seq_len))
    gy, gx = g.grid
    hr_rows = np.arange(T, T + N)
    for a in range(gy):
        for b in range(gx):
            groups.append(hr_rows[(wy[hr_rows] == a) & (wx[hr_rows] == b)])
    for rows in groups:
        if rows.size == 0:
            continue
        keys = allowed_keys_of(g, coords, int(rows[0]))
        out[rows] = _rows_attention(qr, kr, v, rows, keys)
    return out


def rotate_head(g: Geometry, x, theta):
    """RoPE for every row of one head (text rows stay at position (0, 0))."""
    _, pr, pc, _, _ = token_coords(g)
    return rope_rotate(x, pr, pc, theta)


def forward_head(g: Geometry, q, k, v, theta, mode="grouped"):
    """Full path for one head in raster order: RoPE on Q and K, then the
    composite-masked attention.  q, k, v: [L, D] float64."""
    qr = rotate_head(g, q, theta)
    kr = rotate_head(g, k, theta)
    if mode == "dense":
        return attention_dense(qr, kr, v, allowed_dense(g))
    return attention_grouped(g, qr, kr, v)


def forward_rows(g: Geometry, q, k, v, theta, rows):
    """Outputs of selected raster rows of one head (for full-size sampling)."""
    coords = token_coords(g)
    _, pr, pc, _, _ = coords
    rows = np.asarray(rows, np.int64)
    qr = np.zeros_like(q)
    qr[rows] = rope_rotate(q[rows], pr[rows], pc[rows], theta)
    kr = rope_rotate(k, pr, pc, theta)
    out = np.empty((rows.size, v.shape[1]))
    for idx, i in enumerate(rows):
        keys = allowed_keys_of(g, coords, int(i))
        out[idx] = _rows_attention(qr, kr, v, np.array([i]), keys)[0]
    return out


# --------------------------------------------------------------------------
# Backward ([KD3-FT], R11): gradients of O = softmax(S) V, S = Qr Kr^T/sqrt(D)
# over the allowed keys, then of the RoPE rotation.
# --------------------------------------------------------------------------

def allowed_queries_of(g: Geometry, coords, j: int) -> np.ndarray:
    """Raster indices of the queries that attend to key row j (the column of
    the composite mask, written out from coordinates like allowed_keys_of)."""
    kind, _, _, wy, wx = coords
    if kind[j] == TEXT:      # text, HR and LR queries all see text keys
        ok = np.ones(kind.size, bool)
    elif kind[j] == HR:      # text queries see all HR; HR queries of nearby windows
        near = np.maximum(np.abs(wy - wy[j]), np.abs(wx - wx[j])) <= g.radius
        ok = (kind == TEXT) | ((kind == HR) & near)
    else:                    # HR queries (all, or nearby windows for lr_mode 1) and LR queries
        if g.lr_mode == 1:
            near = np.maximum(np.abs(wy - wy[j]), np.abs(wx - wx[j])) <= g.radius
            inside = bool(_in_window_grid(g, wy[j:j + 1], wx[j:j + 1])[0])
            hr_ok = (kind == HR) & near & inside
        else:
            hr_ok = kind == HR
        ok = hr_ok | (kind == LR)
    return np.nonzero(ok)[0]


def rope_rotate_transpose(x, pos_r, pos_c, theta):
    """Transpose of the RoPE rotation (each 2x2 block is orthogonal, so the
    transpose is the rotation by the negated angle): maps dL/d(rotated x)
    to dL/dx."""
    return rope_rotate(x, -np.asarray(pos_r), -np.asarray(pos_c), theta)


def _row_stats(qr, kr, v, i, keys):
    """Softmax row i over `keys`: probabilities, natural-log LSE of the scaled
    logits, and the output row."""
    D = qr.shape[1]
    s = (kr[keys] @ qr[i]) / math.sqrt(D)
    mx = s.max()
    e = np.exp(s - mx)
    z = e.sum()
    p = e / z
    return p, mx + math.log(z), p @ v[keys]


def lse_grouped(g: Geometry, qr, kr) -> np.ndarray:
    """Natural-log log-sum-exp of the scaled logits over each row's allowed
    keys (one head, raster order)."""
    coords = token_coords(g)
    D = qr.shape[1]
    out = np.empty(g.seq_len)
    for i in range(g.seq_len):
        keys = allowed_keys_of(g, coords, i)
        s = (kr[keys] @ qr[i]) / math.sqrt(D)
        mx = s.max()
        out[i] = mx + math.log(np.exp(s - mx).sum())
    return out


def attention_backward_grouped(g: Geometry, qr, kr, v, do):
    """Gradients (dQr, dKr, dV) of the masked attention of one head with
    respect to the rotated Q, K and to V, given dO (raster order):
      P = softmax(S) over allowed keys, dP = dO V^T, Delta_i = sum_j P_ij dP_ij,
      dS = P * (dP - Delta), dQr = dS Kr / sqrt(D), dKr = dS^T Qr / sqrt(D),
      dV = P^T dO.
    Query rows are grouped by the key set they share, as in the forward."""
    coords = token_coords(g)
    kind, _, _, wy, wx = coords
    T, N = g.n_text, g.n_hr
    D = qr.shape[1]
    dq = np.zeros_like(qr, dtype=np.float64)
    dk = np.zeros_like(kr, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    groups = []
    if T:
        groups.append(np.arange(T))
    if g.n_lr:
        groups.append(np.arange(T + N, g.seq_len))
    gy, gx = g.grid
    hr_rows = np.arange(T, T + N)
    for a in range(gy):
        for b in range(gx):
            groups.append(hr_rows[(wy[hr_rows] == a) & (wx[hr_rows] == b)])
    for rows in groups:
        if rows.size == 0:
            continue
        keys = allowed_keys_of(g, coords, int(rows[0]))
        p = _softmax_rows((qr[rows] @ kr[keys].T) / math.sqrt(D))
        dp = do[rows] @ v[keys].T
        delta = (p * dp).sum(axis=1)
        ds = p * (dp - delta[:, None])
        dq[rows] = ds @ kr[keys] / math.sqrt(D)
        dk[keys] += ds.T @ qr[rows] / math.sqrt(D)
        dv[keys] += p.T @ do[rows]
    return dq, dk, dv


def backward_head(g: Geometry, q, k, v, do, theta):
    """Full-layer backward of one head in raster order: (dq, dk, dv) with
    respect to the un-rotated q, k and v."""
    _, pr, pc, _, _ = token_coords(g)
    qr, kr = rope_rotate(q, pr, pc, theta), rope_rotate(k, pr, pc, theta)
    dqr, dkr, dv = attention_backward_grouped(g, qr, kr, v, do)
    return rope_rotate_transpose(dqr, pr, pc, theta), rope_rotate_transpose(dkr, pr, pc, theta), dv


def backward_query_rows(g: Geometry, q, k, v, do, theta, rows):
    """dq of selected raster rows of one head (each row needs only its own
    allowed keys)."""
    coords = token_coords(g)
    _, pr, pc, _, _ = coords
    rows = np.asarray(rows, np.int64)
    kr = rope_rotate(k, pr, pc, theta)
    qr = np.zeros_like(q, dtype=np.float64)
    qr[rows] = rope_rotate(q[rows], pr[rows], pc[rows], theta)
    D = q.shape[1]
    out = np.empty((rows.size, D))
    for idx, i in enumerate(rows):
        keys = allowed_keys_of(g, coords, int(i))
        p, _, o = _row_stats(qr, kr, v, int(i), keys)
        dp = v[keys] @ do[i]
        ds = p * (dp - do[i] @ o)
        out[idx] = ds @ kr[keys] / math.sqrt(D)
    return rope_rotate_transpose(out, pr[rows], pc[rows], theta)


def backward_key_rows(g: Geometry, q, k, v, do, theta, keys):
    """(dk, dv) of selected raster key rows of one head.  Every query that
    sees one of the keys needs its full softmax row (LSE and output)."""
    coords = token_coords(g)
    _, pr, pc, _, _ = coords
    keys = np.asarray(keys, np.int64)
    qr = rope_rotate(q, pr, pc, theta)
    kr = rope_rotate(k, pr, pc, theta)
    D = q.shape[1]
    cols = [allowed_queries_of(g, coords, int(j)) for j in keys]
    need = np.unique(np.concatenate(cols))
    lse, delta = {}, {}
    for i in need:
        kk = allowed_keys_of(g, coords, int(i))
        _, lse[int(i)], o = _row_stats(qr, kr, v, int(i), kk)
        delta[int(i)] = do[i] @ o
    dk = np.empty((keys.size, D))
    dv = np.empty((keys.size, D))
    for idx, (j, qs) in enumerate(zip(keys, cols)):
        s = (qr[qs] @ kr[j]) / math.sqrt(D)
        p = np.exp(s - np.array([lse[int(i)] for i in qs]))
        dp = do[qs] @ v[j]
        ds = p * (dp - np.array([delta[int(i)] for i in qs]))
        dk[idx] = ds @ qr[qs] / math.sqrt(D)
        dv[idx] = p @ do[qs]
    return rope_rotate_transpose(dk, pr[keys], pc[keys], theta), dv


# --------------------------------------------------------------------------
# Warm start ([KD4], R12): X_hr = alpha * noise + (1 - alpha) * sharpen(up(X_lr))
# on latents laid out [H, W, C] (HR) and [h, w, C] (LR), channels last.
# --------------------------------------------------------------------------

def upsample_bilinear(x_lr: np.ndarray, hr_h: int, hr_w: int, rho: int) -> np.ndarray:
    """U[r, c] = bilinear interpolation of x_lr at (r / rho, c / rho): LR
    sample (m, n) sits at HR (rho*m, rho*n); past the last LR row or column
    the last sample's value is kept."""
    h, w, C = x_lr.shape
    out = np.empty((hr_h, hr_w, C))
    for r in range(hr_h):
        y = r / rho
        y0 = min(int(math.floor(y)), h - 1)
        fy = y - y0 if y0 < h - 1 else 0.0
        y1 = min(y0 + 1, h - 1)
        for c in range(hr_w):
            x = c / rho
            x0 = min(int(math.floor(x)), w - 1)
            fx = x - x0 if x0 < w - 1 else 0.0
            x1 = min(x0 + 1, w - 1)
            out[r, c] = ((1 - fy) * ((1 - fx) * x_lr[y0, x0] + fx * x_lr[y0, x1]) +
                         fy * ((1 - fx) * x_lr[y1, x0] + fx * x_lr[y1, x1]))
    return out


def sharpen_unsharp(u: np.ndarray, strength: float) -> np.ndarray:
    """Unsharp masking u + s * (u - blur(u)), blur = 3x3 binomial kernel
    (outer product of [1, 2, 1] / 4) with replicated edges."""
    H, W, _ = u.shape
    b = (0.25, 0.5, 0.25)
    blur = np.zeros_like(u, dtype=np.float64)
    for dy in (-1, 0, 1):
        rows = np.clip(np.arange(H) + dy, 0, H - 1)
        for dx in (-1, 0, 1):
            cols = np.clip(np.arange(W) + dx, 0, W - 1)
            blur += b[dy + 1] * b[dx + 1] * u[rows][:, cols]
    return u + strength * (u - blur)


def warm_start(x_lr: np.ndarray, noise: np.ndarray, rho: int, alpha: float, strength: float) -> np.ndarray:
    """HR start latent at normalised time alpha = t/T for one image."""
    hr_h, hr_w, _ = noise.shape
    ref = sharpen_unsharp(upsample_bilinear(x_lr, hr_h, hr_w, rho), strength)
    return alpha * noise + (1.0 - alpha) * ref
