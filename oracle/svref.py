"""ctypes wrapper of the CPU oracle (oracle/libsvref.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py, never by the GPU library.  Inputs are numpy
arrays on the host: float32 logits, or bf16 logits given as their uint16 bit
patterns.
"""
import contextlib
import ctypes as C
import os

import numpy as np

from . import build as _build

SVREF_FP32, SVREF_BF16 = 0, 1
TOPP_TARGET_ONLY = 1

ROW_NONFINITE_LOGIT = 1 << 0
ROW_NO_FINITE = 1 << 1
ROW_BAD_TOKEN = 1 << 2
ROW_BAD_K = 1 << 3
ROW_BAD_TEMPERATURE = 1 << 4
ROW_BAD_TOP_P = 1 << 5
ROW_BAD_PAGES = 1 << 6
ROW_FREE_OVERFLOW = 1 << 7
ROW_BAD_ACCEPTED = 1 << 8

POISON_BF16 = 0xFFFF

_P = C.c_void_p


class VerifyArgs(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("k_max", C.c_int32), ("V", C.c_int32), ("dtype", C.c_int32),
        ("target", _P), ("target_vec_stride", C.c_int64),
        ("draft", _P), ("draft_vec_stride", C.c_int64),
        ("draft_tokens", _P), ("k_per_row", _P), ("temperature", _P), ("top_p", _P),
        ("seed", C.c_uint64), ("offset", C.c_uint64), ("flags", C.c_uint32),
        ("nthreads", C.c_int32), ("row_ids", _P),
        ("out_tokens", _P), ("accepted", _P), ("num_emitted", _P),
        ("p_at_draft", _P), ("q_at_draft", _P), ("row_status", _P),
        ("diag_rho", _P), ("diag_acc_margin", _P), ("diag_cdf_margin", _P),
        ("diag_topp_margin_t", _P), ("diag_topp_margin_d", _P),
        ("diag_residual_mass", _P),
        ("forced_accepted", _P), ("probe_token", _P), ("diag_probe", _P),
    ]


class RollbackArgs(C.Structure):
    _fields_ = [
        ("B", C.c_int32), ("k_max", C.c_int32), ("page_size", C.c_int32),
        ("max_pages_per_seq", C.c_int32),
        ("kv_len", _P), ("k_per_row", _P), ("accepted", _P), ("page_table", _P),
        ("num_pages", C.c_int32), ("free_pages", _P), ("free_top", _P), ("free_capacity", C.c_int32),
        ("kv_pool", _P), ("num_layers", C.c_int32), ("kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("row_status", _P),
    ]


class DynkArgs(C.Structure):
    _fields_ = [("B", C.c_int32), ("window", C.c_int32), ("k_min", C.c_int32), ("k_max", C.c_int32),
                ("up_num", C.c_int32), ("up_den", C.c_int32), ("down_num", C.c_int32),
                ("down_den", C.c_int32), ("accepted", _P), ("k_per_row", _P),
                ("hist_accepted", _P), ("hist_proposed", _P), ("hist_len", _P),
                ("capacity", C.c_int32)]


_lib = None


def load_library(path):
    """Loads an oracle build and declares its C signatures."""
    L = C.CDLL(path)
    L.svref_philox4x64_10.argtypes = [_P, _P, _P]
    L.svref_uniform.argtypes = [C.c_uint64] * 5
    L.svref_uniform.restype = C.c_double
    L.svref_softmax_topp.argtypes = [_P, C.c_int32, C.c_double, C.c_double,
                                     _P, _P, _P, _P]
    L.svref_softmax_topp.restype = C.c_int
    for f in (L.svref_verify_sample, L.svref_verify_greedy):
        f.argtypes = [C.POINTER(VerifyArgs)]
        f.restype = C.c_int
    L.svref_draft_sample.argtypes = [C.POINTER(VerifyArgs), _P]
    L.svref_draft_sample.restype = C.c_int
    L.svref_kv_rollback.argtypes = [C.POINTER(RollbackArgs)]
    L.svref_kv_rollback.restype = C.c_int
    L.svref_dynamic_k.argtypes = [C.POINTER(DynkArgs)]
    L.svref_dynamic_k.restype = C.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        _lib = load_library(_build.build(force=False))
    return _lib


@contextlib.contextmanager
def using_library(path):
    """Temporarily routes every call of this module to another build (used by
    the mutation test, which plants mistakes in copies of the oracle)."""
    global _lib
    saved = lib()
    _lib = load_library(path)
    try:
        yield
    finally:
        _lib = saved


def _ptr(a):
    return None if a is None else a.ctypes.data


def philox(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib().svref_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed, row, pos, draw, offset):
    return lib().svref_uniform(seed, row, pos, draw, offset)


def softmax_topp(z, T=1.0, top_p=1.0):
    """Returns (status, p', kept_mass G, mass_above, n_kept) for one vector."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    p = np.zeros_like(z)
    G = C.c_double(0)
    above = C.c_double(0)
    n = C.c_int64(0)
    st = lib().svref_softmax_topp(_ptr(z), z.size, float(T), float(top_p), _ptr(p),
                                  C.addressof(G), C.addressof(above), C.addressof(n))
    return st, p, G.value, above.value, n.value


def _logits(x):
    """numpy float32 -> (array, FP32); uint16 bf16 bit patterns -> (array, BF16)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, SVREF_FP32
    if x.dtype == np.uint16:
        return x, SVREF_BF16
    raise TypeError("logits must be float32 or uint16 (bf16 bits), got %s" % x.dtype)


def _verify_args(target, draft, draft_tokens, temperature, top_p, k_per_row,
                 seed, offset, flags, nthreads, V=None, row_ids=None):
    target, dt = _logits(target)
    B, K1, Vs = target.shape
    K = K1 - 1
    V = Vs if V is None else V
    keep = {"target": target}
    a = VerifyArgs()
    a.B, a.k_max, a.V, a.dtype = B, K, V, dt
    a.target, a.target_vec_stride = _ptr(target), Vs
    if draft is not None:
        draft, dd = _logits(draft)
        assert dd == dt and draft.shape[:2] == (B, K)
        keep["draft"] = draft
        a.draft, a.draft_vec_stride = _ptr(draft), draft.shape[2]
    if draft_tokens is not None:
        keep["tok"] = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, K)
        a.draft_tokens = _ptr(keep["tok"])
    if k_per_row is not None:
        keep["k"] = np.ascontiguousarray(k_per_row, dtype=np.int32).reshape(B)
        a.k_per_row = _ptr(keep["k"])
    if temperature is not None:
        keep["T"] = np.ascontiguousarray(np.broadcast_to(
            np.asarray(temperature, dtype=np.float32), (B,)))
        a.temperature = _ptr(keep["T"])
    if top_p is not None:
        keep["P"] = np.ascontiguousarray(np.broadcast_to(
            np.asarray(top_p, dtype=np.float32), (B,)))
        a.top_p = _ptr(keep["P"])
    a.seed, a.offset, a.flags = int(seed), int(offset), int(flags)
    a.nthreads = int(nthreads)
    if row_ids is not None:
        keep["rows"] = np.ascontiguousarray(row_ids, dtype=np.int32).reshape(B)
        a.row_ids = _ptr(keep["rows"])
    return a, keep, B, K


def _take(x, sel):
    if x is None:
        return None
    x = np.asarray(x)
    return x if x.ndim == 0 else x[sel]


def verify_sample(target, draft, draft_tokens, temperature, top_p=None,
                  k_per_row=None, seed=0, offset=0, flags=0, nthreads=1, V=None,
                  row_ids=None, forced_accepted=None, probe_token=None):
    """Sampled verification of every row; returns a dict of numpy outputs and
    the comparator diagnostics.  row_ids: the batch row index of each given
    row (for checking a subset of a batch).

    forced_accepted / probe_token ([B] int32): the what-if run -- the draw is
    taken where forced_accepted says, and "probe" [B][4] gives the probe
    token's interval {C_(t-1)/R, C_t/R, r_t/R, u} in the drawn distribution.
    The returned dict's "rerun"(forced, probe, sel) repeats the call on the
    rows `sel` (indices into this call's rows) with those inputs."""
    a, keep, B, K = _verify_args(target, draft, draft_tokens, temperature, top_p,
                                 k_per_row, seed, offset, flags, nthreads, V, row_ids)
    if forced_accepted is not None:
        keep["forced"] = np.ascontiguousarray(forced_accepted, dtype=np.int32).reshape(B)
        a.forced_accepted = _ptr(keep["forced"])
    if probe_token is not None:
        keep["probe"] = np.ascontiguousarray(probe_token, dtype=np.int32).reshape(B)
        a.probe_token = _ptr(keep["probe"])
    out = {
        "out_tokens": np.full((B, K + 1), -7, np.int32),
        "accepted": np.full(B, -7, np.int32),
        "num_emitted": np.full(B, -7, np.int32),
        "p_at_draft": np.full((B, K), np.nan),
        "q_at_draft": np.full((B, K), np.nan),
        "row_status": np.full(B, -7, np.int32),
        "rho": np.full((B, K), np.nan),
        "acc_margin": np.full((B, K), np.nan),
        "cdf_margin": np.full(B, np.inf),
        "topp_margin_t": np.full((B, K + 1), np.inf),
        "topp_margin_d": np.full((B, K), np.inf),
        "residual_mass": np.full(B, np.nan),
    }
    a.out_tokens, a.accepted = _ptr(out["out_tokens"]), _ptr(out["accepted"])
    a.num_emitted, a.row_status = _ptr(out["num_emitted"]), _ptr(out["row_status"])
    a.p_at_draft, a.q_at_draft = _ptr(out["p_at_draft"]), _ptr(out["q_at_draft"])
    a.diag_rho, a.diag_acc_margin = _ptr(out["rho"]), _ptr(out["acc_margin"])
    a.diag_cdf_margin = _ptr(out["cdf_margin"])
    a.diag_topp_margin_t = _ptr(out["topp_margin_t"])
    a.diag_topp_margin_d = _ptr(out["topp_margin_d"])
    a.diag_residual_mass = _ptr(out["residual_mass"])
    out["probe"] = np.full((B, 4), np.nan)
    a.diag_probe = _ptr(out["probe"])
    out["draft_tokens_in"] = keep["tok"].copy()
    rc = lib().svref_verify_sample(C.byref(a))
    if rc != 0:
        raise ValueError("svref_verify_sample rejected its arguments")

    def rerun(forced, probe, sel):
        sel = np.asarray(sel, dtype=np.int64)
        ids = sel if row_ids is None else np.asarray(row_ids)[sel]
        return verify_sample(_take(target, sel), _take(draft, sel), _take(draft_tokens, sel),
                             _take(temperature, sel), _take(top_p, sel),
                             _take(k_per_row, sel), seed, offset, flags, nthreads, V,
                             row_ids=ids, forced_accepted=forced, probe_token=probe)

    out["rerun"] = rerun
    return out


def verify_greedy(target, draft=None, draft_tokens=None, k_per_row=None, nthreads=1,
                  V=None):
    a, keep, B, K = _verify_args(target, draft, draft_tokens, None, None, k_per_row,
                                 0, 0, 0, nthreads, V)
    out = {
        "out_tokens": np.full((B, K + 1), -7, np.int32),
        "accepted": np.full(B, -7, np.int32),
        "num_emitted": np.full(B, -7, np.int32),
        "row_status": np.full(B, -7, np.int32),
    }
    a.out_tokens, a.accepted = _ptr(out["out_tokens"]), _ptr(out["accepted"])
    a.num_emitted, a.row_status = _ptr(out["num_emitted"]), _ptr(out["row_status"])
    rc = lib().svref_verify_greedy(C.byref(a))
    if rc != 0:
        raise ValueError("svref_verify_greedy rejected its arguments")
    return out


def draft_sample(draft, temperature, top_p=None, k_per_row=None, seed=0, offset=0,
                 flags=0, nthreads=1, V=None, diagnostics=False, probe_tokens=None,
                 row_ids=None):
    """Draft tokens x_i ~ q'_i with draw 2 (int32 [B][k_max]) and row status;
    with diagnostics=True also the CDF and top-p margins of every draw.
    probe_tokens ([B][k_max]): also returns, last, each probe token's
    interval {C_(t-1)/R, C_t/R, r_t/R, u} in q'_i ([B][k_max][4])."""
    draft, dt = _logits(draft)
    B, K, Vs = draft.shape
    # the argument block wants a target; point it at the draft (unused here)
    a, keep, _, _ = _verify_args(np.zeros((B, K + 1, 1), draft.dtype), None, None,
                                 temperature, top_p, k_per_row, seed, offset, flags,
                                 nthreads, row_ids=row_ids)
    a.V = Vs if V is None else V
    a.draft, a.draft_vec_stride = _ptr(draft), Vs
    a.dtype = dt
    toks = np.full((B, K), -7, np.int32)
    st = np.full(B, -7, np.int32)
    a.row_status = _ptr(st)
    cdf = np.full((B, K), np.inf)
    topp = np.full((B, K), np.inf)
    a.diag_acc_margin, a.diag_topp_margin_d = _ptr(cdf), _ptr(topp)
    probe = None
    if probe_tokens is not None:
        keep["probe"] = np.ascontiguousarray(probe_tokens, dtype=np.int32).reshape(B, K)
        a.probe_token = _ptr(keep["probe"])
        probe = np.full((B, K, 4), np.nan)
        a.diag_probe = _ptr(probe)
    rc = lib().svref_draft_sample(C.byref(a), _ptr(toks))
    if rc != 0:
        raise ValueError("svref_draft_sample rejected its arguments")
    res = (toks, st) + ((cdf, topp) if diagnostics else ())
    return res + (probe,) if probe is not None else res


def kv_rollback(kv_len, accepted, page_table, page_size, k_max, k_per_row=None,
                free_pages=None, free_top=None, free_capacity=0, kv_pool=None,
                num_layers=0, kv_heads=0, head_dim=0, num_pages=0):
    """Runs the oracle rollback IN PLACE on the given numpy arrays; returns the
    row status array."""
    B = kv_len.shape[0]
    a = RollbackArgs()
    a.B, a.k_max, a.page_size = B, k_max, page_size
    a.max_pages_per_seq = page_table.shape[1]
    for arr in (kv_len, accepted, page_table):
        assert arr.dtype == np.int32 and arr.flags.c_contiguous
    a.kv_len, a.accepted, a.page_table = _ptr(kv_len), _ptr(accepted), _ptr(page_table)
    a.num_pages = int(num_pages if kv_pool is None or num_pages else kv_pool.shape[0])
    keep = []
    if k_per_row is not None:
        kp = np.ascontiguousarray(k_per_row, dtype=np.int32)
        keep.append(kp)
        a.k_per_row = _ptr(kp)
    if free_pages is not None:
        assert free_pages.dtype == np.int32 and free_top.dtype == np.int32
        a.free_pages, a.free_top = _ptr(free_pages), _ptr(free_top)
        a.free_capacity = int(free_capacity)
    if kv_pool is not None:
        assert kv_pool.dtype == np.uint16 and kv_pool.flags.c_contiguous
        a.kv_pool = _ptr(kv_pool)
        a.num_layers, a.kv_heads, a.head_dim = num_layers, kv_heads, head_dim
    st = np.full(B, -7, np.int32)
    a.row_status = _ptr(st)
    rc = lib().svref_kv_rollback(C.byref(a))
    if rc != 0:
        raise ValueError("svref_kv_rollback rejected its arguments")
    return st


class DynkHistory:
    """The controller's per-row history (oracle form): the accepted count and
    proposed k of every round recorded so far, oldest first."""

    def __init__(self, B, capacity):
        self.accepted = np.zeros((B, capacity), np.int32)
        self.proposed = np.zeros((B, capacity), np.int32)
        self.length = np.zeros(B, np.int32)

    def windows(self, W):
        """Every row's last min(W, rounds) rounds as [B][W] accepted and
        proposed arrays (oldest first, -1 past the row's count) and the
        counts."""
        B = self.length.shape[0]
        n = np.minimum(self.length, W)
        acc = np.full((B, W), -1, np.int32)
        prop = np.full((B, W), -1, np.int32)
        for b in range(B):
            L = int(self.length[b])
            acc[b, :n[b]] = self.accepted[b, L - n[b]:L]
            prop[b, :n[b]] = self.proposed[b, L - n[b]:L]
        return acc, prop, n

    def window(self, b, W):
        """The last min(W, rounds) (accepted, proposed) pairs of row b, oldest first."""
        n = int(self.length[b])
        s = max(0, n - W)
        return list(zip(self.accepted[b, s:n].tolist(), self.proposed[b, s:n].tolist()))


def dynamic_k(accepted, k_per_row, hist, window=64, k_min=2, k_max=8, up=(17, 20),
              down=(7, 10)):
    """One controller update, IN PLACE on k_per_row (numpy int32) and the
    DynkHistory `hist`."""
    B = k_per_row.shape[0]
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    assert k_per_row.dtype == np.int32 and k_per_row.flags.c_contiguous
    assert hist.accepted.shape[0] == B
    a = DynkArgs(B, window, k_min, k_max, up[0], up[1], down[0], down[1], _ptr(acc),
                 _ptr(k_per_row), _ptr(hist.accepted), _ptr(hist.proposed), _ptr(hist.length),
                 hist.accepted.shape[1])
    if lib().svref_dynamic_k(C.byref(a)) != 0:
        raise ValueError("svref_dynamic_k rejected its arguments")
