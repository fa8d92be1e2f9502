"""Plant one mistake at a time in a copy of the oracle's source (on the CPU)
and require the pins to catch every one.  This is what makes the pins worth
trusting: a dropped term, a wrong sign, a wrong index or axis, or a transposed
operand anywhere in the oracle fails at least one of them."""
import os
import types

import pytest

import oracle_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "attention.py")
DIST_SRC = os.path.join(ORACLE_DIR, "distance.py")
FP8_SRC = os.path.join(ORACLE_DIR, "fp8.py")

MUTANTS = [
    ("diagonal dropped from causal mask", "return cols <= rows", "return cols < rows"),
    ("causal mask reversed", "return cols <= rows", "return cols >= rows"),
    ("scale dropped", "s = scale * (q[r0:r1] @ k[:kend].T)", "s = (q[r0:r1] @ k[:kend].T)"),
    ("scale squared", "s = scale * (q[r0:r1] @ k[:kend].T)",
     "s = scale * scale * (q[r0:r1] @ k[:kend].T)"),
    ("keys in reverse order", "s = scale * (q[r0:r1] @ k[:kend].T)",
     "s = scale * (q[r0:r1] @ k[:kend][::-1].T)"),
    ("causal key range stops one short", "kend = r1 if causal else k.shape[0]",
     "kend = r1 - 1 if causal and r1 > 1 else (r1 if causal else k.shape[0])"),
    ("no max shift", "e = np.exp(s - m)", "e = np.exp(s)"),
    ("max over the wrong axis", "m = s.max(axis=1, keepdims=True)",
     "m = s.max(axis=0, keepdims=True)"),
    ("row sum over the wrong axis", "ell = e.sum(axis=1, keepdims=True)",
     "ell = e.sum(axis=0, keepdims=True)"),
    ("no normalisation", "p = e / ell", "p = e"),
    ("values shifted by one row", "o[r0:r1] = p @ v[:kend]",
     "o[r0:r1] = p @ np.roll(v[:kend], 1, axis=0)"),
    ("lse without log", "lse[r0:r1] = m[:, 0] + np.log(ell[:, 0])",
     "lse[r0:r1] = m[:, 0] + ell[:, 0]"),
    ("lse without max", "lse[r0:r1] = m[:, 0] + np.log(ell[:, 0])",
     "lse[r0:r1] = np.log(ell[:, 0])"),
    ("scale 1/d", "return 1.0 / math.sqrt(head_dim)", "return 1.0 / head_dim"),
    ("P rows normalised over columns", "return w / w.sum(axis=1, keepdims=True)",
     "return w / w.sum(axis=0, keepdims=True)"),
    ("P without max shift", "w = np.exp(s - top)", "w = np.exp(s - top.mean())"),
    ("int8 key scale dropped", "return scale * sq[r0:r1, None] * sk[None, :kend] * dots",
     "return scale * sq[r0:r1, None] * dots"),
    ("int8 scales swapped", "return scale * sq[r0:r1, None] * sk[None, :kend] * dots",
     "return scale * sk[r0:r1, None] * sq[None, :kend] * dots"),
    ("int8 scores transposed", "return np.rint(qf @ kt).astype(np.int64)",
     "return np.rint(kf @ np.swapaxes(qf, -1, -2)).astype(np.int64)"),
    ("quantiser truncates", "codes = np.clip(np.rint(ratio), -127.0, 127.0)",
     "codes = np.clip(np.trunc(ratio), -127.0, 127.0)"),
    ("quantiser rounds half away", "codes = np.clip(np.rint(ratio), -127.0, 127.0)",
     "codes = np.clip(np.sign(ratio) * np.floor(np.abs(ratio) + 0.5), -127.0, 127.0)"),
    ("quantiser divides by 128", "\n    scale = (absmax / np.float32(127.0))",
     "\n    scale = (absmax / np.float32(128.0))"),
    ("quantiser zero-row guard dropped",
     "\n    scale = np.where(scale == np.float32(0.0), np.float32(1.0), scale)",
     "\n    scale = np.where(scale == np.float32(0.0), np.float32(0.0), scale)"),
    ("quantiser clamps at 128", "codes = np.clip(np.rint(ratio), -127.0, 127.0)",
     "codes = np.clip(np.rint(ratio * np.float32(128.0 / 127.0)), -128.0, 127.0)"),
    ("signed mean takes |e|", "mean_signed=float(ef.sum() / n_fin)",
     "mean_signed=float(np.abs(ef).sum() / n_fin)"),
    ("argmax reports the last tie", "arg = int(np.argmax(a))",
     "arg = int(a.size - 1 - np.argmax(a[::-1]))"),
    ("mean over all n", "mean_abs=float(np.abs(ef).sum() / n_fin)",
     "mean_abs=float(np.abs(ef).sum() / n)"),
    ("rms without root", "rms=float(math.sqrt((ef * ef).sum() / n_fin))",
     "rms=float((ef * ef).sum() / n_fin)"),
    ("delta sums over rows", "return prod.sum(axis=-1)", "return prod.sum(axis=-2)"),
    ("delta drops the last column", "return prod.sum(axis=-1)",
     "return prod[..., :-1].sum(axis=-1)"),
    ("delta adds instead of multiplying", "prod = g64 * o64", "prod = g64 + o64"),
    ("delta squares O", "prod = g64 * o64", "prod = o64 * o64"),
    ("backward: dV without the transpose", "dv = p.T @ g", "dv = p @ g"),
    ("backward: dS sign flipped", "ds = p * (dp - delta[:, None])", "ds = p * (delta[:, None] - dp)"),
    ("backward: delta from O alone", "delta = (g * o).sum(axis=1)", "delta = (o * o).sum(axis=1)"),
    ("backward: delta from dO alone", "delta = (g * o).sum(axis=1)", "delta = (g * g).sum(axis=1)"),
    ("backward: dQ without the scale", "dq = scale * (ds @ k)", "dq = ds @ k"),
    ("backward: dK from dS, not its transpose", "dk = scale * (ds.T @ q)",
     "dk = scale * (ds @ q)"),
    ("backward: dP without V transposed", "dp = g @ v.T", "dp = g @ v[::-1].T"),
    ("tile scale from the first row only", "absmax = np.max(np.abs(tile), axis=(-2, -1))",
     "absmax = np.max(np.abs(tile[..., :1, :]), axis=(-2, -1))"),
    ("ragged last tile dropped", "for r0 in range(0, n, tile_rows):",
     "for r0 in range(0, max(n - tile_rows + 1, 1), tile_rows):"),
    ("tile scale divides by 128",
     "scale = (absmax / np.float32(127.0)).astype(np.float32)\n        scale = np.where",
     "scale = (absmax / np.float32(128.0)).astype(np.float32)\n        scale = np.where"),
    ("tile codes clamp at 128", "codes[..., r0:r1, :] = np.clip(np.rint(ratio), -127.0, 127.0)",
     "codes[..., r0:r1, :] = np.clip(np.rint(ratio * np.float32(128 / 127)), -128.0, 127.0)"),
]


DIST_MUTANTS = [
    ("quantiles not sorted", "return np.sort(a), bad", "return a, bad"),
    ("quantile index one late", "ia = -(-ends // m) - 1", "ia = np.minimum(-(-ends // m), n - 1)"),
    ("quantile indices from the wrong size", "ib = -(-ends // n) - 1", "ib = -(-ends // m) - 1"),
    ("interval widths dropped", "w1 = float((width * gap).sum())", "w1 = float(gap.mean())"),
    ("W2 without root", "w2 = float(math.sqrt((width * gap * gap).sum()))",
     "w2 = float((width * gap * gap).sum())"),
    ("W_inf as a mean", "winf = float(gap.max())", "winf = float(gap.mean())"),
    ("intervals start one step late", "starts = np.concatenate(([0], ends[:-1]))",
     "starts = np.concatenate(([0, 0], ends[:-2]))"),
    ("CDF counts strictly below", 'fa = np.searchsorted(a, z[:-1], side="right") / a.size',
     'fa = np.searchsorted(a, z[:-1], side="left") / a.size'),
    ("CDF difference without abs", "return float((np.diff(z) * np.abs(fa - fb)).sum())",
     "return float((np.diff(z) * (fa - fb)).sum())"),
    ("non-finite values ignored", "bad = int((~np.isfinite(a)).sum())", "bad = 0"),
]


FP8_MUTANTS = [
    ("E4M3 exponent bias 8", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)",
     "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    ("E4M3 subnormals one binade low", "return sign * (m / 8.0) * 2.0 ** -6",
     "return sign * (m / 8.0) * 2.0 ** -7"),
    ("E4M3 ties away from zero", "pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))",
     "pick_hi = (d_hi <= d_lo)"),
    ("E4M3 ties to odd", "pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))",
     "pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 1))"),
    ("E4M3 sign of -0 lost", "np.where(np.signbit(x), 0x80, 0)", "np.where(x < 0, 0x80, 0)"),
    ("E4M3 NaN not mapped", "code = np.where(np.isnan(x), 0x7F, code)", "code = code"),
    ("fp8 quantiser divides by 447", "scale = (absmax / np.float32(E4M3_MAX))",
     "scale = (absmax / np.float32(447.0))"),
    ("fp8 quantiser zero-row guard dropped",
     "scale = np.where(scale == np.float32(0.0), np.float32(1.0), scale)",
     "scale = np.where(scale == np.float32(0.0), np.float32(0.0), scale)"),
    ("fp8 key scale dropped", "return scale * sq[r0:r1, None] * sk[None, :kend] * dots",
     "return scale * sq[r0:r1, None] * dots"),
    ("fp8 scores transposed", "return qd @ np.swapaxes(kd, -1, -2)",
     "return kd @ np.swapaxes(qd, -1, -2)"),
]


def _mutant_module(old, new, path=SRC):
    """The oracle's modules in one namespace (their relative imports then
    resolve there), one of them mutated."""
    mod = types.ModuleType("oracle_mutant")
    for src_path in (SRC, DIST_SRC, FP8_SRC):
        src = open(src_path).read()
        if src_path == path:
            assert src.count(old) == 1, f"mutation site not unique: {old!r}"
            src = src.replace(old, new)
        src = "\n".join(line for line in src.split("\n") if not line.startswith("from ."))
        exec(compile(src, src_path + " (mutant)", "exec"), mod.__dict__)
    return mod


ALL_MUTANTS = [(n, o, w, SRC) for n, o, w in MUTANTS] + \
              [(n, o, w, DIST_SRC) for n, o, w in DIST_MUTANTS] + \
              [(n, o, w, FP8_SRC) for n, o, w in FP8_MUTANTS]


@pytest.mark.parametrize("name,old,new,path", ALL_MUTANTS, ids=[m[0] for m in ALL_MUTANTS])
def test_pins_catch_mutant(name, old, new, path):
    mod = _mutant_module(old, new, path)
    caught = []
    for check in oracle_pins.PINS:
        try:
            check(mod)
        except Exception as exc:               # AssertionError, or a crash
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin catches mutant: {name}"


def test_unmutated_copy_passes_all_pins():
    mod = _mutant_module("def default_scale", "def default_scale")
    for check in oracle_pins.PINS:
        check(mod)
    mod = _mutant_module("def wasserstein(", "def wasserstein(", DIST_SRC)
    for check in oracle_pins.PINS:
        check(mod)
    mod = _mutant_module("def e4m3_encode(", "def e4m3_encode(", FP8_SRC)
    for check in oracle_pins.PINS:
        check(mod)
