"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks
that the pins catch every one of them: a pin set that a wrong oracle passes
would pin nothing."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from pins import ALL_PINS

SRC = open(obuild.SRC).read()

MUTANTS = {
    # decay of token t taken from the previous token's dt
    "decay_index": ("const double decay = exp(dtt * A[h]);",
                    "const double decay = exp(dt[(size_t)(t > t0 ? t - 1 : t) * H + h] * A[h]);"),
    # wrong sign of A
    "sign_A": ("const double decay = exp(dtt * A[h]);",
               "const double decay = exp(-dtt * A[h]);"),
    # skip term dropped
    "drop_D": ("yt[p] += acc + Dh * xt[p];", "yt[p] += acc;"),
    # dt dropped from the input term
    "drop_dt_input": ("hp[n] = decay * hp[n] + dtt * Bt[n] * xt[p];",
                      "hp[n] = decay * hp[n] + Bt[n] * xt[p];"),
    # B and C exchanged
    "swap_BC": ("const double *Bt = B + ((size_t)t * G + g) * N;\n        const double *Ct = C + ((size_t)t * G + g) * N;",
                "const double *Bt = C + ((size_t)t * G + g) * N;\n        const double *Ct = B + ((size_t)t * G + g) * N;"),
    # reverse stream not reversed
    "no_reverse": ("const int t = reverse ? (t1 - 1 - step) : (t0 + step);",
                   "const int t = t0 + step;"),
    # output read before the state update (y_t from h_{t-1})
    "stale_output": ("                hp[n] = decay * hp[n] + dtt * Bt[n] * xt[p];\n                acc += Ct[n] * hp[n];",
                     "                acc += Ct[n] * hp[n];\n                hp[n] = decay * hp[n] + dtt * Bt[n] * xt[p];"),
    # wrong head -> group map
    "group_map": ("const int g = h / (H / G);", "const int g = h % G;"),
    # state layout [n][p] instead of [p][n]
    "state_layout": ("hp[n] = decay * hp[n] + dtt * Bt[n] * xt[p];\n                acc += Ct[n] * hp[n];",
                     "state[(size_t)n * P + p] = decay * state[(size_t)n * P + p] + dtt * Bt[n] * xt[p];\n                acc += Ct[n] * state[(size_t)n * P + p];"),
    # reverse stream starts from the forward stream's final state
    "no_reset_between": ("            if (xb) {\n                memset(state, 0, sizeof(double) * sz);",
                         "            if (xb) {"),
    # merge by subtraction instead of addition
    "merge_sub": ("scan_one_head(1, t0, t1, h, H, P, N, G, xb + xo, dtb + to, Ab,",
                  "scan_one_head(1, t0, t1, h, H, P, N, G, xb + xo, dtb + to, Ab,"),
}


def _mutant_src(name):
    a, b = MUTANTS[name]
    assert a in SRC, f"mutation site for {name} not found"
    if name == "merge_sub":
        # negate the reverse stream's contribution
        return SRC.replace("            yt[p] += acc + Dh * xt[p];",
                           "            yt[p] += (reverse ? -1.0 : 1.0) * (acc + Dh * xt[p]);")
    return SRC.replace(a, b)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = tmp_path / "mutant.c"
    text = _mutant_src(name)
    assert text != SRC, f"mutation {name} changed nothing"
    src.write_text(text)
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    str(src), "-o", lib_path, "-lm"], check=True)
    lib = oracle.bind(lib_path)
    caught = []
    with np.errstate(all="ignore"):
        for pin, (fn, tol) in ALL_PINS.items():
            try:
                err = fn(lib)
            except Exception:
                caught.append(pin)
                continue
            if not (err <= tol):
                caught.append(pin)
    assert caught, f"no pin catches mutant {name}"


CONV_SRC = open(os.path.join(os.path.dirname(oracle.__file__), "conv.py")).read()

CONV_MUTANTS = {
    # forward taps applied in the wrong order (filter not reversed in time)
    "conv_tap_order": ("            src = padded[k:k + T]",
                       "            src = padded[W - 1 - k:W - 1 - k + T]"),
    # reverse direction uses the forward (causal) window
    "conv_reverse_window": ("            src = padded[W - 1 - k:W - 1 - k + T]",
                            "            src = padded[k:k + T]"),
    # bias dropped
    "conv_drop_bias": ("    out = np.zeros((T, ch)) if bias is None else np.tile(bias, (T, 1))",
                       "    out = np.zeros((T, ch))"),
    # SiLU with the wrong sign inside the exponential
    "conv_silu_sign": ("return v / (1.0 + np.exp(-v))", "return v / (1.0 + np.exp(v))"),
    # taps shifted one token into the past
    "conv_shift": ("        head = np.zeros((W - 1, ch)) if ctx is None else ctx",
                   "        head = np.zeros((W, ch)) if ctx is None else np.concatenate([np.zeros((1, ch)), ctx])"),
    # carried context ignored
    "conv_ignore_ctx": ("        head = np.zeros((W - 1, ch)) if ctx is None else ctx",
                        "        head = np.zeros((W - 1, ch))"),
    # final context written newest first
    "conv_final_order": ("        final[r] = seq[seq.shape[0] - (W - 1):]",
                         "        final[r] = seq[seq.shape[0] - (W - 1):][::-1]"),
    # packed sequences see their neighbours
    "conv_packed_leak": ("                out[0, a:e] = _filter_row(u[0, a:e], w, b, reverse, None)",
                         "                out[0, a:e] = _filter_row(u[0], w, b, reverse, None)[a:e]"),
    # x, B and C split in the wrong order
    "conv_split_order": ("            out[..., hp:hp + gn].reshape(batch, L, ngroups, d_state),\n            out[..., hp + gn:]",
                         "            out[..., hp + gn:].reshape(batch, L, ngroups, d_state),\n            out[..., hp:hp + gn]"),
}


@pytest.mark.parametrize("name", sorted(CONV_MUTANTS))
def test_conv_pins_catch_mutant(name):
    import types
    from conv_pins import CONV_PINS
    a, b = CONV_MUTANTS[name]
    assert CONV_SRC.count(a) == 1, f"mutation site for {name} not found once"
    mod = types.ModuleType("conv_mutant")
    exec(compile(CONV_SRC.replace(a, b), "conv_mutant.py", "exec"), mod.__dict__)
    caught = []
    with np.errstate(all="ignore"):
        for pin, (fn, tol) in CONV_PINS.items():
            try:
                err = fn(mod)
            except Exception:
                caught.append(pin)
                continue
            if not (err <= tol):
                caught.append(pin)
    assert caught, f"no pin catches mutant {name}"


BWD_MUTANTS = {
    # the gradient of h_t propagated before the token's own output term
    "bwd_order": ("                gp[n] += Ct[n] * dyt[p];\n",
                  "                gp[n] = decay * gp[n] + Ct[n] * dyt[p];\n"),
    # decay term of ddt dropped
    "bwd_ddt_decay": ("ddt[(size_t)t * H + h] = r + A[h] * decay * q;",
                      "ddt[(size_t)t * H + h] = r;"),
    # <g_t, h_t> used where <g_t, h_{t-1}> belongs
    "bwd_q_current": ("                    q += gp[n] * prev[(size_t)p * N + n];",
                      "                    q += gp[n] * cur[(size_t)p * N + n];"),
    # dt missing from dB
    "bwd_dB_dt": ("dBt[n] += dtt * gp[n] * xt[p];", "dBt[n] += gp[n] * xt[p];"),
    # skip term missing from dx
    "bwd_dx_D": ("dx[((size_t)t * H + h) * P + p] = Dh * dyt[p] + dtt * gb;",
                 "dx[((size_t)t * H + h) * P + p] = dtt * gb;"),
    # dt missing from dA
    "bwd_dA_dt": ("*dA += dtt * decay * q;", "*dA += decay * q;"),
    # dC from h_{t-1}
    "bwd_dC_prev": ("dCt[n] += cur[(size_t)p * N + n] * dyt[p];",
                    "dCt[n] += (prev ? prev[(size_t)p * N + n] : 0.0) * dyt[p];"),
    # the reverse stream's gradient walked in the forward order
    "bwd_no_reverse": ("        const int t = reverse ? (t1 - 1 - step) : (t0 + step);\n        const double dtt = dt[(size_t)t * H + h];\n        const double decay = exp(dtt * A[h]);\n        const double *Bt = B + ((size_t)t * G + g) * N;\n        const double *xt = x + ((size_t)t * H + h) * P;\n        const double *prev",
                       "        const int t = t0 + step;\n        const double dtt = dt[(size_t)t * H + h];\n        const double decay = exp(dtt * A[h]);\n        const double *Bt = B + ((size_t)t * G + g) * N;\n        const double *xt = x + ((size_t)t * H + h) * P;\n        const double *prev"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_pins_catch_mutant(name, tmp_path):
    from bwd_pins import BWD_PINS
    a, b = BWD_MUTANTS[name]
    assert SRC.count(a) == 1, f"mutation site for {name} not found once"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(a, b))
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    str(src), "-o", lib_path, "-lm"], check=True)
    lib = oracle.bind(lib_path)
    caught = []
    with np.errstate(all="ignore"):
        for pin, (fn, tol) in BWD_PINS.items():
            if pin == "bwd_finite_differences":
                continue  # slow; the others must catch every mutant on their own
            try:
                err = fn(lib)
            except Exception:
                caught.append(pin)
                continue
            if not (err <= tol):
                caught.append(pin)
    assert caught, f"no pin catches mutant {name}"


EPI_SRC = open(os.path.join(os.path.dirname(oracle.__file__), "epilogue.py")).read()

EPI_MUTANTS = {
    # eps added outside the square root
    "epi_eps_outside": ("part / np.sqrt(ms + eps)", "part / (np.sqrt(ms) + eps)"),
    # the gate dropped
    "epi_no_gate": ("    v = y * silu(z)\n", "    v = y\n"),
    # the gate's sigmoid without the factor z
    "epi_sigmoid_gate": ("return u / (1.0 + np.exp(-u))", "return 1.0 / (1.0 + np.exp(-u))"),
    # mean over the whole row instead of the group
    "epi_whole_row": ("ms = np.mean(part * part, axis=-1, keepdims=True)",
                      "ms = np.mean(v * v, axis=-1, keepdims=True)"),
    # per-channel weight dropped
    "epi_no_weight": (" * w[g0:g0 + group_size]", ""),
    # sum of squares instead of their mean
    "epi_sum_not_mean": ("ms = np.mean(part * part, axis=-1, keepdims=True)",
                         "ms = np.sum(part * part, axis=-1, keepdims=True)"),
}


@pytest.mark.parametrize("name", sorted(EPI_MUTANTS))
def test_epilogue_pins_catch_mutant(name):
    import types
    from epilogue_pins import EPILOGUE_PINS
    a, b = EPI_MUTANTS[name]
    assert EPI_SRC.count(a) == 1, f"mutation site for {name} not found once"
    mod = types.ModuleType("epilogue_mutant")
    exec(compile(EPI_SRC.replace(a, b), "epilogue_mutant.py", "exec"), mod.__dict__)
    caught = []
    with np.errstate(all="ignore"):
        for pin, (fn, tol) in EPILOGUE_PINS.items():
            try:
                err = fn(mod)
            except Exception:
                caught.append(pin)
                continue
            if not (err <= tol):
                caught.append(pin)
    assert caught, f"no pin catches mutant {name}"


DT_SRC = open(os.path.join(os.path.dirname(oracle.__file__), "dt.py")).read()

DT_MUTANTS = {
    # the naive form: overflows, loses very negative inputs
    "dt_naive": ("return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))",
                 "return np.log(1.0 + np.exp(v))"),
    # bias subtracted
    "dt_bias_sign": ("raw = raw + _f64(bias)", "raw = raw - _f64(bias)"),
    # exp instead of softplus
    "dt_exp": ("return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))", "return np.exp(v)"),
}


@pytest.mark.parametrize("name", sorted(DT_MUTANTS))
def test_dt_pins_catch_mutant(name):
    import types
    from epilogue_pins import DT_PINS
    a, b = DT_MUTANTS[name]
    assert DT_SRC.count(a) == 1, f"mutation site for {name} not found once"
    mod = types.ModuleType("dt_mutant")
    exec(compile(DT_SRC.replace(a, b), "dt_mutant.py", "exec"), mod.__dict__)
    caught = []
    with np.errstate(all="ignore"):
        for pin, (fn, tol) in DT_PINS.items():
            try:
                err = fn(mod)
            except Exception:
                caught.append(pin)
                continue
            if not (err <= tol):
                caught.append(pin)
    assert caught, f"no pin catches mutant {name}"


MERGE_SRC = open(os.path.join(os.path.dirname(oracle.__file__), "merge.py")).read()

MERGE_MUTANTS = {
    # the streams concatenated in the other order
    "merge_order": ("cat = np.concatenate([yf, yb], axis=-1)", "cat = np.concatenate([yb, yf], axis=-1)"),
    # bias dropped
    "merge_no_bias": ("        out = out + b\n", "        out = out\n"),
    # the streams summed instead of concatenated (first half of W only)
    "merge_sum": ("    cat = np.concatenate([yf, yb], axis=-1)\n    out = cat @ w.T\n",
                  "    out = (yf + yb) @ w[:, :yf.shape[-1]].T\n"),
}


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_pins_catch_mutant(name):
    import types
    from epilogue_pins import MERGE_PINS
    a, b = MERGE_MUTANTS[name]
    assert MERGE_SRC.count(a) == 1, f"mutation site for {name} not found once"
    mod = types.ModuleType("merge_mutant")
    exec(compile(MERGE_SRC.replace(a, b), "merge_mutant.py", "exec"), mod.__dict__)
    caught = []
    with np.errstate(all="ignore"):
        for pin, (fn, tol) in MERGE_PINS.items():
            try:
                err = fn(mod)
            except Exception:
                caught.append(pin)
                continue
            if not (err <= tol):
                caught.append(pin)
    assert caught, f"no pin catches mutant {name}"
