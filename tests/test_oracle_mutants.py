"""Plant plausible mistakes in copies of the oracle (CPU only) and check that
the pin suite catches every one of them.

Each mutant is the oracle's C source with one textual change, compiled into a
temporary directory and exercised in a child process (a mutant that indexes
out of bounds may crash; a crash counts as caught).  The real oracle is never
modified.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "fastvim_oracle.c")

# (name, original text, replacement, occurrences)
MUTANTS = [
    ("A sign flipped", "const double A = -exp((double)A_log[e * N + n]);\n                    const double a = (reset",
     "const double A = exp((double)A_log[e * N + n]);\n                    const double a = (reset", 1),
    ("output taken before the state update",
     "H[n] = a * H[n] + d * vt[R + n] * ut;\n                    acc += vt[R + N + n] * H[n];",
     "acc += vt[R + N + n] * H[n];\n                    H[n] = a * H[n] + d * vt[R + n] * ut;", 1),
    ("delta dropped from the input term", "H[n] = a * H[n] + d * vt[R + n] * ut;",
     "H[n] = a * H[n] + vt[R + n] * ut;", 1),
    ("input term dropped u", "H[n] = a * H[n] + d * vt[R + n] * ut;", "H[n] = a * H[n] + d * vt[R + n];", 1),
    ("B and C swapped", "H[n] = a * H[n] + d * vt[R + n] * ut;\n                    acc += vt[R + N + n] * H[n];",
     "H[n] = a * H[n] + d * vt[R + N + n] * ut;\n                    acc += vt[R + n] * H[n];", 1),
    ("delta not in the decay", "? 0.0 : exp(d * A)", "? 0.0 : exp(A)", 1),
    ("backward scan not reversed", "reverse ? T - 1 - step : step", "step", 1),
    ("dense pool not normalised", "        for (int64_t k = 0; k < T * E; ++k) ub[k] /= (double)P;\n    }\n}\n\n/*\n * Producer side",
     "    }\n}\n\n/*\n * Producer side", 1),
    ("masked pool normalised by K", "            for (int64_t e = 0; e < E; ++e) ub[t * E + e] += xd ? xd[c + e] : (double)x[c + e];\n        }\n        for (int64_t k = 0; k < T * E; ++k) ub[k] /= (double)P;",
     "            for (int64_t e = 0; e < E; ++e) ub[t * E + e] += xd ? xd[c + e] : (double)x[c + e];\n        }\n        for (int64_t k = 0; k < T * E; ++k) ub[k] /= (double)K;", 1),
    ("only the forward D in the skip", "((double)pf->D[e] + (double)pb->D[e])", "((double)pf->D[e])", 1),
    ("gate uses sigmoid(-z)", "return q / (1.0 + exp(-q));", "return q / (1.0 + exp(q));", 1),
    ("softplus without log", "log1p(exp(-fabs(q)))", "exp(-fabs(q))", 1),
    ("dt_proj transposed", "q += (double)dt_proj_w[e * R + r]", "q += (double)dt_proj_w[r * E + e]", 1),
    ("x_proj transposed", "acc += (double)x_proj_w[o * E + e]", "acc += (double)x_proj_w[e * NX + o]", 1),
    ("ROWS pooling scans rows", "case FVO_ROWS: return j;", "case FVO_ROWS: return i;", 1),
    ("column-major uses w", "default: return j * h + i;", "default: return j * w + i;", 1),
    ("masked ROWS uses the row", "q / w : q % w", "q / w : q / w", 1),
    ("bias dropped from delta", "double q = (double)dt_proj_b[e];", "double q = 0.0;", 1),
    ("low-rank delta reads B", "q += (double)dt_proj_w[e * R + r] * v[m * NX + r]",
     "q += (double)dt_proj_w[e * R + r] * v[m * NX + R + r]", 1),
    ("repeat uses the wrong direction sum", "y[e] = sf[e] + sb[e] + skip;", "y[e] = sf[e] + sf[e] + skip;", 1),
    ("repeat reads the wrong scan row", "output_token(sf + (b * T + t) * E, sb + (b * T + t) * E, x + c",
     "output_token(sf + (b * T + t / 2) * E, sb + (b * T + t / 2) * E, x + c", 2),
    ("LayerNorm with the unbiased variance", "var /= (double)E;", "var /= (double)(E - 1);", 1),
    ("LayerNorm eps outside the root", "1.0 / sqrt(var + ln_eps)", "1.0 / (sqrt(var) + ln_eps)", 1),
    ("LayerNorm without centring", "y[e] = (y[e] - mean) * r", "y[e] = y[e] * r", 1),
    ("LayerNorm scale and shift swapped", "* (double)ln_w[e] + (double)ln_b[e]", "* (double)ln_b[e] + (double)ln_w[e]", 1),
    ("pool scale not applied", "    for (int64_t i = 0; i < M * E; ++i) u[i] *= pool_scale;\n\n    rc = run_direction",
     "\n    rc = run_direction", 1),
    ("pool scale applied as a divisor", "    for (int64_t i = 0; i < M * E; ++i) u[i] *= pool_scale;\n\n    rc = run_direction",
     "    for (int64_t i = 0; i < M * E; ++i) u[i] /= pool_scale;\n\n    rc = run_direction", 1),
    ("backward recomputes u without the pool scale",
     "    for (int64_t i = 0; i < M * E; ++i) u[i] *= pool_scale;\n    for (int d = 0; d < 2; ++d) {",
     "    for (int d = 0; d < 2; ++d) {", 1),
    ("reset ignored", "(reset && reset[t]) ? 0.0 : exp(d * A)", "exp(d * A)", 1),
    ("duplicate mask index accepted", "if (q < 0 || q >= h * w || seen[q])", "if (q < 0 || q >= h * w)", 1),
    # producer Conv1D
    ("conv taps reversed", "acc += (double)conv_w[e * KC + k] *", "acc += (double)conv_w[e * KC + (KC - 1 - k)] *", 1),
    ("conv centred instead of causal", "const int64_t rr = r - KC + 1 + k;\n                    if (rr < 0) continue;",
     "const int64_t rr = r - KC / 2 + k;\n                    if (rr < 0 || rr >= n) continue;", 1),
    ("conv without its bias", "double acc = (double)conv_b[e];", "double acc = 0.0;", 1),
    ("conv without SiLU", "xc[(b * n + cell) * E + e] = acc / (1.0 + exp(-acc));", "xc[(b * n + cell) * E + e] = acc;", 1),
    ("conv row-major on the transposed grid", "const int colmajor = axis == FVO_ROWS || axis == FVO_NONE_COLMAJOR;",
     "const int colmajor = axis == FVO_NONE_COLMAJOR;", 1),
    ("skip reads the conv's input", "(xd ? xd[e] : (double)x[e])", "((double)x[e])", 1),
    ("pool reads the conv's input", "xd ? xd[c + e] : (double)x[c + e];\n            }",
     "(double)x[c + e];\n            }", 1),
    # LBMamba local backward scan
    ("local windows aligned one step late", "reset[t] = (unsigned char)(t % local_window == local_window - 1);",
     "reset[t] = (unsigned char)(t % local_window == 0);", 1),
    ("local windows never reset", "rc = run_direction(u, B, T, E, N, R, &pl, 1, reset, bwd, sb);",
     "rc = run_direction(u, B, T, E, N, R, &pl, 1, NULL, bwd, sb);", 1),
    ("local scan reads the backward projection", "const fvo_dir pl = {pf->x_proj_w, pf->dt_proj_w,",
     "const fvo_dir pl = {pb->x_proj_w, pf->dt_proj_w,", 1),
    ("local scan runs forward", "rc = run_direction(u, B, T, E, N, R, &pl, 1, reset, bwd, sb);",
     "rc = run_direction(u, B, T, E, N, R, &pl, 0, reset, bwd, sb);", 1),
    # backward pass
    ("adjoint carried without the decay", "carry[n] = a * lam[n];", "carry[n] = lam[n];", 1),
    ("adjoint decay term with the wrong sign", "dd += lam[n] * (A * a * prev + Bn * ut);",
     "dd += lam[n] * (-A * a * prev + Bn * ut);", 1),
    ("step-size adjoint without the decay term", "dd += lam[n] * (A * a * prev + Bn * ut);",
     "dd += lam[n] * (Bn * ut);", 1),
    ("dC from the previous state", "dv[m * NX + R + N + n] += g * Hs[k * N + n];",
     "dv[m * NX + R + N + n] += g * prev;", 1),
    ("dB without u", "dv[m * NX + R + n] += lam[n] * d * ut;", "dv[m * NX + R + n] += lam[n] * d;", 1),
    ("dA without delta", "dA[e * N + n] += lam[n] * a * d * prev;", "dA[e * N + n] += lam[n] * a * prev;", 1),
    ("dA_log chain factor dropped", "o->A_log[i] *= -exp((double)pd[d]->A_log[i]);", "o->A_log[i] *= -1.0;", 1),
    ("softplus derivative taken as exp", "ddelta[m * E + e] * sigmoid(q[m * E + e])",
     "ddelta[m * E + e] * exp(q[m * E + e])", 1),
    ("dW_dt reads B", "dWdt[e * R + r] += dq * v[m * NX + r];", "dWdt[e * R + r] += dq * v[m * NX + R + r];", 1),
    ("dt_proj adjoint does not reach dv", "dv[m * NX + r] += (double)dt_proj_w[e * R + r] * dq;", "(void)dv;", 1),
    ("x_proj adjoint does not reach du", "du[m * E + e] += (double)x_proj_w[o * E + e] * dv[m * NX + o];",
     "(void)du;", 1),
    ("pool adjoint not normalised", "du[mt + e] * pool_scale / (double)P", "du[mt + e] * pool_scale", 1),
    ("pool adjoint without the pool scale", "du[mt + e] * pool_scale / (double)P", "du[mt + e] / (double)P", 1),
    ("silu derivative without its second term", "sg * (1.0 + ze * (1.0 - sg))", "sg", 2),
    ("dz without the skip", "const double y = sf[e] + sb[e] + Ds * xe;", "const double y = sf[e] + sb[e];", 1),
    ("dD of the backward direction zero", "o->D[e] = dD[e];", "o->D[e] = d == 0 ? dD[e] : 0.0;", 1),
    ("scan adjoint fed dout without the gate", "g[e] = de * silu(ze);", "g[e] = de;", 1),
    ("backward direction's adjoint not reversed", "pd[d]->A_log, d, d == 1 ? reset : NULL, du, dd",
     "pd[d]->A_log, 0, d == 1 ? reset : NULL, du, dd", 1),
    ("dx without the skip", "dx[off + e] = dxs[off + e] + du[mt + e] * pool_scale / (double)P;",
     "dx[off + e] = du[mt + e] * pool_scale / (double)P;", 1),
    ("du of the scan without B", "duk += lam[n] * d * Bn;", "duk += lam[n] * d;", 1),
    # backward pass through the post-SSM LayerNorm
    ("LayerNorm adjoint without the mean of dn", "g[e] = r * (g[e] - m1 - ny[e] * m2);",
     "g[e] = r * (g[e] - ny[e] * m2);", 1),
    ("LayerNorm adjoint without the variance term", "g[e] = r * (g[e] - m1 - ny[e] * m2);",
     "g[e] = r * (g[e] - m1);", 1),
    ("LayerNorm adjoint without the scale r", "g[e] = r * (g[e] - m1 - ny[e] * m2);",
     "g[e] = g[e] - m1 - ny[e] * m2;", 1),
    ("LayerNorm adjoint with the unbiased variance", "sqrt(var / (double)E + ln_eps)",
     "sqrt(var / (double)(E - 1) + ln_eps)", 1),
    ("LayerNorm weight gradient without the normalised value", "dln_w[e] += go * ny[e];", "dln_w[e] += go;", 1),
    ("LayerNorm bias gradient without the gate", "dln_b[e] += go;", "dln_b[e] += de;", 1),
    ("LayerNorm adjoint without its weight", "g[e] = go * (double)ln_w[e];", "g[e] = go;", 1),
    ("LayerNorm adjoint's skip with only the forward D",
     "const double Ds = (double)pf->D[e] + (double)pb->D[e];\n        g[e] = r",
     "const double Ds = (double)pf->D[e];\n        g[e] = r", 1),
    ("LayerNorm adjoint's recomputed input without the skip",
     "ny[e] = sf[e] + sb[e] + Ds * xe;", "ny[e] = sf[e] + sb[e];", 1),
    ("dz through the norm without its affine map", "dz[e] = de * o * sg", "dz[e] = de * ny[e] * sg", 1),
    # backward pass of the local backward scan
    ("adjoint's state recompute ignores the reset",
     "const double a = (reset && reset[t]) ? 0.0 : exp(delta[m * E + e] * A);",
     "const double a = exp(delta[m * E + e] * A);", 1),
    ("adjoint's reverse sweep ignores the reset", "const double a = reset && reset[t] ? 0.0 : exp(A * d);",
     "const double a = exp(A * d);", 1),
    ("backward's local windows aligned one step early", "reset[t] = (unsigned char)((t + 1) % local_window == 0);",
     "reset[t] = (unsigned char)(t % local_window == 0);", 1),
    ("local scan's x_proj gradient not added to the forward set",
     "gf->x_proj_w[i] += gb->x_proj_w[i]; gb->x_proj_w[i] = 0.0;", "gb->x_proj_w[i] = 0.0;", 1),
    ("local scan's A_log gradient left in the backward set",
     "gf->A_log[i] += gb->A_log[i]; gb->A_log[i] = 0.0;", "gf->A_log[i] += gb->A_log[i];", 1),
    ("local scan's adjoint with the backward set's parameters",
     "const fvo_dir *pd[2] = {pf, local_window > 0 ? &pl : pb};", "const fvo_dir *pd[2] = {pf, pb};", 1),
    # backward pass through the producer Conv1D
    ("conv adjoint without the SiLU derivative", "const double da = gxc[(b * n + cell) * E + e] * sg * (1.0 + a * (1.0 - sg));",
     "const double da = gxc[(b * n + cell) * E + e] * sg;", 1),
    ("conv adjoint spreads to the wrong tap", "dx[(b * n + cc) * E + e] += (double)conv_w[e * KC + k] * da;",
     "dx[(b * n + cc) * E + e] += (double)conv_w[e * KC + (KC - 1 - k)] * da;", 1),
    ("conv weight gradient from the output position", "dcw[e * KC + k] += da * (double)x[(b * n + cc) * E + e];",
     "dcw[e * KC + k] += da * (double)x[(b * n + cell) * E + e];", 1),
    ("conv bias gradient without the SiLU derivative", "                dcb[e] += da;",
     "                dcb[e] += gxc[(b * n + cell) * E + e];", 1),
    ("backward pools the conv's input", "        pool_dense_any(x, xc, B, h, w, E, axis, u);\n    }\n    for (int64_t i = 0; i < M * E; ++i) u[i] *= pool_scale;\n    for (int d",
     "        pool_dense_any(x, NULL, B, h, w, E, axis, u);\n    }\n    for (int64_t i = 0; i < M * E; ++i) u[i] *= pool_scale;\n    for (int d", 1),
    ("conv adjoint row-major on the transposed grid",
     "const int colmajor = axis == FVO_NONE_COLMAJOR || axis == FVO_ROWS;",
     "const int colmajor = axis == FVO_NONE_COLMAJOR;", 1),
    ("output adjoint reads the conv's input", "const double *xco = xc ? xc + off : NULL;", "const double *xco = NULL;", 1),
    ("adjoint uses the current state for the decay", "dd += lam[n] * (A * a * prev + Bn * ut);",
     "dd += lam[n] * (A * a * Hs[k * N + n] + Bn * ut);", 1),
    # Conv1D with masked layers (along the kept tokens)
    ("masked skip reads x, not the conv's output",
     "x + c, xc ? xc + c : NULL, z + c, pf, pb,\n                             E, ln_w",
     "x + c, NULL, z + c, pf, pb,\n                             E, ln_w", 1),
    ("masked pool reads x, not the conv's output", "pool_masked_any(x, xc, rows, B, K, T, P, E, u);",
     "pool_masked_any(x, NULL, rows, B, K, T, P, E, u);", 2),
    ("masked conv adjoint one tap short",
     "conv_silu_adjoint(x, dxc, B, K, 1, E, FVO_COLS, conv_w, conv_b, conv_k, dx, dconv_w, dconv_b);",
     "conv_silu_adjoint(x, dxc, B, K, 1, E, FVO_COLS, conv_w, conv_b, conv_k - 1, dx, dconv_w, dconv_b);", 1),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, count, source, tmp_path):
    assert source.count(old) == count, "mutation site for %r not found %d times" % (name, count)
    mutated = source.replace(old, new)
    src = tmp_path / "mutant.c"
    src.write_text(mutated)
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / "libmutant.so"))
    # one OpenMP thread per child: the pins are small, and parallel test workers
    # each running a full team of spinning threads oversubscribe the cores
    env = dict(os.environ, OMP_NUM_THREADS="1")
    proc = subprocess.run([sys.executable, "-c", _CHILD, lib], capture_output=True, text=True,
                          timeout=300, cwd=os.path.dirname(os.path.dirname(SRC)), env=env)
    if proc.returncode < 0:
        return  # the mutant crashed: caught
    assert proc.returncode == 0, proc.stderr[-2000:]
    caught = [ln for ln in proc.stdout.splitlines() if ln.startswith("CAUGHT ")]
    assert caught, "mutant %r passes every pin" % name


_CHILD = """
import sys
sys.path[:0] = ['.', 'tests']
import oracle, pins
O = oracle.Oracle(sys.argv[1])
for pin in pins.ALL_PINS:
    try:
        pin(O)
    except (AssertionError, ValueError, FloatingPointError) as e:
        print('CAUGHT', pin.__name__, str(e)[:200], flush=True)
"""
