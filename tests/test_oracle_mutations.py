"""The oracle's pins must catch plausible mistakes.

Each case plants one bug in a copy of the oracle's C source (on the CPU only),
builds it, and runs the oracle pin tests against that build; the run must
fail.  A mutant that survives means some part of the oracle is not pinned."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hc_oracle.c")

PIN_TESTS = [os.path.join(ROOT, "tests", f) for f in (
    "test_oracle_storage.py", "test_oracle_pre.py", "test_oracle_post.py",
    "test_oracle_weights.py", "test_oracle_sinkhorn.py", "test_oracle_backward.py",
    "test_oracle_weights_backward.py")]

MUTANTS = {
    "post: A transposed": ("y += A[i * n + j] * orc_load", "y += A[j * n + i] * orc_load"),
    "post: first column of A transposed": ("double y = A[i * n + 0]", "double y = A[0 * n + i]"),
    "post: write-back dropped": ("y += beta[i] * orc_load", "y += 0.0 * beta[i] * orc_load"),
    "post: write-back sign": ("y += beta[i] * orc_load", "y -= beta[i] * orc_load"),
    "pre: eps outside the root": ("double denom = sqrt(ms + eps);", "double denom = sqrt(ms) + eps;"),
    "pre: mean over n*d": ("double ms = ss / d;", "double ms = ss / ((double)d * n);"),
    "pre: first stream dropped": ("double x = alpha[0] * orc_load(H, row0 + k, dt);", "double x = 0.0;"),
    "pre: alpha index": ("x += alpha[i] * orc_load", "x += alpha[0] * orc_load"),
    "pre: gain dropped": ("ut[k] = gamma[k] * ut[k] / denom;", "ut[k] = ut[k] / denom;"),
    "weights: sum instead of mean": ("hbar[k] = s / n;", "hbar[k] = s;"),
    "weights: abs instead of square": ("ss += h * h;", "ss += fabs(h);"),
    "weights: tanh dropped": ("out[c] = w_static[c] + scale * tanh(z[c]);", "out[c] = w_static[c] + scale * z[c];"),
    "weights: no per-stream norm": ("s += r[i] * orc_load", "s += r[0] * orc_load"),
    "sinkhorn: column step dropped": ("for (int i = 0; i < n; ++i) M[i * n + j] /= s;", ";"),
    "sinkhorn: row step dropped": ("for (int j = 0; j < n; ++j) M[i * n + j] /= s;", ";"),
    "sinkhorn: sigmoid sign": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "sinkhorn: beta from alpha logits": ("out[n + i] = orc_sigmoid(l[n + i]);", "out[n + i] = orc_sigmoid(l[i]);"),
    "storage: truncating bf16": ("double m = rint(ldexp(a, -q));", "double m = floor(ldexp(a, -q));"),
    "block: tanh replaced": ("F[e] = tanh(orc_load(u, e, dt));", "F[e] = sin(orc_load(u, e, dt));"),
    "post bwd: dH not transposed": ("s += A[i * n + j] * orc_load(dHo", "s += A[j * n + i] * orc_load(dHo"),
    "post bwd: dbeta from H": ("g[n + i] += go * f;", "g[n + i] += go;"),
    "post bwd: dF unweighted": ("df += beta[i] * go;", "df += go;"),
    "pre bwd: no projection term": ("dx[k] = r * (dy - x[k] * r * r * sdx / d);", "dx[k] = r * dy;"),
    "pre bwd: dgamma missing r": ("dgamma[k] += g * x[k] * r;", "dgamma[k] += g * x[k];"),
    "pre bwd: dalpha from x": ("s += dx[k] * orc_load(H, e, dt);", "s += dx[k];"),
    "pre bwd: accumulation dropped": ("dH[e] = alpha[i] * dx[k] + (dH_in ? dH_in[e] : 0.0);", "dH[e] = alpha[i] * dx[k];"),
    "storage: no subnormal range": ("int q = (e - 1 >= -126) ? e - 8 : -133;", "int q = e - 8;"),
    "fp8: exponent bias 8": ("else v = ldexp((double)(8 + m), e - 10);", "else v = ldexp((double)(8 + m), e - 11);"),
    "fp8: subnormal scale": ("else if (e == 0) v = ldexp((double)m, -9);", "else if (e == 0) v = ldexp((double)m, -10);"),
    "fp8: truncating": ("const double r = ldexp(rint(ldexp(a, -q)), q);", "const double r = ldexp(floor(ldexp(a, -q)), q);"),
    "fp8: overflow to NaN": ("if (a > 448.0) a = 448.0;", "if (a > 464.0) return (uint8_t)(sign | 0x7F);"),
    "mhc bwd: column step projection dropped": ("gr[i * n + j] = (g[i * n + j] - s) / cs[it * n + j];", "gr[i * n + j] = g[i * n + j] / cs[it * n + j];"),
    "mhc bwd: row step projection dropped": ("g[i * n + j] = (gr[i * n + j] - s) / rs[it * n + i];", "g[i * n + j] = gr[i * n + j] / rs[it * n + i];"),
    "mhc bwd: sigmoid derivative": ("dl[i] = dout[i] * s * (1.0 - s);", "dl[i] = dout[i] * s;"),
    "mhc bwd: exp derivative dropped": ("dl[2 * n + e] = g[e] * Ms[e];", "dl[2 * n + e] = g[e];"),
    "weights bwd: tanh derivative": ("dz[c] = g[c] * scale * (1.0 - th * th);", "dz[c] = g[c] * scale * (1.0 + th * th);"),
    "weights bwd: norm term dropped": ("dH[e] = (r[i] * dhbar[k] - r[i] * r[i] * r[i] * s * orc_load(H, e, dt) / d) / n;", "dH[e] = (r[i] * dhbar[k]) / n;"),
    "weights bwd: dW from z": ("dW[(int64_t)c * d + k] += dz[c] * hbar[k];", "dW[(int64_t)c * d + k] += z[c] * hbar[k];"),
    "weights bwd: scale dropped in mhc": ("for (int c = 0; c < K; ++c) dz[c] = scale * dl[c];", "for (int c = 0; c < K; ++c) dz[c] = dl[c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    # an anchor found more than once is a formula written out in several
    # routines (forward and backward); the mistake is planted in all of them
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                           "-o", str(so), str(mutant), "-lm"])
    env = dict(os.environ, HC_ORACLE_SO=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_TESTS], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode != 0, f"mutant survived the pins: {name}\n{r.stdout[-2000:]}"
