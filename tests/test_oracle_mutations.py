"""Planted mistakes in the CPU oracle must fail its CPU pins.

Each case copies oracle/oracle.c, makes one plausible mistake in the copy
(a reciprocal instead of the division, a dropped term, a wrong index, a
product kept in fp64 where the reading rounds it to fp32, ...), builds it
with the oracle's own gcc flags and runs the pin tests of the function it
touches (hand-worked fixtures, closed forms, invariants, brute force) with
that copy loaded in place of the oracle.  At least one pin must fail.  The
numpy twin (oracle/ref_tiny.py) is left out: the mutant must be caught by
pins that do not come from a second implementation.

This is what makes the oracle's own correctness checkable: if a mistake of
this kind could pass every pin, the GPU comparison would be pinning the
oracle to the kernel instead of the other way round.
"""
import concurrent.futures
import importlib
import inspect
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as obuild

# (name, function anchor, text to replace (first occurrence after the anchor),
#  replacement, pin modules)
MUTANTS = [
    # block quantization
    ("quantize: reciprocal division", "int oracle_quantize_block(",
     "rintf(oracle_bf16_to_f32(x[r * cols + c]) / sc)", "rintf(oracle_bf16_to_f32(x[r * cols + c]) * (1.0f / sc))",
     ["test_oracle_quantize"]),
    ("quantize: x * 127 / a", "int oracle_quantize_block(",
     "rintf(oracle_bf16_to_f32(x[r * cols + c]) / sc)", "rintf(oracle_bf16_to_f32(x[r * cols + c]) * 127.0f / a)",
     ["test_oracle_quantize"]),
    ("quantize: ties away from zero", "int oracle_quantize_block(",
     "float t = rintf(", "float t = roundf(", ["test_oracle_quantize"]),
    ("quantize: divisor 128", "int oracle_quantize_block(",
     "const float sc = a / 127.0f;", "const float sc = a / 128.0f;", ["test_oracle_quantize"]),
    ("quantize: absmax over the block's first row only", "int oracle_quantize_block(",
     "for (int64_t r = r0; r < r0 + ORACLE_BLOCK; ++r)", "for (int64_t r = r0; r < r0 + 1; ++r)",
     ["test_oracle_quantize"]),
    # partials and the dequantized output
    ("partials: K-block off by one", "int oracle_kblock_partials(",
     "for (int64_t k = kb * ORACLE_BLOCK; k < (kb + 1) * ORACLE_BLOCK; ++k)",
     "for (int64_t k = kb * ORACLE_BLOCK + 1; k < (kb + 1) * ORACLE_BLOCK; ++k)", ["test_oracle_gemm"]),
    ("linear: activation scales transposed", "int oracle_linear_int8_rows(",
     "(double)sx[(m / ORACLE_BLOCK) * kbs + kb]", "(double)sx[kb * (M / ORACLE_BLOCK) + m / ORACLE_BLOCK]",
     ["test_oracle_gemm"]),
    ("linear: weight scale of K-block 0 only", "int oracle_linear_int8_rows(",
     "(double)sw[(n / ORACLE_BLOCK) * kbs + kb]", "(double)sw[(n / ORACLE_BLOCK) * kbs]", ["test_oracle_gemm"]),
    ("linear: bias dropped", "int oracle_linear_int8_rows(",
     "if (bias) acc += (double)oracle_bf16_to_f32(bias[n]);", "if (bias) acc += 0.0;", ["test_oracle_gemm"]),
    ("linear: rounded through fp32 (double rounding)", "int oracle_linear_int8_rows(",
     "if (y) y[t * N + n] = oracle_f64_to_bf16(acc);", "if (y) y[t * N + n] = oracle_f64_to_bf16((double)(float)acc);",
     ["test_oracle_gemm", "test_oracle_arith"]),
    ("bf16 rounding: ties away from zero", "uint16_t oracle_f64_to_bf16(",
     "double n = nearbyint(ldexp(a, -qexp));", "double n = round(ldexp(a, -qexp));", ["test_oracle_arith"]),
    # fallback and guard
    ("fallback: fp32 input not rounded to bf16", "static double load_as_bf16(",
     "return (double)oracle_bf16_to_f32(oracle_f64_to_bf16((double)((const float *)x)[idx]));",
     "return (double)((const float *)x)[idx];", ["test_oracle_gemm"]),
    ("guard: K ignored", "int oracle_route(",
     "M % ORACLE_BLOCK == 0 && K % ORACLE_BLOCK == 0 &&", "M % ORACLE_BLOCK == 0 &&", ["test_oracle_arith"]),
    # post-scale form
    ("post-scale: eps floor dropped", "int oracle_quantize_rows(",
     "if (a < eps) a = eps;", "(void)eps;", ["test_oracle_postscale"]),
    ("post-scale: eps floor 1e-3", "int oracle_quantize_rows(",
     "const float eps = 1e-4f;", "const float eps = 1e-3f;", ["test_oracle_postscale"]),
    ("post-scale: sum over half of K", "int oracle_linear_postscale_rows(",
     "for (int64_t k = 0; k < K; ++k) acc +=", "for (int64_t k = 0; k < K / 2; ++k) acc +=",
     ["test_oracle_postscale"]),
    ("post-scale: weight scale dropped", "int oracle_linear_postscale_rows(",
     "double v = (double)acc * (double)sx[m] * (double)sw[n];", "double v = (double)acc * (double)sx[m];",
     ["test_oracle_postscale"]),
    # attention Q/K and V
    ("Q/K: written sequence-major", "int oracle_quantize_qk(",
     "q[(bh * L + l) * D + d] = out;", "q[((b * L + l) * H + h) * D + d] = out;", ["test_oracle_qk"]),
    ("Q/K: 64-token blocks", "int oracle_quantize_qk(",
     "const int64_t l1 = l0 + ORACLE_BLOCK < L ? l0 + ORACLE_BLOCK : L;",
     "const int64_t l1 = l0 + 64 < L ? l0 + 64 : L;", ["test_oracle_qk"]),
    ("E4M3: ties away from zero", "uint8_t oracle_f32_to_e4m3(",
     "if (d > 0.5 || (d == 0.5 && fmod(f, 2.0) == 1.0)) f += 1.0;", "if (d >= 0.5) f += 1.0;",
     ["test_oracle_fp8"]),
    ("V: scaled by max-abs / 447", "int oracle_quantize_v_fp8(",
     "const float sc = a / 448.0f;", "const float sc = a / 447.0f;", ["test_oracle_fp8"]),
    # GELU producer
    ("GELU through 1 + erf", "int oracle_gelu_bf16(",
     "0.5 * v * erfc(-v / sqrt(2.0))", "0.5 * v * (1.0 + erf(v / sqrt(2.0)))", ["test_oracle_gelu"]),
    ("GELU with x / 2 for x / sqrt 2", "int oracle_gelu_bf16(",
     "erfc(-v / sqrt(2.0))", "erfc(-v / 2.0)", ["test_oracle_gelu"]),
    # modulated RMSNorm
    ("RMSNorm: x * r kept in fp64", "int oracle_rmsnorm_modulate(",
     "const float t = oracle_bf16_to_f32(xr[k]) * r;", "const double t = (double)oracle_bf16_to_f32(xr[k]) * r;",
     ["test_oracle_rmsnorm"]),
    ("RMSNorm: eps dropped", "int oracle_rmsnorm_modulate(",
     "sqrt(S / (double)K + eps)", "sqrt(S / (double)K)", ["test_oracle_rmsnorm"]),
    ("RMSNorm: scale instead of 1 + scale", "int oracle_rmsnorm_modulate(",
     "const float one_s = 1.0f + oracle_bf16_to_f32(scale[b * K + k]);",
     "const float one_s = oracle_bf16_to_f32(scale[b * K + k]);", ["test_oracle_rmsnorm"]),
    ("RMSNorm: shift subtracted", "int oracle_rmsnorm_modulate(",
     "const float v = u + oracle_bf16_to_f32(shift[b * K + k]);",
     "const float v = u - oracle_bf16_to_f32(shift[b * K + k]);", ["test_oracle_rmsnorm"]),
    ("RMSNorm: batch entry by row modulo B", "int oracle_rmsnorm_modulate(",
     "const int64_t b = i / L;", "const int64_t b = i % B;", ["test_oracle_rmsnorm"]),
    # modulated LayerNorm
    ("LayerNorm: (x - m) * r kept in fp64", "int oracle_layernorm_modulate(",
     "const float t = c * r;", "const double t = (double)c * r;", ["test_oracle_layernorm"]),
    ("LayerNorm: fp64 mean subtracted", "int oracle_layernorm_modulate(",
     "const float c = oracle_bf16_to_f32(xr[k]) - m;", "const float c = (float)((double)oracle_bf16_to_f32(xr[k]) - mu);",
     ["test_oracle_layernorm"]),
    ("LayerNorm: not centred in the output", "int oracle_layernorm_modulate(",
     "const float c = oracle_bf16_to_f32(xr[k]) - m;", "const float c = oracle_bf16_to_f32(xr[k]);",
     ["test_oracle_layernorm"]),
    ("LayerNorm: variance over K - 1", "int oracle_layernorm_modulate(",
     "sqrt(V / (double)K + eps)", "sqrt(V / (double)(K - 1) + eps)", ["test_oracle_layernorm"]),
    # split rotary embedding
    ("RoPE: sign of the lower half flipped", "int oracle_rope(",
     "oracle_f64_to_bf16((double)(a - b));", "oracle_f64_to_bf16((double)(a + b));", ["test_oracle_rope"]),
    ("RoPE: products kept in fp64", "int oracle_rope(",
     "oracle_f64_to_bf16((double)(a - b));", "oracle_f64_to_bf16((double)x1 * c - (double)x2 * s);",
     ["test_oracle_rope"]),
    ("RoPE: fused multiply-add", "int oracle_rope(",
     "oracle_f64_to_bf16((double)(a - b));", "oracle_f64_to_bf16((double)fmaf(x1, c, -b));", ["test_oracle_rope"]),
    # gated residual update
    ("gated residual: fp64 sum", "int oracle_gated_residual(",
     "const float s = oracle_bf16_to_f32(h[i * N + n]) + p;", "const double s = (double)oracle_bf16_to_f32(h[i * N + n]) + p;",
     ["test_oracle_gated_residual"]),
    ("gated residual: gate dropped", "int oracle_gated_residual(",
     "const float p = oracle_bf16_to_f32(gate[b * N + n]) * oracle_bf16_to_f32(o[i * N + n]);",
     "const float p = oracle_bf16_to_f32(o[i * N + n]);", ["test_oracle_gated_residual"]),
]


def _mutate(src, anchor, old, new):
    a = src.index(anchor)
    i = src.index(old, a)
    # the mistake must land inside the anchored function (before the next one)
    nxt = src.find("\nint oracle_", a + len(anchor))
    assert nxt < 0 or i < nxt, f"{old!r} not found inside {anchor!r}"
    return src[:i] + new + src[i + len(old):]


def _build(args):
    idx, text, outdir = args
    c = os.path.join(outdir, f"mutant{idx}.c")
    so = os.path.join(outdir, f"mutant{idx}.so")
    with open(c, "w") as f:
        f.write(text)
    cflags = [f for f in obuild.CFLAGS if f != "-Werror"]  # an unused variable is fine in a mutant
    subprocess.run(["gcc", *cflags, c, "-o", so, "-lm"], check=True, capture_output=True)
    return so


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    with open(obuild.SRC) as f:
        src = f.read()
    outdir = str(tmp_path_factory.mktemp("mutants"))
    jobs = [(i, _mutate(src, anchor, old, new), outdir) for i, (_, anchor, old, new, _) in enumerate(MUTANTS)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return list(ex.map(_build, jobs))


def _pins(module_name):
    """(label, zero-argument callable) for every pin test of a module, one per
    parameter value for parametrized tests; tests taking fixtures are left out."""
    mod = importlib.import_module(module_name)
    out = []
    for name, fn in sorted(vars(mod).items()):
        if not name.startswith("test_") or not callable(fn):
            continue
        params = inspect.signature(fn).parameters
        if not params:
            out.append((name, fn))
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if len(params) == 1 and len(marks) == 1 and marks[0].args[0] == next(iter(params)):
            for v in marks[0].args[1]:
                out.append((f"{name}[{v}]", lambda fn=fn, v=v: fn(v)))
    return out


def test_every_mutant_applies_to_the_current_source():
    with open(obuild.SRC) as f:
        src = f.read()
    for name, anchor, old, new, _ in MUTANTS:
        assert _mutate(src, anchor, old, new) != src, name


@pytest.mark.parametrize("idx", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(idx, mutant_libs, monkeypatch):
    name, _, _, _, modules = MUTANTS[idx]
    monkeypatch.setattr(oracle, "_lib", oracle.load(mutant_libs[idx]))
    caught = []
    for mod in modules:
        for label, pin in _pins(mod):
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(f"{mod}::{label}")
    assert caught, f"planted mistake '{name}' passed every pin of {modules}"
