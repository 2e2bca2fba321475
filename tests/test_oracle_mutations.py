"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, index or operand, a wrong rounding or bookkeeping rule),
builds it, and runs the CPU pin tests against that build in a subprocess
(ZDP_ORACLE_LIB points the oracle at it). Every planted mistake must make a
pin fail; the unmodified source, built the same way, must pass them all."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_encodings.py", "tests/test_oracle_partition.py",
        "tests/test_oracle_average_norm.py", "tests/test_oracle_adam.py",
        "tests/test_oracle_step.py", "tests/test_oracle_clip.py"]

MUTATIONS = [
    ("first-moment bias correction dropped", "float mhat = mt / b1;", "float mhat = mt;"),
    ("second-moment bias correction dropped", "float vhat = vt / b2;", "float vhat = vt;"),
    ("beta1 used for the variance", "float vt = beta2f * v[j]", "float vt = beta1f * v[j]"),
    ("1-beta2 used for the momentum", "float mt = beta1f * m[j] + c1 * g;", "float mt = beta1f * m[j] + c2 * g;"),
    ("g instead of g^2 in the variance", "c2 * (g * g);", "c2 * g;"),
    ("eps inside the square root", "float denom = sqrtf(vhat) + epsf;", "float denom = sqrtf(vhat + epsf);"),
    ("update sign flipped", "float next = theta - lrf * upd;", "float next = theta + lrf * upd;"),
    ("bias power off by one", "(float)(1.0 - beta_pow(beta1, t))", "(float)(1.0 - beta_pow(beta1, t - 1 > 0 ? t - 1 : 1))"),
    ("weight decay dropped", "theta = theta * decay;", "theta = theta;"),
    ("weight decay coupled to the gradient", "float g = a[j] * inv_scale;              /* unscale */",
     "float g = a[j] * inv_scale + (float)weight_decay * master[j];"),
    ("unscale dropped in the update", "float g = a[j] * inv_scale;              /* unscale */",
     "float g = a[j];"),
    ("average not divided by N_d", "out[j] = acc / nd;", "out[j] = acc;"),
    ("average over N_d - 1 copies", "for (int32_t r = 0; r < n_d; ++r)\n            acc = acc + decode16",
     "for (int32_t r = 0; r < n_d - 1; ++r)\n            acc = acc + decode16"),
    ("remainder given to the last ranks", "int64_t size = base + (r < rem ? 1 : 0);",
     "int64_t size = base + (r >= n_d - rem ? 1 : 0);"),
    ("norm of the scaled gradient", "float g = a[j] * inv_scale;\n        acc += (double)g * (double)g;",
     "float g = a[j];\n        acc += (double)g * (double)g;"),
    ("overflow flag never set", "if (!isfinite(a[j]))\n            f = 1;", "if (0)\n            f = 1;"),
    ("skip does not lower the scale", "double s = (double)st->loss_scale * policy->backoff;",
     "double s = (double)st->loss_scale;"),
    ("skipped step still counted", "st->good_steps = 0;\n        st->skipped = 1;",
     "st->good_steps = 0;\n        st->skipped = 1;\n        st->step += 1;"),
    ("average-fed step ignores the shard flag", "apply_verdict(groups, n_groups, avg, policy, st, norm2, flag != 0);",
     "apply_verdict(groups, n_groups, avg, policy, st, norm2, 0);"),
    ("skip ignored", "if (flag && policy->skip_on_overflow) {", "if (0) {"),
    ("scale never grows", "st->loss_scale = (float)((double)st->loss_scale * policy->growth);", "(void)0;"),
    ("ties rounded away from zero", "r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "r = fl + 1.0;"),
    ("fp16 subnormal spacing wrong", "if (q < -24)\n        q = -24;", "if (q < -25)\n        q = -25;"),
    ("bf16 keeps 9 bits", "int q = e - 8;      /* 8 significant bits */", "int q = e - 9;"),
    ("fp16 decode exponent bias off by one", "mag = ldexpf((float)(frac + 1024), e - 25);",
     "mag = ldexpf((float)(frac + 1024), e - 24);"),
    ("tensor slice begins at the shard start", "tensor_begin[count] = ob - b;", "tensor_begin[count] = 0;"),
    ("clip multiplier not applied", "g = g * clip;                            /* clip (1 = none) */", "(void)clip;"),
    ("clip from the squared norm", "double c = max_norm / (sqrt(norm2) + 1e-6);", "double c = max_norm / (norm2 + 1e-6);"),
    ("clip allowed to scale up", "return (float)(c < 1.0 ? c : 1.0);", "return (float)c;"),
    ("shard norm ignored for a sample", "            norm2 = given_norm2;\n", ""),
    ("shard flag ignored for a sample", "            flag = given_flag;\n", ""),
    ("scale floor ignored", "        if (s < policy->min_scale)\n            s = policy->min_scale;\n", ""),
    ("growth ignores its window", "st->good_steps == policy->growth_interval) {", "st->good_steps >= 1) {"),
    ("clip guard dropped", "double c = max_norm / (sqrt(norm2) + 1e-6);", "double c = max_norm / sqrt(norm2);"),
    ("padding one unit too far", "padded = numel + (align_elems - r);",
     "padded = numel + (align_elems - r) + align_elems;"),
    ("skip keeps the growth window", "        st->good_steps = 0;\n        st->skipped = 1;\n",
     "        st->skipped = 1;\n"),
    ("fp16 NaN not canonical", "return 0x7e00; /* canonical quiet NaN */", "return sign | 0x7e01;"),
    ("bf16 decode shifted by 15", "uint32_t bits = (uint32_t)h << 16;", "uint32_t bits = (uint32_t)h << 15;"),
    ("decay after the update", "        float next = theta - lrf * upd;\n",
     "        float next = (theta - lrf * upd) * (weight_decay != 0.0 ? decay : 1.0f);\n"),
    ("decay without the learning rate", "const float decay = (float)(1.0 - lr * weight_decay);",
     "const float decay = (float)(1.0 - weight_decay);"),
    ("clip multiplier squared", "        g = g * clip;                            /* clip (1 = none) */\n",
     "        g = g * (clip < 1.0f ? clip * clip : 1.0f);\n"),
    ("parameter written from the pre-update master", "            param[j] = encode16(param_dt, next);",
     "            param[j] = encode16(param_dt, theta);"),
]


def _build_variant(src_text, out_dir, tag):
    c = os.path.join(out_dir, f"{tag}.c")
    so = os.path.join(out_dir, f"{tag}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *oracle_build.CFLAGS, c, "-o", so, "-lm"], check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return so


def _pins_pass(so):
    env = dict(os.environ, ZDP_ORACLE_LIB=so, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "--hypothesis-seed=0", *PINS], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return r.returncode == 0, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(oracle_build.SRC).read()
    for name, old, _ in MUTATIONS:
        assert src.count(old) == 1, f"mutation site not unique or missing: {name}"
    control = _build_variant(src, str(tmp_path), "control")
    variants = [(name, _build_variant(src.replace(old, new), str(tmp_path), f"m{i}"))
                for i, (name, old, new) in enumerate(MUTATIONS)]
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        ok_control, log = ex.submit(_pins_pass, control).result()
        assert ok_control, "the unmodified oracle fails its pins:\n" + log
        results = list(ex.map(lambda v: (v[0], _pins_pass(v[1])[0]), variants))
    escaped = [name for name, passed in results if passed]
    assert not escaped, f"pins did not catch: {escaped}"
