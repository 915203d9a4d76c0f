"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/zf_oracle.c (a dropped
term, a wrong sign or index, a transposed operand, an off-by-one), builds
it into a temporary library and runs the pin suite against it
(tests/test_oracle_pins.py, via ZF_ORACLE_LIB).  The suite must fail.
CPU only; the shipped oracle is never modified.  The selected mutants are
built and checked up front, several at a time (each in its own process),
and every case then reads its own outcome.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import build as ob

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zf_oracle.c")
HDR = os.path.join(ROOT, "oracle", "zf_oracle.h")

# (name, text in zf_oracle.c, replacement)
MUTANTS = [
    ("bf16 rounding loses ties-to-even",
     "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x7FFFu;"),
    ("fp16 rounding rounds half up",
     "if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q += 1u;",
     "if (rem >= 0x1000u) q += 1u;"),
    ("fp16 subnormal shift off by one",
     "shift = -(e + 1);", "shift = -e;"),
    ("reduce-scatter starts from the last replica",
     "float acc = widen(grad_dtype, grads[0][p]);\n"
     "        for (q = 1; q < n_ranks; ++q) acc = acc + widen(grad_dtype, grads[q][p]);",
     "float acc = widen(grad_dtype, grads[n_ranks - 1][p]);\n"
     "        for (q = 0; q < n_ranks - 1; ++q) acc = acc + widen(grad_dtype, grads[q][p]);"),
    ("epsilon inside the square root",
     "float d = sqrtf(vv / sc->bc2) + sc->ef;", "float d = sqrtf(vv / sc->bc2 + sc->ef);"),
    ("first moment not bias-corrected",
     "float mh = mm / sc->bc1;", "float mh = mm;"),
    ("weight decay dropped",
     "float pp = p[i] * sc->dec;", "float pp = p[i];"),
    ("update added instead of subtracted",
     "pp = pp - sc->lrf * (mh / d);", "pp = pp + sc->lrf * (mh / d);"),
    ("second moment uses g instead of g*g",
     "float vv = sc->b2 * v[i] + sc->c2 * (g * g);", "float vv = sc->b2 * v[i] + sc->c2 * g;"),
    ("clip coefficient without the 1e-6",
     "coef = hp->max_norm / (norm + 1e-6);", "coef = hp->max_norm / norm;"),
    ("norm not averaged over ranks",
     "norm = sqrt(sumsq) / (S * (double)n_ranks);", "norm = sqrt(sumsq) / S;"),
    ("bias-correction power off by one",
     "for (i = 1; i < st->t; ++i) {", "for (i = 0; i < st->t; ++i) {"),
    ("loss scale not halved on overflow",
     "st->loss_scale = st->loss_scale * 0.5;", "st->loss_scale = st->loss_scale;"),
    ("skipped step still counts",
     "    res->scale_next = st->loss_scale;\n    res->t = st->t;\n    return 0;\n  }",
     "    res->scale_next = st->loss_scale;\n    st->t += 1;\n    res->t = st->t;\n    return 0;\n  }"),
    ("padding rounds up one shard too many",
     "u->P = ((u->L + n_ranks - 1) / n_ranks) * n_ranks;", "u->P = (u->L / n_ranks + 1) * n_ranks;"),
    ("stage-2 ledger keeps full gradients",
     "case 2: *after_backward_bytes = 2 * psi_pad + 2 * s_tot + 12 * s_tot; break;",
     "case 2: *after_backward_bytes = 2 * psi_pad + 2 * psi_pad + 12 * s_tot; break;"),
    ("unit gather transposes rank and offset",
     "unit_buf[(int64_t)r * units[u].S + j] = param_shards[r][units[u].M + j];",
     "unit_buf[j * n_ranks + r] = param_shards[r][units[u].M + j];"),
    ("fp32 draws scaled by sigma twice",
     "for (i = 0; i < n; ++i) dst[i] = or_normal_z(st, logical_base + i) * sf;",
     "for (i = 0; i < n; ++i) dst[i] = or_normal_z(st, logical_base + i) * sf * sf;"),
    ("fp32 draws multiplied by sigma in double",
     "for (i = 0; i < n; ++i) dst[i] = or_normal_z(st, logical_base + i) * sf;",
     "for (i = 0; i < n; ++i) dst[i] = (float)((double)or_normal_z(st, logical_base + i) * sigma);"),
    ("fp32 draws ignore sigma",
     "for (i = 0; i < n; ++i) dst[i] = or_normal_z(st, logical_base + i) * sf;",
     "for (i = 0; i < n; ++i) dst[i] = or_normal_z(st, logical_base + i) * (sf / sf);"),
    ("squared norm of an array skips its last value",
     "  for (i = 0; i < n; ++i) {\n    if (!isfinite(x[i])) nf = 1;\n    ss += (double)x[i] * (double)x[i];",
     "  for (i = 0; i < n; ++i) {\n    if (!isfinite(x[i])) nf = 1;\n    if (i + 1 < n) ss += (double)x[i] * (double)x[i];"),
    ("squared norm of an array squares in binary32",
     "    ss += (double)x[i] * (double)x[i];\n  }\n  *sumsq = ss;",
     "    ss += (double)(x[i] * x[i]);\n  }\n  *sumsq = ss;"),
    ("overflow flag of an array misses NaN",
     "    if (!isfinite(x[i])) nf = 1;\n    ss += (double)x[i] * (double)x[i];\n  }\n  *sumsq = ss;",
     "    if (isinf(x[i])) nf = 1;\n    ss += (double)x[i] * (double)x[i];\n  }\n  *sumsq = ss;"),
    ("Irwin-Hall centred on the wrong mean",
     "return (float)(sum - 393210) / 65536.0f;", "return (float)(sum - 393216) / 65536.0f;"),
    ("FSDP2 chunk rows rounded the wrong way",
     "c = (R + n_ranks - 1) / n_ranks;", "c = R / n_ranks + 1;"),
    ("FSDP2 gather transposes rank and offset",
     "int64_t r = e / U->S, j = e % U->S;", "int64_t r = e % n_ranks, j = e / n_ranks;"),
    ("FSDP2 update reads rank 0's gradient shard on every rank",
     "or_adamw_array(s_tot, grad_shards[r], &sc, master[r], exp_avg[r], exp_avg_sq[r]);",
     "or_adamw_array(s_tot, grad_shards[0], &sc, master[r], exp_avg[r], exp_avg_sq[r]);"),
    ("FSDP2 ledger counts a 16-bit parameter copy",
     "*after_backward_bytes = 4 * s_tot + 4 * s_tot + 8 * s_tot;",
     "*after_backward_bytes = 2 * s_tot + 4 * s_tot + 4 * s_tot + 8 * s_tot;"),
    ("accumulating reduce-scatter drops the previous shard",
     "shards[r][U->M + j] = accumulate ? shards[r][U->M + j] + sum : sum;",
     "shards[r][U->M + j] = sum;"),
    ("local accumulation overwrites",
     "acc[i] = accumulate ? acc[i] + g : g;", "acc[i] = g;"),
    ("bucket closes one segment late",
     "if (fill >= B && s + 1 < nseg) {", "if (fill > B && s + 1 < nseg) {"),
    ("default bucket size ignores the DP size",
     "B = bucket_numel > 0 ? bucket_numel : 1000000LL * n_ranks;",
     "B = bucket_numel > 0 ? bucket_numel : 40000000LL;"),
    ("fp32 replicas read as 16-bit values",
     "if (dtype == OR_F32) return ((const float*)g)[p];",
     "if (dtype == OR_F32) return widen(OR_BF16, ((const uint16_t*)g)[p]);"),
    ("reduced step never flags an overflow",
     "if (!isfinite(acc[r][k])) overflow = 1;", "if (0 && !isfinite(acc[r][k])) overflow = 1;"),
    ("micro-batch streams overlap the next step's",
     "((uint64_t)micro << 8)", "((uint64_t)micro << 20)"),
    ("no_sync regeneration sums ranks before micro-batches",
     "  if (mode == 0) {\n    for (a = 0; a < n_micro; ++a) {",
     "  if (mode == 0 || mode == 1) {\n    for (a = 0; a < n_micro; ++a) {"),
    ("reshard leaves the new padding unwritten",
     "        else\n          memset(dst, 0, (size_t)elem_bytes);",
     "        else\n          (void)dst;"),
    ("reshard places later ranks one element early",
     "memcpy(dst, logical + (ub[u].lam + e) * elem_bytes, (size_t)elem_bytes);",
     "memcpy(dst, logical + (ub[u].lam + e - (r > 0)) * elem_bytes, (size_t)elem_bytes);"),
    ("first moment decays with beta2",
     "float mm = sc->b1 * m[i] + sc->c1 * g;", "float mm = sc->b2 * m[i] + sc->c1 * g;"),
    ("gradient neither unscaled nor clipped",
     "float g = acc[i] * sc->gs;", "float g = acc[i];"),
    ("clip coefficient not capped at 1",
     "if (coef > 1.0) coef = 1.0;", "if (coef > 2.0) coef = 1.0;"),
    ("dynamic loss scale never grows",
     "st->loss_scale = S * 2.0;", "st->loss_scale = S;"),
    ("growth counter kept after the scale doubles",
     "    st->loss_scale = S * 2.0;\n    st->growth_ctr = 0;",
     "    st->loss_scale = S * 2.0;"),
    ("weight decay not scaled by the learning rate",
     "sc->dec = (float)(1.0 - hp->lr * hp->weight_decay);",
     "sc->dec = (float)(1.0 - hp->weight_decay);"),
    ("bias correction uses beta^t instead of 1 - beta^t",
     "sc->bc1 = (float)(1.0 - B1);", "sc->bc1 = (float)B1;"),
    ("ring traffic without the (N-1)/N factor",
     "return passes * ((double)(n_ranks - 1) / (double)n_ranks) * 2.0 * (double)psi_pad;",
     "return passes * 2.0 * (double)psi_pad;"),
]


WORKERS = max(1, min(6, os.cpu_count() or 1))


def run_mutant(workdir, name, old, new):
    """Build one mutant and run the pin suite against it: (the suite's exit
    status, the end of its output), or (None, why) if the site is missing."""
    src = open(SRC).read()
    if src.count(old) != 1:
        return None, f"mutation site not found once: {name}"
    os.makedirs(workdir, exist_ok=True)
    with open(os.path.join(workdir, "zf_oracle.c"), "w") as f:
        f.write(src.replace(old, new))
    shutil.copy(HDR, os.path.join(workdir, "zf_oracle.h"))
    lib = os.path.join(workdir, "libmutant.so")
    subprocess.run(["gcc", *ob.CFLAGS, "-o", lib, os.path.join(workdir, "zf_oracle.c"), "-lm"],
                   check=True)
    env = dict(os.environ, ZF_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def outcomes(request, tmp_path_factory):
    """Outcome of every mutant this session selected, computed together."""
    picked = {item.callspec.params["name"] for item in request.session.items
              if getattr(item, "originalname", None) == "test_pins_catch_mutant"}
    todo = [m for m in MUTANTS if m[0] in picked]
    base = tmp_path_factory.mktemp("mutants")
    with ThreadPoolExecutor(WORKERS) as ex:
        res = ex.map(lambda km: run_mutant(str(base / f"m{km[0]}"), *km[1]), enumerate(todo))
        return dict(zip((m[0] for m in todo), res))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(outcomes, name, old, new):
    rc, out = outcomes[name]
    assert rc is not None, out
    assert rc != 0, f"the pins did not catch: {name}\n{out}"
