"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default split, the whole batch in one decode call): one
flush -> append -> decode step, then the outputs of sampled (request, KV head)
pairs against the oracle (max |delta o| <= 1e-5, certificate relative 1e-5)
and their stored codes, statistics, windows and state bit-exact.  The
samples include the shortest and the longest request of each batch."""
import numpy as np
import pytest

from bit_kv_cache_kivi_amd import inputs

pytestmark = pytest.mark.gpu

TOL_O = 1e-5
TOL_CERT = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_kv_cache_kivi_amd import kvq
    kvq.lib()


def _sample(w, n_mid=3, seed=11):
    ctx = np.asarray(w.ctx)
    picks = {int(np.argmin(ctx)), int(np.argmax(ctx))}
    rng = np.random.default_rng(seed)
    picks |= set(int(b) for b in rng.choice(w.B, size=min(n_mid, w.B), replace=False))
    out = []
    for i, b in enumerate(sorted(picks)):
        out.append((b, int(rng.integers(w.Hkv))))
        if i == 0:
            out.append((b, w.Hkv - 1))
    return sorted(set(out))


def _run(w, steps=1, kappa=0.0, cert_check=False):
    from gpu_harness import Case
    case = Case(w, extra_tokens=steps + 8, sample=_sample(w))
    print(f"[fullsize] {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} sample={sorted(case.streams)}",
          flush=True)
    worst = 0.0
    for _ in range(steps):
        out, cert, q = case.step(decode=True, kappa=kappa)
    o = out.cpu().numpy()
    c = cert.cpu().numpy()
    g = w.group
    for (b, h) in case.streams:
        ref, rc = case.oracle_decode(q, b, h, kappa)
        got = o[b, h * g:(h + 1) * g]
        assert np.all(np.isfinite(got)), (b, h)
        err = float(np.abs(got.astype(np.float64) - ref).max())
        worst = max(worst, err)
        assert err <= TOL_O, (b, h, err)
        if cert_check:
            gc = c[b, h * g:(h + 1) * g].astype(np.float64)
            both_inf = np.isinf(gc) & np.isinf(rc)
            rel = np.abs(gc - rc) / np.maximum(np.abs(rc), 1e-30)
            assert np.all(both_inf | (rel <= TOL_CERT)), (b, h, gc, rc)
    assert np.all(np.isfinite(o)), "an unsampled output is not finite"
    case.check_status()
    case.check_state()
    case.check_store()
    print(f"[fullsize] {w.name}: max |delta o| = {worst:.3g}", flush=True)


def test_gqa_paged_32q8kv_b64_ctx8k_32k():
    _run(inputs.workload(3))


def test_mha_b16_h32_ctx4096_flush_step():
    # context 4096: the key residual is full, so the step's flush quantizes
    # a whole residual before the append
    _run(inputs.workload(2), steps=2)


def test_kitty_b16_h32_ctx32768():
    _run(inputs.workload(4))


def test_kitty_dynamic_b16_h32_ctx32768():
    _run(inputs.workload(6))


def test_kitty_pro_b16_h32_ctx32768():
    _run(inputs.workload(8))


def test_kivi4_b16_h32_ctx32768():
    _run(inputs.workload(9))


def test_gqa_sink32_b64_ctx8k_32k():
    _run(inputs.workload(7))


def test_gqa8_paged_64q8kv_b32_ctx8k_32k():
    # a group of 8: two query quads per KV head in the group kernel
    _run(inputs.workload(11))


def test_witcert_paged_b32_32q8kv_ctx16384_certificate():
    _run(inputs.workload(10), kappa=2.0, cert_check=True)


def test_witcert_b32_32q8kv_ctx16384_certificate():
    _run(inputs.workload(5), kappa=2.0, cert_check=True)
