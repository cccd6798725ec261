"""The float32 CPU reference (oracle/cpu_reference.py, the bench's full-N CPU comparison)
against the float64 oracle: the same choice on tokens with clear margins, and the output
within float32 rounding, for every router and both activations."""
import numpy as np
import pytest

from oracle import cpu_reference as R
from oracle import moe_oracle as O


@pytest.mark.parametrize("router,norm,scale,act,bias,shared", [
    ("softmax_topk", True, 1.0, "swiglu", False, False), ("softmax_topk", False, 1.0, "gelu", True, False),
    ("topk_softmax", True, 1.0, "swiglu", False, True), ("sigmoid", True, 2.5, "swiglu", False, False),
    ("sigmoid", False, 1.0, "gelu", False, True)])
def test_reference_matches_oracle(router, norm, scale, act, bias, shared):
    rng = np.random.default_rng(31)
    N, d, f, E, k = 300, 48, 40, 9, 3
    params = {"w_g": rng.normal(0, 0.3, (E, d)), "w1": rng.normal(0, 0.2, (E, f, d)),
              "w2": rng.normal(0, 0.2, (E, d, f))}
    if act == "swiglu":
        params["w3"] = rng.normal(0, 0.2, (E, f, d))
    if bias:
        params["b1"] = rng.normal(0, 0.2, (E, f))
        params["b2"] = rng.normal(0, 0.2, (E, d))
    if shared:
        params["s_w1"] = rng.normal(0, 0.2, (16, d))
        params["s_w2"] = rng.normal(0, 0.2, (d, 16))
        if act == "swiglu":
            params["s_w3"] = rng.normal(0, 0.2, (16, d))
    x = rng.normal(size=(N, d))
    lb = rng.normal(0, 0.5, E)
    sb = rng.uniform(-0.1, 0.1, E) if router == "sigmoid" else None
    spec = O.Spec(n_experts=E, top_k=k, router=router, norm_topk=norm, routed_scaling=scale, act=act)
    y64, r = O.forward_loop(x, params, spec, lb, sb)
    p32 = {n: None if v is None else np.asarray(v, np.float32) for n, v in params.items()}
    y32, ids = R.forward_f32(x.astype(np.float32), p32, E, k, act, router, norm, scale, lb, sb)
    clean = (r.gap > 1e-4) & (r.intra_gap > 1e-4)
    assert clean.mean() > 0.95
    assert np.array_equal(ids[clean], r.ids[clean])
    err = np.abs(y32[clean] - y64[clean]).max()
    assert err <= 1e-4 * np.abs(y64).max(), err


def test_reference_tie_goes_to_lowest_id():
    """The [L7.8] §3 worked example's exact tie (token 1: z_0 = z_2 = ln 3) picks expert 0 first."""
    z = np.log(np.array([[2, 4, 1, 1], [3, 1, 3, 2]], np.float32))
    ids, w = R.route_f32(z, np.eye(4, dtype=np.float32), 4, 2)
    assert ids.tolist() == [[1, 0], [0, 2]]
    np.testing.assert_allclose(w, [[2 / 3, 1 / 3], [1 / 2, 1 / 2]], rtol=1e-6)
