"""The GPU accuracy study (quantized_kv_cache_attend_amd.accuracy) against
the oracle: on the page's recipe (N = 128 / 512, D = 32, four queries,
clean and biased keys, three seeds) every per-input relative L2 error the
GPU measures matches the float64 oracle's for the same input (quantized
cache vs float32 cache), and the packed byte counts match the oracle's
ledger."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import Workload, make_qkv

from gpu_helpers import announce

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")


def test_study_matches_oracle():
    from quantized_kv_cache_attend_amd import accuracy
    announce("accuracy study n=128,512 d=32")
    rows = accuracy.study([128, 512], [32])
    assert len(rows) == 2 * 3 * 3 * 4
    for r in rows:
        w = Workload("acc", 1, 1, 1, 4, r["n"], r["d"], ((r["bits"], r["group"]),))
        q, k, v = make_qkv(w, r["seed"], r["dist"])
        kc, ks = O.pack_k(k, r["bits"], r["group"])
        vc, vs = O.pack_v(v, r["bits"], r["group"])
        want = O.rel_l2(O.attend_packed(q, kc, ks, vc, vs, r["n"], r["bits"], r["group"]),
                        O.attend_dense(q, k, v))
        assert abs(r["rel_l2"] - want) <= 1e-4 * want + 1e-6, r
        assert r["packed_bytes"] == O.packed_payload_bytes(r["n"], r["d"], r["bits"], r["group"],
                                                           shape_record=False)
    # the page's ordering of the formats on clean inputs
    mean = {}
    for b, g in accuracy.FORMATS:
        mean[(b, g)] = np.mean([r["rel_l2"] for r in rows
                                if (r["bits"], r["group"], r["dist"]) == (b, g, "clean")])
    assert mean[(8, 8)] < mean[(8, 32)] < mean[(4, 8)] < mean[(4, 32)]


def test_window_study_matches_oracle():
    """The mixed cache in the study: per-input errors equal the oracle's
    attend_window errors, and a 16-token float32 window cuts the error of
    late-biased inputs."""
    from quantized_kv_cache_attend_amd import accuracy
    announce("accuracy study with windows")
    rows = accuracy.study([512], [32], dists=("late", "early"), formats=((4, 32),),
                          windows=(0, 16))
    for r in rows:
        w = Workload("acc", 1, 1, 1, 4, r["n"], r["d"], ((4, 32),))
        q, k, v = make_qkv(w, r["seed"], r["dist"])
        want = O.rel_l2(O.attend_window(q, k, v, r["window"], 4, 32), O.attend_dense(q, k, v))
        assert abs(r["rel_l2"] - want) <= 1e-4 * want + 1e-6, r
    late = {win: np.mean([r["rel_l2"] for r in rows if (r["dist"], r["window"]) == ("late", win)])
            for win in (0, 16)}
    assert late[16] < 0.5 * late[0]
