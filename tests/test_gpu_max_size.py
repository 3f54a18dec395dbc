"""The matrix-core and streaming kernels at their largest token count per KV
head, N = 2^25 - 32 for 4-bit and 2^24 - 32 for 8-bit codes (a head's packed
arrays reach 2^31 - 2048 or 2^31 - 4096 bytes, the limit of their 32-bit
buffer offsets; at group 8 the K and V scale arrays reach it too), on
structured inputs with a closed-form
answer: every key is zero except one token at each end of the cache, both
aligned with the query, and the values of those two tokens differ from the
rest.  A skipped, repeated or misaddressed block anywhere moves the result.
K, V live only on the device (2 x 17 GB float32 at 4-bit); the oracle packs the few
distinct rows and the expected output is the softmax over three classes of
tokens in float64."""
import math

import numpy as np
import pytest

from oracle import kvq_oracle as O

from gpu_helpers import announce, host

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")

N_MAX = {4: (1 << 25) - 32, 8: (1 << 24) - 32}
D = 128


def _decoded_k_row(k_row, t_in_group, bits, group):
    """Decoded K of a token that is the only non-zero one of its group (K
    groups run along tokens)."""
    grp = np.zeros((1, 1, group, D), np.float32)
    grp[0, 0, t_in_group] = k_row
    kc, ks = O.pack_k(grp, bits, group)
    return O.dequant_k(kc, ks, grp.shape, bits, group)[0, 0, t_in_group].astype(np.float64)


def _decoded_v_row(v_row, bits, group):
    r = v_row.reshape(1, 1, 1, D).astype(np.float32)
    vc, vs = O.pack_v(r, bits, group)
    return O.dequant_v(vc, vs, r.shape, bits, group)[0, 0, 0].astype(np.float64)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("hq,r,group,variant", [
    (4, 1, 32, "mfma"),      # 4 rows: 4-row matrix-core kernel
    (16, 2, 32, "mfma"),     # 32 rows: 32-row matrix-core kernel
    (4, 1, 8, "stream"),     # streaming kernel, 4 rows, group 8 (scale arrays at the limit)
    (8, 1, 16, "stream"),    # streaming kernel, 8 rows
])
def test_largest_token_count(hq, r, group, variant, bits):
    import torch
    N = N_MAX[bits]
    rng = np.random.default_rng(21)
    a = rng.uniform(-1, 1, D).astype(np.float32)       # values of the zero-key tokens
    b = rng.uniform(-1, 1, D).astype(np.float32)       # value of token N - 1
    c = rng.uniform(-1, 1, D).astype(np.float32)       # value of token 0
    kdir = rng.standard_normal(D).astype(np.float32)
    kdir /= np.linalg.norm(kdir)
    # scores of the two special tokens about ln N, so all three classes weigh in
    k_last = (kdir * 19.0).astype(np.float32)
    k_first = (kdir * 16.0).astype(np.float32)
    q = np.zeros((1, hq, r, D), np.float32)
    q[:] = kdir * np.float32(math.sqrt(D))
    announce(f"max size N={N} {bits}-bit g{group} hq={hq} R={r} {variant}")
    dev = torch.device("cuda:0")
    k = torch.zeros((1, 1, N, D), dtype=torch.float32, device=dev)
    k[0, 0, N - 1] = torch.from_numpy(k_last).to(dev)
    k[0, 0, 0] = torch.from_numpy(k_first).to(dev)
    kc, ks = kvq.pack_k(k, bits, group)
    del k
    v = torch.from_numpy(a).to(dev).expand(1, 1, N, D).contiguous()
    v[0, 0, N - 1] = torch.from_numpy(b).to(dev)
    v[0, 0, 0] = torch.from_numpy(c).to(dev)
    vc, vs = kvq.pack_v(v, bits, group)
    del v
    torch.cuda.empty_cache()
    got = host(kvq.attend(torch.from_numpy(q).to(dev), kc, ks, vc, vs, N, bits, group,
                          variant=variant))

    ka = _decoded_k_row(k_first, 0, bits, group)
    kb = _decoded_k_row(k_last, (N - 1) % group, bits, group)
    s_first = float(q[0, 0, 0].astype(np.float64) @ ka) / math.sqrt(D)
    s_last = float(q[0, 0, 0].astype(np.float64) @ kb) / math.sqrt(D)
    m = max(s_first, s_last, 0.0)
    w0, w1, wr = math.exp(s_first - m), math.exp(s_last - m), (N - 2) * math.exp(-m)
    want = (w0 * _decoded_v_row(c, bits, group) + w1 * _decoded_v_row(b, bits, group) +
            wr * _decoded_v_row(a, bits, group)) / (w0 + w1 + wr)
    assert min(w0, w1, wr) / max(w0, w1, wr) > 1e-3     # every class matters
    err = np.max(np.abs(got - want[None, None, None, :]))
    assert err <= 1e-4, err
    del kc, ks, vc, vs
    torch.cuda.empty_cache()
