"""csa_decode_noalloc (the decode step with the library's own scratch array as its
workspace, for callers that cannot allocate) against csa_decode with a workspace of
the caller's, on the same inputs: two calls in a row, the second smaller than the
first, then the first shape again (the array keeps the previous call's contents), and
a step too large for the array rejected before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

from long_context_compressed_04_amd import csa
from long_context_compressed_04_amd import workloads as W

from _helpers import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    csa.lib()


def _i32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).cuda()


def _pair(B, T, seed, k=1024):
    """Two decoders over the same inputs with separate outputs: one for each entry point."""
    c = W.csa_decode(seed, B=B, T=T, k=k)
    ins = (dev(c["q"][:, None]), dev(c["kv"]), dev(c["kv_raw"]), _i32(c["raw_base"]), _i32(c["q_pos"][:, None]),
           dev(c["qI"][:, None]), dev(c["w"][:, None]), dev(c["kI"]), _i32(c["n_entries"]))
    mk = lambda: csa.Decoder(*ins, m=4, topk=k, window=128,
                             lse=torch.empty((B, 1, 128), dtype=torch.float32, device="cuda"))
    return mk(), mk()


def _check_same(ref, na):
    out_r, idx_r = ref()
    out_n, idx_n = na.call_noalloc()
    torch.cuda.synchronize()
    # the same kernels in the same configuration: identical results
    assert torch.equal(idx_r, idx_n)
    assert torch.equal(out_r.view(torch.int16), out_n.view(torch.int16))
    assert torch.equal(ref.lse, na.lse)


def csa_noalloc_bytes():
    return 32 << 20               # CSA_NOALLOC_SCRATCH_BYTES


def test_noalloc_matches_decode():
    big = _pair(8, 65536, 5)          # the 64K workload's shape: 26.6 MiB of workspace
    small = _pair(2, 12000, 6, k=256)
    assert csa.lib().csa_decode_workspace_size(ctypes.byref(big[1].args)) <= csa_noalloc_bytes()
    _check_same(*big)
    _check_same(*small)               # smaller, in the array the first call filled
    _check_same(*big)


def test_noalloc_rejects_a_step_beyond_the_scratch():
    ref, na = _pair(64, 16384, 7)     # 64 sequences of 4,096 entries: 65 MiB of workspace
    need = csa.lib().csa_decode_workspace_size(ctypes.byref(na.args))
    assert need > csa_noalloc_bytes()
    na.out.fill_(0)
    with pytest.raises(csa.CsaError) as e:
        na.call_noalloc()
    assert e.value.status == 5 and b"scratch" in csa.lib().csa_last_error()
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(na.out.view(torch.int16))) == 0   # nothing ran
