"""GPU parity of the head exchange layout calls (cp_a2a_pack, cp_a2a_unpack
and their inverses) against the oracle's index-by-index definitions, through
the C ABI.  Data movement only: every comparison is bit-exact (bf16 compared
as its 16-bit patterns)."""
import numpy as np
import pytest
import torch

import oracle as orc
import context_causal_attention_amd as cpa
from gpu_cases import announce

pytestmark = pytest.mark.gpu

_BITS = {torch.bfloat16: torch.int16, torch.float32: torch.int32}


def _bits(t):
    """The tensor's raw bits as a numpy integer array (exact for any dtype)."""
    return t.contiguous().view(_BITS[t.dtype]).cpu().numpy()


def _rand(shape, dtype, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_pack_unpack_and_inverses(dtype, d, g):
    """Ragged rows (1000: not a multiple of the 256-thread blocks' rows)."""
    rows, H = 1000, 32
    announce(f"a2a {dtype} d={d} g={g}")
    x = _rand((rows, H, d), dtype, seed=80 + g).cuda()
    send = cpa.cp_a2a_pack(x, g)
    assert np.array_equal(_bits(send), orc.a2a_pack(_bits(x), g))
    back = torch.zeros_like(x)
    cpa.cp_a2a_pack_inverse(send, back)
    assert torch.equal(back.view(_BITS[dtype]), x.view(_BITS[dtype]))
    recv = _rand((g, H // g, rows, d), dtype, seed=90 + g).cuda()
    y = cpa.cp_a2a_unpack(recv)
    assert np.array_equal(_bits(y), orc.a2a_unpack(_bits(recv)))
    r2 = cpa.cp_a2a_unpack_inverse(y, g)
    assert torch.equal(r2.view(_BITS[dtype]), recv.view(_BITS[dtype]))


def test_strided_shard_rows():
    """The shard as a row-range view of a wider buffer: row stride 40 heads * d."""
    rows, H, d, g = 300, 32, 128, 4
    announce("a2a strided shard")
    wide = _rand((rows, 40, d), torch.bfloat16, seed=81).cuda()
    x = wide[:, 3:3 + H]
    assert x.stride(0) == 40 * d and x.stride(1) == d
    send = cpa.cp_a2a_pack(x, g)
    assert np.array_equal(_bits(send), orc.a2a_pack(_bits(x), g))
    target = torch.zeros_like(wide)
    cpa.cp_a2a_pack_inverse(send, target[:, 3:3 + H])
    assert torch.equal(target[:, 3:3 + H].view(torch.int16), x.view(torch.int16))
    assert torch.all(target[:, :3] == 0) and torch.all(target[:, 3 + H:] == 0)


@pytest.mark.parametrize("g", [2, 8])
def test_whole_exchange_gives_head_blocks(g):
    """g ranks' sequence shards of one tensor X [S, H, d]: pack on each rank,
    the exchange (done here with plain indexing, it is the collective's part),
    unpack on each rank; rank j then holds X[:, heads of j] head-major, and the
    reverse path restores every shard."""
    rows, H, d = 512, 32, 128
    announce(f"a2a whole exchange g={g}")
    X = _rand((g * rows, H, d), torch.bfloat16, seed=82).cuda()
    sends = [cpa.cp_a2a_pack(X[i * rows:(i + 1) * rows], g) for i in range(g)]
    recvs = [torch.stack([sends[i][j] for i in range(g)]) for j in range(g)]
    Xb = _bits(X)
    ref = [orc.a2a_unpack(r) for r in orc.a2a_exchange([orc.a2a_pack(Xb[i * rows:(i + 1) * rows], g)
                                                         for i in range(g)])]
    Hg = H // g
    ys = []
    for j in range(g):
        y = cpa.cp_a2a_unpack(recvs[j])
        assert np.array_equal(_bits(y), ref[j])
        assert np.array_equal(_bits(y), np.transpose(Xb, (1, 0, 2))[j * Hg:(j + 1) * Hg])
        ys.append(y)
    back_blocks = [cpa.cp_a2a_unpack_inverse(ys[j], g) for j in range(g)]
    for i in range(g):
        recv_back = torch.stack([back_blocks[j][i] for j in range(g)])
        shard = torch.empty(rows, H, d, dtype=torch.bfloat16, device="cuda")
        cpa.cp_a2a_pack_inverse(recv_back, shard)
        assert torch.equal(shard.view(torch.int16), X[i * rows:(i + 1) * rows].view(torch.int16))


def test_bench_size_and_empty():
    """The 131072-token cp=8 shard (16384 rows, 32 heads, d = 128, bf16), and rows = 0."""
    rows, H, d, g = 16384, 32, 128, 2
    announce("a2a 16384 rows")
    x = _rand((rows, H, d), torch.bfloat16, seed=83).cuda()
    send = cpa.cp_a2a_pack(x, g)
    y = cpa.cp_a2a_unpack(send)
    xb = _bits(x)
    assert np.array_equal(_bits(send), orc.a2a_pack(xb, g))
    assert np.array_equal(_bits(y), orc.a2a_unpack(orc.a2a_pack(xb, g)))
    e = torch.empty(0, H, d, dtype=torch.bfloat16, device="cuda")
    assert cpa.cp_a2a_pack(e, g).numel() == 0
