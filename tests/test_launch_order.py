"""The work-item maps of the forward launch and of the dQ/dK/dV launch,
restated from their definitions and checked on the CPU for many shapes.

A launch has `total` workgroups.  With total a multiple of 8 the hardware's
round-robin over the eight XCDs is undone (workgroup i goes to position
(i mod 8) * total/8 + i div 8).  Positions are split into groups of G heads,
one group per XCD, and a group into chunks of `chunk` heads, block-major
within a chunk; the dQ/dK/dV launch has both kinds per block.  The maps
must reach every (head, block) of every kind exactly once, with every other
position a padding head past the last, for every chunk size the launchers
choose."""
import pytest

from test_gpu_parity import _order_chunk


def _remap(i, total):
    return (i & 7) * (total >> 3) + (i >> 3) if total % 8 == 0 else i


def _forward_items(BH, n, chunk):
    G = (BH + 7) // 8
    total = -(-BH // G) * G * n
    for i in range(total):
        g, r = divmod(_remap(i, total), G * n)
        ck, cw = divmod(r, chunk * n)
        yield g * G + ck * chunk + cw % chunk, n - 1 - cw // chunk


def _grads_items(BH, n, chunk):
    G = (BH + 7) // 8
    total = -(-BH // G) * 2 * G * n
    pc = chunk * n
    for i in range(total):
        g, r = divmod(_remap(i, total), 2 * G * n)
        if 1 < chunk < G:  # each chunk's dK/dV workgroups, then its dQ ones
            c, w = divmod(r, 2 * pc)
            dq = w >= pc
            r2 = c * pc + (w - pc if dq else w)
        else:  # the group's dK/dV workgroups, then its dQ ones
            dq = r >= G * n
            r2 = r - G * n if dq else r
        ck, cw = divmod(r2, pc)
        yield dq, g * G + ck * chunk + cw % chunk, cw // chunk


SHAPES = [(BH, n) for BH in (1, 3, 8, 11, 40, 44, 48, 112, 128, 200) for n in (1, 2, 7, 32, 60)]


@pytest.mark.parametrize("BH,n", SHAPES)
@pytest.mark.parametrize("d", [64, 128])
def test_every_block_once(BH, n, d):
    G = (BH + 7) // 8
    chunks = {_order_chunk(BH, n, 1, d), _order_chunk(BH, n, 2, d), 1, G}
    chunks |= {c for c in (2, 4) if G % c == 0}
    for chunk in sorted(chunks):
        fwd = [(bh, qb) for bh, qb in _forward_items(BH, n, chunk) if bh < BH]
        assert sorted(fwd) == [(bh, qb) for bh in range(BH) for qb in range(n)], chunk
        grads = [it for it in _grads_items(BH, n, chunk) if it[1] < BH]
        assert sorted(grads) == [(dq, bh, b) for dq in (False, True) for bh in range(BH) for b in range(n)], chunk


def test_chunk_choice():
    # short launches block-major over the group; long causal ones in chunks of
    # four, two or one head by the group's head count; non-causal head-major
    assert _order_chunk(32, 8, 1, 64) == 4          # 256 workgroups
    assert _order_chunk(128, 32, 1, 128) == 4       # 4x32x4096x128: 4096 > 2816
    assert _order_chunk(48, 22, 1, 128) == 6        # 1056 workgroups
    assert _order_chunk(48, 60, 1, 128) == 2
    assert _order_chunk(40, 72, 1, 128) == 1
    assert _order_chunk(128, 32, 1, 128, causal=False) == 1
    assert _order_chunk(256, 8, 2, 64) == 32        # 16x16x1024x64: 4096 workgroups, 5.3 rounds
