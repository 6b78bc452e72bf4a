"""CPU-only: the tables the packed-document path builds, and the update
kernel's per-step arithmetic on them, for the layouts the GPU tests run.

The block table and the apply's tile list come from the library itself
(ttt_packed_tables, host code only). Everything the kernels then derive
from them is emulated here step by step in plain Python integers:

* load_step_bits: every lane l of a packed update workgroup holds the
  chunk-start and document-start bits of K steps 32 l .. 32 l + 31 (one step
  = one 64-token block) and the chunk of step 32 l;
* the update's hook at step kt: it reads lane kt >> 5's registers, resets the
  state at a document start (kt > 0) and stores nothing there, and at any
  other chunk start stores the snapshot into slot base + popcount(chunk-start
  bits of steps 32 l + 1 .. kt), clamped to the chunk count;
* the apply reads, for each tile, the slot its table entry names.

Each is checked against what the document starts alone imply (iplexlaw
explainer §6: the state returns to W_down0 at every document start, the
chunks restart there): every chunk that does not start a document is stored
exactly once, in its own slot; every document's first chunk reads slot 0
(which holds W_down0, stored at step 0); every tile lies in one chunk and
the tiles cover the sequence once; every step's conv bounds are its
document's and chunk's ends.
"""
import os

import pytest

from test_layer_gate_amd import _binding as bnd

CHUNK_START, DOC_START = 1, 2
U32 = 0xFFFFFFFF

LAYOUTS = {
    # the 64k Qwen3-4B five-document layout of test_packed_full_size_sampled
    "five_uneven_64k": (65536, 1024, [0, 20480, 21568, 45056, 63488]),
    # the 32 equal documents bench.py --variant packed times
    "equal32_64k": (65536, 1024, list(range(0, 65536, 2048))),
    # the 131072-token step limit of test_packed_at_the_step_limit
    "limit_128k": (131072, 256, [0, 640, 65536, 130560, 131008]),
    # the mid-size layouts of test_packed_matches_oracle
    "mixed": (2048, 256, [0, 512, 576, 1344]),
    "tiny_docs": (2048, 256, list(range(0, 2048, 64))),
    "ragged": (1000, 128, [0, 320, 640]),
}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bnd.LIB_PATH):
        pytest.fail("libttt_layer.so is not built (run __graft_entry__.build())")
    return bnd.lib()


def expected_steps(T, C, starts):
    """Per 64-token block (index = K step), from the document starts alone:
    (global chunk index, chunk starts here, document starts here, document
    end, chunk end)."""
    out = []
    bounds = list(starts) + [T]
    n = 0
    for r in range(len(starts)):
        a, e = bounds[r], bounds[r + 1]
        for c0 in range(a, e, C):
            c1 = min(e, c0 + C)
            for t in range(c0, c1, 64):
                out.append((n, t == c0, t == a, e, c1))
            n += 1
    return out, n


def step_bits(blocks, nk, n_chunks):
    """The per-lane registers load_step_bits builds (64 lanes)."""
    lanes = []
    for lane in range(64):
        cs = ds = base = 0
        for j in range(32):
            k = lane * 32 + j
            if k < nk:
                chunk, flags = blocks[k][0], blocks[k][1]
                word = (chunk & 0x3FFFFFFF) | ((flags & 3) << 30)
                if (word >> 30) & CHUNK_START:
                    cs |= 1 << j
                if (word >> 30) & DOC_START:
                    ds |= 1 << j
                if j == 0:
                    base = min(word & 0x3FFFFFFF, n_chunks - 1)
        lanes.append((cs, ds, base))
    return lanes


def hook(lanes, kt, n_chunks):
    """What the packed update's hook does at step kt: ("reset", None),
    ("store", slot) or (None, None)."""
    lane, bit = kt >> 5, kt & 31
    cs, ds, base = lanes[lane]
    doc = bool((ds >> bit) & 1) and kt > 0
    if doc:
        return "reset", None
    if not (cs >> bit) & 1:
        return None, None
    later = (((2 << bit) & U32) - 1) & U32 & ~1
    return "store", min(base + bin(cs & later).count("1"), n_chunks - 1)


@pytest.mark.parametrize("name", sorted(LAYOUTS))
def test_packed_tables_and_update_steps(lib, name):
    T, C, starts = LAYOUTS[name]
    desc = bnd.make_desc(1, T, 2560, 9728, 4)
    blocks, tiles, n_chunks = bnd.packed_tables(desc, C, starts)
    want, n_want = expected_steps(T, C, starts)
    assert n_chunks == n_want
    nk = -(-T // 64)                     # the update's K steps over the sequence
    T_pad = -(-T // 256) * 256
    assert len(blocks) == T_pad // 64
    for k, (chunk, cstart, dstart, dend, cend) in enumerate(want):
        assert blocks[k] == (chunk, (CHUNK_START if cstart else 0) | (DOC_START if dstart else 0),
                             dend, cend), f"block {k}"
    for k in range(len(want), len(blocks)):
        assert blocks[k] == (n_chunks - 1, 0, T, T), f"padding block {k}"
    assert nk <= 2048, "the step registers hold 2048 steps"

    lanes = step_bits(blocks, nk, n_chunks)
    stored = {}
    # hook(0) runs before the loop and always stores slot 0 (kt = 0 is a
    # chunk and document start, and never a reset)
    act, slot = hook(lanes, 0, n_chunks)
    assert act == "store" and slot == 0
    stored[0] = 0
    resets = []
    for kt in range(1, nk):
        act, slot = hook(lanes, kt, n_chunks)
        chunk, cstart, dstart, _, _ = want[kt]
        if dstart:
            assert act == "reset", f"step {kt}: document start without a reset"
            resets.append(kt)
        elif cstart:
            assert act == "store" and slot == chunk, f"step {kt}: slot {slot} for chunk {chunk}"
            assert slot not in stored, f"slot {slot} stored twice"
            stored[slot] = kt
        else:
            assert act is None, f"step {kt}: {act} inside a chunk"
    assert resets == [s // 64 for s in starts[1:]]
    doc_first = {want[s // 64][0] for s in starts}
    assert set(stored) == ({c for c in range(n_chunks) if c not in doc_first} | {0})

    # apply tiles: inside one chunk, covering [0, T) once, the right slot
    covered = 0
    for t0, t1, snap in tiles:
        assert t0 == covered and t0 < t1 <= T and t1 - t0 <= 256
        chunk, _, _, _, cend = want[t0 // 64]
        assert t1 <= cend, "a tile straddles a chunk end"
        assert snap == (0 if chunk in doc_first else chunk)
        assert snap in stored
        covered = t1
    assert covered == T


def test_packed_tables_reject_bad_layouts(lib):
    desc = bnd.make_desc(1, 4096, 256, 1024, 4)
    with pytest.raises(bnd.TTTError) as e:
        bnd.packed_tables(desc, 256, [0, 100])
    assert e.value.name == "TTT_ERR_UNSUPPORTED"
    with pytest.raises(bnd.TTTError) as e:
        bnd.packed_tables(desc, 256, [0, 512, 512])
    assert e.value.name == "TTT_ERR_INVALID_ARG"
    with pytest.raises(bnd.TTTError) as e:
        bnd.packed_tables(bnd.make_desc(1, 131073, 256, 1024, 4), 256, [0])
    assert e.value.name == "TTT_ERR_UNSUPPORTED"
