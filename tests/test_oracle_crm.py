"""Pins of the oracle's CRM routines (ScalingAttention, section 7.2: Compressed
Row Mask; section 7.3, Algorithm 2: the forward iterator).

* build_crm: numpy's packbits with little bit order over the dense keep
  matrix (library routine), read as little-endian uint32 words.
* crm_walk: numpy's nonzero over the unpacked words (library routine), and
  hand-built words whose walk is known (empty rows, full words, set bits
  only in the last word, padding bits above nKB).
* Together: crm_walk(build_crm(mask)) is the oracle's CSR, and the counts
  are the keep matrix's row sums.
"""
import numpy as np
import pytest

import oracle
import synth
from test_oracle_csr_sched import keep_matrix


def packbits_words(keep):
    """Dense bool [R][nKB] -> uint32 [R][ceil(nKB / 32)] via numpy.packbits."""
    R, nKB = keep.shape
    W = -(-nKB // 32)
    padded = np.zeros((R, W * 32), np.uint8)
    padded[:, :nKB] = keep
    return np.packbits(padded, axis=1, bitorder="little").view("<u4").astype(np.uint32)


@pytest.mark.parametrize("nKB", [1, 31, 32, 33, 64, 100])
@pytest.mark.parametrize("use_T", [False, True])
def test_build_crm_matches_packbits(nKB, use_T):
    rng = np.random.default_rng(nKB * 2 + use_T)
    R = 3 * nKB
    mask = (rng.random((R, nKB)) < 0.3).astype(np.uint8) if not use_T else None
    T = rng.random((R, nKB)).astype(np.float32) if use_T else None
    p = 0.3
    words = oracle.build_crm(mask, T, p, nKB, True)
    keep = keep_matrix(mask, T, p, nKB)
    np.testing.assert_array_equal(words, packbits_words(keep))
    # without the forced diagonal too
    words = oracle.build_crm(mask, T, p, nKB, False)
    np.testing.assert_array_equal(words, packbits_words(keep_matrix(mask, T, p, nKB, False)))


def test_build_crm_nan_threshold_never_kept():
    T = np.full((2, 40), np.nan, np.float32)
    T[1, 39] = -np.inf
    words = oracle.build_crm(None, T, 0.0, 2, False)
    assert words.tolist() == [[0, 0], [0, 1 << 7]]


@pytest.mark.parametrize("nKB", [5, 32, 70, 591])
def test_crm_walk_matches_nonzero(nKB):
    rng = np.random.default_rng(nKB)
    R = 40
    keep = rng.random((R, nKB)) < rng.random((R, 1))   # densities from 0 to 1 per row
    keep[3] = False
    keep[4] = True
    rp, col = oracle.crm_walk(packbits_words(keep), nKB)
    rr, cc = np.nonzero(keep)
    np.testing.assert_array_equal(col, cc.astype(np.int32))
    np.testing.assert_array_equal(rp, np.concatenate([[0], np.cumsum(keep.sum(1))]).astype(np.int32))


def test_crm_walk_hand_built_words():
    nKB = 96                                              # three words per row
    words = np.array([
        [0, 0, 0],                                        # empty row
        [1, 0, 0],                                        # block 0 only
        [0, 0, 0x80000000],                               # block 95 only: two empty words skipped
        [0xFFFFFFFF, 0, 0xFFFFFFFF],                      # full word, empty word, full word
        [0x80000001, 0x00010000, 0x00000002],             # 0, 31, 48, 65
    ], np.uint32)
    rp, col = oracle.crm_walk(words, nKB)
    rows = [col[rp[r]:rp[r + 1]].tolist() for r in range(len(words))]
    assert rows[0] == []
    assert rows[1] == [0]
    assert rows[2] == [95]
    assert rows[3] == list(range(32)) + list(range(64, 96))
    assert rows[4] == [0, 31, 48, 65]


def test_crm_walk_skips_padding_bits():
    nKB = 40                                              # last word holds blocks 32..39
    words = np.array([[0, 0xFFFFFF00], [0, 0xFFFFFFFF], [0x2, 0]], np.uint32)
    rp, col = oracle.crm_walk(words, nKB)
    assert rp.tolist() == [0, 0, 8, 9]
    assert col.tolist() == list(range(32, 40)) + [1]


@pytest.mark.parametrize("use_T", [False, True])
def test_crm_roundtrip_is_csr(use_T):
    w = synth.random_case(31, B=2, Hq=2, Hkv=1, N=128 * 75 - 17, d=8, block=128, density=0.25,
                          use_T=use_T)
    words = oracle.build_crm(w.mask, w.T, w.p, w.nQB, True)
    assert words.shape == (w.R, -(-w.nQB // 32))
    rp, col = oracle.crm_walk(words, w.nQB)
    rp2, col2, _ = oracle.build_csr(w.mask, w.T, w.p, None, w.nQB, True)
    np.testing.assert_array_equal(rp, rp2)
    np.testing.assert_array_equal(col, col2)


def test_crm_walk_capacity_error():
    words = np.array([[0xF]], np.uint32)
    row_ptr = np.zeros(2, np.int32)
    col = np.zeros(2, np.int32)
    n = oracle.lib().oracle_crm_walk(oracle._p(words), 1, 4, oracle._p(row_ptr), oracle._p(col), 2)
    assert n < 0
