"""Checks of what a realigned batch must satisfy, independent of any implementation.

"Batch Speculative Decoding Done Right", section 2.1: rectangular alignment
(pad + content length equal for every row) and position-id contiguity (ids
0,1,.. over the content as the mask marks it); section 2.2: the new content of a
row is its old content followed by its committed tokens.  "Inference
Engineering Part 5/8", section "Draft Possible Tokens, Then Verify Them
Together": a cycle commits between 1 and D+1 tokens.
"""
import numpy as np


class InvariantError(AssertionError):
    pass


def _fail(msg):
    raise InvariantError(msg)


def unpad_row(tokens_row, mask_row, width):
    m = np.asarray(mask_row[:width]).astype(bool)
    return np.asarray(tokens_row[:width])[m]


def check_rect(tokens, pos, mask, lens, width, pad_token=0):
    """I1 rectangular alignment, I2 position-id contiguity, I5 tight width."""
    B = len(lens)
    pads = []
    for b in range(B):
        m = np.asarray(mask[b][:width]).astype(np.int64)
        c = int(lens[b])
        pad = width - c
        if pad < 0:
            _fail("row %d: length %d exceeds width %d" % (b, c, width))
        if not (np.all(m[:pad] == 0) and np.all(m[pad:] == 1)):
            _fail("row %d: mask is not 0^pad 1^len (rectangular alignment broken)" % b)
        want = np.concatenate([np.zeros(pad, np.int64), np.arange(c, dtype=np.int64)])
        if not np.array_equal(np.asarray(pos[b][:width]).astype(np.int64), want):
            _fail("row %d: position ids are not 0..len-1 over the content" % b)
        if not np.all(np.asarray(tokens[b][:pad]) == pad_token):
            _fail("row %d: pad positions do not hold the pad token" % b)
        pads.append(pad)
    if B and min(pads) != 0:
        _fail("width %d is not the longest row" % width)


def check_round(before_tokens, before_mask, before_width, after_tokens, after_pos, after_mask, after_lens,
                after_width, accept_len, committed, D, pad_token=0):
    """Full post-condition of one EQSPEC round on the token side.

    committed[b]: the ids the round commits for row b (accepted drafts + the
    replacement/bonus)."""
    B = len(accept_len)
    for b in range(B):
        a = int(accept_len[b])
        if not 0 <= a <= D:
            _fail("row %d: accepted length %d outside [0, D]" % (b, a))
        if not 1 <= len(committed[b]) <= D + 1 or len(committed[b]) != a + 1:
            _fail("row %d: commits %d tokens" % (b, len(committed[b])))
    check_rect(after_tokens, after_pos, after_mask, after_lens, after_width, pad_token)
    for b in range(B):
        old = unpad_row(before_tokens[b], before_mask[b], before_width)
        new = unpad_row(after_tokens[b], after_mask[b], after_width)
        want = np.concatenate([old, np.asarray(committed[b], dtype=old.dtype)])
        if not np.array_equal(new, want):
            _fail("row %d: content is not old content ++ committed tokens" % b)


def check_kv_round(kv_before, lens_before, width_before, kv_after, lens_after, width_after, kv_new, accept_len):
    """KV side: each (layer, K|V, row, head) sequence is old content ++ first
    a+1 speculative entries, left-padded with zeros to the new width."""
    L, two, B, H, _, Dh = kv_after.shape
    for b in range(B):
        c0, c1, n = int(lens_before[b]), int(lens_after[b]), int(accept_len[b]) + 1
        if c1 != c0 + n:
            _fail("row %d: length %d != %d + %d" % (b, c1, c0, n))
        old = kv_before[:, :, b, :, width_before - c0:width_before, :]
        want = np.concatenate([old, kv_new[:, :, b, :, :n, :]], axis=3)
        got = kv_after[:, :, b, :, width_after - c1:width_after, :]
        if not np.array_equal(got.view(np.uint8), want.view(np.uint8)):
            _fail("row %d: KV content is not old content ++ committed entries" % b)
        pad = kv_after[:, :, b, :, :width_after - c1, :]
        if np.any(pad.view(np.uint8) != 0):
            _fail("row %d: pad KV entries are not zero" % b)
