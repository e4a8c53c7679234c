"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  Each mutation replaces one oracle function for the
duration of a test; the pin that must fail is run and expected to raise."""
import numpy as np
import pytest

import oracle.swa_oracle as so
import tests.test_oracle_pins as pins

_real_mask = so.key_mask
_real_rope = so.rope
_real_attention = so.swa_attention


def mask_wide(qpos, kpos, window, n_sink=0, dilation=1):       # i - W <= j <= i  (W + 1 keys)
    return _real_mask(qpos, kpos, window + 1, n_sink, dilation)


def mask_excl_self(qpos, kpos, window, n_sink=0, dilation=1):  # i - W <= j < i  (self excluded)
    qi = np.asarray(qpos)[:, None]
    kj = np.asarray(kpos)[None, :]
    return (kj < qi) & (kj >= qi - window) & (kj >= 0) | ((kj < n_sink) & (kj < qi) & (kj >= 0))


def mask_no_sinks(qpos, kpos, window, n_sink=0, dilation=1):
    return _real_mask(qpos, kpos, window, 0, dilation)


def mask_dil_span(qpos, kpos, window, n_sink=0, dilation=1):   # the span grows to W*d (W keys)
    return _real_mask(qpos, kpos, window * dilation, n_sink, dilation)


def mask_dil_phase(qpos, kpos, window, n_sink=0, dilation=1):  # keys at distance 1 (mod d) instead of 0
    qi = np.asarray(qpos, dtype=np.int64)[:, None]
    kj = np.asarray(kpos, dtype=np.int64)[None, :]
    causal = (kj <= qi) & (kj >= 0)
    d = int(dilation)
    win = (kj > qi - int(window)) & (((qi - kj) % d == (1 % d)) | (kj == qi))
    return causal & (win | (kj < int(n_sink)))


def mask_dil_ignored(qpos, kpos, window, n_sink=0, dilation=1):
    return _real_mask(qpos, kpos, window, n_sink, 1)


def rope_sign(x, pos, theta):                           # clockwise rotation
    return _real_rope(x, -np.asarray(pos), theta)


def rope_freq(x, pos, theta):                           # theta^(-k/D) instead of theta^(-2k/D)
    if theta == 0:
        return np.array(x, dtype=np.float64)
    D = np.asarray(x).shape[-1]
    return _real_rope(x, pos, theta ** 0.5) if D else x


def rope_halves(x, pos, theta):                         # pairs (k, k + D/2) instead of (2k, 2k+1)
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    perm = np.empty(D, dtype=int)
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    y = _real_rope(x[..., perm], pos, theta)
    out = np.empty_like(y)
    out[..., perm] = y
    return out


def attention_gqa_mod(q, k, v, qpos, kpos, window, n_sink=0, scale=None, rows_per_pass=256, dilation=1):
    # head h uses KV head h % Hkv instead of h // G
    q = np.asarray(q, dtype=np.float64)
    Hq, Hkv = q.shape[1], np.asarray(k).shape[1]
    G = Hq // Hkv
    perm = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
    inv = np.argsort(perm)
    o, l = _real_attention(q[:, inv], k, v, qpos, kpos, window, n_sink, scale, rows_per_pass, dilation)
    return o[:, perm], l[perm]


def attention_no_scale(q, k, v, qpos, kpos, window, n_sink=0, scale=None, rows_per_pass=256, dilation=1):
    return _real_attention(q, k, v, qpos, kpos, window, n_sink, 1.0 if scale is None else scale, rows_per_pass,
                           dilation)


def attention_kv_swapped(q, k, v, qpos, kpos, window, n_sink=0, scale=None, rows_per_pass=256, dilation=1):
    return _real_attention(q, v, k, qpos, kpos, window, n_sink, scale, rows_per_pass, dilation)


def prefill_write_first(cache, q, k, v, start, theta=10000.0, scale=None):
    # writes the chunk into the buffer before attending, then reads the buffer
    C = q.shape[0]
    pos = np.arange(start, start + C)
    k_rot = so.rope(k, pos, theta)
    cache.write(k_rot, np.asarray(v, dtype=np.float64), pos)
    ck, cv, cpos = cache.entries()
    return so.swa_attention(so.rope(q, pos, theta), ck, cv, pos, cpos, cache.window, cache.n_sink, scale,
                            dilation=cache.dilation)


class CacheFirstWriterWins(so.RollingCache):
    def write(self, k_rot, v, positions):
        for t, p in enumerate(np.asarray(positions)):
            s = self.slot(p)
            if self.tag[s] < 0 or self.tag[s] < p - self.window - 10**9:
                self.k[s], self.v[s], self.tag[s] = k_rot[t], v[t], int(p)


class CacheSlotModFull(so.RollingCache):                # sinks also roll: slot = p mod (W + S)
    def slot(self, p):
        return int(p) % (self.n_sink + self.window)


MUTATIONS = [
    ("key_mask", mask_wide, lambda: pins.test_scale_zero_counts_and_mean_position(7, 0)),
    ("key_mask", mask_wide, lambda: pins.test_key_set_of_decode_is_read_range()),
    ("key_mask", mask_excl_self, lambda: pins.test_window_one_returns_own_value()),
    ("key_mask", mask_no_sinks, lambda: pins.test_scale_zero_counts_and_mean_position(10, 3)),
    ("rope", rope_sign, lambda: pins.test_rope_closed_form_angles()),
    ("rope", rope_freq, lambda: pins.test_rope_closed_form_angles()),
    ("rope", rope_halves, lambda: pins.test_rope_matches_brute_force()),
    ("swa_attention", attention_gqa_mod, lambda: pins.test_gqa_equals_mha_with_replicated_kv()),
    ("swa_attention", attention_no_scale, lambda: pins.test_full_window_equals_sdpa(37, 4, 1, 16)),
    ("swa_attention", attention_kv_swapped, lambda: pins.test_full_window_equals_sdpa(37, 4, 1, 16)),
    ("prefill_chunk", prefill_write_first, lambda: pins.test_chunked_prefill_equals_unchunked(16, 0)),
    ("RollingCache", CacheFirstWriterWins, lambda: pins.test_rolling_buffer_w4_worked_example()),
    ("RollingCache", CacheSlotModFull, lambda: pins.test_rolling_decode_reproduces_full_sequence(3)),
    ("key_mask", mask_dil_span, lambda: pins.test_dilated_scale_zero_counts_and_mean_position(12, 0, 3)),
    ("key_mask", mask_dil_phase, lambda: pins.test_dilation_is_swa_within_each_residue(3)),
    ("key_mask", mask_dil_ignored, lambda: pins.test_dilated_matches_brute_force(14, 4, 2, 4, 9, 0, 2)),
    ("key_mask", mask_dil_span, lambda: pins.test_dilated_rolling_decode_reproduces_full_sequence(0, 3)),
]


@pytest.mark.parametrize("name,mutant,pin", MUTATIONS,
                         ids=[f"{n}-{m.__name__}" for n, m, _ in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, name, mutant, pin):
    pin()                                   # the real oracle passes the pin
    monkeypatch.setattr(so, name, mutant)
    with pytest.raises((AssertionError, ValueError)):
        pin()
