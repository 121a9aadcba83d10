"""The pins are strong enough: plant plausible mistakes in copies of the
oracle (on the CPU) and check that at least one pin fails for each, while the
real oracle passes them all."""

import copy

import numpy as np
import pytest

import oracle
from oracle import BlockManagerError, BlockManagerModel
from tests import pins


def plain_decode(mistake=None):
    """The decode definition with one planted mistake (None = correct)."""
    def decode(q, kv, bt, cl, scale, window=0):
        q = np.asarray(q, dtype=np.float64)
        S, Hq, D = q.shape
        Hkv, bs = kv.shape[2], kv.shape[3]
        G = Hq // Hkv
        out = np.zeros((S, Hq, D))
        for s in range(S):
            n = int(cl[s])
            if mistake == "whole_last_block":
                n = -(-n // bs) * bs
            if n == 0:
                continue
            lo = max(0, n - window) if window > 0 else 0
            if mistake == "window_off_by_one" and window > 0:
                lo = max(0, n - window - 1)
            t = np.arange(lo, n)
            row = (t + 1) % bs if mistake == "row_off_by_one" else t % bs
            blk = np.asarray(bt[s])[t // bs]
            k = kv[blk, 0, :, row, :].astype(np.float64)
            v = kv[blk, 1, :, row, :].astype(np.float64)
            if mistake == "k_v_swapped":
                k, v = v, k
            for h in range(Hq):
                g = h % Hkv if mistake == "gqa_modulo" else h // G
                sc = 1.0 if mistake == "scale_dropped" else scale
                z = sc * (k[:, g] @ q[s, h])
                if mistake == "per_block_softmax":   # the block loop some pages print
                    o = np.zeros(D)
                    for b0 in range(0, len(t), bs):
                        zz = z[b0:b0 + bs]
                        w = np.exp(zz - zz.max())
                        o += (w / w.sum()) @ v[b0:b0 + bs, g]
                    out[s, h] = o
                    continue
                w = np.exp(z.max() - z) if mistake == "sign_flipped" else np.exp(z - z.max())
                out[s, h] = (w @ v[:, g]) / w.sum()
        return out
    return decode


DECODE_MISTAKES = ["whole_last_block", "row_off_by_one", "k_v_swapped", "gqa_modulo",
                   "scale_dropped", "per_block_softmax", "sign_flipped"]


def window_pins_fail(decode):
    ok = all(pins.window_is_sdpa_on_last_tokens(decode, w) for w in (1, 7, 33))
    return not (ok and pins.window_one_is_last_value(decode))


def test_window_pins_catch_off_by_one_and_pass_the_oracle():
    assert not window_pins_fail(oracle.decode_ref)
    assert not window_pins_fail(plain_decode(None))
    assert window_pins_fail(plain_decode("window_off_by_one"))


def test_real_oracle_passes_every_decode_pin():
    assert pins.failing(oracle.decode_ref) == []
    assert pins.failing(plain_decode(None)) == []


@pytest.mark.parametrize("mistake", DECODE_MISTAKES)
def test_decode_pins_catch_planted_mistake(mistake):
    assert pins.failing(plain_decode(mistake)), mistake


def cache_write_mutant(mistake):
    def write(kv, key, value, slots, cow_pairs=()):
        out = np.array(kv, copy=True)
        bs = out.shape[3]

        def copies():
            for src, dst in cow_pairs:
                out[int(dst)] = out[int(src)]
        if mistake != "copy_after_scatter":
            copies()
        for i, slot in enumerate(np.asarray(slots).tolist()):
            if slot < 0:
                continue
            b, o = divmod(int(slot), bs)
            if mistake == "row_from_block":
                b, o = o % out.shape[0], b % bs
            kk, vv = (value[i], key[i]) if mistake == "k_v_swapped" else (key[i], value[i])
            out[b, 0, :, o, :] = kk
            out[b, 1, :, o, :] = vv
        if mistake == "copy_after_scatter":
            copies()
        return out
    return write


def test_real_cache_write_passes_its_pins():
    assert pins.cache_round_trip(oracle.cache_write_ref, oracle.gather_sequence)
    assert pins.cow_before_scatter(oracle.cache_write_ref)


@pytest.mark.parametrize("mistake", ["row_from_block", "k_v_swapped", "copy_after_scatter"])
def test_cache_pins_catch_planted_mistake(mistake):
    w = cache_write_mutant(mistake)
    assert not (pins.cache_round_trip(w, oracle.gather_sequence) and pins.cow_before_scatter(w))


class ForkWithoutRefs(BlockManagerModel):
    def fork(self, parent, child):
        self._need(parent)
        self.tables[child] = list(self.tables[parent])
        self.num_tokens[child] = self.num_tokens[parent]


class NoCopyOnWrite(BlockManagerModel):
    def append_slot(self, seq):
        self._need(seq)
        table = self.tables[seq]
        t = self.num_tokens[seq]
        if t % self.block_size == 0:
            table.append(self._take())
        self.num_tokens[seq] = t + 1
        return table[-1] * self.block_size + t % self.block_size, -1, -1


class FreeIgnoresRefs(BlockManagerModel):
    def free(self, seq):
        self._need(seq)
        for b in self.tables.pop(seq):
            self.ref_counts[b] = 0
            if b not in self.free_blocks:
                self.free_blocks.append(b)
        del self.num_tokens[seq]


def test_real_block_manager_passes_its_pins():
    assert pins.bm_fork_cow_example(BlockManagerModel)
    assert pins.bm_scripted_lifecycle(BlockManagerModel)


@pytest.mark.parametrize("cls", [ForkWithoutRefs, NoCopyOnWrite, FreeIgnoresRefs])
def test_block_manager_pins_catch_planted_mistake(cls):
    def passes(pin):
        try:
            return pin(cls)
        except (BlockManagerError, KeyError, IndexError, AssertionError):
            return False
    assert not (passes(pins.bm_fork_cow_example) and passes(pins.bm_scripted_lifecycle))


# --------------------------------------------------------------------------
# INT8 quantisation mutants
# --------------------------------------------------------------------------
def quantize_mutant(mistake):
    def quantize(x):
        xf = np.asarray(x).astype(np.float32)
        if mistake == "per_tensor":
            amax = np.broadcast_to(np.abs(xf).max(), xf.shape[:-1])
        else:
            amax = np.abs(xf).max(axis=-1)
        q = np.float32(128 if mistake == "divide_by_128" else 127)
        scales = (amax / q).astype(np.float32)
        codes = np.zeros(xf.shape, dtype=np.int8)
        live = scales > 0
        r = xf[live] / scales[live][..., None]
        if mistake == "truncate":
            r = np.trunc(r)
        elif mistake == "half_away":
            r = np.sign(r) * np.floor(np.abs(r) + 0.5)
        else:
            r = np.rint(r)
        codes[live] = np.clip(r, -127, 127).astype(np.int8)
        return codes, scales
    return quantize


@pytest.mark.parametrize("mistake", ["per_tensor", "divide_by_128", "truncate", "half_away"])
def test_quant_pins_catch(mistake):
    assert pins.quant_failing(quantize_mutant(mistake), oracle.dequantize_ref)


def test_quant_pins_pass_oracle_and_clean_copy():
    assert not pins.quant_failing(oracle.quantize_rows_ref, oracle.dequantize_ref)
    assert not pins.quant_failing(quantize_mutant(None), oracle.dequantize_ref)


def i8_write_mutant(mistake):
    def write(codes, scales, key, value, slots, cow_pairs=()):
        codes, scales = np.array(codes, copy=True), np.array(scales, copy=True)
        bs = codes.shape[3]
        for src, dst in cow_pairs:
            codes[dst] = codes[src]
            if mistake != "cow_skips_scales":
                scales[dst] = scales[src]
        kq, ks = oracle.quantize_rows_ref(key)
        vq, vs = oracle.quantize_rows_ref(value)
        if mistake == "scales_swapped":
            ks, vs = vs, ks
        for i, slot in enumerate(np.asarray(slots).tolist()):
            if slot < 0:
                continue
            b, r = divmod(int(slot), bs)
            rs = 0 if mistake == "scale_row_zero" else r
            codes[b, 0, :, r], codes[b, 1, :, r] = kq[i], vq[i]
            scales[b, :, 0, rs], scales[b, :, 1, rs] = ks[i], vs[i]
        return codes, scales
    return write


@pytest.mark.parametrize("mistake", ["cow_skips_scales", "scales_swapped", "scale_row_zero"])
def test_i8_write_pins_catch(mistake):
    w = i8_write_mutant(mistake)
    ok = (pins.i8_cache_round_trip(w, oracle.quantize_rows_ref, oracle.dequantize_ref)
          and pins.i8_cow_before_scatter(w))
    assert not ok
    c = i8_write_mutant(None)
    assert pins.i8_cache_round_trip(c, oracle.quantize_rows_ref, oracle.dequantize_ref)
    assert pins.i8_cow_before_scatter(c)


# --------------------------------------------------------------------------
# prefix-cache mutants
# --------------------------------------------------------------------------
import oracle.block_manager as obm


class PositionFreeMatch(BlockManagerModel):
    """Matches a prompt block with any cached block holding the same tokens,
    wherever it stood."""

    def allocate_prompt(self, seq, tokens):
        by_tokens = {tuple(k[2]): b for b, k in self.block_key.items()}
        bs = self.block_size
        first = tokens[:bs]
        b = by_tokens.get(tuple(int(t) for t in first))
        if b is not None and len(tokens) >= bs:
            # pretend the block was cached under the chain that leads here
            h, _, toks = self.block_key[b]
            del self.cache[h]
            nh = obm.block_hash(0, toks)
            self.cache[nh] = b
            self.block_key[b] = (nh, 0, toks)
        return super().allocate_prompt(seq, tokens)


class MostRecentEviction(BlockManagerModel):
    def _take(self):
        if not self.free_blocks and self.evictable:
            newest = max(self.evictable, key=lambda b: self.evictable[b][1])
            self.evictable[newest] = (False, -1)          # make it the victim
        return super()._take()


class NoProtection(BlockManagerModel):
    def enable_prefix_cache(self, protect_hits=0, admit_after=1):
        super().enable_prefix_cache(0, admit_after)


class AdmitsOneEarly(BlockManagerModel):
    """The admission threshold applied as 'at least admit_after - 1'."""

    def enable_prefix_cache(self, protect_hits=0, admit_after=1):
        super().enable_prefix_cache(protect_hits, max(1, admit_after - 1))


class UnboundedAdmissionTable(BlockManagerModel):
    def _admission_capacity(self):
        return 1 << 40


class CachesPartialBlocks(BlockManagerModel):
    def register(self, seq):
        added = super().register(seq)
        n = len(self.tokens[seq])
        if n % self.block_size and len(self.tables[seq]) > n // self.block_size:
            b = self.tables[seq][n // self.block_size]
            if b not in self.block_key:
                h = obm.block_hash(0, self.tokens[seq][-(n % self.block_size):] + [seq])
                self.cache[h] = b
                self.block_key[b] = (h, 0, [])
                added += 1
        return added


class NoReferenceOnHit(BlockManagerModel):
    def allocate_prompt(self, seq, tokens):
        table, cached = super().allocate_prompt(seq, tokens)
        for b in table[:cached // self.block_size]:
            if self.ref_counts[b] > 1:
                self.ref_counts[b] -= 1
        return table, cached


PREFIX_PINS = [pins.system_prompt_stored_once, pins.position_matters,
               pins.multi_turn_reuses_full_blocks, pins.lru_spares_referenced_blocks,
               pins.protection_keeps_hot_prefix,
               pins.admission_threshold_keeps_one_shot_prompts_out,
               pins.admission_table_is_bounded]


def _prefix_pins_fail(cls):
    bad = []
    for p in PREFIX_PINS:
        try:
            ok = p(cls)
        except BlockManagerError:
            ok = False
        if not ok:
            bad.append(p.__name__)
    return bad


@pytest.mark.parametrize("cls", [PositionFreeMatch, MostRecentEviction, NoProtection,
                                 CachesPartialBlocks, NoReferenceOnHit, AdmitsOneEarly,
                                 UnboundedAdmissionTable])
def test_prefix_pins_catch(cls):
    assert _prefix_pins_fail(cls), cls.__name__


def test_prefix_pins_pass_the_model():
    assert not _prefix_pins_fail(BlockManagerModel)


# --------------------------------------------------------------------------
# multi-token (causal) mutants
# --------------------------------------------------------------------------
def prefill_mutant(mistake):
    def prefill(q, kv, bt, cl, qstart, scale, window=0):
        q = np.asarray(q, dtype=np.float64)
        total, hq, d = q.shape
        hkv, bs = kv.shape[2], kv.shape[3]
        G = hq // hkv
        out = np.zeros((total, hq, d))
        for s in range(len(cl)):
            n, q0, q1 = int(cl[s]), int(qstart[s]), int(qstart[s + 1])
            T = q1 - q0
            t = np.arange(n)
            blk = np.asarray(bt[s])[t // bs]
            k = kv[blk, 0, :, t % bs, :].astype(np.float64)
            v = kv[blk, 1, :, t % bs, :].astype(np.float64)
            for i in range(T):
                p = n - T + i
                if mistake == "top_left":       # the square mask applied to the first keys
                    p = i
                if mistake == "strict":
                    p -= 1
                p = max(p, 0)
                lo = max(0, p + 1 - window) if window > 0 else 0
                if mistake == "window_off_by_one" and window > 0:
                    lo = max(0, p - window)
                if mistake == "window_from_context_end" and window > 0:
                    lo = min(p, max(0, n - window))     # the decode's window for every query
                for h in range(hq):
                    z = scale * (k[lo:p + 1, h // G] @ q[q0 + i, h])
                    w = np.exp(z - z.max())
                    out[q0 + i, h] = (w @ v[lo:p + 1, h // G]) / w.sum()
        return out
    return prefill


def _prefill_pins_fail(f):
    return not (pins.prefill_is_masked_sdpa(f) and pins.chunked_equals_whole(f)
                and pins.prefill_single_token_is_decode(f, oracle.decode_ref))


@pytest.mark.parametrize("mistake", ["top_left", "strict"])
def test_prefill_pins_catch(mistake):
    assert _prefill_pins_fail(prefill_mutant(mistake))


def test_prefill_pins_pass_clean_copy():
    assert not _prefill_pins_fail(prefill_mutant(None))
    assert not _prefill_pins_fail(oracle.prefill_ref)


def _prefill_window_pins_fail(f):
    ok = all(pins.prefill_window_is_banded_sdpa(f, w) for w in (1, 3, 16, 39))
    return not (ok and pins.prefill_window_one_is_own_value_row(f))


@pytest.mark.parametrize("mistake", ["window_off_by_one", "window_from_context_end"])
def test_prefill_window_pins_catch(mistake):
    assert _prefill_window_pins_fail(prefill_mutant(mistake))


def test_prefill_window_pins_pass_clean_copy():
    assert not _prefill_window_pins_fail(prefill_mutant(None))
    assert not _prefill_window_pins_fail(oracle.prefill_ref)


def i8_prefill_mutant(mistake):
    """The INT8 prefill as the dequantised pool's prefill, with a planted
    mistake in how the scales are read."""
    def prefill(q, codes, scales, bt, cl, qstart, scale, window=0):
        sc = np.asarray(scales)
        if mistake == "scales_swapped":            # K and V scales exchanged
            sc = sc[:, :, ::-1, :]
        per_row = np.swapaxes(sc, 1, 2)
        if mistake == "scales_as_codes_layout":    # [NB, 2, Hkv, bs] read as [NB, Hkv, 2, bs]
            per_row = sc.reshape(sc.shape[0], sc.shape[2], sc.shape[1], sc.shape[3])
        return oracle.prefill_ref(q, oracle.dequantize_ref(codes, per_row), bt, cl, qstart,
                                  scale, window=window)
    return prefill


@pytest.mark.parametrize("mistake", ["scales_swapped", "scales_as_codes_layout"])
def test_i8_prefill_pins_catch(mistake):
    assert not pins.i8_prefill_is_masked_sdpa_on_dequantised(i8_prefill_mutant(mistake))
    assert pins.i8_prefill_is_masked_sdpa_on_dequantised(i8_prefill_mutant(None))
