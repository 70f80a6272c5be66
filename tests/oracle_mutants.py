"""Planted mistakes in the oracle, for checking that its CPU pins catch them.

Each mutant names an oracle module, a piece of its source text that must
occur exactly once, and the text that replaces it: a plausible slip (a dropped
term, a wrong sign or index, a swapped operand, a changed rounding rule).
`apply(name)` re-executes the module's source with the replacement in the
module's own namespace, so every caller of the module sees the mutated code,
including tables the module builds at import time. Nothing here is imported
by the library, the oracle or the GPU tests; tests/conftest.py applies a
mutant only when the ORACLE_MUTANT environment variable names one, in a
pytest process of its own that tests/test_oracle_mutations.py starts.
"""

import importlib

# name -> (module, original text, mutated text)
MUTANTS = {
    # attention
    "head_map": ("oracle.paged",
                 "            g = h // G\n            out[b, h], w = attention_one(",
                 "            g = h % n_kv\n            out[b, h], w = attention_one("),
    "dropped_scale": ("oracle.paged",
                      "    s = scale * (k @ q)\n",
                      "    s = (k @ q)\n"),
    "unnormalised_weights": ("oracle.paged",
                             "    w = e / np.sum(e)\n",
                             "    w = e\n"),
    "max_not_subtracted_right": ("oracle.paged",
                                 "    e = np.exp(s - m)\n    w = e",
                                 "    e = np.exp(m - s)\n    w = e"),
    # gather and mapping
    "reversed_gather": ("oracle.paged",
                        "cache[blk, :, :n, :].transpose(1, 0, 2)",
                        "cache[blk, :, :n, :][:, ::-1].transpose(1, 0, 2)"),
    "gather_block_off_by_one": ("oracle.paged",
                                "        blk = int(block_table_row[i])\n",
                                "        blk = int(block_table_row[max(i - 1, 0)])\n"),
    "slot_formula": ("oracle.paged",
                     "return blk * block_size + pos % block_size",
                     "return blk * block_size + pos // block_size"),
    # split-K
    "merge_sign": ("oracle.paged",
                   "l * np.exp(np.where(live, m, M) - M)",
                   "l * np.exp(M - np.where(live, m, M))"),
    "merge_drops_l": ("oracle.paged",
                      "w = np.where(live, l * np.exp(",
                      "w = np.where(live, 1.0 * np.exp("),
    "partition_overlap": ("oracle.paged",
                          "        ks = k[j * partition:(j + 1) * partition]\n",
                          "        ks = k[j * partition:(j + 1) * partition + 1]\n"),
    # dequantisation and codecs
    "fp8_scale_dropped": ("oracle.paged",
                          "        vals = _fp8.decode(raw)\n"
                          "        s = np.asarray(scale, dtype=np.float32).astype(np.float64)\n"
                          "        return vals * s[:, None]\n",
                          "        vals = _fp8.decode(raw)\n"
                          "        return vals\n"),
    "fp4_scale_dropped": ("oracle.paged",
                          "        vals = _fp4.decode(_fp4.unpack(raw))\n"
                          "        s = np.asarray(scale, dtype=np.float32).astype(np.float64)\n"
                          "        return vals * s[:, None]\n",
                          "        vals = _fp4.decode(_fp4.unpack(raw))\n"
                          "        return vals\n"),
    "fp8_bias": ("oracle.fp8_e4m3",
                 "return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)",
                 "return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 8)"),
    "fp8_subnormal_exponent": ("oracle.fp8_e4m3",
                               "return sign * (mant / 8.0) * 2.0 ** (1 - 7)",
                               "return sign * (mant / 8.0) * 2.0 ** (0 - 7)"),
    "fp8_tie_direction": ("oracle.fp8_e4m3",
                          "(hi != lo) & (lo % 2 == 1))",
                          "(hi != lo) & (lo % 2 == 0))"),
    "fp8_no_saturation": ("oracle.fp8_e4m3",
                          "    code = np.where(sat, np.uint8(0x7E), code)\n",
                          "    code = np.where(sat, NAN_CODE, code)\n"),
    "fp8_multiplies_scale": ("oracle.fp8_e4m3",
                             "q = np.divide(x, s, dtype=np.float32)",
                             "q = np.multiply(x, s, dtype=np.float32)"),
    "fp8_division_in_f64": ("oracle.fp8_e4m3",
                            "q = np.divide(x, s, dtype=np.float32)",
                            "q = np.divide(x.astype(np.float64), s.astype(np.float64))"),
    "fp4_bias": ("oracle.fp4_e2m1",
                 "2.0 ** (exp_field - 1)",
                 "2.0 ** exp_field"),
    "fp4_nibble_order": ("oracle.fp4_e2m1",
                         "    out[..., 0::2] = p & 0xF\n    out[..., 1::2] = p >> 4\n",
                         "    out[..., 0::2] = p >> 4\n    out[..., 1::2] = p & 0xF\n"),
    "fp4_tie_direction": ("oracle.fp4_e2m1",
                          "(hi != lo) & (lo % 2 == 1))",
                          "(hi != lo) & (lo % 2 == 0))"),
    "bf16_widen_shift": ("oracle.bf16",
                         "    wide = b.astype(np.uint32) << np.uint32(16)\n",
                         "    wide = b.astype(np.uint32) << np.uint32(15)\n"),
    # cache writes
    "append_kv_swapped": ("oracle.paged",
                          "            kc[blk, :, off, :] = k_new_bits[i]\n"
                          "            vc[blk, :, off, :] = v_new_bits[i]\n",
                          "            kc[blk, :, off, :] = v_new_bits[i]\n"
                          "            vc[blk, :, off, :] = k_new_bits[i]\n"),
    "append_offset": ("oracle.paged",
                      "        blk, off = divmod(int(slot), bs)\n",
                      "        blk, off = divmod(int(slot) + 1, bs)\n"),
    "copy_direction": ("oracle.paged",
                       "        out[dst] = cache[src]\n",
                       "        out[src] = cache[dst]\n"),
    # several queries, shared prefix, swap
    "causal_off_by_one": ("oracle.paged",
                          "            p = ctx - ql + i\n",
                          "            p = ctx - ql + i - 1\n"),
    "cascade_order": ("oracle.paged",
                      "np.concatenate([np.tile(pre, (B, 1)), block_tables], axis=1)",
                      "np.concatenate([block_tables, np.tile(pre, (B, 1))], axis=1)"),
    "swap_out_kv_swapped": ("oracle.paged",
                            "            out[0, i] = k_cache[blk]\n"
                            "            out[1, i] = v_cache[blk]\n",
                            "            out[0, i] = v_cache[blk]\n"
                            "            out[1, i] = k_cache[blk]\n"),
    # byte accounting
    "dropped_kv_factor": ("oracle.sizing",
                          "return 2 * L * n_kv * d * S * B * p",
                          "return L * n_kv * d * S * B * p"),
    # allocator
    "allocator_order": ("oracle.block_manager",
                        "        blk = self.free_pool.pop()\n",
                        "        blk = self.free_pool.pop(0)\n"),
    "cow_keeps_shared_count": ("oracle.block_manager",
                               "                new = self._pop()\n"
                               "                self.ref[last] -= 1\n",
                               "                new = self._pop()\n"),
    "lru_evicts_newest": ("oracle.block_manager",
                          "blk = min(victims, key=lambda b: self.stamp[b])",
                          "blk = max(victims, key=lambda b: self.stamp[b])"),
    "fork_without_ref": ("oracle.block_manager",
                         "        for blk in self.tables[child]:\n"
                         "            self.ref[blk] += 1\n",
                         "        for blk in self.tables[child]:\n"
                         "            pass\n"),
}


def source_of(module_name):
    mod = importlib.import_module(module_name)
    with open(mod.__file__) as f:
        return mod, f.read()


def apply(name):
    """Re-execute the mutant's module with its replacement in place."""
    module_name, old, new = MUTANTS[name]
    mod, src = source_of(module_name)
    n = src.count(old)
    if n != 1:
        raise RuntimeError(f"mutant {name}: original text found {n} times in {module_name}")
    code = compile(src.replace(old, new), mod.__file__, "exec")
    exec(code, mod.__dict__)
