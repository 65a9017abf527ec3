"""Plant plausible mistakes in copies of the oracle and check that the pins catch
every one (CPU only; the mutants are built in a temporary directory)."""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kvm_ref.c")

# (label, exact text in kvm_ref.c, replacement)
MUTANTS = [
    ("full block layer-major instead of token-major",
     "return t * token_stride + (l * p->sides + s) * p->row_bytes;",
     "return l * token_stride + (t * p->sides + s) * p->row_bytes;"),
    ("dropped side term in the pool",
     "return l * p->layer_stride + s * p->side_stride + n * p->block_stride + r * p->row_bytes;",
     "return l * p->layer_stride + n * p->block_stride + r * p->row_bytes;"),
    ("side and layer swapped inside a token row",
     "return t * token_stride + (l * p->sides + s) * p->row_bytes;",
     "return t * token_stride + (s * p->sides + l) * p->row_bytes;"),
    ("row index uses division",
     "        int64_t row = t % p->block_tokens;\n        for (int64_t l = 0;",
     "        int64_t row = t / p->block_tokens;\n        for (int64_t l = 0;"),
    ("unpack block table indexed by row",
     "        int64_t block = block_table[t / p->block_tokens];\n        int64_t row = t % p->block_tokens;\n        for (int64_t s = 0;",
     "        int64_t block = block_table[t % p->block_tokens];\n        int64_t row = t % p->block_tokens;\n        for (int64_t s = 0;"),
    ("dense token stride forgets the sides",
     "return (int64_t)num_layers * p->sides * p->row_bytes;",
     "return (int64_t)num_layers * p->row_bytes;"),
    ("miss rows start one row early",
     "memcpy(out + (t_hit + i) * out_stride, miss + i * miss_stride, (size_t)row_bytes);",
     "memcpy(out + (t_hit + i - 1) * out_stride, miss + i * miss_stride, (size_t)row_bytes);"),
    ("hit rows read with the output stride",
     "memcpy(out + t * out_stride, hit + t * hit_stride, (size_t)row_bytes);",
     "memcpy(out + t * out_stride, hit + t * out_stride, (size_t)row_bytes);"),
    ("batch copy swaps source and destination offsets",
     "if (len) memcpy(dst + d_o, src + so, (size_t)len);",
     "if (len) memcpy(dst + so, src + d_o, (size_t)len);"),
    ("overlap check misses touching-by-one",
     "if (spans[i].begin < spans[i - 1].end) bad = 1;",
     "if (spans[i].begin + 1 < spans[i - 1].end) bad = 1;"),
    ("unpack copies one token too few",
     "    for (int64_t t = 0; t < num_tokens; ++t) {\n        int64_t block = block_table[t / p->block_tokens];\n        int64_t row = t % p->block_tokens;\n        for (int64_t s = 0;",
     "    for (int64_t t = 0; t + 1 < num_tokens; ++t) {\n        int64_t block = block_table[t / p->block_tokens];\n        int64_t row = t % p->block_tokens;\n        for (int64_t s = 0;"),
    ("object count forgets the sides",
     "return sides * layers * ref_blocks_for_tokens(tokens, block_tokens);",
     "return layers * ref_blocks_for_tokens(tokens, block_tokens);"),
    ("block count rounds down",
     "return (tokens + block_tokens - 1) / block_tokens;",
     "return tokens / block_tokens;"),
]


def _all_pins_pass(lib):
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError):
            return False
    return True


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(label, old, new, tmp_path):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site not unique or missing: {label}"
    mut = tmp_path / "kvm_ref_mut.c"
    mut.write_text(text.replace(old, new))
    so = tmp_path / "libmut.so"
    oracle.build(out=str(so), src=str(mut), extra_flags=["-I", os.path.dirname(SRC)])
    lib = oracle.load(str(so))
    assert not _all_pins_pass(lib), f"pins did not catch: {label}"


def test_unmutated_copy_passes(tmp_path):
    so = tmp_path / "libref.so"
    oracle.build(out=str(so))
    assert _all_pins_pass(oracle.load(str(so)))
