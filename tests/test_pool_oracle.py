"""The block-pool reference model against its pins, and planted mistakes in
copies of the model against the same pins (each must fail one)."""
import importlib.util
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import pool_pins  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "block_pool.py")


def load_model(path, name):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("pin", pool_pins.PINS, ids=[p.__name__ for p in pool_pins.PINS])
def test_pool_model_pin(pin):
    from oracle import block_pool

    pin(block_pool)


# (name, original text, planted text).  Not listed: dropping the count of how
# often an id was handed out from the cache key.  Under this pool's policy it
# cannot change a result: every table that holds a cached block also holds the
# block before it, blocks are freed last first and reused oldest first, so a
# block is always reused before the block it follows.  The count keeps the key
# exact under any other eviction order.
MUTANTS = [
    ("free_leaks_blocks", "self.ref[b] -= 1\n            if self.ref[b] == 0:",
     "if self.ref[b] == 1:"),
    ("no_copy_on_write", "elif self.ref[blocks[-1]] > 1:", "elif False:"),
    ("copy_keeps_old_reference", "self.ref[old] -= 1", "pass"),
    ("prompt_fully_cached", "for i in range((n - 1) // bs):", "for i in range(n // bs):"),
    ("key_ignores_previous_block", "return (prev_block, self.gen[prev_block], tuple(block_tokens))",
     "return (-1, 0, tuple(block_tokens))"),
    ("reused_block_stays_cached", "del self.cache[self.identity[b]]\n            self.identity[b] = None",
     "pass"),
    ("capacity_ignores_revived_hits", "if need > len(self.free) - revived:", "if need > len(self.free):"),
    ("lifo_takes_freed_prefix_first", "b = self.free.pop(0)", "b = self.free.pop()"),
]


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pool_mutant_fails_a_pin(tmp_path, name, orig, planted):
    text = open(SRC).read()
    assert text.count(orig) == 1, f"mutation site for {name} not found"
    path = tmp_path / f"mutant_{name}.py"
    path.write_text(text.replace(orig, planted))
    mod = load_model(str(path), f"mutant_{name}")
    failed = []
    for pin in pool_pins.PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 -- any failure of a pin counts
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
