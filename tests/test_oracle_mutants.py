"""Planted mistakes in copies of the oracle must fail its pins.

Each case takes the source of one oracle module, makes one plausible mistake
in it (a window bound off by one, interleaved GQA groups, a dropped or wrong
scale, a swapped operand, the wrong end of the free list, a wrong rounding
rule, ...), loads the result as a separate module, points the pin module at
that copy and runs the pins named for the case: every one of them must fail.
The real oracle is never modified, and a control case runs the same pins on
an unmodified copy to show the harness itself lets them pass.

A mistake that no pin catches would show up here as a failing case; the
table is the record of which pin guards which step of the definition.
"""
import importlib
import os
import types

import pytest

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _load_copy(module: str, old: str, new: str) -> types.ModuleType:
    with open(os.path.join(ORACLE, module + ".py")) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique in oracle/{module}.py: {old!r}"
    mod = types.ModuleType(f"oracle_copy_{module}")
    code = compile(src.replace(old, new), f"<copy of oracle/{module}.py>", "exec")
    exec(code, mod.__dict__)
    return mod


# pin module -> (oracle module, names the pin module binds from it)
BINDINGS = {
    "test_oracle:A": ("attention", {"A": None}),
    "test_oracle:CF": ("closed_forms", {"CF": None}),
    "test_oracle_pool": ("pool", {"PoolSim": "PoolSim", "NoSpace": "NoSpace"}),
    "test_oracle_fp8": ("fp8", {"F": None}),
    "test_oracle_transfer": ("transfer", {"T": None}),
}

SDPA_GQA = ("test_matches_torch_sdpa_fp64", dict(kind=1, window=5, hq=8, hkv=2, d=16))
SDPA_FULL = ("test_matches_torch_sdpa_fp64", dict(kind=0, window=0, hq=6, hkv=1, d=32))
FSUM = ("test_brute_force_fsum", dict(window=5))
POOL_RANDOM = [("test_random_operations_against_second_simulator", dict(seed=s)) for s in range(12)]
FORK_RANDOM = ("test_random_forks_against_second_simulator", {})

# (name, binding, old text, new text, pins that must each fail; a list
# inside the list means "at least one of these")
CASES = [
    # -- attention: the window, GQA grouping, scale and softmax ---------------
    ("window_one_key_too_many", "test_oracle:A",
     "lo = max(0, pos - window + 1)", "lo = max(0, pos - window)",
     [SDPA_GQA, FSUM, ("test_window_one_returns_own_value", {}),
      ("test_out_of_window_keys_do_not_matter", {}),
      ("test_one_hot_values_expose_weights", {}),
      ("test_valid_length_and_pair_counts", dict(window=7))]),
    ("window_one_key_too_few", "test_oracle:A",
     "lo = max(0, pos - window + 1)", "lo = max(0, pos - window + 2)",
     [SDPA_GQA, FSUM, ("test_window_one_returns_own_value", {}),
      ("test_zero_query_gives_window_mean", dict(kind=1, window=6))]),
    ("query_does_not_see_itself", "test_oracle:A",
     "return lo, pos + 1", "return lo, pos",
     [SDPA_GQA, SDPA_FULL, FSUM, ("test_window_one_returns_own_value", {})]),
    ("gqa_groups_interleaved", "test_oracle:A",
     "heads = slice(kv * g, (kv + 1) * g)", "heads = slice(kv, hq, hkv)",
     [SDPA_GQA, ("test_gqa_groups_are_contiguous", {})]),
    ("scale_one_over_d", "test_oracle:A",
     "tau = 1.0 / np.sqrt(d) if", "tau = 1.0 / d if",
     [SDPA_GQA, SDPA_FULL, FSUM, ("test_one_hot_values_expose_weights", {})]),
    ("explicit_scale_ignored", "test_oracle:A",
     "tau = 1.0 / np.sqrt(d) if scale is None else float(scale)", "tau = 1.0 / np.sqrt(d)",
     [("test_explicit_scale_matches_sdpa", {})]),
    ("values_read_from_keys", "test_oracle:A",
     "(w @ v[lo:hi, kv])", "(w @ k[lo:hi, kv])",
     [SDPA_GQA, SDPA_FULL, FSUM, ("test_zero_query_gives_window_mean", dict(kind=0, window=0))]),
    ("normaliser_over_whole_group", "test_oracle:A",
     "w.sum(axis=1, keepdims=True)", "w.sum()",
     [SDPA_GQA, FSUM, ("test_zero_query_gives_window_mean", dict(kind=1, window=6))]),
    ("max_taken_per_key", "test_oracle:A",
     "s.max(axis=1, keepdims=True)", "s.max(axis=0, keepdims=True)",
     [SDPA_GQA, FSUM, ("test_one_hot_values_expose_weights", {})]),
    # -- closed forms ---------------------------------------------------------
    ("swa_pairs_triangle_off_by_one", "test_oracle:CF",
     "window * (window - 1) // 2", "window * (window + 1) // 2",
     [("test_valid_length_and_pair_counts", dict(window=7))]),
    ("full_pairs_without_diagonal", "test_oracle:CF",
     "n * (n + 1) // 2", "n * (n - 1) // 2",
     [("test_valid_length_and_pair_counts", dict(window=7)),
      ("test_short_sequences_have_no_saving", {})]),
    ("swa_kv_not_capped_by_length", "test_oracle:CF",
     "n_swa * min(n, window)", "n_swa * window",
     [("test_short_sequences_have_no_saving", {})]),
    ("flops_count_one_product", "test_oracle:CF",
     "4 * head_dim * num_q_heads", "2 * head_dim * num_q_heads",
     [("test_flop_count", {})]),
    ("kv_ratio_uses_pair_counts", "test_oracle:CF",
     "(n_swa * min(n, window) + n_full * n) / ((n_swa + n_full) * n)",
     "(n_swa * pairs_swa(n, window) + n_full * pairs_full(n)) / ((n_swa + n_full) * pairs_full(n))",
     [("test_page_facts_one_seventh_and_seven_x", {})]),
    # -- dual pool --------------------------------------------------------------
    ("evict_keeps_whole_window", "test_oracle_pool",
     "keep_from = max(0, self.length[b] - self.W + 1)", "keep_from = max(0, self.length[b] - self.W)",
     [("test_hand_worked_fixtures", {}), ("test_decode_steps_evict_one_token_each", {}),
      POOL_RANDOM]),
    ("import_keeps_whole_window", "test_oracle_pool",
     "keep_from = max(0, new_len - self.W + 1)", "keep_from = max(0, new_len - self.W)",
     [("test_hand_worked_fixtures", {}), POOL_RANDOM]),
    ("ring_indexed_by_window", "test_oracle_pool",
     "r = pos % self.C", "r = pos % (self.C - PAGE if self.C > PAGE else self.C)",
     [("test_hand_worked_fixtures", {}), POOL_RANDOM]),
    ("ring_capacity_off_by_one", "test_oracle_pool",
     "+ n > self.C:", "+ n >= self.C:",
     [POOL_RANDOM]),
    ("released_pages_to_head", "test_oracle_pool",
     "self.free.extend(pg for pg in self.pages[b] if self._drop_page(pg))",
     "self.free.extendleft(pg for pg in self.pages[b] if self._drop_page(pg))",
     [("test_hand_worked_fixtures", {}), POOL_RANDOM]),
    # -- prefix reuse (fork) -------------------------------------------------------
    ("fork_shares_the_window_page", "test_oracle_pool",
     "            own = start // PAGE\n", "            own = -(-start // PAGE)\n",
     [("test_hand_worked_fixtures", {}), FORK_RANDOM]),
    ("fork_takes_no_reference", "test_oracle_pool",
     "                self.refs[pg] += 1\n", "                self.refs[pg] += 0\n",
     [("test_hand_worked_fixtures", {}), FORK_RANDOM]),
    ("fork_window_one_position_short", "test_oracle_pool",
     "            for pos in range(start, m):", "            for pos in range(start + 1, m):",
     [("test_hand_worked_fixtures", {}), FORK_RANDOM]),
    ("match_reads_another_holders_entries", "test_oracle_pool",
     "if all(pos >= self.res_start[b] and self.full_slot(b, pos) in self.map",
     "if all(self.full_slot(b, pos) in self.map",
     [("test_hand_worked_fixtures", {}), FORK_RANDOM]),
    ("cut_into_shared_page_allowed", "test_oracle_pool",
     "            if n < self.length[b] and n < PAGE * self.shared_pages(b):",
     "            if False:",
     [("test_hand_worked_fixtures", {}),
      [("test_cut_into_shared_page_refused", dict(seed=s)) for s in range(8)]]),
    ("fork_not_window_safe_accepted", "test_oracle_pool",
     "            if self.window_safe_len(a, m, self.W - 1) != m:",
     "            if self.window_safe_len(a, m, 0) != m:",
     [FORK_RANDOM]),
    ("truncated_pages_to_tail", "test_oracle_pool",
     "self.free.extendleft(reversed(freed))", "self.free.extend(freed)",
     [("test_hand_worked_fixtures", {}), POOL_RANDOM]),
    ("truncate_keeps_one_stale_map_entry", "test_oracle_pool",
     "for pos in range(n, self.length[b]):", "for pos in range(n + 1, self.length[b]):",
     [POOL_RANDOM]),
    ("full_check_off_by_one", "test_oracle_pool",
     "if self._pages_needed(ids, counts) > len(self.free):\n            raise NoSpace(\"Full pool exhausted\")\n        for b",
     "if self._pages_needed(ids, counts) >= len(self.free):\n            raise NoSpace(\"Full pool exhausted\")\n        for b",
     [POOL_RANDOM]),
    ("match_tail_one_short", "test_oracle_pool",
     "range(max(0, k - tail), k)", "range(max(0, k - tail + 1), k)",
     [("test_hand_worked_fixtures", {}), POOL_RANDOM]),
    # -- fp8 ----------------------------------------------------------------------
    ("subnormal_step_halved", "test_oracle_fp8",
     "(m / 8.0) * 2.0 ** -6", "(m / 8.0) * 2.0 ** -7",
     [("test_value_table_facts", {})]),
    ("exponent_bias_eight", "test_oracle_fp8",
     "2.0 ** (e - 7)", "2.0 ** (e - 8)",
     [("test_value_table_facts", {})]),
    ("ties_to_odd_in_search", "test_oracle_fp8",
     "(c & 1) == 0", "(c & 1) == 1",
     [("test_vector_encoder_matches_nearest_code_search", {})]),
    ("fraction_truncated", "test_oracle_fp8",
     "np.rint((2 * m - 1) * 8)", "np.floor((2 * m - 1) * 8)",
     [("test_vector_encoder_matches_nearest_code_search", {}), ("test_quantize_rows_bounds", {})]),
    ("no_saturation", "test_oracle_fp8",
     "a = np.minimum(np.abs(y), E4M3_MAX)", "a = np.abs(y)",
     [("test_vector_encoder_matches_nearest_code_search", {})]),
    ("subnormal_boundary_low", "test_oracle_fp8",
     "sub = a < 2.0 ** -6", "sub = a < 2.0 ** -7",
     [("test_vector_encoder_matches_nearest_code_search", {}),
      ("test_encode_of_every_finite_value_is_its_code", {})]),
    ("scale_inverted", "test_oracle_fp8",
     "scale = (amax / np.float32(E4M3_MAX))", "scale = (np.float32(E4M3_MAX) / amax)",
     [("test_quantize_rows_bounds", {})]),
    # -- window-masked transfer ------------------------------------------------------
    ("transfer_moves_whole_window", "test_oracle_transfer",
     "range(max(0, length - window + 1), length)", "range(max(0, length - window), length)",
     [("test_swa_mask_is_the_resident_set_after_eviction", dict(seed=0)),
      ("test_byte_counts_closed_form", {}), ("test_host_image_packs_windows_in_order", {})]),
    ("transfer_bytes_one_tensor", "test_oracle_transfer",
     "* hkv * d * 4", "* hkv * d * 2",
     [("test_byte_counts_closed_form", {})]),
    ("v_left_in_bf16", "test_oracle_transfer",
     "vs.append(v32.astype(np.float16).view(np.uint16))", "vs.append(v[sel])",
     [("test_v_conversion_matches_binary16_definition", {})]),
    ("fp8_bytes_without_scales", "test_oracle_transfer",
     "* hkv * (2 * d + 8)", "* hkv * 2 * d",
     [("test_fp8_byte_counts_closed_form", {})]),
    ("fp8_v_quantized_from_k", "test_oracle_transfer",
     "cv, sv = fp8.quantize_rows(v[sel])", "cv, sv = fp8.quantize_rows(k[sel])",
     [("test_host_image_fp8_packs_windows_in_order", {})]),
    ("fp8_image_whole_sequence", "test_oracle_transfer",
     "ck, sk = fp8.quantize_rows(k[sel])", "ck, sk = fp8.quantize_rows(k[:len(pos)])",
     [("test_host_image_fp8_packs_windows_in_order", {})]),
    ("sequences_packed_in_reverse", "test_oracle_transfer",
     "return np.concatenate(ks), np.concatenate(vs)",
     "return np.concatenate(ks[::-1]), np.concatenate(vs[::-1])",
     [("test_host_image_packs_windows_in_order", {})]),
]


def _bind(monkeypatch, binding: str, copy: types.ModuleType):
    pin_module = importlib.import_module(binding.split(":")[0])
    for name, attr in BINDINGS[binding][1].items():
        monkeypatch.setattr(pin_module, name, copy if attr is None else getattr(copy, attr))
    return pin_module


def _fails(pin_module, name: str, kwargs: dict) -> bool:
    try:
        getattr(pin_module, name)(**kwargs)
    except (Exception, pytest.fail.Exception):
        return True
    return False


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_fails_its_pins(case, monkeypatch):
    _, binding, old, new, pins = case
    pin_module = _bind(monkeypatch, binding, _load_copy(BINDINGS[binding][0], old, new))
    survived = []
    for pin in pins:
        group = pin if isinstance(pin, list) else [pin]
        if not any(_fails(pin_module, n, kw) for n, kw in group):
            survived.append(group[0][0] if len(group) == 1 else f"all of {group[0][0]}[*]")
    assert not survived, f"planted mistake passed: {survived}"


@pytest.mark.parametrize("binding", sorted(BINDINGS))
def test_unmodified_copy_passes_the_same_pins(binding, monkeypatch):
    module = BINDINGS[binding][0]
    pin_module = _bind(monkeypatch, binding, _load_copy(module, "from __future__", "from __future__"))
    pins = {(n, tuple(sorted(kw.items())))
            for c in CASES if c[1] == binding
            for p in c[4] for n, kw in (p if isinstance(p, list) else [p])}
    for n, kw in sorted(pins):
        assert not _fails(pin_module, n, dict(kw)), n
