"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant is a one-token edit of a copy of pa_oracle.c, built on the CPU
into a temporary directory: a dropped term, a wrong index, an off-by-one, a
transposed operand, a wrong sign.  None of them reads out of bounds.
"""
import os
import shutil
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "pa_oracle.c")

MUTANTS = {
    "kv_head_modulo": ("int32_t kvh = h / G;", "int32_t kvh = h % j->num_kv_heads;"),
    "causal_off_by_one": ("if (pos + 1 < end) end = pos + 1;", "if (pos < end) end = pos;"),
    "scale_dropped": ("z[t - t_begin] = j->scale * acc;", "z[t - t_begin] = acc;"),
    "slot_wrong": ("int64_t slot = token % j->page_size;",
                   "int64_t slot = token % (j->page_size / 2);"),
    "page_always_first": ("+ token / j->page_size];", "+ (token / j->page_size) * 0];"),
    "not_normalised": ("for (int32_t d = 0; d < D; ++d) o[d] /= sum;", ""),
    "lse_without_max": ("*lse = m + log(sum);", "*lse = log(sum);"),
    "exp_without_max": ("double w = exp(z[t - t_begin] - m);", "double w = exp(z[t - t_begin]);"),
    "merge_weight_sign": ("double w = exp(pl[k] - M);", "double w = exp(M - pl[k]);"),
    "merge_lse_no_max": ("lse[r] = M + log(wsum);", "lse[r] = log(wsum);"),
    "k_dims_reversed": ("bf16_to_f64(krow[d])", "bf16_to_f64(krow[D - 1 - d])"),
    "v_read_from_k": ("const uint16_t *vrow = j->v_pool", "const uint16_t *vrow = j->k_pool"),
    "split_drops_token": ("int64_t e = b + j->split_tokens;",
                          "int64_t e = b + j->split_tokens - 1;"),
    "append_position_shifted": ("int64_t pos = L - q_s + i;", "int64_t pos = L - q_s + i + 1;"),
    "append_slot_is_block": ("int64_t slot = pos % page_size;", "int64_t slot = block;"),
    "append_head_row_dropped": ("((first + i) * num_kv_heads + h)", "((first + i) + h)"),
    "append_v_from_k": ("v_pool[dst + d] = v_new[src + d];", "v_pool[dst + d] = k_new[src + d];"),
    "append_decode_first_row": ("first = query_start_loc ? query_start_loc[s] : s;",
                                "first = query_start_loc ? query_start_loc[s] : 0;"),
    "append_page_from_block": ("int64_t page = block_tables[(int64_t)s * max_blocks + block];",
                               "int64_t page = block;"),
    "query_row_head_swapped": ("j->q + (t * Hq + h) * (int64_t)D",
                               "j->q + (t * Hq + (Hq - 1 - h)) * (int64_t)D"),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="pa_oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(force=True, src=path, out=os.path.join(workdir, f"lib{name}.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
