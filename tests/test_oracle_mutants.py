"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one of them (the mistakes live in temporary builds on the CPU;
the committed oracle is untouched)."""
import os

import pytest

import oracle
from tests import oracle_pins

SRC = oracle.SRC

# (name, exact text in oracle.c, replacement).  Each text must occur once.
MUTANTS = [
    ("rs_send_index_sign", "int c = mod(r - s, n);\n            const orc_fault* f = nt->fault;\n"
     "            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_RS",
     "int c = mod(r + s, n);\n            const orc_fault* f = nt->fault;\n"
     "            if (f && f->kind == ORC_FAULT_WRONG_CHUNK && f->phase == ORC_PHASE_RS"),
    ("rs_schedule_shifted", "for (int r = 0; r < n; r++) {\n            int c = mod(r - 1 - s, n);\n"
     "            msg* m;\n            int rc = receive(nt, r, ORC_PHASE_RS",
     "for (int r = 0; r < n; r++) {\n            int c = mod(r - s, n);\n"
     "            msg* m;\n            int rc = receive(nt, r, ORC_PHASE_RS"),
    ("fp32_add_becomes_sub", "z = x + y;\n        memcpy(dst, &z, 4);\n        break;\n    }\n"
     "    case ORC_FP16",
     "z = x - y;\n        memcpy(dst, &z, 4);\n        break;\n    }\n    case ORC_FP16"),
    ("int_add_drops_carry", "z = x + y; /* wraps modulo 2^32 */", "z = x ^ y;"),
    ("remainder_dropped", "return (c == g->n - 1) ? g->count - base * (uint64_t)(g->n - 1) : base;",
     "return base;"),
    ("rounding_truncates", "double r = rint(q);", "double r = floor(q);"),
    ("rounding_ties_away", "double r = rint(q);", "double r = round(q);"),
    ("fused_fp16_rounds_each_step",
     "case ORC_FP16: memcpy(&h, x, 2); acc->f = acc->f + f16_decode(h); break;",
     "case ORC_FP16: memcpy(&h, x, 2); acc->f = f16_decode(f16_encode(acc->f + f16_decode(h))); break;"),
    ("fused_skips_rank0",
     "acc_set(dt, &acc, (const unsigned char*)x[0] + i * esz);\n        for (int r = 1; r < n; r++) "
     "acc_add(dt, &acc, (const unsigned char*)x[r] + i * esz);\n        for (int r = 0; r < n; r++)",
     "acc_set(dt, &acc, (const unsigned char*)x[1 % n] + i * esz);\n        for (int r = 2; r < n; r++) "
     "acc_add(dt, &acc, (const unsigned char*)x[r] + i * esz);\n        for (int r = 0; r < n; r++)"),
    ("ag_relays_partial_blocks", "int c = mod(r + 1 - s, n);", "int c = mod(r - s, n);"),
    ("ag_receive_index", "int c = mod(r - s, n);\n            msg* m;\n            int rc = receive(nt, r, ORC_PHASE_AG",
     "int c = mod(r + 1 - s, n);\n            msg* m;\n            int rc = receive(nt, r, ORC_PHASE_AG"),
    ("bf16_field_widths", "static float bf16_decode(uint16_t b) { return small_decode(b, 8, 7); }",
     "static float bf16_decode(uint16_t b) { return small_decode(b, 7, 8); }"),
    ("fp16_subnormals_lost", "if (e < emin) e = emin; /* subnormal range: fixed scale */", ""),
    ("closed_form_starts_next_block", "int c = chunk_of(count, n, i);\n        memcpy(partial",
     "int c = mod(chunk_of(count, n, i) + 1, n);\n        memcpy(partial"),
    ("rs_delivers_from_wrong_holder", "int holder = mod(c - 1, n);", "int holder = mod(c + 1, n);"),
    ("column_block_stride", "return o * g->row + (uint64_t)c * w + j;", "return o * w * g->n + (uint64_t)c * w + j + o;"),
    ("ag_slab_column", "memcpy(buf[r] + (o * g.row * (uint64_t)n + (uint64_t)slab * g.row + j) * esz,",
     "memcpy(buf[r] + (o * g.row * (uint64_t)n + (uint64_t)r * g.row + j) * esz,"),
    ("traffic_not_counted_for_ag", "if (t->sent_elems) t->sent_elems[m->src] += m->elems;",
     "if (t->sent_elems && m->phase == ORC_PHASE_RS) t->sent_elems[m->src] += m->elems;"),
    ("received_block_overwrites", "elem_add(nt->dt, mine, mine, m->payload + k * nt->esz);",
     "memcpy(mine, m->payload + k * nt->esz, nt->esz);"),
    ("decode_bias_off_by_one", "int bias = (1 << (ebits - 1)) - 1;\n    uint32_t sign = (bits",
     "int bias = (1 << (ebits - 1));\n    uint32_t sign = (bits"),
    # halving-doubling
    ("hd_keeps_other_half",
     "int upper = (r & d) != 0;\n            int give_lo",
     "int upper = (r & d) == 0;\n            int give_lo"),
    ("hd_distances_ascending", "for (int d = n / 2; d >= 1 && step < steps; d /= 2, step++) {",
     "for (int d = 1; d < n && step < steps; d *= 2, step++) {"),
    ("hd_doubling_does_not_merge", "lo[r] = plo[r] < plo[p] ? plo[r] : plo[p];", "lo[r] = plo[r];"),
    ("hd_closed_form_sequential",
     "for (int d = n / 2; d >= 1; d /= 2)\n            for (int r = 0; r < d; r++) elem_add(dt, v + r * esz, v + r * esz, v + (r + d) * esz);",
     "for (int r = 1; r < n; r++) elem_add(dt, v, v, v + r * esz);"),
    ("hd_received_half_overwrites", "elem_add(nt->dt, mine, m->payload + k * nt->esz, mine);",
     "memcpy(mine, m->payload + k * nt->esz, nt->esz);"),
    ("hd_range_drops_remainder", "for (int b = lo; b < hi; b++) total += chunk_len(g, b);",
     "for (int b = lo; b < hi; b++) total += g->count / (uint64_t)g->n;"),
    # binomial-tree all-gather
    ("tree_gather_sends_own_slab_only", "int lo = r, top = hi[r];", "int lo = r, top = r + 1;"),
    ("tree_gather_stops_at_floor_log2", "for (int d = 1; d < n; d *= 2, step++) {\n        for (int r = 0; r < n; r++) {\n"
     "            if (r % (2 * d) != d) continue;",
     "for (int d = 1; 2 * d <= n; d *= 2, step++) {\n        for (int r = 0; r < n; r++) {\n"
     "            if (r % (2 * d) != d) continue;"),
    ("tree_gather_lands_on_own_slab",
     "memcpy(buf[r] + slab_range_elem(g, p, hi[p], k) * nt->esz, m->payload + k * nt->esz, nt->esz);",
     "memcpy(buf[r] + slab_range_elem(g, r, r + hi[p] - p, k) * nt->esz, m->payload + k * nt->esz, nt->esz);"),
    ("tree_bcast_skips_distance_one", "for (int d = top; n > 1 && d >= 1; d /= 2, step++) {",
     "for (int d = top; n > 1 && d >= 2; d /= 2, step++) {"),
    ("tree_bcast_top_rounds_up", "while (2 * top < n) top *= 2;", "while (top < n) top *= 2;"),
]


def test_mutant_patterns_match_source():
    text = open(SRC).read()
    for name, old, _new in MUTANTS:
        assert text.count(old) == 1, f"mutant {name}: pattern occurs {text.count(old)} times"


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(workdir, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1
    src = os.path.join(workdir, f"{name}.c")
    lib = os.path.join(workdir, f"lib{name}.so")
    with open(src, "w") as fh:
        fh.write(text.replace(old, new))
    oracle.build(src, lib)
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
            break
    assert caught, f"no pin caught mutant {name}"
