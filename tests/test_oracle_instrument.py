"""Testing the instrument: a build of the oracle with one planted mistake must
fail at least one pin, and the pin named for it in particular. The mistakes are
planted in the oracle, on the CPU ("The kernel reference interpreter", section
Testing the instrument)."""
import os

import pytest

import oracle
import pins

FAULTS = {
    "XQO_FAULT_TIES_AWAY": "pin_q8k_unit_scale_ties",
    "XQO_FAULT_NIBBLE_SWAP": "pin_q4k_closed_forms",
    "XQO_FAULT_MIN_SIGN": "pin_q4k_brute_force",
    "XQO_FAULT_SCALE_HIBITS": "pin_q4k_pack_roundtrip",
    "XQO_FAULT_IQ4_HALVES": "pin_iq4nl_layout",
    "XQO_FAULT_Q40_OFFSET": "pin_q4_0_layout",
    "XQO_FAULT_T_DOUBLE": "pin_q4k_magnitudes_one_hot",
    "XQO_FAULT_TB_SUBBLOCK": "pin_q4k_magnitudes_cancel",
    "XQO_FAULT_TB_IQ4_ELEM": "pin_iq4nl_magnitudes",
}


@pytest.mark.parametrize("fault", sorted(FAULTS))
def test_planted_mistake_is_caught(tmp_path, fault):
    path = oracle.compile_oracle(os.path.join(str(tmp_path), "lib_%s.so" % fault), [fault])
    faulty = oracle.Oracle(path)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(faulty)
        except AssertionError:
            failed.append(pin.__name__)
    assert FAULTS[fault] in failed, (fault, failed)
