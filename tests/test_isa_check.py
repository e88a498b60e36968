"""Host-side tests of the device-assembly dependency check (no GPU needed)."""
from kalman_delta_rule_amd import isa_check


def _seq(nops):
    return (["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0"]
            + ["v_add_u32_e32 v20, 1, v21"] * nops
            + ["v_mfma_f32_16x16x16_bf16 v[12:15], v[16:17], v[18:19], v[0:3]"])


def test_flags_close_cross_opcode_accumulator_dependency():
    hz = isa_check.find_hazards(_seq(2))
    assert len(hz) == 1 and hz[0][2] == 2


def test_padded_dependency_is_accepted():
    assert isa_check.find_hazards(_seq(isa_check.MIN_WAIT_STATES)) == []
    nop_pad = (["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0", "s_nop 15"]
               + ["v_mfma_f32_16x16x16_bf16 v[12:15], v[16:17], v[18:19], v[0:3]"])
    assert isa_check.find_hazards(nop_pad) == []


def test_same_opcode_chain_is_accepted():
    seq = ["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
           "v_mfma_f32_16x16x32_bf16 v[0:3], v[12:15], v[16:19], v[0:3]"]
    assert isa_check.find_hazards(seq) == []


def test_follows_branches_and_stops_at_overwrite():
    seq = ["v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0",
           "s_cbranch_scc1 .LBB0_2",
           "v_mov_b32_e32 v0, 0",          # fall-through path overwrites the result
           "v_mfma_f32_16x16x16_bf16 v[12:15], v[16:17], v[18:19], v[0:3]",
           ".LBB0_2:",
           "v_mfma_f32_16x16x16_bf16 v[20:23], v[16:17], v[18:19], v[0:3]"]
    hz = isa_check.find_hazards(seq)
    assert len(hz) == 1 and hz[0][1].startswith("v_mfma_f32_16x16x16_bf16 v[20:23]")


def test_parses_kernel_bodies():
    text = "\n".join(["_Z3fooPf:", "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0 ; c",
                      "\ts_endpgm", ".Lfunc_end0:"])
    ks = isa_check.parse_kernels(text)
    assert list(ks) == ["_Z3fooPf"] and ks["_Z3fooPf"][0].startswith("v_mfma")


def test_flags_device_side_calls():
    body = ["s_getpc_b64 s[0:1]", "s_add_u32 s0, s0, fn@rel32@lo+4",
            "s_swappc_b64 s[30:31], s[0:1]", "s_endpgm"]
    assert isa_check.find_calls(body) == ["s_swappc_b64 s[30:31], s[0:1]"]
    assert isa_check.find_calls(["v_add_u32_e32 v1, 1, v2", "s_endpgm"]) == []
