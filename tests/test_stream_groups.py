"""CPU: the decode-stream grouping used for merged launches only joins
projections of one layer that read the same activation vector."""
from quant_dequant_gemv_amd import synth


def test_groups_partition_the_stream_in_order():
    e = synth.decode_stream()
    g = synth.decode_groups(e)
    assert [i for idx in g for i in idx] == list(range(len(e)))
    assert len(e) == 448 and len(g) == 64 * 4


def test_group_members_share_layer_input_and_K():
    e = synth.decode_stream()
    for idx in synth.decode_groups(e):
        assert len({e[i]["layer"] for i in idx}) == 1
        assert len({synth.X_GROUP[e[i]["name"]] for i in idx}) == 1
        assert len({e[i]["K"] for i in idx}) == 1
        assert len(idx) <= 16
    names = {tuple(e[i]["name"] for i in idx) for idx in synth.decode_groups(e)}
    assert ("attn_qkv", "ssm_alpha", "ssm_beta") in names and ("attn_q", "attn_k", "attn_v") in names
    assert ("ffn_gate", "ffn_up") in names and ("ffn_down",) in names
