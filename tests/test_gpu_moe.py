"""GPU parity of the routed-expert path: routing (ids exact, weights to fp32 rounding), the
device plan (word for word against the oracle's grouping), and the routed Q8_0 forward against
the oracle at small shapes and at the full 512-expert workload."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import to_dev, to_host
from oracle.moe import moe_forward, plan, route
from oracle.q8 import quantize_q8_0, quantize_q8_1_bf16
from tests.helpers import check_bf16

pytestmark = pytest.mark.gpu


def _route(gpu, logits, topk):
    T, E = logits.shape
    ids = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    gpu.gq8_moe_route(to_dev(logits), T, E, topk, ids, w)
    return to_host(ids), to_host(w)


@pytest.mark.parametrize("T,E,topk", [(4, 512, 8), (1, 16, 1), (7, 300, 5), (16, 4096, 16)])
def test_route_matches_oracle(gpu, T, E, topk):
    logits = synth.normal_f32(40, "gpu.moe.logits", (T, E))
    ids, w = _route(gpu, logits, topk)
    ids_ref, p_ref = route(logits, topk)
    assert np.array_equal(ids, ids_ref)
    assert np.allclose(w, p_ref, rtol=1e-5, atol=0)


def _decode_plan(words, P):
    U = int(words[0])
    slots = []
    for u in range(U):
        e, c, st = int(words[1 + u]), int(words[1 + P + u]), int(words[1 + 2 * P + u])
        slots.append((e, [int(v) for v in words[1 + 3 * P + st: 1 + 3 * P + st + c]]))
    return U, slots


@pytest.mark.parametrize("T,topk,E", [(4, 8, 512), (3, 3, 6), (16, 16, 64), (1, 1, 1)])
def test_plan_word_for_word(gpu, T, topk, E):
    g = np.random.default_rng(T * 100 + topk)
    ids = np.stack([g.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    P = T * topk
    out = torch.empty(gpu.gq8_moe_plan_words(T, topk), dtype=torch.int32, device="cuda")
    gpu.gq8_moe_plan(to_dev(ids), T, topk, E, out)
    words = to_host(out)
    U, slots = _decode_plan(words, P)
    assert slots == plan(ids)
    assert sorted(i for _, es in slots for i in es) == list(range(P))   # every entry once
    assert all(words[1 + u] == -1 for u in range(U, P))


def test_plan_error_on_bad_id(gpu):
    ids = np.array([[0, 5], [1, 9]], np.int32)
    out = torch.empty(gpu.gq8_moe_plan_words(2, 2), dtype=torch.int32, device="cuda")
    gpu.gq8_moe_plan(to_dev(ids), 2, 2, 8, out)
    assert int(to_host(out)[0]) == -1


def _arena(gpu, experts, E, D, F, routed, seed, fill_unrouted=0x7F):
    """Device arenas with the routed experts quantized in place; the others hold junk bytes
    (so reading them would show)."""
    gu_b, dn_b = gpu.gq8_q8_0_bytes(2 * F, D), gpu.gq8_q8_0_bytes(D, F)
    agu = torch.full((E * gu_b,), fill_unrouted, dtype=torch.uint8, device="cuda")
    adn = torch.full((E * dn_b,), fill_unrouted, dtype=torch.uint8, device="cuda")
    for e in routed:
        w = experts(e)
        gpu.gq8_q8_0_quantize(to_dev(w["gate_up"]), 2 * F, D, agu[e * gu_b:(e + 1) * gu_b])
        gpu.gq8_q8_0_quantize(to_dev(w["down"]), D, F, adn[e * dn_b:(e + 1) * dn_b])
    return agu, adn


def _moe_case(gpu, T, E, topk, D, F, seed):
    inp = synth.moe_inputs(T=T, E=E, D=D, seed=seed)
    ids_ref, p_ref = route(inp["logits"], topk)
    experts = lambda e: synth.moe_expert_weights(e, D=D, F=F, seed=seed)  # noqa: E731
    routed = sorted(set(ids_ref.ravel().tolist()))
    agu, adn = _arena(gpu, experts, E, D, F, routed, seed)
    # device routing and q8_1 quantization (the product path's own)
    ids = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    w = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    gpu.gq8_moe_route(to_dev(inp["logits"]), T, E, topk, ids, w)
    xq = torch.empty((T, D), dtype=torch.int8, device="cuda")
    xd = torch.empty((T, D // 32), dtype=torch.int16, device="cuda")
    gpu.gq8_q8_1_quantize(to_dev(inp["x"]), T, D, xq, xd, None)
    nb = gpu.gq8_moe_workspace_bytes(T, topk, D, F)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, D), dtype=torch.int16, device="cuda")
    gpu.gq8_moe_q8_0_routed(xq, xd, ids, w, agu, adn, out, T, topk, E, D, F, ws, nb)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ids), ids_ref)
    x81 = quantize_q8_1_bf16(inp["x"])
    blocks = lambda e: (quantize_q8_0(experts(e)["gate_up"]), quantize_q8_0(experts(e)["down"]))  # noqa: E731
    y_ref, S = moe_forward(x81, ids_ref, p_ref, blocks)
    check_bf16(to_host(out, np.uint16), y_ref, S, f"moe T={T} E={E} topk={topk} D={D} F={F}")
    return out, (xq, xd, ids, w, agu, adn, ws, nb)


@pytest.mark.parametrize("T,E,topk,D,F", [(1, 8, 2, 64, 32), (3, 20, 4, 128, 64), (6, 40, 6, 1056, 96),
                                          (16, 64, 4, 256, 128),
                                          # MFMA down read (F = 256, 512, 1024): ragged D, an
                                          # expert with 16 entries (two chunks of 8)
                                          (16, 1, 1, 160, 256), (2, 10, 2, 96, 512),
                                          (5, 12, 3, 544, 1024), (16, 3, 2, 64, 512)])
def test_moe_small(gpu, T, E, topk, D, F):
    _moe_case(gpu, T, E, topk, D, F, seed=41)


def test_moe_full_size(gpu):
    T, E, topk, D, F = 4, 512, 8, 2048, 512
    out, (xq, xd, ids, w, agu, adn, ws, nb) = _moe_case(gpu, T, E, topk, D, F, seed=0)
    # replay determinism with the workspace poisoned
    out2 = torch.empty_like(out)
    ws.fill_(0xFF)
    gpu.gq8_moe_q8_0_routed(xq, xd, ids, w, agu, adn, out2, T, topk, E, D, F, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("D,F", [(2048, 512), (160, 96)])
def test_moe_crowded_expert(gpu, D, F):
    """ids given directly (the routed call accepts any ids in range): a token may name an expert
    twice and one expert takes 20 of the 32 entries, more than one 16-entry chunk of the gate/up
    kernel and one 8-entry chunk of the down kernel."""
    T, topk, E, seed = 16, 2, 3, 43
    inp = synth.moe_inputs(T=T, E=E, D=D, seed=seed)
    ids_ref = np.zeros((T, topk), np.int32)
    ids_ref[10:, 1] = 1
    ids_ref[12:, 0] = 2
    p_ref = synth.uniform_f32(seed, "moe.crowded.w", (T, topk), 0.1, 0.9)
    experts = lambda e: synth.moe_expert_weights(e, D=D, F=F, seed=seed)  # noqa: E731
    agu, adn = _arena(gpu, experts, E, D, F, [0, 1, 2], seed)
    xq = torch.empty((T, D), dtype=torch.int8, device="cuda")
    xd = torch.empty((T, D // 32), dtype=torch.int16, device="cuda")
    gpu.gq8_q8_1_quantize(to_dev(inp["x"]), T, D, xq, xd, None)
    nb = gpu.gq8_moe_workspace_bytes(T, topk, D, F)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, D), dtype=torch.int16, device="cuda")
    gpu.gq8_moe_q8_0_routed(xq, xd, to_dev(ids_ref), to_dev(p_ref), agu, adn, out, T, topk, E, D, F,
                            ws, nb)
    torch.cuda.synchronize()
    x81 = quantize_q8_1_bf16(inp["x"])
    blocks = lambda e: (quantize_q8_0(experts(e)["gate_up"]), quantize_q8_0(experts(e)["down"]))  # noqa: E731
    y_ref, S = moe_forward(x81, ids_ref, p_ref, blocks)
    check_bf16(to_host(out, np.uint16), y_ref, S, f"moe crowded D={D} F={F}")


@pytest.mark.parametrize("T,topk,E,D,F", [(1, 32, 64, 2048, 512), (2, 17, 40, 544, 256),
                                          (1, 20, 20, 160, 1024),
                                          # more entries x F than the grouped down read stages
                                          (2, 32, 80, 256, 512), (3, 20, 64, 96, 1024)])
def test_moe_more_than_16_slots(gpu, T, topk, E, D, F):
    """topk > 16 (ids given directly: the routing call stops at 16): more slots per token than
    the per-token down kernel keeps on chip, so the plan-based kernels run; the output passes the
    rules against the oracle."""
    seed = 49
    inp = synth.moe_inputs(T=T, E=E, D=D, seed=seed)
    g = np.random.default_rng(seed)
    ids_ref = np.stack([g.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    p_ref = synth.uniform_f32(seed, "moe.many.w", (T, topk), 0.01, 0.1)
    experts = lambda e: synth.moe_expert_weights(e, D=D, F=F, seed=seed)  # noqa: E731
    agu, adn = _arena(gpu, experts, E, D, F, sorted(set(ids_ref.ravel().tolist())), seed)
    xq = torch.empty((T, D), dtype=torch.int8, device="cuda")
    xd = torch.empty((T, D // 32), dtype=torch.int16, device="cuda")
    gpu.gq8_q8_1_quantize(to_dev(inp["x"]), T, D, xq, xd, None)
    nb = gpu.gq8_moe_workspace_bytes(T, topk, D, F)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, D), dtype=torch.int16, device="cuda")
    gpu.gq8_moe_q8_0_routed(xq, xd, to_dev(ids_ref), to_dev(p_ref), agu, adn, out, T, topk, E, D,
                            F, ws, nb)
    torch.cuda.synchronize()
    x81 = quantize_q8_1_bf16(inp["x"])
    blocks = lambda e: (quantize_q8_0(experts(e)["gate_up"]), quantize_q8_0(experts(e)["down"]))  # noqa: E731
    y_ref, S = moe_forward(x81, ids_ref, p_ref, blocks)
    check_bf16(to_host(out, np.uint16), y_ref, S, f"moe topk={topk} T={T} D={D} F={F}")


@pytest.mark.parametrize("T,E,topk,D,F", [(4, 512, 8, 2048, 512),      # the full workload
                                          (3, 20, 4, 128, 64),         # VALU down + plan
                                          (6, 40, 6, 1056, 96),        # ragged last chunk
                                          (5, 12, 3, 544, 1024),
                                          (2, 6, 2, 4160, 256)])       # D > 4096: quantize step
def test_moe_bf16_input_is_quantize_then_routed(gpu, T, E, topk, D, F):
    """The routed call on the bf16 input quantizes it to q8_1 on the device: bitwise the output of
    gq8_q8_1_quantize followed by gq8_moe_q8_0_routed (itself checked against the oracle)."""
    seed = 44
    out, (xq, xd, ids, w, agu, adn, ws, nb) = _moe_case(gpu, T, E, topk, D, F, seed=seed)
    x = to_dev(synth.moe_inputs(T=T, E=E, D=D, seed=seed)["x"])
    out2 = torch.empty_like(out)
    ws.fill_(0xFF)
    gpu.gq8_moe_q8_0_routed_bf16(x, ids, w, agu, adn, out2, T, topk, E, D, F, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), f"T={T} D={D} F={F}"


def _tie_input(T, D):
    """bf16 input whose 32-blocks hold 127 s (so the block scale is exactly s, a power of two)
    and half-integer multiples (j + 0.5) s, j = -127..126: every other quant is an exact tie of
    round(x / d), which goes away from zero."""
    x = np.empty((T, D), np.float32)
    j = np.arange(T * D) % 254 - 127
    x.ravel()[:] = j + 0.5
    x = x.reshape(T, D // 32, 32)
    x[:, :, 0] = 127.0
    s = 2.0 ** (np.arange(D // 32) % 7 - 3)
    x = (x * s[None, :, None]).astype(np.float32).reshape(T, D)
    return (x.view(np.uint32) >> 16).astype(np.uint16)    # exact: 8-bit significands


@pytest.mark.parametrize("D,F", [(2048, 512), (1056, 96)])
def test_moe_bf16_input_ties(gpu, D, F):
    """Exact ties in the q8_1 quantization of the input: the fused quantization agrees bitwise
    with gq8_q8_1_quantize (whose bytes match the oracle's quantizer) through the routed output."""
    from oracle.q8 import quantize_q8_1_bf16 as q81
    T, E, topk, seed = 3, 6, 2, 45
    xb = _tie_input(T, D)
    ids = np.array([[0, 3], [5, 0], [2, 4]], np.int32)
    p = synth.uniform_f32(seed, "moe.ties.w", (T, topk), 0.1, 0.9)
    experts = lambda e: synth.moe_expert_weights(e, D=D, F=F, seed=seed)  # noqa: E731
    agu, adn = _arena(gpu, experts, E, D, F, range(E), seed)
    xq = torch.empty((T, D), dtype=torch.int8, device="cuda")
    xd = torch.empty((T, D // 32), dtype=torch.int16, device="cuda")
    gpu.gq8_q8_1_quantize(to_dev(xb), T, D, xq, xd, None)
    ref = q81(xb)
    assert np.array_equal(to_host(xq).reshape(ref.q.shape), ref.q)   # the standalone quantizer at ties
    nb = gpu.gq8_moe_workspace_bytes(T, topk, D, F)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out1 = torch.empty((T, D), dtype=torch.int16, device="cuda")
    out2 = torch.empty_like(out1)
    dids, dp = to_dev(ids), to_dev(p)
    gpu.gq8_moe_q8_0_routed(xq, xd, dids, dp, agu, adn, out1, T, topk, E, D, F, ws, nb)
    gpu.gq8_moe_q8_0_routed_bf16(to_dev(xb), dids, dp, agu, adn, out2, T, topk, E, D, F, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("T,E,topk,D,F", [(16, 300, 16, 1024, 256), (16, 40, 16, 160, 512)])
def test_moe_most_entries(gpu, T, E, topk, D, F):
    """T * topk = 256 entries, the most the routed call takes: the entries of an expert span all
    four 64-entry words of the id ballot (E = 40: every expert has several entries)."""
    out, (xq, xd, ids, w, agu, adn, ws, nb) = _moe_case(gpu, T, E, topk, D, F, seed=46)
    x = to_dev(synth.moe_inputs(T=T, E=E, D=D, seed=46)["x"])
    out2 = torch.empty_like(out)
    gpu.gq8_moe_q8_0_routed_bf16(x, ids, w, agu, adn, out2, T, topk, E, D, F, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("T,E,topk,D,F", [(4, 512, 8, 2048, 512), (3, 20, 4, 544, 256),
                                          (5, 12, 3, 1056, 1024), (16, 40, 16, 160, 512)])
def test_moe_flags(gpu, T, E, topk, D, F):
    """gq8_moe_q8_0_routed_flags: flags 0 and X_BF16 are bitwise the two named calls; H_Q8_1 (the
    down read on q8_1(h), integer dots) passes the rule against the oracle's variant, on the int8
    and on the bf16 input (bitwise the same)."""
    seed = 47
    out, (xq, xd, ids, w, agu, adn, ws, nb) = _moe_case(gpu, T, E, topk, D, F, seed=seed)
    inp = synth.moe_inputs(T=T, E=E, D=D, seed=seed)
    xb = to_dev(inp["x"])
    o = {f: torch.empty_like(out) for f in (0, 1, 2, 3)}
    gpu.gq8_moe_q8_0_routed_flags(xq, xd, ids, w, agu, adn, o[0], T, topk, E, D, F, 0, ws, nb)
    gpu.gq8_moe_q8_0_routed_flags(xb, None, ids, w, agu, adn, o[1], T, topk, E, D, F,
                                  gpu.MOE_X_BF16, ws, nb)
    gpu.gq8_moe_q8_0_routed_flags(xq, xd, ids, w, agu, adn, o[2], T, topk, E, D, F,
                                  gpu.MOE_H_Q8_1, ws, nb)
    gpu.gq8_moe_q8_0_routed_flags(xb, None, ids, w, agu, adn, o[3], T, topk, E, D, F,
                                  gpu.MOE_X_BF16 | gpu.MOE_H_Q8_1, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(o[0], out) and torch.equal(o[1], out)
    assert torch.equal(o[3], o[2])
    ids_ref, p_ref = route(inp["logits"], topk)
    experts = lambda e: synth.moe_expert_weights(e, D=D, F=F, seed=seed)  # noqa: E731
    blocks = lambda e: (quantize_q8_0(experts(e)["gate_up"]), quantize_q8_0(experts(e)["down"]))  # noqa: E731
    y_ref, S = moe_forward(quantize_q8_1_bf16(inp["x"]), ids_ref, p_ref, blocks, h_q8_1=True)
    check_bf16(to_host(o[2], np.uint16), y_ref, S, f"moe q8_1(h) T={T} D={D} F={F}",
               page=False)   # its own rule: h re-quantized on both sides, codes may flip
    assert not torch.equal(o[2], out)                           # a different read


def _tile16_ref(split, rows, K, count):
    """The tiled layout by index arithmetic: per matrix, quants [rows][K] as 1 KiB tiles (row
    group G, column group c), piece l of a tile = row 16G + l%16, columns 64c + 16(l/16)..+16;
    scales unchanged."""
    mb = rows * K + rows * K // 16
    out = np.empty_like(split)
    for m in range(count):
        q = split[m * mb:m * mb + rows * K].reshape(rows // 16, 16, K // 64, 4, 16)
        out[m * mb:m * mb + rows * K] = q.transpose(0, 2, 3, 1, 4).reshape(-1)
        out[m * mb + rows * K:(m + 1) * mb] = split[m * mb + rows * K:(m + 1) * mb]
    return out


@pytest.mark.parametrize("rows,K,count", [(16, 64, 1), (32, 128, 3), (2048, 512, 2), (48, 1024, 2)])
def test_tile16_layout(gpu, rows, K, count):
    """gq8_q8_0_tile16 against the layout's definition written as index arithmetic, on random
    bytes (every byte distinct in position, so a misplaced piece shows)."""
    n = count * gpu.gq8_q8_0_bytes(rows, K)
    split = np.random.default_rng(rows + K + count).integers(0, 256, n, dtype=np.uint8)
    tiled = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    gpu.gq8_q8_0_tile16(to_dev(split), rows, K, count, tiled)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(tiled), _tile16_ref(split, rows, K, count))


@pytest.mark.parametrize("T,E,topk,D,F", [(4, 512, 8, 2048, 512), (3, 20, 4, 544, 256),
                                          (5, 12, 3, 1056, 1024), (16, 40, 16, 160, 512)])
def test_moe_down_tiled_is_the_split_read(gpu, T, E, topk, D, F):
    """GQ8_MOE_DOWN_TILED with the down arena tiled by gq8_q8_0_tile16: bitwise the output of the
    same call on the split-layout arena, for every combination of the other flags."""
    seed = 49
    out, (xq, xd, ids, w, agu, adn, ws, nb) = _moe_case(gpu, T, E, topk, D, F, seed=seed)
    xb = to_dev(synth.moe_inputs(T=T, E=E, D=D, seed=seed)["x"])
    adn_t = torch.empty_like(adn)
    gpu.gq8_q8_0_tile16(adn, D, F, E, adn_t)
    for flags in (0, gpu.MOE_X_BF16, gpu.MOE_H_Q8_1, gpu.MOE_X_BF16 | gpu.MOE_H_Q8_1):
        xx, xs = (xb, None) if flags & gpu.MOE_X_BF16 else (xq, xd)
        o_s = torch.full_like(out, 0x5555)
        o_t = torch.full_like(out, 0x2222)
        gpu.gq8_moe_q8_0_routed_flags(xx, xs, ids, w, agu, adn, o_s, T, topk, E, D, F, flags, ws, nb)
        gpu.gq8_moe_q8_0_routed_flags(xx, xs, ids, w, agu, adn_t, o_t, T, topk, E, D, F,
                                      flags | gpu.MOE_DOWN_TILED, ws, nb)
        torch.cuda.synchronize()
        assert torch.equal(o_t, o_s), f"flags={flags}"
        if flags in (0, gpu.MOE_X_BF16):
            assert torch.equal(o_t, out), f"flags={flags}"


@pytest.mark.parametrize("bad", [8, -1, 1 << 30])
@pytest.mark.parametrize("D,F", [(64, 256), (96, 64)])
@pytest.mark.parametrize("general", [False, True])
def test_moe_invalid_id_writes_zeros(gpu, monkeypatch, bad, D, F, general):
    """An id outside [0, E) anywhere in ids: every routed call writes an all-zero output (bf16
    +0) and reads no expert (the arenas hold junk). Every flag combination, the token down read
    (F = 256) and the plan-based kernels (F = 64, or forced)."""
    if general:
        monkeypatch.setenv("GQ8_FORCE_GENERIC", "1")
    T, E, topk = 2, 8, 2
    agu, adn = _arena(gpu, None, E, D, F, [], seed=0)
    ids = to_dev(np.array([[1, 3], [bad, 5]], np.int32))
    w = to_dev(np.full((T, topk), 0.5, np.float32))
    x = to_dev(np.full((T, D), 0x3F80, np.uint16))                # bf16 1.0
    xq = to_dev(np.ones((T, D), np.int8))
    xd = to_dev(np.full((T, D // 32), 0x2000, np.uint16))
    nb = gpu.gq8_moe_workspace_bytes(T, topk, D, F)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for flags in range(8):           # every combination of X_BF16, H_Q8_1 and DOWN_TILED
        if (flags & (gpu.MOE_H_Q8_1 | gpu.MOE_DOWN_TILED)) and F not in (256, 512, 1024):
            continue
        out = torch.full((T, D), 0x5555, dtype=torch.int16, device="cuda")
        xx, xs = (x, None) if flags & gpu.MOE_X_BF16 else (xq, xd)
        gpu.gq8_moe_q8_0_routed_flags(xx, xs, ids, w, agu, adn, out, T, topk, E, D, F, flags, ws, nb)
        torch.cuda.synchronize()
        assert not out.any(), f"flags={flags}"


def test_moe_graph_replay(gpu):
    """The routed calls (each flag combination) captured into one hipGraph and replayed, with
    eager work and a poisoned workspace between replays: every replay equals the eager output."""
    T, E, topk, D, F = 4, 64, 8, 2048, 512
    out, (xq, xd, ids, w, agu, adn, ws, nb) = _moe_case(gpu, T, E, topk, D, F, seed=48)
    xb = to_dev(synth.moe_inputs(T=T, E=E, D=D, seed=48)["x"])
    flags = (0, gpu.MOE_X_BF16, gpu.MOE_H_Q8_1, gpu.MOE_X_BF16 | gpu.MOE_H_Q8_1)
    outs = [torch.empty_like(out) for _ in flags]

    def calls(stream=None):
        for f, o in zip(flags, outs):
            xx, xs = (xb, None) if f & gpu.MOE_X_BF16 else (xq, xd)
            gpu.gq8_moe_q8_0_routed_flags(xx, xs, ids, w, agu, adn, o, T, topk, E, D, F, f, ws, nb, stream)

    calls()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert torch.equal(ref[0], out)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            calls(s)
    for _ in range(3):
        for o in outs:
            o.zero_()
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r)
