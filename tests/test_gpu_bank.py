"""GPU tests of the partial-residency expert bank: experts in pinned host memory, brought into HBM
slots route-aware in refill groups ("feat(v4/cuda): the CUDA tier wired into the DeepSeek V4
engine", PR #1055, "What it is", the Prefill MoE item).

The bank runs the grouped-GEMM kernels on the same weight bytes (now in slots), one refill group
per launch, so its output must equal the resident GEMM path bit for bit; one case is also checked
against the float64 oracle directly.
"""
import numpy as np
import pytest
import torch

import moe_synth as synth
import oracle
from helpers import random_experts, screened_tokens
from gpu_util import (check_outputs, check_routing, make_layer, oracle_routing, pack_weights, require_gpu, say,
                      stack_groups, x_to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _host_copy(packed):
    """Kernel-layout device weights -> pinned host copies (what a bank serves from)."""
    out = {}
    for mat, (c, s) in packed.items():
        hc = torch.empty(c.shape, dtype=torch.uint8, pin_memory=True)
        hs = torch.empty(s.shape, dtype=torch.uint8, pin_memory=True)
        hc.copy_(c)
        hs.copy_(s)
        out[mat] = (hc, hs)
    torch.cuda.synchronize()
    return out


def _pair(w_router, packed, top_k, shared, bias=None):
    """A resident GEMM-path layer and a host-weights layer over the same packed bytes."""
    from fp4_routed_expert_moe_amd import MoeLayer
    wr = torch.from_numpy(np.ascontiguousarray(w_router, dtype=np.float32)).cuda()
    b = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).cuda()
    resident = MoeLayer(wr, packed["gate"], packed["up"], packed["down"], top_k, shared, b, "gemm")
    host = _host_copy(packed)
    hosted = MoeLayer(wr, host["gate"], host["up"], host["down"], top_k, shared, b, "gemm", host_weights=True)
    return resident, hosted


def _run_both(resident, bank, x_bits):
    x = x_to_device(x_bits)
    t = x.shape[0]
    r1, r2 = resident.route_buffers(t), resident.route_buffers(t)
    want = resident.forward(x, route=r1)
    got = bank.forward(x, route=r2)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32)), "bank output differs from the resident GEMM path"
    for k in r1:
        assert torch.equal(r1[k], r2[k]), k
    return {k: v.cpu().numpy() for k, v in r2.items()} | {"y": got.cpu().numpy()}


def _case(seed, hidden, experts, top_k, inter, shared=1):
    rng = np.random.default_rng(seed)
    groups = random_experts(rng, hidden, inter, experts + shared)
    wr = (0.02 * rng.standard_normal((experts, hidden))).astype(np.float32)
    return groups, wr


def test_small_bank_many_refill_groups_matches_resident_and_oracle():
    # 17 groups through a 4-slot bank two at a time: slots are reused within a call (after the
    # kernels of the refill group two back), and across calls
    from fp4_routed_expert_moe_amd import MoeBank
    groups, wr = _case(61, 256, 16, 4, 128)
    resident, hosted = _pair(wr, pack_weights(stack_groups(groups)), 4, 1)
    bank = MoeBank(hosted, n_slots=4, group=2)
    wl = synth.custom_workload("bank1", 256, 16, 4, 1, 128, 100)
    x = screened_tokens(wl, wr, None)
    got = _run_both(resident, bank, x)
    ref = oracle.moe_forward(x, wr, None, groups, 4, 1)
    check_routing(got, ref, x, wr)
    check_outputs(got["y"], ref["y"], "bank vs oracle")
    st = bank.stats()
    need = int((got["counts"] > 0).sum()) + 1
    assert st["calls"] == 1 and st["refill_groups"] == (need + 1) // 2
    assert st["resident_hits"] == 0 and st["uploads"] == need
    for t in (37, 1, 100):
        _run_both(resident, bank, x[:t])
    st2 = bank.stats()
    say(f"[bank 4 slots] {st2}")
    assert st2["calls"] == 4 and st2["uploads"] >= st["uploads"]


def test_bank_holding_every_group_uploads_once():
    from fp4_routed_expert_moe_amd import MoeBank
    groups, wr = _case(62, 256, 16, 4, 128)
    resident, hosted = _pair(wr, pack_weights(stack_groups(groups)), 4, 1)
    bank = MoeBank(hosted, n_slots=17, group=4)
    wl = synth.custom_workload("bank2", 256, 16, 4, 1, 128, 64)
    x = screened_tokens(wl, wr, None)
    got = _run_both(resident, bank, x)
    need = int((got["counts"] > 0).sum()) + 1
    first = bank.stats()
    assert first["uploads"] == need and first["resident_hits"] == 0
    _run_both(resident, bank, x)
    second = bank.stats()
    assert second["uploads"] == need, "a resident expert was uploaded again"
    assert second["resident_hits"] == need
    per_expert = sum(int(t.numel()) for c, s in hosted._keep[1:4] for t in (c[0], s[0]))
    assert second["bytes_uploaded"] == need * per_expert


@pytest.mark.parametrize("n_slots,group", [(6, 3), (8, 1), (12, 6)])
def test_bank_shapes_and_varying_batches(n_slots, group):
    from fp4_routed_expert_moe_amd import MoeBank
    groups, wr = _case(63, 512, 64, 6, 256, shared=0)      # no shared expert, 64 experts
    resident, hosted = _pair(wr, pack_weights(stack_groups(groups)), 6, 0)
    bank = MoeBank(hosted, n_slots=n_slots, group=group)
    wl = synth.custom_workload("bank3", 512, 64, 6, 0, 256, 300)
    x = screened_tokens(wl, wr, None)
    for t in (300, 5, 129, 300):
        _run_both(resident, bank, x[:t])
    st = bank.stats()
    assert st["calls"] == 4 and st["uploads"] + st["resident_hits"] > 0


def test_bank_with_wide_gateup_slices():
    # 300 tokens over 8 experts + shared (100 grouped rows a group) take the gate/up kernel's
    # 256-column slices (I = 384: the second slice runs past I); 40 tokens take the 128-column
    # ones.  Both through a 4-slot bank with refills, bitwise against the resident layer.
    from fp4_routed_expert_moe_amd import MoeBank
    groups, wr = _case(66, 256, 8, 2, 384)
    resident, hosted = _pair(wr, pack_weights(stack_groups(groups)), 2, 1)
    bank = MoeBank(hosted, n_slots=4, group=2)
    wl = synth.custom_workload("bank4", 256, 8, 2, 1, 384, 300)
    x = screened_tokens(wl, wr, None)
    for t in (300, 40):
        got = _run_both(resident, bank, x[:t])
        ref = oracle.moe_forward(x[:t], wr, None, groups, 2, 1)
        check_routing(got, ref, x[:t], wr)
        check_outputs(got["y"], ref["y"], f"bank, {t} tokens, vs oracle")
    assert bank.stats()["calls"] == 2


def test_bank_rejects_device_weights_and_small_banks():
    from fp4_routed_expert_moe_amd import MoeBank, MoeError
    groups, wr = _case(64, 256, 8, 2, 128)
    packed = pack_weights(stack_groups(groups))
    resident, hosted = _pair(wr, packed, 2, 1)
    with pytest.raises(MoeError) as ei:
        MoeBank(resident, n_slots=4, group=2)          # weights on the device, not page-locked host memory
    assert ei.value.status == 1
    with pytest.raises(MoeError):
        MoeBank(hosted, n_slots=3, group=2)
    with pytest.raises(ValueError):                    # pageable host tensors are refused by the binding
        from fp4_routed_expert_moe_amd import MoeLayer
        cpu = {m: (c.cpu(), s.cpu()) for m, (c, s) in packed.items()}
        MoeLayer(resident._keep[0], cpu["gate"], cpu["up"], cpu["down"], 2, 1, host_weights=True)


def test_prefill_512_through_a_bank_full_size():
    # V4 Flash dims: 3.4 GB of experts in pinned host memory, a 48-slot bank (0.64 GB) refilled
    # 16 experts at a time; the output equals the resident GEMM path bit for bit
    from fp4_routed_expert_moe_amd import MoeBank
    wl = synth.WORKLOADS["prefill_t512"]
    packed = pack_weights(synth.layer_weights(wl, 0, device="cuda"))
    wr = synth.router_weights(wl, 0)
    resident, hosted = _pair(wr, packed, wl.top_k, wl.shared)
    bank = MoeBank(hosted, n_slots=48, group=16)
    x = screened_tokens(wl, wr, None)
    got = _run_both(resident, bank, x)
    check_routing(got, oracle_routing(x, wr, None, wl.top_k), x, wr)
    st = bank.stats()
    say(f"[bank prefill_t512] {st}")
    need = int((got["counts"] > 0).sum()) + 1
    assert st["uploads"] == need and st["refill_groups"] == (need + 15) // 16
