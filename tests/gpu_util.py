"""Helpers for the GPU tests: move a seeded case to the device and run the
HIP verify through the C ABI binding."""
import numpy as np

import speculative_decoding_verification_07_amd as sv

MODES = {"sample": sv.SAMPLE, "greedy": sv.GREEDY, "point": sv.POINT}


def logits_to_dev(a, torch, offset=0):
    """numpy logits (float32 or bf16 bits) -> device tensor; `offset` > 0
    places the data `offset` elements into a larger buffer, so the base
    pointer is only element-aligned."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    if offset == 0:
        return t.cuda()
    flat = torch.empty(t.numel() + offset, dtype=t.dtype, device="cuda")
    flat[offset:] = t.reshape(-1).cuda()
    return flat[offset:].view(t.shape)


def case_to_dev(case, torch, offset=0):
    return dict(
        target=logits_to_dev(case.target, torch, offset),
        draft=None if case.mode == "point" else logits_to_dev(case.draft, torch, offset),
        tokens=torch.from_numpy(np.ascontiguousarray(case.tokens)).cuda(),
        uniforms=torch.from_numpy(np.ascontiguousarray(case.uniforms)).cuda(),
        gamma=torch.from_numpy(np.ascontiguousarray(case.gamma)).cuda(),
        kv=torch.from_numpy(np.ascontiguousarray(case.kv_len)).cuda())


def run(case, torch, probe=True, workspace=None, dev=None, offset=0):
    d = dev if dev is not None else case_to_dev(case, torch, offset)
    mode = MODES[case.mode]
    # point-mass drafts have no draft logits: pass none, so a read would fault loudly
    draft = None if case.mode == "point" else d["draft"]
    res = sv.verify(d["target"], draft, d["tokens"], d["uniforms"], d["gamma"], d["kv"],
                    temperature=case.T, mode=mode, workspace=workspace, probe=probe)
    torch.cuda.synchronize()
    out = [r.cpu().numpy() for r in res[:3]]
    pr = {k: v.cpu().numpy() for k, v in res[3].items()} if probe else None
    return out[0], out[1], out[2], pr
