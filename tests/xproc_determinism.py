"""Bitwise determinism across processes: writes a hash of every output of one
point of each workload, in each mode and output dtype, to a JSON file.  Run it
twice, in two separate processes, with different padding allocations (so the
operands sit at other device addresses), and compare the two files:

    python tests/xproc_determinism.py a.json 1
    python tests/xproc_determinism.py b.json 777
    python tests/xproc_determinism.py --compare a.json b.json

(Not collected by pytest: the comparison needs two fresh processes.)"""
import hashlib
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def compare(path_a, path_b):
    a, b = (json.load(open(p)) for p in (path_a, path_b))
    diff = sorted(k for k in set(a) | set(b) if a.get(k) != b.get(k))
    print("%d outputs, %d differ%s" % (len(a), len(diff), (": " + ", ".join(diff[:10])) if diff else ""))
    return 1 if diff else 0


def hashes(path, pad_mib):
    import torch
    import dpg_inputs
    import deterministic_bf16_projection_amd as dpg
    dev = torch.device("cuda:0")

    def bf(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

    def h(t):
        return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()[:16]

    # padding allocation: the operands land at other addresses than in the other run
    pad = torch.empty(pad_mib << 20, dtype=torch.uint8, device=dev)
    out = {}
    for (T, N, K) in ((64, 1024, 4096), (16384, 12288, 4096), (16231, 12288, 4096), (4031, 128, 4096),
                      (65537, 64, 4096), (16384, 1024, 4096)):
        x, w, dy = dpg_inputs.dense(T, N, K, seed_group=3)
        X, W, DY = bf(x), bf(w), bf(dy)
        for det, split in ((True, 0), (False, 0), (False, 1), (False, 2)):
            for od in (torch.bfloat16, torch.float32):
                key = "%d,%d,%d det=%d split=%d %s" % (T, N, K, det, split, str(od)[6:])
                out[key + " fwd"] = h(dpg.dpg_forward(X, W, out_dtype=od, deterministic=det, split_k=split))
                out[key + " dgrad"] = h(dpg.dpg_dgrad(DY, W, out_dtype=od, deterministic=det, split_k=split))
                out[key + " wgrad"] = h(dpg.dpg_wgrad(DY, X, out_dtype=od, deterministic=det, split_k=split))
        del X, W, DY
    for T in (64, 256, 1024):
        x, w, dy = dpg_inputs.router(T, 256, 4096, seed_group=3)
        X, W, DY = (torch.from_numpy(a).to(dev) for a in (x, w, dy))
        for det, split in ((True, 0), (False, 0), (False, 2)):
            key = "router T=%d det=%d split=%d" % (T, det, split)
            out[key + " fwd"] = h(dpg.dpg_router_forward(X, W, deterministic=det, split_k=split))
            out[key + " dgrad"] = h(dpg.dpg_router_dgrad(DY, W, deterministic=det, split_k=split))
            out[key + " wgrad"] = h(dpg.dpg_router_wgrad(DY, X, deterministic=det, split_k=split))
    torch.cuda.synchronize()
    del pad
    json.dump(out, open(path, "w"), indent=0)
    print(len(out), "hashes")
    return 0


if __name__ == "__main__":
    if len(sys.argv) == 4 and sys.argv[1] == "--compare":
        sys.exit(compare(sys.argv[2], sys.argv[3]))
    if len(sys.argv) != 3:
        sys.exit(__doc__)
    sys.exit(hashes(sys.argv[1], int(sys.argv[2])))
