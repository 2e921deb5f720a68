"""Plain device-to-device copy of a known size, for calibrating HBM byte
counters (FETCH_SIZE / WRITE_SIZE) against a transfer whose bytes are known:
one launch reads N bytes and writes N bytes.

    python -m token_level_sparse_amd.hbm_copy_probe [--mib 1024] [--reps 3]
"""
import argparse

import torch


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    a = ap.parse_args()
    n = a.mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(a.reps):
        ev[0].record()
        dst.copy_(src)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1])
        print(f"copy {a.mib} MiB: {ms * 1e3:.1f} us, {2 * n / ms / 1e6:.1f} GB/s (read+write)", flush=True)


if __name__ == "__main__":
    main()
