"""Plain device copy of a known size, the reference kernel for scaling HBM
traffic counters (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE): one dispatch
reads exactly BYTES and writes exactly BYTES.

    python -m compressed_kv_cache_compress_amd.calibrate
"""
import torch

BYTES = 1 << 30


def main(reps=3):
    src = torch.ones(BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {BYTES} bytes x {reps}")


if __name__ == "__main__":
    main()
