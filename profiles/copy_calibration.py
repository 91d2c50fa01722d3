"""Counter calibration: a plain device copy of a known size.

Run under `rocprofv3 --pmc FETCH_SIZE` (and separately WRITE_SIZE); the
counter read for this kernel, divided by the bytes it must move, is the
scale applied to the decode kernels' counters.
"""
import torch

N = 256 << 20  # bytes per buffer
x = torch.ones(N // 4, dtype=torch.float32, device="cuda:0")
y = torch.empty_like(x)
torch.cuda.synchronize()
for _ in range(3):
    torch.add(x, 1.0, out=y)  # reads N bytes, writes N bytes
torch.cuda.synchronize()
print(f"copy_calibration: {N} bytes read and {N} bytes written per launch")
