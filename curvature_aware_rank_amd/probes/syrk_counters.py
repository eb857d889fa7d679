"""Counter driver for the covariance SYRK: three accumulations of a 65536 x 4096 bf16
token block (the attention-projection workload) into a 4096 x 4096 fp32 sum, then one
plain 256 MiB device copy that calibrates FETCH_SIZE / WRITE_SIZE.  Run it under
rocprofv3 --pmc (one counter group per run), from the repository root."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import torch  # noqa: E402

import curvature_aware_rank_amd as lrc  # noqa: E402

d, n = 4096, 65536
dev = torch.device("cuda:0")
g = torch.Generator(device="cuda")
g.manual_seed(1)
a = torch.randn(n, d, generator=g, device=dev).to(torch.bfloat16)
cov = torch.zeros(d, d, dtype=torch.float32, device=dev)
for _ in range(3):
    cov.zero_()
    lrc.lrc_accumulate_cov(a, cov)
torch.cuda.synchronize()
src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)   # 256 MiB
dst = torch.empty_like(src)
dst.copy_(src)
torch.cuda.synchronize()
print("done", flush=True)
