// O_cache correction: the decision scale's residual output (full minus
// sparse attention output) upsampled nearest onto a later scale and added to
// that scale's sparse attention output (SparVAR, ai.info summary,
// "Methodology in Plain English", first module; "Main Findings", the item on
// the two modules' increments).
//
// Element-wise and HBM-bound: one lane per 16 bytes (8 bf16 of one token's
// head dimension), consecutive lanes on consecutive 16-byte units of a row, so
// every access is a full 16-byte vector and a wave reads whole rows.  Target
// token (y, x) at side h_T reads decision token (floor(y h_D / h_T),
// floor(x h_D / h_T)); the (h_T / h_D)^2 target tokens sharing a source read
// it from L2.  Arithmetic in fp32, one rounding to bf16 (nearest-even).
#include "kernel_args.h"

namespace vs {

__global__ __launch_bounds__(256) void ocache_correct_kernel(const OcacheArgs a) {
    const int bh = blockIdx.y;
    const int b = bh / a.H, h = bh - b * a.H;
    const int units = a.head_dim >> 3;                        // 16-byte units per row
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nt = (int64_t)a.side_t * a.side_t;
    if (e >= nt * units) return;
    const int t = (int)(e / units), u = (int)(e - (int64_t)t * units);
    const int y = t / a.side_t, x = t - y * a.side_t;
    const int s = (int)(((int64_t)y * a.side_d) / a.side_t) * a.side_d + (int)(((int64_t)x * a.side_d) / a.side_t);

    const bf16x8 f = *(const bf16x8*)(a.o_full + b * a.sf_b + h * a.sf_h + s * a.sf_t + 8 * u);
    const bf16x8 p = *(const bf16x8*)(a.o_sparse + b * a.sp_b + h * a.sp_h + s * a.sp_t + 8 * u);
    __bf16* op = a.o_t + b * a.so_b + h * a.so_h + t * a.so_t + 8 * u;
    const bf16x8 o = *(const bf16x8*)op;
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)((float)o[i] + ((float)f[i] - (float)p[i]));
    *(bf16x8*)op = r;
}

hipError_t launch_ocache_correct(const OcacheArgs& a, hipStream_t stream) {
    const int64_t work = (int64_t)a.side_t * a.side_t * (a.head_dim >> 3);
    dim3 grid((unsigned)((work + 255) / 256), (unsigned)(a.B * a.H)), block(256);
    hipLaunchKernelGGL(ocache_correct_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace vs
