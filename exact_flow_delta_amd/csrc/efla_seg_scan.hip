// efla_seg_scan.hip -- the scan between the segments of the segment-parallel forward.
//
// The state recurrence is affine in the state: over a segment of chunks, S_out = M S_in + S_out(0), with M the
// product of the chunks' transitions (I - K^T Ta K) and S_out(0) the segment's final state from a zero start
// ("Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4: chunks are joined by passing the
// state; "Exact Flow Linear Attention" (gist.science), Metodologia item 3: the update is linear in S).  A first
// state pass over every segment at once, on the state augmented with d_k transition columns that start as the
// identity and see zero values, leaves [S_g(0) | M_g] per (head, segment g); this kernel chains them:
//   S_in[0] = S0 (or 0),   S_in[g + 1] = M_g S_in[g] + S_g(0)
// and a second state pass over every segment from its S_in writes the outputs.  fp32 throughout; one
// workgroup per (head, 16 state columns) walks the segments in order.
#include "efla_common.hpp"
#include "efla_launch.hpp"

namespace efla {

template <int DK>
__global__ __launch_bounds__(256) void seg_scan_kernel(const float* __restrict__ seg_states, const float* __restrict__ s0,
                                                       float* __restrict__ s_in, int nseg, int DV) {
    constexpr int PER = DK * 16 / 256;   // outputs per thread: rows (tid + 256 j) / 16, column tid % 16
    static_assert(PER >= 1, "d_k of at least 16");
    __shared__ float sS[DK][17];
    const int tid = threadIdx.x;
    const int ntile = DV / 16;
    const int bh = blockIdx.x / ntile;
    const int col0 = (blockIdx.x % ntile) * 16;
    const int col = tid % 16;
    const int ld = DV + DK;
    float cur[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int row = (tid + 256 * j) / 16;
        cur[j] = s0 ? s0[((int64_t)bh * DK + row) * DV + col0 + col] : 0.0f;
    }
    for (int g = 0; g < nseg; ++g) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int row = (tid + 256 * j) / 16;
            s_in[(((int64_t)bh * nseg + g) * DK + row) * DV + col0 + col] = cur[j];
        }
        if (g + 1 == nseg) break;
        __syncthreads();   // every thread is done reading the previous S_in[g - 1] from LDS
#pragma unroll
        for (int j = 0; j < PER; ++j) sS[(tid + 256 * j) / 16][col] = cur[j];
        __syncthreads();
        const float* st = seg_states + ((int64_t)bh * nseg + g) * DK * ld;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int row = (tid + 256 * j) / 16;
            const float* mrow = st + (int64_t)row * ld + DV;   // row of M_g
            float acc = st[(int64_t)row * ld + col0 + col];   // S_g(0)
            for (int m = 0; m < DK; ++m) acc = fmaf(mrow[m], sS[m][col], acc);
            cur[j] = acc;
        }
    }
}

hipError_t launch_seg_scan(const float* seg_states, const float* s0, float* s_in, int BH, int nseg, int d_k, int d_v,
                           hipStream_t stream) {
    const dim3 grid((unsigned)(BH * (d_v / 16)));
    switch (d_k) {
        case 16: hipLaunchKernelGGL((seg_scan_kernel<16>), grid, dim3(256), 0, stream, seg_states, s0, s_in, nseg, d_v); break;
        case 32: hipLaunchKernelGGL((seg_scan_kernel<32>), grid, dim3(256), 0, stream, seg_states, s0, s_in, nseg, d_v); break;
        case 64: hipLaunchKernelGGL((seg_scan_kernel<64>), grid, dim3(256), 0, stream, seg_states, s0, s_in, nseg, d_v); break;
        case 128: hipLaunchKernelGGL((seg_scan_kernel<128>), grid, dim3(256), 0, stream, seg_states, s0, s_in, nseg, d_v); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace efla
