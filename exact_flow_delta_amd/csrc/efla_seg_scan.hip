// efla_seg_scan.hip -- the scan between the segments of the segment-parallel forward.
//
// The state recurrence is affine in the state: over a segment of chunks, S_out = M S_in + S_out(0), with M the
// product of the chunks' transitions (I - K^T Ta K) and S_out(0) the segment's final state from a zero start
// ("Error-Free Linear Attention is a Free Lunch" (howistudyai.com), Step 4: chunks are joined by passing the
// state; "Exact Flow Linear Attention" (gist.science), Metodologia item 3: the update is linear in S).  A first
// state pass over every segment at once, on the state augmented with d_k transition columns that start as the
// identity and see zero values, leaves [S_g(0) | M_g] per (head, segment g); this kernel chains them:
//   S_in[0] = S0 (or 0),   S_in[g + 1] = M_g S_in[g] + S_g(0)
// and a second state pass over every segment from its S_in writes the outputs.
//
// One workgroup per (head, 16 state columns) walks the segments in order.  Per segment, M_g (d_k x d_k fp32) is
// staged in LDS with 16-byte loads (the next segment's already in registers) and the d_k x 16 product M_g S_in[g]
// runs on fp32 matrix cores (16x16x4), each wave owning 16-row tiles, accumulating onto S_g(0).  fp32 throughout.
#include "efla_common.hpp"
#include "efla_launch.hpp"

namespace efla {

template <int DK>
__global__ __launch_bounds__(256) void seg_scan_kernel(const float* __restrict__ seg_states, const float* __restrict__ s0,
                                                       float* __restrict__ s_in, int nseg, int DV) {
    constexpr int LDM = DK + 4;                 // row stride of the staged M (floats)
    constexpr int NRT = DK / 16;                // 16-row tiles of the product
    constexpr int TPW = (NRT + 3) / 4;          // tiles per wave (tile w + 4 s)
    constexpr int NV = DK * DK / 4 / 256;       // 16-byte pieces of M per thread (>= 1 for d_k >= 32)
    static_assert(DK >= 16, "d_k of at least 16");
    __shared__ __attribute__((aligned(16))) float sM[DK * LDM];
    __shared__ float sS[DK * 17];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int ntile = DV / 16;
    const int bh = blockIdx.x / ntile;
    const int col0 = (blockIdx.x % ntile) * 16;
    const int ld = DV + DK;

    // the state entering segment g: tile s of wave w, lane (r, g), element i = S[16 (w + 4 s) + 4 g + i][col0 + r]
    f32x4 cur[TPW];
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
        const int ti = w + 4 * s;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * ti + 4 * g + i;
            cur[s][i] = (ti < NRT && s0) ? s0[((int64_t)bh * DK + row) * DV + col0 + r] : 0.0f;
        }
    }
    // M_g in 16-byte pieces: piece p = tid + 256 j covers row p / (DK / 4), columns 4 (p % (DK / 4)) .. +3
    auto load_m = [&](int seg, f32x4* mv) __attribute__((always_inline)) {
        const float* st = seg_states + ((int64_t)bh * nseg + seg) * DK * ld + DV;
        if constexpr (NV >= 1) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int p = tid + 256 * j, row = p / (DK / 4), c4 = p % (DK / 4);
                mv[j] = *reinterpret_cast<const f32x4*>(st + (int64_t)row * ld + 4 * c4);
            }
        } else {
            const int row = tid / (DK / 4), c4 = tid % (DK / 4);
            if (row < DK) mv[0] = *reinterpret_cast<const f32x4*>(st + (int64_t)row * ld + 4 * c4);
        }
    };
    f32x4 mv[NV >= 1 ? NV : 1];
    if (nseg > 1) load_m(0, mv);
    for (int seg = 0; seg < nseg; ++seg) {
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int ti = w + 4 * s;
            if (ti < NRT) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s_in[(((int64_t)bh * nseg + seg) * DK + 16 * ti + 4 * g + i) * DV + col0 + r] = cur[s][i];
            }
        }
        if (seg + 1 == nseg) break;
        __syncthreads();   // every wave is done reading the previous segment's M and S from LDS
#pragma unroll
        for (int j = 0; j < (NV >= 1 ? NV : 1); ++j) {
            const int p = tid + 256 * j, row = p / (DK / 4), c4 = p % (DK / 4);
            if (NV >= 1 || row < DK) *reinterpret_cast<f32x4*>(&sM[row * LDM + 4 * c4]) = mv[j];
        }
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int ti = w + 4 * s;
            if (ti < NRT) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sS[(16 * ti + 4 * g + i) * 17 + r] = cur[s][i];
            }
        }
        __syncthreads();
        if (seg + 2 < nseg) load_m(seg + 1, mv);   // the next segment's M, under this product
        const float* st = seg_states + ((int64_t)bh * nseg + seg) * DK * ld;
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int ti = w + 4 * s;
            if (ti < NRT) {
                f32x4 acc;   // S_g(0), then += M_g S_in[g]
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = st[(int64_t)(16 * ti + 4 * g + i) * ld + col0 + r];
                const float* pa = &sM[(16 * ti + r) * LDM + g];
                const float* pb = &sS[g * 17 + r];
#pragma unroll 8
                for (int k = 0; k < DK; k += 4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k], pb[k * 17], acc, 0, 0, 0);
                cur[s] = acc;
            }
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
