// efla_alpha.hip -- the exact gate alpha_t = (1 - e^{-beta_t ||k_t||^2}) / ||k_t||^2 for a batch of keys.
// ("Error-Free Linear Attention is a Free Lunch", Step 1; "Exact Flow Linear Attention",
// Metodologia item 3.)  HBM-bound: each key is read once with 16-byte loads; the lanes that share a
// key reduce ||k||^2 with cross-lane adds and one lane writes alpha.
#include "efla_common.hpp"
#include "efla_launch.hpp"

namespace efla {

template <typename E, int DK>
__global__ __launch_bounds__(256) void alpha_kernel(const E* __restrict__ k, const float* __restrict__ beta,
                                                    float* __restrict__ alpha, int64_t n, int gate) {
    typedef typename Vec16<E>::type V;
    constexpr int VEC = Vec16<E>::N;
    constexpr int LPT = DK / VEC;     // lanes per key
    constexpr int TPB = 256 / LPT;    // keys per workgroup
    const int64_t tok = (int64_t)blockIdx.x * TPB + threadIdx.x / LPT;
    const int part = threadIdx.x % LPT;
    float s = 0.0f;
    if (tok < n) {
        const V x = *reinterpret_cast<const V*>(k + tok * DK + part * VEC);
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            const float f = to_f32<E>(x[i]);
            s += f * f;
        }
    }
    s = group_sum<LPT>(s);
    if (tok < n && part == 0) alpha[tok] = gate_alpha(beta[tok], s, gate);
}

template <typename E, int DK>
static hipError_t launch_alpha_t(const void* k, const float* beta, float* alpha, int64_t n, int gate,
                                 hipStream_t stream) {
    constexpr int TPB = 256 / (DK / Vec16<E>::N);
    const int64_t blocks = (n + TPB - 1) / TPB;
    hipLaunchKernelGGL((alpha_kernel<E, DK>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const E*>(k), beta, alpha, n, gate);
    return hipGetLastError();
}

hipError_t launch_alpha(const void* k, efla_dtype dt, const float* beta, float* alpha, int64_t n, int d_k,
                        int gate, hipStream_t stream) {
    if (dt == EFLA_BF16) {
        switch (d_k) {
            case 16: return launch_alpha_t<bf16, 16>(k, beta, alpha, n, gate, stream);
            case 32: return launch_alpha_t<bf16, 32>(k, beta, alpha, n, gate, stream);
            case 64: return launch_alpha_t<bf16, 64>(k, beta, alpha, n, gate, stream);
            case 128: return launch_alpha_t<bf16, 128>(k, beta, alpha, n, gate, stream);
        }
    } else {
        switch (d_k) {
            case 16: return launch_alpha_t<float, 16>(k, beta, alpha, n, gate, stream);
            case 32: return launch_alpha_t<float, 32>(k, beta, alpha, n, gate, stream);
            case 64: return launch_alpha_t<float, 64>(k, beta, alpha, n, gate, stream);
            case 128: return launch_alpha_t<float, 128>(k, beta, alpha, n, gate, stream);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace efla
