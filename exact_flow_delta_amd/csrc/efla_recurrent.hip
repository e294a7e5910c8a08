// efla_recurrent.hip -- one EFLA decode token for many independent (sequence, head) states, in place.
//
// Per state S (d_k x d_v, fp32), with a = S^T k and b = S^T q read from the state before the update:
//   lambda = ||k||^2,  alpha = (1 - e^{-beta lambda}) / lambda
//   S <- S + alpha k (v - a)^T                  (= (I - alpha k k^T) S + alpha k v^T)
//   o  = b + alpha (k^T q) (v - a)              (= S_new^T q, the post-update readout)
// ("Error-Free Linear Attention is a Free Lunch", pipeline summary and Steps 1-3; "Exact Flow Linear
// Attention", Metodologia item 3.)  The rearranged readout needs one read and one write of S.
//
// Bound by HBM: one workgroup streams one state.  Thread (rg, cg) owns the 4 columns 4cg..4cg+3 of
// rows rg, rg+RG, rg+2RG, ...; each load instruction of a wave covers consecutive rows, so a wave
// reads and writes contiguous 1 KB runs.  All loads of the state are issued before any arithmetic.
// Partial k^T S and q^T S are reduced across the row groups of a wave with cross-lane adds and
// across waves through LDS.
#include "efla_common.hpp"
#include "efla_launch.hpp"

namespace efla {

template <int DK, int DV>
struct StepShape {
    static constexpr int CG = DV / 4;                                  // float4 column groups
    static constexpr int NT = (CG * DK < 256) ? CG * DK : 256;         // threads per state
    static constexpr int RG = NT / CG;                                 // row groups
    static constexpr int RPT = DK / RG;                                // rows per thread
    static constexpr int NW = NT / 64;                                 // waves
    static constexpr int RGW = 64 / CG;                                // row groups per wave
};

template <typename E, int DK, int DV>
__global__ __launch_bounds__((StepShape<DK, DV>::NT)) void recurrent_step_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const float* __restrict__ beta,
    float* __restrict__ state, E* __restrict__ o, int gate) {
    typedef StepShape<DK, DV> SH;
    __shared__ float red_a[SH::NW][DV];
    __shared__ float red_b[SH::NW][DV];
    __shared__ float red_s[SH::NW][2];

    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % SH::CG;
    const int rg = tid / SH::CG;
    const int wave = tid >> 6;
    float* S = state + n * (int64_t)(DK * DV);

    f32x4 s[SH::RPT];
#pragma unroll
    for (int i = 0; i < SH::RPT; ++i) {
        const int r = rg + SH::RG * i;
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + r * DV + 4 * cg));
    }
    float kr[SH::RPT], qr[SH::RPT];
#pragma unroll
    for (int i = 0; i < SH::RPT; ++i) {
        const int r = rg + SH::RG * i;
        kr[i] = to_f32<E>(k[n * DK + r]);
        qr[i] = to_f32<E>(q[n * DK + r]);
    }
    const float bt = beta[n];
    f32x4 vv;
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = to_f32<E>(v[n * DV + 4 * cg + j]);

    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    float lam = 0.f, kq = 0.f;
#pragma unroll
    for (int i = 0; i < SH::RPT; ++i) {
        a += kr[i] * s[i];
        b += qr[i] * s[i];
        lam += kr[i] * kr[i];
        kq += kr[i] * qr[i];
    }
    // reduce over the row groups held by this wave (lanes CG apart)
#pragma unroll
    for (int off = SH::CG; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] += __shfl_xor(a[j], off, 64);
            b[j] += __shfl_xor(b[j], off, 64);
        }
        lam += __shfl_xor(lam, off, 64);
        kq += __shfl_xor(kq, off, 64);
    }
    const int lane = tid & 63;
    if (lane < SH::CG) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            red_a[wave][4 * cg + j] = a[j];
            red_b[wave][4 * cg + j] = b[j];
        }
        if (cg == 0) {
            red_s[wave][0] = lam;
            red_s[wave][1] = kq;
        }
    }
    __syncthreads();
    a = f32x4{0.f, 0.f, 0.f, 0.f};
    b = f32x4{0.f, 0.f, 0.f, 0.f};
    lam = 0.f;
    kq = 0.f;
#pragma unroll
    for (int w = 0; w < SH::NW; ++w) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] += red_a[w][4 * cg + j];
            b[j] += red_b[w][4 * cg + j];
        }
        lam += red_s[w][0];
        kq += red_s[w][1];
    }
    // every row of the key was summed exactly once into lambda and k^T q
    const float alpha = gate_alpha(bt, lam, gate);
    const f32x4 d = vv - a;
#pragma unroll
    for (int i = 0; i < SH::RPT; ++i) {
        const int r = rg + SH::RG * i;
        const f32x4 ns = s[i] + (alpha * kr[i]) * d;
        __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(S + r * DV + 4 * cg));
    }
    if (rg == 0) {
        const f32x4 ov = b + (alpha * kq) * d;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[n * DV + 4 * cg + j] = from_f32<E>(ov[j]);
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_step_t(const void* q, const void* k, const void* v, const float* beta, float* state,
                                void* o, int64_t NH, int gate, hipStream_t stream) {
    hipLaunchKernelGGL((recurrent_step_kernel<E, DK, DV>), dim3((unsigned)NH), dim3(StepShape<DK, DV>::NT), 0,
                       stream, static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), beta,
                       state, static_cast<E*>(o), gate);
    return hipGetLastError();
}

template <typename E, int DK>
static hipError_t launch_step_dv(const void* q, const void* k, const void* v, const float* beta, float* state,
                                 void* o, int64_t NH, int d_v, int gate, hipStream_t stream) {
    switch (d_v) {
        case 16: return launch_step_t<E, DK, 16>(q, k, v, beta, state, o, NH, gate, stream);
        case 32: return launch_step_t<E, DK, 32>(q, k, v, beta, state, o, NH, gate, stream);
        case 64: return launch_step_t<E, DK, 64>(q, k, v, beta, state, o, NH, gate, stream);
        case 128: return launch_step_t<E, DK, 128>(q, k, v, beta, state, o, NH, gate, stream);
    }
    return hipErrorInvalidValue;
}

template <typename E>
static hipError_t launch_step_e(const void* q, const void* k, const void* v, const float* beta, float* state,
                                void* o, int64_t NH, int d_k, int d_v, int gate, hipStream_t stream) {
    switch (d_k) {
        case 16: return launch_step_dv<E, 16>(q, k, v, beta, state, o, NH, d_v, gate, stream);
        case 32: return launch_step_dv<E, 32>(q, k, v, beta, state, o, NH, d_v, gate, stream);
        case 64: return launch_step_dv<E, 64>(q, k, v, beta, state, o, NH, d_v, gate, stream);
        case 128: return launch_step_dv<E, 128>(q, k, v, beta, state, o, NH, d_v, gate, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_recurrent_step(const void* q, const void* k, const void* v, const float* beta, efla_dtype dt,
                                 float* state, void* o, int64_t NH, int d_k, int d_v, int gate, hipStream_t stream) {
    if (dt == EFLA_BF16) return launch_step_e<bf16>(q, k, v, beta, state, o, NH, d_k, d_v, gate, stream);
    return launch_step_e<float>(q, k, v, beta, state, o, NH, d_k, d_v, gate, stream);
}

}  // namespace efla
