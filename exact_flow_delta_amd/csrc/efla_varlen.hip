// efla_varlen.hip -- token and chunk offsets of packed sequences.
//
// With packed sequences every sequence is cut into its own chunks (a chunk never spans two sequences, since
// each sequence starts from its own state), so the UT workspace holds, per head, ceil(len_b / C) chunks of
// sequence b.  This kernel sanitises the caller's offsets -- clamped to [0, L], then a running maximum, so
// that whatever they hold the sequences are disjoint ranges of [0, L) and their chunks fit the workspace sized
// for ceil(L / C) + nseq per head -- and writes the exclusive prefix of the chunk counts.  The UT transform
// and the state pass find a sequence's tokens and chunks from these arrays; a second kernel inverts the chunk
// prefix (chunk -> sequence), so that the UT transform finds a chunk's sequence with one lookup.
#include "efla_launch.hpp"

namespace efla {

__global__ __launch_bounds__(256) void varlen_prep_kernel(const int* __restrict__ cu_seqlens, int* __restrict__ cu_tok,
                                                          int* __restrict__ cu_chunks, int nseq, int L, int C) {
    __shared__ int pmax[256];
    __shared__ int psum[256];
    const int tid = threadIdx.x;
    auto clamped = [&](int b) { const int x = cu_seqlens[b]; return x < 0 ? 0 : x > L ? L : x; };
    int mcarry = 0;   // running maximum of the offsets before this block of 256
    int ccarry = 0;   // chunks of the sequences before this block
    for (int base = 0; base <= nseq; base += 256) {
        const int b = base + tid;
        // inclusive running maximum of the clamped offsets b = base .. base + 255 (<= nseq)
        pmax[tid] = b <= nseq ? clamped(b) : 0;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int y = tid >= off ? pmax[tid - off] : 0;
            __syncthreads();
            pmax[tid] = pmax[tid] > y ? pmax[tid] : y;
            __syncthreads();
        }
        const int m = pmax[tid] > mcarry ? pmax[tid] : mcarry;
        if (b <= nseq) cu_tok[b] = m;
        // the next offset's maximum: from this block, or for the block's last thread the next entry itself
        int m1 = m;
        if (b < nseq) {
            const int x1 = tid < 255 ? pmax[tid + 1] : clamped(b + 1);
            m1 = x1 > m ? x1 : m;
        }
        const int n = (m1 - m + C - 1) / C;   // chunks of sequence b (0 past the last)
        psum[tid] = n;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int y = tid >= off ? psum[tid - off] : 0;
            __syncthreads();
            psum[tid] += y;
            __syncthreads();
        }
        if (b < nseq) cu_chunks[b] = ccarry + psum[tid] - n;
        mcarry = pmax[255] > mcarry ? pmax[255] : mcarry;
        ccarry += psum[255];
        __syncthreads();
    }
    if (tid == 0) cu_chunks[nseq] = ccarry;
}

// chunk_seq[j] for every chunk j of a head: the last sequence whose chunks start at or before j (empty
// sequences share their start with the next one, so the last of equal starts is the one holding j)
__global__ __launch_bounds__(256) void varlen_chunk_seq_kernel(const int* __restrict__ cu_chunks,
                                                               int* __restrict__ chunk_seq, int nseq) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= cu_chunks[nseq]) return;
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_chunks[mid] <= j) lo = mid; else hi = mid - 1;
    }
    chunk_seq[j] = lo;
}

hipError_t launch_varlen_prep(const int* cu_seqlens, int* cu_tok, int* cu_chunks, int* chunk_seq, int nseq, int L,
                              int C, int max_chunks, hipStream_t stream) {
    hipLaunchKernelGGL(varlen_prep_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, cu_tok, cu_chunks, nseq, L, C);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || max_chunks <= 0) return e;
    hipLaunchKernelGGL(varlen_chunk_seq_kernel, dim3((unsigned)((max_chunks + 255) / 256)), dim3(256), 0, stream,
                       cu_chunks, chunk_seq, nseq);
    return hipGetLastError();
}

}  // namespace efla
