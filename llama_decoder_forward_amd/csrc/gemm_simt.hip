// LDS-tiled vector-ALU GEMM for the fp32 (debug/reference precision) instantiation:
// acc[m][n] = sum_k A[m][k] W[n][k] in fp32.  64 x 64 output tile per 256-thread block,
// each thread 4 rows (m) x 4 consecutive columns (n).  Any M, N % 4 == 0, any K.
#include "launch.hpp"

namespace lk {

namespace {

constexpr int TS = 64, TK = 16;

template <typename T, bool DUAL, typename Epi>
__global__ __launch_bounds__(256) void gemm_simt_kernel(const T* __restrict__ A, int lda,
                                                        WeightRows<T> W, WeightRows<T> W3,
                                                        int M, int N, int K, Epi epi) {
    __shared__ float As[TK][TS + 4];
    __shared__ float Ws[TK][TS + 4];
    __shared__ float W3s[DUAL ? TK : 1][TS + 4];
    const int t = threadIdx.x;
    const int m0 = blockIdx.y * TS, n0 = blockIdx.x * TS;
    const int tx = t & 15, ty = t >> 4;  // columns tx*4.., rows ty*4..
    float acc[4][4] = {}, acc3[DUAL ? 4 : 1][4] = {};
    // loader: 64 rows x 16 k, each thread one row-quarter (4 consecutive k)
    const int lr = t >> 2, lk4 = (t & 3) * 4;
    const T* wrow = (n0 + lr < N) ? W.row(n0 + lr) : nullptr;
    const T* w3row = (DUAL && n0 + lr < N) ? W3.row(n0 + lr) : nullptr;
    const T* arow = (m0 + lr < M) ? A + (size_t)(m0 + lr) * lda : nullptr;
    for (int k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + lk4 + i;
            As[lk4 + i][lr] = (arow && k < K) ? to_f32(arow[k]) : 0.0f;
            Ws[lk4 + i][lr] = (wrow && k < K) ? to_f32(wrow[k]) : 0.0f;
            if (DUAL) W3s[lk4 + i][lr] = (w3row && k < K) ? to_f32(w3row[k]) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], w[4], w3[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = As[kk][ty * 4 + i];
                w[i] = Ws[kk][tx * 4 + i];
                if (DUAL) w3[i] = W3s[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
                    if (DUAL) acc3[i][j] = fmaf(a[i], w3[j], acc3[i][j]);
                }
        }
        __syncthreads();
    }
    const int n = n0 + tx * 4;
    if (n >= N) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty * 4 + i;
        if (m >= M) continue;
        if constexpr (DUAL) epi(m, n, acc[i], acc3[i]);
        else epi(m, n, acc[i]);
    }
}

template <typename T, bool DUAL, typename Epi>
hipError_t launch(const GemmArgs<void>& g, const Epi& e, hipStream_t s) {
    if (g.M == 0) return hipSuccess;
    const WeightRows<T> W{(const T*)g.W.p0, (const T*)g.W.p1, (const T*)g.W.p2, g.W.end0, g.W.end1, g.W.ld};
    const WeightRows<T> W3{(const T*)g.W3.p0, (const T*)g.W3.p1, (const T*)g.W3.p2, g.W3.end0, g.W3.end1, g.W3.ld};
    dim3 grid((g.N + TS - 1) / TS, (g.M + TS - 1) / TS);
    gemm_simt_kernel<T, DUAL, Epi><<<grid, 256, 0, s>>>((const T*)g.A, g.lda, W, W3, g.M, g.N, g.K, e);
    return hipGetLastError();
}

}  // namespace

// The vector-ALU path serves the fp32 instantiation; the bf16 instantiation uses the MFMA
// kernels (gemm_mfma.hip / gemm_skinny.hip) whose dispatchers call these for fp32.
hipError_t simt_store_f32(const GemmArgs<void>& g, EpiStoreF32 e, hipStream_t s) {
    return launch<float, false>(g, e, s);
}
hipError_t simt_residual(const GemmArgs<void>& g, EpiResidual e, hipStream_t s) {
    return launch<float, false>(g, e, s);
}
hipError_t simt_swiglu(const GemmArgs<void>& g, void* out, int ld, hipStream_t s) {
    return launch<float, true>(g, EpiSwiGLU<float>{(float*)out, ld}, s);
}
hipError_t simt_qkv(const GemmArgs<void>& g, const EpiQKV<void>& e, hipStream_t s) {
    // fp32 caches always keep the plain layouts (the packed one is bf16-only)
    EpiQKV<float> ef{(float*)e.q, (float*)e.kc, (float*)e.vc, e.rope, e.Nq, e.Nk, e.d, e.S,
                     e.start_pos, e.G, e.seq_stride, e.pos_dev, e.pos_stride, e.max_pos, 0};
    return launch<float, false>(g, ef, s);
}

}  // namespace lk
