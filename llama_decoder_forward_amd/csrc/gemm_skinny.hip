// bf16 weight-streaming GEMM for few token rows (decode: M = batch <= 64):
// acc[m][n] = sum_k A[m][k] W[n][k], fp32 accumulate on 16x16x32 MFMAs.
//
// The cost is reading W once from HBM, so the kernel is shaped for bandwidth.  A workgroup
// owns a strip of RT x 16 weight rows (and as many of W3 for the SwiGLU pair); its NW waves
// split K between them and stream their share in 128-wide k blocks straight from global
// memory into MFMA operands, two blocks in flight (no LDS staging: the activations are a few
// hundred KB and stay in L2).  Lane (row n = l%16, quarter kq = l/16) reads 64 contiguous
// bytes of its row per block; the activation operand uses the same k permutation.  The
// waves' partial tiles are summed through LDS in wave order (deterministic), and the
// result, lane (token m = l%16 + 16 mb, quarter kq) holding rows n = 4kq..4kq+3, goes to the
// epilogue in the four-column groups it takes.
#include "launch.hpp"

namespace lk {

namespace {

constexpr int SK_ROWS = 16;  // weight rows per strip
constexpr int SK_KB = 128;   // k per block

template <int NW, int RT, int MB, bool DUAL, typename Epi>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(
    const bf16* __restrict__ A, int lda, WeightRows<bf16> W, WeightRows<bf16> W3, int M, int N,
    int K, Epi epi) {
    constexpr int NA = DUAL ? 2 : 1;
    __shared__ f32x4 red[NW > 1 ? NW - 1 : 1][NA * RT * MB][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int strip = blockIdx.x;             // RT tiles of 16 weight rows
    const int n0 = strip * SK_ROWS * RT;
    const int col = lane & 15, kq = lane >> 4;

    const bf16* wrow[RT];
    const bf16* w3row[DUAL ? RT : 1];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        wrow[r] = W.row(n0 + 16 * r + col) + kq * 32;
        if constexpr (DUAL) w3row[r] = W3.row(n0 + 16 * r + col) + kq * 32;
    }
    const bf16* arow[MB];
    bool avalid[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = mb * 16 + col;
        avalid[mb] = m < M;
        arow[mb] = A + (size_t)(avalid[mb] ? m : 0) * lda + kq * 32;
    }

    f32x4 acc[RT][MB], acc3[DUAL ? RT : 1][MB];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            acc[r][mb] = f32x4{};
            if constexpr (DUAL) acc3[r][mb] = f32x4{};
        }
    // this wave's share of the k blocks
    const int blocks = K / SK_KB;
    const int per = (blocks + NW - 1) / NW;
    const int kb0 = wave * per;
    const int kb1 = min(blocks, kb0 + per);

    // two register stages when they fit, one otherwise (then other waves hide the latency)
    constexpr int NS = (RT * NA + MB) <= 4 ? 2 : 1;
    u32x4 w[NS][RT][4], w3[NS][DUAL ? RT : 1][4], a[NS][MB][4];
    auto load = [&](int st, int kb) {
        const int k = kb * SK_KB;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                w[st][r][j] = *reinterpret_cast<const u32x4*>(wrow[r] + k + 8 * j);
                if constexpr (DUAL) w3[st][r][j] = *reinterpret_cast<const u32x4*>(w3row[r] + k + 8 * j);
            }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a[st][mb][j] = avalid[mb] ? *reinterpret_cast<const u32x4*>(arow[mb] + k + 8 * j)
                                          : u32x4{0, 0, 0, 0};
    };
    auto compute = [&](int st) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, w[st][r][j]), __builtin_bit_cast(bf16x8, a[st][mb][j]), acc[r][mb], 0, 0, 0);
                    if constexpr (DUAL)
                        acc3[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, w3[st][r][j]), __builtin_bit_cast(bf16x8, a[st][mb][j]), acc3[r][mb], 0, 0, 0);
                }
    };
    if constexpr (NS == 2) {
        if (kb0 < kb1) load(0, kb0);
        int kb = kb0;
        for (; kb + 1 < kb1; kb += 2) {
            load(1, kb + 1);
            compute(0);
            if (kb + 2 < kb1) load(0, kb + 2);
            compute(1);
        }
        if (kb < kb1) compute(0);
    } else {
        for (int kb = kb0; kb < kb1; ++kb) {
            load(0, kb);
            compute(0);
        }
    }

    if constexpr (NW > 1) {
        if (wave > 0) {
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    red[wave - 1][r * MB + mb][lane] = acc[r][mb];
                    if constexpr (DUAL) red[wave - 1][(RT + r) * MB + mb][lane] = acc3[r][mb];
                }
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w2 = 0; w2 < NW - 1; ++w2)
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[r][mb] += red[w2][r * MB + mb][lane];
                    if constexpr (DUAL) acc3[r][mb] += red[w2][(RT + r) * MB + mb][lane];
                }
    }

#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int m = mb * 16 + col;
            if (m >= M) continue;
            float v[4] = {acc[r][mb][0], acc[r][mb][1], acc[r][mb][2], acc[r][mb][3]};
            if constexpr (DUAL) {
                float u[4] = {acc3[r][mb][0], acc3[r][mb][1], acc3[r][mb][2], acc3[r][mb][3]};
                epi(m, n0 + 16 * r + 4 * kq, v, u);
            } else {
                epi(m, n0 + 16 * r + 4 * kq, v);
            }
        }
}

template <int RT, int MB, bool DUAL, typename Epi>
hipError_t launch_mb(const GemmArgs<void>& g, const Epi& e, hipStream_t s) {
    const WeightRows<bf16> W{(const bf16*)g.W.p0, (const bf16*)g.W.p1, (const bf16*)g.W.p2, g.W.end0, g.W.end1, g.W.ld};
    const WeightRows<bf16> W3{(const bf16*)g.W3.p0, (const bf16*)g.W3.p1, (const bf16*)g.W3.p2, g.W3.end0, g.W3.end1, g.W3.ld};
    const int strips = g.N / (SK_ROWS * RT);
    const bf16* A = (const bf16*)g.A;
    // waves per strip: enough waves in flight to cover HBM latency (about 2-4k waves)
    if (strips >= 2048)
        gemm_skinny_kernel<2, RT, MB, DUAL, Epi><<<strips, 128, 0, s>>>(A, g.lda, W, W3, g.M, g.N, g.K, e);
    else if (strips >= 384)
        gemm_skinny_kernel<4, RT, MB, DUAL, Epi><<<strips, 256, 0, s>>>(A, g.lda, W, W3, g.M, g.N, g.K, e);
    else
        gemm_skinny_kernel<8, RT, MB, DUAL, Epi><<<strips, 512, 0, s>>>(A, g.lda, W, W3, g.M, g.N, g.K, e);
    return hipGetLastError();
}

}  // namespace

bool skinny_ok(const GemmArgs<void>& g) {
    return g.M <= 64 && g.N % SK_ROWS == 0 && g.K % SK_KB == 0;
}

// Row tiles per wave (RT): every activation fragment serves RT weight tiles, which keeps the
// L2 traffic for activations below the weight stream when the batch is 32 or more; but RT
// also divides the number of waves, so it is used only where N leaves enough strips (the
// vocabulary projection, the gate/up pair).  Measured on MI355X at batch 4 and 32.
template <bool DUAL, typename Epi>
hipError_t skinny_launch(const GemmArgs<void>& g, const Epi& e, hipStream_t s) {
    const bool wide = g.N >= 16384;
    if (g.M <= 16) return launch_mb<1, 1, DUAL>(g, e, s);
    if constexpr (DUAL) {
        if (g.M <= 32 && g.N % (SK_ROWS * 2) == 0) return launch_mb<2, 2, DUAL>(g, e, s);
        if (g.M <= 32) return launch_mb<1, 2, DUAL>(g, e, s);
        return launch_mb<1, 4, DUAL>(g, e, s);
    } else {
        if (g.M <= 32 && wide && g.N % (SK_ROWS * 4) == 0) return launch_mb<4, 2, DUAL>(g, e, s);
        if (g.M <= 32) return launch_mb<1, 2, DUAL>(g, e, s);
        if (wide && g.N % (SK_ROWS * 2) == 0) return launch_mb<2, 4, DUAL>(g, e, s);
        return launch_mb<1, 4, DUAL>(g, e, s);
    }
}

template hipError_t skinny_launch<false, EpiStoreF32>(const GemmArgs<void>&, const EpiStoreF32&, hipStream_t);
template hipError_t skinny_launch<false, EpiResidual>(const GemmArgs<void>&, const EpiResidual&, hipStream_t);
template hipError_t skinny_launch<true, EpiSwiGLU<bf16>>(const GemmArgs<void>&, const EpiSwiGLU<bf16>&, hipStream_t);
template hipError_t skinny_launch<false, EpiQKV<bf16>>(const GemmArgs<void>&, const EpiQKV<bf16>&, hipStream_t);

}  // namespace lk
