// bf16 GEMM on the gfx950 matrix cores: acc[m][n] = sum_k A[m][k] W[n][k], fp32 accumulate.
//
// Both operands are K-contiguous ([rows][K] row-major), the layout of the checkpoint's
// [out, in] weights and of the activations.  The weight tile is the MFMA "A" operand (32
// weight rows per instruction) and the token tile the "B" operand (32 tokens), so that each
// lane of the 32x32 result holds four consecutive output columns n of one token row m:
// the RoPE pairs (2i, 2i+1) and the SwiGLU gate/up columns meet in one lane, and the
// epilogue stores 8- or 16-byte vectors.
//
// Block tile BN (weight rows) x BM (tokens) x 64 (k), staged through LDS in two buffers,
// 16-byte chunks XOR-swizzled by row (chunk c of row r at c ^ (r & 7)) so that the 32 lanes
// of an MFMA operand read hit distinct banks.  Global loads of step k+1 are issued before
// the MFMAs of step k.  Requires K % 64 == 0 and N % 4 == 0; M and N tails are masked.
#include "launch.hpp"

namespace lk {

hipError_t simt_store_f32(const GemmArgs<void>& g, EpiStoreF32 e, hipStream_t s);
hipError_t simt_residual(const GemmArgs<void>& g, EpiResidual e, hipStream_t s);
hipError_t simt_swiglu(const GemmArgs<void>& g, void* out, int ld, hipStream_t s);
hipError_t simt_qkv(const GemmArgs<void>& g, const EpiQKV<void>& e, hipStream_t s);

namespace {

constexpr int BK = 64;

template <int BN, int BM, int WN, int WM, bool DUAL, typename Epi>
__global__ __launch_bounds__(WN * WM * 64) void gemm_mfma_kernel(
    const bf16* __restrict__ A, int lda, WeightRows<bf16> W, WeightRows<bf16> W3, int M, int N,
    int K, Epi epi) {
    constexpr int NT = WN * WM * 64;
    constexpr int NA = DUAL ? 2 : 1;
    constexpr int ROWS = NA * BN + BM;       // rows of one LDS stage (64 bf16 = 8 chunks each)
    constexpr int CH = ROWS * 8 / NT;        // 16-byte chunks loaded per thread per stage
    constexpr int TN = BN / WN / 32, TM = BM / WM / 32;
    static_assert(ROWS * 8 % NT == 0, "tile/thread mismatch");
    extern __shared__ u32x4 lds[];           // [2][ROWS * 8]

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wn = wave / WM, wm = wave % WM;
    const int nt_m = (M + BM - 1) / BM;
    const int tile_m = blockIdx.x % nt_m, tile_n = blockIdx.x / nt_m;
    const int n0 = tile_n * BN, m0 = tile_m * BM;

    // each thread loads chunk (t & 7) of rows (t >> 3) + i * NT/8
    const int c = t & 7;
    const bf16* src[CH];
    int row_of[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int r = (t >> 3) + i * (NT / 8);
        row_of[i] = r;
        const bf16* p = nullptr;
        if (r < BN) {
            if (n0 + r < N) p = W.row(n0 + r);
        } else if (DUAL && r < 2 * BN) {
            if (n0 + r - BN < N) p = W3.row(n0 + r - BN);
        } else {
            const int m = m0 + r - NA * BN;
            if (m < M) p = A + (size_t)m * lda;
        }
        src[i] = p ? p + c * 8 : nullptr;
    }

    u32x4 regs[CH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CH; ++i)
            regs[i] = src[i] ? *reinterpret_cast<const u32x4*>(src[i] + k0) : u32x4{0, 0, 0, 0};
    };
    auto swrite = [&](int st) {
        u32x4* base = lds + st * ROWS * 8;
#pragma unroll
        for (int i = 0; i < CH; ++i) base[row_of[i] * 8 + (c ^ (row_of[i] & 7))] = regs[i];
    };

    f32x16 acc[TN][TM];
    f32x16 acc3[DUAL ? TN : 1][DUAL ? TM : 1];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            acc[i][j] = f32x16{};
            if constexpr (DUAL) acc3[i][j] = f32x16{};
        }

    const int lr = lane & 31, lh = lane >> 5;
    const int nk = K / BK;
    gload(0);
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        swrite(st);
        __syncthreads();
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const u32x4* base = lds + st * ROWS * 8;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = (kk * 2 + lh) ^ (lr & 7);
            bf16x8 a[TN], a3[DUAL ? TN : 1], b[TM];
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const int r = wn * (BN / WN) + i * 32 + lr;
                a[i] = __builtin_bit_cast(bf16x8, base[r * 8 + ch]);
                if constexpr (DUAL) a3[i] = __builtin_bit_cast(bf16x8, base[(BN + r) * 8 + ch]);
            }
#pragma unroll
            for (int j = 0; j < TM; ++j) {
                const int r = NA * BN + wm * (BM / WM) + j * 32 + lr;
                b[j] = __builtin_bit_cast(bf16x8, base[r * 8 + ch]);
            }
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
                    if constexpr (DUAL)
                        acc3[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3[i], b[j], acc3[i][j], 0, 0, 0);
                }
        }
    }

    // 32x32 result layout: lane (lr, lh), register 4g+q holds row 8g + 4lh + q (weight row
    // n) and column lr (token m).
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int m = m0 + wm * (BM / WM) + j * 32 + lr;
            if (m >= M) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * (BN / WN) + i * 32 + 8 * g + 4 * lh;
                if (n >= N) continue;
                float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
                if constexpr (DUAL) {
                    float u[4] = {acc3[i][j][4 * g], acc3[i][j][4 * g + 1], acc3[i][j][4 * g + 2], acc3[i][j][4 * g + 3]};
                    epi(m, n, v, u);
                } else {
                    epi(m, n, v);
                }
            }
        }
}

template <int BN, int BM, int WN, int WM, bool DUAL, typename Epi>
hipError_t launch_cfg(const GemmArgs<void>& g, const Epi& e, hipStream_t s) {
    const WeightRows<bf16> W{(const bf16*)g.W.p0, (const bf16*)g.W.p1, (const bf16*)g.W.p2, g.W.end0, g.W.end1, g.W.ld};
    const WeightRows<bf16> W3{(const bf16*)g.W3.p0, (const bf16*)g.W3.p1, (const bf16*)g.W3.p2, g.W3.end0, g.W3.end1, g.W3.ld};
    constexpr int ROWS = (DUAL ? 2 : 1) * BN + BM;
    constexpr size_t lds_bytes = 2 * ROWS * 8 * sizeof(u32x4);
    auto kern = gemm_mfma_kernel<BN, BM, WN, WM, DUAL, Epi>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    const int tiles = ((g.N + BN - 1) / BN) * ((g.M + BM - 1) / BM);
    kern<<<tiles, WN * WM * 64, lds_bytes, s>>>((const bf16*)g.A, g.lda, W, W3, g.M, g.N, g.K, e);
    return hipGetLastError();
}

template <bool DUAL, typename Epi>
hipError_t launch(const GemmArgs<void>& g, const Epi& e, hipStream_t s) {
    if (g.M == 0) return hipSuccess;
    if (skinny_ok(g)) return skinny_launch<DUAL>(g, e, s);
    if (g.M <= 32) return launch_cfg<128, 32, 4, 1, DUAL>(g, e, s);
    return launch_cfg<128, 128, 2, 2, DUAL>(g, e, s);
}

}  // namespace

hipError_t gemm_store_f32(Dt dt, const GemmArgs<void>& g, EpiStoreF32 e, hipStream_t s) {
    if (dt == Dt::F32) return simt_store_f32(g, e, s);
    return launch<false>(g, e, s);
}
hipError_t gemm_residual(Dt dt, const GemmArgs<void>& g, EpiResidual e, hipStream_t s) {
    if (dt == Dt::F32) return simt_residual(g, e, s);
    return launch<false>(g, e, s);
}
hipError_t gemm_swiglu(Dt dt, const GemmArgs<void>& g, void* out, int ld, hipStream_t s) {
    if (dt == Dt::F32) return simt_swiglu(g, out, ld, s);
    return launch<true>(g, EpiSwiGLU<bf16>{(bf16*)out, ld}, s);
}
hipError_t gemm_qkv(Dt dt, const GemmArgs<void>& g, const EpiQKV<void>& e, hipStream_t s) {
    if (dt == Dt::F32) return simt_qkv(g, e, s);
    EpiQKV<bf16> eb{(bf16*)e.q, (bf16*)e.kc, (bf16*)e.vc, e.rope, e.Nq, e.Nk, e.d, e.S,
                    e.start_pos, e.G, e.seq_stride, e.pos_dev};
    return launch<false>(g, eb, s);
}

}  // namespace lk
