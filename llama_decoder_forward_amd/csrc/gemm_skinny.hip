// bf16 weight-streaming GEMM for few token rows (decode: M = batch <= 64):
// acc[m][n] = sum_k A[m][k] W[n][k], fp32 accumulate on 16x16x32 MFMAs.
//
// The cost is reading W once from HBM, so the kernel is shaped for bandwidth.  A workgroup
// owns a strip of RT x 16 weight rows (and as many of W3 for the SwiGLU pair); its NW waves
// split K between them and stream their share in 128-wide k blocks straight from global
// memory into MFMA operands, up to three blocks in flight (no LDS staging: the activations
// are a few hundred KB and stay in L2).  For k-block kb and slice j (32 k),
// lane (row n = l%16, quarter kq = l/16) reads the 8 weights k = 128 kb + 32 j + 8 kq ..;
// the four lanes of a row cover 64 contiguous bytes.  The activations arrive in the packed
// layout of act_offset, where the matching operand of every (kb, j, row block) is one
// contiguous 1 KB run: a fully coalesced load, where the row-major layout would touch 16
// rows per load (measured on MI355X: half the time at batch 32).  The waves' partial tiles
// are summed through LDS in wave order (deterministic), and the result, lane (token
// m = l%16 + 16 mb, quarter kq) holding rows n = 4kq..4kq+3, goes to the epilogue in the
// four-column groups it takes.
#include "launch.hpp"

namespace lk {

namespace {

constexpr int SK_ROWS = 16;  // weight rows per strip
constexpr int SK_KB = 128;   // k per block

// Workgroup x owns weight rows n0 = x * rows .. min(N, n0 + rows) - 1 (rows a multiple of 8,
// at most 16 RT); the lanes of rows past the end load the last row again (the same lines as
// that row's lanes, so no extra memory traffic) and their results are dropped.
template <int NW, int RT, int MB, bool DUAL, int BUDGET, typename Epi>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(
    const bf16* __restrict__ A, int pack, WeightRows<bf16> W, WeightRows<bf16> W3, int M, int N,
    int K, int rows, Epi epi) {
    constexpr int NA = DUAL ? 2 : 1;
    __shared__ f32x4 red[NW > 1 ? NW - 1 : 1][NA * RT * MB][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * rows;
    const int n_end = min(N, n0 + rows);
    const int col = lane & 15, kq = lane >> 4;

    const bf16* wrow[RT];
    const bf16* w3row[DUAL ? RT : 1];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int n = min(n0 + 16 * r + col, n_end - 1);
        wrow[r] = W.row(n) + kq * 8;
        if constexpr (DUAL) w3row[r] = W3.row(n) + kq * 8;
    }
    // packed activations (act_offset): run (kb, j, mb) is 32 R values; lane (col, kq) takes
    // the 8 of row col % R
    const int R = pack < 16 ? pack : 16;
    const bf16* abase = A + (kq * R + (col & (R - 1))) * 8;

    f32x4 acc[RT][MB], acc3[DUAL ? RT : 1][MB];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            acc[r][mb] = f32x4{};
            if constexpr (DUAL) acc3[r][mb] = f32x4{};
        }
    // this wave's share of the k blocks: split blockIdx.y of gridDim.y takes a contiguous
    // range of blocks, its NW waves divide that range
    const int blocks = K / SK_KB;
    const int bps = (blocks + gridDim.y - 1) / gridDim.y;
    const int sb0 = min(blocks, (int)blockIdx.y * bps), sb1 = min(blocks, sb0 + bps);
    const int per = (sb1 - sb0 + NW - 1) / NW;
    const int kb0 = sb0 + wave * per;
    const int kb1 = min(sb1, kb0 + per);

    // register stages: as many blocks in flight as BUDGET VGPRs hold (a block takes 16
    // VGPRs per weight tile and per activation row block).  Deeper pipelines cost more in
    // occupancy than they gain (measured on MI355X, batch 1 to 64).
    constexpr int NS0 = BUDGET / ((RT * NA + MB) * 16);
    constexpr int NS = NS0 < 1 ? 1 : NS0 > 4 ? 4 : NS0;
    u32x4 w[NS][RT][4], w3[NS][DUAL ? RT : 1][4], a[NS][MB][4];
    auto load = [&](int st, int kb) {
        const int k = kb * SK_KB;
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                w[st][r][j] = *reinterpret_cast<const u32x4*>(wrow[r] + k + 32 * j);
                if constexpr (DUAL) w3[st][r][j] = *reinterpret_cast<const u32x4*>(w3row[r] + k + 32 * j);
            }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a[st][mb][j] = *reinterpret_cast<const u32x4*>(
                    abase + ((size_t)(kb * 4 + j) * MB + mb) * 32 * R);
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
    // Block kb0 + i lives in stage i % NS, NS - 1 blocks ahead are in flight.  The loads
    // are unconditional (past the end they reread the last block, which the cache holds):
    // a branch around a load makes the compiler wait for every outstanding load.
    if (kb0 < kb1) {
        const int last = kb1 - 1;
#pragma unroll
        for (int i = 0; i < NS - 1; ++i) load(i, min(kb0 + i, last));
        int kb = kb0;
        for (; kb + NS <= kb1; kb += NS) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                load((i + NS - 1) % NS, min(kb + i + NS - 1, last));
                __builtin_amdgcn_sched_barrier(0);  // issue the loads before waiting on block i
                compute(i);
            }
        }
        // the last < NS blocks are already loaded
#pragma unroll
        for (int i = 0; i < NS - 1; ++i)
            if (kb + i < kb1) compute(i);
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
#pragma unroll 1
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
            if (m >= M || n0 + 16 * r + 4 * kq >= n_end) continue;
            float v[4] = {acc[r][mb][0], acc[r][mb][1], acc[r][mb][2], acc[r][mb][3]};
            if constexpr (DUAL) {
                float u[4] = {acc3[r][mb][0], acc3[r][mb][1], acc3[r][mb][2], acc3[r][mb][3]};
                epi(m, n0 + 16 * r + 4 * kq, v, u);
            } else {
                epi(m, n0 + 16 * r + 4 * kq, v);
            }
        }
}

WeightRows<bf16> bf16_rows(const WeightRows<void>& w) {
    return WeightRows<bf16>{(const bf16*)w.p0, (const bf16*)w.p1, (const bf16*)w.p2, w.end0, w.end1, w.ld};
}

template <int RT, int MB, bool DUAL, typename Epi>
hipError_t launch_mb(const GemmArgs<void>& g, const Epi& e, hipStream_t s) {
    const WeightRows<bf16> W = bf16_rows(g.W), W3 = bf16_rows(g.W3);
    const int strips = g.N / (SK_ROWS * RT);
    const bf16* A = (const bf16*)g.A;
    // waves per strip: enough waves in flight to cover HBM latency (about 2-4k waves)
    const int rows = SK_ROWS * RT;
    if (strips >= 2048)
        gemm_skinny_kernel<2, RT, MB, DUAL, 96, Epi><<<strips, 128, 0, s>>>(A, g.a_pack, W, W3, g.M, g.N, g.K, rows, e);
    else if (strips >= 384)
        gemm_skinny_kernel<4, RT, MB, DUAL, 96, Epi><<<strips, 256, 0, s>>>(A, g.a_pack, W, W3, g.M, g.N, g.K, rows, e);
    else
        gemm_skinny_kernel<8, RT, MB, DUAL, 96, Epi><<<strips, 512, 0, s>>>(A, g.a_pack, W, W3, g.M, g.N, g.K, rows, e);
    return hipGetLastError();
}

// Split-K layout of the residual GEMMs: strips of SPLIT_RT x 16 rows, `splits` k ranges of
// NW waves, about LLAMA_SPLIT_TARGET_WGS workgroups (4 splits of 64 row strips for WO and
// W2 of the 8B shape: 13 and 29 us at batch 32 against 17 and 39 us unsplit, on MI355X).
#ifndef LLAMA_SPLIT_RT
#define LLAMA_SPLIT_RT 4
#endif
#ifndef LLAMA_SPLIT_TARGET_WGS
#define LLAMA_SPLIT_TARGET_WGS 256
#endif
#ifndef LLAMA_SPLIT_NW
#define LLAMA_SPLIT_NW 8
#endif
#ifndef LLAMA_SPLIT_BUDGET
#define LLAMA_SPLIT_BUDGET 96
#endif
constexpr int SPLIT_RT = LLAMA_SPLIT_RT;

template <int MB>
hipError_t launch_split(const GemmArgs<void>& g, float* part, int splits, hipStream_t s) {
    const EpiPartial e{part, g.N, (size_t)g.M * g.N};
    const dim3 grid(g.N / (SK_ROWS * SPLIT_RT), splits);
    gemm_skinny_kernel<LLAMA_SPLIT_NW, SPLIT_RT, MB, false, LLAMA_SPLIT_BUDGET, EpiPartial>
        <<<grid, LLAMA_SPLIT_NW * 64, 0, s>>>((const bf16*)g.A, g.a_pack, bf16_rows(g.W),
                                              bf16_rows(g.W3), g.M, g.N, g.K, SK_ROWS * SPLIT_RT, e);
    return hipGetLastError();
}

}  // namespace

int act_pack(Dt dt, int M, int N, int K) {
    if (dt != Dt::BF16 || M < 1 || M > 64 || N % SK_ROWS != 0 || K % SK_KB != 0) return 0;
    int P = 1;
    while (P < M) P *= 2;
    return P;
}

// Activation fragments are loaded once per weight tile of a wave, so at batch 32 a wave with
// one 16-row tile loads two bytes of activations per weight byte, and a compute unit streams
// only about 36 GB/s of loads, cache hits included (measured on MI355X).  A residual GEMM with
// few output rows (N = 4096) therefore gives each wave SPLIT_RT tiles and splits K over
// workgroups instead, to keep every compute unit busy; the splits' sums go to `part` and
// the next RMSNorm adds them to the residual stream.
int residual_splits(Dt dt, int M, int N, int K) {
    if (M > 64) return tiled_residual_splits(dt, M, N, K);
    if (act_pack(dt, M, N, K) == 0 || N % (SK_ROWS * SPLIT_RT) != 0) return 0;
    const int strips = N / (SK_ROWS * SPLIT_RT);
    const int blocks = K / SK_KB;
    int splits = (LLAMA_SPLIT_TARGET_WGS + strips - 1) / strips;
    splits = splits < blocks ? splits : blocks;
    splits = splits < LLAMA_MAX_KSPLITS ? splits : LLAMA_MAX_KSPLITS;
    return splits >= 2 ? splits : 0;
}

hipError_t gemm_residual_split(Dt dt, const GemmArgs<void>& g, float* part, int splits,
                               hipStream_t s) {
    if (dt == Dt::BF16 && g.M > 64) return gemm_residual_split_tiled(g, part, splits, s);
    if (dt != Dt::BF16 || splits != residual_splits(dt, g.M, g.N, g.K) ||
        g.a_pack != act_pack(dt, g.M, g.N, g.K))
        return hipErrorInvalidValue;
    const int mb = g.a_pack < 16 ? 1 : g.a_pack / 16;
    if (mb == 1) return launch_split<1>(g, part, splits, s);
    if (mb == 2) return launch_split<2>(g, part, splits, s);
    return launch_split<4>(g, part, splits, s);
}

// Row tiles per wave (RT): every activation fragment serves RT weight tiles, which keeps the
// L2 traffic for activations below the weight stream; but RT also divides the number of
// waves, so it is used only where N leaves enough strips (the vocabulary projection, the
// gate/up pair).  Measured on MI355X, 8B shape:
//   - vocabulary projection: 1 row 197 -> 176 us with RT 4; batch 32 209 -> 197 us with RT 8
//     (against RT 4);
//   - gate/up pair: batch 4 50 -> 45 us with RT 2; batch 32 52.9 -> 51.0 us with RT 4 and
//     4 waves per strip (RT 4 with the 8 waves its strip count would get: no faster);
//   - Q/K/V: at batch 4 RT 2 is slower (17 -> 21 us), so RT 1; from 17 rows on (two or
//     more 16-row blocks) two activation bytes per weight byte make RT 2 pay (batch 32:
//     24.6 -> 21.7 us).
// Compute units of the current device (the balanced launches give each one workgroup);
// 256 if the device cannot be queried.
int cu_count() {
    static PerDevice known;
    static std::atomic<int> cus[64];
    int n = 256;
    const hipError_t e = known.once([](int dev) {
        int v = 0;
        hipError_t r = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
        if (r == hipSuccess && v > 0 && dev < 64) cus[dev].store(v, std::memory_order_relaxed);
        return r;
    });
    int dev = 0;
    if (e == hipSuccess && hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        const int v = cus[dev].load(std::memory_order_relaxed);
        if (v > 0) n = v;
    }
    return n;
}

#ifndef LLAMA_SK_BALANCE
#define LLAMA_SK_BALANCE 1
#endif

// Weight rows per workgroup when whole strips of 16 RT rows would leave compute units idle
// (fewer strips than units): an equal share of N per unit, rounded up to 8 rows, or 0 when
// the strips fill the device or the share exceeds 16 RT rows.
int balanced_rows(int N, int RT) {
    if (!LLAMA_SK_BALANCE) return 0;
    const int cus = cu_count();
    if (N / (SK_ROWS * RT) >= cus) return 0;
    const int rows = ((N + cus - 1) / cus + 7) / 8 * 8;
    return rows <= SK_ROWS * RT && rows > SK_ROWS * (RT / 2) ? rows : 0;
}

template <bool DUAL, typename Epi>
hipError_t skinny_launch(const GemmArgs<void>& g, const Epi& e, hipStream_t s) {
    if (g.a_pack != act_pack(Dt::BF16, g.M, g.N, g.K)) return hipErrorInvalidValue;
    const int mb = g.a_pack < 16 ? 1 : g.a_pack / 16;  // 16-row MFMA column blocks
    const bool wide = g.N >= 16384;
    if constexpr (DUAL) {
        if (mb == 2 && g.N % (SK_ROWS * 4) == 0) {
            const int bal = balanced_rows(g.N, 4);
            const int rows = bal > 0 ? bal : SK_ROWS * 4;
            gemm_skinny_kernel<4, 4, 2, DUAL, 96, Epi><<<(g.N + rows - 1) / rows, 256, 0, s>>>(
                (const bf16*)g.A, g.a_pack, bf16_rows(g.W), bf16_rows(g.W3), g.M, g.N, g.K, rows, e);
            return hipGetLastError();
        }
        if (mb <= 2 && g.N % (SK_ROWS * 2) == 0) {
            if (mb == 1) return launch_mb<2, 1, DUAL>(g, e, s);
            return launch_mb<2, 2, DUAL>(g, e, s);
        }
        if (mb == 1) return launch_mb<1, 1, DUAL>(g, e, s);
        if (mb == 2) return launch_mb<1, 2, DUAL>(g, e, s);
        return launch_mb<1, 4, DUAL>(g, e, s);
    } else {
        if (mb == 1 && wide && g.N % (SK_ROWS * 4) == 0) return launch_mb<4, 1, DUAL>(g, e, s);
        if (mb == 1) return launch_mb<1, 1, DUAL>(g, e, s);
        if (mb == 2 && wide && g.N % (SK_ROWS * 8) == 0) return launch_mb<8, 2, DUAL>(g, e, s);
        if (mb == 2 && wide && g.N % (SK_ROWS * 4) == 0) return launch_mb<4, 2, DUAL>(g, e, s);
        if (mb == 2 && g.N % (SK_ROWS * 2) == 0) {
            const int bal = balanced_rows(g.N, 2);
            if (bal > 0) {
                gemm_skinny_kernel<8, 2, 2, DUAL, 96, Epi><<<(g.N + bal - 1) / bal, 512, 0, s>>>(
                    (const bf16*)g.A, g.a_pack, bf16_rows(g.W), bf16_rows(g.W3), g.M, g.N, g.K, bal, e);
                return hipGetLastError();
            }
            return launch_mb<2, 2, DUAL>(g, e, s);
        }
        if (mb == 2) return launch_mb<1, 2, DUAL>(g, e, s);
        if (g.N % (SK_ROWS * 2) == 0) return launch_mb<2, 4, DUAL>(g, e, s);
        return launch_mb<1, 4, DUAL>(g, e, s);
    }
}

template hipError_t skinny_launch<false, EpiStoreF32>(const GemmArgs<void>&, const EpiStoreF32&, hipStream_t);
template hipError_t skinny_launch<false, EpiResidual>(const GemmArgs<void>&, const EpiResidual&, hipStream_t);
template hipError_t skinny_launch<true, EpiSwiGLU<bf16>>(const GemmArgs<void>&, const EpiSwiGLU<bf16>&, hipStream_t);
template hipError_t skinny_launch<false, EpiQKV<bf16>>(const GemmArgs<void>&, const EpiQKV<bf16>&, hipStream_t);

}  // namespace lk
