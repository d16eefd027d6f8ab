// bf16 GEMM on the gfx950 matrix cores: acc[m][n] = sum_k A[m][k] W[n][k], fp32 accumulate.
//
// Both operands are K-contiguous ([rows][K] row-major), the layout of the checkpoint's
// [out, in] weights and of the activations.  The weight tile is the MFMA "A" operand (32
// weight rows per instruction) and the token tile the "B" operand (32 tokens), so that each
// lane of the 32x32 result holds four consecutive output columns n of one token row m:
// the RoPE pairs (2i, 2i+1) and the SwiGLU gate/up columns meet in one lane, and the
// epilogue stores 8- or 16-byte vectors.
//
// Block tile BN (weight rows) x BM (tokens) x 64 (k), staged through two LDS buffers, 16-byte
// chunks XOR-swizzled by row so that the 32 lanes of an MFMA operand read hit distinct banks.
// The operand copies pass through registers: a tile is loaded from global memory two tiles
// ahead of the MFMAs and written to LDS one tile ahead.  Requires K % 64 == 0 and N % 4 == 0;
// M and N tails are masked.
#include "launch.hpp"

#include <type_traits>
#include <utility>

namespace lk {

hipError_t simt_store_f32(const GemmArgs<void>& g, EpiStoreF32 e, hipStream_t s);
hipError_t simt_residual(const GemmArgs<void>& g, EpiResidual e, hipStream_t s);
hipError_t simt_swiglu(const GemmArgs<void>& g, void* out, int ld, hipStream_t s);
hipError_t simt_qkv(const GemmArgs<void>& g, const EpiQKV<void>& e, hipStream_t s);

namespace {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Block tile BN weight rows x BM tokens x BK, two LDS buffers; the grid covers weight
// rows [n_begin, N) and all M tokens.  LDS row = BK bf16
// (RB bytes) split in 16-byte chunks; chunk c of row r is stored at c ^ swz(r) so that the
// MFMA operand reads of consecutive rows hit distinct banks.
template <int BN, int BM, int BK, int WN, int WM, bool DUAL, typename Epi>
__global__ __launch_bounds__(WN * WM * 64) void gemm_mfma_kernel(
    const bf16* __restrict__ A, int lda, WeightRows<bf16> W, WeightRows<bf16> W3, int M, int N,
    int K, int n_begin, int group_m, Epi epi) {
    constexpr int NW = WN * WM;
    constexpr int NA = DUAL ? 2 : 1;
    constexpr int ROWS = NA * BN + BM;
    constexpr int RB = BK * 2;                 // bytes per LDS row
    constexpr int CPR = RB / 16;               // 16-byte chunks per row
    constexpr int STAGE = ROWS * RB;           // bytes per stage
    constexpr int SPW = STAGE / 1024 / NW;     // 1 KB copies per wave per stage
    constexpr int TN = BN / WN / 32, TM = BM / WM / 32;
    static_assert(STAGE % (1024 * NW) == 0, "stage must split into whole 1 KB copies per wave");
    extern __shared__ u32x4 lds[];

    // 8 consecutive rows (one 128-byte bank window) and 16 consecutive rows (a 256-byte one)
    // both land on distinct 16-byte slots
    auto swz = [](int r) {
        return CPR == 8 ? (((r >> 1) ^ (r << 2)) & 7) : (((r >> 1) ^ (r >> 3)) & 3);
    };

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wn = wave / WM, wm = wave % WM;
    const int nt_m = (M + BM - 1) / BM, nt_n = (N - n_begin + BN - 1) / BN;
    const int tiles = nt_m * nt_n;
    int bid = blockIdx.x;
    // workgroups are dealt round-robin to the 8 XCDs: give each XCD a contiguous run of
    // tiles, ordered in bands of up to group_m token tiles x all weight strips (token tiles
    // fastest), so that the ~32 tiles an XCD runs at once cover group_m token tiles x
    // 32 / group_m weight strips and share their panels in that XCD's L2
    if (tiles % 8 == 0) bid = (bid & 7) * (tiles >> 3) + (bid >> 3);
    const int per_group = group_m * nt_n;
    const int first_m = (bid / per_group) * group_m;
    const int gsize = min(nt_m - first_m, group_m);
    const int tile_m = first_m + (bid % per_group) % gsize, tile_n = (bid % per_group) / gsize;
    const int n0 = n_begin + tile_n * BN, m0 = tile_m * BM;

    // split z = blockIdx.y of a split-K launch (the fp32 partial-sum epilogue) takes k in
    // [z K, z K + K) of the rows; every other launch has one split, compiled without it
    const int k_off = std::is_same<Epi, EpiPartial>::value ? (int)blockIdx.y * K : 0;
    // this lane's source address for each of its wave's copies of a stage
    const bf16* src[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int byte = (wave + i * NW) * 1024 + lane * 16;
        const int r = byte / RB, pc = (byte % RB) / 16;
        const int c = pc ^ swz(r);
        const bf16* p;
        if (r < BN) {
            p = W.row(n0 + r < N ? n0 + r : 0);
        } else if (DUAL && r < 2 * BN) {
            p = W3.row(n0 + r - BN < N ? n0 + r - BN : 0);
        } else {
            const int m = m0 + r - NA * BN;
            p = A + (size_t)(m < M ? m : 0) * lda;   // rows past M / N load row 0, unused
        }
        src[i] = p + k_off + c * 8;
    }
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
    constexpr int KSTEPS = BK / 16;
    static_assert(KSTEPS % 2 == 0, "the fragment double buffer alternates per k-step");

    // Copies go through registers: tile kt+1, loaded from global memory during tile kt-1,
    // is written into the other LDS buffer over the first KSTEPS-1 k-steps of tile kt, and
    // each write is followed by the load of the same share of tile kt+2 into the registers
    // it frees.  The barrier after k-step KSTEPS-2 publishes tile kt+1 and ends every read
    // of tile kt's buffer (the last k-step's fragments are in registers by then), so the
    // last k-step's MFMAs run while the fragments of tile kt+1's first k-step are read.
    constexpr int WSTEPS = KSTEPS - 1;
    constexpr int WPS = (SPW + WSTEPS - 1) / WSTEPS;  // copies per k-step
    u32x4 stg[SPW];
    char* ldsb = reinterpret_cast<char*>(lds);
    auto gload = [&](int i, int k0) { stg[i] = *reinterpret_cast<const u32x4*>(src[i] + k0); };
    auto lwrite = [&](int st, int i) {
        *reinterpret_cast<u32x4*>(ldsb + st * STAGE + (wave + i * NW) * 1024 + lane * 16) = stg[i];
    };
    bf16x8 fa[2][TN], fa3[2][DUAL ? TN : 1], fb[2][TM];
    auto frags = [&](int buf, const char* base, int kk) {
        const int ch = kk * 2 + lh;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const int r = wn * (BN / WN) + i * 32 + lr;
            fa[buf][i] = *reinterpret_cast<const bf16x8*>(base + r * RB + (ch ^ swz(r)) * 16);
            if constexpr (DUAL)
                fa3[buf][i] = *reinterpret_cast<const bf16x8*>(base + (BN + r) * RB + (ch ^ swz(BN + r)) * 16);
        }
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            const int r = NA * BN + wm * (BM / WM) + j * 32 + lr;
            fb[buf][j] = *reinterpret_cast<const bf16x8*>(base + r * RB + (ch ^ swz(r)) * 16);
        }
    };
#pragma unroll
    for (int i = 0; i < SPW; ++i) gload(i, 0);
#pragma unroll
    for (int i = 0; i < SPW; ++i) lwrite(0, i);
    if (nk > 1) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) gload(i, BK);
    }
    wait_lgkm_and_barrier();
    frags(0, ldsb, 0);
    // WR: a tile kt+1 exists (write it, read its first fragments); LD: a tile kt+2 exists
    auto tile = [&](int kt, auto wr_c, auto ld_c) {
        constexpr bool WR = decltype(wr_c)::value, LD = decltype(ld_c)::value;
        const char* base = ldsb + (kt & 1) * STAGE;
        const char* nbase = ldsb + ((kt + 1) & 1) * STAGE;
        const int wst = (kt + 1) & 1, k2 = (kt + 2) * BK;
        static_for<KSTEPS>([&](auto kk_c) {
            constexpr int kk = decltype(kk_c)::value;
            constexpr int cur = kk & 1;
            if constexpr (kk + 1 < KSTEPS) frags(cur ^ 1, base, kk + 1);
            else if constexpr (WR) frags(cur ^ 1, nbase, 0);
#pragma unroll
            for (int i = 0; i < TN; ++i)
#pragma unroll
                for (int j = 0; j < TM; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
                    if constexpr (DUAL)
                        acc3[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa3[cur][i], fb[cur][j], acc3[i][j], 0, 0, 0);
                }
            // one scheduling region per k-step: an LDS read after each of the first MFMAs,
            // then one LDS write and one global load after each of the next ones
            constexpr int NREAD = NA * TN + TM, NMFMA = NA * TN * TM;
            constexpr int NWR = (WR && kk < WSTEPS) ? ((kk + 1) * WPS <= SPW ? WPS : SPW - kk * WPS) : 0;
            constexpr int NRD = (kk + 1 < KSTEPS || WR) ? NREAD : 0;
            if constexpr (NRD + NWR <= NMFMA) {
#pragma unroll
                for (int q = 0; q < NRD; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                }
#pragma unroll
                for (int q = 0; q < NWR; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
                    if constexpr (LD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - NRD - NWR, 0);
            } else {
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (WR) {
                if (kk < WSTEPS) {
#pragma unroll
                    for (int q = 0; q < WPS; ++q) {
                        const int i = kk * WPS + q;
                        if (i < SPW) {
                            lwrite(wst, i);
                            if constexpr (LD) gload(i, k2);
                        }
                    }
                }
            }
            if constexpr (kk == KSTEPS - 2) wait_lgkm_and_barrier();
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    int kt = 0;
    for (; kt + 2 < nk; ++kt) tile(kt, std::true_type{}, std::true_type{});
    if (kt + 1 < nk) {
        tile(kt, std::true_type{}, std::false_type{});
        ++kt;
    }
    tile(kt, std::false_type{}, std::false_type{});

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
            // one 32x32 tile at a time: keeps the epilogue's loads from raising the kernel's
            // register count (and so its occupancy)
            __builtin_amdgcn_sched_barrier(0);
        }
}

template <int BN, int BM, int BK, int WN, int WM, bool DUAL, typename Epi>
hipError_t launch_cfg(const GemmArgs<void>& g, const Epi& e, hipStream_t s, int n_begin = 0,
                      int splits = 1) {
    const WeightRows<bf16> W{(const bf16*)g.W.p0, (const bf16*)g.W.p1, (const bf16*)g.W.p2, g.W.end0, g.W.end1, g.W.ld};
    const WeightRows<bf16> W3{(const bf16*)g.W3.p0, (const bf16*)g.W3.p1, (const bf16*)g.W3.p2, g.W3.end0, g.W3.end1, g.W3.ld};
    constexpr int ROWS = (DUAL ? 2 : 1) * BN + BM;
    constexpr size_t lds_bytes = (size_t)2 * ROWS * BK * 2;
    static_assert(lds_bytes <= 160 * 1024, "LDS");
    auto kern = gemm_mfma_kernel<BN, BM, BK, WN, WM, DUAL, Epi>;
    static PerDevice attr;
    hipError_t err = attr.once([&](int) {
        return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
    });
    if (err != hipSuccess) return err;
    const int nt_m = (g.M + BM - 1) / BM;
    const int tiles = ((g.N - n_begin + BN - 1) / BN) * nt_m;
    // Token tiles per band of the tile order, measured on MI355X (8B-shaped layer): the
    // SwiGLU pair runs fastest with bands of 2 token tiles at 2048 tokens (446 -> 430 us
    // against 8) and of 4 beyond (8192 tokens 1656 -> 1562 us, 32768 tokens 6702 -> 6407
    // us); the other GEMMs with bands of 8, except a long K at many token tiles (W2 at
    // 32768 tokens 3145 -> 3078 us with 2).
    int group_m = 8;
    if (DUAL) group_m = nt_m <= 8 ? 2 : 4;
    else if (g.K >= 8192 && nt_m > 8) group_m = 2;
    kern<<<dim3(tiles, splits), WN * WM * 64, lds_bytes, s>>>((const bf16*)g.A, g.lda, W, W3, g.M,
                                                              g.N, g.K / splits, n_begin, group_m, e);
    return hipGetLastError();
}

// Tile shapes per GEMM shape, measured on MI355X (8B-shaped layer at 2048 tokens):
//  - wide weight matrices (Q/K/V, the vocabulary) and every GEMM with many token tiles:
//    256 tokens x 256 or 192 weight rows, 8 waves.  192 rows is taken when it covers the
//    256 CUs in fewer rounds of tiles for the same work (Q/K/V at 2048 tokens: 256 tiles
//    instead of 192, 117 us instead of 150);
//  - the SwiGLU gate/up pair: 128 rows of W1 + 128 of W3 against 256 tokens, 4 waves of
//    64 + 64 rows x 128 tokens (a third fewer LDS fragment reads than 8 waves).  When
//    the tiles fill the CUs a few times over plus a final round less than half full (2048
//    tokens: 896 tiles = 3.5 rounds), the weight rows of that last round go to a second
//    launch of half-height tiles (128 tokens) that fills one round: the last round then
//    takes about half a tile's time instead of a whole one;
//  - N = dim outputs (WO, W2) at a few thousand tokens: 256 weight rows x 128 tokens, 8 waves
//    (4 x 2) of 64 x 64 (256 tiles at 2048 tokens; the per-tile operand traffic of 128 x 128
//    tiles left those GEMMs bound by the operand copies).  Two waves per SIMD against one
//    for 4 waves of 128 x 64: WO 82 -> 78 us and W2 245 -> 237 us at 2048 tokens; 2 x 4
//    waves gained half as much.
template <bool DUAL, typename Epi>
hipError_t launch(const GemmArgs<void>& g, const Epi& e, hipStream_t s) {
    if (g.M == 0) return hipSuccess;
    if (g.a_pack > 0) return skinny_launch<DUAL>(g, e, s);
    if (g.M <= 32) return launch_cfg<128, 32, 64, 4, 1, DUAL>(g, e, s);
    if constexpr (DUAL) {
        const int strips = (g.N + 127) / 128, mt = (g.M + 255) / 256;
        const long long tiles = (long long)strips * mt, rest = tiles % 256;
        if (tiles > 256 && tiles <= 8 * 256 && rest > 0 && rest <= 128 && rest % mt == 0) {
            const int n_tail = (int)(strips - rest / mt) * 128;  // rows of the last round
            GemmArgs<void> head = g;
            head.N = n_tail;
            hipError_t err = launch_cfg<128, 256, 64, 2, 2, DUAL>(head, e, s);
            if (err != hipSuccess) return err;
            return launch_cfg<128, 128, 64, 2, 2, DUAL>(g, e, s, n_tail);
        }
        return launch_cfg<128, 256, 64, 2, 2, DUAL>(g, e, s);
    } else {
        const long long mt = (g.M + 255) / 256;
        const long long t256 = (long long)((g.N + 255) / 256) * mt;
        if (g.N >= 6144 || t256 >= 512) {
            // rounds of 256 tiles x rows per tile: the smaller wins, ties go to 256 rows
            const long long t192 = (long long)((g.N + 191) / 192) * mt;
            if (((t192 + 255) / 256) * 192 < ((t256 + 255) / 256) * 256)
                return launch_cfg<192, 256, 64, 2, 4, DUAL>(g, e, s);
            return launch_cfg<256, 256, 64, 2, 4, DUAL>(g, e, s);
        }
        return launch_cfg<256, 128, 64, 4, 2, DUAL>(g, e, s);
    }
}

}  // namespace

// Split-K form of a residual GEMM with many token rows (the down projection of a prefill of
// up to a few thousand tokens): 256 x 256 tiles, each of the `splits` k ranges in its own
// workgroup, writing fp32 sums to part (EpiPartial); the next RMSNorm of the residual stream
// adds them.  Used where the unsplit 256 x 256 grid would fill at most half the CUs, so that
// the split grid fills them once: there the alternative is 256 x 128 tiles, whose operand
// copies per FLOP are a third higher.
int tiled_residual_splits(Dt dt, int M, int N, int K) {
    if (dt != Dt::BF16 || M <= 64 || M > LLAMA_TILED_SPLIT_MAX_ROWS || N % 256 != 0 ||
        K < 8192 || K % 128 != 0)
        return 0;
    const long long tiles = (long long)((M + 255) / 256) * (N / 256);
    return 2 * tiles <= cu_count() ? 2 : 0;
}

hipError_t gemm_residual_split_tiled(const GemmArgs<void>& g, float* part, int splits,
                                     hipStream_t s) {
    if (splits != tiled_residual_splits(Dt::BF16, g.M, g.N, g.K) || g.a_pack != 0)
        return hipErrorInvalidValue;
    return launch_cfg<256, 256, 64, 2, 4, false>(g, EpiPartial{part, g.N, (size_t)g.M * g.N}, s,
                                                 0, splits);
}

hipError_t gemm_store_f32(Dt dt, const GemmArgs<void>& g, EpiStoreF32 e, hipStream_t s) {
    if (dt == Dt::F32) return simt_store_f32(g, e, s);
    return launch<false>(g, e, s);
}
hipError_t gemm_residual(Dt dt, const GemmArgs<void>& g, EpiResidual e, hipStream_t s) {
    if (dt == Dt::F32) return simt_residual(g, e, s);
    return launch<false>(g, e, s);
}
hipError_t gemm_swiglu(Dt dt, const GemmArgs<void>& g, void* out, int ld, int out_pack,
                       hipStream_t s) {
    if (dt == Dt::F32) return simt_swiglu(g, out, ld, s);
    return launch<true>(g, EpiSwiGLU<bf16>{(bf16*)out, ld, out_pack}, s);
}
hipError_t gemm_qkv(Dt dt, const GemmArgs<void>& g, const EpiQKV<void>& e, hipStream_t s) {
    if (dt == Dt::F32) return simt_qkv(g, e, s);
    EpiQKV<bf16> eb{(bf16*)e.q, (bf16*)e.kc, (bf16*)e.vc, e.rope, e.Nq, e.Nk, e.d, e.S,
                    e.start_pos, e.G, e.seq_stride, e.pos_dev, e.pos_stride, e.max_pos, e.packed};
    return launch<false>(g, eb, s);
}

}  // namespace lk
