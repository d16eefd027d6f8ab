// Causal grouped-query attention over the KV cache (article, sections 查询和键相乘, 掩码,
// 注意力向量, 多头注意力): for query head h of the token at position p,
//   o = sum_{n <= p} softmax_n(q . k_n / sqrt(d)) v_n,  k and v of KV head h / (H/G).
// Cache layout: K [b][g][pos][d] (seq_stride positions per (b, g)); V transposed in
// blocks of 64 positions, [b][g][pos/64][d][64] (vt_offset in epilogue.hpp).
#include "launch.hpp"

#include <type_traits>

namespace lk {

namespace {

// Generic path (any even d <= 256, fp32 or bf16): one wave per (query row, head), keys in
// chunks of 64 (one per lane) with an online softmax; lane owns output dims lane + 64 i.
template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ kc,
                                                           const T* __restrict__ vc,
                                                           T* __restrict__ out, int S,
                                                           int start_pos, const int* pos_dev,
                                                           int pos_stride, int max_pos,
                                                           int H, int G, int d, int seq_stride,
                                                           float scale_log2, int out_pack) {
    const int row = blockIdx.x;  // b * S + s
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int b = row / S, s = row - b * S;
    const int qpos = max(seq_pos(pos_dev, pos_stride, b, start_pos, max_pos), 0) + s;
    const int g = h / (H / G);
    __shared__ float qs[256];
    const T* qr = q + (size_t)row * H * d + (size_t)h * d;
    for (int i = lane; i < d; i += 64) qs[i] = to_f32(qr[i]);
    __syncthreads();

    const T* kb = kc + ((size_t)b * G + g) * seq_stride * d;
    const T* vb = vc + ((size_t)b * G + g) * d * seq_stride;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;
    const int nkeys = qpos + 1;
    for (int c0 = 0; c0 < nkeys; c0 += 64) {
        const int j = c0 + lane;
        float sc = -INFINITY;
        if (j < nkeys) {
            const T* kr = kb + (size_t)j * d;
            float acc = 0.f;
            for (int i = 0; i < d; ++i) acc = fmaf(qs[i], to_f32(kr[i]), acc);
            sc = acc * scale_log2;  // score in log2 units
        }
        const float cmax = wave_max(sc);
        const float mnew = fmaxf(mrun, cmax);
        const float corr = exp2f(mrun - mnew);  // 0 on the first chunk (mrun = -inf)
        const float p = (j < nkeys) ? exp2f(sc - mnew) : 0.f;
        lrun = lrun * corr + wave_sum(p);
        mrun = mnew;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= corr;
        const int cn = min(64, nkeys - c0);
        for (int jj = 0; jj < cn; ++jj) {
            const float pj = __shfl(p, jj, 64);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dd = lane + 64 * i;
                if (dd < d)
                    o[i] = fmaf(pj, to_f32(vb[((size_t)((c0 + jj) / VT_BLOCK) * d + dd) * VT_BLOCK +
                                                 (c0 + jj) % VT_BLOCK]), o[i]);
            }
        }
    }
    const float inv = 1.0f / lrun;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dd = lane + 64 * i;
        if (dd < d) out[act_offset(row, h * d + dd, H * d, out_pack)] = from_f32<T>(o[i] * inv);
    }
}

template <typename T>
hipError_t launch_generic(const AttnArgs& a, hipStream_t s) {
    const int rows = a.B * a.S;
    if (rows == 0) return hipSuccess;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)a.d);
    dim3 grid(rows, a.H);
    attn_generic_kernel<T><<<grid, 64, 0, s>>>((const T*)a.q, (const T*)a.kc, (const T*)a.vc,
                                               (T*)a.out, a.S, a.start_pos, a.pos_dev,
                                               a.pos_stride, a.max_pos, a.H, a.G,
                                               a.d, a.seq_stride, scale_log2, a.out_pack);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Prefill, bf16, head_dim 128: flash-style attention on the matrix cores.
//
// One workgroup (4 waves) takes one (sequence b, KV head g) and a block of BQ = 128/group
// positions for all `group` = H/G query heads that read KV head g, i.e. 128 query rows
// sharing every K/V tile it stages.  Wave w owns query rows 32w..32w+31 (row r: head
// g*group + r / BQ, position r % BQ).  Keys go through LDS in blocks of 64 (double
// buffered); each block does
//   S^T = K Q^T      (MFMA A = K rows, B = the wave's Q held in registers)
//   online softmax   (each lane owns one query column: max/sum over its 32 values and the
//                     partner lane l^32; rescaling O needs no data exchange)
//   O^T += V^T P^T   (A = V^T from the transposed cache, B = P^T straight from registers,
//                     P rounded to bf16 as the article casts the softmax output)
// Keys beyond the block's last position are never read; keys after a row's own position
// get a score of -inf (article, section 多头注意力: the upper-triangular -inf mask).
// ------------------------------------------------------------------------------------
constexpr int FA_D = 128, FA_BKV = 64, FA_ROWS = 128;
static_assert(FA_BKV == VT_BLOCK, "a key block is one V^T block");
constexpr int FA_KBYTES = FA_BKV * FA_D * 2;   // K tile: 64 keys x 256 B
constexpr int FA_STAGE_BYTES = 2 * FA_KBYTES;  // + V^T tile: 128 d x 128 B

__device__ __forceinline__ u32x4 mask_keys8(u32x4 v, int first_key, int limit) {
    // zero the bf16 elements whose key index (first_key + e) is >= limit
    if (first_key + 8 <= limit) return v;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int k0 = first_key + 2 * w;
        uint32_t x = v[w];
        if (k0 >= limit) x &= 0xFFFF0000u;
        if (k0 + 1 >= limit) x &= 0x0000FFFFu;
        v[w] = x;
    }
    return v;
}

// One 32-row query tile of a wave: Q fragments (B operand of S^T = K Q^T, lane lr holds
// query row lr, d = 8 (2 kk + lh) ..), the O^T accumulator and the online-softmax state of
// the lane's query column.
struct FaTile {
    bf16x8 qf[8];
    f32x16 o[4];
    float m, l;
    int hq, sq, qpos, p_lo, nkb;
    bool valid;
};

// Rows of a workgroup's 128-row query tile: row r is query head g*group + r/BQ at position
// blk*BQ + r%BQ of the call.  In LDS a tile row (128 d, 256 B) keeps its 16-byte chunk c
// at slot c ^ (r & 15), as the K tile does.
__device__ __forceinline__ void fa_tile_init(FaTile& T, int blk, int r, int g, int S,
                                             int start_pos, int group, int BQ) {
    T.hq = g * group + r / BQ;
    T.sq = blk * BQ + r % BQ;
    T.valid = T.sq < S;
    T.qpos = start_pos + T.sq;
    T.p_lo = start_pos + blk * BQ;
    const int p_hi = start_pos + min(S, blk * BQ + BQ) - 1;
    T.nkb = (p_hi + 1 + FA_BKV - 1) / FA_BKV;   // keys this tile's block needs: 0..p_hi
#pragma unroll
    for (int i = 0; i < 4; ++i) T.o[i] = f32x16{};
    T.m = -INFINITY;
    T.l = 0.0f;
}

// Causal mask and online softmax of one key block's raw scores (two 32-key tiles; with the
// key order of the S^T tiles, register e of tile i is key kv0 + 32i + 16(e/8) + 8lh + e%8);
// returns P^T as the four k-step operands of O^T += V^T P^T: k-step j takes registers
// 8(j%2)..+7 of tile j/2, the keys 32(j/2) + 16(j%2) + 8lh + 0..7.
// Maxima are in log2 units and the score scale is folded into the exponent.  The
// exponentials are taken against a reference maximum T.m that is raised only when some row
// of the wave sees a block maximum more than 8 above its reference: then every row rescales
// O and l to its new maximum (a wave-uniform branch; O lives in accumulation registers and a
// rescale costs three instructions per element).  Otherwise p <= 2^8, well inside bf16 and
// fp32 range.  O and l share the reference, so O / l is the softmax-weighted sum.
// EMPTY_ROWS: the block may hold rows that have seen no unmasked key yet, in this block or
// before it (a workgroup's second set of key blocks, which does not start at key 0).
constexpr float FA_RESCALE_SLACK = 8.0f;
template <bool EMPTY_ROWS>
__device__ __forceinline__ void fa_softmax(FaTile& T, f32x16 (&sacc)[2], bf16x8 (&pf)[4], int kv0,
                                           int lh, float scale_log2) {
    if (kv0 + FA_BKV - 1 > T.p_lo) {  // the block reaches past some row's own position
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = kv0 + 32 * i + 16 * (e >> 3) + 8 * lh + (e & 7);
                if (key > T.qpos) sacc[i][e] = -INFINITY;
            }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[i][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > T.m + FA_RESCALE_SLACK) != 0) {
        const float m_new = fmaxf(T.m, mx);
        // 0 while T.m = -inf (O = 0, l = 0): with EMPTY_ROWS also where the row's new
        // maximum is still -inf
        const float corr = EMPTY_ROWS && T.m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(T.m - m_new);
        T.l *= corr;
        // in groups of 8, so that few registers hold values on their way back
#pragma unroll
        for (int td = 0; td < 4; ++td)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int e = 0; e < 8; ++e) T.o[td][8 * h + e] *= corr;
                __builtin_amdgcn_sched_barrier(0);
            }
        T.m = m_new;
    }
    // With EMPTY_ROWS a row whose keys so far were all masked still has T.m = -inf; its
    // exponentials are then taken against 0, so that masked keys give 0 rather than
    // 2^(-inf + inf).
    const float msub = EMPTY_ROWS && T.m == -INFINITY ? 0.0f : T.m;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[i][e], scale_log2, -msub));
            psum += p;
            sacc[i][e] = p;
        }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int s = 0; s < 8; ++s) pf[j][s] = from_f32<bf16>(sacc[j >> 1][8 * (j & 1) + s]);
    T.l += psum + __shfl_xor(psum, 32, 64);
}

// Workgroup = (sequence b, KV head g, query block qb): BQ = 128/group positions for the
// group's query heads, 128 query rows; wave w of a 4-wave set owns rows 32w..32w+31 as one
// query tile.
//
// NH = 1: one 4-wave set takes every key block; two workgroups share a CU (64 KB of LDS
// each), so each SIMD runs two waves and one wave's softmax overlaps the other's MFMAs.
// Grid order (pair_order): for a grid of about one round the first half of the workgroups
// take the late (long) query blocks, latest first, the second half the matching early
// ones, so that the two workgroups of a CU cover about the same number of key blocks; for
// larger grids the latest (longest) query block comes first throughout, so that the last
// workgroups to start are the shortest (4 x 8192 tokens: 2161-2170 -> 2116-2135 us on
// MI355X, results unchanged).
//
// NH = 2: two 4-wave sets over the same 128 query rows, set h taking key blocks h, h + 2,
// h + 4, ..; each set has its own double buffer (128 KB, one workgroup per CU), and set 1
// hands its softmax state (max, sum, unnormalised O) to set 0 through LDS at the end, where
// the two partial softmaxes merge exactly as the online softmax merges two key blocks.
// Wave w of each set runs on SIMD w, so every SIMD again holds two waves with the same
// work.  The grid runs latest query block first: a CU that finishes a short block takes
// the next longest one, so every CU ends up with about the same number of key blocks.
// The launcher takes it for grids of at most about two rounds of workgroups whose query
// blocks differ widely in length (a call from near position 0, e.g. 2048 tokens), where
// with NH = 1 the CU that holds the longest query block runs it alone at one wave per SIMD
// once its short partner has finished.
template <int NH>
__global__ __launch_bounds__(256 * NH, 2 / NH) void attn_prefill_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    bf16* __restrict__ out, int S, int start_pos, int H, int G, int seq_stride,
    float scale_log2, int nqb, int out_pack, int pair_order) {
    static_assert(NH == 1 || NH == 2, "one or two key-block sets");
    extern __shared__ u32x4 fa_smem[];
    const int group = H / G, BQ = FA_ROWS / group;
    const int GB = G * (gridDim.x / (nqb * G));  // (b, g) pairs
    const int idx = (int)blockIdx.x;
    int qb;
    if (NH == 1 && pair_order) {
        const int heavy = (nqb + 1) / 2;         // blocks nqb-1 .. nqb-heavy come first
        qb = idx < heavy * GB ? nqb - 1 - idx / GB : (idx - heavy * GB) / GB;
    } else {
        qb = nqb - 1 - idx / GB;
    }
    const int gb = idx % GB;
    const int b = gb / G, g = gb % G;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, lr = lane & 31, lh = lane >> 5;
    const int wq = wave & 3;                     // the wave's query tile within its set

    FaTile T;
    fa_tile_init(T, qb, wq * 32 + lr, g, S, start_pos, group, BQ);
    const int nkb = T.nkb;

    const bf16* kbase = kc + ((size_t)b * G + g) * seq_stride * FA_D;
    const bf16* vbase = vc + ((size_t)b * G + g) * FA_D * seq_stride;

    // Stage layout (LDS): K tile [64 keys][16 chunks of 16 B], chunk c of key row kr at slot
    // c ^ (kr & 15); V^T tile [128 d][8 chunks of 16 B], chunk c of row d at slot
    // c ^ ((d >> 1) & 7).  Both arrive by direct global -> LDS copies, 1 KB (4 key rows /
    // 8 d rows) per copy, each lane fetching its 16-byte piece from the packed cache layout
    // (kc_packed_offset, vc_packed_offset); both operand reads below are conflict-free
    // 16-byte reads.  Keys past the sequence's context are read too (whole 64-position
    // blocks inside the cache); the causal mask gives them probability 0 and the cache holds
    // finite values.  Set h of the workgroup owns the two stage buffers at 2 h STAGE.
    //
    // Addressing is kept off the vector ALU: copy i of a wave moves key rows kr = 16 i + 4 wv
    // + lane / 16 and d rows 32 i + 8 wv + lane / 8, whose swizzles do not depend on i.  In
    // the packed layout key row kr, chunk c sits in run (2 (i / 2) + wv % 2) * 4 + c / 4 at
    // 16-byte position 16 (2 (i % 2) + wv / 2) + 4 (c % 4) + lane / 16; d row dr, chunk c in
    // run (2 i + wv / 2) * 2 + c / 4 at position 8 (wv % 2) + lane / 8 + 16 (c % 4).  So one
    // per-lane byte offset serves all four copies of each tile, the block and copy parts of
    // the address (8192 (i / 2) + 512 (i % 2) bytes for K, 4096 i for V) are scalar, and each
    // copy reads 8 whole 128-byte lines.
    const int wv = __builtin_amdgcn_readfirstlane(wq);      // the wave index in its set, scalar
    const int set = NH == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave >> 2);
    const unsigned lds0 = lds_addr(fa_smem);
    const unsigned set0 = lds0 + set * 2 * FA_STAGE_BYTES;
    const int kc_ = (lane & 15) ^ ((4 * wv + (lane >> 4)) & 15);
    const unsigned koff = (unsigned)(((wv & 1) * 4 + (kc_ >> 2)) * 1024 +
                                     (16 * (wv >> 1) + 4 * (kc_ & 3) + (lane >> 4)) * 16);
    const int vc_ = (lane & 7) ^ ((4 * wv + (lane >> 4)) & 7);
    const unsigned voff = (unsigned)(2 * (((wv >> 1) * 2 + (vc_ >> 2)) * 512 +
                                          (8 * (wv & 1) + (lane >> 3) + 16 * (vc_ & 3)) * 8));
    auto issue = [&](int st, int kb) {
        const char* ksrc = reinterpret_cast<const char*>(kbase + (size_t)kb * FA_BKV * FA_D);
        const char* vsrc = reinterpret_cast<const char*>(vbase + (size_t)kb * FA_D * VT_BLOCK);
        const unsigned dst = set0 + st * FA_STAGE_BYTES + wv * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lds_dma16_s(ksrc + (i >> 1) * 8192 + (i & 1) * 512, koff, dst + i * 4096);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_dma16_s(vsrc + i * 4096, voff, dst + FA_KBYTES + i * 4096);
    };

    // The query tile arrives through set 0's second stage buffer by the same direct copies
    // (each 1 KB copy = 4 whole rows, so every global read is a full 256-byte row segment;
    // rows past the call's tokens read its last token and are never stored), while each
    // set's first key block lands in its first buffer.
    if (set < nkb) issue(0, set);
    {
        const unsigned qdst = lds0 + FA_STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < 8 / NH; ++i) {
            const int ci = wave + 4 * NH * i;
            const int qr = 4 * ci + (lane >> 4), slot = lane & 15;
            const int sq = min(qb * BQ + qr % BQ, S - 1);
            const bf16* qsrc = q + ((size_t)(b * S + sq) * H + g * group + qr / BQ) * FA_D;
            lds_dma16(qsrc + ((slot ^ (qr & 15)) * 8), qdst + ci * 1024);
        }
        wait_copies_and_barrier();
        const int r = wq * 32 + lr;
        const u32x4* qs = fa_smem + FA_STAGE_BYTES / 16;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            T.qf[kk] = __builtin_bit_cast(bf16x8, qs[r * 16 + ((kk * 2 + lh) ^ (r & 15))]);
        // every wave's reads of the query tile end before the loop copies a key block there
        wait_lgkm_and_barrier();
    }

    // Operand reads.  S^T = K Q^T runs on two 32-key tiles; MFMA row r of tile i is key
    // 32i + pi(r), pi(r) = 16(r/16) + 8((r/4)%2) + 4((r/8)%2) + r%4, so that each lane's
    // eight P values of one P.V k-step are eight consecutive keys.  K k-step kk reads chunk
    // 2 kk + lh of its key row, at byte (32i + krow) 256 + ((2kk ^ lh ^ (krow & 15)) 16) =
    // (ka ^ 32kk) + 8192 i; V^T k-step j of d tile td reads chunk 2j + lh of row d = 32 td
    // + lr, at (va ^ 32j) + 4096 td.  The stage offset is a compile-time constant of each
    // of the loop's two unrolled halves, so every read is one XOR and an immediate offset.
    const int krow = 16 * (lr >> 4) + 8 * ((lr >> 2) & 1) + 4 * ((lr >> 3) & 1) + (lr & 3);
    // (the set's buffer offset, a multiple of 64 KB, is part of the per-lane address and
    // leaves the XOR bits alone)
    const unsigned ka = (unsigned)(krow * 256 + ((lh ^ (krow & 15)) * 16) + set * 2 * FA_STAGE_BYTES);
    const unsigned va = (unsigned)(lr * 128 + ((lh ^ ((lr >> 1) & 7)) * 16) + set * 2 * FA_STAGE_BYTES);
    const char* lds_c = reinterpret_cast<const char*>(fa_smem);
    // Step j of the loop: the set's key block kb = NH j + set.  Both sets pass the same
    // number of barriers; set 1 skips the work of a step past the last block (odd nkb).
    auto block = [&](int j, auto st_c) {
        constexpr int st = decltype(st_c)::value;
        const int kb = NH * j + set;
        // block kb has landed, and every wave's reads of the other slot have returned
        wait_copies_and_barrier();
        if (kb + NH < nkb) issue(st ^ 1, kb + NH);
        if (kb >= nkb) return;
        const int kv0 = kb * FA_BKV;
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            bf16x8 kf[2][2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int kk = 2 * h + k2;
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    kf[k2][i] = *reinterpret_cast<const bf16x8*>(
                        lds_c + ((ka ^ (32u * kk)) + 8192 * i + st * FA_STAGE_BYTES));
            }
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k2][i], T.qf[2 * h + k2], sacc[i], 0, 0, 0);
        }
        bf16x8 pf[4];
        fa_softmax<NH == 2>(T, sacc, pf, kv0, lh, scale_log2);
        // O^T += V^T P^T: the V^T operand of k-step j for lane lh is keys 16j + 8lh .. +7 of
        // row d, the 16-byte chunk 2j + lh
#pragma unroll
        for (int td = 0; td < 4; ++td) {
            bf16x8 vf[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                vf[j] = *reinterpret_cast<const bf16x8*>(
                    lds_c + ((va ^ (32u * j)) + 4096 * td + FA_KBYTES + st * FA_STAGE_BYTES));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                T.o[td] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[j], pf[j], T.o[td], 0, 0, 0);
        }
    };
    const int nsteps = (nkb + NH - 1) / NH;
    int j = 0;
    for (; j + 1 < nsteps; j += 2) {
        block(j, std::integral_constant<int, 0>{});
        block(j + 1, std::integral_constant<int, 1>{});
    }
    if (j < nsteps) block(j, std::integral_constant<int, 0>{});

    // every wave is past its last key block and its LDS reads have returned
    wait_lgkm_and_barrier();
    if constexpr (NH == 2) {
        // Set 1's state leaves through LDS in lane order (each store one contiguous 1 KB):
        // O^T tile td, registers 4c..4c+3 at ((wq 4 + td) 4 + c) KB + 16 lane, then (m, l)
        // at 64 KB + 512 wq + 8 lane.  Set 0 merges it into its own:
        //   m = max(m0, m1), O = O0 2^(m0 - m) + O1 2^(m1 - m), l likewise,
        // with set 1's state empty (m = -inf, l = 0, O = 0) when it saw no key block.
        char* sb = reinterpret_cast<char*>(fa_smem);
        if (set == 1) {
#pragma unroll
            for (int td = 0; td < 4; ++td)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<f32x4*>(sb + ((wq * 4 + td) * 4 + c) * 1024 + lane * 16) =
                        f32x4{T.o[td][4 * c], T.o[td][4 * c + 1], T.o[td][4 * c + 2], T.o[td][4 * c + 3]};
            *reinterpret_cast<float2*>(sb + 65536 + wq * 512 + lane * 8) = float2{T.m, T.l};
        }
        wait_lgkm_and_barrier();
        if (set == 0) {
            const float2 ml = *reinterpret_cast<const float2*>(sb + 65536 + wq * 512 + lane * 8);
            const float m_new = fmaxf(T.m, ml.x);
            const float c0 = __builtin_amdgcn_exp2f(T.m - m_new);
            const float c1 = __builtin_amdgcn_exp2f(ml.x - m_new);
            T.l = T.l * c0 + ml.y * c1;
#pragma unroll
            for (int td = 0; td < 4; ++td)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const f32x4 o1 = *reinterpret_cast<const f32x4*>(sb + ((wq * 4 + td) * 4 + c) * 1024 + lane * 16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) T.o[td][4 * c + e] = T.o[td][4 * c + e] * c0 + o1[e] * c1;
                }
        }
    }

    // The normalised output goes through LDS (the first stage buffer, free once every wave
    // is past its last key block; with two sets the last 32 KB, clear of set 1's state) and
    // leaves as whole 16-byte chunks of each row: lane (lr, lh) holds d = 32 td + 8 gg + 4 lh
    // .. +3 of its row, half of chunk 4 td + gg.
    constexpr int OUT0 = NH == 2 ? 3 * FA_STAGE_BYTES : 0;
    if (set == 0) {
        const float inv = 1.0f / T.l;
        const int r = wq * 32 + lr;
        char* ob = reinterpret_cast<char*>(fa_smem) + OUT0;
#pragma unroll
        for (int td = 0; td < 4; ++td)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int c = 4 * td + gg;
                *reinterpret_cast<bf16x4*>(ob + r * 256 + ((c ^ (r & 15)) * 16) + lh * 8) =
                    bf16x4{from_f32<bf16>(T.o[td][4 * gg] * inv), from_f32<bf16>(T.o[td][4 * gg + 1] * inv),
                           from_f32<bf16>(T.o[td][4 * gg + 2] * inv), from_f32<bf16>(T.o[td][4 * gg + 3] * inv)};
            }
    }
    wait_lgkm_and_barrier();
    const u32x4* os = fa_smem + OUT0 / 16;
#pragma unroll
    for (int i = 0; i < 8 / NH; ++i) {
        const int ch = i * 256 * NH + t, r = ch >> 4, c = ch & 15;
        const int sq = qb * BQ + r % BQ;
        if (sq < S) {
            const u32x4 v = os[r * 16 + (c ^ (r & 15))];
            *reinterpret_cast<u32x4*>(out + act_offset(b * S + sq, (g * group + r / BQ) * FA_D + c * 8,
                                                       H * FA_D, out_pack)) = v;
        }
    }
}

template <int NH>
hipError_t launch_prefill_nh(const AttnArgs& a, int nqb, float scale_log2, hipStream_t s) {
    static PerDevice attr;
    hipError_t e = attr.once([](int) {
        return hipFuncSetAttribute((const void*)attn_prefill_mfma_kernel<NH>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)(2 * NH * FA_STAGE_BYTES));
    });
    if (e != hipSuccess) return e;
    const long wgs = (long)nqb * a.G * a.B;
    const int pair_order = wgs <= 4L * cu_count() ? 1 : 0;   // up to two workgroups per CU
    attn_prefill_mfma_kernel<NH><<<wgs, 256 * NH, 2 * NH * FA_STAGE_BYTES, s>>>(
        (const bf16*)a.q, (const bf16*)a.kc, (const bf16*)a.vc, (bf16*)a.out, a.S, a.start_pos,
        a.H, a.G, a.seq_stride, scale_log2, nqb, a.out_pack, pair_order);
    return hipGetLastError();
}

hipError_t launch_prefill_mfma(const AttnArgs& a, hipStream_t s) {
    const int group = a.H / a.G, BQ = FA_ROWS / group;
    const int nqb = (a.S + BQ - 1) / BQ;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)FA_D);
    // Two key-block sets per workgroup while the grid is at most about two rounds of one
    // workgroup per CU and the query blocks' key counts differ widely (the call starts
    // within one chunk of position 0, so that its last block reads at least twice the keys
    // of its first).  A chunk far into a sequence (start_pos >= S) has blocks of nearly
    // equal length, which two 4-wave workgroups per CU run better (measured on MI355X,
    // 2048 tokens after a 2048-token prefix).
    if ((long)nqb * a.G * a.B <= 2L * cu_count() && a.S >= a.start_pos + 2 * BQ)
        return launch_prefill_nh<2>(a, nqb, scale_log2, s);
    return launch_prefill_nh<1>(a, nqb, scale_log2, s);
}

// ------------------------------------------------------------------------------------
// Decode, bf16, head_dim 128: split-K over the cached context on the matrix cores.
//
// Workgroup = (split of the context, KV head g, sequence b), NWV waves.  Each iteration the
// waves take consecutive 64-key blocks and stream their K (16 KB) and V^T (16 KB) straight
// from HBM into 16x16x32 MFMA operands, with the `group` query heads of g as the B-operand
// columns (the rest zero): S^T = K Q^T, an online softmax per head, O^T += V^T P^T.  The
// waves' states are merged through LDS.  With one split (enough (b, g) pairs to fill the
// chip) the workgroup writes the attention output itself; otherwise it writes one partial
// (max, sum, unnormalised o[128]) per query head and a second kernel merges the splits.
//
// Index maps (all 16-byte loads): lane (c = l%16, kq = l/16).  K tile t = 2j + h of a
// 64-key block holds in MFMA row i the key 32j + 8(i/4) + 4h + i%4, so that the result
// register e of lane (c, kq) is key 32j + 8kq + 4h + e; the P^T operand of k-step j is then
// keys 32j + 8kq + 0..7 of the lane's own registers, and the matching V^T operand is one
// 16-byte run of row d.  Along d, lane kq supplies d = 32jj + 8kq .. +7 for k-step jj.  The
// cache is stored in exactly this order (kc_packed_offset, vc_packed_offset), so each load
// is one contiguous 1 KB run, read with nontemporal loads (the cache is read once per call):
// 83 against 90 us per layer at batch 32, context 4096, on MI355X.
// ------------------------------------------------------------------------------------
constexpr int DEC_BLOCK = 64;  // keys per wave per iteration

template <int NWV>
__global__ __launch_bounds__(NWV * 64) void attn_decode_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    float* __restrict__ part, bf16* __restrict__ out, int out_pack, int start_pos,
    const int* pos_dev, int pos_stride, int max_pos, int H, int G, int seq_stride,
    int chunk, int max_splits, float scale_log2) {
    __shared__ float sm_m[NWV][16], sm_l[NWV][16];
    __shared__ f32x4 sm_o[NWV - 1][8][64];
    const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int pos = max(seq_pos(pos_dev, pos_stride, b, start_pos, max_pos), 0);
    const int ctx = pos + 1;
    const int c0 = split * chunk;
    if (c0 >= ctx) return;  // no cached key in this split; the merge skips it
    const int c1 = min(ctx, c0 + chunk);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int group = H / G;
    const int col = lane & 15, kq = lane >> 4;

    bf16x8 qf[4];
    {
        const bool real = col < group;
        const bf16* qrow = q + ((size_t)b * H + g * group + (real ? col : 0)) * FA_D + 8 * kq;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            qf[jj] = real ? *reinterpret_cast<const bf16x8*>(qrow + 32 * jj) : bf16x8{};
    }
    const bf16* kbase = kc + ((size_t)b * G + g) * seq_stride * FA_D;
    const bf16* vbase = vc + ((size_t)b * G + g) * FA_D * seq_stride;

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 oacc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{};

    for (int kb = c0 + wave * DEC_BLOCK; kb < c1; kb += NWV * DEC_BLOCK) {
        // kb is a multiple of 64: the block is 16 contiguous 1 KB runs of K and of V^T in the
        // packed layout, run t * 4 + jj of K and dt * 2 + j of V^T being the operand of one load
        u32x4 kr[4][4], vr[8][2];
        const char* kblk = reinterpret_cast<const char*>(kbase + (size_t)kb * FA_D) +
                           (16 * (col >> 2) + 4 * kq + (col & 3)) * 16;
        const char* vblk = reinterpret_cast<const char*>(vbase + (size_t)kb * FA_D) + lane * 16;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int key = kb + 32 * (t >> 1) + 8 * (col >> 2) + 4 * (t & 1) + (col & 3);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                kr[t][jj] = (key < c1) ? load_stream16(kblk + (t * 4 + jj) * 1024) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int key = kb + 32 * j + 8 * kq;
                vr[dt][j] = (key < c1) ? load_stream16(vblk + (dt * 2 + j) * 1024) : u32x4{0, 0, 0, 0};
            }
        }
        f32x4 sacc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            sacc[t] = f32x4{};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, kr[t][jj]), qf[jj], sacc[t], 0, 0, 0);
        }
        if (kb + DEC_BLOCK > c1) {  // the block runs past the context
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = kb + 32 * (t >> 1) + 8 * kq + 4 * (t & 1) + e;
                    if (key >= c1) sacc[t][e] = -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[t][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx * scale_log2);  // log2 units
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        float psum = 0.0f;
        bf16x8 pf[2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][e], scale_log2, -m_new));
                psum += p;
                pf[t >> 1][4 * (t & 1) + e] = from_f32<bf16>(p);
            }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run = l_run * corr + psum;
        m_run = m_new;
        // the V^T keys past the context are zeroed here, after the S^T MFMAs, so that those
        // need not wait for the V^T loads (batch 4, context 8200: 31.7 -> 30.2 us on MI355X)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            oacc[dt] *= corr;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, mask_keys8(vr[dt][j], kb + 32 * j + 8 * kq, c1)),
                    pf[j], oacc[dt], 0, 0, 0);
        }
    }

    // merge the waves (a wave with no key keeps m = -inf, l = 0, o = 0)
    if (kq == 0) { sm_m[wave][col] = m_run; sm_l[wave][col] = l_run; }
    if (wave > 0) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) sm_o[wave - 1][dt][lane] = oacc[dt];
    }
    __syncthreads();
    if (wave > 0 || col >= group) return;
    float M = sm_m[0][col];
#pragma unroll
    for (int w = 1; w < NWV; ++w) M = fmaxf(M, sm_m[w][col]);
    float wsc[NWV], L = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        wsc[w] = (sm_m[w][col] == -INFINITY) ? 0.0f : exp2f(sm_m[w][col] - M);
        L += wsc[w] * sm_l[w][col];
    }
    const int h = g * group + col;
    if (gridDim.x == 1) {
        // the whole context in this workgroup: o / l is the attention output
        const float inv = 1.0f / L;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            f32x4 o = oacc[dt] * wsc[0];
#pragma unroll
            for (int w = 1; w < NWV; ++w) o += sm_o[w - 1][dt][lane] * wsc[w];
            const float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
            store4(out + act_offset(b, h * FA_D + 16 * dt + 4 * kq, H * FA_D, out_pack), v);
        }
        return;
    }
    float* pp = part + ((size_t)(b * H + h) * max_splits + split) * (FA_D + 2);
    if (kq == 0) { pp[0] = M; pp[1] = L; }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        f32x4 o = oacc[dt] * wsc[0];
#pragma unroll
        for (int w = 1; w < NWV; ++w) o += sm_o[w - 1][dt][lane] * wsc[w];
        *reinterpret_cast<f32x4*>(pp + 2 + 16 * dt + 4 * kq) = o;
    }
}

// Merge the splits of one (sequence, head): o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Thread t owns split t for the weights and dimension t for the sum; the splits are summed
// in order, 16 loads in flight at a time (the partials were just written and sit in L2).
constexpr int MERGE_BATCH = 16;
template <typename T>
__global__ __launch_bounds__(128) void attn_decode_merge_kernel(const float* __restrict__ part,
                                                                T* __restrict__ out, int start_pos,
                                                                const int* pos_dev,
                                                                int pos_stride, int max_pos, int H,
                                                                int d, int max_splits, int chunk,
                                                                int out_pack) {
    __shared__ float wts[128 + MERGE_BATCH];
    __shared__ float red_m[2], red_l[2];
    const int h = blockIdx.x, b = blockIdx.y;
    const int pos = max(seq_pos(pos_dev, pos_stride, b, start_pos, max_pos), 0);
    const int nsplit = (pos + 1 + chunk - 1) / chunk;  // 1 .. 128
    const float* pp = part + (size_t)(b * H + h) * max_splits * (d + 2);
    const int t = threadIdx.x;
    const float mt = t < nsplit ? pp[(size_t)t * (d + 2)] : -INFINITY;
    const float wmax = wave_max(mt);
    if ((t & 63) == 0) red_m[t >> 6] = wmax;
    __syncthreads();
    const float M = fmaxf(red_m[0], red_m[1]);
    const float w = t < nsplit ? exp2f(mt - M) : 0.0f;
    const float lw = t < nsplit ? w * pp[(size_t)t * (d + 2) + 1] : 0.0f;
    wts[t] = w;
    if (t < MERGE_BATCH) wts[128 + t] = 0.0f;
    const float lsum = wave_sum(lw);
    if ((t & 63) == 0) red_l[t >> 6] = lsum;
    __syncthreads();
    const float den = red_l[0] + red_l[1];
    for (int i = t; i < d; i += blockDim.x) {
        float num = 0.0f;
        for (int s0 = 0; s0 < nsplit; s0 += MERGE_BATCH) {
            float v[MERGE_BATCH];
#pragma unroll
            for (int j = 0; j < MERGE_BATCH; ++j)  // past the last split: reread it, weight 0
                v[j] = pp[(size_t)min(s0 + j, nsplit - 1) * (d + 2) + 2 + i];
#pragma unroll
            for (int j = 0; j < MERGE_BATCH; ++j) num += wts[s0 + j] * v[j];
        }
        out[act_offset(b, h * d + i, H * d, out_pack)] = from_f32<T>(num / den);
    }
}

// Grid of the decode attention.  Where the (sequence, KV head) pairs alone fill the chip
// and every sequence sits at the same position, one workgroup of 8 waves takes a pair's
// whole context and writes the output (no partials, no merge kernel).  Otherwise the
// context is split: keys per split grow until there are about LLAMA_DEC_TARGET_WGS
// workgroups of 4 waves, at most 128 splits for the merge.  With a position per sequence
// (ragged batches) whole-context workgroups would all wait on the longest context, and the
// many small splits balance the CUs (measured on MI355X at batch 32 with contexts spread
// over 2048..4096: 83 against 91 us on one machine, equal on another; the wider the spread,
// the more the whole-context grid leaves idle).
#ifndef LLAMA_DEC_TARGET_WGS
#define LLAMA_DEC_TARGET_WGS 8192
#endif
#ifndef LLAMA_DEC_DIRECT_MIN_PAIRS
#define LLAMA_DEC_DIRECT_MIN_PAIRS 256
#endif
struct DecodeGrid { int waves, chunk, splits; };
DecodeGrid decode_grid(const AttnArgs& a) {
    // one split covers every position of the cache
    const bool ragged = a.pos_dev && a.pos_stride != 0;
    if (!ragged && (long long)a.B * a.G >= LLAMA_DEC_DIRECT_MIN_PAIRS) return {8, a.seq_stride, 1};
    int chunk = 4 * DEC_BLOCK;
    while (chunk < 16 * 4 * DEC_BLOCK) {
        const long long splits = (a.max_ctx + chunk - 1) / chunk;
        if (splits * a.G * a.B <= LLAMA_DEC_TARGET_WGS && splits <= 128) break;
        chunk *= 2;
    }
    while ((a.max_ctx + chunk - 1) / chunk > 128) chunk *= 2;
    return {4, chunk, (a.max_ctx + chunk - 1) / chunk};
}

// splits a decode partial slot is sized for: the most a context of seq_stride positions takes
int decode_max_splits(int seq_stride) { return (seq_stride + 4 * DEC_BLOCK - 1) / (4 * DEC_BLOCK); }

hipError_t launch_decode_mfma(const AttnArgs& a, hipStream_t s) {
    const DecodeGrid dg = decode_grid(a);
    const int max_splits = decode_max_splits(a.seq_stride);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)FA_D);
    const dim3 grid(dg.splits, a.G, a.B);
    if (dg.waves == 8)
        attn_decode_mfma_kernel<8><<<grid, 512, 0, s>>>(
            (const bf16*)a.q, (const bf16*)a.kc, (const bf16*)a.vc, a.partials, (bf16*)a.out,
            a.out_pack, a.start_pos, a.pos_dev, a.pos_stride, a.max_pos, a.H, a.G, a.seq_stride,
            dg.chunk, max_splits, scale_log2);
    else
        attn_decode_mfma_kernel<4><<<grid, 256, 0, s>>>(
            (const bf16*)a.q, (const bf16*)a.kc, (const bf16*)a.vc, a.partials, (bf16*)a.out,
            a.out_pack, a.start_pos, a.pos_dev, a.pos_stride, a.max_pos, a.H, a.G, a.seq_stride,
            dg.chunk, max_splits, scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || dg.splits == 1) return e;
    attn_decode_merge_kernel<bf16><<<dim3(a.H, a.B), 128, 0, s>>>(
        a.partials, (bf16*)a.out, a.start_pos, a.pos_dev, a.pos_stride, a.max_pos, a.H, FA_D,
        max_splits, dg.chunk, a.out_pack);
    return hipGetLastError();
}

bool mfma_path(const AttnArgs& a) {
    const int group = a.H / a.G;
    return a.d == FA_D && group <= 16 && FA_ROWS % group == 0;
}

}  // namespace

bool kv_cache_packed(Dt dt, int H, int G, int d) {
    AttnArgs a{};
    a.H = H; a.G = G; a.d = d;
    return dt == Dt::BF16 && G > 0 && H % G == 0 && mfma_path(a);
}

hipError_t attention_prefill(Dt dt, const AttnArgs& a, hipStream_t s) {
    if (a.B * a.S == 0) return hipSuccess;
    if (dt == Dt::BF16 && mfma_path(a)) return launch_prefill_mfma(a, s);
    if (dt == Dt::BF16) return launch_generic<bf16>(a, s);
    return launch_generic<float>(a, s);
}

size_t decode_partials_bytes(int B, int H, int d, int seq_stride) {
    return (size_t)B * H * decode_max_splits(seq_stride) * (d + 2) * sizeof(float);
}

hipError_t attention_decode(Dt dt, const AttnArgs& a, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    if (dt == Dt::BF16 && mfma_path(a)) return launch_decode_mfma(a, s);
    if (dt == Dt::BF16) return launch_generic<bf16>(a, s);
    return launch_generic<float>(a, s);
}

}  // namespace lk
