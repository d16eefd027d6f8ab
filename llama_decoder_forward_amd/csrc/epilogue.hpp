// GEMM epilogues.  Every GEMM computes acc[m][n] = sum_k A[m][k] * W[n][k] (token row m,
// weight row n) in fp32 and hands the result to an epilogue in groups of four consecutive
// output columns n, n+1, n+2, n+3 (n % 4 == 0) of one row m.
#pragma once
#include "common.hpp"

// The V cache holds V transposed inside blocks of VT_BLOCK positions: element (pos, i) of
// sequence/head context c sits at [c][pos / VT_BLOCK][i][pos % VT_BLOCK].  A block of keys
// is then one contiguous d x VT_BLOCK run, and the P.V operand (keys contiguous for a fixed
// i) is a plain 16-byte load.
constexpr int VT_BLOCK = 64;
__host__ __device__ __forceinline__ size_t vt_offset(size_t ctx_index, int pos, int i, int d,
                                                     int seq_stride) {
    return ctx_index * (size_t)d * seq_stride + ((size_t)(pos / VT_BLOCK) * d + i) * VT_BLOCK +
           (pos % VT_BLOCK);
}

// Packed KV-cache layout of the bf16 matrix-core attention path (head_dim 128).  A block of
// 64 positions of one (sequence, KV head) context keeps the same 8192-element place as in the
// plain layouts, but is ordered as the decode attention loads it: sixteen runs of 1 KB, each
// the operand of one 16-byte-per-lane load, so that every load is one contiguous 1 KB run.
//  - K: run t * 4 + jj holds, at 16-byte position 16 (col / 4) + 4 kq + col % 4, the 8 values
//    d = 32 jj + 8 kq .. of key r = 32 (t / 2) + 8 (col / 4) + 4 (t % 2) + col % 4 of the
//    block (the decode load of lane col + 16 kq reads that position; the order within the run
//    puts the 16 pieces of four consecutive keys in one 256-byte span, so that a prefill copy
//    of four key rows reads whole cache lines);
//  - V: run dt * 2 + j holds, at lane l = col + 16 kq, the values of dimension d = 16 dt + col
//    for keys r = 32 j + 8 kq .. +7 of the block.
// The prefill attention's direct global -> LDS copies address the same 16-byte pieces, so its
// LDS tiles are unchanged.  Offsets in elements; pos - pos % 64 is the block's first position.
constexpr int KVP_D = 128;
__host__ __device__ __forceinline__ size_t kc_packed_offset(size_t ctx_index, int pos, int i,
                                                            int seq_stride) {
    const int r = pos & 63;
    const int t = 2 * (r >> 5) + ((r >> 2) & 1), col = 4 * ((r >> 3) & 3) + (r & 3);
    const int jj = i >> 5, kq = (i >> 3) & 3, e = i & 7;
    return (ctx_index * seq_stride + (pos - r)) * KVP_D +
           (size_t)((t * 4 + jj) * 512 + (16 * (col >> 2) + 4 * kq + (col & 3)) * 8 + e);
}
__host__ __device__ __forceinline__ size_t vc_packed_offset(size_t ctx_index, int pos, int i,
                                                            int seq_stride) {
    const int r = pos & 63;
    const int dt = i >> 4, col = i & 15, j = r >> 5, kq = (r >> 3) & 3, e = r & 7;
    return (ctx_index * seq_stride + (pos - r)) * KVP_D +
           (size_t)((dt * 2 + j) * 512 + (col + 16 * kq) * 8 + e);
}

// Activation layout of the few-row (decode) GEMMs.  pack == 0: plain row-major [m][ld].
// pack = P > 0 (a power of two >= the row count, at most 64): the values are stored in the
// order the weight-streaming GEMM feeds them to its 16x16x32 MFMAs, so that each of its
// activation loads is one contiguous run.  Rows are grouped in blocks of R = min(P, 16); for
// k-block kb = k / 128, slice j = (k / 32) % 4 and row block mb = m / R, the run holds the
// 8 values k - k % 8 .. of row m at position (m % R) + R * ((k / 8) % 4).  With P < 16 the
// GEMM's 16 operand lanes reread the R stored rows (their results are never stored), so a
// batch of 4 moves 4 rows, not 16.  Any four consecutive k starting at a multiple of 4 stay
// contiguous.  The producers of a GEMM's input (RMSNorm, attention output, SwiGLU) write
// this layout when that GEMM runs on the weight-streaming path.
__host__ __device__ __forceinline__ size_t act_offset(int m, int k, int ld, int pack) {
    if (pack == 0) return (size_t)m * ld + k;
    const int R = pack < 16 ? pack : 16;
    const size_t blk = ((size_t)(k >> 7) * 4 + ((k >> 5) & 3)) * (pack / R) + m / R;
    return ((blk * 4 + ((k >> 3) & 3)) * R + (m & (R - 1))) * 8 + (k & 7);
}

// Position of sequence b's first token in this call: start_pos, or read from device memory
// as pos_dev[b * pos_stride] (stride 0: one position shared by every sequence).  A device
// value outside [0, max_pos) gives -1: readers then use position 0 and the KV-cache writes
// are skipped, so no access leaves the cache or the rotary table and no valid cache entry
// is overwritten (a check kernel raises the call's error flag).
__device__ __forceinline__ int seq_pos(const int* pos_dev, int pos_stride, int b, int start_pos,
                                       int max_pos) {
    if (!pos_dev) return start_pos;
    const int p = pos_dev[b * pos_stride];
    return (p >= 0 && p < max_pos) ? p : -1;
}

// Weight rows of a GEMM, possibly split over up to three matrices stacked along n
// (Q, K and V projections share one GEMM: rows [0,end0) of p0, then p1, then p2).
template <typename T>
struct WeightRows {
    const T* p0; const T* p1; const T* p2;
    int end0, end1;  // cumulative row ends of p0 and p1
    int ld;          // row stride (= K)
    __device__ __forceinline__ const T* row(int n) const {
        if (n < end0) return p0 + (size_t)n * ld;
        if (n < end1) return p1 + (size_t)(n - end0) * ld;
        return p2 + (size_t)(n - end1) * ld;
    }
};

// logits (or any plain fp32 output): C[m][n] = acc
struct EpiStoreF32 {
    float* C; int ldc;
    __device__ __forceinline__ void operator()(int m, int n, float v[4]) const {
        store4(C + (size_t)m * ldc + n, v);
    }
};

// Residual add into the fp32 hidden state (article, section 相加与归一化 and the add after
// the feed-forward): xout[m][n] = xin[m][n] + acc.  xin may equal xout.
struct EpiResidual {
    const float* xin; float* xout; int ld;
    __device__ __forceinline__ void operator()(int m, int n, float v[4]) const {
        const f32x4 r = *reinterpret_cast<const f32x4*>(xin + (size_t)m * ld + n);
        float o[4] = {r[0] + v[0], r[1] + v[1], r[2] + v[2], r[3] + v[3]};
        store4(xout + (size_t)m * ld + n, o);
    }
};

// One K split of a residual GEMM (split z = blockIdx.y): part[z][m][n] = the split's sum.
// The RMSNorm that next reads the residual stream adds the splits in order z = 0, 1, ...
struct EpiPartial {
    float* part; int ld; size_t split_stride;
    __device__ __forceinline__ void operator()(int m, int n, float v[4]) const {
        store4(part + blockIdx.y * split_stride + (size_t)m * ld + n, v);
    }
};

// SwiGLU gate (article, section 前馈神经网络层): g[m][n] = silu(h.w1_n) * (h.w3_n),
// silu(z) = z / (1 + exp(-z)).
// g is stored in the activation layout of the down projection (act_offset, pack).
template <typename T>
struct EpiSwiGLU {
    T* g; int ld; int pack;
    __device__ __forceinline__ void operator()(int m, int n, float gate[4], float up[4]) const {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = gate[i] / (1.0f + __expf(-gate[i])) * up[i];
        store4(g + act_offset(m, n, ld, pack), o);
    }
};

// Q/K/V projection epilogue: rotary embedding of q and k (article, section 位置编码:
// adjacent pairs (x[2i], x[2i+1]) rotated by the angle pos * theta_i), q stored for the
// attention kernel, k and v written to the KV cache at their positions.
//   q   : [M][Nq] with Nq = H*d, row m = token (sequence m / S, position start + m % S)
//   kc  : this layer's K cache [max_batch][G][seq_stride][d]
//   vc  : this layer's V cache, transposed within blocks of 64 positions:
//         [max_batch][G][seq_stride/64][d][64] (see VT_BLOCK)
//   (with `packed`, both caches in the packed layout above: kc_packed_offset, vc_packed_offset)
//   rope: [max_seq][d/2] of (cos, sin)
template <typename T>
struct EpiQKV {
    T* q; T* kc; T* vc;
    const float2* rope;
    int Nq, Nk, d, S, start_pos, G, seq_stride;
    const int* pos_dev;  // if set, the start positions are read from device memory (seq_pos)
    int pos_stride, max_pos;
    int packed;          // caches in the packed layout (bf16, head_dim 128, matrix-core path)

    __device__ __forceinline__ void operator()(int m, int n, float v[4]) const {
        const int b = m / S;
        const int p0 = seq_pos(pos_dev, pos_stride, b, start_pos, max_pos);
        const bool write_cache = p0 >= 0;
        const int pos = (p0 >= 0 ? p0 : 0) + (m - b * S);
        if (n < Nq + Nk) {
            const int j = (n < Nq ? n : n - Nq) % d;  // even; pairs (j, j+1), (j+2, j+3)
            const float2 cs0 = rope[(size_t)pos * (d / 2) + j / 2];
            const float2 cs1 = rope[(size_t)pos * (d / 2) + j / 2 + 1];
            const float a0 = v[0], b0 = v[1], a1 = v[2], b1 = v[3];
            v[0] = a0 * cs0.x - b0 * cs0.y;
            v[1] = a0 * cs0.y + b0 * cs0.x;
            v[2] = a1 * cs1.x - b1 * cs1.y;
            v[3] = a1 * cs1.y + b1 * cs1.x;
        }
        if (n < Nq) {
            store4(q + (size_t)m * Nq + n, v);
        } else if (!write_cache) {
        } else if (n < Nq + Nk) {
            const int nk = n - Nq, g = nk / d, j = nk - g * d;
            const size_t ctx = (size_t)b * G + g;
            // j % 4 == 0: the four values are contiguous in either layout
            store4(kc + (packed ? kc_packed_offset(ctx, pos, j, seq_stride)
                                : (ctx * seq_stride + pos) * d + j), v);
        } else {
            const int nv = n - Nq - Nk, g = nv / d, j = nv - g * d;
            const size_t ctx = (size_t)b * G + g;
            if (packed) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vc[vc_packed_offset(ctx, pos, j + i, seq_stride)] = from_f32<T>(v[i]);
            } else {
                T* base = vc + vt_offset(ctx, pos, j, d, seq_stride);
#pragma unroll
                for (int i = 0; i < 4; ++i) base[(size_t)i * VT_BLOCK] = from_f32<T>(v[i]);
            }
        }
    }
};
