// Host-side launchers of the kernels (internal to the library).  Each returns the
// hipError_t of its launch.  Shapes are validated by the caller (api.hip).
#pragma once
#include "epilogue.hpp"

#include <atomic>

namespace lk {

enum class Dt { BF16, F32 };

// Per-device, set-once state of the launchers (kernel attributes, device properties): a bit
// per device ordinal below 64, safe to test and set from several host threads.
struct PerDevice {
    std::atomic<unsigned long long> done{0};
    // Run `set` once on the current device; later calls on that device return at once.
    template <typename F>
    hipError_t once(F&& set) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
        if (bit != 0 && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
        e = set(dev);
        if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
        return e;
    }
};

// Compute units of the current device (gemm_skinny.hip); 256 if it cannot be queried.
int cu_count();

// ---- elementwise / reductions (elementwise.hip)
hipError_t rope_table(float2* rope, int max_seq, int d, float theta, hipStream_t s);
hipError_t embed(Dt dt, const int* tokens, const void* E, float* x, int rows, int D, int V,
                 uint32_t* err, hipStream_t s);
// y[r] = rmsnorm(x[r * in_stride_rows + in_offset_rows]) for r < rows, y in the activation
// layout act_offset(r, i, D, y_pack)
hipError_t rmsnorm(Dt dt, const float* x, int in_row_step, int in_row_offset, const void* w,
                   void* y, int y_pack, int rows, int D, float eps, hipStream_t s);
// The same after folding pending split-K sums into the residual stream: for each row read,
// x' = x + sum_z parts[z] (z = 0 .. nsplit-1 in order, split stride `split_stride` floats,
// same row indexing as x) is written to x_out (may equal x) and normalised.
hipError_t rmsnorm_fold(Dt dt, const float* x, const float* parts, int nsplit, size_t split_stride,
                        float* x_out, int in_row_step, int in_row_offset, const void* w, void* y,
                        int y_pack, int rows, int D, float eps, hipStream_t s);
size_t argmax_scratch_bytes(int rows, int V);
// out[r] = argmax of logits row r * row_step + row_off, r < rows (and the token log out2)
hipError_t argmax(const float* logits, int rows, int row_step, int row_off, int V, int* out,
                  int* out2, int out2_step, const int* counter, void* scratch, uint32_t* err,
                  hipStream_t s);
// dst[r] = src[r * step + off], rows of D floats (D % 4 == 0)
hipError_t copy_rows(const float* src, int step, int off, float* dst, int rows, int D,
                     hipStream_t s);
hipError_t bump_counters(int* pos, int* step, hipStream_t s);
hipError_t zero_u32(uint32_t* p, int n, hipStream_t s);
// fill `bytes` bytes (a multiple of 16, 16-byte aligned) with zeros
hipError_t zero_bytes(void* p, size_t bytes, hipStream_t s);
hipError_t copy_tokens(const int* src, int* dst, int n, hipStream_t s);
hipError_t set_counters(int* pos, int pos_value, int* step, hipStream_t s);
// raise DEVERR_POSITION_RANGE if some pos[b], b < B, lies outside [0, max_pos)
hipError_t check_positions(const int* pos, int B, int max_pos, uint32_t* err, hipStream_t s);

// ---- GEMMs: acc[m][n] = sum_k A[m][k] W[n][k]  (gemm_mfma.hip, gemm_simt.hip, gemm_skinny.hip)
template <typename T> struct GemmArgs {
    const T* A; int lda;
    int a_pack;         // activation layout of A (act_offset); > 0 selects the weight-streaming path
    WeightRows<T> W;
    WeightRows<T> W3;  // second weight set of the SwiGLU gate/up GEMM
    int M, N, K;
};
// Weight-streaming path for few rows (gemm_skinny.hip).  act_pack returns the activation
// layout (row blocks of 16) its input must be written in, or 0 where the GEMM of these sizes
// takes the tiled or fp32 path and reads plain row-major A.
int act_pack(Dt dt, int M, int N, int K);
template <bool DUAL, typename Epi>
hipError_t skinny_launch(const GemmArgs<void>& g, const Epi& e, hipStream_t s);
hipError_t gemm_store_f32(Dt dt, const GemmArgs<void>& g, EpiStoreF32 e, hipStream_t s);
hipError_t gemm_residual(Dt dt, const GemmArgs<void>& g, EpiResidual e, hipStream_t s);
// Split-K form of a residual GEMM: part[z][m][n] (z < splits, splits = residual_splits(...),
// split stride M*N floats) holds split z's share of acc; the residual itself is not touched.
// residual_splits returns 0 where this form is not used.  Up to 64 rows it is the
// weight-streaming path's; beyond, the tiled path's (tiled_residual_splits).
constexpr int LLAMA_MAX_KSPLITS = 16;
// Rows up to which a residual GEMM on the tiled path may be split over K (the workspace
// holds two splits' sums of that many rows).
constexpr int LLAMA_TILED_SPLIT_MAX_ROWS = 4096;
int residual_splits(Dt dt, int M, int N, int K);
int tiled_residual_splits(Dt dt, int M, int N, int K);
hipError_t gemm_residual_split_tiled(const GemmArgs<void>& g, float* part, int splits, hipStream_t s);
hipError_t gemm_residual_split(Dt dt, const GemmArgs<void>& g, float* part, int splits, hipStream_t s);
hipError_t gemm_swiglu(Dt dt, const GemmArgs<void>& g, void* out, int ld, int out_pack, hipStream_t s);
hipError_t gemm_qkv(Dt dt, const GemmArgs<void>& g, const EpiQKV<void>& e, hipStream_t s);

// ---- attention (attention.hip)
struct AttnArgs {
    const void* q;   // [rows][H*d], row = b*S + s
    const void* kc;  // layer K cache
    const void* vc;  // layer V^T cache
    void* out;       // [rows][H*d] in the activation layout act_offset(row, col, H*d, out_pack)
    int out_pack;
    int B, S, start_pos, H, G, d, seq_stride;
    const int* pos_dev;  // per-sequence start positions in device memory (seq_pos) or NULL
    int pos_stride, max_pos;
    float* partials; // decode split-K scratch
    int max_ctx;     // upper bound of start_pos + S (sizing of decode grids)
};
// The KV cache of a model with these shapes uses the packed layout (kc_packed_offset,
// vc_packed_offset): exactly when its attention runs on the bf16 matrix-core kernels.
bool kv_cache_packed(Dt dt, int H, int G, int d);
hipError_t attention_prefill(Dt dt, const AttnArgs& a, hipStream_t s);
hipError_t attention_decode(Dt dt, const AttnArgs& a, hipStream_t s);
// bytes of decode split partials (AttnArgs::partials) for B sequences of H heads
size_t decode_partials_bytes(int B, int H, int d, int seq_stride);

}  // namespace lk
