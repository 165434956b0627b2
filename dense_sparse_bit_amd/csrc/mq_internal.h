// Internal launcher interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

struct GemmArgs {
    const uint8_t* xq;
    const float* sx;
    const uint8_t* wq;
    const uint16_t* sw;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const int32_t* rmap;       // dense block map [N/bn][K/64] (CSR position or -1), or null
    const uint8_t* rq;
    int nnz;
    int M, N, K, bn;
    void* y;
    int y_bf16;
    int32_t* acc_dump;
    float* ws;
    // the GEMM that quantizes its own activations: x [M][K] (fp32 or bf16), and
    // where the codes and scales go (then read back as xq / sx), plus the
    // producer/consumer counters (int32 [4], zero between calls)
    const void* x;
    int x_bf16;
    uint8_t* xq_w;
    float* sx_w;
    int* sync;
};

// int32 words of the self-quantizing GEMM's counter array: one 128-byte line for
// the count of quantized tokens and the give-up flag, one per XCD slot (16)
constexpr int kSyncWords = 32 * 17;

enum class GemmKind { Fused, Dense, DenseToWorkspace, FusedQuantAct };

// How the decode GEMM (M <= 32) is split: nw waves per workgroup share K.
struct DecodePlan {
    int nw;
};
DecodePlan plan_decode(int M, int N, int K);
// scratch bytes of the selection: per-block ranks (4 nb, padded to 8) and, when the
// caller passes no delta output, the fp64 scores (8 nb)
inline size_t select_scratch_bytes(int64_t nb, bool scores) {
    const size_t ranks = (static_cast<size_t>(nb) * 4 + 7) & ~static_cast<size_t>(7);
    return ranks + (scores ? static_cast<size_t>(nb) * 8 : 0);
}

// colscale: per-channel multipliers r_k applied to x before the step (the migrated
// activations x^ = fp32(x * r_k)), or null
hipError_t launch_hessian(const void* x, int bf16, int64_t M, int64_t K, const float* colscale, float* h,
                          hipStream_t st);
// threads per token of the stand-alone activation quantizer
int quant_act_threads(int64_t M, int64_t K);
hipError_t launch_quant_act(const void* x, int bf16, int64_t M, int64_t K, const float* colscale, uint8_t* xq,
                            float* sx, hipStream_t st);
hipError_t launch_smooth(const void* x, int bf16, int64_t M, int64_t K, const float* w, int64_t N, float* s,
                         float* r, hipStream_t st);
hipError_t launch_scale_cols(const float* in, int64_t rows, int64_t K, const float* c, float* out, hipStream_t st);
// scratch: select_scratch_bytes(nb, delta == null) bytes, or null for a stream-ordered allocation
hipError_t launch_select(const float* w, const float* h, int64_t N, int64_t K, int bn,
                         int64_t k_blocks, int32_t* row_ptr, int32_t* col_idx, double* delta,
                         void* scratch, hipStream_t st);
hipError_t launch_pack(const float* w, int64_t N, int64_t K, int bn, const int32_t* row_ptr,
                       const int32_t* col_idx, int64_t nnz, uint8_t* wq, uint16_t* sw, uint8_t* rq,
                       hipStream_t st);
hipError_t launch_block_map(const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz, int64_t N, int64_t K,
                            int bn, int32_t* rmap, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, GemmKind kind, hipStream_t st);
// streaming-read probe: at most kReadProbeMaxBlocks workgroups, one output word each
constexpr int kReadProbeMaxBlocks = 8192;
int read_probe_blocks(int64_t bytes);
hipError_t launch_read_probe(const void* p, int64_t bytes, uint32_t* out, hipStream_t st);
hipError_t launch_residual_merge(const GemmArgs& a, hipStream_t st);

}  // namespace mq
