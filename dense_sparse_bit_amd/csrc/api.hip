// C ABI of the MosaicQuant library: argument checks, then kernel launches.
// Declarations and the meaning of every argument are in include/mq.h.
#include <stdint.h>

#include <mutex>

#include "../../include/mq.h"
#include "mq_device.h"
#include "mq_internal.h"

// Static scratch of mq_select_blocks_noalloc, one copy per GPU. In host code
// `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current) and
// only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[MQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 10100;   // 1.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MQ_OK : MQ_ERR_HIP; }

bool bad_dtype(int d) { return d != MQ_F32 && d != MQ_BF16; }

// shapes the GPU path supports (see mq.h)
int check_layer(int64_t N, int64_t K, int group, int bn, int bk) {
    if (N <= 0 || K <= 0) return MQ_ERR_INVALID_ARG;
    if (group != mq::kGroup || bk != mq::kBk || (bn != 64 && bn != 128)) return MQ_ERR_UNSUPPORTED;
    if (K % mq::kGroup || N % bn) return MQ_ERR_UNSUPPORTED;
    // K <= 65536: the kernels' per-row block tables hold up to 1024 column blocks
    if (K > 65536 || N > (int64_t(1) << 30) || N * K > (int64_t(1) << 40)) return MQ_ERR_UNSUPPORTED;
    return MQ_OK;
}

int check_gemm(const uint8_t* xq, const float* sx, const uint8_t* wq, const uint16_t* sw, int64_t M,
               int64_t N, int64_t K, int group, int bn, int bk, const void* y, int y_dtype) {
    int rc = check_layer(N, K, group, bn, bk);
    if (rc) return rc;
    if (M < 0 || M > (int64_t(1) << 24)) return MQ_ERR_INVALID_ARG;
    if (bad_dtype(y_dtype)) return MQ_ERR_INVALID_ARG;
    if (M > 0 && (!xq || !sx || !y)) return MQ_ERR_INVALID_ARG;
    if (!wq || !sw) return MQ_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || (reinterpret_cast<uintptr_t>(sw) & 7u)) return MQ_ERR_INVALID_ARG;
    // every int32 index the kernels form must fit
    if (M * N > (int64_t(1) << 31) - 1 || M * N * (K / mq::kGroup) > (int64_t(1) << 40))
        return MQ_ERR_UNSUPPORTED;
    return MQ_OK;
}

int check_csr(const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* rq, int64_t nnz,
              int64_t N, int64_t K, int bn, int bk) {
    if (nnz < 0 || nnz > (N / bn) * (K / bk)) return MQ_ERR_INVALID_ARG;
    if (!row_ptr) return MQ_ERR_INVALID_ARG;
    if (nnz > 0 && (!col_idx || !rq || !aligned16(rq))) return MQ_ERR_INVALID_ARG;
    return MQ_OK;
}

mq::GemmArgs make_args(const uint8_t* xq, const float* sx, const uint8_t* wq, const uint16_t* sw,
                       const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* rq,
                       int64_t nnz, int64_t M, int64_t N, int64_t K, int bn, void* y, int y_dtype,
                       int32_t* acc_dump, float* ws) {
    mq::GemmArgs a;
    a.xq = xq;
    a.sx = sx;
    a.wq = wq;
    a.sw = sw;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.rmap = nullptr;
    a.rq = rq;
    a.nnz = static_cast<int>(nnz);
    a.M = static_cast<int>(M);
    a.N = static_cast<int>(N);
    a.K = static_cast<int>(K);
    a.bn = bn;
    a.y = y;
    a.y_bf16 = y_dtype == MQ_BF16;
    a.acc_dump = acc_dump;
    a.ws = ws;
    a.x = nullptr;
    a.x_bf16 = 0;
    a.xq_w = nullptr;
    a.sx_w = nullptr;
    a.sync = nullptr;
    return a;
}

// argument checks of mq_select_blocks; the scratch (caller workspace or the
// library's own) is checked by the caller of this helper
int check_select(const float* w, const float* h, int64_t N, int64_t K, int group, int bn, int bk,
                 int64_t k_blocks, const int32_t* row_ptr, const int32_t* col_idx) {
    int rc = check_layer(N, K, group, bn, bk);
    if (rc) return rc;
    const int64_t nb = (N / bn) * (K / bk);
    if (k_blocks < 0 || k_blocks > nb) return MQ_ERR_INVALID_ARG;
    if (!w || !h || !row_ptr || (k_blocks > 0 && !col_idx) || !aligned16(w) || !aligned16(h))
        return MQ_ERR_INVALID_ARG;
    return MQ_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's address of `scratch` (looked up on first use), or null on error
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* mq_status_string(int status) {
    switch (status) {
        case MQ_OK: return "ok";
        case MQ_ERR_INVALID_ARG: return "invalid argument (null pointer, size, alignment or count)";
        case MQ_ERR_UNSUPPORTED: return "unsupported shape (needs K % 128 == 0, group 128, bk 64, bn 64 or 128, N % bn == 0)";
        case MQ_ERR_HIP: return "HIP runtime error";
        case MQ_ERR_SCRATCH: return "shape needs more scratch than the library's static array (MQ_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int mq_version(void) { return kVersion; }

int mq_hessian_diag(const void* x, int x_dtype, int64_t M, int64_t K, float* h, void* stream) {
    if (M <= 0 || K <= 0 || !x || !h || bad_dtype(x_dtype)) return MQ_ERR_INVALID_ARG;
    if (M * K > (int64_t(1) << 40)) return MQ_ERR_UNSUPPORTED;
    return hip_status(mq::launch_hessian(x, x_dtype == MQ_BF16, M, K, nullptr, h, static_cast<hipStream_t>(stream)));
}

int mq_hessian_diag_scaled(const void* x, int x_dtype, int64_t M, int64_t K, const float* r, float* h,
                           void* stream) {
    if (M <= 0 || K <= 0 || !x || !h || !r || bad_dtype(x_dtype)) return MQ_ERR_INVALID_ARG;
    if (M * K > (int64_t(1) << 40)) return MQ_ERR_UNSUPPORTED;
    return hip_status(mq::launch_hessian(x, x_dtype == MQ_BF16, M, K, r, h, static_cast<hipStream_t>(stream)));
}

int mq_smooth_factors(const void* x, int x_dtype, int64_t M, int64_t K, const float* w, int64_t N, float* s,
                      float* r, void* stream) {
    if (M <= 0 || K <= 0 || N <= 0 || !x || !w || !s || !r || bad_dtype(x_dtype)) return MQ_ERR_INVALID_ARG;
    if (M * K > (int64_t(1) << 40) || N * K > (int64_t(1) << 40)) return MQ_ERR_UNSUPPORTED;
    return hip_status(mq::launch_smooth(x, x_dtype == MQ_BF16, M, K, w, N, s, r, static_cast<hipStream_t>(stream)));
}

int mq_scale_columns(const float* w, int64_t N, int64_t K, const float* s, float* w_hat, void* stream) {
    if (N <= 0 || K <= 0 || (K & 3) || !w || !s || !w_hat) return MQ_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(s) || !aligned16(w_hat)) return MQ_ERR_INVALID_ARG;
    if (N * K > (int64_t(1) << 40)) return MQ_ERR_UNSUPPORTED;
    return hip_status(mq::launch_scale_cols(w, N, K, s, w_hat, static_cast<hipStream_t>(stream)));
}

int mq_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* xq, float* sx,
                    void* stream) {
    if (M < 0 || K <= 0 || (K & 1) || bad_dtype(x_dtype)) return MQ_ERR_INVALID_ARG;
    if (K % mq::kGroup || M > (int64_t(1) << 31) - 1 || M * K > (int64_t(1) << 40)) return MQ_ERR_UNSUPPORTED;
    if (M == 0) return MQ_OK;
    if (!x || !xq || !sx || !aligned16(x) || !aligned16(xq)) return MQ_ERR_INVALID_ARG;
    return hip_status(mq::launch_quant_act(x, x_dtype == MQ_BF16, M, K, nullptr, xq, sx,
                                           static_cast<hipStream_t>(stream)));
}

int mq_quantize_act_scaled(const void* x, int x_dtype, int64_t M, int64_t K, const float* r, uint8_t* xq,
                           float* sx, void* stream) {
    if (M < 0 || K <= 0 || (K & 1) || bad_dtype(x_dtype)) return MQ_ERR_INVALID_ARG;
    if (K % mq::kGroup || M > (int64_t(1) << 31) - 1 || M * K > (int64_t(1) << 40)) return MQ_ERR_UNSUPPORTED;
    if (M == 0) return MQ_OK;
    if (!x || !xq || !sx || !r || !aligned16(x) || !aligned16(xq) || !aligned16(r)) return MQ_ERR_INVALID_ARG;
    return hip_status(mq::launch_quant_act(x, x_dtype == MQ_BF16, M, K, r, xq, sx, static_cast<hipStream_t>(stream)));
}

int mq_select_blocks(const float* w, const float* h, int64_t N, int64_t K, int group, int bn, int bk,
                     int64_t k_blocks, int32_t* row_ptr, int32_t* col_idx, double* delta,
                     void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_select(w, h, N, K, group, bn, bk, k_blocks, row_ptr, col_idx);
    if (rc) return rc;
    const int64_t nb = (N / bn) * (K / bk);
    if (workspace && (workspace_bytes < mq::select_scratch_bytes(nb, delta == nullptr) ||
                      (reinterpret_cast<uintptr_t>(workspace) & 7u)))
        return MQ_ERR_INVALID_ARG;
    return hip_status(mq::launch_select(w, h, N, K, bn, k_blocks, row_ptr, col_idx, delta, workspace,
                                        static_cast<hipStream_t>(stream)));
}

int mq_select_blocks_noalloc(const float* w, const float* h, int64_t N, int64_t K, int group, int bn,
                             int bk, int64_t k_blocks, int32_t* row_ptr, int32_t* col_idx, double* delta,
                             void* stream) {
    int rc = check_select(w, h, N, K, group, bn, bk, k_blocks, row_ptr, col_idx);
    if (rc) return rc;
    const int64_t nb = (N / bn) * (K / bk);
    if (mq::select_scratch_bytes(nb, delta == nullptr) > MQ_NOALLOC_SCRATCH_BYTES) return MQ_ERR_SCRATCH;
    void* buf = device_scratch();
    if (!buf) return MQ_ERR_HIP;
    // the kernels clear and fully rewrite the ranks and scores they use: nothing
    // from an earlier call is read
    return hip_status(mq::launch_select(w, h, N, K, bn, k_blocks, row_ptr, col_idx, delta, buf,
                                        static_cast<hipStream_t>(stream)));
}

size_t mq_select_workspace_bytes(int64_t N, int64_t K, int bn, int bk) {
    if (check_layer(N, K, mq::kGroup, bn, bk)) return 0;
    return mq::select_scratch_bytes((N / bn) * (K / bk), true);
}

int mq_pack_weights(const float* w, int64_t N, int64_t K, int group, int bn, int bk,
                    const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz, uint8_t* wq,
                    uint16_t* sw, uint8_t* rq, void* stream) {
    int rc = check_layer(N, K, group, bn, bk);
    if (rc) return rc;
    if (!w || !wq || !sw || !aligned16(w) || !aligned16(wq)) return MQ_ERR_INVALID_ARG;
    rc = check_csr(row_ptr, col_idx, rq, nnz, N, K, bn, bk);
    if (rc) return rc;
    return hip_status(mq::launch_pack(w, N, K, bn, row_ptr, col_idx, nnz, wq, sw, rq,
                                      static_cast<hipStream_t>(stream)));
}

int mq_gemm_w4a4_residual(const uint8_t* xq, const float* sx, const uint8_t* wq, const uint16_t* sw,
                          const int32_t* row_ptr, const int32_t* col_idx, const uint8_t* rq,
                          int64_t nnz, int64_t M, int64_t N, int64_t K, int group, int bn, int bk,
                          void* y, int y_dtype, int32_t* acc_dump, void* stream) {
    int rc = check_gemm(xq, sx, wq, sw, M, N, K, group, bn, bk, y, y_dtype);
    if (rc) return rc;
    rc = check_csr(row_ptr, col_idx, rq, nnz, N, K, bn, bk);
    if (rc) return rc;
    if (M == 0) return MQ_OK;
    const mq::GemmArgs a = make_args(xq, sx, wq, sw, row_ptr, col_idx, rq, nnz, M, N, K, bn, y, y_dtype,
                                     acc_dump, nullptr);
    return hip_status(mq::launch_gemm(a, mq::GemmKind::Fused, static_cast<hipStream_t>(stream)));
}

int mq_block_map(const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz, int64_t N, int64_t K,
                 int bn, int bk, int32_t* rmap, void* stream) {
    int rc = check_layer(N, K, mq::kGroup, bn, bk);
    if (rc) return rc;
    if (nnz < 0 || nnz > (N / bn) * (K / bk) || !row_ptr || !rmap || (nnz > 0 && !col_idx))
        return MQ_ERR_INVALID_ARG;
    return hip_status(mq::launch_block_map(row_ptr, col_idx, nnz, N, K, bn, rmap, static_cast<hipStream_t>(stream)));
}

int mq_gemm_w4a4_residual_mapped(const uint8_t* xq, const float* sx, const uint8_t* wq, const uint16_t* sw,
                                 const int32_t* rmap, const uint8_t* rq, int64_t nnz, int64_t M, int64_t N,
                                 int64_t K, int group, int bn, int bk, void* y, int y_dtype, int32_t* acc_dump,
                                 void* stream) {
    int rc = check_gemm(xq, sx, wq, sw, M, N, K, group, bn, bk, y, y_dtype);
    if (rc) return rc;
    if (nnz < 0 || nnz > (N / bn) * (K / bk) || !rmap || (nnz > 0 && (!rq || !aligned16(rq))))
        return MQ_ERR_INVALID_ARG;
    // the kernels address the whole payload with 32-bit byte offsets
    if (nnz * bn * (bk / 2) > (int64_t(1) << 31)) return MQ_ERR_UNSUPPORTED;
    if (M == 0) return MQ_OK;
    mq::GemmArgs a = make_args(xq, sx, wq, sw, nullptr, nullptr, rq, nnz, M, N, K, bn, y, y_dtype, acc_dump,
                               nullptr);
    a.rmap = rmap;
    return hip_status(mq::launch_gemm(a, mq::GemmKind::Fused, static_cast<hipStream_t>(stream)));
}

static_assert(mq::kSyncWords == MQ_SYNC_WORDS, "sync array size");


// Measured crossover on MI355X (K x N from 4096 x 1024 to 28672 x 8192, M = 1..32).
// The one-launch form quantizes each token in one workgroup of the decode plan's
// nw waves; where that is narrower than the stand-alone quantizer's workgroup, its
// tokens take longer and two launches were faster at every M measured. Otherwise
// one launch saves the second launch and hides the quantization behind the first
// weight loads: it was faster for one token, and for up to 16 tokens of rows of
// at least 12288 inputs, and slower (or level) at more tokens.
int mq_act_one_launch(int64_t M, int64_t N, int64_t K) {
    // outside the shapes the GEMM accepts (K <= 65536, M N < 2^31) there is no plan
    if (M < 1 || M > 32 || N < 16 || K < mq::kGroup || K > 65536 || N > (int64_t(1) << 30)) return 0;
    if (64 * mq::plan_decode(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K)).nw <
        mq::quant_act_threads(M, K))
        return 0;
    return (M == 1 && N >= 4096) ? 1 : 0;
}

int mq_gemm_w4a4_residual_act(const void* x, int x_dtype, const uint8_t* wq, const uint16_t* sw,
                              const int32_t* rmap, const uint8_t* rq, int64_t nnz, int64_t M, int64_t N,
                              int64_t K, int group, int bn, int bk, uint8_t* xq, float* sx, int32_t* sync,
                              int launch, void* y, int y_dtype, void* stream) {
    if (bad_dtype(x_dtype)) return MQ_ERR_INVALID_ARG;
    if (launch != MQ_ACT_AUTO && launch != MQ_ACT_ONE_LAUNCH && launch != MQ_ACT_TWO_LAUNCHES)
        return MQ_ERR_INVALID_ARG;
    int rc = check_gemm(xq, sx, wq, sw, M, N, K, group, bn, bk, y, y_dtype);
    if (rc) return rc;
    if (nnz < 0 || nnz > (N / bn) * (K / bk) || !rmap || (nnz > 0 && (!rq || !aligned16(rq))))
        return MQ_ERR_INVALID_ARG;
    if (nnz * bn * (bk / 2) > (int64_t(1) << 31)) return MQ_ERR_UNSUPPORTED;
    if (launch == MQ_ACT_ONE_LAUNCH && M > 32) return MQ_ERR_INVALID_ARG;
    const bool one = launch == MQ_ACT_ONE_LAUNCH || (launch == MQ_ACT_AUTO && mq_act_one_launch(M, N, K));
    if (M == 0) return MQ_OK;
    if (!x || !aligned16(x) || (one && (!sync || (reinterpret_cast<uintptr_t>(sync) & 3u))))
        return MQ_ERR_INVALID_ARG;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    mq::GemmArgs a = make_args(xq, sx, wq, sw, nullptr, nullptr, rq, nnz, M, N, K, bn, y, y_dtype, nullptr,
                               nullptr);
    a.rmap = rmap;
    if (!one) {
        // quantization with its own launch (one workgroup per token), then the GEMM
        hipError_t e = mq::launch_quant_act(x, x_dtype == MQ_BF16, M, K, nullptr, xq, sx, st);
        if (e == hipSuccess) e = mq::launch_gemm(a, mq::GemmKind::Fused, st);
        return hip_status(e);
    }
    a.x = x;
    a.x_bf16 = x_dtype == MQ_BF16;
    a.xq_w = xq;
    a.sx_w = sx;
    a.sync = sync;
    return hip_status(mq::launch_gemm(a, mq::GemmKind::FusedQuantAct, st));
}

static_assert(mq::kReadProbeMaxBlocks == MQ_READ_PROBE_WORDS, "read probe output size");

int mq_read_probe(const void* p, int64_t bytes, uint32_t* out, void* stream) {
    if (bytes < 0 || (bytes & 15) || (bytes > 0 && (!p || !aligned16(p))) || !out) return MQ_ERR_INVALID_ARG;
    if (bytes == 0) return MQ_OK;
    return hip_status(mq::launch_read_probe(p, bytes, out, static_cast<hipStream_t>(stream)));
}

int mq_gemm_w4a4_dense(const uint8_t* xq, const float* sx, const uint8_t* wq, const uint16_t* sw,
                       int64_t M, int64_t N, int64_t K, int group, void* y, int y_dtype,
                       int32_t* acc_dump, void* stream) {
    int rc = check_gemm(xq, sx, wq, sw, M, N, K, group, 64, mq::kBk, y, y_dtype);
    if (rc) return rc;
    if (M == 0) return MQ_OK;
    const mq::GemmArgs a = make_args(xq, sx, wq, sw, nullptr, nullptr, nullptr, 0, M, N, K, 64, y, y_dtype,
                                     acc_dump, nullptr);
    return hip_status(mq::launch_gemm(a, mq::GemmKind::Dense, static_cast<hipStream_t>(stream)));
}

int mq_gemm_residual_separate(const uint8_t* xq, const float* sx, const uint8_t* wq,
                              const uint16_t* sw, const int32_t* row_ptr, const int32_t* col_idx,
                              const uint8_t* rq, int64_t nnz, int64_t M, int64_t N, int64_t K,
                              int group, int bn, int bk, void* y, int y_dtype, float* ws,
                              void* stream) {
    int rc = check_gemm(xq, sx, wq, sw, M, N, K, group, bn, bk, y, y_dtype);
    if (rc) return rc;
    rc = check_csr(row_ptr, col_idx, rq, nnz, N, K, bn, bk);
    if (rc) return rc;
    if (M > 0 && !ws) return MQ_ERR_INVALID_ARG;
    if (M == 0) return MQ_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const mq::GemmArgs a = make_args(xq, sx, wq, sw, row_ptr, col_idx, rq, nnz, M, N, K, bn, y, y_dtype,
                                     nullptr, ws);
    hipError_t e = mq::launch_gemm(a, mq::GemmKind::DenseToWorkspace, st);
    if (e == hipSuccess) e = mq::launch_residual_merge(a, st);
    return hip_status(e);
}

}  // extern "C"
