// mxs_internal.h -- host-side launchers shared between the kernel files and
// the C-ABI entry points. Every launcher validates nothing (the entry points
// do) and returns the HIP status of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mxsens.h"

namespace mxs {

constexpr int64_t kChunkRows = 256;        // rows per ordered partial sum
constexpr int64_t kRunChunks = 16;         // chunks per run of the calibration sum
constexpr int64_t kMaxChunksPerLaunch = 65520;   // grid.y limit, whole runs

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// calibrate / score (mxs_colsum.hip)
hipError_t launch_calibrate(const void *X, mxs_dtype dt, int64_t M, int64_t K, int64_t ldx,
                            double *hdiag, double *ws, hipStream_t st);
hipError_t launch_score(const void *W, mxs_dtype dt, int64_t N, int64_t K, int64_t ldw,
                        const double *hdiag, double *score, double *ws, hipStream_t st);

// allocate (mxs_allocate.hip)
hipError_t launch_allocate(const double *score, int64_t K, int32_t c8, int32_t c6,
                           uint8_t *bits, int32_t *perm, hipStream_t st);

// quantize (mxs_quantize.hip)
hipError_t launch_quantize(const void *X, mxs_dtype dt, int64_t ldx, const int32_t *perm,
                           const mxs_qmat &out, hipStream_t st);

// mixed GEMM (mxs_gemm.hip): int8 block sums with fp32 scale epilogues, and
// the variant on the block-scaled fp6 matrix cores (prefill kernels only)
// Prefill calls take W's prepared operand from wprep (filled by
// launch_prepare_weights) or, with wprep NULL, prepare it in the workspace.
size_t gemm_workspace(const mxs_qmat &A, const mxs_qmat &W, bool w_prepared);
size_t gemm_fused_workspace(int64_t M, mxs_dtype dt, const mxs_qmat &W, bool w_prepared);
size_t wprep_bytes(const mxs_qmat &W);
hipError_t launch_prepare_weights(const mxs_qmat &W, void *wprep, hipStream_t st);
hipError_t launch_mixed_gemm_fused(const void *X, mxs_dtype dt, int64_t M, int64_t ldx, const int32_t *perm,
                                   const mxs_qmat &W, const void *wprep, float *Y, int64_t ldy, void *ws,
                                   hipStream_t st);
hipError_t launch_mixed_gemm(const mxs_qmat &A, const mxs_qmat &W, const void *wprep, float *Y, int64_t ldy,
                             void *ws, hipStream_t st);
size_t gemm_workspace_mx(const mxs_qmat &A, const mxs_qmat &W);
hipError_t launch_mixed_gemm_mx(const mxs_qmat &A, const mxs_qmat &W, float *Y, int64_t ldy,
                                void *ws, size_t ws_bytes, hipStream_t st);

// layer sensitivity and layer-wise budget (mxs_layerwise.hip)
size_t output_error_workspace(int64_t M, int64_t N);
hipError_t launch_output_error(const void *X, const void *W, mxs_dtype dtype, int64_t M, int64_t N, int64_t K,
                               int64_t ldx, int64_t ldw, const float *Yq, int64_t ldy, double *err, void *ws,
                               hipStream_t st);
int layer_budget(int32_t L, const double *S, const int64_t *rows, const int64_t *K, double B, int32_t *nblk,
                 double *R_out);

// attention over the 4-bit K/V cache (mxs_attention.hip)
size_t attend_kv4_workspace(int64_t T, int64_t Hq, int64_t Hkv, int64_t D);
bool attend_kv4_supported(int64_t Hq, int64_t Hkv, int64_t D);
hipError_t launch_attend_kv4(const float *q, const uint8_t *kc, const uint8_t *ks, const uint8_t *vc,
                             const uint8_t *vs, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                             float *out, void *ws, hipStream_t st);

}  // namespace mxs
