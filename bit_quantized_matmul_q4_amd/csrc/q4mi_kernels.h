// q4mi_kernels.h -- launchers of the library's kernels (internal to libq4mi).
// Arguments are validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4mi {

struct DeviceInfo {
    int num_cus;
    int lds_bytes;
};

hipError_t launch_q4_pack(const float *W, int64_t N, int64_t K, int group, uint8_t *qs, uint16_t *sm,
                          int num_cus, hipStream_t stream);
hipError_t launch_q8_1_quantize(const float *x, int64_t M, int64_t K, int8_t *qa, uint16_t *ds,
                                int num_cus, hipStream_t stream);

// group: the (scale, minimum) group along K, 256 or 32.
// The GEMV plan depends on the whole shape only: MR activation rows on the
// VALU arm (0 = matrix-core arm) and, for the matrix-core arm, the K split.
struct GemvPlan {
    int MR, nsplit, gps;
};
GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, int group);
size_t gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int group);
// false for shapes whose output the plan cannot address (see q4_gemv)
bool gemv_shape_supported(int64_t M, int64_t N, int64_t K, int group);
hipError_t launch_gemv(const float *x, int M, const uint8_t *qs, const uint16_t *sm, int64_t N,
                       int K, int group, float *y, void *workspace, size_t ws_bytes, const DeviceInfo &dev,
                       hipStream_t stream);

size_t mmq_workspace_bytes(int64_t M, int64_t N, int64_t K);
// the int8 matrix-core design on its own, at any shape
size_t mmq_int8_workspace_bytes(int64_t M, int64_t N, int64_t K);
// pipelined int8 kernels (mmq_i8.hip) for grids of 128 x 128 tiles: shape
// limits, workspace (per-row and per-weight-row records) and launch; fp32 y,
// or with y null Q8_1 output into qo / dso (N a multiple of 32)
bool mmqi_supported(int64_t M, int64_t N, int64_t K);
size_t mmqi_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_mmqi(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs, const uint16_t *sm,
                       int64_t N, int K, float *y, int8_t *qo, uint16_t *dso, void *workspace,
                       hipStream_t stream);
hipError_t launch_mmq_int8(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                           const uint16_t *sm, int64_t N, int K, float *y, void *workspace,
                           const DeviceInfo &dev, hipStream_t stream);
hipError_t launch_mmq(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                      const uint16_t *sm, int64_t N, int K, float *y, void *workspace,
                      const DeviceInfo &dev, hipStream_t stream);
hipError_t launch_mmq_g32(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                          const uint16_t *sm, int64_t N, int K, float *y, void *workspace,
                          const DeviceInfo &dev, hipStream_t stream);
hipError_t launch_mmq_q8_1(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                           const uint16_t *sm, int64_t N, int K, int8_t *qo, uint16_t *dso,
                           void *workspace, const DeviceInfo &dev, hipStream_t stream);
// fp16 matrix-core MMQ (mmq_f16.hip): y (fp32) or, with y null, Q8_1 output;
// g32: group-32 weights (fp32 output only)
size_t mmqf_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_mmqf(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                       const uint16_t *sm, int64_t N, int K, bool g32, float *y, int8_t *qo, uint16_t *dso,
                       void *workspace, int num_cus, hipStream_t stream);
hipError_t launch_block_dots(const int8_t *qa, int64_t M, const uint8_t *qs, int64_t N, int K,
                             int32_t *idot, const DeviceInfo &dev, hipStream_t stream);

}  // namespace q4mi
