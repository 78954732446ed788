// q4mi_api.hip -- the C ABI of libq4mi (declared in include/q4mi.h):
// argument validation, the gfx950 gate, the per-device property cache and the
// calls into the kernel launchers.  Validation runs before any HIP call, so an
// invalid call touches no device and enqueues nothing.
#include <atomic>
#include <mutex>
#include <string.h>

#include "q4mi.h"
#include "q4mi_kernels.h"

using q4mi::DeviceInfo;

namespace {

constexpr int kMaxDevices = 64;

struct DeviceSlot {
    std::once_flag once;
    int status;  // Q4_OK, Q4_ERR_ARCH or Q4_ERR_DEVICE
    DeviceInfo info;
};
DeviceSlot g_devices[kMaxDevices];

void probe_device(int dev, DeviceSlot &slot)
{
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        slot.status = Q4_ERR_DEVICE;
        return;
    }
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        slot.status = Q4_ERR_ARCH;
        return;
    }
    slot.info.num_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
    slot.info.lds_bytes = (int)prop.sharedMemPerBlock;
    slot.status = Q4_OK;
}

// Current device's properties, queried once per device.
int current_device(const DeviceInfo **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4_ERR_DEVICE;
    DeviceSlot &slot = g_devices[dev];
    std::call_once(slot.once, probe_device, dev, std::ref(slot));
    if (slot.status != Q4_OK) return slot.status;
    *out = &slot.info;
    return Q4_OK;
}

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline bool valid_k(int64_t K, int64_t unit) { return K > 0 && K <= Q4_MAX_K && K % unit == 0; }

inline int launch_status(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_LAUNCH; }

// Device memory of q4_gemv_noalloc: its K-split partials live here instead of
// in a caller's workspace.  Each device the library runs on holds its own copy
// of the array until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: kernels and copies only ever
// see the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[Q4_NOALLOC_SCRATCH_BYTES];

struct ScratchSlot {
    std::once_flag once;
    int status;  // Q4_OK or Q4_ERR_DEVICE
    void *ptr;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's address of `scratch`, looked up once per device with
// that device current.
int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4_ERR_DEVICE;
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot]() {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        slot.ptr = p;
        slot.status = (e == hipSuccess && p != nullptr) ? Q4_OK : Q4_ERR_DEVICE;
    });
    if (slot.status != Q4_OK) return slot.status;
    *out = slot.ptr;
    return Q4_OK;
}

}  // namespace

extern "C" {

int q4_abi_version(void) { return Q4MI_ABI_VERSION; }

const char *q4_strerror(int code)
{
    switch (code) {
    case Q4_OK: return "success";
    case Q4_ERR_ARG: return "invalid argument (null pointer, dimension or size)";
    case Q4_ERR_ALIGN: return "pointer not aligned as required";
    case Q4_ERR_WORKSPACE: return "workspace missing or too small";
    case Q4_ERR_ARCH: return "current device is not gfx950";
    case Q4_ERR_LAUNCH: return "kernel launch failed";
    case Q4_ERR_DEVICE: return "no usable HIP device";
    default: return "unknown error";
    }
}

static int pack_common(const float *W, int64_t N, int64_t K, int group, uint8_t *qs, uint16_t *sm,
                       void *stream)
{
    if (N < 0 || N > Q4_MAX_N || !valid_k(K, 256)) return Q4_ERR_ARG;
    if (N == 0) return Q4_OK;
    if (!W || !qs || !sm) return Q4_ERR_ARG;
    if (!aligned(W, 16) || !aligned(qs, 16) || !aligned(sm, 4)) return Q4_ERR_ALIGN;
    const DeviceInfo *dev = nullptr;
    if (int rc = current_device(&dev)) return rc;
    return launch_status(q4mi::launch_q4_pack(W, N, K, group, qs, sm, dev->num_cus, (hipStream_t)stream));
}

int q4_pack(const float *W, int64_t N, int64_t K, uint8_t *qs, uint16_t *sm, void *stream)
{
    return pack_common(W, N, K, 256, qs, sm, stream);
}

int q4_pack_g32(const float *W, int64_t N, int64_t K, uint8_t *qs, uint16_t *sm, void *stream)
{
    return pack_common(W, N, K, 32, qs, sm, stream);
}

int q8_1_quantize(const float *x, int64_t M, int64_t K, int8_t *qa, uint16_t *ds, void *stream)
{
    if (M < 0 || M > Q4_MAX_M_MMQ || !valid_k(K, 32)) return Q4_ERR_ARG;
    if (M == 0) return Q4_OK;
    if (!x || !qa || !ds) return Q4_ERR_ARG;
    if (!aligned(x, 16) || !aligned(qa, 16) || !aligned(ds, 4)) return Q4_ERR_ALIGN;
    const DeviceInfo *dev = nullptr;
    if (int rc = current_device(&dev)) return rc;
    return launch_status(q4mi::launch_q8_1_quantize(x, M, K, qa, ds, dev->num_cus, (hipStream_t)stream));
}

// shape rules of q4_gemv / q4_gemv_g32 (pointers aside)
static bool gemv_shape_ok(int64_t M, int64_t N, int64_t K, int group)
{
    return M >= 0 && M <= Q4_GEMV_MAX_M && N >= 0 && N <= Q4_MAX_N && valid_k(K, 256) &&
           q4mi::gemv_shape_supported(M, N, K, group);
}

static size_t gemv_ws_common(int64_t M, int64_t N, int64_t K, int group)
{
    if (!gemv_shape_ok(M, N, K, group)) return 0;
    return q4mi::gemv_workspace_bytes(M, N, K, group);
}

size_t q4_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K) { return gemv_ws_common(M, N, K, 256); }
size_t q4_gemv_g32_workspace_bytes(int64_t M, int64_t N, int64_t K) { return gemv_ws_common(M, N, K, 32); }

static int gemv_common(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm, int64_t N,
                       int64_t K, int group, float *y, void *workspace, size_t ws_bytes, void *stream)
{
    if (!gemv_shape_ok(M, N, K, group)) return Q4_ERR_ARG;
    if (M == 0 || N == 0) return Q4_OK;
    if (!x || !qs || !sm || !y) return Q4_ERR_ARG;
    if (!aligned(x, 16) || !aligned(qs, 16) || !aligned(sm, 4) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    const size_t need = q4mi::gemv_workspace_bytes(M, N, K, group);
    if (need > 0 && (!workspace || ws_bytes < need)) return Q4_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return Q4_ERR_ALIGN;
    const DeviceInfo *dev = nullptr;
    if (int rc = current_device(&dev)) return rc;
    return launch_status(q4mi::launch_gemv(x, (int)M, qs, sm, N, (int)K, group, y, workspace,
                                           need > 0 ? ws_bytes : 0, *dev, (hipStream_t)stream));
}

int q4_gemv(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm, int64_t N, int64_t K,
            float *y, void *workspace, size_t ws_bytes, void *stream)
{
    return gemv_common(x, M, qs, sm, N, K, 256, y, workspace, ws_bytes, stream);
}

int q4_gemv_g32(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm, int64_t N, int64_t K,
                float *y, void *workspace, size_t ws_bytes, void *stream)
{
    return gemv_common(x, M, qs, sm, N, K, 32, y, workspace, ws_bytes, stream);
}

int q4_gemv_noalloc(const float *x, int64_t M, const uint8_t *qs, const uint16_t *sm, int64_t N, int64_t K,
                    float *y, void *stream)
{
    if (!gemv_shape_ok(M, N, K, 256)) return Q4_ERR_ARG;
    if (M == 0 || N == 0) return Q4_OK;
    if (!x || !qs || !sm || !y) return Q4_ERR_ARG;
    if (!aligned(x, 16) || !aligned(qs, 16) || !aligned(sm, 4) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    const size_t need = q4mi::gemv_workspace_bytes(M, N, K, 256);
    if (need > (size_t)Q4_NOALLOC_SCRATCH_BYTES) return Q4_ERR_WORKSPACE;
    const DeviceInfo *dev = nullptr;
    if (int rc = current_device(&dev)) return rc;
    void *ws = nullptr;
    if (need > 0) {
        if (int rc = scratch_address(&ws)) return rc;
    }
    // the partials are written in full before they are read: nothing in the
    // array has to start at zero
    return launch_status(q4mi::launch_gemv(x, (int)M, qs, sm, N, (int)K, 256, y, ws, need > 0 ? need : 0, *dev,
                                           (hipStream_t)stream));
}

size_t q4_mmq_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || M > Q4_MAX_M_MMQ || N < 0 || N > Q4_MAX_N || !valid_k(K, 256)) return 0;
    return q4mi::mmq_workspace_bytes(M, N, K);
}

enum MmqRoute { kRouteShape, kRouteShapeG32, kRouteInt8 };

static int mmq_common(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                      const uint16_t *sm, int64_t N, int64_t K, MmqRoute route, float *y, void *workspace,
                      size_t ws_bytes, void *stream)
{
    if (M < 0 || M > Q4_MAX_M_MMQ || N < 0 || N > Q4_MAX_N || !valid_k(K, 256)) return Q4_ERR_ARG;
    if (M == 0 || N == 0) return Q4_OK;
    if (!qa || !ds || !qs || !sm || !y) return Q4_ERR_ARG;
    if (!aligned(qa, 16) || !aligned(ds, 4) || !aligned(qs, 16) || !aligned(sm, 4) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    const size_t need =
        route == kRouteInt8 ? q4mi::mmq_int8_workspace_bytes(M, N, K) : q4mi::mmq_workspace_bytes(M, N, K);
    if (need > 0 && (!workspace || ws_bytes < need)) return Q4_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return Q4_ERR_ALIGN;
    const DeviceInfo *dev = nullptr;
    if (int rc = current_device(&dev)) return rc;
    hipStream_t st = (hipStream_t)stream;
    switch (route) {
    case kRouteShapeG32: return launch_status(q4mi::launch_mmq_g32(qa, ds, M, qs, sm, N, (int)K, y, workspace, *dev, st));
    case kRouteInt8: return launch_status(q4mi::launch_mmq_int8(qa, ds, M, qs, sm, N, (int)K, y, workspace, *dev, st));
    default: return launch_status(q4mi::launch_mmq(qa, ds, M, qs, sm, N, (int)K, y, workspace, *dev, st));
    }
}

int q4_mmq_gemm(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                const uint16_t *sm, int64_t N, int64_t K, float *y, void *workspace,
                size_t ws_bytes, void *stream)
{
    return mmq_common(qa, ds, M, qs, sm, N, K, kRouteShape, y, workspace, ws_bytes, stream);
}

int q4_mmq_gemm_g32(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                    const uint16_t *sm, int64_t N, int64_t K, float *y, void *workspace,
                    size_t ws_bytes, void *stream)
{
    return mmq_common(qa, ds, M, qs, sm, N, K, kRouteShapeG32, y, workspace, ws_bytes, stream);
}

size_t q4_mmq_int8_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || M > Q4_MAX_M_MMQ || N < 0 || N > Q4_MAX_N || !valid_k(K, 256)) return 0;
    return q4mi::mmq_int8_workspace_bytes(M, N, K);
}

int q4_mmq_gemm_int8(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                     const uint16_t *sm, int64_t N, int64_t K, float *y, void *workspace,
                     size_t ws_bytes, void *stream)
{
    return mmq_common(qa, ds, M, qs, sm, N, K, kRouteInt8, y, workspace, ws_bytes, stream);
}

int q4_mmq_gemm_q8_1(const int8_t *qa, const uint16_t *ds, int64_t M, const uint8_t *qs,
                     const uint16_t *sm, int64_t N, int64_t K, int8_t *qa_out, uint16_t *ds_out,
                     void *workspace, size_t ws_bytes, void *stream)
{
    if (M < 0 || M > Q4_MAX_M_MMQ || N < 0 || N > Q4_MAX_N || N % 32 != 0 || !valid_k(K, 256))
        return Q4_ERR_ARG;
    if (M == 0 || N == 0) return Q4_OK;
    if (!qa || !ds || !qs || !sm || !qa_out || !ds_out) return Q4_ERR_ARG;
    if (!aligned(qa, 16) || !aligned(ds, 4) || !aligned(qs, 16) || !aligned(sm, 4) ||
        !aligned(qa_out, 4) || !aligned(ds_out, 4))
        return Q4_ERR_ALIGN;
    const size_t need = q4mi::mmq_workspace_bytes(M, N, K);
    if (need > 0 && (!workspace || ws_bytes < need)) return Q4_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return Q4_ERR_ALIGN;
    const DeviceInfo *dev = nullptr;
    if (int rc = current_device(&dev)) return rc;
    return launch_status(q4mi::launch_mmq_q8_1(qa, ds, M, qs, sm, N, (int)K, qa_out, ds_out, workspace,
                                               *dev, (hipStream_t)stream));
}

int q4_mmq_block_dots(const int8_t *qa, int64_t M, const uint8_t *qs, int64_t N, int64_t K,
                      int32_t *idot, void *stream)
{
    if (M < 0 || M > Q4_MAX_M_MMQ || N < 0 || N > Q4_MAX_N || !valid_k(K, 256)) return Q4_ERR_ARG;
    if (M == 0 || N == 0) return Q4_OK;
    if (!qa || !qs || !idot) return Q4_ERR_ARG;
    if ((double)M * (double)N * (double)(K / 32) > 2147483648.0) return Q4_ERR_ARG;
    if (!aligned(qa, 16) || !aligned(qs, 16) || !aligned(idot, 4)) return Q4_ERR_ALIGN;
    const DeviceInfo *dev = nullptr;
    if (int rc = current_device(&dev)) return rc;
    return launch_status(q4mi::launch_block_dots(qa, M, qs, N, (int)K, idot, *dev, (hipStream_t)stream));
}

}  // extern "C"
